// decode_mfma_heads_append.hip -- the per-block e4m3 decode kernels that
// also do the step's append (pa_decode_append), instantiated apart from the
// plain ones of decode_mfma_heads.hip.
#include "decode_mfma_heads_kernel.h"

namespace pa {

heads_kernel::HeadsKernel decode_mfma_heads_append_kernel(int kv_type, int d, int bs, int group,
                                                          int hk, bool acc_bf16)
{
    return heads_kernel::pick<true>(kv_type, d, bs, group, hk, acc_bf16);
}

}  // namespace pa
