// decode_mfma_append.hip -- the single-query matrix-core decode kernels that
// also do the step's append (pa_decode_append), instantiated apart from the
// plain ones of decode_mfma.hip (decode_mfma_kernel.h says why).
#include "decode_mfma_kernel.h"

namespace pa {

mfma_kernel::DecodeKernel decode_mfma_append_kernel(int kv_type, int d, int bs, int group,
                                                   bool acc_bf16)
{
    return mfma_kernel::pick<true>(kv_type, d, bs, group, acc_bf16);
}

}  // namespace pa
