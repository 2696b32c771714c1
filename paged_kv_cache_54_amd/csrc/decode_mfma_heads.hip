// decode_mfma_heads.hip -- launch of the per-block e4m3 decode kernel
// (decode_mfma_heads_kernel.h): the plain instances, or with the step's
// append those of decode_mfma_heads_append.hip.
#include "decode_mfma_heads_kernel.h"

namespace pa {

using heads_kernel::HeadsKernel;

namespace {

HeadsKernel pick(int kv_type, int d, int bs, int group, int hk, bool acc_bf16)
{
    return heads_kernel::pick<false>(kv_type, d, bs, group, hk, acc_bf16);
}

}  // namespace

bool decode_mfma_heads_supported(int kv_type, int head_dim, int block_size, int group,
                                 int num_kv_heads)
{
    return pick(kv_type, head_dim, block_size, group, num_kv_heads, false) != nullptr;
}

hipError_t launch_decode_mfma_heads(const DecodeArgs &a, int kv_type, int head_dim,
                                    int block_size, int group, int workgroups,
                                    hipStream_t stream)
{
    const bool ab = (a.flags & kPartialsBf16) != 0;
    const HeadsKernel k =
        a.new_k ? decode_mfma_heads_append_kernel(kv_type, head_dim, block_size, group,
                                                  a.num_kv_heads, ab)
                : pick(kv_type, head_dim, block_size, group, a.num_kv_heads, ab);
    if (!k || workgroups <= 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(k, dim3((unsigned)workgroups), dim3(64 * a.num_kv_heads), 0, stream, a);
    return hipGetLastError();
}

hipError_t decode_mfma_heads_occupancy(int kv_type, int head_dim, int block_size, int group,
                                       int num_kv_heads, bool acc_bf16, int *groups_per_cu)
{
    const HeadsKernel k = pick(kv_type, head_dim, block_size, group, num_kv_heads, acc_bf16);
    if (!k)
        return hipErrorInvalidValue;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        groups_per_cu, reinterpret_cast<const void *>(k), 64 * num_kv_heads, 0);
}

}  // namespace pa
