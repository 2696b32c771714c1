// decode_mfma.hip -- launch of the single-query matrix-core decode kernel
// (decode_mfma_kernel.h): the plain instances, or with the step's append
// those of decode_mfma_append.hip.
#include "decode_mfma_kernel.h"

namespace pa {

using mfma_kernel::DecodeKernel;
using mfma_kernel::kWavesPerGroup;

namespace {

DecodeKernel pick(int kv_type, int d, int bs, int group, bool acc_bf16)
{
    return mfma_kernel::pick<false>(kv_type, d, bs, group, acc_bf16);
}

}  // namespace

bool mfma_supported(int q_type, int kv_type, int head_dim, int block_size, int group)
{
    return q_type == KT_BF16 && (kv_type == KT_BF16 || kv_type == KT_E4M3) &&
           (head_dim == 64 || head_dim == 128) && (block_size == 16 || block_size == 32) &&
           (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_decode_mfma(const DecodeArgs &a, int kv_type, int head_dim, int block_size,
                              int group, hipStream_t stream)
{
    const bool ab = (a.flags & kPartialsBf16) != 0;
    const DecodeKernel k = a.new_k
                               ? decode_mfma_append_kernel(kv_type, head_dim, block_size, group, ab)
                               : pick(kv_type, head_dim, block_size, group, ab);
    if (!k)
        return hipErrorInvalidValue;
    const unsigned groups = (unsigned)((a.num_waves + kWavesPerGroup - 1) / kWavesPerGroup);
    hipLaunchKernelGGL(k, dim3(groups), dim3(64 * kWavesPerGroup), 0, stream, a);
    return hipGetLastError();
}

hipError_t decode_mfma_occupancy(int kv_type, int head_dim, int block_size, int group,
                                 bool acc_bf16, int *waves_per_cu)
{
    const DecodeKernel k = pick(kv_type, head_dim, block_size, group, acc_bf16);
    if (!k)
        return hipErrorInvalidValue;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        waves_per_cu, reinterpret_cast<const void *>(k), 64 * kWavesPerGroup, 0);
    *waves_per_cu *= kWavesPerGroup;
    return e;
}

}  // namespace pa
