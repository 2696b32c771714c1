// merge.hip -- second pass of split-KV decode: combine the per-partition
// partial results of one (sequence, query head) by log-sum-exp.
//
// Partition p holds acc_p = sum_t 2^(z_t - m_p) v_t, l_p = sum_t 2^(z_t - m_p)
// and m_p (scores z in log2 units).  With M = max_p m_p and
// w_p = 2^(m_p - M): out = sum_p w_p acc_p / sum_p w_p l_p, which equals the
// softmax-weighted sum over the whole sequence.  Partitions with no tokens
// (m_p = -inf) get weight 0 by selection.  Rows whose sequence fits in one
// partition were finished by the first pass and are skipped here.
#include "pa_device.h"

namespace pa {
namespace {

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x += __shfl_xor(x, off);
    return x;
}

template <int OT, int D>
__global__ __launch_bounds__(64) void merge_kernel(DecodeArgs a, int block_size)
{
    constexpr int PER = D / 64;                  // output elements per lane
    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;              // s * H + h
    const int s = (int)(row / a.num_heads);
    const int L = min(a.seq_lens[s], a.max_nb * block_size);
    if (L <= a.part_tokens)
        return;
    const int n = (L + a.part_tokens - 1) / a.part_tokens;
    const float2 *ml = reinterpret_cast<const float2 *>(a.ws_ml) + row * a.num_parts;
    const float *acc = a.ws_acc + row * a.num_parts * D + lane * PER;

    float M = -INFINITY;
    for (int i = lane; i < n; i += 64)
        M = fmaxf(M, ml[i].x);
    M = wave_max(M);

    // Lane i of each 64-partition chunk computes partition i's weight once;
    // the accumulation loop then broadcasts it with readlane.
    float o[PER], den = 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k)
        o[k] = 0.f;
    for (int c = 0; c < n; c += 64) {
        float w = 0.f;
        if (c + lane < n) {
            const float2 v = ml[c + lane];
            w = (v.x == -INFINITY) ? 0.f : exp2f(v.x - M);
            den += w * v.y;
        }
        const int cnt = min(64, n - c);
#pragma unroll 4
        for (int i = 0; i < cnt; ++i) {
            const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), i));
            const float *src = acc + (int64_t)(c + i) * D;
#pragma unroll
            for (int k = 0; k < PER; ++k)
                o[k] = fmaf(wi, src[k], o[k]);
        }
    }
    den = wave_sum(den);
    const float inv = den > 0.f ? 1.f / den : 0.f;
    const int64_t base = row * D + lane * PER;
    if constexpr (OT == KT_F32) {
#pragma unroll
        for (int k = 0; k < PER; ++k)
            static_cast<float *>(a.out)[base + k] = o[k] * inv;
    } else {
#pragma unroll
        for (int k = 0; k < PER; ++k)
            static_cast<uint16_t *>(a.out)[base + k] = (uint16_t)f32_to_bf16(o[k] * inv);
    }
}

}  // namespace

hipError_t launch_merge(const DecodeArgs &a, int out_type, int head_dim, int block_size,
                        hipStream_t stream)
{
    dim3 grid((unsigned)((int64_t)a.num_seqs * a.num_heads)), block(64);
    if (out_type == KT_F32 && head_dim == 64)
        hipLaunchKernelGGL((merge_kernel<KT_F32, 64>), grid, block, 0, stream, a, block_size);
    else if (out_type == KT_F32 && head_dim == 128)
        hipLaunchKernelGGL((merge_kernel<KT_F32, 128>), grid, block, 0, stream, a, block_size);
    else if (out_type == KT_BF16 && head_dim == 64)
        hipLaunchKernelGGL((merge_kernel<KT_BF16, 64>), grid, block, 0, stream, a, block_size);
    else if (out_type == KT_BF16 && head_dim == 128)
        hipLaunchKernelGGL((merge_kernel<KT_BF16, 128>), grid, block, 0, stream, a, block_size);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pa
