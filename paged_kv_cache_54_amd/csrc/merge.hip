// merge.hip -- second pass of paged decode: combine, by log-sum-exp, the
// partial results of every (sequence, query head) whose KV segment was split
// between several chunks, and write the zero rows of empty sequences.
//
// A chunk's partial for one head holds acc_p = sum_t 2^(z_t - m_p) v_t,
// l_p = sum_t 2^(z_t - m_p) and m_p (scores z in log2 units).  With
// M = max_p m_p and w_p = 2^(m_p - M): out = sum_p w_p acc_p / sum_p w_p l_p,
// which equals the softmax-weighted sum over the whole sequence.  Partials
// with no tokens (m_p = -inf) get weight 0 by selection.  The segment record
// gives the first and last slot of the segment; equal slots mean a single
// chunk covered the segment and already wrote the output.
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
    const int H = a.num_heads, G = a.num_heads / a.num_kv_heads;
    const int s = (int)(row / H), h = (int)(row % H);
    const int64_t obase = row * D + lane * PER;
    const int L = min(a.seq_lens[s], a.max_nb * block_size);
    float o[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k)
        o[k] = 0.f;
    float inv = 0.f;
    if (L > 0) {
        const int g = s * a.num_kv_heads + h / G;
        const int first = a.ws_seg[2 * g], last = a.ws_seg[2 * g + 1];
        if (first == last)
            return;                              // one chunk wrote the output
        const int n = last - first + 1;
        const int hig = h % G;
        // partial p of this row lives at slot first + p, head hig
        const float2 *ml = reinterpret_cast<const float2 *>(a.ws_ml) + (int64_t)first * G + hig;
        const float *acc = a.ws_acc + ((int64_t)first * G + hig) * D + lane * PER;

        float M = -INFINITY;
        for (int i = lane; i < n; i += 64)
            M = fmaxf(M, ml[(int64_t)i * G].x);
        M = wave_max(M);

        // Lane i of each 64-partial chunk computes partial i's weight once;
        // the accumulation loop then broadcasts it with readlane.
        float den = 0.f;
        for (int c = 0; c < n; c += 64) {
            float wgt = 0.f;
            if (c + lane < n) {
                const float2 v = ml[(int64_t)(c + lane) * G];
                wgt = (v.x == -INFINITY) ? 0.f : exp2f(v.x - M);
                den += wgt * v.y;
            }
            const int cnt = min(64, n - c);
#pragma unroll 4
            for (int i = 0; i < cnt; ++i) {
                const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), i));
                const float *src = acc + (int64_t)(c + i) * G * D;
#pragma unroll
                for (int k = 0; k < PER; ++k)
                    o[k] = fmaf(wi, src[k], o[k]);
            }
        }
        den = wave_sum(den);
        inv = den > 0.f ? 1.f / den : 0.f;
    }
    if constexpr (OT == KT_F32) {
#pragma unroll
        for (int k = 0; k < PER; ++k)
            static_cast<float *>(a.out)[obase + k] = o[k] * inv;
    } else {
#pragma unroll
        for (int k = 0; k < PER; ++k)
            static_cast<uint16_t *>(a.out)[obase + k] = (uint16_t)f32_to_bf16(o[k] * inv);
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
