// merge.hip -- second pass of paged decode: combine, by log-sum-exp, the
// partial results of every query row (sequence or query token, head) whose KV
// segment was split between several chunks, and write the zero rows of empty
// sequences.
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

constexpr int kMergeThreads = 256;

template <int OT, int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(DecodeArgs a, int block_size)
{
    constexpr int NT = kMergeThreads;
    constexpr int LPP = D / 4;                   // threads per partial row (4 floats each)
    constexpr int NSUB = NT / LPP;               // partial rows read per pass
    __shared__ float wts[NT];
    __shared__ float red[NT / 64];
    __shared__ float4 part[NSUB][LPP];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int sub = t / LPP, col = (t % LPP) * 4;
    const int H = a.num_heads, G = a.num_heads / a.num_kv_heads;
    const int RPS = a.rows_per_slot;
    // Output row and the row of its partials within a slot: one query token
    // per sequence -- workgroup s * H + h, partial row h % G; several --
    // workgroup (s * max_query_len + i) * H + h for query token i, partial
    // row i * G + h % G (absent when the sequence has at most i tokens).
    int s, h, prow;
    int64_t row;
    int L;
    if (a.query_start_loc) {
        const int64_t r = blockIdx.x;
        h = (int)(r % H);
        const int i = (int)((r / H) % a.max_query_len);
        s = (int)(r / ((int64_t)H * a.max_query_len));
        L = min(a.seq_lens[s], a.max_nb * block_size);
        int qs, ql;
        query_span(a, s, max(L, 0), &qs, &ql, nullptr);
        if (i >= ql)
            return;
        row = (int64_t)(qs + i) * H + h;
        prow = i * G + h % G;
    } else {
        row = blockIdx.x;
        s = (int)(row / H);
        h = (int)(row % H);
        L = min(a.seq_lens[s], a.max_nb * block_size);
        prow = h % G;
    }

    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float inv = 0.f;
    if (L > 0) {
        const int g = s * a.num_kv_heads + h / G;
        const int first = a.ws_seg[2 * g], last = a.ws_seg[2 * g + 1];
        if (first == last)
            return;                              // one chunk wrote the output
        const int n = last - first + 1;
        // partial p of this row lives at slot first + p, row prow
        const float2 *ml = reinterpret_cast<const float2 *>(a.ws_ml) + (int64_t)first * RPS + prow;
        const float *acc = a.ws_acc + ((int64_t)first * RPS + prow) * D + col;

        float M = -INFINITY;
        for (int i = t; i < n; i += NT)
            M = fmaxf(M, ml[(int64_t)i * RPS].x);
        M = wave_max(M);
        if (lane == 0)
            red[wave] = M;
        __syncthreads();
        M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        __syncthreads();

        // Thread i of each NT-partial chunk computes partial i's weight once;
        // all threads then read it from LDS while accumulating 16-byte pieces.
        float den = 0.f;
        for (int c = 0; c < n; c += NT) {
            float wgt = 0.f;
            if (c + t < n) {
                const float2 v = ml[(int64_t)(c + t) * RPS];
                wgt = (v.x == -INFINITY) ? 0.f : exp2f(v.x - M);
                den += wgt * v.y;
            }
            wts[t] = wgt;
            __syncthreads();
            const int cnt = min(NT, n - c);
#pragma unroll 4
            for (int i = sub; i < cnt; i += NSUB) {
                const float wi = wts[i];
                const float4 x = *reinterpret_cast<const float4 *>(acc + (int64_t)(c + i) * RPS * D);
                o.x = fmaf(wi, x.x, o.x);
                o.y = fmaf(wi, x.y, o.y);
                o.z = fmaf(wi, x.z, o.z);
                o.w = fmaf(wi, x.w, o.w);
            }
            __syncthreads();
        }
        den = wave_sum(den);
        if (lane == 0)
            red[wave] = den;
        part[sub][t % LPP] = o;
        __syncthreads();
        den = red[0] + red[1] + red[2] + red[3];
        inv = den > 0.f ? 1.f / den : 0.f;
        if (sub != 0)
            return;
#pragma unroll
        for (int k = 1; k < NSUB; ++k) {
            const float4 y = part[k][t];
            o.x += y.x;
            o.y += y.y;
            o.z += y.z;
            o.w += y.w;
        }
    } else if (sub != 0) {
        return;
    }
    const int64_t obase = row * D + col;
    const float r[4] = {o.x * inv, o.y * inv, o.z * inv, o.w * inv};
    if constexpr (OT == KT_F32) {
        *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + obase) =
            make_float4(r[0], r[1], r[2], r[3]);
    } else {
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + obase) =
            make_uint2(f32_to_bf16(r[0]) | (f32_to_bf16(r[1]) << 16),
                       f32_to_bf16(r[2]) | (f32_to_bf16(r[3]) << 16));
    }
}

}  // namespace

hipError_t launch_merge(const DecodeArgs &a, int out_type, int head_dim, int block_size,
                        hipStream_t stream)
{
    const int64_t rows = (int64_t)a.num_seqs * a.num_heads *
                         (a.query_start_loc ? a.max_query_len : 1);
    if (rows > INT32_MAX)
        return hipErrorInvalidValue;
    dim3 grid((unsigned)rows), block(kMergeThreads);
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
