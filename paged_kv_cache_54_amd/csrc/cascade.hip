// cascade.hip -- decode for a batch whose sequences share a prefix of whole
// blocks (the shared-prefix case of the vLLM internals blog, section 1: a
// common prompt is one set of physical blocks that every sequence's table
// names).  Plain decode reads the shared blocks once per sequence; here the
// attention is split at the prefix boundary (log-sum-exp makes the split
// exact):
//
//   prefix pass  all sequences' queries against the shared blocks, read once
//                per group of SPG sequences: the matrix-core multi-query
//                kernel over a virtual batch whose "query tokens" are the
//                group's sequences (no causal bound), partials only;
//   suffix pass  each sequence against its own blocks from the prefix on: the
//                single-query kernel over shifted tables, partials only;
//   merge        per (sequence, head): log-sum-exp over both passes' parts.
//
// This file holds the setup kernel, which writes the two passes' tables,
// lengths and query layout into the workspace and checks the contract, and
// the two-source merge.
#include "pa_device.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void cascade_setup_kernel(CascadeSetupArgs a)
{
    const int N = a.prefix_blocks, S = a.num_seqs, V = a.num_virtual;
    const int sfx = a.max_nb - N;
    const int64_t n_p = (int64_t)V * N, n_s = (int64_t)S * sfx;
    const int64_t n_chk = (int64_t)S * N;
    const int64_t total = n_p + n_s + n_chk + S + V + 1;
    const int cap = a.max_nb * a.block_size;
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * kThreads) {
        int64_t x = e;
        if (x < n_p) {                       // prefix tables: row 0's first N blocks
            a.p_tables[x] = a.block_tables[x % N];
            continue;
        }
        x -= n_p;
        if (x < n_s) {                       // suffix tables: blocks N .. max_nb-1
            const int64_t s = x / sfx, j = x % sfx;
            a.s_tables[x] = a.block_tables[s * a.max_nb + N + j];
            continue;
        }
        x -= n_s;
        if (x < n_chk) {                     // contract: every table starts with the prefix
            const int64_t s = x / N, j = x % N;
            if (a.block_tables[s * a.max_nb + j] != a.block_tables[j])
                raise_flag(a.err_flag, PA_DEVERR_PREFIX);
            continue;
        }
        x -= n_chk;
        if (x < S) {                         // suffix lengths; contract: prefix fully covered
            const int L = min(a.seq_lens[x], cap);
            if (L < N * a.block_size)
                raise_flag(a.err_flag, PA_DEVERR_PREFIX);
            a.s_lens[x] = max(0, L - N * a.block_size);
            continue;
        }
        x -= S;
        if (x < V) {                         // every virtual sequence is the whole prefix
            a.p_lens[x] = N * a.block_size;
            continue;
        }
        x -= V;
        for (int v = 0; v <= V; ++v)         // virtual sequence v carries sequences v*SPG ..
            a.p_qsl[v] = min(v * a.seqs_per_virtual, S);
    }
}

struct Lse {
    float M, den;
    float4 o;
};

__device__ __forceinline__ void lse_add(Lse &s, float m, float l, float4 x)
{
    const float mn = fmaxf(s.M, m);
    const float a = (s.M == mn) ? 1.f : __builtin_amdgcn_exp2f(s.M - mn);
    const float w = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
    s.M = mn;
    s.den = s.den * a + w * l;
    s.o.x = fmaf(w, x.x, s.o.x * a);
    s.o.y = fmaf(w, x.y, s.o.y * a);
    s.o.z = fmaf(w, x.z, s.o.z * a);
    s.o.w = fmaf(w, x.w, s.o.w * a);
}

__device__ __forceinline__ void lse_fold(Lse &s, const Lse &t)
{
    const float mn = fmaxf(s.M, t.M);
    const float a = (s.M == mn) ? 1.f : __builtin_amdgcn_exp2f(s.M - mn);
    const float b = (t.M == mn) ? 1.f : __builtin_amdgcn_exp2f(t.M - mn);
    s.M = mn;
    s.den = s.den * a + t.den * b;
    s.o.x = s.o.x * a + t.o.x * b;
    s.o.y = s.o.y * a + t.o.y * b;
    s.o.z = s.o.z * a + t.o.z * b;
    s.o.w = s.o.w * a + t.o.w * b;
}

// Fold parts [first, last] of one partial source (rows_per_slot rps, row
// prow) into st; the lanes' groups take parts p0, p0 + step, ...
template <int D>
__device__ __forceinline__ void add_parts(Lse &st, const float *acc_ws, const float *ml_ws,
                                          int first, int last, int rps, int prow, int col,
                                          int p0, int step)
{
    const float2 *ml = reinterpret_cast<const float2 *>(ml_ws) + (int64_t)first * rps + prow;
    const float *acc = acc_ws + ((int64_t)first * rps + prow) * D + col;
    const int n = last - first + 1;
    for (int p = p0; p < n; p += 2 * step) {
        float2 m0 = make_float2(-INFINITY, 0.f), m1 = m0;
        float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
        m0 = ml[(int64_t)p * rps];
        x0 = *reinterpret_cast<const float4 *>(acc + (int64_t)p * rps * D);
        if (p + step < n) {
            m1 = ml[(int64_t)(p + step) * rps];
            x1 = *reinterpret_cast<const float4 *>(acc + (int64_t)(p + step) * rps * D);
        }
        lse_add(st, m0.x, m0.y, x0);
        lse_add(st, m1.x, m1.y, x1);
    }
}

// One wavefront per (sequence, head) row, four rows per workgroup.
template <int OT, int D>
__global__ __launch_bounds__(kThreads) void cascade_merge_kernel(CascadeMergeArgs a)
{
    constexpr int LPP = D / 4;                   // lanes per partial row
    constexpr int PPW = 64 / LPP;                // parts per wavefront pass
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane / LPP, col = (lane % LPP) * 4;
    const int64_t r = (int64_t)blockIdx.x * 4 + wave;
    const int H = a.num_heads, Hkv = a.num_kv_heads, G = H / Hkv;
    if (r >= (int64_t)a.num_seqs * H)
        return;
    const int s = (int)(r / H), h = (int)(r % H), kvh = h / G;

    Lse st{-INFINITY, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
    if (a.s_lens[s] > 0) {                       // the sequence's own blocks
        const int g = s * Hkv + kvh;
        add_parts<D>(st, a.s_acc, a.s_ml, a.s_seg[2 * g], a.s_seg[2 * g + 1], G, h % G, col,
                     sub, PPW);
    }
    {                                            // the shared prefix
        const int spg = a.seqs_per_virtual, v = s / spg;
        const int g = v * Hkv + kvh;
        add_parts<D>(st, a.p_acc, a.p_ml, a.p_seg[2 * g], a.p_seg[2 * g + 1], G * spg,
                     (s % spg) * G + h % G, col, sub, PPW);
    }
#pragma unroll
    for (int off = LPP; off < 64; off <<= 1) {
        Lse t;
        t.M = __shfl_xor(st.M, off);
        t.den = __shfl_xor(st.den, off);
        t.o.x = __shfl_xor(st.o.x, off);
        t.o.y = __shfl_xor(st.o.y, off);
        t.o.z = __shfl_xor(st.o.z, off);
        t.o.w = __shfl_xor(st.o.w, off);
        lse_fold(st, t);
    }
    if (sub != 0)
        return;
    const float inv = st.den > 0.f ? 1.f / st.den : 0.f;
    const int64_t obase = r * D + col;
    const float o[4] = {st.o.x * inv, st.o.y * inv, st.o.z * inv, st.o.w * inv};
    if constexpr (OT == KT_F32) {
        *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + obase) =
            make_float4(o[0], o[1], o[2], o[3]);
    } else {
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + obase) =
            make_uint2(f32_to_bf16(o[0]) | (f32_to_bf16(o[1]) << 16),
                       f32_to_bf16(o[2]) | (f32_to_bf16(o[3]) << 16));
    }
}

}  // namespace

hipError_t launch_cascade_setup(const CascadeSetupArgs &a, hipStream_t stream)
{
    const int64_t total = (int64_t)a.num_virtual * a.prefix_blocks +
                          (int64_t)a.num_seqs * a.max_nb + a.num_seqs + a.num_virtual + 1;
    int64_t wgs = (total + 4 * kThreads - 1) / (4 * kThreads);
    wgs = wgs < 1 ? 1 : (wgs > 1024 ? 1024 : wgs);
    hipLaunchKernelGGL(cascade_setup_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_cascade_merge(const CascadeMergeArgs &a, int out_type, int head_dim,
                                hipStream_t stream)
{
    const int64_t rows = (int64_t)a.num_seqs * a.num_heads;
    dim3 grid((unsigned)((rows + 3) / 4)), block(kThreads);
    if (out_type == KT_BF16 && head_dim == 64)
        hipLaunchKernelGGL((cascade_merge_kernel<KT_BF16, 64>), grid, block, 0, stream, a);
    else if (out_type == KT_BF16 && head_dim == 128)
        hipLaunchKernelGGL((cascade_merge_kernel<KT_BF16, 128>), grid, block, 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pa
