// merge.hip -- second pass of paged decode: combine, by log-sum-exp, the
// partial results of every query row (sequence or query token, head) whose KV
// segment was split between several chunks, and write the zero rows of empty
// sequences.
//
// A chunk's partial for one head holds acc_p = sum_t 2^(z_t - m_p) v_t,
// l_p = sum_t 2^(z_t - m_p) and m_p (scores z in log2 units).  With
// M = max_p m_p and w_p = 2^(m_p - M): out = sum_p w_p acc_p / sum_p w_p l_p,
// which equals the softmax-weighted sum over the whole sequence.  The sum is
// taken online (M raised part by part, earlier terms rescaled), so every
// partial is read once, in one pass.  Partials with no tokens (m_p = -inf)
// get weight 0 by selection.  The segment record gives the first and last
// slot of the segment (its slots step by a.slot_stride); equal slots mean a
// single chunk covered the segment and already wrote the output.
//
// Layout: WPR wavefronts per output row.  A partial row (D floats) is read
// by D/4 lanes, so a wavefront reads 64/(D/4) partials per pass, four passes
// unrolled; the lane groups' running (M, sum, acc) are combined by shuffles,
// the wavefronts of a row through LDS.  One wavefront per row when there are
// many rows (most segments split into a few parts), two rows per wavefront
// when there are very many, eight wavefronts (a 512-thread workgroup) per row
// when there are few (long sequences cut into hundreds of parts: 16.6 ->
// 13.2 us against four on the long-context batch).
#include <type_traits>

#include "pa_device.h"

namespace pa {
namespace {

constexpr int kMergeThreads = 256;        // four wavefronts, except the few-row form

// Running log-sum-exp state of one lane: max M, weighted sum den, weighted
// accumulator o (4 floats of the row).
struct Lse {
    float M, den;
    float4 o;
};

__device__ __forceinline__ void lse_add(Lse &s, float m, float l, float4 x)
{
    const float mn = fmaxf(s.M, m);
    const float a = (s.M == mn) ? 1.f : __builtin_amdgcn_exp2f(s.M - mn);   // 0 when M = -inf
    const float w = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
    s.M = mn;
    s.den = s.den * a + w * l;
    s.o.x = fmaf(w, x.x, s.o.x * a);
    s.o.y = fmaf(w, x.y, s.o.y * a);
    s.o.z = fmaf(w, x.z, s.o.z * a);
    s.o.w = fmaf(w, x.w, s.o.w * a);
}

// Fold another state (its sum already weighted by its own M) into s.
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

// WPR wavefronts per row, or (WPR = 0) two rows per wavefront, one per
// 32-lane half; NW wavefronts per workgroup.  Partial accumulators are f32,
// or bf16 with ACC_BF16.
template <int OT, bool ACC_BF16, int D, int WPR, int NW = 4>
__global__ __launch_bounds__(64 * NW) void merge_kernel(DecodeArgs a, int block_size,
                                                        int64_t num_rows)
{
    constexpr int LPP = D / 4;                   // lanes per partial row (4 floats each)
    constexpr int RW = WPR == 0 ? 2 : 1;         // rows per wavefront
    constexpr int LPR = 64 / RW;                 // lanes per row
    constexpr int PPW = LPR / LPP;               // partials per wavefront pass
    constexpr int UNROLL = 4;
    constexpr int RPW = WPR == 0 ? 2 * NW : NW / WPR;   // rows per workgroup
    __shared__ Lse part[NW][LPP];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int half = lane / LPR, hl = lane % LPR;
    const int sub = hl / LPP, col = (hl % LPP) * 4;
    const int wr = WPR > 1 ? wave % WPR : 0;     // wavefront within its row
    const int64_t r =
        (int64_t)blockIdx.x * RPW + (WPR == 0 ? 2 * wave + half : wave / (WPR > 0 ? WPR : 1));
    const int H = a.num_heads, G = a.num_heads / a.num_kv_heads;
    const int RPS = a.rows_per_slot;

    // Output row and the row of its partials within a slot: one query token
    // per sequence -- grid row s * H + h, partial row h % G; several -- grid
    // row (s * max_query_len + i) * H + h for query token i, partial row
    // i * G + h % G (absent when the sequence has at most i tokens).
    // The segment record is read with the length (and the query span), not
    // after it: the three loads are independent, so a row waits for one
    // memory latency before its partials instead of two.  A sequence with no
    // tokens has no record this call; its stale one is read and not used.
    bool live = r < num_rows;
    int s = 0, h = 0, prow = 0, L = 0, first = 0, n = 0;
    int64_t row = 0;
    int2 rec = make_int2(0, 0);
    if (live) {
        if (a.query_start_loc) {
            h = (int)(r % H);
            const int i = (int)((r / H) % a.max_query_len);
            s = (int)(r / ((int64_t)H * a.max_query_len));
            rec = *reinterpret_cast<const int2 *>(a.ws_seg + 2 * (s * a.num_kv_heads + h / G));
            L = min(a.seq_lens[s], a.max_nb * block_size);
            int qs, ql;
            query_span(a, s, max(L, 0), &qs, &ql, nullptr);
            live = i < ql;
            row = (int64_t)(qs + i) * H + h;
            prow = i * G + h % G;
        } else {
            row = r;
            s = (int)(r / H);
            h = (int)(r % H);
            rec = *reinterpret_cast<const int2 *>(a.ws_seg + 2 * (s * a.num_kv_heads + h / G));
            L = min(a.seq_lens[s], a.max_nb * block_size);
            prow = h % G;
        }
    }
    bool zero_row = live && L <= 0;
    // a fused append for a sequence with no tokens has no position to take
    // the row: it is not written, and the contract violation is reported
    if (zero_row && a.new_k && h == 0 && a.new_slots[s] >= 0)
        raise_flag(a.err_flag, PA_DEVERR_SLOT);
    const int ss = a.slot_stride;                // slots of a segment: first, first + ss, ..
    if (live && L > 0) {
        // The decode pass writes both ends of every segment with tokens.  A
        // record outside the workspace's slots (a workspace that an
        // overlapping call overwrote) is not followed: the row becomes zeros.
        first = rec.x;
        const bool valid = first >= 0 && rec.y >= first && rec.y < a.num_slots;
        zero_row = !valid;
        live = valid && first != rec.y;          // else one chunk wrote the output
        n = (rec.y - first) / ss + 1;
    }

    Lse st{-INFINITY, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
    if (live && !zero_row) {
        // partial p of this row: slot first + p * ss, row prow
        const float2 *ml = reinterpret_cast<const float2 *>(a.ws_ml) + (int64_t)first * RPS + prow;
        using AT = typename std::conditional<ACC_BF16, uint16_t, float>::type;
        const AT *acc = static_cast<const AT *>(a.ws_acc) + ((int64_t)first * RPS + prow) * D + col;
        const int stride = (WPR > 1 ? WPR : 1) * PPW;
        for (int p0 = wr * PPW + sub; p0 < n; p0 += UNROLL * stride) {
            float2 mlv[UNROLL];
            float4 x[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int p = p0 + u * stride;
                if (p < n) {
                    const int64_t ps = (int64_t)p * ss * RPS;
                    mlv[u] = ml[ps];
                    if constexpr (!ACC_BF16) {
                        x[u] = *reinterpret_cast<const float4 *>(acc + ps * D);
                    } else {
                        const uint2 v = *reinterpret_cast<const uint2 *>(acc + ps * D);
                        x[u] = make_float4(__uint_as_float(v.x << 16),
                                           __uint_as_float(v.x & 0xffff0000u),
                                           __uint_as_float(v.y << 16),
                                           __uint_as_float(v.y & 0xffff0000u));
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                if (p0 + u * stride < n)
                    lse_add(st, mlv[u].x, mlv[u].y, x[u]);
        }
    }
    // lane groups of the row hold the same columns for different parts
#pragma unroll
    for (int off = LPP; off < LPR; off <<= 1) {
        Lse t;
        t.M = __shfl_xor(st.M, off);
        t.den = __shfl_xor(st.den, off);
        t.o.x = __shfl_xor(st.o.x, off);
        t.o.y = __shfl_xor(st.o.y, off);
        t.o.z = __shfl_xor(st.o.z, off);
        t.o.w = __shfl_xor(st.o.w, off);
        lse_fold(st, t);
    }
    if constexpr (WPR > 1) {
        if (sub == 0)
            part[wave][lane] = st;
        __syncthreads();
        if (wr != 0)
            return;
#pragma unroll
        for (int k = 1; k < WPR; ++k)
            if (sub == 0)
                lse_fold(st, part[wave + k][lane]);
    }
    if (sub != 0 || !(live || zero_row))
        return;
    const float inv = st.den > 0.f ? 1.f / st.den : 0.f;
    const int64_t obase = row * D + col;
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

template <int OT, bool ACC_BF16, int D>
hipError_t launch(const DecodeArgs &a, int block_size, int64_t rows, hipStream_t stream)
{
    // Few rows: their sequences are long and cut into many parts; give each
    // row a workgroup of eight wavefronts.
    // Many rows (several query tokens per sequence): two rows per wavefront,
    // so every row's loads are in flight in one round of wavefronts.
    const bool wide = rows < 2048, packed = rows >= 8192;
    const int64_t wgs = wide ? rows : packed ? (rows + 7) / 8 : (rows + 3) / 4;
    if (wgs > INT32_MAX)
        return hipErrorInvalidValue;
    dim3 grid((unsigned)wgs), block(kMergeThreads);
    if (wide)
        hipLaunchKernelGGL((merge_kernel<OT, ACC_BF16, D, 8, 8>), grid, dim3(512), 0, stream, a, block_size,
                           rows);
    else if (packed)
        hipLaunchKernelGGL((merge_kernel<OT, ACC_BF16, D, 0>), grid, block, 0, stream, a, block_size, rows);
    else
        hipLaunchKernelGGL((merge_kernel<OT, ACC_BF16, D, 1>), grid, block, 0, stream, a, block_size, rows);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const DecodeArgs &a, int out_type, int head_dim, int block_size,
                        hipStream_t stream)
{
    const int64_t rows = (int64_t)a.num_seqs * a.num_heads *
                         (a.query_start_loc ? a.max_query_len : 1);
    const bool acc_bf16 = (a.flags & kPartialsBf16) != 0;
    if (out_type == KT_F32 && !acc_bf16 && head_dim == 64)
        return launch<KT_F32, false, 64>(a, block_size, rows, stream);
    if (out_type == KT_F32 && !acc_bf16 && head_dim == 128)
        return launch<KT_F32, false, 128>(a, block_size, rows, stream);
    if (out_type == KT_BF16 && head_dim == 64)
        return acc_bf16 ? launch<KT_BF16, true, 64>(a, block_size, rows, stream)
                        : launch<KT_BF16, false, 64>(a, block_size, rows, stream);
    if (out_type == KT_BF16 && head_dim == 128)
        return acc_bf16 ? launch<KT_BF16, true, 128>(a, block_size, rows, stream)
                        : launch<KT_BF16, false, 128>(a, block_size, rows, stream);
    return hipErrorInvalidValue;
}

}  // namespace pa
