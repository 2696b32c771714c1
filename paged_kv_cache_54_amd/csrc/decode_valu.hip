// decode_valu.hip -- paged decode attention on the vector ALUs, for every
// supported dtype (f32, bf16, e4m3 caches) and group size.
//
// What is computed (vLLM concept page, "Technical principles": the
// PagedAttention pseudocode and the fused-gather remark after it): for
// sequence s and KV head g, the query heads g*G .. g*G+G-1 attend over the
// first seq_len tokens of the KV rows gathered block by block through the
// sequence's block table; the gather happens inside this kernel, straight from
// the pool into registers, with no concatenated copy.
//
// Work split: the batch's (sequence, KV head, block) units are cut into
// equal chunks, one per wavefront (see the work-list notes in pa_device.h).
// Lane layout within a block: a token row of D elements is split into D/8
// chunks of 8 elements, lane = row_in_pass * (D/8) + chunk, so one pass of
// the wavefront covers 64/(D/8) rows of the block with loads that read whole
// rows.  Scores: per-lane partial dot products reduced across the D/8 lanes
// of a row.  Softmax: online (running max m, running sum l, in log2 units
// with the scale folded into q), one rescale per block.  The unfilled tail
// of the last block is masked by selection: score := -inf, weight := 0 and
// the V row replaced by 0 before it is multiplied, so NaN/Inf bits in slots
// past seq_len never reach the sum (vLLM v0.17.1 notes, fix #35219).  A
// wavefront that covers a whole segment writes the final output; otherwise
// it writes (acc, m, l) for the merge kernel.
#include "pa_device.h"

namespace pa {
namespace {

template <int QT, int KT, int D, int BS, int G>
__global__ __launch_bounds__(64) void decode_valu_kernel(DecodeArgs a)
{
    constexpr int TPR = D / 8;          // lanes per row
    constexpr int R = 64 / TPR;         // rows per pass
    constexpr int PASSES = BS / R;
    static_assert(BS % R == 0, "block must be a whole number of passes");

    const int lane = threadIdx.x;
    const int rl = lane / TPR;
    const int ch = lane % TPR;
    const int H = a.num_heads, Hkv = a.num_kv_heads;
    const int cap = a.max_nb * BS;
    const int w = blockIdx.x;

    const Lens lens{a.seq_lens, 0};
    const Chunk chunk = my_chunk<BS>(a, lens, w, a.num_waves, (a.flags & kRuns) != 0);
    if (chunk.n == 0)
        return;

    const int64_t slot_elems = (int64_t)Hkv * D;
    const int64_t lane_elem = (int64_t)rl * slot_elems + ch * 8;

    struct Tile {
        Raw8<KT> k[PASSES], v[PASSES];
    };
    auto load_tile = [&](int id, int kvh, Tile &t) {
        const int64_t base = (int64_t)id * BS * slot_elems + lane_elem + (int64_t)kvh * D;
#pragma unroll
        for (int r = 0; r < PASSES; ++r) {
            t.k[r] = stream_raw8<KT>(a.key_cache, base + (int64_t)r * R * slot_elems);
            t.v[r] = stream_raw8<KT>(a.value_cache, base + (int64_t)r * R * slot_elems);
        }
    };

    // per-segment state: query rows of the head group with scale * log2(e)
    // (* k_scale) folded in, running max m, sums l and weighted V sums acc
    float qf[G][8], m[G], l[G], acc[G][8];
    bool seg_starts = false;

    auto begin_segment = [&](const Cursor &c) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            load_q8<QT>(a.q, ((int64_t)c.s * H + c.kvh * G + g) * D + ch * 8, qf[g]);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                qf[g][i] *= a.qk_scale_log2;
            m[g] = -INFINITY;
            l[g] = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[g][i] = 0.f;
        }
        seg_starts = c.j == 0;
    };

    auto finish_segment = [&](const Cursor &c, bool ends) {
        // Sum the row groups' partial (l, acc); m is already uniform across the wave.
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int off = TPR; off < 64; off <<= 1) {
                l[g] += __shfl_xor(l[g], off);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    acc[g][i] += __shfl_xor(acc[g][i], off);
            }
        }
        const int gseg = c.s * Hkv + c.kvh;
        const int slot = w + gseg;
        record_segment(a, gseg, slot, seg_starts, ends);
        if (rl != 0)
            return;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float o[8];
            if (seg_starts && ends) {
                const float inv = l[g] > 0.f ? a.v_scale / l[g] : 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    o[i] = acc[g][i] * inv;
                store8<QT>(a.out, ((int64_t)c.s * H + c.kvh * G + g) * D + ch * 8, o);
            } else {
                const int64_t pi = (int64_t)slot * G + g;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    o[i] = acc[g][i] * a.v_scale;
                if (QT == KT_BF16 && (a.flags & kPartialsBf16))
                    store8<KT_BF16>(a.ws_acc, pi * D + ch * 8, o);
                else
                    store8<KT_F32>(a.ws_acc, pi * D + ch * 8, o);
                if (ch == 0)
                    *reinterpret_cast<float2 *>(a.ws_ml + pi * 2) = make_float2(m[g], l[g]);
            }
        }
    };

    auto process = [&](const Cursor &c, const Tile &t) {
        const int t1 = c.L;
        const int tok0 = c.j * BS + rl;
        float sc[PASSES][G];
        bool valid[PASSES];
#pragma unroll
        for (int r = 0; r < PASSES; ++r) {
            float kf[8];
            unpack8(t.k[r], kf);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    d = fmaf(qf[g][i], kf[i], d);
#pragma unroll
                for (int off = TPR / 2; off > 0; off >>= 1)
                    d += __shfl_xor(d, off);
                sc[r][g] = d;
            }
            valid[r] = (tok0 + r * R) < t1;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float bm = -INFINITY;
#pragma unroll
            for (int r = 0; r < PASSES; ++r)
                bm = fmaxf(bm, valid[r] ? sc[r][g] : -INFINITY);
#pragma unroll
            for (int off = TPR; off < 64; off <<= 1)
                bm = fmaxf(bm, __shfl_xor(bm, off));
            const float mn = fmaxf(m[g], bm);
            const float alpha = (mn == m[g]) ? 1.f : exp2f(m[g] - mn);
            m[g] = mn;
            l[g] *= alpha;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[g][i] *= alpha;
        }
#pragma unroll
        for (int r = 0; r < PASSES; ++r) {
            float vf[8];
            unpack8(t.v[r], vf);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                vf[i] = valid[r] ? vf[i] : 0.f;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float p = valid[r] ? exp2f(sc[r][g] - m[g]) : 0.f;
                l[g] += p;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    acc[g][i] = fmaf(p, vf[i], acc[g][i]);
            }
        }
    };

    // Walk the chunk; the next block's loads are issued before this one is used.
    BlockIds ids(a.block_tables, a.max_nb, a.max_nb, a.num_blocks, a.err_flag);
    Cursor cc = chunk.start;
    Cursor lc = cc;
    const int n = chunk.n;

    Tile cur, nxt;
    int id = ids.get(lc.s, lc.j);
    if (id >= 0)
        load_tile(id, lc.kvh, cur);
    for (int k = 0; k < n; ++k) {
        int id_next = -1;
        if (k + 1 < n) {
            advance<BS>(lc, lens, Hkv, cap);
            id_next = ids.get(lc.s, lc.j);
            if (id_next >= 0)
                load_tile(id_next, lc.kvh, nxt);
        }
        if (k == 0 || cc.j == 0)
            begin_segment(cc);
        if (id >= 0)
            process(cc, cur);
        const bool ends = cc.j == cc.nb - 1;
        if (ends || k == n - 1)
            finish_segment(cc, ends);
        if (k + 1 < n)
            advance<BS>(cc, lens, Hkv, cap);
        id = id_next;
        cur = nxt;
    }
}

typedef void (*DecodeKernel)(DecodeArgs);

template <int QT, int KT, int D, int BS>
DecodeKernel pick_g(int group)
{
    switch (group) {
    case 1: return decode_valu_kernel<QT, KT, D, BS, 1>;
    case 2: return decode_valu_kernel<QT, KT, D, BS, 2>;
    case 4: return decode_valu_kernel<QT, KT, D, BS, 4>;
    case 8: return decode_valu_kernel<QT, KT, D, BS, 8>;
    default: return nullptr;
    }
}

template <int QT, int KT>
DecodeKernel pick_shape(int d, int bs, int group)
{
    if (d == 64 && bs == 16) return pick_g<QT, KT, 64, 16>(group);
    if (d == 64 && bs == 32) return pick_g<QT, KT, 64, 32>(group);
    if (d == 128 && bs == 16) return pick_g<QT, KT, 128, 16>(group);
    if (d == 128 && bs == 32) return pick_g<QT, KT, 128, 32>(group);
    return nullptr;
}

DecodeKernel pick(int q_type, int kv_type, int d, int bs, int group)
{
    if (q_type == KT_F32 && kv_type == KT_F32)
        return pick_shape<KT_F32, KT_F32>(d, bs, group);
    if (q_type == KT_BF16 && kv_type == KT_BF16)
        return pick_shape<KT_BF16, KT_BF16>(d, bs, group);
    if (q_type == KT_BF16 && kv_type == KT_E4M3)
        return pick_shape<KT_BF16, KT_E4M3>(d, bs, group);
    return nullptr;
}

}  // namespace

hipError_t launch_decode_valu(const DecodeArgs &a, int q_type, int kv_type, int head_dim,
                              int block_size, int group, hipStream_t stream)
{
    const DecodeKernel k = pick(q_type, kv_type, head_dim, block_size, group);
    if (!k)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(k, dim3(a.num_waves), dim3(64), 0, stream, a);
    return hipGetLastError();
}

hipError_t decode_valu_occupancy(int q_type, int kv_type, int head_dim, int block_size, int group,
                                 int *waves_per_cu)
{
    const DecodeKernel k = pick(q_type, kv_type, head_dim, block_size, group);
    if (!k)
        return hipErrorInvalidValue;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(waves_per_cu,
                                                        reinterpret_cast<const void *>(k), 64, 0);
}

}  // namespace pa
