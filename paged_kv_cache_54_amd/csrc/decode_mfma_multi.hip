// decode_mfma_multi.hip -- paged attention for several new query tokens per
// sequence on the gfx950 matrix cores (bf16 query; bf16 or e4m3 cache): the
// verify step of speculative decoding, where the target model checks K
// drafted tokens in one pass (P-EAGLE page).
//
// Sequence s owns query tokens query_start_loc[s] .. query_start_loc[s+1]-1;
// they are its last q_len positions (already appended to the cache), and
// query token i attends to positions 0 .. L - q_len + i (causal within the
// new tokens).  Everything else -- the work list of (sequence, KV head,
// block) units cut into equal chunks, the gather through the block table,
// bf16 LDS tiles, online softmax in log2 units, selection masking, partials
// and the log-sum-exp merge -- is the single-token matrix-core kernel's.  The
// difference is the MFMA column space: a KV head's query rows are the
// (query token, head of the group) pairs, column c = i * G + g, and there are
// NT tiles of 16 columns.  Each K operand read from LDS feeds the QK MFMAs of
// all NT column tiles, each transposed V operand the PV MFMAs of all NT, so
// the KV bytes of a block are read once for all q_len * G query rows.
// Causality is one more bound per column: column c sees tokens below
// lim_c = L - q_len + i + 1, applied by selection like the sequence end.
//
// One wavefront takes a chunk (decode_mfma_multi_kernel) up to 16 columns,
// and up to 32 with a bf16 cache; with more, two wavefronts share it
// (decode_mfma_multi_coop_kernel): each loads half of every tile (K or V)
// into a shared LDS tile and computes half of the column tiles, so a
// wavefront holds half the operands and accumulators.  At 32 columns (the
// Llama-shaped verify step) the two-wavefront kernel beat one wavefront
// holding both column tiles at two wavefronts per SIMD (147.4 against
// 152.2 us per step); one wavefront per SIMD, the single-query kernel's
// setting for a bf16 cache, turned that around (155.5 against 156.9 us).
#include "mfma_common.h"

namespace pa {
namespace {

// s_waitcnt operand: memory loads and stores counter 0, the other counters
// not waited on (expcnt 7, lgkmcnt 15).
constexpr int kWaitVm0 = 0x0F70;

// One wavefront's NT column tiles of a segment, columns col0 .. col0 + 16 NT
// - 1: per tile the Q^T operand, accumulators, running max and lane-partial
// sum, the causal bound and the output row; and the three steps both kernels
// apply to them (start a segment, attend a staged tile, write the result).
template <int KT, int D, int BS, int NT, bool AB>
struct MultiCols {
    using Geo = MfmaGeo<KT, D, BS>;
    static constexpr int NC = Geo::NC, ND = Geo::ND, TILE = Geo::TILE, MT = Geo::MT;
    static constexpr int KROWB = Geo::KROWB, VROWB = Geo::VROWB;

    bf16x8 qop[NT][NC];
    f32x4 acc[NT][ND];
    float m[NT], l[NT];
    int lim[NT];                               // tokens [0, lim) visible; 0 = unused column
    int64_t orow[NT];                          // (token * H + head), -1 = unused column
    int full_end = 0;                          // tiles ending by here need no mask
    bool seg_starts = false;
    const int col0, g4, c16;

    __device__ __forceinline__ MultiCols(int col0_, int lane)
        : col0(col0_), g4(lane >> 4), c16(lane & 15)
    {
    }

    // Load the segment's query columns; `flag` (if set) takes layout errors.
    __device__ __forceinline__ void begin(const DecodeArgs &a, const Cursor &c, uint32_t *flag)
    {
        const int H = a.num_heads, G = H / a.num_kv_heads, lg = a.log2_group;
        int qs, ql;
        query_span(a, c.s, c.L, &qs, &ql, flag);
        qs = __builtin_amdgcn_readfirstlane(qs);
        ql = __builtin_amdgcn_readfirstlane(ql);
        full_end = c.L - ql + 1;               // the first query token's bound, the smallest
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int col = col0 + 16 * nt + c16;
            const int i = col >> lg, g = col & (G - 1);
            const bool valid = i < ql;
            lim[nt] = valid ? c.L - ql + i + 1 : 0;
            orow[nt] = valid ? (int64_t)(qs + i) * H + c.kvh * G + g : -1;
            const uint16_t *qrow =
                static_cast<const uint16_t *>(a.q) + (valid ? orow[nt] : 0) * D + 8 * g4;
#pragma unroll
            for (int k = 0; k < NC; ++k)
                qop[nt][k] = valid ? as_bf16x8(*reinterpret_cast<const uint4 *>(qrow + 32 * k))
                                   : as_bf16x8(make_uint4(0, 0, 0, 0));
#pragma unroll
            for (int d = 0; d < ND; ++d)
                acc[nt][d] = f32x4{0.f, 0.f, 0.f, 0.f};
            m[nt] = -INFINITY;
            l[nt] = 0.f;
        }
        seg_starts = c.j == 0;
    }

    // The segment's result: the output rows when this chunk covered the whole
    // segment, else a partial in slot `slot`.
    __device__ __forceinline__ void finish(const DecodeArgs &a, int slot, bool ends)
    {
        const int RPS = a.rows_per_slot;       // partial rows per slot: G * max_query_len
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const float lt = rows_sum(l[nt]);  // sum the four 16-lane groups
            if (orow[nt] < 0)
                continue;
            if (seg_starts && ends && !(a.flags & kPartialOnly)) {
                const float inv = lt > 0.f ? a.v_scale / lt : 0.f;
                uint16_t *o = static_cast<uint16_t *>(a.out) + orow[nt] * D + 4 * g4;
#pragma unroll
                for (int d = 0; d < ND; ++d)
                    *reinterpret_cast<uint2 *>(o + 16 * d) =
                        make_uint2(pack_bf16x2(acc[nt][d][0] * inv, acc[nt][d][1] * inv),
                                   pack_bf16x2(acc[nt][d][2] * inv, acc[nt][d][3] * inv));
            } else {
                const int64_t pi = (int64_t)slot * RPS + col0 + 16 * nt + c16;
                store_partial<ND, AB>(a.ws_acc, pi, g4, acc[nt], a.v_scale);
                if (g4 == 0)
                    *reinterpret_cast<float2 *>(a.ws_ml + pi * 2) = make_float2(m[nt], lt);
            }
        }
    }

    // QK^T for every column tile from the staged K tile, online softmax per
    // column, PV from the staged V tile (each LDS operand read once for all
    // NT tiles).
    __device__ __forceinline__ void process(const DecodeArgs &a, const Cursor &c, int half,
                                            const uint8_t *kt, const uint8_t *vt)
    {
        const int tok_base = c.j * BS + half * TILE;
        const bool full = tok_base + TILE <= full_end;   // every column sees the whole tile
        f32x4 sc[MT][NT];
#pragma unroll
        for (int h = 0; h < MT; ++h) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                sc[h][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const uint8_t *krow = kt + (16 * h + c16) * KROWB + 16 * g4;
#pragma unroll
            for (int k = 0; k < NC; ++k) {
                const bf16x8 kop = as_bf16x8(*reinterpret_cast<const uint4 *>(krow + 64 * k));
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    sc[h][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[nt][k],
                                                                      sc[h][nt], 0, 0, 0);
            }
        }

        bf16x4 pop[MT][NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            // scale, mask (sequence end and causality) by selection, column max
            float bm = -INFINITY;
#pragma unroll
            for (int h = 0; h < MT; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = sc[h][nt][i] * a.qk_scale_log2;
                    if (!full)
                        v = tok_base + 16 * h + 4 * g4 + i < lim[nt] ? v : -INFINITY;
                    sc[h][nt][i] = v;
                    bm = fmaxf(bm, v);
                }
            const float tm = rows_max(bm);
            if (__ballot(tm > m[nt] + kRebase)) {
                const float mn = fmaxf(m[nt], tm);
                const float alpha = (mn > m[nt]) ? __builtin_amdgcn_exp2f(m[nt] - mn) : 1.f;
                l[nt] *= alpha;
#pragma unroll
                for (int d = 0; d < ND; ++d)
                    acc[nt][d] *= alpha;
                m[nt] = mn;
            }
#pragma unroll
            for (int h = 0; h < MT; ++h) {
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] = (!full && sc[h][nt][i] == -INFINITY)
                               ? 0.f
                               : __builtin_amdgcn_exp2f(sc[h][nt][i] - m[nt]);
                    l[nt] += p[i];
                }
                pop[h][nt] = __builtin_bit_cast(
                    bf16x4, make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])));
            }
        }

        // O^T += V^T P^T per column tile, each V^T operand read once from LDS
#pragma unroll
        for (int h = 0; h < MT; ++h) {
            const int row = 16 * h + 4 * g4 + (c16 >> 2);
#pragma unroll
            for (int d = 0; d < ND; ++d) {
                const int addr = row * VROWB + 32 * d + 8 * (c16 & 3);
                const s16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)((__attribute__((address_space(3))) uint8_t *)vt + addr));
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[nt][d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                        as_bf16x4(raw), pop[h][nt], acc[nt][d], 0, 0, 0);
            }
        }
    }
};

// One wavefront per chunk, all NT column tiles.  AB: bf16 partial accumulators.
template <int KT, int D, int BS, int NT, bool AB>
__global__ __launch_bounds__(64) void decode_mfma_multi_kernel(DecodeArgs a)
{
    using Geo = MfmaGeo<KT, D, BS>;
    constexpr int TILE = Geo::TILE, HALVES = Geo::HALVES;
    __shared__ __attribute__((aligned(16))) uint8_t kt[TILE * Geo::KROWB];
    __shared__ __attribute__((aligned(16))) uint8_t vt[TILE * Geo::VROWB];

    const int lane = threadIdx.x;
    const int Hkv = a.num_kv_heads;
    const int cap = a.max_nb * BS;
    const int w = blockIdx.x;

    const Lens lens{a.seq_lens, 0};
    const Chunk chunk = my_chunk<BS>(a, lens, w, a.num_waves, (a.flags & kRuns) != 0);
    if (chunk.n == 0)
        return;

    const MfmaLoader<Geo> loader(a, lane);
    using Tile = MfmaTile<Geo>;
    MultiCols<KT, D, BS, NT, AB> cols(0, lane);

    // Walk the chunk tile by tile with one register tile in flight: tile k is
    // staged into LDS, then the loads of tile k+1 are issued into the same
    // registers and stay in flight while tile k is computed from LDS.
    BlockIds ids(a.block_tables, a.max_nb, a.max_nb, a.num_blocks, a.err_flag);
    Cursor cc = chunk.start;
    Cursor lc = cc;
    const int n = chunk.n;
    const int steps = n * HALVES;

    int l_half = 0;
    int l_id = ids.get(lc.s, lc.j);
    auto next_load = [&](int k) {
        if (k >= steps) {
            l_id = -1;
            return;
        }
        if (++l_half == HALVES) {
            l_half = 0;
            advance<BS>(lc, lens, Hkv, cap);
            l_id = ids.get(lc.s, lc.j);
        }
    };

    Tile t;
    int id = l_id, half = l_half;
    loader.load(id, lc.kvh, half, t);
    for (int k = 0; k < steps; ++k) {
        const int unit = k / HALVES;
        if (half == 0 && (unit == 0 || cc.j == 0))
            cols.begin(a, cc, cc.kvh == 0 && lane == 0 ? a.err_flag : nullptr);
        if (id >= 0)
            stage_tile<Geo>(loader, kt, vt, t, cc.j * BS + half * TILE, cc.L);
        next_load(k + 1);
        const int id_next = l_id, half_next = l_half;
        loader.load(id_next, lc.kvh, half_next, t);
        if (id >= 0)
            cols.process(a, cc, half, kt, vt);
        if (half == HALVES - 1) {
            const bool ends = cc.j == cc.nb - 1;
            if (ends || unit == n - 1) {
                const int g = cc.s * Hkv + cc.kvh;
                record_segment(a, g, w + g, cols.seg_starts, ends);
                cols.finish(a, w + g, ends);
            }
            if (unit + 1 < n)
                advance<BS>(cc, lens, Hkv, cap);
        }
        id = id_next;
        half = half_next;
    }
}

// Two wavefronts per chunk: the workgroup's wavefronts walk the same chunk,
// wavefront 0 loading each tile's K rows and wavefront 1 its V rows into a
// shared LDS tile (two buffers, one barrier per tile), and each computing its
// own NTW column tiles.  DEPTH tiles are in flight in registers.  Tile k is
// staged into buffer k & 1, which tile k - 2 last read: both wavefronts
// finished that before the barrier of tile k - 1.  Loads are nontemporal
// global loads from the block address (2.3 % faster than per-block buffer
// resources on the verify step); a tile past the chunk's end reads block 0
// and is never staged.
constexpr int kCoopWaves = 2;

template <int KT, int D, int BS, int NTW, int DEPTH, bool AB>
__global__ __launch_bounds__(64 * kCoopWaves) void decode_mfma_multi_coop_kernel(DecodeArgs a)
{
    using Geo = MfmaGeo<KT, D, BS>;
    constexpr int TILE = Geo::TILE, HALVES = Geo::HALVES, NLOAD = Geo::NLOAD;
    constexpr int KROWB = Geo::KROWB, VROWB = Geo::VROWB;

    __shared__ __attribute__((aligned(16))) uint8_t kt_all[2][TILE * KROWB];
    __shared__ __attribute__((aligned(16))) uint8_t vt_all[2][TILE * VROWB];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int Hkv = a.num_kv_heads;
    const int cap = a.max_nb * BS;
    const int w = blockIdx.x;

    const Lens lens{a.seq_lens, 0};
    const Chunk chunk = my_chunk<BS>(a, lens, w, a.num_waves, (a.flags & kRuns) != 0);
    if (chunk.n == 0)
        return;

    // this wavefront's tensor of each tile
    const void *cache = wave == 0 ? a.key_cache : a.value_cache;
    const int slot_bytes = Hkv * D * Geo::EB;
    const int64_t block_bytes = (int64_t)BS * slot_bytes;
    const int l_row = lane / Geo::RCH, l_chunk = lane % Geo::RCH;
    const int l_voff = l_row * slot_bytes + l_chunk * 16;
    struct Part {
        uint4 v[NLOAD];
    };
    auto load_part = [&](int id, int kvh, int half, Part &p) {
        const int64_t base = (int64_t)(id < 0 ? 0 : id) * block_bytes + l_voff +
                             kvh * D * Geo::EB + half * TILE * slot_bytes;
        const u32x4 *src =
            reinterpret_cast<const u32x4 *>(static_cast<const char *>(cache) + base);
        const int step = Geo::LROWS * slot_bytes / 16;
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            const u32x4 x = __builtin_nontemporal_load(src + i * step);
            p.v[i] = make_uint4(x.x, x.y, x.z, x.w);
        }
    };
    // K rows as they are; V rows at or past the sequence end as zeros
    auto stage_part = [&](const Part &p, int buf, int tok_base, int t1) {
        const bool mask = wave == 1 && tok_base + TILE > t1;
        uint8_t *tile = wave == 0 ? kt_all[buf] : vt_all[buf];
        const int rowb = wave == 0 ? KROWB : VROWB;
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            const int row = i * Geo::LROWS + l_row;
            const bool ok = !mask || tok_base + row < t1;
            if constexpr (KT == KT_BF16) {
                *reinterpret_cast<uint4 *>(tile + row * rowb + l_chunk * 16) =
                    ok ? p.v[i] : make_uint4(0, 0, 0, 0);
            } else {
                uint4 lo = e4m3x8_to_bf16x8(make_uint2(p.v[i].x, p.v[i].y));
                uint4 hi = e4m3x8_to_bf16x8(make_uint2(p.v[i].z, p.v[i].w));
                if (!ok)
                    lo = hi = make_uint4(0, 0, 0, 0);
                *reinterpret_cast<uint4 *>(tile + row * rowb + l_chunk * 32) = lo;
                *reinterpret_cast<uint4 *>(tile + row * rowb + l_chunk * 32 + 16) = hi;
            }
        }
    };

    MultiCols<KT, D, BS, NTW, AB> cols(16 * NTW * wave, lane);

    // Both wavefronts walk the same cursors, so every branch below and the
    // barrier are uniform over the workgroup.
    BlockIds ids(a.block_tables, a.max_nb, a.max_nb, a.num_blocks, a.err_flag);
    Cursor cc = chunk.start;
    Cursor lc = cc;
    const int n = chunk.n;
    const int steps = n * HALVES;
    int l_half = 0;
    int l_id = ids.get(lc.s, lc.j);
    auto next_load = [&](int k) {
        if (k >= steps) {
            l_id = -1;
            return;
        }
        if (++l_half == HALVES) {
            l_half = 0;
            advance<BS>(lc, lens, Hkv, cap);
            l_id = ids.get(lc.s, lc.j);
        }
    };

    Part pf[DEPTH];
    int pid[DEPTH], phalf[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        if (d > 0)
            next_load(d);
        pid[d] = l_id;
        phalf[d] = l_half;
        load_part(l_id, lc.kvh, l_half, pf[d]);
    }
    for (int k0 = 0; k0 < steps; k0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int k = k0 + d;
            if (k >= steps)
                break;
            const int unit = k / HALVES;
            const int half = phalf[d], id = pid[d];
            if (half == 0 && (unit == 0 || cc.j == 0))
                cols.begin(a, cc, cc.kvh == 0 && lane == 0 && wave == 0 ? a.err_flag : nullptr);
            if (id >= 0)
                stage_part(pf[d], k & 1, cc.j * BS + half * TILE, cc.L);
            __syncthreads();
            next_load(k + DEPTH);
            pid[d] = l_id;
            phalf[d] = l_half;
            // Every part issued earlier is in before this one is issued:
            // with one part per wavefront in flight (about 8 MB over the
            // device) the verify batch streams fastest; letting all DEPTH
            // parts fly measured 6 % slower, waiting only for the oldest
            // 1.5 % slower.
            __builtin_amdgcn_s_waitcnt(kWaitVm0);
            load_part(l_id, lc.kvh, l_half, pf[d]);
            if (id >= 0)
                cols.process(a, cc, half, kt_all[k & 1], vt_all[k & 1]);
            if (half == HALVES - 1) {
                const bool ends = cc.j == cc.nb - 1;
                if (ends || unit == n - 1) {
                    const int g = cc.s * Hkv + cc.kvh;
                    if (wave == 0)
                        record_segment(a, g, w + g, cols.seg_starts, ends);
                    cols.finish(a, w + g, ends);
                }
                if (unit + 1 < n)
                    advance<BS>(cc, lens, Hkv, cap);
            }
        }
    }
}

typedef void (*DecodeKernel)(DecodeArgs);

// Tiles in flight with four column tiles (two per wavefront): three, except
// for e4m3 32-token tiles, where three would take more than 256 registers
// (one wavefront per SIMD) and two keep two.
template <int KT, int BS>
constexpr int coop_depth4()
{
    return (KT == KT_E4M3 && BS == 32) ? 2 : 3;
}

// Threads of a chunk's workgroup for nt column tiles.
int threads_for(int kv_type, int nt)
{
    return nt >= 4 || (nt == 2 && kv_type != KT_BF16) ? 64 * kCoopWaves : 64;
}

template <int KT, int D, int BS, bool AB>
DecodeKernel pick_nt(int nt)
{
    switch (nt) {
    case 1: return decode_mfma_multi_kernel<KT, D, BS, 1, AB>;
    case 2:
        if constexpr (KT == KT_BF16)
            return decode_mfma_multi_kernel<KT, D, BS, 2, AB>;
        else
            return decode_mfma_multi_coop_kernel<KT, D, BS, 1, 3, AB>;
    case 4: return decode_mfma_multi_coop_kernel<KT, D, BS, 2, coop_depth4<KT, BS>(), AB>;
    default: return nullptr;
    }
}

template <int KT, bool AB>
DecodeKernel pick_shape(int d, int bs, int nt)
{
    if (d == 64 && bs == 16) return pick_nt<KT, 64, 16, AB>(nt);
    if (d == 64 && bs == 32) return pick_nt<KT, 64, 32, AB>(nt);
    if (d == 128 && bs == 16) return pick_nt<KT, 128, 16, AB>(nt);
    if (d == 128 && bs == 32) return pick_nt<KT, 128, 32, AB>(nt);
    return nullptr;
}

DecodeKernel pick(int kv_type, int d, int bs, int nt, bool acc_bf16)
{
    if (kv_type == KT_BF16)
        return acc_bf16 ? pick_shape<KT_BF16, true>(d, bs, nt)
                        : pick_shape<KT_BF16, false>(d, bs, nt);
    if (kv_type == KT_E4M3)
        return acc_bf16 ? pick_shape<KT_E4M3, true>(d, bs, nt)
                        : pick_shape<KT_E4M3, false>(d, bs, nt);
    return nullptr;
}

}  // namespace

hipError_t launch_decode_mfma_multi(const DecodeArgs &a, int kv_type, int head_dim,
                                    int block_size, int col_tiles, hipStream_t stream)
{
    const DecodeKernel k =
        pick(kv_type, head_dim, block_size, col_tiles, (a.flags & kPartialsBf16) != 0);
    if (!k)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(k, dim3(a.num_waves), dim3(threads_for(kv_type, col_tiles)), 0, stream, a);
    return hipGetLastError();
}

hipError_t decode_mfma_multi_occupancy(int kv_type, int head_dim, int block_size, int col_tiles,
                                       bool acc_bf16, int *waves_per_cu)
{
    const DecodeKernel k = pick(kv_type, head_dim, block_size, col_tiles, acc_bf16);
    if (!k)
        return hipErrorInvalidValue;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        waves_per_cu, reinterpret_cast<const void *>(k), threads_for(kv_type, col_tiles), 0);
}

}  // namespace pa
