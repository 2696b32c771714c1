// cascade.hip -- decode for a batch whose sequences share a prefix of whole
// blocks (the shared-prefix case of the vLLM internals blog, section 1: a
// common prompt is one set of physical blocks that every sequence's table
// names).  Plain decode reads the shared blocks once per sequence; here the
// attention is split at the prefix boundary (log-sum-exp makes the split
// exact):
//
//   prefix pass  every query row of a KV head against the shared blocks:
//                a dense attention of R = S * G rows over N * bs tokens,
//                cut into (KV head, token split, row block) workgroups whose
//                four wavefronts share each K/V tile through LDS;
//   suffix pass  each sequence against its own blocks from the prefix on:
//                the single-query decode wavefronts over the batch viewed
//                from block N on (table column and length offsets), partials
//                only;
//   merge        per (sequence, head): log-sum-exp over both passes' parts.
//
// The two passes share one launch: the prefix workgroups come first in the
// grid (one per compute unit or so, bound by issue and latency), then a few
// that check the contract, then the suffix pass's (bound by memory), so the
// prefix pass runs in the shadow of the suffix pass instead of before it.
// (Running them as two kernels on two streams cost more in the cross-stream
// waits than the overlap saved.)  The merge is a second kernel.
#include "decode_mfma_wave.h"

namespace pa {
namespace {

constexpr int kPrefixWaves = 4;     // wavefronts per prefix workgroup
constexpr int kPrefixColTiles = 1;  // 16-row column tiles per wavefront
constexpr int kPrefixDepth = 4;     // tiles in flight per workgroup
constexpr int kThreads = 256;
constexpr int kSuffixWaves = kThreads / 64;   // suffix-pass wavefronts per workgroup
static_assert(kPrefixWaves * 64 == kThreads, "a prefix item takes a whole workgroup");

// The contract: every table starts with row 0's prefix and every sequence
// covers it.  Workgroup wg of nwg.
__device__ void check_contract(const CascadePrefixArgs &a, int wg, int nwg)
{
    const int N = a.prefix_blocks, S = a.num_seqs;
    const int64_t n_chk = (int64_t)S * N;
    const int64_t total = n_chk + S;
    const int cap = a.max_nb * a.block_size;
    for (int64_t e = (int64_t)wg * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)nwg * blockDim.x) {
        int64_t x = e;
        if (x < n_chk) {
            const int64_t s = x / N, j = x % N;
            if (a.block_tables[s * a.max_nb + j] != a.block_tables[j])
                raise_flag(a.err_flag, PA_DEVERR_PREFIX);
            continue;
        }
        x -= n_chk;
        if (min(a.seq_lens[x], cap) < N * a.block_size)
            raise_flag(a.err_flag, PA_DEVERR_PREFIX);
    }
}

// One K or V row chunk of a tile into its LDS tile as bf16 (e4m3 converted
// exactly).
template <class Geo, int ROWB>
__device__ __forceinline__ void stage_chunk(uint8_t *tile, int row, int chunk, uint4 v)
{
    if constexpr (Geo::KT == KT_BF16) {
        *reinterpret_cast<uint4 *>(tile + row * ROWB + chunk * 16) = v;
    } else {
        *reinterpret_cast<uint4 *>(tile + row * ROWB + chunk * 32) =
            e4m3x8_to_bf16x8(make_uint2(v.x, v.y));
        *reinterpret_cast<uint4 *>(tile + row * ROWB + chunk * 32 + 16) =
            e4m3x8_to_bf16x8(make_uint2(v.z, v.w));
    }
}

// Prefix pass, one work item.  Workgroup = four wavefronts over RB = 4 * 16 *
// NTW query rows; wavefront w owns rows w * 16 * NTW .. of the block as NTW
// MFMA column tiles.  The 2 * NLOAD load instructions of a tile (K rows, then
// V rows) are dealt round-robin to the wavefronts; each tile is staged into
// one of two LDS buffers (kt0/vt0 + buffer * tile bytes) and, after a
// barrier, read by all four.  DEPTH tiles are in flight in registers.  Every
// prefix token is valid (the contract), so no masking.
template <int KT, int D, int BS, int NTW, bool AB>
__device__ __forceinline__ void prefix_item(const CascadePrefixArgs &a, int item, uint8_t *kt0,
                                            uint8_t *vt0)
{
    using Geo = MfmaGeo<KT, D, BS>;
    constexpr int NC = Geo::NC, ND = Geo::ND, TILE = Geo::TILE, MT = Geo::MT;
    constexpr int HALVES = Geo::HALVES, NLOAD = Geo::NLOAD;
    constexpr int KROWB = Geo::KROWB, VROWB = Geo::VROWB;
    constexpr int NQ = 2 * NLOAD;                                   // load instructions per tile
    constexpr int NPW = (NQ + kPrefixWaves - 1) / kPrefixWaves;      // ... per wavefront
    constexpr int DEPTH = kPrefixDepth;
    constexpr int RB = kPrefixWaves * 16 * NTW;

    auto kt_buf = [&](int buf) { return kt0 + buf * (TILE * KROWB); };
    auto vt_buf = [&](int buf) { return vt0 + buf * (TILE * VROWB); };

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar selects
    const int lane = threadIdx.x & 63;
    const int g4 = lane >> 4, c16 = lane & 15;

    const int Hkv = a.num_kv_heads, H = a.num_heads, lg = a.log2_group;
    const int rb = item % a.row_blocks;
    const int pair = item / a.row_blocks;
    const int split = pair % a.num_splits, kvh = pair / a.num_splits;
    const int j0 = split * a.split_blocks;
    const int nblk = min(a.prefix_blocks - j0, a.split_blocks);
    const int ntiles = nblk * HALVES;

    // loads: this wavefront's instructions u -> q = wave + 4u
    const int slot_bytes = Hkv * D * Geo::EB;
    const int64_t block_bytes = (int64_t)BS * slot_bytes;
    const int l_row = lane / Geo::RCH, l_chunk = lane % Geo::RCH;
    const int voff = l_row * slot_bytes + l_chunk * 16 + kvh * D * Geo::EB;
    // block ids of the split (at most 64 blocks), checked once; a bad id
    // reads zeros
    int my_ids = lane < nblk ? a.block_tables[j0 + lane] : 0;
    const bool bad = lane < nblk && (my_ids < 0 || my_ids >= a.num_blocks);
    if (bad)
        my_ids = -1;
    if (__ballot(bad) && wave == 0 && lane == 0)
        raise_flag(a.err_flag, PA_DEVERR_BLOCK_ID);
    struct Part {
        uint4 v[NPW];
    };
    // Every load is issued unconditionally (tiles past the split through a
    // zero-size resource), so the compiler counts the loads in flight exactly
    // and each stage waits for its own tile only.
    auto block_id = [&](int t) {
        const int id = __builtin_amdgcn_readlane(my_ids, min(t / HALVES, 63));
        return __builtin_amdgcn_readfirstlane(t >= ntiles ? -1 : id);
    };
    auto load = [&](int t, Part &p) {
        const int id = block_id(t);
        const int soff = (t % HALVES) * TILE * slot_bytes;
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
            const int q = wave + kPrefixWaves * u;
            const bool is_v = q >= NLOAD;
            const int i = is_v ? q - NLOAD : q;
            const __amdgpu_buffer_rsrc_t r = block_rsrc(is_v ? a.value_cache : a.key_cache,
                                                        block_bytes, q < NQ ? id : -1);
            p.v[u] = buf_load16(r, voff, soff + i * Geo::LROWS * slot_bytes);
        }
    };
    auto stage = [&](const Part &p, int buf) {
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
            const int q = wave + kPrefixWaves * u;
            if (q < NLOAD)
                stage_chunk<Geo, KROWB>(kt_buf(buf), q * Geo::LROWS + l_row, l_chunk, p.v[u]);
            else if (q < NQ)
                stage_chunk<Geo, VROWB>(vt_buf(buf), (q - NLOAD) * Geo::LROWS + l_row, l_chunk,
                                        p.v[u]);
        }
    };

    // query operands of this wavefront's rows (rows past R are zeros)
    const int R = a.rows;
    const int row0 = rb * RB + wave * 16 * NTW;
    bf16x8 qop[NTW][NC];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const int r = row0 + 16 * nt + c16;
        const bool valid = r < R;
        const int rr = valid ? r : 0;
        const int s = rr >> lg, g = rr & ((1 << lg) - 1);
        const uint16_t *qrow = static_cast<const uint16_t *>(a.q) +
                               ((int64_t)s * H + kvh * (1 << lg) + g) * D + 8 * g4;
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const uint4 v = *reinterpret_cast<const uint4 *>(qrow + 32 * k);
            qop[nt][k] = as_bf16x8(valid ? v : make_uint4(0, 0, 0, 0));
        }
    }

    // Tile loads after the query loads (the first tile's wait covers the
    // queries), in tile order: the loop waits for tile t with every later
    // tile's loads still in flight.
    Part pf[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        load(d, pf[d]);
        __builtin_amdgcn_sched_barrier(0);
    }

    f32x4 acc[NTW][ND];
    float m[NTW], l[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
        for (int d = 0; d < ND; ++d)
            acc[nt][d] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[nt] = -INFINITY;
        l[nt] = 0.f;
    }

    // One tile from LDS: every K and Vt operand read is issued first, so the
    // reads' latencies overlap each other and the QK products and softmax.
    auto process = [&](int buf) {
        const uint8_t *kt = kt_buf(buf);
        const uint8_t *vt = vt_buf(buf);
        bf16x8 kop[MT][NC];
        s16x4 vop[MT][ND];
#pragma unroll
        for (int h = 0; h < MT; ++h) {
            const uint8_t *krow = kt + (16 * h + c16) * KROWB + 16 * g4;
#pragma unroll
            for (int k = 0; k < NC; ++k)
                kop[h][k] = as_bf16x8(*reinterpret_cast<const uint4 *>(krow + 64 * k));
        }
#pragma unroll
        for (int h = 0; h < MT; ++h) {
            const int row = 16 * h + 4 * g4 + (c16 >> 2);
#pragma unroll
            for (int d = 0; d < ND; ++d)
                vop[h][d] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)((__attribute__((address_space(3))) uint8_t *)vt + row * VROWB +
                                  32 * d + 8 * (c16 & 3)));
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4 sc[MT][NTW];
#pragma unroll
        for (int h = 0; h < MT; ++h)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                sc[h][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < NC; ++k)
                    sc[h][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[h][k], qop[nt][k],
                                                                      sc[h][nt], 0, 0, 0);
            }
        bf16x4 pop[MT][NTW];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            float bm = -INFINITY;
#pragma unroll
            for (int h = 0; h < MT; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sc[h][nt][i] *= a.qk_scale_log2;
                    bm = fmaxf(bm, sc[h][nt][i]);
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
                    p[i] = __builtin_amdgcn_exp2f(sc[h][nt][i] - m[nt]);
                    l[nt] += p[i];
                }
                pop[h][nt] = __builtin_bit_cast(
                    bf16x4, make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])));
            }
        }
#pragma unroll
        for (int h = 0; h < MT; ++h)
#pragma unroll
            for (int d = 0; d < ND; ++d)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
                    acc[nt][d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                        as_bf16x4(vop[h][d]), pop[h][nt], acc[nt][d], 0, 0, 0);
    };

    // Tile t: stage from registers into buffer t & 1, barrier, refill the
    // registers with tile t + DEPTH, compute from LDS.  Buffer t & 1 was last
    // read by tile t - 2, which every wavefront finished before the barrier
    // of tile t - 1.
    for (int t0 = 0; t0 < ntiles; t0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int t = t0 + d;
            const bool live = t < ntiles;
            if (live)
                stage(pf[d], t & 1);
            __syncthreads();
            load(t + DEPTH, pf[d]);
            if (live)
                process(t & 1);
        }
    }

    // partials of the valid rows
    const int64_t pbase = ((int64_t)split * Hkv + kvh) * R;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const float lt = rows_sum(l[nt]);
        const int r = row0 + 16 * nt + c16;
        if (r >= R)
            continue;
        store_partial<ND, AB>(a.p_acc, pbase + r, g4, acc[nt], a.v_scale);
        if (g4 == 0)
            *reinterpret_cast<float2 *>(a.p_ml + (pbase + r) * 2) = make_float2(m[nt], lt);
    }
}

// Both passes in one launch.  Workgroups [0, 8 * items_per_xcd) take the
// prefix items: workgroups are dispatched round-robin over the 8 XCDs, and
// consecutive items -- the row blocks of one (KV head, split), which read the
// same tiles -- go to workgroups of one XCD, so the tiles come from its L2
// after the first read.  The next check_wgs check the contract; the rest run
// four suffix-pass wavefronts each.  LDS holds a prefix item's two K and two
// V tile buffers, or one K and one V tile per suffix wavefront.
//
// Register use sets how many suffix workgroups share a compute unit with a
// prefix workgroup.  The bf16, 128-dimension, 16-token-block kernel needs
// about 180 registers per lane, which allows two wavefronts per SIMD (one
// suffix workgroup per compute unit); held to 168 it fits three without
// spilling, and the suffix pass gets twice the wavefronts.  (Other shapes
// either fit three or more already or spill at 168.)
template <int KT, int D, int BS>
constexpr int cascade_waves_per_simd()
{
    return (KT == KT_BF16 && D == 128 && BS == 16) ? 3 : 1;
}

// AB: partial accumulators (prefix and suffix) stored as bf16, else f32.
template <int KT, int D, int BS, int NTW, int G, bool AB>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(cascade_waves_per_simd<KT, D, BS>()))) void cascade_kernel(
    CascadePrefixArgs p, DecodeArgs s)
{
    using Geo = MfmaGeo<KT, D, BS>;
    constexpr int KTILE = Geo::TILE * Geo::KROWB, VTILE = Geo::TILE * Geo::VROWB;
    static_assert(kSuffixWaves >= 2, "a prefix item takes two buffers of each");
    __shared__ __attribute__((aligned(16))) uint8_t lds[kSuffixWaves * (KTILE + VTILE)];
    uint8_t *const vt0 = lds + kSuffixWaves * KTILE;

    int wg = blockIdx.x;
    const int item_wgs = 8 * p.items_per_xcd;
    if (wg < item_wgs) {
        const int item = (wg & 7) * p.items_per_xcd + (wg >> 3);
        if (item < p.num_items)
            prefix_item<KT, D, BS, NTW, AB>(p, item, lds, vt0);
        return;
    }
    wg -= item_wgs;
    if (wg < p.check_wgs) {
        check_contract(p, wg, p.check_wgs);
        return;
    }
    wg -= p.check_wgs;
    const int wave = threadIdx.x >> 6;
    // wavefronts past s.num_waves get no chunk
    const TableView view{p.max_nb, p.prefix_blocks * p.block_size, true};
    decode_mfma_wave<KT, D, BS, G, AB>(s, view, wg * kSuffixWaves + wave, lds + wave * KTILE,
                                   vt0 + wave * VTILE);
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

// Fold parts [first, last] of one partial source (part stride rps rows, row
// prow; accumulators f32, or bf16 with ACC_BF16) into st; the lanes' groups
// take parts p0, p0 + step, ...
template <int D, bool ACC_BF16>
__device__ __forceinline__ void add_parts(Lse &st, const void *acc_ws, const float *ml_ws,
                                          int first, int last, int64_t rps, int64_t prow, int col,
                                          int p0, int step)
{
    const float2 *ml = reinterpret_cast<const float2 *>(ml_ws) + (int64_t)first * rps + prow;
    const int64_t acc0 = ((int64_t)first * rps + prow) * D + col;
    const int n = last - first + 1;
    auto acc_at = [&](int p) {
        const int64_t e = acc0 + (int64_t)p * rps * D;
        if constexpr (ACC_BF16) {
            const uint2 v = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(acc_ws) + e);
            return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                               __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
        } else {
            return *reinterpret_cast<const float4 *>(static_cast<const float *>(acc_ws) + e);
        }
    };
    for (int p = p0; p < n; p += 2 * step) {
        float2 m0 = make_float2(-INFINITY, 0.f), m1 = m0;
        float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
        m0 = ml[(int64_t)p * rps];
        x0 = acc_at(p);
        if (p + step < n) {
            m1 = ml[(int64_t)(p + step) * rps];
            x1 = acc_at(p + step);
        }
        lse_add(st, m0.x, m0.y, x0);
        lse_add(st, m1.x, m1.y, x1);
    }
}

// One wavefront per (sequence, head) row, four rows per workgroup.
template <int OT, bool ACC_BF16, int D>
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

    // The length and the suffix's segment record are loaded together, and the
    // prefix parts (which need neither) are folded in first, so their loads
    // overlap those two.  A sequence with no own tokens has no record this
    // call; its stale one is read and not used.  A record outside the
    // workspace's slots (never written so by the suffix pass) is not
    // followed.
    const int2 rec = *reinterpret_cast<const int2 *>(a.s_seg + 2 * (s * Hkv + kvh));
    const int L = a.seq_lens[s];
    Lse st{-INFINITY, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
    {                                            // the shared prefix: one part per split
        const int64_t R = (int64_t)a.num_seqs * G;
        add_parts<D, ACC_BF16>(st, a.p_acc, a.p_ml, 0, a.num_splits - 1, Hkv * R,
                     kvh * R + (int64_t)s * G + h % G, col, sub, PPW);
    }
    if (min(L, a.capacity) > a.prefix_tokens && rec.x >= 0 && rec.y >= rec.x &&
        rec.y < a.num_slots)                     // the sequence's own blocks
        add_parts<D, ACC_BF16>(st, a.s_acc, a.s_ml, rec.x, rec.y, G, h % G, col, sub, PPW);
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

typedef void (*CascadeKernel)(CascadePrefixArgs, DecodeArgs);

template <int KT, int D, int BS, bool AB>
CascadeKernel pick_g(int group)
{
    switch (group) {
    case 1: return cascade_kernel<KT, D, BS, kPrefixColTiles, 1, AB>;
    case 2: return cascade_kernel<KT, D, BS, kPrefixColTiles, 2, AB>;
    case 4: return cascade_kernel<KT, D, BS, kPrefixColTiles, 4, AB>;
    case 8: return cascade_kernel<KT, D, BS, kPrefixColTiles, 8, AB>;
    default: return nullptr;
    }
}

template <int KT, bool AB>
CascadeKernel pick_shape(int d, int bs, int group)
{
    if (d == 64 && bs == 16) return pick_g<KT, 64, 16, AB>(group);
    if (d == 64 && bs == 32) return pick_g<KT, 64, 32, AB>(group);
    if (d == 128 && bs == 16) return pick_g<KT, 128, 16, AB>(group);
    if (d == 128 && bs == 32) return pick_g<KT, 128, 32, AB>(group);
    return nullptr;
}

CascadeKernel pick(int kv_type, int d, int bs, int group, bool acc_bf16)
{
    if (kv_type == KT_BF16)
        return acc_bf16 ? pick_shape<KT_BF16, true>(d, bs, group)
                        : pick_shape<KT_BF16, false>(d, bs, group);
    if (kv_type == KT_E4M3)
        return acc_bf16 ? pick_shape<KT_E4M3, true>(d, bs, group)
                        : pick_shape<KT_E4M3, false>(d, bs, group);
    return nullptr;
}

}  // namespace

int cascade_prefix_rows() { return kPrefixWaves * 16 * kPrefixColTiles; }

hipError_t cascade_suffix_occupancy(int kv_type, int head_dim, int block_size, int group,
                                    bool acc_bf16, int *waves_per_cu)
{
    const CascadeKernel k = pick(kv_type, head_dim, block_size, group, acc_bf16);
    if (!k)
        return hipErrorInvalidValue;
    int wgs = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &wgs, reinterpret_cast<const void *>(k), kThreads, 0);
    *waves_per_cu = (wgs > 1 ? wgs - 1 : 1) * kSuffixWaves;
    return e;
}

hipError_t launch_cascade(const CascadePrefixArgs &p, const DecodeArgs &s, int kv_type,
                          int head_dim, int block_size, int group, hipStream_t stream)
{
    const CascadeKernel k = pick(kv_type, head_dim, block_size, group, p.partials_bf16 != 0);
    if (!k)
        return hipErrorInvalidValue;
    // item workgroups, those for the contract check (about 1k elements
    // each), then the suffix pass's
    CascadePrefixArgs args = p;
    const int64_t check = (int64_t)p.num_seqs * (p.prefix_blocks + 1);
    int64_t check_wgs = (check + 4 * kThreads - 1) / (4 * kThreads);
    args.check_wgs = (int32_t)(check_wgs < 1 ? 1 : (check_wgs > 256 ? 256 : check_wgs));
    const int64_t wgs = 8 * (int64_t)p.items_per_xcd + args.check_wgs +
                        ((int64_t)s.num_waves + kSuffixWaves - 1) / kSuffixWaves;
    if (wgs > INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(k, dim3((unsigned)wgs), dim3(kThreads), 0, stream, args, s);
    return hipGetLastError();
}

hipError_t launch_cascade_merge(const CascadeMergeArgs &a, int out_type, int head_dim,
                                hipStream_t stream)
{
    const int64_t rows = (int64_t)a.num_seqs * a.num_heads;
    dim3 grid((unsigned)((rows + 3) / 4)), block(kThreads);
    if (out_type != KT_BF16)
        return hipErrorInvalidValue;
    if (head_dim == 64 && a.partials_bf16)
        hipLaunchKernelGGL((cascade_merge_kernel<KT_BF16, true, 64>), grid, block, 0, stream, a);
    else if (head_dim == 64)
        hipLaunchKernelGGL((cascade_merge_kernel<KT_BF16, false, 64>), grid, block, 0, stream, a);
    else if (head_dim == 128 && a.partials_bf16)
        hipLaunchKernelGGL((cascade_merge_kernel<KT_BF16, true, 128>), grid, block, 0, stream, a);
    else if (head_dim == 128)
        hipLaunchKernelGGL((cascade_merge_kernel<KT_BF16, false, 128>), grid, block, 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pa
