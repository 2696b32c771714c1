// decode_mfma_wave.h -- one wavefront of paged decode attention on the gfx950
// matrix cores, for a bf16 query with a bf16 or OCP e4m3 KV cache.
//
// What is computed is the same as the vector-ALU kernel (vLLM concept page,
// "Technical principles": PagedAttention gathers the blocks named by the page
// table inside one fused kernel and runs scaled-dot-product attention over
// them; grouped-query heads share a KV head).  The work split (equal chunks
// of the batch's (sequence, KV head, block) list, one per wavefront),
// selection masking and the partial/merge contract are also the same; what
// differs is how one block of one KV head is processed by a wavefront:
//
//   loads K and V arrive in tiles of 8 KB per KV head (16 bf16 tokens, a
//         32-token bf16 block being two tiles, or 32 e4m3 tokens) through
//         16-byte row-contiguous nontemporal loads (a wavefront instruction
//         reads whole 256-byte rows; reading K directly in MFMA operand
//         order -- 16 rows x 64 bytes per instruction -- measured 15-20 %
//         slower) and are stored to LDS as bf16 rows.
//   QK^T  v_mfma_f32_16x16x32_bf16, A = K tile (M = 16 tokens, K = 32 dims)
//         read from LDS, B = Q^T (N = 16 columns; column n is query head
//         n mod G of the group).  Lane l gets S[token 4*(l/16)+i][column l%16]
//         in its 4 accumulators.
//   softmax  per column: max over the lane's 4 tokens and across the four
//         16-lane groups; running max m, lane-partial sum l, one (lazy)
//         rescale of the accumulators when some column's max grows.
//   PV    v_mfma_f32_16x16x16bf16_1k computing O^T = V^T P^T: B = P^T is
//         exactly the QK accumulator layout (converted to bf16), A = V^T is
//         read from LDS with ds_read_b64_tr_b16, which transposes 16-bit
//         elements within each 16-lane group.  A 32-token tile takes one
//         v_mfma_f32_16x16x32_bf16 per 16 dimensions instead of two.
//
// An e4m3 cache is converted to bf16 (exact) in registers before K and V are
// stored to LDS; k_scale is folded into the score scale
// and v_scale applied to the result.  Tokens at or beyond seq_len in the last
// block are excluded by selection: their scores become -inf and their V rows
// are stored to LDS as zeros, so stale NaN/Inf bits never enter an MFMA.
//
// decode_mfma_wave is the whole of a wavefront's work: its chunk of the work
// list, walked tile by tile through its own LDS tiles kt and vt (TILE * KROWB
// and TILE * VROWB bytes).  It is the body of the single-query decode kernel
// and of the cascade's suffix pass, which runs it over a batch viewed from a
// later block on: row s of the tables at a.block_tables + s * v.stride, each
// length less v.len_offset ({a.max_nb, 0} for a plain batch); v.deep asks
// for two register tiles in flight with balanced chunks (below).
//
// The single-query kernels can also do the step's append (the new token's
// K/V rows written to their slots, concept page "15-minute deep dive"): the
// wavefront that holds a segment's last position writes that KV head's new
// row to the cache and puts it into the staged tile in place of the stale
// row it loaded, so no read has to wait for the write.
#pragma once

#include "mfma_common.h"

namespace pa {

struct TableView {
    int stride, len_offset;
    bool deep = false;
};

// Partials of G <= 8 rows written by lane pairs in whole lines.
constexpr bool kPairedPartials = true;

// One wavefront's attention state for the G query heads of one KV head over
// a run of staged tiles: the Q^T operand, the fp32 accumulators, the running
// softmax base and the lane-partial sum.  begin() starts a segment (a
// sequence's KV head, or the part of it a chunk holds), attend() takes one
// tile staged in LDS, finish() writes the segment's output rows or its
// partial.  AB: partial accumulators stored as bf16 (else f32).  APP: the
// fused append is compiled in (append_row; its rows are loaded with Q).
template <int KT, int D, int BS, int G, bool AB, bool APP = false>
struct WaveAttn {
    using Geo = MfmaGeo<KT, D, BS>;
    static constexpr int NC = Geo::NC, ND = Geo::ND, TILE = Geo::TILE, MT = Geo::MT;
    static constexpr int KROWB = Geo::KROWB, VROWB = Geo::VROWB;
    static_assert(G >= 1 && G <= 16 && 16 % G == 0, "group must divide 16");

    const int g4, c16;                         // 16-lane group; token row / output column
    bf16x8 qop[NC];
    f32x4 acc[ND];
    float m = -INFINITY, l = 0.f;
    bool seg_starts = false;
    // fused append: this lane's 16 bytes of the segment's new K row (lanes
    // [0, RC)) or V row (lanes [RC, 2 RC)), and the slot it goes to.  bf16:
    // the row arrives with the last tile's own loads (load_with_row) and the
    // slot is read with Q.  e4m3 (the row must be encoded first): both are
    // read when the last tile is attended, a memory round trip per segment
    // end; loaded earlier (with Q, or right behind the last tile's loads)
    // they took registers the tile loads needed, and waits between a tile's
    // loads cut the tiles in flight to one.
    static constexpr int RC = D / 8;           // 16-byte chunks of a bf16 row
    uint4 nrow = make_uint4(0, 0, 0, 0);
    int64_t nslot = -1;

    __device__ __forceinline__ explicit WaveAttn(int lane) : g4(lane >> 4), c16(lane & 15) {}

    // Q^T operand of the segment's query rows: column c16 is query head
    // kvh*G + c16 % G; 8 dims per lane per MFMA.
    __device__ __forceinline__ void load_q(const DecodeArgs &a, const Cursor &c)
    {
        const uint16_t *qrow = static_cast<const uint16_t *>(a.q) +
                               ((int64_t)c.s * a.num_heads + c.kvh * G + (c16 % G)) * D + 8 * g4;
#pragma unroll
        for (int k = 0; k < NC; ++k)
            qop[k] = as_bf16x8(*reinterpret_cast<const uint4 *>(qrow + 32 * k));
        // The slot through the scalar cache (the kernel never writes it): a
        // vector load would have to be moved to a scalar register at once,
        // and that wait would drain the tile loads in flight.
        if (APP && KT == KT_BF16 && a.new_k)
            nslot = *(const __attribute__((address_space(4))) int64_t *)(a.new_slots + c.s);
    }

    // Empty accumulators and softmax state for a run of tiles starting at c.
    __device__ __forceinline__ void reset(const Cursor &c)
    {
#pragma unroll
        for (int d = 0; d < ND; ++d)
            acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
        m = -INFINITY;
        l = 0.f;
        seg_starts = c.j == 0;
    }

    __device__ __forceinline__ void begin(const DecodeArgs &a, const Cursor &c)
    {
        load_q(a, c);
        reset(c);
    }

    // Fused append, by the wavefront that staged the tile holding the
    // segment's last position c.L - 1 (tile tokens tok_base ..).  The new
    // rows go to cache slot nslot (e4m3: encoded as the append kernel
    // encodes them); when nslot is that position's slot (block `id`) they
    // also replace the staged rows, so the attention reads exactly what an
    // append before the decode would have left there.  (A length clamped to
    // the table makes c.L - 1 the last position the decode reads, and a row
    // appended to its slot is what that read would find.)  id < 0: the block
    // was out of range (nothing staged or replaced; the row is still
    // written).
    // append_row does the replacement (before the tile is attended) and
    // marks the segment; append_store writes the cache rows with the
    // segment's results, so a wavefront waits for its stores once per
    // segment, not twice.  A slot outside the pool, or one that is not that
    // position's, raises PA_DEVERR_SLOT (the first is not written).
    bool nmark = false;                        // this wavefront writes the segment's rows

    // the 8 values of this lane's 16 bytes of the new row, encoded as e4m3
    __device__ __forceinline__ uint2 encode_new(float inv) const
    {
        const uint32_t w[4] = {nrow.x, nrow.y, nrow.z, nrow.w};
        uint2 q = make_uint2(0, 0);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            q.x |= f32_to_e4m3(bf16_lo(w[i]) * inv) << (16 * i);
            q.x |= f32_to_e4m3(bf16_hi(w[i]) * inv) << (16 * i + 8);
            q.y |= f32_to_e4m3(bf16_lo(w[2 + i]) * inv) << (16 * i);
            q.y |= f32_to_e4m3(bf16_hi(w[2 + i]) * inv) << (16 * i + 8);
        }
        return q;
    }

    __device__ __forceinline__ void append_row(const DecodeArgs &a, uint8_t *kt, uint8_t *vt,
                                               const Cursor &c, int id, int tok_base)
    {
        const int pos = c.L - 1 - tok_base;
        if (!APP || !a.new_k || c.j != c.nb - 1 || pos < 0 || pos >= TILE)
            return;
        if constexpr (KT == KT_BF16) {
            // The tile's loads brought the new rows in at pos.  Kept when
            // nslot is that position's slot (and read back for the cache
            // store); otherwise the cache's own row goes back in (and the new
            // row, if any, is read for the store), as after a separate
            // append.  Both are rare.
            const int lane = 16 * g4 + c16, which = lane / RC, ch = lane % RC;
            nmark = nslot >= 0;
            const bool keep = id >= 0 && nslot == (int64_t)id * BS + (c.L - 1) % BS;
            if (which >= 2)
                return;
            uint8_t *row = (which ? vt + pos * VROWB : kt + pos * KROWB) + 16 * ch;
            if (keep) {
                nrow = *reinterpret_cast<const uint4 *>(row);
                return;
            }
            const int64_t hrow = ((int64_t)c.s * a.num_kv_heads + c.kvh) * D + 8 * ch;
            if (nmark)        // settled: the store at the segment's end waits for
                              // this rare load here, not on every segment
                nrow = settled(*reinterpret_cast<const uint4 *>(
                    static_cast<const uint16_t *>(which ? a.new_v : a.new_k) + hrow));
            if (id >= 0) {
                const int64_t e =
                    (((int64_t)id * BS + (c.L - 1) % BS) * a.num_kv_heads + c.kvh) * D + 8 * ch;
                *reinterpret_cast<uint4 *>(row) = *reinterpret_cast<const uint4 *>(
                    static_cast<const uint16_t *>(which ? a.value_cache : a.key_cache) + e);
            }
            return;
        }
        nslot = a.new_slots[c.s];
        if (nslot < 0)
            return;                            // nothing appended
        nmark = true;
        const int lane = 16 * g4 + c16, which = lane / RC, ch = lane % RC;
        if (which < 2)
            nrow = *reinterpret_cast<const uint4 *>(
                static_cast<const uint16_t *>(which ? a.new_v : a.new_k) +
                ((int64_t)c.s * a.num_kv_heads + c.kvh) * D + 8 * ch);
        if (id < 0 || nslot != (int64_t)id * BS + (c.L - 1) % BS || which >= 2)
            return;
        uint4 lds_row = nrow;
        if constexpr (KT == KT_E4M3)
            lds_row = e4m3x8_to_bf16x8(encode_new(which ? a.v_inv_scale : a.k_inv_scale));
        uint8_t *row = which ? vt + pos * VROWB : kt + pos * KROWB;
        *reinterpret_cast<uint4 *>(row + 16 * ch) = lds_row;
    }

    // The cache rows of a segment append_row marked (c: its cursor, id: the
    // block of its last position).
    __device__ __forceinline__ void append_store(const DecodeArgs &a, const Cursor &c, int id)
    {
        if (!APP || !nmark)
            return;
        nmark = false;
        const int64_t pool = (int64_t)a.num_blocks * BS;
        const int64_t want = id >= 0 ? (int64_t)id * BS + (c.L - 1) % BS : -1;
        if ((nslot != want || nslot >= pool) && g4 == 0 && c16 == 0)
            raise_flag(a.err_flag, PA_DEVERR_SLOT);
        const int lane = 16 * g4 + c16, which = lane / RC, ch = lane % RC;
        if (nslot >= pool || which >= 2)
            return;
        const int64_t e = (nslot * a.num_kv_heads + c.kvh) * D + 8 * ch;   // element offset
        void *cache = const_cast<void *>(which ? a.value_cache : a.key_cache);
        if constexpr (KT == KT_E4M3)
            *reinterpret_cast<uint2 *>(static_cast<uint8_t *>(cache) + e) =
                encode_new(which ? a.v_inv_scale : a.k_inv_scale);
        else
            *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(cache) + e) = nrow;
    }

    // The segment's result in partial slot `slot` (segment record too): the
    // output rows when this run of tiles covered the whole segment, else the
    // partial (m, l, acc).
    __device__ __forceinline__ void finish(const DecodeArgs &a, const Cursor &c, int slot,
                                           bool ends)
    {
        const float lt = rows_sum(l);          // sum the four 16-lane groups
        const int g = c.s * a.num_kv_heads + c.kvh;
        record_segment(a, g, slot, seg_starts, ends);
        const bool whole = seg_starts && ends && !(a.flags & kPartialOnly);
        if constexpr (kPairedPartials && G <= 8) {
            if (!whole) {
                store_partial_pairs<ND, AB, G>(a.ws_acc, (int64_t)slot * G, g4, c16, acc,
                                                   a.v_scale);
                if (g4 == 0 && c16 < G)
                    *reinterpret_cast<float2 *>(a.ws_ml + ((int64_t)slot * G + c16) * 2) =
                        make_float2(m, lt);
                return;
            }
        }
        if (c16 >= G)
            return;                            // replicated columns
        const int64_t row = (int64_t)c.s * a.num_heads + c.kvh * G + c16;
        if (whole) {
            const float inv = lt > 0.f ? a.v_scale / lt : 0.f;
            uint16_t *o = static_cast<uint16_t *>(a.out) + row * D + 4 * g4;
#pragma unroll
            for (int d = 0; d < ND; ++d)
                *reinterpret_cast<uint2 *>(o + 16 * d) =
                    make_uint2(pack_bf16x2(acc[d][0] * inv, acc[d][1] * inv),
                               pack_bf16x2(acc[d][2] * inv, acc[d][3] * inv));
        } else {
            const int64_t pi = (int64_t)slot * G + c16;
            store_partial<ND, AB>(a.ws_acc, pi, g4, acc, a.v_scale);
            if (g4 == 0)
                *reinterpret_cast<float2 *>(a.ws_ml + pi * 2) = make_float2(m, lt);
        }
    }

    // QK^T, online softmax and PV of the tile staged in kt / vt, whose first
    // token is tok_base; tokens at or beyond t1 (the sequence's length) are
    // masked by selection.
    __device__ __forceinline__ void attend(const DecodeArgs &a, const uint8_t *kt,
                                           const uint8_t *vt, int tok_base, int t1)
    {
        // S = K Q^T per 16-token sub-tile; K operand: token c16, dims 32k + 8*g4
        f32x4 sc[MT];
#pragma unroll
        for (int h = 0; h < MT; ++h) {
            sc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
            const uint8_t *krow = kt + (16 * h + c16) * KROWB + 16 * g4;
#pragma unroll
            for (int k = 0; k < NC; ++k) {
                const bf16x8 kop = as_bf16x8(*reinterpret_cast<const uint4 *>(krow + 64 * k));
                sc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[k], sc[h], 0, 0, 0);
            }
        }

        // scale; mask by selection (only a tile reaching past the sequence
        // end); tile max per column
        const bool full = tok_base + TILE <= t1;
        float bm = -INFINITY;
#pragma unroll
        for (int h = 0; h < MT; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = sc[h][i] * a.qk_scale_log2;
                if (!full)
                    v = tok_base + 16 * h + 4 * g4 + i < t1 ? v : -INFINITY;
                sc[h][i] = v;
                bm = fmaxf(bm, v);
            }
        const float tm = rows_max(bm);
        if (__ballot(tm > m + kRebase)) {
            const float mn = fmaxf(m, tm);
            const float alpha = (mn > m) ? __builtin_amdgcn_exp2f(m - mn) : 1.f;
            l *= alpha;
#pragma unroll
            for (int d = 0; d < ND; ++d)
                acc[d] *= alpha;
            m = mn;
        }

        // P = 2^(S - m), summed per lane; bf16 copy is the PV B operand.  In a
        // full tile every score is finite and m is (the first tile of a
        // segment always sets it).
        bf16x4 pop[MT];
#pragma unroll
        for (int h = 0; h < MT; ++h) {
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = (!full && sc[h][i] == -INFINITY) ? 0.f
                                                        : __builtin_amdgcn_exp2f(sc[h][i] - m);
                l += p[i];
            }
            pop[h] = __builtin_bit_cast(
                bf16x4, make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])));
        }

        // O^T += V^T P^T, V^T read transposed from LDS
        if constexpr (MT == 2) {
            // A 32-token tile in one K = 32 product per 16 dimensions: the
            // sum over tokens takes them in the order lane group g4 holds
            // them, tokens 4*g4 .. 4*g4+3 of each 16-token half, in P and in
            // the two transposed V reads alike.
            const bf16x8 pp = __builtin_shufflevector(pop[0], pop[1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int d = 0; d < ND; ++d) {
                s16x4 raw[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int row = 16 * h + 4 * g4 + (c16 >> 2);
                    raw[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4 *)((__attribute__((address_space(3))) uint8_t *)vt +
                                      row * VROWB + 32 * d + 8 * (c16 & 3)));
                }
                const bf16x8 vv = __builtin_shufflevector(as_bf16x4(raw[0]), as_bf16x4(raw[1]), 0,
                                                          1, 2, 3, 4, 5, 6, 7);
                acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pp, acc[d], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int h = 0; h < MT; ++h) {
                const int row = 16 * h + 4 * g4 + (c16 >> 2);
#pragma unroll
                for (int d = 0; d < ND; ++d) {
                    const int addr = row * VROWB + 32 * d + 8 * (c16 & 3);
                    const s16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4 *)((__attribute__((address_space(3))) uint8_t *)vt + addr));
                    acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_bf16x4(raw), pop[h],
                                                                     acc[d], 0, 0, 0);
                }
            }
        }
    }
};

// A wavefront's whole share of single-query decode: its chunk of the work list
// (balanced or fixed), walked tile by tile through its own LDS tiles kt and vt
// (TILE * KROWB and TILE * VROWB bytes).  AB, APP as WaveAttn.
template <int KT, int D, int BS, int G, bool AB, bool APP = false>
__device__ __forceinline__ void decode_mfma_wave(const DecodeArgs &a, TableView v, int w,
                                                 uint8_t *const kt, uint8_t *const vt)
{
    using Geo = MfmaGeo<KT, D, BS>;
    constexpr int TILE = Geo::TILE, HALVES = Geo::HALVES;

    const int lane = threadIdx.x & 63;
    const int Hkv = a.num_kv_heads;
    const int cap = a.max_nb * BS;

    const bool runs = (a.flags & kRuns) != 0;
    const Lens lens{a.seq_lens, v.len_offset};
    const Chunk chunk = my_chunk<BS>(a, lens, w, a.num_waves, runs);
    if (chunk.n == 0)
        return;

    // Register tiles in flight while a tile is computed: two for a chunk of
    // one fixed partition (short chunks, many rounds of wavefronts or a small
    // batch: the second tile shortens each chunk's start) and for a deep view
    // (the cascade's suffix pass: a small batch, where start-up dominates);
    // one for balanced chunks and longer runs of partitions.  One tile per
    // wavefront puts about 8 MB in flight at one wavefront per SIMD, and that
    // streams fastest: two measured 6 % slower on the Llama-shaped batch and
    // 2 % on the Qwen-shaped one (3 % faster on the shared-prefix suffix
    // pass).
    const bool pingpong = v.deep || (a.chunk_units > 0 && chunk.n <= a.chunk_units);

    const MfmaLoader<Geo> loader(a, lane);
    using Tile = MfmaTile<Geo>;
    WaveAttn<KT, D, BS, G, AB, APP> att(lane);

    // Walk the chunk tile by tile: the load cursor runs one tile ahead of the
    // compute cursor, across block and segment boundaries.
    BlockIds ids(a.block_tables, v.stride, a.max_nb, a.num_blocks, a.err_flag);
    Cursor cc = chunk.start;
    Cursor lc = cc;

    // Tile loads at the load cursor; with a bf16 append inside, a segment's
    // last tile brings the new rows in place of the cache's at its last
    // position.
    auto load_tile = [&](int id, int kvh, int half, Tile &t) {
        if constexpr (APP && KT == KT_BF16) {
            int rpos = lc.L - 1 - (lc.j * BS + half * TILE);
            if (!a.new_k || lc.j != lc.nb - 1 || rpos >= TILE)
                rpos = -1;
            // Plain loads on every other tile: the per-lane address select
            // on each tile cost the Llama-shaped kernel 2 % at one wavefront
            // per SIMD.
            if (rpos < 0) {
                loader.load(id, kvh, half, t);
            } else {
                const int64_t r = ((int64_t)lc.s * Hkv + lc.kvh) * D * 2;
                load_with_row<Geo>(loader, id, kvh, half, t, rpos,
                                   static_cast<const char *>(a.new_k) + r,
                                   static_cast<const char *>(a.new_v) + r);
            }
        } else {
            loader.load(id, kvh, half, t);
        }
    };
    const int n = chunk.n;                     // units (blocks)
    const int steps = n * HALVES;              // tiles

    // next_load moves the load cursor to tile `k`; past the chunk's last tile
    // it yields no block (id -1), whose loads read nothing.
    int l_half = 0;
    // The cascade's suffix view (short segments, many sequence changes per
    // chunk) reads the walk's next table window ahead; plain decode reads a
    // window when the walk enters it (the read-ahead measured 0.3 % slower on
    // the Qwen-shaped batch and equal on the Llama-shaped one).
    auto block_id = [&](const Cursor &c) {
        return v.deep ? ids.walk(c, Hkv, a.num_seqs) : ids.get(c.s, c.j);
    };
    int l_id = block_id(lc);
    auto next_load = [&](int k) {
        if (k >= steps) {
            l_id = -1;
            return;
        }
        if (++l_half == HALVES) {
            l_half = 0;
            advance<BS>(lc, lens, Hkv, cap);
            l_id = block_id(lc);
        }
    };

    // A tile's segment is started (its query rows loaded) before the loads of
    // the following tile are issued: loads retire in order, so query loads
    // issued after them would make the tile wait for the following one.
    auto pre_step = [&](int k, int half) {
        const int unit = k / HALVES;
        if (half == 0 && (unit == 0 || cc.j == 0))
            att.begin(a, cc);
    };
    auto step = [&](int k, int id, int half, const Tile &t, auto issue_next) {
        const int unit = k / HALVES;
        const int tok_base = cc.j * BS + half * TILE;
        // Stage as bf16, V rows past the sequence end as zeros.  A missing
        // block (id < 0, block 0 read) is staged too and never attended:
        // staging on every path is what tells the compiler that this
        // register tile's loads are done, so the next loads into it do not
        // wait for the other tile's.
        stage_tile<Geo>(loader, kt, vt, t, tok_base, cc.L);
        issue_next();
        // after the next tile's loads: the append waits for the rows loaded
        // with Q, as the attention does
        att.append_row(a, kt, vt, cc, id, tok_base);
        if (id >= 0)
            att.attend(a, kt, vt, tok_base, cc.L);
        if (half == HALVES - 1) {
            const bool ends = cc.j == cc.nb - 1;
            if (ends || unit == n - 1) {
                att.append_store(a, cc, id);
                att.finish(a, cc, w + cc.s * Hkv + cc.kvh, ends);
            }
            if (unit + 1 < n)
                advance<BS>(cc, lens, Hkv, cap);
        }
    };

    // Loads are issued unconditionally (a missing block reads block 0), so the
    // wait before staging a tile counts exactly the loads issued after it.
    if (pingpong) {
        // Two register tiles: tile k+1 is loaded into the other tile before
        // tile k is waited on, so two tiles are in flight at the wait.  The
        // loop takes whole pairs and an odd last tile follows it: an exit
        // from the middle of the loop body would reach the loop's back edge
        // in the compiler's view with the second tile still loading, and it
        // would then wait for that tile at every pair.
        Tile ta, tb;
        int ida = l_id, ha = l_half;
        load_tile(ida, lc.kvh, ha, ta);
        int k = 0;
        for (; k + 1 < steps; k += 2) {
            pre_step(k, ha);
            next_load(k + 1);
            const int idb = l_id, hb = l_half;
            load_tile(idb, lc.kvh, hb, tb);
            step(k, ida, ha, ta, [] {});
            pre_step(k + 1, hb);
            next_load(k + 2);
            ida = l_id;
            ha = l_half;
            load_tile(ida, lc.kvh, ha, ta);
            step(k + 1, idb, hb, tb, [] {});
        }
        if (k < steps) {
            pre_step(k, ha);
            step(k, ida, ha, ta, [] {});
        }
    } else {
        // One register tile: tile k is staged into LDS, then the loads of tile
        // k+1 are issued into the same registers and stay in flight while
        // tile k is computed from LDS.
        Tile t;
        int id = l_id, half = l_half;
        load_tile(id, lc.kvh, half, t);
        for (int k = 0; k < steps; ++k) {
            int id_next = -1, half_next = 0;
            pre_step(k, half);
            step(k, id, half, t, [&] {
                next_load(k + 1);
                id_next = l_id;
                half_next = l_half;
                load_tile(id_next, lc.kvh, half_next, t);
            });
            id = id_next;
            half = half_next;
        }
    }
}

}  // namespace pa
