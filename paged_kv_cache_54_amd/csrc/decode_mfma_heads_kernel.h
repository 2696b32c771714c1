// decode_mfma_heads_kernel.h -- single-query paged decode on the gfx950 matrix
// cores for an OCP e4m3 cache, with the KV heads of a block read together.
//
// What is computed is the single-query decode of decode_mfma_wave.h (vLLM
// concept page, "Technical principles": the blocks named by the page table
// are gathered inside one fused kernel and attended with scaled dot-product
// attention; a KV head serves its group of query heads).  What differs is the
// work unit and the read order.  The per-wavefront kernel walks (sequence,
// KV head, block) units, so one KV head's rows of a block -- 128 bytes per
// token at head_dim 128 -- are read apart from the other heads' rows of the
// same token slots.  With that order a block's 1 KB token slots are fetched
// as eight strided streams; reading the same bytes with every head of a
// block together (each load instruction a contiguous 1 KB) measured 25-30 %
// faster on the 131072-token batch (a read-only probe: 431 against 317-324
// us for the 2 GiB of K and V).
//
// Here a workgroup has one wavefront per KV head (HK = num_kv_heads) and
// walks (sequence, block) units.  For each block the HK wavefronts load its K
// and V tiles as 1 KB pieces (piece i * HK + w to wavefront w), convert them
// to bf16 and store each row's head slices into that head's LDS tiles; after
// a barrier wavefront w attends head w's tiles with WaveAttn, the same
// per-head state, operand layout and online softmax as the per-wavefront
// kernel.  A second barrier keeps the next block's staging from overwriting
// tiles still being read; the next block's loads are issued between the two,
// so they are in flight while the current block is attended.
//
// Work split: the (sequence, block) list is cut into partitions -- equal
// ones, one per resident workgroup, or fixed ones of chunk_units blocks --
// and each workgroup walks one contiguous run of them (with fixed partitions,
// an equal run per workgroup of a grid no larger than the device holds at
// once: the same read pattern as the balanced split).  A wavefront carries its
// softmax state across the partition boundaries inside its run, so a segment
// leaves one partial per run that touches it, not one per partition: the
// log-sum-exp merge is associative, and a run that holds a whole segment
// writes the output itself.  Head w of run c writes the partial of segment
// (s, w) to slot (c + s) * HK + w: distinct over all (c, s, w), as runs hold
// non-decreasing sequences, and the slots of one segment step by HK from the
// first run touching it to the last (the merge's slot stride).
//
// decode_mfma_heads.hip instantiates the plain kernels and launches them;
// decode_mfma_heads_append.hip the ones that also do the step's append
// (APP), apart for the same reason as decode_mfma_kernel.h's.
#pragma once

#include "decode_mfma_wave.h"

namespace pa {
namespace heads_kernel {

// Cooperative load geometry: a tile is TILE token slots of SB bytes (all HK
// heads), read as 1 KB pieces; PPR token slots per piece.
template <int KT, int D, int BS, int HK>
struct HeadsGeo {
    using Geo = MfmaGeo<KT, D, BS>;
    static_assert(KT == KT_E4M3 && Geo::HALVES == 1, "e4m3 tiles are whole blocks");
    static constexpr int TILE = Geo::TILE;
    static constexpr int HB = D * Geo::EB;                // bytes of one head's row
    static constexpr int SB = HK * HB;                    // bytes of one token slot
    static_assert(SB <= 1024 && 1024 % SB == 0, "a 1 KB piece holds whole slots");
    static constexpr int PPR = 1024 / SB;                 // slots per piece
    static constexpr int PIECES = TILE * SB / 1024;       // pieces per tensor tile
    static_assert(PIECES % HK == 0, "pieces split evenly over the wavefronts");
    static constexpr int NL = PIECES / HK;                // pieces per wavefront and tensor
    static constexpr int KTB = TILE * Geo::KROWB;         // one head's LDS K tile
    static constexpr int VTB = TILE * Geo::VROWB;
    static constexpr int LDS = HK * (KTB + VTB);
};

// APP: the step's append compiled in.
template <int KT, int D, int BS, int G, bool AB, int HK, bool APP>
__global__ __launch_bounds__(64 * HK) void decode_mfma_heads_kernel(DecodeArgs a)
{
    using HG = HeadsGeo<KT, D, BS, HK>;
    using Geo = MfmaGeo<KT, D, BS>;
    constexpr int NL = HG::NL;
    __shared__ __attribute__((aligned(16))) uint8_t lds[HG::LDS];

    const int lane = threadIdx.x & 63;
    const int kvh = threadIdx.x >> 6;                     // this wavefront's KV head
    const int c = blockIdx.x;
    const int cap = a.max_nb * BS;

    // the work list of (sequence, block) units: one KV head in the split's view
    DecodeArgs u = a;
    u.num_kv_heads = 1;
    const Lens lens{a.seq_lens, 0};
    const Chunk chunk = my_chunk<BS>(u, lens, c, (int)gridDim.x, true);
    if (chunk.n == 0)
        return;                                           // uniform over the workgroup
    const int n = chunk.n;

    // This lane's 16 bytes of piece i * HK + kvh: token slot row_i, head hd,
    // bytes 16 * ch .. of that head's row.
    const int lo = lane * 16;
    const int row0 = kvh * HG::PPR + lo / HG::SB;         // + i * HK * PPR
    const int hd = (lo % HG::SB) / HG::HB;
    const int ch = (lo % HG::HB) / 16;
    const int64_t block_bytes = (int64_t)BS * HG::SB;
    const char *kbase = static_cast<const char *>(a.key_cache) + kvh * 1024 + lo;
    const char *vbase = static_cast<const char *>(a.value_cache) + kvh * 1024 + lo;
    uint8_t *const kt_w = lds + hd * HG::KTB + ch * 32;   // this lane's LDS columns
    uint8_t *const vt_w = lds + HK * HG::KTB + hd * HG::VTB + ch * 32;
    uint8_t *const kt = lds + kvh * HG::KTB;              // the tiles this wavefront attends
    uint8_t *const vt = lds + HK * HG::KTB + kvh * HG::VTB;

    uint4 tk[NL], tv[NL];
    // A missing block (id < 0) reads block 0 -- in bounds, never staged.
    auto load = [&](int id) {
        const int64_t off = (int64_t)(id < 0 ? 0 : id) * block_bytes;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const u32x4 x = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(kbase + off + (int64_t)i * HK * 1024));
            const u32x4 y = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(vbase + off + (int64_t)i * HK * 1024));
            tk[i] = make_uint4(x.x, x.y, x.z, x.w);
            tv[i] = make_uint4(y.x, y.y, y.z, y.w);
        }
    };
    // bf16 rows into the heads' tiles; V rows at or beyond t1 as zeros
    auto stage = [&](int tok_base, int t1) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int row = row0 + i * HK * HG::PPR;
            const uint4 k0 = e4m3x8_to_bf16x8(make_uint2(tk[i].x, tk[i].y));
            const uint4 k1 = e4m3x8_to_bf16x8(make_uint2(tk[i].z, tk[i].w));
            uint4 v0 = e4m3x8_to_bf16x8(make_uint2(tv[i].x, tv[i].y));
            uint4 v1 = e4m3x8_to_bf16x8(make_uint2(tv[i].z, tv[i].w));
            if (tok_base + row >= t1)
                v0 = v1 = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4 *>(kt_w + row * Geo::KROWB) = k0;
            *reinterpret_cast<uint4 *>(kt_w + row * Geo::KROWB + 16) = k1;
            *reinterpret_cast<uint4 *>(vt_w + row * Geo::VROWB) = v0;
            *reinterpret_cast<uint4 *>(vt_w + row * Geo::VROWB + 16) = v1;
        }
    };

    WaveAttn<KT, D, BS, G, AB, APP> att(lane);
    BlockIdsAhead ids(a.block_tables, a.max_nb, a.max_nb, a.num_blocks, a.err_flag);
    Cursor cc = chunk.start;                              // compute cursor (kvh 0)
    Cursor lc = cc;                                       // load cursor, one unit ahead
    int id = ids.get(lc.s, lc.j);
    load(id);
    for (int k = 0; k < n; ++k) {
        Cursor hc = cc;
        hc.kvh = kvh;
        // A segment's query rows are loaded before the next block's loads
        // (loads retire in order).
        if (k == 0 || cc.j == 0)
            att.begin(a, hc);
        const int tok_base = cc.j * BS;
        __syncthreads();                                  // previous tiles fully read
        if (id >= 0)
            stage(tok_base, cc.L);
        int id_next = -1;
        if (k + 1 < n) {
            advance<BS>(lc, lens, 1, cap);
            id_next = ids.get(lc.s, lc.j);
        }
        load(id_next);
        __syncthreads();                                  // tiles staged
        // a fused append's row replaces this head's staged one (after the
        // barrier: every wavefront staged some of this head's rows)
        att.append_row(a, kt, vt, hc, id, tok_base);
        if (id >= 0)
            att.attend(a, kt, vt, tok_base, cc.L);
        const bool ends = cc.j == cc.nb - 1;
        if (ends || k == n - 1) {
            att.append_store(a, hc, id);
            att.finish(a, hc, (c + cc.s) * HK + kvh, ends);
        }
        if (k + 1 < n)
            advance<BS>(cc, lens, 1, cap);
        id = id_next;
    }
}

typedef void (*HeadsKernel)(DecodeArgs);

template <int D, int BS, bool AB, int HK, bool APP>
HeadsKernel pick_g(int group)
{
    switch (group) {
    case 1: return decode_mfma_heads_kernel<KT_E4M3, D, BS, 1, AB, HK, APP>;
    case 2: return decode_mfma_heads_kernel<KT_E4M3, D, BS, 2, AB, HK, APP>;
    case 4: return decode_mfma_heads_kernel<KT_E4M3, D, BS, 4, AB, HK, APP>;
    case 8: return decode_mfma_heads_kernel<KT_E4M3, D, BS, 8, AB, HK, APP>;
    default: return nullptr;
    }
}

template <bool AB, int HK, bool APP>
HeadsKernel pick_bs(int bs, int group)
{
    if (bs == 16) return pick_g<128, 16, AB, HK, APP>(group);
    if (bs == 32) return pick_g<128, 32, AB, HK, APP>(group);
    return nullptr;
}

template <int HK, bool APP>
HeadsKernel pick_ab(int bs, int group, bool acc_bf16)
{
    return acc_bf16 ? pick_bs<true, HK, APP>(bs, group) : pick_bs<false, HK, APP>(bs, group);
}

template <bool APP>
HeadsKernel pick(int kv_type, int d, int bs, int group, int hk, bool acc_bf16)
{
    if (kv_type != KT_E4M3 || d != 128)
        return nullptr;
    if (hk == 4)
        return pick_ab<4, APP>(bs, group, acc_bf16);
    if (hk == 8)
        return pick_ab<8, APP>(bs, group, acc_bf16);
    return nullptr;
}

}  // namespace heads_kernel

// The append-carrying instance (decode_mfma_heads_append.hip).
heads_kernel::HeadsKernel decode_mfma_heads_append_kernel(int kv_type, int d, int bs, int group,
                                                          int hk, bool acc_bf16);

}  // namespace pa
