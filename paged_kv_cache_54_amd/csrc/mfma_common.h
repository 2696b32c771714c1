// mfma_common.h -- pieces shared by the gfx950 matrix-core decode kernels
// (one query token per sequence, and several): operand types, e4m3 -> bf16
// conversion, the tile geometry, the buffer loads of a KV tile and its staging
// into LDS as bf16 rows.
#pragma once

#include <type_traits>

#include "pa_device.h"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v)
{
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x4 as_bf16x4(s16x4 v)
{
    return __builtin_bit_cast(bf16x4, v);
}

// Two e4m3 codes (byte pair HI of w) -> two packed bf16, in one gfx950
// instruction (v_cvt_scalef32_pk_bf16_fp8; a scale of 1.0 scales by 2^0).
// Every e4m3 value, subnormals included, has an exact bf16 encoding; over all
// 65,536 byte pairs this gives the same bits as converting to binary32 and
// keeping the upper halves (v_cvt_pk_f32_fp8 + v_perm, two instructions).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 v)
{
    return make_uint4(e4m3x2_to_bf16x2<false>(v.x), e4m3x2_to_bf16x2<true>(v.x),
                      e4m3x2_to_bf16x2<false>(v.y), e4m3x2_to_bf16x2<true>(v.y));
}

// Two floats -> packed bf16 pair with the hardware converter (v_cvt_pk_bf16_f32,
// round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Store one column's unnormalised partial accumulator row `row` of a
// workspace whose rows are D = 16 * ND values: lane group g4 holds dims
// 16 * d + 4 * g4 .. + 3 of the MFMA output in acc[d].  Each value is
// multiplied by `scale` in place (the caller's accumulators are dead after
// the store; scaling in place needs no extra registers), then stored as f32
// (16-byte stores) or, with BF16, rounded to nearest even bf16.  The storage
// type is a template parameter of the kernels: a run-time choice between the
// two stores cost registers (the two-wavefront verify kernel fell to one
// wavefront per SIMD).
template <int ND, bool BF16>
__device__ __forceinline__ void store_partial(void *ws_acc, int64_t row, int g4,
                                              f32x4 (&acc)[ND], float scale)
{
    constexpr int D = 16 * ND;
#pragma unroll
    for (int d = 0; d < ND; ++d)
        acc[d] *= scale;
    if constexpr (BF16) {
        uint16_t *o = static_cast<uint16_t *>(ws_acc) + row * D + 4 * g4;
#pragma unroll
        for (int d = 0; d < ND; ++d)
            *reinterpret_cast<uint2 *>(o + 16 * d) =
                make_uint2(pack_bf16x2(acc[d][0], acc[d][1]), pack_bf16x2(acc[d][2], acc[d][3]));
    } else {
        float *o = static_cast<float *>(ws_acc) + row * D + 4 * g4;
#pragma unroll
        for (int d = 0; d < ND; ++d)
            *reinterpret_cast<f32x4 *>(o + 16 * d) = acc[d];
    }
}

// store_partial for the single-query kernels' output layout with G <= 8
// query heads per KV head: lanes c16 and c16 + 8 hold the same column
// (c16 mod G), so the pair writes two consecutive 16-dimension slices of row
// r = c16 & 7 in one instruction -- lane c16 slice 2p, lane c16 + 8 slice
// 2p + 1 -- and every store covers whole 128-byte lines of a row (f32)
// instead of their halves, in half as many instructions.  Rows r >= G store
// nothing.
template <int ND, bool BF16, int G>
__device__ __forceinline__ void store_partial_pairs(void *ws_acc, int64_t slot_row0, int g4,
                                                    int c16, f32x4 (&acc)[ND], float scale)
{
    static_assert(G <= 8 && ND % 2 == 0, "pairs need replicated columns");
    constexpr int D = 16 * ND;
    const int r = c16 & 7, hi = c16 >> 3;
    if (r >= G)
        return;
#pragma unroll
    for (int d = 0; d < ND; ++d)
        acc[d] *= scale;
    const int64_t base = (slot_row0 + r) * D + 4 * g4 + 16 * hi;
#pragma unroll
    for (int p = 0; p < ND / 2; ++p) {
        const f32x4 v = hi ? acc[2 * p + 1] : acc[2 * p];
        if constexpr (BF16) {
            u32x2 *o = reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(ws_acc) + base + 32 * p);
            *o = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        } else {
            *reinterpret_cast<f32x4 *>(static_cast<float *>(ws_acc) + base + 32 * p) = v;
        }
    }
}

// Max and sum over the four 16-lane rows (lanes c, c + 16, c + 32, c + 48):
// gfx950's row-swap permutes exchange rows 0<->1, 2<->3 (16-lane swap) and
// the two halves (32-lane swap) on the vector ALU, with no LDS round trip.
// Called with the same register twice, each swap returns the lane's own row
// in one result and its partner row in the other, so every lane ends with
// the same value.
__device__ __forceinline__ float rows_max(float x)
{
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float x)
{
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Online softmax with a lazily moved base: a column's running base m (log2
// units) moves to a new maximum only when some column's tile maximum exceeds
// it by more than kRebase, so most tiles skip rescaling the accumulators.
// The unnormalised weights 2^(s - m) then stay below 2^kRebase; the base
// cancels in the final acc / l, and a partial's (m, l, acc) stays
// consistent for the log-sum-exp merge.
constexpr float kRebase = 8.0f;

// Tile geometry of one KV head's rows for a cache of element type KT.
template <int KT_, int D_, int BS_>
struct MfmaGeo {
    static constexpr int KT = KT_, D = D_, BS = BS_;
    static constexpr int EB = (KT == KT_BF16) ? 2 : 1;
    static constexpr int NC = D / 32;          // QK MFMAs per 16 tokens
    static constexpr int ND = D / 16;          // PV MFMAs (16 output dims each) per 16 tokens
    // A tile is 8 KB of one KV head (K and V): 16 bf16 or 32 e4m3 tokens,
    // never more than a block; MT 16-token MFMA tiles, BS/TILE tiles a block.
    static constexpr int TILE = (32 / EB < BS) ? 32 / EB : BS;
    static constexpr int MT = TILE / 16;
    static constexpr int HALVES = BS / TILE;
    static constexpr int RCH = D * EB / 16;    // 16-byte chunks of one cache row
    static constexpr int LROWS = 64 / RCH;     // rows one load instruction covers
    static constexpr int NLOAD = TILE / LROWS; // load instructions per tile and tensor
    // K and V tiles in LDS as bf16 rows of D elements plus padding, chosen so
    // that each read pattern touches distinct banks: K operand reads take 16
    // bytes from 16 consecutive rows (rows 4 banks apart: 16-byte pad), the
    // transposed V reads take 32 bytes from 4 consecutive rows per 16 lanes
    // (rows 8 banks apart: 32-byte pad).  Every address is a per-lane base
    // plus a constant.
    static constexpr int KROWB = 2 * D + 16;
    static constexpr int VROWB = 2 * D + 32;
};

template <class Geo>
struct MfmaTile {
    uint4 k[Geo::NLOAD];
    uint4 v[Geo::NLOAD];
};

// Row-contiguous loads of a tile: load instruction i reads row
// i * LROWS + lane / RCH, 16-byte chunk lane % RCH, of both tensors, as
// nontemporal global loads from the block's address (measured 0.2-1.1 %
// faster than buffer loads through a per-block resource on the decode
// batches).  A missing block (id < 0) reads block 0 instead -- in bounds,
// and the caller never attends that tile -- so the loads can still be issued
// unconditionally.
template <class Geo>
struct MfmaLoader {
    const void *key_cache, *value_cache;
    int slot_bytes;
    int64_t block_bytes;
    int l_row, l_chunk, l_voff;

    __device__ __forceinline__ MfmaLoader(const DecodeArgs &a, int lane)
        : key_cache(a.key_cache), value_cache(a.value_cache),
          slot_bytes(a.num_kv_heads * Geo::D * Geo::EB),
          block_bytes((int64_t)Geo::BS * a.num_kv_heads * Geo::D * Geo::EB),
          l_row(lane / Geo::RCH), l_chunk(lane % Geo::RCH),
          l_voff((lane / Geo::RCH) * a.num_kv_heads * Geo::D * Geo::EB + (lane % Geo::RCH) * 16)
    {
    }

    // tile `half` (tokens TILE*half ..) of block `id`, KV head kvh
    __device__ __forceinline__ void load(int id, int kvh, int half, MfmaTile<Geo> &t) const
    {
        const int64_t base = (int64_t)(id < 0 ? 0 : id) * block_bytes + l_voff +
                             kvh * Geo::D * Geo::EB + half * Geo::TILE * slot_bytes;
        const u32x4 *pk =
            reinterpret_cast<const u32x4 *>(static_cast<const char *>(key_cache) + base);
        const u32x4 *pv =
            reinterpret_cast<const u32x4 *>(static_cast<const char *>(value_cache) + base);
        const int step = Geo::LROWS * slot_bytes / 16;   // in 16-byte units
#pragma unroll
        for (int i = 0; i < Geo::NLOAD; ++i) {
            const u32x4 a = __builtin_nontemporal_load(pk + i * step);
            const u32x4 b = __builtin_nontemporal_load(pv + i * step);
            t.k[i] = make_uint4(a.x, a.y, a.z, a.w);
            t.v[i] = make_uint4(b.x, b.y, b.z, b.w);
        }
    }
};

// Loads of a bf16 tile as MfmaLoader::load, except that the row at tile
// position rpos (if 0 <= rpos < TILE) comes from the bf16 rows nk / nv (D
// elements each; this lane reads its chunk) instead of the cache: the new
// token's rows of a step whose append the decode kernel does, brought in by
// the tile's own load instructions (no extra load, no wait).  Used for a
// segment's last tile only (rpos < 0: none replaced); other tiles take the
// plain loads, since the per-lane select on every tile cost 2 %.
template <class Geo>
__device__ __forceinline__ void load_with_row(const MfmaLoader<Geo> &ld, int id, int kvh, int half,
                                              MfmaTile<Geo> &t, int rpos, const char *nk,
                                              const char *nv)
{
    static_assert(Geo::KT == KT_BF16, "the new rows are bf16, as the cache rows");
    const int64_t base = (int64_t)(id < 0 ? 0 : id) * ld.block_bytes + ld.l_voff +
                         kvh * Geo::D * Geo::EB + half * Geo::TILE * ld.slot_bytes;
    const char *pk = static_cast<const char *>(ld.key_cache) + base;
    const char *pv = static_cast<const char *>(ld.value_cache) + base;
    const int step = Geo::LROWS * ld.slot_bytes;
    const bool mine = rpos >= 0 && ld.l_row == rpos % Geo::LROWS;   // this lane: the new row
#pragma unroll
    for (int i = 0; i < Geo::NLOAD; ++i) {
        const char *ak = pk + i * step, *av = pv + i * step;
        if (mine && i == rpos / Geo::LROWS) {
            ak = nk + ld.l_chunk * 16;
            av = nv + ld.l_chunk * 16;
        }
        const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ak));
        const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(av));
        t.k[i] = make_uint4(a.x, a.y, a.z, a.w);
        t.v[i] = make_uint4(b.x, b.y, b.z, b.w);
    }
}

// Store one tensor's rows into an LDS tile (row stride ROWB) as bf16; with
// MASK, rows whose token is at or beyond t1 are stored as zeros.
template <class Geo, int ROWB, bool MASK>
__device__ __forceinline__ void store_rows(const MfmaLoader<Geo> &ld, uint8_t *tile,
                                           const uint4 (&src)[Geo::NLOAD], int tok_base, int t1)
{
#pragma unroll
    for (int i = 0; i < Geo::NLOAD; ++i) {
        const int row = i * Geo::LROWS + ld.l_row;
        const bool ok = !MASK || (tok_base + row < t1);
        if constexpr (Geo::KT == KT_BF16) {
            uint4 v = src[i];
            if (MASK && !ok)
                v = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4 *>(tile + row * ROWB + ld.l_chunk * 16) = v;
        } else {
            uint4 lo = e4m3x8_to_bf16x8(make_uint2(src[i].x, src[i].y));
            uint4 hi = e4m3x8_to_bf16x8(make_uint2(src[i].z, src[i].w));
            if (MASK && !ok)
                lo = hi = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4 *>(tile + row * ROWB + ld.l_chunk * 32) = lo;
            *reinterpret_cast<uint4 *>(tile + row * ROWB + ld.l_chunk * 32 + 16) = hi;
        }
    }
}

// Stage a tile whose first token is tok_base into the K and V LDS tiles; V
// rows at or beyond t1 (the sequence length) become zeros, so stale NaN/Inf
// bits past the end never enter an MFMA (K rows there only produce scores
// that the kernels replace by -inf).
template <class Geo>
__device__ __forceinline__ void stage_tile(const MfmaLoader<Geo> &ld, uint8_t *kt, uint8_t *vt,
                                           const MfmaTile<Geo> &t, int tok_base, int t1)
{
    store_rows<Geo, Geo::KROWB, false>(ld, kt, t.k, tok_base, t1);
    if (tok_base + Geo::TILE > t1)
        store_rows<Geo, Geo::VROWB, true>(ld, vt, t.v, tok_base, t1);
    else
        store_rows<Geo, Geo::VROWB, false>(ld, vt, t.v, tok_base, t1);
}

}  // namespace pa
