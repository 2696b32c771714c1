// pa_device.h -- device-side element codecs and row loaders shared by the
// gfx950 kernels of libpa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// binary32 -> bfloat16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float x)
{
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (u >> 16) | 0x40u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// ---------------------------------------------------------------- OCP E4M3FN
// Code layout S.EEEE.MMM, exponent bias 7, no infinities, S.1111.111 = NaN,
// largest finite value 448 (S.1111.110), subnormals m * 2^-9.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c)
{
    const uint32_t e = (c >> 3) & 0xFu, m = c & 0x7u;
    float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
    if ((c & 0x7Fu) == 0x7Fu)
        mag = __uint_as_float(0x7FC00000u);
    return (c & 0x80u) ? -mag : mag;
}

// binary32 -> E4M3FN code: nearest value, ties to even mantissa; NaN -> S.1111.111;
// magnitudes >= 448 (infinity included) saturate to S.1111.110.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x)
{
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u)
        return sign | 0x7Fu;
    if (a >= 0x43E00000u)                       // 448.0f
        return sign | 0x7Eu;
    if (a >= 0x3C800000u) {                     // 2^-6: normal range of E4M3
        // round the 23-bit mantissa to 3 bits (ties to even), then rebias 127 -> 7
        const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
        return sign | ((r >> 20) - (120u << 3));
    }
    // subnormal range: count units of 2^-9; the scaling by 2^9 is exact and
    // rintf rounds half to even
    const float units = __uint_as_float(a) * 512.0f;
    return sign | (uint32_t)rintf(units);
}

// ---------------------------------------------------------------- 8-element rows
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// KV rows are read exactly once per call, so they are loaded with the
// nontemporal hint: on gfx950 this keeps the streaming gather from allocating
// in the caches, which measured ~1.6x faster than plain loads for 256-byte row
// segments of scattered blocks.
__device__ __forceinline__ uint4 stream_load16(const void *p)
{
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint2 stream_load8(const void *p)
{
    const u32x2 v = __builtin_nontemporal_load(static_cast<const u32x2 *>(p));
    return make_uint2(v.x, v.y);
}

// A lane's raw chunk of 8 consecutive elements of one row.
template <int KT> struct Raw8;
template <> struct Raw8<KT_F32> { uint4 a, b; };
template <> struct Raw8<KT_BF16> { uint4 a; };
template <> struct Raw8<KT_E4M3> { uint2 a; };

// Plain loads (q, small tensors).
template <int KT>
__device__ __forceinline__ Raw8<KT> load_raw8(const void *base, int64_t elem);

template <>
__device__ __forceinline__ Raw8<KT_F32> load_raw8<KT_F32>(const void *base, int64_t elem)
{
    const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const float *>(base) + elem);
    return Raw8<KT_F32>{p[0], p[1]};
}

template <>
__device__ __forceinline__ Raw8<KT_BF16> load_raw8<KT_BF16>(const void *base, int64_t elem)
{
    return Raw8<KT_BF16>{
        *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + elem)};
}

template <>
__device__ __forceinline__ Raw8<KT_E4M3> load_raw8<KT_E4M3>(const void *base, int64_t elem)
{
    return Raw8<KT_E4M3>{
        *reinterpret_cast<const uint2 *>(static_cast<const uint8_t *>(base) + elem)};
}

// Streaming loads of KV cache rows.
template <int KT>
__device__ __forceinline__ Raw8<KT> stream_raw8(const void *base, int64_t elem);

template <>
__device__ __forceinline__ Raw8<KT_F32> stream_raw8<KT_F32>(const void *base, int64_t elem)
{
    const float *p = static_cast<const float *>(base) + elem;
    return Raw8<KT_F32>{stream_load16(p), stream_load16(p + 4)};
}

template <>
__device__ __forceinline__ Raw8<KT_BF16> stream_raw8<KT_BF16>(const void *base, int64_t elem)
{
    return Raw8<KT_BF16>{stream_load16(static_cast<const uint16_t *>(base) + elem)};
}

template <>
__device__ __forceinline__ Raw8<KT_E4M3> stream_raw8<KT_E4M3>(const void *base, int64_t elem)
{
    return Raw8<KT_E4M3>{stream_load8(static_cast<const uint8_t *>(base) + elem)};
}

__device__ __forceinline__ void unpack8(const Raw8<KT_F32> &r, float (&x)[8])
{
    x[0] = __uint_as_float(r.a.x); x[1] = __uint_as_float(r.a.y);
    x[2] = __uint_as_float(r.a.z); x[3] = __uint_as_float(r.a.w);
    x[4] = __uint_as_float(r.b.x); x[5] = __uint_as_float(r.b.y);
    x[6] = __uint_as_float(r.b.z); x[7] = __uint_as_float(r.b.w);
}

__device__ __forceinline__ void unpack8(const Raw8<KT_BF16> &r, float (&x)[8])
{
    x[0] = bf16_lo(r.a.x); x[1] = bf16_hi(r.a.x);
    x[2] = bf16_lo(r.a.y); x[3] = bf16_hi(r.a.y);
    x[4] = bf16_lo(r.a.z); x[5] = bf16_hi(r.a.z);
    x[6] = bf16_lo(r.a.w); x[7] = bf16_hi(r.a.w);
}

__device__ __forceinline__ void unpack8(const Raw8<KT_E4M3> &r, float (&x)[8])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = e4m3_to_f32((r.a.x >> (8 * i)) & 0xFFu);
        x[4 + i] = e4m3_to_f32((r.a.y >> (8 * i)) & 0xFFu);
    }
}

// Store 8 floats as 8 elements of type OT (f32 or bf16, RNE).
template <int OT>
__device__ __forceinline__ void store8(void *base, int64_t elem, const float (&x)[8]);

template <>
__device__ __forceinline__ void store8<KT_F32>(void *base, int64_t elem, const float (&x)[8])
{
    float4 *p = reinterpret_cast<float4 *>(static_cast<float *>(base) + elem);
    p[0] = make_float4(x[0], x[1], x[2], x[3]);
    p[1] = make_float4(x[4], x[5], x[6], x[7]);
}

template <>
__device__ __forceinline__ void store8<KT_BF16>(void *base, int64_t elem, const float (&x)[8])
{
    uint4 w;
    w.x = f32_to_bf16(x[0]) | (f32_to_bf16(x[1]) << 16);
    w.y = f32_to_bf16(x[2]) | (f32_to_bf16(x[3]) << 16);
    w.z = f32_to_bf16(x[4]) | (f32_to_bf16(x[5]) << 16);
    w.w = f32_to_bf16(x[6]) | (f32_to_bf16(x[7]) << 16);
    *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(base) + elem) = w;
}

// 8 floats of a q row, f32 or bf16 storage.
template <int QT>
__device__ __forceinline__ void load_q8(const void *base, int64_t elem, float (&x)[8])
{
    if constexpr (QT == KT_F32)
        unpack8(load_raw8<KT_F32>(base, elem), x);
    else
        unpack8(load_raw8<KT_BF16>(base, elem), x);
}

__device__ __forceinline__ void raise_flag(uint32_t *flag, uint32_t bit)
{
    if (flag)
        atomicOr(flag, bit);
}

// ---------------------------------------------------------------- block walk
// Buffer resource over one pool block: the block base is wave-uniform, so the
// descriptor lives in scalar registers and every lane addresses its rows with
// one loop-invariant 32-bit offset.  Loads past the record size return zero
// without touching memory; id < 0 gives a zero-size resource, so a pipeline
// can issue the loads of a block that does not exist unconditionally (and the
// compiler can count outstanding loads exactly).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void *cache, int64_t block_bytes,
                                                             int id)
{
    const char *p = static_cast<const char *>(cache) + (int64_t)(id < 0 ? 0 : id) * block_bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(p), 0,
                                             id < 0 ? 0 : (int)block_bytes, 0x00020000);
}

// Streaming (nontemporal) buffer loads: voffset per lane, soffset uniform.
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 2);
    return make_uint2(v.x, v.y);
}

// ---------------------------------------------------------------- work list
// The decode work of a batch is the flattened list of units (s, kvh, j): for
// each sequence s, each KV head kvh, each logical block j < nb_s, with
// nb_s = ceil(min(max(L_s, 0), capacity) / bs).  Segment g = s * Hkv + kvh is
// the run of units of one (sequence, KV head).  The list is cut into chunks
// of consecutive units, one chunk per wavefront; a chunk may start or end
// inside a segment.  The partial result of chunk c for segment g goes to slot
// c + g: slots are unique (a later chunk never touches an earlier segment)
// and the slots of one segment are consecutive, [c_first + g, c_last + g].

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// v itself, as a fresh register value.  A value loaded on a rarely taken path
// and read on the common one (a block-id window refreshed every 64 blocks)
// makes the compiler wait for it on the common path as if the load were still
// outstanding; the memory-load counter retires in order, so that wait also
// drains every tile load in flight.  Passing the value through this opaque
// move right after its load puts the wait on the rare path, where it is due.
__device__ __forceinline__ int settled(int v)
{
    int r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

__device__ __forceinline__ uint4 settled(uint4 v)
{
    return make_uint4(settled((int)v.x), settled((int)v.y), settled((int)v.z), settled((int)v.w));
}

__device__ __forceinline__ int wave_sum_i(int x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x += __shfl_xor(x, off);
    return x;
}

__device__ __forceinline__ int wave_incl_scan_i(int x)
{
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off)
            x += y;
    }
    return x;
}

// Sequence lengths as the work split sees them: seq_lens[s] - off (off > 0
// for a batch viewed from a later block on, 0 otherwise).
struct Lens {
    const int32_t *p;
    int off;
    __device__ __forceinline__ int operator[](int s) const { return p[s] - off; }
    // A wave-uniform index, read through the scalar cache: its wait does not
    // drain the vector loads in flight (the lengths are never written by a
    // kernel that reads them).
    __device__ __forceinline__ int uniform(int s) const
    {
        return *(const __attribute__((address_space(4))) int32_t *)(p + s) - off;
    }
};

template <int BS>
__device__ __forceinline__ int seq_blocks(int L, int cap)
{
    L = min(L, cap);
    return L > 0 ? (L + BS - 1) / BS : 0;
}

// Units of the whole batch; raises PA_DEVERR_SEQ_LEN through `flag` (if
// non-null) when some seq_len exceeds the capacity.
template <int BS>
__device__ int64_t total_units(Lens lens, int S, int Hkv, int cap, uint32_t *flag)
{
    int64_t total = 0;
    bool over = false;
    for (int c = 0; c < S; c += 64) {
        const int s = c + lane_id();
        const int L = s < S ? lens[s] : 0;
        over |= L > cap;
        total += wave_sum_i(seq_blocks<BS>(L, cap));
    }
    if (flag && __ballot(over))
        raise_flag(flag, PA_DEVERR_SEQ_LEN);
    return total * Hkv;
}

// Position of a wavefront in the work list.
struct Cursor {
    int s, kvh, j;     // sequence, KV head, logical block
    int nb, L;         // blocks and (clamped) tokens of sequence s
};

// Cursor of unit u (< total units).
template <int BS>
__device__ Cursor locate(Lens lens, int S, int Hkv, int cap, int64_t u)
{
    int64_t base = 0;
    for (int c = 0; c < S; c += 64) {
        const int s = c + lane_id();
        const int L = s < S ? min(lens[s], cap) : 0;
        const int nb = seq_blocks<BS>(L, cap);
        const int incl = wave_incl_scan_i(nb * Hkv);
        const uint64_t hit = __ballot(base + incl > u);
        if (hit) {
            const int f = __builtin_ctzll(hit);
            Cursor cur;
            cur.s = c + f;
            cur.nb = __builtin_amdgcn_readlane(nb, f);
            cur.L = __builtin_amdgcn_readlane(L, f);
            const int64_t r = u - (base + __builtin_amdgcn_readlane(incl, f) - cur.nb * Hkv);
            cur.kvh = (int)(r / cur.nb);
            cur.j = (int)(r % cur.nb);
            return cur;
        }
        base += __builtin_amdgcn_readlane(incl, 63);
    }
    return Cursor{S, 0, 0, 0, 0};   // not reached for u < total units
}

// Next unit; only called when one exists, so a non-empty sequence lies ahead.
template <int BS>
__device__ __forceinline__ void advance(Cursor &c, Lens lens, int Hkv, int cap)
{
    if (++c.j < c.nb)
        return;
    c.j = 0;
    if (++c.kvh < Hkv)
        return;
    c.kvh = 0;
    do {
        ++c.s;
        c.L = min(lens.uniform(c.s), cap);
        c.nb = seq_blocks<BS>(c.L, cap);
    } while (c.nb == 0);
}

// Physical block id of a cursor position, wave-uniform; ids of one sequence
// are read 64 at a time by the lanes, in windows starting at multiples of 64
// (a walk that moves to the next KV head of the same sequence restarts at
// block 0, which then stays in the window), and handed out with readlane.
// An id outside [0, num_blocks) comes back as -1 and raises
// PA_DEVERR_BLOCK_ID.  Row s of the tables starts at tables + s * stride;
// max_nb entries are read.
struct BlockIds {
    const int32_t *tables;
    int stride, max_nb, num_blocks;
    uint32_t *err;
    int s = -1, base = 0, ids = 0;
    int ns = -1, nbase = 0, next = 0;

    __device__ __forceinline__ BlockIds(const int32_t *tables_, int stride_, int max_nb_,
                                        int nblocks, uint32_t *err_)
        : tables(tables_), stride(stride_), max_nb(max_nb_), num_blocks(nblocks), err(err_)
    {
    }

    __device__ __forceinline__ int get(int s_, int j)
    {
        if (s_ != s || j < base || j >= base + 64) {
            s = s_;
            base = j & ~63;
            const int jj = base + lane_id();
            ids = settled(jj < max_nb ? tables[(int64_t)s_ * stride + jj] : 0);
        }
        const int id = __builtin_amdgcn_readlane(ids, j - base);
        const bool bad = id < 0 || id >= num_blocks;
        if (bad)
            raise_flag(err, PA_DEVERR_BLOCK_ID);
        return __builtin_amdgcn_readfirstlane(bad ? -1 : id);
    }

    // get() for a walk in work-list order that also reads the walk's next
    // window ahead: the next 64 entries of the row while the sequence has
    // blocks there, else row s's first window when the next KV head needs it
    // back, else the next sequence's first window (a guess: an empty
    // sequence in between reads its window when entered).  Rows at or past
    // S are never read.
    __device__ __forceinline__ int walk(const Cursor &c, int Hkv, int S)
    {
        const int j = c.j;
        if (c.s != s || j < base || j >= base + 64) {
            const int b = j & ~63;
            const bool hit = c.s == ns && b == nbase;
            const int jj = b + lane_id();
            const int row = hit ? ns : c.s;
            ids = settled(hit ? next : (jj < max_nb ? tables[(int64_t)row * stride + jj] : 0));
            s = c.s;
            base = b;
            if (base + 64 < c.nb) {
                ns = s;
                nbase = base + 64;
            } else if (c.kvh + 1 < Hkv && base != 0) {
                ns = s;
                nbase = 0;
            } else {
                ns = s + 1;
                nbase = 0;
            }
            const int nj = nbase + lane_id();
            next = ns < S && nj < max_nb ? tables[(int64_t)ns * stride + nj] : 0;
        }
        const int id = __builtin_amdgcn_readlane(ids, j - base);
        const bool bad = id < 0 || id >= num_blocks;
        if (bad)
            raise_flag(err, PA_DEVERR_BLOCK_ID);
        return __builtin_amdgcn_readfirstlane(bad ? -1 : id);
    }
};

// BlockIds whose following 64 entries of the same table row are read one
// window ahead, so a walk along a sequence waits for the table only at its
// first block (and at a jump), not every 64 blocks.  Windows start at
// multiples of 64 as in BlockIds.
struct BlockIdsAhead {
    const int32_t *tables;
    int stride, max_nb, num_blocks;
    uint32_t *err;
    int s = -1, base = 0, ids = 0, next = 0;

    __device__ __forceinline__ BlockIdsAhead(const int32_t *tables_, int stride_, int max_nb_,
                                             int nblocks, uint32_t *err_)
        : tables(tables_), stride(stride_), max_nb(max_nb_), num_blocks(nblocks), err(err_)
    {
    }

    __device__ __forceinline__ int fetch(int s_, int j) const
    {
        const int jj = j + lane_id();
        return jj < max_nb ? tables[(int64_t)s_ * stride + jj] : 0;
    }

    __device__ __forceinline__ int get(int s_, int j)
    {
        if (s_ != s || j < base || j >= base + 64) {
            if (s_ == s && j >= base + 64 && j < base + 128) {
                ids = next;                    // the window read ahead
                base += 64;
            } else {
                s = s_;
                base = j & ~63;
                ids = fetch(s_, base);
            }
            next = fetch(s, base + 64);
        }
        const int id = __builtin_amdgcn_readlane(ids, j - base);
        const bool bad = id < 0 || id >= num_blocks;
        if (bad)
            raise_flag(err, PA_DEVERR_BLOCK_ID);
        return __builtin_amdgcn_readfirstlane(bad ? -1 : id);
    }
};

// Chunk [u0, u0 + n) of the work list for wavefront w of W (n = 0: none) and
// the cursor of its first unit.  Batches of up to 256 sequences read their
// lengths once, with independent loads, and derive both the total and the
// start position from registers; larger batches take two passes.
struct Chunk {
    int64_t u0;
    int n;
    Cursor start;
};

// Units per chunk of a work list of U units over W chunks: chunk_units, or
// (0) ceil(U / W).  runs: chunk_units > 0 names partitions, and each of the W
// chunks takes an equal run of whole partitions.
__device__ __forceinline__ int64_t chunk_len(const DecodeArgs &a, int64_t U, int W, bool runs)
{
    if (a.chunk_units <= 0)
        return (U + W - 1) / W;
    if (!runs)
        return a.chunk_units;
    const int64_t parts = (U + a.chunk_units - 1) / a.chunk_units;
    return a.chunk_units * ((parts + W - 1) / W);
}

template <int BS>
__device__ Chunk find_chunk(const DecodeArgs &a, Lens lens, int w, int W, bool runs)
{
    const int S = a.num_seqs, Hkv = a.num_kv_heads;
    const int cap = a.max_nb * BS;
    uint32_t *flag = w == 0 ? a.err_flag : nullptr;
    if (S > 256) {
        const int64_t U = total_units<BS>(lens, S, Hkv, cap, flag);
        const int64_t cl = chunk_len(a, U, W, runs);
        const int64_t u0 = (int64_t)w * cl;
        if (u0 >= U)
            return Chunk{0, 0, Cursor{}};
        return Chunk{u0, (int)min(cl, U - u0), locate<BS>(lens, S, Hkv, cap, u0)};
    }
    const int lane = lane_id();
    int L[4], nb[4], incl[4], tot[4];
    bool over = false;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int s = 64 * k + lane;
        L[k] = (64 * k < S && s < S) ? lens[s] : 0;
    }
    int64_t U = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        over |= L[k] > cap;
        L[k] = min(L[k], cap);
        nb[k] = seq_blocks<BS>(L[k], cap);
        incl[k] = wave_incl_scan_i(nb[k] * Hkv);
        tot[k] = __builtin_amdgcn_readlane(incl[k], 63);
        U += tot[k];
    }
    if (flag && __ballot(over))
        raise_flag(flag, PA_DEVERR_SEQ_LEN);
    const int64_t cl = chunk_len(a, U, W, runs);
    const int64_t u0 = (int64_t)w * cl;
    if (u0 >= U)
        return Chunk{0, 0, Cursor{}};
    Cursor cur{S, 0, 0, 0, 0};
    int64_t base = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (base + tot[k] > u0) {
            const int f = __builtin_ctzll(__ballot(base + incl[k] > u0));
            cur.s = 64 * k + f;
            cur.nb = __builtin_amdgcn_readlane(nb[k], f);
            cur.L = __builtin_amdgcn_readlane(L[k], f);
            const int64_t r = u0 - (base + __builtin_amdgcn_readlane(incl[k], f) - cur.nb * Hkv);
            cur.kvh = (int)(r / cur.nb);
            cur.j = (int)(r % cur.nb);
            break;
        }
        base += tot[k];
    }
    return Chunk{u0, (int)min(cl, U - u0), cur};
}

__device__ __forceinline__ int uniform_i(int x) { return __builtin_amdgcn_readfirstlane(x); }

// find_chunk's result, every field marked wave-uniform (it is: it derives
// from kernel arguments, block ids and cross-lane reductions).  The compiler
// cannot prove that through find_chunk's branches; without the mark the
// chunk walk's loop exits become per-lane branches, and their joins make the
// compiler wait for register tiles that are in fact complete.
template <int BS>
__device__ Chunk my_chunk(const DecodeArgs &a, Lens lens, int w, int W, bool runs = false)
{
    Chunk c = find_chunk<BS>(a, lens, w, W, runs);
    c.n = uniform_i(c.n);
    c.u0 = ((int64_t)uniform_i((int)(c.u0 >> 32)) << 32) | (uint32_t)uniform_i((int)c.u0);
    c.start.s = uniform_i(c.start.s);
    c.start.kvh = uniform_i(c.start.kvh);
    c.start.j = uniform_i(c.start.j);
    c.start.nb = uniform_i(c.start.nb);
    c.start.L = uniform_i(c.start.L);
    return c;
}

// Slot of chunk w's result for segment g, and the record the merge reads:
// seg_slots[g] = (first slot, last slot) of the segment.  The chunk that
// starts a segment writes the first entry, the one that ends it the last;
// first == last means one chunk held the whole segment and wrote the output.
__device__ __forceinline__ void record_segment(const DecodeArgs &a, int g, int slot, bool starts,
                                               bool ends)
{
    if (lane_id() != 0)
        return;
    int *rec = a.ws_seg + 2 * (int64_t)g;
    if (starts)
        rec[0] = slot;
    if (ends)
        rec[1] = slot;
}

// Query tokens of sequence s: first token and count, clamped to what the
// layout allows (0 <= qs <= qe <= T, count <= max_query_len and <= L); a
// sequence whose layout breaks the contract raises PA_DEVERR_QUERY when
// `flag` is set.  Used by the multi-token decode kernel and the merge, so both
// clamp alike.
__device__ __forceinline__ void query_span(const DecodeArgs &a, int s, int L, int *qs_out,
                                           int *ql_out, uint32_t *flag)
{
    const int qs = a.query_start_loc[s], qe = a.query_start_loc[s + 1];
    const bool bad_range = qs < 0 || qe < qs || qe > a.num_tokens;
    int ql = bad_range ? 0 : qe - qs;
    const bool too_many = ql > a.max_query_len || ql > L;
    ql = min(ql, min(a.max_query_len, L));
    if ((bad_range || too_many) && flag)
        raise_flag(flag, PA_DEVERR_QUERY);
    *qs_out = bad_range ? 0 : qs;
    *ql_out = ql;
}

}  // namespace pa
