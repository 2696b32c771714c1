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
// one loop-invariant 32-bit offset.  Loads past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void *cache, int64_t block_bytes,
                                                             int id)
{
    const char *p = static_cast<const char *>(cache) + (int64_t)id * block_bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(p), 0, (int)block_bytes,
                                             0x00020000);
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

// Physical block ids of logical blocks [jb0, jb1) of one sequence, read 64 at
// a time by the lanes of the wavefront and handed out wave-uniformly, so the
// walk does not wait on a dependent scalar load per block.  An id outside
// [0, num_blocks) comes back as -1 and raises PA_DEVERR_BLOCK_ID.
struct BlockIds {
    const int32_t *row;
    int jb1, base, ids, num_blocks;
    uint32_t *err;

    __device__ __forceinline__ BlockIds(const int32_t *row_, int jb0, int jb1_, int nblocks,
                                        uint32_t *err_)
        : row(row_), jb1(jb1_), base(jb0), num_blocks(nblocks), err(err_)
    {
        fetch(jb0);
    }

    __device__ __forceinline__ void fetch(int j0)
    {
        base = j0;
        const int j = j0 + (int)threadIdx.x % 64;
        ids = j < jb1 ? row[j] : 0;
    }

    __device__ __forceinline__ int get(int j)
    {
        if (j - base >= 64)
            fetch(j);
        const int id = __builtin_amdgcn_readlane(ids, j - base);
        const bool bad = id < 0 || id >= num_blocks;
        if (bad)
            raise_flag(err, PA_DEVERR_BLOCK_ID);
        return __builtin_amdgcn_readfirstlane(bad ? -1 : id);
    }
};

}  // namespace pa
