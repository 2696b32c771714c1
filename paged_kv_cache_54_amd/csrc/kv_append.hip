// kv_append.hip -- the KV-append scatter: each new token's key and value rows
// go into the block slot named by slot_mapping (vLLM concept page, "15-minute
// deep dive": blocks are allocated on demand at write time; the same page names
// the pack/unpack kernels that move KV rows into the block layout).
//
// Layout facts used: a slot s = block * bs + offset of the pool
// [NB, bs, Hkv, D] starts at element s * Hkv * D, and a token's [Hkv, D] row is
// contiguous both in k/v and in the cache, so the scatter is a row copy to a
// computed address.  One thread moves one 8-element chunk (16 B of bf16,
// 32 B of f32 in, 8 B of e4m3 out), so a wavefront covers 512 consecutive
// elements of a row: fully coalesced on both sides.
#include "pa_device.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

// Store one loaded 8-element chunk at element d of the cache (quantised to
// e4m3 with the inverse scale `inv` for an fp8 cache, else copied).
template <int IT, int CT>
__device__ __forceinline__ void store8(const Raw8<IT> &r, void *dst, int64_t d, float inv)
{
    if constexpr (CT == KT_E4M3) {
        float x[8];
        unpack8(r, x);
        uint2 w;
        w.x = w.y = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w.x |= f32_to_e4m3(x[i] * inv) << (8 * i);
            w.y |= f32_to_e4m3(x[4 + i] * inv) << (8 * i);
        }
        *reinterpret_cast<uint2 *>(static_cast<uint8_t *>(dst) + d) = w;
    } else if constexpr (CT == KT_F32) {
        uint4 *p = reinterpret_cast<uint4 *>(static_cast<float *>(dst) + d);
        p[0] = r.a;
        p[1] = r.b;
    } else {
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(dst) + d) = r.a;
    }
}

template <int IT, int CT>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(AppendArgs a)
{
    const int64_t chunks = a.row_elems / 8;     // per token
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= a.num_tokens * chunks)
        return;
    const int64_t t = idx / chunks, c = idx - t * chunks;
    // The rows are read before the slot is known: the three loads do not
    // depend on each other, so they share one memory latency.
    const int64_t s = t * a.row_elems + c * 8;
    const Raw8<IT> k = load_raw8<IT>(a.k, s);
    const Raw8<IT> v = load_raw8<IT>(a.v, s);
    const int64_t slot = a.slots[t];
    if (slot < 0)
        return;                                  // padding token
    if (slot >= a.num_slots) {
        if (c == 0)
            raise_flag(a.err_flag, PA_DEVERR_SLOT);
        return;
    }
    const int64_t d = slot * a.row_elems + c * 8;
    store8<IT, CT>(k, a.key_cache, d, a.k_inv_scale);
    store8<IT, CT>(v, a.value_cache, d, a.v_inv_scale);
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs &a, int in_type, int cache_type, hipStream_t stream)
{
    const int64_t threads = a.num_tokens * (a.row_elems / 8);
    const int64_t blocks = (threads + kThreads - 1) / kThreads;
    if (blocks > INT32_MAX)
        return hipErrorInvalidValue;
    dim3 grid((unsigned)blocks), block(kThreads);
    if (cache_type == KT_F32 && in_type == KT_F32)
        hipLaunchKernelGGL((kv_append_kernel<KT_F32, KT_F32>), grid, block, 0, stream, a);
    else if (cache_type == KT_BF16 && in_type == KT_BF16)
        hipLaunchKernelGGL((kv_append_kernel<KT_BF16, KT_BF16>), grid, block, 0, stream, a);
    else if (cache_type == KT_E4M3 && in_type == KT_BF16)
        hipLaunchKernelGGL((kv_append_kernel<KT_BF16, KT_E4M3>), grid, block, 0, stream, a);
    else if (cache_type == KT_E4M3 && in_type == KT_F32)
        hipLaunchKernelGGL((kv_append_kernel<KT_F32, KT_E4M3>), grid, block, 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pa
