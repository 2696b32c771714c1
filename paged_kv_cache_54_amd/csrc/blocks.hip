// blocks.hip -- whole-block maintenance of paged KV caches: clearing newly
// allocated blocks, and copying blocks between pools.
//
// Clearing (vLLM v0.17.1 release notes, fix #35219): a block that another
// layer type used before may hold bit patterns that read as NaN/Inf in the
// cache dtype, so blocks handed to attention layers are cleared on the GPU
// before use, all caches in one batched launch over precomputed per-cache
// block addresses, with the block ids handed to the GPU through pinned memory
// so that no host-device synchronisation is needed.  Copying: a shared prefix
// block is duplicated before a sequence writes into it (copy-on-write, vLLM
// internals blog, section 1), and a preempted sequence's blocks move between
// the GPU pool and a host pool (swap out / swap in, vLLM concept page,
// "15-minute deep dive", scheduler item).
//
// Both are pure data movement, bound by HBM write (clear) or read + write
// (copy) bandwidth.  A "region" is one cache (say the K cache of one layer):
// block b of region r occupies bytes [base_r + b * stride, + bytes).  The
// work is the list (item group, region, 16 KiB chunk); one 256-thread
// workgroup clears or copies one chunk of every block of its item group in
// one region, four 16-byte stores per thread per chunk: plain stores when
// clearing, nontemporal loads and stores when copying (each measured the
// faster of the two for its operation).
// The item group's ids are read once per workgroup with one coalesced load
// (they may live in host memory) and kept in LDS.
//
// For large operations whose id and base tables are in device memory, a
// second kernel is used: one 256-thread workgroup per (item, region, 4 KiB
// piece), one 16-byte store (clear) or nontemporal load and store (copy) per
// thread, the id and base read once per workgroup, 32-bit index arithmetic
// (its per-workgroup cost shows: 64-bit divisions made it 11 % slower).
// Many short workgroups keep more stores in flight than looping ones: on a
// 1 GiB buffer this pattern wrote 6.7 TB/s where 16-byte stores in a loop per
// workgroup reached 5.0-5.5 TB/s, and copied 6.7 TB/s (read + write) against
// 5.6-6.0.  Tables in host memory keep the grouped kernel, which reads each
// id from host memory once.
#include "pa_device.h"

namespace pa {
namespace {

constexpr int kBlockThreads = 256;
constexpr int kChunkBytes = kBlockThreads * 4 * 16;   // 16 KiB per workgroup pass

__device__ __forceinline__ void store_nt16(void *p, uint4 v)
{
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, static_cast<u32x4 *>(p));
}

template <bool COPY>
__global__ __launch_bounds__(kBlockThreads) void block_op_kernel(BlockOpArgs a)
{
    __shared__ int32_t src_ids[kMaxGroupItems];
    __shared__ int32_t dst_ids[kMaxGroupItems];

    const int t = threadIdx.x;
    const int64_t wg = blockIdx.x;
    const int64_t chunk = wg % a.chunks;
    const int64_t region = (wg / a.chunks) % a.num_regions;
    const int64_t group = wg / (a.chunks * a.num_regions);
    const int64_t i0 = group * a.group_items;
    const int n = (int)min((int64_t)a.group_items, a.num_items - i0);

    // the group's ids: one coalesced read; invalid ids become -1
    if (t < n) {
        int32_t d, s = 0;
        if constexpr (COPY) {
            const int2 pr = reinterpret_cast<const int2 *>(a.ids)[i0 + t];
            s = pr.x;
            d = pr.y;
        } else {
            d = a.ids[i0 + t];
        }
        const bool bad = d < 0 || d >= a.dst_num_blocks ||
                         (COPY && (s < 0 || s >= a.src_num_blocks));
        if (bad && region == 0 && chunk == 0)
            raise_flag(a.err_flag, PA_DEVERR_BLOCK_ID);
        dst_ids[t] = bad ? -1 : d;
        src_ids[t] = bad ? -1 : s;
    }
    uint8_t *dst = static_cast<uint8_t *>(a.dst_bases[region]);
    const uint8_t *src = COPY ? static_cast<const uint8_t *>(a.src_bases[region]) : nullptr;
    __syncthreads();

    const bool bad_region = dst == nullptr || (reinterpret_cast<uintptr_t>(dst) & 15) ||
                            (COPY && (src == nullptr || (reinterpret_cast<uintptr_t>(src) & 15)));
    if (bad_region) {
        if (t == 0 && group == 0 && chunk == 0)
            raise_flag(a.err_flag, PA_DEVERR_REGION);
        return;
    }

    const int64_t c0 = chunk * kChunkBytes;
    for (int i = 0; i < n; ++i) {
        const int32_t d = dst_ids[i];
        if (d < 0)
            continue;
        uint8_t *db = dst + (int64_t)d * a.block_stride + c0;
        if constexpr (COPY) {
            const uint8_t *sb = src + (int64_t)src_ids[i] * a.block_stride + c0;
            uint4 v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t off = (int64_t)(k * kBlockThreads + t) * 16;
                if (c0 + off < a.block_bytes)
                    v[k] = stream_load16(sb + off);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t off = (int64_t)(k * kBlockThreads + t) * 16;
                if (c0 + off < a.block_bytes)
                    store_nt16(db + off, v[k]);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t off = (int64_t)(k * kBlockThreads + t) * 16;
                if (c0 + off < a.block_bytes)
                    *reinterpret_cast<uint4 *>(db + off) = make_uint4(0, 0, 0, 0);
            }
        }
    }
}

constexpr int kPieceBytes = kBlockThreads * 16;   // 4 KiB per workgroup

template <bool COPY>
__global__ __launch_bounds__(kBlockThreads) void block_piece_kernel(BlockOpArgs a)
{
    const int t = threadIdx.x;
    const uint32_t wg = blockIdx.x;
    const uint32_t rest = wg / (uint32_t)a.pieces;
    const int piece = (int)(wg - rest * (uint32_t)a.pieces);
    const uint32_t item32 = rest / (uint32_t)a.num_regions;
    const int region = (int)(rest - item32 * (uint32_t)a.num_regions);
    const int64_t item = item32;

    int32_t d, s = 0;
    if constexpr (COPY) {
        const int2 pr = reinterpret_cast<const int2 *>(a.ids)[item];
        s = pr.x;
        d = pr.y;
    } else {
        d = a.ids[item];
    }
    if (d < 0 || d >= a.dst_num_blocks || (COPY && (s < 0 || s >= a.src_num_blocks))) {
        if (t == 0 && region == 0 && piece == 0)
            raise_flag(a.err_flag, PA_DEVERR_BLOCK_ID);
        return;
    }
    uint8_t *dst = static_cast<uint8_t *>(a.dst_bases[region]);
    const uint8_t *src = COPY ? static_cast<const uint8_t *>(a.src_bases[region]) : nullptr;
    if (dst == nullptr || (reinterpret_cast<uintptr_t>(dst) & 15) ||
        (COPY && (src == nullptr || (reinterpret_cast<uintptr_t>(src) & 15)))) {
        if (t == 0 && item == 0 && piece == 0)
            raise_flag(a.err_flag, PA_DEVERR_REGION);
        return;
    }
    const int64_t off = (int64_t)piece * kPieceBytes + t * 16;
    if (off >= a.block_bytes)
        return;
    uint8_t *db = dst + (int64_t)d * a.block_stride + off;
    if constexpr (COPY)
        store_nt16(db, stream_load16(src + (int64_t)s * a.block_stride + off));
    else
        *reinterpret_cast<uint4 *>(db) = make_uint4(0, 0, 0, 0);
}

}  // namespace

int64_t block_op_chunk_bytes() { return kChunkBytes; }
int64_t block_op_piece_bytes() { return kPieceBytes; }

hipError_t launch_block_piece_op(const BlockOpArgs &a, bool copy, hipStream_t stream)
{
    const int64_t wgs = a.num_items * a.num_regions * a.pieces;
    if (wgs <= 0 || wgs > INT32_MAX)
        return hipErrorInvalidValue;
    dim3 grid((unsigned)wgs), block(kBlockThreads);
    if (copy)
        hipLaunchKernelGGL(block_piece_kernel<true>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(block_piece_kernel<false>, grid, block, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_block_op(const BlockOpArgs &a, bool copy, hipStream_t stream)
{
    const int64_t groups = (a.num_items + a.group_items - 1) / a.group_items;
    const int64_t wgs = groups * a.num_regions * a.chunks;
    if (wgs <= 0 || wgs > INT32_MAX || a.group_items > kMaxGroupItems)
        return hipErrorInvalidValue;
    dim3 grid((unsigned)wgs), block(kBlockThreads);
    if (copy)
        hipLaunchKernelGGL(block_op_kernel<true>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(block_op_kernel<false>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace pa
