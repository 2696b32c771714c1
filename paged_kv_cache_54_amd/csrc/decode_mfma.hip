// decode_mfma.hip -- the single-query paged decode kernel on the gfx950
// matrix cores (bf16 query, bf16 or OCP e4m3 KV cache): workgroups of
// kWavesPerGroup independent wavefronts, each running decode_mfma_wave over
// its own chunk of the batch's (sequence, KV head, block) list with its own
// LDS tiles.
#include "decode_mfma_wave.h"

namespace pa {
namespace {

// Wavefronts per workgroup.  Each wavefront walks its own chunk with its own
// LDS tiles.  Two per workgroup measured ~1.3 % faster than one on the Llama-
// and Qwen-shaped batches when every resident wavefront had a chunk, and the
// same as one with the bf16 split over half of them; four were slower in both
// cases (9 % at half), eight no better.
constexpr int kWavesPerGroup = 2;

template <int KT, int D, int BS, int G, bool AB>
__global__ __launch_bounds__(64 * kWavesPerGroup) void decode_mfma_kernel(DecodeArgs a)
{
    using Geo = MfmaGeo<KT, D, BS>;
    __shared__ __attribute__((aligned(16))) uint8_t kt_all[kWavesPerGroup][Geo::TILE * Geo::KROWB];
    __shared__ __attribute__((aligned(16))) uint8_t vt_all[kWavesPerGroup][Geo::TILE * Geo::VROWB];
    const int wave = threadIdx.x >> 6;
    // wavefronts past a.num_waves get no chunk
    decode_mfma_wave<KT, D, BS, G, AB>(a, TableView{a.max_nb, 0},
                                       blockIdx.x * kWavesPerGroup + wave, kt_all[wave],
                                       vt_all[wave]);
}

typedef void (*DecodeKernel)(DecodeArgs);

template <int KT, int D, int BS, bool AB>
DecodeKernel pick_g(int group)
{
    switch (group) {
    case 1: return decode_mfma_kernel<KT, D, BS, 1, AB>;
    case 2: return decode_mfma_kernel<KT, D, BS, 2, AB>;
    case 4: return decode_mfma_kernel<KT, D, BS, 4, AB>;
    case 8: return decode_mfma_kernel<KT, D, BS, 8, AB>;
    default: return nullptr;
    }
}

template <int KT, bool AB>
DecodeKernel pick_shape(int d, int bs, int group)
{
    if (d == 64 && bs == 16) return pick_g<KT, 64, 16, AB>(group);
    if (d == 64 && bs == 32) return pick_g<KT, 64, 32, AB>(group);
    if (d == 128 && bs == 16) return pick_g<KT, 128, 16, AB>(group);
    if (d == 128 && bs == 32) return pick_g<KT, 128, 32, AB>(group);
    return nullptr;
}

DecodeKernel pick(int kv_type, int d, int bs, int group, bool acc_bf16)
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

bool mfma_supported(int q_type, int kv_type, int head_dim, int block_size, int group)
{
    return q_type == KT_BF16 && (kv_type == KT_BF16 || kv_type == KT_E4M3) &&
           (head_dim == 64 || head_dim == 128) && (block_size == 16 || block_size == 32) &&
           (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_decode_mfma(const DecodeArgs &a, int kv_type, int head_dim, int block_size,
                              int group, hipStream_t stream)
{
    const DecodeKernel k =
        pick(kv_type, head_dim, block_size, group, (a.flags & kPartialsBf16) != 0);
    if (!k)
        return hipErrorInvalidValue;
    const unsigned groups = (unsigned)((a.num_waves + kWavesPerGroup - 1) / kWavesPerGroup);
    hipLaunchKernelGGL(k, dim3(groups), dim3(64 * kWavesPerGroup), 0, stream, a);
    return hipGetLastError();
}

hipError_t decode_mfma_occupancy(int kv_type, int head_dim, int block_size, int group,
                                 bool acc_bf16, int *waves_per_cu)
{
    const DecodeKernel k = pick(kv_type, head_dim, block_size, group, acc_bf16);
    if (!k)
        return hipErrorInvalidValue;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        waves_per_cu, reinterpret_cast<const void *>(k), 64 * kWavesPerGroup, 0);
    *waves_per_cu *= kWavesPerGroup;
    return e;
}

}  // namespace pa
