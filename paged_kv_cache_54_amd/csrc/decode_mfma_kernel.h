// decode_mfma_kernel.h -- the single-query paged decode kernel on the gfx950
// matrix cores (bf16 query, bf16 or OCP e4m3 KV cache): workgroups of
// kWavesPerGroup independent wavefronts, each running decode_mfma_wave over
// its own chunk of the batch's (sequence, KV head, block) list with its own
// LDS tiles.  APP: the instance that also does the step's append
// (pa_decode_append); decode_mfma.hip instantiates the plain kernels and
// decode_mfma_append.hip those with the append, so that neither pays for
// the other's registers (the append's live rows moved the plain kernel's
// load registers onto ones still awaiting loads: waits between a tile's
// loads, 13 % slower) and the two compile in parallel.
#pragma once

#include "decode_mfma_wave.h"

namespace pa {
namespace mfma_kernel {

// Wavefronts per workgroup.  Each wavefront walks its own chunk with its own
// LDS tiles.  Two per workgroup measured ~1.3 % faster than one on the Llama-
// and Qwen-shaped batches when every resident wavefront had a chunk, and the
// same as one with the bf16 split over half of them; four were slower in both
// cases (9 % at half), eight no better.
constexpr int kWavesPerGroup = 2;

template <int KT, int D, int BS, int G, bool AB, bool APP>
__global__ __launch_bounds__(64 * kWavesPerGroup) void decode_mfma_kernel(DecodeArgs a)
{
    using Geo = MfmaGeo<KT, D, BS>;
    __shared__ __attribute__((aligned(16))) uint8_t kt_all[kWavesPerGroup][Geo::TILE * Geo::KROWB];
    __shared__ __attribute__((aligned(16))) uint8_t vt_all[kWavesPerGroup][Geo::TILE * Geo::VROWB];
    const int wave = threadIdx.x >> 6;
    // wavefronts past a.num_waves get no chunk
    decode_mfma_wave<KT, D, BS, G, AB, APP>(a, TableView{a.max_nb, 0},
                                       blockIdx.x * kWavesPerGroup + wave, kt_all[wave],
                                       vt_all[wave]);
}

typedef void (*DecodeKernel)(DecodeArgs);

template <int KT, int D, int BS, bool AB, bool APP>
DecodeKernel pick_g(int group)
{
    switch (group) {
    case 1: return decode_mfma_kernel<KT, D, BS, 1, AB, APP>;
    case 2: return decode_mfma_kernel<KT, D, BS, 2, AB, APP>;
    case 4: return decode_mfma_kernel<KT, D, BS, 4, AB, APP>;
    case 8: return decode_mfma_kernel<KT, D, BS, 8, AB, APP>;
    default: return nullptr;
    }
}

template <int KT, bool AB, bool APP>
DecodeKernel pick_shape(int d, int bs, int group)
{
    if (d == 64 && bs == 16) return pick_g<KT, 64, 16, AB, APP>(group);
    if (d == 64 && bs == 32) return pick_g<KT, 64, 32, AB, APP>(group);
    if (d == 128 && bs == 16) return pick_g<KT, 128, 16, AB, APP>(group);
    if (d == 128 && bs == 32) return pick_g<KT, 128, 32, AB, APP>(group);
    return nullptr;
}

template <bool APP>
DecodeKernel pick(int kv_type, int d, int bs, int group, bool acc_bf16)
{
    if (kv_type == KT_BF16)
        return acc_bf16 ? pick_shape<KT_BF16, true, APP>(d, bs, group)
                        : pick_shape<KT_BF16, false, APP>(d, bs, group);
    if (kv_type == KT_E4M3)
        return acc_bf16 ? pick_shape<KT_E4M3, true, APP>(d, bs, group)
                        : pick_shape<KT_E4M3, false, APP>(d, bs, group);
    return nullptr;
}

}  // namespace mfma_kernel

// The append-carrying instance for these shapes (decode_mfma_append.hip).
mfma_kernel::DecodeKernel decode_mfma_append_kernel(int kv_type, int d, int bs, int group,
                                                   bool acc_bf16);

}  // namespace pa
