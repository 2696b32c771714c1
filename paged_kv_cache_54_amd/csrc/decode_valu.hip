// decode_valu.hip -- paged decode attention on the vector ALUs, for every
// supported dtype (f32, bf16, e4m3 caches) and group size.
//
// What is computed (vLLM concept page, "Technical principles": the
// PagedAttention pseudocode and the fused-gather remark after it): for
// sequence s and KV head g, the query heads g*G .. g*G+G-1 attend over the
// first seq_len tokens of the KV rows gathered block by block through the
// sequence's block table; the gather happens inside this kernel, straight from
// the pool into registers, with no concatenated copy.
//
// Work split: one wavefront per (partition p, KV head, sequence).  A partition
// is P consecutive tokens (P a multiple of bs), i.e. whole blocks.  Lane
// layout: a token row of D elements is split into D/8 chunks of 8 elements,
// lane = row_in_pass * (D/8) + chunk, so one pass of the wavefront covers
// 64/(D/8) rows of the block with 16-byte (bf16) loads that read whole rows.
// Scores: per-lane partial dot products reduced across the D/8 lanes of a
// row.  Softmax: online (running max m, running sum l, in log2 units with
// the scale folded into q), one rescale per block.  The unfilled tail of the
// last block is masked by selection: score := -inf, weight := 0 and the V row
// replaced by 0 before it is multiplied, so NaN/Inf bits in slots past
// seq_len never reach the sum (vLLM v0.17.1 notes, fix #35219).
// When the sequence fits in one partition the wavefront writes the final
// output; otherwise it writes (acc, m, l) for the merge kernel.
#include "pa_device.h"

namespace pa {
namespace {

template <int QT, int KT, int D, int BS, int G>
__global__ __launch_bounds__(64) void decode_valu_kernel(DecodeArgs a)
{
    constexpr int TPR = D / 8;          // lanes per row
    constexpr int R = 64 / TPR;         // rows per pass
    constexpr int PASSES = BS / R;
    static_assert(BS % R == 0, "block must be a whole number of passes");

    const int lane = threadIdx.x;
    const int rl = lane / TPR;
    const int ch = lane % TPR;
    const int part = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
    const int H = a.num_heads, Hkv = a.num_kv_heads;
    const int cap = a.max_nb * BS;

    int L = a.seq_lens[s];
    if (L > cap) {
        if (part == 0 && kvh == 0 && lane == 0)
            raise_flag(a.err_flag, PA_DEVERR_SEQ_LEN);
        L = cap;
    }
    const int t0 = part * a.part_tokens;
    if (L <= 0) {
        if (part == 0 && rl == 0) {
            float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int g = 0; g < G; ++g)
                store8<QT>(a.out, ((int64_t)s * H + kvh * G + g) * D + ch * 8, z);
        }
        return;
    }
    if (t0 >= L)
        return;
    const int t1 = min(t0 + a.part_tokens, L);
    const bool whole = (t0 == 0) && (t1 == L);

    // Query rows of this head group; scale * log2(e) (* k_scale) folded in.
    float qf[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        load_q8<QT>(a.q, ((int64_t)s * H + kvh * G + g) * D + ch * 8, qf[g]);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            qf[g][i] *= a.qk_scale_log2;
    }

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[g][i] = 0.f;
    }

    const int32_t *bt = a.block_tables + (int64_t)s * a.max_nb;
    const int jb0 = t0 / BS, jb1 = (t1 + BS - 1) / BS;
    const int64_t slot_elems = (int64_t)Hkv * D;
    const int64_t lane_elem = (int64_t)rl * slot_elems + (int64_t)kvh * D + ch * 8;

    auto block_id = [&](int j) -> int {
        const int id = bt[j];
        if (id < 0 || id >= a.num_blocks) {
            if (lane == 0)
                raise_flag(a.err_flag, PA_DEVERR_BLOCK_ID);
            return -1;
        }
        return id;
    };

    Raw8<KT> kr[PASSES], vr[PASSES];
    int id = block_id(jb0);
    if (id >= 0) {
        const int64_t base = (int64_t)id * BS * slot_elems + lane_elem;
#pragma unroll
        for (int r = 0; r < PASSES; ++r) {
            kr[r] = stream_raw8<KT>(a.key_cache, base + (int64_t)r * R * slot_elems);
            vr[r] = stream_raw8<KT>(a.value_cache, base + (int64_t)r * R * slot_elems);
        }
    }

    for (int j = jb0; j < jb1; ++j) {
        // Issue the next block's loads before working on this one.
        Raw8<KT> kn[PASSES], vn[PASSES];
        const int id_next = (j + 1 < jb1) ? block_id(j + 1) : -1;
        if (id_next >= 0) {
            const int64_t base = (int64_t)id_next * BS * slot_elems + lane_elem;
#pragma unroll
            for (int r = 0; r < PASSES; ++r) {
                kn[r] = stream_raw8<KT>(a.key_cache, base + (int64_t)r * R * slot_elems);
                vn[r] = stream_raw8<KT>(a.value_cache, base + (int64_t)r * R * slot_elems);
            }
        }

        if (id >= 0) {
            const int tok0 = j * BS + rl;
            float sc[PASSES][G];
            bool valid[PASSES];
#pragma unroll
            for (int r = 0; r < PASSES; ++r) {
                float kf[8];
                unpack8(kr[r], kf);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float d = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        d = fmaf(qf[g][i], kf[i], d);
#pragma unroll
                    for (int off = TPR / 2; off > 0; off >>= 1)
                        d += __shfl_xor(d, off);
                    sc[r][g] = d;
                }
                valid[r] = (tok0 + r * R) < t1;
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float bm = -INFINITY;
#pragma unroll
                for (int r = 0; r < PASSES; ++r)
                    bm = fmaxf(bm, valid[r] ? sc[r][g] : -INFINITY);
#pragma unroll
                for (int off = TPR; off < 64; off <<= 1)
                    bm = fmaxf(bm, __shfl_xor(bm, off));
                const float mn = fmaxf(m[g], bm);
                const float alpha = (mn == m[g]) ? 1.f : exp2f(m[g] - mn);
                m[g] = mn;
                l[g] *= alpha;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    acc[g][i] *= alpha;
            }
#pragma unroll
            for (int r = 0; r < PASSES; ++r) {
                float vf[8];
                unpack8(vr[r], vf);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    vf[i] = valid[r] ? vf[i] : 0.f;
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float p = valid[r] ? exp2f(sc[r][g] - m[g]) : 0.f;
                    l[g] += p;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        acc[g][i] = fmaf(p, vf[i], acc[g][i]);
                }
            }
        }

        id = id_next;
#pragma unroll
        for (int r = 0; r < PASSES; ++r) {
            kr[r] = kn[r];
            vr[r] = vn[r];
        }
    }

    // Sum the row groups' partial (l, acc); m is already uniform across the wave.
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int off = TPR; off < 64; off <<= 1) {
            l[g] += __shfl_xor(l[g], off);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[g][i] += __shfl_xor(acc[g][i], off);
        }
    }
    if (rl != 0)
        return;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int64_t row = (int64_t)s * H + kvh * G + g;
        if (whole) {
            const float inv = l[g] > 0.f ? a.v_scale / l[g] : 0.f;
            float o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                o[i] = acc[g][i] * inv;
            store8<QT>(a.out, row * D + ch * 8, o);
        } else {
            const int64_t pi = row * a.num_parts + part;
            float o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                o[i] = acc[g][i] * a.v_scale;
            store8<KT_F32>(a.ws_acc, pi * D + ch * 8, o);
            if (ch == 0)
                *reinterpret_cast<float2 *>(a.ws_ml + pi * 2) = make_float2(m[g], l[g]);
        }
    }
}

template <int QT, int KT, int D, int BS>
hipError_t launch_g(const DecodeArgs &a, int group, hipStream_t stream)
{
    dim3 grid(a.num_parts, a.num_kv_heads, a.num_seqs), block(64);
    switch (group) {
    case 1: hipLaunchKernelGGL((decode_valu_kernel<QT, KT, D, BS, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_valu_kernel<QT, KT, D, BS, 2>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_valu_kernel<QT, KT, D, BS, 4>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((decode_valu_kernel<QT, KT, D, BS, 8>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int QT, int KT>
hipError_t launch_shape(const DecodeArgs &a, int d, int bs, int group, hipStream_t stream)
{
    if (d == 64 && bs == 16) return launch_g<QT, KT, 64, 16>(a, group, stream);
    if (d == 64 && bs == 32) return launch_g<QT, KT, 64, 32>(a, group, stream);
    if (d == 128 && bs == 16) return launch_g<QT, KT, 128, 16>(a, group, stream);
    if (d == 128 && bs == 32) return launch_g<QT, KT, 128, 32>(a, group, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_valu(const DecodeArgs &a, int q_type, int kv_type, int head_dim,
                              int block_size, int group, hipStream_t stream)
{
    if (q_type == KT_F32 && kv_type == KT_F32)
        return launch_shape<KT_F32, KT_F32>(a, head_dim, block_size, group, stream);
    if (q_type == KT_BF16 && kv_type == KT_BF16)
        return launch_shape<KT_BF16, KT_BF16>(a, head_dim, block_size, group, stream);
    if (q_type == KT_BF16 && kv_type == KT_E4M3)
        return launch_shape<KT_BF16, KT_E4M3>(a, head_dim, block_size, group, stream);
    return hipErrorInvalidValue;
}

}  // namespace pa
