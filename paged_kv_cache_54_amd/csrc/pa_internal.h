// pa_internal.h -- types shared by the host dispatch code and the gfx950
// kernels of libpa.so.  Not installed; the public ABI is include/pa.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "pa.h"

namespace pa {

// Element types as the kernels see them (template parameters).
enum KvType : int { KT_F32 = 0, KT_BF16 = 1, KT_E4M3 = 2 };

// Everything a decode kernel needs; passed by value as the kernel argument.
struct DecodeArgs {
    const void *q;               // [S, H, D]
    const void *key_cache;       // [NB, bs, Hkv, D]
    const void *value_cache;
    const int32_t *block_tables; // [S, max_nb]
    const int32_t *seq_lens;     // [S]
    void *out;                   // [S, H, D]
    float *ws_acc;               // [S, H, NP, D]  unnormalised partial outputs
    float *ws_ml;                // [S, H, NP, 2]  (running max in log2 units, sum)
    uint32_t *err_flag;          // optional
    int32_t num_seqs, num_heads, num_kv_heads, max_nb, num_blocks;
    int32_t part_tokens;         // P: tokens per partition (multiple of bs)
    int32_t num_parts;           // NP = ceil(max_nb * bs / P)
    float qk_scale_log2;         // scale * log2(e) * k_scale (k_scale = 1 unless fp8)
    float v_scale;               // 1 unless fp8
};

struct AppendArgs {
    const void *k;               // [T, Hkv, D]
    const void *v;
    const int64_t *slots;        // [T]
    void *key_cache;             // [NB, bs, Hkv, D]
    void *value_cache;
    uint32_t *err_flag;
    int64_t num_tokens;
    int64_t row_elems;           // Hkv * D
    int64_t num_slots;           // NB * bs
    float k_inv_scale;           // 1.0f / k_scale, rounded in binary32 (fp8 caches)
    float v_inv_scale;
};

// Launchers (defined in the .hip translation units).  Each returns a
// hipError_t from hipGetLastError() after the launch.
hipError_t launch_kv_append(const AppendArgs &a, int in_type, int cache_type,
                            hipStream_t stream);

// Vector-ALU decode: grid (NP, Hkv, S) of one wavefront each.
hipError_t launch_decode_valu(const DecodeArgs &a, int q_type, int kv_type, int head_dim,
                              int block_size, int group, hipStream_t stream);

// Matrix-core decode (bf16 q; bf16 or e4m3 cache).
hipError_t launch_decode_mfma(const DecodeArgs &a, int kv_type, int head_dim, int block_size,
                              int group, hipStream_t stream);
bool mfma_supported(int q_type, int kv_type, int head_dim, int block_size, int group);

// Log-sum-exp merge of split-KV partials: grid (S * H) of one wavefront.
hipError_t launch_merge(const DecodeArgs &a, int out_type, int head_dim, int block_size,
                        hipStream_t stream);

}  // namespace pa
