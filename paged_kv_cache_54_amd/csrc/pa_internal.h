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
// The work of a call is the flattened list of (sequence, KV head, block)
// units, cut into chunks of `chunk_units` units (0: ceil(total / waves)), one
// per wavefront of the grid.
struct DecodeArgs {
    const void *q;               // [S, H, D]
    const void *key_cache;       // [NB, bs, Hkv, D]
    const void *value_cache;
    const int32_t *block_tables; // [S, max_nb]
    const int32_t *seq_lens;     // [S]
    void *out;                   // [S, H, D]
    void *ws_acc;                // [slots, rows, D] unnormalised partial outputs: f32, or
                                 // bf16 with kPartialsBf16
    float *ws_ml;                // [slots, rows, 2] (softmax base in log2 units, sum)
    int32_t *ws_seg;             // [S * Hkv, 2]   first and last slot of each segment
    uint32_t *err_flag;          // optional
    int32_t num_seqs, num_heads, num_kv_heads, max_nb, num_blocks;
    int32_t chunk_units;         // units per chunk, 0 = balanced over the grid
    int32_t num_waves;           // grid size (one wavefront per workgroup)
    int32_t rows_per_slot;       // partial rows per slot: G, or G * max_query_len
    // several query tokens per sequence (NULL query_start_loc: one per sequence)
    const int32_t *query_start_loc; // [S + 1]
    int32_t max_query_len;
    int32_t num_tokens;          // T, rows of q and out
    int32_t log2_group;          // G = 2^log2_group
    float qk_scale_log2;         // scale * log2(e) * k_scale (k_scale = 1 unless fp8)
    float v_scale;               // 1 unless fp8
    int32_t flags;               // kPartialOnly | kPartialsBf16
    int32_t slot_stride;         // slots of one segment's partials step by this (>= 1)
    int32_t num_slots;           // slots of the workspace
    // Append fused into the decode (matrix-core single-query kernels): row s
    // of new_k / new_v [S, Hkv, D] (bf16) goes to cache slot new_slots[s],
    // which should be the slot of position seq_lens[s] - 1, and the attention
    // takes it at that position.  new_k NULL: no append.
    const void *new_k, *new_v;
    const int64_t *new_slots;    // [S]; < 0: nothing appended
    float k_inv_scale, v_inv_scale;   // e4m3 caches: 1 / k_scale, 1 / v_scale (binary32)
};

// DecodeArgs.flags.  kPartialOnly (matrix-core kernels): every segment ends
// as a partial (acc, m, l), also one a single chunk covers, so that a second
// pass can combine it with another source.  kPartialsBf16: partial
// accumulators are stored as bf16 (bf16 outputs only); otherwise f32.
// kRuns (per-wavefront kernels, chunk_units > 0): chunk_units names
// partitions, and each of the num_waves chunks is an equal run of whole
// partitions.
constexpr int32_t kPartialOnly = 1;
constexpr int32_t kPartialsBf16 = 2;
constexpr int32_t kRuns = 4;

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

// Whole-block clear or copy over a set of regions (caches): block b of region
// r is bytes [bases[r] + b * block_stride, + block_bytes).  Items are block ids
// (clear) or (src, dst) id pairs (copy); each workgroup handles up to
// group_items consecutive items x one region x one chunk of the block.
constexpr int kMaxGroupItems = 64;

struct BlockOpArgs {
    const int32_t *ids;          // [num_items] or [num_items, 2]; device-readable
    void *const *dst_bases;      // [num_regions]; device-readable
    const void *const *src_bases;// [num_regions] (copy only)
    uint32_t *err_flag;
    int64_t num_items;
    int64_t block_stride;        // bytes
    int64_t block_bytes;         // bytes per block per region, multiple of 16
    int64_t dst_num_blocks, src_num_blocks;
    int64_t chunks;              // ceil(block_bytes / chunk bytes)
    int32_t num_regions;
    int32_t group_items;         // 1 .. kMaxGroupItems
    int32_t pieces;              // per-piece kernel: ceil(block_bytes / piece bytes)
};

// One step's attention inputs gathered from a per-request state table.
constexpr int kMaxPrepReqs = 2048;

struct StepPrepArgs {
    const int32_t *idx_mapping;   // [S] state row of each batch entry
    const int32_t *num_scheduled; // [S] new tokens of each entry
    const int32_t *num_computed;  // [R] tokens already in the cache, per state row
    const int32_t *block_table;   // [R, max_blocks]
    const int32_t *token_ids;     // [R, max_len]
    int32_t *query_start_loc;     // [S + 1]
    int32_t *seq_lens;            // [S]
    int64_t *positions;           // [max_tokens]
    int32_t *input_ids;           // [max_tokens]
    int64_t *slot_mapping;        // [max_tokens]
    int32_t *block_tables;        // [S, max_blocks]
    uint32_t *err_flag;
    int32_t num_reqs, num_rows, max_blocks, max_len, max_tokens, block_size, num_blocks;
};

// Cascade decode for a batch whose sequences share their first N blocks.
//
// Prefix pass: the query rows of KV head kvh are the (sequence, head of the
// group) pairs, row r = s * G + g, R = S * G of them.  Work item
// (kvh, split p, row block) attends the row block's rows to blocks
// [p * bps, min(N, (p + 1) * bps)) of the shared prefix (row 0 of the block
// table) and writes, per row, the partial (m, l, acc) to
// p_acc/p_ml[(p * Hkv + kvh) * R + r].
//
// Suffix pass: the single-query decode over the batch viewed from block N on
// (tables from column N, lengths less N * bs), partials only.  Both passes and
// check_wgs workgroups checking the shared-prefix contract run in one
// launch: items first, then the check, then the decode's workgroups.
struct CascadePrefixArgs {
    const void *q;                // [S, H, D] bf16
    const void *key_cache, *value_cache;
    const int32_t *block_tables;  // [S, max_nb]
    const int32_t *seq_lens;      // [S]
    void *p_acc;                  // [P, Hkv, R, D] f32, or bf16 with partials_bf16
    float *p_ml;                  // [P, Hkv, R, 2]
    uint32_t *err_flag;
    int32_t num_seqs, num_heads, num_kv_heads, max_nb, num_blocks, block_size;
    int32_t prefix_blocks, num_splits, split_blocks;   // N, P, bps
    int32_t rows, row_blocks;                          // R, row blocks per KV head
    int32_t num_items, items_per_xcd, log2_group, check_wgs;
    int32_t partials_bf16;        // prefix partial accumulators stored as bf16
    float qk_scale_log2, v_scale;
};

// Combination of each row's suffix partials (rows_per_slot G) and its P
// prefix partials (layout above).
struct CascadeMergeArgs {
    void *out;                    // [S, H, D]
    const void *s_acc;            // suffix partials (acc f32 or bf16, m and l f32)
    const float *s_ml;
    const int32_t *s_seg;
    const int32_t *seq_lens;      // [S]; a sequence's suffix is its tokens past N * bs
    int32_t prefix_tokens, capacity;   // N * bs, max_nb * bs
    const void *p_acc;            // prefix partials (same types)
    const float *p_ml;
    int32_t num_seqs, num_heads, num_kv_heads, num_splits;
    int32_t partials_bf16;        // both accumulators stored as bf16
    int32_t num_slots;            // suffix partial slots of the workspace
};

// Launchers (defined in the .hip translation units).  Each returns a
// hipError_t from hipGetLastError() after the launch.
hipError_t launch_kv_append(const AppendArgs &a, int in_type, int cache_type,
                            hipStream_t stream);

// Vector-ALU decode: one wavefront per chunk.
hipError_t launch_decode_valu(const DecodeArgs &a, int q_type, int kv_type, int head_dim,
                              int block_size, int group, hipStream_t stream);

// Matrix-core decode (bf16 q; bf16 or e4m3 cache).
hipError_t launch_decode_mfma(const DecodeArgs &a, int kv_type, int head_dim, int block_size,
                              int group, hipStream_t stream);
bool mfma_supported(int q_type, int kv_type, int head_dim, int block_size, int group);

// Matrix-core decode of an e4m3 cache with workgroups of one wavefront per KV
// head (a.num_kv_heads of them) walking (sequence, block) units; partial slots
// of a segment step by num_kv_heads (a.slot_stride).  Occupancy in workgroups.
bool decode_mfma_heads_supported(int kv_type, int head_dim, int block_size, int group,
                                 int num_kv_heads);
hipError_t launch_decode_mfma_heads(const DecodeArgs &a, int kv_type, int head_dim,
                                    int block_size, int group, int workgroups,
                                    hipStream_t stream);
hipError_t decode_mfma_heads_occupancy(int kv_type, int head_dim, int block_size, int group,
                                       int num_kv_heads, bool acc_bf16, int *groups_per_cu);

// Matrix-core decode of several query tokens per sequence; col_tiles = 16-column
// tiles of (query token, head) pairs per KV head, 1, 2 or 4.
hipError_t launch_decode_mfma_multi(const DecodeArgs &a, int kv_type, int head_dim,
                                    int block_size, int col_tiles, hipStream_t stream);
hipError_t decode_mfma_multi_occupancy(int kv_type, int head_dim, int block_size, int col_tiles,
                                       bool acc_bf16, int *waves_per_cu);

// Wavefronts of the matching decode kernel that one compute unit holds at
// once (acc_bf16: the instance storing bf16 partial accumulators).
hipError_t decode_valu_occupancy(int q_type, int kv_type, int head_dim, int block_size, int group,
                                 int *waves_per_cu);
hipError_t decode_mfma_occupancy(int kv_type, int head_dim, int block_size, int group,
                                 bool acc_bf16, int *waves_per_cu);

// Log-sum-exp merge of the chunk partials of every segment that more than
// one chunk touched; zero rows for empty sequences.  Grid (S * H), or
// (S * max_query_len * H) with several query tokens per sequence, of
// 256-thread workgroups.
hipError_t launch_merge(const DecodeArgs &a, int out_type, int head_dim, int block_size,
                        hipStream_t stream);

// Prefix pass, contract check and suffix pass (s: partials only, tables
// starting at column N, lengths counted from token N * bs, s.max_nb = max_nb -
// N, s.num_waves wavefronts) in one launch.
hipError_t launch_cascade(const CascadePrefixArgs &p, const DecodeArgs &s, int kv_type,
                          int head_dim, int block_size, int group, hipStream_t stream);
// Rows of one prefix-pass workgroup.
int cascade_prefix_rows();
// Suffix-pass wavefronts per compute unit of the cascade kernel: those of the
// workgroups a compute unit holds at once beside one prefix workgroup.
hipError_t cascade_suffix_occupancy(int kv_type, int head_dim, int block_size, int group,
                                    bool acc_bf16, int *waves_per_cu);
hipError_t launch_cascade_merge(const CascadeMergeArgs &a, int out_type, int head_dim,
                                hipStream_t stream);

// The static device buffer of pa_decode_noalloc: its bytes, and its address
// on the current device (looked up once per device).
constexpr size_t kStaticScratchBytes = PA_NOALLOC_MAX_WORKSPACE;
int static_scratch(void **ptr);

// Step metadata from the state table; num_reqs <= kMaxPrepReqs.
hipError_t launch_step_prep(const StepPrepArgs &a, hipStream_t stream);

// Block clear (copy = false) or copy; chunk bytes per workgroup pass.
hipError_t launch_block_op(const BlockOpArgs &a, bool copy, hipStream_t stream);
int64_t block_op_chunk_bytes();
// One workgroup per (item, region, piece): for id and base tables in device
// memory.
hipError_t launch_block_piece_op(const BlockOpArgs &a, bool copy, hipStream_t stream);
int64_t block_op_piece_bytes();

}  // namespace pa
