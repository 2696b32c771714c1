/*
 * pa.h -- C ABI of libpa.so: paged KV-cache append and paged decode attention
 * on AMD Instinct MI355X (gfx950).
 *
 * The operations (the pages' definitions):
 *
 *   pa_kv_append -- the write side of PagedAttention: the KV cache of a layer
 *     is cut into fixed-size blocks held in one shared pool, and a new token's
 *     key and value rows are written into a block slot on demand (vLLM concept
 *     page, "15-minute deep dive", memory-manager item; the same page names
 *     the high-bandwidth pack/unpack kernels that do this on the GPU).  Token t
 *     goes to slot slot_mapping[t] = block * block_size + offset.
 *
 *   pa_decode -- the read side: for each sequence, gather the blocks its
 *     block table names in logical order and run scaled-dot-product attention
 *     of its one new query token over them (vLLM concept page, "Technical
 *     principles": PagedAttention pseudocode, and the remark that the real
 *     kernel gathers by page table inside one fused GPU kernel, without first
 *     concatenating into HBM).  Query head h reads KV head h / (H / Hkv)
 *     (grouped-query attention, same page).  Only the first seq_len tokens are
 *     attended over; the unfilled tail of the last block is excluded by
 *     selection, never by multiplying with zero, so stale NaN/Inf bits in
 *     unused slots cannot leak (vLLM v0.17.1 release notes, fix #35219).
 *
 * Conventions for every entry point:
 *   - Tensors are described by pa_tensor: a DEVICE pointer, a dtype, and shape
 *     and strides in elements.  Layouts must be dense row-major (strides
 *     matching the shape) and the data pointer 16-byte aligned; otherwise
 *     PA_ERR_LAYOUT / PA_ERR_ALIGN.
 *   - The caller owns every buffer.  The library allocates no device memory,
 *     never reads device memory from the host and never synchronises: work is
 *     queued on `hip_stream` (a hipStream_t; NULL = the null stream) and the
 *     call returns.  Calls are safe from several host threads.
 *   - A dtype combination the library was not written for is refused with
 *     PA_ERR_DTYPE rather than reinterpreted (the dtype-guard lesson of vLLM
 *     0.25.1, fix #48330, in the vLLM-internals blog, section 4.3).
 *   - Errors are returned as a pa_status; nothing is printed or thrown.  On an
 *     error nothing has been queued.
 *   - Contract on device data (not checked on the host, checked in-kernel):
 *     0 <= block_tables[s][j] < num_blocks for j < ceil(seq_lens[s] / bs);
 *     0 <= seq_lens[s] <= max_blocks_per_seq * block_size; slot_mapping
 *     entries unique and < num_blocks * block_size (negative = skip the token).
 *     A kernel never reads or writes out of bounds when the contract is broken:
 *     an out-of-range block id is skipped (its tokens are left out), an
 *     over-long seq_len is clamped to the table's capacity, an out-of-range
 *     slot is not written, and if opts->err_flag is set the matching
 *     PA_DEVERR_* bit is OR-ed into that device word.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_VERSION 3

/* Bytes of the static workspace of pa_decode_noalloc (see there). */
#define PA_NOALLOC_MAX_WORKSPACE ((size_t)96 << 20)

typedef enum pa_dtype {
    PA_F32 = 0,       /* IEEE binary32 */
    PA_BF16 = 1,      /* bfloat16 */
    PA_FP8_E4M3 = 2,  /* OCP 8-bit E4M3FN (max 448, no infinities, S.1111.111 = NaN) */
    PA_I32 = 3,
    PA_I64 = 4
} pa_dtype;

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_NULL = 1,         /* a required descriptor or data pointer is NULL */
    PA_ERR_DTYPE = 2,        /* dtype or dtype combination not supported */
    PA_ERR_SHAPE = 3,        /* ranks or sizes inconsistent */
    PA_ERR_LAYOUT = 4,       /* strides not dense row-major */
    PA_ERR_ALIGN = 5,        /* data pointer not 16-byte aligned */
    PA_ERR_UNSUPPORTED = 6,  /* head_dim, block_size, group size or option not supported */
    PA_ERR_WORKSPACE = 7,    /* split-KV workspace missing or too small */
    PA_ERR_HIP = 8,          /* the HIP runtime reported an error */
    PA_ERR_SCRATCH = 9       /* pa_decode_noalloc: the call needs more workspace than the
                                library's static buffer holds */
} pa_status;

/* Bits OR-ed into *opts->err_flag by a kernel that met broken device data. */
#define PA_DEVERR_BLOCK_ID 0x1u  /* block id outside [0, num_blocks): block skipped */
#define PA_DEVERR_SEQ_LEN 0x2u   /* seq_len > table capacity: clamped */
#define PA_DEVERR_SLOT 0x4u      /* slot >= num_blocks * block_size: token not written;
                                    pa_decode_append also: an appended row whose slot is not
                                    that of its sequence's last position (see there) */
#define PA_DEVERR_REGION 0x8u    /* block-op region base NULL or not 16-byte aligned: skipped */
#define PA_DEVERR_STEP 0x20u     /* pa_prepare_step: bad state row, count or position, or the
                                    step's tokens exceed max_tokens (see there) */
#define PA_DEVERR_PREFIX 0x40u   /* pa_decode_cascade: a table not starting with the shared
                                    prefix, or a sequence shorter than it (its output is
                                    then not the attention over its own blocks) */
#define PA_DEVERR_QUERY 0x10u    /* query_start_loc outside [0, T] or decreasing, or a sequence
                                    with more query tokens than max_query_len or seq_len: its
                                    query count clamped, rows beyond left unwritten */

typedef struct pa_tensor {
    void *data;         /* device pointer (16-byte aligned) */
    int32_t dtype;      /* pa_dtype */
    int32_t ndim;       /* 1..4 */
    int64_t shape[4];
    int64_t stride[4];  /* in elements; must be dense row-major */
} pa_tensor;

/* Storage type of split-KV partial accumulators (pa_opts.partials). */
#define PA_PARTIALS_F32 0   /* fp32 (default): a split segment's accumulators are merged
                               exactly as they were accumulated */
#define PA_PARTIALS_BF16 1  /* bf16 for a bf16 output (f32 outputs keep fp32): half the
                               workspace bytes, one extra bf16 rounding per partial */

/* Decode kernel families (pa_opts.variant). */
#define PA_VARIANT_AUTO 0  /* library choice: MFMA where supported, else VALU */
#define PA_VARIANT_VALU 1  /* vector-ALU kernel: every supported dtype and group size */
#define PA_VARIANT_MFMA 2  /* matrix-core kernel: bf16 q with a bf16 or fp8 cache */

typedef struct pa_opts {
    /* Per-tensor scales of an fp8 cache: stored code c means value(c) * scale.
       Ignored for f32 / bf16 caches.  Must be finite and > 0. */
    float k_scale;
    float v_scale;
    /* Work split.  The batch's work is the list of (sequence, KV head,
       logical block) units, sequence-major; it is cut into chunks of
       consecutive units, one per wavefront, and a KV head's sequence split
       between chunks is finished by a log-sum-exp merge.  (One-query decode
       of an e4m3 cache with 4 or 8 KV heads at head_dim 128 cuts the list of
       (sequence, logical block) units instead, every KV head of a block
       together, one chunk per workgroup of one wavefront per KV head.)
       0 (default): as many equal chunks as the device holds at once, so
       every compute unit streams the same number of blocks.  Otherwise:
       partitions of partition_tokens / block_size units (a multiple of
       block_size); a grid of at most as many chunks as the device holds at
       once walks them in equal runs of whole partitions, and a run carries
       its softmax state across their boundaries (one partial per segment it
       touches, not per partition).  The workspace is sized for one chunk
       per partition of the largest batch the tables allow. */
    int32_t partition_tokens;
    int32_t variant;            /* PA_VARIANT_* */
    void *workspace;            /* device buffer, pa_decode_workspace_size bytes,
                                   16-byte aligned; no initial contents needed */
    size_t workspace_bytes;
    uint32_t *err_flag;         /* optional device word, see PA_DEVERR_* */
    /* Profiling hook: an optional pair of hipEvent_t recorded on hip_stream
       immediately before and after the attention kernel of pa_decode,
       pa_decode_multi or pa_decode_cascade (not the merge), so callers can
       time that kernel alone.  NULL to skip (the default). */
    void *kernel_events[2];
    /* PA_PARTIALS_*: how split-KV partial accumulators are stored in the
       workspace (the workspace size depends on it). */
    int32_t partials;
} pa_opts;

/* Fills *opts with the defaults: scales 1.0, library partition choice,
   automatic variant, no workspace, no error word, no events, fp32 partials. */
void pa_opts_init(pa_opts *opts);

/*
 * pa_kv_append -- write new key/value rows into their cache slots.
 *
 *   k, v          [T, Hkv, D]            rows to write (read only)
 *   slot_mapping  [T]  PA_I64            slot = block * bs + offset; < 0 = skip
 *   key_cache,
 *   value_cache   [NB, bs, Hkv, D]       written in place
 *   opts          may be NULL (defaults); k_scale / v_scale used for fp8 caches
 *
 * Dtypes (k/v -> cache): F32 -> F32 and BF16 -> BF16 are bit copies;
 * BF16 or F32 -> FP8_E4M3 stores the nearest E4M3FN value of
 * x * (1.0f / scale), the reciprocal and the product rounded in binary32,
 * ties to even, NaN kept as NaN, magnitudes beyond 448 saturated to +-448.
 * D in {64, 128}; bs in {16, 32}.  T = 0 is allowed (nothing is queued).
 */
int pa_kv_append(const pa_tensor *k, const pa_tensor *v, const pa_tensor *slot_mapping,
                 pa_tensor *key_cache, pa_tensor *value_cache, const pa_opts *opts,
                 void *hip_stream);

/*
 * pa_decode -- paged decode attention for one new query token per sequence.
 *
 *   q             [S, H, D]               F32 or BF16
 *   key_cache,
 *   value_cache   [NB, bs, Hkv, D]        same dtype (F32, BF16 or FP8_E4M3)
 *   block_tables  [S, max_nb]  PA_I32     physical block of each logical block;
 *                                         entries at j >= ceil(seq_len/bs) unread
 *   seq_lens      [S]          PA_I32     tokens to attend over (the new token,
 *                                         already appended, included); 0 gives 0
 *   scale         multiplies q.k (usually 1/sqrt(D))
 *   out           [S, H, D]               same dtype as q; rounded to nearest even
 *   opts          may be NULL when no workspace is needed (see below)
 *
 * Supported: (q, cache, out) in {(F32, F32, F32), (BF16, BF16, BF16),
 * (BF16, FP8_E4M3, BF16)}; D in {64, 128}; bs in {16, 32};
 * G = H / Hkv in {1, 2, 4, 8}.  opts->workspace (pa_decode_workspace_size
 * bytes) is required whenever S > 0: it receives the partial results of KV
 * heads whose sequence is split between chunks (see partition_tokens) and a
 * second kernel merges them by log-sum-exp.  Accumulation is in fp32, and so
 * are the partials unless opts->partials asks for bf16.  With S > 0 the pool
 * must hold at least one block (NB >= 1), else PA_ERR_SHAPE.
 */
int pa_decode(const pa_tensor *q, const pa_tensor *key_cache, const pa_tensor *value_cache,
              const pa_tensor *block_tables, const pa_tensor *seq_lens, float scale,
              pa_tensor *out, const pa_opts *opts, void *hip_stream);

/*
 * pa_decode_workspace_size -- bytes of workspace pa_decode needs for these
 * descriptors and options (data pointers are not read; 0 means none).  Takes
 * the same arguments as pa_decode minus the data it does not need; the plan
 * depends on the current device's compute-unit count, so call it with the
 * device that will run pa_decode current.
 */
int pa_decode_workspace_size(const pa_tensor *q, const pa_tensor *key_cache,
                             const pa_tensor *block_tables, const pa_opts *opts,
                             size_t *bytes);

/*
 * pa_decode_append -- pa_kv_append(k, v, slot_mapping, caches) followed by
 * pa_decode(q, caches, ...) on the same stream: one decode step's write of
 * the new token's K/V rows into their slots and the attention that reads
 * them (vLLM concept page, "15-minute deep dive": rows are written into
 * their block slots, and attention then reads the blocks the table names).
 *
 *   k, v, slot_mapping   as pa_kv_append
 *   other arguments      as pa_decode (same workspace size)
 *
 * Results, caches and the error word are those of the two calls.  Where the
 * decode runs on the matrix cores with one new BF16 row per sequence (T = S,
 * row s belonging to sequence s) and the batch has at most twice as many
 * (sequence, KV head) pairs as the decode kernel has wavefronts (a number
 * the plan takes from the device's compute units and the kernel's
 * occupancy), the append is done
 * inside the decode kernel: the row of sequence s is written to
 * slot_mapping[s] and taken as the key/value at position seq_lens[s] - 1
 * without a round trip through the cache -- one launch less.  That form needs slot_mapping[s] to be the
 * slot of position seq_lens[s] - 1 (or < 0, nothing appended) and
 * seq_lens[s] >= 1 where a row is appended; a sequence breaking this raises
 * PA_DEVERR_SLOT: its row is written to slot_mapping[s] when that lies in
 * the pool (not when its seq_len is 0), and its attention reads position
 * seq_lens[s] - 1 from the cache as it found it (as does a read of the slot
 * the row was written to, if any sequence of the call reads it: it may see
 * the old or the new row).  A sequence whose last block id is out of range
 * (PA_DEVERR_BLOCK_ID) also raises PA_DEVERR_SLOT; its row is written.  Any
 * other case (VALU variant, F32, T != S) runs the append as its own launch
 * first.  A validation error queues nothing.
 */
int pa_decode_append(const pa_tensor *k, const pa_tensor *v, const pa_tensor *slot_mapping,
                     const pa_tensor *q, pa_tensor *key_cache, pa_tensor *value_cache,
                     const pa_tensor *block_tables, const pa_tensor *seq_lens, float scale,
                     pa_tensor *out, const pa_opts *opts, void *hip_stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and results, but the split-KV
 * workspace is a fixed device buffer the library owns, so the caller passes
 * only inputs and outputs and the call allocates nothing.
 *
 *   arguments as pa_decode; opts may be NULL; opts->workspace and
 *   opts->workspace_bytes are ignored.
 *
 * The buffer holds PA_NOALLOC_MAX_WORKSPACE bytes (96 MiB) on each device
 * the library runs on, kept until the process ends.  A call whose
 * pa_decode_workspace_size exceeds it returns PA_ERR_SCRATCH and queues
 * nothing.  Every call on one device shares that device's buffer, and it
 * keeps the last call's contents (nothing in it needs to start at zero):
 * calls whose kernels may overlap on one device -- queued on different
 * streams without an order between them -- race and must not be made.
 */
int pa_decode_noalloc(const pa_tensor *q, const pa_tensor *key_cache, const pa_tensor *value_cache,
                      const pa_tensor *block_tables, const pa_tensor *seq_lens, float scale,
                      pa_tensor *out, const pa_opts *opts, void *hip_stream);


/*
 * pa_decode_multi -- paged attention for several new query tokens per
 * sequence: the verify step of speculative decoding, where the target model
 * checks the K tokens a draft model proposed in one pass (P-EAGLE page:
 * parallel drafting of K tokens, verified together).  Sequence s owns query
 * tokens query_start_loc[s] .. query_start_loc[s+1]-1 of q; they are its last
 * q_len positions (their K/V rows already appended, so seq_lens counts them),
 * and query token i attends to positions 0 .. L - q_len + i: causal within
 * the new tokens, everything before them.  With q_len = 1 everywhere this is
 * pa_decode.
 *
 *   q, out           [T, H, D] BF16          T = total query tokens
 *   query_start_loc  [S + 1] PA_I32          0 = qsl[0] <= qsl[1] <= ... <= qsl[S] = T
 *   max_query_len    >= every q_len, 1 .. 16, with G * max_query_len <= 64
 *   key_cache, value_cache, block_tables, seq_lens, scale, opts: as pa_decode
 *                    (S = block_tables rows); caches BF16 or FP8_E4M3
 * Matrix-core kernel only: opts->variant PA_VARIANT_VALU is refused with
 * PA_ERR_UNSUPPORTED, as are f32 tensors.  Device contract: q_len <= seq_len;
 * a violation raises PA_DEVERR_QUERY (see there).  Workspace:
 * pa_decode_multi_workspace_size bytes.
 */
int pa_decode_multi(const pa_tensor *q, const pa_tensor *query_start_loc, int32_t max_query_len,
                    const pa_tensor *key_cache, const pa_tensor *value_cache,
                    const pa_tensor *block_tables, const pa_tensor *seq_lens, float scale,
                    pa_tensor *out, const pa_opts *opts, void *hip_stream);

/* Workspace bytes of pa_decode_multi (same rules as pa_decode_workspace_size). */
int pa_decode_multi_workspace_size(const pa_tensor *q, int32_t max_query_len,
                                   const pa_tensor *key_cache, const pa_tensor *block_tables,
                                   const pa_opts *opts, size_t *bytes);

/*
 * pa_decode_cascade -- pa_decode for a batch whose sequences share their
 * first prefix_blocks logical blocks (the same physical blocks: a common
 * prompt, vLLM internals blog section 1 and figure 1).  Equal to pa_decode
 * within its tolerance, but the shared blocks are read once per group of
 * sequences instead of once per sequence: the attention is split at the
 * prefix boundary into a pass of all queries over the shared blocks and a
 * pass of each query over its own later blocks, joined by log-sum-exp.
 *
 *   prefix_blocks  0 <= N < max_blocks_per_seq (0: exactly pa_decode)
 *   the rest as pa_decode; matrix-core kernels only (bf16 q, bf16 or e4m3
 *   cache; PA_ERR_UNSUPPORTED otherwise).  Workspace:
 *   pa_decode_cascade_workspace_size bytes.
 * Contract on device data: block_tables[s][j] == block_tables[0][j] for
 * j < N and seq_lens[s] >= N * block_size for every s; a violation raises
 * PA_DEVERR_PREFIX.
 */
int pa_decode_cascade(const pa_tensor *q, const pa_tensor *key_cache,
                      const pa_tensor *value_cache, const pa_tensor *block_tables,
                      const pa_tensor *seq_lens, int32_t prefix_blocks, float scale,
                      pa_tensor *out, const pa_opts *opts, void *hip_stream);

int pa_decode_cascade_workspace_size(const pa_tensor *q, const pa_tensor *key_cache,
                                     const pa_tensor *block_tables, int32_t prefix_blocks,
                                     const pa_opts *opts, size_t *bytes);

/*
 * Block maintenance.  A "region" is one cache of the pool layout, for example
 * the K cache or the V cache of one layer: block b of region r occupies the
 * bytes [region_bases[r] + b * block_stride, + block_bytes).  Every region of
 * one call has the same block geometry.  For the caches of this library
 * ([NB, bs, Hkv, D], dense) block_stride = block_bytes = bs * Hkv * D * elt.
 *
 * The id and base arrays are read by the kernel, not by the host: they may be
 * device memory or host memory the device can read (hipHostMalloc /
 * pinned), which hands freshly chosen ids to the GPU with no copy and no
 * synchronisation.  They must stay unchanged until the queued work has run.
 * Alignment: ids 4 bytes (pairs 8 bytes), bases 8 bytes; every region base
 * must be 16-byte aligned (a NULL or misaligned base is skipped and raises
 * PA_DEVERR_REGION).  block_stride and block_bytes are multiples of 16, with
 * 0 < block_bytes <= block_stride.  An id outside [0, num_blocks) is skipped
 * and raises PA_DEVERR_BLOCK_ID.  opts may be NULL; only err_flag is used.
 * num_ids (num_pairs) == 0 or num_regions == 0 queues nothing.
 */

/*
 * pa_zero_blocks -- clear (write zero bytes over) every listed block in every
 * region, in one launch.  A block that another layer type used before can
 * hold bit patterns that are NaN/Inf in the cache dtype; clearing newly
 * allocated blocks before attention uses them keeps such bits out of any
 * kernel that masks by multiplying with zero (vLLM v0.17.1 release notes,
 * fix #35219: batched clearing over precomputed cache segment addresses,
 * block ids passed through pinned memory, no synchronisation).
 *
 *   block_ids     [num_ids] int32; duplicates allowed
 */
int pa_zero_blocks(const int32_t *block_ids, int64_t num_ids, void *const *region_bases,
                   int32_t num_regions, int64_t block_stride, int64_t block_bytes,
                   int64_t num_blocks, const pa_opts *opts, void *hip_stream);

/*
 * pa_copy_blocks -- copy whole blocks: for each pair (src, dst), block src of
 * src region r is copied over block dst of dst region r, for every region.
 * Uses: copy-on-write of a block shared by a common prefix before one
 * sequence writes into it (vLLM internals blog, section 1, the page-table
 * analogy and figure 1), and moving a preempted sequence's blocks between the
 * GPU pool and a host pool and back (swap out / swap in, vLLM concept page,
 * "15-minute deep dive", scheduler item); a host pool must be device-readable
 * (and -writable for swap out) pinned memory, and that traffic is bound by
 * the host link.
 *
 *   block_pairs   [num_pairs, 2] int32: (src block, dst block); src ids are
 *                 checked against src_num_blocks, dst ids against dst_num_blocks
 *   src_bases, dst_bases  [num_regions] each
 * Contract: no dst block of a call is also a src block or a second dst block
 * of that call in the same memory (the order of the copies is unspecified).
 */
int pa_copy_blocks(const int32_t *block_pairs, int64_t num_pairs, const void *const *src_bases,
                   void *const *dst_bases, int32_t num_regions, int64_t block_stride,
                   int64_t block_bytes, int64_t src_num_blocks, int64_t dst_num_blocks,
                   const pa_opts *opts, void *hip_stream);

/*
 * pa_prepare_step -- one step's attention inputs, built on the GPU from a
 * persistent per-request state table (Model Runner V2 page, "better
 * persistent batch and GPU-native input preparation": every active request
 * keeps a stable row of a fixed-size state table and each step gathers its
 * inputs in the current request order on the device, so that no host-device
 * synchronisation is needed and device-side results -- the accepted token
 * counts of speculative decoding -- can feed the next step directly).
 *
 * For batch entry i with state row r = idx_mapping[i] and n_i =
 * num_scheduled[i] new tokens (token k at position num_computed[r] + k):
 *   query_start_loc[i+1] = query_start_loc[i] + n_i      (query_start_loc[0] = 0)
 *   seq_lens[i]          = num_computed[r] + n_i
 *   block_tables[i, :]   = state block_table[r, :]
 *   positions[t], input_ids[t] = token_ids[r, position], slot_mapping[t] =
 *       block_table[r, position / block_size] * block_size + position % block_size
 * Rows t >= query_start_loc[S] up to max_tokens are padding: slot -1 (which
 * pa_kv_append skips), position 0, input id 0.  The outputs feed pa_kv_append
 * (slot_mapping), pa_decode / pa_decode_multi (block_tables, seq_lens,
 * query_start_loc) and the model (positions, input_ids).
 *
 * Every pointer is device memory (or device-readable host memory); int32
 * arrays 4-byte and int64 arrays 8-byte aligned.  1 <= num_reqs <= 2048.
 * Contract on device data: rows in [0, num_rows), counts and num_computed
 * >= 0, the step's total <= max_tokens, positions < max_len and their blocks
 * in the table and the pool.  A violation raises PA_DEVERR_STEP (entry
 * dropped, or its count cut at max_tokens, or input id 0, or slot -1) or
 * PA_DEVERR_BLOCK_ID (slot -1).
 */
typedef struct pa_step_state {
    const int32_t *num_computed;  /* [num_rows] tokens of each request already in the cache */
    const int32_t *block_table;   /* [num_rows, max_blocks] physical block ids */
    const int32_t *token_ids;     /* [num_rows, max_len] each request's token ids */
    int32_t num_rows, max_blocks, max_len;
} pa_step_state;

typedef struct pa_step_inputs {
    int32_t *query_start_loc;     /* [num_reqs + 1] */
    int32_t *seq_lens;            /* [num_reqs] */
    int64_t *positions;           /* [max_tokens] */
    int32_t *input_ids;           /* [max_tokens] */
    int64_t *slot_mapping;        /* [max_tokens] */
    int32_t *block_tables;        /* [num_reqs, max_blocks] */
    int32_t max_tokens;
} pa_step_inputs;

int pa_prepare_step(const int32_t *idx_mapping, const int32_t *num_scheduled, int32_t num_reqs,
                    const pa_step_state *state, int32_t block_size, int32_t num_blocks,
                    const pa_step_inputs *out, const pa_opts *opts, void *hip_stream);

/* Static description of a status code. */
const char *pa_status_string(int status);

/* PA_VERSION of the library. */
int pa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PA_H */
