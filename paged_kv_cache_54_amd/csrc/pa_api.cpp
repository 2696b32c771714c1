// pa_api.cpp -- the C ABI of libpa.so (include/pa.h): descriptor validation,
// launch planning and dispatch to the gfx950 kernels.  Host code only; it
// never reads device memory and never synchronises.
#include "pa.h"

#include <math.h>
#include <string.h>

#include <initializer_list>
#include <mutex>
#include <vector>

#include "pa_internal.h"

namespace {

using namespace pa;

constexpr float kLog2e = 1.4426950408889634f;

// Dense row-major: each stride the product of the sizes after it.  The
// stride of a dimension of size 1 addresses nothing, and a tensor with no
// elements has nothing to address (frameworks give both arbitrary strides).
bool is_dense(const pa_tensor *t)
{
    bool empty = false;
    for (int i = 0; i < t->ndim; ++i) {
        if (t->shape[i] < 0)
            return false;
        empty |= t->shape[i] == 0;
    }
    if (empty)
        return true;
    int64_t expect = 1;
    for (int i = t->ndim - 1; i >= 0; --i) {
        if (t->shape[i] != 1 && t->stride[i] != expect)
            return false;
        expect *= t->shape[i];
    }
    return true;
}

int64_t numel(const pa_tensor *t)
{
    int64_t n = 1;
    for (int i = 0; i < t->ndim; ++i)
        n *= t->shape[i];
    return n;
}

// Common checks of one descriptor: rank, dtype, dense layout, alignment.
int check_tensor(const pa_tensor *t, int ndim, uintptr_t align)
{
    if (!t)
        return PA_ERR_NULL;
    if (t->ndim != ndim)
        return PA_ERR_SHAPE;
    if (!is_dense(t))
        return PA_ERR_LAYOUT;
    if (numel(t) > 0 && !t->data)
        return PA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(t->data) % align)
        return PA_ERR_ALIGN;
    return PA_OK;
}

int kv_type_of(int dtype)
{
    switch (dtype) {
    case PA_F32: return KT_F32;
    case PA_BF16: return KT_BF16;
    case PA_FP8_E4M3: return KT_E4M3;
    default: return -1;
    }
}

bool supported_head_dim(int64_t d) { return d == 64 || d == 128; }
bool supported_block_size(int64_t bs) { return bs == 16 || bs == 32; }
bool supported_group(int64_t g) { return g == 1 || g == 2 || g == 4 || g == 8; }

// Compute units of the current device, cached per device id.
int device_cu_count(int *cus)
{
    static std::mutex mu;
    static std::vector<int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return PA_ERR_HIP;
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= (int)cache.size())
        cache.resize(dev + 1, 0);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return PA_ERR_HIP;
        cache[dev] = n;
    }
    *cus = cache[dev];
    return PA_OK;
}

struct DecodePlan {
    int64_t S, H, Hkv, D, bs, NB, max_nb, G;
    int64_t T;               // query rows of q: S, or the total query tokens
    int64_t QM;              // 0: one query token per sequence; else max_query_len
    int64_t col_tiles;       // multi-token: 16-column tiles of (token, head) pairs
    int64_t rows;            // partial rows per slot: G, or G * QM
    int q_type, kv_type;
    int variant;             // PA_VARIANT_VALU or PA_VARIANT_MFMA
    int64_t chunk_units;     // units per chunk, 0 = balanced over the waves
    int64_t heads;           // > 0: the e4m3 kernel whose workgroups hold one wavefront
                             // per KV head (heads = Hkv) and walk (sequence, block) units
    int64_t waves;           // grid size in wavefronts; with heads > 0, partitions * heads
    int64_t groups;          // heads > 0: workgroups to launch (fixed partitions: at most
                             // the partition count, capped at launch by the resident ones)
    int64_t slots;           // partial slots = waves + segments
    bool acc_bf16;           // partial accumulators stored as bf16
    size_t ws_bytes;
};


// Workspace layout: acc [slots, rows, D] | ml [slots, rows, 2] f32 | seg [S*Hkv, 2] i32
// Partial accumulators are f32; PA_PARTIALS_BF16 stores them as bf16 for a
// bf16 output (half the bytes a split segment writes and the merge reads).
size_t acc_bytes(const DecodePlan &p)
{
    return (p.acc_bf16 ? 2 : 4) * (size_t)(p.slots * p.rows) * (size_t)p.D;
}

size_t workspace_bytes(const DecodePlan &p)
{
    return acc_bytes(p) + sizeof(float) * (size_t)(p.slots * p.rows) * 2 +
           sizeof(int32_t) * 2 * (size_t)(p.S * p.Hkv);
}

// Wavefronts of the chosen kernel one compute unit holds at once, cached per
// (device, kernel instance).  cascade: the suffix-pass wavefronts of the
// cascade kernel, which shares each compute unit with a prefix workgroup.
int resident_waves_per_cu(const DecodePlan &p, int *waves, bool cascade = false)
{
    static std::mutex mu;
    static std::vector<std::pair<long long, int>> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return PA_ERR_HIP;
    const long long key = ((((((((((long long)dev * 4 + p.variant) * 4 + p.q_type) * 4 + p.kv_type) *
                              256 + p.D) * 64 + p.bs) * 32 + p.G) * 8 + p.col_tiles) * 2 +
                          cascade) * 2 + p.acc_bf16) * 16 + p.heads;
    std::lock_guard<std::mutex> lock(mu);
    for (auto &kv : cache)
        if (kv.first == key) {
            *waves = kv.second;
            return PA_OK;
        }
    int n = 0;
    hipError_t e =
        cascade    ? cascade_suffix_occupancy(p.kv_type, (int)p.D, (int)p.bs, (int)p.G,
                                            p.acc_bf16, &n)
        : p.QM > 0 ? decode_mfma_multi_occupancy(p.kv_type, (int)p.D, (int)p.bs,
                                               (int)p.col_tiles, p.acc_bf16, &n)
        : p.heads > 0 ? decode_mfma_heads_occupancy(p.kv_type, (int)p.D, (int)p.bs, (int)p.G,
                                                  (int)p.heads, p.acc_bf16, &n)
        : p.variant == PA_VARIANT_MFMA
            ? decode_mfma_occupancy(p.kv_type, (int)p.D, (int)p.bs, (int)p.G, p.acc_bf16, &n)
            : decode_valu_occupancy(p.q_type, p.kv_type, (int)p.D, (int)p.bs, (int)p.G, &n);
    if (e != hipSuccess || n <= 0)
        return PA_ERR_HIP;
    if (p.heads > 0 && !cascade)
        n *= (int)p.heads;                   // workgroups -> wavefronts
    cache.emplace_back(key, n);
    *waves = n;
    return PA_OK;
}

// Chunks of the balanced split of a per-wavefront or multi-token plan: one
// per wavefront (workgroup, for the two-wavefront multi-token kernel) the
// device holds at once, halved where one wavefront per SIMD streams faster.
int balanced_chunks(const DecodePlan &p, int64_t qm, int64_t *chunks)
{
    int cus = 0, per_cu = 0, rc;
    if ((rc = device_cu_count(&cus)) || (rc = resident_waves_per_cu(p, &per_cu)))
        return rc;
    int64_t n = (int64_t)cus * per_cu;
    // Single-query decode of a bf16 cache on the matrix cores: half as many
    // wavefronts, each with a chunk twice as long.  One register tile in
    // flight per wavefront (about 8 MB over the device) still keeps enough
    // bytes moving, and a chunk's pipeline start and partial writes come
    // half as often (1-4 % faster over bf16 batches of 8-256 sequences; a
    // quarter of the wavefronts with two tiles each was 30 % slower).  An
    // e4m3 cache's per-wavefront kernel needs every resident wavefront.
    if (p.variant == PA_VARIANT_MFMA && qm == 0 && p.kv_type == KT_BF16)
        n = (n + 1) / 2;
    // The same for the one-wavefront multi-token kernel holding two column
    // tiles (a bf16 cache, 17-32 query rows per KV head): one wavefront per
    // SIMD, 1 % faster than the two-wavefront kernel on the Llama-shaped
    // verify step (3 % slower at two per SIMD).  Halving the two-wavefront
    // kernel's workgroups was 27 % slower.
    if (p.variant == PA_VARIANT_MFMA && qm > 0 && p.col_tiles == 2 && p.kv_type == KT_BF16)
        n = (n + 1) / 2;
    *chunks = n;
    return PA_OK;
}

// Shapes, dtypes and options common to the decode entry points and their
// workspace queries.  qm = 0: one query token per sequence (q [S, H, D]);
// qm > 0: several per sequence, at most qm (q [T, H, D], S from the tables).
// allow_heads: single-query e4m3 decode may use the per-block kernel (not for
// the cascade's suffix pass, which runs the per-wavefront body).
int plan_decode(const pa_tensor *q, const pa_tensor *kc, const pa_tensor *bt,
                const pa_opts *opts, int64_t qm, DecodePlan *p, bool allow_heads = true)
{
    if (!q || !kc || !bt)
        return PA_ERR_NULL;
    if (q->ndim != 3 || kc->ndim != 4 || bt->ndim != 2)
        return PA_ERR_SHAPE;
    if ((q->dtype != PA_F32 && q->dtype != PA_BF16) || bt->dtype != PA_I32)
        return PA_ERR_DTYPE;
    const int kvt = kv_type_of(kc->dtype);
    if (kvt < 0)
        return PA_ERR_DTYPE;
    // Supported (q, cache) pairs: (f32, f32), (bf16, bf16), (bf16, e4m3).
    if (q->dtype == PA_F32 ? kvt != KT_F32 : kvt == KT_F32)
        return PA_ERR_DTYPE;
    p->T = q->shape[0];
    p->S = qm > 0 ? bt->shape[0] : q->shape[0];
    p->QM = qm;
    p->H = q->shape[1];
    p->D = q->shape[2];
    p->NB = kc->shape[0];
    p->bs = kc->shape[1];
    p->Hkv = kc->shape[2];
    p->max_nb = bt->shape[1];
    if (kc->shape[3] != p->D || bt->shape[0] != p->S || p->Hkv <= 0 || p->H <= 0 ||
        p->H % p->Hkv)
        return PA_ERR_SHAPE;
    p->G = p->H / p->Hkv;
    if (!supported_head_dim(p->D) || !supported_block_size(p->bs) || !supported_group(p->G))
        return PA_ERR_UNSUPPORTED;
    if (p->S > INT32_MAX || p->NB > INT32_MAX || p->max_nb > INT32_MAX / p->bs ||
        p->S * p->Hkv > INT32_MAX / 2 || p->T > INT32_MAX / p->H)
        return PA_ERR_UNSUPPORTED;
    p->q_type = kv_type_of(q->dtype);
    p->kv_type = kvt;

    const int partials = opts ? opts->partials : PA_PARTIALS_F32;
    if (partials != PA_PARTIALS_F32 && partials != PA_PARTIALS_BF16)
        return PA_ERR_UNSUPPORTED;
    p->acc_bf16 = partials == PA_PARTIALS_BF16 && p->q_type == KT_BF16;

    const int variant = opts ? opts->variant : PA_VARIANT_AUTO;
    const bool mfma_ok = mfma_supported(p->q_type, kvt, (int)p->D, (int)p->bs, (int)p->G);
    p->col_tiles = 0;
    p->rows = p->G;
    if (qm > 0) {
        // (query token, head) columns in tiles of 16, matrix cores only
        if (!mfma_ok || variant == PA_VARIANT_VALU || qm > 16 || p->G * qm > 64)
            return PA_ERR_UNSUPPORTED;
        const int64_t cols = p->G * qm;
        p->col_tiles = cols <= 16 ? 1 : (cols <= 32 ? 2 : 4);
        p->rows = cols;
    }
    if (variant == PA_VARIANT_AUTO)
        p->variant = mfma_ok ? PA_VARIANT_MFMA : PA_VARIANT_VALU;
    else if (variant == PA_VARIANT_VALU)
        p->variant = PA_VARIANT_VALU;
    else if (variant == PA_VARIANT_MFMA && mfma_ok)
        p->variant = PA_VARIANT_MFMA;
    else
        return PA_ERR_UNSUPPORTED;
    // e4m3 cache, one query token: workgroups of one wavefront per KV head
    // that read each block's K and V whole (every head of a token slot
    // together) where that kernel has an instance.
    p->heads = allow_heads && p->variant == PA_VARIANT_MFMA && qm == 0 &&
                       decode_mfma_heads_supported(kvt, (int)p->D, (int)p->bs, (int)p->G,
                                                   (int)p->Hkv)
                   ? p->Hkv
                   : 0;

    // Chunking of the (sequence, KV head, block) work list, or of the
    // (sequence, block) list with heads > 0.
    const int64_t P = opts ? opts->partition_tokens : 0;
    if (P < 0 || P % p->bs)
        return PA_ERR_UNSUPPORTED;
    const int64_t max_units = p->S * p->Hkv * p->max_nb;
    p->groups = 0;
    if (p->heads > 0) {
        // partitions of the (sequence, block) list; each workgroup walks a run
        const int64_t max_blocks = p->S * p->max_nb;
        int64_t groups = 1;
        if (P > 0) {
            p->chunk_units = P / p->bs;
            groups = max_blocks > 0 ? (max_blocks + p->chunk_units - 1) / p->chunk_units : 1;
        } else {
            // balanced: one chunk per workgroup the device holds at once
            p->chunk_units = 0;
            if (p->S > 0) {
                int cus = 0, per_cu = 0, rc;
                if ((rc = device_cu_count(&cus)) || (rc = resident_waves_per_cu(*p, &per_cu)))
                    return rc;
                groups = (int64_t)cus * (per_cu / p->heads);
                if (max_blocks > 0 && max_blocks < groups)
                    groups = max_blocks;
            }
        }
        if (groups > INT32_MAX / 16)
            return PA_ERR_UNSUPPORTED;
        p->groups = groups;
        p->waves = groups * p->heads;
    } else if (P > 0) {
        // fixed partitions: a chunk (and partial slot) for each partition of
        // the largest possible batch; the launch walks them in runs
        p->chunk_units = P / p->bs;
        p->waves = max_units > 0 ? (max_units + p->chunk_units - 1) / p->chunk_units : 1;
    } else {
        // balanced: one chunk per wavefront the device holds at once (half
        // that for bf16 caches), but no more wavefronts than the largest
        // batch of these shapes has units (a small batch then launches only
        // the wavefronts it can use)
        p->chunk_units = 0;
        p->waves = 1;
        if (p->S > 0) {
            int rc;
            if ((rc = balanced_chunks(*p, qm, &p->waves)))
                return rc;
            if (max_units > 0 && max_units < p->waves)
                p->waves = max_units;
        }
    }
    if (p->waves > INT32_MAX / 2 || p->chunk_units > INT32_MAX)
        return PA_ERR_UNSUPPORTED;
    p->slots = p->waves + p->S * p->Hkv;
    p->ws_bytes = p->S > 0 ? workspace_bytes(*p) : 0;
    return PA_OK;
}

// Whether HIP knows p as device memory (a host query of the runtime's
// allocation table: no device access, no synchronisation).  Pinned host
// memory, or a pointer the runtime does not know, is not; a failed query
// leaves no error behind for the launch check.
bool in_device_memory(const void *p)
{
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return at.type == hipMemoryTypeDevice;
}

// Shared validation and launch of pa_zero_blocks (src_bases == NULL) and
// pa_copy_blocks.
int block_op(const int32_t *ids, int64_t n, const void *const *src_bases,
             void *const *dst_bases, int32_t num_regions, int64_t block_stride,
             int64_t block_bytes, int64_t src_num_blocks, int64_t dst_num_blocks,
             const pa_opts *opts, void *hip_stream)
{
    const bool copy = src_bases != nullptr;
    if (n < 0 || num_regions < 0)
        return PA_ERR_SHAPE;
    if (n == 0 || num_regions == 0)
        return PA_OK;
    if (!ids || !dst_bases)
        return PA_ERR_NULL;
    if (block_stride <= 0 || block_bytes <= 0 || block_bytes > block_stride ||
        dst_num_blocks <= 0)
        return PA_ERR_SHAPE;
    if (block_stride % 16 || block_bytes % 16)
        return PA_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(ids) % (copy ? 8 : 4) ||
        reinterpret_cast<uintptr_t>(dst_bases) % 8 ||
        reinterpret_cast<uintptr_t>(src_bases) % 8)
        return PA_ERR_ALIGN;
    // every addressed byte offset, and the operation's total bytes, must fit int64
    const int64_t max_blocks = dst_num_blocks > src_num_blocks ? dst_num_blocks : src_num_blocks;
    int64_t item_regions = 0, total_bytes = 0;
    if (max_blocks > INT64_MAX / block_stride ||
        __builtin_mul_overflow(n, (int64_t)num_regions, &item_regions) ||
        __builtin_mul_overflow(item_regions, block_bytes, &total_bytes))
        return PA_ERR_UNSUPPORTED;

    BlockOpArgs a;
    a.ids = ids;
    a.dst_bases = dst_bases;
    a.src_bases = src_bases;
    a.err_flag = opts ? opts->err_flag : nullptr;
    a.num_items = n;
    a.block_stride = block_stride;
    a.block_bytes = block_bytes;
    a.dst_num_blocks = dst_num_blocks;
    a.src_num_blocks = copy ? src_num_blocks : 0;
    a.chunks = (block_bytes + block_op_chunk_bytes() - 1) / block_op_chunk_bytes();
    a.num_regions = num_regions;
    // Items per workgroup: enough workgroups to fill the device several times
    // over, but each reads its ids (possibly from host memory) only once.
    int cus = 0, rc;
    if ((rc = device_cu_count(&cus)))
        return rc;
    const int64_t units = item_regions * a.chunks;
    const int64_t target = 8 * (int64_t)cus;
    int64_t g = units / target;
    a.group_items = (int32_t)(g < 1 ? 1 : (g > kMaxGroupItems ? kMaxGroupItems : g));
    const int64_t groups = (n + a.group_items - 1) / a.group_items;
    if (groups > INT32_MAX / ((int64_t)num_regions * a.chunks))
        return PA_ERR_UNSUPPORTED;
    a.pieces = (int32_t)((block_bytes + block_op_piece_bytes() - 1) / block_op_piece_bytes());
    // Large operations with tables in device memory: one workgroup per (item,
    // region, piece).  Below 128 MiB the grouped kernel's fewer, longer
    // workgroups measured faster (a 57 MiB clear: 12.1 against 13.5 us).
    const int64_t pieces = item_regions * (int64_t)a.pieces;
    const bool large = total_bytes >= (int64_t(128) << 20);
    const bool device_tables = large && in_device_memory(ids) && in_device_memory(dst_bases) &&
                               (!copy || in_device_memory(src_bases));
    hipError_t e = device_tables && pieces <= INT32_MAX
                       ? launch_block_piece_op(a, copy, static_cast<hipStream_t>(hip_stream))
                       : launch_block_op(a, copy, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// Validation and arguments of pa_kv_append (and of pa_decode_append's append).
int plan_append(const pa_tensor *k, const pa_tensor *v, const pa_tensor *slot_mapping,
                const pa_tensor *key_cache, const pa_tensor *value_cache, const pa_opts *opts,
                AppendArgs *a, int *in_type, int *cache_type)
{
    int rc;
    if ((rc = check_tensor(k, 3, 16)) || (rc = check_tensor(v, 3, 16)) ||
        (rc = check_tensor(slot_mapping, 1, 8)) || (rc = check_tensor(key_cache, 4, 16)) ||
        (rc = check_tensor(value_cache, 4, 16)))
        return rc;
    if (slot_mapping->dtype != PA_I64)
        return PA_ERR_DTYPE;
    if (k->dtype != v->dtype || key_cache->dtype != value_cache->dtype)
        return PA_ERR_DTYPE;
    const int in_t = kv_type_of(k->dtype), cache_t = kv_type_of(key_cache->dtype);
    if (in_t < 0 || in_t == KT_E4M3 || cache_t < 0)
        return PA_ERR_DTYPE;
    if (cache_t != KT_E4M3 && cache_t != in_t)
        return PA_ERR_DTYPE;
    for (int i = 0; i < 3; ++i)
        if (k->shape[i] != v->shape[i])
            return PA_ERR_SHAPE;
    for (int i = 0; i < 4; ++i)
        if (key_cache->shape[i] != value_cache->shape[i])
            return PA_ERR_SHAPE;
    const int64_t T = k->shape[0], Hkv = k->shape[1], D = k->shape[2];
    if (slot_mapping->shape[0] != T || key_cache->shape[2] != Hkv || key_cache->shape[3] != D)
        return PA_ERR_SHAPE;
    if (!supported_head_dim(D) || !supported_block_size(key_cache->shape[1]))
        return PA_ERR_UNSUPPORTED;
    float ks = opts ? opts->k_scale : 1.0f, vs = opts ? opts->v_scale : 1.0f;
    if (cache_t == KT_E4M3 && !(isfinite(ks) && ks > 0.0f && isfinite(vs) && vs > 0.0f))
        return PA_ERR_UNSUPPORTED;
    a->k = k->data;
    a->v = v->data;
    a->slots = static_cast<const int64_t *>(slot_mapping->data);
    a->key_cache = key_cache->data;
    a->value_cache = value_cache->data;
    a->err_flag = opts ? opts->err_flag : nullptr;
    a->num_tokens = T;
    a->row_elems = Hkv * D;
    a->num_slots = key_cache->shape[0] * key_cache->shape[1];
    a->k_inv_scale = 1.0f / ks;
    a->v_inv_scale = 1.0f / vs;
    *in_type = in_t;
    *cache_type = cache_t;
    return PA_OK;
}

// pa_decode (qsl == NULL, qm == 0), pa_decode_multi, pa_decode_noalloc
// (use_static: the workspace is the library's static device buffer) and
// pa_decode_append (app: its append, validated; fused into the decode
// kernel where that kernel takes one, else launched before it).
int run_decode(const pa_tensor *q, const pa_tensor *qsl, int64_t qm, const pa_tensor *key_cache,
               const pa_tensor *value_cache, const pa_tensor *block_tables,
               const pa_tensor *seq_lens, float scale, pa_tensor *out, const pa_opts *opts,
               void *hip_stream, bool use_static = false, const AppendArgs *app = nullptr,
               int app_in_type = 0)
{
    int rc;
    if ((rc = check_tensor(q, 3, 16)) || (rc = check_tensor(key_cache, 4, 16)) ||
        (rc = check_tensor(value_cache, 4, 16)) || (rc = check_tensor(block_tables, 2, 4)) ||
        (rc = check_tensor(seq_lens, 1, 4)) || (rc = check_tensor(out, 3, 16)) ||
        (qsl && (rc = check_tensor(qsl, 1, 4))))
        return rc;
    if (value_cache->dtype != key_cache->dtype || out->dtype != q->dtype ||
        seq_lens->dtype != PA_I32 || (qsl && qsl->dtype != PA_I32))
        return PA_ERR_DTYPE;
    for (int i = 0; i < 4; ++i)
        if (value_cache->shape[i] != key_cache->shape[i])
            return PA_ERR_SHAPE;
    for (int i = 0; i < 3; ++i)
        if (out->shape[i] != q->shape[i])
            return PA_ERR_SHAPE;
    const int64_t S = qsl ? block_tables->shape[0] : q->shape[0];
    if (seq_lens->shape[0] != S || (qsl && qsl->shape[0] != S + 1))
        return PA_ERR_SHAPE;
    if (!isfinite(scale))
        return PA_ERR_UNSUPPORTED;
    // a call with work reads table entries, each of which must name a block
    if (S > 0 && q->shape[0] > 0 && key_cache->shape[0] < 1)
        return PA_ERR_SHAPE;
    const bool fp8 = key_cache->dtype == PA_FP8_E4M3;
    const float ks = (fp8 && opts) ? opts->k_scale : 1.0f;
    const float vs = (fp8 && opts) ? opts->v_scale : 1.0f;
    if (fp8 && !(isfinite(ks) && ks > 0.0f && isfinite(vs) && vs > 0.0f))
        return PA_ERR_UNSUPPORTED;
    DecodePlan p;
    if ((rc = plan_decode(q, key_cache, block_tables, opts, qm, &p)))
        return rc;
    if (p.S == 0 || p.T == 0) {
        if (app && app->num_tokens > 0 &&
            launch_kv_append(*app, app_in_type, p.kv_type,
                             static_cast<hipStream_t>(hip_stream)) != hipSuccess)
            return PA_ERR_HIP;
        return PA_OK;
    }
    pa_opts o;
    pa_opts_init(&o);
    if (opts)
        o = *opts;
    if (use_static) {
        if (p.ws_bytes > kStaticScratchBytes)
            return PA_ERR_SCRATCH;
        if ((rc = static_scratch(&o.workspace)))
            return rc;
        o.workspace_bytes = kStaticScratchBytes;
    }
    if (!o.workspace || o.workspace_bytes < p.ws_bytes)
        return PA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(o.workspace) % 16)
        return PA_ERR_ALIGN;

    DecodeArgs a;
    a.q = q->data;
    a.key_cache = key_cache->data;
    a.value_cache = value_cache->data;
    a.block_tables = static_cast<const int32_t *>(block_tables->data);
    a.seq_lens = static_cast<const int32_t *>(seq_lens->data);
    a.out = out->data;
    a.ws_acc = o.workspace;
    a.ws_ml = reinterpret_cast<float *>(static_cast<uint8_t *>(o.workspace) + acc_bytes(p));
    a.ws_seg = reinterpret_cast<int32_t *>(a.ws_ml + p.slots * p.rows * 2);
    a.err_flag = o.err_flag;
    a.num_seqs = (int32_t)p.S;
    a.num_heads = (int32_t)p.H;
    a.num_kv_heads = (int32_t)p.Hkv;
    a.max_nb = (int32_t)p.max_nb;
    a.num_blocks = (int32_t)p.NB;
    a.chunk_units = (int32_t)p.chunk_units;
    a.num_waves = (int32_t)p.waves;
    a.rows_per_slot = (int32_t)p.rows;
    a.query_start_loc = qsl ? static_cast<const int32_t *>(qsl->data) : nullptr;
    a.max_query_len = (int32_t)(qm > 0 ? qm : 1);
    a.num_tokens = (int32_t)p.T;
    a.log2_group = __builtin_ctz((unsigned)p.G);
    a.qk_scale_log2 = scale * kLog2e * ks;
    a.v_scale = vs;
    a.flags = p.acc_bf16 ? kPartialsBf16 : 0;
    a.slot_stride = p.heads > 0 ? (int32_t)p.heads : 1;
    a.num_slots = (int32_t)p.slots;
    // Fixed partitions on the per-wavefront kernels: the balanced split's
    // grid, each chunk an equal run of whole partitions whose softmax state
    // runs on across their boundaries (one partial per run and segment, not
    // per partition: the Qwen-shaped batch in 512-token partitions 137 -> 131
    // us, the balanced split's time; the Llama-shaped one 117 -> 115 us, its
    // 2.35 partitions per wavefront rounding up to runs of 3).  The
    // workspace keeps a slot per partition of the largest batch, so its size
    // needs no device query.
    if (p.heads == 0 && p.chunk_units > 0) {
        int64_t runs = 0;
        if ((rc = balanced_chunks(p, qm, &runs)))
            return rc;
        if (runs > 0 && runs < p.waves)
            a.num_waves = (int32_t)runs;
        a.flags |= kRuns;
    }
    // The matrix-core single-query kernels take one new bf16 row per
    // sequence themselves (a bf16 cache's new rows come in with the last
    // tile's own loads; an e4m3 cache's are read and encoded when that tile
    // is attended), where the batch has at most two (sequence, KV head)
    // segments per wavefront: there the work at each segment end costs less
    // than the append's own launch (Llama-shaped batch, 0.5 per wavefront:
    // step 107.3 against 110.4 us, the kernel unchanged; Qwen-shaped, 2:
    // 136.3 against 137.3 us, the kernel 2 % slower).  Any other append
    // runs as its own launch first.
    const bool fuse = app && p.variant == PA_VARIANT_MFMA && qm == 0 &&
                      app_in_type == KT_BF16 && app->num_tokens == p.S &&
                      p.S * p.Hkv <= 2 * (int64_t)a.num_waves;
    a.new_k = fuse ? app->k : nullptr;
    a.new_v = fuse ? app->v : nullptr;
    a.new_slots = fuse ? app->slots : nullptr;
    a.k_inv_scale = app ? app->k_inv_scale : 1.0f;
    a.v_inv_scale = app ? app->v_inv_scale : 1.0f;

    // Fixed partitions on the per-block e4m3 kernel: no more workgroups than
    // the device holds at once, each walking an equal run of partitions (the
    // workspace has a slot per partition, sized without the device).
    int64_t groups = p.groups;
    if (p.heads > 0 && p.chunk_units > 0) {
        int cus = 0, per_cu = 0;
        if ((rc = device_cu_count(&cus)) || (rc = resident_waves_per_cu(p, &per_cu)))
            return rc;
        const int64_t resident = (int64_t)cus * (per_cu / p.heads);
        if (resident > 0 && resident < groups)
            groups = resident;
    }

    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (app && !fuse && app->num_tokens > 0 &&
        launch_kv_append(*app, app_in_type, p.kv_type, stream) != hipSuccess)
        return PA_ERR_HIP;
    hipEvent_t ev0 = static_cast<hipEvent_t>(o.kernel_events[0]);
    hipEvent_t ev1 = static_cast<hipEvent_t>(o.kernel_events[1]);
    if (ev0 && hipEventRecord(ev0, stream) != hipSuccess)
        return PA_ERR_HIP;
    hipError_t e;
    if (qm > 0)
        e = launch_decode_mfma_multi(a, p.kv_type, (int)p.D, (int)p.bs, (int)p.col_tiles, stream);
    else if (p.heads > 0)
        e = launch_decode_mfma_heads(a, p.kv_type, (int)p.D, (int)p.bs, (int)p.G,
                                     (int)groups, stream);
    else if (p.variant == PA_VARIANT_MFMA)
        e = launch_decode_mfma(a, p.kv_type, (int)p.D, (int)p.bs, (int)p.G, stream);
    else
        e = launch_decode_valu(a, p.q_type, p.kv_type, (int)p.D, (int)p.bs, (int)p.G, stream);
    if (e != hipSuccess)
        return PA_ERR_HIP;
    if (ev1 && hipEventRecord(ev1, stream) != hipSuccess)
        return PA_ERR_HIP;
    e = launch_merge(a, p.q_type, (int)p.D, (int)p.bs, stream);
    if (e != hipSuccess)
        return PA_ERR_HIP;
    return PA_OK;
}

// A descriptor with another shape (data pointer and dtype kept); dense strides.
pa_tensor reshaped(const pa_tensor *t, std::initializer_list<int64_t> shape)
{
    pa_tensor r = *t;
    r.ndim = (int32_t)shape.size();
    int i = 0;
    for (int64_t n : shape)
        r.shape[i++] = n;
    int64_t acc = 1;
    for (int k = r.ndim - 1; k >= 0; --k) {
        r.stride[k] = acc;
        acc *= r.shape[k];
    }
    return r;
}

// The cascade's plan: the prefix pass's work items and partials, the suffix
// pass's tables, lengths and decode plan; workspace regions 256-byte aligned.
struct CascadePlan {
    DecodePlan suf;
    int64_t S, N, G, R, row_blocks, P, split_blocks, items, per_xcd;
    size_t acc_off, ml_off, suf_off, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int plan_cascade(const pa_tensor *q, const pa_tensor *kc, const pa_tensor *bt, int64_t N,
                 const pa_opts *opts, CascadePlan *c)
{
    if (!q || !kc || !bt)
        return PA_ERR_NULL;
    if (q->ndim != 3 || kc->ndim != 4 || bt->ndim != 2)
        return PA_ERR_SHAPE;
    const int64_t S = q->shape[0], max_nb = bt->shape[1];
    if (N < 1 || N >= max_nb)
        return PA_ERR_UNSUPPORTED;
    // token positions of the whole table row (prefix included) are int32
    if (kc->shape[1] > 0 && max_nb > INT32_MAX / kc->shape[1])
        return PA_ERR_UNSUPPORTED;
    if (q->shape[1] <= 0 || kc->shape[2] <= 0 || q->shape[1] % kc->shape[2])
        return PA_ERR_SHAPE;
    const int64_t G = q->shape[1] / kc->shape[2];
    if (!supported_group(G))
        return PA_ERR_UNSUPPORTED;
    pa_opts o;
    pa_opts_init(&o);
    if (opts)
        o = *opts;
    o.variant = PA_VARIANT_MFMA;
    const pa_tensor bt_suf = reshaped(bt, {S, max_nb - N});
    int rc;
    if ((rc = plan_decode(q, kc, &bt_suf, &o, 0, &c->suf, false)))
        return rc;
    if (c->suf.chunk_units == 0 && S > 0) {
        // balanced chunks: the suffix wavefronts the cascade kernel holds
        // beside the prefix workgroups
        int cus = 0, per_cu = 0;
        if ((rc = device_cu_count(&cus)) || (rc = resident_waves_per_cu(c->suf, &per_cu, true)))
            return rc;
        c->suf.waves = (int64_t)cus * per_cu;
        const int64_t max_units = c->suf.S * c->suf.Hkv * c->suf.max_nb;
        if (max_units > 0 && max_units < c->suf.waves)
            c->suf.waves = max_units;
        c->suf.slots = c->suf.waves + c->suf.S * c->suf.Hkv;
        c->suf.ws_bytes = workspace_bytes(c->suf);
    }
    const int64_t Hkv = c->suf.Hkv, D = c->suf.D;
    c->S = S;
    c->N = N;
    c->G = G;
    c->R = S * G;
    const int64_t rb = cascade_prefix_rows();
    c->row_blocks = (c->R + rb - 1) / rb;
    // Token splits of the prefix: about one workgroup per compute unit, at
    // most 64 blocks per split (a wavefront holds a split's block ids in one
    // register), no empty split.
    int cus = 1;
    if (S > 0 && (rc = device_cu_count(&cus)))
        return rc;
    const int64_t pairs = Hkv * (c->row_blocks > 0 ? c->row_blocks : 1);
    int64_t P = (cus + pairs - 1) / pairs;
    if (P < (N + 63) / 64)
        P = (N + 63) / 64;
    if (P > N)
        P = N;
    c->split_blocks = (N + P - 1) / P;
    c->P = (N + c->split_blocks - 1) / c->split_blocks;
    c->items = pairs * c->P;
    c->per_xcd = (c->items + 7) / 8;
    if (c->R > INT32_MAX / 2 || c->items > INT32_MAX / 2)
        return PA_ERR_UNSUPPORTED;
    const size_t prow = (size_t)(c->P * Hkv * c->R);
    c->acc_off = 0;
    c->ml_off = c->acc_off + align256((c->suf.acc_bf16 ? 2 : 4) * prow * (size_t)D);
    c->suf_off = c->ml_off + align256(sizeof(float) * prow * 2);
    c->total = S > 0 ? c->suf_off + align256(c->suf.ws_bytes) : 0;
    return PA_OK;
}

}  // namespace

extern "C" {

void pa_opts_init(pa_opts *opts)
{
    if (!opts)
        return;
    memset(opts, 0, sizeof *opts);
    opts->k_scale = 1.0f;
    opts->v_scale = 1.0f;
    opts->variant = PA_VARIANT_AUTO;
}

int pa_version(void) { return PA_VERSION; }

const char *pa_status_string(int status)
{
    switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required descriptor or data pointer is NULL";
    case PA_ERR_DTYPE: return "dtype or dtype combination not supported";
    case PA_ERR_SHAPE: return "tensor ranks or sizes are inconsistent";
    case PA_ERR_LAYOUT: return "tensor strides are not dense row-major";
    case PA_ERR_ALIGN: return "data pointer not 16-byte aligned";
    case PA_ERR_UNSUPPORTED: return "head_dim, block_size, group size or option not supported";
    case PA_ERR_WORKSPACE: return "split-KV workspace missing or too small";
    case PA_ERR_HIP: return "the HIP runtime reported an error";
    case PA_ERR_SCRATCH:
        return "the call needs more workspace than the static buffer of pa_decode_noalloc holds";
    default: return "unknown status";
    }
}

int pa_kv_append(const pa_tensor *k, const pa_tensor *v, const pa_tensor *slot_mapping,
                 pa_tensor *key_cache, pa_tensor *value_cache, const pa_opts *opts,
                 void *hip_stream)
{
    AppendArgs a;
    int in_t = 0, cache_t = 0;
    int rc = plan_append(k, v, slot_mapping, key_cache, value_cache, opts, &a, &in_t, &cache_t);
    if (rc || a.num_tokens == 0)
        return rc;
    hipError_t e = launch_kv_append(a, in_t, cache_t, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_zero_blocks(const int32_t *block_ids, int64_t num_ids, void *const *region_bases,
                   int32_t num_regions, int64_t block_stride, int64_t block_bytes,
                   int64_t num_blocks, const pa_opts *opts, void *hip_stream)
{
    return block_op(block_ids, num_ids, nullptr, region_bases, num_regions, block_stride,
                    block_bytes, 0, num_blocks, opts, hip_stream);
}

int pa_copy_blocks(const int32_t *block_pairs, int64_t num_pairs, const void *const *src_bases,
                   void *const *dst_bases, int32_t num_regions, int64_t block_stride,
                   int64_t block_bytes, int64_t src_num_blocks, int64_t dst_num_blocks,
                   const pa_opts *opts, void *hip_stream)
{
    if (num_pairs > 0 && num_regions > 0 && !src_bases)
        return PA_ERR_NULL;
    if (src_num_blocks <= 0 && num_pairs > 0)
        return PA_ERR_SHAPE;
    return block_op(block_pairs, num_pairs, src_bases, dst_bases, num_regions, block_stride,
                    block_bytes, src_num_blocks, dst_num_blocks, opts, hip_stream);
}

int pa_prepare_step(const int32_t *idx_mapping, const int32_t *num_scheduled, int32_t num_reqs,
                    const pa_step_state *state, int32_t block_size, int32_t num_blocks,
                    const pa_step_inputs *out, const pa_opts *opts, void *hip_stream)
{
    if (!idx_mapping || !num_scheduled || !state || !out || !state->num_computed ||
        !state->block_table || !state->token_ids || !out->query_start_loc || !out->seq_lens ||
        !out->block_tables ||
        (out->max_tokens > 0 && (!out->positions || !out->input_ids || !out->slot_mapping)))
        return PA_ERR_NULL;
    if (num_reqs < 1 || state->num_rows < 1 || state->max_blocks < 1 || state->max_len < 1 ||
        out->max_tokens < 0 || block_size < 1 || num_blocks < 1)
        return PA_ERR_SHAPE;
    if (num_reqs > kMaxPrepReqs)
        return PA_ERR_UNSUPPORTED;
    const void *p4[] = {idx_mapping, num_scheduled, state->num_computed, state->block_table,
                        state->token_ids, out->query_start_loc, out->seq_lens, out->input_ids,
                        out->block_tables};
    for (const void *p : p4)
        if (reinterpret_cast<uintptr_t>(p) % 4)
            return PA_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(out->positions) % 8 ||
        reinterpret_cast<uintptr_t>(out->slot_mapping) % 8)
        return PA_ERR_ALIGN;
    StepPrepArgs a;
    a.idx_mapping = idx_mapping;
    a.num_scheduled = num_scheduled;
    a.num_computed = state->num_computed;
    a.block_table = state->block_table;
    a.token_ids = state->token_ids;
    a.query_start_loc = out->query_start_loc;
    a.seq_lens = out->seq_lens;
    a.positions = out->positions;
    a.input_ids = out->input_ids;
    a.slot_mapping = out->slot_mapping;
    a.block_tables = out->block_tables;
    a.err_flag = opts ? opts->err_flag : nullptr;
    a.num_reqs = num_reqs;
    a.num_rows = state->num_rows;
    a.max_blocks = state->max_blocks;
    a.max_len = state->max_len;
    a.max_tokens = out->max_tokens;
    a.block_size = block_size;
    a.num_blocks = num_blocks;
    hipError_t e = launch_step_prep(a, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_decode_workspace_size(const pa_tensor *q, const pa_tensor *key_cache,
                             const pa_tensor *block_tables, const pa_opts *opts, size_t *bytes)
{
    if (!bytes)
        return PA_ERR_NULL;
    DecodePlan p;
    int rc = plan_decode(q, key_cache, block_tables, opts, 0, &p);
    if (rc)
        return rc;
    *bytes = p.ws_bytes;
    return PA_OK;
}

int pa_decode_multi_workspace_size(const pa_tensor *q, int32_t max_query_len,
                                   const pa_tensor *key_cache, const pa_tensor *block_tables,
                                   const pa_opts *opts, size_t *bytes)
{
    if (!bytes)
        return PA_ERR_NULL;
    if (max_query_len < 1)
        return PA_ERR_UNSUPPORTED;
    DecodePlan p;
    int rc = plan_decode(q, key_cache, block_tables, opts, max_query_len, &p);
    if (rc)
        return rc;
    *bytes = p.ws_bytes;
    return PA_OK;
}

int pa_decode(const pa_tensor *q, const pa_tensor *key_cache, const pa_tensor *value_cache,
              const pa_tensor *block_tables, const pa_tensor *seq_lens, float scale,
              pa_tensor *out, const pa_opts *opts, void *hip_stream)
{
    return run_decode(q, nullptr, 0, key_cache, value_cache, block_tables, seq_lens, scale, out,
                      opts, hip_stream);
}

int pa_decode_append(const pa_tensor *k, const pa_tensor *v, const pa_tensor *slot_mapping,
                     const pa_tensor *q, pa_tensor *key_cache, pa_tensor *value_cache,
                     const pa_tensor *block_tables, const pa_tensor *seq_lens, float scale,
                     pa_tensor *out, const pa_opts *opts, void *hip_stream)
{
    AppendArgs app;
    int in_t = 0, cache_t = 0;
    int rc = plan_append(k, v, slot_mapping, key_cache, value_cache, opts, &app, &in_t, &cache_t);
    if (rc)
        return rc;
    return run_decode(q, nullptr, 0, key_cache, value_cache, block_tables, seq_lens, scale, out,
                      opts, hip_stream, false, &app, in_t);
}

int pa_decode_noalloc(const pa_tensor *q, const pa_tensor *key_cache, const pa_tensor *value_cache,
                      const pa_tensor *block_tables, const pa_tensor *seq_lens, float scale,
                      pa_tensor *out, const pa_opts *opts, void *hip_stream)
{
    return run_decode(q, nullptr, 0, key_cache, value_cache, block_tables, seq_lens, scale, out,
                      opts, hip_stream, true);
}

int pa_decode_cascade_workspace_size(const pa_tensor *q, const pa_tensor *key_cache,
                                     const pa_tensor *block_tables, int32_t prefix_blocks,
                                     const pa_opts *opts, size_t *bytes)
{
    if (!bytes)
        return PA_ERR_NULL;
    if (prefix_blocks == 0)
        return pa_decode_workspace_size(q, key_cache, block_tables, opts, bytes);
    CascadePlan c;
    int rc = plan_cascade(q, key_cache, block_tables, prefix_blocks, opts, &c);
    if (rc)
        return rc;
    *bytes = c.total;
    return PA_OK;
}

int pa_decode_cascade(const pa_tensor *q, const pa_tensor *key_cache,
                      const pa_tensor *value_cache, const pa_tensor *block_tables,
                      const pa_tensor *seq_lens, int32_t prefix_blocks, float scale,
                      pa_tensor *out, const pa_opts *opts, void *hip_stream)
{
    if (prefix_blocks == 0)
        return pa_decode(q, key_cache, value_cache, block_tables, seq_lens, scale, out, opts,
                         hip_stream);
    if (prefix_blocks < 0)
        return PA_ERR_UNSUPPORTED;
    int rc;
    if ((rc = check_tensor(q, 3, 16)) || (rc = check_tensor(key_cache, 4, 16)) ||
        (rc = check_tensor(value_cache, 4, 16)) || (rc = check_tensor(block_tables, 2, 4)) ||
        (rc = check_tensor(seq_lens, 1, 4)) || (rc = check_tensor(out, 3, 16)))
        return rc;
    if (value_cache->dtype != key_cache->dtype || out->dtype != q->dtype ||
        seq_lens->dtype != PA_I32)
        return PA_ERR_DTYPE;
    for (int i = 0; i < 4; ++i)
        if (value_cache->shape[i] != key_cache->shape[i])
            return PA_ERR_SHAPE;
    for (int i = 0; i < 3; ++i)
        if (out->shape[i] != q->shape[i])
            return PA_ERR_SHAPE;
    if (seq_lens->shape[0] != q->shape[0] || block_tables->shape[0] != q->shape[0])
        return PA_ERR_SHAPE;
    if (!isfinite(scale))
        return PA_ERR_UNSUPPORTED;
    if (q->dtype != PA_BF16 || (opts && opts->variant == PA_VARIANT_VALU))
        return PA_ERR_UNSUPPORTED;
    if (q->shape[0] > 0 && key_cache->shape[0] < 1)
        return PA_ERR_SHAPE;
    const bool fp8 = key_cache->dtype == PA_FP8_E4M3;
    const float ks = (fp8 && opts) ? opts->k_scale : 1.0f;
    const float vs = (fp8 && opts) ? opts->v_scale : 1.0f;
    if (fp8 && !(isfinite(ks) && ks > 0.0f && isfinite(vs) && vs > 0.0f))
        return PA_ERR_UNSUPPORTED;
    CascadePlan c;
    if ((rc = plan_cascade(q, key_cache, block_tables, prefix_blocks, opts, &c)))
        return rc;
    if (c.S == 0)
        return PA_OK;
    if (!opts || !opts->workspace || opts->workspace_bytes < c.total)
        return PA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(opts->workspace) % 16)
        return PA_ERR_ALIGN;
    const DecodePlan &sp = c.suf;
    uint8_t *ws = static_cast<uint8_t *>(opts->workspace);

    CascadePrefixArgs pr;
    pr.q = q->data;
    pr.key_cache = key_cache->data;
    pr.value_cache = value_cache->data;
    pr.block_tables = static_cast<const int32_t *>(block_tables->data);
    pr.seq_lens = static_cast<const int32_t *>(seq_lens->data);
    pr.p_acc = ws + c.acc_off;
    pr.p_ml = reinterpret_cast<float *>(ws + c.ml_off);
    pr.err_flag = opts->err_flag;
    pr.num_seqs = (int32_t)c.S;
    pr.num_heads = (int32_t)sp.H;
    pr.num_kv_heads = (int32_t)sp.Hkv;
    pr.max_nb = (int32_t)block_tables->shape[1];
    pr.num_blocks = (int32_t)sp.NB;
    pr.block_size = (int32_t)sp.bs;
    pr.prefix_blocks = (int32_t)c.N;
    pr.num_splits = (int32_t)c.P;
    pr.split_blocks = (int32_t)c.split_blocks;
    pr.rows = (int32_t)c.R;
    pr.row_blocks = (int32_t)c.row_blocks;
    pr.num_items = (int32_t)c.items;
    pr.items_per_xcd = (int32_t)c.per_xcd;
    pr.log2_group = __builtin_ctz((unsigned)c.G);
    pr.check_wgs = 0;   // the launcher sizes the check
    pr.partials_bf16 = sp.acc_bf16;
    pr.qk_scale_log2 = scale * kLog2e * ks;
    pr.v_scale = vs;

    // suffix pass: single-query decode wavefronts over the batch viewed from
    // block N on, partials only
    DecodeArgs sa;
    sa.q = q->data;
    sa.key_cache = key_cache->data;
    sa.value_cache = value_cache->data;
    sa.block_tables = pr.block_tables + c.N;
    sa.seq_lens = pr.seq_lens;
    sa.out = out->data;
    sa.ws_acc = ws + c.suf_off;
    sa.ws_ml = reinterpret_cast<float *>(ws + c.suf_off + acc_bytes(sp));
    sa.ws_seg = reinterpret_cast<int32_t *>(sa.ws_ml + sp.slots * sp.rows * 2);
    sa.err_flag = opts->err_flag;
    sa.num_seqs = (int32_t)sp.S;
    sa.num_heads = (int32_t)sp.H;
    sa.num_kv_heads = (int32_t)sp.Hkv;
    sa.max_nb = (int32_t)sp.max_nb;
    sa.num_blocks = (int32_t)sp.NB;
    sa.chunk_units = (int32_t)sp.chunk_units;
    sa.num_waves = (int32_t)sp.waves;
    sa.rows_per_slot = (int32_t)sp.rows;
    sa.query_start_loc = nullptr;
    sa.max_query_len = 1;
    sa.num_tokens = (int32_t)sp.T;
    sa.log2_group = __builtin_ctz((unsigned)sp.G);
    sa.qk_scale_log2 = scale * kLog2e * ks;
    sa.v_scale = vs;
    sa.flags = kPartialOnly | (sp.acc_bf16 ? kPartialsBf16 : 0);
    sa.slot_stride = 1;
    sa.num_slots = (int32_t)sp.slots;
    sa.new_k = sa.new_v = nullptr;
    sa.new_slots = nullptr;
    sa.k_inv_scale = sa.v_inv_scale = 1.0f;

    CascadeMergeArgs ma;
    ma.out = out->data;
    ma.s_acc = sa.ws_acc;
    ma.s_ml = sa.ws_ml;
    ma.s_seg = sa.ws_seg;
    ma.seq_lens = pr.seq_lens;
    ma.prefix_tokens = (int32_t)(c.N * sp.bs);
    ma.capacity = pr.max_nb * pr.block_size;
    ma.p_acc = pr.p_acc;
    ma.p_ml = pr.p_ml;
    ma.num_seqs = (int32_t)c.S;
    ma.num_heads = (int32_t)sp.H;
    ma.num_kv_heads = (int32_t)sp.Hkv;
    ma.num_splits = (int32_t)c.P;
    ma.partials_bf16 = sp.acc_bf16;
    ma.num_slots = (int32_t)sp.slots;

    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    hipEvent_t ev0 = static_cast<hipEvent_t>(opts->kernel_events[0]);
    hipEvent_t ev1 = static_cast<hipEvent_t>(opts->kernel_events[1]);
    if (ev0 && hipEventRecord(ev0, stream) != hipSuccess)
        return PA_ERR_HIP;
    hipError_t e;
    if ((e = launch_cascade(pr, sa, sp.kv_type, (int)sp.D, (int)sp.bs, (int)sp.G, stream)) !=
        hipSuccess)
        return PA_ERR_HIP;
    if (ev1 && hipEventRecord(ev1, stream) != hipSuccess)
        return PA_ERR_HIP;
    e = launch_cascade_merge(ma, sp.q_type, (int)sp.D, stream);
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_decode_multi(const pa_tensor *q, const pa_tensor *query_start_loc, int32_t max_query_len,
                    const pa_tensor *key_cache, const pa_tensor *value_cache,
                    const pa_tensor *block_tables, const pa_tensor *seq_lens, float scale,
                    pa_tensor *out, const pa_opts *opts, void *hip_stream)
{
    if (!query_start_loc)
        return PA_ERR_NULL;
    if (max_query_len < 1)
        return PA_ERR_UNSUPPORTED;
    return run_decode(q, query_start_loc, max_query_len, key_cache, value_cache, block_tables,
                      seq_lens, scale, out, opts, hip_stream);
}

}  // extern "C"
