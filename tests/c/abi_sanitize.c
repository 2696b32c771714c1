/*
 * Calls every entry point of libpa.so on its host-side validation paths:
 * descriptors and options that each entry point must refuse, nothing-to-do
 * calls, and workspace-size queries that need no device.  Built with
 * AddressSanitizer and UndefinedBehaviorSanitizer (host code only), so the
 * library's descriptor checks and launch planning are checked for bad host
 * memory accesses.  No call here launches a kernel; the data pointers are a
 * fake aligned address that is never dereferenced.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pa.h"

#define FAKE ((void *)(uintptr_t)0x7F0000000000ull)

static int failures = 0;
#define EXPECT(call, want)                                                                     \
    do {                                                                                       \
        int rc_ = (call);                                                                      \
        if (rc_ != (want)) {                                                                   \
            printf("line %d: %s returned %d, expected %d\n", __LINE__, #call, rc_, (want));   \
            ++failures;                                                                        \
        }                                                                                      \
    } while (0)

static pa_tensor desc(int ndim, const int64_t *shape, int dtype, void *data)
{
    pa_tensor t;
    memset(&t, 0, sizeof t);
    t.data = data;
    t.dtype = dtype;
    t.ndim = ndim;
    int64_t acc = 1;
    for (int i = ndim - 1; i >= 0; --i) {
        t.shape[i] = shape[i];
        t.stride[i] = acc;
        acc *= shape[i];
    }
    return t;
}

struct dec {
    pa_tensor q, kc, vc, bt, lens, out;
};

static struct dec decode_args(int64_t S, int64_t H, int64_t Hkv, int64_t D, int64_t bs, int64_t NB,
                              int64_t max_nb, int qd, int kd)
{
    struct dec a;
    const int64_t qs[3] = {S, H, D}, cs[4] = {NB, bs, Hkv, D}, bts[2] = {S, max_nb}, ls[1] = {S};
    a.q = desc(3, qs, qd, FAKE);
    a.kc = desc(4, cs, kd, FAKE);
    a.vc = desc(4, cs, kd, FAKE);
    a.bt = desc(2, bts, PA_I32, FAKE);
    a.lens = desc(1, ls, PA_I32, FAKE);
    a.out = desc(3, qs, qd, FAKE);
    return a;
}

static int call_decode(struct dec *a, const pa_opts *o, float scale)
{
    return pa_decode(&a->q, &a->kc, &a->vc, &a->bt, &a->lens, scale, &a->out, o, NULL);
}

int main(void)
{
    pa_opts o, fixed;
    memset(&o, 0xFF, sizeof o);
    pa_opts_init(&o);
    if (o.k_scale != 1.0f || o.partials != PA_PARTIALS_F32 || o.workspace || o.kernel_events[0])
        ++failures;
    pa_opts_init(&fixed);
    fixed.partition_tokens = 32;
    if (pa_version() != PA_VERSION)
        ++failures;
    for (int s = 0; s <= 10; ++s)
        if (!pa_status_string(s) || !pa_status_string(s)[0])
            ++failures;
    (void)pa_status_string(-1);

    /* decode */
    struct dec a = decode_args(2, 8, 2, 64, 16, 10, 4, PA_F32, PA_F32);
    struct dec z = decode_args(0, 8, 2, 64, 16, 10, 4, PA_F32, PA_F32);
    EXPECT(call_decode(&z, &fixed, 0.125f), PA_OK);
    EXPECT(pa_decode(NULL, &a.kc, &a.vc, &a.bt, &a.lens, 0.125f, &a.out, NULL, NULL), PA_ERR_NULL);
    struct dec b = decode_args(2, 8, 2, 64, 16, 10, 4, PA_BF16, PA_F32);
    EXPECT(call_decode(&b, NULL, 0.125f), PA_ERR_DTYPE);
    struct dec c = decode_args(2, 6, 4, 64, 16, 10, 4, PA_F32, PA_F32);
    EXPECT(call_decode(&c, NULL, 0.125f), PA_ERR_SHAPE);
    struct dec d = a;
    d.kc.stride[1] = 3;
    EXPECT(call_decode(&d, NULL, 0.125f), PA_ERR_LAYOUT);
    struct dec e = a;
    e.q.data = (char *)FAKE + 4;
    EXPECT(call_decode(&e, NULL, 0.125f), PA_ERR_ALIGN);
    struct dec f = decode_args(2, 8, 2, 96, 16, 10, 4, PA_F32, PA_F32);
    EXPECT(call_decode(&f, NULL, 0.125f), PA_ERR_UNSUPPORTED);
    EXPECT(call_decode(&a, NULL, 0.0f / 0.0f), PA_ERR_UNSUPPORTED);
    pa_opts bad = fixed;
    bad.partials = 5;
    EXPECT(call_decode(&a, &bad, 0.125f), PA_ERR_UNSUPPORTED);
    bad = fixed;
    bad.partition_tokens = 24;
    EXPECT(call_decode(&a, &bad, 0.125f), PA_ERR_UNSUPPORTED);
    EXPECT(call_decode(&a, &fixed, 0.125f), PA_ERR_WORKSPACE);
    struct dec empty = decode_args(2, 8, 2, 64, 16, 0, 4, PA_F32, PA_F32);
    EXPECT(call_decode(&empty, &fixed, 0.125f), PA_ERR_SHAPE);
    struct dec f8 = decode_args(8, 64, 8, 128, 32, 32768, 4096, PA_BF16, PA_FP8_E4M3);
    bad = fixed;
    bad.k_scale = 0.0f;
    EXPECT(call_decode(&f8, &bad, 0.125f), PA_ERR_UNSUPPORTED);

    size_t n = 0;
    EXPECT(pa_decode_workspace_size(&a.q, &a.kc, &a.bt, &fixed, &n), PA_OK);
    EXPECT(pa_decode_workspace_size(&a.q, &a.kc, &a.bt, &fixed, NULL), PA_ERR_NULL);
    EXPECT(pa_decode_workspace_size(NULL, &a.kc, &a.bt, &fixed, &n), PA_ERR_NULL);
    pa_opts bp = fixed;
    bp.partials = PA_PARTIALS_BF16;
    EXPECT(pa_decode_workspace_size(&f8.q, &f8.kc, &f8.bt, &bp, &n), PA_OK);

    /* the allocation-free variant */
    EXPECT(pa_decode_noalloc(&z.q, &z.kc, &z.vc, &z.bt, &z.lens, 0.125f, &z.out, NULL, NULL), PA_OK);
    EXPECT(pa_decode_noalloc(&b.q, &b.kc, &b.vc, &b.bt, &b.lens, 0.125f, &b.out, NULL, NULL),
           PA_ERR_DTYPE);
    EXPECT(pa_decode_noalloc(&f8.q, &f8.kc, &f8.vc, &f8.bt, &f8.lens, 0.125f, &f8.out, &fixed, NULL),
           PA_ERR_SCRATCH);

    /* multi-token decode */
    struct dec m = decode_args(10, 8, 2, 128, 16, 10, 4, PA_BF16, PA_BF16);
    const int64_t s3[1] = {3}, s4[1] = {4};
    m.bt = desc(2, (const int64_t[]){3, 4}, PA_I32, FAKE);
    m.lens = desc(1, s3, PA_I32, FAKE);
    pa_tensor qsl = desc(1, s4, PA_I32, FAKE);
    EXPECT(pa_decode_multi(&m.q, NULL, 4, &m.kc, &m.vc, &m.bt, &m.lens, 0.1f, &m.out, NULL, NULL),
           PA_ERR_NULL);
    EXPECT(pa_decode_multi(&m.q, &qsl, 0, &m.kc, &m.vc, &m.bt, &m.lens, 0.1f, &m.out, NULL, NULL),
           PA_ERR_UNSUPPORTED);
    EXPECT(pa_decode_multi(&m.q, &qsl, 17, &m.kc, &m.vc, &m.bt, &m.lens, 0.1f, &m.out, NULL, NULL),
           PA_ERR_UNSUPPORTED);
    EXPECT(pa_decode_multi(&m.q, &qsl, 4, &m.kc, &m.vc, &m.bt, &m.lens, 0.1f, &m.out, &fixed, NULL),
           PA_ERR_WORKSPACE);
    EXPECT(pa_decode_multi_workspace_size(&m.q, 4, &m.kc, &m.bt, &fixed, &n), PA_OK);
    EXPECT(pa_decode_multi_workspace_size(&m.q, 0, &m.kc, &m.bt, &fixed, &n), PA_ERR_UNSUPPORTED);

    /* cascade */
    struct dec cs = decode_args(4, 8, 2, 128, 16, 10, 8, PA_BF16, PA_BF16);
    EXPECT(pa_decode_cascade(&cs.q, &cs.kc, &cs.vc, &cs.bt, &cs.lens, -1, 0.1f, &cs.out, NULL, NULL),
           PA_ERR_UNSUPPORTED);
    EXPECT(pa_decode_cascade(&cs.q, &cs.kc, &cs.vc, &cs.bt, &cs.lens, 8, 0.1f, &cs.out, NULL, NULL),
           PA_ERR_UNSUPPORTED);
    EXPECT(pa_decode_cascade(&a.q, &a.kc, &a.vc, &a.bt, &a.lens, 2, 0.1f, &a.out, NULL, NULL),
           PA_ERR_UNSUPPORTED);
    struct dec ce = decode_args(4, 8, 2, 128, 16, 0, 8, PA_BF16, PA_BF16);
    EXPECT(pa_decode_cascade(&ce.q, &ce.kc, &ce.vc, &ce.bt, &ce.lens, 2, 0.1f, &ce.out, NULL, NULL),
           PA_ERR_SHAPE);
    EXPECT(pa_decode_cascade_workspace_size(&cs.q, &cs.kc, &cs.bt, 0, &fixed, &n), PA_OK);
    EXPECT(pa_decode_cascade_workspace_size(&cs.q, &cs.kc, &cs.bt, 1, &fixed, NULL), PA_ERR_NULL);

    /* append */
    const int64_t ks[3] = {4, 2, 64}, cache[4] = {10, 16, 2, 64}, sl[1] = {4};
    pa_tensor k = desc(3, ks, PA_BF16, FAKE), kc = desc(4, cache, PA_BF16, FAKE);
    pa_tensor slots = desc(1, sl, PA_I64, FAKE), slots32 = desc(1, sl, PA_I32, FAKE);
    pa_tensor k0 = desc(3, (const int64_t[]){0, 2, 64}, PA_BF16, FAKE);
    pa_tensor s0 = desc(1, (const int64_t[]){0}, PA_I64, FAKE);
    EXPECT(pa_kv_append(&k0, &k0, &s0, &kc, &kc, NULL, NULL), PA_OK);
    EXPECT(pa_kv_append(NULL, &k, &slots, &kc, &kc, NULL, NULL), PA_ERR_NULL);
    EXPECT(pa_kv_append(&k, &k, &slots32, &kc, &kc, NULL, NULL), PA_ERR_DTYPE);
    pa_tensor c8 = desc(4, cache, PA_FP8_E4M3, FAKE);
    bad = fixed;
    bad.v_scale = 1.0f / 0.0f;
    EXPECT(pa_kv_append(&k, &k, &slots, &c8, &c8, &bad, NULL), PA_ERR_UNSUPPORTED);

    /* block operations */
    EXPECT(pa_zero_blocks(FAKE, 0, FAKE, 4, 4096, 4096, 100, NULL, NULL), PA_OK);
    EXPECT(pa_zero_blocks(NULL, 5, FAKE, 4, 4096, 4096, 100, NULL, NULL), PA_ERR_NULL);
    EXPECT(pa_zero_blocks(FAKE, 5, FAKE, 4, 4096, 8192, 100, NULL, NULL), PA_ERR_SHAPE);
    EXPECT(pa_zero_blocks(FAKE, 5, FAKE, 4, 4100, 4096, 100, NULL, NULL), PA_ERR_ALIGN);
    EXPECT(pa_zero_blocks(FAKE, (int64_t)1 << 55, FAKE, 4, 4096, 4096, 100, NULL, NULL),
           PA_ERR_UNSUPPORTED);
    EXPECT(pa_copy_blocks(FAKE, 5, NULL, FAKE, 4, 4096, 4096, 100, 100, NULL, NULL), PA_ERR_NULL);
    EXPECT(pa_copy_blocks(FAKE, 5, FAKE, FAKE, 4, 4096, 4096, 0, 100, NULL, NULL), PA_ERR_SHAPE);

    /* step metadata */
    pa_step_state st = {FAKE, FAKE, FAKE, 10, 8, 128};
    pa_step_inputs io = {FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64};
    EXPECT(pa_prepare_step(NULL, FAKE, 4, &st, 16, 100, &io, NULL, NULL), PA_ERR_NULL);
    EXPECT(pa_prepare_step(FAKE, FAKE, 0, &st, 16, 100, &io, NULL, NULL), PA_ERR_SHAPE);
    EXPECT(pa_prepare_step(FAKE, FAKE, 4096, &st, 16, 100, &io, NULL, NULL), PA_ERR_UNSUPPORTED);
    EXPECT(pa_prepare_step((const int32_t *)((char *)FAKE + 2), FAKE, 4, &st, 16, 100, &io, NULL, NULL),
           PA_ERR_ALIGN);

    printf("C ABI sanitizer run: %d failure(s)\n", failures);
    return failures != 0;
}
