/*
 * Drives the host side of the C ABI (include/moe.h) under AddressSanitizer
 * and UndefinedBehaviorSanitizer, with no GPU: the test-suite links this file
 * with the library's objects, the C-ABI source compiled with both sanitizers
 * on its host side, and runs it.
 *
 * Only host work is reached: workspace and kernel-count queries, status
 * strings, stage names, and every argument check that refuses a call before
 * anything is enqueued (no call here reaches a device call).  Pointers are a
 * fake aligned address that these calls only test and never dereference.
 * Each call's status is checked against the header's contract.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"

#define FAKE ((void *)(uintptr_t)0x10000)
#define FAKE_AT(off) ((void *)((uintptr_t)0x10000 + (off)))

static int failures;

static void expect(long got, long want, const char *what, int line)
{
    if (got != want) {
        fprintf(stderr, "line %d: %s: got %ld, want %ld\n", line, what, got, want);
        failures++;
    }
}
#define EXPECT(call, want) expect((long)(call), (long)(want), #call, __LINE__)

static moe_dims dims(int32_t T, int32_t H, int32_t E, int32_t k, int32_t I, int32_t Is)
{
    moe_dims d;
    d.T = T;
    d.H = H;
    d.E = E;
    d.top_k = k;
    d.I = I;
    d.I_shared = Is;
    d.group = 64;
    d.sb_dtype = MOE_BF16;
    d.out_dtype = MOE_F32;
    return d;
}

static moe_dims qwen(int32_t T) { return dims(T, 2048, 256, 8, 512, 512); }

static moe_qmat qmat(uintptr_t off)
{
    moe_qmat m;
    m.q = FAKE_AT(off);
    m.scale = FAKE_AT(off);
    m.bias = FAKE_AT(off);
    return m;
}

static moe_weights weights(int shared)
{
    moe_weights w;
    memset(&w, 0, sizeof w);
    w.router = FAKE;
    w.experts.gate = w.experts.up = w.experts.down = qmat(0);
    if (shared)
        w.shared.gate = w.shared.up = w.shared.down = qmat(0);
    return w;
}

static void status_strings(void)
{
    for (int s = -8; s <= 2; s++) {
        const char *t = moe_status_string((moe_status)s);
        if (!t || !t[0]) {
            fprintf(stderr, "status %d has no text\n", s);
            failures++;
        }
    }
}

static void workspace_sizes(void)
{
    static const int32_t Ts[] = {0, 1, 2, 3, 63, 64, 65, 511, 512, 4096, 1 << 20, 1 << 22};
    size_t prev = 0;
    for (size_t i = 0; i < sizeof Ts / sizeof Ts[0]; i++) {
        moe_dims d = qwen(Ts[i]);
        const size_t n = moe_workspace_size(&d);
        if (n == 0 || n < prev) {
            fprintf(stderr, "workspace for T=%d: %zu after %zu\n", Ts[i], n, prev);
            failures++;
        }
        prev = n;
        const int32_t stages = moe_layer_stage_count(&d);
        if (Ts[i] == 0)
            EXPECT(stages, 0);
        else if (stages < 1)
            failures++;
        EXPECT(moe_layer_stage_name(&d, -1) == NULL, 1);
        EXPECT(moe_layer_stage_name(&d, stages) == NULL, 1);
        for (int32_t s = 0; s < stages; s++) {
            const char *name = moe_layer_stage_name(&d, s);
            if (!name || !name[0]) {
                fprintf(stderr, "stage %d of T=%d has no name\n", s, Ts[i]);
                failures++;
            }
        }
    }
    moe_dims over = qwen((1 << 22) + 1);
    EXPECT(moe_workspace_size(&over), 0);
    EXPECT(moe_workspace_size(NULL), 0);
    EXPECT(moe_layer_stage_count(NULL), 0);
    EXPECT(moe_layer_stage_name(NULL, 0) == NULL, 1);
    moe_dims small = dims(5, 64, 8, 2, 64, 0);
    if (moe_workspace_size(&small) == 0)
        failures++;
}

static void invalid_dims(void)
{
    struct {
        int field; /* 0 H, 1 I, 2 top_k, 3 T, 4 E, 5 group, 6 I_shared, 7 out_dtype, 8 sb_dtype */
        int32_t value;
        moe_status status;
    } cases[] = {
        {0, 100, MOE_ERR_SHAPE},      {1, 96, MOE_ERR_SHAPE},          {2, 0, MOE_ERR_SHAPE},
        {2, 300, MOE_ERR_SHAPE},      {3, -1, MOE_ERR_SHAPE},          {4, 0, MOE_ERR_SHAPE},
        {5, 32, MOE_ERR_UNSUPPORTED}, {4, 512, MOE_ERR_UNSUPPORTED},   {2, 9, MOE_ERR_UNSUPPORTED},
        {0, 32768, MOE_ERR_UNSUPPORTED}, {6, 1024, MOE_ERR_UNSUPPORTED}, {7, 5, MOE_ERR_SHAPE},
        {8, 7, MOE_ERR_SHAPE},        {5, 0, MOE_ERR_SHAPE},           {6, -64, MOE_ERR_SHAPE},
        {0, INT32_MAX, MOE_ERR_SHAPE}, {3, INT32_MAX, MOE_ERR_UNSUPPORTED},
    };
    for (size_t i = 0; i < sizeof cases / sizeof cases[0]; i++) {
        moe_dims d = qwen(8);
        int32_t *f[] = {&d.H, &d.I, &d.top_k, &d.T, &d.E, &d.group, &d.I_shared, &d.out_dtype, &d.sb_dtype};
        *f[cases[i].field] = cases[i].value;
        EXPECT(moe_workspace_size(&d), 0);
        EXPECT(moe_layer_stage_count(&d), 0);
        EXPECT(moe_permute(&d, FAKE, FAKE, FAKE, FAKE, FAKE, (size_t)1 << 30, NULL), cases[i].status);
        EXPECT(moe_route(&d, FAKE, FAKE, NULL, FAKE, FAKE, NULL), cases[i].status);
        moe_weights w = weights(1);
        EXPECT(moe_layer(&d, &w, FAKE, FAKE, NULL, NULL, NULL, FAKE, (size_t)1 << 30, NULL), cases[i].status);
    }
}

static void layer_checks(void)
{
    moe_dims d = qwen(8);
    const size_t need = moe_workspace_size(&d);
    moe_weights w = weights(1);
    EXPECT(moe_layer(&d, NULL, FAKE, FAKE, NULL, NULL, NULL, FAKE, need, NULL), MOE_ERR_NULL);
    EXPECT(moe_layer(&d, &w, NULL, FAKE, NULL, NULL, NULL, FAKE, need, NULL), MOE_ERR_NULL);
    EXPECT(moe_layer(&d, &w, FAKE_AT(2), FAKE, NULL, NULL, NULL, FAKE, need, NULL), MOE_ERR_ALIGN);
    EXPECT(moe_layer(&d, &w, FAKE, FAKE, NULL, NULL, NULL, FAKE_AT(16), need, NULL), MOE_ERR_ALIGN);
    EXPECT(moe_layer(&d, &w, FAKE, FAKE, NULL, NULL, NULL, FAKE, need - 1, NULL), MOE_ERR_WORKSPACE);
    EXPECT(moe_layer(&d, &w, FAKE, FAKE, NULL, NULL, NULL, NULL, need, NULL), MOE_ERR_NULL);
    EXPECT(moe_layer(NULL, &w, FAKE, FAKE, NULL, NULL, NULL, FAKE, need, NULL), MOE_ERR_NULL);
    EXPECT(moe_layer(&d, &w, FAKE, FAKE, FAKE_AT(4), NULL, NULL, FAKE, need, NULL), MOE_ERR_ALIGN);
    moe_weights bad = weights(1);
    bad.experts.down.scale = NULL;
    EXPECT(moe_layer(&d, &bad, FAKE, FAKE, NULL, NULL, NULL, FAKE, need, NULL), MOE_ERR_NULL);
    bad = weights(1);
    bad.experts.up.q = FAKE_AT(4);
    EXPECT(moe_layer(&d, &bad, FAKE, FAKE, NULL, NULL, NULL, FAKE, need, NULL), MOE_ERR_ALIGN);
    moe_weights noshared = weights(0);
    EXPECT(moe_layer(&d, &noshared, FAKE, FAKE, NULL, NULL, NULL, FAKE, need, NULL), MOE_ERR_NULL);
    moe_dims d0 = d;
    d0.I_shared = 0;
    EXPECT(moe_layer(&d0, &w, FAKE, FAKE, NULL, NULL, NULL, FAKE, need, NULL), MOE_ERR_SHAPE);
    /* shared expert gate */
    w.shared_expert_gate = FAKE_AT(2);
    EXPECT(moe_layer(&d, &w, FAKE, FAKE, NULL, NULL, NULL, FAKE, need, NULL), MOE_ERR_ALIGN);
    noshared.shared_expert_gate = FAKE;
    EXPECT(moe_layer(&d0, &noshared, FAKE, FAKE, NULL, NULL, NULL, FAKE, need, NULL), MOE_ERR_SHAPE);
    /* 8-bit router */
    w = weights(1);
    w.router_q8 = FAKE;
    w.router_scale = FAKE;
    w.router_bias = FAKE;
    EXPECT(moe_layer(&d, &w, FAKE, FAKE, NULL, NULL, NULL, FAKE, need, NULL), MOE_ERR_SHAPE);
    w.router = NULL;
    w.router_scale = NULL;
    EXPECT(moe_layer(&d, &w, FAKE, FAKE, NULL, NULL, NULL, FAKE, need, NULL), MOE_ERR_NULL);
    w.router_scale = FAKE_AT(4);
    EXPECT(moe_layer(&d, &w, FAKE, FAKE, NULL, NULL, NULL, FAKE, need, NULL), MOE_ERR_ALIGN);
    w.router_q8 = NULL;
    w.router_scale = FAKE;
    EXPECT(moe_layer(&d, &w, FAKE, FAKE, NULL, NULL, NULL, FAKE, need, NULL), MOE_ERR_NULL);
    /* empty calls enqueue nothing */
    moe_dims e = qwen(0);
    EXPECT(moe_layer(&e, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), MOE_OK);
    EXPECT(moe_route(&e, NULL, NULL, NULL, NULL, NULL, NULL), MOE_OK);
    EXPECT(moe_combine(&e, NULL, NULL, NULL, NULL, NULL), MOE_OK);
    EXPECT(moe_shared_gate(&e, NULL, NULL, NULL, NULL), MOE_OK);
    EXPECT(moe_combine_gated(&e, NULL, NULL, NULL, NULL, NULL, NULL), MOE_OK);
    /* the output dtype of each entry point */
    moe_dims d16 = d;
    d16.out_dtype = MOE_BF16;
    w = weights(1);
    EXPECT(moe_layer(&d16, &w, FAKE, FAKE, NULL, NULL, NULL, FAKE, need, NULL), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_layer_residual(&d, &w, FAKE, NULL, FAKE, FAKE, need, NULL), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_layer_residual(&d16, &w, FAKE, NULL, NULL, FAKE, need, NULL), MOE_ERR_NULL);
    EXPECT(moe_layer_residual(&d16, &w, FAKE, FAKE_AT(2), FAKE, FAKE, need, NULL), MOE_ERR_ALIGN);
    EXPECT(moe_layer_residual(&d16, &w, FAKE, NULL, FAKE, FAKE, need - 1, NULL), MOE_ERR_WORKSPACE);
    moe_dims e16 = e;
    e16.out_dtype = MOE_BF16;
    EXPECT(moe_layer_residual(&e16, NULL, NULL, NULL, NULL, NULL, 0, NULL), MOE_OK);
    /* events */
    hipEvent_t ev[16];
    for (int i = 0; i < 16; i++)
        ev[i] = (hipEvent_t)FAKE;
    const int32_t stages = moe_layer_stage_count(&d);
    EXPECT(moe_layer_events(&d, &w, FAKE, FAKE, NULL, NULL, NULL, FAKE, need, NULL, NULL, 0), MOE_ERR_NULL);
    EXPECT(moe_layer_events(&d, &w, FAKE, FAKE, NULL, NULL, NULL, FAKE, need, NULL, ev, stages), MOE_ERR_SHAPE);
    ev[stages] = NULL;
    EXPECT(moe_layer_events(&d, &w, FAKE, FAKE, NULL, NULL, NULL, FAKE, need, NULL, ev, stages + 1), MOE_ERR_NULL);
}

static void other_call_checks(void)
{
    moe_dims d = qwen(8);
    const size_t need = moe_workspace_size(&d);
    moe_ffn f;
    f.gate = f.up = f.down = qmat(0);
    EXPECT(moe_route(&d, FAKE, FAKE, FAKE_AT(8), FAKE, FAKE, NULL), MOE_ERR_ALIGN);
    EXPECT(moe_route(&d, FAKE, NULL, NULL, FAKE, FAKE, NULL), MOE_ERR_NULL);
    EXPECT(moe_permute(&d, FAKE, FAKE, FAKE, FAKE, FAKE, need - 256, NULL), MOE_ERR_WORKSPACE);
    EXPECT(moe_expert_ffn(&d, FAKE, FAKE, FAKE, NULL, NULL, FAKE, NULL, FAKE, need, NULL), MOE_ERR_NULL);
    EXPECT(moe_expert_ffn(&d, FAKE, FAKE, FAKE, &f, NULL, NULL, NULL, FAKE, need, NULL), MOE_ERR_NULL);
    EXPECT(moe_combine(&d, FAKE, FAKE, FAKE_AT(4), FAKE, NULL), MOE_ERR_ALIGN);
    EXPECT(moe_combine(&d, FAKE, NULL, NULL, FAKE, NULL), MOE_ERR_NULL);
    EXPECT(moe_shared_gate(&d, FAKE, NULL, FAKE, NULL), MOE_ERR_NULL);
    EXPECT(moe_shared_gate(&d, FAKE, FAKE_AT(2), FAKE, NULL), MOE_ERR_ALIGN);
    EXPECT(moe_combine_gated(&d, FAKE, FAKE, FAKE, FAKE_AT(4), FAKE, NULL), MOE_ERR_ALIGN);
    EXPECT(moe_combine_gated(&d, NULL, FAKE, NULL, NULL, FAKE, NULL), MOE_ERR_NULL);
    EXPECT(moe_router_dequant(&d, FAKE, FAKE, NULL, FAKE, NULL), MOE_ERR_NULL);
    EXPECT(moe_router_dequant(&d, FAKE_AT(8), FAKE, FAKE, FAKE, NULL), MOE_ERR_ALIGN);
    moe_dims bad = d;
    bad.H = 100;
    EXPECT(moe_router_dequant(&bad, FAKE, FAKE, FAKE, FAKE, NULL), MOE_ERR_SHAPE);
    /* moe_permute sorts at most 2^22 slots in one call */
    moe_dims big = qwen(1 << 20);
    big.top_k = 4;
    EXPECT(moe_permute(&big, FAKE, FAKE, FAKE, FAKE, FAKE, moe_workspace_size(&big) - 256, NULL),
           MOE_ERR_WORKSPACE);
    big.top_k = 5;
    EXPECT(moe_permute(&big, FAKE, FAKE, FAKE, FAKE, FAKE, (size_t)1 << 40, NULL), MOE_ERR_UNSUPPORTED);
}

static void stack_checks(void)
{
    moe_dims d = qwen(1);
    d.out_dtype = MOE_BF16;
    const size_t need = moe_workspace_size(&d);
    moe_weights w = weights(1);
    moe_dims two = d;
    two.T = 2;
    EXPECT(moe_decode_stack(&two, &w, NULL, NULL, 2, FAKE, FAKE, NULL, NULL, NULL, NULL, NULL, FAKE, need, NULL),
           MOE_ERR_UNSUPPORTED);
    EXPECT(moe_decode_stack(&d, &w, NULL, NULL, 0, FAKE, FAKE, NULL, NULL, NULL, NULL, NULL, FAKE, need, NULL),
           MOE_ERR_SHAPE);
    EXPECT(moe_decode_stack(&d, NULL, NULL, NULL, 2, FAKE, FAKE, NULL, NULL, NULL, NULL, NULL, FAKE, need, NULL),
           MOE_ERR_NULL);
    moe_dims f32 = d;
    f32.out_dtype = MOE_F32;
    EXPECT(moe_decode_stack(&f32, &w, NULL, NULL, 2, FAKE, FAKE, NULL, NULL, NULL, NULL, NULL, FAKE, need, NULL),
           MOE_ERR_UNSUPPORTED);
    moe_dims odd = d;
    odd.I = 384;
    odd.I_shared = 384;
    EXPECT(moe_decode_stack(&odd, &w, NULL, NULL, 2, FAKE, FAKE, NULL, NULL, NULL, NULL, NULL, FAKE, need, NULL),
           MOE_ERR_UNSUPPORTED);
    moe_weights q8 = w;
    q8.router_q8 = FAKE;
    EXPECT(moe_decode_stack(&d, &q8, NULL, NULL, 2, FAKE, FAKE, NULL, NULL, NULL, NULL, NULL, FAKE, need, NULL),
           MOE_ERR_UNSUPPORTED);
    EXPECT(moe_decode_stack(&d, &w, NULL, NULL, 2, NULL, FAKE, NULL, NULL, NULL, NULL, NULL, FAKE, need, NULL),
           MOE_ERR_NULL);
    EXPECT(moe_decode_stack(&d, &w, FAKE_AT(2), NULL, 2, FAKE, FAKE, NULL, NULL, NULL, NULL, NULL, FAKE, need,
                            NULL),
           MOE_ERR_ALIGN);
    moe_layer_strides st;
    memset(&st, 0, sizeof st);
    st.experts.down.scale = 8;
    EXPECT(moe_decode_stack(&d, &w, NULL, &st, 2, FAKE, FAKE, NULL, NULL, NULL, NULL, NULL, FAKE, need, NULL),
           MOE_ERR_ALIGN);
    st.experts.down.scale = 0;
    st.logit_bias = 2;
    EXPECT(moe_decode_stack(&d, &w, NULL, &st, 2, FAKE, FAKE, NULL, NULL, NULL, NULL, NULL, FAKE, need, NULL),
           MOE_ERR_ALIGN);
    st.logit_bias = 4;
    EXPECT(moe_decode_stack(&d, &w, NULL, &st, 2, FAKE, FAKE, NULL, NULL, NULL, NULL, NULL, FAKE, need - 1, NULL),
           MOE_ERR_WORKSPACE);
    EXPECT(moe_decode_stack(&d, &w, NULL, NULL, 2, FAKE, FAKE, NULL, NULL, NULL, NULL, NULL, FAKE, need - 1, NULL),
           MOE_ERR_WORKSPACE);
    moe_dims e = d;
    e.T = 0;
    EXPECT(moe_decode_stack(&e, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL),
           MOE_OK);
}

static void no_alloc_checks(void)
{
    moe_dims big = qwen(1024);
    moe_weights w = weights(1);
    if (moe_workspace_size(&big) <= MOE_NO_ALLOC_SCRATCH_BYTES)
        failures++;
    EXPECT(moe_layer_no_alloc(&big, &w, FAKE, FAKE, NULL, NULL, NULL, NULL), MOE_ERR_WORKSPACE);
    moe_dims d16 = qwen(8);
    d16.out_dtype = MOE_BF16;
    EXPECT(moe_layer_no_alloc(&d16, &w, FAKE, FAKE, NULL, NULL, NULL, NULL), MOE_ERR_UNSUPPORTED);
    moe_dims e = qwen(0);
    EXPECT(moe_layer_no_alloc(&e, NULL, NULL, NULL, NULL, NULL, NULL, NULL), MOE_OK);
    EXPECT(moe_layer_no_alloc(NULL, &w, FAKE, FAKE, NULL, NULL, NULL, NULL), MOE_ERR_NULL);
}

static moe_gqa_dims gqa(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S)
{
    moe_gqa_dims g;
    g.B = B;
    g.n_q_heads = Hq;
    g.n_kv_heads = Hkv;
    g.head_dim = D;
    g.max_seq = S;
    return g;
}

static void gqa_checks(void)
{
    moe_gqa_dims ok = gqa(32, 16, 2, 256, 32768);
    const size_t need = moe_gqa_workspace_size(&ok);
    if (need == 0)
        failures++;
    /* the largest dims the header allows: the size must not wrap */
    moe_gqa_dims top = gqa(65535, 16 * 65535, 65535, 256, 1 << 24);
    const size_t top_need = moe_gqa_workspace_size(&top);
    if (top_need < need || top_need < ((size_t)65535 * 65535 * 65536))
        failures++;
    const moe_gqa_dims bad[] = {
        gqa(-1, 16, 2, 256, 8), gqa(1, 0, 2, 256, 8),  gqa(1, 16, 0, 256, 8), gqa(1, 16, 3, 256, 8),
        gqa(1, 16, 2, 0, 8),    gqa(1, 16, 2, 256, 0), gqa(1, 34, 2, 256, 8), gqa(1, 16, 2, 96, 8),
        gqa(65536, 16, 2, 256, 8), gqa(1, 16, 2, 256, (1 << 24) + 1),
    };
    for (size_t i = 0; i < sizeof bad / sizeof bad[0]; i++) {
        EXPECT(moe_gqa_workspace_size(&bad[i]), 0);
        EXPECT(moe_gqa_decode_kernels(&bad[i]), 0);
        if (moe_gqa_decode(&bad[i], FAKE, FAKE, FAKE, FAKE, 0.125f, FAKE, FAKE, (size_t)1 << 40, NULL) >= 0)
            failures++;
    }
    EXPECT(moe_gqa_workspace_size(NULL), 0);
    moe_gqa_dims none = gqa(0, 16, 2, 256, 8);
    EXPECT(moe_gqa_decode_kernels(&none), 0);
    EXPECT(moe_gqa_decode(&none, NULL, NULL, NULL, NULL, 0.125f, NULL, NULL, 0, NULL), MOE_OK);
    EXPECT(moe_gqa_decode(&ok, FAKE, FAKE, FAKE, FAKE, NAN, FAKE, FAKE, need, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_gqa_decode(&ok, FAKE, FAKE, FAKE, FAKE, INFINITY, FAKE, FAKE, need, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_gqa_decode(&ok, FAKE, FAKE, FAKE, NULL, 0.125f, FAKE, FAKE, need, NULL), MOE_ERR_NULL);
    EXPECT(moe_gqa_decode(&ok, FAKE, FAKE, FAKE, FAKE_AT(2), 0.125f, FAKE, FAKE, need, NULL), MOE_ERR_ALIGN);
    EXPECT(moe_gqa_decode(&ok, FAKE_AT(8), FAKE, FAKE, FAKE, 0.125f, FAKE, FAKE, need, NULL), MOE_ERR_ALIGN);
    EXPECT(moe_gqa_decode(&ok, FAKE, FAKE, FAKE, FAKE, 0.125f, FAKE, NULL, need, NULL), MOE_ERR_NULL);
    EXPECT(moe_gqa_decode(&ok, FAKE, FAKE, FAKE, FAKE, 0.125f, FAKE, FAKE_AT(16), need, NULL), MOE_ERR_ALIGN);
    EXPECT(moe_gqa_decode(&ok, FAKE, FAKE, FAKE, FAKE, 0.125f, FAKE, FAKE, need - 1, NULL), MOE_ERR_WORKSPACE);
    hipEvent_t ev[3] = {(hipEvent_t)FAKE, (hipEvent_t)FAKE, (hipEvent_t)FAKE};
    EXPECT(moe_gqa_decode_events(&ok, FAKE, FAKE, FAKE, FAKE, 0.125f, FAKE, FAKE, need, NULL, NULL, 3),
           MOE_ERR_NULL);
    EXPECT(moe_gqa_decode_events(&ok, FAKE, FAKE, FAKE, FAKE, 0.125f, FAKE, FAKE, need, NULL, ev, 2), MOE_ERR_SHAPE);
    EXPECT(moe_gqa_decode_events(&ok, FAKE, FAKE, FAKE, FAKE, 0.125f, FAKE, FAKE, need - 1, NULL, ev, 3),
           MOE_ERR_WORKSPACE);
}

int main(void)
{
    status_strings();
    workspace_sizes();
    invalid_dims();
    layer_checks();
    other_call_checks();
    stack_checks();
    no_alloc_checks();
    gqa_checks();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("C-ABI host sanitizer driver: all checks passed\n");
    return 0;
}
