/*
 * Runs every function of the C oracle (oracle/moe_oracle.c) on small seeded
 * inputs under AddressSanitizer and UndefinedBehaviorSanitizer: the test-suite
 * compiles this file together with the oracle, with both sanitizers on and
 * recovery off, so an out-of-bounds access, a leak or undefined arithmetic
 * ends the run with a report and a nonzero status.
 *
 * Every buffer is allocated at its exact size, so an access one element past
 * its end is caught.  The cases cover the degenerate inputs the method has:
 * no tokens, a listed subset of tokens, top_k == E, experts that receive no
 * token, equal logits, sequences with no cached rows and lengths beyond the
 * cache (clamped).  A few cheap invariants are checked on the way (weights of
 * a token sum to one, the permutation is a permutation); the values
 * themselves are the oracle's own pinned tests' business.
 *
 * Inputs come from splitmix64; they are input synthesis only and hold none of
 * the method's arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

static uint64_t rng_state;

static uint64_t next_u64(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* uniform in [lo, hi) */
static float uniform(float lo, float hi) { return lo + (hi - lo) * (float)((next_u64() >> 40) * 0x1p-24); }

/* the upper half of a float32: a bfloat16 bit pattern (input synthesis) */
static uint16_t bf16_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static void *xmalloc(size_t bytes)
{
    /* one byte for an empty buffer, so every pointer is distinct and valid */
    void *p = malloc(bytes ? bytes : 1);
    if (!p) {
        fprintf(stderr, "out of host memory\n");
        exit(2);
    }
    return p;
}

static uint16_t *bf16_array(size_t n, float lo, float hi)
{
    uint16_t *p = xmalloc(n * sizeof *p);
    for (size_t i = 0; i < n; i++)
        p[i] = bf16_bits(uniform(lo, hi));
    return p;
}

static uint32_t *word_array(size_t n)
{
    uint32_t *p = xmalloc(n * sizeof *p);
    for (size_t i = 0; i < n; i++)
        p[i] = (uint32_t)next_u64();
    return p;
}

/* scales (positive) or biases, as float32 or bfloat16 bit patterns */
static void *sb_array(size_t n, int bf16, float lo, float hi)
{
    if (bf16)
        return bf16_array(n, lo, hi);
    float *p = xmalloc(n * sizeof *p);
    for (size_t i = 0; i < n; i++)
        p[i] = uniform(lo, hi);
    return p;
}

static int failures;

static void check(int ok, const char *what, int case_id)
{
    if (!ok) {
        fprintf(stderr, "case %d: %s\n", case_id, what);
        failures++;
    }
}

typedef struct {
    int32_t T, H, E, k, I, shared, sb_bf16, gate, bias, n_tok;
} layer_case;

static void run_layer(const layer_case *c, int id)
{
    const int32_t T = c->T, H = c->H, E = c->E, k = c->k, I = c->I, G = 64;
    const int32_t Is = c->shared ? I : 0;
    oracle_layer L;
    memset(&L, 0, sizeof L);
    L.T = T;
    L.H = H;
    L.E = E;
    L.top_k = k;
    L.I = I;
    L.I_shared = Is;
    L.group = G;
    L.sb_bf16 = c->sb_bf16;
    uint16_t *x = bf16_array((size_t)T * H, -1.0f, 1.0f);
    uint16_t *router = bf16_array((size_t)E * H, -0.2f, 0.2f);
    float *bias = NULL;
    if (c->bias) {
        bias = xmalloc(sizeof(float) * (size_t)E);
        for (int32_t e = 0; e < E; e++)
            bias[e] = uniform(-0.5f, 0.5f);
    }
    L.x = x;
    L.router = router;
    L.logit_bias = bias;
    uint32_t *gq = word_array((size_t)E * I * (H / 8)), *uq = word_array((size_t)E * I * (H / 8));
    uint32_t *dq = word_array((size_t)E * H * (I / 8));
    void *gs = sb_array((size_t)E * I * (H / G), c->sb_bf16, 0.002f, 0.02f);
    void *gb = sb_array((size_t)E * I * (H / G), c->sb_bf16, -0.1f, 0.0f);
    void *us = sb_array((size_t)E * I * (H / G), c->sb_bf16, 0.002f, 0.02f);
    void *ub = sb_array((size_t)E * I * (H / G), c->sb_bf16, -0.1f, 0.0f);
    void *ds = sb_array((size_t)E * H * (I / G), c->sb_bf16, 0.002f, 0.02f);
    void *db = sb_array((size_t)E * H * (I / G), c->sb_bf16, -0.1f, 0.0f);
    L.gate_q = gq;
    L.up_q = uq;
    L.down_q = dq;
    L.gate_s = gs;
    L.gate_b = gb;
    L.up_s = us;
    L.up_b = ub;
    L.down_s = ds;
    L.down_b = db;
    uint32_t *sgq = NULL, *suq = NULL, *sdq = NULL;
    void *sgs = NULL, *sgb = NULL, *sus = NULL, *sub = NULL, *sds = NULL, *sdb = NULL;
    uint16_t *sgate = NULL;
    if (Is) {
        sgq = word_array((size_t)Is * (H / 8));
        suq = word_array((size_t)Is * (H / 8));
        sdq = word_array((size_t)H * (Is / 8));
        sgs = sb_array((size_t)Is * (H / G), c->sb_bf16, 0.002f, 0.02f);
        sgb = sb_array((size_t)Is * (H / G), c->sb_bf16, -0.1f, 0.0f);
        sus = sb_array((size_t)Is * (H / G), c->sb_bf16, 0.002f, 0.02f);
        sub = sb_array((size_t)Is * (H / G), c->sb_bf16, -0.1f, 0.0f);
        sds = sb_array((size_t)H * (Is / G), c->sb_bf16, 0.002f, 0.02f);
        sdb = sb_array((size_t)H * (Is / G), c->sb_bf16, -0.1f, 0.0f);
        if (c->gate)
            sgate = bf16_array((size_t)H, -0.1f, 0.1f);
    }
    L.sh_gate_q = sgq;
    L.sh_up_q = suq;
    L.sh_down_q = sdq;
    L.sh_gate_s = sgs;
    L.sh_gate_b = sgb;
    L.sh_up_s = sus;
    L.sh_up_b = sub;
    L.sh_down_s = sds;
    L.sh_down_b = sdb;
    L.sh_expert_gate = sgate;

    /* listed tokens: all (tok NULL) or every other token, last first */
    int32_t *tok = NULL;
    int32_t nt = T;
    if (c->n_tok >= 0) {
        nt = c->n_tok;
        tok = xmalloc(sizeof(int32_t) * (size_t)nt);
        for (int32_t i = 0; i < nt; i++)
            tok[i] = T - 1 - 2 * i;
    }
    double *out = xmalloc(sizeof(double) * (size_t)nt * H);
    double *logits = xmalloc(sizeof(double) * (size_t)T * E);
    int32_t *idx = xmalloc(sizeof(int32_t) * (size_t)T * k);
    double *w = xmalloc(sizeof(double) * (size_t)T * k);
    int32_t *counts = xmalloc(sizeof(int32_t) * (size_t)E);
    int32_t *offsets = xmalloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *sorted = xmalloc(sizeof(int32_t) * (size_t)T * k);

    check(oracle_moe_layer(&L, nt, tok, out, logits, idx, w, counts, offsets, sorted) == 0, "layer status", id);
    /* the nullable outputs left to the oracle's own buffers */
    double *out2 = xmalloc(sizeof(double) * (size_t)nt * H);
    check(oracle_moe_layer(&L, nt, tok, out2, NULL, idx, w, counts, offsets, NULL) == 0, "layer status 2", id);
    check(nt == 0 || memcmp(out, out2, sizeof(double) * (size_t)nt * H) == 0, "nullable outputs change out", id);

    for (int32_t t = 0; t < T; t++) {
        double s = 0.0;
        for (int32_t j = 0; j < k; j++) {
            const int32_t e = idx[(size_t)t * k + j];
            check(e >= 0 && e < E, "expert index in range", id);
            for (int32_t i = 0; i < j; i++)
                check(idx[(size_t)t * k + i] != e, "experts of a token distinct", id);
            s += w[(size_t)t * k + j];
        }
        check(fabs(s - 1.0) < 1e-12, "weights sum to one", id);
    }
    check(offsets[0] == 0 && offsets[E] == T * k, "offsets span the slots", id);
    unsigned char *seen = calloc((size_t)T * k + 1, 1);
    for (int32_t r = 0; r < T * k; r++) {
        const int32_t s = sorted[r];
        check(s >= 0 && s < T * k && !seen[s], "sorted slots a permutation", id);
        if (s >= 0 && s < T * k)
            seen[s] = 1;
    }
    for (size_t i = 0; i < (size_t)nt * H; i++)
        check(isfinite(out[i]), "finite output", id);

    free(seen);
    free(out2);
    free(sorted);
    free(offsets);
    free(counts);
    free(w);
    free(idx);
    free(logits);
    free(out);
    free(tok);
    free(sgate);
    free(sdb);
    free(sds);
    free(sub);
    free(sus);
    free(sgb);
    free(sgs);
    free(sdq);
    free(suq);
    free(sgq);
    free(db);
    free(ds);
    free(ub);
    free(us);
    free(gb);
    free(gs);
    free(dq);
    free(uq);
    free(gq);
    free(bias);
    free(router);
    free(x);
}

static void run_gqa(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S_max, const int32_t *lens, int id)
{
    uint16_t *q = bf16_array((size_t)B * Hq * D, -1.0f, 1.0f);
    uint16_t *kc = bf16_array((size_t)B * Hkv * S_max * D, -1.0f, 1.0f);
    uint16_t *vc = bf16_array((size_t)B * Hkv * S_max * D, -1.0f, 1.0f);
    int32_t *len = xmalloc(sizeof(int32_t) * (size_t)B);
    memcpy(len, lens, sizeof(int32_t) * (size_t)B);
    double *out = xmalloc(sizeof(double) * (size_t)B * Hq * D);
    check(oracle_gqa_decode(B, Hq, Hkv, D, S_max, q, kc, vc, len, 1.0 / sqrt((double)D), out) == 0, "gqa status",
          id);
    for (int32_t b = 0; b < B; b++)
        for (size_t i = 0; i < (size_t)Hq * D; i++) {
            const double o = out[(size_t)b * Hq * D + i];
            check(isfinite(o) && fabs(o) <= 1.0, "gqa output a convex mix of v", id);
            if (lens[b] <= 0)
                check(o == 0.0, "no rows give zeros", id);
        }
    free(out);
    free(len);
    free(vc);
    free(kc);
    free(q);
}

static void run_small_functions(void)
{
    /* root-mean-square normalisation with and without gamma */
    const int32_t H = 128;
    uint16_t *x = bf16_array(H, -2.0f, 2.0f), *g = bf16_array(H, 0.5f, 1.5f);
    uint16_t *o = xmalloc(sizeof(uint16_t) * H);
    oracle_rmsnorm(H, x, g, 1e-6, o);
    oracle_rmsnorm(H, x, NULL, 1e-6, o);
    free(o);
    free(g);
    free(x);

    /* 8-bit router restored to bfloat16, float32 and bfloat16 scales */
    for (int bf = 0; bf < 2; bf++) {
        const int32_t E = 3;
        uint32_t *codes = word_array((size_t)E * (H / 4));
        void *s = sb_array((size_t)E * (H / 64), bf, 0.001f, 0.01f);
        void *b = sb_array((size_t)E * (H / 64), bf, -0.5f, 0.5f);
        uint16_t *r = xmalloc(sizeof(uint16_t) * (size_t)E * H);
        oracle_router_dequant_q8(E, H, codes, s, b, bf, r);
        free(r);
        free(b);
        free(s);
        free(codes);
    }

    /* selection on equal logits: the lowest indices, in order */
    {
        const int32_t T = 2, E = 6, k = 3;
        double *l = xmalloc(sizeof(double) * T * E);
        for (int32_t i = 0; i < T * E; i++)
            l[i] = 0.25;
        int32_t *idx = xmalloc(sizeof(int32_t) * T * k);
        double *w = xmalloc(sizeof(double) * T * k);
        oracle_select(T, E, k, l, idx, w);
        for (int32_t t = 0; t < T; t++)
            for (int32_t j = 0; j < k; j++) {
                check(idx[t * k + j] == j, "equal logits keep the lowest indices", 100);
                check(fabs(w[t * k + j] - 1.0 / k) < 1e-15, "equal logits share the weight", 100);
            }
        free(w);
        free(idx);
        free(l);
    }

    /* permutation with no slots and with experts that receive none */
    {
        const int32_t E = 5;
        int32_t counts[5], offsets[6];
        oracle_permute(0, 2, E, NULL, counts, offsets, NULL);
        check(offsets[E] == 0, "empty permutation", 101);
        int32_t *idx = xmalloc(sizeof(int32_t) * 6);
        const int32_t pick[6] = {4, 0, 4, 4, 0, 4};
        memcpy(idx, pick, sizeof pick);
        int32_t *sorted = xmalloc(sizeof(int32_t) * 6);
        oracle_permute(3, 2, E, idx, counts, offsets, sorted);
        check(counts[0] == 2 && counts[1] == 0 && counts[4] == 4, "counts", 101);
        check(sorted[0] == 1 && sorted[1] == 4 && sorted[2] == 0 && sorted[5] == 5, "stable order", 101);
        free(sorted);
        free(idx);
    }

    /* one 4-bit code read back at every position of a word */
    {
        uint32_t *q = xmalloc(sizeof(uint32_t) * 2);
        q[0] = 0x76543210u;
        q[1] = 0xFEDCBA98u;
        oracle_qmat m;
        memset(&m, 0, sizeof m);
        m.q = q;
        m.N = 1;
        m.K = 16;
        m.group = 16;
        for (int32_t k = 0; k < 16; k++)
            check(oracle_code(&m, 0, k) == k, "code position", 102);
        free(q);
    }
}

int main(void)
{
    rng_state = 20260612u;
    static const layer_case cases[] = {
        /* T    H    E  k    I  sh bf gate bias n_tok */
        {0, 128, 8, 2, 64, 1, 1, 1, 0, -1},   /* no tokens */
        {1, 64, 4, 1, 64, 0, 0, 0, 0, -1},    /* one token, no shared expert */
        {5, 128, 8, 3, 128, 1, 1, 1, 1, -1},  /* ragged, shared expert with its gate, logit offsets */
        {7, 128, 16, 4, 64, 1, 0, 0, 0, 3},   /* a listed subset of the tokens, float32 scales */
        {3, 64, 2, 2, 64, 1, 1, 0, 1, -1},    /* top_k == E */
        {9, 192, 32, 8, 128, 0, 1, 0, 0, 0},  /* many experts without a token, no token listed */
    };
    for (size_t i = 0; i < sizeof cases / sizeof cases[0]; i++)
        run_layer(&cases[i], (int)i);

    static const int32_t lens0[4] = {0, 5, 9, -3};
    run_gqa(4, 4, 2, 64, 5, lens0, 10);
    static const int32_t lens1[1] = {1};
    run_gqa(1, 8, 1, 128, 1, lens1, 11);
    static const int32_t lens2[2] = {2, 3};
    run_gqa(2, 16, 2, 256, 3, lens2, 12);

    run_small_functions();

    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver: all cases ran clean\n");
    return 0;
}
