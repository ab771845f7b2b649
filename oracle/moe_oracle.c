/*
 * Oracle for one mixture-of-experts layer of Qwen3.6-35B-A3B with MLX affine
 * 4-bit expert weights, as described on the pages about Lily (Perplexity's
 * inference engine).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is compiled on its own with gcc into
 * liboracle.so and is called by the test-suite, by the smoke check and by the
 * CPU-baseline leg of the benchmark.  The HIP product path never links,
 * loads or calls it, and it shares no code with that path.
 *
 * Plain, slow, obviously correct: every floating-point step runs in double
 * precision, in the order the definition states, with no blocking or fusion.
 *
 * What is computed, and where the pages say it:
 *   - every token scores all 256 routed experts, keeps 8 and adds one shared
 *     expert (aimanavo.com page, section "Qwen3.6's 256 experts and two layer
 *     types make the MLX-Lily gap");
 *   - routing is the MoE's own step, kept on the GPU in Lily (same page,
 *     section "Lily does not treat prefill and decode as the same job";
 *     dzen.guru page, section "Where does the speed-up come from?");
 *   - expert weights are MLX affine 4-bit, group size 64, restored inside the
 *     grouped matrix product (aimanavo.com page, sections on the single 4-bit
 *     checkpoint and on prefill vs decode; news.mantis.guru page, section
 *     "Rust drives the model, Metal does the compute").
 * The pages give no formulas.  Readings taken where they are silent:
 *   R1 scores are a softmax over the E router logits; the k largest logits are
 *      kept and their probabilities renormalised to sum to one;
 *   R2 ranking key: the logit rounded to float32 (the kernel's precision),
 *      larger first, lower expert index first on equal keys; the rank order is
 *      the slot order j = 0..k-1;
 *   R3 an optional per-expert additive logit offset enters before selection
 *      and softmax;
 *   R4 each expert is a SwiGLU feed-forward block: h = silu(W_gate x) * (W_up x),
 *      y = W_down h, silu(z) = z / (1 + exp(-z));
 *   R5 the shared expert's output is added with weight one, no gate;
 *   R6 nibble k of an output row sits at bits [4*(k%8), 4*(k%8)+4) of word k/8;
 *      groups are 64 consecutive input columns of one output row;
 *      dequantised value = scale * code + bias;
 *   R7 combine: out[t] = sum_j w[t][j] * y[t][j] + y_shared[t].
 *   R14 (checkpoint conformity, not on the pages) an optional gate on the
 *      shared expert: a bfloat16 vector g [H] scales the shared expert's
 *      output by sigmoid(sum_h x[t][h] * g[h]); without g the weight is one (R5).
 *      This is the shared-expert gate of Qwen's mixture-of-experts checkpoints.
 *   R17 (decode stack, not on the pages) each layer of a stack of layers reads
 *      the root-mean-square normalisation of the bf16 residual stream,
 *      bf16(x / sqrt(mean(x^2) + eps) * gamma), and adds its output to the
 *      stream: how a pre-norm decoder feeds its mixture-of-experts blocks.
 *   R16 (checkpoint conformity, not on the pages) an optional 8-bit router in
 *      the MLX affine layout: byte k of a row sits at bits [8*(k%4), 8*(k%4)+8)
 *      of word k/4, groups of 64 columns carry a scale and a bias, and the
 *      router weight is the float32 fused multiply-add scale * code + bias
 *      rounded to bfloat16 (nearest, ties to even); the scores then follow R1
 *      with that bfloat16 matrix.  The router is restored to the precision the
 *      dense router has, so both sides take every ranking decision on the
 *      same matrix.
 *   R19 (decode attention, the pages' GQA packing) a full-attention layer's
 *      decode step for one token per sequence: 16 query heads share 2 KV
 *      heads, 8 query heads per KV head (aimanavo.com page, section
 *      "Qwen3.6's 256 experts and two layer types make the MLX-Lily gap"),
 *      consecutive query heads sharing one KV head, h -> h / (Hq / Hkv).
 *      The pages name the packing (each KV row read once for the query heads
 *      that share it) but not the formula: the plain one is taken, scores
 *      s_j = scale * q_h . k_j over the sequence's cached rows, softmax over
 *      them, out_h = sum_j p_j v_j, with the current token's key and value
 *      already in the cache.  A sequence with no rows gives zeros.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

static double bf16_bits_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double sb_value(const void *p, int bf16, size_t i)
{
    if (bf16)
        return bf16_bits_value(((const uint16_t *)p)[i]);
    return (double)((const float *)p)[i];
}

/* The 4-bit code of element (n, k): R6. */
int32_t oracle_code(const oracle_qmat *m, int32_t n, int32_t k)
{
    uint32_t word = m->q[(size_t)n * (size_t)(m->K / 8) + (size_t)(k / 8)];
    return (int32_t)((word >> (4 * (k % 8))) & 15u);
}

/* Dequantise a whole matrix: W[n][k] = s[n][k/group] * code(n,k) + b[n][k/group]. */
void oracle_dequant(const oracle_qmat *m, double *W)
{
    int32_t ng = m->K / m->group;
    for (int32_t n = 0; n < m->N; n++) {
        for (int32_t k = 0; k < m->K; k++) {
            size_t gi = (size_t)n * (size_t)ng + (size_t)(k / m->group);
            double s = sb_value(m->s, m->sb_bf16, gi);
            double b = sb_value(m->b, m->sb_bf16, gi);
            W[(size_t)n * (size_t)m->K + (size_t)k] = s * (double)oracle_code(m, n, k) + b;
        }
    }
}

/* float32 -> bfloat16 bits, nearest with ties to even (finite inputs). */
static uint16_t f32_to_bf16_nearest_even(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    const uint32_t lower = u & 0xFFFFu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1;
    return (uint16_t)upper;
}

/* double -> bfloat16 bits, rounded once to the nearest (ties to even): the
 * value's significand is rounded to 8 bits in double precision, which is
 * exact, and the result is then exactly representable in float32. */
static uint16_t f64_to_bf16_nearest_even(double v)
{
    if (v == 0.0)
        return signbit(v) ? 0x8000u : 0u;
    int e;
    const double m = frexp(v, &e);            /* v = m * 2^e, 0.5 <= |m| < 1 */
    const double r = nearbyint(ldexp(m, 8));  /* 8 significant bits, ties to even */
    const float f = (float)ldexp(r, e - 8);
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* Root-mean-square normalisation of one row of the residual stream, the input
 * of each layer of a decode stack (R17, not on the pages: how a pre-norm
 * decoder feeds its mixture-of-experts block):
 *   out[h] = bf16(x[h] / sqrt(mean_h x[h]^2 + eps) * gamma[h]),
 * gamma[h] = 1 when gamma is NULL; double precision, rounded once to bf16. */
void oracle_rmsnorm(int32_t H, const uint16_t *x, const uint16_t *gamma, double eps, uint16_t *out)
{
    double ss = 0.0;
    for (int32_t h = 0; h < H; h++) {
        const double v = bf16_bits_value(x[h]);
        ss += v * v;
    }
    const double r = 1.0 / sqrt(ss / (double)H + eps);
    for (int32_t h = 0; h < H; h++) {
        const double g = gamma ? bf16_bits_value(gamma[h]) : 1.0;
        out[h] = f64_to_bf16_nearest_even(bf16_bits_value(x[h]) * r * g);
    }
}

/* The 8-bit router restored to bfloat16: out[e][h] = bf16(fmaf(s, q, b)) with
 * q byte h % 4 of word [e][h / 4] and (s, b) of group h / 64: R16. */
void oracle_router_dequant_q8(int32_t E, int32_t H, const uint32_t *codes, const void *scale,
                              const void *bias, int32_t sb_bf16, uint16_t *out)
{
    const int32_t groups = H / 64;
    for (int32_t e = 0; e < E; e++)
        for (int32_t h = 0; h < H; h++) {
            const uint32_t word = codes[(size_t)e * (H / 4) + h / 4];
            const uint32_t q = (word >> (8 * (h % 4))) & 0xFFu;
            const float sv = (float)sb_value(scale, sb_bf16, (size_t)e * groups + h / 64);
            const float bv = (float)sb_value(bias, sb_bf16, (size_t)e * groups + h / 64);
            out[(size_t)e * H + h] = f32_to_bf16_nearest_even(fmaf(sv, (float)q, bv));
        }
}

/* Router logits l[t][e] = sum_h x[t][h] * router[e][h] (+ logit_bias[e]): R1, R3. */
void oracle_router_logits(int32_t T, int32_t H, int32_t E, const uint16_t *x,
                          const uint16_t *router, const float *logit_bias, double *logits)
{
    for (int32_t t = 0; t < T; t++) {
        for (int32_t e = 0; e < E; e++) {
            double acc = 0.0;
            for (int32_t h = 0; h < H; h++)
                acc += bf16_bits_value(x[(size_t)t * H + h]) * bf16_bits_value(router[(size_t)e * H + h]);
            if (logit_bias)
                acc += (double)logit_bias[e];
            logits[(size_t)t * E + e] = acc;
        }
    }
}

/* Top-k selection and renormalised softmax weights for each token: R1, R2. */
void oracle_select(int32_t T, int32_t E, int32_t k, const double *logits, int32_t *idx, double *w)
{
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    for (int32_t t = 0; t < T; t++) {
        const double *l = logits + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        /* k rounds of arg-max on the float32 key; the scan is ascending in e and
           only a strictly larger key replaces the best, so equal keys keep the
           lower index */
        for (int32_t j = 0; j < k; j++) {
            int32_t best = -1;
            float best_key = 0.0f;
            for (int32_t e = 0; e < E; e++) {
                if (taken[e])
                    continue;
                float key = (float)l[e];
                if (best < 0 || key > best_key) {
                    best = e;
                    best_key = key;
                }
            }
            taken[best] = 1;
            idx[(size_t)t * k + j] = best;
        }
        /* softmax over all E logits ... */
        double lmax = l[0];
        for (int32_t e = 1; e < E; e++)
            if (l[e] > lmax)
                lmax = l[e];
        double z = 0.0;
        for (int32_t e = 0; e < E; e++) {
            p[e] = exp(l[e] - lmax);
            z += p[e];
        }
        for (int32_t e = 0; e < E; e++)
            p[e] /= z;
        /* ... then renormalised over the k kept experts */
        double kept = 0.0;
        for (int32_t j = 0; j < k; j++)
            kept += p[idx[(size_t)t * k + j]];
        for (int32_t j = 0; j < k; j++)
            w[(size_t)t * k + j] = p[idx[(size_t)t * k + j]] / kept;
    }
    free(p);
    free(taken);
}

/* Counting sort of the T*k slots (slot = t*k + j) by expert, stable in slot order. */
void oracle_permute(int32_t T, int32_t k, int32_t E, const int32_t *idx,
                    int32_t *counts, int32_t *offsets, int32_t *sorted_slot)
{
    int32_t n = T * k;
    for (int32_t e = 0; e < E; e++)
        counts[e] = 0;
    for (int32_t s = 0; s < n; s++)
        counts[idx[s]]++;
    offsets[0] = 0;
    for (int32_t e = 0; e < E; e++)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int32_t e = 0; e < E; e++)
        cursor[e] = offsets[e];
    for (int32_t s = 0; s < n; s++)
        sorted_slot[cursor[idx[s]]++] = s;
    free(cursor);
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One expert applied to n activation rows (R4).  g, u (nullable) receive the
   pre-activation gate and up projections [n][I]; y receives [n][H]. */
void oracle_expert_ffn(const oracle_qmat *gate, const oracle_qmat *up, const oracle_qmat *down,
                       int32_t n, const uint16_t *const *rows, double *g_out, double *u_out, double *y)
{
    int32_t H = gate->K, I = gate->N;
    double *Wg = (double *)malloc(sizeof(double) * (size_t)I * H);
    double *Wu = (double *)malloc(sizeof(double) * (size_t)I * H);
    double *Wd = (double *)malloc(sizeof(double) * (size_t)H * I);
    double *xv = (double *)malloc(sizeof(double) * (size_t)H);
    double *a = (double *)malloc(sizeof(double) * (size_t)I);
    oracle_dequant(gate, Wg);
    oracle_dequant(up, Wu);
    oracle_dequant(down, Wd);
    for (int32_t r = 0; r < n; r++) {
        for (int32_t h = 0; h < H; h++)
            xv[h] = bf16_bits_value(rows[r][h]);
        for (int32_t i = 0; i < I; i++) {
            double g = 0.0, u = 0.0;
            for (int32_t h = 0; h < H; h++) {
                g += Wg[(size_t)i * H + h] * xv[h];
                u += Wu[(size_t)i * H + h] * xv[h];
            }
            if (g_out)
                g_out[(size_t)r * I + i] = g;
            if (u_out)
                u_out[(size_t)r * I + i] = u;
            a[i] = silu(g) * u;
        }
        for (int32_t o = 0; o < H; o++) {
            double acc = 0.0;
            for (int32_t i = 0; i < I; i++)
                acc += Wd[(size_t)o * I + i] * a[i];
            y[(size_t)r * H + o] = acc;
        }
    }
    free(a);
    free(xv);
    free(Wd);
    free(Wu);
    free(Wg);
}

/* Weight of the shared expert for each of T tokens: s[t] = sigmoid(sum_h x[t][h] * g[h])  (R14). */
void oracle_shared_gate(int32_t T, int32_t H, const uint16_t *x, const uint16_t *g, double *s)
{
    for (int32_t t = 0; t < T; t++) {
        double z = 0.0;
        for (int32_t h = 0; h < H; h++)
            z += bf16_bits_value(x[(size_t)t * H + h]) * bf16_bits_value(g[h]);
        s[t] = 1.0 / (1.0 + exp(-z));
    }
}

/* out[t] = sum_j w[t][j] * y_slot[t][j] + s[t] * y_shared[t]  (R5, R7, R14), j in slot
   order; s[t] = shared_w[t], or 1 when shared_w is NULL. */
void oracle_combine(int32_t n, int32_t k, int32_t H, const double *y_slot, const double *w,
                    const double *y_shared, const double *shared_w, double *out)
{
    for (int32_t t = 0; t < n; t++) {
        for (int32_t h = 0; h < H; h++) {
            double acc = 0.0;
            for (int32_t j = 0; j < k; j++)
                acc += w[(size_t)t * k + j] * y_slot[((size_t)t * k + j) * H + h];
            if (y_shared)
                acc += (shared_w ? shared_w[t] : 1.0) * y_shared[(size_t)t * H + h];
            out[(size_t)t * H + h] = acc;
        }
    }
}

static oracle_qmat expert_mat(const uint32_t *q, const void *s, const void *b, int32_t e,
                              int32_t N, int32_t K, int32_t group, int32_t sb_bf16)
{
    size_t esz = sb_bf16 ? 2 : 4;
    oracle_qmat m;
    m.q = q + (size_t)e * N * (K / 8);
    m.s = (const char *)s + (size_t)e * N * (K / group) * esz;
    m.b = (const char *)b + (size_t)e * N * (K / group) * esz;
    m.sb_bf16 = sb_bf16;
    m.N = N;
    m.K = K;
    m.group = group;
    return m;
}

/*
 * The whole layer.  Routing, counts and offsets cover all T tokens; the
 * expert outputs and the combined output are computed for the n_tok tokens
 * listed in tok (all T, in order, when tok is NULL).  Expert-major: each
 * expert that has a listed token is dequantised once and applied to its
 * listed slots in stable slot order.
 * Outputs: out [n_tok][H]; logits [T][E] (nullable); idx [T][k]; w [T][k];
 * counts [E]; offsets [E+1]; sorted_slot [T*k] (nullable).
 * Returns 0, or -1 if a working buffer could not be allocated (every buffer
 * this call allocated is freed either way).
 */
int oracle_moe_layer(const oracle_layer *L, int32_t n_tok, const int32_t *tok, double *out,
                     double *logits, int32_t *idx, double *w, int32_t *counts, int32_t *offsets,
                     int32_t *sorted_slot)
{
    int32_t T = L->T, H = L->H, E = L->E, k = L->top_k, I = L->I, G = L->group;
    int32_t nt = tok ? n_tok : T;
    double *lg = logits ? logits : (double *)malloc(sizeof(double) * (size_t)T * E);
    int32_t *ss = sorted_slot ? sorted_slot : (int32_t *)malloc(sizeof(int32_t) * (size_t)T * k);
    /* position of each listed token in the output, or -1 */
    int32_t *pos = (int32_t *)malloc(sizeof(int32_t) * (size_t)T);
    double *y_slot = (double *)calloc((size_t)nt * k * H, sizeof(double));
    double *y_sh = L->sh_gate_q ? (double *)calloc((size_t)nt * H, sizeof(double)) : NULL;
    double *w_sub = (double *)malloc(sizeof(double) * (size_t)nt * k + 1);
    const uint16_t **rows = (const uint16_t **)malloc(sizeof(uint16_t *) * ((size_t)nt * k + 1));
    int32_t *rdst = (int32_t *)malloc(sizeof(int32_t) * ((size_t)nt * k + 1));
    double *ybuf = (double *)malloc(sizeof(double) * ((size_t)nt * k + 1) * H);
    double *s_sh = L->sh_expert_gate ? (double *)malloc(sizeof(double) * ((size_t)nt + 1)) : NULL;
    int status = -1;
    if (!lg || !ss || !pos || !y_slot || (L->sh_gate_q && !y_sh) || !w_sub || !rows || !rdst || !ybuf ||
        (L->sh_expert_gate && !s_sh))
        goto done;

    oracle_router_logits(T, H, E, L->x, L->router, L->logit_bias, lg);
    oracle_select(T, E, k, lg, idx, w);
    oracle_permute(T, k, E, idx, counts, offsets, ss);

    for (int32_t t = 0; t < T; t++)
        pos[t] = -1;
    for (int32_t i = 0; i < nt; i++)
        pos[tok ? tok[i] : i] = i;

    for (int32_t e = 0; e < E; e++) {
        int32_t n = 0;
        for (int32_t r = offsets[e]; r < offsets[e + 1]; r++) {
            int32_t slot = ss[r], t = slot / k, j = slot % k;
            if (pos[t] < 0)
                continue;
            rows[n] = L->x + (size_t)t * H;
            rdst[n] = pos[t] * k + j;
            n++;
        }
        if (n == 0)
            continue;
        oracle_qmat mg = expert_mat(L->gate_q, L->gate_s, L->gate_b, e, I, H, G, L->sb_bf16);
        oracle_qmat mu = expert_mat(L->up_q, L->up_s, L->up_b, e, I, H, G, L->sb_bf16);
        oracle_qmat md = expert_mat(L->down_q, L->down_s, L->down_b, e, H, I, G, L->sb_bf16);
        oracle_expert_ffn(&mg, &mu, &md, n, rows, NULL, NULL, ybuf);
        for (int32_t r = 0; r < n; r++)
            memcpy(y_slot + (size_t)rdst[r] * H, ybuf + (size_t)r * H, sizeof(double) * (size_t)H);
    }
    if (L->sh_gate_q) {
        int32_t Is = L->I_shared;
        for (int32_t i = 0; i < nt; i++)
            rows[i] = L->x + (size_t)(tok ? tok[i] : i) * H;
        oracle_qmat mg = expert_mat(L->sh_gate_q, L->sh_gate_s, L->sh_gate_b, 0, Is, H, G, L->sb_bf16);
        oracle_qmat mu = expert_mat(L->sh_up_q, L->sh_up_s, L->sh_up_b, 0, Is, H, G, L->sb_bf16);
        oracle_qmat md = expert_mat(L->sh_down_q, L->sh_down_s, L->sh_down_b, 0, H, Is, G, L->sb_bf16);
        oracle_expert_ffn(&mg, &mu, &md, nt, rows, NULL, NULL, y_sh);
    }
    for (int32_t i = 0; i < nt; i++) {
        int32_t t = tok ? tok[i] : i;
        for (int32_t j = 0; j < k; j++)
            w_sub[(size_t)i * k + j] = w[(size_t)t * k + j];
    }
    if (s_sh)
        for (int32_t i = 0; i < nt; i++)
            oracle_shared_gate(1, H, L->x + (size_t)(tok ? tok[i] : i) * H, L->sh_expert_gate, s_sh + i);
    oracle_combine(nt, k, H, y_slot, w_sub, y_sh, s_sh, out);
    status = 0;

done:
    free(s_sh);
    free(ybuf);
    free(rdst);
    free(rows);
    free(w_sub);
    free(y_sh);
    free(y_slot);
    free(pos);
    if (!sorted_slot)
        free(ss);
    if (!logits)
        free(lg);
    return status;
}

/* Decode attention with grouped-query KV sharing (R19).  q [B][Hq][D],
 * k and v [B][Hkv][S_max][D] (bfloat16 bits), seq_len [B] (values clamped to
 * [0, S_max]); out [B][Hq][D].  For sequence b, query head h and its KV head
 * g = h / (Hq / Hkv):
 *     s_j = scale * sum_d q[b][h][d] * k[b][g][j][d],   j < seq_len[b],
 *     p_j = exp(s_j - max_j s_j) / sum_j exp(s_j - max_j s_j),
 *     out[b][h][d] = sum_j p_j * v[b][g][j][d].
 * Double precision throughout.  Returns 0, or -1 if a buffer could not be
 * allocated. */
int oracle_gqa_decode(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S_max, const uint16_t *q,
                      const uint16_t *k, const uint16_t *v, const int32_t *seq_len, double scale, double *out)
{
    const int32_t per_kv = Hq / Hkv;
    double *p = malloc(sizeof(double) * (size_t)(S_max > 0 ? S_max : 1));
    if (!p)
        return -1;
    for (int32_t b = 0; b < B; b++) {
        int32_t n = seq_len[b];
        if (n < 0)
            n = 0;
        if (n > S_max)
            n = S_max;
        for (int32_t h = 0; h < Hq; h++) {
            const int32_t g = h / per_kv;
            const uint16_t *qh = q + ((size_t)b * Hq + h) * D;
            const uint16_t *kg = k + ((size_t)b * Hkv + g) * S_max * D;
            const uint16_t *vg = v + ((size_t)b * Hkv + g) * S_max * D;
            double *o = out + ((size_t)b * Hq + h) * D;
            if (n == 0) {
                for (int32_t d = 0; d < D; d++)
                    o[d] = 0.0;
                continue;
            }
            double smax = -INFINITY;
            for (int32_t j = 0; j < n; j++) {
                double acc = 0.0;
                for (int32_t d = 0; d < D; d++)
                    acc += bf16_bits_value(qh[d]) * bf16_bits_value(kg[(size_t)j * D + d]);
                p[j] = scale * acc;
                if (p[j] > smax)
                    smax = p[j];
            }
            double z = 0.0;
            for (int32_t j = 0; j < n; j++) {
                p[j] = exp(p[j] - smax);
                z += p[j];
            }
            for (int32_t d = 0; d < D; d++) {
                double acc = 0.0;
                for (int32_t j = 0; j < n; j++)
                    acc += p[j] * bf16_bits_value(vg[(size_t)j * D + d]);
                o[d] = acc / z;
            }
        }
    }
    free(p);
    return 0;
}
