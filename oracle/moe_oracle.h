/*
 * Declarations of the oracle in moe_oracle.c (what each function computes and
 * which page passage it follows is stated there, beside its definition).
 *
 * TEST INFRASTRUCTURE ONLY: included by moe_oracle.c and by the test-suite's
 * sanitizer driver; the HIP product path never includes it.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

typedef struct {
    const uint32_t *q; /* [N][K/8] packed 4-bit codes */
    const void *s;     /* [N][K/group] scales: float32, or bfloat16 bits */
    const void *b;     /* [N][K/group] biases, same type as s */
    int32_t sb_bf16;   /* 1: s and b hold bfloat16 bit patterns */
    int32_t N, K, group;
} oracle_qmat;

typedef struct {
    int32_t T, H, E, top_k, I, I_shared, group, sb_bf16;
    const uint16_t *x;          /* [T][H] bfloat16 bits */
    const uint16_t *router;     /* [E][H] bfloat16 bits */
    const float *logit_bias;    /* [E] or NULL */
    /* routed experts, stacked: gate/up q [E][I][H/8], s/b [E][I][H/group];
       down q [E][H][I/8], s/b [E][H][I/group] */
    const uint32_t *gate_q, *up_q, *down_q;
    const void *gate_s, *gate_b, *up_s, *up_b, *down_s, *down_b;
    /* shared expert (single); gate_q == NULL means no shared expert */
    const uint32_t *sh_gate_q, *sh_up_q, *sh_down_q;
    const void *sh_gate_s, *sh_gate_b, *sh_up_s, *sh_up_b, *sh_down_s, *sh_down_b;
    const uint16_t *sh_expert_gate; /* [H] bfloat16 bits, or NULL: shared weight 1 (R14) */
} oracle_layer;

int32_t oracle_code(const oracle_qmat *m, int32_t n, int32_t k);
void oracle_dequant(const oracle_qmat *m, double *W);
void oracle_rmsnorm(int32_t H, const uint16_t *x, const uint16_t *gamma, double eps, uint16_t *out);
void oracle_router_dequant_q8(int32_t E, int32_t H, const uint32_t *codes, const void *scale,
                              const void *bias, int32_t sb_bf16, uint16_t *out);
void oracle_router_logits(int32_t T, int32_t H, int32_t E, const uint16_t *x,
                          const uint16_t *router, const float *logit_bias, double *logits);
void oracle_select(int32_t T, int32_t E, int32_t k, const double *logits, int32_t *idx, double *w);
void oracle_permute(int32_t T, int32_t k, int32_t E, const int32_t *idx,
                    int32_t *counts, int32_t *offsets, int32_t *sorted_slot);
void oracle_expert_ffn(const oracle_qmat *gate, const oracle_qmat *up, const oracle_qmat *down,
                       int32_t n, const uint16_t *const *rows, double *g_out, double *u_out, double *y);
void oracle_shared_gate(int32_t T, int32_t H, const uint16_t *x, const uint16_t *g, double *s);
void oracle_combine(int32_t n, int32_t k, int32_t H, const double *y_slot, const double *w,
                    const double *y_shared, const double *shared_w, double *out);
int oracle_moe_layer(const oracle_layer *L, int32_t n_tok, const int32_t *tok, double *out,
                     double *logits, int32_t *idx, double *w, int32_t *counts, int32_t *offsets,
                     int32_t *sorted_slot);
int oracle_gqa_decode(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S_max, const uint16_t *q,
                      const uint16_t *k, const uint16_t *v, const int32_t *seq_len, double scale, double *out);

#endif
