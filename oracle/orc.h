/*
 * Oracle for the Qwen3 decoder-block forward pass: a plain, slow, strict-f32
 * CPU evaluation of the method, token by token.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this code; only the tests, the smoke check and the benchmark's
 * cpu_baseline leg use it.
 *
 * Numerical policy ("Scalar-Native Qwen3 Reference Runtime As The Numerical
 * Authority", section 4 "Floating-Point and Determinism Policy"): every
 * activation, accumulation and nonlinearity is f32; sums are `acc = acc + a*b`
 * in index order; no FMA contraction (built with -ffp-contract=off), no fast
 * math, gradual underflow.  exp, cos and sin are evaluated in double and
 * rounded once to f32 so the result does not depend on the host libm's float
 * routines ("Portable WebAssembly Runtime Architecture for TinyRustLM",
 * "Floating-point reference policy", recommendation against platform libm).
 *
 * Rows of a matrix-vector product may be spread over threads; each output
 * element is summed by one thread in index order, so results are bit-identical
 * for any thread count (same page, "Partitioning decision").
 */
#ifndef QW3_ORACLE_H
#define QW3_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_OK = 0, ORC_INVALID_ARGUMENT = 1, ORC_UNSUPPORTED_QUANT = 12, ORC_UNSUPPORTED_SHAPE = 13,
       ORC_CONTEXT_EXCEEDED = 14, ORC_NUMERICAL_FAILURE = 18 };
enum { ORC_FMT_BF16 = 1, ORC_FMT_Q8 = 2, ORC_FMT_Q8_0 = 3, ORC_FMT_Q8_ACT8 = 4 };

typedef struct {
    int32_t fmt;        /* ORC_FMT_BF16, ORC_FMT_Q8, ORC_FMT_Q8_0, or ORC_FMT_Q8_ACT8 (Q8 weights, int8 activations) */
    int32_t input_mode; /* 0: token ids, 1: fp32 hidden vectors (no embedding / final norm / logits) */
    int32_t vocab, hidden, n_layers, n_q_heads, n_kv_heads, head_dim, inter, max_ctx, n_seq;
    int32_t kv_f32;     /* 0: cache holds bf16-rounded K/V (default); 1: cache keeps f32 K/V */
    float eps;
    double theta;
} orc_cfg_t;

/* Canonical [rows, cols] row-major matrix: bf16 bits, or Q8 codes + f32 scale per 32 along cols, or
 * Q8_0 blocks: per row cols/32 blocks of 34 bytes (little-endian f16 scale, then 32 int8 codes). */
typedef struct {
    int32_t rows, cols;
    const uint16_t *bf16;
    const int8_t *codes;
    const float *scales;
    const uint8_t *q8_0;
} orc_mat_t;

/* Norm weights are bf16 bits when fmt == BF16 and f32 when fmt == Q8 or Q8_0. */
typedef struct {
    const void *attn_norm, *q_norm, *k_norm, *mlp_norm;
    orc_mat_t q, k, v, o, gate, up, down;
} orc_layer_t;

typedef struct orc_model orc_model_t;

/* ---- building blocks (each exported so tests can pin it alone) ---- */
float orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16(float f);
float orc_exp(float x);
void orc_rmsnorm(const float *x, const float *w, int32_t n, float eps, float *out);
void orc_rope_table(double theta, int32_t head_dim, int32_t pos, float *cos_out, float *sin_out);
void orc_rope_apply(float *v, int32_t head_dim, const float *cos_t, const float *sin_t);
int32_t orc_softmax(const float *s, int32_t n, float *p);
int32_t orc_attention_head(const float *q, const float *k_rows, const float *v_rows, int32_t n, int32_t head_dim,
                           float *out);
int32_t orc_gqa_attention(const float *q, int32_t n_q, int32_t n_kv, const float *k_heads, const float *v_heads,
                          size_t head_stride, int32_t n, int32_t head_dim, float *out);
float orc_silu(float z);
float orc_q8_dot(const int8_t *codes, const float *scales, const float *act, int32_t n);
float orc_bf16_dot(const uint16_t *w, const float *act, int32_t n);
void orc_dequant_row(const orc_mat_t *m, int32_t row, float *out);
void orc_matvec(const orc_mat_t *m, const float *x, float *out);
int32_t orc_argmax(const float *v, int32_t n, int32_t *idx);
float orc_f16_to_f32(uint16_t h);
float orc_q8_0_dot(const uint8_t *blocks, const float *act, int32_t n);
void orc_quantize_act8(const float *x, int32_t n, int8_t *q, float *d);
float orc_q8q8_dot(const int8_t *wq, const float *ws, const int8_t *aq, const float *ad, int32_t n);

/* Deterministic sampling ([P1] section 7; [P4] "Deterministic sampling contract", "Sampling order"). */
typedef struct {
    uint64_t state, inc; /* PCG32 state and (odd) increment */
} orc_pcg32_t;
void orc_pcg32_seed(uint64_t seed, uint64_t stream_id, orc_pcg32_t *r);
uint32_t orc_pcg32_next(orc_pcg32_t *r);
float orc_pcg32_uniform(uint32_t word);
typedef struct {
    float temperature;        /* 0: greedy (no draw); else positive and finite */
    float top_p;              /* (0, 1] */
    float repetition_penalty; /* positive and finite; 1 leaves the logits unchanged */
    int32_t top_k;            /* >= 1 */
} orc_sample_params_t;
int32_t orc_sample_prepare(const float *logits, int32_t vocab, float penalty, const int32_t *history,
                           int32_t n_history, const int32_t *forbid, int32_t n_forbid, float *z, unsigned char *seen);
int32_t orc_sample(const float *logits, int32_t vocab, const orc_sample_params_t *p, const int32_t *history,
                   int32_t n_history, const int32_t *forbid, int32_t n_forbid, orc_pcg32_t *rng, int32_t *token,
                   float *probs_out, int32_t *ids_out, int32_t *n_out);
void orc_set_threads(int32_t n);
int32_t orc_get_threads(void);

/* ---- whole model ---- */
orc_model_t *orc_create(const orc_cfg_t *cfg, const orc_mat_t *embed, const void *final_norm,
                        const orc_layer_t *layers);
void orc_destroy(orc_model_t *m);
/* One token at position len[seq]: tok (token ids) or hidden_in (hidden mode). Writes hidden_out
 * and/or logits (vocab f32) and argmax when non-NULL.  KV length advances only on success. */
int32_t orc_step(orc_model_t *m, int32_t seq, int32_t tok, const float *hidden_in, float *hidden_out,
                 float *logits, int32_t *argmax);
int32_t orc_step_kv(orc_model_t *m, int32_t seq, int32_t tok, const float *hidden_in, float *hidden_out,
                    float *logits, int32_t *argmax, const uint16_t *kv_force, uint16_t *kv_own);
int32_t orc_kv_write(orc_model_t *m, int32_t seq, int32_t layer, int32_t pos0, int32_t n_pos, const uint16_t *k,
                     const uint16_t *v);
int32_t orc_kv_read(const orc_model_t *m, int32_t seq, int32_t layer, int32_t pos0, int32_t n_pos, uint16_t *k,
                    uint16_t *v);
int32_t orc_set_len(orc_model_t *m, int32_t seq, int32_t len);
int32_t orc_get_len(const orc_model_t *m, int32_t seq);

#ifdef __cplusplus
}
#endif
#endif
