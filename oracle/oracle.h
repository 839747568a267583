/*
 * Oracle for the per-token decode step of a Llama-style decoder — TEST
 * INFRASTRUCTURE ONLY. Only tests, the smoke check and the benchmark's CPU
 * baseline may load it. The HIP path never links, includes or calls it.
 *
 * Plain, slow and obviously correct. Every activation is a double in the default
 * build (liboracle.so), the parity reference. A second build with -DORC_FP32
 * (liboracle_f32.so) computes the same definition in fp32 throughout; it measures
 * how far fp32 rounding alone moves the results. The interface is double in both.
 * Weights and the KV cache are bf16 bit patterns (uint16_t), read exactly.
 * Loops run in a fixed order, so results do not depend on the thread count
 * (OpenMP splits only independent rows and heads).
 *
 * What is computed: an autoregressive decoder step with a KV cache. Prefill
 * fills the cache and decode makes one token at a time. The cached keys and
 * values of earlier positions are reused ("Compiling LLMs into a MegaKernel";
 * "LLM inference engine from scratch in C++/CUDA", section 1.1). The layer
 * math is the standard Llama-family block: RMSNorm, QKV projection (+ bias),
 * rotate-half RoPE, grouped-query attention, output projection, RMSNorm,
 * SwiGLU FFN, final RMSNorm, LM head and argmax. The slide deck's GQA slide
 * says several query heads share one K/V pair. The pages print no formula for
 * the norm, rotary embedding or FFN; the readings used are listed in the
 * design notes.
 */
#ifndef MK_ORACLE_H
#define MK_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int n_layers, d, hq, hk, dh, f, v;
  double eps, theta;
  int tied, qkv_bias;
} orc_config;

/* Tensor pointer table, in this order:
 *   [0] embed [v, d]   [1] final_norm [d]   [2] lm_head [v, d] (NULL when tied)
 *   then per layer l, 12 entries at 3 + 12*l:
 *   attn_norm [d], wq [hq*dh, d], wk [hk*dh, d], wv [hk*dh, d], bq [hq*dh], bk [hk*dh], bv [hk*dh]
 *   (the three biases NULL without qkv bias), wo [d, hq*dh], ffn_norm [d], wg [f, d], wu [f, d], wd [d, f].
 * Matrices are row-major [out, in]. */
#define ORC_T_EMBED 0
#define ORC_T_FINAL_NORM 1
#define ORC_T_LM_HEAD 2
#define ORC_T_LAYER0 3
#define ORC_T_PER_LAYER 12

typedef struct orc_model orc_model;

/* Allocates bf16 K and V caches [n_layers][n_seqs][max_pos][hk][dh], zero-filled.
 * `tensors` must stay valid for the model's lifetime. NULL on bad arguments. */
orc_model* orc_create(const orc_config* cfg, const uint16_t* const* tensors, int n_seqs, int max_pos);
void orc_destroy(orc_model* m);
/* Write cache rows [pos0, pos0+npos) of one layer and sequence from [npos][hk][dh] bf16. */
int orc_set_kv(orc_model* m, int layer, int seq, int pos0, int npos, const uint16_t* k, const uint16_t* v);
int orc_get_kv(const orc_model* m, int layer, int seq, int pos0, int npos, uint16_t* k, uint16_t* v);
/* One decode step of sequence `seq`: input `token` stored at cache position `pos`, attending to
 * positions 0..pos, rotary angle taken at `rope_pos` (normally == pos). Writes v logits, returns argmax,
 * or -1 on bad arguments. */
int orc_step(orc_model* m, int seq, int token, int pos, double rope_pos, double* logits);
/* The same model evaluated without a cache: all n tokens at positions 0..n-1 (rotary angle rope_off + t),
 * layer by layer, causal attention; keys and values rounded to bf16 as the cache stores them.
 * Writes the logits of the last position, returns their argmax. */
int orc_forward_nocache(const orc_model* m, const int* tokens, int n, double rope_off, double* logits_last);

/* Pieces of the step, exposed for the pins. */
void orc_rmsnorm(const double* x, const uint16_t* g, int d, double eps, double* out);
void orc_gemv(const uint16_t* w, int n, int k, const double* x, const uint16_t* bias, double* y);
void orc_rope(double* u, int dh, double pos, double theta);
void orc_softmax(double* s, int n);
void orc_attention(const double* q, const uint16_t* kc, const uint16_t* vc, int npos, int hq, int hk, int dh,
                   double* out);
double orc_silu(double z);
void orc_swiglu(const double* a, const double* b, int n, double* h);
int orc_argmax(const double* v, int n);
uint16_t orc_bf16(double x);
double orc_from_bf16(uint16_t b);
int orc_threads(void);
void orc_set_threads(int n);

/* FP8 weights: OCP E4M3 codes with one power-of-two scale per output row (see oracle.c). */
double orc_fp8_decode(uint8_t c);
uint8_t orc_fp8_encode(double x);
int orc_fp8_row_exp(const uint16_t* w, int k);
void orc_fp8_quantize(const uint16_t* w, int n, int k, uint8_t* codes, int32_t* exps);
void orc_fp8_dequantize(const uint8_t* codes, const int32_t* exps, int n, int k, uint16_t* w_out);

#ifdef __cplusplus
}
#endif
#endif
