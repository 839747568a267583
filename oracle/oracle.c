/*
 * Oracle for the decode step — TEST INFRASTRUCTURE ONLY (see oracle.h).
 * Only tests, the smoke check and the benchmark's CPU baseline may load it.
 *
 * Plain fp64 CPU definition of one decode step. Each function names the passage
 * or reading it follows. Source pages:
 *   [MK]  "LLMs in einen MegaKernel kompilieren, um Low-Latency-Inferenz zu
 *         ermöglichen" (GeekNews summary of "Compiling LLMs into a MegaKernel")
 *   [SL]  "LLM高速化勉強会資料" (slide deck on LLM inference speed-ups)
 *   [KN]  "Hạt nhân là gì và tại sao mọi người lại viết hạt nhân mới"
 *   [IE]  "Crear desde cero un motor de inferencia para LLM usando C++ y CUDA"
 * The layer formulas (RMSNorm, rotate-half RoPE, SwiGLU, argmax with lowest
 * index on ties) are not printed on the pages. They are the standard
 * Llama-family definitions, taken as the plainest reading of the decoder the
 * pages describe.
 */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* Arithmetic type of every activation and accumulation. The default build is fp64, the
 * reference for parity. Built with -DORC_FP32 it is fp32 throughout: the same definition in
 * the precision a GPU computes in. It measures how much fp32 rounding alone moves the results.
 * Rotary angles are formed in double in both builds, then rounded to `real`. */
#ifdef ORC_FP32
typedef float real;
#define R_SQRT sqrtf
#define R_EXP expf
#else
typedef double real;
#define R_SQRT sqrt
#define R_EXP exp
#endif

struct orc_model {
  orc_config c;
  const uint16_t** t;
  int n_seqs, max_pos;
  uint16_t* kc; /* [L][n_seqs][max_pos][hk][dh] */
  uint16_t* vc;
};

/* bf16 -> double is exact: the bf16 bits are the top half of an fp32. */
double orc_from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Cache storage format: the activation rounded to fp32 and then to bf16, both round-to-nearest-even. */
uint16_t orc_bf16(double x) {
  float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

int orc_threads(void) { return omp_get_max_threads(); }
void orc_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}

static real bf(uint16_t b) { return (real)orc_from_bf16(b); }

/* RMSNorm: out_i = x_i / sqrt(mean_j x_j^2 + eps) * g_i. */
static void rmsnorm_r(const real* x, const uint16_t* g, int d, real eps, real* out) {
  real ss = 0;
  for (int i = 0; i < d; ++i) ss += x[i] * x[i];
  const real r = (real)1 / R_SQRT(ss / (real)d + eps);
  for (int i = 0; i < d; ++i) out[i] = x[i] * r * bf(g[i]);
}

/* y = W x (+ b), W row-major [n, k]: y_r = sum_c W[r][c] * x[c], summed in column order.
 * The matrix-vector product that dominates decode ([IE] sections 1.2 and 3.2). */
static void gemv_r(const uint16_t* w, int n, int k, const real* x, const uint16_t* bias, real* y) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < n; ++r) {
    const uint16_t* row = w + (size_t)r * k;
    real s = 0;
    for (int c = 0; c < k; ++c) s += bf(row[c]) * x[c];
    y[r] = bias ? s + bf(bias[r]) : s;
  }
}

/* Rotary position embedding, rotate-half pairing: for i < dh/2, angle a = pos * theta^(-2i/dh),
 * (u_i, u_{i+dh/2}) -> (u_i cos a - u_{i+dh/2} sin a, u_{i+dh/2} cos a + u_i sin a). */
static void rope_r(real* u, int dh, double pos, double theta) {
  const int h = dh / 2;
  for (int i = 0; i < h; ++i) {
    const double a = pos * pow(theta, -2.0 * i / dh);
    const real c = (real)cos(a), s = (real)sin(a);
    const real x0 = u[i], x1 = u[i + h];
    u[i] = x0 * c - x1 * s;
    u[i + h] = x1 * c + x0 * s;
  }
}

/* softmax: subtract the max, exponentiate, divide by the sum. */
static void softmax_r(real* s, int n) {
  real m = -INFINITY;
  for (int j = 0; j < n; ++j) m = s[j] > m ? s[j] : m;
  real z = 0;
  for (int j = 0; j < n; ++j) {
    s[j] = R_EXP(s[j] - m);
    z += s[j];
  }
  for (int j = 0; j < n; ++j) s[j] /= z;
}

/* Grouped-query attention for one query position over npos cached positions ([SL] slide 28:
 * several query heads share one K/V pair; query head h reads KV head h / (hq/hk)).
 * kc, vc: [npos][hk][dh] bf16. Scores q.k / sqrt(dh), softmax over positions, weighted sum of V:
 * the plain (materialised-score) attention of [KN], one query row at a time. */
static void attention_r(const real* q, const uint16_t* kc, const uint16_t* vc, int npos, int hq, int hk, int dh,
                        real* out) {
  const int grp = hq / hk;
  const real scale = (real)1 / R_SQRT((real)dh);
#pragma omp parallel for schedule(static)
  for (int h = 0; h < hq; ++h) {
    const int kh = h / grp;
    real* s = (real*)malloc(sizeof(real) * (size_t)(npos > 0 ? npos : 1));
    for (int j = 0; j < npos; ++j) {
      const uint16_t* kr = kc + ((size_t)j * hk + kh) * dh;
      real a = 0;
      for (int i = 0; i < dh; ++i) a += q[(size_t)h * dh + i] * bf(kr[i]);
      s[j] = a * scale;
    }
    softmax_r(s, npos);
    for (int i = 0; i < dh; ++i) out[(size_t)h * dh + i] = 0;
    for (int j = 0; j < npos; ++j) {
      const uint16_t* vr = vc + ((size_t)j * hk + kh) * dh;
      for (int i = 0; i < dh; ++i) out[(size_t)h * dh + i] += s[j] * bf(vr[i]);
    }
    free(s);
  }
}

/* SiLU(z) = z / (1 + e^-z). */
static real silu_r(real z) { return z / ((real)1 + R_EXP(-z)); }

/* SwiGLU combination of the gate (a) and up (b) projections: h = silu(a) * b. */
static void swiglu_r(const real* a, const real* b, int n, real* h) {
  for (int i = 0; i < n; ++i) h[i] = silu_r(a[i]) * b[i];
}

/* argmax with the lowest index on ties (greedy decoding). */
static int argmax_r(const real* v, int n) {
  int best = 0;
  for (int i = 1; i < n; ++i)
    if (v[i] > v[best]) best = i;
  return best;
}

/* ---- the pieces with a double interface (for the pins); they compute in `real` */
static real* to_real(const double* x, int n) {
  real* r = (real*)malloc(sizeof(real) * (size_t)(n > 0 ? n : 1));
  for (int i = 0; i < n; ++i) r[i] = (real)x[i];
  return r;
}
static void from_real(const real* r, int n, double* x) {
  for (int i = 0; i < n; ++i) x[i] = (double)r[i];
}
void orc_rmsnorm(const double* x, const uint16_t* g, int d, double eps, double* out) {
  real* xr = to_real(x, d);
  real* o = (real*)malloc(sizeof(real) * (size_t)(d > 0 ? d : 1));
  rmsnorm_r(xr, g, d, (real)eps, o);
  from_real(o, d, out);
  free(xr); free(o);
}
void orc_gemv(const uint16_t* w, int n, int k, const double* x, const uint16_t* bias, double* y) {
  real* xr = to_real(x, k);
  real* yr = (real*)malloc(sizeof(real) * (size_t)(n > 0 ? n : 1));
  gemv_r(w, n, k, xr, bias, yr);
  from_real(yr, n, y);
  free(xr); free(yr);
}
void orc_rope(double* u, int dh, double pos, double theta) {
  real* r = to_real(u, dh);
  rope_r(r, dh, pos, theta);
  from_real(r, dh, u);
  free(r);
}
void orc_softmax(double* s, int n) {
  real* r = to_real(s, n);
  softmax_r(r, n);
  from_real(r, n, s);
  free(r);
}
void orc_attention(const double* q, const uint16_t* kc, const uint16_t* vc, int npos, int hq, int hk, int dh,
                   double* out) {
  real* qr = to_real(q, hq * dh);
  real* o = (real*)malloc(sizeof(real) * (size_t)(hq * dh > 0 ? hq * dh : 1));
  attention_r(qr, kc, vc, npos, hq, hk, dh, o);
  from_real(o, hq * dh, out);
  free(qr); free(o);
}
double orc_silu(double z) { return (double)silu_r((real)z); }
void orc_swiglu(const double* a, const double* b, int n, double* h) {
  for (int i = 0; i < n; ++i) h[i] = (double)silu_r((real)a[i]) * (real)b[i];
}
int orc_argmax(const double* v, int n) {
  int best = 0;
  for (int i = 1; i < n; ++i)
    if (v[i] > v[best]) best = i;
  return best;
}

/* ------------------------------------------------------------------ FP8 weights
 * Weight-only quantisation ("LLM高速化勉強会資料", slides 33 and 34: fewer bits per parameter cut the
 * bytes a step moves; block-wise scaling keeps the precision, and products accumulate in a wider
 * format). Format: OCP 8-bit floating point E4M3 ("E4M3FN"): a sign bit, 4 exponent bits with bias 7
 * and 3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9; S.1111.111 is NaN; there is no
 * infinity, and the largest finite value is 448 (0x7E). Each output row of a weight matrix is one block
 * with a power-of-two scale 2^e, so the dequantised weight decode(code) * 2^e is exact. */

/* The value of an E4M3 code, from the format's definition. */
double orc_fp8_decode(uint8_t c) {
  const int sign = c >> 7, ef = (c >> 3) & 15, mf = c & 7;
  double v;
  if (ef == 15 && mf == 7) return NAN;
  if (ef == 0) v = ldexp((double)mf, -9);
  else v = ldexp(1.0 + mf / 8.0, ef - 7);
  return sign ? -v : v;
}

/* The finite E4M3 code nearest to x (|x| <= 448), ties to the code with an even mantissa. The
 * non-negative finite codes 0x00..0x7E decode to increasing values, so the candidates are the largest
 * code not above |x| and the next one. */
uint8_t orc_fp8_encode(double x) {
  const double a = fabs(x);
  int lo = 0, hi = 0x7E;  /* invariant: decode(lo) <= a; find the largest such code */
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (orc_fp8_decode((uint8_t)mid) <= a) lo = mid;
    else hi = mid - 1;
  }
  int c = lo;
  if (lo < 0x7E) {
    const double dl = a - orc_fp8_decode((uint8_t)lo), du = orc_fp8_decode((uint8_t)(lo + 1)) - a;
    if (du < dl || (du == dl && ((lo + 1) & 1) == 0)) c = lo + 1;
  }
  return (uint8_t)(c | (signbit(x) ? 0x80 : 0));
}

/* The row's scale exponent: the smallest integer e with max_k |w_k| <= 448 * 2^e, clamped to
 * [-100, 100]; 0 for an all-zero row. */
int orc_fp8_row_exp(const uint16_t* w, int k) {
  double m = 0.0;
  for (int j = 0; j < k; ++j) m = fmax(m, fabs(orc_from_bf16(w[j])));
  if (m == 0.0) return 0;
  int e = -100;
  while (e < 100 && m > ldexp(448.0, e)) ++e;
  return e;
}

/* codes[i][j] = encode(w[i][j] * 2^-e_i), exps[i] = e_i, for n rows of k bf16 weights. */
void orc_fp8_quantize(const uint16_t* w, int n, int k, uint8_t* codes, int32_t* exps) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; ++i) {
    const uint16_t* row = w + (size_t)i * k;
    const int e = orc_fp8_row_exp(row, k);
    exps[i] = e;
    for (int j = 0; j < k; ++j) codes[(size_t)i * k + j] = orc_fp8_encode(ldexp(orc_from_bf16(row[j]), -e));
  }
}

/* The bf16 bits of decode(codes[i][j]) * 2^exps[i]: exact, since an E4M3 value has at most 4
 * significant bits and the scaled value stays inside bf16's range. */
void orc_fp8_dequantize(const uint8_t* codes, const int32_t* exps, int n, int k, uint16_t* w_out) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < k; ++j)
      w_out[(size_t)i * k + j] = orc_bf16(ldexp(orc_fp8_decode(codes[(size_t)i * k + j]), exps[i]));
}

/* ------------------------------------------------------------------ model */
#define T_EMBED(m) ((m)->t[ORC_T_EMBED])
#define T_FNORM(m) ((m)->t[ORC_T_FINAL_NORM])
#define T_LAYER(m, l, j) ((m)->t[ORC_T_LAYER0 + ORC_T_PER_LAYER * (l) + (j)])
enum { L_ANORM, L_WQ, L_WK, L_WV, L_BQ, L_BK, L_BV, L_WO, L_FNORM, L_WG, L_WU, L_WD };

static const uint16_t* lm_weight(const orc_model* m) {
  return m->c.tied ? m->t[ORC_T_EMBED] : m->t[ORC_T_LM_HEAD];   /* tied head reuses the embedding */
}

orc_model* orc_create(const orc_config* cfg, const uint16_t* const* tensors, int n_seqs, int max_pos) {
  if (!cfg || !tensors || n_seqs <= 0 || max_pos <= 0) return NULL;
  const orc_config* c = cfg;
  if (c->n_layers <= 0 || c->d <= 0 || c->hq <= 0 || c->hk <= 0 || c->hq % c->hk || c->dh <= 0 || c->dh % 2 ||
      c->f <= 0 || c->v <= 0)
    return NULL;
  const int nt = ORC_T_LAYER0 + ORC_T_PER_LAYER * c->n_layers;
  for (int i = 0; i < nt; ++i) {
    int optional = (i == ORC_T_LM_HEAD && c->tied);
    if (i >= ORC_T_LAYER0) {
      int j = (i - ORC_T_LAYER0) % ORC_T_PER_LAYER;
      if ((j == L_BQ || j == L_BK || j == L_BV) && !c->qkv_bias) optional = 1;
    }
    if (!tensors[i] && !optional) return NULL;
  }
  orc_model* m = (orc_model*)calloc(1, sizeof(orc_model));
  m->c = *c;
  m->t = (const uint16_t**)malloc(sizeof(uint16_t*) * nt);
  memcpy(m->t, tensors, sizeof(uint16_t*) * nt);
  m->n_seqs = n_seqs;
  m->max_pos = max_pos;
  const size_t n = (size_t)c->n_layers * n_seqs * max_pos * c->hk * c->dh;
  m->kc = (uint16_t*)calloc(n, 2);
  m->vc = (uint16_t*)calloc(n, 2);
  if (!m->kc || !m->vc) {
    orc_destroy(m);
    return NULL;
  }
  return m;
}

void orc_destroy(orc_model* m) {
  if (!m) return;
  free(m->kc);
  free(m->vc);
  free(m->t);
  free(m);
}

static size_t kv_index(const orc_model* m, int layer, int seq, int pos) {
  return (((size_t)layer * m->n_seqs + seq) * m->max_pos + pos) * m->c.hk * m->c.dh;
}

int orc_set_kv(orc_model* m, int layer, int seq, int pos0, int npos, const uint16_t* k, const uint16_t* v) {
  if (!m || layer < 0 || layer >= m->c.n_layers || seq < 0 || seq >= m->n_seqs || pos0 < 0 || npos < 0 ||
      pos0 + npos > m->max_pos)
    return -1;
  const size_t n = (size_t)npos * m->c.hk * m->c.dh;
  memcpy(m->kc + kv_index(m, layer, seq, pos0), k, n * 2);
  memcpy(m->vc + kv_index(m, layer, seq, pos0), v, n * 2);
  return 0;
}

int orc_get_kv(const orc_model* m, int layer, int seq, int pos0, int npos, uint16_t* k, uint16_t* v) {
  if (!m || layer < 0 || layer >= m->c.n_layers || seq < 0 || seq >= m->n_seqs || pos0 < 0 || npos < 0 ||
      pos0 + npos > m->max_pos)
    return -1;
  const size_t n = (size_t)npos * m->c.hk * m->c.dh;
  memcpy(k, m->kc + kv_index(m, layer, seq, pos0), n * 2);
  memcpy(v, m->vc + kv_index(m, layer, seq, pos0), n * 2);
  return 0;
}

/* Final RMSNorm, LM head and greedy argmax. */
static int lm_head(const orc_model* m, const real* x, double* logits) {
  const orc_config* c = &m->c;
  real* xn = (real*)malloc(sizeof(real) * c->d);
  real* lg = (real*)malloc(sizeof(real) * c->v);
  rmsnorm_r(x, T_FNORM(m), c->d, (real)c->eps, xn);
  gemv_r(lm_weight(m), c->v, c->d, xn, NULL, lg);
  from_real(lg, c->v, logits);
  const int tok = argmax_r(lg, c->v);
  free(xn); free(lg);
  return tok;
}

/* SwiGLU feed-forward with residual: x += Wd (silu(Wg xn) * (Wu xn)), xn = RMSNorm(x, g_ffn). */
static void ffn_block(const orc_model* m, int l, real* x) {
  const orc_config* c = &m->c;
  real* xn = (real*)malloc(sizeof(real) * c->d);
  real* a = (real*)malloc(sizeof(real) * c->f);
  real* b = (real*)malloc(sizeof(real) * c->f);
  real* h = (real*)malloc(sizeof(real) * c->f);
  real* y = (real*)malloc(sizeof(real) * c->d);
  rmsnorm_r(x, T_LAYER(m, l, L_FNORM), c->d, (real)c->eps, xn);
  gemv_r(T_LAYER(m, l, L_WG), c->f, c->d, xn, NULL, a);
  gemv_r(T_LAYER(m, l, L_WU), c->f, c->d, xn, NULL, b);
  swiglu_r(a, b, c->f, h);
  gemv_r(T_LAYER(m, l, L_WD), c->d, c->f, h, NULL, y);
  for (int i = 0; i < c->d; ++i) x[i] += y[i];
  free(xn); free(a); free(b); free(h); free(y);
}

/* QKV projection of the normed input, plus rotary embedding of every q and k head. */
static void qkv_rope(const orc_model* m, int l, const real* x, double rope_pos, real* q, real* k, real* v) {
  const orc_config* c = &m->c;
  real* xn = (real*)malloc(sizeof(real) * c->d);
  rmsnorm_r(x, T_LAYER(m, l, L_ANORM), c->d, (real)c->eps, xn);
  gemv_r(T_LAYER(m, l, L_WQ), c->hq * c->dh, c->d, xn, T_LAYER(m, l, L_BQ), q);
  gemv_r(T_LAYER(m, l, L_WK), c->hk * c->dh, c->d, xn, T_LAYER(m, l, L_BK), k);
  gemv_r(T_LAYER(m, l, L_WV), c->hk * c->dh, c->d, xn, T_LAYER(m, l, L_BV), v);
  for (int h = 0; h < c->hq; ++h) rope_r(q + (size_t)h * c->dh, c->dh, rope_pos, c->theta);
  for (int h = 0; h < c->hk; ++h) rope_r(k + (size_t)h * c->dh, c->dh, rope_pos, c->theta);
  free(xn);
}

/* One decode step with the KV cache ([IE] section 1.1: decode produces one token at a time and
 * the cache keeps earlier keys and values; [SL] slide 9). */
int orc_step(orc_model* m, int seq, int token, int pos, double rope_pos, double* logits) {
  if (!m) return -1;
  const orc_config* c = &m->c;
  if (!logits || seq < 0 || seq >= m->n_seqs || token < 0 || token >= c->v || pos < 0 || pos >= m->max_pos)
    return -1;
  const int qd = c->hq * c->dh, kd = c->hk * c->dh;
  real* x = (real*)malloc(sizeof(real) * c->d);
  real* q = (real*)malloc(sizeof(real) * qd);
  real* k = (real*)malloc(sizeof(real) * kd);
  real* v = (real*)malloc(sizeof(real) * kd);
  real* o = (real*)malloc(sizeof(real) * qd);
  real* y = (real*)malloc(sizeof(real) * c->d);
  /* embedding lookup: token id -> its row of E ([IE] section 1.1) */
  for (int i = 0; i < c->d; ++i) x[i] = bf(T_EMBED(m)[(size_t)token * c->d + i]);
  for (int l = 0; l < c->n_layers; ++l) {
    qkv_rope(m, l, x, rope_pos, q, k, v);
    /* append this position's key and value to the cache in its bf16 storage format */
    uint16_t* kr = m->kc + kv_index(m, l, seq, pos);
    uint16_t* vr = m->vc + kv_index(m, l, seq, pos);
    for (int i = 0; i < kd; ++i) {
      kr[i] = orc_bf16(k[i]);
      vr[i] = orc_bf16(v[i]);
    }
    /* attend to positions 0..pos, the current one included */
    attention_r(q, m->kc + kv_index(m, l, seq, 0), m->vc + kv_index(m, l, seq, 0), pos + 1, c->hq, c->hk, c->dh, o);
    gemv_r(T_LAYER(m, l, L_WO), c->d, qd, o, NULL, y);
    for (int i = 0; i < c->d; ++i) x[i] += y[i];
    ffn_block(m, l, x);
  }
  const int tok = lm_head(m, x, logits);
  free(x); free(q); free(k); free(v); free(o); free(y);
  return tok;
}

/* The same network over a whole prefix with no cache: every layer processes all positions, each
 * position attending causally to positions <= itself. Keys and values pass through the bf16 storage
 * rounding, as the cache would store them. Independent of orc_step's cache bookkeeping. */
int orc_forward_nocache(const orc_model* m, const int* tokens, int n, double rope_off, double* logits_last) {
  if (!m) return -1;
  const orc_config* c = &m->c;
  if (!tokens || n <= 0 || !logits_last) return -1;
  for (int t = 0; t < n; ++t)
    if (tokens[t] < 0 || tokens[t] >= c->v) return -1;
  const int qd = c->hq * c->dh, kd = c->hk * c->dh;
  real* X = (real*)malloc(sizeof(real) * (size_t)n * c->d);
  real* Q = (real*)malloc(sizeof(real) * (size_t)n * qd);
  uint16_t* K = (uint16_t*)malloc(2 * (size_t)n * kd);
  uint16_t* V = (uint16_t*)malloc(2 * (size_t)n * kd);
  real* k = (real*)malloc(sizeof(real) * kd);
  real* v = (real*)malloc(sizeof(real) * kd);
  real* o = (real*)malloc(sizeof(real) * qd);
  real* y = (real*)malloc(sizeof(real) * c->d);
  for (int t = 0; t < n; ++t)
    for (int i = 0; i < c->d; ++i) X[(size_t)t * c->d + i] = bf(T_EMBED(m)[(size_t)tokens[t] * c->d + i]);
  for (int l = 0; l < c->n_layers; ++l) {
    for (int t = 0; t < n; ++t) {
      qkv_rope(m, l, X + (size_t)t * c->d, rope_off + t, Q + (size_t)t * qd, k, v);
      for (int i = 0; i < kd; ++i) {
        K[(size_t)t * kd + i] = orc_bf16(k[i]);
        V[(size_t)t * kd + i] = orc_bf16(v[i]);
      }
    }
    for (int t = 0; t < n; ++t) {
      attention_r(Q + (size_t)t * qd, K, V, t + 1, c->hq, c->hk, c->dh, o);
      gemv_r(T_LAYER(m, l, L_WO), c->d, qd, o, NULL, y);
      for (int i = 0; i < c->d; ++i) X[(size_t)t * c->d + i] += y[i];
      ffn_block(m, l, X + (size_t)t * c->d);
    }
  }
  const int tok = lm_head(m, X + (size_t)(n - 1) * c->d, logits_last);
  free(X); free(Q); free(K); free(V); free(k); free(v); free(o); free(y);
  return tok;
}
