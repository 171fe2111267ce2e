/*
 * oracle.c -- plain, slow CPU reference of one batch-1 decoder step (TEST INFRASTRUCTURE ONLY).
 *
 * Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may load this file's
 * library. It shares no code, header, table or constant with the GPU library.
 *
 * What it computes. The pages describe batch-1 autoregressive decoding of a dense decoder-only
 * transformer: for each new token every active weight is read once, and the work is "MatMul,
 * attention, normalization and sampling" inside one GPU-resident program (agentlenshq.com,
 * 《突破内存墙：在标准 GPU 上实现 3,000 tokens/s 的推理速度》, sections "瓶颈：是内存带宽，而非计算" and
 * "Kog 的解决方案 / The Monokernel Runtime"; aikraft.ru «3000 токенов в секунду…», §02 and §04
 * "Моноядро"). The pages never write the decoder down, so this file follows the plainest
 * Llama-style reading, listed in the design notes:
 *   pre-RMSNorm blocks, no biases, untied LM head; RoPE with rotate-half pairs (i, i+hd/2) and
 *   angles p * theta^(-2i/hd) computed in fp64; grouped-query attention where query head h reads
 *   KV head h / (n_heads / n_kv_heads); causal softmax with scale 1/sqrt(hd); SwiGLU FFN
 *   silu(Wg u) * (Wu u); K (after RoPE) and V rounded to bf16 (round-to-nearest-even) when written
 *   to the cache. A mixture-of-experts layer replaces the FFN by a router and n_experts SwiGLU
 *   experts of which n_experts_active run per token (oc_moe_route, oc_moe_ffn).
 *
 * Precision: bf16 weights are widened exactly to fp32; activations and dot products are fp32 with
 * one accumulator per output summed in ascending index order (oc_set_gemv_order(1) sums the
 * same terms in descending order instead: a second, equally valid rounding of the same model that
 * the tests use to measure how far two correct fp32 renditions of a deep model drift apart); the softmax denominator and the
 * attention-weighted sum of V are fp64 (stored as fp32). No -ffast-math: every reduction runs in
 * the order written here. Row loops may be split over threads (rows only), which cannot change
 * any result bit.
 *
 * 8-bit weights (weight_format 1). The pages note that 8-bit weights halve the bytes read per
 * token and so roughly double a bandwidth-bound decoder's ceiling, at some cost in accuracy
 * (aikraft.ru, §02; wink.run, 《GPU 算力越堆越高,生成 token 为什么还是慢》, the section on what
 * optimisations change), while the engine they describe itself quantizes nothing (zdabc.icu,
 * 《Kog 推理引擎：不砍精度，单请求冲到 3000 tokens/s》). They fix no 8-bit format, so this file reads
 * it as the OCP E4M3 encoding (e4m3fn) with one fp32 scale per matrix: the matrix is the scale
 * times the decoded codes (oc_e4m3_to_f32, oc_gemv_e4m3). Everything else is the bf16 model.
 *
 * Sampling: greedy = argmax with ties to the lower index. Top-k: z = logits / T (fp32); the k
 * largest z (ties to the lower index) in descending order; p_j = exp(z_j - z_0) / sum (fp64);
 * u = (splitmix64(seed ^ splitmix64(pos)) >> 40) * 2^-24; the first j whose running fp64 sum of
 * p exceeds u is chosen (the last one if none does). SplitMix64 is Steele, Lea & Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab_size;
  float rms_eps, rope_theta;
  int32_t max_seq;
  int32_t n_experts, n_experts_active, expert_ffn_dim; /* n_experts == 0: dense feed-forward */
  int32_t weight_format; /* 0: bf16 matrices; 1: fp8 e4m3fn codes with one fp32 scale per matrix */
} oc_config;

/* All matrices row-major [out][in], bf16 bit patterns. Per-layer arrays hold n_layers pointers.
 * Mixture-of-experts layers (n_experts > 0) use w_router[l] [E][d] and, per layer, the experts'
 * matrices stacked: moe_gate[l] and moe_up[l] [E][Fe][d], moe_down[l] [E][d][Fe]; w_gate, w_up and
 * w_down are then unused. */
typedef struct {
  const uint16_t *embed, *final_norm, *lm_head;
  const uint16_t *const *attn_norm, *const *wq, *const *wk, *const *wv, *const *wo;
  const uint16_t *const *ffn_norm, *const *w_gate, *const *w_up, *const *w_down;
  const uint16_t *const *w_router, *const *moe_gate, *const *moe_up, *const *moe_down;
  /* weight_format 1: wq, wk, wv, wo, w_gate, w_up, w_down and lm_head hold one byte per weight
   * (e4m3fn codes, same [out][in] layout) and the matrix is scale * decoded codes, with the scales
   * in w_scale: [n_layers][7] in the order wq, wk, wv, wo, w_gate, w_up, w_down, then lm_head.
   * Embedding and norm gains stay bf16. */
  const float* w_scale;
} oc_weights;

static int g_threads = 1;
static int g_gemv_desc = 0;
/* optional log of the router logits of oc_step: [max_pos][n_layers][n_experts] fp32 */
static float* g_route_log = NULL;
static int g_route_log_pos = 0;

void oc_set_threads(int n) { g_threads = n < 1 ? 1 : n; }
void oc_set_gemv_order(int descending) { g_gemv_desc = descending ? 1 : 0; }
int oc_get_threads(void) { return g_threads; }
/* Record the router logits of every mixture-of-experts layer of oc_step at positions < max_pos
 * into buf ([max_pos][n_layers][n_experts]); NULL stops recording. */
void oc_set_route_log(float* buf, int max_pos) {
  g_route_log = buf;
  g_route_log_pos = max_pos;
}

/* ------------------------------------------------------------------ scalar helpers */

float oc_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Value of an fp8 e4m3fn code (the OCP 8-bit floating-point format's E4M3 encoding): sign bit 7,
 * exponent bits 6..3 with bias 7, mantissa bits 2..0; exponent 0 encodes the subnormals
 * m * 2^-9; there are no infinities, and exponent 15 with mantissa 7 is NaN. Every value is exact
 * in fp32. */
float oc_e4m3_to_f32(uint8_t b) {
  const int sign = b >> 7, e = (b >> 3) & 15, m = b & 7;
  float v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexpf((float)m, -9);
  else
    v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
  return sign ? -v : v;
}

/* fp32 -> bf16 with round-to-nearest-even (NaN kept quiet). */
uint16_t oc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

uint64_t oc_splitmix64(uint64_t x) {
  uint64_t z = x + 0x9e3779b97f4a7c15ull;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

/* uniform in [0,1) with 24 random bits, a function of (seed, pos) only */
double oc_uniform(uint64_t seed, int64_t pos) {
  uint64_t r = oc_splitmix64(seed ^ oc_splitmix64((uint64_t)pos));
  return (double)(r >> 40) * (1.0 / 16777216.0);
}

/* ------------------------------------------------------------------ building blocks */

/* y[r] = sum_k W[r][k] * x[k], fp32, k ascending. W is [rows][cols] bf16. */
void oc_gemv(const uint16_t* W, const float* x, float* y, int rows, int cols) {
  int r;
#pragma omp parallel for num_threads(g_threads) schedule(static) if (g_threads > 1)
  for (r = 0; r < rows; r++) {
    const uint16_t* w = W + (size_t)r * cols;
    float acc = 0.0f;
    if (g_gemv_desc)
      for (int k = cols - 1; k >= 0; k--) acc += oc_bf16_to_f32(w[k]) * x[k];
    else
      for (int k = 0; k < cols; k++) acc += oc_bf16_to_f32(w[k]) * x[k];
    y[r] = acc;
  }
}

/* y[r] = scale * sum_k q(W[r][k]) * x[k] for a matrix of e4m3fn codes: the products and the sum
 * are fp32 in the order of oc_gemv, and the scale multiplies the finished sum. */
void oc_gemv_e4m3(const uint8_t* W, float scale, const float* x, float* y, int rows, int cols) {
  int r;
#pragma omp parallel for num_threads(g_threads) schedule(static) if (g_threads > 1)
  for (r = 0; r < rows; r++) {
    const uint8_t* w = W + (size_t)r * cols;
    float acc = 0.0f;
    if (g_gemv_desc)
      for (int k = cols - 1; k >= 0; k--) acc += oc_e4m3_to_f32(w[k]) * x[k];
    else
      for (int k = 0; k < cols; k++) acc += oc_e4m3_to_f32(w[k]) * x[k];
    y[r] = acc * scale;
  }
}

/* Matrix m (0..6: wq, wk, wv, wo, w_gate, w_up, w_down) of layer l, or the LM head (l == n_layers),
 * in the model's weight format. */
static void mat_gemv(const oc_config* c, const oc_weights* w, int l, int m, const uint16_t* W, const float* x,
                     float* y, int rows, int cols) {
  if (c->weight_format == 1)
    oc_gemv_e4m3((const uint8_t*)W, w->w_scale[l < c->n_layers ? l * 7 + m : c->n_layers * 7], x, y, rows, cols);
  else
    oc_gemv(W, x, y, rows, cols);
}

/* u = x * (1/sqrt(mean(x^2) + eps)) * g ; the sum of squares is fp32, i ascending. */
void oc_rmsnorm(const float* x, const uint16_t* g, float* u, int n, float eps) {
  float ss = 0.0f;
  for (int i = 0; i < n; i++) ss += x[i] * x[i];
  float r = 1.0f / sqrtf(ss / (float)n + eps);
  for (int i = 0; i < n; i++) u[i] = (x[i] * r) * oc_bf16_to_f32(g[i]);
}

/* Rotate each pair (y[i], y[i+hd/2]) of one head by angle pos * theta^(-2i/hd). */
void oc_rope(float* y, int hd, int pos, float theta) {
  int half = hd / 2;
  for (int i = 0; i < half; i++) {
    double freq = pow((double)theta, -2.0 * (double)i / (double)hd);
    double phi = (double)pos * freq;
    float c = (float)cos(phi), s = (float)sin(phi);
    float a = y[i], b = y[i + half];
    y[i] = a * c - b * s;
    y[i + half] = b * c + a * s;
  }
}

float oc_silu(float g) { return g / (1.0f + expf(-g)); }

/* Softmax attention of one query over n cached rows (K, V rows of length hd, bf16, row stride
 * `stride` elements). Scores fp32 (dot then / sqrt(hd)); exp, sum and weighted V sum in fp64.
 * Writes out[hd]; if probs != NULL also the n probabilities (fp64). */
void oc_attend(const float* q, const uint16_t* K, const uint16_t* V, int n, int hd, size_t stride,
               float* out, double* probs) {
  float* s = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
  double* acc = (double*)calloc((size_t)hd, sizeof(double));
  float scale_div = sqrtf((float)hd);
  float m = -INFINITY;
  for (int t = 0; t < n; t++) {
    const uint16_t* kr = K + (size_t)t * stride;
    float dot = 0.0f;
    for (int i = 0; i < hd; i++) dot += q[i] * oc_bf16_to_f32(kr[i]);
    s[t] = dot / scale_div;
    if (s[t] > m) m = s[t];
  }
  double S = 0.0;
  for (int t = 0; t < n; t++) S += exp((double)s[t] - (double)m);
  for (int t = 0; t < n; t++) {
    double p = exp((double)s[t] - (double)m) / S;
    if (probs) probs[t] = p;
    const uint16_t* vr = V + (size_t)t * stride;
    for (int i = 0; i < hd; i++) acc[i] += p * (double)oc_bf16_to_f32(vr[i]);
  }
  for (int i = 0; i < hd; i++) out[i] = (float)acc[i];
  free(s);
  free(acc);
}

int oc_argmax(const float* v, int n) {
  int best = 0;
  for (int i = 1; i < n; i++)
    if (v[i] > v[best]) best = i;
  return best;
}

/* Top-k candidates of z = logits / T in descending order (ties -> lower index), their fp64
 * probabilities, the uniform draw and the chosen token. Returns the token. */
int oc_topk_sample(const float* logits, int n, int k, float temperature, uint64_t seed, int64_t pos,
                   int* cand_idx, double* cand_p, double* u_out) {
  if (k < 1) k = 1;
  if (k > n) k = n;
  float* z = (float*)malloc(sizeof(float) * (size_t)n);
  for (int i = 0; i < n; i++) z[i] = logits[i] / temperature;
  /* selection by repeated scans: each round takes the largest remaining (lowest index on ties) */
  char* used = (char*)calloc((size_t)n, 1);
  int* idx = (int*)malloc(sizeof(int) * (size_t)k);
  for (int j = 0; j < k; j++) {
    int b = -1;
    for (int i = 0; i < n; i++) {
      if (used[i]) continue;
      if (b < 0 || z[i] > z[b]) b = i;
    }
    idx[j] = b;
    used[b] = 1;
  }
  double* e = (double*)malloc(sizeof(double) * (size_t)k);
  double S = 0.0;
  for (int j = 0; j < k; j++) {
    e[j] = exp((double)z[idx[j]] - (double)z[idx[0]]);
    S += e[j];
  }
  double u = oc_uniform(seed, pos);
  int chosen = idx[k - 1];
  double cum = 0.0;
  int done = 0;
  for (int j = 0; j < k; j++) {
    double p = e[j] / S;
    if (cand_idx) cand_idx[j] = idx[j];
    if (cand_p) cand_p[j] = p;
    cum += p;
    if (!done && cum > u) {
      chosen = idx[j];
      done = 1;
    }
  }
  if (u_out) *u_out = u;
  free(z);
  free(used);
  free(idx);
  free(e);
  return chosen;
}

/* ------------------------------------------------------------------ mixture of experts */

/* Router of a mixture-of-experts layer (the pages: only the routed experts' weights are read per
 * token, so bandwidth follows the active parameters -- aikraft.ru «3000 токенов в секунду…», §02;
 * agentlenshq.com, 《突破内存墙…》, opening section). The pages fix no router; the reading here:
 * p = softmax(z) over all E router logits (fp64), the A experts with the largest z (ties -> lower
 * index, i.e. the A largest p) in descending order, and their weights renormalised to sum to 1:
 * w_i = p_i / sum of the selected p. Writes idx[A] and w[A] (fp64); returns 0, or -1 on bad sizes. */
int oc_moe_route(const float* z, int E, int A, int* idx, double* w) {
  if (E < 1 || A < 1 || A > E) return -1;
  double m = -INFINITY;
  for (int e = 0; e < E; e++)
    if ((double)z[e] > m) m = (double)z[e];
  double* p = (double*)malloc(sizeof(double) * (size_t)E);
  double Z = 0.0;
  for (int e = 0; e < E; e++) {
    p[e] = exp((double)z[e] - m);
    Z += p[e];
  }
  for (int e = 0; e < E; e++) p[e] /= Z;
  char* used = (char*)calloc((size_t)E, 1);
  double S = 0.0;
  for (int j = 0; j < A; j++) {
    int b = -1;
    for (int e = 0; e < E; e++) {
      if (used[e]) continue;
      if (b < 0 || z[e] > z[b]) b = e;
    }
    used[b] = 1;
    idx[j] = b;
    S += p[b];
  }
  for (int j = 0; j < A; j++) w[j] = p[idx[j]] / S;
  free(p);
  free(used);
  return 0;
}

/* Feed-forward output of a mixture-of-experts layer for the normalised input u[d]:
 * y = sum over the routed experts i (in rank order) of (float)w_i * down_i(silu(gate_i u) * up_i u),
 * accumulated in fp32. Writes y[d]; z_out[E] (if not NULL) receives the router logits. */
void oc_moe_ffn(const oc_config* c, const oc_weights* w, int l, const float* u, float* y, float* z_out) {
  const int d = c->d_model, E = c->n_experts, A = c->n_experts_active, Fe = c->expert_ffn_dim;
  float* z = (float*)malloc(sizeof(float) * (size_t)E);
  int* idx = (int*)malloc(sizeof(int) * (size_t)A);
  double* wt = (double*)malloc(sizeof(double) * (size_t)A);
  float* g = (float*)malloc(sizeof(float) * (size_t)Fe);
  float* up = (float*)malloc(sizeof(float) * (size_t)Fe);
  float* t = (float*)malloc(sizeof(float) * (size_t)d);
  oc_gemv(w->w_router[l], u, z, E, d);
  oc_moe_route(z, E, A, idx, wt);
  for (int i = 0; i < d; i++) y[i] = 0.0f;
  for (int j = 0; j < A; j++) {
    const int e = idx[j];
    oc_gemv(w->moe_gate[l] + (size_t)e * Fe * d, u, g, Fe, d);
    oc_gemv(w->moe_up[l] + (size_t)e * Fe * d, u, up, Fe, d);
    for (int i = 0; i < Fe; i++) g[i] = oc_silu(g[i]) * up[i];
    oc_gemv(w->moe_down[l] + (size_t)e * d * Fe, g, t, d, Fe);
    const float wj = (float)wt[j];
    for (int i = 0; i < d; i++) y[i] += wj * t[i];
  }
  if (z_out)
    for (int e = 0; e < E; e++) z_out[e] = z[e];
  free(z); free(idx); free(wt); free(g); free(up); free(t);
}

/* ------------------------------------------------------------------ one decode step */

/* KV cache of the oracle: K and V planes, each [n_layers][n_kv_heads][max_seq][head_dim] bf16. */
static size_t kv_off(const oc_config* c, int l, int j, int t) {
  return (((size_t)l * c->n_kv_heads + j) * c->max_seq + t) * c->head_dim;
}

/* Process `token` at position `pos`: append its K/V to the cache, return the logits [V]. */
int oc_step(const oc_config* c, const oc_weights* w, uint16_t* kc, uint16_t* vc, int token, int pos,
            float* logits) {
  const int d = c->d_model, hd = c->head_dim, nq = c->n_heads, nkv = c->n_kv_heads, F = c->ffn_dim;
  if (pos < 0 || pos >= c->max_seq || token < 0 || token >= c->vocab_size) return -1;
  if (nq % nkv != 0) return -1;
  if (c->weight_format != 0 && (c->weight_format != 1 || c->n_experts > 0 || !w->w_scale)) return -1;
  const int group = nq / nkv;
  float* x = (float*)malloc(sizeof(float) * d);
  float* u = (float*)malloc(sizeof(float) * d);
  float* q = (float*)malloc(sizeof(float) * nq * hd);
  float* k = (float*)malloc(sizeof(float) * nkv * hd);
  float* v = (float*)malloc(sizeof(float) * nkv * hd);
  float* o = (float*)malloc(sizeof(float) * nq * hd);
  float* t = (float*)malloc(sizeof(float) * (d > F ? d : F));
  float* g = (float*)malloc(sizeof(float) * F);
  float* up = (float*)malloc(sizeof(float) * F);

  for (int i = 0; i < d; i++) x[i] = oc_bf16_to_f32(w->embed[(size_t)token * d + i]);

  for (int l = 0; l < c->n_layers; l++) {
    /* attention block */
    oc_rmsnorm(x, w->attn_norm[l], u, d, c->rms_eps);
    mat_gemv(c, w, l, 0, w->wq[l], u, q, nq * hd, d);
    mat_gemv(c, w, l, 1, w->wk[l], u, k, nkv * hd, d);
    mat_gemv(c, w, l, 2, w->wv[l], u, v, nkv * hd, d);
    for (int h = 0; h < nq; h++) oc_rope(q + h * hd, hd, pos, c->rope_theta);
    for (int j = 0; j < nkv; j++) oc_rope(k + j * hd, hd, pos, c->rope_theta);
    for (int j = 0; j < nkv; j++)
      for (int i = 0; i < hd; i++) {
        kc[kv_off(c, l, j, pos) + i] = oc_f32_to_bf16(k[j * hd + i]);
        vc[kv_off(c, l, j, pos) + i] = oc_f32_to_bf16(v[j * hd + i]);
      }
    for (int h = 0; h < nq; h++) {
      int j = h / group;
      oc_attend(q + h * hd, kc + kv_off(c, l, j, 0), vc + kv_off(c, l, j, 0), pos + 1, hd, (size_t)hd,
                o + h * hd, NULL);
    }
    mat_gemv(c, w, l, 3, w->wo[l], o, t, d, nq * hd);
    for (int i = 0; i < d; i++) x[i] += t[i];
    /* feed-forward block */
    oc_rmsnorm(x, w->ffn_norm[l], u, d, c->rms_eps);
    if (c->n_experts > 0) {
      float* zl = g_route_log && pos < g_route_log_pos
                      ? g_route_log + ((size_t)pos * c->n_layers + l) * c->n_experts : NULL;
      oc_moe_ffn(c, w, l, u, t, zl);
    } else {
      mat_gemv(c, w, l, 4, w->w_gate[l], u, g, F, d);
      mat_gemv(c, w, l, 5, w->w_up[l], u, up, F, d);
      for (int i = 0; i < F; i++) g[i] = oc_silu(g[i]) * up[i];
      mat_gemv(c, w, l, 6, w->w_down[l], g, t, d, F);
    }
    for (int i = 0; i < d; i++) x[i] += t[i];
  }
  oc_rmsnorm(x, w->final_norm, u, d, c->rms_eps);
  mat_gemv(c, w, c->n_layers, 0, w->lm_head, u, logits, c->vocab_size, d);

  free(x); free(u); free(q); free(k); free(v); free(o); free(t); free(g); free(up);
  return 0;
}

/* ------------------------------------------------------------------ brute-force recompute */

/* Whole-sequence pass in matrix form with no cache reuse: every position's hidden state is
 * carried through all layers as a [n][d] matrix and attention applies an explicit causal mask.
 * K and V are rounded to bf16 like the cache. Writes logits [n][V]. Written independently of
 * oc_step so that caching, position bookkeeping and masking are cross-checked. */
int oc_full_recompute(const oc_config* c, const oc_weights* w, const int* tokens, int n, float* logits) {
  const int d = c->d_model, hd = c->head_dim, nq = c->n_heads, nkv = c->n_kv_heads, F = c->ffn_dim;
  if (n <= 0 || nq % nkv != 0) return -1;
  if (c->weight_format != 0 && (c->weight_format != 1 || c->n_experts > 0 || !w->w_scale)) return -1;
  for (int r = 0; r < n; r++)
    if (tokens[r] < 0 || tokens[r] >= c->vocab_size) return -1;
  const int group = nq / nkv;
  float* X = (float*)malloc(sizeof(float) * (size_t)n * d);
  float* U = (float*)malloc(sizeof(float) * (size_t)n * d);
  float* Q = (float*)malloc(sizeof(float) * (size_t)n * nq * hd);
  float* Kf = (float*)malloc(sizeof(float) * (size_t)n * nkv * hd);
  float* Vf = (float*)malloc(sizeof(float) * (size_t)n * nkv * hd);
  uint16_t* Kb = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)nkv * n * hd); /* [j][t][i] */
  uint16_t* Vb = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)nkv * n * hd);
  float* O = (float*)malloc(sizeof(float) * (size_t)n * nq * hd);
  float* T = (float*)malloc(sizeof(float) * (size_t)n * (d > F ? d : F));
  float* G = (float*)malloc(sizeof(float) * (size_t)n * F);
  float* Up = (float*)malloc(sizeof(float) * (size_t)n * F);
  float* sc = (float*)malloc(sizeof(float) * (size_t)n);

  for (int r = 0; r < n; r++) {
    int tok = tokens[r] < 0 || tokens[r] >= c->vocab_size ? 0 : tokens[r];
    for (int i = 0; i < d; i++) X[(size_t)r * d + i] = oc_bf16_to_f32(w->embed[(size_t)tok * d + i]);
  }
  for (int l = 0; l < c->n_layers; l++) {
    for (int r = 0; r < n; r++) oc_rmsnorm(X + (size_t)r * d, w->attn_norm[l], U + (size_t)r * d, d, c->rms_eps);
    for (int r = 0; r < n; r++) {
      mat_gemv(c, w, l, 0, w->wq[l], U + (size_t)r * d, Q + (size_t)r * nq * hd, nq * hd, d);
      mat_gemv(c, w, l, 1, w->wk[l], U + (size_t)r * d, Kf + (size_t)r * nkv * hd, nkv * hd, d);
      mat_gemv(c, w, l, 2, w->wv[l], U + (size_t)r * d, Vf + (size_t)r * nkv * hd, nkv * hd, d);
      for (int h = 0; h < nq; h++) oc_rope(Q + (size_t)r * nq * hd + h * hd, hd, r, c->rope_theta);
      for (int j = 0; j < nkv; j++) oc_rope(Kf + (size_t)r * nkv * hd + j * hd, hd, r, c->rope_theta);
    }
    for (int j = 0; j < nkv; j++)
      for (int r = 0; r < n; r++)
        for (int i = 0; i < hd; i++) {
          Kb[((size_t)j * n + r) * hd + i] = oc_f32_to_bf16(Kf[(size_t)r * nkv * hd + j * hd + i]);
          Vb[((size_t)j * n + r) * hd + i] = oc_f32_to_bf16(Vf[(size_t)r * nkv * hd + j * hd + i]);
        }
    /* masked attention: row r attends to columns s <= r; masked columns get probability 0 */
    float scale_div = sqrtf((float)hd);
    for (int r = 0; r < n; r++)
      for (int h = 0; h < nq; h++) {
        int j = h / group;
        const float* qr = Q + (size_t)r * nq * hd + h * hd;
        float m = -INFINITY;
        for (int s = 0; s < n; s++) {
          if (s > r) { sc[s] = -INFINITY; continue; }
          const uint16_t* kr = Kb + ((size_t)j * n + s) * hd;
          float dot = 0.0f;
          for (int i = 0; i < hd; i++) dot += qr[i] * oc_bf16_to_f32(kr[i]);
          sc[s] = dot / scale_div;
          if (sc[s] > m) m = sc[s];
        }
        double S = 0.0;
        for (int s = 0; s < n; s++)
          if (s <= r) S += exp((double)sc[s] - (double)m);
        for (int i = 0; i < hd; i++) {
          double a = 0.0;
          for (int s = 0; s <= r; s++) {
            double p = exp((double)sc[s] - (double)m) / S;
            a += p * (double)oc_bf16_to_f32(Vb[((size_t)j * n + s) * hd + i]);
          }
          O[(size_t)r * nq * hd + h * hd + i] = (float)a;
        }
      }
    for (int r = 0; r < n; r++) {
      mat_gemv(c, w, l, 3, w->wo[l], O + (size_t)r * nq * hd, T + (size_t)r * d, d, nq * hd);
      for (int i = 0; i < d; i++) X[(size_t)r * d + i] += T[(size_t)r * d + i];
    }
    for (int r = 0; r < n; r++) oc_rmsnorm(X + (size_t)r * d, w->ffn_norm[l], U + (size_t)r * d, d, c->rms_eps);
    if (c->n_experts > 0) {
      /* grouped by expert: route every row, then run each expert over the rows sent to it and add
       * its weighted output to those rows (the rank-order sum of oc_step, in another order) */
      const int E = c->n_experts, A = c->n_experts_active, Fe = c->expert_ffn_dim;
      float* Z = (float*)malloc(sizeof(float) * (size_t)E);
      int* SI = (int*)malloc(sizeof(int) * (size_t)n * A);
      double* SW = (double*)malloc(sizeof(double) * (size_t)n * A);
      float* ge = (float*)malloc(sizeof(float) * (size_t)Fe);
      float* ue = (float*)malloc(sizeof(float) * (size_t)Fe);
      float* te = (float*)malloc(sizeof(float) * (size_t)d);
      float* Y = (float*)calloc((size_t)n * d, sizeof(float));
      for (int r = 0; r < n; r++) {
        oc_gemv(w->w_router[l], U + (size_t)r * d, Z, E, d);
        oc_moe_route(Z, E, A, SI + (size_t)r * A, SW + (size_t)r * A);
      }
      for (int e = 0; e < E; e++)
        for (int r = 0; r < n; r++)
          for (int j = 0; j < A; j++) {
            if (SI[(size_t)r * A + j] != e) continue;
            oc_gemv(w->moe_gate[l] + (size_t)e * Fe * d, U + (size_t)r * d, ge, Fe, d);
            oc_gemv(w->moe_up[l] + (size_t)e * Fe * d, U + (size_t)r * d, ue, Fe, d);
            for (int i = 0; i < Fe; i++) ge[i] = oc_silu(ge[i]) * ue[i];
            oc_gemv(w->moe_down[l] + (size_t)e * d * Fe, ge, te, d, Fe);
            const float wj = (float)SW[(size_t)r * A + j];
            for (int i = 0; i < d; i++) Y[(size_t)r * d + i] += wj * te[i];
          }
      for (size_t i = 0; i < (size_t)n * d; i++) X[i] += Y[i];
      free(Z); free(SI); free(SW); free(ge); free(ue); free(te); free(Y);
      continue;
    }
    for (int r = 0; r < n; r++) {
      mat_gemv(c, w, l, 4, w->w_gate[l], U + (size_t)r * d, G + (size_t)r * F, F, d);
      mat_gemv(c, w, l, 5, w->w_up[l], U + (size_t)r * d, Up + (size_t)r * F, F, d);
      for (int i = 0; i < F; i++) G[(size_t)r * F + i] = oc_silu(G[(size_t)r * F + i]) * Up[(size_t)r * F + i];
      mat_gemv(c, w, l, 6, w->w_down[l], G + (size_t)r * F, T + (size_t)r * d, d, F);
      for (int i = 0; i < d; i++) X[(size_t)r * d + i] += T[(size_t)r * d + i];
    }
  }
  for (int r = 0; r < n; r++) {
    oc_rmsnorm(X + (size_t)r * d, w->final_norm, U + (size_t)r * d, d, c->rms_eps);
    mat_gemv(c, w, c->n_layers, 0, w->lm_head, U + (size_t)r * d, logits + (size_t)r * c->vocab_size,
             c->vocab_size, d);
  }
  free(X); free(U); free(Q); free(Kf); free(Vf); free(Kb); free(Vb); free(O); free(T); free(G); free(Up); free(sc);
  return 0;
}
