/* Drives the C oracle (oracle/oracle.c) under AddressSanitizer and UndefinedBehaviorSanitizer on
 * the CPU: a tiny dense model, its fp8 variant and a tiny mixture-of-experts model each run a
 * short prompt through oc_step, the dense ones also through oc_full_recompute, and the sampler and
 * router run on edge cases (ties, k larger than the vocabulary, too many experts). Any
 * out-of-bounds access, use after free or undefined operation aborts the process; the numbers are
 * only sanity-checked (finite, recompute close to the step-by-step pass). Prints "ok". Test code
 * only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab_size;
  float rms_eps, rope_theta;
  int32_t max_seq;
  int32_t n_experts, n_experts_active, expert_ffn_dim;
  int32_t weight_format;
} oc_config;
typedef struct {
  const uint16_t *embed, *final_norm, *lm_head;
  const uint16_t *const *attn_norm, *const *wq, *const *wk, *const *wv, *const *wo;
  const uint16_t *const *ffn_norm, *const *w_gate, *const *w_up, *const *w_down;
  const uint16_t *const *w_router, *const *moe_gate, *const *moe_up, *const *moe_down;
  const float* w_scale;
} oc_weights;

int oc_step(const oc_config* c, const oc_weights* w, uint16_t* kc, uint16_t* vc, int token, int pos, float* logits);
int oc_full_recompute(const oc_config* c, const oc_weights* w, const int* tokens, int n, float* logits);
int oc_topk_sample(const float* logits, int n, int k, float temperature, uint64_t seed, int64_t pos, int* cand_idx,
                   double* cand_p, double* u_out);
int oc_moe_route(const float* z, int E, int A, int* idx, double* w);
int oc_argmax(const float* v, int n);
void oc_set_threads(int n);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(g_state >> 33);
}
/* a bf16 of magnitude below ~0.05 (exponent field at most 121), random sign and mantissa */
static uint16_t small_bf16(void) {
  const uint32_t r = next_u32();
  return (uint16_t)(((r & 1u) << 15) | ((110u + (r >> 1) % 12u) << 7) | ((r >> 8) & 0x7fu));
}
static uint16_t* bf16_array(size_t n) {
  uint16_t* p = (uint16_t*)malloc(n * sizeof(uint16_t));
  for (size_t i = 0; i < n; i++) p[i] = small_bf16();
  return p;
}
static uint16_t* gain_array(size_t n) { /* norm gains near 1.0 */
  uint16_t* p = (uint16_t*)malloc(n * sizeof(uint16_t));
  for (size_t i = 0; i < n; i++) p[i] = (uint16_t)(0x3f80u + (next_u32() & 7u));
  return p;
}
static uint16_t* code_array(size_t n) { /* e4m3 codes, the NaN code 0x7f/0xff excluded */
  uint8_t* p = (uint8_t*)malloc(n);
  for (size_t i = 0; i < n; i++) {
    uint8_t b = (uint8_t)next_u32();
    if ((b & 0x7f) == 0x7f) b ^= 1;
    p[i] = b;
  }
  return (uint16_t*)p;
}

typedef struct {
  oc_config c;
  oc_weights w;
  const uint16_t** arrays[13];
  float* scales;
} model;

static model make_model(oc_config c) {
  model m;
  memset(&m, 0, sizeof m);
  m.c = c;
  const int L = c.n_layers, d = c.d_model, q = c.n_heads * c.head_dim, kv = c.n_kv_heads * c.head_dim;
  const int F = c.ffn_dim, E = c.n_experts, Fe = c.expert_ffn_dim;
  const int fp8 = c.weight_format == 1;
  for (int a = 0; a < 13; a++) m.arrays[a] = (const uint16_t**)calloc((size_t)L, sizeof(uint16_t*));
  for (int l = 0; l < L; l++) {
    m.arrays[0][l] = gain_array((size_t)d);
    m.arrays[1][l] = fp8 ? code_array((size_t)q * d) : bf16_array((size_t)q * d);
    m.arrays[2][l] = fp8 ? code_array((size_t)kv * d) : bf16_array((size_t)kv * d);
    m.arrays[3][l] = fp8 ? code_array((size_t)kv * d) : bf16_array((size_t)kv * d);
    m.arrays[4][l] = fp8 ? code_array((size_t)d * q) : bf16_array((size_t)d * q);
    m.arrays[5][l] = gain_array((size_t)d);
    if (E > 0) {
      m.arrays[9][l] = bf16_array((size_t)E * d);
      m.arrays[10][l] = bf16_array((size_t)E * Fe * d);
      m.arrays[11][l] = bf16_array((size_t)E * Fe * d);
      m.arrays[12][l] = bf16_array((size_t)E * d * Fe);
    } else {
      m.arrays[6][l] = fp8 ? code_array((size_t)F * d) : bf16_array((size_t)F * d);
      m.arrays[7][l] = fp8 ? code_array((size_t)F * d) : bf16_array((size_t)F * d);
      m.arrays[8][l] = fp8 ? code_array((size_t)d * F) : bf16_array((size_t)d * F);
    }
  }
  m.w.embed = bf16_array((size_t)c.vocab_size * d);
  m.w.final_norm = gain_array((size_t)d);
  m.w.lm_head = fp8 ? code_array((size_t)c.vocab_size * d) : bf16_array((size_t)c.vocab_size * d);
  m.w.attn_norm = m.arrays[0];
  m.w.wq = m.arrays[1];
  m.w.wk = m.arrays[2];
  m.w.wv = m.arrays[3];
  m.w.wo = m.arrays[4];
  m.w.ffn_norm = m.arrays[5];
  m.w.w_gate = m.arrays[6];
  m.w.w_up = m.arrays[7];
  m.w.w_down = m.arrays[8];
  m.w.w_router = m.arrays[9];
  m.w.moe_gate = m.arrays[10];
  m.w.moe_up = m.arrays[11];
  m.w.moe_down = m.arrays[12];
  if (fp8) {
    m.scales = (float*)malloc(sizeof(float) * (size_t)(7 * L + 1));
    for (int i = 0; i < 7 * L + 1; i++) m.scales[i] = 0.002f + 0.0001f * (float)i;
    m.w.w_scale = m.scales;
  }
  return m;
}

static void free_model(model* m) {
  for (int a = 0; a < 13; a++) {
    for (int l = 0; l < m->c.n_layers; l++) free((void*)m->arrays[a][l]);
    free((void*)m->arrays[a]);
  }
  free((void*)m->w.embed);
  free((void*)m->w.final_norm);
  free((void*)m->w.lm_head);
  free(m->scales);
}

/* a prompt of n tokens step by step; the dense models also through the whole-sequence pass */
static int run_model(const char* name, oc_config c, int n, int recompute) {
  model m = make_model(c);
  const size_t cache = (size_t)c.n_layers * c.n_kv_heads * c.max_seq * c.head_dim;
  uint16_t* kc = (uint16_t*)calloc(cache, sizeof(uint16_t));
  uint16_t* vc = (uint16_t*)calloc(cache, sizeof(uint16_t));
  int* tokens = (int*)malloc(sizeof(int) * (size_t)n);
  float* step = (float*)malloc(sizeof(float) * (size_t)n * c.vocab_size);
  for (int t = 0; t < n; t++) tokens[t] = (int)(next_u32() % (uint32_t)c.vocab_size);
  int bad = 0;
  for (int t = 0; t < n && !bad; t++)
    if (oc_step(&c, &m.w, kc, vc, tokens[t], t, step + (size_t)t * c.vocab_size) != 0) bad = 1;
  for (size_t i = 0; i < (size_t)n * c.vocab_size && !bad; i++)
    if (!isfinite(step[i])) bad = 2;
  if (!bad && recompute) {
    float* full = (float*)malloc(sizeof(float) * (size_t)n * c.vocab_size);
    if (oc_full_recompute(&c, &m.w, tokens, n, full) != 0) bad = 3;
    double num = 0, den = 0;
    for (size_t i = 0; i < (size_t)n * c.vocab_size && !bad; i++) {
      num += (double)(full[i] - step[i]) * (full[i] - step[i]);
      den += (double)step[i] * step[i];
    }
    if (!bad && !(sqrt(num / (den > 0 ? den : 1)) < 1e-3)) bad = 4;
    free(full);
  }
  /* the out-of-range token and position are rejected, not read */
  if (!bad && oc_step(&c, &m.w, kc, vc, c.vocab_size, 0, step) == 0) bad = 5;
  if (!bad && oc_step(&c, &m.w, kc, vc, 0, c.max_seq, step) == 0) bad = 6;
  if (bad) printf("%s: failure %d\n", name, bad);
  free(kc);
  free(vc);
  free(tokens);
  free(step);
  free_model(&m);
  return bad;
}

static int run_sampler(void) {
  float v[9] = {1.0f, 3.0f, 3.0f, -2.0f, 0.5f, 3.0f, -1.0f, 0.0f, 2.0f};
  if (oc_argmax(v, 9) != 1) return 1;
  int cand[9];
  double p[9], u = 0;
  for (int64_t pos = 0; pos < 64; pos++) {
    const int tok = oc_topk_sample(v, 9, 4, 0.8f, 1234u, pos, cand, p, &u);
    if (tok < 0 || tok >= 9 || !(u >= 0 && u < 1)) return 2;
  }
  /* k above the vocabulary is clamped to it */
  if (oc_topk_sample(v, 9, 50, 1.0f, 7u, 3, NULL, NULL, NULL) < 0) return 3;
  float z[16];
  for (int i = 0; i < 16; i++) z[i] = (float)((i * 7) % 5); /* ties */
  int idx[4];
  double w[4];
  if (oc_moe_route(z, 16, 4, idx, w) != 0) return 4;
  if (oc_moe_route(z, 16, 17, idx, w) != -1) return 5; /* more experts than there are */
  double s = 0;
  for (int i = 0; i < 4; i++) {
    if (idx[i] < 0 || idx[i] >= 16) return 6;
    for (int j = 0; j < i; j++)
      if (idx[j] == idx[i]) return 7;
    s += w[i];
  }
  return fabs(s - 1.0) < 1e-12 ? 0 : 8;
}

int main(void) {
  oc_set_threads(1);
  const oc_config dense = {2, 256, 4, 2, 64, 1024, 512, 1e-6f, 10000.0f, 12, 0, 0, 0, 0};
  oc_config fp8 = dense;
  fp8.weight_format = 1;
  const oc_config moe = {2, 256, 8, 1, 128, 0, 512, 1e-6f, 10000.0f, 12, 16, 4, 256, 0};
  int bad = run_model("dense", dense, 10, 1);
  bad |= run_model("fp8", fp8, 10, 1);
  bad |= run_model("moe", moe, 10, 0);
  const int sb = run_sampler();
  if (sb) printf("sampler/router: failure %d\n", sb);
  if (bad || sb) return 1;
  printf("ok\n");
  return 0;
}
