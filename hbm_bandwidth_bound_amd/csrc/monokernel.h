// monokernel.h -- parameters of the persistent decode kernel and of the set-up kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace kie {

// device error word bits
enum : uint32_t {
  KERR_TIMEOUT = 1u << 0,    // a wait for another workgroup's data timed out
  KERR_ABORTED = 1u << 1,    // the host's abort word was set during the launch
  KERR_BAD_TOKEN = 1u << 2,  // an input token id was out of range (it was replaced by 0)
};

struct KParams {
  Shape s;
  Exch exo;
  const uint8_t* packed;     // tile streams of all waves
  const uint16_t* embed;     // [V][d] bf16 (inside the packed image)
  const uint16_t* norms;     // [L][2][d] + [d] bf16 (in the workspace)
  uint16_t* kv;              // [L][2][nkv][max_seq][hd] bf16
  uint64_t* ex;              // exchange words
  const float2* rope;        // [max_seq][hd/2] (cos, sin)
  const int64_t* wbase;      // [nwg * 8 + 1] first tile of each wave's stream (and the total)
  uint32_t* err;             // device error word
  uint64_t* trace;           // [nwg][8 waves][16] cycle counters (written by KIE_TRACE builds only)
  const int32_t* first_tok;  // [1]
  const int32_t* forced;     // [n_steps-1] or null
  int32_t* tokens_out;       // [n_steps] or null
  int32_t* last_tok_out;     // [1] or null
  int32_t* tok_ring;         // host ring [1 + ring_cap] (count, then tokens) or null
  int32_t ring_cap;
  int64_t ring_base;         // tokens streamed to the ring before this launch
  float* logits_out;         // [n_steps][V], or [V] when lm_last_only, or null
  int32_t pos0, n_steps;
  uint32_t epoch0;           // exchange tag of step s is epoch0 + s (never 0)
  int32_t lm_last_only;      // run the LM head and sampler only on the last step (prompt pass)
  int32_t top_k;             // <= 1: greedy; else top-k sampling (k <= kMaxTopK)
  float temperature;         // top-k: logits are divided by it (> 0)
  uint64_t seed;             // top-k: random stream of the draw
  int64_t timeout_ticks;     // per wait, in s_memrealtime ticks (100 MHz)
  const int32_t* abort_word; // device view of the caller's pinned host abort word, or null
  uint32_t skew;             // > 0: each WG idles a pseudo-random 0..skew-1 x ~3.4 us before
                             // every stage boundary (protocol stress; results must not change)
  uint32_t xb_lds;           // byte offset of the extra-batch LDS slots in the dynamic LDS
                             // (lds_slot_offset; used where the slot is read in assembly)
  const float* wscale;       // 8-bit weights: [L][7] + [1] matrix scales (wq, wk, wv, wo, w_gate,
                             // w_up, w_down; then the LM head), else null
};

typedef void (*KernelFn)(KParams);
KernelFn decode_kernel_for(int group, int head_dim, bool prompt, bool moe, bool w8);
int32_t lds_bytes_for(const Shape& s);
int32_t lds_slot_offset(const Shape& s);  // where the extra-batch slots start in the dynamic LDS
int32_t topk_capacity_floats(const Shape& s);  // WG-local floats available to the top-k merge

// set-up kernels (pack.hip)
struct PackArgs {
  Shape s;
  uint8_t* packed;
  const int64_t* wbase;  // device [nwg * 8]
  int32_t layer;         // 0..L-1, or L for the LM head
  const uint16_t *wq, *wk, *wv, *wo, *wgate, *wup, *wdown;  // layer matrices (layer < L)
  const uint16_t* lm_head;                                   // layer == L
  // mixture of experts (layer < L): router [E][d]; gate, up [E][Fe][d]; down [E][d][Fe]
  const uint16_t *wrouter, *egate, *eup, *edown;
  int64_t expert_offset;  // byte offset of the expert region in the packed image
  int32_t w8;             // the layer matrices are one-byte codes (tiles of 2 * kTileK weights)
};
hipError_t launch_pack_layer(const PackArgs& a, hipStream_t st);
hipError_t launch_pack_experts(const PackArgs& a, hipStream_t st);
hipError_t launch_rope_table(float2* rope, int32_t max_seq, int32_t hd, float theta, hipStream_t st);
hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t st);
hipError_t launch_stream_bases(const Shape& s, bool w8, int64_t* wbase, hipStream_t st);
hipError_t launch_ptab(const Shape& s, bool w8, const int64_t* wbase, int32_t* tab, hipStream_t st);
constexpr int32_t kFloatChunk = 256;
struct FloatChunk {
  float* dst;
  int32_t n;
  float v[kFloatChunk];
};
hipError_t launch_set_floats(float* dst, const float* src, int32_t n, hipStream_t st);

}  // namespace kie
