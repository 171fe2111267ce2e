// prefill.h -- the prompt pass on the matrix cores (prefill.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace kie {

// Buffers and tables of one prompt pass. The scratch buffers live in the workspace and hold one
// chunk of at most kPrefillChunk positions.
struct PrefillArgs {
  Shape s;
  const uint8_t* packed;     // packed weight image
  const int64_t* wbase;      // [nwg * 8 + 1] first tile of each stream
  const uint16_t* embed;     // [V][d] bf16
  const uint16_t* norms;     // [L][2][d] bf16 gains
  const float2* rope;        // [max_seq][hd/2] (cos, sin)
  uint16_t* kv;              // cache [L][2][nkv][max_seq][hd] bf16
  uint32_t* err;             // device error word
  const int32_t* tokens;     // [n] prompt ids
  float* x;                  // [chunk][d] residual stream
  uint16_t* a3;              // [2][chunk][kmax] GEMM input in two bf16 parts
  int64_t a_part;            // elements between the parts
  uint16_t* h2;              // [2][chunk][F] down-projection input in two bf16 parts
  float* c;                  // [chunk][nmax] split-K partial sums
  float* q;                  // [chunk][nq * hd] rotated queries
  float* attn_part;          // [segments][chunk][nq][hd + 2] partial attention states
  const float* wscale;       // 8-bit weights: the matrix scales [L][7] (+ the LM head's); null for bf16
  const int32_t* ptab;       // first tile of every unit of the streamed stages (ptab_index)
  // mixture of experts (moe_prefill_layout; null for dense models)
  float* rlogits;            // [chunk][E] router logits
  int32_t* sel;              // [chunk][A] chosen experts, rank order
  float* wt;                 // [chunk][A] their routing weights
  int32_t* place;            // [chunk][A] each choice's place in its expert's token list
  int32_t* lists;            // [E][chunk] position << 4 | rank, in position order
  int32_t* counts;           // [E] list lengths
  int32_t* offs;             // [E] first row of each expert's rows in ey (and in h2)
  float* ey;                 // [chunk * A][d] the experts' down-projection rows
};

// What the GEMM does with its result C[i][n]:
enum GemmEpilogue : int32_t {
  EPI_STORE = 0,   // out[i][n] = (or +=) C
  EPI_ROPE_KV = 1, // QKV: RoPE on each (A, B) pair of a query or key head; queries to q (fp32),
                   // keys and values to the cache rows of positions p0 + i (bf16)
  EPI_SWIGLU = 2,  // gate/up: h = silu(gate) * up into the two-part down-projection input h2
};

struct GemmStage {
  int32_t st, layer, K, N;
  const uint16_t* in;    // [2][chunk][K] two-part input
  int64_t in_part;       // elements between its parts
  int32_t epi, p0;       // GemmEpilogue; position of row 0 (EPI_ROPE_KV)
  float* out;
  int32_t ldo, accumulate;
  int32_t splits, kper;  // K is cut into `splits` shares of kper each
  float* part;           // [splits][chunk][N] partial sums when splits > 1
};

// Run every layer over positions p0 .. p0 + n - 1 (writes their K/V rows).
hipError_t launch_prefill(const PrefillArgs& a, int32_t p0, int32_t n, hipStream_t stream);
// Whether launch_prefill handles the shape: a mixture of experts needs whole output tiles and K
// chunks in its experts' products (d and the expert width multiples of 128) and at most 15 experts
// routed per position.
bool prefill_supports(const Shape& s);

}  // namespace kie
