// monokernel_impl.h -- the persistent batch-1 decode kernel for MI355X (gfx950): device code.
// Included by the translation units that instantiate the kernels (kernels_hd64.hip,
// kernels_hd128.hip), which the build compiles in parallel.
//
// One launch decodes n tokens; control never returns to the host in between (agentlenshq.com,
// 《突破内存墙：在标准 GPU 上实现 3,000 tokens/s 的推理速度》, "The Monokernel Runtime"; aikraft.ru
// «3000 токенов в секунду…», §04 "Моноядро": one resident GPU program covering MatMul,
// attention, normalisation and sampling, with tight control of synchronisation, prefetch and
// execution order). The design below is this library's own for CDNA4; the pages only say that
// such kernels exist.
//
// Grid: one 512-thread workgroup (WG) per compute unit, all co-resident (cooperative launch).
// Every one of the 8 waves streams its own contiguous slice of the packed weights from HBM into
// registers with 16-byte-per-lane buffer loads, one batch of 8 KiB ahead of the batch it is
// reducing. That batch is issued before the wave waits for the inputs of the next stage, so the
// weight stream keeps flowing across every synchronisation point (the prefetch across
// synchronisation points the pages call for); 64 KiB in flight per CU keep the HBM pipe busy.
// Where LDS has room, the batch after that one also streams in across the O, gate/up and down
// boundaries, straight into an 8 KiB LDS slot per wave (Wk::issue_x), with no registers held.
// GEMV arithmetic: a lane holds 4 bf16 weights of each of two rows at the same k, so one 16-byte
// LDS read of the fp32 stage input feeds 8 weights of two rows; the weights are widened to fp32
// and accumulated with fp32 FMA (the unit has VALU to spare at the streaming rate).
// Inter-WG exchange uses 64-bit tagged words (fp32 value << 32 | epoch) written and read with
// agent-scope atomics, so a reader knows a word is current by its tag alone: no grid barrier, no
// flag round trip, no cache flush. Epochs are unique per decode step and buffers are per layer.
// Inside a WG the waves meet at the hardware barrier with LDS-only fences, which never wait for
// the weight loads in flight.
//
// Per layer: RMSNorm -> QKV (+RoPE) -> attention over a chunk of positions of one KV head
// (split-K; online softmax per wave, waves merged in LDS) -> merge of the chunk partials ->
// O (+residual) -> RMSNorm -> gate/up (SwiGLU) -> down (+residual). Then the final RMSNorm, the
// LM head and the sampler. A mixture-of-experts layer runs the router after the second RMSNorm;
// every WG chooses the same experts from the gathered router logits, and gate/up and down then
// stream only the chosen experts' tiles (the pages' point that bandwidth follows the active
// parameters: aikraft.ru «3000 токенов в секунду…», §02).
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.h"
#include "layout.h"
#include "monokernel.h"

namespace kie {

// The kernels' dynamic LDS (the layout of lds_map).
extern __shared__ __align__(16) uint8_t kie_smem[];

// Optional per-wave cycle counters (compile with -DKIE_TRACE); free in normal builds.
#ifdef KIE_TRACE
#define TR_NOW() __builtin_readcyclecounter()
#else
#define TR_NOW() 0ull
#endif
// Hop timeline of a KIE_TRACE or KIE_TRACE_HOPS build (the latter without the cycle counters): wave 0 of every WG stores the absolute time (s_memrealtime,
// 100 MHz, one clock for the whole chip) of each boundary event of one sampled (step, layer)
// into trace words kTraceHop + event, so that publication spreads and per-XCD gather latencies
// can be read off afterwards. Free in normal builds.
constexpr int kHopStep = 8, kHopLayer = 12;
enum HopEvent : int {
  H_QKV_IN = 0, H_QKV_PUB = 1, H_ATT_IN = 2, H_ATT_PUB = 3, H_MERGE_PUB = 4, H_O_GOT = 5, H_O_IN = 6,
  H_XA_PUB = 7, H_XA_GOT = 8, H_GU_IN = 9, H_H_PUB = 10, H_H_GOT = 11, H_DN_IN = 12, H_XF_PUB = 13,
  H_XF_GOT = 14, H_NORM_DONE = 15, H_ATT_ALLQ = 16, H_ATT_DONE = 17, H_ATT_COMB = 18
};
// GEMV batches of the sampled layer: 2 b = batch b taken, 2 b + 1 = reduced (wave 0's batches;
// at most 16), stored after the events.
// The stamps go to a small LDS area (kHopWords words) and are copied to the trace words of waves 0
// (events) and 1 (batches) when the kernel ends, so that taking them adds no vector-memory
// operation that the kernel's own waits would have to drain.
#if defined(KIE_TRACE) || defined(KIE_TRACE_HOPS)
constexpr int kHopWords = 64;
#define TR_HOP(K, ev)                                                                                     \
  do {                                                                                                    \
    if ((K).hop_on && (K).v == 0) /* wave-uniform: every lane stores the same time */                      \
      *(volatile uint64_t*)((K).L.hopt + (ev)) = now_ticks();                                             \
  } while (0)
#define TR_BATCH(K, ev)                                                                                   \
  do {                                                                                                    \
    if ((K).v == 0 && (ev) < 32) *(volatile uint64_t*)((K).L.hopt + 32 + (ev)) = now_ticks();            \
  } while (0)
#else
constexpr int kHopWords = 0;
#define TR_HOP(K, ev) \
  do {                \
  } while (0)
#define TR_BATCH(K, ev) \
  do {                  \
  } while (0)
#endif
enum TraceSlot : int {
  T_FETCH = 0, T_GEMV = 1, T_FIN = 2, T_ATT = 3, T_MERGE = 4, T_BAR = 5, T_TOTAL = 6, T_BATCHES = 7,
  T_NORM = 8, T_SAMPLE = 9
};
struct Tracer {
#ifdef KIE_TRACE
  uint64_t c[kTraceWords];
  __device__ __forceinline__ Tracer() {
    for (int i = 0; i < kTraceWords; ++i) c[i] = 0;
  }
  __device__ __forceinline__ void add(int k, uint64_t v) { c[k] += v; }
  __device__ __forceinline__ void flush(uint64_t* dst, int lane) {
    if (lane == 0)
      for (int i = 0; i < kTraceWords; ++i) dst[i] = c[i];
  }
#else
  __device__ __forceinline__ void add(int, uint64_t) {}
  __device__ __forceinline__ void flush(uint64_t*, int) {}
#endif
};

// ------------------------------------------------------------------------------------------
// LDS layout
// ------------------------------------------------------------------------------------------
struct Lds {
  float* act;      // GEMV input of the current stage (fp32)
  float* xres;     // residual stream, two buffers of d floats (the current one alternates)
  float* part;     // [kMaxUnits][2] per-unit dot products of the current stage
  float* scr;      // attention / merge / reduction scratch
  float* q;        // attention: the group's queries [G][hd], the current k [hd] and v [hd]
  float2* rope;    // (cos, sin) of the current position, hd/2 entries
  uint32_t* ctl;   // control words
  int32_t* moe;    // mixture of experts: the layer's chosen experts [kMaxActive], then their
                   // routing weights [kMaxActive] (fp32 bits)
  uint8_t* xb;     // one extra weight batch per wave (kBatch tiles), or null where LDS is short
  uint64_t* hopt;  // KIE_TRACE / KIE_TRACE_HOPS builds: the hop timeline stamps (kHopWords)
};
enum Ctl : int { C_ABORT = 0, C_COUNT = 4 };

__host__ __device__ inline int32_t act_floats(const Shape& s) {
  int32_t a = s.d;
  if (s.qdim() > a) a = s.qdim();
  if (s.F > a) a = s.F;
  return a;
}
// The LDS layout, for a kernel compiled for GC query heads per KV head (the host's versions below
// take the group from the shape). With 8 query heads per KV head attention runs as two passes of
// 4 heads and its scratch holds one pass.
template <int GC>
__host__ __device__ inline int32_t scr_floats_g(const Shape& s) {
  int32_t a = GC > 4 ? kWaves * 4 * (s.hd + 2) : kWaves * s.group() * (s.hd + 2);
  if (kWaves * kMergeDims * 3 > a) a = kWaves * kMergeDims * 3;
  if (2 * s.nwg > a) a = 2 * s.nwg;
  if (lm_rows_max(s) > a) a = lm_rows_max(s);  // the WG's LM outputs for the top-k draw
  if (s.E > a) a = s.E;                          // router logits
  if (a < 64) a = 64;
  return (a + 3) & ~3;
}
__host__ __device__ inline int32_t scr_floats(const Shape& s) {
  return s.group() > 4 ? scr_floats_g<8>(s) : scr_floats_g<1>(s);
}
// act, xres, part and a pad are contiguous: once the LM outputs are final they hold the top-k
// merge, and the pad makes room for the largest k where the three are smaller
__host__ __device__ inline int32_t merge_pad_floats(const Shape& s) {
  const int32_t kmax = kMaxTopK < s.V ? kMaxTopK : s.V;
  const int32_t need = (topk_merge_floats(s, kmax) + 3) & ~3;
  const int32_t have = act_floats(s) + 2 * s.d + 2 * kMaxUnits;
  return need > have ? need - have : 0;
}
__host__ __device__ inline int32_t merge_floats(const Shape& s) {
  return act_floats(s) + 2 * s.d + 2 * kMaxUnits + merge_pad_floats(s);
}
// The extra batch slots (8 KiB per wave) are placed where the rest leaves room for them.
constexpr int32_t kLdsCapacity = 160 * 1024;
constexpr int32_t kXbBytes = kWaves * kBatch * kTileBytes;
__host__ __device__ inline int32_t moe_words(const Shape& s) { return s.moe() ? 2 * kMaxActive : 0; }
template <int GC>
__host__ __device__ inline int32_t lds_base_bytes_g(const Shape& s) {
  return (merge_floats(s) + scr_floats_g<GC>(s) + (s.group() + 2) * s.hd + s.hd) * 4 + C_COUNT * 4 + moe_words(s) * 4 +
         kHopWords * 8;
}
template <int GC>
__host__ __device__ inline bool xb_fits_g(const Shape& s) { return lds_base_bytes_g<GC>(s) + kXbBytes <= kLdsCapacity; }
__host__ __device__ inline int32_t lds_base_bytes(const Shape& s) {
  return s.group() > 4 ? lds_base_bytes_g<8>(s) : lds_base_bytes_g<1>(s);
}
__host__ __device__ inline bool xb_fits(const Shape& s) { return lds_base_bytes(s) + kXbBytes <= kLdsCapacity; }
inline int32_t lds_bytes_for_impl(const Shape& s) { return lds_base_bytes(s) + (xb_fits(s) ? kXbBytes : 0); }
template <int GC>
__device__ __forceinline__ Lds lds_map(uint8_t* smem, const Shape& s) {
  Lds L;
  uint8_t* p = smem;
  L.act = (float*)p; p += (size_t)act_floats(s) * 4;
  L.xres = (float*)p; p += (size_t)2 * s.d * 4;
  L.part = (float*)p; p += (size_t)2 * kMaxUnits * 4;
  p += (size_t)merge_pad_floats(s) * 4;
  L.scr = (float*)p; p += (size_t)scr_floats_g<GC>(s) * 4;
  L.q = (float*)p; p += (size_t)(s.group() + 2) * s.hd * 4;
  L.rope = (float2*)p; p += (size_t)s.hd * 4;
  L.ctl = (uint32_t*)p;
  p += C_COUNT * 4;  // 16-byte aligned: every piece above is a multiple of 4 floats
  L.moe = (int32_t*)p;
  p += moe_words(s) * 4;
  L.hopt = (uint64_t*)p;  // 16-byte aligned: the pieces above are multiples of 16 bytes
  p += kHopWords * 8;
  L.xb = xb_fits_g<GC>(s) ? p : nullptr;
  return L;
}

// ------------------------------------------------------------------------------------------
// Attention work of this WG at context length n = pos + 1: KV head j over position chunk `chunk`.
// ------------------------------------------------------------------------------------------
struct Att {
  int32_t j, chunk, c0, c1, ncache, nkt, has_p, cs, nch;
};
__device__ __forceinline__ Att att_info(const Shape& s, int32_t w, int32_t pos) {
  Att a;
  const int32_t n = pos + 1;
  a.j = w % s.nkv;
  a.chunk = w / s.nkv;
  a.cs = att_chunk_len(s, n);
  a.nch = (n + a.cs - 1) / a.cs;
  a.c0 = a.chunk * a.cs;
  a.c1 = a.c0 + a.cs < n ? a.c0 + a.cs : n;
  if (a.c0 >= n) {
    a.c1 = a.c0;
    a.ncache = 0;
    a.nkt = 0;
    a.has_p = 0;
  } else {
    const int32_t ce = a.c1 < pos ? a.c1 : pos;  // cached positions end (pos itself is exchanged)
    a.ncache = ce > a.c0 ? ce - a.c0 : 0;
    const int32_t ppt = att_pos_per_tile(s);
    a.nkt = (a.ncache + ppt - 1) / ppt;
    a.has_p = pos < a.c1 ? 1 : 0;
  }
  return a;
}

__device__ __forceinline__ bool step_has_lm(const KParams& P, int32_t step) {
  return !P.lm_last_only || step == P.n_steps - 1;
}

// A token id that indexes memory is always kept inside [0, V).
__device__ __forceinline__ int32_t clamp_token(int32_t t, int32_t V) { return t < 0 ? 0 : (t >= V ? V - 1 : t); }

// ------------------------------------------------------------------------------------------
// Failure handling: every wait is bounded; on expiry the WG records an error and stops.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void raise_error(const KParams& P, const Lds& L, uint32_t code) {
  lds_st(&L.ctl[C_ABORT], 1u);
  __hip_atomic_fetch_or(P.err, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t lds_ld_u(const uint32_t* p) { return __builtin_amdgcn_readfirstlane(lds_ld(p)); }
__device__ __forceinline__ bool aborted(const Lds& L) { return lds_ld_u(&L.ctl[C_ABORT]) != 0; }
__device__ __forceinline__ bool global_error(const KParams& P) {
  return __builtin_amdgcn_readfirstlane(__hip_atomic_load(P.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0;
}

// The caller's abort word (pinned host memory), read at system scope; 0 when there is none.
__device__ __forceinline__ int32_t host_abort(const KParams& P) {
  return P.abort_word ? __hip_atomic_load(P.abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : 0;
}

// Bounded spin: call expired() after every unsuccessful poll. Every 64th call it checks the WG's
// abort flag, the host's abort word and the elapsed time of this wait (wave-uniform); `why` then
// names the error to raise. Poll rounds follow each other without a sleep: each round already
// waits for its own loads, which paces it.
struct Waiter {
  uint32_t spins = 0;
  uint64_t start = 0;
  uint32_t why = KERR_TIMEOUT;
  __device__ __forceinline__ bool expired(const KParams& P, const Lds& L) {
    if ((++spins & 63u) != 0) return false;
    if (aborted(L)) return true;
    if (__builtin_amdgcn_readfirstlane(host_abort(P)) != 0) {
      why = KERR_ABORTED;
      return true;
    }
    const uint64_t t = now_ticks();
    if (start == 0) {
      start = t;
      return false;
    }
    return t - start > (uint64_t)P.timeout_ticks;
  }
};

// Barrier of the WG's 8 waves. The fences order LDS only, so weight loads stay in flight.
__device__ __forceinline__ void bar() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// argmax candidate order: larger value first, then the lower index
__device__ __forceinline__ bool better(float v, int32_t i, float bv, int32_t bi) {
  return v > bv || (v == bv && i < bi);
}

// Candidate (z, id) as one unsigned 64-bit key that orders like the candidate order: an
// order-preserving image of the float bits above, the complement of the id below (a lower id
// wins a tie). z is never NaN or -0 here.
__device__ __forceinline__ uint64_t cand_key(float v, int32_t id) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t hi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)hi << 32) | (uint32_t)(0x7fffffff - id);
}
__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t hi = (uint32_t)(k >> 32);
  return __uint_as_float((hi & 0x80000000u) ? (hi & 0x7fffffffu) : ~hi);
}
__device__ __forceinline__ int32_t key_id(uint64_t k) { return 0x7fffffff - (int32_t)(uint32_t)k; }
// Number of keys of kk[0 .. n) (16-byte aligned) greater than key; eight per step with 16-byte
// LDS reads, so that the reads overlap.
__device__ __forceinline__ int32_t count_greater(const uint64_t* kk, int32_t n, uint64_t key) {
  typedef uint64_t v2u64 __attribute__((ext_vector_type(2)));
  int32_t c = 0, i = 0;
  for (; i + 8 <= n; i += 8) {
    const v2u64 a = *(const v2u64*)(kk + i), b = *(const v2u64*)(kk + i + 2);
    const v2u64 e = *(const v2u64*)(kk + i + 4), f = *(const v2u64*)(kk + i + 6);
    c += (a.x > key ? 1 : 0) + (a.y > key ? 1 : 0) + (b.x > key ? 1 : 0) + (b.y > key ? 1 : 0) + (e.x > key ? 1 : 0) +
         (e.y > key ? 1 : 0) + (f.x > key ? 1 : 0) + (f.y > key ? 1 : 0);
  }
  for (; i < n; ++i) c += kk[i] > key ? 1 : 0;
  return c;
}

// ------------------------------------------------------------------------------------------
// One wave's state: its weight stream, the batch in flight, the WG's stage geometry. MOE: the
// layers are mixture-of-experts layers, whose gate/up and down batches are read from the expert
// region at the chosen experts' tiles (routed batches) instead of from the fixed stream.
// ------------------------------------------------------------------------------------------
template <bool MOE, bool W8 = false>
struct Wk {
  // W8: the layer matrices and the LM head are one-byte e4m3fn codes, 2 * kTileK of a row per tile
  static constexpr int TK = W8 ? 2 * kTileK : kTileK;
  const KParams& P;
  const Lds& L;
  int32_t w, v, lane, tid;
  bool fail;
  Tracer tr;
  StageGeo g[ST_COUNT];
  int32_t nb[ST_COUNT];  // this wave's batches per stage
  int32_t layer_b, lm_b;
  const uint8_t* stream;  // this wave's first tile
  v4u nxt[kBatch];        // the next batch of the stream (loads in flight)
  int32_t pidx, pstep;    // the last batch issued: index in its step's stream, and the step
  // The batch after nxt may also be in flight, loaded straight into this wave's LDS slot: xpend
  // while nxt is still ahead of it, xnext once it is the next to reduce.
  bool xpend = false, xnext = false;
  // MOE. A step's batches are, per layer, layer_b fixed-stream batches and then dyn_b routed ones
  // (gate/up, then down), and finally the LM head's. A routed batch can be issued only once its
  // layer's experts are chosen: until then nxt receives zeros from empty loads (deferred) and the
  // router boundary issues it for real. L.moe holds the experts of layer sel_key (= step * L +
  // layer) and their weights.
  int32_t dyn_b = 0;
  int32_t sel_key = -1;
  bool deferred = false;
  const uint8_t* xreg = nullptr;  // expert region of the packed image
  bool hop_on = false;            // KIE_TRACE: this boundary belongs to the sampled (step, layer)

  __device__ __forceinline__ Wk(const KParams& p, const Lds& l, int32_t w_, int32_t v_, int32_t lane_)
      : P(p), L(l), w(w_), v(v_), lane(lane_), tid(v_ * kWave + lane_), fail(false) {
    layer_b = 0;
    for (int st = 0; st < ST_COUNT; ++st) {
      if (!MOE && st == ST_RT) {  // dense layers have no router: constant zeros
        g[st] = StageGeo{0, 0, 1, 1, 1, kBatch, 0};
        nb[st] = 0;
        continue;
      }
      g[st] = stage_geo<TK>(P.s, st, w);
      nb[st] = wave_batches(g[st], v);
      if (st <= ST_DN && (!MOE || P.s.in_stream(st))) layer_b += nb[st];
    }
    lm_b = nb[ST_LM];
    stream = P.packed + (size_t)P.wbase[w * kWaves + v] * kTileBytes;
    pidx = -1;
    pstep = 0;
    if constexpr (MOE) {
      dyn_b = nb[ST_GU] + nb[ST_DN];
      xreg = P.packed + (size_t)P.wbase[P.s.nwg * kWaves] * kTileBytes;
    }
  }

  // ------------------------------------------------------------ weight stream
  __device__ __forceinline__ int32_t step_batches(int32_t step) const {
    return P.s.L * (layer_b + dyn_b) + (step_has_lm(P, step) ? lm_b : 0);
  }
  // advance (pidx, pstep) to the next batch of the launch; pstep == n_steps once there is none
  __device__ __forceinline__ void advance() {
    ++pidx;
    while (pstep < P.n_steps && pidx >= step_batches(pstep)) {
      pidx = 0;
      ++pstep;
    }
  }
  // MOE: where batch (pidx, pstep) lies. Returns the fixed-stream batch index, or -1 for a routed
  // batch (then *lb is its layer and *jd its index among the layer's routed batches).
  __device__ __forceinline__ int32_t locate(int32_t* lb, int32_t* jd) const {
    const int32_t per = layer_b + dyn_b;
    if (pidx >= P.s.L * per) return P.s.L * layer_b + (pidx - P.s.L * per);  // the LM head
    const int32_t l = pidx / per;
    const int32_t j = pidx - l * per;
    if (j < layer_b) return l * layer_b + j;
    *lb = l;
    *jd = j - layer_b;
    return -1;
  }
  // routing weight of chosen expert `slot` (0 <= slot < A)
  __device__ __forceinline__ float weight_of(int32_t slot) const { return __int_as_float(L.moe[kMaxActive + slot]); }
  // Tile index (in the expert region) of slot (lane mod 8) of routed batch jd of layer lb, or
  // 0xffffffff for a slot of a missing unit. Gate/up pair gp is row gp mod Fe of chosen expert
  // gp / Fe; k-tile t of a down pair lies in chosen expert t / (Fe / 256). Callers read the 8
  // indices lane by lane.
  __device__ __forceinline__ uint32_t routed_index(int32_t lb, int32_t jd) const {
    const Shape& s = P.s;
    const bool gu = jd < nb[ST_GU];
    const StageGeo gs = gu ? g[ST_GU] : g[ST_DN];
    const int32_t bi = gu ? jd : jd - nb[ST_GU];
    int32_t ln = lane;
    asm volatile("" : "+v"(ln));  // formed here, not hoisted (see route)
    const int32_t b = ln & (kBatch - 1);
    const int32_t lks = gs.ks == 8 ? 3 : (gs.ks == 4 ? 2 : (gs.ks == 2 ? 1 : 0));
    const int32_t us = b >> lks, tt = b & (gs.ks - 1);
    const int32_t u = v + kWaves * (bi * gs.upb + us);
    const int32_t lp = gs.S == 1 ? u : u / gs.S, r = u - lp * gs.S;
    const int32_t gp = gs.pb + lp, kt = r * gs.ks + tt;
    const int32_t kte = s.Fe / kTileK;
    // chosen-expert slot of the tile: gp / Fe (gate/up) or kt / kte (down), slot < A <= 8
    const int32_t q = gu ? gp : kt, span = gu ? s.Fe : kte;
    int32_t slot = 0;
#pragma unroll
    for (int i = 1; i < kMaxActive; ++i) slot += q >= i * span ? 1 : 0;
    const bool live = u < gs.nu;
    const int32_t e = live ? L.moe[slot] : 0;
    const int64_t t = gu ? expert_gu_tile(s, lb, e, gp - slot * s.Fe, kt) : expert_dn_tile(s, lb, e, gp, kt - slot * kte);
    return live ? (uint32_t)t : 0xffffffffu;  // the region has fewer than 2^32 - 1 tiles
  }
  // MOE: where the 8 tiles of batch (pidx, pstep) are -- the fixed stream, the expert region
  // (routed), or nowhere (past the launch, or a routed batch whose experts are not chosen yet:
  // deferred). f(b, resource of tile b) for b < 8; an empty resource loads zeros.
  template <typename F>
  __device__ __forceinline__ void batch_tiles(F f) {
    const bool live = pstep < P.n_steps;
    bool stat = false, routed = false;
    size_t off = 0;
    uint32_t t32 = 0xffffffffu;
    deferred = false;
    if (live) {
      int32_t lb = 0, jd = 0;
      const int32_t sidx = locate(&lb, &jd);
      if (sidx >= 0) {
        stat = true;
        off = (size_t)sidx * kBatch * kTileBytes;
      } else if (sel_key == pstep * P.s.L + lb) {
        routed = true;
        t32 = routed_index(lb, jd);
      } else {
        deferred = true;
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const uint32_t ti = routed ? __builtin_amdgcn_readlane(t32, b) : 0xffffffffu;
      const bool okr = ti != 0xffffffffu;
      const uint8_t* base = okr ? xreg + (size_t)ti * kTileBytes : stream + off + (size_t)b * kTileBytes;
      f(b, make_rsrc(base, (okr || stat) ? kTileBytes : 0));
    }
  }
  // Bytes of batch idx of a step's stream that hold weights. A wave's last batch of a stage can end
  // in zero tiles (fewer units left than a batch holds); W8 streams do not read those (loads past
  // the resource's end return zeros without touching memory), since at 8 bits the QKV and O
  // stages of the 1.6B shape give each wave half a batch. bf16 streams read whole batches.
  __device__ __forceinline__ uint32_t batch_bytes(int32_t idx) const {
    if constexpr (!W8) {
      return kBatch * kTileBytes;
    } else {
      int32_t r = idx, st = ST_LM;
      const int32_t lb = P.s.L * layer_b;
      if (r < lb) {
        r = r % layer_b;
        st = ST_QKV;
        while (st < ST_DN && r >= nb_of(st)) {  // (the router stage of a dense layer has none)
          r -= nb_of(st);
          ++st;
        }
      } else {
        r -= lb;
      }
      const StageGeo gs = geo_of(st);
      const int32_t left = wave_units(gs, v) - r * gs.upb;
      return (uint32_t)((left < gs.upb ? left : gs.upb) * gs.ks * kTileBytes);
    }
  }
  // 8 loads of batch (pidx, pstep); past the launch's last batch the resource is empty and the
  // loads return zeros without touching memory. MOE: a routed batch of a layer whose experts are
  // not chosen yet is left deferred.
  __device__ __forceinline__ void issue(v4u* buf) {
    const bool live = pstep < P.n_steps;
    if constexpr (!MOE) {
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(stream + (live ? (size_t)pidx * kBatch * kTileBytes : 0), live ? batch_bytes(pidx) : 0);
#pragma unroll
      for (int b = 0; b < kBatch; ++b) buf[b] = load16(rs, (uint32_t)(lane * 16 + b * kTileBytes));
    } else {
      // always 8 loads into buf (zeros for a deferred batch), so that every path writes it alike
      batch_tiles([&](int b, __amdgpu_buffer_rsrc_t rs) { buf[b] = load16(rs, (uint32_t)(lane * 16)); });
    }
  }
  // the launch's first batch
  __device__ __forceinline__ void start() {
    advance();
    issue(nxt);
  }
  // hand the next batch of the stream to the caller and keep the one after it in flight
  __device__ __forceinline__ void take(v4u* cur) {
    if (xnext) {
      // The batch in the LDS slot. At least nxt's kBatch loads were issued after its loads, and
      // the counter drains in issue order, so with at most kBatch operations outstanding the slot
      // is filled.
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kBatch) : "memory");
      if constexpr (MOE) {
        // The lane's slot address is formed inside the block from the lane id and the wave's
        // slot base (the kernel-argument offset of the slots, a scalar), so that no long-lived
        // register holds it: where registers are short it would be spilled, and reloading it from
        // scratch memory would wait behind the weight loads in flight. The reads complete inside
        // the block.
        const uint32_t sb = lds_addr(kie_smem) + P.xb_lds + (uint32_t)v * (kBatch * kTileBytes);
        uint32_t a;
        asm volatile(
            "v_mbcnt_lo_u32_b32 %8, -1, 0\n"
            "v_mbcnt_hi_u32_b32 %8, -1, %8\n"
            "v_lshl_add_u32 %8, %8, 4, %9\n"
            "ds_read_b128 %0, %8\n"
            "ds_read_b128 %1, %8 offset:1024\n"
            "ds_read_b128 %2, %8 offset:2048\n"
            "ds_read_b128 %3, %8 offset:3072\n"
            "ds_read_b128 %4, %8 offset:4096\n"
            "ds_read_b128 %5, %8 offset:5120\n"
            "ds_read_b128 %6, %8 offset:6144\n"
            "ds_read_b128 %7, %8 offset:7168\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(cur[0]), "=&v"(cur[1]), "=&v"(cur[2]), "=&v"(cur[3]), "=&v"(cur[4]), "=&v"(cur[5]),
              "=&v"(cur[6]), "=&v"(cur[7]), "=&v"(a)
            : "s"(sb)
            : "memory");
      } else {
        const uint8_t* xs = L.xb + (size_t)v * kBatch * kTileBytes + lane * 16;
#pragma unroll
        for (int b = 0; b < kBatch; ++b) cur[b] = *(const v4u*)(xs + b * kTileBytes);
      }
      xnext = false;
      return;
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) cur[b] = nxt[b];
    advance();
    issue(nxt);
    if (xpend) {
      xpend = false;
      xnext = true;
    }
  }
  // Before a wait at a stage boundary: load the batch after nxt into this wave's LDS slot with
  // direct buffer->LDS loads, so that two batches stream in across the wait. The loads are
  // written as assembly so that the compiler, which would otherwise wait for them before every
  // LDS read, adds no waits; take() waits for them itself. They hold no registers.
  __device__ __forceinline__ void issue_x() {
    if (L.xb == nullptr || xpend || xnext) return;
    const uint32_t base = lds_addr(L.xb + (size_t)v * kBatch * kTileBytes);
    if constexpr (MOE) {
      if (deferred) return;  // nxt itself holds no data yet
      const int32_t sp = pidx, ss = pstep;
      advance();
      batch_tiles([&](int b, __amdgpu_buffer_rsrc_t rs) {
        if (!deferred) load16_lds(rs, (uint32_t)(lane * 16), base + b * kTileBytes);
      });
      if (deferred) {  // a routed batch whose experts are not chosen yet: leave it to the stream
        deferred = false;
        pidx = sp;
        pstep = ss;
        return;
      }
      xpend = true;
      return;
    }
    advance();
    const bool live = pstep < P.n_steps;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(stream + (live ? (size_t)pidx * kBatch * kTileBytes : 0), live ? batch_bytes(pidx) : 0);
#pragma unroll
    for (int b = 0; b < kBatch; ++b) load16_lds(rs, (uint32_t)(lane * 16 + b * kTileBytes), base + b * kTileBytes);
    xpend = true;
  }

  // MOE, at the router boundary of layer l: router logits (all E) are in scr. Every WG takes the
  // same decision: the A largest logits (ties to the lower index; NaN ranks lowest) and weights
  // w_i = exp(z_i - z_0) / sum_j exp(z_j - z_0) over the chosen, z_0 the largest -- the softmax
  // over all experts restricted to the chosen and renormalised -- into L.moe. Then the deferred
  // batch, if any, is issued.
  __device__ __forceinline__ void route(int32_t step, int32_t l) {
    const Shape& s = P.s;
    // The thread index is made opaque here, so that the LDS addresses below are formed where
    // they are used: hoisted to the kernel start they would live across the whole decode loop,
    // be spilled, and each reload from scratch memory would wait for every load in flight.
    int32_t t = tid;
    asm volatile("" : "+v"(t));
    // part is free between the router stage's finalize and gate/up: the E candidate keys (the
    // argmax order as one 64-bit integer; NaN ranks as -inf and -0 as +0), then the chosen ids
    uint64_t* keys = (uint64_t*)L.part;
    int32_t* sel = (int32_t*)(keys + s.E);
    const uint64_t trk = TR_NOW();
    uint64_t key = 0;
    if (t < s.E) {
      float z = L.scr[t];
      z = z == z ? (z == 0.f ? 0.f : z) : -INFINITY;
      key = cand_key(z, t);
      keys[t] = key;
    }
    bar();
    if (4 * s.E <= kThreads) {
      // four lanes per candidate (a quad), each counting a quarter of the keys; the quad's sum is
      // the rank. The quarters start at even indices, so the 16-byte key reads stay aligned.
      const int32_t c = t >> 2, q = t & 3;
      const int32_t chunk = ((s.E + 7) / 8) * 2;
      const int32_t b0 = q * chunk < s.E ? q * chunk : s.E, b1 = b0 + chunk < s.E ? b0 + chunk : s.E;
      uint64_t ck = 0;
      if (c < s.E) {
        float z = L.scr[c];
        z = z == z ? (z == 0.f ? 0.f : z) : -INFINITY;
        ck = cand_key(z, c);
      }
      int32_t part = c < s.E ? count_greater(keys + b0, b1 - b0, ck) : 0;
      part += __builtin_amdgcn_update_dpp(0, part, kDppQuad1032, 0xF, 0xF, false);
      part += __builtin_amdgcn_update_dpp(0, part, kDppQuad2301, 0xF, 0xF, false);
      if (c < s.E && q == 0 && part < s.A) sel[part] = c;
    } else if (t < s.E) {
      const int32_t rank = count_greater(keys, s.E, key);
      if (rank < s.A) sel[rank] = t;
    }
    uint64_t tq = TR_NOW();
    tr.add(31, tq - trk);
    bar();
    tr.add(19, TR_NOW() - tq);
    tq = TR_NOW();
    if (v == 0) {  // one wave turns the ranks into the table of chosen experts and weights
      const int32_t r = t;
      int32_t e = r < s.A ? sel[r] : 0;
      e = e < 0 ? 0 : (e >= s.E ? s.E - 1 : e);
      float z = L.scr[e];
      z = z == z ? z : -INFINITY;
      const float z0 = readlane_f(z, 0);
      const float x = r < s.A ? expf(z - z0) : 0.f;
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxActive; ++i) sum += readlane_f(x, i);  // in rank order
      if (r < kMaxActive) {
        L.moe[r] = e;
        L.moe[kMaxActive + r] = __float_as_int(x / sum);
      }
    }
    bar();  // the table is complete, and sel and scr are read before the gate/up stage writes part
    tr.add(20, TR_NOW() - tq);
    tq = TR_NOW();
    sel_key = step * s.L + l;
    // The first routed batch could not be prefetched: start it now. (Also starting the next one
    // into the LDS slot here measured slower: 346 against 352 tok/s at the 128-expert shape.)
    if (deferred) issue(nxt);
    tr.add(21, TR_NOW() - tq);
  }

  // ------------------------------------------------------------ GEMV of one stage
  // Stage fields selected through a switch, so that the arrays stay in scalar registers.
  __device__ __forceinline__ StageGeo geo_of(int st) const {
    switch (st) {
      case ST_QKV: return g[ST_QKV];
      case ST_O: return g[ST_O];
      case ST_RT: return g[ST_RT];
      case ST_GU: return g[ST_GU];
      case ST_DN: return g[ST_DN];
      default: return g[ST_LM];
    }
  }
  __device__ __forceinline__ int32_t nb_of(int st) const {
    switch (st) {
      case ST_QKV: return nb[ST_QKV];
      case ST_O: return nb[ST_O];
      case ST_RT: return nb[ST_RT];
      case ST_GU: return nb[ST_GU];
      case ST_DN: return nb[ST_DN];
      default: return nb[ST_LM];
    }
  }
  // Batch b of this wave in stage gs (units of KS tiles), against the input in LDS: the two dot
  // products of each unit u land in part[2u] and part[2u + 1]. The unit's k-slice (u mod S) is
  // computed once per unit; every branch inside is wave-uniform.
  template <int KS>
  __device__ __forceinline__ void reduce_batch_ks(const StageGeo& gs, int32_t b, const v4u* cur) {
    constexpr int UPB = kBatch / KS;
#pragma unroll
    for (int us = 0; us < UPB; ++us) {
      const int32_t u = v + kWaves * (b * UPB + us);
      if (u < gs.nu) {
        const int32_t r = gs.S == 1 ? 0 : u % gs.S;
        const float* xa = L.act + (size_t)r * KS * TK + lane * 4;
        float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
        if constexpr (W8) {
          // lane's 16 B: row A's codes at k = 4 lane .. +3 and 256 + 4 lane .. +3 of the tile's 512,
          // then row B's at the same k; each code widens exactly to fp32
#pragma unroll
          for (int t = 0; t < KS; ++t) {
            const v4f x0 = *(const v4f*)(xa + t * TK);
            const v4f x1 = *(const v4f*)(xa + t * TK + kTileK);
            const v4u wt = cur[us * KS + t];
            v2f p = __builtin_amdgcn_cvt_pk_f32_fp8((int)wt.x, false);
            a0 = fmaf(p.x, x0.x, a0);
            a1 = fmaf(p.y, x0.y, a1);
            p = __builtin_amdgcn_cvt_pk_f32_fp8((int)wt.x, true);
            a0 = fmaf(p.x, x0.z, a0);
            a1 = fmaf(p.y, x0.w, a1);
            p = __builtin_amdgcn_cvt_pk_f32_fp8((int)wt.y, false);
            a0 = fmaf(p.x, x1.x, a0);
            a1 = fmaf(p.y, x1.y, a1);
            p = __builtin_amdgcn_cvt_pk_f32_fp8((int)wt.y, true);
            a0 = fmaf(p.x, x1.z, a0);
            a1 = fmaf(p.y, x1.w, a1);
            p = __builtin_amdgcn_cvt_pk_f32_fp8((int)wt.z, false);
            b0 = fmaf(p.x, x0.x, b0);
            b1 = fmaf(p.y, x0.y, b1);
            p = __builtin_amdgcn_cvt_pk_f32_fp8((int)wt.z, true);
            b0 = fmaf(p.x, x0.z, b0);
            b1 = fmaf(p.y, x0.w, b1);
            p = __builtin_amdgcn_cvt_pk_f32_fp8((int)wt.w, false);
            b0 = fmaf(p.x, x1.x, b0);
            b1 = fmaf(p.y, x1.y, b1);
            p = __builtin_amdgcn_cvt_pk_f32_fp8((int)wt.w, true);
            b0 = fmaf(p.x, x1.z, b0);
            b1 = fmaf(p.y, x1.w, b1);
          }
        } else {
        // the unit's activations are read from LDS before its products (the schedule barrier keeps
        // the KS reads together), so that their latency is paid once per unit: read tile by tile,
        // each read was waited for on its own before the tile's products
        v4f xs[KS];
#pragma unroll
        for (int t = 0; t < KS; ++t) xs[t] = *(const v4f*)(xa + t * kTileK);
        __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);
#pragma unroll
        for (int t = 0; t < KS; ++t) {
          const v4f x = xs[t];
          const v4u wt = cur[us * KS + t];
          a0 = fmaf(bf16lo(wt.x), x.x, a0);
          a1 = fmaf(bf16hi(wt.x), x.y, a1);
          a0 = fmaf(bf16lo(wt.y), x.z, a0);
          a1 = fmaf(bf16hi(wt.y), x.w, a1);
          b0 = fmaf(bf16lo(wt.z), x.x, b0);
          b1 = fmaf(bf16hi(wt.z), x.y, b1);
          b0 = fmaf(bf16lo(wt.w), x.z, b0);
          b1 = fmaf(bf16hi(wt.w), x.w, b1);
        }
        }
        const float ya = wave_sum(a0 + a1), yb = wave_sum(b0 + b1);
        if (lane == 0) {
          L.part[2 * u] = ya;
          L.part[2 * u + 1] = yb;
        }
      }
    }
  }
  __device__ __forceinline__ void reduce_batch(const StageGeo& gs, int32_t b, const v4u* cur) {
    switch (gs.ks) {
      case 8: reduce_batch_ks<8>(gs, b, cur); break;
      case 4: reduce_batch_ks<4>(gs, b, cur); break;
      case 2: reduce_batch_ks<2>(gs, b, cur); break;
      default: reduce_batch_ks<1>(gs, b, cur); break;
    }
  }
  // After the stage's barrier: pair lp's outputs (the sum of its S units in a fixed order) go to
  // fin(global pair, ya, yb).
  template <int ST, typename Fin>
  __device__ __forceinline__ void finalize(Fin fin) {
    const StageGeo& gs = g[ST];
    const uint64_t t0 = TR_NOW();
    for (int32_t lp = tid; lp < gs.np; lp += kThreads) {
      float ya = 0.f, yb = 0.f;
      if (gs.S == 2) {  // the pair's two units in one 16-byte read, added in the same order
        const v4f q = *(const v4f*)(L.part + 4 * lp);
        ya = (ya + q.x) + q.z;
        yb = (yb + q.y) + q.w;
      } else {
        for (int32_t k = 0; k < gs.S; ++k) {
          ya += L.part[2 * (lp * gs.S + k)];
          yb += L.part[2 * (lp * gs.S + k) + 1];
        }
      }
      fin(stage_pair(P.s, ST, gs.pb + lp), ya, yb);
    }
    tr.add(T_FIN, TR_NOW() - t0);
  }

  // ------------------------------------------------------------ reductions
  // sum over the WG's 512 threads in a fixed order; every thread gets the result
  __device__ __forceinline__ float block_sum(float x) {
    const float s = wave_sum(x);
    if (lane == 0) L.scr[v] = s;
    bar();
    // the 8 wave sums in two 16-byte reads, then added in wave order
    static_assert(kWaves == 8, "two 16-byte reads hold the wave sums");
    const v4f lo = *(const v4f*)L.scr, hi = *(const v4f*)(L.scr + 4);
    const float t = (((((((0.f + lo.x) + lo.y) + lo.z) + lo.w) + hi.x) + hi.y) + hi.z) + hi.w;
    bar();
    return t;
  }

  // ------------------------------------------------------------ exchange gathers
  // Poll the tagged words addr(k) of this thread's slots k < KM with valid(k) until each carries
  // `epoch`; got(k, value) receives every value once. All waves of the WG call it; the wait is
  // bounded. k is a compile-time index after unrolling, so per-slot values stay in registers.
  template <int KM, typename Valid, typename Addr, typename Got>
  __device__ __forceinline__ void poll(uint32_t epoch, Valid valid, Addr addr, Got got) {
    uint32_t missing = 0;
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (valid(k)) missing |= 1u << k;
    uint64_t wv[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (missing & (1u << k)) wv[k] = ld_x(addr(k));
    Waiter wt;
    while (true) {
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        if ((missing & (1u << k)) && (uint32_t)wv[k] == epoch) {
          missing &= ~(1u << k);
          got(k, __uint_as_float((uint32_t)(wv[k] >> 32)));
        }
      }
      if (__builtin_amdgcn_ballot_w64(missing != 0) == 0 || fail) break;
      if (wt.expired(P, L) || ((wt.spins & 63u) == 0 && global_error(P))) {
        fail = true;
        raise_error(P, L, wt.why);
        break;
      }
#pragma unroll
      for (int k = 0; k < KM; ++k)
        if (missing & (1u << k)) wv[k] = ld_x(addr(k));
    }
  }
  // n words into LDS floats dst; returns their sum of squares (fixed order) if want_ss.
  // Ends with a barrier: dst is complete for every wave.
  template <int KM = 8>
  __device__ __forceinline__ float fetch_f32(const uint64_t* src, int32_t n, float* dst, uint32_t epoch,
                                             bool want_ss) {
    const uint64_t t0 = TR_NOW();
    for (int32_t base = 0; base < n; base += KM * kThreads) {
      const int32_t e0 = base + tid;
      poll<KM>(
          epoch, [&](int k) { return e0 + k * kThreads < n; }, [&](int k) { return src + e0 + k * kThreads; },
          [&](int k, float x) { dst[e0 + k * kThreads] = x; });
    }
    tr.add(T_FETCH, TR_NOW() - t0);
    float ss = 0.f;
    if (want_ss) {
      for (int32_t e = tid; e < n; e += kThreads) ss = fmaf(dst[e], dst[e], ss);  // this thread's own words
      ss = block_sum(ss);
    } else {
      bar();
    }
    return ss;
  }
  // n words at addresses addr(q), q < n, into LDS floats dst (bit copies). Ends with a barrier.
  template <int KM, typename Addr>
  __device__ __forceinline__ void fetch_map(int32_t n, Addr addr, float* dst, uint32_t epoch) {
    const uint64_t t0 = TR_NOW();
    for (int32_t base = 0; base < n; base += KM * kThreads) {
      const int32_t e0 = base + tid;
      poll<KM>(
          epoch, [&](int k) { return e0 + k * kThreads < n; }, [&](int k) { return addr(e0 + k * kThreads); },
          [&](int k, float x) { dst[e0 + k * kThreads] = x; });
    }
    tr.add(T_FETCH, TR_NOW() - t0);
    bar();
  }
  // The gains of the next RMSNorm, loaded before the wait for its input so that their latency
  // overlaps the wait (the first kNormPre groups of 4 of this thread; the rest load on use).
  static constexpr int kNormPre = 2;
  uint2 gpre[kNormPre];
  const uint16_t* gnext;
  __device__ __forceinline__ void prefetch_gain(const uint16_t* gain) {
    gnext = gain;
#pragma unroll
    for (int k = 0; k < kNormPre; ++k) {
      const int32_t rec = tid + k * kThreads;
      gpre[k] = rec < P.s.d / 4 ? *(const uint2*)(gain + 4 * rec) : uint2{0u, 0u};
    }
  }
  // act = (x * r) * g with r = 1 / sqrt(ss / d + eps), x the residual buffer xs and g the gains
  // of the last prefetch_gain. Ends with a barrier.
  __device__ __forceinline__ void norm_to_act(float ss, const float* xs) {
    const uint64_t t0 = TR_NOW();
    const int32_t d = P.s.d;
    const float r = 1.0f / sqrtf(ss / (float)d + P.s.eps);
#pragma unroll
    for (int k = 0; k < kNormPre; ++k) {
      const int32_t rec = tid + k * kThreads;
      if (rec < d / 4) {
        const v4f x = *(const v4f*)(xs + 4 * rec);
        const uint2 gg = gpre[k];
        *(v4f*)(L.act + 4 * rec) = v4f{(x.x * r) * bf16lo(gg.x), (x.y * r) * bf16hi(gg.x), (x.z * r) * bf16lo(gg.y),
                                       (x.w * r) * bf16hi(gg.y)};
      }
    }
    for (int32_t rec = tid + kNormPre * kThreads; rec < d / 4; rec += kThreads) {
      const v4f x = *(const v4f*)(xs + 4 * rec);
      const uint2 gg = *(const uint2*)(gnext + 4 * rec);
      *(v4f*)(L.act + 4 * rec) = v4f{(x.x * r) * bf16lo(gg.x), (x.y * r) * bf16hi(gg.x), (x.z * r) * bf16lo(gg.y),
                                     (x.w * r) * bf16hi(gg.y)};
    }
    tr.add(T_NORM, TR_NOW() - t0);
    bar();
  }

  // argmax over the WG's threads (each holds a candidate); every thread gets the winner
  __device__ __forceinline__ void block_argmax(float* bv, int32_t* bi) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(*bv, o, kWave);
      const int32_t oi = __shfl_xor(*bi, o, kWave);
      if (better(ov, oi, *bv, *bi)) {
        *bv = ov;
        *bi = oi;
      }
    }
    if (lane == 0) {
      L.scr[2 * v] = *bv;
      L.scr[2 * v + 1] = __int_as_float(*bi);
    }
    bar();
    float bv2 = L.scr[0];
    int32_t bi2 = __float_as_int(L.scr[1]);
    for (int k = 1; k < kWaves; ++k) {
      const float ov = L.scr[2 * k];
      const int32_t oi = __float_as_int(L.scr[2 * k + 1]);
      if (better(ov, oi, bv2, bi2)) {
        bv2 = ov;
        bi2 = oi;
      }
    }
    bar();
    *bv = bv2;
    *bi = bi2;
  }
};

// ------------------------------------------------------------------------------------------
// Attention for KV head j over this WG's chunk of positions. Wave v takes the chunk's K/V tiles
// v, v + 8, ...; each lane keeps an online softmax (exp2 domain) over the positions it sees, the
// position rows of a wave are combined with shuffles and the 8 waves in LDS; one partial
// (acc[hd], m, l) per query head of the group is published, m being the chunk maximum.
// ------------------------------------------------------------------------------------------
template <int G, int HD, typename WK>
__device__ __forceinline__ void attention(WK& K, const Att& at, int32_t l, int32_t pos, uint32_t ep) {
  const KParams& P = K.P;
  const Lds& L = K.L;
  const Shape& s = P.s;
  const Exch& X = P.exo;
  constexpr int LPP = HD / 8;    // lanes per position
  constexpr int PPT = 64 / LPP;  // positions per tile
  constexpr int AB = 2;  // K (and V) tiles per batch
  const int lane = K.lane, v = K.v;
  const int lpos = lane / LPP, dg = lane % LPP;
  const int32_t ntw = at.nkt > v ? (at.nkt - v + kWaves - 1) / kWaves : 0;  // this wave's tiles
  const int32_t nbw = (ntw + AB - 1) / AB;
  const uint32_t kvbytes = (uint32_t)at.ncache * HD * 2;  // lanes past the cached rows read zeros
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(P.kv + kv_offset(s, l, 0, at.j, at.c0), kvbytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(P.kv + kv_offset(s, l, 1, at.j, at.c0), kvbytes);
  // Batch bi's K and V tiles, always 2 AB loads: a tile past this wave's last lies wholly past the
  // resources' end (tile t >= nkt starts at or past ncache rows), so its loads read zeros without
  // touching memory. With no branch around them, every path of the batch loop below issues the
  // same loads, and the wait before a batch is used need not cover the batch issued after it.
  auto kv_issue = [&](int32_t bi, v4u* kb, v4u* vb) {
#pragma unroll
    for (int e = 0; e < AB; ++e) {
      const uint32_t off = (uint32_t)((v + kWaves * (bi * AB + e)) * kTileBytes + lane * 16);
      kb[e] = load16(krs, off);
      vb[e] = load16(vrs, off);
    }
  };
  v4u kn[AB], vn[AB];
  if (nbw > 0) kv_issue(0, kn, vn);  // cached rows do not depend on this step: load before the inputs

  // inputs: the group's queries, then the current position's k and v when it lies in this chunk
  {
    const uint64_t t0 = TR_NOW();
    const uint64_t* qsrc = P.ex + X.q + (int64_t)l * s.qdim() + (int64_t)at.j * G * HD;
    const uint64_t* ksrc = P.ex + X.k + (int64_t)l * s.kvdim() + at.j * HD;
    const uint64_t* vsrc = P.ex + X.v + (int64_t)l * s.kvdim() + at.j * HD;
    const int32_t n = G * HD + (at.has_p ? 2 * HD : 0);
    constexpr int KM = ((G + 2) * HD + kThreads - 1) / kThreads;
    K.template poll<KM>(
        ep, [&](int k) { return K.tid + k * kThreads < n; },
        [&](int k) {
          const int32_t e = K.tid + k * kThreads;
          return e < G * HD ? qsrc + e : (e < (G + 1) * HD ? ksrc + (e - G * HD) : vsrc + (e - (G + 1) * HD));
        },
        [&](int k, float x) { L.q[K.tid + k * kThreads] = x; });
    K.tr.add(T_FETCH, TR_NOW() - t0);
    TR_HOP(K, H_ATT_IN);
    bar();
    TR_HOP(K, H_ATT_ALLQ);
  }
  const uint64_t ta = TR_NOW();
  const float scale = 1.4426950408889634f / sqrtf((float)HD);  // softmax in the exp2 domain
  // With 4 or more query heads per KV head the queries are read from LDS at each use: held in
  // registers next to the accumulators and the weight batch in flight they would spill, and a
  // spill reload waits behind that batch's loads.
  if constexpr (G > 4) {
    // Two passes of 4 query heads over the chunk's K/V tiles (the second pass loads them again,
    // from L2): the accumulators of 8 heads at once would not fit next to the weight batch in
    // flight without spilling.
    constexpr int GP = 4;
    // each pass's heads are combined over the 8 waves and published before the next pass, so
    // the scratch holds one pass (which leaves LDS room for the extra weight-batch slot)
    float* ws = L.scr + v * GP * (HD + 2);
    uint64_t* part = P.ex + X.part + ((int64_t)l * s.nwg + K.w) * X.part_words;
#pragma unroll 1
    for (int g0 = 0; g0 < G; g0 += GP) {
      if (g0 > 0 && nbw > 0) kv_issue(0, kn, vn);
      float m[GP], ls[GP], acc[GP][8];
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        m[g] = -INFINITY;
        ls[g] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
      }
      auto update = [&](const v4u kw, const v4u vw, bool valid) {
        const float kf[8] = {bf16lo(kw.x), bf16hi(kw.x), bf16lo(kw.y), bf16hi(kw.y),
                             bf16lo(kw.z), bf16hi(kw.z), bf16lo(kw.w), bf16hi(kw.w)};
        const float vf[8] = {bf16lo(vw.x), bf16hi(vw.x), bf16lo(vw.y), bf16hi(vw.y),
                             bf16lo(vw.z), bf16hi(vw.z), bf16lo(vw.w), bf16hi(vw.w)};
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          const v4f a = *(const v4f*)(L.q + (g0 + g) * HD + dg * 8);
          const v4f b = *(const v4f*)(L.q + (g0 + g) * HD + dg * 8 + 4);
          float d = 0.f;
          d = fmaf(a.x, kf[0], d);
          d = fmaf(a.y, kf[1], d);
          d = fmaf(a.z, kf[2], d);
          d = fmaf(a.w, kf[3], d);
          d = fmaf(b.x, kf[4], d);
          d = fmaf(b.y, kf[5], d);
          d = fmaf(b.z, kf[6], d);
          d = fmaf(b.w, kf[7], d);
          d = LPP == 16 ? row16_sum(d) : row8_sum(d);
          const float sc = d * scale;
          if (valid) {
            const float mn = fmaxf(m[g], sc);
            const float c = exp2f(m[g] - mn);  // 0 while m is -inf
            const float pr = exp2f(sc - mn);
            ls[g] = fmaf(ls[g], c, pr);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(acc[g][e], c, pr * vf[e]);
            m[g] = mn;
          }
        }
      };
      auto kv_batch = [&](int32_t bi, const v4u* kc, const v4u* vc) {
#pragma unroll
        for (int e = 0; e < AB; ++e) {
          const int32_t i = bi * AB + e;
          if (i < ntw) update(kc[e], vc[e], (v + kWaves * i) * PPT + lpos < at.ncache);
        }
      };
      // every batch but the last with the next one in flight; the last on its own, with no loads
      for (int32_t bi = 0; bi + 1 < nbw; ++bi) {
        v4u kc[AB], vc[AB];
#pragma unroll
        for (int e = 0; e < AB; ++e) {
          kc[e] = kn[e];
          vc[e] = vn[e];
        }
        kv_issue(bi + 1, kn, vn);
        kv_batch(bi, kc, vc);
      }
      if (nbw > 0) kv_batch(nbw - 1, kn, vn);
      if (at.has_p && v == at.nkt % kWaves) {  // the current position, rounded to bf16 like the cache
        auto cur_row = [&](const float* src) {  // the lane's 8 values in two 16-byte LDS reads
          const v4f a = *(const v4f*)(src + dg * 8);
          const v4f c = *(const v4f*)(src + dg * 8 + 4);
          return v4u{f32_to_bf16(a.x) | (f32_to_bf16(a.y) << 16), f32_to_bf16(a.z) | (f32_to_bf16(a.w) << 16),
                     f32_to_bf16(c.x) | (f32_to_bf16(c.y) << 16), f32_to_bf16(c.z) | (f32_to_bf16(c.w) << 16)};
        };
        update(cur_row(L.q + G * HD), cur_row(L.q + (G + 1) * HD), lpos == 0);
      }
#pragma unroll
      for (int off = LPP; off < kWave; off <<= 1) {  // the position rows of the wave (lane pairs, no LDS)
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          float ma, mb, la, lb;
          lane_pair(m[g], off, lane, &ma, &mb);
          lane_pair(ls[g], off, lane, &la, &lb);
          const float M = fmaxf(ma, mb);
          const float f = ma == -INFINITY ? 0.f : exp2f(ma - M);
          const float fo = mb == -INFINITY ? 0.f : exp2f(mb - M);
          ls[g] = la * f + lb * fo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float aa, ab;
            lane_pair(acc[g][e], off, lane, &aa, &ab);
            acc[g][e] = aa * f + ab * fo;
          }
          m[g] = M;
        }
      }
      if (lpos == 0) {
#pragma unroll
        for (int g = 0; g < GP; ++g)
#pragma unroll
          for (int e = 0; e < 8; ++e) ws[g * (HD + 2) + dg * 8 + e] = acc[g][e];
      }
      if (lane == 0) {
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          ws[g * (HD + 2) + HD] = m[g];
          ws[g * (HD + 2) + HD + 1] = ls[g];
        }
      }
      bar();
      for (int e = K.tid; e < GP * (HD + 2); e += kThreads) {  // combine the 8 waves and publish
        const int g = e / (HD + 2), k = e % (HD + 2);
        // every wave's maximum and value first, so that the 16 LDS reads are in flight together
        float mw[kWaves], vw[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          mw[w] = L.scr[(w * GP + g) * (HD + 2) + HD];
          vw[w] = L.scr[(w * GP + g) * (HD + 2) + k];
        }
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mw[w]);
        float out;
        if (k == HD) {
          out = M;
        } else {
          out = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) out = fmaf(vw[w], mw[w] == -INFINITY ? 0.f : exp2f(mw[w] - M), out);
        }
        st_x(part + g0 * (HD + 2) + e, tag_f(out, ep));
      }
      bar();  // the next pass reuses the scratch
    }
  } else {
    constexpr bool kQInLds = G >= 4;
    constexpr int GR = kQInLds ? 1 : G;
    float qr[GR][8];
#pragma unroll
    for (int g = 0; g < GR; ++g) {
      const v4f a = *(const v4f*)(L.q + g * HD + dg * 8);
      const v4f b = *(const v4f*)(L.q + g * HD + dg * 8 + 4);
      qr[g][0] = a.x; qr[g][1] = a.y; qr[g][2] = a.z; qr[g][3] = a.w;
      qr[g][4] = b.x; qr[g][5] = b.y; qr[g][6] = b.z; qr[g][7] = b.w;
    }
    float m[G], ls[G], acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = -INFINITY;
      ls[g] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
    }
    auto update = [&](const v4u kw, const v4u vw, bool valid) {
      const float kf[8] = {bf16lo(kw.x), bf16hi(kw.x), bf16lo(kw.y), bf16hi(kw.y),
                           bf16lo(kw.z), bf16hi(kw.z), bf16lo(kw.w), bf16hi(kw.w)};
      const float vf[8] = {bf16lo(vw.x), bf16hi(vw.x), bf16lo(vw.y), bf16hi(vw.y),
                           bf16lo(vw.z), bf16hi(vw.z), bf16lo(vw.w), bf16hi(vw.w)};
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.f;
        if constexpr (kQInLds) {
          const v4f a = *(const v4f*)(L.q + g * HD + dg * 8);
          const v4f b = *(const v4f*)(L.q + g * HD + dg * 8 + 4);
          d = fmaf(a.x, kf[0], d);
          d = fmaf(a.y, kf[1], d);
          d = fmaf(a.z, kf[2], d);
          d = fmaf(a.w, kf[3], d);
          d = fmaf(b.x, kf[4], d);
          d = fmaf(b.y, kf[5], d);
          d = fmaf(b.z, kf[6], d);
          d = fmaf(b.w, kf[7], d);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) d = fmaf(qr[g][e], kf[e], d);
        }
        d = LPP == 16 ? row16_sum(d) : row8_sum(d);
        const float sc = d * scale;
        if (valid) {
          const float mn = fmaxf(m[g], sc);
          const float c = exp2f(m[g] - mn);  // 0 while m is -inf
          const float pr = exp2f(sc - mn);
          ls[g] = fmaf(ls[g], c, pr);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(acc[g][e], c, pr * vf[e]);
          m[g] = mn;
        }
      }
    };
    auto kv_batch = [&](int32_t bi, const v4u* kc, const v4u* vc) {
#pragma unroll
      for (int e = 0; e < AB; ++e) {
        const int32_t i = bi * AB + e;
        if (i < ntw) update(kc[e], vc[e], (v + kWaves * i) * PPT + lpos < at.ncache);
      }
    };
    // every batch but the last with the next one in flight; the last on its own, with no loads
    for (int32_t bi = 0; bi + 1 < nbw; ++bi) {
      v4u kc[AB], vc[AB];
#pragma unroll
      for (int e = 0; e < AB; ++e) {
        kc[e] = kn[e];
        vc[e] = vn[e];
      }
      kv_issue(bi + 1, kn, vn);
      kv_batch(bi, kc, vc);
    }
    if (nbw > 0) kv_batch(nbw - 1, kn, vn);
    // the current position: its K/V come from the exchange, rounded to bf16 like the cache
    if (at.has_p && v == at.nkt % kWaves) {
      auto cur_row = [&](const float* src) {  // the lane's 8 values in two 16-byte LDS reads
        const v4f a = *(const v4f*)(src + dg * 8);
        const v4f c = *(const v4f*)(src + dg * 8 + 4);
        return v4u{f32_to_bf16(a.x) | (f32_to_bf16(a.y) << 16), f32_to_bf16(a.z) | (f32_to_bf16(a.w) << 16),
                   f32_to_bf16(c.x) | (f32_to_bf16(c.y) << 16), f32_to_bf16(c.z) | (f32_to_bf16(c.w) << 16)};
      };
      update(cur_row(L.q + G * HD), cur_row(L.q + (G + 1) * HD), lpos == 0);
    }
    TR_HOP(K, H_ATT_DONE);
    // combine the position rows of the wave (lanes with the same dims: pairs exchanged in registers)
#pragma unroll
    for (int off = LPP; off < kWave; off <<= 1) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float ma, mb, la, lb;
        lane_pair(m[g], off, lane, &ma, &mb);
        lane_pair(ls[g], off, lane, &la, &lb);
        const float M = fmaxf(ma, mb);
        const float f = ma == -INFINITY ? 0.f : exp2f(ma - M);
        const float fo = mb == -INFINITY ? 0.f : exp2f(mb - M);
        ls[g] = la * f + lb * fo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float aa, ab;
          lane_pair(acc[g][e], off, lane, &aa, &ab);
          acc[g][e] = aa * f + ab * fo;
        }
        m[g] = M;
      }
    }
    float* ws = L.scr + v * G * (HD + 2);
    if (lpos == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) ws[g * (HD + 2) + dg * 8 + e] = acc[g][e];
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        ws[g * (HD + 2) + HD] = m[g];
        ws[g * (HD + 2) + HD + 1] = ls[g];
      }
    }
  }
  if constexpr (G <= 4) {
    bar();
    // combine the 8 waves and publish
    uint64_t* part = P.ex + X.part + ((int64_t)l * s.nwg + K.w) * X.part_words;
    for (int e = K.tid; e < G * (HD + 2); e += kThreads) {
      const int g = e / (HD + 2), k = e % (HD + 2);
      // every wave's maximum and value first, so that the 16 LDS reads are in flight together
      float mw[kWaves], vw[kWaves];
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        mw[w] = L.scr[(w * G + g) * (HD + 2) + HD];
        vw[w] = L.scr[(w * G + g) * (HD + 2) + k];
      }
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mw[w]);
      float out;
      if (k == HD) {
        out = M;
      } else {
        out = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) out = fmaf(vw[w], mw[w] == -INFINITY ? 0.f : exp2f(mw[w] - M), out);
      }
      st_x(part + e, tag_f(out, ep));
    }
    TR_HOP(K, H_ATT_COMB);
  }
  // the WG whose chunk holds the current position appends its K/V rows to the cache
  if (at.has_p) {
    const float* kp = L.q + G * HD;
    const float* vp = L.q + (G + 1) * HD;
    for (int e = K.tid; e < HD / 2; e += kThreads) {
      const uint32_t k2 = f32_to_bf16(kp[2 * e]) | (f32_to_bf16(kp[2 * e + 1]) << 16);
      const uint32_t v2 = f32_to_bf16(vp[2 * e]) | (f32_to_bf16(vp[2 * e + 1]) << 16);
      st_x32((uint32_t*)(P.kv + kv_offset(s, l, 0, at.j, pos)) + e, k2);
      st_x32((uint32_t*)(P.kv + kv_offset(s, l, 1, at.j, pos)) + e, v2);
    }
  }
  K.tr.add(T_ATT, TR_NOW() - ta);
  bar();  // scratch reuse
}

// Online-softmax state (m, S, A) of a set of positions, m in the exp2 domain: combine two.
__device__ __forceinline__ void softmax_combine(float& M, float& S, float& A, float m2, float s2, float a2) {
  const float Mn = fmaxf(M, m2);
  const float fo = M == -INFINITY ? 0.f : exp2f(M - Mn);
  const float fn = m2 == -INFINITY ? 0.f : exp2f(m2 - Mn);
  S = S * fo + s2 * fn;
  A = A * fo + a2 * fn;
  M = Mn;
}

// Merge of the chunk partials of one (query head, kMergeDims-dim slice). Thread (chunk lane cl,
// dim) folds chunks cl, cl + CL, ... in order; the chunk lanes of a wave are combined with
// shuffles and the 8 waves in LDS, always in the same order.
template <typename WK>
__device__ __forceinline__ void merge_unit(WK& K, const Att& at, int32_t l, int32_t u, uint32_t epoch) {
  const KParams& P = K.P;
  const Lds& L = K.L;
  const Shape& s = P.s;
  constexpr int D = kMergeDims;
  const int32_t slices = s.hd / D;
  const int32_t h = u / slices, sl = u % slices;
  const int32_t G = s.group();
  const int32_t j = h / G, g = h % G;
  constexpr int CL = kThreads / D;  // chunk lanes
  const int dim = K.tid % D, cl = K.tid / D;
  float M = -INFINITY, S = 0.f, A = 0.f;
  constexpr int KM = 4;  // chunks per thread in one pass (chunk lane stride CL)
  for (int32_t c0 = cl; c0 < at.nch && !K.fail; c0 += CL * KM) {
    uint64_t wm[KM], wl[KM], wa[KM];
    uint32_t todo = 0;
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (c0 + CL * k < at.nch) todo |= 1u << k;
    const uint32_t present = todo;
    Waiter wt;
    while (__builtin_amdgcn_ballot_w64(todo != 0) != 0) {
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        if (todo & (1u << k)) {
          const int32_t ch = c0 + CL * k;
          const uint64_t* pp =
              P.ex + P.exo.part + ((int64_t)l * s.nwg + ch * s.nkv + j) * P.exo.part_words + g * (s.hd + 2);
          wm[k] = ld_x(pp + s.hd);
          wl[k] = ld_x(pp + s.hd + 1);
          wa[k] = ld_x(pp + sl * D + dim);
        }
      }
#pragma unroll
      for (int k = 0; k < KM; ++k)
        if ((todo & (1u << k)) && (uint32_t)wm[k] == epoch && (uint32_t)wl[k] == epoch && (uint32_t)wa[k] == epoch)
          todo &= ~(1u << k);
      if (__builtin_amdgcn_ballot_w64(todo != 0) != 0) {
        if (wt.expired(P, L) || ((wt.spins & 63u) == 0 && global_error(P))) {
          K.fail = true;
          raise_error(P, L, wt.why);
          break;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (present & (1u << k))
        softmax_combine(M, S, A, __uint_as_float((uint32_t)(wm[k] >> 32)), __uint_as_float((uint32_t)(wl[k] >> 32)),
                        __uint_as_float((uint32_t)(wa[k] >> 32)));
  }
  // chunk lanes of this wave (lanes dim, dim + D, ...): butterfly over the lane bits above D
#pragma unroll
  for (int o = D; o < kWave; o <<= 1) {  // lane pairs exchanged in registers, lower lane first
    float m1, m2, s1, s2, a1, a2;
    lane_pair(M, o, K.lane, &m1, &m2);
    lane_pair(S, o, K.lane, &s1, &s2);
    lane_pair(A, o, K.lane, &a1, &a2);
    M = m1;
    S = s1;
    A = a1;
    softmax_combine(M, S, A, m2, s2, a2);
  }
  float* ms = L.scr;  // [8 waves][D][3]
  if (K.lane < D) {
    ms[(K.v * D + dim) * 3 + 0] = M;
    ms[(K.v * D + dim) * 3 + 1] = S;
    ms[(K.v * D + dim) * 3 + 2] = A;
  }
  bar();
  if (K.tid < D) {
    float mv[kWaves], sv[kWaves], av[kWaves];  // all 24 LDS reads in flight together
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      mv[k] = ms[(k * D + K.tid) * 3];
      sv[k] = ms[(k * D + K.tid) * 3 + 1];
      av[k] = ms[(k * D + K.tid) * 3 + 2];
    }
    float Mt = mv[0], St = sv[0], At = av[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) softmax_combine(Mt, St, At, mv[k], sv[k], av[k]);
    st_x(P.ex + P.exo.o + (int64_t)l * s.qdim() + h * s.hd + sl * D + K.tid, tag_f(At / St, epoch));
  }
  bar();
}

// Two merge units at once (units u and u + 1 when `two`; the workgroup's halves take one each):
// one round of polls instead of two where a workgroup owns several units (32 query heads over
// 256 workgroups). Thread (dim, chunk lane cl) of its half folds chunks cl, cl + 32, ... in
// order; the chunk lanes of a wave are combined with shuffles and the half's 4 waves in LDS,
// always in the same order.
template <typename WK>
__device__ __forceinline__ void merge_two_units(WK& K, const Att& at, int32_t l, int32_t u, bool two, uint32_t epoch) {
  const KParams& P = K.P;
  const Lds& L = K.L;
  const Shape& s = P.s;
  constexpr int D = kMergeDims;
  constexpr int HT = kThreads / 2;  // threads per unit
  constexpr int CL = HT / D;        // chunk lanes per unit
  const int32_t ui = K.tid / HT, th = K.tid % HT;
  const bool mine = ui == 0 || two;
  const int32_t uu = u + ui;
  const int32_t slices = s.hd / D;
  const int32_t h = uu / slices, sl = uu % slices;
  const int32_t G = s.group();
  const int32_t j = h / G, g = h % G;
  const int dim = th % D, cl = th / D;
  float M = -INFINITY, S = 0.f, A = 0.f;
  constexpr int KM = 4;
  for (int32_t c0 = cl; c0 < at.nch && !K.fail; c0 += CL * KM) {
    uint64_t wm[KM], wl[KM], wa[KM];
    uint32_t todo = 0;
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (mine && c0 + CL * k < at.nch) todo |= 1u << k;
    const uint32_t present = todo;
    Waiter wt;
    while (__builtin_amdgcn_ballot_w64(todo != 0) != 0) {
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        if (todo & (1u << k)) {
          const int32_t ch = c0 + CL * k;
          const uint64_t* pp =
              P.ex + P.exo.part + ((int64_t)l * s.nwg + ch * s.nkv + j) * P.exo.part_words + g * (s.hd + 2);
          wm[k] = ld_x(pp + s.hd);
          wl[k] = ld_x(pp + s.hd + 1);
          wa[k] = ld_x(pp + sl * D + dim);
        }
      }
#pragma unroll
      for (int k = 0; k < KM; ++k)
        if ((todo & (1u << k)) && (uint32_t)wm[k] == epoch && (uint32_t)wl[k] == epoch && (uint32_t)wa[k] == epoch)
          todo &= ~(1u << k);
      if (__builtin_amdgcn_ballot_w64(todo != 0) != 0) {
        if (wt.expired(P, L) || ((wt.spins & 63u) == 0 && global_error(P))) {
          K.fail = true;
          raise_error(P, L, wt.why);
          break;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (present & (1u << k))
        softmax_combine(M, S, A, __uint_as_float((uint32_t)(wm[k] >> 32)), __uint_as_float((uint32_t)(wl[k] >> 32)),
                        __uint_as_float((uint32_t)(wa[k] >> 32)));
  }
#pragma unroll
  for (int o = D; o < kWave; o <<= 1) {  // chunk lanes of this wave: lane pairs in registers, lower first
    float m1, m2, s1, s2, a1, a2;
    lane_pair(M, o, K.lane, &m1, &m2);
    lane_pair(S, o, K.lane, &s1, &s2);
    lane_pair(A, o, K.lane, &a1, &a2);
    M = m1;
    S = s1;
    A = a1;
    softmax_combine(M, S, A, m2, s2, a2);
  }
  float* ms = L.scr;  // [8 waves][D][3]
  if (K.lane < D) {
    ms[(K.v * D + dim) * 3 + 0] = M;
    ms[(K.v * D + dim) * 3 + 1] = S;
    ms[(K.v * D + dim) * 3 + 2] = A;
  }
  bar();
  constexpr int WPU = kWaves / 2;  // waves per unit
  if (K.tid < 2 * D && (K.tid < D || two)) {
    const int32_t ut = K.tid / D, dt = K.tid % D;
    const int32_t un = u + ut, hn = un / slices, sn = un % slices;
    const int w0 = ut * WPU;
    float mv[WPU], sv[WPU], av[WPU];  // all LDS reads in flight together
#pragma unroll
    for (int k = 0; k < WPU; ++k) {
      mv[k] = ms[((w0 + k) * D + dt) * 3];
      sv[k] = ms[((w0 + k) * D + dt) * 3 + 1];
      av[k] = ms[((w0 + k) * D + dt) * 3 + 2];
    }
    float Mt = mv[0], St = sv[0], At = av[0];
#pragma unroll
    for (int k = 1; k < WPU; ++k) softmax_combine(Mt, St, At, mv[k], sv[k], av[k]);
    st_x(P.ex + P.exo.o + (int64_t)l * s.qdim() + hn * s.hd + sn * D + dt, tag_f(At / St, epoch));
  }
  bar();
}

// ------------------------------------------------------------------------------------------
// Top-k sampling on the GPU (aikraft.ru «3000 токенов в секунду…», §04: sampling runs inside the
// monokernel, not on the host). Every WG computes the same token from the same exchanged words.
// ------------------------------------------------------------------------------------------
// SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014)
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9e3779b97f4a7c15ull;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
__device__ __forceinline__ double readlane_d(double v, int lane) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), lane);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// On entry the WG's LM outputs divided by the temperature, z, are in scr[0 .. 2 np) (row 2 pb +
// i at i) and every wave has passed a barrier after they were written. Candidate order is the
// argmax order (larger z, then the lower id), a strict total order once the padding ids (past V)
// are unique.
//  1. Each WG ranks its own rows and publishes its k best, in order, to rank slots [r][WG];
//     slots past its row count get padding (-inf, unique id >= V).
//  2. Every WG reads all heads (rank 0) and keeps the nsel = min(k, nwg) best lists: a row of the
//     global top k is in one of them (k better heads would otherwise precede it), at a list rank
//     below k, and not worse than H, the k-th best head (when nsel == k).
//  3. It reads those lists' first ke entries. The active ones (not worse than H; all when
//     nsel < k) form a prefix of each list and are compacted; an active entry's rank is the
//     number of active entries better than it. Every row better than a global top-k row is
//     active, so ranks below k are exact and every other entry counts at least k.
//  4. z_j of the k winners (in order) -> p_j = exp(z_j - z_0) / S with S summed in fp64 in order;
//     u = (splitmix64(seed ^ splitmix64(pos)) >> 40) * 2^-24; the first j whose running sum of
//     p_j exceeds u is drawn, the last candidate if none does.
// The rank loops read LDS at independent addresses and are unrolled so that the reads overlap.
template <typename WK>
__device__ __forceinline__ int32_t sample_topk(WK& K, const StageGeo& gl, uint64_t* lmx, uint32_t ep, int32_t pos) {
  const KParams& P = K.P;
  const Lds& L = K.L;
  const Shape& s = P.s;
  const int32_t kk = P.top_k, nwg = s.nwg, tid = K.tid;
  const int32_t nr = 2 * gl.np, r0 = 2 * gl.pb;
  uint64_t tp = TR_NOW();
  auto phase = [&](int slot) {  // top-k phase times of a KIE_TRACE build (constant slots)
    const uint64_t t = TR_NOW();
    K.tr.add(slot, t - tp);
    tp = t;
  };
  // 1.
  for (int32_t i = tid; i < nr; i += kThreads) {
    const float zi = L.scr[i];
    int32_t rank = 0;
#pragma unroll 8
    for (int32_t j = 0; j < nr; ++j) rank += better(L.scr[j], j, zi, i) ? 1 : 0;
    if (rank < kk) {
      st_x(lmx + ((int64_t)rank * nwg + K.w) * 2, tag_f(zi, ep));
      st_x(lmx + ((int64_t)rank * nwg + K.w) * 2 + 1, tag_u((uint32_t)(r0 + i), ep));
    }
  }
  if (tid >= nr && tid < kk) {
    st_x(lmx + ((int64_t)tid * nwg + K.w) * 2, tag_f(-INFINITY, ep));
    st_x(lmx + ((int64_t)tid * nwg + K.w) * 2 + 1, tag_u((uint32_t)(s.V + K.w * kMaxTopK + tid), ep));
  }
  // 2.
  const TopkLayout tl = topk_layout(s, kk);
  const int32_t nsel = tl.nsel, ke = tl.ke;
  float* const mg = L.act;  // act, xres and part are free once the LM outputs are final
  float* heads = mg + tl.heads;
  int32_t* sel = (int32_t*)(mg + tl.sel);
  int32_t* alen = (int32_t*)(mg + tl.alen);
  int32_t* off = (int32_t*)(mg + tl.off);
  float* top = mg + tl.top;
  float* ent = mg + tl.ent;
  uint64_t* ckey = (uint64_t*)(mg + tl.cmp);
  if (tid < nsel) {
    sel[tid] = tid;  // (every slot is overwritten below; this keeps it in range)
    alen[tid] = 0;
  }
  phase(16);
  K.template fetch_map<8>(2 * nwg, [&](int32_t q) { return lmx + q; }, heads, ep);
  phase(17);
  uint64_t* hkey = (uint64_t*)heads;  // each (z, id) pair becomes its key, in place
  uint64_t myk[(kMaxWG + kThreads - 1) / kThreads];
#pragma unroll
  for (int q = 0; q < (kMaxWG + kThreads - 1) / kThreads; ++q) {
    const int32_t x = tid + q * kThreads;
    myk[q] = x < nwg ? cand_key(heads[2 * x], __float_as_int(heads[2 * x + 1])) : 0;
  }
  bar();
#pragma unroll
  for (int q = 0; q < (kMaxWG + kThreads - 1) / kThreads; ++q)
    if (tid + q * kThreads < nwg) hkey[tid + q * kThreads] = myk[q];
  bar();
#pragma unroll
  for (int q = 0; q < (kMaxWG + kThreads - 1) / kThreads; ++q) {
    const int32_t x = tid + q * kThreads;
    if (x < nwg) {
      const int32_t rank = count_greater(hkey, nwg, myk[q]);
      if (rank < nsel) sel[rank] = x;
    }
  }
  if (tid < kk) {
    top[2 * tid] = -INFINITY;
    top[2 * tid + 1] = __int_as_float(0x7fffffff);
  }
  bar();
  phase(18);
  // 3.
  K.template fetch_map<16>(
      2 * nsel * ke,
      [&](int32_t q) {
        const int32_t e = q >> 1, j = e / ke, r = e - j * ke;
        return lmx + ((int64_t)r * nwg + sel[j]) * 2 + (q & 1);
      },
      ent, ep);
  phase(19);
  const bool bounded = nsel == kk;
  const uint64_t hb = hkey[sel[nsel - 1]];  // H
  for (int32_t e = tid; e < nsel * ke; e += kThreads)
    if (!bounded || cand_key(ent[2 * e], __float_as_int(ent[2 * e + 1])) >= hb)
      __hip_atomic_fetch_add(&alen[e / ke], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  bar();
  if (K.v == 0) {  // exclusive scan of the active lengths (nsel <= 64 lists: one wave)
    const int32_t lane = K.lane;
    const int32_t c = lane < nsel ? alen[lane] : 0;
    int32_t incl = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int32_t up = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += up;
    }
    if (lane < nsel) off[lane] = incl - c;
    if (lane == kWave - 1) off[nsel] = incl;
  }
  bar();
  for (int32_t e = tid; e < nsel * ke; e += kThreads) {  // compaction of the active entries
    const int32_t j = e / ke, r = e - j * ke;
    if (r < alen[j]) ckey[off[j] + r] = cand_key(ent[2 * e], __float_as_int(ent[2 * e + 1]));
  }
  bar();
  phase(20);
  const int32_t m = off[nsel];
  for (int32_t i = tid; i < m; i += kThreads) {
    const uint64_t ck = ckey[i];
    const int32_t rank = count_greater(ckey, m, ck);
    if (rank < kk) {
      top[2 * rank] = key_value(ck);
      top[2 * rank + 1] = __int_as_float(key_id(ck));
    }
  }
  bar();
  phase(21);
  // 4. (every wave, redundantly: no further barrier is needed to share the token)
  const int32_t lane = K.lane;
  const double z0 = (double)top[0];
  double e = 0.0;
  int32_t id = 0x7fffffff;
  if (lane < kk) {
    e = exp((double)top[2 * lane] - z0);
    id = __float_as_int(top[2 * lane + 1]);
  }
  double S = 0.0;
  for (int32_t j = 0; j < kk; ++j) S += readlane_d(e, j);
  const double p = e / S;
  const double u = (double)(splitmix64(P.seed ^ splitmix64((uint64_t)(int64_t)pos)) >> 40) * (1.0 / 16777216.0);
  int32_t chosen = __builtin_amdgcn_readlane(id, kk - 1);
  double cum = 0.0;
  for (int32_t j = 0; j < kk; ++j) {
    cum += readlane_d(p, j);
    if (cum > u) {
      chosen = __builtin_amdgcn_readlane(id, j);
      break;
    }
  }
  phase(22);
  bar();  // every wave has read top before the next step reuses this memory
  return chosen;
}

// The decode program of one wave. Its weight batches are consumed by one loop; the batch after
// the current one is always in flight. Between batches, boundary() runs the work that separates
// two stages -- finalising the outputs,
// attention, the merge, the exchange gathers, RMSNorm, sampling -- whenever the current stage has
// no batch left for this wave. Every wave runs every boundary, so the WG barriers inside match.
// MOE: after O the router stage runs, and its boundary (B_RT) chooses the layer's experts.
enum Boundary : int { B_START = 0, B_QKV = 1, B_O = 2, B_GU = 3, B_DN = 4, B_LM = 5, B_END = 6, B_RT = 7 };

template <int G, int HD, bool MOE, bool W8>
__device__ __forceinline__ void decode(Wk<MOE, W8>& K) {
  const KParams& P = K.P;
  const Lds& L = K.L;
  const Shape& s = P.s;
  const Exch& X = P.exo;
  uint64_t* ex = P.ex;
  const uint64_t t_start = TR_NOW();
  const int32_t tid = K.tid;
  int32_t tok = P.first_tok[0];
  if (tok < 0 || tok >= s.V) {
    if (K.w == 0 && tid == 0) __hip_atomic_fetch_or(P.err, KERR_BAD_TOKEN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    tok = 0;
  }
  tok = clamp_token(__builtin_amdgcn_readfirstlane(tok), s.V);
  K.start();  // the stream's first batch

  int32_t step = 0, l = 0;
  int32_t pos = P.pos0;
  uint32_t ep = P.epoch0;
  Att at = att_info(s, K.w, pos);
  bool lm = step_has_lm(P, 0);
  float ss = 0.f;
  float* xres = L.xres;  // the current residual buffer (of two)
  int bnd = B_START;  // the next boundary
  int st = -1;        // stage of the batches being reduced
  int32_t rem = 0, b = 0;
  bool done = false;

  auto boundary = [&]() {
    while (rem == 0 && !done) {
      if (P.skew) {  // a WG-uniform, deterministic delay per (WG, step, layer, boundary)
        uint32_t hsh = (uint32_t)K.w * 0x9E3779B1u ^ (uint32_t)step * 0x85EBCA77u ^ (uint32_t)l * 0xC2B2AE3Du ^
                       (uint32_t)bnd * 0x27D4EB2Fu;
        hsh ^= hsh >> 15;
        hsh *= 0x2C1B3C6Du;
        hsh ^= hsh >> 12;
        for (uint32_t i = hsh % P.skew; i > 0; --i) __builtin_amdgcn_s_sleep(127);
      }
      const uint64_t tb = TR_NOW();
      const int bnd_run = bnd;
#if defined(KIE_TRACE) || defined(KIE_TRACE_HOPS)
      K.hop_on = step == kHopStep && l == kHopLayer;
#endif
      bool routed = false;  // the router boundary of a mixture-of-experts layer (not in the switch,
                            // so that the dense program is compiled as if it did not exist)
      if constexpr (MOE) {
        if (bnd == B_RT) {  // router logits -> gather all E -> the layer's experts (the same in every WG)
          // phase times of a KIE_TRACE build in slots 16-18 (the top-k sampler's, unused when greedy)
          uint64_t tr0 = TR_NOW();
          bar();
          uint64_t* rx = ex + X.rt + (int64_t)l * s.E;
          K.template finalize<ST_RT>([&](int32_t gp, float ya, float yb) {
            st_x(rx + 2 * gp, tag_f(ya, ep));
            st_x(rx + 2 * gp + 1, tag_f(yb, ep));
          });
          uint64_t tr1 = TR_NOW();
          K.tr.add(16, tr1 - tr0);
          K.template fetch_f32<8>(rx, s.E, L.scr, ep, false);
          tr0 = TR_NOW();
          K.tr.add(17, tr0 - tr1);
          K.route(step, l);
          K.tr.add(18, TR_NOW() - tr0);
          st = ST_GU;
          bnd = B_GU;
          routed = true;
        }
      }
      if (!routed) switch (bnd) {
        case B_START: {  // embedding row -> residual stream, RMSNorm of layer 0
          if (tid < s.hd / 2) L.rope[tid] = P.rope[(int64_t)pos * (s.hd / 2) + tid];
          K.prefetch_gain(P.norms);
          float sq = 0.f;
          for (int32_t i = tid; i < s.d; i += kThreads) {
            const float x = __uint_as_float((uint32_t)P.embed[(int64_t)tok * s.d + i] << 16);
            xres[i] = x;
            sq = fmaf(x, x, sq);
          }
          ss = K.block_sum(sq);
          K.norm_to_act(ss, xres);
          st = ST_QKV;
          bnd = B_QKV;
          break;
        }
        case B_QKV: {  // QKV outputs (+RoPE) -> attention -> merge -> gather o
          bar();
          TR_HOP(K, H_QKV_IN);
          uint64_t* qx = ex + X.q + (int64_t)l * s.qdim();
          uint64_t* kx = ex + X.k + (int64_t)l * s.kvdim();
          uint64_t* vx = ex + X.v + (int64_t)l * s.kvdim();
          float sq = 1.f, sk = 1.f, sv = 1.f;
          if constexpr (W8) {
            sq = P.wscale[l * 7];
            sk = P.wscale[l * 7 + 1];
            sv = P.wscale[l * 7 + 2];
          }
          K.template finalize<ST_QKV>([&](int32_t gp, float ya, float yb) {
            const int32_t half = s.hd / 2;
            const int32_t hs = gp / half, i = gp % half;
            if constexpr (W8) {  // the matrix's scale times the codes' dot product
              const float sc = hs < s.nq ? sq : (hs < s.nq + s.nkv ? sk : sv);
              ya *= sc;
              yb *= sc;
            }
            if (hs < s.nq + s.nkv) {  // query and key heads are rotated
              const float2 cs = L.rope[i];
              const float ra = ya * cs.x - yb * cs.y, rb = yb * cs.x + ya * cs.y;
              ya = ra;
              yb = rb;
            }
            uint64_t* dst;
            int32_t h;
            if (hs < s.nq) {
              dst = qx;
              h = hs;
            } else if (hs < s.nq + s.nkv) {
              dst = kx;
              h = hs - s.nq;
            } else {
              dst = vx;
              h = hs - s.nq - s.nkv;
            }
            st_x(dst + h * s.hd + i, tag_f(ya, ep));
            st_x(dst + h * s.hd + i + half, tag_f(yb, ep));
          });
          TR_HOP(K, H_QKV_PUB);
          if (at.c0 <= pos) attention<G, HD>(K, at, l, pos, ep);
          TR_HOP(K, H_ATT_PUB);
          {
            const uint64_t tm = TR_NOW();
            const int32_t nu = merge_units(s);
            const int32_t rk = xcd_rank(s.nwg, K.w);
            const int32_t u0 = (int32_t)(((int64_t)rk * nu + s.nwg - 1) / s.nwg);
            if constexpr (G >= 8) {  // several units per workgroup at these head counts: two at a time
              for (int32_t u = u0; u < nu && merge_unit_rank(s, u) == rk; u += 2)
                merge_two_units(K, at, l, u, u + 1 < nu && merge_unit_rank(s, u + 1) == rk, ep);
            } else {
              for (int32_t u = u0; u < nu && merge_unit_rank(s, u) == rk; ++u) merge_unit(K, at, l, u, ep);
            }
            K.tr.add(T_MERGE, TR_NOW() - tm);
          }
          TR_HOP(K, H_MERGE_PUB);
          K.fetch_f32(ex + X.o + (int64_t)l * s.qdim(), s.qdim(), L.act, ep, false);
          TR_HOP(K, H_O_GOT);
          // The K/V rows this WG appended are complete before it publishes anything more. Here
          // the wave has just waited for its polls, so nothing newer is queued and the wait
          // costs nothing; after the next stage's first batch is issued it would wait for that.
          if (at.has_p) __builtin_amdgcn_s_waitcnt(kWaitVm0);
          st = ST_O;
          bnd = B_O;
          break;
        }
        case B_O: {  // O outputs + residual -> gather xa -> RMSNorm
          bar();
          TR_HOP(K, H_O_IN);
          uint64_t* xa = ex + X.xa + (int64_t)l * s.d;
          K.prefetch_gain(P.norms + (int64_t)l * 2 * s.d + s.d);
          const float so = W8 ? P.wscale[l * 7 + 3] : 1.f;
          K.template finalize<ST_O>([&](int32_t gp, float ya, float yb) {
            if constexpr (W8) {
              ya *= so;
              yb *= so;
            }
            const float2 r = *(const float2*)(xres + 2 * gp);  // the residual pair in one read
            st_x(xa + 2 * gp, tag_f(r.x + ya, ep));
            st_x(xa + 2 * gp + 1, tag_f(r.y + yb, ep));
          });
          TR_HOP(K, H_XA_PUB);
          K.issue_x();  // the gate/up stage is the longest: start its second batch now
          xres = xres == L.xres ? L.xres + s.d : L.xres;  // the other buffer: no wave reads it now
          ss = K.fetch_f32(xa, s.d, xres, ep, true);
          K.norm_to_act(ss, xres);
          TR_HOP(K, H_XA_GOT);
          st = MOE ? ST_RT : ST_GU;
          bnd = MOE ? B_RT : B_GU;
          break;
        }
        case B_GU: {  // SwiGLU outputs -> gather h
          bar();
          TR_HOP(K, H_GU_IN);
          uint64_t* hx = ex + X.h + (int64_t)l * s.F;
          const float sg = W8 ? P.wscale[l * 7 + 4] : 1.f, su = W8 ? P.wscale[l * 7 + 5] : 1.f;
          K.template finalize<ST_GU>([&](int32_t gp, float ya, float yb) {
            if constexpr (W8) {
              ya *= sg;
              yb *= su;
            }
            float h = (ya / (1.0f + expf(-ya))) * yb;
            if constexpr (MOE) h = K.weight_of(gp / s.Fe) * h;  // the routing weight of its expert
            st_x(hx + gp, tag_f(h, ep));
          });
          TR_HOP(K, H_H_PUB);
          K.issue_x();
          K.template fetch_f32<kGatherH>(hx, s.F, L.act, ep, false);
          TR_HOP(K, H_H_GOT);
          st = ST_DN;
          bnd = B_DN;
          break;
        }
        case B_DN: {  // down outputs + residual -> next layer's input (or the LM head's)
          uint64_t td = TR_NOW();
          auto dphase = [&](int slot) {  // phase times of this boundary in a KIE_TRACE build
            const uint64_t t = TR_NOW();
            K.tr.add(slot, t - td);
            td = t;
          };
          bar();
          TR_HOP(K, H_DN_IN);
          dphase(24);
          uint64_t* xf = ex + X.xf + (int64_t)(l + 1) * s.d;
          K.prefetch_gain(P.norms + (l + 1 < s.L ? (int64_t)(l + 1) * 2 * s.d : (int64_t)s.L * 2 * s.d));
          const float sd = W8 ? P.wscale[l * 7 + 6] : 1.f;
          K.template finalize<ST_DN>([&](int32_t gp, float ya, float yb) {
            if constexpr (W8) {
              ya *= sd;
              yb *= sd;
            }
            const float2 r = *(const float2*)(xres + 2 * gp);  // the residual pair in one read
            st_x(xf + 2 * gp, tag_f(r.x + ya, ep));
            st_x(xf + 2 * gp + 1, tag_f(r.y + yb, ep));
          });
          dphase(25);
          TR_HOP(K, H_XF_PUB);
          K.issue_x();  // the next layer's stages
#ifdef KIE_TRACE
          if (step == 8 && l == 12) K.tr.c[29] = now_ticks();  // one sample of absolute times
#endif
          xres = xres == L.xres ? L.xres + s.d : L.xres;  // the other buffer: no wave reads it now
          dphase(26);
          if (aborted(L)) {
            bar();
            bnd = B_END;
            st = -1;
          } else if (l + 1 < s.L) {
            ++l;
            ss = K.fetch_f32(xf, s.d, xres, ep, true);
#ifdef KIE_TRACE
            if (step == 8 && l == 13) K.tr.c[30] = now_ticks();
#endif
            TR_HOP(K, H_XF_GOT);
            dphase(27);
            K.norm_to_act(ss, xres);
            TR_HOP(K, H_NORM_DONE);
            dphase(28);
            st = ST_QKV;
            bnd = B_QKV;
          } else if (lm) {
            ss = K.fetch_f32(xf, s.d, xres, ep, true);
            K.norm_to_act(ss, xres);
            st = ST_LM;
            bnd = B_LM;
          } else {
            st = -1;
            bnd = B_END;
          }
          break;
        }
        case B_LM:
        case B_END: {  // LM outputs and this WG's argmax candidate; the grid-wide join; next token
          // Once per step, wave 0 reads the caller's abort word. Its decision reaches the other
          // waves through the LDS flag, which they read only after the barriers below.
          if (P.abort_word && K.v == 0 && __builtin_amdgcn_readfirstlane(host_abort(P)) != 0)
            raise_error(P, L, KERR_ABORTED);
          float bv = -INFINITY;
          int32_t bi = 0x7fffffff;
          const bool topk = bnd == B_LM && P.top_k > 1;
          if (bnd == B_LM) {
            bar();
            float* lo = P.logits_out ? P.logits_out + (P.lm_last_only ? 0 : (int64_t)step * s.V) : nullptr;
            const int32_t pb = K.g[ST_LM].pb;
            const float sl = W8 ? P.wscale[s.L * 7] : 1.f;
            K.template finalize<ST_LM>([&](int32_t gp, float ya, float yb) {
              const int32_t ra = 2 * gp, rb = 2 * gp + 1;
              if constexpr (W8) {
                ya *= sl;
                yb *= sl;
              }
              if (better(ya, ra, bv, bi)) {
                bv = ya;
                bi = ra;
              }
              if (better(yb, rb, bv, bi)) {
                bv = yb;
                bi = rb;
              }
              if (lo) {
                lo[ra] = ya;
                lo[rb] = yb;
              }
              if (topk) {  // NaN ranks as -inf and -0 as +0, so the candidate order stays strict
                const float za = ya / P.temperature, zb = yb / P.temperature;
                L.scr[2 * (gp - pb)] = za == za ? (za == 0.f ? 0.f : za) : -INFINITY;
                L.scr[2 * (gp - pb) + 1] = zb == zb ? (zb == 0.f ? 0.f : zb) : -INFINITY;
              }
            });
          }
          const uint64_t tsm = TR_NOW();
          int32_t next;
          if (topk) {
            bar();
            next = clamp_token(sample_topk(K, K.g[ST_LM], ex + X.lm, ep, pos), s.V);
          } else {
            // every WG gathers all candidates: no WG reuses a step's exchange buffers before every
            // WG has finished reading them
            K.block_argmax(&bv, &bi);
            if (tid == 0) {
              st_x(ex + X.lm + 2 * K.w, tag_f(bv, ep));
              st_x(ex + X.lm + 2 * K.w + 1, tag_u((uint32_t)bi, ep));
            }
            K.fetch_f32(ex + X.lm, 2 * s.nwg, L.scr, ep, false);
            bv = -INFINITY;
            bi = 0x7fffffff;
            for (int k = tid; k < s.nwg; k += kThreads) {
              const float cv = L.scr[2 * k];
              const int32_t ci = __float_as_int(L.scr[2 * k + 1]);
              if (better(cv, ci, bv, bi)) {
                bv = cv;
                bi = ci;
              }
            }
            bar();  // every thread has read its candidates before scr is reused
            K.block_argmax(&bv, &bi);
            next = clamp_token(bi, s.V);
          }
          K.tr.add(T_SAMPLE, TR_NOW() - tsm);
          if (lm && K.w == 0 && tid == 0) {
            if (P.tokens_out) P.tokens_out[step] = next;
            if (P.last_tok_out && step == P.n_steps - 1) P.last_tok_out[0] = next;
            if (P.tok_ring) {  // the host sees each token while the launch goes on
              const int64_t c = P.ring_base + step;
              __hip_atomic_store(P.tok_ring + 1 + (int32_t)(c % P.ring_cap), next, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_SYSTEM);
              __hip_atomic_store(P.tok_ring, (int32_t)(c + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
            }
          }
          if (P.forced && step + 1 < P.n_steps) {
            int32_t f = P.forced[step];
            if (f < 0 || f >= s.V) {
              if (K.w == 0 && tid == 0)
                __hip_atomic_fetch_or(P.err, KERR_BAD_TOKEN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              f = 0;
            }
            next = clamp_token(__builtin_amdgcn_readfirstlane(f), s.V);
          }
          tok = next;
          ++step;
          if (step >= P.n_steps || aborted(L)) {
            done = true;
          } else {
            l = 0;
            pos = P.pos0 + step;
            ep = P.epoch0 + (uint32_t)step;
            at = att_info(s, K.w, pos);
            lm = step_has_lm(P, step);
          }
          st = -1;
          bnd = B_START;
          break;
        }
      }
      K.tr.add(T_BAR, TR_NOW() - tb);
      {
        const uint64_t dt = TR_NOW() - tb;  // per boundary kind (constant slots keep the counters in registers)
        switch (bnd_run) {
          case B_START: K.tr.add(10, dt); break;
          case B_QKV: K.tr.add(11, dt); break;
          case B_O: K.tr.add(12, dt); break;
          case B_GU: K.tr.add(13, dt); break;
          case B_DN: K.tr.add(14, dt); break;
          case B_RT: K.tr.add(23, dt); break;
          default: K.tr.add(15, dt); break;
        }
      }
      rem = st >= 0 ? K.nb_of(st) : 0;
      b = 0;
    }
  };

#if defined(KIE_TRACE) || defined(KIE_TRACE_HOPS)
  int32_t lbatch = 0;  // wave 0's batches of the current layer so far
#endif
  while (true) {
    boundary();
    if (done) break;
    const uint64_t tg = TR_NOW();
    v4u cur[kBatch];
#if defined(KIE_TRACE) || defined(KIE_TRACE_HOPS)
    if (st == ST_QKV && b == 0) lbatch = 0;
    const bool bt = step == kHopStep && l == kHopLayer && st != ST_LM;
#endif
    K.take(cur);
#if defined(KIE_TRACE) || defined(KIE_TRACE_HOPS)
    if (bt) TR_BATCH(K, 2 * lbatch);
#endif
    K.reduce_batch(K.geo_of(st), b, cur);
#if defined(KIE_TRACE) || defined(KIE_TRACE_HOPS)
    if (bt) TR_BATCH(K, 2 * lbatch + 1);
    ++lbatch;
#endif
    K.tr.add(T_GEMV, TR_NOW() - tg);
    K.tr.add(T_BATCHES, 1);
    --rem;
    ++b;
  }
  // a batch loaded into LDS past the launch's last step may still be in flight: the wave must
  // not end (and give up its LDS) before that load has landed
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#if defined(KIE_TRACE) || defined(KIE_TRACE_HOPS)
  if (K.v == 0) {  // wave 0's stamps, to the trace words of waves 0 (events) and 1 (batches)
    const int64_t base = (int64_t)K.w * kWaves * kTraceWords + kTraceHop;
    if (K.lane < 32) P.trace[base + K.lane] = L.hopt[K.lane];
    else P.trace[base + kTraceWords + (K.lane - 32)] = L.hopt[K.lane];
  }
#endif
  K.tr.add(T_TOTAL, TR_NOW() - t_start);
  K.tr.flush(P.trace + ((int64_t)K.w * kWaves + K.v) * kTraceWords, K.lane);
}

// The kernels. The prompt pass (teacher-forced steps whose only output is the last logits and
// the first token) runs the same program under its own symbol, so that profiles separate it
// from decoding.
#define KIE_KERNEL_BODY(G, HD, MOE, W8)                                     \
  const Lds L = lds_map<G>(kie_smem, P.s);                                 \
  if (threadIdx.x < C_COUNT) L.ctl[threadIdx.x] = 0;                       \
  if (threadIdx.x < kHopWords) L.hopt[threadIdx.x] = 0;                    \
  __syncthreads();                                                         \
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);    \
  Wk<MOE, W8> K(P, L, blockIdx.x, wave, threadIdx.x % kWave);              \
  decode<G, HD, MOE, W8>(K);

template <int G, int HD>
__global__ void __launch_bounds__(kThreads, 1) kie_decode_kernel(KParams P) {
  KIE_KERNEL_BODY(G, HD, false, false)
}
template <int G, int HD>
__global__ void __launch_bounds__(kThreads, 1) kie_prompt_kernel(KParams P) {
  KIE_KERNEL_BODY(G, HD, false, false)
}
// Mixture-of-experts layers (the same program with the router stage and routed expert batches)
template <int G, int HD>
__global__ void __launch_bounds__(kThreads, 1) kie_moe_decode_kernel(KParams P) {
  KIE_KERNEL_BODY(G, HD, true, false)
}
template <int G, int HD>
__global__ void __launch_bounds__(kThreads, 1) kie_moe_prompt_kernel(KParams P) {
  KIE_KERNEL_BODY(G, HD, true, false)
}
// 8-bit (e4m3fn) layer matrices and LM head with one scale per matrix
template <int G, int HD>
__global__ void __launch_bounds__(kThreads, 1) kie_fp8_decode_kernel(KParams P) {
  KIE_KERNEL_BODY(G, HD, false, true)
}
template <int G, int HD>
__global__ void __launch_bounds__(kThreads, 1) kie_fp8_prompt_kernel(KParams P) {
  KIE_KERNEL_BODY(G, HD, false, true)
}

}  // namespace kie
