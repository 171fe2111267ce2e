// monokernel.hip -- the persistent batch-1 decode kernel for MI355X (gfx950).
//
// One launch decodes n tokens; control never returns to the host in between (agentlenshq.com,
// 《突破内存墙：在标准 GPU 上实现 3,000 tokens/s 的推理速度》, "The Monokernel Runtime"; aikraft.ru
// «3000 токенов в секунду…», §04 "Моноядро": one resident GPU program covering MatMul,
// attention, normalisation and sampling, with tight control of synchronisation, prefetch and
// execution order). The design below is this library's own for CDNA4; the pages only say that the
// vendor's kernels exist.
//
// Grid: one 512-thread workgroup (WG) per compute unit, all co-resident (cooperative launch).
// Each WG runs two kinds of waves:
//   * 4 producer waves stream the WG's packed weight slice -- and its share of the KV cache --
//     from HBM into a ring of 1 KiB tiles in LDS, as far ahead as the ring allows. Weights do
//     not depend on activations, so the HBM stream keeps flowing while the consumers wait for
//     the inputs of the next stage (the prefetch across synchronisation points the pages name).
//   * 4 consumer waves wait for a stage's input vector, then reduce the ring's tiles against it
//     (fp32 FMA on widened bf16 weights), and publish their outputs.
// Producers publish one progress counter each ("my tiles below index 4m+p are in the ring") and
// consumers one watermark each ("I have read all my tiles below index W"); both are updated
// once per batch of tiles.
// Inter-WG exchange uses 64-bit tagged words (fp32 value << 32 | epoch) written and read with
// agent-scope atomics, so a reader knows a word is current by its tag alone: no grid barrier,
// no flag round trip, no L2 flush. Epochs are unique per decode step and buffers are per layer.
//
// Per layer the stages are: QKV (+RMSNorm, RoPE) -> attention over a chunk of positions of one
// KV head (split-K: scores, then softmax-weighted values) -> merge of the chunk partials -> O
// (+residual) -> gate/up (+RMSNorm, SwiGLU) -> down (+residual). Then the final RMSNorm + LM
// head and the sampler.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "layout.h"
#include "monokernel.h"

namespace kie {

// Optional per-wave cycle counters (compile with -DKIE_TRACE); free in normal builds.
#ifdef KIE_TRACE
#define TR_NOW() __builtin_readcyclecounter()
#else
#define TR_NOW() 0ull
#endif
enum TraceSlot : int {
  TC_WAIT_TILE = 0, TC_FETCH = 1, TC_CSYNC = 2, TC_GEMV = 3, TC_ATT = 4, TC_MERGE = 5, TC_TOTAL = 6, TC_TILES = 7,
  TC_SAMPLE = 8, TC_NORM = 9,
  TP_WAIT_FREE = 0, TP_WRITE = 1, TP_GATE = 2, TP_ISSUE = 3, TP_TOTAL = 6, TP_TILES = 7
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
  uint8_t* ring;      // R x 1 KiB
  float* act;         // stage input vector (fp32); during attention: q, k_p, v_p, scores
  float* xres;        // residual stream of the current layer (fp32, d)
  float* scr;         // scratch for reductions / attention partials / sampler
  float* stage;       // per consumer wave: the stage outputs of its pairs, published after the stage
  float2* rope;       // (cos, sin) of the current position, hd/2 entries
  uint32_t* ctl;      // control words
};
enum Ctl : int {
  C_BAR = 0,    // consumer barrier counter
  C_STEP = 1,   // step the consumers have started
  C_ABORT = 2,  // set on any failure in this WG
  C_DONE = 4,   // [4] per producer p: its tiles 4m+p with m below this value are in the ring
  C_WM = 8,     // [4] per consumer: every one of its tiles below this stream index has been read
  C_COUNT = 16
};
constexpr int kStageWords = 128;  // per consumer wave: at most 64 pairs per wave and stage

__host__ __device__ inline int32_t att_scores_max(const Shape& s) { return s.group() * att_chunk_len(s, s.max_seq); }
__host__ __device__ inline int32_t act_floats(const Shape& s) {
  int32_t a = s.d;
  if (s.qdim() > a) a = s.qdim();
  if (s.F > a) a = s.F;
  const int32_t att = (s.group() + 2) * s.hd + att_scores_max(s);
  if (att > a) a = att;
  return (a + 3) & ~3;
}
__host__ __device__ inline int32_t scr_floats(const Shape& s) {
  int32_t a = kConsumerWaves * s.group() * (s.hd + 2);
  if (8 * kMergeDims * 3 > a) a = 8 * kMergeDims * 3;
  if (2 * s.nwg > a) a = 2 * s.nwg;
  if (a < 64) a = 64;
  return (a + 3) & ~3;
}
__host__ __device__ inline int32_t lds_fixed_bytes(const Shape& s) {
  return (act_floats(s) + s.d + scr_floats(s) + kConsumerWaves * kStageWords + s.hd) * 4 + C_COUNT * 4;
}
int32_t lds_bytes_for(const Shape& s, int32_t ring) { return ring * kTileBytes + lds_fixed_bytes(s); }
int32_t max_ring_slots(const Shape& s, int32_t lds_limit) {
  int32_t r = (lds_limit - lds_fixed_bytes(s)) / kTileBytes;
  r &= ~7;
  if (r > 128) r = 128;
  return r;
}

__device__ __forceinline__ Lds lds_map(uint8_t* smem, const Shape& s, int32_t R) {
  Lds L;
  uint8_t* p = smem;
  L.ring = p; p += (size_t)R * kTileBytes;
  L.act = (float*)p; p += (size_t)act_floats(s) * 4;
  L.xres = (float*)p; p += (size_t)s.d * 4;
  L.scr = (float*)p; p += (size_t)scr_floats(s) * 4;
  L.stage = (float*)p; p += (size_t)kConsumerWaves * kStageWords * 4;
  L.rope = (float2*)p; p += (size_t)s.hd * 4;
  L.ctl = (uint32_t*)p;
  return L;
}

// ------------------------------------------------------------------------------------------
// Per-WG plan and the token stream's segments
// ------------------------------------------------------------------------------------------
struct Plan {
  int32_t w;
  int32_t pb[ST_COUNT];   // first global pair of each stage
  int32_t np[ST_COUNT];   // pairs owned
  int32_t kt[ST_COUNT];   // k-tiles per pair
  int32_t pre[ST_COUNT];  // tile offset of the stage inside one layer's weight stream (LM: 0)
  int32_t t_layer;        // weight tiles per layer
  int64_t wbase;          // first tile of this WG in the packed image
};

// GEMV inputs are stored in LDS permuted so that lane l's 8 inputs of k-tile j are two 16-byte
// rows at (j, half h, lane l): element k = 256 j + 8 l + t lives at 256 j + 128 (t >> 2) + 4 l +
// (t & 3). Each ds_read_b128 of a wave then touches 512 contiguous bytes (no bank conflicts).
__device__ __forceinline__ int32_t act_perm(int32_t k) {
  return (k & ~255) | ((k & 4) << 5) | ((k & 248) >> 1) | (k & 3);
}

// Per-stage fields selected through a switch, so that the arrays stay in registers.
__device__ __forceinline__ int32_t pick(const int32_t* a, int st) {
  switch (st) {
    case ST_QKV: return a[ST_QKV];
    case ST_O: return a[ST_O];
    case ST_GU: return a[ST_GU];
    case ST_DN: return a[ST_DN];
    default: return a[ST_LM];
  }
}

__device__ __forceinline__ Plan make_plan(const KParams& P, int32_t w) {
  Plan pl;
  pl.w = w;
  int32_t acc = 0;
  for (int st = 0; st < ST_COUNT; ++st) {
    const int32_t n = P.s.stage_pairs(st);
    pl.pb[st] = split_begin(n, P.s.nwg, w);
    pl.np[st] = split_end(n, P.s.nwg, w) - pl.pb[st];
    pl.kt[st] = P.s.stage_kt(st);
    if (st <= ST_DN) {
      pl.pre[st] = acc;
      acc += pl.np[st] * pl.kt[st];
    } else {
      pl.pre[st] = 0;
    }
  }
  pl.t_layer = acc;
  pl.wbase = P.wbase[w];
  return pl;
}

// Attention work of this WG at context length n (= pos + 1).
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

// Segment q of a step's stream: q = 6 l + k with k 0 QKV, 1 K rows, 2 V rows, 3 O, 4 gate/up,
// 5 down; q = 6 L is the LM head. Every segment is one linear range of 1 KiB tiles.
struct SegD {
  const uint8_t* base;  // first tile
  int32_t len;          // tiles
  int32_t kv;           // K/V rows (the last tile may be partly past the cached positions)
  int32_t nval_last;    // lanes of the last tile holding data (64 for weights)
};
__device__ __forceinline__ SegD seg_desc(const KParams& P, const Plan& pl, const Att& at, int32_t step, int32_t q) {
  SegD g;
  const Shape& s = P.s;
  g.kv = 0;
  g.nval_last = kWave;
  if (q == 6 * s.L) {
    g.base = P.packed + (size_t)(pl.wbase + (int64_t)s.L * pl.t_layer) * kTileBytes;
    g.len = step_has_lm(P, step) ? pl.np[ST_LM] * pl.kt[ST_LM] : 0;
    return g;
  }
  const int32_t l = q / 6, k = q % 6;
  if (k == 1 || k == 2) {
    g.kv = 1;
    g.base = (const uint8_t*)(P.kv + kv_offset(s, l, k - 1, at.j, at.c0));
    g.len = at.nkt;
    const int32_t ppt = att_pos_per_tile(s);
    g.nval_last = (at.ncache - (at.nkt - 1) * ppt) * (s.hd / 8);
    return g;
  }
  const int st = k == 0 ? ST_QKV : (k == 3 ? ST_O : (k == 4 ? ST_GU : ST_DN));
  g.base = P.packed + (size_t)(pl.wbase + (int64_t)l * pl.t_layer + pick(pl.pre, st)) * kTileBytes;
  g.len = pick(pl.np, st) * pick(pl.kt, st);
  return g;
}

// ------------------------------------------------------------------------------------------
// Failure handling: every wait is bounded; on expiry the WG records an error and stops.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void raise_error(const KParams& P, const Lds& L, uint32_t code) {
  lds_st(&L.ctl[C_ABORT], 1u);
  __hip_atomic_fetch_or(P.err, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// LDS word read by the whole wave (same address): the value is made wave-uniform so that every
// decision taken on it is a scalar branch.
__device__ __forceinline__ uint32_t lds_ld_u(const uint32_t* p) { return __builtin_amdgcn_readfirstlane(lds_ld(p)); }
__device__ __forceinline__ bool aborted(const Lds& L) { return lds_ld_u(&L.ctl[C_ABORT]) != 0; }

// Bounded spin: call expired() after every unsuccessful poll. Every 256th call it checks the
// WG's abort flag and the elapsed time of this wait (wave-uniform; no global memory access, so
// the compiler never has to drain outstanding stores inside an LDS wait loop). Waits on global
// memory additionally watch the grid's error word (global_error()).
struct Waiter {
  uint32_t spins = 0;
  uint64_t start = 0;
  __device__ __forceinline__ bool expired(const KParams& P, const Lds& L) {
    if ((++spins & 255u) != 0) return false;
    if (aborted(L)) return true;
    const uint64_t t = now_ticks();
    if (start == 0) {
      start = t;
      return false;
    }
    return t - start > (uint64_t)P.timeout_ticks;
  }
};
__device__ __forceinline__ bool global_error(const KParams& P) {
  return __builtin_amdgcn_readfirstlane(__hip_atomic_load(P.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0;
}

// ------------------------------------------------------------------------------------------
// Producer waves
// ------------------------------------------------------------------------------------------
constexpr int kProdBatch = 8;

struct PBatch {
  uint32_t first;     // stream index of the batch's first tile (the others follow at stride 4)
  int32_t n;          // tiles in the batch
  int32_t nval_last;  // lanes of the last tile holding data
};

// Producer wave pw handles the WG's stream tiles pw, pw+4, pw+8, ... . It walks the segments of
// each step; within a segment its tiles form batches of up to 8 that are loaded with 8
// unconditional 16-byte-per-lane loads. Two batches are in flight: while batch X is loading,
// batch Y (issued before) is written into the ring once the consumers' watermarks show that the
// slots' previous tiles have been read. K/V rows of step s are only loaded once the consumers
// have started step s (every row they read is final by then).
__device__ __forceinline__ void producer(const KParams& P, const Lds& L, const Plan& pl, int pw, int lane) {
  const uint32_t R = (uint32_t)P.ring_slots;
  const Shape& s = P.s;
  Tracer tr;
  const uint64_t t_start = TR_NOW();
  bool fail = false;
  v4u bufA[kProdBatch], bufB[kProdBatch];
  PBatch ba, bb;
  ba.first = bb.first = 0;
  ba.n = bb.n = 0;
  ba.nval_last = bb.nval_last = kWave;
  bool pend_a = false, pend_b = false;  // issued and not yet written

  auto write = [&](const PBatch& b, const v4u* buf) {
    const uint32_t last = b.first + (uint32_t)(4 * (b.n - 1));
    // every slot of the batch is free once all consumers have read past (last - R)
    if (last >= R) {
      const uint64_t t0 = TR_NOW();
      Waiter wt;
      for (;;) {
        const uint32_t w0 = lds_ld(&L.ctl[C_WM + 0]), w1 = lds_ld(&L.ctl[C_WM + 1]);
        const uint32_t w2 = lds_ld(&L.ctl[C_WM + 2]), w3 = lds_ld(&L.ctl[C_WM + 3]);
        uint32_t m = w0 < w1 ? w0 : w1;
        m = m < w2 ? m : w2;
        m = m < w3 ? m : w3;
        m = __builtin_amdgcn_readfirstlane(m);
        if (m + R > last) break;
        __builtin_amdgcn_s_sleep(1);
        if (wt.expired(P, L)) {
          fail = true;
          return;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      tr.add(TP_WAIT_FREE, TR_NOW() - t0);
    }
    const uint64_t t0 = TR_NOW();
    uint32_t slot = b.first % R;
#pragma unroll
    for (int k = 0; k < kProdBatch; ++k) {
      if (k < b.n) {
        v4u v = buf[k];
        if (k == b.n - 1 && lane >= b.nval_last) v = v4u{0u, 0u, 0u, 0u};
        *(v4u*)(L.ring + slot * kTileBytes + lane * 16) = v;
        slot += kProducerWaves;
        if (slot >= R) slot -= R;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) lds_st(&L.ctl[C_DONE + pw], (last >> 2) + 1);
    tr.add(TP_WRITE, TR_NOW() - t0);
    tr.add(TP_TILES, (uint64_t)b.n);
  };
  // 8 loads, always issued (slots beyond n are never written); lanes of a last K/V tile past the
  // cached positions re-read its first row (zeroed on write)
  auto issue = [&](v4u* buf, const uint8_t* base, uint32_t t, int32_t n, bool last_partial, int32_t nval_last) {
#pragma unroll
    for (int k = 0; k < kProdBatch; ++k) {
      const uint32_t tk = k < n ? t + 4u * (uint32_t)k : t;
      // unused slots (k >= n) read only the first row of the batch's first tile, which exists
      const bool masked = k >= n || (last_partial && k == n - 1 && lane >= nval_last);
      const uint8_t* src = base + (size_t)tk * kTileBytes + (masked ? 0 : lane * 16);
      buf[k] = __builtin_nontemporal_load((const v4u*)src);
    }
  };

  uint32_t spos = 0;  // stream index of the current segment's first tile
  for (int32_t step = 0; step < P.n_steps && !fail; ++step) {
    const Att at = att_info(s, pl.w, P.pos0 + step);
    for (int32_t q = 0; q <= 6 * s.L && !fail; ++q) {
      const SegD g = seg_desc(P, pl, at, step, q);
      if (g.len == 0) continue;
      if (g.kv && step > 0 && (int32_t)lds_ld_u(&L.ctl[C_STEP]) < step) {
        // flush what is in flight (oldest first), then wait until the consumers have started
        // this step
        if (pend_a && pend_b && bb.first < ba.first) {
          write(bb, bufB);
          pend_b = false;
        }
        if (pend_a && !fail) { write(ba, bufA); pend_a = false; }
        if (pend_b && !fail) { write(bb, bufB); pend_b = false; }
        const uint64_t t0 = TR_NOW();
        Waiter wt;
        while (!fail && (int32_t)lds_ld_u(&L.ctl[C_STEP]) < step) {
          __builtin_amdgcn_s_sleep(2);
          if (wt.expired(P, L)) fail = true;
        }
        tr.add(TP_GATE, TR_NOW() - t0);
        if (fail) break;
      }
      uint32_t t = ((uint32_t)pw - spos) & 3u;  // this producer's first tile in the segment
      while (t < (uint32_t)g.len && !fail) {
        const int32_t left = (int32_t)(((uint32_t)g.len - t + 3u) >> 2);
        const int32_t n = left < kProdBatch ? left : kProdBatch;
        const bool lastp = g.kv && (t + 4u * (uint32_t)(n - 1) == (uint32_t)g.len - 1u) && g.nval_last < kWave;
        // the two buffers alternate; the older pending batch is written after the new issue
        if (!pend_a) {
          issue(bufA, g.base, t, n, lastp, g.nval_last);
          ba.first = spos + t;
          ba.n = n;
          ba.nval_last = lastp ? g.nval_last : kWave;
          pend_a = true;
          if (pend_b) { write(bb, bufB); pend_b = false; }
        } else {
          issue(bufB, g.base, t, n, lastp, g.nval_last);
          bb.first = spos + t;
          bb.n = n;
          bb.nval_last = lastp ? g.nval_last : kWave;
          pend_b = true;
          write(ba, bufA);
          pend_a = false;
        }
        t += 4u * (uint32_t)n;
      }
      spos += (uint32_t)g.len;
    }
  }
  // drain, oldest first
  if (!fail && pend_a && pend_b && bb.first < ba.first) {
    write(bb, bufB);
    pend_b = false;
  }
  if (!fail && pend_a) write(ba, bufA);
  if (!fail && pend_b) write(bb, bufB);
  tr.add(TP_TOTAL, TR_NOW() - t_start);
  tr.flush(P.trace + ((int64_t)pl.w * (kThreads / kWave) + pw) * kTraceWords, lane);
  if (fail) raise_error(P, L, KERR_PRODUCER);
}

// ------------------------------------------------------------------------------------------
// Consumer waves
// ------------------------------------------------------------------------------------------
struct Cons {
  const KParams& P;
  const Lds& L;
  const Plan& pl;
  int c;     // consumer wave 0..3 (wave-uniform)
  int lane;
  int tid;   // 0..255 among consumer threads
  uint32_t bar_target;
  bool fail;
  Tracer tr;
  __device__ __forceinline__ Cons(const KParams& p, const Lds& l, const Plan& q, int c_, int lane_)
      : P(p), L(l), pl(q), c(c_), lane(lane_), tid(c_ * kWave + lane_), bar_target(0), fail(false) {}

  // barrier of the 4 consumer waves (LDS counter; the producers are not involved)
  __device__ __forceinline__ void csync() {
    fail = __builtin_amdgcn_ballot_w64(fail) != 0;  // one lane's failure is the wave's
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) __hip_atomic_fetch_add(&L.ctl[C_BAR], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    bar_target += kConsumerWaves;
    Waiter wt;
    const uint64_t t0 = TR_NOW();
    while ((int32_t)(lds_ld_u(&L.ctl[C_BAR]) - bar_target) < 0) {
      __builtin_amdgcn_s_sleep(1);
      if (wt.expired(P, L)) {
        fail = true;
        break;
      }
    }
    tr.add(TC_CSYNC, TR_NOW() - t0);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }

  // Wait until the ring holds the NB tiles i, i+nr, ... (one read of the 4 producer counters).
  template <int NB>
  __device__ __forceinline__ void wait_ready(uint32_t i, uint32_t nr) {
    const uint64_t t0 = TR_NOW();
    bool waited = false;
    Waiter wt;
    for (;;) {
      const uint32_t d0 = lds_ld(&L.ctl[C_DONE + 0]), d1 = lds_ld(&L.ctl[C_DONE + 1]);
      const uint32_t d2 = lds_ld(&L.ctl[C_DONE + 2]), d3 = lds_ld(&L.ctl[C_DONE + 3]);
      const uint32_t e0 = __builtin_amdgcn_readfirstlane(d0), e1 = __builtin_amdgcn_readfirstlane(d1);
      const uint32_t e2 = __builtin_amdgcn_readfirstlane(d2), e3 = __builtin_amdgcn_readfirstlane(d3);
      bool ok = true;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint32_t ib = i + (uint32_t)b * nr;
        const uint32_t p = ib & 3u, need = (ib >> 2) + 1u;
        const uint32_t have = p == 0 ? e0 : (p == 1 ? e1 : (p == 2 ? e2 : e3));
        ok &= (int32_t)(have - need) >= 0;
      }
      if (ok) break;
      waited = true;
      __builtin_amdgcn_s_sleep(1);
      if (wt.expired(P, L)) {
        fail = true;
        break;
      }
    }
    if (waited) tr.add(TC_WAIT_TILE, TR_NOW() - t0);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }
  // every tile of this wave below stream index w has been read (its data are in registers)
  __device__ __forceinline__ void watermark(uint32_t w) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) lds_st(&L.ctl[C_WM + c], w);
  }
  __device__ __forceinline__ uint32_t slot_of(uint32_t i) const { return i % (uint32_t)P.ring_slots; }
  __device__ __forceinline__ const v4u* tile_ptr(uint32_t slot) const {
    return (const v4u*)(L.ring + slot * kTileBytes + lane * 16);
  }

  // Gather n tagged words with the given epoch from src into LDS floats dst. Every consumer
  // thread polls its words tid, tid+256, ... (all in flight at once), writes each value as soon
  // as its tag is current, and re-polls only the missing ones. If want_ss, returns the sum of
  // squares of the n values (fixed summation order) to every consumer thread.
  // The consumer barrier below is reached by every consumer thread, whatever its word count.
  __device__ __forceinline__ float fetch(const uint64_t* src, int n, float* dst, uint32_t epoch, bool want_ss,
                                        bool permute = false) {
    constexpr int KMAX = 16;
    const uint64_t tf = TR_NOW();
    for (int base = 0; base < n; base += KMAX * kConsumerThreads) {
      const uint64_t* sp = src + base + tid;
      float* dp = dst + base + tid;
      uint32_t missing = 0;
#pragma unroll
      for (int k = 0; k < KMAX; ++k)
        if (base + tid + k * kConsumerThreads < n) missing |= 1u << k;
      uint64_t wv[KMAX];
#pragma unroll
      for (int k = 0; k < KMAX; ++k)
        if (missing & (1u << k)) wv[k] = ld_x(sp + k * kConsumerThreads);
      if (base == 0) csync();  // earlier readers of dst are done before it is overwritten
      Waiter wt;
      while (true) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          if ((missing & (1u << k)) && (uint32_t)wv[k] == epoch) {
            missing &= ~(1u << k);
            const float v = __uint_as_float((uint32_t)(wv[k] >> 32));
            if (permute)
              dst[act_perm(base + tid + k * kConsumerThreads)] = v;
            else
              dp[k * kConsumerThreads] = v;
          }
        }
        if (__builtin_amdgcn_ballot_w64(missing != 0) == 0 || fail) break;  // the whole wave is done
        __builtin_amdgcn_s_sleep(1);
        if (wt.expired(P, L) || ((wt.spins & 255u) == 0 && global_error(P))) {
          fail = true;
          break;
        }
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
          if (missing & (1u << k)) wv[k] = ld_x(sp + k * kConsumerThreads);
      }
    }
    tr.add(TC_FETCH, TR_NOW() - tf);
    float ss = 0.f;
    if (want_ss) {
      const uint64_t tn = TR_NOW();
      for (int e = tid; e < n; e += kConsumerThreads) ss = fmaf(dst[e], dst[e], ss);
      ss = block_sum(ss);
      tr.add(TC_NORM, TR_NOW() - tn);
    }
    csync();
    return ss;
  }

  // Gather up to three short ranges (query heads and the current K/V row) into LDS floats.
  __device__ __forceinline__ void fetch3(const uint64_t* s0, int n0, float* d0, const uint64_t* s1, int n1, float* d1,
                                         const uint64_t* s2, int n2, float* d2, uint32_t epoch) {
    constexpr int KM = 8;
    const uint64_t tf = TR_NOW();
    const int ntot = n0 + n1 + n2;
    for (int base = 0; base < ntot; base += KM * kConsumerThreads) {
      uint32_t missing = 0;
#pragma unroll
      for (int k = 0; k < KM; ++k)
        if (base + tid + k * kConsumerThreads < ntot) missing |= 1u << k;
      uint64_t wv[KM];
      auto reload = [&]() {
#pragma unroll
        for (int k = 0; k < KM; ++k) {
          if (missing & (1u << k)) {
            const int e = base + tid + k * kConsumerThreads;
            const uint64_t* p = e < n0 ? s0 + e : (e < n0 + n1 ? s1 + (e - n0) : s2 + (e - n0 - n1));
            wv[k] = ld_x(p);
          }
        }
      };
      reload();
      if (base == 0) csync();
      Waiter wt;
      while (true) {
#pragma unroll
        for (int k = 0; k < KM; ++k) {
          if ((missing & (1u << k)) && (uint32_t)wv[k] == epoch) {
            missing &= ~(1u << k);
            const int e = base + tid + k * kConsumerThreads;
            float* d = e < n0 ? d0 + e : (e < n0 + n1 ? d1 + (e - n0) : d2 + (e - n0 - n1));
            *d = __uint_as_float((uint32_t)(wv[k] >> 32));
          }
        }
        if (__builtin_amdgcn_ballot_w64(missing != 0) == 0 || fail) break;
        __builtin_amdgcn_s_sleep(1);
        if (wt.expired(P, L) || ((wt.spins & 255u) == 0 && global_error(P))) {
          fail = true;
          break;
        }
        reload();
      }
    }
    tr.add(TC_FETCH, TR_NOW() - tf);
    csync();
  }

  // sum over the 256 consumer threads, in a fixed order; every consumer thread gets the result
  __device__ __forceinline__ float block_sum(float v) {
    float lo, hi;
    half_wave_sums(v, &lo, &hi);
    v = lo + hi;
    csync();  // scr may still be read by a previous user
    if (lane == 0) L.scr[c] = v;
    csync();
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < kConsumerWaves; ++k) t += L.scr[k];
    return t;
  }

  // act[i] = (xres[i] * r) * g[i],  r = 1/sqrt(ss/d + eps)
  __device__ __forceinline__ void rmsnorm_to_act(float ss, const uint16_t* g) {
    const int d = P.s.d;
    const float r = 1.0f / sqrtf(ss / (float)d + P.s.eps);
    for (int i = tid; i < d; i += kConsumerThreads) {
      const float gi = __uint_as_float((uint32_t)g[i] << 16);
      L.act[act_perm(i)] = (L.xres[i] * r) * gi;
    }
    csync();
  }

  // ------------------------------------------------------------------ GEMV stage
  // NB tiles of one pair: tiles i, i+nr, ... covering k-tiles j0 .. j0+NB-1.
  template <int NB>
  __device__ __forceinline__ void gemv_batch(uint32_t i, uint32_t nr, int32_t j0, float& a0, float& a1) {
    wait_ready<NB>(i, nr);
    v4u w[NB];
    uint32_t slot = slot_of(i);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      w[b] = *tile_ptr(slot);
      slot += nr;
      if (slot >= (uint32_t)P.ring_slots) slot -= (uint32_t)P.ring_slots;
    }
    v4f x0[NB], x1[NB];
    const float* ap = L.act + j0 * kTileK + (lane & 31) * 4;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      x0[b] = *(const v4f*)(ap + b * kTileK);
      x1[b] = *(const v4f*)(ap + b * kTileK + 128);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      a0 = fmaf(bf16lo(w[b].x), x0[b].x, a0);
      a1 = fmaf(bf16hi(w[b].x), x0[b].y, a1);
      a0 = fmaf(bf16lo(w[b].y), x0[b].z, a0);
      a1 = fmaf(bf16hi(w[b].y), x0[b].w, a1);
      a0 = fmaf(bf16lo(w[b].z), x1[b].x, a0);
      a1 = fmaf(bf16hi(w[b].z), x1[b].y, a1);
      a0 = fmaf(bf16lo(w[b].w), x1[b].z, a0);
      a1 = fmaf(bf16hi(w[b].w), x1[b].w, a1);
    }
    watermark(i + (uint32_t)(NB - 1) * nr + 1u);
  }

  __device__ __forceinline__ void gemv_pair(uint32_t i, uint32_t nr, int32_t kt, float& a0, float& a1) {
    constexpr int B = 8;
    int32_t j0 = 0;
    for (; j0 + B <= kt; j0 += B, i += (uint32_t)B * nr) gemv_batch<B>(i, nr, j0, a0, a1);
    switch (kt - j0) {  // remainder (kt is not a multiple of 8 for small K)
      case 1: gemv_batch<1>(i, nr, j0, a0, a1); break;
      case 2: gemv_batch<2>(i, nr, j0, a0, a1); break;
      case 3: gemv_batch<3>(i, nr, j0, a0, a1); break;
      case 4: gemv_batch<4>(i, nr, j0, a0, a1); break;
      case 5: gemv_batch<5>(i, nr, j0, a0, a1); break;
      case 6: gemv_batch<6>(i, nr, j0, a0, a1); break;
      case 7: gemv_batch<7>(i, nr, j0, a0, a1); break;
      default: break;
    }
  }

  // Each consumer wave takes pairs lp = c, c+4, ...; per tile, lane l multiplies its 8 bf16
  // weights by act[256 j + 8 (l mod 32) ...]; the two half-waves reduce to the pair's two dot
  // products. val(gp, ya, yb) turns them into the pair's two outputs (e.g. RoPE, residual);
  // they are staged in LDS and published by pub(gp, half, value) after the wave's last pair, all
  // lanes storing at once (no exchange store inside the tile loop, so the compiler never drains
  // outstanding stores there).
  template <typename Val, typename Pub>
  __device__ __forceinline__ void gemv(int st, uint32_t tile_base, Val val, Pub pub) {
    const uint64_t tg = TR_NOW();
    const int32_t np = pick(pl.np, st), kt = pick(pl.kt, st);
    const int32_t pb = pick(pl.pb, st);
    const int32_t full = np / kConsumerWaves;
    float* stg = L.stage + c * kStageWords;
    int32_t k = 0;
    for (int32_t lp = c; lp < np; lp += kConsumerWaves, ++k) {
      const int32_t r = lp / kConsumerWaves;
      const uint32_t nr = r < full ? (uint32_t)kConsumerWaves : (uint32_t)(np - full * kConsumerWaves);
      const uint32_t i = tile_base + (uint32_t)(r * kConsumerWaves * kt + c);  // tile j = 0 of the pair
      float a0 = 0.f, a1 = 0.f;
      gemv_pair(i, nr, kt, a0, a1);
      if (fail) return;
      float ya, yb;
      half_wave_sums(a0 + a1, &ya, &yb);
      const float2 o = val(pb + lp, ya, yb);
      if (lane == 0) {
        stg[2 * k] = o.x;
        stg[2 * k + 1] = o.y;
      }
    }
    watermark(tile_base + (uint32_t)(np * kt));  // nothing of this stage is left for this wave
    // publish: lane 2q+h stores output h of the wave's q-th pair
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    for (int32_t q0 = 0; q0 < k; q0 += kWave / 2) {
      const int32_t q = q0 + (lane >> 1), h = lane & 1;
      if (q < k) pub(pb + c + kConsumerWaves * q, h, stg[2 * q + h]);
    }
    tr.add(TC_TILES, (uint64_t)k * kt);
    tr.add(TC_GEMV, TR_NOW() - tg);
  }
};

// ------------------------------------------------------------------------------------------
// Attention for one KV head over this WG's chunk of positions: pass 1 computes the scores of
// the chunk (K tiles), pass 2 the softmax-weighted sum of V rows (V tiles) with the chunk's
// maximum; the 4 consumer waves' partial sums are added and one partial (acc[hd], m, l) per
// query head of the group is published (exp2 domain; m is the chunk maximum).
// ------------------------------------------------------------------------------------------
template <int G, int HD>
__device__ __forceinline__ void attention_chunk(Cons& C, const Att& at, int32_t l, int32_t pos, uint32_t tile_base,
                                                uint32_t epoch) {
  const KParams& P = C.P;
  const Lds& L = C.L;
  const Shape& s = P.s;
  constexpr int LPP = HD / 8;    // lanes per position
  constexpr int PPT = 64 / LPP;  // positions per tile
  const int lane = C.lane;
  const int lpos = lane / LPP, dg = lane % LPP;
  const float* q = L.act;              // [G][HD]
  const float* kp = L.act + G * HD;    // current position's k (fp32, after RoPE)
  const float* vp = L.act + (G + 1) * HD;
  float* sc = L.act + (G + 2) * HD;    // scores [G][positions of the chunk]
  const int32_t npos = at.ncache + (at.has_p ? 1 : 0);
  const float scale = 1.4426950408889634f / sqrtf((float)HD);

  float qr[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const v4f a = *(const v4f*)(q + g * HD + dg * 8);
    const v4f b = *(const v4f*)(q + g * HD + dg * 8 + 4);
    qr[g][0] = a.x; qr[g][1] = a.y; qr[g][2] = a.z; qr[g][3] = a.w;
    qr[g][4] = b.x; qr[g][5] = b.y; qr[g][6] = b.z; qr[g][7] = b.w;
  }
  auto score = [&](v4u kw, float* out) {
    const float kf[8] = {bf16lo(kw.x), bf16hi(kw.x), bf16lo(kw.y), bf16hi(kw.y),
                         bf16lo(kw.z), bf16hi(kw.z), bf16lo(kw.w), bf16hi(kw.w)};
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(qr[g][e], kf[e], d);
      d = LPP == 16 ? row16_sum(d) : row8_sum(d);
      out[g] = d * scale;
    }
  };
  // the current position's K/V come from the exchange, rounded to bf16 like the cache
  auto cur_row = [&](const float* src) {
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = f32_to_bf16(src[dg * 8 + e]);
    return v4u{b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16)};
  };

  // pass 1: scores of the cached positions (K tiles) and of the current position
  for (int32_t tp = C.c; tp < at.nkt; tp += kConsumerWaves) {
    const uint32_t i = tile_base + (uint32_t)tp;
    C.wait_ready<1>(i, 1);
    if (C.fail) return;
    const v4u kw = *C.tile_ptr(C.slot_of(i));
    float sg[G];
    score(kw, sg);
    C.watermark(i + 1);
    const int32_t p = tp * PPT + lpos;
    if (dg == 0 && p < at.ncache) {
#pragma unroll
      for (int g = 0; g < G; ++g) sc[g * at.cs + p] = sg[g];
    }
  }
  if (at.has_p && C.c == (at.nkt % kConsumerWaves)) {
    float sg[G];
    score(cur_row(kp), sg);
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) sc[g * at.cs + at.ncache] = sg[g];
    }
  }
  C.csync();
  // chunk maximum per head (every wave computes it; fixed order)
  float mx[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m = -INFINITY;
    for (int32_t p = lane; p < npos; p += kWave) m = fmaxf(m, sc[g * at.cs + p]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    mx[g] = m;
  }
  // pass 2: V tiles; lane (lpos, dg) accumulates p * V over its positions for dims dg*8..+8
  float acc[G][8], lsum[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    lsum[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }
  auto accumulate = [&](v4u vw, int32_t p, bool valid) {
    const float vf[8] = {bf16lo(vw.x), bf16hi(vw.x), bf16lo(vw.y), bf16hi(vw.y),
                         bf16lo(vw.z), bf16hi(vw.z), bf16lo(vw.w), bf16hi(vw.w)};
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float pr = valid ? exp2f(sc[g * at.cs + p] - mx[g]) : 0.f;
      lsum[g] += pr;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(pr, vf[e], acc[g][e]);
    }
  };
  const uint32_t vbase = tile_base + (uint32_t)at.nkt;
  for (int32_t tp = C.c; tp < at.nkt; tp += kConsumerWaves) {
    const uint32_t i = vbase + (uint32_t)tp;
    C.wait_ready<1>(i, 1);
    if (C.fail) return;
    const v4u vw = *C.tile_ptr(C.slot_of(i));
    const int32_t p = tp * PPT + lpos;
    accumulate(vw, p < at.ncache ? p : 0, p < at.ncache);
    C.watermark(i + 1);
  }
  if (at.has_p && C.c == (at.nkt % kConsumerWaves)) accumulate(cur_row(vp), at.ncache, lpos == 0);
  C.watermark(tile_base + (uint32_t)(2 * at.nkt));
  // sums over the positions of a tile (lanes with the same dims); lsum counts each position
  // once (its LPP lanes hold the same probability)
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[g][e];
#pragma unroll
      for (int o = LPP; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
      acc[g][e] = v;
    }
    float v = lsum[g];
#pragma unroll
    for (int o = LPP; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
    lsum[g] = v;
  }
  float* ws = L.scr + C.c * G * (HD + 2);
  if (lpos == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) ws[g * (HD + 2) + dg * 8 + e] = acc[g][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) ws[g * (HD + 2) + HD + 1] = lsum[g];
  }
  C.csync();
  uint64_t* part = P.ex + P.exo.part + ((int64_t)l * s.nwg + C.pl.w) * P.exo.part_words;
  for (int e = C.tid; e < G * (HD + 2); e += kConsumerThreads) {
    const int g = e / (HD + 2), k = e % (HD + 2);
    float out;
    if (k == HD) {
      out = mx[g];
    } else {
      out = 0.f;
#pragma unroll
      for (int w = 0; w < kConsumerWaves; ++w) out += L.scr[w * G * (HD + 2) + g * (HD + 2) + k];
    }
    st_x(part + e, tag_f(out, epoch));
  }
  // the WG whose chunk holds the current position appends its K/V rows to the cache
  if (at.has_p) {
    for (int e = C.tid; e < HD / 2; e += kConsumerThreads) {
      const uint32_t k2 = f32_to_bf16(kp[2 * e]) | (f32_to_bf16(kp[2 * e + 1]) << 16);
      const uint32_t v2 = f32_to_bf16(vp[2 * e]) | (f32_to_bf16(vp[2 * e + 1]) << 16);
      st_x32((uint32_t*)(P.kv + kv_offset(s, l, 0, at.j, pos)) + e, k2);
      st_x32((uint32_t*)(P.kv + kv_offset(s, l, 1, at.j, pos)) + e, v2);
    }
  }
  C.csync();  // scratch reuse
}

// merge of the chunk partials of one (query head, 32-dim slice)
__device__ __forceinline__ void merge_unit(Cons& C, const Att& at, int32_t l, int32_t u, uint32_t epoch) {
  const KParams& P = C.P;
  const Lds& L = C.L;
  const Shape& s = P.s;
  const int32_t slices = s.hd / kMergeDims;
  const int32_t h = u / slices, sl = u % slices;
  const int32_t G = s.group();
  const int32_t j = h / G, g = h % G;
  const int dim = C.tid % kMergeDims, cl = C.tid / kMergeDims;  // 8 chunk lanes
  float M = -INFINITY, S = 0.f, A = 0.f;
  constexpr int KM = 8;  // chunks per thread in one pass (chunk lane stride 8)
  for (int32_t c0 = cl; c0 < at.nch && !C.fail; c0 += 8 * KM) {
    uint64_t wm[KM], wl[KM], wa[KM];
    uint32_t missing = 0;
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (c0 + 8 * k < at.nch) missing |= 1u << k;
    Waiter wt;
    uint32_t todo = missing;
    while (__builtin_amdgcn_ballot_w64(todo != 0) != 0) {
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        if (todo & (1u << k)) {
          const int32_t ch = c0 + 8 * k;
          const uint64_t* pp =
              P.ex + P.exo.part + ((int64_t)l * s.nwg + ch * s.nkv + j) * P.exo.part_words + g * (s.hd + 2);
          wm[k] = ld_x(pp + s.hd);
          wl[k] = ld_x(pp + s.hd + 1);
          wa[k] = ld_x(pp + sl * kMergeDims + dim);
        }
      }
#pragma unroll
      for (int k = 0; k < KM; ++k)
        if ((todo & (1u << k)) && (uint32_t)wm[k] == epoch && (uint32_t)wl[k] == epoch && (uint32_t)wa[k] == epoch)
          todo &= ~(1u << k);
      if (__builtin_amdgcn_ballot_w64(todo != 0) != 0) {
        __builtin_amdgcn_s_sleep(1);
        if (wt.expired(P, L) || ((wt.spins & 255u) == 0 && global_error(P))) {
          C.fail = true;
          break;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (missing & (1u << k)) {
        const float mk = __uint_as_float((uint32_t)(wm[k] >> 32));
        const float lk = __uint_as_float((uint32_t)(wl[k] >> 32));
        const float ak = __uint_as_float((uint32_t)(wa[k] >> 32));
        const float Mn = fmaxf(M, mk);
        const float fo = M == -INFINITY ? 0.f : exp2f(M - Mn);
        const float fn = mk == -INFINITY ? 0.f : exp2f(mk - Mn);
        S = S * fo + lk * fn;
        A = A * fo + ak * fn;
        M = Mn;
      }
    }
  }
  C.csync();
  float* ms = C.L.scr;  // [8][32][3]
  ms[(cl * kMergeDims + dim) * 3 + 0] = M;
  ms[(cl * kMergeDims + dim) * 3 + 1] = S;
  ms[(cl * kMergeDims + dim) * 3 + 2] = A;
  C.csync();
  if (C.tid < kMergeDims) {
    float Mt = -INFINITY;
    for (int k = 0; k < 8; ++k) Mt = fmaxf(Mt, ms[(k * kMergeDims + C.tid) * 3]);
    float St = 0.f, At = 0.f;
    for (int k = 0; k < 8; ++k) {
      const float mk = ms[(k * kMergeDims + C.tid) * 3];
      const float f = mk == -INFINITY ? 0.f : exp2f(mk - Mt);
      St = fmaf(ms[(k * kMergeDims + C.tid) * 3 + 1], f, St);
      At = fmaf(ms[(k * kMergeDims + C.tid) * 3 + 2], f, At);
    }
    st_x(P.ex + P.exo.o + (int64_t)l * s.qdim() + h * s.hd + sl * kMergeDims + C.tid, tag_f(At / St, epoch));
  }
  C.csync();
}

// A token id that indexes memory is always kept inside [0, V).
__device__ __forceinline__ int32_t clamp_token(int32_t t, int32_t V) { return t < 0 ? 0 : (t >= V ? V - 1 : t); }

template <int G, int HD>
__device__ __forceinline__ void consumer(const KParams& P, const Lds& L, const Plan& pl, int c, int lane) {
  Cons C(P, L, pl, c, lane);
  const uint64_t t_start = TR_NOW();
  const Shape& s = P.s;
  const Exch& X = P.exo;
  uint64_t* ex = P.ex;
  uint32_t tbase = 0;  // stream index of the next segment's first tile
  int32_t tok = 0;
  if (C.tid == 0) {
    tok = P.first_tok[0];
    if (tok < 0 || tok >= s.V) {
      if (pl.w == 0) __hip_atomic_fetch_or(P.err, KERR_BAD_TOKEN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      tok = 0;
    }
  }
  // the token is uniform across consumer waves: broadcast through LDS
  if (C.tid == 0) L.scr[0] = __int_as_float(tok);
  C.csync();
  tok = clamp_token(__float_as_int(L.scr[0]), s.V);
  C.csync();

  for (int32_t step = 0; step < P.n_steps && !C.fail; ++step) {
    const int32_t pos = P.pos0 + step;
    const uint32_t ep = P.epoch0 + (uint32_t)step;
    const Att at = att_info(s, pl.w, pos);
    if (C.tid == 0) lds_st(&L.ctl[C_STEP], (uint32_t)step);
    if (C.tid < s.hd / 2) L.rope[C.tid] = P.rope[(int64_t)pos * (s.hd / 2) + C.tid];  // visible after block_sum
    // embedding row -> residual stream; RMSNorm inputs
    float ss = 0.f;
    for (int i = C.tid; i < s.d; i += kConsumerThreads) {
      const float v = __uint_as_float((uint32_t)P.embed[(int64_t)tok * s.d + i] << 16);
      L.xres[i] = v;
      ss = fmaf(v, v, ss);
    }
    ss = C.block_sum(ss);

    for (int32_t l = 0; l < s.L && !C.fail; ++l) {
      // ---------------- QKV
      if (l > 0) ss = C.fetch(ex + X.xf + (int64_t)l * s.d, s.d, L.xres, ep, true);
      C.rmsnorm_to_act(ss, P.norms + (int64_t)l * 2 * s.d);
      if (C.fail) break;
      {
        uint64_t* qx = ex + X.q + (int64_t)l * s.qdim();
        uint64_t* kx = ex + X.k + (int64_t)l * s.kvdim();
        uint64_t* vx = ex + X.v + (int64_t)l * s.kvdim();
        C.gemv(
            ST_QKV, tbase,
            [&](int32_t gp, float ya, float yb) {
              if (gp / (s.hd / 2) < s.nq + s.nkv) {  // query and key heads are rotated
                const float2 cs = L.rope[gp % (s.hd / 2)];
                return make_float2(ya * cs.x - yb * cs.y, yb * cs.x + ya * cs.y);
              }
              return make_float2(ya, yb);
            },
            [&](int32_t gp, int h, float v) {
              int mat;
              int32_t ra, rb;
              pair_rows(s, ST_QKV, gp, &mat, &ra, &rb);
              uint64_t* dst = mat == 0 ? qx : (mat == 1 ? kx : vx);
              st_x(dst + (h ? rb : ra), tag_f(v, ep));
            });
        tbase += (uint32_t)(pl.np[ST_QKV] * pl.kt[ST_QKV]);
      }
      // ---------------- attention over this WG's chunk
      if (at.c0 <= pos) {
        const int32_t G_ = s.group();
        const uint64_t* qsrc = ex + X.q + (int64_t)l * s.qdim() + (int64_t)at.j * G_ * s.hd;
        if (at.has_p)
          C.fetch3(qsrc, G_ * s.hd, L.act, ex + X.k + (int64_t)l * s.kvdim() + at.j * s.hd, s.hd, L.act + G_ * s.hd,
                   ex + X.v + (int64_t)l * s.kvdim() + at.j * s.hd, s.hd, L.act + (G_ + 1) * s.hd, ep);
        else
          C.fetch(qsrc, G_ * s.hd, L.act, ep, false);
        if (C.fail) break;
        const uint64_t ta = TR_NOW();
        attention_chunk<G, HD>(C, at, l, pos, tbase, ep);
        C.tr.add(TC_ATT, TR_NOW() - ta);
        tbase += (uint32_t)(2 * at.nkt);
      }
      // ---------------- merge of chunk partials (the WGs that own merge units)
      {
        const int32_t nu = merge_units(s);
        const int32_t u0 = (int32_t)(((int64_t)pl.w * nu + s.nwg - 1) / s.nwg);
        const uint64_t tm = TR_NOW();
        for (int32_t u = u0; u < nu && merge_unit_wg(s, u) == pl.w && !C.fail; ++u) merge_unit(C, at, l, u, ep);
        C.tr.add(TC_MERGE, TR_NOW() - tm);
      }
      // ---------------- O projection + residual
      C.fetch(ex + X.o + (int64_t)l * s.qdim(), s.qdim(), L.act, ep, false, true);
      if (C.fail) break;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this WG's K/V rows are complete before its next outputs
      {
        uint64_t* xa = ex + X.xa + (int64_t)l * s.d;
        C.gemv(
            ST_O, tbase,
            [&](int32_t gp, float ya, float yb) { return make_float2(L.xres[2 * gp] + ya, L.xres[2 * gp + 1] + yb); },
            [&](int32_t gp, int h, float v) { st_x(xa + 2 * gp + h, tag_f(v, ep)); });
        tbase += (uint32_t)(pl.np[ST_O] * pl.kt[ST_O]);
      }
      // ---------------- gate/up + SwiGLU
      C.csync();  // every wave has finished reading xres before it is replaced
      ss = C.fetch(ex + X.xa + (int64_t)l * s.d, s.d, L.xres, ep, true);
      C.rmsnorm_to_act(ss, P.norms + (int64_t)l * 2 * s.d + s.d);
      if (C.fail) break;
      {
        uint64_t* hx = ex + X.h + (int64_t)l * s.F;
        C.gemv(
            ST_GU, tbase,
            [&](int32_t gp, float ya, float yb) { return make_float2((ya / (1.0f + expf(-ya))) * yb, 0.f); },
            [&](int32_t gp, int h, float v) {
              if (h == 0) st_x(hx + gp, tag_f(v, ep));
            });
        tbase += (uint32_t)(pl.np[ST_GU] * pl.kt[ST_GU]);
      }
      // ---------------- down + residual
      C.csync();
      C.fetch(ex + X.h + (int64_t)l * s.F, s.F, L.act, ep, false, true);
      if (C.fail) break;
      {
        uint64_t* xf = ex + X.xf + (int64_t)(l + 1) * s.d;
        C.gemv(
            ST_DN, tbase,
            [&](int32_t gp, float ya, float yb) { return make_float2(L.xres[2 * gp] + ya, L.xres[2 * gp + 1] + yb); },
            [&](int32_t gp, int h, float v) { st_x(xf + 2 * gp + h, tag_f(v, ep)); });
        tbase += (uint32_t)(pl.np[ST_DN] * pl.kt[ST_DN]);
      }
      C.csync();
    }
    if (C.fail) break;

    // ---------------- final norm + LM head + local argmax
    float best_v = -INFINITY;
    int32_t best_i = 0x7fffffff;
    const bool lm = step_has_lm(P, step);
    if (lm) {
      ss = C.fetch(ex + X.xf + (int64_t)s.L * s.d, s.d, L.xres, ep, true);
      C.rmsnorm_to_act(ss, P.norms + (int64_t)s.L * 2 * s.d);
      if (C.fail) break;
      float* lo = P.logits_out ? P.logits_out + (P.lm_last_only ? 0 : (int64_t)step * s.V) : nullptr;
      C.gemv(
          ST_LM, tbase,
          [&](int32_t gp, float ya, float yb) {
            const int32_t ra = 2 * gp, rb = 2 * gp + 1;
            if (ya > best_v || (ya == best_v && ra < best_i)) { best_v = ya; best_i = ra; }
            if (yb > best_v || (yb == best_v && rb < best_i)) { best_v = yb; best_i = rb; }
            return make_float2(ya, yb);
          },
          [&](int32_t gp, int h, float v) {
            if (lo) lo[2 * gp + h] = v;
          });
      tbase += (uint32_t)(pl.np[ST_LM] * pl.kt[ST_LM]);
    }
    // combine the 4 waves' candidates, publish this WG's (value, index)
    C.csync();
    if (lane == 0) {
      L.scr[2 * c] = best_v;
      L.scr[2 * c + 1] = __int_as_float(best_i);
    }
    C.csync();
    if (C.tid == 0) {
      float bv = L.scr[0];
      int32_t bi = __float_as_int(L.scr[1]);
      for (int k = 1; k < kConsumerWaves; ++k) {
        const float v = L.scr[2 * k];
        const int32_t i = __float_as_int(L.scr[2 * k + 1]);
        if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
      }
      st_x(ex + X.lm + 2 * pl.w, tag_f(bv, ep));
      st_x(ex + X.lm + 2 * pl.w + 1, tag_u((uint32_t)bi, ep));
    }
    C.csync();
    // every WG gathers all candidates (this is also the step's grid-wide synchronisation)
    const uint64_t tsm = TR_NOW();
    C.fetch(ex + X.lm, 2 * s.nwg, L.scr, ep, false);
    C.tr.add(TC_SAMPLE, TR_NOW() - tsm);
    if (C.fail) break;
    int32_t next = 0;
    {
      // argmax over nwg candidates; each thread scans a strided subset, then a fixed-order merge
      float bv = -INFINITY;
      int32_t bi = 0x7fffffff;
      for (int k = C.tid; k < s.nwg; k += kConsumerThreads) {
        const float v = L.scr[2 * k];
        const int32_t i = __float_as_int(L.scr[2 * k + 1]);
        if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int32_t oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      C.csync();
      if (lane == 0) {
        L.scr[2 * c] = bv;
        L.scr[2 * c + 1] = __int_as_float(bi);
      }
      C.csync();
      bv = L.scr[0];
      bi = __float_as_int(L.scr[1]);
      for (int k = 1; k < kConsumerWaves; ++k) {
        const float v = L.scr[2 * k];
        const int32_t i = __float_as_int(L.scr[2 * k + 1]);
        if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
      }
      next = clamp_token(bi, s.V);
      C.csync();
    }
    if (lm && pl.w == 0 && C.tid == 0) {
      if (P.tokens_out) P.tokens_out[step] = next;
      if (P.last_tok_out && step == P.n_steps - 1) P.last_tok_out[0] = next;
    }
    if (P.forced && step + 1 < P.n_steps) {
      if (C.tid == 0) {
        int32_t f = P.forced[step];
        if (f < 0 || f >= s.V) {
          if (pl.w == 0) __hip_atomic_fetch_or(P.err, KERR_BAD_TOKEN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          f = 0;
        }
        L.scr[0] = __int_as_float(f);
      }
      C.csync();
      next = clamp_token(__float_as_int(L.scr[0]), s.V);
      C.csync();
    }
    tok = next;
  }
  C.tr.add(TC_TOTAL, TR_NOW() - t_start);
  C.tr.flush(P.trace + ((int64_t)pl.w * (kThreads / kWave) + kProducerWaves + c) * kTraceWords, lane);
  if (C.fail) raise_error(P, L, KERR_CONSUMER);
}

template <int G, int HD>
__global__ void __launch_bounds__(kThreads, 1) kie_decode_kernel(KParams P) {
  extern __shared__ __align__(16) uint8_t smem[];
  const Lds L = lds_map(smem, P.s, P.ring_slots);
  if (threadIdx.x < C_COUNT) L.ctl[threadIdx.x] = 0;
  __syncthreads();
  const Plan pl = make_plan(P, blockIdx.x);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int lane = threadIdx.x % kWave;
  if (wave < kProducerWaves)
    producer(P, L, pl, wave, lane);
  else
    consumer<G, HD>(P, L, pl, wave - kProducerWaves, lane);
}

// Instantiations for the supported (group size, head_dim) combinations.
KernelFn decode_kernel_for(int G, int HD) {
  if (HD == 128) {
    switch (G) {
      case 1: return kie_decode_kernel<1, 128>;
      case 2: return kie_decode_kernel<2, 128>;
      case 4: return kie_decode_kernel<4, 128>;
      case 8: return kie_decode_kernel<8, 128>;
    }
  } else if (HD == 64) {
    switch (G) {
      case 1: return kie_decode_kernel<1, 64>;
      case 2: return kie_decode_kernel<2, 64>;
      case 4: return kie_decode_kernel<4, 64>;
      case 8: return kie_decode_kernel<8, 64>;
    }
  }
  return nullptr;
}

}  // namespace kie
