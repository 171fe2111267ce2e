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
// Inter-WG exchange uses 64-bit tagged words (fp32 value << 32 | epoch) written and read with
// agent-scope atomics, so a reader knows a word is current by its tag alone: no grid barrier,
// no flag round trip, no L2 flush. Epochs are unique per decode step and buffers are per layer.
//
// Per layer the stages are: QKV (+RMSNorm, RoPE) -> attention over a chunk of positions of one
// KV head (split-K, online softmax) -> merge of the chunk partials -> O (+residual) -> gate/up
// (+RMSNorm, SwiGLU) -> down (+residual). Then the final RMSNorm + LM head and the sampler.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "layout.h"
#include "monokernel.h"

namespace kie {

// ------------------------------------------------------------------------------------------
// LDS layout
// ------------------------------------------------------------------------------------------
struct Lds {
  uint8_t* ring;      // R x 1 KiB
  uint32_t* ready;    // R : stream index + 1 of the tile the slot holds
  uint32_t* freed;    // R : stream index + 1 of the last tile consumed from the slot
  float* act;         // stage input vector (fp32)
  float* xres;        // residual stream of the current layer (fp32, d)
  float* scr;         // scratch for reductions / attention partials / sampler
  uint32_t* ctl;      // control words
};
enum Ctl : int { C_BAR = 0, C_STEP = 1, C_ABORT = 2, C_PDONE = 3, C_COUNT = 16 };

__host__ __device__ __forceinline__ int32_t act_floats(const Shape& s) {
  int32_t a = s.d;
  if (s.qdim() > a) a = s.qdim();
  if (s.F > a) a = s.F;
  if ((s.group() + 2) * s.hd > a) a = (s.group() + 2) * s.hd;
  return a;
}
__host__ __device__ __forceinline__ int32_t scr_floats(const Shape& s) {
  int32_t a = kConsumerWaves * s.group() * (s.hd + 2);
  if (8 * kMergeDims * 3 > a) a = 8 * kMergeDims * 3;
  if (2 * s.nwg > a) a = 2 * s.nwg;
  if (a < 64) a = 64;
  return a;
}
__host__ __device__ __forceinline__ int32_t lds_fixed_bytes(const Shape& s) {
  return (act_floats(s) + s.d + scr_floats(s)) * 4 + C_COUNT * 4;
}
int32_t lds_bytes_for(const Shape& s, int32_t ring) { return ring * (kTileBytes + 8) + lds_fixed_bytes(s); }
int32_t max_ring_slots(const Shape& s, int32_t lds_limit) {
  int32_t r = (lds_limit - lds_fixed_bytes(s)) / (kTileBytes + 8);
  r &= ~3;
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
  L.ready = (uint32_t*)p; p += (size_t)R * 4;
  L.freed = (uint32_t*)p; p += (size_t)R * 4;
  L.ctl = (uint32_t*)p;
  return L;
}

// ------------------------------------------------------------------------------------------
// Per-WG plan and the token stream's segments
// ------------------------------------------------------------------------------------------
struct Plan {
  int32_t w;
  int32_t pb[ST_COUNT];  // first global pair of each stage
  int32_t np[ST_COUNT];  // pairs owned
  int32_t kt[ST_COUNT];  // k-tiles per pair
  int32_t pre[ST_COUNT]; // tile offset of the stage inside one layer's weight stream (LM: 0)
  int32_t t_layer;       // weight tiles per layer
  int64_t wbase;         // first tile of this WG in the packed image
};

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

// Segment seg of a step: 0..5L-1 = (layer, kind) with kind 0 QKV, 1 ATT, 2 O, 3 GU, 4 DN;
// 5L = LM head (only when the step runs the LM head).
enum SegKind : int { SK_W = 0, SK_KV = 1 };
struct Seg {
  int32_t kind, len, layer;
  int64_t wofs;  // weights: tile offset inside this WG's token stream
};
__device__ __forceinline__ bool step_has_lm(const KParams& P, int32_t step) {
  return !P.lm_last_only || step == P.n_steps - 1;
}
__device__ __forceinline__ Seg seg_info(const KParams& P, const Plan& pl, const Att& at, int32_t step, int32_t seg) {
  Seg g;
  const int32_t L = P.s.L;
  if (seg == 5 * L) {
    g.kind = SK_W;
    g.layer = L;
    g.len = step_has_lm(P, step) ? pl.np[ST_LM] * pl.kt[ST_LM] : 0;
    g.wofs = (int64_t)L * pl.t_layer;
    return g;
  }
  const int32_t l = seg / 5, k = seg % 5;
  g.layer = l;
  if (k == 1) {
    g.kind = SK_KV;
    g.len = 2 * at.nkt;
    g.wofs = 0;
    return g;
  }
  const int st = k == 0 ? ST_QKV : (k == 2 ? ST_O : (k == 3 ? ST_GU : ST_DN));
  g.kind = SK_W;
  g.len = pl.np[st] * pl.kt[st];
  g.wofs = (int64_t)l * pl.t_layer + pl.pre[st];
  return g;
}

// ------------------------------------------------------------------------------------------
// Failure handling: every wait is bounded; on expiry the WG records an error and stops.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void raise_error(const KParams& P, const Lds& L, uint32_t code) {
  lds_st(&L.ctl[C_ABORT], 1u);
  __hip_atomic_fetch_or(P.err, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool aborted(const Lds& L) { return lds_ld(&L.ctl[C_ABORT]) != 0; }

// Bounded spin: call expired() after every unsuccessful poll. Every 256th call it checks the
// WG's abort flag, the grid's error word and the elapsed time of this wait.
struct Waiter {
  uint32_t spins = 0;
  uint64_t start = 0;
  __device__ __forceinline__ bool expired(const KParams& P, const Lds& L) {
    if ((++spins & 255u) != 0) return false;
    if (aborted(L)) return true;
    if (__hip_atomic_load(P.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return true;
    const uint64_t t = now_ticks();
    if (start == 0) {
      start = t;
      return false;
    }
    return t - start > (uint64_t)P.timeout_ticks;
  }
};

// ------------------------------------------------------------------------------------------
// Producer waves
// ------------------------------------------------------------------------------------------
constexpr int kProdDepth = 16;  // tiles in flight per producer wave

struct Cursor {
  uint32_t next;       // next stream index this producer will issue
  uint32_t seg_start;  // stream index of the current segment's first tile
  int32_t step, seg;
  Seg g;
  Att at;
  bool end;
};

__device__ __forceinline__ void cursor_load_seg(const KParams& P, const Plan& pl, Cursor& c) {
  if (c.seg == 0) c.at = att_info(P.s, pl.w, P.pos0 + c.step);
  c.g = seg_info(P, pl, c.at, c.step, c.seg);
}
__device__ __forceinline__ void cursor_seek(const KParams& P, const Plan& pl, Cursor& c) {
  // advance segments until `next` falls inside the current one
  while (!c.end && c.next >= c.seg_start + (uint32_t)c.g.len) {
    c.seg_start += (uint32_t)c.g.len;
    c.seg++;
    if (c.seg > 5 * P.s.L) {
      c.seg = 0;
      c.step++;
      if (c.step >= P.n_steps) {
        c.end = true;
        break;
      }
    }
    cursor_load_seg(P, pl, c);
  }
}

// Producer wave pw handles the WG's stream tiles pw, pw+4, pw+8, ...: it keeps kProdDepth of
// them in flight in registers and writes each into its ring slot once the slot's previous tile
// has been consumed. Tiles are written in the order they were issued. K/V tiles of step s are
// only issued once the consumers have started step s (their rows are final by then).
__device__ __forceinline__ void producer(const KParams& P, const Lds& L, const Plan& pl, int pw, int lane) {
  const uint32_t R = (uint32_t)P.ring_slots;
  const Shape& s = P.s;
  const int lpp = s.hd / 8;  // lanes per KV position
  const int ppt = att_pos_per_tile(s);
  Cursor cur;
  cur.next = (uint32_t)pw;
  cur.seg_start = 0;
  cur.step = 0;
  cur.seg = 0;
  cur.end = P.n_steps <= 0;
  if (!cur.end) cursor_load_seg(P, pl, cur);
  cursor_seek(P, pl, cur);

  v4u buf[kProdDepth];
#pragma unroll
  for (int u = 0; u < kProdDepth; ++u) buf[u] = v4u{0u, 0u, 0u, 0u};
  uint32_t valid = 0;                 // bit u: buf[u] holds an issued, unwritten tile
  uint32_t wr_next = (uint32_t)pw;    // stream index of the oldest unwritten tile
  uint32_t wr_slot = (uint32_t)pw % R;
  bool fail = false;

  while (!fail) {
    bool gated = false;
#pragma unroll
    for (int u = 0; u < kProdDepth; ++u) {
      if (!fail && (valid & (1u << u))) {
        if (wr_next >= R) {
          const uint32_t need = wr_next - R + 1;  // freed value that makes the slot free
          Waiter wt;
          while ((int32_t)(lds_ld(&L.freed[wr_slot]) - need) < 0) {
            __builtin_amdgcn_s_sleep(1);
            if (wt.expired(P, L)) {
              fail = true;
              break;
            }
          }
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        }
        if (!fail) {
          *(v4u*)(L.ring + wr_slot * kTileBytes + lane * 16) = buf[u];
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
          if (lane == 0) lds_st(&L.ready[wr_slot], wr_next + 1);
        }
        valid &= ~(1u << u);
        wr_next += kProducerWaves;
        wr_slot += kProducerWaves;
        if (wr_slot >= R) wr_slot -= R;
      }
      if (!fail && !cur.end && !gated) {
        const uint32_t t = cur.next - cur.seg_start;
        if (cur.g.kind == SK_KV && (int32_t)lds_ld(&L.ctl[C_STEP]) < cur.step) {
          gated = true;
        } else {
          v4u v = v4u{0u, 0u, 0u, 0u};
          if (cur.g.kind == SK_W) {
            const v4u* src = (const v4u*)(P.packed + (size_t)(pl.wbase + cur.g.wofs + t) * kTileBytes) + lane;
            v = __builtin_nontemporal_load(src);
          } else {
            const int32_t tp = (int32_t)(t >> 1), kvsel = (int32_t)(t & 1);
            const int32_t pos = cur.at.c0 + tp * ppt + lane / lpp;
            if (pos < cur.at.c0 + cur.at.ncache) {
              const v4u* src = (const v4u*)(P.kv + kv_offset(s, cur.g.layer, kvsel, cur.at.j, pos)) + (lane % lpp);
              v = *src;
            }
          }
          buf[u] = v;
          valid |= 1u << u;
          cur.next += kProducerWaves;
          cursor_seek(P, pl, cur);
        }
      }
    }
    if (fail) break;
    if (valid == 0) {
      if (cur.end) break;
      if (gated) {
        // drained: wait until the consumers have started the step
        Waiter wt;
        while ((int32_t)lds_ld(&L.ctl[C_STEP]) < cur.step) {
          __builtin_amdgcn_s_sleep(2);
          if (wt.expired(P, L)) {
            fail = true;
            break;
          }
        }
      }
    }
  }
  if (fail) raise_error(P, L, KERR_PRODUCER);
}

// ------------------------------------------------------------------------------------------
// Consumer waves
// ------------------------------------------------------------------------------------------
struct Cons {
  const KParams& P;
  const Lds& L;
  const Plan& pl;
  int c;        // consumer wave 0..3
  int lane;
  int tid;      // 0..255 among consumer threads
  uint32_t bar_target;
  bool fail;
  __device__ __forceinline__ Cons(const KParams& p, const Lds& l, const Plan& q, int c_, int lane_)
      : P(p), L(l), pl(q), c(c_), lane(lane_), tid(c_ * kWave + lane_), bar_target(0), fail(false) {}

  // barrier of the 4 consumer waves (LDS counter; the producers are not involved)
  __device__ __forceinline__ void csync() {
    fail = __builtin_amdgcn_ballot_w64(fail) != 0;  // one lane's failure is the wave's
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) __hip_atomic_fetch_add(&L.ctl[C_BAR], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    bar_target += kConsumerWaves;
    Waiter wt;
    while ((int32_t)(lds_ld(&L.ctl[C_BAR]) - bar_target) < 0) {
      __builtin_amdgcn_s_sleep(1);
      if (wt.expired(P, L)) {
        fail = true;
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }

  // wait until ring tile i is present
  __device__ __forceinline__ void wait_tile(int64_t i, int32_t slot) {
    const uint32_t want = (uint32_t)(i + 1);
    if (lds_ld(&L.ready[slot]) != want) {
      Waiter wt;
      while (lds_ld(&L.ready[slot]) != want) {
        __builtin_amdgcn_s_sleep(1);
        if (wt.expired(P, L)) {
          fail = true;
          return;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }
  // the slot's data has been read (its values are in registers): hand the slot back
  __device__ __forceinline__ void free_tile(int64_t i, int32_t slot) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) lds_st(&L.freed[slot], (uint32_t)(i + 1));
  }
  __device__ __forceinline__ int32_t slot_of(int64_t i) const { return (int32_t)((uint32_t)i % (uint32_t)P.ring_slots); }

  // Gather n tagged words with the given epoch from src into LDS floats dst. Every consumer
  // thread polls its words tid, tid+256, ... (all in flight at once), writes each value as soon
  // as its tag is current, and re-polls only the missing ones. If want_ss, returns the sum of
  // squares of the n values (fixed summation order) to every consumer thread.
  // The consumer barrier below is reached by every consumer thread, whatever its word count.
  __device__ __forceinline__ float fetch(const uint64_t* src, int n, float* dst, uint32_t epoch, bool want_ss) {
    constexpr int KMAX = 16;
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
            dp[k * kConsumerThreads] = __uint_as_float((uint32_t)(wv[k] >> 32));
          }
        }
        if (missing == 0 || fail) break;
        __builtin_amdgcn_s_sleep(1);
        if (wt.expired(P, L)) {
          fail = true;
          break;
        }
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
          if (missing & (1u << k)) wv[k] = ld_x(sp + k * kConsumerThreads);
      }
    }
    float ss = 0.f;
    if (want_ss) {
      for (int e = tid; e < n; e += kConsumerThreads) ss = fmaf(dst[e], dst[e], ss);
      ss = block_sum(ss);
    }
    csync();
    return ss;
  }

  // Gather up to three short ranges (query heads and the current K/V row) into LDS floats.
  __device__ __forceinline__ void fetch3(const uint64_t* s0, int n0, float* d0, const uint64_t* s1, int n1, float* d1,
                                         const uint64_t* s2, int n2, float* d2, uint32_t epoch) {
    constexpr int KM = 8;
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
        if (missing == 0 || fail) break;
        __builtin_amdgcn_s_sleep(1);
        if (wt.expired(P, L)) {
          fail = true;
          break;
        }
        reload();
      }
    }
    csync();
  }

  // sum over the 256 consumer threads, in a fixed order; every consumer thread gets the result
  __device__ __forceinline__ float block_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
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
      L.act[i] = (L.xres[i] * r) * gi;
    }
    csync();
  }

  // ------------------------------------------------------------------ GEMV stage
  // Each consumer wave takes pairs lp = c, c+4, ...; per tile, lane l multiplies its 8 bf16
  // weights by act[256 j + 8 (l mod 32) ...]; halves reduce to the pair's two dot products.
  template <typename Epi>
  __device__ __forceinline__ void gemv(int st, int64_t tile_base, Epi epi) {
    const int32_t np = pl.np[st], kt = pl.kt[st];
    const int ql = lane & 31;
    for (int32_t lp = c; lp < np && !fail; lp += kConsumerWaves) {
      float a0 = 0.f, a1 = 0.f;
      for (int32_t j = 0; j < kt; ++j) {
        const int64_t i = tile_base + tile_index(np, kt, lp, j);
        const int32_t slot = slot_of(i);
        wait_tile(i, slot);
        if (fail) return;
        const v4u w = *(const v4u*)(L.ring + (size_t)slot * kTileBytes + lane * 16);
        const float* ap = L.act + j * kTileK + ql * 8;
        const v4f x0 = *(const v4f*)ap;
        const v4f x1 = *(const v4f*)(ap + 4);
        a0 = fmaf(bf16lo(w.x), x0.x, a0);
        a1 = fmaf(bf16hi(w.x), x0.y, a1);
        a0 = fmaf(bf16lo(w.y), x0.z, a0);
        a1 = fmaf(bf16hi(w.y), x0.w, a1);
        a0 = fmaf(bf16lo(w.z), x1.x, a0);
        a1 = fmaf(bf16hi(w.z), x1.y, a1);
        a0 = fmaf(bf16lo(w.w), x1.z, a0);
        a1 = fmaf(bf16hi(w.w), x1.w, a1);
        free_tile(i, slot);
      }
      float v = a0 + a1;
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
      const float ya = readlane_f(v, 0), yb = readlane_f(v, 32);
      epi(pl.pb[st] + lp, ya, yb);
    }
  }
};

// ------------------------------------------------------------------------------------------
// Attention for one KV head over this WG's chunk of positions (split-K with online softmax,
// exp2 domain), then the combine of the 4 consumer waves into one partial (m, l, acc[hd]) per
// query head of the group.
// ------------------------------------------------------------------------------------------
template <int G, int HD>
__device__ __forceinline__ void attention_chunk(Cons& C, const Att& at, int32_t l, int32_t pos, int64_t tile_base, uint32_t epoch) {
  const KParams& P = C.P;
  const Lds& L = C.L;
  const Shape& s = P.s;
  constexpr int LPP = HD / 8;      // lanes per position
  constexpr int PPT = 64 / LPP;    // positions per tile
  const int lane = C.lane;
  const int lpos = lane / LPP, dg = lane % LPP;
  const float* q = L.act;              // [G][HD]
  const float* kp = L.act + G * HD;    // current position's k (fp32, after RoPE)
  const float* vp = L.act + (G + 1) * HD;
  const float sc = 1.4426950408889634f / sqrtf((float)HD);

  float m[G], lsum[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    lsum[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }
  float qr[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const v4f a = *(const v4f*)(q + g * HD + dg * 8);
    const v4f b = *(const v4f*)(q + g * HD + dg * 8 + 4);
    qr[g][0] = a.x; qr[g][1] = a.y; qr[g][2] = a.z; qr[g][3] = a.w;
    qr[g][4] = b.x; qr[g][5] = b.y; qr[g][6] = b.z; qr[g][7] = b.w;
  }

  // one block of PPT positions: kv = 8 bf16 K values and 8 bf16 V values of this lane's position
  auto block = [&](v4u kw, v4u vw, bool valid) {
    float kf[8] = {bf16lo(kw.x), bf16hi(kw.x), bf16lo(kw.y), bf16hi(kw.y),
                   bf16lo(kw.z), bf16hi(kw.z), bf16lo(kw.w), bf16hi(kw.w)};
    float vf[8] = {bf16lo(vw.x), bf16hi(vw.x), bf16lo(vw.y), bf16hi(vw.y),
                   bf16lo(vw.z), bf16hi(vw.z), bf16lo(vw.w), bf16hi(vw.w)};
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(qr[g][e], kf[e], d);
#pragma unroll
      for (int o = LPP / 2; o >= 1; o >>= 1) d += __shfl_xor(d, o, 64);
      const float s2 = valid ? d * sc : -INFINITY;
      float mx = s2;
#pragma unroll
      for (int o = LPP; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      const float mn = fmaxf(m[g], mx);
      if (mn == -INFINITY) continue;  // nothing valid yet
      const float alpha = m[g] == -INFINITY ? 0.f : exp2f(m[g] - mn);
      const float pr = valid ? exp2f(s2 - mn) : 0.f;
      float ps = pr;
#pragma unroll
      for (int o = LPP; o < 64; o <<= 1) ps += __shfl_xor(ps, o, 64);
      lsum[g] = lsum[g] * alpha + ps;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(pr, vf[e], acc[g][e] * alpha);
      m[g] = mn;
    }
  };

  for (int32_t tp = C.c; tp < at.nkt && !C.fail; tp += kConsumerWaves) {
    const int64_t ik = tile_base + 2 * tp, iv = ik + 1;
    const int32_t sk = C.slot_of(ik), sv = C.slot_of(iv);
    C.wait_tile(ik, sk);
    C.wait_tile(iv, sv);
    if (C.fail) return;
    const v4u kw = *(const v4u*)(L.ring + (size_t)sk * kTileBytes + lane * 16);
    const v4u vw = *(const v4u*)(L.ring + (size_t)sv * kTileBytes + lane * 16);
    const int32_t p = at.c0 + tp * PPT + lpos;
    block(kw, vw, p < at.c0 + at.ncache);
    C.free_tile(ik, sk);
    C.free_tile(iv, sv);
  }
  // the current position: its K/V come from the exchange, rounded to bf16 like the cache
  if (at.has_p && C.c == (at.nkt % kConsumerWaves)) {
    v4u kw = v4u{0u, 0u, 0u, 0u}, vw = v4u{0u, 0u, 0u, 0u};
    if (lpos == 0) {
      uint32_t kb[8], vb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kb[e] = f32_to_bf16(kp[dg * 8 + e]);
        vb[e] = f32_to_bf16(vp[dg * 8 + e]);
      }
      kw = v4u{kb[0] | (kb[1] << 16), kb[2] | (kb[3] << 16), kb[4] | (kb[5] << 16), kb[6] | (kb[7] << 16)};
      vw = v4u{vb[0] | (vb[1] << 16), vb[2] | (vb[3] << 16), vb[4] | (vb[5] << 16), vb[6] | (vb[7] << 16)};
    }
    block(kw, vw, lpos == 0);
  }
  // reduce acc over the positions of a tile (lanes with the same dims)
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[g][e];
#pragma unroll
      for (int o = LPP; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
      acc[g][e] = v;
    }
  // wave partials -> LDS scratch [wave][g][HD + 2]
  C.csync();
  float* ws = L.scr + C.c * G * (HD + 2);
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
      ws[g * (HD + 2) + HD + 1] = lsum[g];
    }
  }
  C.csync();
  // combine the 4 waves; publish (acc[HD], m, l) per query head of the group
  uint64_t* part = P.ex + P.exo.part + ((int64_t)l * s.nwg + C.pl.w) * P.exo.part_words;
  for (int e = C.tid; e < G * (HD + 2); e += kConsumerThreads) {
    const int g = e / (HD + 2), k = e % (HD + 2);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kConsumerWaves; ++w) M = fmaxf(M, L.scr[w * G * (HD + 2) + g * (HD + 2) + HD]);
    float out = 0.f;
    if (k == HD) {
      out = M;
    } else {
#pragma unroll
      for (int w = 0; w < kConsumerWaves; ++w) {
        const float mw = L.scr[w * G * (HD + 2) + g * (HD + 2) + HD];
        const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
        const float v = k == HD + 1 ? L.scr[w * G * (HD + 2) + g * (HD + 2) + HD + 1]
                                    : L.scr[w * G * (HD + 2) + g * (HD + 2) + k];
        out = fmaf(v, f, out);
      }
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
    while (todo) {
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
      if (todo) {
        __builtin_amdgcn_s_sleep(1);
        if (wt.expired(P, L)) {
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
  const Shape& s = P.s;
  const Exch& X = P.exo;
  uint64_t* ex = P.ex;
  int64_t tbase = 0;  // stream index of the next segment's first tile
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
        const float2* rope = P.rope + (int64_t)pos * (s.hd / 2);
        uint64_t* qx = ex + X.q + (int64_t)l * s.qdim();
        uint64_t* kx = ex + X.k + (int64_t)l * s.kvdim();
        uint64_t* vx = ex + X.v + (int64_t)l * s.kvdim();
        C.gemv(ST_QKV, tbase, [&](int32_t gp, float ya, float yb) {
          int mat;
          int32_t ra, rb;
          pair_rows(s, ST_QKV, gp, &mat, &ra, &rb);
          if (mat < 2) {
            const float2 cs = rope[gp % (s.hd / 2)];
            const float a = ya * cs.x - yb * cs.y;
            const float b = yb * cs.x + ya * cs.y;
            ya = a;
            yb = b;
          }
          uint64_t* dst = mat == 0 ? qx : (mat == 1 ? kx : vx);
          if (lane == 0) st_x(dst + ra, tag_f(ya, ep));
          if (lane == 1) st_x(dst + rb, tag_f(yb, ep));
        });
        tbase += (int64_t)pl.np[ST_QKV] * pl.kt[ST_QKV];
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
        attention_chunk<G, HD>(C, at, l, pos, tbase, ep);
        tbase += 2 * at.nkt;
      }
      // ---------------- merge of chunk partials (the WGs that own merge units)
      {
        const int32_t nu = merge_units(s);
        // units owned by this WG: u with merge_unit_wg(u) == w
        int32_t u0 = (int32_t)(((int64_t)pl.w * nu + s.nwg - 1) / s.nwg);
        for (int32_t u = u0; u < nu && merge_unit_wg(s, u) == pl.w && !C.fail; ++u) merge_unit(C, at, l, u, ep);
      }
      // ---------------- O projection + residual
      C.fetch(ex + X.o + (int64_t)l * s.qdim(), s.qdim(), L.act, ep, false);
      if (C.fail) break;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this WG's K/V rows are complete before its next outputs
      {
        uint64_t* xa = ex + X.xa + (int64_t)l * s.d;
        C.gemv(ST_O, tbase, [&](int32_t gp, float ya, float yb) {
          const int32_t ra = 2 * gp, rb = 2 * gp + 1;
          if (lane == 0) st_x(xa + ra, tag_f(L.xres[ra] + ya, ep));
          if (lane == 1) st_x(xa + rb, tag_f(L.xres[rb] + yb, ep));
        });
        tbase += (int64_t)pl.np[ST_O] * pl.kt[ST_O];
      }
      // ---------------- gate/up + SwiGLU
      C.csync();  // every wave has finished reading xres before it is replaced
      ss = C.fetch(ex + X.xa + (int64_t)l * s.d, s.d, L.xres, ep, true);
      C.rmsnorm_to_act(ss, P.norms + (int64_t)l * 2 * s.d + s.d);
      if (C.fail) break;
      {
        uint64_t* hx = ex + X.h + (int64_t)l * s.F;
        C.gemv(ST_GU, tbase, [&](int32_t gp, float ya, float yb) {
          const float hv = (ya / (1.0f + expf(-ya))) * yb;
          if (lane == 0) st_x(hx + gp, tag_f(hv, ep));
        });
        tbase += (int64_t)pl.np[ST_GU] * pl.kt[ST_GU];
      }
      // ---------------- down + residual
      C.csync();
      C.fetch(ex + X.h + (int64_t)l * s.F, s.F, L.act, ep, false);
      if (C.fail) break;
      {
        uint64_t* xf = ex + X.xf + (int64_t)(l + 1) * s.d;
        C.gemv(ST_DN, tbase, [&](int32_t gp, float ya, float yb) {
          const int32_t ra = 2 * gp, rb = 2 * gp + 1;
          if (lane == 0) st_x(xf + ra, tag_f(L.xres[ra] + ya, ep));
          if (lane == 1) st_x(xf + rb, tag_f(L.xres[rb] + yb, ep));
        });
        tbase += (int64_t)pl.np[ST_DN] * pl.kt[ST_DN];
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
      C.gemv(ST_LM, tbase, [&](int32_t gp, float ya, float yb) {
        const int32_t ra = 2 * gp, rb = 2 * gp + 1;
        if (lo) {
          if (lane == 0) lo[ra] = ya;
          if (lane == 1) lo[rb] = yb;
        }
        if (ya > best_v || (ya == best_v && ra < best_i)) { best_v = ya; best_i = ra; }
        if (yb > best_v || (yb == best_v && rb < best_i)) { best_v = yb; best_i = rb; }
      });
      tbase += (int64_t)pl.np[ST_LM] * pl.kt[ST_LM];
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
    C.fetch(ex + X.lm, 2 * s.nwg, L.scr, ep, false);
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
  if (C.fail) raise_error(P, L, KERR_CONSUMER);
}

template <int G, int HD>
__global__ void __launch_bounds__(kThreads, 1) kie_decode_kernel(KParams P) {
  extern __shared__ __align__(16) uint8_t smem[];
  const Lds L = lds_map(smem, P.s, P.ring_slots);
  for (int i = threadIdx.x; i < P.ring_slots; i += blockDim.x) {
    L.ready[i] = 0;
    L.freed[i] = 0;
  }
  if (threadIdx.x < C_COUNT) L.ctl[threadIdx.x] = 0;
  __syncthreads();
  const Plan pl = make_plan(P, blockIdx.x);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (wave < kProducerWaves)
    producer(P, L, pl, wave, lane);
  else
    consumer<G, HD>(P, L, pl, wave - kProducerWaves, lane);
}

// Instantiations for the supported (group size, head_dim) combinations.
typedef void (*KernelFn)(KParams);
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
