// layout.h -- where every weight byte and every exchange word lives (host and device).
//
// Decoding one token at batch 1 streams every active weight once (agentlenshq.com,
// 《突破内存墙：在标准 GPU 上实现 3,000 tokens/s 的推理速度》, "瓶颈：是内存带宽，而非计算"). The packer
// therefore lays the weights out in exactly the order in which each wave of the persistent kernel
// consumes them within one token: every wave streams one contiguous slice with 16-byte lane loads
// and can issue its next loads before the inputs they will be multiplied with exist.
//
// Vocabulary
//   WG       one persistent workgroup of 8 waves per compute unit.
//   pair     two weight rows (A, B) that one wave reduces together: RoPE partners, gate/up
//            partners, or neighbours. Their dot products share every activation load.
//   tile     1 KiB = 64 lanes x 16 B covering 256 consecutive k of both rows: lane l holds
//            A[4l..4l+3] then B[4l..4l+3] (bf16, little-endian pairs). K is a multiple of 256.
//   unit     (pair, k-slice): ks consecutive k-tiles of one pair, ks = 8 when the row has a
//            multiple of 8 tiles (else 4, 2 or 1); a pair of kt tiles has S = kt / ks units.
//   batch    8 tile slots = 8 / ks units of one wave; the unit of a WG's stage with index u
//            belongs to wave u mod 8. Slots of a missing unit are zero tiles.
//   stream   one wave's batches for a whole token: L x [QKV, O, GU, DN], then the LM head.
//
// Mixture-of-experts layers (E > 0) stream L x [QKV, O, RT] (RT: the router's E rows), then the
// LM head. Which experts a token needs is known only after the router, so their gate/up and down
// tiles cannot sit in a fixed stream: they live in an expert region, per (layer, expert), where a
// wave finds the tiles of its units once the experts are chosen. The stages over the A chosen
// experts have the dense geometry with F = A x Fe: gate/up pair g is row g mod Fe of chosen
// expert g / Fe, and the down projection's K runs over the chosen experts' Fe columns in turn.
#pragma once
#include <stdint.h>

#ifdef __HIPCC__
#define KIE_HD __host__ __device__ __forceinline__
#else
#define KIE_HD inline
#endif

namespace kie {

constexpr int kWave = 64;
constexpr int kWaves = 8;  // per WG
constexpr int kThreads = kWaves * kWave;  // 512
constexpr int kTileBytes = 1024;
constexpr int kTileK = 256;  // k per tile and row
constexpr int kBatch = 8;    // tile slots per batch
constexpr int kMaxWG = 1024;
constexpr int kMaxUnits = 2048;  // units of one stage per WG (LDS partial sums)
constexpr int kMaxTopK = 64;     // largest k of top-k sampling
// Exchange words each thread of the decode kernel has in flight per pass of the FFN-width gather
// (the other gathers take 8): 16 * 512 covers the FFN widths of the models here in one pass.
constexpr int kGatherH = 16;

enum Stage : int { ST_QKV = 0, ST_O = 1, ST_RT = 2, ST_GU = 3, ST_DN = 4, ST_LM = 5, ST_COUNT = 6 };
constexpr int kMaxActive = 8;  // most experts routed per token

struct Shape {
  int32_t L, d, nq, nkv, hd, F, V, max_seq;  // F: FFN width (A x Fe for a mixture of experts)
  float eps, theta;
  int32_t nwg;
  int32_t E, A, Fe;  // experts, routed per token, FFN width of one expert (E == 0: dense)
  KIE_HD bool moe() const { return E > 0; }
  KIE_HD int32_t qdim() const { return nq * hd; }
  KIE_HD int32_t kvdim() const { return nkv * hd; }
  KIE_HD int32_t group() const { return nq / nkv; }
  // whether a stage's tiles are part of the fixed per-wave streams
  KIE_HD bool in_stream(int st) const { return !(moe() && (st == ST_GU || st == ST_DN)); }
  // pairs and row length (K) of each stage
  KIE_HD int32_t stage_pairs(int st) const {
    switch (st) {
      case ST_QKV: return (nq + 2 * nkv) * (hd / 2);
      case ST_O: return d / 2;
      case ST_RT: return E / 2;
      case ST_GU: return F;
      case ST_DN: return d / 2;
      default: return V / 2;
    }
  }
  KIE_HD int32_t stage_k(int st) const {
    switch (st) {
      case ST_O: return qdim();
      case ST_DN: return F;
      default: return d;
    }
  }
  // k-tiles of a row: TK weights per tile row (kTileK for bf16; 8-bit weights pack 2 * kTileK)
  template <int TK = kTileK>
  KIE_HD int32_t stage_kt(int st) const { return stage_k(st) / TK; }
};

// Even split of n items over nwg workgroups: WG w owns [begin, end).
KIE_HD int32_t split_begin(int64_t n, int32_t nwg, int32_t w) { return (int32_t)((n * w) / nwg); }
KIE_HD int32_t split_end(int64_t n, int32_t nwg, int32_t w) { return (int32_t)((n * (w + 1)) / nwg); }

// Chiplet-major order of the workgroups. The dispatcher hands consecutive workgroups to the 8
// chiplets (XCDs) in turn, so the workgroups with one value of w mod 8 share a chiplet (which one
// can change from launch to launch). rank(w) = (w mod 8) * (nwg / 8) + w / 8 numbers those of
// residue 0 first, then those of residue 1, and so on (the identity where nwg is not a multiple of
// 8): work split over the ranks in order keeps neighbouring shares on one chiplet. Placement only:
// any bijection is correct.
constexpr int kXcds = 8;
KIE_HD int32_t xcd_rank(int32_t nwg, int32_t w) {
  return nwg % kXcds ? w : (w % kXcds) * (nwg / kXcds) + w / kXcds;
}
KIE_HD int32_t xcd_wg(int32_t nwg, int32_t r) {  // the inverse of xcd_rank
  return nwg % kXcds ? r : (r % (nwg / kXcds)) * kXcds + r / (nwg / kXcds);
}

// k-tiles per unit for a row of kt tiles
KIE_HD int32_t unit_tiles(int32_t kt) { return kt % 8 == 0 ? 8 : (kt % 4 == 0 ? 4 : (kt % 2 == 0 ? 2 : 1)); }

// One stage of one WG: its pairs and how they are cut into units and batches.
struct StageGeo {
  int32_t pb, np;   // first position, positions owned (a position is a pair; see stage_pair)
  int32_t kt, ks;   // k-tiles per pair, per unit
  int32_t S;        // units per pair
  int32_t upb;      // units per batch (8 / ks)
  int32_t nu;       // units of the WG (np * S)
};
// The QKV stage orders its pairs by KV group -- the query heads of group j, then K head j, then V
// head j -- and splits them over the workgroups in chiplet-major order: with 8 KV groups and a
// multiple of 8 workgroups, group j is computed by the workgroups w = j mod 8, the chiplet where
// the attention of KV head j runs (att_info), so its queries, key and value stay on one chiplet.
// Position p of the QKV stage is pair qkv_pair(p); the other stages take pair p at position p.
KIE_HD int32_t qkv_pair(const Shape& s, int32_t p) {
  const int32_t half = s.hd / 2, G = s.group();
  const int32_t per = (G + 2) * half;  // pairs of one KV group
  const int32_t j = p / per, t = p % per, slot = t / half;
  const int32_t hs = slot < G ? j * G + slot : (slot == G ? s.nq + j : s.nq + s.nkv + j);
  return hs * half + t % half;
}
KIE_HD int32_t qkv_position(const Shape& s, int32_t gp) {  // the inverse of qkv_pair
  const int32_t half = s.hd / 2, G = s.group();
  const int32_t hs = gp / half, i = gp % half;
  int32_t j, slot;
  if (hs < s.nq) {
    j = hs / G;
    slot = hs % G;
  } else if (hs < s.nq + s.nkv) {
    j = hs - s.nq;
    slot = G;
  } else {
    j = hs - s.nq - s.nkv;
    slot = G + 1;
  }
  return j * (G + 2) * half + slot * half + i;
}
KIE_HD int32_t stage_pair(const Shape& s, int st, int32_t p) { return st == ST_QKV ? qkv_pair(s, p) : p; }
template <int TK = kTileK>
KIE_HD StageGeo stage_geo(const Shape& s, int st, int32_t w) {
  StageGeo g;
  const int32_t n = s.stage_pairs(st);
  const int32_t r = st == ST_QKV ? xcd_rank(s.nwg, w) : w;
  g.pb = split_begin(n, s.nwg, r);
  g.np = split_end(n, s.nwg, r) - g.pb;
  g.kt = s.stage_kt<TK>(st);
  g.ks = unit_tiles(g.kt);
  g.S = g.kt / g.ks;
  g.upb = kBatch / g.ks;
  g.nu = g.np * g.S;
  return g;
}
// units of wave v (u = v, v + 8, ...) and its batches
KIE_HD int32_t wave_units(const StageGeo& g, int32_t v) { return g.nu > v ? (g.nu - v + kWaves - 1) / kWaves : 0; }
KIE_HD int32_t wave_batches(const StageGeo& g, int32_t v) { return (wave_units(g, v) + g.upb - 1) / g.upb; }

// Batches of one layer in the stream of (WG w, wave v), and of the LM head. (TK: as stage_kt; a
// tile is kTileBytes either way, 2 rows of TK weights.)
template <int TK = kTileK>
KIE_HD int32_t layer_batches(const Shape& s, int32_t w, int32_t v) {
  int32_t b = 0;
  for (int st = ST_QKV; st <= ST_DN; ++st)
    if (s.in_stream(st)) b += wave_batches(stage_geo<TK>(s, st, w), v);
  return b;
}
template <int TK = kTileK>
KIE_HD int32_t lm_batches(const Shape& s, int32_t w, int32_t v) { return wave_batches(stage_geo<TK>(s, ST_LM, w), v); }
template <int TK = kTileK>
KIE_HD int64_t stream_tiles(const Shape& s, int32_t w, int32_t v) {
  return ((int64_t)s.L * layer_batches<TK>(s, w, v) + lm_batches<TK>(s, w, v)) * kBatch;
}

// Source rows of global pair gp of a stage. mat selects the matrix: for QKV 0 = Wq, 1 = Wk, 2 = Wv.
// (The router's pairs are neighbouring rows, like O, DN and the LM head.)
KIE_HD void pair_rows(const Shape& s, int st, int32_t gp, int* mat, int32_t* ra, int32_t* rb) {
  if (st == ST_QKV) {
    const int32_t half = s.hd / 2;
    const int32_t hs = gp / half, i = gp % half;
    int32_t h = hs;
    if (hs < s.nq) {
      *mat = 0;
    } else if (hs < s.nq + s.nkv) {
      *mat = 1;
      h = hs - s.nq;
    } else {
      *mat = 2;
      h = hs - s.nq - s.nkv;
    }
    *ra = h * s.hd + i;
    *rb = h * s.hd + i + half;
  } else if (st == ST_GU) {
    *mat = 0;  // row gp of W_gate (A) and of W_up (B)
    *ra = gp;
    *rb = gp;
  } else {
    *mat = 0;
    *ra = 2 * gp;
    *rb = 2 * gp + 1;
  }
}

// LM-head rows of the WG that owns the most of them (an even split never gives more than this)
KIE_HD int32_t lm_rows_max(const Shape& s) { return 2 * ((s.V / 2 + s.nwg - 1) / s.nwg); }

// Top-k merge of the per-WG candidate lists, in floats of WG-local memory (16-byte aligned
// pieces): the list heads [nwg][2], the selected lists [nsel], their active lengths [nsel] and
// offsets [nsel + 1], the merged top k [k][2], the selected lists' entries [nsel][ke][2] and the
// compacted active entries (as many), where nsel = min(k, nwg) and ke = min(k, lm_rows_max).
struct TopkLayout {
  int32_t nsel, ke;
  int32_t heads, sel, alen, off, top, ent, cmp, total;
};
KIE_HD int32_t align4(int32_t x) { return (x + 3) & ~3; }
KIE_HD TopkLayout topk_layout(const Shape& s, int32_t k) {
  TopkLayout t;
  const int32_t lr = lm_rows_max(s);
  t.nsel = k < s.nwg ? k : s.nwg;
  t.ke = k < lr ? k : lr;
  int32_t o = 0;
  t.heads = o; o = align4(o + 2 * s.nwg);
  t.sel = o; o = align4(o + t.nsel);
  t.alen = o; o = align4(o + t.nsel);
  t.off = o; o = align4(o + t.nsel + 1);
  t.top = o; o = align4(o + 2 * k);
  t.ent = o; o = align4(o + 2 * t.nsel * t.ke);
  t.cmp = o; o = align4(o + 2 * t.nsel * t.ke);
  t.total = o;
  return t;
}
KIE_HD int32_t topk_merge_floats(const Shape& s, int32_t k) { return topk_layout(s, k).total; }

// ---------------------------------------------------------------------------------------------
// Attention split: WG w handles KV head (w mod nkv) over position chunk (w / nkv).
// ---------------------------------------------------------------------------------------------
KIE_HD int32_t att_chunks(const Shape& s) { return s.nwg / s.nkv; }
KIE_HD int32_t att_pos_per_tile(const Shape& s) { return kTileBytes / (s.hd * 2); }
// chunk length (positions) for a context of n positions; a multiple of the positions per tile
KIE_HD int32_t att_chunk_len(const Shape& s, int32_t n) {
  const int32_t nc = att_chunks(s), ppt = att_pos_per_tile(s);
  int32_t cs = (n + nc - 1) / nc;
  cs = ((cs + ppt - 1) / ppt) * ppt;
  return cs < ppt ? ppt : cs;
}
// merge units: (query head, slice of kMergeDims dims), split over the workgroups in chiplet-major
// order (xcd_rank), so that the units of KV group j's query heads sit on chiplet j with that
// group's attention partials. merge_unit_rank(u) is the rank of unit u's workgroup.
constexpr int kMergeDims = 8;
KIE_HD int32_t merge_units(const Shape& s) { return s.nq * (s.hd / kMergeDims); }
KIE_HD int32_t merge_unit_rank(const Shape& s, int32_t u) { return (int32_t)(((int64_t)u * s.nwg) / merge_units(s)); }

// ---------------------------------------------------------------------------------------------
// Exchange buffers (64-bit tagged words: value bits << 32 | epoch), per layer, in the workspace.
// ---------------------------------------------------------------------------------------------
struct Exch {
  int64_t xf, xa, q, k, v, part, o, h, rt, lm, end;  // word offsets
  int32_t part_words;                             // per WG per layer
};
KIE_HD Exch exch_layout(const Shape& s) {
  Exch e;
  const int32_t G = s.group();
  e.part_words = G * (s.hd + 2);
  int64_t o = 0;
  e.xf = o; o += (int64_t)(s.L + 1) * s.d;
  e.xa = o; o += (int64_t)s.L * s.d;
  e.q = o; o += (int64_t)s.L * s.qdim();
  e.k = o; o += (int64_t)s.L * s.kvdim();
  e.v = o; o += (int64_t)s.L * s.kvdim();
  e.part = o; o += (int64_t)s.L * s.nwg * e.part_words;
  e.o = o; o += (int64_t)s.L * s.qdim();
  e.h = o; o += (int64_t)s.L * s.F;
  e.rt = o; o += (int64_t)s.L * s.E;  // router logits
  e.lm = o; o += (int64_t)kMaxTopK * s.nwg * 2;  // [rank][WG][value, id] sampling candidates
  e.end = o;
  return e;
}

// Prompt pass scratch: positions per chunk, and the widest GEMM input and output rows.
constexpr int kPrefillChunk = 512;
constexpr int kPrefillAttnSeg = 2048;  // key positions per attention block of the prompt pass
KIE_HD int32_t prefill_attn_segs(const Shape& s) { return (s.max_seq + kPrefillAttnSeg - 1) / kPrefillAttnSeg; }
KIE_HD int32_t prefill_kmax(const Shape& s) {
  int32_t k = s.d;
  if (s.qdim() > k) k = s.qdim();
  if (s.F > k) k = s.F;
  return k;
}
KIE_HD int32_t prefill_nmax(const Shape& s) {
  int32_t n = 2 * s.stage_pairs(ST_QKV);
  if (2 * s.F > n) n = 2 * s.F;
  if (s.d > n) n = s.d;
  return n;
}

// The prompt pass's tile table: for every layer, stage of the fixed streams (QKV, O, the router,
// gate/up, down), pair and unit (a run of consecutive k-tiles of one pair, unit_tiles long), the
// unit's first tile in the packed image as packed_tile gives it, so that the prompt pass's GEMMs
// look the placement up instead of recomputing it (int32: the image holds fewer than 2^31 tiles).
template <int TK = kTileK>
KIE_HD int32_t ptab_units(const Shape& s, int st) {  // entries of one stage of one layer
  if (!s.in_stream(st)) return 0;
  const int32_t kt = s.stage_kt<TK>(st);
  return s.stage_pairs(st) * (kt / unit_tiles(kt));
}
template <int TK = kTileK>
KIE_HD int64_t ptab_layer(const Shape& s) {
  int64_t n = 0;
  for (int st = ST_QKV; st <= ST_DN; ++st) n += ptab_units<TK>(s, st);
  return n;
}
template <int TK = kTileK>
KIE_HD int64_t ptab_index(const Shape& s, int st, int32_t l, int32_t gp, int32_t unit) {
  int64_t o = (int64_t)l * ptab_layer<TK>(s);
  for (int st2 = ST_QKV; st2 < st; ++st2) o += ptab_units<TK>(s, st2);
  const int32_t kt = s.stage_kt<TK>(st);
  return o + (int64_t)gp * (kt / unit_tiles(kt)) + unit;
}
// Workspace (bytes, 256-aligned pieces): exchange words, RoPE table [max_seq][hd/2] of (cos,sin),
// per-stream base (in tiles, [nwg][8] + total), error word, norm gains [L][2][d] + final [d] (bf16),
// trace counters, the prompt-pass scratch (residual [chunk][d] fp32, GEMM input [2][chunk][kmax]
// bf16, down-projection input [2][chunk][F] bf16, split-K partial sums [chunk][nmax] fp32, queries
// [chunk][nq hd] fp32, for long contexts the per-segment attention states
// [segments][chunk][nq][hd + 2] fp32, with experts moe_prefill_layout's pieces, and the tile table
// of ptab_index, int32), and the matrix scales of 8-bit weights [L][7] + [1] fp32.
struct Workspace {
  int64_t exch, rope, wbase, err, norms, trace, px, pa3, ph2, pc, pq, pattn, pmoe, ptab, wscale, end;
};
constexpr int kTraceWords = 64;  // per wave: cycle counters of a KIE_TRACE build (0..31), and the
                                 // hop timeline of one sampled layer (32..63, wave 0 only)
constexpr int kTraceHop = 32;    // first word of the hop timeline
KIE_HD int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }
// The mixture-of-experts part of the prompt pass's scratch (one chunk of positions): router logits
// [chunk][E] fp32; per position its A chosen experts [chunk][A] int32 in rank order, their
// weights [chunk][A] fp32 and each choice's place in its expert's token list [chunk][A] int32;
// the token lists [E][chunk] int32 (position << 4 | rank); the lists' lengths [E] and first rows
// [E] int32; the experts' down-projection rows [chunk * A][d] fp32 (expert e's rows from its
// first row on, in list order).
struct MoePrefill {
  int64_t logits, sel, wt, place, lists, counts, offs, y, end;
};
KIE_HD MoePrefill moe_prefill_layout(const Shape& s) {
  MoePrefill m;
  const int64_t C = kPrefillChunk;
  int64_t o = 0;
  m.logits = o; o = align256(o + C * s.E * 4);
  m.sel = o; o = align256(o + C * s.A * 4);
  m.wt = o; o = align256(o + C * s.A * 4);
  m.place = o; o = align256(o + C * s.A * 4);
  m.lists = o; o = align256(o + (int64_t)s.E * C * 4);
  m.counts = o; o = align256(o + (int64_t)s.E * 4);
  m.offs = o; o = align256(o + (int64_t)s.E * 4);
  m.y = o; o = align256(o + C * s.A * s.d * 4);
  m.end = o;
  return m;
}
// prefill == false: without the matrix-core prompt pass's scratch (a context whose prompt runs
// through the decode program); px .. pmoe are then empty pieces at the end of the rest.
KIE_HD Workspace workspace_layout(const Shape& s, bool prefill = true) {
  Workspace w;
  int64_t o = 0;
  w.exch = o; o = align256(o + exch_layout(s).end * 8);
  w.rope = o; o = align256(o + (int64_t)s.max_seq * (s.hd / 2) * 8);
  w.wbase = o; o = align256(o + ((int64_t)s.nwg * kWaves + 1) * 8);
  w.err = o; o = align256(o + 64);
  w.norms = o; o = align256(o + ((int64_t)s.L * 2 + 1) * s.d * 2);
  w.trace = o; o = align256(o + (int64_t)s.nwg * kWaves * kTraceWords * 8);
  w.wscale = o; o = align256(o + ((int64_t)s.L * 7 + 1) * 4);  // 8-bit weights: the matrix scales
  if (!prefill) {
    w.px = w.pa3 = w.ph2 = w.pc = w.pq = w.pattn = w.pmoe = w.ptab = w.end = o;
    return w;
  }
  w.px = o; o = align256(o + (int64_t)kPrefillChunk * s.d * 4);
  w.pa3 = o; o = align256(o + (int64_t)2 * kPrefillChunk * prefill_kmax(s) * 2);
  w.ph2 = o; o = align256(o + (int64_t)2 * kPrefillChunk * s.F * 2);
  w.pc = o; o = align256(o + (int64_t)kPrefillChunk * prefill_nmax(s) * 4);
  w.pq = o; o = align256(o + (int64_t)kPrefillChunk * s.qdim() * 4);
  w.pattn = o;
  if (prefill_attn_segs(s) > 1) o = align256(o + (int64_t)prefill_attn_segs(s) * kPrefillChunk * s.nq * (s.hd + 2) * 4);
  w.pmoe = o;
  if (s.moe()) o = align256(o + moe_prefill_layout(s).end);
  w.ptab = o;
  {  // sized for either weight format (tiles of 256 bf16 or 512 8-bit weights per row)
    const int64_t a = ptab_layer<kTileK>(s), b = ptab_layer<2 * kTileK>(s);
    o = align256(o + (int64_t)s.L * (a > b ? a : b) * 4);
  }
  w.end = o;
  return w;
}

// Packed image: the streams of (WG 0, wave 0), (WG 0, wave 1), ..., (WG nwg-1, wave 7), the
// expert region (mixture of experts), then the embedding table [V][d] bf16 as is.
template <int TK = kTileK>
KIE_HD int64_t packed_stream_tiles(const Shape& s) {
  int64_t t = 0;
  for (int32_t w = 0; w < s.nwg; ++w)
    for (int32_t v = 0; v < kWaves; ++v) t += stream_tiles<TK>(s, w, v);
  return t;
}
// Expert region, in tiles from its start: gate/up tiles [L][E][Fe pairs][d / 256] (pair p = row p
// of the expert's W_gate (A) and W_up (B)), then down tiles [L][d / 2 pairs][E][Fe / 256] (pair p
// = rows 2p, 2p + 1 of the expert's W_down). A WG's gate/up share lies in one expert, so its
// tiles are contiguous; its down share (the same output rows in every chosen expert) spans all
// experts, so the experts are the inner index there and its tiles stay within one short span.
KIE_HD int64_t expert_gu_tile(const Shape& s, int32_t l, int32_t e, int32_t p, int32_t kt) {
  return (((int64_t)l * s.E + e) * s.Fe + p) * (s.d / kTileK) + kt;
}
KIE_HD int64_t expert_gu_tiles(const Shape& s) { return (int64_t)s.L * s.E * s.Fe * (s.d / kTileK); }
KIE_HD int64_t expert_dn_tile(const Shape& s, int32_t l, int32_t e, int32_t p, int32_t kt) {
  return expert_gu_tiles(s) + (((int64_t)l * (s.d / 2) + p) * s.E + e) * (s.Fe / kTileK) + kt;
}
KIE_HD int64_t expert_tiles(const Shape& s) { return s.moe() ? 2 * expert_gu_tiles(s) : 0; }
KIE_HD int64_t packed_expert_offset(const Shape& s) { return packed_stream_tiles(s) * kTileBytes; }
template <int TK = kTileK>
KIE_HD int64_t packed_embed_offset(const Shape& s) {
  return (packed_stream_tiles<TK>(s) + expert_tiles(s)) * kTileBytes;
}

// The share (rank or WG) owning position p of a stage with n positions (the inverse of the even
// split).
KIE_HD int32_t pair_owner(int64_t n, int32_t nwg, int32_t p) {
  int32_t w = (int32_t)(((int64_t)p * nwg) / n);
  while (w + 1 < nwg && split_begin(n, nwg, w + 1) <= p) ++w;
  while (w > 0 && split_begin(n, nwg, w) > p) --w;
  return w;
}
// Where k-tile kt of pair gp of stage st in layer l lives in the packed image (in tiles); the LM
// head is st == ST_LM (l ignored). wbase[w * kWaves + v] is the first tile of stream (w, v). This
// inverts the packer's placement, so that a kernel can read the weights of any row in place.
// (Stages in the fixed streams only; TK as stage_geo: kTileK for bf16, 2 * kTileK for 8-bit.)
template <int TK = kTileK>
KIE_HD int64_t packed_tile(const Shape& s, const int64_t* wbase, int st, int32_t l, int32_t gp, int32_t kt) {
  const int32_t p = st == ST_QKV ? qkv_position(s, gp) : gp;
  const int32_t owner = pair_owner(s.stage_pairs(st), s.nwg, p);
  const int32_t w = st == ST_QKV ? xcd_wg(s.nwg, owner) : owner;
  const StageGeo g = stage_geo<TK>(s, st, w);
  const int32_t u = (p - g.pb) * g.S + kt / g.ks;
  const int32_t v = u % kWaves, m = u / kWaves;
  const int32_t b = m / g.upb, slot = (m % g.upb) * g.ks + kt % g.ks;
  int64_t bt;
  if (st == ST_LM) {
    bt = (int64_t)s.L * layer_batches<TK>(s, w, v);
  } else {
    bt = (int64_t)l * layer_batches<TK>(s, w, v);
    for (int st2 = ST_QKV; st2 < st; ++st2)
      if (s.in_stream(st2)) bt += wave_batches(stage_geo<TK>(s, st2, w), v);
  }
  return wbase[w * kWaves + v] + (bt + b) * kBatch + slot;
}
template <int TK = kTileK>
KIE_HD int64_t packed_bytes(const Shape& s) { return packed_embed_offset<TK>(s) + (int64_t)s.V * s.d * 2; }

// KV cache: [L][2][nkv][max_seq][hd] bf16 (K plane, then V plane, per layer).
KIE_HD int64_t kv_offset(const Shape& s, int32_t l, int32_t kv, int32_t j, int32_t pos) {
  return ((((int64_t)l * 2 + kv) * s.nkv + j) * s.max_seq + pos) * s.hd;
}
KIE_HD int64_t kv_bytes(const Shape& s) { return (int64_t)s.L * 2 * s.nkv * s.max_seq * s.hd * 2; }

}  // namespace kie
