// Host-side check of the packed-stream geometry in layout.h: for every workgroup and stage, the
// batches of the 8 waves cover each (pair, k-tile) exactly once, unit slots beyond the stage stay
// empty, and the stream lengths add up to the packed image. With mixture-of-experts layers, the
// expert region's placement is checked to be one-to-one as well. Prints "ok" or the first
// violation.
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "layout.h"

using namespace kie;

template <int TK>
static int check(const Shape& s) {
  int64_t total = 0;
  for (int32_t w = 0; w < s.nwg; ++w) {
    for (int st = ST_QKV; st < ST_COUNT; ++st) {
      const StageGeo g = stage_geo<TK>(s, st, w);
      if (g.ks * g.S != g.kt || g.upb * g.ks != kBatch || g.kt * TK != s.stage_k(st)) {
        std::printf("bad unit geometry w=%d st=%d\n", w, st);
        return 1;
      }
      std::vector<int> seen((size_t)g.np * g.kt, 0);
      for (int32_t v = 0; v < kWaves; ++v) {
        const int32_t nbv = wave_batches(g, v);
        for (int32_t b = 0; b < nbv; ++b)
          for (int32_t sl = 0; sl < kBatch; ++sl) {
            const int32_t us = sl / g.ks, tt = sl % g.ks;
            const int32_t u = v + kWaves * (b * g.upb + us);
            if (u >= g.nu) continue;
            const int32_t lp = u / g.S, j = (u % g.S) * g.ks + tt;
            if (lp >= g.np || j >= g.kt) {
              std::printf("slot out of range w=%d st=%d v=%d b=%d sl=%d\n", w, st, v, b, sl);
              return 1;
            }
            seen[(size_t)lp * g.kt + j] += 1;
          }
        // the batch count is the least that holds the wave's units
        const int32_t nu_v = wave_units(g, v);
        if (nbv * g.upb < nu_v || (nbv > 0 && (nbv - 1) * g.upb >= nu_v)) {
          std::printf("batch count w=%d st=%d v=%d\n", w, st, v);
          return 1;
        }
      }
      for (size_t i = 0; i < seen.size(); ++i)
        if (seen[i] != 1) {
          std::printf("tile %zu of w=%d st=%d covered %d times\n", i, w, st, seen[i]);
          return 1;
        }
    }
    for (int32_t v = 0; v < kWaves; ++v) total += stream_tiles<TK>(s, w, v);
  }
  if (total != packed_stream_tiles<TK>(s)) {
    std::printf("stream total mismatch\n");
    return 1;
  }
  for (int st = ST_QKV; st < ST_COUNT; ++st) {
    int64_t np = 0;
    for (int32_t w = 0; w < s.nwg; ++w) np += stage_geo<TK>(s, st, w).np;
    if (np != s.stage_pairs(st)) {
      std::printf("pairs of stage %d do not add up\n", st);
      return 1;
    }
    // positions map one-to-one onto pairs, and every position has exactly one owning workgroup
    const int32_t n = s.stage_pairs(st);
    std::vector<int> hit((size_t)n, 0), own((size_t)n, 0);
    for (int32_t p = 0; p < n; ++p) {
      const int32_t gp = stage_pair(s, st, p);
      if (gp < 0 || gp >= n || (st == ST_QKV && qkv_position(s, gp) != p)) {
        std::printf("stage %d: position %d maps to pair %d\n", st, p, gp);
        return 1;
      }
      hit[(size_t)gp] += 1;
    }
    for (int32_t w = 0; w < s.nwg; ++w) {
      const StageGeo g = stage_geo<TK>(s, st, w);
      for (int32_t lp = 0; lp < g.np; ++lp) own[(size_t)(g.pb + lp)] += 1;
    }
    for (int32_t i = 0; i < n; ++i)
      if (hit[(size_t)i] != 1 || own[(size_t)i] != 1) {
        std::printf("stage %d: pair %d hit %d times, position %d owned %d times\n", st, i, hit[(size_t)i], i,
                    own[(size_t)i]);
        return 1;
      }
  }
  for (int32_t w = 0; w < s.nwg; ++w)
    if (xcd_wg(s.nwg, xcd_rank(s.nwg, w)) != w || xcd_rank(s.nwg, w) < 0 || xcd_rank(s.nwg, w) >= s.nwg) {
      std::printf("chiplet-major rank of workgroup %d does not invert\n", w);
      return 1;
    }
  // packed_tile inverts the placement: stream (w, v), batch b, slot sl of stage st in layer l
  std::vector<int64_t> wbase((size_t)s.nwg * kWaves + 1);
  int64_t acc = 0;
  for (int32_t w = 0; w < s.nwg; ++w)
    for (int32_t v = 0; v < kWaves; ++v) {
      wbase[(size_t)w * kWaves + v] = acc;
      acc += stream_tiles<TK>(s, w, v);
    }
  const int32_t layers[3] = {0, s.L - 1, s.L};  // first layer, last layer, LM head
  for (int li = 0; li < 3; ++li) {
    const int32_t l = layers[li];
    for (int32_t w = 0; w < s.nwg; ++w)
      for (int32_t v = 0; v < kWaves; ++v) {
        int64_t t0 = wbase[(size_t)w * kWaves + v] + (int64_t)l * layer_batches<TK>(s, w, v) * kBatch;
        for (int st = (l == s.L ? ST_LM : ST_QKV); st <= (l == s.L ? ST_LM : ST_DN); ++st) {
          if (!s.in_stream(st)) continue;
          const StageGeo g = stage_geo<TK>(s, st, w);
          const int32_t nbv = wave_batches(g, v);
          for (int32_t b = 0; b < nbv; ++b)
            for (int32_t sl = 0; sl < kBatch; ++sl) {
              const int32_t u = v + kWaves * (b * g.upb + sl / g.ks);
              if (u >= g.nu) continue;
              const int32_t gp = stage_pair(s, st, g.pb + u / g.S), kt = (u % g.S) * g.ks + sl % g.ks;
              const int64_t got = packed_tile<TK>(s, wbase.data(), st, l, gp, kt);
              if (got != t0 + (int64_t)b * kBatch + sl) {
                std::printf("packed_tile mismatch l=%d st=%d gp=%d kt=%d: %lld vs %lld\n", l, st, gp, kt, (long long)got,
                            (long long)(t0 + (int64_t)b * kBatch + sl));
                return 1;
              }
            }
          t0 += (int64_t)nbv * kBatch;
        }
      }
  }
  if (s.moe()) {  // expert region: every (layer, expert, pair, k-tile) has its own tile
    const int64_t n = expert_tiles(s);
    std::vector<uint8_t> seen((size_t)n, 0);
    for (int32_t l = 0; l < s.L; ++l)
      for (int32_t e = 0; e < s.E; ++e) {
        for (int32_t p = 0; p < s.Fe; ++p)
          for (int32_t kt = 0; kt < s.d / kTileK; ++kt) {
            const int64_t t = expert_gu_tile(s, l, e, p, kt);
            if (t < 0 || t >= n || seen[(size_t)t]++) {
              std::printf("gate/up tile l=%d e=%d p=%d kt=%d misplaced\n", l, e, p, kt);
              return 1;
            }
          }
        for (int32_t p = 0; p < s.d / 2; ++p)
          for (int32_t kt = 0; kt < s.Fe / kTileK; ++kt) {
            const int64_t t = expert_dn_tile(s, l, e, p, kt);
            if (t < 0 || t >= n || seen[(size_t)t]++) {
              std::printf("down tile l=%d e=%d p=%d kt=%d misplaced\n", l, e, p, kt);
              return 1;
            }
          }
      }
    if (packed_embed_offset<TK>(s) != (packed_stream_tiles<TK>(s) + n) * kTileBytes) {
      std::printf("embedding offset does not follow the expert region\n");
      return 1;
    }
  }
  std::printf("ok %lld tiles\n", (long long)total);
  return 0;
}

int main(int argc, char** argv) {
  // a trailing "fp8": the geometry of 8-bit weights (2 * kTileK weights of a row per tile)
  const bool w8 = argc > 1 && std::string(argv[argc - 1]) == "fp8";
  if (w8) --argc;
  if (argc != 10 && argc != 13) {
    std::printf("usage: L d nq nkv hd F V max_seq nwg [E A Fe] [fp8]\n");
    return 2;
  }
  Shape s;
  s.E = s.A = s.Fe = 0;
  if (argc == 13) {  // mixture of experts: F is the width of the A routed experts
    s.E = std::atoi(argv[10]);
    s.A = std::atoi(argv[11]);
    s.Fe = std::atoi(argv[12]);
  }
  s.L = std::atoi(argv[1]);
  s.d = std::atoi(argv[2]);
  s.nq = std::atoi(argv[3]);
  s.nkv = std::atoi(argv[4]);
  s.hd = std::atoi(argv[5]);
  s.F = std::atoi(argv[6]);
  s.V = std::atoi(argv[7]);
  s.max_seq = std::atoi(argv[8]);
  s.nwg = std::atoi(argv[9]);
  s.eps = 1e-5f;
  s.theta = 10000.f;
  if (s.moe()) s.F = s.A * s.Fe;
  return w8 ? check<2 * kTileK>(s) : check<kTileK>(s);
}
