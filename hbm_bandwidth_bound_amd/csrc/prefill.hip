// prefill.hip -- the prompt pass as dense matrix products on the matrix cores (MFMA).
//
// A prompt of P tokens is the same decoder applied to P positions at once, so its projections are
// real GEMMs (P x K by K x N) and run on gfx950's bf16 MFMA; only the last prompt position goes
// through the decode kernel, which adds the LM head and the sampler. The pages treat the prompt
// pass as compute-bound and outside the per-token budget (wink.run, 《GPU 算力越堆越高,生成 token
// 为什么还是慢》, the prefill/decode contrast; zdabc.icu 《Kog 推理引擎…》, the time-to-first-token
// measurement), so nothing here is on the decode path.
//
// Precision: activations are fp32 like the decode path. A GEMM input x is split into two bf16
// parts hi + lo (hi the bf16 rounding of x, lo that of x - hi; about 16 significant bits, a
// relative error below 2^-17) and every weight tile is multiplied by both, accumulating in fp32
// inside the MFMA: each product of a part with a bf16 weight is exact. The
// weights are read in place from the packed image (the packer's placement, inverted per tile by
// packed_tile), so no second copy of the model is kept.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.h"
#include "layout.h"
#include "monokernel.h"
#include "prefill.h"

namespace kie {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// x ~ hi + lo (bf16 bits): hi = bf16(x) and lo = bf16(x - hi), both rounded to nearest even
__device__ __forceinline__ void split2(float x, uint16_t* hi, uint16_t* lo) {
  const uint32_t h = f32_to_bf16(x);
  *hi = (uint16_t)h;
  *lo = (uint16_t)f32_to_bf16(x - bf16_to_f32(h));
}

// ------------------------------------------------------------------------------------------
// Embedding rows: X[i] = E[tok[i]] (fp32). An id out of range is replaced by 0 and reported.
// ------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) prefill_embed_kernel(PrefillArgs a, int32_t c0, int32_t pc) {
  const int32_t i = blockIdx.x;
  if (i >= pc) return;
  int32_t t = a.tokens[c0 + i];
  if (t < 0 || t >= a.s.V) {
    if (threadIdx.x == 0) __hip_atomic_fetch_or(a.err, KERR_BAD_TOKEN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    t = 0;
  }
  for (int32_t e = threadIdx.x; e < a.s.d; e += blockDim.x)
    a.x[(int64_t)i * a.s.d + e] = bf16_to_f32(a.embed[(int64_t)t * a.s.d + e]);
}

// ------------------------------------------------------------------------------------------
// RMSNorm of each row of X with gain g, written as the two-part GEMM input (row stride d).
// The sum of squares runs in a fixed order (per-thread strided partials, then a fixed tree).
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void norm_split_row(const PrefillArgs& a, const uint16_t* gain, int32_t i, float* red) {
  const int32_t d = a.s.d;
  const float* xr = a.x + (int64_t)i * d;
  float ss = 0.f;
  for (int32_t e = threadIdx.x; e < d; e += 256) ss = fmaf(xr[e], xr[e], ss);
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const float r = 1.0f / sqrtf(red[0] / (float)d + a.s.eps);
  for (int32_t e = threadIdx.x; e < d; e += 256) {
    const float u = (xr[e] * r) * bf16_to_f32(gain[e]);
    const int64_t o = (int64_t)i * d + e;
    split2(u, a.a3 + o, a.a3 + a.a_part + o);
  }
}
__global__ void __launch_bounds__(256) prefill_norm_split_kernel(PrefillArgs a, const uint16_t* gain, int32_t pc) {
  __shared__ float red[256];
  if ((int32_t)blockIdx.x >= pc) return;
  norm_split_row(a, gain, blockIdx.x, red);
}

// ------------------------------------------------------------------------------------------
// GEMM on the matrix cores: C[i][n] (= or +=) sum_k A[i][k] W[n][k] for the rows n of one stage
// in pair order (n = 2 gp + 0 for the pair's row A, + 1 for its row B), A given in two bf16 parts.
// Block: 64 tokens x 128 rows, 4 waves of 32 rows (two 16-row MFMA columns each, so every A
// operand read from LDS feeds two MFMAs); K in chunks of 128. The next chunk's weight operands
// and activations are loaded into registers while the current chunk is multiplied.
// MFMA 16x16x32 bf16 operand layout (gfx950): lane l holds A[l%16][8(l/16) .. +7] and
// B[8(l/16) .. +7][l%16]; the result D[4(l/16) + r][l%16] for r < 4.
// ------------------------------------------------------------------------------------------
constexpr int kGemmM = 64, kGemmN = 128, kGemmKC = 128, kGemmParts = 2;
constexpr int kALd = kGemmKC + 8;  // padded LDS row (bf16), spreads the rows over the banks

// Eight e4m3fn codes (k .. k+3 in c0, k+4 .. k+7 in c1, lowest k in the lowest byte) as eight
// bf16, exactly: each code widens exactly to fp32 (gfx950 pair conversion), and an e4m3 value
// has 3 significand bits and an exponent inside bf16's range, so the fp32's upper half is it.
typedef float v2f_t __attribute__((ext_vector_type(2)));
template <bool HI>
__device__ __forceinline__ uint32_t codes2_to_bf16(uint32_t c) {  // codes 0, 1 (or 2, 3 with HI)
  const v2f_t f = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, HI);
  return (__float_as_uint(f.x) >> 16) | (__float_as_uint(f.y) & 0xffff0000u);
}
__device__ __forceinline__ bf16x8 codes8_to_bf16(uint32_t c0, uint32_t c1) {
  return __builtin_bit_cast(bf16x8, uint4{codes2_to_bf16<false>(c0), codes2_to_bf16<true>(c0),
                                          codes2_to_bf16<false>(c1), codes2_to_bf16<true>(c1)});
}

// W8: the weights are e4m3fn codes (8-bit tiles: lane q holds row A's codes at k = 4q .. 4q+3
// and 256 + 4q .. +3 of the tile's 512, then row B's at the same k), widened to bf16 as they are
// read; the matrix's scale multiplies the products in the epilogue.
//
// XM (mixture of experts; bf16): 1 = an expert's gate/up product, 2 = its down product, over the
// positions that chose it. blockIdx.y is the expert e; the block's rows are rows of e's token
// list (XM 1: the rows of the positions in the list, from the RMSNorm input a3; XM 2: e's rows of
// h2 from its first row offs[e] on), and its weights are e's tiles in the expert region.
template <bool W8, int XM = 0>
__global__ void __launch_bounds__(256) prefill_gemm_kernel(PrefillArgs a, GemmStage g, int32_t pc) {
  constexpr int TK = W8 ? 2 * kTileK : kTileK;  // weights of a row per tile
  constexpr int KSTEPS = kGemmKC / 32;
  constexpr int NB = kGemmN / 64;                                  // 16-row columns per wave
  constexpr int APER = kGemmParts * kGemmM * (kGemmKC / 8) / 256;  // 16-byte pieces per thread
  __shared__ __align__(16) uint16_t As[kGemmParts][kGemmM][kALd];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // XM: this block's expert, its number of positions (the GEMM's rows) and its first row
  const int32_t ex = XM ? (int32_t)blockIdx.y : 0;
  const int32_t rows = XM ? a.counts[ex] : pc;
  const int32_t erow0 = XM ? a.offs[ex] : 0;
  // Tile of this block. The token tiles of one weight tile run on one XCD in consecutive slots
  // (workgroup b goes to XCD b mod 8), so the weight tile is fetched from HBM once and then served
  // by that XCD's L2 to the other token tiles.
  const int32_t nM = ((XM ? kPrefillChunk : pc) + kGemmM - 1) / kGemmM, nN = (g.N + kGemmN - 1) / kGemmN;
  const int32_t b = (int32_t)blockIdx.x % (nM * nN), split = (int32_t)blockIdx.x / (nM * nN);
  const int32_t kbeg = split * g.kper, kend = kbeg + g.kper;  // this block's share of K
  int32_t mt, nt;
  if (XM) {
    mt = b % nM;
    nt = b / nM;
    if (mt * kGemmM >= rows) return;  // (uniform over the block)
  } else if (nN % 8 == 0) {
    mt = (b / 8) % nM;
    nt = b % 8 + 8 * ((b / 8) / nM);
  } else {
    mt = b % nM;
    nt = b / nM;
  }
  const int32_t m0 = mt * kGemmM;
  const int nl = lane & 15, kg = lane >> 4;
  int32_t n[NB], gp[NB];
  bool nvalid[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    n[nb] = nt * kGemmN + wv * (16 * NB) + 16 * nb + nl;
    nvalid[nb] = n[nb] < g.N;
    gp[nb] = nvalid[nb] ? n[nb] >> 1 : 0;
  }
  const int sel = nl & 1;  // row A or B of the pair (n and nl have the same parity)
  // XM: an expert pair's k-tiles are contiguous in the expert region, so one unit spans them all
  const int32_t ks_unit = XM ? g.K / kTileK : unit_tiles(a.s.template stage_kt<TK>(g.st));
  const int64_t xregion = XM ? a.wbase[a.s.nwg * kWaves] : 0;  // the expert region's first tile
  int64_t tbase[NB] = {};  // first tile of the current unit of each column's pair
  f4 acc[4][NB];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f4{0.f, 0.f, 0.f, 0.f};

  uint2 w0[NB][KSTEPS], w1[NB][KSTEPS];
  uint4 av4[APER];
  auto fetch = [&](int32_t kc) {  // weight operands of chunk kc into w0/w1, activations into av4
    const int32_t kt = kc / TK;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (kc == kbeg || (kt % ks_unit == 0 && kc % TK == 0)) {
        if constexpr (XM == 1)
          tbase[nb] = nvalid[nb] ? xregion + expert_gu_tile(a.s, g.layer, ex, gp[nb], 0) : 0;
        else if constexpr (XM == 2)
          tbase[nb] = nvalid[nb] ? xregion + expert_dn_tile(a.s, g.layer, ex, gp[nb], 0) : 0;
        else
          tbase[nb] = nvalid[nb] ? a.ptab[ptab_index<TK>(a.s, g.st, g.layer, gp[nb], kt / ks_unit)] : 0;
      }
      const uint8_t* tp = a.packed + (tbase[nb] + kt % ks_unit) * kTileBytes + 8 * sel;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        if constexpr (W8) {  // codes k .. k+7 of row sel: words of tile lanes q and q + 1
          const int kk = kc % TK + ks * 32 + kg * 8;
          const uint8_t* pw = tp + 4 * (kk >> 8);  // the word of the tile's first or second 256
          const int q = (kk & 255) >> 2;
          w0[nb][ks] = nvalid[nb] ? uint2{*(const uint32_t*)(pw + 16 * q), *(const uint32_t*)(pw + 16 * (q + 1))}
                                  : uint2{0u, 0u};
        } else {
          const int L = (kc % kTileK + ks * 32 + kg * 8) >> 2;  // tile lane holding k .. k+3
          w0[nb][ks] = nvalid[nb] ? *(const uint2*)(tp + 16 * L) : uint2{0u, 0u};
          w1[nb][ks] = nvalid[nb] ? *(const uint2*)(tp + 16 * (L + 1)) : uint2{0u, 0u};
        }
      }
    }
#pragma unroll
    for (int jj = 0; jj < APER; ++jj) {
      const int q = tid + jj * 256;
      const int p = q / (kGemmM * (kGemmKC / 8)), r = (q / (kGemmKC / 8)) % kGemmM, c = q % (kGemmKC / 8);
      const int32_t i = m0 + r;
      int64_t src = i;  // the input row of GEMM row i
      if constexpr (XM == 1) src = i < rows ? a.lists[(int64_t)ex * kPrefillChunk + i] >> 4 : 0;
      if constexpr (XM == 2) src = erow0 + i;
      av4[jj] = i < rows ? *(const uint4*)(g.in + p * g.in_part + src * g.K + kc + c * 8) : uint4{0u, 0u, 0u, 0u};
    }
  };

  fetch(kbeg);
  for (int32_t kc = kbeg; kc < kend; kc += kGemmKC) {
    __syncthreads();  // every wave is done with the previous chunk's activations
#pragma unroll
    for (int jj = 0; jj < APER; ++jj) {
      const int q = tid + jj * 256;
      const int p = q / (kGemmM * (kGemmKC / 8)), r = (q / (kGemmKC / 8)) % kGemmM, c = q % (kGemmKC / 8);
      *(uint4*)&As[p][r][c * 8] = av4[jj];
    }
    bf16x8 b[NB][KSTEPS];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        b[nb][ks] = W8 ? codes8_to_bf16(w0[nb][ks].x, w0[nb][ks].y)
                       : __builtin_bit_cast(bf16x8, uint4{w0[nb][ks].x, w0[nb][ks].y, w1[nb][ks].x, w1[nb][ks].y});
    __syncthreads();
    if (kc + kGemmKC < kend) fetch(kc + kGemmKC);  // in flight while this chunk is multiplied
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int p = 0; p < kGemmParts; ++p) {
          const bf16x8 av = *(const bf16x8*)&As[p][mb * 16 + nl][ks * 32 + kg * 8];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[nb][ks], acc[mb][nb], 0, 0, 0);
        }
      }
    }
  }
  // 8-bit: matrix m of this layer is its scale times the codes (scales [L][7]: wq, wk, wv, wo,
  // w_gate, w_up, w_down)
  auto scale = [&](int m) { return W8 ? a.wscale[g.layer * 7 + m] : 1.f; };
  if (g.epi == EPI_STORE) {
    const float sc = scale(g.st == ST_O ? 3 : 6);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (!nvalid[nb]) continue;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int32_t i = m0 + mb * 16 + kg * 4 + r;
          if (i >= rows) continue;
          const float y = W8 ? acc[mb][nb][r] * sc : acc[mb][nb][r];
          if (XM == 2) {  // the expert's down-projection row of this position and rank
            a.ey[(int64_t)(erow0 + i) * g.N + n[nb]] = y;
          } else if (g.splits > 1) {  // partial sum of this share of K, summed by prefill_splitk_reduce_kernel
            g.part[((int64_t)split * pc + i) * g.N + n[nb]] = y;
          } else {
            float* dst = g.out + (int64_t)i * g.ldo + n[nb];
            *dst = (g.accumulate ? *dst : 0.f) + y;
          }
        }
    }
    return;
  }
  // pair epilogues: the other row of this lane's pair is in lane nl ^ 1
  const Shape& s = a.s;
  const int32_t half = s.hd / 2;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = acc[mb][nb][r];
        const float u = __shfl_xor(v, 1, 64);
        const int32_t i = m0 + mb * 16 + kg * 4 + r;
        if (!nvalid[nb] || i >= rows) continue;
        float ya = sel ? u : v, yb = sel ? v : u;  // rows A and B of pair gp
        const int32_t q = gp[nb];
        if (XM == 1) {  // pair q = gate row q and up row q of the expert; h times the routing weight
          if (sel == 0) {
            const int32_t le = a.lists[(int64_t)ex * kPrefillChunk + i];
            const float w = a.wt[(int64_t)(le >> 4) * s.A + (le & 15)];
            const int64_t o = (int64_t)(erow0 + i) * s.Fe + q;
            split2(w * ((ya / (1.0f + expf(-ya))) * yb), a.h2 + o, a.h2 + (int64_t)kPrefillChunk * s.F + o);
          }
        } else if (g.epi == EPI_SWIGLU) {  // pair q = gate row q and up row q
          if (W8) {
            ya *= scale(4);
            yb *= scale(5);
          }
          if (sel == 0) {
            const int64_t o = (int64_t)i * s.F + q;
            split2((ya / (1.0f + expf(-ya))) * yb, a.h2 + o, a.h2 + (int64_t)kPrefillChunk * s.F + o);
          }
        } else {  // EPI_ROPE_KV: pair q = dims (e, e + hd/2) of head hs
          const int32_t hs = q / half, e = q % half, pos = g.p0 + i;
          if (W8) {  // the scale of Wq, Wk or Wv
            const float sc = scale(hs < s.nq ? 0 : (hs < s.nq + s.nkv ? 1 : 2));
            ya *= sc;
            yb *= sc;
          }
          float y = sel ? yb : ya;
          if (hs < s.nq + s.nkv) {  // query and key heads are rotated
            const float2 cs = a.rope[(int64_t)pos * half + e];
            y = sel ? yb * cs.x + ya * cs.y : ya * cs.x - yb * cs.y;
          }
          const int32_t dim = e + sel * half;
          if (hs < s.nq) {
            a.q[(int64_t)i * s.qdim() + hs * s.hd + dim] = y;
          } else {
            const int kv = hs < s.nq + s.nkv ? 0 : 1;
            const int32_t jh = kv == 0 ? hs - s.nq : hs - s.nq - s.nkv;
            a.kv[kv_offset(s, g.layer, kv, jh, pos) + dim] = (uint16_t)f32_to_bf16(y);
          }
        }
      }
}

// ------------------------------------------------------------------------------------------
// The dense bf16 products (QKV, O, gate/up, down) as a pipelined GEMM on a larger tile: 128 tokens x
// 64 pairs (128 rows) per block, 4 waves of 64 tokens x 32 pairs (2 x 2). Both operands are
// staged in LDS by direct loads (gfx950 global_load_lds_dwordx4: 16 bytes per lane written at
// M0 + 16 lane, no registers held while in flight), through kMmStages stages of 64 k, so that the
// next stages' loads are in flight while one is multiplied; the 64 x 64 wave tile reads 12
// operands from LDS per 32 MFMAs (LDS bandwidth, not the matrix cores, bounds smaller tiles).
// Each weight operand is a whole packed tile lane: 4 k of the pair's row A and 4 k of its row B,
// so a lane reading tile lanes L and L + 1 holds 8 k of both rows -- the operands of two MFMAs,
// one for the pair's row A and one for its row B -- and its results hold both rows of the pair
// (the epilogues need no lane exchange). Every accumulator takes its products in the same order
// as in prefill_gemm_kernel (k ascending, the high part before the low part at each k step).
// LDS layout of a stage (48 KB):
//   A: [part 2][row 128][8 pieces of 16 bytes], piece c of row r stored at slot c ^ sa(r);
//   B: [pair 64][16 pieces], tile lane L of pair P (16 per stage) stored at slot L ^ (P mod 16);
// the XOR placements put the lanes of an operand read on distinct banks.
// ------------------------------------------------------------------------------------------
constexpr int kMmM = 128, kMmKC = 64, kMmStages = 3;
constexpr int kMmPairs = kGemmN / 2;                      // pairs per block
constexpr int kMmABytes = kGemmParts * kMmM * kMmKC * 2;  // 32 KB
constexpr int kMmStageBytes = kMmABytes + kMmPairs * kMmKC * 4;
// the first tile of each unit (a run of consecutive k-tiles of one pair) the block reads, per pair
constexpr int kMmUnits = 16;
constexpr int kMmLds = kMmStages * kMmStageBytes + kMmUnits * kMmPairs * 8;
constexpr int kMmLoads = (kMmABytes + kMmPairs * kMmKC * 4) / 1024 / 4;  // wave loads per stage and wave
extern __shared__ __align__(16) uint8_t mm_smem[];

__device__ __forceinline__ int mm_sa(int r) { return (r ^ (r >> 3)) & 7; }
// s_waitcnt immediate that waits until at most n vector memory operations are outstanding
constexpr int mm_vmcnt(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
static_assert(kMmLoads * (kMmStages - 2) < 64, "vmcnt holds at most 63");
// 16 bytes per lane from the 64-bit address p into LDS at lds_base + 16 * lane
__device__ __forceinline__ void mm_load_lds(const void* p, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(p), "{m0}"(lds_base) : "memory");
}
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u4v lds_read16(uint32_t addr) {
  return *(const __attribute__((address_space(3))) u4v*)(uintptr_t)addr;
}

// One block per CU (its LDS), so one wave per SIMD: the compiler is told so, and schedules the
// operand reads ahead of the MFMAs instead of saving registers for waves that cannot run.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
prefill_mm_kernel(PrefillArgs a, GemmStage g, int32_t pc) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int p = lane & 15, kg = lane >> 4, wm = wv & 1, wn = wv >> 1;
  const int32_t nM = (pc + kMmM - 1) / kMmM, nN = g.N / kGemmN;
  const int32_t b = (int32_t)blockIdx.x % (nM * nN), split = (int32_t)blockIdx.x / (nM * nN);
  int32_t mt, nt;
  if (nN % 8 == 0) {  // the token tiles of one weight tile on one XCD (as in prefill_gemm_kernel)
    mt = (b / 8) % nM;
    nt = b % 8 + 8 * ((b / 8) / nM);
  } else {
    mt = b % nM;
    nt = b / nM;
  }
  const int32_t m0 = mt * kMmM;
  const int32_t kbeg = split * g.kper, nk = g.kper / kMmKC;
  const int32_t ks_unit = unit_tiles(a.s.stage_kt(g.st));
  const uint32_t smem = lds_addr(mm_smem);

  // the first packed tile of units u0 .. u0 + nu - 1 of the block's 64 pairs, from the tile table
  int64_t* tbl = (int64_t*)(mm_smem + kMmStages * kMmStageBytes);
  const int32_t u0 = (kbeg / kTileK) / ks_unit;
  const int32_t nu = ((kbeg + g.kper - 1) / kTileK) / ks_unit - u0 + 1;  // at most kMmUnits (host)
  for (int e = tid; e < kMmPairs * nu; e += 256) {
    const int P = e % kMmPairs, ui = e / kMmPairs;
    tbl[e] = a.ptab[ptab_index(a.s, g.st, g.layer, nt * kMmPairs + P, u0 + ui)];
  }
  __syncthreads();

  // this lane's loads of a stage: A wave loads t = 8 wv + q (part t / 16, rows 8 (t % 16) ..
  // + 7), B wave loads t = 4 wv + q (pairs 4 t .. 4 t + 3)
  const uint8_t* abase[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int t = 8 * wv + q, part = t / 16, r = 8 * (t % 16) + (lane >> 3);
    const int c = (lane & 7) ^ mm_sa(r);
    abase[q] = (const uint8_t*)(g.in + part * g.in_part + (int64_t)(m0 + r) * g.K) + 16 * c;
  }
  // this lane's B sources in the current unit (the table is read again when a unit begins)
  const uint8_t* bptr[4];
  int32_t cur_unit = -1;
  auto issue = [&](int32_t c) {  // chunk c of K into stage c % kMmStages
    const int32_t k0 = kbeg + c * kMmKC, kt = k0 / kTileK;
    const uint32_t st = smem + (uint32_t)(c % kMmStages) * kMmStageBytes;
    if (kt / ks_unit != cur_unit) {
      cur_unit = kt / ks_unit;
      const int64_t* trow = tbl + (cur_unit - u0) * kMmPairs + 16 * wv + kg;
#pragma unroll
      for (int q = 0; q < 4; ++q) bptr[q] = a.packed + trow[4 * q] * kTileBytes + 16 * ((lane & 15) ^ ((4 * q + kg) & 15));
    }
    const int64_t boff = (int64_t)(kt % ks_unit) * kTileBytes + 16 * ((k0 % kTileK) >> 2);
#pragma unroll
    for (int q = 0; q < 4; ++q) mm_load_lds(bptr[q] + boff, st + kMmABytes + (16 * wv + 4 * q) * 256);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int t = 8 * wv + q;
      mm_load_lds(abase[q] + 2 * (int64_t)k0, st + (t / 16) * (kMmM * kMmKC * 2) + (t % 16) * 1024);
    }
  };

  f4 acc[4][2][2];  // [mb][pair group][row A, row B]
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[mb][j][0] = acc[mb][j][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < kMmStages - 1; ++c)
    if (c < nk) issue(c);
  for (int32_t c = 0; c < nk; ++c) {
    // chunk c's loads of this wave have landed when at most the later chunks' loads remain
    if (c + kMmStages - 2 < nk)
      __builtin_amdgcn_s_waitcnt(mm_vmcnt(kMmLoads * (kMmStages - 2)));
    else
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();  // every wave's loads of chunk c landed; chunk c - 1's stage is free
    const uint32_t st = smem + (uint32_t)(c % kMmStages) * kMmStageBytes;
    // every operand of the chunk is read before the first MFMA, so the reads overlap
    constexpr int KS = kMmKC / 32;
    u4v bu[KS][2][2], av[KS][4][kGemmParts];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int L = ks * 8 + 2 * kg;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t bs = st + kMmABytes + (32 * wn + 16 * j + p) * (kMmKC * 4);
        bu[ks][j][0] = lds_read16(bs + 16 * (L ^ p));
        bu[ks][j][1] = lds_read16(bs + 16 * ((L + 1) ^ p));
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int r = 64 * wm + mb * 16 + p, cc = ks * 4 + kg;
#pragma unroll
        for (int part = 0; part < kGemmParts; ++part)
          av[ks][mb][part] = lds_read16(st + part * (kMmM * kMmKC * 2) + r * (kMmKC * 2) + 16 * (cc ^ mm_sa(r)));
      }
    }
    // the loads of chunk c + 2, issued after this chunk's operand reads
    if (c + kMmStages - 1 < nk) issue(c + kMmStages - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 bx[2], by[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bx[j] = __builtin_bit_cast(bf16x8, u4v{bu[ks][j][0].x, bu[ks][j][0].y, bu[ks][j][1].x, bu[ks][j][1].y});
        by[j] = __builtin_bit_cast(bf16x8, u4v{bu[ks][j][0].z, bu[ks][j][0].w, bu[ks][j][1].z, bu[ks][j][1].w});
      }
#pragma unroll
      for (int part = 0; part < kGemmParts; ++part)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const bf16x8 A = __builtin_bit_cast(bf16x8, av[ks][mb][part]);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            acc[mb][j][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bx[j], acc[mb][j][0], 0, 0, 0);
            acc[mb][j][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, by[j], acc[mb][j][1], 0, 0, 0);
          }
        }
    }
    // schedule: the chunk's LDS reads (12 per k step), then its MFMAs (32 per k step)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) __builtin_amdgcn_sched_group_barrier(0x100, 4 + 4 * kGemmParts, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) __builtin_amdgcn_sched_group_barrier(0x008, 16 * kGemmParts, 0);
  }

  // epilogue: the lane holds rows A and B of pair gp for tokens m0 + 64 wm + 16 mb + 4 kg + r
  const Shape& s = a.s;
  const int32_t half = s.hd / 2;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int32_t gp = nt * kMmPairs + 32 * wn + 16 * j + p;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int32_t i = m0 + 64 * wm + mb * 16 + kg * 4 + r;
        if (i >= pc) continue;
        const float ya = acc[mb][j][0][r], yb = acc[mb][j][1][r];
        if (g.epi == EPI_STORE) {
          if (g.splits > 1) {
            *(float2*)(g.part + ((int64_t)split * pc + i) * g.N + 2 * gp) = float2{ya, yb};
          } else {
            float2* dst = (float2*)(g.out + (int64_t)i * g.ldo + 2 * gp);
            float2 o = g.accumulate ? *dst : float2{0.f, 0.f};
            o.x += ya;
            o.y += yb;
            *dst = o;
          }
        } else if (g.epi == EPI_SWIGLU) {
          const int64_t o = (int64_t)i * s.F + gp;
          split2((ya / (1.0f + expf(-ya))) * yb, a.h2 + o, a.h2 + (int64_t)kPrefillChunk * s.F + o);
        } else {  // EPI_ROPE_KV: pair gp = dims (e, e + hd/2) of head hs
          const int32_t hs = gp / half, e = gp % half, pos = g.p0 + i;
          float y0 = ya, y1 = yb;
          if (hs < s.nq + s.nkv) {
            const float2 cs = a.rope[(int64_t)pos * half + e];
            y0 = ya * cs.x - yb * cs.y;
            y1 = yb * cs.x + ya * cs.y;
          }
          if (hs < s.nq) {
            float* qr = a.q + (int64_t)i * s.qdim() + hs * s.hd;
            qr[e] = y0;
            qr[e + half] = y1;
          } else {
            const int kv = hs < s.nq + s.nkv ? 0 : 1;
            const int32_t jh = kv == 0 ? hs - s.nq : hs - s.nq - s.nkv;
            uint16_t* row = a.kv + kv_offset(s, g.layer, kv, jh, pos);
            row[e] = (uint16_t)f32_to_bf16(y0);
            row[e + half] = (uint16_t)f32_to_bf16(y1);
          }
        }
      }
  }
}

// Row i of the residual: x += the K shares' partial sums (in share order), then the RMSNorm of
// the new row as the next GEMM's two-part input.
__global__ void __launch_bounds__(256) prefill_splitk_reduce_norm_kernel(PrefillArgs a, GemmStage g, const uint16_t* gain,
                                                                          int32_t pc) {
  __shared__ float red[256];
  const int32_t i = blockIdx.x;
  if (i >= pc) return;
  float* xr = g.out + (int64_t)i * g.ldo;
  for (int32_t n4 = threadIdx.x; n4 < g.N / 4; n4 += 256) {
    float4 sum = *(const float4*)(g.part + (int64_t)i * g.N + 4 * n4);
    for (int32_t sp = 1; sp < g.splits; ++sp) {
      const float4 v = *(const float4*)(g.part + ((int64_t)sp * pc + i) * g.N + 4 * n4);
      sum.x += v.x;
      sum.y += v.y;
      sum.z += v.z;
      sum.w += v.w;
    }
    float4 o = *(const float4*)(xr + 4 * n4);
    o.x += sum.x;
    o.y += sum.y;
    o.z += sum.z;
    o.w += sum.w;
    *(float4*)(xr + 4 * n4) = o;
  }
  __syncthreads();  // the norm reads the row by other columns per thread
  norm_split_row(a, gain, i, red);
}

// out (= or +=) the sum of the K shares' partial sums, in share order (the same every run)
__global__ void __launch_bounds__(256) prefill_splitk_reduce_kernel(GemmStage g, int32_t pc) {
  const int32_t nq4 = g.N / 4;
  const int64_t total = (int64_t)pc * nq4;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int32_t i = (int32_t)(e / nq4), n4 = (int32_t)(e % nq4);
    float4 sum = *(const float4*)(g.part + (int64_t)i * g.N + 4 * n4);
    for (int32_t sp = 1; sp < g.splits; ++sp) {
      const float4 v = *(const float4*)(g.part + ((int64_t)sp * pc + i) * g.N + 4 * n4);
      sum.x += v.x;
      sum.y += v.y;
      sum.z += v.z;
      sum.w += v.w;
    }
    float4* dst = (float4*)(g.out + (int64_t)i * g.ldo + 4 * n4);
    if (g.accumulate) {
      const float4 o = *dst;
      sum.x += o.x;
      sum.y += o.y;
      sum.z += o.z;
      sum.w += o.w;
    }
    *dst = sum;
  }
}

// ------------------------------------------------------------------------------------------
// Causal attention of the chunk's queries over positions 0 .. pos (cache rows, this chunk's rows
// included), on the matrix cores. Block: 64 (query, head) rows of one KV head --
// row r is query r / G and head j G + r % G, so the G heads of a group share every K/V tile -- in
// 4 waves of 16 rows; keys in tiles of 64 staged in LDS (K as stored, V transposed). Per tile a
// wave computes S^T = K Q^T on the MFMA (A = 16 keys x 32 dims of K, B = Q^T of its rows), takes
// the online softmax of each row in the exp2 domain, and adds P V on the MFMA (A = P of its 16
// rows x 32 keys, B = 32 keys x 16 dims of V). The 32 keys of a P operand are taken in the order
// the S^T result leaves them in the lanes, and V is read in that same order. Q and P enter as two
// bf16 parts (hi + lo, about 16 significant bits); K and V are bf16 already, so every product is
// exact and the sums are fp32. With one key segment (blockIdx.z) the output is written as the
// two-part input of the O projection; with several, each block writes its partial state
// (acc, m, l) and prefill_attn_merge_kernel combines the segments.
// ------------------------------------------------------------------------------------------
constexpr int kFaRows = 64, kFaKT = 64;

// two values to a bf16 pair (round to nearest even; gfx950 converts both in one instruction)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
// eight values as two bf16 operands, x ~ hi + lo
__device__ __forceinline__ void split2x8(const float* x, bf16x8* hi, bf16x8* lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = cvt_bf16x2(x[2 * e], x[2 * e + 1]);
    l[e] = cvt_bf16x2(x[2 * e] - bf16lo(h[e]), x[2 * e + 1] - bf16hi(h[e]));
  }
  *hi = __builtin_bit_cast(bf16x8, uint4{h[0], h[1], h[2], h[3]});
  *lo = __builtin_bit_cast(bf16x8, uint4{l[0], l[1], l[2], l[3]});
}

template <int HD, bool SPLIT>
__global__ void __launch_bounds__(256, 2) prefill_fattn_kernel(PrefillArgs a, int32_t layer, int32_t p0, int32_t pc) {
  constexpr int KP = HD + 8;     // padded K row (bf16): the 16 rows a lane group reads hit distinct banks
  constexpr int VP = kFaKT + 8;  // padded V^T row (bf16)
  constexpr int NKP = kFaKT * HD / 8 / 256;          // K pieces (16 bytes) per thread and tile
  constexpr int NVP = (kFaKT / 2) * (HD / 8) / 256;  // V pieces (two keys x 8 dims) per thread
  __shared__ __align__(16) uint16_t Ks[kFaKT][KP];
  __shared__ __align__(16) uint16_t Vt[HD][VP];
  const Shape& s = a.s;
  const int32_t G = s.group(), j = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int rl = lane & 15, lg = lane >> 4;
  // the row of this lane in the S^T and P layouts (column rl of the wave's 16)
  const int32_t r = (int32_t)blockIdx.x * kFaRows + wv * 16 + rl;
  const bool valid = r < pc * G;
  const int32_t qi = valid ? r / G : pc - 1, h = j * G + r % G;
  const int32_t qpos = p0 + qi;
  const int32_t rlast = min((int32_t)(blockIdx.x + 1) * kFaRows, pc * G) - 1;
  const int32_t kend = p0 + rlast / G;  // last key any row of the block needs
  const int32_t kbeg = SPLIT ? (int32_t)blockIdx.z * kPrefillAttnSeg : 0;
  const int32_t klast = SPLIT ? min(kend, kbeg + kPrefillAttnSeg - 1) : kend;
  const uint16_t* kbase = a.kv + kv_offset(s, layer, 0, j, 0);
  const uint16_t* vbase = a.kv + kv_offset(s, layer, 1, j, 0);
  // keys up to kfull are visible to every row of this wave: tiles below it need no mask
  const int32_t kfull = min(klast, p0 + min(((int32_t)blockIdx.x * kFaRows + wv * 16) / G, pc - 1));

  // Q^T operand of this lane: row rl, dims 32c + 8lg .. +7, scaled into the exp2 domain
  const float scale = 1.4426950408889634f / sqrtf((float)HD);
  bf16x8 qh[HD / 32], ql[HD / 32];
  {
    const float* qrow = a.q + (int64_t)qi * s.qdim() + h * HD;
#pragma unroll
    for (int c = 0; c < HD / 32; ++c) {
      const float4 x0 = *(const float4*)(qrow + 32 * c + 8 * lg);
      const float4 x1 = *(const float4*)(qrow + 32 * c + 8 * lg + 4);
      const float x[8] = {x0.x * scale, x0.y * scale, x0.z * scale, x0.w * scale,
                          x1.x * scale, x1.y * scale, x1.z * scale, x1.w * scale};
      split2x8(x, &qh[c], &ql[c]);
    }
  }
  f4 o[HD / 16];
#pragma unroll
  for (int c = 0; c < HD / 16; ++c) o[c] = f4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // softmax state of row rl (the same in the 4 lane groups)

  // two register sets of K/V pieces: tile t + 2 is loaded while tile t is multiplied
  uint4 kr0[NKP], vr0[NVP][2], kr1[NKP], vr1[NVP][2];
  auto fetch = [&](uint4(&kr)[NKP], uint4(&vr)[NVP][2], int32_t k0) {  // rows past klast read as 0
#pragma unroll
    for (int e = 0; e < NKP; ++e) {
      const int q = tid + 256 * e, row = q / (HD / 8), c8 = q % (HD / 8);
      const int32_t kp = k0 + row;
      kr[e] = kp <= klast ? *(const uint4*)(kbase + (int64_t)kp * HD + 8 * c8) : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int e = 0; e < NVP; ++e) {
      const int q = tid + 256 * e, row = 2 * (q % (kFaKT / 2)), c8 = q / (kFaKT / 2);
      const int32_t kp = k0 + row;
      vr[e][0] = kp <= klast ? *(const uint4*)(vbase + (int64_t)kp * HD + 8 * c8) : uint4{0u, 0u, 0u, 0u};
      vr[e][1] = kp + 1 <= klast ? *(const uint4*)(vbase + (int64_t)(kp + 1) * HD + 8 * c8) : uint4{0u, 0u, 0u, 0u};
    }
  };
  auto stage = [&](const uint4(&kr)[NKP], const uint4(&vr)[NVP][2]) {  // K as is; V as V^T, 2 keys a word
#pragma unroll
    for (int e = 0; e < NKP; ++e) {
      const int q = tid + 256 * e, row = q / (HD / 8), c8 = q % (HD / 8);
      *(uint4*)&Ks[row][8 * c8] = kr[e];
    }
#pragma unroll
    for (int e = 0; e < NVP; ++e) {
      const int q = tid + 256 * e, row = 2 * (q % (kFaKT / 2)), c8 = q / (kFaKT / 2);
      const uint32_t a0[4] = {vr[e][0].x, vr[e][0].y, vr[e][0].z, vr[e][0].w};
      const uint32_t a1[4] = {vr[e][1].x, vr[e][1].y, vr[e][1].z, vr[e][1].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        *(uint32_t*)&Vt[8 * c8 + 2 * w][row] = (a0[w] & 0xffffu) | (a1[w] << 16);
        *(uint32_t*)&Vt[8 * c8 + 2 * w + 1][row] = (a0[w] >> 16) | (a1[w] & 0xffff0000u);
      }
    }
  };

  auto tile = [&](int32_t k0) {
    // S^T: st[ks][i] = score of key k0 + 16 ks + 4 lg + i for row rl
    f4 st[kFaKT / 16];
#pragma unroll
    for (int ks = 0; ks < kFaKT / 16; ++ks) {
      st[ks] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < HD / 32; ++c) {
        const bf16x8 kv = *(const bf16x8*)&Ks[16 * ks + rl][32 * c + 8 * lg];
        st[ks] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qh[c], st[ks], 0, 0, 0);
        st[ks] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, ql[c], st[ks], 0, 0, 0);
      }
    }
    if (k0 + kFaKT - 1 > kfull) {  // the tile reaches past some row's position or past klast
#pragma unroll
      for (int ks = 0; ks < kFaKT / 16; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int32_t kp = k0 + 16 * ks + 4 * lg + i;
          if (kp > qpos || kp > klast) st[ks][i] = -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < kFaKT / 16; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) mt = fmaxf(mt, st[ks][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mn = fmaxf(m, mt);
    const float mu = mn == -INFINITY ? 0.f : mn;  // a row with no key yet keeps p = 0
    const float corr = __builtin_amdgcn_exp2f(m - mu);  // v_exp_f32: 2^x, 0 at -inf
    float ps = 0.f;
#pragma unroll
    for (int ks = 0; ks < kFaKT / 16; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        st[ks][i] = __builtin_amdgcn_exp2f(st[ks][i] - mu);
        ps += st[ks][i];
      }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l = l * corr + ps;
    m = mn;
    // O rows are 4 lg + i: their factors come from the lanes that hold those rows' state
    float cr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cr[i] = __shfl(corr, 4 * lg + i, 64);
#pragma unroll
    for (int c = 0; c < HD / 16; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[c][i] *= cr[i];
    // O += P V over the tile's 32-key halves; operand slot 8 lg + e is key 32 kc + 4 lg + e
    // (e < 4) or 32 kc + 16 + 4 lg + (e - 4)
#pragma unroll
    for (int kc = 0; kc < kFaKT / 32; ++kc) {
      const float pv[8] = {st[2 * kc][0], st[2 * kc][1], st[2 * kc][2], st[2 * kc][3],
                           st[2 * kc + 1][0], st[2 * kc + 1][1], st[2 * kc + 1][2], st[2 * kc + 1][3]};
      bf16x8 ph, pl;
      split2x8(pv, &ph, &pl);
#pragma unroll
      for (int c = 0; c < HD / 16; ++c) {
        const uint2 b0 = *(const uint2*)&Vt[16 * c + rl][32 * kc + 4 * lg];
        const uint2 b1 = *(const uint2*)&Vt[16 * c + rl][32 * kc + 16 + 4 * lg];
        const bf16x8 vb = __builtin_bit_cast(bf16x8, uint4{b0.x, b0.y, b1.x, b1.y});
        o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vb, o[c], 0, 0, 0);
        o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, o[c], 0, 0, 0);
      }
    }
  };

  if (kbeg <= klast) fetch(kr0, vr0, kbeg);
  if (kbeg + kFaKT <= klast) fetch(kr1, vr1, kbeg + kFaKT);
  for (int32_t k0 = kbeg; k0 <= klast; k0 += 2 * kFaKT) {
    __syncthreads();  // every wave is done with the previous tile
    stage(kr0, vr0);
    __syncthreads();
    if (k0 + 2 * kFaKT <= klast) fetch(kr0, vr0, k0 + 2 * kFaKT);
    tile(k0);
    if (k0 + kFaKT > klast) break;
    __syncthreads();
    stage(kr1, vr1);
    __syncthreads();
    if (k0 + 3 * kFaKT <= klast) fetch(kr1, vr1, k0 + 3 * kFaKT);
    tile(k0 + kFaKT);
  }
  // rows 4 lg + i of O: their softmax state, then the output
  float lr[4], mr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lr[i] = __shfl(l, 4 * lg + i, 64);
    mr[i] = __shfl(m, 4 * lg + i, 64);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t r2 = (int32_t)blockIdx.x * kFaRows + wv * 16 + 4 * lg + i;
    if (r2 >= pc * G) continue;
    const int32_t q2 = r2 / G, h2 = j * G + r2 % G;
    if (SPLIT) {  // partial state of this segment: [segment][query][head][acc[HD], m, l]
      float* st = a.attn_part + (((int64_t)blockIdx.z * kPrefillChunk + q2) * s.nq + h2) * (HD + 2);
#pragma unroll
      for (int c = 0; c < HD / 16; ++c) st[16 * c + rl] = o[c][i];
      if (rl == 0) {
        st[HD] = mr[i];
        st[HD + 1] = lr[i];
      }
    } else {
      const float inv = 1.0f / lr[i];
#pragma unroll
      for (int c = 0; c < HD / 16; ++c) {
        const int64_t off = (int64_t)q2 * s.qdim() + h2 * HD + 16 * c + rl;
        split2(o[c][i] * inv, a.a3 + off, a.a3 + a.a_part + off);
      }
    }
  }
}

// Combination of the segments' partial states (in segment order) for one query and head: thread
// e owns output dimension e.
template <int HD>
__global__ void __launch_bounds__(HD) prefill_attn_merge_kernel(PrefillArgs a, int32_t nseg, int32_t pc) {
  const Shape& s = a.s;
  const int32_t i = blockIdx.x, h = blockIdx.y, e = threadIdx.x;
  if (i >= pc) return;
  float M = -INFINITY, S = 0.f, A = 0.f;
  for (int32_t g = 0; g < nseg; ++g) {
    const float* st = a.attn_part + (((int64_t)g * kPrefillChunk + i) * s.nq + h) * (HD + 2);
    const float m2 = st[HD];
    if (m2 == -INFINITY) continue;
    const float Mn = fmaxf(M, m2);
    const float fo = M == -INFINITY ? 0.f : exp2f(M - Mn), fn = exp2f(m2 - Mn);
    S = S * fo + st[HD + 1] * fn;
    A = A * fo + st[e] * fn;
    M = Mn;
  }
  const int64_t o = (int64_t)i * s.qdim() + h * HD + e;
  split2(A / S, a.a3 + o, a.a3 + a.a_part + o);
}

// ------------------------------------------------------------------------------------------
// Mixture-of-experts layers: routing, per-expert token lists, and the weighted sum of the experts'
// outputs. The choice follows the decode kernel's: the A largest logits (ties to the lower index;
// NaN ranks lowest, -0 as +0) and weights exp(z_i - z_0) / sum_j exp(z_j - z_0) over the chosen
// in rank order, z_0 the largest.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ uint64_t route_key(float z, int32_t e) {  // larger key = ranks first
  z = z == z ? (z == 0.f ? 0.f : z) : -INFINITY;
  const uint32_t u = __float_as_uint(z);
  return ((uint64_t)((u & 0x80000000u) ? ~u : (u | 0x80000000u)) << 32) | (uint32_t)(0x7fffffff - e);
}
// one block per position: sel[i][rank] and wt[i][rank]
__global__ void __launch_bounds__(256) prefill_route_kernel(PrefillArgs a, int32_t pc) {
  const Shape& s = a.s;
  const int32_t i = blockIdx.x;
  if (i >= pc) return;
  __shared__ int32_t chosen[kMaxActive];
  const float* z = a.rlogits + (int64_t)i * s.E;
  for (int32_t e = threadIdx.x; e < s.E; e += blockDim.x) {
    const uint64_t k = route_key(z[e], e);
    int32_t rank = 0;
    for (int32_t f = 0; f < s.E; ++f) rank += route_key(z[f], f) > k ? 1 : 0;
    if (rank < s.A) chosen[rank] = e;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float x[kMaxActive];
    const float z0 = z[chosen[0]] == z[chosen[0]] ? z[chosen[0]] : -INFINITY;
    float sum = 0.f;
    for (int32_t r = 0; r < s.A; ++r) {
      const float zr = z[chosen[r]] == z[chosen[r]] ? z[chosen[r]] : -INFINITY;
      x[r] = expf(zr - z0);
      sum += x[r];
    }
    for (int32_t r = 0; r < s.A; ++r) {
      a.sel[(int64_t)i * s.A + r] = chosen[r];
      a.wt[(int64_t)i * s.A + r] = x[r] / sum;
    }
  }
}
// one block per expert: its positions in order (lists), their number (counts), and each choice's
// place in the list (place)
__global__ void __launch_bounds__(256) prefill_expert_lists_kernel(PrefillArgs a, int32_t pc) {
  const int32_t e = blockIdx.x, A = a.s.A, t = threadIdx.x;
  __shared__ int32_t scan[256];
  int32_t base = 0;
  for (int32_t i0 = 0; i0 < pc; i0 += 256) {
    const int32_t i = i0 + t;
    int32_t rank = -1;
    if (i < pc)
      for (int32_t r = 0; r < A; ++r)
        if (a.sel[(int64_t)i * A + r] == e) rank = r;
    scan[t] = rank >= 0 ? 1 : 0;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {  // inclusive prefix sum over the block
      const int32_t add = t >= o ? scan[t - o] : 0;
      __syncthreads();
      scan[t] += add;
      __syncthreads();
    }
    if (rank >= 0) {
      const int32_t at = base + scan[t] - 1;
      a.lists[(int64_t)e * kPrefillChunk + at] = (i << 4) | rank;
      a.place[(int64_t)i * A + rank] = at;
    }
    base += scan[255];
    __syncthreads();  // scan is reused
  }
  if (t == 0) a.counts[e] = base;
}
// the experts' first rows: the exclusive prefix sum of the list lengths (one thread, E is small)
__global__ void __launch_bounds__(64) prefill_expert_offsets_kernel(PrefillArgs a) {
  if (threadIdx.x != 0) return;
  int32_t o = 0;
  for (int32_t e = 0; e < a.s.E; ++e) {
    a.offs[e] = o;
    o += a.counts[e];
  }
}
// Row i of the residual: x += the chosen experts' down-projection rows (already weighted), summed
// in rank order; then the RMSNorm with gain (when given) as the next GEMM's two-part input.
__global__ void __launch_bounds__(256) prefill_moe_combine_kernel(PrefillArgs a, const uint16_t* gain, int32_t pc) {
  __shared__ float red[256];
  const Shape& s = a.s;
  const int32_t i = blockIdx.x;
  if (i >= pc) return;
  int64_t row[kMaxActive];
  for (int32_t r = 0; r < s.A; ++r)
    row[r] = (int64_t)(a.offs[a.sel[(int64_t)i * s.A + r]] + a.place[(int64_t)i * s.A + r]) * s.d;
  float* xr = a.x + (int64_t)i * s.d;
  for (int32_t c = threadIdx.x; c < s.d; c += 256) {
    float y = 0.f;
    for (int32_t r = 0; r < s.A; ++r) y += a.ey[row[r] + c];
    xr[c] += y;
  }
  __syncthreads();  // the norm reads the row by other columns per thread
  if (gain) norm_split_row(a, gain, i, red);
}

// ------------------------------------------------------------------------------------------
// The chunked prompt pass: positions p0 .. p0 + n - 1, every layer, K/V rows written to the cache.
// ------------------------------------------------------------------------------------------
// One GEMM of a layer stage. The QKV and gate/up products end in their pair epilogues; the O and
// down products add into the residual stream, followed by the RMSNorm with gain norm_after when
// it is given (written as the next GEMM's input).
static hipError_t gemm(const PrefillArgs& a, int st, int32_t layer, int32_t p0, int32_t pc, hipStream_t stream,
                       const uint16_t* norm_after = nullptr) {
  const Shape& s = a.s;
  GemmStage g;
  g.st = st;
  g.layer = layer;
  g.K = s.stage_k(st);
  g.N = 2 * s.stage_pairs(st);
  g.in = st == ST_DN ? a.h2 : a.a3;
  g.in_part = st == ST_DN ? (int64_t)kPrefillChunk * s.F : a.a_part;
  g.epi = st == ST_QKV ? EPI_ROPE_KV : (st == ST_GU ? EPI_SWIGLU : EPI_STORE);
  g.p0 = p0;
  g.out = a.x;  // EPI_STORE: x += C
  g.ldo = s.d;
  g.accumulate = 1;
  if (st == ST_RT) {  // the router: logits = C
    g.out = a.rlogits;
    g.ldo = s.E;
    g.accumulate = 0;
  }
  const int32_t K = g.K;
  // A GEMM with few output tiles (the O and down projections, N = d) splits K over up to 8
  // blocks per tile so that about two blocks run per CU; the partial sums go to the scratch
  // buffer c, summed in a fixed order by prefill_splitk_reduce_kernel.
  const int32_t tiles = ((g.N + kGemmN - 1) / kGemmN) * ((pc + kGemmM - 1) / kGemmM);
  g.splits = 1;
  if (g.epi == EPI_STORE && g.N % 4 == 0)
    while (g.splits < 8 && tiles * g.splits < 512 && K % (2 * g.splits * kGemmKC) == 0 &&
           2 * g.splits * g.N <= prefill_nmax(a.s))
      g.splits *= 2;
  g.kper = K / g.splits;
  g.part = a.c;
  const int32_t ks = unit_tiles(s.stage_kt(st));
  // prefill_mm_kernel holds a CU's LDS per block: it is used where its grid covers every CU (the
  // QKV product of a 512-token chunk of the 1.6B shape has 128 blocks and runs faster on the
  // smaller tiles of prefill_gemm_kernel, whose products are accumulated in the same order)
  const int32_t mm_blocks = (g.N / kGemmN) * ((pc + kMmM - 1) / kMmM) * g.splits;
  if (!a.wscale && g.N % kGemmN == 0 && (g.kper / kTileK + ks - 1) / ks + 1 <= kMmUnits && mm_blocks >= s.nwg)
    hipLaunchKernelGGL(prefill_mm_kernel, dim3(mm_blocks), dim3(256), kMmLds, stream, a, g, pc);
  else if (a.wscale)
    hipLaunchKernelGGL(prefill_gemm_kernel<true>, dim3(tiles * g.splits), dim3(256), 0, stream, a, g, pc);
  else
    hipLaunchKernelGGL(prefill_gemm_kernel<false>, dim3(tiles * g.splits), dim3(256), 0, stream, a, g, pc);
  if (g.splits > 1 && norm_after) {
    hipLaunchKernelGGL(prefill_splitk_reduce_norm_kernel, dim3(pc), dim3(256), 0, stream, a, g, norm_after, pc);
  } else {
    if (g.splits > 1) {
      const int64_t n4 = (int64_t)pc * (g.N / 4);
      hipLaunchKernelGGL(prefill_splitk_reduce_kernel,
                         dim3((unsigned)((n4 + 255) / 256 < 2048 ? (n4 + 255) / 256 : 2048)), dim3(256), 0, stream, g, pc);
    }
    if (norm_after) hipLaunchKernelGGL(prefill_norm_split_kernel, dim3(pc), dim3(256), 0, stream, a, norm_after, pc);
  }
  return hipGetLastError();
}

// A mixture-of-experts FFN over the chunk (its RMSNorm input in a3): router logits, the choice of
// experts per position, the experts' token lists, each expert's gate/up and down products over its
// positions (grouped GEMMs, one grid row per expert), and the weighted sum into the residual
// followed by the next RMSNorm.
static hipError_t moe_ffn(const PrefillArgs& a, int32_t layer, int32_t p0, int32_t pc, hipStream_t stream,
                          const uint16_t* next_gain) {
  const Shape& s = a.s;
  hipError_t e = gemm(a, ST_RT, layer, p0, pc, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_route_kernel, dim3(pc), dim3(256), 0, stream, a, pc);
  hipLaunchKernelGGL(prefill_expert_lists_kernel, dim3(s.E), dim3(256), 0, stream, a, pc);
  hipLaunchKernelGGL(prefill_expert_offsets_kernel, dim3(1), dim3(64), 0, stream, a);
  const int32_t nM = kPrefillChunk / kGemmM;  // token tiles per expert at most
  GemmStage g{};
  g.layer = layer;
  g.p0 = p0;
  g.splits = 1;
  g.st = ST_GU;  // gate/up of the chosen experts: rows of a3, h (weighted) into h2
  g.K = s.d;
  g.N = 2 * s.Fe;
  g.kper = g.K;
  g.in = a.a3;
  g.in_part = a.a_part;
  g.epi = EPI_SWIGLU;
  hipLaunchKernelGGL((prefill_gemm_kernel<false, 1>), dim3(nM * (g.N / kGemmN), s.E), dim3(256), 0, stream, a, g, pc);
  g.st = ST_DN;  // down: rows of h2 into the experts' rows of ey
  g.K = s.Fe;
  g.N = s.d;
  g.kper = g.K;
  g.in = a.h2;
  g.in_part = (int64_t)kPrefillChunk * s.F;
  g.epi = EPI_STORE;
  hipLaunchKernelGGL((prefill_gemm_kernel<false, 2>), dim3(nM * (g.N / kGemmN), s.E), dim3(256), 0, stream, a, g, pc);
  hipLaunchKernelGGL(prefill_moe_combine_kernel, dim3(pc), dim3(256), 0, stream, a, next_gain, pc);
  return hipGetLastError();
}

bool prefill_supports(const Shape& s) {
  if (!s.moe()) return true;
  return s.A >= 1 && s.A <= kMaxActive && s.A <= 15 && (2 * s.Fe) % kGemmN == 0 && s.d % kGemmN == 0 &&
         s.Fe % kGemmKC == 0 && s.d % kGemmKC == 0;
}

hipError_t launch_prefill(const PrefillArgs& a, int32_t p0, int32_t n, hipStream_t stream) {
  const Shape& s = a.s;
  hipError_t e0 = hipFuncSetAttribute((const void*)prefill_mm_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kMmLds);
  if (e0 != hipSuccess) return e0;
  for (int32_t c0 = 0; c0 < n; c0 += kPrefillChunk) {
    const int32_t pc = n - c0 < kPrefillChunk ? n - c0 : kPrefillChunk;
    const int32_t pos = p0 + c0;
    hipLaunchKernelGGL(prefill_embed_kernel, dim3(pc), dim3(256), 0, stream, a, c0, pc);
    hipLaunchKernelGGL(prefill_norm_split_kernel, dim3(pc), dim3(256), 0, stream, a, a.norms, pc);
    for (int32_t l = 0; l < s.L; ++l) {
      // the attention RMSNorm of layer l is in a3 here (after the embedding, or layer l-1's down)
      hipError_t e = gemm(a, ST_QKV, l, pos, pc, stream);  // with RoPE; K/V rows to the cache
      if (e != hipSuccess) return e;
      // keys split into segments when the context is long, so that enough blocks run at once
      const int32_t nseg = (pos + pc + kPrefillAttnSeg - 1) / kPrefillAttnSeg;
      const dim3 ag((pc * s.group() + kFaRows - 1) / kFaRows, s.nkv, nseg);
      if (nseg > 1) {
        if (s.hd == 128) {
          hipLaunchKernelGGL((prefill_fattn_kernel<128, true>), ag, dim3(256), 0, stream, a, l, pos, pc);
          hipLaunchKernelGGL(prefill_attn_merge_kernel<128>, dim3(pc, s.nq), dim3(128), 0, stream, a, nseg, pc);
        } else {
          hipLaunchKernelGGL((prefill_fattn_kernel<64, true>), ag, dim3(256), 0, stream, a, l, pos, pc);
          hipLaunchKernelGGL(prefill_attn_merge_kernel<64>, dim3(pc, s.nq), dim3(64), 0, stream, a, nseg, pc);
        }
      } else if (s.hd == 128) {
        hipLaunchKernelGGL((prefill_fattn_kernel<128, false>), ag, dim3(256), 0, stream, a, l, pos, pc);
      } else {
        hipLaunchKernelGGL((prefill_fattn_kernel<64, false>), ag, dim3(256), 0, stream, a, l, pos, pc);
      }
      if ((e = gemm(a, ST_O, l, pos, pc, stream, a.norms + (int64_t)l * 2 * s.d + s.d)) != hipSuccess) return e;
      const uint16_t* next_gain = l + 1 < s.L ? a.norms + (int64_t)(l + 1) * 2 * s.d : nullptr;
      if (s.moe()) {
        if ((e = moe_ffn(a, l, pos, pc, stream, next_gain)) != hipSuccess) return e;
        continue;
      }
      if ((e = gemm(a, ST_GU, l, pos, pc, stream)) != hipSuccess) return e;  // SwiGLU into h2
      if ((e = gemm(a, ST_DN, l, pos, pc, stream, next_gain)) != hipSuccess) return e;
    }
  }
  return hipGetLastError();
}

}  // namespace kie
