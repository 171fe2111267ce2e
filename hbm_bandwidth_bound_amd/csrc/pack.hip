// pack.hip -- set-up kernels: the weight packer and the RoPE table; plus two plain streaming
// kernels used to measure the memory system (copy and read) next to the decoder.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.h"
#include "layout.h"
#include "monokernel.h"

namespace kie {

// One block row per stream (WG w = x / 8, wave v = x % 8); it writes the stream's tiles of one
// layer (or of the LM head). Each thread writes one lane (16 B) of a tile: 8 B of row A and 8 B of
// row B at the same k (4 bf16 weights each; with TK = 2 * kTileK, 8 one-byte codes: 4 from each
// half of the tile's 512). Slots of missing units are written as zeros.
template <int TK>
__global__ void __launch_bounds__(256) pack_layer_kernel(PackArgs a) {
  constexpr int EB = 2 * kTileK / TK;  // bytes per weight
  const Shape& s = a.s;
  const int32_t w = blockIdx.x / kWaves, v = blockIdx.x % kWaves;
  const bool lm = a.layer == s.L;
  int32_t boff[ST_COUNT + 1];
  int32_t acc = 0;
  for (int st = ST_QKV; st <= ST_DN; ++st) {
    boff[st] = acc;
    if (s.in_stream(st)) acc += wave_batches(stage_geo<TK>(s, st, w), v);
  }
  boff[ST_LM] = acc;
  const int32_t layer_b = acc;
  const int32_t nb = lm ? lm_batches<TK>(s, w, v) : layer_b;
  const int64_t base = a.wbase[blockIdx.x] + (int64_t)a.layer * layer_b * kBatch;
  const int q = threadIdx.x % 64;
  for (int32_t t = blockIdx.y * 4 + threadIdx.x / 64; t < nb * kBatch; t += gridDim.y * 4) {
    int st = ST_LM;
    int32_t b = t / kBatch;
    if (!lm) {
      st = ST_QKV;
      while (st < ST_DN && b >= boff[st + 1]) ++st;
      b -= boff[st];
    }
    const StageGeo g = stage_geo<TK>(s, st, w);
    const int32_t sl = t % kBatch, us = sl / g.ks, tt = sl % g.ks;
    const int32_t u = v + kWaves * (b * g.upb + us);
    v4u out = v4u{0u, 0u, 0u, 0u};
    if (u < g.nu) {
      const int32_t lp = u / g.S, j = (u % g.S) * g.ks + tt;
      int mat;
      int32_t ra, rb;
      pair_rows(s, st, stage_pair(s, st, g.pb + lp), &mat, &ra, &rb);
      const uint16_t *ma, *mb;
      if (st == ST_QKV) {
        ma = mb = mat == 0 ? a.wq : (mat == 1 ? a.wk : a.wv);
      } else if (st == ST_O) {
        ma = mb = a.wo;
      } else if (st == ST_RT) {
        ma = mb = a.wrouter;
      } else if (st == ST_GU) {
        ma = a.wgate;
        mb = a.wup;
      } else if (st == ST_DN) {
        ma = mb = a.wdown;
      } else {
        ma = mb = a.lm_head;
      }
      const int32_t K = s.stage_k(st);
      if constexpr (EB == 2) {  // bf16: k = 4q .. 4q + 3 of the tile's 256
        const int32_t k = j * TK + q * 4;
        const uint2 xa = *(const uint2*)(ma + (int64_t)ra * K + k);
        const uint2 xb = *(const uint2*)(mb + (int64_t)rb * K + k);
        out = v4u{xa.x, xa.y, xb.x, xb.y};
      } else {  // 8-bit: k = 4q .. 4q + 3 and 256 + 4q .. + 3 of the tile's 512 (one word each)
        const uint8_t* pa = (const uint8_t*)ma + (int64_t)ra * K + j * TK + q * 4;
        const uint8_t* pb = (const uint8_t*)mb + (int64_t)rb * K + j * TK + q * 4;
        out = v4u{*(const uint32_t*)pa, *(const uint32_t*)(pa + kTileK), *(const uint32_t*)pb,
                  *(const uint32_t*)(pb + kTileK)};
      }
    }
    *(v4u*)(a.packed + (base + t) * kTileBytes + q * 16) = out;
  }
}

hipError_t launch_pack_layer(const PackArgs& a, hipStream_t st) {
  if (a.w8)
    hipLaunchKernelGGL(pack_layer_kernel<2 * kTileK>, dim3(a.s.nwg * kWaves, 16), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(pack_layer_kernel<kTileK>, dim3(a.s.nwg * kWaves, 16), dim3(256), 0, st, a);
  return hipGetLastError();
}

// The expert region of one mixture-of-experts layer: every expert's gate/up pairs (row p of W_gate
// and of W_up) and down pairs (rows 2p, 2p + 1 of W_down), each as whole tiles in k order (the
// placement of expert_gu_tile / expert_dn_tile). One thread writes one lane of a tile.
__global__ void __launch_bounds__(256) pack_experts_kernel(PackArgs a) {
  const Shape& s = a.s;
  const int32_t ktd = s.d / kTileK, kte = s.Fe / kTileK, hp = s.d / 2;
  const int64_t ngu = (int64_t)s.E * s.Fe * ktd, ndn = (int64_t)s.E * hp * kte;
  const int q = threadIdx.x % 64;
  uint8_t* region = a.packed + a.expert_offset;
  for (int64_t t = (int64_t)blockIdx.x * 4 + threadIdx.x / 64; t < ngu + ndn; t += (int64_t)gridDim.x * 4) {
    uint2 xa, xb;
    int64_t dst;
    if (t < ngu) {
      const int32_t kt = (int32_t)(t % ktd);
      const int64_t r = t / ktd;
      const int32_t p = (int32_t)(r % s.Fe), e = (int32_t)(r / s.Fe);
      const int64_t off = ((int64_t)e * s.Fe + p) * s.d + kt * kTileK + q * 4;
      xa = *(const uint2*)(a.egate + off);
      xb = *(const uint2*)(a.eup + off);
      dst = expert_gu_tile(s, a.layer, e, p, kt);
    } else {
      const int64_t t2 = t - ngu;
      const int32_t kk = (int32_t)(t2 % kte);
      const int64_t r = t2 / kte;
      const int32_t p = (int32_t)(r % hp), e = (int32_t)(r / hp);
      const int64_t off = ((int64_t)e * s.d + 2 * p) * s.Fe + kk * kTileK + q * 4;
      xa = *(const uint2*)(a.edown + off);
      xb = *(const uint2*)(a.edown + off + s.Fe);
      dst = expert_dn_tile(s, a.layer, e, p, kk);
    }
    *(v4u*)(region + dst * kTileBytes + q * 16) = v4u{xa.x, xa.y, xb.x, xb.y};
  }
}

hipError_t launch_pack_experts(const PackArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(pack_experts_kernel, dim3(2048), dim3(256), 0, st, a);
  return hipGetLastError();
}

// rope[p][i] = (cos, sin) of p * theta^(-2i/hd), angle in fp64, rounded to fp32
// Zero `bytes` bytes at p (16-byte aligned, bytes a multiple of 4): 16-byte stores for the body,
// then 4-byte stores. A kernel rather than a memset, so that the set-up can be captured in a graph.
__global__ void __launch_bounds__(256) fill_zero_kernel(uint8_t* p, int64_t bytes) {
  const int64_t n16 = bytes / 16;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    ((v4u*)p)[i] = v4u{0u, 0u, 0u, 0u};
  const int64_t t = n16 * 16 + ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (t < bytes) *(uint32_t*)(p + t) = 0u;
}
hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t st) {
  if (bytes <= 0) return hipSuccess;
  int64_t blocks = (bytes / 16 + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 4096 ? 4096 : blocks);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((uint32_t)blocks), dim3(256), 0, st, (uint8_t*)p, bytes);
  return hipGetLastError();
}

// First tile of every wave's stream in the packed image (an exclusive prefix sum of the stream
// lengths in (WG, wave) order) and the total, wbase[nwg * 8]. One block: each thread sums a run of
// consecutive streams, the block scans the run totals.
template <int TK>
__global__ void __launch_bounds__(1024) stream_bases_kernel(Shape s, int64_t* wbase) {
  __shared__ int64_t part[1024];
  const int32_t n = s.nwg * kWaves;
  const int32_t per = (n + 1023) / 1024;
  const int32_t b0 = threadIdx.x * per, b1 = b0 + per < n ? b0 + per : n;
  int64_t sum = 0;
  for (int32_t i = b0; i < b1; ++i) sum += stream_tiles<TK>(s, i / kWaves, i % kWaves);
  part[threadIdx.x] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {  // 1024 run totals, in order
    int64_t acc = 0;
    for (int i = 0; i < 1024; ++i) {
      const int64_t x = part[i];
      part[i] = acc;
      acc += x;
    }
    wbase[n] = acc;
  }
  __syncthreads();
  int64_t acc = part[threadIdx.x];
  for (int32_t i = b0; i < b1; ++i) {
    wbase[i] = acc;
    acc += stream_tiles<TK>(s, i / kWaves, i % kWaves);
  }
}
// The prompt pass's tile table (ptab_index): one thread per entry, each a packed_tile lookup;
// blockIdx.y is the layer.
template <int TK>
__global__ void __launch_bounds__(256) ptab_kernel(Shape s, const int64_t* wbase, int32_t* tab) {
  const int32_t l = blockIdx.y;
  const int64_t per = ptab_layer<TK>(s);
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < per; e += (int64_t)gridDim.x * 256) {
    int st = ST_QKV;
    int64_t o = e;
    while (o >= ptab_units<TK>(s, st)) o -= ptab_units<TK>(s, st++);
    const int32_t kt = s.stage_kt<TK>(st), ks = unit_tiles(kt), S = kt / ks;
    tab[(int64_t)l * per + e] = (int32_t)packed_tile<TK>(s, wbase, st, l, (int32_t)(o / S), (int32_t)(o % S) * ks);
  }
}
hipError_t launch_ptab(const Shape& s, bool w8, const int64_t* wbase, int32_t* tab, hipStream_t st) {
  const int64_t per = w8 ? ptab_layer<2 * kTileK>(s) : ptab_layer<kTileK>(s);
  const dim3 grid((unsigned)((per + 255) / 256 < 1024 ? (per + 255) / 256 : 1024), (unsigned)s.L);
  if (w8)
    hipLaunchKernelGGL(ptab_kernel<2 * kTileK>, grid, dim3(256), 0, st, s, wbase, tab);
  else
    hipLaunchKernelGGL(ptab_kernel<kTileK>, grid, dim3(256), 0, st, s, wbase, tab);
  return hipGetLastError();
}
hipError_t launch_stream_bases(const Shape& s, bool w8, int64_t* wbase, hipStream_t st) {
  if (w8)
    hipLaunchKernelGGL(stream_bases_kernel<2 * kTileK>, dim3(1), dim3(1024), 0, st, s, wbase);
  else
    hipLaunchKernelGGL(stream_bases_kernel<kTileK>, dim3(1), dim3(1024), 0, st, s, wbase);
  return hipGetLastError();
}

// Host floats to device memory through kernel arguments (no host staging, capturable): chunks of
// up to kFloatChunk values.
__global__ void set_floats_kernel(FloatChunk c) {
  if ((int32_t)threadIdx.x < c.n) c.dst[threadIdx.x] = c.v[threadIdx.x];
}
hipError_t launch_set_floats(float* dst, const float* src, int32_t n, hipStream_t st) {
  for (int32_t i = 0; i < n; i += kFloatChunk) {
    FloatChunk c;
    c.dst = dst + i;
    c.n = n - i < kFloatChunk ? n - i : kFloatChunk;
    for (int32_t j = 0; j < c.n; ++j) c.v[j] = src[i + j];
    hipLaunchKernelGGL(set_floats_kernel, dim3(1), dim3(kFloatChunk), 0, st, c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

__global__ void rope_table_kernel(float2* rope, int32_t max_seq, int32_t hd, float theta) {
  const int32_t half = hd / 2;
  const int64_t n = (int64_t)max_seq * half;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int32_t p = (int32_t)(e / half), i = (int32_t)(e % half);
    const double freq = pow((double)theta, -2.0 * (double)i / (double)hd);
    const double phi = (double)p * freq;
    rope[e] = make_float2((float)cos(phi), (float)sin(phi));
  }
}

hipError_t launch_rope_table(float2* rope, int32_t max_seq, int32_t hd, float theta, hipStream_t st) {
  hipLaunchKernelGGL(rope_table_kernel, dim3(1024), dim3(256), 0, st, rope, max_seq, hd, theta);
  return hipGetLastError();
}

// ------------------------------------------------------------------ memory-system probes
// Plain copy of n16 16-byte words, one contiguous slice per block (the calibration kernel for the
// hardware traffic counters: it reads and writes exactly 16 * n16 bytes each).
__global__ void __launch_bounds__(512) stream_copy_kernel(v4u* __restrict__ dst, const v4u* __restrict__ src, int64_t n16) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b = per * blockIdx.x;
  const int64_t e = b + per < n16 ? b + per : n16;
  for (int64_t i = b + threadIdx.x; i < e; i += blockDim.x) dst[i] = __builtin_nontemporal_load(src + i);
}

// Read-only stream: the ceiling a weight-streaming kernel can reach (one slice per block, 8 loads
// in flight per thread).
__global__ void __launch_bounds__(512) stream_read_kernel(const v4u* __restrict__ src, int64_t n16, uint32_t* sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b = per * blockIdx.x;
  const int64_t e = b + per < n16 ? b + per : n16;
  uint32_t acc = 0;
  int64_t i = b + threadIdx.x;
  for (; i + 7 * 512 < e; i += 8 * 512) {
    v4u v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 512);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < e; i += 512) {
    const v4u v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the loads; practically never taken
}

hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, int32_t blocks, hipStream_t st) {
  hipLaunchKernelGGL(stream_copy_kernel, dim3(blocks), dim3(512), 0, st, (v4u*)dst, (const v4u*)src, bytes / 16);
  return hipGetLastError();
}
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t blocks, hipStream_t st) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(512), 0, st, (const v4u*)src, bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace kie
