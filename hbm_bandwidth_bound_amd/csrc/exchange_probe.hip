// Exchange-latency probes: the cost of the decode kernel's inter-workgroup hops measured on their
// own, per chiplet (XCD).
//
// The pages' account of the MI300X: eight compute dies (XCDs) sit on four I/O dies, each I/O die
// with two XCDs and two HBM stacks; an access that crosses to another I/O die pays extra latency
// (up to ~150 ns), so a grid barrier polled by every XCD from one place is uneven, and replicating
// the polled buffers so that each XCD polls memory behind its own I/O die brings the barrier to
// ~600 ns, even across compute units (aikraft.ru «3000 токенов в секунду…», §05, on the chiplet
// topology). These probes measure the same quantities on the running GPU:
//   * ping-pong between two workgroups on chosen chiplets (one-way latency = half a round trip);
//   * an all-gather hop of the decode kernel's shape (every workgroup publishes w tagged words and
//     waits for all of them), from one buffer or from one replica per chiplet;
//   * write-to-visible latency per 4 KiB page and reader chiplet, to find whether some pages are
//     nearer to some chiplets (the locality that replication relies on).
// Words are the decode kernel's exchange words: 64 bits, value << 32 | tag, written and read with
// agent-scope relaxed atomics. Every wait is bounded (kSpinTicks); a probe that gives up reports
// it instead of hanging. Times are s_memrealtime ticks (100 MHz).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kie_measure.h"
#include "layout.h"

namespace kie {
namespace {

constexpr uint64_t kSpinTicks = 20000000;  // 200 ms: a wait this long means a lost word
constexpr int kProbeThreads = 512;
constexpr int kGatherMax = 16;  // words each thread polls in one all-gather round

__device__ __forceinline__ uint64_t rt_ticks() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ uint32_t xcc_of_wave() {
  uint32_t x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(x));
  return x;
}

// Workgroups a and b bounce a counter `iters` times; a records the elapsed ticks.
// out: [0] ticks (0 if a wait gave up), [1] chiplet of a, [2] chiplet of b.
__global__ void __launch_bounds__(64) pingpong_kernel(uint64_t* flags, int32_t a, int32_t b, int32_t iters,
                                                      uint64_t* out) {
  const int32_t w = blockIdx.x;
  if (w != a && w != b) return;
  const bool is_a = w == a;
  if (threadIdx.x == 0) out[is_a ? 1 : 2] = xcc_of_wave();
  uint64_t* mine = flags + (is_a ? 0 : 32);  // separate 256-byte lines
  const uint64_t* theirs = flags + (is_a ? 32 : 0);
  const uint64_t t0 = rt_ticks();
  bool ok = true;
  for (int32_t i = 1; i <= iters && ok; ++i) {
    if (is_a && threadIdx.x == 0) st_x(mine, (uint64_t)i);
    const uint64_t s = rt_ticks();
    while (__builtin_amdgcn_readfirstlane((uint32_t)ld_x(theirs)) != (uint32_t)i) {
      if (rt_ticks() - s > kSpinTicks) {
        ok = false;
        break;
      }
    }
    if (!is_a && ok && threadIdx.x == 0) st_x(mine, (uint64_t)i);
  }
  if (is_a && threadIdx.x == 0) out[0] = ok ? rt_ticks() - t0 : 0;
}

// `rounds` all-gather hops: each workgroup publishes wpw words (to every replica), then polls all
// nwg * wpw words of its own chiplet's replica (replica xcc mod reps) until every tag matches.
// lat[w * rounds + r]: ticks from the workgroup's publication to its gather being complete.
// Buffers alternate by round parity; a workgroup can publish round r + 2 only after every
// workgroup has published r + 1, i.e. finished gathering r, so no unread word is overwritten.
__global__ void __launch_bounds__(kProbeThreads, 1) allgather_kernel(uint64_t* ex, int32_t wpw, int32_t rounds,
                                                                      int32_t reps, uint32_t* lat, uint32_t* xccs,
                                                                      uint32_t* fail) {
  __shared__ int32_t s_fail;
  const int32_t w = blockIdx.x, t = threadIdx.x, nwg = gridDim.x, n = nwg * wpw;
  const uint32_t x = xcc_of_wave();
  if (t == 0) {
    xccs[w] = x;
    s_fail = 0;
  }
  __syncthreads();
  const int32_t rep = reps > 1 ? (int32_t)(x % (uint32_t)reps) : 0;
  for (int32_t r = 1; r <= rounds; ++r) {
    uint64_t* buf = ex + (size_t)(r & 1) * reps * n;
    const uint64_t t0 = rt_ticks();
    if (t < wpw * reps) {
      const int32_t k = t % wpw;
      st_x(buf + (size_t)(t / wpw) * n + (size_t)w * wpw + k, ((uint64_t)(uint32_t)(w * wpw + k) << 32) | (uint32_t)r);
    }
    const uint64_t* src = buf + (size_t)rep * n;
    uint64_t wv[kGatherMax];
    uint32_t miss = 0;
#pragma unroll
    for (int k = 0; k < kGatherMax; ++k) {
      const int32_t e = t + k * kProbeThreads;
      if (e < n) {
        miss |= 1u << k;
        wv[k] = ld_x(src + e);
      }
    }
    const uint64_t s = rt_ticks();
    bool ok = true;
    while (true) {
#pragma unroll
      for (int k = 0; k < kGatherMax; ++k)
        if ((miss >> k & 1u) && (uint32_t)wv[k] == (uint32_t)r) miss &= ~(1u << k);
      if (!miss) break;
      if (rt_ticks() - s > kSpinTicks) {
        ok = false;
        break;
      }
#pragma unroll
      for (int k = 0; k < kGatherMax; ++k)
        if (miss >> k & 1u) wv[k] = ld_x(src + t + k * kProbeThreads);
    }
    if (!ok) s_fail = 1;
    __syncthreads();
    if (t == 0) lat[(size_t)w * rounds + (r - 1)] = (uint32_t)(rt_ticks() - t0);
    const bool give_up = s_fail != 0;
    __syncthreads();
    if (give_up) break;
  }
  if (t == 0 && s_fail) __hip_atomic_fetch_or(fail, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Page locality: `writer` writes (time << 32 | p + 1) into the first word of page p; one reader
// workgroup per chiplet (workgroups 8 .. 15 of the dispatch order) polls it and records the
// ticks from the write to the moment it sees it, then acknowledges; the writer moves to the next
// page once all eight have. out[p * 8 + c]: latency seen by the reader on chiplet c; acks[256]:
// the writer's chiplet.
__global__ void __launch_bounds__(64) page_latency_kernel(uint64_t* buf, int32_t npages, int32_t page_words,
                                                          int32_t writer, uint64_t* acks, uint32_t* out,
                                                          uint32_t* fail) {
  const int32_t w = blockIdx.x;
  const bool reader = w >= kXcds && w < 2 * kXcds;
  if (w != writer && !reader) return;
  const uint32_t c = xcc_of_wave() % kXcds;
  if (w == writer && threadIdx.x == 0) st_x(acks + kXcds * 32, (uint64_t)c);  // the writer's chiplet
  bool ok = true;
  for (int32_t p = 0; p < npages && ok; ++p) {
    uint64_t* word = buf + (size_t)p * page_words;
    if (w == writer) {
      if (threadIdx.x == 0) st_x(word, ((uint64_t)(uint32_t)rt_ticks() << 32) | (uint32_t)(p + 1));
      const uint64_t s = rt_ticks();
      for (int r = 0; r < kXcds && ok; ++r)  // every reader has seen page p
        while (__builtin_amdgcn_readfirstlane((uint32_t)ld_x(acks + r * 32)) != (uint32_t)(p + 1)) {
          if (rt_ticks() - s > kSpinTicks) {
            ok = false;
            break;
          }
        }
    }
    if (reader) {
      const uint64_t s = rt_ticks();
      uint64_t v = 0;
      while (true) {
        v = ld_x(word);
        if (__builtin_amdgcn_readfirstlane((uint32_t)v) == (uint32_t)(p + 1)) break;
        if (rt_ticks() - s > kSpinTicks) {
          ok = false;
          break;
        }
      }
      const uint32_t seen = (uint32_t)rt_ticks();
      if (threadIdx.x == 0) {
        out[(size_t)p * kXcds + c] = ok ? seen - __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) : 0xffffffffu;
        st_x(acks + (w - kXcds) * 32, (uint64_t)(p + 1));
      }
    }
  }
  if (!ok && threadIdx.x == 0) __hip_atomic_fetch_or(fail, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int32_t compute_units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

}  // namespace
}  // namespace kie

using namespace kie;

extern "C" {

kie_status kie_probe_pingpong(int32_t wg_a, int32_t wg_b, int32_t iters, uint64_t* flags_dev, uint64_t* out_dev,
                              void* hip_stream) {
  const int32_t nwg = compute_units();
  if (nwg <= 0) return KIE_ERR_HIP;
  if (!flags_dev || !out_dev || wg_a < 0 || wg_b < 0 || wg_a >= nwg || wg_b >= nwg || wg_a == wg_b || iters < 1 ||
      iters > 1000000)
    return KIE_ERR_INVALID_ARG;
  hipLaunchKernelGGL(pingpong_kernel, dim3(nwg), dim3(64), 0, (hipStream_t)hip_stream, flags_dev, wg_a, wg_b, iters,
                     out_dev);
  return hipGetLastError() == hipSuccess ? KIE_OK : KIE_ERR_HIP;
}

kie_status kie_probe_allgather(int32_t words_per_wg, int32_t rounds, int32_t replicas, uint64_t* ex_dev,
                               uint32_t* lat_dev, uint32_t* xcc_dev, uint32_t* fail_dev, void* hip_stream) {
  const int32_t nwg = compute_units();
  if (nwg <= 0) return KIE_ERR_HIP;
  if (!ex_dev || !lat_dev || !xcc_dev || !fail_dev || words_per_wg < 1 || rounds < 1 || rounds > 100000 ||
      (replicas != 1 && replicas != kXcds) || (int64_t)words_per_wg * replicas > kProbeThreads ||
      (int64_t)nwg * words_per_wg > (int64_t)kGatherMax * kProbeThreads)
    return KIE_ERR_INVALID_ARG;
  void* args[] = {&ex_dev, &words_per_wg, &rounds, &replicas, &lat_dev, &xcc_dev, &fail_dev};
  // every workgroup waits for every other: they must all be resident at once
  return hipLaunchCooperativeKernel((const void*)allgather_kernel, dim3(nwg), dim3(kProbeThreads), args, 0,
                                    (hipStream_t)hip_stream) == hipSuccess
             ? KIE_OK
             : KIE_ERR_HIP;
}

kie_status kie_probe_page_latency(int32_t npages, int32_t page_words, int32_t writer_wg, uint64_t* buf_dev,
                                  uint64_t* acks_dev, uint32_t* out_dev, uint32_t* fail_dev, void* hip_stream) {
  const int32_t nwg = compute_units();
  if (nwg <= 0) return KIE_ERR_HIP;
  if (!buf_dev || !acks_dev || !out_dev || !fail_dev || npages < 1 || page_words < 1 || nwg < 2 * kXcds ||
      writer_wg < 0 || writer_wg >= nwg || (writer_wg >= kXcds && writer_wg < 2 * kXcds))
    return KIE_ERR_INVALID_ARG;
  hipLaunchKernelGGL(page_latency_kernel, dim3(nwg), dim3(64), 0, (hipStream_t)hip_stream, buf_dev, npages,
                     page_words, writer_wg, acks_dev, out_dev, fail_dev);
  return hipGetLastError() == hipSuccess ? KIE_OK : KIE_ERR_HIP;
}

}  // extern "C"
