// device_common.h -- small device helpers shared by the kernels of this library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace kie {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0]|[15:14], expcnt[6:4], lgkmcnt[11:8])
constexpr int kWaitLgkm0 = 0xC07F;
constexpr int kWaitVm0 = 0x0F70;

__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// Exchange words live in ordinary device memory shared by all XCDs. Agent-scope relaxed atomic
// loads and stores are coherent across the XCDs' separate L2 caches (they carry the sc1 policy
// bit), so a 64-bit word written by one CU is seen whole, with its tag, by any other CU.
__device__ __forceinline__ uint64_t ld_x(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_x(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_x32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tag_f(float v, uint32_t epoch) {
  return ((uint64_t)__float_as_uint(v) << 32) | epoch;
}
__device__ __forceinline__ uint64_t tag_u(uint32_t v, uint32_t epoch) { return ((uint64_t)v << 32) | epoch; }

// LDS words shared by the waves of one workgroup.
__device__ __forceinline__ uint32_t lds_ld(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet). Written as a select,
// so that no branch (and no change of the execution mask) surrounds each conversion.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  return (u & 0x7fffffffu) > 0x7f800000u ? ((u >> 16) | 0x40u) : rne;
}

// Buffer resource over [base, base + bytes): a raw buffer load through it whose per-lane offset
// (VGPR offset + immediate) is at or past `bytes` returns zeros without touching memory. The
// scalar offset is not part of that check, so all offsets here are per-lane.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int kLoadNT = 2;  // cache policy of weight and KV loads: streamed once (nontemporal)
__device__ __forceinline__ v4u load16(__amdgpu_buffer_rsrc_t rs, uint32_t voff) {
  return __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, kLoadNT));
}
// LDS byte address of a pointer into the workgroup's shared memory
typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_u8*)p; }
// 16 bytes per lane from the buffer straight into LDS at lds_base + 16 * lane (gfx950
// buffer_load_dwordx4 ... lds; M0 holds the wave-uniform LDS address). Nothing is returned to
// registers: the caller waits on the vector memory counter before reading the LDS.
__device__ __forceinline__ void load16_lds(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t lds_base) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rs), "{m0}"(lds_base) : "memory");
}

template <typename T>
__device__ __forceinline__ T wave_bcast(T v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}
__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), lane));
}

}  // namespace kie

namespace kie {
// DPP lane permutations (gfx9 encodings) used for in-register reductions: no LDS round trip.
constexpr int kDppQuad1032 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuad2301 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowRor8 = 0x128;  // row_ror:8 -- within each row of 16 lanes, lane i reads lane i ^ 8

template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xF, false));
}
// Sum over each row of 16 lanes; every lane of the row receives the row's sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kDppQuad1032>(v);
  v += dpp_f<kDppQuad2301>(v);
  v += dpp_f<kDppRowHalfMirror>(v);
  v += dpp_f<kDppRowMirror>(v);
  return v;
}
// Sum over each row of 8 lanes (half rows); every lane receives its half row's sum.
__device__ __forceinline__ float row8_sum(float v) {
  v += dpp_f<kDppQuad1032>(v);
  v += dpp_f<kDppQuad2301>(v);
  v += dpp_f<kDppRowHalfMirror>(v);
  return v;
}
// Sum over all 64 lanes in a fixed order, returned wave-uniform.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const float r0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0));
  const float r1 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 16));
  const float r2 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 32));
  const float r3 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 48));
  return (r0 + r1) + (r2 + r3);
}
// The two values of the lane pair {i, i ^ off}, off = 8, 16 or 32 (a compile-time constant after
// unrolling), in a fixed order: *lo from the lane whose bit `off` is clear, *hi from the other;
// both lanes of the pair get the same two values. No LDS round trip: off 8 is a DPP rotation by 8
// within the rows of 16 lanes; 16 and 32 are the gfx950 lane-swap instructions, which exchange a
// row of 16 lanes with its neighbour row (v_permlane16_swap) and a half wave with the other half
// (v_permlane32_swap). Given the same register twice, the swap leaves the even row's (lower
// half's) values in its first result and the odd row's (upper half's) in its second, in every lane.
__device__ __forceinline__ void lane_pair(float v, int off, int lane, float* lo, float* hi) {
  if (off == 8) {
    const float o = dpp_f<kDppRowRor8>(v);
    const bool up = (lane & 8) != 0;
    *lo = up ? o : v;
    *hi = up ? v : o;
  } else if (off == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    *lo = __uint_as_float(r[0]);
    *hi = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    *lo = __uint_as_float(r[0]);
    *hi = __uint_as_float(r[1]);
  }
}
// Sums of lanes 0..31 and of lanes 32..63 (fixed order), returned wave-uniform.
__device__ __forceinline__ void half_wave_sums(float v, float* lo, float* hi) {
  v = row16_sum(v);
  v += dpp_f<kDppRowBcast15, 0xA>(v);  // rows 1 and 3 add the last lane of rows 0 and 2
  *lo = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 31));
  *hi = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}
}  // namespace kie
