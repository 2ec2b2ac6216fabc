// Device helpers shared by the HIP kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs2 {

// Enqueue `kernel` on `st`; with events (the timed entry points) hipExtLaunchKernelGGL
// sets them to the kernel's own start and end times.
template <typename Ev, typename K, typename... Args>
inline void launch_on(const Ev* ev, K kernel, dim3 grid, dim3 block, uint32_t shm, hipStream_t st, Args... args) {
  if (ev != nullptr)
    hipExtLaunchKernelGGL(kernel, grid, block, shm, st, ev->begin, ev->end, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shm, st, args...);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

constexpr float kNegInf = -__builtin_huge_valf();

// v_dot2_f32_bf16: c + a.lo*b.lo + a.hi*b.hi; bf16 x bf16 products are exact in fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// DPP lane permutations inside a row of 16 lanes.
constexpr int kDppXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppXor3 = 0x1B;   // quad_perm [3,2,1,0]
constexpr int kDppMirror8 = 0x141;  // row_half_mirror: lane i <-> 7-i inside each 8
constexpr int kDppRor8 = 0x128;  // row_ror:8: lane i <-> i^8 inside each 16

// Every lane has a source lane under these permutations, so bound_ctrl (read 0 from a
// missing source) changes nothing; it lets the compiler fold the move into the VALU
// instruction that consumes it (v_add_f32_dpp, v_max_f32_dpp, ...).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}

// Streaming loads with the non-temporal hint (global_load ... nt): data read once is
// not kept for reuse in the caches.  On MI355X a 2 GiB stream read this way runs at
// ~7.0 TB/s against ~6.2 TB/s with ordinary loads.
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ uint2 load_nt(const uint2* p) {
  const u32x2_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(t[0], t[1]);
}
__device__ __forceinline__ float load_nt(const float* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

// bf16 pair word -> two fp32 values (low element, high element).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Two OCP E4M3FN codes (bytes 0-1 or 2-3 of w) -> two fp32 values (exact).
__device__ __forceinline__ f32x2_t fp8x2_to_f32(uint32_t w, bool high) {
  return high ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true)
              : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
}

// Two OCP E4M3FN codes -> one bf16 pair word (exact: 3 mantissa bits fit in 7).
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool high) {
  bf16x2_t r = high ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                    : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts inside each row
// (a lane without a source lane adds 0)
// of 16 lanes, then the row totals (lanes 15, 31, 47) are added to the later rows.
__device__ __forceinline__ uint32_t wave_prefix_incl(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
  const int row = (int)(__lane_id() >> 4);
  x += (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
  return x;
}

// Number of set bits of `mask` in the lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Maximum over the 64 lanes of a wave, returned in every lane.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppMirror8>(x));
  x = fmaxf(x, dpp<kDppRor8>(x));
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

template <typename T>
__device__ __forceinline__ T atomic_load_relaxed(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace hs2
