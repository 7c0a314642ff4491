// Shared device helpers for the PISA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pisa.h"

namespace pisa {

constexpr int kWave = 64;
constexpr int kMaxGroup = 16;  // query heads per KV head supported by the kernels

// Pyramid geometry passed to kernels by value: level l (1-based) holds
// size[l-1] rows starting at row off[l-1] of a KV head's [R, d] pyramid.
struct LevelTable {
  int n;
  int rows;
  int size[PISA_MAX_LEVELS];
  int off[PISA_MAX_LEVELS];
};

typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float -> bfloat16 bits (NaN stays NaN), branch-free.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t nan = (u >> 16) | 0x40u;
  return uint16_t((u & 0x7fffffffu) > 0x7f800000u ? nan : r);
}

// Elements of T covered by one 16-byte load.
template <typename T> struct Vec16;
template <> struct Vec16<float> { static constexpr int n = 4; };
template <> struct Vec16<bf16_t> { static constexpr int n = 8; };

// Load 16 bytes at p (16-byte aligned) and widen to floats.
__device__ __forceinline__ void load16(const float* p, float* out) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}
__device__ __forceinline__ void load16(const bf16_t* p, float* out) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ void store_from_f32(float* p, float x) { *p = x; }
__device__ __forceinline__ void store_from_f32(bf16_t* p, float x) { *p = f32_to_bf16(x); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Lanes below this one whose bit is set in mask.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int readlane_i(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}
__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Compiler ordering point for LDS traffic between lanes of one wave (the
// hardware keeps a wave's LDS operations in order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier for data that LDS stores wrote before it: waits only for
// this thread's LDS operations (s_waitcnt lgkmcnt(0), no memory fence), so
// global loads and stores still in flight keep running across it.  The empty
// asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt(63) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N): wait until at most the N most recent vector memory
// operations of this thread are outstanding (gfx9 counts loads and stores
// together and retires them in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Hardware exp2/log2 (v_exp_f32 / v_log_f32, about 1 ulp).  Used where the
// argument of exp2 is <= 0 (results below 2^-126 flush to 0, which a
// log-sum-exp does not notice) and the argument of log2 is >= 1.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float pos_inf() { return __int_as_float(0x7f800000); }
__device__ __forceinline__ float neg_inf() { return __int_as_float(0xff800000); }

// Ranking order of the selection: higher score first, ties to the lower index.
// Bitwise (not short-circuit) so that it compiles to compares and selects.
__device__ __forceinline__ bool ranks_before(float s1, int i1, float s2, int i2) {
  return (s1 > s2) | ((s1 == s2) & (i1 < i2));
}

// Packed 32-bit rank key of a candidate in slot `slot` (0..31) whose score is
// s, given the best score smax among the candidates being ranked.  The upper
// 27 bits hold the distance below smax in fixed point (quantum 2^-12 of the
// score's unit, saturating 2^15 units below smax); the low 5 bits hold
// 31 - slot.  A larger key ranks first, so candidates whose scores differ by
// more than 2^-11 units (plus the fp32 rounding of smax - s) are ordered by
// score whatever their magnitude, and equal scores go to the lower slot, i.e.
// the lower node index.  Keys of ranked candidates are >= 32, so 0 can mark an
// unranked slot.
__device__ __forceinline__ uint32_t rank_key_rel(float s, float smax, int slot) {
  constexpr uint32_t kTop = (1u << 27) - 1u;
  // (smax - s) * 4096 as one fma: scaling by a power of two commutes with
  // the rounding, and smax * 4096 is shared by every slot of a decision
  const float dq = fmaf(s, -4096.f, smax * 4096.f);  // >= 0; NaN when both are -inf
  const uint32_t qv = dq < float(kTop - 1u) ? uint32_t(dq) : kTop - 1u;
  return ((kTop - qv) << 5) | uint32_t(31 - slot);
}

}  // namespace pisa
