// bsa_device.h -- device helpers shared by the gfx950 kernels of libbsa.
// Internal to the library (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// streaming (non-temporal) 16-byte loads of data read exactly once
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream(const uint2* p) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ float4 ld_stream(const float4* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// bf16 pair in a dword -> two fp32 (exact)
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const uint4& w, float* f) {
  f[0] = bf_lo(w.x); f[1] = bf_hi(w.x);
  f[2] = bf_lo(w.y); f[3] = bf_hi(w.y);
  f[4] = bf_lo(w.z); f[5] = bf_hi(w.z);
  f[6] = bf_lo(w.w); f[7] = bf_hi(w.w);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// a.x*b.x + a.y*b.y + c on bf16 pairs, fp32 accumulate (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// DPP lane movement inside a row of 16 lanes
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL,
                                                    0xf, 0xf, false));
}
constexpr int DPP_QUAD_1032 = 0xb1;  // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4e;  // quad_perm [2,3,0,1]
constexpr int DPP_ROW_ROR4 = 0x124;
constexpr int DPP_ROW_ROR8 = 0x128;

// all-reduce over each row of 16 lanes; every lane of the row gets the result
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<DPP_QUAD_1032>(x);
  x += dpp<DPP_QUAD_2301>(x);
  x += dpp<DPP_ROW_ROR4>(x);
  x += dpp<DPP_ROW_ROR8>(x);
  return x;
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<DPP_QUAD_1032>(x));
  x = fmaxf(x, dpp<DPP_QUAD_2301>(x));
  x = fmaxf(x, dpp<DPP_ROW_ROR4>(x));
  x = fmaxf(x, dpp<DPP_ROW_ROR8>(x));
  return x;
}

__device__ __forceinline__ float readlane(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// wave64 reductions; the (wave-uniform) result is returned in every lane
__device__ __forceinline__ float wave_max(float x) {
  x = row16_max(x);
  return fmaxf(fmaxf(readlane(x, 0), readlane(x, 16)), fmaxf(readlane(x, 32), readlane(x, 48)));
}
__device__ __forceinline__ float wave_sum(float x) {
  x = row16_sum(x);
  return (readlane(x, 0) + readlane(x, 16)) + (readlane(x, 32) + readlane(x, 48));
}

// max(a, b) for non-NaN operands as a median with +inf: the compiler emits
// v_max3 directly, with none of the canonicalising v_max x, x, x that fmaxf
// puts before every operand
__device__ __forceinline__ float fmax_nc(float a, float b) {
  return __builtin_amdgcn_fmed3f(a, b, INFINITY);
}

// max of x over the lane pair (l, l ^ 16), resp. (l, l ^ 32), in both lanes:
// v_permlane16_swap exchanges the odd 16-lane rows of its first operand with
// the even rows of its second, v_permlane32_swap the upper half of the first
// with the lower half of the second; with x in both operands the two results
// hold x of the two partners.  VALU only (no LDS round trip as for a
// ds_bpermute shuffle).  The maximum is a v_med3 against +inf held in an SGPR
// the compiler cannot see into: with the constant it would fold the median to
// a plain max and canonicalise both swap results first.
__device__ __forceinline__ float opaque_inf() {
  float x;
  asm("s_mov_b32 %0, 0x7f800000" : "=s"(x));
  return x;
}
__device__ __forceinline__ float pair16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return __builtin_amdgcn_fmed3f(__uint_as_float(r[0]), __uint_as_float(r[1]), opaque_inf());
}
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return __builtin_amdgcn_fmed3f(__uint_as_float(r[0]), __uint_as_float(r[1]), opaque_inf());
}

// order LDS traffic between the lanes of one wave (no cross-wave barrier)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// fp32 -> uint32 key with the same order (-0 folded onto +0)
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  // negative: all bits flipped; otherwise the sign bit set (no compare mask)
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ uint32_t lane_prefix(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

}  // namespace bsa
