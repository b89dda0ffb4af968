// Device helpers for the gfx950 (CDNA4) kernels: wave64 lane arithmetic,
// DPP row reductions, bounded buffer loads and E4M3 -> fp16 conversion.
#pragma once
#include <hip/hip_runtime.h>
#include <cfloat>
#include <cstdint>

namespace pkv {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;
// XCDs of an MI355X; the workgroups of a launch are handed to them round-robin
// (workgroup i runs on XCD i % 8).
constexpr int kXcds = 8;

// gfx9 buffer resource word 3 for raw (untyped, stride 0) dword access.
constexpr int kRawBufferFlags = 0x00020000;

// DPP controls (gfx9 encoding)
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15-i within each 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, CTRL, 0xF, 0xF, false);
}

// Sum over aligned groups of N lanes (N in {1,2,4,8,16}); every lane of the
// group receives the group total.  Uses only row-local DPP moves.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group of 1..16 lanes");
  if constexpr (N >= 2) x += dpp<kDppQuadXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer resource over [base, base + bytes); loads past `bytes` return 0
// without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRawBufferFlags);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

__device__ __forceinline__ half2_t as_half2(uint32_t w) { return __builtin_bit_cast(half2_t, w); }

// Two E4M3 (OCP FN) codes in the low (hi == false) or high half of `w` to
// two fp16 values, exactly (every finite E4M3 value is an fp16 value).
// One gfx950 conversion (scale 1.0, so no rounding happens).
template <bool HI>
__device__ __forceinline__ half2_t e4m3x2_to_half2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// The same conversion multiplied by the power-of-two part of `scale`: the
// gfx950 instruction applies 2^floor(log2 scale) (the exponent of the fp32
// scale, as for MX block scales; checked on MI355X for every code and for
// scales 0, 2^-20 .. 2^10 and non-powers of two), so the product is the
// exact value code * 2^e rounded once to fp16 (exact unless it is an fp16
// subnormal).
template <bool HI>
__device__ __forceinline__ half2_t e4m3x2_to_half2_pow2(uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, scale, HI);
}

template <bool HI>
__device__ __forceinline__ float2_t e4m3x2_to_float2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

// scale / 2^floor(log2 scale), in [1, 2) for a normal positive scale (1.0 for
// zero): the part of the scale that the conversion above leaves out.
__device__ __forceinline__ float scale_mantissa(float scale) {
  return __uint_as_float((__float_as_uint(scale) & 0x007FFFFFu) | 0x3F800000u);
}

}  // namespace pkv
