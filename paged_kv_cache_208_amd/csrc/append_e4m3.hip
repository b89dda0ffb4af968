// Appending a token's K/V into E4M3 blocks with per-(block, kv head) scales
// for gfx950.  The quantized (Q8/FP8) KV cache is a listed item of
// "Roadmap: vLLM-style serving features for TornadoVM batched decode"
// (Sampling / logits); the policy kept here holds each block's scale at the
// running amax of its rows over 448:
//   a = max |x| of the new row; s_old = scale (0 for a block's first row);
//   a > 448 * s_old: s_new = a / 448 and rows 0..r-1 are re-encoded as
//                    enc((dec(c) * s_old) / s_new);   else s_new = s_old;
//   row r = enc(x / s_new)  (zeros while s_new is 0).
// Every step is a float32 operation in that order (IEEE multiply and
// correctly rounded divide), enc rounds to nearest even on gfx950's
// converter after clamping to +-448.
//
// One wave per (token, kv head, pool): the new row is D fp16 values (one or
// two per lane), the block's earlier rows r * D bytes (four per lane per
// pass); blocks of 16 or 32 tokens.  The decode step appends through this
// kernel too, each sequence's new token at its last position.
#include "device.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -kE4M3Max), kE4M3Max); }

// Two float32 values to two E4M3 codes (low 16 bits), round to nearest even.
__device__ __forceinline__ uint32_t enc2(float a, float b) {
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false)) & 0xffffu;
}

template <int D>
__global__ __launch_bounds__(kWave) void append_e4m3_kernel(AppendE4m3Args a) {
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const int lane = threadIdx.x;
  int64_t slot = -1;
  if (a.slot_mapping) {
    slot = a.slot_mapping[t];
  } else {
    const int L = a.context_lens[t];
    if (L > 0) slot = int64_t(a.block_tables[size_t(t) * a.MBS + (L - 1) / a.bs]) * a.bs + (L - 1) % a.bs;
  }
  if (slot < 0) return;
  const int64_t n = slot / a.bs;
  const int r = int(slot % a.bs);
  uint8_t* tile = (is_v ? a.v_pool : a.k_pool) + (size_t(n) * a.Hkv + h) * a.bs * D;
  float* scale = (is_v ? a.v_scale : a.k_scale) + size_t(n) * a.Hkv + h;
  const _Float16* x = static_cast<const _Float16*>(is_v ? a.v_new : a.k_new) + (size_t(t) * a.Hkv + h) * D;

  constexpr int E = D / kWave;  // new-row elements per lane (1 or 2)
  float xv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) xv[e] = float(x[lane * E + e]);
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(xv[e]));
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));

  const float s_old = r > 0 ? *scale : 0.0f;
  float s_new = s_old;
  if (amax > kE4M3Max * s_old) {
    s_new = amax / kE4M3Max;
    if (r > 0 && s_old != 0.0f) {
      uint32_t* w = reinterpret_cast<uint32_t*>(tile);
      for (int i = lane; i < r * D / 4; i += kWave) {
        const uint32_t c = w[i];
        const float2_t lo = e4m3x2_to_float2<false>(c);
        const float2_t hi = e4m3x2_to_float2<true>(c);
        const float v0 = (lo.x * s_old) / s_new, v1 = (lo.y * s_old) / s_new;
        const float v2 = (hi.x * s_old) / s_new, v3 = (hi.y * s_old) / s_new;
        w[i] = enc2(v0, v1) | (enc2(v2, v3) << 16);
      }
    }
  }
  float q[2] = {0.0f, 0.0f};
  if (s_new != 0.0f)
#pragma unroll
    for (int e = 0; e < E; ++e) q[e] = xv[e] / s_new;
  const uint32_t codes = enc2(q[0], q[1]);
  uint8_t* row = tile + r * D + lane * E;
  if constexpr (E == 2)
    *reinterpret_cast<uint16_t*>(row) = uint16_t(codes);
  else
    *row = uint8_t(codes);
  if (lane == 0) *scale = s_new;
}

}  // namespace

hipError_t launch_append_e4m3(const AppendE4m3Args& a, int T, int D, hipStream_t stream) {
  const dim3 grid(unsigned(T), unsigned(a.Hkv), 2u);
  if (D == 64)
    hipLaunchKernelGGL(append_e4m3_kernel<64>, grid, dim3(kWave), 0, stream, a);
  else if (D == 128)
    hipLaunchKernelGGL(append_e4m3_kernel<128>, grid, dim3(kWave), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
