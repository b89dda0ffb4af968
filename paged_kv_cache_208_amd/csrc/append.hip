// paged_kv_append kernels for gfx950.
//
// Plain scatter ("Distributed LLM Inference Serving Platform", section
// 5.1): token i's K and V rows go to pool slot s = slot_mapping[i], i.e.
// block s / BS, row s % BS of every kv head's rows (BS = 16 or 32 tokens per
// block); s < 0 skips the token.
//
// Fused Qwen3 prologue ("Roadmap: vLLM-style serving features for TornadoVM
// batched decode", Core batched decode): before the scatter, every q head
// (rewritten in place) and k head of the token is RMS-normalised over D with
// its gamma and rotated by split-half RoPE at pos = context_lens[i] - 1.
// The rotation angles depend only on (pos, pair index), so a workgroup
// computes them once per token in fp64 and keeps cos/sin in LDS.
#include "device.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kAppendThreads = 256;

// Plain scatter: each thread moves 16-byte chunks of the token's K and V.
template <int D>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  const int t = blockIdx.x;
  const int64_t slot = a.slot_mapping[t];
  if (slot < 0) return;
  const int64_t blk = slot / a.bs;
  const int row = int(slot % a.bs);
  constexpr int CPH = D / 8;  // 16-byte chunks per head row
  const int chunks = a.Hkv * CPH;
  for (int i = threadIdx.x; i < chunks; i += kAppendThreads) {
    const int h = i / CPH;
    const int cc = i % CPH;
    const size_t src = (size_t(t) * a.Hkv + h) * D + cc * 8;
    const size_t dst = ((size_t(blk) * a.Hkv + h) * a.bs + row) * D + cc * 8;
    const u32x4 kx = *reinterpret_cast<const u32x4*>(static_cast<const _Float16*>(a.k_new) + src);
    const u32x4 vx = *reinterpret_cast<const u32x4*>(static_cast<const _Float16*>(a.v_new) + src);
    *reinterpret_cast<u32x4*>(static_cast<_Float16*>(a.k_pool) + dst) = kx;
    *reinterpret_cast<u32x4*>(static_cast<_Float16*>(a.v_pool) + dst) = vx;
  }
}

// Fused: one token per workgroup.  A head row of D fp16 values is held by
// LPH = D / 8 lanes (8 values each); a wave covers 64 / LPH heads at once.
template <int D>
__global__ __launch_bounds__(kAppendThreads) void append_fused_kernel(AppendArgs a) {
  constexpr int LPH = D / 8;
  constexpr int HALF = D / 2;
  constexpr int HPW = kWave / LPH;                    // heads per wave pass
  constexpr int HPB = HPW * (kAppendThreads / kWave);  // heads per block pass
  __shared__ float s_cos[HALF];
  __shared__ float s_sin[HALF];

  const int t = blockIdx.x;
  const int64_t slot = a.slot_mapping[t];
  const int pos = a.context_lens[t] - 1;
  for (int i = threadIdx.x; i < HALF; i += kAppendThreads) {
    const double freq = pow(double(a.theta), -2.0 * double(i) / double(D));
    const double ang = double(pos) * freq;
    double sn, cs;
    sincos(ang, &sn, &cs);
    s_cos[i] = float(cs);
    s_sin[i] = float(sn);
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane % LPH;
  const bool upper = c >= LPH / 2;
  const int pair0 = (c % (LPH / 2)) * 8;  // pair index of this lane's first element
  const int nheads = a.Hq + 2 * a.Hkv;
  const int64_t blk = slot / a.bs;
  const int row = int(slot % a.bs);

  for (int hh = (threadIdx.x / kWave) * HPW + lane / LPH; hh < nheads; hh += HPB) {
    const _Float16* src;
    _Float16* dst;
    const float* gamma = nullptr;
    if (hh < a.Hq) {
      src = static_cast<const _Float16*>(a.q) + (size_t(t) * a.Hq + hh) * D;
      dst = static_cast<_Float16*>(a.q) + (size_t(t) * a.Hq + hh) * D;
      gamma = a.gamma_q;
    } else {
      const bool is_k = hh < a.Hq + a.Hkv;
      const int h = is_k ? hh - a.Hq : hh - a.Hq - a.Hkv;
      src = static_cast<const _Float16*>(is_k ? a.k_new : a.v_new) + (size_t(t) * a.Hkv + h) * D;
      dst = slot < 0 ? nullptr
                     : static_cast<_Float16*>(is_k ? a.k_pool : a.v_pool) +
                           ((size_t(blk) * a.Hkv + h) * a.bs + row) * D;
      if (is_k) gamma = a.gamma_k;
    }
    const u32x4 raw = *reinterpret_cast<const u32x4*>(src + c * 8);
    u32x4 res = raw;
    if (gamma != nullptr) {
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
      float x[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const half2_t h2 = as_half2(w[k]);
        x[2 * k] = float(h2.x);
        x[2 * k + 1] = float(h2.y);
      }
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
      ss = group_sum<LPH>(ss);
      const float inv = 1.0f / sqrtf(ss / float(D) + a.eps);
      float rr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) rr[e] = x[e] * inv * gamma[c * 8 + e];
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float y[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int e = 2 * k + u;
          const float partner = __shfl_xor(rr[e], LPH / 2);
          const float cs = s_cos[pair0 + e];
          const float sn = s_sin[pair0 + e];
          y[u] = upper ? fmaf(rr[e], cs, partner * sn) : fmaf(rr[e], cs, -partner * sn);
        }
        o[k] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)y[0], (_Float16)y[1]});
      }
      res = u32x4{o[0], o[1], o[2], o[3]};
    }
    if (dst != nullptr) *reinterpret_cast<u32x4*>(dst + c * 8) = res;
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int T, int D, bool fused, hipStream_t stream) {
  const dim3 grid{unsigned(T)}, block{unsigned(kAppendThreads)};
  if (D == 128) {
    if (fused) hipLaunchKernelGGL(append_fused_kernel<128>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(append_kernel<128>, grid, block, 0, stream, a);
  } else if (D == 64) {
    if (fused) hipLaunchKernelGGL(append_fused_kernel<64>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(append_kernel<64>, grid, block, 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
