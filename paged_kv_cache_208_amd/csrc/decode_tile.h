// MFMA tile machinery shared by the decode kernels (gfx950).
//
// A (block, kv head) tile holds 16 token rows of K or V.  Lane l = 16 g + n16
// (g = lane group 0..3, n16 = 0..15) of a wave:
//   K:  row n16 of the tile, 16-byte pieces 4u + g of that row
//   QK: S^T = K Q^T with v_mfma_f32_16x16x32_f16; rows are tokens, columns
//       head slots; the lane receives tokens 4g .. 4g+3 of head slot n16
//   V:  rows 4g .. 4g+3, the D/16 dims starting at n16 * D/16
//   PV: O^T += V^T P^T with v_mfma_f32_16x16x16_f16; product i covers dim
//       (row * D/16 + i), so the lane accumulates head n16, dims
//       (4g + r) * D/16 + i.
// The QK result layout is exactly the B-operand layout of the PV product, so
// P never leaves the registers.
#pragma once
#include "device.h"
#include "kernels.h"

namespace pkv {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));


// Keeps the instruction scheduler from moving work on the current tile (and
// so its wait for that tile's data) above the next tile's loads.
__device__ __forceinline__ void issue_fence() { __builtin_amdgcn_sched_barrier(0); }

// s_waitcnt operand that waits until at most n vector memory operations of
// the wave are outstanding (they complete in issue order) and leaves the
// other counters alone.
constexpr int vmcnt_at_most(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// Read of a wave-uniform address that nothing writes during the launch (block
// tables, context lengths) through the scalar cache.  A vector load here would
// share the vmcnt counter with the KV loads in flight, and waiting for its
// result would drain them too.
__device__ __forceinline__ int32_t load_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}
__device__ __forceinline__ float load_uniform_f32(const float* p) {
  return *(const __attribute__((address_space(4))) float*)p;
}

// Partition statistics handed from one workgroup to another inside a launch
// are written and read with device-scope (agent) relaxed atomics, which the
// hardware keeps coherent across the XCDs' separate L2 caches without
// writing back or invalidating whole caches.  Ordinary accesses are used
// when the handoff happens across launches.
// 16-byte forms of the same coherent accesses (cache policy sc1, as the
// agent-scope atomics use), through a buffer resource; store16<false> is the
// plain store.
constexpr int kCoherentAux = 16;
__device__ __forceinline__ u32x4 load16_coherent(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherentAux);
}
template <bool COHERENT>
__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, int off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, COHERENT ? kCoherentAux : 0);
}

template <bool COHERENT>
__device__ __forceinline__ void store_f32(float* p, float v) {
  if constexpr (COHERENT) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}

__device__ __forceinline__ float load_f32_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// Reductions over the four lane groups of a head (lanes l, l^16, l^32,
// l^48) with VALU lane swaps (no LDS traffic).
__device__ __forceinline__ float group4_max(float x) {
  typedef uint32_t u2 __attribute__((ext_vector_type(2)));
  const u2 a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a.x), __uint_as_float(a.y));
  const u2 b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b.x), __uint_as_float(b.y));
}

__device__ __forceinline__ float group4_sum(float x) {
  typedef uint32_t u2 __attribute__((ext_vector_type(2)));
  const u2 a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a.x) + __uint_as_float(a.y);
  const u2 b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b.x) + __uint_as_float(b.y);
}

// cos / sin of the split-half RoPE angles pos * theta^(-2i/D), i < D/2,
// evaluated in fp64 once per workgroup ("Roadmap: vLLM-style serving features
// for TornadoVM batched decode", Core batched decode: Qwen3 split-half RoPE).
template <int D, int NW>
__device__ __forceinline__ void rope_table(float* s_cos, float* s_sin, int pos, float theta) {
  for (int i = threadIdx.x; i < D / 2; i += NW * kWave) {
    const double ang = double(pos) * pow(double(theta), -2.0 * double(i) / double(D));
    double sn, cs;
    sincos(ang, &sn, &cs);
    s_cos[i] = float(cs);
    s_sin[i] = float(sn);
  }
}

// Rotation frequencies f_i = theta^(-2i/D), i < D/2, in fp64, written by the
// lanes of one wave.  They do not depend on the position, so a wave that
// visits several sequences computes them once.
template <int D>
__device__ __forceinline__ void rope_freqs(double* s_f, float theta) {
  for (int i = threadIdx.x; i < D / 2; i += kWave) s_f[i] = pow(double(theta), -2.0 * double(i) / double(D));
}

// cos / sin of pos * f_i (angle in fp64, rounded to fp32 once).
template <int D>
__device__ __forceinline__ void rope_angles(const double* s_f, float* s_cos, float* s_sin, int pos) {
  for (int i = threadIdx.x; i < D / 2; i += kWave) {
    double sn, cs;
    sincos(double(pos) * s_f[i], &sn, &cs);
    s_cos[i] = float(cs);
    s_sin[i] = float(sn);
  }
}

template <int D, bool FP8>
struct MfmaGeo {
  static constexpr int kBytes = FP8 ? 1 : 2;
  static constexpr int kRow = D * kBytes;       // bytes of one token row
  static constexpr int kTile = 16 * kRow;       // bytes of a (block, kv head) tile
  static constexpr int kPieces = kRow / 16;     // 16-byte pieces per row
  static constexpr int kKLoads = kPieces / 4;   // K pieces per lane: 4u + lane group
  static constexpr int kQK = D / 32;            // 16x16x32 products per tile
  static constexpr int kPV = D / 16;            // 16x16x16 products per tile
  static constexpr int kVBytes = kRow / 16;     // V bytes per lane per row (D/16 dims)
  static constexpr int kVWords = kVBytes / 4;
};

template <int W>
struct Words;
template <>
struct Words<1> {
  using T = uint32_t;
};
template <>
struct Words<2> {
  using T = u32x2;
};
template <>
struct Words<4> {
  using T = u32x4;
};

// Cache policy of the KV tile loads: non-temporal (the gfx9 "nt" bit).  A
// step reads each KV byte once, so the lines are marked for streaming and do
// not displace lines that are reused (block tables, q, partials) in L2 and
// the Infinity Cache.  Measured on MI355X: the streaming rate of the decode
// step rose by ~10%, and a plain read of 1 GiB from 5.9 to 6.8 TB/s.
constexpr int kKvAux = 2;
__device__ __forceinline__ u32x4 buffer_load16_kv(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kKvAux);
}

template <int W, int AUX>
__device__ __forceinline__ typename Words<W>::T buffer_load_words(__amdgpu_buffer_rsrc_t r, int off) {
  if constexpr (W == 4) return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
  else if constexpr (W == 2) return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
  else return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
}

template <int W>
__device__ __forceinline__ uint32_t word(const typename Words<W>::T& v, int k) {
  if constexpr (W == 1) return v;
  else return v[k];
}

// E4M3 scales of a tile: the K scale multiplies the logits (fp32); the V
// scale is split in two factors so that neither fp16 operand of the P.V
// product leaves the normal range whatever the data's magnitude: its
// power-of-two part is applied exactly in the conversion of the V codes,
// and its mantissa vm in [1, 2) multiplies the softmax weights (in [0, 1])
// before they are rounded to fp16.
template <int D, bool FP8>
struct MTile {
  using Geo = MfmaGeo<D, FP8>;
  u32x4 k[Geo::kKLoads];
  typename Words<Geo::kVWords>::T v[4];
  float ks, vs, vm;
  int rows;  // rows [lo, rows) take part; the others are masked out
  int lo;
};

// The K and V loads of one tile with cache policy AUX.
template <int D, bool FP8, int AUX>
__device__ __forceinline__ void mtile_loads(MTile<D, FP8>& t, __amdgpu_buffer_rsrc_t rk,
                                            __amdgpu_buffer_rsrc_t rv, int k_off, int v_off) {
  using Geo = MfmaGeo<D, FP8>;
#pragma unroll
  for (int i = 0; i < Geo::kKLoads; ++i)
    t.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, k_off + i * 64, 0, AUX);
#pragma unroll
  for (int j = 0; j < 4; ++j) t.v[j] = buffer_load_words<Geo::kVWords, AUX>(rv, v_off + j * Geo::kRow);
}

// Issue the loads of one tile: `base` is the byte offset of its (block, kv
// head) tile, `rows` its valid rows (0: nothing is read).  `cached`: the
// caller said that blocks are shared between sequences in this call, so the
// tile is loaded with the default policy, which keeps it in the caches for
// the other readers; otherwise it is streamed (non-temporal).
template <int D, bool FP8>
__device__ __forceinline__ void load_mtile_at(MTile<D, FP8>& t, const DecodeArgs& a, size_t base,
                                              int rows, int k_off, int v_off, bool cached = false) {
  using Geo = MfmaGeo<D, FP8>;
  t.rows = rows;
  t.lo = 0;
  const int nbytes = rows * Geo::kRow;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k_pool + base, nbytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v_pool + base, nbytes);
  if (cached) mtile_loads<D, FP8, 0>(t, rk, rv, k_off, v_off);
  else mtile_loads<D, FP8, kKvAux>(t, rk, rv, k_off, v_off);
  t.ks = t.vs = t.vm = 1.0f;
  if constexpr (FP8) {
    if (rows > 0) {
      const size_t s = (base / Geo::kTile) >> a.bs_shift;  // == block id * Hkv + kv head
      t.ks = load_uniform_f32(a.k_scale + s);
      t.vs = load_uniform_f32(a.v_scale + s);
      t.vm = scale_mantissa(t.vs);
    }
  }
}

// A operand (K rows) of QK product c: 8 dims per lane.
template <int D, bool FP8>
__device__ __forceinline__ half8_t k_operand(const MTile<D, FP8>& t, int c) {
  if constexpr (!FP8) {
    return __builtin_bit_cast(half8_t, t.k[c]);
  } else {
    const u32x4& p = t.k[c / 2];
    const uint32_t w0 = p[2 * (c % 2)], w1 = p[2 * (c % 2) + 1];
    const half2_t a = e4m3x2_to_half2<false>(w0), b = e4m3x2_to_half2<true>(w0);
    const half2_t e = e4m3x2_to_half2<false>(w1), f = e4m3x2_to_half2<true>(w1);
    return half8_t{a.x, a.y, b.x, b.y, e.x, e.y, f.x, f.y};
  }
}

// First of the 8 dims that QK product c takes from lane group g (the K
// operand above and the q operand must agree on it).
template <bool FP8>
__device__ __forceinline__ int qk_dim0(int c, int g) {
  if constexpr (!FP8) return 8 * (4 * c + g);
  else return 16 * (4 * (c / 2) + g) + 8 * (c % 2);
}

// A operand (V^T) of PV product i: element i of the lane's V slice in each
// of its four rows 4g + 0..3.
template <int D, bool FP8>
__device__ __forceinline__ half4_t v_operand(const MTile<D, FP8>& t, int i) {
  using Geo = MfmaGeo<D, FP8>;
  if constexpr (!FP8) {
    const int wi = i / 2;
    const uint32_t x0 = word<Geo::kVWords>(t.v[0], wi), x1 = word<Geo::kVWords>(t.v[1], wi);
    const uint32_t x2 = word<Geo::kVWords>(t.v[2], wi), x3 = word<Geo::kVWords>(t.v[3], wi);
    uint32_t lo, hi;
    if (i % 2 == 0) {
      lo = (x0 & 0xFFFFu) | (x1 << 16);
      hi = (x2 & 0xFFFFu) | (x3 << 16);
    } else {
      lo = (x0 >> 16) | (x1 & 0xFFFF0000u);
      hi = (x2 >> 16) | (x3 & 0xFFFF0000u);
    }
    const u32x2 r = {lo, hi};
    return __builtin_bit_cast(half4_t, r);
  } else {
    // byte i % 4 of word i / 4 of rows 0..3 gathered into one word by byte
    // permutes: rows (0, 1) and (2, 3) pair up the bytes of i and its
    // neighbour i ^ 1, and a third permute picks i's half of each pair
    const int wi = i / 4, k = i % 4 & ~1;
    const uint32_t x0 = word<Geo::kVWords>(t.v[0], wi), x1 = word<Geo::kVWords>(t.v[1], wi);
    const uint32_t x2 = word<Geo::kVWords>(t.v[2], wi), x3 = word<Geo::kVWords>(t.v[3], wi);
    // perm(hi, lo, sel): selector byte s takes byte s of {hi:lo} (lo = bytes 0..3)
    const uint32_t sel = uint32_t(k) | uint32_t(k + 4) << 8 | uint32_t(k + 1) << 16 |
                         uint32_t(k + 5) << 24;
    const uint32_t p01 = __builtin_amdgcn_perm(x1, x0, sel);
    const uint32_t p23 = __builtin_amdgcn_perm(x3, x2, sel);
    const uint32_t w = __builtin_amdgcn_perm(p23, p01, i % 2 ? 0x07060302u : 0x05040100u);
    const half2_t a = e4m3x2_to_half2_pow2<false>(w, t.vs), c = e4m3x2_to_half2_pow2<true>(w, t.vs);
    return half4_t{a.x, a.y, c.x, c.y};
  }
}

template <int D, bool FP8>
struct MState {
  float m;  // running max of head slot n16, log2 units of the scaled logit
  float l;  // this lane's share of the exp-sum (its 4 tokens per tile)
  float4_t acc[MfmaGeo<D, FP8>::kPV];
};

template <int D, bool FP8>
__device__ __forceinline__ void mfma_tile(MState<D, FP8>& st, const MTile<D, FP8>& t,
                                          const half8_t* qop, float scale_log2, int g,
                                          int col_hi = 16) {
  using Geo = MfmaGeo<D, FP8>;
  float4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < Geo::kQK; ++c)
    s = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand<D, FP8>(t, c), qop[c], s, 0, 0, 0);
  // logit factor in log2 units.  An E4M3 K scale of 0 (a block whose rows
  // are all zero) is replaced by 1e-30: the masked rows' -inf must not meet a
  // zero factor (-inf * 0 is NaN), and the valid rows' logits stay ~1e-27,
  // whose exp2 rounds exactly as that of 0 in fp32.
  const float cs = scale_log2 * (t.ks != 0.0f ? t.ks : 1e-30f);
  float tm = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s[r] = (4 * g + r) < min(t.rows, col_hi) && (4 * g + r) >= t.lo ? s[r] : -INFINITY;
    tm = fmaxf(tm, s[r]);
  }
  // the head's 16 tokens sit in lanes n16, n16+16, n16+32, n16+48
  tm = group4_max(tm);
  const float mn = fmaxf(st.m, tm * cs);
  const float alpha = fast_exp2(st.m - mn);
  st.m = mn;
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {  // skip the rescale when no max moved
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < Geo::kPV; ++i) st.acc[i] *= alpha;
  }
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    p[r] = fast_exp2(fmaf(s[r], cs, -mn));
    st.l += p[r];
  }
  half4_t pv;
#pragma unroll
  for (int r = 0; r < 4; ++r) pv[r] = (_Float16)(FP8 ? p[r] * t.vm : p[r]);
#pragma unroll
  for (int i = 0; i < Geo::kPV; ++i)
    st.acc[i] = __builtin_amdgcn_mfma_f32_16x16x16f16(v_operand<D, FP8>(t, i), pv, st.acc[i], 0, 0, 0);
}

// RMSNorm over the head (its four lane groups) and split-half RoPE of the
// head held in the lane's QK chunks: chunk c of lane group g covers dims
// 32c + 8g + 0..7, so chunk c + D/64 holds the rotation partners (dims
// + D/2) of chunk c in the same lane.  fp32 arithmetic, angles from the
// fp64 table, one rounding to fp16.
template <int D>
__device__ __forceinline__ void norm_rope_chunks(half8_t* x, const float* gamma, float eps,
                                                 const float* s_cos, const float* s_sin, int g) {
  constexpr int NC = D / 32, HALF = NC / 2;
  float v[NC][8];
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[c][e] = float(x[c][e]);
      ss = fmaf(v[c][e], v[c][e], ss);
    }
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  const float inv = 1.0f / sqrtf(ss / float(D) + eps);
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) v[c][e] = v[c][e] * inv * gamma[qk_dim0<false>(c, g) + e];
#pragma unroll
  for (int c = 0; c < HALF; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = qk_dim0<false>(c, g) + e;
      const float cs = s_cos[i], sn = s_sin[i];
      const float lo = v[c][e], hi = v[c + HALF][e];
      x[c][e] = (_Float16)fmaf(lo, cs, -hi * sn);
      x[c + HALF][e] = (_Float16)fmaf(hi, cs, lo * sn);
    }
}


}  // namespace pkv
