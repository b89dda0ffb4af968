// paged_attn_decode kernels for gfx950.
//
// One workgroup handles one work unit (sequence b, kv head, partition p):
// the tokens [p*PS, min(L_b, (p+1)*PS)) of that sequence (all of them when
// PS == 0).  The g query heads of the kv head's GQA group share every K/V
// byte that is read, and one online softmax per q head runs over the unit.
//
// Block-table walk ("Distributed LLM Inference Serving Platform", section
// 2): logical block n of sequence b is physical block block_tables[b][n];
// its (block, kv head) tile of 16 token rows is contiguous in the pool
// ([NB][Hkv][16][D] layout), 16 * D * bytes long.  The waves of a workgroup
// take the unit's tiles round-robin.
//
// Lane mapping: a token row of one head is ROW = D * bytes long and is read
// by LPT = ROW / 16 lanes with one 16-byte load each, so one wave load
// covers TPI = 64 / LPT consecutive rows (a contiguous 1 KiB) and a tile
// takes NI = 16 / TPI loads.  Each lane dots its 16 bytes of K with the
// matching slice of the g query heads; a DPP reduction inside the LPT-lane
// group completes the logit.  Every lane group (one token row of each wave
// load) keeps its own running max / sum / accumulator; groups and waves are
// merged once at the end of the unit.
//
// Rows past the end of the context are never fetched: the tile's buffer
// resource is bounded to its valid rows, loads beyond return zero, and the
// logits of those rows are replaced by -inf before the softmax, so pad rows
// holding anything (NaN included) cannot reach the output.
#include "device.h"
#include "kernels.h"

namespace pkv {
namespace {

template <int D, bool FP8>
struct Geometry {
  static constexpr int kBytes = FP8 ? 1 : 2;
  static constexpr int kRow = D * kBytes;     // bytes of one token row
  static constexpr int kLpt = kRow / 16;      // lanes per token row
  static constexpr int kTpi = kWave / kLpt;   // token rows per wave load
  static constexpr int kNi = 16 / kTpi;       // wave loads per tile
  static constexpr int kEpl = 16 / kBytes;    // elements per lane
  static constexpr int kTile = 16 * kRow;     // bytes per (block, kv head) tile
  static_assert(kLpt >= 4 && kLpt <= 16, "row must span 4..16 lanes");
};

template <int D, bool FP8>
struct TileRegs {
  using Geo = Geometry<D, FP8>;
  u32x4 k[Geo::kNi];
  u32x4 v[Geo::kNi];
  float ks, vs;  // E4M3 tile scales (1 for fp16)
  int rows;      // valid token rows in the tile (0 = past the unit)
};

template <int D, bool FP8>
__device__ __forceinline__ void load_tile(TileRegs<D, FP8>& t, const DecodeArgs& a,
                                          const int32_t* trow, int n, int n_hi, int tok_hi,
                                          int kvh, int lane_off) {
  using Geo = Geometry<D, FP8>;
  int id = 0;
  t.rows = 0;
  if (n < n_hi) {
    id = __builtin_amdgcn_readfirstlane(trow[n]);
    t.rows = min(16, tok_hi - n * 16);
  }
  const size_t tile = (size_t(id) * a.Hkv + kvh) * Geo::kTile;
  const int nbytes = t.rows * Geo::kRow;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k_pool + tile, nbytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v_pool + tile, nbytes);
#pragma unroll
  for (int i = 0; i < Geo::kNi; ++i) t.k[i] = buffer_load16(rk, lane_off + i * Geo::kTpi * Geo::kRow);
#pragma unroll
  for (int i = 0; i < Geo::kNi; ++i) t.v[i] = buffer_load16(rv, lane_off + i * Geo::kTpi * Geo::kRow);
  if constexpr (FP8) {
    t.ks = 1.0f;
    t.vs = 1.0f;
    if (n < n_hi) {
      t.ks = a.k_scale[size_t(id) * a.Hkv + kvh];
      t.vs = a.v_scale[size_t(id) * a.Hkv + kvh];
    }
  } else {
    t.ks = t.vs = 1.0f;
  }
}

// Partial dot of one lane's 16 bytes of K with one q head's matching slice.
template <int D, bool FP8>
__device__ __forceinline__ float lane_dot(const u32x4& kw, const half2_t* qh) {
  float s = 0.0f;
  if constexpr (FP8) {
    const uint32_t w[4] = {kw.x, kw.y, kw.z, kw.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      s = __builtin_amdgcn_fdot2(e4m3x2_to_half2<false>(w[k]), qh[2 * k], s, false);
      s = __builtin_amdgcn_fdot2(e4m3x2_to_half2<true>(w[k]), qh[2 * k + 1], s, false);
    }
  } else {
    s = __builtin_amdgcn_fdot2(as_half2(kw.x), qh[0], s, false);
    s = __builtin_amdgcn_fdot2(as_half2(kw.y), qh[1], s, false);
    s = __builtin_amdgcn_fdot2(as_half2(kw.z), qh[2], s, false);
    s = __builtin_amdgcn_fdot2(as_half2(kw.w), qh[3], s, false);
  }
  return s;
}

// The lane's 16 bytes of V as EPL floats.
template <bool FP8>
__device__ __forceinline__ void lane_values(const u32x4& vw, float* out) {
  const uint32_t w[4] = {vw.x, vw.y, vw.z, vw.w};
  if constexpr (FP8) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float2_t lo = e4m3x2_to_float2<false>(w[k]);
      const float2_t hi = e4m3x2_to_float2<true>(w[k]);
      out[4 * k + 0] = lo.x;
      out[4 * k + 1] = lo.y;
      out[4 * k + 2] = hi.x;
      out[4 * k + 3] = hi.y;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const half2_t h = as_half2(w[k]);
      out[2 * k + 0] = float(h.x);
      out[2 * k + 1] = float(h.y);
    }
  }
}

template <int D, int G, bool FP8, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_kernel(DecodeArgs a) {
  using Geo = Geometry<D, FP8>;
  constexpr int LPT = Geo::kLpt, TPI = Geo::kTpi, NI = Geo::kNi, EPL = Geo::kEpl;

  const int lane = threadIdx.x & (kWave - 1);
  // wave index as a scalar: keeps the tile walk, block ids and buffer
  // resources in SGPRs
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r = lane / LPT;  // token row within a wave load
  const int c = lane % LPT;  // 16-byte column within the row

  int unit = blockIdx.x;
  const int p = unit % a.max_partitions;
  unit /= a.max_partitions;
  const int kvh = unit % a.Hkv;
  const int b = unit / a.Hkv;

  const int L = a.context_lens[b];
  int tok_lo = 0, tok_hi = L;
  if (a.partition_size) {
    tok_lo = p * a.partition_size;
    if (tok_lo >= L) return;  // whole workgroup: partition past the context
    tok_hi = min(L, tok_lo + a.partition_size);
  }

  // q slice of every head of the group: elements [c*EPL, c*EPL + EPL)
  half2_t qv[G][EPL / 2];
  {
    const _Float16* qb = static_cast<const _Float16*>(a.q) + (size_t(b) * a.Hq + kvh * G) * D + c * EPL;
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int k = 0; k < EPL / 8; ++k) {
        const u32x4 t = *reinterpret_cast<const u32x4*>(qb + j * D + k * 8);
        qv[j][4 * k + 0] = as_half2(t.x);
        qv[j][4 * k + 1] = as_half2(t.y);
        qv[j][4 * k + 2] = as_half2(t.z);
        qv[j][4 * k + 3] = as_half2(t.w);
      }
    }
  }

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -FLT_MAX;
    l[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = 0.0f;
  }

  const int n_lo = tok_lo / 16;
  const int n_hi = (tok_hi + 15) / 16;
  const int32_t* trow = a.block_tables + size_t(b) * a.MBS;
  const int lane_off = r * Geo::kRow + c * 16;

  TileRegs<D, FP8> cur;
  int n = n_lo + w;
  load_tile<D, FP8>(cur, a, trow, n, n_hi, tok_hi, kvh, lane_off);
  for (; n < n_hi; n += NW) {
    TileRegs<D, FP8> nxt;
    load_tile<D, FP8>(nxt, a, trow, n + NW, n_hi, tok_hi, kvh, lane_off);

    // logits of the NI rows this lane group holds, for every head
    float s[NI][G];
    const float cs = a.scale_log2 * cur.ks;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool valid = (i * TPI + r) < cur.rows;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float d = group_sum<LPT>(lane_dot<D, FP8>(cur.k[i], qv[j]));
        s[i][j] = valid ? d * cs : -INFINITY;
      }
    }

    float vals[NI][EPL];
#pragma unroll
    for (int i = 0; i < NI; ++i) lane_values<FP8>(cur.v[i], vals[i]);

#pragma unroll
    for (int j = 0; j < G; ++j) {
      float tmax = s[0][j];
#pragma unroll
      for (int i = 1; i < NI; ++i) tmax = fmaxf(tmax, s[i][j]);
      const float mn = fmaxf(m[j], tmax);
      const float alpha = fast_exp2(m[j] - mn);
      m[j] = mn;
      l[j] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const float pij = fast_exp2(s[i][j] - mn);
        l[j] += pij;
        const float pv = pij * cur.vs;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] = fmaf(pv, vals[i][e], acc[j][e]);
      }
    }
    cur = nxt;
  }

  // merge the TPI row groups of the wave (lanes with the same column c)
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float mo = __shfl_xor(m[j], off);
      const float lo = __shfl_xor(l[j], off);
      const float mn = fmaxf(m[j], mo);
      const float fa = fast_exp2(m[j] - mn);
      const float fb = fast_exp2(mo - mn);
      l[j] = l[j] * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] = acc[j][e] * fa + __shfl_xor(acc[j][e], off) * fb;
      m[j] = mn;
    }
  }

  // merge the waves through LDS
  __shared__ float s_acc[NW][G][D];
  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];
  if (r == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[w][j][c * EPL + e] = acc[j][e];
      if (c == 0) {
        s_m[w][j] = m[j];
        s_l[w][j] = l[j];
      }
    }
  }
  __syncthreads();

  const int h0 = kvh * G;
  for (int idx = threadIdx.x; idx < G * D; idx += NW * kWave) {
    const int j = idx / D;
    const int d = idx % D;
    float M = s_m[0][j];
#pragma unroll
    for (int u = 1; u < NW; ++u) M = fmaxf(M, s_m[u][j]);
    float den = 0.0f, num = 0.0f;
#pragma unroll
    for (int u = 0; u < NW; ++u) {
      const float f = fast_exp2(s_m[u][j] - M);
      den = fmaf(s_l[u][j], f, den);
      num = fmaf(s_acc[u][j][d], f, num);
    }
    const size_t row = size_t(b) * a.Hq + h0 + j;
    if (a.partition_size == 0) {
      // an empty context is a zero row; anything else divides, so a NaN that
      // reached the sums stays visible
      static_cast<_Float16*>(a.out)[row * D + d] = (_Float16)(tok_hi > 0 ? num / den : 0.0f);
    } else {
      const size_t pr = row * a.max_partitions + p;
      a.part_out[pr * D + d] = num / den;
      if (d == 0) {
        a.part_max[pr] = M * kLn2;
        a.part_sum[pr] = den;
      }
    }
  }
}

constexpr int kWavesPerGroup = 4;

template <int D, int G, bool FP8>
hipError_t launch_typed(const DecodeArgs& a, int B, hipStream_t stream) {
  const int64_t units = int64_t(B) * a.Hkv * a.max_partitions;
  hipLaunchKernelGGL((decode_kernel<D, G, FP8, kWavesPerGroup>), dim3(unsigned(units)),
                     dim3(kWavesPerGroup * kWave), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool FP8>
hipError_t launch_group(const DecodeArgs& a, int B, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_typed<D, 1, FP8>(a, B, stream);
    case 2: return launch_typed<D, 2, FP8>(a, B, stream);
    case 4: return launch_typed<D, 4, FP8>(a, B, stream);
    case 8: return launch_typed<D, 8, FP8>(a, B, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int B, int D, int group, bool fp8,
                         hipStream_t stream) {
  if (D == 128) return fp8 ? launch_group<128, true>(a, B, group, stream)
                           : launch_group<128, false>(a, B, group, stream);
  if (D == 64) return fp8 ? launch_group<64, true>(a, B, group, stream)
                          : launch_group<64, false>(a, B, group, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
