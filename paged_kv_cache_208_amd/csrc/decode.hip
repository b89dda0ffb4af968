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
// take the unit's tiles round-robin, and each wave keeps the next tile's
// loads in flight while it computes on the current one (two register
// buffers used alternately).
//
// Rows past the end of the context are never fetched: a tile's buffer
// resource is bounded to its valid rows, loads beyond return zero, and the
// logits of those rows are replaced by -inf before the softmax, so pad rows
// holding anything (NaN included) cannot reach the output.
//
// Tile engine (MFMA): S^T = K Q^T with v_mfma_f32_16x16x32_f16 (16 tokens x
// 16 head slots, the g real heads padded with zero queries), then
// O^T += V^T P^T with v_mfma_f32_16x16x16_f16.  The QK result layout is
// exactly the B-operand layout the PV product needs, so P never leaves the
// registers; V is regrouped into token-major quads with byte permutes.
// About 50 VALU instructions per fp16 tile.
#include <type_traits>

#include "decode_tile.h"
#include "device.h"
#include "kernels.h"
#include "shape_limits.h"

// Tuning knobs (compile-time): waves per workgroup, the occupancy the
// register allocator is asked to reach (waves per SIMD), and the order in
// which work units are dispatched.
#ifndef PKV_DECODE_WAVES
#define PKV_DECODE_WAVES 4
#endif
#ifndef PKV_DECODE_WAVES_PER_EU
#define PKV_DECODE_WAVES_PER_EU 3
#endif
#ifndef PKV_DECODE_PARTITION_MAJOR
#define PKV_DECODE_PARTITION_MAJOR 1
#endif

#define PKV_DECODE_BOUNDS(NW) \
  __launch_bounds__((NW) * kWave) __attribute__((amdgpu_waves_per_eu(PKV_DECODE_WAVES_PER_EU, 8)))

namespace pkv {
namespace {

// ---------------------------------------------------------------------------
// Shared: unit bounds, tile addressing and the cross-wave combine.

struct Unit {
  int b, kvh, p;
  int L;               // context length of the sequence
  int tok_lo, tok_hi;  // token range of the unit
  int n_lo, n_hi;      // logical block range
  bool empty;          // partitioned and past the context: nothing to write
};

__device__ __forceinline__ Unit decode_unit(const DecodeArgs& a) {
  Unit u;
  int x = blockIdx.x;
#if PKV_DECODE_PARTITION_MAJOR
  // partition-major: every sequence's first partitions are dispatched before
  // any sequence's later (shorter or empty) ones
  const int bh = gridDim.x / a.max_partitions;  // B * Hkv
  u.p = x / bh;
  x %= bh;
#else
  u.p = x % a.max_partitions;
  x /= a.max_partitions;
#endif
  u.kvh = x % a.Hkv;
  u.b = x / a.Hkv;
  const int L = a.context_lens[u.b];
  u.L = L;
  u.tok_lo = 0;
  u.tok_hi = L;
  u.empty = false;
  if (a.partition_size) {
    u.tok_lo = u.p * a.partition_size;
    u.empty = u.tok_lo >= L;
    u.tok_hi = min(L, u.tok_lo + a.partition_size);
  }
  u.n_lo = u.tok_lo / 16;
  u.n_hi = (u.tok_hi + 15) / 16;
  return u;
}

// The tiles one wave visits in a unit: logical blocks n0 + NW*k, k < count.
// Their physical block ids are read into a VGPR window (lane j holds the id
// of tile base + j) once per chunk of up to 64 tiles and picked out with
// readlane.  The window is filled only outside the tile loop, so the loop
// never waits on it and the next tile's loads stay in flight while the
// current tile is computed.
template <int NW>
struct TileWalk {
  const int32_t* trow;
  int n0, count;   // the wave's tiles
  int base, end;   // tiles [base, end) are in the window
  int win;

  __device__ __forceinline__ void init(const int32_t* row, const Unit& u, int w) {
    trow = row;
    n0 = u.n_lo + w;
    count = n0 < u.n_hi ? (u.n_hi - n0 + NW - 1) / NW : 0;
  }
  __device__ __forceinline__ void fill(int first) {
    const int k = first + int(threadIdx.x & (kWave - 1));
    base = first;
    end = min(count, first + kWave);
    win = k < end ? trow[n0 + NW * k] : 0;
  }
};

// Byte offset of the wave's tile k for the unit's kv head, and its number of
// valid rows.  Tiles outside the current window (past the chunk or the
// wave's last tile) give 0 rows: their buffer resource has zero size and
// nothing is read.
template <int TILE, int NW>
__device__ __forceinline__ int tile_base(const DecodeArgs& a, const TileWalk<NW>& walk, int k,
                                         const Unit& u, size_t& base) {
  int id = 0, rows = 0;
  if (k < walk.end) {
    id = __builtin_amdgcn_readlane(walk.win, k - walk.base);
    rows = min(16, u.tok_hi - (walk.n0 + NW * k) * 16);
  }
  base = (size_t(id) * a.Hkv + u.kvh) * TILE;
  return rows;
}

// Combine the NW waves' (m, l, acc) held in LDS and write the result: the
// fp16 output when `direct` (single pass, or a context that fits one
// partition in the step kernel), else the unit's partition statistics.
// m is in log2 units of the scaled logit; acc is unnormalised.
template <int D, int G, int NW, bool COHERENT = false>
__device__ __forceinline__ void combine_and_store(const DecodeArgs& a, const Unit& u,
                                                  float (*s_acc)[G][D], float (*s_m)[G],
                                                  float (*s_l)[G], bool direct) {
  const int h0 = u.kvh * G;
  for (int idx = threadIdx.x; idx < G * D; idx += NW * kWave) {
    const int j = idx / D;
    const int d = idx % D;
    float M = s_m[0][j];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][j]);
    float den = 0.0f, num = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(s_m[w][j] - M);
      den = fmaf(s_l[w][j], f, den);
      num = fmaf(s_acc[w][j][d], f, num);
    }
    const size_t row = size_t(u.b) * a.Hq + h0 + j;
    if (direct) {
      // an empty context is a zero row; anything else divides, so a NaN that
      // reached the sums stays visible
      static_cast<_Float16*>(a.out)[row * D + d] = (_Float16)(u.tok_hi > 0 ? num / den : 0.0f);
    } else {
      const size_t pr = row * a.max_partitions + u.p;
      store_f32<COHERENT>(a.part_out + pr * D + d, num / den);
      if (d == 0) {
        store_f32<COHERENT>(a.part_max + pr, M * kLn2);
        store_f32<COHERENT>(a.part_sum + pr, den);
      }
    }
  }
}

// Log-sum-exp combine of the P partitions of the unit's G heads, written as
// the fp16 output (the same arithmetic as paged_attn_reduce, partitions in
// ascending order).  The (m, l) pairs are fetched in parallel into LDS, then
// each output element's P partial values are loaded eight at a time so their
// latencies overlap.
template <int D, int G, int NW>
__device__ __forceinline__ void combine_partitions(const DecodeArgs& a, const Unit& u, int P) {
  __shared__ float s_pm[G][kMaxStepPartitions];  // the host check bounds P by this
  __shared__ float s_pw[G][kMaxStepPartitions];
  const size_t row0 = size_t(u.b) * a.Hq + u.kvh * G;
  for (int t = threadIdx.x; t < G * P; t += NW * kWave) {
    const int j = t / P, p = t % P;
    const size_t pr = (row0 + j) * a.max_partitions + p;
    s_pm[j][p] = load_f32_coherent(a.part_max + pr);
    s_pw[j][p] = load_f32_coherent(a.part_sum + pr);
  }
  __syncthreads();
  // weights w_p = l_p exp(m_p - M) per head, in place
  for (int j = threadIdx.x; j < G; j += NW * kWave) {
    float M = -FLT_MAX;
    for (int p = 0; p < P; ++p) M = fmaxf(M, s_pm[j][p]);
    float den = 0.0f;
    for (int p = 0; p < P; ++p) {
      const float wgt = s_pw[j][p] * fast_exp2((s_pm[j][p] - M) * kLog2e);
      den += wgt;
      s_pw[j][p] = wgt;
    }
    s_pm[j][0] = den;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += NW * kWave) {
    const int j = idx / D;
    const int d = idx % D;
    const float* po = a.part_out + (row0 + j) * a.max_partitions * D + d;
    float num = 0.0f;
    for (int p0 = 0; p0 < P; p0 += 8) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = p0 + k < P ? load_f32_coherent(po + size_t(p0 + k) * D) : 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (p0 + k < P) num = fmaf(s_pw[j][p0 + k], v[k], num);
    }
    static_cast<_Float16*>(a.out)[(row0 + j) * D + d] = (_Float16)(num / s_pm[j][0]);
  }
}

// Zero output rows of the unit's G heads (empty context).
template <int D, int G, int NW>
__device__ __forceinline__ void store_zero_rows(const DecodeArgs& a, const Unit& u) {
  for (int idx = threadIdx.x; idx < G * D; idx += NW * kWave)
    static_cast<_Float16*>(a.out)[(size_t(u.b) * a.Hq + u.kvh * G) * D + idx] = (_Float16)0.0f;
}

// ---------------------------------------------------------------------------
// MFMA engine.
//
// Lane l = 16 g + n16 (g = lane group 0..3, n16 = 0..15):
//   K:  row n16 of the tile, 16-byte pieces 4u + g of that row
//   QK: S^T rows are tokens, columns head slots; the lane receives tokens
//       4g .. 4g+3 of head slot n16
//   V:  rows 4g .. 4g+3, the D/16 dims starting at n16 * D/16
//   PV: O^T rows are dims, columns head slots; product i covers dim
//       (row * D/16 + i), so the lane accumulates head n16, dims
//       (4g + r) * D/16 + i.

template <int D, bool FP8, int NW>
__device__ __forceinline__ void load_mtile(MTile<D, FP8>& t, const DecodeArgs& a, const TileWalk<NW>& walk,
                                           int k, const Unit& u, int k_off, int v_off) {
  size_t base;
  const int rows = tile_base<MfmaGeo<D, FP8>::kTile, NW>(a, walk, k, u, base);
  load_mtile_at<D, FP8>(t, a, base, rows, k_off, v_off, a.cached_kv != 0);
}

template <int D, int G, bool FP8, int NW, int MODE>
__global__ PKV_DECODE_BOUNDS(NW) void decode_mfma_kernel(DecodeArgs a) {
  using Geo = MfmaGeo<D, FP8>;
  constexpr bool APPEND = (MODE & kModeAppend) != 0;
  constexpr bool QKNORM = (MODE & kModeQkNorm) != 0;
  constexpr bool COMBINE = (MODE & kModeCombine) != 0;
  static_assert(G <= 16, "head slots of one 16-wide product");
  static_assert(!(APPEND && FP8), "the step kernel appends fp16 rows only");
  static_assert(!QKNORM || APPEND, "QK-norm comes with the append of the new row");
  const Unit u = decode_unit(a);
  if (u.empty) {  // whole workgroup: a partition past the context
    if constexpr (COMBINE)
      if (u.p == 0) store_zero_rows<D, G, NW>(a, u);  // empty context: zero row
    return;
  }

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane / 16;
  const int n16 = lane % 16;
  const int32_t* trow = a.block_tables + size_t(u.b) * a.MBS;
  const int k_off = n16 * Geo::kRow + g * 16;
  const int v_off = (4 * g) * Geo::kRow + n16 * Geo::kVBytes;

  __shared__ float s_cos[QKNORM ? D / 2 : 1];
  __shared__ float s_sin[QKNORM ? D / 2 : 1];
  if constexpr (QKNORM) {
    rope_table<D, NW>(s_cos, s_sin, u.L - 1, a.theta);
    __syncthreads();
  }

  // B operand of the QK products: q of head slot n16 (zero past the group)
  half8_t qop[Geo::kQK];
  {
    const _Float16* qh =
        static_cast<const _Float16*>(a.q) + (size_t(u.b) * a.Hq + u.kvh * G + min(n16, G - 1)) * D;
#pragma unroll
    for (int c = 0; c < Geo::kQK; ++c)
      qop[c] = __builtin_bit_cast(half8_t, *reinterpret_cast<const u32x4*>(qh + qk_dim0<FP8>(c, g)));
    if constexpr (QKNORM) norm_rope_chunks<D>(qop, a.gamma_q, a.eps, s_cos, s_sin, g);
    if (n16 >= G)
#pragma unroll
      for (int c = 0; c < Geo::kQK; ++c) qop[c] = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
  }

  // The step's new row (token L-1) lives in the last tile of the unit that
  // ends the context.  The wave that will read that tile writes it first,
  // each lane storing exactly the 16-byte pieces it later loads, so the
  // loads observe the stores (same lane, same address, program order).
  if constexpr (APPEND) {
    if (u.tok_hi == u.L) {
      const int t = u.L - 1;
      const int n_last = t / 16, r_new = t % 16;
      if (w == (n_last - u.n_lo) % NW) {
        const int id = __builtin_amdgcn_readfirstlane(trow[n_last]);
        const size_t base = (size_t(id) * a.Hkv + u.kvh) * Geo::kTile;
        const size_t row = size_t(u.b) * a.Hkv + u.kvh;
        const _Float16* kn = static_cast<const _Float16*>(a.k_new) + row * D;
        const _Float16* vn = static_cast<const _Float16*>(a.v_new) + row * D;
        half8_t kc[Geo::kKLoads];
#pragma unroll
        for (int i = 0; i < Geo::kKLoads; ++i)
          kc[i] = __builtin_bit_cast(half8_t, *reinterpret_cast<const u32x4*>(kn + (4 * i + g) * 8));
        if constexpr (QKNORM) norm_rope_chunks<D>(kc, a.gamma_k, a.eps, s_cos, s_sin, g);
        uint8_t* kt = const_cast<uint8_t*>(a.k_pool) + base;
        uint8_t* vt = const_cast<uint8_t*>(a.v_pool) + base;
        if (n16 == r_new)
#pragma unroll
          for (int i = 0; i < Geo::kKLoads; ++i)
            *reinterpret_cast<u32x4*>(kt + k_off + i * 64) = __builtin_bit_cast(u32x4, kc[i]);
        if (g == r_new / 4) {
          using VW = typename Words<Geo::kVWords>::T;
          *reinterpret_cast<VW*>(vt + v_off + (r_new % 4) * Geo::kRow) =
              *reinterpret_cast<const VW*>(vn + n16 * (D / 16));
        }
      }
    }
  }

  MState<D, FP8> st;
  st.m = -FLT_MAX;
  st.l = 0.0f;
#pragma unroll
  for (int i = 0; i < Geo::kPV; ++i) st.acc[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  TileWalk<NW> walk;
  walk.init(trow, u, w);
  MTile<D, FP8> ta, tb;
  for (int c0 = 0; c0 < walk.count; c0 += kWave) {
    walk.fill(c0);
    load_mtile<D, FP8, NW>(ta, a, walk, c0, u, k_off, v_off);
    for (int k = c0; k < walk.end;) {
      load_mtile<D, FP8, NW>(tb, a, walk, k + 1, u, k_off, v_off);
      issue_fence();
      mfma_tile<D, FP8>(st, ta, qop, a.scale_log2, g);
      if (++k >= walk.end) break;
      load_mtile<D, FP8, NW>(ta, a, walk, k + 1, u, k_off, v_off);
      issue_fence();
      mfma_tile<D, FP8>(st, tb, qop, a.scale_log2, g);
      ++k;
    }
  }

  // the four lane groups of a head hold disjoint tokens: add their sums
  st.l = group4_sum(st.l);

  __shared__ float s_acc[NW][G][D];
  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];
  if (n16 < G) {
#pragma unroll
    for (int i = 0; i < Geo::kPV; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_acc[w][n16][(4 * g + r) * (D / 16) + i] = st.acc[i][r];
    if (g == 0) {
      s_m[w][n16] = st.m;
      s_l[w][n16] = st.l;
    }
  }
  __syncthreads();

  // number of partitions of this sequence (1 for a single pass)
  const int P = a.partition_size ? (u.L + a.partition_size - 1) / a.partition_size : 1;
  const bool direct = a.partition_size == 0 || (COMBINE && P == 1);
  combine_and_store<D, G, NW, COMBINE>(a, u, s_acc, s_m, s_l, direct);

  bool finisher = direct;  // writes q' back: the last workgroup of the (b, kv head)
  if constexpr (COMBINE) {
    if (!direct) {
      // Publish this partition and count arrivals; the last one combines.
      // The barrier waits for every thread's (coherent) partial stores to
      // complete before thread 0 increments the counter, and the last
      // workgroup reads the partials only after its increment returned.
      __shared__ int s_last;
      __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
      __syncthreads();
      uint32_t* ctr = a.counters + size_t(u.b) * a.Hkv + u.kvh;
      if (threadIdx.x == 0)
        s_last = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 uint32_t(P - 1);
      __syncthreads();
      if (!s_last) return;  // whole workgroup
      combine_partitions<D, G, NW>(a, u, P);
      if (threadIdx.x == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      finisher = true;
    }
  }
  if constexpr (QKNORM) {
    if (finisher && w == 0 && n16 < G) {
      _Float16* qh = const_cast<_Float16*>(static_cast<const _Float16*>(a.q)) +
                     (size_t(u.b) * a.Hq + u.kvh * G + n16) * D;
#pragma unroll
      for (int c = 0; c < Geo::kQK; ++c)
        *reinterpret_cast<u32x4*>(qh + qk_dim0<false>(c, g)) = __builtin_bit_cast(u32x4, qop[c]);
    }
  }
}

// ---------------------------------------------------------------------------
// Dispatch.

constexpr int kWavesPerGroup = PKV_DECODE_WAVES;

template <int D, int G, bool FP8, int MODE>
hipError_t launch_mfma(const DecodeArgs& a, int B, hipStream_t stream) {
  const unsigned units = unsigned(int64_t(B) * a.Hkv * a.max_partitions);
  hipLaunchKernelGGL((decode_mfma_kernel<D, G, FP8, kWavesPerGroup, MODE>), dim3(units),
                     dim3(kWavesPerGroup * kWave), 0, stream, a);
  return hipGetLastError();
}

template <int D, int G, bool FP8>
hipError_t launch_typed(const DecodeArgs& a, int B, hipStream_t stream) {
  return launch_mfma<D, G, FP8, kModeAttend>(a, B, stream);
}

template <int D, int G, bool FP8>
hipError_t launch_step_typed(const DecodeArgs& a, int B, int mode, hipStream_t stream) {
  if constexpr (FP8) {
    if (mode == kModeCombine) return launch_mfma<D, G, true, kModeCombine>(a, B, stream);
    return hipErrorInvalidValue;
  } else {
    switch (mode) {
      case kModeCombine: return launch_mfma<D, G, false, kModeCombine>(a, B, stream);
      case kModeAppend | kModeCombine:
        return launch_mfma<D, G, false, kModeAppend | kModeCombine>(a, B, stream);
      case kModeAppend | kModeQkNorm | kModeCombine:
        return launch_mfma<D, G, false, kModeAppend | kModeQkNorm | kModeCombine>(a, B, stream);
      default: return hipErrorInvalidValue;
    }
  }
}

template <int D, bool FP8, typename F>
hipError_t by_group(int group, F&& f) {
  switch (group) {
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 8: return f(std::integral_constant<int, 8>{});
    default: return hipErrorInvalidValue;
  }
}

template <int D, bool FP8>
hipError_t launch_group(const DecodeArgs& a, int B, int group, hipStream_t stream) {
  return by_group<D, FP8>(group, [&](auto gc) {
    return launch_typed<D, decltype(gc)::value, FP8>(a, B, stream);
  });
}

template <int D, bool FP8>
hipError_t launch_step_group(const DecodeArgs& a, int B, int group, int mode, hipStream_t stream) {
  return by_group<D, FP8>(group, [&](auto gc) {
    return launch_step_typed<D, decltype(gc)::value, FP8>(a, B, mode, stream);
  });
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

hipError_t launch_decode_step(const DecodeArgs& a, int B, int D, int group, bool fp8, int mode,
                              hipStream_t stream) {
  if (D == 128) return fp8 ? launch_step_group<128, true>(a, B, group, mode, stream)
                           : launch_step_group<128, false>(a, B, group, mode, stream);
  if (D == 64) return fp8 ? launch_step_group<64, true>(a, B, group, mode, stream)
                          : launch_step_group<64, false>(a, B, group, mode, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
