// Balanced decode step for gfx950: append (+ QK-norm/RoPE), attention and
// the combine of split contexts in one launch, with every wave given the
// same amount of KV to read.
//
// The batch's tiles are laid out in one flattened order: sequence b, then kv
// head, then the sequence's 16-token tiles ("Distributed LLM Inference
// Serving Platform", section 2: logical block n of a sequence is found
// through its block table).  With W tiles in total and C waves (a fixed
// number per CU), wave w reads the contiguous range [w*tpw, (w+1)*tpw),
// tpw = ceil(W / C).  Every wave therefore moves the same number of bytes,
// whatever the mix of context lengths, and streams straight across the
// boundaries between (sequence, kv head) segments: the next tile's loads are
// issued before the current tile is computed, whichever segment it belongs
// to.
//
// A segment that lies inside one wave's range is finished by that wave (the
// normalised output is written directly).  A segment shared by several
// consecutive waves leaves one partial (m, l, o) per wave; the last wave to
// finish its piece combines them (log-sum-exp), as paged_attn_reduce does.
// Partials and arrival counters use device-scope coherent accesses; the
// counters return to zero.
//
// Each wave is its own 64-thread workgroup; the tile engine is the MFMA one
// of decode_tile.h.
#include "decode_tile.h"
#include "shape_limits.h"

// Waves resident per SIMD (the register budget follows from it); the grid is
// one wave per resident slot, four SIMDs per CU.
#ifndef PKV_STREAM_WAVES_PER_EU
#define PKV_STREAM_WAVES_PER_EU 2
#endif

namespace pkv {
namespace {

// Position of one tile in the flattened order.
struct Cursor {
  int b, kvh, n;  // sequence, kv head, tile within the segment
  int L, T;       // context length of b, tiles per segment
  int64_t S;      // flattened index of the segment's first tile
};

__device__ __forceinline__ int64_t readlane64(int64_t v, int lane) {
  const int lo = __builtin_amdgcn_readlane(int(uint64_t(v) & 0xffffffffu), lane);
  const int hi = __builtin_amdgcn_readlane(int(uint64_t(v) >> 32), lane);
  return int64_t((uint64_t(uint32_t(hi)) << 32) | uint32_t(lo));
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int64_t wave_scan(int64_t x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int64_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Total tiles of the batch (all kv heads).
__device__ __forceinline__ int64_t total_tiles(const DecodeArgs& a, int B) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t tot = 0;
  for (int c = 0; c < B; c += kWave) {
    const int b = c + lane;
    const int L = b < B ? a.context_lens[b] : 0;
    const int64_t incl = wave_scan(int64_t((L + 15) / 16));
    tot += readlane64(incl, kWave - 1);
  }
  return tot * a.Hkv;
}

// Cursor of flattened tile t (t < total).
__device__ __forceinline__ Cursor locate(const DecodeArgs& a, int B, int64_t t) {
  const int lane = threadIdx.x & (kWave - 1);
  Cursor c{};
  int64_t carry = 0;
  for (int c0 = 0; c0 < B; c0 += kWave) {
    const int b = c0 + lane;
    const int L = b < B ? a.context_lens[b] : 0;
    const int64_t w = int64_t(a.Hkv) * ((L + 15) / 16);
    const int64_t hi = carry + wave_scan(w);
    const int64_t lo = hi - w;
    const uint64_t here = __builtin_amdgcn_ballot_w64(b < B && lo <= t && t < hi);
    if (here) {
      const int src = __builtin_ctzll(here);
      c.b = c0 + src;
      c.L = __builtin_amdgcn_readlane(L, src);
      c.T = (c.L + 15) / 16;
      const int64_t off = t - readlane64(lo, src);
      c.kvh = int(off / c.T);
      c.n = int(off % c.T);
      c.S = readlane64(lo, src) + int64_t(c.kvh) * c.T;
      return c;
    }
    carry = readlane64(hi, kWave - 1);
  }
  return c;  // not reached for t < total
}

// Next tile in the flattened order (skips sequences with no tokens).
__device__ __forceinline__ void advance(Cursor& c, const DecodeArgs& a, int B) {
  if (++c.n < c.T) return;
  c.n = 0;
  c.S += c.T;
  if (++c.kvh < a.Hkv) return;
  c.kvh = 0;
  do {
    if (++c.b >= B) return;
    c.L = load_uniform(a.context_lens + c.b);
  } while (c.L == 0);
  c.T = (c.L + 15) / 16;
}

// What the loop needs to know about a tile besides its data.
struct Meta {
  int b, kvh, n, L, T;
  int id;      // physical block of the tile
  int64_t S;
  bool first;  // first tile of the wave's piece of the segment
  bool last;   // last tile of the wave's piece of the segment
};

__device__ __forceinline__ Meta meta_of(const Cursor& c, const DecodeArgs& a, int64_t t, int64_t t0,
                                        int64_t t1) {
  Meta m;
  // a scalar load; its result is first needed one loop step later
  m.id = load_uniform(a.block_tables + size_t(c.b) * a.MBS + c.n);
  m.b = c.b;
  m.kvh = c.kvh;
  m.n = c.n;
  m.L = c.L;
  m.T = c.T;
  m.S = c.S;
  m.first = c.n == 0 || t == t0;
  m.last = c.n == c.T - 1 || t == t1 - 1;
  return m;
}

template <int D, int G, bool FP8, int MODE>
struct StreamKernel {
  using Geo = MfmaGeo<D, FP8>;
  static constexpr bool APPEND = (MODE & kModeAppend) != 0;
  static constexpr bool QKNORM = (MODE & kModeQkNorm) != 0;

  // q of head slot n16 of the segment's group (QK-norm applied when asked),
  // as the B operand of the QK products; zero past the group.
  static __device__ __forceinline__ void load_q(half8_t* qop, const DecodeArgs& a, int b, int kvh,
                                                int g, int n16, const float* s_cos,
                                                const float* s_sin) {
    const _Float16* qh =
        static_cast<const _Float16*>(a.q) + (size_t(b) * a.Hq + kvh * G + min(n16, G - 1)) * D;
#pragma unroll
    for (int c = 0; c < Geo::kQK; ++c)
      qop[c] = __builtin_bit_cast(half8_t, *reinterpret_cast<const u32x4*>(qh + qk_dim0<FP8>(c, g)));
    if constexpr (QKNORM) norm_rope_chunks<D>(qop, a.gamma_q, a.eps, s_cos, s_sin, g);
    if (n16 >= G)
#pragma unroll
      for (int c = 0; c < Geo::kQK; ++c) qop[c] = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
  }

  // Write the step's new row (token L-1) of segment m into the tile about to
  // be read, from the lanes that will load each piece (same lane, same
  // address, program order: the loads observe the stores).
  static __device__ __forceinline__ void append_row(const DecodeArgs& a, const Meta& m, size_t base,
                                                    int g, int n16, int k_off, int v_off,
                                                    const float* s_cos, const float* s_sin) {
    const int r_new = (m.L - 1) % 16;
    const size_t row = size_t(m.b) * a.Hkv + m.kvh;
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

  // Issue the loads of tile m (writing the new row first when this is its
  // segment's last tile).  A tile that is not live issues the same loads with
  // no valid rows: they read nothing, but every loop step then has the same
  // number of loads in flight behind the tile being computed, so the wait
  // before the products stays partial on every path.
  static __device__ __forceinline__ void issue(MTile<D, FP8>& t, const DecodeArgs& a, const Meta& m,
                                               bool live, int g, int n16, int k_off, int v_off,
                                               const float* s_cos, const float* s_sin) {
    const size_t base = live ? (size_t(m.id) * a.Hkv + m.kvh) * Geo::kTile : 0;
    if constexpr (APPEND)
      if (live && m.n == m.T - 1) append_row(a, m, base, g, n16, k_off, v_off, s_cos, s_sin);
    load_mtile_at<D, FP8>(t, a, base, live ? min(16, m.L - 16 * m.n) : 0, k_off, v_off);
  }

  // End of the wave's piece of segment m: write the output directly, or a
  // partial that the last arriving piece combines.
  static __device__ __forceinline__ void flush(MState<D, FP8>& st, const DecodeArgs& a, const Meta& m,
                                               const half8_t* qop, int64_t tpw, int worker, int g,
                                               int n16, float* s_w) {
    const float l = group4_sum(st.l);
    const int64_t j0 = m.S / tpw;
    const int pieces = int((m.S + m.T - 1) / tpw - j0 + 1);
    const size_t row0 = size_t(m.b) * a.Hq + m.kvh * G;
    bool finisher = pieces == 1;
    if (pieces == 1) {
      if (n16 < G) {
        const float inv = 1.0f / l;
        _Float16* o = static_cast<_Float16*>(a.out) + (row0 + n16) * D;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          _Float16 h[Geo::kPV];
#pragma unroll
          for (int i = 0; i < Geo::kPV; ++i) h[i] = (_Float16)(st.acc[i][r] * inv);
          typedef _Float16 hv __attribute__((ext_vector_type(Geo::kPV)));
          hv v;
#pragma unroll
          for (int i = 0; i < Geo::kPV; ++i) v[i] = h[i];
          *reinterpret_cast<hv*>(o + (4 * g + r) * Geo::kPV) = v;
        }
      }
    } else {
      store_partial(st, l, a, row0, int(worker - j0), g, n16, s_w);
      __builtin_amdgcn_s_waitcnt(0);  // the partial has reached device scope
      uint32_t* ctr = a.counters + size_t(m.b) * a.Hkv + m.kvh;
      uint32_t prev = 0;
      if ((threadIdx.x & (kWave - 1)) == 0)
        prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      prev = __builtin_amdgcn_readfirstlane(prev);
      if (prev == uint32_t(pieces - 1)) {
        combine(a, row0, pieces, s_w);
        if ((threadIdx.x & (kWave - 1)) == 0)
          __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        finisher = true;
      }
    }
    if constexpr (QKNORM) {
      // q' goes back in place once no other wave of the segment needs q
      if (finisher && n16 < G) {
        _Float16* qh = const_cast<_Float16*>(static_cast<const _Float16*>(a.q)) + (row0 + n16) * D;
#pragma unroll
        for (int c = 0; c < Geo::kQK; ++c)
          *reinterpret_cast<u32x4*>(qh + qk_dim0<false>(c, g)) = __builtin_bit_cast(u32x4, qop[c]);
      }
    }
    st.m = -FLT_MAX;
    st.l = 0.0f;
#pragma unroll
    for (int i = 0; i < Geo::kPV; ++i) st.acc[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // Float4 pieces of one partial (G rows of D) and how many each lane owns.
  static constexpr int kF4 = G * D / 4;
  static constexpr int kOwn = (kF4 + kWave - 1) / kWave;

  // Buffer over the G partial rows of output row0 (all partitions).
  static __device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rows(const DecodeArgs& a,
                                                                        size_t row0) {
    const size_t stride = size_t(a.max_partitions) * D;
    return make_rsrc(a.part_out + row0 * stride, int(G * stride * sizeof(float)));
  }
  static __device__ __forceinline__ int partial_offset(const DecodeArgs& a, int c, int j) {
    return int(((4 * c / D) * size_t(a.max_partitions) * D + size_t(j) * D + 4 * c % D) *
               sizeof(float));
  }

  // Piece j of the segment at output row row0: o / l, max (natural-log
  // units) and l.  The normalised rows go through LDS so each lane writes
  // whole 16-byte pieces of them.
  static __device__ __forceinline__ void store_partial(const MState<D, FP8>& st, float l,
                                                       const DecodeArgs& a, size_t row0, int j, int g,
                                                       int n16, float* s_o) {
    static_assert(D <= 2 * kMaxStepPartitions, "staging fits the weights' LDS");
    const int lane = threadIdx.x & (kWave - 1);
    if (n16 < G) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < Geo::kPV; ++i) s_o[n16 * D + (4 * g + r) * Geo::kPV + i] = st.acc[i][r] * inv;
    }
    const __amdgpu_buffer_rsrc_t rs = partial_rows(a, row0);
#pragma unroll
    for (int k = 0; k < kOwn; ++k) {
      const int c = lane + k * kWave;
      if (c < kF4)
        store16_coherent(rs, partial_offset(a, c, j), *reinterpret_cast<const u32x4*>(s_o + 4 * c));
    }
    if (g == 0 && n16 < G) {
      const size_t pr = (row0 + n16) * a.max_partitions + j;
      store_f32<true>(a.part_max + pr, st.m * kLn2);
      store_f32<true>(a.part_sum + pr, l);
    }
  }

  // Log-sum-exp combine of `pieces` partials of the G heads starting at
  // output row row0 (one wave; weights staged in LDS).  A lane owns float4
  // pieces of the G rows and keeps a batch of partials' loads in flight.
  static __device__ __forceinline__ void combine(const DecodeArgs& a, size_t row0, int pieces,
                                                 float* s_w) {
    const int lane = threadIdx.x & (kWave - 1);
    for (int t = lane; t < G * pieces; t += kWave) {
      const int j = t / pieces, p = t % pieces;
      const size_t pr = (row0 + j) * a.max_partitions + p;
      s_w[2 * (j * kMaxStepPartitions + p)] = load_f32_coherent(a.part_max + pr);
      s_w[2 * (j * kMaxStepPartitions + p) + 1] = load_f32_coherent(a.part_sum + pr);
    }
    __builtin_amdgcn_s_waitcnt(0);
    for (int j = lane; j < G; j += kWave) {
      float* w = s_w + 2 * j * kMaxStepPartitions;
      float M = -FLT_MAX;
      for (int p = 0; p < pieces; ++p) M = fmaxf(M, w[2 * p]);
      float den = 0.0f;
      for (int p = 0; p < pieces; ++p) {
        const float wgt = w[2 * p + 1] * fast_exp2((w[2 * p] - M) * kLog2e);
        den += wgt;
        w[2 * p + 1] = wgt;
      }
      w[0] = den;
    }
    __builtin_amdgcn_s_waitcnt(0);
    constexpr int kBatch = kOwn >= 4 ? 1 : 4 / kOwn;
    const __amdgpu_buffer_rsrc_t rs = partial_rows(a, row0);
    float4_t num[kOwn];
#pragma unroll
    for (int k = 0; k < kOwn; ++k) num[k] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int p0 = 0; p0 < pieces; p0 += kBatch) {
      u32x4 v[kBatch][kOwn];
#pragma unroll
      for (int q = 0; q < kBatch; ++q)
#pragma unroll
        for (int k = 0; k < kOwn; ++k) {
          const int c = lane + k * kWave;
          v[q][k] = p0 + q < pieces && c < kF4 ? load16_coherent(rs, partial_offset(a, c, p0 + q))
                                               : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
      for (int q = 0; q < kBatch; ++q)
#pragma unroll
        for (int k = 0; k < kOwn; ++k) {
          const int c = lane + k * kWave;
          if (p0 + q < pieces && c < kF4) {
            const float wgt = s_w[2 * ((4 * c / D) * kMaxStepPartitions + p0 + q) + 1];
            num[k] += wgt * __builtin_bit_cast(float4_t, v[q][k]);
          }
        }
    }
#pragma unroll
    for (int k = 0; k < kOwn; ++k) {
      const int c = lane + k * kWave;
      if (c < kF4) {
        const int h = 4 * c / D;
        const float den = s_w[2 * h * kMaxStepPartitions];
        half4_t o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (_Float16)(num[k][e] / den);
        *reinterpret_cast<half4_t*>(static_cast<_Float16*>(a.out) + (row0 + h) * D + 4 * c % D) = o;
      }
    }
  }
};

template <int D, int G, bool FP8, int MODE>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(PKV_STREAM_WAVES_PER_EU, 8)))
void decode_stream_kernel(DecodeArgs a, int B, int workers) {
  using K = StreamKernel<D, G, FP8, MODE>;
  using Geo = MfmaGeo<D, FP8>;
  static_assert(G <= 16, "head slots of one 16-wide product");
  const int lane = threadIdx.x;
  const int worker = blockIdx.x;
  const int g = lane / 16;
  const int n16 = lane % 16;
  const int k_off = n16 * Geo::kRow + g * 16;
  const int v_off = (4 * g) * Geo::kRow + n16 * Geo::kVBytes;

  __shared__ float s_w[2 * G * kMaxStepPartitions];
  __shared__ float s_cos[K::QKNORM ? D / 2 : 1];
  __shared__ float s_sin[K::QKNORM ? D / 2 : 1];

  const int64_t W = total_tiles(a, B);
  // equal shares, but long enough that a segment spans at most max_partitions
  const int64_t tpw = max((W + workers - 1) / workers,
                          int64_t(a.MBS + a.max_partitions - 3) / (a.max_partitions - 2));
  const int64_t t0 = int64_t(worker) * tpw;
  const int64_t t1 = min(W, t0 + tpw);

  if (t0 < t1) {
    Cursor cur = locate(a, B, t0);
    int rope_b = -1;  // sequence whose angles are in s_cos / s_sin
    auto prepare_segment = [&](const Meta& m, half8_t* qdst) {
      if constexpr (K::QKNORM) {
        if (m.b != rope_b) {
          rope_table<D, 1>(s_cos, s_sin, m.L - 1, a.theta);
          rope_b = m.b;
        }
      }
      K::load_q(qdst, a, m.b, m.kvh, g, n16, s_cos, s_sin);
    };

    MState<D, FP8> st;
    st.m = -FLT_MAX;
    st.l = 0.0f;
#pragma unroll
    for (int i = 0; i < Geo::kPV; ++i) st.acc[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    half8_t qop[Geo::kQK], qnext[Geo::kQK];
    MTile<D, FP8> ta, tb;
    // metas run one tile ahead of the data loads: `ahead` is the tile after
    // the one being loaded, so its block id has a whole step to arrive
    Meta ma = meta_of(cur, a, t0, t0, t1), mb, ahead;
    if (t0 + 1 < t1) {
      advance(cur, a, B);
      ahead = meta_of(cur, a, t0 + 1, t0, t1);
    }
    prepare_segment(ma, qnext);
    K::issue(ta, a, ma, true, g, n16, k_off, v_off, s_cos, s_sin);

    // process tile X (meta mx), loading the tile after it into Y
    auto step = [&](MTile<D, FP8>& x, const Meta& mx, MTile<D, FP8>& y, Meta& my, int64_t t) {
      if (mx.first)
#pragma unroll
        for (int c = 0; c < Geo::kQK; ++c) qop[c] = qnext[c];
      const bool live = t + 1 < t1;
      if (live) {
        my = ahead;
        if (my.first) prepare_segment(my, qnext);
      }
      K::issue(y, a, my, live, g, n16, k_off, v_off, s_cos, s_sin);
      if (t + 2 < t1) {
        advance(cur, a, B);
        ahead = meta_of(cur, a, t + 2, t0, t1);
      }
      issue_fence();
      mfma_tile<D, FP8>(st, x, qop, a.scale_log2, g);
      if (mx.last) K::flush(st, a, mx, qop, tpw, worker, g, n16, s_w);
    };

    for (int64_t t = t0; t < t1;) {
      step(ta, ma, tb, mb, t);
      if (++t >= t1) break;
      step(tb, mb, ta, ma, t);
      ++t;
    }
  }

  // sequences with no tokens: zero output rows, one wave each
  for (int b = worker; b < B; b += workers)
    if (load_uniform(a.context_lens + b) == 0)
      for (int i = lane; i < a.Hq * D; i += kWave)
        static_cast<_Float16*>(a.out)[size_t(b) * a.Hq * D + i] = (_Float16)0.0f;
}

int stream_workers() {
  static int workers = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    return cus * 4 * PKV_STREAM_WAVES_PER_EU;
  }();
  return workers;
}

template <int D, int G, bool FP8, int MODE>
hipError_t launch_stream(const DecodeArgs& a, int B, hipStream_t stream) {
  const int workers = stream_workers();
  hipLaunchKernelGGL((decode_stream_kernel<D, G, FP8, MODE>), dim3(workers), dim3(kWave), 0, stream,
                     a, B, workers);
  return hipGetLastError();
}

template <int D, int G, bool FP8>
hipError_t launch_stream_mode(const DecodeArgs& a, int B, int mode, hipStream_t stream) {
  if constexpr (FP8) {
    if (mode == kModeCombine) return launch_stream<D, G, true, kModeCombine>(a, B, stream);
    return hipErrorInvalidValue;
  } else {
    switch (mode) {
      case kModeCombine: return launch_stream<D, G, false, kModeCombine>(a, B, stream);
      case kModeAppend | kModeCombine:
        return launch_stream<D, G, false, kModeAppend | kModeCombine>(a, B, stream);
      case kModeAppend | kModeQkNorm | kModeCombine:
        return launch_stream<D, G, false, kModeAppend | kModeQkNorm | kModeCombine>(a, B, stream);
      default: return hipErrorInvalidValue;
    }
  }
}

template <int D, bool FP8>
hipError_t launch_stream_group(const DecodeArgs& a, int B, int group, int mode, hipStream_t stream) {
  switch (group) {
    case 1: return launch_stream_mode<D, 1, FP8>(a, B, mode, stream);
    case 2: return launch_stream_mode<D, 2, FP8>(a, B, mode, stream);
    case 4: return launch_stream_mode<D, 4, FP8>(a, B, mode, stream);
    case 8: return launch_stream_mode<D, 8, FP8>(a, B, mode, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_stream(const DecodeArgs& a, int B, int D, int group, bool fp8, int mode,
                                hipStream_t stream) {
  if (D == 128) return fp8 ? launch_stream_group<128, true>(a, B, group, mode, stream)
                           : launch_stream_group<128, false>(a, B, group, mode, stream);
  if (D == 64) return fp8 ? launch_stream_group<64, true>(a, B, group, mode, stream)
                          : launch_stream_group<64, false>(a, B, group, mode, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
