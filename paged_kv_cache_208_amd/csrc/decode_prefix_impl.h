// Balanced decode step for a batch whose tables all start with the same
// physical blocks (a shared prompt prefix prefilled once into blocks that
// every sequence maps: "Roadmap: vLLM-style serving features for TornadoVM
// batched decode", Serving / scheduling; "Distributed LLM Inference Serving
// Platform", sections 2 and 11, reference-counted shared blocks).
//
// The prefix's tiles are read once per group of 16 / g sequences instead of
// once per sequence: the g q heads of each sequence of a group fill the 16
// columns of the same products, so one read of a prefix tile serves the
// whole group.  Per kv head the flattened order is
//     [prefix span of group 0] .. [prefix span of group NG-1]
//     [own tiles of sequence 0] .. [own tiles of sequence B-1]
// (a prefix span is the Tp prefix tiles with the group's 16 columns; a
// sequence's own tiles are the ones after the prefix, with its g columns).
// The waves' ranges split this order evenly exactly as in the plain
// balanced step.  All tiles load with the non-temporal policy.
//
// Every (sequence, kv head) output combines its group's np prefix pieces
// and its own pieces (log-sum-exp, as paged_attn_reduce does), in a second
// launch: with the combine in the same launch, the last piece of an output
// to arrive would combine it, and the waves that finish last (those holding
// the prefix spans of whole groups) would pile up the combines of every
// member.  The attend launch writes each piece's partial (prefix pieces in
// slots 0..np-1, own pieces after them); the own part's first piece also
// stores np + (own pieces) in the output's counter, which the combine
// launch reads, uses and clears (one wave per output).
//
// A piece that ends inside a wave's range is parked in LDS and written out
// with the range's last piece: a store issued between tile loads would hold
// up the wait for every tile behind it (vector memory operations complete
// in issue order).  A wave with more pieces than LDS slots writes early.
#pragma once
#include "decode_stream_impl.h"

namespace pkv {
namespace {

// Tiles of a sequence's own part (after the shared prefix of Tp tiles).
__device__ __forceinline__ int own_tiles(int L, int Tp) { return max(0, (L + 15) / 16 - Tp); }

struct PrefixGeom {
  int Tp;      // prefix tiles (16-token)
  int NG;      // groups of spp sequences
  int spp;     // sequences per group: 16 / g
  int64_t wh;  // tiles per kv head: NG * Tp + sum of own tiles
};

// Cursor over the prefix order: kind 1 = prefix span of group grp (whose
// leader, sequence grp * spp, supplies the table row), kind 0 = own tiles
// of sequence b.
struct PCursor {
  int kind, grp, b, kvh, n;
  int L, T, f;
  int64_t S;
};

__device__ __forceinline__ void p_set_prefix(PCursor& c, const PrefixGeom& pg, int grp) {
  c.kind = 1;
  c.grp = grp;
  c.b = grp * pg.spp;
  c.L = 16 * pg.Tp;
  c.T = pg.Tp;
  c.f = 0;
}

// Own tiles of all sequences, the largest segment, and the first chunk's
// inclusive scan (reused by p_locate).
__device__ __forceinline__ Totals p_totals(const DecodeArgs& a, int B, int L0, const PrefixGeom& pg) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t tot = 0;
  int mx = pg.Tp, incl0 = 0;
  for (int c = 0; c < B; c += kWave) {
    const int b = c + lane;
    const int T = own_tiles(c == 0 ? L0 : b < B ? a.context_lens[b] : 0, pg.Tp);
    const int incl = wave_scan(T);
    if (c == 0) incl0 = incl;
    tot += __builtin_amdgcn_readlane(incl, kWave - 1);
    mx = max(mx, T);
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) mx = max(mx, __shfl_xor(mx, off));
  const int64_t per_head = int64_t(pg.NG) * pg.Tp + tot;
  return Totals{per_head * a.Hkv, per_head, __builtin_amdgcn_readfirstlane(mx), incl0};
}

__device__ __forceinline__ PCursor p_locate(const DecodeArgs& a, int B, int64_t t, const PrefixGeom& pg,
                                           int L0, int incl0) {
  const int lane = threadIdx.x & (kWave - 1);
  PCursor c{};
  c.kvh = int(div_nn(t, pg.wh));
  const int64_t r = t - int64_t(c.kvh) * pg.wh;
  const int64_t pre = int64_t(pg.NG) * pg.Tp;
  if (r < pre) {
    const int grp = int(div_nn(r, pg.Tp));
    p_set_prefix(c, pg, grp);
    c.n = int(r - int64_t(grp) * pg.Tp);
    c.S = int64_t(c.kvh) * pg.wh + int64_t(grp) * pg.Tp;
    return c;
  }
  const int64_t r2 = r - pre;
  int64_t carry = 0;
  for (int c0 = 0; c0 < B; c0 += kWave) {
    const int b = c0 + lane;
    const int L = c0 == 0 ? L0 : b < B ? a.context_lens[b] : 0;
    const int w = own_tiles(L, pg.Tp);
    const int incl = c0 == 0 ? incl0 : wave_scan(w);
    const int64_t hi = carry + incl;
    const int64_t lo = hi - w;
    const uint64_t here = __builtin_amdgcn_ballot_w64(b < B && lo <= r2 && r2 < hi);
    if (here) {
      const int src = __builtin_ctzll(here);
      c.kind = 0;
      c.b = c0 + src;
      c.L = __builtin_amdgcn_readlane(L, src);
      c.T = own_tiles(c.L, pg.Tp);
      c.f = pg.Tp;
      const int64_t lo_src = carry + __builtin_amdgcn_readlane(incl - w, src);
      c.n = int(r2 - lo_src);
      c.S = int64_t(c.kvh) * pg.wh + pre + lo_src;
      return c;
    }
    carry += __builtin_amdgcn_readlane(incl, kWave - 1);
  }
  return c;  // not reached for t < total
}

// Next tile of the prefix order; past the last tile c.b == B.
__device__ __forceinline__ void p_advance(PCursor& c, const DecodeArgs& a, int B, const PrefixGeom& pg) {
  if (++c.n < c.T) return;
  c.n = 0;
  c.S += c.T;
  if (c.kind == 1) {
    if (c.grp + 1 < pg.NG) {
      p_set_prefix(c, pg, c.grp + 1);
      return;
    }
    c.kind = 0;
    c.b = -1;
  }
  for (;;) {
    if (++c.b >= B) {
      if (++c.kvh >= a.Hkv) {
        c.b = B;
        return;
      }
      p_set_prefix(c, pg, 0);
      return;
    }
    c.L = load_uniform(a.context_lens + c.b);
    c.T = own_tiles(c.L, pg.Tp);
    c.f = pg.Tp;
    if (c.T > 0) return;
  }
}

template <int D, int C, bool FP8, int MODE, bool EXT>
struct PrefixKernel {
  using K = StreamKernel<D, C, FP8, MODE, EXT, false>;
  using Geo = MfmaGeo<D, FP8>;
  static constexpr int kSpp = 16 / C;             // sequences of a group
  static constexpr int kStage = 16 * D + 2 * 16;  // a 16-column partial in LDS

  static __device__ __forceinline__ Meta meta_of(const PCursor& c, const DecodeArgs& a, int64_t t,
                                                 int64_t t0, int64_t t1) {
    Meta m;
    m.id = load_uniform(a.block_tables + size_t(c.b) * a.MBS + ((c.f + c.n) >> K::BSS(a)));
    m.half = (c.f + c.n) & (K::BST(a) - 1);
    m.slot = 0;
    m.f = c.f;
    m.lo = 0;
    m.b = c.b;
    m.kvh = c.kvh;
    m.cg = 0;
    m.kind = c.kind;
    m.grp = c.grp;
    m.n = c.n;
    m.L = c.L;
    m.T = c.T;
    m.S = c.S;
    m.first = c.n == 0 || t == t0;
    m.last = c.n == c.T - 1 || t == t1 - 1;
    return m;
  }

  // q of the segment: a sequence's g heads, or the 16 columns of a group
  // (column col: sequence leader + col / g, head kvh * g + col % g; zero
  // past the batch).
  static __device__ __forceinline__ void load_q(half8_t* qop, const DecodeArgs& a, const Meta& m, int B,
                                                int g, int n16) {
    if (m.kind == 0) {
      K::load_q(qop, a, m.b, m.kvh, 0, g, n16);
      return;
    }
    const int lead = m.b;
    const int nseq = min(kSpp, B - lead);
    const _Float16* qs = static_cast<const _Float16*>(a.q) + size_t(lead) * a.Hq * D;
    const int span = nseq * a.Hq * D;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(qs, span * int(sizeof(_Float16)));
    const int row = (n16 / C) * a.Hq + m.kvh * C + n16 % C;
#pragma unroll
    for (int c = 0; c < Geo::kQK; ++c)
      qop[c] = __builtin_bit_cast(half8_t, buffer_load16(r, (row * D + qk_dim0<FP8>(c, g)) * int(sizeof(_Float16))));
  }

  // Every tile is streamed (non-temporal): with the prefix read once per
  // group instead of once per sequence, keeping it cached gains less than a
  // load form chosen per tile costs in the loop.
  static __device__ __forceinline__ void issue(MTile<D, FP8>& t, const DecodeArgs& a, const Meta& m,
                                               bool live, int k_off, int v_off) {
    const size_t base =
        live ? ((size_t(m.id) * a.Hkv + m.kvh) * K::BST(a) + m.half) * Geo::kTile : 0;
    load_mtile_at<D, FP8>(t, a, base, live ? min(16, m.L - 16 * (m.f + m.n)) : 0, k_off, v_off);
    t.lo = 0;
  }

  // The NC columns' o / l, maxima and sums of a piece, into LDS.
  template <int NC>
  static __device__ __forceinline__ void stage(const MState<D, FP8>& st, float l, int g, int n16,
                                               float* s_o) {
    if (n16 >= NC) return;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < Geo::kPV; ++i) s_o[n16 * D + (4 * g + r) * Geo::kPV + i] = st.acc[i][r] * inv;
    if (g == 0) {
      s_o[NC * D + n16] = st.m * kLn2;
      s_o[NC * D + NC + n16] = l;
    }
  }

  // Slot j of the C partial rows of segment seg from LDS: o rows at o, maxima
  // at mv, sums at lv (plain stores: the combine launch reads them).
  static __device__ __forceinline__ void write_rows(const DecodeArgs& a, int seg, int j, const float* o,
                                                    const float* mv, const float* lv) {
    const int lane = threadIdx.x & (kWave - 1);
    const size_t row0 = size_t(seg) * C;
    const __amdgpu_buffer_rsrc_t rs = K::partial_rows(a, row0);
#pragma unroll
    for (int k = 0; k < K::kOwn; ++k) {
      const int c = lane + k * kWave;
      if (c < K::kF4)
        store16<false>(rs, K::partial_offset(a, c, j), *reinterpret_cast<const u32x4*>(o + 4 * c));
    }
    if (lane < C) {
      const size_t pr = (row0 + lane) * a.max_partitions + j;
      store_f32<false>(a.part_max + pr, mv[lane]);
      store_f32<false>(a.part_sum + pr, lv[lane]);
    }
  }

  // Pieces of the prefix span of group grp (kv head kvh).
  static __device__ __forceinline__ int prefix_pieces(const Ranges& rg, const PrefixGeom& pg, int kvh,
                                                      int grp) {
    const int64_t S = int64_t(kvh) * pg.wh + int64_t(grp) * pg.Tp;
    return int(rg.of(S + pg.Tp - 1) - rg.of(S) + 1);
  }

  // LDS slots for parked pieces: four for fp16 waves (one per SIMD), two
  // for E4M3 waves (two per SIMD), so that a CU's waves fit in its LDS.
  static constexpr int kSlots = FP8 ? 2 : 4;
  // Row entries: at most kSpp per parked piece.
  static constexpr int kEntries = kSlots * kSpp;

  // Row entry e (3 ints in LDS): the (sequence, kv head) output, the piece
  // count it stores in the output's counter (own part's first piece; else
  // 0), and where the rows are: partial slot j in memory, member s of LDS
  // slot k, kind (1: a prefix span's 16 staged columns, 0: an own piece's C).
  static __device__ __forceinline__ void put_entry(int* s_ent, int e, int seg, int count, int j, int s,
                                                   int kind, int k) {
    s_ent[3 * e] = seg;
    s_ent[3 * e + 1] = count;
    s_ent[3 * e + 2] = j | (s << 8) | (kind << 16) | (k << 20);
  }

  // Park the partial of piece m (which ends in this range) in LDS slot k
  // and append its row entries (every member with own tiles for a prefix
  // span: the others have no output) to the nent so far; returns the new
  // count.
  static __device__ __forceinline__ int park(const DecodeArgs& a, int B, const Meta& m,
                                             const MState<D, FP8>& st, const Ranges& rg,
                                             const PrefixGeom& pg, int64_t rw, int64_t t0, int64_t t1,
                                             int g, int n16, int k, float* s_stage, int* s_ent,
                                             int nent) {
    const int lane = threadIdx.x & (kWave - 1);
    const float l = group4_sum(st.l);
    const int64_t r_first = m.S >= t0 ? rw : rg.of(m.S);
    const int64_t r_last = m.S + m.T <= t1 ? rw : rg.of(m.S + m.T - 1);
    const int pieces = int(r_last - r_first + 1);
    const int j = int(rw - r_first);
    float* s_k = s_stage + k * kStage;
    if (m.kind == 0) {
      const int np = prefix_pieces(rg, pg, m.kvh, m.b / kSpp);
      stage<C>(st, l, g, n16, s_k);
      if (lane == 0) put_entry(s_ent, nent, m.b * a.Hkv + m.kvh, j == 0 ? np + pieces : 0, np + j, 0, 0, k);
      return nent + 1;
    }
    stage<16>(st, l, g, n16, s_k);
#pragma unroll
    for (int s = 0; s < kSpp; ++s) {
      const int b = m.b + s;
      const int Lb = load_uniform(a.context_lens + min(b, B - 1));  // in bounds either way
      if (b < B && own_tiles(Lb, pg.Tp) > 0) {
        if (lane == 0) put_entry(s_ent, nent, b * a.Hkv + m.kvh, 0, j, s, 1, k);
        ++nent;
      }
    }
    return nent;
  }

  // Write out the parked partials (and the piece counts).
  static __device__ __forceinline__ void flush(const DecodeArgs& a, int nent, const float* s_stage,
                                               const int* s_ent) {
    for (int e = 0; e < nent; ++e) {
      const int seg = __builtin_amdgcn_readfirstlane(s_ent[3 * e]);
      const int count = __builtin_amdgcn_readfirstlane(s_ent[3 * e + 1]);
      const int w = __builtin_amdgcn_readfirstlane(s_ent[3 * e + 2]);
      const int j = w & 0xFF, s = (w >> 8) & 0xFF, k = w >> 20;
      const float* s_k = s_stage + k * kStage;
      if ((w >> 16) & 0xF)
        write_rows(a, seg, j, s_k + s * C * D, s_k + 16 * D + s * C, s_k + 16 * D + 16 + s * C);
      else
        write_rows(a, seg, j, s_k, s_k + C * D, s_k + C * D + C);
      if (count > 0 && (threadIdx.x & (kWave - 1)) == 0) a.counters[seg] = uint32_t(count);
    }
  }

  // The step's new row (token L - 1, an own tile) of every sequence whose
  // own tiles in [t0, t1) hold it, written before the loop by the lanes
  // that later load it.
  static __device__ __forceinline__ void append_rows(const DecodeArgs& a, int B, PCursor c, int64_t t0,
                                                     int64_t t1, const PrefixGeom& pg, int g, int n16,
                                                     int k_off, int v_off) {
    using VW = typename Words<Geo::kVWords>::T;
    while (c.S < t1 && c.b < B) {
      if (c.kind == 0) {
        const int p = c.L - 1;
        const int64_t tile = c.S + (p / 16 - c.f);
        if (p >= 16 * pg.Tp && tile >= t0 && tile < t1) {
          const int id = load_uniform(a.block_tables + size_t(c.b) * a.MBS + ((p / 16) >> K::BSS(a)));
          const size_t row = size_t(c.b) * a.Hkv + c.kvh;
          const _Float16* kn = static_cast<const _Float16*>(a.k_new) + row * D;
          const _Float16* vn = static_cast<const _Float16*>(a.v_new) + row * D;
          u32x4 kc[Geo::kKLoads];
#pragma unroll
          for (int k = 0; k < Geo::kKLoads; ++k)
            kc[k] = *reinterpret_cast<const u32x4*>(kn + (4 * k + g) * 8);
          const VW vc = *reinterpret_cast<const VW*>(vn + n16 * (D / 16));
          const int r_new = p % 16;
          const size_t base =
              ((size_t(id) * a.Hkv + c.kvh) * K::BST(a) + ((p / 16) & (K::BST(a) - 1))) * Geo::kTile;
          uint8_t* kt = const_cast<uint8_t*>(a.k_pool) + base;
          uint8_t* vt = const_cast<uint8_t*>(a.v_pool) + base;
          if (n16 == r_new)
#pragma unroll
            for (int k = 0; k < Geo::kKLoads; ++k) *reinterpret_cast<u32x4*>(kt + k_off + k * 64) = kc[k];
          if (g == r_new / 4) *reinterpret_cast<VW*>(vt + v_off + (r_new % 4) * Geo::kRow) = vc;
        }
      }
      c.n = c.T - 1;
      p_advance(c, a, B, pg);
    }
  }
};

template <int D, int C, bool FP8, int MODE, bool EXT>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(stream_waves_per_eu<FP8>(), 8)))
void decode_prefix_kernel(const int32_t* __restrict__ lens, int B, int workers, DecodeArgs a) {
  using P = PrefixKernel<D, C, FP8, MODE, EXT>;
  using K = typename P::K;
  using Geo = MfmaGeo<D, FP8>;
  static_assert(16 % C == 0, "a group fills the 16 columns of a product");
  const int lane = threadIdx.x;
  const int worker = blockIdx.x;
  const int g = lane / 16;
  const int n16 = lane % 16;
  const int k_off = n16 * Geo::kRow + g * 16;
  const int v_off = (4 * g) * Geo::kRow + n16 * Geo::kVBytes;

  __shared__ float s_stage[P::kSlots * P::kStage];  // parked partials
  __shared__ int s_ent[3 * P::kEntries];            // their rows

  PrefixGeom pg;
  pg.Tp = a.prefix_tiles;
  pg.spp = P::kSpp;
  pg.NG = (B + P::kSpp - 1) / P::kSpp;
  const int L0 = lane < B ? lens[lane] : 0;  // lens = a.context_lens, preloaded
  const Totals tot = p_totals(a, B, L0, pg);
  pg.wh = tot.per_head;
  const int64_t W = tot.tiles;
  const Ranges rg = make_ranges<FP8>(W, tot.max_tiles, workers, a.max_partitions / 2);
  const int64_t rw = range_of_worker(worker, workers);
  const int64_t t0 = min(rg.start(rw), W);
  const int64_t t1 = min(W, rg.start(rw + 1));

  if (t0 < t1) {
    PCursor cur = p_locate(a, B, t0, pg, L0, tot.incl0);
    if constexpr (K::APPEND) P::append_rows(a, B, cur, t0, t1, pg, g, n16, k_off, v_off);

    MState<D, FP8> st;
    K::reset(st);
    constexpr int NB = K::kDepth;
    MTile<D, FP8> tl[NB];
    Meta mt[NB];
    Meta ahead;
    Meta mfin;
    half8_t qop[Geo::kQK];
    half8_t qbuf[NB][Geo::kQK];
    auto take = [&](Meta& m, half8_t* qdst) {
      if (m.first) P::load_q(qdst, a, m, B, g, n16);
    };
    mt[0] = P::meta_of(cur, a, t0, t0, t1);
    mt[0].first = true;
    take(mt[0], qbuf[0]);
    P::issue(tl[0], a, mt[0], true, k_off, v_off);
#pragma unroll
    for (int k = 1; k < NB; ++k) {
      const bool live = t0 + k < t1;
      if (live) {
        p_advance(cur, a, B, pg);
        Meta m = P::meta_of(cur, a, t0 + k, t0, t1);
        if (k < NB - 1) {
          mt[k] = m;
          take(mt[k], qbuf[k]);
        } else {
          ahead = m;
        }
      }
      if (k < NB - 1) P::issue(tl[k], a, mt[k], live, k_off, v_off);
    }

    int npark = 0, nent = 0;  // parked pieces and their row entries

    auto step = [&](MTile<D, FP8>& x, const Meta& mx, const half8_t* qx, MTile<D, FP8>& y, Meta& my,
                    half8_t* qy, int64_t t) {
      const bool live = t + NB - 1 < t1;
      if (live) {
        my = ahead;
        take(my, qy);
      }
      P::issue(y, a, my, live, k_off, v_off);
      if (t + NB < t1) {
        p_advance(cur, a, B, pg);
        ahead = P::meta_of(cur, a, t + NB, t0, t1);
      }
      issue_fence();
      if (mx.first) {
#pragma unroll
        for (int c = 0; c < Geo::kQK; ++c) qop[c] = qx[c];
      }
      issue_fence();
      const int col_hi = EXT ? mx.L - 16 * (mx.f + mx.n) : 16;
      mfma_tile<D, FP8>(st, x, qop, a.scale_log2, g, col_hi);
      if (t + 1 >= t1) {
        mfin = mx;
        return;
      }
      if (mx.last) {
        if (npark == P::kSlots) {
          P::flush(a, nent, s_stage, s_ent);
          npark = nent = 0;
        }
        nent = P::park(a, B, mx, st, rg, pg, rw, t0, t1, g, n16, npark, s_stage, s_ent, nent);
        ++npark;
        K::reset(st);
      }
    };

    for (int64_t t = t0; t < t1;) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int v = (u + NB - 1) % NB;
        step(tl[u], mt[u], qbuf[u], tl[v], mt[v], qbuf[v], t);
        if (++t >= t1) break;
      }
    }
    // the range's last piece, and every piece parked before it
    if (npark == P::kSlots) {
      P::flush(a, nent, s_stage, s_ent);
      npark = nent = 0;
    }
    nent = P::park(a, B, mfin, st, rg, pg, rw, t0, t1, g, n16, npark, s_stage, s_ent, nent);
    P::flush(a, nent, s_stage, s_ent);
  }

  // sequences with no tokens: zero output rows, one wave each
  for (int b = worker; b < B; b += workers)
    if (load_uniform(a.context_lens + b) == 0)
      for (int i = lane; i < a.Hq * D; i += kWave)
        static_cast<_Float16*>(a.out)[size_t(b) * a.Hq * D + i] = (_Float16)0.0f;
}

template <int D, int C, bool FP8, int MODE>
hipError_t launch_prefix(const DecodeArgs& a, int B, hipStream_t stream) {
  const int workers = device_cus() * 4 * stream_waves_per_eu<FP8>();
  if (a.bs_tiles > 1)
    hipLaunchKernelGGL((decode_prefix_kernel<D, C, FP8, MODE, true>), dim3(workers), dim3(kWave), 0,
                       stream, a.context_lens, B, workers, a);
  else
    hipLaunchKernelGGL((decode_prefix_kernel<D, C, FP8, MODE, false>), dim3(workers), dim3(kWave), 0,
                       stream, a.context_lens, B, workers, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nseg = B * a.Hkv;
  // the balanced step's combine launch: one output (sequence, kv head) per
  // segment, nq = 1, so the plain layout applies
  hipLaunchKernelGGL((stream_combine_kernel<D, C, FP8, false>), dim3(min(nseg, 2 * workers)),
                     (combine_block<D, C, FP8, false>()),
                     0, stream, a.counters, nseg, a);
  return hipGetLastError();
}

template <int D, int C, bool FP8>
hipError_t launch_prefix_mode(const DecodeArgs& a, int B, int mode, hipStream_t stream) {
  if (mode == kModeCombine) return launch_prefix<D, C, FP8, kModeCombine>(a, B, stream);
  if constexpr (!FP8)
    if (mode == (kModeAppend | kModeCombine))
      return launch_prefix<D, C, false, kModeAppend | kModeCombine>(a, B, stream);
  return hipErrorInvalidValue;
}

template <int D, bool FP8>
hipError_t launch_prefix_cols(const DecodeArgs& a, int B, int cols, int mode, hipStream_t stream) {
  switch (cols) {
    case 1: return launch_prefix_mode<D, 1, FP8>(a, B, mode, stream);
    case 2: return launch_prefix_mode<D, 2, FP8>(a, B, mode, stream);
    case 4: return launch_prefix_mode<D, 4, FP8>(a, B, mode, stream);
    case 8: return launch_prefix_mode<D, 8, FP8>(a, B, mode, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace pkv
