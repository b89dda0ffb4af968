// Balanced decode step for gfx950: append (+ QK-norm/RoPE), attention and
// the combine of split contexts, with every wave given the same amount of
// KV to read: an attend launch and a combine launch, or one launch with
// QK-norm.
//
// The batch's tiles are laid out in one flattened order: kv head, then
// sequence b, then the sequence's 16-token tiles ("Distributed LLM Inference
// Serving Platform", section 2: logical block n of a sequence is found
// through its block table).  With W tiles in total and C waves (a fixed
// number per CU), the ranges are contiguous runs of about W / C tiles (with
// two waves per SIMD the first-placed waves' ranges are a little longer; see
// Ranges), and the waves of one XCD take one contiguous block of ranges: an
// XCD reads about one kv head's tiles, so the blocks that several sequences
// share (a common prefix) are re-read through that XCD's own L2, and the
// pieces of a split segment mostly come from one XCD.  Every wave therefore
// moves about the same number of bytes, whatever the mix of context
// lengths, and streams straight
// across the boundaries between (sequence, kv head) segments: the next
// tile's loads are issued before the current tile is computed, whichever
// segment it belongs to.
//
// A segment that lies inside one wave's range is finished by that wave (the
// normalised output is written directly).  A segment shared by several
// consecutive waves leaves one partial (m, l, o) per wave, combined
// (log-sum-exp, as paged_attn_reduce does) by the combine launch, which
// reads the piece count the segment's first piece left in its counter; each
// of its lanes keeps a running log-sum-exp of its own float4s of the rows.
// With QK-norm the last wave to finish its piece combines them in the same
// launch (and writes q' back), counting arrivals with device-scope coherent
// accesses.  The counters return to zero either way.
//
// Inside the loop a wave issues only loads (KV tiles, and q when a tile
// starts a segment): vector memory operations complete in issue order, so a
// store would hold up the wait for every tile behind it.  The step's new rows
// are therefore written before the loop (by the wave whose range holds the
// segment's last tile), and a partial that ends mid-range stays in LDS until
// the range is done.  Block ids and lengths come through the scalar cache.
//
// Each wave is its own 64-thread workgroup; the tile engine is the MFMA one
// of decode_tile.h.
//
// This header holds the kernel and its launchers for either cache policy of
// the KV loads; decode_stream.hip (non-temporal) and decode_stream_cached.hip
// (default policy, the caller's shared-blocks hint) each instantiate one, so
// the two halves compile in parallel.
#pragma once
#include "decode_tile.h"
#include "shape_limits.h"

// Waves resident per SIMD, which sets the register budget; the grid is one
// wave per resident slot, four SIMDs per CU.  fp16 tiles (8 KiB of K and V)
// keep enough bytes in flight with one wave per SIMD and its full register
// file; E4M3 tiles are half the size and want two.
#ifndef PKV_STREAM_WAVES_PER_EU_F16
#define PKV_STREAM_WAVES_PER_EU_F16 1
#endif
#ifndef PKV_STREAM_WAVES_PER_EU_FP8
#define PKV_STREAM_WAVES_PER_EU_FP8 2
#endif
#ifndef PKV_STREAM_DEPTH
#define PKV_STREAM_DEPTH 2
#endif

namespace pkv {
namespace {

template <bool FP8>
constexpr int stream_waves_per_eu() {
  return FP8 ? PKV_STREAM_WAVES_PER_EU_FP8 : PKV_STREAM_WAVES_PER_EU_F16;
}

// Position of one tile in the flattened order.
// A segment is one (sequence, kv head, column group): with cg > 1 column
// groups the query columns of a sequence (g heads times its new tokens) are
// split over cg 16-column products, each of which reads the sequence's
// tiles once.
struct Cursor {
  int b, kvh, n;  // sequence, kv head, tile within the segment
  int cg;         // column group
  int L, T;       // context length of b, tiles per segment
  int f;          // block-table index of the segment's first tile
  int64_t S;      // flattened index of the segment's first tile
};

// With a sliding window of W tokens (W > 0) a sequence of length L reads
// positions max(0, L - W) .. L - 1: its segment starts at the tile holding
// the first of them.
__device__ __forceinline__ int window_start(int L, int W) { return (W > 0 && L > W) ? L - W : 0; }
__device__ __forceinline__ int first_tile(int L, int W) { return window_start(L, W) / 16; }
__device__ __forceinline__ int seg_tiles(int L, int W) { return (L + 15) / 16 - first_tile(L, W); }

// Quotient of non-negative a / b, with the 32-bit division when both fit
// (every realistic batch: a 64-bit division is a long software sequence).
__device__ __forceinline__ int64_t div_nn(int64_t a, int64_t b) {
  if (((uint64_t(a) | uint64_t(b)) >> 32) == 0) return int64_t(uint32_t(a) / uint32_t(b));
  return a / b;
}

// Inclusive prefix sum over the 64 lanes (tile counts: a chunk of 64
// sequences holds far fewer than 2^31 tiles).
__device__ __forceinline__ int wave_scan(int x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Tiles of the batch (all kv heads), of one kv head, and the most tiles of
// one sequence; incl0: this lane's inclusive prefix sum over the first
// chunk of 64 sequences (all of them when B <= 64), which locate() reuses.
struct Totals {
  int64_t tiles, per_head;
  int max_tiles;
  int incl0;
};

// L0: this lane's length in the first chunk of 64 sequences, read once by
// the caller and used by both scans.
__device__ __forceinline__ Totals total_tiles(const DecodeArgs& a, int B, int L0, int W, int CG) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t tot = 0;
  int mx = 0, incl0 = 0;
  for (int c = 0; c < B; c += kWave) {
    const int b = c + lane;
    const int T = seg_tiles(c == 0 ? L0 : b < B ? a.context_lens[b] : 0, W);
    const int incl = wave_scan(T * CG);
    if (c == 0) incl0 = incl;
    tot += __builtin_amdgcn_readlane(incl, kWave - 1);
    mx = max(mx, T);
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) mx = max(mx, __shfl_xor(mx, off));
  return Totals{tot * a.Hkv, tot, __builtin_amdgcn_readfirstlane(mx), incl0};
}

// Cursor of flattened tile t (t < total); wh = tiles of one kv head.
__device__ __forceinline__ Cursor locate(const DecodeArgs& a, int B, int64_t t, int64_t wh, int L0,
                                        int incl0, int W, int CG) {
  const int lane = threadIdx.x & (kWave - 1);
  Cursor c{};
  c.kvh = int(div_nn(t, wh));
  const int64_t r = t - int64_t(c.kvh) * wh;  // position within the head's run
  int64_t carry = 0;
  for (int c0 = 0; c0 < B; c0 += kWave) {
    const int b = c0 + lane;
    const int L = c0 == 0 ? L0 : b < B ? a.context_lens[b] : 0;
    const int w = seg_tiles(L, W) * CG;
    const int incl = c0 == 0 ? incl0 : wave_scan(w);
    const int64_t hi = carry + incl;
    const int64_t lo = hi - w;
    const uint64_t here = __builtin_amdgcn_ballot_w64(b < B && lo <= r && r < hi);
    if (here) {
      const int src = __builtin_ctzll(here);
      c.b = c0 + src;
      c.L = __builtin_amdgcn_readlane(L, src);
      c.T = seg_tiles(c.L, W);
      c.f = first_tile(c.L, W);
      const int64_t lo_src = carry + __builtin_amdgcn_readlane(incl - w, src);
      const int nn = int(r - lo_src);  // tile within the sequence's cg segments
      c.cg = CG == 1 ? 0 : nn / c.T;
      c.n = nn - c.cg * c.T;
      c.S = int64_t(c.kvh) * wh + lo_src + int64_t(c.cg) * c.T;
      return c;
    }
    carry += __builtin_amdgcn_readlane(incl, kWave - 1);
  }
  return c;  // not reached for t < total
}

// Next tile in the flattened order (skips sequences with no tokens); past
// the last tile c.b == B.
__device__ __forceinline__ void advance(Cursor& c, const DecodeArgs& a, int B, int W, int CG) {
  if (++c.n < c.T) return;
  c.n = 0;
  c.S += c.T;
  if (++c.cg < CG) return;  // the sequence's next column group
  c.cg = 0;
  do {
    if (++c.b >= B) {
      c.b = 0;
      if (++c.kvh >= a.Hkv) {
        c.b = B;
        return;
      }
    }
    c.L = load_uniform(a.context_lens + c.b);
  } while (c.L == 0);
  c.T = seg_tiles(c.L, W);
  c.f = first_tile(c.L, W);
}

// 115: measured on the 70B-shaped E4M3 batch with the lane-local combine
// launch (100 to 150 swept; 110 and 120 run 0.3-0.8 us slower, 100 and 135
// 1-1.5 us slower).
#ifndef PKV_STREAM_SKEW_FP8
#define PKV_STREAM_SKEW_FP8 115
#endif

// The wave ranges, back to back in the flattened order, in nblk blocks of
// per = workers / nblk ranges (one block per XCD when the grid allows it).
// Wave w (on XCD w % nblk) reads range (w % nblk) * per + w / nblk, so an
// XCD's waves read one contiguous block, and the first half of the waves (w
// < workers / 2) read the first nh = per / 2 ranges of each block.  With two
// waves per SIMD the first wave placed on a SIMD is served first when both
// are ready to issue, and equal shares end far apart; that half then takes
// the larger share (skew, in percent of the other half's).
//
// Even split (the usual case): block x covers tiles [floor(x W / nblk),
// floor((x + 1) W / nblk)); its first half of ranges share A = its tiles *
// skew / (skew + 100), the second half the rest, and n ranges share S tiles
// as [floor(i S / n), floor((i + 1) S / n)), so no two ranges of a half
// differ by more than one tile.  Every range must still be long enough that
// no sequence is cut into more than P pieces (T tiles span at most
// (T - 1) / r + 2 ranges of r >= rmin tiles); when the shares are shorter
// than that (small batches) the ranges are rmin tiles each, back to back.
// a / d for a >= 0, a shift when d = 2^lg (lg >= 0).
__device__ __forceinline__ int64_t div_by(int64_t a, int64_t d, int lg) {
  return lg >= 0 ? a >> lg : div_nn(a, d);
}

__device__ __forceinline__ int log2_if_pow2(int64_t d) {
  return d > 0 && (d & (d - 1)) == 0 ? int(__builtin_ctzll(uint64_t(d))) : -1;
}

struct Ranges {
  int64_t W;        // tiles in total
  int64_t nblk, per, nh;
  int lg_nblk, lg_per, lg_nh, lg_rest;  // log2 of nblk, per, nh, per - nh when powers of two
  int skew;         // percent
  bool even;
  int64_t r;        // range length when !even
  __device__ __forceinline__ int64_t block_start(int64_t x) const { return div_by(x * W, nblk, lg_nblk); }
  __device__ __forceinline__ int64_t half_tiles(int64_t S) const {
    return skew == 100 ? S >> 1 : div_nn(S * skew, skew + 100);
  }
  __device__ __forceinline__ int64_t start(int64_t i) const {
    if (!even) return min(W, i * r);
    const int64_t x = div_by(i, per, lg_per), j = i - x * per;
    if (x >= nblk) return W;
    const int64_t b = block_start(x), S = block_start(x + 1) - b, A = half_tiles(S);
    return j < nh ? b + div_by(j * A, nh, lg_nh) : b + A + div_by((j - nh) * (S - A), per - nh, lg_rest);
  }
  __device__ __forceinline__ int64_t of(int64_t t) const {  // range holding tile t < W
    if (!even) return div_nn(t, r);
    const int64_t x = div_nn((t + 1) * nblk - 1, W);
    const int64_t b = block_start(x), S = block_start(x + 1) - b, A = half_tiles(S), u = t - b;
    const int64_t j = u < A ? div_nn((u + 1) * nh - 1, A)
                            : nh + div_nn((u - A + 1) * (per - nh) - 1, S - A);
    return x * per + j;
  }
};

__host__ __device__ constexpr int range_blocks(int workers) {
  return workers % (2 * kXcds) == 0 ? kXcds : 1;
}

__device__ __forceinline__ int64_t range_of_worker(int w, int workers) {
  const int nblk = range_blocks(workers);
  return int64_t(w % nblk) * (workers / nblk) + w / nblk;
}

template <bool FP8>
__device__ __forceinline__ Ranges make_ranges(int64_t W, int Tmax, int workers, int P) {
  const int64_t rmin = max(int64_t(1), int64_t(Tmax + P - 3) / (P - 2));
  Ranges rg;
  rg.W = max(W, int64_t(1));
  rg.nblk = range_blocks(workers);
  rg.per = workers / rg.nblk;
  rg.nh = max(int64_t(1), rg.per / 2);
  rg.skew = FP8 ? PKV_STREAM_SKEW_FP8 : 100;
  if (rg.per < 2) rg.skew = 100;
  rg.lg_nblk = log2_if_pow2(rg.nblk);
  rg.lg_per = log2_if_pow2(rg.per);
  rg.lg_nh = log2_if_pow2(rg.nh);
  rg.lg_rest = log2_if_pow2(rg.per - rg.nh);
  // shortest range of the even split: a block has at least floor(W / nblk)
  // tiles, each half at least that times its share, less one for rounding
  const int64_t smin = div_by(W, rg.nblk, rg.lg_nblk);
  const int64_t amin = rg.skew == 100 ? smin >> 1 : div_nn(smin * 100, rg.skew + 100);
  const int64_t shortest = min(div_by(amin, rg.nh, rg.lg_nh),
                               div_nn(max(int64_t(0), smin - amin - 1), max(int64_t(1), rg.per - rg.nh))) - 1;
  rg.even = rg.per >= 2 && shortest >= rmin;
  rg.r = max(div_by(W + workers - 1, workers, log2_if_pow2(workers)), rmin);
  return rg;
}

// What the loop needs to know about a tile besides its data.
struct Meta {
  int b, kvh, n, L, T, f;
  int cg;      // column group
  int kind;    // shared-prefix step: 1 a group's prefix span, 0 a sequence's own tiles
  int grp;     // shared-prefix step: the group
  int lo;      // rows of the tile before the window (first tile only)
  int id;      // physical block of the tile
  int half;    // which 16-token tile of a 32-token block
  int slot;    // angle table of the segment (QK-norm modes)
  int64_t S;
  bool first;  // first tile of the wave's piece of the segment
  bool last;   // last tile of the wave's piece of the segment
};

// W: window (0 = full); bst / shift: 16-token tiles per block and log2.
__device__ __forceinline__ Meta meta_of(const Cursor& c, const DecodeArgs& a, int64_t t, int64_t t0,
                                        int64_t t1, int W, int bst, int shift) {
  Meta m;
  // a scalar load; its result is first needed one loop step later
  m.id = load_uniform(a.block_tables + size_t(c.b) * a.MBS + ((c.f + c.n) >> shift));
  m.half = (c.f + c.n) & (bst - 1);
  m.slot = 0;
  m.f = c.f;
  m.lo = c.n == 0 ? window_start(c.L, W) - 16 * c.f : 0;
  m.b = c.b;
  m.kvh = c.kvh;
  m.cg = c.cg;
  m.n = c.n;
  m.L = c.L;
  m.T = c.T;
  m.S = c.S;
  m.first = c.n == 0 || t == t0;
  m.last = c.n == c.T - 1 || t == t1 - 1;
  return m;
}

// EXT: the window, several new tokens per sequence or 32-token blocks are in
// use; without it they are compile-time constants (full attention, one
// token, 16-token blocks) and the common kernel carries none of their code.
// CACHED: the caller's shared-blocks hint; KV tiles are loaded with the
// default cache policy instead of the non-temporal one.  A compile-time
// choice: a branch between the two load forms in the loop cost 2-10%.
template <int D, int C, bool FP8, int MODE, bool EXT, bool CACHED>
struct StreamKernel {
  using Geo = MfmaGeo<D, FP8>;
  static __device__ __forceinline__ int W(const DecodeArgs& a) { return EXT ? a.window : 0; }
  static __device__ __forceinline__ int NQ(const DecodeArgs& a) { return EXT ? a.nq : 1; }
  static __device__ __forceinline__ int GRP(const DecodeArgs& a) { return EXT ? a.group : C; }
  static __device__ __forceinline__ int BST(const DecodeArgs& a) { return EXT ? a.bs_tiles : 1; }
  static __device__ __forceinline__ int BSS(const DecodeArgs& a) { return EXT ? a.bs_shift : 0; }
  // column groups per (sequence, kv head) and query columns per (sequence,
  // kv head): g * nq; with more than one group each holds C = 16 columns
  static __device__ __forceinline__ int CG(const DecodeArgs& a) { return EXT ? a.cgroups : 1; }
  static __device__ __forceinline__ int NCOLS(const DecodeArgs& a) { return EXT ? a.ncols : C; }
  static constexpr bool APPEND = (MODE & kModeAppend) != 0;
  static constexpr bool QKNORM = (MODE & kModeQkNorm) != 0;
  // tiles in the load pipeline of a wave
  static constexpr int kDepth = PKV_STREAM_DEPTH;

  // The columns of a segment's 16-wide products: query column col (0 ..
  // g * nq - 1 of the sequence and kv head) is new query token col / g of q
  // head kvh * g + col % g (g = Hq / Hkv; one new token per sequence unless
  // nq > 1); column group cg holds columns cg * C .. cg * C + C - 1.  Row of
  // q and of out [B][nq][Hq][D]:
  static __device__ __forceinline__ size_t qrow(const DecodeArgs& a, int b, int kvh, int col) {
    return (size_t(b) * NQ(a) + col / GRP(a)) * a.Hq + kvh * GRP(a) + col % GRP(a);
  }
  // A segment's index (its arrival counter) and, from it, its sequence, kv
  // head and column group; its partial rows start at row0 (one row per query
  // column, in (sequence, kv head, column) order).
  static __device__ __forceinline__ int seg_id(const DecodeArgs& a, int b, int kvh, int cg) {
    return (b * a.Hkv + kvh) * CG(a) + cg;
  }
  static __device__ __forceinline__ size_t seg_row0(const DecodeArgs& a, int seg) {
    const int bk = CG(a) == 1 ? seg : seg / CG(a);
    return size_t(bk) * NCOLS(a) + size_t(seg - bk * CG(a)) * C;
  }
  static __device__ __forceinline__ size_t seg_qrow(const DecodeArgs& a, int seg, int col) {
    const int bk = CG(a) == 1 ? seg : seg / CG(a);
    return qrow(a, bk / a.Hkv, bk % a.Hkv, (seg - bk * CG(a)) * C + col);
  }

  // q of head slot n16 of the segment's group, laid out as the B operand of
  // the QK products; zero past the group.  Slots past the group read outside
  // the buffer's bound, which returns zeros, so no lane overwrites a register
  // that a load is still filling.  QK-norm is applied when the segment's
  // first tile is computed, once the loads have landed.
  static __device__ __forceinline__ void load_q(half8_t* qop, const DecodeArgs& a, int b, int kvh,
                                                int cg, int g, int n16) {
    const size_t base = size_t(b) * NQ(a) * a.Hq;
    const _Float16* qs = static_cast<const _Float16*>(a.q) + base * D;
    const int span = NQ(a) * a.Hq * D;  // the sequence's q rows
    const __amdgpu_buffer_rsrc_t r = make_rsrc(qs, span * int(sizeof(_Float16)));
    const int row = n16 < C ? int(qrow(a, b, kvh, cg * C + n16) - base) * D : span;
#pragma unroll
    for (int c = 0; c < Geo::kQK; ++c)
      qop[c] = __builtin_bit_cast(half8_t, buffer_load16(r, (row + qk_dim0<FP8>(c, g)) * int(sizeof(_Float16))));
  }

  // Write the step's nq new k and v rows (tokens L-nq .. L-1) of every
  // segment into the tiles of this wave's range [t0, t1) that hold them,
  // before any tile of the range is loaded.  The lanes that store each piece
  // are the ones that later load it (same lane, same address, program
  // order: the loads observe the stores); rows in tiles of another wave's
  // range are that wave's to write.  The loop then carries no append work.
  // c is the cursor of tile t0; s_cos / s_sin hold scratch angle tables
  // (QK-norm, nq = 1).
  static __device__ __forceinline__ void append_rows(const DecodeArgs& a, int B, Cursor c, int64_t t0,
                                                     int64_t t1, int g, int n16, int k_off, int v_off,
                                                     float* s_cos, float* s_sin, const double* s_f,
                                                     const float* s_gk) {
    using VW = typename Words<Geo::kVWords>::T;
    while (c.S < t1) {
      for (int i = 0; i < NQ(a); ++i) {
        const int p = c.L - NQ(a) + i;            // position of new token i
        const int64_t tile = c.S + (p / 16 - c.f);
        if (p < 0 || tile < t0 || tile >= t1) continue;
        const int id = load_uniform(a.block_tables + size_t(c.b) * a.MBS + ((p / 16) >> BSS(a)));
        const size_t row = (size_t(c.b) * NQ(a) + i) * a.Hkv + c.kvh;
        const _Float16* kn = static_cast<const _Float16*>(a.k_new) + row * D;
        const _Float16* vn = static_cast<const _Float16*>(a.v_new) + row * D;
        half8_t kc[Geo::kKLoads];
#pragma unroll
        for (int k = 0; k < Geo::kKLoads; ++k)
          kc[k] = __builtin_bit_cast(half8_t, *reinterpret_cast<const u32x4*>(kn + (4 * k + g) * 8));
        const VW vc = *reinterpret_cast<const VW*>(vn + n16 * (D / 16));
        if constexpr (QKNORM) {
          rope_angles<D>(s_f, s_cos, s_sin, p);
          norm_rope_chunks<D>(kc, s_gk, a.eps, s_cos, s_sin, g);
        }
        const int r_new = p % 16;
        const size_t base =
            ((size_t(id) * a.Hkv + c.kvh) * BST(a) + ((p / 16) & (BST(a) - 1))) * Geo::kTile;
        uint8_t* kt = const_cast<uint8_t*>(a.k_pool) + base;
        uint8_t* vt = const_cast<uint8_t*>(a.v_pool) + base;
        if (n16 == r_new)
#pragma unroll
          for (int k = 0; k < Geo::kKLoads; ++k)
            *reinterpret_cast<u32x4*>(kt + k_off + k * 64) = __builtin_bit_cast(u32x4, kc[k]);
        if (g == r_new / 4) *reinterpret_cast<VW*>(vt + v_off + (r_new % 4) * Geo::kRow) = vc;
      }
      // on to the next segment (the new rows are written once, by the
      // column group 0 segment; more groups exist only without an append)
      c.n = c.T - 1;
      c.cg = CG(a) - 1;
      advance(c, a, B, W(a), CG(a));
      if (c.b >= B) break;
    }
  }

  // Issue the loads of tile m.  A tile that is not live issues the same
  // loads with no valid rows: they read nothing, but every loop step then has
  // the same number of loads in flight behind the tile being computed, so the
  // wait before the products stays partial on every path.
  static __device__ __forceinline__ void issue(MTile<D, FP8>& t, const DecodeArgs& a, const Meta& m,
                                               bool live, int k_off, int v_off) {
    const size_t base =
        live ? ((size_t(m.id) * a.Hkv + m.kvh) * BST(a) + m.half) * Geo::kTile : 0;
    load_mtile_at<D, FP8>(t, a, base, live ? min(16, m.L - 16 * (m.f + m.n)) : 0, k_off, v_off,
                          CACHED);
    t.lo = live ? m.lo : 0;
  }

  // The first and last range holding a tile of segment m, for a tile of m in
  // range rw = [t0, t1), and the number of pieces the ranges cut it into.
  static __device__ __forceinline__ int64_t first_range(const Meta& m, const Ranges& rg, int64_t rw,
                                                        int64_t t0) {
    return m.S >= t0 ? rw : rg.of(m.S);
  }
  static __device__ __forceinline__ int64_t last_range(const Meta& m, const Ranges& rg, int64_t rw,
                                                       int64_t t1) {
    return m.S + m.T <= t1 ? rw : rg.of(m.S + m.T - 1);
  }

  // Output rows of a segment that lies inside one wave's range: o / l.
  static __device__ __forceinline__ void store_direct(const MState<D, FP8>& st, float l,
                                                      const DecodeArgs& a, int seg, int g, int n16) {
    if (n16 >= C) return;
    const float inv = 1.0f / l;
    _Float16* o = static_cast<_Float16*>(a.out) + seg_qrow(a, seg, n16) * D;
    typedef _Float16 hv __attribute__((ext_vector_type(Geo::kPV)));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      hv v;
#pragma unroll
      for (int i = 0; i < Geo::kPV; ++i) v[i] = (_Float16)(st.acc[i][r] * inv);
      *reinterpret_cast<hv*>(o + (4 * g + r) * Geo::kPV) = v;
    }
  }

  static __device__ __forceinline__ void reset(MState<D, FP8>& st) {
    st.m = -FLT_MAX;
    st.l = 0.0f;
#pragma unroll
    for (int i = 0; i < Geo::kPV; ++i) st.acc[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // q' (QK-norm) back in place, from the operand registers or from the LDS
  // copy taken when the piece ended; done by the wave that finishes the
  // segment, when no other wave still needs q.
  static __device__ __forceinline__ void write_q(const DecodeArgs& a, int seg, const half8_t* qop,
                                                 int g, int n16) {
    if (n16 >= C) return;
    _Float16* qh = const_cast<_Float16*>(static_cast<const _Float16*>(a.q)) + seg_qrow(a, seg, n16) * D;
#pragma unroll
    for (int c = 0; c < Geo::kQK; ++c)
      *reinterpret_cast<u32x4*>(qh + qk_dim0<false>(c, g)) = __builtin_bit_cast(u32x4, qop[c]);
  }
  static __device__ __forceinline__ void stash_q(_Float16* s_q, const half8_t* qop, int g, int n16) {
    if (n16 >= C) return;
#pragma unroll
    for (int c = 0; c < Geo::kQK; ++c)
      *reinterpret_cast<u32x4*>(s_q + n16 * D + qk_dim0<false>(c, g)) = __builtin_bit_cast(u32x4, qop[c]);
  }
  static __device__ __forceinline__ void write_q_stashed(const DecodeArgs& a, int seg,
                                                         const _Float16* s_q, int g, int n16) {
    half8_t q[Geo::kQK];
#pragma unroll
    for (int c = 0; c < Geo::kQK; ++c)
      q[c] = __builtin_bit_cast(half8_t, *reinterpret_cast<const u32x4*>(s_q + min(n16, C - 1) * D +
                                                                         qk_dim0<false>(c, g)));
    write_q(a, seg, q, g, n16);
  }

  // Count this piece's arrival at its segment (the partial must already be at
  // device scope); returns the previous count in lane 0.
  static __device__ __forceinline__ uint32_t arrive(const DecodeArgs& a, int seg) {
    uint32_t prev = 0;
    if ((threadIdx.x & (kWave - 1)) == 0)
      prev = __hip_atomic_fetch_add(a.counters + seg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return prev;
  }

  // Vector memory loads that issue() enqueues for one tile.
  static constexpr int kTileLoads = Geo::kKLoads + 4;

  // Float4 pieces of one partial (C rows of D) and how many each lane owns.
  static constexpr int kF4 = C * D / 4;
  static constexpr int kOwn = (kF4 + kWave - 1) / kWave;

  // Buffer over the C partial rows of output row0 (all partitions).
  static __device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rows(const DecodeArgs& a,
                                                                        size_t row0) {
    const size_t stride = size_t(a.max_partitions) * D;
    return make_rsrc(a.part_out + row0 * stride, int(C * stride * sizeof(float)));
  }
  static __device__ __forceinline__ int partial_offset(const DecodeArgs& a, int c, int j) {
    return int(((4 * c / D) * size_t(a.max_partitions) * D + size_t(j) * D + 4 * c % D) *
               sizeof(float));
  }

  // A piece's partial, kept in LDS until it is written out: o / l of the C
  // rows (C * D floats), then the C maxima (natural-log units) and C sums.
  static constexpr int kStage = C * D + 2 * C;

  static __device__ __forceinline__ void stage_partial(const MState<D, FP8>& st, float l, int g,
                                                       int n16, float* s_o) {
    if (n16 >= C) return;
    // a causal column can see no token of a piece (l = 0): its o is 0 and
    // its weight in the combine exp(m - M) l is 0
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < Geo::kPV; ++i) s_o[n16 * D + (4 * g + r) * Geo::kPV + i] = st.acc[i][r] * inv;
    if (g == 0) {
      s_o[C * D + n16] = st.m * kLn2;
      s_o[C * D + C + n16] = l;
    }
  }

  // Piece j of the segment at output row row0, from its LDS copy: each lane
  // writes whole 16-byte pieces of the rows.  With QK-norm a wave of the
  // same launch combines them, so the stores are device-scope coherent; the
  // combine launch reads them after the launch boundary, so plain stores do.
  static __device__ __forceinline__ void write_partial(const DecodeArgs& a, size_t row0, int j,
                                                       const float* s_o) {
    const int lane = threadIdx.x & (kWave - 1);
    const __amdgpu_buffer_rsrc_t rs = partial_rows(a, row0);
#pragma unroll
    for (int k = 0; k < kOwn; ++k) {
      const int c = lane + k * kWave;
      if (c < kF4)
        store16<QKNORM>(rs, partial_offset(a, c, j), *reinterpret_cast<const u32x4*>(s_o + 4 * c));
    }
    if (lane < C) {
      const size_t pr = (row0 + lane) * a.max_partitions + j;
      store_f32<QKNORM>(a.part_max + pr, s_o[C * D + lane]);
      store_f32<QKNORM>(a.part_sum + pr, s_o[C * D + C + lane]);
    }
  }

  // Log-sum-exp combine of the `pieces` partials of segment seg's C columns
  // by the last piece to arrive (QK-norm modes; one wave, weights staged in
  // LDS), which then clears the counter.  A lane owns float4 pieces of the C
  // rows.
  // The loads of the statistics and of the first batch of partial rows all
  // go out together (one round trip when pieces <= kBatch); a wave that
  // finishes two segments issues both segments' loads before computing
  // either.
  static constexpr int kBatch = kOwn >= 16 ? 1 : 16 / kOwn;
  static constexpr int kStat = (C * kMaxStepPartitions + kWave - 1) / kWave;
  struct CombineLoads {
    float mv[kStat], lv[kStat];
    u32x4 v[kBatch][kOwn];
  };

  static __device__ __forceinline__ void load_batch(const DecodeArgs& a, __amdgpu_buffer_rsrc_t rs,
                                                    int pieces, int p0, u32x4 (*v)[kOwn]) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
#pragma unroll
      for (int k = 0; k < kOwn; ++k) {
        const int c = lane + k * kWave;
        v[q][k] = p0 + q < pieces && c < kF4 ? load16_coherent(rs, partial_offset(a, c, p0 + q))
                                             : u32x4{0u, 0u, 0u, 0u};
      }
  }

  static __device__ __forceinline__ void combine_issue(const DecodeArgs& a, int seg, int pieces,
                                                       CombineLoads& ld) {
    const int lane = threadIdx.x & (kWave - 1);
    const size_t row0 = seg_row0(a, seg);  // the segment's partial rows
#pragma unroll
    for (int i = 0; i < kStat; ++i) {
      const int t = lane + i * kWave;
      ld.mv[i] = ld.lv[i] = 0.0f;
      if (t < C * pieces) {
        const size_t pr = (row0 + t / pieces) * a.max_partitions + t % pieces;
        ld.mv[i] = load_f32_coherent(a.part_max + pr);
        ld.lv[i] = load_f32_coherent(a.part_sum + pr);
      }
    }
    load_batch(a, partial_rows(a, row0), pieces, 0, ld.v);
  }

  static __device__ __forceinline__ void combine_finish(const DecodeArgs& a, int seg, int pieces,
                                                        CombineLoads& ld, float* s_w) {
    const int lane = threadIdx.x & (kWave - 1);
    const __amdgpu_buffer_rsrc_t rs = partial_rows(a, seg_row0(a, seg));
#pragma unroll
    for (int i = 0; i < kStat; ++i) {
      const int t = lane + i * kWave;
      if (t < C * pieces) {
        const int j = t / pieces, p = t % pieces;
        s_w[2 * (j * kMaxStepPartitions + p)] = ld.mv[i];
        s_w[2 * (j * kMaxStepPartitions + p) + 1] = ld.lv[i];
      }
    }
    for (int j = lane; j < C; j += kWave) {
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
    float4_t num[kOwn];
#pragma unroll
    for (int k = 0; k < kOwn; ++k) num[k] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int p0 = 0; p0 < pieces; p0 += kBatch) {
      if (p0 > 0) load_batch(a, rs, pieces, p0, ld.v);
#pragma unroll
      for (int q = 0; q < kBatch; ++q)
#pragma unroll
        for (int k = 0; k < kOwn; ++k) {
          const int c = lane + k * kWave;
          if (p0 + q < pieces && c < kF4) {
            const float wgt = s_w[2 * ((4 * c / D) * kMaxStepPartitions + p0 + q) + 1];
            num[k] += wgt * __builtin_bit_cast(float4_t, ld.v[q][k]);
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
        *reinterpret_cast<half4_t*>(static_cast<_Float16*>(a.out) + seg_qrow(a, seg, h) * D +
                                    4 * c % D) = o;
      }
    }
    if (lane == 0) __hip_atomic_store(a.counters + seg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  static __device__ __forceinline__ void finish(const DecodeArgs& a, int seg, int pieces, float* s_w) {
    CombineLoads ld;
    combine_issue(a, seg, pieces, ld);
    combine_finish(a, seg, pieces, ld, s_w);
  }

  // The combine launch's form: every lane keeps a running log-sum-exp of
  // the float4 pieces it owns in registers (the statistics of its own heads
  // loaded next to the partial rows, no LDS, no cross-lane step), kOW pieces
  // per lane and kRW waves per segment.  One wave covers a segment of up to
  // 128 float4s (C * D <= 512); larger segments take one wave per 64 float4s
  // (e.g. 8 heads of 128: four waves), which measured faster than fewer
  // waves with more pieces per lane.
  static constexpr int kOW = kOwn >= 4 ? 1 : kOwn;
  static constexpr int kRW = kOwn / kOW;
  static constexpr int kRB = 16 / kOW;  // partitions per round trip

  static __device__ __forceinline__ void combine_rows(const DecodeArgs& a, int seg, int pieces, int part) {
    const int lane = threadIdx.x & (kWave - 1);
    const size_t row0 = seg_row0(a, seg);
    const int P = a.max_partitions;
    const __amdgpu_buffer_rsrc_t rs = partial_rows(a, row0);
    float M[kOW], den[kOW];
    float4_t num[kOW];
#pragma unroll
    for (int k = 0; k < kOW; ++k) {
      M[k] = -FLT_MAX;
      den[k] = 0.0f;
      num[k] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    for (int p0 = 0; p0 < pieces; p0 += kRB) {
      float mv[kOW][kRB], lv[kOW][kRB];
      u32x4 v[kOW][kRB];
#pragma unroll
      for (int k = 0; k < kOW; ++k) {
        const int c = (part * kOW + k) * kWave + lane;
        const int h = c < kF4 ? 4 * c / D : 0;
        const float* pm = a.part_max + (row0 + h) * P;
        const float* pl = a.part_sum + (row0 + h) * P;
#pragma unroll
        for (int q = 0; q < kRB; ++q) {
          const bool ok = p0 + q < pieces && c < kF4;
          mv[k][q] = ok ? pm[p0 + q] : -FLT_MAX;
          lv[k][q] = ok ? pl[p0 + q] : 0.0f;
          v[k][q] = ok ? buffer_load16(rs, partial_offset(a, c, p0 + q)) : u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int k = 0; k < kOW; ++k) {
        float Mn = M[k];
#pragma unroll
        for (int q = 0; q < kRB; ++q) Mn = fmaxf(Mn, mv[k][q]);
        const float r = fast_exp2((M[k] - Mn) * kLog2e);
        den[k] *= r;
        num[k] *= r;
#pragma unroll
        for (int q = 0; q < kRB; ++q) {
          const float w = lv[k][q] * fast_exp2((mv[k][q] - Mn) * kLog2e);
          den[k] += w;
          num[k] += w * __builtin_bit_cast(float4_t, v[k][q]);
        }
        M[k] = Mn;
      }
    }
#pragma unroll
    for (int k = 0; k < kOW; ++k) {
      const int c = (part * kOW + k) * kWave + lane;
      if (c < kF4) {
        half4_t o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (_Float16)(num[k][e] / den[k]);
        *reinterpret_cast<half4_t*>(static_cast<_Float16*>(a.out) + seg_qrow(a, seg, 4 * c / D) * D +
                                    4 * c % D) = o;
      }
    }
  }

  // Two segments finished by the same wave: one round trip for both.
  static __device__ __forceinline__ void finish2(const DecodeArgs& a, int seg0, int pieces0, int seg1,
                                                 int pieces1, float* s_w0, float* s_w1) {
    CombineLoads l0, l1;
    combine_issue(a, seg0, pieces0, l0);
    combine_issue(a, seg1, pieces1, l1);
    combine_finish(a, seg0, pieces0, l0, s_w0);
    combine_finish(a, seg1, pieces1, l1, s_w1);
  }
};

template <int D, int C, bool FP8, int MODE, bool EXT, bool CACHED>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(stream_waves_per_eu<FP8>(), 8)))
void decode_stream_kernel(const int32_t* __restrict__ lens, int B, int workers, DecodeArgs a) {
  using K = StreamKernel<D, C, FP8, MODE, EXT, CACHED>;
  // without QK-norm the pieces of split segments are combined by a second
  // launch (stream_combine_kernel); with it, by the piece that arrives last
  // (it also writes q' back, which no other wave may do before every piece
  // of the segment has read q)
  constexpr bool TWO = !K::QKNORM;
  const int win = K::W(a);
  using Geo = MfmaGeo<D, FP8>;
  static_assert(C <= 16, "head slots of one 16-wide product");
  const int lane = threadIdx.x;
  const int worker = blockIdx.x;
  const int g = lane / 16;
  const int n16 = lane % 16;
  const int k_off = n16 * Geo::kRow + g * 16;
  const int v_off = (4 * g) * Geo::kRow + n16 * Geo::kVBytes;

  __shared__ float s_w[2 * C * kMaxStepPartitions];  // combine weights
  __shared__ float s_w2[2 * C * kMaxStepPartitions];  // a second segment's
  __shared__ float s_fin[K::kStage];                  // the range's last piece
  __shared__ float s_pend[K::kStage];                 // a piece that ended earlier
  // rotation angles of the positions of up to kDepth segments (QK-norm
  // modes): a segment's table is written when its first tile is issued and
  // read when that tile is computed, and at most kDepth - 1 tiles are issued
  // in between, so kDepth tables taken in turn never overwrite one in use
  // (one table per new token of the segment: nq <= C / g tokens)
  __shared__ float s_cos[K::QKNORM ? K::kDepth * C * (D / 2) : 1];
  __shared__ float s_sin[K::QKNORM ? K::kDepth * C * (D / 2) : 1];
  __shared__ _Float16 s_q[K::QKNORM ? C * D : 1];
  __shared__ double s_f[K::QKNORM ? D / 2 : 1];      // rotation frequencies
  __shared__ float s_gq[K::QKNORM ? D : 1];          // RMSNorm weights of q and k
  __shared__ float s_gk[K::QKNORM ? D : 1];

  // lens (= a.context_lens), B and workers lead the argument list, so that
  // the build preloads them into SGPRs at dispatch and the lengths load goes
  // out before any load of the argument block
  const int L0 = lane < B ? lens[lane] : 0;
  const Totals tot = total_tiles(a, B, L0, win, K::CG(a));
  const int64_t W = tot.tiles;
  // equal shares, but long enough that no sequence's segment is cut into more
  // than max_partitions pieces: T tiles span at most (T-1)/tpw + 2 ranges
  const Ranges rg = make_ranges<FP8>(W, tot.max_tiles, workers, a.max_partitions);
  const int64_t rw = range_of_worker(worker, workers);  // this wave's range
  const int64_t t0 = min(rg.start(rw), W);
  const int64_t t1 = min(W, rg.start(rw + 1));

  if (t0 < t1) {
    Cursor cur = locate(a, B, t0, tot.per_head, L0, tot.incl0, win, K::CG(a));
    int rope_b[K::kDepth];  // sequence whose angles are in each table
#pragma unroll
    for (int i = 0; i < K::kDepth; ++i) rope_b[i] = -1;
    int ord = 0;  // segments entered so far; picks the table in turn
    if constexpr (K::QKNORM) {
      rope_freqs<D>(s_f, a.theta);
      for (int i = lane; i < D; i += kWave) {
        s_gq[i] = a.gamma_q[i];
        s_gk[i] = a.gamma_k[i];
      }
    }
    if constexpr (K::APPEND)
      K::append_rows(a, B, cur, t0, t1, g, n16, k_off, v_off, s_cos, s_sin, s_f, s_gk);
    auto prepare_segment = [&](Meta& m) {
      m.slot = ord++ % K::kDepth;
      if constexpr (K::QKNORM) {
        if (m.b != rope_b[m.slot]) {
          // token j of the nq new ones sits at position L - nq + j
          for (int j = 0; j < K::NQ(a); ++j)
            rope_angles<D>(s_f, s_cos + (m.slot * C + j) * (D / 2), s_sin + (m.slot * C + j) * (D / 2),
                           m.L - K::NQ(a) + j);
          rope_b[m.slot] = m.b;
        }
      }
    };

    MState<D, FP8> st;
    K::reset(st);

    // NB tile buffers: while tile t is computed, tiles t+1 .. t+NB-1 are in
    // flight.  Metas run one tile further ahead (`ahead`), so each block id
    // has a whole step to arrive.
    constexpr int NB = K::kDepth;
    MTile<D, FP8> tl[NB];
    Meta mt[NB];
    Meta ahead;
    Meta mfin;          // the range's last tile
    int last_slot = 0;  // angle table of the most recently issued tile
    // q of the segment of the tile being computed (qop), and of the segments
    // that start at the tiles in flight: a tile that starts a segment loads
    // its q into the buffer of its own slot, just before its K and V, and the
    // buffer moves into qop when the tile is computed.
    half8_t qop[Geo::kQK];
    half8_t qbuf[NB][Geo::kQK];
    auto take = [&](Meta& m, half8_t* qdst) {
      if (m.first) {
        prepare_segment(m);
        K::load_q(qdst, a, m.b, m.kvh, m.cg, g, n16);
      } else {
        m.slot = last_slot;
      }
      last_slot = m.slot;
    };
    mt[0] = meta_of(cur, a, t0, t0, t1, win, K::BST(a), K::BSS(a));
    mt[0].first = true;  // the range starts with a piece of a segment
    take(mt[0], qbuf[0]);
    K::issue(tl[0], a, mt[0], true, k_off, v_off);
#pragma unroll
    for (int k = 1; k < NB; ++k) {
      const bool live = t0 + k < t1;
      if (live) {
        advance(cur, a, B, win, K::CG(a));
        Meta m = meta_of(cur, a, t0 + k, t0, t1, win, K::BST(a), K::BSS(a));
        if (k < NB - 1) {
          mt[k] = m;
          take(mt[k], qbuf[k]);
        } else {
          ahead = m;
        }
      }
      if (k < NB - 1) K::issue(tl[k], a, mt[k], live, k_off, v_off);
    }

    // A shared segment whose piece ends before the range does (only the
    // range's first segment can: it is that segment's last piece) is parked
    // in LDS.  Without QK-norm it is written out when the range ends.  With
    // QK-norm it publishes its partial right away and arrives one loop step
    // later, so that the segment's combine falls to one of the waves whose
    // ranges end with its other pieces, and no wave has two combines to do
    // when its range ends: the partial's stores go out behind the next
    // tile's loads; one step later a counted wait that leaves the newest
    // tile's loads in flight (vector memory operations complete in issue
    // order) makes sure they have completed before the arrival, whose
    // result is read when the range is done.
    int pend = 0;  // 0 none, 1 partial written, 2 arrived (prev count in pprev)
    int pseg = 0, ppieces = 0, pj = 0;
    uint32_t pprev = 0;

    // compute tile t (X, meta mx, q buffer qx); load tile t+NB-1 into Y
    // (meta my, q buffer qy)
    auto step = [&](MTile<D, FP8>& x, const Meta& mx, const half8_t* qx, MTile<D, FP8>& y, Meta& my,
                    half8_t* qy, int64_t t) {
      const bool live = t + NB - 1 < t1;
      if (live) {
        my = ahead;
        take(my, qy);
      }
      K::issue(y, a, my, live, k_off, v_off);
      if (t + NB < t1) {
        advance(cur, a, B, win, K::CG(a));
        ahead = meta_of(cur, a, t + NB, t0, t1, win, K::BST(a), K::BSS(a));
      }
      issue_fence();  // Y's loads stay ahead of the waits below
      if (mx.first) {
#pragma unroll
        for (int c = 0; c < Geo::kQK; ++c) qop[c] = qx[c];
        if constexpr (K::QKNORM)
        {
          // the lane's column belongs to new token (column / g)
          const int tq = min(n16, C - 1) / K::GRP(a);
          norm_rope_chunks<D>(qop, s_gq, a.eps, s_cos + (mx.slot * C + tq) * (D / 2),
                              s_sin + (mx.slot * C + tq) * (D / 2), g);
        }
      }
      issue_fence();
      // causal limit of this lane's column: new token j sees positions up to
      // L - nq + j (rows of tile f + n at or past the limit are masked)
      const int jcol = EXT ? (mx.cg * C + min(n16, C - 1)) / K::GRP(a) : 0;
      const int col_hi = EXT ? mx.L - K::NQ(a) + 1 + jcol - 16 * (mx.f + mx.n) : 16;
      mfma_tile<D, FP8>(st, x, qop, a.scale_log2, g, col_hi);
      if (t + 1 >= t1) {
        mfin = mx;
        return;
      }
      if (mx.last) {
        // the segment ends inside the range: its last range is this one
        const int64_t r_first = K::first_range(mx, rg, rw, t0);
        const int pieces = int(rw - r_first + 1);
        const int seg = K::seg_id(a, mx.b, mx.kvh, mx.cg);
        const float l = group4_sum(st.l);
        if (pieces == 1) {
          K::store_direct(st, l, a, seg, g, n16);
          if constexpr (K::QKNORM) K::write_q(a, seg, qop, g, n16);
        } else {
          K::stage_partial(st, l, g, n16, s_pend);
          if constexpr (K::QKNORM) K::stash_q(s_q, qop, g, n16);
          pseg = seg;
          ppieces = pieces;
          pj = int(rw - r_first);
          if constexpr (!TWO) K::write_partial(a, K::seg_row0(a, pseg), pj, s_pend);
          pend = 1;
          K::reset(st);
          return;
        }
        K::reset(st);
      }
      if (!TWO && pend == 1) {
        // the partial's stores were issued before this step's tile loads;
        // everything but the newest NB - 1 tiles' loads has completed
        issue_fence();
        __builtin_amdgcn_s_waitcnt(vmcnt_at_most((NB - 1) * K::kTileLoads));
        issue_fence();
        pprev = K::arrive(a, pseg);
        pend = 2;
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

    // the range's last piece
    const Meta& mf = mfin;
    const int64_t f_first = K::first_range(mf, rg, rw, t0);
    const int fpieces = int(K::last_range(mf, rg, rw, t1) - f_first + 1);
    const int fseg = K::seg_id(a, mf.b, mf.kvh, mf.cg);
    const float l = group4_sum(st.l);
    if (fpieces == 1) {
      K::store_direct(st, l, a, fseg, g, n16);
      if constexpr (K::QKNORM) K::write_q(a, fseg, qop, g, n16);
    } else {
      K::stage_partial(st, l, g, n16, s_fin);
      K::write_partial(a, K::seg_row0(a, fseg), int(rw - f_first), s_fin);
    }
    if constexpr (TWO) {
      // the parked piece goes out now; a split segment's first piece tells
      // the combine launch how many pieces to combine
      if (pend == 1) K::write_partial(a, K::seg_row0(a, pseg), pj, s_pend);
      if (fpieces > 1 && f_first == rw && lane == 0) a.counters[fseg] = uint32_t(fpieces);
    } else {
    uint32_t fprev = 0;
    if (pend == 1 || fpieces > 1) {
      __builtin_amdgcn_s_waitcnt(0);  // partials at device scope
      if (pend == 1) {
        pprev = K::arrive(a, pseg);
        pend = 2;
      }
      if (fpieces > 1) fprev = K::arrive(a, fseg);
    }
    // the last arrival of a segment combines it; the early piece is rarely
    // the last (its segment's other pieces end with their ranges)
    const bool pfin = pend == 2 && __builtin_amdgcn_readfirstlane(pprev) == uint32_t(ppieces - 1);
    const bool ffin = fpieces > 1 && __builtin_amdgcn_readfirstlane(fprev) == uint32_t(fpieces - 1);
    if (pfin && ffin) {
      K::finish2(a, pseg, ppieces, fseg, fpieces, s_w, s_w2);
    } else if (pfin) {
      K::finish(a, pseg, ppieces, s_w);
    } else if (ffin) {
      K::finish(a, fseg, fpieces, s_w);
    }
    if constexpr (K::QKNORM) {
      if (pfin) K::write_q_stashed(a, pseg, s_q, g, n16);
      if (ffin) K::write_q(a, fseg, qop, g, n16);
    }
    }
  }

  // sequences with no tokens: zero output rows, one wave each
  for (int b = worker; b < B; b += workers)
    if (load_uniform(a.context_lens + b) == 0)
      for (int i = lane; i < K::NQ(a) * a.Hq * D; i += kWave)
        static_cast<_Float16*>(a.out)[size_t(b) * K::NQ(a) * a.Hq * D + i] = (_Float16)0.0f;
}

// The combine launch of the balanced step (modes without QK-norm): workgroup
// seg (a grid-stride loop beyond the grid), kRW waves, combines the pieces
// segment seg's counter holds and clears it; 0 = a segment that one wave
// finished.  Partials and counts were written by the attend launch, so plain
// loads see them.
template <int D, int C, bool FP8, bool EXT>
__global__ __launch_bounds__((kWave * StreamKernel<D, C, FP8, kModeCombine, EXT, false>::kRW))
void stream_combine_kernel(uint32_t* __restrict__ counters, int nseg, DecodeArgs a) {
  using K = StreamKernel<D, C, FP8, kModeCombine, EXT, false>;
  const int part = int(threadIdx.x / kWave);  // this wave's share of the segment
  for (int seg = blockIdx.x; seg < nseg; seg += gridDim.x) {
    const int pieces = __builtin_amdgcn_readfirstlane(int(counters[seg]));
    if (pieces > 0) K::combine_rows(a, seg, pieces, part);
    // every wave of the workgroup has read the count before it is cleared
    if constexpr (K::kRW > 1) __syncthreads();
    if (pieces > 0 && threadIdx.x == 0) counters[seg] = 0u;
  }
}

// Workgroup shape of the combine launch.
template <int D, int C, bool FP8, bool EXT>
dim3 combine_block() {
  return dim3(kWave * StreamKernel<D, C, FP8, kModeCombine, EXT, false>::kRW);
}

// Compute units of the current device (queried once per device).
int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] <= 0) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                       n > 0
                   ? n
                   : 256;
  }
  return cus[dev];
}

template <int D, int C, bool FP8, int MODE, bool CACHED>
hipError_t launch_stream(const DecodeArgs& a, int B, hipStream_t stream) {
  const int workers = device_cus() * 4 * stream_waves_per_eu<FP8>();
  const bool ext = a.window > 0 || a.nq > 1 || a.bs_tiles > 1;
  if (ext)
    hipLaunchKernelGGL((decode_stream_kernel<D, C, FP8, MODE, true, CACHED>), dim3(workers),
                       dim3(kWave), 0, stream, a.context_lens, B, workers, a);
  else
    hipLaunchKernelGGL((decode_stream_kernel<D, C, FP8, MODE, false, CACHED>), dim3(workers),
                       dim3(kWave), 0, stream, a.context_lens, B, workers, a);
  if constexpr ((MODE & kModeQkNorm) != 0) return hipGetLastError();
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nseg = B * a.Hkv * (ext ? a.cgroups : 1);
  if (ext)
    hipLaunchKernelGGL((stream_combine_kernel<D, C, FP8, true>), dim3(min(nseg, 2 * workers)),
                       (combine_block<D, C, FP8, true>()),
                       0, stream, a.counters, nseg, a);
  else
    hipLaunchKernelGGL((stream_combine_kernel<D, C, FP8, false>), dim3(min(nseg, 2 * workers)),
                       (combine_block<D, C, FP8, false>()),
                       0, stream, a.counters, nseg, a);
  return hipGetLastError();
}

template <int D, int C, bool FP8, bool CACHED>
hipError_t launch_stream_mode(const DecodeArgs& a, int B, int mode, hipStream_t stream) {
  if constexpr (FP8) {
    if (mode == kModeCombine) return launch_stream<D, C, true, kModeCombine, CACHED>(a, B, stream);
    return hipErrorInvalidValue;
  } else {
    switch (mode) {
      case kModeCombine: return launch_stream<D, C, false, kModeCombine, CACHED>(a, B, stream);
      case kModeAppend | kModeCombine:
        return launch_stream<D, C, false, kModeAppend | kModeCombine, CACHED>(a, B, stream);
      case kModeAppend | kModeQkNorm | kModeCombine:
        // QK-norm runs with at most 8 query columns (g * nq): one rotation
        // table per new token and pipeline slot in LDS
        if constexpr (C <= 8)
          return launch_stream<D, C, false, kModeAppend | kModeQkNorm | kModeCombine, CACHED>(
              a, B, stream);
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
  }
}

template <int D, bool FP8, bool CACHED>
hipError_t launch_stream_cols(const DecodeArgs& a, int B, int cols, int mode, hipStream_t stream) {
  switch (cols) {
    case 1: return launch_stream_mode<D, 1, FP8, CACHED>(a, B, mode, stream);
    case 2: return launch_stream_mode<D, 2, FP8, CACHED>(a, B, mode, stream);
    case 4: return launch_stream_mode<D, 4, FP8, CACHED>(a, B, mode, stream);
    case 8: return launch_stream_mode<D, 8, FP8, CACHED>(a, B, mode, stream);
    case 16: return launch_stream_mode<D, 16, FP8, CACHED>(a, B, mode, stream);
    default: return hipErrorInvalidValue;
  }
}

// The balanced step with cache policy CACHED for the KV loads.
template <bool CACHED>
hipError_t launch_stream_policy(const DecodeArgs& a, int B, int D, int cols, bool fp8, int mode,
                                hipStream_t stream) {
  if (D == 128) return fp8 ? launch_stream_cols<128, true, CACHED>(a, B, cols, mode, stream)
                           : launch_stream_cols<128, false, CACHED>(a, B, cols, mode, stream);
  if (D == 64) return fp8 ? launch_stream_cols<64, true, CACHED>(a, B, cols, mode, stream)
                          : launch_stream_cols<64, false, CACHED>(a, B, cols, mode, stream);
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace pkv
