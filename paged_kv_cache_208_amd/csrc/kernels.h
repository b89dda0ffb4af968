// Kernel argument blocks and launchers shared by the C-ABI layer (api.hip)
// and the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace pkv {

struct DecodeArgs {
  void* out;                  // [B][Hq][D] fp16: single pass, or combined in the step kernel
  const void* q;              // [B][Hq][D] fp16 (step kernel with QK-norm: rewritten in place)
  const uint8_t* k_pool;      // [NB][Hkv][16][D] fp16 or E4M3 (step kernel: the new row is written)
  const uint8_t* v_pool;
  const float* k_scale;       // [NB][Hkv], E4M3 only
  const float* v_scale;
  const int32_t* block_tables;  // [B][MBS]
  const int32_t* context_lens;  // [B]
  float* part_out;            // [B][Hq][P][D]
  float* part_max;            // [B][Hq][P]
  float* part_sum;            // [B][Hq][P]
  int Hq, Hkv, MBS;
  int partition_size;         // 0 = single pass
  int max_partitions;         // P (partitioned) or 1
  float scale_log2;           // softmax scale * log2(e)
  // decode step only
  const void* k_new;          // [B][Hkv][D] fp16: row of token L_b - 1
  const void* v_new;
  const float* gamma_q;       // [D] (QK-norm)
  const float* gamma_k;
  float eps, theta;
  uint32_t* counters;         // [B][Hkv * CG] piece counts or arrivals per segment; zero between steps
  int window;                 // > 0: attend to the last `window` tokens only (balanced step)
  int nq;                     // new query tokens per sequence (balanced step; 1 otherwise)
  int ncols;                  // query columns per (sequence, kv head): group * nq
  int cgroups;                // 16-column groups they are split into (1 when ncols <= 16)
  int prefix_tiles;           // > 0: every table starts with these shared 16-token tiles
  int group;                  // Hq / Hkv
  int bs_tiles;               // 16-token tiles per block: 1, or 2 for 32-token blocks
  int bs_shift;               // log2(bs_tiles)
  int cached_kv;              // nonzero: KV tiles with the default cache policy (shared blocks)
};

// What a decode launch does besides attending (bit flags).
enum DecodeMode : int {
  kModeAttend = 0,
  kModeAppend = 1,    // write each sequence's new K/V row before reading it
  kModeQkNorm = 2,    // Qwen3 QK-RMSNorm + split-half RoPE of q and the new k
  kModeCombine = 4,   // the last workgroup of each (sequence, kv head) combines partitions
};

struct ReduceArgs {
  void* out;                  // [B][Hq][D] fp16
  const float* part_out;
  const float* part_max;
  const float* part_sum;
  const int32_t* context_lens;
  int Hq, D, partition_size, max_partitions;
};

struct AppendArgs {
  const void* k_new;          // [T][Hkv][D] fp16
  const void* v_new;
  void* k_pool;               // [NB][Hkv][16][D] fp16
  void* v_pool;
  const int64_t* slot_mapping;  // [T]
  void* q;                    // [T][Hq][D] fp16, fused only (in place)
  const float* gamma_q;       // [D], fused only
  const float* gamma_k;
  const int32_t* context_lens;  // [T], fused only
  int Hq, Hkv;
  float eps, theta;
  int bs;                     // tokens per block (16 or 32)
};

struct AppendE4m3Args {
  const void* k_new;          // [T][Hkv][D] fp16
  const void* v_new;
  uint8_t* k_pool;            // [NB][Hkv][16][D] E4M3 codes
  uint8_t* v_pool;
  float* k_scale;             // [NB][Hkv]
  float* v_scale;
  const int64_t* slot_mapping;  // [T]; NULL: token t is sequence t's last one (below)
  int Hkv;
  int bs;                     // tokens per block (16 or 32)
  // without slot_mapping: token t goes to position context_lens[t] - 1 of
  // sequence t (block_tables [T][MBS]); sequences with no tokens are skipped
  const int32_t* block_tables;
  const int32_t* context_lens;
  int MBS;
};

struct CopyArgs {
  uint8_t* k_pool;            // [NB][Hkv][16][D] elements of elem_bytes
  uint8_t* v_pool;
  float* k_scale;             // [NB][Hkv], E4M3 only (else null)
  float* v_scale;
  const int32_t* src;         // [n]
  const int32_t* dst;
  int64_t block_bytes;        // Hkv * 16 * D * elem_bytes (a multiple of 16)
  int Hkv;
};

// Launchers return the hipError_t of the launch.
hipError_t launch_decode(const DecodeArgs& a, int B, int D, int group, bool fp8,
                         hipStream_t stream);
hipError_t launch_decode_step(const DecodeArgs& a, int B, int D, int group, bool fp8, int mode,
                              hipStream_t stream);
// cols = (Hq / Hkv) * nq, the used columns of the 16-wide products (1..16)
hipError_t launch_decode_stream(const DecodeArgs& a, int B, int D, int cols, bool fp8, int mode,
                                hipStream_t stream);
// tables that all start with a.prefix_tiles shared tiles (cols = Hq / Hkv)
hipError_t launch_decode_prefix(const DecodeArgs& a, int B, int D, int cols, bool fp8, int mode,
                                hipStream_t stream);
// the same with the default cache policy for the KV tiles (shared-blocks hint)
hipError_t launch_decode_stream_cached(const DecodeArgs& a, int B, int D, int cols, bool fp8,
                                       int mode, hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs& a, int B, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, int T, int D, bool fused, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyArgs& a, int n, hipStream_t stream);
hipError_t launch_append_e4m3(const AppendE4m3Args& a, int T, int D, hipStream_t stream);

}  // namespace pkv
