// C-ABI entry points of libpagedkv.so (declared and documented in
// include/pagedkv.h): validate on the host, then enqueue the kernels.
#include "pagedkv.h"
#include "kernels.h"
#include "read_probe.h"
#include "device.h"
#include "shape_limits.h"

#include <mutex>


namespace {

int launch_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ELAUNCH; }

// ---------------------------------------------------------------------------
// Static scratch of paged_decode_step_static: the step's counters (first
// kScratchCounterBytes, zero between calls) and then the partials.  One copy
// per GPU, held until the process ends.  The host never uses the array's
// name as an address (in host code it is only a stand-in for the symbol):
// its device address is looked up once per device and kept.
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr size_t kScratchCounterBytes = size_t(1) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceScratch {
  std::once_flag addr_once, fill_once;
  unsigned char* ptr = nullptr;
  hipError_t addr_err = hipSuccess, fill_err = hipSuccess;
};
DeviceScratch g_scratch[kMaxDevices];

__global__ void fill_zero_u32(uint32_t* p, int n) {
  const int i = int(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) p[i] = 0u;
}

// This device's scratch: its device address, looked up once per device with
// the device current (nothing is enqueued).
int scratch_address(int* dev_out, unsigned char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKV_ELAUNCH;
  DeviceScratch& d = g_scratch[dev];
  std::call_once(d.addr_once, [&] {
    void* p = nullptr;
    d.addr_err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (d.addr_err == hipSuccess) d.ptr = static_cast<unsigned char*>(p);
  });
  if (d.addr_err != hipSuccess || d.ptr == nullptr) return PKV_ELAUNCH;
  *dev_out = dev;
  *out = d.ptr;
  return PKV_OK;
}

// The first call on a device zeroes the counters with a fill kernel on its
// stream (ahead of its own step kernel); every step leaves them at zero.
int scratch_fill_once(int dev, unsigned char* base, hipStream_t stream) {
  DeviceScratch& d = g_scratch[dev];
  std::call_once(d.fill_once, [&] {
    const int n = int(kScratchCounterBytes / sizeof(uint32_t));
    hipLaunchKernelGGL(fill_zero_u32, dim3((n + 255) / 256), dim3(256), 0, stream,
                       reinterpret_cast<uint32_t*>(base), n);
    d.fill_err = hipGetLastError();
  });
  return d.fill_err == hipSuccess ? PKV_OK : PKV_ELAUNCH;
}

}  // namespace

extern "C" int paged_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                               const int64_t* slot_mapping, int T, int Hkv, int D, int BS,
                               int64_t NB, void* q_inout, int Hq, const float* gamma_q,
                               const float* gamma_k, const int32_t* context_lens, float eps,
                               float rope_theta, void* stream) {
  const int st = pkv_validate_append(k_new, v_new, k_pool, v_pool, slot_mapping, T, Hkv, D, BS,
                                     NB, q_inout, Hq, gamma_q, gamma_k, context_lens, eps,
                                     rope_theta);
  if (st != PKV_OK || T == 0) return st;
  const bool fused = gamma_k != nullptr;
  pkv::AppendArgs a{k_new, v_new, k_pool, v_pool, slot_mapping,
                    fused ? q_inout : nullptr, fused ? gamma_q : nullptr, gamma_k,
                    fused ? context_lens : nullptr, fused ? Hq : 0, Hkv, eps, rope_theta, BS};
  return launch_status(pkv::launch_append(a, T, D, fused, static_cast<hipStream_t>(stream)));
}

extern "C" int paged_attn_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
                                 const float* k_scale, const float* v_scale,
                                 const int32_t* block_tables, const int32_t* context_lens, int B,
                                 int Hq, int Hkv, int D, int BS, int MBS, int64_t NB, float scale,
                                 int kv_dtype, int partition_size, float* part_out,
                                 float* part_max, float* part_sum, int max_partitions,
                                 void* stream) {
  const int st = pkv_validate_decode(out, q, k_pool, v_pool, k_scale, v_scale, block_tables,
                                     context_lens, B, Hq, Hkv, D, BS, MBS, NB, scale, kv_dtype,
                                     partition_size, part_out, part_max, part_sum,
                                     max_partitions);
  if (st != PKV_OK || B == 0) return st;
  const bool fp8 = (kv_dtype & ~PKV_KV_SHARED_BLOCKS) == PKV_KV_E4M3;
  pkv::DecodeArgs a{};
  a.cached_kv = (kv_dtype & PKV_KV_SHARED_BLOCKS) != 0;
  a.out = out;
  a.q = q;
  a.k_pool = static_cast<const uint8_t*>(k_pool);
  a.v_pool = static_cast<const uint8_t*>(v_pool);
  a.k_scale = fp8 ? k_scale : nullptr;
  a.v_scale = fp8 ? v_scale : nullptr;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.part_out = part_out;
  a.part_max = part_max;
  a.part_sum = part_sum;
  a.bs_tiles = 1;
  a.nq = 1;
  a.group = Hq / Hkv;
  a.ncols = a.group;
  a.cgroups = 1;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.MBS = MBS;
  a.partition_size = partition_size;
  a.max_partitions = partition_size ? max_partitions : 1;
  a.scale_log2 = scale * pkv::kLog2e;
  return launch_status(
      pkv::launch_decode(a, B, D, Hq / Hkv, fp8, static_cast<hipStream_t>(stream)));
}

extern "C" int paged_attn_reduce(void* out, const float* part_out, const float* part_max,
                                 const float* part_sum, const int32_t* context_lens, int B,
                                 int Hq, int D, int partition_size, int max_partitions,
                                 void* stream) {
  const int st = pkv_validate_reduce(out, part_out, part_max, part_sum, context_lens, B, Hq, D,
                                     partition_size, max_partitions);
  if (st != PKV_OK || B == 0) return st;
  pkv::ReduceArgs a{out, part_out, part_max, part_sum, context_lens,
                    Hq, D, partition_size, max_partitions};
  return launch_status(pkv::launch_reduce(a, B, static_cast<hipStream_t>(stream)));
}

extern "C" int paged_decode_step(void* out, void* q, const void* k_new, const void* v_new,
                                 void* k_pool, void* v_pool, float* k_scale,
                                 float* v_scale, const int32_t* block_tables,
                                 const int32_t* context_lens, int B, int Hq, int Hkv, int D,
                                 int BS, int MBS, int64_t NB, float scale, int kv_dtype,
                                 int partition_size, int window, int n_query,
                                 int prefix_blocks, const float* gamma_q, const float* gamma_k,
                                 float eps, float rope_theta, float* part_out, float* part_max,
                                 float* part_sum, uint32_t* counters, int max_partitions,
                                 void* stream) {
  const int st = pkv_validate_step(out, q, k_new, v_new, k_pool, v_pool, k_scale, v_scale,
                                   block_tables, context_lens, B, Hq, Hkv, D, BS, MBS, NB, scale,
                                   kv_dtype, partition_size, window, n_query, prefix_blocks,
                                   gamma_q, gamma_k, eps, rope_theta, part_out, part_max,
                                   part_sum, counters, max_partitions);
  if (st != PKV_OK || B == 0) return st;
  const bool fp8 = (kv_dtype & ~PKV_KV_SHARED_BLOCKS) == PKV_KV_E4M3;
  pkv::DecodeArgs a{};
  a.cached_kv = (kv_dtype & PKV_KV_SHARED_BLOCKS) != 0;
  a.out = out;
  a.q = q;
  a.k_pool = static_cast<const uint8_t*>(k_pool);
  a.v_pool = static_cast<const uint8_t*>(v_pool);
  a.k_scale = fp8 ? k_scale : nullptr;
  a.v_scale = fp8 ? v_scale : nullptr;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.part_out = part_out;
  a.part_max = part_max;
  a.part_sum = part_sum;
  a.window = window;
  a.bs_tiles = BS / pkv::kBlockSize;
  a.bs_shift = a.bs_tiles == 2 ? 1 : 0;
  a.nq = n_query;
  a.group = Hq / Hkv;
  a.ncols = a.group * n_query;
  a.cgroups = a.ncols > pkv::kColsPerProduct ? a.ncols / pkv::kColsPerProduct : 1;
  a.prefix_tiles = prefix_blocks * a.bs_tiles;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.MBS = MBS;
  a.partition_size = partition_size;
  a.max_partitions = max_partitions;
  a.scale_log2 = scale * pkv::kLog2e;
  a.k_new = k_new;
  a.v_new = v_new;
  a.gamma_q = gamma_q;
  a.gamma_k = gamma_k;
  a.eps = eps;
  a.theta = rope_theta;
  a.counters = counters;
  int mode = pkv::kModeCombine;
  if (k_new && fp8) {
    // E4M3: the new rows (and their blocks' scales) are written by the E4M3
    // append first; the attention then reads them from the pools
    pkv::AppendE4m3Args ap{k_new, v_new, static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool),
                           k_scale, v_scale, nullptr, Hkv, BS,
                           block_tables, context_lens, MBS};
    const int sa = launch_status(pkv::launch_append_e4m3(ap, B, D, static_cast<hipStream_t>(stream)));
    if (sa != PKV_OK) return sa;
    a.k_new = a.v_new = nullptr;
  } else if (k_new) {
    mode |= pkv::kModeAppend;
  }
  if (gamma_k) mode |= pkv::kModeQkNorm;
  if (prefix_blocks > 0)  // balanced split, shared prefix read once per group of sequences
    return launch_status(pkv::launch_decode_prefix(a, B, D, a.ncols, fp8, mode,
                                                   static_cast<hipStream_t>(stream)));
  if (partition_size == 0)  // balanced split across a fixed number of waves
    return launch_status(pkv::launch_decode_stream(a, B, D, a.cgroups > 1 ? pkv::kColsPerProduct : a.ncols,
                                                   fp8, mode, static_cast<hipStream_t>(stream)));
  return launch_status(pkv::launch_decode_step(a, B, D, Hq / Hkv, fp8, mode,
                                               static_cast<hipStream_t>(stream)));
}

extern "C" int paged_kv_copy_blocks(void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                    const int32_t* src, const int32_t* dst, int n, int Hkv,
                                    int D, int BS, int64_t NB, int kv_dtype, void* stream) {
  const int st =
      pkv_validate_copy(k_pool, v_pool, k_scale, v_scale, src, dst, n, Hkv, D, BS, NB, kv_dtype);
  if (st != PKV_OK || n == 0) return st;
  const bool fp8 = kv_dtype == PKV_KV_E4M3;
  pkv::CopyArgs a{static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool),
                  fp8 ? k_scale : nullptr, fp8 ? v_scale : nullptr, src, dst,
                  int64_t(Hkv) * BS * D * (fp8 ? 1 : 2), Hkv};
  return launch_status(pkv::launch_copy_blocks(a, n, static_cast<hipStream_t>(stream)));
}

extern "C" int paged_kv_append_e4m3(const void* k_new, const void* v_new, void* k_pool,
                                    void* v_pool, float* k_scale, float* v_scale,
                                    const int64_t* slot_mapping, int T, int Hkv, int D, int BS,
                                    int64_t NB, void* stream) {
  const int st = pkv_validate_append_e4m3(k_new, v_new, k_pool, v_pool, k_scale, v_scale,
                                          slot_mapping, T, Hkv, D, BS, NB);
  if (st != PKV_OK || T == 0) return st;
  pkv::AppendE4m3Args a{k_new, v_new, static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool),
                        k_scale, v_scale, slot_mapping, Hkv, BS};
  return launch_status(pkv::launch_append_e4m3(a, T, D, static_cast<hipStream_t>(stream)));
}

extern "C" int pkv_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (buf == nullptr || sink == nullptr || bytes < 0 || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return PKV_EINVAL;
  if (bytes == 0) return PKV_OK;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return launch_status(pkv::launch_stream_read(buf, bytes, sink, cus,
                                               static_cast<hipStream_t>(stream)));
}

extern "C" int pkv_tile_read(const void* k_pool, const void* v_pool, int64_t pool_tiles,
                             const int32_t* ids, int64_t n, int row_bytes, int waves, uint32_t* sink,
                             void* stream) {
  if (k_pool == nullptr || v_pool == nullptr || ids == nullptr || sink == nullptr || n < 0 ||
      pool_tiles < 1 || waves < 1 || waves > pkv::kMaxTileReadWaves ||
      (row_bytes != 256 && row_bytes != 128 && row_bytes != 64))
    return PKV_EINVAL;
  if (n == 0) return PKV_OK;
  return launch_status(pkv::launch_tile_read(k_pool, v_pool, pool_tiles, ids, n, row_bytes, waves, sink,
                                             static_cast<hipStream_t>(stream)));
}

extern "C" int paged_decode_step_static_partitions(int B, int Hq, int Hkv, int D, int BS, int MBS,
                                                   int n_query, int partition_size) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || BS <= 0 || MBS <= 0 || n_query < 1 ||
      partition_size < 0)
    return PKV_EINVAL;
  const int64_t cols = int64_t(Hq / Hkv) * n_query;
  const int64_t cgroups = cols > pkv::kColsPerProduct ? (cols + pkv::kColsPerProduct - 1) / pkv::kColsPerProduct : 1;
  if (int64_t(B) * Hkv * cgroups * int64_t(sizeof(uint32_t)) > int64_t(kScratchCounterBytes))
    return PKV_ENOSPACE;
  // bytes of one partial slot of every output row
  const int64_t per_slot = int64_t(B) * Hq * n_query * (int64_t(D) + 2) * int64_t(sizeof(float));
  const int64_t room = int64_t(kScratchBytes - kScratchCounterBytes);
  int P;
  if (partition_size > 0) {
    P = int((int64_t(MBS) * BS + partition_size - 1) / partition_size);
  } else {
    const int64_t fit = per_slot > 0 ? room / per_slot : pkv::kStaticStepPartitions;
    P = int(fit < pkv::kStaticStepPartitions ? fit : pkv::kStaticStepPartitions);
    if (P < 3) return PKV_ENOSPACE;
  }
  if (int64_t(P) * per_slot > room) return PKV_ENOSPACE;
  return P;
}

extern "C" int paged_decode_step_static(void* out, void* q, const void* k_new, const void* v_new,
                                        void* k_pool, void* v_pool, float* k_scale,
                                        float* v_scale, const int32_t* block_tables,
                                        const int32_t* context_lens, int B, int Hq, int Hkv, int D,
                                        int BS, int MBS, int64_t NB, float scale, int kv_dtype,
                                        int partition_size, int window, int n_query,
                                        int prefix_blocks, const float* gamma_q,
                                        const float* gamma_k, float eps, float rope_theta,
                                        void* stream) {
  const int P = paged_decode_step_static_partitions(B, Hq, Hkv, D, BS, MBS, n_query,
                                                    partition_size);
  if (P < 0) return P;
  int dev = 0;
  unsigned char* base = nullptr;
  const int sa = scratch_address(&dev, &base);
  if (sa != PKV_OK) return sa;
  const size_t rows = size_t(B) * Hq * n_query * P;
  uint32_t* counters = reinterpret_cast<uint32_t*>(base);
  float* part_out = reinterpret_cast<float*>(base + kScratchCounterBytes);
  float* part_max = part_out + rows * D;
  float* part_sum = part_max + rows;
  const int st = pkv_validate_step(out, q, k_new, v_new, k_pool, v_pool, k_scale, v_scale,
                                   block_tables, context_lens, B, Hq, Hkv, D, BS, MBS, NB, scale,
                                   kv_dtype, partition_size, window, n_query, prefix_blocks,
                                   gamma_q, gamma_k, eps, rope_theta, part_out, part_max, part_sum,
                                   counters, P);
  if (st != PKV_OK || B == 0) return st;
  const int sf = scratch_fill_once(dev, base, static_cast<hipStream_t>(stream));
  if (sf != PKV_OK) return sf;
  return paged_decode_step(out, q, k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_tables,
                           context_lens, B, Hq, Hkv, D, BS, MBS, NB, scale, kv_dtype,
                           partition_size, window, n_query, prefix_blocks, gamma_q, gamma_k, eps,
                           rope_theta, part_out, part_max, part_sum, counters, P, stream);
}
