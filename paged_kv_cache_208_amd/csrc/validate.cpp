// Host-side argument checks for the pagedkv C ABI.  Pure C++: no HIP call,
// so the checks run (and are tested) on machines without a GPU.  Each entry
// point of the library calls the matching check first and enqueues nothing
// when it fails.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "pagedkv.h"
#include "shape_limits.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_head_dim(int D) { return D == 64 || D == 128; }

bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

// Block sizes of the entry points that take either (the rest take 16 only).
bool supported_block_size(int BS) { return BS == pkv::kBlockSize || BS == pkv::kBlockSizeLarge; }

}  // namespace

extern "C" const char* pkv_strerror(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument (null or misaligned pointer, or inconsistent sizes)";
    case PKV_EUNSUPPORTED: return "unsupported configuration (head_dim, GQA group, block size or partition size)";
    case PKV_ELAUNCH: return "HIP kernel launch failed";
    case PKV_ENOSPACE: return "the batch does not fit the library's static scratch (32 MiB per GPU)";
    default: return "unknown pkv status";
  }
}

extern "C" size_t paged_attn_workspace_size(int B, int Hq, int D, int max_partitions) {
  if (B < 0 || Hq < 0 || D < 0 || max_partitions < 0) return 0;
  const uint64_t rows = uint64_t(B) * uint64_t(Hq) * uint64_t(max_partitions);
  const uint64_t bytes = rows * (uint64_t(D) + 2) * sizeof(float);
  if (rows != 0 && bytes / rows != (uint64_t(D) + 2) * sizeof(float)) return 0;
  return size_t(bytes);
}

extern "C" int pkv_validate_append(const void* k_new, const void* v_new, const void* k_pool,
                                   const void* v_pool, const int64_t* slot_mapping, int T,
                                   int Hkv, int D, int BS, int64_t NB, const void* q_inout,
                                   int Hq, const float* gamma_q, const float* gamma_k,
                                   const int32_t* context_lens, float eps, float rope_theta) {
  if (T < 0 || Hkv <= 0 || NB <= 0 || D <= 0 || BS <= 0) return PKV_EINVAL;
  if (!supported_head_dim(D)) return PKV_EUNSUPPORTED;
  if (!supported_block_size(BS)) return PKV_EUNSUPPORTED;
  if (int64_t(T) * Hkv > pkv::kMaxAppendRows) return PKV_EUNSUPPORTED;
  if (T == 0) return PKV_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !slot_mapping) return PKV_EINVAL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pool, 16) ||
      !aligned(v_pool, 16) || !aligned(slot_mapping, 8))
    return PKV_EINVAL;
  if (gamma_k != nullptr) {  // fused QK-norm + RoPE
    if (!q_inout || !gamma_q || !context_lens) return PKV_EINVAL;
    if (!aligned(q_inout, 16) || !aligned(gamma_q, 4) || !aligned(gamma_k, 4) ||
        !aligned(context_lens, 4))
      return PKV_EINVAL;
    if (Hq <= 0 || Hq % Hkv != 0) return PKV_EINVAL;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return PKV_EINVAL;
    if (!(rope_theta > 0.0f) || !std::isfinite(rope_theta)) return PKV_EINVAL;
  }
  return PKV_OK;
}

extern "C" int pkv_validate_decode(const void* out, const void* q, const void* k_pool,
                                   const void* v_pool, const float* k_scale,
                                   const float* v_scale, const int32_t* block_tables,
                                   const int32_t* context_lens, int B, int Hq, int Hkv, int D,
                                   int BS, int MBS, int64_t NB, float scale, int kv_dtype,
                                   int partition_size, const float* part_out,
                                   const float* part_max, const float* part_sum,
                                   int max_partitions) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || BS <= 0 || MBS <= 0 || NB <= 0)
    return PKV_EINVAL;
  if (Hq % Hkv != 0) return PKV_EINVAL;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return PKV_EINVAL;
  kv_dtype &= ~PKV_KV_SHARED_BLOCKS;  // a cache-policy hint, not part of the dtype
  if (kv_dtype != PKV_KV_F16 && kv_dtype != PKV_KV_E4M3) return PKV_EINVAL;
  if (partition_size < 0) return PKV_EINVAL;
  if (!supported_head_dim(D) || !supported_group(Hq / Hkv)) return PKV_EUNSUPPORTED;
  if (BS != pkv::kBlockSize) return PKV_EUNSUPPORTED;
  if (partition_size != 0 &&
      (partition_size % pkv::kPartitionQuantum != 0 || partition_size > pkv::kMaxPartition))
    return PKV_EUNSUPPORTED;
  if (int64_t(MBS) * BS > pkv::kMaxContext) return PKV_EUNSUPPORTED;
  if (B == 0) return PKV_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens) return PKV_EINVAL;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PKV_EINVAL;
  if (kv_dtype == PKV_KV_E4M3) {
    if (!k_scale || !v_scale || !aligned(k_scale, 4) || !aligned(v_scale, 4)) return PKV_EINVAL;
  }
  int64_t units;
  if (partition_size == 0) {
    if (!out || !aligned(out, 16)) return PKV_EINVAL;
    units = int64_t(B) * Hkv;
  } else {
    if (!part_out || !part_max || !part_sum) return PKV_EINVAL;
    if (!aligned(part_out, 16) || !aligned(part_max, 4) || !aligned(part_sum, 4))
      return PKV_EINVAL;
    const int64_t need = (int64_t(MBS) * BS + partition_size - 1) / partition_size;
    if (max_partitions < need) return PKV_EINVAL;
    units = int64_t(B) * Hkv * max_partitions;
  }
  if (units > pkv::kMaxGrid) return PKV_EUNSUPPORTED;
  return PKV_OK;
}

extern "C" int pkv_validate_reduce(const void* out, const float* part_out,
                                   const float* part_max, const float* part_sum,
                                   const int32_t* context_lens, int B, int Hq, int D,
                                   int partition_size, int max_partitions) {
  if (B < 0 || Hq <= 0 || D <= 0 || partition_size <= 0 || max_partitions <= 0)
    return PKV_EINVAL;
  if (!supported_head_dim(D)) return PKV_EUNSUPPORTED;
  if (partition_size % pkv::kPartitionQuantum != 0 || partition_size > pkv::kMaxPartition)
    return PKV_EUNSUPPORTED;
  if (int64_t(B) * Hq > pkv::kMaxGrid) return PKV_EUNSUPPORTED;
  if (B == 0) return PKV_OK;
  if (!out || !part_out || !part_max || !part_sum || !context_lens) return PKV_EINVAL;
  if (!aligned(out, 16) || !aligned(part_out, 16) || !aligned(part_max, 4) ||
      !aligned(part_sum, 4) || !aligned(context_lens, 4))
    return PKV_EINVAL;
  return PKV_OK;
}

extern "C" int pkv_validate_step(const void* out, const void* q, const void* k_new,
                                 const void* v_new, const void* k_pool, const void* v_pool,
                                 const float* k_scale, const float* v_scale,
                                 const int32_t* block_tables, const int32_t* context_lens, int B,
                                 int Hq, int Hkv, int D, int BS, int MBS, int64_t NB, float scale,
                                 int kv_dtype, int partition_size, int window, int n_query,
                                 int prefix_blocks, const float* gamma_q, const float* gamma_k,
                                 float eps,
                                 float rope_theta, const float* part_out, const float* part_max,
                                 const float* part_sum, const uint32_t* counters,
                                 int max_partitions) {
  // 32-token blocks: balanced split only; they are checked as 16-token
  // tiles (two per block) from here on
  if (!supported_block_size(BS)) return PKV_EUNSUPPORTED;
  if (BS != pkv::kBlockSize && partition_size != 0) return PKV_EUNSUPPORTED;
  const int tiles = BS / pkv::kBlockSize;
  // the attention part is checked as paged_attn_decode checks it: fixed
  // partitions as partitioned work (one workgroup per partition), the
  // balanced split as a single pass (its grid does not grow with the
  // context; its workspace is checked below)
  int st = pkv_validate_decode(out, q, k_pool, v_pool, k_scale, v_scale, block_tables,
                               context_lens, B, Hq, Hkv, D, pkv::kBlockSize, MBS * tiles,
                               NB * tiles, scale, kv_dtype, partition_size, part_out, part_max,
                               part_sum, partition_size == 0 ? 1 : max_partitions);
  if (st != PKV_OK) return st;
  if (window < 0) return PKV_EINVAL;
  if (window > 0 && partition_size != 0) return PKV_EUNSUPPORTED;  // balanced split only
  if (n_query < 1) return PKV_EINVAL;
  if (n_query > 1) {
    // several new tokens: balanced split, no window.  Their (Hq / Hkv) *
    // n_query query columns fill one 16-wide product (a power of two up to
    // 16; with QK-norm up to 8) or whole 16-column groups, which take their
    // new rows already appended (k_new == NULL, no QK-norm)
    if (partition_size != 0 || window != 0) return PKV_EUNSUPPORTED;
    if (n_query > pkv::kMaxNewTokens) return PKV_EUNSUPPORTED;
    const int cols = (Hq / Hkv) * n_query;
    if (gamma_k != nullptr && cols > pkv::kQkNormCols) return PKV_EUNSUPPORTED;
    if (cols <= pkv::kColsPerProduct) {
      if ((cols & (cols - 1)) != 0) return PKV_EUNSUPPORTED;
    } else {
      if (cols % pkv::kColsPerProduct != 0 || k_new != nullptr) return PKV_EUNSUPPORTED;
    }
  }
  if (prefix_blocks < 0 || prefix_blocks > MBS) return PKV_EINVAL;
  if (prefix_blocks > 0) {
    // the shared-prefix step: balanced split, one new token, no window or
    // QK-norm; a (sequence, kv head) takes up to max_partitions / 2 prefix
    // and own pieces each
    if (partition_size != 0 || n_query != 1 || window != 0 || gamma_k != nullptr)
      return PKV_EUNSUPPORTED;
    if (max_partitions < 6) return PKV_EINVAL;
  }
  if (B == 0) return st;
  if (!out || !aligned(out, 16)) return PKV_EINVAL;
  if (!counters || !aligned(counters, 4)) return PKV_EINVAL;
  if (partition_size == 0) {
    // balanced split: between 3 and 64 pieces per sequence
    if (!part_out || !part_max || !part_sum) return PKV_EINVAL;
    if (!aligned(part_out, 16) || !aligned(part_max, 4) || !aligned(part_sum, 4))
      return PKV_EINVAL;
    if (max_partitions < 3) return PKV_EINVAL;
    if (max_partitions > pkv::kMaxStepPartitions) return PKV_EUNSUPPORTED;
  } else {
    // the in-kernel combine holds at most 64 partitions per sequence
    if ((int64_t(MBS) * BS + partition_size - 1) / partition_size > pkv::kMaxStepPartitions)
      return PKV_EUNSUPPORTED;
  }
  if (k_new != nullptr) {
    // E4M3 rows go through the E4M3 append (its own launch ahead of the
    // attention), one new token per sequence: its slots lie in distinct
    // blocks, as that append requires; no QK-norm
    if ((kv_dtype & ~PKV_KV_SHARED_BLOCKS) == PKV_KV_E4M3 && (n_query != 1 || gamma_k != nullptr))
      return PKV_EUNSUPPORTED;
    if (int64_t(B) > pkv::kMaxGrid || Hkv > 65535) return PKV_EUNSUPPORTED;
    if (!v_new || !aligned(k_new, 16) || !aligned(v_new, 16)) return PKV_EINVAL;
  } else if (v_new != nullptr) {
    return PKV_EINVAL;
  }
  if (gamma_k != nullptr) {
    if (!k_new || !gamma_q || !aligned(gamma_q, 4) || !aligned(gamma_k, 4)) return PKV_EINVAL;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return PKV_EINVAL;
    if (!(rope_theta > 0.0f) || !std::isfinite(rope_theta)) return PKV_EINVAL;
  } else if (gamma_q != nullptr) {
    return PKV_EINVAL;
  }
  return PKV_OK;
}

extern "C" int pkv_validate_copy(const void* k_pool, const void* v_pool, const float* k_scale,
                                 const float* v_scale, const int32_t* src, const int32_t* dst,
                                 int n, int Hkv, int D, int BS, int64_t NB, int kv_dtype) {
  if (n < 0 || Hkv <= 0 || D <= 0 || BS <= 0 || NB <= 0) return PKV_EINVAL;
  if (kv_dtype != PKV_KV_F16 && kv_dtype != PKV_KV_E4M3) return PKV_EINVAL;
  if (!supported_head_dim(D)) return PKV_EUNSUPPORTED;
  if (!supported_block_size(BS)) return PKV_EUNSUPPORTED;
  if (int64_t(n) > pkv::kMaxGrid) return PKV_EUNSUPPORTED;
  if (n == 0) return PKV_OK;
  if (!k_pool || !v_pool || !src || !dst) return PKV_EINVAL;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(src, 4) || !aligned(dst, 4))
    return PKV_EINVAL;
  if (kv_dtype == PKV_KV_E4M3) {
    if (!k_scale || !v_scale) return PKV_EINVAL;
    if (!aligned(k_scale, 4) || !aligned(v_scale, 4)) return PKV_EINVAL;
  }
  return PKV_OK;
}

extern "C" int pkv_validate_append_e4m3(const void* k_new, const void* v_new, const void* k_pool,
                                        const void* v_pool, const float* k_scale,
                                        const float* v_scale, const int64_t* slot_mapping, int T,
                                        int Hkv, int D, int BS, int64_t NB) {
  if (T < 0 || Hkv <= 0 || NB <= 0 || D <= 0 || BS <= 0) return PKV_EINVAL;
  if (!supported_head_dim(D)) return PKV_EUNSUPPORTED;
  if (!supported_block_size(BS)) return PKV_EUNSUPPORTED;
  if (int64_t(T) > pkv::kMaxGrid || Hkv > 65535) return PKV_EUNSUPPORTED;
  if (T == 0) return PKV_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !k_scale || !v_scale || !slot_mapping)
    return PKV_EINVAL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pool, 16) ||
      !aligned(v_pool, 16) || !aligned(k_scale, 4) || !aligned(v_scale, 4) ||
      !aligned(slot_mapping, 8))
    return PKV_EINVAL;
  return PKV_OK;
}
