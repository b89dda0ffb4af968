// Copy-on-write block copy for gfx950 ("Distributed LLM Inference Serving
// Platform", section 11, Lab 1 worked solution: a sequence that appends into
// a shared tail block writes into a fresh copy of it).
//
// One 256-thread workgroup per (pair, pool): the block's Hkv x 16 x D
// elements are one contiguous run of block_bytes in the pool, moved in
// 16-byte pieces, eight loads in flight per lane before their stores.  The
// E4M3 scales of the block (Hkv floats per pool) go along.  The source is
// read once, so its loads are non-temporal (measured 4.1 -> 5.3 TB/s of read
// + write on MI355X); non-temporal stores gained nothing and are not used.
#include "device.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyBatch = 8;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyArgs a) {
  const int pair = blockIdx.x;
  const bool v = blockIdx.y != 0;
  const int64_t src = __builtin_amdgcn_readfirstlane(a.src[pair]);
  const int64_t dst = __builtin_amdgcn_readfirstlane(a.dst[pair]);
  uint8_t* pool = v ? a.v_pool : a.k_pool;
  const u32x4* from = reinterpret_cast<const u32x4*>(pool + src * a.block_bytes);
  u32x4* to = reinterpret_cast<u32x4*>(pool + dst * a.block_bytes);
  const int64_t pieces = a.block_bytes / 16;
  for (int64_t i0 = 0; i0 < pieces; i0 += int64_t(kCopyThreads) * kCopyBatch) {
    u32x4 buf[kCopyBatch];
#pragma unroll
    for (int k = 0; k < kCopyBatch; ++k) {
      const int64_t i = i0 + k * kCopyThreads + threadIdx.x;
      if (i < pieces) buf[k] = __builtin_nontemporal_load(&from[i]);
    }
#pragma unroll
    for (int k = 0; k < kCopyBatch; ++k) {
      const int64_t i = i0 + k * kCopyThreads + threadIdx.x;
      if (i < pieces) to[i] = buf[k];
    }
  }
  float* scale = v ? a.v_scale : a.k_scale;
  if (scale != nullptr)
    for (int h = threadIdx.x; h < a.Hkv; h += kCopyThreads) scale[dst * a.Hkv + h] = scale[src * a.Hkv + h];
}

}  // namespace

hipError_t launch_copy_blocks(const CopyArgs& a, int n, hipStream_t stream) {
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(unsigned(n), 2u), dim3(kCopyThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
