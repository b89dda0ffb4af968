// Streaming read of one buffer: the measured read ceiling of the GPU that the
// step kernels' KV rates are compared with.  Not part of the attention path.
//
// Each wave owns one contiguous span of the buffer and reads it 1 KiB per
// load instruction (lane i takes the i-th 16 bytes), 16 instructions in
// flight; 32 four-wave workgroups per CU.  The loads are non-temporal, as the
// decode kernels' KV loads are (5.9 TB/s with the default policy, 6.8 with
// this one, 1 GiB).  Of the shapes measured on this
// GPU (grid-stride loops with 4-16 loads in flight, spans with 8-16, 4-32
// workgroups per CU) this one read fastest.  The loaded words are
// XOR-folded and the fold is stored only if it equals a value it cannot
// take for the buffers used (so the loads stay live); nothing else is
// written.
#include "device.h"
#include "read_probe.h"

namespace pkv {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadDepth = 16;
constexpr int kReadGroupsPerCu = 32;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* buf, int64_t n16,
                                                                  uint32_t* sink) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t waves = int64_t(gridDim.x) * (kReadThreads / kWave);
  const int64_t w = int64_t(blockIdx.x) * (kReadThreads / kWave) + threadIdx.x / kWave;
  const int64_t rows = (n16 + kWave - 1) / kWave;  // 1 KiB rows (the last may be partial)
  const int64_t per = (rows + waves - 1) / waves;
  const int64_t r0 = min(w * per, rows), r1 = min(r0 + per, rows);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t r = r0; r < r1; r += kReadDepth) {
    u32x4 v[kReadDepth];
#pragma unroll
    for (int k = 0; k < kReadDepth; ++k) {
      const int64_t i = (r + k) * kWave + lane;
      v[k] = r + k < r1 && i < n16 ? __builtin_nontemporal_load(&buf[i]) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kReadDepth; ++k) acc ^= v[k];
  }
  const uint32_t fold = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (fold == 0x9E3779B9u) sink[0] = fold;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int cus,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(cus * kReadGroupsPerCu), dim3(kReadThreads), 0,
                     stream, static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pkv
