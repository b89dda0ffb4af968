// paged_attn_reduce: combine split-context partitions.
//
// Each partition p of sequence b left its max logit m_p (natural-log
// units), its exp-sum l_p relative to m_p and its normalised output o_p.
// With M = max_p m_p the partition's share of the softmax mass is
// w_p = l_p exp(m_p - M), and out = sum_p w_p o_p / sum_p w_p.  One
// workgroup per (b, q head); partitions are visited in ascending order, so
// the result is bitwise reproducible.
#include "device.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kReduceThreads = 64;

template <int D>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(ReduceArgs a) {
  constexpr int PER = D / kReduceThreads;  // dims per thread
  const int row = blockIdx.x;              // b * Hq + h
  const int b = row / a.Hq;
  const int L = a.context_lens[b];
  const int P = (L + a.partition_size - 1) / a.partition_size;
  const size_t base = size_t(row) * a.max_partitions;
  _Float16* out = static_cast<_Float16*>(a.out) + size_t(row) * D;

  float M = -FLT_MAX;
  for (int p = 0; p < P; ++p) M = fmaxf(M, a.part_max[base + p]);

  float num[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) num[k] = 0.0f;
  float den = 0.0f;
  for (int p = 0; p < P; ++p) {
    const float wgt = a.part_sum[base + p] * fast_exp2((a.part_max[base + p] - M) * kLog2e);
    den += wgt;
    const float* o = a.part_out + (base + p) * D;
#pragma unroll
    for (int k = 0; k < PER; ++k) num[k] = fmaf(wgt, o[threadIdx.x + k * kReduceThreads], num[k]);
  }
#pragma unroll
  for (int k = 0; k < PER; ++k)
    out[threadIdx.x + k * kReduceThreads] = (_Float16)(P > 0 ? num[k] / den : 0.0f);
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, int B, hipStream_t stream) {
  const unsigned grid = unsigned(int64_t(B) * a.Hq);
  if (a.D == 128)
    hipLaunchKernelGGL(reduce_kernel<128>, dim3(grid), dim3(kReduceThreads), 0, stream, a);
  else if (a.D == 64)
    hipLaunchKernelGGL(reduce_kernel<64>, dim3(grid), dim3(kReduceThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
