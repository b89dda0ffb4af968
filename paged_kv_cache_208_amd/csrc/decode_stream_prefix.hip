// Balanced decode step for batches whose tables share a prefix (each prefix
// tile read once per group of sequences); the kernel is in
// decode_prefix_impl.h.
#include "decode_prefix_impl.h"

namespace pkv {

hipError_t launch_decode_prefix(const DecodeArgs& a, int B, int D, int cols, bool fp8, int mode,
                                hipStream_t stream) {
  if (D == 128) return fp8 ? launch_prefix_cols<128, true>(a, B, cols, mode, stream)
                           : launch_prefix_cols<128, false>(a, B, cols, mode, stream);
  if (D == 64) return fp8 ? launch_prefix_cols<64, true>(a, B, cols, mode, stream)
                          : launch_prefix_cols<64, false>(a, B, cols, mode, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
