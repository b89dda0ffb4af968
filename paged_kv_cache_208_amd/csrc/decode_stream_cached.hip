// Balanced decode step with the default cache policy for the KV tiles: the
// caller said that blocks are shared by several sequences in the call, so the
// tiles stay in L2 / the Infinity Cache for their other readers.  The kernel
// is in decode_stream_impl.h.
#include "decode_stream_impl.h"

namespace pkv {

hipError_t launch_decode_stream_cached(const DecodeArgs& a, int B, int D, int cols, bool fp8,
                                       int mode, hipStream_t stream) {
  return launch_stream_policy<true>(a, B, D, cols, fp8, mode, stream);
}

}  // namespace pkv
