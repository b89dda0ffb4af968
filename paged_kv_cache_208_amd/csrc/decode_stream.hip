// Balanced decode step, KV tiles streamed with the non-temporal cache policy
// (the default), and the launcher that picks the policy from the caller's
// shared-blocks hint.  The kernel itself is in decode_stream_impl.h.
#include "decode_stream_impl.h"

namespace pkv {

hipError_t launch_decode_stream(const DecodeArgs& a, int B, int D, int cols, bool fp8, int mode,
                                hipStream_t stream) {
  if (a.cached_kv) return launch_decode_stream_cached(a, B, D, cols, fp8, mode, stream);
  return launch_stream_policy<false>(a, B, D, cols, fp8, mode, stream);
}

}  // namespace pkv
