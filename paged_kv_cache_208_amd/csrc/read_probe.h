// Launcher of the streaming-read yardstick (read_probe.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace pkv {
// Reads bytes (a multiple of 16) of buf once; cus = compute units of the device.
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int cus,
                              hipStream_t stream);
}  // namespace pkv
