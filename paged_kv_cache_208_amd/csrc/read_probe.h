// Launcher of the streaming-read yardstick (read_probe.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace pkv {
// Reads bytes (a multiple of 16) of buf once; cus = compute units of the device.
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int cus,
                              hipStream_t stream);
// Reads the n listed tiles (16 rows of row_bytes in K and in V each, ntiles
// in each pool) once, split over `waves` single-wave workgroups.
hipError_t launch_tile_read(const void* k_pool, const void* v_pool, int64_t ntiles, const int32_t* ids,
                            int64_t n, int row_bytes, int waves, uint32_t* sink, hipStream_t stream);
}  // namespace pkv
