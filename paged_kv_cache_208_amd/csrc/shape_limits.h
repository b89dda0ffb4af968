// Shape limits shared by the host checks and the launchers.
#pragma once
#include <cstdint>

namespace pkv {
constexpr int kBlockSize = 16;            // tokens per physical KV block (and per tile)
constexpr int kBlockSizeLarge = 32;       // the other block size some entry points take
constexpr int kPartitionQuantum = 16;     // partition sizes are whole blocks
constexpr int kMaxPartition = 16384;      // tokens per split-context partition
constexpr int64_t kMaxContext = int64_t(1) << 24;   // MBS * BS
constexpr int64_t kMaxGrid = (int64_t(1) << 24) - 1;  // workgroups per launch (x <= 2^32 / 256)
constexpr int64_t kMaxAppendRows = int64_t(1) << 24;
constexpr int kMaxStepPartitions = 64;     // partitions one step combines in-kernel
constexpr int kStaticStepPartitions = 16;  // pieces per sequence of the static-scratch step
constexpr int kColsPerProduct = 16;        // query columns of one 16-wide MFMA product
constexpr int kMaxNewTokens = 4096;        // new query tokens per sequence in one step
constexpr int kQkNormCols = 8;             // query columns of the QK-norm step (g * nq)
constexpr int kMaxTileReadWaves = 1 << 16; // workgroups of the paged tile-read yardstick
}  // namespace pkv
