// Model dimensions and fixed sizes of libcsa2 ([N] 1 of the DeepSeek-V4.1
// reading notes: indexer 32 heads x 128, attention 64 heads x 512, 2048
// blocks x 8 positions; [N] 2.3: one scale per 16 channels).
#pragma once

namespace csa2 {

constexpr int kIdxHeads = 32;
constexpr int kIdxDim = 128;
constexpr int kHeads = 64;
constexpr int kDim = 512;
constexpr int kGroup = 16;
constexpr int kBlock = 8;
constexpr int kTopkSegment = 16384;  // elements one top-k workgroup holds
constexpr int kTopkMaxK = 8192;

}  // namespace csa2
