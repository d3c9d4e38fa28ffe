// Model dimensions and fixed sizes of libcsa2 ([N] 1 of the DeepSeek-V4.1
// reading notes: indexer 32 heads x 128, attention 64 heads x 512, 2048
// blocks x 8 positions; [N] 2.3: one scale per 16 channels).
#pragma once

#include <stddef.h>

namespace csa2 {

constexpr int kIdxHeads = 32;
constexpr int kIdxDim = 128;
constexpr int kHeads = 64;
constexpr int kDim = 512;
constexpr int kGroup = 16;
constexpr int kBlock = 8;
constexpr int kTopkSegment = 16384;  // elements one top-k workgroup holds
constexpr int kTopkMaxK = 8192;
// Bytes of the static device workspace of csa2_topk_noalloc (per GPU).
constexpr size_t kTopkScratchBytes = (size_t)8 << 20;

// Indexer-key code cache layout: tiles of 32 consecutive entries (flat entry
// index f = b * n_cap + j), each tile 2048 bytes stored as four planes of
// 16-byte chunks: byte c of entry f sits at
//   (f / 32) * 2048 + (c / 16) * 512 + (f % 32) * 16 + c % 16,
// so the 32 entries' chunk p form one contiguous 512-byte plane.  A scan
// lane that owns one entry and reads 16 bytes then makes every load
// instruction of a wave cover whole cache lines.
constexpr int kKeyTile = 32;
constexpr int kKeyPlane = kKeyTile * 16;        // 512
constexpr int kKeyTileBytes = kKeyTile * kIdxDim / 2;  // 2048

}  // namespace csa2
