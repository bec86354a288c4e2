// Tile geometry of the split kernels: the one definition that both the HIP
// kernels (split_mfma.hip, split_valu.hip) and the host planner (api.cpp,
// plan.cpp) read, so the planner's split boundaries always match the tiles
// the kernels stream.
#pragma once

// Waves per split workgroup, both kernels: 4 unless the build sets another
// value (decode_attention_fd_amd/build.py --waves; for measurements).
#ifndef FD_SPLIT_WAVES
#define FD_SPLIT_WAVES 4
#endif

namespace fd {

constexpr int kSplitWaves = FD_SPLIT_WAVES;   // waves per split workgroup, both kernels
static_assert(kSplitWaves >= 1 && kSplitWaves <= 16, "1 to 16 waves per split workgroup");
constexpr int kMfmaTileTokens = 32;      // KV tokens per wave tile, MFMA kernel
constexpr int kValuLoadsPerTile = 8;     // 16-byte load instructions per wave tile per tensor, VALU kernel

// VALU kernel: a K/V row of head_dim elements is read by head_dim * elt / 16
// lanes (16 bytes each), so one wave load instruction covers 64 / that many
// rows, and a wave tile is kValuLoadsPerTile such instructions.
constexpr int valu_tile_tokens_for(int head_dim, int elt_bytes) {
  return kValuLoadsPerTile * (64 / (head_dim * elt_bytes / 16));
}

}  // namespace fd
