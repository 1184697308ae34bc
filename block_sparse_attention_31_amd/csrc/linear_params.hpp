// Launch parameters of the complement linear branch and the two-branch
// fusion, shared by the C-ABI front end and the HIP kernels.
#pragma once

#include <cstdint>

namespace vdn {

// Rows of one linear-branch apply tile (a tile never spans two frame blocks).
#ifndef VDN_LIN_ROW_TILE
#define VDN_LIN_ROW_TILE 512
#endif
constexpr int kLinRowTile = VDN_LIN_ROW_TILE;

struct LinParams {
  const void* q;   // [B,S,H,D] bf16
  const void* k;
  const void* v;
  void* out;       // [B,S,H,D] bf16
  float* fstate;   // workspace [B*H][F-2][D*D + D]: per-frame sum_t v phi(k)^T
                   // ([d2][d1], fp32) followed by sum_t phi(k) ([d1])
  void* bstate;    // workspace [B*H][nb][D*D] bf16: per-block state, [d2][d1]
  float* bz;       // workspace [B*H][nb][D] fp32: per-block normaliser
  float* ss;       // optional [B,S,H] fp32: sum over d of each output row's
                   // squares (before rounding to bf16), or nullptr
  int32_t B, S, H, F, T, Bf, nb;
  int32_t tiles_per_block;  // apply tiles of a full frame block
  int32_t tiles_last;       // apply tiles of the last frame block
  int32_t tiles_text;       // apply tiles of the text rows
  int32_t tiles_per_bh;     // sum of the three counts above
  int32_t total_tiles;      // tiles_per_bh * B * H
};

// Byte offsets of the three workspace regions and the total size.
struct LinWorkspace {
  uint64_t fstate_off, bstate_off, bz_off, total;
};

inline LinWorkspace linear_workspace(int64_t B, int64_t H, int64_t F, int64_t nb, int64_t D) {
  auto up = [](uint64_t x) { return (x + 255u) & ~uint64_t(255); };
  const uint64_t bh = uint64_t(B) * uint64_t(H);
  const uint64_t nf = F > 2 ? uint64_t(F - 2) : 0u;
  LinWorkspace w;
  w.fstate_off = 0;
  w.bstate_off = up(bh * nf * uint64_t(D * D + D) * 4u);
  w.bz_off = w.bstate_off + up(bh * uint64_t(nb) * uint64_t(D * D) * 2u);
  w.total = w.bz_off + up(bh * uint64_t(nb) * uint64_t(D) * 4u);
  return w;
}

struct FuseParams {
  const void* soft;     // [rows, H*D] bf16: gated softmax-branch output
  const void* lin;      // [rows, H*D] bf16: linear-branch output
  const float* gate;    // [rows, H] fp32 logits of the linear branch's gate
  const float* weight;  // [H*D] fp32 RMSNorm weight
  void* out;            // [rows, H*D] bf16 (may be the same buffer as soft)
  int64_t rows;
  int32_t H, D, HD;
  float eps;
};

int launch_linear(const LinParams& p, int head_dim, void* stream);
int launch_fuse(const FuseParams& p, void* stream);

}  // namespace vdn
