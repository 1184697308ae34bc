// Launch parameters shared by the C-ABI front end and the HIP forward kernels.
#pragma once

#include <cstdint>

namespace vdn {

constexpr int kMaxQueryBlocks = 64;

// One query block as the kernel sees it.  The key list is the virtual
// concatenation of up to three token intervals: virtual key index
// j in [iv_start[i], iv_start[i+1]) maps to token j + iv_delta[i].
struct QBlockDesc {
  int32_t row_lo;       // first query token
  int32_t rows;         // query tokens in the block
  int32_t n_keys;       // length of the virtual key list
  int32_t tile_prefix;  // tiles of the blocks before this one in launch order
  int32_t n_iv;
  int32_t iv_start[3];  // virtual start of each interval (iv_start[0] == 0)
  int32_t iv_delta[3];  // token = virtual index + delta
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const float* gate;    // [B,S,H] or nullptr
  float* lse;           // [B,H,S] or nullptr
  const float* scales;  // fp8: [3][H], else nullptr
  int32_t B, S, H;
  float score_scale_log2;  // softmax scale * log2(e)
  int32_t n_qblocks;       // entries of blk[], in launch order
  int32_t tiles_per_bh;    // query tiles per (sample, head)
  int32_t total_tiles;     // tiles_per_bh * B * H
  int32_t per_xcd;         // ceil(total_tiles / 8)
  QBlockDesc blk[kMaxQueryBlocks];
};

// Kernel-variant properties used by the front end.
int kernel_tile_m(int head_dim, int dtype);

// Enqueues the forward kernel for an already validated FwdParams.  Returns
// hipSuccess or the HIP error code.
int launch_fwd(const FwdParams& p, int head_dim, int dtype, void* stream);

// fp8 (e4m3) variant, head_dim 128 only.
int launch_fwd_fp8(const FwdParams& p, int head_dim, void* stream);

}  // namespace vdn
