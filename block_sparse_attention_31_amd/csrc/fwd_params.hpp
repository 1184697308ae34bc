// Launch parameters shared by the C-ABI front end and the HIP kernels.
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

// Trailing tiles of each XCD's share of the tile list that run as two
// half-height tiles: -1 picks the count from the number of tiles, n >= 0
// fixes it (0 turns the split off).
#ifndef VDN_SPLIT_TAIL
#define VDN_SPLIT_TAIL -1
#endif
#ifndef VDN_DEAL
#define VDN_DEAL 1
#endif

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
  int32_t split_tail;      // trailing tiles of each XCD's share run as two halves
  int32_t deal;            // piles each (sample, head)'s tile list is dealt into
  // Optional two-branch fusion in the epilogue (bf16 kernel; lin == nullptr
  // turns it off): out = softmax branch + sigmoid(gate_lin) * lin * lin_w /
  // sqrt(sum_h lin_ss / (H*D) + lin_eps).
  const void* lin;         // [B,S,H,D] bf16 linear-branch output
  const float* lin_ss;     // [B,S,H] per (token, head) sum of squares of lin
  const float* gate_lin;   // [B,S,H] linear-branch gate logits
  const float* lin_w;      // [H*D] RMSNorm weight
  float lin_eps;
  // Persistent launch (nullptr: one workgroup per slot): this
  // launch's claim counters, kQueueInts ints (one per XCD queue, then the
  // count of finished workgroups), zero at the start and reset to zero by
  // the last workgroup; queue_wg workgroups per XCD start on slots 0 ..
  // queue_wg-1 of their queue and claim the rest.
  int* queue;
  int32_t queue_wg;
  QBlockDesc blk[kMaxQueryBlocks];
};

// ---- backward pass ----------------------------------------------------

// A group of keys seen by the same query rows (the key side of the
// structure), as the dK/dV kernel sees it.  Both lists are virtual
// concatenations of token intervals in the KeyList form: virtual key j in
// [kiv_start[i], kiv_start[i+1]) is token j + kiv_delta[i] (kiv_start[0] = 0,
// unused starts = n_keys); likewise for the query rows with <= 2 intervals.
struct KBlockDesc {
  int32_t n_keys;
  int32_t n_rows;
  int32_t tile_prefix;  // tiles of the groups before this one in launch order
  int32_t kiv_start[2];  // starts of key intervals 1 and 2
  int32_t kiv_delta[3];
  int32_t qiv_start;     // start of query interval 1
  int32_t qiv_delta[2];
};

// Tensors and sizes shared by the backward kernels.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* gate;   // [B,S,H] or nullptr
  const float* lse;    // [B,H,S], natural log
  float* dw;           // workspace [B,H,S]: (sum_d dout * out) / sg, 0 where sg is 0
  float* lw;           // workspace [B,H,S]: lse log2(e) - log2(sg), so that
                       // sg p_ij = exp2(scale log2(e) q_i.k_j - lw_i)
                       // (sg = sigmoid(gate), 1 without a gate)
  void* dq;
  void* dk;
  void* dv;
  float* dgate;        // [B,S,H] or nullptr
  int32_t B, S, H;
  float scale;             // softmax scale
  float score_scale_log2;  // scale * log2(e)
};

struct BwdDqParams {
  BwdArgs a;
  int32_t n_blocks, tiles_per_bh, total_tiles, per_xcd;
  int32_t split_tail, deal;  // as in FwdParams
  QBlockDesc blk[kMaxQueryBlocks];  // query blocks in launch order
};

struct BwdKvParams {
  BwdArgs a;
  int32_t n_blocks, tiles_per_bh, total_tiles, per_xcd;
  int32_t split_tail, deal;  // as in FwdParams
  KBlockDesc blk[kMaxQueryBlocks];  // key groups in launch order
};

// Query rows per dQ tile and keys per dK/dV tile.
int bwd_dq_tile_m();
int bwd_dkv_tile_n();

// Enqueues the backward kernels (bf16 only): the per-row pass, dQ, dK/dV.
int launch_bwd(const BwdDqParams& dq, const BwdKvParams& kv, int head_dim, void* stream);

// Fixed device scratch of the allocation-free backward entry point: room for
// the per-row constants of batch * heads * S <= kBwdScratchFloats / 2 rows
// (32 MiB per GPU).  bwd_scratch returns its address on the current device
// (hipSuccess or the HIP error code).
constexpr int64_t kBwdScratchFloats = int64_t(8) << 20;
constexpr int kMaxScratchDevices = 64;
int bwd_scratch(float** ptr);

// Kernel-variant properties used by the front end.
int kernel_tile_m(int head_dim, int dtype);

// Enqueues the forward kernel for an already validated FwdParams.  Returns
// hipSuccess or the HIP error code.
int launch_fwd(const FwdParams& p, int head_dim, int dtype, void* stream);
// Claim counters of the persistent forward launch: kQueueSlots sets of
// kQueueInts ints in one static device array, handed out round robin (a
// set is reused only after kQueueSlots further launches in this process).
constexpr int kQueueInts = 16;
constexpr int kQueueSlots = 4096;
// Kernel instances that run persistent (a cache index each).
constexpr int kQueueBf16D64 = 0, kQueueBf16D128 = 1, kQueueFp8 = 2, kQueueKernels = 3;
// The counter set and resident workgroups per XCD for one persistent launch
// of `kernel` on the current device (queue = nullptr: launch one workgroup
// per slot instead).
int queue_for(const void* kernel, int kind, int* wg_per_xcd, int** queue);

// fp8 (e4m3) variant, head_dim 128 only.
int launch_fwd_fp8(const FwdParams& p, int head_dim, void* stream);

}  // namespace vdn
