// C-ABI front end: argument validation, schedule construction and launch of
// the forward kernels.  Every check runs before the first HIP call.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>
#include <algorithm>

#include "../../include/vdn_local_attn.h"
#include "fwd_params.hpp"
#include "linear_params.hpp"
#include "schedule.hpp"

namespace {

// Tiles of each XCD's share (32 compute units) that run as two half-height
// tiles at its end, from the share's size (measured on the 768p shape with
// 1 to 32 heads): at most half a round in all, every tile (one round of
// halves); a last round at most half full in one to four rounds, 16; else
// none (a split then costs more than the idle end it fills).
int split_tail_for(int per_xcd) {
  if (per_xcd <= 16) return per_xcd;
  if (per_xcd >= 32 && per_xcd < 128 && per_xcd % 32 <= 16) return 16;
  return 0;
}

// Dispatch fields shared by the tiled kernels: each XCD's share of the tile
// list, the half tiles at its end, and how many piles a (sample, head)'s
// tiles are dealt into when it spans several shares.
template <class P>
void set_dispatch(P& p) {
  p.per_xcd = (p.total_tiles + 7) / 8;
  p.split_tail = VDN_SPLIT_TAIL < 0 ? split_tail_for(p.per_xcd) : std::min(p.per_xcd, VDN_SPLIT_TAIL);
  p.deal = (VDN_DEAL && p.per_xcd < p.tiles_per_bh)
               ? std::min(8, (p.tiles_per_bh + p.per_xcd - 1) / p.per_xcd)
               : 1;
}

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int ok() {
  g_last_error.clear();
  return VDN_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

bool aligned(const void* ptr, uintptr_t n) { return (reinterpret_cast<uintptr_t>(ptr) % n) == 0; }

// The linear branch's share of vdn_hybrid_attn_fwd, passed to the softmax
// branch's epilogue.
struct FuseArgs {
  const void* lin;
  const float* ss;
  const float* gate_lin;
  const float* weight;
  float eps;
};

uint64_t up256(uint64_t x) { return (x + 255u) & ~uint64_t(255); }

// The tiled kernels address the rows of one DMA batch (at most 128 keys or
// query rows of one (sample, head)) with 32-bit per-lane byte offsets from a
// scalar base: 128 token strides of heads * head_dim elements must fit.
bool dma_offsets_fit(int heads, int head_dim, int elem_bytes) {
  return int64_t(128) * heads * head_dim * elem_bytes < (int64_t(1) << 32);
}

}  // namespace

extern "C" {

const char* vdn_last_error(void) { return g_last_error.c_str(); }

int vdn_local_attn_num_query_blocks(int F, int tokens_per_frame, int n_text, int block_frames) {
  vdn::Geometry g;
  std::string err;
  if (!vdn::make_geometry(F, tokens_per_frame, n_text, block_frames, &g, &err))
    return fail(VDN_ERR_INVALID_ARG, err);
  ok();
  return int(g.nb + (g.N > 0 ? 1 : 0));
}

int vdn_local_attn_key_intervals(int F, int tokens_per_frame, int n_text, int block_frames,
                                 int64_t* query_rows, int64_t* key_intervals, int capacity,
                                 int* n_qblocks) {
  vdn::Geometry g;
  std::string err;
  if (!vdn::make_geometry(F, tokens_per_frame, n_text, block_frames, &g, &err))
    return fail(VDN_ERR_INVALID_ARG, err);
  if (n_qblocks == nullptr) return fail(VDN_ERR_INVALID_ARG, "n_qblocks is NULL");
  const auto blocks = vdn::build_query_blocks(g);
  *n_qblocks = int(blocks.size());
  if (capacity < int(blocks.size()))
    return fail(VDN_ERR_CAPACITY, "capacity " + std::to_string(capacity) + " < " +
                                      std::to_string(blocks.size()) + " query blocks");
  for (size_t i = 0; i < blocks.size(); ++i) {
    if (query_rows != nullptr) {
      query_rows[2 * i] = blocks[i].row_lo;
      query_rows[2 * i + 1] = blocks[i].row_hi;
    }
    if (key_intervals != nullptr) {
      int64_t* dst = key_intervals + i * VDN_MAX_KEY_INTERVALS * 2;
      for (int j = 0; j < VDN_MAX_KEY_INTERVALS; ++j) {
        const bool used = j < blocks[i].n_iv;
        dst[2 * j] = used ? blocks[i].iv[j].lo : -1;
        dst[2 * j + 1] = used ? blocks[i].iv[j].hi : -1;
      }
    }
  }
  return ok();
}

int vdn_local_attn_count_pairs(int F, int tokens_per_frame, int n_text, int block_frames,
                               int64_t* allowed, int64_t* anchor_added) {
  vdn::Geometry g;
  std::string err;
  if (!vdn::make_geometry(F, tokens_per_frame, n_text, block_frames, &g, &err))
    return fail(VDN_ERR_INVALID_ARG, err);
  if (allowed == nullptr || anchor_added == nullptr)
    return fail(VDN_ERR_INVALID_ARG, "allowed / anchor_added is NULL");
  vdn::count_pairs(g, allowed, anchor_added);
  return ok();
}

int vdn_local_attn_tile_schedule(int F, int tokens_per_frame, int n_text, int block_frames,
                                 int tile_m, int32_t* out, int capacity, int* n_entries) {
  vdn::Geometry g;
  std::string err;
  if (!vdn::make_geometry(F, tokens_per_frame, n_text, block_frames, &g, &err))
    return fail(VDN_ERR_INVALID_ARG, err);
  if (tile_m <= 0) return fail(VDN_ERR_INVALID_ARG, "tile_m must be >= 1");
  if (n_entries == nullptr) return fail(VDN_ERR_INVALID_ARG, "n_entries is NULL");
  if (g.S > INT32_MAX) return fail(VDN_ERR_OVERFLOW, "S does not fit int32");
  const auto tiles = vdn::tile_schedule(vdn::build_query_blocks(g), tile_m);
  *n_entries = int(tiles.size());
  if (capacity < int(tiles.size()))
    return fail(VDN_ERR_CAPACITY, "capacity " + std::to_string(capacity) + " < " +
                                      std::to_string(tiles.size()) + " tiles");
  if (out == nullptr && !tiles.empty()) return fail(VDN_ERR_INVALID_ARG, "out is NULL");
  for (size_t i = 0; i < tiles.size(); ++i) {
    out[4 * i] = tiles[i].qblock;
    out[4 * i + 1] = tiles[i].row0;
    out[4 * i + 2] = tiles[i].rows;
    out[4 * i + 3] = tiles[i].keys;
  }
  return ok();
}

int vdn_local_attn_key_blocks(int F, int tokens_per_frame, int n_text, int block_frames,
                              int64_t* key_intervals, int64_t* query_intervals, int capacity,
                              int* n_kblocks) {
  vdn::Geometry g;
  std::string err;
  if (!vdn::make_geometry(F, tokens_per_frame, n_text, block_frames, &g, &err))
    return fail(VDN_ERR_INVALID_ARG, err);
  if (n_kblocks == nullptr) return fail(VDN_ERR_INVALID_ARG, "n_kblocks is NULL");
  const auto blocks = vdn::build_key_blocks(g);
  *n_kblocks = int(blocks.size());
  if (capacity < int(blocks.size()))
    return fail(VDN_ERR_CAPACITY, "capacity " + std::to_string(capacity) + " < " +
                                      std::to_string(blocks.size()) + " key blocks");
  for (size_t i = 0; i < blocks.size(); ++i) {
    const vdn::KeyBlock& kb = blocks[i];
    for (int side = 0; side < 2; ++side) {
      int64_t* base = side == 0 ? key_intervals : query_intervals;
      if (base == nullptr) continue;
      int64_t* dst = base + i * VDN_MAX_KEY_INTERVALS * 2;
      const int n = side == 0 ? kb.n_kiv : kb.n_qiv;
      const vdn::Interval* iv = side == 0 ? kb.kiv : kb.qiv;
      for (int j = 0; j < VDN_MAX_KEY_INTERVALS; ++j) {
        dst[2 * j] = j < n ? iv[j].lo : -1;
        dst[2 * j + 1] = j < n ? iv[j].hi : -1;
      }
    }
  }
  return ok();
}

int vdn_local_attn_kernel_tile_m(int head_dim, int dtype) {
  if (head_dim != 64 && head_dim != 128)
    return fail(VDN_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (dtype != VDN_BF16 && dtype != VDN_FP8_E4M3) return fail(VDN_ERR_UNSUPPORTED, "unknown dtype");
  ok();
  return vdn::kernel_tile_m(head_dim, dtype);
}

static int local_attn_fwd_impl(const void* q, const void* k, const void* v, const float* gate,
                               void* out, int F, int tokens_per_frame, int n_text, int block_frames,
                               int heads, int head_dim, int dtype, int batch,
                               const float* qkv_scales, float softmax_scale, float* lse,
                               void* hip_stream, const FuseArgs* fuse, bool validate_only = false) {
  vdn::Geometry g;
  std::string err;
  if (!vdn::make_geometry(F, tokens_per_frame, n_text, block_frames, &g, &err))
    return fail(VDN_ERR_INVALID_ARG, err);
  if (heads <= 0 || batch <= 0)
    return fail(VDN_ERR_INVALID_ARG, "heads and batch must be >= 1");
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
    return fail(VDN_ERR_INVALID_ARG, "q, k, v and out must be non-NULL");
  if (head_dim != 64 && head_dim != 128)
    return fail(VDN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got " + std::to_string(head_dim) + ")");
  if (dtype != VDN_BF16 && dtype != VDN_FP8_E4M3)
    return fail(VDN_ERR_UNSUPPORTED, "unknown dtype " + std::to_string(dtype));
  if (dtype == VDN_FP8_E4M3 && qkv_scales == nullptr)
    return fail(VDN_ERR_UNSUPPORTED, "fp8 inputs need qkv_scales");
  if (dtype == VDN_FP8_E4M3 && head_dim != 128)
    return fail(VDN_ERR_UNSUPPORTED, "fp8 inputs need head_dim 128");
  if (dtype == VDN_BF16 && qkv_scales != nullptr)
    return fail(VDN_ERR_INVALID_ARG, "qkv_scales must be NULL for bf16 inputs");
  if (!std::isfinite(softmax_scale))
    return fail(VDN_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(VDN_ERR_ALIGNMENT, "q, k, v and out must be 16-byte aligned");
  if (!aligned(gate, 4) || !aligned(lse, 4) || !aligned(qkv_scales, 4))
    return fail(VDN_ERR_ALIGNMENT, "gate, lse and qkv_scales must be 4-byte aligned");
  // Index types: token indices and per-sample offsets in int32 inside the
  // kernel's loops, element offsets in int64.
  if (g.S > INT32_MAX / 2)
    return fail(VDN_ERR_OVERFLOW, "sequence length " + std::to_string(g.S) + " too large");
  const int64_t elems = int64_t(batch) * g.S * int64_t(heads) * int64_t(head_dim);
  if (elems / batch / heads / head_dim != g.S || elems > (int64_t(1) << 46))
    return fail(VDN_ERR_OVERFLOW, "tensor element count overflows");
  if (int64_t(batch) * heads > INT32_MAX / 4096)
    return fail(VDN_ERR_OVERFLOW, "batch * heads too large");
  if (!dma_offsets_fit(heads, head_dim, dtype == VDN_BF16 ? 2 : 1))
    return fail(VDN_ERR_OVERFLOW, "128 token strides of heads * head_dim elements exceed 2^32 bytes");

  const size_t in_bytes = size_t(elems) * (dtype == VDN_BF16 ? 2u : 1u);
  const size_t out_bytes = size_t(elems) * 2u;
  const size_t gate_bytes = gate ? size_t(batch) * size_t(g.S) * size_t(heads) * 4u : 0u;
  const size_t lse_bytes = lse ? size_t(batch) * size_t(heads) * size_t(g.S) * 4u : 0u;
  const size_t sc_bytes = qkv_scales ? size_t(3) * size_t(heads) * 4u : 0u;
  const void* ins[] = {q, k, v, gate, qkv_scales};
  const size_t in_sz[] = {in_bytes, in_bytes, in_bytes, gate_bytes, sc_bytes};
  for (int i = 0; i < 5; ++i) {
    if (overlaps(out, out_bytes, ins[i], in_sz[i]))
      return fail(VDN_ERR_INVALID_ARG, "out overlaps an input");
    if (overlaps(lse, lse_bytes, ins[i], in_sz[i]))
      return fail(VDN_ERR_INVALID_ARG, "lse overlaps an input");
  }
  if (overlaps(out, out_bytes, lse, lse_bytes)) return fail(VDN_ERR_INVALID_ARG, "out overlaps lse");

  const auto blocks = vdn::build_query_blocks(g);
  if (int(blocks.size()) > vdn::kMaxQueryBlocks)
    return fail(VDN_ERR_UNSUPPORTED, std::to_string(blocks.size()) + " query blocks exceed the limit of " +
                                         std::to_string(vdn::kMaxQueryBlocks));

  const int tile_m = vdn::kernel_tile_m(head_dim, dtype);
  vdn::FwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.gate = gate;
  p.lse = lse;
  p.scales = qkv_scales;
  p.B = batch;
  p.S = int32_t(g.S);
  p.H = heads;
  const float sm = softmax_scale > 0.f ? softmax_scale : float(1.0 / std::sqrt(double(head_dim)));
  p.score_scale_log2 = float(double(sm) * 1.4426950408889634);
  int prefix = 0;
  int n = 0;
  for (int bi : vdn::cost_order(blocks)) {
    const vdn::QueryBlock& qb = blocks[size_t(bi)];
    vdn::QBlockDesc& d = p.blk[n++];
    d.row_lo = int32_t(qb.row_lo);
    d.rows = int32_t(qb.row_hi - qb.row_lo);
    d.n_keys = int32_t(qb.n_keys);
    d.tile_prefix = prefix;
    d.n_iv = qb.n_iv;
    int64_t start = 0;
    for (int i = 0; i < qb.n_iv; ++i) {
      d.iv_start[i] = int32_t(start);
      d.iv_delta[i] = int32_t(qb.iv[i].lo - start);
      start += qb.iv[i].hi - qb.iv[i].lo;
    }
    prefix += (d.rows + tile_m - 1) / tile_m;
  }
  p.n_qblocks = n;
  p.tiles_per_bh = prefix;
  p.total_tiles = prefix * batch * heads;
  set_dispatch(p);
  if (validate_only) return ok();
  if (fuse != nullptr) {
    p.lin = fuse->lin;
    p.lin_ss = fuse->ss;
    p.gate_lin = fuse->gate_lin;
    p.lin_w = fuse->weight;
    p.lin_eps = fuse->eps;
  }

  const int rc = vdn::launch_fwd(p, head_dim, dtype, hip_stream);
  if (rc != 0)
    return fail(VDN_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(hipError_t(rc)));
  return ok();
}

int vdn_local_attn_fwd(const void* q, const void* k, const void* v, const float* gate, void* out,
                       int F, int tokens_per_frame, int n_text, int block_frames, int heads,
                       int head_dim, int dtype, int batch, const float* qkv_scales,
                       float softmax_scale, float* lse, void* hip_stream) {
  return local_attn_fwd_impl(q, k, v, gate, out, F, tokens_per_frame, n_text, block_frames, heads,
                             head_dim, dtype, batch, qkv_scales, softmax_scale, lse, hip_stream,
                             nullptr);
}

// The backward pass; with `fixed_scratch` the per-row constants go to the
// library's static device array instead of the caller's workspace.
static int local_attn_bwd_impl(const void* q, const void* k, const void* v, const float* gate,
                               const void* out, const void* dout, const float* lse, void* dq,
                               void* dk, void* dv, float* dgate, int F, int tokens_per_frame,
                               int n_text, int block_frames, int heads, int head_dim, int batch,
                               float softmax_scale, float* workspace, bool fixed_scratch,
                               void* hip_stream) {
  vdn::Geometry g;
  std::string err;
  if (!vdn::make_geometry(F, tokens_per_frame, n_text, block_frames, &g, &err))
    return fail(VDN_ERR_INVALID_ARG, err);
  if (heads <= 0 || batch <= 0)
    return fail(VDN_ERR_INVALID_ARG, "heads and batch must be >= 1");
  const void* need[] = {q, k, v, out, dout, lse, dq, dk, dv, fixed_scratch ? q : workspace};
  for (const void* x : need)
    if (x == nullptr)
      return fail(VDN_ERR_INVALID_ARG, "q, k, v, out, dout, lse, dq, dk, dv and workspace must be non-NULL");
  if ((gate == nullptr) != (dgate == nullptr))
    return fail(VDN_ERR_INVALID_ARG, "dgate must be given exactly when gate is");
  if (head_dim != 64 && head_dim != 128)
    return fail(VDN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got " + std::to_string(head_dim) + ")");
  if (!std::isfinite(softmax_scale))
    return fail(VDN_ERR_INVALID_ARG, "softmax_scale is not finite");
  const void* a16[] = {q, k, v, out, dout, dq, dk, dv};
  for (const void* x : a16)
    if (!aligned(x, 16)) return fail(VDN_ERR_ALIGNMENT, "q, k, v, out, dout, dq, dk and dv must be 16-byte aligned");
  if (!aligned(gate, 4) || !aligned(lse, 4) || !aligned(dgate, 4) || !aligned(workspace, 4))
    return fail(VDN_ERR_ALIGNMENT, "gate, lse, dgate and workspace must be 4-byte aligned");
  if (g.S > INT32_MAX / 2)
    return fail(VDN_ERR_OVERFLOW, "sequence length " + std::to_string(g.S) + " too large");
  const int64_t elems = int64_t(batch) * g.S * int64_t(heads) * int64_t(head_dim);
  if (elems / batch / heads / head_dim != g.S || elems > (int64_t(1) << 46))
    return fail(VDN_ERR_OVERFLOW, "tensor element count overflows");
  if (int64_t(batch) * heads > INT32_MAX / 4096)
    return fail(VDN_ERR_OVERFLOW, "batch * heads too large");
  if (!dma_offsets_fit(heads, head_dim, 2))
    return fail(VDN_ERR_OVERFLOW, "128 token strides of heads * head_dim elements exceed 2^32 bytes");

  if (fixed_scratch && 2 * int64_t(batch) * heads * g.S > vdn::kBwdScratchFloats)
    return fail(VDN_ERR_CAPACITY, "batch * heads * S = " + std::to_string(int64_t(batch) * heads * g.S) +
                                      " rows exceed the fixed scratch's " +
                                      std::to_string(vdn::kBwdScratchFloats / 2));

  const size_t t_bytes = size_t(elems) * 2u;
  const size_t row_bytes = size_t(batch) * size_t(g.S) * size_t(heads) * 4u;
  const void* ins[] = {q, k, v, out, dout, lse, gate};
  const size_t in_sz[] = {t_bytes, t_bytes, t_bytes, t_bytes, t_bytes, row_bytes, gate ? row_bytes : 0u};
  const void* outs[] = {dq, dk, dv, dgate, workspace};
  const size_t out_sz[] = {t_bytes, t_bytes, t_bytes, dgate ? row_bytes : 0u,
                           fixed_scratch ? 0u : 2 * row_bytes};
  for (int i = 0; i < 5; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlaps(outs[i], out_sz[i], ins[j], in_sz[j]))
        return fail(VDN_ERR_INVALID_ARG, "an output or the workspace overlaps an input");
    for (int j = i + 1; j < 5; ++j)
      if (overlaps(outs[i], out_sz[i], outs[j], out_sz[j]))
        return fail(VDN_ERR_INVALID_ARG, "outputs and workspace must not overlap each other");
  }

  const auto qblocks = vdn::build_query_blocks(g);
  const auto kblocks = vdn::build_key_blocks(g);
  if (int(qblocks.size()) > vdn::kMaxQueryBlocks || int(kblocks.size()) > vdn::kMaxQueryBlocks)
    return fail(VDN_ERR_UNSUPPORTED, "more than " + std::to_string(vdn::kMaxQueryBlocks) + " query blocks");

  vdn::BwdDqParams dq_p;
  vdn::BwdKvParams kv_p;
  std::memset(&dq_p, 0, sizeof(dq_p));
  std::memset(&kv_p, 0, sizeof(kv_p));
  vdn::BwdArgs& a = dq_p.a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.dout = dout;
  a.gate = gate;
  a.lse = lse;
  a.dw = workspace;  // (the fixed scratch's address is filled in after validation)
  a.lw = workspace != nullptr ? workspace + size_t(batch) * size_t(heads) * size_t(g.S) : nullptr;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dgate = dgate;
  a.B = batch;
  a.S = int32_t(g.S);
  a.H = heads;
  const float sm = softmax_scale > 0.f ? softmax_scale : float(1.0 / std::sqrt(double(head_dim)));
  a.scale = sm;
  a.score_scale_log2 = float(double(sm) * 1.4426950408889634);
  kv_p.a = a;

  // dQ: query tiles, longest key list first
  const int tile_m = vdn::bwd_dq_tile_m();
  int prefix = 0, n = 0;
  for (int bi : vdn::cost_order(qblocks)) {
    const vdn::QueryBlock& qb = qblocks[size_t(bi)];
    vdn::QBlockDesc& d = dq_p.blk[n++];
    d.row_lo = int32_t(qb.row_lo);
    d.rows = int32_t(qb.row_hi - qb.row_lo);
    d.n_keys = int32_t(qb.n_keys);
    d.tile_prefix = prefix;
    d.n_iv = qb.n_iv;
    int64_t start = 0;
    for (int i = 0; i < qb.n_iv; ++i) {
      d.iv_start[i] = int32_t(start);
      d.iv_delta[i] = int32_t(qb.iv[i].lo - start);
      start += qb.iv[i].hi - qb.iv[i].lo;
    }
    prefix += (d.rows + tile_m - 1) / tile_m;
  }
  dq_p.n_blocks = n;
  dq_p.tiles_per_bh = prefix;
  dq_p.total_tiles = prefix * batch * heads;
  set_dispatch(dq_p);

  // dK/dV: key tiles, most query rows first
  const int tile_n = vdn::bwd_dkv_tile_n();
  std::vector<int> korder(kblocks.size());
  for (size_t i = 0; i < korder.size(); ++i) korder[i] = int(i);
  std::stable_sort(korder.begin(), korder.end(), [&](int x, int y) {
    return kblocks[size_t(x)].n_rows > kblocks[size_t(y)].n_rows;
  });
  prefix = 0;
  n = 0;
  for (int ki : korder) {
    const vdn::KeyBlock& kb = kblocks[size_t(ki)];
    vdn::KBlockDesc& d = kv_p.blk[n++];
    d.n_keys = int32_t(kb.n_keys);
    d.n_rows = int32_t(kb.n_rows);
    d.tile_prefix = prefix;
    int64_t start = 0;
    d.kiv_start[0] = d.kiv_start[1] = d.n_keys;
    for (int i = 0; i < kb.n_kiv; ++i) {
      if (i > 0) d.kiv_start[i - 1] = int32_t(start);
      d.kiv_delta[i] = int32_t(kb.kiv[i].lo - start);
      start += kb.kiv[i].hi - kb.kiv[i].lo;
    }
    start = 0;
    d.qiv_start = d.n_rows;
    for (int i = 0; i < kb.n_qiv; ++i) {
      if (i > 0) d.qiv_start = int32_t(start);
      d.qiv_delta[i] = int32_t(kb.qiv[i].lo - start);
      start += kb.qiv[i].hi - kb.qiv[i].lo;
    }
    prefix += (d.n_keys + tile_n - 1) / tile_n;
  }
  kv_p.n_blocks = n;
  kv_p.tiles_per_bh = prefix;
  kv_p.total_tiles = prefix * batch * heads;
  set_dispatch(kv_p);

  if (fixed_scratch) {
    float* ws = nullptr;
    const int se = vdn::bwd_scratch(&ws);
    if (se != 0)
      return fail(VDN_ERR_HIP, std::string("fixed scratch address: ") + hipGetErrorString(hipError_t(se)));
    for (vdn::BwdArgs* x : {&dq_p.a, &kv_p.a}) {
      x->dw = ws;
      x->lw = ws + size_t(batch) * size_t(heads) * size_t(g.S);
    }
  }
  const int rc = vdn::launch_bwd(dq_p, kv_p, head_dim, hip_stream);
  if (rc != 0)
    return fail(VDN_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(hipError_t(rc)));
  return ok();
}

int vdn_local_attn_bwd(const void* q, const void* k, const void* v, const float* gate,
                       const void* out, const void* dout, const float* lse, void* dq, void* dk,
                       void* dv, float* dgate, int F, int tokens_per_frame, int n_text,
                       int block_frames, int heads, int head_dim, int batch, float softmax_scale,
                       float* workspace, void* hip_stream) {
  return local_attn_bwd_impl(q, k, v, gate, out, dout, lse, dq, dk, dv, dgate, F, tokens_per_frame,
                             n_text, block_frames, heads, head_dim, batch, softmax_scale, workspace,
                             false, hip_stream);
}

int vdn_local_attn_bwd_noalloc(const void* q, const void* k, const void* v, const float* gate,
                               const void* out, const void* dout, const float* lse, void* dq,
                               void* dk, void* dv, float* dgate, int F, int tokens_per_frame,
                               int n_text, int block_frames, int heads, int head_dim, int batch,
                               float softmax_scale, void* hip_stream) {
  return local_attn_bwd_impl(q, k, v, gate, out, dout, lse, dq, dk, dv, dgate, F, tokens_per_frame,
                             n_text, block_frames, heads, head_dim, batch, softmax_scale, nullptr,
                             true, hip_stream);
}

int64_t vdn_linear_branch_workspace_bytes(int F, int tokens_per_frame, int n_text, int block_frames,
                                          int heads, int head_dim, int batch) {
  vdn::Geometry g;
  std::string err;
  if (!vdn::make_geometry(F, tokens_per_frame, n_text, block_frames, &g, &err))
    return fail(VDN_ERR_INVALID_ARG, err);
  if (heads <= 0 || batch <= 0) return fail(VDN_ERR_INVALID_ARG, "heads and batch must be >= 1");
  if (head_dim != 64 && head_dim != 128)
    return fail(VDN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got " + std::to_string(head_dim) + ")");
  if (int64_t(batch) * heads > 65535) return fail(VDN_ERR_OVERFLOW, "batch * heads above 65535");
  ok();
  return int64_t(vdn::linear_workspace(batch, heads, g.F, g.nb, head_dim).total);
}

static int linear_branch_fwd_impl(const void* q, const void* k, const void* v, void* out, int F,
                                  int tokens_per_frame, int n_text, int block_frames, int heads,
                                  int head_dim, int batch, void* workspace,
                                  int64_t workspace_bytes, void* hip_stream, float* row_ss) {
  const int64_t need = vdn_linear_branch_workspace_bytes(F, tokens_per_frame, n_text, block_frames,
                                                         heads, head_dim, batch);
  if (need < 0) return int(need);
  vdn::Geometry g;
  std::string err;
  vdn::make_geometry(F, tokens_per_frame, n_text, block_frames, &g, &err);
  const void* need_ptr[] = {q, k, v, out, workspace};
  for (const void* x : need_ptr)
    if (x == nullptr) return fail(VDN_ERR_INVALID_ARG, "q, k, v, out and workspace must be non-NULL");
  if (workspace_bytes < need)
    return fail(VDN_ERR_INVALID_ARG, "workspace of " + std::to_string(workspace_bytes) + " bytes, " +
                                         std::to_string(need) + " needed");
  const void* a16[] = {q, k, v, out};
  for (const void* x : a16)
    if (!aligned(x, 16)) return fail(VDN_ERR_ALIGNMENT, "q, k, v and out must be 16-byte aligned");
  if (!aligned(workspace, 256)) return fail(VDN_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  if (g.S > INT32_MAX / 2) return fail(VDN_ERR_OVERFLOW, "sequence length " + std::to_string(g.S) + " too large");
  const int64_t elems = int64_t(batch) * g.S * int64_t(heads) * int64_t(head_dim);
  if (elems / batch / heads / head_dim != g.S || elems > (int64_t(1) << 46))
    return fail(VDN_ERR_OVERFLOW, "tensor element count overflows");
  const size_t t_bytes = size_t(elems) * 2u;
  const void* ins[] = {q, k, v};
  for (const void* x : ins) {
    if (overlaps(out, t_bytes, x, t_bytes)) return fail(VDN_ERR_INVALID_ARG, "out overlaps an input");
    if (overlaps(workspace, size_t(need), x, t_bytes))
      return fail(VDN_ERR_INVALID_ARG, "the workspace overlaps an input");
  }
  if (overlaps(workspace, size_t(need), out, t_bytes))
    return fail(VDN_ERR_INVALID_ARG, "the workspace overlaps out");

  vdn::LinParams p;
  std::memset(&p, 0, sizeof(p));
  const vdn::LinWorkspace w = vdn::linear_workspace(batch, heads, g.F, g.nb, head_dim);
  char* ws = static_cast<char*>(workspace);
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.fstate = reinterpret_cast<float*>(ws + w.fstate_off);
  p.bstate = ws + w.bstate_off;
  p.bz = reinterpret_cast<float*>(ws + w.bz_off);
  p.B = batch;
  p.S = int32_t(g.S);
  p.H = heads;
  p.F = int32_t(g.F);
  p.T = int32_t(g.T);
  p.Bf = int32_t(g.Bf);
  p.nb = int32_t(g.nb);
  const int64_t rt = vdn::kLinRowTile;
  const int64_t full_rows = g.Bf * g.T;
  const int64_t last_rows = (g.F - (g.nb - 1) * g.Bf) * g.T;
  p.tiles_per_block = int32_t((full_rows + rt - 1) / rt);
  p.tiles_last = int32_t((last_rows + rt - 1) / rt);
  p.tiles_text = int32_t((g.N + rt - 1) / rt);
  const int64_t per_bh = int64_t(p.tiles_per_block) * (g.nb - 1) + p.tiles_last + p.tiles_text;
  const int64_t total = per_bh * batch * heads;
  if (total > INT32_MAX / 2) return fail(VDN_ERR_OVERFLOW, "too many row tiles");
  p.tiles_per_bh = int32_t(per_bh);
  p.total_tiles = int32_t(total);
  p.ss = row_ss;

  const int rc = vdn::launch_linear(p, head_dim, hip_stream);
  if (rc != 0)
    return fail(VDN_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(hipError_t(rc)));
  return ok();
}

int vdn_linear_branch_fwd(const void* q, const void* k, const void* v, void* out, int F,
                          int tokens_per_frame, int n_text, int block_frames, int heads,
                          int head_dim, int batch, void* workspace, int64_t workspace_bytes,
                          void* hip_stream) {
  return linear_branch_fwd_impl(q, k, v, out, F, tokens_per_frame, n_text, block_frames, heads,
                                head_dim, batch, workspace, workspace_bytes, hip_stream, nullptr);
}

int64_t vdn_hybrid_attn_workspace_bytes(int F, int tokens_per_frame, int n_text, int block_frames,
                                        int heads, int head_dim, int batch) {
  const int64_t lin = vdn_linear_branch_workspace_bytes(F, tokens_per_frame, n_text, block_frames,
                                                        heads, head_dim, batch);
  if (lin < 0) return lin;
  vdn::Geometry g;
  std::string err;
  vdn::make_geometry(F, tokens_per_frame, n_text, block_frames, &g, &err);
  const uint64_t rows = uint64_t(batch) * uint64_t(g.S) * uint64_t(heads);
  if (rows > (uint64_t(1) << 40) / uint64_t(head_dim)) return fail(VDN_ERR_OVERFLOW, "tensor element count overflows");
  ok();
  return int64_t(up256(uint64_t(lin)) + up256(rows * uint64_t(head_dim) * 2u) + up256(rows * 4u));
}

int vdn_hybrid_attn_fwd(const void* q, const void* k, const void* v, const float* gate,
                        const float* gate_lin, const float* norm_weight, float eps, void* out,
                        int F, int tokens_per_frame, int n_text, int block_frames, int heads,
                        int head_dim, int batch, float softmax_scale, float* lse, void* workspace,
                        int64_t workspace_bytes, void* hip_stream) {
  const int64_t need = vdn_hybrid_attn_workspace_bytes(F, tokens_per_frame, n_text, block_frames,
                                                       heads, head_dim, batch);
  if (need < 0) return int(need);
  const int64_t lin_need = vdn_linear_branch_workspace_bytes(F, tokens_per_frame, n_text,
                                                             block_frames, heads, head_dim, batch);
  vdn::Geometry g;
  std::string err;
  vdn::make_geometry(F, tokens_per_frame, n_text, block_frames, &g, &err);
  if (gate_lin == nullptr || norm_weight == nullptr || workspace == nullptr)
    return fail(VDN_ERR_INVALID_ARG, "gate_lin, norm_weight and workspace must be non-NULL");
  // eps > 0: a token whose linear row is all zeros (text, or a block with no
  // linear keys) would otherwise scale 0 by 1/sqrt(0)
  if (!std::isfinite(eps) || !(eps > 0.f)) return fail(VDN_ERR_INVALID_ARG, "eps must be finite and > 0");
  if (workspace_bytes < need)
    return fail(VDN_ERR_INVALID_ARG, "workspace of " + std::to_string(workspace_bytes) + " bytes, " +
                                         std::to_string(need) + " needed");
  if (!aligned(workspace, 256)) return fail(VDN_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  if (!aligned(norm_weight, 16)) return fail(VDN_ERR_ALIGNMENT, "norm_weight must be 16-byte aligned");
  if (!aligned(gate_lin, 4)) return fail(VDN_ERR_ALIGNMENT, "gate_lin must be 4-byte aligned");
  const uint64_t rows = uint64_t(batch) * uint64_t(g.S) * uint64_t(heads);
  const size_t t_bytes = size_t(rows) * size_t(head_dim) * 2u;
  const size_t g_bytes = size_t(rows) * 4u;
  const size_t w_bytes = size_t(heads) * size_t(head_dim) * 4u;
  const size_t l_bytes = size_t(rows) * 4u;
  struct Span {
    const void* p;
    size_t n;
  };
  const Span others[] = {{q, t_bytes}, {k, t_bytes}, {v, t_bytes}, {out, t_bytes}, {gate, g_bytes},
                         {gate_lin, g_bytes}, {norm_weight, w_bytes}, {lse, l_bytes}};
  for (const Span& x : others)
    if (x.p != nullptr && overlaps(workspace, size_t(need), x.p, x.n))
      return fail(VDN_ERR_INVALID_ARG, "the workspace overlaps an input or output");
  const Span fuse_in[] = {{gate_lin, g_bytes}, {norm_weight, w_bytes}};
  for (const Span& x : fuse_in)
    if (overlaps(out, t_bytes, x.p, x.n) || (lse != nullptr && overlaps(lse, l_bytes, x.p, x.n)))
      return fail(VDN_ERR_INVALID_ARG, "out or lse overlaps gate_lin or norm_weight");

  // the softmax branch's arguments are checked before the linear branch is
  // launched, so that a failing call launches nothing
  const FuseArgs probe{nullptr, nullptr, gate_lin, norm_weight, eps};
  int rc = local_attn_fwd_impl(q, k, v, gate, out, F, tokens_per_frame, n_text, block_frames, heads,
                               head_dim, VDN_BF16, batch, nullptr, softmax_scale, lse, hip_stream,
                               &probe, true);
  if (rc != 0) return rc;

  // workspace: the linear branch's own, then its output, then the per
  // (token, head) sums of squares of that output
  char* ws = static_cast<char*>(workspace);
  void* lin_out = ws + up256(uint64_t(lin_need));
  float* row_ss = reinterpret_cast<float*>(ws + up256(uint64_t(lin_need)) + up256(uint64_t(t_bytes)));
  rc = linear_branch_fwd_impl(q, k, v, lin_out, F, tokens_per_frame, n_text, block_frames, heads,
                              head_dim, batch, ws, lin_need, hip_stream, row_ss);
  if (rc != 0) return rc;
  const FuseArgs fuse{lin_out, row_ss, gate_lin, norm_weight, eps};
  return local_attn_fwd_impl(q, k, v, gate, out, F, tokens_per_frame, n_text, block_frames, heads,
                             head_dim, VDN_BF16, batch, nullptr, softmax_scale, lse, hip_stream, &fuse);
}

int vdn_hybrid_fuse(const void* soft_out, const void* lin_out, const float* gate_lin,
                    const float* norm_weight, float eps, void* out, int64_t tokens, int heads,
                    int head_dim, void* hip_stream) {
  if (tokens < 0 || heads <= 0 || head_dim <= 0)
    return fail(VDN_ERR_INVALID_ARG, "tokens must be >= 0, heads and head_dim >= 1");
  if (head_dim % 8 != 0)
    return fail(VDN_ERR_UNSUPPORTED, "head_dim must be a multiple of 8 (got " + std::to_string(head_dim) + ")");
  const int64_t hd = int64_t(heads) * head_dim;
  if (hd > 8192) return fail(VDN_ERR_UNSUPPORTED, "heads * head_dim above 8192");
  // eps > 0: a token whose linear row is all zeros (text, or a block with no
  // linear keys) would otherwise scale 0 by 1/sqrt(0)
  if (!std::isfinite(eps) || !(eps > 0.f)) return fail(VDN_ERR_INVALID_ARG, "eps must be finite and > 0");
  const void* need_ptr[] = {soft_out, lin_out, gate_lin, norm_weight, out};
  for (const void* x : need_ptr)
    if (x == nullptr)
      return fail(VDN_ERR_INVALID_ARG, "soft_out, lin_out, gate_lin, norm_weight and out must be non-NULL");
  const void* a16[] = {soft_out, lin_out, norm_weight, out};
  for (const void* x : a16)
    if (!aligned(x, 16))
      return fail(VDN_ERR_ALIGNMENT, "soft_out, lin_out, norm_weight and out must be 16-byte aligned");
  if (!aligned(gate_lin, 4)) return fail(VDN_ERR_ALIGNMENT, "gate_lin must be 4-byte aligned");
  if (tokens > (int64_t(1) << 40) / hd) return fail(VDN_ERR_OVERFLOW, "tokens * heads * head_dim too large");
  if (tokens > int64_t(INT32_MAX) * 4 - 4) return fail(VDN_ERR_OVERFLOW, "too many tokens");
  const size_t t_bytes = size_t(tokens * hd) * 2u;
  const size_t g_bytes = size_t(tokens) * size_t(heads) * 4u;
  const size_t w_bytes = size_t(hd) * 4u;
  if (out != soft_out && overlaps(out, t_bytes, soft_out, t_bytes))
    return fail(VDN_ERR_INVALID_ARG, "out overlaps soft_out without being the same buffer");
  if (overlaps(out, t_bytes, lin_out, t_bytes) || overlaps(out, t_bytes, gate_lin, g_bytes) ||
      overlaps(out, t_bytes, norm_weight, w_bytes))
    return fail(VDN_ERR_INVALID_ARG, "out overlaps lin_out, gate_lin or norm_weight");
  if (tokens == 0) return ok();

  vdn::FuseParams p;
  p.soft = soft_out;
  p.lin = lin_out;
  p.gate = gate_lin;
  p.weight = norm_weight;
  p.out = out;
  p.rows = tokens;
  p.H = heads;
  p.D = head_dim;
  p.HD = int32_t(hd);
  p.eps = eps;
  const int rc = vdn::launch_fuse(p, hip_stream);
  if (rc != 0)
    return fail(VDN_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(hipError_t(rc)));
  return ok();
}

}  // extern "C"
