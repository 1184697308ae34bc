// Host-side key-structure scheduler for the local-window attention forward.
//
// Builds, from (F, T, N, block_frames) alone, each query block's canonical key
// intervals and the query-tile work list.  The rule it encodes (openi.cn
// "VDN-MiniMax-H3", technical principles; nav.superapi.store "VDN-MiniMax-H3
// - OpenVDN's Open-Source Video Generation Acceleration Solution", Technical
// Principles, "Local Softmax Branch" and "Text Dual-Branch Injection"):
// 5-frame blocks see themselves and both neighbouring blocks, frames 0 and
// F-1 are anchor keys for every query, text keys are visible to all, text
// queries see everything.  Pure C++17, no HIP.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace vdn {

constexpr int kMaxIntervals = 3;  // [0,T), the window, [(F-1)T, S)

struct Geometry {
  int64_t F = 0, T = 0, N = 0, Bf = 0;
  int64_t V = 0;   // video tokens F*T
  int64_t S = 0;   // all tokens
  int64_t nb = 0;  // frame blocks
};

struct Interval {
  int64_t lo, hi;  // half-open token range
};

struct QueryBlock {
  int64_t row_lo = 0, row_hi = 0;  // query tokens [row_lo, row_hi)
  int n_iv = 0;
  Interval iv[kMaxIntervals];
  int64_t n_keys = 0;              // sum of interval lengths
};

struct Tile {
  int32_t qblock, row0, rows, keys;
};

// Validates and fills the geometry; returns false with a message on error.
bool make_geometry(int F, int T, int N, int Bf, Geometry* g, std::string* err);

// Query blocks in index order: frame blocks 0..nb-1, then text (if N > 0).
std::vector<QueryBlock> build_query_blocks(const Geometry& g);

// Allowed pairs and anchor-added pairs per (sample, head).
void count_pairs(const Geometry& g, int64_t* allowed, int64_t* anchor_added);

// Block indices sorted by key count, largest first (stable by index).
std::vector<int> cost_order(const std::vector<QueryBlock>& blocks);

// Per-(sample, head) tile list in launch order.
std::vector<Tile> tile_schedule(const std::vector<QueryBlock>& blocks, int tile_m);

// The key side of the structure (gradients of the keys and values): a group
// of keys seen by exactly the same query rows.  Keys of a frame block that
// are not anchor frames are seen by the video rows of the block and its two
// neighbours and by the text rows; anchor-frame keys and text keys are seen
// by every row.
struct KeyBlock {
  int n_kiv = 0;
  Interval kiv[kMaxIntervals];  // key tokens (canonical)
  int64_t n_keys = 0;
  int n_qiv = 0;
  Interval qiv[kMaxIntervals];  // query rows that see them (canonical)
  int64_t n_rows = 0;
};

// Key groups: frame blocks by index (their non-anchor frames; skipped when
// empty), then the anchor and text keys (skipped when empty).
std::vector<KeyBlock> build_key_blocks(const Geometry& g);

}  // namespace vdn
