// Host-side key-structure scheduler (see schedule.hpp for the rule).
#include "schedule.hpp"

#include <algorithm>
#include <climits>

namespace vdn {

bool make_geometry(int F, int T, int N, int Bf, Geometry* g, std::string* err) {
  if (F <= 0 || T <= 0 || Bf <= 0 || N < 0) {
    *err = "F, tokens_per_frame and block_frames must be >= 1 and n_text >= 0 (got F=" +
           std::to_string(F) + ", T=" + std::to_string(T) + ", n_text=" + std::to_string(N) +
           ", block_frames=" + std::to_string(Bf) + ")";
    return false;
  }
  g->F = F;
  g->T = T;
  g->N = N;
  g->Bf = Bf;
  g->V = int64_t(F) * int64_t(T);
  g->S = g->V + N;
  g->nb = (int64_t(F) + Bf - 1) / Bf;
  return true;
}

// Key intervals of frame block `beta`.  Built in token order: the first
// anchor frame (when the window does not start at frame 0), the window, then
// the last anchor frame (when the window stops short of it) followed by the
// text tokens.  Pieces that touch are joined.
static void video_block_intervals(const Geometry& g, int64_t beta, QueryBlock* qb) {
  const int64_t lo = g.Bf * std::max<int64_t>(0, beta - 1);
  const int64_t hi = std::min<int64_t>(g.F, g.Bf * (beta + 2));
  Interval pieces[4];
  int n = 0;
  if (lo > 0) pieces[n++] = {0, g.T};
  pieces[n++] = {lo * g.T, hi * g.T};
  if (hi < g.F) pieces[n++] = {(g.F - 1) * g.T, g.F * g.T};
  if (g.N > 0) pieces[n++] = {g.V, g.S};
  qb->n_iv = 0;
  for (int i = 0; i < n; ++i) {
    if (qb->n_iv > 0 && pieces[i].lo <= qb->iv[qb->n_iv - 1].hi) {
      qb->iv[qb->n_iv - 1].hi = std::max(qb->iv[qb->n_iv - 1].hi, pieces[i].hi);
    } else {
      qb->iv[qb->n_iv++] = pieces[i];
    }
  }
  qb->n_keys = 0;
  for (int i = 0; i < qb->n_iv; ++i) qb->n_keys += qb->iv[i].hi - qb->iv[i].lo;
}

std::vector<QueryBlock> build_query_blocks(const Geometry& g) {
  std::vector<QueryBlock> out;
  out.reserve(size_t(g.nb) + 1);
  for (int64_t beta = 0; beta < g.nb; ++beta) {
    QueryBlock qb;
    qb.row_lo = beta * g.Bf * g.T;
    qb.row_hi = std::min(g.F, (beta + 1) * g.Bf) * g.T;
    video_block_intervals(g, beta, &qb);
    out.push_back(qb);
  }
  if (g.N > 0) {
    QueryBlock qb;
    qb.row_lo = g.V;
    qb.row_hi = g.S;
    qb.n_iv = 1;
    qb.iv[0] = {0, g.S};
    qb.n_keys = g.S;
    out.push_back(qb);
  }
  return out;
}

void count_pairs(const Geometry& g, int64_t* allowed, int64_t* anchor_added) {
  int64_t a = 0, x = 0;
  for (int64_t beta = 0; beta < g.nb; ++beta) {
    const int64_t lo = g.Bf * std::max<int64_t>(0, beta - 1);
    const int64_t hi = std::min<int64_t>(g.F, g.Bf * (beta + 2));
    const int64_t rows = (std::min(g.F, (beta + 1) * g.Bf) - beta * g.Bf) * g.T;
    const int64_t anchors = int64_t(lo > 0) + int64_t(hi < g.F);
    a += rows * (g.T * (hi - lo + anchors) + g.N);
    x += rows * g.T * anchors;
  }
  a += g.N * g.S;
  *allowed = a;
  *anchor_added = x;
}

std::vector<int> cost_order(const std::vector<QueryBlock>& blocks) {
  std::vector<int> order(blocks.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = int(i);
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) {
    return blocks[size_t(x)].n_keys > blocks[size_t(y)].n_keys;
  });
  return order;
}

std::vector<Tile> tile_schedule(const std::vector<QueryBlock>& blocks, int tile_m) {
  std::vector<Tile> out;
  for (int i : cost_order(blocks)) {
    const QueryBlock& qb = blocks[size_t(i)];
    for (int64_t r = qb.row_lo; r < qb.row_hi; r += tile_m) {
      Tile t;
      t.qblock = i;
      t.row0 = int32_t(r);
      t.rows = int32_t(std::min<int64_t>(tile_m, qb.row_hi - r));
      t.keys = int32_t(qb.n_keys);
      out.push_back(t);
    }
  }
  return out;
}

// Appends [lo, hi) to a canonical list being built in increasing order,
// joining it with the previous interval when they touch.
static void push_interval(Interval* iv, int* n, int64_t lo, int64_t hi) {
  if (hi <= lo) return;
  if (*n > 0 && lo <= iv[*n - 1].hi) {
    iv[*n - 1].hi = std::max(iv[*n - 1].hi, hi);
  } else {
    iv[(*n)++] = {lo, hi};
  }
}

std::vector<KeyBlock> build_key_blocks(const Geometry& g) {
  std::vector<KeyBlock> out;
  for (int64_t beta = 0; beta < g.nb; ++beta) {
    // non-anchor frames of the block form one contiguous range: the anchors
    // 0 and F-1 can only be its first or last frame
    int64_t f0 = beta * g.Bf, f1 = std::min(g.F, (beta + 1) * g.Bf);
    if (f0 == 0) f0 = 1;
    if (f1 == g.F) f1 = g.F - 1;
    if (f1 <= f0) continue;
    KeyBlock kb;
    push_interval(kb.kiv, &kb.n_kiv, f0 * g.T, f1 * g.T);
    kb.n_keys = (f1 - f0) * g.T;
    const int64_t lo = g.Bf * std::max<int64_t>(0, beta - 1);
    const int64_t hi = std::min<int64_t>(g.F, g.Bf * (beta + 2));
    push_interval(kb.qiv, &kb.n_qiv, lo * g.T, hi * g.T);
    push_interval(kb.qiv, &kb.n_qiv, g.V, g.S);
    kb.n_rows = 0;
    for (int i = 0; i < kb.n_qiv; ++i) kb.n_rows += kb.qiv[i].hi - kb.qiv[i].lo;
    out.push_back(kb);
  }
  KeyBlock gk;
  push_interval(gk.kiv, &gk.n_kiv, 0, g.T);
  if (g.F > 1) push_interval(gk.kiv, &gk.n_kiv, (g.F - 1) * g.T, g.V);
  push_interval(gk.kiv, &gk.n_kiv, g.V, g.S);
  gk.n_keys = 0;
  for (int i = 0; i < gk.n_kiv; ++i) gk.n_keys += gk.kiv[i].hi - gk.kiv[i].lo;
  if (gk.n_keys > 0) {
    push_interval(gk.qiv, &gk.n_qiv, 0, g.S);
    gk.n_rows = g.S;
    out.push_back(gk);
  }
  return out;
}

}  // namespace vdn
