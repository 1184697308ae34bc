// Backward pass of the local-window attention for gfx950, bf16 inputs.
//
// Gradients of the forward (local Softmax branch of VDN-H3 attention:
// frame-block window, first/last-frame anchors, global text keys, per-token
// sigmoid gate; openi.cn "VDN-MiniMax-H3", technical principles;
// nav.superapi.store "VDN-MiniMax-H3 - OpenVDN's Open-Source Video Generation
// Acceleration Solution", Technical Principles and training stages, where
// adapters on the attention projections are trained through this branch).
// With p_ij = exp(scale q_i.k_j - lse_i) over the key set, sg_i = sigmoid of
// the gate logit and out_i = sg_i sum_j p_ij v_j:
//   delta_i = sum_d dout_i out_i        (the gate cancels: dout.a sg = dout.out)
//   dgate_i = delta_i (1 - sg_i)
//   dp_ij   = dout_i . v_j
//   ds_ij   = p_ij (sg_i dp_ij - delta_i)
//   dq_i    = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,
//   dv_j    = sum_i sg_i p_ij dout_i.
// The gate folds into two per-row constants, lw_i = lse_i log2(e) - log2(sg_i)
// and dw_i = delta_i / sg_i, so that sg_i p_ij = exp2(scale log2(e) q_i.k_j -
// lw_i) and ds_ij = sg_i p_ij (dp_ij - dw_i): one exponential per pair yields
// the dV weight directly.
// Three kernels: a per-row pass (delta, dgate, lw, dw), dQ over query tiles
// with the keys streaming through LDS (the forward's schedule), and dK/dV over
// key tiles with the query rows streaming through LDS.
//
// Both tiled kernels read one LDS tile in two ways: as MFMA row operands
// (ds_read_b128 of 16-byte chunks) and transposed (ds_read_b64_tr_b16).  The
// swizzle stores chunk c of row r at c ^ (4 (r % 4) + (r / 4) % 4): sixteen
// consecutive rows put one logical chunk on sixteen distinct chunks, and four
// consecutive rows (a transposing read) spread four logical chunks over
// sixteen.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "fwd_common.hpp"

namespace vdn {

namespace {

// Per-row pass: D/8 lanes per (sample, token, head) row, 16 bytes of out and
// dout each, so one load instruction covers whole rows; the dot product is
// reduced across the row's lanes and its first lane writes the results.
template <int D>
__global__ __launch_bounds__(256) void bwd_rows_kernel(const BwdArgs a, int64_t total) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int LPR = D / 8;  // lanes per row (a power of two dividing 64)
  const int64_t idx = (int64_t(blockIdx.x) * 256 + threadIdx.x) / LPR;  // ((b * S) + i) * H + h
  const int c = int(threadIdx.x) % LPR;
  const bool live = idx < total;
  float acc = 0.f;
  if (live) {
    const bf16x8 x = reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.out) + idx * D)[c];
    const bf16x8 y = reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.dout) + idx * D)[c];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(float(x[e]), float(y[e]), acc);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (!live || c != 0) return;
  const int h = int(idx % a.H);
  const int64_t bi = idx / a.H;
  const int i = int(bi % a.S);
  const int b = int(bi / a.S);
  float sgv = 1.f;
  if (a.gate != nullptr) {
    sgv = 1.f / (1.f + __builtin_amdgcn_exp2f(-a.gate[idx] * kLog2e));
    a.dgate[idx] = acc * (1.f - sgv);
  }
  const int64_t r = (int64_t(b) * a.H + h) * a.S + i;
  // the gate folded into the row's constants: sg p = exp2(S c - lw) and
  // ds = sg p (dp - dw); a gate that rounds to 0 gives lw = +inf (weights 0)
  a.lw[r] = a.lse[r] * kLog2e - __log2f(sgv);
  a.dw[r] = sgv > 0.f ? acc / sgv : 0.f;
#endif
}

}  // namespace

// ---------------------------------------------------------------------------
// dQ: one workgroup = NW waves x 32 query rows of one (sample, head, query
// block), keys in steps of KT through an NS-stage LDS ring (as the forward).
// Per step, in the transposed score layout (one query per lane):
//   S^T  = K Q^T        (A = K rows from LDS, B = Q in registers)
//   dP^T = V dO^T       (A = V rows from LDS, B = dO in registers)
//   dS^T = W (dP - dw) scale, W = sg P = exp2(S c - lw)
//   dQ^T += K^T dS^T    (A = K^T by transposing reads, B = dS^T packed to bf16)
template <int D, int NW, int KT, int NS>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_kernel(const BwdDqParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int QW = 32;
  constexpr int M = NW * QW;
  constexpr int RB = 2 * D;
  constexpr int CH = D / 8;
  constexpr int TILE = KT * RB;
  constexpr int NI = TILE / 1024 / NW;
  constexpr int RPI = 1024 / RB;
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NKB = KT / 32;
  static_assert(NI >= 1 && NI * NW * 1024 == TILE, "tile shape");
  static_assert(NS == 2 || NS == 3, "two or three stages");
  const BwdArgs& a = p.a;

  // one array per stage (the third is a single byte when unused)
  __shared__ __attribute__((aligned(1024))) char Ks0[TILE];
  __shared__ __attribute__((aligned(1024))) char Ks1[TILE];
  __shared__ __attribute__((aligned(1024))) char Ks2[NS > 2 ? TILE : 1];
  __shared__ __attribute__((aligned(1024))) char Vs0[TILE];
  __shared__ __attribute__((aligned(1024))) char Vs1[TILE];
  __shared__ __attribute__((aligned(1024))) char Vs2[NS > 2 ? TILE : 1];
  auto kstage = [&](auto st) -> char* {
    constexpr int i = decltype(st)::value;
    return i == 0 ? Ks0 : i == 1 ? Ks1 : Ks2;
  };
  auto vstage = [&](auto st) -> char* {
    constexpr int i = decltype(st)::value;
    return i == 0 ? Vs0 : i == 1 ? Vs1 : Vs2;
  };

  const TileSlot slot = tile_slot(blockIdx.x, p.per_xcd, p.split_tail);
  const int t = slot.tile;
  if (t >= p.total_tiles) return;
  const int bh = t / p.tiles_per_bh;
  const int rank = undeal(t - bh * p.tiles_per_bh, p.tiles_per_bh, p.deal);
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  int bi = 0;
  while (bi + 1 < p.n_blocks && p.blk[bi + 1].tile_prefix <= rank) ++bi;
  const KeyList kl = load_key_list(p.blk[bi]);
  int row0 = p.blk[bi].row_lo + (rank - p.blk[bi].tile_prefix) * M;
  int rows = min(M, p.blk[bi].row_lo + p.blk[bi].rows - row0);
  if (slot.half != 0) {
    const int off = (slot.half - 1) * (M / 2);
    row0 += off;
    rows = min(M / 2, rows - off);
    if (rows <= 0) return;  // a tile of at most M/2 rows has no second half
  }
  const int n_keys = kl.n_keys;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int lr = lane & 31;
  const int hh = lane >> 5;

  const int64_t rs = int64_t(a.H) * D;
  const int64_t rsb = rs * 2;
  const int64_t bh_off = int64_t(b) * a.S * rs + int64_t(h) * D;
  const char* __restrict__ kg = reinterpret_cast<const char*>(static_cast<const __bf16*>(a.k) + bh_off);
  const char* __restrict__ vg = reinterpret_cast<const char*>(static_cast<const __bf16*>(a.v) + bh_off);

  // Q and dO rows of this wave (MFMA B operands), and the row's constants
  const int lrow = wave * QW + lr;
  const bool row_ok = lrow < rows;
  bf16x8 qreg[NDS], oreg[NDS];
  {
    const int64_t off = bh_off + int64_t(row0 + lrow) * rs + hh * 8;
    const __bf16* qs = static_cast<const __bf16*>(a.q) + off;
    const __bf16* os = static_cast<const __bf16*>(a.dout) + off;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      qreg[ds] = row_ok ? *reinterpret_cast<const bf16x8*>(qs + ds * 16) : bf16x8{};
      oreg[ds] = row_ok ? *reinterpret_cast<const bf16x8*>(os + ds * 16) : bf16x8{};
    }
  }
  // sg P = exp2(S c - L) with L = lw; rows past the tile get L = +inf (P = 0)
  float L = __builtin_inff(), dls = 0.f;
  const float sgs = a.scale;
  if (row_ok) {
    const int64_t r = (int64_t(b) * a.H + h) * a.S + row0 + lrow;
    L = a.lw[r];
    dls = a.dw[r] * a.scale;
  }
  // these loads complete before any DMA is issued: the compiler cannot count
  // the DMA, and with loads of its own still pending at the loop it would
  // wait on the DMA ring inside every step
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  // DMA of K and V rows (swizzled), as in the forward
  int dma_row[NI];
  uint32_t goff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int q = wave * NI + i;
    const int r = q * RPI + lane / CH;
    const int pc = lane % CH;
    dma_row[i] = r;
    goff[i] = uint32_t(r * rsb + ((pc ^ dual_swz<CH>(r)) * 16));
  }
  auto issue = [&](int step, char* lbase, const char* gbase) {
    const int j0 = step * KT;
    const int iv_end = interval_end(kl, j0);
    const int delta = interval_delta(kl, j0);
    if (j0 + KT <= iv_end) {
      const char* base = gbase + int64_t(j0 + delta) * rsb;
#pragma unroll
      for (int i = 0; i < NI; ++i) lds_dma16(base, goff[i], lbase + (wave * NI + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int j = min(j0 + dma_row[i], n_keys - 1);
        lds_dma16(gbase + int64_t(vtoken(kl, j)) * rsb + (goff[i] - uint32_t(dma_row[i] * rsb)),
                  lbase + (wave * NI + i) * 1024);
      }
    }
  };

  // row-operand offsets: row lr (+32 kb), logical chunk 2 ds + hh
  const uint32_t row_off0 = uint32_t(lr * RB + ((hh ^ dual_swz<CH>(lr)) * 16));
  auto row_off = [&](int ds) { return row_off0 ^ uint32_t(32 * ds); };
  // transposed-operand offsets: row 4 hh + i/4 (+ 8 for the second read),
  // columns 32 db + 16 (g % 2) + 4 (i % 4); db XORs bits 6.. of the offset
  uint32_t tr_off0[2];
  {
    const int g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int row = 4 * hh + (i >> 2) + 8 * rr;
      const int col = 16 * (g & 1) + 4 * (i & 3);
      tr_off0[rr] = uint32_t(row * RB + (((col >> 3) ^ dual_swz<CH>(row)) * 16) + (col & 7) * 2);
    }
  }

  const float c = a.score_scale_log2;
  const int nsteps = (n_keys + KT - 1) / KT;
  const bool active = __builtin_amdgcn_readfirstlane(wave) * QW < rows;

  // X^T = rows(X stage) * B^T for the KT keys of a stage (X = K or V)
  auto rowprod = [&](const char* xs, const bf16x8 (&breg)[NDS], f32x16 (&s)[NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(xs + kb * 32 * RB + row_off(ds));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, breg[ds], s[kb], 0, 0, 0);
      }
    }
  };

  // per step: the K and V of step + NS - 1 are issued into the stage freed
  // by the previous step, and the step's own stage is read
  auto body = [&](int step, auto st) {
    constexpr int s_ = decltype(st)::value;
    issue(step + NS - 1, kstage(IC<(s_ + NS - 1) % NS>{}), kg);
    issue(step + NS - 1, vstage(IC<(s_ + NS - 1) % NS>{}), vg);
    if (active) {
      const char* ks = kstage(st);
      f32x16 sc[NKB], dp[NKB];
      rowprod(ks, qreg, sc);
      rowprod(vstage(st), oreg, dp);
      const int j0 = step * KT;
      if (j0 + KT > n_keys) mask_tail<NKB>(sc, n_keys - j0, hh);
      bf16x8 pk[NKB][2];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8 v8;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = half * 8 + e;
            const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r], c, -L));
            v8[e] = static_cast<__bf16>(pr * __builtin_fmaf(sgs, dp[kb][r], -dls));
          }
          pk[kb][half] = v8;
        }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const char* base = ks + (kb * 32 + half * 16) * RB;
            const bf16x8 x = tr_frag(base + (tr_off0[0] ^ uint32_t(64 * db)), base + (tr_off0[1] ^ uint32_t(64 * db)));
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, pk[kb][half], acc[db], 0, 0, 0);
          }
    }
    // the next step reads stage step + 1; the batches of steps step + 2 ..
    // step + NS - 1 may still be in flight
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * 2 * NI));
    lds_barrier();
  };

  // prologue: steps 0 .. NS - 2 in flight (past the key list's end a step
  // re-fetches its last key, so every step issues the same batch)
  issue(0, Ks0, kg);
  issue(0, Vs0, vg);
  if constexpr (NS > 2) {
    issue(1, Ks1, kg);
    issue(1, Vs1, vg);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * 2 * NI));
  lds_barrier();
  for (int step = 0;;) {
    body(step, IC<0>{});
    if (++step >= nsteps) break;
    body(step, IC<1 % NS>{});
    if (++step >= nsteps) break;
    if constexpr (NS > 2) {
      body(step, IC<2 % NS>{});
      if (++step >= nsteps) break;
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no DMA outlives the workgroup

  if (row_ok) {
    __bf16* dst = static_cast<__bf16*>(a.dq) + bh_off + int64_t(row0 + lrow) * rs;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 o4;
#pragma unroll
        for (int r = 0; r < 4; ++r) o4[r] = static_cast<__bf16>(acc[db][g4 * 4 + r]);
        *reinterpret_cast<bf16x4*>(dst + db * 32 + g4 * 8 + hh * 4) = o4;
      }
  }
#endif
}

// ---------------------------------------------------------------------------
// dK / dV: one workgroup = NW waves x 32 keys of one (sample, head, key
// group); the query rows that see the group stream through a 2-stage LDS ring
// in steps of QT rows.  Per 32-row block of a step, in the score layout (one
// key per lane):
//   S  = Q K^T      (A = Q rows from LDS, B = K in registers)
//   dP = dO V^T     (A = dO rows from LDS, B = V rows from the LDS key tile)
//   W = sg P = exp2(S c - lw), dS = W (dP - dw)
//   dV^T += dO^T W,  dK^T += Q^T dS  (A by transposing reads; B packed)
// V of the workgroup's keys stays in LDS for the whole tile (read as B
// operands), which keeps a wave within 256 registers: two waves per SIMD.
template <int D, int NW, int QT>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dkv_kernel(const BwdKvParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int KW = 32;          // keys per wave
  constexpr int N = NW * KW;      // keys per workgroup
  constexpr int RB = 2 * D;
  constexpr int CH = D / 8;
  constexpr int TILE = QT * RB;   // bytes per Q (or dO) stage
  constexpr int NI = TILE / 1024 / NW;
  constexpr int RPI = 1024 / RB;
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NQB = QT / 32;    // 32-row blocks per step
  constexpr int NVI = KW * RB / 1024;  // DMA instructions per wave for its V rows
  static_assert(NI >= 1 && NI * NW * 1024 == TILE, "tile shape");
  static_assert(NW >= 2 && QT <= 64, "two waves stage the per-row constants, one row per lane");
  const BwdArgs& a = p.a;

  __shared__ __attribute__((aligned(1024))) char Qs0[TILE];
  __shared__ __attribute__((aligned(1024))) char Qs1[TILE];
  __shared__ __attribute__((aligned(1024))) char Os0[TILE];
  __shared__ __attribute__((aligned(1024))) char Os1[TILE];
  __shared__ __attribute__((aligned(1024))) char Vt[N * RB];   // V rows of the tile's keys
  __shared__ __attribute__((aligned(16))) float Rs[2][2][QT];  // per stage: lw, dw
  auto qstage = [&](auto st) -> char* { return decltype(st)::value == 0 ? Qs0 : Qs1; };
  auto ostage = [&](auto st) -> char* { return decltype(st)::value == 0 ? Os0 : Os1; };

  const TileSlot slot = tile_slot(blockIdx.x, p.per_xcd, p.split_tail);
  const int t = slot.tile;
  if (t >= p.total_tiles) return;
  const int bh = t / p.tiles_per_bh;
  const int rank = undeal(t - bh * p.tiles_per_bh, p.tiles_per_bh, p.deal);
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  int gi = 0;
  while (gi + 1 < p.n_blocks && p.blk[gi + 1].tile_prefix <= rank) ++gi;
  const KBlockDesc& kd = p.blk[gi];
  KeyList kl;  // keys of the group
  kl.n_keys = __builtin_amdgcn_readfirstlane(kd.n_keys);
  kl.start1 = __builtin_amdgcn_readfirstlane(kd.kiv_start[0]);
  kl.start2 = __builtin_amdgcn_readfirstlane(kd.kiv_start[1]);
  kl.delta0 = __builtin_amdgcn_readfirstlane(kd.kiv_delta[0]);
  kl.delta1 = __builtin_amdgcn_readfirstlane(kd.kiv_delta[1]);
  kl.delta2 = __builtin_amdgcn_readfirstlane(kd.kiv_delta[2]);
  KeyList rl;  // query rows that see them
  rl.n_keys = __builtin_amdgcn_readfirstlane(kd.n_rows);
  rl.start1 = __builtin_amdgcn_readfirstlane(kd.qiv_start);
  rl.start2 = rl.n_keys;
  rl.delta0 = __builtin_amdgcn_readfirstlane(kd.qiv_delta[0]);
  rl.delta1 = __builtin_amdgcn_readfirstlane(kd.qiv_delta[1]);
  rl.delta2 = 0;
  // keys [key0, key_end) of the group belong to this tile (or half tile)
  int key0 = (rank - kd.tile_prefix) * N;
  int key_end = min(kl.n_keys, key0 + N);
  if (slot.half != 0) {
    key0 += (slot.half - 1) * (N / 2);
    key_end = min(key_end, key0 + N / 2);
    if (key0 >= key_end) return;  // a tile of at most N/2 keys has no second half
  }
  const int n_rows = rl.n_keys;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int lr = lane & 31;
  const int hh = lane >> 5;

  const int64_t rs = int64_t(a.H) * D;
  const int64_t rsb = rs * 2;
  const int64_t bh_off = int64_t(b) * a.S * rs + int64_t(h) * D;
  const char* __restrict__ qg = reinterpret_cast<const char*>(static_cast<const __bf16*>(a.q) + bh_off);
  const char* __restrict__ og = reinterpret_cast<const char*>(static_cast<const __bf16*>(a.dout) + bh_off);
  const char* __restrict__ vg = reinterpret_cast<const char*>(static_cast<const __bf16*>(a.v) + bh_off);
  const int64_t row_base = (int64_t(b) * a.H + h) * a.S;  // per-row arrays [B,H,S]

  // this lane's key (B-operand column lr): K row in registers
  const int kj = key0 + wave * KW + lr;
  const bool key_ok = kj < key_end;
  // a wave whose keys all lie past the tile only helps with the DMA and the
  // barriers
  const bool active = key0 + wave * KW < key_end;
  const int ktok = vtoken(kl, min(kj, kl.n_keys - 1));
  bf16x8 kreg[NDS];
  {
    const __bf16* ks = static_cast<const __bf16*>(a.k) + bh_off + int64_t(ktok) * rs + hh * 8;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) kreg[ds] = key_ok ? *reinterpret_cast<const bf16x8*>(ks + ds * 16) : bf16x8{};
  }
  // V rows of this wave's keys into the key tile (keys past the group's end
  // repeat its last key; their columns are never stored)
  char* vt = Vt + wave * KW * RB;
#pragma unroll
  for (int i = 0; i < NVI; ++i) {
    const int r = i * RPI + lane / CH;
    const int pc = lane % CH;
    const int tok = vtoken(kl, min(key0 + wave * KW + r, kl.n_keys - 1));
    lds_dma16(vg + int64_t(tok) * rsb + (pc ^ dual_swz<CH>(r)) * 16, vt + i * 1024);
  }

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  // DMA of Q and dO rows (swizzled)
  int dma_row[NI];
  uint32_t goff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int q = wave * NI + i;
    const int r = q * RPI + lane / CH;
    const int pc = lane % CH;
    dma_row[i] = r;
    goff[i] = uint32_t(r * rsb + ((pc ^ dual_swz<CH>(r)) * 16));
  }
  auto issue = [&](int step, char* lbase, const char* gbase) {
    const int i0 = step * QT;
    const int iv_end = interval_end(rl, i0);
    const int delta = interval_delta(rl, i0);
    if (i0 + QT <= iv_end) {
      const char* base = gbase + int64_t(i0 + delta) * rsb;
#pragma unroll
      for (int i = 0; i < NI; ++i) lds_dma16(base, goff[i], lbase + (wave * NI + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int j = min(i0 + dma_row[i], n_rows - 1);
        lds_dma16(gbase + int64_t(vtoken(rl, j)) * rsb + (goff[i] - uint32_t(dma_row[i] * rsb)),
                  lbase + (wave * NI + i) * 1024);
      }
    }
  };
  // per-row constants of a step: waves 0 and 1 fetch lw and dw for one row
  // per lane (rows past the end: lw = +inf, dw = 0, which zeroes their
  // weights)
  // (the value is used, and so waited for, only when stored at the end of
  // the step: a wait right after the load would also drain the DMA)
  const float* rsrc = (wave == 0 ? a.lw : a.dw) + row_base;
  auto fetch_rows = [&](int step) -> float {
    const int i = step * QT + lane;
    if (wave > 1 || lane >= QT) return 0.f;
    if (i >= n_rows) return wave == 0 ? __builtin_inff() : 0.f;
    return rsrc[vtoken(rl, i)];
  };
  auto store_rows = [&](int stage, float x) {
    if (wave <= 1 && lane < QT) Rs[stage][wave][lane] = x;
  };

  // row-operand offsets (row lr, logical chunk 2 ds + hh), for the streamed
  // Q / dO blocks and for this wave's V rows alike
  const uint32_t row_off0 = uint32_t(lr * RB + ((hh ^ dual_swz<CH>(lr)) * 16));
  auto row_off = [&](int ds) { return row_off0 ^ uint32_t(32 * ds); };
  uint32_t tr_off0[2];
  {
    const int g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int row = 4 * hh + (i >> 2) + 8 * rr;
      const int col = 16 * (g & 1) + 4 * (i & 3);
      tr_off0[rr] = uint32_t(row * RB + (((col >> 3) ^ dual_swz<CH>(row)) * 16) + (col & 7) * 2);
    }
  }

  const float c = a.score_scale_log2;
  const int nsteps = (n_rows + QT - 1) / QT;

  auto body = [&](int step, auto st) {
    constexpr int s_ = decltype(st)::value;
    issue(step + 1, qstage(IC<1 - s_>{}), qg);
    issue(step + 1, ostage(IC<1 - s_>{}), og);
    const float nxt = fetch_rows(step + 1);
    const char* qsb = qstage(st);
    const char* osb = ostage(st);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      if (!active) break;
      const char* qs = qsb + qb * 32 * RB;
      const char* os = osb + qb * 32 * RB;
      f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const bf16x8 xq = *reinterpret_cast<const bf16x8*>(qs + row_off(ds));
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xq, kreg[ds], sc, 0, 0, 0);
      }
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const bf16x8 xo = *reinterpret_cast<const bf16x8*>(os + row_off(ds));
        const bf16x8 vb = *reinterpret_cast<const bf16x8*>(vt + row_off(ds));
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xo, vb, dp, 0, 0, 0);
      }
      // score register r holds query row 8 (r/4) + 4 hh + r % 4 of the block
      bf16x8 pg[2], dsb[2];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int row = qb * 32 + 8 * g4 + 4 * hh;
        const float4 Lr = *reinterpret_cast<const float4*>(&Rs[s_][0][row]);
        const float4 Dr = *reinterpret_cast<const float4*>(&Rs[s_][1][row]);
        const float Lv[4] = {Lr.x, Lr.y, Lr.z, Lr.w};
        const float Dv[4] = {Dr.x, Dr.y, Dr.z, Dr.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * g4 + u;
          const float w = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], c, -Lv[u]));  // sg P
          pg[r / 8][r % 8] = static_cast<__bf16>(w);
          dsb[r / 8][r % 8] = static_cast<__bf16>(w * (dp[r] - Dv[u]));
        }
      }
      // dV^T += dO^T (sg P), dK^T += Q^T dS over the block's two 16-row halves
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const char* ob = os + half * 16 * RB;
        const char* qb2 = qs + half * 16 * RB;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint32_t x0 = tr_off0[0] ^ uint32_t(64 * db), x1 = tr_off0[1] ^ uint32_t(64 * db);
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(ob + x0, ob + x1), pg[half], dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(qb2 + x0, qb2 + x1), dsb[half], dk[db], 0, 0, 0);
        }
      }
    }
    store_rows(1 - s_, nxt);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
  };

  issue(0, Qs0, qg);
  issue(0, Os0, og);
  store_rows(0, fetch_rows(0));
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // V tile, step 0's rows
  lds_barrier();
  for (int step = 0;;) {
    body(step, IC<0>{});
    if (++step >= nsteps) break;
    body(step, IC<1>{});
    if (++step >= nsteps) break;
  }

  if (key_ok) {
    const int64_t off = bh_off + int64_t(ktok) * rs;
    __bf16* dkd = static_cast<__bf16*>(a.dk) + off;
    __bf16* dvd = static_cast<__bf16*>(a.dv) + off;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 k4, v4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          k4[r] = static_cast<__bf16>(dk[db][g4 * 4 + r] * a.scale);
          v4[r] = static_cast<__bf16>(dv[db][g4 * 4 + r]);
        }
        *reinterpret_cast<bf16x4*>(dkd + db * 32 + g4 * 8 + hh * 4) = k4;
        *reinterpret_cast<bf16x4*>(dvd + db * 32 + g4 * 8 + hh * 4) = v4;
      }
  }
#endif
}

#ifndef VDN_KV_QT
#define VDN_KV_QT 32
#endif
#ifndef VDN_DQ_KT
#define VDN_DQ_KT 64
#endif
#ifndef VDN_DQ_NS
#define VDN_DQ_NS 2
#endif
constexpr int kDqWaves = 8;
constexpr int kDqKeys = VDN_DQ_KT;
constexpr int kDqStages = VDN_DQ_NS;
constexpr int kKvWaves = 8;
constexpr int kKvRows128 = VDN_KV_QT;  // query rows per dK/dV step at head_dim 128

// ---- fixed scratch for callers that cannot allocate
// The per-row constants (lw, dw) of vdn_local_attn_bwd_noalloc live in this
// file-scope device array: each GPU the library runs on holds its own copy
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host it only stands in for the symbol): it takes the array's
// address on the current device from hipGetSymbolAddress, once per device.
namespace {
static __device__ __align__(256) float scratch[kBwdScratchFloats];
std::mutex g_scratch_mu;
float* g_scratch_addr[kMaxScratchDevices] = {};
}  // namespace

int bwd_scratch(float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  if (dev < 0 || dev >= kMaxScratchDevices) return int(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return int(e);
    g_scratch_addr[dev] = static_cast<float*>(addr);
  }
  *ptr = g_scratch_addr[dev];
  return int(hipSuccess);
}

int bwd_dq_tile_m() { return 32 * kDqWaves; }
int bwd_dkv_tile_n() { return 32 * kKvWaves; }

int launch_bwd(const BwdDqParams& dq, const BwdKvParams& kv, int head_dim, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const BwdArgs& a = dq.a;
  const int64_t total = int64_t(a.B) * a.S * a.H;
  const int64_t rows_per_block = 256 / (head_dim / 8);
  const int64_t row_blocks = (total + rows_per_block - 1) / rows_per_block;
  if (row_blocks > INT32_MAX) return int(hipErrorInvalidConfiguration);
  const dim3 rgrid(static_cast<unsigned>(row_blocks));
  const dim3 qgrid(unsigned(dq.per_xcd + dq.split_tail) * 8u), qblock(64 * kDqWaves);
  const dim3 kgrid(unsigned(kv.per_xcd + kv.split_tail) * 8u), kblock(64 * kKvWaves);
  if (head_dim == 128) {
    hipLaunchKernelGGL((bwd_rows_kernel<128>), rgrid, dim3(256), 0, st, a, total);
    hipLaunchKernelGGL((bwd_dq_kernel<128, kDqWaves, kDqKeys, kDqStages>), qgrid, qblock, 0, st, dq);
    hipLaunchKernelGGL((bwd_dkv_kernel<128, kKvWaves, kKvRows128>), kgrid, kblock, 0, st, kv);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL((bwd_rows_kernel<64>), rgrid, dim3(256), 0, st, a, total);
    hipLaunchKernelGGL((bwd_dq_kernel<64, kDqWaves, kDqKeys, kDqStages>), qgrid, qblock, 0, st, dq);
    hipLaunchKernelGGL((bwd_dkv_kernel<64, kKvWaves, 64>), kgrid, kblock, 0, st, kv);
  } else {
    return int(hipErrorInvalidValue);
  }
  return int(hipGetLastError());
}

}  // namespace vdn
