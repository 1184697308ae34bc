// Complement linear branch of VDN-H3 hybrid video attention, and the
// two-branch fusion, for gfx950.
//
// The linear branch (openi.cn "VDN-MiniMax-H3", technical principles; the
// complement of the local softmax window, summarising the frames before and
// after a block's window, window frames and boundary anchors left out):
// with phi(x) = elu(x) + 1, a video query i of frame block beta gets
//   o_i = phi(q_i)^T S_beta / (phi(q_i) . z_beta),
//   S_beta = sum_j phi(k_j) v_j^T,  z_beta = sum_j phi(k_j),
// over the video keys j of frames f, 1 <= f <= F-2, outside the block's
// window [lo, hi).  Text rows, and rows of a block with no such frame, get 0.
//
// Three kernels, all one pass over their inputs:
//   1. frame states: per (sample, head, non-anchor frame), S_f^T = V_f^T
//      phi(K_f) on bf16 MFMA with K and V staged through LDS by DMA and read
//      back transposed, plus z_f = sum phi(k), to an fp32 workspace;
//   2. block states: per four state elements, the sum over each block's
//      frames (fp32, in frame order), written as bf16 S_beta^T and fp32
//      z_beta;
//   3. apply: per (sample, head, row tile of one block), O^T = S_beta^T
//      phi(Q)^T on bf16 MFMA with S_beta^T in LDS, the normaliser
//      phi(q) . z_beta from the same products (z split into two bf16 rows).
// The fusion (same page and section: the linear branch is RMS-normalised,
// then gated by its own sigmoid gate, then added to the gated softmax
// branch) is one wave per token over the token's H*D outputs.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fwd_common.hpp"
#include "linear_params.hpp"

#ifndef VDN_FUSE_NT
#define VDN_FUSE_NT 1
#endif
#ifndef VDN_LIN_APPLY_STAGE
#define VDN_LIN_APPLY_STAGE 1
#endif
// waves per SIMD the apply kernel is compiled for: 2, the two 4-wave
// workgroups per CU that its LDS allows (one wave per SIMD each)
#ifndef VDN_LIN_APPLY_MINW
#define VDN_LIN_APPLY_MINW 2
#endif

namespace vdn {

namespace {

// phi(x) = elu(x) + 1 = max(x, 0) + exp(min(x, 0)).
[[maybe_unused]] __device__ __forceinline__ float phi(float x) {
  return fmaxf(x, 0.f) + __builtin_amdgcn_exp2f(fminf(x, 0.f) * kLog2e);
}

// Number of non-anchor frames outside frame block beta's window.
[[maybe_unused]] __device__ __forceinline__ int linear_frames(int beta, int F, int Bf) {
  const int lo = Bf * max(0, beta - 1);
  const int hi = min(F, Bf * (beta + 2));
  return max(0, min(lo, F - 1) - 1) + max(0, (F - 1) - max(hi, 1));
}

// Waits until a step's DMA has landed while `ahead` later steps (clamped to
// 0..MAXA) stay in flight, each PER DMA instructions of this wave.
template <int PER, int MAXA>
__device__ __forceinline__ void wait_steps_ahead(int ahead) {
  static_assert(MAXA <= 4 && PER * MAXA < 64, "vmcnt range");
  if (MAXA >= 4 && ahead >= 4)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * PER));
  else if (MAXA >= 3 && ahead >= 3)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * PER));
  else if (MAXA >= 2 && ahead >= 2)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PER));
  else if (MAXA >= 1 && ahead >= 1)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// ---------------------------------------------------------------------------
// 1. Frame states.  One workgroup per (frame 1..F-2, sample * head); wave w
// owns d1 columns [32w, 32w + 32) of S_f^T = sum_t v_t phi(k_t)^T, i.e. the
// MFMA C[i = d2][j = d1] with A = V^T (transposing reads of the V tile) and
// B = phi(K) (transposing reads of the K tile, phi applied in registers).
// Both operands come from the same transposing read pattern, so their
// k slots (token rows {4hh..4hh+3, 8+4hh..8+4hh+3} of a 16-row group) agree.
template <int D, int NS, int KT>
__global__ __launch_bounds__(D / 32 * 64) void lin_frame_state_kernel(const LinParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NW = D / 32;
  constexpr int RB = 2 * D;
  constexpr int CH = D / 8;
  constexpr int TILE = KT * RB;          // KT tokens per stage
  constexpr int NI = TILE / 1024 / NW;   // DMA instructions per wave per tile
  constexpr int RPI = 1024 / RB;
  constexpr int NDB = D / 32;
  static_assert(NI * NW * 1024 == TILE && KT % 16 == 0 && NS >= 2 && NS <= 6, "tile shape");
  __shared__ __attribute__((aligned(1024))) char Ks[NS][TILE];
  __shared__ __attribute__((aligned(1024))) char Vs[NS][TILE];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;
  const int f = 1 + int(blockIdx.x);
  const int bh = int(blockIdx.y);
  const int b = bh / p.H, h = bh % p.H;
  const int T = p.T;
  const int64_t rs = int64_t(p.H) * D;
  const int64_t rsb = rs * 2;
  const int64_t base = (int64_t(b) * p.S + int64_t(f) * T) * rs + int64_t(h) * D;
  const char* __restrict__ kg = reinterpret_cast<const char*>(static_cast<const __bf16*>(p.k) + base);
  const char* __restrict__ vg = reinterpret_cast<const char*>(static_cast<const __bf16*>(p.v) + base);
  const int nsteps = (T + KT - 1) / KT;

  int drow[NI];
  uint32_t goff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = (wave * NI + i) * RPI + lane / CH;
    const int pc = lane % CH;
    drow[i] = r;
    goff[i] = uint32_t(r * rsb + ((pc ^ dual_swz<CH>(r)) * 16));
  }
  auto issue = [&](int step) {
    if (step >= nsteps) return;
    const int t0 = step * KT;
    char* kl = Ks[step % NS];
    char* vl = Vs[step % NS];
    if (t0 + KT <= T) {
      const char* kb = kg + int64_t(t0) * rsb;
      const char* vb = vg + int64_t(t0) * rsb;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        lds_dma16(kb, goff[i], kl + (wave * NI + i) * 1024);
        lds_dma16(vb, goff[i], vl + (wave * NI + i) * 1024);
      }
    } else {
      // last, partial step: rows past the frame repeat its last token (their
      // phi(k) is zeroed before use)
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int t = min(t0 + drow[i], T - 1);
        const int64_t off = int64_t(t) * rsb + (goff[i] - uint32_t(drow[i] * rsb));
        lds_dma16(kg + off, kl + (wave * NI + i) * 1024);
        lds_dma16(vg + off, vl + (wave * NI + i) * 1024);
      }
    }
  };

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
  const uint32_t kx0 = tr_off0[0] ^ uint32_t(64 * wave), kx1 = tr_off0[1] ^ uint32_t(64 * wave);

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  for (int s = 0; s < NS - 1; ++s) issue(s);
  wait_steps_ahead<2 * NI, NS - 2>(min(NS - 2, nsteps - 1));
  lds_barrier();
  // one step: all K and V fragments of the step read first, then phi on
  // the K fragments (rows past the frame zeroed on the partial last step),
  // then the MFMAs.  z = sum_t phi(k_t) comes from one more product per
  // 16 tokens, with an all-ones A operand (every row of zacc holds z).
  const bf16x8 ones = {__bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f),
                       __bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f)};
  f32x16 zacc = f32x16{};
  auto compute = [&](const char* kl, const char* vl, int rem, auto tail) {
    constexpr bool TAIL = decltype(tail)::value;
    constexpr int NKS = KT / 16;
    bf16x8 kraw[NKS], va[NKS][NDB];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const char* kr = kl + ks * 16 * RB;
      const char* vr = vl + ks * 16 * RB;
      kraw[ks] = tr_frag(kr + kx0, kr + kx1);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        va[ks][db] = tr_frag(vr + (tr_off0[0] ^ uint32_t(64 * db)), vr + (tr_off0[1] ^ uint32_t(64 * db)));
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 kb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = phi(float(kraw[ks][e]));
        if constexpr (TAIL) {
          // token row 16 ks + 4 hh + e % 4 + 8 (e / 4) of the step
          const float lim = float(rem - 16 * ks - 4 * hh - (e & 3) - 8 * (e >> 2)) - 0.5f;
          x = __builtin_amdgcn_fmed3f(x, 0.f, lim * __builtin_inff());
        }
        kb[e] = static_cast<__bf16>(x);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks][db], kb, acc[db], 0, 0, 0);
      zacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, kb, zacc, 0, 0, 0);
    }
  };
  auto step_end = [&](int step) {
    wait_steps_ahead<2 * NI, NS - 2>(min(NS - 2, nsteps - 2 - step));
    lds_barrier();
  };
  // full steps in the loop; a partial last step (T % KT != 0) after it
  const int nfull = T / KT;
  for (int step = 0; step < nfull; ++step) {
    issue(step + NS - 1);
    compute(Ks[step % NS], Vs[step % NS], KT, IC<0>{});
    step_end(step);
  }
  if (nfull < nsteps) compute(Ks[nfull % NS], Vs[nfull % NS], T - nfull * KT, IC<1>{});


  float* fs = p.fstate + (int64_t(bh) * (p.F - 2) + (f - 1)) * (D * D + D);
  const int d1 = 32 * wave + (lane & 31);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d2 = 32 * db + 8 * (r >> 2) + 4 * hh + (r & 3);
      fs[d2 * D + d1] = acc[db][r];
    }
  // zacc register 0 of lanes 0..31 is row 0 of the ones product: z[d1]
  if (hh == 0) fs[D * D + d1] = zacc[0];
#endif
}

// ---------------------------------------------------------------------------
// 2. Block states: one thread per 4 consecutive state elements (D*D entries
// of S^T, then D of z; D*D + D is a multiple of 4) and sample * head.  The
// frames' values are loaded in batches of up to FB frames in flight together,
// then summed in frame order into each block outside whose window they lie.
template <int D>
__global__ __launch_bounds__(256) void lin_block_state_kernel(const LinParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int E = D * D + D;
  constexpr int E4 = E / 4;
  constexpr int FB = 20;   // frames per load batch
  constexpr int BB = 8;    // blocks per pass
  static_assert(E % 4 == 0, "state size");
  const int e4 = int(blockIdx.x) * 256 + int(threadIdx.x);
  if (e4 >= E4) return;
  const int bh = int(blockIdx.y);
  const int nf = p.F - 2;
  const float4* src = reinterpret_cast<const float4*>(p.fstate + int64_t(bh) * (nf > 0 ? nf : 0) * E) + e4;
  for (int b0 = 0; b0 < p.nb; b0 += BB) {
    float4 acc[BB];
    int lo[BB], hi[BB];
#pragma unroll
    for (int j = 0; j < BB; ++j) {
      acc[j] = float4{0.f, 0.f, 0.f, 0.f};
      lo[j] = p.Bf * max(0, b0 + j - 1);
      hi[j] = min(p.F, p.Bf * (b0 + j + 2));
    }
    for (int f0 = 1; f0 <= nf; f0 += FB) {
      float4 x[FB];
#pragma unroll
      for (int u = 0; u < FB; ++u) x[u] = src[int64_t(min(f0 + u, nf) - 1) * E4];
#pragma unroll
      for (int u = 0; u < FB; ++u) {
        const int f = f0 + u;
#pragma unroll
        for (int j = 0; j < BB; ++j)
          if (f <= nf && (f < lo[j] || f >= hi[j])) {
            acc[j].x += x[u].x;
            acc[j].y += x[u].y;
            acc[j].z += x[u].z;
            acc[j].w += x[u].w;
          }
      }
    }
#pragma unroll
    for (int j = 0; j < BB; ++j) {
      const int beta = b0 + j;
      if (beta >= p.nb) break;
      const int64_t blk = int64_t(bh) * p.nb + beta;
      const int e = 4 * e4;
      if (e < D * D) {
        bf16x4 v4;
        v4[0] = static_cast<__bf16>(acc[j].x);
        v4[1] = static_cast<__bf16>(acc[j].y);
        v4[2] = static_cast<__bf16>(acc[j].z);
        v4[3] = static_cast<__bf16>(acc[j].w);
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.bstate) + blk * (D * D) + e) = v4;
      } else {
        *reinterpret_cast<float4*>(p.bz + blk * D + (e - D * D)) = acc[j];
      }
    }
  }
#endif
}

// ---------------------------------------------------------------------------
// 3. Apply.  One workgroup per (sample, head, tile of <= kLinRowTile rows of
// one frame block, or of the text rows), four waves.  Each wave takes
// 32-row groups: B = phi(Q)^T straight from global rows (16 bytes per lane),
// A = rows of the LDS state, C[i = d2][j = row] holding one query per lane.
// The LDS state has D rows of S^T plus a 32-row block whose rows 0 and 1
// hold z in two bf16 parts (z_hi = bf16(z), z_lo = bf16(z - z_hi)) and the
// rest zeros: its product gives the normaliser phi(q) . z with fp32
// accumulation on the matrix cores, to about 2^-17 of z.  The output leaves
// through a per-wave LDS tile so that stores write whole 128-byte lines.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, VDN_LIN_APPLY_MINW) void lin_apply_kernel(const LinParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int RB = 2 * D;
  constexpr int CH = D / 8;
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int SR = D + 32;  // LDS state rows
  __shared__ __attribute__((aligned(1024))) char Ss[SR * RB];
#if VDN_LIN_APPLY_STAGE
  // per-wave output staging: 32 rows x 128 bytes (two 32-column blocks)
  __shared__ __attribute__((aligned(16))) char Os[NW][32 * 128];
#endif

  // heads fastest: the workgroups in flight together cover whole token
  // rows (measured faster than keeping a block state's tiles on one XCD)
  const int logical = int(blockIdx.x);
  if (logical >= p.total_tiles) return;
  const int nbh = p.B * p.H;
  const int bh = logical % nbh;
  const int tile = logical / nbh;
  const int b = bh / p.H, h = bh % p.H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;
  const int lr = lane & 31;

  const int V = p.F * p.T;
  const int blk_rows = p.Bf * p.T;
  const int tpb = p.tiles_per_block;
  int beta, r_lo, r_hi;
  if (tile < (p.nb - 1) * tpb) {
    beta = tile / tpb;
    r_lo = beta * blk_rows + (tile % tpb) * kLinRowTile;
    r_hi = min(r_lo + kLinRowTile, (beta + 1) * blk_rows);
  } else if (tile < (p.nb - 1) * tpb + p.tiles_last) {
    beta = p.nb - 1;
    r_lo = beta * blk_rows + (tile - (p.nb - 1) * tpb) * kLinRowTile;
    r_hi = min(r_lo + kLinRowTile, V);
  } else {
    beta = -1;
    r_lo = V + (tile - (p.nb - 1) * tpb - p.tiles_last) * kLinRowTile;
    r_hi = min(r_lo + kLinRowTile, p.S);
  }
  const int64_t rs = int64_t(p.H) * D;
  const int64_t bh_off = int64_t(b) * p.S * rs + int64_t(h) * D;
  __bf16* __restrict__ og = static_cast<__bf16*>(p.out) + bh_off;

  float* __restrict__ ssg = p.ss == nullptr ? nullptr : p.ss + int64_t(b) * p.S * p.H + h;
  if (beta < 0 || linear_frames(beta, p.F, p.Bf) == 0) {
    // text rows, or a block with no linear keys: zeros
    const int n = (r_hi - r_lo) * CH;
    for (int c = int(threadIdx.x); c < n; c += NW * 64) {
      const int r = r_lo + c / CH;
      *reinterpret_cast<u32x4*>(og + int64_t(r) * rs + (c % CH) * 8) = u32x4{0u, 0u, 0u, 0u};
    }
    if (ssg != nullptr)
      for (int r = r_lo + int(threadIdx.x); r < r_hi; r += NW * 64) ssg[int64_t(r) * p.H] = 0.f;
    return;
  }

  // block state into LDS (rows swizzled for row reads), then the normaliser
  // block
  {
    const int64_t blk = int64_t(bh) * p.nb + beta;
    const char* src = reinterpret_cast<const char*>(static_cast<const __bf16*>(p.bstate) + blk * (D * D));
    for (int c = int(threadIdx.x); c < D * CH; c += NW * 64) {
      const int r = c / CH, pc = c % CH;
      *reinterpret_cast<u32x4*>(Ss + r * RB + ((pc ^ dual_swz<CH>(r)) * 16)) =
          *reinterpret_cast<const u32x4*>(src + r * RB + pc * 16);
    }
    const float* zsrc = p.bz + blk * D;
    for (int c = int(threadIdx.x); c < 32 * CH; c += NW * 64) {
      const int r = c / CH, pc = c % CH;
      bf16x8 x{};
      if (r < 2) {
        const float4 z0 = *reinterpret_cast<const float4*>(zsrc + 8 * pc);
        const float4 z1 = *reinterpret_cast<const float4*>(zsrc + 8 * pc + 4);
        const float zz[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const __bf16 hi = static_cast<__bf16>(zz[e]);
          x[e] = r == 0 ? hi : static_cast<__bf16>(zz[e] - float(hi));
        }
      }
      *reinterpret_cast<bf16x8*>(Ss + (D + r) * RB + ((pc ^ dual_swz<CH>(r)) * 16)) = x;
    }
  }
  __syncthreads();

  const __bf16* __restrict__ qg = static_cast<const __bf16*>(p.q) + bh_off;
  const uint32_t row_off0 = uint32_t(lr * RB + ((hh ^ dual_swz<CH>(lr)) * 16));
  const int ngroups = (r_hi - r_lo + 31) / 32;

  auto load_q = [&](int g, bf16x8 (&qf)[NDS]) {
    const __bf16* src = qg + int64_t(min(r_lo + 32 * g + lr, r_hi - 1)) * rs + 8 * hh;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qf[ds] = *reinterpret_cast<const bf16x8*>(src + 16 * ds);
  };
  // one 32-row group of Q ahead in registers
  bf16x8 qn[NDS];
  if (wave < ngroups) load_q(wave, qn);
  for (int g = wave; g < ngroups; g += NW) {
    bf16x8 bq[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) bq[ds] = qn[ds];
    if (g + NW < ngroups) load_q(g + NW, qn);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
      for (int e = 0; e < 8; ++e) bq[ds][e] = static_cast<__bf16>(phi(float(bq[ds][e])));

    // normaliser block first, then the output columns two blocks at a time
    auto block = [&](int db) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ss + db * 32 * RB + (row_off0 ^ uint32_t(32 * ds)));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[ds], acc, 0, 0, 0);
      }
      return acc;
    };
    const f32x16 zacc = block(NDB);
    const float den = xhalf_sum(zacc[0] + zacc[1]);
    const float inv = den > 0.f ? 1.f / den : 0.f;
#if VDN_LIN_APPLY_STAGE
    // the result layout holds one row per lane; the rows go out through LDS
    // so that every store instruction writes whole 128-byte lines (8 rows x
    // 128 bytes).  16-byte chunk c of a staged row sits at c ^ ((row/2) % 8):
    // the 8-byte writes of 32 rows meet at most two to a bank, the row reads
    // not at all.
    char* os = Os[wave];
    float ssq = 0.f;  // this lane's half of the row's sum of squares
#pragma unroll
    for (int pair = 0; pair < NDB / 2; ++pair) {
#pragma unroll
      for (int dd = 0; dd < 2; ++dd) {
        const f32x16 acc = block(2 * pair + dd);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bf16x4 o4;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = acc[4 * g4 + r] * inv;
            ssq = __builtin_fmaf(x, x, ssq);
            o4[r] = static_cast<__bf16>(x);
          }
          const int ch = (4 * dd + g4) ^ ((lr >> 1) & 7);
          *reinterpret_cast<bf16x4*>(os + lr * 128 + ch * 16 + hh * 8) = o4;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 8 * i + (lane >> 3), pc = lane & 7;
        const u32x4 v = *reinterpret_cast<const u32x4*>(os + rr * 128 + ((pc ^ ((rr >> 1) & 7)) * 16));
        const int orow = r_lo + 32 * g + rr;
        if (orow < r_hi) *reinterpret_cast<u32x4*>(og + int64_t(orow) * rs + pair * 64 + pc * 8) = v;
      }
    }
    if (ssg != nullptr) {
      ssq = xhalf_sum(ssq);
      const int row = r_lo + 32 * g + lr;
      if (hh == 0 && row < r_hi) ssg[int64_t(row) * p.H] = ssq;
    }
#else
    const int row = r_lo + 32 * g + lr;
    __bf16* dst = og + int64_t(row) * rs;
    float ssq = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const f32x16 acc = block(db);
      if (row < r_hi) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bf16x4 o4;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = acc[4 * g4 + r] * inv;
            ssq = __builtin_fmaf(x, x, ssq);
            o4[r] = static_cast<__bf16>(x);
          }
          *reinterpret_cast<bf16x4*>(dst + 32 * db + 8 * g4 + 4 * hh) = o4;
        }
      }
    }
    if (ssg != nullptr) {
      ssq = xhalf_sum(ssq);
      if (hh == 0 && row < r_hi) ssg[int64_t(row) * p.H] = ssq;
    }
#endif
  }
#endif
}

// ---------------------------------------------------------------------------
// Fusion: one wave per token; lane l holds elements 512 c + 8 l .. +7 of the
// token's H*D outputs (NCH * 512 >= H*D).
//   out = soft + sigmoid(gate_h) * lin * weight / sqrt(mean(lin^2) + eps)
// The token rows stream through once (non-temporal loads and stores, so the
// weight row, read by every token, stays cached); soft_out is loaded up
// front with lin_out, before the reduction.
template <typename T>
__device__ __forceinline__ T stream_load(const T* p) {
#if VDN_FUSE_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}
template <typename T>
__device__ __forceinline__ void stream_store(T x, T* p) {
#if VDN_FUSE_NT
  __builtin_nontemporal_store(x, p);
#else
  *p = x;
#endif
}

template <int NCH>
__global__ __launch_bounds__(256) void fuse_kernel(const FuseParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + wave;
  if (row >= p.rows) return;
  const int HD = p.HD;
  const u32x4* lin = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(p.lin) + row * HD);
  const u32x4* soft = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(p.soft) + row * HD);
  u32x4* out = reinterpret_cast<u32x4*>(static_cast<__bf16*>(p.out) + row * HD);
  u32x4 lraw[NCH], sraw[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int e = 512 * c + 8 * lane;
    lraw[c] = e < HD ? stream_load(lin + e / 8) : u32x4{0u, 0u, 0u, 0u};
    sraw[c] = e < HD ? stream_load(soft + e / 8) : u32x4{0u, 0u, 0u, 0u};
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const bf16x8 lv = __builtin_bit_cast(bf16x8, lraw[c]);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(float(lv[i]), float(lv[i]), ss);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  const float rinv = 1.f / __builtin_sqrtf(ss / float(HD) + p.eps);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int e = 512 * c + 8 * lane;
    if (e < HD) {
      const float g = p.gate[row * p.H + e / p.D];
      const float sg = 1.f / (1.f + __builtin_amdgcn_exp2f(-g * kLog2e));
      const float sc = sg * rinv;
      const float4 w0 = *reinterpret_cast<const float4*>(p.weight + e);
      const float4 w1 = *reinterpret_cast<const float4*>(p.weight + e + 4);
      const float ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      const bf16x8 lv = __builtin_bit_cast(bf16x8, lraw[c]);
      const bf16x8 s8 = __builtin_bit_cast(bf16x8, sraw[c]);
      bf16x8 o8;
#pragma unroll
      for (int i = 0; i < 8; ++i) o8[i] = static_cast<__bf16>(__builtin_fmaf(float(lv[i]) * ww[i], sc, float(s8[i])));
      stream_store(__builtin_bit_cast(u32x4, o8), out + e / 8);
    }
  }
#endif
}

#ifndef VDN_LIN_NS
#define VDN_LIN_NS 2
#endif
#ifndef VDN_LIN_KT
#define VDN_LIN_KT 32
#endif

#ifndef VDN_LIN_APPLY_NW
#define VDN_LIN_APPLY_NW 4
#endif

template <int D>
int launch_linear_d(const LinParams& p, hipStream_t st) {
  if (p.F > 2) {
    const dim3 fs_grid(p.F - 2, p.B * p.H);
    hipLaunchKernelGGL((lin_frame_state_kernel<D, VDN_LIN_NS, VDN_LIN_KT>), fs_grid, dim3(D / 32 * 64), 0, st, p);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return int(e);
  }
  hipLaunchKernelGGL((lin_block_state_kernel<D>), dim3(((D * D + D) / 4 + 255) / 256, p.B * p.H), dim3(256), 0, st, p);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return int(e);
  hipLaunchKernelGGL((lin_apply_kernel<D, VDN_LIN_APPLY_NW>), dim3(p.total_tiles), dim3(VDN_LIN_APPLY_NW * 64), 0, st, p);
  return int(hipGetLastError());
}

}  // namespace

int launch_linear(const LinParams& p, int head_dim, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  return head_dim == 64 ? launch_linear_d<64>(p, st) : launch_linear_d<128>(p, st);
}

int launch_fuse(const FuseParams& p, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(unsigned((p.rows + 3) / 4));
  const int nch = (p.HD + 511) / 512;
  if (nch <= 1)
    hipLaunchKernelGGL((fuse_kernel<1>), grid, dim3(256), 0, st, p);
  else if (nch <= 2)
    hipLaunchKernelGGL((fuse_kernel<2>), grid, dim3(256), 0, st, p);
  else if (nch <= 4)
    hipLaunchKernelGGL((fuse_kernel<4>), grid, dim3(256), 0, st, p);
  else if (nch <= 8)
    hipLaunchKernelGGL((fuse_kernel<8>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((fuse_kernel<16>), grid, dim3(256), 0, st, p);
  return int(hipGetLastError());
}

}  // namespace vdn
