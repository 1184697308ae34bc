// Block-sparse flash-attention forward for gfx950, OCP fp8 e4m3 inputs.
//
// Same operation and schedule as the bf16 kernel (local Softmax branch of
// VDN-H3 attention: frame-block window, first/last-frame anchors, global
// text keys, per-token sigmoid gate; openi.cn "VDN-MiniMax-H3", technical
// principles; nav.superapi.store "VDN-MiniMax-H3 - OpenVDN's Open-Source
// Video Generation Acceleration Solution", Technical Principles), with the
// two products on the fp8 matrix cores (v_mfma_f32_32x32x64_f8f6f4):
//
//   scores  S = sum_d q8 k8 (exact products, fp32 accumulation); the real
//           score is S * s_q[h] * s_k[h] * scale, folded into one factor;
//   weights P = 2^7 exp2(S c - m) with m a running maximum that lags the
//           row's true maximum by at most 1 (the accumulator is rescaled
//           only when the maximum grows by more), so P <= 2^8 < 448 and
//           weights down to 2^-16..2^-17 of the row maximum stay above
//           e4m3's smallest subnormal (2^-9); rounded to e4m3 with
//           v_cvt_pk_fp8_f32 (round to nearest even).  The 2^7 cancels in
//           O = acc / l and is taken out of the log-sum-exp;
//   output  O = (P8 V8) * s_v[h] / l, where l = sum of the rounded P8, taken
//           by one extra MFMA against an all-ones operand so that numerator
//           and denominator use the same weights.
//
// Operand layouts (per 32x32x64 MFMA, each lane supplies 32 bytes of k):
//   S^T = K Q^T: A = 32 bytes of a K row (two 16-byte LDS reads), B = the same
//   32 bytes of the Q row, held in registers.
//   O^T = V^T P^T: B = the lane's 32 P values (keys 32 kb + 8 (r/4) +
//   4 (l/32) + r%4 of the S^T layout, byte 16 kb + r); A = V^T bytes for the
//   same keys, gathered by four ds_read_b64_tr_b8: in each 16-lane group lane
//   i receives byte i % 8 of the blocks addressed by lanes 2e + i/8 (e = 0..7),
//   so pointing lanes 2e and 2e+1 at the two 8-column halves of key row e
//   hands lane i column c0 + i of eight keys.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fwd_common.hpp"

namespace vdn {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// e4m3fn encoding of 1.0 in every byte.
[[maybe_unused]] constexpr int kFp8Ones = 0x38383838;
// log2 of the factor applied to the weights before rounding them to e4m3.
// The running maximum may lag the true one by up to kFp8Slack (log2 units):
// the accumulator is rescaled only when a row's maximum grows by more, and
// P = 2^(8 - slack) exp2(S c - m) then still stays <= 2^8.
#ifndef VDN_FP8_SLACK
#define VDN_FP8_SLACK 1
#endif
[[maybe_unused]] constexpr float kFp8Slack = float(VDN_FP8_SLACK);
[[maybe_unused]] constexpr float kFp8PShift = 8.0f - kFp8Slack;

template <int D, int NW, int NS, int KT, int KPF>
__global__ __launch_bounds__(NW * 64, 2) void fwd_fp8_kernel(const FwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  constexpr int QW = 32;          // query rows per wave
  constexpr int M = NW * QW;      // query rows per workgroup
  constexpr int RB = D;           // bytes per key row
  constexpr int CH = D / 16;      // 16-byte chunks per row
  constexpr int TILE = KT * RB;   // bytes per K (or V) stage
  constexpr int NI = TILE / 1024 / NW;  // DMA instructions per wave per tensor per step
  constexpr int RPI = 1024 / RB;  // key rows per DMA instruction
  constexpr int NQK = D / 64;     // QK^T MFMAs per 32-key block
  constexpr int NDB = D / 32;     // 32-wide d blocks of the output
  constexpr int NKB = KT / 32;    // 32-key blocks per step
  constexpr int NPV = KT / 64;    // 64-key PV MFMAs per d block per step
  static_assert(D == 128 && NI >= 1 && NI * NW * 1024 == TILE, "tile shape");
  static_assert(NS == 2 || NS == 4, "the main loop is unrolled for a 2- or 4-stage ring");
  // Row swizzles (16-byte chunk c of key row r stored at c ^ swz(r)):
  //   K: (r >> 1) % 8 -- 16 consecutive rows (two per 256 bytes of banks) of
  //      a 16-byte fragment read land on distinct banks;
  //   V: 2 * ((r >> 1) & 1 | (r >> 2) & 2) -- the eight rows x 16 bytes read
  //      by 32 lanes of a ds_read_b64_tr_b8 cover all banks.
  auto kswz = [](int r) { return (r >> 1) & (CH - 1); };
  auto vswz = [](int r) { return 2 * (((r >> 1) & 1) | ((r >> 2) & 2)); };

  // K and V rings, one LDS array per stage (measured 1-2% faster than one
  // array holding all stages).  The DMA is inline asm that the compiler does
  // not track: stage reuse is ordered by explicit vmcnt waits and barriers.
  constexpr int T2 = NS > 2 ? TILE : 16;  // stages 2 and 3 exist only in the 4-stage ring
  __shared__ __attribute__((aligned(1024))) char Ks0[TILE];
  __shared__ __attribute__((aligned(1024))) char Ks1[TILE];
  __shared__ __attribute__((aligned(1024))) char Ks2[T2];
  __shared__ __attribute__((aligned(1024))) char Ks3[T2];
  __shared__ __attribute__((aligned(1024))) char Vs0[TILE];
  __shared__ __attribute__((aligned(1024))) char Vs1[TILE];
  __shared__ __attribute__((aligned(1024))) char Vs2[T2];
  __shared__ __attribute__((aligned(1024))) char Vs3[T2];
  auto kstage = [&](auto stage_c) -> char* {
    constexpr int st = decltype(stage_c)::value;
    return st == 0 ? Ks0 : st == 1 ? Ks1 : st == 2 ? Ks2 : Ks3;
  };
  auto vstage = [&](auto stage_c) -> char* {
    constexpr int st = decltype(stage_c)::value;
    return st == 0 ? Vs0 : st == 1 ? Vs1 : st == 2 ? Vs2 : Vs3;
  };

  __shared__ int s_next;  // the next tile's slot, handed from wave 0 to the others

  // One query tile, given its slot in the XCD queues (slot w: queue w % 8,
  // position w / 8); `claim` is the pending claim on the next one.
  auto run_tile = [&](const int wslot, PendingClaim& claim) __attribute__((always_inline)) {
  // ---- which tile (XCD-aware, the last tiles of each XCD in halves)
  const TileSlot slot = tile_slot(wslot, p.per_xcd, p.split_tail);
  const int t = slot.tile;
  if (t >= p.total_tiles) return;
  // (divisors opaque per tile: their reciprocals are then formed here, not
  // hoisted out of the tile loop and held in registers across every step)
  int tpb = p.tiles_per_bh, deal = p.deal, nh = p.H;
  asm volatile("" : "+s"(tpb), "+s"(deal), "+s"(nh));
  const int bh = t / tpb;
  const int rank = undeal(t - bh * tpb, tpb, deal);
  const int b = bh / nh;
  const int h = bh - b * nh;
  int bi = 0;
  while (bi + 1 < p.n_qblocks && p.blk[bi + 1].tile_prefix <= rank) ++bi;
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

  const int64_t rsb = int64_t(p.H) * D;  // token stride (bytes = elements)
  const int64_t bh_off = int64_t(b) * p.S * rsb + int64_t(h) * D;
  const char* __restrict__ qg = static_cast<const char*>(p.q) + bh_off;
  const char* __restrict__ kg = static_cast<const char*>(p.k) + bh_off;
  const char* __restrict__ vg = static_cast<const char*>(p.v) + bh_off;

  // per-head dequantisation scales
  auto uniform = [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x))); };
  const float s_q = uniform(p.scales[h]);
  const float s_k = uniform(p.scales[p.H + h]);
  const float s_v = uniform(p.scales[2 * p.H + h]);
  const float c = s_q * s_k * p.score_scale_log2;

  // ---- Q rows: for QK MFMA m, this lane supplies bytes 64 m + 32 hh .. +31.
  i32x8 q8[NQK];
  {
    const int lrow = wave * QW + lr;
    const char* src = qg + int64_t(row0 + lrow) * rsb + 32 * hh;
#pragma unroll
    for (int m = 0; m < NQK; ++m) {
      if (lrow < rows) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(src + 64 * m);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(src + 64 * m + 16);
        q8[m] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      } else {
        q8[m] = i32x8{};
      }
    }
  }
  // Q lands before any DMA is issued: the compiler cannot count the DMA, and
  // with its own loads still pending at the loop it would wait on the whole
  // ring inside every step
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  f32x16 acc[NDB];
  f32x16 lacc = f32x16{};  // every element: the row sum of the rounded weights
  float m_run = -__builtin_inff();
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  // ---- DMA addressing (one 1 KB block = RPI key rows per instruction)
  int dma_row[NI];
  uint32_t k_goff[NI], v_goff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int q = wave * NI + i;
    const int r = q * RPI + lane / CH;
    const int pc = lane % CH;
    dma_row[i] = r;
    k_goff[i] = uint32_t(r * rsb + ((pc ^ kswz(r)) * 16));
    v_goff[i] = uint32_t(r * rsb + ((pc ^ vswz(r)) * 16));
  }
  // (the tensor is a compile-time tag: choosing between the two offset arrays
  // at run time would force them out of registers)
  auto issue = [&](int step, auto stage_c, auto is_k_c) {
    constexpr bool is_k = decltype(is_k_c)::value != 0;
    uint32_t goff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (is_k) {
        goff[i] = k_goff[i];
      } else {
        goff[i] = v_goff[i];
      }
    }
    const char* gbase = is_k ? kg : vg;
    char* lbase = is_k ? kstage(stage_c) : vstage(stage_c);
    const int j0 = step * KT;
    const int iv_end = interval_end(kl, j0);
    const int delta = interval_delta(kl, j0);
    if (j0 + KT <= iv_end) {
      const char* base = gbase + int64_t(j0 + delta) * rsb;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        lds_dma16(base, goff[i], lbase + (wave * NI + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int j = min(j0 + dma_row[i], n_keys - 1);
        lds_dma16(gbase + int64_t(vtoken(kl, j)) * rsb + (goff[i] - uint32_t(dma_row[i] * rsb)),
                  lbase + (wave * NI + i) * 1024);
      }
    }
  };
  auto issue_step = [&](int step, auto stage_c) {
    issue(step, stage_c, IC<1>{});
    issue(step, stage_c, IC<0>{});
  };

  // ---- LDS read offsets (bytes within a stage)
  // K fragment for QK MFMA m: row lr (+32 kb), logical chunks 4m + 2hh (+1).
  uint32_t k_roff[NQK][2];
#pragma unroll
  for (int m = 0; m < NQK; ++m)
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) k_roff[m][t2] = uint32_t(lr * RB + (((4 * m + 2 * hh + t2) ^ kswz(lr)) * 16));
  // V^T fragment for d block db, tr read r (rows +16 r): lane j of 16-lane
  // group g points at key 8 (j/8) + 4 hh + (j/2) % 4, columns
  // 32 db + 16 (g % 2) + 8 (j % 2) .. +7.
  uint32_t v_roff[NDB];
  {
    const int g = lane >> 4, j = lane & 15;
    const int key = 8 * (j >> 3) + 4 * hh + ((j >> 1) & 3);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int chunk = (2 * db + (g & 1)) ^ vswz(key);
      v_roff[db] = uint32_t(key * RB + chunk * 16 + 8 * (j & 1));
    }
  }

  const int nsteps = (n_keys + KT - 1) / KT;
  const i32x8 ones8 = {kFp8Ones, kFp8Ones, kFp8Ones, kFp8Ones, kFp8Ones, kFp8Ones, kFp8Ones, kFp8Ones};

  // S^T = K Q^T; the K fragments (two 16-byte reads each) run KPF MFMAs
  // ahead of their consumers, pinned there against the scheduler.
  auto qk = [&](auto stage_c, f32x16 (&s)[NKB]) {
    const char* ks = kstage(stage_c);
    constexpr int NF = NQK * NKB;
    constexpr int PF = KPF < NF ? KPF : NF;
    auto frag = [&](int f) {
      const int m = f / NKB, kb = f % NKB;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(ks + kb * 32 * RB + k_roff[m][0]);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(ks + kb * 32 * RB + k_roff[m][1]);
      return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    i32x8 fr[PF];
#pragma unroll
    for (int f = 0; f < PF; ++f) fr[f] = frag(f);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      s[f % NKB] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fr[f % PF], q8[f / NKB], s[f % NKB], 0, 0, 0, 0, 0, 0);
      if (f + PF < NF) fr[f % PF] = frag(f + PF);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // the next step reads K and V of step+1: batches step+2 .. step+NS-1 may
  // still be in flight
  auto sync_step = [&]() {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * 2 * NI));
    lds_barrier();
  };
  // a wave whose rows all lie past the end of the query block only helps
  // with the DMA and the barriers
  const bool active = __builtin_amdgcn_readfirstlane(wave) * QW < rows;

  auto compute = [&](int step, auto stage_c, auto dma_k, auto dma_v) {
    f32x16 s_cur[NKB];
    qk(stage_c, s_cur);
    dma_k();
    const int j0 = step * KT;
    if (j0 + KT > n_keys) mask_tail<NKB>(s_cur, n_keys - j0, hh);
    {
      // one running maximum per key block folding two scores per three-input
      // max (the compiler's own form needs 3 ops per 4 scores)
      float mb[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        mb[kb] = fmaxf(s_cur[kb][0], s_cur[kb][1]);
#pragma unroll
        for (int r = 2; r < 16; r += 2)
          asm("v_max3_f32 %0, %0, %1, %2" : "+v"(mb[kb]) : "v"(s_cur[kb][r]), "v"(s_cur[kb][r + 1]));
      }
      float mx = mb[0];
#pragma unroll
      for (int kb = 1; kb < NKB; ++kb) mx = fmaxf(mx, mb[kb]);
      mx = xhalf_max(mx) * c;
      if (__any(mx > m_run + kFp8Slack)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
#pragma unroll
        for (int r = 0; r < 16; ++r) lacc[r] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      }
    }

    // P = 2^8 exp2(S c - m) <= 2^8, rounded to e4m3: byte 16 (kb % 2) + r of
    // the lane's operand for PV MFMA kb / 2
    i32x8 p8[NPV];
    {
      const float mneg = kFp8PShift - m_run;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float e[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) e[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[kb][4 * q4 + u], c, mneg));
          int wv = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
          wv = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], wv, true);
          p8[kb / 2][4 * (kb % 2) + q4] = wv;
        }
      }
    }
    dma_v();
    // row sums of the rounded weights, then O^T += V^T P^T
    const char* vs = vstage(stage_c);
#pragma unroll
    for (int t = 0; t < NPV; ++t) {
      lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones8, p8[t], lacc, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        i32x8 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const i32x2 v2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) i32x2*)(vs + (64 * t + 16 * r) * RB + v_roff[db]));
          a[2 * r] = v2[0];
          a[2 * r + 1] = v2[1];
        }
        acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, p8[t], acc[db], 0, 0, 0, 0, 0, 0);
      }
    }
  };
  auto body = [&](int step, auto stage_c) {
    constexpr int st = decltype(stage_c)::value;
    // K of step + NS - 1 goes out once this step's QK products are issued,
    // V once its weights are formed (waves with no rows issue both at once);
    // issued together at the start of the step, the batch held back the QK
    // products behind it
    auto dma_k = [&]() __attribute__((always_inline)) { issue(step + NS - 1, IC<(st + NS - 1) % NS>{}, IC<1>{}); };
    auto dma_v = [&]() __attribute__((always_inline)) { issue(step + NS - 1, IC<(st + NS - 1) % NS>{}, IC<0>{}); };
    // the claim on the next tile goes out with this tile's last step (tiles
    // are then handed out in the order workgroups finish; the end-of-step
    // wait covers the atomic)
    if (step + 1 >= nsteps) claim.issue(p.queue, tid);
    if (active) {
      compute(step, stage_c, dma_k, dma_v);
    } else {
      dma_k();
      dma_v();
    }
    sync_step();
  };

  // prologue: steps 0 .. NS-2 in flight
  issue_step(0, IC<0>{});
  if constexpr (NS > 2) {
    issue_step(1, IC<1>{});
    issue_step(2, IC<2 % NS>{});
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * 2 * NI));  // step 0 has landed
  lds_barrier();
  for (int step = 0;;) {
    body(step, IC<0>{});
    if (++step >= nsteps) break;
    body(step, IC<1 % NS>{});
    if (++step >= nsteps) break;
    if constexpr (NS > 2) {
      body(step, IC<2 % NS>{});
      if (++step >= nsteps) break;
      body(step, IC<3 % NS>{});
      if (++step >= nsteps) break;
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no DMA outlives the workgroup

  // ---- epilogue: O = acc * s_v / l (* gate), bf16
  __bf16* og = static_cast<__bf16*>(p.out) + (int64_t(b) * p.S * p.H + int64_t(h)) * D;
  const int lrow = wave * QW + lr;
  const float l_tot = lacc[0];
  if (lrow < rows) {
    const int row = row0 + lrow;
    float scale = s_v / l_tot;
    if (p.gate != nullptr) {
      const float g = p.gate[(int64_t(b) * p.S + row) * p.H + h];
      scale *= 1.0f / (1.0f + __builtin_amdgcn_exp2f(-g * kLog2e));
    }
    __bf16* dst = og + int64_t(row) * p.H * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 o4;
#pragma unroll
        for (int r = 0; r < 4; ++r) o4[r] = static_cast<__bf16>(acc[db][g4 * 4 + r] * scale);
        *reinterpret_cast<bf16x4*>(dst + db * 32 + g4 * 8 + hh * 4) = o4;
      }
    }
    if (p.lse != nullptr && hh == 0) {
      p.lse[(int64_t(b) * p.H + h) * p.S + row] = (m_run - kFp8PShift + __log2f(l_tot)) * kLn2;
    }
  }
  };  // run_tile

  // Each workgroup starts on its own slot; persistent (p.queue set), it then
  // claims slots of its home queue (block index % 8) and, once that is
  // empty, of the other XCDs' queues.  Otherwise that one slot is all.
  int wslot = blockIdx.x;
  int steal = 1;  // next queue to try once the home queue is empty
  for (;;) {
    PendingClaim claim;
    run_tile(wslot, claim);
    if (p.queue == nullptr) break;
    if (threadIdx.x == 0) s_next = next_slot(p.queue, claim, p.per_xcd + p.split_tail, p.queue_wg, steal);
    lds_barrier();
    wslot = __builtin_amdgcn_readfirstlane(s_next);
    lds_barrier();  // every wave has read the slot before wave 0 writes the next one
    if (wslot < 0) break;
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// 128 keys per step over a 2-stage ring (64-key steps with the next
// step's scores pipelined under the softmax measured 10% slower on the 768p
// fp8 workload); K fragments 4 MFMAs ahead.
#ifndef VDN_FP8_KT
#define VDN_FP8_KT 128
#endif
#ifndef VDN_FP8_STAGES
#define VDN_FP8_STAGES 2
#endif
#ifndef VDN_FP8_KPF
#define VDN_FP8_KPF 4
#endif

int launch_fwd_fp8(const FwdParams& p_in, int head_dim, void* stream) {
  constexpr int kWaves = 8;
  constexpr int kStages = VDN_FP8_STAGES;
  constexpr int kKeysPerStep = VDN_FP8_KT;
  constexpr int kReadAhead = VDN_FP8_KPF;
  if (head_dim != 128) return int(hipErrorInvalidValue);
  const auto kernel = fwd_fp8_kernel<128, kWaves, kStages, kKeysPerStep, kReadAhead>;
  FwdParams p = p_in;
  p.queue = nullptr;
  p.queue_wg = 0;
  const int slots = p.per_xcd + p.split_tail;  // per XCD queue
  int wg = 0;
  int* queue = nullptr;
  const int rc = queue_for(reinterpret_cast<const void*>(kernel), kQueueFp8, &wg, &queue);
  if (rc != 0) return rc;
  dim3 grid(unsigned(slots) * 8u);
  if (queue != nullptr && wg < slots) {
    p.queue = queue;
    p.queue_wg = wg;
    grid = dim3(unsigned(wg) * 8u);
  }
  hipLaunchKernelGGL(kernel, grid, dim3(64 * kWaves), 0, static_cast<hipStream_t>(stream), p);
  return int(hipGetLastError());
}

}  // namespace vdn
