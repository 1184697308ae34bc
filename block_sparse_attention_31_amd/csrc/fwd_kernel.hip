// Block-sparse flash-attention forward for gfx950 (CDNA4), bf16 inputs.
//
// Computes the local Softmax branch of VDN-H3 hybrid video attention: each
// query token attends with exact softmax to its frame block and the two
// neighbouring blocks, the first/last-frame anchors and all text tokens
// (openi.cn "VDN-MiniMax-H3", technical principles; nav.superapi.store
// "VDN-MiniMax-H3 - OpenVDN's Open-Source Video Generation Acceleration
// Solution", Technical Principles), then applies the per-token sigmoid gate
// ("Gated Fusion Mechanism" on the same page).
//
// Work decomposition
//   A tile is 32*NW query rows of one (sample, head, query block); each wave
//   owns 32 of them.  The key list of the block is the virtual concatenation
//   of <= 3 token intervals, walked in steps of KT keys; only the last step
//   can be partial.  Default shape: 8 waves (two per SIMD), 128 keys per
//   step, a 2-stage LDS ring.  The launch is persistent: one resident
//   workgroup per CU takes tiles from its XCD's queue and, once that is
//   empty, from the other XCDs' (one atomic claim per tile).  A half tile
//   (128 rows, at the end of a queue) runs on all 8 waves with each step's
//   key blocks split between waves w and w+4, which merge their rows at the
//   end.
//
// Softmax
//   Each row's weights are exponentiated against a reference point fixed at
//   its first step's maximum + 16 (log2 units): no per-step maximum and no
//   rescale.  A row whose sum would pass 2^32 sends its workgroup through the
//   key list again under the online maximum.
//
// Matrix layout on the MFMA units (v_mfma_f32_32x32x16_bf16)
//   S^T = K Q^T: A = K rows from LDS, B = Q rows held in registers.  The
//   32x32 result puts one query per lane column: lane l holds query l%32 and
//   keys {8g + 4(l/32) + r}, so the row max/sum is an in-lane reduction plus
//   one exchange with lane l^32.
//   O^T = V^T P^T: B = P straight from the S^T registers (packed to bf16;
//   the key order inside the 32-key block only has to agree between A and
//   B), A = V^T fragments from transposing LDS reads of row-major V.  The
//   accumulator again has one query per lane, so the online-softmax rescale
//   is a per-lane scalar multiply.
//
// Fused instance (FUSE): the same kernel also adds the linear branch's gated,
// RMS-normalised output row before the one rounding (openi.cn "VDN-MiniMax-
// H3", technical principles: the branches are summed after the linear one's
// RMSNorm and gate); its rows come into LDS with the last step.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "fwd_common.hpp"

#ifndef VDN_PIN_QK
#define VDN_PIN_QK 1
#endif
// persistent workgroups take tiles from other XCDs' queues once their own is
// empty (1) or stop there (0)
#ifndef VDN_STEAL
#define VDN_STEAL 1
#endif
// row sums by bf16 dot products over the rounded weights (1) or fp32 adds (0)
#ifndef VDN_ROWSUM_DOT
#define VDN_ROWSUM_DOT 0
#endif

namespace vdn {

// K and V stream through a ring of NS LDS stages filled by
// global_load_lds_dwordx4 (16 bytes per lane, written to LDS at lane*16 of a
// wave-uniform base), NS-1 steps ahead of use; no register staging.  Rows are
// stored unpadded, 16-byte chunks XOR-swizzled so that fragment reads hit
// distinct banks:
//   K: chunk c of key row r is stored at chunk c ^ (r % (D/8)) -- the 32 rows
//      of a QK^T A-operand read are spread over all chunks;
//   V: chunk c of key row r is stored at chunk c ^ 4(r % 4) -- the four rows
//      read by 32 lanes of a ds_read_b64_tr_b16 land on different banks.
// V^T fragments come from two ds_read_b64_tr_b16 per MFMA: in each group of
// 16 lanes, lane i receives element (i % 4) of the 8-byte blocks addressed by
// lanes 4e + i/4 (e = 0..3), so if those lanes point at keys k+e, columns
// d0 + 4(i/4).., lane i holds V[k..k+3][d0 + i]: the MFMA A-operand layout.
template <int D, int NW, int NS, int KT, int KPF, int VPF, bool FUSE, bool FIXREF>
__global__ __launch_bounds__(NW * 64, 2) void fwd_bf16_kernel(const FwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  constexpr int QW = 32;          // query rows per wave
  constexpr int M = NW * QW;      // query rows per workgroup
  constexpr int RB = 2 * D;       // bytes per key row
  constexpr int CH = D / 8;       // 16-byte chunks per row
  constexpr int TILE = KT * RB;   // bytes per K (or V) stage
  constexpr int NI = TILE / 1024 / NW;  // DMA instructions per wave per tensor per step
  constexpr int RPI = 1024 / RB;  // key rows per DMA instruction
  constexpr int NDS = D / 16;     // k-steps of the QK^T MFMA
  constexpr int NDB = D / 32;     // 32-wide d blocks of the output
  constexpr int NKB = KT / 32;    // 32-key blocks per step
  static_assert(NI >= 1 && NI * NW * 1024 == TILE, "tile shape");
  static_assert(NS == 2 || NS == 4, "the main loop is unrolled for a 2- or 4-stage ring");
  static_assert(!FIXREF || NS == 2, "the fixed-reference loop is unrolled for a 2-stage ring");
  static_assert(!FUSE || (NS == 2 && NW == 8 && TILE >= 4 * 32 * RB),
                "the fused epilogue stages each wave's 32 linear rows in the two free ring stages");
  // V row swizzle: whole groups of four 16-byte chunks move with key % 4, so
  // the 32 lanes of a transposing read (4 keys x 32 columns) cover all banks.
  auto vswz = [](int r) { return (4 * (r & 3)) % CH; };

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

  __shared__ int redo;    // the workgroup's vote for an online-maximum rerun
  __shared__ int s_next;  // the next tile's slot, handed from wave 0 to the others

  // One query tile, given its slot in the XCD queues (slot w: queue w % 8,
  // position w / 8).  `claim` is the pending claim on the home queue, issued
  // once the tile's first DMA has landed so that its latency hides under the
  // first step.
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
  // The block's descriptor, copied once into wave-uniform registers (reading
  // the kernel-argument table with a runtime index inside the loop would be a
  // vector-memory load, and its wait would also drain the DMA in flight).
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
  // A half tile (128 rows) runs on all 8 waves with the keys of every step
  // split between two: waves w and w+4 take the same 32 rows, key blocks
  // 0-1 and 2-3 of each step, and merge their partial rows at the end.  Not
  // in the fused instance, nor for a key list of one step of at most KT/2
  // keys (the second half of its only step would hold no key).
  const bool ksplit = !FUSE && slot.half != 0 && n_keys > KT / 2;
  const int rwave = ksplit ? (wave & 3) : wave;  // which 32 rows of the tile
  const int kbo = ksplit ? (NKB / 2) * (wave >> 2) : 0;  // first key block of the step

  const int64_t rs = int64_t(p.H) * D;  // token stride (elements)
  const int64_t rsb = rs * 2;           // token stride (bytes)
  const int64_t bh_off = int64_t(b) * p.S * rs + int64_t(h) * D;
  const __bf16* __restrict__ qg = static_cast<const __bf16*>(p.q) + bh_off;
  const char* __restrict__ kg = reinterpret_cast<const char*>(static_cast<const __bf16*>(p.k) + bh_off);
  const char* __restrict__ vg = reinterpret_cast<const char*>(static_cast<const __bf16*>(p.v) + bh_off);

  // ---- Q rows for this wave, kept in registers as MFMA B operands.
  bf16x8 qreg[NDS];
  {
    const int lrow = rwave * QW + lr;
    const __bf16* src = qg + int64_t(row0 + lrow) * rs + hh * 8;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
      qreg[ds] = lrow < rows ? *reinterpret_cast<const bf16x8*>(src + ds * 16) : bf16x8{};
  }
  // The row's gate logit, read with Q so that its load overlaps Q's.
  float g_pre = 0.f;
  {
    const int lrow = rwave * QW + lr;
    if (p.gate != nullptr && lrow < rows) g_pre = p.gate[(int64_t(b) * p.S + row0 + lrow) * p.H + h];
  }
  // With the two-branch fusion: the row's linear-branch factor, sigmoid of
  // its gate over the token's RMS (from the per-head sums of squares), read
  // here so that its loads overlap Q's.
  float lin_coef = 0.f;
  if constexpr (FUSE) {
    const int lrow = wave * QW + lr;
    if (lrow < rows) {
      const int64_t tok = int64_t(b) * p.S + row0 + lrow;
      const float* ssr = p.lin_ss + tok * p.H;
      float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int i = 0; i < p.H; ++i) s4[i & 3] += ssr[i];
      const float gl = 1.f / (1.f + __builtin_amdgcn_exp2f(-p.gate_lin[tok * p.H + h] * kLog2e));
      lin_coef = gl / __builtin_sqrtf((s4[0] + s4[1] + s4[2] + s4[3]) / float(p.H * D) + p.lin_eps);
    }
  }
  // Q lands before any DMA is issued: the compiler cannot count the DMA, and
  // with its own loads still pending at the loop it would wait on the whole
  // ring inside every step
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  f32x16 acc[NDB];
  float m_run = -__builtin_inff(), l_run = 0.f;
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  // ---- DMA addressing.  Instruction i of this wave covers key rows
  // dma_row[i] .. (RPI rows per instruction); lane -> (row, physical chunk);
  // it fetches the logical chunk that the swizzle stores there.
  // Row of instruction i is r0 + i RPI.  The K swizzle XORs the chunk with
  // r % CH = (r0 % CH) ^ ((i RPI) % CH) (r0 % CH < RPI, so no carry), the V
  // swizzle depends on r % 4 = r0 % 4 only; so one lane offset per tensor
  // serves every instruction: instruction i adds i RPI rows through the
  // scalar base and, for K, XORs a constant into the chunk.
  const int r0 = wave * NI * RPI + lane / CH;
  const uint32_t k_chunk0 = uint32_t(((lane % CH) ^ (r0 % CH)) * 16);
  const uint32_t v_chunk0 = uint32_t(((lane % CH) ^ vswz(r0)) * 16);
  auto kx = [](int i) { return uint32_t(((i * RPI) % CH) * 16); };

  // Addresses of one step's keys: a scalar base when the step lies inside
  // one key interval, else key by key (rows past the end of the key list are
  // clamped to its last key and masked out of the softmax).
  // (the tensor is a compile-time tag)
  auto issue = [&](int step, char* lbase, auto is_k_c) __attribute__((always_inline)) {
    constexpr bool is_k = decltype(is_k_c)::value != 0;
    const char* gbase = is_k ? kg : vg;
    const uint32_t chunk0 = is_k ? k_chunk0 : v_chunk0;
    const int j0 = step * KT;
    // interval holding j0, its end and offset (scalar selects)
    const int iv_end = interval_end(kl, j0);
    const int delta = interval_delta(kl, j0);
    // This wave's LDS destination, recomputed at every call (opaque to the
    // compiler): hoisted, the per-instruction destinations of both stages and
    // tensors would hold a dozen scalar registers across the loop.
    uint32_t wdst = uint32_t(wave * NI * 1024);
    asm volatile("" : "+s"(wdst));
    if (j0 + KT <= iv_end) {
      const char* base = gbase + int64_t(j0 + delta) * rsb;
      int64_t step_b = int64_t(RPI) * rsb;
      asm volatile("" : "+s"(step_b));
      const uint32_t off0 = uint32_t(r0 * rsb) + chunk0;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        lds_dma16(base, is_k ? off0 ^ kx(i) : off0, lbase + wdst + i * 1024);
        base += step_b;
      }
    } else {
      // (chunk offset opaque here: its per-instruction 64-bit forms are then
      // formed on this rare path, not held in registers across the loop)
      uint32_t ch0 = chunk0;
      asm volatile("" : "+v"(ch0));
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int j = min(j0 + r0 + i * RPI, n_keys - 1);
        lds_dma16(gbase + int64_t(vtoken(kl, j)) * rsb + (is_k ? ch0 ^ kx(i) : ch0),
                  lbase + wdst + i * 1024);
      }
    }
  };

  // ---- LDS read offsets (bytes, relative to a stage).
  // K A-operand for k-step ds: row lr (+32 kb), logical chunk 2 ds + hh,
  // stored at chunk (2 ds + hh) ^ (lr % CH): bits 5.. of the offset carry
  // ds, so the offset for ds is k_roff0 ^ (32 ds) (one VALU op per read
  // instead of a register per k-step).
  const uint32_t k_roff0 = uint32_t(lr * RB + ((hh ^ (lr % CH)) * 16));
  auto k_roff = [&](int ds) { return k_roff0 ^ uint32_t(32 * ds); };
  // V^T A-operand (tr reads) for d block db: 16-lane group g, lane i in it:
  // key 4 hh + i/4 (+ 32 kb + 16 half + 8 r), columns 32 db + 16 (g % 2) + 4 (i % 4).
  // db only moves bits 6.. of the offset (chunk bits 2..), which the V
  // swizzle XORs, so the offset for db is v_roff0 ^ (64 db).
  uint32_t v_roff0;
  {
    const int g = lane >> 4, i = lane & 15;
    const int key = 4 * hh + (i >> 2);
    const int col = 16 * (g & 1) + 4 * (i & 3);
    const int chunk = (col >> 3) ^ vswz(key);
    v_roff0 = uint32_t(key * RB + chunk * 16 + (col & 7) * 2);
  }
  auto v_roff = [&](int db) { return v_roff0 ^ uint32_t(64 * db); };

  // a wave whose rows all lie past the end of the query block (the last
  // tile of a block) only helps with the DMA and the barriers
  const bool active = rwave * 32 < rows;
  const float c = p.score_scale_log2;
  const int nsteps = (n_keys + KT - 1) / KT;
  [[maybe_unused]] const bf16x2 kOnes2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

  // S^T = K Q^T for the KT keys in K stage `stage_c`.  The K fragments run
  // KPF reads ahead of the MFMAs that consume them (a read issued just
  // before its MFMA leaves the LDS latency on the critical path).
  auto qk = [&](const char* ks, auto& s) {
    constexpr int NK = std::extent<std::remove_reference_t<decltype(s)>>::value;  // key blocks
    constexpr int NF = NDS * NK;  // fragments (= MFMAs) per step
    constexpr int PF = KPF < NF ? KPF : NF;
    // fragment f: key block f % NK, k-step f / NK (the NK accumulators
    // rotate, so consecutive MFMAs never share one)
    auto frag = [&](int f) {
      return *reinterpret_cast<const bf16x8*>(ks + (f % NK) * 32 * RB + k_roff(f / NK));
    };
    bf16x8 fr[PF];
#pragma unroll
    for (int f = 0; f < PF; ++f) fr[f] = frag(f);
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      s[f % NK] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[f % PF], qreg[f / NK], s[f % NK], 0, 0, 0);
      if (f + PF < NF) fr[f % PF] = frag(f + PF);
#if VDN_PIN_QK
      // keep this order: the scheduler would otherwise pull the reads back
      // next to their MFMAs to save registers
      __builtin_amdgcn_sched_barrier(0);
#endif
    }
  };

  // O^T += V^T P^T for the KT keys in V stage `stage_c` (V^T fragments by
  // transposing LDS reads).
  auto pv = [&](const char* vs, const auto& pk) {
    constexpr int NK = std::extent<std::remove_reference_t<decltype(pk)>>::value;  // key blocks
    constexpr int NF = NK * 2 * NDB;  // fragments (= MFMAs) per step: (kb, half, db)
    constexpr int PF = VPF < NF ? VPF : NF;
    auto frag = [&](int f) {
      const int db = f % NDB, kh = f / NDB;  // kh = 2 kb + half
      const char* base = vs + kh * 16 * RB + v_roff(db);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base + 8 * RB));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 fr[PF];
#pragma unroll
    for (int f = 0; f < PF; ++f) fr[f] = frag(f);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int db = f % NDB, kh = f / NDB;
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[f % PF], pk[kh / 2][kh % 2], acc[db], 0, 0, 0);
      if (f + PF < NF) fr[f % PF] = frag(f + PF);
    }
  };

  // Row maximum of a step's scores (both halves of the wave), in log2 units.
  auto row_max = [&](const auto& s) {
    constexpr int NK = std::extent<std::remove_reference_t<decltype(s)>>::value;
    // one running maximum per key block, each step folding two scores with
    // a three-input max (the compiler's own form takes a two-input max per
    // pair and a three-input max per two pairs: 3 ops per 4 scores, not 2)
    float mb[NK];
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) {
      mb[kb] = fmaxf(s[kb][0], s[kb][1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2)
        asm("v_max3_f32 %0, %0, %1, %2" : "+v"(mb[kb]) : "v"(s[kb][r]), "v"(s[kb][r + 1]));
    }
    float mx = mb[0];
#pragma unroll
    for (int kb = 1; kb < NK; ++kb) mx = fmaxf(mx, mb[kb]);
    return xhalf_max(mx) * c;
  };
  // Raise the running maximum only when the step's maximum exceeds it by
  // more than the slack; the accumulator and row sum are rescaled then.
  auto rescale = [&](float mx) {
    if (__any(mx > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }
  };
  // P = exp2(S c - m), packed to bf16, and its row sum.  The row sum adds
  // the fp32 weights (two partial sums per lane): the bf16 dot-product form
  // over the rounded weights issues on the matrix pipe's side of the SIMD
  // and stalls the MFMAs running beside it, while fp32 adds co-issue.
  auto exp_pack = [&](const auto& s, auto& pk) {
    constexpr int NK = std::extent<std::remove_reference_t<decltype(s)>>::value;
    const float mneg = -m_run;
    float l0 = 0.f, l1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8 v8;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][half * 8 + e], c, mneg));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][half * 8 + e + 1], c, mneg));
          v8[e] = static_cast<__bf16>(p0);
          v8[e + 1] = static_cast<__bf16>(p1);
#if VDN_ROWSUM_DOT
          const bf16x2 pr = {v8[e], v8[e + 1]};
          l0 = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes2, l0, false);
#else
          l0 += p0;
          l1 += p1;
#endif
        }
        pk[kb][half] = v8;
      }
    }
    l_run += l0 + l1;
  };

  // ---- main loop: per step, S = K Q^T, softmax, O += P V, with the
  // K and V of the next NS-1 steps landing meanwhile.  Every step issues
  // exactly one batch (past the end of the key list a harmless re-fetch
  // of the last key into the free stage), so the wait count is the same
  // on every step.
  // With the fused epilogue, the last step brings this wave's 32 rows of the
  // linear-branch output into the free stage pair instead of re-fetching past
  // the end of the key list (waves 0-3 into the K stage, 4-7 into the V
  // stage, 32 rows each; 16-byte chunk c of row r at c ^ (r % CH)).
  auto lin_stage = [&](auto stage_c) -> char* {
    return wave < 4 ? kstage(stage_c) + wave * 32 * RB : vstage(stage_c) + (wave - 4) * 32 * RB;
  };
  auto issue_lin = [&](char* dst) {
    const char* lg = static_cast<const char*>(p.lin) + bh_off * 2;
#pragma unroll
    for (int i = 0; i < 32 * RB / 1024; ++i) {
      const int r = i * RPI + lane / CH, c = (lane % CH) ^ (r % CH);
      const int grow = row0 + min(wave * QW + r, rows - 1);
      lds_dma16(lg + int64_t(grow) * rsb + c * 16, dst + i * 1024);
    }
  };
  // One step.  `last` (compile-time) makes it the fused kernel's last step,
  // which brings in the linear rows instead of re-fetching past the end.
  // `kind`: kOnline keeps the running maximum (raised by more than the
  // slack, with a rescale); kFirst sets the reference point of the row to
  // the step's maximum; kFixed exponentiates against the reference point as
  // it stands, with no maximum and no branch between the two products.
  // `tail` (compile-time) allows a partial step (masked past the end of the
  // key list).
  constexpr int kOnline = 0, kFirst = 1, kFixed = 2;
  // `ks_c` (compile-time) selects the key-split half tile: this wave's half of
  // every step's key blocks.
  auto body = [&](int step, auto stage_c, auto last_c, auto kind_c, auto tail_c, auto ks_c) __attribute__((always_inline)) {
    constexpr int st = decltype(stage_c)::value;
    constexpr int kind = decltype(kind_c)::value;
    constexpr bool KS = decltype(ks_c)::value != 0;
    constexpr int NK = KS ? NKB / 2 : NKB;  // key blocks of the step this wave scores
    constexpr bool LAST = decltype(last_c)::value != 0;
    if constexpr (LAST) issue_lin(lin_stage(IC<(st + NS - 1) % NS>{}));
    // K of step + NS - 1 goes out once this step's QK products are issued,
    // V once its weights are formed (waves with no rows issue both at once).
    // Issued together at the start of the step, the batch held back the QK
    // products behind it.
    auto dma_k = [&]() __attribute__((always_inline)) {
      if constexpr (!LAST) issue(step + NS - 1, kstage(IC<(st + NS - 1) % NS>{}), IC<1>{});
    };
    auto dma_v = [&]() __attribute__((always_inline)) {
      if constexpr (!LAST) issue(step + NS - 1, vstage(IC<(st + NS - 1) % NS>{}), IC<0>{});
    };
    // The claim on the next tile goes out with the tile's last step (the one
    // that may be partial; the first such step once, so a rerun or the
    // online loop claims early): tiles are then handed out in the order their
    // workgroups finish, and the end-of-step wait covers the atomic.
    if constexpr (!FUSE && decltype(tail_c)::value != 0) claim.issue(p.queue, tid);
    if (active) {
      const int kofs = KS ? kbo * 32 * RB : 0;  // bytes to the wave's first key block
      f32x16 s[NK];
      qk(kstage(stage_c) + kofs, s);
      dma_k();
      if constexpr (decltype(tail_c)::value != 0) {
        const int j0 = step * KT + (KS ? 32 * kbo : 0);
        if (step * KT + KT > n_keys) mask_tail<NK>(s, n_keys - j0, hh);
      }
      if constexpr (kind == kOnline) {
        rescale(row_max(s));
      } else if constexpr (kind == kFirst) {
        m_run = row_max(s) + kRefHeadroom;
      }
      bf16x8 pk[NK][2];
      exp_pack(s, pk);
      dma_v();
      pv(vstage(stage_c) + kofs, pk);
    } else {
      dma_k();
      dma_v();
    }
    // the next step reads K and V of step+1: batches step+2 .. step+NS-1
    // may still be in flight
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * 2 * NI));
    lds_barrier();
  };
  // prologue: steps 0 .. NS-2 in flight
  auto prologue = [&]() __attribute__((always_inline)) {
    issue(0, kstage(IC<0>{}), IC<1>{});
    issue(0, vstage(IC<0>{}), IC<0>{});
    if constexpr (NS > 2) {
      issue(1, kstage(IC<1>{}), IC<1>{});
      issue(1, vstage(IC<1>{}), IC<0>{});
      issue(2, kstage(IC<2 % NS>{}), IC<1>{});
      issue(2, vstage(IC<2 % NS>{}), IC<0>{});
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * 2 * NI));  // step 0 has landed
    lds_barrier();
  };
  // The whole key list with the online maximum.
  auto run_online = [&](auto ks_c) __attribute__((always_inline)) {
    prologue();
    if constexpr (!FUSE) {
      for (int step = 0;;) {
        body(step, IC<0>{}, IC<0>{}, IC<kOnline>{}, IC<1>{}, ks_c);
        if (++step >= nsteps) break;
        body(step, IC<1 % NS>{}, IC<0>{}, IC<kOnline>{}, IC<1>{}, ks_c);
        if (++step >= nsteps) break;
        if constexpr (NS > 2) {
          body(step, IC<2 % NS>{}, IC<0>{}, IC<kOnline>{}, IC<1>{}, ks_c);
          if (++step >= nsteps) break;
          body(step, IC<3 % NS>{}, IC<0>{}, IC<kOnline>{}, IC<1>{}, ks_c);
          if (++step >= nsteps) break;
        }
      }
    } else {
      // the same loop with the last step (nsteps >= 1) taken out of it
      int step = 0;
      for (; step + 2 < nsteps; step += 2) {
        body(step, IC<0>{}, IC<0>{}, IC<kOnline>{}, IC<1>{}, ks_c);
        body(step + 1, IC<1>{}, IC<0>{}, IC<kOnline>{}, IC<1>{}, ks_c);
      }
      if (step + 2 == nsteps) {
        body(step, IC<0>{}, IC<0>{}, IC<kOnline>{}, IC<1>{}, ks_c);
        body(step + 1, IC<1>{}, IC<1>{}, IC<kOnline>{}, IC<1>{}, ks_c);
      } else {
        body(step, IC<0>{}, IC<1>{}, IC<kOnline>{}, IC<1>{}, ks_c);
      }
    }
  };
  // Every row's weights are exponentiated against a fixed reference point.
  // It starts kRefHeadroom above the row's first-step maximum, so the row
  // sum is at least 2^-kRefHeadroom and a weight lost to underflow
  // (< 2^-126) is below 2^-110 of the largest.  Results are exact up to
  // rounding unless a later key exceeds the point by so much that a weight
  // overflows: a row sum above 2^32 (no weight above it, no sum near the
  // fp32 range) sends the workgroup through the key list again.
  auto vote_redo = [&]() __attribute__((always_inline)) {
    const float l_chk = xhalf_sum(l_run);
    const bool bad = rwave * QW + lr < rows && !(l_chk <= 0x1p32f);
    if (tid == 0) redo = 0;
    lds_barrier();
    if (__any(bad) && lane == 0) redo = 1;
    lds_barrier();
    const bool again = __builtin_amdgcn_readfirstlane(redo) != 0;
    lds_barrier();  // every wave has read the flag before it is reset or the ring refills
    return again;
  };
  auto reset = [&]() __attribute__((always_inline)) {
    l_run = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  };
  auto run_keys = [&](auto ks_c) __attribute__((always_inline)) {
  if constexpr (FIXREF) {
    // step 0 sets the reference point (peeled); only the last step can be
    // partial (peeled; fused, it fetches the linear rows); a rerun takes the
    // online maximum
    prologue();
    if (nsteps == 1) {
      body(0, IC<0>{}, IC<FUSE ? 1 : 0>{}, IC<kFirst>{}, IC<1>{}, ks_c);
    } else {
      body(0, IC<0>{}, IC<0>{}, IC<kFirst>{}, IC<0>{}, ks_c);
      int step = 1;
      for (; step + 2 < nsteps; step += 2) {
        body(step, IC<1>{}, IC<0>{}, IC<kFixed>{}, IC<0>{}, ks_c);
        body(step + 1, IC<0>{}, IC<0>{}, IC<kFixed>{}, IC<0>{}, ks_c);
      }
      if (step + 2 == nsteps) {
        body(step, IC<1>{}, IC<0>{}, IC<kFixed>{}, IC<0>{}, ks_c);
        body(step + 1, IC<0>{}, IC<FUSE ? 1 : 0>{}, IC<kFixed>{}, IC<1>{}, ks_c);
      } else {
        body(step, IC<1>{}, IC<FUSE ? 1 : 0>{}, IC<kFixed>{}, IC<1>{}, ks_c);
      }
    }
    if (vote_redo()) {
      m_run = -__builtin_inff();
      reset();
      run_online(ks_c);
    }
  } else {
    run_online(ks_c);
  }
  };
  if (ksplit)
    run_keys(IC<1>{});
  else
    run_keys(IC<0>{});
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no DMA outlives the workgroup
  if (ksplit) {
    // Waves 4-7 hand their partial rows (accumulator, reference point, row
    // sum, in the same lane layout) to the wave with the same rows, through
    // the ring, which every wave has finished reading and whose last DMA
    // has landed once all have passed the barrier.
    lds_barrier();
    float* xacc = reinterpret_cast<float*>((wave & 2) ? Ks1 : Ks0) + (wave & 1) * (NDB * 16 * 64);
    float* xml = reinterpret_cast<float*>(Vs0) + (wave & 3) * 128;
    if (wave >= 4) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xacc[(db * 16 + r) * 64 + lane] = acc[db][r];
      xml[lane] = m_run;
      xml[64 + lane] = l_run;
    }
    lds_barrier();
    if (wave < 4) {
      const float mp = xml[lane], lp = xml[64 + lane];
      const float mn = fmaxf(m_run, mp);
      const float aw = __builtin_amdgcn_exp2f(m_run - mn), ap = __builtin_amdgcn_exp2f(mp - mn);
      l_run = l_run * aw + lp * ap;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = acc[db][r] * aw + xacc[(db * 16 + r) * 64 + lane] * ap;
      m_run = mn;
    }
  }

  // ---- epilogue: normalise, gate, store bf16, optional log-sum-exp
  // (lane-derived offsets re-formed here from an opaque thread index, so
  // that they are not hoisted out of the tile loop and held across the steps)
  int etid = threadIdx.x;
  asm volatile("" : "+v"(etid));
  const int lr_e = etid & 31, hh_e = (etid >> 5) & 1;
  __bf16* og = static_cast<__bf16*>(p.out) + bh_off;
  const int lrow = wave * QW + lr_e;
  const float l_tot = xhalf_sum(l_run);
  if (lrow < rows && !(ksplit && wave >= 4)) {
    const int row = row0 + lrow;
    float scale = 1.0f / l_tot;
    if (p.gate != nullptr) {
      scale *= 1.0f / (1.0f + __builtin_amdgcn_exp2f(-g_pre * kLog2e));
    }
    __bf16* dst = og + int64_t(row) * rs;
    if constexpr (!FUSE) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bf16x4 o4;
#pragma unroll
          for (int r = 0; r < 4; ++r) o4[r] = static_cast<__bf16>(acc[db][g4 * 4 + r] * scale);
          *reinterpret_cast<bf16x4*>(dst + db * 32 + g4 * 8 + hh_e * 4) = o4;
        }
      }
    } else {
      // the two branches summed before the one rounding: the token's
      // linear-branch row, scaled by its factor and the norm weight, joins
      // this row
      const float coef = lin_coef;
      // the row landed in LDS with the last step (stage (nsteps - 1 + NS - 1)
      // % NS, the one the last step did not read)
      const char* lrow_lds = ((nsteps - 1) % NS == 0 ? lin_stage(IC<1 % NS>{}) : lin_stage(IC<0>{})) + lr_e * RB;
      const float* wsrc = p.lin_w + h * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int col = db * 32 + g4 * 8 + hh_e * 4;
          const int c = (db * 4 + g4) ^ (lr_e % CH);
          const bf16x4 l4 = *reinterpret_cast<const bf16x4*>(lrow_lds + c * 16 + hh_e * 8);
          const float4 w4 = *reinterpret_cast<const float4*>(wsrc + col);
          const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
          bf16x4 o4;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            o4[r] = static_cast<__bf16>(__builtin_fmaf(coef * wv[r], float(l4[r]), acc[db][g4 * 4 + r] * scale));
          *reinterpret_cast<bf16x4*>(dst + col) = o4;
        }
      }
    }
    if (p.lse != nullptr && hh_e == 0) {
      p.lse[(int64_t(b) * p.H + h) * p.S + row] = (m_run + __log2f(l_tot)) * kLn2;
    }
  }
  };  // run_tile

  // Each workgroup starts on its own slot.  Persistent (p.queue set), it
  // then claims slots of its home queue (block index % 8, the XCD it runs
  // on) and, once that is empty, of the other XCDs' queues; the last one out
  // resets the counters.  Otherwise that one slot is all.
  if constexpr (FUSE) {
    // (the fused instance runs one tile per workgroup: its registers are
    // already at the limit, and the tile loop's would spill in the steps)
    PendingClaim none;
    run_tile(blockIdx.x, none);
    return;
  }
  int wslot = blockIdx.x;
  int steal = VDN_STEAL ? 1 : 8;  // next queue to try once the home queue is empty
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

// The bf16 kernel's shape: waves per workgroup (32 query rows each), keys
// per step and LDS ring stages.
#ifndef VDN_BF16_NW
#define VDN_BF16_NW 8
#endif
#ifndef VDN_BF16_KT
#define VDN_BF16_KT 128
#endif
#ifndef VDN_BF16_NS
#define VDN_BF16_NS 2
#endif
#ifndef VDN_BF16_KPF
#define VDN_BF16_KPF 4
#endif
constexpr int kWaves = VDN_BF16_NW;
constexpr int kKeysPerStep = VDN_BF16_KT;
constexpr int kStages = VDN_BF16_NS;
constexpr int kReadAhead = VDN_BF16_KPF;  // K fragments in flight ahead of the QK MFMAs
#ifndef VDN_BF16_VPF
#define VDN_BF16_VPF 2
#endif
constexpr int kReadAheadV = VDN_BF16_VPF;  // V^T fragments in flight ahead of the PV MFMAs
// Each row's reference point for the exponentials fixed at its first step's
// maximum (with a range check and an online-maximum rerun), or the online
// maximum throughout.
#ifndef VDN_FIXREF
#define VDN_FIXREF 1
#endif
constexpr bool kFixRef = VDN_FIXREF != 0;

int kernel_tile_m(int head_dim, int dtype) {
  (void)head_dim;
  (void)dtype;
  return 32 * kWaves;
}

namespace {
// Claim counters of the persistent launches (zero at load; every launch
// leaves its set zero again).
__device__ int fwd_queues[kQueueSlots * kQueueInts];

// Per device: the counters' address and, per kernel instance, the
// workgroups per XCD that fill the device (0: not persistent).
struct QueueDevice {
  int* base = nullptr;
  int wg[kQueueKernels] = {-1, -1, -1};
};
std::mutex g_queue_mu;
QueueDevice g_queue_dev[kMaxScratchDevices];
std::atomic<unsigned> g_queue_seq{0};
}  // namespace

// The counter set and workgroups per XCD for one launch of `kernel` (one
// resident workgroup per CU as its resources allow, the CUs split evenly
// over the 8 XCDs), or queue = nullptr for a launch of one workgroup per
// slot.  `kind` < kQueueKernels names the kernel instance.
int queue_for(const void* kernel, int kind, int* wg_per_xcd, int** queue) {
  *queue = nullptr;
  *wg_per_xcd = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  if (dev < 0 || dev >= kMaxScratchDevices) return 0;
  std::lock_guard<std::mutex> lock(g_queue_mu);
  QueueDevice& qd = g_queue_dev[dev];
  if (qd.base == nullptr) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(fwd_queues));
    if (e != hipSuccess) return int(e);
    qd.base = static_cast<int*>(addr);
  }
  int& wg = qd.wg[kind];
  if (wg < 0) {
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return int(e);
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * kWaves, 0);
    if (e != hipSuccess) return int(e);
    wg = cus % 8 == 0 ? per_cu * (cus / 8) : 0;
  }
  *wg_per_xcd = wg;
  if (wg > 0) *queue = qd.base + int64_t(g_queue_seq.fetch_add(1) % kQueueSlots) * kQueueInts;
  return 0;
}

namespace {

template <int D, bool FUSE>
int launch_bf16(const FwdParams& p_in, hipStream_t st) {
  constexpr int NS = FUSE ? 2 : kStages;
  const auto kernel = fwd_bf16_kernel<D, kWaves, NS, kKeysPerStep, kReadAhead, kReadAheadV, FUSE, kFixRef>;
  FwdParams p = p_in;
  p.queue = nullptr;
  p.queue_wg = 0;
  const int slots = p.per_xcd + p.split_tail;  // per XCD queue
  int wg = 0;
  int* queue = nullptr;
  if constexpr (!FUSE) {
    const int rc = queue_for(reinterpret_cast<const void*>(kernel), D == 128 ? kQueueBf16D128 : kQueueBf16D64, &wg, &queue);
    if (rc != 0) return rc;
  }
  dim3 grid(unsigned(slots) * 8u);
  if (!FUSE && queue != nullptr && wg < slots) {
    p.queue = queue;
    p.queue_wg = wg;
    grid = dim3(unsigned(wg) * 8u);
  }
  hipLaunchKernelGGL(kernel, grid, dim3(64 * kWaves), 0, st, p);
  return int(hipGetLastError());
}
}  // namespace

int launch_fwd(const FwdParams& p, int head_dim, int dtype, void* stream) {
  if (dtype == 1) return launch_fwd_fp8(p, head_dim, stream);
  if (dtype != 0) return int(hipErrorInvalidValue);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool fuse = p.lin != nullptr;
  if (head_dim == 128) return fuse ? launch_bf16<128, true>(p, st) : launch_bf16<128, false>(p, st);
  if (head_dim == 64) return fuse ? launch_bf16<64, true>(p, st) : launch_bf16<64, false>(p, st);
  return int(hipErrorInvalidValue);
}

}  // namespace vdn
