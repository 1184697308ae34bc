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
//   One workgroup = NW waves = one tile of 32*NW query rows of one (sample,
//   head, query block); each wave owns 32 query rows.  The key list of the
//   block is the virtual concatenation of <= 3 token intervals, walked in
//   steps of KT keys; only the last step can be partial.  Default shape: 8
//   waves (two per SIMD), 128 keys per step, a 2-stage LDS ring.
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

#include <cstdint>

#include "fwd_common.hpp"

#ifndef VDN_PIN_QK
#define VDN_PIN_QK 1
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
template <int D, int NW, int NS, int KT, int KPF, int VPF, bool FUSE>
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

  // ---- which tile (XCD-aware, the last tiles of each XCD in halves)
  const TileSlot slot = tile_slot(blockIdx.x, p.per_xcd, p.split_tail);
  const int t = slot.tile;
  if (t >= p.total_tiles) return;
  const int bh = t / p.tiles_per_bh;
  const int rank = undeal(t - bh * p.tiles_per_bh, p.tiles_per_bh, p.deal);
  const int b = bh / p.H;
  const int h = bh - b * p.H;
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

  const int64_t rs = int64_t(p.H) * D;  // token stride (elements)
  const int64_t rsb = rs * 2;           // token stride (bytes)
  const int64_t bh_off = int64_t(b) * p.S * rs + int64_t(h) * D;
  const __bf16* __restrict__ qg = static_cast<const __bf16*>(p.q) + bh_off;
  const char* __restrict__ kg = reinterpret_cast<const char*>(static_cast<const __bf16*>(p.k) + bh_off);
  const char* __restrict__ vg = reinterpret_cast<const char*>(static_cast<const __bf16*>(p.v) + bh_off);

  // ---- Q rows for this wave, kept in registers as MFMA B operands.
  bf16x8 qreg[NDS];
  {
    const int lrow = wave * QW + lr;
    const __bf16* src = qg + int64_t(row0 + lrow) * rs + hh * 8;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
      qreg[ds] = lrow < rows ? *reinterpret_cast<const bf16x8*>(src + ds * 16) : bf16x8{};
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
  int dma_row[NI];
  uint32_t k_goff[NI], v_goff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int q = wave * NI + i;
    const int r = q * RPI + lane / CH;
    const int pc = lane % CH;
    dma_row[i] = r;
    k_goff[i] = uint32_t(r * rsb + ((pc ^ (r % CH)) * 16));
    v_goff[i] = uint32_t(r * rsb + ((pc ^ vswz(r)) * 16));
  }

  // Addresses of one step's keys: a scalar base when the step lies inside
  // one key interval, else key by key (rows past the end of the key list are
  // clamped to its last key and masked out of the softmax).
  // (the tensor is a compile-time tag: choosing between the two offset arrays
  // at run time would force them out of registers)
  auto issue = [&](int step, char* lbase, auto is_k_c) {
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
    const int j0 = step * KT;
    // interval holding j0, its end and offset (scalar selects)
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
  const bool active = __builtin_amdgcn_readfirstlane(wave) * 32 < rows;
  const float c = p.score_scale_log2;
  const int nsteps = (n_keys + KT - 1) / KT;
  const bf16x2 kOnes2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

  // S^T = K Q^T for the KT keys in K stage `stage_c`.  The K fragments run
  // KPF reads ahead of the MFMAs that consume them (a read issued just
  // before its MFMA leaves the LDS latency on the critical path).
  auto qk = [&](const char* ks, f32x16 (&s)[NKB]) {
    constexpr int NF = NDS * NKB;  // fragments (= MFMAs) per step
    constexpr int PF = KPF < NF ? KPF : NF;
    auto frag = [&](int f) {
      return *reinterpret_cast<const bf16x8*>(ks + (f % NKB) * 32 * RB + k_roff(f / NKB));
    };
    bf16x8 fr[PF];
#pragma unroll
    for (int f = 0; f < PF; ++f) fr[f] = frag(f);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      s[f % NKB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[f % PF], qreg[f / NKB], s[f % NKB], 0, 0, 0);
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
  auto pv = [&](const char* vs, const bf16x8 (&pk)[NKB][2]) {
    constexpr int NF = NKB * 2 * NDB;  // fragments (= MFMAs) per step: (kb, half, db)
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
  auto row_max = [&](const f32x16 (&s)[NKB]) {
    // one running maximum per key block, each step folding two scores with
    // a three-input max (the compiler's own form takes a two-input max per
    // pair and a three-input max per two pairs: 3 ops per 4 scores, not 2)
    float mb[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      mb[kb] = fmaxf(s[kb][0], s[kb][1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2)
        asm("v_max3_f32 %0, %0, %1, %2" : "+v"(mb[kb]) : "v"(s[kb][r]), "v"(s[kb][r + 1]));
    }
    float mx = mb[0];
#pragma unroll
    for (int kb = 1; kb < NKB; ++kb) mx = fmaxf(mx, mb[kb]);
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
  // P = exp2(S c - m), packed to bf16; row sums over the rounded weights.
  auto exp_pack = [&](const f32x16 (&s)[NKB], bf16x8 (&pk)[NKB][2]) {
    const float mneg = -m_run;
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8 v8;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v8[e] = static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][half * 8 + e], c, mneg)));
        pk[kb][half] = v8;
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v8, v8, 0, 1), kOnes2, lsum, false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v8, v8, 2, 3), kOnes2, lsum, false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v8, v8, 4, 5), kOnes2, lsum, false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v8, v8, 6, 7), kOnes2, lsum, false);
      }
    }
    l_run += lsum;
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
  // one step; `last` (compile-time) makes it the fused kernel's last step,
  // which brings in the linear rows instead of re-fetching past the end
  auto body = [&](int step, auto stage_c, auto last_c) {
    constexpr int st = decltype(stage_c)::value;
    if constexpr (decltype(last_c)::value != 0) {
      issue_lin(lin_stage(IC<(st + NS - 1) % NS>{}));
    } else {
      issue(step + NS - 1, kstage(IC<(st + NS - 1) % NS>{}), IC<1>{});
      issue(step + NS - 1, vstage(IC<(st + NS - 1) % NS>{}), IC<0>{});
    }
    if (active) {
      f32x16 s[NKB];
      qk(kstage(stage_c), s);
      const int j0 = step * KT;
      if (j0 + KT > n_keys) mask_tail<NKB>(s, n_keys - j0, hh);
      rescale(row_max(s));
      bf16x8 pk[NKB][2];
      exp_pack(s, pk);
      pv(vstage(stage_c), pk);
    }
    // the next step reads K and V of step+1: batches step+2 .. step+NS-1
    // may still be in flight
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * 2 * NI));
    lds_barrier();
  };
  // prologue: steps 0 .. NS-2 in flight
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
  if constexpr (!FUSE) {
    for (int step = 0;;) {
      body(step, IC<0>{}, IC<0>{});
      if (++step >= nsteps) break;
      body(step, IC<1 % NS>{}, IC<0>{});
      if (++step >= nsteps) break;
      if constexpr (NS > 2) {
        body(step, IC<2 % NS>{}, IC<0>{});
        if (++step >= nsteps) break;
        body(step, IC<3 % NS>{}, IC<0>{});
        if (++step >= nsteps) break;
      }
    }
  } else {
    // the same loop with the last step (nsteps >= 1) taken out of it
    int step = 0;
    for (; step + 2 < nsteps; step += 2) {
      body(step, IC<0>{}, IC<0>{});
      body(step + 1, IC<1>{}, IC<0>{});
    }
    if (step + 2 == nsteps) {
      body(step, IC<0>{}, IC<0>{});
      body(step + 1, IC<1>{}, IC<1>{});
    } else {
      body(step, IC<0>{}, IC<1>{});
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no DMA outlives the workgroup

  // ---- epilogue: normalise, gate, store bf16, optional log-sum-exp
  __bf16* og = static_cast<__bf16*>(p.out) + bh_off;
  const int lrow = wave * QW + lr;
  const float l_tot = xhalf_sum(l_run);
  if (lrow < rows) {
    const int row = row0 + lrow;
    float scale = 1.0f / l_tot;
    if (p.gate != nullptr) {
      const float g = p.gate[(int64_t(b) * p.S + row) * p.H + h];
      scale *= 1.0f / (1.0f + __builtin_amdgcn_exp2f(-g * kLog2e));
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
          *reinterpret_cast<bf16x4*>(dst + db * 32 + g4 * 8 + hh * 4) = o4;
        }
      }
    } else {
      // the two branches summed before the one rounding: the token's
      // linear-branch row, scaled by its factor and the norm weight, joins
      // this row
      const float coef = lin_coef;
      // the row landed in LDS with the last step (stage (nsteps - 1 + NS - 1)
      // % NS, the one the last step did not read)
      const char* lrow_lds = ((nsteps - 1) % NS == 0 ? lin_stage(IC<1 % NS>{}) : lin_stage(IC<0>{})) + lr * RB;
      const float* wsrc = p.lin_w + h * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int col = db * 32 + g4 * 8 + hh * 4;
          const int c = (db * 4 + g4) ^ (lr % CH);
          const bf16x4 l4 = *reinterpret_cast<const bf16x4*>(lrow_lds + c * 16 + hh * 8);
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
    if (p.lse != nullptr && hh == 0) {
      p.lse[(int64_t(b) * p.H + h) * p.S + row] = (m_run + __log2f(l_tot)) * kLn2;
    }
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

int kernel_tile_m(int head_dim, int dtype) {
  (void)head_dim;
  (void)dtype;
  return 32 * kWaves;
}

int launch_fwd(const FwdParams& p, int head_dim, int dtype, void* stream) {
  const dim3 grid(unsigned(p.per_xcd + p.split_tail) * 8u);
  const dim3 block(64 * kWaves);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == 1) return launch_fwd_fp8(p, head_dim, stream);
  if (dtype != 0) return int(hipErrorInvalidValue);
  if (head_dim == 128) {
    if (p.lin != nullptr)
      hipLaunchKernelGGL((fwd_bf16_kernel<128, kWaves, 2, kKeysPerStep, kReadAhead, kReadAheadV, true>), grid, block, 0, st, p);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<128, kWaves, kStages, kKeysPerStep, kReadAhead, kReadAheadV, false>), grid, block, 0, st, p);
  } else if (head_dim == 64) {
    if (p.lin != nullptr)
      hipLaunchKernelGGL((fwd_bf16_kernel<64, kWaves, 2, kKeysPerStep, kReadAhead, kReadAheadV, true>), grid, block, 0, st, p);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<64, kWaves, kStages, kKeysPerStep, kReadAhead, kReadAheadV, false>), grid, block, 0, st, p);
  } else {
    return int(hipErrorInvalidValue);
  }
  return int(hipGetLastError());
}

}  // namespace vdn
