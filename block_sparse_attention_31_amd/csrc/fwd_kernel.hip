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
//   One workgroup = 4 waves = one tile of M query rows of one (sample, head,
//   query block); each wave owns 32*QB query rows.  The key list of the block
//   is the virtual concatenation of <= 3 token intervals, walked in steps of
//   KT = 64 keys; only the last step can be partial.
//
// Matrix layout on the MFMA units (v_mfma_f32_32x32x16_bf16)
//   S^T = K Q^T: A = K rows from LDS, B = Q rows held in registers.  The
//   32x32 result puts one query per lane column: lane l holds query l%32 and
//   keys {8g + 4(l/32) + r}, so the row max/sum is an in-lane reduction plus
//   one exchange with lane l^32.
//   O^T = V^T P^T: B = P straight from the S^T registers (packed to bf16),
//   A = V^T read from an LDS copy of V stored transposed, with keys placed so
//   that the 8 keys a half-wave contributes are contiguous (bits 2 and 3 of
//   the key index swapped).  The accumulator again has one query per lane,
//   so the online-softmax rescale is a per-lane scalar multiply.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fwd_params.hpp"

namespace vdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int vtoken(const QBlockDesc& d, int j) {
  int t = j + d.iv_delta[0];
  if (d.n_iv > 1 && j >= d.iv_start[1]) t = j + d.iv_delta[1];
  if (d.n_iv > 2 && j >= d.iv_start[2]) t = j + d.iv_delta[2];
  return t;
}

// Position of key r (0..KT-1) inside the transposed V tile: bits 2 and 3
// swapped, so that within each group of 16 keys the two half-waves' key sets
// {0-3, 8-11} and {4-7, 12-15} become contiguous runs of 8.
__device__ __forceinline__ int vt_pos(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Online-softmax reference point may lag the running maximum by up to 2^8 in
// the base-2 domain: P then stays below 256, exact in bf16 up to rounding,
// and the accumulator rescale is skipped unless the maximum grows by more.
constexpr float kRescaleSlack = 8.0f;

template <int D, int QB, int NW>
__global__ __launch_bounds__(NW * 64, 2) void fwd_bf16_kernel(const FwdParams p) {
  constexpr int QW = 32 * QB;     // query rows per wave
  constexpr int M = NW * QW;      // query rows per workgroup
  constexpr int KT = 64;          // keys per step
  constexpr int KP = D + 8;       // K tile row pitch (bf16), 16-byte pad
  constexpr int VP = KT + 8;      // V^T tile row pitch (bf16), 16-byte pad
  constexpr int DC = D / 8;       // 16-byte chunks per row
  // Staging: threads [K0, K0 + 256) load K, threads [0, 256) load V (with 8
  // waves the two halves of the workgroup split the work).
  constexpr int K0 = NW > 4 ? 256 : 0;
  constexpr int KCH = KT * DC / 256;          // K chunks per K thread
  constexpr int VITEMS = (KT / 4) * DC;       // (4 keys x 8 d) V items
  constexpr int NDS = D / 16;     // k-steps of the QK^T MFMA
  constexpr int NDB = D / 32;     // 32-wide d blocks of the output
  constexpr int NKB = KT / 32;    // 32-key blocks per step
  constexpr int KBUF = KT * KP;
  constexpr int VBUF = D * VP;
  static_assert(KCH >= 1 && VITEMS <= 256, "tile shape");

  // Two LDS buffers: step s computes from buffer s&1 while step s+1's tile
  // is staged into the other one.
  __shared__ __attribute__((aligned(16))) __bf16 Ks[2 * KBUF];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[2 * VBUF];

  // ---- which tile: XCD-aware remap so that consecutive tiles of one
  // (sample, head) land on the same XCD (workgroups are dealt round-robin
  // over the 8 XCDs).
  const int w = blockIdx.x;
  const int t = (w & 7) * p.per_xcd + (w >> 3);
  if (t >= p.total_tiles) return;
  const int bh = t / p.tiles_per_bh;
  const int rank = t - bh * p.tiles_per_bh;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  int bi = 0;
  while (bi + 1 < p.n_qblocks && p.blk[bi + 1].tile_prefix <= rank) ++bi;
  const QBlockDesc& d = p.blk[bi];
  const int row0 = d.row_lo + (rank - d.tile_prefix) * M;
  const int rows = min(M, d.row_lo + d.rows - row0);
  const int n_keys = d.n_keys;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;
  const int hh = lane >> 5;

  const int64_t rs = int64_t(p.H) * D;  // token stride (elements)
  const int64_t bh_off = int64_t(b) * p.S * rs + int64_t(h) * D;
  const __bf16* __restrict__ qg = static_cast<const __bf16*>(p.q) + bh_off;
  const char* __restrict__ kg = reinterpret_cast<const char*>(static_cast<const __bf16*>(p.k) + bh_off);
  const char* __restrict__ vg = reinterpret_cast<const char*>(static_cast<const __bf16*>(p.v) + bh_off);

  // ---- Q rows for this wave, kept in registers as MFMA B operands.
  bf16x8 qreg[QB][NDS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int lrow = wave * QW + qb * 32 + lr;
    const bool ok = lrow < rows;
    const __bf16* src = qg + int64_t(row0 + lrow) * rs + hh * 8;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      if (ok) {
        qreg[qb][ds] = *reinterpret_cast<const bf16x8*>(src + ds * 16);
      } else {
        qreg[qb][ds] = bf16x8{};
      }
    }
  }

  f32x16 acc[QB][NDB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -__builtin_inff();
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[qb][db] = f32x16{};
  }

  // ---- global -> register staging of one K/V step.  Per-thread byte
  // offsets relative to the tile's first key are fixed; a tile that lies
  // inside one key interval is addressed from a scalar base.
  const int64_t rsb = rs * 2;  // token stride in bytes
  constexpr int KROWS = 256 / DC;  // key rows covered by one K chunk pass
  const int ktid = tid - K0;
  const bool k_loader = ktid >= 0 && ktid < 256;
  const int k_r0 = ktid / DC;
  const uint32_t k_off = uint32_t(k_r0 * rsb + (ktid - k_r0 * DC) * 16);
  const int v_kq = tid % (KT / 4);
  const int v_cc = tid / (KT / 4);
  const uint32_t v_off = uint32_t(v_kq * 4 * rsb + v_cc * 16);

  u32x4 kst[KCH];
  u32x4 vst[4];
  // How a step's KT keys are addressed: from one scalar base when they lie
  // inside one key interval (the common case), else key by key.  K runs two
  // steps ahead of the softmax and V one step ahead, so each keeps its own
  // interval cursor.
  struct Plan {
    bool fast;
    int64_t base;  // byte offset of the step's first key (fast path)
  };
  auto plan = [&](int step, int& iv) -> Plan {
    const int j0 = step * KT;
    while (iv + 1 < d.n_iv && j0 >= d.iv_start[iv + 1]) ++iv;
    const int iv_end = (iv + 1 < d.n_iv) ? d.iv_start[iv + 1] : n_keys;
    return Plan{j0 + KT <= iv_end, int64_t(j0 + d.iv_delta[iv]) * rsb};
  };
  auto load_k = [&](int step, const Plan& pl) {
    if (!k_loader) return;
    if (pl.fast) {
#pragma unroll
      for (int c = 0; c < KCH; ++c)
        kst[c] = *reinterpret_cast<const u32x4*>(kg + (pl.base + c * KROWS * rsb) + k_off);
    } else {
      const int j0 = step * KT;
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        const int j = j0 + c * KROWS + k_r0;
        if (j < n_keys) {
          kst[c] = *reinterpret_cast<const u32x4*>(kg + int64_t(vtoken(d, j)) * rsb +
                                                    (k_off - uint32_t(k_r0 * rsb)));
        } else {
          kst[c] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  auto load_v = [&](int step, const Plan& pl) {
    if (tid >= VITEMS) return;
    if (pl.fast) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vst[i] = *reinterpret_cast<const u32x4*>(vg + (pl.base + i * rsb) + v_off);
    } else {
      const int j0 = step * KT;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + v_kq * 4 + i;
        if (j < n_keys) {
          vst[i] = *reinterpret_cast<const u32x4*>(vg + int64_t(vtoken(d, j)) * rsb + v_cc * 16);
        } else {
          vst[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  auto store_k = [&](int buf) {
    if (!k_loader) return;
    __bf16* ks = Ks + buf * KBUF;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int u = c * 256 + ktid;
      const int kr = u / DC;
      const int cc = u - kr * DC;
      *reinterpret_cast<u32x4*>(&ks[kr * KP + cc * 8]) = kst[c];
    }
  };
  auto store_v = [&](int buf) {
    if (tid >= VITEMS) return;
    __bf16* vt = Vt + buf * VBUF;
    // 4 keys x 8 d in registers -> 8 rows of V^T, 4 keys (8 bytes) each.
    const int pos = vt_pos(v_kq * 4);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t a0 = vst[0][m], a1 = vst[1][m], a2 = vst[2][m], a3 = vst[3][m];
      const u32x2 even = {__builtin_amdgcn_perm(a1, a0, 0x05040100u), __builtin_amdgcn_perm(a3, a2, 0x05040100u)};
      const u32x2 odd = {__builtin_amdgcn_perm(a1, a0, 0x07060302u), __builtin_amdgcn_perm(a3, a2, 0x07060302u)};
      *reinterpret_cast<u32x2*>(&vt[(v_cc * 8 + 2 * m) * VP + pos]) = even;
      *reinterpret_cast<u32x2*>(&vt[(v_cc * 8 + 2 * m + 1) * VP + pos]) = odd;
    }
  };

  const float c = p.score_scale_log2;
  const int nsteps = (n_keys + KT - 1) / KT;
  const bf16x2 kOnes2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

  // S^T = K Q^T for the KT keys in K buffer `buf`.
  auto qk = [&](int buf, f32x16 (&s)[NKB][QB]) {
    const __bf16* ks = Ks + buf * KBUF;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&ks[(kb * 32 + lr) * KP + ds * 16 + hh * 8]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[qb][ds], s[kb][qb], 0, 0, 0);
      }
    }
  };

  // One step of the software pipeline: softmax of step `step` (scores in
  // s_cur) and P V with V buffer step&1, while the MFMA units compute the
  // scores of step+1 into s_next from K buffer (step+1)&1.  On the last step
  // that product reads a stale buffer and is discarded.
  int ivk = 0, ivv = 0;
  auto body = [&](int step, f32x16 (&s_cur)[NKB][QB], f32x16 (&s_next)[NKB][QB]) {
    const int buf = step & 1;
    const bool has1 = step + 1 < nsteps;
    const bool has2 = step + 2 < nsteps;
    if (has2) load_k(step + 2, plan(step + 2, ivk));
    if (has1) load_v(step + 1, plan(step + 1, ivv));

    // mask the tail of the key list
    const int j0 = step * KT;
    if (j0 + KT > n_keys) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (j >= n_keys) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s_cur[kb][qb][r] = -__builtin_inff();
          }
        }
    }
    // running maximum; rescale only when it grew by more than the slack
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = fmaxf(s_cur[0][qb][0], s_cur[0][qb][1]);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = (kb == 0 ? 2 : 0); r < 16; r += 2)
          mx = fmaxf(mx, fmaxf(s_cur[kb][qb][r], s_cur[kb][qb][r + 1]));
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * c;
      if (__any(mx > m_run[qb] + kRescaleSlack)) {
        const float m_new = fmaxf(m_run[qb], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha;
      }
    }

    // scores of the next step (independent of the softmax below)
    qk(buf ^ 1, s_next);

    // P = exp2(S c - m), packed to bf16; row sums over the rounded weights
    bf16x8 pk[QB][NKB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mneg = -m_run[qb];
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8 v8;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            v8[e] = static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[kb][qb][half * 8 + e], c, mneg)));
          pk[qb][kb][half] = v8;
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v8, v8, 0, 1), kOnes2, lsum, false);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v8, v8, 2, 3), kOnes2, lsum, false);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v8, v8, 4, 5), kOnes2, lsum, false);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v8, v8, 6, 7), kOnes2, lsum, false);
        }
      }
      l_run[qb] += lsum;
    }

    // O^T += V^T P^T
    const __bf16* vt = Vt + buf * VBUF;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&vt[(db * 32 + lr) * VP + kb * 32 + half * 16 + hh * 8]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[qb][kb][half], acc[qb][db], 0, 0, 0);
        }
      }
    }

    // K of step+2 replaces K of step (read one step ago, before the last
    // barrier); V of step+1 replaces V of step-1.
    if (has2) store_k(buf);
    if (has1) store_v(buf ^ 1);
    __syncthreads();
  };

  // prologue: K of steps 0 and 1, V of step 0, scores of step 0
  load_k(0, plan(0, ivk));
  load_v(0, plan(0, ivv));
  store_k(0);
  store_v(0);
  if (nsteps > 1) {
    load_k(1, plan(1, ivk));
    store_k(1);
  }
  __syncthreads();
  f32x16 sA[NKB][QB], sB[NKB][QB];
  qk(0, sA);
  for (int step = 0;;) {
    body(step, sA, sB);
    if (++step >= nsteps) break;
    body(step, sB, sA);
    if (++step >= nsteps) break;
  }

  // ---- epilogue: normalise, gate, store bf16, optional log-sum-exp
  __bf16* og = static_cast<__bf16*>(p.out) + bh_off;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int lrow = wave * QW + qb * 32 + lr;
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
    if (lrow < rows) {
      const int row = row0 + lrow;
      float scale = 1.0f / l_tot;
      if (p.gate != nullptr) {
        const float g = p.gate[(int64_t(b) * p.S + row) * p.H + h];
        scale *= 1.0f / (1.0f + __builtin_amdgcn_exp2f(-g * kLog2e));
      }
      __bf16* dst = og + int64_t(row) * rs;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bf16x4 o4;
#pragma unroll
          for (int r = 0; r < 4; ++r) o4[r] = static_cast<__bf16>(acc[qb][db][g4 * 4 + r] * scale);
          *reinterpret_cast<bf16x4*>(dst + db * 32 + g4 * 8 + hh * 4) = o4;
        }
      }
      if (p.lse != nullptr && hh == 0) {
        p.lse[(int64_t(b) * p.H + h) * p.S + row] = (m_run[qb] + __log2f(l_tot)) * kLn2;
      }
    }
  }
}

// Waves per workgroup of the bf16 kernel: each wave owns 32 query rows.
constexpr int kWaves = 8;

int kernel_tile_m(int head_dim, int dtype) {
  (void)head_dim;
  (void)dtype;
  return 32 * kWaves;
}

int launch_fwd(const FwdParams& p, int head_dim, int dtype, void* stream) {
  const dim3 grid(unsigned(p.per_xcd) * 8u);
  const dim3 block(64 * kWaves);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype != 0) return int(hipErrorInvalidValue);
  if (head_dim == 128) {
    hipLaunchKernelGGL((fwd_bf16_kernel<128, 1, kWaves>), grid, block, 0, st, p);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL((fwd_bf16_kernel<64, 1, kWaves>), grid, block, 0, st, p);
  } else {
    return int(hipErrorInvalidValue);
  }
  return int(hipGetLastError());
}

}  // namespace vdn
