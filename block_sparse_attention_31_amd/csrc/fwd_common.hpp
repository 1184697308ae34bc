// Device helpers shared by the attention kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "fwd_params.hpp"

namespace vdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

[[maybe_unused]] constexpr float kLog2e = 1.4426950408889634f;
[[maybe_unused]] constexpr float kLn2 = 0.6931471805599453f;

// A query block's key list in registers: virtual key j in [start_i,
// start_{i+1}) is token j + delta_i; unused intervals start at n_keys.
struct KeyList {
  int n_keys;
  int start1, start2;
  int delta0, delta1, delta2;
};

__device__ __forceinline__ KeyList load_key_list(const QBlockDesc& d) {
  KeyList k;
  k.n_keys = __builtin_amdgcn_readfirstlane(d.n_keys);
  k.start1 = __builtin_amdgcn_readfirstlane(d.n_iv > 1 ? d.iv_start[1] : d.n_keys);
  k.start2 = __builtin_amdgcn_readfirstlane(d.n_iv > 2 ? d.iv_start[2] : d.n_keys);
  k.delta0 = __builtin_amdgcn_readfirstlane(d.iv_delta[0]);
  k.delta1 = __builtin_amdgcn_readfirstlane(d.n_iv > 1 ? d.iv_delta[1] : 0);
  k.delta2 = __builtin_amdgcn_readfirstlane(d.n_iv > 2 ? d.iv_delta[2] : 0);
  return k;
}
// Maximum / sum of a value over lanes l and l^32 (the two halves of a wave
// hold the two halves of one query's keys), with the gfx950 cross-half swap:
// v_permlane32_swap a, b trades lanes 32..63 of a with lanes 0..31 of b, so
// with a = b = x every lane then holds x[l % 32] in a and x[l % 32 + 32] in b.
// Written as inline asm with both registers read-write: the compiler's
// builtin for it drops its second result.  The s_nop pads cover the
// VALU-write/permlane-read hazard on either side (no memory is touched).
__device__ __forceinline__ void xhalf_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float xhalf_max(float x) {
  float a = x, b = x;
  xhalf_swap(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float xhalf_sum(float x) {
  float a = x, b = x;
  xhalf_swap(a, b);
  return a + b;
}

// Three-way select on values.  (A conditional over struct members is an
// lvalue, and the compiler then picks between their addresses, which forces
// the struct into memory; going through value parameters keeps it in
// registers.)
__device__ __forceinline__ int pick3(int j, int s1, int s2, int a0, int a1, int a2) {
  return j >= s2 ? a2 : (j >= s1 ? a1 : a0);
}

// Token of virtual key j (0 <= j < n_keys).
__device__ __forceinline__ int vtoken(const KeyList& k, int j) {
  return j + pick3(j, k.start1, k.start2, k.delta0, k.delta1, k.delta2);
}

// End (exclusive) and token offset of the interval holding virtual key j.
__device__ __forceinline__ int interval_end(const KeyList& k, int j) {
  return pick3(j, k.start1, k.start2, k.start1, k.start2, k.n_keys);
}
__device__ __forceinline__ int interval_delta(const KeyList& k, int j) {
  return pick3(j, k.start1, k.start2, k.delta0, k.delta1, k.delta2);
}

// Online-softmax reference point may lag the running maximum by up to 2^8 in
// the base-2 domain: P then stays below 256, exact in bf16 up to rounding,
// and the accumulator rescale is skipped unless the maximum grows by more.
[[maybe_unused]] constexpr float kRescaleSlack = 8.0f;
// With the reference point fixed per row, it is set this far (log2 units)
// above the row's first-step maximum: later keys may then exceed that
// maximum by up to 48 before a weight passes 2^32.
[[maybe_unused]] constexpr float kRefHeadroom = 16.0f;

template <int N>
using IC = std::integral_constant<int, N>;

// Workgroup slot -> query tile.  Workgroups are dealt round-robin over the 8
// XCDs, and XCD x takes the tiles [x per_xcd, (x + 1) per_xcd) of the tile
// list in order, so consecutive tiles of one (sample, head) share an L2.  The
// last `split` tiles of each XCD's share run as two half tiles each (slots
// per_xcd - split .. per_xcd + split - 1): dispatched last, the shorter work
// evens out when the XCD's compute units finish.  `half` is 0 for a whole
// tile, 1 or 2 for its first or second half.
struct TileSlot {
  int tile, half;
};
// A (sample, head)'s tiles, sorted longest first, are dealt into `k` piles
// (tile s to pile s mod k) when the head spans k XCDs' shares, so that each
// share gets an even mix of long and short tiles; position r in the dealt
// order -> position in the sorted order.
__device__ __forceinline__ int undeal(int r, int n, int k) {
  if (k <= 1) return r;
  const int q = (n + k - 1) / k;       // entries of the first piles
  const int full = n % k == 0 ? k : n % k;  // piles holding q entries
  int pile, i;
  if (r < full * q) {
    pile = r / q;
    i = r - pile * q;
  } else {
    const int r2 = r - full * q;
    pile = full + r2 / (q - 1);
    i = r2 - (pile - full) * (q - 1);
  }
  return i * k + pile;
}

__device__ __forceinline__ TileSlot tile_slot(int w, int per_xcd, int split) {
  const int x = w & 7, u = w >> 3;
  const int whole = per_xcd - split;
  if (u < whole) return {x * per_xcd + u, 0};
  const int hs = u - whole;
  return {x * per_xcd + whole + (hs >> 1), 1 + (hs & 1)};
}

// Persistent launch: each XCD's share of the tile slots is a queue whose
// positions are claimed with one atomic add on its counter (a workgroup's
// first slot is its own block index, so the counters count from queue_wg).
// Claims need only be distinct: relaxed device-scope atomics.
__device__ __forceinline__ int queue_claim(int* queue, int q) {
  return __hip_atomic_fetch_add(queue + q, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The claim on the home queue (block index % 8) for the tile after the
// current one, taken by thread 0 while the current tile runs.
struct PendingClaim {
  int raw = 0;          // thread 0: the home counter's value before the add
  bool issued = false;  // wave-uniform
  __device__ __forceinline__ void issue(int* queue, int tid) {
    if (queue == nullptr || issued) return;
    issued = true;
    if (tid == 0) raw = queue_claim(queue, int(blockIdx.x & 7));
  }
};
// Thread 0: the next slot (queue + 8 * position), or -1 once every queue is
// empty.  `steal` is the next other queue to try (home + steal) % 8.  The
// workgroup that finds all queues empty last clears the counters for the
// next launch that uses them.
__device__ __forceinline__ int next_slot(int* queue, const PendingClaim& c, int qlen, int queue_wg, int& steal) {
  const int home = int(blockIdx.x & 7);
  int pos = (c.issued ? c.raw : queue_claim(queue, home)) + queue_wg;
  if (pos < qlen) return pos * 8 + home;
  for (; steal < 8; ++steal) {
    const int y = (home + steal) & 7;
    pos = queue_claim(queue, y) + queue_wg;
    if (pos < qlen) return pos * 8 + y;
  }
  if (queue_claim(queue, 8) == int(gridDim.x) - 1) {
#pragma unroll
    for (int i = 0; i < 9; ++i) __hip_atomic_store(queue + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return -1;
}

// Sets the scores of keys past the end of the key list to -inf on a partial
// last step.  Score register (kb, r) of a 32x32 MFMA result holds key
// 32 kb + 8 (r / 4) + 4 (lane / 32) + r % 4 of the step, so in each lane the
// keys rise with the register index e = 16 kb + r and the valid ones (below
// `lim`, wave-uniform) form a prefix of the lane's registers, of length
// 4 floor(y / 8) + min(4, y % 8) with y = lim - 4 (lane / 32).  One integer
// compare of e (an inline constant) against that length per register: no
// per-register float constants for the compiler to materialise.
template <int NKB>
__device__ __forceinline__ void mask_tail(f32x16 (&s)[NKB], int lim, int hh) {
  const int y = lim - 4 * hh;
  const int nv = y <= 0 ? 0 : 4 * (y >> 3) + min(4, y & 7);
  const float ninf = -__builtin_inff();
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = kb * 16 + r < nv ? s[kb][r] : ninf;
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left unconstrained).
__host__ __device__ constexpr int vmcnt_imm(int n) {
  return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14);
}

#define VDN_LDS(p) ((__attribute__((address_space(3))) void*)(p))

#ifndef VDN_ASM_DMA
#define VDN_ASM_DMA 1
#endif

// LDS DMA, 16 bytes per lane: lane L's 16 bytes at its global address land
// at LDS byte lds + 16 L (lds wave-uniform).  Two forms: a scalar base plus
// a 32-bit per-lane offset, and a full per-lane address.
// Issued through inline asm rather than the compiler's builtin: while a
// builtin LDS DMA is outstanding (until a joint vmcnt(0) lgkmcnt(0) wait) the
// compiler turns every wait for an LDS read into lgkmcnt(0), so no LDS read
// can be in flight while the MFMAs consume earlier ones.  The asm form is
// invisible to that bookkeeping; the hardware counts the DMA on vmcnt only,
// and the kernels order the destination with explicit vmcnt waits and
// barriers.  No VGPR is written by the asm (the data goes to LDS), and the
// leading s_nop covers the M0 write and the SGPR-base write that precede it.
__device__ __forceinline__ void lds_dma16(const char* sbase, uint32_t voff, const char* lds) {
#if VDN_ASM_DMA
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(lds)));
  // the base is wave-uniform by contract; saying so keeps it in scalar
  // registers where the compiler cannot prove it (free where it can)
  const uint64_t a = reinterpret_cast<uintptr_t>(sbase);
  // (the builtin returns int: both halves go through uint32_t, or the low
  // word would be sign-extended into the high one)
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(a >> 32)));
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(a)));
  const uint64_t su = (uint64_t(hi) << 32) | uint64_t(lo);
  const char* sb = reinterpret_cast<const char*>(su);
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb), "{m0}"(m0) : "memory");
#else
  __builtin_amdgcn_global_load_lds(sbase + voff, VDN_LDS(lds), 16, 0, 0);
#endif
}
__device__ __forceinline__ void lds_dma16(const char* gaddr, const char* lds) {
#if VDN_ASM_DMA
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(lds)));
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr), "{m0}"(m0) : "memory");
#else
  __builtin_amdgcn_global_load_lds(gaddr, VDN_LDS(lds), 16, 0, 0);
#endif
}

// Workgroup barrier that orders LDS accesses for the compiler but makes no
// wave wait for its outstanding vector-memory operations (LDS DMA included);
// callers wait on vmcnt themselves.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F & ~0xF00);  // lgkmcnt(0): LDS ops issued so far are done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// LDS tile swizzle read both by rows (ds_read_b128 of 16-byte chunks) and
// transposed (ds_read_b64_tr_b16): chunk c of row r sits at
// c ^ (4 (r % 4) + (r / 4) % 4) (CH chunks per row).  Sixteen consecutive
// rows put one logical chunk on sixteen distinct chunks, and four
// consecutive rows (a transposing read) spread four logical chunks over
// sixteen.  Period 16 in r.
template <int CH>
__device__ __forceinline__ int dual_swz(int r) {
  return (4 * (r & 3) + ((r >> 2) & 3)) & (CH - 1);
}

// Transposing fragment read: lanes of a 16-lane group point at rows
// rbase + 4 hh + i/4 (and + 8 for the second read), columns col0 + 4 (i % 4),
// so lane i receives column col0 + i of rows {4hh .. 4hh+3, 8+4hh .. 8+4hh+3}:
// the MFMA A-operand layout matching a score-layout B operand.
__device__ __forceinline__ bf16x8 tr_frag(const char* p_lo, const char* p_hi) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p_lo));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p_hi));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}


}  // namespace vdn
