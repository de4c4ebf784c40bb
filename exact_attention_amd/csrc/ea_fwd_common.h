// Device helpers shared by the gfx950 forward kernels that stage K/V through
// LDS DMA and pace their waves with workgroup barriers.
//
// The helpers that wrap asm statements or scheduling builtins are device
// functions on purpose: written directly inside a kernel's lambda, target
// builtins and register constraints are also checked in the host compilation
// pass, and that failure silently drops the host-side kernel stub.
#pragma once
#include "ea_device.h"

namespace ea {
namespace {

// s_waitcnt with only the vector-memory counter set (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Waits for this wave's LDS accesses (and scalar loads) only: lgkmcnt = 0,
// vmcnt and expcnt left at their maxima.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier that neither the compiler nor the scheduler moves memory
// operations across, and that adds no wait of its own (a __syncthreads would
// also wait for the DMA still in flight).
__device__ __forceinline__ void pp_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// keeps the instructions on either side in program order
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
// the value must exist here (stops the compiler sinking its computation)
__device__ __forceinline__ void keep(const f32x16& x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void keep(const bf16x8& x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void keep(float x) { asm volatile("" ::"v"(x)); }
// x, computed here: the compiler may no longer move its computation under a
// branch that uses it
__device__ __forceinline__ float keep_val(float x) {
  asm volatile("" : "+v"(x));
  return x;
}
// the compiler forgets where x came from (stops it hoisting x + constant out
// of a loop, so a constant added to it later folds into an LDS offset field)
__device__ __forceinline__ int launder(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// the same for a wave-uniform value held in a scalar register
__device__ __forceinline__ int launder_s(int x) {
  asm volatile("" : "+s"(x));
  return x;
}

__device__ __forceinline__ const uint16_t* launder_s(const uint16_t* p) {
  asm volatile("" : "+s"(p));
  return p;
}
__device__ __forceinline__ uint32_t launder_s(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}

// elements B .. B+7 of a score accumulator, rounded to bf16 and packed as an
// MFMA operand
template <int B>
__device__ __forceinline__ bf16x8 pack_p8(const f32x16 v) {
  const i32x4 t = {(int)pack_bf16x2(v[B + 0], v[B + 1]), (int)pack_bf16x2(v[B + 2], v[B + 3]),
                   (int)pack_bf16x2(v[B + 4], v[B + 5]), (int)pack_bf16x2(v[B + 6], v[B + 7])};
  return __builtin_bit_cast(bf16x8, t);
}

// Persistent workgroups: one per CU walks its share of an XCD-grouped work
// list (entry j of XCD x is global tile 8 j + x, as in the one-tile-per-
// workgroup launch). A new workgroup launch on a CU that just retired one
// costs ~11 us on this GPU; a persistent workgroup goes straight to its next
// tile. The dynamic dispatch of one workgroup per tile balanced a
// heaviest-first list by itself; the static split keeps that balance with a
// snake order: workgroup i of the W on an XCD takes entry r W + i in even
// rounds r and r W + W - 1 - i in odd ones, so a heavy entry pairs with a
// light one.
template <typename F>
__device__ __forceinline__ void persistent_snake(int per_xcd, F&& tile) {
  const int xcd = blockIdx.x & 7, i = blockIdx.x >> 3, W = gridDim.x >> 3;
  for (int r = 0; r * W < per_xcd; ++r) {
    const int jj = r * W + ((r & 1) ? W - 1 - i : i);
    if (jj < per_xcd) tile(xcd, jj);
  }
}

// Weight of a packed sequence in the heaviest-first (LPT) batch order of
// "FlashAttention4 close reading", section 3.3: the key tiles (block_n keys
// each) of the main loop of its last block of block_m query rows -- causal,
// bottom-right aligned: keys up to that block's last row; non-causal: all
// keys -- and 0 for a sequence without queries.
__device__ __forceinline__ int lpt_weight(long long lq, long long lk, int causal, int block_m, int block_n) {
  long long wt = 0;
  if (lq > 0) {
    long long nkeys = lk;
    if (causal) {
      const long long n_mb = (lq + block_m - 1) / block_m;
      nkeys = min(lk, n_mb * block_m + lk - lq);
    }
    if (nkeys < 0) nkeys = 0;
    wt = (nkeys + block_n - 1) / block_n;
  }
  return (int)min(wt, (long long)0x7fffffff);
}

// The heaviest-first order of n packed sequences, computed by one
// workgroup of at least n threads into LDS: w[b] = weight of sequence b, then
// order[rank(b)] = b with rank(b) = #{heavier} + #{equal and earlier} (a
// stable descending sort by counting). Every thread of the workgroup must
// call it (it holds two workgroup barriers).
__device__ __forceinline__ void lpt_order_lds(const int* cu_q, const int* cu_k, int n, int causal, int block_m,
                                              int block_n, EA_LDS int* w, EA_LDS int* order) {
  const int b = threadIdx.x;
  int wb = 0;
  if (b < n) {
    wb = lpt_weight((long long)cu_q[b + 1] - cu_q[b], (long long)cu_k[b + 1] - cu_k[b], causal, block_m, block_n);
    w[b] = wb;
  }
  __syncthreads();
  if (b < n) {
    int rank = 0;
    for (int t = 0; t < n; ++t) {
      const int wt = w[t];
      rank += (wt > wb) || (wt == wb && t < b);
    }
    order[rank] = b;
  }
  __syncthreads();
}

template <int EXPMODE>
__device__ __forceinline__ float pp_exp2(float x, int i) {
  if constexpr (EXPMODE == 0) {
    return exp2_hw(x);
  } else if constexpr (EXPMODE == 1) {
    return exp2_poly(x);
  } else {
    return ((i & 3) == 3) ? exp2_poly(x) : exp2_hw(x);
  }
}

}  // namespace
}  // namespace ea
