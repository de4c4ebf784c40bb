// Varlen batch order for the forward ("FlashAttention4 close reading",
// section 3.3, scheduling): the item whose heaviest work tile is longest goes
// first, and a preprocessing step writes a virtual -> actual permutation of
// the batch instead of moving any data. The forward's varlen kernels then
// walk the (virtual sequence, head) groups round-robin over the XCDs, so the
// heaviest sequences' tiles start first on every XCD.
//
// Two small kernels:
//  * weights: one thread per sequence; weight = key tiles of its last row
//    block, the longest main loop of the sequence (causal, bottom-right: keys
//    up to the block's last row; non-causal: all keys; 0 without queries).
//  * ranks: a stable descending sort by counting -- rank(b) = #{heavier} +
//    #{equal and earlier} -- with the weights streamed through LDS in tiles,
//    O(n^2) comparisons spread over n threads; order[rank(b)] = b.
#include "ea_device.h"
#include "ea_fwd_common.h"
#include "ea_internal.h"

namespace ea {

namespace {

constexpr int kSchedThreads = 256;

__global__ __launch_bounds__(kSchedThreads) void lpt_weight_kernel(const int* cu_q, const int* cu_k, int n,
                                                                   int causal, int block_m, int block_n, int* w) {
  const int b = blockIdx.x * kSchedThreads + threadIdx.x;
  if (b >= n) return;
  w[b] = lpt_weight((long long)cu_q[b + 1] - cu_q[b], (long long)cu_k[b + 1] - cu_k[b], causal, block_m, block_n);
}

__global__ __launch_bounds__(kSchedThreads) void lpt_rank_kernel(const int* w, int n, int* order) {
  __shared__ int tile[kSchedThreads];
  const int b = blockIdx.x * kSchedThreads + threadIdx.x;
  const int wb = b < n ? w[b] : 0;
  int rank = 0;
  for (int j0 = 0; j0 < n; j0 += kSchedThreads) {
    const int jj = j0 + (int)threadIdx.x;
    tile[threadIdx.x] = jj < n ? w[jj] : 0;
    __syncthreads();
    const int cnt = min(kSchedThreads, n - j0);
    for (int t = 0; t < cnt; ++t) {
      const int wj = tile[t];
      rank += (wj > wb) || (wj == wb && j0 + t < b);
    }
    __syncthreads();
  }
  if (b < n) order[rank] = b;
}

// Test-only: the order the forward's workgroups compute for themselves
// (lpt_order_lds), written out by one workgroup of the forward's size.
__global__ __launch_bounds__(512) void lpt_lds_kernel(const int* cu_q, const int* cu_k, int n, int causal,
                                                      int block_m, int* out) {
  __shared__ int w[kLptLds], order[kLptLds];
  lpt_order_lds(cu_q, cu_k, n, causal, block_m, kFwdBlockN, (EA_LDS int*)w, (EA_LDS int*)order);
  if ((int)threadIdx.x < n) out[threadIdx.x] = order[threadIdx.x];
}

}  // namespace

hipError_t launch_lpt_lds_order(const int* cu_q, const int* cu_k, int n, int causal, int* out, hipStream_t s) {
  hipLaunchKernelGGL(lpt_lds_kernel, dim3(1), dim3(512), 0, s, cu_q, cu_k, n, causal, kPpBlockM, out);
  return hipGetLastError();
}

hipError_t launch_lpt_order(const int* cu_q, const int* cu_k, int n, int causal, int block_m, int* weights,
                            int* order, hipStream_t s) {
  const int blocks = (n + kSchedThreads - 1) / kSchedThreads;
  hipLaunchKernelGGL(lpt_weight_kernel, dim3(blocks), dim3(kSchedThreads), 0, s, cu_q, cu_k, n, causal, block_m,
                     kFwdBlockN, weights);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lpt_rank_kernel, dim3(blocks), dim3(kSchedThreads), 0, s, (const int*)weights, n, order);
  return hipGetLastError();
}

}  // namespace ea
