// Test-only kernels: run the library's device functions on caller data.
#include "ea.h"
#include "ea_device.h"
#include "ea_test.h"

namespace {

__global__ void exp2_kernel(const float* x, float* y, int n, int mode) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  y[i] = (mode == EA_EXP_POLY) ? ea::exp2_poly(x[i]) : ea::exp2_hw(x[i]);
}

// A calibration loop: each wave issues iters x 16 v_mfma_f32_32x32x16_bf16
// into four independent accumulators from register operands (no memory
// traffic), so the launch measures the rate the matrix cores sustain on this
// device under full load. Each lane writes one sum so nothing is eliminated.
__global__ __launch_bounds__(512) void mfma_loop_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  ea::bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)(lane + i));
    b[i] = (__bf16)(1e-3f * (float)(lane - i));
  }
  ea::f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c0 = ea::mfma32x32x16(a, b, c0);
      c1 = ea::mfma32x32x16(a, b, c1);
      c2 = ea::mfma32x32x16(a, b, c2);
      c3 = ea::mfma32x32x16(a, b, c3);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// A streaming read: each thread reads kStreamUnroll 16-byte chunks per pass
// (grid-stride, non-temporal) and folds them into one value, so the launch
// measures the HBM read rate a plain kernel sustains on this device.
constexpr int kStreamUnroll = 16;
__global__ __launch_bounds__(256) void stream_read_kernel(const ea::i32x4* __restrict__ p, size_t n16, int* out) {
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t nt = (size_t)gridDim.x * blockDim.x;
  ea::i32x4 acc = {0, 0, 0, 0};
  for (size_t base = tid; base + (kStreamUnroll - 1) * nt < n16; base += kStreamUnroll * nt) {
    ea::i32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(p + base + u * nt);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u];
  }
  out[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

extern "C" ea_status ea_test_stream_read(const void* buf, size_t bytes, int* out, int blocks, void* stream) {
  if (buf == nullptr || out == nullptr || blocks <= 0 || blocks > 65536) return EA_ERR_INVALID;
  const size_t pass = (size_t)16 * kStreamUnroll * 256 * (size_t)blocks;  // bytes per grid pass
  if (bytes == 0 || bytes % pass != 0) return EA_ERR_INVALID;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const ea::i32x4*)buf, bytes / 16, out);
  return hipGetLastError() == hipSuccess ? EA_OK : EA_ERR_HIP;
}

extern "C" ea_status ea_test_mfma_loop(float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks <= 0 || iters <= 0 || blocks > 65536) return EA_ERR_INVALID;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream, out, iters);
  return hipGetLastError() == hipSuccess ? EA_OK : EA_ERR_HIP;
}

extern "C" ea_status ea_test_exp2(const float* x, float* y, int n, int mode, void* stream) {
  if (n < 0 || (n > 0 && (x == nullptr || y == nullptr))) return EA_ERR_INVALID;
  if (mode != EA_EXP_HW && mode != EA_EXP_POLY) return EA_ERR_INVALID;
  if (n == 0) return EA_OK;
  hipLaunchKernelGGL(exp2_kernel, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, x, y, n, mode);
  return hipGetLastError() == hipSuccess ? EA_OK : EA_ERR_HIP;
}
