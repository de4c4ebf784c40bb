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

}  // namespace

extern "C" ea_status ea_test_exp2(const float* x, float* y, int n, int mode, void* stream) {
  if (n < 0 || (n > 0 && (x == nullptr || y == nullptr))) return EA_ERR_INVALID;
  if (mode != EA_EXP_HW && mode != EA_EXP_POLY) return EA_ERR_INVALID;
  if (n == 0) return EA_OK;
  hipLaunchKernelGGL(exp2_kernel, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, x, y, n, mode);
  return hipGetLastError() == hipSuccess ? EA_OK : EA_ERR_HIP;
}
