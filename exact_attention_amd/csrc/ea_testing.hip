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

// The same loop with operands that change from one MFMA to the next: each
// lane holds kDataSets (A, B) operand pairs read once from a caller buffer
// (for instance random N(0,1) values, like the attention workloads'), and
// consecutive MFMAs take consecutive pairs, so the matrix core's inputs
// toggle as they do under a real contraction. The loop above repeats one
// operand pair, which draws less power, so under the same power limit it runs
// at a higher clock. FMT 0: v_mfma_f32_32x32x16_bf16 (pairs of bf16x8);
// FMT 1: v_mfma_scale_f32_32x32x64_f8f6f4 with e4m3 operands (pairs of 32
// bytes) and unit scales.
constexpr int kDataSets = 8;
template <int FMT>
__global__ __launch_bounds__(512) void mfma_loop_data_kernel(const ea::i32x4* __restrict__ ops, float* out,
                                                             int iters) {
  constexpr int W = FMT == 0 ? 1 : 2;  // 16-byte pieces per operand
  const ea::i32x4* src = ops + (size_t)threadIdx.x * kDataSets * 2 * W;
  ea::i32x4 a[kDataSets][W], b[kDataSets][W];
#pragma unroll
  for (int j = 0; j < kDataSets; ++j) {
#pragma unroll
    for (int u = 0; u < W; ++u) {
      a[j][u] = src[(2 * j) * W + u];
      b[j][u] = src[(2 * j + 1) * W + u];
    }
  }
  ea::f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  auto mf = [&](int ja, int jb, ea::f32x16 c) __attribute__((always_inline)) {
    if constexpr (FMT == 0) {
      return ea::mfma32x32x16(__builtin_bit_cast(ea::bf16x8, a[ja][0]), __builtin_bit_cast(ea::bf16x8, b[jb][0]), c);
    } else {
      const ea::i32x8 av = {a[ja][0][0], a[ja][0][1], a[ja][0][2], a[ja][0][3],
                            a[ja][1][0], a[ja][1][1], a[ja][1][2], a[ja][1][3]};
      const ea::i32x8 bv = {b[jb][0][0], b[jb][0][1], b[jb][0][2], b[jb][0][3],
                            b[jb][1][0], b[jb][1][1], b[jb][1][2], b[jb][1][3]};
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
    }
  };
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; j += 4) {
      c0 = mf(j % kDataSets, (j + 3) % kDataSets, c0);
      c1 = mf((j + 1) % kDataSets, (j + 4) % kDataSets, c1);
      c2 = mf((j + 2) % kDataSets, (j + 5) % kDataSets, c2);
      c3 = mf((j + 3) % kDataSets, (j + 6) % kDataSets, c3);
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) sum += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
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

extern "C" size_t ea_test_mfma_loop_data_bytes(int fmt) {
  if (fmt != 0 && fmt != 1) return 0;
  return (size_t)512 * kDataSets * 2 * (fmt == 0 ? 16 : 32);
}

extern "C" ea_status ea_test_mfma_loop_data(const void* operands, size_t operands_bytes, float* out, int blocks,
                                            int iters, int fmt, void* stream) {
  if (operands == nullptr || out == nullptr || blocks <= 0 || iters <= 0 || blocks > 65536 || (fmt != 0 && fmt != 1))
    return EA_ERR_INVALID;
  if (operands_bytes < ea_test_mfma_loop_data_bytes(fmt)) return EA_ERR_WORKSPACE;
  if (fmt == 0) {
    hipLaunchKernelGGL(mfma_loop_data_kernel<0>, dim3(blocks), dim3(512), 0, (hipStream_t)stream,
                       (const ea::i32x4*)operands, out, iters);
  } else {
    hipLaunchKernelGGL(mfma_loop_data_kernel<1>, dim3(blocks), dim3(512), 0, (hipStream_t)stream,
                       (const ea::i32x4*)operands, out, iters);
  }
  return hipGetLastError() == hipSuccess ? EA_OK : EA_ERR_HIP;
}

extern "C" ea_status ea_test_exp2(const float* x, float* y, int n, int mode, void* stream) {
  if (n < 0 || (n > 0 && (x == nullptr || y == nullptr))) return EA_ERR_INVALID;
  if (mode != EA_EXP_HW && mode != EA_EXP_POLY) return EA_ERR_INVALID;
  if (n == 0) return EA_OK;
  hipLaunchKernelGGL(exp2_kernel, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, x, y, n, mode);
  return hipGetLastError() == hipSuccess ? EA_OK : EA_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Two-role issue probe. The forward kernels pair two waves on each SIMD: one
// feeds the matrix core while the other runs the softmax on the vector ALU.
// This kernel measures what each role sustains alone and beside the other:
// waves 0-3 run role_a, waves 4-7 (the same SIMDs) run role_b, each in a loop
// of identical iterations until `budget` shader-clock cycles (s_memtime) have
// passed, then record how many iterations they finished in how many cycles.
// One workgroup per CU (the 96 KB of LDS it declares leave no room for a
// second), so each SIMD holds exactly the two probed waves.
//
// Roles (one iteration each):
//   IDLE       nothing (the wave exits at once)
//   MFMA_REG   32 v_mfma_f32_32x32x16_bf16, operands in registers, four
//              accumulators in VGPRs
//   MFMA_LDS   the forward's product part: 16 MFMAs whose A operand comes
//              from ds_read_b128 (a 64 x 128 K stage) and 16 whose A operand
//              comes from two ds_read_b64_tr_b16 each (a V^T stage), three
//              stages in turn, reads issued ahead of their MFMA
//   SOFTMAX    the forward's softmax of one 64-key step on 32 scores per
//              lane: three-input max chain, lane-swap max, wave vote on the
//              lazy-rescale test, 32 FMA + 32 exp2, two sum chains, 16 bf16
//              packs
//   EXP        32 independent v_exp_f32
//   FMA        32 independent v_fma_f32
//   MFMA_AGPR  MFMA_REG with the accumulators in AGPRs
//   MFMA_LDS_PRIO MFMA_LDS at raised wave priority (s_setprio 1), as the
//              forward runs its product part
//   MIX        8 MFMAs from registers interleaved, one by one, with 2 v_exp_f32
//              and 2 v_fma_f32 each (independent data): a wave that feeds the
//              matrix core and the vector ALU at once
//   LDS_B128   8 ds_read_b128 (an 8 KB operand tile into registers), then a
//              wait for them
//   LDS_TR     16 ds_read_b64_tr_b16 (an 8 KB transposed operand tile into
//              registers), then a wait for them
//   MFMA_LDS_DEEP MFMA_LDS with 14 operand reads issued before the first
//              MFMA instead of 6
//   MFMA_LDS_ALT  MFMA_LDS with the S and P V products alternating, so each
//              pair of MFMAs needs one plain and two transposed reads
//   FUSED32    one 32-key step of a wave that overlaps its own softmax with
//              its own products: 8 MFMAs fed by ds_read_b128, 8 fed by
//              transposed reads, and the softmax of an independent 32-key
//              score tile (16 scores per lane), interleaved
// ---------------------------------------------------------------------------
namespace {

constexpr int kProbeStage = 64 * 128;  // bf16 elements per K or V stage

__device__ __forceinline__ void probe_launder(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void probe_keep(float x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void probe_keep16(const ea::f32x16& x) { asm volatile("" ::"v"(x)); }

__device__ __forceinline__ ea::f32x16 mfma_agpr(ea::bf16x8 a, ea::bf16x8 b, ea::f32x16 c) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  return c;
}

__device__ __forceinline__ void wait_lgkm_probe() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

struct ProbeCounts {
  long long iters, cycles;
};

template <typename F>
__device__ __forceinline__ ProbeCounts probe_run(long long budget, F&& body) {
  const long long t0 = __builtin_amdgcn_s_memtime();
  long long t = t0, n = 0;
  while (t - t0 < budget) {
#pragma unroll 1
    for (int u = 0; u < 4; ++u) body((int)(n + u));
    n += 4;
    t = __builtin_amdgcn_s_memtime();
  }
  return {n, t - t0};
}

// AGPRS: the instantiation that holds the AGPR-accumulator role (a kernel
// that uses AGPRs at all gets its register budget split evenly between VGPRs
// and AGPRs, so the other roles run in the instantiation without it)
template <bool AGPRS>
__global__ __launch_bounds__(512, 1) void pair_probe_kernel(long long* out, int role_a, int role_b,
                                                            long long budget) {
  __shared__ __attribute__((aligned(1024))) uint16_t kst[3 * kProbeStage];
  __shared__ __attribute__((aligned(1024))) uint16_t vst[3 * kProbeStage];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < 3 * kProbeStage; i += 512) {
    kst[i] = (uint16_t)(0x3c00 + (i & 63));  // small positive bf16 values
    vst[i] = (uint16_t)(0x3c00 + ((i >> 3) & 63));
  }
  __syncthreads();
  const int role = __builtin_amdgcn_readfirstlane(w < 4 ? role_a : role_b);
  const int hh = lane >> 5, c = lane & 31;
  ea::bf16x8 qa, qb;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    qa[i] = (__bf16)(1e-3f * (float)(lane + i));
    qb[i] = (__bf16)(1e-3f * (float)(lane - i));
  }
  ProbeCounts r{0, 0};
  if (role == EA_PROBE_MFMA_REG || role == EA_PROBE_MFMA_AGPR) {
    ea::f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    if (role == EA_PROBE_MFMA_REG) {
      r = probe_run(budget, [&](int) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          c0 = ea::mfma32x32x16(qa, qb, c0);
          c1 = ea::mfma32x32x16(qa, qb, c1);
          c2 = ea::mfma32x32x16(qa, qb, c2);
          c3 = ea::mfma32x32x16(qa, qb, c3);
        }
      });
    } else if constexpr (AGPRS) {
      r = probe_run(budget, [&](int) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          c0 = mfma_agpr(qa, qb, c0);
          c1 = mfma_agpr(qa, qb, c1);
          c2 = mfma_agpr(qa, qb, c2);
          c3 = mfma_agpr(qa, qb, c3);
        }
      });
      asm volatile("s_nop 15\n s_nop 15\n s_nop 15" ::: "memory");
    }
    probe_keep16(c0);
    probe_keep16(c1);
    probe_keep16(c2);
    probe_keep16(c3);
  } else if (role == EA_PROBE_MFMA_LDS || role == EA_PROBE_MFMA_LDS_PRIO || role == EA_PROBE_MFMA_LDS_DEEP ||
             role == EA_PROBE_MFMA_LDS_ALT) {
    // operand offsets of the forward (bytes): K rows c and c + 32 at d chunk
    // 16 kk + 8 hh; V^T transposed reads of 4 rows x 4 columns per 16 lanes
    int k_off[8], v_off[4][2];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) k_off[kk] = 2 * ea::tile_off<128>(c, 16 * kk + 8 * hh);
    const int tr_row = 4 * hh + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      v_off[dt][0] = 2 * ea::tile_off<128>(tr_row, 32 * dt + tr_col);
      v_off[dt][1] = 2 * ea::tile_off<128>(tr_row + 8, 32 * dt + tr_col);
    }
    ea::f32x16 s0 = {}, s1 = {}, o[4] = {};
    const bool prio = role == EA_PROBE_MFMA_LDS_PRIO;
    auto kread = [&](const char EA_LDS* kb, int kk, int half) {
      return ea::lds_load<ea::bf16x8>(kb + k_off[kk] + half * 64 * 128);
    };
    auto vread = [&](const char EA_LDS* vb, int sj, int dt) {
      const ea::i16x4 lo = ea::ds_read_tr16((const EA_LDS uint16_t*)(vb + v_off[dt][0] + 32 * sj * 128));
      const ea::i16x4 hi = ea::ds_read_tr16((const EA_LDS uint16_t*)(vb + v_off[dt][1] + 32 * sj * 128));
      const ea::i32x4 t = {__builtin_bit_cast(ea::i32x2, lo)[0], __builtin_bit_cast(ea::i32x2, lo)[1],
                           __builtin_bit_cast(ea::i32x2, hi)[0], __builtin_bit_cast(ea::i32x2, hi)[1]};
      return __builtin_bit_cast(ea::bf16x8, t);
    };
    if (role == EA_PROBE_MFMA_LDS_ALT) {
      // S and P V products alternate: each pair of MFMAs needs one plain and
      // two transposed reads, so the two read kinds are spread evenly
      r = probe_run(budget, [&](int it) {
        const int st = it % 3;
        const char EA_LDS* kb = (const char EA_LDS*)((EA_LDS uint16_t*)kst + st * kProbeStage);
        const char EA_LDS* vb = (const char EA_LDS*)((EA_LDS uint16_t*)vst + st * kProbeStage);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = i >> 1, half = i & 1, sj = i >> 2, dt = i & 3;
          const ea::bf16x8 ka = kread(kb, kk, half);
          const ea::bf16x8 va = vread(vb, sj, dt);
          if (half) s1 = ea::mfma32x32x16(ka, qa, s1); else s0 = ea::mfma32x32x16(ka, qa, s0);
          o[dt] = ea::mfma32x32x16(va, qb, o[dt]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 9, 0);
#pragma unroll
        for (int i = 0; i < 13; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
      });
    } else {
      // the two products of the forward's MFMA part; the read-ahead pattern is
      // set per variant by scheduling groups after the body
      auto body = [&](int it) {
        const int st = it % 3;
        const char EA_LDS* kb = (const char EA_LDS*)((EA_LDS uint16_t*)kst + st * kProbeStage);
        const char EA_LDS* vb = (const char EA_LDS*)((EA_LDS uint16_t*)vst + st * kProbeStage);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const ea::bf16x8 k0 = kread(kb, kk, 0);
          const ea::bf16x8 k1 = kread(kb, kk, 1);
          s0 = ea::mfma32x32x16(k0, qa, s0);
          s1 = ea::mfma32x32x16(k1, qa, s1);
        }
#pragma unroll
        for (int sj = 0; sj < 4; ++sj) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) o[dt] = ea::mfma32x32x16(vread(vb, sj, dt), qb, o[dt]);
        }
      };
      if (role == EA_PROBE_MFMA_LDS_DEEP) {
        r = probe_run(budget, [&](int it) {
          body(it);
          // 14 reads primed, one read per S product, then two per P V product
          __builtin_amdgcn_sched_group_barrier(0x100, 14, 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
#pragma unroll
          for (int i = 0; i < 9; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 7, 0);
        });
      } else {
        r = probe_run(budget, [&](int it) {
          if (prio) __builtin_amdgcn_s_setprio(1);
          body(it);
          __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
#pragma unroll
          for (int i = 0; i < 13; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
          if (prio) __builtin_amdgcn_s_setprio(0);
        });
      }
    }
    probe_keep16(s0);
    probe_keep16(s1);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) probe_keep16(o[dt]);
  } else if (role == EA_PROBE_FUSED32) {
    // one 32-key step of a wave that overlaps its own softmax with its own
    // products: S_next = K Q^T (8 MFMAs, K by ds_read_b128), O += V^T P
    // (8 MFMAs, V^T by ds_read_b64_tr_b16) and the softmax of an independent
    // 32 x 32 score tile (16 scores per lane) interleaved in one block
    int k_off[8], v_off[4][2];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) k_off[kk] = 2 * ea::tile_off<128>(c, 16 * kk + 8 * hh);
    const int tr_row = 4 * hh + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      v_off[dt][0] = 2 * ea::tile_off<128>(tr_row, 32 * dt + tr_col);
      v_off[dt][1] = 2 * ea::tile_off<128>(tr_row + 8, 32 * dt + tr_col);
    }
    ea::f32x16 sn = {}, sc = {}, o[4] = {};
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = 0.01f * (float)((lane * 7 + i * 13) & 127) - 0.5f;
    ea::bf16x8 pb0 = qb, pb1 = qa;
    float m_run = 1.0f, l_run = 0.f;
    r = probe_run(budget, [&](int it) {
      const int st = it % 3;
      const char EA_LDS* kb = (const char EA_LDS*)((EA_LDS uint16_t*)kst + st * kProbeStage);
      const char EA_LDS* vb = (const char EA_LDS*)((EA_LDS uint16_t*)vst + st * kProbeStage);
      asm volatile("" : "+v"(sc));
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const ea::bf16x8 ka = ea::lds_load<ea::bf16x8>(kb + k_off[kk]);
        sn = ea::mfma32x32x16(ka, qa, kk == 0 ? ea::f32x16{} : sn);
      }
#pragma unroll
      for (int sj = 0; sj < 2; ++sj) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const ea::i16x4 lo = ea::ds_read_tr16((const EA_LDS uint16_t*)(vb + v_off[dt][0] + 32 * sj * 128));
          const ea::i16x4 hi = ea::ds_read_tr16((const EA_LDS uint16_t*)(vb + v_off[dt][1] + 32 * sj * 128));
          const ea::i32x4 t = {__builtin_bit_cast(ea::i32x2, lo)[0], __builtin_bit_cast(ea::i32x2, lo)[1],
                               __builtin_bit_cast(ea::i32x2, hi)[0], __builtin_bit_cast(ea::i32x2, hi)[1]};
          o[dt] = ea::mfma32x32x16(__builtin_bit_cast(ea::bf16x8, t), sj ? pb1 : pb0, o[dt]);
        }
      }
      // softmax of the current tile
      float mx = ea::kNegInf;
#pragma unroll
      for (int i = 0; i < 8; ++i) mx = __builtin_fmaxf(__builtin_fmaxf(mx, sc[i]), sc[i + 8]);
      mx = ea::max_with_partner32(mx);
      const float m_new = __builtin_fmaxf(m_run, mx * 0.127f);
      if (__ballot(m_new > m_run + 8.0f)) {
        l_run *= ea::exp2_hw(m_run - m_new);
        m_run = m_new;
      }
      float pp[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) pp[i] = ea::exp2_hw(__builtin_fmaf(sc[i], 0.127f, -m_run));
      float l0 = 0.f, l1 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        l0 += pp[i];
        l1 += pp[i + 8];
      }
      l_run += l0 + l1;
      const ea::i32x4 t0 = {(int)ea::pack_bf16x2(pp[0], pp[1]), (int)ea::pack_bf16x2(pp[2], pp[3]),
                            (int)ea::pack_bf16x2(pp[4], pp[5]), (int)ea::pack_bf16x2(pp[6], pp[7])};
      const ea::i32x4 t1 = {(int)ea::pack_bf16x2(pp[8], pp[9]), (int)ea::pack_bf16x2(pp[10], pp[11]),
                            (int)ea::pack_bf16x2(pp[12], pp[13]), (int)ea::pack_bf16x2(pp[14], pp[15])};
      pb0 = __builtin_bit_cast(ea::bf16x8, t0);
      pb1 = __builtin_bit_cast(ea::bf16x8, t1);
      // interleave: reads two ahead, each MFMA followed by a share of the vector work
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
    });
    probe_keep16(sn);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) probe_keep16(o[dt]);
    probe_keep(l_run + m_run);
  } else if (role == EA_PROBE_SOFTMAX) {
    float s[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) s[i] = 0.01f * (float)((lane * 7 + i * 13) & 127) - 0.5f;
    float m_run = 1.0f, l_run = 0.f;
    r = probe_run(budget, [&](int) {
#pragma unroll
      for (int i = 0; i < 32; ++i) probe_launder(s[i]);
      float mx = ea::kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(__builtin_fmaxf(mx, s[i]), s[i + 16]);
      mx = ea::max_with_partner32(mx);
      const float m_new = __builtin_fmaxf(m_run, mx * 0.127f);
      if (__ballot(m_new > m_run + 8.0f)) {
        l_run *= ea::exp2_hw(m_run - m_new);
        m_run = m_new;
      }
      float p[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) p[i] = ea::exp2_hw(__builtin_fmaf(s[i], 0.127f, -m_run));
      float l0 = 0.f, l1 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        l0 += p[i];
        l1 += p[i + 16];
      }
      l_run += l0 + l1;
#pragma unroll
      for (int i = 0; i < 16; ++i) probe_keep(__builtin_bit_cast(float, ea::pack_bf16x2(p[2 * i], p[2 * i + 1])));
    });
    probe_keep(l_run + m_run);
  } else if (role == EA_PROBE_MIX) {
    ea::f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = -0.03f * (float)(lane + i);
    r = probe_run(budget, [&](int) {
      float y[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) probe_launder(x[i]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        c0 = ea::mfma32x32x16(qa, qb, c0);
        c1 = ea::mfma32x32x16(qa, qb, c1);
        c2 = ea::mfma32x32x16(qa, qb, c2);
        c3 = ea::mfma32x32x16(qa, qb, c3);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = ea::exp2_hw(x[i]);
#pragma unroll
      for (int i = 16; i < 32; ++i) y[i] = __builtin_fmaf(x[i], 1.0001f, 0.5f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);  // transcendental
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) probe_keep(y[i]);
    });
    probe_keep16(c0);
    probe_keep16(c1);
    probe_keep16(c2);
    probe_keep16(c3);
  } else if (role == EA_PROBE_LDS_B128 || role == EA_PROBE_LDS_TR) {
    const int tr_row = 4 * hh + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int kofs = 2 * ea::tile_off<128>(c, 8 * hh);
    const int vofs = 2 * ea::tile_off<128>(tr_row, tr_col);
    if (role == EA_PROBE_LDS_B128) {
      r = probe_run(budget, [&](int it) {
        const char EA_LDS* kb = (const char EA_LDS*)((EA_LDS uint16_t*)kst + (it % 3) * kProbeStage);
        ea::bf16x8 t[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) t[kk] = ea::lds_load<ea::bf16x8>(kb + kofs + 32 * kk);
        wait_lgkm_probe();
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) asm volatile("" ::"v"(t[kk]));
      });
    } else {
      r = probe_run(budget, [&](int it) {
        const char EA_LDS* vb = (const char EA_LDS*)((EA_LDS uint16_t*)vst + (it % 3) * kProbeStage);
        ea::i16x4 t[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          t[j] = ea::ds_read_tr16((const EA_LDS uint16_t*)(vb + vofs + 64 * (j & 3) + 4096 * (j >> 2)));
        wait_lgkm_probe();
#pragma unroll
        for (int j = 0; j < 16; ++j) asm volatile("" ::"v"(t[j]));
      });
    }
  } else if (role == EA_PROBE_EXP || role == EA_PROBE_FMA) {
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = -0.03f * (float)(lane + i);
    // all inputs laundered first, all results kept last, so no result is
    // consumed right after the instruction that makes it
    if (role == EA_PROBE_EXP) {
      r = probe_run(budget, [&](int) {
        float y[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) probe_launder(x[i]);
#pragma unroll
        for (int i = 0; i < 32; ++i) y[i] = ea::exp2_hw(x[i]);
#pragma unroll
        for (int i = 0; i < 32; ++i) probe_keep(y[i]);
      });
    } else {
      r = probe_run(budget, [&](int) {
        float y[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) probe_launder(x[i]);
#pragma unroll
        for (int i = 0; i < 32; ++i) y[i] = __builtin_fmaf(x[i], 1.0001f, 0.5f);
#pragma unroll
        for (int i = 0; i < 32; ++i) probe_keep(y[i]);
      });
    }
  }
  if (lane == 0) {
    out[2 * (blockIdx.x * 8 + w)] = r.iters;
    out[2 * (blockIdx.x * 8 + w) + 1] = r.cycles;
  }
}

}  // namespace

extern "C" ea_status ea_test_pair_probe(long long* out, int blocks, int role_a, int role_b, long long budget,
                                        void* stream) {
  if (out == nullptr || blocks <= 0 || blocks > 4096) return EA_ERR_INVALID;
  if (role_a < 0 || role_a > EA_PROBE_FUSED32 || role_b < 0 || role_b > EA_PROBE_FUSED32)
    return EA_ERR_INVALID;
  if (budget <= 0 || budget > (1LL << 32)) return EA_ERR_INVALID;
  if (role_a == EA_PROBE_MFMA_AGPR || role_b == EA_PROBE_MFMA_AGPR) {
    hipLaunchKernelGGL(pair_probe_kernel<true>, dim3(blocks), dim3(512), 0, (hipStream_t)stream, out, role_a, role_b,
                       budget);
  } else {
    hipLaunchKernelGGL(pair_probe_kernel<false>, dim3(blocks), dim3(512), 0, (hipStream_t)stream, out, role_a,
                       role_b, budget);
  }
  return hipGetLastError() == hipSuccess ? EA_OK : EA_ERR_HIP;
}
