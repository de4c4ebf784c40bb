// Fused exact attention forward for gfx950 (bf16 in, fp32 accumulate).
//
// Method: each workgroup owns 128 query rows of one (sequence, head) and
// streams over 64-key K/V tiles with the online-softmax recurrence -- running
// row max m, running sum l, unnormalised accumulator rescaled by exp(m - m')
// ("FlashAttention: not less compute, less data movement", section 02, Q-block
// outer loop; section 03 for keeping only O and the log-sum-exp). The score
// matrix never leaves registers.
//
// gfx950 mapping (this file's own design, not the pages' Blackwell pipeline):
//  * 4 waves x 32 query rows. Each wave computes S^T = K Q^T with
//    v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T held in VGPRs), so a lane
//    owns one query column: the row max and row sum are in-lane plus one
//    v_permlane32_swap with lane l^32.
//  * P^T leaves the S^T accumulator already in the B-operand layout of
//    O^T = V^T P^T (the keys inside each 16-key MFMA step are permuted; V^T's
//    A operand uses the same permutation), so P never touches LDS.
//  * V^T operands are read straight from the row-major V tile with
//    ds_read_b64_tr_b16.
//  * K/V tiles are double-buffered in LDS (64 KB per workgroup at d = 128, two
//    workgroups per CU), one barrier per tile.
//  * Lazy rescale: the accumulator and l are rescaled only when some lane's max
//    grew by more than tau (log2 units), decided wave-uniformly
//    ("FlashAttention-4: algorithm-pipeline co-design for Blackwell",
//    conditional softmax rescaling section; "FlashAttention4 close reading",
//    section 3.1.4). Otherwise the stale max stays; O = acc / l and
//    lse = m + log l are unchanged in exact arithmetic.
//  * Work order: tiles of one (sequence, head) stay on one XCD (workgroup id
//    mod 8 selects the XCD) so its K/V is served from that XCD's L2; within a
//    (sequence, head), causal row blocks run heaviest first (the
//    longest-processing-time order of "FlashAttention4 close reading",
//    section 3.3, with batch/head grouping for cache locality).
#include "ea_device.h"
#include "ea_internal.h"

namespace ea {

template <int D, int EXPMODE>
__device__ __forceinline__ float softmax_exp2(float x, int i) {
  if constexpr (EXPMODE == 0) {
    return exp2_hw(x);
  } else if constexpr (EXPMODE == 1) {
    return exp2_poly(x);
  } else {
    // hybrid: one element in four on the FMA pipe
    return ((i & 3) == 3) ? exp2_poly(x) : exp2_hw(x);
  }
}

template <int D, bool CAUSAL, bool VARLEN, int EXPMODE>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int BM = kFwdBlockM, BN = kFwdBlockN;
  constexpr int KCH = D / 8;               // 16-byte chunks per row
  constexpr int TILE = BN * D;             // bf16 elements per K or V tile
  constexpr int CPT = BN * KCH / 256;      // chunks per thread per tile
  constexpr int NDT = D / 32;              // 32-wide d tiles of O^T
  __shared__ __attribute__((aligned(16))) uint16_t smem_raw[2 * 2 * TILE];
  EA_LDS uint16_t* sm = (EA_LDS uint16_t*)smem_raw;

  // ---------------- tile assignment (XCD-grouped, heaviest first)
  const int xcd = blockIdx.x & 7;
  int j = blockIdx.x >> 3;
  int seq, h, mb;
  const int ngroups = a.nseq * a.Hq;
  if constexpr (!VARLEN) {
    const int kg = j / a.n_mb;
    const int r = j - kg * a.n_mb;
    const int g = xcd + 8 * kg;
    if (g >= ngroups) return;
    seq = g / a.Hq;
    h = g - seq * a.Hq;
    mb = a.natural ? r : a.n_mb - 1 - r;
  } else {
    int g = xcd, nm = 0;
    for (; g < ngroups; g += 8) {
      const int s = g / a.Hq;
      nm = (a.cu_q[s + 1] - a.cu_q[s] + BM - 1) / BM;
      if (j < nm) break;
      j -= nm;
    }
    if (g >= ngroups) return;
    seq = g / a.Hq;
    h = g - seq * a.Hq;
    mb = a.natural ? j : nm - 1 - j;
  }

  int q0, lq, k0, lk;
  if constexpr (VARLEN) {
    q0 = a.cu_q[seq];
    lq = a.cu_q[seq + 1] - q0;
    k0 = a.cu_k[seq];
    lk = a.cu_k[seq + 1] - k0;
  } else {
    q0 = seq * a.Nq;
    lq = a.Nq;
    k0 = seq * a.Nk;
    lk = a.Nk;
  }
  const int hk = h / a.group;
  const int off = lk - lq;  // bottom-right causal alignment
  const int row_lo = mb * BM;
  int nkeys = lk;
  if constexpr (CAUSAL) nkeys = min(lk, row_lo + BM + off);
  if (nkeys < 0) nkeys = 0;
  const int nkb = (nkeys + BN - 1) / BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, hh = lane >> 5, c = lane & 31;
  const int qi = row_lo + w * 32 + c;  // this lane's query row (sequence-local)
  const size_t qstride = (size_t)a.Hq * D, kstride = (size_t)a.Hkv * D;

  // ---------------- Q^T operand (B of S^T = K Q^T), kept in VGPRs
  bf16x8 qf[D / 16];
  {
    const uint16_t* qp = a.q + (size_t)(q0 + qi) * qstride + (size_t)h * D + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (qi < lq) {
        qf[kk] = *(const bf16x8*)(qp + 16 * kk);
      } else {
        qf[kk] = bf16x8{};
      }
    }
  }

  // ---------------- K/V tile staging (global -> VGPR -> swizzled LDS)
  const uint16_t* kg_base = a.k + (size_t)k0 * kstride + (size_t)hk * D;
  const uint16_t* vg_base = a.v + (size_t)k0 * kstride + (size_t)hk * D;
  i32x4 rk[CPT], rv[CPT];
  auto gload = [&](int kb) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int ci = tid + 256 * u;
      const int row = ci / KCH, ch = ci % KCH;
      const int key = kb * BN + row;
      if (key < lk) {
        rk[u] = *(const i32x4*)(kg_base + (size_t)key * kstride + ch * 8);
        rv[u] = *(const i32x4*)(vg_base + (size_t)key * kstride + ch * 8);
      } else {
        rk[u] = i32x4{0, 0, 0, 0};  // rows past the end: zeros (never NaN)
        rv[u] = i32x4{0, 0, 0, 0};
      }
    }
  };
  auto sstore = [&](int buf) {
    EA_LDS uint16_t* ks = sm + buf * 2 * TILE;
    EA_LDS uint16_t* vs = ks + TILE;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int ci = tid + 256 * u;
      const int row = ci / KCH, ch = ci % KCH;
      const int o = row * D + ((ch ^ swz<D>(row)) << 3);
      lds_store<i32x4>(ks + o, rk[u]);
      lds_store<i32x4>(vs + o, rv[u]);
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
  const float sl = a.scale_log2;

  if (nkb > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  // transposed-read lane geometry (see ea_device.h for the instruction's layout)
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int wave_last_q = row_lo + w * 32 + 31;

  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nkb) gload(kb + 1);
    const EA_LDS uint16_t* ks = sm + cur * 2 * TILE;
    const EA_LDS uint16_t* vs = ks + TILE;
    const int kbase = kb * BN;
    bool active = true;
    if constexpr (CAUSAL) active = kbase <= wave_last_q + off;
    if (active) {
      // ---- S^T = K Q^T (two 32-key tiles)
      f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 ka0 = lds_load<bf16x8>(ks + tile_off<D>(c, 16 * kk + 8 * hh));
        const bf16x8 ka1 = lds_load<bf16x8>(ks + tile_off<D>(32 + c, 16 * kk + 8 * hh));
        s0 = mfma32x32x16(ka0, qf[kk], s0);
        s1 = mfma32x32x16(ka1, qf[kk], s1);
      }
      // ---- mask: keys past the sequence end, and above the causal diagonal
      bool need_mask = kbase + BN > lk;
      if constexpr (CAUSAL) need_mask = need_mask || (kbase + BN - 1 > row_lo + w * 32 + off);
      if (need_mask) {
        int lim = lk;
        if constexpr (CAUSAL) lim = min(lk, qi + off + 1);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kbase + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (key >= lim) s0[i] = kNegInf;
          if (key + 32 >= lim) s1[i] = kNegInf;
        }
      }
      // ---- row max (raw scores; scale > 0 commutes with max)
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, __builtin_fmaxf(s0[i], s1[i]));
      mx = max_with_partner32(mx);
      const float m_new = __builtin_fmaxf(m_run, mx * sl);
      // ---- lazy rescale, wave-uniform
      if (__ballot(m_new > m_run + a.tau)) {
        const float alpha = (m_run == kNegInf) ? 0.f : exp2_hw(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
        m_run = m_new;
      }
      const float neg_m = (m_run == kNegInf) ? 0.f : -m_run;
      // ---- P = 2^(s*scale*log2e - m) in fp32; the row sum is taken before the
      //      bf16 rounding (keeps the log-sum-exp accurate on short rows)
      float p0[16], p1[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p0[i] = softmax_exp2<D, EXPMODE>(__builtin_fmaf(s0[i], sl, neg_m), i);
        p1[i] = softmax_exp2<D, EXPMODE>(__builtin_fmaf(s1[i], sl, neg_m), i);
      }
      float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        ls0 += p0[i];
        ls1 += p1[i];
      }
      l_run += ls0 + ls1;
      uint32_t pk[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pk[i] = pack_bf16x2(p0[2 * i], p0[2 * i + 1]);
        pk[8 + i] = pack_bf16x2(p1[2 * i], p1[2 * i + 1]);
      }
      bf16x8 pb[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        i32x4 t = {(int)pk[4 * st], (int)pk[4 * st + 1], (int)pk[4 * st + 2], (int)pk[4 * st + 3]};
        pb[st] = __builtin_bit_cast(bf16x8, t);
      }
      // ---- O^T += V^T P^T
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int r0 = 16 * st + tr_row;
          const int col = 32 * dt + tr_col;
          const i16x4 lo = ds_read_tr16(vs + tile_off<D>(r0, col));
          const i16x4 hi = ds_read_tr16(vs + tile_off<D>(r0 + 8, col));
          i32x4 t = {__builtin_bit_cast(i32x2, lo)[0], __builtin_bit_cast(i32x2, lo)[1],
                     __builtin_bit_cast(i32x2, hi)[0], __builtin_bit_cast(i32x2, hi)[1]};
          oacc[dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, t), pb[st], oacc[dt]);
        }
      }
    }
    if (kb + 1 < nkb) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---------------- epilogue: O = acc / l (bf16), lse = ln2 * (m + log2 l)
  const float l_tot = sum_with_partner32(l_run);
  const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
  if (qi < lq) {
    uint16_t* op = a.o + (size_t)(q0 + qi) * qstride + (size_t)h * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * dt + 8 * g4 + 4 * hh;
        uint2 val;
        val.x = pack_bf16x2(oacc[dt][4 * g4] * inv, oacc[dt][4 * g4 + 1] * inv);
        val.y = pack_bf16x2(oacc[dt][4 * g4 + 2] * inv, oacc[dt][4 * g4 + 3] * inv);
        *(uint2*)(op + d0) = val;
      }
    }
    if (a.lse != nullptr && hh == 0) {
      const float v = (l_tot > 0.f && m_run != kNegInf) ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
      size_t idx;
      if constexpr (VARLEN) {
        idx = (size_t)h * a.total_q + q0 + qi;
      } else {
        idx = ((size_t)seq * a.Hq + h) * a.Nq + qi;
      }
      a.lse[idx] = v;
    }
  }
}

int fwd_grid(const FwdArgs& a, bool varlen) {
  (void)varlen;
  const int ngroups = a.nseq * a.Hq;
  const int per_xcd_groups = (ngroups + 7) / 8;
  return 8 * per_xcd_groups * a.n_mb;
}

template <int D, bool CAUSAL, bool VARLEN, int EXPMODE>
static hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
  const int grid = fwd_grid(a, VARLEN);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, VARLEN, EXPMODE>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool VARLEN>
static hipError_t launch_e(const FwdArgs& a, int exp_mode, hipStream_t s) {
  switch (exp_mode) {
    case 1: return launch_t<D, CAUSAL, VARLEN, 1>(a, s);
    case 2: return launch_t<D, CAUSAL, VARLEN, 2>(a, s);
    default: return launch_t<D, CAUSAL, VARLEN, 0>(a, s);
  }
}

template <int D>
static hipError_t launch_d(const FwdArgs& a, bool causal, bool varlen, int exp_mode, hipStream_t s) {
  if (causal) {
    return varlen ? launch_e<D, true, true>(a, exp_mode, s) : launch_e<D, true, false>(a, exp_mode, s);
  }
  return varlen ? launch_e<D, false, true>(a, exp_mode, s) : launch_e<D, false, false>(a, exp_mode, s);
}

hipError_t launch_fwd(const FwdArgs& a, int d, bool causal, bool varlen, int exp_mode, hipStream_t s) {
  if (d == 64) return launch_d<64>(a, causal, varlen, exp_mode, s);
  return launch_d<128>(a, causal, varlen, exp_mode, s);
}

}  // namespace ea
