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

template <int D, bool CAUSAL, bool VARLEN, int EXPMODE, int NW>
__global__ __launch_bounds__(64 * NW, 2) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int BM = 32 * NW, BN = kFwdBlockN;
  constexpr int NT = 64 * NW;              // threads per workgroup
  constexpr int KCH = D / 8;               // 16-byte chunks per row
  constexpr int TILE = BN * D;             // bf16 elements per K or V tile
  constexpr int CPT = BN * KCH / NT;       // chunks per thread per tile
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
    // groups (virtual sequence, head), dealt to the XCDs in snake order
    // (round k: XCD x takes group 8k + x for even k, 8k + 7 - x for odd k),
    // so a heaviest-first order pairs heavy groups with light ones; the
    // optional order maps a virtual sequence to the actual one
    int g = xcd, nm = 0, s = 0;
    for (int k = 0;; ++k) {
      g = 8 * k + ((k & 1) ? 7 - xcd : xcd);
      if (g >= ngroups) break;
      s = varlen_seq(a.seq_order, a.nseq, g / a.Hq);
      nm = s < 0 ? 0 : (a.cu_q[s + 1] - a.cu_q[s] + BM - 1) / BM;
      if (j < nm) break;
      j -= nm;
    }
    if (g >= ngroups) return;
    seq = s;
    h = g - (g / a.Hq) * a.Hq;
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
  seq = uniform(seq);
  h = uniform(h);
  mb = uniform(mb);
  q0 = uniform(q0);
  lq = uniform(lq);
  k0 = uniform(k0);
  lk = uniform(lk);
  const int hk = uniform(h / a.group);
  const int off = lk - lq;  // bottom-right causal alignment
  const int row_lo = mb * BM;
  int nkeys = lk;
  if constexpr (CAUSAL) nkeys = min(lk, row_lo + BM + off);
  if (nkeys < 0) nkeys = 0;
  const int nkb = uniform((nkeys + BN - 1) / BN);

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
  // Buffer loads: the resource of tile kb starts at its first row and ends
  // after the sequence's last valid row, so rows past the end read as zeros
  // with no branch, and the per-lane byte offsets are loop-invariant.
  const uint16_t* kg_base = a.k + (size_t)k0 * kstride + (size_t)hk * D;
  const uint16_t* vg_base = a.v + (size_t)k0 * kstride + (size_t)hk * D;
  uint32_t g_off[CPT];
  int s_off[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int ci = tid + NT * u;
    const int row = ci / KCH, ch = ci % KCH;
    g_off[u] = (uint32_t)((row * (int)kstride + ch * 8) * 2);
    s_off[u] = row * D + ((ch ^ swz<D>(row)) << 3);
  }
  i32x4 rk[CPT], rv[CPT];
  auto gload = [&](int kb) {
    const int rows = min(lk - kb * BN, BN);
    const uint32_t nrec = (uint32_t)((rows - 1) * (int)kstride * 2 + D * 2);
    const size_t t0 = (size_t)kb * BN * kstride;
    const __amdgpu_buffer_rsrc_t rsk = make_rsrc(kg_base + t0, nrec);
    const __amdgpu_buffer_rsrc_t rsv = make_rsrc(vg_base + t0, nrec);
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      rk[u] = buffer_load16(rsk, g_off[u]);
      rv[u] = buffer_load16(rsv, g_off[u]);
    }
  };
  auto sstore = [&](int buf) {
    EA_LDS uint16_t* ks = sm + buf * 2 * TILE;
    EA_LDS uint16_t* vs = ks + TILE;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      lds_store<i32x4>(ks + s_off[u], rk[u]);
      lds_store<i32x4>(vs + s_off[u], rv[u]);
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
  // nothing outstanding when the loop starts (Q and tile 0 have landed)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // loop-invariant LDS element offsets of this lane's operand reads:
  //   K (A of S^T): rows c and c + 32 (+32 rows = +32*D), chunk 2*kk + hh
  //   V^T (A of O^T, transposed reads): rows 16*st + 8*r + tr_row (+16 rows =
  //   +16*D), columns 32*dt + tr_col
  int k_off[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) k_off[kk] = tile_off<D>(c, 16 * kk + 8 * hh);
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int v_off[NDT][2];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    v_off[dt][0] = tile_off<D>(tr_row, 32 * dt + tr_col);
    v_off[dt][1] = tile_off<D>(tr_row + 8, 32 * dt + tr_col);
  }
  const int wave_last_q = row_lo + w * 32 + 31;
  const int wave_first_q = row_lo + w * 32;

  auto compute = [&](int kb) {
    const EA_LDS uint16_t* ks = sm + (kb & 1) * 2 * TILE;
    const EA_LDS uint16_t* vs = ks + TILE;
    const int kbase = kb * BN;
    if (CAUSAL && kbase > wave_last_q + off) return;  // wave-uniform: fully masked
    // ---- S^T = K Q^T (two 32-key tiles)
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8 ka0 = lds_load<bf16x8>(ks + k_off[kk]);
      const bf16x8 ka1 = lds_load<bf16x8>(ks + k_off[kk] + 32 * D);
      s0 = mfma32x32x16(ka0, qf[kk], s0);
      s1 = mfma32x32x16(ka1, qf[kk], s1);
    }
    __builtin_amdgcn_s_setprio(0);
    // ---- mask: keys past the sequence end, and above the causal diagonal
    bool need_mask = kbase + BN > lk;
    if constexpr (CAUSAL) need_mask = need_mask || (kbase + BN - 1 > wave_first_q + off);
    if (need_mask) {
      int lim = lk;
      if constexpr (CAUSAL) lim = min(lk, qi + off + 1);
      const int rel = lim - kbase - 4 * hh;  // element i is valid iff its key offset < rel
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ko = 8 * (i >> 2) + (i & 3);
        s0[i] = (ko < rel) ? s0[i] : kNegInf;
        s1[i] = (ko + 32 < rel) ? s1[i] : kNegInf;
      }
    }
    // ---- row max (raw scores; scale > 0 commutes with max)
    float mx = kNegInf;
#pragma unroll
    // max(max(acc, a), b) per pair of scores folds into one three-input max
    for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(__builtin_fmaxf(mx, s0[i]), s1[i]);
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
    bf16x8 pb[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const float* src = (st < 2) ? p0 : p1;
      const int base = 8 * (st & 1);
      i32x4 t = {(int)pack_bf16x2(src[base + 0], src[base + 1]), (int)pack_bf16x2(src[base + 2], src[base + 3]),
                 (int)pack_bf16x2(src[base + 4], src[base + 5]), (int)pack_bf16x2(src[base + 6], src[base + 7])};
      pb[st] = __builtin_bit_cast(bf16x8, t);
    }
    // ---- O^T += V^T P^T
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const i16x4 lo = ds_read_tr16(vs + v_off[dt][0] + 16 * st * D);
        const i16x4 hi = ds_read_tr16(vs + v_off[dt][1] + 16 * st * D);
        i32x4 t = {__builtin_bit_cast(i32x2, lo)[0], __builtin_bit_cast(i32x2, lo)[1],
                   __builtin_bit_cast(i32x2, hi)[0], __builtin_bit_cast(i32x2, hi)[1]};
        oacc[dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, t), pb[st], oacc[dt]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // main loop: prefetch tile kb+1 into VGPRs, compute tile kb, park kb+1 in the
  // other LDS buffer; one barrier per tile. The last tile is peeled.
  for (int kb = 0; kb + 1 < nkb; ++kb) {
    gload(kb + 1);
    compute(kb);
    sstore((kb + 1) & 1);
    __syncthreads();
  }
  if (nkb > 0) compute(nkb - 1);

  // ---------------- epilogue: O = acc / l (bf16), lse = ln2 * (m + log2 l)
  const float l_tot = sum_with_partner32(l_run);
  const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
  uint4 pk[NDT][2];  // 16-byte row pieces (every lane takes part)
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) pack_rows16(oacc[dt], inv, pk[dt]);
  if (qi < lq) {
    uint16_t* op = a.o + (size_t)(q0 + qi) * qstride + (size_t)h * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int j = 0; j < 2; ++j) *(uint4*)(op + 32 * dt + 16 * j + 8 * hh) = pk[dt][j];
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
  constexpr int NW = kFwdBlockM / 32;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, VARLEN, EXPMODE, NW>), dim3(grid), dim3(64 * NW), 0, s, a);
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
