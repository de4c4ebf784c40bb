// Exact attention forward with MX-scaled FP8 (OCP e4m3) inputs for gfx950.
//
// Method ("Low-precision FlashAttention-4: end-to-end block-scaled attention
// for Blackwell", section 2.1): both contractions use block-scaled MMA with
// one e8m0 scale per 32 elements along the GEMM K dimension -- for Q K^T that
// is the head dimension of Q and K, for P V it is the sequence dimension of V.
// P is re-quantised to FP8 on the fly before P V (section 2.1.3), here with a
// constant scale of 1: with the lazy rescale below, P <= 2^8 = 256, inside the
// e4m3 range (448), which is the constant-P-scale option of that section.
// The online softmax (running max, running sum, rescaled accumulator) is that
// of "FlashAttention: not less compute, less data movement", section 02; the
// softmax runs in fp32.
//
// gfx950 mapping: same workgroup layout as the bf16 forward (4 waves x 32
// query rows, 64-key tiles double-buffered in LDS, S^T = K Q^T so each lane
// owns a query column), with v_mfma_scale_f32_32x32x64_f8f6f4 for both
// products. Lane layout of that instruction for fp8 operands: lane l holds
// row/column l%32 and k = 16*(l/32) + 0..15 (bytes 0..15) and
// 32 + 16*(l/32) + 0..15 (bytes 16..31); the scale of (row m, k-block b) comes
// from lane m + 32*b. The P^T bytes come straight from the S^T accumulator
// (k-local block b <-> key tile b, keys permuted inside it); V^T operands are
// read from the row-major V tile with ds_read_b64_tr_b8 using the same key
// permutation.
#include "ea_device.h"
#include "ea_internal.h"

namespace ea {

namespace {

// fp8 tiles: rows of 128 bytes (8 chunks of 16 bytes), chunk position =
// chunk ^ swz8(row). A linear map of row bits 1..3 chosen so that both the
// MFMA operand reads (16 rows at one chunk) and the transposed V reads
// (8 rows x 2 chunks per 32 lanes) hit 16 distinct 16-byte bank groups when a
// 256-byte bank line holds two rows. Depends on row % 16 only.
__device__ __forceinline__ int swz8(int row) {
  return (((row >> 1) & 1) << 1) | ((row >> 2) & 1) | (((row >> 3) & 1) << 2);
}
__device__ __forceinline__ int tile8_off(int row, int col) {
  return row * 128 + (((col >> 4) ^ swz8(row)) << 4) + (col & 15);
}

__device__ __forceinline__ f32x16 mfma_mx8(i32x8 a, i32x8 b, f32x16 c, int scale_a, int scale_b) {
  // formats: 0 = fp8 e4m3 for both operands
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}

__device__ __forceinline__ i32x2 ds_read_tr8(const EA_LDS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((EA_LDS i32x2*)p);
}

// four fp32 -> four e4m3 bytes (round to nearest even; inputs stay below 448)
__device__ __forceinline__ int pack_fp8x4(float x0, float x1, float x2, float x3) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, lo, true);
}

constexpr int kScaleOne = 127;  // e8m0 encoding of 1.0

}  // namespace

template <bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_mx8_kernel(Mx8Args a) {
  constexpr int D = 128, BM = kFwdBlockM, BN = kFwdBlockN;
  constexpr int TILE = BN * D;            // bytes per K or V tile
  constexpr int CPT = TILE / 16 / 256;    // 16-byte chunks per thread per tile
  constexpr int NDT = D / 32;
  __shared__ __attribute__((aligned(16))) uint8_t smem_raw[2 * 2 * TILE];
  EA_LDS uint8_t* sm = (EA_LDS uint8_t*)smem_raw;

  // ---------------- tile assignment: XCD-grouped, heaviest causal row blocks first
  const int xcd = blockIdx.x & 7;
  const int j = blockIdx.x >> 3;
  const int kg = j / a.n_mb;
  const int r = j - kg * a.n_mb;
  const int g = xcd + 8 * kg;
  if (g >= a.B * a.Hq) return;
  const int b = uniform(g / a.Hq);
  const int h = uniform(g - b * a.Hq);
  const int mb = uniform(a.n_mb - 1 - r);
  const int hk = uniform(h / a.group);
  const int N = a.N;
  const int row_lo = mb * BM;
  int nkeys = N;
  if constexpr (CAUSAL) nkeys = min(N, row_lo + BM);
  const int nkb = uniform((nkeys + BN - 1) / BN);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, hh = lane >> 5, c = lane & 31;
  const int qi = row_lo + w * 32 + c;
  const size_t qstride = (size_t)a.Hq * D, kstride = (size_t)a.Hkv * D;

  // ---------------- Q^T operand and its scales (B of S^T), kept in VGPRs
  i32x8 qf[2];
  int qsc[2];
  {
    const uint8_t* qp = a.q + ((size_t)b * N + qi) * qstride + (size_t)h * D;
    uint32_t s4 = 0x7f7f7f7fu;
    if (qi < N) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const i32x4 lo = *(const i32x4*)(qp + 64 * ks + 16 * hh);
        const i32x4 hi = *(const i32x4*)(qp + 64 * ks + 32 + 16 * hh);
        qf[ks] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      s4 = *(const uint32_t*)(a.qs + (((size_t)b * N + qi) * a.Hq + h) * 4);
    } else {
      qf[0] = i32x8{};
      qf[1] = i32x8{};
    }
    qsc[0] = (s4 >> (8 * hh)) & 0xFF;
    qsc[1] = (s4 >> (8 * (2 + hh))) & 0xFF;
  }

  // ---------------- K/V tiles (buffer loads, zero past the end) and scales
  const uint8_t* kg_base = a.k + ((size_t)b * N) * kstride + (size_t)hk * D;
  const uint8_t* vg_base = a.v + ((size_t)b * N) * kstride + (size_t)hk * D;
  const uint8_t* ksc_base = a.ks + ((size_t)b * N * a.Hkv + hk) * 4;
  const int nkb32 = N / 32;
  const uint8_t* vsc_base = a.vs + ((size_t)b * nkb32 * a.Hkv + hk) * D;
  const __amdgpu_buffer_rsrc_t rs_ksc = make_rsrc(ksc_base, (uint32_t)((N - 1) * a.Hkv * 4 + 4));
  const __amdgpu_buffer_rsrc_t rs_vsc = make_rsrc(vsc_base, (uint32_t)((nkb32 - 1) * a.Hkv * D + D));
  uint32_t g_off[CPT];
  int s_off[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int ci = tid + 256 * u;
    const int row = ci >> 3, ch = ci & 7;
    g_off[u] = (uint32_t)(row * (int)kstride + ch * 16);
    s_off[u] = row * D + ((ch ^ swz8(row)) << 4);
  }
  i32x4 rk[CPT], rv[CPT];
  uint32_t rks[2];   // K scale dwords of keys kbase + c and kbase + 32 + c
  uint32_t rvs[NDT]; // V scale bytes of key block kbase/32 + hh, columns 32*dt + c
  auto gload = [&](int kb) {
    const int rows = min(N - kb * BN, BN);
    const uint32_t nrec = (uint32_t)((rows - 1) * (int)kstride + D);
    const size_t t0 = (size_t)kb * BN * kstride;
    const __amdgpu_buffer_rsrc_t rsk = make_rsrc(kg_base + t0, nrec);
    const __amdgpu_buffer_rsrc_t rsv = make_rsrc(vg_base + t0, nrec);
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      rk[u] = buffer_load16(rsk, g_off[u]);
      rv[u] = buffer_load16(rsv, g_off[u]);
    }
    const int key0 = kb * BN + c;
#pragma unroll
    for (int t = 0; t < 2; ++t)
      rks[t] = __builtin_amdgcn_raw_buffer_load_b32(rs_ksc, (key0 + 32 * t) * a.Hkv * 4, 0, 0);
    const int kb32 = kb * 2 + hh;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      rvs[dt] = __builtin_amdgcn_raw_buffer_load_b8(rs_vsc, kb32 * a.Hkv * D + 32 * dt + c, 0, 0);
  };
  int ksc[2][2], vsc[NDT];
  auto sstore = [&](int buf) {
    EA_LDS uint8_t* ks = sm + buf * 2 * TILE;
    EA_LDS uint8_t* vs = ks + TILE;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      lds_store<i32x4>(ks + s_off[u], rk[u]);
      lds_store<i32x4>(vs + s_off[u], rv[u]);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) ksc[t][ks2] = (rks[t] >> (8 * (2 * ks2 + hh))) & 0xFF;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) vsc[dt] = (int)(rvs[dt] & 0xFF);
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
  const float sl = a.scale_log2;
  const int wave_first_q = row_lo + w * 32;

  // loop-invariant LDS byte offsets: K operand (rows c, c + 32; chunks
  // 4*ks + hh and 4*ks + 2 + hh) and V^T transposed reads
  int k_off[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    k_off[ks][0] = tile8_off(c, 64 * ks + 16 * hh);
    k_off[ks][1] = tile8_off(c, 64 * ks + 32 + 16 * hh);
  }
  const int jj = (lane & 15) >> 1;
  const int tr_row = 4 * hh + jj + 4 * (jj >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
  int v_off[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) v_off[dt] = tile8_off(tr_row, 32 * dt + tr_col);

  if (nkb > 0) {
    gload(0);
    sstore(0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  auto compute = [&](int kb, const int (&kscale)[2][2], const int (&vscale)[NDT]) {
    const EA_LDS uint8_t* ks = sm + (kb & 1) * 2 * TILE;
    const EA_LDS uint8_t* vs = ks + TILE;
    const int kbase = kb * BN;
    // ---- S^T = K Q^T (two 32-key tiles, block-scaled)
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      const i32x4 a0l = lds_load<i32x4>(ks + k_off[kq][0]);
      const i32x4 a0h = lds_load<i32x4>(ks + k_off[kq][1]);
      const i32x4 a1l = lds_load<i32x4>(ks + k_off[kq][0] + 32 * D);
      const i32x4 a1h = lds_load<i32x4>(ks + k_off[kq][1] + 32 * D);
      s0 = mfma_mx8(i32x8{a0l[0], a0l[1], a0l[2], a0l[3], a0h[0], a0h[1], a0h[2], a0h[3]}, qf[kq], s0,
                    kscale[0][kq], qsc[kq]);
      s1 = mfma_mx8(i32x8{a1l[0], a1l[1], a1l[2], a1l[3], a1h[0], a1h[1], a1h[2], a1h[3]}, qf[kq], s1,
                    kscale[1][kq], qsc[kq]);
    }
    __builtin_amdgcn_s_setprio(0);
    // ---- mask
    bool need_mask = kbase + BN > N;
    if constexpr (CAUSAL) need_mask = need_mask || (kbase + BN - 1 > wave_first_q);
    if (need_mask) {
      int lim = N;
      if constexpr (CAUSAL) lim = min(N, qi + 1);
      const int rel = lim - kbase - 4 * hh;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ko = 8 * (i >> 2) + (i & 3);
        s0[i] = (ko < rel) ? s0[i] : kNegInf;
        s1[i] = (ko + 32 < rel) ? s1[i] : kNegInf;
      }
    }
    // ---- online softmax (fp32), lazy rescale with threshold tau (log2)
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, __builtin_fmaxf(s0[i], s1[i]));
    mx = max_with_partner32(mx);
    const float m_new = __builtin_fmaxf(m_run, mx * sl);
    if (__ballot(m_new > m_run + a.tau)) {
      const float alpha = (m_run == kNegInf) ? 0.f : exp2_hw(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
      m_run = m_new;
    }
    const float neg_m = (m_run == kNegInf) ? 0.f : -m_run;
    float p0[16], p1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p0[i] = exp2_hw(__builtin_fmaf(s0[i], sl, neg_m));
      p1[i] = exp2_hw(__builtin_fmaf(s1[i], sl, neg_m));
    }
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ls0 += p0[i];
      ls1 += p1[i];
    }
    l_run += ls0 + ls1;
    // ---- P^T -> e4m3 (scale 1), B operand: bytes 0..15 key tile 0, 16..31 key tile 1
    i32x8 pb;
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      pb[wd] = pack_fp8x4(p0[4 * wd], p0[4 * wd + 1], p0[4 * wd + 2], p0[4 * wd + 3]);
      pb[4 + wd] = pack_fp8x4(p1[4 * wd], p1[4 * wd + 1], p1[4 * wd + 2], p1[4 * wd + 3]);
    }
    // ---- O^T += V^T P^T (block-scaled along keys)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const i32x2 r0 = ds_read_tr8(vs + v_off[dt]);
      const i32x2 r1 = ds_read_tr8(vs + v_off[dt] + 16 * D);
      const i32x2 r2 = ds_read_tr8(vs + v_off[dt] + 32 * D);
      const i32x2 r3 = ds_read_tr8(vs + v_off[dt] + 48 * D);
      const i32x8 va = {r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
      oacc[dt] = mfma_mx8(va, pb, oacc[dt], vscale[dt], kScaleOne);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  for (int kb = 0; kb + 1 < nkb; ++kb) {
    const int kcur[2][2] = {{ksc[0][0], ksc[0][1]}, {ksc[1][0], ksc[1][1]}};
    const int vcur[NDT] = {vsc[0], vsc[1], vsc[2], vsc[3]};
    gload(kb + 1);
    compute(kb, kcur, vcur);
    sstore((kb + 1) & 1);
    __syncthreads();
  }
  if (nkb > 0) compute(nkb - 1, ksc, vsc);

  // ---------------- epilogue
  const float l_tot = sum_with_partner32(l_run);
  const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
  if (qi < N) {
    uint16_t* op = a.o + ((size_t)b * N + qi) * qstride + (size_t)h * D;
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
      a.lse[((size_t)b * a.Hq + h) * N + qi] = v;
    }
  }
}

hipError_t launch_fwd_mx8(const Mx8Args& a, bool causal, hipStream_t s) {
  const int grid = 8 * ((a.B * a.Hq + 7) / 8) * a.n_mb;
  if (causal) {
    hipLaunchKernelGGL(fwd_mx8_kernel<true>, dim3(grid), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(fwd_mx8_kernel<false>, dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace ea
