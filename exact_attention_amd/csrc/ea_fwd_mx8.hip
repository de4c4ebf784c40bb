// Exact attention forward with MX-scaled FP8 inputs (OCP e4m3, or e5m2 as
// "Faster, more flexible FlashAttention-4 for LLM inference", PR 2109, also
// allows) for gfx950. The input format only changes the format fields of the
// scaled MFMA; P is re-quantised to e4m3 in both cases.
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
#include "ea_fwd_common.h"
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

// Operand formats of the scaled MFMA (its cbsz / blgp fields): 0 = fp8 OCP
// e4m3, 1 = bf8 OCP e5m2.
constexpr int kFmtE4M3 = 0;
constexpr int kFmtE5M2 = 1;

template <int FA, int FB>
__device__ __forceinline__ f32x16 mfma_mx8(i32x8 a, i32x8 b, f32x16 c, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, scale_a, 0, scale_b);
}
// same, with the scale of A taken from byte SA of its register (the
// instruction's own byte select; the other bytes are ignored)
template <int SA, int FA, int FB>
__device__ __forceinline__ f32x16 mfma_mx8_sel(i32x8 a, i32x8 b, f32x16 c, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, SA, scale_a, 0, scale_b);
}

__device__ __forceinline__ i32x2 ds_read_tr8(const EA_LDS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((EA_LDS i32x2*)p);
}

// four fp32 -> four e4m3 bytes (round to nearest even; inputs stay below 448).
// The first conversion writes the low half of its destination and keeps the
// rest of the register it is given, which the second conversion then
// overwrites, so any register serves (x0's own bits: no zeroing move).
__device__ __forceinline__ int pack_fp8x4(float x0, float x1, float x2, float x3) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, __float_as_int(x0), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, lo, true);
}

constexpr int kScaleOne = 127;  // e8m0 encoding of 1.0

// the value must exist here (see keep() in ea_fwd_common.h)
__device__ __forceinline__ void keep8(const i32x8& x) { asm volatile("" ::"v"(x)); }

}  // namespace

// FMT: format of Q, K and V (kFmtE4M3 or kFmtE5M2); P is always e4m3.
template <bool CAUSAL, int FMT>
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
      s4 = *(const uint32_t*)(a.qs + (((size_t)b * a.Hq + h) * N + qi) * 4);
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
  const uint8_t* ksc_base = a.ks + ((size_t)b * a.Hkv + hk) * N * 4;
  const int nkb32 = N / 32;
  const uint8_t* vsc_base = a.vs + ((size_t)b * nkb32 * a.Hkv + hk) * D;
  const __amdgpu_buffer_rsrc_t rs_ksc = make_rsrc(ksc_base, (uint32_t)((N - 1) * 4 + 4));
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
      rks[t] = __builtin_amdgcn_raw_buffer_load_b32(rs_ksc, (key0 + 32 * t) * 4, 0, 0);
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
      s0 = mfma_mx8<FMT, FMT>(i32x8{a0l[0], a0l[1], a0l[2], a0l[3], a0h[0], a0h[1], a0h[2], a0h[3]}, qf[kq], s0,
                    kscale[0][kq], qsc[kq]);
      s1 = mfma_mx8<FMT, FMT>(i32x8{a1l[0], a1l[1], a1l[2], a1l[3], a1h[0], a1h[1], a1h[2], a1h[3]}, qf[kq], s1,
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
    // max(max(acc, a), b) per pair of scores folds into one three-input max
    for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(__builtin_fmaxf(mx, s0[i]), s1[i]);
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
      oacc[dt] = mfma_mx8<FMT, kFmtE4M3>(va, pb, oacc[dt], vscale[dt], kScaleOne);
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

// ---------------------------------------------------------------------------
// Software-pipelined 8-wave variant (same method and numerics as above; this
// file's own scheduling design). The fp8 products are twice as fast as bf16
// ones while the softmax costs the same, so a wave that runs them one after
// the other waits on each in turn. Here each wave issues, in one
// straight-line block per step, the MX MFMAs of S_{s+1} = K_{s+1} Q^T and of
// O += V_{s-1} P_{s-1} interleaved with the softmax of S_s (nothing in the
// block depends on anything else in it), in eight fenced slots of one MFMA
// each. 8 waves x 32 query rows; K/V tiles (64 keys x 128 bytes) arrive by
// LDS DMA into three stages per operand; the K scales of the next tile and
// the V scales of the current one are loaded a step ahead into registers.
// Masking runs before the block under a branch (diagonal and ragged tiles,
// and tiles past a wave's causal limit), the lazy O rescale after it.
template <bool CAUSAL, int FMT>
__device__ __forceinline__ void mx8_sp_tile(const Mx8Args& a, const int xcd, const int j) {
  constexpr int D = 128, BM = kPpBlockM, BN = kFwdBlockN;
  constexpr int TILE = BN * D;  // bytes per K or V tile
  constexpr int NDT = D / 32;
  static_assert(TILE == 8 * 1024, "one 1 KB DMA piece per wave per tile");
  __shared__ __attribute__((aligned(1024))) uint8_t ks0[TILE], ks1[TILE], ks2[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vs0[TILE], vs1[TILE], vs2[TILE];

  // ---------------- tile assignment: XCD-grouped, heaviest causal row blocks first
  const int kg = j / a.n_mb;
  const int r0 = j - kg * a.n_mb;
  const int g = xcd + 8 * kg;
  if (g >= a.B * a.Hq) return;
  const int b = uniform(g / a.Hq);
  const int h = uniform(g - b * a.Hq);
  const int mb = uniform(a.n_mb - 1 - r0);
  const int hk = uniform(h / a.group);
  const int N = a.N;
  const int row_lo = mb * BM;
  int nkeys = N;
  if constexpr (CAUSAL) nkeys = min(N, row_lo + BM);
  const int nkb = uniform((nkeys + BN - 1) / BN);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = uniform(tid >> 6), hh = lane >> 5, c = lane & 31;
  const int wave_first_q = row_lo + w * 32;
  const int qi = wave_first_q + c;
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
      s4 = *(const uint32_t*)(a.qs + (((size_t)b * a.Hq + h) * N + qi) * 4);
    } else {
      qf[0] = i32x8{};
      qf[1] = i32x8{};
    }
    qsc[0] = (s4 >> (8 * hh)) & 0xFF;
    qsc[1] = (s4 >> (8 * (2 + hh))) & 0xFF;
  }

  // ---------------- K/V DMA: wave w fills 1 KB piece w of a tile. Lane s
  // lands at tile byte 1024 w + 16 s = row 8 w + s / 8, slot s % 8; it fetches
  // the global chunk (s % 8) ^ swz8(row) of that row. A tile at or past nkb
  // gets no records, so its DMA writes zeros without touching memory; only
  // the last tile can be partial.
  const uint8_t* kg_base = a.k + ((size_t)b * N) * kstride + (size_t)hk * D;
  const uint8_t* vg_base = a.v + ((size_t)b * N) * kstride + (size_t)hk * D;
  const int drow = 8 * w + (lane >> 3);
  const uint32_t dma_off = (uint32_t)(drow * (int)kstride + (((lane & 7) ^ swz8(drow)) << 4));
  const uint32_t nrec_full = (uint32_t)uniform((BN - 1) * (int)kstride + D);
  const uint32_t nrec_last = (uint32_t)uniform(nkb > 0 ? (min(N - (nkb - 1) * BN, BN) - 1) * (int)kstride + D : 0);
  auto tile_rsrc = [&](const uint8_t* gbase, int t) __attribute__((always_inline)) {
    const uint32_t nrec = t < nkb - 1 ? nrec_full : (t == nkb - 1 ? nrec_last : 0u);
    return make_rsrc(gbase + (size_t)t * (BN * kstride), nrec);
  };
  auto kstage = [&](int r) __attribute__((always_inline)) -> EA_LDS uint8_t* {
    return r == 0 ? (EA_LDS uint8_t*)ks0 : r == 1 ? (EA_LDS uint8_t*)ks1 : (EA_LDS uint8_t*)ks2;
  };
  auto vstage = [&](int r) __attribute__((always_inline)) -> EA_LDS uint8_t* {
    return r == 0 ? (EA_LDS uint8_t*)vs0 : r == 1 ? (EA_LDS uint8_t*)vs1 : (EA_LDS uint8_t*)vs2;
  };
  auto dma_issue = [&](EA_LDS uint8_t* stage, __amdgpu_buffer_rsrc_t rs) __attribute__((always_inline)) {
    buffer_load16_lds(rs, (EA_LDS void*)(stage + 1024 * w), dma_off);
  };

  // ---------------- scales: K scale dwords of keys 64 t + c and 64 t + 32 + c,
  // V scale bytes of key block 2 t + hh, columns 32 dt + c (zero past the end)
  const uint8_t* ksc_base = a.ks + ((size_t)b * a.Hkv + hk) * N * 4;
  const int nkb32 = N / 32;
  const uint8_t* vsc_base = a.vs + ((size_t)b * nkb32 * a.Hkv + hk) * D;
  const __amdgpu_buffer_rsrc_t rs_ksc = make_rsrc(ksc_base, (uint32_t)((N - 1) * 4 + 4));
  const __amdgpu_buffer_rsrc_t rs_vsc = make_rsrc(vsc_base, (uint32_t)((nkb32 - 1) * a.Hkv * D + D));
  auto load_kscale = [&](int t, uint32_t (&dst)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      dst[u] = __builtin_amdgcn_raw_buffer_load_b32(rs_ksc, (t * BN + 32 * u + c) * 4, 0, 0);
  };
  auto load_vscale = [&](int t, uint32_t (&dst)[NDT]) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      dst[dt] = __builtin_amdgcn_raw_buffer_load_b8(rs_vsc, (2 * t + hh) * a.Hkv * D + 32 * dt + c, 0, 0);
  };

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

  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
  f32x16 sc0, sc1;                        // S of the tile whose softmax runs in this step
  f32x16 sn0 = f32x16{}, sn1 = f32x16{};  // S of the next tile
  i32x8 pprev = i32x8{}, pcur = i32x8{};  // P^T (e4m3) of the previous tile, of this one
  uint32_t kraw_cur[2], kraw_nxt[2];      // K scales of tile s + 1 (this step), s + 2
  uint32_t vraw_cur[NDT], vraw_nxt[NDT];  // V scales of tile s - 1 (this step), s
  const float sl = a.scale_log2;
  const float tau = a.tau;

  auto need_mask = [&](int s) __attribute__((always_inline)) {
    const int kbase = s * BN;
    bool m = kbase + BN > N;
    if constexpr (CAUSAL) m = m || (kbase + BN - 1 > wave_first_q);
    return m;
  };
  auto apply_mask = [&](int s) __attribute__((always_inline)) {
    int lim = N;
    if constexpr (CAUSAL) lim = min(N, qi + 1);
    const int rel = lim - s * BN - 4 * hh;  // element i is valid iff its key offset < rel
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int ko = 8 * (i >> 2) + (i & 3);
      sc0[i] = (ko < rel) ? sc0[i] : kNegInf;
      sc1[i] = (ko + 32 < rel) ? sc1[i] : kNegInf;
    }
  };

  // ---- the pipelined block of step s (stage r = s mod 3): slot j holds MFMA
  // j (j < 4: S_{s+1} key half j % 2, d half j / 2; j >= 4: PV for d tile
  // j - 4), the operand reads of the MFMA two slots later, and a share of the
  // softmax of S_s: the row max (slots 0-1), the rescale test (slot 1), exp2
  // and the row sum (slots 2-6), the e4m3 packing (slot 7). The scale loads
  // for the next step go in slot 0, this wave's DMA piece in slot 7.
  constexpr int NMF = 8, RA = 2, EXPS = 5;
  float alpha = 1.f;
  auto block = [&](int r, int s, __amdgpu_buffer_rsrc_t rs_k, __amdgpu_buffer_rsrc_t rs_v)
                   __attribute__((always_inline)) -> bool {
    const EA_LDS uint8_t* ks = kstage((r + 1) % 3);
    const EA_LDS uint8_t* vs = vstage((r + 2) % 3);
    const auto& ko = k_off;
    const auto& vo = v_off;
    // K scale of (key row, d block 2 k2 + hh) is byte 2 k2 + hh of its dword:
    // after a shift by 8 hh it is byte 2 k2, which the MFMA selects itself; a
    // V scale is byte 0 of its (zero-extended) load
    int ksh[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) ksh[t] = (int)(kraw_cur[t] >> (8 * hh));

    i32x8 opnd[NMF];
    auto read_operand = [&](int jx) __attribute__((always_inline)) {
      if (jx < 4) {
        const int t = jx & 1, k2 = jx >> 1;
        const i32x4 lo = lds_load<i32x4>(ks + ko[k2][0] + 32 * D * t);
        const i32x4 hi = lds_load<i32x4>(ks + ko[k2][1] + 32 * D * t);
        opnd[jx] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
        const int dt = jx - 4;
        const i32x2 q0 = ds_read_tr8(vs + vo[dt]);
        const i32x2 q1 = ds_read_tr8(vs + vo[dt] + 16 * D);
        const i32x2 q2 = ds_read_tr8(vs + vo[dt] + 32 * D);
        const i32x2 q3 = ds_read_tr8(vs + vo[dt] + 48 * D);
        opnd[jx] = i32x8{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
      }
    };
    auto elem = [&](int e) __attribute__((always_inline)) -> float { return e < 16 ? sc0[e] : sc1[e - 16]; };
    auto set_elem = [&](int e, float v) __attribute__((always_inline)) {
      if (e < 16) {
        sc0[e] = v;
      } else {
        sc1[e - 16] = v;
      }
    };
    auto exp_first = [](int k) { return (32 * k) / EXPS; };
    float mx0 = kNegInf, mx1 = kNegInf, neg_m = 0.f;
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
    bool resc = false;

#pragma unroll
    for (int jx = 0; jx < RA; ++jx) read_operand(jx);
    sched_fence();
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      if (i + RA < NMF) read_operand(i + RA);
      if (i < 4) {
        const int t = i & 1, k2 = i >> 1;
        f32x16& sn = t ? sn1 : sn0;
        if (k2 == 0) {
          sn = mfma_mx8_sel<0, FMT, FMT>(opnd[i], qf[0], f32x16{}, ksh[t], qsc[0]);
        } else {
          sn = mfma_mx8_sel<2, FMT, FMT>(opnd[i], qf[1], sn, ksh[t], qsc[1]);
        }
      } else {
        const int dt = i - 4;
        oacc[dt] = mfma_mx8<FMT, kFmtE4M3>(opnd[i], pprev, oacc[dt], (int)vraw_cur[dt], kScaleOne);
      }
      if (i == 0) {
        load_kscale(s + 2, kraw_nxt);
        load_vscale(s, vraw_nxt);
      }
      if (i < 2) {
        // row max over this lane's 32 keys, two chains of max3
#pragma unroll
        for (int e = 16 * i; e < 16 * i + 16; e += 4) {
          mx0 = __builtin_fmaxf(__builtin_fmaxf(mx0, elem(e)), elem(e + 2));
          mx1 = __builtin_fmaxf(__builtin_fmaxf(mx1, elem(e + 1)), elem(e + 3));
        }
      }
      if (i == 1) {
        // with the partner lane's 32 keys: the row max; the lazy rescale test;
        // rows that have seen no key yet keep m = -inf and get alpha = 0
        const float mx = max_with_partner32(__builtin_fmaxf(mx0, mx1));
        const float m_new = __builtin_fmaxf(m_run, mx * sl);
        resc = __ballot(m_new > m_run + tau) != 0;
        const float a_raw = exp2_hw(m_run - m_new);
        alpha = resc ? ((m_run == kNegInf) ? 0.f : a_raw) : 1.f;
        m_run = resc ? m_new : m_run;
        neg_m = (m_run == kNegInf) ? 0.f : -m_run;
      } else if (i >= 2 && i < 2 + EXPS) {
        const int e0 = exp_first(i - 2), e1 = exp_first(i - 1);
#pragma unroll
        for (int e = e0; e < e1; ++e) {
          const float p = exp2_hw(__builtin_fmaf(elem(e), sl, neg_m));
          set_elem(e, p);
          ls[e & 3] += p;
        }
      } else if (i == NMF - 1) {
        // P^T -> e4m3 (scale 1): bytes 0..15 key tile 0, 16..31 key tile 1
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          pcur[wd] = pack_fp8x4(sc0[4 * wd], sc0[4 * wd + 1], sc0[4 * wd + 2], sc0[4 * wd + 3]);
          pcur[4 + wd] = pack_fp8x4(sc1[4 * wd], sc1[4 * wd + 1], sc1[4 * wd + 2], sc1[4 * wd + 3]);
        }
        l_run = l_run * alpha + ((ls[0] + ls[1]) + (ls[2] + ls[3]));
        // this wave's piece of K_{s+3} (into the stage K_s left) and V_{s+1}
        // (into the stage V_{s-2} left)
        dma_issue(kstage(r), rs_k);
        dma_issue(vstage((r + 1) % 3), rs_v);
      }
      sched_fence();
    }
    // the softmax results and the next tile's scores must exist inside this
    // block (the compiler would otherwise sink their computation below the
    // rescale branch, or into the next step, next to their first use)
    keep(sn0);
    keep(sn1);
    keep8(pcur);
    keep(l_run);
    keep(m_run);
    keep(alpha);
    return resc;
  };

  // ---- one step: mask, block, rescale, rotate the pipeline registers, then
  // retire a stage: everything but this step's two DMA instructions (the
  // scale loads were issued before them) has landed, and every wave is past
  // its reads of the stages the next step's DMA overwrites
  auto step = [&](int r, int s) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs_k = tile_rsrc(kg_base, s + 3);
    const __amdgpu_buffer_rsrc_t rs_v = tile_rsrc(vg_base, s + 1);
    if (need_mask(s)) apply_mask(s);
    const bool resc = block(r, s, rs_k, rs_v);
    if (resc) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
    }
    sc0 = sn0;
    sc1 = sn1;
    pprev = pcur;
#pragma unroll
    for (int u = 0; u < 2; ++u) kraw_cur[u] = kraw_nxt[u];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) vraw_cur[dt] = vraw_nxt[dt];
    wait_vmcnt<2>();
    pp_barrier();
  };

  // prologue: K_0, K_1, K_2 and V_0 with the scales of K_0 and K_1; the V
  // stage that step 0 multiplies by P = 0 is zeroed; S_0 is computed here and
  // all waves are past their reads of K_0 before step 0 overwrites its stage
  lds_store<i32x4>((EA_LDS uint8_t*)vs2 + 16 * tid, i32x4{});
  uint32_t kraw0[2];
  load_kscale(0, kraw0);
  load_kscale(1, kraw_cur);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) vraw_cur[dt] = kScaleOne;
  // (under a branch: with no tiles there is nothing to fetch, and the wait
  // tracking then places no full wait at the loop head)
  if (nkb > 0) {
    dma_issue(kstage(0), tile_rsrc(kg_base, 0));
    dma_issue(kstage(1), tile_rsrc(kg_base, 1));
    dma_issue(kstage(2), tile_rsrc(kg_base, 2));
    dma_issue(vstage(0), tile_rsrc(vg_base, 0));
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const int s0k = (kraw0[0] >> (8 * (2 * k2 + hh))) & 0xFF;
    const int s1k = (kraw0[1] >> (8 * (2 * k2 + hh))) & 0xFF;
    const i32x4 a0l = lds_load<i32x4>((EA_LDS uint8_t*)ks0 + k_off[k2][0]);
    const i32x4 a0h = lds_load<i32x4>((EA_LDS uint8_t*)ks0 + k_off[k2][1]);
    const i32x4 a1l = lds_load<i32x4>((EA_LDS uint8_t*)ks0 + k_off[k2][0] + 32 * D);
    const i32x4 a1h = lds_load<i32x4>((EA_LDS uint8_t*)ks0 + k_off[k2][1] + 32 * D);
    sc0 = mfma_mx8<FMT, FMT>(i32x8{a0l[0], a0l[1], a0l[2], a0l[3], a0h[0], a0h[1], a0h[2], a0h[3]}, qf[k2],
                   k2 == 0 ? f32x16{} : sc0, s0k, qsc[k2]);
    sc1 = mfma_mx8<FMT, FMT>(i32x8{a1l[0], a1l[1], a1l[2], a1l[3], a1h[0], a1h[1], a1h[2], a1h[3]}, qf[k2],
                   k2 == 0 ? f32x16{} : sc1, s1k, qsc[k2]);
  }
  __syncthreads();

  // steps 0 .. nkb; the exits are breaks so that only the path through the
  // third step returns to the loop head
  for (int s = 0;; s += 3) {
    step(0, s);
    if (s + 1 > nkb) break;
    step(1, s + 1);
    if (s + 2 > nkb) break;
    step(2, s + 2);
    if (s + 3 > nkb) break;
  }
  // no DMA may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(0);

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

// ---------------------------------------------------------------------------
// Ping-pong variant (same method and numerics; the bf16 ping-pong kernel's
// schedule with the scaled products). 8 waves in two groups of four: wave w
// and wave w + 4 share a SIMD, and workgroup barriers keep the groups half a
// step apart, so while one group issues the eight MX MFMAs of a step (S_s =
// K_s Q^T and O += V_{s-1} P_{s-1}) from LDS operands, the other runs the
// softmax of S_{s-1} on the vector ALU. A single wave that interleaves both
// streams itself issues its vector work at half the rate of two waves; here
// the matrix core of each SIMD always has one wave feeding it and the vector
// work of a step is not split into slots around the products.
// Each wave owns 32 query rows, interleaved between the groups (wave w: rows
// 64 (w mod 4) + 32 (w div 4)) so both waves of a SIMD meet the causal
// diagonal at the same step. K/V tiles (64 keys x 128 B) and their scales
// arrive by LDS DMA -- K issued by group A, V by group B, each at the end of
// its MFMA part -- into three stages per operand: a stage holds the 8 KB
// tile and, behind it, 256
// scale bytes -- for K the 64 dwords of its keys (one e8m0 byte per 32-wide
// block of d), for V the two 32-key blocks' 128 bytes (one per d column) --
// so the MFMA part reads every operand, scales included, from LDS. Stages
// are distinct LDS objects and the loop is unrolled by three, so the
// compiler's wait tracking sees which stage each read uses. Two changes to
// the bf16 schedule move work out of the softmax phase, which bounds this
// kernel (the fp8 products take half the matrix-core time of bf16 ones while
// the exponentials cost the same): the masking and the row max of S_s run in
// the MFMA part, under its P V products, and each group issues half of the
// DMA at the end of its MFMA part.
template <bool CAUSAL, int FMT>
__device__ __forceinline__ void mx8_pp_tile(const Mx8Args& a, const int xcd, const int j) {
  constexpr int D = 128, BM = kPpBlockM, BN = kFwdBlockN;
  constexpr int TILE = BN * D;  // bytes per K or V tile
  constexpr int NDT = D / 32;
  constexpr int STAGE = TILE + 256;  // tile, then its scale bytes
  __shared__ __attribute__((aligned(1024))) uint8_t ks0[STAGE], ks1[STAGE], ks2[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t vs0[STAGE], vs1[STAGE], vs2[STAGE];

  // ---------------- tile assignment: XCD-grouped. One workgroup per tile:
  // heaviest causal row blocks first (dynamic dispatch balances the end).
  // Persistent form: a (batch, head)'s row blocks in ascending order. The
  // snake walk hands each workgroup a light and a heavy block, so every
  // workgroup's load is as balanced as in descending order; when a head has
  // more row blocks than its XCD has workgroups, the heavy blocks of the
  // later round then start on the keys the light blocks of the earlier round
  // have just brought into the XCD's L2, instead of rereading them from HBM.
  const int kg = j / a.n_mb;
  const int r0 = j - kg * a.n_mb;
  const int g = xcd + 8 * kg;
  if (g >= a.B * a.Hq) return;
  const int b = uniform(g / a.Hq);
  const int h = uniform(g - b * a.Hq);
  const int mb = uniform(a.persist_wgs > 0 ? r0 : a.n_mb - 1 - r0);
  const int hk = uniform(h / a.group);
  const int N = a.N;
  const int row_lo = mb * BM;
  int nkeys = N;
  if constexpr (CAUSAL) nkeys = min(N, row_lo + BM);
  const int nkb = uniform((nkeys + BN - 1) / BN);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = uniform(tid >> 6), hh = lane >> 5, c = lane & 31;
  const int grp = w >> 2;
  const int wave_first_q = row_lo + 64 * (w & 3) + 32 * grp;
  const int qi = wave_first_q + c;
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
      s4 = *(const uint32_t*)(a.qs + (((size_t)b * a.Hq + h) * N + qi) * 4);
    } else {
      qf[0] = i32x8{};
      qf[1] = i32x8{};
    }
    qsc[0] = (s4 >> (8 * hh)) & 0xFF;
    qsc[1] = (s4 >> (8 * (2 + hh))) & 0xFF;
  }

  // ---------------- DMA. Tiles: wave w of the issuing group fills 1 KB pieces
  // 2 (w mod 4) and 2 (w mod 4) + 1 of a tile; lane s of piece p lands at tile byte
  // 1024 p + 16 s = row 8 p + s / 8, slot s % 8, and fetches the global chunk
  // (s % 8) ^ swz8(row) of that row. A tile at or past nkb gets no records,
  // so its DMA writes zeros without touching memory; only the last tile can
  // be partial. Scales (one dword per lane): wave 0 the K scale dwords of the
  // tile's 64 keys, wave 5 the V scale bytes of its two 32-key blocks (lane s:
  // block s / 32, columns 4 (s % 32) .. +3).
  const uint8_t* kg_base = a.k + ((size_t)b * N) * kstride + (size_t)hk * D;
  const uint8_t* vg_base = a.v + ((size_t)b * N) * kstride + (size_t)hk * D;
  uint32_t dma_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int drow = 8 * (2 * (w & 3) + i) + (lane >> 3);
    dma_off[i] = (uint32_t)(drow * (int)kstride + (((lane & 7) ^ swz8(drow)) << 4));
  }
  const uint32_t nrec_full = (uint32_t)uniform((BN - 1) * (int)kstride + D);
  const uint32_t nrec_last = (uint32_t)uniform(nkb > 0 ? (min(N - (nkb - 1) * BN, BN) - 1) * (int)kstride + D : 0);
  const uint8_t* ksc_base = a.ks + ((size_t)b * a.Hkv + hk) * N * 4;
  const int nkb32 = N / 32;
  const uint8_t* vsc_base = a.vs + ((size_t)b * nkb32 * a.Hkv + hk) * D;
  const uint32_t ksc_off = (uint32_t)(lane * 4);
  const uint32_t vsc_off = (uint32_t)((lane >> 5) * a.Hkv * D + 4 * (lane & 31));
  auto dma_k = [&](EA_LDS uint8_t* stage, int t) __attribute__((always_inline)) {
    const uint32_t nrec = t < nkb - 1 ? nrec_full : (t == nkb - 1 ? nrec_last : 0u);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(kg_base + (size_t)t * (BN * kstride), nrec);
#pragma unroll
    for (int i = 0; i < 2; ++i) buffer_load16_lds(rs, (EA_LDS void*)(stage + 1024 * (2 * (w & 3) + i)), dma_off[i]);
    if (w == 0) {
      const int keys = t < nkb ? min(N - t * BN, BN) : 0;
      const __amdgpu_buffer_rsrc_t rsc =
          make_rsrc(ksc_base + (size_t)t * BN * 4, keys > 0 ? (uint32_t)((keys - 1) * 4 + 4) : 0u);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, (EA_LDS void*)(stage + TILE), 4, (int)ksc_off, 0, 0, 0);
    }
  };
  auto dma_v = [&](EA_LDS uint8_t* stage, int t) __attribute__((always_inline)) {
    const uint32_t nrec = t < nkb - 1 ? nrec_full : (t == nkb - 1 ? nrec_last : 0u);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(vg_base + (size_t)t * (BN * kstride), nrec);
#pragma unroll
    for (int i = 0; i < 2; ++i) buffer_load16_lds(rs, (EA_LDS void*)(stage + 1024 * (2 * (w & 3) + i)), dma_off[i]);
    if (w == 5) {
      const int blocks = t < nkb ? min(nkb32 - 2 * t, 2) : 0;
      const __amdgpu_buffer_rsrc_t rsc = make_rsrc(vsc_base + (size_t)(2 * t) * a.Hkv * D,
                                                   blocks > 0 ? (uint32_t)((blocks - 1) * a.Hkv * D + D) : 0u);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, (EA_LDS void*)(stage + TILE), 4, (int)vsc_off, 0, 0, 0);
    }
  };
  auto kstage = [&](int r) __attribute__((always_inline)) -> EA_LDS uint8_t* {
    return r == 0 ? (EA_LDS uint8_t*)ks0 : r == 1 ? (EA_LDS uint8_t*)ks1 : (EA_LDS uint8_t*)ks2;
  };
  auto vstage = [&](int r) __attribute__((always_inline)) -> EA_LDS uint8_t* {
    return r == 0 ? (EA_LDS uint8_t*)vs0 : r == 1 ? (EA_LDS uint8_t*)vs1 : (EA_LDS uint8_t*)vs2;
  };

  // LDS byte offsets of this lane's operand reads: K rows c and c + 32
  // (chunks 4 k2 + hh and 4 k2 + 2 + hh), V^T transposed reads, the K scale
  // dword of key c, the V scale byte of (block hh, column 32 dt + c)
  int k_off[2][2];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    k_off[k2][0] = tile8_off(c, 64 * k2 + 16 * hh);
    k_off[k2][1] = tile8_off(c, 64 * k2 + 32 + 16 * hh);
  }
  const int jj = (lane & 15) >> 1;
  const int tr_row = 4 * hh + jj + 4 * (jj >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
  int v_off[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) v_off[dt] = tile8_off(tr_row, 32 * dt + tr_col);
  int ksc_lds = TILE + 4 * c;
  int vsc_lds = TILE + 128 * hh + c;

  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
  f32x16 s0 = f32x16{}, s1 = f32x16{};
  i32x8 pb = i32x8{};  // P^T (e4m3) of the last softmax phase
  const float sl = a.scale_log2;
  const float tau = a.tau;
  const float thr = __builtin_amdgcn_exp2f(tau);  // 2^tau
  float neg_m_run = 0.f, thr_run = -1.f;

  // ---- MFMA part of step s: S_s = K_s Q^T into s0, s1, the masking of S_s
  // (diagonal and ragged tiles), then O += V_{s-1} P_{s-1} (pb). Vector work
  // placed under the four P V products measured slower than the same work
  // in the softmax phase. For a tile this wave skips, the softmax phase left P = 0; stages past the end hold zeros from
  // the DMA (scale code 0 is 2^-127, finite), and the V stage read at the
  // first step is zeroed, so the extra products add exact zeros.
  auto mfma_part = [&](const EA_LDS uint8_t* kst, const EA_LDS uint8_t* vst, int s) __attribute__((always_inline)) {
    // the offsets pass through an empty asm, so the stage base folds into
    // the ds_read offset field here instead of a register per stage
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      k_off[k2][0] = launder(k_off[k2][0]);
      k_off[k2][1] = launder(k_off[k2][1]);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) v_off[dt] = launder(v_off[dt]);
    ksc_lds = launder(ksc_lds);
    vsc_lds = launder(vsc_lds);
    // (at normal wave priority: here the softmax phase, not this part, sets
    // the step's length, and raising this part's priority, as the bf16
    // kernel does, measured 0.7% slower)
    // K scale of (key row, d block 2 k2 + hh) is byte 2 k2 + hh of its
    // dword: after a shift by 8 hh it is byte 2 k2, which the MFMA selects
    const int ksh0 = (int)(lds_load<uint32_t>(kst + ksc_lds) >> (8 * hh));
    const int ksh1 = (int)(lds_load<uint32_t>(kst + ksc_lds + 128) >> (8 * hh));
    i32x8 ka[4];
#pragma unroll
    for (int jx = 0; jx < 4; ++jx) {
      const int t = jx & 1, k2 = jx >> 1;
      const i32x4 lo = lds_load<i32x4>(kst + k_off[k2][0] + 32 * D * t);
      const i32x4 hi = lds_load<i32x4>(kst + k_off[k2][1] + 32 * D * t);
      ka[jx] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    int vsc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) vsc[dt] = (int)lds_load<uint8_t>(vst + vsc_lds + 32 * dt);
    i32x8 va[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const i32x2 q0 = ds_read_tr8(vst + v_off[dt]);
      const i32x2 q1 = ds_read_tr8(vst + v_off[dt] + 16 * D);
      const i32x2 q2 = ds_read_tr8(vst + v_off[dt] + 32 * D);
      const i32x2 q3 = ds_read_tr8(vst + v_off[dt] + 48 * D);
      va[dt] = i32x8{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
    }
    s0 = mfma_mx8_sel<0, FMT, FMT>(ka[0], qf[0], f32x16{}, ksh0, qsc[0]);
    s1 = mfma_mx8_sel<0, FMT, FMT>(ka[1], qf[0], f32x16{}, ksh1, qsc[0]);
    s0 = mfma_mx8_sel<2, FMT, FMT>(ka[2], qf[1], s0, ksh0, qsc[1]);
    s1 = mfma_mx8_sel<2, FMT, FMT>(ka[3], qf[1], s1, ksh1, qsc[1]);
    // the K scales and operands (10 reads) first, then four reads after each
    // S product and the last four behind them: every product's operands were
    // asked for at least one product (64 cycles) earlier
    __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    // masking (diagonal and ragged tiles only: this branch waits for S_s)
    const int kbase = s * BN;
    bool need_mask = kbase + BN > N;
    if constexpr (CAUSAL) need_mask = need_mask || (kbase + BN - 1 > wave_first_q);
    if (need_mask) {
      int lim = N;
      if constexpr (CAUSAL) lim = min(N, qi + 1);
      const int rel = lim - kbase - 4 * hh;  // element i is valid iff its key offset < rel
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ko = 8 * (i >> 2) + (i & 3);
        s0[i] = (ko < rel) ? s0[i] : kNegInf;
        s1[i] = (ko + 32 < rel) ? s1[i] : kNegInf;
      }
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = mfma_mx8<FMT, kFmtE4M3>(va[dt], pb, oacc[dt], vsc[dt], kScaleOne);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    // the products are issued here, before the barrier (the compiler would
    // otherwise sink them into the softmax phase, next to their first use)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) keep(oacc[dt]);
    keep(s0);
    keep(s1);
  };

  // ---- softmax phase of step s: P_s (e4m3, in pb) from S_s, with the lazy
  // rescale of O and l (threshold tau, log2) decided without the row max in
  // the common case. P is first formed against the running max m. If every
  // lane's sum of its 32 new P values is at most 2^tau, no P exceeds 2^tau, so
  // no row max exceeds m + tau and the rule keeps m: the P already formed are
  // the ones it forms. Otherwise (and while a row has no max yet) the row max
  // is taken from S_s, which is still intact, and the rule applied as
  // written, forming P again if m moved.
  auto p_half = [&](const f32x16& sv, int w0, float neg_m) __attribute__((always_inline)) -> float {
    // P over one 32-key half (this lane's 16 scores): fp32 sum (four partial
    // sums, so the adds do not form one dependent chain), and P^T as e4m3
    // (scale 1) in four dwords of pb: bytes 0..15 key tile 0, 16..31 tile 1
    float ls[4];
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      float p[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        p[k] = exp2_hw(__builtin_fmaf(sv[4 * wd + k], sl, neg_m));
        ls[k] = wd == 0 ? p[k] : ls[k] + p[k];
      }
      pb[w0 + wd] = pack_fp8x4(p[0], p[1], p[2], p[3]);
    }
    return (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };
  auto valu_part = [&](bool act) __attribute__((always_inline)) {
    if (!act) {
      pb = i32x8{};
      return;
    }
    const float ls0 = p_half(s0, 0, neg_m_run);
    float lsum = ls0 + p_half(s1, 4, neg_m_run);
    // thr_run is 2^tau, or -1 while the row has no max (the test then fails)
    if (__ballot(!(lsum <= thr_run))) {
      // row max over this lane's 32 keys in two chains of three-input max,
      // then over the partner lane's 32
      float mx0 = kNegInf, mx1 = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        mx0 = __builtin_fmaxf(__builtin_fmaxf(mx0, s0[i]), s1[i]);
        mx1 = __builtin_fmaxf(__builtin_fmaxf(mx1, s0[i + 1]), s1[i + 1]);
      }
      const float mx = max_with_partner32(__builtin_fmaxf(mx0, mx1));
      const float m_new = __builtin_fmaxf(m_run, mx * sl);
      if (__ballot(m_new > m_run + tau)) {
        const float alpha = (m_run == kNegInf) ? 0.f : exp2_hw(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
        m_run = m_new;
        neg_m_run = (m_run == kNegInf) ? 0.f : -m_run;
        thr_run = (m_run == kNegInf) ? -1.f : thr;
        const float l0 = p_half(s0, 0, neg_m_run);
        lsum = l0 + p_half(s1, 4, neg_m_run);
      }
    }
    // the row sum in fp32, before the e4m3 rounding of P
    l_run += lsum;
  };

  // a tile is fully masked for this wave (wave-uniform) if its first key lies
  // beyond the wave's last row
  auto tile_dead = [&](int s) __attribute__((always_inline)) { return CAUSAL && s * BN > wave_first_q + 31; };

  // ---- one step: MFMA part, DMA, barrier, softmax phase, barrier. Group B
  // starts one barrier late. At the end of its MFMA part group A issues
  // K_{s+2} (into the stage K_{s-1} left, which both groups finished reading
  // in step s - 1) and waits for it at the end of its next softmax phase;
  // group B issues V_{s+1} (into the stage of V_{s-2}) and waits for it at the
  // end of its next MFMA part. Either wait leaves only the newest pieces in
  // flight and comes before the barrier after which the other group reads
  // them. Waves 0 and 5 issue one scale DMA more.
  auto step = [&](int r, int s) __attribute__((always_inline)) {
    const bool act = s < nkb && !tile_dead(s);
    mfma_part(kstage(r), vstage((r + 2) % 3), s);
    if (grp == 0) {
      dma_k(kstage((r + 2) % 3), s + 2);
    } else {
      dma_v(vstage((r + 1) % 3), s + 1);
      // V_s (issued one step earlier) has landed before the barrier after
      // which group A reads it
      if (w == 5) {
        wait_vmcnt<3>();
      } else {
        wait_vmcnt<2>();
      }
    }
    pp_barrier();
    valu_part(act);
    if (grp == 0) {
      if (w == 0) {
        wait_vmcnt<3>();
      } else {
        wait_vmcnt<2>();
      }
    }
    pp_barrier();
  };

  // prologue: K_0, K_1 and V_0 with their scales; the V stage (tile and
  // scales) that step 0 multiplies by P = 0 is zeroed so it holds no NaN code
  lds_store<i32x4>((EA_LDS uint8_t*)vs2 + 16 * tid, i32x4{});
  if (tid < 16) lds_store<i32x4>((EA_LDS uint8_t*)vs2 + TILE + 16 * tid, i32x4{});
  if (nkb > 0) {
    if (grp == 0) {
      dma_k(kstage(0), 0);
      dma_k(kstage(1), 1);
    } else {
      dma_v(vstage(0), 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  if (grp == 1) pp_barrier();  // group B runs one phase behind
  for (int s = 0; s <= nkb; s += 3) {
    step(0, s);
    if (s + 1 <= nkb) step(1, s + 1);
    if (s + 2 <= nkb) step(2, s + 2);
  }
  if (grp == 0) pp_barrier();
  // no DMA may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(0);

  // ---------------- epilogue
  const float l_tot = sum_with_partner32(l_run);
  const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
  uint4 pk[NDT][2];  // 16-byte row pieces (every lane takes part)
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) pack_rows16(oacc[dt], inv, pk[dt]);
  if (qi < N) {
    uint16_t* op = a.o + ((size_t)b * N + qi) * qstride + (size_t)h * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      // (plain stores: streaming ones measured 1.2% faster here but let the
      // 32-byte row pieces reach HBM unmerged, 1.10x the algorithmic bytes
      // instead of 1.00x)
      for (int j = 0; j < 2; ++j) *(uint4*)(op + 32 * dt + 16 * j + 8 * hh) = pk[dt][j];
    }
    if (a.lse != nullptr && hh == 0) {
      const float v = (l_tot > 0.f && m_run != kNegInf) ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
      a.lse[((size_t)b * a.Hq + h) * N + qi] = v;
    }
  }
}

template <bool CAUSAL, int FMT>
__global__ __launch_bounds__(512, 1) void fwd_mx8_pp_kernel(Mx8Args a) {
  mx8_pp_tile<CAUSAL, FMT>(a, blockIdx.x & 7, blockIdx.x >> 3);
}

template <bool CAUSAL, int FMT>
__global__ __launch_bounds__(512, 1) void fwd_mx8_pp_persistent_kernel(Mx8Args a) {
  persistent_snake(uniform(a.tiles_per_xcd), [&](int xcd, int j) { mx8_pp_tile<CAUSAL, FMT>(a, xcd, j); });
}

template <bool CAUSAL, int FMT>
__global__ __launch_bounds__(512, 1) void fwd_mx8_sp_kernel(Mx8Args a) {
  mx8_sp_tile<CAUSAL, FMT>(a, blockIdx.x & 7, blockIdx.x >> 3);
}


template <int FMT>
static hipError_t launch_mx8_f(const Mx8Args& a, bool causal, bool pipelined, hipStream_t s) {
  const int grid = 8 * ((a.B * a.Hq + 7) / 8) * a.n_mb;
  if (pipelined) {
    if (causal) {
      hipLaunchKernelGGL((fwd_mx8_sp_kernel<true, FMT>), dim3(grid), dim3(512), 0, s, a);
    } else {
      hipLaunchKernelGGL((fwd_mx8_sp_kernel<false, FMT>), dim3(grid), dim3(512), 0, s, a);
    }
  } else {
    if (causal) {
      hipLaunchKernelGGL((fwd_mx8_kernel<true, FMT>), dim3(grid), dim3(256), 0, s, a);
    } else {
      hipLaunchKernelGGL((fwd_mx8_kernel<false, FMT>), dim3(grid), dim3(256), 0, s, a);
    }
  }
  return hipGetLastError();
}

// persistent form (one workgroup per CU walking the XCD-grouped tile list,
// persistent_snake in ea_fwd_common.h) when a.persist_wgs > 0
template <int FMT>
static hipError_t launch_mx8_pp_f(const Mx8Args& a, bool causal, hipStream_t s) {
  const int grid = 8 * ((a.B * a.Hq + 7) / 8) * a.n_mb;
  if (a.persist_wgs > 0) {
    Mx8Args b = a;
    b.tiles_per_xcd = grid / 8;
    const int w = max(1, min(a.persist_wgs / 8, b.tiles_per_xcd));  // workgroups per XCD
    if (causal) {
      hipLaunchKernelGGL((fwd_mx8_pp_persistent_kernel<true, FMT>), dim3(8 * w), dim3(512), 0, s, b);
    } else {
      hipLaunchKernelGGL((fwd_mx8_pp_persistent_kernel<false, FMT>), dim3(8 * w), dim3(512), 0, s, b);
    }
  } else if (causal) {
    hipLaunchKernelGGL((fwd_mx8_pp_kernel<true, FMT>), dim3(grid), dim3(512), 0, s, a);
  } else {
    hipLaunchKernelGGL((fwd_mx8_pp_kernel<false, FMT>), dim3(grid), dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_mx8_pp(const Mx8Args& a, bool causal, hipStream_t s) {
  return a.fmt == kFmtE5M2 ? launch_mx8_pp_f<kFmtE5M2>(a, causal, s) : launch_mx8_pp_f<kFmtE4M3>(a, causal, s);
}

hipError_t launch_fwd_mx8_sp(const Mx8Args& a, bool causal, hipStream_t s) {
  return a.fmt == kFmtE5M2 ? launch_mx8_f<kFmtE5M2>(a, causal, true, s) : launch_mx8_f<kFmtE4M3>(a, causal, true, s);
}

hipError_t launch_fwd_mx8(const Mx8Args& a, bool causal, hipStream_t s) {
  return a.fmt == kFmtE5M2 ? launch_mx8_f<kFmtE5M2>(a, causal, false, s) : launch_mx8_f<kFmtE4M3>(a, causal, false, s);
}

}  // namespace ea
