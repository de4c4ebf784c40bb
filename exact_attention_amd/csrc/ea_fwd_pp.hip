// Fused exact attention forward for gfx950, 8-wave ping-pong variant
// (bf16 in, fp32 accumulate).
//
// Method: as in the 4-wave kernel -- each workgroup owns a block of query rows
// of one (sequence, head) and streams over 64-key K/V tiles with the online
// softmax ("FlashAttention: not less compute, less data movement", sections
// 02-03), lazy rescale ("FlashAttention-4: algorithm-pipeline co-design for
// Blackwell", conditional softmax rescaling section) and the XCD-grouped,
// heaviest-first tile order ("FlashAttention4 close reading", section 3.3).
//
// The pages overlap the two matrix products with the exponentials by giving
// them to different warps of a Blackwell CTA. The gfx950 form of that idea
// (this file's own design):
//  * 8 waves = two groups of 4. Wave w and wave w + 4 run on the same SIMD, and
//    the groups are kept half a step apart by workgroup barriers: while group A
//    issues its MFMAs (S = K Q^T for tile s, O += V P for tile s - 1), group B
//    runs the softmax of tile s - 1 on the vector ALU, then they swap. The
//    matrix core of each SIMD thus always has one wave feeding it.
//  * Each wave owns 32 query rows (256 per workgroup); rows are interleaved
//    between the groups (wave w: rows 64 (w mod 4) + 32 (w / 4)) so both waves
//    of a SIMD meet the causal diagonal at the same step.
//  * K/V tiles arrive by LDS DMA (buffer_load ... lds, 16 bytes per lane) into
//    three stages per operand, issued four phases before use, so no VGPRs stage
//    them and every byte lands in the swizzled layout the operand reads
//    expect: each lane fetches the global chunk that belongs at its LDS
//    position. The four waves of group A issue a quarter of each tile each
//    and wait for it just before the barrier after which all read it.
//  * Both groups run the same straight-line step (MFMA part, barrier, VALU
//    part, barrier); group B is offset by one initial barrier. Code that
//    branched on the group kept both orders' temporaries alive and spilled.
//  * Stages are distinct LDS objects and the loop is unrolled by three, so the
//    compiler's own wait tracking sees which stage each read uses. The lane
//    offsets are re-materialised in each MFMA part so the stage base folds
//    into the 16-bit LDS offset field where it fits, instead of one hoisted
//    register copy per stage and offset.
//  * Operand layouts (S^T = K Q^T, P^T passed in registers to O^T = V^T P^T,
//    V^T from ds_read_b64_tr_b16) are those of the 4-wave kernel.
#include <type_traits>

#include "ea_device.h"
#include "ea_fwd_common.h"
#include "ea_internal.h"

namespace ea {

// One work tile (256 query rows of one (sequence, head)): the whole forward of
// those rows. xcd and j locate the tile in the XCD-grouped, heaviest-first order.
// D: head dim of Q and K; DV: head dim of V and O (equal, or 192 / 128).
template <int D, int DV, bool CAUSAL, bool VARLEN, int EXPMODE>
__device__ __forceinline__ void pp_tile(const FwdArgs& a, const int xcd, int j) {
  constexpr int BM = kPpBlockM, BN = kFwdBlockN;
  constexpr int TILE = BN * D;               // bf16 elements per K stage
  constexpr int VTILE = BN * DV;             // ... per V stage
  constexpr int NDT = DV / 32;               // 32-wide d tiles of O^T
  constexpr int ROWB = D * 2;                // bytes per K row
  constexpr int VROWB = DV * 2;              // bytes per V row
  constexpr int NI = TILE * 2 / 1024;        // 1 KB DMA instructions per K tile
  constexpr int IPW = NI / 4;                // ... per wave of group A
  constexpr int NIV = VTILE * 2 / 1024;      // ... per V tile
  constexpr int IPWV = NIV / 4;
  static_assert(IPW >= 1 && NI % 4 == 0 && IPWV >= 1 && NIV % 4 == 0,
                "tiles must split into 4 waves of 1 KB DMA");
  __shared__ __attribute__((aligned(1024))) uint16_t ks0[TILE], ks1[TILE], ks2[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vs0[VTILE], vs1[VTILE], vs2[VTILE];

  // ---------------- tile assignment (XCD-grouped, heaviest first)
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
  const int lane = tid & 63, w = uniform(tid >> 6), hh = lane >> 5, c = lane & 31;
  const int grp = w >> 2;                               // 0: group A, 1: group B
  const int wrow = row_lo + 64 * (w & 3) + 32 * grp;    // wave's first query row
  const int qi = wrow + c;                              // this lane's query row
  const size_t qstride = (size_t)a.Hq * D, kstride = (size_t)a.Hkv * D;
  const size_t ostride = (size_t)a.Hq * DV, vstride = (size_t)a.Hkv * DV;

  // ---------------- Q^T operand (B of S^T = K Q^T), kept in VGPRs
  bf16x8 qf[D / 16];
  {
    const uint16_t* qp = a.q + (size_t)(q0 + qi) * qstride + (size_t)h * D + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = (qi < lq) ? *(const bf16x8*)(qp + 16 * kk) : bf16x8{};
  }

  // ---------------- K/V DMA: wave w of group A fills 1 KB pieces w*IPW ..
  // w*IPW+IPW-1 of a tile. Lane s of piece p lands at stage byte 1024 p + 16 s = row r, slot sl;
  // it fetches the global 16-byte chunk sl ^ swz(r) of row r.
  const uint16_t* kg_base = a.k + (size_t)k0 * kstride + (size_t)hk * D;
  const uint16_t* vg_base = a.v + (size_t)k0 * vstride + (size_t)hk * DV;
  uint32_t dma_off[IPW], dma_voff[IPWV];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int p = 1024 * ((w & 3) * IPW + i) + 16 * lane;
    const int r = p / ROWB, sl = (p % ROWB) / 16;
    dma_off[i] = (uint32_t)(r * (int)kstride * 2 + ((sl ^ swz<D>(r)) << 4));
  }
#pragma unroll
  for (int i = 0; i < IPWV; ++i) {
    const int p = 1024 * ((w & 3) * IPWV + i) + 16 * lane;
    const int r = p / VROWB, sl = (p % VROWB) / 16;
    dma_voff[i] = (uint32_t)(r * (int)vstride * 2 + ((sl ^ swz<DV>(r)) << 4));
  }
  // one K (V_TILE = false) or V tile into a stage; rows past the sequence land as zeros
  auto dma_tile = [&](EA_LDS uint16_t* stage, const uint16_t* gbase, int t, auto v_tile) __attribute__((always_inline)) {
    constexpr bool V = decltype(v_tile)::value;
    constexpr int DD = V ? DV : D, NP = V ? IPWV : IPW;
    const size_t stride = V ? vstride : kstride;
    const int rows = t < nkb ? min(lk - t * BN, BN) : 0;  // tiles past the causal bound are not fetched
    const uint32_t nrec = rows > 0 ? (uint32_t)((rows - 1) * (int)stride * 2 + DD * 2) : 0u;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(gbase + (size_t)(rows > 0 ? t : 0) * BN * stride, nrec);
#pragma unroll
    for (int i = 0; i < NP; ++i)
      buffer_load16_lds(rs, (EA_LDS void*)(stage + 512 * ((w & 3) * NP + i)), V ? dma_voff[i] : dma_off[i]);
  };
  using KTILE = std::integral_constant<bool, false>;
  using VTILE_ = std::integral_constant<bool, true>;
  // stage r is a constant wherever these are inlined, so every access names
  // one LDS object
  auto kstage = [&](int r) __attribute__((always_inline)) -> EA_LDS uint16_t* {
    return r == 0 ? (EA_LDS uint16_t*)ks0 : r == 1 ? (EA_LDS uint16_t*)ks1 : (EA_LDS uint16_t*)ks2;
  };
  auto vstage = [&](int r) __attribute__((always_inline)) -> EA_LDS uint16_t* {
    return r == 0 ? (EA_LDS uint16_t*)vs0 : r == 1 ? (EA_LDS uint16_t*)vs1 : (EA_LDS uint16_t*)vs2;
  };

  // loop-invariant LDS element offsets of this lane's operand reads (see the
  // 4-wave kernel): K rows c and c + 32, V^T transposed reads
  int k_off[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) k_off[kk] = tile_off<D>(c, 16 * kk + 8 * hh);
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int v_off[NDT][2];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    v_off[dt][0] = tile_off<DV>(tr_row, 32 * dt + tr_col);
    v_off[dt][1] = tile_off<DV>(tr_row + 8, 32 * dt + tr_col);
  }
  const int wave_last_q = wrow + 31;
  const int wave_first_q = wrow;
  // a tile is fully masked for this wave (wave-uniform) if its first key lies
  // beyond the wave's last row's causal limit
  auto tile_dead = [&](int t) __attribute__((always_inline)) { return CAUSAL && t * BN > wave_last_q + off; };

  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
  f32x16 s0 = f32x16{}, s1 = f32x16{};
  bf16x8 pb[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) pb[st] = bf16x8{};
  const float sl = a.scale_log2;

  // ---- MFMA part of step s: S_s = K_s Q^T, then O += V_{s-1} P_{s-1}, as one
  // straight-line block so the V^T reads overlap the S products. Both run for
  // every step: for a tile this wave skips (past its causal limit, or s = nkb)
  // the VALU part leaves P = 0, stages past the end hold zeros from the DMA,
  // and the V stage read at step 0 is zeroed before the loop, so the extra
  // products add exact zeros.
  auto mfma_part = [&](int r) __attribute__((always_inline)) {
    const EA_LDS uint16_t* ks = kstage(r);
    const EA_LDS uint16_t* vs = vstage((r + 2) % 3);
    // The lane offsets pass through an empty asm here so that the stage base
    // is added inside this block, where it folds into the ds_read offset
    // field, instead of a hoisted register copy per stage and offset.
    int ko[D / 16], vo[NDT][2];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      ko[kk] = launder(k_off[kk]);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      vo[dt][0] = launder(v_off[dt][0]);
      vo[dt][1] = launder(v_off[dt][1]);
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8 ka0 = lds_load<bf16x8>(ks + ko[kk]);
      const bf16x8 ka1 = lds_load<bf16x8>(ks + ko[kk] + 32 * D);
      s0 = mfma32x32x16(ka0, qf[kk], kk == 0 ? f32x16{} : s0);
      s1 = mfma32x32x16(ka1, qf[kk], kk == 0 ? f32x16{} : s1);
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const i16x4 lo = ds_read_tr16(vs + vo[dt][0] + 16 * st * DV);
        const i16x4 hi = ds_read_tr16(vs + vo[dt][1] + 16 * st * DV);
        const i32x4 t = {__builtin_bit_cast(i32x2, lo)[0], __builtin_bit_cast(i32x2, lo)[1],
                         __builtin_bit_cast(i32x2, hi)[0], __builtin_bit_cast(i32x2, hi)[1]};
        oacc[dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, t), pb[st], oacc[dt]);
      }
    }
    // operand reads stay about five ahead of the MFMA that consumes them:
    // 6 primed, one per S product (the last six already fetch V^T), two per
    // PV product, the final three products after the last read
    constexpr int NS = D / 8, NPV = 4 * NDT;
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < NPV - 3; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- VALU part of step s: softmax of S_s into P_s (bf16, computed in place
  // over S), m, l, rescale
  auto valu_part = [&](int s, bool act) __attribute__((always_inline)) {
    if (!act) {
#pragma unroll
      for (int st = 0; st < 4; ++st) pb[st] = bf16x8{};
      return;
    }
    const int kbase = s * BN;
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
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = pp_exp2<EXPMODE>(__builtin_fmaf(s0[i], sl, neg_m), i);
      s1[i] = pp_exp2<EXPMODE>(__builtin_fmaf(s1[i], sl, neg_m), i);
    }
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ls0 += s0[i];
      ls1 += s1[i];
    }
    l_run += ls0 + ls1;
    pb[0] = pack_p8<0>(s0);
    pb[1] = pack_p8<8>(s0);
    pb[2] = pack_p8<0>(s1);
    pb[3] = pack_p8<8>(s1);
  };

  // ---- one step: MFMA part, barrier, VALU part, barrier. Group B starts one
  // barrier late, so in phase 2s group A runs the MFMA part of step s while B
  // runs the VALU part of step s - 1, and in phase 2s + 1 A runs the VALU
  // part of s while B runs the MFMA part of s. Group A alone issues the DMA,
  // at the start of its VALU part (phase 2s + 1, off the MFMA issue path):
  // K_{s+2} and V_{s+1}, whose stages were last read in phase 2s - 1. It
  // waits for them at the end of phase 2s + 3 -- leaving the next step's
  // pieces in flight -- before the barrier after which both groups read them.
  auto step = [&](int r, int s) __attribute__((always_inline)) {
    const bool act = s < nkb && !tile_dead(s);
    mfma_part(r);
    pp_barrier();
    if (grp == 0) {
      dma_tile(kstage((r + 2) % 3), kg_base, s + 2, KTILE{});
      dma_tile(vstage((r + 1) % 3), vg_base, s + 1, VTILE_{});
    }
    valu_part(s, act);
    if (grp == 0) wait_vmcnt<IPW + IPWV>();
    pp_barrier();
  };

  // prologue: K_0, K_1 and V_0 (read in steps 0 and 1); the V stage that
  // step 0 multiplies by P = 0 is zeroed so it holds no stale NaN
  {
    static_assert(VTILE % (8 * 512) == 0, "stage zeroing covers the tile");
#pragma unroll
    for (int i = 0; i < VTILE / (8 * 512); ++i)
      lds_store<i32x4>((EA_LDS uint16_t*)vs2 + 8 * (tid + 512 * i), i32x4{});
  }
  if (grp == 0) {
    dma_tile(kstage(0), kg_base, 0, KTILE{});
    dma_tile(kstage(1), kg_base, 1, KTILE{});
    dma_tile(vstage(0), vg_base, 0, VTILE_{});
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

  // ---------------- epilogue: O = acc / l (bf16), lse = ln2 * (m + log2 l)
  const float l_tot = sum_with_partner32(l_run);
  const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
  if (qi < lq) {
    uint16_t* op = a.o + (size_t)(q0 + qi) * ostride + (size_t)h * DV;
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

template <int D, int DV, bool CAUSAL, bool VARLEN, int EXPMODE>
__global__ __launch_bounds__(512, 1) void fwd_pp_kernel(FwdArgs a) {
  pp_tile<D, DV, CAUSAL, VARLEN, EXPMODE>(a, blockIdx.x & 7, blockIdx.x >> 3);
}

// Persistent form: one workgroup per CU walks its XCD's tile list. Launching a
// new workgroup on a CU that just retired one takes ~11 us on this GPU (about
// 8% of a prefill forward that runs eight workgroups per CU); a persistent
// workgroup goes straight to its next tile. The hardware's dynamic dispatch
// balanced the heaviest-first list by itself; a static assignment must keep
// that balance, so workgroup i of an XCD with W workgroups takes, in round r,
// list entry r W + i for even r and r W + W - 1 - i for odd r (snake order):
// the heaviest row block of one (sequence, head) pairs with the lightest of
// the next.
template <int D, int DV, bool CAUSAL, bool VARLEN, int EXPMODE>
__global__ __launch_bounds__(512, 1) void fwd_pp_persistent_kernel(FwdArgs a) {
  const int xcd = blockIdx.x & 7, i = blockIdx.x >> 3, W = gridDim.x >> 3;
  const int per_xcd = uniform(a.tiles_per_xcd);
  for (int r = 0; r * W < per_xcd; ++r) {
    const int jj = r * W + ((r & 1) ? W - 1 - i : i);
    if (jj < per_xcd) pp_tile<D, DV, CAUSAL, VARLEN, EXPMODE>(a, xcd, jj);
  }
}

template <int D, int DV, bool CAUSAL, bool VARLEN, int EXPMODE>
static hipError_t launch_pp_t(const FwdArgs& a, hipStream_t s) {
  const int grid = fwd_grid(a, VARLEN);
  if (a.persist_wgs > 0) {
    FwdArgs b = a;
    b.tiles_per_xcd = grid / 8;
    const int w = min(a.persist_wgs / 8, b.tiles_per_xcd);  // workgroups per XCD
    hipLaunchKernelGGL((fwd_pp_persistent_kernel<D, DV, CAUSAL, VARLEN, EXPMODE>), dim3(8 * max(w, 1)), dim3(512), 0,
                       s, b);
  } else {
    hipLaunchKernelGGL((fwd_pp_kernel<D, DV, CAUSAL, VARLEN, EXPMODE>), dim3(grid), dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

template <int D, int DV, bool CAUSAL, bool VARLEN>
static hipError_t launch_pp_e(const FwdArgs& a, int exp_mode, hipStream_t s) {
  switch (exp_mode) {
    case 1: return launch_pp_t<D, DV, CAUSAL, VARLEN, 1>(a, s);
    case 2: return launch_pp_t<D, DV, CAUSAL, VARLEN, 2>(a, s);
    default: return launch_pp_t<D, DV, CAUSAL, VARLEN, 0>(a, s);
  }
}

template <int D, int DV>
static hipError_t launch_pp_d(const FwdArgs& a, bool causal, bool varlen, int exp_mode, hipStream_t s) {
  if (causal) {
    return varlen ? launch_pp_e<D, DV, true, true>(a, exp_mode, s) : launch_pp_e<D, DV, true, false>(a, exp_mode, s);
  }
  return varlen ? launch_pp_e<D, DV, false, true>(a, exp_mode, s) : launch_pp_e<D, DV, false, false>(a, exp_mode, s);
}

hipError_t launch_fwd_pp(const FwdArgs& a, int d, int dv, bool causal, bool varlen, int exp_mode, hipStream_t s) {
  if (d == 64 && dv == 64) return launch_pp_d<64, 64>(a, causal, varlen, exp_mode, s);
  if (d == 192 && dv == 128) return launch_pp_d<192, 128>(a, causal, varlen, exp_mode, s);
  if (d == 128 && dv == 128) return launch_pp_d<128, 128>(a, causal, varlen, exp_mode, s);
  return hipErrorInvalidValue;
}

}  // namespace ea
