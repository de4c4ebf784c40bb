// Fused exact attention forward for gfx950, 8-wave software-pipelined variant
// (bf16 in, fp32 accumulate).
//
// Method: as in the 4-wave kernel -- each workgroup owns a block of query rows
// of one (sequence, head) and streams over 64-key K/V tiles with the online
// softmax ("FlashAttention: not less compute, less data movement", sections
// 02-03), lazy rescale ("FlashAttention-4: algorithm-pipeline co-design for
// Blackwell", conditional softmax rescaling section) and the XCD-grouped,
// heaviest-first tile order ("FlashAttention4 close reading", section 3.3).
//
// The pages overlap the matrix products with the exponentials by giving them
// to different warps. Here each wave overlaps them itself (this file's own
// design): a gfx950 wave keeps issuing independent vector ALU and LDS
// instructions while its own MFMAs run, so one straight-line block per step
// holds three independent streams --
//   * S_{s+1} = K_{s+1} Q^T        (MFMA, K read from LDS)
//   * O      += V_{s-1} P_{s-1}    (MFMA, V^T read transposed from LDS)
//   * P_s     = softmax part of S_s (vector ALU: max, rescale test, exp2, sums,
//                                    bf16 packing)
// plus this wave's share of the K/V DMA, interleaved MFMA by MFMA. Nothing in
// the block depends on anything else in it, so no stream waits for another.
//  * 8 waves x 32 query rows (256 per workgroup), two waves per SIMD. One
//    workgroup barrier per step retires a stage.
//  * K/V tiles arrive by LDS DMA (buffer_load ... lds, 16 bytes per lane; every
//    lane fetches the global chunk that belongs at its swizzled LDS position)
//    into three stages per operand: step s reads K_{s+1} and V_{s-1} and fetches
//    K_{s+3} and V_{s+1}, which land by the end of step s + 1.
//  * Masking (diagonal and ragged tiles, and tiles entirely past a wave's
//    causal limit) is applied to S_s before the block, under a branch taken
//    on few steps; the O rescale, when the lazy test asks for it, after it.
//  * Stages are distinct LDS objects and the loop is unrolled by three, so the
//    compiler's own wait tracking sees which stage each access uses.
//  * Operand layouts (S^T = K Q^T, P^T passed in registers to O^T = V^T P^T,
//    V^T from ds_read_b64_tr_b16) are those of the 4-wave kernel.
#include "ea_device.h"
#include "ea_fwd_common.h"
#include "ea_internal.h"

namespace ea {

template <int D, bool CAUSAL, bool VARLEN, int EXPMODE>
__global__ __launch_bounds__(512, 1) void fwd_sp_kernel(FwdArgs a) {
  constexpr int BM = kPpBlockM, BN = kFwdBlockN;
  constexpr int TILE = BN * D;  // bf16 elements per stage
  constexpr int NDT = D / 32;   // 32-wide d tiles of O^T
  constexpr int ROWB = D * 2;   // bytes per K/V row
  constexpr int NI = TILE * 2 / 1024;  // 1 KB DMA instructions per tile
  constexpr int IPW = NI / 8;          // ... per wave
  static_assert(IPW >= 1 && NI % 8 == 0, "tile must split into 8 waves of 1 KB DMA");
  __shared__ __attribute__((aligned(1024))) uint16_t ks0[TILE], ks1[TILE], ks2[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vs0[TILE], vs1[TILE], vs2[TILE];

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
  const int lane = tid & 63, w = uniform(tid >> 6), hh = lane >> 5, c = lane & 31;
  const int wrow = row_lo + 32 * w;  // wave's first query row
  const int qi = wrow + c;           // this lane's query row
  const size_t qstride = (size_t)a.Hq * D, kstride = (size_t)a.Hkv * D;

  // ---------------- Q^T operand (B of S^T = K Q^T), kept in VGPRs
  bf16x8 qf[D / 16];
  {
    const uint16_t* qp = a.q + (size_t)(q0 + qi) * qstride + (size_t)h * D + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = (qi < lq) ? *(const bf16x8*)(qp + 16 * kk) : bf16x8{};
  }

  // ---------------- K/V DMA: wave w fills 1 KB pieces w*IPW .. w*IPW+IPW-1 of
  // a tile. Lane s of piece p lands at stage byte 1024 p + 16 s = row r, slot
  // sl; it fetches the global 16-byte chunk sl ^ swz(r) of row r.
  const uint16_t* kg_base = a.k + (size_t)k0 * kstride + (size_t)hk * D;
  const uint16_t* vg_base = a.v + (size_t)k0 * kstride + (size_t)hk * D;
  uint32_t dma_off[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int p = 1024 * (w * IPW + i) + 16 * lane;
    const int r = p / ROWB, sl = (p % ROWB) / 16;
    dma_off[i] = (uint32_t)(r * (int)kstride * 2 + ((sl ^ swz<D>(r)) << 4));
  }
  // Buffer resource of tile t: its rows up to the end of the sequence; a tile
  // at or past nkb (past the causal bound) gets no records, so its DMA writes
  // zeros without touching memory. Only the last tile can be partial; both
  // record counts are fixed here, so a step only selects between scalars.
  const int row_bytes = (int)kstride * 2;
  const uint32_t nrec_full = (uint32_t)uniform((BN - 1) * row_bytes + D * 2);
  const uint32_t nrec_last =
      (uint32_t)uniform(nkb > 0 ? (min(lk - (nkb - 1) * BN, BN) - 1) * row_bytes + D * 2 : 0);
  auto tile_rsrc = [&](const uint16_t* gbase, int t) __attribute__((always_inline)) {
    const uint32_t nrec = t < nkb - 1 ? nrec_full : (t == nkb - 1 ? nrec_last : 0u);
    return make_rsrc(gbase + (size_t)t * (BN * kstride), nrec);
  };
  auto dma_issue = [&](EA_LDS uint16_t* stage, __amdgpu_buffer_rsrc_t rs) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < IPW; ++i)
      buffer_load16_lds(rs, (EA_LDS void*)(stage + 512 * (w * IPW + i)), dma_off[i]);
  };
  auto dma_tile = [&](EA_LDS uint16_t* stage, const uint16_t* gbase, int t) __attribute__((always_inline)) {
    dma_issue(stage, tile_rsrc(gbase, t));
  };
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
  for (int kk = 0; kk < D / 16; ++kk) k_off[kk] = 2 * tile_off<D>(c, 16 * kk + 8 * hh);  // bytes
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int v_off[NDT][2];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    v_off[dt][0] = 2 * tile_off<D>(tr_row, 32 * dt + tr_col);  // bytes
    v_off[dt][1] = 2 * tile_off<D>(tr_row + 8, 32 * dt + tr_col);
  }
  const int wave_first_q = wrow;

  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
  f32x16 sc0, sc1;  // S of the tile whose softmax runs in the current step
  f32x16 sn0 = f32x16{}, sn1 = f32x16{};  // S of the next tile
  bf16x8 pprev[4], pcur[4];  // P of the previous tile (operand of this step's PV), of this one
#pragma unroll
  for (int st = 0; st < 4; ++st) pprev[st] = bf16x8{};
  const float sl = a.scale_log2;
  const float tau = a.tau;

  // ---- mask of S_s: keys past the end, and past a row's causal limit, get
  // -inf (a tile entirely past the wave's limit is masked whole)
  auto need_mask = [&](int s) __attribute__((always_inline)) {
    const int kbase = s * BN;
    bool m = kbase + BN > lk;
    if constexpr (CAUSAL) m = m || (kbase + BN - 1 > wave_first_q + off);
    return m;
  };
  auto apply_mask = [&](int s) __attribute__((always_inline)) {
    int lim = lk;
    if constexpr (CAUSAL) lim = min(lk, qi + off + 1);
    const int rel = lim - s * BN - 4 * hh;  // element i is valid iff its key offset < rel
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int ko = 8 * (i >> 2) + (i & 3);
      sc0[i] = (ko < rel) ? sc0[i] : kNegInf;
      sc1[i] = (ko + 32 < rel) ? sc1[i] : kNegInf;
    }
  };

  // ---- the pipelined block of step s (stage r = s mod 3): NMF slots, each
  // one MFMA (the S_{s+1} products first, then the PV products), the operand
  // reads of the MFMA RA slots later, and a share of the softmax of S_s --
  // row max, then the rescale test, then exp2 and the row sum two or four
  // elements at a time, then the bf16 packing -- and, in the last slots, the
  // DMA. A scheduling fence closes each slot, so the order is this one.
  // Returns whether O must be rescaled by alpha once the block's products
  // are done.
  constexpr int NS = D / 8, NPV = 4 * NDT, NMF = NS + NPV;
  constexpr int RA = 3;                 // operand reads this many MFMAs ahead
  constexpr int MAXS = NMF / 8;         // slots of the row max
  constexpr int EXPS = NMF - MAXS - 3;  // slots of the exponentials
  constexpr int MPS = 32 / MAXS;        // elements per max slot
  constexpr int PACK0 = MAXS + 1 + EXPS;  // first packing slot
  static_assert(PACK0 + 2 <= NMF, "slots for the packing");
  static_assert(32 % MAXS == 0 && MPS % 4 == 0 && EXPS <= 32, "element split");
  // first element of exponential slot k: the 32 elements spread as evenly as
  // the slots allow
  auto exp_first = [](int k) { return (32 * k) / EXPS; };
  float alpha = 1.f;
  auto block = [&](int r, int s, __amdgpu_buffer_rsrc_t rs_k, __amdgpu_buffer_rsrc_t rs_v)
                   __attribute__((always_inline)) -> bool {
    const EA_LDS uint16_t* ks = kstage((r + 1) % 3);
    const EA_LDS uint16_t* vs = vstage((r + 2) % 3);
    // The lane offsets (bytes) pass through an empty asm in place, so to the
    // compiler they change every step: the stage base is added inside this
    // block, where it folds into the ds_read offset field, instead of a
    // hoisted register per stage and offset, and no copy is made per step.
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) k_off[kk] = launder(k_off[kk]);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      v_off[dt][0] = launder(v_off[dt][0]);
      v_off[dt][1] = launder(v_off[dt][1]);
    }
    // operand of MFMA j: j < NS reads K row block (j mod 2) at d slice j / 2;
    // j >= NS reads V^T for P slice st and d tile dt
    bf16x8 opnd[NMF];
    auto read_operand = [&](int j) __attribute__((always_inline)) {
      if (j < NS) {
        opnd[j] = lds_load<bf16x8>((const EA_LDS char*)ks + k_off[j >> 1] + 64 * D * (j & 1));
      } else {
        const int st = (j - NS) / NDT, dt = (j - NS) % NDT;
        const i16x4 lo = ds_read_tr16((const EA_LDS uint16_t*)((const EA_LDS char*)vs + v_off[dt][0] + 32 * st * D));
        const i16x4 hi = ds_read_tr16((const EA_LDS uint16_t*)((const EA_LDS char*)vs + v_off[dt][1] + 32 * st * D));
        const i32x4 t = {__builtin_bit_cast(i32x2, lo)[0], __builtin_bit_cast(i32x2, lo)[1],
                         __builtin_bit_cast(i32x2, hi)[0], __builtin_bit_cast(i32x2, hi)[1]};
        opnd[j] = __builtin_bit_cast(bf16x8, t);
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
    float mx0 = kNegInf, mx1 = kNegInf, neg_m = 0.f;
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
    bool resc = false;

#pragma unroll
    for (int j = 0; j < RA; ++j) read_operand(j);
    sched_fence();
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      if (i + RA < NMF) read_operand(i + RA);
      if (i < NS) {
        const int kk = i >> 1;
        if (i & 1) {
          sn1 = mfma32x32x16(opnd[i], qf[kk], kk == 0 ? f32x16{} : sn1);
        } else {
          sn0 = mfma32x32x16(opnd[i], qf[kk], kk == 0 ? f32x16{} : sn0);
        }
      } else {
        const int st = (i - NS) / NDT, dt = (i - NS) % NDT;
        oacc[dt] = mfma32x32x16(opnd[i], pprev[st], oacc[dt]);
      }
      if (i < MAXS) {
        // row max over this lane's 32 keys, two chains of max3
#pragma unroll
        for (int e = i * MPS; e < i * MPS + MPS; e += 4) {
          mx0 = __builtin_fmaxf(__builtin_fmaxf(mx0, elem(e)), elem(e + 2));
          mx1 = __builtin_fmaxf(__builtin_fmaxf(mx1, elem(e + 1)), elem(e + 3));
        }
      } else if (i == MAXS) {
        // with the partner lane's 32 keys: the row max; the lazy rescale test;
        // rows that have seen no key yet keep m = -inf and get alpha = 0
        const float mx = max_with_partner32(__builtin_fmaxf(mx0, mx1));
        const float m_new = __builtin_fmaxf(m_run, mx * sl);
        resc = __ballot(m_new > m_run + tau) != 0;
        const float a_raw = exp2_hw(m_run - m_new);
        alpha = resc ? ((m_run == kNegInf) ? 0.f : a_raw) : 1.f;
        m_run = resc ? m_new : m_run;
        neg_m = (m_run == kNegInf) ? 0.f : -m_run;
      } else if (i < PACK0) {
        const int e0 = exp_first(i - MAXS - 1), e1 = exp_first(i - MAXS);
#pragma unroll
        for (int e = e0; e < e1; ++e) {
          const float p = pp_exp2<EXPMODE>(__builtin_fmaf(elem(e), sl, neg_m), e & 15);
          set_elem(e, p);
          ls[e & 3] += p;
        }
      } else if (i == PACK0) {
        pcur[0] = pack_p8<0>(sc0);
        pcur[1] = pack_p8<8>(sc0);
      } else if (i == PACK0 + 1) {
        pcur[2] = pack_p8<0>(sc1);
        pcur[3] = pack_p8<8>(sc1);
        l_run = l_run * alpha + ((ls[0] + ls[1]) + (ls[2] + ls[3]));
      }
      // this wave's share of K_{s+3} (into the stage K_s left) and V_{s+1}
      // (into the stage V_{s-2} left)
      if (i == NMF - 2) dma_issue(kstage(r), rs_k);
      if (i == NMF - 1) dma_issue(vstage((r + 1) % 3), rs_v);
      sched_fence();
    }
    // the softmax results must exist inside this block: left alone, the
    // compiler sinks their computation below the rescale branch
#pragma unroll
    for (int st = 0; st < 4; ++st) keep(pcur[st]);
    keep(l_run);
    keep(m_run);
    keep(alpha);
    return resc;
  };

  // ---- one step: mask S_s if needed, the block, the rescale, rotate the
  // pipeline registers, then retire a stage: K_{s+2} and V_s (fetched in step
  // s - 1) must have landed, and every wave must be past its reads of the
  // stages the next step's DMA overwrites
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
#pragma unroll
    for (int st = 0; st < 4; ++st) pprev[st] = pcur[st];
    wait_vmcnt<2 * IPW>();
    pp_barrier();
  };

  // prologue: K_0, K_1, K_2 and V_0; the V stage that step 0 multiplies by
  // P = 0 is zeroed so it holds no stale NaN; S_0 is computed here, and all
  // waves are past their reads of K_0 before step 0 overwrites its stage
  {
    static_assert(TILE % (8 * 512) == 0, "stage zeroing covers the tile");
#pragma unroll
    for (int i = 0; i < TILE / (8 * 512); ++i)
      lds_store<i32x4>((EA_LDS uint16_t*)vs2 + 8 * (tid + 512 * i), i32x4{});
  }
  // (with no tiles there is nothing to fetch; the steps then only see masked
  // scores. Issuing these under a branch also keeps the compiler's wait
  // tracking from placing a full wait at the loop head.)
  if (nkb > 0) {
    dma_tile(kstage(0), kg_base, 0);
    dma_tile(kstage(1), kg_base, 1);
    dma_tile(kstage(2), kg_base, 2);
    dma_tile(vstage(0), vg_base, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const bf16x8 ka0 = lds_load<bf16x8>((const EA_LDS char*)ks0 + k_off[kk]);
    const bf16x8 ka1 = lds_load<bf16x8>((const EA_LDS char*)ks0 + k_off[kk] + 64 * D);
    sc0 = mfma32x32x16(ka0, qf[kk], kk == 0 ? f32x16{} : sc0);
    sc1 = mfma32x32x16(ka1, qf[kk], kk == 0 ? f32x16{} : sc1);
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

template <int D, bool CAUSAL, bool VARLEN, int EXPMODE>
static hipError_t launch_sp_t(const FwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((fwd_sp_kernel<D, CAUSAL, VARLEN, EXPMODE>), dim3(fwd_grid(a, VARLEN)), dim3(512), 0, s, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool VARLEN>
static hipError_t launch_sp_e(const FwdArgs& a, int exp_mode, hipStream_t s) {
  switch (exp_mode) {
    case 1: return launch_sp_t<D, CAUSAL, VARLEN, 1>(a, s);
    case 2: return launch_sp_t<D, CAUSAL, VARLEN, 2>(a, s);
    default: return launch_sp_t<D, CAUSAL, VARLEN, 0>(a, s);
  }
}

template <int D>
static hipError_t launch_sp_d(const FwdArgs& a, bool causal, bool varlen, int exp_mode, hipStream_t s) {
  if (causal) {
    return varlen ? launch_sp_e<D, true, true>(a, exp_mode, s) : launch_sp_e<D, true, false>(a, exp_mode, s);
  }
  return varlen ? launch_sp_e<D, false, true>(a, exp_mode, s) : launch_sp_e<D, false, false>(a, exp_mode, s);
}

hipError_t launch_fwd_sp(const FwdArgs& a, int d, bool causal, bool varlen, int exp_mode, hipStream_t s) {
  if (d == 64) return launch_sp_d<64>(a, causal, varlen, exp_mode, s);
  return launch_sp_d<128>(a, causal, varlen, exp_mode, s);
}

}  // namespace ea
