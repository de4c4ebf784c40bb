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

// One work tile: 256 query rows of one (sequence, head), located in the
// XCD-grouped, heaviest-first order.
struct PpTile {
  int seq, h, row_lo, q0, lq, k0, lk, hk, nkb;
};

// Tile j of XCD xcd; false when that entry holds no rows (padding of the grid
// to whole XCDs, or past the packed sequences).
template <bool CAUSAL, bool VARLEN>
__device__ __forceinline__ bool pp_locate(const FwdArgs& a, int xcd, int j, PpTile& t) {
  constexpr int BM = kPpBlockM, BN = kFwdBlockN;
  // scalar from here on: the branches below are then uniform, and the fields
  // they produce stay in scalar registers
  xcd = uniform(xcd);
  j = uniform(j);
  int seq, h, mb;
  const int ngroups = a.nseq * a.Hq;
  if constexpr (!VARLEN) {
    const int kg = j / a.n_mb;
    const int r = j - kg * a.n_mb;
    const int g = xcd + 8 * kg;
    if (g >= ngroups) return false;
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
    if (g >= ngroups) return false;
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
  t.seq = uniform(seq);
  t.h = uniform(h);
  t.row_lo = uniform(mb) * BM;
  t.q0 = uniform(q0);
  t.lq = uniform(lq);
  t.k0 = uniform(k0);
  t.lk = uniform(lk);
  t.hk = uniform(t.h / a.group);
  int nkeys = t.lk;
  if constexpr (CAUSAL) nkeys = min(t.lk, t.row_lo + BM + (t.lk - t.lq));  // bottom-right causal alignment
  if (nkeys < 0) nkeys = 0;
  t.nkb = uniform((nkeys + BN - 1) / BN);
  return true;
}

// The per-wave state of the ping-pong forward and its two phase bodies,
// shared by the one-tile kernel and the persistent walk.
// D: head dim of Q and K; DV: head dim of V and O (equal, or 192 / 128).
// STATS: count this wave's steps with live keys and its lazy-rescale
// decisions (the test-only statistics launch).
template <int D, int DV, bool CAUSAL, int EXPMODE, bool STATS = false>
struct PpCore {
  static constexpr int BN = kFwdBlockN;
  static constexpr int NDT = DV / 32;  // 32-wide d tiles of O^T

  int lane, hh, c, w, grp;
  // LDS byte offsets of this lane's operand reads (see the 4-wave kernel):
  // K rows c and c + 32, V^T transposed reads
  int k_off[D / 16];
  int v_off[NDT][2];
  bf16x8 qf[D / 16];  // Q^T operand (B of S^T = K Q^T)
  f32x16 oacc[NDT];
  f32x16 s0, s1;
  bf16x8 pb[4];
  float m_run, l_run;
  // -m (0 while the row has no max) and the lazy-rescale test's bound on the
  // sum of a step's P: 2^tau, or -1 while the row has no max (the test then
  // fails); both change only when m does
  float neg_m_run, thr_run;
  float thr_tau = 1.f;  // 2^tau
  int n_live = 0, n_rescale = 0;  // STATS only

  __device__ __forceinline__ void init() {
    const int tid = threadIdx.x;
    lane = tid & 63;
    w = uniform(tid >> 6);
    hh = lane >> 5;
    c = lane & 31;
    grp = w >> 2;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) k_off[kk] = 2 * tile_off<D>(c, 16 * kk + 8 * hh);
    const int tr_row = 4 * hh + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      v_off[dt][0] = 2 * tile_off<DV>(tr_row, 32 * dt + tr_col);
      v_off[dt][1] = 2 * tile_off<DV>(tr_row + 8, 32 * dt + tr_col);
    }
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int st = 0; st < 4; ++st) pb[st] = bf16x8{};
    reset();
  }
  __device__ __forceinline__ void reset() {
    m_run = kNegInf;
    l_run = 0.f;
    neg_m_run = 0.f;
    thr_run = -1.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
  }
  __device__ __forceinline__ void set_tau(float tau) { thr_tau = __builtin_amdgcn_exp2f(tau); }

  // first query row of this wave in a tile starting at row_lo
  __device__ __forceinline__ int wave_row(int row_lo) const { return row_lo + 64 * (w & 3) + 32 * grp; }

  // Q^T rows of this lane from global memory (zeros past the sequence end)
  __device__ __forceinline__ void load_q(const FwdArgs& a, const PpTile& t) {
    const int qi = wave_row(t.row_lo) + c;
    const uint16_t* qp = a.q + (size_t)(t.q0 + qi) * ((size_t)a.Hq * D) + (size_t)t.h * D + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = (qi < t.lq) ? *(const bf16x8*)(qp + 16 * kk) : bf16x8{};
  }

  // ---- MFMA part of a step: S = K_s Q^T into s0, s1, then O += V_{s-1} P_{s-1}
  // (pb), as one straight-line block so the V^T reads overlap the S products.
  // Both run for every step: for a tile this wave skips (past its causal
  // limit, or the pipeline tail) the VALU part leaves P = 0, stages past the
  // end hold zeros from the DMA, and the V stage read at the first step is
  // zeroed, so the extra products add exact zeros.
  __device__ __forceinline__ void mfma_part(const EA_LDS uint16_t* ks, const EA_LDS uint16_t* vs) {
    // The lane offsets pass through an empty asm in place, so to the compiler
    // they change every step: the stage base is then added here, where it
    // folds into the ds_read offset field, instead of a hoisted register per
    // stage and offset, and no copy or shift is made per step.
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) k_off[kk] = launder(k_off[kk]);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      v_off[dt][0] = launder(v_off[dt][0]);
      v_off[dt][1] = launder(v_off[dt][1]);
    }
    const EA_LDS char* kb = (const EA_LDS char*)ks;
    const EA_LDS char* vb = (const EA_LDS char*)vs;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8 ka0 = lds_load<bf16x8>(kb + k_off[kk]);
      const bf16x8 ka1 = lds_load<bf16x8>(kb + k_off[kk] + 64 * D);
      s0 = mfma32x32x16(ka0, qf[kk], kk == 0 ? f32x16{} : s0);
      s1 = mfma32x32x16(ka1, qf[kk], kk == 0 ? f32x16{} : s1);
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const i16x4 lo = ds_read_tr16((const EA_LDS uint16_t*)(vb + v_off[dt][0] + 32 * st * DV));
        const i16x4 hi = ds_read_tr16((const EA_LDS uint16_t*)(vb + v_off[dt][1] + 32 * st * DV));
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
  }

  // ---- VALU part of step s of a tile: softmax of S_s into P_s (bf16, in
  // pb), m, l, rescale. act: the tile holds keys this
  // wave sees. qi: this lane's query row; wave_first_q: the wave's first row;
  // lk: keys of the sequence; off = lk - lq (bottom-right causal alignment).
  // NDMA > 0: dma(i) for i < NDMA issues the wave's DMA pieces; they are
  // spread over the exponentials of the first P (piece i after quarter i mod
  // 4), so the CU's address unit takes them one at a time instead of the
  // wave stalling behind a burst.
  template <int NDMA = 0, typename F = int>
  __device__ __forceinline__ void valu_part(int s, bool act, int qi, int wave_first_q, int lk, int off, float sl,
                                            float tau, const F& dma = 0) {
    if (!act) {
      if constexpr (NDMA > 0) {
#pragma unroll
        for (int i = 0; i < NDMA; ++i) dma(i);
      }
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
    // Lazy rescale (threshold tau, log2) decided without the row max in the
    // common case: P is first formed against the running max m. If every
    // lane's sum of its 32 new P values is at most 2^tau, no P exceeds 2^tau,
    // so no row max exceeds m + tau and the rule keeps m: the P already
    // formed are the ones it forms. Otherwise (and while a row has no max
    // yet) the row max is taken from S, still intact, and the rule applied as
    // written, forming P again if m moved.
    if constexpr (STATS) ++n_live;
    float lsum = form_p<NDMA>(neg_m_run, sl, dma);
    if (__ballot(!(lsum <= thr_run))) {
      float mx = kNegInf;
#pragma unroll
      // max(max(acc, a), b) per pair of scores folds into one three-input max
      for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(__builtin_fmaxf(mx, s0[i]), s1[i]);
      mx = max_with_partner32(mx);
      const float m_new = __builtin_fmaxf(m_run, mx * sl);
      if (__ballot(m_new > m_run + tau)) {
        if constexpr (STATS) ++n_rescale;
        const float alpha = (m_run == kNegInf) ? 0.f : exp2_hw(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
        m_run = m_new;
        neg_m_run = (m_run == kNegInf) ? 0.f : -m_run;
        thr_run = (m_run == kNegInf) ? -1.f : thr_tau;
        lsum = form_p<0>(neg_m_run, sl, 0);
      }
    }
    // the row sum in fp32, before the bf16 rounding of P
    l_run += lsum;
  }

  // P = 2^(S sl + neg_m) over this lane's 32 scores (S is left intact): P^T
  // as bf16 MFMA operands in pb (keys 0..15 of s0, 16..31, then s1), and the
  // fp32 sum of the 32 values (four partial sums, so the adds do not form one
  // dependent chain). NDMA > 0: DMA pieces issued between the quarters.
  template <int NDMA, typename F>
  __device__ __forceinline__ float form_p(float neg_m, float sl, const F& dma) {
    float ls4[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if constexpr (NDMA > 0) {
#pragma unroll
        for (int i = st; i < NDMA; i += 4) dma(i);
      }
      const f32x16& sv = st < 2 ? s0 : s1;
      const int i0 = 8 * (st & 1);
      float p[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        p[k] = pp_exp2<EXPMODE>(__builtin_fmaf(sv[i0 + k], sl, neg_m), i0 + k);
        ls4[k & 3] = (st == 0 && k < 4) ? p[k] : ls4[k & 3] + p[k];
      }
      const i32x4 t = {(int)pack_bf16x2(p[0], p[1]), (int)pack_bf16x2(p[2], p[3]), (int)pack_bf16x2(p[4], p[5]),
                       (int)pack_bf16x2(p[6], p[7])};
      pb[st] = __builtin_bit_cast(bf16x8, t);
    }
    if constexpr (NDMA > 0) {
      // each quarter's DMA pieces, then about a quarter of the vector work
      __builtin_amdgcn_sched_group_barrier(0x010, (NDMA + 3) / 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 28, 0);
      __builtin_amdgcn_sched_group_barrier(0x010, (NDMA + 2) / 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 28, 0);
      __builtin_amdgcn_sched_group_barrier(0x010, (NDMA + 1) / 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 28, 0);
      __builtin_amdgcn_sched_group_barrier(0x010, NDMA / 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 28, 0);
    }
    return (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]);
  }

  // ---- end of a tile: O = acc / l (bf16), lse = ln2 * (m + log2 l)
  template <bool VARLEN>
  __device__ __forceinline__ void store(const FwdArgs& a, int seq, int h, int row_lo, int q0, int lq) {
    const float l_tot = sum_with_partner32(l_run);
    const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
    const int qi = wave_row(row_lo) + c;
    uint4 pk[NDT][2];  // 16-byte row pieces (every lane takes part)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) pack_rows16(oacc[dt], inv, pk[dt]);
    if (qi < lq) {
      uint16_t* op = a.o + (size_t)(q0 + qi) * ((size_t)a.Hq * DV) + (size_t)h * DV;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // streaming stores: O does not displace the K/V lines other
          // workgroups of the XCD are about to read from L2
          const uint4 u = pk[dt][j];
          const i32x4 v4 = {(int)u.x, (int)u.y, (int)u.z, (int)u.w};
          __builtin_nontemporal_store(v4, (i32x4*)(op + 32 * dt + 16 * j + 8 * hh));
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
};

// Per-lane global byte offsets of LDS DMA: wave slot ws (0..3) fills 1 KB
// pieces ws*NP .. ws*NP+NP-1 of a tile of rows of DD bf16. Lane s of piece p
// lands at tile byte 1024 p + 16 s = row r, slot sl; it fetches the global
// 16-byte chunk sl ^ swz(r) of row r (rows `stride` elements apart).
template <int DD>
__device__ __forceinline__ uint32_t dma_lane_off(int piece, int lane, size_t stride) {
  constexpr int ROWB = DD * 2;
  const int p = 1024 * piece + 16 * lane;
  const int r = p / ROWB, sl = (p % ROWB) / 16;
  return (uint32_t)(r * (int)stride * 2 + ((sl ^ swz<DD>(r)) << 4));
}

// One work tile: the whole forward of its 256 rows. STATS 1: also write, per
// wave, the number of steps with live keys, of lazy rescales, and the shader
// clock cycles (s_memtime) and constant-rate wall clock ticks (s_memrealtime)
// its step loop took, to a.stats[4 (8 (8 j + xcd) + wave) + {0, 1, 2, 3}]
// (plain vector stores). STATS 2: add, per wave, the shader cycles of each
// phase of the tile to a.cycles[8 (8 blockIdx + wave) + {0..7}]: the MFMA
// parts, the waits at the barriers after them, the VALU parts (with the DMA
// issue of group A), the waits at the barriers after those, the prologue
// (tile start to the first step), the epilogue (last step to the issued
// stores), the steps and the tiles (each read with an immediate wait, so the
// launch runs a few per cent slower than the plain one).
template <int D, int DV, bool CAUSAL, bool VARLEN, int EXPMODE, int STATS = 0>
__device__ __forceinline__ void pp_tile(const FwdArgs& a, const int xcd, int j) {
  constexpr int BN = kFwdBlockN;
  constexpr int TILE = BN * D;               // bf16 elements per K stage
  constexpr int VTILE = BN * DV;             // ... per V stage
  constexpr int NI = TILE * 2 / 1024;        // 1 KB DMA instructions per K tile
  constexpr int IPW = NI / 4;                // ... per wave of group A
  constexpr int NIV = VTILE * 2 / 1024;      // ... per V tile
  constexpr int IPWV = NIV / 4;
  static_assert(IPW >= 1 && NI % 4 == 0 && IPWV >= 1 && NIV % 4 == 0,
                "tiles must split into 4 waves of 1 KB DMA");
  __shared__ __attribute__((aligned(1024))) uint16_t ks0[TILE], ks1[TILE], ks2[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vs0[VTILE], vs1[VTILE], vs2[VTILE];

  // packed sequences without a caller's order: the heaviest-first order,
  // computed by the workgroup itself into LDS (lpt_order_lds; wave-uniform
  // condition, every thread takes part)
  __shared__ int lpt_w[VARLEN ? kLptLds : 1], lpt_o[VARLEN ? kLptLds : 1];
  FwdArgs al = a;
  if constexpr (VARLEN) {
    if (a.lpt_auto) {
      lpt_order_lds(a.cu_q, a.cu_k, a.nseq, CAUSAL ? 1 : 0, kPpBlockM, BN, (EA_LDS int*)lpt_w, (EA_LDS int*)lpt_o);
      al.seq_order = lpt_o;
    }
  }
  // STATS 2: shader clock now (low 32 bits: a tile's phases take fewer than
  // 2^32 cycles), read with an immediate wait
  auto stamp = [&]() __attribute__((always_inline)) -> uint32_t {
    sched_fence();
    const uint32_t c = (uint32_t)__builtin_amdgcn_s_memtime();
    wait_lgkm0();
    sched_fence();
    return c;
  };
  uint32_t ph[6] = {0, 0, 0, 0, 0, 0};
  uint32_t t_entry = 0;
  if constexpr (STATS == 2) t_entry = stamp();
  PpTile t;
  if (!pp_locate<CAUSAL, VARLEN>(al, xcd, j, t)) return;
  const int off = t.lk - t.lq;  // bottom-right causal alignment
  const int nkb = t.nkb;

  PpCore<D, DV, CAUSAL, EXPMODE, STATS == 1> cr;
  cr.init();
  cr.set_tau(a.tau);
  const int tid = threadIdx.x;
  const int lane = cr.lane, w = cr.w, grp = cr.grp;
  const int wrow = cr.wave_row(t.row_lo);  // wave's first query row
  const int qi = wrow + cr.c;              // this lane's query row
  const size_t kstride = (size_t)a.Hkv * D, vstride = (size_t)a.Hkv * DV;
  cr.load_q(a, t);

  // ---------------- K/V DMA: wave w of the group that fetches an operand
  // (K: group A, V: group B) fills 1 KB pieces (w mod 4) NP .. (w mod 4) NP +
  // NP - 1 of its tile (NP = IPW for K, IPWV for V)
  const uint16_t* kg_base = a.k + (size_t)t.k0 * kstride + (size_t)t.hk * D;
  const uint16_t* vg_base = a.v + (size_t)t.k0 * vstride + (size_t)t.hk * DV;
  uint32_t dma_off[IPW], dma_voff[IPWV];
#pragma unroll
  for (int i = 0; i < IPW; ++i) dma_off[i] = dma_lane_off<D>((w & 3) * IPW + i, lane, kstride);
#pragma unroll
  for (int i = 0; i < IPWV; ++i) dma_voff[i] = dma_lane_off<DV>((w & 3) * IPWV + i, lane, vstride);
  // one K (V_TILE = false) or V tile into a stage; rows past the sequence land as zeros
  auto dma_tile = [&](EA_LDS uint16_t* stage, const uint16_t* gbase, int tt, auto v_tile) __attribute__((always_inline)) {
    constexpr bool V = decltype(v_tile)::value;
    constexpr int DD = V ? DV : D, NP = V ? IPWV : IPW;
    const size_t stride = V ? vstride : kstride;
    const int rows = tt < nkb ? min(t.lk - tt * BN, BN) : 0;  // tiles past the causal bound are not fetched
    const uint32_t nrec = rows > 0 ? (uint32_t)((rows - 1) * (int)stride * 2 + DD * 2) : 0u;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(gbase + (size_t)(rows > 0 ? tt : 0) * BN * stride, nrec);
#pragma unroll
    for (int i = 0; i < NP; ++i)
      buffer_load16_lds(rs, (EA_LDS void*)(stage + 512 * ((w & 3) * NP + i)), V ? dma_voff[i] : dma_off[i]);
  };
  // The DMA inside the step loop with little scalar work in front of the
  // softmax it runs in: the tile's address advances by one tile per step
  // from a running pointer, and its record count is that of a whole tile, of
  // the last fetched tile (nkb - 1), or 0 past it. A tile at or past nkb gets
  // no records, so nothing is read from wherever its address points.
  const int rows_last = nkb > 0 ? min(t.lk - (nkb - 1) * BN, BN) : 0;
  const uint32_t nrk_full = uniform((BN - 1) * (int)kstride * 2 + D * 2);
  const uint32_t nrk_last = uniform(rows_last > 0 ? (rows_last - 1) * (int)kstride * 2 + D * 2 : 0);
  // next tiles the loop fetches: K_2 by group A and V_2 by group B (the
  // prologue fetches K_0, K_1, V_0, V_1)
  const uint16_t* kdma = uniform_ptr(kg_base + (size_t)2 * BN * kstride);
  const uint16_t* vdma = uniform_ptr(vg_base + (size_t)2 * BN * vstride);
  // The DMA of step s as pieces for the VALU part to issue between its
  // exponentials: group A's K_{s+2} into kst (IPW pieces per wave), group B's
  // V_{s+2} into vst (IPWV pieces per wave).
  auto dma_k_pieces = [&](EA_LDS uint16_t* kst, int s) __attribute__((always_inline)) {
    const int tk = s + 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kdma, tk < nkb - 1 ? nrk_full : (tk == nkb - 1 ? nrk_last : 0u));
    kdma += (size_t)BN * kstride;
    EA_LDS uint16_t* kd = kst + 512 * ((w & 3) * IPW);
    return [=](int i) __attribute__((always_inline)) { buffer_load16_lds(rk, (EA_LDS void*)(kd + 512 * i), dma_off[i]); };
  };
  auto dma_v_pieces = [&](EA_LDS uint16_t* vst, int s) __attribute__((always_inline)) {
    uint32_t vfull = nrk_full, vlast = nrk_last;
    if constexpr (DV != D) {  // V rows differ from K rows only for (192, 128)
      vfull = uniform((BN - 1) * (int)vstride * 2 + DV * 2);
      vlast = uniform(rows_last > 0 ? (rows_last - 1) * (int)vstride * 2 + DV * 2 : 0);
    }
    const int tv = s + 2;
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vdma, tv < nkb - 1 ? vfull : (tv == nkb - 1 ? vlast : 0u));
    vdma += (size_t)BN * vstride;
    EA_LDS uint16_t* vd = vst + 512 * ((w & 3) * IPWV);
    return [=](int i) __attribute__((always_inline)) { buffer_load16_lds(rv, (EA_LDS void*)(vd + 512 * i), dma_voff[i]); };
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
  const int wave_last_q = wrow + 31;
  // a tile is fully masked for this wave (wave-uniform) if its first key lies
  // beyond the wave's last row's causal limit
  auto tile_dead = [&](int s) __attribute__((always_inline)) { return CAUSAL && s * BN > wave_last_q + off; };
  const float sl = a.scale_log2;

  // ---- one step: MFMA part, barrier, VALU part, barrier. Group B starts one
  // barrier late, so in phase 2s group A runs the MFMA part of step s while B
  // runs the VALU part of step s - 1, and in phase 2s + 1 A runs the VALU
  // part of s while B runs the MFMA part of s. Each group issues half of the
  // DMA in its VALU part (off the MFMA issue path), spread over the
  // exponentials, so the data lands in both groups' MFMA parts alike:
  //  * group A, phase 2s + 1: K_{s+2}, into the stage K_{s-1} left (last read
  //    in phase 2s - 1); it waits for it at the end of phase 2s + 3, leaving
  //    the next step's pieces in flight;
  //  * group B, phase 2s + 2: V_{s+2}, into the stage V_{s-1} left (last read
  //    in phase 2s + 1); it waits for it at the end of its MFMA part of step
  //    s + 2 (phase 2s + 5), leaving V_{s+3} in flight.
  // Either wait comes before the barrier after which the other group first
  // reads the tile (K_{s+2} in phase 2s + 4, V_{s+2} in phase 2s + 6).
  auto step = [&](int r, int s, auto issuer) __attribute__((always_inline)) {
    constexpr bool A = decltype(issuer)::value;  // group A (fetches K; group B fetches V)
    const bool act = s < nkb && !tile_dead(s);
    uint32_t c0 = 0, c1 = 0, c2 = 0, c3 = 0;
    if constexpr (STATS == 2) c0 = stamp();
    cr.mfma_part(kstage(r), vstage((r + 2) % 3));
    // group B: V_s (issued two steps earlier) has landed before the barrier
    // after which group A reads it; V_{s+1} may stay in flight
    if constexpr (!A) wait_vmcnt<IPWV>();
    if constexpr (STATS == 2) c1 = stamp();
    pp_barrier();
    if constexpr (STATS == 2) c2 = stamp();
    if constexpr (A) {
      cr.template valu_part<IPW>(s, act, qi, wrow, t.lk, off, sl, a.tau, dma_k_pieces(kstage((r + 2) % 3), s));
    } else {
      cr.template valu_part<IPWV>(s, act, qi, wrow, t.lk, off, sl, a.tau, dma_v_pieces(vstage((r + 2) % 3), s));
    }
    if constexpr (STATS == 2) c3 = stamp();
    if constexpr (A) wait_vmcnt<IPW>();
    pp_barrier();
    if constexpr (STATS == 2) {
      const uint32_t c4 = stamp();
      // the sums live in vector registers (launder): the scalar file is full
      ph[0] = (uint32_t)launder((int)(ph[0] + (c1 - c0)));
      ph[1] = (uint32_t)launder((int)(ph[1] + (c2 - c1)));
      ph[2] = (uint32_t)launder((int)(ph[2] + (c3 - c2)));
      ph[3] = (uint32_t)launder((int)(ph[3] + (c4 - c3)));
    }
  };

  // prologue: K_0, K_1 by group A, V_0, V_1 by group B (read in steps 0 to
  // 2); the V stage that step 0 multiplies by P = 0 is zeroed so it holds no
  // stale NaN
  {
    static_assert(VTILE % (8 * 512) == 0, "stage zeroing covers the tile");
#pragma unroll
    for (int i = 0; i < VTILE / (8 * 512); ++i)
      lds_store<i32x4>((EA_LDS uint16_t*)vs2 + 8 * (tid + 512 * i), i32x4{});
  }
  if (grp == 0) {
    dma_tile(kstage(0), kg_base, 0, KTILE{});
    dma_tile(kstage(1), kg_base, 1, KTILE{});
  } else {
    dma_tile(vstage(0), vg_base, 0, VTILE_{});
    dma_tile(vstage(1), vg_base, 1, VTILE_{});
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (STATS == 2) ph[4] = stamp() - t_entry;

  unsigned long long cyc0 = 0, rt0 = 0;
  if constexpr (STATS == 1) {
    cyc0 = __builtin_amdgcn_s_memtime();
    rt0 = __builtin_amdgcn_s_memrealtime();
  }
  // each group runs its own copy of the step loop (only group A's issues the
  // DMA), so no branch on the group sits inside a step
  auto loop = [&](auto issuer) __attribute__((always_inline)) {
    for (int s = 0; s <= nkb; s += 3) {
      step(0, s, issuer);
      if (s + 1 <= nkb) step(1, s + 1, issuer);
      if (s + 2 <= nkb) step(2, s + 2, issuer);
    }
  };
  if (grp == 0) {
    loop(std::integral_constant<bool, true>{});
    pp_barrier();
  } else {
    pp_barrier();  // group B runs one phase behind
    loop(std::integral_constant<bool, false>{});
  }
  // no DMA may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(0);
  uint32_t t_loop_end = 0;
  if constexpr (STATS == 2) t_loop_end = stamp();
  if constexpr (STATS == 1) {
    const unsigned long long cyc1 = __builtin_amdgcn_s_memtime();
    const unsigned long long rt1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) {
      int* st = a.stats + 4 * (8 * (8 * j + xcd) + w);
      st[0] = cr.n_live;
      st[1] = cr.n_rescale;
      st[2] = (int)(cyc1 - cyc0);
      st[3] = (int)(rt1 - rt0);
    }
  }
  cr.template store<VARLEN>(a, t.seq, t.h, t.row_lo, t.q0, t.lq);
  if constexpr (STATS == 2) {
    ph[5] = stamp() - t_loop_end;
    if (lane == 0) {
      // this wave's slots: only it adds to them, one tile after the other
      unsigned long long* cyc = a.cycles + 8 * (8 * blockIdx.x + w);
#pragma unroll
      for (int i = 0; i < 6; ++i) cyc[i] += (unsigned long long)ph[i];
      cyc[6] += (unsigned long long)(nkb + 1);
      cyc[7] += 1;
    }
  }
}

// Persistent walk with the K/V pipeline running on across tiles (the
// unroll-KV schedule of "Low-precision FlashAttention-4: end-to-end
// block-scaled attention for Blackwell", section 2.1.2, in this kernel's
// terms): one workgroup per CU runs one continuous sequence of steps over its
// tiles (persistent_snake's order). Step 0 of tile n+1 computes S_0 of tile
// n+1 in the same MFMA block as the last O += V P of tile n, and its VALU part
// first stores tile n's O and LSE, then starts tile n+1's softmax. The DMA
// issued two steps ahead simply continues into the next tile's K/V tiles, and
// the next tile's Q rows arrive by LDS DMA into a fourth LDS region while the
// current tile runs, so no tile waits on HBM at its start, and the pipeline
// fills and drains once per workgroup instead of once per tile.
//  * Every tile runs at least kMinSteps steps (steps past its keys multiply
//    P = 0 by zero stages, adding exact zeros): the next tile's Q pieces are
//    issued at step 1 and read at the last step, which needs two steps of
//    DMA waits in between.
//  * Results are bitwise those of the one-tile kernel: each row sees the same
//    products in the same order.
//  * Measured on MI355X it is not faster than the one-tile body in a
//    persistent loop: this kernel's tile boundaries already cost little (the
//    other wave group keeps the matrix core busy through them), while the
//    boundary bookkeeping adds scalar instructions to every step's softmax
//    phase, the longer of the two.
template <int D, int DV, bool CAUSAL, bool VARLEN, int EXPMODE>
__device__ __forceinline__ void pp_walk(const FwdArgs& a) {
  static_assert(D == DV, "the next tile's Q is staged in LDS: equal head dims only");
  constexpr int BN = kFwdBlockN;
  constexpr int TILE = BN * D;               // bf16 elements per K or V stage
  constexpr int IPW = TILE * 2 / 1024 / 4;   // 1 KB DMA pieces per wave of group A per tile
  constexpr int QTILE = kPpBlockM * D;       // the next tile's Q rows
  constexpr int NQ = QTILE * 2 / 1024 / 4;   // ... pieces per wave of group A (one 64-row block)
  constexpr int kMinSteps = 4;
  static_assert(NQ * 1024 == TILE * 2, "a wave's Q block is one stage-sized tile");
  static_assert(2 * IPW + NQ < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint16_t ks0[TILE], ks1[TILE], ks2[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vs0[TILE], vs1[TILE], vs2[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t qs[QTILE];

  // ---------------- this workgroup's tiles, in persistent_snake's order
  const int per_xcd = uniform(a.tiles_per_xcd);
  const int xcd = uniform(blockIdx.x & 7), wi = uniform(blockIdx.x >> 3), W = uniform(gridDim.x >> 3);
  int it = 0;
  auto next_tile = [&](PpTile& t) __attribute__((always_inline)) -> bool {
    while (it * W < per_xcd) {
      const int r = it++;
      const int jj = r * W + ((r & 1) ? W - 1 - wi : wi);
      if (jj < per_xcd && pp_locate<CAUSAL, VARLEN>(a, xcd, jj, t)) return true;
    }
    return false;
  };
  PpTile cur, nxt;
  if (!next_tile(cur)) return;
  bool has_nxt = next_tile(nxt);
  int steps = max(cur.nkb, kMinSteps);
  int s = 0;          // step of cur
  bool live = true;   // false: the drain step after the last tile
  bool has_prv = false;
  int p_seq = 0, p_h = 0, p_row_lo = 0, p_q0 = 0, p_lq = 0;  // the tile whose O is in the accumulators

  PpCore<D, D, CAUSAL, EXPMODE> cr;
  cr.init();
  cr.set_tau(a.tau);
  const int tid = threadIdx.x;
  const int lane = cr.lane, w = cr.w, grp = cr.grp;
  const size_t kstride = (size_t)a.Hkv * D, qstride = (size_t)a.Hq * D;
  const float sl = a.scale_log2;
  cr.load_q(a, cur);

  // K and V rows of each tile's KV head; nxt_nkb = 0 when there is no next tile
  auto kv_base = [&](const uint16_t* tensor, const PpTile& t) __attribute__((always_inline)) {
    return tensor + (size_t)t.k0 * kstride + (size_t)t.hk * D;
  };
  const uint16_t* cur_kb = kv_base(a.k, cur);
  const uint16_t* cur_vb = kv_base(a.v, cur);
  const uint16_t* nxt_kb = has_nxt ? kv_base(a.k, nxt) : a.k;
  const uint16_t* nxt_vb = has_nxt ? kv_base(a.v, nxt) : a.v;
  int nxt_nkb = has_nxt ? nxt.nkb : 0;

  uint32_t dma_off[IPW];  // K and V rows have the same stride
#pragma unroll
  for (int i = 0; i < IPW; ++i) dma_off[i] = dma_lane_off<D>((w & 3) * IPW + i, lane, kstride);
  // Source of key tile t of a tile in K or V: base and byte range (0 for
  // tiles at or past nkb, so those stages fill with zeros). kb: the tile's
  // first key row of its KV head in that tensor. Branch-free scalar work,
  // done at the start of a step, where it issues between the MFMAs; the empty
  // asm keeps the compiler from sinking it into the DMA issue after the
  // barrier, whose length the other group waits for.
  struct KvSrc {
    const uint16_t* base;
    uint32_t nrec;
  };
  const size_t tile_elems = (size_t)BN * kstride;
  const uint32_t row_bytes = (uint32_t)(kstride * 2);
  auto kv_src = [&](const uint16_t* kb, int lk, int nkb, int t) __attribute__((always_inline)) {
    const int rows = t < nkb ? min(lk - t * BN, BN) : 0;
    KvSrc r;
    r.nrec = launder_s(rows > 0 ? (uint32_t)(rows - 1) * row_bytes + (uint32_t)(D * 2) : 0u);
    r.base = launder_s(kb + (size_t)(uint32_t)t * tile_elems);
    return r;
  };
  // one K or V tile into a stage. The wave's slot passes through an empty asm
  // at every use, so the LDS destinations are formed here (one scalar add
  // each) rather than hoisted out of the loop as one scalar register per
  // stage and piece.
  auto dma_kv = [&](EA_LDS uint16_t* stage, const KvSrc& src) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src.base, src.nrec);
    EA_LDS uint16_t* dst = stage + 512 * IPW * launder_s(w & 3);
#pragma unroll
    for (int i = 0; i < IPW; ++i) buffer_load16_lds(rs, (EA_LDS void*)(dst + 512 * i), dma_off[i]);
  };
  // the next tile's Q rows: wave w of group A fills 64-row block w of the Q
  // region in the K-stage layout (rows past the sequence land as zeros)
  auto dma_q = [&]() __attribute__((always_inline)) {
    const int rb = nxt.row_lo + 64 * (w & 3);
    const int rows = min(nxt.lq - rb, 64);
    const uint32_t nrec = rows > 0 ? (uint32_t)((rows - 1) * (int)qstride * 2 + D * 2) : 0u;
    const uint16_t* base = a.q + (rows > 0 ? (size_t)(nxt.q0 + rb) * qstride + (size_t)nxt.h * D : (size_t)0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, nrec);
    // per-lane offsets formed here from a laundered lane id, not hoisted out
    // of the loop as NQ live registers
    const int ln = launder(lane);
    EA_LDS uint16_t* dst = (EA_LDS uint16_t*)qs + TILE * launder_s(w & 3);
#pragma unroll
    for (int p = 0; p < NQ; ++p)
      buffer_load16_lds(rs, (EA_LDS void*)(dst + 512 * p), dma_lane_off<D>(p, ln, qstride));
  };
  // this wave's Q^T operand of the next tile, from the Q region
  auto read_q = [&]() __attribute__((always_inline)) {
    const EA_LDS uint16_t* qb = (const EA_LDS uint16_t*)qs + (w & 3) * TILE + 32 * grp * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) cr.qf[kk] = lds_load<bf16x8>((const EA_LDS char*)qb + cr.k_off[kk]);
    wait_lgkm0();  // the region is refilled two steps later
  };
  auto kstage = [&](int r) __attribute__((always_inline)) -> EA_LDS uint16_t* {
    return r == 0 ? (EA_LDS uint16_t*)ks0 : r == 1 ? (EA_LDS uint16_t*)ks1 : (EA_LDS uint16_t*)ks2;
  };
  auto vstage = [&](int r) __attribute__((always_inline)) -> EA_LDS uint16_t* {
    return r == 0 ? (EA_LDS uint16_t*)vs0 : r == 1 ? (EA_LDS uint16_t*)vs1 : (EA_LDS uint16_t*)vs2;
  };

  // ---- one step (global step g, stage r = g mod 3): as in the one-tile
  // kernel, plus the tile boundary work in the VALU part. Group A's DMA at
  // step g fetches what step g + 2 reads: its K tile and the V tile of step
  // g + 1's scores, from cur or, near cur's end, from nxt.
  auto wstep = [&](auto rc) __attribute__((always_inline)) -> bool {
    constexpr int r = decltype(rc)::value;
    KvSrc ksrc, vsrc;
    {
      const bool kin = s + 2 < steps, vin = s + 1 < steps;
      ksrc = kv_src(kin ? cur_kb : nxt_kb, kin ? cur.lk : nxt.lk, kin ? cur.nkb : nxt_nkb, kin ? s + 2 : s + 2 - steps);
      vsrc = kv_src(vin ? cur_vb : nxt_vb, vin ? cur.lk : nxt.lk, vin ? cur.nkb : nxt_nkb, vin ? s + 1 : 0);
    }
    cr.mfma_part(kstage(r), vstage((r + 2) % 3));
    pp_barrier();
    if (!live) {  // drain: the last tile's final O += V P is in
      cr.template store<VARLEN>(a, p_seq, p_h, p_row_lo, p_q0, p_lq);
      pp_barrier();
      return false;
    }
    if (grp == 0) {
      dma_kv(kstage((r + 2) % 3), ksrc);
      dma_kv(vstage((r + 1) % 3), vsrc);
      if (s == 1 && has_nxt) dma_q();
    }
    if (s == 0 && has_prv) {  // tile boundary: the previous tile's final O += V P just ran
      cr.template store<VARLEN>(a, p_seq, p_h, p_row_lo, p_q0, p_lq);
      cr.reset();
    }
    {
      const int wrow = cr.wave_row(cur.row_lo);
      const int off = cur.lk - cur.lq;
      const bool act = s < cur.nkb && !(CAUSAL && s * BN > wrow + 31 + off);
      cr.valu_part(s, act, wrow + cr.c, wrow, cur.lk, off, sl, a.tau);
    }
    if (s == steps - 1 && has_nxt) read_q();
    if (grp == 0) {
      if (s == 1 && has_nxt) {
        wait_vmcnt<2 * IPW + NQ>();  // the Q pieces may stay in flight one more step
      } else {
        wait_vmcnt<2 * IPW>();
      }
    }
    pp_barrier();
    if (++s == steps) {
      s = 0;
      has_prv = true;
      p_seq = cur.seq;
      p_h = cur.h;
      p_row_lo = cur.row_lo;
      p_q0 = cur.q0;
      p_lq = cur.lq;
      if (has_nxt) {
        cur = nxt;
        cur_kb = nxt_kb;
        cur_vb = nxt_vb;
        steps = max(cur.nkb, kMinSteps);
        has_nxt = next_tile(nxt);
        nxt_nkb = has_nxt ? nxt.nkb : 0;
        if (has_nxt) {
          nxt_kb = kv_base(a.k, nxt);
          nxt_vb = kv_base(a.v, nxt);
        }
      } else {
        live = false;
      }
    }
    return true;
  };

  // prologue: K_0, K_1 and V_0 of the first tile; the V stage that the first
  // step multiplies by P = 0 is zeroed so it holds no stale NaN
  {
    static_assert(TILE % (8 * 512) == 0, "stage zeroing covers the tile");
#pragma unroll
    for (int i = 0; i < TILE / (8 * 512); ++i)
      lds_store<i32x4>((EA_LDS uint16_t*)vs2 + 8 * (tid + 512 * i), i32x4{});
  }
  if (grp == 0) {
    dma_kv(kstage(0), kv_src(cur_kb, cur.lk, cur.nkb, 0));
    dma_kv(kstage(1), kv_src(cur_kb, cur.lk, cur.nkb, 1));
    dma_kv(vstage(0), kv_src(cur_vb, cur.lk, cur.nkb, 0));
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  using R0 = std::integral_constant<int, 0>;
  using R1 = std::integral_constant<int, 1>;
  using R2 = std::integral_constant<int, 2>;
  if (grp == 1) pp_barrier();  // group B runs one phase behind
  for (;;) {
    if (!wstep(R0{})) break;
    if (!wstep(R1{})) break;
    if (!wstep(R2{})) break;
  }
  if (grp == 0) pp_barrier();
  // no DMA may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(0);
}

template <int D, int DV, bool CAUSAL, bool VARLEN, int EXPMODE>
__global__ __launch_bounds__(512, 1) void fwd_pp_kernel(FwdArgs a) {
  pp_tile<D, DV, CAUSAL, VARLEN, EXPMODE>(a, blockIdx.x & 7, blockIdx.x >> 3);
}

// Persistent form (persistent_snake in ea_fwd_common.h): one workgroup per
// CU runs the one-tile body for each tile of its list. STATS: the test-only
// statistics launch (per-wave step and rescale counts in a.stats).
template <int D, int DV, bool CAUSAL, bool VARLEN, int EXPMODE, int STATS = 0>
__global__ __launch_bounds__(512, 1) void fwd_pp_persistent_kernel(FwdArgs a) {
  persistent_snake(uniform(a.tiles_per_xcd),
                   [&](int xcd, int j) { pp_tile<D, DV, CAUSAL, VARLEN, EXPMODE, STATS>(a, xcd, j); });
}

// Test-only: the default dense forward (persistent ping-pong, d = 128,
// hardware exp) with per-wave lazy-rescale and clock statistics in a.stats,
// which must hold 32 ints per work tile.
// mode 1: a.stats; mode 2: the per-phase shader cycles in a.cycles (8 per
// wave of each of the launch's workgroups, added to, so zeroed by the caller)
hipError_t launch_fwd_pp_stats(const FwdArgs& a, bool causal, int mode, hipStream_t s) {
  FwdArgs b = a;
  const int grid = fwd_grid(a, false);
  b.tiles_per_xcd = grid / 8;
  const int w = max(min(a.persist_wgs / 8, b.tiles_per_xcd), 1);
  if (mode == 2) {
    if (causal) {
      hipLaunchKernelGGL((fwd_pp_persistent_kernel<128, 128, true, false, 0, 2>), dim3(8 * w), dim3(512), 0, s, b);
    } else {
      hipLaunchKernelGGL((fwd_pp_persistent_kernel<128, 128, false, false, 0, 2>), dim3(8 * w), dim3(512), 0, s, b);
    }
  } else if (causal) {
    hipLaunchKernelGGL((fwd_pp_persistent_kernel<128, 128, true, false, 0, 1>), dim3(8 * w), dim3(512), 0, s, b);
  } else {
    hipLaunchKernelGGL((fwd_pp_persistent_kernel<128, 128, false, false, 0, 1>), dim3(8 * w), dim3(512), 0, s, b);
  }
  return hipGetLastError();
}

// workgroups of the persistent launch for this problem (the cycles array
// holds 64 entries per workgroup)
int fwd_pp_persistent_grid(const FwdArgs& a) {
  const int tiles_per_xcd = fwd_grid(a, false) / 8;
  return 8 * max(min(a.persist_wgs / 8, tiles_per_xcd), 1);
}

// Test-only: work tile t of the dense per-tile launch (t = 8 j + XCD, the
// dispatch order) as (sequence, head, row block), or -1s for a padding entry,
// from the same pp_locate the kernels call. One wave per tile: pp_locate
// takes its arguments as wave-uniform.
template <bool CAUSAL>
__global__ __launch_bounds__(64) void fwd_tile_order_kernel(FwdArgs a, int* out) {
  const int t = blockIdx.x;
  PpTile tile;
  const bool ok = pp_locate<CAUSAL, false>(a, t & 7, t >> 3, tile);
  if (threadIdx.x == 0) {
    out[3 * t] = ok ? tile.seq : -1;
    out[3 * t + 1] = ok ? tile.h : -1;
    out[3 * t + 2] = ok ? tile.row_lo / kPpBlockM : -1;
  }
}

hipError_t launch_fwd_tile_order(const FwdArgs& a, bool causal, int* out, hipStream_t s) {
  const int grid = fwd_grid(a, false);
  if (causal) {
    hipLaunchKernelGGL((fwd_tile_order_kernel<true>), dim3(grid), dim3(64), 0, s, a, out);
  } else {
    hipLaunchKernelGGL((fwd_tile_order_kernel<false>), dim3(grid), dim3(64), 0, s, a, out);
  }
  return hipGetLastError();
}

// Persistent form with the K/V pipeline running on across tiles (pp_walk);
// equal head dims only: the next tile's Q of (192, 128) does not fit beside
// its stages in LDS.
template <int D, bool CAUSAL, bool VARLEN, int EXPMODE>
__global__ __launch_bounds__(512, 1) void fwd_pp_unrollkv_kernel(FwdArgs a) {
  pp_walk<D, D, CAUSAL, VARLEN, EXPMODE>(a);
}

template <int D, int DV, bool CAUSAL, bool VARLEN, int EXPMODE>
static hipError_t launch_pp_t(const FwdArgs& a, hipStream_t s) {
  const int grid = fwd_grid(a, VARLEN);
  if (a.persist_wgs > 0) {
    FwdArgs b = a;
    b.tiles_per_xcd = grid / 8;
    const int w = min(a.persist_wgs / 8, b.tiles_per_xcd);  // workgroups per XCD
    if (a.unroll_kv) {
      if constexpr (D == DV) {
        hipLaunchKernelGGL((fwd_pp_unrollkv_kernel<D, CAUSAL, VARLEN, EXPMODE>), dim3(8 * max(w, 1)), dim3(512), 0,
                           s, b);
      } else {
        return hipErrorInvalidValue;
      }
    } else {
      hipLaunchKernelGGL((fwd_pp_persistent_kernel<D, DV, CAUSAL, VARLEN, EXPMODE>), dim3(8 * max(w, 1)), dim3(512),
                         0, s, b);
    }
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
