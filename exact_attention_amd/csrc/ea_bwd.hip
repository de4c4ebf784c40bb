// Exact attention backward for gfx950 (bf16 in, fp32 accumulate, bf16 out).
//
// Method: the gradients of the forward O = softmax(scale Q K^T) V for an output
// gradient dO are the five products the pages list for the backward
// ("Low-precision FlashAttention-4: end-to-end block-scaled attention for
// Blackwell", section 2.2; "FlashAttention-4: algorithm-pipeline co-design for
// Blackwell", backward sections): S = Q K^T, P = softmax(S) recomputed from
// the forward's saved log-sum-exp, dP = dO V^T, dS = P (dP - D) with
// D_i = dO_i . O_i, dV = P^T dO, dK = scale dS^T Q, dQ = scale dS K. The N x N
// matrices S, P, dP and dS never leave registers.
//
// gfx950 mapping (this file's own design):
//  * No atomics. The pages accumulate dQ over key blocks with atomic adds to a
//    global fp32 buffer (and serialise them for the deterministic mode). At
//    N = 8192 with 128-key blocks that is 64 read-modify-writes per dQ element.
//    Here two kernels split the work instead, each owning its outputs:
//      - bwd_dkdv_kernel: one workgroup per (sequence, KV head, 128 keys), 8
//        waves in two roles on each 32-key block (below), loops over every
//        query tile of every query head of the KV head's group; dK and dV
//        accumulate in registers (4 products: S, dP, dV, dK);
//      - bwd_dq_kernel: one workgroup per (sequence, head, 128 query rows), 4
//        waves x 32 rows, loops over the key tiles (3 products: S, dP, dQ).
//    S and dP are computed twice (7 products instead of 5); in exchange every
//    output is written once, in a fixed order, so the result is
//    deterministic run to run and independent of the tile order.
//  * bwd_prep_kernel computes D_i = dO_i . O_i and lse_i * log2(e) once per
//    row into a caller workspace, read by both kernels.
//  * Operand layouts follow the forward's (lane layouts in ea_device.h):
//      dQ kernel:   S^T = K Q^T and dP^T = V dO^T (K, V from LDS, Q^T and dO^T
//                   in VGPRs), so a lane owns one query row and its D and lse
//                   are one register each; dQ^T += K^T dS^T with K^T read by
//                   ds_read_b64_tr_b16 and dS^T packed straight from the
//                   accumulator layout (the permuted-key trick of the forward);
//      dK/dV kernel: S = Q K^T and dP = dO V^T (Q, dO from LDS, K and V held as
//                   B operands), so a lane owns one key; dV^T += dO^T P and
//                   dK^T += Q^T dS with dO^T and Q^T read transposed. The
//                   two waves on a SIMD take one role each (S, P, dV / dP,
//                   dS, dK) and hand P over through LDS, so one wave's vector
//                   work overlaps the other's matrix products.
//  * Tiles arrive by LDS DMA (buffer_load ... lds) into two stages, issued a
//    tile ahead; rows past the sequence land as zeros.
#include <type_traits>

#include "ea_device.h"
#include "ea_fwd_common.h"
#include "ea_internal.h"

namespace ea {

namespace {
constexpr int kBwdTileQ = 64;   // query rows per dK/dV step
constexpr int kBwdTileK = 64;   // keys per dQ step
}  // namespace

// ---------------------------------------------------------------------------
// D_i = sum_c dO[i,c] O[i,c] and lse2_i = lse_i log2(e), for every (b, h, i):
// 16 lanes per row, 16 bytes each (d = 128: 8 values; d = 64: lanes 8..15
// idle). Outputs [B, Hq, Nq] fp32.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4);  // (b, n, h) row, BSHD order
  const int l16 = threadIdx.x & 15;
  const int rows = a.B * a.Nq * a.Hq;
  float acc = 0.f;
  if (t < rows && 8 * l16 < D) {
    const size_t base = (size_t)t * D + 8 * l16;
    // streaming loads: each byte of O and dO is read once here
    const bf16x8 o = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const i32x4*)(a.o + base)));
    const bf16x8 g = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const i32x4*)(a.dout + base)));
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf((float)o[i], (float)g[i], acc);
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) acc += __shfl_xor(acc, m);
  if (t < rows && l16 == 0) {
    const int h = t % a.Hq;
    const int n = (t / a.Hq) % a.Nq;
    const int b = t / (a.Hq * a.Nq);
    const size_t idx = ((size_t)b * a.Hq + h) * a.Nq + n;
    a.dd[idx] = acc;
    a.lse2[idx] = a.lse[idx] * kLog2e;
  }
}

// DMA of one tile of R rows x D bf16 (row stride `stride` elements in global
// memory) into a swizzled LDS stage: wave w of NWAVES issues pieces w, w +
// NWAVES, ... of 1 KB; lane s of piece p lands at stage byte 1024 p + 16 s =
// (row r, slot sl) and fetches the global chunk sl ^ swz(r) of row r. Rows
// past `rows` read as zeros (buffer range).
template <int D, int R, int NWAVES>
struct TileDma {
  static constexpr int NP = R * D * 2 / 1024;  // pieces per tile
  static constexpr int PPW = NP / NWAVES;      // pieces per wave
  static_assert(NP % NWAVES == 0 && PPW >= 1, "tile must split evenly into 1 KB pieces");
  uint32_t off[PPW];
  __device__ __forceinline__ void init(int w, int lane, size_t stride) {
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int p = 1024 * (w * PPW + i) + 16 * lane;
      const int r = p / (D * 2), sl = (p % (D * 2)) / 16;
      off[i] = (uint32_t)(r * (int)stride * 2 + ((sl ^ swz<D>(r)) << 4));
    }
  }
  // stage: LDS tile base; gbase: global row 0 of the tile; rows: valid rows
  __device__ __forceinline__ void issue(EA_LDS uint16_t* stage, const uint16_t* gbase, int rows, size_t stride,
                                        int w) const {
    const uint32_t nrec = rows > 0 ? (uint32_t)((rows - 1) * (int)stride * 2 + D * 2) : 0u;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(gbase, nrec);
#pragma unroll
    for (int i = 0; i < PPW; ++i) buffer_load16_lds(rs, (EA_LDS void*)(stage + 512 * (w * PPW + i)), off[i]);
  }
};

// ---------------------------------------------------------------------------
// dQ: one workgroup = 4 waves x 32 query rows of one (sequence, head); key
// tiles of 64 in two LDS stages.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_tile(const BwdArgs& a, const int xcd, const int j) {
  constexpr int BM = 128, BN = kBwdTileK, NDT = D / 32;
  constexpr int TILE = BN * D;
  __shared__ __attribute__((aligned(1024))) uint16_t smem_raw[2 * 2 * TILE];
  EA_LDS uint16_t* sm = (EA_LDS uint16_t*)smem_raw;

  // XCD-grouped, heaviest first: all row blocks of one (sequence, head) on one XCD
  const int kg = j / a.n_mb;
  const int r = j - kg * a.n_mb;
  const int g = xcd + 8 * kg;
  if (g >= a.B * a.Hq) return;
  const int seq = uniform(g / a.Hq);
  const int h = uniform(g - seq * a.Hq);
  const int mb = uniform(a.natural ? r : a.n_mb - 1 - r);
  const int hk = uniform(h / a.group);
  const int lq = a.Nq, lk = a.Nk;
  const int off = lk - lq;  // bottom-right causal alignment
  const int row_lo = mb * BM;
  int nkeys = lk;
  if constexpr (CAUSAL) nkeys = min(lk, row_lo + BM + off);
  if (nkeys < 0) nkeys = 0;
  const int nkb = uniform((nkeys + BN - 1) / BN);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = uniform(tid >> 6), hh = lane >> 5, c = lane & 31;
  const int qi = row_lo + w * 32 + c;
  const size_t qstride = (size_t)a.Hq * D, kstride = (size_t)a.Hkv * D;
  const size_t q0 = (size_t)seq * lq, k0 = (size_t)seq * lk;

  // Q^T and dO^T operands (B of S^T = K Q^T and dP^T = V dO^T), and the row's
  // lse2 and D (rows past the end: lse2 = +inf makes P = 0)
  bf16x8 qf[D / 16], gf[D / 16];
  {
    const size_t ro = (q0 + qi) * qstride + (size_t)h * D + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qf[kk] = (qi < lq) ? *(const bf16x8*)(a.q + ro + 16 * kk) : bf16x8{};
      gf[kk] = (qi < lq) ? *(const bf16x8*)(a.dout + ro + 16 * kk) : bf16x8{};
    }
  }
  const size_t rowidx = ((size_t)seq * a.Hq + h) * lq + qi;
  const float lse2 = (qi < lq) ? a.lse2[rowidx] : __builtin_inff();
  const float dval = (qi < lq) ? a.dd[rowidx] : 0.f;

  TileDma<D, BN, 4> dma;
  dma.init(w, lane, kstride);
  const uint16_t* kg_base = a.k + k0 * kstride + (size_t)hk * D;
  const uint16_t* vg_base = a.v + k0 * kstride + (size_t)hk * D;
  auto issue = [&](int kb) {
    EA_LDS uint16_t* ks = sm + (kb & 1) * 2 * TILE;
    const int rows = min(lk - kb * BN, BN);
    dma.issue(ks, kg_base + (size_t)kb * BN * kstride, rows, kstride, w);
    dma.issue(ks + TILE, vg_base + (size_t)kb * BN * kstride, rows, kstride, w);
  };

  int k_off[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) k_off[kk] = tile_off<D>(c, 16 * kk + 8 * hh);
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int t_off[NDT][2];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    t_off[dt][0] = tile_off<D>(tr_row, 32 * dt + tr_col);
    t_off[dt][1] = tile_off<D>(tr_row + 8, 32 * dt + tr_col);
  }
  const int wave_last_q = row_lo + w * 32 + 31;
  const int wave_first_q = row_lo + w * 32;
  const float sl = a.scale_log2;

  f32x16 dq[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dq[dt] = f32x16{};

  // one 32-key half of a tile: S^T and dP^T, P, dS^T, packed as two B operands
  auto half = [&](const EA_LDS uint16_t* ks, const EA_LDS uint16_t* vs, int kbase, int hk32, bf16x8& d0,
                  bf16x8& d1) {
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      s = mfma32x32x16(lds_load<bf16x8>(ks + k_off[kk] + 32 * hk32 * D), qf[kk], s);
      dp = mfma32x32x16(lds_load<bf16x8>(vs + k_off[kk] + 32 * hk32 * D), gf[kk], dp);
    }
    bool need_mask = kbase + 32 * hk32 + 32 > lk;
    if constexpr (CAUSAL) need_mask = need_mask || (kbase + 32 * hk32 + 31 > wave_first_q + off);
    int rel = 64;
    if (need_mask) {
      int lim = lk;
      if constexpr (CAUSAL) lim = min(lk, qi + off + 1);
      rel = lim - kbase - 32 * hk32 - 4 * hh;  // element i valid iff its key offset < rel
    }
    float ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int ko = 8 * (i >> 2) + (i & 3);
      const float p = (ko < rel) ? exp2_hw(__builtin_fmaf(s[i], sl, -lse2)) : 0.f;
      ds[i] = p * (dp[i] - dval);
    }
    const i32x4 t0 = {(int)pack_bf16x2(ds[0], ds[1]), (int)pack_bf16x2(ds[2], ds[3]),
                      (int)pack_bf16x2(ds[4], ds[5]), (int)pack_bf16x2(ds[6], ds[7])};
    const i32x4 t1 = {(int)pack_bf16x2(ds[8], ds[9]), (int)pack_bf16x2(ds[10], ds[11]),
                      (int)pack_bf16x2(ds[12], ds[13]), (int)pack_bf16x2(ds[14], ds[15])};
    d0 = __builtin_bit_cast(bf16x8, t0);
    d1 = __builtin_bit_cast(bf16x8, t1);
  };

  if (nkb > 0) issue(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) issue(kb + 1);
    const EA_LDS uint16_t* ks = sm + (kb & 1) * 2 * TILE;
    const EA_LDS uint16_t* vs = ks + TILE;
    const int kbase = kb * BN;
    if (!(CAUSAL && kbase > wave_last_q + off)) {
      bf16x8 dsb[4];
      half(ks, vs, kbase, 0, dsb[0], dsb[1]);
      half(ks, vs, kbase, 1, dsb[2], dsb[3]);
      // dQ^T += K^T dS^T (the d tiles inner, so consecutive MFMAs use
      // different accumulators)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const i16x4 lo = ds_read_tr16(ks + t_off[dt][0] + 16 * st * D);
          const i16x4 hi = ds_read_tr16(ks + t_off[dt][1] + 16 * st * D);
          const i32x4 t = {__builtin_bit_cast(i32x2, lo)[0], __builtin_bit_cast(i32x2, lo)[1],
                           __builtin_bit_cast(i32x2, hi)[0], __builtin_bit_cast(i32x2, hi)[1]};
          dq[dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, t), dsb[st], dq[dt]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // dQ = scale * acc, rows in lanes, d in elements (the forward's O layout),
  // written as 16-byte row pieces (every lane takes part in the packing)
  uint4 pk[NDT][2];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) pack_rows16(dq[dt], a.scale, pk[dt]);
  if (qi < lq) {
    uint16_t* op = a.dq + (q0 + qi) * qstride + (size_t)h * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int j = 0; j < 2; ++j) *(uint4*)(op + 32 * dt + 16 * j + 8 * hh) = pk[dt][j];
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  dq_tile<D, CAUSAL>(a, blockIdx.x & 7, blockIdx.x >> 3);
}
// persistent form (persistent_snake in ea_fwd_common.h)
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_persistent_kernel(BwdArgs a) {
  persistent_snake(uniform(a.tiles_per_xcd), [&](int xcd, int j) { dq_tile<D, CAUSAL>(a, xcd, j); });
}


// ---------------------------------------------------------------------------
// dK, dV: one workgroup = 8 waves for 128 keys of one (sequence, KV head); it
// walks every query tile (64 rows, two 32-row slices) of every query head of
// the group. Waves w and w + 4 share a SIMD and a 32-key block and split the
// products by role, half a step apart:
//   phase k, role A (w < 4):  dV^T += dO^T P(k-1), then S(k) = Q K^T,
//                             P(k) = 2^(S scale log2e - lse2) -> LDS;
//   phase k, role B (w >= 4): dS(k-1) = P(k-1) (dP(k-1) - D) with P from LDS,
//                             dK^T += Q^T dS(k-1), then dP(k) = dO V^T.
// One workgroup barrier ends each phase. On every SIMD role A's matrix
// products run beside role B's vector work at the start of a phase and the
// other way round at its end. A tile serves three phases (its two slices and
// the deferred second products of the last), so tiles sit in three LDS stages
// and each one's DMA is issued three phases before its first use.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_tile(const BwdArgs& a, const int xcd, const int j) {
  constexpr int BK = 128, BQ = kBwdTileQ, NDT = D / 32;
  constexpr int TILE = BQ * D;
  constexpr int NSTAGE = 3;
  __shared__ __attribute__((aligned(1024))) uint16_t smem_raw[NSTAGE * 2 * TILE];
  __shared__ __attribute__((aligned(16))) float rowstat[NSTAGE][2][BQ];  // [stage][lse2, D][row]
  __shared__ __attribute__((aligned(16))) float pxch[2][4][4 * 64 * 4];  // [parity][pair][chunk][lane][4]
  EA_LDS uint16_t* sm = (EA_LDS uint16_t*)smem_raw;

  // XCD-grouped; causal: the key blocks with the most query rows (lowest) first
  const int kg = j / a.n_kb;
  const int r = j - kg * a.n_kb;
  const int g = xcd + 8 * kg;
  if (g >= a.B * a.Hkv) return;
  const int seq = uniform(g / a.Hkv);
  const int hk = uniform(g - seq * a.Hkv);
  const int kblk = uniform(a.natural ? a.n_kb - 1 - r : r);
  const int lq = a.Nq, lk = a.Nk;
  const int off = lk - lq;
  const int k_lo = kblk * BK;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = uniform(tid >> 6), hh = lane >> 5, c = lane & 31;
  const int pr = w & 3;              // 32-key block of this wave pair
  const bool role_b = w >= 4;        // wave-uniform
  const int kj = k_lo + pr * 32 + c;  // this lane's key
  const size_t qstride = (size_t)a.Hq * D, kstride = (size_t)a.Hkv * D;
  const size_t q0 = (size_t)seq * lq, k0 = (size_t)seq * lk;

  // the pair's stationary operand (B of the first product): K for role A, V for role B
  bf16x8 opnd[D / 16];
  {
    const uint16_t* src = role_b ? a.v : a.k;
    const size_t ro = (k0 + kj) * kstride + (size_t)hk * D + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) opnd[kk] = (kj < lk) ? *(const bf16x8*)(src + ro + 16 * kk) : bf16x8{};
  }

  // query tiles: causal rows i see key k_lo iff i + off >= k_lo
  int qt0 = 0;
  if constexpr (CAUSAL) qt0 = max(0, k_lo - off) / BQ;
  const int nqt = uniform(max(0, (lq + BQ - 1) / BQ - qt0));
  const int ntiles = uniform(nqt * a.group);
  const int nslices = 2 * ntiles;

  TileDma<D, BQ, 8> dma;
  dma.init(w, lane, qstride);
  constexpr int kDmaOps = 2 * TileDma<D, BQ, 8>::PPW;  // vector memory ops per wave per tile
  // tiles are issued in order; the next one's (head, row block, stage) advance
  // incrementally (no divisions in the loop)
  int iss_t = 0, iss_hq = hk * a.group, iss_qt = qt0, iss_st = 0;
  auto next_stage = [](int st) { return st == NSTAGE - 1 ? 0 : st + 1; };
  // wave 0 also loads the tile's row statistics (two more vector memory ops)
  float st_lse[2] = {0.f, 0.f}, st_d[2] = {0.f, 0.f};
  auto issue_next = [&]() {
    const int t = iss_t, hq = iss_hq, qt = iss_qt;
    EA_LDS uint16_t* qs = sm + iss_st * 2 * TILE;
    const int rows = min(lq - qt * BQ, BQ);
    const size_t go = (q0 + (size_t)qt * BQ) * qstride + (size_t)hq * D;
    dma.issue(qs, a.q + go, rows, qstride, w);
    dma.issue(qs + TILE, a.dout + go, rows, qstride, w);
    if (w == 0) {
      const int row = qt * BQ + lane;
      const size_t idx = ((size_t)seq * a.Hq + hq) * lq + row;
      st_lse[t & 1] = row < lq ? a.lse2[idx] : __builtin_inff();  // rows past the end: P = 0
      st_d[t & 1] = row < lq ? a.dd[idx] : 0.f;
    }
    ++iss_t;
    iss_st = next_stage(iss_st);
    if (++iss_qt == qt0 + nqt) {
      iss_qt = qt0;
      ++iss_hq;
    }
  };
  // tile t's statistics into its stage st
  auto park_stats = [&](int t, int st) {
    if (w == 0) {
      lds_store<float>((EA_LDS float*)rowstat[st][0] + lane, st_lse[t & 1]);
      lds_store<float>((EA_LDS float*)rowstat[st][1] + lane, st_d[t & 1]);
    }
  };

  int q_off[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) q_off[kk] = tile_off<D>(c, 16 * kk + 8 * hh);
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int t_off[NDT][2];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    t_off[dt][0] = tile_off<D>(tr_row, 32 * dt + tr_col);
    t_off[dt][1] = tile_off<D>(tr_row + 8, 32 * dt + tr_col);
  }
  const float sl = a.scale_log2;

  f32x16 acc[NDT];  // dV^T (role A) or dK^T (role B)
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};

  if (ntiles > 0) issue_next();
  if (ntiles > 1) issue_next();
  __builtin_amdgcn_s_waitcnt(0);
  if (ntiles > 0) park_stats(0, 0);
  if (ntiles > 1) park_stats(1, 1);
  __syncthreads();

  // stages of the current slice's tile and of the previous tile
  int st_cur = 0, st_prev = NSTAGE - 1;
  // phase k opens by issuing tile k / 2 + 2 on the second slice of tile k / 2
  // (its stage was freed by the barrier that ended phase k - 1, the last one
  // tile k / 2 - 1 used); the first slice of a tile moves the stages on
  auto phase_begin = [&](int k) __attribute__((always_inline)) {
    if ((k & 1) && iss_t < ntiles) issue_next();
    if (!(k & 1) && k > 0) {
      st_prev = st_cur;
      st_cur = next_stage(st_cur);
    }
  };
  // phase k closes: P stores done; before the first phase of tile u =
  // (k + 1) / 2 >= 2 its DMA (issued at phase 2u - 3) has landed -- only tile
  // u + 1's, issued at this phase's start, may still be in flight
  auto phase_end = [&](int k) __attribute__((always_inline)) {
    wait_lgkm0();
    if ((k & 1) && (k >> 1) + 1 < ntiles && (k >> 1) + 1 >= 2) {
      const int u = (k >> 1) + 1;
      if (u + 1 < ntiles) {
        if (w == 0) wait_vmcnt<kDmaOps + 2>(); else wait_vmcnt<kDmaOps>();
      } else {
        __builtin_amdgcn_s_waitcnt(0);
      }
      park_stats(u, next_stage(st_cur));
      wait_lgkm0();
    }
    pp_barrier();
  };
  // first product of slice k: X = T1 opnd^T over the 32 rows, two independent
  // accumulation chains (even and odd d chunks)
  auto first_product = [&](int k, const EA_LDS uint16_t* t1) __attribute__((always_inline)) -> f32x16 {
    const int rs = k & 1;
    f32x16 x0 = f32x16{}, x1 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; kk += 2) {
      x0 = mfma32x32x16(lds_load<bf16x8>(t1 + q_off[kk] + 32 * rs * D), opnd[kk], x0);
      x1 = mfma32x32x16(lds_load<bf16x8>(t1 + q_off[kk + 1] + 32 * rs * D), opnd[kk + 1], x1);
    }
    return x0 + x1;
  };
  // second product of slice kp: acc += T2^T Y (T2 read transposed, rows permuted
  // like the packed B operand)
  auto second_product = [&](int kp, const EA_LDS uint16_t* t2, const bf16x8 (&yb)[2]) __attribute__((always_inline)) {
    const int rs = kp & 1;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int ro = (32 * rs + 16 * st) * D;
        const i16x4 lo = ds_read_tr16(t2 + t_off[dt][0] + ro);
        const i16x4 hi = ds_read_tr16(t2 + t_off[dt][1] + ro);
        const i32x4 ta = {__builtin_bit_cast(i32x2, lo)[0], __builtin_bit_cast(i32x2, lo)[1],
                          __builtin_bit_cast(i32x2, hi)[0], __builtin_bit_cast(i32x2, hi)[1]};
        acc[dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, ta), yb[st], acc[dt]);
      }
    }
  };
  auto pack16 = [&](const float (&y)[16], bf16x8 (&yb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int b0 = 8 * st;
      const i32x4 t = {(int)pack_bf16x2(y[b0], y[b0 + 1]), (int)pack_bf16x2(y[b0 + 2], y[b0 + 3]),
                       (int)pack_bf16x2(y[b0 + 4], y[b0 + 5]), (int)pack_bf16x2(y[b0 + 6], y[b0 + 7])};
      yb[st] = __builtin_bit_cast(bf16x8, t);
    }
  };
  // LDS tile of slice k (the current one) or of slice k - 1 (deferred product)
  auto stage_cur = [&]() { return sm + st_cur * 2 * TILE; };
  auto stage_prev_slice = [&](int k) { return sm + ((k & 1) ? st_cur : st_prev) * 2 * TILE; };

  // The phases are straight-line code: a slice that causal masking hides from
  // the pair still runs its products (P = 0 there, so they add exact zeros).
  if (!role_b) {
    // ---------------- role A: S, P (to LDS), dV
    bf16x8 pk[2];
    int hq = hk * a.group, qt = qt0;  // tile of the current slice
    auto phase_a = [&](int k, auto has_prev, auto has_cur) __attribute__((always_inline)) {
      phase_begin(k);
      if constexpr (decltype(has_prev)::value) second_product(k - 1, stage_prev_slice(k) + TILE, pk);  // dO^T P
      if constexpr (decltype(has_cur)::value) {
        const EA_LDS uint16_t* qs = stage_cur();
        const f32x16 x = first_product(k, qs);  // S = Q K^T
        const int rs = k & 1;
        const int rbase = qt * BQ + 32 * rs;
        const EA_LDS float* lst = (const EA_LDS float*)rowstat[st_cur][0];
        EA_LDS f32x4* xp = (EA_LDS f32x4*)pxch[k & 1][pr];
        float p[16];
        // element i = row rbase + 8 (i / 4) + 4 hh + i % 4 of key kj
        auto probs = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 l4 = lds_load<f32x4>(lst + 32 * rs + 8 * i4 + 4 * hh);
            f32x4 p4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              bool ok = true;
              if constexpr (decltype(masked)::value) ok = kj <= rbase + 8 * i4 + 4 * hh + e + off;
              p4[e] = ok ? exp2_hw(__builtin_fmaf(x[4 * i4 + e], sl, -l4[e])) : 0.f;
              p[4 * i4 + e] = p4[e];
            }
            lds_store<f32x4>(xp + 64 * i4 + lane, p4);
          }
        };
        // wave-uniform: the wave's last key is at or before the causal limit
        // of the slice's first row, so no element of the slice is masked
        if (!CAUSAL || k_lo + pr * 32 + 31 <= rbase + off)
          probs(std::integral_constant<bool, false>{});
        else
          probs(std::integral_constant<bool, true>{});
        pack16(p, pk);
        if (rs == 1 && ++qt == qt0 + nqt) {
          qt = qt0;
          ++hq;
        }
      }
      phase_end(k);
    };
    using T = std::integral_constant<bool, true>;
    using F = std::integral_constant<bool, false>;
    if (nslices > 0) {
      phase_a(0, F{}, T{});
      for (int k = 1; k < nslices; ++k) phase_a(k, T{}, T{});
      phase_a(nslices, T{}, F{});
    }
    (void)hq;
  } else {
    // ---------------- role B: dP, dS (P from LDS), dK
    f32x16 dpk = f32x16{};
    auto phase_b = [&](int k, auto has_prev, auto has_cur) __attribute__((always_inline)) {
      phase_begin(k);
      if constexpr (decltype(has_prev)::value) {
        const int kp = k - 1, rs = kp & 1;
        const EA_LDS float* dst_ = (const EA_LDS float*)rowstat[(k & 1) ? st_cur : st_prev][1];
        const EA_LDS f32x4* xp = (const EA_LDS f32x4*)pxch[kp & 1][pr];
        float y[16];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 d4 = lds_load<f32x4>(dst_ + 32 * rs + 8 * i4 + 4 * hh);
          const f32x4 p4 = lds_load<f32x4>(xp + 64 * i4 + lane);
#pragma unroll
          for (int e = 0; e < 4; ++e) y[4 * i4 + e] = p4[e] * (dpk[4 * i4 + e] - d4[e]);
        }
        bf16x8 yb[2];
        pack16(y, yb);
        second_product(kp, stage_prev_slice(k), yb);  // Q^T dS
      }
      if constexpr (decltype(has_cur)::value) dpk = first_product(k, stage_cur() + TILE);  // dP = dO V^T
      phase_end(k);
    };
    using T = std::integral_constant<bool, true>;
    using F = std::integral_constant<bool, false>;
    if (nslices > 0) {
      phase_b(0, F{}, T{});
      for (int k = 1; k < nslices; ++k) phase_b(k, T{}, T{});
      phase_b(nslices, T{}, F{});
    }
  }

  // no DMA may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(0);

  // dV = acc (role A), dK = scale * acc (role B): keys in lanes, d in elements
  const float f = role_b ? a.scale : 1.0f;
  uint4 pk[NDT][2];  // 16-byte row pieces (every lane takes part)
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) pack_rows16(acc[dt], f, pk[dt]);
  if (kj < lk) {
    uint16_t* dst = (role_b ? a.dk : a.dv) + (k0 + kj) * kstride + (size_t)hk * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int j = 0; j < 2; ++j) *(uint4*)(dst + 32 * dt + 16 * j + 8 * hh) = pk[dt][j];
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(BwdArgs a) {
  dkdv_tile<D, CAUSAL>(a, blockIdx.x & 7, blockIdx.x >> 3);
}
// persistent form (persistent_snake in ea_fwd_common.h)
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_persistent_kernel(BwdArgs a) {
  persistent_snake(uniform(a.tiles_per_xcd), [&](int xcd, int j) { dkdv_tile<D, CAUSAL>(a, xcd, j); });
}


template <int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  const int rows = a.B * a.Nq * a.Hq;
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((rows + 15) / 16), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int gq = 8 * ((a.B * a.Hq + 7) / 8) * a.n_mb;
  const int gk = 8 * ((a.B * a.Hkv + 7) / 8) * a.n_kb;
  if (a.persist_wgs > 0) {
    // persistent forms: the dQ kernel fits two workgroups per CU, the dK/dV
    // kernel one
    BwdArgs b = a;
    b.tiles_per_xcd = gq / 8;
    const int wq = max(1, min(2 * a.persist_wgs / 8, b.tiles_per_xcd));
    hipLaunchKernelGGL((bwd_dq_persistent_kernel<D, CAUSAL>), dim3(8 * wq), dim3(256), 0, s, b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    b.tiles_per_xcd = gk / 8;
    const int wk = max(1, min(a.persist_wgs / 8, b.tiles_per_xcd));
    hipLaunchKernelGGL((bwd_dkdv_persistent_kernel<D, CAUSAL>), dim3(8 * wk), dim3(512), 0, s, b);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(gq), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(gk), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int d, bool causal, hipStream_t s) {
  if (d == 64) return causal ? launch_bwd_t<64, true>(a, s) : launch_bwd_t<64, false>(a, s);
  return causal ? launch_bwd_t<128, true>(a, s) : launch_bwd_t<128, false>(a, s);
}

size_t bwd_workspace_bytes(int B, int Hq, int Nq) {
  const size_t n = (size_t)B * Hq * Nq * sizeof(float);
  return 2 * ((n + 255) & ~(size_t)255);
}

void bwd_bind_workspace(BwdArgs& a, void* workspace) {
  const size_t n = (size_t)a.B * a.Hq * a.Nq * sizeof(float);
  char* p = (char*)workspace;
  a.dd = (float*)p;
  a.lse2 = (float*)(p + ((n + 255) & ~(size_t)255));
}

}  // namespace ea
