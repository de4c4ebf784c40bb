// Paged split-KV decode and the log-sum-exp combine for gfx950.
//
// Method ("Faster, more flexible FlashAttention-4 for LLM inference"):
//  * split-KV (section on PR 1940): the KV sequence of every (sequence, KV head)
//    is cut into splits of split_len tokens, one workgroup per split, each
//    producing a normalised partial output and its log-sum-exp; a second
//    kernel merges the splits (lse = log sum exp lse_s, o = sum
//    exp(lse_s - lse) o_s) in fp32;
//  * paged KV of any page size (sections on PR 1999/2104): token t of sequence
//    b is read from page block_table[b, t / page_size], slot t % page_size;
//  * one query tile per workgroup (PR 1993) and all query heads of one KV head
//    packed into that tile (PR 2186), so every KV byte is read once.
//
// gfx950 mapping (this file's design): 4 waves per workgroup take 32-token
// chunks in turn. A chunk is two 16-token tiles; 16 divides page_size, so a
// tile lies in one page and its page index is wave-uniform (a scalar load), and
// only 32-bit row offsets are formed per lane. Each wave copies its chunk's K
// and V rows (256 contiguous bytes per row) into its own LDS region (no
// workgroup barrier in the loop), prefetching the next chunk into VGPRs while
// it computes the current one. S^T = K Q^T and O^T = V^T P^T use
// v_mfma_f32_16x16x32_bf16 with the packed query heads as the 16-wide column
// block; V^T operands come from ds_read_b64_tr_b16. Tokens at or past the
// sequence length are never loaded (zero-filled), so stale or poisoned slots of
// a last page cannot leak.
#include "ea_device.h"
#include "ea_internal.h"

namespace ea {

namespace {
constexpr int kD = 128;
constexpr int kChunk = 32;  // tokens per wave step
constexpr int kWaves = 4;
}  // namespace

__device__ __forceinline__ float xor16_max(float x) {
  return __builtin_fmaxf(x, __shfl_xor(x, 16));
}
__device__ __forceinline__ float xor16_sum(float x) { return x + __shfl_xor(x, 16); }

template <int G>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeArgs a) {
  constexpr int D = kD;
  constexpr int TILE = kChunk * D;  // bf16 elements per K or V chunk
  __shared__ __attribute__((aligned(16))) uint16_t smem_raw[kWaves * 2 * TILE];
  EA_LDS uint16_t* sm = (EA_LDS uint16_t*)smem_raw;

  const int split = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  // lengths beyond the block table's capacity are clamped (never index past it)
  const int L = min(a.seq_lens[b], a.max_pages * a.page_size);
  const int t_begin = split * a.split_len;
  if (t_begin >= L && !(split == 0 && L <= 0)) return;
  const int t_end = min(L, t_begin + a.split_len);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int grp = lane >> 4, col = lane & 15;
  const int ps = a.page_size;
  const size_t row_stride = (size_t)a.Hkv * D;  // elements between consecutive slots
  const int* bt = a.block_table + (size_t)b * a.max_pages;
  const uint16_t* kbase = a.kc + (size_t)hkv * D;
  const uint16_t* vbase = a.vc + (size_t)hkv * D;

  // Q^T operand (B of S^T = K Q^T): column = packed query head, k = d
  bf16x8 qf[D / 32];
  {
    const int head = col;
    const uint16_t* qp = a.q + ((size_t)b * a.Hq + (size_t)hkv * G + head) * D + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) qf[kk] = (head < G) ? *(const bf16x8*)(qp + 32 * kk) : bf16x8{};
  }

  EA_LDS uint16_t* ks = sm + w * 2 * TILE;
  EA_LDS uint16_t* vs = ks + TILE;

  // chunk staging: lane handles rows 4u + grp (u = 0..7), 16-byte column chunk `col`
  i32x4 rk[8], rv[8];
  auto gload = [&](int t0) {
    const int p0 = (t0 < t_end) ? bt[t0 / ps] : 0;
    const int p1 = (t0 + 16 < t_end) ? bt[(t0 + 16) / ps] : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = 4 * u + grp;
      const int tok = t0 + row;
      const int page = (u < 4) ? p0 : p1;
      if (tok < t_end && (unsigned)page < (unsigned)a.num_pages) {
        const size_t off = ((size_t)page * ps + (tok % ps)) * row_stride + col * 8;
        rk[u] = *(const i32x4*)(kbase + off);
        rv[u] = *(const i32x4*)(vbase + off);
      } else {
        rk[u] = i32x4{0, 0, 0, 0};
        rv[u] = i32x4{0, 0, 0, 0};
      }
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = 4 * u + grp;
      const int o = row * D + ((col ^ swz<D>(row)) << 3);
      lds_store<i32x4>(ks + o, rk[u]);
      lds_store<i32x4>(vs + o, rv[u]);
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x4 oacc[D / 16];
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) oacc[mt] = f32x4{};
  const float sl = a.scale_log2;
  const float tau = 8.0f;

  int t0 = t_begin + kChunk * w;
  if (t0 < t_end) {
    gload(t0);
    sstore();
  }
  for (; t0 < t_end; t0 += kChunk * kWaves) {
    const int tn = t0 + kChunk * kWaves;
    if (tn < t_end) gload(tn);
    // ---- S^T = K Q^T for two 16-token tiles
    f32x4 s[2];
#pragma unroll
    for (int tl = 0; tl < 2; ++tl) {
      s[tl] = f32x4{};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const bf16x8 ka = lds_load<bf16x8>(ks + tile_off<D>(16 * tl + col, 32 * kk + 8 * grp));
        s[tl] = mfma16x16x32(ka, qf[kk], s[tl]);
      }
    }
    if (t0 + kChunk > t_end) {
#pragma unroll
      for (int tl = 0; tl < 2; ++tl)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + 16 * tl + 4 * grp + i >= t_end) s[tl][i] = kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = __builtin_fmaxf(mx, __builtin_fmaxf(s[0][i], s[1][i]));
    mx = xor16_max(mx);
    mx = max_with_partner32(mx);
    const float m_new = __builtin_fmaxf(m_run, mx * sl);
    if (__ballot(m_new > m_run + tau)) {
      const float alpha = (m_run == kNegInf) ? 0.f : exp2_hw(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) oacc[mt] *= alpha;
      m_run = m_new;
    }
    const float neg_m = (m_run == kNegInf) ? 0.f : -m_run;
    float pv[2][4];
#pragma unroll
    for (int tl = 0; tl < 2; ++tl)
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[tl][i] = exp2_hw(__builtin_fmaf(s[tl][i], sl, neg_m));
    l_run += (pv[0][0] + pv[0][1]) + (pv[0][2] + pv[0][3]) + (pv[1][0] + pv[1][1]) + (pv[1][2] + pv[1][3]);
    uint32_t pk[4];
    pk[0] = pack_bf16x2(pv[0][0], pv[0][1]);
    pk[1] = pack_bf16x2(pv[0][2], pv[0][3]);
    pk[2] = pack_bf16x2(pv[1][0], pv[1][1]);
    pk[3] = pack_bf16x2(pv[1][2], pv[1][3]);
    const i32x4 pt = {(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pt);
    // ---- O^T += V^T P^T (k = 32 tokens: tile-0 tokens 4*grp+0..3, tile-1 tokens 16+4*grp+0..3)
    const int tr_row = 4 * grp + ((lane >> 2) & 3);
    const int tr_col = 4 * (lane & 3);
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) {
      const i16x4 lo = ds_read_tr16(vs + tile_off<D>(tr_row, 16 * mt + tr_col));
      const i16x4 hi = ds_read_tr16(vs + tile_off<D>(16 + tr_row, 16 * mt + tr_col));
      const i32x4 t = {__builtin_bit_cast(i32x2, lo)[0], __builtin_bit_cast(i32x2, lo)[1],
                       __builtin_bit_cast(i32x2, hi)[0], __builtin_bit_cast(i32x2, hi)[1]};
      oacc[mt] = mfma16x16x32(__builtin_bit_cast(bf16x8, t), pb, oacc[mt]);
    }
    if (tn < t_end) sstore();
  }

  // ---- merge the four waves of this split through LDS
  float l_tot = xor16_sum(l_run);
  l_tot = sum_with_partner32(l_tot);
  __syncthreads();  // all waves done with their K/V regions
  float* red = (float*)smem_raw;                   // [4 waves][16 heads][D]
  float* red_m = red + kWaves * 16 * D;            // [4][16]
  float* red_l = red_m + kWaves * 16;              // [4][16]
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(w * 16 + col) * D + 16 * mt + 4 * grp + i] = oacc[mt][i];
  if (grp == 0) {
    red_m[w * 16 + col] = m_run;
    red_l[w * 16 + col] = l_tot;
  }
  __syncthreads();
  // 256 threads: thread -> (head, 8 consecutive d)
  for (int idx = tid; idx < G * (D / 8); idx += 256) {
    const int head = idx / (D / 8), d0 = (idx % (D / 8)) * 8;
    float mstar = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) mstar = __builtin_fmaxf(mstar, red_m[ww * 16 + head]);
    float wt[kWaves], lsum = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = red_m[ww * 16 + head];
      wt[ww] = (mw == kNegInf) ? 0.f : exp2_hw(mw - mstar);
      lsum += wt[ww] * red_l[ww * 16 + head];
    }
    const float inv = (lsum > 0.f) ? 1.0f / lsum : 0.f;
    const size_t prow = (((size_t)b * a.Hkv + hkv) * a.max_splits + split) * G + head;
    float* po = a.part_o + prow * D + d0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) acc += wt[ww] * red[(ww * 16 + head) * D + d0 + e];
      po[e] = acc * inv;
    }
    if (d0 == 0)
      a.part_lse[prow] = (lsum > 0.f && mstar != kNegInf) ? (mstar + __log2f(lsum)) * kLn2 : kNegInf;
  }
}

// One workgroup of 128 threads per (sequence, query head): merge the splits.
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int hkv = h / a.group, head = h % a.group;
  const int L = min(a.seq_lens[b], a.max_pages * a.page_size);
  const int nsp = L > 0 ? (L + a.split_len - 1) / a.split_len : 1;
  const int d = threadIdx.x;
  const size_t base = (((size_t)b * a.Hkv + hkv) * a.max_splits) * a.group + head;
  float mx = kNegInf;
  for (int s = 0; s < nsp; ++s) mx = __builtin_fmaxf(mx, a.part_lse[base + (size_t)s * a.group]);
  float acc = 0.f, wsum = 0.f;
  if (mx != kNegInf) {
    for (int s = 0; s < nsp; ++s) {
      const float ls = a.part_lse[base + (size_t)s * a.group];
      const float wgt = (ls == kNegInf) ? 0.f : __expf(ls - mx);
      wsum += wgt;
      acc += wgt * a.part_o[(base + (size_t)s * a.group) * kD + d];
    }
  }
  const float o = (wsum > 0.f) ? acc / wsum : 0.f;
  bf16x2 v;
  v[0] = (__bf16)o;
  a.o[((size_t)b * a.Hq + h) * kD + d] = __builtin_bit_cast(uint16_t, v[0]);
  if (a.lse != nullptr && d == 0) a.lse[(size_t)b * a.Hq + h] = (wsum > 0.f) ? mx + __logf(wsum) : kNegInf;
}

size_t decode_workspace_bytes(int B, int Hq, int d, int max_splits) {
  return (size_t)B * Hq * max_splits * d * sizeof(float) + (size_t)B * Hq * max_splits * sizeof(float);
}

template <int G>
static hipError_t launch_g(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(decode_split_kernel<G>, dim3(a.max_splits, a.Hkv, a.B), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.B * a.Hq), dim3(kD), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  switch (a.group) {
    case 1: return launch_g<1>(a, s);
    case 2: return launch_g<2>(a, s);
    case 4: return launch_g<4>(a, s);
    case 8: return launch_g<8>(a, s);
    default: return launch_g<16>(a, s);
  }
}

}  // namespace ea
