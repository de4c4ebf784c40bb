// Paged split-KV decode and the log-sum-exp combine for gfx950.
//
// Method ("Faster, more flexible FlashAttention-4 for LLM inference"):
//  * split-KV (section on PR 1940): the KV sequence of every (sequence, KV head)
//    is cut into pieces, one workgroup per piece, each producing a normalised
//    partial output and its log-sum-exp; a second kernel merges the pieces
//    (lse = log sum exp lse_s, o = sum exp(lse_s - lse) o_s) in fp32;
//  * paged KV of any page size (sections on PR 1999/2104): token t of sequence
//    b is read from page block_table[b, t / page_size], slot t % page_size;
//  * one query tile per workgroup (PR 1993) and all query heads of one KV head
//    packed into that tile (PR 2186), so every KV byte is read once.
//
// gfx950 mapping (this file's design):
//  * Balanced pieces. Every sequence's context is a run of 32-token chunks;
//    laid end to end over the batch they form Tc chunks, which are cut into W
//    equal ranges, one per workgroup (W = gridDim.x, one workgroup per CU by
//    default). A range meets one or more sequences; for each of them the
//    workgroup runs the online-softmax loop over its chunks and writes one
//    partial into slot w + b. Walking the pieces in order, each step moves to
//    the next workgroup, the next sequence or both, so w + b never repeats and
//    W + B slots suffice whatever the lengths. Every workgroup gets the same
//    work up to one chunk, so there is no tail of long splits.
//  * A workgroup of 8 waves serves 8 KV heads, one wave per head, all walking
//    the same chunks. In the [pages, page_size, Hkv, d] cache a token's rows for
//    all KV heads are adjacent, so the workgroup streams whole contiguous rows.
//  * A chunk is two 16-token tiles, loaded token by token for every page size
//    (down to 1). Address generation is decoupled from use, as in the pages'
//    transposed scheme for small pages: lane i < 32 looks up the page of the
//    chunk's token i once (block-table entry prefetched one chunk ahead) and
//    forms its row index; each lane then fetches the row indices of the 8
//    tokens it copies with lane shuffles instead of recomputing them. Tokens
//    at or past the sequence end and pages outside the pool read as zeros.
//    Every K/V byte is read once per launch, so the loads are streaming
//    (non-temporal). (A per-tile path for page sizes that 16 divides -- one
//    buffer resource per 16-token tile -- measured 1.8% slower than this one
//    at page 16 once both used streaming loads.)
//  * Query heads: the G = Hq / Hkv heads of one KV head are packed as columns
//    of 16-wide blocks (PR 2186's GQA packing for any ratio). G <= 16 leaves
//    unused columns; G > 16 gives a KV head several blocks, one wave each, and
//    those waves of one workgroup read the same K/V rows (from cache after the
//    first).
//  * Each wave copies its chunk's K and V rows into its own LDS region (no
//    workgroup barrier anywhere), prefetching the next chunk into VGPRs while
//    it computes the current one. S^T = K Q^T and O^T = V^T P^T use
//    v_mfma_f32_16x16x32_bf16 with the packed query heads as the 16-wide
//    column block; V^T operands come from ds_read_b64_tr_b16.
#include "ea_device.h"
#include "ea_internal.h"

#include <mutex>

namespace ea {

namespace {
constexpr int kD = 128;
constexpr int kChunk = 32;  // tokens per wave step
constexpr int kWaves = 8;  // one wave per KV head of a group of 8
}  // namespace

__device__ __forceinline__ float xor16_max(float x) {
  return __builtin_fmaxf(x, __shfl_xor(x, 16));
}
__device__ __forceinline__ float xor16_sum(float x) { return x + __shfl_xor(x, 16); }

// Chunks of sequence b: its length clamped to [0, block-table capacity].
__device__ __forceinline__ int seq_len_clamped(const DecodeArgs& a, int b) {
  return min(max(a.seq_lens[b], 0), a.max_pages * a.page_size);
}
__device__ __forceinline__ int seq_chunks(const DecodeArgs& a, int b) {
  return (seq_len_clamped(a, b) + kChunk - 1) / kChunk;
}
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}
// Total chunks over the batch (every lane gets the same value).
__device__ __forceinline__ int total_chunks(const DecodeArgs& a, int lane) {
  int t = 0;
  for (int base = 0; base < a.B; base += 64)
    if (base + lane < a.B) t += seq_chunks(a, base + lane);
  return uniform(wave_sum(t));
}
// First chunk of workgroup w's range: floor(w * Tc / W).
__device__ __forceinline__ int range_start(int w, int Tc, int W) {
  return (int)(((long long)w * Tc) / W);
}

// DUMP (test-only): every wave of a KV head's first column block also writes
// the K and V rows it staged for each chunk, as gathered, to a.dump_k /
// a.dump_v at (sequence, token, KV head).
template <bool DUMP = false>
__global__ __launch_bounds__(64 * kWaves, 1) void decode_split_kernel(DecodeArgs a) {
  constexpr int D = kD;
  constexpr int TILE = kChunk * D;  // bf16 elements per K or V chunk
  __shared__ __attribute__((aligned(16))) uint16_t smem_raw[kWaves * 2 * TILE];
  EA_LDS uint16_t* sm = (EA_LDS uint16_t*)smem_raw;

  // grid: x = workgroup range w of W, y = group of kWaves (KV head, column
  // block) pairs; wave i owns pair kWaves*y + i: KV head vh / ncb, query heads
  // 16 * (vh % ncb) + 0..15 of its group.
  const int wg = blockIdx.x, W = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
  const int G = a.group, ncb = (G + 15) / 16;
  const int vh = uniform(kWaves * (int)blockIdx.y + wv);
  if (vh >= a.Hkv * ncb) return;  // no barriers below: idle waves may leave
  const int hkv = uniform(vh / ncb);
  const int c_lo = uniform(16 * (vh - hkv * ncb));  // first query head of this wave's block
  const int ncols = uniform(min(16, G - c_lo));
  const int Tc = total_chunks(a, lane);
  // lane 0 of the first wave of head group 0 records Tc (workgroup 0, whose
  // range may be empty) and which ranges hold each sequence's first and last
  // chunk, for the combine
  const bool record = blockIdx.y == 0 && wv == 0 && lane == 0;
  if (record && wg == 0) a.plan[2 * a.B] = Tc;
  const int g0 = uniform(range_start(wg, Tc, W)), g1 = uniform(range_start(wg + 1, Tc, W));
  if (g0 >= g1) return;

  const int grp = lane >> 4, col = lane & 15;
  const int ps = a.page_size;
  EA_LDS uint16_t* ks = sm + wv * 2 * TILE;
  EA_LDS uint16_t* vs = ks + TILE;

  // loop-invariant LDS offsets
  int st_off[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int row = 4 * u + grp;
    st_off[u] = row * D + ((col ^ swz<D>(row)) << 3);
  }
  int k_off[2][D / 32];
#pragma unroll
  for (int tl = 0; tl < 2; ++tl)
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) k_off[tl][kk] = tile_off<D>(16 * tl + col, 32 * kk + 8 * grp);
  const int tr_row = 4 * grp + ((lane >> 2) & 3);
  const int tr_col = 4 * (lane & 3);
  int v_off[D / 16][2];
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) {
    v_off[mt][0] = tile_off<D>(tr_row, 16 * mt + tr_col);
    v_off[mt][1] = tile_off<D>(16 + tr_row, 16 * mt + tr_col);
  }
  const float sl = a.scale_log2;
  const float tau = 8.0f;

  // ---- one piece: chunks [c0, c1) of sequence b, partial into slot wg + b
  auto run_piece = [&](int b, int c0, int c1) {
    const int L = uniform(seq_len_clamped(a, b));
    const int t_begin = uniform(kChunk * c0);
    const int t_end = uniform(min(L, kChunk * c1));
    const int nck = uniform(c1 - c0);
    const int* bt = uniform_ptr(a.block_table + (size_t)b * a.max_pages);

    // Q^T operand (B of S^T = K Q^T): column = packed query head, k = d
    bf16x8 qf[D / 32];
    {
      const uint16_t* qp = a.q + ((size_t)b * a.Hq + (size_t)hkv * G + c_lo + col) * D + 8 * grp;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) qf[kk] = (col < ncols) ? *(const bf16x8*)(qp + 32 * kk) : bf16x8{};
    }

    // chunk staging: lane handles rows 4u + grp (u = 0..7), 16-byte column chunk col
    i32x4 rk[8], rv[8];
    // lane i < 32 holds the
    // block-table entry and slot of token i of a chunk, and from them the row
    // index page * page_size + slot, or -1 for a token past the end or a page
    // outside the pool.
    auto bt_entry = [&](int ci, int& slot) -> int {
      const int t = t_begin + kChunk * ci + lane;
      const int pi = t / ps;
      slot = t - pi * ps;
      return (lane < kChunk && t < t_end) ? bt[pi] : -1;
    };
    auto row_index = [&](int ent, int slot) -> int {
      return (unsigned)ent < (unsigned)a.num_pages ? ent * ps + slot : -1;
    };
    const size_t row_elems = (size_t)a.Hkv * D;
    const uint16_t* kbase = a.kc + (size_t)hkv * D + 8 * col;
    const uint16_t* vbase = a.vc + (size_t)hkv * D + 8 * col;
    auto gload_rows = [&](int rows) {
#pragma unroll
      for (int tl = 0; tl < 2; ++tl)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int ri = __shfl(rows, 16 * tl + 4 * u + grp);
          i32x4 kx = i32x4{}, vx = i32x4{};
          if (ri >= 0) {
            kx = __builtin_nontemporal_load((const i32x4*)(kbase + (size_t)ri * row_elems));
            vx = __builtin_nontemporal_load((const i32x4*)(vbase + (size_t)ri * row_elems));
          }
          rk[4 * tl + u] = kx;
          rv[4 * tl + u] = vx;
        }
    };
    auto sstore = [&]() {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        lds_store<i32x4>(ks + st_off[u], rk[u]);
        lds_store<i32x4>(vs + st_off[u], rv[u]);
      }
    };
    // rk[u] / rv[u] hold chunk row 4 u + grp, columns 8 col .. 8 col + 7
    auto dump = [&](int ci) {
      if constexpr (DUMP) {
        if (c_lo == 0) {
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int t = t_begin + kChunk * ci + 4 * u + grp;
            if (t < t_end) {
              const size_t at = (((size_t)b * a.dump_t + t) * a.Hkv + hkv) * D + 8 * col;
              *(i32x4*)(a.dump_k + at) = rk[u];
              *(i32x4*)(a.dump_v + at) = rv[u];
            }
          }
        }
      }
    };

    float m_run = kNegInf, l_run = 0.f;
    f32x4 oacc[D / 16];
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) oacc[mt] = f32x4{};

    int ent_next = -1, slot_next = 0;  // entry of chunk ci + 1
    {
      int slot0;
      const int ent0 = bt_entry(0, slot0);
      if (nck > 1) ent_next = bt_entry(1, slot_next);
      gload_rows(row_index(ent0, slot0));
    }
    sstore();
    dump(0);
    __builtin_amdgcn_s_waitcnt(0);
    for (int ci = 0; ci < nck; ++ci) {
      const int t0 = t_begin + kChunk * ci;
      if (ci + 1 < nck) {
        // the entry of chunk ci + 1 was loaded one chunk ago (before the
        // loads of chunk ci, which the last sstore waited for)
        const int rows = row_index(ent_next, slot_next);
        if (ci + 2 < nck) ent_next = bt_entry(ci + 2, slot_next);
        gload_rows(rows);
      }
      // ---- S^T = K Q^T for two 16-token tiles
      f32x4 s[2];
#pragma unroll
      for (int tl = 0; tl < 2; ++tl) {
        s[tl] = f32x4{};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
          s[tl] = mfma16x16x32(lds_load<bf16x8>(ks + k_off[tl][kk]), qf[kk], s[tl]);
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
      const i32x4 pt = {(int)pack_bf16x2(pv[0][0], pv[0][1]), (int)pack_bf16x2(pv[0][2], pv[0][3]),
                        (int)pack_bf16x2(pv[1][0], pv[1][1]), (int)pack_bf16x2(pv[1][2], pv[1][3])};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pt);
      // ---- O^T += V^T P^T (k = 32 tokens: tile-0 tokens 4*grp+0..3, tile-1 tokens 16+4*grp+0..3)
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) {
        const i16x4 lo = ds_read_tr16(vs + v_off[mt][0]);
        const i16x4 hi = ds_read_tr16(vs + v_off[mt][1]);
        const i32x4 t = {__builtin_bit_cast(i32x2, lo)[0], __builtin_bit_cast(i32x2, lo)[1],
                         __builtin_bit_cast(i32x2, hi)[0], __builtin_bit_cast(i32x2, hi)[1]};
        oacc[mt] = mfma16x16x32(__builtin_bit_cast(bf16x8, t), pb, oacc[mt]);
      }
      if (ci + 1 < nck) {
        sstore();
        dump(ci + 1);
      }
    }

    // ---- this piece's normalised partial output and log-sum-exp
    float l_tot = xor16_sum(l_run);
    l_tot = sum_with_partner32(l_tot);
    const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
    if (col < ncols) {
      const size_t prow = (((size_t)(wg + b)) * a.Hkv + hkv) * G + c_lo + col;
      float* po = a.part_o + prow * D;
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) {
        const float4 v = {oacc[mt][0] * inv, oacc[mt][1] * inv, oacc[mt][2] * inv, oacc[mt][3] * inv};
        *(float4*)(po + 16 * mt + 4 * grp) = v;
      }
      if (grp == 0)
        a.part_lse[prow] = (l_tot > 0.f && m_run != kNegInf) ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
    }
  };

  // ---- walk the sequences whose chunks meet [g0, g1), 64 at a time
  int carry = 0;  // chunks of the sequences before this block of 64
  for (int base = 0; base < a.B && carry < g1; base += 64) {
    const int bb = base + lane;
    const int n = bb < a.B ? seq_chunks(a, bb) : 0;
    const int incl = wave_inclusive_scan(n, lane);
    const int cs = carry + incl - n, ce = carry + incl;
    uint64_t hit = __ballot(n > 0 && cs < g1 && ce > g0);
    while (hit) {
      const int i = __builtin_ctzll(hit);
      hit &= hit - 1;
      const int b = base + i;
      const int sb = __builtin_amdgcn_readlane(cs, i), eb = __builtin_amdgcn_readlane(ce, i);
      const int c0 = max(g0, sb) - sb, c1 = min(g1, eb) - sb;
      if (record && c0 == 0) a.plan[b] = wg;
      if (record && c1 == eb - sb) a.plan[a.B + b] = wg;
      run_piece(b, c0, c1);
    }
    carry = uniform(__builtin_amdgcn_readlane(ce, 63));
  }
}

// One workgroup of 128 threads per (sequence, query head): merge the pieces.
// plan[b] and plan[B + b] are the first and last workgroup ranges holding
// sequence b's chunks; ranges in between that are empty (possible when there
// are fewer chunks than ranges) wrote nothing and are skipped.
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int hkv = h / a.group, head = h % a.group;
  const int d = threadIdx.x;
  const int W = a.num_ranges;
  float acc = 0.f, wsum = 0.f, mx = kNegInf;
  if (seq_chunks(a, b) > 0) {
    const int Tc = a.plan[2 * a.B];
    const int wf = a.plan[b], wl = a.plan[a.B + b];
    auto row = [&](int w) { return (((size_t)(w + b)) * a.Hkv + hkv) * a.group + head; };
    for (int w = wf; w <= wl; ++w)
      if (range_start(w, Tc, W) < range_start(w + 1, Tc, W)) mx = __builtin_fmaxf(mx, a.part_lse[row(w)]);
    if (mx != kNegInf) {
      for (int w = wf; w <= wl; ++w) {
        if (range_start(w, Tc, W) >= range_start(w + 1, Tc, W)) continue;
        const float ls = a.part_lse[row(w)];
        const float wgt = (ls == kNegInf) ? 0.f : __expf(ls - mx);
        wsum += wgt;
        acc += wgt * a.part_o[row(w) * kD + d];
      }
    }
  }
  const float o = (wsum > 0.f) ? acc / wsum : 0.f;
  bf16x2 v;
  v[0] = (__bf16)o;
  a.o[((size_t)b * a.Hq + h) * kD + d] = __builtin_bit_cast(uint16_t, v[0]);
  if (a.lse != nullptr && d == 0) a.lse[(size_t)b * a.Hq + h] = (wsum > 0.f) ? mx + __logf(wsum) : kNegInf;
}

namespace {
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

// Workspace: part_o [(W + B) slots, Hkv, group, d] fp32, part_lse [(W + B) slots,
// Hkv, group] fp32, plan [2B + 1] int32 (first range, last range per sequence,
// then Tc), each starting on a 256-byte boundary.
size_t decode_workspace_bytes(int B, int Hq, int d, int num_ranges) {
  const size_t slots = (size_t)num_ranges + (size_t)B;
  return round256(slots * Hq * d * sizeof(float)) + round256(slots * Hq * sizeof(float)) +
         (2 * (size_t)B + 1) * sizeof(int);
}

void decode_bind_workspace(DecodeArgs& a, void* workspace) {
  const size_t slots = (size_t)a.num_ranges + (size_t)a.B;
  char* p = (char*)workspace;
  a.part_o = (float*)p;
  p += round256(slots * a.Hq * kD * sizeof(float));
  a.part_lse = (float*)p;
  p += round256(slots * a.Hq * sizeof(float));
  a.plan = (int*)p;
}

static hipError_t launch_p(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(decode_split_kernel<false>, dim3(a.num_ranges, decode_head_groups(a.Hkv, a.group)),
                     dim3(64 * kWaves), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.B * a.Hq), dim3(kD), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_gather_dump(const DecodeArgs& a, hipStream_t s) {
  if (a.num_ranges <= 0 || a.part_o == nullptr || a.plan == nullptr || a.dump_k == nullptr || a.dump_v == nullptr)
    return hipErrorInvalidValue;
  const dim3 grid(a.num_ranges, decode_head_groups(a.Hkv, a.group));
  hipLaunchKernelGGL((decode_split_kernel<true>), grid, dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.num_ranges <= 0 || a.part_o == nullptr || a.plan == nullptr) return hipErrorInvalidValue;
  return launch_p(a, s);
}

// ---------------------------------------------------------------------------
// Allocation-free decode: the split partials and the plan live in a
// file-scope device array instead of a caller workspace. Every device the
// library runs on holds its own copy until the process ends. In host code the
// array's name is only a stand-in: its device address comes from
// hipGetSymbolAddress, once per device, with that device current.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  static std::mutex mu;
  static void* per_device[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

int decode_head_groups(int Hkv, int group) {
  const int ncb = (group + 15) / 16;
  return (Hkv * ncb + kWaves - 1) / kWaves;
}

}  // namespace ea
