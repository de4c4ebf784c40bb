// Internal launcher interfaces between the C ABI (ea_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ea {

// Forward (bf16). Dense inputs are BSHD, packed inputs THD with cu_seqlens.
struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;          // may be null
  const int* cu_q;     // packed sequences only
  const int* cu_k;
  int nseq;            // batch (dense) or number of packed sequences
  int Nq, Nk;          // dense sequence lengths
  int Hq, Hkv, group;  // group = Hq / Hkv
  int total_q;         // packed: lse row stride per head
  int n_mb;            // row blocks per sequence (dense) / upper bound (packed)
  float scale_log2;    // softmax scale * log2(e)
  float tau;           // lazy-rescale threshold in log2 units
  int natural;         // 1: ascending row-block order
  const int* seq_order;  // packed only: virtual -> actual sequence, or null (input order)
  int lpt_auto;        // packed, seq_order null, nseq <= kLptLds: the ping-pong kernel's
                       // workgroups order the sequences heaviest first themselves
  int persist_wgs;     // ping-pong kernel: > 0 runs the persistent form with this many
                       // workgroups (a multiple of 8, one per CU); 0: one workgroup per tile
  int tiles_per_xcd;   // set by the launcher for the persistent form
  int unroll_kv;       // with persist_wgs > 0 and equal head dims: 1 runs the walk whose
                       // K/V pipeline continues across tiles (unroll-KV schedule)
  int* stats;          // test-only statistics launch: per-wave counts (else unused)
  unsigned long long* cycles;  // test-only phase-cycle launch: per-wave sums (else unused)
};

constexpr int kFwdBlockM = 128;  // query rows per workgroup (4 waves x 32)
constexpr int kFwdBlockN = 64;   // keys per K/V tile
constexpr int kPpBlockM = 256;   // query rows per workgroup of the 8-wave ping-pong kernel
// most packed sequences whose heaviest-first order a ping-pong workgroup
// computes itself, one per thread of its 512
constexpr int kLptLds = 512;

// grid size for the forward (workgroups)
int fwd_grid(const FwdArgs& a, bool varlen);
hipError_t launch_fwd(const FwdArgs& a, int d, bool causal, bool varlen, int exp_mode,
                      hipStream_t s);
// 8-wave ping-pong forward; a.n_mb counts kPpBlockM-row blocks
// d: head dim of Q and K, dv: of V and O ((64, 64), (128, 128) or (192, 128))
hipError_t launch_fwd_pp(const FwdArgs& a, int d, int dv, bool causal, bool varlen, int exp_mode,
                         hipStream_t s);
// test-only: the persistent ping-pong forward (dense, d = 128, hardware exp)
// writing per-wave live-step and lazy-rescale counts to a.stats (16 ints per
// work tile); a.n_mb counts kPpBlockM-row blocks, a.persist_wgs is set
hipError_t launch_fwd_pp_stats(const FwdArgs& a, bool causal, int mode, hipStream_t s);
int fwd_pp_persistent_grid(const FwdArgs& a);
// test-only: (sequence, head, row block) of every dense work tile, 3 ints each
hipError_t launch_fwd_tile_order(const FwdArgs& a, bool causal, int* out, hipStream_t s);

// varlen batch order (heaviest sequence first): weights[b] and order[virtual] = actual
// Test-only: the heaviest-first order a ping-pong workgroup computes for
// itself (n <= kLptLds sequences, 256-row blocks) into out[n].
hipError_t launch_lpt_lds_order(const int* cu_q, const int* cu_k, int n, int causal, int* out, hipStream_t s);
hipError_t launch_lpt_order(const int* cu_q, const int* cu_k, int n, int causal, int block_m, int* weights,
                            int* order, hipStream_t s);

// MX fp8 forward
struct Mx8Args {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const uint8_t* qs;
  const uint8_t* ks;
  const uint8_t* vs;
  uint16_t* o;
  float* lse;
  int B, N, Hq, Hkv, group;
  int n_mb;
  float scale_log2;
  float tau;
  int fmt;  // Q/K/V codes: 0 = OCP e4m3, 1 = OCP e5m2
  int persist_wgs;    // ping-pong kernel: > 0 runs the persistent form (workgroups, multiple of 8)
  int tiles_per_xcd;  // set by the launcher for the persistent form
};
hipError_t launch_fwd_mx8(const Mx8Args& a, bool causal, hipStream_t s);
// 8-wave software-pipelined MX fp8 forward (one workgroup per tile); a.n_mb
// counts kPpBlockM-row blocks
hipError_t launch_fwd_mx8_sp(const Mx8Args& a, bool causal, hipStream_t s);
// 8-wave ping-pong MX fp8 forward (persistent when a.persist_wgs > 0); a.n_mb
// counts kPpBlockM-row blocks
hipError_t launch_fwd_mx8_pp(const Mx8Args& a, bool causal, hipStream_t s);

// Backward (bf16, dense BSHD): dQ, dK, dV of O = softmax(scale Q K^T) V for
// the output gradient dout, from the forward's O and lse.
struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;    // [B, Hq, Nq] natural log, scale included
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dd;           // workspace [B, Hq, Nq]: dO . O per row
  float* lse2;         // workspace [B, Hq, Nq]: lse * log2(e)
  int B, Nq, Nk, Hq, Hkv, group;
  int n_mb;            // 128-row query blocks (dQ kernel)
  int n_kb;            // 128-key blocks (dK/dV kernel)
  float scale, scale_log2;
  int natural;         // 1: ascending block order (results do not depend on it)
  int persist_wgs;     // > 0: persistent dQ and dK/dV kernels with this many workgroups (multiple of 8)
  int tiles_per_xcd;   // set by the launcher for each persistent kernel
};
hipError_t launch_bwd(const BwdArgs& a, int d, bool causal, hipStream_t s);
size_t bwd_workspace_bytes(int B, int Hq, int Nq);
void bwd_bind_workspace(BwdArgs& a, void* workspace);

// Paged split-KV decode
struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int* block_table;
  const int* seq_lens;
  uint16_t* o;
  float* lse;
  float* part_o;     // [num_ranges + B slots, Hkv, group, d] fp32
  float* part_lse;   // [num_ranges + B slots, Hkv, group] fp32
  int* plan;         // [2B + 1]: first / last range of each sequence, total chunks
  int B, Hq, Hkv, group;
  int page_size, max_pages;
  int num_pages;     // pool size: page indices outside [0, num_pages) read as zeros
  int num_ranges;    // W: equal shares of the batch's chunks, one workgroup each
  float scale_log2;
  // test-only gather dump: the K and V rows each chunk staged, by sequence and
  // token, into dense [B, dump_t, Hkv, d] buffers (null otherwise)
  uint16_t* dump_k;
  uint16_t* dump_v;
  int dump_t;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
// the split kernel alone, writing the gather dump as well (a.dump_* set)
hipError_t launch_decode_gather_dump(const DecodeArgs& a, hipStream_t s);
size_t decode_workspace_bytes(int B, int Hq, int d, int num_ranges);
// workgroups along y: groups of 8 (KV head, 16-column block of its query heads) pairs
int decode_head_groups(int Hkv, int group);
// points part_o / part_lse / plan into a workspace of decode_workspace_bytes
void decode_bind_workspace(DecodeArgs& a, void* workspace);
// the allocation-free decode's device array: size, and its address on the
// current device (looked up once per device)
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace ea
