// C ABI of libexactattn.so: argument validation (host only, before any HIP
// call), tuning defaults, work decomposition parameters and kernel dispatch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "ea.h"
#include "ea_internal.h"
#include "ea_test.h"

namespace {

thread_local char g_err[512] = "";

ea_status fail(ea_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

ea_status ok() {
  g_err[0] = '\0';
  return EA_OK;
}

ea_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(EA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool finite_pos(float x) { return std::isfinite(x) && x > 0.f; }

// largest lazy-rescale threshold of the MX fp8 forward: floor(log2(448) * 1000) / 1000
constexpr float kMx8MaxRescaleLog2 = 8.807f;

ea_status check_tuning(const ea_fwd_tuning* t) {
  if (t == nullptr) return EA_OK;
  if (t->exp_mode < 0 || t->exp_mode > 2) return fail(EA_ERR_INVALID, "tuning.exp_mode must be 0, 1 or 2");
  if (!(t->rescale_log2 >= 0.f && t->rescale_log2 <= 16.f))
    return fail(EA_ERR_INVALID, "tuning.rescale_log2 must be in [0, 16]");
  if (t->natural_order != 0 && t->natural_order != 1)
    return fail(EA_ERR_INVALID, "tuning.natural_order must be 0 or 1");
  if (t->kernel < EA_FWD_KERNEL_AUTO || t->kernel > EA_FWD_KERNEL_UNROLL_KV)
    return fail(EA_ERR_INVALID, "tuning.kernel must be 0, 1, 2, 3, 4 or 5");
  return EA_OK;
}

// Workgroups of the persistent ping-pong form: one per CU of the current
// device, rounded down to a multiple of 8 (the tile order deals work to the 8
// XCDs by workgroup id). Cached per device; 0 if the count is unavailable.
// Threads may race to fill an entry: each stores the same value, atomically.
int persistent_workgroups() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    n = (cus / 8) * 8;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The 8-wave kernels cover 256-row blocks, the 4-wave kernel 128-row blocks;
// a.n_mb arrives counted in 128-row blocks.
// d / dv: head dims of Q, K and of V, O; d != dv (192 / 128) runs the
// ping-pong kernel only (checked by the callers).
hipError_t dispatch_fwd(ea::FwdArgs a, int d, int dv, bool causal, bool varlen, const ea_fwd_tuning& tt,
                        hipStream_t s) {
  if (d != dv) {
    a.n_mb = (a.n_mb + 1) / 2;
    // AUTO: the persistent form for dense inputs here too (1.36 against
    // 1.39 ms at B=4 H=16 N=8192 causal)
    if (tt.kernel == EA_FWD_KERNEL_PERSISTENT || (tt.kernel == EA_FWD_KERNEL_AUTO && !varlen)) {
      a.persist_wgs = persistent_workgroups();
      if (a.persist_wgs <= 0) return hipErrorInvalidDevice;
    }
    return ea::launch_fwd_pp(a, d, dv, causal, varlen, tt.exp_mode, s);
  }
  const bool pp = tt.kernel == EA_FWD_KERNEL_PINGPONG || tt.kernel == EA_FWD_KERNEL_PERSISTENT ||
                  tt.kernel == EA_FWD_KERNEL_UNROLL_KV || (tt.kernel == EA_FWD_KERNEL_AUTO && d == 128);
  if (pp) {
    a.n_mb = (a.n_mb + 1) / 2;
    // AUTO: the persistent form for dense inputs (2.5% faster at B=4 H=16
    // N=8192 causal, bitwise the same results); packed inputs keep one
    // workgroup per row block, whose dynamic dispatch balances irregular
    // sequence lengths
    if (tt.kernel == EA_FWD_KERNEL_PERSISTENT || tt.kernel == EA_FWD_KERNEL_UNROLL_KV ||
        (tt.kernel == EA_FWD_KERNEL_AUTO && !varlen)) {
      a.persist_wgs = persistent_workgroups();
      if (a.persist_wgs <= 0) return hipErrorInvalidDevice;
      a.unroll_kv = tt.kernel == EA_FWD_KERNEL_UNROLL_KV;
    }
    return ea::launch_fwd_pp(a, d, d, causal, varlen, tt.exp_mode, s);
  }
  return ea::launch_fwd(a, d, causal, varlen, tt.exp_mode, s);
}

}  // namespace

extern "C" {

int ea_version(void) { return 1; }

const char* ea_last_error(void) { return g_err; }

void ea_fwd_tuning_default(ea_fwd_tuning* t) {
  if (t == nullptr) return;
  t->exp_mode = EA_EXP_HW;
  t->rescale_log2 = 8.0f;
  t->natural_order = 0;
  t->kernel = EA_FWD_KERNEL_AUTO;
}

ea_status ea_attn_fwd_hd(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Nq, int Nk, int Hq, int Hkv, int d_qk, int d_v, int causal,
                         float scale, const ea_fwd_tuning* tuning, void* stream) {
  const int d = d_qk;
  if (!q || !k || !v || !o) return fail(EA_ERR_INVALID, "q, k, v and o must be non-null");
  if (B <= 0 || Nq <= 0 || Nk <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || d_v <= 0)
    return fail(EA_ERR_INVALID, "B, Nq, Nk, Hq, Hkv and the head dims must be positive");
  if (Hq % Hkv) return fail(EA_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (!((d == 64 && d_v == 64) || (d == 128 && d_v == 128) || (d == 192 && d_v == 128)))
    return fail(EA_ERR_UNSUPPORTED, "head dims (%d, %d) not supported: (64, 64), (128, 128) or (192, 128)", d, d_v);
  if (!finite_pos(scale)) return fail(EA_ERR_INVALID, "scale must be finite and positive");
  if (causal != 0 && causal != 1) return fail(EA_ERR_INVALID, "causal must be 0 or 1");
  if (ea_status st = check_tuning(tuning); st != EA_OK) return st;
  if (tuning != nullptr && tuning->kernel == EA_FWD_KERNEL_PIPELINED)
    return fail(EA_ERR_UNSUPPORTED, "the bf16 forward has no pipelined kernel (kernel 3 is MX fp8 only)");
  if (d != d_v && tuning != nullptr && tuning->kernel != EA_FWD_KERNEL_AUTO &&
      tuning->kernel != EA_FWD_KERNEL_PINGPONG && tuning->kernel != EA_FWD_KERNEL_PERSISTENT)
    return fail(EA_ERR_UNSUPPORTED, "head dims (%d, %d) run on the ping-pong kernel only", d, d_v);
  if ((long long)B * Nq >= (1LL << 31) || (long long)B * Nk >= (1LL << 31))
    return fail(EA_ERR_UNSUPPORTED, "B * N must be below 2^31");
  const int n_mb = (Nq + ea::kFwdBlockM - 1) / ea::kFwdBlockM;
  if ((long long)((B * (long long)Hq + 7) / 8) * 8 * n_mb >= (1LL << 31))
    return fail(EA_ERR_UNSUPPORTED, "problem too large for one launch");
  ea_fwd_tuning tt;
  ea_fwd_tuning_default(&tt);
  if (tuning) tt = *tuning;

  ea::FwdArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.nseq = B;
  a.Nq = Nq;
  a.Nk = Nk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = Hq / Hkv;
  a.total_q = B * Nq;
  a.n_mb = n_mb;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.tau = tt.rescale_log2;
  a.natural = tt.natural_order;
  return hip_status(dispatch_fwd(a, d, d_v, causal != 0, false, tt, (hipStream_t)stream),
                    "attention forward launch");
}

size_t ea_test_fwd_rescale_stats_len(int B, int Nq, int Hq) {
  if (B <= 0 || Nq <= 0 || Hq <= 0) return 0;
  const long long tiles = ((B * (long long)Hq + 7) / 8) * 8 * ((Nq + ea::kPpBlockM - 1) / ea::kPpBlockM);
  return (size_t)tiles * 32;
}

size_t ea_test_fwd_tiles(int B, int Nq, int Hq) {
  if (B <= 0 || Nq <= 0 || Hq <= 0) return 0;
  return (size_t)(((B * (long long)Hq + 7) / 8) * 8 * ((Nq + ea::kPpBlockM - 1) / ea::kPpBlockM));
}

ea_status ea_test_fwd_tile_order(int B, int Nq, int Nk, int Hq, int causal, int* out, size_t out_len, void* stream) {
  if (out == nullptr) return fail(EA_ERR_INVALID, "out must be non-null");
  if (B <= 0 || Nq <= 0 || Nk <= 0 || Hq <= 0) return fail(EA_ERR_INVALID, "B, Nq, Nk and Hq must be positive");
  if (causal != 0 && causal != 1) return fail(EA_ERR_INVALID, "causal must be 0 or 1");
  if ((long long)B * Nq >= (1LL << 31) || (long long)B * Nk >= (1LL << 31))
    return fail(EA_ERR_UNSUPPORTED, "B * N must be below 2^31");
  const size_t need = 3 * ea_test_fwd_tiles(B, Nq, Hq);
  if (out_len < need) return fail(EA_ERR_WORKSPACE, "out needs %zu ints, %zu given", need, out_len);
  ea::FwdArgs a{};
  a.nseq = B;
  a.Nq = Nq;
  a.Nk = Nk;
  a.Hq = Hq;
  a.Hkv = Hq;
  a.group = 1;
  a.total_q = B * Nq;
  a.n_mb = (Nq + ea::kPpBlockM - 1) / ea::kPpBlockM;
  return hip_status(ea::launch_fwd_tile_order(a, causal != 0, out, (hipStream_t)stream), "tile order launch");
}

ea_status ea_test_wall_clock_khz(int device, int* khz) {
  if (khz == nullptr) return fail(EA_ERR_INVALID, "khz must be non-null");
  return hip_status(hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, device), "wall clock rate query");
}

ea_status ea_test_fwd_rescale_stats(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                    int Nq, int Nk, int Hq, int Hkv, int causal, float scale, float rescale_log2,
                                    int* stats, size_t stats_len, void* stream) {
  if (!q || !k || !v || !o || !stats) return fail(EA_ERR_INVALID, "q, k, v, o and stats must be non-null");
  if (B <= 0 || Nq <= 0 || Nk <= 0 || Hq <= 0 || Hkv <= 0)
    return fail(EA_ERR_INVALID, "B, Nq, Nk, Hq and Hkv must be positive");
  if (Hq % Hkv) return fail(EA_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (!finite_pos(scale)) return fail(EA_ERR_INVALID, "scale must be finite and positive");
  if (causal != 0 && causal != 1) return fail(EA_ERR_INVALID, "causal must be 0 or 1");
  if (!(rescale_log2 >= 0.f && rescale_log2 <= 16.f)) return fail(EA_ERR_INVALID, "rescale_log2 must be in [0, 16]");
  if ((long long)B * Nq >= (1LL << 31) || (long long)B * Nk >= (1LL << 31))
    return fail(EA_ERR_UNSUPPORTED, "B * N must be below 2^31");
  const size_t need = ea_test_fwd_rescale_stats_len(B, Nq, Hq);
  if (stats_len < need) return fail(EA_ERR_WORKSPACE, "stats needs %zu ints, %zu given", need, stats_len);
  ea::FwdArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.nseq = B;
  a.Nq = Nq;
  a.Nk = Nk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = Hq / Hkv;
  a.total_q = B * Nq;
  a.n_mb = (Nq + ea::kPpBlockM - 1) / ea::kPpBlockM;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.tau = rescale_log2;
  a.stats = stats;
  a.persist_wgs = persistent_workgroups();
  if (a.persist_wgs <= 0) return fail(EA_ERR_HIP, "device CU count unavailable");
  return hip_status(ea::launch_fwd_pp_stats(a, causal != 0, 1, (hipStream_t)stream), "statistics forward launch");
}

size_t ea_test_fwd_phase_cycles_len(int B, int Nq, int Hq) {
  if (B <= 0 || Nq <= 0 || Hq <= 0) return 0;
  ea::FwdArgs a{};
  a.nseq = B;
  a.Nq = Nq;
  a.Hq = Hq;
  a.n_mb = (Nq + ea::kPpBlockM - 1) / ea::kPpBlockM;
  a.persist_wgs = persistent_workgroups();
  if (a.persist_wgs <= 0) return 0;
  return (size_t)ea::fwd_pp_persistent_grid(a) * 64;
}

ea_status ea_test_fwd_phase_cycles(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Nq,
                                   int Nk, int Hq, int Hkv, int causal, float scale, unsigned long long* cycles,
                                   size_t cycles_len, void* stream) {
  if (!q || !k || !v || !o || !cycles) return fail(EA_ERR_INVALID, "q, k, v, o and cycles must be non-null");
  if (B <= 0 || Nq <= 0 || Nk <= 0 || Hq <= 0 || Hkv <= 0)
    return fail(EA_ERR_INVALID, "B, Nq, Nk, Hq and Hkv must be positive");
  if (Hq % Hkv) return fail(EA_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (!finite_pos(scale)) return fail(EA_ERR_INVALID, "scale must be finite and positive");
  if (causal != 0 && causal != 1) return fail(EA_ERR_INVALID, "causal must be 0 or 1");
  if ((long long)B * Nq >= (1LL << 31) || (long long)B * Nk >= (1LL << 31))
    return fail(EA_ERR_UNSUPPORTED, "B * N must be below 2^31");
  const size_t need = ea_test_fwd_phase_cycles_len(B, Nq, Hq);
  if (need == 0) return fail(EA_ERR_HIP, "device CU count unavailable");
  if (cycles_len < need) return fail(EA_ERR_WORKSPACE, "cycles needs %zu entries, %zu given", need, cycles_len);
  ea::FwdArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.nseq = B;
  a.Nq = Nq;
  a.Nk = Nk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = Hq / Hkv;
  a.total_q = B * Nq;
  a.n_mb = (Nq + ea::kPpBlockM - 1) / ea::kPpBlockM;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.tau = 8.0f;
  a.cycles = cycles;
  a.persist_wgs = persistent_workgroups();
  if (hipError_t e = hipMemsetAsync(cycles, 0, need * sizeof(unsigned long long), (hipStream_t)stream);
      e != hipSuccess)
    return hip_status(e, "phase-cycle clear");
  return hip_status(ea::launch_fwd_pp_stats(a, causal != 0, 2, (hipStream_t)stream), "phase-cycle forward launch");
}

ea_status ea_attn_fwd_tuned(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal,
                            float scale, const ea_fwd_tuning* tuning, void* stream) {
  if (d > 0 && d != 64 && d != 128) return fail(EA_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", d);
  return ea_attn_fwd_hd(q, k, v, o, lse, B, Nq, Nk, Hq, Hkv, d, d, causal, scale, tuning, stream);
}

ea_status ea_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int Nq, int Nk, int Hq, int Hkv, int d, int causal, float scale,
                      void* stream) {
  return ea_attn_fwd_tuned(q, k, v, o, lse, B, Nq, Nk, Hq, Hkv, d, causal, scale, nullptr, stream);
}

namespace {

// The packed forward. lpt_auto: without a caller's order, the ping-pong
// kernel's workgroups order up to kLptLds sequences heaviest first themselves.
ea_status varlen_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens_q,
                     const int* cu_seqlens_k, int num_seqs, int total_q, int total_k, int max_seqlen_q, int Hq,
                     int Hkv, int d, int causal, float scale, const int* seq_order, bool lpt_auto,
                     const ea_fwd_tuning* tuning, void* stream) {
  if (!q || !k || !v || !o || !cu_seqlens_q || !cu_seqlens_k)
    return fail(EA_ERR_INVALID, "q, k, v, o and cu_seqlens must be non-null");
  if (num_seqs <= 0 || total_q <= 0 || total_k <= 0 || max_seqlen_q <= 0 || Hq <= 0 || Hkv <= 0 ||
      d <= 0)
    return fail(EA_ERR_INVALID, "num_seqs, totals, max_seqlen_q, Hq, Hkv and d must be positive");
  if (Hq % Hkv) return fail(EA_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (d != 64 && d != 128) return fail(EA_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", d);
  if (!finite_pos(scale)) return fail(EA_ERR_INVALID, "scale must be finite and positive");
  if (causal != 0 && causal != 1) return fail(EA_ERR_INVALID, "causal must be 0 or 1");
  if (ea_status st = check_tuning(tuning); st != EA_OK) return st;
  if (tuning != nullptr && tuning->kernel == EA_FWD_KERNEL_PIPELINED)
    return fail(EA_ERR_UNSUPPORTED, "the bf16 forward has no pipelined kernel (kernel 3 is MX fp8 only)");
  if (max_seqlen_q > total_q) return fail(EA_ERR_INVALID, "max_seqlen_q exceeds total_q");
  const int n_mb = (max_seqlen_q + ea::kFwdBlockM - 1) / ea::kFwdBlockM;
  if ((long long)((num_seqs * (long long)Hq + 7) / 8) * 8 * n_mb >= (1LL << 31))
    return fail(EA_ERR_UNSUPPORTED, "problem too large for one launch");
  ea_fwd_tuning tt;
  ea_fwd_tuning_default(&tt);
  if (tuning) tt = *tuning;

  ea::FwdArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.nseq = num_seqs;
  a.Nq = 0;
  a.Nk = 0;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = Hq / Hkv;
  a.total_q = total_q;
  a.n_mb = n_mb;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.tau = tt.rescale_log2;
  a.natural = tt.natural_order;
  a.seq_order = seq_order;
  // heaviest first by default where the order decides the end time: fewer
  // (sequence, head) groups than CUs, so the tail of the heaviest groups is
  // not covered by other work (measured: 16 sequences x 2 heads 2.97 -> 2.67
  // ms; 8 sequences x 32 heads 20.75 -> 21.05 ms, so not there)
  const int cus = persistent_workgroups();
  a.lpt_auto = (lpt_auto && seq_order == nullptr && num_seqs <= ea::kLptLds &&
                (long long)num_seqs * Hq < (long long)(cus > 0 ? cus : 256))
                   ? 1
                   : 0;
  return hip_status(dispatch_fwd(a, d, d, causal != 0, true, tt, (hipStream_t)stream),
                    "varlen attention forward launch");
}

}  // namespace

ea_status ea_attn_fwd_varlen_ordered(const void* q, const void* k, const void* v, void* o, float* lse,
                                     const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs,
                                     int total_q, int total_k, int max_seqlen_q, int Hq, int Hkv, int d,
                                     int causal, float scale, const int* seq_order,
                                     const ea_fwd_tuning* tuning, void* stream) {
  return varlen_fwd(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q, Hq, Hkv,
                    d, causal, scale, seq_order, false, tuning, stream);
}

ea_status ea_attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                             const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs,
                             int total_q, int total_k, int max_seqlen_q, int Hq, int Hkv, int d,
                             int causal, float scale, const ea_fwd_tuning* tuning, void* stream) {
  return varlen_fwd(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q, Hq, Hkv,
                    d, causal, scale, nullptr, true, tuning, stream);
}

ea_status ea_test_varlen_lds_order(const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs, int causal,
                                   int* order, void* stream) {
  if (!cu_seqlens_q || !cu_seqlens_k || !order) return fail(EA_ERR_INVALID, "cu_seqlens and order must be non-null");
  if (num_seqs <= 0) return fail(EA_ERR_INVALID, "num_seqs must be positive");
  if (num_seqs > ea::kLptLds) return fail(EA_ERR_UNSUPPORTED, "at most %d sequences", ea::kLptLds);
  if (causal != 0 && causal != 1) return fail(EA_ERR_INVALID, "causal must be 0 or 1");
  return hip_status(ea::launch_lpt_lds_order(cu_seqlens_q, cu_seqlens_k, num_seqs, causal, order, (hipStream_t)stream),
                    "LDS LPT order launch");
}

ea_status ea_varlen_lpt_order(const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs, int causal,
                              int block_m, int* weights, int* order, void* stream) {
  if (!cu_seqlens_q || !cu_seqlens_k || !weights || !order)
    return fail(EA_ERR_INVALID, "cu_seqlens, weights and order must be non-null");
  if (num_seqs <= 0) return fail(EA_ERR_INVALID, "num_seqs must be positive");
  if (num_seqs > (1 << 16)) return fail(EA_ERR_UNSUPPORTED, "at most 65536 sequences (the ranking is quadratic)");
  if (causal != 0 && causal != 1) return fail(EA_ERR_INVALID, "causal must be 0 or 1");
  if (block_m != ea::kFwdBlockM && block_m != ea::kPpBlockM)
    return fail(EA_ERR_INVALID, "block_m must be %d or %d (the forward kernels' row blocks)", ea::kFwdBlockM,
                ea::kPpBlockM);
  return hip_status(ea::launch_lpt_order(cu_seqlens_q, cu_seqlens_k, num_seqs, causal, block_m, weights, order,
                                         (hipStream_t)stream),
                    "varlen LPT order launch");
}

ea_status ea_attn_fwd_mx8_fmt(const void* q8, const void* k8, const void* v8, const uint8_t* q_scale,
                              const uint8_t* k_scale, const uint8_t* v_scale, void* o, float* lse,
                              int B, int N, int Hq, int Hkv, int d, int causal, float scale, int in_format,
                              const ea_fwd_tuning* tuning, void* stream) {
  if (!q8 || !k8 || !v8 || !q_scale || !k_scale || !v_scale || !o)
    return fail(EA_ERR_INVALID, "tensor pointers must be non-null");
  if (B <= 0 || N <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0)
    return fail(EA_ERR_INVALID, "B, N, Hq, Hkv and d must be positive");
  if (Hq % Hkv) return fail(EA_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (d != 128) return fail(EA_ERR_UNSUPPORTED, "MX fp8 forward supports d = 128 only");
  if (N % 32) return fail(EA_ERR_UNSUPPORTED, "MX fp8 forward needs N %% 32 == 0");
  if (!finite_pos(scale)) return fail(EA_ERR_INVALID, "scale must be finite and positive");
  if (causal != 0 && causal != 1) return fail(EA_ERR_INVALID, "causal must be 0 or 1");
  if ((long long)B * N >= (1LL << 31)) return fail(EA_ERR_UNSUPPORTED, "B * N must be below 2^31");
  if (in_format != EA_FP8_E4M3 && in_format != EA_FP8_E5M2)
    return fail(EA_ERR_INVALID, "in_format must be EA_FP8_E4M3 (0) or EA_FP8_E5M2 (1)");
  if (ea_status st = check_tuning(tuning); st != EA_OK) return st;
  ea_fwd_tuning tt;
  ea_fwd_tuning_default(&tt);
  if (tuning != nullptr) tt = *tuning;
  if (tt.exp_mode != EA_EXP_HW || tt.natural_order != 0)
    return fail(EA_ERR_UNSUPPORTED, "MX fp8 forward: hardware exponential and heaviest-first order only");
  if (tt.kernel == EA_FWD_KERNEL_UNROLL_KV)
    return fail(EA_ERR_UNSUPPORTED, "MX fp8 forward: kernel 0, 1, 2, 3 or 4 (no unroll-KV kernel)");

  // P is rounded to e4m3 with scale 1 and is at most 2^rescale_log2, so the
  // threshold must keep it under e4m3's largest finite value 448 (2^8.807...)
  if (tt.rescale_log2 > kMx8MaxRescaleLog2)
    return fail(EA_ERR_UNSUPPORTED, "MX fp8 forward: rescale_log2 %g lets P exceed e4m3's 448 (at most %g)",
                (double)tt.rescale_log2, (double)kMx8MaxRescaleLog2);
  // the 8-wave kernels take 256-row blocks, the 4-wave one 128
  const bool pipelined = tt.kernel != EA_FWD_KERNEL_4WAVE;
  ea::Mx8Args a{};
  a.q = (const uint8_t*)q8;
  a.k = (const uint8_t*)k8;
  a.v = (const uint8_t*)v8;
  a.qs = q_scale;
  a.ks = k_scale;
  a.vs = v_scale;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.B = B;
  a.N = N;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = Hq / Hkv;
  const int bm = pipelined ? ea::kPpBlockM : ea::kFwdBlockM;
  a.n_mb = (N + bm - 1) / bm;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.tau = tt.rescale_log2;
  a.fmt = in_format;
  // AUTO: the ping-pong kernel in its persistent form (B=2 H=16 N=16384
  // d=128 causal: 1.21 ms against 1.29 ms for the software-pipelined kernel)
  if (tt.kernel == EA_FWD_KERNEL_PERSISTENT || tt.kernel == EA_FWD_KERNEL_AUTO) {
    a.persist_wgs = persistent_workgroups();
    if (a.persist_wgs <= 0) return fail(EA_ERR_HIP, "device CU count unavailable");
  }
  const bool pingpong = tt.kernel == EA_FWD_KERNEL_PINGPONG || tt.kernel == EA_FWD_KERNEL_PERSISTENT ||
                        tt.kernel == EA_FWD_KERNEL_AUTO;
  const hipError_t e = pingpong    ? ea::launch_fwd_mx8_pp(a, causal != 0, (hipStream_t)stream)
                       : pipelined ? ea::launch_fwd_mx8_sp(a, causal != 0, (hipStream_t)stream)
                                   : ea::launch_fwd_mx8(a, causal != 0, (hipStream_t)stream);
  return hip_status(e, "MX fp8 forward launch");
}

ea_status ea_attn_fwd_mx8_tuned(const void* q8, const void* k8, const void* v8, const uint8_t* q_scale,
                                const uint8_t* k_scale, const uint8_t* v_scale, void* o, float* lse,
                                int B, int N, int Hq, int Hkv, int d, int causal, float scale,
                                const ea_fwd_tuning* tuning, void* stream) {
  return ea_attn_fwd_mx8_fmt(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, N, Hq, Hkv, d, causal, scale,
                             EA_FP8_E4M3, tuning, stream);
}

ea_status ea_attn_fwd_mx8(const void* q8, const void* k8, const void* v8, const uint8_t* q_scale,
                          const uint8_t* k_scale, const uint8_t* v_scale, void* o, float* lse,
                          int B, int N, int Hq, int Hkv, int d, int causal, float scale,
                          void* stream) {
  return ea_attn_fwd_mx8_tuned(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, N, Hq, Hkv, d, causal,
                               scale, nullptr, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------
extern "C" {

size_t ea_attn_bwd_workspace_size(int B, int Hq, int Nq) {
  if (B <= 0 || Hq <= 0 || Nq <= 0) return 0;
  return ea::bwd_workspace_bytes(B, Hq, Nq);
}

ea_status ea_attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv, int B, int Nq, int Nk, int Hq, int Hkv,
                         int d, int causal, float scale, int schedule, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (schedule < EA_BWD_SCHEDULE_AUTO || schedule > EA_BWD_SCHEDULE_PERSISTENT)
    return fail(EA_ERR_INVALID, "schedule must be 0, 1 or 2");
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
    return fail(EA_ERR_INVALID, "tensor pointers must be non-null");
  if (B <= 0 || Nq <= 0 || Nk <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0)
    return fail(EA_ERR_INVALID, "B, Nq, Nk, Hq, Hkv and d must be positive");
  if (Hq % Hkv) return fail(EA_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (d != 64 && d != 128) return fail(EA_ERR_UNSUPPORTED, "backward head dim %d not supported (64 or 128)", d);
  if (!finite_pos(scale)) return fail(EA_ERR_INVALID, "scale must be finite and positive");
  if (causal != 0 && causal != 1) return fail(EA_ERR_INVALID, "causal must be 0 or 1");
  if ((long long)B * Nq * Hq >= (1LL << 31) || (long long)B * Nk * Hkv >= (1LL << 31))
    return fail(EA_ERR_UNSUPPORTED, "B * N * H must be below 2^31");
  const size_t need = ea::bwd_workspace_bytes(B, Hq, Nq);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(EA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  ea::BwdArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (const uint16_t*)o;
  a.dout = (const uint16_t*)dout;
  a.lse = lse;
  a.dq = (uint16_t*)dq;
  a.dk = (uint16_t*)dk;
  a.dv = (uint16_t*)dv;
  a.B = B;
  a.Nq = Nq;
  a.Nk = Nk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = Hq / Hkv;
  a.n_mb = (Nq + 127) / 128;
  a.n_kb = (Nk + 127) / 128;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.natural = 0;
  // AUTO: one workgroup per tile. The persistent schedule measured 1% slower
  // on both kernels at B=4 H=16 N=8192 d=128 causal (dQ 1.485 against 1.471 ms,
  // dK/dV 2.81 against 2.77 ms): a tile here runs 100-300 us, so the launch
  // gap it saves is small next to the balance that dynamic dispatch keeps.
  if (schedule == EA_BWD_SCHEDULE_PERSISTENT) {
    a.persist_wgs = persistent_workgroups();
    if (a.persist_wgs <= 0) return fail(EA_ERR_HIP, "device CU count unavailable");
  }
  ea::bwd_bind_workspace(a, workspace);
  return hip_status(ea::launch_bwd(a, d, causal != 0, (hipStream_t)stream), "attention backward launch");
}

ea_status ea_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, int B, int Nq, int Nk, int Hq, int Hkv,
                      int d, int causal, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return ea_attn_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, B, Nq, Nk, Hq, Hkv, d, causal, scale,
                        EA_BWD_SCHEDULE_AUTO, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// paged decode
// ---------------------------------------------------------------------------
namespace {

// Number of equal shares W the batch's KV chunks are cut into (one workgroup
// per group of 8 (KV head, query-head block) pairs each). By default one
// workgroup per CU: 256 CUs over those groups, fixed so the workspace size
// does not depend on the device. Any W gives the same result up to rounding.
int choose_ranges(int Hq, int Hkv, int num_splits) {
  if (num_splits > 0) return num_splits;
  const int head_groups = ea::decode_head_groups(Hkv, Hq / Hkv);
  const int w = (256 + head_groups - 1) / head_groups;
  return w < 1 ? 1 : w;
}

}  // namespace

extern "C" {

size_t ea_decode_workspace_size(int B, int Hq, int Hkv, int d, int max_seqlen, int page_size,
                                int num_splits) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || max_seqlen < 0 || page_size <= 0 || num_splits < 0 ||
      Hq % Hkv)
    return 0;
  (void)max_seqlen;
  (void)page_size;
  return ea::decode_workspace_bytes(B, Hq, d, choose_ranges(Hq, Hkv, num_splits));
}

}  // extern "C"

namespace {

// Checks and argument block shared by the two decode entry points (host
// only, before any HIP call).
ea_status decode_args(const void* q, const void* k_cache, const void* v_cache, const int* block_table,
                      const int* seq_lens, void* o, float* lse, int B, int Hq, int Hkv, int d, int page_size,
                      int num_pages, int max_pages_per_seq, float scale, int num_splits, ea::DecodeArgs& a,
                      size_t& need) {
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o)
    return fail(EA_ERR_INVALID, "tensor pointers must be non-null");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || page_size <= 0 || num_pages <= 0 ||
      max_pages_per_seq <= 0)
    return fail(EA_ERR_INVALID, "sizes must be positive");
  if (Hq % Hkv) return fail(EA_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  const int group = Hq / Hkv;
  if (d != 128) return fail(EA_ERR_UNSUPPORTED, "paged decode supports d = 128 only");
  if (!finite_pos(scale)) return fail(EA_ERR_INVALID, "scale must be finite and positive");
  if (num_splits < 0) return fail(EA_ERR_INVALID, "num_splits must be >= 0");
  if (num_splits > 65536) return fail(EA_ERR_UNSUPPORTED, "num_splits above 65536");
  if ((long long)B * max_pages_per_seq * page_size / 32 >= (1LL << 31))
    return fail(EA_ERR_UNSUPPORTED, "batch context too long (2^31 32-token chunks)");
  if ((long long)max_pages_per_seq * page_size >= (1LL << 31))
    return fail(EA_ERR_UNSUPPORTED, "max context too long");
  if ((long long)num_pages * page_size * Hkv * d >= (1LL << 40) || (long long)num_pages * page_size >= (1LL << 31))
    return fail(EA_ERR_UNSUPPORTED, "KV pool too large");
  const int max_seqlen = max_pages_per_seq * page_size;
  need = ea_decode_workspace_size(B, Hq, Hkv, d, max_seqlen, page_size, num_splits);
  a = ea::DecodeArgs{};
  a.q = (const uint16_t*)q;
  a.kc = (const uint16_t*)k_cache;
  a.vc = (const uint16_t*)v_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = group;
  a.page_size = page_size;
  a.max_pages = max_pages_per_seq;
  a.num_pages = num_pages;
  a.num_ranges = choose_ranges(Hq, Hkv, num_splits);
  a.scale_log2 = scale * 1.4426950408889634f;
  return EA_OK;
}

}  // namespace

extern "C" {

ea_status ea_attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                               const int* block_table, const int* seq_lens, void* o, float* lse,
                               int B, int Hq, int Hkv, int d, int page_size, int num_pages,
                               int max_pages_per_seq, float scale, int num_splits, void* workspace,
                               size_t workspace_bytes, void* stream) {
  ea::DecodeArgs a;
  size_t need = 0;
  if (ea_status st = decode_args(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, Hq, Hkv, d, page_size,
                                 num_pages, max_pages_per_seq, scale, num_splits, a, need);
      st != EA_OK)
    return st;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(EA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  ea::decode_bind_workspace(a, workspace);
  return hip_status(ea::launch_decode(a, (hipStream_t)stream), "paged decode launch");
}

ea_status ea_test_decode_gather(const void* q, const void* k_cache, const void* v_cache, const int* block_table,
                                const int* seq_lens, int B, int Hq, int Hkv, int d, int page_size, int num_pages,
                                int max_pages_per_seq, int num_splits, void* dump_k, void* dump_v,
                                size_t dump_elems, void* workspace, size_t workspace_bytes, void* stream) {
  ea::DecodeArgs a;
  size_t need = 0;
  // the split kernel writes no output or lse; dump_k stands in for the
  // output pointer that the shared checks require
  if (ea_status st = decode_args(q, k_cache, v_cache, block_table, seq_lens, dump_k, nullptr, B, Hq, Hkv, d,
                                 page_size, num_pages, max_pages_per_seq, 1.0f, num_splits, a, need);
      st != EA_OK)
    return st;
  if (!dump_k || !dump_v) return fail(EA_ERR_INVALID, "dump buffers must be non-null");
  const size_t want = (size_t)B * max_pages_per_seq * page_size * Hkv * d;
  if (dump_elems < want) return fail(EA_ERR_WORKSPACE, "dump buffers need %zu elements, %zu given", want, dump_elems);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(EA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  ea::decode_bind_workspace(a, workspace);
  a.o = nullptr;
  a.lse = nullptr;
  a.dump_k = (uint16_t*)dump_k;
  a.dump_v = (uint16_t*)dump_v;
  a.dump_t = max_pages_per_seq * page_size;
  return hip_status(ea::launch_decode_gather_dump(a, (hipStream_t)stream), "decode gather dump launch");
}

size_t ea_decode_noalloc_max_bytes(void) { return ea::kDecodeScratchBytes; }

ea_status ea_attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                       const int* block_table, const int* seq_lens, void* o, float* lse, int B,
                                       int Hq, int Hkv, int d, int page_size, int num_pages,
                                       int max_pages_per_seq, float scale, int num_splits, void* stream) {
  ea::DecodeArgs a;
  size_t need = 0;
  if (ea_status st = decode_args(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, Hq, Hkv, d, page_size,
                                 num_pages, max_pages_per_seq, scale, num_splits, a, need);
      st != EA_OK)
    return st;
  if (need > ea::kDecodeScratchBytes)
    return fail(EA_ERR_UNSUPPORTED,
                "allocation-free decode: its partials need %zu bytes, above the library's fixed %zu "
                "(use ea_attn_decode_paged with a workspace)",
                need, ea::kDecodeScratchBytes);
  void* scratch = nullptr;
  if (ea_status st = hip_status(ea::decode_scratch(&scratch), "decode scratch lookup"); st != EA_OK) return st;
  ea::decode_bind_workspace(a, scratch);
  return hip_status(ea::launch_decode(a, (hipStream_t)stream), "allocation-free paged decode launch");
}

}  // extern "C"
