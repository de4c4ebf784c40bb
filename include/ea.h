/*
 * ea.h -- C ABI of libexactattn.so, exact attention for AMD MI355X (gfx950).
 *
 * What is computed (cited by page title and section):
 *   O = softmax(scale * Q K^T) V  and the per-row natural log-sum-exp
 *   lse_i = log sum_j exp(scale * q_i . k_j), exactly (no approximation beyond
 *   floating-point rounding order) -- "FlashAttention: not less compute, less
 *   data movement", sections 01 (the formula), 02 (the online-softmax
 *   recurrence the kernels use) and 03 (the forward keeps O and the row
 *   log-sum-exp, never the N x N score matrix).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers allocated by the caller, who owns
 *     them. The library allocates nothing and keeps no per-call state.
 *   - bf16 tensors are raw IEEE bfloat16 bit patterns (uint16 storage).
 *   - Dense Q/K/V/O are contiguous BSHD: element (b, n, h, c) lives at
 *     ((b * N + n) * H + h) * d + c. Packed variable-length tensors are THD:
 *     (t, h, c) at (t * H + h) * d + c.
 *   - Grouped-query attention: Hq must be a multiple of Hkv; query head h reads
 *     KV head h / (Hq / Hkv) (consecutive groups; "FlashAttention: not less
 *     compute, less data movement", section 05 requires only divisibility).
 *   - causal = 1 masks key j for query i when j > i + (Nk - Nq) (bottom-right
 *     alignment; identical to j > i when Nq == Nk).
 *   - A query row with no allowed key yields o = 0 and lse = -inf.
 *   - stream is a hipStream_t (NULL = the default stream). Work is enqueued on
 *     it; calls never synchronise. Device faults surface at the caller's next
 *     synchronisation.
 *   - Argument checks run on the host before any HIP call: on failure nothing
 *     is launched, the status is returned and ea_last_error() describes it.
 */
#ifndef EXACT_ATTENTION_EA_H
#define EXACT_ATTENTION_EA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  EA_OK = 0,
  EA_ERR_INVALID = -1,      /* null pointer, non-positive size, Hq % Hkv, bad scale */
  EA_ERR_UNSUPPORTED = -2,  /* valid but not built: head dim, page size, ... */
  EA_ERR_HIP = -3,          /* a HIP launch failed */
  EA_ERR_WORKSPACE = -4     /* caller's workspace too small */
} ea_status;

/* Softmax exponential used by the forward kernels.
 *   EA_EXP_HW     the hardware v_exp_f32.
 *   EA_EXP_POLY   range reduction 2^x = 2^floor(x) * 2^frac(x) with a cubic
 *                 polynomial for 2^frac on [0,1) and the integer part added to
 *                 the exponent field; inputs clamped at -127
 *                 ("FlashAttention-4: algorithm-pipeline co-design for
 *                 Blackwell", hybrid exponent section; "FlashAttention4 close
 *                 reading", section 3.1.3).
 *   EA_EXP_HYBRID a fixed fraction of each score tile takes the polynomial,
 *                 the rest the hardware unit (same sections). */
enum { EA_EXP_HW = 0, EA_EXP_POLY = 1, EA_EXP_HYBRID = 2 };

/* Forward tuning knobs (results differ only by rounding). */
typedef struct {
  int exp_mode;            /* EA_EXP_*; default EA_EXP_HW */
  float rescale_log2;      /* lazy rescale: rescale the accumulator only when the
                              running row max grows by more than this many
                              powers of two ("FlashAttention-4: ... co-design",
                              conditional softmax rescaling section; reading: a
                              factor of 256, i.e. 8.0). 0 = rescale on every
                              increase. Must be in [0, 16]. Default 8.0. */
  int natural_order;       /* 0 (default): causal tiles heaviest first; 1: tiles
                              in ascending row-block order. */
  int kernel;              /* EA_FWD_KERNEL_*: which forward kernel runs.
                              Default EA_FWD_KERNEL_AUTO. */
} ea_fwd_tuning;

/* Forward kernels (same results up to rounding order):
 *   EA_FWD_KERNEL_AUTO      for d_qk = 128 or 192 the ping-pong kernel, in
 *                           persistent form for dense inputs; for d = 64 the
 *                           4-wave one
 *   EA_FWD_KERNEL_4WAVE     4 waves x 32 query rows, two workgroups per CU
 *   EA_FWD_KERNEL_PINGPONG  8 waves x 32 rows in two groups that alternate
 *                           matrix products and softmax on each SIMD
 *   EA_FWD_KERNEL_PIPELINED MX fp8 forward only (ea_attn_fwd_mx8_tuned): 8
 *                           waves x 32 rows, each wave overlapping the softmax
 *                           of one tile with its own matrix products of the
 *                           next and previous tiles; the bf16 entry points
 *                           return EA_ERR_UNSUPPORTED for it
 *   EA_FWD_KERNEL_PERSISTENT the ping-pong kernel in persistent form: one
 *                           workgroup per CU walks a static, load-balanced
 *                           list of row blocks instead of one workgroup per
 *                           row block (the pages' persistent tile scheduler,
 *                           "FlashAttention4 close reading", section 3.3)
 *   EA_FWD_KERNEL_UNROLL_KV the persistent form with the K/V pipeline running
 *                           on across row blocks: the first S of the next
 *                           block is computed with the last O += V P of the
 *                           current one (the unroll-KV schedule of
 *                           "Low-precision FlashAttention-4: end-to-end
 *                           block-scaled attention for Blackwell", section
 *                           2.1.2); bitwise the results of the ping-pong
 *                           kernel; (d_qk, d_v) = (64, 64) and (128, 128) only */
enum {
  EA_FWD_KERNEL_AUTO = 0,
  EA_FWD_KERNEL_4WAVE = 1,
  EA_FWD_KERNEL_PINGPONG = 2,
  EA_FWD_KERNEL_PIPELINED = 3,
  EA_FWD_KERNEL_PERSISTENT = 4,
  EA_FWD_KERNEL_UNROLL_KV = 5
};

/* Default tuning values. */
void ea_fwd_tuning_default(ea_fwd_tuning* t);

/*
 * ea_attn_fwd -- fused exact attention forward, bf16 in, bf16 O + fp32 LSE out.
 *   q   [B, Nq, Hq, d] bf16        k, v [B, Nk, Hkv, d] bf16
 *   o   [B, Nq, Hq, d] bf16 (written)
 *   lse [B, Hq, Nq] fp32 (written; natural log, scale included), or NULL
 *   d in {64, 128}; scale finite and > 0 (usually 1/sqrt(d)).
 * One pass: each row block of queries streams over K/V tiles with the online
 * softmax, so the N x N matrix never reaches HBM ("FlashAttention: not less
 * compute, less data movement", sections 02-03).
 */
ea_status ea_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal,
                      float scale, void* stream);

/* ea_attn_fwd with explicit tuning (NULL = defaults). */
ea_status ea_attn_fwd_tuned(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal,
                            float scale, const ea_fwd_tuning* tuning, void* stream);

/*
 * ea_attn_fwd_hd -- ea_attn_fwd_tuned with separate head dims for the scores
 * and the values: q [B, Nq, Hq, d_qk], k [B, Nk, Hkv, d_qk], v [B, Nk, Hkv,
 * d_v], o [B, Nq, Hq, d_v]. (d_qk, d_v) is (64, 64), (128, 128) or (192, 128),
 * the last being the non-standard pair "FlashAttention-4: algorithm-pipeline
 * co-design for Blackwell" (kernel-level performance section) benchmarks for
 * the DeepSeek V3 architecture; other pairs return EA_ERR_UNSUPPORTED.
 * (192, 128) runs on the ping-pong kernel only (tuning->kernel AUTO,
 * PINGPONG or PERSISTENT). The usual scale is 1/sqrt(d_qk).
 */
ea_status ea_attn_fwd_hd(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Nq, int Nk, int Hq, int Hkv, int d_qk, int d_v, int causal,
                         float scale, const ea_fwd_tuning* tuning, void* stream);
/*
 * ea_attn_fwd_varlen -- packed variable-length sequences (THD layout).
 *   q [total_q, Hq, d], k/v [total_k, Hkv, d], o [total_q, Hq, d] bf16
 *   lse [Hq, total_q] fp32 or NULL
 *   cu_seqlens_q / cu_seqlens_k: device int32 [num_seqs + 1], nondecreasing,
 *   starting at 0 and ending at total_q / total_k; sequence s owns rows
 *   [cu[s], cu[s+1]); positions and the causal mask are local to each
 *   sequence. max_seqlen_q must bound every query length (it sizes the grid).
 *   Rows outside every sequence are neither read nor written.
 * Packing without padding follows the unpadded-batch advice in "FlashAttention:
 * not less compute, less data movement", section 05.
 * Work order: when the batch has fewer (sequence, head) groups than the GPU
 * has CUs and at most 512 sequences, the default kernels (d = 128; 8-wave
 * ping-pong) visit the sequences heaviest first (the order of
 * ea_varlen_lpt_order, computed by each workgroup in its LDS), so the longest
 * sequences' tiles start first; otherwise in input order. The results do not
 * depend on the order.
 */
ea_status ea_attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                             const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs,
                             int total_q, int total_k, int max_seqlen_q, int Hq, int Hkv, int d,
                             int causal, float scale, const ea_fwd_tuning* tuning, void* stream);

/*
 * ea_varlen_lpt_order -- the varlen batch order of "FlashAttention4 close
 * reading", section 3.3 (scheduling): a preprocessing step weighs each
 * sequence by its heaviest work tile -- the number of 64-key tiles in the
 * main loop of its last block of block_m query rows (causal: keys up to that
 * block's last row, bottom-right aligned; non-causal: all keys; 0 without
 * queries) -- and sorts the sequences by weight, heaviest first, equal
 * weights in input order. No data moves: the result is a permutation.
 *   cu_seqlens_q / cu_seqlens_k: device int32 [num_seqs + 1], as for the
 *     varlen forward.
 *   block_m: 256 for the 8-wave forward kernels (the default for d = 128),
 *     128 for the 4-wave kernel; any of the two gives a valid order.
 *   weights: device int32 [num_seqs], written (the weights above).
 *   order: device int32 [num_seqs], written: order[v] = the actual sequence
 *     at virtual position v.
 * Both buffers belong to the caller. Enqueued on stream; the ranking is a
 * quadratic count spread over num_seqs threads, so num_seqs <= 65536
 * (EA_ERR_UNSUPPORTED beyond). Lengths are read on the device, so every layer
 * of a model that shares cu_seqlens can reuse one order.
 */
ea_status ea_varlen_lpt_order(const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs, int causal,
                              int block_m, int* weights, int* order, void* stream);

/*
 * ea_attn_fwd_varlen_ordered -- ea_attn_fwd_varlen whose workgroups visit the
 * sequences in the order given by seq_order (device int32 [num_seqs],
 * order[v] = actual sequence; NULL = input order), e.g. from
 * ea_varlen_lpt_order. The results do not depend on the order. seq_order
 * must be a permutation of 0..num_seqs-1: an entry outside that range
 * contributes no rows, and a sequence listed twice is computed twice.
 */
ea_status ea_attn_fwd_varlen_ordered(const void* q, const void* k, const void* v, void* o, float* lse,
                                     const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs,
                                     int total_q, int total_k, int max_seqlen_q, int Hq, int Hkv, int d,
                                     int causal, float scale, const int* seq_order,
                                     const ea_fwd_tuning* tuning, void* stream);

/*
 * ea_attn_fwd_mx8 -- forward with MX-scaled FP8 (OCP e4m3) inputs.
 *   q8, k8, v8     [B, N, H*, d] e4m3 codes (uint8)
 *   q_scale, k_scale [B, H*, N, d/32] e8m0 scale bytes (2^(s-127)), one per 32
 *                  consecutive elements along d; head-major, so the scales of
 *                  a tile of rows of one head are contiguous;
 *   v_scale        [B, N/32, Hkv, d] e8m0, one per 32 consecutive keys
 *                  (the contraction dimension of P V) -- "Low-precision
 *                  FlashAttention-4: end-to-end block-scaled attention for
 *                  Blackwell", section 2.1.
 *   P is re-quantised to e4m3 before the P V product (same page, 2.1.3).
 *   o [B, N, Hq, d] bf16, lse [B, Hq, N] fp32 or NULL. N % 32 == 0, d == 128.
 */
ea_status ea_attn_fwd_mx8(const void* q8, const void* k8, const void* v8,
                          const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                          void* o, float* lse, int B, int N, int Hq, int Hkv, int d, int causal,
                          float scale, void* stream);

/*
 * ea_attn_fwd_mx8_tuned -- ea_attn_fwd_mx8 with forward tuning (NULL = the
 * defaults). tuning->kernel selects EA_FWD_KERNEL_4WAVE,
 * EA_FWD_KERNEL_PINGPONG (8 waves in two groups alternating the scaled
 * products and the softmax, as the bf16 ping-pong kernel), EA_FWD_KERNEL_PERSISTENT
 * (that kernel with one workgroup per CU; AUTO: this form) or
 * EA_FWD_KERNEL_PIPELINED (8 waves, each interleaving its own products and
 * softmax). The per-tile forms take the causal row blocks heaviest first;
 * the persistent form takes a (batch, head)'s row blocks in ascending order
 * (its snake walk pairs light and heavy blocks on each workgroup either way;
 * ascending, a head whose row blocks outnumber its XCD's workgroups rereads
 * fewer keys from HBM). EA_FWD_KERNEL_UNROLL_KV,
 * exp_mode other than EA_EXP_HW and natural_order = 1 return
 * EA_ERR_UNSUPPORTED. rescale_log2 is the lazy-rescale threshold, which also
 * bounds P before its e4m3 rounding (P <= 2^rescale_log2): values above 8.807
 * (log2 448, e4m3's largest finite value, rounded down) return
 * EA_ERR_UNSUPPORTED.
 */
ea_status ea_attn_fwd_mx8_tuned(const void* q8, const void* k8, const void* v8,
                                const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                                void* o, float* lse, int B, int N, int Hq, int Hkv, int d, int causal,
                                float scale, const ea_fwd_tuning* tuning, void* stream);

/*
 * Backward of the dense bf16 forward ("Low-precision FlashAttention-4:
 * end-to-end block-scaled attention for Blackwell", section 2.2, lists its
 * five products; "FlashAttention-4: algorithm-pipeline co-design for
 * Blackwell", backward sections): for the output gradient dout it writes
 *   dq = scale dS K,  dk = scale dS^T Q,  dv = P^T dout,
 * with P = softmax(scale Q K^T) recomputed from lse, dP = dout V^T and
 * dS = P (dP - rowsum(dout * o)). GQA: dk / dv of a KV head sum over the query
 * heads that read it. Deterministic: every output element is written once by
 * one workgroup, in a fixed order (no atomics), so repeated calls give the
 * same bits.
 *   q, o, dout, dq [B, Nq, Hq, d] bf16; k, v, dk, dv [B, Nk, Hkv, d] bf16
 *     (dq, dk, dv written);
 *   lse [B, Hq, Nq] fp32: the forward's log-sum-exp (natural log, scale
 *     included), as ea_attn_fwd writes it; rows with no allowed key (lse =
 *     -inf) get dq = 0;
 *   d in {64, 128}; causal / scale as for the forward that produced o and lse;
 *   workspace: device memory of at least ea_attn_bwd_workspace_size(B, Hq, Nq)
 *     bytes (per-row statistics), owned by the caller, contents ignored.
 */
size_t ea_attn_bwd_workspace_size(int B, int Hq, int Nq);
/* Work schedule of the backward kernels (results bitwise identical):
 *   EA_BWD_SCHEDULE_AUTO       the library's choice (one workgroup per tile);
 *   EA_BWD_SCHEDULE_PER_TILE   one workgroup per work tile;
 *   EA_BWD_SCHEDULE_PERSISTENT one workgroup per CU (two for the dQ kernel)
 *                              walking a load-balanced static tile list. */
enum { EA_BWD_SCHEDULE_AUTO = 0, EA_BWD_SCHEDULE_PER_TILE = 1, EA_BWD_SCHEDULE_PERSISTENT = 2 };
/* ea_attn_bwd with an explicit schedule (anything else is EA_ERR_INVALID). */
ea_status ea_attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv, int B, int Nq, int Nk, int Hq, int Hkv,
                         int d, int causal, float scale, int schedule, void* workspace, size_t workspace_bytes,
                         void* stream);
ea_status ea_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, int B, int Nq, int Nk, int Hq, int Hkv,
                      int d, int causal, float scale, void* workspace, size_t workspace_bytes, void* stream);
/* FP8 element formats of the MX inputs (OCP FP8): e4m3 = 4 exponent bits
 * (bias 7), 3 mantissa bits, largest finite 448, no infinities; e5m2 = 5
 * exponent bits (bias 15), 2 mantissa bits, largest finite 57344, with
 * infinities. "Faster, more flexible FlashAttention-4 for LLM inference", PR
 * 2109, accepts both for the attention inputs. */
enum { EA_FP8_E4M3 = 0, EA_FP8_E5M2 = 1 };
/*
 * ea_attn_fwd_mx8_fmt -- ea_attn_fwd_mx8_tuned with the element format of the
 * q8 / k8 / v8 codes given by in_format (EA_FP8_E4M3 or EA_FP8_E5M2; anything
 * else is EA_ERR_INVALID). Scales, layouts, tuning and outputs are those of
 * ea_attn_fwd_mx8_tuned; P is re-quantised to e4m3 in both cases (P <=
 * 2^rescale_log2, which the rescale_log2 <= 8.807 bound keeps within e4m3's
 * 448).
 */
ea_status ea_attn_fwd_mx8_fmt(const void* q8, const void* k8, const void* v8,
                              const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                              void* o, float* lse, int B, int N, int Hq, int Hkv, int d, int causal,
                              float scale, int in_format, const ea_fwd_tuning* tuning, void* stream);
/*
 * Paged split-KV decode ("Faster, more flexible FlashAttention-4 for LLM
 * inference": PR 1999/2104 for KV pages of any size, PR 1940 for splitting the
 * KV sequence over workgroups plus a combine kernel, PR 1993 for one query tile
 * per workgroup, PR 2186 for packing the query heads of one KV head together,
 * for any ratio Hq / Hkv).
 *
 *   q      [B, Hq, d] bf16 (one query token per sequence)
 *   k_cache, v_cache [num_pages, page_size, Hkv, d] bf16
 *   block_table [B, max_pages_per_seq] int32: token t of sequence b lives in
 *          page block_table[b, t / page_size], slot t % page_size; entries past
 *          the sequence's last page are never read; an entry outside
 *          [0, num_pages) reads as zeros (no fault).
 *   seq_lens [B] int32, each in [0, max_pages_per_seq * page_size] (larger
 *          values are clamped to that capacity)
 *   o      [B, Hq, d] bf16 (written); lse [B, Hq] fp32 or NULL
 *   page_size >= 1 (every size takes the same token-by-token load path).
 *          The arithmetic follows the logical token order
 *          only, so the same tokens give bitwise the same output whatever the
 *          page size and page placement. d == 128; any Hq that is a multiple
 *          of Hkv; num_pages * page_size < 2^31.
 *   num_splits: the batch's KV tokens, taken in 32-token chunks and laid end
 *          to end over the sequences, are cut into num_splits equal ranges, one
 *          workgroup (of up to 8 KV heads, or blocks of 16 query heads) each; a sequence is split wherever a
 *          range boundary falls in it. 0 = one workgroup per CU (256 over the
 *          groups of 8 (KV head, block of 16 of its query heads) pairs). At
 *          most 65536.
 *   workspace: device memory of at least ea_decode_workspace_size(B, Hq, Hkv,
 *          d, max_pages_per_seq * page_size, page_size, num_splits) bytes
 *          (it depends on B, Hq, d and the range count only), owned by the
 *          caller; contents on entry are ignored.
 * The decode attends to all seq_lens[b] tokens (no mask).
 */
size_t ea_decode_workspace_size(int B, int Hq, int Hkv, int d, int max_seqlen, int page_size,
                                int num_splits);

ea_status ea_attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                               const int* block_table, const int* seq_lens, void* o, float* lse,
                               int B, int Hq, int Hkv, int d, int page_size, int num_pages,
                               int max_pages_per_seq, float scale, int num_splits,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * ea_attn_decode_paged_noalloc -- ea_attn_decode_paged without a workspace,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). Arguments,
 * layouts, results and errors are those of ea_attn_decode_paged minus the
 * workspace. The split partials and the plan live in a device array of
 * ea_decode_noalloc_max_bytes() bytes (16 MiB) inside the library, one per
 * GPU it runs on, held until the process ends; a call whose partials need more
 * (ea_decode_workspace_size above that size) returns EA_ERR_UNSUPPORTED
 * before any launch. Nothing is allocated per call. The array holds no state
 * between calls that a later call reads (it is rewritten before use), but every
 * call on one GPU uses the same array: calls that may overlap on one GPU (other
 * streams, other threads) race and give wrong results, so serialise them.
 */
size_t ea_decode_noalloc_max_bytes(void);
ea_status ea_attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                       const int* block_table, const int* seq_lens, void* o, float* lse, int B,
                                       int Hq, int Hkv, int d, int page_size, int num_pages,
                                       int max_pages_per_seq, float scale, int num_splits, void* stream);

/* Human-readable description of the last failure on the calling thread
 * (thread-local; valid until the next library call on that thread). */
const char* ea_last_error(void);

/* Library ABI version (this header: 1). */
int ea_version(void);

#ifdef __cplusplus
}
#endif
#endif /* EXACT_ATTENTION_EA_H */
