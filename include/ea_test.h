/*
 * ea_test.h -- test-only entry points of libexactattn.so.
 *
 * They run the library's own device functions on caller data so unit tests can
 * check them in isolation. Not part of the attention API; no stability promise.
 */
#ifndef EXACT_ATTENTION_EA_TEST_H
#define EXACT_ATTENTION_EA_TEST_H

#include <stddef.h>

#include "ea.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * ea_test_exp2 -- y[i] = 2^x[i] with the forward kernels' exponential:
 *   mode EA_EXP_HW (v_exp_f32) or EA_EXP_POLY (range reduction + cubic, inputs
 *   clamped at -127; "FlashAttention4 close reading", section 3.1.3).
 *   x, y: device float arrays of n elements (n >= 0). stream: hipStream_t.
 */
ea_status ea_test_exp2(const float* x, float* y, int n, int mode, void* stream);

/*
 * ea_test_mfma_loop -- calibration of the bf16 matrix-core rate: blocks
 * workgroups of 8 waves each issue iters x 16 v_mfma_f32_32x32x16_bf16 (32768
 * FLOP each) from register operands into four independent accumulators, with
 * no memory traffic. FLOPs per launch = blocks * 8 * iters * 16 * 32768.
 *   out: device float array of blocks * 512 elements (written, one value per
 *   lane, meaningless beyond keeping the work alive). 0 < blocks <= 65536,
 *   iters > 0; otherwise EA_ERR_INVALID.
 */
ea_status ea_test_mfma_loop(float* out, int blocks, int iters, void* stream);

/*
 * ea_test_mfma_loop_data -- the same calibration with operands that change
 * from one MFMA to the next, as in a real contraction: each of the 512 threads
 * of a workgroup reads 8 operand pairs once from operands (thread t at byte
 * t * 8 * 2 * P, pair j = (A, B) at 2 j P and (2 j + 1) P, P = 16 bytes for
 * fmt 0, 32 for fmt 1) and each MFMA takes the next pair. fmt 0:
 * v_mfma_f32_32x32x16_bf16, 32768 FLOP each; fmt 1:
 * v_mfma_scale_f32_32x32x64_f8f6f4 with OCP e4m3 operands and unit e8m0
 * scales, 131072 FLOP each. blocks workgroups of 8 waves issue iters x 16
 * MFMAs each: FLOPs per launch = blocks * 8 * iters * 16 * (FLOP per MFMA).
 * With random operands the matrix cores draw more power than with the fixed
 * operands of ea_test_mfma_loop, and under the device's power limit the rate
 * is what a contraction on such data can sustain.
 *   operands: device buffer of at least ea_test_mfma_loop_data_bytes(fmt)
 *   bytes (EA_ERR_WORKSPACE otherwise); out: device float array of blocks *
 *   512 elements (one value per lane). EA_ERR_INVALID for null pointers,
 *   blocks outside 1..65536, iters <= 0 or fmt not 0/1.
 * ea_test_mfma_loop_data_bytes returns that size (0 for a bad fmt).
 */
size_t ea_test_mfma_loop_data_bytes(int fmt);
ea_status ea_test_mfma_loop_data(const void* operands, size_t operands_bytes, float* out, int blocks, int iters,
                                 int fmt, void* stream);

/*
 * ea_test_stream_read -- calibration of the HBM read rate: blocks workgroups
 * of 256 threads read the device buffer buf once, 16 bytes per load, 16 loads
 * in flight per thread (grid-stride, non-temporal), and fold it into one value
 * per thread. Bytes read per launch = bytes.
 *   out: device int array of blocks * 256 elements (written, meaningless
 *   beyond keeping the reads alive). 0 < blocks <= 65536 and bytes a positive
 *   multiple of 65536 * blocks (one grid pass); otherwise EA_ERR_INVALID.
 */
ea_status ea_test_stream_read(const void* buf, size_t bytes, int* out, int blocks, void* stream);

/*
 * ea_test_pair_probe -- calibration of two waves sharing one SIMD, the pairing
 * the forward kernels are built on. blocks workgroups of 8 waves (one per CU:
 * each declares 96 KB of LDS) run: waves 0-3 role_a, waves 4-7 role_b (wave
 * w and w + 4 share a SIMD). Each wave repeats one iteration of its role until
 * budget shader-clock cycles (s_memtime) have passed and writes
 * out[2 (8 b + w)] = iterations done, out[2 (8 b + w) + 1] = cycles taken.
 * Roles (one iteration): EA_PROBE_IDLE (the wave exits), EA_PROBE_MFMA_REG
 * (32 v_mfma_f32_32x32x16_bf16 from registers), EA_PROBE_MFMA_LDS (the
 * forward's product part: 16 MFMAs fed by ds_read_b128, 16 by two
 * ds_read_b64_tr_b16 each), EA_PROBE_SOFTMAX (the forward's softmax of a
 * 64-key step on 32 scores per lane), EA_PROBE_EXP (32 independent v_exp_f32),
 * EA_PROBE_FMA (32 independent v_fma_f32), EA_PROBE_MFMA_AGPR (MFMA_REG with
 * AGPR accumulators), EA_PROBE_MFMA_LDS_PRIO (MFMA_LDS at raised wave
 * priority), EA_PROBE_MIX (8 MFMAs from registers interleaved one by one with
 * 2 v_exp_f32 and 2 v_fma_f32 each), EA_PROBE_LDS_B128 (8 ds_read_b128 of an
 * 8 KB operand tile, then a wait), EA_PROBE_LDS_TR (16 ds_read_b64_tr_b16 of
 * an 8 KB transposed operand tile, then a wait), EA_PROBE_MFMA_LDS_DEEP
 * (MFMA_LDS with 14 operand reads issued ahead instead of 6),
 * EA_PROBE_MFMA_LDS_ALT (MFMA_LDS with S and P V products alternating),
 * EA_PROBE_FUSED32 (a 32-key step whose 16 LDS-fed MFMAs are interleaved
 * with the softmax of an independent 32-key score tile, in one wave).
 *   out: device int64 array of 16 * blocks elements. 0 < blocks <= 4096,
 *   0 < budget <= 2^32, roles in range; otherwise EA_ERR_INVALID.
 */
/*
 * ea_test_fwd_rescale_stats -- the library's default dense forward (the
 * persistent ping-pong kernel, d = 128, hardware exponential, bf16 in the
 * layouts of ea_attn_fwd) with lazy-rescale threshold rescale_log2 ("the
 * conditional softmax rescaling" of "FlashAttention-4: algorithm-pipeline
 * co-design for Blackwell": rescale the accumulator only when the running row
 * max grows by more than that many powers of two), which also writes, for
 * every work tile t (256 query rows of one (batch, head); tile index as the
 * kernel numbers them) and wave w (0..7, 32 rows each):
 *   stats[4 (8 t + w)]     = steps (64-key tiles) in which the wave saw keys,
 *   stats[4 (8 t + w) + 1] = steps in which it rescaled (its running max grew
 *                            by more than the threshold for some row, or
 *                            it met its first keys),
 *   stats[4 (8 t + w) + 2] = shader clock cycles (s_memtime) of the tile's
 *                            step loop on that wave,
 *   stats[4 (8 t + w) + 3] = wall clock ticks (s_memrealtime, at the rate
 *                            ea_test_wall_clock_khz reports) of the same loop;
 *                            their ratio is the shader clock under this load.
 * o and lse are written as by ea_attn_fwd, bit for bit. stats: device int32
 * array of at least ea_test_fwd_rescale_stats_len(B, Nq, Hq) elements (padding
 * tiles keep their contents). Errors as for ea_attn_fwd; EA_ERR_WORKSPACE
 * when stats_len is short.
 */
size_t ea_test_fwd_rescale_stats_len(int B, int Nq, int Hq);
/*
 * ea_test_varlen_lds_order -- the heaviest-first order that the ping-pong
 * forward's workgroups compute for themselves when ea_attn_fwd_varlen gets no
 * order ("FlashAttention4 close reading", section 3.3: weight = 64-key tiles
 * of a sequence's last 256-row block, heaviest first, equal weights in input
 * order), computed by one workgroup with the forward's own device code.
 *   order: device int32 [num_seqs], written: order[v] = actual sequence.
 *   EA_ERR_INVALID for null pointers, num_seqs <= 0 or causal not 0/1;
 *   EA_ERR_UNSUPPORTED for num_seqs > 512 (the forward then keeps the input
 *   order).
 */
ea_status ea_test_varlen_lds_order(const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs, int causal,
                                   int* order, void* stream);

/*
 * ea_test_fwd_phase_cycles -- the default dense forward of ea_test_fwd_rescale_stats
 * (persistent ping-pong, d = 128, lazy-rescale threshold 2^8) with a shader-
 * clock stamp (s_memtime, read with an immediate wait) at every phase edge,
 * adding per wave of each of its workgroups (one per CU, 8 waves each):
 *   cycles[8 (8 g + w) + 0] MFMA parts (issue of S = K Q^T and O += V P),
 *                       + 1 waits at the barriers after them,
 *                       + 2 VALU parts (softmax; waves 0-3 also issue the K/V DMA),
 *                       + 3 waits at the barriers after those,
 *                       + 4 tile prologues (tile start to the first step),
 *                       + 5 tile epilogues (last step to the output stores issued),
 *                       + 6 steps, + 7 tiles.
 * With two waves per SIMD, a wave's MFMA part runs beside the other group's
 * VALU part. o and lse are written as by ea_attn_fwd; the stamps make the
 * launch a few per cent slower. cycles: device array of at least
 * ea_test_fwd_phase_cycles_len(B, Nq, Hq) entries (EA_ERR_WORKSPACE otherwise),
 * cleared by the call (hipMemsetAsync) before it adds. Other errors as for
 * ea_test_fwd_rescale_stats. ea_test_fwd_phase_cycles_len returns 0 for
 * non-positive sizes or when the CU count is unavailable.
 */
size_t ea_test_fwd_phase_cycles_len(int B, int Nq, int Hq);
ea_status ea_test_fwd_phase_cycles(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Nq,
                                   int Nk, int Hq, int Hkv, int causal, float scale, unsigned long long* cycles,
                                   size_t cycles_len, void* stream);

/*
 * ea_test_fwd_tiles / ea_test_fwd_tile_order -- the work order of the dense
 * bf16 forward ("FlashAttention4 close reading", section 3.3: the cache-aware
 * hierarchical LPT traversal). ea_test_fwd_tiles returns the number of work
 * tiles of the per-tile launch (0 for non-positive sizes);
 * ea_test_fwd_tile_order writes, for every tile t in dispatch order (t = 8 j
 * + XCD), out[3 t .. 3 t + 2] = (batch, head, 256-row block), or -1s for a
 * padding entry, computed by the kernels' own tile-location code. out: device
 * int32 array of at least 3 ea_test_fwd_tiles(B, Nq, Hq) elements
 * (EA_ERR_WORKSPACE otherwise); EA_ERR_INVALID for a null out, non-positive
 * sizes or causal not 0/1; EA_ERR_UNSUPPORTED for B * N >= 2^31.
 */
size_t ea_test_fwd_tiles(int B, int Nq, int Hq);
ea_status ea_test_fwd_tile_order(int B, int Nq, int Nk, int Hq, int causal, int* out, size_t out_len, void* stream);
/*
 * ea_test_decode_gather -- the page-gather dump of the paged decode ("Faster,
 * more flexible FlashAttention-4 for LLM inference", PR 1999/2104 sections:
 * token t of sequence b lives in page block_table[b, t / page_size], slot
 * t % page_size). Runs the decode's split kernel on the arguments of
 * ea_attn_decode_paged (q, caches, block table, lengths, sizes, num_splits,
 * workspace) and, besides its partials, writes every K and V row it gathers
 * for a chunk to dump_k / dump_v, dense [B, max_pages_per_seq * page_size,
 * Hkv, d] bf16 at (sequence, token, KV head), through the same loads the
 * decode uses: tokens at or past a sequence's (clamped) length are not
 * written; rows of page indices outside [0, num_pages) read as zeros.
 * dump_elems: the capacity of each dump buffer in elements (EA_ERR_WORKSPACE
 * when short); other errors as for ea_attn_decode_paged.
 */
ea_status ea_test_decode_gather(const void* q, const void* k_cache, const void* v_cache, const int* block_table,
                                const int* seq_lens, int B, int Hq, int Hkv, int d, int page_size, int num_pages,
                                int max_pages_per_seq, int num_splits, void* dump_k, void* dump_v,
                                size_t dump_elems, void* workspace, size_t workspace_bytes, void* stream);
/*
 * ea_test_wall_clock_khz -- *khz = the rate of the device's constant wall
 * clock counter (s_memrealtime) for HIP device `device`, in kHz. EA_ERR_INVALID
 * for a null khz, EA_ERR_HIP if the runtime cannot answer.
 */
ea_status ea_test_wall_clock_khz(int device, int* khz);
ea_status ea_test_fwd_rescale_stats(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                    int Nq, int Nk, int Hq, int Hkv, int causal, float scale, float rescale_log2,
                                    int* stats, size_t stats_len, void* stream);

enum {
  EA_PROBE_IDLE = 0,
  EA_PROBE_MFMA_REG = 1,
  EA_PROBE_MFMA_LDS = 2,
  EA_PROBE_SOFTMAX = 3,
  EA_PROBE_EXP = 4,
  EA_PROBE_FMA = 5,
  EA_PROBE_MFMA_AGPR = 6,
  EA_PROBE_MFMA_LDS_PRIO = 7,
  EA_PROBE_MIX = 8,
  EA_PROBE_LDS_B128 = 9,
  EA_PROBE_LDS_TR = 10,
  EA_PROBE_MFMA_LDS_DEEP = 11,
  EA_PROBE_MFMA_LDS_ALT = 12,
  EA_PROBE_FUSED32 = 13
};
ea_status ea_test_pair_probe(long long* out, int blocks, int role_a, int role_b, long long budget, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* EXACT_ATTENTION_EA_TEST_H */
