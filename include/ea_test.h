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
 * ea_test_stream_read -- calibration of the HBM read rate: blocks workgroups
 * of 256 threads read the device buffer buf once, 16 bytes per load, 16 loads
 * in flight per thread (grid-stride, non-temporal), and fold it into one value
 * per thread. Bytes read per launch = bytes.
 *   out: device int array of blocks * 256 elements (written, meaningless
 *   beyond keeping the reads alive). 0 < blocks <= 65536 and bytes a positive
 *   multiple of 65536 * blocks (one grid pass); otherwise EA_ERR_INVALID.
 */
ea_status ea_test_stream_read(const void* buf, size_t bytes, int* out, int blocks, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* EXACT_ATTENTION_EA_TEST_H */
