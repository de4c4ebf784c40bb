"""GPU parity of the bf16 attention backward against the fp64 oracle.

The backward consumes what the forward produced: q, k, v, the forward's bf16
output o and fp32 lse (from ea.attn_fwd on the same inputs), and an output
gradient dout drawn iid N(0,1) and rounded to bf16. The oracle computes dq, dk,
dv from q, k, v, dout alone (full-row softmax in fp64).

Tolerance (per (batch, head) slice of each gradient), from the bf16 steps of
the computation, each a relative rounding of at most u = 2^-9: the kernel
rounds P and dS to bf16 as MFMA operands (independent errors of u per term
of a sum over up to N keys or rows, which average out), takes D =
rowsum(dout * o) from the forward's bf16 o (one more u on every dS term of a
row, the same sign across the row), and stores bf16 (u per element). The
criteria allow about 2.5 u normwise, ||g - g_ref||_F <= 5e-3 ||g_ref||_F, and
elementwise |g - g_ref| <= 4 u max|g_ref| + 2 u |g_ref| (the first term
covers the summed operand roundings, which scale with the slice, not the
element; the second the output rounding and the D error).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _helpers import dev_bf16, f64, host_bits, log

pytestmark = pytest.mark.gpu

U = 2.0 ** -9       # bf16 unit roundoff
NORM_TOL = 5e-3
ELEM_ABS = 4 * U    # times max |g_ref| over the slice
ELEM_REL = 2 * U    # times |g_ref|


def run_bwd(inp, do_bits, schedule=0):
    import exact_attention_amd as ea
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    o, lse = ea.attn_fwd(q, k, v, inp.causal, inp.scale)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, dev_bf16(do_bits), lse, inp.causal, inp.scale, schedule=schedule)
    torch.cuda.synchronize()
    return tuple(f64(host_bits(x)) for x in (dq, dk, dv))


def check(got, ref, what):
    """got / ref [B, N, H, d]; per (b, h) slice."""
    B, N, H, d = ref.shape
    worst_n, worst_e = 0.0, 0.0
    for b in range(B):
        for h in range(H):
            g, r = got[b, :, h], ref[b, :, h]
            den = np.linalg.norm(r)
            if den == 0:
                assert np.all(g == 0), f"{what}[b={b},h={h}] should be zero"
                continue
            worst_n = max(worst_n, np.linalg.norm(g - r) / den)
            lim = ELEM_ABS * np.abs(r).max() + ELEM_REL * np.abs(r)
            worst_e = max(worst_e, float(np.max(np.abs(g - r) / lim)))
    log(f"  {what}: normwise {worst_n:.2e}, elementwise {worst_e:.2f} of the bound")
    assert np.isfinite(got).all(), what
    assert worst_n <= NORM_TOL, f"{what}: normwise {worst_n:.3e}"
    assert worst_e <= 1.0, f"{what}: elementwise {worst_e:.2f} of the bound"


SHAPES = [
    # B, Nq, Nk, Hq, Hkv, d, causal
    (1, 256, 256, 2, 2, 128, False),
    (1, 256, 256, 2, 2, 128, True),
    (2, 300, 300, 4, 2, 128, True),      # ragged tail, GQA 2:1
    (1, 77, 77, 2, 2, 64, False),
    (1, 129, 257, 2, 1, 128, True),      # Nq < Nk, bottom-right causal
    (1, 200, 50, 2, 2, 64, True),        # Nq > Nk: leading rows have no key
    (1, 1, 1, 1, 1, 128, True),
    (1, 640, 640, 3, 1, 128, True),      # GQA 3:1, several blocks
    (1, 384, 384, 2, 2, 64, False),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_bwd_shapes(shape):
    B, Nq, Nk, Hq, Hkv, d, causal = shape
    log(f"bwd shape {shape}")
    inp = W.dense(B, Nq, Nk, Hq, Hkv, d, causal, seed=500 + Nq + Nk + d)
    do_bits = W.normal_bf16_bits(500 + Nq, W.STREAM_DO, (B, Nq, Hq, d))
    dq, dk, dv = run_bwd(inp, do_bits)
    rq, rk, rv = oracle.attention_backward(f64(inp.q), f64(inp.k), f64(inp.v), f64(do_bits), causal, inp.scale)
    check(dq, rq, "dq")
    check(dk, rk, "dk")
    check(dv, rv, "dv")


def test_bwd_deterministic():
    inp = W.dense(2, 700, 700, 4, 2, 128, True, seed=530)
    do_bits = W.normal_bf16_bits(530, W.STREAM_DO, (2, 700, 4, 128))
    a = run_bwd(inp, do_bits)
    b = run_bwd(inp, do_bits)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_2k_full():
    """B=1, H=4, N=2048, d=128, causal: every element against the oracle."""
    inp = W.dense(1, 2048, 2048, 4, 4, 128, True, seed=540)
    do_bits = W.normal_bf16_bits(540, W.STREAM_DO, (1, 2048, 4, 128))
    dq, dk, dv = run_bwd(inp, do_bits)
    rq, rk, rv = oracle.attention_backward(f64(inp.q), f64(inp.k), f64(inp.v), f64(do_bits), True, inp.scale)
    check(dq, rq, "dq")
    check(dk, rk, "dk")
    check(dv, rv, "dv")


def test_bwd_prefill_size_heads():
    """The prefill workload's size (B=4, H=16, N=8192, d=128, causal): two
    whole heads against the oracle."""
    inp = W.prefill(True)
    B, N, H, d = inp.q.shape
    do_bits = W.normal_bf16_bits(1002, W.STREAM_DO, (B, N, H, d))
    dq, dk, dv = run_bwd(inp, do_bits)
    for (b, h) in [(0, 0), (3, 11)]:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        rq, rk, rv = oracle.attention_backward(f64(inp.q[sl]), f64(inp.k[sl]), f64(inp.v[sl]), f64(do_bits[sl]),
                                               True, inp.scale)
        check(dq[sl], rq, f"dq[b={b},h={h}]")
        check(dk[sl], rk, f"dk[b={b},h={h}]")
        check(dv[sl], rv, f"dv[b={b},h={h}]")
    assert all(np.isfinite(x).all() for x in (dq, dk, dv))


def test_bwd_schedules_bitwise_equal():
    """One workgroup per tile and the persistent schedule run the same per-tile
    arithmetic: bitwise equal gradients (causal and not, GQA, d = 64)."""
    for (B, N, Hq, Hkv, d, causal) in [(2, 700, 4, 2, 128, True), (1, 1500, 8, 8, 128, False), (2, 333, 2, 1, 64, True)]:
        inp = W.dense(B, N, N, Hq, Hkv, d, causal, seed=560 + N)
        do_bits = W.normal_bf16_bits(560 + N, W.STREAM_DO, (B, N, Hq, d))
        a = run_bwd(inp, do_bits, schedule=1)
        b = run_bwd(inp, do_bits, schedule=2)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
