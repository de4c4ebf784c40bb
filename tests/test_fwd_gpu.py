"""GPU parity of the bf16 forward (dense and packed) against the fp64 oracle.

Every comparison is element by element on the same seeded bf16 inputs:
|o - o_ref| <= 1e-2 + 1e-2 |o_ref| and |lse - lse_ref| <= 1e-3. Small cases are
checked in full (several tiles plus a ragged tail); the full-size workloads are
checked on sampled rows that the oracle computes one by one, in the same launch
configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _helpers import assert_lse_close, assert_o_close, dev_bf16, f64, host_bits, log

pytestmark = pytest.mark.gpu


def run_dense(inp, tuning=None):
    import exact_attention_amd as ea
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    o, lse = ea.attn_fwd(q, k, v, inp.causal, inp.scale, tuning=tuning)
    torch.cuda.synchronize()
    return f64(host_bits(o)), lse.cpu().numpy().astype(np.float64)


def check_full(inp, tuning=None):
    o, lse = run_dense(inp, tuning)
    ro, rl = oracle.attention(f64(inp.q), f64(inp.k), f64(inp.v), inp.causal, inp.scale)
    e = assert_o_close(o, ro)
    el = assert_lse_close(lse, rl)
    return e, el


@pytest.mark.parametrize("causal", [False, True])
def test_tiny_workload(causal):
    inp = W.tiny(causal)
    log(f"fwd tiny causal={causal} shape={inp.q.shape}")
    e, el = check_full(inp)
    log(f"  max|do|={e:.2e} max|dlse|={el:.2e}")


SHAPES = [
    # B, Nq, Nk, Hq, Hkv, d, causal
    (2, 300, 300, 4, 2, 128, True),
    (2, 300, 300, 4, 2, 128, False),
    (1, 77, 77, 2, 2, 64, False),
    (1, 1, 1, 1, 1, 128, True),
    (2, 129, 257, 4, 4, 128, True),      # Nq < Nk, bottom-right causal
    (1, 200, 50, 2, 1, 64, True),        # Nq > Nk: leading rows have no key
    (3, 513, 513, 8, 8, 128, False),
    (1, 640, 640, 3, 1, 128, True),      # GQA 3:1, multi-block
]


# 1: the 4-wave kernel, 2: the 8-wave ping-pong kernel, 4: the ping-pong
# kernel in persistent form, 5: its unroll-KV form (each against the oracle)
KERNELS = [1, 2, 4, 5]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("shape", SHAPES)
def test_shapes(shape, kernel):
    import exact_attention_amd as ea
    B, Nq, Nk, Hq, Hkv, d, causal = shape
    log(f"fwd shape {shape} kernel {kernel}")
    inp = W.dense(B, Nq, Nk, Hq, Hkv, d, causal, seed=77 + Nq + Nk)
    check_full(inp, tuning=ea.tuning(kernel=kernel))


def _rows(inp, b, h, rows):
    g = inp.q.shape[2] // inp.k.shape[2]
    q = f64(inp.q[b:b + 1, :, h:h + 1, :])
    k = f64(inp.k[b:b + 1, :, h // g:h // g + 1, :])
    v = f64(inp.v[b:b + 1, :, h // g:h // g + 1, :])
    return oracle.attention_rows(q, k, v, 0, 0, rows, inp.causal, inp.scale)


def _sample_rows(N, rng, n=24):
    fixed = [0, 1, 63, 64, 127, 128, N // 2, N - 129, N - 128, N - 2, N - 1]
    rand = rng.integers(0, N, size=n).tolist()
    return sorted(set(r for r in fixed + rand if 0 <= r < N))


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_workload_sampled(causal):
    inp = W.prefill(causal)
    log(f"fwd prefill workload causal={causal} shape={inp.q.shape}")
    o, lse = run_dense(inp)
    B, N, H, d = inp.q.shape
    rng = np.random.default_rng(5)
    pairs = [(0, 0), (B - 1, H - 1), (1, 7), (2, 12)]
    rows = _sample_rows(N, rng)
    for (b, h) in pairs:
        ro, rl = _rows(inp, b, h, rows)
        assert_o_close(o[b, rows, h, :], ro, what=f"o[b={b},h={h}]")
        assert_lse_close(lse[b, h, rows], rl, what=f"lse[b={b},h={h}]")
    assert np.isfinite(o).all() and np.isfinite(lse).all()


def test_long_context_sampled():
    inp = W.long_context()
    log(f"fwd long-context workload shape={inp.q.shape}")
    o, lse = run_dense(inp)
    B, N, H, d = inp.q.shape
    rng = np.random.default_rng(6)
    rows = _sample_rows(N, rng, n=12)
    for (b, h) in [(0, 0), (0, 31), (0, 17)]:
        ro, rl = _rows(inp, b, h, rows)
        assert_o_close(o[b, rows, h, :], ro, what=f"o[h={h}]")
        assert_lse_close(lse[b, h, rows], rl, what=f"lse[h={h}]")
    assert np.isfinite(o).all() and np.isfinite(lse).all()


def run_varlen(inp, poison_rows=0, tuning=None):
    import exact_attention_amd as ea
    Hq, d = inp.q.shape[1], inp.q.shape[2]
    Hkv = inp.k.shape[1]
    # rows outside every sequence hold NaN and must never be read
    nan = np.full((poison_rows, Hq, d), 0x7FC0, np.uint16)
    nank = np.full((poison_rows, Hkv, d), 0x7FC0, np.uint16)
    q = dev_bf16(np.concatenate([inp.q, nan]))
    k = dev_bf16(np.concatenate([inp.k, nank]))
    v = dev_bf16(np.concatenate([inp.v, nank]))
    cu_q = torch.from_numpy(inp.cu_q).cuda()
    cu_k = torch.from_numpy(inp.cu_k).cuda()
    maxq = int(np.diff(inp.cu_q).max())
    o, lse = ea.attn_fwd_varlen(q, k, v, cu_q, cu_k, maxq, inp.causal, inp.scale, tuning=tuning)
    torch.cuda.synchronize()
    Tq = int(inp.cu_q[-1])
    return f64(host_bits(o))[:Tq], lse.cpu().numpy().astype(np.float64)[:, :Tq]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_small_with_poison(causal, kernel):
    import exact_attention_amd as ea
    L = [1, 129, 300, 64, 1000, 17]
    inp = W.varlen(L, L, 4, 2, 128, causal, seed=90)
    log(f"fwd varlen lengths={L} causal={causal} kernel={kernel}")
    o, lse = run_varlen(inp, poison_rows=70, tuning=ea.tuning(kernel=kernel))
    ro, rl = oracle.attention_varlen(f64(inp.q), f64(inp.k), f64(inp.v), inp.cu_q, inp.cu_k, causal, inp.scale)
    assert_o_close(o, ro)
    assert_lse_close(lse, rl)


@pytest.mark.parametrize("kernel", KERNELS)
def test_varlen_rectangular_lengths(kernel):
    import exact_attention_amd as ea
    Lq = [5, 200, 64]
    Lk = [40, 260, 64]
    inp = W.varlen(Lq, Lk, 2, 2, 64, True, seed=91)
    o, lse = run_varlen(inp, tuning=ea.tuning(kernel=kernel))
    ro, rl = oracle.attention_varlen(f64(inp.q), f64(inp.k), f64(inp.v), inp.cu_q, inp.cu_k, True, inp.scale)
    assert_o_close(o, ro)
    assert_lse_close(lse, rl)


def test_long_ragged_sampled():
    inp = W.long_ragged()
    L = np.diff(inp.cu_q)
    log(f"fwd ragged workload lengths={L.tolist()}")
    o, lse = run_varlen(inp)
    rng = np.random.default_rng(7)
    H = inp.q.shape[1]
    for s in (int(np.argmax(L)), int(np.argmin(L)), 3):
        a, n = int(inp.cu_q[s]), int(L[s])
        rows = _sample_rows(n, rng, n=6)
        for h in (0, H - 1):
            q = f64(inp.q[None, a:a + n, h:h + 1])
            k = f64(inp.k[None, a:a + n, h:h + 1])
            v = f64(inp.v[None, a:a + n, h:h + 1])
            ro, rl = oracle.attention_rows(q, k, v, 0, 0, rows, True, inp.scale)
            assert_o_close(o[[a + r for r in rows], h, :], ro, what=f"o[s={s},h={h}]")
            assert_lse_close(lse[h, [a + r for r in rows]], rl, what=f"lse[s={s},h={h}]")


def test_determinism_and_order_invariance():
    import exact_attention_amd as ea
    inp = W.dense(2, 1000, 1000, 4, 4, 128, True, seed=92)
    o1, l1 = run_dense(inp)
    o2, l2 = run_dense(inp)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, l3 = run_dense(inp, tuning=ea.tuning(natural_order=1))
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)
    # the 4-wave kernel is deterministic and order-invariant too
    o4, l4 = run_dense(inp, tuning=ea.tuning(kernel=1))
    o5, l5 = run_dense(inp, tuning=ea.tuning(kernel=1, natural_order=1))
    assert np.array_equal(o4, o5) and np.array_equal(l4, l5)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("mode", [1, 2])
def test_exp_modes(mode, kernel):
    """The polynomial and hybrid exponentials on a square causal shape, on
    Nq > Nk (leading rows see no key: masked scores must give exactly 0, so
    those rows stay O = 0, lse = -inf) and on packed sequences with no keys."""
    import exact_attention_amd as ea
    tun = ea.tuning(exp_mode=mode, kernel=kernel)
    inp = W.dense(2, 700, 700, 2, 2, 128, True, seed=93)
    check_full(inp, tuning=tun)
    inp = W.dense(1, 200, 50, 2, 1, 64 if kernel == 1 else 128, True, seed=193)
    check_full(inp, tuning=tun)
    Lq = [5, 300, 64, 200, 1]
    Lk = [0, 300, 0, 260, 700]
    vin = W.varlen(Lq, Lk, 4, 2, 128, True, seed=293)
    o, lse = run_varlen(vin, poison_rows=17, tuning=tun)
    ro, rl = oracle.attention_varlen(f64(vin.q), f64(vin.k), f64(vin.v), vin.cu_q, vin.cu_k, True, vin.scale)
    assert_o_close(o, ro)
    assert_lse_close(lse, rl)


def test_eager_rescale_matches():
    import exact_attention_amd as ea
    inp = W.dense(1, 900, 900, 2, 2, 128, True, seed=94)
    e0, _ = check_full(inp, tuning=ea.tuning(rescale_log2=0.0))
    e8, _ = check_full(inp, tuning=ea.tuning(rescale_log2=8.0))
    log(f"  eager max|do|={e0:.2e} lazy max|do|={e8:.2e}")


# ---------------------------------------------------------------- head dims (d_qk, d_v) = (192, 128)

HD_SHAPES = [
    # B, Nq, Nk, Hq, Hkv, causal
    (2, 300, 300, 4, 2, True),           # ragged tail, GQA 2:1
    (1, 256, 256, 2, 2, False),
    (1, 129, 257, 2, 1, True),           # Nq < Nk, bottom-right causal
    (1, 1, 1, 1, 1, True),
    (1, 200, 50, 2, 2, True),            # Nq > Nk: leading rows have no key
    (2, 640, 640, 3, 3, True),           # several row blocks
]


@pytest.mark.parametrize("shape", HD_SHAPES)
def test_head_dims_192_128(shape):
    """Scores over d_qk = 192, values and output of d_v = 128 (the pair the
    pages benchmark for DeepSeek V3), on the ping-pong kernel."""
    B, Nq, Nk, Hq, Hkv, causal = shape
    log(f"fwd (192,128) shape {shape}")
    inp = W.dense(B, Nq, Nk, Hq, Hkv, 192, causal, seed=177 + Nq + Nk, dv=128)
    assert inp.v.shape[3] == 128 and abs(inp.scale - 1 / np.sqrt(192)) < 1e-12
    e, el = check_full(inp)
    log(f"  max|do|={e:.2e} max|dlse|={el:.2e}")


def test_head_dims_192_128_prefill_sampled():
    """(192, 128) at the prefill workload's size (B=4, H=16, N=8192, causal),
    sampled rows; determinism and tile-order invariance."""
    import exact_attention_amd as ea
    inp = W.dense(4, 8192, 8192, 16, 16, 192, True, seed=1192, dv=128)
    log(f"fwd (192,128) prefill shape q={inp.q.shape} v={inp.v.shape}")
    o, lse = run_dense(inp)
    B, N, H, _ = inp.q.shape
    rng = np.random.default_rng(15)
    rows = _sample_rows(N, rng, n=12)
    for (b, h) in [(0, 0), (3, 15), (2, 5)]:
        ro, rl = _rows(inp, b, h, rows)
        assert_o_close(o[b, rows, h, :], ro, what=f"o[b={b},h={h}]")
        assert_lse_close(lse[b, h, rows], rl, what=f"lse[b={b},h={h}]")
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    o2, l2 = run_dense(inp, tuning=ea.tuning(natural_order=1))
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)


def test_persistent_bitwise_equals_per_tile_launch():
    """The persistent form runs the same per-tile arithmetic as the ping-pong
    kernel launched once per tile, so the outputs match bit for bit; shapes with
    fewer tiles than workgroups, more tiles than one round, causal and not,
    GQA, and (192, 128)."""
    import exact_attention_amd as ea
    cases = [((1, 300, 300, 2, 2, 128, True), None), ((2, 4096, 4096, 8, 4, 128, True), None),
             ((1, 2000, 2000, 16, 16, 128, False), None), ((2, 1000, 1000, 4, 4, 192, True), 128),
             # tiles with fewer key tiles than the walk's minimum step count
             ((3, 100, 100, 16, 8, 128, True), None), ((2, 130, 70, 24, 24, 128, False), None),
             # d = 64; rows with no key; more tiles than workgroups, mixed lengths
             ((2, 3000, 3000, 12, 4, 64, True), None), ((1, 1200, 300, 40, 8, 128, True), None),
             ((1, 1, 1, 600, 600, 128, False), None)]
    for (B, Nq, Nk, Hq, Hkv, d, causal), dv in cases:
        inp = W.dense(B, Nq, Nk, Hq, Hkv, d, causal, seed=600 + Nq + Hq, dv=dv)
        o2, l2 = run_dense(inp, tuning=ea.tuning(kernel=2))
        for kern in ((4,) if dv not in (None, d) else (4, 5)):
            o4, l4 = run_dense(inp, tuning=ea.tuning(kernel=kern))
            log(f"kernel {kern} vs per-tile {B, Nq, Nk, Hq, Hkv, d, dv, causal}: equal={np.array_equal(o2, o4)}")
            assert np.array_equal(o2, o4) and np.array_equal(l2, l4)


@pytest.mark.parametrize("causal", [True, False])
def test_persistent_varlen_bitwise_equals_per_tile_launch(causal):
    """Packed sequences through the persistent walk: lengths from 1 row to
    several blocks (tiles of every step count, empty-looking tails), bitwise
    equal to one workgroup per tile."""
    import exact_attention_amd as ea
    L = [1, 700, 64, 2000, 3, 255, 256, 257, 1500, 90]
    inp = W.varlen(L, L, 6, 2, 128, causal, seed=95)
    o2, l2 = run_varlen(inp, tuning=ea.tuning(kernel=2))
    for kern in (4, 5):
        o4, l4 = run_varlen(inp, tuning=ea.tuning(kernel=kern))
        log(f"kernel {kern} varlen causal={causal}: equal={np.array_equal(o2, o4)}")
        assert np.array_equal(o2, o4) and np.array_equal(l2, l4)


def test_persistent_prefill_workload_sampled():
    import exact_attention_amd as ea
    inp = W.prefill(True)
    o, lse = run_dense(inp, tuning=ea.tuning(kernel=4))
    B, N, H, d = inp.q.shape
    rng = np.random.default_rng(25)
    rows = _sample_rows(N, rng)
    for (b, h) in [(0, 0), (B - 1, H - 1), (2, 9)]:
        ro, rl = _rows(inp, b, h, rows)
        assert_o_close(o[b, rows, h, :], ro, what=f"o[b={b},h={h}]")
        assert_lse_close(lse[b, h, rows], rl, what=f"lse[b={b},h={h}]")
    assert np.isfinite(o).all() and np.isfinite(lse).all()


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_empty_sequences_all_kernels(causal):
    """Packed sequences with no query rows, with no keys (their rows get O = 0,
    lse = -inf), or both, between ordinary ones: every kernel against the
    oracle, and the persistent and unroll-KV forms bit for bit against the
    ping-pong kernel."""
    import exact_attention_amd as ea
    Lq = [5, 0, 300, 64, 0, 200, 1, 257]
    Lk = [0, 10, 300, 0, 0, 260, 700, 257]
    inp = W.varlen(Lq, Lk, 4, 2, 128, causal, seed=97)
    ro, rl = oracle.attention_varlen(f64(inp.q), f64(inp.k), f64(inp.v), inp.cu_q, inp.cu_k, causal, inp.scale)
    res = {}
    for kern in KERNELS:
        o, lse = run_varlen(inp, poison_rows=33, tuning=ea.tuning(kernel=kern))
        log(f"varlen empty sequences causal={causal} kernel={kern}")
        assert_o_close(o, ro, what=f"o[kernel {kern}]")
        assert_lse_close(lse, rl, what=f"lse[kernel {kern}]")
        res[kern] = (o, lse)
    for kern in (4, 5):
        assert np.array_equal(res[kern][0], res[2][0]) and np.array_equal(res[kern][1], res[2][1])
