"""Pins of the oracle's attention backward (CPU only).

``oracle.attention_backward`` evaluates the gradients of L = sum(dO * O) by the
backward's five products ("Low-precision FlashAttention-4: end-to-end
block-scaled attention for Blackwell", section 2.2). It is pinned here against
things that do not share its formula:
  * central finite differences of the oracle's forward (a different function),
  * torch autograd in float64 through a plain softmax forward,
  * invariants the mathematics fixes (key-shift invariance, value-gradient
    mass, causal row 0, identical keys, GQA as repeated heads),
and plausible mistakes planted in a copy of the formula must fail the finite
difference check.
"""
import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss(q, k, v, do, causal, scale):
    o, _ = oracle.attention(q, k, v, causal, scale, threads=1, row_block=3)
    return float((o * do).sum())


def _fd_grad(x, f, h=1e-5):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp = x.copy(); xp[i] += h
        xm = x.copy(); xm[i] -= h
        g[i] = (f(xp) - f(xm)) / (2 * h)
    return g


CASES = [
    # B, Nq, Nk, Hq, Hkv, d, dv, causal
    (1, 5, 5, 2, 2, 3, 3, False),
    (1, 5, 5, 2, 1, 3, 2, True),      # GQA 2:1, d_v != d_qk
    (2, 3, 6, 2, 2, 4, 4, True),      # Nq < Nk, bottom-right causal
    (1, 6, 3, 1, 1, 3, 3, True),      # Nq > Nk: leading rows have no key
]


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_finite_differences(case):
    B, Nq, Nk, Hq, Hkv, d, dv, causal = case
    seed = sum(case[:7])
    q = _rand((B, Nq, Hq, d), seed)
    k = _rand((B, Nk, Hkv, d), seed + 1)
    v = _rand((B, Nk, Hkv, dv), seed + 2)
    do = _rand((B, Nq, Hq, dv), seed + 3)
    scale = 0.7
    dq, dk, dvv = oracle.attention_backward(q, k, v, do, causal, scale, threads=2, row_block=2)
    fq = _fd_grad(q, lambda x: _loss(x, k, v, do, causal, scale))
    fk = _fd_grad(k, lambda x: _loss(q, x, v, do, causal, scale))
    fv = _fd_grad(v, lambda x: _loss(q, k, x, do, causal, scale))
    for got, ref in ((dq, fq), (dk, fk), (dvv, fv)):
        np.testing.assert_allclose(got, ref, rtol=1e-7, atol=1e-8)


def _torch_grads(q, k, v, do, causal, scale):
    """Autograd through a plain float64 softmax forward (rows with no key give
    zero output)."""
    Q, K, V = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    Kr = K.repeat_interleave(g, dim=2)
    Vr = V.repeat_interleave(g, dim=2)
    s = scale * torch.einsum("bihc,bjhc->bhij", Q, Kr)
    if causal:
        i = torch.arange(Nq)[:, None]
        j = torch.arange(Nk)[None, :]
        s = s.masked_fill(j > i + (Nk - Nq), float("-inf"))
    empty = torch.isinf(s).all(dim=-1, keepdim=True)
    p = torch.softmax(s.masked_fill(empty, 0.0), dim=-1).masked_fill(empty, 0.0)
    o = torch.einsum("bhij,bjhc->bihc", p, Vr)
    (o * torch.tensor(do)).sum().backward()
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 40, 40, 4, 2, 16, 16), (1, 33, 70, 2, 1, 12, 8), (1, 70, 33, 3, 3, 8, 8)])
def test_backward_matches_autograd(shape, causal):
    B, Nq, Nk, Hq, Hkv, d, dv = shape
    q = _rand((B, Nq, Hq, d), 31)
    k = _rand((B, Nk, Hkv, d), 32)
    v = _rand((B, Nk, Hkv, dv), 33)
    do = _rand((B, Nq, Hq, dv), 34)
    dq, dk, dvv = oracle.attention_backward(q, k, v, do, causal, 0.3, threads=3, row_block=16)
    tq, tk, tv = _torch_grads(q, k, v, do, causal, 0.3)
    for got, ref in ((dq, tq), (dk, tk), (dvv, tv)):
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11)


def test_key_shift_invariance():
    """Adding one vector c to every key adds q.c to a whole score row, which the
    softmax ignores: all three gradients are unchanged. A wrong rowsum term
    (the dsoftmax projection) would make dQ pick up scale * c * sum_j dS_ij."""
    q = _rand((1, 20, 2, 8), 41); k = _rand((1, 20, 2, 8), 42); v = _rand((1, 20, 2, 8), 43)
    do = _rand((1, 20, 2, 8), 44)
    c = _rand(8, 45) * 3
    for causal in (False, True):
        a = oracle.attention_backward(q, k, v, do, causal, 0.5, threads=2, row_block=7)
        b = oracle.attention_backward(q, k + c, v, do, causal, 0.5, threads=2, row_block=7)
        for x, y in zip(a, b):
            np.testing.assert_allclose(x, y, rtol=1e-9, atol=1e-10)


def test_value_gradient_mass_and_closed_forms():
    q = _rand((1, 12, 1, 6), 51); k = _rand((1, 12, 1, 6), 52); v = _rand((1, 12, 1, 5), 53)
    do = _rand((1, 12, 1, 5), 54)
    # every row's probabilities sum to one, so the value gradients sum to sum_i dO_i
    for causal in (False, True):
        dq, dk, dvv = oracle.attention_backward(q, k, v, do, causal, 0.4, threads=1)
        np.testing.assert_allclose(dvv.sum(axis=1), do.sum(axis=1), rtol=1e-12, atol=1e-12)
        # sum_j dS_ij = 0 for every row, so the key gradients sum to zero
        np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    # causal row 0 attends to one key only: P = 1, dS = 0, dQ_0 = 0
    dq, _, _ = oracle.attention_backward(q, k, v, do, True, 0.4, threads=1)
    assert np.abs(dq[0, 0]).max() < 1e-14
    # identical keys: uniform softmax, dQ = 0
    kk = np.repeat(k[:, :1], 12, axis=1)
    dq, _, _ = oracle.attention_backward(q, kk, v, do, False, 0.4, threads=1)
    assert np.abs(dq).max() < 1e-12


def test_gqa_equals_repeated_heads_summed():
    q = _rand((2, 15, 4, 6), 61); k = _rand((2, 15, 2, 6), 62); v = _rand((2, 15, 2, 6), 63)
    do = _rand((2, 15, 4, 6), 64)
    dq, dk, dvv = oracle.attention_backward(q, k, v, do, True, 0.5, threads=2)
    kr, vr = np.repeat(k, 2, axis=2), np.repeat(v, 2, axis=2)
    rq, rk, rv = oracle.attention_backward(q, kr, vr, do, True, 0.5, threads=2)
    np.testing.assert_allclose(dq, rq, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk, rk.reshape(2, 15, 2, 2, 6).sum(axis=3), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dvv, rv.reshape(2, 15, 2, 2, 6).sum(axis=3), rtol=1e-12, atol=1e-13)


def test_heads_subset_and_row_blocks_do_not_change_results():
    q = _rand((2, 30, 2, 8), 71); k = _rand((2, 30, 2, 8), 72); v = _rand((2, 30, 2, 8), 73)
    do = _rand((2, 30, 2, 8), 74)
    full = oracle.attention_backward(q, k, v, do, True, 0.5, threads=2, row_block=512)
    blk = oracle.attention_backward(q, k, v, do, True, 0.5, threads=3, row_block=4)
    for x, y in zip(full, blk):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-13)
    sub = oracle.attention_backward(q, k, v, do, True, 0.5, heads=[(1, 1)])
    np.testing.assert_allclose(sub[0][1, :, 1], full[0][1, :, 1], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sub[1][1, :, 1], full[1][1, :, 1], rtol=1e-12, atol=1e-13)
    assert np.all(sub[0][0] == 0) and np.all(sub[2][0] == 0)


def test_planted_mistakes_fail_finite_differences():
    """Copies of the backward formula with a plausible mistake each disagree
    with the finite differences that the oracle matches."""
    rng = np.random.default_rng(81)
    qh, kh, vh, doh = (rng.standard_normal((6, 4)) for _ in range(4))
    scale = 0.8
    q, k, v, do = (x[None, :, None, :] for x in (qh, kh, vh, doh))
    fq = _fd_grad(q, lambda x: _loss(x, k, v, do, False, scale))[0, :, 0]
    fk = _fd_grad(k, lambda x: _loss(q, x, v, do, False, scale))[0, :, 0]
    s = scale * qh @ kh.T
    p = np.exp(s - s.max(1, keepdims=True)); p /= p.sum(1, keepdims=True)
    dp = doh @ vh.T
    ds = p * (dp - (p * dp).sum(1, keepdims=True))
    good_q, good_k = scale * ds @ kh, scale * ds.T @ qh
    np.testing.assert_allclose(good_q, fq, rtol=1e-7, atol=1e-8)
    np.testing.assert_allclose(good_k, fk, rtol=1e-7, atol=1e-8)
    wrong = {
        "dropped rowsum term": scale * (p * dp) @ kh,
        "missing scale": ds @ kh,
        "transposed dS": scale * ds.T @ kh,
        "rowsum of dP without P": scale * (p * (dp - dp.sum(1, keepdims=True))) @ kh,
    }
    for name, g in wrong.items():
        assert not np.allclose(g, fq, rtol=1e-4, atol=1e-5), name
    assert not np.allclose(scale * ds @ qh, fk, rtol=1e-4, atol=1e-5)        # dK from dS instead of dS^T
