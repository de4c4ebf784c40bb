"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test pins the oracle against something it does not compute itself: the
page's worked example, closed forms, a 50-digit brute force, library routines
for the number encodings, or an algebraic invariant. A plausible slip in the
oracle (dropped scale, wrong max, transposed operand, wrong causal bound, wrong
GQA grouping, wrong page index) fails at least one of them; see
``test_planted_mistakes_are_caught``.
"""
import json
import os

import mpmath
import numpy as np
import pytest
import torch

import oracle
import importlib
oa = importlib.import_module("oracle.attention")
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- worked example

def _within_printed(x, printed):
    val, digits = printed
    return abs(x - val) <= 10.0 ** (-digits) + 1e-12


def test_worked_example_streaming_and_full_row():
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    sb, vb = g["score_blocks"], g["value_blocks"]
    # block 1 alone: m, l, a before normalisation
    s1 = np.array(sb[0]); v1 = np.array(vb[0])
    m1 = s1.max(); p1 = np.exp(s1 - m1)
    assert _within_printed(m1, g["after_block_1"]["m"])
    assert _within_printed(p1.sum(), g["after_block_1"]["l"])
    assert _within_printed(p1 @ v1, g["after_block_1"]["a"])
    # streaming recurrence (oracle restatement)
    o_stream, lse_stream = oracle.online_softmax_row([np.array(b) for b in sb],
                                                     [np.array(b) for b in vb])
    l2 = np.exp(m1 - 3.0) * p1.sum() + 1.0
    a2 = np.exp(m1 - 3.0) * (p1 @ v1) + 30.0
    assert _within_printed(l2, g["after_block_2"]["l"])
    assert _within_printed(a2, g["after_block_2"]["a"])
    assert _within_printed(float(o_stream), g["o"])
    # full-row oracle on the same problem: q=[1], keys [1],[2],[3], scale 1
    q = np.array([[[[1.0]]]])
    k = np.array([[[[1.0]], [[2.0]], [[3.0]]]])
    v = np.array([[[[10.0]], [[20.0]], [[30.0]]]])
    o_full, lse_full = oracle.attention(q, k, v, causal=False, scale=1.0, threads=1)
    assert _within_printed(o_full[0, 0, 0, 0], g["o"])
    # both formulations agree to rounding, and match the closed form
    closed = (10 * np.e + 20 * np.e ** 2 + 30 * np.e ** 3) / (np.e + np.e ** 2 + np.e ** 3)
    assert abs(o_full[0, 0, 0, 0] - closed) < 1e-12
    assert abs(float(o_stream) - closed) < 1e-12
    assert abs(lse_full[0, 0, 0] - np.log(np.e + np.e ** 2 + np.e ** 3)) < 1e-12
    assert abs(lse_stream - lse_full[0, 0, 0]) < 1e-12


# ---------------------------------------------------------------- brute force

def _brute(q, k, v, causal, scale):
    """Triple loop in 50-digit arithmetic straight from the definition."""
    mpmath.mp.dps = 50
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, dv = v.shape
    g = Hq // Hkv
    o = np.zeros((B, Nq, Hq, dv))
    lse = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            for i in range(Nq):
                js = [j for j in range(Nk) if (not causal) or j <= i + (Nk - Nq)]
                if not js:
                    continue
                s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[b, i, h, c]) * mpmath.mpf(k[b, j, h // g, c])
                                                     for c in range(d)) for j in js]
                e = [mpmath.e ** x for x in s]
                z = mpmath.fsum(e)
                for c in range(dv):
                    o[b, i, h, c] = float(mpmath.fsum(e[t] * mpmath.mpf(v[b, j, h // g, c]) for t, j in enumerate(js)) / z)
                lse[b, h, i] = float(mpmath.log(z))
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 5, 2, 2, 3), (2, 16, 4, 2, 4), (1, 7, 1, 1, 8)])
def test_brute_force_small(causal, shape):
    B, N, Hq, Hkv, d = shape
    q = _rand((B, N, Hq, d), 1) * 2
    k = _rand((B, N, Hkv, d), 2) * 2
    v = _rand((B, N, Hkv, d), 3)
    scale = 1 / np.sqrt(d)
    o, lse = oracle.attention(q, k, v, causal, scale, threads=2, row_block=4)
    ob, lb = _brute(q, k, v, causal, scale)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_value_dim_differs(causal):
    """Scores over d_qk = 6, values of d_v = 4 (the (192, 128) head-dim pair in
    miniature); GQA 2:1."""
    q = _rand((1, 9, 2, 6), 21) * 2
    k = _rand((1, 9, 1, 6), 22) * 2
    v = _rand((1, 9, 1, 4), 23)
    o, lse = oracle.attention(q, k, v, causal, 1 / np.sqrt(6), threads=2, row_block=4)
    assert o.shape == (1, 9, 2, 4)
    ob, lb = _brute(q, k, v, causal, 1 / np.sqrt(6))
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=1e-13, atol=1e-13)
    ro, rl = oracle.attention_rows(q[:, :, 1:2], k, v, 0, 0, [0, 4, 8], causal, 1 / np.sqrt(6))
    np.testing.assert_allclose(ro, ob[0, [0, 4, 8], 1], rtol=1e-12, atol=1e-13)


def test_brute_force_rectangular_causal():
    # Nq != Nk: bottom-right aligned causal bound (a reading; unexercised by the workloads)
    q = _rand((1, 3, 2, 4), 4); k = _rand((1, 9, 2, 4), 5); v = _rand((1, 9, 2, 4), 6)
    o, lse = oracle.attention(q, k, v, True, 0.5, threads=1)
    ob, lb = _brute(q, k, v, True, 0.5)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=1e-13)


# ---------------------------------------------------------------- invariants and closed forms

def test_rows_sum_to_one():
    q = _rand((2, 40, 3, 16), 7); k = _rand((2, 40, 3, 16), 8)
    v = np.ones((2, 40, 3, 1))
    for causal in (False, True):
        o, _ = oracle.attention(q, k, v, causal, 0.25, threads=2, row_block=16)
        assert np.max(np.abs(o - 1.0)) < 1e-12


def test_online_equals_full_random():
    rng = np.random.default_rng(11)
    for trial in range(20):
        n = int(rng.integers(1, 60))
        s = rng.standard_normal(n) * 4
        v = rng.standard_normal((n, 5))
        cuts = np.sort(rng.choice(np.arange(1, n), size=min(n - 1, 3), replace=False)) if n > 1 else []
        sb = np.split(s, cuts); vb = np.split(v, cuts)
        o_s, l_s = oracle.online_softmax_row(sb, vb)
        p = np.exp(s - s.max())
        o_f = p @ v / p.sum(); l_f = s.max() + np.log(p.sum())
        assert np.max(np.abs(o_s - o_f)) < 1e-12 and abs(l_s - l_f) < 1e-12


def test_zero_query_gives_mean_of_allowed_values():
    k = _rand((1, 10, 1, 4), 9); v = _rand((1, 10, 1, 3), 10)
    q = np.zeros((1, 10, 1, 4))
    o, lse = oracle.attention(q, k, v, True, 0.7, threads=1)
    for i in range(10):
        np.testing.assert_allclose(o[0, i, 0], v[0, :i + 1, 0].mean(axis=0), rtol=1e-13, atol=1e-14)
        assert abs(lse[0, 0, i] - np.log(i + 1)) < 1e-13


def test_causal_row_zero_and_single_key():
    q = _rand((1, 6, 2, 4), 12); k = _rand((1, 6, 2, 4), 13); v = _rand((1, 6, 2, 4), 14)
    o, lse = oracle.attention(q, k, v, True, 0.3, threads=1)
    for h in range(2):
        assert np.array_equal(o[0, 0, h], v[0, 0, h])
        assert abs(lse[0, h, 0] - 0.3 * q[0, 0, h] @ k[0, 0, h]) < 1e-14
    o1, _ = oracle.attention(q, k[:, :1], v[:, :1], False, 0.3, threads=1)
    assert np.array_equal(o1[0, :, 0], np.repeat(v[0, :1, 0], 6, axis=0))


def test_dominant_key_selects_its_value():
    q = _rand((1, 1, 1, 8), 15)
    k = _rand((1, 12, 1, 8), 16) * 0.01
    k[0, 7, 0] = q[0, 0, 0] * 40.0
    v = _rand((1, 12, 1, 5), 17)
    o, _ = oracle.attention(q, k, v, False, 1.0, threads=1)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 7, 0], atol=1e-9)


def test_causal_row_equals_prefix_noncausal():
    q = _rand((1, 24, 2, 8), 18); k = _rand((1, 24, 2, 8), 19); v = _rand((1, 24, 2, 8), 20)
    o, lse = oracle.attention(q, k, v, True, 0.35, threads=2, row_block=8)
    for i in (0, 5, 13, 23):
        oi, li = oracle.attention(q[:, i:i + 1], k[:, :i + 1], v[:, :i + 1], False, 0.35, threads=1)
        np.testing.assert_allclose(o[0, i], oi[0, 0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[0, :, i], li[0, :, 0], rtol=1e-13)


def test_gqa_equals_repeated_heads():
    q = _rand((2, 20, 8, 8), 21); k = _rand((2, 20, 2, 8), 22); v = _rand((2, 20, 2, 8), 23)
    o, lse = oracle.attention(q, k, v, True, 0.4, threads=2)
    o2, lse2 = oracle.attention(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), True, 0.4, threads=2)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # head 5 reads kv head 1 (consecutive grouping), not kv head 5 % 2
    o3, _ = oracle.attention(q[:, :, 5:6], k[:, :, 1:2], v[:, :, 1:2], True, 0.4, threads=1)
    assert np.array_equal(o[:, :, 5:6], o3)


def test_attention_rows_matches_attention():
    q = _rand((2, 50, 4, 8), 24); k = _rand((2, 50, 2, 8), 25); v = _rand((2, 50, 2, 8), 26)
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, causal, 0.3, threads=2, row_block=16)
        rows = [0, 1, 17, 49]
        orr, lr = oracle.attention_rows(q, k, v, 1, 3, rows, causal, 0.3)
        np.testing.assert_allclose(orr, o[1, rows, 3], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lr, lse[1, 3, rows], rtol=1e-13)


def test_varlen_equals_per_sequence_dense():
    lens = [5, 1, 17, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = _rand((cu[-1], 4, 8), 27); k = _rand((cu[-1], 2, 8), 28); v = _rand((cu[-1], 2, 8), 29)
    o, lse = oracle.attention_varlen(q, k, v, cu, cu, True, 0.3, threads=2)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        od, ld = _brute(q[None, a:b], k[None, a:b], v[None, a:b], True, 0.3)
        np.testing.assert_allclose(o[a:b], od[0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[:, a:b], ld[0], rtol=1e-13)


def test_split_combine_invariance():
    rng = np.random.default_rng(30)
    for trial in range(10):
        n = int(rng.integers(2, 200))
        s = rng.standard_normal(n) * 3
        v = rng.standard_normal((n, 6))
        cuts = np.sort(rng.choice(np.arange(1, n), size=min(n - 1, int(rng.integers(1, 6))), replace=False))
        parts_o, parts_l = [], []
        for sb, vb in zip(np.split(s, cuts), np.split(v, cuts)):
            p = np.exp(sb - sb.max())
            parts_o.append(p @ vb / p.sum()); parts_l.append(sb.max() + np.log(p.sum()))
        parts_o.append(np.zeros(6)); parts_l.append(-np.inf)          # an empty split
        o, l = oracle.lse_combine(parts_o, parts_l)
        p = np.exp(s - s.max())
        assert np.max(np.abs(o - p @ v / p.sum())) < 1e-12
        assert abs(l - (s.max() + np.log(p.sum()))) < 1e-12
    # batched rows
    po = rng.standard_normal((3, 4, 5)); pl = rng.standard_normal((3, 4))
    o, l = oracle.lse_combine(po, pl)
    for r in range(4):
        o1, l1 = oracle.lse_combine(po[:, r], pl[:, r])
        np.testing.assert_allclose(o[r], o1, rtol=1e-14); assert abs(l[r] - l1) < 1e-14


# ---------------------------------------------------------------- paged decode

def test_paged_decode_matches_dense_and_ignores_poison():
    L = [1, 16, 17, 40, 5]
    pg = W.paged(5, 8, 2, 16, 16, L, seed=31, permute=True, poison=True)
    o, lse = oracle.decode_paged(pg.q, pg.k_cache, pg.v_cache, pg.block_table, pg.seq_lens, pg.scale, threads=2)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    for b, n in enumerate(L):
        # re-lay the sequence densely by walking pages by hand
        kd = np.zeros((n, 2, 16), np.uint16); vd = np.zeros((n, 2, 16), np.uint16)
        for t in range(n):
            page = pg.block_table[b, t // 16]
            kd[t] = pg.k_cache[page, t % 16]; vd[t] = pg.v_cache[page, t % 16]
        qd = oracle.bf16_to_f64(pg.q[b])[None, None]
        od, ld = _brute(qd, oracle.bf16_to_f64(kd)[None], oracle.bf16_to_f64(vd)[None], False, pg.scale)
        np.testing.assert_allclose(o[b], od[0, 0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[b], ld[0, :, 0], rtol=1e-13)


def test_paged_gather_permutation_invariance():
    L = [33, 7, 64]
    a = W.paged(3, 4, 2, 8, 16, L, seed=32, permute=True, poison=True)
    b = W.paged(3, 4, 2, 8, 16, L, seed=32, permute=False, poison=True)
    # same draws per physical slot, different placement: re-lay a's pool by its table
    for s, n in enumerate(L):
        ga = oracle.gather_pages(a.k_cache, a.block_table, s, n)
        rows = [a.k_cache[a.block_table[s, t // 16], t % 16] for t in range(n)]
        assert np.array_equal(ga, np.stack(rows))
    # identity table on a pool re-laid in logical order gives the same bits
    pool = np.concatenate([oracle.gather_pages(a.k_cache, a.block_table, s, -(-n // 16) * 16) for s, n in enumerate(L)])
    pool = pool.reshape(-1, 16, 2, 8)
    ident = np.full_like(a.block_table, -1)
    off = 0
    for s, n in enumerate(L):
        np_ = -(-n // 16); ident[s, :np_] = np.arange(off, off + np_); off += np_
    for s, n in enumerate(L):
        assert np.array_equal(oracle.gather_pages(pool, ident, s, n), oracle.gather_pages(a.k_cache, a.block_table, s, n))
    assert b.block_table[0, 0] == 0


# ---------------------------------------------------------------- number encodings

def test_bf16_decode_and_encode_match_torch():
    x = np.concatenate([_rand(10000, 33).astype(np.float32) * 100,
                        np.array([0.0, -0.0, 1e-40, 3.4e38, -3.4e38, np.inf, -np.inf], np.float32)])
    bits = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    dec = oracle.bf16_to_f64(bits)
    ref_dec = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(dec, ref_dec)


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_e4m3_encode_matches_torch_in_range_and_roundtrips():
    x = np.concatenate([_rand(20000, 34) * 50, _rand(2000, 35) * 1e-2, _rand(200, 36) * 1e-4])
    x = x[np.abs(x) <= 448]
    ours = W.f32_to_e4m3_bits(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.e4m3_to_f64(finite)
    back = W.f32_to_e4m3_bits(vals)
    # +0 and -0 both decode to 0; compare values
    assert np.array_equal(oracle.e4m3_to_f64(back), vals)
    assert W.f32_to_e4m3_bits(np.array([1000.0, -1000.0])).tolist() == [0x7E, 0xFE]


def test_e5m2_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e5m2_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7B] == 57344.0 and ours[0x7C] == np.inf and ours[0x01] == 2.0 ** -16 and ours[0x04] == 2.0 ** -14


def test_e5m2_encode_matches_torch_in_range_and_roundtrips():
    x = np.concatenate([_rand(20000, 44) * 3000, _rand(2000, 45) * 1e-3, _rand(200, 46) * 1e-5])
    x = x[np.abs(x) <= 57344]
    ours = W.f32_to_e5m2_bits(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    finite = np.array([c for c in range(256) if ((c >> 2) & 0x1F) != 0x1F], dtype=np.uint8)
    vals = oracle.e5m2_to_f64(finite)
    assert np.array_equal(oracle.e5m2_to_f64(W.f32_to_e5m2_bits(vals)), vals)
    assert W.f32_to_e5m2_bits(np.array([1e6, -1e6])).tolist() == [0x7B, 0xFB]


def test_mx_quantiser_e5m2_invariants():
    x = _rand((2, 64, 2, 64), 47).astype(np.float32)
    x[1, 3, 1, 32:] = 0.0
    codes, sc = W.mx_quantize(x, axis=3, fmt="e5m2")
    deq = oracle.dequant_mx(codes, sc, axis=3, fmt="e5m2")
    vals = oracle.e5m2_to_f64(codes)
    assert np.all(np.isfinite(vals)) and np.all(np.abs(vals) <= 57344)
    nz = sc != 0
    blkmax = np.abs(vals).reshape(2, 64, 2, 2, 32).max(-1)
    assert np.all(blkmax[nz] >= 28672) and np.all(blkmax[nz] <= 57344)     # ceil rule: in [fmax/2, fmax]
    assert np.all(deq[1, 3, 1, 32:] == 0)
    rel = np.abs(deq - x) / np.maximum(np.abs(x), 1e-30)
    normal = np.abs(vals) >= 2.0 ** -14
    assert np.all(rel[normal] <= 2.0 ** -3 + 1e-12)                        # 2 mantissa bits
    # an e5m2 tensor decoded as e4m3 is a different tensor (the format matters)
    assert not np.allclose(oracle.dequant_mx(codes, sc, axis=3), deq)


def test_e8m0_and_mx_quantiser_invariants():
    assert oracle.e8m0_to_f64(np.array([127, 0, 254, 128])).tolist() == [1.0, 2.0 ** -127, 2.0 ** 127, 2.0]
    x = _rand((3, 64, 2, 96), 37).astype(np.float32)
    x[0, 0, 0, :32] = 0.0                                   # an all-zero block
    codes, sc = W.mx_quantize_e4m3(x, axis=3)
    assert sc.shape == (3, 64, 2, 3)
    deq = oracle.dequant_mx(codes, sc, axis=3)
    assert sc[0, 0, 0, 0] == 0 and np.all(deq[0, 0, 0, :32] == 0)
    vals = oracle.e4m3_to_f64(codes)
    assert np.all(np.abs(vals) <= 448)
    # the block maximum lands in [224, 448] under the ceil rule
    blkmax = np.abs(vals).reshape(3, 64, 2, 3, 32).max(-1)
    nz = sc != 0
    assert np.all(blkmax[nz] >= 224) and np.all(blkmax[nz] <= 448)
    rel = np.abs(deq - x) / np.maximum(np.abs(x), 1e-30)
    normal = np.abs(vals) >= 2.0 ** -6
    assert np.all(rel[normal] <= 2.0 ** -4 + 1e-12)
    # sequence-axis scaling (V layout)
    c2, s2 = W.mx_quantize_e4m3(x, axis=1)
    assert s2.shape == (3, 2, 2, 96)
    d2 = oracle.dequant_mx(c2, s2, axis=1)
    assert np.max(np.abs(d2 - x)) <= 448 * 2.0 ** -4 * np.max(oracle.e8m0_to_f64(s2))


# ---------------------------------------------------------------- the exp2 polynomial claim

def test_exp2_cubic_printed_coefficients_accuracy():
    """The printed degree-3 coefficients give about 1e-4 max relative error on
    [0,1) in exact arithmetic; the page's fp32 minimax figure is 8.77e-5. This
    pins the device exp2 tolerance used by the GPU sweep."""
    g = json.load(open(os.path.join(GOLD, "exp2_poly.json")))
    p0, p1, p2, p3 = g["coefficients_printed"]
    f = np.linspace(0, 1, 200001)[:-1]
    approx = p0 + f * (p1 + f * (p2 + f * p3))
    rel = np.abs(approx / np.exp2(f) - 1)
    assert 0.9e-4 < rel.max() < 1.1e-4
    assert rel.max() < g["bf16_rel_step"] / 30


# ---------------------------------------------------------------- planted mistakes

def test_planted_mistakes_are_caught(monkeypatch):
    """Variants of the oracle with a typical slip must fail the brute-force pin."""
    q = _rand((1, 9, 4, 4), 40); k = _rand((1, 9, 2, 4), 41); v = _rand((1, 9, 2, 4), 42)
    ob, lb = _brute(q, k, v, True, 0.5)
    orig = oa._rows_block

    def bad_scale(qh, kh, vh, r0, r1, Nq, causal, scale):
        return orig(qh, kh, vh, r0, r1, Nq, causal, 1.0)

    def bad_causal(qh, kh, vh, r0, r1, Nq, causal, scale):
        return orig(qh, kh, vh, r0, r1, Nq, False, scale)

    def bad_transpose(qh, kh, vh, r0, r1, Nq, causal, scale):
        return orig(qh, vh, kh, r0, r1, Nq, causal, scale)

    for bad in (bad_scale, bad_causal, bad_transpose):
        monkeypatch.setattr(oa, "_rows_block", bad)
        o, lse = oracle.attention(q, k, v, True, 0.5, threads=1)
        assert not (np.allclose(o, ob, atol=1e-6) and np.allclose(lse, lb, atol=1e-6)), bad.__name__
    monkeypatch.setattr(oa, "_rows_block", orig)
    # wrong GQA grouping (h % Hkv instead of h // g) is caught too
    o_mod = np.stack([oracle.attention(q[:, :, h:h + 1], k[:, :, h % 2:h % 2 + 1], v[:, :, h % 2:h % 2 + 1], True, 0.5, threads=1)[0][:, :, 0]
                      for h in range(4)], axis=2)
    assert not np.allclose(o_mod, ob, atol=1e-6)


def test_split_pages_view_gathers_the_same_tokens():
    """Seeing a pool of 16-token pages as pages of 1, 4 or 8 tokens (no data
    moved, block table rewritten) gathers the same tokens, so the oracle's
    decode is bitwise unchanged."""
    pg = W.paged(3, 8, 2, 128, 16, [1, 37, 160], seed=77)
    ro, rl = oracle.decode_paged(pg.q, pg.k_cache, pg.v_cache, pg.block_table, pg.seq_lens, pg.scale)
    for ps in (1, 4, 8):
        sp = W.split_pages(pg, ps)
        assert sp.k_cache.shape[1] == ps and sp.block_table.shape[1] == pg.block_table.shape[1] * 16 // ps
        assert sp.block_table.flags.c_contiguous
        so, sl = oracle.decode_paged(sp.q, sp.k_cache, sp.v_cache, sp.block_table, sp.seq_lens, sp.scale)
        assert np.array_equal(so, ro) and np.array_equal(sl, rl)
