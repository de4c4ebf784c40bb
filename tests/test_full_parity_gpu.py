"""Whole-output parity at the full workload sizes, in the launch configuration
the benchmark times (the library defaults): every element of the HIP output is
compared with the fp64 oracle on the same seeded inputs.

  * prefill (B=4, H=16, N=8192, d=128), causal and non-causal: all 2^21 rows of
    o (|o - o_ref| <= 1e-2 + 1e-2 |o_ref|) and lse (|lse - lse_ref| <= 1e-3);
  * long context (B=1, H=32, N=32768, causal) and the ragged batch (8 packed
    sequences of U{1024..32768} tokens, H=32, causal): the same bounds on every
    row;
  * paged decode (B=64, Hq=32, Hkv=8, contexts U{512..32768}, page 16): every
    sequence and head, and the same pool viewed as pages of 4 tokens;
  * MX fp8 prefill (B=2, H=16, N=16384, causal): every (batch, head) slice
    normwise, ||o - o_ref||_F <= 5e-2 ||o_ref||_F, and every lse within 5e-2.
The oracle is the plain two-pass softmax of "FlashAttention: not less compute,
less data movement" (section 01) in fp64, on a thread pool over rows.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _helpers import assert_lse_close, assert_o_close, dev_bf16, f64, host_bits, log

pytestmark = pytest.mark.gpu


def _fwd(inp):
    import exact_attention_amd as ea
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    o, lse = ea.attn_fwd(q, k, v, inp.causal, inp.scale)
    torch.cuda.synchronize()
    del q, k, v
    return f64(host_bits(o)), lse.cpu().numpy().astype(np.float64)


def _check_dense_per_batch(inp, o, lse):
    """Oracle one batch entry at a time (bounds the fp64 working set)."""
    B = inp.q.shape[0]
    for b in range(B):
        ro, rl = oracle.attention(f64(inp.q[b:b + 1]), f64(inp.k[b:b + 1]), f64(inp.v[b:b + 1]), inp.causal,
                                  inp.scale)
        e = assert_o_close(o[b:b + 1], ro, what=f"o[b={b}]")
        el = assert_lse_close(lse[b:b + 1], rl, what=f"lse[b={b}]")
        log(f"  b={b}: max|do|={e:.2e} max|dlse|={el:.2e}")


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_every_element(causal):
    inp = W.prefill(causal)
    log(f"full parity: prefill causal={causal} shape={inp.q.shape}")
    o, lse = _fwd(inp)
    _check_dense_per_batch(inp, o, lse)


def test_long_context_every_element():
    inp = W.long_context()
    log(f"full parity: long context shape={inp.q.shape}")
    o, lse = _fwd(inp)
    B, N, H, d = inp.q.shape
    # eight heads at a time (the oracle's fp64 copies of one head group stay small)
    for h0 in range(0, H, 8):
        sl = slice(h0, h0 + 8)
        ro, rl = oracle.attention(f64(inp.q[:, :, sl]), f64(inp.k[:, :, sl]), f64(inp.v[:, :, sl]), True,
                                  inp.scale)
        e = assert_o_close(o[:, :, sl], ro, what=f"o[h={h0}..{h0 + 7}]")
        el = assert_lse_close(lse[:, sl], rl, what=f"lse[h={h0}..{h0 + 7}]")
        log(f"  heads {h0}..{h0 + 7}: max|do|={e:.2e} max|dlse|={el:.2e}")


_RAGGED = {}


def _ragged():
    if "out" not in _RAGGED:
        import exact_attention_amd as ea
        inp = W.long_ragged()
        q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
        cu = torch.from_numpy(inp.cu_q).cuda()
        L = np.diff(inp.cu_q)
        o, lse = ea.attn_fwd_varlen(q, k, v, cu, cu, int(L.max()), True, inp.scale)
        torch.cuda.synchronize()
        _RAGGED["inp"] = inp
        _RAGGED["out"] = (f64(host_bits(o)), lse.cpu().numpy().astype(np.float64))
    return _RAGGED["inp"], _RAGGED["out"]


# the 8 sequences in four groups of similar oracle cost
@pytest.mark.parametrize("group", [0, 1, 2, 3])
def test_long_ragged_every_element(group):
    inp, (o, lse) = _ragged()
    L = np.diff(inp.cu_q)
    order = np.argsort(-L, kind="stable")
    seqs = {0: [order[0]], 1: [order[1], order[7]], 2: [order[2], order[6], order[5]], 3: [order[3], order[4]]}[group]
    for s in seqs:
        a, n = int(inp.cu_q[s]), int(L[s])
        log(f"full parity: ragged sequence {s} ({n} tokens)")
        ro, rl = oracle.attention(f64(inp.q[None, a:a + n]), f64(inp.k[None, a:a + n]), f64(inp.v[None, a:a + n]),
                                  True, inp.scale)
        e = assert_o_close(o[a:a + n], ro[0], what=f"o[s={s}]")
        el = assert_lse_close(lse[:, a:a + n], rl[0], what=f"lse[s={s}]")
        log(f"  max|do|={e:.2e} max|dlse|={el:.2e}")


def _decode(pg):
    import exact_attention_amd as ea
    q = dev_bf16(pg.q)
    bt = torch.from_numpy(np.ascontiguousarray(pg.block_table)).cuda()
    sl = torch.from_numpy(np.ascontiguousarray(pg.seq_lens)).cuda()
    o, lse = ea.attn_decode_paged(q, pg.k_cache, pg.v_cache, bt, sl, pg.page_size, pg.scale)
    torch.cuda.synchronize()
    return f64(host_bits(o)), lse.cpu().numpy().astype(np.float64)


def test_decode_every_sequence():
    pg = W.paged_decode_device("cuda")
    B = pg.q.shape[0]
    log(f"full parity: decode B={B} pages={pg.k_cache.shape[0]}")
    o16, l16 = _decode(pg)
    o4, l4 = _decode(W.split_pages(pg, 4))
    for b0 in range(0, B, 16):
        batch = list(range(b0, min(B, b0 + 16)))
        sub = W.host_subpool(pg, batch)
        ro, rl = oracle.decode_paged(sub.q, sub.k_cache, sub.v_cache, sub.block_table, sub.seq_lens, sub.scale)
        e = assert_o_close(o16[batch], ro, what=f"o[b={b0}..]")
        el = assert_lse_close(l16[batch], rl, what=f"lse[b={b0}..]")
        assert_o_close(o4[batch], ro, what=f"o page 4 [b={b0}..]")
        assert_lse_close(l4[batch], rl, what=f"lse page 4 [b={b0}..]")
        log(f"  sequences {b0}..{batch[-1]}: max|do|={e:.2e} max|dlse|={el:.2e}")


def test_fp8_prefill_every_slice():
    import exact_attention_amd as ea
    m = W.fp8_prefill()
    log(f"full parity: MX fp8 prefill shape={m.q8.shape}")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    o, lse = ea.attn_fwd_mx8(t(m.q8), t(m.k8), t(m.v8), t(m.q_scale_dev), t(m.k_scale_dev), t(m.v_scale), m.causal,
                             m.scale, fmt=m.fmt)
    torch.cuda.synchronize()
    o, lse = f64(host_bits(o)), lse.cpu().numpy().astype(np.float64)
    B, N, H, d = m.q8.shape
    worst = worst_l = 0.0
    for b in range(B):
        q = oracle.dequant_mx(m.q8[b:b + 1], m.q_scale[b:b + 1], axis=3, fmt=m.fmt)
        k = oracle.dequant_mx(m.k8[b:b + 1], m.k_scale[b:b + 1], axis=3, fmt=m.fmt)
        v = oracle.dequant_mx(m.v8[b:b + 1], m.v_scale[b:b + 1], axis=1, fmt=m.fmt)
        ro, rl = oracle.attention(q, k, v, True, m.scale)
        for h in range(H):
            num = np.linalg.norm(o[b, :, h] - ro[0, :, h])
            den = np.linalg.norm(ro[0, :, h])
            worst = max(worst, num / den)
        worst_l = max(worst_l, float(np.abs(lse[b] - rl[0]).max()))
        assert np.isfinite(o[b]).all()
    log(f"  worst normwise {worst:.3e}, max|dlse| {worst_l:.3e}")
    assert worst <= 5e-2 and worst_l <= 5e-2
