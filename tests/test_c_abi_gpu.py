"""The plain C entry points of include/ea.h called directly (ctypes, raw
device pointers, the default stream), not through the Python binding's
tuned / ordered / format variants: ea_attn_fwd, ea_attn_fwd_varlen,
ea_attn_fwd_mx8 and ea_attn_decode_paged, each against the fp64 oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _helpers import assert_lse_close, assert_o_close, dev_bf16, f64, host_bits, log

pytestmark = pytest.mark.gpu


def P(t):
    return ctypes.c_void_p(t.data_ptr())


def test_ea_attn_fwd_plain():
    import exact_attention_amd as ea
    lib = ea.lib()
    for (B, Nq, Nk, Hq, Hkv, d, causal) in [(2, 300, 300, 4, 2, 128, True), (1, 129, 257, 2, 1, 64, False)]:
        inp = W.dense(B, Nq, Nk, Hq, Hkv, d, causal, seed=800 + Nq)
        q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device="cuda")
        st = lib.ea_attn_fwd(P(q), P(k), P(v), P(o), P(lse), B, Nq, Nk, Hq, Hkv, d, int(causal), inp.scale, None)
        assert st == 0, lib.ea_last_error()
        torch.cuda.synchronize()
        ro, rl = oracle.attention(f64(inp.q), f64(inp.k), f64(inp.v), causal, inp.scale)
        e = assert_o_close(f64(host_bits(o)), ro)
        assert_lse_close(lse.cpu().numpy(), rl)
        # lse may be omitted
        o2 = torch.empty_like(q)
        st = lib.ea_attn_fwd(P(q), P(k), P(v), P(o2), None, B, Nq, Nk, Hq, Hkv, d, int(causal), inp.scale, None)
        assert st == 0
        torch.cuda.synchronize()
        assert torch.equal(o, o2)
        log(f"ea_attn_fwd {B, Nq, Nk, Hq, Hkv, d, causal}: max|do|={e:.2e}")


def test_ea_attn_fwd_varlen_plain():
    import exact_attention_amd as ea
    lib = ea.lib()
    L = [5, 300, 64, 1000]
    inp = W.varlen(L, L, 4, 2, 128, True, seed=810)
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    cu = torch.from_numpy(inp.cu_q).cuda()
    T = int(inp.cu_q[-1])
    o = torch.empty_like(q)
    lse = torch.empty((4, T), dtype=torch.float32, device="cuda")
    st = lib.ea_attn_fwd_varlen(P(q), P(k), P(v), P(o), P(lse), P(cu), P(cu), len(L), T, T, max(L), 4, 2, 128, 1,
                                inp.scale, None, None)
    assert st == 0, lib.ea_last_error()
    torch.cuda.synchronize()
    ro, rl = oracle.attention_varlen(f64(inp.q), f64(inp.k), f64(inp.v), inp.cu_q, inp.cu_k, True, inp.scale)
    assert_o_close(f64(host_bits(o)), ro)
    assert_lse_close(lse.cpu().numpy(), rl)


def test_ea_attn_fwd_mx8_plain():
    import exact_attention_amd as ea
    lib = ea.lib()
    m = W.mx8(1, 512, 2, 128, True, seed=820)
    t = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (m.q8, m.k8, m.v8, m.q_scale_dev, m.k_scale_dev,
                                                                      m.v_scale)]
    o = torch.empty((1, 512, 2, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 2, 512), dtype=torch.float32, device="cuda")
    st = lib.ea_attn_fwd_mx8(*[P(x) for x in t], P(o), P(lse), 1, 512, 2, 2, 128, 1, m.scale, None)
    assert st == 0, lib.ea_last_error()
    torch.cuda.synchronize()
    q = oracle.dequant_mx(m.q8, m.q_scale, axis=3)
    k = oracle.dequant_mx(m.k8, m.k_scale, axis=3)
    v = oracle.dequant_mx(m.v8, m.v_scale, axis=1)
    ro, rl = oracle.attention(q, k, v, True, m.scale)
    got = f64(host_bits(o))
    for h in range(2):
        rel = np.linalg.norm(got[0, :, h] - ro[0, :, h]) / np.linalg.norm(ro[0, :, h])
        assert rel <= 5e-2, rel
    assert np.abs(lse.cpu().numpy() - rl).max() <= 5e-2


def test_ea_attn_decode_paged_plain():
    import exact_attention_amd as ea
    lib = ea.lib()
    L = [1, 100, 2000, 16]
    pg = W.paged(len(L), 8, 2, 128, 16, L, seed=830)
    q, kc, vc = dev_bf16(pg.q), dev_bf16(pg.k_cache), dev_bf16(pg.v_cache)
    bt = torch.from_numpy(pg.block_table).cuda()
    sl = torch.from_numpy(pg.seq_lens).cuda()
    B, mp = pg.block_table.shape
    need = lib.ea_decode_workspace_size(B, 8, 2, 128, mp * 16, 16, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, 8), dtype=torch.float32, device="cuda")
    st = lib.ea_attn_decode_paged(P(q), P(kc), P(vc), P(bt), P(sl), P(o), P(lse), B, 8, 2, 128, 16,
                                  kc.shape[0], mp, pg.scale, 0, P(ws), need, None)
    assert st == 0, lib.ea_last_error()
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged(pg.q, pg.k_cache, pg.v_cache, pg.block_table, pg.seq_lens, pg.scale)
    assert_o_close(f64(host_bits(o)), ro)
    assert_lse_close(lse.cpu().numpy(), rl)
