"""The allocation-free decode entry point (ea_attn_decode_paged_noalloc), for
callers that cannot allocate: through the C ABI, two calls in a row (the
second on a smaller batch, so the library's device array still holds the
first call's partials), each equal bit for bit to ea_attn_decode_paged with a
caller workspace on the same inputs, and within the oracle's tolerance."""
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


def _inputs(pg):
    q, kc, vc = dev_bf16(pg.q), dev_bf16(pg.k_cache), dev_bf16(pg.v_cache)
    bt = torch.from_numpy(pg.block_table).cuda()
    sl = torch.from_numpy(pg.seq_lens).cuda()
    return q, kc, vc, bt, sl


def test_noalloc_matches_workspace_entry_twice():
    import exact_attention_amd as ea
    lib = ea.lib()
    cases = [(W.paged(40, 32, 8, 128, 16, np.random.default_rng(900).integers(1, 6000, size=40), seed=900), 0),
             (W.paged(5, 8, 2, 128, 5, [1, 77, 300, 2, 1500], seed=901), 3)]
    for i, (pg, ns) in enumerate(cases):
        q, kc, vc, bt, sl = _inputs(pg)
        B, Hq, d = pg.q.shape
        Hkv, mp = pg.k_cache.shape[2], pg.block_table.shape[1]
        ps = pg.page_size
        need = lib.ea_decode_workspace_size(B, Hq, Hkv, d, mp * ps, ps, ns)
        assert 0 < need <= lib.ea_decode_noalloc_max_bytes()
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        o1, l1 = torch.empty_like(q), torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        o2, l2 = torch.empty_like(q), torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        log(f"no-alloc decode call {i}: B={B} Hq={Hq} Hkv={Hkv} page={ps} splits={ns} partials={need} B")
        st = lib.ea_attn_decode_paged(P(q), P(kc), P(vc), P(bt), P(sl), P(o1), P(l1), B, Hq, Hkv, d, ps,
                                      kc.shape[0], mp, pg.scale, ns, P(ws), need, None)
        assert st == 0, lib.ea_last_error()
        st = lib.ea_attn_decode_paged_noalloc(P(q), P(kc), P(vc), P(bt), P(sl), P(o2), P(l2), B, Hq, Hkv, d, ps,
                                              kc.shape[0], mp, pg.scale, ns, None)
        assert st == 0, lib.ea_last_error()
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        ro, rl = oracle.decode_paged(pg.q, pg.k_cache, pg.v_cache, pg.block_table, pg.seq_lens, pg.scale)
        assert_o_close(f64(host_bits(o2)), ro)
        assert_lse_close(l2.cpu().numpy(), rl)


def test_noalloc_rejects_partials_beyond_its_array():
    import exact_attention_amd as ea
    lib = ea.lib()
    # 4096 ranges x 64 query heads x 128 dims of fp32 partials: 134 MB > 16 MiB
    P0 = ctypes.c_void_p(0x1000)   # never dereferenced: the size check fails first
    st = lib.ea_attn_decode_paged_noalloc(P0, P0, P0, P0, P0, P0, None, 4, 64, 8, 128, 16, 100, 64, 0.1, 4096,
                                          None)
    assert st == -2 and b"16777216" in lib.ea_last_error()
