"""GPU tests of the work order against the scheduling oracle: the varlen LPT
batch order (ea_varlen_lpt_order), the forward walking sequences in that
order, and the dense forward's own tile order (the hierarchical traversal)."""
import numpy as np
import pytest
import torch

import oracle
import oracle.schedule as S
import workloads as W
from _helpers import assert_lse_close, assert_o_close, f64, host_bits, log

pytestmark = pytest.mark.gpu


def dev_order(cu_q, cu_k, causal, block_m):
    import exact_attention_amd as ea
    order, weights = ea.varlen_lpt_order(torch.from_numpy(np.asarray(cu_q, np.int32)).cuda(),
                                         torch.from_numpy(np.asarray(cu_k, np.int32)).cuda(), causal, block_m)
    torch.cuda.synchronize()
    return order.cpu().numpy().tolist(), weights.cpu().numpy().tolist()


def cu_of(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("block_m", [128, 256])
def test_order_matches_oracle(causal, block_m):
    rng = np.random.default_rng(41)
    for n in (1, 3, 7, 300, 1000):          # several ranking workgroups for n > 256
        lq = rng.integers(0, 5000, n)
        lk = lq + rng.integers(-200, 400, n) * (rng.random(n) < 0.5)
        lk = np.maximum(lk, 0)
        lq[rng.random(n) < 0.05] = 0          # sequences without queries
        lk[:n // 3] = lk[0]                   # many equal weights (ties keep input order)
        cu_q, cu_k = cu_of(lq), cu_of(lk)
        log(f"lpt order n={n} causal={causal} block_m={block_m}")
        order, weights = dev_order(cu_q, cu_k, causal, block_m)
        want_w = [S.seq_weight(int(a), int(b), causal, block_m, 64) for a, b in zip(lq, lk)]
        assert weights == want_w
        assert order == S.lpt_order(cu_q, cu_k, causal, block_m, 64)


def test_order_of_the_pages_example():
    # the close-reading page's permutation: 0,1,2,3 -> 1,2,3,0
    order, _ = dev_order([0, 64, 128, 192, 256], [0, 64, 320, 512, 640], False, 256)
    assert order == [1, 2, 3, 0]


@pytest.mark.parametrize("causal", [True, False])
def test_workgroup_order_matches_oracle(causal):
    """The order the ping-pong forward's workgroups compute for themselves
    (default varlen call) equals the scheduling oracle's LPT order with
    256-row blocks: weights, ties in input order, sequences without queries."""
    import exact_attention_amd as ea
    rng = np.random.default_rng(43)
    for n in (1, 2, 7, 64, 300, 512):
        lq = rng.integers(0, 9000, n)
        lk = np.maximum(lq + rng.integers(-300, 600, n) * (rng.random(n) < 0.5), 0)
        lq[rng.random(n) < 0.05] = 0
        lk[: n // 3] = lk[0]
        cu_q, cu_k = cu_of(lq), cu_of(lk)
        out = torch.full((n,), -7, dtype=torch.int32, device="cuda")
        log(f"workgroup LPT order n={n} causal={causal}")
        dq, dk = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()  # alive until the kernel ran
        st = ea.lib().ea_test_varlen_lds_order(ea._ptr(dq), ea._ptr(dk), n, int(causal), ea._ptr(out), None)
        assert st == 0
        torch.cuda.synchronize()
        assert out.cpu().numpy().tolist() == S.lpt_order(cu_q, cu_k, causal, 256, 64)


@pytest.mark.parametrize("kernel", [0, 2, 4])
@pytest.mark.parametrize("causal", [True, False])
def test_default_varlen_order_is_bitwise_the_input_order(kernel, causal):
    """The default varlen forward (its workgroups walk the sequences heaviest
    first) gives the bits of the input-order walk, and matches the oracle."""
    import exact_attention_amd as ea
    L = [40, 1300, 7, 600, 2100, 0, 333, 5000, 1]
    inp = W.varlen(L, L, 4, 2, 128, causal, seed=44)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    q, k, v = t(inp.q).view(torch.bfloat16), t(inp.k).view(torch.bfloat16), t(inp.v).view(torch.bfloat16)
    cu = t(inp.cu_q)
    log(f"default varlen order, kernel {kernel} causal {causal}")
    res = []
    for inorder in (False, True):
        o, lse = ea.attn_fwd_varlen(q, k, v, cu, cu, max(L), causal, inp.scale, tuning=ea.tuning(kernel=kernel),
                                    input_order=inorder)
        torch.cuda.synchronize()
        res.append((f64(host_bits(o)), lse.cpu().numpy().astype(np.float64)))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
    ro, rl = oracle.attention_varlen(f64(inp.q), f64(inp.k), f64(inp.v), inp.cu_q, inp.cu_k, causal, inp.scale)
    assert_o_close(res[0][0], ro)
    assert_lse_close(res[0][1], rl)


def run_varlen_ordered(inp, kernel, order=None, poison=None):
    import exact_attention_amd as ea
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    q, k, v = t(inp.q).view(torch.bfloat16), t(inp.k).view(torch.bfloat16), t(inp.v).view(torch.bfloat16)
    cu_q, cu_k = t(inp.cu_q), t(inp.cu_k)
    maxq = int(np.diff(inp.cu_q).max())
    o, lse = ea.attn_fwd_varlen(q, k, v, cu_q, cu_k, maxq, inp.causal, inp.scale,
                                tuning=ea.tuning(kernel=kernel), seq_order=order)
    torch.cuda.synchronize()
    return f64(host_bits(o)), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("kernel", [1, 2, 4, 5])
def test_forward_in_lpt_order_is_bitwise_the_same(kernel):
    import exact_attention_amd as ea
    L = [40, 1300, 7, 600, 2100, 0, 333]
    inp = W.varlen(L, L, 4, 2, 128, True, seed=42)
    cu_q = torch.from_numpy(inp.cu_q).cuda()
    order, _ = ea.varlen_lpt_order(cu_q, cu_q, True, 128 if kernel == 1 else 256)
    assert order.cpu().numpy().tolist() == S.lpt_order(inp.cu_q, inp.cu_k, True, 128 if kernel == 1 else 256, 64)
    log(f"varlen forward in LPT order, kernel {kernel}: {order.cpu().numpy().tolist()}")
    o1, l1 = run_varlen_ordered(inp, kernel)
    o2, l2 = run_varlen_ordered(inp, kernel, order)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    ro, rl = oracle.attention_varlen(f64(inp.q), f64(inp.k), f64(inp.v), inp.cu_q, inp.cu_k, True, inp.scale)
    assert_o_close(o2, ro)
    assert_lse_close(l2, rl)


def test_order_entry_out_of_range_contributes_no_rows():
    # documented behaviour: an entry outside [0, num_seqs) is skipped (and its
    # sequence, missing from the order, is not computed); the other sequences
    # are unaffected
    L = [100, 70, 200]
    inp = W.varlen(L, L, 2, 2, 128, True, seed=43)
    order = torch.tensor([2, -1, 0], dtype=torch.int32).cuda()
    o_all, _ = run_varlen_ordered(inp, 2)
    o, _ = run_varlen_ordered(inp, 2, order)
    a, b = int(inp.cu_q[1]), int(inp.cu_q[2])
    assert np.array_equal(o[:a], o_all[:a]) and np.array_equal(o[b:], o_all[b:])


@pytest.mark.parametrize("B,Hq,N,causal", [(4, 16, 8192, True), (2, 8, 1000, False), (1, 32, 700, True),
                                           (3, 2, 600, True), (1, 3, 300, False)])
def test_dense_order_is_hierarchical_lpt(B, Hq, N, causal):
    """The dense forward's work tiles, in dispatch order and as the kernels
    locate them on the device, follow the cache-aware hierarchical LPT
    traversal of "FlashAttention4 close reading" section 3.3 with sections of
    8 (batch, head) groups -- one per XCD, so each XCD's L2 serves one head at
    a time -- laid end to end; with Hq a multiple of 8 that is the page's
    batch-outermost loop with sections of 8 heads."""
    import exact_attention_amd as ea
    got = [tuple(int(x) for x in r) for r in ea.test_fwd_tile_order(B, N, N, Hq, causal).numpy()]
    n_mb = -(-N // 256)
    groups = B * Hq
    padded = 8 * -(-groups // 8)
    want = []
    for _, g, mb in S.hierarchical_tile_order(1, padded, n_mb, 8):
        want.append((g // Hq, g % Hq, mb) if g < groups else (-1, -1, -1))
    log(f"tile order B={B} Hq={Hq} N={N} causal={causal}: {len(got)} tiles")
    assert got == want
    if Hq % 8 == 0:
        assert [t for t in got if t[0] >= 0] == S.hierarchical_tile_order(B, Hq, n_mb, 8)
