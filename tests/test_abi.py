"""C ABI checks that need no GPU: the library builds, loads and exports every
function include/ea.h declares, and invalid arguments come back as error codes
from the host-side checks (no HIP call is reached)."""
import ctypes
import os
import re

import pytest

from _helpers import ROOT

HEADERS = [os.path.join(ROOT, "include", f) for f in ("ea.h", "ea_test.h")]


@pytest.fixture(scope="module")
def lib():
    import exact_attention_amd as ea
    if not os.path.exists(ea.LIB_PATH):
        from exact_attention_amd import build
        build.build()
    return ea.lib()


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ea_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("ea_attn_fwd", "ea_attn_fwd_hd", "ea_attn_bwd", "ea_attn_bwd_ex", "ea_attn_bwd_workspace_size", "ea_attn_fwd_varlen", "ea_attn_fwd_varlen_ordered", "ea_varlen_lpt_order",
              "ea_attn_fwd_mx8", "ea_attn_fwd_mx8_tuned", "ea_attn_fwd_mx8_fmt", "ea_attn_decode_paged",
              "ea_decode_workspace_size", "ea_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} missing from libexactattn.so"
    assert lib.ea_version() == 1


def _err(lib):
    return lib.ea_last_error().decode()


P = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def test_fwd_argument_errors(lib):
    f = lib.ea_attn_fwd
    assert f(None, P, P, P, None, 1, 8, 8, 2, 2, 128, 0, 0.1, None) == -1 and "non-null" in _err(lib)
    assert f(P, P, P, P, None, 0, 8, 8, 2, 2, 128, 0, 0.1, None) == -1
    assert f(P, P, P, P, None, 1, 8, 8, 3, 2, 128, 0, 0.1, None) == -1 and "multiple" in _err(lib)
    assert f(P, P, P, P, None, 1, 8, 8, 2, 2, 96, 0, 0.1, None) == -2
    assert f(P, P, P, P, None, 1, 8, 8, 2, 2, 128, 0, float("nan"), None) == -1
    assert f(P, P, P, P, None, 1, 8, 8, 2, 2, 128, 0, -1.0, None) == -1
    assert f(P, P, P, P, None, 1, 8, 8, 2, 2, 128, 2, 0.1, None) == -1


def test_fwd_head_dim_pair_errors(lib):
    import exact_attention_amd as ea
    g = lib.ea_attn_fwd_hd
    assert g(P, P, P, P, None, 1, 8, 8, 2, 2, 192, 64, 0, 0.1, None, None) == -2 and "(192, 64)" in _err(lib)
    assert g(P, P, P, P, None, 1, 8, 8, 2, 2, 128, 64, 0, 0.1, None, None) == -2
    assert g(P, P, P, P, None, 1, 8, 8, 2, 2, 192, 0, 0, 0.1, None, None) == -1
    assert g(None, P, P, P, None, 1, 8, 8, 2, 2, 192, 128, 0, 0.1, None, None) == -1
    for kern in (1, 3, 5):                                # (192, 128): ping-pong kernel (or its persistent form) only
        t = ea.tuning(kernel=kern)
        assert g(P, P, P, P, None, 1, 8, 8, 2, 2, 192, 128, 0, 0.1, ctypes.byref(t), None) == -2
    assert lib.ea_attn_fwd(P, P, P, P, None, 1, 8, 8, 2, 2, 192, 0, 0.1, None) == -2   # needs the _hd entry


def test_tuning_errors(lib):
    import exact_attention_amd as ea
    t = ea.tuning(exp_mode=7)
    assert lib.ea_attn_fwd_tuned(P, P, P, P, None, 1, 8, 8, 2, 2, 128, 0, 0.1, ctypes.byref(t), None) == -1
    t = ea.tuning(rescale_log2=-1.0)
    assert lib.ea_attn_fwd_tuned(P, P, P, P, None, 1, 8, 8, 2, 2, 128, 0, 0.1, ctypes.byref(t), None) == -1
    t = ea.tuning(kernel=6)
    assert lib.ea_attn_fwd_tuned(P, P, P, P, None, 1, 8, 8, 2, 2, 128, 0, 0.1, ctypes.byref(t), None) == -1
    assert "0, 1, 2, 3, 4 or 5" in _err(lib)
    # kernel 3 (pipelined) exists for MX fp8 only
    t = ea.tuning(kernel=3)
    assert lib.ea_attn_fwd_tuned(P, P, P, P, None, 1, 8, 8, 2, 2, 128, 0, 0.1, ctypes.byref(t), None) == -2
    assert "fp8 only" in _err(lib)
    assert lib.ea_attn_fwd_varlen(P, P, P, P, None, P, P, 2, 10, 10, 5, 2, 2, 128, 1, 0.1, ctypes.byref(t),
                                  None) == -2
    d = ea.default_tuning()
    assert d.exp_mode == 0 and d.rescale_log2 == 8.0 and d.natural_order == 0 and d.kernel == 0


def test_varlen_argument_errors(lib):
    f = lib.ea_attn_fwd_varlen
    assert f(P, P, P, P, None, None, P, 2, 10, 10, 5, 2, 2, 128, 1, 0.1, None, None) == -1
    assert f(P, P, P, P, None, P, P, 2, 10, 10, 50, 2, 2, 128, 1, 0.1, None, None) == -1  # max > total
    assert f(P, P, P, P, None, P, P, 2, 10, 10, 5, 2, 2, 80, 1, 0.1, None, None) == -2


def test_mx8_argument_errors(lib):
    f = lib.ea_attn_fwd_mx8
    assert f(P, P, P, P, P, None, P, None, 1, 64, 2, 2, 128, 1, 0.1, None) == -1
    assert f(P, P, P, P, P, P, P, None, 1, 48, 2, 2, 128, 1, 0.1, None) == -2   # N % 32
    assert f(P, P, P, P, P, P, P, None, 1, 64, 2, 2, 64, 1, 0.1, None) == -2    # d
    g = lib.ea_attn_fwd_mx8_fmt
    assert g(P, P, P, P, P, P, P, None, 1, 64, 2, 2, 128, 1, 0.1, 2, None, None) == -1   # no such format
    assert "in_format" in _err(lib)
    assert g(P, P, P, P, P, P, P, None, 1, 64, 2, 2, 64, 1, 0.1, 1, None, None) == -2    # d, e5m2


def test_mx8_tuning_errors(lib):
    import exact_attention_amd as ea
    f = lib.ea_attn_fwd_mx8_tuned

    def call(t):
        return f(P, P, P, P, P, P, P, None, 1, 64, 2, 2, 128, 1, 0.1, ctypes.byref(t), None)

    assert call(ea.tuning(exp_mode=1)) == -2    # hardware exponential only
    assert call(ea.tuning(natural_order=1)) == -2
    assert call(ea.tuning(kernel=5)) == -2      # no unroll-KV fp8 kernel
    assert call(ea.tuning(kernel=6)) == -1
    # P <= 2^rescale_log2 is rounded to e4m3 with scale 1: the threshold must
    # keep it under e4m3's 448 = 2^8.807...
    assert call(ea.tuning(rescale_log2=8.9)) == -2 and "448" in _err(lib)
    assert call(ea.tuning(rescale_log2=16.0)) == -2


def test_decode_argument_errors(lib):
    f = lib.ea_attn_decode_paged
    ws = lib.ea_decode_workspace_size(4, 8, 2, 128, 1024, 16, 0)
    assert ws > 0
    ok_args = dict(B=4, Hq=8, Hkv=2, d=128, ps=16, P=100, mp=64)

    def call(q=P, B=4, Hq=8, Hkv=2, d=128, ps=16, npages=100, mp=64, scale=0.1, ns=0, wsp=P, wsb=ws):
        return f(q, P, P, P, P, P, None, B, Hq, Hkv, d, ps, npages, mp, scale, ns, wsp, wsb, None)

    assert call(q=None) == -1
    assert call(Hq=6, Hkv=4) == -1
    assert call(d=64) == -2
    assert call(ps=8, npages=1 << 28) == -2  # pool of 2^31 token slots
    assert call(scale=0.0) == -1
    assert call(ns=-1) == -1
    assert call(wsb=ws - 1) == -4 and "workspace" in _err(lib)
    assert call(wsp=None) == -4
    # query heads beyond 16 per KV head take more (KV head, block) pairs per
    # range group, so the default range count and the workspace shrink
    assert lib.ea_decode_workspace_size(4, 64, 1, 128, 1024, 16, 0) > 0
    assert lib.ea_decode_workspace_size(4, 6, 4, 128, 1024, 16, 0) == 0   # Hq % Hkv
    # more splits need more workspace
    assert lib.ea_decode_workspace_size(4, 8, 2, 128, 1024, 16, 8) >= lib.ea_decode_workspace_size(4, 8, 2, 128, 1024, 16, 1)


def test_mfma_loop_argument_errors(lib):
    assert lib.ea_test_mfma_loop(None, 4, 10, None) == -1
    assert lib.ea_test_mfma_loop(P, 0, 10, None) == -1
    assert lib.ea_test_mfma_loop(P, 4, 0, None) == -1
    assert lib.ea_test_mfma_loop(P, 1 << 17, 10, None) == -1


def test_mfma_loop_data_argument_errors(lib):
    assert lib.ea_test_mfma_loop_data_bytes(0) == 512 * 8 * 2 * 16
    assert lib.ea_test_mfma_loop_data_bytes(1) == 512 * 8 * 2 * 32
    assert lib.ea_test_mfma_loop_data_bytes(2) == 0
    n0 = lib.ea_test_mfma_loop_data_bytes(0)
    f = lib.ea_test_mfma_loop_data
    assert f(None, n0, P, 4, 10, 0, None) == -1
    assert f(P, n0, None, 4, 10, 0, None) == -1
    assert f(P, n0, P, 0, 10, 0, None) == -1
    assert f(P, n0, P, 1 << 17, 10, 0, None) == -1
    assert f(P, n0, P, 4, 0, 0, None) == -1
    assert f(P, n0, P, 4, 10, 2, None) == -1
    assert f(P, n0 - 1, P, 4, 10, 0, None) == -4
    assert f(P, n0, P, 4, 10, 1, None) == -4     # fp8 pairs take twice the bytes


def test_phase_cycles_argument_errors(lib):
    assert lib.ea_test_fwd_phase_cycles_len(0, 8, 2) == 0
    f = lib.ea_test_fwd_phase_cycles

    def call(q=P, cyc=P, B=1, Nq=8, Nk=8, Hq=2, Hkv=2, causal=1, scale=0.1, n=1 << 20):
        return f(q, P, P, P, None, B, Nq, Nk, Hq, Hkv, causal, scale, cyc, n, None)

    assert call(q=None) == -1
    assert call(cyc=None) == -1
    assert call(Nk=0) == -1
    assert call(Hq=3) == -1
    assert call(causal=2) == -1
    assert call(scale=0.0) == -1


def test_varlen_lds_order_argument_errors(lib):
    f = lib.ea_test_varlen_lds_order
    assert f(None, P, 4, 1, P, None) == -1
    assert f(P, P, 4, 1, None, None) == -1
    assert f(P, P, 0, 1, P, None) == -1
    assert f(P, P, 4, 2, P, None) == -1
    assert f(P, P, 513, 1, P, None) == -2      # beyond one workgroup's threads


def test_bwd_argument_errors(lib):
    ws = lib.ea_attn_bwd_workspace_size(1, 2, 8)
    assert ws >= 2 * 2 * 8 * 4 and lib.ea_attn_bwd_workspace_size(0, 2, 8) == 0
    f = lib.ea_attn_bwd

    def call(q=P, lse=P, B=1, Nq=8, Nk=8, Hq=2, Hkv=2, d=128, causal=0, scale=0.1, wsp=P, wsb=ws):
        return f(q, P, P, P, P, lse, P, P, P, B, Nq, Nk, Hq, Hkv, d, causal, scale, wsp, wsb, None)

    assert call(q=None) == -1 and "non-null" in _err(lib)
    assert call(lse=None) == -1
    assert call(Nk=0) == -1
    assert call(Hq=3) == -1 and "multiple" in _err(lib)
    assert call(d=96) == -2
    assert call(scale=float("inf")) == -1
    assert call(causal=3) == -1
    assert call(wsb=ws - 1) == -4 and "workspace" in _err(lib)
    assert call(wsp=None) == -4
    g = lib.ea_attn_bwd_ex
    assert g(P, P, P, P, P, P, P, P, P, 1, 8, 8, 2, 2, 128, 0, 0.1, 3, P, ws, None) == -1 and "schedule" in _err(lib)


def test_binding_refuses_cpu_tensors():
    import torch
    import exact_attention_amd as ea
    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ea.attn_fwd(q, q, q)


def test_varlen_lpt_order_argument_errors(lib):
    f = lib.ea_varlen_lpt_order
    assert f(None, P, 4, 1, 256, P, P, None) == -1
    assert f(P, P, 4, 1, 256, None, P, None) == -1
    assert f(P, P, 0, 1, 256, P, P, None) == -1
    assert f(P, P, 4, 2, 256, P, P, None) == -1
    assert f(P, P, 4, 1, 100, P, P, None) == -1        # not a forward row block
    assert f(P, P, 1 << 17, 1, 256, P, P, None) == -2  # quadratic ranking: capped


def test_stream_read_errors(lib):
    f = lib.ea_test_stream_read
    out = ctypes.c_void_p(1)
    assert f(None, 1 << 20, out, 16, None) == -1
    assert f(P, 1 << 20, None, 16, None) == -1
    assert f(P, 1 << 20, out, 0, None) == -1
    assert f(P, 1000, out, 1, None) == -1          # not a whole grid pass
    assert f(P, 0, out, 1, None) == -1
