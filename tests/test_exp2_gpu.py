"""Device exp2 units against float64 exp2, with the error bounds of
"FlashAttention4 close reading", section 3.1.3 (degree-3 maximum relative error
8.77e-5 and mean 5.43e-5 for a minimax fit; the kernel's own refit reaches
8.57e-5 / 5.44e-5 in fp32) and the clamp at -127 of the co-design page's hybrid
exponent section."""
import json
import os

import numpy as np
import pytest
import torch

import workloads as W
from _helpers import log

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden", "exp2_poly.json")


def _sweep():
    x = np.concatenate([np.linspace(-127, 0, 2_000_001, dtype=np.float64),
                        -np.logspace(-12, 0, 20001), [0.0, -1e-30, -126.5, -127.0]]).astype(np.float32)
    return x


@pytest.mark.parametrize("mode", [0, 1])
def test_exp2_accuracy(mode):
    import exact_attention_amd as ea
    g = json.load(open(GOLD))
    x = _sweep()
    y = ea.test_exp2(torch.from_numpy(x).cuda(), mode).cpu().numpy().astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    ok = ref > 2.0 ** -126          # normal-range results
    rel = np.abs(y[ok] / ref[ok] - 1)
    log(f"exp2 mode {mode}: max rel {rel.max():.3e} mean {rel.mean():.3e}")
    if mode == 0:
        assert rel.max() < 1e-6
    else:
        assert rel.max() <= 1.05 * g["max_rel_err"]["degree3"]
        assert rel.mean() <= 1.05 * g["mean_rel_err"]["degree3"]
        # after rounding to bf16, within one bf16 step of the rounded exact value on >= 99% of inputs
        yb = W.bf16_bits_to_f32(W.f32_to_bf16_bits(y[ok].astype(np.float32))).astype(np.float64)
        rb = W.bf16_bits_to_f32(W.f32_to_bf16_bits(ref[ok].astype(np.float32))).astype(np.float64)
        step = np.abs(rb) * 2.0 ** -7
        assert np.mean(np.abs(yb - rb) <= step) >= 0.99
        # clamp: far below -127 gives (almost) zero
        z = ea.test_exp2(torch.tensor([-200.0, -1e30, float("-inf")], device="cuda"), mode).cpu().numpy()
        assert np.all(np.abs(z) <= 2.0 ** -126)


def test_mfma_loop_calibration_runs():
    """The calibration loop used by bench.py launches and writes every lane."""
    import exact_attention_amd as ea
    out = torch.full((8 * 512,), float("nan"), dtype=torch.float32, device="cuda")
    assert ea.lib().ea_test_mfma_loop(ea._ptr(out), 8, 10, None) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("fmt", [0, 1])
def test_mfma_loop_data_calibration_runs(fmt):
    """The random-operand calibration loop (bf16, then MX e4m3) launches and
    writes a finite value on every lane."""
    import exact_attention_amd as ea
    nbytes = ea.lib().ea_test_mfma_loop_data_bytes(fmt)
    g = torch.Generator().manual_seed(7)
    x = torch.randn(nbytes // 2, generator=g) * 0.05
    ops = (x.to(torch.bfloat16).view(torch.uint8) if fmt == 0
           else torch.randn(nbytes, generator=g).to(torch.float8_e4m3fn).view(torch.uint8)).to("cuda")
    out = torch.full((8 * 512,), float("nan"), dtype=torch.float32, device="cuda")
    assert ea.lib().ea_test_mfma_loop_data(ea._ptr(ops), ops.numel(), ea._ptr(out), 8, 10, fmt, None) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


def test_stream_read_calibration_reads_every_byte():
    """The streaming-read calibration used by bench.py visits every 16-byte
    chunk once: with all chunks zero but one, exactly one thread's folded
    value is nonzero, and it equals that chunk's words folded by XOR."""
    import exact_attention_amd as ea
    blocks = 16
    nbytes = 65536 * blocks * 2                       # two grid passes
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    buf[4 * 12345: 4 * 12345 + 4] = torch.tensor([1, 2, 4, 8], dtype=torch.int32)
    out = torch.full((blocks * 256,), -1, dtype=torch.int32, device="cuda")
    assert ea.lib().ea_test_stream_read(ea._ptr(buf), nbytes, ea._ptr(out), blocks, None) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    nz = np.nonzero(o)[0]
    assert len(nz) == 1 and o[nz[0]] == (1 ^ 2 ^ 4 ^ 8)
    assert nz[0] == 12345 % (blocks * 256)             # chunk c is read by thread c mod (threads)
