"""Benchmark of the exact-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * the fused causal prefill forward at B=4, H=16, N=8192, d=128 (bf16),
  * the paged split-KV decode at B=64, Hq=32, Hkv=8, d=128, contexts
    U{512..32768}, page 16 (bf16), including its combine kernel,
  * the MX fp8 causal prefill forward at B=2, H=16, N=16384, d=128 (e4m3
    inputs with e8m0 block scales, P re-quantised to e4m3).
Inputs are resident in HBM before timing starts. Each kernel launch is timed
with HIP events recorded on the stream the kernels run on; the step time is the
wall clock over K steps between device synchronisations.

After the timed steps, further legs are timed on their own (HIP events, same
stream): the non-causal prefill, the long-context prefill (B=1, H=32, N=32768,
causal), the ragged batch (8 packed sequences of U{1024..32768} tokens, H=32,
causal) in input order and in the heaviest-first order of ea_varlen_lpt_order,
and the decode over 100 launches alternating between two copies of its pool.

Printed: one JSON line. ``value`` is the causal prefill throughput in TFLOP/s
(causal FLOPs counted as 4*B*H*N^2*d/2); the decode rate in GB/s of
algorithmic HBM bytes sits under ``decode``, the fp8 forward under ``fp8``, the
other legs under ``legs``. ``roofline`` describes the dominant kernel (the bf16
prefill forward, MFMA-bound); ``roofline_decode`` the decode (HBM-bound),
``roofline_fp8`` the fp8 forward. ``cpu_baseline`` times the CPU fp64 oracle on
a bounded sample of each workload on this host's cores, and ``parity`` compares
the GPU outputs of the timed launches with those oracle results element by
element (fp8: per (batch, head) slice, normwise). ``clock`` holds the shader
clock the driver reports while the prefill runs and the one measured inside
the kernel (shader cycles over wall clock ticks of its step loops), on which
``roofline.at_clock`` scales the MFMA peak; ``config`` holds the device and
ROCm version.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s (bf16 d=128 8K causal) + paged decode HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
O_ATOL, O_RTOL, LSE_ATOL = 1e-2, 1e-2, 1e-3       # bf16 outputs (elementwise), lse (absolute)
FP8_NORM_TOL, FP8_LSE_TOL = 5e-2, 5e-2            # MX fp8: normwise per (batch, head) slice
# HBM bytes per launch measured by rocprofv3 (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0,
# the factors a plain 1 GiB copy reads), keyed by the kernel they were taken
# on; a kernel not listed (or changed since) reports traffic null. Sources:
# profiles/*_counters.md.
TRAFFIC = {
    # fwd_pp_persistent_kernel<128, 128, causal>: 203,929 KiB fetched, 160,455 KiB written
    "ea::fwd_pp_persistent_kernel<128, 128, causal>": 581_953_599,
    # decode_split_kernel + combine: 2,372,532 KiB fetched, 5,728 KiB written
    "ea::decode_split_kernel + ea::decode_combine_kernel": 4_864_811_069,

    # fwd_mx8_sp_kernel<causal, e4m3>: 173,648 KiB fetched, 133,336 KiB written
    "ea::fwd_mx8_sp_kernel<causal, e4m3>": 492_166_827,
    # fwd_mx8_pp_persistent_kernel<causal, e4m3>: 101,508 KiB fetched, 133,125 KiB written
    "ea::fwd_mx8_pp_persistent_kernel<causal, e4m3>": 344_207_563,
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=30,
                   help="untimed steps first: the first tens of launches after idle run slower")
    p.add_argument("--exp-mode", type=int, default=0)
    p.add_argument("--rescale-log2", type=float, default=8.0, help="lazy-rescale threshold of the bf16 prefill")
    p.add_argument("--only", choices=["prefill", "decode", "fp8", "bwd"], default=None,
                   help="time one kernel family only (profiling runs; no extra legs)")
    p.add_argument("--with-bwd", action="store_true",
                   help="also time the backward (dQ, dK, dV) on the prefill workload; reported under 'bwd'")
    p.add_argument("--no-extra", action="store_true", help="skip the legs timed after the steps")
    p.add_argument("--extra-reps", type=int, default=5, help="timed launches per extra leg")
    p.add_argument("--decode-reps", type=int, default=100, help="timed launches of the long decode leg")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-gemm-calibration", action="store_true",
                   help="skip the vendor-GEMM rate measured after the timed region")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle time budget per main leg")
    p.add_argument("--cpu-seconds-extra", type=float, default=5.0, help="CPU oracle time budget per extra leg")
    p.add_argument("--prefill-kernel", type=int, default=0,
                   help="forward kernel for the bf16 prefill (EA_FWD_KERNEL_*; 0 = library default)")
    p.add_argument("--prefill-dims", choices=["128,128", "192,128", "64,64"], default="128,128",
                   help="head dims (d_qk, d_v) of the bf16 prefill forward")
    p.add_argument("--fp8-kernel", type=int, default=0, help="fp8 forward kernel (EA_FWD_KERNEL_*; 0 = default)")
    p.add_argument("--bwd-schedule", type=int, default=0, help="backward schedule (EA_BWD_SCHEDULE_*; 0 = default)")
    p.add_argument("--fp8-format", choices=["e4m3", "e5m2"], default="e4m3",
                   help="element format of the fp8 forward's MX inputs")
    p.add_argument("--decode-page-size", type=int, choices=[1, 2, 4, 8, 16], default=16,
                   help="view the decode pool as pages of this many tokens (same tokens, same memory)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy (calibrates HBM byte counters)")
    return p.parse_args()


def copy_calibration():
    """A plain copy of 1 GiB (reads 1 GiB, writes 1 GiB), repeated 3 times, so
    rocprofv3 FETCH_SIZE / WRITE_SIZE per dispatch can be scaled to bytes."""
    import torch
    x = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    x.fill_(1)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": 1 << 30, "calls": 3}))


def gemm_rate(torch, dev, dtype_name, n, reps=10):
    """TFLOP/s of one n^3 GEMM through the vendor BLAS (median of reps), or None."""
    try:
        if dtype_name == "bf16":
            a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
            b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
            run = lambda: a @ b  # noqa: E731
        else:
            a = torch.randn(n, n, device=dev).to(torch.float8_e4m3fn)
            b = torch.randn(n, n, device=dev).to(torch.float8_e4m3fn).t().contiguous().t()
            one = torch.ones((), device=dev)
            run = lambda: torch._scaled_mm(a, b, scale_a=one, scale_b=one, out_dtype=torch.bfloat16)  # noqa: E731
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        del a, b
        return 2.0 * n ** 3 / (float(np.median(ts)) * 1e-3) / 1e12
    except Exception:  # noqa: BLE001 -- an unavailable GEMM type leaves the field null
        return None


def mfma_loop_rate(torch, ea, dev, reps=5):
    """TFLOP/s of the library's calibration loop (ea_test_mfma_loop: bf16
    32x32x16 MFMAs from registers, 8 waves per workgroup, 1024 workgroups),
    median of reps launches, or None."""
    blocks, iters = 1024, 4000
    out = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream(dev)
    ts = []
    for i in range(reps + 1):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        if ea.lib().ea_test_mfma_loop(ea._ptr(out), blocks, iters, s.cuda_stream) != 0:
            return None
        e1.record(s)
        torch.cuda.synchronize()
        if i:
            ts.append(e0.elapsed_time(e1))
    flops = blocks * 8.0 * iters * 16 * 32768
    return flops / (float(np.median(ts)) * 1e-3) / 1e12


def mfma_loop_data_rate(torch, ea, dev, fmt, reps=5):
    """TFLOP/s of the random-operand calibration loop (ea_test_mfma_loop_data:
    fmt 0 bf16 32x32x16, fmt 1 MX e4m3 32x32x64; every MFMA takes new operands
    drawn N(0,1) like the workloads', so the matrix cores toggle as in the
    attention products), 8 waves per workgroup, 1024 workgroups, median of
    reps launches, or None."""
    blocks = 1024
    iters = 4000 if fmt == 0 else 1000
    nbytes = ea.lib().ea_test_mfma_loop_data_bytes(fmt)
    g = torch.Generator().manual_seed(11 + fmt)
    if fmt == 0:
        ops = torch.randn(nbytes // 2, generator=g).to(torch.bfloat16).view(torch.uint8).to(dev)
    else:
        ops = torch.randn(nbytes, generator=g).to(torch.float8_e4m3fn).view(torch.uint8).to(dev)
    out = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream(dev)
    ts = []
    for i in range(reps + 1):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        if ea.lib().ea_test_mfma_loop_data(ea._ptr(ops), ops.numel(), ea._ptr(out), blocks, iters, fmt,
                                           s.cuda_stream) != 0:
            return None
        e1.record(s)
        torch.cuda.synchronize()
        if i:
            ts.append(e0.elapsed_time(e1))
    flops = blocks * 8.0 * iters * 16 * (32768 if fmt == 0 else 131072)
    return flops / (float(np.median(ts)) * 1e-3) / 1e12


def stream_read_rate(torch, ea, dev, reps=5):
    """GB/s of the library's streaming-read calibration (ea_test_stream_read:
    4 GiB read once by 8192 workgroups of 256 threads, 16 loads of 16 B in
    flight per thread), best of reps launches, or None."""
    nbytes, blocks = 4 << 30, 8192
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream(dev)
    best = None
    for i in range(reps + 1):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        if ea.lib().ea_test_stream_read(ea._ptr(buf), nbytes, ea._ptr(out), blocks, s.cuda_stream) != 0:
            return None
        e1.record(s)
        torch.cuda.synchronize()
        if i:
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
    del buf
    return nbytes / (best * 1e-3) / 1e9


class ClockSampler:
    """Shader (gfx) clock and socket power read from the driver (amdsmi GPU
    metrics) every ~10 ms on a thread while the GPU works; None if the metrics
    are unavailable."""

    def __init__(self):
        self.samples, self.power, self._stop, self._th, self._h = [], [], threading.Event(), None, None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception:  # noqa: BLE001 -- no metrics: the clock fields stay null
            self._h = None

    def _read(self):
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._h)
        clks = m.get("current_gfxclks")
        if isinstance(clks, (list, tuple)):
            vals = [c for c in clks if isinstance(c, (int, float)) and 0 < c < 10000]
            if vals:
                return float(np.mean(vals)), m.get("average_socket_power")
        c = m.get("current_gfxclk")
        if isinstance(c, (int, float)) and 0 < c < 10000:
            return float(c), m.get("average_socket_power")
        return None, None

    def __enter__(self):
        if self._h is not None:
            def loop():
                while not self._stop.is_set():
                    try:
                        c, p = self._read()
                        if c is not None:
                            self.samples.append(c)
                        if isinstance(p, (int, float)) and p > 0:
                            self.power.append(float(p))
                    except Exception:  # noqa: BLE001
                        return
                    time.sleep(0.01)
            self._th = threading.Thread(target=loop, daemon=True)
            self._th.start()
        return self

    def __exit__(self, *a):
        self._stop.set()
        if self._th is not None:
            self._th.join()

    def result(self):
        if not self.samples:
            return None
        s = np.asarray(self.samples)
        return {"sclk_mhz_median": float(np.median(s)), "sclk_mhz_min": float(s.min()),
                "sclk_mhz_max": float(s.max()), "samples": int(s.size),
                "socket_power_w_median": float(np.median(self.power)) if self.power else None,
                "source": "amdsmi GPU metrics (current gfx clock, mean over XCDs), polled while the causal "
                          "prefill forward runs back to back; the driver's figure, which can stay at the "
                          "clock's upper limit while the cores run slower (see clock.in_kernel)"}


def device_market_name():
    """The GPU's marketing name from the driver (amdsmi), when torch reports none."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
        name = amdsmi.amdsmi_get_gpu_asic_info(h).get("market_name")
        return str(name) if name else None
    except Exception:  # noqa: BLE001 -- no driver metrics: the field stays null
        return None


def rocm_version():
    try:
        with open("/opt/rocm/.info/version") as f:
            v = f.read().strip()
    except OSError:
        v = None
    import torch
    return {"rocm": v, "torch_hip": torch.version.hip, "torch": torch.__version__}


def prefill_flops(B, H, N, d, dv=None, causal=True):
    """Forward FLOPs: 2 N^2 d (scores) + 2 N^2 dv (P V) per (batch, head);
    causal counted as half of the full N x N work."""
    f = 2.0 * B * H * N * N * (d + (dv or d))
    return f / 2.0 if causal else f


def varlen_flops(lengths, H, d, causal=True):
    L = np.asarray(lengths, dtype=np.float64)
    f = float((2.0 * H * L * L * (2 * d)).sum())
    return f / 2.0 if causal else f


def decode_bytes(seq_lens, Hq, Hkv, d, page_size):
    L = np.asarray(seq_lens, dtype=np.int64)
    kv = int(L.sum()) * Hkv * d * 2 * 2                 # K and V, bf16
    qo = 2 * len(L) * Hq * d * 2                        # q read + o written, bf16
    bt = 4 * int(((L + page_size - 1) // page_size).sum()) + 4 * len(L)
    return kv + qo + bt


def _f64(bits):
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


class Parity:
    """Running elementwise comparison of GPU outputs with oracle results."""

    def __init__(self, normwise=False):
        self.normwise = normwise
        self.max_o = self.max_excess = self.max_lse = self.max_norm = 0.0
        self.units = 0
        self.finite = True

    def add(self, o, ro, lse, rl):
        o, ro = np.asarray(o, np.float64), np.asarray(ro, np.float64)
        lse, rl = np.asarray(lse, np.float64), np.asarray(rl, np.float64)
        self.finite &= bool(np.isfinite(o).all())
        if o.size:
            self.max_o = max(self.max_o, float(np.abs(o - ro).max()))
            self.max_excess = max(self.max_excess, float((np.abs(o - ro) - O_RTOL * np.abs(ro)).max()))
            den = np.linalg.norm(ro)
            if den > 0:
                self.max_norm = max(self.max_norm, float(np.linalg.norm(o - ro) / den))
        both = np.isneginf(lse) & np.isneginf(rl)
        dl = np.where(both, 0.0, np.abs(lse - rl))
        if dl.size:
            self.max_lse = max(self.max_lse, float(np.nanmax(dl)) if not np.isnan(dl).any() else float("inf"))
        self.units += 1

    def result(self, what):
        if self.units == 0:
            return None
        if self.normwise:
            ok = self.finite and self.max_norm <= FP8_NORM_TOL and self.max_lse <= FP8_LSE_TOL
            crit = f"||o - o_ref||_F <= {FP8_NORM_TOL} ||o_ref||_F per slice, |lse - lse_ref| <= {FP8_LSE_TOL}"
        else:
            ok = self.finite and self.max_excess <= O_ATOL and self.max_lse <= LSE_ATOL
            crit = f"|o - o_ref| <= {O_ATOL} + {O_RTOL} |o_ref|, |lse - lse_ref| <= {LSE_ATOL}"
        return {"compared": what, "max_abs_o": self.max_o, "max_normwise_o": self.max_norm,
                "max_abs_lse": self.max_lse, "criterion": crit, "within_tol": bool(ok)}


def oracle_dense_slices(inp, o_gpu, lse_gpu, budget_s, causal, threads):
    """The oracle on whole (batch, head) slices of a dense workload until the
    time budget is used: achieved TFLOP/s and parity against the GPU outputs."""
    import oracle
    B, N, H, d = inp.q.shape
    Hkv = inp.k.shape[2]
    g = H // Hkv
    par = Parity()
    done, t_cpu, n = 0.0, 0.0, 0
    for b in range(B):
        for h in range(H):
            q = _f64(inp.q[b:b + 1, :, h:h + 1])
            k = _f64(inp.k[b:b + 1, :, h // g:h // g + 1])
            v = _f64(inp.v[b:b + 1, :, h // g:h // g + 1])
            t0 = time.perf_counter()
            ro, rl = oracle.attention(q, k, v, causal, inp.scale, threads=threads)
            t_cpu += time.perf_counter() - t0
            done += prefill_flops(1, 1, N, d, inp.v.shape[3], causal)
            n += 1
            if o_gpu is not None:
                par.add(o_gpu[b, :, h], ro[0, :, 0], lse_gpu[b, h], rl[0, 0])
            if t_cpu > budget_s:
                break
        if t_cpu > budget_s:
            break
    return done / t_cpu / 1e12, n, t_cpu, par


def oracle_varlen_slices(inp, o_gpu, lse_gpu, budget_s, threads):
    """The oracle on whole (sequence, head) slices of a packed workload, the
    sequences shortest first, until the time budget is used."""
    import oracle
    L = np.diff(inp.cu_q)
    H = inp.q.shape[1]
    d = inp.q.shape[2]
    par = Parity()
    done, t_cpu, n = 0.0, 0.0, 0
    for s in np.argsort(L, kind="stable"):
        a, m = int(inp.cu_q[s]), int(L[s])
        for h in range(H):
            t0 = time.perf_counter()
            ro, rl = oracle.attention(_f64(inp.q[None, a:a + m, h:h + 1]), _f64(inp.k[None, a:a + m, h:h + 1]),
                                      _f64(inp.v[None, a:a + m, h:h + 1]), True, inp.scale, threads=threads)
            t_cpu += time.perf_counter() - t0
            done += varlen_flops([m], 1, d)
            n += 1
            par.add(o_gpu[a:a + m, h], ro[0, :, 0], lse_gpu[h, a:a + m], rl[0, 0])
            if t_cpu > budget_s:
                return done / t_cpu / 1e12, n, t_cpu, par
    return done / t_cpu / 1e12, n, t_cpu, par


def oracle_decode(pg, o_gpu, lse_gpu, budget_s, threads):
    import oracle
    import workloads as W
    par = Parity()
    t_total, nbytes, seqs = 0.0, 0, 0
    for b in range(pg.q.shape[0]):
        sub = W.host_subpool(pg, [b])            # copy to host, untimed
        t0 = time.perf_counter()
        ro, rl = oracle.decode_paged(sub.q, sub.k_cache, sub.v_cache, sub.block_table, sub.seq_lens, sub.scale,
                                     threads=threads)
        t_total += time.perf_counter() - t0
        nbytes += decode_bytes(sub.seq_lens, pg.q.shape[1], sub.k_cache.shape[2], pg.q.shape[2], pg.page_size)
        seqs += 1
        par.add(o_gpu[b], ro[0], lse_gpu[b], rl[0])
        if t_total > budget_s:
            break
    return nbytes / t_total / 1e9, seqs, t_total, par


def oracle_mx8_slices(m8, o_gpu, lse_gpu, budget_s, threads):
    """The oracle on the dequantised inputs of whole (batch, head) slices."""
    import oracle
    B, N, H, d = m8.q8.shape
    par = Parity(normwise=True)
    done, t_cpu, n = 0.0, 0.0, 0
    for b in range(B):
        for h in range(H):
            q = oracle.dequant_mx(m8.q8[b:b + 1, :, h:h + 1], m8.q_scale[b:b + 1, :, h:h + 1], axis=3, fmt=m8.fmt)
            k = oracle.dequant_mx(m8.k8[b:b + 1, :, h:h + 1], m8.k_scale[b:b + 1, :, h:h + 1], axis=3, fmt=m8.fmt)
            v = oracle.dequant_mx(m8.v8[b:b + 1, :, h:h + 1], m8.v_scale[b:b + 1, :, h:h + 1], axis=1, fmt=m8.fmt)
            t0 = time.perf_counter()
            ro, rl = oracle.attention(q, k, v, True, m8.scale, threads=threads)
            t_cpu += time.perf_counter() - t0
            done += prefill_flops(1, 1, N, d)
            n += 1
            par.add(o_gpu[b, :, h], ro[0, :, 0], lse_gpu[b, h], rl[0, 0])
            if t_cpu > budget_s:
                return done / t_cpu / 1e12, n, t_cpu, par
    return done / t_cpu / 1e12, n, t_cpu, par


def time_events(torch, stream, fn, reps, warmup=1):
    """Per-launch milliseconds of fn() from HIP events on stream."""
    for _ in range(warmup):
        fn()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        ts.append((e0, e1))
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ts])


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path: the per-GPU kernels are each GPU's share.", file=sys.stderr)
        sys.exit(2)
    import torch

    import exact_attention_amd as ea
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    threads = len(os.sched_getaffinity(0))

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def host_f64(t):
        return _f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))

    run_prefill = args.only in (None, "prefill")
    run_decode = args.only in (None, "decode")
    run_fp8 = args.only in (None, "fp8")
    run_bwd = args.only == "bwd" or (args.only is None and args.with_bwd)
    run_extra = args.only is None and not args.no_extra
    t_gen = time.perf_counter()
    if run_prefill:
        d_qk, d_v = (int(x) for x in args.prefill_dims.split(","))
        inp = W.prefill(True) if d_qk == 128 else W.dense(4, 8192, 8192, 16, 16, d_qk, True, seed=1192, dv=d_v)
        q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
        o = torch.empty_like(q) if d_v == d_qk else torch.empty(q.shape[:3] + (d_v,), dtype=q.dtype, device=dev)
        B, N, H, d = inp.q.shape
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        tun = ea.tuning(exp_mode=args.exp_mode, kernel=args.prefill_kernel, rescale_log2=args.rescale_log2)
    if run_decode:
        pg = W.paged_decode_device(dev)
        if args.decode_page_size != 16:
            pg = W.split_pages(pg, args.decode_page_size)
        dq = dev_bf16(pg.q)
        bt = torch.from_numpy(np.ascontiguousarray(pg.block_table)).to(dev)
        sl = torch.from_numpy(np.ascontiguousarray(pg.seq_lens)).to(dev)
        assert bt.is_contiguous() and pg.k_cache.is_contiguous() and pg.v_cache.is_contiguous()
        Bd, Hq, dd = pg.q.shape
        Hkv = pg.k_cache.shape[2]
        ws = torch.empty(ea.decode_workspace_size(Bd, Hq, Hkv, dd, bt.shape[1] * pg.page_size, pg.page_size),
                         dtype=torch.uint8, device=dev)
        # a second copy of the pool with its pages in another order, so repeats
        # alternate between two 4.4 GB pools and cannot be served from cache
        perm = torch.randperm(pg.k_cache.shape[0], generator=torch.Generator().manual_seed(5)).to(dev)
        inv = torch.empty_like(perm)
        inv[perm] = torch.arange(perm.numel(), device=dev)
        kc2, vc2 = pg.k_cache[perm], pg.v_cache[perm]
        bt2 = torch.where(bt >= 0, inv[bt.clamp(min=0).long()].int(), bt)
        pools = [(pg.k_cache, pg.v_cache, bt), (kc2, vc2, bt2)]
        do = torch.empty_like(dq)
        dlse = torch.empty((Bd, Hq), dtype=torch.float32, device=dev)
    if run_bwd:
        bin_ = W.prefill(True)
        bq, bk, bv = dev_bf16(bin_.q), dev_bf16(bin_.k), dev_bf16(bin_.v)
        bB, bN, bH, bd = bin_.q.shape
        bdo = dev_bf16(W.normal_bf16_bits(1002, W.STREAM_DO, (bB, bN, bH, bd)))
        bo, blse = ea.attn_fwd(bq, bk, bv, True, bin_.scale)
        bws = torch.empty(ea.lib().ea_attn_bwd_workspace_size(bB, bH, bN), dtype=torch.uint8, device=dev)
        bdq, bdk, bdv = torch.empty_like(bq), torch.empty_like(bk), torch.empty_like(bv)
    if run_fp8:
        m8 = W.fp8_prefill(args.fp8_format)
        t8 = [torch.from_numpy(np.ascontiguousarray(x)).to(dev)
              for x in (m8.q8, m8.k8, m8.v8, m8.q_scale_dev, m8.k_scale_dev, m8.v_scale)]
        B8, N8, H8, d8 = m8.q8.shape
        o8 = torch.empty((B8, N8, H8, d8), dtype=torch.bfloat16, device=dev)
        tun8 = ea.tuning(kernel=args.fp8_kernel)
        lse8 = torch.empty((B8, H8, N8), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen

    def launch_decode(i):
        kc_, vc_, bt_ = pools[i % 2]
        r = ea.lib().ea_attn_decode_paged(ea._ptr(dq), ea._ptr(kc_), ea._ptr(vc_), ea._ptr(bt_), ea._ptr(sl),
                                        ea._ptr(do), ea._ptr(dlse), Bd, Hq, Hkv, dd, pg.page_size,
                                        kc_.shape[0], bt_.shape[1], pg.scale, 0, ea._ptr(ws), ws.numel(),
                                        stream.cuda_stream)
        ea._check(r, "ea_attn_decode_paged")

    def launch_prefill():
        ea.attn_fwd(q, k, v, True, inp.scale, tuning=tun, out=o, lse=lse)

    def step(i, ev):
        if run_bwd:
            ev[6].record(stream)
            r = ea.lib().ea_attn_bwd_ex(ea._ptr(bq), ea._ptr(bk), ea._ptr(bv), ea._ptr(bo), ea._ptr(bdo),
                                        ea._ptr(blse), ea._ptr(bdq), ea._ptr(bdk), ea._ptr(bdv), bB, bN, bN, bH, bH, bd,
                                        1, bin_.scale, args.bwd_schedule, ea._ptr(bws), bws.numel(),
                                        stream.cuda_stream)
            ea._check(r, "ea_attn_bwd_ex")
            ev[7].record(stream)
        if run_prefill:
            ev[0].record(stream)
            launch_prefill()
            ev[1].record(stream)
        if run_decode:
            ev[2].record(stream)
            launch_decode(i)
            ev[3].record(stream)
        if run_fp8:
            ev[4].record(stream)
            r = ea.lib().ea_attn_fwd_mx8_fmt(*[ea._ptr(x) for x in t8], ea._ptr(o8), ea._ptr(lse8), B8, N8, H8, H8,
                                            d8, 1, m8.scale, ea.FP8_FORMATS[m8.fmt], ctypes.byref(tun8),
                                            stream.cuda_stream)
            ea._check(r, "ea_attn_fwd_mx8_fmt")
            ev[5].record(stream)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(args.steps)]
    wev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    for i in range(args.warmup):
        step(i, wev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1), bf16-rounded)"}
    pf_dims = "d=128" if args.prefill_dims == "128,128" else f"(d_qk,d_v)=({args.prefill_dims})"
    cfg = {"workload": f"prefill fwd B=4 H=16 N=8192 {pf_dims} causal bf16 + paged decode B=64 Hq=32 Hkv=8 "
                       f"d=128 ctx U[512,32768] page {args.decode_page_size} bf16 (split-KV + LSE combine) + "
                       f"MX fp8 prefill fwd B=2 H=16 N=16384 d=128 causal",
           "exp_mode": args.exp_mode, "rescale_log2": args.rescale_log2, "prefill_kernel": args.prefill_kernel,
           "input_gen_s": round(t_gen, 1)}
    # GPU outputs of the last timed launch of each leg, for the parity records
    res = {}
    if run_prefill:
        res["prefill"] = (host_f64(o), lse.cpu().numpy().astype(np.float64))
        t_pf = np.array([e[0].elapsed_time(e[1]) for e in evs])      # ms
        flops = prefill_flops(B, H, N, d, d_v)
        tf = flops / (t_pf.mean() * 1e-3) / 1e12
        out["value"] = tf
        out["unit"] = "TFLOP/s"
        out["prefill"] = {"ms_mean": float(t_pf.mean()), "ms_min": float(t_pf.min()), "ms_median": float(np.median(t_pf)),
                          "tflops_best": flops / (t_pf.min() * 1e-3) / 1e12, "flop_per_launch": flops}
        out["roofline"] = {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": tf / PEAK_BF16_TFLOPS,
                           "kernel": ("ea::fwd_pp_unrollkv_kernel" if args.prefill_kernel == 5 else
                                      "ea::fwd_pp_persistent_kernel"
                                      if args.prefill_kernel == 4 or (args.prefill_kernel == 0 and d >= 128) else
                                      "ea::fwd_pp_kernel" if args.prefill_kernel == 2 else
                                      "ea::fwd_bf16_kernel") + f"<{d}, {d_v}, causal>"}
        out["roofline"]["traffic"] = TRAFFIC.get(out["roofline"]["kernel"])
    if run_decode:
        res["decode"] = (host_f64(do), dlse.cpu().numpy().astype(np.float64))
        t_dc = np.array([e[2].elapsed_time(e[3]) for e in evs])
        nbytes = decode_bytes(pg.seq_lens, Hq, Hkv, dd, pg.page_size)
        gbs = nbytes / (t_dc.mean() * 1e-3) / 1e9
        out["decode"] = {"value": gbs, "unit": "GB/s", "ms_mean": float(t_dc.mean()), "ms_min": float(t_dc.min()),
                         "bytes_per_launch": nbytes, "gbs_best": nbytes / (t_dc.min() * 1e-3) / 1e9,
                         "launches": int(t_dc.size)}
        out["roofline_decode"] = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": gbs / PEAK_HBM_GBS,
                                  "kernel": "ea::decode_split_kernel"
                                            " + ea::decode_combine_kernel"}
        # the counters were taken at page size 16
        out["roofline_decode"]["traffic"] = (TRAFFIC.get(out["roofline_decode"]["kernel"])
                                             if pg.page_size == 16 else None)
        if not run_prefill:
            out["value"], out["unit"] = gbs, "GB/s"
    if run_fp8:
        res["fp8"] = (host_f64(o8), lse8.cpu().numpy().astype(np.float64))
        t_8 = np.array([e[4].elapsed_time(e[5]) for e in evs])
        flops8 = prefill_flops(B8, H8, N8, d8)
        tf8 = flops8 / (t_8.mean() * 1e-3) / 1e12
        out["fp8"] = {"value": tf8, "unit": "TFLOP/s", "ms_mean": float(t_8.mean()), "ms_min": float(t_8.min()),
                      "flop_per_launch": flops8, "workload": f"B=2 H=16 N=16384 d=128 causal MX {m8.fmt}"}
        if run_prefill:
            out["fp8"]["ratio_to_bf16"] = tf8 / out["value"]
        out["roofline_fp8"] = {"bound": "mfma", "achieved": tf8, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                               "frac": tf8 / PEAK_FP8_TFLOPS,
                               "kernel": {0: "ea::fwd_mx8_pp_persistent_kernel", 4: "ea::fwd_mx8_pp_persistent_kernel",
                                          2: "ea::fwd_mx8_pp_kernel", 3: "ea::fwd_mx8_sp_kernel",
                                          1: "ea::fwd_mx8_kernel"}.get(
                                              args.fp8_kernel, f"fp8 kernel {args.fp8_kernel}")
                                         + f"<causal, {m8.fmt}>"}
        out["roofline_fp8"]["traffic"] = TRAFFIC.get(out["roofline_fp8"]["kernel"])
        if not (run_prefill or run_decode):
            out["value"], out["unit"], out["dtype"] = tf8, "TFLOP/s", f"fp8_{m8.fmt}"
    if run_bwd:
        t_bw = np.array([e[6].elapsed_time(e[7]) for e in evs])
        # algorithmic FLOPs of the backward: its five products (S, dP, dV, dK,
        # dQ), 2 N^2 d each, causal half
        flops_b = 5 * 2.0 * bB * bH * bN * bN * bd / 2.0
        tfb = flops_b / (t_bw.mean() * 1e-3) / 1e12
        out["bwd"] = {"value": tfb, "unit": "TFLOP/s", "ms_mean": float(t_bw.mean()), "ms_min": float(t_bw.min()),
                      "flop_per_launch": flops_b, "workload": "B=4 H=16 N=8192 d=128 causal bf16 (dQ, dK, dV)",
                      "flop_convention": "5 products x 2 N^2 d, causal half; the kernels compute 7 (S and dP twice)",
                      "kernels": ("ea::bwd_prep_kernel + ea::bwd_dq_persistent_kernel + ea::bwd_dkdv_persistent_kernel"
                                  if args.bwd_schedule == 2 else
                                  "ea::bwd_prep_kernel + ea::bwd_dq_kernel + ea::bwd_dkdv_kernel"),
                      "frac_of_peak": tfb / PEAK_BF16_TFLOPS}
        if not (run_prefill or run_decode or run_fp8):
            out["value"], out["unit"] = tfb, "TFLOP/s"

    # ---- legs timed after the steps
    legs = {}
    if run_decode and args.decode_reps > 0:
        t_long = time_events(torch, stream, lambda c=[0]: (launch_decode(c[0]), c.__setitem__(0, c[0] + 1)),
                             args.decode_reps)
        gl = nbytes / (t_long.mean() * 1e-3) / 1e9
        out["decode"]["long"] = {"launches": int(t_long.size), "ms_mean": float(t_long.mean()),
                                 "ms_median": float(np.median(t_long)), "ms_min": float(t_long.min()),
                                 "value": gl, "unit": "GB/s", "frac": gl / PEAK_HBM_GBS}
    if run_prefill and d == 128 and d_v == 128:
        sampler = ClockSampler()
        with sampler:
            time_events(torch, stream, launch_prefill, 200, warmup=0)
        out["clock"] = {"driver": sampler.result()}
        # lazy rescale and the shader clock under this load: back-to-back
        # launches of the statistics variant of the same kernel (outputs bit
        # for bit those of the timed kernel); the last launch's per-wave
        # counts, and its step loops' shader clock cycles (s_memtime) over
        # wall clock ticks (s_memrealtime at the device's wall clock rate)
        for _ in range(30):
            _, _, st = ea.test_fwd_rescale_stats(q, k, v, True, inp.scale, args.rescale_log2)
        t_st = time_events(torch, stream, lambda: ea.test_fwd_rescale_stats(q, k, v, True, inp.scale,
                                                                            args.rescale_log2), 1, warmup=0)
        _, _, st = ea.test_fwd_rescale_stats(q, k, v, True, inp.scale, args.rescale_log2)
        st = st.cpu().numpy().astype(np.int64)
        live, resc = int(st[:, :, 0].sum()), int(st[:, :, 1].sum())
        first = int((st[:, :, 0] > 0).sum())
        out["prefill"]["lazy_rescale"] = {
            "threshold_log2": args.rescale_log2, "wave_steps_with_keys": live, "rescaled": resc,
            "skipped_fraction": 1 - resc / live,
            "skipped_fraction_after_first_step": 1 - (resc - first) / max(live - first, 1),
            "what": "per wave of 32 rows and 64-key step: the running max moved (O and l rescaled) or not; a "
                    "wave's first step with keys always moves it off -inf"}
        has = st[:, :, 0] > 0
        khz = ea.test_wall_clock_khz()
        mhz = float(st[:, :, 2][has].sum() / st[:, :, 3][has].sum() * khz / 1e3)
        out["clock"]["in_kernel"] = {
            "shader_mhz": mhz, "wall_clock_khz": khz, "stats_launch_ms": float(t_st.mean()),
            "what": "sum over waves of shader clock cycles (s_memtime) / wall clock ticks (s_memrealtime) over the "
                    "forward's step loops, in the statistics launch after 30 back-to-back launches"}
        # where a step's cycles go: the phase-stamped launch of the same kernel
        # (one launch after the statistics launches; it runs a few per cent
        # slower than the plain kernel because of the stamps' waits)
        _, _, cy = ea.test_fwd_phase_cycles(q, k, v, True, inp.scale)
        cy = cy.cpu().numpy().astype(np.float64)
        steps = cy[:, :, 6].sum(axis=0)
        tiles = cy[:, :, 7].sum(axis=0)
        part = cy[:, :, :4].sum(axis=0) / steps[:, None]
        bound = cy[:, :, 4:6].sum(axis=0) / tiles[:, None]
        wave_cycles = cy[:, :, :6].sum()
        out["prefill"]["phases"] = {
            "what": "shader cycles per 64-key step and per tile, mean over waves (ea_test_fwd_phase_cycles); "
                    "waves 0-3 fetch K and waves 4-7 fetch V, spread over their VALU parts; a wave's MFMA part runs beside "
                    "the other group's VALU part on the same SIMD; ideal MFMA part = 32 MFMAs x 32 cycles = 1024",
            "group_a_per_step": {"mfma_part": float(part[:4, 0].mean()), "wait_after_mfma": float(part[:4, 1].mean()),
                                 "valu_part": float(part[:4, 2].mean()),
                                 "wait_after_valu": float(part[:4, 3].mean())},
            "group_b_per_step": {"mfma_part": float(part[4:, 0].mean()), "wait_after_mfma": float(part[4:, 1].mean()),
                                 "valu_part": float(part[4:, 2].mean()), "wait_after_valu": float(part[4:, 3].mean())},
            "per_tile": {"prologue": float(bound[:, 0].mean()), "epilogue": float(bound[:, 1].mean())},
            "tile_boundary_share": float(cy[:, :, 4:6].sum() / wave_cycles)}
        at_clock = PEAK_BF16_TFLOPS * mhz / 2400.0
        if "roofline" in out:
            tf = out["roofline"]["achieved"]
            out["roofline"]["at_clock"] = {
                "what": "dense bf16 MFMA peak scaled to the shader clock measured inside the kernel under this "
                        "load (2.5 PF/s at 2.4 GHz)", "clock_mhz": mhz, "peak": at_clock, "achieved": tf,
                "frac": tf / at_clock}
    if run_extra and run_prefill and d == 128 and d_v == 128:
        # non-causal prefill: same inputs
        o_nc = torch.empty_like(q)
        lse_nc = torch.empty_like(lse)
        t_nc = time_events(torch, stream, lambda: ea.attn_fwd(q, k, v, False, inp.scale, tuning=tun, out=o_nc,
                                                              lse=lse_nc), args.extra_reps)
        f_nc = prefill_flops(B, H, N, d, causal=False)
        legs["prefill_noncausal"] = {"workload": "B=4 H=16 N=8192 d=128 non-causal bf16", "ms_mean": float(t_nc.mean()),
                                     "flop_per_launch": f_nc, "value": f_nc / (t_nc.mean() * 1e-3) / 1e12,
                                     "unit": "TFLOP/s"}
        res["prefill_noncausal"] = (host_f64(o_nc), lse_nc.cpu().numpy().astype(np.float64))
        del o_nc, lse_nc
        # long context 5(i)
        lc = W.long_context()
        lq, lk, lv = dev_bf16(lc.q), dev_bf16(lc.k), dev_bf16(lc.v)
        lo = torch.empty_like(lq)
        llse = torch.empty((1, lc.q.shape[2], lc.q.shape[1]), dtype=torch.float32, device=dev)
        t_lc = time_events(torch, stream, lambda: ea.attn_fwd(lq, lk, lv, True, lc.scale, out=lo, lse=llse),
                           args.extra_reps)
        f_lc = prefill_flops(1, lc.q.shape[2], lc.q.shape[1], 128)
        legs["long_context"] = {"workload": "B=1 H=32 N=32768 d=128 causal bf16", "ms_mean": float(t_lc.mean()),
                                "flop_per_launch": f_lc, "value": f_lc / (t_lc.mean() * 1e-3) / 1e12,
                                "unit": "TFLOP/s"}
        res["long_context"] = (host_f64(lo), llse.cpu().numpy().astype(np.float64))
        del lq, lk, lv, lo, llse
        # ragged 5(ii), input order and heaviest-first order
        rg = W.long_ragged()
        Lr = np.diff(rg.cu_q)
        rq, rk, rv = dev_bf16(rg.q), dev_bf16(rg.k), dev_bf16(rg.v)
        cu = torch.from_numpy(rg.cu_q).to(dev)
        f_rg = varlen_flops(Lr, rg.q.shape[1], 128)
        ro_ = {}
        for name, ordered in (("ragged", False), ("ragged_lpt", True)):
            order = None
            if ordered:
                order, _ = ea.varlen_lpt_order(cu, cu, True, 256)
            box = {}

            def run_rg(order=order, box=box):
                box["r"] = ea.attn_fwd_varlen(rq, rk, rv, cu, cu, int(Lr.max()), True, rg.scale, seq_order=order)

            t_rg = time_events(torch, stream, run_rg, args.extra_reps)
            legs[name] = {"workload": f"8 packed sequences (lengths {Lr.tolist()}) H=32 d=128 causal bf16"
                                      + (", heaviest-first sequence order (ea_varlen_lpt_order)" if ordered else
                                         ", the default order (input order at 256 (sequence, head) groups)"),
                          "ms_mean": float(t_rg.mean()), "flop_per_launch": f_rg,
                          "value": f_rg / (t_rg.mean() * 1e-3) / 1e12, "unit": "TFLOP/s"}
            ro_[name] = box["r"]
        if "ragged" in legs and "ragged_lpt" in legs:
            legs["ragged_lpt"]["speedup_vs_input_order"] = legs["ragged"]["ms_mean"] / legs["ragged_lpt"]["ms_mean"]
        res["ragged"] = (host_f64(ro_["ragged"][0]), ro_["ragged"][1].cpu().numpy().astype(np.float64))
        res["ragged_lpt"] = (host_f64(ro_["ragged_lpt"][0]), ro_["ragged_lpt"][1].cpu().numpy().astype(np.float64))
        del rq, rk, rv, ro_
        for leg in legs.values():
            if leg.get("unit") == "TFLOP/s":
                leg["roofline"] = {"bound": "mfma", "peak": PEAK_BF16_TFLOPS, "frac": leg["value"] / PEAK_BF16_TFLOPS}
    if legs:
        out["legs"] = legs

    if not args.no_gemm_calibration:
        for key, dt_name, n in (("roofline", "bf16", 8192), ("roofline_fp8", "fp8", 16384)):
            if key in out:
                r = gemm_rate(torch, dev, dt_name, n)
                out[key]["sustained"] = {
                    "what": f"vendor BLAS {dt_name} GEMM {n}^3 on this GPU", "unit": "TFLOP/s",
                    "value": r, "frac": (out[key]["achieved"] / r) if r else None}
        if "roofline_decode" in out:
            r = stream_read_rate(torch, ea, dev)
            out["roofline_decode"]["sustained"] = {
                "what": "streaming 16-B read of 4 GiB on all CUs (ea_test_stream_read), this GPU",
                "unit": "GB/s", "value": r, "frac": (out["roofline_decode"]["achieved"] / r) if r else None}
        if "roofline" in out:
            r = mfma_loop_rate(torch, ea, dev)
            out["roofline"]["mfma_loop"] = {
                "what": "register-operand bf16 MFMA loop on all CUs (ea_test_mfma_loop), this GPU",
                "unit": "TFLOP/s", "value": r, "frac": (out["roofline"]["achieved"] / r) if r else None}
        for key, fmt, dt_name in (("roofline", 0, "bf16"), ("roofline_fp8", 1, "MX e4m3")):
            if key in out:
                r = mfma_loop_data_rate(torch, ea, dev, fmt)
                out[key]["mfma_loop_random"] = {
                    "what": f"{dt_name} MFMA loop on all CUs with new N(0,1) operands for every MFMA "
                            "(ea_test_mfma_loop_data): the matrix-core rate under this GPU's power limit on "
                            "data like the workload's", "unit": "TFLOP/s", "value": r,
                    "frac": (out[key]["achieved"] / r) if r else None}
    props = torch.cuda.get_device_properties(dev)
    cfg["device"] = device_market_name() or props.name
    cfg["device_runtime_name"] = props.name
    cfg["gcn_arch"] = getattr(props, "gcnArchName", None)
    cfg["cus"] = props.multi_processor_count
    cfg["versions"] = rocm_version()
    out["config"] = cfg

    if not args.no_cpu_baseline:
        cb = {"kind": "oracle", "cores": threads}
        parity = {}
        if run_prefill and d == 128 and d_v == 128:
            o_h, l_h = res["prefill"]
            tfc, n_sl, dt, par = oracle_dense_slices(inp, o_h, l_h, args.cpu_seconds, True, threads)
            cb.update({"value": tfc, "unit": "TFLOP/s",
                       "sample": f"fp64 oracle on {n_sl} of {B * H} whole causal (batch, head) slices of the "
                                 f"prefill workload ({dt:.1f} s)"})
            parity["prefill"] = par.result(f"{n_sl} of {B * H} (batch, head) slices, every row and column")
        if run_decode:
            gbc, seqs, dt, par = oracle_decode(pg, *res["decode"], args.cpu_seconds, threads)
            cb["decode"] = {"value": gbc, "unit": "GB/s", "cores": threads,
                            "sample": f"fp64 oracle on {seqs} of {Bd} whole sequences of the decode workload "
                                      f"({dt:.1f} s)"}
            parity["decode"] = par.result(f"{seqs} of {Bd} sequences, all heads")
            if not run_prefill:
                cb.update({"value": gbc, "unit": "GB/s", "sample": cb["decode"]["sample"]})
        if run_fp8:
            tf8c, n_sl, dt, par = oracle_mx8_slices(m8, *res["fp8"], args.cpu_seconds, threads)
            cb["fp8"] = {"value": tf8c, "unit": "TFLOP/s", "cores": threads,
                         "sample": f"fp64 oracle on the dequantised inputs of {n_sl} of {B8 * H8} whole causal "
                                   f"(batch, head) slices of the MX fp8 workload ({dt:.1f} s)"}
            parity["fp8"] = par.result(f"{n_sl} of {B8 * H8} (batch, head) slices, normwise per slice")
        if "prefill_noncausal" in legs:
            tfc, n_sl, dt, par = oracle_dense_slices(inp, *res["prefill_noncausal"], args.cpu_seconds_extra,
                                                     False, threads)
            legs["prefill_noncausal"]["cpu_baseline"] = {
                "value": tfc, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                "sample": f"fp64 oracle on {n_sl} whole non-causal (batch, head) slices ({dt:.1f} s)"}
            legs["prefill_noncausal"]["parity"] = par.result(f"{n_sl} of {B * H} (batch, head) slices")
            tfc, n_sl, dt, par = oracle_dense_slices(lc, *res["long_context"], args.cpu_seconds_extra, True, threads)
            legs["long_context"]["cpu_baseline"] = {
                "value": tfc, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                "sample": f"fp64 oracle on {n_sl} whole heads of 32 ({dt:.1f} s)"}
            legs["long_context"]["parity"] = par.result(f"{n_sl} of 32 heads, every row")
            for name in ("ragged", "ragged_lpt"):
                tfc, n_sl, dt, par = oracle_varlen_slices(rg, *res[name], args.cpu_seconds_extra, threads)
                legs[name]["cpu_baseline"] = {
                    "value": tfc, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                    "sample": f"fp64 oracle on {n_sl} whole (sequence, head) slices, shortest sequences "
                              f"first ({dt:.1f} s)"}
                legs[name]["parity"] = par.result(f"{n_sl} (sequence, head) slices, every row")
        out["cpu_baseline"] = cb
        out["parity"] = parity
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
