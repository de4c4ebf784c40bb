"""Interleaved timing of two or more builds of the library on one workload.

    python -m exact_attention_amd.abtime WHAT LIB.so [LIB.so ...] [--rounds R] [--launches L]

WHAT is one of
  bf16     the prefill forward, B=4 H=16 N=8192 d=128 causal (ea_attn_fwd_hd)
  bf16nc   the same, non-causal
  bf16d64  the same shape with d = 64, causal (the 4-wave kernel by default)
  fp8      the MX fp8 forward, B=2 H=16 N=16384 d=128 causal e4m3 (ea_attn_fwd_mx8_fmt)
  decode   the paged decode, B=64 Hq=32 Hkv=8 d=128, contexts U[512, 32768], page 16 (ea_attn_decode_paged)
  bwd      the backward of the bf16 prefill workload (ea_attn_bwd_ex)
with the default tuning of each build. Each library is loaded on its own
(RTLD_LOCAL) before the GPU is touched; every build gets 30 warm-up launches,
then R rounds visit the builds in turn, each timing L launches (after 3
untimed ones) with HIP events on the current stream. A box's speed drifts by
a few per cent from run to run and within a run, so builds are only compared
within one invocation, round by round. Prints per build the median, min and
max milliseconds per launch over the rounds, and whether each build's outputs
equal the first one's bit for bit.
"""
from __future__ import annotations

import argparse
import ctypes

import numpy as np


def _load(path, signatures):
    lib = ctypes.CDLL(path, mode=ctypes.RTLD_LOCAL)
    for name, (args, res) in signatures.items():
        if hasattr(lib, name):  # an older build may lack newer entry points
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
    return lib


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=["bf16", "bf16nc", "bf16d64", "fp8", "bwd", "decode"])
    ap.add_argument("libs", nargs="+")
    ap.add_argument("--rounds", type=int, default=5)
    ap.add_argument("--launches", type=int, default=20)
    args = ap.parse_args(argv)
    import exact_attention_amd as ea
    import workloads as W

    libs = [_load(p, ea._SIGNATURES) for p in args.libs]
    import torch

    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    P = ea._ptr

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.what == "fp8":
        m8 = W.fp8_prefill("e4m3")
        t8 = [torch.from_numpy(np.ascontiguousarray(x)).to(dev)
              for x in (m8.q8, m8.k8, m8.v8, m8.q_scale_dev, m8.k_scale_dev, m8.v_scale)]
        B, N, H, d = m8.q8.shape
        outs = [(torch.empty((B, N, H, d), dtype=torch.bfloat16, device=dev),
                 torch.empty((B, H, N), dtype=torch.float32, device=dev)) for _ in libs]
        tun = ea.tuning()

        def launch(i):
            st = libs[i].ea_attn_fwd_mx8_fmt(*[P(x) for x in t8], P(outs[i][0]), P(outs[i][1]), B, N, H, H, d, 1,
                                             m8.scale, 0, ctypes.byref(tun), stream.cuda_stream)
            if st != 0:
                raise RuntimeError(f"{args.libs[i]}: ea_attn_fwd_mx8_fmt returned {st}")
    elif args.what == "decode":
        pg = W.paged_decode_device(dev)
        q = bf16(pg.q)
        kc, vc = pg.k_cache, pg.v_cache
        bt = torch.from_numpy(pg.block_table).to(dev)
        sl = torch.from_numpy(pg.seq_lens).to(dev)
        B, Hq, d = q.shape
        P_, ps, Hkv, _ = kc.shape
        max_pages = bt.shape[1]
        wsb = int(libs[0].ea_decode_workspace_size(B, Hq, Hkv, d, max_pages * ps, ps, 0))
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        outs = [(torch.empty_like(q), torch.empty((B, Hq), dtype=torch.float32, device=dev)) for _ in libs]

        def launch(i):
            st = libs[i].ea_attn_decode_paged(P(q), P(kc), P(vc), P(bt), P(sl), P(outs[i][0]), P(outs[i][1]), B, Hq,
                                              Hkv, d, ps, P_, max_pages, pg.scale, 0, P(ws), ws.numel(),
                                              stream.cuda_stream)
            if st != 0:
                raise RuntimeError(f"{args.libs[i]}: ea_attn_decode_paged returned {st}")
    elif args.what == "bwd":
        inp = W.prefill(True)
        q, k, v = bf16(inp.q), bf16(inp.k), bf16(inp.v)
        B, N, H, d = q.shape
        o, lse = ea.attn_fwd(q, k, v, True, inp.scale)
        g = torch.randn(q.shape, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(dev)
        wsb = int(libs[0].ea_attn_bwd_workspace_size(B, H, N))
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        outs = [tuple(torch.empty_like(q) for _ in range(3)) for _ in libs]

        def launch(i):
            dq, dk, dv = outs[i]
            st = libs[i].ea_attn_bwd_ex(P(q), P(k), P(v), P(o), P(g), P(lse), P(dq), P(dk), P(dv), B, N, N, H, H,
                                        d, 1, inp.scale, 0, P(ws), wsb, stream.cuda_stream)
            if st != 0:
                raise RuntimeError(f"{args.libs[i]}: ea_attn_bwd_ex returned {st}")
    else:
        causal = args.what != "bf16nc"
        inp = W.dense(4, 8192, 8192, 16, 16, 64, True, seed=1002) if args.what == "bf16d64" else W.prefill(causal)
        q, k, v = bf16(inp.q), bf16(inp.k), bf16(inp.v)
        B, N, H, d = q.shape
        outs = [(torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device=dev)) for _ in libs]
        tun = ea.tuning()

        def launch(i):
            st = libs[i].ea_attn_fwd_hd(P(q), P(k), P(v), P(outs[i][0]), P(outs[i][1]), B, N, N, H, H, d, d,
                                        int(causal), inp.scale, ctypes.byref(tun), stream.cuda_stream)
            if st != 0:
                raise RuntimeError(f"{args.libs[i]}: ea_attn_fwd_hd returned {st}")

    torch.cuda.synchronize()
    for i in range(len(libs)):
        for _ in range(30):
            launch(i)
    torch.cuda.synchronize()
    res = [[] for _ in libs]
    for _ in range(args.rounds):
        for i in range(len(libs)):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            for _ in range(3):
                launch(i)
            e0.record(stream)
            for _ in range(args.launches):
                launch(i)
            e1.record(stream)
            torch.cuda.synchronize()
            res[i].append(e0.elapsed_time(e1) / args.launches)
    for path, r in zip(args.libs, res):
        ms = np.array(r)
        print(f"{path}: ms per launch median {np.median(ms):.4f} min {ms.min():.4f} max {ms.max():.4f}", flush=True)
    for i in range(1, len(libs)):
        same = all(torch.equal(a, b) for a, b in zip(outs[i], outs[0]))
        print(f"{args.libs[i]} outputs bitwise equal to {args.libs[0]}'s: {same}", flush=True)


if __name__ == "__main__":
    main()
