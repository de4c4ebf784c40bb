"""Device calibration: what one MI355X sustains on the operations the kernels
are built from, measured by the library's own test-only kernels.

    python -m exact_attention_amd.calibrate [--budget CYCLES] [--json PATH]

Prints one JSON object:
  pair_probe  for each pair of roles (waves 0-3 / waves 4-7 of a workgroup,
              one workgroup per CU, so each SIMD holds one wave of each role):
              shader-clock cycles per iteration of each role, median over the
              256 x 4 waves of that role (ea_test_pair_probe).
  clock_ghz   the shader clock during the probe, from s_memtime cycles over
              the launch's HIP-event time.
Roles, per iteration: mfma_reg (32 bf16 32x32x16 MFMAs from registers, 1024
cycles at the nominal rate), mfma_lds (the forward's product part: the same 32
MFMAs fed from LDS), softmax (the forward's softmax of one 64-key step on 32
scores per lane), exp / fma (32 independent instructions), mfma_agpr
(mfma_reg with AGPR accumulators), mfma_lds_prio (mfma_lds at raised wave
priority), mix (8 MFMAs from registers, each with 2 exp and 2 fma interleaved:
256 matrix cycles at the nominal rate), lds_b128 / lds_tr (an 8 KB operand
tile read from LDS into registers, plain or transposed, then waited for),
mfma_lds_deep (mfma_lds with 14 reads issued ahead instead of 6), mfma_lds_alt
(mfma_lds with the two products' MFMAs alternating), fused32 (a 32-key step:
16 LDS-fed MFMAs interleaved with the softmax of an independent 32-key tile,
512 matrix cycles at the nominal rate).
"""
from __future__ import annotations

import argparse
import ctypes
import json

import numpy as np

ROLES = {"idle": 0, "mfma_reg": 1, "mfma_lds": 2, "softmax": 3, "exp": 4, "fma": 5, "mfma_agpr": 6,
         "mfma_lds_prio": 7, "mix": 8, "lds_b128": 9, "lds_tr": 10, "mfma_lds_deep": 11, "mfma_lds_alt": 12,
         "fused32": 13}

PAIRS = [
    ("mfma_reg", "idle"), ("mfma_lds", "idle"), ("idle", "softmax"), ("idle", "exp"), ("idle", "fma"),
    ("mfma_reg", "softmax"), ("mfma_lds", "softmax"), ("mfma_lds_prio", "softmax"), ("mfma_reg", "exp"),
    ("mfma_reg", "fma"), ("mfma_agpr", "idle"), ("mfma_agpr", "softmax"), ("mfma_agpr", "fma"),
    ("mfma_reg", "mfma_reg"), ("softmax", "softmax"), ("mfma_lds", "mfma_lds"), ("exp", "exp"),
    ("fma", "fma"), ("fma", "idle"), ("exp", "idle"), ("softmax", "idle"), ("mix", "idle"), ("idle", "mix"),
    ("mix", "lds_tr"), ("mix", "lds_b128"), ("mix", "mix"), ("lds_tr", "idle"), ("lds_b128", "idle"),
    ("mfma_reg", "lds_tr"), ("lds_tr", "lds_tr"), ("mix", "softmax"),
    ("mfma_lds_deep", "idle"), ("mfma_lds_alt", "idle"), ("mfma_lds_deep", "softmax"), ("mfma_lds_alt", "softmax"),
    ("fused32", "idle"), ("fused32", "fused32"),
]


def pair_probe(torch, ea, role_a: str, role_b: str, budget: int, blocks: int = 256):
    dev = torch.device("cuda")
    lib = ea.lib()
    out = torch.zeros(16 * blocks, dtype=torch.int64, device=dev)
    s = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    st = lib.ea_test_pair_probe(ctypes.c_void_p(out.data_ptr()), blocks, ROLES[role_a], ROLES[role_b],
                                ctypes.c_longlong(budget), ctypes.c_void_p(s.cuda_stream))
    e1.record(s)
    torch.cuda.synchronize()
    if st != 0:
        raise RuntimeError(f"ea_test_pair_probe failed ({st})")
    r = out.cpu().numpy().reshape(blocks, 8, 2)
    res = {}
    for name, waves in ((role_a, slice(0, 4)), (role_b, slice(4, 8))):
        it, cy = r[:, waves, 0].ravel(), r[:, waves, 1].ravel()
        if name == "idle":
            continue
        key = name if name not in res else name + "_b"
        res[key] = float(np.median(cy / np.maximum(it, 1)))
    ms = e0.elapsed_time(e1)
    res["clock_ghz"] = float(np.median(r[:, :, 1][r[:, :, 0] > 0])) / (ms * 1e-3) / 1e9
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--budget", type=int, default=2_000_000, help="shader-clock cycles per probe")
    ap.add_argument("--json", default=None, help="also write the result to this file")
    args = ap.parse_args(argv)
    import torch

    import exact_attention_amd as ea
    lib = ea.lib()
    lib.ea_test_pair_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_longlong, ctypes.c_void_p]
    lib.ea_test_pair_probe.restype = ctypes.c_int
    pair_probe(torch, ea, "mfma_reg", "softmax", args.budget // 4)  # warm-up
    table = {}
    for a, b in PAIRS:
        table[f"{a}+{b}"] = pair_probe(torch, ea, a, b, args.budget)
        print(f"{a:>14} + {b:<10} {json.dumps(table[f'{a}+{b}'])}", flush=True)
    res = {"pair_probe": table, "budget_cycles": args.budget,
           "device": torch.cuda.get_device_properties(0).name}
    print(json.dumps(res), flush=True)
    if args.json:
        with open(args.json, "w") as f:
            json.dump(res, f, indent=1)


if __name__ == "__main__":
    main()
