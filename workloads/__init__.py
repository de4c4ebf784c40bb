"""Seeded synthetic inputs for the exact-attention workloads.

This module is shared by the HIP path's tests/benchmark and by the CPU oracle's
tests. It holds only random draws, number encodings (bf16, OCP e4m3 with e8m0
block scales) and shape bookkeeping -- none of the attention arithmetic.

Recipe (stated once here, repeated in the design notes):
  * every tensor is drawn from numpy ``Generator(PCG64(SeedSequence([seed,
    stream, chunk])))`` in chunks of 2**22 float32 normals, chunks filled by a
    thread pool; ``stream`` numbers the tensor (0=Q, 1=K, 2=V, 3=K cache,
    4=V cache) and lengths / permutations use stream 9;
  * values are rounded once on the CPU to bf16 with round-to-nearest-even, or
    to OCP e4m3 (satfinite, RNE) under a power-of-two e8m0 scale per block of
    32 elements;
  * seed = 1000 + workload number (1..5) for the default workloads.

Workloads (sizes from the benchmark definitions):
  1 tiny   B=1  H=2   N=256   d=64   (causal and not)
  2 prefill B=4 H=16  N=8192  d=128  (causal and not)
  3 decode B=64 Hq=32 Hkv=8   d=128, context ~ U{512..32768}, page 16
  4 fp8    B=2  H=16  N=16384 d=128  causal, MX e4m3
  5 long   B=1  H=32  N=32768 d=128  causal, and 8 ragged sequences U{1024..32768}
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

CHUNK = 1 << 22
STREAM_Q, STREAM_K, STREAM_V, STREAM_KC, STREAM_VC, STREAM_META = 0, 1, 2, 3, 4, 9
STREAM_DO = 5   # output gradients for the backward


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------------------
# number encodings
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits (uint16) to float32 (exact)."""
    b = np.ascontiguousarray(bits).view(np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


E4M3_MAX = 448.0


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Encode finite values as OCP FP8 E4M3 (bias 7, no infinities), round to
    nearest even, saturating to +-448. Returns uint8 codes. Works in float32:
    every step (power-of-two scaling, rounding to an integer) is exact there."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x)
    sign = np.signbit(x).astype(np.uint8)
    # quantisation step: 2^(floor(log2 a) - 3) for normals, 2^-9 below 2^-6
    _, e = np.frexp(np.maximum(a, np.float32(2.0 ** -6)))   # a = f * 2^e, f in [0.5, 1)
    step = np.ldexp(np.float32(1.0), (e - 4).astype(np.int32))
    q = np.round(a / step) * step                             # ties to even
    q = np.minimum(q, np.float32(E4M3_MAX))
    _, e2 = np.frexp(np.maximum(q, np.float32(2.0 ** -6)))
    E = (e2 - 1).astype(np.int32)                             # floor(log2 q) for normals
    normal = q >= np.float32(2.0 ** -6)
    exp_field = np.where(normal, E + 7, 0).astype(np.uint8)
    mant = np.where(normal, (q / np.ldexp(np.float32(1.0), E) - np.float32(1.0)) * np.float32(8.0),
                    q / np.float32(2.0 ** -9))
    code = (sign << 7) | (exp_field << 3) | np.rint(mant).astype(np.uint8)
    return code.astype(np.uint8)


E5M2_MAX = 57344.0


def f32_to_e5m2_bits(x: np.ndarray) -> np.ndarray:
    """Encode finite values as OCP FP8 E5M2 (bias 15, 2 mantissa bits, largest
    finite 57344), round to nearest even, saturating to +-57344 (the MX
    quantiser never exceeds it). Returns uint8 codes; exact in float32."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x)
    sign = np.signbit(x).astype(np.uint8)
    # quantisation step: 2^(floor(log2 a) - 2) for normals, 2^-16 below 2^-14
    _, e = np.frexp(np.maximum(a, np.float32(2.0 ** -14)))
    step = np.ldexp(np.float32(1.0), (e - 3).astype(np.int32))
    q = np.round(a / step) * step
    q = np.minimum(q, np.float32(E5M2_MAX))
    _, e2 = np.frexp(np.maximum(q, np.float32(2.0 ** -14)))
    E = (e2 - 1).astype(np.int32)
    normal = q >= np.float32(2.0 ** -14)
    exp_field = np.where(normal, E + 15, 0).astype(np.uint8)
    mant = np.where(normal, (q / np.ldexp(np.float32(1.0), E) - np.float32(1.0)) * np.float32(4.0),
                    q / np.float32(2.0 ** -16))
    code = (sign << 7) | (exp_field << 2) | np.rint(mant).astype(np.uint8)
    return code.astype(np.uint8)


FP8_FORMATS = {"e4m3": (E4M3_MAX, f32_to_e4m3_bits), "e5m2": (E5M2_MAX, f32_to_e5m2_bits)}


def _mx_rows(blk: np.ndarray, fmt: str = "e4m3"):
    """MX quantisation of rows of 32-element blocks: blk [..., 32] float32."""
    fmax, encode = FP8_FORMATS[fmt]
    amax = np.abs(blk).max(axis=-1).astype(np.float64)
    ratio = amax / fmax
    f, e = np.frexp(np.where(ratio > 0, ratio, 1.0))      # ratio = f * 2^e, f in [0.5,1)
    E = np.where(f == 0.5, e - 1, e)                       # ceil(log2 ratio)
    E = np.where(amax > 0, E, -127)
    E = np.clip(E, -127, 127).astype(np.int32)
    scaled = blk * np.ldexp(np.float32(1.0), -E)[..., None].astype(np.float32)
    return encode(scaled), (E + 127).astype(np.uint8)


def mx_quantize_e4m3(x: np.ndarray, axis: int, block: int = 32, threads: int | None = None):
    """mx_quantize with e4m3 element codes."""
    return mx_quantize(x, axis, block, threads, fmt="e4m3")


def mx_quantize(x: np.ndarray, axis: int, block: int = 32, threads: int | None = None, fmt: str = "e4m3"):
    """Quantise float data to fp8 codes (``fmt`` "e4m3" or "e5m2") with one
    e8m0 scale per ``block`` consecutive elements along ``axis``.

    Scale rule (one of two readings of the block-scaling recipe; the other one,
    floor(log2 amax) - emax, can saturate the block maximum): E =
    ceil(log2(amax / fmax)) computed from the exponent and mantissa bits, with
    fmax the format's largest finite value (448 or 57344), clamped to
    [-127, 127]; an all-zero block gets E = -127. The stored scale byte is
    E + 127 and the element codes are fp8(x / 2^E).

    Returns (codes uint8 same shape as x, scales uint8 with ``axis`` shortened
    by ``block``)."""
    x = np.asarray(x, dtype=np.float32)
    axis = axis % x.ndim
    n = x.shape[axis]
    if n % block:
        raise ValueError("length along the scaled axis must be a multiple of the block")
    xs = np.ascontiguousarray(np.moveaxis(x, axis, -1))
    lead = xs.shape[:-1]
    blk = xs.reshape(-1, n // block, block)
    codes = np.empty(blk.shape, np.uint8)
    scales = np.empty(blk.shape[:2], np.uint8)
    rows = blk.shape[0]
    step = max(1, (1 << 20) // max(1, n))

    def run(lo):
        hi = min(rows, lo + step)
        c, s_ = _mx_rows(blk[lo:hi], fmt)
        codes[lo:hi] = c
        scales[lo:hi] = s_

    starts = list(range(0, rows, step))
    if len(starts) <= 1:
        for lo in starts:
            run(lo)
    else:
        with ThreadPoolExecutor(threads or _threads()) as ex:
            list(ex.map(run, starts))
    codes = np.moveaxis(codes.reshape(lead + (n,)), -1, axis)
    scales = np.moveaxis(scales.reshape(lead + (n // block,)), -1, axis)
    return np.ascontiguousarray(codes), np.ascontiguousarray(scales)


# ----------------------------------------------------------------------------
# random draws
# ----------------------------------------------------------------------------

def normal_f32(seed: int, stream: int, n: int, threads: int | None = None) -> np.ndarray:
    """n iid N(0,1) float32 draws, chunked and filled in parallel."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, c])))
        g.standard_normal(out=out[lo:hi], dtype=np.float32)

    if nchunks <= 1:
        if n:
            fill(0)
    else:
        with ThreadPoolExecutor(threads or _threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def normal_bf16_bits(seed: int, stream: int, shape, threads: int | None = None) -> np.ndarray:
    """iid N(0,1) draws rounded to bf16; returns uint16 bits of the given shape."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, c])))
        tmp = g.standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = f32_to_bf16_bits(tmp)

    if nchunks <= 1:
        if n:
            fill(0)
    else:
        with ThreadPoolExecutor(threads or _threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def meta_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, STREAM_META])))


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

@dataclass
class Dense:
    """Dense BSHD inputs: q [B,Nq,Hq,d], k/v [B,Nk,Hkv,d] as bf16 bits."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    causal: bool
    scale: float


def dense(B: int, Nq: int, Nk: int, Hq: int, Hkv: int, d: int, causal: bool,
          seed: int, scale: float | None = None, dv: int | None = None) -> Dense:
    """Dense BSHD bf16 inputs; v has head dim ``dv`` (default d)."""
    q = normal_bf16_bits(seed, STREAM_Q, (B, Nq, Hq, d))
    k = normal_bf16_bits(seed, STREAM_K, (B, Nk, Hkv, d))
    v = normal_bf16_bits(seed, STREAM_V, (B, Nk, Hkv, dv or d))
    return Dense(q, k, v, causal, float(scale if scale is not None else 1.0 / np.sqrt(d)))


def tiny(causal: bool) -> Dense:
    """Workload 1: B=1, H=2, N=256, d=64."""
    return dense(1, 256, 256, 2, 2, 64, causal, seed=1001)


def prefill(causal: bool = True) -> Dense:
    """Workload 2: B=4, H=16, N=8192, d=128."""
    return dense(4, 8192, 8192, 16, 16, 128, causal, seed=1002)


def long_context() -> Dense:
    """Workload 5(i): B=1, H=32, N=32768, d=128, causal."""
    return dense(1, 32768, 32768, 32, 32, 128, True, seed=1005)


@dataclass
class Varlen:
    """Packed THD inputs: q [Tq,Hq,d], k/v [Tk,Hkv,d] bf16 bits; cu_seqlens int32."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    cu_q: np.ndarray
    cu_k: np.ndarray
    causal: bool
    scale: float


def varlen(lengths_q, lengths_k, Hq: int, Hkv: int, d: int, causal: bool, seed: int,
           scale: float | None = None) -> Varlen:
    lq = np.asarray(lengths_q, dtype=np.int64)
    lk = np.asarray(lengths_k, dtype=np.int64)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = normal_bf16_bits(seed, STREAM_Q, (int(cu_q[-1]), Hq, d))
    k = normal_bf16_bits(seed, STREAM_K, (int(cu_k[-1]), Hkv, d))
    v = normal_bf16_bits(seed, STREAM_V, (int(cu_k[-1]), Hkv, d))
    return Varlen(q, k, v, cu_q, cu_k, causal, float(scale if scale is not None else 1.0 / np.sqrt(d)))


def ragged_lengths(n_seqs: int, lo: int, hi: int, seed: int) -> np.ndarray:
    return meta_rng(seed).integers(lo, hi + 1, size=n_seqs).astype(np.int64)


def long_ragged() -> Varlen:
    """Workload 5(ii): 8 sequences, lengths ~ U{1024..32768}, H=32, d=128, causal."""
    L = ragged_lengths(8, 1024, 32768, seed=1005)
    return varlen(L, L, 32, 32, 128, True, seed=1005)


@dataclass
class Paged:
    """Paged decode inputs.

    q [B,Hq,d] bf16 bits; k_cache/v_cache [num_pages,page,Hkv,d] bf16 bits with
    the unused tail slots of every sequence's last page set to NaN;
    block_table int32 [B, max_pages] (-1 where unused); seq_lens int32 [B]."""
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray
    page_size: int
    scale: float


BF16_NAN = np.uint16(0x7FC0)


def paged(B: int, Hq: int, Hkv: int, d: int, page_size: int, lengths, seed: int,
          max_pages: int | None = None, scale: float | None = None,
          permute: bool = True, poison: bool = True) -> Paged:
    L = np.asarray(lengths, dtype=np.int64)
    npages_seq = (L + page_size - 1) // page_size
    P = int(npages_seq.sum())
    if max_pages is None:
        max_pages = int(npages_seq.max()) if B else 0
    rng = meta_rng(seed)
    phys = rng.permutation(P).astype(np.int32) if permute else np.arange(P, dtype=np.int32)
    bt = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(npages_seq[b])
        bt[b, :n] = phys[off:off + n]
        off += n
    q = normal_bf16_bits(seed, STREAM_Q, (B, Hq, d))
    kc = normal_bf16_bits(seed, STREAM_KC, (P, page_size, Hkv, d))
    vc = normal_bf16_bits(seed, STREAM_VC, (P, page_size, Hkv, d))
    if poison:
        for b in range(B):
            n = int(npages_seq[b])
            used = int(L[b] - (n - 1) * page_size)
            if n and used < page_size:
                pg = bt[b, n - 1]
                kc[pg, used:] = BF16_NAN
                vc[pg, used:] = BF16_NAN
    return Paged(q, kc, vc, bt, L.astype(np.int32), page_size,
                 float(scale if scale is not None else 1.0 / np.sqrt(d)))


def decode_lengths(B: int, lo: int, hi: int, seed: int) -> np.ndarray:
    return meta_rng(seed).integers(lo, hi + 1, size=B).astype(np.int64)


def paged_decode() -> Paged:
    """Workload 3: B=64, Hq=32, Hkv=8, d=128, context ~ U{512..32768}, page 16,
    block table = seeded permutation of the page pool; max_pages = 2048.
    Host-generated (slow for the full pool: prefer paged_decode_device)."""
    L = decode_lengths(64, 512, 32768, seed=1003)
    return paged(64, 32, 8, 128, 16, L, seed=1003, max_pages=32768 // 16)


def split_pages(pg: Paged, page_size: int) -> Paged:
    """The same pool seen as pages of ``page_size`` tokens, a divisor of the
    pool's page size: page p of the pool becomes pages p*r .. p*r + r - 1
    (r = old / new size), so no data moves; the block table is rewritten."""
    old = pg.page_size
    assert old % page_size == 0, (old, page_size)
    r = old // page_size
    kc = pg.k_cache.reshape((pg.k_cache.shape[0] * r, page_size) + tuple(pg.k_cache.shape[2:]))
    vc = pg.v_cache.reshape((pg.v_cache.shape[0] * r, page_size) + tuple(pg.v_cache.shape[2:]))
    bt = np.asarray(pg.block_table)
    B, mp = bt.shape
    j = np.arange(mp * r)
    src = bt[:, j // r]
    # (fancy indexing may return a column-major array; the table must be row-major)
    nbt = np.ascontiguousarray(np.where(src >= 0, src * r + (j % r)[None, :], -1), dtype=np.int32)
    return Paged(pg.q, kc, vc, nbt, pg.seq_lens, page_size, pg.scale)


def normal_bf16_device(seed: int, stream: int, shape, device, chunk: int = 1 << 28):
    """iid N(0,1) draws rounded (RNE) to bf16 on a GPU: torch's seeded
    Philox generator on ``device``, drawn in chunks of ``chunk`` elements
    (chunk c seeded with (seed, stream, c)). Returns a torch bf16 tensor."""
    import torch
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=torch.bfloat16, device=device)
    for c, lo in enumerate(range(0, n, chunk)):
        hi = min(n, lo + chunk)
        g = torch.Generator(device=device)
        g.manual_seed((seed * 1_000_003 + stream * 10_007 + c) & 0x7FFFFFFFFFFFFFFF)
        out[lo:hi] = torch.randn(hi - lo, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    return out.view(*shape)


def paged_decode_device(device="cuda", seed: int = 1003) -> Paged:
    """Workload 3 with the KV pool drawn on the GPU (same lengths, block table,
    q and NaN-poisoned tails as the host recipe; cache values from
    ``normal_bf16_device``). k_cache / v_cache are torch bf16 tensors on
    ``device``; q, block_table and seq_lens stay numpy."""
    import torch
    B, Hq, Hkv, d, ps = 64, 32, 8, 128, 16
    L = decode_lengths(B, 512, 32768, seed=seed)
    npages_seq = (L + ps - 1) // ps
    P = int(npages_seq.sum())
    rng = meta_rng(seed)
    phys = rng.permutation(P).astype(np.int32)
    max_pages = 32768 // ps
    bt = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(npages_seq[b])
        bt[b, :n] = phys[off:off + n]
        off += n
    q = normal_bf16_bits(seed, STREAM_Q, (B, Hq, d))
    kc = normal_bf16_device(seed, STREAM_KC, (P, ps, Hkv, d), device)
    vc = normal_bf16_device(seed, STREAM_VC, (P, ps, Hkv, d), device)
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16, device=device)
    for b in range(B):
        n = int(npages_seq[b])
        used = int(L[b] - (n - 1) * ps)
        if used < ps:
            pg = int(bt[b, n - 1])
            kc[pg, used:] = nan
            vc[pg, used:] = nan
    return Paged(q, kc, vc, bt, L.astype(np.int32), ps, float(1.0 / np.sqrt(d)))


def host_subpool(pg: Paged, batches):
    """Copy the pages of the listed sequences of a device-resident pool to the
    host (bf16 bits) with a remapped block table, for oracle checks. Returns a
    host Paged holding only those sequences (in the given order)."""
    import torch
    ps = pg.page_size
    rows, tables, lens, qs = [], [], [], []
    off = 0
    mp = pg.block_table.shape[1]
    for b in batches:
        n = -(-int(pg.seq_lens[b]) // ps)
        idx = torch.from_numpy(pg.block_table[b, :n].astype(np.int64)).to(pg.k_cache.device)
        rows.append((pg.k_cache.index_select(0, idx), pg.v_cache.index_select(0, idx)))
        t = np.full(mp, -1, np.int32)
        t[:n] = np.arange(off, off + n)
        tables.append(t)
        lens.append(pg.seq_lens[b])
        qs.append(pg.q[b])
        off += n
    kc = torch.cat([r[0] for r in rows]).view(torch.int16).cpu().numpy().view(np.uint16)
    vc = torch.cat([r[1] for r in rows]).view(torch.int16).cpu().numpy().view(np.uint16)
    return Paged(np.stack(qs), kc, vc, np.stack(tables), np.array(lens, np.int32), ps, pg.scale)


@dataclass
class MX8:
    """MX fp8 inputs (OCP e4m3 codes + e8m0 scales).

    q8/k8/v8 [B,N,H,d] uint8; q_scale/k_scale [B,N,H,d/32] (blocks along d);
    v_scale [B,N/32,H,d] (blocks along the sequence). The library takes the
    Q and K scales head-major, [B,H,N,d/32]: ``q_scale_dev`` / ``k_scale_dev``
    (the same bytes, transposed)."""
    q8: np.ndarray
    k8: np.ndarray
    v8: np.ndarray
    q_scale: np.ndarray
    k_scale: np.ndarray
    v_scale: np.ndarray
    causal: bool
    scale: float
    fmt: str = "e4m3"    # element format of q8 / k8 / v8

    @property
    def q_scale_dev(self) -> np.ndarray:
        return np.ascontiguousarray(self.q_scale.transpose(0, 2, 1, 3))

    @property
    def k_scale_dev(self) -> np.ndarray:
        return np.ascontiguousarray(self.k_scale.transpose(0, 2, 1, 3))


def mx8(B: int, N: int, H: int, d: int, causal: bool, seed: int, scale: float | None = None,
        fmt: str = "e4m3") -> MX8:
    n = B * N * H * d
    q = normal_f32(seed, STREAM_Q, n).reshape(B, N, H, d)
    q8, qs = mx_quantize(q, axis=3, fmt=fmt)
    del q
    k = normal_f32(seed, STREAM_K, n).reshape(B, N, H, d)
    k8, ks = mx_quantize(k, axis=3, fmt=fmt)
    del k
    v = normal_f32(seed, STREAM_V, n).reshape(B, N, H, d)
    v8, vs = mx_quantize(v, axis=1, fmt=fmt)
    del v
    return MX8(q8, k8, v8, qs, ks, vs, causal, float(scale if scale is not None else 1.0 / np.sqrt(d)), fmt)


def fp8_prefill(fmt: str = "e4m3") -> MX8:
    """Workload 4: B=2, H=16, N=16384, d=128, causal, MX e4m3 (or e5m2)."""
    return mx8(2, 16384, 16, 128, True, seed=1004, fmt=fmt)
