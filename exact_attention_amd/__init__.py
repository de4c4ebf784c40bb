"""exact_attention_amd -- exact fused attention for AMD MI355X (gfx950).

A thin ctypes binding of ``libexactattn.so`` (built in-tree by
``exact_attention_amd.build``). Every step of the computation runs in the
library's HIP kernels; this module only checks tensor metadata, allocates
outputs with torch (device memory + streams) and passes raw pointers. There is
no CPU or PyTorch fallback: if the library is missing, calls raise.

Entry points mirror include/ea.h:
  attn_fwd(q, k, v, causal, scale) -> (o, lse)
  attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, causal, scale) -> (o, lse)
  attn_fwd_mx8(q8, k8, v8, q_scale, k_scale, v_scale, causal, scale) -> (o, lse)
  attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, page_size) -> (o, lse)
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libexactattn.so")

EA_EXP_HW, EA_EXP_POLY, EA_EXP_HYBRID = 0, 1, 2
EA_FWD_KERNEL_AUTO, EA_FWD_KERNEL_4WAVE, EA_FWD_KERNEL_PINGPONG, EA_FWD_KERNEL_PIPELINED = 0, 1, 2, 3
EA_FWD_KERNEL_PERSISTENT, EA_FWD_KERNEL_UNROLL_KV = 4, 5

_c_int, _c_float, _c_void_p, _c_size_t = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class FwdTuning(ctypes.Structure):
    _fields_ = [("exp_mode", _c_int), ("rescale_log2", _c_float), ("natural_order", _c_int), ("kernel", _c_int)]


class EAError(RuntimeError):
    pass


_SIGNATURES = {
    "ea_version": ([], _c_int),
    "ea_last_error": ([], ctypes.c_char_p),
    "ea_fwd_tuning_default": ([ctypes.POINTER(FwdTuning)], None),
    "ea_attn_fwd": ([_c_void_p] * 5 + [_c_int] * 7 + [_c_float, _c_void_p], _c_int),
    "ea_attn_fwd_tuned": ([_c_void_p] * 5 + [_c_int] * 7 + [_c_float, ctypes.POINTER(FwdTuning), _c_void_p], _c_int),
    "ea_attn_fwd_hd": ([_c_void_p] * 5 + [_c_int] * 8 + [_c_float, ctypes.POINTER(FwdTuning), _c_void_p], _c_int),
    "ea_attn_fwd_varlen": ([_c_void_p] * 7 + [_c_int] * 8 + [_c_float, ctypes.POINTER(FwdTuning), _c_void_p], _c_int),
    "ea_attn_fwd_varlen_ordered": ([_c_void_p] * 7 + [_c_int] * 8 + [_c_float, _c_void_p, ctypes.POINTER(FwdTuning),
                                                                    _c_void_p], _c_int),
    "ea_varlen_lpt_order": ([_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_void_p, _c_void_p], _c_int),
    "ea_attn_fwd_mx8": ([_c_void_p] * 8 + [_c_int] * 6 + [_c_float, _c_void_p], _c_int),
    "ea_attn_fwd_mx8_tuned": ([_c_void_p] * 8 + [_c_int] * 6 + [_c_float, ctypes.POINTER(FwdTuning), _c_void_p],
                              _c_int),
    "ea_attn_fwd_mx8_fmt": ([_c_void_p] * 8 + [_c_int] * 6 + [_c_float, _c_int, ctypes.POINTER(FwdTuning), _c_void_p],
                            _c_int),
    "ea_attn_bwd_workspace_size": ([_c_int] * 3, _c_size_t),
    "ea_attn_bwd": ([_c_void_p] * 9 + [_c_int] * 7 + [_c_float, _c_void_p, _c_size_t, _c_void_p], _c_int),
    "ea_attn_bwd_ex": ([_c_void_p] * 9 + [_c_int] * 7 + [_c_float, _c_int, _c_void_p, _c_size_t, _c_void_p], _c_int),
    "ea_decode_workspace_size": ([_c_int] * 7, _c_size_t),
    "ea_attn_decode_paged": ([_c_void_p] * 7 + [_c_int] * 7 + [_c_float, _c_int, _c_void_p, _c_size_t, _c_void_p], _c_int),
    "ea_decode_noalloc_max_bytes": ([], _c_size_t),
    "ea_attn_decode_paged_noalloc": ([_c_void_p] * 7 + [_c_int] * 7 + [_c_float, _c_int, _c_void_p], _c_int),
    "ea_test_exp2": ([_c_void_p, _c_void_p, _c_int, _c_int, _c_void_p], _c_int),
    "ea_test_mfma_loop": ([_c_void_p, _c_int, _c_int, _c_void_p], _c_int),
    "ea_test_mfma_loop_data_bytes": ([_c_int], _c_size_t),
    "ea_test_mfma_loop_data": ([_c_void_p, _c_size_t, _c_void_p, _c_int, _c_int, _c_int, _c_void_p], _c_int),
    "ea_test_stream_read": ([_c_void_p, _c_size_t, _c_void_p, _c_int, _c_void_p], _c_int),
    "ea_test_pair_probe": ([_c_void_p, _c_int, _c_int, _c_int, ctypes.c_longlong, _c_void_p], _c_int),
    "ea_test_fwd_rescale_stats_len": ([_c_int] * 3, _c_size_t),
    "ea_test_fwd_rescale_stats": ([_c_void_p] * 5 + [_c_int] * 6 + [_c_float, _c_float, _c_void_p, _c_size_t,
                                                                   _c_void_p], _c_int),
    "ea_test_wall_clock_khz": ([_c_int, _c_void_p], _c_int),
    "ea_test_fwd_tiles": ([_c_int] * 3, _c_size_t),
    "ea_test_fwd_phase_cycles_len": ([_c_int] * 3, _c_size_t),
    "ea_test_fwd_phase_cycles": ([_c_void_p] * 5 + [_c_int] * 6 + [_c_float, _c_void_p, _c_size_t, _c_void_p], _c_int),
    "ea_test_varlen_lds_order": ([_c_void_p, _c_void_p, _c_int, _c_int, _c_void_p, _c_void_p], _c_int),
    "ea_test_decode_gather": ([_c_void_p] * 5 + [_c_int] * 8 + [_c_void_p, _c_void_p, _c_size_t, _c_void_p,
                                                                _c_size_t, _c_void_p], _c_int),
    "ea_test_fwd_tile_order": ([_c_int] * 5 + [_c_void_p, _c_size_t, _c_void_p], _c_int),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libexactattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise EAError(f"{LIB_PATH} is missing; build it with exact_attention_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = lib().ea_last_error().decode(errors="replace")
        raise EAError(f"{what} failed with status {status}: {msg}")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name: str, dtype, dim: int):
    """Type, dtype, rank and layout of one tensor argument (device checked
    separately, after the shapes, by _on_gpu)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(t, name: str, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _on_gpu(*named) -> None:
    """Every tensor on the same GPU (the kernels dereference all pointers on
    the device of the first)."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def default_tuning() -> FwdTuning:
    t = FwdTuning()
    lib().ea_fwd_tuning_default(ctypes.byref(t))
    return t


def tuning(exp_mode: int = EA_EXP_HW, rescale_log2: float = 8.0, natural_order: int = 0,
           kernel: int = 0) -> FwdTuning:
    """Forward tuning; kernel: 0 auto, 1 the 4-wave kernel, 2 the 8-wave ping-pong kernel,
    3 the 8-wave software-pipelined kernel (MX fp8 only), 4 the ping-pong kernel in persistent
    form (the fp8 pipelined kernel in persistent form for attn_fwd_mx8), 5 that persistent form
    with the K/V pipeline running on across row blocks (unroll-KV; bf16 only)."""
    return FwdTuning(exp_mode, rescale_log2, natural_order, kernel)


def attn_fwd(q, k, v, causal: bool = False, scale: float | None = None, *, tuning: FwdTuning | None = None,
             out: torch.Tensor | None = None, lse: torch.Tensor | None = None, want_lse: bool = True):
    """Exact attention forward. q [B,Nq,Hq,d], k [B,Nk,Hkv,d], v [B,Nk,Hkv,dv]
    bf16 (BSHD); dv = d, or (d, dv) = (192, 128). Returns (o [B,Nq,Hq,dv]
    bf16, lse [B,Hq,Nq] fp32 natural log or None)."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    dv = v.shape[3]
    if tuple(v.shape[:3]) != tuple(k.shape[:3]) or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k must be [B, Nk, Hkv, d] matching q and v [B, Nk, Hkv, dv]")
    if out is not None:
        _need(out, "out", torch.bfloat16, 4)
        _shape(out, "out", (B, Nq, Hq, dv))
    if lse is not None:
        _need(lse, "lse", torch.float32, 3)
        _shape(lse, "lse", (B, Hq, Nq))
    _on_gpu(("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = out if out is not None else torch.empty((B, Nq, Hq, dv), dtype=q.dtype, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    st = lib().ea_attn_fwd_hd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Nq, Nk, Hq, Hkv, d, dv,
                              int(bool(causal)), float(scale),
                              ctypes.byref(tuning) if tuning is not None else None, _stream(q))
    _check(st, "ea_attn_fwd")
    return o, lse


def varlen_lpt_order(cu_seqlens_q, cu_seqlens_k, causal: bool, block_m: int = 256):
    """Heaviest-sequence-first order of a packed batch (ea_varlen_lpt_order).
    Returns (order, weights), int32 [S] on the GPU: order[v] = actual sequence."""
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    S = cu_seqlens_q.shape[0] - 1
    if cu_seqlens_k.shape[0] != S + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    _on_gpu(("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k))
    order = torch.empty(S, dtype=torch.int32, device=cu_seqlens_q.device)
    weights = torch.empty(S, dtype=torch.int32, device=cu_seqlens_q.device)
    st = lib().ea_varlen_lpt_order(_ptr(cu_seqlens_q), _ptr(cu_seqlens_k), S, int(bool(causal)), int(block_m),
                                   _ptr(weights), _ptr(order), _stream(cu_seqlens_q))
    _check(st, "ea_varlen_lpt_order")
    return order, weights


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, causal: bool = False,
                    scale: float | None = None, *, tuning: FwdTuning | None = None, want_lse: bool = True,
                    seq_order: torch.Tensor | None = None, input_order: bool = False):
    """Packed variable-length forward. q [Tq,Hq,d], k/v [Tk,Hkv,d] bf16 (THD);
    cu_seqlens int32 [S+1] on the GPU; seq_order (int32 [S] on the GPU, e.g.
    from varlen_lpt_order) sets the order the workgroups visit the sequences.
    Without one, the default kernels (d = 128) order up to 512 sequences
    heaviest first themselves when there are fewer (sequence, head) groups
    than CUs (ea_attn_fwd_varlen); input_order=True keeps the input order
    instead. The results do not depend on the order.
    Returns (o [Tq,Hq,d], lse [Hq,Tq])."""
    if seq_order is not None:
        _need(seq_order, "seq_order", torch.int32, 1)
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    Tq, Hq, d = q.shape
    Tk, Hkv, _ = k.shape
    if k.shape[2] != d:
        raise ValueError(f"k must be [Tk, Hkv, {d}] (q's head dim), got {tuple(k.shape)}")
    _shape(v, "v", k.shape)
    S = cu_seqlens_q.shape[0] - 1
    if S < 1:
        raise ValueError("cu_seqlens_q must hold at least two entries")
    if cu_seqlens_k.shape[0] != S + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if seq_order is not None and seq_order.shape[0] != S:
        raise ValueError("seq_order must have one entry per sequence")
    _on_gpu(("q", q), ("k", k), ("v", v), ("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k),
            ("seq_order", seq_order))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device) if want_lse else None
    tun = ctypes.byref(tuning) if tuning is not None else None
    if seq_order is None and not input_order:
        st = lib().ea_attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens_q),
                                      _ptr(cu_seqlens_k), S, Tq, Tk, int(max_seqlen_q), Hq, Hkv, d,
                                      int(bool(causal)), float(scale), tun, _stream(q))
    else:
        st = lib().ea_attn_fwd_varlen_ordered(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens_q),
                                              _ptr(cu_seqlens_k), S, Tq, Tk, int(max_seqlen_q), Hq, Hkv, d,
                                              int(bool(causal)), float(scale), _ptr(seq_order), tun, _stream(q))
    _check(st, "ea_attn_fwd_varlen")
    return o, lse


FP8_FORMATS = {"e4m3": 0, "e5m2": 1}


def attn_fwd_mx8(q8, k8, v8, q_scale, k_scale, v_scale, causal: bool = True, scale: float | None = None,
                 *, tuning: FwdTuning | None = None, want_lse: bool = True, fmt: str = "e4m3"):
    """MX fp8 forward. q8/k8/v8 [B,N,H,d] uint8 codes in ``fmt`` ("e4m3" or
    "e5m2"); q_scale/k_scale [B,H,N,d/32] (head-major) and v_scale [B,N/32,Hkv,d] uint8
    e8m0. Returns (o bf16, lse)."""
    if fmt not in FP8_FORMATS:
        raise ValueError(f"fmt must be one of {sorted(FP8_FORMATS)}")
    named = (("q8", q8), ("k8", k8), ("v8", v8), ("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale))
    for n, t in named:
        _need(t, n, torch.uint8, 4)
    B, N, Hq, d = q8.shape
    Hkv = k8.shape[2]
    _shape(k8, "k8", (B, N, Hkv, d))
    _shape(v8, "v8", (B, N, Hkv, d))
    if d % 32 or N % 32:
        raise ValueError(f"N ({N}) and d ({d}) must be multiples of 32 (the MX block)")
    _shape(q_scale, "q_scale", (B, Hq, N, d // 32))
    _shape(k_scale, "k_scale", (B, Hkv, N, d // 32))
    _shape(v_scale, "v_scale", (B, N // 32, Hkv, d))
    _on_gpu(*named)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty((B, N, Hq, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q8.device) if want_lse else None
    st = lib().ea_attn_fwd_mx8_fmt(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
                                   _ptr(o), _ptr(lse), B, N, Hq, Hkv, d, int(bool(causal)), float(scale),
                                   FP8_FORMATS[fmt], ctypes.byref(tuning) if tuning is not None else None,
                                   _stream(q8))
    _check(st, "ea_attn_fwd_mx8")
    return o, lse


def attn_bwd(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None, *,
             workspace: torch.Tensor | None = None, schedule: int = 0):
    """Backward of attn_fwd. q, o, dout [B,Nq,Hq,d], k, v [B,Nk,Hkv,d] bf16;
    lse [B,Hq,Nq] fp32 from the forward. schedule: 0 library default, 1 one
    workgroup per tile, 2 persistent. Returns (dq, dk, dv) bf16."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _need(t, n, torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    if tuple(v.shape) != tuple(k.shape) or tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("shapes: q, o, dout [B,Nq,Hq,d]; k, v [B,Nk,Hkv,d]")
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"k must be [{B}, Nk, Hkv, {d}] to match q, got {tuple(k.shape)}")
    if tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("lse must be [B, Hq, Nq]")
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1)
    _on_gpu(("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("lse", lse), ("workspace", workspace))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = int(lib().ea_attn_bwd_workspace_size(B, Hq, Nq))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = lib().ea_attn_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                              _ptr(dv), B, Nq, Nk, Hq, Hkv, d, int(bool(causal)), float(scale), int(schedule),
                              _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q))
    _check(st, "ea_attn_bwd")
    return dq, dk, dv


def decode_workspace_size(B: int, Hq: int, Hkv: int, d: int, max_seqlen: int, page_size: int,
                          num_splits: int = 0) -> int:
    return int(lib().ea_decode_workspace_size(B, Hq, Hkv, d, max_seqlen, page_size, num_splits))


def attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, page_size: int | None = None,
                      scale: float | None = None, *, num_splits: int = 0, workspace: torch.Tensor | None = None,
                      want_lse: bool = True):
    """Paged split-KV decode. q [B,Hq,d] bf16; k/v_cache [P,page,Hkv,d] bf16;
    block_table int32 [B,max_pages]; seq_lens int32 [B]. Returns (o [B,Hq,d], lse [B,Hq])."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    B, Hq, d = q.shape
    P, ps, Hkv, dk = k_cache.shape
    _shape(v_cache, "v_cache", k_cache.shape)
    if dk != d:
        raise ValueError(f"k_cache head dim {dk} differs from q's {d}")
    if block_table.shape[0] != B:
        raise ValueError(f"block_table must have {B} rows (one per sequence), got {block_table.shape[0]}")
    _shape(seq_lens, "seq_lens", (B,))
    if page_size is not None and page_size != ps:
        raise ValueError("page_size does not match k_cache.shape[1]")
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1)
    _on_gpu(("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("block_table", block_table),
            ("seq_lens", seq_lens), ("workspace", workspace))
    max_pages = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = decode_workspace_size(B, Hq, Hkv, d, max_pages * ps, ps, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if want_lse else None
    st = lib().ea_attn_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                    _ptr(o), _ptr(lse), B, Hq, Hkv, d, ps, P, max_pages, float(scale),
                                    int(num_splits), _ptr(workspace), workspace.numel(), _stream(q))
    _check(st, "ea_attn_decode_paged")
    return o, lse


def test_decode_gather(q, k_cache, v_cache, block_table, seq_lens, *, num_splits: int = 0, fill: int = 0x7FC1):
    """Test-only page-gather dump of the paged decode: the K and V rows its
    split kernel gathers, by (sequence, token, KV head), as dense bf16
    [B, max_pages * page, Hkv, d] tensors; rows it does not write keep the
    16-bit pattern ``fill``. Arguments as for attn_decode_paged."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _shape(v_cache, "v_cache", k_cache.shape)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    B, Hq, d = q.shape
    P, ps, Hkv, _ = k_cache.shape
    max_pages = block_table.shape[1]
    shape = (B, max_pages * ps, Hkv, d)
    dk = torch.full(shape, fill, dtype=torch.int16, device=q.device)
    dv = torch.full(shape, fill, dtype=torch.int16, device=q.device)
    need = decode_workspace_size(B, Hq, Hkv, d, max_pages * ps, ps, num_splits)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib().ea_test_decode_gather(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                     B, Hq, Hkv, d, ps, P, max_pages, int(num_splits), _ptr(dk), _ptr(dv),
                                     dk.numel(), _ptr(ws), ws.numel(), _stream(q))
    _check(st, "ea_test_decode_gather")
    return dk, dv


def test_fwd_rescale_stats(q, k, v, causal: bool, scale: float | None = None, rescale_log2: float = 8.0):
    """Test-only: the default dense forward (d = 128) plus its per-wave
    lazy-rescale and clock statistics. Returns (o, lse, stats int32
    [tiles, 8, 4]: steps with live keys, steps that rescaled, shader clock
    cycles of the step loop, wall clock ticks of the same loop)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, 4)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    if d != 128 or tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("q [B,Nq,Hq,128], k/v [B,Nk,Hkv,128]")
    _on_gpu(("q", q), ("k", k), ("v", v))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    n = int(lib().ea_test_fwd_rescale_stats_len(B, Nq, Hq))
    stats = torch.zeros(n, dtype=torch.int32, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    st = lib().ea_test_fwd_rescale_stats(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Nq, Nk, Hq, Hkv,
                                         int(bool(causal)), float(scale), float(rescale_log2), _ptr(stats), n,
                                         _stream(q))
    _check(st, "ea_test_fwd_rescale_stats")
    return o, lse, stats.view(-1, 8, 4)


def test_fwd_phase_cycles(q, k, v, causal: bool, scale: float | None = None):
    """Test-only: the default dense forward (d = 128) with shader-clock stamps
    at its phase edges. Returns (o, lse, cycles uint64 as int64 [workgroups, 8,
    8]: per wave the summed cycles of the MFMA parts, the barrier waits after
    them, the VALU parts, the barrier waits after those, the tile prologues and
    epilogues, then the steps and the tiles)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, 4)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    if d != 128 or tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("q [B,Nq,Hq,128], k/v [B,Nk,Hkv,128]")
    _on_gpu(("q", q), ("k", k), ("v", v))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    n = int(lib().ea_test_fwd_phase_cycles_len(B, Nq, Hq))
    if n == 0:
        raise EAError("ea_test_fwd_phase_cycles_len: no CU count")
    cyc = torch.zeros(n, dtype=torch.int64, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    st = lib().ea_test_fwd_phase_cycles(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Nq, Nk, Hq, Hkv,
                                        int(bool(causal)), float(scale), _ptr(cyc), n, _stream(q))
    _check(st, "ea_test_fwd_phase_cycles")
    return o, lse, cyc.view(-1, 8, 8)


def test_fwd_tile_order(B: int, Nq: int, Nk: int, Hq: int, causal: bool, device="cuda"):
    """Test-only: (batch, head, 256-row block) of every work tile of the dense
    forward in dispatch order, as computed on the device; -1 rows are padding.
    Returns an int32 tensor [tiles, 3] on the host."""
    n = int(lib().ea_test_fwd_tiles(B, Nq, Hq))
    out = torch.full((3 * n,), -2, dtype=torch.int32, device=device)
    st = lib().ea_test_fwd_tile_order(B, Nq, Nk, Hq, int(bool(causal)), _ptr(out), 3 * n,
                                      _stream(out))
    _check(st, "ea_test_fwd_tile_order")
    return out.view(n, 3).cpu()


def test_wall_clock_khz(device: int = 0) -> int:
    """Test-only: the rate of the device's constant wall clock counter (kHz)."""
    out = _c_int(0)
    _check(lib().ea_test_wall_clock_khz(int(device), ctypes.byref(out)), "ea_test_wall_clock_khz")
    return int(out.value)


def test_exp2(x: torch.Tensor, mode: int) -> torch.Tensor:
    """Test-only: 2^x with the kernels' exponential (EA_EXP_HW or EA_EXP_POLY)."""
    _need(x, "x", torch.float32, 1)
    _on_gpu(("x", x))
    y = torch.empty_like(x)
    _check(lib().ea_test_exp2(_ptr(x), _ptr(y), x.numel(), int(mode), _stream(x)), "ea_test_exp2")
    return y
