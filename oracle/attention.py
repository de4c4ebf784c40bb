"""Plain fp64 attention -- the oracle (test infrastructure only; see package doc).

Citations name the page and its section:
  [P4 §01]  "FlashAttention: not less compute, less data movement", section 01
            (the exact attention formula).
  [P4 §02]  same page, section 02 (online softmax recurrence, worked example).
  [P4 §03]  same page, section 03 (forward keeps O and the row log-sum-exp).
  [P4 §05]  same page, section 05 (SDPA conventions: causal flag, GQA needs Hq
            divisible by Hkv).
  [P3 paged] "Faster, more flexible FlashAttention-4 for LLM inference",
            section on PR 1999/2104 (KV cache pages of arbitrary size).
  [P3 split] same page, section on PR 1940 (split-KV with a combine step).
  [P5 §2.1] "Low-precision FlashAttention-4: end-to-end block-scaled attention
            for Blackwell", section 2.1 (MX block scales along the GEMM K dim:
            Q, K along d; V along the sequence).
  [P5 §2.2] same page, section 2.2 (the backward: the five GEMMs S = K Q^T,
            dP = V dO^T, dV = P^T dO, dK = dS^T Q, dQ = dS K, with P = softmax(S)
            and dS = dsoftmax(dP, P)).
  [P1 bwd]  "FlashAttention-4: algorithm-pipeline co-design for Blackwell",
            backward sections (five matrix products, the softmax recomputed from
            the saved statistics, a deterministic mode with a fixed reduction
            order).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

try:
    from threadpoolctl import threadpool_limits
except Exception:  # pragma: no cover
    threadpool_limits = None


def _pool_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


# ----------------------------------------------------------------------------
# decoding of the input encodings (the oracle's own, independent of the encoder)
# ----------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bits -> float64 (exact): the bf16 pattern is the top half of a float32."""
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 codes -> float64: sign, 4-bit exponent (bias 7), 3-bit
    mantissa; exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no inf."""
    c = np.asarray(codes).astype(np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def e5m2_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E5M2 codes -> float64: sign, 5-bit exponent (bias 15), 2-bit
    mantissa; exponent 0 is subnormal (m * 2^-16); exponent 31 is infinity
    (m = 0) or NaN."""
    c = np.asarray(codes).astype(np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    m = c & 0x3
    val = np.where(e == 0, m * 2.0 ** -16, (1.0 + m / 4.0) * np.ldexp(1.0, e - 15))
    val = np.where(e == 31, np.where(m == 0, np.inf, np.nan), val)
    return s * val


def e8m0_to_f64(scales: np.ndarray) -> np.ndarray:
    """E8M0 scale bytes -> 2^(byte - 127) (0xFF is NaN)."""
    s = np.asarray(scales).astype(np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))


def dequant_mx(codes: np.ndarray, scales: np.ndarray, axis: int, block: int = 32, fmt: str = "e4m3") -> np.ndarray:
    """Dequantise MX fp8 data (``fmt`` "e4m3" or "e5m2"): element value times
    the e8m0 scale of its block of ``block`` consecutive elements along
    ``axis`` [P5 §2.1]."""
    vals = {"e4m3": e4m3_to_f64, "e5m2": e5m2_to_f64}[fmt](codes)
    sc = np.repeat(e8m0_to_f64(scales), block, axis=axis)
    return vals * sc


# ----------------------------------------------------------------------------
# dense attention
# ----------------------------------------------------------------------------

def allowed_keys(i: int, Nq: int, Nk: int, causal: bool) -> int:
    """Number of keys query row i may attend to: all Nk, or for causal the keys
    j <= i + (Nk - Nq) (bottom-right alignment; equal to j <= i when Nq == Nk).
    The pages state causal masking only for Nq == Nk [P4 §05]; the alignment
    for Nq != Nk is a reading."""
    if not causal:
        return Nk
    return max(0, min(Nk, i + (Nk - Nq) + 1))


def _rows_block(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, r0: int, r1: int,
                Nq: int, causal: bool, scale: float):
    """Full-row two-pass softmax attention for query rows [r0, r1) of one head.

    qh [Nq,d], kh/vh [Nk,d] float64. Returns (o [r1-r0, d], lse [r1-r0])."""
    Nk = kh.shape[0]
    d = vh.shape[1]
    n_last = allowed_keys(r1 - 1, Nq, Nk, causal)      # widest row in the block
    o = np.zeros((r1 - r0, d))
    lse = np.full(r1 - r0, -np.inf)
    if n_last == 0:
        return o, lse
    s = scale * (qh[r0:r1] @ kh[:n_last].T)             # [rows, n_last]   [P4 §01]
    if causal:
        lim = np.array([allowed_keys(i, Nq, Nk, True) for i in range(r0, r1)])
        mask = np.arange(n_last)[None, :] >= lim[:, None]
        s[mask] = -np.inf
    else:
        lim = np.full(r1 - r0, n_last)
    m = s.max(axis=1)                                    # row max (pass 1)
    ok = lim > 0
    m_safe = np.where(ok, m, 0.0)
    p = np.exp(s - m_safe[:, None])                      # pass 2
    ell = p.sum(axis=1)
    o[ok] = (p[ok] @ vh[:n_last]) / ell[ok, None]
    lse[ok] = m_safe[ok] + np.log(ell[ok])               # natural log, scale included [P4 §03]
    return o, lse


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, scale: float,
              threads: int | None = None, row_block: int = 512):
    """Exact attention on dense BSHD float arrays [P4 §01].

    q [B,Nq,Hq,d], k/v [B,Nk,Hkv,d]; query head h reads KV head h // (Hq/Hkv)
    (consecutive grouping; the pages only require Hq divisible by Hkv [P4 §05]).
    Returns (o [B,Nq,Hq,d] float64, lse [B,Hq,Nq] float64). Rows with no allowed
    key get o = 0 and lse = -inf.

    Work is split over (batch, head, row block) on a thread pool (numpy's BLAS
    and exp release the GIL); BLAS itself is held to one thread per task."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    if Hq % Hkv:
        raise ValueError("Hq must be divisible by Hkv")
    g = Hq // Hkv
    o = np.zeros((B, Nq, Hq, v.shape[3]))
    lse = np.full((B, Hq, Nq), -np.inf)
    tasks = [(b, h, r0, min(Nq, r0 + row_block))
             for b in range(B) for h in range(Hq) for r0 in range(0, Nq, row_block)]
    heads = {}

    def head(b, h):
        key = (b, h)
        if key not in heads:
            heads[key] = (np.ascontiguousarray(q[b, :, h, :]),
                          np.ascontiguousarray(k[b, :, h // g, :]),
                          np.ascontiguousarray(v[b, :, h // g, :]))
        return heads[key]

    for b in range(B):
        for h in range(Hq):
            head(b, h)

    def run(t):
        b, h, r0, r1 = t
        qh, kh, vh = heads[(b, h)]
        ob, lb = _rows_block(qh, kh, vh, r0, r1, Nq, causal, scale)
        o[b, r0:r1, h, :] = ob
        lse[b, h, r0:r1] = lb

    n = threads or _pool_threads()
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            if n == 1:
                for t in tasks:
                    run(t)
            else:
                with ThreadPoolExecutor(n) as ex:
                    list(ex.map(run, tasks))
    else:  # pragma: no cover
        for t in tasks:
            run(t)
    return o, lse


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, b: int, h: int, rows,
                   causal: bool, scale: float):
    """Exact attention for selected query rows of one (batch, head); inputs as in
    ``attention`` (any float dtype). Returns (o [len(rows), d], lse [len(rows)])."""
    B, Nq, Hq, d = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    Nk = k.shape[1]
    rows = np.asarray(rows, dtype=np.int64)
    qh = np.asarray(q[b, rows, h, :], dtype=np.float64)
    o = np.zeros((len(rows), v.shape[3]))
    lse = np.full(len(rows), -np.inf)
    for t, i in enumerate(rows):
        n = allowed_keys(int(i), Nq, Nk, causal)
        if n == 0:
            continue
        kh = np.asarray(k[b, :n, h // g, :], dtype=np.float64)
        vh = np.asarray(v[b, :n, h // g, :], dtype=np.float64)
        s = scale * (kh @ qh[t])
        m = s.max()
        p = np.exp(s - m)
        ell = p.sum()
        o[t] = (p @ vh) / ell
        lse[t] = m + np.log(ell)
    return o, lse


def attention_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q, cu_k, causal: bool,
                     scale: float, threads: int | None = None):
    """Packed variable-length attention: sequence s owns query rows
    [cu_q[s], cu_q[s+1]) and key rows [cu_k[s], cu_k[s+1]); indices (and the
    causal mask) are local to each sequence. q [Tq,Hq,d], k/v [Tk,Hkv,d].
    Returns (o [Tq,Hq,d], lse [Hq,Tq])."""
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    Tq, Hq, d = q.shape
    o = np.zeros((Tq, Hq, v.shape[2]))
    lse = np.full((Hq, Tq), -np.inf)
    for s in range(len(cu_q) - 1):
        a, bq = int(cu_q[s]), int(cu_q[s + 1])
        c, e = int(cu_k[s]), int(cu_k[s + 1])
        if bq == a:
            continue
        os_, ls_ = attention(q[None, a:bq], k[None, c:e], v[None, c:e], causal, scale, threads)
        o[a:bq] = os_[0]
        lse[:, a:bq] = ls_[0]
    return o, lse


# ----------------------------------------------------------------------------
# paged decode
# ----------------------------------------------------------------------------

def gather_pages(cache: np.ndarray, block_table: np.ndarray, b: int, L: int) -> np.ndarray:
    """Logical KV rows 0..L-1 of sequence b: token t lives in physical page
    block_table[b, t // page] at slot t % page [P3 paged]. cache is
    [num_pages, page, Hkv, d]; returns [L, Hkv, d] with the cache's dtype (a
    pure gather, so bit-exact comparisons are meaningful)."""
    page = cache.shape[1]
    t = np.arange(L)
    pages = np.asarray(block_table)[b, t // page]
    return cache[pages, t % page]


def decode_paged_heads(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                       block_table: np.ndarray, seq_lens, scale: float, b: int, heads=None):
    """One decode query per head of sequence b attending to all of its
    seq_lens[b] cached tokens (no mask). Cache values may be bf16 bits
    (uint16) or floats. Returns (o [len(heads), d], lse [len(heads)])."""
    Hq = q.shape[1]
    Hkv = k_cache.shape[2]
    g = Hq // Hkv
    heads = range(Hq) if heads is None else heads
    L = int(np.asarray(seq_lens)[b])
    kb = gather_pages(k_cache, block_table, b, L)
    vb = gather_pages(v_cache, block_table, b, L)
    if kb.dtype == np.uint16:
        kb, vb = bf16_to_f64(kb), bf16_to_f64(vb)
    kb = np.asarray(kb, dtype=np.float64)
    vb = np.asarray(vb, dtype=np.float64)
    qb = q[b]
    if qb.dtype == np.uint16:
        qb = bf16_to_f64(qb)
    qb = np.asarray(qb, dtype=np.float64)
    heads = list(heads)
    o = np.zeros((len(heads), vb.shape[2]))
    lse = np.full(len(heads), -np.inf)
    if L == 0:
        return o, lse
    for t, h in enumerate(heads):
        s = scale * (kb[:, h // g, :] @ qb[h])           # [L]   [P4 §01]
        m = s.max()
        p = np.exp(s - m)
        ell = p.sum()
        o[t] = (p @ vb[:, h // g, :]) / ell
        lse[t] = m + np.log(ell)
    return o, lse


def decode_paged(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                 block_table: np.ndarray, seq_lens, scale: float, batches=None,
                 threads: int | None = None):
    """Paged decode for every (or the listed) sequence: q [B,Hq,d].
    Returns (o [nb,Hq,d], lse [nb,Hq]) in the order of ``batches``."""
    B = q.shape[0]
    batches = list(range(B) if batches is None else batches)
    res = [None] * len(batches)

    def run(i):
        res[i] = decode_paged_heads(q, k_cache, v_cache, block_table, seq_lens, scale, batches[i])

    n = threads or _pool_threads()
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            with ThreadPoolExecutor(n) as ex:
                list(ex.map(run, range(len(batches))))
    else:  # pragma: no cover
        for i in range(len(batches)):
            run(i)
    o = np.stack([r[0] for r in res]) if res else np.zeros((0, q.shape[1], q.shape[2]))
    lse = np.stack([r[1] for r in res]) if res else np.zeros((0, q.shape[1]))
    return o, lse


# ----------------------------------------------------------------------------
# the two algebraic facts the fast paths rest on (restated for the pins)
# ----------------------------------------------------------------------------

def online_softmax_row(score_blocks, value_blocks):
    """The streaming recurrence for one query row [P4 §02]: keep a running max
    m, a running sum l and an unnormalised accumulator a; for each arriving
    block of scores s_j with values v_j take m' = max(m, max s_j), rescale l and
    a by exp(m - m'), add sum exp(s_j - m') and sum exp(s_j - m') v_j; the
    output is a / l and the log-sum-exp is m + log l.

    Inputs are lists of 1-D score arrays and matching [n_j, d] (or [n_j])
    value arrays, float64. Returns (o, lse)."""
    m = -np.inf
    ell = 0.0
    acc = None
    for s, vv in zip(score_blocks, value_blocks):
        s = np.asarray(s, dtype=np.float64)
        vv = np.asarray(vv, dtype=np.float64)
        if s.size == 0:
            continue
        m_new = max(m, float(s.max()))
        alpha = 0.0 if m == -np.inf else np.exp(m - m_new)
        p = np.exp(s - m_new)
        contrib = np.tensordot(p, vv, axes=(0, 0))
        acc = contrib if acc is None else alpha * acc + contrib
        ell = alpha * ell + p.sum()
        m = m_new
    if acc is None:
        return None, -np.inf
    return acc / ell, m + np.log(ell)


def lse_combine(o_parts, lse_parts):
    """Merge partial results over disjoint key sets [P3 split]: with part s
    holding a normalised output o_s and log-sum-exp lse_s over its keys, the
    whole has lse = log sum_s exp(lse_s) and o = sum_s exp(lse_s - lse) o_s.
    Parts with lse = -inf (no keys) contribute nothing; a row whose parts are
    all empty gets o = 0, lse = -inf.

    o_parts [S, ..., d], lse_parts [S, ...]; float64."""
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o_parts = np.asarray(o_parts, dtype=np.float64)
    mx = np.max(lse_parts, axis=0)
    empty = np.isneginf(mx)
    mx_safe = np.where(empty, 0.0, mx)
    w = np.where(np.isneginf(lse_parts), 0.0, np.exp(lse_parts - mx_safe))
    tot = w.sum(axis=0)
    tot_safe = np.where(empty, 1.0, tot)
    lse = np.where(empty, -np.inf, mx_safe + np.log(tot_safe))
    o = ((w / tot_safe)[..., None] * o_parts).sum(axis=0)
    return o, lse


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------

def _bwd_rows_block(qh, kh, vh, doh, r0, r1, Nq, causal, scale):
    """Gradients of L = sum(dO * O) from query rows [r0, r1) of one head, by the
    definition [P5 §2.2]: with S = scale Q K^T (masked), P = softmax(S) per row,
    dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(P * dP)) (the softmax
    Jacobian applied to dP), dQ = scale dS K, dK = scale dS^T Q.
    Returns (dq [rows, d], dk [Nk, d], dv [Nk, dv]) -- dk / dv are this block's
    contributions."""
    Nk, d = kh.shape
    dv_dim = vh.shape[1]
    n_last = allowed_keys(r1 - 1, Nq, Nk, causal)
    dq = np.zeros((r1 - r0, d))
    dk = np.zeros((Nk, d))
    dvv = np.zeros((Nk, dv_dim))
    if n_last == 0:
        return dq, dk, dvv
    s = scale * (qh[r0:r1] @ kh[:n_last].T)
    lim = np.array([allowed_keys(i, Nq, Nk, causal) for i in range(r0, r1)])
    s[np.arange(n_last)[None, :] >= lim[:, None]] = -np.inf
    ok = lim > 0
    m = np.where(ok, s.max(axis=1), 0.0)
    p = np.exp(s - m[:, None])
    p[~ok] = 0.0
    ell = p.sum(axis=1)
    p[ok] /= ell[ok, None]                                   # P = softmax(S), rows with no key stay 0
    do_blk = doh[r0:r1]
    dvv[:n_last] = p.T @ do_blk                              # dV = P^T dO
    dp = do_blk @ vh[:n_last].T                              # dP = dO V^T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))     # dS = dsoftmax(dP, P)
    dq[:] = scale * (ds @ kh[:n_last])                       # dQ = scale dS K
    dk[:n_last] = scale * (ds.T @ qh[r0:r1])                 # dK = scale dS^T Q
    return dq, dk, dvv


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, causal: bool,
                       scale: float, threads: int | None = None, row_block: int = 512, heads=None):
    """Gradients of exact attention [P5 §2.2; P1 bwd] for dense BSHD inputs:
    q [B,Nq,Hq,d], k [B,Nk,Hkv,d], v [B,Nk,Hkv,dv], do [B,Nq,Hq,dv] (the
    gradient of the output). Returns (dq [B,Nq,Hq,d], dk [B,Nk,Hkv,d],
    dv [B,Nk,Hkv,dv]) in float64. GQA: the gradients of a KV head are summed
    over the query heads that read it. The softmax is recomputed from the
    inputs (no saved statistics), rows with no allowed key contribute nothing.
    ``heads`` restricts the work to a list of (b, hq) pairs (the other
    gradients are left at zero), for spot checks of large inputs."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    if Hq % Hkv:
        raise ValueError("Hq must be divisible by Hkv")
    g = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    pairs = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    tasks = [(b, h, r0, min(Nq, r0 + row_block)) for (b, h) in pairs for r0 in range(0, Nq, row_block)]
    res = [None] * len(tasks)

    def run(t):
        b, h, r0, r1 = tasks[t]
        res[t] = _bwd_rows_block(q[b, :, h, :], k[b, :, h // g, :], v[b, :, h // g, :], do[b, :, h, :],
                                 r0, r1, Nq, causal, scale)

    n = threads or _pool_threads()
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            if n == 1:
                for t in range(len(tasks)):
                    run(t)
            else:
                with ThreadPoolExecutor(n) as ex:
                    list(ex.map(run, range(len(tasks))))
    else:  # pragma: no cover
        for t in range(len(tasks)):
            run(t)
    # sums in a fixed order (task order), so the oracle is deterministic
    for t, (b, h, r0, r1) in enumerate(tasks):
        bq, bk, bv = res[t]
        dq[b, r0:r1, h, :] = bq
        dk[b, :, h // g, :] += bk
        dv[b, :, h // g, :] += bv
    return dq, dk, dv
