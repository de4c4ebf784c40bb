"""Work-tile scheduling of the forward, written out plainly -- the oracle's
part for the varlen batch order (test infrastructure only; see package doc).

Citations name the page and its section:
  [P2 §3.3] "FlashAttention4 close reading", section 3.3 (scheduling): the
            cost of a causal row block grows with its index; longest tiles
            first; the worked example of 8 tasks on 4 processors; for varlen
            inputs a preprocessing step weighs each batch item by its
            heaviest work tile (not by its token count) and emits a
            virtual -> actual batch permutation instead of moving data.
  [P1 LPT]  "FlashAttention-4: algorithm-pipeline co-design for Blackwell",
            section on LPT scheduling (heaviest query blocks first for
            variable lengths and causal masks).

Everything here is integer bookkeeping; nothing is shared with the library.
"""
from __future__ import annotations


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def tile_kv_blocks(lq: int, lk: int, causal: bool, block_m: int, block_n: int, mb: int) -> int:
    """Key tiles the main loop of row block ``mb`` visits [P2 §3.3].

    Non-causal: all ceil(lk / block_n). Causal, aligned bottom-right (query i
    sees keys j <= i + lk - lq): keys up to the block's last row, clamped to
    [0, lk]. For lq = lk this is mb + 1 tiles when block_m = block_n, the
    triangle the page tabulates."""
    if not causal:
        return _ceil_div(lk, block_n)
    nkeys = min(lk, (mb + 1) * block_m + lk - lq)
    return _ceil_div(max(nkeys, 0), block_n)


def seq_weight(lq: int, lk: int, causal: bool, block_m: int, block_n: int) -> int:
    """Weight of one batch item: the longest main loop over its row blocks
    [P2 §3.3]; 0 for an item without queries."""
    n_mb = _ceil_div(lq, block_m)
    return max((tile_kv_blocks(lq, lk, causal, block_m, block_n, mb) for mb in range(n_mb)), default=0)


def lpt_order(cu_q, cu_k, causal: bool, block_m: int, block_n: int) -> list[int]:
    """virtual index -> actual batch index, heaviest item first [P2 §3.3].
    Items of equal weight keep their original order (a stable sort)."""
    n = len(cu_q) - 1
    w = [seq_weight(int(cu_q[b + 1] - cu_q[b]), int(cu_k[b + 1] - cu_k[b]), causal, block_m, block_n)
         for b in range(n)]
    return sorted(range(n), key=lambda b: (-w[b], b))


def hierarchical_tile_order(batches: int, heads: int, n_mblocks: int, section: int) -> list[tuple[int, int, int]]:
    """Dense work tiles (batch, head, mblock) in the cache-aware hierarchical
    LPT traversal [P2 §3.3]: batch outermost; within a batch the heads in
    sections of ``section`` consecutive heads; within a section the row blocks
    from the last (the longest causal main loop) down to the first; for each
    row block the section's heads in turn."""
    out = []
    for b in range(batches):
        for h0 in range(0, heads, section):
            for mb in reversed(range(n_mblocks)):
                for h in range(h0, min(h0 + section, heads)):
                    out.append((b, h, mb))
    return out


def list_schedule_makespan(durations, processors: int) -> int:
    """Greedy dispatch in the given order: each task goes to the processor
    that becomes free first [P2 §3.3]. Returns the finishing time of the last
    processor."""
    free = [0] * processors
    for d in durations:
        i = min(range(processors), key=lambda p: (free[p], p))
        free[i] += d
    return max(free)
