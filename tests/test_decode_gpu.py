"""GPU parity of the paged split-KV decode against the fp64 oracle.

Inputs follow the decode workload's recipe: seeded lengths, the block table a
seeded permutation of the page pool, unused slots of every last page set to
NaN (they must never leak). Checks: element-wise tolerance on o and lse,
bit-exact gathers (a permuted table gives the same bits as the identity table
over the re-laid pool), split-count changes stay within tolerance, and
determinism.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _helpers import assert_lse_close, assert_o_close, dev_bf16, f64, host_bits, log

pytestmark = pytest.mark.gpu


def run_decode(pg, num_splits=0, want_lse=True):
    import exact_attention_amd as ea
    q = dev_bf16(pg.q)
    if isinstance(pg.k_cache, torch.Tensor):
        kc, vc = pg.k_cache, pg.v_cache
    else:
        kc, vc = dev_bf16(pg.k_cache), dev_bf16(pg.v_cache)
    bt = torch.from_numpy(pg.block_table).cuda()
    sl = torch.from_numpy(pg.seq_lens).cuda()
    o, lse = ea.attn_decode_paged(q, kc, vc, bt, sl, pg.page_size, pg.scale, num_splits=num_splits,
                                  want_lse=want_lse)
    torch.cuda.synchronize()
    return f64(host_bits(o)), (lse.cpu().numpy().astype(np.float64) if lse is not None else None)


@pytest.mark.parametrize("group", [1, 4, 8, 16])
def test_small_paged_decode(group):
    L = [1, 16, 17, 40, 100, 513]
    Hkv = 2
    pg = W.paged(len(L), Hkv * group, Hkv, 128, 16, L, seed=200 + group)
    log(f"decode small group={group} lengths={L}")
    o, lse = run_decode(pg)
    ro, rl = oracle.decode_paged(pg.q, pg.k_cache, pg.v_cache, pg.block_table, pg.seq_lens, pg.scale)
    assert_o_close(o, ro)
    assert_lse_close(lse, rl)


@pytest.mark.parametrize("page_size", [32, 64])
def test_larger_pages(page_size):
    L = [3, 64, 65, 1000]
    pg = W.paged(len(L), 8, 2, 128, page_size, L, seed=210 + page_size)
    o, lse = run_decode(pg)
    ro, rl = oracle.decode_paged(pg.q, pg.k_cache, pg.v_cache, pg.block_table, pg.seq_lens, pg.scale)
    assert_o_close(o, ro)
    assert_lse_close(lse, rl)


@pytest.mark.parametrize("num_splits", [1, 3, 7, 1000])
def test_split_counts(num_splits):
    """num_splits = number of equal ranges of the batch's 32-token chunks; 1000
    ranges over 135 chunks leaves most ranges empty."""
    L = [700, 2048, 31, 1500]
    pg = W.paged(len(L), 8, 2, 128, 16, L, seed=220)
    o, lse = run_decode(pg, num_splits=num_splits)
    ro, rl = oracle.decode_paged(pg.q, pg.k_cache, pg.v_cache, pg.block_table, pg.seq_lens, pg.scale)
    assert_o_close(o, ro)
    assert_lse_close(lse, rl)


def test_many_sequences_and_head_groups():
    """150 sequences (the schedule scans lengths 64 at a time) and Hkv = 16
    (two workgroups of 8 KV heads per range)."""
    rng = np.random.default_rng(250)
    L = rng.integers(1, 300, size=150).tolist()
    pg = W.paged(len(L), 32, 16, 128, 16, L, seed=250)
    o, lse = run_decode(pg, num_splits=37)
    ro, rl = oracle.decode_paged(pg.q, pg.k_cache, pg.v_cache, pg.block_table, pg.seq_lens, pg.scale)
    assert_o_close(o, ro)
    assert_lse_close(lse, rl)


def test_lengths_clamped_to_capacity():
    """seq_lens beyond max_pages_per_seq * page_size attend to the whole table
    (full tables here, so no poisoned slot is in range)."""
    L = [112, 112, 112]
    pg = W.paged(len(L), 8, 2, 128, 16, L, seed=260)
    cap = pg.block_table.shape[1] * 16
    assert cap == 112 and (pg.block_table >= 0).all()
    big = W.Paged(pg.q, pg.k_cache, pg.v_cache, pg.block_table, np.array([cap + 5, 1 << 30, cap], np.int32), 16,
                  pg.scale)
    o1, l1 = run_decode(pg)
    o2, l2 = run_decode(big)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    ro, rl = oracle.decode_paged(pg.q, pg.k_cache, pg.v_cache, pg.block_table, pg.seq_lens, pg.scale)
    assert_o_close(o1, ro)
    assert_lse_close(l1, rl)


def test_empty_sequence():
    L = [0, 5, 0]
    pg = W.paged(3, 4, 1, 128, 16, [1, 5, 1], seed=230)
    pg.seq_lens[:] = np.array(L, np.int32)
    o, lse = run_decode(pg)
    assert np.all(o[0] == 0) and np.all(o[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))
    ro, rl = oracle.decode_paged(pg.q, pg.k_cache, pg.v_cache, pg.block_table, pg.seq_lens, pg.scale, batches=[1])
    assert_o_close(o[1:2], ro)
    assert_lse_close(lse[1:2], rl)


def test_gather_bit_exact_under_permutation():
    """Decoding through a random page table gives the same bits as decoding the
    same tokens laid out in order with the identity table."""
    L = [33, 200, 16, 1111]
    a = W.paged(len(L), 8, 2, 128, 16, L, seed=240, permute=True)
    # re-lay a's pool in logical order
    pages = []
    ident = np.full_like(a.block_table, -1)
    off = 0
    for s, n in enumerate(L):
        npg = -(-n // 16)
        pages.append(a.k_cache[a.block_table[s, :npg]])
        ident[s, :npg] = np.arange(off, off + npg)
        off += npg
    kc = np.concatenate(pages)
    vc = np.concatenate([a.v_cache[a.block_table[s, :-(-n // 16)]] for s, n in enumerate(L)])
    b = W.Paged(a.q, kc, vc, ident, a.seq_lens, 16, a.scale)
    o1, l1 = run_decode(a)
    o2, l2 = run_decode(b)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, l3 = run_decode(a)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


def test_decode_workload_sampled():
    pg = W.paged_decode_device("cuda")
    log(f"decode workload: B={pg.q.shape[0]} pages={pg.k_cache.shape[0]} "
        f"lengths min={pg.seq_lens.min()} max={pg.seq_lens.max()}")
    o, lse = run_decode(pg)
    L = pg.seq_lens
    pick = sorted(set([int(np.argmin(L)), int(np.argmax(L)), 0, 17, 63]))
    sub = W.host_subpool(pg, pick)
    ro, rl = oracle.decode_paged(sub.q, sub.k_cache, sub.v_cache, sub.block_table, sub.seq_lens, sub.scale)
    assert_o_close(o[pick], ro)
    assert_lse_close(lse[pick], rl)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
