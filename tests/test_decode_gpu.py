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


@pytest.mark.parametrize("group", [1, 3, 4, 5, 6, 7, 8, 12, 16, 20, 32, 64])
def test_small_paged_decode(group):
    """Any number of query heads per KV head: up to 16 share one column block
    (unused columns padded), more take several blocks of 16."""
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


@pytest.mark.parametrize("page_size", [16, 1, 4])
def test_decode_workload_sampled(page_size):
    """The decode workload (B=64, Hq=32, Hkv=8, contexts U{512..32768}); page
    sizes 1 and 4 view the same pool as smaller pages (per-token path)."""
    pg = W.paged_decode_device("cuda")
    if page_size != 16:
        pg = W.split_pages(pg, page_size)
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


@pytest.mark.parametrize("page_size", [1, 2, 3, 5, 8, 12, 24, 40])
def test_any_page_size(page_size):
    """Page sizes 16 does not divide (down to one token per page) take the
    per-token load path; lengths end inside, at and past page boundaries."""
    L = [1, 2, 31, 32, 33, 97, 640, 1001]
    pg = W.paged(len(L), 8, 2, 128, page_size, L, seed=300 + page_size)
    log(f"decode page_size={page_size} lengths={L}")
    o, lse = run_decode(pg)
    ro, rl = oracle.decode_paged(pg.q, pg.k_cache, pg.v_cache, pg.block_table, pg.seq_lens, pg.scale)
    assert_o_close(o, ro)
    assert_lse_close(lse, rl)


def relayout(pg, page_size, seed):
    """The same logical tokens as pg in a pool of another page size: pages in a
    seeded random order, the unused slots of every last page NaN-poisoned."""
    B = pg.q.shape[0]
    L = pg.seq_lens.astype(np.int64)
    tail = pg.k_cache.shape[2:]
    ks, vs = [], []
    for b in range(B):
        n = int(L[b])
        t = np.arange(n)
        pages = pg.block_table[b, t // pg.page_size]
        ks.append(pg.k_cache[pages, t % pg.page_size])
        vs.append(pg.v_cache[pages, t % pg.page_size])
    npg = (L + page_size - 1) // page_size
    P = int(npg.sum())
    phys = np.random.default_rng(seed).permutation(P).astype(np.int32)
    kc = np.full((P, page_size) + tail, W.BF16_NAN, dtype=np.uint16)
    vc = np.full((P, page_size) + tail, W.BF16_NAN, dtype=np.uint16)
    bt = np.full((B, int(npg.max())), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        for j in range(int(npg[b])):
            lo, hi = j * page_size, min(int(L[b]), (j + 1) * page_size)
            kc[phys[off], :hi - lo] = ks[b][lo:hi]
            vc[phys[off], :hi - lo] = vs[b][lo:hi]
            bt[b, j] = phys[off]
            off += 1
    return W.Paged(pg.q, kc, vc, bt, pg.seq_lens.copy(), page_size, pg.scale)


def test_page_size_invariance_bitwise():
    """The arithmetic follows the logical token order only: the same tokens
    laid out in pages of 16, 1, 5, 24 or 64 (each pool in its own random page
    order) decode to the same bits, through both load paths."""
    L = [5, 48, 129, 700, 1500, 3]
    base = W.paged(len(L), 12, 2, 128, 16, L, seed=320)
    o0, l0 = run_decode(base)
    for ps in (1, 5, 24, 64):
        o1, l1 = run_decode(relayout(base, ps, seed=321 + ps))
        log(f"page size {ps} vs 16: max |do| = {np.nanmax(np.abs(o1 - o0)):.3g}")
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1), ps
    ro, rl = oracle.decode_paged(base.q, base.k_cache, base.v_cache, base.block_table, base.seq_lens, base.scale)
    assert_o_close(o0, ro)
    assert_lse_close(l0, rl)


def test_small_pages_many_sequences_odd_group():
    """One-token pages, 6 query heads per KV head, 130 sequences, several
    range counts (ranges cut sequences at arbitrary chunks)."""
    rng = np.random.default_rng(330)
    L = rng.integers(0, 400, size=130).tolist()
    pg = W.paged(len(L), 24, 4, 128, 1, L, seed=330)
    ro, rl = oracle.decode_paged(pg.q, pg.k_cache, pg.v_cache, pg.block_table, pg.seq_lens, pg.scale)
    nz = np.asarray(L) > 0
    for ns in (0, 7, 300):
        o, lse = run_decode(pg, num_splits=ns)
        assert_o_close(o[nz], ro[nz])
        assert_lse_close(lse[nz], rl[nz])
        assert np.all(o[~nz] == 0) and np.all(np.isneginf(lse[~nz]))


def _one_hot_keys(pg, targets):
    """Queries that are unit vectors (query head h of every sequence points
    along axis h) and keys that are zero except key targets[b, h] of
    sequence b, which is 2^14 times that axis: every query then has one
    dominant key whose score beats all others by 2^14 scale, so its softmax
    weight is exactly 1 and every other weight underflows to exactly 0, and
    the output row is that key's V row bit for bit (a gather through the page
    table, made visible). Returns a new Paged with k_cache / q rewritten."""
    B, Hq, d = pg.q.shape
    Hkv = pg.k_cache.shape[2]
    g = Hq // Hkv
    one = W.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    big = W.f32_to_bf16_bits(np.full(1, 2.0 ** 14, np.float32))[0]
    q = np.zeros_like(pg.q)
    kc = np.where(pg.k_cache == W.BF16_NAN, W.BF16_NAN, np.uint16(0)).astype(np.uint16)
    for b in range(B):
        for h in range(Hq):
            q[b, h, h] = one
            t = int(targets[b, h])
            page = pg.block_table[b, t // pg.page_size]
            kc[page, t % pg.page_size, h // g, h] = big
    return W.Paged(q, kc, pg.v_cache, pg.block_table, pg.seq_lens, pg.page_size, pg.scale)


@pytest.mark.parametrize("page_size", [16, 1, 5])
def test_gather_exact_dominant_key(page_size):
    """Bit-exact page-table gathers, checked directly: for each (sequence,
    query head) the output equals, bit for bit, the V row of the token the
    host picks through the block table (random tokens, pages in a seeded
    random order, NaN-poisoned tails, several range counts)."""
    rng = np.random.default_rng(700 + page_size)
    L = [1, 17, 300, 1024, 33, 4000, 2, 129]
    Hq, Hkv = 32, 8
    pg = W.paged(len(L), Hq, Hkv, 128, page_size, L, seed=700 + page_size)
    for trial in range(3):
        targets = np.stack([rng.integers(0, n, size=Hq) for n in L])
        if trial == 0:
            targets[:, 0] = 0
            targets[:, 1] = np.asarray(L) - 1        # first and last token of every sequence
        pq = _one_hot_keys(pg, targets)
        for ns in (0, 3):
            o, _ = run_decode(pq, num_splits=ns)
            got = W.f32_to_bf16_bits(o.astype(np.float32))
            g = Hq // Hkv
            want = np.stack([np.stack([pg.v_cache[pg.block_table[b, targets[b, h] // page_size],
                                                  targets[b, h] % page_size, h // g]
                                       for h in range(Hq)]) for b in range(len(L))])
            assert np.array_equal(got, want), f"page {page_size} trial {trial} splits {ns}"
    log(f"  page {page_size}: {3 * 2 * len(L) * Hq} gathered rows bit-exact")


def _host_gather(pg):
    """Host indexing of the paged pool: token t of sequence b is slot t % page
    of page block_table[b, t // page] ("Faster, more flexible FlashAttention-4
    for LLM inference", PR 1999/2104 sections); a page index outside the pool
    reads as zeros. Returns, per sequence, its rows [L_b, Hkv, d] as bf16 bits
    for K and V."""
    P, ps = pg.k_cache.shape[:2]
    out = []
    for b in range(pg.block_table.shape[0]):
        L = int(min(max(int(pg.seq_lens[b]), 0), pg.block_table.shape[1] * ps))
        ks, vs = [], []
        for t in range(L):
            page = int(pg.block_table[b, t // ps])
            if 0 <= page < P:
                ks.append(pg.k_cache[page, t % ps])
                vs.append(pg.v_cache[page, t % ps])
            else:
                ks.append(np.zeros_like(pg.k_cache[0, 0]))
                vs.append(np.zeros_like(pg.v_cache[0, 0]))
        shape = (0,) + pg.k_cache.shape[2:]
        out.append((np.array(ks).reshape(-1, *shape[1:]) if ks else np.zeros(shape, np.uint16),
                    np.array(vs).reshape(-1, *shape[1:]) if vs else np.zeros(shape, np.uint16)))
    return out


@pytest.mark.parametrize("page_size", [16, 32, 5, 1])
@pytest.mark.parametrize("num_splits", [0, 3])
def test_page_gather_dump(page_size, num_splits):
    """The page-gather dump: the K and V rows the decode's split kernel stages
    for every chunk, through its own loads, equal host indexing of the pool
    through the block table bit for bit -- permuted table, ragged and empty
    sequences, NaN-poisoned tails, table entries outside the pool (rows of
    zeros) -- and nothing is written past a sequence's length."""
    import exact_attention_amd as ea
    L = [1, 15, 16, 17, 100, 333, 0, 64]
    pg = W.paged(len(L), 8, 2, 128, page_size, L, seed=270 + page_size, permute=True)
    P = pg.k_cache.shape[0]
    pg.block_table[5, 1] = P + 7     # past the pool
    pg.block_table[4, 0] = -3        # negative
    log(f"gather dump page {page_size} splits {num_splits}")
    fill = 0x7FC1
    dk, dv = ea.test_decode_gather(dev_bf16(pg.q), dev_bf16(pg.k_cache), dev_bf16(pg.v_cache),
                                   torch.from_numpy(pg.block_table).cuda(), torch.from_numpy(pg.seq_lens).cuda(),
                                   num_splits=num_splits, fill=fill)
    torch.cuda.synchronize()
    gk = dk.cpu().numpy().view(np.uint16)
    gv = dv.cpu().numpy().view(np.uint16)
    for b, (hk, hv) in enumerate(_host_gather(pg)):
        n = hk.shape[0]
        assert np.array_equal(gk[b, :n], hk), f"K rows of sequence {b}"
        assert np.array_equal(gv[b, :n], hv), f"V rows of sequence {b}"
        assert np.all(gk[b, n:] == fill) and np.all(gv[b, n:] == fill), f"rows past the end of sequence {b}"
