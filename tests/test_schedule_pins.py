"""Pins of the scheduling oracle (oracle/schedule.py) against what the pages
print in "FlashAttention4 close reading", section 3.3 (scheduling), and
against closed forms."""
import random

import oracle.schedule as S


def test_eight_tasks_on_four_processors():
    # the page's example: tasks 1..8 on 4 processors finish at 12 when the
    # short ones go first and at 9 when the long ones do
    assert S.list_schedule_makespan(range(1, 9), 4) == 12
    assert S.list_schedule_makespan(range(8, 0, -1), 4) == 9
    # 9 is the lower bound (36 units of work on 4 processors)
    assert 9 * 4 == sum(range(1, 9))


def test_virtual_to_actual_example():
    # the page's permutation: original order 0,1,2,3 whose estimated times
    # sort as 1,2,3,0 gives virtual 0..3 -> actual 1,2,3,0
    cu_q = [0, 64, 128, 192, 256]
    cu_k = [0, 64, 320, 512, 640]      # lk = 64, 256, 192, 128 -> 1, 4, 3, 2 tiles
    assert S.lpt_order(cu_q, cu_k, False, 256, 64) == [1, 2, 3, 0]


def test_causal_triangle():
    # 8 query blocks of the tile size: block m visits m + 1 key tiles
    assert [S.tile_kv_blocks(512, 512, True, 64, 64, m) for m in range(8)] == list(range(1, 9))
    # non-causal: every block visits all of them
    assert [S.tile_kv_blocks(512, 512, False, 64, 64, m) for m in range(8)] == [8] * 8


def test_bottom_right_alignment_and_empty_items():
    # 100 queries against 300 keys, causal: row i sees keys < i + 201
    assert S.tile_kv_blocks(100, 300, True, 64, 64, 0) == 5      # rows 0..63 -> keys < 264
    assert S.tile_kv_blocks(100, 300, True, 64, 64, 1) == 5      # rows 64..99 -> keys < 300
    # more queries than keys: the first block sees nothing
    assert S.tile_kv_blocks(300, 100, True, 64, 64, 0) == 0
    assert S.seq_weight(0, 500, True, 256, 64) == 0
    assert S.seq_weight(300, 100, True, 256, 64) == 2


def test_weight_is_the_heaviest_tile_not_the_total():
    # A: 64 queries over 8192 keys (one tile of 128 key blocks);
    # B: 4096 x 4096 non-causal (64 tiles of 64 key blocks: 32x A's work).
    # The page orders by the longest tile, so A goes first.
    cu_q = [0, 4096, 4160]
    cu_k = [0, 4096, 4096 + 8192]
    assert S.lpt_order(cu_q, cu_k, False, 64, 64) == [1, 0]


def test_ties_keep_the_input_order():
    cu = [0, 128, 256, 384]
    assert S.lpt_order(cu, cu, True, 256, 64) == [0, 1, 2]


def test_lpt_on_ragged_batches():
    # Graham's bound for longest-first list scheduling, LPT <= (4/3) OPT with
    # OPT >= max(total / m, longest task), always holds; that LPT also beats
    # shortest-first (the page's bad order) is checked on these seeded cases
    rng = random.Random(5)
    for _ in range(50):
        n = rng.randint(2, 12)
        lens = [rng.randint(1, 40) * 64 for _ in range(n)]
        cu = [0]
        for L in lens:
            cu.append(cu[-1] + L)
        order = S.lpt_order(cu, cu, True, 64, 64)
        # durations of whole items (their tiles back to back) in each order
        dur = [sum(S.tile_kv_blocks(L, L, True, 64, 64, m) for m in range(L // 64)) for L in lens]
        # with the heaviest-tile weight, for lq = lk items the order is by length
        assert [lens[b] for b in order] == sorted(lens, reverse=True)
        lpt = S.list_schedule_makespan([dur[b] for b in order], 4)
        assert 3 * lpt <= 4 * max(-(-sum(dur) // 4), max(dur))
        assert lpt <= S.list_schedule_makespan(sorted(dur), 4)


def test_planted_mistake_is_caught():
    # sorting ascending instead of descending breaks the page's permutation
    cu_q = [0, 64, 128, 192, 256]
    cu_k = [0, 64, 320, 512, 640]
    w = [S.seq_weight(64, L, False, 256, 64) for L in (64, 256, 192, 128)]
    assert sorted(range(4), key=lambda b: (w[b], b)) != [1, 2, 3, 0]


def test_hierarchical_traversal_example():
    # the page's printed traversal: batch 0, sections of two heads, row blocks
    # from the last to the first, the section's heads for each row block
    import json
    import pathlib
    fx = json.loads((pathlib.Path(__file__).parent / "golden" / "traversal_example.json").read_text())
    want = [tuple(x) for x in fx["order_batch0"]]
    assert S.hierarchical_tile_order(fx["batches"], fx["heads"], fx["mblocks"], fx["section"]) == want
    # "then batch 1": with two batches the second one's tiles all follow
    two = S.hierarchical_tile_order(2, 4, 4, 2)
    assert two[:16] == want and all(b == 1 for b, _, _ in two[16:]) and len(two) == 32
    # every (batch, head, mblock) exactly once, whatever the section size
    for sec in (1, 3, 4, 8):
        o = S.hierarchical_tile_order(3, 5, 7, sec)
        assert sorted(o) == sorted((b, h, m) for b in range(3) for h in range(5) for m in range(7))
        # within a batch and section, row blocks never increase
        for b in range(3):
            for h in range(5):
                mbs = [m for (bb, hh, m) in o if bb == b and hh == h]
                assert mbs == sorted(mbs, reverse=True)
