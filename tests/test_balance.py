"""Host-side load-balance diagnostics of block-sparse attention
(long_sequence_head_amd/balance.py), checked on hand-computed cases."""
import numpy as np
import pytest

from long_sequence_head_amd import balance as BL


def test_imbalance_ratio():
    assert BL.imbalance_ratio([1, 1, 1]) == 1.0
    assert BL.imbalance_ratio([3, 0, 0]) == 3.0
    assert BL.imbalance_ratio([2, 1]) == pytest.approx(4 / 3)
    assert BL.imbalance_ratio([0, 0]) == 1.0
    with pytest.raises(ValueError):
        BL.imbalance_ratio([])


def test_kept_counts():
    m = np.zeros((1, 2, 2, 3), dtype=np.uint8)
    m[0, 0, 0] = [1, 0, 1]
    m[0, 1, 1] = [1, 1, 7]
    assert BL.kept_counts(m).tolist() == [[[2, 0], [0, 3]]]


def _counts(rows_per_head):
    return np.array([rows_per_head], dtype=np.int64)   # B = 1


def test_ulysses_and_ring_splits():
    c = _counts([[3, 1], [0, 0], [2, 2], [1, 1]])      # heads 4, 0, 4, 2
    assert BL.ulysses_head_loads(c, 2).tolist() == [4, 6]
    assert BL.ulysses_head_loads(c, 4).tolist() == [4, 0, 4, 2]
    assert BL.ring_row_loads(c, 2).tolist() == [6, 4]   # row 0: 3+0+2+1, row 1: 1+0+2+1
    with pytest.raises(ValueError):
        BL.ulysses_head_loads(c, 3)
    with pytest.raises(ValueError):
        BL.ring_row_loads(c, 3)


def test_balanced_head_split_hand_case():
    # head totals 5, 4, 3, 3, 3, 0; two parts of three heads each:
    # h0 -> p0 (5), h1 -> p1 (4), h2 -> p1 (7), h3 -> p0 (8), h4 -> p1 (10,
    # full), h5 -> p0 (8)
    c = _counts([[5], [4], [3], [3], [3], [0]])
    assign, loads = BL.balanced_head_split(c, 2)
    assert assign == [[0, 3, 5], [1, 2, 4]]
    assert loads.tolist() == [8, 10]


def test_balanced_head_split_properties():
    rng = np.random.default_rng(3)
    c = rng.integers(0, 50, size=(2, 16, 9))
    for parts in (1, 2, 4, 8, 16):
        assign, loads = BL.balanced_head_split(c, parts)
        flat = sorted(h for a in assign for h in a)
        assert flat == list(range(16))
        assert all(len(a) == 16 // parts for a in assign)
        assert loads.sum() == c.sum()
        per_head = c.sum(axis=(0, 2))
        assert [int(per_head[a].sum()) for a in assign] == loads.tolist()
        # never worse than the contiguous split on this input
        assert BL.imbalance_ratio(loads) <= BL.imbalance_ratio(BL.ulysses_head_loads(c, parts))


def test_schedule_from_workspace_layout():
    n, heads = 70, 3
    counts = np.arange(n, dtype=np.int32) % 7
    order = np.arange(n, dtype=np.int32)[::-1].copy()
    totals = np.array([10, 2 ** 40, 5], dtype=np.int64)
    region = (n * 4 + 255) // 256 * 256
    ws = np.zeros(16 + 2 * region + heads * 8 + 40, dtype=np.uint8)
    base = 16
    ws[base:base + n * 4] = counts.view(np.uint8)
    ws[base + region:base + region + n * 4] = order.view(np.uint8)
    ws[base + 2 * region:base + 2 * region + heads * 8] = totals.view(np.uint8)
    c2, o2, t2 = BL.schedule_from_workspace(ws, n, heads, offset=base)
    assert c2.tolist() == counts.tolist() and o2.tolist() == order.tolist()
    assert t2.tolist() == totals.tolist()
    with pytest.raises(ValueError):
        BL.schedule_from_workspace(ws[:100], n, heads)


def test_schedule_loads_hand_case():
    counts = [4, 3, 2, 1, 1, 1, 1, 1]
    order = list(range(8))
    # two XCDs: slots 0, 2, 4, 6 -> 4 + 2 + 1 + 1 = 8; slots 1, 3, 5, 7 -> 6
    r = BL.schedule_loads(counts, order, n_xcd=2, cus_per_xcd=1)
    assert r["xcd_loads"].tolist() == [8, 6]
    assert r["xcd_ratio"] == pytest.approx(8 / 7)
    assert r["makespan"] == 8 and r["makespan_ratio"] == pytest.approx(8 / 7)
    # two CUs per XCD: XCD 0 runs 4 | 2, 1, 1 -> 4; XCD 1 runs 3 | 1, 1, 1 -> 3
    r = BL.schedule_loads(counts, order, n_xcd=2, cus_per_xcd=2)
    assert r["makespan"] == 4 and r["makespan_ratio"] == pytest.approx(4 / 3.5)
    # a per-workgroup overhead adds to every duration
    r = BL.schedule_loads(counts, order, n_xcd=2, cus_per_xcd=1, overhead=1.0)
    assert r["xcd_loads"].tolist() == [12, 10]
    with pytest.raises(ValueError):
        BL.schedule_loads(counts, [0, 0, 1, 2, 3, 4, 5, 6])


def test_descending_order_beats_ascending_on_cus():
    """Longest-first starts shorten the makespan of list scheduling here:
    durations 1 x 6 and 6 on 2 CUs: shortest first ends at 9, longest
    first at 6."""
    counts = [1, 1, 1, 1, 1, 1, 6]
    asc = list(range(7))
    desc = [6] + list(range(6))
    a = BL.schedule_loads(counts, asc, n_xcd=1, cus_per_xcd=2)
    d = BL.schedule_loads(counts, desc, n_xcd=1, cus_per_xcd=2)
    assert a["makespan"] == 9 and d["makespan"] == 6


def test_balanced_row_split_is_optimal_by_brute_force():
    import itertools
    rng = np.random.default_rng(7)
    for _ in range(120):
        n = int(rng.integers(1, 9))
        parts = int(rng.integers(1, n + 1))
        w = rng.integers(0, 10, size=n)
        bounds, loads = BL.balanced_row_split(w, parts)
        assert bounds[0] == 0 and bounds[-1] == n and len(bounds) == parts + 1
        assert all(bounds[i] < bounds[i + 1] for i in range(parts))
        assert loads.sum() == w.sum()
        best = min(max(w[x[i]:x[i + 1]].sum() for i in range(parts))
                   for cuts in itertools.combinations(range(1, n), parts - 1)
                   for x in [[0, *cuts, n]])
        assert loads.max() == best


def test_balanced_row_split_hand_case():
    bounds, loads = BL.balanced_row_split([1, 1, 1, 1, 4], 2)
    assert loads.max() == 4 and bounds == [0, 4, 5]
    with pytest.raises(ValueError):
        BL.balanced_row_split([1, 2], 3)


def test_dual_level_plan_picks_the_better_grid():
    # head 0 keeps 8 blocks in its first row, head 1 one block per row.
    # 1 x 2 grid: rows 9, 1, 1, 1 -> best cut 9 | 3 -> ratio 9 / 6 = 1.5;
    # 2 x 1 grid: heads 8 | 4 -> ratio 8 / 6.
    c = _counts([[8, 0, 0, 0], [1, 1, 1, 1]])
    plans = BL.dual_level_plan(c, 2)
    assert [(p["Ph"], p["Pr"]) for p in plans] == [(2, 1), (1, 2)]
    assert plans[0]["ratio"] == pytest.approx(8 / 6)
    assert plans[1]["ratio"] == pytest.approx(9 / 6)
    assert plans[0]["loads"].tolist() == [8, 4]
    with pytest.raises(ValueError):
        BL.dual_level_plan(_counts([[1]]), 2)   # one head, one row: no 2-device grid
