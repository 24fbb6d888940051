"""Load balance of block-sparse attention: host-side diagnostics and plans.

The work unit is one kept 128x128 block of the mask: every kept block
costs the same matrix work (4 * 128 * 128 * D flops). The db-SP page
("db-SP: Accelerating Sparse Attention for Visual Generative Models with
Dual-Balanced Sequence Parallelism", Abstract) traces the imbalance of
sparse attention under sequence parallelism to two sources: sparsity that
differs between heads (which hurts a split along heads, as in Ulysses) and
kept blocks spread irregularly over the mask (which hurts a split along
blocks, as in Ring Attention). It names a "sparse imbalance ratio" but does
not print it. Here the imbalance ratio of a split of the work into parts
with loads W_1..W_P is defined as

    R = max_p W_p / mean_p W_p,

the ratio of the slowest part to a perfectly balanced one (1 = balanced,
P = one part does everything).

Functions:
  kept_counts             kept blocks of every mask row, [B, H, n_qb]
  imbalance_ratio         R of a list of loads
  ulysses_head_loads      loads of a split into contiguous head ranges
  ring_row_loads          loads of a split into contiguous query-row ranges
  balanced_head_split     a sparsity-aware split of the heads: heaviest head
                          first, to the least-loaded part that still has
                          room (every part gets H / P heads)
  balanced_row_split      the contiguous split of the query rows into P
                          ranges with the smallest largest load
  dual_level_plan         P devices as a grid of Ph head groups x Pr row
                          ranges, every factorization P = Ph * Pr tried
                          (the page's dual-level partitioning with its
                          degrees chosen from the mask)
  schedule_from_workspace the launch schedule lsh_attn_fwd_blocksparse
                          leaves in its workspace
  schedule_loads          per-XCD loads of that schedule and the makespan
                          of its CUs, simulated
This module is plain numpy on the host; it runs no attention arithmetic.
"""
from __future__ import annotations

import heapq

import numpy as np

__all__ = ["kept_counts", "imbalance_ratio", "ulysses_head_loads", "ring_row_loads",
           "balanced_head_split", "balanced_row_split", "dual_level_plan",
           "schedule_from_workspace", "schedule_loads"]


def kept_counts(mask) -> np.ndarray:
    """mask [B, H, n_qb, n_kb] (nonzero = kept) -> int64 [B, H, n_qb]."""
    m = np.asarray(mask)
    if m.ndim != 4:
        raise ValueError("mask must be [B, H, n_qb, n_kb]")
    return (m != 0).sum(axis=-1).astype(np.int64)


def imbalance_ratio(loads) -> float:
    """max / mean of the loads; 1.0 for an all-zero load vector."""
    w = np.asarray(loads, dtype=np.float64).ravel()
    if w.size == 0:
        raise ValueError("no parts")
    mean = w.mean()
    return 1.0 if mean == 0 else float(w.max() / mean)


def ulysses_head_loads(counts, parts: int) -> np.ndarray:
    """Heads split into `parts` contiguous ranges of H / parts heads (every
    batch entry's copy of a head goes with it)."""
    c = np.asarray(counts, dtype=np.int64)
    B, H, _ = c.shape
    if parts < 1 or H % parts:
        raise ValueError(f"H={H} is not a multiple of {parts}")
    per_head = c.sum(axis=(0, 2))
    return per_head.reshape(parts, H // parts).sum(axis=1)


def ring_row_loads(counts, parts: int) -> np.ndarray:
    """Query-block rows split into `parts` contiguous ranges (sizes differ
    by at most one), each part holding its rows of every head."""
    c = np.asarray(counts, dtype=np.int64)
    n_qb = c.shape[2]
    if parts < 1 or parts > n_qb:
        raise ValueError(f"cannot split {n_qb} rows into {parts} parts")
    per_row = c.sum(axis=(0, 1))
    bounds = np.linspace(0, n_qb, parts + 1).round().astype(int)
    return np.array([per_row[bounds[p]:bounds[p + 1]].sum() for p in range(parts)],
                    dtype=np.int64)


def balanced_head_split(counts, parts: int):
    """Sparsity-aware head split: heads in descending total (ties: lower
    index first), each to the part with the smallest load among those with
    fewer than H / parts heads (ties: lower part index).
    Returns (heads per part as lists, loads)."""
    c = np.asarray(counts, dtype=np.int64)
    B, H, _ = c.shape
    if parts < 1 or H % parts:
        raise ValueError(f"H={H} is not a multiple of {parts}")
    cap = H // parts
    per_head = c.sum(axis=(0, 2))
    heads = sorted(range(H), key=lambda h: (-per_head[h], h))
    assign = [[] for _ in range(parts)]
    loads = np.zeros(parts, dtype=np.int64)
    for h in heads:
        p = min((q for q in range(parts) if len(assign[q]) < cap), key=lambda q: (loads[q], q))
        assign[p].append(h)
        loads[p] += per_head[h]
    return assign, loads


def balanced_row_split(row_loads, parts: int):
    """Contiguous split of rows (in order) into `parts` non-empty ranges
    whose largest load is as small as possible: a binary search on that
    load, each candidate checked by filling ranges greedily. Returns
    (range boundaries [0 = b_0 < ... < b_parts = n], loads)."""
    w = np.asarray(row_loads, dtype=np.int64).ravel()
    n = w.size
    if parts < 1 or parts > n:
        raise ValueError(f"cannot split {n} rows into {parts} parts")

    def cuts_for(cap):
        # greedy: close a range when the next row would exceed cap, keeping
        # enough rows for the remaining ranges
        bounds, acc, left = [0], 0, parts
        for i in range(n):
            rows_after = n - i
            if bounds[-1] < i and (acc + w[i] > cap or rows_after < left):
                bounds.append(i)
                acc, left = 0, left - 1
            if w[i] > cap:
                return None
            acc += w[i]
        if len(bounds) > parts:
            return None
        # split the largest ranges further until there are `parts` of them
        while len(bounds) < parts:
            spans = [(bounds[j + 1] if j + 1 < len(bounds) else n) - bounds[j]
                     for j in range(len(bounds))]
            j = max(range(len(spans)), key=lambda q: (spans[q], -q))
            bounds.insert(j + 1, bounds[j] + spans[j] // 2)
        return bounds + [n]

    lo, hi = int(w.max(initial=0)), int(w.sum())
    while lo < hi:
        mid = (lo + hi) // 2
        if cuts_for(mid) is None:
            lo = mid + 1
        else:
            hi = mid
    bounds = cuts_for(lo)
    loads = np.array([w[bounds[p]:bounds[p + 1]].sum() for p in range(parts)], dtype=np.int64)
    return bounds, loads


def dual_level_plan(counts, devices: int):
    """Every grid Ph x Pr = devices with H % Ph == 0 and Pr <= query rows:
    heads split into Ph groups by balanced_head_split, each group's rows
    (its kept blocks summed over its heads) into Pr ranges by
    balanced_row_split. Returns the plans sorted by imbalance ratio (then
    fewer head groups), each a dict with Ph, Pr, the ratio and the device
    loads."""
    c = np.asarray(counts, dtype=np.int64)
    B, H, n_qb = c.shape
    plans = []
    for ph in range(1, devices + 1):
        if devices % ph or H % ph:
            continue
        pr = devices // ph
        if pr > n_qb:
            continue
        groups, _ = balanced_head_split(c, ph)
        loads = []
        for heads in groups:
            rows = c[:, heads, :].sum(axis=(0, 1))
            loads.extend(balanced_row_split(rows, pr)[1].tolist())
        loads = np.array(loads, dtype=np.int64)
        plans.append({"Ph": ph, "Pr": pr, "ratio": imbalance_ratio(loads), "loads": loads})
    if not plans:
        raise ValueError(f"no grid of {devices} devices fits H={H} and {n_qb} query rows")
    return sorted(plans, key=lambda d: (d["ratio"], d["Ph"]))


def schedule_from_workspace(ws, n_items: int, n_heads: int, offset: int = 0):
    """(counts, order, totals) from the bytes of a block-sparse workspace
    (the layout lsh.h documents: int32 counts[n], int32 order[n], int64
    totals[n_heads], each region starting on a 256-byte boundary).
    `ws` is a uint8 array (or anything numpy can view as one); `offset` is
    the byte offset of the library's workspace inside it."""
    raw = np.ascontiguousarray(np.asarray(ws).view(np.uint8).ravel()[offset:])
    region = (n_items * 4 + 255) // 256 * 256
    need = 2 * region + n_heads * 8
    if raw.size < need:
        raise ValueError(f"workspace holds {raw.size} bytes, the schedule needs {need}")
    counts = raw[:n_items * 4].view(np.int32).astype(np.int64)
    order = raw[region:region + n_items * 4].view(np.int32).astype(np.int64)
    totals = raw[2 * region:2 * region + n_heads * 8].view(np.int64).copy()
    return counts, order, totals


def schedule_loads(counts, order, n_xcd: int = 8, cus_per_xcd: int = 32,
                   overhead: float = 0.0):
    """Loads of a launch schedule on one GPU.

    Launch slot s runs item order[s] on XCD s % n_xcd (the dispatcher deals
    workgroups to the XCDs in turn). Inside an XCD the items start in slot
    order, each on the CU that becomes free first (ties: lower CU), and take
    counts[item] + overhead time units. Returns a dict with the per-XCD
    loads, their imbalance ratio, the makespan and its ratio to the
    balanced makespan (total time / number of CUs)."""
    c = np.asarray(counts, dtype=np.float64).ravel()
    o = np.asarray(order, dtype=np.int64).ravel()
    if np.sort(o).tolist() != list(range(c.size)):
        raise ValueError("order is not a permutation of the items")
    dur = c[o] + overhead
    xcd_loads = np.array([dur[x::n_xcd].sum() for x in range(n_xcd)])
    makespan = 0.0
    for x in range(n_xcd):
        free = [(0.0, cu) for cu in range(cus_per_xcd)]
        heapq.heapify(free)
        end = 0.0
        for d in dur[x::n_xcd]:
            t, cu = heapq.heappop(free)
            heapq.heappush(free, (t + d, cu))
            end = max(end, t + d)
        makespan = max(makespan, end)
    ideal = float(dur.sum()) / (n_xcd * cus_per_xcd)
    return {"xcd_loads": xcd_loads, "xcd_ratio": imbalance_ratio(xcd_loads),
            "makespan": float(makespan),
            "makespan_ratio": 1.0 if ideal == 0 else float(makespan) / ideal}
