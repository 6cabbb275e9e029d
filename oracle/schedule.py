"""Longest-first ordering of query-tile work items (plain definition).

TEST INFRASTRUCTURE (only tests/, ``__graft_entry__.smoke()`` and bench.py's
``cpu_baseline`` leg may use oracle/).

Under a causal mask or with packed sequences of different lengths the work items
differ in cost, and the method dispatches the most expensive ones first
(fdeinterviews.com FA4 summary, features paragraph).  A work item is one
block of ``block_m`` consecutive query rows of one sequence (and one head); its
length is the number of ``block_n``-key tiles it must visit: all of the
sequence's key tiles without a mask, and under the causal mask only the tiles
holding a key at or before the item's last row.

Any order whose costs never increase is a valid longest-first order (equal costs
may come in any order), so checks compare the multiset of items and the cost
sequence, and verify monotonicity.

The pages do not fix the granularity at which items go most expensive first.  The
library reads it at the granularity of cost buckets (the grouped order below): items
whose costs fall in the same bucket of ``width`` cost units are equally long for
dispatch, buckets go most expensive first, and inside a bucket each sequence's items
stay together, longest first, so that neighbouring tiles of one sequence run at the
same time.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple


def item_cost(row0: int, block_m: int, seqlen_q: int, seqlen_k: int, block_n: int,
              causal: bool) -> int:
    """Key tiles visited by the query rows [row0, min(row0+block_m, seqlen_q))."""
    if seqlen_k <= 0:
        return 0
    if not causal:
        keys = seqlen_k
    else:
        # bottom-right causal alignment: row i sees keys j <= i + seqlen_k - seqlen_q
        last_row = min(row0 + block_m, seqlen_q) - 1
        keys = max(0, min(last_row + 1 + seqlen_k - seqlen_q, seqlen_k))
    return -(-keys // block_n)


def work_items(seqlens: Sequence[int], block_m: int, block_n: int,
               causal: bool) -> List[Tuple[int, int, int]]:
    """All (sequence, query-tile index, cost) items, in natural order."""
    items = []
    for b, length in enumerate(seqlens):
        length = int(length)
        for t in range(-(-length // block_m)):
            items.append((b, t, item_cost(t * block_m, block_m, length, length, block_n, causal)))
    return items


def longest_first(items: Sequence[Tuple[int, int, int]]) -> List[Tuple[int, int, int]]:
    """One valid longest-first order: stable sort by decreasing cost."""
    return sorted(items, key=lambda it: -it[2])


def is_longest_first(order: Sequence[Tuple[int, int, int]],
                     items: Sequence[Tuple[int, int, int]]) -> bool:
    """True if ``order`` is a permutation of ``items`` with non-increasing cost."""
    if sorted(order) != sorted(items):
        return False
    costs = [c for _, _, c in order]
    return all(a >= b for a, b in zip(costs, costs[1:]))


def bucket_width(block_m: int, block_n: int, group: int = 16) -> int:
    """Cost units per bucket of the grouped order: the cost growth of ``group``
    consecutive causal items of one sequence (each item adds block_m / block_n key
    tiles), at least 1."""
    return max(1, group * block_m // block_n)


def grouped_longest_first(items: Sequence[Tuple[int, int, int]], width: int) -> List[Tuple[int, int, int]]:
    """One valid grouped order: buckets (cost // width) most expensive first; inside a
    bucket, sequence by sequence, each sequence's items by decreasing cost."""
    return sorted(items, key=lambda it: (-(it[2] // width), it[0], -it[2], it[1]))


def is_grouped_longest_first(order: Sequence[Tuple[int, int, int]],
                             items: Sequence[Tuple[int, int, int]], width: int) -> bool:
    """True if ``order`` is a permutation of ``items`` whose bucket index (cost // width)
    never increases and in which, inside each bucket, every sequence's items form one
    contiguous run of non-increasing cost."""
    if sorted(order) != sorted(items):
        return False
    buckets = [c // width for _, _, c in order]
    if any(a < b for a, b in zip(buckets, buckets[1:])):
        return False
    runs_seen = set()
    run = None
    last_cost = 0
    for b, _, c in order:
        key = (b, c // width)
        if key != run:
            if key in runs_seen:
                return False  # the sequence's run in this bucket was interrupted
            runs_seen.add(key)
            run = key
        elif c > last_cost:
            return False
        last_cost = c
    return True
