"""Brute-force maximum non-overlapped occurrence count, for tiny streams only.

Independent of the oracle's state machine: it enumerates every occurrence of a
serial episode (events t_1 < ... < t_N of the episode's types with
lo_i < t_{i+1} - t_i <= hi_i; page "Towards Chip-on-Chip Neuroscience: Fast
Mining of Frequent Episodes Using Graphics Processors", episode definition in
"Design of MapConcatenate") and then finds the largest set of occurrences that
pairwise do not overlap in time (one starts strictly after the other ends;
Fig. 3 text), two ways: exhaustive search over subsets, and the textbook
dynamic programme for unit-weight interval scheduling.
"""
from __future__ import annotations

from functools import lru_cache


def occurrence_spans(times, types, ep_types, lo, hi):
    """Set of (t_first, t_last) over all occurrences, by exhaustive extension."""
    n = len(times)
    N = len(ep_types)
    spans = set()

    def extend(level, idx, t_first):
        if level == N - 1:
            spans.add((t_first, int(times[idx])))
            return
        want = ep_types[level + 1]
        for j in range(n):
            if types[j] != want:
                continue
            d = int(times[j]) - int(times[idx])
            if lo[level] < d <= hi[level]:
                extend(level + 1, j, t_first)

    for i in range(n):
        if types[i] == ep_types[0]:
            extend(0, i, int(times[i]))
    return spans


def max_disjoint_exhaustive(spans):
    """Largest pairwise-disjoint subset of closed spans, by trying every subset."""
    spans = sorted(spans)
    m = len(spans)
    if m > 16:
        raise ValueError("too many spans for exhaustive search")

    def disjoint(u, v):
        return u[0] > v[1] or v[0] > u[1]

    best = 0
    # enumerate subsets; keep those that are pairwise disjoint
    for mask in range(1 << m):
        chosen = [spans[i] for i in range(m) if mask >> i & 1]
        if len(chosen) <= best:
            continue
        ok = all(disjoint(chosen[i], chosen[j])
                 for i in range(len(chosen)) for j in range(i + 1, len(chosen)))
        if ok:
            best = len(chosen)
    return best


def max_disjoint_dp(spans):
    """Unit-weight interval scheduling by dynamic programming over end times."""
    spans = sorted(spans, key=lambda s: (s[1], s[0]))
    m = len(spans)
    ends = [s[1] for s in spans]

    @lru_cache(maxsize=None)
    def best(i):
        # best over spans[0..i-1]
        if i == 0:
            return 0
        s, e = spans[i - 1]
        # spans with end < s among the first i-1 (ends sorted)
        j = 0
        while j < i - 1 and ends[j] < s:
            j += 1
        return max(best(i - 1), 1 + best(j))

    return best(m)


def brute_count(times, types, ep_types, lo, hi, exhaustive_limit=12):
    """Max non-overlapped count; cross-checks the two optimisers when feasible."""
    spans = occurrence_spans(times, types, ep_types, lo, hi)
    dp = max_disjoint_dp(spans)
    if len(spans) <= exhaustive_limit:
        ex = max_disjoint_exhaustive(spans)
        if ex != dp:
            raise AssertionError("brute-force optimisers disagree: %d vs %d" % (ex, dp))
    return dp
