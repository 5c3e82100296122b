"""Test-only Python model of MapConcatenate's tuple algebra.

Page "Towards Chip-on-Chip Neuroscience: Fast Mining of Frequent Episodes Using
Graphics Processors", "Design of MapConcatenate": the stream is cut into P
segments (tau_p, tau_{p+1}]; segment p runs N machines, machine k reset at
tau_p - (hi_1 + ... + hi_k) (Fig. 4); each emits (a, count, b) (Map rules 1-4,
Fig. 5), and a log-depth tree joins adjacent segments where b_s = a_t
(Concatenate rules 1-3, Fig. 6).

Readings this model settles before any GPU code exists:
  * a-window and b-window are (tau, tau + Span], closed on the right.
  * a and b are stored as offsets from their segment's left / right cut, so
    the left block's b and the right block's a share one base; 0 is the
    sentinel ("no completion within Span": equivalent to a reset at the cut).
  * A machine reset at x has the same future as any other reset at x, so equal
    keys mean identical tuples.
  * When a segment's exit has no matching key in the next segment (possible
    when some t_low > 0), a repair tuple is made by a machine reset exactly at
    that exit; repairs repeat along the stream until every exit is matched.
The windows here are merged half-open intervals (one deque per node), a
representation separate from the oracle's raw timestamp lists.
"""
from __future__ import annotations

import numpy as np


def cuts(t_min: int, t_max: int, P: int):
    """Equal-time cuts tau_0..tau_P with tau_0 = t_min - 1 and tau_P = t_max."""
    return [t_min - 1 + (p * (t_max - t_min + 1)) // P for p in range(P + 1)]


class Machine:
    """The serial counting machine with merged-interval windows.

    windows[k] holds disjoint, sorted intervals (s, e]: a node k+2 event at time
    t may extend a prefix iff t lies in one of them.
    """

    def __init__(self, ep, lo, hi, reset_at):
        self.ep = [int(v) for v in ep]
        self.lo = [int(v) for v in lo]
        self.hi = [int(v) for v in hi]
        self.N = len(self.ep)
        self.r = reset_at
        self.win = [[] for _ in range(max(self.N - 1, 0))]
        self.max_live = 0

    def _in(self, k, t):
        w = self.win[k]
        while w and w[0][1] < t:
            w.pop(0)
        return bool(w) and w[0][0] < t

    def _insert(self, k, t):
        w = self.win[k]
        while w and w[0][1] < t:
            w.pop(0)
        s, e = t + self.lo[k], t + self.hi[k]
        if w and w[-1][1] >= s:
            w[-1] = (w[-1][0], e)
        else:
            w.append((s, e))
        self.max_live = max(self.max_live, len(w))

    def step(self, t, y) -> bool:
        """Feed one event; True if it completes an occurrence (then reset at t)."""
        if t <= self.r:
            return False
        N = self.N
        if y == self.ep[N - 1] and (N == 1 or self._in(N - 2, t)):
            self.r = t
            for w in self.win:
                w.clear()
            return True
        for k in range(N - 1):
            if y == self.ep[k] and (k == 0 or self._in(k - 1, t)):
                self._insert(k, t)
        return False


def run(times, types, ep, lo, hi, reset_at, tau_lo, tau_hi, span):
    """Machine reset at ``reset_at`` over one segment (tau_lo, tau_hi].

    Returns (a_off, count, b_off): a = first completion in (tau_lo, tau_lo+span]
    (offset from tau_lo, 0 if none), count = completions in (tau_lo, tau_hi],
    b = first completion in (tau_hi, tau_hi+span] (offset from tau_hi, 0 if none).
    """
    m = Machine(ep, lo, hi, reset_at)
    i = int(np.searchsorted(times, reset_at, side="right"))
    first_after = None
    count = 0
    b = None
    while i < len(times):
        t = int(times[i])
        if t > tau_hi + span:
            break
        if m.step(t, int(types[i])) and t > tau_lo:
            if first_after is None:
                first_after = t
            if t <= tau_hi:
                count += 1
            else:
                b = t
                break
        i += 1
    a_off = first_after - tau_lo if (first_after is not None and first_after <= tau_lo + span) else 0
    b_off = b - tau_hi if b is not None else 0
    return a_off, count, b_off


def repair(times, types, ep, lo, hi, x, tau_lo, tau_hi, span):
    """Tuple of a chain that completed at x in (tau_lo, tau_lo+span] (reset at x)."""
    if x > tau_hi:
        return x - tau_lo, 0, x - tau_hi
    _, c, b_off = run(times, types, ep, lo, hi, x, tau_lo, tau_hi, span)
    # every completion of the machine is after x > tau_lo: ``c`` counts them up
    # to tau_hi; the completion at x itself is counted here.
    return x - tau_lo, c + 1, b_off


def map_tuples(times, types, ep, lo, hi, tau):
    P = len(tau) - 1
    N = len(ep)
    prefix = np.concatenate([[0], np.cumsum(np.asarray(hi, dtype=np.int64))]).astype(np.int64)
    span = int(prefix[-1])
    T = []
    for p in range(P):
        row = []
        for k in range(N):
            row.append(run(times, types, ep, lo, hi, tau[p] - int(prefix[k]), tau[p], tau[p + 1], span))
        T.append(row)
    return T, span


def close(times, types, ep, lo, hi, tau, T, span):
    """Add repair tuples until every exit of segment p is a key of segment p+1."""
    P = len(tau) - 1
    misses = 0
    for p in range(P - 1):
        q = p + 1
        pending = [tup[2] for tup in T[p]]
        while pending:
            x_off = pending.pop()
            keys = {tup[0] for tup in T[q]}
            if x_off in keys:
                continue
            misses += 1
            x = tau[q] + x_off
            T[q].append(repair(times, types, ep, lo, hi, x, tau[q], tau[q + 1], span))
        # new tuples of q are checked when q becomes the left side
    return misses


def concatenate_tree(T):
    """Level-wise joins of adjacent blocks (Concatenate rules 1-3).

    A block's tuples are keyed by its first segment's keys; joining left block
    L with right block R maps each left tuple (a, c, b) to (a, c + c', b') for
    the first right tuple whose key a' equals b.
    """
    blocks = [list(row) for row in T]
    while len(blocks) > 1:
        nxt = []
        for j in range(0, len(blocks), 2):
            if j + 1 == len(blocks):
                nxt.append(blocks[j])
                continue
            L, R = blocks[j], blocks[j + 1]
            merged = []
            for (a, c, b) in L:
                hit = next((t for t in R if t[0] == b), None)
                if hit is None:
                    raise AssertionError("unmatched exit %d" % b)
                merged.append((a, c + hit[1], hit[2]))
            nxt.append(merged)
        blocks = nxt
    return blocks[0]


def count_mapconcat(times, types, ep, lo, hi, P, with_stats=False):
    times = np.asarray(times)
    types = np.asarray(types)
    if times.size == 0:
        return (0, {"misses": 0}) if with_stats else 0
    tau = cuts(int(times[0]), int(times[-1]), P)
    T, span = map_tuples(times, types, ep, lo, hi, tau)
    misses = close(times, types, ep, lo, hi, tau, T, span)
    root = concatenate_tree(T)
    # segment 0's machine k=0 is reset before the first event: it is alpha_0
    result = root[0][1]
    # segment 0's machines all see the whole prefix: their counts must agree
    assert all(t[1] == result for t in root[:len(ep)])
    return (result, {"misses": misses}) if with_stats else result
