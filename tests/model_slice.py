"""Test-only Python model of the type-sliced Map kernel for two-node episodes.

Page "Towards Chip-on-Chip Neuroscience: Fast Mining of Frequent Episodes Using
Graphics Processors", "Design of MapConcatenate" (Map rules 1-4, Fig. 4): every
(segment, episode, machine) yields the tuple (a, count, b) of one counting
machine.  For a two-node episode A -(lo, hi]-> B the machine completes at a
B event at t iff some A event lies in [max(r + 1, t - hi), t - lo - 1], r being
its last reset.  That holds iff A has an event in [t - hi, t - lo - 1] (W) and
one in (r, t - lo - 1] (the machine is "fresh"): the later of the two lies in
the intersection.  Episodes sharing (B, lo, hi) therefore step together, one
bit per node-0 type: hit = W & ~blocked, where blocked holds the types whose
last reset has no A event after it yet.

The model follows the kernel's own schedule and state so that its invariants
can be checked on the CPU before any GPU run:
  * chunks of C ticks held with a 64-tick halo (window [c0 - 64, c0 + C));
    every range query stays inside the window and spans at most 64 ticks;
  * a chunk after a stretch of >= 128 event-free ticks starts at the next
    event, and the lane's reset state is dropped (every reset is then more
    than t_high ticks old);
  * resets at ticks after x = t - lo - 1 are "pending" (no A event can be
    after them yet); each pending type remembers its reset tick mod 64 (the
    kernel's six bit planes); a pending reset settles when x reaches it, found
    by walking the B ticks in (x_prev, min(x, last B tick)];
  * settled resets are one entry (tick, mask): an older entry, pruned up to
    x, merges into a newer settled one exactly;
  * the count is a bit-sliced counter of a few planes, flushed every
    ``flush`` in-range B events (the kernel uses eight planes, flush 255).
The reference is ``model_mapconcat.run``: the plain machine on the raw events.
"""
from __future__ import annotations

import numpy as np

import model_mapconcat as MC

FAR = 1 << 60


def groups_of(ep_types, t_low, t_high):
    """Episodes by (node-1 type, lo, hi); within a group, node-0 type -> episode.
    (Node-0 types are the bits of one word: the kernel splits groups of more
    than 64 node-0 types; the model keeps a dict.)"""
    g = {}
    for e in range(len(ep_types)):
        key = (int(ep_types[e][1]), int(t_low[e][0]), int(t_high[e][0]))
        g.setdefault(key, {})
        a = int(ep_types[e][0])
        assert a not in g[key], "duplicate episode"
        g[key][a] = e
    return g


def lane(times, types, beg, end, tau_lo, tau_hi, max_span, r0, B, lo, hi, amap,
         win=512, flush=255, stats=None):
    """Tuples {A: (a, c, b)} of one lane: segment (tau_lo, tau_hi] with event
    range [beg, end), machine reset at r0, node-1 type B, interval (lo, hi],
    node-0 types amap (type -> bit).  win: ticks held per chunk (halo 64)."""
    C = win - 64
    stop = tau_hi + hi
    A_all = set(amap)
    # lane state
    DS, tS = set(A_all), r0            # settled entry: types with no A event after tS
    PA, pend = set(), {}               # pending resets: type -> reset tick mod 64
    xprev, lastb = -FAR, -FAR
    fa, fb = set(), set()
    a_val, b_val = {}, {}
    cnt = {A: 0 for A in A_all}
    planes = {A: 0 for A in A_all}     # the bit-sliced counter, as small ints
    n_in = 0

    c0 = tau_lo - max_span + 1
    ev_lo = beg
    if beg < end and int(times[beg]) >= c0 + 128:
        c0 = int(times[beg])
        DS = set()
    while True:
        base = c0 - 64
        # the window's per-tick node-0 type sets and node-1 ticks
        T, Bt = {}, set()
        i = ev_lo
        while i < end and int(times[i]) < base + win:
            t, y = int(times[i]), int(types[i])
            assert t >= base
            if y in A_all:
                T.setdefault(t, set()).add(y)
            if y == B:
                Bt.add(t)
            i += 1
        s_next = i

        def rng(l, r):
            if l > r:
                return set()
            assert base <= l and r < base + win and r - l + 1 <= 64, (l, r, base)
            out = set()
            for t in range(l, r + 1):
                out |= T.get(t, set())
            return out

        def settle(t, x):
            nonlocal DS, tS, PA
            if DS:
                if tS < t - hi:
                    DS = set()
                else:
                    DS -= rng(tS + 1, x)
            top = min(x, lastb)
            if PA and top > xprev:
                assert top - xprev <= 63
                for tp in sorted(u for u in Bt if xprev < u <= top):
                    Dp = {A for A in PA if pend[A] == tp % 64}
                    if not Dp:
                        continue
                    PA -= Dp
                    if stats is not None:
                        stats["settles"] = stats.get("settles", 0) + 1
                    if tp >= t - hi:
                        DS |= Dp - rng(tp + 1, x)
                        tS = tp

        for t in sorted(u for u in Bt if c0 <= u < c0 + C):
            if t > stop:
                break
            x = t - lo - 1
            settle(t, x)
            xprev = x
            W = rng(t - hi, x)
            hit = W - (DS | PA)
            lastb = t
            if not hit:
                continue
            PA |= hit
            for A in hit:
                pend[A] = t % 64
            if tau_lo < t <= tau_lo + hi:
                for A in hit - fa:
                    a_val[A] = t - tau_lo
                fa |= hit
            if tau_lo < t <= tau_hi:
                for A in hit:
                    planes[A] += 1
                n_in += 1
                if n_in == flush:
                    for A in A_all:
                        cnt[A] += planes[A]
                        planes[A] = 0
                    n_in = 0
                    if stats is not None:
                        stats["flushes"] = stats.get("flushes", 0) + 1
            if t > tau_hi:
                for A in hit - fb:
                    b_val[A] = t - tau_hi
                fb |= hit
        # chunk end: settle as of the first tick of the next chunk
        tv = c0 + C
        xv = tv - lo - 1
        settle(tv, xv)
        xprev = xv
        # next chunk
        if s_next >= end:
            break
        tn = int(times[s_next])
        if tn >= c0 + C + 128:
            c0 = tn
            ev_lo = s_next
            DS, PA = set(), set()
            xprev, lastb = -FAR, -FAR
            if stats is not None:
                stats["jumps"] = stats.get("jumps", 0) + 1
        else:
            c0 = c0 + C
            j = ev_lo
            while j < end and int(times[j]) < c0 - 64:
                j += 1
            ev_lo = j
        if c0 > stop:
            break
    for A in A_all:
        cnt[A] += planes[A]
    return {A: (a_val.get(A, 0), cnt[A], b_val.get(A, 0)) for A in A_all}


def map_tuples(times, types, ep_types, t_low, t_high, P, machines=2, win=512, flush=255,
               stats=None):
    """Tuples of every (segment, episode, machine) as the kernel computes them:
    {(e, p, k): (a, c, b)}."""
    times = np.asarray(times)
    types = np.asarray(types)
    t_min, t_max = int(times[0]), int(times[-1])
    tau = MC.cuts(t_min, t_max, P)
    max_span = int(np.max(t_high))
    out = {}
    for (B, lo, hi), amap in groups_of(ep_types, t_low, t_high).items():
        for p in range(P):
            beg = int(np.searchsorted(times, tau[p] - max_span, side="right"))
            end = int(np.searchsorted(times, tau[p + 1] + max_span, side="right"))
            for k in range(machines):
                r0 = tau[p] - (hi if k == 1 else 0)
                res = lane(times, types, beg, end, tau[p], tau[p + 1], max_span, r0, B, lo, hi,
                           amap, win=win, flush=flush, stats=stats)
                for A, e in amap.items():
                    out[(e, p, k)] = res[A]
    return out, tau


def reference_tuples(times, types, ep_types, t_low, t_high, tau, machines=2):
    """The same tuples from the plain machine (model_mapconcat.run)."""
    out = {}
    P = len(tau) - 1
    for e in range(len(ep_types)):
        ep = [int(v) for v in ep_types[e]]
        lo, hi = [int(t_low[e][0])], [int(t_high[e][0])]
        for p in range(P):
            for k in range(machines):
                r0 = tau[p] - (hi[0] if k == 1 else 0)
                out[(e, p, k)] = MC.run(times, types, ep, lo, hi, r0, tau[p], tau[p + 1], hi[0])
    return out
