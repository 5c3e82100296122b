"""Seeded synthetic event streams and candidate-episode sets.

These generators are the only code shared by the GPU path's tests and the CPU
oracle's tests.  They hold none of the counting arithmetic: they draw spike
trains and episode definitions with numpy's ``default_rng`` and nothing else.

The shapes follow the workloads of the page "Towards Chip-on-Chip Neuroscience:
Fast Mining of Frequent Episodes Using Graphics Processors" (experiments
section: a few dozen neuron types firing as Poisson processes at ~20 Hz with
embedded causal chains), scaled to five configurations:

  tiny        10,000 events, 26 types, gaps U{1..4}, 20 planted A->B->C chains,
              64 three-node episodes with (0,5] delays.
  ptpe        1,000,000 events, 64 types at 20 Hz on a 1 ms tick, 200 planted
              four-node chains with delays U{3..8}, 1,024 four-node episodes
              with (2,8] delays.
  mapconcat   100,000,000 events, 128 types at 10 Hz on a 0.1 ms tick, 8
              planted five-node episodes with (1,20] delays, ~10,000 planted
              occurrences each, one across each of 4,095 equal-time grid
              points, 4,096 segments.
  level2      10,000,000 events, 64 types at 20 Hz, all 64x64 ordered type
              pairs x delay bins (0,5],(5,10],(10,20],(20,40] = 16,384 two-node
              episodes.
  longchain   500,000,000 events, 256 types, bursty gaps floor(Gamma(0.5, 4)),
              4 eight-node episodes with delays (0,3],(2,11],(3,19],(5,27],
              (7,34],(8,42],(10,50], ~10,000 planted occurrences each, 65,536
              segments.

Every generator takes ``n`` so that tests can draw the same shape at a size the
oracle finishes in seconds.  Events are sorted by time; events that share a
tick are in random order (the count does not depend on that order).
"""
from __future__ import annotations

import dataclasses

import numpy as np

BASE_SEED = 20261201


@dataclasses.dataclass
class Workload:
    name: str
    times: np.ndarray        # int32[n], non-decreasing
    types: np.ndarray        # uint16[n]
    ep_types: np.ndarray     # uint16[S, N]
    t_low: np.ndarray        # int32[S, N-1]
    t_high: np.ndarray       # int32[S, N-1]
    n_segments: int          # segment count the workload is specified with (0: any)
    description: str

    @property
    def n_events(self) -> int:
        return int(self.times.shape[0])

    @property
    def n_episodes(self) -> int:
        return int(self.ep_types.shape[0])

    @property
    def n_nodes(self) -> int:
        return int(self.ep_types.shape[1])


def _sort_events(times: np.ndarray, types: np.ndarray):
    key = times.astype(np.int64) * 65536 + types.astype(np.int64)
    order = np.argsort(key, kind="stable")
    return (np.ascontiguousarray(times[order], dtype=np.int32),
            np.ascontiguousarray(types[order], dtype=np.uint16))


def _sorted_uniform_ticks(rng, count: int, t_first: int, t_last: int) -> np.ndarray:
    """``count`` sorted integer ticks, i.i.d. uniform on [t_first, t_last].

    Order statistics of uniforms via normalised exponential spacings, so no
    sort of the full array is needed.
    """
    if count <= 0:
        return np.zeros(0, dtype=np.int32)
    span = t_last - t_first + 1
    out = np.empty(count, dtype=np.int32)
    e = rng.standard_exponential(count + 1)
    total = e.sum()
    acc = 0.0
    step = 1 << 24
    for s in range(0, count, step):
        c = np.cumsum(e[s:min(s + step, count)]) + acc
        acc = c[-1]
        u = c / total
        out[s:s + step] = t_first + np.minimum((u * span).astype(np.int64), span - 1)
    return out


def _random_episodes(rng, S: int, N: int, n_types: int) -> np.ndarray:
    return rng.integers(0, n_types, size=(S, N), dtype=np.int64).astype(np.uint16)


def _merge_planted(times_bg, types_bg, pt, py, n, rng):
    """Merge planted events into a time-sorted background and trim/pad to exactly n.

    The result is sorted by time; events sharing a tick keep the background's
    random order, with planted events after them.
    """
    pt = np.asarray(pt, dtype=np.int64)
    py = np.asarray(py, dtype=np.int64)
    keep = n - pt.size
    if keep < 0:
        raise ValueError("more planted events than n")
    bg_n = times_bg.size
    if bg_n > keep:
        drop = rng.choice(bg_n, size=bg_n - keep, replace=False)
        mask = np.ones(bg_n, dtype=bool)
        mask[drop] = False
        times_bg, types_bg = times_bg[mask], types_bg[mask]
    elif bg_n < keep:
        lo, hi = int(times_bg.min()), int(times_bg.max())
        extra_t = np.sort(rng.integers(lo, hi + 1, size=keep - bg_n))
        extra_y = rng.integers(0, int(types_bg.max()) + 1, size=keep - bg_n)
        pos = np.searchsorted(times_bg, extra_t, side="right")
        times_bg = np.insert(times_bg, pos, extra_t.astype(times_bg.dtype))
        types_bg = np.insert(types_bg, pos, extra_y.astype(types_bg.dtype))
    order = np.argsort(pt, kind="stable")
    pt, py = pt[order], py[order]
    pos = np.searchsorted(times_bg, pt, side="right")
    times = np.insert(np.asarray(times_bg, dtype=np.int32), pos, pt.astype(np.int32))
    types = np.insert(np.asarray(types_bg, dtype=np.uint16), pos, py.astype(np.uint16))
    return np.ascontiguousarray(times), np.ascontiguousarray(types)


def tiny(n: int = 10_000, seed: int = BASE_SEED + 0, n_types: int = 26,
         n_planted: int = 20, S: int = 64) -> Workload:
    """Gaps U{1..4}; 20 A->B->C chains (types 0,1,2) written over the types of
    three consecutive events at disjoint positions; 64 three-node episodes,
    #0 = A->B->C, the rest random (repeats allowed); all delays (0,5]."""
    rng = np.random.default_rng(seed)
    gaps = rng.integers(1, 5, size=n)
    times = np.cumsum(gaps).astype(np.int32)
    types = rng.integers(0, n_types, size=n).astype(np.uint16)
    # disjoint planting slots at least 8 events apart
    n_slots = max(1, (n - 3) // 8)
    slots = np.sort(rng.choice(n_slots, size=min(n_planted, n_slots), replace=False)) * 8
    for i in slots:
        types[i:i + 3] = np.array([0, 1, 2], dtype=np.uint16)
    ep = _random_episodes(rng, S, 3, n_types)
    ep[0] = [0, 1, 2]
    lo = np.zeros((S, 2), dtype=np.int32)
    hi = np.full((S, 2), 5, dtype=np.int32)
    return Workload("tiny", times, types, ep, lo, hi, 0,
                    "%d events, %d types, gaps U{1..4}, %d planted A->B->C, %d x 3-node (0,5]"
                    % (n, n_types, len(slots), S))


def _poisson_background(rng, n_bg: int, n_types: int, rate_per_type: float):
    """Superposed per-type Bernoulli/Poisson spike trains on an integer tick.

    ``rate_per_type`` is the firing probability per type per tick; the number of
    ticks is chosen so that ~n_bg events fall in [1, T].
    """
    T = max(1, int(round(n_bg / (n_types * rate_per_type))))
    ticks = _sorted_uniform_ticks(rng, n_bg, 1, T)
    ticks[0] = 1
    ticks[-1] = T
    types = rng.integers(0, n_types, size=n_bg).astype(np.uint16)
    return ticks, types, T


def ptpe(n: int = 1_000_000, seed: int = BASE_SEED + 1, n_types: int = 64,
         n_planted: int = 200, S: int = 1024) -> Workload:
    """20 Hz per type on a 1 ms tick (p = 0.02 per tick); 200 non-overlapping
    planted chains of one fixed four-type episode with delays U{3..8}; 1,024
    four-node episodes (#0 = the planted one), all delays (2,8]."""
    rng = np.random.default_rng(seed)
    N = 4
    n_bg = n - N * n_planted
    t_bg, y_bg, T = _poisson_background(rng, n_bg, n_types, 0.02)
    planted_ep = rng.choice(n_types, size=N, replace=False).astype(np.uint16)
    # chain starts on a coarse grid so chains never overlap (span <= 24 ticks)
    grid = max(32, T // max(1, n_planted))
    starts = np.arange(n_planted, dtype=np.int64) * grid + 1 + rng.integers(0, grid - 30, size=n_planted)
    pt, py = [], []
    for s in starts:
        t = int(s)
        for k in range(N):
            pt.append(t)
            py.append(int(planted_ep[k]))
            t += int(rng.integers(3, 9))
    times, types = _merge_planted(t_bg, y_bg, pt, py, n, rng)
    ep = _random_episodes(rng, S, N, n_types)
    ep[0] = planted_ep
    lo = np.full((S, N - 1), 2, dtype=np.int32)
    hi = np.full((S, N - 1), 8, dtype=np.int32)
    return Workload("ptpe", times, types, ep, lo, hi, 0,
                    "%d events, %d types @20Hz/1ms, %d planted 4-chains, %d x 4-node (2,8]"
                    % (n, n_types, n_planted, S))


def _plant_across_grid(rng, ep_types, lo, hi, T, P, per_episode, pt, py):
    """Plant occurrences of each episode: one across each interior grid point
    floor(j*T/P), j=1..P-1 (as many as ``per_episode`` allows), the rest at
    uniform positions.  Delays are drawn uniformly inside each (lo, hi]."""
    S, N = ep_types.shape
    grid = (np.arange(1, P, dtype=np.int64) * T) // P
    for e in range(S):
        n_cross = min(per_episode, grid.size)
        cross_at = grid[:n_cross] if n_cross == grid.size else np.sort(
            rng.choice(grid, size=n_cross, replace=False))
        n_free = per_episode - n_cross
        free_at = rng.integers(1, T, size=n_free)
        delays = np.stack([rng.integers(lo[e, k] + 1, hi[e, k] + 1, size=per_episode)
                           for k in range(N - 1)], axis=1) if N > 1 else np.zeros((per_episode, 0), np.int64)
        offs = np.concatenate([np.zeros((per_episode, 1), np.int64), np.cumsum(delays, axis=1)], axis=1)
        first = np.empty(per_episode, dtype=np.int64)
        if n_cross:
            # split position s in 1..N-1: nodes 1..s at or before the grid point
            split = rng.integers(1, N, size=n_cross) if N > 1 else np.zeros(n_cross, np.int64)
            before = offs[np.arange(n_cross), split - 1]          # offset of node s
            gap = offs[np.arange(n_cross), split] - before        # delay s -> s+1
            back = rng.integers(0, np.maximum(gap, 1))            # node s sits `back` ticks before
            first[:n_cross] = cross_at - before - back
        first[n_cross:] = free_at
        t = first[:, None] + offs
        ok = (t[:, 0] >= 1) & (t[:, -1] <= T)
        t = t[ok]
        pt.append(t.reshape(-1))
        py.append(np.broadcast_to(ep_types[e].astype(np.int64), t.shape).reshape(-1))


def mapconcat(n: int = 100_000_000, seed: int = BASE_SEED + 2, n_types: int = 128,
              S: int = 8, N: int = 5, P: int = 4096, per_episode: int = 10_000) -> Workload:
    """10 Hz per type on a 0.1 ms tick (p = 1e-3 per tick); eight planted
    five-node episodes with delays U inside (1,20]; ~10,000 occurrences each,
    one across each interior equal-time grid point of P segments."""
    rng = np.random.default_rng(seed)
    n_planted = S * N * per_episode
    n_bg = n - n_planted
    t_bg, y_bg, T = _poisson_background(rng, n_bg, n_types, 1e-3)
    ep = np.stack([rng.choice(n_types, size=N, replace=False) for _ in range(S)]).astype(np.uint16)
    lo = np.full((S, N - 1), 1, dtype=np.int32)
    hi = np.full((S, N - 1), 20, dtype=np.int32)
    pt, py = [], []
    _plant_across_grid(rng, ep, lo, hi, T, P, per_episode, pt, py)
    times, types = _merge_planted(t_bg, y_bg, np.concatenate(pt), np.concatenate(py), n, rng)
    return Workload("mapconcat", times, types, ep, lo, hi, P,
                    "%d events, %d types @10Hz/0.1ms, %d x %d-node (1,20] planted ~%d each, P=%d"
                    % (n, n_types, S, N, per_episode, P))


LEVEL2_BINS = ((0, 5), (5, 10), (10, 20), (20, 40))


def level2(n: int = 10_000_000, seed: int = BASE_SEED + 3, n_types: int = 64) -> Workload:
    """20 Hz per type on a 1 ms tick; every ordered type pair (A->A included)
    with each delay bin (0,5],(5,10],(10,20],(20,40]: n_types^2 * 4 episodes,
    ordered by (first type, second type, bin)."""
    rng = np.random.default_rng(seed)
    times, types, T = _poisson_background(rng, n, n_types, 0.02)
    a = np.repeat(np.arange(n_types), n_types * len(LEVEL2_BINS))
    b = np.tile(np.repeat(np.arange(n_types), len(LEVEL2_BINS)), n_types)
    bins = np.tile(np.arange(len(LEVEL2_BINS)), n_types * n_types)
    ep = np.stack([a, b], axis=1).astype(np.uint16)
    lo = np.array([LEVEL2_BINS[i][0] for i in bins], dtype=np.int32)[:, None]
    hi = np.array([LEVEL2_BINS[i][1] for i in bins], dtype=np.int32)[:, None]
    return Workload("level2", times, types, ep, lo, hi, 0,
                    "%d events, %d types @20Hz/1ms, %d two-node episodes (4 delay bins)"
                    % (n, n_types, ep.shape[0]))


LONGCHAIN_INTERVALS = ((0, 3), (2, 11), (3, 19), (5, 27), (7, 34), (8, 42), (10, 50))


def longchain(n: int = 500_000_000, seed: int = BASE_SEED + 4, n_types: int = 256,
              S: int = 4, P: int = 65536, per_episode: int = 10_000) -> Workload:
    """Bursty stream: gaps floor(G), G ~ Gamma(shape 0.5, scale 4) (many ties);
    types uniform over 256; four eight-node episodes with delays
    (0,3],(2,11],(3,19],(5,27],(7,34],(8,42],(10,50]; ~10,000 planted
    occurrences each, one across each of the first interior grid points."""
    rng = np.random.default_rng(seed)
    N = len(LONGCHAIN_INTERVALS) + 1
    n_planted = S * N * per_episode
    n_bg = n - n_planted
    t_bg = np.empty(n_bg, dtype=np.int32)
    acc = 0
    step = 1 << 24
    for s in range(0, n_bg, step):
        g = np.floor(rng.gamma(0.5, 4.0, size=min(step, n_bg - s))).astype(np.int64)
        c = np.cumsum(g) + acc
        acc = int(c[-1])
        t_bg[s:s + c.size] = c + 1
    if acc + 1 >= 2 ** 31 - 1:
        raise ValueError("longchain stream overflows int32 ticks")
    T = int(t_bg[-1])
    y_bg = rng.integers(0, n_types, size=n_bg).astype(np.uint16)
    ep = np.stack([rng.choice(n_types, size=N, replace=False) for _ in range(S)]).astype(np.uint16)
    lo = np.tile(np.array([iv[0] for iv in LONGCHAIN_INTERVALS], dtype=np.int32), (S, 1))
    hi = np.tile(np.array([iv[1] for iv in LONGCHAIN_INTERVALS], dtype=np.int32), (S, 1))
    pt, py = [], []
    _plant_across_grid(rng, ep, lo, hi, T, P, per_episode, pt, py)
    times, types = _merge_planted(t_bg, y_bg, np.concatenate(pt), np.concatenate(py), n, rng)
    return Workload("longchain", times, types, ep, lo, hi, P,
                    "%d events, %d types, Gamma(0.5,4) gaps, %d x %d-node, ~%d planted each, P=%d"
                    % (n, n_types, S, N, per_episode, P))


@dataclasses.dataclass
class MiningWorkload:
    name: str
    times: np.ndarray        # int32[n], non-decreasing
    types: np.ndarray        # uint16[n]
    alphabet: np.ndarray     # uint16[], the types mined over
    bins: list               # [(lo, hi)] delay intervals candidates may use
    max_nodes: int
    threshold: int
    description: str

    @property
    def n_events(self) -> int:
        return int(self.times.shape[0])


SYM26_SHORT = [0, 1, 2, 3]
SYM26_LONG = [10, 11, 12, 13, 14, 15, 16, 17]


def sym26(seconds: float = 60.0, seed: int = BASE_SEED + 6, rate_hz: float = 34.0,
          link_p: float = 0.9, threshold: int = 300) -> MiningWorkload:
    """The shape of the page's Sym26 model data: 26 neurons firing as Poisson
    processes at 20 Hz on a 1 ms tick, with one short (4-node) and one long
    (8-node) causal chain embedded.  Each chain starts as a Poisson process at
    ``rate_hz``; each link fires with probability ``link_p`` after U{2..6} ms.
    Mined over all 26 types with delay bins (0,5], (5,10], (10,20] up to 8
    nodes; about 50,000 events in 60 s."""
    rng = np.random.default_rng(seed)
    n_types = 26
    T = int(round(seconds * 1000))
    n_bg = int(rng.binomial(n_types * T, 0.02))
    t_bg = np.sort(rng.integers(1, T + 1, size=n_bg)).astype(np.int64)
    y_bg = rng.integers(0, n_types, size=n_bg).astype(np.uint16)
    pt, py = [t_bg], [y_bg]
    for chain in (SYM26_SHORT, SYM26_LONG):
        n_start = int(rng.poisson(rate_hz * seconds))
        starts = rng.integers(1, T + 1, size=n_start)
        for s0 in starts:
            t = int(s0)
            ts, ys = [t], [chain[0]]
            for node in chain[1:]:
                if rng.random() >= link_p:
                    break
                t += int(rng.integers(2, 7))
                ts.append(t)
                ys.append(node)
            pt.append(np.array(ts, np.int64))
            py.append(np.array(ys, np.uint16))
    times = np.concatenate(pt)
    types = np.concatenate(py)
    key = rng.random(times.size)
    o = np.lexsort((key, times))
    times = times[o].astype(np.int32)
    types = types[o]
    bins = [(0, 5), (5, 10), (10, 20)]
    return MiningWorkload("sym26", times, types, np.arange(n_types, dtype=np.uint16), bins, 8,
                          threshold, "%d events over %.0f s, 26 types @20Hz/1ms, a 4-node and an "
                          "8-node chain at %.0f Hz (links p=%.1f, U{2..6} ms), bins %s, threshold %d"
                          % (times.size, seconds, rate_hz, link_p, bins, threshold))


MINING = {"sym26": sym26}


def make_mining(name: str, **overrides) -> MiningWorkload:
    return MINING[name](**overrides)


CONFIGS = {
    "tiny": tiny,
    "ptpe": ptpe,
    "mapconcat": mapconcat,
    "level2": level2,
    "longchain": longchain,
}

# Sizes at which the CPU oracle finishes in seconds while keeping each shape.
SMALL = {
    "tiny": dict(),
    "ptpe": dict(n=200_000, S=256),
    "mapconcat": dict(n=2_000_000, P=256, per_episode=600),
    "level2": dict(n=200_000),
    "longchain": dict(n=2_000_000, P=1024, per_episode=1500),
}


def make(name: str, **overrides) -> Workload:
    return CONFIGS[name](**overrides)


def make_small(name: str, **overrides) -> Workload:
    kw = dict(SMALL[name])
    kw.update(overrides)
    return CONFIGS[name](**kw)


def random_stream(rng, n: int, n_types: int, max_gap: int = 2):
    """Small random stream with many equal-time ties (gaps U{0..max_gap})."""
    gaps = rng.integers(0, max_gap + 1, size=n)
    times = np.cumsum(gaps).astype(np.int32)
    types = rng.integers(0, n_types, size=n).astype(np.uint16)
    return times, types


def random_episodes(rng, S: int, N: int, n_types: int, max_hi: int = 6, lo_max: int | None = None):
    """S random N-node episodes (types may repeat) with random 0 <= lo < hi <= max_hi."""
    ep = rng.integers(0, n_types, size=(S, N)).astype(np.uint16)
    m = max(N - 1, 0)
    hi = rng.integers(1, max_hi + 1, size=(S, m)).astype(np.int32)
    lo_cap = hi if lo_max is None else np.minimum(hi, lo_max + 1)
    lo = (rng.random(size=(S, m)) * lo_cap).astype(np.int32)
    lo = np.minimum(lo, hi - 1)
    return ep, lo, hi
