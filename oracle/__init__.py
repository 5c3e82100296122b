"""CPU oracle for serial-episode counting -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library's product path never does;
it shares no code with the HIP path.

The arithmetic lives in ``alpha0.c`` (the reference serial state machine
alpha_0 of the page "Towards Chip-on-Chip Neuroscience: Fast Mining of Frequent
Episodes Using Graphics Processors", Fig. 3 text and the opening section's
Algorithm 1, restated from its description; and the upper-bound-only machine of
Algorithm A2).  This module compiles it with gcc and marshals numpy arrays
through ctypes; :func:`two_pass` strings the two machines together in the order
of the two-pass elimination section (A2+A1).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "alpha0.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile alpha0.c into liboracle.so with plain gcc (no GPU code)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
             "-pthread", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.oracle_count_one.restype = ctypes.c_int64
        lib.oracle_count_one.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_count_batch.restype = ctypes.c_int
        lib.oracle_count_batch.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int]
        lib.oracle_count_batch_mode.restype = ctypes.c_int
        lib.oracle_count_batch_mode.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
        lib.oracle_count_one_upper.restype = ctypes.c_int64
        lib.oracle_count_one_upper.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def _prep(times, types, ep_types, t_low, t_high):
    times = np.ascontiguousarray(times, dtype=np.int32)
    types = np.ascontiguousarray(types, dtype=np.uint16)
    ep_types = np.ascontiguousarray(ep_types, dtype=np.uint16)
    if ep_types.ndim == 1:
        ep_types = ep_types[None, :]
    S, N = ep_types.shape
    t_low = np.ascontiguousarray(t_low, dtype=np.int32).reshape(S, max(N - 1, 0))
    t_high = np.ascontiguousarray(t_high, dtype=np.int32).reshape(S, max(N - 1, 0))
    if times.shape != types.shape:
        raise ValueError("times and types differ in length")
    if np.any(t_low < 0) or np.any(t_low >= t_high):
        raise ValueError("intervals must satisfy 0 <= t_low < t_high")
    if times.size > 1 and np.any(np.diff(times.astype(np.int64)) < 0):
        raise ValueError("times must be non-decreasing")
    return times, types, ep_types, t_low, t_high


def count(times, types, ep_types, t_low, t_high, n_threads: int | None = None):
    """Counts of S episodes (rows of ``ep_types``) over one stream, as int64[S].

    ``ep_types``: [S, N] event types; ``t_low``/``t_high``: [S, N-1] delay
    bounds of the half-open intervals (t_low, t_high].
    """
    times, types, ep_types, t_low, t_high = _prep(times, types, ep_types, t_low, t_high)
    S, N = ep_types.shape
    out = np.zeros(S, dtype=np.int64)
    if S == 0:
        return out
    if n_threads is None:
        n_threads = os.cpu_count() or 1
    lib = _load()
    lib.oracle_count_batch(times.ctypes.data, types.ctypes.data, times.size, N,
                           ep_types.ctypes.data, t_low.ctypes.data, t_high.ctypes.data,
                           S, out.ctypes.data, int(n_threads))
    if np.any(out < 0):
        raise MemoryError("oracle ran out of memory")
    return out


def count_upper(times, types, ep_types, t_high, n_threads: int | None = None):
    """Counts of the relaxed episodes alpha' (Algorithm A2: every lower bound 0,
    upper bounds kept), as int64[S].  ``ep_types``: [S, N]; ``t_high``: [S, N-1].
    """
    ep_types = np.ascontiguousarray(ep_types, dtype=np.uint16)
    if ep_types.ndim == 1:
        ep_types = ep_types[None, :]
    S, N = ep_types.shape
    t_high = np.ascontiguousarray(t_high, dtype=np.int32).reshape(S, max(N - 1, 0))
    t_low = np.zeros_like(t_high)
    times, types, ep_types, t_low, t_high = _prep(times, types, ep_types, t_low, t_high)
    out = np.zeros(S, dtype=np.int64)
    if S == 0:
        return out
    if n_threads is None:
        n_threads = os.cpu_count() or 1
    lib = _load()
    lib.oracle_count_batch_mode(times.ctypes.data, types.ctypes.data, times.size, N,
                                ep_types.ctypes.data, t_low.ctypes.data, t_high.ctypes.data,
                                S, out.ctypes.data, int(n_threads), 1)
    if np.any(out < 0):
        raise MemoryError("oracle ran out of memory")
    return out


def two_pass(times, types, ep_types, t_low, t_high, threshold: int,
             n_threads: int | None = None):
    """Algorithm A2+A1 (two-pass elimination section) for a support threshold.

    First pass: count every relaxed episode alpha' (:func:`count_upper`) and
    drop the episodes whose relaxed count is below ``threshold``.  Second
    pass: count the remaining episodes alpha exactly (:func:`count`).
    Returns ``(counts, upper)``: ``upper`` = the first pass's counts;
    ``counts[e]`` = count(alpha_e) for the episodes kept, -1 for the dropped
    ones.  The frequent episodes are those with ``counts >= threshold``.
    """
    ep_types = np.ascontiguousarray(ep_types, dtype=np.uint16)
    if ep_types.ndim == 1:
        ep_types = ep_types[None, :]
    S, N = ep_types.shape
    t_low = np.ascontiguousarray(t_low, dtype=np.int32).reshape(S, max(N - 1, 0))
    t_high = np.ascontiguousarray(t_high, dtype=np.int32).reshape(S, max(N - 1, 0))
    _prep(times, types, ep_types, t_low, t_high)  # validates the full table
    upper = count_upper(times, types, ep_types, t_high, n_threads)
    keep = np.flatnonzero(upper >= threshold)
    counts = np.full(S, -1, dtype=np.int64)
    if keep.size:
        counts[keep] = count(times, types, ep_types[keep], t_low[keep], t_high[keep], n_threads)
    return counts, upper


def mine(times, types, alphabet, bins, max_nodes: int, threshold: int,
         n_threads: int | None = None):
    """Level-wise mining of frequent serial episodes (the mining loop the page
    counts candidates for: episodes of one size are counted together, and the
    frequent ones of size k give the candidates of size k+1).

    ``alphabet``: event types to mine over; ``bins``: list of (lo, hi) delay
    intervals a candidate may use between consecutive nodes.  An episode is
    frequent when its count reaches ``threshold``.  Candidates:
      size 1: every alphabet type;
      size 2: every ordered pair (a, c) of frequent types, once per bin;
      size k+1: alpha joined with beta when beta without its last node equals
        alpha without its first node (types and bins): alpha's nodes followed
        by beta's last bin and type.
    A node dropped from either end of an occurrence leaves an occurrence of
    the shorter episode, and non-overlapped occurrences stay non-overlapped,
    so every sub-episode obtained that way is at least as frequent: the join
    reaches every frequent episode.

    Returns {k: (ep_types [S,k], t_low [S,k-1], t_high [S,k-1], counts [S])}
    for every k with a frequent episode, rows in increasing order of
    (type 1, bin 1, type 2, bin 2, ..., type k) with bins by their index.
    """
    bins = [(int(lo), int(hi)) for lo, hi in bins]
    out = {}
    # an episode is (types tuple, bin-index tuple)
    level = [((int(a),), ()) for a in sorted(set(int(a) for a in alphabet))]
    k = 1
    while level and k <= max_nodes:
        ep = np.array([t for t, _ in level], dtype=np.uint16).reshape(len(level), k)
        lo = np.array([[bins[b][0] for b in bs] for _, bs in level], dtype=np.int32).reshape(len(level), k - 1)
        hi = np.array([[bins[b][1] for b in bs] for _, bs in level], dtype=np.int32).reshape(len(level), k - 1)
        cnt = count(times, types, ep, lo, hi, n_threads)
        keep = cnt >= threshold
        if not keep.any():
            break
        out[k] = (ep[keep], lo[keep], hi[keep], cnt[keep])
        frequent = [level[i] for i in np.flatnonzero(keep)]
        if k == max_nodes:
            break
        nxt = []
        if k == 1:
            for (a,), _ in frequent:
                for b in range(len(bins)):
                    for (c,), _ in frequent:
                        nxt.append(((a, c), (b,)))
        else:
            by_prefix = {}
            for t, bs in frequent:
                by_prefix.setdefault((t[:-1], bs[:-1]), []).append((t, bs))
            for t, bs in frequent:
                for t2, bs2 in by_prefix.get((t[1:], bs[1:]), []):
                    nxt.append((t + (t2[-1],), bs + (bs2[-1],)))
        nxt.sort(key=lambda e: [v for pair in zip(e[0], e[1] + (-1,)) for v in pair])
        level = nxt
        k += 1
    return out


def count_timed(times, types, ep_types, t_low, t_high, n_threads: int | None = None):
    """Like :func:`count`, also returning (seconds, threads used)."""
    times, types, ep_types, t_low, t_high = _prep(times, types, ep_types, t_low, t_high)
    S, N = ep_types.shape
    out = np.zeros(S, dtype=np.int64)
    if n_threads is None:
        n_threads = os.cpu_count() or 1
    lib = _load()
    t0 = time.perf_counter()
    used = lib.oracle_count_batch(times.ctypes.data, types.ctypes.data, times.size, N,
                                  ep_types.ctypes.data, t_low.ctypes.data,
                                  t_high.ctypes.data, S, out.ctypes.data, int(n_threads))
    dt = time.perf_counter() - t0
    return out, dt, used
