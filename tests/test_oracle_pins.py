"""Pins for the CPU oracle (alpha_0), independent of the oracle itself.

Each test checks the oracle against something the page or mathematics fixes:
hand-derived fixtures (tests/golden/), brute-force enumeration on tiny streams,
a closed form (single-node episodes), and invariants of the definition
(page "Towards Chip-on-Chip Neuroscience: Fast Mining of Frequent Episodes
Using Graphics Processors": episode definition in "Design of MapConcatenate",
non-overlapped counting in the Fig. 3 text).  ``test_pins_catch_mutants``
plants plausible mistakes in a copy of the oracle's C source and checks that
these pins catch every one of them.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from bruteforce import brute_count
from golden_io import all_cases
from frequent_episode_mining_amd import workloads as W

CASES = all_cases()


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_fixtures(case):
    got = oracle.count(case["times"], case["types"], case["ep_types"], case["t_low"], case["t_high"])
    assert got[0] == case["expect"]["count"][0]
    # the brute force agrees with the hand derivation too
    assert brute_count(case["times"], case["types"], case["ep_types"], case["t_low"],
                       case["t_high"]) == case["expect"]["count"][0]
    if "upper" in case["expect"]:
        # Algorithm A2: the relaxed episode (lower bounds 0), by hand and by brute force
        got_u = oracle.count_upper(case["times"], case["types"], case["ep_types"], case["t_high"])
        assert got_u[0] == case["expect"]["upper"][0]
        assert brute_count(case["times"], case["types"], case["ep_types"],
                           np.zeros_like(case["t_low"]), case["t_high"]) == case["expect"]["upper"][0]
    if "two_pass" in case["expect"]:
        tp = case["expect"]["two_pass"]
        for theta, want in zip(tp[0::2], tp[1::2]):
            counts, upper = oracle.two_pass(case["times"], case["types"], case["ep_types"],
                                            case["t_low"], case["t_high"], theta)
            assert counts[0] == want and upper[0] == case["expect"]["upper"][0]
    if "segments" in case["expect"]:
        cut = case["cut"]
        left = case["times"] <= cut
        segs = []
        for m in (left, ~left):
            segs.append(int(oracle.count(case["times"][m], case["types"][m], case["ep_types"],
                                         case["t_low"], case["t_high"])[0]))
        assert segs == case["expect"]["segments"]


def _random_cases(seed, count):
    rng = np.random.default_rng(seed)
    for _ in range(count):
        n = int(rng.integers(0, 26))
        n_types = int(rng.integers(1, 5))
        N = int(rng.integers(1, 5))
        times, types = W.random_stream(rng, n, n_types, max_gap=int(rng.integers(0, 4)))
        ep, lo, hi = W.random_episodes(rng, 1, N, n_types, max_hi=6)
        yield times, types, ep[0], lo[0], hi[0]


def test_oracle_matches_bruteforce_on_tiny_streams():
    checked = 0
    nonzero = 0
    for times, types, ep, lo, hi in _random_cases(7, 1500):
        want = brute_count(times, types, ep, lo, hi)
        got = oracle.count(times, types, ep[None], lo[None], hi[None])[0]
        assert got == want, (times.tolist(), types.tolist(), ep.tolist(), lo.tolist(), hi.tolist())
        checked += 1
        nonzero += want > 0
    assert checked == 1500 and nonzero > 300


def test_single_node_closed_form():
    # N = 1: every event of type E(1) is an occurrence; equal times overlap, so
    # the count is the number of distinct times that carry the type.
    rng = np.random.default_rng(11)
    for _ in range(200):
        times, types = W.random_stream(rng, int(rng.integers(0, 300)), 5, max_gap=3)
        y = int(rng.integers(0, 5))
        got = oracle.count(times, types, np.array([[y]], np.uint16), np.zeros((1, 0), np.int32),
                           np.zeros((1, 0), np.int32))[0]
        assert got == np.unique(times[types == y]).size


def test_planted_chains_in_private_alphabet():
    # Chains whose types occur nowhere else, spaced more than Span apart, are
    # exactly the occurrences: the count equals the number planted, whatever
    # the background does.
    rng = np.random.default_rng(12)
    for trial in range(20):
        N = int(rng.integers(2, 7))
        lo = rng.integers(0, 4, size=N - 1).astype(np.int32)
        hi = (lo + rng.integers(1, 6, size=N - 1)).astype(np.int32)
        span = int(hi.sum())
        k = int(rng.integers(1, 40))
        starts = np.cumsum(rng.integers(span + 1, span + 30, size=k))
        pt, py = [], []
        for s in starts:
            t = int(s)
            for j in range(N):
                pt.append(t)
                py.append(100 + j)
                if j < N - 1:
                    t += int(rng.integers(lo[j] + 1, hi[j] + 1))
        bt, by = W.random_stream(rng, 3000, 20, max_gap=1)
        times = np.concatenate([bt, np.array(pt, np.int32)])
        types = np.concatenate([by, np.array(py, np.uint16)])
        o = np.argsort(times, kind="stable")
        ep = np.arange(100, 100 + N, dtype=np.uint16)[None]
        got = oracle.count(times[o], types[o], ep, lo[None], hi[None])[0]
        assert got == k


def _shuffle_within_ticks(rng, times, types):
    key = rng.random(times.size)
    o = np.lexsort((key, times))
    return times[o], types[o]


def test_invariants():
    rng = np.random.default_rng(13)
    for _ in range(60):
        times, types = W.random_stream(rng, int(rng.integers(50, 800)), 4, max_gap=2)
        ep, lo, hi = W.random_episodes(rng, 8, int(rng.integers(1, 5)), 4, max_hi=8)
        base = oracle.count(times, types, ep, lo, hi)
        # order of events inside one tick does not matter
        t2, y2 = _shuffle_within_ticks(rng, times, types)
        assert np.array_equal(oracle.count(t2, y2, ep, lo, hi), base)
        # shifting every time by a constant does not matter
        sh = int(rng.integers(-1000, 1000))
        assert np.array_equal(oracle.count(times + sh, types, ep, lo, hi), base)
        # two streams separated by more than Span: counts add
        span = int(hi.sum(axis=1).max()) if hi.size else 0
        times_b, types_b = W.random_stream(rng, int(rng.integers(0, 400)), 4, max_gap=2)
        off = (int(times[-1]) if times.size else 0) + span + 1 - (int(times_b[0]) if times_b.size else 0)
        cat_t = np.concatenate([times, times_b + off])
        cat_y = np.concatenate([types, types_b])
        assert np.array_equal(oracle.count(cat_t, cat_y, ep, lo, hi),
                              base + oracle.count(times_b, types_b, ep, lo, hi))
        # widening an interval never lowers the count (more occurrences exist)
        if lo.size:
            lo_w = np.maximum(lo - rng.integers(0, 2, size=lo.shape), 0).astype(np.int32)
            hi_w = (hi + rng.integers(0, 3, size=hi.shape)).astype(np.int32)
            assert np.all(oracle.count(times, types, ep, lo_w, hi_w) >= base)
        # a count can not exceed the events available for any node's type
        for e in range(ep.shape[0]):
            vals, mult = np.unique(ep[e], return_counts=True)
            cap = min(np.unique(times[types == v]).size // m for v, m in zip(vals, mult))
            assert base[e] <= cap


# ---- Algorithm A2 (upper bounds only) and the two-pass elimination A2+A1 ----


def test_upper_only_matches_bruteforce_on_tiny_streams():
    # the relaxed episode's count is the most disjoint occurrences with 0 < dt <= hi
    nonzero = 0
    for times, types, ep, lo, hi in _random_cases(11, 1500):
        want = brute_count(times, types, ep, np.zeros_like(lo), hi)
        got = oracle.count_upper(times, types, ep[None], hi[None])[0]
        assert got == want, (times.tolist(), types.tolist(), ep.tolist(), hi.tolist())
        nonzero += want > 0
    assert nonzero > 300


def test_upper_only_agrees_with_list_machine():
    # two machines for the same relaxed episode: the O(1) latest-entry check and
    # alpha_0's list scan run with every lower bound set to 0
    rng = np.random.default_rng(17)
    for _ in range(40):
        times, types = W.random_stream(rng, int(rng.integers(100, 3000)), 5, max_gap=3)
        ep, lo, hi = W.random_episodes(rng, 12, int(rng.integers(1, 6)), 5, max_hi=12)
        assert np.array_equal(oracle.count_upper(times, types, ep, hi),
                              oracle.count(times, types, ep, np.zeros_like(lo), hi))


def test_upper_only_bounds_the_count():
    # every occurrence of alpha is one of alpha', so count(alpha') >= count(alpha)
    rng = np.random.default_rng(19)
    strictly = 0
    for _ in range(40):
        times, types = W.random_stream(rng, int(rng.integers(100, 2000)), 4, max_gap=3)
        ep, lo, hi = W.random_episodes(rng, 12, int(rng.integers(2, 5)), 4, max_hi=10)
        up = oracle.count_upper(times, types, ep, hi)
        ex = oracle.count(times, types, ep, lo, hi)
        assert np.all(up >= ex)
        strictly += int(np.sum(up > ex))
    assert strictly > 50


def test_two_pass_keeps_exactly_the_frequent_episodes():
    # A2+A1 returns the exact count of every episode whose relaxed count reaches
    # the threshold, and drops only episodes whose exact count is below it
    rng = np.random.default_rng(23)
    for _ in range(20):
        times, types = W.random_stream(rng, int(rng.integers(200, 3000)), 4, max_gap=3)
        ep, lo, hi = W.random_episodes(rng, 24, int(rng.integers(2, 5)), 4, max_hi=10)
        exact = oracle.count(times, types, ep, lo, hi)
        theta = int(np.quantile(exact, rng.uniform(0.2, 0.9))) if exact.size else 0
        counts, upper = oracle.two_pass(times, types, ep, lo, hi, theta)
        kept = counts >= 0
        assert np.array_equal(kept, upper >= theta)
        assert np.array_equal(counts[kept], exact[kept])
        assert np.all(exact[~kept] < theta)
        assert np.array_equal(np.flatnonzero(counts >= theta), np.flatnonzero(exact >= theta))


def test_tiny_workload_planted_floor():
    # the tiny workload plants 20 A->B->C chains with gaps <= 4 inside (0,5]
    wl = W.make("tiny")
    got = oracle.count(wl.times, wl.types, wl.ep_types, wl.t_low, wl.t_high)
    assert got[0] >= 20


def test_empty_and_degenerate():
    e = np.zeros(0, np.int32)
    assert oracle.count(e, e.astype(np.uint16), np.array([[1, 2]], np.uint16),
                        np.array([[0]], np.int32), np.array([[5]], np.int32))[0] == 0
    with pytest.raises(ValueError):
        oracle.count(np.array([1], np.int32), np.array([1], np.uint16), np.array([[1, 2]], np.uint16),
                     np.array([[3]], np.int32), np.array([[3]], np.int32))


# ---- mutation check: the pins above must reject plausible mistakes ----

MUTANTS = {
    "lower_bound_inclusive": ("if (d > lo && d <= hi) return 1;", "if (d >= lo && d <= hi) return 1;"),
    "upper_bound_exclusive": ("if (d > lo && d <= hi) return 1;", "if (d > lo && d < hi) return 1;"),
    "overlap_allowed_on_tie": ("if (t <= r) continue;", "if (t < r) continue;"),
    "no_list_reset": ("for (int k = 0; k < N - 1; ++k) L[k].head = L[k].size = 0;", ";"),
    "wrong_interval_index": ("tlist_has_predecessor(&L[k - 1], t, lo[k - 1], hi[k - 1])",
                             "tlist_has_predecessor(&L[k - 1], t, lo[0], hi[0])"),
    "completion_also_extends": ("        r = t;\n        for (int k = 0; k < N - 1; ++k) L[k].head = L[k].size = 0;\n        continue;",
                                "        r = t;\n        for (int k = 0; k < N - 1; ++k) L[k].head = L[k].size = 0;"),
    "append_to_wrong_list": ("if (ok && tlist_push(&L[k], (int32_t)t) != 0)",
                             "if (ok && tlist_push(&L[k > 0 ? k - 1 : 0], (int32_t)t) != 0)"),
    "prune_too_early": ("t - (int64_t)L->v[L->head] > hi", "t - (int64_t)L->v[L->head] >= hi"),
}


MUTANTS_UPPER = {
    "upper_forgets_earlier_entry": ("? L->last : L->before;", "? L->last : TLAST_NONE;"),
    "upper_same_tick_chains": ("int64_t p = (L->last != TLAST_NONE && L->last < t) ? L->last : L->before;\n"
                               "  return p != TLAST_NONE && p < t && t - p <= hi;",
                               "int64_t p = L->last;\n  return p != TLAST_NONE && p <= t && t - p <= hi;"),
    "upper_bound_exclusive_a2": ("return p != TLAST_NONE && p < t && t - p <= hi;",
                                 "return p != TLAST_NONE && p < t && t - p < hi;"),
    "upper_no_reset": ("        count += 1;\n        r = t;\n        for (int k = 0; k < N - 1; ++k) L[k].last",
                       "        count += 1;\n        r = t;\n        if (0) for (int k = 0; k < N - 1; ++k) L[k].last"),
    "upper_keeps_first_time": ("if (L->last == TLAST_NONE || t > L->last) {", "if (L->last == TLAST_NONE) {"),
    "upper_wrong_interval_index": ("tlast_has_predecessor(&L[k - 1], t, hi[k - 1])",
                                   "tlast_has_predecessor(&L[k - 1], t, hi[0])"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "alpha0.c")).read()
    assert old in src, name
    mut = src.replace(old, new, 1)
    c = tmp_path / (name + ".c")
    so = tmp_path / (name + ".so")
    c.write_text(mut)
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-shared", "-fPIC", "-pthread", str(c), "-o", str(so)])
    lib = ctypes.CDLL(str(so))
    lib.oracle_count_one.restype = ctypes.c_int64
    lib.oracle_count_one.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int64, ctypes.c_int32] + [ctypes.c_void_p] * 3
    lib.oracle_count_one_upper.restype = ctypes.c_int64
    lib.oracle_count_one_upper.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int64, ctypes.c_int32] + [ctypes.c_void_p] * 2
    return lib


def _mutant_count(lib, times, types, ep, lo, hi):
    times = np.ascontiguousarray(times, np.int32)
    types = np.ascontiguousarray(types, np.uint16)
    ep = np.ascontiguousarray(ep, np.uint16)
    lo = np.ascontiguousarray(lo, np.int32)
    hi = np.ascontiguousarray(hi, np.int32)
    return lib.oracle_count_one(times.ctypes.data, types.ctypes.data, times.size, ep.size,
                                ep.ctypes.data, lo.ctypes.data, hi.ctypes.data)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutants(tmp_path, name):
    old, new = MUTANTS[name]
    lib = _build_mutant(tmp_path, name, old, new)
    caught = False
    for case in CASES:
        if _mutant_count(lib, case["times"], case["types"], case["ep_types"], case["t_low"],
                         case["t_high"]) != case["expect"]["count"][0]:
            caught = True
            break
    if not caught:
        for times, types, ep, lo, hi in _random_cases(7, 1500):
            if _mutant_count(lib, times, types, ep, lo, hi) != brute_count(times, types, ep, lo, hi):
                caught = True
                break
    assert caught, "mutant %s survived the pins" % name


def _mutant_count_upper(lib, times, types, ep, hi):
    times = np.ascontiguousarray(times, np.int32)
    types = np.ascontiguousarray(types, np.uint16)
    ep = np.ascontiguousarray(ep, np.uint16)
    hi = np.ascontiguousarray(hi, np.int32)
    return lib.oracle_count_one_upper(times.ctypes.data, types.ctypes.data, times.size, ep.size,
                                      ep.ctypes.data, hi.ctypes.data)


@pytest.mark.parametrize("name", sorted(MUTANTS_UPPER))
def test_pins_catch_upper_only_mutants(tmp_path, name):
    old, new = MUTANTS_UPPER[name]
    lib = _build_mutant(tmp_path, name, old, new)
    caught = False
    for case in CASES:
        if "upper" in case["expect"] and _mutant_count_upper(
                lib, case["times"], case["types"], case["ep_types"], case["t_high"]) != case["expect"]["upper"][0]:
            caught = True
            break
    if not caught:
        for times, types, ep, lo, hi in _random_cases(11, 1500):
            if _mutant_count_upper(lib, times, types, ep, hi) != brute_count(times, types, ep, np.zeros_like(lo), hi):
                caught = True
                break
    assert caught, "mutant %s survived the pins" % name
