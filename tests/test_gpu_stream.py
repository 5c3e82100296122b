"""GPU parity of streaming counts (ep_stream_*) against the CPU oracle.

After every pushed batch the running counts must equal the oracle's count of
the concatenation of all batches pushed so far (page "Towards Chip-on-Chip
Neuroscience: Fast Mining of Frequent Episodes Using Graphics Processors":
the (a, count, b) carry of the Concatenate section, here across calls).
Batches are cut anywhere, also inside a tick, and may be empty, single
events, or shorter than an episode's Span.
"""
import numpy as np
import pytest

import oracle
from golden_io import all_cases
from frequent_episode_mining_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fem():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import frequent_episode_mining_amd as m
    m.load_library()
    return m


def _log(msg):
    print(msg, flush=True)


def _check(got, want, label):
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0][:8]
        raise AssertionError("%s: %d mismatches, episodes %s got %s want %s" % (
            label, int((got != want).sum()), bad.tolist(), got[bad].tolist(), want[bad].tolist()))


def _run(fem, times, types, ep, lo, hi, cuts, label, mode="auto", upper_only=False, every=True, plan=None):
    """Push the stream cut at `cuts` (sorted indices) and check after each push."""
    st = fem.EpisodeStream(ep, None if upper_only else lo, hi, mode=mode, upper_only=upper_only, plan=plan)
    bounds = [0] + list(cuts) + [times.size]
    try:
        for i in range(len(bounds) - 1):
            a, b = bounds[i], bounds[i + 1]
            t, y = fem.to_device(times[a:b], types[a:b], "cuda")
            st.push(t, y)
            if every or i == len(bounds) - 2:
                got = st.counts().cpu().numpy()
                if upper_only:
                    want = oracle.count_upper(times[:b], types[:b], ep, hi)
                else:
                    want = oracle.count(times[:b], types[:b], ep, lo, hi)
                _check(got, want, "%s after batch %d (events %d..%d)" % (label, i, a, b))
        assert st.events == times.size
    finally:
        st.close()


@pytest.mark.parametrize("case", all_cases(), ids=lambda c: c["name"])
def test_stream_golden_every_split(fem, case):
    times, types = case["times"], case["types"]
    ep, lo, hi = case["ep_types"][None], case["t_low"][None], case["t_high"][None]
    for c in range(times.size + 1):
        _run(fem, times, types, ep, lo, hi, [c], "%s cut %d" % (case["name"], c))


@pytest.mark.parametrize("mode", ["auto", "mapconcat", "mapconcat-list", "mapconcat-rings"])
def test_stream_fuzz(fem, mode):
    plan = None
    if mode == "mapconcat-list":
        # few episodes through the filter and the list kernel on every segment
        plan = ["positions", "list"]
    if mode == "mapconcat-rings":
        plan = ["ring-windows"]
    mode = "auto" if mode == "auto" else "mapconcat"
    rng = np.random.default_rng(71)
    for trial in range(40):
        n = int(rng.integers(1, 1500))
        n_types = int(rng.integers(1, 5))
        N = int(rng.integers(1, 5))
        times, types = W.random_stream(rng, n, n_types, max_gap=int(rng.integers(0, 5)))
        S = int(rng.integers(1, 40))
        ep = rng.integers(0, n_types, size=(S, N)).astype(np.uint16)
        # some windows beyond 63 ticks, narrow ones too (runs in registers or rings)
        top = 12 if trial % 3 else 120
        hi = rng.integers(1, top, size=(S, N - 1)).astype(np.int32)
        lo = (hi - rng.integers(1, 12, size=hi.shape)).clip(0).astype(np.int32)
        lo = np.minimum(lo, hi - 1)
        k = int(rng.integers(1, 8))
        cuts = np.sort(rng.integers(0, n + 1, size=k))  # repeats give empty batches
        _run(fem, times, types, ep, lo, hi, cuts.tolist(), "fuzz %d %s" % (trial, mode), mode=mode, plan=plan)


def test_stream_upper_only(fem):
    rng = np.random.default_rng(73)
    for trial in range(12):
        times, types = W.random_stream(rng, int(rng.integers(10, 1200)), 4, max_gap=3)
        N = int(rng.integers(2, 5))
        ep = rng.integers(0, 4, size=(20, N)).astype(np.uint16)
        hi = rng.integers(1, 100, size=(20, N - 1)).astype(np.int32)
        cuts = np.sort(rng.integers(0, times.size + 1, size=4)).tolist()
        _run(fem, times, types, ep, None, hi, cuts, "upper %d" % trial, upper_only=True)


@pytest.mark.parametrize("batches", [2, 7, 33])
@pytest.mark.parametrize("name", ["tiny", "ptpe", "mapconcat", "level2", "longchain"])
def test_stream_configs_small(fem, name, batches):
    wl = W.make_small(name)
    rng = np.random.default_rng(batches)
    cuts = np.sort(rng.choice(np.arange(1, wl.n_events), size=batches - 1, replace=False)).tolist()
    _log("stream %s small in %d batches: n=%d S=%d" % (name, batches, wl.n_events, wl.n_episodes))
    _run(fem, wl.times, wl.types, wl.ep_types, wl.t_low, wl.t_high, cuts,
         "%s %d batches" % (name, batches), every=batches <= 7)


def test_stream_rejects_batch_before_the_last(fem):
    st = fem.EpisodeStream(np.array([[0, 1]], np.uint16), [[0]], [[5]])
    try:
        t, y = fem.to_device(np.array([3, 7, 9], np.int32), np.array([0, 1, 0], np.uint16), "cuda")
        st.push(t, y)
        t2, y2 = fem.to_device(np.array([8, 12], np.int32), np.array([1, 1], np.uint16), "cuda")
        with pytest.raises(fem.EpError) as ei:
            st.push(t2, y2)
        assert ei.value.status == -4
        # an equal time continues the last tick
        t3, y3 = fem.to_device(np.array([9, 12], np.int32), np.array([1, 1], np.uint16), "cuda")
        st.push(t3, y3)
        want = oracle.count(np.array([3, 7, 9, 9, 12], np.int32), np.array([0, 1, 0, 1, 1], np.uint16),
                            np.array([[0, 1]], np.uint16), [[0]], [[5]])
        assert st.counts().cpu().numpy().tolist() == want.tolist()
    finally:
        st.close()
