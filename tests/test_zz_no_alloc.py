"""GPU check of ep_count_episodes_noalloc, the entry point for callers that
cannot allocate device memory: through the C ABI, its counts must equal those
of ep_count_episodes_ex with the same arguments and options, call after call
on the one scratch array (a call followed by a smaller one), and a call whose
plan needs more than the array holds is refused before anything runs."""
import ctypes

import numpy as np
import pytest

import oracle
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


def _call(fem, entry, times, types, ep, lo, hi, mode="auto", P=0, plan=None):
    """One call through the C ABI on torch's current stream; (status, counts)."""
    lib = fem.load_library()
    t, y = fem.to_device(times, types, "cuda")
    table = fem.EpisodeTable(ep, lo, hi)
    out = torch.full((table.n_episodes,), -7, dtype=torch.int64, device="cuda")
    opt = fem.EpOptions(fem.MODES[mode], P, 0, 0, None, fem.plan_bits(plan), 0)
    fn = lib.ep_count_episodes_noalloc if entry == "noalloc" else lib.ep_count_episodes_ex
    status = fn(t.data_ptr() if t.numel() else None, y.data_ptr() if y.numel() else None, t.numel(),
                table.as_struct(), table.n_episodes, out.data_ptr() if out.numel() else None,
                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), ctypes.byref(opt))
    torch.cuda.synchronize()
    return status, out.cpu().numpy()


def _same_twice(fem, first, second, label, **kw):
    """The no-alloc entry on `first` then on the smaller `second`, each against
    ep_count_episodes_ex (and the oracle)."""
    for i, case in enumerate((first, second)):
        times, types, ep, lo, hi = case
        st_a, got = _call(fem, "noalloc", times, types, ep, lo, hi, **kw)
        st_b, ref = _call(fem, "ex", times, types, ep, lo, hi, **kw)
        assert st_a == 0 and st_b == 0, (label, i, st_a, st_b)
        assert np.array_equal(got, ref), "%s call %d: %s vs %s" % (label, i, got[:8], ref[:8])
        assert np.array_equal(got, oracle.count(times, types, ep, lo, hi)), (label, i)


def _shrink(case, n, S):
    times, types, ep, lo, hi = case
    return times[:n], types[:n], ep[:S], lo[:S], hi[:S]


@pytest.mark.parametrize("name", ["tiny", "ptpe", "mapconcat", "level2", "longchain"])
@pytest.mark.parametrize("mode,P", [("auto", 0), ("ptpe", 0), ("mapconcat", 16)])
def test_noalloc_matches_ex(fem, name, mode, P):
    wl = W.make_small(name)
    big = (wl.times, wl.types, wl.ep_types, wl.t_low, wl.t_high)
    small = _shrink(big, wl.n_events // 3, max(1, wl.n_episodes // 2))
    _same_twice(fem, big, small, "%s %s P=%d" % (name, mode, P), mode=mode, P=P)


@pytest.mark.parametrize("plan", [["no-reduce"], ["positions", "list", "prune"], ["ring-windows"],
                                  ["recount"]])
def test_noalloc_plans(fem, plan):
    wl = W.make_small("ptpe")
    big = (wl.times, wl.types, wl.ep_types[:32], wl.t_low[:32], wl.t_high[:32])
    small = _shrink(big, wl.n_events // 4, 5)
    _same_twice(fem, big, small, "plan %s" % plan, mode="mapconcat", P=48, plan=plan)


def test_noalloc_mixed_window_kinds(fem):
    # one group per window kind, the groups sharing the array one after another
    rng = np.random.default_rng(79)
    gaps = rng.integers(1, 3, size=3000)
    times = np.cumsum(gaps).astype(np.int32)
    types = rng.integers(0, 3, size=times.size).astype(np.uint16)
    ep = np.array([[0, 1], [0, 1], [2, 0], [1, 1], [0, 2]], np.uint16)
    lo = np.array([[10], [0], [99], [0], [60]], np.int32)
    hi = np.array([[11], [100], [100], [7], [64]], np.int32)
    big = (times, types, ep, lo, hi)
    _same_twice(fem, big, _shrink(big, 900, 3), "mixed kinds", mode="mapconcat", P=16)


def test_noalloc_refuses_past_the_array(fem):
    # 16,384 episodes x 1,024 segments needs far more than the array: refused
    # before any work, the output untouched; a smaller call still works
    rng = np.random.default_rng(83)
    times, types = W.random_stream(rng, 5000, 8, max_gap=3)
    ep = rng.integers(0, 8, size=(16384, 2)).astype(np.uint16)
    lo = np.zeros((16384, 1), np.int32)
    hi = np.full((16384, 1), 5, np.int32)
    st, out = _call(fem, "noalloc", times, types, ep, lo, hi, mode="mapconcat", P=1024)
    assert st == -8 and (out == -7).all()
    assert fem.status_string(-8)
    st, got = _call(fem, "noalloc", times, types, ep[:100], lo[:100], hi[:100], mode="mapconcat", P=16)
    assert st == 0 and np.array_equal(got, oracle.count(times, types, ep[:100], lo[:100], hi[:100]))
