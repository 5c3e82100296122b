"""CPU-side checks of the C ABI: the library loads, exports every function
include/epcount.h declares, and rejects bad arguments on the host before
anything touches a GPU.  Also the planner (hybrid rule of the page "Towards
Chip-on-Chip Neuroscience: Fast Mining of Frequent Episodes Using Graphics
Processors": PTPE when the episodes fill the GPU, else MapConcatenate) on
described devices, and the documented equal-time cut rule."""
import ctypes
import os
import re

import numpy as np
import pytest

import frequent_episode_mining_amd as fem

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "epcount.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|int32_t|int64_t|void|const char\*)\s+(ep_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    lib = fem.load_library()
    names = declared_functions()
    assert {"ep_count_episodes", "ep_count_episodes_ex", "ep_plan", "ep_segment_cut",
            "ep_status_string"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    for code in fem.STATUS:
        assert fem.status_string(code)
    assert fem.status_string(12345) == "unknown status"


def _call(n_events=10, S=1, N=2, lo=(0,), hi=(5,), times=1, types=1, out=1, opt=None):
    lib = fem.load_library()
    ep_t = np.zeros(max(S, 1) * N, np.uint16)
    lo_a = np.array(list(lo) * max(S, 1), np.int32)
    hi_a = np.array(list(hi) * max(S, 1), np.int32)
    eps = fem.EpEpisodes(N, ep_t.ctypes.data, lo_a.ctypes.data if lo_a.size else None,
                         hi_a.ctypes.data if hi_a.size else None)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every case here fails on the host
    return lib.ep_count_episodes_ex(fake if times else None, fake if types else None, n_events, eps,
                                    S, fake if out else None, None, opt)


def test_host_argument_errors():
    assert _call(n_events=-1) == -1
    assert _call(S=-1) == -1
    assert _call(n_events=2 ** 31) == -1
    assert _call(out=0) == -1
    assert _call(times=0) == -1
    assert _call(N=0, lo=(), hi=()) == -2
    assert _call(N=17, lo=(0,) * 16, hi=(5,) * 16) == -2
    assert _call(lo=(5,), hi=(5,)) == -3
    assert _call(lo=(-1,), hi=(5,)) == -3
    assert _call(N=3, lo=(0, 0), hi=(2 ** 31 - 1, 2)) == -3
    bad_mode = fem.EpOptions(7, 0, 0, 0, None)
    assert _call(opt=ctypes.byref(bad_mode)) == -1
    bad_p = fem.EpOptions(2, -4, 0, 0, None)
    assert _call(opt=ctypes.byref(bad_p)) == -1
    # no episodes: a no-op that needs no device at all
    assert _call(S=0, out=0) == 0


def _call_two_pass(n_events=10, S=1, N=2, lo=(0,), hi=(5,), out=1, upper=1, opt=None):
    lib = fem.load_library()
    ep_t = np.zeros(max(S, 1) * N, np.uint16)
    lo_a = np.array(list(lo) * max(S, 1), np.int32)
    hi_a = np.array(list(hi) * max(S, 1), np.int32)
    eps = fem.EpEpisodes(N, ep_t.ctypes.data, lo_a.ctypes.data if lo_a.size else None,
                         hi_a.ctypes.data if hi_a.size else None)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every case here fails on the host
    kept = ctypes.c_int64(-5)
    st = lib.ep_count_two_pass(fake, fake, n_events, eps, S, 1, fake if out else None,
                               fake if upper else None, ctypes.byref(kept), None, opt)
    return st, kept.value


def test_upper_only_host_checks():
    # the relaxed count reads no lower bounds: a NULL t_low is accepted up to the
    # device work, so only host-side failures are exercised here
    relaxed = fem.EpOptions(0, 0, 0, 1, None)
    assert _call(lo=(0,), hi=(0,), opt=ctypes.byref(relaxed)) == -3  # t_high must be > 0
    assert _call(lo=(0,), hi=(-4,), opt=ctypes.byref(relaxed)) == -3
    assert _call(n_events=-1, opt=ctypes.byref(relaxed)) == -1
    assert _call(S=0, out=0, opt=ctypes.byref(relaxed)) == 0


def test_two_pass_host_errors():
    assert _call_two_pass(n_events=-1) == (-1, 0)
    assert _call_two_pass(S=-1) == (-1, 0)
    assert _call_two_pass(N=0, lo=(), hi=()) == (-2, 0)
    assert _call_two_pass(out=0) == (-1, 0)
    assert _call_two_pass(upper=0) == (-1, 0)
    # the full table is checked before the first pass, lower bounds included
    assert _call_two_pass(lo=(5,), hi=(5,)) == (-3, 0)
    assert _call_two_pass(lo=(-1,), hi=(5,)) == (-3, 0)
    relaxed = fem.EpOptions(0, 0, 0, 1, None)
    assert _call_two_pass(opt=ctypes.byref(relaxed)) == (-1, 0)
    assert _call_two_pass(S=0, out=0, upper=0) == (0, 0)


def _mine_call(max_nodes=2, threshold=1, bins=((0, 5),), n_events=10, alphabet=(1, 2), out=True,
               mode=0):
    lib = fem.load_library()
    lo = np.array([b[0] for b in bins], np.int32)
    hi = np.array([b[1] for b in bins], np.int32)
    al = np.array(alphabet, np.uint16)
    opt = fem.EpMineOptions(len(bins), lo.ctypes.data if lo.size else None,
                            hi.ctypes.data if hi.size else None, max_nodes, threshold, 0, mode, 0)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every case here fails on the host
    handle = ctypes.c_void_p(0x77)
    st = lib.ep_mine(fake, fake, n_events, al.ctypes.data if al.size else None, al.size,
                     ctypes.byref(opt), None, ctypes.byref(handle) if out else None)
    return st, handle.value


def test_mine_host_errors():
    assert _mine_call(out=False)[0] == -1
    assert _mine_call(max_nodes=0) == (-2, None)
    assert _mine_call(max_nodes=17) == (-2, None)
    assert _mine_call(threshold=0) == (-1, None)
    assert _mine_call(n_events=-1) == (-1, None)
    assert _mine_call(mode=5) == (-1, None)
    assert _mine_call(bins=()) == (-1, None)
    assert _mine_call(bins=((3, 3),)) == (-3, None)
    assert _mine_call(bins=((-1, 3),)) == (-3, None)
    assert _mine_call(bins=((0, 3), (0, 3))) == (-1, None)
    lib = fem.load_library()
    # accessors on no result
    assert lib.ep_mined_max_nodes(None) == 0
    assert lib.ep_mined_count(None, 1) == 0
    assert lib.ep_mined_candidates(None, 1) == 0
    assert lib.ep_mined_get(None, 1, None, None, None, None) == -1
    lib.ep_mined_free(None)


def test_stream_host_errors():
    lib = fem.load_library()
    ep_t = np.zeros(2, np.uint16)
    lo = np.array([0], np.int32)
    hi = np.array([5], np.int32)
    bad = np.array([5], np.int32)
    h = ctypes.c_void_p(0x55)
    ok_eps = fem.EpEpisodes(2, ep_t.ctypes.data, lo.ctypes.data, hi.ctypes.data)
    assert lib.ep_stream_create(ok_eps, 1, None, None, None) == -1
    assert lib.ep_stream_create(ok_eps, -1, None, None, ctypes.byref(h)) == -1 and h.value is None
    assert lib.ep_stream_create(fem.EpEpisodes(0, ep_t.ctypes.data, None, None), 1, None, None,
                                ctypes.byref(h)) == -2
    assert lib.ep_stream_create(fem.EpEpisodes(2, None, lo.ctypes.data, hi.ctypes.data), 1, None, None,
                                ctypes.byref(h)) == -1
    assert lib.ep_stream_create(fem.EpEpisodes(2, ep_t.ctypes.data, bad.ctypes.data, hi.ctypes.data), 1,
                                None, None, ctypes.byref(h)) == -3
    bad_mode = fem.EpOptions(9, 0, 0, 0, None)
    assert lib.ep_stream_create(ok_eps, 1, ctypes.byref(bad_mode), None, ctypes.byref(h)) == -1
    # a relaxed table needs no lower bounds
    relaxed = fem.EpOptions(0, 0, 0, 1, None)
    zero_hi = np.array([0], np.int32)
    assert lib.ep_stream_create(fem.EpEpisodes(2, ep_t.ctypes.data, None, zero_hi.ctypes.data), 1,
                                ctypes.byref(relaxed), None, ctypes.byref(h)) == -3
    assert lib.ep_stream_push(None, None, None, 0, None) == -1
    assert lib.ep_stream_counts(None, None, None) == -1
    assert lib.ep_stream_events(None) == 0
    lib.ep_stream_destroy(None)


def test_planner_rule():
    # episodes alone fill 256 CUs x 2048 lanes six times over -> PTPE; the
    # measured crossover lies above one lane per episode
    assert fem.plan(6 * 256 * 2048, 4, 10 ** 7, cu_count=256, lanes_per_cu=2048) == ("ptpe", 1)
    assert fem.plan(6 * 256 * 2048 - 1, 4, 10 ** 7, cu_count=256, lanes_per_cu=2048)[0] == "mapconcat"
    assert fem.plan(600_000, 4, 10 ** 7, cu_count=256, lanes_per_cu=2048)[0] == "mapconcat"
    # 1,024 four-node episodes: MapConcatenate; a lane carries the N machines of
    # one (segment, episode), so P is the smallest 2^q with S * P filling the device
    mode, P = fem.plan(1024, 4, 10 ** 6, cu_count=256, lanes_per_cu=2048)
    assert mode == "mapconcat" and P == 512 and 1024 * P >= 256 * 2048 > 1024 * P // 2
    # few episodes, long stream
    assert fem.plan(8, 5, 10 ** 8, cu_count=256, lanes_per_cu=2048) == ("mapconcat", 65536)
    # many episodes, long stream: segments are kept to <= 32,768 events
    assert fem.plan(16384, 2, 10 ** 7, cu_count=256, lanes_per_cu=2048) == ("mapconcat", 512)
    # beyond 8 nodes a lane carries one machine: S * N * P lanes
    assert fem.plan(100, 12, 10 ** 7, cu_count=256, lanes_per_cu=2048) == ("mapconcat", 512)
    # the segment count is capped so a segment keeps >= 256 events on average,
    # >= 64 when there are fewer than 256 episodes
    assert fem.plan(1, 2, 10_000, cu_count=256, lanes_per_cu=2048) == ("mapconcat", 128)
    assert fem.plan(300, 2, 10_000, cu_count=256, lanes_per_cu=2048) == ("mapconcat", 32)
    # forced choices pass through
    assert fem.plan(8, 5, 10 ** 8, mode="mapconcat", n_segments=4096) == ("mapconcat", 4096)
    assert fem.plan(8, 5, 10 ** 8, mode="ptpe") == ("ptpe", 1)
    # a smaller device needs fewer segments
    m1, p1 = fem.plan(64, 3, 10 ** 7, cu_count=8, lanes_per_cu=1024)
    m2, p2 = fem.plan(64, 3, 10 ** 7, cu_count=256, lanes_per_cu=1024)
    assert m1 == m2 == "mapconcat" and p1 < p2


def test_segment_cut_rule():
    # cut p of [t_min, t_max] into P equal-time segments
    assert fem.segment_cut(1, 100, 4, 0) == 0
    assert fem.segment_cut(1, 100, 4, 4) == 100
    assert [fem.segment_cut(90, 111, 2, p) for p in range(3)] == [89, 100, 111]
    cuts = [fem.segment_cut(-2 ** 31, 2 ** 31 - 1, 1024, p) for p in range(1025)]
    assert cuts[0] == -2 ** 31 - 1 and cuts[-1] == 2 ** 31 - 1
    assert all(b >= a for a, b in zip(cuts, cuts[1:]))


def test_struct_layouts_match_header(tmp_path):
    # the binding's ctypes mirrors of the option and statistics structs have
    # the sizes and field offsets the C compiler gives the header's structs
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "epcount.h"\n'
        'int main(void) { printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(ep_options), sizeof(ep_stats),'
        ' offsetof(ep_options, plan), offsetof(ep_stats, groups), sizeof(ep_episodes),'
        ' sizeof(ep_mine_options)); return 0; }\n')
    exe = tmp_path / "layout"
    inc = os.path.dirname(HEADER)
    import subprocess
    subprocess.check_call(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", inc, "-I", "/opt/rocm/include", str(src),
                           "-o", str(exe)])
    got = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    want = [ctypes.sizeof(fem.EpOptions), ctypes.sizeof(fem.EpStats), fem.EpOptions.plan.offset,
            fem.EpStats.groups.offset, ctypes.sizeof(fem.EpEpisodes), ctypes.sizeof(fem.EpMineOptions)]
    assert got == want


def test_plan_switch_names():
    # every EP_PLAN_* flag of the header has a name in the binding, with its value
    text = open(HEADER).read()
    flags = dict((m.group(1), int(m.group(2))) for m in re.finditer(r"EP_PLAN_(\w+)\s*=\s*1 << (\d+)", text))
    assert len(flags) == len(fem.PLAN)
    for name, bit in flags.items():
        assert fem.PLAN[name.lower().replace("_", "-")] == 1 << bit
    assert fem.plan_bits(["ring-windows", "recount"]) == fem.PLAN["ring-windows"] | fem.PLAN["recount"]
