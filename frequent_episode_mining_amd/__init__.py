"""MI355X-native serial-episode counting: Python binding of libepcount.so.

Argument marshalling only: every step of the counting runs in the library's
HIP kernels.  PyTorch provides device memory and the stream.  The library is
loaded from this package directory; if it is missing, every call raises.

Page: "Towards Chip-on-Chip Neuroscience: Fast Mining of Frequent Episodes
Using Graphics Processors" -- counting the non-overlapped occurrences of serial
episodes E(1) -(t_low,t_high]-> ... -> E(N) in a time-sorted event stream,
with the thread-per-episode (PTPE) and MapConcatenate schemes.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libepcount.so")

EP_OK = 0
STATUS = {
    0: "EP_OK", -1: "EP_ERR_ARG", -2: "EP_ERR_NODES", -3: "EP_ERR_INTERVAL",
    -4: "EP_ERR_UNSORTED", -5: "EP_ERR_WORKSPACE", -6: "EP_ERR_HIP", -7: "EP_ERR_UNSUPPORTED",
    -8: "EP_ERR_SCRATCH_LIMIT",
}
NOALLOC_SCRATCH_BYTES = 64 << 20
MODES = {"auto": 0, "ptpe": 1, "mapconcat": 2}
MODE_NAMES = {v: k for k, v in MODES.items()}
MAX_NODES = 16


class EpEpisodes(ctypes.Structure):
    _fields_ = [("n_nodes", ctypes.c_int32), ("types", ctypes.c_void_p),
                ("t_low", ctypes.c_void_p), ("t_high", ctypes.c_void_p)]


class EpStats(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("n_segments", ctypes.c_int32),
                ("max_runs", ctypes.c_int32), ("kernels", ctypes.c_int32),
                ("repairs", ctypes.c_int64), ("fallbacks", ctypes.c_int64),
                ("groups", ctypes.c_int32), ("pad", ctypes.c_int32)]


class EpOptions(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("n_segments", ctypes.c_int32),
                ("validate", ctypes.c_int32), ("upper_only", ctypes.c_int32),
                ("stats", ctypes.POINTER(EpStats)), ("plan", ctypes.c_uint32),
                ("pad", ctypes.c_int32)]


# EP_PLAN_* switches of ep_options.plan: which kernels produce the (same) counts
PLAN = {"ticks": 1 << 0, "positions": 1 << 1, "list": 1 << 2, "no-list": 1 << 3,
        "prune": 1 << 4, "no-prune": 1 << 5, "group-steps": 1 << 6, "no-group-steps": 1 << 7,
        "run-windows": 1 << 8, "ring-windows": 1 << 9, "machine-lanes": 1 << 10,
        "no-reduce": 1 << 11, "no-repair-queue": 1 << 12, "recount": 1 << 13, "no-split": 1 << 14,
        "slice": 1 << 15, "no-slice": 1 << 16, "tiny-repair-queue": 1 << 17}


def plan_bits(plan) -> int:
    """EP_PLAN_* bits from an int or an iterable of PLAN names."""
    if plan is None:
        return 0
    if isinstance(plan, int):
        return plan
    if isinstance(plan, str):
        plan = [plan]
    bits = 0
    for name in plan:
        bits |= PLAN[name]
    return bits


class EpMineOptions(ctypes.Structure):
    _fields_ = [("n_bins", ctypes.c_int32), ("bin_lo", ctypes.c_void_p), ("bin_hi", ctypes.c_void_p),
                ("max_nodes", ctypes.c_int32), ("threshold", ctypes.c_int64),
                ("two_pass", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("max_candidates", ctypes.c_int64)]


class EpProfile(ctypes.Structure):
    _fields_ = [("map_ms", ctypes.c_double), ("closure_ms", ctypes.c_double),
                ("concat_ms", ctypes.c_double), ("other_ms", ctypes.c_double),
                ("calls", ctypes.c_int64), ("map_ticks_ms", ctypes.c_double),
                ("map_positions_ms", ctypes.c_double), ("map_filter_ms", ctypes.c_double),
                ("map_prune_ms", ctypes.c_double)]


class EpError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s (%d): %s" % (STATUS.get(status, "?"), status, msg))
        self.status = status


_lib = None


def load_library(path: str | None = None):
    """Load libepcount.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libepcount.so is not built (%s); run __graft_entry__.build()" % p)
    lib = ctypes.CDLL(p)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.ep_count_episodes.restype = ctypes.c_int
    lib.ep_count_episodes.argtypes = [vp, vp, i64, EpEpisodes, i64, vp, vp]
    lib.ep_count_episodes_ex.restype = ctypes.c_int
    lib.ep_count_episodes_ex.argtypes = [vp, vp, i64, EpEpisodes, i64, vp, vp,
                                         ctypes.POINTER(EpOptions)]
    lib.ep_count_episodes_noalloc.restype = ctypes.c_int
    lib.ep_count_episodes_noalloc.argtypes = [vp, vp, i64, EpEpisodes, i64, vp, vp,
                                              ctypes.POINTER(EpOptions)]
    lib.ep_count_two_pass.restype = ctypes.c_int
    lib.ep_count_two_pass.argtypes = [vp, vp, i64, EpEpisodes, i64, i64, vp, vp,
                                      ctypes.POINTER(ctypes.c_int64), vp, ctypes.POINTER(EpOptions)]
    lib.ep_mine.restype = ctypes.c_int
    lib.ep_mine.argtypes = [vp, vp, i64, vp, i32, ctypes.POINTER(EpMineOptions), vp,
                            ctypes.POINTER(ctypes.c_void_p)]
    lib.ep_mined_max_nodes.restype = i32
    lib.ep_mined_max_nodes.argtypes = [vp]
    lib.ep_mined_count.restype = i64
    lib.ep_mined_count.argtypes = [vp, i32]
    lib.ep_mined_candidates.restype = i64
    lib.ep_mined_candidates.argtypes = [vp, i32]
    lib.ep_mined_get.restype = ctypes.c_int
    lib.ep_mined_get.argtypes = [vp, i32, vp, vp, vp, vp]
    lib.ep_mined_free.restype = None
    lib.ep_mined_free.argtypes = [vp]
    lib.ep_stream_create.restype = ctypes.c_int
    lib.ep_stream_create.argtypes = [EpEpisodes, i64, ctypes.POINTER(EpOptions), vp,
                                     ctypes.POINTER(ctypes.c_void_p)]
    lib.ep_stream_push.restype = ctypes.c_int
    lib.ep_stream_push.argtypes = [vp, vp, vp, i64, vp]
    lib.ep_stream_counts.restype = ctypes.c_int
    lib.ep_stream_counts.argtypes = [vp, vp, vp]
    lib.ep_stream_events.restype = i64
    lib.ep_stream_events.argtypes = [vp]
    lib.ep_stream_destroy.restype = None
    lib.ep_stream_destroy.argtypes = [vp]
    lib.ep_plan.restype = ctypes.c_int
    lib.ep_plan.argtypes = [i64, i32, i64, i32, i32, i32, i32,
                            ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.ep_segment_cut.restype = i64
    lib.ep_segment_cut.argtypes = [i32, i32, i32, i32]
    lib.ep_profile_begin.restype = ctypes.c_int
    lib.ep_profile_begin.argtypes = []
    lib.ep_profile_begin_kernel.restype = ctypes.c_int
    lib.ep_profile_begin_kernel.argtypes = [i32, i32]
    lib.ep_profile_end.restype = ctypes.c_int
    lib.ep_profile_end.argtypes = [ctypes.POINTER(EpProfile)]
    lib.ep_status_string.restype = ctypes.c_char_p
    lib.ep_status_string.argtypes = [ctypes.c_int]
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().ep_status_string(status).decode()


def _check(status: int):
    if status != EP_OK:
        raise EpError(status, status_string(status))


class EpisodeTable:
    """Host-side candidate episode set (uint16 types [S,N], int32 bounds [S,N-1])."""

    def __init__(self, ep_types, t_low, t_high):
        ep_types = np.ascontiguousarray(ep_types, dtype=np.uint16)
        if ep_types.ndim == 1:
            ep_types = ep_types[None, :]
        S, N = ep_types.shape
        self.types = ep_types
        self.t_low = np.ascontiguousarray(np.asarray(t_low, dtype=np.int32).reshape(S, max(N - 1, 0)))
        self.t_high = np.ascontiguousarray(np.asarray(t_high, dtype=np.int32).reshape(S, max(N - 1, 0)))

    @property
    def n_episodes(self) -> int:
        return self.types.shape[0]

    @property
    def n_nodes(self) -> int:
        return self.types.shape[1]

    def as_struct(self) -> EpEpisodes:
        return EpEpisodes(self.n_nodes, self.types.ctypes.data,
                          self.t_low.ctypes.data if self.t_low.size else None,
                          self.t_high.ctypes.data if self.t_high.size else None)


def _device_ptr(t, dtype_ok, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU torch tensor" % name)
    if t.dtype not in dtype_ok:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtype_ok))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr() if t.numel() else None


def _stream_args(times, types):
    import torch
    tp = _device_ptr(times, (torch.int32,), "times")
    yp = _device_ptr(types, (torch.int16, getattr(torch, "uint16", torch.int16)), "types")
    if types.numel() != times.numel():
        raise ValueError("times and types differ in length")
    return tp, yp, times.numel()


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _on_device(device, fn):
    import torch
    if torch.cuda.current_device() == device.index:
        return fn()
    with torch.cuda.device(device):
        return fn()


def _stats_dict(st):
    return {"mode": MODE_NAMES.get(st.mode, st.mode), "n_segments": st.n_segments,
            "max_runs": st.max_runs, "kernels": st.kernels, "repairs": st.repairs,
            "fallbacks": st.fallbacks, "groups": st.groups}


def count_episodes(times, types, ep_types, t_low=None, t_high=None, *, mode: str = "auto",
                   n_segments: int = 0, validate: bool = False, stats: bool = False,
                   upper_only: bool = False, plan=None, out=None, stream=None):
    """Counts of S episodes over one GPU-resident event stream.

    times: int32 [n] GPU tensor, non-decreasing.  types: uint16 (or int16, same
    bits) [n] GPU tensor.  ep_types: [S, N] host array (or an EpisodeTable);
    t_low/t_high: [S, N-1] host arrays.  ``upper_only`` counts the relaxed
    episodes (every lower bound taken as 0; ``t_low`` may be None).  ``plan``:
    EP_PLAN_* switches (names of ``PLAN`` or an int) choosing the kernels.
    Returns an int64 [S] GPU tensor (and the ep_stats dict if ``stats``).
    Enqueued on ``stream`` (default: torch's current stream);
    ``validate``/``stats`` synchronise that stream.
    """
    import torch
    if upper_only and t_low is None and not isinstance(ep_types, EpisodeTable):
        t_low = np.zeros_like(np.asarray(t_high, dtype=np.int32))
    table = ep_types if isinstance(ep_types, EpisodeTable) else EpisodeTable(ep_types, t_low, t_high)
    tp, yp, n = _stream_args(times, types)
    S = table.n_episodes
    if out is None:
        out = torch.empty(S, dtype=torch.int64, device=times.device)
    op = _device_ptr(out, (torch.int64,), "out") if S else None
    sp = _stream_handle(stream, times.device)
    lib = load_library()
    st = EpStats()
    opt = EpOptions(MODES[mode], int(n_segments), int(bool(validate)), int(bool(upper_only)),
                    ctypes.pointer(st) if stats else None, plan_bits(plan), 0)
    status = _on_device(times.device, lambda: lib.ep_count_episodes_ex(
        tp, yp, n, table.as_struct(), S, op, sp, ctypes.byref(opt)))
    _check(status)
    if stats:
        return out, _stats_dict(st)
    return out


def count_two_pass(times, types, ep_types, t_low=None, t_high=None, *, threshold: int,
                   mode: str = "auto", n_segments: int = 0, validate: bool = False,
                   stats: bool = False, plan=None, stream=None):
    """Two-pass elimination (A2 then A1) for a support threshold.

    Returns ``(counts, upper, n_kept)`` (plus the second pass's ep_stats dict
    if ``stats``): ``upper`` = int64 [S] GPU tensor of the relaxed counts,
    ``counts`` = int64 [S] GPU tensor with the exact count of every episode
    whose relaxed count reaches ``threshold`` and -1 for the others, ``n_kept``
    = how many were counted exactly.  Synchronises ``stream`` once between the
    passes.
    """
    import torch
    table = ep_types if isinstance(ep_types, EpisodeTable) else EpisodeTable(ep_types, t_low, t_high)
    tp, yp, n = _stream_args(times, types)
    S = table.n_episodes
    counts = torch.empty(S, dtype=torch.int64, device=times.device)
    upper = torch.empty(S, dtype=torch.int64, device=times.device)
    cp = _device_ptr(counts, (torch.int64,), "counts") if S else None
    up = _device_ptr(upper, (torch.int64,), "upper") if S else None
    sp = _stream_handle(stream, times.device)
    lib = load_library()
    st = EpStats()
    opt = EpOptions(MODES[mode], int(n_segments), int(bool(validate)), 0,
                    ctypes.pointer(st) if stats else None, plan_bits(plan), 0)
    kept = ctypes.c_int64(0)
    status = _on_device(times.device, lambda: lib.ep_count_two_pass(
        tp, yp, n, table.as_struct(), S, int(threshold), cp, up, ctypes.byref(kept), sp,
        ctypes.byref(opt)))
    _check(status)
    if stats:
        return counts, upper, kept.value, _stats_dict(st)
    return counts, upper, kept.value


def mine(times, types, alphabet, bins, *, max_nodes: int, threshold: int, two_pass: bool = False,
         mode: str = "auto", max_candidates: int = 0, stream=None, candidates: bool = False):
    """Level-wise mining of frequent episodes over a GPU-resident stream.

    ``alphabet``: event types to mine over; ``bins``: list of (lo, hi) delay
    intervals candidates may use.  Returns {k: (ep_types [S,k], t_low [S,k-1],
    t_high [S,k-1], counts [S])} (host arrays, rows in increasing order of
    (type 1, bin 1, ..., type k)), and also {k: candidates counted} if
    ``candidates``.  Synchronises ``stream`` once per episode size.
    """
    tp, yp, n = _stream_args(times, types)
    alpha = np.ascontiguousarray(np.asarray(list(alphabet), dtype=np.uint16))
    lo = np.ascontiguousarray(np.array([b[0] for b in bins], dtype=np.int32))
    hi = np.ascontiguousarray(np.array([b[1] for b in bins], dtype=np.int32))
    opt = EpMineOptions(len(bins), lo.ctypes.data if lo.size else None,
                        hi.ctypes.data if hi.size else None, int(max_nodes), int(threshold),
                        int(bool(two_pass)), MODES[mode], int(max_candidates))
    sp = _stream_handle(stream, times.device)
    lib = load_library()
    handle = ctypes.c_void_p()
    status = _on_device(times.device, lambda: lib.ep_mine(
        tp, yp, n, alpha.ctypes.data if alpha.size else None, alpha.size, ctypes.byref(opt), sp,
        ctypes.byref(handle)))
    _check(status)
    try:
        out, cands = {}, {}
        for k in range(1, lib.ep_mined_max_nodes(handle) + 1):
            S = lib.ep_mined_count(handle, k)
            cands[k] = lib.ep_mined_candidates(handle, k)
            ep = np.zeros((S, k), np.uint16)
            tl = np.zeros((S, k - 1), np.int32)
            th = np.zeros((S, k - 1), np.int32)
            cnt = np.zeros(S, np.int64)
            _check(lib.ep_mined_get(handle, k, ep.ctypes.data, tl.ctypes.data if tl.size else None,
                                    th.ctypes.data if th.size else None, cnt.ctypes.data))
            out[k] = (ep, tl, th, cnt)
    finally:
        lib.ep_mined_free(handle)
    return (out, cands) if candidates else out


class EpisodeStream:
    """Counts of a fixed episode table over a stream that arrives in batches.

    ``push(times, types)`` adds one batch (GPU tensors; its first time not
    before the previous batch's last); ``counts()`` returns the counts over
    every event pushed so far (int64 [S] GPU tensor).  Each push synchronises
    its stream.
    """

    def __init__(self, ep_types, t_low=None, t_high=None, *, mode: str = "auto", n_segments: int = 0,
                 validate: bool = False, upper_only: bool = False, plan=None, device="cuda",
                 stream=None):
        import torch
        if upper_only and t_low is None and not isinstance(ep_types, EpisodeTable):
            t_low = np.zeros_like(np.asarray(t_high, dtype=np.int32))
        self.table = ep_types if isinstance(ep_types, EpisodeTable) else EpisodeTable(ep_types, t_low, t_high)
        self.device = torch.device(device)
        if self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self._lib = load_library()
        self._handle = ctypes.c_void_p()
        opt = EpOptions(MODES[mode], int(n_segments), int(bool(validate)), int(bool(upper_only)), None,
                        plan_bits(plan), 0)
        sp = _stream_handle(stream, self.device)
        status = _on_device(self.device, lambda: self._lib.ep_stream_create(
            self.table.as_struct(), self.table.n_episodes, ctypes.byref(opt), sp, ctypes.byref(self._handle)))
        _check(status)

    def push(self, times, types, stream=None):
        tp, yp, n = _stream_args(times, types)
        sp = _stream_handle(stream, times.device)
        _check(_on_device(times.device, lambda: self._lib.ep_stream_push(self._handle, tp, yp, n, sp)))

    def counts(self, stream=None):
        import torch
        out = torch.empty(self.table.n_episodes, dtype=torch.int64, device=self.device)
        op = _device_ptr(out, (torch.int64,), "out") if out.numel() else None
        sp = _stream_handle(stream, self.device)
        _check(_on_device(self.device, lambda: self._lib.ep_stream_counts(self._handle, op, sp)))
        return out

    @property
    def events(self) -> int:
        return int(self._lib.ep_stream_events(self._handle))

    def close(self):
        if self._handle:
            self._lib.ep_stream_destroy(self._handle)
            self._handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def plan(n_episodes: int, n_nodes: int, n_events: int, *, mode: str = "auto", n_segments: int = 0,
         cu_count: int = 256, lanes_per_cu: int = 2048):
    """The planner on a described device (no GPU needed): (mode name, segments)."""
    lib = load_library()
    m = ctypes.c_int32()
    p = ctypes.c_int32()
    _check(lib.ep_plan(n_episodes, n_nodes, n_events, MODES[mode], n_segments, cu_count,
                       lanes_per_cu, ctypes.byref(m), ctypes.byref(p)))
    return MODE_NAMES[m.value], p.value


def profile_begin():
    """Start recording per-phase GPU durations (HIP events) of later calls."""
    _check(load_library().ep_profile_begin())


PROFILE_KERNELS = {"filter": 0, "ticks": 1, "positions": 2, "prune": 3}


def profile_begin_kernel(which: str, every: int = 1) -> None:
    """Time one Map kernel ('filter', 'prune', 'ticks' or 'positions') on one call in
    `every`, recording nothing else."""
    _check(load_library().ep_profile_begin_kernel(PROFILE_KERNELS[which], every))


def profile_end() -> dict:
    """Wait for the recorded events; summed per-phase milliseconds and calls."""
    p = EpProfile()
    _check(load_library().ep_profile_end(ctypes.byref(p)))
    return {"map_ms": p.map_ms, "closure_ms": p.closure_ms, "concat_ms": p.concat_ms,
            "other_ms": p.other_ms, "calls": p.calls, "map_ticks_ms": p.map_ticks_ms,
            "map_positions_ms": p.map_positions_ms, "map_filter_ms": p.map_filter_ms,
            "map_prune_ms": p.map_prune_ms}


def segment_cut(t_min: int, t_max: int, n_segments: int, p: int) -> int:
    return int(load_library().ep_segment_cut(t_min, t_max, n_segments, p))


def to_device(times: np.ndarray, types: np.ndarray, device="cuda"):
    """Copy a host stream to GPU tensors in the layout the library reads."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(times, dtype=np.int32)).to(device)
    y = torch.from_numpy(np.ascontiguousarray(types, dtype=np.uint16).view(np.int16)).to(device)
    return t, y
