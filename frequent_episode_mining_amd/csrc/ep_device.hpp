// Device code of the serial-episode counting library (gfx950 / CDNA4).
//
// Source page: "Towards Chip-on-Chip Neuroscience: Fast Mining of Frequent
// Episodes Using Graphics Processors".
//
// The counting machine is the page's serial state machine (opening section,
// Algorithm 1; Fig. 3 text: alpha_0).  For every node j < N-1 it keeps a
// window of candidate times t' (events of type E(j) that end a valid prefix
// started after the last reset); an event of type E(j+1) at time t extends a
// prefix iff some candidate has t_low_j < t - t' <= t_high_j.  Two exact
// representations of a window are used:
//
//   bit windows  (t_high < W, W = 32 or 64): one W-bit mask per node whose bit
//                d stands for a candidate at time B - d, B being the time of
//                the last event the machine looked at.  Moving to time t
//                shifts every mask left by t - B; the test is a single AND
//                with the bits (t_low, t_high].  Exact for any t_low.
//   run windows  (any t_high): the continuation intervals (t'+t_low, t'+t_high]
//                merged into disjoint runs, each stored as its first and last
//                candidate (f, l) and covering (f+t_low, l+t_high].  At most
//                floor(t_high/(t_high-t_low+1)) + 1 runs are ever live, so a
//                capacity of K runs is exact when that bound is <= K.
//   ring windows (any t_high, any number of live runs): the same runs kept
//                in a ring of device memory owned by the machine, with the
//                oldest and the newest run in registers.  Runs leave at the
//                front (expiry) and enter at the back (new candidates), so
//                every operation touches only the two ends; the ring holds
//                min(that bound, events of the call) runs, which no window
//                can exceed (every run holds at least one event).
//
// All time differences are formed as uint32 of non-negative differences of
// int32 times, and cut arithmetic is int64, so nothing can overflow.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace epk {

constexpr int kWave = 64;
constexpr int kBlock = 256;  // largest workgroup of every kernel here
constexpr int kTile = 2048;  // events staged in LDS per chunk by the scan Map kernel
constexpr int kListBlock = 4096;  // events per block of the filter kernel (256 threads x 16)

// One (a, count, b) tuple of the Map step (Map rules 1-4, Fig. 5), with a and b
// stored as offsets from the segment's left and right cut; 0 is the sentinel
// "no completion within Span after the cut".
struct alignas(16) Tuple {
  int32_t a;
  int32_t c;
  int32_t b;
  int32_t pad;
};

// Tuples of all (episode, segment) pairs.  The first tuple of each pair sits
// in T0, episode-major ([e][p]), so that passes over consecutive segments of
// one episode read contiguous memory; further tuples (more than one distinct
// Map key, or repairs) sit in TX.
struct TupleStore {
  Tuple* T0;        // [S*P]
  Tuple* TX;        // [S*P*(slots-1)]
  int32_t* nmap;    // [S*P] tuples written by the Map step
  int32_t* nslots;  // [S*P] tuples in use (Map + repairs)
  int64_t P;
  int32_t slots;    // capacity per pair

  __device__ int64_t idx(int64_t e, int64_t p) const { return e * P + p; }
  __device__ Tuple* at(int64_t e, int64_t p, int k) const {
    const int64_t i = e * P + p;
    return k == 0 ? T0 + i : TX + i * (slots - 1) + (k - 1);
  }
};

// Device memory of the ring windows: `slots` machines, each owning N-1 rings
// of `cap` runs {first, last} (a power of two), `stride` entries apart.  A
// kernel running one machine per lane gives each lane its own slot; a kernel
// running one machine per wave (all lanes holding the same machine) gives
// the wave its slot, its lanes writing identical values to identical places.
struct RingArena {
  int2* base;
  int64_t stride;
  uint32_t cap;
  int64_t slots;
};

// The slot of the calling wave in a kernel that runs one machine per wave.
__device__ inline int64_t wave_slot() {
  return ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
}

template <int W>
struct BitsOf;
template <>
struct BitsOf<32> {
  using type = uint32_t;
};
template <>
struct BitsOf<64> {
  using type = uint64_t;
};

// Event types of an episode's nodes and its span, in registers.
template <int N>
struct EpTypes {
  uint32_t ty[N];
  int32_t span;  // t_high_1 + ... + t_high_{N-1}

  __device__ void load_types(const uint16_t* ep_types, const int32_t* ep_span, int64_t e) {
#pragma unroll
    for (int j = 0; j < N; ++j) ty[j] = ep_types[e * N + j];
    span = ep_span[e];
  }

  // Bit j set iff node j has event type y (a type may sit at several nodes).
  __device__ uint32_t level_mask(uint32_t y) const {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) m |= (uint32_t)(ty[j] == y) << j;
    return m;
  }
};

// hi_1 + ... + hi_k: machine k of a segment is reset this long before the cut
// (Map step, Fig. 4: alpha_p^k starts at tau_p - sum_{i<=k} t_high).
template <int N>
__device__ inline int64_t prefix_hi(const int32_t* ep_hi, int64_t e, int k) {
  int64_t s = 0;
#pragma unroll
  for (int j = 0; j < N - 1; ++j) s += (j < k) ? (int64_t)ep_hi[e * (N - 1) + j] : 0;
  return s;
}

// First index in [lo, hi) whose time is > v (hi if none).
__device__ inline int64_t upper_bound_time(const int32_t* times, int64_t lo, int64_t hi, int64_t v) {
  while (lo < hi) {
    const int64_t mid = lo + ((hi - lo) >> 1);
    if ((int64_t)times[mid] > v)
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

// ------------------------------------------------------------ run windows

template <int N>
struct RunParams : EpTypes<N> {
  uint32_t lo[N > 1 ? N - 1 : 1];
  uint32_t hi[N > 1 ? N - 1 : 1];
  uint32_t width[N > 1 ? N - 1 : 1];  // hi - lo: merge distance of two candidates

  __device__ void load(const uint16_t* ep_types, const int32_t* ep_lo, const int32_t* ep_hi,
                       const int32_t* ep_span, int64_t e) {
    this->load_types(ep_types, ep_span, e);
#pragma unroll
    for (int j = 0; j < N - 1; ++j) {
      lo[j] = (uint32_t)ep_lo[e * (N - 1) + j];
      hi[j] = (uint32_t)ep_hi[e * (N - 1) + j];
      width[j] = hi[j] - lo[j];
    }
  }
};

template <int K>
struct RunWindow {
  int32_t f[K];
  int32_t l[K];
  int32_t n;

  __device__ void clear() { n = 0; }

  // Drop runs that ended before t: a run is dead once t - l > hi.
  __device__ void expire(int32_t t, uint32_t hi) {
#pragma unroll
    for (int it = 0; it < K; ++it) {
      const bool dead = n > 0 && ((uint32_t)t - (uint32_t)l[0]) > hi;
      if (dead) {
#pragma unroll
        for (int i = 0; i + 1 < K; ++i) {
          f[i] = f[i + 1];
          l[i] = l[i + 1];
        }
        --n;
      }
    }
  }

  __device__ bool contains(int32_t t, uint32_t lo, uint32_t hi) {
    expire(t, hi);
    return n > 0 && ((uint32_t)t - (uint32_t)f[0]) > lo;
  }

  __device__ void insert(int32_t t, uint32_t hi, uint32_t width) {
    expire(t, hi);
    int32_t last_l = l[0];
#pragma unroll
    for (int i = 1; i < K; ++i) last_l = (i == n - 1) ? l[i] : last_l;
    const bool merge = n > 0 && ((uint32_t)t - (uint32_t)last_l) <= width;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      if (merge && i == n - 1) l[i] = t;
      if (!merge && i == n) {
        f[i] = t;
        l[i] = t;
      }
    }
    n += merge ? 0 : 1;
  }
};

template <int N, int K>
struct RunMachine {
  using Params = RunParams<N>;
  static constexpr bool kComparable = false;  // (no same_future test)
  int64_t r;  // time of the last reset (last completion, or the start)
  RunWindow<K> w[N > 1 ? N - 1 : 1];

  __device__ void attach(const RingArena&, int64_t) {}

  __device__ void reset(int64_t at) {
    r = at;
#pragma unroll
    for (int j = 0; j < N - 1; ++j) w[j].clear();
  }

  // Feed an event at time t with level mask lm.  Returns true if it completes
  // an occurrence; the machine is then reset at t.  Events at or before the
  // last reset are ignored: an occurrence must start strictly after the
  // previous counted one ends.
  __device__ bool step(int32_t t, uint32_t lm, const Params& P) {
    if ((int64_t)t <= r) return false;
    if ((lm >> (N - 1)) & 1u) {
      bool done = true;
      if constexpr (N > 1) done = w[N - 2].contains(t, P.lo[N - 2], P.hi[N - 2]);
      if (done) {
        reset(t);
        return true;
      }
    }
#pragma unroll
    for (int j = 0; j < N - 1; ++j) {
      if ((lm >> j) & 1u) {
        bool ok = true;
        if (j > 0) ok = w[j - 1].contains(t, P.lo[j - 1], P.hi[j - 1]);
        if (ok) w[j].insert(t, P.hi[j], P.width[j]);
      }
    }
    return false;
  }
};

// Run windows of any capacity: each node's runs in a ring of device memory.
// The oldest live run (the only one the extension test reads) and the newest
// (the only one a new candidate can merge into) stay in registers; a run is
// written to the ring when a newer run is started behind it, and read back
// when the runs before it have expired.  Same semantics as RunMachine.
template <int N>
struct RingMachine {
  using Params = RunParams<N>;
  static constexpr bool kComparable = false;
  static constexpr int NI = N > 1 ? N - 1 : 1;
  int64_t r;
  int2* ring;        // node j's ring at ring + j * cap
  uint32_t cap;
  uint32_t head[NI];  // ring position of the oldest live run
  uint32_t cnt[NI];   // live runs
  int32_t of[NI], ol[NI];  // the oldest live run (first, last candidate)
  int32_t nf[NI], nl[NI];  // the newest live run

  __device__ void attach(const RingArena& A, int64_t slot) {
    ring = A.base + slot * A.stride;
    cap = A.cap;
  }

  __device__ void reset(int64_t at) {
    r = at;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      cnt[j] = 0;
      head[j] = 0;
    }
  }

  // Drop node j's runs that ended before t (t - last > hi).
  __device__ __forceinline__ void expire(int j, int32_t t, uint32_t hi) {
    while (cnt[j] > 0 && ((uint32_t)t - (uint32_t)ol[j]) > hi) {
      --cnt[j];
      ++head[j];
      if (cnt[j] == 1) {
        of[j] = nf[j];
        ol[j] = nl[j];
      } else if (cnt[j] > 1) {
        const int2 v = ring[(size_t)j * cap + (head[j] & (cap - 1))];
        of[j] = v.x;
        ol[j] = v.y;
      }
    }
  }

  __device__ __forceinline__ bool contains(int j, int32_t t, uint32_t lo, uint32_t hi) {
    expire(j, t, hi);
    return cnt[j] > 0 && ((uint32_t)t - (uint32_t)of[j]) > lo;
  }

  __device__ __forceinline__ void insert(int j, int32_t t, uint32_t hi, uint32_t width) {
    expire(j, t, hi);
    if (cnt[j] > 0 && ((uint32_t)t - (uint32_t)nl[j]) <= width) {
      nl[j] = t;
      if (cnt[j] == 1) ol[j] = t;
      return;
    }
    if (cnt[j] > 0) {
      ring[(size_t)j * cap + ((head[j] + cnt[j] - 1) & (cap - 1))] = make_int2(nf[j], nl[j]);
    } else {
      of[j] = t;
      ol[j] = t;
    }
    nf[j] = t;
    nl[j] = t;
    ++cnt[j];
  }

  __device__ bool step(int32_t t, uint32_t lm, const Params& P) {
    if ((int64_t)t <= r) return false;
    if ((lm >> (N - 1)) & 1u) {
      bool done = true;
      if constexpr (N > 1) done = contains(N - 2, t, P.lo[N - 2], P.hi[N - 2]);
      if (done) {
        reset(t);
        return true;
      }
    }
#pragma unroll
    for (int j = 0; j < N - 1; ++j) {
      if ((lm >> j) & 1u) {
        bool ok = true;
        if (j > 0) ok = contains(j - 1, t, P.lo[j - 1], P.hi[j - 1]);
        if (ok) insert(j, t, P.hi[j], P.width[j]);
      }
    }
    return false;
  }
};

// ------------------------------------------------------------ bit windows

// Bits (lo, hi] of a W-bit window: candidate ages d with lo < d <= hi.
template <int W>
__device__ inline typename BitsOf<W>::type window_bits(uint32_t lo, uint32_t hi) {
  using Bits = typename BitsOf<W>::type;
  const Bits upto_hi = (~(Bits)0) >> (W - 1 - hi);          // bits 0..hi
  const Bits upto_lo = (~(Bits)0) >> (W - 1 - lo);          // bits 0..lo
  return upto_hi & ~upto_lo;
}

template <int N, int W>
struct BitParams : EpTypes<N> {
  using Bits = typename BitsOf<W>::type;
  Bits win[N > 1 ? N - 1 : 1];

  __device__ void load(const uint16_t* ep_types, const int32_t* ep_lo, const int32_t* ep_hi,
                       const int32_t* ep_span, int64_t e) {
    this->load_types(ep_types, ep_span, e);
#pragma unroll
    for (int j = 0; j < N - 1; ++j)
      win[j] = window_bits<W>((uint32_t)ep_lo[e * (N - 1) + j], (uint32_t)ep_hi[e * (N - 1) + j]);
  }
};

// Shift a window from base time B to time t (d = t - B >= 0 ticks later).
template <int W>
__device__ inline typename BitsOf<W>::type age(typename BitsOf<W>::type m, uint32_t d) {
  return d >= (uint32_t)W ? 0 : (m << d);
}

template <int N, int W>
struct BitMachine {
  using Params = BitParams<N, W>;
  using Bits = typename BitsOf<W>::type;
  static constexpr bool kComparable = true;
  int64_t r;
  int32_t B;
  Bits m[N > 1 ? N - 1 : 1];

  __device__ void attach(const RingArena&, int64_t) {}

  // Both machines of one episode, fed the same events, behave alike from here
  // on: windows on one base time with the same candidates, and either both
  // or neither reset at that time (a reset ignores later events on its tick).
  __device__ bool same_future(const BitMachine& o) const {
    bool eq = B == o.B && ((r == (int64_t)B) == (o.r == (int64_t)o.B));
#pragma unroll
    for (int j = 0; j < N - 1; ++j) eq = eq && m[j] == o.m[j];
    return eq;
  }

  __device__ void reset(int64_t at) {
    r = at;
    B = at < (int64_t)INT32_MIN ? INT32_MIN : (at > (int64_t)INT32_MAX ? INT32_MAX : (int32_t)at);
#pragma unroll
    for (int j = 0; j < N - 1; ++j) m[j] = 0;
  }

  __device__ bool step(int32_t t, uint32_t lm, const Params& P) {
    if ((int64_t)t <= r) return false;
    const uint32_t d = (uint32_t)t - (uint32_t)B;
    B = t;
#pragma unroll
    for (int j = 0; j < N - 1; ++j) m[j] = age<W>(m[j], d);
    if ((lm >> (N - 1)) & 1u) {
      bool done = true;
      if constexpr (N > 1) done = (m[N - 2] & P.win[N - 2]) != 0;
      if (done) {
        reset(t);
        return true;
      }
    }
    bool hit[N > 1 ? N - 1 : 1];
#pragma unroll
    for (int j = 0; j < N - 1; ++j) hit[j] = (m[j] & P.win[j]) != 0;
#pragma unroll
    for (int j = 0; j < N - 1; ++j)
      if (((lm >> j) & 1u) && (j == 0 || hit[j > 0 ? j - 1 : 0])) m[j] |= (Bits)1;
    return false;
  }
};

// A machine bound to one segment (tau_lo, tau_hi]: it produces the segment's
// (a, count, b) tuple.  a = first completion in (tau_lo, tau_lo + Span] (else
// 0), count = completions in (tau_lo, tau_hi], b = first completion in
// (tau_hi, tau_hi + Span] (else 0); the windows are closed on the right.
template <class Mach>
struct SegMachine {
  Mach m;
  int64_t tau_lo;
  int64_t tau_hi;
  int64_t stop;  // tau_hi + Span: nothing after it can change the tuple
  int32_t count;
  int32_t a_off;
  int32_t b_off;
  bool first_found;
  bool finished;
  int64_t last;  // the last completion in (tau_lo, tau_hi] (INT64_MIN: none)

  // give a ring-window machine its ring slot (no-op for the other machines)
  __device__ void attach(const RingArena& A, int64_t slot) { m.attach(A, slot); }

  __device__ void init(int64_t reset_at, int64_t lo_cut, int64_t hi_cut, int32_t span) {
    m.reset(reset_at);
    tau_lo = lo_cut;
    tau_hi = hi_cut;
    stop = hi_cut + span;
    count = 0;
    a_off = 0;
    b_off = 0;
    first_found = false;
    finished = false;
    last = INT64_MIN;
  }

  __device__ void feed(int32_t t, uint32_t lm, const typename Mach::Params& P) {
    if (finished || lm == 0) return;
    if ((int64_t)t > stop) {
      finished = true;
      return;
    }
    if (m.step(t, lm, P) && (int64_t)t > tau_lo) {
      if (!first_found) {
        first_found = true;
        const int64_t d = (int64_t)t - tau_lo;
        a_off = d <= (int64_t)P.span ? (int32_t)d : 0;
      }
      if ((int64_t)t <= tau_hi) {
        ++count;
        last = t;
      } else {
        b_off = (int32_t)((int64_t)t - tau_hi);
        finished = true;
      }
    }
  }
};

// ---------------------------------------------------------------- Map step

struct MapArgs {
  const int32_t* times;
  const uint16_t* types;
  const uint16_t* ep_types;  // [S*N]
  const int32_t* ep_lo;      // [S*(N-1)]
  const int32_t* ep_hi;      // [S*(N-1)]
  const int32_t* ep_span;    // [S]
  const uint8_t* ep_slot;    // [S*N] node type -> 1..U (bit kernels)
  const uint64_t* type_seen; // [1024] the call's node types as a 65,536-bit set (bit kernels)
  const uint8_t* type_rank;  // [1024] set bits of type_seen before each 64-bit word
  const int64_t* tau;        // [P+1] cuts
  const int32_t* seg_beg;    // [P] first event index with time > tau_p - maxSpan
  const int32_t* seg_end;    // [P] first event index with time > tau_{p+1} + maxSpan
  TupleStore ts;
  int64_t S;
  int32_t P;
  int32_t M;      // lanes per (segment, episode): machines spread over lanes
  int32_t G;      // episodes per workgroup
  int32_t R;      // segments per workgroup
  int32_t CH;     // events per segment per chunk
  int32_t U;      // distinct node types (bit kernels)
  int32_t n_machines;  // machines per (segment, episode): N (MapConcatenate) or 1 (PTPE)
  int64_t n_egroups;   // episode groups: workgroup b covers segment group b / n_egroups
  int64_t max_span;    // largest Span of the call
  int32_t CW;          // tick kernel: 64-tick words per segment per chunk
  int32_t split;       // 0: each segment to the kernel segment_uses_ticks picks; 1: all to
                       // the tick kernel; 2: all to the position kernel
  int32_t dil_steps;   // tick kernel: doubling steps of the widest interval of the call
  // tick kernel, optional: episode group eg covers episodes ep_perm[eg * G ..
  // eg * G + G) and runs group_k[eg] doubling steps (episodes ordered by their
  // steps, so that groups of narrow windows skip the wide ones' steps)
  const int32_t* ep_perm;
  const int32_t* group_k;
  const int2* lists;        // list kernel: per event block, each episode's entries {time, levels}
  const int32_t* list_off;  // [blocks * S] start of episode e's entries in block b's region
  const int32_t* list_cnt;  // [blocks * S] their number
  int32_t max_share;        // most episodes one node type belongs to (region = kListBlock * this)
  int64_t eg_blocks;   // tick kernel: workgroups that loop over a segment group's episode
                       // groups when its segments fit one chunk each
  RingArena ring;      // scan kernel with ring windows: slot ((p * S) + e) * M + k
  int32_t lazy;        // list kernel: the lazily aged single-class walk (unpruned lists)
};

// A workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits for every global load the thread has in flight (its release fence
// covers all memory), which would end any prefetch into registers issued
// before it; kernels whose threads share data only through LDS use this one.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inclusive prefix sum over the 64 lanes of a wave (every lane active): the
// shifts 1, 2, 4 and 8 within each row of 16 lanes, then the last lane of
// rows 0 and 2 added to rows 1 and 3, then lane 31 to rows 2 and 3.
__device__ inline uint32_t wave_incl_scan(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Node-type slot of event type y: 1 + the rank of y among the call's node
// types, 0 for a type on no node.  seen/rank are the MapArgs tables, copied to
// LDS by each workgroup (two independent LDS reads per event).
__device__ inline uint32_t type_slot(const uint64_t* seen, const uint8_t* rank, uint32_t y) {
  const uint64_t w = seen[y >> 6];
  const uint64_t bit = 1ull << (y & 63);
  return (w & bit) ? (uint32_t)rank[y >> 6] + (uint32_t)__popcll(w & (bit - 1)) + 1u : 0u;
}

__device__ inline void load_type_tables(const MapArgs& A, uint64_t* seen, uint8_t* rank) {
  for (int i = threadIdx.x; i < 1024; i += blockDim.x) {
    seen[i] = A.type_seen[i];
    rank[i] = A.type_rank[i];
  }
}

// Which Map kernel counts a segment: the tick kernel costs ~(N-1) bit
// operations per 64 ticks of the segment, the position kernel ~1 step per
// relevant event, so ticks win where events are dense in time.  Both kernels
// evaluate this on the same inputs, so each segment is counted exactly once.
__device__ inline bool segment_uses_ticks(const MapArgs& A, int64_t p, int N) {
  if (A.split != 0) return A.split == 1;
  const int64_t tick_span = A.tau[p + 1] - A.tau[p] + 2 * A.max_span;
  const int64_t events = (int64_t)A.seg_end[p] - A.seg_beg[p];
  return tick_span * (int64_t)(N > 1 ? N - 1 : 1) <= 4 * events;
}

// Scan Map kernel (run or ring windows): one lane = one machine (segment p,
// episode e, machine k).  A workgroup holds R consecutive segments x G
// episodes x M machines; it streams the R segments' event ranges through LDS
// in lockstep chunks of CH events, and every lane feeds each event of its own
// segment's chunk to its machine.
template <int N, class Mach>
__global__ __launch_bounds__(kBlock) void map_scan_kernel(MapArgs A) {
  __shared__ int32_t s_t[kTile];
  __shared__ uint16_t s_y[kTile];
  __shared__ int32_t s_beg[kBlock];
  __shared__ int32_t s_len[kBlock];
  __shared__ int32_t s_chunks;

  const int tid = threadIdx.x;
  const int per_seg = A.G * A.M;
  const int r_idx = tid / per_seg;
  const int g = (tid / A.M) % A.G;
  const int k = tid % A.M;
  const int64_t seg_group = (int64_t)blockIdx.x / A.n_egroups;
  const int64_t ep_group = (int64_t)blockIdx.x - seg_group * A.n_egroups;
  const int64_t p = seg_group * A.R + r_idx;
  const int64_t e = ep_group * A.G + g;
  const bool active = tid < A.R * per_seg && p < A.P && e < A.S;

  if (tid == 0) s_chunks = 0;
  __syncthreads();
  if (tid < A.R) {
    const int64_t pp = seg_group * A.R + tid;
    int32_t b = 0, len = 0;
    if (pp < A.P) {
      b = A.seg_beg[pp];
      len = A.seg_end[pp] - b;
    }
    s_beg[tid] = b;
    s_len[tid] = len;
    atomicMax(&s_chunks, (len + A.CH - 1) / A.CH);
  }

  typename Mach::Params prm;
  SegMachine<Mach> sm;
  if (active) {
    sm.attach(A.ring, (p * A.S + e) * A.M + k);
    prm.load(A.ep_types, A.ep_lo, A.ep_hi, A.ep_span, e);
    const int64_t lo_cut = A.tau[p];
    const int64_t hi_cut = A.tau[p + 1];
    sm.init(lo_cut - prefix_hi<N>(A.ep_hi, e, k), lo_cut, hi_cut, prm.span);
  }
  __syncthreads();
  const int n_chunks = s_chunks;

  for (int c = 0; c < n_chunks; ++c) {
    if (c > 0) __syncthreads();  // previous chunk fully consumed
    for (int r = 0; r < A.R; ++r) {
      const int32_t base = s_beg[r] + c * A.CH;
      const int32_t avail = s_len[r] - c * A.CH;
      for (int i = tid; i < A.CH; i += blockDim.x) {
        if (i < avail) {
          s_t[r * A.CH + i] = A.times[base + i];
          s_y[r * A.CH + i] = A.types[base + i];
        }
      }
    }
    __syncthreads();
    if (active && !sm.finished) {
      int32_t len = s_len[r_idx] - c * A.CH;
      len = len < A.CH ? len : A.CH;
      const int off = r_idx * A.CH;
      for (int i = 0; i < len; ++i) sm.feed(s_t[off + i], prm.level_mask(s_y[off + i]), prm);
    }
  }

  if (active) {
    Tuple tu;
    tu.a = sm.a_off;
    tu.c = sm.count;
    tu.b = sm.b_off;
    tu.pad = 0;
    *A.ts.at(e, p, k) = tu;
    if (k == 0) {
      A.ts.nmap[A.ts.idx(e, p)] = A.M;
      A.ts.nslots[A.ts.idx(e, p)] = A.M;
    }
  }
}

// The distinct tuples of the M machines of a (segment, episode): equal keys
// (a) mean identical tuples (the same first completion after the cut, or none
// within Span), so one of each is kept; machine 0's tuple stays first.
template <int M>
__device__ inline void write_class_tuples(const MapArgs& A, int64_t e, int64_t p, const int32_t* a_off,
                                          const int32_t* cnt, const int32_t* b_off) {
  int d = 0;
#pragma unroll
  for (int c = 0; c < M; ++c) {
    bool dup = false;
#pragma unroll
    for (int c2 = 0; c2 < c; ++c2) dup |= a_off[c2] == a_off[c];
    if (!dup) {
      Tuple tu;
      tu.a = a_off[c];
      tu.c = cnt[c];
      tu.b = b_off[c];
      tu.pad = 0;
      *A.ts.at(e, p, d) = tu;
      ++d;
    }
  }
  const int64_t pe = A.ts.idx(e, p);
  A.ts.nmap[pe] = d;
  A.ts.nslots[pe] = d;
}

// The Map machines of one (segment, episode) held by one lane (MCH = N) as
// equivalence classes, or one Map machine per lane (MCH = 1), on bit windows.
// Machines that reset at the same time are identical from then on, and so
// are machines whose last reset lies more than Span before the current event
// (every occurrence that can still complete starts after both resets), so the
// lane advances one window state per class; after the boundary halo a lane
// usually carries a single class.  Events are fed in time order as (t, lm),
// lm = the node levels whose type the event has.
template <int N, int W, int MCH>
struct ClassLane {
  using Bits = typename BitsOf<W>::type;
  static constexpr int NI = N > 1 ? N - 1 : 1;
  static constexpr uint32_t kAll = (MCH == 32) ? 0xffffffffu : ((1u << MCH) - 1u);
  uint32_t slot[N];
  Bits win[NI];
  int32_t span;
  Bits m[MCH][NI];
  int64_t r[MCH];
  uint32_t mem[MCH];  // machines in class c (bit k); a class lives while mem != 0
  int32_t cnt[MCH], a_off[MCH], b_off[MCH];
  uint32_t found, fin;
  int64_t tau_lo, tau_hi, stop, check_at;
  int32_t B;
  bool single;  // exactly one class left, held in slot 0
  // the lazily aged single class (step_lazy_if): window 0 anchored at B0, the
  // later windows at B; hiw[j] = interval j's upper bound; dl0 / dlr = a tick
  // after which no candidate of window 0 / of any later window lies within
  // its interval's upper bound any more (INT32_MIN: no candidate)
  int32_t B0, dl0, dlr;
  int32_t hiw[NI];

  __device__ void init(const MapArgs& A, int64_t e, int64_t p, int k_lane, bool active) {
    found = 0;
    fin = 0;
    span = 0;
    tau_lo = tau_hi = stop = 0;
    check_at = INT64_MAX;
    B = INT32_MIN;
    B0 = INT32_MIN;
    dl0 = dlr = INT32_MIN;
#pragma unroll
    for (int j = 0; j < NI; ++j) hiw[j] = 0;
    single = MCH == 1;
    if (!active) {
      fin = kAll;
      return;
    }
#pragma unroll
    for (int j = 0; j < N; ++j) slot[j] = A.ep_slot[e * N + j];
#pragma unroll
    for (int j = 0; j < N - 1; ++j)
      win[j] = window_bits<W>((uint32_t)A.ep_lo[e * (N - 1) + j], (uint32_t)A.ep_hi[e * (N - 1) + j]);
    span = A.ep_span[e];
    tau_lo = A.tau[p];
    tau_hi = A.tau[p + 1];
    stop = tau_hi + span;
#pragma unroll
    for (int c = 0; c < MCH; ++c) {
      const int k = (MCH == 1) ? k_lane : c;
      r[c] = tau_lo - prefix_hi<N>(A.ep_hi, e, k);
      mem[c] = 1u << c;
      cnt[c] = 0;
      a_off[c] = 0;
      b_off[c] = 0;
#pragma unroll
      for (int j = 0; j < N - 1; ++j) m[c][j] = 0;
      if (MCH > 1) check_at = min(check_at, r[c] + span + 1);
    }
  }

  __device__ bool finished() const { return fin == kAll; }

  __device__ uint32_t level_mask(uint32_t u) const {
    uint32_t lm = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) lm |= (uint32_t)(slot[j] == u) << j;
    return lm;
  }

  // completion of the classes in `done` at t: every member machine completes
  // and resets; returns the members
  __device__ uint32_t complete_class(uint32_t done, int32_t t) {
    uint32_t members = 0;
#pragma unroll
    for (int c = 0; c < MCH; ++c)
      if ((done >> c) & 1u) {
        members |= mem[c];
        r[c] = t;
#pragma unroll
        for (int j = 0; j < N - 1; ++j) m[c][j] = 0;
      }
    const uint32_t live = members & ~fin;  // machines still recording their tuple
#pragma unroll
    for (int k = 0; k < MCH; ++k) {
      if ((live >> k) & 1u) {
        if ((int64_t)t > tau_lo) {
          if (!((found >> k) & 1u)) {
            found |= 1u << k;
            const int64_t dd = (int64_t)t - tau_lo;
            a_off[k] = dd <= (int64_t)span ? (int32_t)dd : 0;
          }
          if ((int64_t)t <= tau_hi) {
            ++cnt[k];
          } else {
            b_off[k] = (int32_t)((int64_t)t - tau_hi);
            fin |= 1u << k;
          }
        }
      }
    }
    return members;
  }

  // One event while several classes live (MCH > 1).  Returns false once the
  // lane has finished; `single` is set when one class is left.
  __device__ bool step_many(int32_t t, uint32_t lm) {
    if ((int64_t)t > stop) {
      fin = kAll;
      return false;
    }
    const uint32_t d = (uint32_t)t - (uint32_t)B;
    B = t;
#pragma unroll
    for (int c = 0; c < MCH; ++c)
      if (mem[c]) {
#pragma unroll
        for (int j = 0; j < N - 1; ++j) m[c][j] = age<W>(m[c][j], d);
      }
    {
      // classes with every window empty whose resets lie before t have
      // identical futures (no candidate, and every later event is after both
      // resets): merge them.  At a segment's first events this joins the
      // machines started before the first event of the lane's list.
      uint32_t empty = 0, acc = 0;
#pragma unroll
      for (int c = 0; c < MCH; ++c)
        if (mem[c] && (int64_t)t > r[c]) {
          Bits any = 0;
#pragma unroll
          for (int j = 0; j < N - 1; ++j) any |= m[c][j];
          if (any == 0) {
            empty |= 1u << c;
            acc |= mem[c];
          }
        }
      if (__popc(empty) >= 2) {
        const int lowest = __ffs((int)empty) - 1;
#pragma unroll
        for (int c = 0; c < MCH; ++c)
          if ((empty >> c) & 1u) mem[c] = (c == lowest) ? acc : 0u;
      }
    }
    if ((int64_t)t >= check_at) {
      // classes whose last reset lies more than Span back are identical: merge
      uint32_t stale = 0, acc = 0;
      int64_t next = INT64_MAX;
#pragma unroll
      for (int c = 0; c < MCH; ++c)
        if (mem[c]) {
          if (r[c] + span < (int64_t)t) {
            stale |= 1u << c;
            acc |= mem[c];
          } else {
            next = min(next, r[c] + span + 1);
          }
        }
      if (__popc(stale) >= 2) {
        const int lowest = __ffs((int)stale) - 1;
#pragma unroll
        for (int c = 0; c < MCH; ++c)
          if ((stale >> c) & 1u) mem[c] = (c == lowest) ? acc : 0u;
      }
      check_at = next;
    }
    uint32_t done = 0;
#pragma unroll
    for (int c = 0; c < MCH; ++c) {
      if (mem[c] && (int64_t)t > r[c]) {
        bool hit[NI];
#pragma unroll
        for (int j = 0; j < N - 1; ++j) hit[j] = (m[c][j] & win[j]) != 0;
        bool complete = (lm >> (N - 1)) & 1u;
        if constexpr (N > 1) complete = complete && hit[N - 2];
        if (complete) {
          done |= 1u << c;
        } else {
#pragma unroll
          for (int j = 0; j < N - 1; ++j)
            if (((lm >> j) & 1u) && (j == 0 || hit[j > 0 ? j - 1 : 0])) m[c][j] |= (Bits)1;
        }
      }
    }
    if (done) {
      const uint32_t members = complete_class(done, t);
      // classes that completed together are identical from now on
      if (__popc(done) >= 2) {
        const int lowest = __ffs((int)done) - 1;
#pragma unroll
        for (int c = 0; c < MCH; ++c)
          if ((done >> c) & 1u) mem[c] = (c == lowest) ? members : 0u;
      }
      check_at = min(check_at, (int64_t)t + span + 1);
#pragma unroll
      for (int c = 0; c < MCH; ++c)
        if ((mem[c] & ~fin) == 0u) mem[c] = 0u;
      if (fin == kAll) return false;
    }
    // classes never split; once one is left, move it to slot 0
    uint32_t alive = 0;
#pragma unroll
    for (int c = 0; c < MCH; ++c) alive |= (mem[c] != 0u ? 1u : 0u) << c;
    if (__popc(alive) == 1) {
#pragma unroll
      for (int c = 1; c < MCH; ++c)
        if ((alive >> c) & 1u) {
#pragma unroll
          for (int j = 0; j < N - 1; ++j) m[0][j] = m[c][j];
          r[0] = r[c];
          mem[0] = mem[c];
          mem[c] = 0u;
        }
      single = true;
    }
    return true;
  }

  // One event with a single class left (slot 0).  Returns false once the lane
  // has finished.  Branch-free but for the rare completion: an event at or
  // before the last reset only ages the windows.
  __device__ bool step_one(int32_t t, uint32_t lm) {
    if ((int64_t)t > stop) {
      fin = kAll;
      return false;
    }
    const uint32_t d = (uint32_t)t - (uint32_t)B;
    B = t;
    const uint32_t live = (int64_t)t > r[0] ? 1u : 0u;
    uint32_t hit[NI];
#pragma unroll
    for (int j = 0; j < N - 1; ++j) {
      m[0][j] = age<W>(m[0][j], d);
      hit[j] = (m[0][j] & win[j]) != 0 ? 1u : 0u;
    }
    uint32_t complete = live & (lm >> (N - 1)) & 1u;
    if constexpr (N > 1) complete &= hit[N - 2];
    if (complete) {
      complete_class(1u, t);
      if ((mem[0] & ~fin) == 0u) mem[0] = 0u;
      return fin != kAll;
    }
#pragma unroll
    for (int j = 0; j < N - 1; ++j)
      m[0][j] |= (Bits)(live & (lm >> j) & (j == 0 ? 1u : hit[j > 0 ? j - 1 : 0]));
    return true;
  }

  // The last tick at which the newest candidate of window mm (anchored at
  // `at`) still lies within the upper bound of the interval whose window
  // mask is w (its highest bit): INT32_MIN for an empty window.
  __device__ static int32_t deadline(Bits mm, int32_t at, Bits w) {
    if (mm == 0) return INT32_MIN;
    int newest, top;
    if constexpr (W == 64) {
      newest = __builtin_ctzll((unsigned long long)mm);
      top = 63 - __builtin_clzll((unsigned long long)w);
    } else {
      newest = __builtin_ctz((unsigned)mm);
      top = 31 - __builtin_clz((unsigned)w);
    }
    const int64_t d = (int64_t)at - newest + top;
    return d > (int64_t)INT32_MAX ? INT32_MAX : (d < (int64_t)INT32_MIN ? INT32_MIN : (int32_t)d);
  }

  // Switch the single class to lazy ageing (windows as step_one leaves them).
  __device__ void lazy_begin() {
    B0 = B;
    if constexpr (N > 1) {
#pragma unroll
      for (int j = 0; j < N - 1; ++j)
        hiw[j] = (W == 64) ? 63 - __builtin_clzll((unsigned long long)win[j])
                           : 31 - __builtin_clz((unsigned)win[j]);
      dl0 = deadline(m[0][0], B, win[0]);
      dlr = INT32_MIN;
#pragma unroll
      for (int j = 1; j < N - 1; ++j) dlr = max(dlr, deadline(m[0][j], B, win[j]));
    }
  }

  // The exact step of step_one at t after the lazy windows are aged to t;
  // the event is live (after the last reset) and not past stop.
  __device__ bool step_exact(int32_t t, uint32_t lm) {
    if constexpr (N > 1) m[0][0] = age<W>(m[0][0], (uint32_t)t - (uint32_t)B0);
#pragma unroll
    for (int j = 1; j < N - 1; ++j) m[0][j] = age<W>(m[0][j], (uint32_t)t - (uint32_t)B);
    B0 = B = t;
    bool hit[NI];
#pragma unroll
    for (int j = 0; j < N - 1; ++j) hit[j] = (m[0][j] & win[j]) != 0;
    bool complete = (lm >> (N - 1)) & 1u;
    if constexpr (N > 1) complete = complete && hit[N - 2];
    if (complete) {
      complete_class(1u, t);
      if ((mem[0] & ~fin) == 0u) mem[0] = 0u;
      dl0 = dlr = INT32_MIN;
      return fin != kAll;
    }
    // a candidate added at t is its window's newest: the deadlines move to
    // t + hi (the older candidates' deadlines are earlier)
#pragma unroll
    for (int j = 0; j < N - 1; ++j) {
      const bool add = ((lm >> j) & 1u) && (j == 0 || hit[j > 0 ? j - 1 : 0]);
      m[0][j] |= (Bits)(add ? 1u : 0u);
      const int32_t dl = __builtin_elementwise_add_sat(t, hiw[j]);
      if (j == 0)
        dl0 = add ? dl : dl0;
      else
        dlr = add ? max(dlr, dl) : dlr;
    }
    return true;
  }

  // step_one for the lanes where `use` holds, with lazily aged windows (after
  // lazy_begin).  The windows are relative to their anchors, so an event that
  // changes no window needs no ageing at all.  An event on node levels >= 1
  // only can change the state only through a hit, which needs a candidate of
  // the previous node within that interval's upper bound: past dl0 (level 1)
  // and dlr (levels >= 2) there is none, so nothing happens.  A node-0 event
  // otherwise only adds a candidate to window 0.  Every other live event (a
  // possible hit or completion) takes the exact step, a branch that the wave
  // runs only while one of its lanes needs it.  Returns false once the lane
  // has finished.
  __device__ bool step_lazy_if(bool use, int32_t t, uint32_t lm) {
    lm &= (1u << N) - 1u;
    const bool over = use && (int64_t)t > stop;
    const bool on = use && !over && (int64_t)t > r[0];
    bool slow;
    if constexpr (N == 1) {
      slow = on && (lm & 1u);
    } else {
      slow = on && ((((lm >> 1) & 1u) && t <= dl0) || ((lm >> 2) != 0u && t <= dlr));
      const bool add0 = on && !slow && (lm & 1u);
      const Bits aged = age<W>(m[0][0], (uint32_t)t - (uint32_t)B0) | (Bits)1;
      m[0][0] = add0 ? aged : m[0][0];
      B0 = add0 ? t : B0;
      dl0 = add0 ? __builtin_elementwise_add_sat(t, hiw[0]) : dl0;
    }
    if (slow) {
      if (!step_exact(t, lm)) return false;
    }
    fin = over ? kAll : fin;
    return !over;
  }

  // step_one for the lanes where `use` holds, as predicated arithmetic (the
  // others keep their state): no branch but for the rare completion.
  // Returns false once the lane has finished.
  __device__ bool step_one_if(bool use, int32_t t, uint32_t lm) {
    const bool over = use && (int64_t)t > stop;
    const bool on = use && !over;
    const uint32_t d = on ? (uint32_t)t - (uint32_t)B : 0u;
    B = on ? t : B;
    const uint32_t live = (on && (int64_t)t > r[0]) ? 1u : 0u;
    uint32_t hit[NI];
#pragma unroll
    for (int j = 0; j < N - 1; ++j) {
      m[0][j] = age<W>(m[0][j], d);
      hit[j] = (m[0][j] & win[j]) != 0 ? 1u : 0u;
    }
    uint32_t complete = live & (lm >> (N - 1)) & 1u;
    if constexpr (N > 1) complete &= hit[N - 2];
    if (complete) {
      complete_class(1u, t);
      if ((mem[0] & ~fin) == 0u) mem[0] = 0u;
      return fin != kAll;
    }
#pragma unroll
    for (int j = 0; j < N - 1; ++j)
      m[0][j] |= (Bits)(live & (lm >> j) & (j == 0 ? 1u : hit[j > 0 ? j - 1 : 0]));
    fin = over ? kAll : fin;
    return !over;
  }

  __device__ bool step(int32_t t, uint32_t lm) { return single ? step_one(t, lm) : step_many(t, lm); }

  // The tuples of the (segment, episode): one per machine lane (MCH = 1), or
  // the distinct ones of the classes (equal keys mean identical tuples: same
  // first completion after the cut, or none within Span); machine 0's tuple
  // stays first.
  __device__ void write(const MapArgs& A, int64_t e, int64_t p, int k_lane) const {
    const int64_t pe = A.ts.idx(e, p);
    if (MCH == 1) {
      Tuple tu;
      tu.a = a_off[0];
      tu.c = cnt[0];
      tu.b = b_off[0];
      tu.pad = 0;
      *A.ts.at(e, p, k_lane) = tu;
      if (k_lane == 0) {
        A.ts.nmap[pe] = A.n_machines;
        A.ts.nslots[pe] = A.n_machines;
      }
    } else {
      write_class_tuples<MCH>(A, e, p, a_off, cnt, b_off);
    }
  }
};

// Position Map kernel (bit windows, relevant events only).
//
// Each chunk of events is staged in LDS with, for every node type slot u, a
// presence bitmap over the chunk's positions (bit i of word w: event 64w+i has
// a type on slot u).  A lane ORs the bitmaps of its episode's node types and
// visits only the set bits, in order (the machines ignore every other event
// anyway).  Lanes of one workgroup share the staged chunk.  The lane's
// machines are a ClassLane: MCH = N, all N machines of a (segment, episode) as
// classes; MCH = 1, one machine per lane (M lanes per (segment, episode)).
template <int N, int W, int MCH>
__global__ __launch_bounds__(kBlock) void map_bits_kernel(MapArgs A) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int32_t s_beg[kBlock];
  __shared__ int32_t s_len[kBlock];
  __shared__ int32_t s_chunks;
  __shared__ uint64_t s_seen[1024];  // node-type set and ranks (type_slot)
  __shared__ uint8_t s_rank[1024];

  const int tile = A.R * A.CH;
  const int words = tile >> 6;
  uint64_t* s_bits = (uint64_t*)smem;                       // [words][U], word-major
  int32_t* s_t = (int32_t*)(s_bits + (size_t)A.U * words);  // [tile]
  uint8_t* s_s = (uint8_t*)(s_t + tile);                    // [tile]

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int per_seg = A.G * A.M;
  const int r_idx = tid / per_seg;
  const int g = (tid / A.M) % A.G;
  const int k_lane = tid % A.M;
  const int64_t seg_group = (int64_t)blockIdx.x / A.n_egroups;
  const int64_t ep_group = (int64_t)blockIdx.x - seg_group * A.n_egroups;
  const int64_t p = seg_group * A.R + r_idx;
  const int64_t e = ep_group * A.G + g;
  const bool active = tid < A.R * per_seg && p < A.P && e < A.S && !segment_uses_ticks(A, p, N);

  if (tid == 0) s_chunks = 0;
  __syncthreads();
  if (tid < A.R) {
    const int64_t pp = seg_group * A.R + tid;
    int32_t b = 0, len = 0;
    if (pp < A.P && !segment_uses_ticks(A, pp, N)) {
      b = A.seg_beg[pp];
      len = A.seg_end[pp] - b;
    }
    s_beg[tid] = b;
    s_len[tid] = len;
    atomicMax(&s_chunks, (len + A.CH - 1) / A.CH);
  }
  ClassLane<N, W, MCH> lane;
  lane.init(A, e, p, k_lane, active);
  __syncthreads();
  const int n_chunks = s_chunks;
  if (n_chunks > 0) {
    load_type_tables(A, s_seen, s_rank);
    __syncthreads();
  }

  // The fill: the tile (R segments x CH events, CH a multiple of 64) is read in
  // batches of kPer events per thread with every load of a batch in flight,
  // position pos = segment * CH + offset.
  constexpr int kPer = 4;
  const int CE = kPer * nthr;
  // pos / CH through a float reciprocal: pos + 0.5 is at least 0.5 / CH from a
  // multiple of CH and pos < 2^16, far inside float precision; the two
  // corrections keep it exact regardless
  const float inv_ch = 1.0f / (float)A.CH;
  auto in_tile = [&](int ch, int pos, int32_t* src) -> bool {
    if (pos >= tile) return false;
    int rr = (int)(((float)pos + 0.5f) * inv_ch);
    rr -= rr * A.CH > pos ? 1 : 0;
    rr += (rr + 1) * A.CH <= pos ? 1 : 0;
    const int32_t i = pos - rr * A.CH;
    *src = s_beg[rr] + ch * A.CH + i;
    return i < s_len[rr] - ch * A.CH;
  };

  for (int ch = 0; ch < n_chunks; ++ch) {
    if (ch > 0) __syncthreads();  // previous chunk fully consumed
    for (int i = tid; i < A.U * words; i += nthr) s_bits[i] = 0;
    __syncthreads();
    for (int i0 = 0; i0 < tile; i0 += CE) {
      int32_t tt[kPer];
      uint32_t ty[kPer];
      bool ok[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        int32_t src = 0;
        ok[k] = in_tile(ch, i0 + k * nthr + tid, &src);
        tt[k] = ok[k] ? A.times[src] : 0;
        ty[k] = ok[k] ? A.types[src] : 0u;
      }
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int pos = i0 + k * nthr + tid;
        const uint32_t u = ok[k] ? type_slot(s_seen, s_rank, ty[k]) : 0u;
        if (u) {
          s_t[pos] = tt[k];
          s_s[pos] = (uint8_t)u;
          atomicOr((unsigned long long*)&s_bits[(pos >> 6) * A.U + (u - 1)], 1ull << (pos & 63));
        }
      }
    }
    __syncthreads();
    if (lane.finished()) continue;
    int32_t len = s_len[r_idx] - ch * A.CH;
    len = len < A.CH ? len : A.CH;
    if (len <= 0) continue;
    // cursor over this lane's relevant events of the chunk: word w of the
    // OR of its node slots' presence bitmaps, with `word` its unvisited bits
    const int w0 = (r_idx * A.CH) >> 6;
    const int w1 = w0 + ((len + 63) >> 6);
    int w = w0;
    uint64_t word = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) word |= s_bits[w * A.U + (lane.slot[j] - 1)];
    // next relevant position, or -1 when the chunk is exhausted
    auto next_pos = [&]() -> int {
      while (word == 0) {
        if (++w >= w1) return -1;
#pragma unroll
        for (int j = 0; j < N; ++j) word |= s_bits[w * A.U + (lane.slot[j] - 1)];
      }
      const int pos = (w << 6) + (__ffsll((unsigned long long)word) - 1);
      word &= word - 1;
      return pos;
    };
    // several classes (boundary halo only; MCH > 1)
    if (MCH > 1 && !lane.single) {
      for (;;) {
        const int pos = next_pos();
        if (pos < 0) break;
        if (!lane.step_many(s_t[pos], lane.level_mask(s_s[pos]))) break;
        if (lane.single) break;
      }
    }
    // one class, in slot 0; the next event's LDS reads are issued before the
    // current event is processed
    if (lane.single && !lane.finished()) {
      int pos = next_pos();
      int32_t t_next = pos >= 0 ? s_t[pos] : 0;
      uint32_t u_next = pos >= 0 ? s_s[pos] : 0u;
      while (pos >= 0) {
        const int32_t t = t_next;
        const uint32_t u = u_next;
        pos = next_pos();
        if (pos >= 0) {
          t_next = s_t[pos];
          u_next = s_s[pos];
        }
        if (!lane.step_one(t, lane.level_mask(u))) break;
      }
    }
  }

  if (active) lane.write(A, e, p, k_lane);
}

// The single-class walk of the list Map kernels: the lane's list from cursor
// (block b, entry i of the list at region offset `off`, `cnt` entries; the
// next block's bounds off_next / cnt_next) to its end or until step() reports
// the lane finished.  Batches of kD entries are read as kD / 2 aligned 16-byte
// loads (a lane reads its list in whole lines, which stay useful even when
// the L1 cannot hold every lane's line), the next batch's loads in flight.  A
// batch starts at an even entry of its block's region (region starts are
// 16-byte aligned); entries before the lane's cursor or past the list are
// read (they lie in the region, or in the buffer's slack) and skipped.  Each
// lane carries its own cursor (block, region index) across blocks: the batch
// after a block's last one is the next block's first, loaded ahead like any
// other, so a wave's lanes never wait for one another at block ends.  The
// loads are unconditional so that the compiler can count them and wait only
// for the batch about to be stepped through.  step(use, t, lm) steps the
// lanes where `use` holds and returns false once the lane has finished.
template <class Step>
__device__ __forceinline__ void list_walk(const MapArgs& A, int64_t e, int64_t b, int64_t b_last,
                                          int32_t off, int32_t cnt, int32_t i, int32_t off_next,
                                          int32_t cnt_next, Step&& step) {
  constexpr int kD = 8;
  const int64_t region_len = (int64_t)kListBlock * A.max_share;
  const int4* v = (const int4*)(A.lists + b * region_len);  // the cursor's block region
  int32_t rel = off;    // the list's first entry in it
  int32_t n_end = cnt;
  int32_t first = i;    // entries before it are done
  int32_t j0 = (rel + i) & ~1;  // even region index of the current batch
  bool go = true;
  // the bounds of the list two blocks ahead as well: a batch's address then
  // never waits on a bounds load issued in the iteration before it (on short
  // lists, one block per batch, that would put two loads in a row per block)
  int32_t off_next2 = 0, cnt_next2 = 0;
  if (b + 1 < b_last) {
    off_next2 = A.list_off[(b + 2) * A.S + e];
    cnt_next2 = A.list_cnt[(b + 2) * A.S + e];
  }
  auto advance = [&]() {  // to block b + 1's list, the bounds two blocks ahead loaded
    ++b;
    v = (const int4*)(A.lists + b * region_len);
    rel = off_next;
    n_end = cnt_next;
    first = 0;
    j0 = rel & ~1;
    off_next = off_next2;
    cnt_next = cnt_next2;
    if (b + 1 < b_last) {
      off_next2 = A.list_off[(b + 2) * A.S + e];
      cnt_next2 = A.list_cnt[(b + 2) * A.S + e];
    }
  };
  if (j0 >= rel + n_end) {
    // this block holds nothing more for the lane: the next one
    if (b < b_last)
      advance();
    else
      go = false;
  }
  if (!go) return;
  int4 cur[kD / 2];
#pragma unroll
  for (int q = 0; q < kD / 2; ++q) cur[q] = v[min(j0 + 2 * q, (rel + n_end + 1) & ~1) >> 1];
  while (go) {
    // the batch after this one: the rest of this block, or the next block
    const bool same = j0 + kD < rel + n_end;
    const bool more = same || b < b_last;
    const int4* nv = v;
    int32_t n_rel = rel, n_n = n_end, n_j0 = j0 + kD;
    if (!same && more) {
      nv = (const int4*)(A.lists + (b + 1) * region_len);
      n_rel = off_next;
      n_n = cnt_next;
      n_j0 = off_next & ~1;
    }
    int4 nxt[kD / 2];
#pragma unroll
    for (int q = 0; q < kD / 2; ++q) nxt[q] = nv[min(n_j0 + 2 * q, (n_rel + n_n + 1) & ~1) >> 1];
#pragma unroll
    for (int k = 0; k < kD; ++k) {
      const int32_t idx = j0 + k - rel;  // index within this episode's list
      const int4 w = cur[k >> 1];
      const int32_t t = (k & 1) ? w.z : w.x;
      const uint32_t lm = (uint32_t)((k & 1) ? w.w : w.y);
      go = step(go && idx >= first && idx < n_end, t, lm) && go;
    }
#pragma unroll
    for (int q = 0; q < kD / 2; ++q) cur[q] = nxt[q];
    if (!more) break;
    if (same)
      j0 += kD;
    else
      advance();
  }
}

// List Map kernel (bit windows): the ClassLane machines fed from the filter
// kernel's per-episode event lists instead of a staged chunk.  The lane of
// (segment, episode) reads, in time order, its episode's entries of the event
// blocks its segment's range (tau_p - maxSpan, tau_{p+1} + maxSpan] covers;
// no LDS and no barriers.  The segment's start, while several classes live,
// is stepped one entry at a time; the single class left then walks the rest
// (list_walk), with lazily aged windows where the lists are unpruned (most
// entries then change nothing) and the branch-free step where they are pruned
// (nearly every entry left is a hit).
template <int N, int W, int MCH, bool LAZY>
__global__ __launch_bounds__(kBlock) void map_list_kernel(MapArgs A) {
  const int tid = threadIdx.x;
  const int per_seg = A.G * A.M;
  const int r_idx = tid / per_seg;
  const int g = (tid / A.M) % A.G;
  const int k_lane = tid % A.M;
  const int64_t seg_group = (int64_t)blockIdx.x / A.n_egroups;
  const int64_t ep_group = (int64_t)blockIdx.x - seg_group * A.n_egroups;
  const int64_t p = seg_group * A.R + r_idx;
  const int64_t e = ep_group * A.G + g;
  const bool active = tid < A.R * per_seg && p < A.P && e < A.S && !segment_uses_ticks(A, p, N);
  if (!active) return;
  ClassLane<N, W, MCH> lane;
  lane.init(A, e, p, k_lane, true);
  const int32_t beg = A.seg_beg[p];
  const int32_t end = A.seg_end[p];
  // the range holds times in (lo_t, tau_{p+1} + maxSpan]; the machines stop
  // by themselves at tau_{p+1} + Span
  const int64_t lo_t = lane.tau_lo - A.max_span;
  if (beg < end) {
    const int64_t b_last = (end - 1) / kListBlock;
    int64_t b = beg / kListBlock;
    const int2* list = nullptr;
    int32_t n_here = 0, i = 0, off = 0;
    // block b's list; the next block's bounds are loaded meanwhile
    int32_t off_next = A.list_off[b * A.S + e];
    int32_t cnt_next = A.list_cnt[b * A.S + e];
    auto open = [&]() {
      off = off_next;
      list = A.lists + b * (int64_t)kListBlock * A.max_share + off;
      n_here = cnt_next;
      i = 0;
      if (b < b_last) {
        off_next = A.list_off[(b + 1) * A.S + e];
        cnt_next = A.list_cnt[(b + 1) * A.S + e];
      }
    };
    open();
    // the first block also holds the episode's events before the range: skip
    // them by a binary search for the first entry after lo_t
    {
      int32_t lo = 0, hi = n_here;
      while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if ((int64_t)list[mid].x <= lo_t)
          lo = mid + 1;
        else
          hi = mid;
      }
      i = lo;
    }
    bool go = true;
    if constexpr (MCH > 1) {
      // several classes (the segment's first events): one entry at a time,
      // the next entry's load issued before the current one is stepped
      int2 en = i < n_here ? list[i] : make_int2(0, 0);
      while (go && !lane.single) {
        while (i >= n_here && b < b_last) {
          ++b;
          open();
          if (i < n_here) en = list[i];
        }
        if (i >= n_here) break;
        const int2 cur = en;
        ++i;
        if (i < n_here) en = list[i];
        go = lane.step_many(cur.x, (uint32_t)cur.y);
      }
    }
    if (go && lane.single) {
      if constexpr (LAZY) lane.lazy_begin();
      list_walk(A, e, b, b_last, off, n_here, i, off_next, cnt_next,
                [&](bool use, int32_t t, uint32_t lm) {
                  if constexpr (LAZY)
                    return lane.step_lazy_if(use, t, lm);
                  else
                    return lane.step_one_if(use, t, lm);
                });
    }
  }
  lane.write(A, e, p, k_lane);
}

// ------------------------------------------------------- tick Map kernel

// Dilation program of one interval (lo, hi], hi <= 63: the first shifts lo + 1
// (this word) and 64 - hi (the previous word) and the amounts of the doubling
// steps, 5 bits per step, whose subset sums are exactly 0 .. hi-lo-1 (amounts
// 1, 2, 4, ... then the remainder; steps past the last have amount 0 and
// change nothing).
struct DilProg {
  uint32_t a;   // lo + 1
  uint32_t h;   // 64 - hi
  uint32_t pk;  // step i amount at bits 5i .. 5i+4
};

// Doubling steps an interval (lo, hi] needs; the kernel runs the largest count
// of the call for every episode.
__host__ __device__ inline int dil_steps(uint32_t lo, uint32_t hi) {
  const uint32_t W = hi - lo;
  int k = 0;
  while ((2u << k) <= W) ++k;  // 2^k <= W < 2^(k+1)
  return k + (W != (1u << k) ? 1 : 0);
}

__device__ inline DilProg dil_prog(uint32_t lo, uint32_t hi) {
  const uint32_t W = hi - lo;  // 1 .. 63
  const int k = 31 - __clz((int)W);
  uint32_t pk = 0;
  for (int i = 0; i < k; ++i) pk |= (1u << i) << (5 * i);
  pk |= (W - (1u << k)) << (5 * k);
  return {lo + 1, 64 - hi, pk};
}

// Candidates of node j+1 in one 64-tick word from node j's candidates in the
// previous word (prev) and this word (cur): bit i is set iff some node-j
// candidate lies d ticks earlier with lo < d <= hi.  With W = hi - lo that is
// the OR over m in [0, W) of (cur << (lo+1)) << m, from this word, and of
// (prev >> (64-hi)) >> m, from the previous one (hi <= 63, so no candidate
// older than the previous word can reach this one).  Each part is one 64-bit
// doubling chain over the program's amounts; the two chains are independent,
// and amount-0 padding steps are exact no-ops, so the code has no per-lane
// branches.  K is uniform over the launch.
__device__ inline uint64_t dilate(uint64_t prev, uint64_t cur, DilProg d, int K) {
  uint64_t y = cur << d.a;
  uint64_t x = prev >> d.h;
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    if (i >= K) break;
    const uint32_t s = (d.pk >> (5 * i)) & 31u;
    y |= y << s;
    x |= x >> s;
  }
  return y | x;
}

// dilate() with an empty previous word (right after a reset).
__device__ inline uint64_t dilate_noprev(uint64_t cur, DilProg d, int K) {
  uint64_t y = cur << d.a;
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    if (i >= K) break;
    y |= y << ((d.pk >> (5 * i)) & 31u);
  }
  return y;
}

// The same two with the step count fixed at compile time (KC >= the launch's
// K; the extra steps have amount 0).
template <int KC>
__device__ inline uint64_t dilate_k(uint64_t prev, uint64_t cur, DilProg d) {
  uint64_t y = cur << d.a;
  uint64_t x = prev >> d.h;
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const uint32_t s = (d.pk >> (5 * i)) & 31u;
    y |= y << s;
    x |= x >> s;
  }
  return y | x;
}

template <int KC>
__device__ inline uint64_t dilate_k_noprev(uint64_t cur, DilProg d) {
  uint64_t y = cur << d.a;
#pragma unroll
  for (int i = 0; i < KC; ++i) y |= y << ((d.pk >> (5 * i)) & 31u);
  return y;
}

// The candidate chain of one word: node 0 candidates are e0 (its events after
// the machine's last reset); node j+1 candidates are its events that a node-j
// candidate can precede.  Later nodes need no mask: every candidate descends
// from a node-0 candidate after the reset, and the window only moves forward.
// Writes nodes 0..N-2 to cur and returns node N-1 (completions).  The _noprev
// forms take an empty previous word (the machine reset inside this word).
template <int N>
__device__ inline uint64_t word_chain(const uint64_t* E, uint64_t e0, const uint64_t* prev,
                                      uint64_t* cur, const DilProg* dp, int K) {
  uint64_t c = e0;
#pragma unroll
  for (int j = 1; j < N; ++j) {
    cur[j - 1] = c;
    c = E[j] & dilate(prev[j - 1], c, dp[j - 1], K);
  }
  return c;
}

template <int N>
__device__ inline uint64_t word_chain_noprev(const uint64_t* E, uint64_t e0, uint64_t* cur,
                                             const DilProg* dp, int K) {
  uint64_t c = e0;
#pragma unroll
  for (int j = 1; j < N; ++j) {
    cur[j - 1] = c;
    c = E[j] & dilate_noprev(c, dp[j - 1], K);
  }
  return c;
}

template <int N, int KC>
__device__ inline uint64_t word_chain_k(const uint64_t* E, uint64_t e0, const uint64_t* prev,
                                        uint64_t* cur, const DilProg* dp) {
  uint64_t c = e0;
#pragma unroll
  for (int j = 1; j < N; ++j) {
    cur[j - 1] = c;
    c = E[j] & dilate_k<KC>(prev[j - 1], c, dp[j - 1]);
  }
  return c;
}

template <int N, int KC>
__device__ inline uint64_t word_chain_k_noprev(const uint64_t* E, uint64_t e0, uint64_t* cur,
                                               const DilProg* dp) {
  uint64_t c = e0;
#pragma unroll
  for (int j = 1; j < N; ++j) {
    cur[j - 1] = c;
    c = E[j] & dilate_k_noprev<KC>(c, dp[j - 1]);
  }
  return c;
}

// Tick Map kernel (bit-parallel over time, t_high <= 63).
//
// Each chunk of a segment's time range is staged in LDS as one bitmap per node
// type slot over 64-tick words (events of one type on one tick are
// interchangeable, so a bit per (type, tick) is exact).  A machine's state is,
// per node, the candidate bitmap of the previous word; one word advances all
// 64 ticks at once with shifts and ANDs (word_chain).  A completion (rare)
// resets the machine: the rest of the word is recomputed from an empty state.
// Times inside the word loop are int32 offsets from the current chunk's first
// tick.  Lanes, machine classes and tuples are as in the position kernel.
//
// The grid holds one workgroup per (episode group, group of R segments).  When
// every segment of the group fits one chunk, workgroups 0 .. eg_blocks-1 of
// the group each loop over its episode groups (eg, eg + eg_blocks, ...) and
// build the bitmaps once, reusing them for every later episode group; the
// other workgroups of the group exit at once.  Otherwise each workgroup counts
// its own episode group.
// Up to four nodes the kernel is held to three waves per SIMD (168 VGPRs):
// the few registers it then spills are used outside the word loops.
template <int N, int MCH>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(N <= 4 ? 3 : 1)))
void map_ticks_kernel(MapArgs A) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int64_t s_cur[kBlock];     // first tick of segment r's current chunk
  __shared__ int32_t s_nw[kBlock];      // words of segment r in the current chunk (0: none)
  __shared__ int32_t s_skip[kBlock];    // the chunk starts >= 64 ticks after the last word
  __shared__ int32_t s_ev[kBlock];      // next event index of segment r
  __shared__ int32_t s_end[kBlock];     // first event past the chunk (lowered by the fill)
  __shared__ int32_t s_maxw[kBlock];    // last word of the chunk holding an event
  __shared__ int32_t s_seg_end[kBlock]; // segment r's event range end; 0 for a segment not counted here
  __shared__ int32_t s_built[kBlock];   // first event of the chunk the bitmaps hold (-1: none)
  __shared__ int32_t s_more, s_reuse, s_fit, s_any;
  __shared__ uint64_t s_seen[1024];     // node-type set and ranks (type_slot)
  __shared__ uint8_t s_rank[1024];
  uint64_t* s_tb = (uint64_t*)smem;     // [R*CW words][U], word-major

  constexpr int NI = N > 1 ? N - 1 : 1;
  constexpr int kPer = N >= 3 ? 4 : 8;  // events per thread per fill batch (fewer registers as N grows)
  constexpr int32_t kFar = 1 << 30;     // offsets are clamped to +-kFar
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int per_seg = A.G * A.M;
  const int r_idx = tid / per_seg;
  const int g = (tid / A.M) % A.G;
  const int k_lane = tid % A.M;
  // segment group fastest: the workgroups that loop (eg_id < eg_blocks) are
  // the first ones, spread over every XCD by the round-robin dispatch
  const int64_t seg_groups = (A.P + A.R - 1) / A.R;
  const int64_t eg_id = (int64_t)blockIdx.x / seg_groups;
  const int64_t seg_group = (int64_t)blockIdx.x - eg_id * seg_groups;
  const int64_t p = seg_group * A.R + r_idx;
  const bool seg_here = tid < A.R * per_seg && p < A.P && segment_uses_ticks(A, p, N);
  const int CW = A.CW;
  const int CE = kPer * nthr;
  const uint32_t all = (MCH == 32) ? 0xffffffffu : ((1u << MCH) - 1u);

  if (tid == 0) {
    s_fit = 1;
    s_any = 0;
  }
  __syncthreads();
  if (tid < A.R) {
    const int64_t pp = seg_group * A.R + tid;
    int32_t end = 0;
    if (pp < A.P && segment_uses_ticks(A, pp, N)) {
      s_any = 1;
      end = A.seg_end[pp];
      const int32_t beg = A.seg_beg[pp];
      if (beg < end && (((int64_t)A.times[end - 1] - A.times[beg]) >> 6) >= CW) s_fit = 0;
    }
    s_seg_end[tid] = end;
    s_built[tid] = -1;
  }
  int64_t tau_lo = 0, tau_hi = 0;
  if (seg_here) {
    tau_lo = A.tau[p];
    tau_hi = A.tau[p + 1];
  }
  __syncthreads();
  if (!s_any) return;  // no segment of the group is counted here (whole workgroup)
  const bool fit = s_fit != 0;
  if (fit && eg_id >= A.eg_blocks) return;  // the group's looping workgroups cover it
  load_type_tables(A, s_seen, s_rank);  // first read after the chunk loop's barrier
  const int64_t eg_step = fit ? A.eg_blocks : A.n_egroups;

  for (int64_t eg = eg_id; eg < A.n_egroups; eg += eg_step) {
    const int64_t eo = eg * A.G + g;
    const bool active = seg_here && eo < A.S;
    const int64_t e = (A.ep_perm && eo < A.S) ? A.ep_perm[eo] : eo;
    const int K = A.group_k ? A.group_k[eg] : A.dil_steps;
    if (tid < A.R) {
      const int64_t pp = seg_group * A.R + tid;
      s_ev[tid] = s_seg_end[tid] ? A.seg_beg[pp] : 0;
      s_cur[tid] = INT64_MIN / 2;                // no word processed yet
      s_nw[tid] = 0;
    }

    // ---- lane state
    int32_t lds_slot[N];     // this lane's node-type bitmaps in word 0 of its segment
    DilProg dp[NI];
    int32_t span = 0;
    uint64_t prv[MCH][NI];   // per class: node candidates of the previous word
    int32_t r[MCH];          // per class: last reset, as an offset from org
    uint32_t mem[MCH];
    int32_t cnt[MCH], a_off[MCH], b_off[MCH];
    uint32_t found = 0, fin = 0;
    int64_t stop = 0, org = 0;
    bool single = MCH == 1;
    if (active) {
#pragma unroll
      for (int j = 0; j < N; ++j)
        lds_slot[j] = r_idx * CW * A.U + (A.ep_slot[e * N + j] - 1);
#pragma unroll
      for (int j = 0; j < N - 1; ++j)
        dp[j] = dil_prog((uint32_t)A.ep_lo[e * (N - 1) + j], (uint32_t)A.ep_hi[e * (N - 1) + j]);
      span = A.ep_span[e];
      stop = tau_hi + span;
      org = tau_lo;
#pragma unroll
      for (int c = 0; c < MCH; ++c) {
        const int k = (MCH == 1) ? k_lane : c;
        r[c] = -(int32_t)prefix_hi<N>(A.ep_hi, e, k);
        mem[c] = 1u << c;
        cnt[c] = 0;
        a_off[c] = 0;
        b_off[c] = 0;
#pragma unroll
        for (int j = 0; j < NI; ++j) prv[c][j] = 0;
      }
    } else {
      fin = all;
      single = true;
#pragma unroll
      for (int j = 0; j < N; ++j) lds_slot[j] = 0;
#pragma unroll
      for (int j = 0; j < NI; ++j) dp[j] = {1u, 0u};
#pragma unroll
      for (int c = 0; c < MCH; ++c) {
        r[c] = 0;
        mem[c] = 0;
        cnt[c] = a_off[c] = b_off[c] = 0;
#pragma unroll
        for (int j = 0; j < NI; ++j) prv[c][j] = 0;
      }
    }

    // completion of the machines of class c at tick t
    auto complete_members = [&](uint32_t members, int64_t t) {
      const uint32_t live = members & ~fin;
  #pragma unroll
      for (int k = 0; k < MCH; ++k) {
        if ((live >> k) & 1u) {
          if (t > tau_lo) {
            if (!((found >> k) & 1u)) {
              found |= 1u << k;
              const int64_t dd = t - tau_lo;
              a_off[k] = dd <= (int64_t)span ? (int32_t)dd : 0;
            }
            if (t <= tau_hi) {
              ++cnt[k];
            } else {
              b_off[k] = (int32_t)(t - tau_hi);
              fin |= 1u << k;
            }
          }
        }
      }
    };

    // Chunks are event-driven: a segment's next chunk starts right after its
    // last processed word, or at its next event when that lies 64 or more
    // ticks later (no event in between, and every candidate is then older
    // than any t_high <= 63, so the windows are simply emptied).  A chunk is at
    // most CW words and ends at the word of its last event, so the work is
    // bounded by the events, not the ticks.  The fill reads the events in
    // batches of kPer per thread until a batch reaches past the chunk; the
    // first event past it and the chunk's last word come out of LDS atomics.
    for (;;) {
      __syncthreads();  // previous chunk fully consumed; segment cursors final
      if (tid == 0) {
        s_more = 0;
        s_reuse = 1;
      }
      __syncthreads();
      if (tid < A.R) {
        const int32_t ev = s_ev[tid];
        const int32_t seg_end = s_seg_end[tid];
        if (ev < seg_end) {
          const int64_t next_t = A.times[ev];
          const int64_t contiguous = s_cur[tid] + (int64_t)s_nw[tid] * 64;
          const bool skip = next_t >= contiguous + 64;
          s_cur[tid] = skip ? next_t : contiguous;
          s_skip[tid] = skip ? 1 : 0;
          s_more = 1;
          if (s_built[tid] != ev) s_reuse = 0;
        } else {
          s_skip[tid] = 0;
          s_nw[tid] = 0;
        }
      }
      __syncthreads();
      if (!s_more) break;
      if (!s_reuse) {
        for (int i = tid; i < A.R * CW * A.U; i += nthr) s_tb[i] = 0;
        if (tid < A.R) {
          s_end[tid] = s_seg_end[tid];
          s_maxw[tid] = -1;
        }
        __syncthreads();
        for (int rr = 0; rr < A.R; ++rr) {
          const int32_t b0 = s_ev[rr];
          const int32_t seg_end = s_seg_end[rr];
          if (b0 >= seg_end) continue;
          const int64_t chunk_t0 = s_cur[rr];
          int32_t my_min = INT32_MAX, my_maxw = -1;
          for (int32_t base = b0;; base += CE) {
            // all loads of a batch are issued before any is used
            int32_t tt[kPer];
            uint32_t ty[kPer];
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
              const int32_t i = base + k * nthr + tid;
              tt[k] = i < seg_end ? A.times[i] : 0;
              ty[k] = i < seg_end ? A.types[i] : 0u;
            }
            const int64_t batch_last = (int64_t)base + CE < seg_end ? (int64_t)base + CE - 1 : seg_end - 1;
            const int64_t last_t = A.times[batch_last];
            uint32_t u[kPer];
#pragma unroll
            for (int k = 0; k < kPer; ++k) u[k] = type_slot(s_seen, s_rank, ty[k]);
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
              const int32_t i = base + k * nthr + tid;
              if (i < seg_end) {
                const int64_t w = ((int64_t)tt[k] - chunk_t0) >> 6;  // >= 0
                if (w < CW) {
                  my_maxw = (int32_t)w;  // events are sorted: the last one wins
                  if (u[k])
                    atomicOr((unsigned long long*)&s_tb[((int64_t)rr * CW + w) * A.U + (u[k] - 1)],
                             1ull << ((tt[k] - chunk_t0) & 63));
                } else if (i < my_min) {
                  my_min = i;
                }
              }
            }
            if (batch_last == seg_end - 1 || ((last_t - chunk_t0) >> 6) >= CW) break;
          }
          if (my_min != INT32_MAX) atomicMin(&s_end[rr], my_min);
          if (my_maxw >= 0) atomicMax(&s_maxw[rr], my_maxw);
        }
        __syncthreads();
        if (tid < A.R) {
          // the bitmaps now hold this chunk; a later episode group reuses them
          s_built[tid] = s_ev[tid] < s_seg_end[tid] ? s_ev[tid] : -1;
        }
      }
      if (tid < A.R && s_ev[tid] < s_seg_end[tid]) {
        // a reused chunk has the same extent as when it was built
        s_nw[tid] = s_maxw[tid] + 1;
        s_ev[tid] = s_end[tid];
      }
      __syncthreads();
      const int nw = fin == all ? 0 : s_nw[r_idx];
      int32_t stop_rel = -1;
      if (nw > 0) {
        // move the time origin to this chunk's first tick
        const int64_t chunk_t0 = s_cur[r_idx];
        const int64_t delta = chunk_t0 - org;
  #pragma unroll
        for (int c = 0; c < MCH; ++c) {
          const int64_t v = (int64_t)r[c] - delta;
          r[c] = (int32_t)(v < -kFar ? -kFar : v);
        }
        org = chunk_t0;
        const int64_t stop_d = stop - org;
        stop_rel = (int32_t)(stop_d > kFar ? kFar : (stop_d < -1 ? -1 : stop_d));
        if (s_skip[r_idx]) {
  #pragma unroll
          for (int c = 0; c < MCH; ++c)
  #pragma unroll
            for (int j = 0; j < NI; ++j) prv[c][j] = 0;
        }
      }
      int wi = 0;
      // Words of a lane that still has several machine classes (the first words
      // of a segment, and after a completion while classes differ).
      for (; MCH > 1 && wi < nw && !single; ++wi) {
        const int32_t wb = wi * 64;
        if (wb > stop_rel) {
          fin = all;
          break;
        }
        const int32_t row = wi * A.U;
        uint64_t E[N];
  #pragma unroll
        for (int j = 0; j < N; ++j) E[j] = s_tb[lds_slot[j] + row];
        const int32_t to = stop_rel - wb;  // >= 0
        const uint64_t keep_hi = to >= 63 ? ~0ull : ((~0ull) >> (63 - to));
        {
          // classes whose last reset lies more than Span before this word are
          // identical for the rest of the stream: merge them
          uint32_t stale = 0, acc = 0;
  #pragma unroll
          for (int c = 0; c < MCH; ++c)
            if (mem[c] && r[c] + span < wb) {
              stale |= 1u << c;
              acc |= mem[c];
            }
          if (__popc(stale) >= 2) {
            const int lowest = __ffs((int)stale) - 1;
  #pragma unroll
            for (int c = 0; c < MCH; ++c)
              if ((stale >> c) & 1u) mem[c] = (c == lowest) ? acc : 0u;
          }
        }
        uint32_t done = 0;  // classes that completed in this word (for merging)
  #pragma unroll
        for (int c = 0; c < MCH; ++c) {
          if (!mem[c]) continue;
          const int32_t from = r[c] + 1 - wb;
          const uint64_t keep_lo = from <= 0 ? ~0ull : (from >= 64 ? 0ull : ((~0ull) << from));
          uint64_t cur[NI];
          uint64_t last = word_chain<N>(E, E[0] & keep_lo, prv[c], cur, dp, K) & keep_hi;
          while (last != 0) {
            const int bit = __ffsll((unsigned long long)last) - 1;
            complete_members(mem[c], org + wb + bit);
            r[c] = wb + bit;
            done |= 1u << c;
            const uint64_t after = (~1ull) << bit;  // ticks after the completion (0 for bit 63)
            last = word_chain_noprev<N>(E, E[0] & after, cur, dp, K) & keep_hi;
          }
  #pragma unroll
          for (int j = 0; j < NI; ++j) prv[c][j] = cur[j];
        }
        if (done) {
          // classes that last reset on the same tick are identical
  #pragma unroll
          for (int c = 0; c < MCH; ++c)
  #pragma unroll
            for (int c2 = 0; c2 < c; ++c2)
              if (mem[c] && mem[c2] && ((done >> c) & 1u) && ((done >> c2) & 1u) && r[c] == r[c2]) {
                mem[c2] |= mem[c];
                mem[c] = 0u;
              }
  #pragma unroll
          for (int c = 0; c < MCH; ++c)
            if ((mem[c] & ~fin) == 0u) mem[c] = 0u;
          if (fin == all) break;
        }
        uint32_t alive = 0;
  #pragma unroll
        for (int c = 0; c < MCH; ++c) alive |= (mem[c] != 0u ? 1u : 0u) << c;
        if (__popc(alive) == 1) {
  #pragma unroll
          for (int c = 1; c < MCH; ++c)
            if ((alive >> c) & 1u) {
  #pragma unroll
              for (int j = 0; j < NI; ++j) prv[0][j] = prv[c][j];
              r[0] = r[c];
              mem[0] = mem[c];
            }
          // the other classes are empty from here on
  #pragma unroll
          for (int c = 1; c < MCH; ++c) {
            mem[c] = 0u;
            r[c] = 0;
  #pragma unroll
            for (int j = 0; j < NI; ++j) prv[c][j] = 0;
          }
          single = true;
        }
      }
      // Words of a lane with one class: the lean loop.  Ticks past stop are
      // masked out of the completions, so the loop needs no exit test; a lane
      // whose machines have all finished steps on without effect.  The masks
      // for the last reset and for stop are needed only in a segment's first
      // and last words, so each sits behind a branch that the wave takes only
      // when one of its lanes needs it.  The class's completions are recorded
      // as tick offsets from org (the first after tau_p, the count in
      // (tau_p, tau_{p+1}], the first after tau_{p+1}) and credited to its
      // member machines once, after the loop.
      auto single_words = [&](auto kc) {
        constexpr int KC = decltype(kc)::value;
        constexpr int32_t kNone = INT32_MIN;
        uint64_t pv[NI];
  #pragma unroll
        for (int j = 0; j < NI; ++j) pv[j] = prv[0][j];
        int32_t r0 = r[0];
        const uint32_t m0 = mem[0];
        const int64_t tlo_d = tau_lo - org, thi_d = tau_hi - org;
        const int32_t tlo = (int32_t)(tlo_d < -kFar ? -kFar : (tlo_d > kFar ? kFar : tlo_d));
        const int32_t thi = (int32_t)(thi_d < -kFar ? -kFar : (thi_d > kFar ? kFar : thi_d));
        int32_t c_first = kNone, c_b = kNone, c_cnt = 0;
        int32_t ew[N];  // index of this lane's bitmap word of node j in word wi
  #pragma unroll
        for (int j = 0; j < N; ++j) ew[j] = lds_slot[j] + wi * A.U;
        const int32_t stride = A.U;
        for (; wi < nw; ++wi) {
          const int32_t wb = wi * 64;
          uint64_t E[N];
  #pragma unroll
          for (int j = 0; j < N; ++j) {
            E[j] = s_tb[ew[j]];
            ew[j] += stride;
          }
          uint64_t e0 = E[0];
          if (__ballot(r0 >= wb)) {
            const int32_t from = r0 + 1 - wb;
            e0 &= from <= 0 ? ~0ull : (from >= 64 ? 0ull : ((~0ull) << from));
          }
          uint64_t cur[NI];
          uint64_t last = word_chain_k<N, KC>(E, e0, pv, cur, dp);
          uint64_t kh = ~0ull;
          const int32_t to = stop_rel - wb;
          if (__ballot(to < 63)) {
            kh = to >= 63 ? ~0ull : (to < 0 ? 0ull : ((~0ull) >> (63 - to)));
            last &= kh;
          }
          while (last != 0) {
            const int bit = __ffsll((unsigned long long)last) - 1;
            const int32_t t = wb + bit;
            if (t > tlo) {
              if (c_first == kNone) c_first = t;
              if (t <= thi)
                ++c_cnt;
              else if (c_b == kNone)
                c_b = t;
            }
            r0 = t;
            const uint64_t after = (~1ull) << bit;
            last = word_chain_k_noprev<N, KC>(E, E[0] & after, cur, dp) & kh;
          }
  #pragma unroll
          for (int j = 0; j < NI; ++j) pv[j] = cur[j];
        }
  #pragma unroll
        for (int j = 0; j < NI; ++j) prv[0][j] = pv[j];
        r[0] = r0;
        // every live member completed at the class's completions: the first
        // after tau_p sets a (if the member has none yet), the ones up to
        // tau_{p+1} count, the first after tau_{p+1} sets b and ends the member
        const uint32_t live = m0 & ~fin;
        if (live && c_first != kNone) {
  #pragma unroll
          for (int k = 0; k < MCH; ++k) {
            if ((live >> k) & 1u) {
              if (!((found >> k) & 1u)) {
                found |= 1u << k;
                const int64_t dd = org + c_first - tau_lo;
                a_off[k] = dd <= (int64_t)span ? (int32_t)dd : 0;
              }
              cnt[k] += c_cnt;
              if (c_b != kNone) {
                b_off[k] = (int32_t)(org + c_b - tau_hi);
                fin |= 1u << k;
              }
            }
          }
        }
      };
      if (wi < nw && fin != all) {
        if (K <= 1)
          single_words(std::integral_constant<int, 1>());
        else if (K == 2)
          single_words(std::integral_constant<int, 2>());
        else if (K == 3)
          single_words(std::integral_constant<int, 3>());
        else if (K == 4)
          single_words(std::integral_constant<int, 4>());
        else if (K == 5)
          single_words(std::integral_constant<int, 5>());
        else
          single_words(std::integral_constant<int, 6>());
      }
      if (nw > 0 && stop_rel < nw * 64) fin = all;  // the lane passed its stop tick
    }

    if (active) {
      const int64_t pe = A.ts.idx(e, p);
      if (MCH == 1) {
        Tuple tu;
        tu.a = a_off[0];
        tu.c = cnt[0];
        tu.b = b_off[0];
        tu.pad = 0;
        *A.ts.at(e, p, k_lane) = tu;
        if (k_lane == 0) {
          A.ts.nmap[pe] = A.n_machines;
          A.ts.nslots[pe] = A.n_machines;
        }
      } else {
        int d = 0;
  #pragma unroll
        for (int c = 0; c < MCH; ++c) {
          bool dup = false;
  #pragma unroll
          for (int c2 = 0; c2 < c; ++c2) dup |= a_off[c2] == a_off[c];
          if (!dup) {
            Tuple tu;
            tu.a = a_off[c];
            tu.c = cnt[c];
            tu.b = b_off[c];
            tu.pad = 0;
            *A.ts.at(e, p, d) = tu;
            ++d;
          }
        }
        A.ts.nmap[pe] = d;
        A.ts.nslots[pe] = d;
      }
    }

  }
}

// ------------------------------------------- wave-cooperative single machine

// All 64 lanes hold the same machine(s); they load 64 events at a time with
// one coalesced access, ballot the events whose type sits on a node of the
// episode, and hand those, in order, to on_event(t, level mask), which returns
// false to stop the scan.
// Blocks of kDepth x 64 events; the next block's loads are issued before the
// current one is fed, so one load latency covers kDepth x 64 events (a
// repair rescans a whole segment, thousands of events of which a few percent
// are the episode's: such a scan is bound by load latency).
template <class Mach, int kDepth, class OnEvent>
__device__ __forceinline__ void wave_scan(const int32_t* times, const uint16_t* types, int64_t i0,
                                          int64_t i1, const typename Mach::Params& prm, OnEvent on_event) {
  const int lane = threadIdx.x & (kWave - 1);
  int32_t t_cur[kDepth], t_nxt[kDepth];
  uint32_t y_cur[kDepth], y_nxt[kDepth];
  auto load = [&](int64_t base, int32_t* tt, uint32_t* yy) {
#pragma unroll
    for (int q = 0; q < kDepth; ++q) {
      const int64_t i = base + q * kWave + lane;
      const bool valid = i < i1;
      tt[q] = valid ? times[i] : 0;
      yy[q] = valid ? (uint32_t)types[i] : 0xffffffffu;
    }
  };
  if (i0 >= i1) return;
  load(i0, t_cur, y_cur);
  bool go = true;
  for (int64_t base = i0; base < i1 && go; base += kDepth * kWave) {
    const int64_t nb = base + kDepth * kWave;
    if (nb < i1) load(nb, t_nxt, y_nxt);
#pragma unroll
    for (int q = 0; q < kDepth; ++q) {
      const uint32_t lm = y_cur[q] == 0xffffffffu ? 0u : prm.level_mask(y_cur[q]);
      uint64_t mask = __ballot(lm != 0u);
      while (mask != 0 && go) {
        const int src = __ffsll((unsigned long long)mask) - 1;
        mask &= mask - 1;
        const int32_t tt = __shfl(t_cur[q], src);
        const uint32_t ll = (uint32_t)__shfl((int)lm, src);
        go = on_event(tt, ll);
      }
    }
#pragma unroll
    for (int q = 0; q < kDepth; ++q) {
      t_cur[q] = t_nxt[q];
      y_cur[q] = y_nxt[q];
    }
  }
}

// One machine over events [i0, i1) (the loop of wave_scan, written out so
// that the machine stays in registers): deeper prefetch for the machines with
// little state (two nodes), 4 blocks for the rest as their registers allow.
template <class Mach>
__device__ void wave_feed_range(const int32_t* times, const uint16_t* types, int64_t i0, int64_t i1,
                                SegMachine<Mach>& sm, const typename Mach::Params& prm) {
  constexpr int kDepth = sizeof(SegMachine<Mach>) <= 72 ? 16 : 4;
  const int lane = threadIdx.x & (kWave - 1);
  int32_t t_cur[kDepth], t_nxt[kDepth];
  uint32_t y_cur[kDepth], y_nxt[kDepth];
  auto load = [&](int64_t base, int32_t* tt, uint32_t* yy) {
#pragma unroll
    for (int q = 0; q < kDepth; ++q) {
      const int64_t i = base + q * kWave + lane;
      const bool valid = i < i1;
      tt[q] = valid ? times[i] : 0;
      yy[q] = valid ? (uint32_t)types[i] : 0xffffffffu;
    }
  };
  if (i0 >= i1) return;
  load(i0, t_cur, y_cur);
  for (int64_t base = i0; base < i1 && !sm.finished; base += kDepth * kWave) {
    const int64_t nb = base + kDepth * kWave;
    if (nb < i1) load(nb, t_nxt, y_nxt);
#pragma unroll
    for (int q = 0; q < kDepth; ++q) {
      const uint32_t lm = y_cur[q] == 0xffffffffu ? 0u : prm.level_mask(y_cur[q]);
      uint64_t mask = __ballot(lm != 0u);
      while (mask != 0 && !sm.finished) {
        const int src = __ffsll((unsigned long long)mask) - 1;
        mask &= mask - 1;
        const int32_t tt = __shfl(t_cur[q], src);
        const uint32_t ll = (uint32_t)__shfl((int)lm, src);
        sm.feed(tt, ll, prm);
      }
    }
#pragma unroll
    for (int q = 0; q < kDepth; ++q) {
      t_cur[q] = t_nxt[q];
      y_cur[q] = y_nxt[q];
    }
  }
}

// ------------------------------------------------ closure (match + repair)

struct ClosureArgs {
  const int32_t* times;
  const uint16_t* types;
  const uint16_t* ep_types;
  const int32_t* ep_lo;
  const int32_t* ep_hi;
  const int32_t* ep_span;
  const int64_t* tau;
  const int32_t* seg_beg;
  const int32_t* seg_end;
  TupleStore ts;
  int32_t* flags;               // [S] non-zero: recount this episode with the fallback
  unsigned long long* repairs;  // repair-tuple counter
  int64_t S;
  int32_t P;
  // unmatched exits queued for repair_kernel: item << 5 | machine, queue_n
  // of them (slots past queue_cap are repaired where they are found);
  // queue_head hands them out
  uint64_t* queue;
  int64_t queue_cap;
  unsigned long long* queue_n;
  unsigned long long* queue_head;
  int32_t repair_blocks;  // workgroups of repair_kernel
  RingArena ring;         // ring windows: one slot per wave (wave_slot)
};

// The tuple of a chain that completed at x, x in (tau_q, tau_q + Span]: a
// machine reset at x runs over segment q.  Its count includes the completion
// at x itself when x <= tau_{q+1}.
//
// Bit-window machines take a shortcut: the machine reset at x runs in
// lockstep with segment q's machine 0 (reset at tau_q) until both behave
// alike (BitMachine::same_future), after machine 0's a-window has closed and
// before tau_{q+1}; from there on both complete at the same events, so the
// repair's count is its own so far plus what machine 0's Map tuple (found by
// its key a) counts after that point, and its b is machine 0's.  On this
// path a repair scans the events of a few Spans instead of a whole segment;
// if the machines never meet, or no Map tuple has machine 0's key, the
// machine reset at x runs to the end alone.
template <class Mach>
__device__ Tuple repair_tuple(const ClosureArgs& A, const typename Mach::Params& prm, int64_t e, int64_t q,
                              int64_t x) {
  const int64_t lo_cut = A.tau[q];
  const int64_t hi_cut = A.tau[q + 1];
  Tuple tu;
  tu.a = (int32_t)(x - lo_cut);
  tu.pad = 0;
  if (x > hi_cut) {
    tu.c = 0;
    tu.b = (int32_t)(x - hi_cut);
    return tu;
  }
  if constexpr (Mach::kComparable) {
    if (x > lo_cut) {
      SegMachine<Mach> R, M;
      R.init(x, lo_cut, hi_cut, prm.span);
      M.init(lo_cut, lo_cut, hi_cut, prm.span);
      const int64_t a_closed = lo_cut + prm.span;  // machine 0's a is final after this tick
      bool met = false;
      const int64_t i0 = upper_bound_time(A.times, A.seg_beg[q], A.seg_end[q], lo_cut);
      wave_scan<Mach, 4>(A.times, A.types, i0, A.seg_end[q], prm, [&](int32_t t, uint32_t lm) __attribute__((always_inline)) {
        R.feed(t, lm, prm);
        M.feed(t, lm, prm);
        if ((int64_t)t > a_closed && (int64_t)t > x && (int64_t)t < hi_cut && R.m.same_future(M.m)) {
          met = true;
          return false;
        }
        return !R.finished;
      });
      if (!met) {
        tu.c = R.count + 1;
        tu.b = R.b_off;
        return tu;
      }
      const int nm = A.ts.nmap[A.ts.idx(e, q)];
      for (int m = 0; m < nm && m < A.ts.slots; ++m) {
        const Tuple t0 = *A.ts.at(e, q, m);
        if (t0.a == M.a_off) {
          tu.c = R.count + (t0.c - M.count) + 1;
          tu.b = t0.b;
          return tu;
        }
      }
    }
  }
  SegMachine<Mach> sm;
  sm.attach(A.ring, wave_slot());
  sm.init(x, lo_cut, hi_cut, prm.span);
  const int64_t i0 = upper_bound_time(A.times, A.seg_beg[q], A.seg_end[q], x);
  wave_feed_range<Mach>(A.times, A.types, i0, A.seg_end[q], sm, prm);
  tu.c = sm.count + 1;
  tu.b = sm.b_off;
  return tu;
}

template <int N>
__device__ bool has_map_key(const ClosureArgs& A, int64_t q, int64_t e, int32_t key) {
  const int nm = A.ts.nmap[A.ts.idx(e, q)];
  bool hit = false;
  for (int m = 0; m < nm && m < N; ++m) hit |= A.ts.at(e, q, m)->a == key;
  return hit;
}

// Repairs one unmatched exit (machine k of boundary p of episode e) by the
// whole wave: a machine reset at the exit runs over segment p + 1, and on
// while its own exit finds no key in the next segment.
template <int N, class Mach>
__device__ void repair_exit(const ClosureArgs& A, const typename Mach::Params& prm, int64_t e, int64_t p,
                            int k, int lane) {
  int32_t x_off = A.ts.at(e, p, k)->b;
  int64_t q = p + 1;
  for (;;) {
    if (x_off <= 0) {  // a sentinel exit always has a sentinel key; never repair it
      if (lane == 0) atomicOr(&A.flags[e], 1);
      break;
    }
    const Tuple tu = repair_tuple<Mach>(A, prm, e, q, A.tau[q] + x_off);
    int slot = 0;
    if (lane == 0) slot = atomicAdd(&A.ts.nslots[A.ts.idx(e, q)], 1);
    slot = __shfl(slot, 0);
    if (slot >= A.ts.slots) {
      if (lane == 0) atomicOr(&A.flags[e], 1);
      break;
    }
    if (lane == 0) {
      *A.ts.at(e, q, slot) = tu;
      atomicAdd(A.repairs, 1ull);
    }
    if (q + 1 >= A.P) break;
    if (has_map_key<N>(A, q + 1, e, tu.b)) break;
    x_off = tu.b;
    ++q;
  }
}

// INLINE: misses the queue cannot take are repaired here, one wave at a time
// (the machine's code then sets the kernel's registers, and its occupancy:
// 195 VGPRs for two nodes against 15 for the matching alone); otherwise
// they send their episode to the whole-stream recount, as a full slot list
// does.  The launch takes the inline form only where there is no queue.
template <int N, class Mach, bool INLINE>
__global__ __launch_bounds__(kBlock) void closure_kernel(ClosureArgs A) {
  // items episode-major: consecutive lanes take consecutive boundaries of one
  // episode, so their first tuples are contiguous
  const int64_t n_items = (int64_t)(A.P - 1) * A.S;
  const int64_t item = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  uint32_t missing = 0;
  if (item < n_items) {
    const int64_t e = item / (A.P - 1);
    const int64_t p = item - e * (A.P - 1);
    const int nl = A.ts.nmap[A.ts.idx(e, p)];
    const int nr = A.ts.nmap[A.ts.idx(e, p + 1)];
    int32_t keys[N];
    keys[0] = A.ts.T0[A.ts.idx(e, p + 1)].a;
#pragma unroll
    for (int m = 1; m < N; ++m) keys[m] = m < nr ? A.ts.at(e, p + 1, m)->a : -1;
    // segment 0 of a stream's batch may hold one tuple more (the carried reset's)
    int32_t exits[N + 1];
    exits[0] = A.ts.T0[A.ts.idx(e, p)].b;
#pragma unroll
    for (int k = 1; k <= N; ++k) exits[k] = k < nl ? A.ts.at(e, p, k)->b : -1;
#pragma unroll
    for (int k = 0; k <= N; ++k) {
      bool hit = false, dup = false;
#pragma unroll
      for (int m = 0; m < N; ++m) hit |= keys[m] == exits[k];
#pragma unroll
      for (int j = 0; j < k; ++j) dup |= exits[j] == exits[k];
      if (k < nl && !hit && !dup) missing |= 1u << k;
    }
    // queue the misses for repair_kernel, which spreads them over every
    // wave; those past the queue's capacity are repaired below
    if (missing != 0u && A.queue_cap > 0) {
      const uint32_t n_m = (uint32_t)__popc(missing);
      const unsigned long long base = atomicAdd(A.queue_n, (unsigned long long)n_m);
      uint32_t left = 0, i = 0;
      for (uint32_t m = missing; m; m &= m - 1, ++i) {
        const int k = __ffs((int)m) - 1;
        if (base + i < (unsigned long long)A.queue_cap)
          A.queue[base + i] = (uint64_t)item << 5 | (uint64_t)k;
        else
          left |= 1u << k;
      }
      missing = left;
    }
    if constexpr (!INLINE) {
      if (missing != 0u) atomicOr(&A.flags[item / (A.P - 1)], 1);
    }
  }
  if constexpr (!INLINE) return;
  uint64_t wmask = __ballot(missing != 0u);
  const int lane = threadIdx.x & (kWave - 1);
  while (wmask != 0) {
    const int src = __ffsll((unsigned long long)wmask) - 1;
    wmask &= wmask - 1;
    const int64_t it = (int64_t)__shfl((long long)item, src);
    uint32_t miss = (uint32_t)__shfl((int)missing, src);
    const int64_t e = it / (A.P - 1);
    const int64_t p = it - e * (A.P - 1);
    typename Mach::Params prm;
    prm.load(A.ep_types, A.ep_lo, A.ep_hi, A.ep_span, e);
    while (miss != 0u) {
      const int k = __ffs((int)miss) - 1;
      miss &= miss - 1;
      repair_exit<N, Mach>(A, prm, e, p, k, lane);
    }
  }
}

// The queued repairs, one at a time per wave, taken in order from a shared
// head: every wave leaves once the head has passed the queue's end.
template <int N, class Mach>
__global__ __launch_bounds__(kBlock) void repair_kernel(ClosureArgs A) {
  const int lane = threadIdx.x & (kWave - 1);
  const unsigned long long n = *A.queue_n;
  const unsigned long long count = n < (unsigned long long)A.queue_cap ? n : (unsigned long long)A.queue_cap;
  if (count == 0) return;  // (no wave touches the head: nothing was queued)
  for (;;) {
    unsigned long long idx = 0;
    if (lane == 0) idx = atomicAdd(A.queue_head, 1ull);
    idx = (unsigned long long)__shfl((long long)idx, 0);
    if (idx >= count) break;
    const uint64_t w = A.queue[idx];
    const int64_t it = (int64_t)(w >> 5);
    const int k = (int)(w & 31u);
    const int64_t e = it / (A.P - 1);
    const int64_t p = it - e * (A.P - 1);
    typename Mach::Params prm;
    prm.load(A.ep_types, A.ep_lo, A.ep_hi, A.ep_span, e);
    repair_exit<N, Mach>(A, prm, e, p, k, lane);
  }
}

// ------------------------------------------------------------- fallback

struct FallbackArgs {
  const int32_t* times;
  const uint16_t* types;
  const uint16_t* ep_types;
  const int32_t* ep_lo;
  const int32_t* ep_hi;
  const int32_t* ep_span;
  const int32_t* flags;
  const Tuple* T0;      // segment 0's first tuple of episode e (at e * P) holds the answer
  int64_t P;
  unsigned long long* fallbacks;
  int64_t* out;
  const int32_t* out_map;  // [S] or null: episode e's count goes to out[out_map[e]]
  int64_t n;
  int64_t S;
  RingArena ring;
};

// Result extraction, one wave per episode.  The answer is the chain entering
// segment 0 through machine 0: segment 0's machines all start before the
// first event, so each is the page's reference machine alpha_0 (Fig. 3 text).
// An episode flagged by a repair-slot overflow or a tree miss is instead
// recounted exactly over the whole stream by the wave (alpha_0 on the
// unsegmented stream).
template <class Mach>
__global__ __launch_bounds__(kBlock) void finish_kernel(FallbackArgs A) {
  const int64_t e = (int64_t)blockIdx.x * (kBlock / kWave) + threadIdx.x / kWave;
  if (e >= A.S) return;
  const bool lane0 = (threadIdx.x & (kWave - 1)) == 0;
  const int64_t oe = A.out_map ? (int64_t)A.out_map[e] : e;
  if (A.flags[e] == 0) {
    if (lane0) A.out[oe] = A.T0[e * A.P].c;
    return;
  }
  typename Mach::Params prm;
  prm.load(A.ep_types, A.ep_lo, A.ep_hi, A.ep_span, e);
  const int64_t before = (int64_t)A.times[0] - 1;
  SegMachine<Mach> sm;
  sm.attach(A.ring, wave_slot());
  sm.init(before, before, INT64_MAX / 4, prm.span);
  wave_feed_range<Mach>(A.times, A.types, 0, A.n, sm, prm);
  if (lane0) {
    A.out[oe] = sm.count;
    atomicAdd(A.fallbacks, 1ull);
  }
}

// ------------------------------------------------ closure + tree + result

// For P <= 512 segments one workgroup per episode does the closure, the
// Concatenate tree and the result extraction in LDS, in one launch:
//   1. thread p loads segment p's tuples;
//   2. thread p checks the exits of segment p's Map tuples against the keys
//      of segment p+1 and queues the misses;
//   3. the waves repair the queued misses: each wave takes its share of the
//      queue and follows each chain at once (a machine reset at the exit
//      over the next segment, again while the new exit finds no key); lane 0
//      reads and appends a segment's LDS list under that segment's LDS lock
//      (one lock held at a time), so the waves of an episode repair in
//      parallel;
//   4. the tree joins the members level by level (Concatenate rules 1-3);
//   5. member 0's first tuple (machine 0 of segment 0, i.e. alpha_0) holds
//      the count.
// An episode flagged by a Map kernel, a repair-list overflow or a tree miss
// is recounted over the whole stream by wave 0, as in finish_kernel.
constexpr int kReduceMembers = 512;
constexpr int kReduceQueue = 256;

struct ReduceArgs {
  ClosureArgs c;
  unsigned long long* fallbacks;
  int64_t* out;
  const int32_t* out_map;  // [S] or null: episode e's count goes to out[out_map[e]]
  int64_t n;
};

template <int N, class Mach>
__global__ __launch_bounds__(kReduceMembers) void reduce_kernel(ReduceArgs A) {
  extern __shared__ __align__(16) unsigned char smem[];
  const TupleStore& ts = A.c.ts;
  const int slots = ts.slots;
  const int members = blockDim.x;
  int32_t* s_a = (int32_t*)smem;  // [members][slots]
  int32_t* s_c = s_a + members * slots;
  int32_t* s_b = s_c + members * slots;
  int32_t* s_n = s_b + members * slots;  // [members] tuples held
  int32_t* s_lock = s_n + members;        // [members] 1 while a wave edits segment p's list
  __shared__ int32_t s_q[kReduceQueue];   // misses, as p * slots + k
  __shared__ int32_t s_nq, s_bad;
  const int64_t e = blockIdx.x;
  const int i = threadIdx.x;
  const int lane = i & (kWave - 1);
  const int wave = i / kWave;
  const int n_waves = members / kWave;
  const int64_t P = A.c.P;
  if (i == 0) {
    s_nq = 0;
    s_bad = A.c.flags[e] != 0 ? 1 : 0;
  }
  int n = 0, nm = 0;
  if (i < P) {
    const int64_t pe = ts.idx(e, i);
    n = min(ts.nslots[pe], slots);
    nm = min(ts.nmap[pe], n);
    for (int k = 0; k < n; ++k) {
      const Tuple tu = *ts.at(e, i, k);
      s_a[i * slots + k] = tu.a;
      s_c[i * slots + k] = tu.c;
      s_b[i * slots + k] = tu.b;
    }
  }
  s_n[i] = n;
  s_lock[i] = 0;
  __syncthreads();
  // closure check: every distinct exit of segment i needs a key in segment i+1
  if (i + 1 < P) {
    const int nr = s_n[i + 1];
    for (int k = 0; k < nm; ++k) {
      const int32_t b = s_b[i * slots + k];
      bool dup = false, hit = false;
      for (int k2 = 0; k2 < k; ++k2) dup |= s_b[i * slots + k2] == b;
      for (int m = 0; m < nr; ++m) hit |= s_a[(i + 1) * slots + m] == b;
      if (!dup && !hit) {
        const int q = atomicAdd(&s_nq, 1);
        if (q < kReduceQueue)
          s_q[q] = i * slots + k;
        else
          s_bad = 1;
      }
    }
  }
  __syncthreads();
  const int nq = min(s_nq, kReduceQueue);
  if (nq > 0 && s_bad == 0) {
    typename Mach::Params prm;
    prm.load(A.c.ep_types, A.c.ep_lo, A.c.ep_hi, A.c.ep_span, e);
    auto lock = [&](int64_t q) {
      while (atomicCAS(&s_lock[q], 0, 1) != 0) {
      }
      __threadfence_block();
    };
    auto unlock = [&](int64_t q) {
      __threadfence_block();
      atomicExch(&s_lock[q], 0);
    };
    auto has_key = [&](int64_t q, int32_t key) {
      bool hit = false;
      for (int m = 0; m < s_n[q]; ++m) hit |= s_a[q * slots + m] == key;
      return hit;
    };
    for (int j = wave; j < nq; j += n_waves) {
      const int item = s_q[j];
      int64_t q = item / slots + 1;
      int32_t x_off = s_b[item];
      for (;;) {
        int go = 0;
        if (lane == 0) {
          if (x_off <= 0) {
            s_bad = 1;  // a sentinel exit always has a sentinel key
          } else {
            lock(q);
            go = has_key(q, x_off) ? 0 : 1;  // another chain may have repaired it
            unlock(q);
          }
        }
        go = __shfl(go, 0);
        if (!go) break;
        const Tuple tu = repair_tuple<Mach>(A.c, prm, e, q, A.c.tau[q] + x_off);
        int next = 0;
        if (lane == 0) {
          lock(q);
          bool added = false;
          if (!has_key(q, tu.a)) {
            const int h = s_n[q];
            if (h >= slots) {
              s_bad = 1;
            } else {
              s_a[q * slots + h] = tu.a;
              s_c[q * slots + h] = tu.c;
              s_b[q * slots + h] = tu.b;
              s_n[q] = h + 1;
              added = true;
              atomicAdd(A.c.repairs, 1ull);
            }
          }
          unlock(q);
          if (added && q + 1 < P) {
            lock(q + 1);
            next = has_key(q + 1, tu.b) ? 0 : 1;
            unlock(q + 1);
          }
        }
        next = __shfl(next, 0);
        if (!next) break;
        x_off = tu.b;
        ++q;
      }
    }
  }
  __syncthreads();
  // the tree
  for (int h = 1; h < members; h <<= 1) {
    if ((i & (2 * h - 1)) == 0 && i + h < P) {
      const int nl = s_n[i];
      const int nr = s_n[i + h];
      for (int k = 0; k < nl; ++k) {
        const int32_t b = s_b[i * slots + k];
        int hit = -1;
        for (int m = 0; m < nr; ++m)
          if (hit < 0 && s_a[(i + h) * slots + m] == b) hit = m;
        if (hit >= 0) {
          s_c[i * slots + k] += s_c[(i + h) * slots + hit];
          s_b[i * slots + k] = s_b[(i + h) * slots + hit];
        } else {
          s_bad = 1;  // a chain the answer may pass through lost its way: recount
        }
      }
    }
    __syncthreads();
  }
  const int64_t oe = A.out_map ? (int64_t)A.out_map[e] : e;
  if (s_bad == 0) {
    if (i == 0) A.out[oe] = s_c[0];
    return;
  }
  if (i >= kWave) return;
  typename Mach::Params prm;
  prm.load(A.c.ep_types, A.c.ep_lo, A.c.ep_hi, A.c.ep_span, e);
  const int64_t before = (int64_t)A.c.times[0] - 1;
  SegMachine<Mach> sm;
  sm.attach(A.c.ring, wave_slot());
  sm.init(before, before, INT64_MAX / 4, prm.span);
  wave_feed_range<Mach>(A.c.times, A.c.types, 0, A.n, sm, prm);
  if (lane == 0) {
    A.out[oe] = sm.count;
    atomicAdd(A.fallbacks, 1ull);
  }
}

// ----------------------------------------------------------- launchers

// Window kinds: run windows with K = 1, 2, 4 runs in registers, bit windows of
// 32 / 64 bits, or ring windows (runs in device memory, any number).
enum WinKind { kRuns1 = 0, kRuns2 = 1, kRuns4 = 2, kBits32 = 3, kBits64 = 4, kRing = 5, kNumWin = 6 };

// Per-N entry points, defined in ep_inst.hip (one translation unit per N).
// ------------------------------------------------------------- streaming

// Counting a stream that arrives in batches.  Between calls the stream
// carries the events within maxSpan (the table's largest Span) of the last
// event seen so far, time T (the halo: times >= T - maxSpan), which the next
// call counts again in front of its new events, and each episode carries the
// time r of the last completion of its reference machine alpha_0 when r lies
// in the halo (kNoReset otherwise).  An occurrence completing after T starts
// no earlier than T - Span, so alpha_0 after T behaves like a machine reset
// at r fed the halo and the new events.  With no r in the halo, alpha_0's
// last reset is older than every halo event, so a fresh machine fed the halo
// sees a subset of alpha_0's events and completes nowhere in it (alpha_0
// would have completed too), and after T it completes where alpha_0 does.
// (An r older than Span but inside the halo must be carried: a fresh machine
// could complete at r again.)  Over the combined events:
//   - stream_entry_kernel adds to segment 0 the tuple of a machine reset at r
//     (a repair-style tuple: its count includes the completion at r, counted
//     by the earlier call, which the tail takes off again);
//   - the tree joins segments 0 .. P-2 only;
//   - stream_tail_kernel follows the chain from segment 0 to the last segment
//     and runs it there with one wave to the last event, which gives the
//     count of this call and the new r.  Segments are planned more than
//     maxSpan ticks long, so every completion in the next halo lies in the
//     last segment.
constexpr int64_t kNoReset = INT64_MIN;

struct StreamArgs {
  ClosureArgs c;          // the call's events (halo + batch), table, cuts, tuples, flags
  const int64_t* entry;   // [S] carried reset times (kNoReset: none)
  int64_t* total;         // [S] running counts; this call's completions are added
  int64_t* reset_out;     // [S] reset time to carry into the next call
  int64_t n;              // events of the call
  int64_t t_end;          // time of its last event
  int64_t max_span;       // the table's largest Span (the halo width)
};

// One wave per episode: the tuple of a machine reset at the carried r, added
// to segment 0 after the Map tuples (before the closure checks its exit).
template <int N, class Mach>
__global__ __launch_bounds__(kBlock) void stream_entry_kernel(StreamArgs A) {
  const int64_t e = (int64_t)blockIdx.x * (kBlock / kWave) + threadIdx.x / kWave;
  if (e >= A.c.S) return;
  const int64_t x = A.entry[e];
  if (x == kNoReset) return;
  const bool lane0 = (threadIdx.x & (kWave - 1)) == 0;
  typename Mach::Params prm;
  prm.load(A.c.ep_types, A.c.ep_lo, A.c.ep_hi, A.c.ep_span, e);
  const Tuple tu = repair_tuple<Mach>(A.c, prm, e, 0, x);
  if (!lane0) return;
  const TupleStore& ts = A.c.ts;
  const int64_t pe = ts.idx(e, 0);
  const int nm = ts.nmap[pe];
  for (int m = 0; m < nm; ++m)
    if (ts.at(e, 0, m)->a == tu.a) return;  // an equal key: the same chain
  if (nm >= ts.slots) {
    atomicOr(&A.c.flags[e], 1);
    return;
  }
  *ts.at(e, 0, nm) = tu;
  ts.nmap[pe] = nm + 1;
  ts.nslots[pe] = nm + 1;
}

// One wave per episode: this call's count and the reset time to carry.
template <int N, class Mach>
__global__ __launch_bounds__(kBlock) void stream_tail_kernel(StreamArgs A) {
  const int64_t e = (int64_t)blockIdx.x * (kBlock / kWave) + threadIdx.x / kWave;
  if (e >= A.c.S) return;
  const bool lane0 = (threadIdx.x & (kWave - 1)) == 0;
  const TupleStore& ts = A.c.ts;
  const int64_t x = A.entry[e];
  const int64_t P = A.c.P;
  const int64_t tau0 = A.c.tau[0];
  typename Mach::Params prm;
  prm.load(A.c.ep_types, A.c.ep_lo, A.c.ep_hi, A.c.ep_span, e);
  // the chain through segments 0 .. P-2 (joined by the tree)
  bool whole = A.c.flags[e] != 0 || P == 1;
  int64_t cnt = 0, reset_t = 0, last = kNoReset, i0 = 0;
  if (!whole) {
    const int ns = min(ts.nslots[ts.idx(e, 0)], ts.slots);
    int hit = -1;
    if (x == kNoReset) {
      hit = 0;  // machine 0 of segment 0: alpha_0 from the first event
    } else {
      const int32_t key = (int32_t)(x - tau0);
      for (int m = 0; m < ns; ++m)
        if (hit < 0 && ts.at(e, 0, m)->a == key) hit = m;
    }
    if (hit < 0) {
      whole = true;
    } else {
      const Tuple tu = *ts.at(e, 0, hit);
      const int64_t cut = A.c.tau[P - 1];
      cnt = (int64_t)tu.c - (x == kNoReset ? 0 : 1);
      if (tu.b > 0) {
        reset_t = cut + tu.b;  // the chain's first completion in the last segment
        cnt += 1;
        last = reset_t;
      } else {
        reset_t = cut;  // no completion within Span of the cut: a fresh machine there
      }
      i0 = upper_bound_time(A.c.times, A.c.seg_beg[P - 1], A.n, reset_t);
    }
  }
  if (whole) {
    // one segment, or an episode the tree could not join: the whole call
    reset_t = x == kNoReset ? tau0 : x;
    cnt = 0;
    last = kNoReset;
    i0 = upper_bound_time(A.c.times, 0, A.n, reset_t);
  }
  SegMachine<Mach> sm;
  sm.attach(A.c.ring, wave_slot());
  sm.init(reset_t, reset_t, A.t_end, prm.span);
  wave_feed_range<Mach>(A.c.times, A.c.types, i0, A.n, sm, prm);
  if (!lane0) return;
  cnt += sm.count;
  if (sm.count > 0) last = sm.last;
  // the reset to carry if it lies in the next halo (times >= t_end - maxSpan)
  int64_t carry = kNoReset;
  if (last != kNoReset) {
    if (last >= A.t_end - A.max_span) carry = last;
  } else if (cnt == 0 && x != kNoReset && x >= A.t_end - A.max_span) {
    carry = x;  // no completion in this call: the carried reset still holds
  }
  A.total[e] += cnt;
  A.reset_out[e] = carry;
}

struct Launchers {
  // scan Map kernel (run windows; win must be a run or ring kind)
  hipError_t (*map_scan)(const MapArgs&, int win, dim3 grid, dim3 block, hipStream_t);
  // bit Map kernel (win must be a bit kind); all_machines: one lane holds N machines
  hipError_t (*map_bits)(const MapArgs&, int win, bool all_machines, dim3 grid, dim3 block,
                         size_t lds, hipStream_t);
  // tick Map kernel (bit windows up to 63 ticks)
  hipError_t (*map_ticks)(const MapArgs&, bool all_machines, dim3 grid, dim3 block, size_t lds,
                          hipStream_t);
  // list Map kernel (win must be a bit kind); reads the filter kernel's lists
  hipError_t (*map_list)(const MapArgs&, int win, bool all_machines, dim3 grid, dim3 block,
                         hipStream_t);
  hipError_t (*closure)(const ClosureArgs&, int win, dim3 grid, hipStream_t);
  hipError_t (*finish)(const FallbackArgs&, int win, dim3 grid, hipStream_t);
  // closure + tree + result in one launch for P <= kReduceMembers
  hipError_t (*reduce)(const ReduceArgs&, int win, dim3 grid, dim3 block, size_t lds, hipStream_t);
  // streaming: the carried reset's tuple in segment 0, and the chain's tail
  hipError_t (*stream_entry)(const StreamArgs&, int win, dim3 grid, hipStream_t);
  hipError_t (*stream_tail)(const StreamArgs&, int win, dim3 grid, hipStream_t);
  // resident workgroups per CU of a Map kernel for a block size and LDS size
  hipError_t (*occupancy)(int win, bool all_machines, int block, size_t lds, int* blocks_per_cu);
  // the same for the tick Map kernel
  hipError_t (*occupancy_ticks)(bool all_machines, int block, size_t lds, int* blocks_per_cu);
};

}  // namespace epk
