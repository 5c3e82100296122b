// Device kernels of the library that are not specialised per episode size:
// the per-call set-up (cuts and segment ranges), the event filter of the list
// path, the Concatenate tree, and small helpers (fill, the two-pass scatter,
// the sortedness check).  Included once, by the host unit ep_api.hip.
//
// Source page: "Towards Chip-on-Chip Neuroscience: Fast Mining of Frequent
// Episodes Using Graphics Processors".
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ep_device.hpp"

namespace epk {
namespace {
// ------------------------------------------------------------ small kernels

// Per-call set-up in one launch: the equal-time cuts with each segment's event
// range, and the flag and counter words.
//   cuts   : tau_p = t_min - 1 + floor(p (t_max - t_min + 1) / P) for p = 0..P
//            ("Design of MapConcatenate": segment p holds (tau_p, tau_{p+1}]);
//            segment p needs the events in (tau_p - maxSpan, tau_{p+1} + maxSpan]
//            since its machines start up to maxSpan before the left cut and
//            look up to maxSpan past the right cut for the exit b.
// With few segments each range end is one wave's 64-ary search of the sorted
// times (a handful of dependent loads instead of a binary search's log2 n);
// with many, the searches alone fill the GPU and each is one thread's binary
// search (fewer loads in all).
struct SetupArgs {
  const int32_t* times;
  int64_t n;
  int32_t P;
  int64_t max_span;
  int64_t* tau;
  int32_t* beg;
  int32_t* end;
  int32_t* flags;  // [S + 1]
  int32_t flag_init;  // episodes' flags start at this (1: every episode takes the whole-stream recount)
  int64_t S;
  unsigned long long* counters;  // [4]
  int32_t wave_search;  // range ends by one wave each (small P) or kSearchLanes lanes each
  const uint4* tab_src;  // the episode table in pinned host memory (device-visible)
  uint4* tab_dst;        // its device copy
  int64_t tab_words;     // 16-byte words
};

__device__ inline int64_t cut_of(int64_t t_min, int64_t t_max, int64_t p, int64_t P) {
  return t_min - 1 + (p * (t_max - t_min + 1)) / P;
}

// First index i in [0, n) with times[i] > v, n if none, found by the G lanes
// of an aligned group of a wave (G a power of two up to the wave size), every
// lane of the group calling it with the same v and getting the answer.  Each
// level probes G evenly spaced elements of the range and keeps the part
// before the first one above v: about log_G(n) dependent loads.  Invariant:
// the answer lies in [lo, hi], times[lo-1] <= v and times[hi] > v (or hi = n).
// Groups of one wave may leave the loop at different levels: a ballot counts
// the active lanes only, and each group reads its own bits.
template <int G>
__device__ int64_t group_upper_bound(const int32_t* times, int64_t n, int64_t v) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gl = lane & (G - 1);  // lane in the group
  const int gb = lane - gl;       // the group's first lane
  const uint64_t mask = (G == kWave) ? ~0ull : (((1ull << G) - 1ull) << gb);
  int64_t lo = 0, hi = n;
  while (hi - lo > G) {
    const int64_t step = (hi - lo + G - 1) / G;
    int64_t idx = lo + (int64_t)(gl + 1) * step - 1;
    idx = idx < hi - 1 ? idx : hi - 1;
    const uint64_t gt = (__ballot((int64_t)times[idx] > v) & mask) >> gb;
    if (gt == 0) {
      lo = hi;  // the group's last lane probed hi - 1
    } else {
      const int f = __ffsll((unsigned long long)gt) - 1;
      const int64_t idx_f = lo + (int64_t)(f + 1) * step - 1;
      const int64_t new_lo = f == 0 ? lo : lo + (int64_t)f * step;
      hi = idx_f < hi - 1 ? idx_f : hi - 1;
      lo = new_lo;
    }
  }
  const int64_t idx = lo + gl;
  const bool in = idx < hi;  // lanes past the range read times[0] (n >= 1) and ignore it
  const uint64_t gt = (__ballot(in && (int64_t)times[in ? idx : 0] > v) & mask) >> gb;
  return gt ? lo + (__ffsll((unsigned long long)gt) - 1) : hi;
}

// Segment range ends: a wave per search for few segments, groups of
// kSearchLanes lanes beyond (as many groups as keep the whole search one round
// of resident waves on the largest segment counts)
constexpr int32_t kWaveSearchMaxP = 4096;
constexpr int kSearchLanes = 4;

__host__ __device__ inline int64_t setup_search_threads(int32_t P, bool wave) {
  return (int64_t)2 * P * (wave ? kWave : kSearchLanes);
}

__global__ __launch_bounds__(kBlock) void setup_kernel(SetupArgs A) {
  int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t n_search = setup_search_threads(A.P, A.wave_search != 0);
  if (i < n_search) {
    // lane group w (a wave, or kSearchLanes lanes): w even -> beg[w / 2], w odd
    // -> end[w / 2] (whole groups: n_search is a multiple of the group size,
    // and the other lanes of a partly searching wave do other items)
    const int G = A.wave_search ? kWave : kSearchLanes;
    const int64_t w = i / G;
    const int64_t p = w >> 1;
    const int64_t t_min = A.times[0];
    const int64_t t_max = A.times[A.n - 1];
    const int64_t v = (w & 1) ? cut_of(t_min, t_max, p + 1, A.P) + A.max_span
                              : cut_of(t_min, t_max, p, A.P) - A.max_span;
    const int64_t r = A.wave_search ? group_upper_bound<kWave>(A.times, A.n, v)
                                    : group_upper_bound<kSearchLanes>(A.times, A.n, v);
    if ((threadIdx.x & (G - 1)) == 0) {
      if (w & 1)
        A.end[p] = (int32_t)r;
      else
        A.beg[p] = (int32_t)r;
    }
    return;
  }
  i -= n_search;
  if (i <= A.P) {
    A.tau[i] = cut_of(A.times[0], A.times[A.n - 1], i, A.P);
    return;
  }
  i -= (int64_t)A.P + 1;
  if (i <= A.S) {
    A.flags[i] = i < A.S ? A.flag_init : 0;
    return;
  }
  i -= A.S + 1;
  if (i < 4) {
    A.counters[i] = 0ull;
    return;
  }
  i -= 4;
  // the episode table: read from pinned host memory over the bus, so no copy
  // engine sits between the host and this launch
  if (i < A.tab_words) A.tab_dst[i] = A.tab_src[i];
}

// ------------------------------------------------------------- event filter

// One pass over the stream for the list Map kernel.  Block b holds events
// [b * kListBlock, (b + 1) * kListBlock); each event gets its node-type slot
// and the set of episodes with that type, and for each episode its events are
// written in order to the block's region as {time, node levels | e << 16}
// (the Map kernels read only the level bits, 0..15): episode e's
// entries start at list_off[b][e] and number list_cnt[b][e].  The region holds
// kListBlock * max_share entries (max_share: most episodes one type is on), so
// blocks need nothing from each other.  A thread takes 16 consecutive events;
// its per-episode counts are packed two to a 32-bit word (16-bit fields; a
// block holds at most 4096), so one scan serves two episodes.  Where every
// node type is below kFilterTab, a byte table maps types to slots directly;
// otherwise the 65,536-bit set of node types and per-word ranks do.
constexpr int kFilterPer = kListBlock / kBlock;  // 16
constexpr int kFilterTab = 9216;                  // LDS bytes of the type table
constexpr int kMaxListEpisodes = 32;
constexpr double kMaxListBytes = 32.0 * (1ull << 30);  // list scratch bound of the list path

struct FilterArgs {
  const int32_t* times;
  const uint16_t* types;
  int64_t n;
  const uint64_t* type_seen;     // [1024] the call's node types as a 65,536-bit set
  const uint8_t* type_rank;      // [1024] set bits before each 64-bit word
  const uint32_t* slot_eps;      // [256] episodes with slot u's type (bit e); slot 0: none
  const uint16_t* slot_levels;   // [256 * S] node levels of episode e with slot u's type
  int32_t S;                     // <= kMaxListEpisodes
  int32_t max_share;
  int32_t type_cap;              // node types are below this (direct table when <= kFilterTab)
  int2* lists;
  int32_t* list_off;             // [blocks * S]
  int32_t* list_cnt;             // [blocks * S]
};

// One workgroup loops over blocks b = blockIdx.x, + gridDim.x, ...: the LDS
// tables are loaded once, and the next block's events are loaded before the
// current block is classified and written.  G packed count words serve up to
// 4 G episodes.  A thread keeps its events in LDS ([k][thread]) so that the
// write loop visits only its events of node types, in order.
template <int G, bool DIRECT>
__global__ __launch_bounds__(kBlock) void filter_kernel(FilterArgs A) {
  constexpr int kE = 4 * G;  // episodes this instance serves at most
  __shared__ __align__(8) uint8_t s_tab[kFilterTab];  // type -> slot, or the set + ranks
  uint64_t* s_seen = (uint64_t*)s_tab;
  uint8_t* s_rank = s_tab + 8192;
  __shared__ int32_t s_st[kFilterPer][kBlock];       // thread's event k: time
  __shared__ uint32_t s_ss[kFilterPer / 4][kBlock];  // and slot (a byte of word k / 4)
  __shared__ uint32_t s_eps[256];
  __shared__ uint16_t s_lv[256 * kE];
  __shared__ uint16_t s_pre[kE][kBlock];  // thread's next rank per episode
  __shared__ uint32_t s_wsum[kBlock / kWave][2 * G];
  __shared__ int32_t s_off[kE];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int S = A.S;
  if (DIRECT) {
    for (int i = tid; i < A.type_cap; i += kBlock)
      s_tab[i] = (uint8_t)type_slot(A.type_seen, A.type_rank, (uint32_t)i);
  } else {
    for (int i = tid; i < 1024; i += kBlock) {
      s_seen[i] = A.type_seen[i];
      s_rank[i] = A.type_rank[i];
    }
  }
  for (int i = tid; i < 256; i += kBlock) s_eps[i] = A.slot_eps[i];
  for (int i = tid; i < 256 * S; i += kBlock) s_lv[(i / S) * kE + i % S] = A.slot_levels[i];
  const bool vec = ((uintptr_t)A.times & 15) == 0 && ((uintptr_t)A.types & 15) == 0;
  const int64_t n_blocks = (A.n + kListBlock - 1) / kListBlock;

  int32_t t[kFilterPer], tn[kFilterPer];
  uint32_t y[kFilterPer], yn[kFilterPer];
  auto load = [&](int64_t b, int32_t* tt, uint32_t* yy) {
    const int64_t first = b * kListBlock + (int64_t)tid * kFilterPer;
    if (vec && first + kFilterPer <= A.n) {
      const int4* tv = (const int4*)(A.times + first);
      const uint4* yv = (const uint4*)(A.types + first);
#pragma unroll
      for (int q = 0; q < kFilterPer / 4; ++q) {
        const int4 v = tv[q];
        tt[4 * q] = v.x;
        tt[4 * q + 1] = v.y;
        tt[4 * q + 2] = v.z;
        tt[4 * q + 3] = v.w;
      }
#pragma unroll
      for (int q = 0; q < kFilterPer / 8; ++q) {
        const uint4 v = yv[q];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          yy[8 * q + 2 * h] = w[h] & 0xffffu;
          yy[8 * q + 2 * h + 1] = w[h] >> 16;
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < kFilterPer; ++k) {
        const bool in = first + k < A.n;
        tt[k] = in ? A.times[first + k] : 0;
        yy[k] = in ? A.types[first + k] : 0u;
      }
    }
  };
  int64_t b = blockIdx.x;
  if (b < n_blocks) load(b, tn, yn);
  lds_barrier();  // tables in LDS

  for (; b < n_blocks; b += gridDim.x) {
    const int64_t first = b * kListBlock + (int64_t)tid * kFilterPer;
#pragma unroll
    for (int k = 0; k < kFilterPer; ++k) {
      t[k] = tn[k];
      y[k] = yn[k];
    }
    if (b + gridDim.x < n_blocks) load(b + gridDim.x, tn, yn);  // in flight meanwhile

    // events of this thread that exist (the last block may be partial)
    const int64_t left = A.n - first;
    const int n_valid = left >= kFilterPer ? kFilterPer : (left > 0 ? (int)left : 0);
    // per-thread counts in 8-bit fields, four episodes to a word (at most 16
    // each): x * 0x204081 puts bit i of a 4-bit x at bit 8i with no carries
    uint32_t c8[G];
    uint32_t rel = 0;  // bit k: event k has a node type
#pragma unroll
    for (int g = 0; g < G; ++g) c8[g] = 0;
#pragma unroll
    for (int k = 0; k < kFilterPer; ++k) {
      const uint32_t yk = y[k];
      uint32_t u;
      if (DIRECT) {
        u = (k < n_valid && yk < (uint32_t)A.type_cap) ? (uint32_t)s_tab[yk] : 0u;
      } else {
        const uint64_t w = s_seen[yk >> 6];
        const uint32_t sh = yk & 63u;
        const bool on = k < n_valid && ((w >> sh) & 1ull);
        const uint32_t below = (uint32_t)__popcll(w & ((1ull << sh) - 1ull));
        u = on ? (uint32_t)s_rank[yk >> 6] + below + 1u : 0u;
      }
      const uint32_t ep = s_eps[u];
      rel |= (u != 0u ? 1u : 0u) << k;
#pragma unroll
      for (int g = 0; g < G; ++g) c8[g] += __umul24((ep >> (4 * g)) & 15u, 0x204081u) & 0x01010101u;
      s_st[k][tid] = t[k];
      if ((k & 3) == 0)
        s_ss[k / 4][tid] = u;
      else
        s_ss[k / 4][tid] |= u << (8 * (k & 3));
    }
    // widen to two 16-bit fields per word: word 2g + h holds episodes 4g + 2h
    // and 4g + 2h + 1
    uint32_t c[2 * G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      c[2 * g] = (c8[g] & 0xffu) | ((c8[g] & 0xff00u) << 8);
      c[2 * g + 1] = ((c8[g] >> 16) & 0xffu) | ((c8[g] >> 24) << 16);
    }
    // block-wide exclusive scan of the packed counts: wave scan, then waves
    uint32_t incl[2 * G];
#pragma unroll
    for (int g = 0; g < 2 * G; ++g) {
      incl[g] = wave_incl_scan(c[g]);
      if (lane == kWave - 1) s_wsum[wave][g] = incl[g];
    }
    lds_barrier();
#pragma unroll
    for (int g = 0; g < 2 * G; ++g) {
      uint32_t before = 0;
#pragma unroll
      for (int w = 0; w < kBlock / kWave; ++w) before += w < wave ? s_wsum[w][g] : 0u;
      const uint32_t excl = before + incl[g] - c[g];
      if (2 * g < S) s_pre[2 * g][tid] = (uint16_t)(excl & 0xffffu);
      if (2 * g + 1 < S) s_pre[2 * g + 1][tid] = (uint16_t)(excl >> 16);
    }
    if (tid == 0) {
      int32_t off = 0;
#pragma unroll
      for (int g = 0; g < 2 * G; ++g) {
        uint32_t all = 0;
#pragma unroll
        for (int w = 0; w < kBlock / kWave; ++w) all += s_wsum[w][g];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int e = 2 * g + h;
          if (e < S) {
            const int32_t cnt = (int32_t)((all >> (16 * h)) & 0xffffu);
            s_off[e] = off;
            A.list_off[b * S + e] = off;
            A.list_cnt[b * S + e] = cnt;
            off += cnt;
          }
        }
      }
    }
    lds_barrier();
    int2* region = A.lists + b * (int64_t)kListBlock * A.max_share;
    // this thread's events of node types, in order, from its LDS copy
    while (rel) {
      const int k = __ffs((int)rel) - 1;
      rel &= rel - 1;
      const int32_t tk = s_st[k][tid];
      const uint32_t u = (s_ss[k >> 2][tid] >> (8 * (k & 3))) & 0xffu;
      uint32_t m = s_eps[u];
      while (m) {
        const int e = __ffs((int)m) - 1;
        m &= m - 1;
        const uint16_t r = s_pre[e][tid];
        s_pre[e][tid] = (uint16_t)(r + 1);
        region[s_off[e] + r] = make_int2(tk, (int32_t)((uint32_t)s_lv[u * kE + e] | (uint32_t)e << 16));
      }
    }
    lds_barrier();  // s_wsum, s_pre, s_off, s_st and s_ss are rewritten by the next block
  }
}

// ------------------------------------------------------------- list pruning

// Leaves out of the filter's lists the entries that cannot change what the
// counting machines output.  An event of node j's type acts only through a
// node-j candidate: for j > 0 it becomes one only if a node j-1 candidate
// lies in [t - hi_{j-1}, t - lo_{j-1} - 1], and node j-1 candidates are
// events of node j-1's type, which sit in the same episode's list with bit
// j-1 in their levels; for j < N-1 the candidate is used only by an event of
// node j+1's type in [t + lo_j + 1, t + hi_j].  An entry with no such
// neighbour is dropped: the machines' windows age by elapsed time, not by
// entries, and every completion and reset happens at an entry that stays.
// Each side is decided by the two entries of the list nearest on that side
// (a list is sorted by time, so an entry past the range means every further
// one is too): the side has the neighbour when the nearest is a match, and
// counts as undecided, so kept, when the second nearest still lies within
// the range; an entry with no list entry on a side, or with both past the
// range or failing it, has none there.  A range the block may not hold whole
// (not strictly between its first and last time) and an entry on several
// levels count as having the neighbour.  Times are compared by difference
// in 32 bits: blocks spanning 2^30 ticks or more are left as they are, and
// so is a block with more than kPruneCap entries.
//
// Persistent workgroups loop over blocks, a block's lists read into
// registers one iteration ahead and copied to LDS.  Entry i is tested by
// thread i mod 256, it and its neighbours read from LDS (list membership by
// the episode field the filter writes in bits 16.., two sentinels before the
// block's entries and two after them); a ballot per 64 entries gives the
// kept entries' ranks, and each kept entry is written back in place at its
// rank, consecutive threads to consecutive slots.  Each list's new offset
// is the rank of its first entry.  Two workgroup barriers per block.  Each
// thread copies the next block's entries, and the sentinels after them, into
// LDS slots that no other thread reads after this block's second barrier;
// the ballot words are rewritten only after the next block's first.
constexpr int kPruneCap = 2048;                  // entries a block may have to be pruned
constexpr int kPrunePer = kPruneCap / kBlock;    // entries per thread
constexpr int kPruneWords = kPruneCap / kWave;   // ballot words per block
constexpr int kPruneIv = 16;                     // interval words per episode (slot j: interval j-1)

struct PruneArgs {
  const int32_t* times;
  int64_t n;
  int64_t n_blocks;
  const int32_t* ep_lo;  // [S * (N - 1)] delay intervals (lo, hi], hi <= 64
  const int32_t* ep_hi;
  int32_t S;
  int32_t N;
  int32_t max_share;
  int2* lists;
  int32_t* list_off;     // [blocks * S]
  int32_t* list_cnt;     // [blocks * S]
};

__global__ __launch_bounds__(kBlock) void list_prune_kernel(PruneArgs A) {
  __shared__ int2 s_e[kPruneCap + 4];              // entry i at s_e[i + 2]; 0, 1: sentinels
  __shared__ uint32_t s_iv[kMaxListEpisodes * kPruneIv + 1];
  __shared__ uint64_t s_bal[kPruneWords + 1];     // kept entries 64 w .. 64 w + 63
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int S = A.S, N = A.N;
  // interval j-1 of episode e in slot e * kPruneIv + j: lo + 1, hi - lo and
  // hi, one byte each (slot 0 unused: node 0 has no predecessor; the slot
  // after node N-1's is read for its successor side and not used)
  for (int i = tid; i < S * kPruneIv; i += kBlock) {
    const int e = i / kPruneIv, k = i - e * kPruneIv;
    uint32_t v = 0;
    if (k >= 1 && k <= N - 1) {
      const int32_t lo = A.ep_lo[e * (N - 1) + k - 1], hi = A.ep_hi[e * (N - 1) + k - 1];
      v = (uint32_t)(lo + 1) | (uint32_t)(hi - lo) << 8 | (uint32_t)hi << 16;
    }
    s_iv[i] = v;
  }
  const int2 sentinel = make_int2(0, (int32_t)0xffff0000u);  // episode field in no list
  if (tid < 2) s_e[tid] = sentinel;
  const int64_t grid = gridDim.x;
  // the lists lie one after the other from the region's start, episode by
  // episode: a block's entries are its last list's offset plus count (kept
  // apart until used, so that loading them waits for nothing)
  auto total_of = [&](int64_t bb) -> int2 {
    return bb < A.n_blocks ? make_int2(A.list_off[bb * S + S - 1], A.list_cnt[bb * S + S - 1]) : make_int2(0, 0);
  };
  int2 ent[kPrunePer] = {};
  int32_t off_r = 0, tf_r = 0, tl_r = 0;
  // block bb's entries (entry tid + q * kBlock in ent[q]), offsets and ends
  auto fetch = [&](int64_t bb, int32_t tot) {
    const int2* region = A.lists + bb * (int64_t)kListBlock * A.max_share;
    const bool run = tot > 0 && tot <= kPruneCap;
#pragma unroll
    for (int q = 0; q < kPrunePer; ++q) {
      const int i = tid + q * kBlock;
      if (run && i < tot) ent[q] = region[i];  // (the others are never read)
    }
    off_r = tid < S ? A.list_off[bb * S + tid] : 0;
    tf_r = A.times[bb * kListBlock];
    tl_r = A.times[min(A.n, (bb + 1) * (int64_t)kListBlock) - 1];
  };
  int64_t b = blockIdx.x;
  const int2 t0 = total_of(b);
  int32_t tot = __builtin_amdgcn_readfirstlane(t0.x + t0.y);
  int2 tot_next = total_of(b + grid);
  if (b < A.n_blocks) fetch(b, tot);

  for (; b < A.n_blocks; b += grid) {
    const int32_t total = tot;
    const int32_t tf = tf_r;
    const int32_t off = off_r;
    const int64_t span64 = (int64_t)tl_r - (int64_t)tf_r;
    const int32_t span = (int32_t)span64;
    const bool run = total > 0 && total <= kPruneCap && span64 >= 0 && span64 < (1ll << 30);
    if (run) {
#pragma unroll
      for (int q = 0; q < kPrunePer; ++q) {
        const int i = tid + q * kBlock;
        if (q * kBlock < total + 2) {
          if (i < total)
            s_e[i + 2] = ent[q];
          else if (i < total + 2)
            s_e[i + 2] = sentinel;
        }
      }
      // (sentinels past the last thread's slots: entries kPruneCap, kPruneCap + 1)
      if (tid < 2 && kPruneCap + tid < total + 2) s_e[kPruneCap + 2 + tid] = sentinel;
    }
    // the next block's loads in flight meanwhile
    tot = __builtin_amdgcn_readfirstlane(tot_next.x + tot_next.y);
    if (b + grid < A.n_blocks) fetch(b + grid, tot);
    tot_next = total_of(b + 2 * grid);
    if (!run) continue;
    lds_barrier();

    // entries tid, tid + kBlock, ...: which of them pass
#pragma unroll
    for (int q = 0; q < kPrunePer; ++q) {
      if (q * kBlock < total) {
        const int i = tid + q * kBlock;
        const int2 me = s_e[i + 2];
        const uint32_t y = (uint32_t)me.y;
        const uint32_t lm = y & 0xffffu;
        const uint32_t e = y >> 16;
        // every read below stays inside the arrays for any lane (a lane past
        // the block's entries reads stale slots and keeps nothing), and the
        // conditions are combined without branches, so that the LDS reads go
        // out together
        const int j = __builtin_ctz(lm | 0x8000u);  // the entry's level, if single
        const int ie = (int)(min(e, (uint32_t)S - 1u) * kPruneIv) + j;
        const uint32_t ivp = s_iv[ie], ivs = s_iv[ie + 1];
        const int2 p1 = s_e[i + 1], p2 = s_e[i], s1 = s_e[i + 3], s2 = s_e[i + 4];
        const int32_t tr = (int32_t)((uint32_t)me.x - (uint32_t)tf);  // 0 .. span
        // predecessor side: a node j-1 entry at distance (lo, hi] before
        const uint32_t dp1 = (uint32_t)me.x - (uint32_t)p1.x, dp2 = (uint32_t)me.x - (uint32_t)p2.x;
        const bool p_hit = (((uint32_t)p1.y >> 16) == e) & (((uint32_t)p1.y & (lm >> 1)) != 0u) &
                           (dp1 - (ivp & 0xffu) < ((ivp >> 8) & 0xffu));
        const bool p_open = (((uint32_t)p2.y >> 16) == e) & ((int32_t)dp2 <= (int32_t)(ivp >> 16));
        const bool p_ok = (j == 0) | (tr <= (int32_t)(ivp >> 16)) | p_hit | p_open;
        // successor side: a node j+1 entry at distance (lo, hi] after
        const uint32_t ds1 = (uint32_t)s1.x - (uint32_t)me.x, ds2 = (uint32_t)s2.x - (uint32_t)me.x;
        const bool s_hit = (((uint32_t)s1.y >> 16) == e) & (((uint32_t)s1.y & (lm << 1)) != 0u) &
                           (ds1 - (ivs & 0xffu) < ((ivs >> 8) & 0xffu));
        const bool s_open = (((uint32_t)s2.y >> 16) == e) & ((int32_t)ds2 <= (int32_t)(ivs >> 16));
        const bool s_ok = (j >= N - 1) | (tr + (int32_t)(ivs >> 16) >= span) | s_hit | s_open;
        // several levels (or none): kept
        bool keep = ((lm & (lm - 1u)) != 0u) | (lm == 0u) | (p_ok & s_ok);
        keep = keep && i < total;
        const uint64_t bal = __ballot(keep);
        if (lane == 0) s_bal[q * (kBlock / kWave) + wave] = bal;
      }
    }
    lds_barrier();

    // ranks: kept entries in the ballot words before this one, plus the
    // lanes below in it
    const int n_words = (total + kWave - 1) / kWave;
    const uint64_t wv = lane < n_words ? s_bal[lane] : 0ull;
    const uint32_t wc = (uint32_t)__popcll(wv);
    const uint32_t before = wave_incl_scan(wc) - wc;
    int2* region = A.lists + b * (int64_t)kListBlock * A.max_share;
#pragma unroll
    for (int q = 0; q < kPrunePer; ++q)
      if (q * kBlock < total) {
        const int w = q * (kBlock / kWave) + wave;
        const uint32_t base = __builtin_amdgcn_readlane(before, w);
        const uint64_t bal = s_bal[w];  // (one address for the wave)
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        if ((bal >> lane) & 1ull) region[base + below] = s_e[tid + q * kBlock + 2];
      }
    if (wave == 0) {
      // each list's new offset and count: the ranks of its first entry and of
      // the next list's (lists are consecutive; S <= 32 lanes of wave 0)
      const int32_t nxt = __shfl_down(off, 1);
      const int32_t end = tid == S - 1 ? total : nxt;
      auto rank = [&](int32_t x) -> int32_t {
        const int w = x >> 6, l = x & (kWave - 1);
        const uint32_t base = (uint32_t)__shfl((int)before, w);
        const uint64_t ww = (uint64_t)(uint32_t)__shfl((int)(uint32_t)wv, w) |
                            (uint64_t)(uint32_t)__shfl((int)(uint32_t)(wv >> 32), w) << 32;
        return (int32_t)(base + (uint32_t)__popcll(ww & ((1ull << l) - 1ull)));
      };
      const int32_t a0 = rank(off), z = rank(end);
      if (tid < S) {
        A.list_off[b * S + tid] = a0;
        A.list_cnt[b * S + tid] = z - a0;
      }
    }
  }
}

// ------------------------------------------------------------- Concatenate

// One workgroup joins `members` consecutive members (segments p0, p0 +
// stride, ...) of one episode (Concatenate rules 1-3, Fig. 6) and writes the
// merged tuples back to the first member.  Members hold their tuple list keyed
// by their first segment's keys; joining left block L with right block R maps
// each (a, c, b) of L to (a, c + c', b') for the tuple of R whose key a'
// equals b (no such tuple: a miss, flagged for the episode).  Launched with
// stride 1, then `members`, then members^2, ..., until one member is left.
//
// Thread t first joins members t * per .. t * per + per - 1 in order (their
// first tuples and tuple counts loaded together up front: with stride 1 that
// is one contiguous read per thread), then the threads' lists are joined
// level by level in LDS.  Where the launch has threads to spare (many
// episodes), per = 4 makes a 512-member group two waves: a chain of four
// dependent joins per thread, then seven tree levels, instead of nine
// workgroup barriers over 512 threads (per = 8, one wave, makes the chains of
// joins the longer wait; per = 2 leaves more barriers).
constexpr int kConcatMembers = 512;  // members of a tree workgroup at most
constexpr int kConcatPer = 4;        // members one thread joins in order at most
constexpr int64_t kConcatMinThreads = 65536;  // threads a launch keeps when choosing per

__global__ __launch_bounds__(kConcatMembers) void concat_tree_kernel(TupleStore ts, int32_t* flags, int64_t S,
                                                             int32_t P, int64_t stride, int32_t members,
                                                             int64_t groups, int32_t per) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int slots = ts.slots;
  const int nt = blockDim.x;                          // members / per
  int32_t* s_a = (int32_t*)smem;                      // [nt][slots]
  int32_t* s_c = s_a + nt * slots;
  int32_t* s_b = s_c + nt * slots;
  int32_t* s_n = s_b + nt * slots;                    // [nt]
  __shared__ int32_t s_miss;
  const int64_t e = (int64_t)blockIdx.x / groups;
  const int64_t p0 = ((int64_t)blockIdx.x - e * groups) * stride * members;
  const int i = threadIdx.x;
  const int64_t span = stride * per;                  // segments between threads' first members
  const int64_t p = p0 + (int64_t)i * span;
  if (i == 0) s_miss = 0;
  bool miss = false;
  int n = 0;
  if (p < P) {
    // the thread's members, first tuples and counts loaded together
    Tuple t0[kConcatPer];
    int32_t nm[kConcatPer];
#pragma unroll
    for (int q = 0; q < kConcatPer; ++q) {
      const int64_t pq = p + (int64_t)q * stride;
      const bool in = q < per && pq < P;
      nm[q] = in ? min(ts.nslots[ts.idx(e, pq)], slots) : -1;
      t0[q] = in ? *ts.at(e, pq, 0) : Tuple{0, 0, 0, 0};
    }
    n = nm[0];
    for (int k = 0; k < n; ++k) {
      const Tuple tu = k == 0 ? t0[0] : *ts.at(e, p, k);
      s_a[i * slots + k] = tu.a;
      s_c[i * slots + k] = tu.c;
      s_b[i * slots + k] = tu.b;
    }
#pragma unroll
    for (int q = 1; q < kConcatPer; ++q) {
      if (nm[q] < 0) break;
      const int64_t pq = p + (int64_t)q * stride;
      for (int k = 0; k < n; ++k) {
        const int32_t b = s_b[i * slots + k];
        int hit = -1;
        Tuple hr{0, 0, 0, 0};
        for (int m = 0; m < nm[q] && hit < 0; ++m) {
          const Tuple tr = m == 0 ? t0[q] : *ts.at(e, pq, m);
          if (tr.a == b) {
            hit = m;
            hr = tr;
          }
        }
        if (hit >= 0) {
          s_c[i * slots + k] += hr.c;
          s_b[i * slots + k] = hr.b;
        } else {
          miss = true;
        }
      }
    }
  }
  s_n[i] = n;
  __syncthreads();
  if (miss) s_miss = 1;
  for (int h = 1; h < nt; h <<= 1) {
    if ((i & (2 * h - 1)) == 0 && i + h < nt && p + (int64_t)h * span < P) {
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
          s_miss = 1;
        }
      }
    }
    __syncthreads();
  }
  if (i == 0 && p < P) {
    for (int k = 0; k < s_n[0]; ++k) {
      Tuple tu;
      tu.a = s_a[k];
      tu.c = s_c[k];
      tu.b = s_b[k];
      tu.pad = 0;
      *ts.at(e, p, k) = tu;
    }
    if (s_miss) atomicOr(&flags[e], 2);
  }
}

inline int64_t setup_items(const SetupArgs& A) {
  return setup_search_threads(A.P, A.wave_search != 0) + (int64_t)A.P + 1 + A.S + 1 + 4 + A.tab_words;
}

__global__ __launch_bounds__(kBlock) void fill_i64_kernel(int64_t* p, int64_t n, int64_t v) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i < n) p[i] = v;
}

// Two-pass elimination, last step: the second pass wrote the kept episodes'
// exact counts, in episode order, to out[0 .. kept); spread them to their
// episodes in place and mark the dropped ones -1.  Episode e is kept when
// upper[e] >= theta; its compact index is the number of kept episodes before
// it, which is <= e.  One workgroup walks 1,024-episode chunks from the last
// one down: every thread reads its value, the workgroup waits, then writes.
// A chunk writes only its own indices, which no lower chunk reads (their
// compact indices are below the chunk), and reads happen before the barrier
// that precedes the chunk's writes.
constexpr int kMergeBlock = 1024;
__global__ __launch_bounds__(kMergeBlock) void two_pass_merge_kernel(const int64_t* upper, int64_t S,
                                                                     int64_t theta, int64_t* out) {
  constexpr int kWaves = kMergeBlock / kWave;
  __shared__ int32_t s_wave[kWaves];
  __shared__ int64_t s_part[kWaves];
  __shared__ int64_t s_val[kMergeBlock];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  // kept episodes in all
  int64_t local = 0;
  for (int64_t e = tid; e < S; e += kMergeBlock) local += upper[e] >= theta;
  for (int off = kWave / 2; off > 0; off >>= 1) local += __shfl_xor(local, off);
  if (lane == 0) s_part[wave] = local;
  __syncthreads();
  int64_t total = 0;
  for (int w = 0; w < kWaves; ++w) total += s_part[w];
  int64_t after = 0;  // kept episodes at indices above the current chunk
  for (int64_t c = (S + kMergeBlock - 1) / kMergeBlock - 1; c >= 0; --c) {
    const int64_t e = c * kMergeBlock + tid;
    const bool keep = e < S && upper[e] >= theta;
    const uint64_t ballot = __ballot(keep);
    const int below = __popcll(ballot & ((1ull << lane) - 1));
    __syncthreads();  // the previous chunk is done with s_wave
    if (lane == 0) s_wave[wave] = __popcll(ballot);
    __syncthreads();
    int before = 0, chunk = 0;
    for (int w = 0; w < kWaves; ++w) {
      before += w < wave ? s_wave[w] : 0;
      chunk += s_wave[w];
    }
    const int64_t rank = total - after - chunk + before + below;
    // the value goes through LDS, so the read has landed before the barrier
    s_val[tid] = keep ? out[rank] : -1;
    __syncthreads();
    if (e < S) out[e] = s_val[tid];
    after += chunk;
  }
}

// Streaming: the scalars a push needs on the host, in one launch, written to
// host-mapped memory: the batch's first and last times, the size of the halo
// waiting at the head of the combined buffer, and the halo's first time.
__global__ void stream_info_kernel(const int32_t* batch, int64_t n, const int64_t* halo_n,
                                   const int32_t* halo, int64_t* out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const int64_t hn = *halo_n;
  out[0] = batch[0];
  out[1] = batch[n - 1];
  out[2] = hn;
  out[3] = hn > 0 ? (int64_t)halo[0] : 0;
}

// Streaming: the next halo, the events of [0, n) at or after time `bound`
// (times sorted): its first index and its size.
__global__ void halo_find_kernel(const int32_t* times, int64_t n, int64_t bound, int64_t* first,
                                 int64_t* size) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = lo + ((hi - lo) >> 1);
    if ((int64_t)times[mid] < bound)
      lo = mid + 1;
    else
      hi = mid;
  }
  *first = lo;
  *size = n - lo;
}

// Streaming: the halo halo_find_kernel found, copied to the head of the other
// combined buffer (a grid-stride loop: the halo is usually short).
__global__ __launch_bounds__(kBlock) void halo_move_kernel(const int32_t* st, const uint16_t* sy,
                                                           const int64_t* first, const int64_t* size,
                                                           int32_t* dt, uint16_t* dy) {
  const int64_t h0 = *first, hn = *size;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < hn; i += (int64_t)gridDim.x * kBlock) {
    dt[i] = st[h0 + i];
    dy[i] = sy[h0 + i];
  }
}

__global__ __launch_bounds__(kBlock) void check_sorted_kernel(const int32_t* times, int64_t n,
                                                              int32_t* bad) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i + 1 < n && times[i] > times[i + 1]) atomicOr(bad, 1);
}

inline unsigned grid_for(int64_t items) { return (unsigned)((items + kBlock - 1) / kBlock); }

}  // namespace
}  // namespace epk
