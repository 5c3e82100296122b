// Host side of the serial-episode counting library: argument checks, the
// scheme planner, scratch layout, the small non-templated kernels (cuts,
// Concatenate tree levels, result extraction) and the C ABI of epcount.h.
//
// Source page: "Towards Chip-on-Chip Neuroscience: Fast Mining of Frequent
// Episodes Using Graphics Processors".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "ep_device.hpp"
#include "epcount.h"

namespace epk {
const Launchers* launchers_n1();
const Launchers* launchers_n2();
const Launchers* launchers_n3();
const Launchers* launchers_n4();
const Launchers* launchers_n5();
const Launchers* launchers_n6();
const Launchers* launchers_n7();
const Launchers* launchers_n8();
const Launchers* launchers_n9();
const Launchers* launchers_n10();
const Launchers* launchers_n11();
const Launchers* launchers_n12();
const Launchers* launchers_n13();
const Launchers* launchers_n14();
const Launchers* launchers_n15();
const Launchers* launchers_n16();

namespace {

const Launchers* launchers_for(int N) {
  switch (N) {
    case 1: return launchers_n1();
    case 2: return launchers_n2();
    case 3: return launchers_n3();
    case 4: return launchers_n4();
    case 5: return launchers_n5();
    case 6: return launchers_n6();
    case 7: return launchers_n7();
    case 8: return launchers_n8();
    case 9: return launchers_n9();
    case 10: return launchers_n10();
    case 11: return launchers_n11();
    case 12: return launchers_n12();
    case 13: return launchers_n13();
    case 14: return launchers_n14();
    case 15: return launchers_n15();
    case 16: return launchers_n16();
    default: return nullptr;
  }
}

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
  int64_t S;
  unsigned long long* counters;  // [4]
  int32_t wave_search;  // range ends by one wave each (small P) or one thread each
};

__device__ inline int64_t cut_of(int64_t t_min, int64_t t_max, int64_t p, int64_t P) {
  return t_min - 1 + (p * (t_max - t_min + 1)) / P;
}

// First index i in [0, n) with times[i] > v, n if none; every lane of the wave
// calls it with the same arguments and gets the answer.  Invariant: the
// answer lies in [lo, hi], times[lo-1] <= v and times[hi] > v (or hi = n).
__device__ int64_t wave_upper_bound(const int32_t* times, int64_t n, int64_t v) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t lo = 0, hi = n;
  while (hi - lo > kWave) {
    const int64_t step = (hi - lo + kWave - 1) / kWave;
    int64_t idx = lo + (int64_t)(lane + 1) * step - 1;
    idx = idx < hi - 1 ? idx : hi - 1;
    const uint64_t gt = __ballot((int64_t)times[idx] > v);
    if (gt == 0) {
      lo = hi;  // lane 63 probed hi - 1
    } else {
      const int f = __ffsll((unsigned long long)gt) - 1;
      const int64_t idx_f = lo + (int64_t)(f + 1) * step - 1;
      const int64_t new_lo = f == 0 ? lo : lo + (int64_t)f * step;
      hi = idx_f < hi - 1 ? idx_f : hi - 1;
      lo = new_lo;
    }
  }
  const int64_t idx = lo + lane;
  const bool in = idx < hi;  // lanes past the range read times[0] (n >= 1) and ignore it
  const uint64_t gt = __ballot(in && (int64_t)times[in ? idx : 0] > v);
  return gt ? lo + (__ffsll((unsigned long long)gt) - 1) : hi;
}

constexpr int32_t kWaveSearchMaxP = 4096;

__host__ __device__ inline int64_t setup_search_threads(int32_t P, bool wave) {
  return (int64_t)2 * P * (wave ? kWave : 1);
}

__global__ __launch_bounds__(kBlock) void setup_kernel(SetupArgs A) {
  int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t n_search = setup_search_threads(A.P, A.wave_search != 0);
  if (i < n_search && !A.wave_search) {
    const int64_t p = i >> 1;
    const int64_t t_min = A.times[0];
    const int64_t t_max = A.times[A.n - 1];
    if (i & 1)
      A.end[p] = (int32_t)upper_bound_time(A.times, 0, A.n, cut_of(t_min, t_max, p + 1, A.P) + A.max_span);
    else
      A.beg[p] = (int32_t)upper_bound_time(A.times, 0, A.n, cut_of(t_min, t_max, p, A.P) - A.max_span);
    return;
  }
  if (i < n_search) {
    // wave w: w even -> beg[w / 2], w odd -> end[w / 2] (whole waves: n_search is a
    // multiple of the wave size)
    const int64_t w = i / kWave;
    const int64_t p = w >> 1;
    const int64_t t_min = A.times[0];
    const int64_t t_max = A.times[A.n - 1];
    const int64_t v = (w & 1) ? cut_of(t_min, t_max, p + 1, A.P) + A.max_span
                              : cut_of(t_min, t_max, p, A.P) - A.max_span;
    const int64_t r = wave_upper_bound(A.times, A.n, v);
    if ((threadIdx.x & (kWave - 1)) == 0) {
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
    A.flags[i] = 0;
    return;
  }
  i -= A.S + 1;
  if (i < 4) A.counters[i] = 0ull;
}

// ------------------------------------------------------------- event filter

// One pass over the stream for the list Map kernel.  Block b holds events
// [b * kListBlock, (b + 1) * kListBlock); each event gets its node-type slot
// and the set of episodes with that type, and for each episode its events are
// written in order to the block's region as {time, node levels}: episode e's
// entries start at list_off[b][e] and number list_cnt[b][e].  The region holds
// kListBlock * max_share entries (max_share: most episodes one type is on), so
// blocks need nothing from each other.  A thread takes 16 consecutive events;
// its per-episode counts are packed two to a 32-bit word (16-bit fields; a
// block holds at most 4096), so one scan serves two episodes.
constexpr int kFilterPer = kListBlock / kBlock;  // 16
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
  int2* lists;
  int32_t* list_off;             // [blocks * S]
  int32_t* list_cnt;             // [blocks * S]
};

// One workgroup loops over blocks b = blockIdx.x, + gridDim.x, ...: the LDS
// tables are loaded once, and the next block's events are loaded before the
// current block is classified and written.  G packed count words serve up to
// 4 G episodes.
template <int G>
__global__ __launch_bounds__(kBlock) void filter_kernel(FilterArgs A) {
  constexpr int kE = 4 * G;  // episodes this instance serves at most
  __shared__ uint64_t s_seen[1024];
  __shared__ uint8_t s_rank[1024];
  __shared__ uint32_t s_eps[256];
  __shared__ uint16_t s_lv[256 * kE];
  __shared__ uint16_t s_pre[kE][kBlock];  // thread's next rank per episode
  __shared__ uint32_t s_wsum[kBlock / kWave][2 * G];
  __shared__ int32_t s_off[kE];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int S = A.S;
  for (int i = tid; i < 1024; i += kBlock) {
    s_seen[i] = A.type_seen[i];
    s_rank[i] = A.type_rank[i];
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
  __syncthreads();  // tables in LDS

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
    uint32_t sl[kFilterPer], ep[kFilterPer];
    // per-thread counts in 8-bit fields, four episodes to a word (at most 16
    // each): x * 0x204081 puts bit i of a 4-bit x at bit 8i with no carries
    uint32_t c8[G];
#pragma unroll
    for (int g = 0; g < G; ++g) c8[g] = 0;
#pragma unroll
    for (int k = 0; k < kFilterPer; ++k) {
      const uint32_t yk = y[k];
      const uint64_t w = s_seen[yk >> 6];
      const uint32_t sh = yk & 63u;
      const bool on = k < n_valid && ((w >> sh) & 1ull);
      const uint32_t below = (uint32_t)__popcll(w & ((1ull << sh) - 1ull));
      sl[k] = on ? (uint32_t)s_rank[yk >> 6] + below + 1u : 0u;
      ep[k] = s_eps[sl[k]];
#pragma unroll
      for (int g = 0; g < G; ++g) c8[g] += __umul24((ep[k] >> (4 * g)) & 15u, 0x204081u) & 0x01010101u;
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
      uint32_t v = c[g];
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t u = __shfl_up(v, d, kWave);
        if (lane >= d) v += u;
      }
      incl[g] = v;
      if (lane == kWave - 1) s_wsum[wave][g] = v;
    }
    __syncthreads();
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
    __syncthreads();
    int2* region = A.lists + b * (int64_t)kListBlock * A.max_share;
#pragma unroll
    for (int k = 0; k < kFilterPer; ++k) {
      uint32_t m = ep[k];
      while (m) {
        const int e = __ffs((int)m) - 1;
        m &= m - 1;
        const uint16_t r = s_pre[e][tid];
        s_pre[e][tid] = (uint16_t)(r + 1);
        region[s_off[e] + r] = make_int2(t[k], (int32_t)s_lv[sl[k] * kE + e]);
      }
    }
    __syncthreads();  // s_wsum, s_pre and s_off are rewritten by the next block
  }
}

// ------------------------------------------------------------- Concatenate

// One workgroup joins G consecutive members (segments p0, p0 + stride, ...)
// of one episode in LDS, level by level (Concatenate rules 1-3, Fig. 6), and
// writes the merged tuples back to the first member.  Members hold their
// tuple list keyed by their first segment's keys; joining left block L with
// right block R maps each (a, c, b) of L to (a, c + c', b') for the tuple of R
// whose key a' equals b.  Launched with stride 1, then `members`, then
// members^2, ..., until one member is left.
constexpr int kConcatMembers = 512;  // threads of a tree workgroup at most

__global__ __launch_bounds__(kConcatMembers) void concat_tree_kernel(TupleStore ts, int32_t* flags, int64_t S,
                                                             int32_t P, int64_t stride, int32_t members,
                                                             int64_t groups) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int slots = ts.slots;
  int32_t* s_a = (int32_t*)smem;                      // [members][slots]
  int32_t* s_c = s_a + members * slots;
  int32_t* s_b = s_c + members * slots;
  int32_t* s_n = s_b + members * slots;               // [members]
  __shared__ int32_t s_miss;
  const int64_t e = (int64_t)blockIdx.x / groups;
  const int64_t p0 = ((int64_t)blockIdx.x - e * groups) * stride * members;
  const int i = threadIdx.x;
  const int64_t p = p0 + (int64_t)i * stride;
  if (i == 0) s_miss = 0;
  int n = 0;
  if (p < P) {
    n = min(ts.nslots[ts.idx(e, p)], slots);
    for (int k = 0; k < n; ++k) {
      const Tuple tu = *ts.at(e, p, k);
      s_a[i * slots + k] = tu.a;
      s_c[i * slots + k] = tu.c;
      s_b[i * slots + k] = tu.b;
    }
  }
  s_n[i] = n;
  __syncthreads();
  for (int h = 1; h < members; h <<= 1) {
    if ((i & (2 * h - 1)) == 0 && i + h < members && p + (int64_t)h * stride < P) {
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
  return setup_search_threads(A.P, A.wave_search != 0) + (int64_t)A.P + 1 + A.S + 1 + 4;
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

__global__ __launch_bounds__(kBlock) void check_sorted_kernel(const int32_t* times, int64_t n,
                                                              int32_t* bad) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i + 1 < n && times[i] > times[i + 1]) atomicOr(bad, 1);
}

inline unsigned grid_for(int64_t items) { return (unsigned)((items + kBlock - 1) / kBlock); }

// ------------------------------------------------------------ host helpers

struct DeviceInfo {
  bool ok = false;
  int cu_count = 0;
  // resident tick-kernel workgroups per CU, by [N][one lane holds all machines],
  // for the LDS size tick_lds (queried once: the query is slow)
  int tick_per_cu[EP_MAX_NODES + 1][2] = {};
  size_t tick_lds[EP_MAX_NODES + 1][2] = {};
};

std::mutex g_info_mu;
DeviceInfo g_info[64];

// Pinned staging for the episode-table upload: a ring of slots per device,
// each guarded by the event recorded after its copy, so the host can prepare
// a few calls ahead of the GPU.
constexpr int kStagingSlots = 4;
struct StagingSlot {
  void* buf = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};
struct Staging {
  std::mutex mu;
  StagingSlot slot[kStagingSlots];
  int next = 0;
};
Staging g_staging[64];

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Scratch blocks cached per device.  A call takes a block no other host call
// holds; if the block was last used on another stream, the new stream waits
// for that use on the GPU (hipStreamWaitEvent), never on the host.  Returning
// a block records an event after the call's last kernel.  Blocks grow when a
// call needs more and are kept until the process ends.
struct ScratchBlock {
  void* ptr = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  hipStream_t last_stream = nullptr;
  bool used = false;  // ev has been recorded at least once
  bool held = false;
};
struct ScratchPool {
  std::mutex mu;
  std::vector<ScratchBlock*> blocks;
};
ScratchPool g_scratch[64];

int scratch_acquire(int dev, size_t bytes, hipStream_t stream, ScratchBlock** out) {
  ScratchPool& pool = g_scratch[dev];
  ScratchBlock* b = nullptr;
  {
    std::lock_guard<std::mutex> lock(pool.mu);
    for (ScratchBlock* c : pool.blocks)  // a big enough block, same stream preferred
      if (!c->held && c->cap >= bytes && (!b || c->last_stream == stream)) b = c;
    if (!b)
      for (ScratchBlock* c : pool.blocks)  // else any free block, to grow
        if (!c->held) {
          b = c;
          break;
        }
    if (!b) {
      b = new ScratchBlock();
      pool.blocks.push_back(b);
    }
    b->held = true;
  }
  if (b->used && b->last_stream != stream && hipStreamWaitEvent(stream, b->ev, 0) != hipSuccess) {
    b->held = false;
    return EP_ERR_HIP;
  }
  if (b->cap < bytes) {
    // the old block may still be read by kernels queued on `stream` (ordered
    // after the wait above): free it stream-ordered, then take a bigger one
    if (b->ptr && hipFreeAsync(b->ptr, stream) != hipSuccess) {
      b->held = false;
      return EP_ERR_HIP;
    }
    b->ptr = nullptr;
    b->cap = 0;
    const size_t cap = bytes + bytes / 4;
    if (hipMallocAsync(&b->ptr, cap, stream) != hipSuccess || !b->ptr) {
      b->ptr = nullptr;
      b->held = false;
      return EP_ERR_WORKSPACE;
    }
    b->cap = cap;
  }
  if (!b->ev && hipEventCreateWithFlags(&b->ev, hipEventDisableTiming) != hipSuccess) {
    b->held = false;
    return EP_ERR_HIP;
  }
  *out = b;
  return EP_OK;
}

int scratch_release(int dev, ScratchBlock* b, hipStream_t stream) {
  const bool ok = hipEventRecord(b->ev, stream) == hipSuccess;
  std::lock_guard<std::mutex> lock(g_scratch[dev].mu);
  b->last_stream = stream;
  b->used = b->used || ok;
  b->held = false;
  return ok ? EP_OK : EP_ERR_HIP;
}

// Profiling session: per counting call, events around its phases.  Events
// come from a pool that lives as long as the process, so recording adds no
// event creation to the timed calls once the pool is warm.
constexpr int kProfEvents = 7;
struct ProfRecord {
  // start, before Map (the filter), before the tick Map kernel, after it,
  // after Map, after closure, after Concatenate
  hipEvent_t ev[kProfEvents];
  hipEvent_t end;
  int which;  // -1: every phase; else the one Map kernel timed (EP_PROFILE_*)
};
std::mutex g_prof_mu;
bool g_prof_on = false;
int g_prof_which = -1;   // -1: every phase of every call
int g_prof_every = 1;    // one call in this many is recorded
int64_t g_prof_calls = 0;
std::vector<ProfRecord> g_prof;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pooled_event() {
  // called with g_prof_mu held
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

int prof_record_start(ProfRecord* r, int which, hipStream_t s) {
  r->which = which;
  {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    for (int i = 0; i < kProfEvents; ++i)
      if (!(r->ev[i] = pooled_event())) return EP_ERR_HIP;
    if (!(r->end = pooled_event())) return EP_ERR_HIP;
  }
  if (which >= 0) return EP_OK;
  return hipEventRecord(r->ev[0], s) == hipSuccess ? EP_OK : EP_ERR_HIP;
}

// Lanes per (segment, episode) of the counting kernels: one lane carries all N
// machines up to N = 8, one machine per lane beyond.
constexpr int kMaxClassNodes = 8;

// The hybrid rule (hybrid-algorithm section): the GPU is fully utilised by
// PTPE when the episodes alone give every resident lane of every CU work.
// Otherwise MapConcatenate with the smallest power-of-two P that does, kept
// to >= 256 events per segment on average and P <= 2^20.
int plan_rule(int64_t S, int32_t N, int64_t n, int32_t mode, int32_t n_segments, int32_t cu_count,
              int32_t lanes_per_cu, int32_t* out_mode, int32_t* out_segments) {
  const int64_t full = (int64_t)std::max(cu_count, 1) * std::max(lanes_per_cu, 1);
  int m = mode;
  if (m == EP_MODE_AUTO) m = (S >= full) ? EP_MODE_PTPE : EP_MODE_MAPCONCAT;
  int64_t P = 1;
  if (m == EP_MODE_MAPCONCAT) {
    if (n_segments > 0) {
      P = n_segments;
    } else {
      const int64_t per_seg = std::max<int64_t>(S, 1) * (N <= kMaxClassNodes ? 1 : N);
      const int64_t need = (full + per_seg - 1) / per_seg;
      const int64_t cap_by_events = std::max<int64_t>(1, n / 256);
      P = 2;
      while (P < need && P < (1 << 20)) P <<= 1;
      // keep segments to <= 65,536 events on average: a repair rescans one segment
      while (P * 65536 < n && P < (1 << 20)) P <<= 1;
      while (P > 1 && P > cap_by_events) P >>= 1;
    }
  }
  *out_mode = m;
  *out_segments = (int32_t)P;
  return EP_OK;
}

}  // namespace
}  // namespace epk

using namespace epk;

extern "C" const char* ep_status_string(int status) {
  switch (status) {
    case EP_OK: return "ok";
    case EP_ERR_ARG: return "invalid argument";
    case EP_ERR_NODES: return "episode size outside 1..EP_MAX_NODES";
    case EP_ERR_INTERVAL: return "delay interval violates 0 <= t_low < t_high or the span overflows";
    case EP_ERR_UNSORTED: return "event times are not non-decreasing";
    case EP_ERR_WORKSPACE: return "scratch allocation failed";
    case EP_ERR_HIP: return "HIP runtime error";
    case EP_ERR_UNSUPPORTED: return "a delay window needs more candidate runs than EP_MAX_RUNS";
    default: return "unknown status";
  }
}

extern "C" int64_t ep_segment_cut(int32_t t_min, int32_t t_max, int32_t n_segments, int32_t p) {
  if (n_segments <= 0) return (int64_t)t_min - 1;
  const int64_t width = (int64_t)t_max - (int64_t)t_min + 1;
  return (int64_t)t_min - 1 + ((int64_t)p * width) / n_segments;
}

extern "C" int ep_plan(int64_t n_episodes, int32_t n_nodes, int64_t n_events, int32_t mode,
                       int32_t n_segments, int32_t cu_count, int32_t lanes_per_cu,
                       int32_t* out_mode, int32_t* out_segments) {
  if (!out_mode || !out_segments || n_episodes < 0 || n_events < 0 || n_segments < 0)
    return EP_ERR_ARG;
  if (n_nodes < 1 || n_nodes > EP_MAX_NODES) return EP_ERR_NODES;
  if (mode < EP_MODE_AUTO || mode > EP_MODE_MAPCONCAT) return EP_ERR_ARG;
  return plan_rule(n_episodes, n_nodes, n_events, mode, n_segments, cu_count, lanes_per_cu,
                   out_mode, out_segments);
}

namespace {

#define EP_HIP(call)                                      \
  do {                                                    \
    hipError_t err_ = (call);                             \
    if (err_ != hipSuccess) {                             \
      if (getenv("EP_LOG"))                               \
        fprintf(stderr, "epcount: %s failed: %s\n", #call, \
                hipGetErrorString(err_));                 \
      return EP_ERR_HIP;                                  \
    }                                                     \
  } while (0)

int device_info(int dev, DeviceInfo** out) {
  if (dev < 0 || dev >= 64) return EP_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_info_mu);
  DeviceInfo& d = g_info[dev];
  if (!d.ok) {
    int cus = 0;
    EP_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    d.cu_count = cus;
    d.ok = true;
  }
  *out = &d;
  return EP_OK;
}

// Pinned staging in two steps: staging_acquire() locks the device's ring,
// waits until its next slot's previous copy has finished and hands out the
// slot; staging_commit() enqueues the copy to `dst`, records the slot's event
// and unlocks.  Every acquire is followed by exactly one commit or abort.
int staging_acquire(int dev, size_t bytes, char** out) {
  Staging& st = g_staging[dev];
  st.mu.lock();
  StagingSlot& s = st.slot[st.next];
  int status = EP_OK;
  if (s.pending) {
    if (hipEventSynchronize(s.ev) != hipSuccess) status = EP_ERR_HIP;
    s.pending = false;
  }
  if (status == EP_OK && s.cap < bytes) {
    if (s.buf) hipHostFree(s.buf);
    s.buf = nullptr;
    s.cap = 0;
    const size_t cap = std::max<size_t>(bytes, 1 << 16);
    if (hipHostMalloc(&s.buf, cap, hipHostMallocDefault) != hipSuccess) {
      s.buf = nullptr;
      status = EP_ERR_HIP;
    } else {
      s.cap = cap;
    }
  }
  if (status == EP_OK && !s.ev && hipEventCreateWithFlags(&s.ev, hipEventDisableTiming) != hipSuccess)
    status = EP_ERR_HIP;
  if (status != EP_OK) {
    st.mu.unlock();
    return status;
  }
  *out = (char*)s.buf;
  return EP_OK;
}

int staging_commit(int dev, void* dst, size_t bytes, hipStream_t stream) {
  Staging& st = g_staging[dev];
  StagingSlot& s = st.slot[st.next];
  int status = EP_OK;
  if (hipMemcpyAsync(dst, s.buf, bytes, hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipEventRecord(s.ev, stream) != hipSuccess) {
    status = EP_ERR_HIP;
  } else {
    s.pending = true;
  }
  st.next = (st.next + 1) % kStagingSlots;
  st.mu.unlock();
  return status;
}

const char* win_name(int w) {
  switch (w) {
    case kRuns1: return "runs1";
    case kRuns2: return "runs2";
    case kRuns4: return "runs4";
    case kBits32: return "bits32";
    case kBits64: return "bits64";
    default: return "?";
  }
}

// Everything the launch sequence needs, decided on the host.
struct Launch {
  int mode;        // EP_MODE_PTPE / EP_MODE_MAPCONCAT
  int32_t P;       // segments
  int win;         // window kind of the Map kernel and of the wave machines
  bool bits;       // bit Map kernel (else the scan Map kernel)
  bool all_mach;   // bit kernel: one lane holds all machines of a (segment, episode)
  int M;           // lanes per (segment, episode)
  int G, R, CH;    // episodes and segments per workgroup, events per segment per chunk
  int block;
  size_t lds;
  int CW;          // tick kernel: 64-tick words per segment per chunk
  size_t lds_ticks;
  int split;       // 0: per-segment choice between tick and position kernels; 1: ticks; 2: positions
  bool list;       // sparse segments through the filter + list Map kernels (else the position kernel)
  int slots;
  int n_machines;
};

}  // namespace

namespace {
// phase timestamps of the current call, printed when EP_LOG_TIME is set
thread_local std::chrono::steady_clock::time_point g_tp[16];
thread_local int g_ntp = 0;
inline void mark() {
  if (g_ntp < 16) g_tp[g_ntp++] = std::chrono::steady_clock::now();
}

int count_episodes_impl(const int32_t* times, const uint16_t* types, int64_t n_events,
                        ep_episodes episodes, int64_t n_episodes, int64_t* out_counts,
                        hipStream_t stream, const ep_options* opt) {
  // ---- host-side argument checks (nothing is enqueued before they pass)
  const int32_t N = episodes.n_nodes;
  const int64_t S = n_episodes;
  if (n_events < 0 || S < 0 || n_events > INT32_MAX) return EP_ERR_ARG;
  if (N < 1 || N > EP_MAX_NODES) return EP_ERR_NODES;
  // Algorithm A2: the relaxed episodes, every lower bound taken as 0
  std::vector<int32_t> zero_low;
  if (opt && opt->upper_only && S > 0 && N > 1) {
    zero_low.assign((size_t)(S * (N - 1)), 0);
    episodes.t_low = zero_low.data();
  }
  if (S > 0 && (!out_counts || !episodes.types)) return EP_ERR_ARG;
  if (S > 0 && N > 1 && (!episodes.t_low || !episodes.t_high)) return EP_ERR_ARG;
  if (n_events > 0 && S > 0 && (!times || !types)) return EP_ERR_ARG;
  const int mode = opt ? opt->mode : EP_MODE_AUTO;
  if (mode < EP_MODE_AUTO || mode > EP_MODE_MAPCONCAT) return EP_ERR_ARG;
  if (opt && opt->n_segments < 0) return EP_ERR_ARG;

  int64_t max_span = 0, max_hi = 0;
  int K = 1;
  int dil_k = 0;  // doubling steps of the tick kernel's dilation (windows up to 63 ticks)
  for (int64_t e = 0; e < S; ++e) {
    int64_t span = 0;
    for (int j = 0; j < N - 1; ++j) {
      const int64_t lo = episodes.t_low[e * (N - 1) + j];
      const int64_t hi = episodes.t_high[e * (N - 1) + j];
      if (lo < 0 || lo >= hi) return EP_ERR_INTERVAL;
      span += hi;
      max_hi = std::max(max_hi, hi);
      if (hi <= 63) dil_k = std::max(dil_k, dil_steps((uint32_t)lo, (uint32_t)hi));
      // live disjoint runs of a window are bounded by floor(hi / (hi - lo + 1)) + 1
      const int64_t runs = hi / (hi - lo + 1) + 1;
      while (K < runs && K <= EP_MAX_RUNS) K <<= 1;
    }
    if (span > INT32_MAX) return EP_ERR_INTERVAL;
    max_span = std::max(max_span, span);
  }
  // window kind: bit windows when every t_high fits one mask, else run windows
  int win;
  if (max_hi <= 31)
    win = kBits32;
  else if (max_hi <= 63)
    win = kBits64;
  else if (K <= EP_MAX_RUNS)
    win = K == 1 ? kRuns1 : (K == 2 ? kRuns2 : kRuns4);
  else
    return EP_ERR_UNSUPPORTED;
  if (S == 0) return EP_OK;

  // distinct node types -> slots 1..U by rank (a 65,536-bit set with prefix counts)
  uint64_t seen[1024];
  uint32_t rank_base[1024];
  memset(seen, 0, sizeof(seen));
  for (int64_t i = 0; i < S * N; ++i) seen[episodes.types[i] >> 6] |= 1ull << (episodes.types[i] & 63);
  int U = 0;
  for (int w = 0; w < 1024; ++w) {
    rank_base[w] = (uint32_t)U;
    U += __builtin_popcountll(seen[w]);
  }
  auto slot_of = [&](uint16_t y) -> uint32_t {
    const uint64_t below = seen[y >> 6] & ((1ull << (y & 63)) - 1);
    return rank_base[y >> 6] + (uint32_t)__builtin_popcountll(below) + 1;
  };

  // the list path's tables: per node-type slot, the episodes with that type
  // (bit e) and, per (slot, episode), the node levels with it; max_share is
  // the most episodes one type is on (the filter's per-block region size)
  uint32_t slot_eps[256];
  uint16_t slot_levels[256 * kMaxListEpisodes];
  int max_share = 1;
  if (S <= kMaxListEpisodes && U <= 255) {
    memset(slot_eps, 0, sizeof(slot_eps));
    memset(slot_levels, 0, sizeof(uint16_t) * 256 * S);
    for (int64_t e = 0; e < S; ++e)
      for (int j = 0; j < N; ++j) {
        const uint32_t u = slot_of(episodes.types[e * N + j]);
        slot_eps[u] |= 1u << e;
        slot_levels[u * S + e] |= (uint16_t)(1u << j);
      }
    for (int u = 0; u < 256; ++u) max_share = std::max(max_share, __builtin_popcount(slot_eps[u]));
  }
  const int64_t n_lblocks = (n_events + kListBlock - 1) / kListBlock;
  const double list_bytes = (double)n_lblocks * kListBlock * max_share * sizeof(int2);

  int dev = 0;
  EP_HIP(hipGetDevice(&dev));
  if (n_events == 0) {
    hipLaunchKernelGGL(fill_i64_kernel, dim3(grid_for(S)), dim3(kBlock), 0, stream, out_counts, S,
                       (int64_t)0);
    EP_HIP(hipGetLastError());
    if (opt && opt->stats) {
      EP_HIP(hipStreamSynchronize(stream));
      memset(opt->stats, 0, sizeof(ep_stats));
      opt->stats->mode = EP_MODE_PTPE;
      opt->stats->n_segments = 1;
      opt->stats->max_runs = win >= kBits32 ? (win == kBits32 ? 32 : 64) : K;
    }
    return EP_OK;
  }

  DeviceInfo* info = nullptr;
  if (int st = device_info(dev, &info)) return st;
  const Launchers* Lr = launchers_for(N);

  mark();  // checks, slots
  // ---- plan: scheme, segments, kernel and workgroup layout
  Launch L{};
  L.win = win;
  L.bits = (win == kBits32 || win == kBits64) && U <= 255 && !getenv("EP_FORCE_SCAN");
  if (!L.bits && win >= kBits32) {
    // many node types: the scan kernel with bit windows is not built; use runs if they fit
    if (K > EP_MAX_RUNS) return EP_ERR_UNSUPPORTED;
    L.win = K == 1 ? kRuns1 : (K == 2 ? kRuns2 : kRuns4);
  }
  const int lanes_per_cu_est = 2048;  // 8 waves on each of 4 SIMDs
  int32_t pmode = 0, P = 1;
  plan_rule(S, N, n_events, mode, opt ? opt->n_segments : 0, info->cu_count, lanes_per_cu_est,
            &pmode, &P);
  L.mode = pmode;
  L.P = P;
  L.n_machines = (pmode == EP_MODE_PTPE) ? 1 : N;
  L.block = kBlock;
  if (L.bits) {
    // one lane per (segment, episode) holding every machine, unless that
    // leaves the GPU with too few lanes for a fixed segment count
    const int64_t target = (int64_t)info->cu_count * lanes_per_cu_est;
    L.split = 0;
    if (const char* sp = getenv("EP_SPLIT")) {
      if (!strcmp(sp, "ticks")) L.split = 1;
      if (!strcmp(sp, "positions")) L.split = 2;
    }
    // few episodes: sparse segments read the filter kernel's per-episode lists
    // (one lane per (segment, episode) walks only its episode's events)
    L.list = S <= kMaxListEpisodes && L.split != 1 && list_bytes <= kMaxListBytes &&
             !getenv("EP_NO_LIST");
    L.all_mach = L.n_machines > 1 && N <= kMaxClassNodes && (L.list || S * (int64_t)P * 4 >= target);
    const char* lanes_env = getenv("EP_LANES");
    if (lanes_env && N <= kMaxClassNodes && L.n_machines > 1)
      L.all_mach = strcmp(lanes_env, "machine") != 0;
    L.M = L.all_mach ? 1 : L.n_machines;
    L.G = (int)std::min<int64_t>(S, L.block / L.M);
    L.R = (L.G == S) ? std::max(1, L.block / (L.G * L.M)) : 1;
    L.R = (int)std::min<int64_t>(L.R, P);
    // LDS per workgroup: U presence bitmaps + times + slots of one chunk, <= 64 KiB
    // (the list kernel stages nothing)
    for (; !L.list;) {
      // events per segment per chunk: about 2,048 events per tile, a multiple of
      // 64 (whole presence-bitmap words)
      L.CH = std::max((2048 / L.R) & ~63, 64);
      const int tile = L.R * L.CH;
      L.lds = (size_t)U * (tile / 64) * 8 + (size_t)tile * 5;
      if (L.lds <= 65536 || L.R == 1) break;
      L.R = (L.R + 1) / 2;
    }
    if (L.lds > 65536 || L.list) {
      L.CH = 64;
      L.lds = (size_t)U * 8 + 64 * 5;
    }
    // tick kernel: per chunk, R segments x CW words x U slot bitmaps, <= 32 KiB
    L.CW = (int)std::max<int64_t>(1, std::min<int64_t>(64, 32768 / ((int64_t)L.R * U * 8)));
    L.lds_ticks = (size_t)L.R * L.CW * U * 8;
  } else {
    L.list = false;
    L.all_mach = false;
    L.M = L.n_machines;
    L.G = (int)std::min<int64_t>(S, L.block / L.M);
    L.R = (L.G == S) ? std::max(1, L.block / (L.G * L.M)) : 1;
    L.R = (int)std::min<int64_t>(L.R, P);
    L.CH = kTile / L.R;
    L.lds = 0;
  }
  L.slots = (pmode == EP_MODE_PTPE) ? 1 : 2 * N;
  if (getenv("EP_LOG"))
    fprintf(stderr,
            "epcount: S=%lld N=%d n=%lld U=%d mode=%s P=%d win=%s kernel=%s lanes=%s M=%d G=%d R=%d "
            "CH=%d lds=%zu maxSpan=%lld\n",
            (long long)S, N, (long long)n_events, U, pmode == EP_MODE_PTPE ? "ptpe" : "mapconcat", P,
            win_name(L.win), L.bits ? "bits" : "scan", L.all_mach ? "class" : "machine", L.M, L.G, L.R,
            L.CH, L.lds, (long long)max_span);

  // ---- scratch layout (one stream-ordered allocation)
  const size_t sz_types = align_up(sizeof(uint16_t) * S * N, 256);
  const size_t sz_lohi = align_up(sizeof(int32_t) * S * std::max(N - 1, 1), 256);
  const size_t sz_span = align_up(sizeof(int32_t) * S, 256);
  const size_t sz_slot = align_up((size_t)S * N, 256);
  const size_t sz_seen = sizeof(uint64_t) * 1024;  // node types as a 65,536-bit set
  const size_t sz_rank = 1024;                       // set bits before each 64-bit word
  const size_t sz_seps = L.list ? sizeof(uint32_t) * 256 : 0;
  const size_t sz_slv = L.list ? align_up(sizeof(uint16_t) * 256 * S, 256) : 0;
  const size_t host_bytes =
      sz_types + 2 * sz_lohi + sz_span + sz_slot + sz_seen + sz_rank + sz_seps + sz_slv;
  // (+ slack: the list kernel's aligned batches may read two entries past the
  // last block's region)
  const size_t sz_lists = L.list ? align_up((size_t)list_bytes + 4 * sizeof(int2), 256) : 0;
  const size_t sz_lidx = L.list ? align_up(sizeof(int32_t) * (size_t)n_lblocks * S, 256) : 0;
  const size_t sz_tau = align_up(sizeof(int64_t) * (P + 1), 256);
  const size_t sz_seg = align_up(sizeof(int32_t) * P, 256);
  const size_t sz_t0 = align_up(sizeof(Tuple) * (size_t)P * S, 256);
  const size_t sz_tx = align_up(sizeof(Tuple) * (size_t)P * S * (L.slots - 1), 256);
  const size_t sz_tuples = sz_t0 + sz_tx;
  const size_t sz_nslots = align_up(sizeof(int32_t) * (size_t)P * S, 256);  // also nmap
  const size_t sz_flags = align_up(sizeof(int32_t) * (S + 1), 256);
  const size_t sz_cnt = 256;
  const size_t total =
      host_bytes + sz_tau + 2 * sz_seg + sz_tuples + 2 * sz_nslots + sz_flags + sz_cnt + sz_lists +
      2 * sz_lidx;

  mark();  // plan
  ScratchBlock* block = nullptr;
  if (int st = scratch_acquire(dev, total, stream, &block)) return st;
  char* ws = (char*)block->ptr;
  int status = EP_OK;
  mark();  // malloc
  do {
    size_t off = 0;
    uint16_t* d_types = (uint16_t*)(ws + off); off += sz_types;
    int32_t* d_lo = (int32_t*)(ws + off); off += sz_lohi;
    int32_t* d_hi = (int32_t*)(ws + off); off += sz_lohi;
    int32_t* d_span = (int32_t*)(ws + off); off += sz_span;
    uint8_t* d_slot = (uint8_t*)(ws + off); off += sz_slot;
    uint64_t* d_seen = (uint64_t*)(ws + off); off += sz_seen;
    uint8_t* d_rank = (uint8_t*)(ws + off); off += sz_rank;
    uint32_t* d_seps = (uint32_t*)(ws + off); off += sz_seps;
    uint16_t* d_slv = (uint16_t*)(ws + off); off += sz_slv;
    int64_t* d_tau = (int64_t*)(ws + off); off += sz_tau;
    int32_t* d_beg = (int32_t*)(ws + off); off += sz_seg;
    int32_t* d_end = (int32_t*)(ws + off); off += sz_seg;
    Tuple* d_t0 = (Tuple*)(ws + off); off += sz_t0;
    Tuple* d_tx = (Tuple*)(ws + off); off += sz_tx;
    int32_t* d_nslots = (int32_t*)(ws + off); off += sz_nslots;
    int32_t* d_nmap = (int32_t*)(ws + off); off += sz_nslots;
    TupleStore ts;
    ts.T0 = d_t0; ts.TX = d_tx; ts.nmap = d_nmap; ts.nslots = d_nslots; ts.P = P; ts.slots = L.slots;
    int32_t* d_flags = (int32_t*)(ws + off); off += sz_flags;
    unsigned long long* d_cnt = (unsigned long long*)(ws + off); off += sz_cnt;
    int2* d_lists = (int2*)(ws + off); off += sz_lists;
    int32_t* d_loff = (int32_t*)(ws + off); off += sz_lidx;
    int32_t* d_lcnt = (int32_t*)(ws + off); off += sz_lidx;

    // episode table, spans, node slots and the node-type set, written
    // straight into pinned staging: one upload
    {
      char* host = nullptr;
      if ((status = staging_acquire(dev, host_bytes, &host))) break;
      memcpy(host, episodes.types, sizeof(uint16_t) * S * N);
      if (N > 1) {
        memcpy(host + sz_types, episodes.t_low, sizeof(int32_t) * S * (N - 1));
        memcpy(host + sz_types + sz_lohi, episodes.t_high, sizeof(int32_t) * S * (N - 1));
      }
      int32_t* spans = (int32_t*)(host + sz_types + 2 * sz_lohi);
      uint8_t* slots = (uint8_t*)(host + sz_types + 2 * sz_lohi + sz_span);
      for (int64_t e = 0; e < S; ++e) {
        int64_t sp = 0;
        for (int j = 0; j < N - 1; ++j) sp += episodes.t_high[e * (N - 1) + j];
        spans[e] = (int32_t)sp;
        for (int j = 0; j < N; ++j)
          slots[e * N + j] = (uint8_t)(U <= 255 ? slot_of(episodes.types[e * N + j]) : 0);
      }
      memcpy(host + sz_types + 2 * sz_lohi + sz_span + sz_slot, seen, sz_seen);
      uint8_t* rank = (uint8_t*)(host + sz_types + 2 * sz_lohi + sz_span + sz_slot + sz_seen);
      for (int w = 0; w < 1024; ++w) rank[w] = (uint8_t)(U <= 255 ? rank_base[w] : 0);
      if (L.list) {
        char* at = host + sz_types + 2 * sz_lohi + sz_span + sz_slot + sz_seen + sz_rank;
        memcpy(at, slot_eps, sz_seps);
        memcpy(at + sz_seps, slot_levels, sizeof(uint16_t) * 256 * S);
      }
      if ((status = staging_commit(dev, ws, host_bytes, stream))) break;
    }

    if (opt && opt->validate) {
      hipLaunchKernelGGL(fill_i64_kernel, dim3(1), dim3(kBlock), 0, stream, (int64_t*)d_cnt, (int64_t)1,
                         (int64_t)0);
      hipLaunchKernelGGL(check_sorted_kernel, dim3(grid_for(n_events)), dim3(kBlock), 0, stream, times,
                         n_events, (int32_t*)d_cnt);
      int32_t bad = 0;
      if (hipMemcpyAsync(&bad, d_cnt, sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
          hipStreamSynchronize(stream) != hipSuccess) {
        status = EP_ERR_HIP;
        break;
      }
      if (bad) {
        status = EP_ERR_UNSORTED;
        break;
      }
    }

    mark();  // upload
    bool prof = false;
    int prof_which = -1;
    ProfRecord rec{};
    {
      std::lock_guard<std::mutex> lock(g_prof_mu);
      if (g_prof_on) {
        prof_which = g_prof_which;
        prof = (g_prof_calls++ % g_prof_every) == 0;
      }
    }
    if (prof && (status = prof_record_start(&rec, prof_which, stream))) break;
    // records boundary i when the session times it (every boundary, or the
    // two around the one Map kernel it times)
    auto rec_at = [&](int i) {
      if (prof && (prof_which < 0 || i == prof_which + 1 || i == prof_which + 2))
        (void)hipEventRecord(rec.ev[i], stream);
    };
    SetupArgs sa;
    sa.times = times; sa.n = n_events; sa.P = P; sa.max_span = max_span;
    sa.tau = d_tau; sa.beg = d_beg; sa.end = d_end;
    sa.flags = d_flags; sa.S = S; sa.counters = d_cnt;
    sa.wave_search = P <= kWaveSearchMaxP ? 1 : 0;
    hipLaunchKernelGGL(setup_kernel, dim3(grid_for(setup_items(sa))), dim3(kBlock), 0, stream, sa);
    if (hipGetLastError() != hipSuccess) { status = EP_ERR_HIP; break; }

    mark();  // setup launch
    MapArgs ma;
    ma.times = times; ma.types = types;
    ma.ep_types = d_types; ma.ep_lo = d_lo; ma.ep_hi = d_hi; ma.ep_span = d_span;
    ma.ep_slot = d_slot; ma.type_seen = d_seen; ma.type_rank = d_rank;
    ma.tau = d_tau; ma.seg_beg = d_beg; ma.seg_end = d_end;
    ma.ts = ts;
    ma.S = S; ma.P = P; ma.M = L.M; ma.G = L.G; ma.R = L.R; ma.CH = L.CH;
    ma.U = U; ma.n_machines = L.n_machines;
    ma.max_span = max_span; ma.CW = L.CW; ma.split = L.split; ma.dil_steps = dil_k;
    ma.lists = d_lists; ma.list_off = d_loff; ma.list_cnt = d_lcnt; ma.max_share = max_share;
    // workgroups: (segment group, episode group), episode group fastest
    ma.n_egroups = (S + L.G - 1) / L.G;
    dim3 mgrid((unsigned)(((P + L.R - 1) / L.R) * ma.n_egroups));
    // tick kernel: where a segment group fits one chunk, as few workgroups per
    // group as still fill every CU loop over its episode groups, building the
    // bitmaps once each (the kernel decides per group; the grid is mgrid)
    const int64_t seg_groups = (P + L.R - 1) / L.R;
    ma.eg_blocks = ma.n_egroups;
    if (L.bits && L.split != 2) {
      int per_cu = 0;
      {
        std::lock_guard<std::mutex> lock(g_info_mu);
        int& cached = info->tick_per_cu[N][L.all_mach ? 1 : 0];
        size_t& cached_lds = info->tick_lds[N][L.all_mach ? 1 : 0];
        if (cached == 0 || cached_lds != L.lds_ticks) {
          if (Lr->occupancy_ticks(L.all_mach, L.block, L.lds_ticks, &cached) != hipSuccess || cached < 1)
            cached = 1;
          cached_lds = L.lds_ticks;
        }
        per_cu = cached;
      }
      const int64_t want = (int64_t)info->cu_count * per_cu;
      ma.eg_blocks = std::min<int64_t>(ma.n_egroups, std::max<int64_t>(1, (want + seg_groups - 1) / seg_groups));
    }
    rec_at(1);
    hipError_t le = hipSuccess;
    if (L.list) {
      FilterArgs fa;
      fa.times = times; fa.types = types; fa.n = n_events;
      fa.type_seen = d_seen; fa.type_rank = d_rank; fa.slot_eps = d_seps; fa.slot_levels = d_slv;
      fa.S = (int32_t)S; fa.max_share = max_share;
      fa.lists = d_lists; fa.list_off = d_loff; fa.list_cnt = d_lcnt;
      // persistent workgroups: a few per CU, each looping over blocks
      const int64_t fgrid = std::min<int64_t>(n_lblocks, (int64_t)info->cu_count * 4);
      const dim3 fg((unsigned)fgrid), fb(kBlock);
      if (S <= 4)
        hipLaunchKernelGGL(filter_kernel<1>, fg, fb, 0, stream, fa);
      else if (S <= 8)
        hipLaunchKernelGGL(filter_kernel<2>, fg, fb, 0, stream, fa);
      else if (S <= 16)
        hipLaunchKernelGGL(filter_kernel<4>, fg, fb, 0, stream, fa);
      else
        hipLaunchKernelGGL(filter_kernel<8>, fg, fb, 0, stream, fa);
      le = hipGetLastError();
    }
    rec_at(2);
    if (le == hipSuccess && !L.bits) {
      rec_at(3);  // no tick kernel: an empty interval
      le = Lr->map_scan(ma, L.win, mgrid, dim3(L.block), stream);
    } else if (le == hipSuccess) {
      // each segment goes to the tick kernel or, by segment_uses_ticks, to the
      // list or the position kernel
      if (L.split != 2) le = Lr->map_ticks(ma, L.all_mach, mgrid, dim3(L.block), L.lds_ticks, stream);
      rec_at(3);
      if (le == hipSuccess && L.split != 1)
        le = L.list ? Lr->map_list(ma, L.win, L.all_mach, mgrid, dim3(L.block), stream)
                    : Lr->map_bits(ma, L.win, L.all_mach, mgrid, dim3(L.block), L.lds, stream);
    }
    if (le != hipSuccess) { status = EP_ERR_HIP; break; }
    rec_at(4);

    mark();  // map launches
    if (P > 1) {
      ClosureArgs ca;
      ca.times = times; ca.types = types;
      ca.ep_types = d_types; ca.ep_lo = d_lo; ca.ep_hi = d_hi; ca.ep_span = d_span;
      ca.tau = d_tau; ca.seg_beg = d_beg; ca.seg_end = d_end;
      ca.ts = ts; ca.flags = d_flags; ca.repairs = d_cnt;
      ca.S = S; ca.P = P;
      if (Lr->closure(ca, L.win, dim3(grid_for((int64_t)(P - 1) * S)), stream) != hipSuccess) {
        status = EP_ERR_HIP;
        break;
      }
      rec_at(5);
      // Concatenate tree: each launch joins groups of `members` blocks in LDS
      int members = kConcatMembers;
      while (members > 1 && (size_t)members * (12 * L.slots + 4) > 65536) members >>= 1;
      const size_t lds = (size_t)members * (12 * L.slots + 4);
      for (int64_t stride = 1; stride < P; stride *= members) {
        const int64_t groups = (P + stride * members - 1) / (stride * members);
        hipLaunchKernelGGL(concat_tree_kernel, dim3((unsigned)(groups * S)), dim3(members), lds,
                           stream, ts, d_flags, S, P, stride, members, groups);
        if (hipGetLastError() != hipSuccess) { status = EP_ERR_HIP; break; }
      }
      if (status != EP_OK) break;
    }
    if (P <= 1) rec_at(5);
    rec_at(6);
    mark();  // closure + tree launches
    FallbackArgs fa;
    fa.times = times; fa.types = types;
    fa.ep_types = d_types; fa.ep_lo = d_lo; fa.ep_hi = d_hi; fa.ep_span = d_span;
    fa.flags = d_flags; fa.T0 = d_t0; fa.P = P;
    fa.fallbacks = d_cnt + 1; fa.out = out_counts;
    fa.n = n_events; fa.S = S;
    if (Lr->finish(fa, L.win, dim3((unsigned)((S + 3) / 4)), stream) != hipSuccess) {
      status = EP_ERR_HIP;
      break;
    }
    if (prof) {
      if (prof_which < 0) (void)hipEventRecord(rec.end, stream);
      std::lock_guard<std::mutex> lock(g_prof_mu);
      g_prof.push_back(rec);
    }

    if (opt && opt->stats) {
      unsigned long long cnt[2] = {0, 0};
      if (hipMemcpyAsync(cnt, d_cnt, sizeof(cnt), hipMemcpyDeviceToHost, stream) != hipSuccess ||
          hipStreamSynchronize(stream) != hipSuccess) {
        status = EP_ERR_HIP;
        break;
      }
      opt->stats->mode = pmode;
      opt->stats->n_segments = P;
      opt->stats->max_runs = L.win >= kBits32 ? (L.win == kBits32 ? 32 : 64) : K;
      opt->stats->kernels = (L.bits ? 1 : 0) | (L.all_mach ? 2 : 0) | (L.list ? 4 : 0);
      opt->stats->repairs = (int64_t)cnt[0];
      opt->stats->fallbacks = (int64_t)cnt[1];
    }
  } while (0);

  mark();  // finish launch
  if (scratch_release(dev, block, stream) != EP_OK && status == EP_OK) status = EP_ERR_HIP;
  mark();  // free
  return status;
}

}  // namespace

extern "C" int ep_profile_begin(void) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  g_prof.clear();
  g_prof_on = true;
  g_prof_which = -1;
  g_prof_every = 1;
  g_prof_calls = 0;
  return EP_OK;
}

extern "C" int ep_profile_begin_kernel(int32_t which, int32_t every) {
  if (which < EP_PROFILE_FILTER || which > EP_PROFILE_POSITIONS || every < 1) return EP_ERR_ARG;
  std::lock_guard<std::mutex> lock(g_prof_mu);
  g_prof.clear();
  g_prof_on = true;
  g_prof_which = which;
  g_prof_every = every;
  g_prof_calls = 0;
  return EP_OK;
}

extern "C" int ep_profile_end(ep_profile* out) {
  std::vector<ProfRecord> recs;
  {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    if (!g_prof_on) return EP_ERR_ARG;
    g_prof_on = false;
    recs.swap(g_prof);
  }
  ep_profile acc{};
  int status = EP_OK;
  for (ProfRecord& r : recs) {
    if (r.which >= 0) {
      // one Map kernel: the interval between its two boundaries
      float k_ms = 0.f;
      if (hipEventSynchronize(r.ev[r.which + 2]) != hipSuccess ||
          hipEventElapsedTime(&k_ms, r.ev[r.which + 1], r.ev[r.which + 2]) != hipSuccess)
        status = EP_ERR_HIP;
      double* field = r.which == EP_PROFILE_FILTER
                          ? &acc.map_filter_ms
                          : (r.which == EP_PROFILE_TICKS ? &acc.map_ticks_ms : &acc.map_positions_ms);
      *field += k_ms;
      acc.map_ms += k_ms;
      acc.calls += 1;
      std::lock_guard<std::mutex> lock(g_prof_mu);
      for (int i = 0; i < kProfEvents; ++i) g_event_pool.push_back(r.ev[i]);
      g_event_pool.push_back(r.end);
      continue;
    }
    float ms[kProfEvents] = {};
    if (hipEventSynchronize(r.end) != hipSuccess) status = EP_ERR_HIP;
    hipEvent_t seq[kProfEvents + 1];
    for (int i = 0; i < kProfEvents; ++i) seq[i] = r.ev[i];
    seq[kProfEvents] = r.end;
    for (int i = 0; i < kProfEvents && status == EP_OK; ++i)
      if (hipEventElapsedTime(&ms[i], seq[i], seq[i + 1]) != hipSuccess) status = EP_ERR_HIP;
    acc.other_ms += ms[0] + ms[6];
    acc.map_filter_ms += ms[1];
    acc.map_ticks_ms += ms[2];
    acc.map_positions_ms += ms[3];
    acc.map_ms += ms[1] + ms[2] + ms[3];
    acc.closure_ms += ms[4];
    acc.concat_ms += ms[5];
    acc.calls += 1;
    std::lock_guard<std::mutex> lock(g_prof_mu);
    for (int i = 0; i < kProfEvents; ++i) g_event_pool.push_back(r.ev[i]);
    g_event_pool.push_back(r.end);
  }
  if (out) *out = acc;
  return status;
}

extern "C" int ep_count_episodes_ex(const int32_t* times, const uint16_t* types, int64_t n_events,
                                    ep_episodes episodes, int64_t n_episodes, int64_t* out_counts,
                                    hipStream_t stream, const ep_options* opt) {
  static const bool log_time = getenv("EP_LOG_TIME") != nullptr;
  if (!log_time)
    return count_episodes_impl(times, types, n_events, episodes, n_episodes, out_counts, stream, opt);
  const auto t0 = std::chrono::steady_clock::now();
  g_ntp = 0;
  const int st = count_episodes_impl(times, types, n_events, episodes, n_episodes, out_counts, stream, opt);
  const auto t1 = std::chrono::steady_clock::now();
  fprintf(stderr, "epcount: host %.1f us:", std::chrono::duration<double, std::micro>(t1 - t0).count());
  auto prev = t0;
  for (int i = 0; i < g_ntp; ++i) {
    fprintf(stderr, " %.1f", std::chrono::duration<double, std::micro>(g_tp[i] - prev).count());
    prev = g_tp[i];
  }
  fprintf(stderr, "\n");
  return st;
}

extern "C" int ep_count_two_pass(const int32_t* times, const uint16_t* types, int64_t n_events,
                                 ep_episodes episodes, int64_t n_episodes, int64_t threshold,
                                 int64_t* out_counts, int64_t* out_upper, int64_t* n_kept,
                                 hipStream_t stream, const ep_options* opt) {
  using namespace epk;
  const int32_t N = episodes.n_nodes;
  const int64_t S = n_episodes;
  if (n_kept) *n_kept = 0;
  if (S < 0 || n_events < 0 || n_events > INT32_MAX) return EP_ERR_ARG;
  if (N < 1 || N > EP_MAX_NODES) return EP_ERR_NODES;
  if (opt && opt->upper_only) return EP_ERR_ARG;
  if (S == 0) return EP_OK;
  if (!out_counts || !out_upper || !episodes.types) return EP_ERR_ARG;
  if (N > 1 && (!episodes.t_low || !episodes.t_high)) return EP_ERR_ARG;
  // the whole table is checked here: the second pass sees only the kept rows
  for (int64_t e = 0; e < S; ++e) {
    int64_t span = 0;
    for (int j = 0; j < N - 1; ++j) {
      const int64_t lo = episodes.t_low[e * (N - 1) + j];
      const int64_t hi = episodes.t_high[e * (N - 1) + j];
      if (lo < 0 || lo >= hi) return EP_ERR_INTERVAL;
      span += hi;
    }
    if (span > INT32_MAX) return EP_ERR_INTERVAL;
  }
  // first pass (A2): every relaxed episode
  ep_options o1{};
  if (opt) o1 = *opt;
  o1.upper_only = 1;
  o1.stats = nullptr;
  if (int st = count_episodes_impl(times, types, n_events, episodes, S, out_upper, stream, &o1))
    return st;
  std::vector<int64_t> upper((size_t)S);
  EP_HIP(hipMemcpyAsync(upper.data(), out_upper, (size_t)S * sizeof(int64_t), hipMemcpyDeviceToHost,
                        stream));
  EP_HIP(hipStreamSynchronize(stream));
  // second pass (A1): the kept episodes, exact, written compactly to out_counts
  std::vector<uint16_t> k_types;
  std::vector<int32_t> k_low, k_high;
  int64_t kept = 0;
  for (int64_t e = 0; e < S; ++e) {
    if (upper[(size_t)e] < threshold) continue;
    k_types.insert(k_types.end(), episodes.types + e * N, episodes.types + (e + 1) * N);
    if (N > 1) {
      k_low.insert(k_low.end(), episodes.t_low + e * (N - 1), episodes.t_low + (e + 1) * (N - 1));
      k_high.insert(k_high.end(), episodes.t_high + e * (N - 1), episodes.t_high + (e + 1) * (N - 1));
    }
    ++kept;
  }
  if (kept > 0) {
    ep_episodes sub{N, k_types.data(), N > 1 ? k_low.data() : nullptr,
                    N > 1 ? k_high.data() : nullptr};
    ep_options o2{};
    if (opt) o2 = *opt;
    o2.upper_only = 0;
    o2.validate = 0;  // the first pass checked the stream
    if (int st = count_episodes_impl(times, types, n_events, sub, kept, out_counts, stream, &o2))
      return st;
  }
  hipLaunchKernelGGL(two_pass_merge_kernel, dim3(1), dim3(kMergeBlock), 0, stream, out_upper, S,
                     threshold, out_counts);
  EP_HIP(hipGetLastError());
  if (n_kept) *n_kept = kept;
  return EP_OK;
}

extern "C" int ep_count_episodes(const int32_t* times, const uint16_t* types, int64_t n_events,
                                 ep_episodes episodes, int64_t n_episodes, int64_t* out_counts,
                                 hipStream_t stream) {
  return ep_count_episodes_ex(times, types, n_events, episodes, n_episodes, out_counts, stream,
                              nullptr);
}
