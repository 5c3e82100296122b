// Host side of the serial-episode counting library: argument checks, the
// scheme planner, scratch layout, launches and the C ABI of epcount.h (the
// kernels not specialised per episode size are in ep_kernels.hpp).
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
#include <tuple>
#include <vector>

#include "ep_device.hpp"
#include "ep_kernels.hpp"
#include "ep_slice.hpp"
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


// ------------------------------------------------------------ host helpers

struct DeviceInfo {
  bool ok = false;
  int cu_count = 0;
  // resident tick-kernel workgroups per CU, by [N][one lane holds all machines],
  // for the LDS size tick_lds (queried once: the query is slow)
  int tick_per_cu[EP_MAX_NODES + 1][2] = {};
  size_t tick_lds[EP_MAX_NODES + 1][2] = {};
  // resident lanes per CU of the tick kernel with one lane per (segment,
  // episode), as its registers allow (the planner's T_B * B_MP), by N
  int plan_lanes[EP_MAX_NODES + 1] = {};
  // resident list-pruning workgroups per CU (0: not queried yet)
  int prune_per_cu = 0;
};

std::mutex g_info_mu;
DeviceInfo g_info[64];

// Pinned staging for the episode-table upload: a ring of slots per device,
// each guarded by the event recorded after its copy, so the host can prepare
// a few calls ahead of the GPU.
constexpr int kStagingSlots = 4;
struct StagingSlot {
  void* buf = nullptr;   // coherent pinned host memory
  void* dbuf = nullptr;  // the same memory as the device addresses it
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

// Hands a held block back after a failed acquire (under the pool's lock).
int scratch_abandon(ScratchPool& pool, ScratchBlock* b, int status) {
  std::lock_guard<std::mutex> lock(pool.mu);
  b->held = false;
  return status;
}

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
  if (b->used && b->last_stream != stream && hipStreamWaitEvent(stream, b->ev, 0) != hipSuccess)
    return scratch_abandon(pool, b, EP_ERR_HIP);
  if (b->cap < bytes) {
    // the old block may still be read by kernels queued on `stream` (ordered
    // after the wait above): free it stream-ordered, then take a bigger one
    if (b->ptr && hipFreeAsync(b->ptr, stream) != hipSuccess) return scratch_abandon(pool, b, EP_ERR_HIP);
    b->ptr = nullptr;
    b->cap = 0;
    const size_t cap = bytes + bytes / 4;
    if (hipMallocAsync(&b->ptr, cap, stream) != hipSuccess || !b->ptr) {
      b->ptr = nullptr;
      return scratch_abandon(pool, b, EP_ERR_WORKSPACE);
    }
    b->cap = cap;
  }
  if (!b->ev && hipEventCreateWithFlags(&b->ev, hipEventDisableTiming) != hipSuccess)
    return scratch_abandon(pool, b, EP_ERR_HIP);
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

// Scratch of ep_count_episodes_noalloc: one fixed array per device, in the
// library's code object (the loader places it when the code object is loaded
// on a device, and it stays until the process ends).  Host code never passes
// the array's name to a kernel: it takes the array's device address once per
// device with hipGetSymbolAddress and uses that address everywhere.  Calls
// share the array; calls that overlap on one device race.
constexpr size_t kNoAllocScratchBytes = EP_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_noalloc_mu;
void* g_noalloc_ptr[64] = {};

// The device address of `scratch` on device `dev` (current), taken on first use.
int noalloc_scratch(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return EP_ERR_HIP;
    g_noalloc_ptr[dev] = p;
  }
  *out = g_noalloc_ptr[dev];
  return EP_OK;
}

// Profiling session: per counting call, events around its phases.  Events
// come from a pool that lives as long as the process, so recording adds no
// event creation to the timed calls once the pool is warm.
constexpr int kProfEvents = 8;
struct ProfRecord {
  // start, before Map (the filter), after the filter, after the list
  // pruning (before the tick Map kernel), after it, after Map, after closure,
  // after Concatenate
  hipEvent_t ev[kProfEvents];
  hipEvent_t end;
  int which;  // -1: every phase; else the one Map kernel timed (EP_PROFILE_*)
};
std::mutex g_prof_mu;
bool g_prof_on = false;
int g_prof_which = -1;   // -1: every phase of every call
int g_prof_every = 1;    // one call in this many is recorded
int64_t g_prof_calls = 0;

// the event before one timed Map kernel (EP_PROFILE_*); the next one follows it
int prof_first(int which) {
  switch (which) {
    case EP_PROFILE_FILTER: return 1;
    case EP_PROFILE_PRUNE: return 2;
    case EP_PROFILE_TICKS: return 3;
    default: return 4;
  }
}
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
constexpr int64_t kStreamSegEvents = 4096;
constexpr int64_t kListMinEvents = 1 << 20;  // the list path pays off from streams of about this size  // a stream batch's segments hold about this many events at most

// The hybrid rule (hybrid-algorithm section): PTPE when the episodes alone
// give every resident lane of every CU work, here kPtpeFill times over;
// otherwise MapConcatenate with the smallest power-of-two P that gives every
// lane work, kept to >= 256 events per segment on average (>= 64 with fewer
// than 256 episodes, where the lanes are few) and P <= 2^20.  The factor is
// measured: on MI355X (196,608 resident tick-kernel lanes, 1M events, four
// nodes) MapConcatenate was faster at every episode count up to 1,048,576
// (5.3 x the lanes) and PTPE at 2,097,152 (10.7 x); a segment shares its
// type bitmaps over all episodes of a workgroup, so PTPE's one pass per lane
// over the whole stream pays off only far beyond one lane per episode.
constexpr int64_t kPtpeFill = 6;
int plan_rule(int64_t S, int32_t N, int64_t n, int32_t mode, int32_t n_segments, int32_t cu_count,
              int32_t lanes_per_cu, int32_t* out_mode, int32_t* out_segments) {
  const int64_t full = (int64_t)std::max(cu_count, 1) * std::max(lanes_per_cu, 1);
  int m = mode;
  if (m == EP_MODE_AUTO) m = (S >= kPtpeFill * full) ? EP_MODE_PTPE : EP_MODE_MAPCONCAT;
  int64_t P = 1;
  if (m == EP_MODE_MAPCONCAT) {
    if (n_segments > 0) {
      P = n_segments;
    } else {
      const int64_t per_seg = std::max<int64_t>(S, 1) * (N <= kMaxClassNodes ? 1 : N);
      const int64_t need = (full + per_seg - 1) / per_seg;
      const int64_t cap_by_events = std::max<int64_t>(1, n / (S < 256 ? 64 : 256));
      P = 2;
      while (P < need && P < (1 << 20)) P <<= 1;
      // keep segments to <= 32,768 events on average: a repair rescans one segment
      while (P * 32768 < n && P < (1 << 20)) P <<= 1;
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
    case EP_ERR_UNSUPPORTED: return "more candidates than max_candidates";
    case EP_ERR_SCRATCH_LIMIT: return "the call needs more scratch than the fixed array of ep_count_episodes_noalloc holds";
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

// EP_LOG (read once): print each call's plan and the HIP failures on stderr
bool log_on() {
  static const bool on = getenv("EP_LOG") != nullptr;
  return on;
}

#define EP_HIP(call)                                      \
  do {                                                    \
    hipError_t err_ = (call);                             \
    if (err_ != hipSuccess) {                             \
      if (log_on())                                       \
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
// waits until its next slot's previous reader has finished and hands out the
// slot (host and device addresses); staging_release() records the slot's
// event after the work that reads it (the set-up kernel copies it to the
// device) and unlocks.  Every acquire is followed by exactly one release.
// The slots are coherent host memory, so a kernel reads what the host wrote
// even when a slot comes round again.
int staging_acquire(int dev, size_t bytes, char** out, const void** dout) {
  Staging& st = g_staging[dev];
  st.mu.lock();
  StagingSlot& s = st.slot[st.next];
  int status = EP_OK;
  if (s.pending) {
    if (hipEventSynchronize(s.ev) != hipSuccess) status = EP_ERR_HIP;
    s.pending = false;
  }
  if (status == EP_OK && s.cap < bytes) {
    if (s.buf) (void)hipHostFree(s.buf);
    s.buf = nullptr;
    s.dbuf = nullptr;
    s.cap = 0;
    const size_t cap = std::max<size_t>(bytes, 1 << 16);
    if (hipHostMalloc(&s.buf, cap, hipHostMallocCoherent) != hipSuccess) {
      s.buf = nullptr;
      status = EP_ERR_HIP;
    } else if (hipHostGetDevicePointer(&s.dbuf, s.buf, 0) != hipSuccess || !s.dbuf) {
      (void)hipHostFree(s.buf);
      s.buf = nullptr;
      s.dbuf = nullptr;
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
  *dout = s.dbuf;
  return EP_OK;
}

// `used`: work reading the slot was enqueued on `stream` (record its event).
int staging_release(int dev, bool used, hipStream_t stream) {
  Staging& st = g_staging[dev];
  StagingSlot& s = st.slot[st.next];
  int status = EP_OK;
  if (used) {
    if (hipEventRecord(s.ev, stream) != hipSuccess)
      status = EP_ERR_HIP;
    else
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
    case kRing: return "ring";
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
  bool prune;      // list path: the filter's lists pruned before the list Map kernel
  bool slice;      // two-node episodes: every segment through the type-sliced kernel
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

// A counting call made for one batch of an ep_stream (see stream_entry_kernel):
// the carried reset times, the running counts, where to write the new reset
// times, and the first and last event times of the call's events.
struct StreamHook {
  const int64_t* entry;
  int64_t* total;
  int64_t* reset_out;
  int64_t t_first;
  int64_t t_end;
};

// Tables of the type-sliced two-node kernel (map_slice_kernel): episodes
// grouped by (node-0 type word, node-1 type, lo, hi), node-0 types ranked and
// cut into words of 64 bits; groups of one word padded to whole workgroups.
struct SliceHost {
  std::vector<SliceGroup> groups;
  std::vector<uint64_t> mask;
  std::vector<int32_t> ep;    // 64 per group
  std::vector<uint16_t> tab;  // kSliceTypes per workgroup
  int64_t real_groups = 0;
  int wg_groups = 0, n_wg = 0, n_brows = 0;
};

// Average episodes per group from which the planner takes the sliced kernel
// (a group's lane steps its word of node-0 types at every node-1 tick).
constexpr int64_t kSliceMinFill = 8;
// A workgroup of the sliced kernel steps one segment's events in order: the
// kernel is taken where its workgroups (segments x workgroups per segment)
// fill the CUs, or where segments are short enough that a few workgroups
// finish quickly (PTPE's single segment over a long stream is neither: the
// level-2 sweep took 476 ms there against 63 ms on the tick kernel).
constexpr int64_t kSliceShortSegment = 1 << 16;  // events per segment

// false when the call does not fit the kernel: a node type >= kSliceTypes,
// an episode given twice, or a window wider than 63 ticks
bool slice_plan(const ep_episodes& eps, int64_t S, int n_machines, SliceHost* out) {
  if (eps.n_nodes != 2 || S <= 0 || S >= (1 << 30)) return false;
  std::vector<int32_t> a_rank((size_t)kSliceTypes, -1);
  for (int64_t e = 0; e < S; ++e) {
    const int a = eps.types[e * 2], b = eps.types[e * 2 + 1];
    if (a >= kSliceTypes || b >= kSliceTypes || eps.t_high[e] > 63) return false;
    a_rank[(size_t)a] = 0;
  }
  int32_t r = 0;
  for (int y = 0; y < kSliceTypes; ++y)
    if (a_rank[(size_t)y] == 0) a_rank[(size_t)y] = r++;
  // one sort key per episode: group (word, node-1 type, lo, hi: 28 bits), then
  // node-0 bit (6), then the episode (30)
  std::vector<uint64_t> keyed((size_t)S);
  for (int64_t e = 0; e < S; ++e) {
    const uint64_t ra = (uint64_t)a_rank[eps.types[e * 2]];
    const uint64_t gk = (((ra >> 6) * kSliceTypes + eps.types[e * 2 + 1]) * 64 + (uint64_t)eps.t_low[e]) * 64 +
                        (uint64_t)eps.t_high[e];
    keyed[(size_t)e] = (((gk << 6) | (ra & 63)) << 30) | (uint64_t)e;
  }
  std::sort(keyed.begin(), keyed.end());
  const int wg = kBlock / n_machines;
  SliceHost& h = *out;
  h = SliceHost();
  h.wg_groups = wg;
  h.groups.reserve((size_t)S);
  h.mask.reserve((size_t)S);
  std::vector<int32_t> g_word;  // node-0 word of each group (-1: padding)
  int32_t word = -1;
  uint64_t prev_gk = ~0ull;
  int prev_bit = -1;
  auto add_group = [&](SliceGroup sg, int32_t wd) {
    h.groups.push_back(sg);
    h.mask.push_back(0ull);
    h.ep.resize(h.ep.size() + 64, -1);
    g_word.push_back(wd);
  };
  for (size_t i = 0; i < keyed.size(); ++i) {
    const uint64_t gk = keyed[i] >> 36;
    const int bit = (int)((keyed[i] >> 30) & 63);
    const int64_t e = (int64_t)(keyed[i] & ((1ull << 30) - 1));
    if (gk == prev_gk && bit == prev_bit) return false;  // an episode given twice
    if (gk != prev_gk) {
      const int32_t wd = (int32_t)(gk / ((uint64_t)kSliceTypes * 64 * 64));
      if (wd != word) {
        // a new node-0 word starts a new workgroup
        while (!h.groups.empty() && h.groups.size() % wg) add_group(SliceGroup{0, 1, 0, 0}, -1);
        word = wd;
      }
      add_group(SliceGroup{eps.t_low[e], eps.t_high[e], 0, (int32_t)eps.types[e * 2 + 1]}, word);
      ++h.real_groups;
      prev_gk = gk;
    }
    prev_bit = bit;
    h.mask.back() |= 1ull << bit;
    h.ep[(h.groups.size() - 1) * 64 + bit] = (int32_t)e;
  }
  const int64_t ng = (int64_t)h.groups.size();
  h.n_wg = (int)((ng + wg - 1) / wg);
  h.tab.assign((size_t)h.n_wg * kSliceTypes, 0);
  h.n_brows = 1;
  for (int w = 0; w < h.n_wg; ++w) {
    uint16_t* tab = h.tab.data() + (size_t)w * kSliceTypes;
    int32_t wword = -1, rows = 0;
    for (int64_t g = (int64_t)w * wg; g < std::min<int64_t>(ng, (int64_t)(w + 1) * wg); ++g) {
      if (g_word[(size_t)g] < 0) continue;
      wword = g_word[(size_t)g];
      // the node-1 type is parked in pad until its row is known
      const int32_t b = h.groups[(size_t)g].pad;
      if ((tab[b] >> 7) == 0) tab[b] = (uint16_t)(tab[b] | ((rows++ + 1) << 7));
      h.groups[(size_t)g].brow = (tab[b] >> 7) - 1;
      h.groups[(size_t)g].pad = 0;
    }
    if (wword >= 0)
      for (int y = 0; y < kSliceTypes; ++y)
        if (a_rank[(size_t)y] >= 0 && (a_rank[(size_t)y] >> 6) == wword)
          tab[y] = (uint16_t)(tab[y] | ((a_rank[(size_t)y] & 63) + 1));
    h.n_brows = std::max(h.n_brows, rows);
  }
  return true;
}

// Window kind each episode needs: bit windows when every t_high <= 63, run
// windows in registers when every interval's live-run bound
// floor(t_high / (t_high - t_low + 1)) + 1 is at most EP_MAX_RUNS, ring
// windows otherwise.
enum { kClsBits = 0, kClsRuns = 1, kClsRing = 2, kNumCls = 3 };

// Largest ring-window arena a call plans for: MapConcatenate's P is lowered
// until every Map machine's rings fit (a caller's fixed P is kept).
constexpr double kRingBudget = 2.0 * (1ull << 30);

int count_episodes_impl(const int32_t* times, const uint16_t* types, int64_t n_events,
                        ep_episodes episodes, int64_t n_episodes, int64_t* out_counts,
                        hipStream_t stream, const ep_options* opt, const StreamHook* sh = nullptr,
                        const int32_t* out_map = nullptr, bool no_alloc = false);

// A call whose episodes need different window kinds: one sub-call per kind,
// each over its own episodes and writing their counts through an index map
// into the caller's out_counts (the sub-calls' outputs are disjoint).
int count_split(const int32_t* times, const uint16_t* types, int64_t n_events, ep_episodes episodes,
                int64_t S, int64_t* out_counts, hipStream_t stream, const ep_options* opt,
                const std::vector<uint8_t>& cls, bool no_alloc) {
  const int32_t N = episodes.n_nodes;
  const int NI = N - 1;
  ep_stats acc{};
  int64_t most = -1;
  bool first = true;
  for (int c = 0; c < kNumCls; ++c) {
    std::vector<int32_t> idx;
    for (int64_t e = 0; e < S; ++e)
      if (cls[(size_t)e] == c) idx.push_back((int32_t)e);
    if (idx.empty()) continue;
    const int64_t Sc = (int64_t)idx.size();
    std::vector<uint16_t> ty((size_t)(Sc * N));
    std::vector<int32_t> lo((size_t)(Sc * NI)), hi((size_t)(Sc * NI));
    for (int64_t i = 0; i < Sc; ++i) {
      const int64_t e = idx[(size_t)i];
      memcpy(ty.data() + i * N, episodes.types + e * N, sizeof(uint16_t) * N);
      if (NI > 0) {
        memcpy(lo.data() + i * NI, episodes.t_low + e * NI, sizeof(int32_t) * NI);
        memcpy(hi.data() + i * NI, episodes.t_high + e * NI, sizeof(int32_t) * NI);
      }
    }
    ep_episodes sub{N, ty.data(), NI > 0 ? lo.data() : nullptr, NI > 0 ? hi.data() : nullptr};
    ep_options o{};
    if (opt) o = *opt;
    o.upper_only = 0;  // the table passed in already holds the relaxed bounds
    o.validate = first && opt ? opt->validate : 0;
    ep_stats st{};
    o.stats = (opt && opt->stats) ? &st : nullptr;
    if (int status = count_episodes_impl(times, types, n_events, sub, Sc, out_counts, stream, &o, nullptr,
                                         idx.data(), no_alloc))
      return status;
    first = false;
    if (opt && opt->stats) {
      if (Sc > most) {
        most = Sc;
        acc.mode = st.mode;
        acc.n_segments = st.n_segments;
        acc.max_runs = st.max_runs;
      }
      acc.kernels |= st.kernels;
      acc.repairs += st.repairs;
      acc.fallbacks += st.fallbacks;
      acc.groups += 1;
    }
  }
  if (opt && opt->stats) *opt->stats = acc;
  return EP_OK;
}

int count_episodes_impl(const int32_t* times, const uint16_t* types, int64_t n_events,
                        ep_episodes episodes, int64_t n_episodes, int64_t* out_counts,
                        hipStream_t stream, const ep_options* opt, const StreamHook* sh,
                        const int32_t* out_map, bool no_alloc) {
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
  const uint32_t plan = opt ? opt->plan : 0u;

  int64_t max_span = 0, max_hi = 0;
  int64_t max_bound = 1;  // most live runs any window can hold
  int dil_k = 0;  // doubling steps of the tick kernel's dilation (windows up to 63 ticks)
  std::vector<uint8_t> cls((size_t)S);
  int cls_seen = 0;  // bit c: some episode needs window kind c
  for (int64_t e = 0; e < S; ++e) {
    int64_t span = 0, ep_hi = 0, ep_bound = 1;
    for (int j = 0; j < N - 1; ++j) {
      const int64_t lo = episodes.t_low[e * (N - 1) + j];
      const int64_t hi = episodes.t_high[e * (N - 1) + j];
      if (lo < 0 || lo >= hi) return EP_ERR_INTERVAL;
      span += hi;
      ep_hi = std::max(ep_hi, hi);
      if (hi <= 63) dil_k = std::max(dil_k, dil_steps((uint32_t)lo, (uint32_t)hi));
      // live disjoint runs of a window: at most floor(hi / (hi - lo + 1)) + 1
      ep_bound = std::max(ep_bound, hi / (hi - lo + 1) + 1);
    }
    if (span > INT32_MAX) return EP_ERR_INTERVAL;
    max_span = std::max(max_span, span);
    max_hi = std::max(max_hi, ep_hi);
    max_bound = std::max(max_bound, ep_bound);
    int c = ep_hi <= 63 ? kClsBits : (ep_bound <= EP_MAX_RUNS ? kClsRuns : kClsRing);
    if (plan & EP_PLAN_RUN_WINDOWS) c = ep_bound <= EP_MAX_RUNS ? kClsRuns : kClsRing;
    if (plan & EP_PLAN_RING_WINDOWS) c = kClsRing;
    cls[(size_t)e] = (uint8_t)c;
    cls_seen |= 1 << c;
  }
  if (S == 0) return EP_OK;
  if (!sh && !out_map && !(plan & EP_PLAN_NO_SPLIT) && n_events > 0 && __builtin_popcount(cls_seen) > 1)
    return count_split(times, types, n_events, episodes, S, out_counts, stream, opt, cls, no_alloc);
  // window kind of the call: the widest any of its episodes needs
  const int K = max_bound <= 1 ? 1 : (max_bound <= 2 ? 2 : 4);
  const int run_win = max_bound <= EP_MAX_RUNS ? (K == 1 ? kRuns1 : (K == 2 ? kRuns2 : kRuns4)) : kRing;
  int win;
  if (cls_seen == (1 << kClsBits))
    win = max_hi <= 31 ? kBits32 : kBits64;
  else if (cls_seen & (1 << kClsRing))
    win = kRing;
  else
    win = run_win;
  // ring capacity: the live-run bound, and never more runs than events
  uint32_t ring_cap = 1;
  while ((int64_t)ring_cap < std::min<int64_t>(max_bound, std::max<int64_t>(n_events, 1))) ring_cap <<= 1;

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
      opt->stats->max_runs = win == kBits32 ? 32 : win == kBits64 ? 64 : win == kRing ? (int32_t)ring_cap : K;
      opt->stats->groups = 1;
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
  L.bits = (win == kBits32 || win == kBits64) && U <= 255;
  // many node types: the scan kernel with bit windows is not built; runs or rings
  if (!L.bits && (win == kBits32 || win == kBits64)) L.win = run_win;
  // lanes one CU holds for the counting kernel (the hybrid rule's T_B * B_MP):
  // the tick kernel's workgroups per CU as its registers allow, times its
  // threads, for bit windows; 8 waves on each of 4 SIMDs otherwise
  int lanes_per_cu_est = 2048;
  if (L.bits) {
    std::lock_guard<std::mutex> lock(g_info_mu);
    int& lanes = info->plan_lanes[N];
    if (lanes == 0) {
      int per_cu = 0;
      if (Lr->occupancy_ticks(N <= kMaxClassNodes, kBlock, 0, &per_cu) != hipSuccess || per_cu < 1)
        per_cu = 2048 / kBlock;
      lanes = std::min(per_cu * kBlock, 2048);
    }
    lanes_per_cu_est = lanes;
  }
  int32_t pmode = 0, P = 1;
  plan_rule(S, N, n_events, sh ? EP_MODE_MAPCONCAT : mode, opt ? opt->n_segments : 0,
            info->cu_count, lanes_per_cu_est, &pmode, &P);
  if (sh) {
    // a batch of a stream: the entry and tail kernels scan segment 0 and the
    // last segment with one wave per episode, so segments of at most about
    // kStreamSegEvents events unless the caller fixed P; and segments longer
    // than maxSpan ticks (see the tail)
    if (!(opt && opt->n_segments > 0))
      P = (int32_t)std::max<int64_t>(P, std::min<int64_t>((n_events + kStreamSegEvents - 1) / kStreamSegEvents,
                                                         INT32_MAX));
    const int64_t cap = std::max<int64_t>(1, (sh->t_end - sh->t_first + 1) / (max_span + 1));
    P = (int32_t)std::min<int64_t>(P, cap);
  }
  // ring windows: every Map machine owns N-1 rings of ring_cap runs
  const double ring_slot_bytes = (double)std::max(N - 1, 1) * ring_cap * sizeof(int2);
  if (L.win == kRing && !(opt && opt->n_segments > 0)) {
    const double per_p = (double)S * (pmode == EP_MODE_PTPE ? 1 : N) * ring_slot_bytes;
    while (P > 1 && (double)P * per_p > kRingBudget) P >>= 1;
  }
  // the fixed scratch array of ep_count_episodes_noalloc: fewer segments
  // until the tuple store (and the rings) fit beside the lists and the table
  if (no_alloc && !(opt && opt->n_segments > 0) && pmode == EP_MODE_MAPCONCAT) {
    const double fixed = (S <= kMaxListEpisodes ? list_bytes + 2.0 * n_lblocks * S * 4 : 0.0) +
                         (double)S * (N * 2 + 24) + 2048 * 8 + 65536 * 8 + (1 << 20);
    const double per_p = (double)S * (16.0 * 2 * N + 8) + 16 +
                         (L.win == kRing ? (double)S * N * ring_slot_bytes : 0.0);
    while (P > 1 && fixed + (double)P * per_p > (double)kNoAllocScratchBytes) P >>= 1;
  }
  L.mode = pmode;
  L.P = P;
  L.n_machines = (pmode == EP_MODE_PTPE) ? 1 : N;
  L.block = kBlock;
  if (L.bits) {
    // one lane per (segment, episode) holding every machine, unless that
    // leaves the GPU with too few lanes for a fixed segment count
    const int64_t target = (int64_t)info->cu_count * lanes_per_cu_est;
    L.split = (plan & EP_PLAN_TICKS) ? 1 : ((plan & EP_PLAN_POSITIONS) ? 2 : 0);
    // few episodes: sparse segments read the filter kernel's per-episode lists
    // (one lane per (segment, episode) walks only its episode's events)
    // (on short streams the position kernel, which stages events in LDS, is
    // faster than a filter pass plus lanes reading lists)
    L.list = S <= kMaxListEpisodes && L.split != 1 && list_bytes <= kMaxListBytes &&
             (n_events >= kListMinEvents || (plan & EP_PLAN_LIST)) && !(plan & EP_PLAN_NO_LIST);
    L.all_mach = L.n_machines > 1 && N <= kMaxClassNodes && (L.list || S * (int64_t)P * 4 >= target);
    if (plan & EP_PLAN_MACHINE_LANES) L.all_mach = false;
    L.M = L.all_mach ? 1 : L.n_machines;
    // pruning the lists pays where the list kernel has too few lanes (under
    // two waves per SIMD) to hide their serial walks: it shortens every walk;
    // with more lanes the list kernel is bound by its total work, which
    // pruning cuts by less than pruning itself costs per block
    const int64_t list_lanes = (int64_t)P * S * L.M;
    L.prune = L.list && ((list_lanes < (int64_t)info->cu_count * 4 * 2 * kWave && !(plan & EP_PLAN_NO_PRUNE)) ||
                         (plan & EP_PLAN_PRUNE));
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
    L.prune = false;
    L.all_mach = false;
    L.M = L.n_machines;
    L.G = (int)std::min<int64_t>(S, L.block / L.M);
    L.R = (L.G == S) ? std::max(1, L.block / (L.G * L.M)) : 1;
    L.R = (int)std::min<int64_t>(L.R, P);
    L.CH = kTile / L.R;
    L.lds = 0;
  }
  L.slots = (pmode == EP_MODE_PTPE) ? 1 : 2 * N;
  // two-node episodes: the type-sliced kernel takes every segment where the
  // episodes fill its words (or where a plan switch asks for it; the switches
  // that force another Map kernel keep it out)
  SliceHost slc;
  L.slice = false;
  {
    const uint32_t other = EP_PLAN_TICKS | EP_PLAN_POSITIONS | EP_PLAN_LIST | EP_PLAN_MACHINE_LANES |
                           EP_PLAN_NO_SLICE;
    const bool wanted = (plan & EP_PLAN_SLICE) || !(plan & other);
    if (N == 2 && L.bits && wanted && slice_plan(episodes, S, L.n_machines, &slc) &&
        ((plan & EP_PLAN_SLICE) ||
         (S >= kSliceMinFill * slc.real_groups &&
          ((int64_t)P * slc.n_wg >= info->cu_count || n_events <= (int64_t)P * kSliceShortSegment)))) {
      L.slice = true;
      L.list = false;
      L.prune = false;
      L.split = 1;
    }
  }
  if (log_on())
    fprintf(stderr,
            "epcount: S=%lld N=%d n=%lld U=%d mode=%s P=%d win=%s kernel=%s lanes=%s M=%d G=%d R=%d "
            "CH=%d lds=%zu maxSpan=%lld ring=%u slice=%d groups=%lld wg=%d rows=%d\n",
            (long long)S, N, (long long)n_events, U, pmode == EP_MODE_PTPE ? "ptpe" : "mapconcat", P,
            win_name(L.win), L.bits ? "bits" : "scan", L.all_mach ? "class" : "machine", L.M, L.G, L.R,
            L.CH, L.lds, (long long)max_span, L.win == kRing ? ring_cap : 0u, L.slice ? 1 : 0,
            (long long)slc.real_groups, slc.n_wg, slc.n_brows);

  // tick kernel: episodes ordered by their doubling steps, so that an episode
  // group of narrow windows runs fewer steps than the call's widest needs
  // (only where the steps differ, there are several groups, and the tick
  // kernel's work, about episodes x events, is large enough to repay the
  // ordering's host time)
  std::vector<int32_t> ep_perm, group_k;
  if (L.bits && !L.slice && L.split != 2 && S > L.G &&
      ((double)S * (double)n_events >= 4294967296.0 || (plan & EP_PLAN_GROUP_STEPS))) {
    std::vector<int32_t> steps((size_t)S, 0);
    int32_t lo_k = INT32_MAX, hi_k = 0;
    for (int64_t e = 0; e < S; ++e) {
      int32_t k = 0;
      for (int j = 0; j < N - 1; ++j)
        k = std::max(k, dil_steps((uint32_t)episodes.t_low[e * (N - 1) + j],
                                  (uint32_t)episodes.t_high[e * (N - 1) + j]));
      steps[(size_t)e] = k;
      lo_k = std::min(lo_k, k);
      hi_k = std::max(hi_k, k);
    }
    if (lo_k < hi_k && !(plan & EP_PLAN_NO_GROUP_STEPS)) {
      // a counting sort (steps are 0 .. 6), stable
      int64_t at[8] = {0};
      for (int64_t e = 0; e < S; ++e) ++at[steps[(size_t)e] + 1];
      for (int k = 1; k < 8; ++k) at[k] += at[k - 1];
      ep_perm.resize((size_t)S);
      for (int64_t e = 0; e < S; ++e) ep_perm[(size_t)at[steps[(size_t)e]]++] = (int32_t)e;
      const int64_t groups = (S + L.G - 1) / L.G;
      group_k.assign((size_t)groups, 0);
      for (int64_t i = 0; i < S; ++i)
        group_k[(size_t)(i / L.G)] = std::max(group_k[(size_t)(i / L.G)], steps[(size_t)ep_perm[(size_t)i]]);
    }
  }

  // ---- scratch layout (one stream-ordered allocation)
  const size_t sz_types = align_up(sizeof(uint16_t) * S * N, 256);
  const size_t sz_lohi = align_up(sizeof(int32_t) * S * std::max(N - 1, 1), 256);
  const size_t sz_span = align_up(sizeof(int32_t) * S, 256);
  const size_t sz_slot = align_up((size_t)S * N, 256);
  const size_t sz_seen = sizeof(uint64_t) * 1024;  // node types as a 65,536-bit set
  const size_t sz_rank = 1024;                       // set bits before each 64-bit word
  const size_t sz_seps = L.list ? sizeof(uint32_t) * 256 : 0;
  const size_t sz_slv = L.list ? align_up(sizeof(uint16_t) * 256 * S, 256) : 0;
  const size_t sz_perm = align_up(sizeof(int32_t) * ep_perm.size(), 256);
  const size_t sz_gk = align_up(sizeof(int32_t) * group_k.size(), 256);
  const size_t sz_sgrp = L.slice ? align_up(sizeof(SliceGroup) * slc.groups.size(), 256) : 0;
  const size_t sz_smask = L.slice ? align_up(sizeof(uint64_t) * slc.mask.size(), 256) : 0;
  const size_t sz_sep = L.slice ? align_up(sizeof(int32_t) * slc.ep.size(), 256) : 0;
  const size_t sz_stab = L.slice ? align_up(sizeof(uint16_t) * slc.tab.size(), 256) : 0;
  const size_t sz_slice = sz_sgrp + sz_smask + sz_sep + sz_stab;
  const size_t sz_omap = out_map ? align_up(sizeof(int32_t) * S, 256) : 0;
  const size_t host_bytes = sz_types + 2 * sz_lohi + sz_span + sz_slot + sz_seen + sz_rank + sz_seps + sz_slv +
                            sz_perm + sz_gk + sz_slice + sz_omap;
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
  // closure misses queued for repair_kernel (more are repaired where found)
  // misses past the queue send their episode to the whole-stream recount
  const int64_t queue_cap = P > 1 ? 262144 : 0;
  const size_t sz_queue = align_up(sizeof(uint64_t) * (size_t)queue_cap, 256);
  // ring windows: a slot per Map machine (scan kernel) and per wave of the
  // kernels that run one machine per wave (closure, repair, result, fused
  // reduction, stream entry and tail); the kernels run one after another
  RingArena ring{nullptr, 0, 1, 0};
  if (L.win == kRing) {
    int red_waves = 1;
    while (red_waves * kWave < P) red_waves <<= 1;
    int64_t slots = (int64_t)P * S * L.M;
    slots = std::max<int64_t>(slots, ((S + 3) / 4) * 4);             // finish, stream entry and tail
    slots = std::max<int64_t>(slots, S * (int64_t)red_waves);          // fused reduction
    if (P > 1) {
      slots = std::max<int64_t>(slots, grid_for((int64_t)(P - 1) * S) * (kBlock / kWave));  // closure
      slots = std::max<int64_t>(slots, (int64_t)info->cu_count * 2 * (kBlock / kWave));      // repair
    }
    ring.stride = (int64_t)std::max(N - 1, 1) * ring_cap;
    ring.cap = ring_cap;
    ring.slots = slots;
  }
  const size_t sz_ring = L.win == kRing ? align_up(sizeof(int2) * (size_t)ring.slots * ring.stride, 256) : 0;
  const size_t total =
      host_bytes + sz_tau + 2 * sz_seg + sz_tuples + 2 * sz_nslots + sz_flags + sz_cnt + sz_queue + sz_lists +
      2 * sz_lidx + sz_ring;

  mark();  // plan
  ScratchBlock* block = nullptr;
  char* ws = nullptr;
  if (no_alloc) {
    // the fixed array: nothing is allocated, a call that needs more is refused
    if (total > kNoAllocScratchBytes) return EP_ERR_SCRATCH_LIMIT;
    void* base = nullptr;
    if (int st = noalloc_scratch(dev, &base)) return st;
    ws = (char*)base;
  } else {
    if (int st = scratch_acquire(dev, total, stream, &block)) return st;
    ws = (char*)block->ptr;
  }
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
    int32_t* d_perm = (int32_t*)(ws + off); off += sz_perm;
    int32_t* d_gk = (int32_t*)(ws + off); off += sz_gk;
    SliceGroup* d_sgrp = (SliceGroup*)(ws + off); off += sz_sgrp;
    uint64_t* d_smask = (uint64_t*)(ws + off); off += sz_smask;
    int32_t* d_sep = (int32_t*)(ws + off); off += sz_sep;
    uint16_t* d_stab = (uint16_t*)(ws + off); off += sz_stab;
    int32_t* d_omap = (int32_t*)(ws + off); off += sz_omap;
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
    uint64_t* d_queue = (uint64_t*)(ws + off); off += sz_queue;
    int2* d_lists = (int2*)(ws + off); off += sz_lists;
    int32_t* d_loff = (int32_t*)(ws + off); off += sz_lidx;
    int32_t* d_lcnt = (int32_t*)(ws + off); off += sz_lidx;
    ring.base = (int2*)(ws + off); off += sz_ring;

    // episode table, spans, node slots and the node-type set, written
    // straight into pinned staging; the set-up kernel copies it to the device
    // (no_alloc: written into a host buffer of the calling thread and copied
    // to the scratch array ahead of the set-up kernel, on the stream)
    const void* tab_dev = nullptr;
    bool staged = false;  // a staging slot is held (released after the set-up launch)
    thread_local std::vector<char> na_host;
    auto release_staging = [&](bool used) -> int {
      if (!staged) return EP_OK;
      staged = false;
      return staging_release(dev, used, stream);
    };
    {
      char* host = nullptr;
      if (no_alloc) {
        if (na_host.size() < host_bytes) na_host.resize(host_bytes);
        host = na_host.data();
      } else {
        if ((status = staging_acquire(dev, host_bytes, &host, &tab_dev))) break;
        staged = true;
      }
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
      if (!ep_perm.empty()) {
        char* at = host + sz_types + 2 * sz_lohi + sz_span + sz_slot + sz_seen + sz_rank + sz_seps + sz_slv;
        memcpy(at, ep_perm.data(), sizeof(int32_t) * ep_perm.size());
        memcpy(at + sz_perm, group_k.data(), sizeof(int32_t) * group_k.size());
      }
      if (L.slice) {
        char* at = host + sz_types + 2 * sz_lohi + sz_span + sz_slot + sz_seen + sz_rank + sz_seps + sz_slv +
                   sz_perm + sz_gk;
        memcpy(at, slc.groups.data(), sizeof(SliceGroup) * slc.groups.size());
        memcpy(at + sz_sgrp, slc.mask.data(), sizeof(uint64_t) * slc.mask.size());
        memcpy(at + sz_sgrp + sz_smask, slc.ep.data(), sizeof(int32_t) * slc.ep.size());
        memcpy(at + sz_sgrp + sz_smask + sz_sep, slc.tab.data(), sizeof(uint16_t) * slc.tab.size());
      }
      if (out_map)
        memcpy(host + (host_bytes - sz_omap), out_map, sizeof(int32_t) * S);
      // pageable source: the copy has read it before the call returns
      if (no_alloc && hipMemcpyAsync(ws, host, host_bytes, hipMemcpyHostToDevice, stream) != hipSuccess) {
        status = EP_ERR_HIP;
        break;
      }
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
        release_staging(false);
        break;
      }
      if (bad) {
        status = EP_ERR_UNSORTED;
        release_staging(false);
        break;
      }
    }

    mark();  // upload
    bool prof = false;
    int prof_which = -1;
    ProfRecord rec{};
    {
      std::lock_guard<std::mutex> lock(g_prof_mu);
      if (g_prof_on && !no_alloc) {  // (events come from a pool that may grow)
        prof_which = g_prof_which;
        prof = (g_prof_calls++ % g_prof_every) == 0;
      }
    }
    if (prof && (status = prof_record_start(&rec, prof_which, stream))) {
      release_staging(false);
      break;
    }
    // records boundary i when the session times it (every boundary, or the
    // two around the one Map kernel it times)
    auto rec_at = [&](int i) {
      if (prof && (prof_which < 0 || i == prof_first(prof_which) || i == prof_first(prof_which) + 1))
        (void)hipEventRecord(rec.ev[i], stream);
    };
    SetupArgs sa;
    sa.times = times; sa.n = n_events; sa.P = P; sa.max_span = max_span;
    sa.tau = d_tau; sa.beg = d_beg; sa.end = d_end;
    sa.flags = d_flags; sa.S = S; sa.counters = d_cnt;
    sa.flag_init = (plan & EP_PLAN_RECOUNT) ? 1 : 0;
    sa.wave_search = P <= kWaveSearchMaxP ? 1 : 0;
    sa.tab_src = (const uint4*)tab_dev;
    sa.tab_dst = (uint4*)ws;
    sa.tab_words = no_alloc ? 0 : (int64_t)(host_bytes / sizeof(uint4));
    hipLaunchKernelGGL(setup_kernel, dim3(grid_for(setup_items(sa))), dim3(kBlock), 0, stream, sa);
    const bool launched = hipGetLastError() == hipSuccess;
    if (int st = release_staging(launched)) status = st;
    if (!launched) status = EP_ERR_HIP;
    if (status != EP_OK) break;

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
    ma.ep_perm = ep_perm.empty() ? nullptr : d_perm;
    ma.group_k = ep_perm.empty() ? nullptr : d_gk;
    ma.lists = d_lists; ma.list_off = d_loff; ma.list_cnt = d_lcnt; ma.max_share = max_share;
    ma.ring = ring;
    ma.lazy = L.prune ? 0 : 1;  // pruned lists: nearly every entry left changes the machine
    // workgroups: (segment group, episode group), episode group fastest
    ma.n_egroups = (S + L.G - 1) / L.G;
    dim3 mgrid((unsigned)(((P + L.R - 1) / L.R) * ma.n_egroups));
    // tick kernel: where a segment group fits one chunk, as few workgroups per
    // group as still fill every CU loop over its episode groups, building the
    // bitmaps once each (the kernel decides per group; the grid is mgrid)
    const int64_t seg_groups = (P + L.R - 1) / L.R;
    ma.eg_blocks = ma.n_egroups;
    if (L.bits && !L.slice && L.split != 2) {
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
    const bool skip_map = sh && P == 1;  // one segment of a stream: the tail counts it
    if (L.list && !skip_map) {
      FilterArgs fa;
      fa.times = times; fa.types = types; fa.n = n_events;
      fa.type_seen = d_seen; fa.type_rank = d_rank; fa.slot_eps = d_seps; fa.slot_levels = d_slv;
      fa.S = (int32_t)S; fa.max_share = max_share;
      fa.lists = d_lists; fa.list_off = d_loff; fa.list_cnt = d_lcnt;
      // persistent workgroups: a few per CU, each looping over blocks
      // (as many as fit a CU: the LDS per workgroup grows with S)
      const int64_t fgrid =
          std::min<int64_t>(n_lblocks, (int64_t)info->cu_count * (S <= 8 ? 4 : (S <= 16 ? 3 : 2)));
      const dim3 fg((unsigned)fgrid), fb(kBlock);
      // node types small enough for a direct type -> slot table in LDS
      int32_t type_cap = 0;
      for (int64_t i = 0; i < S * N; ++i) type_cap = std::max<int32_t>(type_cap, (int32_t)episodes.types[i] + 1);
      fa.type_cap = type_cap;
      const bool direct = type_cap <= kFilterTab;
      const int fgw = S <= 4 ? 1 : (S <= 8 ? 2 : (S <= 16 ? 4 : 8));
      switch (fgw * 2 + (direct ? 1 : 0)) {
        case 3: hipLaunchKernelGGL((filter_kernel<1, true>), fg, fb, 0, stream, fa); break;
        case 2: hipLaunchKernelGGL((filter_kernel<1, false>), fg, fb, 0, stream, fa); break;
        case 5: hipLaunchKernelGGL((filter_kernel<2, true>), fg, fb, 0, stream, fa); break;
        case 4: hipLaunchKernelGGL((filter_kernel<2, false>), fg, fb, 0, stream, fa); break;
        case 9: hipLaunchKernelGGL((filter_kernel<4, true>), fg, fb, 0, stream, fa); break;
        case 8: hipLaunchKernelGGL((filter_kernel<4, false>), fg, fb, 0, stream, fa); break;
        case 17: hipLaunchKernelGGL((filter_kernel<8, true>), fg, fb, 0, stream, fa); break;
        default: hipLaunchKernelGGL((filter_kernel<8, false>), fg, fb, 0, stream, fa); break;
      }
      le = hipGetLastError();
    }
    rec_at(2);
    if (L.prune && !skip_map && le == hipSuccess) {
      PruneArgs pa;
      pa.times = times; pa.n = n_events; pa.n_blocks = n_lblocks; pa.ep_lo = d_lo; pa.ep_hi = d_hi;
      pa.S = (int32_t)S; pa.N = N; pa.max_share = max_share;
      pa.lists = d_lists; pa.list_off = d_loff; pa.list_cnt = d_lcnt;
      // persistent workgroups: as many as are resident at once
      int prune_per_cu = 0;
      {
        std::lock_guard<std::mutex> lock(g_info_mu);
        if (info->prune_per_cu == 0) {
          int v = 0;
          if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, list_prune_kernel, kBlock, 0) == hipSuccess)
            info->prune_per_cu = std::max(v, 1);
        }
        prune_per_cu = info->prune_per_cu;
      }
      if (prune_per_cu == 0) {
        status = EP_ERR_HIP;
        break;
      }
      const int64_t pgrid = std::min<int64_t>(n_lblocks, (int64_t)info->cu_count * prune_per_cu);
      hipLaunchKernelGGL(list_prune_kernel, dim3((unsigned)pgrid), dim3(kBlock), 0, stream, pa);
      le = hipGetLastError();
    }
    rec_at(3);
    if (skip_map) {
      rec_at(4);
    } else if (le == hipSuccess && L.slice) {
      SliceArgs sl;
      sl.times = times; sl.types = types; sl.tau = d_tau; sl.seg_beg = d_beg; sl.seg_end = d_end;
      sl.ts = ts; sl.P = P; sl.n_machines = L.n_machines; sl.max_span = (int32_t)max_span;
      sl.n_groups = (int32_t)slc.groups.size(); sl.wg_groups = slc.wg_groups; sl.n_wg = slc.n_wg;
      sl.n_brows = slc.n_brows;
      sl.groups = d_sgrp; sl.g_mask = d_smask; sl.g_ep = d_sep; sl.wg_tab = d_stab;
      hipLaunchKernelGGL(map_slice_kernel, dim3((unsigned)((int64_t)P * slc.n_wg)), dim3(kBlock),
                         slice_lds(slc.n_brows), stream, sl);
      le = hipGetLastError();
      rec_at(4);
    } else if (le == hipSuccess && !L.bits) {
      rec_at(4);  // no tick kernel: an empty interval
      le = Lr->map_scan(ma, L.win, mgrid, dim3(L.block), stream);
    } else if (le == hipSuccess) {
      // each segment goes to the tick kernel or, by segment_uses_ticks, to the
      // list or the position kernel
      if (L.split != 2) le = Lr->map_ticks(ma, L.all_mach, mgrid, dim3(L.block), L.lds_ticks, stream);
      rec_at(4);
      if (le == hipSuccess && L.split != 1)
        le = L.list ? Lr->map_list(ma, L.win, L.all_mach, mgrid, dim3(L.block), stream)
                    : Lr->map_bits(ma, L.win, L.all_mach, mgrid, dim3(L.block), L.lds, stream);
    }
    if (le != hipSuccess) { status = EP_ERR_HIP; break; }
    rec_at(5);
    StreamArgs stra{};
    if (sh) {
      ClosureArgs& c = stra.c;
      c.times = times; c.types = types;
      c.ep_types = d_types; c.ep_lo = d_lo; c.ep_hi = d_hi; c.ep_span = d_span;
      c.tau = d_tau; c.seg_beg = d_beg; c.seg_end = d_end;
      c.ts = ts; c.flags = d_flags; c.repairs = d_cnt;
      c.S = S; c.P = P;
      c.queue = nullptr; c.queue_cap = 0; c.queue_n = c.queue_head = nullptr; c.repair_blocks = 0;
      c.ring = ring;
      stra.entry = sh->entry; stra.total = sh->total; stra.reset_out = sh->reset_out;
      stra.n = n_events; stra.t_end = sh->t_end; stra.max_span = max_span;
      if (P > 1 && Lr->stream_entry(stra, L.win, dim3((unsigned)((S + 3) / 4)), stream) != hipSuccess) {
        status = EP_ERR_HIP;
        break;
      }
    }

    mark();  // map launches
    // up to kReduceMembers segments: closure, tree and result in one launch
    // (a full wave at least: repairs and recounts are wave-cooperative)
    int red_members = kWave;
    while (red_members < P) red_members <<= 1;
    const size_t red_lds = (size_t)red_members * (12 * L.slots + 8);
    // fused when the post-Map work is small enough for its launches to matter
    // (S x P <= 2^20 tuples); beyond, the closure kernel spreads each
    // episode's repairs over the whole grid and wins
    const bool fused = !sh && P <= kReduceMembers && red_lds <= 65536 && S * (int64_t)P <= (1 << 20) &&
                       !(plan & EP_PLAN_NO_REDUCE);
    if (fused) {
      const int members = red_members;
      const size_t lds = red_lds;
      ReduceArgs ra;
      ClosureArgs& c = ra.c;
      c.times = times; c.types = types;
      c.ep_types = d_types; c.ep_lo = d_lo; c.ep_hi = d_hi; c.ep_span = d_span;
      c.tau = d_tau; c.seg_beg = d_beg; c.seg_end = d_end;
      c.ts = ts; c.flags = d_flags; c.repairs = d_cnt;
      c.S = S; c.P = P;
      c.queue = nullptr; c.queue_cap = 0; c.queue_n = c.queue_head = nullptr; c.repair_blocks = 0;
      c.ring = ring;
      ra.fallbacks = d_cnt + 1; ra.out = out_counts; ra.n = n_events;
      ra.out_map = out_map ? d_omap : nullptr;
      if (Lr->reduce(ra, L.win, dim3((unsigned)S), dim3((unsigned)members), lds, stream) !=
          hipSuccess) {
        status = EP_ERR_HIP;
        break;
      }
      rec_at(6);
    }
    if (P > 1 && !fused) {
      ClosureArgs ca;
      ca.times = times; ca.types = types;
      ca.ep_types = d_types; ca.ep_lo = d_lo; ca.ep_hi = d_hi; ca.ep_span = d_span;
      ca.tau = d_tau; ca.seg_beg = d_beg; ca.seg_end = d_end;
      ca.ts = ts; ca.flags = d_flags; ca.repairs = d_cnt;
      ca.S = S; ca.P = P;
      ca.queue = d_queue;
      ca.queue_cap = (plan & EP_PLAN_NO_REPAIR_QUEUE) ? 0 : ((plan & EP_PLAN_TINY_REPAIR_QUEUE) ? 1 : queue_cap);
      ca.queue_n = d_cnt + 2; ca.queue_head = d_cnt + 3;
      ca.repair_blocks = info->cu_count * 2;
      ca.ring = ring;
      if (Lr->closure(ca, L.win, dim3(grid_for((int64_t)(P - 1) * S)), stream) != hipSuccess) {
        status = EP_ERR_HIP;
        break;
      }
      rec_at(6);
      // Concatenate tree: each launch joins groups of `members` blocks, a
      // workgroup per group, each thread `per` consecutive members in order
      // first, then the threads' lists in LDS
      // a stream's batch joins all but the last segment (the tail runs that one)
      const int32_t Pt = sh ? P - 1 : P;
      // members per workgroup: the fewest powers of two covering Pt, within
      // 64 KiB of LDS at one member per thread
      int members = kConcatMembers;
      while (members > 1 && (size_t)members * (12 * L.slots + 4) > 65536) members >>= 1;
      while (members > 1 && members / 2 >= Pt) members >>= 1;
      for (int64_t stride = 1; stride < Pt; stride *= members) {
        const int64_t groups = (Pt + stride * members - 1) / (stride * members);
        // members each thread joins in order: as many as keep the launch at
        // kConcatMinThreads threads or more
        int per = 1;
        while (per < kConcatPer && per * 2 <= members &&
               (int64_t)members * groups * S / (per * 2) >= kConcatMinThreads)
          per *= 2;
        const int threads = members / per;
        const size_t lds = (size_t)threads * (12 * L.slots + 4);
        hipLaunchKernelGGL(concat_tree_kernel, dim3((unsigned)(groups * S)), dim3(threads), lds,
                           stream, ts, d_flags, S, Pt, stride, members, groups, per);
        if (hipGetLastError() != hipSuccess) { status = EP_ERR_HIP; break; }
      }
      if (status != EP_OK) break;
    }
    if (P <= 1 && !fused) rec_at(6);
    rec_at(7);
    mark();  // closure + tree launches
    if (sh) {
      if (Lr->stream_tail(stra, L.win, dim3((unsigned)((S + 3) / 4)), stream) != hipSuccess) {
        status = EP_ERR_HIP;
        break;
      }
    } else if (!fused) {
      FallbackArgs fa;
      fa.times = times; fa.types = types;
      fa.ep_types = d_types; fa.ep_lo = d_lo; fa.ep_hi = d_hi; fa.ep_span = d_span;
      fa.flags = d_flags; fa.T0 = d_t0; fa.P = P;
      fa.fallbacks = d_cnt + 1; fa.out = out_counts;
      fa.out_map = out_map ? d_omap : nullptr;
      fa.n = n_events; fa.S = S; fa.ring = ring;
      if (Lr->finish(fa, L.win, dim3((unsigned)((S + 3) / 4)), stream) != hipSuccess) {
        status = EP_ERR_HIP;
        break;
      }
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
      opt->stats->max_runs = L.win == kBits32 ? 32 : L.win == kBits64 ? 64 : L.win == kRing ? (int32_t)ring_cap : K;
      opt->stats->kernels = (L.bits ? 1 : 0) | (L.all_mach ? 2 : 0) | (L.list ? 4 : 0) | (L.prune ? 8 : 0) |
                            (L.win == kRing ? 16 : 0) | (L.slice ? 32 : 0);
      opt->stats->repairs = (int64_t)cnt[0];
      opt->stats->fallbacks = (int64_t)cnt[1];
      opt->stats->groups = 1;
    }
  } while (0);

  mark();  // finish launch
  if (block && scratch_release(dev, block, stream) != EP_OK && status == EP_OK) status = EP_ERR_HIP;
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
  if (which < EP_PROFILE_FILTER || which > EP_PROFILE_PRUNE || every < 1) return EP_ERR_ARG;
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
      const int f = prof_first(r.which);
      if (hipEventSynchronize(r.ev[f + 1]) != hipSuccess ||
          hipEventElapsedTime(&k_ms, r.ev[f], r.ev[f + 1]) != hipSuccess)
        status = EP_ERR_HIP;
      double* field = r.which == EP_PROFILE_FILTER  ? &acc.map_filter_ms
                      : r.which == EP_PROFILE_PRUNE ? &acc.map_prune_ms
                      : r.which == EP_PROFILE_TICKS ? &acc.map_ticks_ms
                                                    : &acc.map_positions_ms;
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
    acc.other_ms += ms[0] + ms[7];
    acc.map_filter_ms += ms[1];
    acc.map_prune_ms += ms[2];
    acc.map_ticks_ms += ms[3];
    acc.map_positions_ms += ms[4];
    acc.map_ms += ms[1] + ms[2] + ms[3] + ms[4];
    acc.closure_ms += ms[5];
    acc.concat_ms += ms[6];
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

extern "C" int ep_count_episodes_noalloc(const int32_t* times, const uint16_t* types, int64_t n_events,
                                         ep_episodes episodes, int64_t n_episodes, int64_t* out_counts,
                                         hipStream_t stream, const ep_options* opt) {
  return count_episodes_impl(times, types, n_events, episodes, n_episodes, out_counts, stream, opt, nullptr,
                             nullptr, true);
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

// ------------------------------------------------------------- streaming

struct ep_stream {
  int dev = 0;
  int32_t N = 0;
  int64_t S = 0;
  std::vector<uint16_t> types;      // the episode table (host copy)
  std::vector<int32_t> lo, hi;
  ep_options opt{};
  int64_t max_span = 0;
  int64_t t_last = INT64_MIN;       // last event time pushed so far
  int64_t events = 0;               // events pushed so far
  int64_t* total = nullptr;         // device [S] running counts
  int64_t* reset[2] = {nullptr, nullptr};  // device [S] carried reset times (ping-pong)
  int cur = 0;                      // reset[cur] holds the times to carry into the next push
  int64_t* scalar = nullptr;        // device [2]: the pending halo's first index in the last
                                    // combined buffer and its size
  int64_t* info = nullptr;          // host-mapped [4]: what stream_info_kernel reports
  int64_t* info_dev = nullptr;      // its device address
  int32_t* comb_t[2] = {nullptr, nullptr};  // device: halo followed by the batch (ping-pong)
  uint16_t* comb_y[2] = {nullptr, nullptr};
  int64_t comb_cap[2] = {0, 0};
  int cb = 0;                       // comb[cb] holds the pending halo at its head
};

namespace {

// Room for `need` events in a combined buffer; its first `keep` events are
// kept (copied on the stream before the old buffer is freed).
int grow(int32_t** t, uint16_t** y, int64_t* cap, int64_t need, int64_t keep, hipStream_t stream) {
  if (need <= *cap) return EP_OK;
  const int64_t c = std::max<int64_t>(need + need / 4, 1 << 16);
  int32_t* nt = nullptr;
  uint16_t* ny = nullptr;
  if (hipMalloc((void**)&nt, (size_t)c * sizeof(int32_t)) != hipSuccess) return EP_ERR_WORKSPACE;
  if (hipMalloc((void**)&ny, (size_t)c * sizeof(uint16_t)) != hipSuccess) {
    (void)hipFree(nt);
    return EP_ERR_WORKSPACE;
  }
  if (keep > 0 &&
      (hipMemcpyAsync(nt, *t, (size_t)keep * sizeof(int32_t), hipMemcpyDeviceToDevice, stream) != hipSuccess ||
       hipMemcpyAsync(ny, *y, (size_t)keep * sizeof(uint16_t), hipMemcpyDeviceToDevice, stream) != hipSuccess)) {
    (void)hipFree(nt);
    (void)hipFree(ny);
    return EP_ERR_HIP;
  }
  // the old buffers may still be read by queued work: wait for the device first
  if (*t && (hipDeviceSynchronize() != hipSuccess || hipFree(*t) != hipSuccess || hipFree(*y) != hipSuccess)) {
    (void)hipFree(nt);
    (void)hipFree(ny);
    return EP_ERR_HIP;
  }
  *t = nt;
  *y = ny;
  *cap = c;
  return EP_OK;
}

}  // namespace

extern "C" int ep_stream_create(ep_episodes episodes, int64_t n_episodes, const ep_options* opt,
                                hipStream_t stream, ep_stream** out) {
  using namespace epk;
  if (!out) return EP_ERR_ARG;
  *out = nullptr;
  const int32_t N = episodes.n_nodes;
  const int64_t S = n_episodes;
  if (S < 0) return EP_ERR_ARG;
  if (N < 1 || N > EP_MAX_NODES) return EP_ERR_NODES;
  const bool upper_only = opt && opt->upper_only;
  if (S > 0 && (!episodes.types || (N > 1 && (!episodes.t_high || (!upper_only && !episodes.t_low)))))
    return EP_ERR_ARG;
  if (opt && (opt->mode < EP_MODE_AUTO || opt->mode > EP_MODE_MAPCONCAT || opt->n_segments < 0))
    return EP_ERR_ARG;
  ep_stream* st = new ep_stream();
  st->N = N;
  st->S = S;
  st->types.assign(episodes.types, episodes.types + S * N);
  if (N > 1) {
    st->hi.assign(episodes.t_high, episodes.t_high + S * (N - 1));
    if (upper_only)
      st->lo.assign((size_t)(S * (N - 1)), 0);
    else
      st->lo.assign(episodes.t_low, episodes.t_low + S * (N - 1));
  }
  for (int64_t e = 0; e < S; ++e) {
    int64_t span = 0;
    for (int j = 0; j < N - 1; ++j) {
      const int64_t l = st->lo[(size_t)(e * (N - 1) + j)], h = st->hi[(size_t)(e * (N - 1) + j)];
      if (l < 0 || l >= h) {
        delete st;
        return EP_ERR_INTERVAL;
      }
      span += h;
    }
    if (span > INT32_MAX) {
      delete st;
      return EP_ERR_INTERVAL;
    }
    st->max_span = std::max(st->max_span, span);
  }
  if (opt) st->opt = *opt;
  st->opt.upper_only = 0;  // the table copy already holds the relaxed bounds
  st->opt.stats = nullptr;
  int status = EP_OK;
  do {
    if (hipGetDevice(&st->dev) != hipSuccess) { status = EP_ERR_HIP; break; }
    const size_t b = (size_t)std::max<int64_t>(S, 1) * sizeof(int64_t);
    if (hipMalloc((void**)&st->total, b) != hipSuccess || hipMalloc((void**)&st->reset[0], b) != hipSuccess ||
        hipMalloc((void**)&st->reset[1], b) != hipSuccess ||
        hipMalloc((void**)&st->scalar, 2 * sizeof(int64_t)) != hipSuccess ||
        hipHostMalloc((void**)&st->info, 4 * sizeof(int64_t), hipHostMallocMapped | hipHostMallocCoherent) !=
            hipSuccess) {
      status = EP_ERR_WORKSPACE;
      break;
    }
    if (hipHostGetDevicePointer((void**)&st->info_dev, st->info, 0) != hipSuccess) { status = EP_ERR_HIP; break; }
    hipLaunchKernelGGL(fill_i64_kernel, dim3(1), dim3(kBlock), 0, stream, st->scalar, (int64_t)2, (int64_t)0);
    if (S > 0) {
      hipLaunchKernelGGL(fill_i64_kernel, dim3(grid_for(S)), dim3(kBlock), 0, stream, st->total, S, (int64_t)0);
      hipLaunchKernelGGL(fill_i64_kernel, dim3(grid_for(S)), dim3(kBlock), 0, stream, st->reset[0], S, kNoReset);
      if (hipGetLastError() != hipSuccess) { status = EP_ERR_HIP; break; }
    }
  } while (0);
  if (status != EP_OK) {
    ep_stream_destroy(st);
    return status;
  }
  *out = st;
  return EP_OK;
}

extern "C" int ep_stream_push(ep_stream* st, const int32_t* times, const uint16_t* types, int64_t n_events,
                              hipStream_t stream) {
  using namespace epk;
  if (!st || n_events < 0 || n_events > INT32_MAX) return EP_ERR_ARG;
  if (n_events == 0 || st->S == 0) {
    if (n_events > 0) st->events += n_events;
    return EP_OK;
  }
  if (!times || !types) return EP_ERR_ARG;
  int dev = 0;
  EP_HIP(hipGetDevice(&dev));
  if (dev != st->dev) return EP_ERR_ARG;
  // the batch's first and last times and the pending halo (one synchronisation)
  const int cb = st->cb;
  hipLaunchKernelGGL(stream_info_kernel, dim3(1), dim3(kWave), 0, stream, times, n_events, st->scalar + 1,
                     st->comb_t[cb], st->info_dev);
  EP_HIP(hipGetLastError());
  EP_HIP(hipStreamSynchronize(stream));
  const int64_t t_first = st->info[0], t_end = st->info[1], halo_n = st->info[2], halo_first = st->info[3];
  if (st->t_last != INT64_MIN && t_first < st->t_last) return EP_ERR_UNSORTED;
  const int64_t n = halo_n + n_events;
  if (n > INT32_MAX) return EP_ERR_ARG;
  if (int s = grow(&st->comb_t[cb], &st->comb_y[cb], &st->comb_cap[cb], n, halo_n, stream)) return s;
  EP_HIP(hipMemcpyAsync(st->comb_t[cb] + halo_n, times, (size_t)n_events * sizeof(int32_t),
                        hipMemcpyDeviceToDevice, stream));
  EP_HIP(hipMemcpyAsync(st->comb_y[cb] + halo_n, types, (size_t)n_events * sizeof(uint16_t),
                        hipMemcpyDeviceToDevice, stream));
  StreamHook hook;
  hook.entry = st->reset[st->cur];
  hook.total = st->total;
  hook.reset_out = st->reset[1 - st->cur];
  hook.t_first = halo_n > 0 ? halo_first : t_first;
  hook.t_end = t_end;
  ep_episodes eps{st->N, st->types.data(), st->N > 1 ? st->lo.data() : nullptr,
                  st->N > 1 ? st->hi.data() : nullptr};
  if (int s = count_episodes_impl(st->comb_t[cb], st->comb_y[cb], n, eps, st->S, st->total, stream, &st->opt,
                                  &hook))
    return s;
  st->cur = 1 - st->cur;
  // the next halo (events within maxSpan of the last one) to the head of the
  // other combined buffer; its size stays on the device until the next push
  const int nb = 1 - cb;
  if (int s = grow(&st->comb_t[nb], &st->comb_y[nb], &st->comb_cap[nb], n, 0, stream)) return s;
  hipLaunchKernelGGL(halo_find_kernel, dim3(1), dim3(kWave), 0, stream, st->comb_t[cb], n, t_end - st->max_span,
                     st->scalar, st->scalar + 1);
  hipLaunchKernelGGL(halo_move_kernel, dim3((unsigned)std::min<int64_t>(grid_for(n), 256)), dim3(kBlock), 0, stream,
                     st->comb_t[cb], st->comb_y[cb], st->scalar, st->scalar + 1, st->comb_t[nb], st->comb_y[nb]);
  EP_HIP(hipGetLastError());
  st->cb = nb;
  st->t_last = t_end;
  st->events += n_events;
  return EP_OK;
}

extern "C" int ep_stream_counts(const ep_stream* st, int64_t* out_counts, hipStream_t stream) {
  if (!st || (st->S > 0 && !out_counts)) return EP_ERR_ARG;
  if (st->S == 0) return EP_OK;
  EP_HIP(hipMemcpyAsync(out_counts, st->total, (size_t)st->S * sizeof(int64_t), hipMemcpyDeviceToDevice, stream));
  return EP_OK;
}

extern "C" int64_t ep_stream_events(const ep_stream* st) { return st ? st->events : 0; }

extern "C" void ep_stream_destroy(ep_stream* st) {
  if (!st) return;
  if (st->total || st->comb_t[0] || st->comb_t[1]) (void)hipDeviceSynchronize();
  for (void* p : {(void*)st->total, (void*)st->reset[0], (void*)st->reset[1], (void*)st->scalar,
                  (void*)st->comb_t[0], (void*)st->comb_y[0], (void*)st->comb_t[1], (void*)st->comb_y[1]})
    if (p) (void)hipFree(p);
  if (st->info) (void)hipHostFree(st->info);
  delete st;
}

extern "C" int ep_count_episodes(const int32_t* times, const uint16_t* types, int64_t n_events,
                                 ep_episodes episodes, int64_t n_episodes, int64_t* out_counts,
                                 hipStream_t stream) {
  return ep_count_episodes_ex(times, types, n_events, episodes, n_episodes, out_counts, stream,
                              nullptr);
}
