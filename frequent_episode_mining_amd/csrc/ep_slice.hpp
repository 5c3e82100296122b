// Type-sliced Map kernel for two-node episodes (gfx950 / CDNA4).
//
// Source page: "Towards Chip-on-Chip Neuroscience: Fast Mining of Frequent
// Episodes Using Graphics Processors".  The Map step of MapConcatenate
// ("Design of MapConcatenate", Map rules 1-4, Fig. 4): every (segment p,
// episode, machine k) yields the tuple (a, count, b) of one counting machine
// reset at tau_p - k * t_high, as the other Map kernels compute it.
//
// For a two-node episode A -(lo, hi]-> B a machine last reset at r completes
// at a B event at tick t iff some A event lies in [max(r + 1, t - hi),
// t - lo - 1].  That holds iff A has an event in [t - hi, t - lo - 1] and an
// event in (r, t - lo - 1]: the later of the two events lies in both ranges.
// Episodes that share (B, lo, hi) therefore step together, one bit of a
// 64-bit word per node-0 type ("slice"): at each B tick
//
//   hit = W(t) & ~blocked,   W(t) = OR of the node-0 type masks over ticks
//                                   [t - hi, t - lo - 1],
//
// blocked holding the types whose last reset has no A event after it yet.
// One lane steps the 64 machines of a (segment, group, machine) with a few
// 64-bit operations per B tick, instead of one lane per episode.
//
// Blocked types come in two kinds.  A reset at a tick after x = t - lo - 1 is
// *pending*: no A event can lie after it within reach yet.  Each pending type
// keeps its reset tick mod 64 in six bit planes (a pending reset is at most
// lo + 1 <= 63 ticks after x, so the residue names it), and a 64-bit mask
// holds the pending ticks mod 64; a pending reset *settles* once x reaches its
// tick, the lane taking the mask's ticks in (x_prev, min(x, last B tick)] in
// order.  Settled resets form one
// entry (tick tS, mask DS), pruned at every B tick by the A events in
// (tS, x]: an older entry pruned up to x has no A event in (tS, x], so its
// types behave like a reset at any later settled tick, and entries merge
// exactly.  An entry older than t - hi blocks nothing that W lets through and
// is dropped.
//
// The per-tick node-0 type masks of a chunk of the segment sit in LDS as a
// sparse table (ORs over 1, 2, 4, ..., 32 ticks), so an OR over any range of
// up to 64 ticks is two LDS reads.  A chunk holds kSliceWin ticks: a 64-tick
// halo and kSliceChunk new ticks; every range a lane queries lies within 64
// ticks before the B tick it steps, hence inside the window.  After 128 or
// more ticks without events the next chunk starts at the next event and the
// lanes drop their reset state (every reset is then older than t - hi).
//
// The two machines of a segment (resets at tau_p and tau_p - hi) reach the
// same state for a node-0 type once no event of that type lies between their
// resets; from then on they complete together.  Machine-1 lanes fill whole
// waves of their own; at each chunk end (while some are left) a machine-1
// lane compares its state with its machine-0 twin's through LDS, and once
// every type agrees it stops: its tuple becomes its own a, its count up to
// that tick minus the twin's (the twin adds its own final count to it) and
// the twin's b.  The merge tick lies after tau_p + t_high (a is final) and
// before tau_{p+1} (b and the rest of the count are the twin's).
//
// Completions are recorded bit-parallel too: the count in (tau_p, tau_{p+1}]
// in a bit-sliced counter of kSlicePlanes planes, flushed into the tuple
// store every 255 counted B ticks; a (offset <= t_high after tau_p) and b
// (offset <= t_high after tau_{p+1}) in six planes each.  The tuples are
// written at the end of the segment.
#pragma once

#include "ep_device.hpp"

namespace epk {

constexpr int kSliceWin = 512;                   // ticks of a chunk window (64 of halo)
constexpr int kSliceChunk = kSliceWin - 64;      // ticks a chunk moves on (a multiple of 64)
constexpr int kSliceWords = kSliceWin / 64;      // 64-tick words of a node-1 bitmap row
constexpr int kSliceLevels = 6;                  // sparse table: ORs over 1, 2, ..., 32 ticks
constexpr int kSliceTypes = 2048;                // node types below this (LDS type table)
constexpr int kSlicePlanes = 8;                  // counter planes (counts up to 255)
constexpr int kSliceFlush = (1 << kSlicePlanes) - 1;

// One group: the episodes A -(lo, hi]-> B of one node-1 type B and interval,
// their node-0 types being bits of one 64-bit word.
struct SliceGroup {
  int32_t lo, hi;
  int32_t brow;  // row of B's tick bitmap in its workgroup's LDS
  int32_t pad;
};

struct SliceArgs {
  const int32_t* times;
  const uint16_t* types;
  const int64_t* tau;        // [P+1] cuts
  const int32_t* seg_beg;    // [P] first event with time > tau_p - max_span
  const int32_t* seg_end;    // [P] first event with time > tau_{p+1} + max_span
  TupleStore ts;
  int32_t P;
  int32_t n_machines;        // 2 (MapConcatenate) or 1 (PTPE)
  int32_t max_span;          // largest t_high of the call
  int32_t n_groups;          // groups, padded so that no workgroup mixes node-0 type sets
  int32_t wg_groups;         // groups per workgroup (its threads / n_machines)
  int32_t n_wg;              // workgroups per segment
  int32_t n_brows;           // node-1 bitmap rows per workgroup
  const SliceGroup* groups;  // [n_groups]
  const uint64_t* g_mask;    // [n_groups] bits that hold an episode (0: padding)
  const int32_t* g_ep;       // [n_groups * 64] episode of each bit
  const uint16_t* wg_tab;    // [n_wg * kSliceTypes] type -> (node-0 bit + 1) | (row + 1) << 7
};

// OR of the node-0 type masks over window ticks [l, r]: 0 <= l, r <
// kSliceWin and r - l < 64, or l > r (empty).  Two reads of the sparse table
// (level k covers 2^k ticks from its index; two level-k blocks cover any
// range of 2^k .. 2^(k+1) ticks, and two level-5 blocks any up to 64).
__device__ inline uint64_t slice_or(const uint64_t* st, int32_t l, int32_t r) {
  const bool ok = l <= r;
  const int32_t ll = ok ? l : 0, rr = ok ? r : 0;
  const uint32_t len = (uint32_t)(rr - ll + 1);
  int k = 31 - __clz(len);
  k = k > kSliceLevels - 1 ? kSliceLevels - 1 : k;
  const uint64_t v = st[k * kSliceWin + ll] | st[k * kSliceWin + rr - (1 << k) + 1];
  return ok ? v : 0ull;
}

// bit i of v as 0 or all ones
__device__ inline uint32_t slice_sbit(int32_t v, int i) {
  return (uint32_t)(-((v >> i) & 1));
}

// the bits of `m` set to s (0 or all ones), the rest from d: one bitfield
// insert per 32-bit half
__device__ inline uint64_t slice_set(uint64_t m, uint32_t s, uint64_t d) {
  const uint32_t ml = (uint32_t)m, mh = (uint32_t)(m >> 32);
  const uint32_t lo = (ml & s) | (~ml & (uint32_t)d);
  const uint32_t hi = (mh & s) | (~mh & (uint32_t)(d >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// the bits of `m` whose six planes spell v (mod 64)
__device__ inline uint64_t slice_match(uint64_t m, const uint64_t (&pl)[6], int32_t v) {
  uint32_t ml = (uint32_t)m, mh = (uint32_t)(m >> 32);
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const uint32_t s = slice_sbit(v, i);
    ml &= ~((uint32_t)pl[i] ^ s);
    mh &= ~((uint32_t)(pl[i] >> 32) ^ s);
  }
  return ((uint64_t)mh << 32) | ml;
}

// value of bit j over `n` planes
template <int NP>
__device__ inline int32_t slice_get(const uint64_t (&pl)[NP], int j) {
  int32_t v = 0;
#pragma unroll
  for (int i = 0; i < NP; ++i) v |= (int32_t)((pl[i] >> j) & 1ull) << i;
  return v;
}

// Workgroup: (segment p, group range w); thread = (machine, group), machine
// slowest.  Launch: grid P * n_wg, kBlock threads, LDS slice_lds(n_brows).
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4)))
void map_slice_kernel(SliceArgs A) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* s_st = (uint64_t*)smem;                                // [kSliceLevels][kSliceWin]
  uint64_t* s_bw = s_st + kSliceLevels * kSliceWin;                // [n_brows][kSliceWords]
  uint16_t* s_tab = (uint16_t*)(s_bw + (size_t)A.n_brows * kSliceWords);  // [kSliceTypes]
  __shared__ int32_t s_next, s_halo, s_unmerged;
  __shared__ int32_t s_merged[kBlock / 2];  // machine-1 lane of group gi stopped (twin has its count)
  __shared__ int32_t s_xflag[kBlock / 2];   // machine-0 lane of group gi: counter flushed

  constexpr int32_t kFar = 1 << 30;  // offsets are clamped to +-kFar
  constexpr int kPer = 4;            // events per thread per fill batch
  const int tid = threadIdx.x;
  // XCD-aware order: workgroups go to the eight XCDs round-robin by blockIdx,
  // so XCD c takes a contiguous range of logical blocks (segment-major): the
  // tuples of consecutive segments share cache lines of the episode-major
  // tuple store, and written from one XCD they are merged in its L2 instead
  // of reaching memory as partial lines from several
  int64_t lb = blockIdx.x;
  {
    const int64_t nb = gridDim.x, q = nb / 8, r = nb % 8;
    const int64_t c = lb % 8, slot = lb / 8;
    lb = c * q + (c < r ? c : r) + slot;
  }
  const int64_t p = lb / A.n_wg;
  const int w = (int)(lb - p * A.n_wg);
  const int k = tid / A.wg_groups;
  const int gi = tid - k * A.wg_groups;
  const int64_t g = (int64_t)w * A.wg_groups + gi;
  const bool in_range = k < A.n_machines && g < A.n_groups;
  const uint64_t gmask = in_range ? A.g_mask[g] : 0ull;
  const bool active = gmask != 0ull;

  for (int i = tid; i < kSliceTypes; i += kBlock) s_tab[i] = A.wg_tab[(int64_t)w * kSliceTypes + i];
  if (tid < kBlock / 2) s_merged[tid] = 0;
  if (tid == 0) s_unmerged = 0;
  __syncthreads();
  if (active && k == 1) atomicAdd(&s_unmerged, 1);

  const int64_t tau_lo = A.tau[p], tau_hi = A.tau[p + 1];
  const int32_t end = A.seg_end[p];
  int32_t ev_lo = A.seg_beg[p];
  SliceGroup gr{0, 1, 0, 0};
  if (active) gr = A.groups[g];
  const int32_t lo = gr.lo, hi = gr.hi;
  const uint64_t* brow = s_bw + (size_t)gr.brow * kSliceWords;

  // chunk schedule (the same in every thread): the first chunk starts at the
  // first tick a machine of the segment can use, or at the first event after
  // an event-free stretch of 128 ticks or more
  int64_t c0 = tau_lo - A.max_span + 1;
  bool reset = false;
  if (ev_lo < end && (int64_t)A.times[ev_lo] >= c0 + 128) {
    c0 = A.times[ev_lo];
    reset = true;
  }
  int64_t base = c0 - 64;  // tick of window index 0
  auto rel = [&](int64_t v) -> int32_t {
    const int64_t d = v - base;
    return (int32_t)(d < -kFar ? -kFar : (d > kFar ? kFar : d));
  };

  // ---- lane state; ticks are window offsets (clamped to +-kFar)
  int32_t tS = rel(tau_lo - (k == 1 ? (int64_t)hi : 0));  // the machine's reset
  uint64_t DS = reset ? 0ull : ~0ull;   // settled: no A event after tS yet
  uint64_t PA = 0ull;                   // pending resets
  uint64_t pp[6];                       // their ticks mod 64
  uint64_t PT = 0ull;                   // the pending ticks, bit t mod 64
  uint64_t cp[kSlicePlanes];            // counter planes
  uint64_t ap[6], bp[6];                // a and b offsets
  uint64_t fa = 0ull, fb = 0ull;        // a / b recorded
#pragma unroll
  for (int i = 0; i < 6; ++i) pp[i] = ap[i] = bp[i] = 0ull;
#pragma unroll
  for (int i = 0; i < kSlicePlanes; ++i) cp[i] = 0ull;
  int32_t xprev = -kFar, lastb = -kFar;
  uint64_t q0 = 0ull, q1 = 0ull;        // small counter: completions since the last merge (<= 3)
  int32_t n_in = 0;                     // counted B ticks since the last flush
  bool flushed = false;
  // the cuts and the stop tick: from their 64-bit values at every new base
  // (a clamped offset must not be moved again)
  const int64_t stop64 = tau_hi + hi;
  int32_t tlo = rel(tau_lo), thi = rel(tau_hi), stop = rel(stop64);
  bool done = !active;

  // the counter's planes added into the tuple store
  auto flush = [&]() {
    uint64_t m = gmask;
    while (m) {
      const int j = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      const int32_t e = A.g_ep[g * 64 + j];
      Tuple* tu = A.ts.at(e, p, k);
      const int32_t c = slice_get<kSlicePlanes>(cp, j);
      tu->c = flushed ? tu->c + c : c;
    }
#pragma unroll
    for (int i = 0; i < kSlicePlanes; ++i) cp[i] = 0ull;
    n_in = 0;
    flushed = true;
  };

  // settle the pending resets at ticks in [l, r] (r - l < 63): as of x, with
  // resets before exp_t expired (pending ticks are unique mod 64)
  auto settle_range = [&](int32_t l, int32_t r, int32_t x, int32_t exp_t) {
    const uint32_t sh = (uint32_t)l & 63u;
    uint64_t m = __builtin_rotateright64(PT, sh) & ((~0ull) >> (63 - (r - l)));
    while (m) {
      const int32_t tp = l + __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      PT &= ~(1ull << (tp & 63));
      const uint64_t Dp = slice_match(PA, pp, tp);
      PA &= ~Dp;
      if (tp >= exp_t) {
        DS |= Dp & ~slice_or(s_st, tp + 1, x);
        tS = tp;
      }
    }
  };

  // the small counter added into the planes (every third step of a wave and
  // before the planes are read); a lane near 255 counted steps flushes
  auto merge_small = [&]() {
    // plane 0 + q0; plane 1 + q1 + carry; the carry rippled up
    uint64_t c = cp[0] & q0;
    cp[0] ^= q0;
    const uint64_t x1 = cp[1] ^ q1;
    const uint64_t c2 = (cp[1] & q1) | (c & x1);
    cp[1] = x1 ^ c;
    c = c2;
#pragma unroll
    for (int i = 2; i < kSlicePlanes; ++i) {
      const uint64_t carry = cp[i] & c;
      cp[i] ^= c;
      c = carry;
    }
    q0 = q1 = 0ull;
    // every lane of the wave flushes once one needs to (one pass of the
    // flush loop per wave, not one per lane)
    if (__ballot(n_in >= kSliceFlush - 3)) flush();
  };

  // bring the reset state to x (t: the B tick about to be stepped, or the
  // first tick of the next chunk)
  auto advance = [&](int32_t t, int32_t x) {
    const int32_t exp_t = t - hi;
    if (DS) {
      // an expired entry queries nothing (its range may lie outside the window)
      const bool expired = tS < exp_t;
      const uint64_t later = slice_or(s_st, expired ? x + 1 : tS + 1, x);
      DS = expired ? 0ull : (DS & ~later);
    }
    if (PA) {
      const int32_t top = x < lastb ? x : lastb;
      if (top > xprev) settle_range(xprev + 1, top, x, exp_t);
    }
    xprev = x;
  };

  // one B tick t.  The reads of the three ORs it needs (W, the settled
  // entry's pruning, the first pending reset that settles) are issued
  // together; a second settling reset at one step is rare and takes the
  // general loop
  auto step = [&](int32_t t) {
    const int32_t x = t - lo - 1;
    const int32_t e = t - hi;
    const int32_t top = x < lastb ? x : lastb;
    const int32_t len = top - xprev;  // < 64
    // pending ticks in (xprev, top], bit j for tick xprev + 1 + j (branch-free:
    // the common path of a step takes no branch but the rare ones)
    const uint64_t rot = __builtin_rotateright64(PT, (uint32_t)(xprev + 1) & 63u);
    const uint64_t sm = len > 0 ? rot & ((~0ull) >> (64 - (len > 63 ? 63 : (len < 1 ? 1 : len)))) : 0ull;
    const int32_t tp = xprev + __ffsll((unsigned long long)sm);
    const bool live = sm != 0ull && tp >= e;
    const bool expired = tS < e;
    const uint64_t w_or = slice_or(s_st, e, x);
    const uint64_t s_or = slice_or(s_st, expired ? x + 1 : tS + 1, x);
    const uint64_t p_or = slice_or(s_st, live ? tp + 1 : x + 1, x);
    DS = expired ? 0ull : (DS & ~s_or);
    // the first settling reset
    const uint64_t Dp = sm ? slice_match(PA, pp, tp) : 0ull;
    PA &= ~Dp;
    PT &= sm ? ~(1ull << (tp & 63)) : ~0ull;
    DS |= live ? (Dp & ~p_or) : 0ull;
    tS = live ? tp : tS;
    if (sm & (sm - 1)) settle_range(tp + 1, top, x, e);  // rare
    xprev = x;
    const uint64_t hit = w_or & gmask & ~(DS | PA);
    lastb = t;
    // (a zero hit leaves all of this unchanged)
    PA |= hit;
    PT |= hit ? (1ull << (t & 63)) : 0ull;
#pragma unroll
    for (int i = 0; i < 6; ++i) pp[i] = slice_set(hit, slice_sbit(t, i), pp[i]);
    const bool counted = t > tlo && t <= thi;
    const uint64_t hc = counted ? hit : 0ull;
    q1 ^= q0 & hc;
    q0 ^= hc;
    n_in += counted ? 1 : 0;
    if (hit && t > tlo) {
      if (t <= tlo + hi) {
        const uint64_t nw = hit & ~fa;
        fa |= hit;
        const int32_t av = t - tlo;
#pragma unroll
        for (int i = 0; i < 6; ++i) ap[i] = slice_set(nw, slice_sbit(av, i), ap[i]);
      }
      if (t > thi) {
        const uint64_t nw = hit & ~fb;
        fb |= hit;
        const int32_t bv = t - thi;
#pragma unroll
        for (int i = 0; i < 6; ++i) bp[i] = slice_set(nw, slice_sbit(bv, i), bp[i]);
      }
    }
  };

  for (;;) {
    __syncthreads();  // the previous chunk is consumed (and the type table written)
    for (int i = tid; i < kSliceWin; i += kBlock) s_st[i] = 0ull;
    for (int i = tid; i < A.n_brows * kSliceWords; i += kBlock) s_bw[i] = 0ull;
    if (tid == 0) {
      s_next = end;
      s_halo = end;
    }
    __syncthreads();
    // fill: the events of ticks [base, base + kSliceWin); the first event past
    // the window and the first one of the next window's halo come out of LDS
    // atomics
    const int64_t wend = base + kSliceWin;
    const int64_t hstart = wend - 64;
    for (int32_t i0 = ev_lo; i0 < end; i0 += kPer * kBlock) {
      int32_t tt[kPer];
      uint32_t ty[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int32_t i = i0 + j * kBlock + tid;
        tt[j] = i < end ? A.times[i] : 0;
        ty[j] = i < end ? A.types[i] : 0u;
      }
      const int32_t last_i = (int64_t)i0 + kPer * kBlock - 1 < end ? i0 + kPer * kBlock - 1 : end - 1;
      const int64_t last_t = A.times[last_i];
      int32_t my_next = INT32_MAX, my_halo = INT32_MAX;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int32_t i = i0 + j * kBlock + tid;
        if (i < end) {
          const int64_t t = tt[j];
          if (t >= wend) {
            my_next = i < my_next ? i : my_next;
          } else {
            const int32_t off = (int32_t)(t - base);  // >= 0
            const uint32_t code = ty[j] < (uint32_t)kSliceTypes ? s_tab[ty[j]] : 0u;
            const uint32_t ab = code & 127u, br = code >> 7;
            if (ab) atomicOr((unsigned long long*)&s_st[off], 1ull << (ab - 1));
            if (br)
              atomicOr((unsigned long long*)&s_bw[(br - 1) * kSliceWords + (off >> 6)], 1ull << (off & 63));
          }
          if (t >= hstart) my_halo = i < my_halo ? i : my_halo;
        }
      }
      if (my_next != INT32_MAX) atomicMin(&s_next, my_next);
      if (my_halo != INT32_MAX) atomicMin(&s_halo, my_halo);
      if (last_t >= wend) break;
    }
    __syncthreads();
    // sparse table: level lv ORs level lv-1 at i and i + 2^(lv-1)
    for (int lv = 1; lv < kSliceLevels; ++lv) {
      const int h = 1 << (lv - 1);
      for (int i = tid; i < kSliceWin; i += kBlock) {
        const uint64_t v = s_st[(lv - 1) * kSliceWin + i];
        const uint64_t u = i + h < kSliceWin ? s_st[(lv - 1) * kSliceWin + i + h] : 0ull;
        s_st[lv * kSliceWin + i] = v | u;
      }
      __syncthreads();
    }
    // the lane's B ticks of the chunk (one cursor across the chunk's words, so
    // that a wave steps as often as its busiest lane, not the sum over words
    // of each word's busiest), then its state as of the next chunk
    if (!done) {
      // the chunk's non-empty words of the lane's node-1 row
      uint32_t occ = 0;
#pragma unroll
      for (int i = 1; i < kSliceWords; ++i) occ |= (brow[i] != 0ull ? 1u : 0u) << i;
      int wi = 0;
      uint64_t bits = 0ull;
      int it = 0;  // steps of this loop: the same in every lane still in it
      for (;;) {
        if (!bits) {
          if (!occ) break;
          wi = __ffs(occ) - 1;
          occ &= occ - 1;
          bits = brow[wi];
        }
        const int32_t t = wi * 64 + __ffsll((unsigned long long)bits) - 1;
        bits &= bits - 1;
        if (t > stop) {
          done = true;
          break;
        }
        step(t);
        // (the same count in every lane still in the loop: a scalar branch)
        if (__builtin_amdgcn_readfirstlane(++it) == 3) {
          it = 0;
          merge_small();
        }
      }
      merge_small();
      if (!done) advance(kSliceWin, kSliceWin - lo - 1);
    }
    // machine-1 lanes that match their twin's state stop (the chunk ends past
    // tau_p + max_span and before tau_{p+1}; the LDS of the sparse table is
    // free until the next fill)
    const int64_t cend = c0 + kSliceChunk;
    if (A.n_machines == 2 && s_unmerged > 0 && cend > tau_lo + A.max_span && cend < tau_hi) {
      uint64_t* xs = s_st;  // [wg_groups][16]: DS, PA, pp[6], cp[8] of machine 0
      __syncthreads();
      if (active && k == 0) {
        uint64_t* o = xs + (size_t)gi * 16;
        o[0] = DS;
        o[1] = PA;
#pragma unroll
        for (int i = 0; i < 6; ++i) o[2 + i] = pp[i];
#pragma unroll
        for (int i = 0; i < kSlicePlanes; ++i) o[8 + i] = cp[i];
        s_xflag[gi] = flushed ? 1 : 0;
      }
      __syncthreads();
      if (active && k == 1 && !done) {
        const uint64_t* o = xs + (size_t)gi * 16;
        const uint64_t DS0 = o[0], PA0 = o[1];
        uint64_t ppd = 0ull;
#pragma unroll
        for (int i = 0; i < 6; ++i) ppd |= o[2 + i] ^ pp[i];
        // per node-0 type: both blocked, both free, or both pending at one tick
        const uint64_t diff = (DS0 ^ DS) | (PA0 ^ PA) | (PA & ppd);
        if ((diff & gmask) == 0ull) {
          uint64_t cp0[kSlicePlanes];
#pragma unroll
          for (int i = 0; i < kSlicePlanes; ++i) cp0[i] = o[8 + i];
          const bool flushed0 = s_xflag[gi] != 0;
          uint64_t m = gmask;
          while (m) {
            const int j = __ffsll((unsigned long long)m) - 1;
            m &= m - 1;
            const int32_t e = A.g_ep[g * 64 + j];
            Tuple* t1 = A.ts.at(e, p, 1);
            const int32_t c1 = slice_get<kSlicePlanes>(cp, j) + (flushed ? t1->c : 0);
            const int32_t c0 = slice_get<kSlicePlanes>(cp0, j) + (flushed0 ? A.ts.at(e, p, 0)->c : 0);
            t1->a = slice_get<6>(ap, j);
            t1->c = c1 - c0;
          }
          s_merged[gi] = 1;
          atomicSub(&s_unmerged, 1);
          done = true;
        }
      }
    }
    const int32_t nx = s_next, hl = s_halo;  // read before the next chunk's first barrier
    if (nx >= end) break;
    const int64_t tn = A.times[nx];
    const int64_t cnext = c0 + kSliceChunk;
    int64_t d;
    if (tn >= cnext + 128) {
      // an event-free stretch: every reset is older than t_high at the next
      // B tick; the window restarts at the next event
      d = (tn - 64) - base;
      c0 = tn;
      ev_lo = nx;
      DS = 0ull;
      PA = 0ull;
      PT = 0ull;
      xprev = lastb = -kFar;
    } else {
      d = kSliceChunk;
      c0 = cnext;
      ev_lo = hl;
    }
    base += d;
    auto sub = [&](int32_t v) -> int32_t {
      const int64_t u = (int64_t)v - d;
      return (int32_t)(u < -kFar ? -kFar : (u > kFar ? kFar : u));
    };
    // (these lie in the past: clamping them at -kFar keeps their meaning)
    tS = sub(tS);
    xprev = sub(xprev);
    lastb = sub(lastb);
    tlo = rel(tau_lo);
    thi = rel(tau_hi);
    stop = rel(stop64);
  }

  __syncthreads();  // a machine-1 lane's merge writes are seen by its twin
  const bool stopped = A.n_machines == 2 && gi < kBlock / 2 && s_merged[gi] != 0;
  if (active && !(k == 1 && stopped)) {
    // eight node-0 bits at a time: their episodes (two 16-byte loads of the
    // group's row) and the stored values the tuples add to (the flushed
    // count, the stopped twin's tuple) are all loaded before any store, so a
    // lane waits for memory twice per eight episodes instead of per episode
    const int4* row = (const int4*)(A.g_ep + g * 64);
#pragma unroll 1
    for (int c8 = 0; c8 < 8; ++c8) {
      const uint32_t mc = (uint32_t)(gmask >> (8 * c8)) & 0xffu;
      if (mc == 0u) continue;
      const int4 q0 = row[2 * c8], q1 = row[2 * c8 + 1];
      const int32_t ev[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      int32_t prev[8];
      int4 twin[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        prev[jj] = 0;
        twin[jj] = make_int4(0, 0, 0, 0);
        if ((mc >> jj) & 1u) {
          if (flushed) prev[jj] = A.ts.at(ev[jj], p, k)->c;
          if (k == 0 && stopped) twin[jj] = *(const int4*)A.ts.at(ev[jj], p, 1);
        }
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (!((mc >> jj) & 1u)) continue;
        const int j = 8 * c8 + jj;
        const int32_t e = ev[jj];
        Tuple tu;
        tu.a = slice_get<6>(ap, j);
        tu.c = slice_get<kSlicePlanes>(cp, j) + prev[jj];
        tu.b = slice_get<6>(bp, j);
        tu.pad = 0;
        *A.ts.at(e, p, k) = tu;
        if (k == 0) {
          const int64_t pe = A.ts.idx(e, p);
          int32_t n_map = A.n_machines;
          if (stopped) {
            // the stopped twin {a, c, b, -}: its count so far minus ours at
            // the stop, plus our final count; our b.  With our key it is our
            // tuple (equal keys, identical tuples): the pair keeps one Map
            // tuple
            if (twin[jj].x == tu.a) {
              n_map = 1;
            } else {
              Tuple t1;
              t1.a = twin[jj].x;
              t1.c = twin[jj].y + tu.c;
              t1.b = tu.b;
              t1.pad = 0;
              *A.ts.at(e, p, 1) = t1;
            }
          }
          A.ts.nmap[pe] = n_map;
          A.ts.nslots[pe] = n_map;
        }
      }
    }
  }
}

// LDS bytes of map_slice_kernel for n_brows node-1 bitmap rows
inline size_t slice_lds(int n_brows) {
  return sizeof(uint64_t) * ((size_t)kSliceLevels * kSliceWin + (size_t)n_brows * kSliceWords) +
         sizeof(uint16_t) * kSliceTypes;
}

}  // namespace epk
