// Level-wise mining of frequent serial episodes (ep_mine and its result
// accessors): the host loop that builds candidates of size k+1 from the
// frequent episodes of size k and counts each size on the GPU through
// ep_count_episodes_ex or ep_count_two_pass.
//
// Source page: "Towards Chip-on-Chip Neuroscience: Fast Mining of Frequent
// Episodes Using Graphics Processors" (opening section: candidate counting is
// the costly step of mining; two-pass elimination section: candidates counted
// level by level, the first pass culling with upper bounds only).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "epcount.h"

struct ep_mined {
  struct Level {
    int32_t k = 0;
    int64_t candidates = 0;
    std::vector<uint16_t> types;   // [S * k]
    std::vector<int32_t> lo, hi;   // [S * (k-1)]
    std::vector<int64_t> counts;   // [S]
  };
  std::vector<Level> levels;  // levels[k-1]: frequent episodes of size k
};

namespace {

// A candidate set of one size: types [S * k] and bin indices [S * (k-1)].
struct Cands {
  int32_t k = 0;
  std::vector<uint16_t> types;
  std::vector<int32_t> bins;
  int64_t size() const { return k ? (int64_t)types.size() / k : 0; }
};

// Count one size's candidates; counts land in `cnt` (host).
int count_level(const int32_t* times, const uint16_t* types, int64_t n, const Cands& c,
                const ep_mine_options& o, hipStream_t stream, std::vector<int64_t>& cnt) {
  const int64_t S = c.size();
  const int32_t k = c.k;
  std::vector<int32_t> lo((size_t)(S * (k - 1))), hi((size_t)(S * (k - 1)));
  for (size_t i = 0; i < c.bins.size(); ++i) {
    lo[i] = o.bin_lo[c.bins[i]];
    hi[i] = o.bin_hi[c.bins[i]];
  }
  ep_episodes eps{k, c.types.data(), k > 1 ? lo.data() : nullptr, k > 1 ? hi.data() : nullptr};
  const bool two = o.two_pass && k > 1;
  int64_t* d = nullptr;
  if (hipMallocAsync((void**)&d, (size_t)S * sizeof(int64_t) * (two ? 2 : 1), stream) != hipSuccess)
    return EP_ERR_WORKSPACE;
  ep_options eo{};
  eo.mode = o.mode;
  ep_stats stats{};
  static const bool log_stats = getenv("EP_LOG_TIME") != nullptr;
  if (log_stats) eo.stats = &stats;
  int st;
  if (two) {
    st = ep_count_two_pass(times, types, n, eps, S, o.threshold, d, d + S, nullptr, stream, &eo);
  } else {
    st = ep_count_episodes_ex(times, types, n, eps, S, d, stream, &eo);
  }
  cnt.assign((size_t)S, 0);
  if (st == EP_OK &&
      (hipMemcpyAsync(cnt.data(), d, (size_t)S * sizeof(int64_t), hipMemcpyDeviceToHost, stream) !=
           hipSuccess ||
       hipStreamSynchronize(stream) != hipSuccess))
    st = EP_ERR_HIP;
  if (hipFreeAsync(d, stream) != hipSuccess && st == EP_OK) st = EP_ERR_HIP;
  if (log_stats && st == EP_OK)
    fprintf(stderr, "ep_mine: size %d: P = %d, kernels %d, repairs %lld, fallbacks %lld\n", (int)k,
            (int)stats.n_segments, (int)stats.kernels, (long long)stats.repairs, (long long)stats.fallbacks);
  // two passes: a dropped episode reads -1, below any threshold >= 1
  return st;
}

}  // namespace

extern "C" int ep_mine(const int32_t* times, const uint16_t* types, int64_t n_events,
                       const uint16_t* alphabet, int32_t n_alphabet, const ep_mine_options* opt,
                       hipStream_t stream, ep_mined** out) {
  if (!out) return EP_ERR_ARG;
  *out = nullptr;
  if (!opt || n_alphabet < 0 || n_events < 0 || n_events > INT32_MAX) return EP_ERR_ARG;
  if (n_alphabet > 0 && !alphabet) return EP_ERR_ARG;
  if (n_events > 0 && (!times || !types)) return EP_ERR_ARG;
  const ep_mine_options o = *opt;
  if (o.max_nodes < 1 || o.max_nodes > EP_MAX_NODES) return EP_ERR_NODES;
  if (o.threshold < 1) return EP_ERR_ARG;
  if (o.mode < EP_MODE_AUTO || o.mode > EP_MODE_MAPCONCAT) return EP_ERR_ARG;
  if (o.max_nodes > 1) {
    if (o.n_bins < 1 || !o.bin_lo || !o.bin_hi) return EP_ERR_ARG;
    for (int i = 0; i < o.n_bins; ++i) {
      if (o.bin_lo[i] < 0 || o.bin_lo[i] >= o.bin_hi[i]) return EP_ERR_INTERVAL;
      for (int j = 0; j < i; ++j)
        if (o.bin_lo[i] == o.bin_lo[j] && o.bin_hi[i] == o.bin_hi[j]) return EP_ERR_ARG;
    }
  }

  ep_mined* res = new ep_mined();
  Cands cur;
  cur.k = 1;
  {
    std::vector<uint16_t> a(alphabet, alphabet + n_alphabet);
    std::sort(a.begin(), a.end());
    a.erase(std::unique(a.begin(), a.end()), a.end());
    cur.types = a;
  }
  int status = EP_OK;
  // per-size host timings on stderr when EP_LOG_TIME is set
  static const bool log_time = getenv("EP_LOG_TIME") != nullptr;
  using clk = std::chrono::steady_clock;
  while (cur.size() > 0) {
    const int32_t k = cur.k;
    const int64_t S = cur.size();
    if (o.max_candidates > 0 && S > o.max_candidates) {
      status = EP_ERR_UNSUPPORTED;
      break;
    }
    std::vector<int64_t> cnt;
    const auto t0 = clk::now();
    status = count_level(times, types, n_events, cur, o, stream, cnt);
    const auto t1 = clk::now();
    if (status != EP_OK) break;
    ep_mined::Level lv;
    lv.k = k;
    lv.candidates = S;
    std::vector<int64_t> keep;  // candidate indices of the frequent ones, in order
    for (int64_t i = 0; i < S; ++i) {
      if (cnt[(size_t)i] < o.threshold) continue;
      keep.push_back(i);
      lv.types.insert(lv.types.end(), cur.types.begin() + i * k, cur.types.begin() + (i + 1) * k);
      for (int j = 0; j < k - 1; ++j) {
        const int32_t b = cur.bins[(size_t)(i * (k - 1) + j)];
        lv.lo.push_back(o.bin_lo[b]);
        lv.hi.push_back(o.bin_hi[b]);
      }
      lv.counts.push_back(cnt[(size_t)i]);
    }
    if (keep.empty()) break;
    res->levels.push_back(std::move(lv));
    if (k == o.max_nodes) break;

    // candidates of size k+1, generated in increasing key order
    Cands nxt;
    nxt.k = k + 1;
    if (k == 1) {
      for (int64_t ia : keep)
        for (int32_t b = 0; b < o.n_bins; ++b)
          for (int64_t ic : keep) {
            nxt.types.push_back(cur.types[(size_t)ia]);
            nxt.types.push_back(cur.types[(size_t)ic]);
            nxt.bins.push_back(b);
          }
    } else {
      // The frequent episodes are in key order (t1, b1, t2, ..., tk), so
      // those sharing their first k-1 nodes (t1, b1, ..., t_{k-1}: the key's
      // first 2k-3 entries) are contiguous.  Group starts, then for each
      // episode a the group whose first k-1 nodes equal a's last k-1 nodes.
      const int kl = 2 * k - 3;  // entries of a (k-1)-node key
      auto at = [&](int64_t i, int from, int x) -> int32_t {
        // entry x of the (k-1)-node key of episode i starting at node `from`
        return (x & 1) ? cur.bins[(size_t)(i * (k - 1) + from + x / 2)]
                       : (int32_t)cur.types[(size_t)(i * k + from + x / 2)];
      };
      auto cmp = [&](int64_t i, int fi, int64_t j, int fj) {
        for (int x = 0; x < kl; ++x) {
          const int32_t u = at(i, fi, x), v = at(j, fj, x);
          if (u != v) return u < v ? -1 : 1;
        }
        return 0;
      };
      std::vector<int64_t> starts;  // index into keep of each group's first episode
      for (size_t q = 0; q < keep.size(); ++q)
        if (q == 0 || cmp(keep[q - 1], 0, keep[q], 0) != 0) starts.push_back((int64_t)q);
      starts.push_back((int64_t)keep.size());
      int64_t total = 0;
      std::vector<int64_t> hit_group(keep.size(), -1);
      for (size_t qa = 0; qa < keep.size(); ++qa) {
        const int64_t ia = keep[qa];
        int64_t lo = 0, hi = (int64_t)starts.size() - 1;  // search groups [lo, hi)
        while (lo < hi) {
          const int64_t mid = (lo + hi) / 2;
          if (cmp(keep[(size_t)starts[(size_t)mid]], 0, ia, 1) < 0)
            lo = mid + 1;
          else
            hi = mid;
        }
        if (lo < (int64_t)starts.size() - 1 && cmp(keep[(size_t)starts[(size_t)lo]], 0, ia, 1) == 0) {
          hit_group[qa] = lo;
          total += starts[(size_t)lo + 1] - starts[(size_t)lo];
        }
      }
      nxt.types.reserve((size_t)total * (k + 1));
      nxt.bins.reserve((size_t)total * k);
      for (size_t qa = 0; qa < keep.size(); ++qa) {
        if (hit_group[qa] < 0) continue;
        const int64_t ia = keep[qa];
        const int64_t g = hit_group[qa];
        for (int64_t qb = starts[(size_t)g]; qb < starts[(size_t)g + 1]; ++qb) {
          const int64_t ib = keep[(size_t)qb];
          for (int j = 0; j < k; ++j) nxt.types.push_back(cur.types[(size_t)(ia * k + j)]);
          nxt.types.push_back(cur.types[(size_t)(ib * k + k - 1)]);
          for (int j = 0; j < k - 1; ++j) nxt.bins.push_back(cur.bins[(size_t)(ia * (k - 1) + j)]);
          nxt.bins.push_back(cur.bins[(size_t)(ib * (k - 1) + k - 2)]);
        }
      }
    }
    cur = std::move(nxt);
    if (log_time)
      fprintf(stderr, "ep_mine: size %d, %lld candidates: count %.1f us, next size %.1f us\n", (int)k,
              (long long)S, std::chrono::duration<double, std::micro>(t1 - t0).count(),
              std::chrono::duration<double, std::micro>(clk::now() - t1).count());
  }
  if (status != EP_OK) {
    delete res;
    return status;
  }
  *out = res;
  return EP_OK;
}

extern "C" int32_t ep_mined_max_nodes(const ep_mined* m) {
  return m ? (int32_t)m->levels.size() : 0;
}

extern "C" int64_t ep_mined_count(const ep_mined* m, int32_t n_nodes) {
  if (!m || n_nodes < 1 || n_nodes > (int32_t)m->levels.size()) return 0;
  return (int64_t)m->levels[(size_t)n_nodes - 1].counts.size();
}

extern "C" int64_t ep_mined_candidates(const ep_mined* m, int32_t n_nodes) {
  if (!m || n_nodes < 1 || n_nodes > (int32_t)m->levels.size()) return 0;
  return m->levels[(size_t)n_nodes - 1].candidates;
}

extern "C" int ep_mined_get(const ep_mined* m, int32_t n_nodes, uint16_t* types, int32_t* t_low,
                            int32_t* t_high, int64_t* counts) {
  if (!m || n_nodes < 1 || n_nodes > (int32_t)m->levels.size()) return EP_ERR_ARG;
  const ep_mined::Level& lv = m->levels[(size_t)n_nodes - 1];
  const size_t S = lv.counts.size();
  if (S == 0) return EP_OK;
  if (!types || !counts || (n_nodes > 1 && (!t_low || !t_high))) return EP_ERR_ARG;
  memcpy(types, lv.types.data(), lv.types.size() * sizeof(uint16_t));
  if (n_nodes > 1) {
    memcpy(t_low, lv.lo.data(), lv.lo.size() * sizeof(int32_t));
    memcpy(t_high, lv.hi.data(), lv.hi.size() * sizeof(int32_t));
  }
  memcpy(counts, lv.counts.data(), S * sizeof(int64_t));
  return EP_OK;
}

extern "C" void ep_mined_free(ep_mined* m) { delete m; }
