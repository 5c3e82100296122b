/*
 * CPU ORACLE FOR SERIAL-EPISODE COUNTING -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the package smoke check and the benchmark's CPU-baseline
 * leg may load this file's shared object.  The library's product path never
 * does, and this file shares no code, header or constant with the HIP path.
 *
 * Source page: "Towards Chip-on-Chip Neuroscience: Fast Mining of Frequent
 * Episodes Using Graphics Processors".
 *
 * What it computes (plain reading of the page):
 *   - An episode is a serial chain E(1) -(lo_1,hi_1]-> E(2) ... -> E(N): N event
 *     types and N-1 half-open inter-event delay intervals (section "Design of
 *     MapConcatenate", the episode definition before Fig. 4).
 *   - An occurrence picks events (t_1,E(1)) ... (t_N,E(N)) of the stream with
 *     lo_i < t_{i+1} - t_i <= hi_i.  With lo_i >= 0 the times strictly increase.
 *   - The support is the number of non-overlapped occurrences (Fig. 3 text): we
 *     read "non-overlapped" as "each occurrence starts strictly after the
 *     previous one ended", and the count is the largest such set.
 *   - The reference serial state machine (alpha_0 in the Fig. 3 text, Algorithm
 *     1 of the opening section, whose body did not survive) keeps one
 *     timestamp list per node (the s[E(k)] lists of the two-pass elimination
 *     section, whose constraint check is linear in the list length).  We
 *     restate it here from that description:
 *
 *       r := -infinity; lists L[1..N-1] empty; count := 0
 *       for each event (t, y) in stream order:
 *         if t <= r: skip                         (non-overlap is strict in time)
 *         if y = E(N) and (N = 1 or some t' in L[N-1] has lo < t - t' <= hi):
 *             count += 1; r := t; empty every list; next event
 *         for every k < N with y = E(k):          (an episode may repeat a type)
 *             if k = 1 or some t' in L[k-1] has lo < t - t' <= hi: append t to L[k]
 *
 *     Entries t' < t - hi of a list can never satisfy the upper bound again
 *     (times only grow), so the scan drops them from the list's front; this
 *     changes no answer.  Stopping at the first (earliest-ending) completion
 *     after each reset is the earliest-finish greedy rule, which is optimal
 *     for choosing the most pairwise-disjoint occurrences.
 *
 * Inputs are assumed valid: times non-decreasing, 0 <= lo < hi.  Nothing here
 * is tuned; it is meant to be read against the page by eye.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* A growable ascending list of int32 times with a consumed-prefix index. */
typedef struct {
  int32_t* v;
  int64_t head; /* first live entry */
  int64_t size; /* one past the last entry */
  int64_t cap;
} tlist;

static int tlist_push(tlist* L, int32_t t) {
  if (L->size == L->cap) {
    /* reclaim the dropped prefix before growing */
    if (L->head > 0) {
      memmove(L->v, L->v + L->head, (size_t)(L->size - L->head) * sizeof(int32_t));
      L->size -= L->head;
      L->head = 0;
    }
    if (L->size == L->cap) {
      int64_t ncap = L->cap ? 2 * L->cap : 16;
      int32_t* nv = (int32_t*)realloc(L->v, (size_t)ncap * sizeof(int32_t));
      if (!nv) return -1;
      L->v = nv;
      L->cap = ncap;
    }
  }
  L->v[L->size++] = t;
  return 0;
}

/* Is there t' in L with lo < t - t' <= hi?  Drops entries with t - t' > hi. */
static int tlist_has_predecessor(tlist* L, int64_t t, int64_t lo, int64_t hi) {
  while (L->head < L->size && t - (int64_t)L->v[L->head] > hi) L->head++;
  for (int64_t j = L->head; j < L->size; ++j) {
    int64_t d = t - (int64_t)L->v[j];
    if (d > lo && d <= hi) return 1;
  }
  return 0;
}

/*
 * Count the non-overlapped occurrences of one episode over the whole stream.
 *   times[n] (non-decreasing), types[n]
 *   ep_types[N], lo[N-1], hi[N-1]
 * Returns the count, or -1 if memory ran out.
 */
int64_t oracle_count_one(const int32_t* times, const uint16_t* types, int64_t n,
                         int32_t N, const uint16_t* ep_types, const int32_t* lo,
                         const int32_t* hi) {
  if (N < 1) return -1;
  tlist* L = (tlist*)calloc((size_t)(N > 1 ? N - 1 : 1), sizeof(tlist));
  if (!L) return -1;
  int64_t r = INT64_MIN; /* time of the last counted completion */
  int64_t count = 0;
  int failed = 0;
  for (int64_t i = 0; i < n && !failed; ++i) {
    int64_t t = times[i];
    uint16_t y = types[i];
    if (t <= r) continue;
    if (ep_types[N - 1] == y) {
      int done = (N == 1) || tlist_has_predecessor(&L[N - 2], t, lo[N - 2], hi[N - 2]);
      if (done) {
        count += 1;
        r = t;
        for (int k = 0; k < N - 1; ++k) L[k].head = L[k].size = 0;
        continue;
      }
    }
    for (int k = 0; k < N - 1; ++k) {
      if (ep_types[k] != y) continue;
      int ok = (k == 0) || tlist_has_predecessor(&L[k - 1], t, lo[k - 1], hi[k - 1]);
      if (ok && tlist_push(&L[k], (int32_t)t) != 0) failed = 1;
    }
  }
  for (int k = 0; k < N - 1; ++k) free(L[k].v);
  free(L);
  return failed ? -1 : count;
}

/*
 * Algorithm A2 (section on the constrained problem with upper limits only):
 * the episode alpha' keeps the event types and upper bounds of alpha and
 * relaxes every lower bound to 0, so a predecessor qualifies when
 * 0 < t - t' <= hi.  Among the entries of the node list that are earlier
 * than t, the latest one is then the best candidate, so the constraint check
 * needs only that entry instead of a scan of the list (the O(1) check the
 * two-pass elimination section contrasts with the list scan).  A list is
 * therefore kept as its latest time and the latest time strictly before
 * that one (an entry on the tick of t itself is never a predecessor).
 * Counting, resets and non-overlap are those of oracle_count_one.
 */
typedef struct {
  int64_t last;   /* latest appended time, or NONE */
  int64_t before; /* latest appended time < last, or NONE */
} tlast;

#define TLAST_NONE INT64_MIN

static void tlast_push(tlast* L, int64_t t) {
  if (L->last == TLAST_NONE || t > L->last) {
    L->before = L->last;
    L->last = t;
  }
}

/* Is there an appended t' with 0 < t - t' <= hi?  Only the latest t' < t matters. */
static int tlast_has_predecessor(const tlast* L, int64_t t, int64_t hi) {
  int64_t p = (L->last != TLAST_NONE && L->last < t) ? L->last : L->before;
  return p != TLAST_NONE && p < t && t - p <= hi;
}

int64_t oracle_count_one_upper(const int32_t* times, const uint16_t* types, int64_t n,
                               int32_t N, const uint16_t* ep_types, const int32_t* hi) {
  if (N < 1) return -1;
  tlast* L = (tlast*)malloc(sizeof(tlast) * (size_t)(N > 1 ? N - 1 : 1));
  if (!L) return -1;
  for (int k = 0; k < N - 1; ++k) L[k].last = L[k].before = TLAST_NONE;
  int64_t r = INT64_MIN;
  int64_t count = 0;
  for (int64_t i = 0; i < n; ++i) {
    int64_t t = times[i];
    uint16_t y = types[i];
    if (t <= r) continue;
    if (ep_types[N - 1] == y) {
      int done = (N == 1) || tlast_has_predecessor(&L[N - 2], t, hi[N - 2]);
      if (done) {
        count += 1;
        r = t;
        for (int k = 0; k < N - 1; ++k) L[k].last = L[k].before = TLAST_NONE;
        continue;
      }
    }
    for (int k = 0; k < N - 1; ++k) {
      if (ep_types[k] != y) continue;
      if (k == 0 || tlast_has_predecessor(&L[k - 1], t, hi[k - 1])) tlast_push(&L[k], t);
    }
  }
  free(L);
  return count;
}

/* ---- episodes are independent (opening section): count them on a thread pool ---- */

typedef struct {
  const int32_t* times;
  const uint16_t* types;
  int64_t n;
  int32_t N;
  const uint16_t* ep_types; /* [S*N]     */
  const int32_t* lo;        /* [S*(N-1)] */
  const int32_t* hi;        /* [S*(N-1)] */
  int64_t S;
  int64_t* out;
  int upper_only; /* count alpha' (Algorithm A2) instead of alpha */
  int64_t next;   /* shared work counter */
  pthread_mutex_t mu;
} batch_job;

static void* batch_worker(void* arg) {
  batch_job* J = (batch_job*)arg;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int64_t e = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (e >= J->S) break;
    int64_t m = J->N > 1 ? J->N - 1 : 0;
    J->out[e] = J->upper_only
                    ? oracle_count_one_upper(J->times, J->types, J->n, J->N,
                                             J->ep_types + e * J->N, J->hi + e * m)
                    : oracle_count_one(J->times, J->types, J->n, J->N, J->ep_types + e * J->N,
                                       J->lo + e * m, J->hi + e * m);
  }
  return NULL;
}

/*
 * Count S episodes of N nodes each (upper_only: their relaxed versions alpha',
 * lo unused).  n_threads <= 0 means one thread.  Returns the number of threads
 * used.
 */
int oracle_count_batch_mode(const int32_t* times, const uint16_t* types, int64_t n, int32_t N,
                            const uint16_t* ep_types, const int32_t* lo, const int32_t* hi,
                            int64_t S, int64_t* out, int n_threads, int upper_only) {
  if (n_threads < 1) n_threads = 1;
  if ((int64_t)n_threads > S) n_threads = S > 0 ? (int)S : 1;
  batch_job J;
  J.times = times;
  J.types = types;
  J.n = n;
  J.N = N;
  J.ep_types = ep_types;
  J.lo = lo;
  J.hi = hi;
  J.S = S;
  J.out = out;
  J.upper_only = upper_only;
  J.next = 0;
  pthread_mutex_init(&J.mu, NULL);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)n_threads);
  int started = 0;
  for (int i = 0; i < n_threads && th; ++i)
    if (pthread_create(&th[i], NULL, batch_worker, &J) == 0) started++;
  if (started == 0) batch_worker(&J);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J.mu);
  return started > 0 ? started : 1;
}

int oracle_count_batch(const int32_t* times, const uint16_t* types, int64_t n, int32_t N,
                       const uint16_t* ep_types, const int32_t* lo, const int32_t* hi,
                       int64_t S, int64_t* out, int n_threads) {
  return oracle_count_batch_mode(times, types, n, N, ep_types, lo, hi, S, out, n_threads, 0);
}
