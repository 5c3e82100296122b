/*
 * epcount.h -- C ABI of the MI355X (gfx950) serial-episode counting library.
 *
 * Source page: "Towards Chip-on-Chip Neuroscience: Fast Mining of Frequent
 * Episodes Using Graphics Processors".
 *
 * The library counts, for each of S candidate episodes, the number of
 * non-overlapped occurrences of the serial episode
 *     E(1) -(t_low_1, t_high_1]-> E(2) -> ... -> E(N)
 * in one time-sorted event stream (opening section: support counting for M
 * episodes, each counted independently; "Design of MapConcatenate": the
 * episode with half-open inter-event delay intervals, Fig. 3 text: the
 * reference serial machine alpha_0 and non-overlapped occurrences).
 *
 * Definitions used by every entry point:
 *   - An occurrence is a choice of events (t_1,E(1)),...,(t_N,E(N)) of the
 *     stream with t_low_i < t_{i+1} - t_i <= t_high_i for i = 1..N-1.
 *   - Two occurrences are non-overlapped when one starts strictly after the
 *     other ends (equal times overlap).
 *   - The count of an episode is the largest number of pairwise
 *     non-overlapped occurrences.  It is an exact integer; the result does
 *     not depend on the order of events that share a time.
 *
 * The work runs on the GPU in one of two schemes (both exact, same result):
 *   PTPE       one GPU lane runs the serial counting machine for one episode
 *              over the whole stream (opening section, Algorithm 1 per thread).
 *   MAPCONCAT  the stream is cut into P time segments; each segment runs N
 *              machines per episode, machine k reset at
 *              tau_p - (t_high_1 + ... + t_high_k), that emit (a, count, b)
 *              tuples (Map rules 1-4, Figs. 4-5); a log-depth tree joins
 *              adjacent segments where the left exit b equals the right key a
 *              (Concatenate rules 1-3, Fig. 6).
 * AUTO picks PTPE when the episodes alone fill the GPU many times over and
 * MAPCONCAT otherwise (hybrid-algorithm section: "fully utilized" test on
 * episodes, threads per block, multiprocessors and resident blocks per
 * multiprocessor; the margin is measured, see ep_plan).
 *
 * Conventions shared by all calls:
 *   - Device pointers point into memory of the current HIP device; host
 *     pointers into ordinary host memory.  The caller owns every pointer; the
 *     library keeps none of them after the call returns.
 *   - Calls are asynchronous on `stream` unless stated otherwise: on EP_OK the
 *     outputs are valid once the stream has reached the end of the work the
 *     call enqueued.  Host-side argument errors are returned before anything
 *     is enqueued.  Scratch memory comes from blocks the library keeps per
 *     device until the process ends: a call reuses a free block (a block last
 *     used on another stream is waited for on the GPU with an event) and
 *     grows it with hipMallocAsync on `stream` when it is too small.
 *   - Inputs outside the documented domain (unsorted times) give unspecified
 *     counts unless `validate` is set in ep_options.
 *   - The library is thread-safe: concurrent calls never share a scratch
 *     block; the pinned staging ring for the episode table and each cached
 *     per-device figure are guarded by locks.
 *
 * Where this boundary differs from an all-device, allocate-per-call design,
 * and why:
 *   - The episode table is HOST memory.  The planner must read every delay
 *     bound before any launch: the window kind (bit masks, runs in registers,
 *     rings) and capacity follow from each interval ("Design of
 *     MapConcatenate": (t_low, t_high] per node pair; a window can hold up to
 *     floor(t_high / (t_high - t_low + 1)) + 1 separate runs), the segment
 *     halos from the largest Span (Map rules: machines start up to Span before
 *     a cut), and the hybrid choice from the episode count.  Reading a device
 *     table would cost a synchronisation per call; the library uploads the
 *     table itself, stream-ordered.
 *   - Scratch is cached per device (blocks grown on demand and kept) instead
 *     of allocated and freed in every call: a stream-ordered allocation and
 *     free per call cost more than the small workloads' whole count.  Callers
 *     that must not allocate at all use ep_count_episodes_noalloc.
 *   - Status codes beyond argument errors: EP_ERR_UNSUPPORTED (ep_mine's
 *     candidate limit) and EP_ERR_SCRATCH_LIMIT (the fixed array of
 *     ep_count_episodes_noalloc).  Every valid interval is counted.
 */
#ifndef EPCOUNT_H
#define EPCOUNT_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest supported episode size N. */
#define EP_MAX_NODES 16

/* Status codes returned by every entry point (0 = success). */
typedef enum {
  EP_OK = 0,
  EP_ERR_ARG = -1,         /* null pointer with a non-zero size, negative size, n_events > INT32_MAX */
  EP_ERR_NODES = -2,       /* n_nodes outside 1..EP_MAX_NODES */
  EP_ERR_INTERVAL = -3,    /* some t_low < 0, t_low >= t_high, or t_high_1+...+t_high_{N-1} > INT32_MAX */
  EP_ERR_UNSORTED = -4,    /* validate: times are not non-decreasing */
  EP_ERR_WORKSPACE = -5,   /* scratch allocation failed */
  EP_ERR_HIP = -6,         /* a HIP runtime call or kernel launch failed */
  EP_ERR_UNSUPPORTED = -7,   /* ep_mine only: a size has more candidates than max_candidates */
  EP_ERR_SCRATCH_LIMIT = -8  /* ep_count_episodes_noalloc: the call needs more than EP_NOALLOC_SCRATCH_BYTES */
} ep_status;

/*
 * Candidate runs per node window kept in registers.  A node window holds the
 * union of the intervals (t'+t_low, t'+t_high] over the candidate times t' of
 * the previous node; at most floor(t_high/(t_high-t_low+1)) + 1 disjoint runs
 * of it can be live at once.  Windows up to 63 ticks are bit masks; longer
 * ones whose bound is <= EP_MAX_RUNS keep their runs in registers; the rest
 * keep them in a ring of device memory sized by that bound (and by the
 * number of events, which no window can exceed), so every interval with
 * 0 <= t_low < t_high is counted exactly.
 */
#define EP_MAX_RUNS 4

/*
 * The candidate episode set, S episodes of the same size N.  HOST memory:
 * the planner reads the delay bounds to size the kernels' windows, then the
 * library copies the table to the device itself.
 *   n_nodes  N, 1 <= N <= EP_MAX_NODES.
 *   types    [S * N] event types, row-major: episode e's node k is types[e*N+k].
 *            A type may repeat inside an episode.
 *   t_low    [S * (N-1)] lower delay bounds, row-major (may be NULL if N == 1).
 *   t_high   [S * (N-1)] upper delay bounds, 0 <= t_low < t_high.
 */
typedef struct {
  int32_t n_nodes;
  const uint16_t* types;
  const int32_t* t_low;
  const int32_t* t_high;
} ep_episodes;

/*
 * Count S episodes over one event stream (the operation of the opening
 * section; scheme chosen by the hybrid rule).
 *   times       DEVICE, int32[n_events], non-decreasing event times (ticks).
 *   types       DEVICE, uint16[n_events], event types; SoA with `times`.
 *   n_events    0 <= n_events <= INT32_MAX.  0 gives all-zero counts.
 *   episodes    HOST table described above.
 *   n_episodes  S >= 0.  0 is a no-op.
 *   out_counts  DEVICE, int64[n_episodes], written with the counts.
 *   stream      HIP stream all work is enqueued on (0 = default stream).
 * Returns EP_OK or an ep_status error; on error `out_counts` is untouched
 * unless the error is EP_ERR_HIP.
 */
int ep_count_episodes(const int32_t* times, const uint16_t* types, int64_t n_events,
                      ep_episodes episodes, int64_t n_episodes, int64_t* out_counts,
                      hipStream_t stream);

/* Scheme selection for ep_count_episodes_ex. */
enum { EP_MODE_AUTO = 0, EP_MODE_PTPE = 1, EP_MODE_MAPCONCAT = 2 };

/* Optional statistics filled by ep_count_episodes_ex when `stats` is set.  A
 * call whose episodes need different window kinds runs one group per kind
 * (see EP_PLAN_NO_SPLIT); mode, n_segments and max_runs then describe the
 * group with the most episodes, kernels is the union over the groups and
 * repairs and fallbacks are their sums. */
typedef struct {
  int32_t mode;         /* scheme that ran: EP_MODE_PTPE or EP_MODE_MAPCONCAT */
  int32_t n_segments;   /* P (1 for PTPE) */
  int32_t max_runs;     /* window capacity: 32 / 64 (bit masks), else candidate runs per node */
  int32_t kernels;      /* bit 0: bit-window Map kernels (tick/list/position), else the
                           scan kernel; bit 1: one lane holds every machine of a
                           (segment, episode); bit 2: sparse segments through the event
                           filter and the list Map kernel (else the position kernel);
                           bit 3: the filter's lists pruned of entries that cannot act;
                           bit 4: ring windows (runs in device memory); bit 5: two-node
                           episodes through the type-sliced kernel (episodes sharing a
                           node-1 type and interval stepped together, one bit per
                           node-0 type) */
  int64_t repairs;      /* repair tuples made for unmatched segment exits */
  int64_t fallbacks;    /* episodes recounted by the whole-stream fallback */
  int32_t groups;       /* window-kind groups the call ran (1 unless split) */
  int32_t pad;
} ep_stats;

/*
 * Planner switches for ep_options.plan (bit flags, 0 = the planner decides).
 * None of them changes a result: they choose which kernels produce it, so
 * that tests can reach every kernel on small inputs and measurements can
 * compare schemes.
 */
enum {
  EP_PLAN_TICKS = 1 << 0,            /* every segment to the tick Map kernel */
  EP_PLAN_POSITIONS = 1 << 1,        /* every segment to the list or position Map kernel */
  EP_PLAN_LIST = 1 << 2,             /* the event filter + list kernel at any stream length */
  EP_PLAN_NO_LIST = 1 << 3,          /* never the list path (the position kernel instead) */
  EP_PLAN_PRUNE = 1 << 4,            /* list path: always prune the lists */
  EP_PLAN_NO_PRUNE = 1 << 5,         /* list path: never prune them */
  EP_PLAN_GROUP_STEPS = 1 << 6,      /* tick kernel: always order episodes by doubling steps */
  EP_PLAN_NO_GROUP_STEPS = 1 << 7,   /* tick kernel: never */
  EP_PLAN_RUN_WINDOWS = 1 << 8,      /* run windows and the scan kernel where bit windows fit */
  EP_PLAN_RING_WINDOWS = 1 << 9,     /* ring windows and the scan kernel for every episode */
  EP_PLAN_MACHINE_LANES = 1 << 10,   /* one Map machine per lane */
  EP_PLAN_NO_REDUCE = 1 << 11,       /* separate closure, tree and result launches */
  EP_PLAN_NO_REPAIR_QUEUE = 1 << 12, /* closure misses repaired where they are found (else queued
                                        for the repair kernel; past the queue, recounted whole) */
  EP_PLAN_RECOUNT = 1 << 13,         /* every episode taken through the whole-stream recount
                                        that guards repair-list overflow and tree misses */
  EP_PLAN_NO_SPLIT = 1 << 14,        /* one window kind for the whole call: the widest one
                                        any episode needs (else one group per kind) */
  EP_PLAN_SLICE = 1 << 15,           /* two-node episodes: the type-sliced kernel whenever the
                                        call fits it (node types below 2,048, windows up to
                                        63 ticks, no episode twice), however few episodes
                                        share a node-1 type and interval */
  EP_PLAN_NO_SLICE = 1 << 16,        /* two-node episodes: never the type-sliced kernel */
  EP_PLAN_TINY_REPAIR_QUEUE = 1 << 17 /* a one-entry repair queue: the closure's other misses send
                                        their episodes to the whole-stream recount */
};

/*
 * Options for ep_count_episodes_ex (a zeroed struct gives the defaults).
 *   mode        EP_MODE_AUTO, EP_MODE_PTPE or EP_MODE_MAPCONCAT.
 *   n_segments  MAPCONCAT only: P >= 1, 0 = chosen by the planner.  Any P is
 *               valid; the planner picks powers of two (Concatenate section).
 *   validate    non-zero: check on the device that times are non-decreasing
 *               and return EP_ERR_UNSORTED if not.  Synchronises `stream`.
 *   upper_only  non-zero: count the relaxed episodes alpha' of Algorithm A2
 *               (section on the constrained problem with upper limits only):
 *               the same event types and upper bounds with every lower bound
 *               taken as 0, so an occurrence needs 0 < t_{i+1} - t_i <= t_high_i.
 *               `episodes.t_low` is then not read (it may be NULL); every
 *               t_high must be > 0.  Every occurrence of an episode is one of
 *               its relaxed version, so count(alpha') >= count(alpha).  The
 *               relaxed windows never need more than one candidate run.
 *   stats       if non-NULL, filled after the work completes.  Synchronises
 *               `stream`.
 *   plan        EP_PLAN_* switches (0: the planner's choice).
 */
typedef struct {
  int32_t mode;
  int32_t n_segments;
  int32_t validate;
  int32_t upper_only;
  ep_stats* stats;
  uint32_t plan;
  int32_t pad;
} ep_options;

/* ep_count_episodes with explicit options (opt may be NULL = defaults). */
int ep_count_episodes_ex(const int32_t* times, const uint16_t* types, int64_t n_events,
                         ep_episodes episodes, int64_t n_episodes, int64_t* out_counts,
                         hipStream_t stream, const ep_options* opt);

/*
 * For callers that cannot allocate device memory (code being captured into a
 * HIP graph, tight serving loops, harnesses that forbid hipMalloc): the same
 * counts as ep_count_episodes_ex with the same arguments and options, but all
 * scratch comes from one fixed array of EP_NOALLOC_SCRATCH_BYTES per device
 * that the library's code object holds (placed when the library is first
 * used on the device, kept until the process ends), and the call allocates
 * nothing: no hipMalloc/hipFree, no pinned staging, no profiling events.  The
 * episode table reaches the device by a stream-ordered copy from pageable
 * host memory, which HIP reads before the call returns.
 *   When opt leaves n_segments to the planner, MapConcatenate's P is lowered
 *   until the plan fits the array (a speed trade, never a change of counts).
 *   Returns EP_ERR_SCRATCH_LIMIT, before anything is enqueued, when the plan
 *   still needs more scratch than the array holds (the need grows with
 *   episodes x segments and, on the list path, with the stream length);
 *   otherwise as ep_count_episodes_ex.
 *   Every call on a device uses that device's one array, which keeps the last
 *   call's contents: calls enqueued on one stream run one after another, but
 *   calls that overlap on a device (other streams, other host threads without
 *   ordering) race and give unspecified counts.
 */
#define EP_NOALLOC_SCRATCH_BYTES (64u << 20)
int ep_count_episodes_noalloc(const int32_t* times, const uint16_t* types, int64_t n_events,
                              ep_episodes episodes, int64_t n_episodes, int64_t* out_counts,
                              hipStream_t stream, const ep_options* opt);

/*
 * Two-pass elimination A2+A1 for a support threshold (two-pass elimination
 * section): the first pass counts every relaxed episode alpha' (upper_only
 * above); episodes whose relaxed count is below `threshold` cannot be frequent
 * (count(alpha) <= count(alpha') < threshold) and are dropped; the second pass
 * counts the remaining episodes exactly.
 *   times, types, n_events, episodes, n_episodes  as in ep_count_episodes
 *               (the full table, t_low included, is checked before any work).
 *   threshold   support threshold; episodes with relaxed count >= threshold
 *               go to the second pass (threshold <= 0 keeps every episode).
 *   out_counts  DEVICE, int64[n_episodes]: count(alpha_e) for the episodes
 *               kept, -1 for the dropped ones.  The frequent episodes are
 *               those with out_counts[e] >= threshold.
 *   out_upper   DEVICE, int64[n_episodes]: the first pass's counts
 *               count(alpha'_e) of every episode.
 *   n_kept      HOST, may be NULL: receives the number of episodes counted in
 *               the second pass.
 *   stream      as in ep_count_episodes.
 *   opt         may be NULL; mode, n_segments and validate apply to both
 *               passes, stats to the second pass (left untouched when no
 *               episode is kept); upper_only must be 0 (else EP_ERR_ARG).
 * The host needs the first pass's counts to build the second pass's table, so
 * the call synchronises `stream` once between the passes; the second pass and
 * the final scatter are enqueued asynchronously as usual.  Returns EP_OK or an
 * ep_status error (as in ep_count_episodes_ex).
 */
int ep_count_two_pass(const int32_t* times, const uint16_t* types, int64_t n_events,
                      ep_episodes episodes, int64_t n_episodes, int64_t threshold,
                      int64_t* out_counts, int64_t* out_upper, int64_t* n_kept,
                      hipStream_t stream, const ep_options* opt);

/*
 * Level-wise mining of frequent serial episodes: the mining loop whose
 * counting step the schemes above serve (opening section: the counting of
 * candidate episodes is the costly part of mining; two-pass elimination
 * section: candidates counted level by level).  Episodes of one size are
 * counted together on the GPU; the frequent ones (count >= threshold) of size
 * k give the candidates of size k+1:
 *   size 1    every alphabet type;
 *   size 2    every ordered pair (a, c) of frequent types, once per bin;
 *   size k+1  alpha followed by beta's last bin and type, for every frequent
 *             alpha and beta where beta without its last node equals alpha
 *             without its first node (types and bins).
 * Removing the first or last node of an occurrence leaves an occurrence of
 * the shorter episode and keeps occurrences non-overlapped, so these joins
 * reach every frequent episode up to max_nodes.
 */
typedef struct {
  int32_t n_bins;          /* delay intervals a candidate may use between consecutive nodes */
  const int32_t* bin_lo;   /* HOST [n_bins], distinct bins with 0 <= bin_lo[i] < bin_hi[i] */
  const int32_t* bin_hi;   /* HOST [n_bins] */
  int32_t max_nodes;       /* largest episode size mined, 1 .. EP_MAX_NODES */
  int64_t threshold;       /* an episode is frequent when its count >= threshold (>= 1) */
  int32_t two_pass;        /* non-zero: count sizes >= 2 with ep_count_two_pass */
  int32_t mode;            /* scheme of the counting calls: EP_MODE_AUTO / PTPE / MAPCONCAT */
  int64_t max_candidates;  /* > 0: return EP_ERR_UNSUPPORTED when a size has more candidates */
} ep_mine_options;

/* Opaque result of ep_mine: the frequent episodes of each size, in host
 * memory owned by the library until ep_mined_free. */
typedef struct ep_mined ep_mined;

/*
 * Mine the frequent episodes of one event stream.
 *   times, types, n_events  DEVICE event stream as in ep_count_episodes.
 *   alphabet    HOST uint16[n_alphabet], the event types to mine over
 *               (duplicates are ignored).
 *   opt         options above (required).
 *   stream      HIP stream the counting work is enqueued on; the call
 *               synchronises it once per size (the next candidates depend on
 *               the counts).
 *   out         receives the result (NULL on error); free with ep_mined_free.
 * Returns EP_OK, EP_ERR_ARG (null or negative arguments, threshold < 1,
 * n_bins < 1 with max_nodes > 1, duplicate bins), EP_ERR_NODES (max_nodes out
 * of range), EP_ERR_INTERVAL (a bad bin), EP_ERR_UNSUPPORTED (too many
 * candidates, or a bin the counting kernels cannot hold), or an error of the
 * counting calls.  Rows of every size are in increasing order of
 * (type 1, bin 1, type 2, bin 2, ..., type k), bins by their index in opt.
 */
int ep_mine(const int32_t* times, const uint16_t* types, int64_t n_events,
            const uint16_t* alphabet, int32_t n_alphabet, const ep_mine_options* opt,
            hipStream_t stream, ep_mined** out);

/* Largest episode size with a frequent episode (0 if none). */
int32_t ep_mined_max_nodes(const ep_mined* m);
/* Frequent episodes of size n_nodes (0 outside 1..ep_mined_max_nodes). */
int64_t ep_mined_count(const ep_mined* m, int32_t n_nodes);
/* Candidates counted at size n_nodes (0 if that size was not reached). */
int64_t ep_mined_candidates(const ep_mined* m, int32_t n_nodes);
/*
 * Copy the frequent episodes of size k = n_nodes into HOST arrays sized by
 * ep_mined_count: types [count * k], t_low / t_high [count * (k-1)] (may be
 * NULL when k == 1), counts [count].  Returns EP_OK or EP_ERR_ARG.
 */
int ep_mined_get(const ep_mined* m, int32_t n_nodes, uint16_t* types, int32_t* t_low,
                 int32_t* t_high, int64_t* counts);
/* Release a result (NULL is a no-op). */
void ep_mined_free(ep_mined* m);

/*
 * Streaming counts: the stream arrives in batches and the counts after each
 * batch are those of all events pushed so far (the tuple carry of the
 * Concatenate section, across calls).  Between batches each episode keeps
 * the time of the last completion of its reference machine alpha_0 when it
 * lies within Span of the last event pushed, and the stream keeps the events
 * within maxSpan (the largest Span of the table) of that last event: an
 * occurrence completing later starts no earlier than Span before it, so
 * these fix every later count exactly.  Each push counts those kept events
 * again in front of the new ones (device memory: the kept events plus one
 * copy of the batch).  A stream object is used by one host thread at a time.
 */
typedef struct ep_stream ep_stream;

/*
 * Create a stream for a fixed episode table (HOST, copied; as in
 * ep_count_episodes).  opt may be NULL; its mode and n_segments guide the
 * per-batch plans (batches are counted with MAPCONCAT, P capped so that every
 * segment spans at least maxSpan ticks), validate checks each batch's order,
 * upper_only counts the relaxed episodes; stats is ignored.  The running
 * counts start at 0 on the current device, set on `stream`.  Returns EP_OK,
 * EP_ERR_ARG, EP_ERR_NODES, EP_ERR_INTERVAL, EP_ERR_WORKSPACE or EP_ERR_HIP;
 * *out is NULL on error.
 */
int ep_stream_create(ep_episodes episodes, int64_t n_episodes, const ep_options* opt,
                     hipStream_t stream, ep_stream** out);

/*
 * Count one batch: DEVICE times/types [n_events], non-decreasing, the first
 * time not before the last time of the previous batch (equal times are
 * allowed: a tick may span two batches).  Synchronises `stream` (the next
 * batch's plan depends on this one's last events).  Returns EP_OK,
 * EP_ERR_ARG (bad arguments, or another device than the stream's),
 * EP_ERR_UNSORTED (the batch starts before the previous one ended, or with
 * validate, is unsorted), or an error of the counting path.  On an error the
 * stream's counts are unspecified.
 */
int ep_stream_push(ep_stream* st, const int32_t* times, const uint16_t* types, int64_t n_events,
                   hipStream_t stream);

/* Copy the running counts (DEVICE int64[n_episodes]) on `stream`. */
int ep_stream_counts(const ep_stream* st, int64_t* out_counts, hipStream_t stream);

/* Events pushed so far. */
int64_t ep_stream_events(const ep_stream* st);

/* Release a stream (NULL is a no-op); waits for the device. */
void ep_stream_destroy(ep_stream* st);

/*
 * The planner alone, on a described device (no GPU needed): which scheme and
 * segment count a call would use.
 *   n_episodes, n_nodes, n_events  sizes of the call.
 *   mode, n_segments               as in ep_options.
 *   cu_count                       multiprocessors of the device (MP).
 *   lanes_per_cu                   resident lanes per multiprocessor of the
 *                                  counting kernel (T_B * B_MP).
 *   out_mode, out_segments         results (host pointers).
 * Rule (hybrid-algorithm section): PTPE iff n_episodes >= 6 * cu_count *
 * lanes_per_cu (the factor measured on MI355X: MAPCONCAT was faster up to
 * 5.3 times the resident lanes, PTPE from 10.7 times); otherwise MAPCONCAT
 * with the smallest power-of-two P such
 * that lanes(P) >= cu_count * lanes_per_cu, where a lane carries the N
 * machines of one (segment, episode) for N <= 8 (lanes = n_episodes * P) and
 * one machine beyond (lanes = n_episodes * n_nodes * P); P is then raised
 * until segments hold <= 32,768 events on average (a boundary repair rescans
 * one segment), and capped so that a segment keeps on average >= 64 events
 * when n_episodes < 256, >= 256 events otherwise, and P <= 2^20.
 */
int ep_plan(int64_t n_episodes, int32_t n_nodes, int64_t n_events, int32_t mode,
            int32_t n_segments, int32_t cu_count, int32_t lanes_per_cu,
            int32_t* out_mode, int32_t* out_segments);

/* Equal-time cut p (0 <= p <= P) of a stream spanning [t_min, t_max]:
 * t_min - 1 + floor(p * (t_max - t_min + 1) / P).  Segment p (0-based) holds
 * the events with time in (cut(p), cut(p+1)] ("Design of MapConcatenate":
 * events of segment p lie in (tau_p, tau_{p+1}]). */
int64_t ep_segment_cut(int32_t t_min, int32_t t_max, int32_t n_segments, int32_t p);

/*
 * Per-phase GPU durations for measurement.  Between ep_profile_begin() and
 * ep_profile_end(), every counting call also records HIP events on its stream
 * around its phases; nothing is synchronised until ep_profile_end(), which
 * waits for the recorded events and returns the summed durations.  Calls made
 * outside a session record nothing.  Sessions are process-wide (one at a
 * time); ep_profile_end() returns EP_ERR_ARG if none is open.
 *   map_ms            Map step, both kernels (PTPE: the whole count)
 *   closure_ms        boundary match + repair
 *   concat_ms         all Concatenate tree levels
 *   other_ms          cuts, fills, extraction, fallback
 *   calls             counting calls recorded
 *   map_ticks_ms      the tick Map kernel alone (part of map_ms)
 *   map_positions_ms  the list or position Map kernel, or the scan Map kernel
 *                     when windows are runs (part of map_ms)
 *   map_filter_ms     the event filter feeding the list Map kernel (part of
 *                     map_ms; 0 when the call does not use it)
 *   map_prune_ms      the pruning of the filter's lists (part of map_ms; 0
 *                     when the call does not use them)
 */
typedef struct {
  double map_ms;
  double closure_ms;
  double concat_ms;
  double other_ms;
  int64_t calls;
  double map_ticks_ms;
  double map_positions_ms;
  double map_filter_ms;
  double map_prune_ms;
} ep_profile;

int ep_profile_begin(void);
int ep_profile_end(ep_profile* out);

/*
 * A lighter session for timing one Map kernel while the calls themselves are
 * being timed: only the two events around that kernel are recorded, on one
 * call in `every` (every >= 1), so the calls' own duration is barely
 * disturbed (each recorded event costs the stream a few microseconds).
 * ep_profile_end() then fills map_ms, the chosen kernel's field and calls
 * (= calls recorded).  Returns EP_ERR_ARG for an unknown kernel or every < 1.
 */
enum { EP_PROFILE_FILTER = 0, EP_PROFILE_TICKS = 1, EP_PROFILE_POSITIONS = 2, EP_PROFILE_PRUNE = 3 };
int ep_profile_begin_kernel(int32_t which, int32_t every);

/* Static text for a status code. */
const char* ep_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* EPCOUNT_H */
