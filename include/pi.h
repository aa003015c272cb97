/*
 * pi.h -- C ABI of the predictor-gated, neuron-aware sparse FFN for AMD
 * Instinct MI355X (gfx950).
 *
 * The method (PowerInfer pages):
 *  - chatpaper.ai abstract; CSDN article, section on sparse activation: a
 *    small per-layer predictor names the FFN neurons an input will activate,
 *    and neuron-aware sparse operators compute only those neurons.
 *  - CSDN article, section on the CPU/GPU hybrid design and its figure: each
 *    memory partition ("hot" and "cold") computes the predicted neurons it
 *    holds; the partial results are merged.
 *  - CSDN article, overall-architecture section; hada.io README summary
 *    (--vram-budget, GPU index): an offline step profiles activation
 *    frequencies and places the most frequently active neurons in the fast
 *    partition under a memory budget.
 *  - hada.io README summary, quantisation section: INT4 weights in Q4_0.
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers owned by the caller unless marked
 *    [host].  The library never allocates, frees or retains caller memory.
 *  - Every call only enqueues work on `stream` (a hipStream_t passed as
 *    void*, NULL = the default stream) and returns; no call synchronises
 *    the host except pi_kernel_timer_stop and the two calls that compute on
 *    the host cores (pi_host_sparse_ffn, pi_sparse_ffn_hybrid).
 *  - Arguments are validated before anything is enqueued; on an error the
 *    call enqueues nothing and returns a nonzero pi_status.  pi_last_error()
 *    then holds a message (thread-local).
 *  - Weight, input and output tensors must be 16-byte aligned; index lists,
 *    counts and masks 8-byte aligned.
 *  - Layout: one neuron owns one row.  W_up, W_gate and W_downT (the
 *    transpose of W_down) are [rows][d] row-major; P1t is [r][d]; P2t is
 *    [n][r]; biases are float32 [rows].  x is [B][d].
 *  - A Q4_0 row of d elements (d % 256 == 0) is d/2 code bytes followed by
 *    d/32 fp16 scales (9d/16 bytes).  Code byte 16*j + t (t < 16) holds
 *    element 32*j + t in its low nibble and element 32*j + t + 16 in its
 *    high nibble; element value = (code - 8) * scale_j.
 *  - Calls on one stream run in order.  Two calls that share a workspace
 *    must not run concurrently (on different streams).
 */
#ifndef PI_H
#define PI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pi_status;
enum {
    PI_OK = 0,
    PI_ERR_ARG = 1,        /* NULL where a tensor is required, bad enum, bad option */
    PI_ERR_SHAPE = 2,      /* a size out of range or not a multiple the layout needs */
    PI_ERR_ALIGN = 3,      /* a pointer misaligned for its role */
    PI_ERR_DTYPE = 4,      /* unsupported dtype combination */
    PI_ERR_WORKSPACE = 5,  /* workspace missing or smaller than pi_workspace_bytes() */
    PI_ERR_BUDGET = 6,     /* negative budget or non-positive bytes per neuron */
    PI_ERR_HIP = 7         /* the HIP runtime reported an error while enqueueing */
};

/* element storage types */
enum { PI_F32 = 0, PI_F16 = 1, PI_Q4_0 = 2 };
/* FFN activations (hada.io README summary, supported models: ReLU, ReGLU and
 * squared-ReLU models) */
enum { PI_RELU = 0, PI_REGLU = 1, PI_SQRELU = 2 };

/* Largest batch a call accepts. */
#define PI_MAX_BATCH 64

/*
 * Low-rank activation predictor of one layer (CSDN article, section on
 * sparse activation):
 *   u[b][j]     = max(0, sum_k P1t[j][k] * x[b][k])        j < r
 *   logit[b][i] = sum_j P2t[i][j] * u[b][j] + b2[i]        i < n
 *   active(i)   = OR over tokens b of (logit[b][i] > threshold)
 * u and logits are float32 (never rounded to a narrower type).
 */
typedef struct pi_predictor {
    int32_t d;            /* model width, d % 64 == 0 */
    int32_t n;            /* neurons, n >= 1 */
    int32_t r;            /* predictor rank, r % 16 == 0 */
    int32_t wdtype;       /* PI_F32 or PI_F16 for P1t and P2t */
    const void* P1t;      /* [r][d] */
    const void* P2t;      /* [n][r] */
    const float* b2;      /* [n] or NULL (zeros) */
    float threshold;      /* strict: logit > threshold is active */
} pi_predictor;

/*
 * A partition (a contiguous block of rows of the neuron-permuted layer) of a
 * ReLU or ReGLU FFN layer.  Per token b and listed neuron i:
 *   ReLU : h = max(0, W_up[i].x_b + b_up[i])
 *   ReGLU: h = max(0, W_gate[i].x_b + b_gate[i]) * (W_up[i].x_b + b_up[i])
 *   y_b += h * W_downT[i][:]
 * NULL biases are zeros; there is no down-projection bias.
 */
typedef struct pi_ffn_part {
    int32_t d;            /* model width: d % 64 == 0 (d % 256 == 0 for Q4_0) */
    int32_t rows;         /* neurons in this partition, >= 0 */
    int32_t wdtype;       /* PI_F32, PI_F16 or PI_Q4_0 (all three matrices) */
    int32_t act;          /* PI_RELU, PI_REGLU or PI_SQRELU (h = max(0, W_up.x + b_up)^2) */
    const void* W_up;     /* [rows][d] */
    const void* W_gate;   /* [rows][d], required for PI_REGLU, ignored otherwise */
    const float* b_up;    /* [rows] or NULL */
    const float* b_gate;  /* [rows] or NULL */
    const void* W_downT;  /* [rows][d] */
} pi_ffn_part;

/*
 * Active-neuron lists split at n_hot (CSDN article, hybrid-design figure:
 * the predicted ids go to the partition that holds them).  Ids are in the
 * permuted layer: hot ids are < n_hot, cold ids are stored minus n_hot.
 * Both lists are ascending; counts[0] = hot count, counts[1] = cold count
 * (device memory, so no host round trip is needed between calls).
 */
typedef struct pi_active_lists {
    int32_t n_hot;        /* 0 <= n_hot <= n */
    int32_t* hot_idx;     /* [n_hot] capacity */
    int32_t* cold_idx;    /* [n - n_hot] capacity; may be NULL iff n_hot == n */
    int32_t* counts;      /* [2] */
} pi_active_lists;

/*
 * Workspace bytes that suffice for every call below on a layer with these
 * sizes and any batch up to B (d model width, n neurons, r predictor rank).
 * Returns 0 if the sizes are out of range.
 */
size_t pi_workspace_bytes(int32_t d, int32_t n, int32_t r, int32_t B);

/*
 * Zero-fills a workspace (with a fill kernel).  Optional: calls keep no
 * state in the workspace between them and need no particular contents.
 */
pi_status pi_workspace_init(void* ws, size_t ws_bytes, void* stream);

/*
 * Predicts the active neurons of one layer for the B tokens of x [B][d]
 * (xdtype PI_F32 or PI_F16).
 *   mask   [ceil(n/64)] uint64, out: bit i % 64 of word i / 64 is set iff
 *          neuron i is active for some token; bits >= n are 0.
 *   logits [B][n] float32, out, or NULL.
 *   lists  optional: if not NULL, the same call also compacts the mask into
 *          ascending hot/cold lists (it enqueues pi_compact_active's kernel).
 * Needs a workspace (pi_workspace_bytes).
 */
pi_status pi_predict(const pi_predictor* p, const void* x, int32_t B, int32_t xdtype,
                     uint64_t* mask, float* logits, const pi_active_lists* lists,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * Compaction of the predicted set into the lists the partitions compute (CSDN
 * article, section on sparse activation: only the predicted neurons are
 * computed; hybrid-design figure: the predicted ids, e.g. 3, 4, 5, go to the
 * partition that holds each one).  mask [ceil(n/64)] uint64 device, 8-byte
 * aligned, as written by pi_predict; bits >= n are ignored.  lists (see
 * pi_active_lists) receives hot ids < n_hot and cold ids - n_hot, both
 * ascending, and the device counts; the lists must hold n_hot and n - n_hot
 * entries.  One workgroup; no workspace.  Errors (NULL mask or lists, n out
 * of 1..2^24, n_hot outside 0..n, a list missing for a non-empty partition,
 * misalignment) enqueue nothing.
 */
pi_status pi_compact_active(const uint64_t* mask, int32_t n, const pi_active_lists* lists,
                            void* stream);

/*
 * Sparse FFN over one partition (CSDN article, section on sparse activation:
 * neuron-aware operators read and compute only the rows of the predicted
 * neurons; neurons that do not fire contribute nothing):
 *   y[b][:] = sum over the first *count entries i of idx of h_bi * W_downT[i][:]
 * with h as in pi_ffn_part, every token over the same list.  x [B][d]
 * (xdtype PI_F32 or PI_F16, 16-byte aligned); idx int32 device, ascending ids
 * < part->rows (an id outside the partition contributes nothing); count a
 * device int32 scalar (clamped to 0..part->rows); y [B][d] float32,
 * overwritten.  Rows not listed are never read.  Needs a workspace
 * (pi_workspace_bytes); errors enqueue nothing.
 */
pi_status pi_sparse_ffn(const pi_ffn_part* part, const void* x, int32_t B, int32_t xdtype,
                        const int32_t* idx, const int32_t* count, float* y,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * Sparse FFN over the hot and the cold partition in one pass, with the merge
 * fused: y_hot and y_cold receive the two partial outputs (each may be NULL),
 * y receives y_hot + y_cold (may be NULL).  cold may be NULL (or have 0
 * rows) when there is no cold partition.  Both partitions need the same d,
 * wdtype and act, and lists->n_hot == hot->rows.
 *   mask NULL:  the active set is `lists` as given (from pi_predict or
 *               pi_compact_active), an input.
 *   mask given: the active set is mask [ceil(n/64)] (n = hot rows + cold
 *               rows, from pi_predict); the compaction is fused into this
 *               call and `lists` (ids, counts) are outputs, identical to
 *               what pi_compact_active would write.
 */
pi_status pi_sparse_ffn_split(const pi_ffn_part* hot, const pi_ffn_part* cold, const void* x,
                              int32_t B, int32_t xdtype, const uint64_t* mask,
                              const pi_active_lists* lists, float* y_hot, float* y_cold, float* y,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation, arguments and results as pi_sparse_ffn_split, with no workspace
 * argument.  Its scratch (h and the fp32 partials of y) lives in a static
 * device array of PI_SCRATCH_BYTES bytes inside the library; each GPU the
 * library runs on holds its own copy of it until the process ends.  The call
 * allocates nothing (no hipMalloc, no allocating library routine).
 *  - Calls whose scratch need (what pi_workspace_bytes gives for these
 *    shapes) exceeds PI_SCRATCH_BYTES fail with PI_ERR_WORKSPACE and enqueue
 *    nothing.  The five workload shapes of the library's tests fit.
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents (no call needs it to start at any value).  Calls that may
 *    overlap on one GPU (different streams, or host threads without ordering)
 *    race on it and must be ordered by the caller.
 *  - `stream` must belong to the current device (PI_ERR_ARG otherwise).  The
 *    first call on a device looks up that device's copy of the array.
 */
#define PI_SCRATCH_BYTES (32u << 20)
pi_status pi_sparse_ffn_split_noalloc(const pi_ffn_part* hot, const pi_ffn_part* cold,
                                      const void* x, int32_t B, int32_t xdtype,
                                      const uint64_t* mask, const pi_active_lists* lists,
                                      float* y_hot, float* y_cold, float* y, void* stream);

/*
 * Prompt-phase crossover between the sparse and the dense FFN (CSDN article,
 * section on the speed results: the advantage shrinks from input length 1 to
 * 64, where the batch's union of active neurons covers most of the layer).
 * The same call as pi_sparse_ffn_split, and the lists and counts it writes or
 * reads are the same; but when the step's active count (hot + cold, on the
 * device) is at least dense_from, every row of both partitions is computed
 * instead of the listed ones: y_hot and y_cold are then the dense FFN's two
 * partial outputs and y the dense FFN.  The choice is made on the device from
 * the device counts: no host synchronisation.  dense_from >= 1 (a count no
 * step reaches, e.g. n + 1, keeps the sparse path; 1 always takes the dense
 * one).  Takes the two-kernel paths for every batch (the fused batch-1 kernel
 * does not make the choice).
 */
pi_status pi_sparse_ffn_crossover(const pi_ffn_part* hot, const pi_ffn_part* cold, const void* x,
                                  int32_t B, int32_t xdtype, const uint64_t* mask,
                                  const pi_active_lists* lists, int32_t dense_from, float* y_hot,
                                  float* y_cold, float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * Merge of two partial outputs (CSDN article, hybrid-design figure: the
 * partitions' results are combined on the GPU): y = y_hot + y_cold, [B][d]
 * float32; y_cold NULL means zeros; y may alias y_hot or y_cold.
 */
pi_status pi_merge(const float* y_hot, const float* y_cold, int32_t B, int32_t d, float* y,
                   void* stream);

/*
 * Dense FFN of one partition (every row computed): the measurement baseline
 * the sparse path is compared with (hada.io README summary: dense inference
 * mode).  y [B][d] float32, overwritten.
 */
pi_status pi_dense_ffn(const pi_ffn_part* part, const void* x, int32_t B, int32_t xdtype,
                       float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * Offline activation profiling (CSDN article, overall-architecture section:
 * activations are recorded over a general dataset).  counts [part->rows]
 * uint32, overwritten: number of samples s of X [S][d] whose deciding
 * pre-activation (W_up + b_up for ReLU, W_gate + b_gate for ReGLU) is > 0,
 * decided in float32.
 */
pi_status pi_profile_counts(const pi_ffn_part* part, const void* X, int32_t S, int32_t xdtype,
                            uint32_t* counts, void* stream);

/*
 * Neuron index under a memory budget (CSDN article, overall-architecture
 * section; hada.io README summary, --vram-budget / GPU index):
 *   perm [n] int32 device, out: perm[slot] = original neuron id, slots in
 *        order of (counts desc, id asc);
 *   n_hot [host] out: min(n, floor(budget_bytes / bytes_per_neuron)).
 * counts [n] uint32 device.  The hot partition is slots [0, n_hot).
 */
pi_status pi_build_neuron_index(const uint32_t* counts, int32_t n, int64_t budget_bytes,
                                int64_t bytes_per_neuron, int32_t* perm, int32_t* n_hot,
                                void* stream);

/*
 * Adaptive predictor threshold (chatpaper.ai abstract: adaptive predictors;
 * hada.io README summary, hybrid-approach section: a predictor adapted per
 * layer), chosen offline on profiling samples to reach a recall target.
 * Over the S samples of X [S][d] (xdtype PI_F32 or PI_F16) the call computes
 * on the GPU, in float32 as the decode path does:
 *   logit(s, i)  = the predictor's logit (the kernels of pi_predict, in
 *                  batches of up to PI_MAX_BATCH samples),
 *   firing(s, i) = the deciding pre-activation of neuron i (W_up + b_up, or
 *                  W_gate + b_gate for ReGLU) is > 0,
 * and, with N firing pairs and m = ceil(target_recall * N), returns in *tau
 * (device float) the largest float32 threshold for which at least m firing
 * pairs have logit > tau: the float32 just below the m-th largest logit among
 * the firing pairs (an exact radix selection with integer histograms; FLT_MAX
 * when N == 0).  stats (device uint32 [3]): N, m, and the firing pairs whose
 * logit is > tau (>= m).  Using tau as pi_predictor.threshold gives recall >=
 * target_recall on these samples.  part must be the whole layer (rows == n, same
 * d) in the predictor's neuron order.  target_recall in (0, 1]; S * n <= 2^31.
 * Needs a workspace of pi_calibrate_workspace_bytes(d, n, r, S) bytes.
 */
size_t pi_calibrate_workspace_bytes(int32_t d, int32_t n, int32_t r, int32_t S);
pi_status pi_calibrate_threshold(const pi_predictor* p, const pi_ffn_part* part, const void* X,
                                 int32_t S, int32_t xdtype, double target_recall, float* tau,
                                 uint32_t* stats, void* ws, size_t ws_bytes, void* stream);

/*
 * The true firing set of a batch, for measuring a predictor's recall and
 * precision: bit i % 64 of mask word i / 64 is set iff the deciding
 * pre-activation of neuron i (as in pi_calibrate_threshold) is > 0 for some
 * token of x [B][d] (float32 decision).  mask [ceil(part->rows / 64)] uint64
 * device, 8-byte aligned, overwritten (tail bits 0).  Reads every row of the
 * deciding matrix (a dense pass; measurement only).
 */
pi_status pi_true_mask(const pi_ffn_part* part, const void* x, int32_t B, int32_t xdtype,
                       uint64_t* mask, void* stream);

/*
 * The cold partition computed by the host cores (CSDN article, section on the
 * CPU/GPU hybrid design and its figure; hada.io README summary,
 * hybrid-approach section: the cold neurons stay in host memory and the CPU
 * computes the predicted ones among them while the GPU computes the hot ones;
 * the partial results are merged).
 *
 * pi_host_sparse_ffn: the sparse FFN of one partition on the CPU, every
 * pointer a [host] pointer (part's weights and biases, x, idx, y):
 *   y[b][:] = sum over idx[0 .. count) of h_bi * W_downT[i][:]
 * with h as in pi_ffn_part, accumulated in float32.  x [B][d] PI_F32 or
 * PI_F16; idx int32, ids outside 0..part->rows-1 add nothing; y [B][d]
 * float32, overwritten.  Layouts as for the device calls (Q4_0 rows
 * included); no alignment is required.  The work runs on a pool of host
 * threads the library starts on first use (one per CPU the process may run
 * on, at most 64): `threads` of them (0 = all); each takes a contiguous run of
 * the list and the per-thread partials are added in a fixed order, so the
 * result is reproducible for a given thread count.  Calls are serialised.
 * Synchronous; uses no GPU.  Errors: PI_ERR_ARG / PI_ERR_DTYPE / PI_ERR_SHAPE
 * as for pi_sparse_ffn (B in 1..PI_MAX_BATCH, count >= 0, threads >= 0).
 */
pi_status pi_host_sparse_ffn(const pi_ffn_part* part, const void* x, int32_t B, int32_t xdtype,
                             const int32_t* idx, int32_t count, float* y, int32_t threads);

/* Host-side record of one pi_sparse_ffn_hybrid call. */
typedef struct pi_hybrid_info {
    int32_t cold_count;   /* predicted cold neurons the host computed */
    int32_t threads;      /* host threads used */
    double wait_us;       /* host wait for the mask and x to reach host memory */
    double host_us;       /* host FFN time (list + rows + partial sums) */
} pi_hybrid_info;

/*
 * Bytes of pinned host workspace pi_sparse_ffn_hybrid needs for a layer of n
 * neurons, width d and batches up to B (0 if out of range).
 */
size_t pi_hybrid_host_bytes(int32_t d, int32_t n, int32_t B);

/*
 * One hybrid FFN step: hot partition on the GPU, cold partition on the host
 * cores, at the same time, then merged on the GPU.
 *   hot    partition in device memory (rows may be 0);
 *   cold   partition whose weights and biases are in host memory (rows may
 *          be 0); same d, wdtype and act as hot;
 *   x      [B][d] device (PI_F32 or PI_F16), mask as written by pi_predict for
 *          the n = hot rows + cold rows neurons (device);
 *   lists  device, n_hot == hot->rows: receives the hot list and counts[0] as
 *          pi_sparse_ffn_split writes them (nothing when hot has no rows);
 *          the cold list is formed on the host (cold_idx and counts[1] are not
 *          written);
 *   y_cold [B][d] float32 device, out: the host's partial;
 *   y      [B][d] float32 device, out: hot partial + y_cold;
 *   ws     device workspace as for pi_sparse_ffn_split;
 *   host_ws pinned host memory (hipHostMalloc), 64-byte aligned, of at least
 *          pi_hybrid_host_bytes(d, n, B) bytes;
 *   threads host threads for the cold rows (0 = all of the pool);
 *   info   [host] optional record of the call.
 * Order of work: a kernel on `stream` writes mask and x into host_ws (pinned
 * memory is mapped for the GPU), the hot FFN is enqueued behind it, the host
 * waits for that kernel only, computes the cold rows (pi_host_sparse_ffn)
 * while the GPU runs the hot ones into y, then enqueues the merge kernel, which
 * reads the host's partial from host_ws into y_cold and adds it to y.  Unlike
 * the other calls this one blocks the host until mask and x have arrived and
 * the host part is computed; it returns with the merge enqueued.  The host
 * workspace must not be reused from another stream or thread until this
 * stream has passed the merge; calls from different host threads on different
 * streams (each with its own buffers) may run at the same time, their host
 * parts one after the other.  Not capturable in a HIP graph.  Errors are
 * detected before anything is enqueued (host_ws not pinned and cold weights
 * in device memory included: PI_ERR_ARG).
 */
pi_status pi_sparse_ffn_hybrid(const pi_ffn_part* hot, const pi_ffn_part* cold, const void* x,
                               int32_t B, int32_t xdtype, const uint64_t* mask,
                               const pi_active_lists* lists, float* y_cold, float* y, void* ws,
                               size_t ws_bytes, void* host_ws, size_t host_ws_bytes,
                               int32_t threads, pi_hybrid_info* info, void* stream);

/*
 * Hot/cold split from the tiers' read rates and the capacity budget (CSDN
 * article, overall-architecture section: neurons are placed from their
 * activation frequencies and the hardware's bandwidth and capacity;
 * hybrid-design section: the two partitions compute at the same time and
 * their results are merged).  counts_slot [host] n: activation counts in slot
 * order (the order pi_build_neuron_index gives: counts descending).  For K
 * hot slots the per-step read times of the tiers are taken proportional to
 *   T_hot(K)  = (double)(sum of counts of slots <  K) / hbm_gbps
 *   T_cold(K) = (double)(sum of counts of slots >= K) / link_gbps
 * and, since the tiers overlap, a step costs max(T_hot, T_cold).
 *   n_hot [host] out = min(K*, floor(budget_bytes / bytes_per_neuron), n),
 *   K* = the smallest K in [0, n] minimising max(T_hot(K), T_cold(K)).
 * hbm_gbps / link_gbps: measured read rates of the fast and the slow tier
 * (e.g. pi_stream_read on device memory and on pinned host memory).  Host
 * computation only; nothing is enqueued.  Errors: PI_ERR_SHAPE (n out of
 * 0..2^24), PI_ERR_BUDGET, PI_ERR_ARG (rates not positive and finite, NULL).
 */
pi_status pi_plan_hot_split(const uint32_t* counts_slot, int32_t n, int64_t budget_bytes,
                            int64_t bytes_per_neuron, double hbm_gbps, double link_gbps,
                            int32_t* n_hot);

/*
 * Online activation statistics (hada.io README summary: "recent updates"
 * lists online FFN splitting, and the FAQ rebuilds the GPU index on demand):
 * counts[i] += bit i of mask, for i < n (mask as written by pi_predict, in
 * the current slot order).  Accumulated over decode steps, counts feed
 * pi_build_neuron_index again, so the hot partition follows the predicted
 * activations the layer actually sees.  mask [ceil(n/64)] uint64 device,
 * 8-byte aligned; counts [n] uint32 device, 4-byte aligned, updated in place
 * (each counter by one thread: no atomics, exact).  Errors (NULL pointers,
 * misalignment, n < 1) enqueue nothing.
 */
pi_status pi_accumulate_mask(const uint64_t* mask, int32_t n, uint32_t* counts, void* stream);

/*
 * Applies a neuron index to one per-neuron tensor: dst row s = src row
 * perm[s], rows of row_bytes bytes (row_bytes % 4 == 0), s < rows.  src and
 * dst must not overlap.
 */
pi_status pi_permute_rows(const void* src, void* dst, const int32_t* perm, int32_t rows,
                          int64_t row_bytes, void* stream);

/*
 * Plain device copy of `bytes` bytes (bytes % 16 == 0): the reference
 * kernel whose hardware byte counters calibrate traffic measurements.
 */
pi_status pi_copy(const void* src, void* dst, int64_t bytes, void* stream);

/*
 * Plain read stream of `bytes` bytes of src (bytes % 16 == 0, src 16-byte
 * aligned; device or pinned host memory): the attainable read bandwidth of
 * the memory src lives in, the ceiling the weight-streaming kernels are
 * measured against beside the 8 TB/s HBM peak.  sink [PI_STREAM_SINK_WORDS]
 * uint32 device, out: one xor of the words read per workgroup (their value
 * means nothing; they keep the reads from being optimised away).
 */
#define PI_STREAM_SINK_WORDS 2048
pi_status pi_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* Kernel ids for the timing hooks below. */
enum {
    PI_K_PRED_L1 = 0,     /* predictor first layer */
    PI_K_PRED_L2 = 1,     /* predictor second layer + threshold + union */
    PI_K_COMPACT = 2,     /* mask -> active lists */
    PI_K_UP = 3,          /* gathered-row up/gate + activation */
    PI_K_DOWN = 4,        /* column-scatter down into chunk partials */
    PI_K_MERGE = 5,       /* standalone merge */
    PI_K_PROFILE = 6,
    PI_K_INDEX = 7,
    PI_K_COPY = 8,
    PI_K_REDUCE = 9,      /* partials of y -> y_hot, y_cold, y (fused merge) */
    PI_K_FFN = 10,        /* fused compaction + up/gate + activation + down (batch <= 4) */
    PI_K_ACCUMULATE = 11, /* online activation counts from a mask */
    PI_K_STREAM = 12,     /* plain read stream (attainable bandwidth) */
    PI_K_UP_FINISH = 13,  /* sum of the up kernel's K slices + activation (batch >= 2) */
    PI_K_COUNT = 14
};

/*
 * Timing hooks (measurement only).  After pi_kernel_timer_start(kid, max),
 * the next `max` launches of kernel kid made by this host thread carry HIP
 * start/stop events taken at the kernel's own dispatch and completion.
 * pi_kernel_timer_stop synchronises those events and returns the summed
 * duration in milliseconds and the number of timed launches [host].
 */
pi_status pi_kernel_timer_start(int32_t kid, int32_t max_launches);
pi_status pi_kernel_timer_stop(int32_t kid, float* total_ms, int32_t* launches);
const char* pi_kernel_name(int32_t kid);

const char* pi_status_string(pi_status s);
const char* pi_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PI_H */
