/*
 * oracle.c -- plain, slow CPU reference of the predictor-gated sparse FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library; everything here is written
 * out from the method's definition with scalar loops and double-precision
 * accumulation, in the order the method states its steps.
 *
 * Method (PowerInfer pages):
 *  - CSDN article, section on sparse activation: before serving, a small
 *    per-layer router is trained; at run time it predicts which FFN neurons
 *    an input will activate, and only those neurons are computed.  Neurons
 *    that do not fire contribute nothing to the output.
 *  - CSDN article, section on the CPU/GPU hybrid design and its figure: the
 *    predictor names the active neurons of a layer (e.g. 3, 4, 5); each
 *    memory partition computes the active neurons it holds (GPU: 3 and 5,
 *    CPU: 4) and the two partial results are merged.
 *  - CSDN article, overall architecture section: an offline step profiles
 *    activations on a general dataset and places neurons (frequently active
 *    "hot" ones in the fast memory) under the hardware's capacity.
 *  - hada.io README summary, quantisation section: INT4 weights use Q4_0.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - Predictor: two low-rank layers, u = ReLU(P1^T x), logit = P2^T u + b2,
 *    neuron predicted active iff logit > threshold (strict).  Over a batch the
 *    active set is the union of the tokens' sets.
 *  - Sparse FFN over a list L, per token b:
 *      ReLU : h_i = max(0, W_up[i].x_b + b_up[i])
 *      ReGLU: h_i = max(0, W_gate[i].x_b + b_gate[i]) * (W_up[i].x_b + b_up[i])
 *      Squared ReLU: h_i = max(0, W_up[i].x_b + b_up[i])^2 (the third activation
 *             the hada.io README summary lists as supported, next to ReLU and
 *             ReGLU; deciding pre-activation as for ReLU)
 *      y_b  = sum over i in L (ascending) of h_i * W_downT[i][:]
 *    Missing biases are zero.  No down-projection bias.
 *  - Hot/cold: hot = ids < n_hot of the permuted layer, cold = the rest;
 *    lists hold ascending local ids; y = y_hot + y_cold.
 *  - Neuron index: perm = ids sorted by (activation count desc, id asc);
 *    n_hot = min(n, floor(budget_bytes / bytes_per_neuron)).
 *  - Activation count of neuron i over samples: number of samples whose
 *    deciding pre-activation (W_up row for ReLU, W_gate row for ReGLU, with
 *    bias) is > 0.
 *  - Q4_0 row of d elements (d % 32 == 0): d/2 code bytes then d/32 fp16
 *    scales; code byte 16*j + t (t < 16) holds element 32*j + t in its low
 *    nibble and element 32*j + t + 16 in its high nibble; w = (q - 8) * s_j.
 *
 * Decisions taken from floating point (a predicted bit, an activation count)
 * are also reported in float32 rounding of the fp64 value, the precision the
 * GPU library decides in, for the comparison protocol of the tests.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/*
 * Threads: every routine runs single-threaded unless or_set_threads(k > 1) is
 * called; then the independent outer loops (predictor rows, neurons of a
 * list, output columns, profiled rows) are shared among k OpenMP threads.
 * Each output value is still computed by one thread with the same operations
 * in the same order, so the results are bit-identical for any thread count.
 * (Used to time the oracle on all of a host's cores.)
 */
static int or_nthreads = 1;

void or_set_threads(int k) { or_nthreads = k < 1 ? 1 : k; }
int or_get_threads(void) { return or_nthreads; }

enum { OR_F32 = 0, OR_F16 = 1, OR_Q4_0 = 2 };
enum { OR_RELU = 0, OR_REGLU = 1, OR_SQRELU = 2 };
enum { OR_OK = 0, OR_BAD = 1 };

/* ---- storage decoding ------------------------------------------------ */

/* IEEE 754 binary16 -> double, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double or_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1.0 + (double)f / 1024.0, e - 15);
    return sign ? -v : v;
}

static int64_t or_row_bytes(int wdtype, int64_t d)
{
    switch (wdtype) {
    case OR_F32: return 4 * d;
    case OR_F16: return 2 * d;
    case OR_Q4_0: return d / 2 + d / 16;
    }
    return -1;
}

/* Element k of a Q4_0 row (see the header for the encoding). */
double or_q4_0_element(const uint8_t* row, int64_t d, int64_t k)
{
    int64_t j = k / 32, t = k % 32;
    uint8_t byte = row[16 * j + (t % 16)];
    int q = (t < 16) ? (byte & 0x0f) : (byte >> 4);
    uint16_t sbits;
    memcpy(&sbits, row + d / 2 + 2 * j, 2);
    return (double)(q - 8) * or_half_to_double(sbits);
}

/* Elements [k0, k1) of row `row` of a [rows][d] matrix, decoded to double
 * into out[k0 .. k1). */
static void or_load_row_range(const void* W, int wdtype, int64_t d, int64_t row, int64_t k0,
                              int64_t k1, double* out)
{
    const uint8_t* base = (const uint8_t*)W + row * or_row_bytes(wdtype, d);
    for (int64_t k = k0; k < k1; ++k) {
        if (wdtype == OR_F32) {
            float v;
            memcpy(&v, base + 4 * k, 4);
            out[k] = v;
        } else if (wdtype == OR_F16) {
            uint16_t h;
            memcpy(&h, base + 2 * k, 2);
            out[k] = or_half_to_double(h);
        } else {
            out[k] = or_q4_0_element(base, d, k);
        }
    }
}

/* Row `row` of a [rows][d] matrix, decoded to double. */
void or_load_row(const void* W, int wdtype, int64_t d, int64_t row, double* out)
{
    or_load_row_range(W, wdtype, d, row, 0, d, out);
}

/* Token b of an input matrix x[B][d] stored as f32 or f16. */
static void or_load_x(const void* x, int xdtype, int64_t d, int64_t b, double* out)
{
    or_load_row(x, xdtype, d, b, out);
}

static double or_dot(const double* a, const double* b, int64_t len)
{
    double s = 0.0;
    for (int64_t k = 0; k < len; ++k)
        s += a[k] * b[k];
    return s;
}

/* ---- predictor -------------------------------------------------------- */

/*
 * For each token b of x[B][d]:
 *   u_j      = max(0, sum_k P1t[j][k] * x_b[k])            j < r
 *   logit_i  = sum_j P2t[i][j] * u_j + b2[i]                i < n
 *   m_bi     = logit_i > threshold
 * mask[w] bit (i % 64) of word i / 64 is OR over b of m_bi (tail bits 0).
 * logits (nullable) receives logit_bi in double [B][n].
 * mask32 (nullable) receives the same union decided on float32(logit).
 */
int or_predict(int64_t d, int64_t n, int64_t r, int pdtype, const void* P1t, const void* P2t,
               const float* b2, double threshold, const void* x, int xdtype, int64_t B,
               uint64_t* mask, double* logits, uint64_t* mask32)
{
    if (d <= 0 || n <= 0 || r <= 0 || B <= 0 || (pdtype != OR_F32 && pdtype != OR_F16))
        return OR_BAD;
    int64_t words = (n + 63) / 64;
    double* xb = malloc(sizeof(double) * d);
    double* u = malloc(sizeof(double) * r);
    unsigned char* fire = calloc((size_t)n, 1);     /* bit 0: > threshold, bit 1: in float32 */
    if (!xb || !u || !fire) { free(xb); free(u); free(fire); return OR_BAD; }
    int bad = 0;
    for (int64_t b = 0; b < B; ++b) {
        or_load_x(x, xdtype, d, b, xb);
#pragma omp parallel num_threads(or_nthreads) if (or_nthreads > 1)
        {
            double* row = malloc(sizeof(double) * (d > r ? d : r));
            if (!row) {
#pragma omp atomic write
                bad = 1;
            }
#pragma omp for schedule(static)
            for (int64_t j = 0; j < r; ++j) {
                if (!row) continue;
                or_load_row(P1t, pdtype, d, j, row);
                double a = or_dot(row, xb, d);
                u[j] = a > 0.0 ? a : 0.0;
            }
#pragma omp for schedule(static)
            for (int64_t i = 0; i < n; ++i) {
                if (!row) continue;
                or_load_row(P2t, pdtype, r, i, row);
                double lg = or_dot(row, u, r) + (b2 ? (double)b2[i] : 0.0);
                if (logits) logits[b * n + i] = lg;
                if (lg > threshold) fire[i] |= 1;
                if ((float)lg > (float)threshold) fire[i] |= 2;
            }
            free(row);
        }
    }
    for (int64_t w = 0; w < words; ++w) {
        mask[w] = 0;
        if (mask32) mask32[w] = 0;
    }
    for (int64_t i = 0; i < n; ++i) {
        if (fire[i] & 1) mask[i / 64] |= (uint64_t)1 << (i % 64);
        if (mask32 && (fire[i] & 2)) mask32[i / 64] |= (uint64_t)1 << (i % 64);
    }
    free(xb); free(u); free(fire);
    return bad ? OR_BAD : OR_OK;
}

/* ---- compaction ------------------------------------------------------- */

/*
 * A = ascending ids i < n whose mask bit is set.  Split at n_hot:
 *   hot  = [i for i in A if i <  n_hot]
 *   cold = [i - n_hot for i in A if i >= n_hot]
 * counts[0] = |hot|, counts[1] = |cold|.  cold may be NULL when n_hot == n.
 */
int or_compact(const uint64_t* mask, int64_t n, int64_t n_hot, int32_t* hot, int32_t* cold,
               int32_t* counts)
{
    if (n < 0 || n_hot < 0 || n_hot > n || (!cold && n_hot < n))
        return OR_BAD;
    int32_t nh = 0, nc = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (!((mask[i / 64] >> (i % 64)) & 1))
            continue;
        if (i < n_hot)
            hot[nh++] = (int32_t)i;
        else
            cold[nc++] = (int32_t)(i - n_hot);
    }
    counts[0] = nh;
    counts[1] = nc;
    return OR_OK;
}

/* ---- sparse FFN over a list --------------------------------------------- */

typedef struct {
    int64_t d, rows;
    int wdtype, act;
    const void* W_up;
    const void* W_gate;   /* ReGLU only */
    const float* b_up;    /* nullable */
    const float* b_gate;  /* nullable */
    const void* W_downT;
} or_part;

/*
 * y[b][:] = sum over idx[0..count) (in the order given) of h_bi * W_downT[i][:]
 * with h as in the header.  y is [B][d] double, overwritten.
 */
int or_sparse_ffn(const or_part* p, const void* x, int xdtype, int64_t B, const int32_t* idx,
                  int64_t count, double* y)
{
    int64_t d = p->d;
    if (d <= 0 || B < 0 || count < 0 || (p->act == OR_REGLU && !p->W_gate))
        return OR_BAD;
    for (int64_t t = 0; t < count; ++t)
        if (idx[t] < 0 || idx[t] >= p->rows) return OR_BAD;
    enum { COLS = 256 };                           /* output columns per work item */
    const int64_t nblk = (d + COLS - 1) / COLS;
    double* xb = malloc(sizeof(double) * d);
    double* h = malloc(sizeof(double) * (count > 0 ? count : 1));
    if (!xb || !h) { free(xb); free(h); return OR_BAD; }
    int bad = 0;
    for (int64_t b = 0; b < B; ++b) {
        double* yb = y + b * d;
        or_load_x(x, xdtype, d, b, xb);
#pragma omp parallel num_threads(or_nthreads) if (or_nthreads > 1)
        {
            double* row = malloc(sizeof(double) * d);
            if (!row) {
#pragma omp atomic write
                bad = 1;
            }
            /* h of every listed neuron */
#pragma omp for schedule(static)
            for (int64_t t = 0; t < count; ++t) {
                if (!row) continue;
                int64_t i = idx[t];
                or_load_row(p->W_up, p->wdtype, d, i, row);
                double up = or_dot(row, xb, d) + (p->b_up ? (double)p->b_up[i] : 0.0);
                double hv;
                if (p->act == OR_RELU) {
                    hv = up > 0.0 ? up : 0.0;
                } else if (p->act == OR_SQRELU) {
                    const double r = up > 0.0 ? up : 0.0;
                    hv = r * r;
                } else {
                    or_load_row(p->W_gate, p->wdtype, d, i, row);
                    double g = or_dot(row, xb, d) + (p->b_gate ? (double)p->b_gate[i] : 0.0);
                    hv = (g > 0.0 ? g : 0.0) * up;
                }
                h[t] = hv;
            }
            /* y_b[k] = sum over the list, in its order, of h_i * W_downT[i][k] */
#pragma omp for schedule(static)
            for (int64_t cb = 0; cb < nblk; ++cb) {
                if (!row) continue;
                const int64_t k0 = cb * COLS, k1 = k0 + COLS < d ? k0 + COLS : d;
                for (int64_t k = k0; k < k1; ++k)
                    yb[k] = 0.0;
                for (int64_t t = 0; t < count; ++t) {
                    or_load_row_range(p->W_downT, p->wdtype, d, idx[t], k0, k1, row);
                    for (int64_t k = k0; k < k1; ++k)
                        yb[k] += h[t] * row[k];
                }
            }
            free(row);
        }
    }
    free(xb); free(h);
    return bad ? OR_BAD : OR_OK;
}

/* The dense FFN: the sparse FFN with the list [0, rows). */
int or_dense_ffn(const or_part* p, const void* x, int xdtype, int64_t B, double* y)
{
    int32_t* all = malloc(sizeof(int32_t) * (p->rows > 0 ? p->rows : 1));
    if (!all) return OR_BAD;
    for (int64_t i = 0; i < p->rows; ++i)
        all[i] = (int32_t)i;
    int rc = or_sparse_ffn(p, x, xdtype, B, all, p->rows, y);
    free(all);
    return rc;
}

/* ---- merge ------------------------------------------------------------ */

/* y = y_hot + y_cold elementwise over len values; y_cold NULL means zeros. */
void or_merge(const double* y_hot, const double* y_cold, int64_t len, double* y)
{
    for (int64_t k = 0; k < len; ++k)
        y[k] = y_hot[k] + (y_cold ? y_cold[k] : 0.0);
}

/* ---- offline profiling and neuron index -------------------------------- */

/*
 * counts[i] = number of samples s of X[S][d] with pre_i(x_s) > 0, where pre is
 * the deciding pre-activation (W_up + b_up for ReLU, W_gate + b_gate for ReGLU).
 * counts32 (nullable): the same count decided on float32(pre).
 * amb (nullable): number of samples with |pre| <= band (ambiguous decisions).
 */
int or_profile_counts(const or_part* p, const void* X, int xdtype, int64_t S, uint32_t* counts,
                      uint32_t* counts32, uint32_t* amb, double band)
{
    int64_t d = p->d;
    const void* W = p->act == OR_REGLU ? p->W_gate : p->W_up;
    const float* bias = p->act == OR_REGLU ? p->b_gate : p->b_up;
    if (d <= 0 || S < 0 || !W) return OR_BAD;
    double* xs = malloc(sizeof(double) * d * (S > 0 ? S : 1));
    if (!xs) return OR_BAD;
    for (int64_t s = 0; s < S; ++s)
        or_load_x(X, xdtype, d, s, xs + s * d);
    int bad = 0;
#pragma omp parallel num_threads(or_nthreads) if (or_nthreads > 1)
    {
        double* row = malloc(sizeof(double) * d);
        if (!row) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < p->rows; ++i) {
            if (!row) continue;
            or_load_row(W, p->wdtype, d, i, row);
            double bi = bias ? (double)bias[i] : 0.0;
            uint32_t c = 0, c32 = 0, a = 0;
            for (int64_t s = 0; s < S; ++s) {
                double pre = or_dot(row, xs + s * d, d) + bi;
                c += pre > 0.0;
                c32 += (float)pre > 0.0f;
                a += fabs(pre) <= band;
            }
            counts[i] = c;
            if (counts32) counts32[i] = c32;
            if (amb) amb[i] = a;
        }
        free(row);
    }
    free(xs);
    return bad ? OR_BAD : OR_OK;
}

static const uint32_t* or_sort_counts;

static int or_by_count_desc_id_asc(const void* a, const void* b)
{
    int32_t ia = *(const int32_t*)a, ib = *(const int32_t*)b;
    uint32_t ca = or_sort_counts[ia], cb = or_sort_counts[ib];
    if (ca != cb) return ca > cb ? -1 : 1;
    return (ia > ib) - (ia < ib);
}

/*
 * perm[slot] = original id, slots ordered by (count desc, id asc);
 * n_hot = min(n, floor(budget_bytes / bytes_per_neuron)).
 * Not reentrant (qsort comparator reads a file-scope pointer).
 */
int or_build_neuron_index(const uint32_t* counts, int64_t n, int64_t budget_bytes,
                          int64_t bytes_per_neuron, int32_t* perm, int64_t* n_hot)
{
    if (n < 0 || budget_bytes < 0 || bytes_per_neuron <= 0)
        return OR_BAD;
    for (int64_t i = 0; i < n; ++i)
        perm[i] = (int32_t)i;
    or_sort_counts = counts;
    qsort(perm, (size_t)n, sizeof(int32_t), or_by_count_desc_id_asc);
    or_sort_counts = NULL;
    int64_t k = budget_bytes / bytes_per_neuron;
    *n_hot = k < n ? k : n;
    return OR_OK;
}

/*
 * Hot/cold split from the two tiers' read rates (CSDN article, overall
 * architecture section: neurons are placed from their activation frequencies
 * and the hardware's bandwidth and capacity; hybrid-design section: the two
 * partitions compute at the same time and their results are merged).
 * counts_slot[s] is the activation count of the neuron in slot s (slots in
 * index order, counts descending).  With K hot slots, the expected read time
 * per step of each tier is proportional to
 *   T_hot(K)  = (sum of counts of slots <  K) / hbm_rate
 *   T_cold(K) = (sum of counts of slots >= K) / link_rate
 * (every neuron owns the same bytes, so they cancel).  The tiers run
 * concurrently, so a step takes about max(T_hot, T_cold):
 *   K*    = the smallest K in [0, n] that minimises max(T_hot(K), T_cold(K))
 *   n_hot = min(K*, floor(budget_bytes / bytes_per_neuron), n)
 */
int or_plan_hot_split(const uint32_t* counts_slot, int64_t n, int64_t budget_bytes,
                      int64_t bytes_per_neuron, double hbm_rate, double link_rate, int64_t* n_hot)
{
    if (n < 0 || budget_bytes < 0 || bytes_per_neuron <= 0 || !(hbm_rate > 0.0) ||
        !(link_rate > 0.0))
        return OR_BAD;
    int64_t total = 0;
    for (int64_t s = 0; s < n; ++s)
        total += counts_slot[s];
    int64_t best_k = 0;
    double best = 0.0;
    int64_t hot = 0;                                   /* sum of counts of slots < K */
    for (int64_t K = 0; K <= n; ++K) {
        if (K > 0) hot += counts_slot[K - 1];
        double t_hot = (double)hot / hbm_rate;
        double t_cold = (double)(total - hot) / link_rate;
        double t = t_hot > t_cold ? t_hot : t_cold;
        if (K == 0 || t < best) {
            best = t;
            best_k = K;
        }
    }
    int64_t cap = budget_bytes / bytes_per_neuron;
    int64_t k = best_k < cap ? best_k : cap;
    *n_hot = k < n ? k : n;
    return OR_OK;
}

/*
 * Adaptive predictor threshold (chatpaper.ai abstract: adaptive predictors;
 * hada.io README summary, hybrid-approach section: an adaptive predictor per
 * layer).  Over the S profiling samples of X[S][d]:
 *   firing(s, i) = the deciding pre-activation of neuron i (as in
 *                  or_profile_counts) is > 0,
 *   logit(s, i)  = the predictor's logit (as in or_predict).
 * Both are decided in float32 rounding of the double values, the precision the
 * GPU library computes them in.  With N firing pairs and m = ceil(target * N),
 * the threshold is the largest float32 tau for which at least m firing pairs
 * have logit > tau, i.e. the float32 just below the m-th largest logit among
 * the firing pairs; the recall #{firing, logit > tau} / N is then >= target.
 * N == 0 gives tau = FLT_MAX (nothing fires, nothing need be predicted).
 * Outputs: *tau, stats[0] = N, stats[1] = m, stats[2] = firing pairs with
 * logit > tau.
 */
static int or_cmp_float_desc(const void* a, const void* b)
{
    float fa = *(const float*)a, fb = *(const float*)b;
    return (fa < fb) - (fa > fb);
}

int or_calibrate_threshold(int64_t d, int64_t n, int64_t r, int pdtype, const void* P1t,
                           const void* P2t, const float* b2, const or_part* part, const void* X,
                           int xdtype, int64_t S, double target, float* tau, int64_t* stats)
{
    if (d <= 0 || n <= 0 || S < 0 || part->rows != n || part->d != d || !(target > 0.0) ||
        target > 1.0)
        return OR_BAD;
    const void* W = part->act == OR_REGLU ? part->W_gate : part->W_up;
    const float* bias = part->act == OR_REGLU ? part->b_gate : part->b_up;
    double* logits = malloc(sizeof(double) * (n > 0 ? n : 1));
    double* xs = malloc(sizeof(double) * d);
    signed char* fire = malloc((size_t)n);
    float* fired = malloc(sizeof(float) * (S * n > 0 ? S * n : 1));
    uint64_t* mask = malloc(sizeof(uint64_t) * ((n + 63) / 64));
    if (!logits || !xs || !fire || !fired || !mask) {
        free(logits); free(xs); free(fire); free(fired); free(mask);
        return OR_BAD;
    }
    int64_t N = 0;
    int rc = OR_OK;
    for (int64_t s = 0; s < S && rc == OR_OK; ++s) {
        /* the predictor's logits for sample s */
        const uint8_t* xb = (const uint8_t*)X + s * d * (xdtype == OR_F32 ? 4 : 2);
        rc = or_predict(d, n, r, pdtype, P1t, P2t, b2, 0.0, xb, xdtype, 1, mask, logits, NULL);
        or_load_x(X, xdtype, d, s, xs);
        /* firing decided per neuron (independent), collected in neuron order */
#pragma omp parallel num_threads(or_nthreads) if (or_nthreads > 1)
        {
            double* rw = malloc(sizeof(double) * d);
#pragma omp for schedule(static)
            for (int64_t i = 0; i < n; ++i) {
                if (!rw) { fire[i] = -1; continue; }
                or_load_row(W, part->wdtype, d, i, rw);
                double pre = or_dot(rw, xs, d) + (bias ? (double)bias[i] : 0.0);
                fire[i] = (float)pre > 0.0f;
            }
            free(rw);
        }
        for (int64_t i = 0; i < n; ++i) {
            if (fire[i] < 0) rc = OR_BAD;
            else if (fire[i]) fired[N++] = (float)logits[i];
        }
    }
    if (rc == OR_OK) {
        int64_t m = (int64_t)ceil(target * (double)N);
        if (m < 1 && N > 0) m = 1;
        if (m > N) m = N;
        float t;
        int64_t hits = 0;
        if (N == 0) {
            t = FLT_MAX;
        } else {
            qsort(fired, (size_t)N, sizeof(float), or_cmp_float_desc);
            t = nextafterf(fired[m - 1], -INFINITY);
        }
        for (int64_t k = 0; k < N; ++k)
            hits += fired[k] > t;
        *tau = t;
        stats[0] = N;
        stats[1] = m;
        stats[2] = hits;
    }
    free(logits); free(xs); free(fire); free(fired); free(mask);
    return rc;
}

/* ---- one whole layer step ---------------------------------------------- */

/*
 * The method's steps in order for one batch: predict (union mask), compact
 * into hot/cold lists, sparse FFN on each partition, merge.  hot/cold are the
 * two partitions of the permuted layer (cold may be NULL when n_hot == n).
 * Outputs: mask, hot_idx, cold_idx, counts[2], y[B][d] (double).
 */
int or_layer_step(int64_t d, int64_t n, int64_t r, int pdtype, const void* P1t, const void* P2t,
                  const float* b2, double threshold, const or_part* hot, const or_part* cold,
                  const void* x, int xdtype, int64_t B, uint64_t* mask, int32_t* hot_idx,
                  int32_t* cold_idx, int32_t* counts, double* y)
{
    int64_t n_hot = hot->rows;
    if (or_predict(d, n, r, pdtype, P1t, P2t, b2, threshold, x, xdtype, B, mask, NULL, NULL))
        return OR_BAD;
    if (or_compact(mask, n, n_hot, hot_idx, cold_idx, counts))
        return OR_BAD;
    double* yh = malloc(sizeof(double) * (B * d > 0 ? B * d : 1));
    double* yc = malloc(sizeof(double) * (B * d > 0 ? B * d : 1));
    if (!yh || !yc) { free(yh); free(yc); return OR_BAD; }
    int rc = or_sparse_ffn(hot, x, xdtype, B, hot_idx, counts[0], yh);
    if (!rc && cold)
        rc = or_sparse_ffn(cold, x, xdtype, B, cold_idx, counts[1], yc);
    if (!rc)
        or_merge(yh, cold ? yc : NULL, B * d, y);
    free(yh); free(yc);
    return rc;
}
