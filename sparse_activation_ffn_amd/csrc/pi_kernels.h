// pi_kernels.h -- HIP kernels of the predictor-gated sparse FFN (gfx950).
//
// The kernels here, all on one stream with the active counts kept in device
// memory so the host never waits inside a step:
//   k_pred_l1   u = ReLU(P1t x)                       (dense rows of P1t)
//   k_pred_l2   logit = P2t u + b2, > threshold, OR over tokens -> mask words
//   k_compact   mask -> ascending hot / cold lists + device counts
//   k_up        gathered rows of W_up (and W_gate) -> h per active neuron
//   k_down      gathered rows of W_downT scaled by h, 2-D tiled over
//               (column slice x neuron chunk) -> chunk partials
//   k_reduce    chunk partials summed in a fixed order into y_hot, y_cold
//               and y = y_hot + y_cold (the merge)
// plus the offline index kernels.  A batch-1 step uses k_pred_l1, k_pred_l2,
// then the fused FFN kernel of pi_ffn.h and its partial reduction; batches of
// 2..64 use the matrix-core kernels of pi_mfma.h; k_up / k_down serve the
// remaining shapes.
// No kernel synchronises with another workgroup: kernel boundaries order the
// steps, so no device-scope cache write-back is needed inside a kernel.
// Method: PowerInfer pages -- CSDN article, sections on sparse activation
// (predict, then compute only predicted neurons) and on the hybrid design
// (per-partition computation of the predicted neurons, then a merge).
#pragma once
#include "pi_device.h"

namespace pi {

constexpr int THREADS = 256;          // 4 waves per workgroup for every kernel here
constexpr int NWAVES = THREADS / WAVE;

// ===========================================================================
// Predictor, first layer: u[b][j] = max(0, P1t[j] . x_b).  One workgroup per
// row j; threads stride over the row's 16-byte chunks; token groups of BT.
// ===========================================================================
template <int WT, int XT, int BT>
__global__ __launch_bounds__(THREADS) void k_pred_l1(const uint8_t* __restrict__ P1t,
                                                     const uint8_t* __restrict__ x, int d, int r,
                                                     int B, float* __restrict__ u) {
    constexpr int EPC = Chunk<WT>::EPC;
    constexpr int XB = XT == F32 ? 4 : 2;
    __shared__ float red[NWAVES][BT];
    const int j = blockIdx.x;
    const int nch = d / EPC;
    const uint8_t* row = P1t + (int64_t)j * row_bytes(WT, d);
    const int lane = threadIdx.x & (WAVE - 1), wv = threadIdx.x / WAVE;
    for (int b0 = 0; b0 < B; b0 += BT) {
        float acc[BT];
#pragma unroll
        for (int b = 0; b < BT; ++b) acc[b] = 0.0f;
        constexpr int U = 4;                    // chunks in flight per thread
        for (int c0 = threadIdx.x; c0 < nch; c0 += THREADS * U) {
            // branch-free: every weight and x load is issued (clamped addresses)
            // before the first product waits, and a chunk or token past the end
            // is dropped by a select after its product, keeping the summation
            // order of the valid chunks
            u4 w[U];
#pragma unroll
            for (int q = 0; q < U; ++q) w[q] = ld16_stream(row + 16 * (int64_t)min(c0 + THREADS * q, nch - 1));
#pragma unroll
            for (int q = 0; q < U; ++q) {
                const int c = min(c0 + THREADS * q, nch - 1);
                const bool cv = c0 + THREADS * q < nch;
#pragma unroll
                for (int b = 0; b < BT; ++b) {
                    const float t = Dot<WT, XT>::run(
                        w[q], 0.0f, x + ((int64_t)min(b0 + b, B - 1) * d + c * EPC) * XB, acc[b]);
                    acc[b] = cv && b0 + b < B ? t : acc[b];
                }
            }
        }
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            float v = wave_sum(acc[b]);
            if (lane == 0) red[wv][b] = v;
        }
        __syncthreads();
        if (threadIdx.x < BT && b0 + (int)threadIdx.x < B) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) s += red[w][threadIdx.x];
            u[(int64_t)(b0 + threadIdx.x) * r + j] = s > 0.0f ? s : 0.0f;
        }
        __syncthreads();
    }
}

// ===========================================================================
// Compaction of mask words into ascending hot / cold lists, by one workgroup.
// Thread t owns a contiguous run of words, so an exclusive scan of per-thread
// popcounts gives each set bit its position in the ascending list.
// ===========================================================================
struct Lists {
    int32_t n_hot;
    int32_t* hot;
    int32_t* cold;
    int32_t* counts;
};

__device__ void compact_block(const uint64_t* mask, int n, Lists L) {
    __shared__ int s_tot[THREADS];
    __shared__ int s_hot[THREADS];
    const int words = (n + 63) / 64;
    const int per = (words + THREADS - 1) / THREADS;
    const int w0 = threadIdx.x * per, w1 = min(words, w0 + per);
    // bits at or beyond n are ignored, so lists never exceed their capacities
    const uint64_t tail = (n % 64) ? ((1ull << (n % 64)) - 1ull) : ~0ull;
    int tot = 0, hot = 0;
    for (int w = w0; w < w1; ++w) {
        uint64_t v = mask[w];
        if (w == words - 1) v &= tail;
        tot += __popcll(v);
        int lo = 64 * w;
        if (lo + 64 <= L.n_hot) hot += __popcll(v);
        else if (lo < L.n_hot) hot += __popcll(v & ((1ull << (L.n_hot - lo)) - 1ull));
    }
    s_tot[threadIdx.x] = tot;
    s_hot[threadIdx.x] = hot;
    __syncthreads();
    // inclusive scan of totals (Hillis-Steele) and a sum of hot counts
    for (int o = 1; o < THREADS; o <<= 1) {
        int a = threadIdx.x >= o ? s_tot[threadIdx.x - o] : 0;
        int h = threadIdx.x >= o ? s_hot[threadIdx.x - o] : 0;
        __syncthreads();
        s_tot[threadIdx.x] += a;
        s_hot[threadIdx.x] += h;
        __syncthreads();
    }
    const int H = s_hot[THREADS - 1];
    const int T = s_tot[THREADS - 1];
    int pos = s_tot[threadIdx.x] - tot;
    for (int w = w0; w < w1; ++w) {
        uint64_t v = mask[w];
        if (w == words - 1) v &= tail;
        while (v) {
            int bit = __builtin_ctzll(v);
            v &= v - 1;
            int id = 64 * w + bit;
            if (id < L.n_hot) L.hot[pos] = id;
            else L.cold[pos - H] = id - L.n_hot;
            ++pos;
        }
    }
    if (threadIdx.x == 0) {
        L.counts[0] = H;
        L.counts[1] = T - H;
    }
}

__global__ __launch_bounds__(THREADS) void k_compact(const uint64_t* __restrict__ mask, int n,
                                                     Lists L) {
    compact_block(mask, n, L);
}

// ===========================================================================
// Predictor, second layer + threshold + union over tokens.  One workgroup per
// 16 neurons, i.e. one 16-bit quarter of a mask word: small workgroups spread
// the P2t rows evenly over the compute units whatever n is.  Each wave owns 4
// rows and 16 lanes share a row (256 contiguous bytes per row per load).  A
// row's first batch of loads is issued before u is staged in LDS, so the u
// round trip overlaps the weight stream.  The workgroup writes its 16 mask bits
// with one 16-bit store; the grid covers every quarter of every word, so the
// tail bits past n are written as zeros.
// ===========================================================================
constexpr int L2_ROWS = 16;           // neurons per workgroup of k_pred_l2

template <int WT, int BT>
__global__ __launch_bounds__(THREADS) void k_pred_l2(const uint8_t* __restrict__ P2t,
                                                     const float* __restrict__ b2, float thr,
                                                     const float* __restrict__ u, int n, int r,
                                                     int B, uint16_t* __restrict__ mask16,
                                                     float* __restrict__ logits) {
    constexpr int EPC = Chunk<WT>::EPC;
    constexpr int G = 16;                       // lanes per row
    constexpr int U = 8;                        // chunks in flight per lane (a 2 KiB row at once)
    extern __shared__ float s_u[];              // [BT][r]
    __shared__ unsigned s_flag[L2_ROWS];
    const int lane = threadIdx.x & (WAVE - 1), wv = threadIdx.x / WAVE;
    const int gi = lane / G, li = lane % G;
    const int nch = r / EPC;
    const int loc = 4 * wv + gi;                // neuron within the workgroup
    const int i = L2_ROWS * blockIdx.x + loc;
    const bool live = i < n;
    const uint8_t* row = P2t + (int64_t)(live ? i : 0) * row_bytes(WT, r);
    const float bias = (live && b2) ? b2[i] : 0.0f;
    unsigned fire = 0;
    for (int b0 = 0; b0 < B; b0 += BT) {
        const int nb = min(BT, B - b0);
        u4 w[U];
#pragma unroll
        for (int q = 0; q < U; ++q)
            if (live && li + G * q < nch) w[q] = ld16_stream(row + 16 * (int64_t)(li + G * q));
        __syncthreads();                        // the previous group's reads of s_u are done
        for (int k = threadIdx.x; k < nb * r; k += THREADS) s_u[k] = u[(int64_t)b0 * r + k];
        for (int k = nb * r + threadIdx.x; k < BT * r; k += THREADS) s_u[k] = 0.0f;
        __syncthreads();
        float acc[BT];
#pragma unroll
        for (int b = 0; b < BT; ++b) acc[b] = 0.0f;
        if (live) {
            for (int c0 = li;;) {
#pragma unroll
                for (int q = 0; q < U; ++q) {
                    const int c = c0 + G * q;
                    if (c < nch) {
#pragma unroll
                        for (int b = 0; b < BT; ++b)
                            acc[b] = Dot<WT, F32>::run(w[q], 0.0f, s_u + b * r + c * EPC, acc[b]);
                    }
                }
                c0 += G * U;
                if (c0 >= nch) break;
#pragma unroll
                for (int q = 0; q < U; ++q)
                    if (c0 + G * q < nch) w[q] = ld16_stream(row + 16 * (int64_t)(c0 + G * q));
            }
        }
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            const float lg = group_sum<G>(acc[b]) + bias;
            if (b < nb) {
                fire |= lg > thr;
                if (logits && li == 0 && live) logits[(int64_t)(b0 + b) * n + i] = lg;
            }
        }
    }
    if (li == 0) s_flag[loc] = live ? fire : 0u;
    __syncthreads();
    if (wv == 0) {
        const uint64_t bits = __ballot(lane < L2_ROWS && s_flag[lane & (L2_ROWS - 1)] != 0);
        if (lane == 0) mask16[blockIdx.x] = (uint16_t)(bits & 0xffffu);
    }
}

// ===========================================================================
// Gathered rows of the FFN.  Work items are the active neurons of both
// partitions: items [0, H) are hot_idx[0..H), items [H, H+C) cold_idx[0..C).
// In dense mode (no lists) item k is row k of partition 0.
// ===========================================================================
struct FfnArgs {
    const uint8_t* up[2];
    const uint8_t* gate[2];
    const float* bup[2];
    const float* bgate[2];
    const uint8_t* down[2];
    const int32_t* idx[2];
    const int32_t* counts;   // device [nparts] active counts (NULL in dense mode)
    int nparts;              // 1 (no cold partition) or 2
    int rows[2];             // rows of each partition (list capacity and id bound)
    int dense_rows;          // dense mode: rows of partition 0
    int d;
    int B;
    int64_t rb;              // row bytes
    const uint8_t* x;        // [B][d]
    float* h;                // [B][h_ld] per item
    int h_ld;
    // mask mode (k_up only): the active set comes from mask words over the
    // n = rows[0] + rows[1] neurons (hot ids < rows[0]); k_up compacts it and
    // writes the lists and counts that k_down then reads through idx/counts
    const uint64_t* mask;
    int n;
    int32_t* out_idx[2];
    int32_t* out_counts;
    // > 0: when the step's active count (the device counts) reaches dense_from,
    // every row of both partitions is computed instead of the listed ones (the
    // prompt-phase crossover to the dense FFN); the lists and counts still
    // describe the predicted set
    int dense_from;
    // matrix-core up kernel split over K (ksplit > 1): slice k of every tile
    // writes its fp32 pre-activations (bias added by slice 0) to
    // upart[((k NM + g) B + token) upart_ld + item]; up_ht receives H and the
    // item count T, and k_up_finish sums the slices and applies the activation
    int ksplit;
    float* upart;
    int upart_ld;
    int* up_ht;
};

// Largest mask (in 64-bit words) whose compaction k_up does in LDS.
constexpr int MASK_WORDS_MAX = 4096;

// Position of the j-th set bit (0-based) of v; v has more than j set bits.
__device__ __forceinline__ int select_bit(uint64_t v, int j) {
    int pos = 0;
#pragma unroll
    for (int w = 32; w > 0; w >>= 1) {
        const int c = __popcll(v & ((1ull << w) - 1ull));
        if (j >= c) {
            j -= c;
            v >>= w;
            pos += w;
        }
    }
    return pos;
}

// Exclusive prefix of the mask words' popcounts into s_scan[0..words] (s_scan[words]
// = total), with the words copied to s_words; bits at or beyond n are cleared.
// NT = threads of the calling workgroup.
template <int NT>
__device__ void scan_mask(const uint64_t* mask, int n, uint64_t* s_words, int* s_scan) {
    __shared__ int s_part[NT];
    const int words = (n + 63) / 64;
    const int per = (words + NT - 1) / NT;
    const int w0 = min(words, (int)threadIdx.x * per), w1 = min(words, w0 + per);
    const uint64_t tail = (n % 64) ? ((1ull << (n % 64)) - 1ull) : ~0ull;
    int tot = 0;
    for (int w = w0; w < w1; ++w) {
        uint64_t v = mask[w];
        if (w == words - 1) v &= tail;
        s_words[w] = v;
        tot += __popcll(v);
    }
    // inclusive scan of the per-thread totals: within each wave by DPP, then
    // across the NT / 64 wave totals
    const int lane = threadIdx.x & (WAVE - 1), wv = threadIdx.x / WAVE;
    const int inc = wave_incl_scan(tot);
    if (lane == WAVE - 1) s_part[wv] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int k = 0; k < NT / WAVE; ++k) {
            const int t = s_part[k];
            s_part[k] = acc;                 // exclusive prefix of the wave totals
            acc += t;
        }
        s_scan[words] = acc;
    }
    __syncthreads();
    int run = s_part[wv] + inc - tot;
    for (int w = w0; w < w1; ++w) {
        s_scan[w] = run;
        run += __popcll(s_words[w]);
    }
    __syncthreads();
}

// Neuron id of the k-th set bit (ascending) of the scanned mask.
__device__ __forceinline__ int kth_active(const uint64_t* s_words, const int* s_scan, int words,
                                          int k) {
    int lo = 0, hi = words - 1;          // largest w with s_scan[w] <= k
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_scan[mid] <= k) lo = mid;
        else hi = mid - 1;
    }
    return 64 * lo + select_bit(s_words[lo], k - s_scan[lo]);
}

// An argument of the partition `part` (0 hot, 1 cold) when part varies across
// lanes: a select between the two values, which come from the argument segment
// through scalar loads.  Indexing the argument's array with a per-lane index
// instead loads the element with a vector load and waits for it at each use
// (in the matrix-core up kernel's list emission, one memory round trip per
// emitted entry).
// (pointers pass through readfirstlane, a register value: a plain select of the
// two loaded pointers is folded back by the compiler into a load of the
// selected argument address)
template <typename T>
__device__ __forceinline__ T* scalar_ptr(T* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    // through a global-address-space pointer, so accesses stay global (not flat)
    typedef __attribute__((address_space(1))) T GT;
    return (T*)reinterpret_cast<GT*>(((uint64_t)hi << 32) | lo);
}
template <typename T>
__device__ __forceinline__ T* by_part(T* const (&v)[2], int part) {
    T* const p0 = scalar_ptr(v[0]);
    T* const p1 = scalar_ptr(v[1]);
    return part == 0 ? p0 : p1;
}
__device__ __forceinline__ int by_part(const int (&v)[2], int part) {
    return part == 0 ? v[0] : v[1];
}

// Whether a predicted set of T active neurons is computed densely (every row).
__device__ __forceinline__ bool crosses_to_dense(const FfnArgs& a, int T) {
    return a.dense_from > 0 && T >= a.dense_from;
}

// Items of the call: H hot, C cold.  Returns true when item k is row k of its
// partition (dense mode, or the active count reached dense_from), false when
// items are list entries.
__device__ __forceinline__ bool item_counts(const FfnArgs& a, int& H, int& C) {
    if (a.counts) {
        // counts beyond the lists' capacities are clamped (never read past a list)
        H = min(max(a.counts[0], 0), a.rows[0]);
        C = a.nparts > 1 ? min(max(a.counts[1], 0), a.rows[1]) : 0;
        if (!crosses_to_dense(a, H + C)) return false;
        H = a.rows[0];
        C = a.nparts > 1 ? a.rows[1] : 0;
        return true;
    }
    H = a.dense_rows;
    C = 0;
    return true;
}

__device__ __forceinline__ void item_row(const FfnArgs& a, int item, int H, bool dense, int& part,
                                         int& row) {
    if (item < H) {
        part = 0;
        row = dense ? item : a.idx[0][item];
    } else {
        part = 1;
        row = dense ? item - H : a.idx[1][item - H];
    }
}

// Up/gate: one wave per item; lanes stride over the row's 16-byte chunks with U
// chunks in flight per lane; the wave reduces; lane 0 applies bias and
// activation.  x is staged in LDS when BT*d fits (XLDS), so x reads do not
// queue behind the weight stream; item and row ids are wave-uniform (scalar).
// Batches are branch-free: chunks past the row end are clamped and dropped.
template <int WT, int XT, int BT, int ACT, bool XLDS>
__global__ __launch_bounds__(THREADS) void k_up(FfnArgs a) {
    constexpr int EPC = Chunk<WT>::EPC;
    constexpr int XB = XT == F32 ? 4 : 2;
    constexpr int U = WT == Q4 ? 4 : 8;
    // dynamic LDS: [x for BT tokens, when XLDS] [mask words] [their popcount scan]
    extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];
    uint8_t* s_x = s_dyn;
    const int64_t xrow = (int64_t)a.d * XB;
    const int words = a.mask ? (a.n + 63) / 64 : 0;
    uint64_t* s_words = reinterpret_cast<uint64_t*>(s_dyn + (XLDS ? BT * xrow : 0));
    int* s_scan = reinterpret_cast<int*>(s_words + words);
    const int lane = threadIdx.x & (WAVE - 1);
    const int gw = __builtin_amdgcn_readfirstlane((blockIdx.x * THREADS + threadIdx.x) / WAVE);
    const int nw = gridDim.x * NWAVES;
    int H, C, Hm = 0;                         // Hm: hot count of the mask (dense crossover)
    bool dense = false;
    if (a.mask) {
        // compaction fused here: every workgroup scans the (small) mask in LDS and
        // maps item k to the k-th active id; hot ids (< rows[0]) come first
        scan_mask<THREADS>(a.mask, a.n, s_words, s_scan);
        const int T = s_scan[words], nh = a.rows[0];
        if (nh >= a.n) {
            H = T;
        } else {
            const int wh = nh / 64;
            H = s_scan[wh] + __popcll(s_words[wh] & ((1ull << (nh % 64)) - 1ull));
        }
        C = T - H;
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            a.out_counts[0] = H;
            a.out_counts[1] = C;
        }
        if (crosses_to_dense(a, T)) {        // the lists are still written below
            dense = true;
            Hm = H;
            H = a.rows[0];
            C = a.rows[1];
        }
    } else {
        dense = item_counts(a, H, C);
    }
    const int T = H + C;
    const int nch = a.d / EPC;
    for (int b0 = 0; b0 < a.B; b0 += BT) {
        const int nb = min(BT, a.B - b0);
        if (XLDS) {
            __syncthreads();
            const u4* src = reinterpret_cast<const u4*>(a.x + b0 * xrow);
            u4* dst = reinterpret_cast<u4*>(s_x);
            const int n16 = (int)(nb * xrow / 16), all16 = (int)(BT * xrow / 16);
            for (int k = threadIdx.x; k < all16; k += THREADS)
                dst[k] = k < n16 ? src[k] : u4{0u, 0u, 0u, 0u};
            __syncthreads();
        }
        const uint8_t* xg = XLDS ? s_x : a.x + b0 * xrow;
        if (a.mask && dense && b0 == 0) {
            // dense crossover: the items are all rows; the lists still name the
            // predicted set (item k of the mask's ascending order)
            const int Tm = s_scan[words];
            for (int k = gw; k < Tm; k += nw) {
                const int id = kth_active(s_words, s_scan, words, k);
                if (lane == 0) {
                    if (k < Hm) a.out_idx[0][k] = id;
                    else a.out_idx[1][k - Hm] = id - a.rows[0];
                }
            }
        }
        for (int item = gw; item < T; item += nw) {
            int part, row;
            if (a.mask && !dense) {
                const int id = kth_active(s_words, s_scan, words, item);
                part = id < a.rows[0] ? 0 : 1;
                row = part == 0 ? id : id - a.rows[0];
                if (lane == 0 && b0 == 0) by_part(a.out_idx, part)[part == 0 ? item : item - H] = row;
            } else {
                item_row(a, item, H, dense, part, row);
            }
            if ((unsigned)row >= (unsigned)by_part(a.rows, part)) {     // id outside the partition: h = 0
                if (lane == 0)
                    for (int b = 0; b < nb; ++b) a.h[(int64_t)(b0 + b) * a.h_ld + item] = 0.0f;
                continue;
            }
            const uint8_t* wu = by_part(a.up, part) + (int64_t)row * a.rb;
            const uint8_t* wg = ACT == REGLU ? by_part(a.gate, part) + (int64_t)row * a.rb : nullptr;
            float au[BT], ag[BT];
#pragma unroll
            for (int b = 0; b < BT; ++b) au[b] = ag[b] = 0.0f;
            for (int c0 = lane; c0 < nch; c0 += WAVE * U) {
                u4 vu[U], vg[U];
                float su[U], sg[U];
                int cq[U];
#pragma unroll
                for (int q = 0; q < U; ++q) cq[q] = min(c0 + WAVE * q, nch - 1);
#pragma unroll
                for (int q = 0; q < U; ++q) {
                    vu[q] = ld16_stream(wu + 16 * (int64_t)cq[q]);
                    if (ACT == REGLU) vg[q] = ld16_stream(wg + 16 * (int64_t)cq[q]);
                }
#pragma unroll
                for (int q = 0; q < U; ++q) {
                    su[q] = WT == Q4 ? half_f(*(const uint16_t*)(wu + a.d / 2 + 2 * cq[q])) : 0.f;
                    if (ACT == REGLU)
                        sg[q] = WT == Q4 ? half_f(*(const uint16_t*)(wg + a.d / 2 + 2 * cq[q])) : 0.f;
                }
#pragma unroll
                for (int q = 0; q < U; ++q) {
                    const bool valid = c0 + WAVE * q < nch;
#pragma unroll
                    for (int b = 0; b < BT; ++b) {
                        // token slots past B read token nb-1 (in bounds) and are dropped
                        const uint8_t* xp = xg + (b < nb ? b : nb - 1) * xrow +
                                            (int64_t)cq[q] * EPC * XB;
                        const float tu = Dot<WT, XT>::run(vu[q], su[q], xp, 0.0f);
                        au[b] += valid ? tu : 0.0f;
                        if (ACT == REGLU) {
                            const float tg = Dot<WT, XT>::run(vg[q], sg[q], xp, 0.0f);
                            ag[b] += valid ? tg : 0.0f;
                        }
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < BT; ++b) {
                float up = wave_sum(au[b]);
                float g = ACT == REGLU ? wave_sum(ag[b]) : 0.0f;
                if (lane == 0 && b < nb) {
                    const float* pbu = by_part(a.bup, part);
                    up += pbu ? pbu[row] : 0.0f;
                    float hv;
                    if (ACT == RELU) {
                        hv = up > 0.0f ? up : 0.0f;
                    } else if (ACT == SQRELU) {
                        const float r = up > 0.0f ? up : 0.0f;
                        hv = r * r;
                    } else {
                        const float* pbg = by_part(a.bgate, part);
                        g += pbg ? pbg[row] : 0.0f;
                        hv = (g > 0.0f ? g : 0.0f) * up;
                    }
                    a.h[(int64_t)(b0 + b) * a.h_ld + item] = hv;
                }
            }
        }
    }
}

// Down: grid (column slices, neuron chunks).  Chunks are split between the
// partitions in proportion to their active counts so no chunk mixes them.
// Each wave walks the chunk's items with stride NWAVES, U rows in flight; the
// four waves reduce through LDS; the chunk writes its partial; k_reduce then
// sums the partials in chunk order into y_hot / y_cold / y.
struct DownOut {
    float* partials;    // [nch][B][d]
    float* y_part[2];   // [B][d] or NULL
    float* y;           // [B][d] or NULL
    int nch;
};

// floor((a * b + e) / c) for a, b, e >= 0 and c > 0: 32-bit division when the
// numerator fits (the usual case; a 64-bit division is a long instruction
// sequence on the GPU), else 64-bit
__device__ __forceinline__ int muldiv(int a, int b, int e, int c) {
    const uint64_t p = (uint64_t)(uint32_t)a * (uint32_t)b + (uint32_t)e;
    if ((p >> 32) == 0) return (int)((uint32_t)p / (uint32_t)c);
    return (int)(p / (uint32_t)c);
}

__device__ __forceinline__ void chunk_range(int nch, int H, int C, int k, int& part, int& lo,
                                            int& hi, int& nh) {
    const int T = H + C;
    if (C == 0) nh = nch;
    else if (H == 0) nh = 0;
    else nh = min(nch - 1, max(1, muldiv(nch, H, T / 2, T)));
    if (k < nh) {
        part = 0;
        lo = muldiv(k, H, 0, nh);
        hi = muldiv(k + 1, H, 0, nh);
    } else {
        const int kk = k - nh, nc = nch - nh;
        part = 1;
        lo = muldiv(kk, C, 0, nc);
        hi = muldiv(kk + 1, C, 0, nc);
    }
}

template <int WT, int BT>
__global__ __launch_bounds__(THREADS) void k_down(FfnArgs a, DownOut o) {
    using D = Down<WT>;
    constexpr int DCH = D::DCH;
    constexpr int U = 8;              // rows in flight per wave
    constexpr int STAGE = 256;        // rows whose ids and h are staged in LDS at a time
    __shared__ float s_red[NWAVES - 1][DCH][WAVE];
    __shared__ int s_row[STAGE];
    __shared__ float s_h[BT][STAGE];
    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    const int slice = blockIdx.x, k = blockIdx.y;
    // this lane's first column: lanes cover D::COLS consecutive columns
    const int lane_col = WT == Q4 ? 32 * (lane >> 1) + 8 * (lane & 1) : lane * DCH;
    const int col0 = slice * D::COLS + lane_col;
    const bool active_col = col0 < a.d;
    const int colL = active_col ? col0 : 0;   // lanes past d read column 0, drop the result
    int H, C;
    const bool dense = item_counts(a, H, C);
    int part, lo, hi, nh;
    chunk_range(o.nch, H, C, k, part, lo, hi, nh);
    const int hbase = part == 0 ? 0 : H;
    const uint8_t* base = part == 0 ? a.down[0] : a.down[1];
    const int32_t* idx = dense ? nullptr : part == 0 ? a.idx[0] : a.idx[1];
    const int prow_max = part == 0 ? a.rows[0] : a.rows[1];
    const int B = a.B;
    for (int b0 = 0; b0 < B; b0 += BT) {
        float acc[BT][DCH];
#pragma unroll
        for (int b = 0; b < BT; ++b)
#pragma unroll
            for (int e = 0; e < DCH; ++e) acc[b][e] = 0.0f;
        for (int s0 = lo; s0 < hi; s0 += STAGE) {
            const int len = min(STAGE, hi - s0);
            __syncthreads();                  // the previous stage is consumed
            for (int t = threadIdx.x; t < len; t += THREADS) {
                const int row = idx ? idx[s0 + t] : s0 + t;
                // an id outside the partition (k_up gave it h = 0) is not read at all
                s_row[t] = (unsigned)row < (unsigned)prow_max ? row : -1;
#pragma unroll
                for (int b = 0; b < BT; ++b)
                    s_h[b][t] = b0 + b < B ? a.h[(int64_t)(b0 + b) * a.h_ld + hbase + s0 + t] : 0.f;
            }
            __syncthreads();
            // ids come from LDS and the batch is branch-free (rows past the stage are
            // clamped and weighted by 0), so the U weight loads issue back to back
            for (int t0 = wv; t0 < len; t0 += NWAVES * U) {
                typename D::raw w[U];
                int tq[U];
#pragma unroll
                for (int q = 0; q < U; ++q) tq[q] = min(t0 + NWAVES * q, len - 1);
#pragma unroll
                for (int q = 0; q < U; ++q) {
                    const int row = __builtin_amdgcn_readfirstlane(s_row[tq[q]]);
                    w[q] = D::load(base + (int64_t)max(row, 0) * a.rb, a.d, colL);
                }
#pragma unroll
                for (int q = 0; q < U; ++q) {
                    // slots past the stage and ids that are not rows take zero weights
                    // (replaced here, where they are consumed), so only listed rows
                    // of the partition contribute, and a non-finite value in any
                    // other row never reaches y
                    const bool valid = t0 + NWAVES * q < len && s_row[tq[q]] >= 0;
                    const typename D::raw wq = valid ? w[q] : D::zero();
#pragma unroll
                    for (int b = 0; b < BT; ++b) D::axpy(wq, valid ? s_h[b][tq[q]] : 0.0f, acc[b]);
                }
            }
        }
        // reduce the four waves' accumulators, one token at a time through LDS
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            if (b0 + b < B) {                       // uniform across the workgroup
                if (wv > 0) {
#pragma unroll
                    for (int e = 0; e < DCH; ++e) s_red[wv - 1][e][lane] = acc[b][e];
                }
                __syncthreads();
                if (wv == 0 && active_col) {
                    float* prow = o.partials + ((int64_t)k * B + b0 + b) * a.d + col0;
#pragma unroll
                    for (int e = 0; e < DCH; ++e) {
                        float s = acc[b][e];
#pragma unroll
                        for (int w = 1; w < NWAVES; ++w) s += s_red[w - 1][e][lane];
                        prow[D::col(e)] = s;
                    }
                }
                __syncthreads();
            }
        }
    }
}

// Reduction of the chunk partials, one thread per 4 consecutive outputs: the
// hot chunks in order give y_hot, the cold chunks in order give y_cold, and
// y = y_hot + y_cold is the merge.  Deterministic (fixed order, no atomics).
__global__ __launch_bounds__(THREADS) void k_reduce(FfnArgs a, DownOut o) {
    const int64_t len = (int64_t)a.B * a.d;           // a multiple of 4 (d % 64 == 0)
    const int64_t len4 = len / 4;
    const int64_t stride = (int64_t)gridDim.x * THREADS;
    const f4* P = reinterpret_cast<const f4*>(o.partials);
    constexpr int R = 8;       // partial loads in flight per thread (branch-free batches)
    f4 v[R];
    auto load = [&](int64_t at, int k0) {
        const int64_t ac = at < len4 ? at : len4 - 1;
#pragma unroll
        for (int q = 0; q < R; ++q) v[q] = P[min(k0 + q, o.nch - 1) * len4 + ac];
    };
    // the first partials are loaded before the item counts, which they do not
    // depend on (the counts take dependent loads and a division)
    const int64_t at0 = (int64_t)blockIdx.x * THREADS + threadIdx.x;
    load(at0, 0);
    int H, C;
    item_counts(a, H, C);
    int part, lo, hi, nh;
    chunk_range(o.nch, H, C, 0, part, lo, hi, nh);
    for (int64_t at = at0; at < len4; at += stride) {
        f4 yh = {0.f, 0.f, 0.f, 0.f}, yc = {0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0;;) {
#pragma unroll
            for (int q = 0; q < R; ++q) {
                const int kk = k0 + q;
                if (kk < nh) {
                    yh.x += v[q].x; yh.y += v[q].y; yh.z += v[q].z; yh.w += v[q].w;
                } else if (kk < o.nch) {
                    yc.x += v[q].x; yc.y += v[q].y; yc.z += v[q].z; yc.w += v[q].w;
                }
            }
            k0 += R;
            if (k0 >= o.nch) break;
            load(at, k0);
        }
        if (at + stride < len4) load(at + stride, 0);
        if (o.y_part[0]) reinterpret_cast<f4*>(o.y_part[0])[at] = yh;
        if (o.y_part[1]) reinterpret_cast<f4*>(o.y_part[1])[at] = yc;
        if (o.y) reinterpret_cast<f4*>(o.y)[at] = f4{yh.x + yc.x, yh.y + yc.y, yh.z + yc.z, yh.w + yc.w};
    }
}

// ===========================================================================
// Merge of two partial outputs: y = a + b (b may be NULL).
// ===========================================================================
__global__ __launch_bounds__(THREADS) void k_merge(const float* __restrict__ a,
                                                   const float* __restrict__ b, int64_t len,
                                                   float* __restrict__ y) {
    const int64_t stride = (int64_t)gridDim.x * THREADS;
    for (int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x; i < len; i += stride)
        y[i] = b ? a[i] + b[i] : a[i];
}

// ===========================================================================
// Hybrid step, the two ends of the host's share.
// k_export: the predicted mask words and x, written straight into the host
// workspace (pinned host memory) for the host cores to read.
// k_merge_host: the host's partial of y, read straight from pinned host
// memory: y_cold = host partial, y = (y_hot or 0) + host partial.  len and the
// x bytes are multiples of 16 bytes (d % 64 == 0).
// ===========================================================================
__global__ __launch_bounds__(THREADS) void k_export(const uint64_t* __restrict__ mask, int words,
                                                    const uint4* __restrict__ x, int x16,
                                                    uint64_t* __restrict__ mask_out,
                                                    uint4* __restrict__ x_out) {
    const int i = blockIdx.x * THREADS + threadIdx.x;
    if (i < words) mask_out[i] = mask[i];
    if (i < x16) x_out[i] = x[i];
}

__global__ __launch_bounds__(THREADS) void k_merge_host(const float4* __restrict__ host_part,
                                                        int64_t len4, bool has_hot,
                                                        float4* __restrict__ y_cold,
                                                        float4* __restrict__ y) {
    const int64_t stride = (int64_t)gridDim.x * THREADS;
    for (int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x; i < len4; i += stride) {
        const float4 c = host_part[i];
        y_cold[i] = c;
        if (has_hot) {
            const float4 h = y[i];
            y[i] = make_float4(h.x + c.x, h.y + c.y, h.z + c.z, h.w + c.w);
        } else {
            y[i] = c;
        }
    }
}

// ===========================================================================
// Offline profiling: counts[i] = #{s : pre_i(X_s) > 0}.  One wave per row,
// samples in groups of BT.  (Offline, not on the decode path.)
// ===========================================================================
template <int WT, int XT, int BT>
__global__ __launch_bounds__(THREADS) void k_profile(const uint8_t* __restrict__ W,
                                                     const float* __restrict__ bias,
                                                     const uint8_t* __restrict__ X, int d, int rows,
                                                     int S, uint32_t* __restrict__ counts) {
    constexpr int EPC = Chunk<WT>::EPC;
    constexpr int XB = XT == F32 ? 4 : 2;
    const int lane = threadIdx.x & (WAVE - 1);
    const int row = (blockIdx.x * THREADS + threadIdx.x) / WAVE;
    if (row >= rows) return;
    const int64_t rb = row_bytes(WT, d);
    const uint8_t* w = W + (int64_t)row * rb;
    const int nch = d / EPC;
    const float bi = bias ? bias[row] : 0.0f;
    uint32_t cnt = 0;
    for (int s0 = 0; s0 < S; s0 += BT) {
        float acc[BT];
#pragma unroll
        for (int b = 0; b < BT; ++b) acc[b] = 0.0f;
        for (int c = lane; c < nch; c += WAVE) {
            u4 v = ld16(w + 16 * (int64_t)c);
            float sc = WT == Q4 ? half_f(*(const uint16_t*)(w + d / 2 + 2 * c)) : 0.0f;
#pragma unroll
            for (int b = 0; b < BT; ++b)
                if (s0 + b < S)
                    acc[b] = Dot<WT, XT>::run(v, sc, X + ((int64_t)(s0 + b) * d + c * EPC) * XB,
                                              acc[b]);
        }
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            float pre = wave_sum(acc[b]) + bi;
            cnt += (s0 + b < S && pre > 0.0f) ? 1u : 0u;
        }
    }
    if (lane == 0) counts[row] = cnt;
}

// ===========================================================================
// Adaptive predictor threshold (offline): the firing (sample, neuron) pairs'
// logits as order-preserving integer keys, then an exact radix selection of
// the m-th largest (three passes of 11, 11 and 10 bits, integer histograms).
// ===========================================================================
// key(a) < key(b) iff a < b for non-NaN floats (-0 just below +0); 0 is never a
// key of a float (the smallest, key(-inf), is 0x007fffff) and marks "no pair".
__device__ __forceinline__ uint32_t fkey(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t k) {
    return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// keys[i * S + s] = fkey(logits[s * rows + i]) if neuron i fires on sample s
// (deciding pre-activation > 0, decided in float32 as k_profile decides), else 0.
// One wave per neuron, samples in groups of BT.
template <int WT, int XT, int BT>
__global__ __launch_bounds__(THREADS) void k_fire_keys(const uint8_t* __restrict__ W,
                                                       const float* __restrict__ bias,
                                                       const uint8_t* __restrict__ X, int d, int rows,
                                                       int S, const float* __restrict__ logits,
                                                       uint32_t* __restrict__ keys) {
    constexpr int EPC = Chunk<WT>::EPC;
    constexpr int XB = XT == F32 ? 4 : 2;
    const int lane = threadIdx.x & (WAVE - 1);
    const int row = (blockIdx.x * THREADS + threadIdx.x) / WAVE;
    if (row >= rows) return;
    const int64_t rb = row_bytes(WT, d);
    const uint8_t* w = W + (int64_t)row * rb;
    const int nch = d / EPC;
    const float bi = bias ? bias[row] : 0.0f;
    for (int s0 = 0; s0 < S; s0 += BT) {
        float acc[BT];
#pragma unroll
        for (int b = 0; b < BT; ++b) acc[b] = 0.0f;
        for (int c = lane; c < nch; c += WAVE) {
            const u4 v = ld16(w + 16 * (int64_t)c);
            const float sc = WT == Q4 ? half_f(*(const uint16_t*)(w + d / 2 + 2 * c)) : 0.0f;
#pragma unroll
            for (int b = 0; b < BT; ++b)
                if (s0 + b < S)
                    acc[b] = Dot<WT, XT>::run(v, sc, X + ((int64_t)(s0 + b) * d + c * EPC) * XB, acc[b]);
        }
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            const float pre = wave_sum(acc[b]) + bi;
            if (lane == b && s0 + b < S)
                keys[(int64_t)row * S + s0 + b] = pre > 0.0f ? fkey(logits[(int64_t)(s0 + b) * rows + row]) : 0u;
        }
    }
}

// Selection state: [0] key prefix fixed so far, [1] its bit mask, [2] rank still
// wanted below the prefix (1 = the largest), [3] N keys, [4] m = ceil(target N).
constexpr int SEL_BINS = 2048;

// hist[digit] += number of keys that carry the current prefix, by their `bits`-bit
// digit at `shift` (bits <= 11)
__global__ __launch_bounds__(THREADS) void k_key_hist(const uint32_t* __restrict__ keys, int64_t len,
                                                      const uint32_t* __restrict__ state, int shift,
                                                      int bits, uint32_t* __restrict__ hist) {
    __shared__ uint32_t s_h[SEL_BINS];
    for (int b = threadIdx.x; b < SEL_BINS; b += THREADS) s_h[b] = 0u;
    __syncthreads();
    const uint32_t prefix = state[0], pmask = state[1], dmask = (1u << bits) - 1u;
    const int64_t stride = (int64_t)gridDim.x * THREADS;
    for (int64_t j = (int64_t)blockIdx.x * THREADS + threadIdx.x; j < len; j += stride) {
        const uint32_t k = keys[j];
        if (k != 0u && (k & pmask) == prefix) atomicAdd(&s_h[(k >> shift) & dmask], 1u);
    }
    __syncthreads();
    for (int b = threadIdx.x; b < SEL_BINS; b += THREADS)
        if (s_h[b]) atomicAdd(&hist[b], s_h[b]);
}

// One workgroup: fixes the next digit of the m-th largest key and clears hist.
__global__ __launch_bounds__(THREADS) void k_key_select(uint32_t* __restrict__ hist, int shift, int bits,
                                                        int first, double target, uint32_t* __restrict__ state) {
    if (threadIdx.x == 0) {
        const int bins = 1 << bits;
        if (first) {
            uint32_t N = 0;
            for (int b = 0; b < bins; ++b) N += hist[b];
            uint32_t m = (uint32_t)ceil(target * (double)N);
            if (N > 0 && m < 1) m = 1;
            if (m > N) m = N;
            state[2] = m;
            state[3] = N;
            state[4] = m;
        }
        const uint32_t rem = state[2];
        if (rem > 0) {
            uint32_t cum = 0;
            for (int b = bins - 1; b >= 0; --b) {
                const uint32_t h = hist[b];
                if (cum + h >= rem) {
                    state[0] |= (uint32_t)b << shift;
                    state[1] |= (uint32_t)(bins - 1) << shift;
                    state[2] = rem - cum;
                    break;
                }
                cum += h;
            }
        }
    }
    __syncthreads();
    for (int b = threadIdx.x; b < SEL_BINS; b += THREADS) hist[b] = 0u;
}

// tau = the float just below the selected logit (FLT_MAX without keys);
// stats [0] = N, [1] = m, [2] = 0 (counted by k_key_count)
__global__ void k_key_finish(const uint32_t* __restrict__ state, float* __restrict__ tau,
                             uint32_t* __restrict__ stats) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        const uint32_t N = state[3];
        *tau = N ? nextafterf(fkey_inv(state[0]), -INFINITY) : 3.402823466e38f;
        stats[0] = N;
        stats[1] = state[4];
        stats[2] = 0u;
    }
}

// stats[2] += number of keys whose logit is > tau
__global__ __launch_bounds__(THREADS) void k_key_count(const uint32_t* __restrict__ keys, int64_t len,
                                                       const float* __restrict__ tau,
                                                       uint32_t* __restrict__ stats) {
    __shared__ uint32_t s_c[NWAVES];
    const uint32_t kt = fkey(*tau);
    uint32_t c = 0;
    const int64_t stride = (int64_t)gridDim.x * THREADS;
    for (int64_t j = (int64_t)blockIdx.x * THREADS + threadIdx.x; j < len; j += stride) {
        const uint32_t k = keys[j];
        c += (k != 0u && k > kt) ? 1u : 0u;
    }
    c = (uint32_t)wave_sum_int((int)c);
    if ((threadIdx.x & (WAVE - 1)) == 0) s_c[threadIdx.x / WAVE] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < NWAVES; ++w) t += s_c[w];
        if (t) atomicAdd(&stats[2], t);
    }
}

// The true firing set of a batch: bit i of mask = OR over tokens of (deciding
// pre-activation of neuron i > 0, in float32).  One workgroup per mask word:
// each wave decides 16 neurons, then one ballot writes the word.
template <int WT, int XT>
__global__ __launch_bounds__(THREADS) void k_true_mask(const uint8_t* __restrict__ W,
                                                       const float* __restrict__ bias,
                                                       const uint8_t* __restrict__ X, int d, int rows,
                                                       int B, uint64_t* __restrict__ mask) {
    constexpr int EPC = Chunk<WT>::EPC;
    constexpr int XB = XT == F32 ? 4 : 2;
    __shared__ unsigned s_fire[64];
    const int lane = threadIdx.x & (WAVE - 1), wv = threadIdx.x / WAVE;
    const int64_t rb = row_bytes(WT, d);
    const int nch = d / EPC;
    for (int j = 0; j < 16; ++j) {
        const int loc = 16 * wv + j, row = 64 * blockIdx.x + loc;
        unsigned fire = 0;
        if (row < rows) {
            const uint8_t* w = W + (int64_t)row * rb;
            const float bi = bias ? bias[row] : 0.0f;
            for (int b = 0; b < B; ++b) {
                float acc = 0.0f;
                for (int c = lane; c < nch; c += WAVE) {
                    const u4 v = ld16(w + 16 * (int64_t)c);
                    const float sc = WT == Q4 ? half_f(*(const uint16_t*)(w + d / 2 + 2 * c)) : 0.0f;
                    acc = Dot<WT, XT>::run(v, sc, X + ((int64_t)b * d + c * EPC) * XB, acc);
                }
                fire |= (wave_sum(acc) + bi) > 0.0f ? 1u : 0u;
            }
        }
        if (lane == 0) s_fire[loc] = fire;
    }
    __syncthreads();
    if (wv == 0) {
        const uint64_t word = __ballot(s_fire[lane] != 0u);
        if (lane == 0) mask[blockIdx.x] = word;
    }
}

// ===========================================================================
// Neuron index: rank_i = #{j : c_j > c_i} + #{j < i : c_j == c_i}; perm[rank_i] = i.
// Exact, deterministic, O(n^2) compares over LDS tiles of the counts.
// ===========================================================================
// Online activation counts: counter i owned by thread i, so no atomics and the
// result is exact and independent of scheduling.
__global__ __launch_bounds__(THREADS) void k_accumulate_mask(const uint64_t* __restrict__ mask, int n,
                                                             uint32_t* __restrict__ counts) {
    const int i = blockIdx.x * THREADS + threadIdx.x;
    if (i < n) counts[i] += (uint32_t)((mask[i >> 6] >> (i & 63)) & 1ull);
}

__global__ __launch_bounds__(THREADS) void k_index(const uint32_t* __restrict__ counts, int n,
                                                   int32_t* __restrict__ perm) {
    constexpr int TILE = 4096;
    __shared__ uint32_t s_c[TILE];
    const int i = blockIdx.x * THREADS + threadIdx.x;
    const uint32_t ci = i < n ? counts[i] : 0u;
    int rank = 0;
    for (int t0 = 0; t0 < n; t0 += TILE) {
        const int len = min(TILE, n - t0);
        __syncthreads();
        for (int k = threadIdx.x; k < len; k += THREADS) s_c[k] = counts[t0 + k];
        __syncthreads();
        if (i < n) {
            for (int k = 0; k < len; ++k) {
                const uint32_t cj = s_c[k];
                rank += (cj > ci) | ((cj == ci) & (t0 + k < i));
            }
        }
    }
    if (i < n) perm[rank] = i;
}

// dst row s = src row perm[s]; 4-byte words.
__global__ __launch_bounds__(THREADS) void k_permute_rows(const uint32_t* __restrict__ src,
                                                          uint32_t* __restrict__ dst,
                                                          const int32_t* __restrict__ perm,
                                                          int64_t words_per_row) {
    const int s = blockIdx.x;
    const int p = perm[s];
    if ((unsigned)p >= gridDim.x) return;      // not a row id: dst row left as it was
    const uint32_t* from = src + (int64_t)p * words_per_row;
    uint32_t* to = dst + (int64_t)s * words_per_row;
    for (int64_t k = threadIdx.x; k < words_per_row; k += THREADS) to[k] = from[k];
}

// Plain 16-byte copy (traffic calibration); also used to zero workspaces.
__global__ __launch_bounds__(THREADS) void k_copy(const u4* __restrict__ src, u4* __restrict__ dst,
                                                  int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * THREADS;
    for (int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

// Plain read stream (the attainable-bandwidth ceiling for weight streams):
// reads n16 16-byte words with non-temporal loads, U loads in flight per thread,
// and stores one xor of them per workgroup so the loads cannot be dropped.
constexpr int STREAM_WG = 2048;      // workgroups of k_stream_read (8 per compute unit)
__global__ __launch_bounds__(THREADS) void k_stream_read(const u4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
    constexpr int U = 4;
    __shared__ unsigned s_x[NWAVES];
    const int64_t stride = (int64_t)gridDim.x * THREADS;
    int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x;
    unsigned acc = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u4 v[U];
#pragma unroll
        for (int q = 0; q < U; ++q) v[q] = ld16_stream(src + i + q * stride);
#pragma unroll
        for (int q = 0; q < U; ++q) acc ^= v[q].x ^ v[q].y ^ v[q].z ^ v[q].w;
    }
    for (; i < n16; i += stride) {
        const u4 v = ld16_stream(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int o = WAVE / 2; o > 0; o >>= 1) acc ^= (unsigned)__shfl_xor((int)acc, o, WAVE);
    if ((threadIdx.x & (WAVE - 1)) == 0) s_x[threadIdx.x / WAVE] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned t = 0;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) t ^= s_x[w];
        sink[blockIdx.x] = t;
    }
}

__global__ __launch_bounds__(THREADS) void k_zero(u4* __restrict__ dst, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * THREADS;
    for (int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x; i < n16; i += stride)
        dst[i] = u4{0u, 0u, 0u, 0u};
}

}  // namespace pi
