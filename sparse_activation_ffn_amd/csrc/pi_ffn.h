// pi_ffn.h -- fused sparse FFN kernel for small batches (gfx950).
//
// One workgroup per compute unit streams whole active neurons: for a group of
// G rows it loads the W_up (and W_gate) rows and the W_downT rows together,
// reduces the up/gate dot products across the workgroup, applies the
// activation, and accumulates h * W_downT[i][:] into per-thread columns.  Each
// workgroup ends with one full-width fp32 partial of y; k_reduce_parts sums
// the partials (hot workgroups into y_hot, cold ones into y_cold, y = y_hot +
// y_cold).  With a mask, the compaction into ascending hot / cold lists runs
// in the prologue of every workgroup (the mask is small and scanned in LDS),
// and the lists are written as a side output.
//
// PowerInfer pages: CSDN article, section on sparse activation (only the
// predicted neurons' rows are read and computed) and hybrid-design figure
// (each partition computes its predicted neurons; the results are merged).
#pragma once
#include "pi_kernels.h"

namespace pi {

#ifndef PI_FFN_THREADS
#define PI_FFN_THREADS 512
#endif
constexpr int FT = PI_FFN_THREADS;    // threads of the fused kernel (8 waves)
constexpr int FW = FT / WAVE;
constexpr int FSTAGE = 256;           // item rows resolved into LDS at a time
// Largest mask (64-bit words, n <= 65536) that the fused kernel compacts in its
// prologue (at most two words per thread); a larger mask is compacted by
// k_compact first and the fused kernel reads the lists.  The bound keeps the
// prologue short: two unrolled words per thread instead of eight (measured
// 0.25 us less from launch to the first row loads on the OPT-30B layer).
constexpr int FUSED_MASK_WORDS = 1024;

// acc[0..EPC) += h * (one 16-byte weight chunk, decoded); columns are the
// chunk's elements in order.
template <int WT> struct Axpy;
template <> struct Axpy<F32> {
    __device__ static void run(u4 w, float, float h, float* acc) {
        acc[0] = fmaf(h, bits_f(w.x), acc[0]);
        acc[1] = fmaf(h, bits_f(w.y), acc[1]);
        acc[2] = fmaf(h, bits_f(w.z), acc[2]);
        acc[3] = fmaf(h, bits_f(w.w), acc[3]);
    }
};
template <> struct Axpy<F16> {
    __device__ static void run(u4 w, float, float h, float* acc) {
        const unsigned v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            acc[2 * m] = fmaf(h, half_lo(v[m]), acc[2 * m]);
            acc[2 * m + 1] = fmaf(h, half_hi(v[m]), acc[2 * m + 1]);
        }
    }
};
template <> struct Axpy<Q4> {
    // one whole block: code byte t -> element t (low nibble), t + 16 (high nibble).
    // hs = h * scale.  acc gets hs * q for the codes q; the caller adds the
    // -8 hs of the whole block once per block (a running sum of hs), so each
    // element costs one byte-to-float conversion and one FMA.
    __device__ static void run(u4 w, float, float hs, float* acc) {
        const unsigned v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            unsigned lo = v[m] & 0x0f0f0f0fu, hi = (v[m] >> 4) & 0x0f0f0f0fu;
            // keep the byte pattern visible, so each byte converts in one
            // instruction (v_cvt_f32_ubyte0..3) instead of an extract + convert
            asm volatile("" : "+v"(lo), "+v"(hi));
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                acc[4 * m + b] = fmaf(hs, (float)((lo >> (8 * b)) & 0xffu), acc[4 * m + b]);
                acc[16 + 4 * m + b] = fmaf(hs, (float)((hi >> (8 * b)) & 0xffu), acc[16 + 4 * m + b]);
            }
        }
    }
};

// Fused gathered FFN.  NC = 16-byte chunks of a row per thread (d <= NC * FT * EPC);
// G = rows per group so a group has 8 chunks per matrix in flight per thread.
template <int WT, int XT, int BT, int ACT, int NC>
__global__ __launch_bounds__(FT) void k_ffn(FfnArgs a, DownOut o) {
    constexpr int EPC = Chunk<WT>::EPC;
    constexpr int XB = XT == F32 ? 4 : 2;
    // rows per group: the register buffers of the ring (G rows x NC chunks x 2 or
    // 3 matrices each) plus BT x NC x EPC accumulators must fit in 256 VGPRs.
    // Two buffers of G2 rows, or, where it holds more rows without spilling,
    // three buffers of G3 rows (a group's loads are then issued two groups ahead)
    constexpr int G0 = (WT == Q4 ? 4 : 8) / NC / (ACT == REGLU ? 2 : 1) / (BT >= 2 ? 2 : 1);
    constexpr int G2 = G0 > 0 ? G0 : 1;
    constexpr int G3 = (2 * G2 + 2) / 3;
    constexpr bool RING3 = BT == 1 && NC <= (WT == Q4 ? 1 : 2) && 3 * G3 > 2 * G2;
    constexpr int G = RING3 ? G3 : G2;
    constexpr int NM = ACT == REGLU ? 2 : 1;          // dot products per row (up, gate)
    // dynamic LDS: [x for BT tokens] [mask words]
    extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];
    __shared__ int s_row[FSTAGE];
    __shared__ float s_red[2][FW][G][NM][BT];
    __shared__ int s_wtot[FW];
    __shared__ int s_whot[FW];
    const int64_t xrow = (int64_t)a.d * XB;
    uint8_t* s_x = s_dyn;
    uint64_t* s_words = reinterpret_cast<uint64_t*>(s_dyn + BT * xrow);
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int wv = tid / WAVE;
    const int nch = a.d / EPC;                         // 16-byte (code) chunks of a row
    // The chunk of a row that this thread takes in the up (and gate) dot
    // products, and the one it accumulates in the down projection.  With one
    // chunk per thread and fewer chunks than threads, the down chunks go first
    // to the threads that hold no up chunk: at d = 12288 (Q4_0, 384 chunks)
    // waves 0-3 take both, 4-5 up only and 6-7 down only, so each SIMD carries
    // three of the row's 768 chunk units instead of four on two of them.
    auto up_chunk = [&](int k) { return tid + FT * k; };
    auto down_chunk = [&](int k) {
        if constexpr (NC == 1) return tid >= nch ? tid - nch : tid + (FT - nch);
        return tid + FT * k;
    };

    // Prologue, one memory round trip: this thread's share of x and its run of
    // mask words are loaded before anything waits on either (x first, so the
    // wait at the join after the conditional mask loads covers both).
    constexpr int PMAX = (FUSED_MASK_WORDS + FT - 1) / FT;
    constexpr int XCH = BT * NC * EPC * XB / 16;       // 16-byte x pieces per thread (d <= NC FT EPC)
    const int words = a.mask ? (a.n + 63) / 64 : 0;
    const int per = (words + FT - 1) / FT;             // mask words per thread (<= PMAX)
    const int w0 = tid * per;
    const int all16 = (int)(BT * xrow / 16);
    auto load_x = [&](u4 (&xv)[XCH], int b0) {
        const int n16 = (int)(min(BT, a.B - b0) * xrow / 16);
        const u4* src = reinterpret_cast<const u4*>(a.x + b0 * xrow);
#pragma unroll
        for (int j = 0; j < XCH; ++j) xv[j] = src[min(tid + FT * j, n16 - 1)];
    };
    auto store_x = [&](const u4 (&xv)[XCH], int b0) {
        const int n16 = (int)(min(BT, a.B - b0) * xrow / 16);
        u4* dst = reinterpret_cast<u4*>(s_x);
#pragma unroll
        for (int j = 0; j < XCH; ++j) {
            const int k = tid + FT * j;
            if (k < all16) dst[k] = k < n16 ? xv[j] : u4{0u, 0u, 0u, 0u};
        }
    };
    u4 xv0[XCH];
    load_x(xv0, 0);
    uint64_t mw[PMAX];
#pragma unroll
    for (int q = 0; q < PMAX; ++q) {
        mw[q] = 0;
        if (q < per) mw[q] = a.mask[min(w0 + q, words - 1)];
    }
    // the weight and bias pointers and the output descriptor sit in
    // kernel-argument cache lines that nothing above reads: fetch them now,
    // while x and the mask are in flight, rather than as scalar-cache misses
    // after the scan
    asm volatile("" ::"s"(a.up[0]), "s"(a.bup[0]), "s"(o.partials), "s"(o.nch));
    store_x(xv0, 0);
    int H, C;
    bool dense = false;                                // item k is row k (no list)
    int run = 0;                                       // rank of this thread's first set bit
    if (a.mask) {
        // per-thread totals and counts below n_hot (hot ranks are [0, H))
        const int nhot = a.rows[0];
        int tot = 0, hot = 0;
#pragma unroll
        for (int q = 0; q < PMAX; ++q) {
            if (q < per) {
                const int w = w0 + q;
                uint64_t v = w < words ? mw[q] : 0ull;
                if (w == words - 1 && a.n % 64) v &= (1ull << (a.n % 64)) - 1ull;   // bits past n
                tot += __popcll(v);
                hot += 64 * w + 64 <= nhot ? __popcll(v)
                       : 64 * w < nhot     ? __popcll(v & ((1ull << (nhot - 64 * w)) - 1ull))
                                           : 0;
                if (w < words) s_words[w] = v;         // read back by this thread only
            }
        }
        // exclusive scan of the per-thread totals: DPP in the wave, then the
        // FW wave totals through LDS; the hot counts are only summed
        const int inc = wave_incl_scan(tot);
        hot = wave_sum_int(hot);
        if (lane == WAVE - 1) s_wtot[wv] = inc;
        if (lane == 0) s_whot[wv] = hot;
        __syncthreads();
        int before = 0, T = 0;
        H = 0;
#pragma unroll
        for (int w = 0; w < FW; ++w) {
            const int t = s_wtot[w];
            before += w < wv ? t : 0;
            T += t;
            H += s_whot[w];
        }
        run = before + inc - tot;
        C = T - H;
        if (blockIdx.x == 0 && tid == 0) {
            a.out_counts[0] = H;
            a.out_counts[1] = C;
        }
    } else {
        dense = item_counts(a, H, C);
    }
    int part, lo, hi, nh;
    chunk_range(o.nch, H, C, blockIdx.x, part, lo, hi, nh);
    const int hbase = part == 0 ? 0 : H;              // first item of this partition
    const uint8_t* wup = part == 0 ? a.up[0] : a.up[1];
    const uint8_t* wgt = part == 0 ? a.gate[0] : a.gate[1];
    const uint8_t* wdn = part == 0 ? a.down[0] : a.down[1];
    const float* bup = part == 0 ? a.bup[0] : a.bup[1];
    const float* bgt = part == 0 ? a.bgate[0] : a.bgate[1];
    const int32_t* idx = dense ? nullptr : part == 0 ? a.idx[0] : a.idx[1];
    const int prows = part == 0 ? a.rows[0] : a.rows[1];
    int32_t* const oidx = part == 0 ? a.out_idx[0] : a.out_idx[1];   // (mask mode) list output

    for (int b0 = 0; b0 < a.B; b0 += BT) {
        const int nb = min(BT, a.B - b0);
        if (b0 > 0) {                                  // next token group of x
            u4 xv[XCH];
            load_x(xv, b0);
            __syncthreads();
            store_x(xv, b0);
        }
        float acc[BT][NC][EPC];
        float hsum[BT][NC];                            // Q4_0: running sum of h * scale per chunk
#pragma unroll
        for (int b = 0; b < BT; ++b)
#pragma unroll
            for (int k = 0; k < NC; ++k) {
                hsum[b][k] = 0.0f;
#pragma unroll
                for (int e = 0; e < EPC; ++e) acc[b][k][e] = 0.0f;
            }

        for (int s0 = lo; s0 < hi; s0 += FSTAGE) {
            const int len = min(FSTAGE, hi - s0);
            __syncthreads();                           // x staged; previous stage consumed
            if (a.mask) {
                // each thread emits the set bits of its words whose ranks fall in
                // this stage's item range [gb, ge) (all in this partition)
                const int gb = hbase + s0, ge = gb + len;
                int r0 = run;
#pragma unroll
                for (int q = 0; q < PMAX; ++q) {
                    if (q < per && w0 + q < words) {
                        uint64_t v = s_words[w0 + q];
                        const int pc = __popcll(v);
                        if (pc > 0 && r0 < ge && r0 + pc > gb) {
                            const int skip = max(0, gb - r0);
                            if (skip > 0) v &= ~((1ull << select_bit(v, skip)) - 1ull);
                            for (int rank = r0 + skip; v != 0 && rank < ge; ++rank) {
                                const int id = 64 * (w0 + q) + __builtin_ctzll(v);
                                v &= v - 1ull;
                                const int row = part == 0 ? id : id - a.rows[0];
                                s_row[rank - gb] = (unsigned)row < (unsigned)prows ? row : -1;
                                if (b0 == 0) oidx[rank - hbase] = row;
                            }
                        }
                        r0 += pc;
                    }
                }
            } else {
                for (int t = tid; t < len; t += FT) {  // resolve this stage's rows
                    const int row = idx ? idx[s0 + t] : s0 + t;
                    s_row[t] = (unsigned)row < (unsigned)prows ? row : -1;   // -1: not a row, h = 0
                }
            }
            __syncthreads();
            // groups of G rows, software-pipelined: the loads of the next group are
            // in flight while the current one is reduced and accumulated; the LDS
            // reduction slots alternate so each group needs one barrier
            struct Regs {
                u4 wu[G][NC], wg[G][NC], wd[G][NC];
                // Q4_0 scales stay raw f16 bits until they are used: converting
                // right after the load would make the next group's loads wait
                uint16_t su[G][NC], sg[G][NC], sd[G][NC];
                float bu[G], bg[G];                    // biases of the group's rows
                int row[G];
            };
            // the biases are loaded with the group's weights: a load consumed
            // right away would make the wait before this group also wait for the
            // next group's loads, which are in flight by then
            const float* bsu = bup ? bup : reinterpret_cast<const float*>(a.x);
            const float* bsg = bgt ? bgt : reinterpret_cast<const float*>(a.x);
            auto load_group = [&](Regs& R, int g0) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int r = s_row[min(g0 + g, len - 1)];
                    R.row[g] = g0 + g < len ? r : -1;
                }
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    R.bu[g] = bsu[bup ? max(R.row[g], 0) : 0];
                    if (ACT == REGLU) R.bg[g] = bsg[bgt ? max(R.row[g], 0) : 0];
                }
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int64_t rbase = (int64_t)max(R.row[g], 0) * a.rb;
#pragma unroll
                    for (int k = 0; k < NC; ++k) {
                        const int cu = min(up_chunk(k), nch - 1), cd = min(down_chunk(k), nch - 1);
                        R.wu[g][k] = ld16_stream(wup + rbase + 16 * (int64_t)cu);
                        if (ACT == REGLU) R.wg[g][k] = ld16_stream(wgt + rbase + 16 * (int64_t)cu);
                        R.wd[g][k] = ld16_stream(wdn + rbase + 16 * (int64_t)cd);
                    }
                }
                if (WT == Q4) {
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const int64_t sbase = (int64_t)max(R.row[g], 0) * a.rb + a.d / 2;
#pragma unroll
                        for (int k = 0; k < NC; ++k) {
                            const int cu = min(up_chunk(k), nch - 1), cd = min(down_chunk(k), nch - 1);
                            R.su[g][k] = *(const uint16_t*)(wup + sbase + 2 * cu);
                            if (ACT == REGLU)
                                R.sg[g][k] = *(const uint16_t*)(wgt + sbase + 2 * cu);
                            R.sd[g][k] = *(const uint16_t*)(wdn + sbase + 2 * cd);
                        }
                    }
                }
            };
            auto process_group = [&](const Regs& R, int slot) {
                // partial dot products of this thread's chunks, then wave sums
#pragma unroll
                for (int g = 0; g < G; ++g) {
#pragma unroll
                    for (int b = 0; b < BT; ++b) {
                        float pu = 0.0f, pg = 0.0f;
#pragma unroll
                        for (int k = 0; k < NC; ++k) {
                            const int c = up_chunk(k);
                            if (c < nch) {
                                const uint8_t* xp = s_x + b * xrow + (int64_t)c * EPC * XB;
                                pu = Dot<WT, XT>::run(R.wu[g][k], WT == Q4 ? half_f(R.su[g][k]) : 0.f, xp, pu);
                                if (ACT == REGLU)
                                    pg = Dot<WT, XT>::run(R.wg[g][k], WT == Q4 ? half_f(R.sg[g][k]) : 0.f, xp,
                                                          pg);
                            }
                        }
                        pu = wave_sum_last(pu);
                        if (ACT == REGLU) pg = wave_sum_last(pg);
                        if (lane == WAVE - 1) {
                            s_red[slot][wv][g][0][b] = pu;
                            if (ACT == REGLU) s_red[slot][wv][g][NM - 1][b] = pg;
                        }
                    }
                }
                __syncthreads();
                // every thread forms h for the group (same order everywhere), then axpy
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int r = R.row[g];
                    const float bu = (r >= 0 && bup) ? R.bu[g] : 0.0f;
                    const float bg = (ACT == REGLU && r >= 0 && bgt) ? R.bg[g] : 0.0f;
#pragma unroll
                    for (int b = 0; b < BT; ++b) {
                        float up = 0.0f, gt = 0.0f;
#pragma unroll
                        for (int w = 0; w < FW; ++w) {
                            up += s_red[slot][w][g][0][b];
                            if (ACT == REGLU) gt += s_red[slot][w][g][NM - 1][b];
                        }
                        up += bu;
                        float hv;
                        if (ACT == RELU) {
                            hv = up > 0.0f ? up : 0.0f;
                        } else if (ACT == SQRELU) {
                            const float r = up > 0.0f ? up : 0.0f;
                            hv = r * r;
                        } else {
                            gt += bg;
                            hv = (gt > 0.0f ? gt : 0.0f) * up;
                        }
                        if (r < 0 || b >= nb) hv = 0.0f;
#pragma unroll
                        for (int k = 0; k < NC; ++k) {
                            // one chunk per thread: threads without a down chunk skip it
                            // (whole waves); with more chunks per thread the accumulation
                            // stays unconditional (a branch here cost the ReGLU-70B batch-1
                            // kernel 2 us in code generation)
                            if (NC == 1 && down_chunk(k) >= nch) continue;
                            // a slot that holds no row read row 0 of the partition
                            // (clamped, unconditional loads): its weights are replaced by
                            // zeros here, where they are consumed, so a non-finite value
                            // in a row outside the active set never reaches y
                            if (WT == Q4) {
                                const float hs = r >= 0 ? hv * half_f(R.sd[g][k]) : 0.0f;
                                hsum[b][k] += hs;
                                Axpy<WT>::run(R.wd[g][k], 0.f, hs, acc[b][k]);
                            } else {
                                const u4 wd = r >= 0 ? R.wd[g][k] : u4{0u, 0u, 0u, 0u};
                                Axpy<WT>::run(wd, 0.f, hv, acc[b][k]);
                            }
                        }
                    }
                }
            };
            // groups go round a ring of register buffers: a buffer is refilled
            // with the group after next (two-buffer ring) or the group three
            // ahead (three-buffer ring) as soon as it is consumed; reduction
            // slots alternate with the group index
            if constexpr (RING3) {
                Regs R0, R1, R2;
                load_group(R0, 0);
                if (G < len) load_group(R1, G);
                for (int g0 = 0; g0 < len; g0 += 3 * G) {
                    const int k = g0 / G;              // index of the group in R0
                    if (g0 + 2 * G < len) load_group(R2, g0 + 2 * G);
                    process_group(R0, k & 1);
                    if (g0 + 3 * G < len) load_group(R0, g0 + 3 * G);
                    if (g0 + G < len) process_group(R1, (k + 1) & 1);
                    if (g0 + 4 * G < len) load_group(R1, g0 + 4 * G);
                    if (g0 + 2 * G < len) process_group(R2, k & 1);
                }
            } else {
                Regs A, Bn;
                load_group(A, 0);
                for (int g0 = 0; g0 < len; g0 += 2 * G) {
                    if (g0 + G < len) load_group(Bn, g0 + G);
                    process_group(A, 0);
                    if (g0 + 2 * G < len) load_group(A, g0 + 2 * G);
                    if (g0 + G < len) process_group(Bn, 1);
                }
            }
            __syncthreads();                           // s_red and s_row free for reuse
        }
        // this workgroup's partial of y for the token group, staged in LDS so the
        // global stores are contiguous (a thread's columns are a whole chunk
        // away from its neighbours': direct stores would hit a cache line per lane)
        __syncthreads();                               // every wave is done with x and the mask words
        float* s_part = reinterpret_cast<float*>(s_dyn);
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            if (b < nb) {
#pragma unroll
                for (int k = 0; k < NC; ++k) {
                    const int c = down_chunk(k);
                    if (c < nch) {
                        if (WT == Q4) {                // the codes' offset of 8: -8 * sum of h * scale
#pragma unroll
                            for (int e = 0; e < EPC; ++e) acc[b][k][e] = fmaf(-8.0f, hsum[b][k], acc[b][k][e]);
                        }
                        f4* dst = reinterpret_cast<f4*>(s_part + (int64_t)b * a.d + (int64_t)c * EPC);
#pragma unroll
                        for (int e = 0; e < EPC / 4; ++e)
                            dst[e] = f4{acc[b][k][4 * e], acc[b][k][4 * e + 1], acc[b][k][4 * e + 2],
                                        acc[b][k][4 * e + 3]};
                    }
                }
            }
        }
        __syncthreads();
        {
            const int n4 = nb * a.d / 4;               // tokens b0 .. b0 + nb - 1 are contiguous rows
            f4* dst = reinterpret_cast<f4*>(o.partials + ((int64_t)blockIdx.x * a.B + b0) * a.d);
            const f4* src = reinterpret_cast<const f4*>(s_part);
            for (int i = tid; i < n4; i += FT) dst[i] = src[i];
        }
    }
}

// Sum of the workgroup partials, fixed order: thread (s, e) adds partials s,
// s + RS, ... of element e for the hot range and the cold range; the RS slices
// are then added in slice order.  y_hot, y_cold, y = y_hot + y_cold.
constexpr int RE = 32;                // output elements per workgroup (one 128-byte line)
constexpr int RS = 16;                // partial slices per element
__global__ __launch_bounds__(RE * RS) void k_reduce_parts(FfnArgs a, DownOut o) {
    __shared__ float s_h[RS][RE], s_c[RS][RE];
    const int e = threadIdx.x % RE, s = threadIdx.x / RE;
    const int64_t len = (int64_t)a.B * a.d;
    const int64_t at = (int64_t)blockIdx.x * RE + e;
    const int64_t atc = at < len ? at : len - 1;
    constexpr int R = 16;              // partials in flight per thread (256 partials per pass)
    // the first pass's partials are loaded before the hot / cold counts: their
    // addresses do not depend on the counts, which take a chain of dependent
    // scalar loads and a division to turn into the hot workgroup count
    float v[R];
    auto load = [&](int k0) {
#pragma unroll
        for (int q = 0; q < R; ++q) v[q] = o.partials[min(k0 + RS * q, o.nch - 1) * len + atc];
    };
    load(s);
    int H, C;
    if (a.mask) {                      // counts were written by the fused kernel
        H = a.out_counts[0];
        C = a.out_counts[1];
    } else {
        item_counts(a, H, C);
    }
    int part, lo, hi, nh;
    chunk_range(o.nch, H, C, 0, part, lo, hi, nh);
    float yh = 0.0f, yc = 0.0f;
    for (int k0 = s;;) {
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const int kk = k0 + RS * q;
            if (kk < nh) yh += v[q];
            else if (kk < o.nch) yc += v[q];
        }
        k0 += RS * R;
        if (k0 >= o.nch) break;
        load(k0);
    }
    s_h[s][e] = yh;
    s_c[s][e] = yc;
    __syncthreads();
    if (s == 0 && at < len) {
        float th = 0.0f, tc = 0.0f;
#pragma unroll
        for (int q = 0; q < RS; ++q) {
            th += s_h[q][e];
            tc += s_c[q][e];
        }
        if (o.y_part[0]) o.y_part[0][at] = th;
        if (o.y_part[1]) o.y_part[1][at] = tc;
        if (o.y) o.y[at] = th + tc;
    }
}

}  // namespace pi
