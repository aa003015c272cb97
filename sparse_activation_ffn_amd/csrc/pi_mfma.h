// pi_mfma.h -- matrix-core (MFMA) path of the sparse FFN for batches of 16..64
// tokens on gfx950.
//
// At a prompt-sized batch the union of the tokens' active sets is most of the
// layer, and the gathered FFN is a real contraction: up = X [B x d] . W[rows]^T,
// then y = h [B x T] . W_downT[rows].  Both run on v_mfma_f32_16x16x32_f16 with
// fp32 accumulation; operands are staged in LDS as f16 (Q4_0 weights are
// dequantised to f16 on the way in, h is rounded to f16 once).
//
// Operand layout used here (wave64, lane l = 16 q + c): lane l supplies
// A[m = c][k = 8 q + i] and B[k = 8 q + i][n = c] for i = 0..7 (one 16-byte LDS
// read each) and receives D[m = 4 q + i][n = c] for i = 0..3.  Any numbering of
// k works as long as A and B agree, which they do by construction.
//
// Every LDS operand tile has 256-byte rows (128 f16 of K) whose sixteen 16-byte
// blocks are XOR-swizzled by the row index (swz): a fragment read (16 rows,
// one block each per 16 lanes) and the staging stores used here touch every
// bank once, where rows padded by 16 bytes measure 2-way conflicts on gfx950.
//
// All kernels are software-pipelined: the global loads of step s + D are
// issued into a register ring right after step s's registers are written to
// LDS, so D steps of weights are in flight while the matrix cores work.
//
// PowerInfer pages: CSDN article, section on sparse activation (only predicted
// neurons are computed; over a batch the union of the tokens' sets).
#pragma once
#include "pi_kernels.h"

namespace pi {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef float f4m __attribute__((ext_vector_type(4)));

constexpr int MM = 64;          // largest token tile (batches up to 64)
constexpr int KS = 128;         // K per pipeline step: one 256-byte LDS row
constexpr int DC = 128;         // output columns per down workgroup (32 per wave)
constexpr int DK = 128;         // active rows (K) per down step
constexpr int MFMA_WG = 256;    // threads of the up and predictor kernels (4 waves)
constexpr int NXCD = 8;         // accelerator complex dies (XCDs) of the MI355X, one L2 each
constexpr int DOWN_WG = 256;    // threads of the down kernel (4 waves)

// Byte offset of 16-byte block kb (0..15) of row r in a [rows][256 B] tile.
__device__ __forceinline__ int swz(int r, int kb) { return r * 256 + 16 * (kb ^ (r & 15)); }

// Weight loads of the up kernel.  A step reads only part of each 128-byte line of
// a row (Q4_0: 64 bytes of codes); the rest of the line is read one step later,
// so the loads are ordinary (cached) ones: with non-temporal loads the line was
// often gone by then (measured FETCH_SIZE, OPT-175B-shaped Q4_0 layer, batch 64:
// 287 MB non-temporal against 206 MB plain for 199 MB of algorithmic bytes).
#ifndef PI_UP_NT
#define PI_UP_NT 0
#endif
__device__ __forceinline__ u4 ld16_up(const void* p) {
#if PI_UP_NT
    return ld16_stream(p);
#else
    return ld16(p);
#endif
}

__device__ __forceinline__ f4m mfma32(h8 a, h8 b, f4m c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Two 4-bit codes -> two f16 values (q - 8) * s, each rounded once: the f16
// with bits 0x6400 | q is 1024 + q, and 1024 + q - 1032 is exact (the "magic
// number" int4-to-fp16 conversion of Kim et al., arXiv 2211.10017).  q4_bits
// builds the two halves 0x640q from two bytes of v in one byte permute (the
// 0x64 bytes come from the constant operand) and one AND that keeps the low
// nibbles; sel picks bytes 0, 1 (Q4_SEL01) or 2, 3 (Q4_SEL23) of v.
constexpr unsigned Q4_SEL01 = 0x04010400u, Q4_SEL23 = 0x04030402u;
__device__ __forceinline__ unsigned q4_bits(unsigned v, unsigned sel) {
    return __builtin_amdgcn_perm(0x64646464u, v, sel) & 0xff0fff0fu;
}
__device__ __forceinline__ unsigned q4_scaled(unsigned bits, h2v s2) {
    h2v t = __builtin_bit_cast(h2v, bits);
    t = (t - h2v{(_Float16)1032.0f, (_Float16)1032.0f}) * s2;
    return __builtin_bit_cast(unsigned, t);
}

// One Q4_0 block (16 code bytes, scale s) -> its 32 weights as f16, in order:
// element t < 16 is the low nibble of byte t, element t >= 16 the high nibble
// of byte t - 16.  out[0..3] hold elements 0..7, 8..15, 16..23, 24..31.
__device__ __forceinline__ void deq_block(u4 c, _Float16 s, u4 out[4]) {
    const h2v s2 = {s, s};
    const unsigned w[4] = {c.x, c.y, c.z, c.w};
    unsigned lo[8], hi[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const unsigned ws = w[p] >> 4;                 // high nibbles moved to the low ones
        lo[2 * p] = q4_scaled(q4_bits(w[p], Q4_SEL01), s2);
        lo[2 * p + 1] = q4_scaled(q4_bits(w[p], Q4_SEL23), s2);
        hi[2 * p] = q4_scaled(q4_bits(ws, Q4_SEL01), s2);
        hi[2 * p + 1] = q4_scaled(q4_bits(ws, Q4_SEL23), s2);
    }
    out[0] = u4{lo[0], lo[1], lo[2], lo[3]};
    out[1] = u4{lo[4], lo[5], lo[6], lo[7]};
    out[2] = u4{hi[0], hi[1], hi[2], hi[3]};
    out[3] = u4{hi[4], hi[5], hi[6], hi[7]};
}

// Eight consecutive codes of a block half (8 bytes; HIGH selects the high
// nibbles) -> 8 f16 weights.
__device__ __forceinline__ u4 deq8(u2 c, _Float16 s, bool high) {
    const h2v s2 = {s, s};
    const unsigned w[2] = {high ? c.x >> 4 : c.x, high ? c.y >> 4 : c.y};
    unsigned o[4];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        o[2 * p] = q4_scaled(q4_bits(w[p], Q4_SEL01), s2);
        o[2 * p + 1] = q4_scaled(q4_bits(w[p], Q4_SEL23), s2);
    }
    return u4{o[0], o[1], o[2], o[3]};
}

__device__ __forceinline__ int round8(int v) { return (v + 7) & ~7; }

// Position of item `item` in the f16 h buffer: hot items at [0, H), cold items
// from the next multiple of 8, so every chunk of the down kernel starts on a
// 16-byte boundary.
__device__ __forceinline__ int h_pos(int item, int H) { return item < H ? item : item - H + round8(H); }

// Software pipeline over K steps [s0, s1): D stages of global loads in a
// register ring; step s's registers go to LDS, then step s + D is loaded into
// the freed registers while the matrix cores work on step s.  Every stage
// issues the same loads (past the end it reloads the last step), so the
// compiler's wait counts are static inside an unrolled round and a store waits
// only for its own stage, never for the D - 1 stages issued after it.  The
// compiler cannot carry exact wait counts around a loop back edge (it waits for
// everything at the loop head), so the steps run in rounds of ROUND steps
// (several rings); the remainder runs in rings of D steps whose padding steps
// past the end are stored with their token operand zeroed (store(R, false))
// and computed, adding exact zeros.
template <int D, int ROUND, typename Stage, typename Step>
__device__ __forceinline__ void pipeline_rounds(int s0, int s1, Stage (&R)[D], Step step) {
    static_assert(ROUND % D == 0, "a round is whole rings");
    int sb = s0;
    for (; sb + ROUND <= s1; sb += ROUND) {
#pragma unroll
        for (int dd = 0; dd < ROUND; ++dd) step(R[dd % D], sb + dd, true);
    }
    for (; sb < s1; sb += D) {
#pragma unroll
        for (int dd = 0; dd < D; ++dd) step(R[dd % D], sb + dd, sb + dd < s1);
    }
}

// Rounds of ROUND steps only, the last one padded (one copy of the body: for
// step counts that are a multiple of ROUND, where the remainder loop's extra
// code only costs registers).
template <int D, int ROUND, typename Stage, typename Step>
__device__ __forceinline__ void pipeline_rounds_padded(int s0, int s1, Stage (&R)[D], Step step) {
    static_assert(ROUND % D == 0, "a round is whole rings");
    for (int sb = s0; sb < s1; sb += ROUND) {
#pragma unroll
        for (int dd = 0; dd < ROUND; ++dd) step(R[dd % D], sb + dd, sb + dd < s1);
    }
}

template <int D, typename Stage, int ROUND = 12 / D * D, bool PADDED = false, typename Load, typename Store,
          typename Compute>
__device__ __forceinline__ void run_pipeline(int s0, int s1, Load load, Store store, Compute compute) {
    if (s1 <= s0) return;                             // uniform
    Stage R[D];
#pragma unroll
    for (int dd = 0; dd < D; ++dd) load(R[dd], min(s0 + dd, s1 - 1));
    auto step = [&](Stage& St, int s, bool live) {
        __syncthreads();                              // the previous step's LDS reads are done
        store(St, live);
        load(St, min(s + D, s1 - 1));
        __syncthreads();
        compute();
    };
    if constexpr (PADDED) pipeline_rounds_padded<D, ROUND>(s0, s1, R, step);
    else pipeline_rounds<D, ROUND>(s0, s1, R, step);
}

// ===========================================================================
// Up/gate.  Workgroup = 4 waves; tile = 16 MT tokens x UR = 64 NT items (16 NT
// per wave).  A step stages K = 128 of every row (Q4_0: 4 blocks of 32; f16:
// 16 chunks of 8) and the matching token x K slice of x.  With a mask the
// workgroup scans it (all of it, in LDS) and resolves its own UR items;
// workgroup 0 writes the counts and every workgroup its items of the ascending
// lists.  Writes h (f16) [B][h_ld] at h_pos(item).
// ===========================================================================
template <int WT, int MT, int NT> struct UpShape {
    static constexpr int CH = WT == Q4 ? 4 : 16;       // 16-byte chunks per row per step
    static constexpr int UR = 64 * NT;                 // items per workgroup
    static constexpr int J = UR * CH / MFMA_WG;        // chunks per thread per matrix
    static constexpr int XN = 16 * MT * 16;            // 16-byte pieces of the x slice
    static constexpr int XJ = (XN + MFMA_WG - 1) / MFMA_WG;
    static constexpr int D = 3;                        // steps in flight
};

// Chunk t of a step -> (row, chunk).  f16: 16 lanes cover one row's 256 bytes;
// Q4_0: 16 lanes cover one block of 16 rows, so each of the 4 stores of a
// dequantised block hits 16 different swizzled positions.
template <int WT>
__device__ __forceinline__ void up_task(int t, int& r, int& ch) {
    if (WT == Q4) {
        r = (t & 15) + 16 * (t >> 6);
        ch = (t >> 4) & 3;
    } else {
        r = t >> 4;
        ch = t & 15;
    }
}

// Items [i0, i0 + UR) of an up workgroup -> s_row / s_part (row -1: not a row).
// With a mask the workgroup scans all of it in LDS (s_words) and writes the list
// entries of ranks [i0, i0 + UR); workgroup 0 writes the counts.  When the
// active count reaches the dense crossover (a.dense_from), the items are all
// rows of both partitions instead (the lists still name the predicted set).
// Returns false (uniformly) when the workgroup has no items.
template <int UR>
__device__ bool up_resolve(const FfnArgs& a, int i0, int* s_row, int* s_part, uint64_t* s_words,
                           int& H, int& C, bool lists_out = true) {
    __shared__ int s_cnt[2];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    bool dense;
    if (a.mask) {
        // block-wide scan of the mask words: thread t owns words [t per, t per + per)
        const int words = (a.n + 63) / 64;
        const int per = (words + MFMA_WG - 1) / MFMA_WG;
        const int w0 = tid * per;
        int tot = 0;
        for (int w = w0; w < min(words, w0 + per); ++w) {
            uint64_t v = a.mask[w];
            if (w == words - 1 && a.n % 64) v &= (1ull << (a.n % 64)) - 1ull;
            s_words[w] = v;
            tot += __popcll(v);
        }
        __shared__ int s_wtot[MFMA_WG / 64];
        const int inc = wave_incl_scan(tot);   // inclusive, DPP within the wave
        if (lane == 63) s_wtot[wv] = inc;
        __syncthreads();
        int before = 0, T = 0;
#pragma unroll
        for (int w = 0; w < MFMA_WG / 64; ++w) {
            before += w < wv ? s_wtot[w] : 0;
            T += s_wtot[w];
        }
        const int run0 = before + inc - tot;              // rank of this thread's first set bit
        // rank of the first set bit of each word (this thread's words), for the
        // search below
        int* const s_scan = reinterpret_cast<int*>(s_words + words);
        {
            int rr = run0;
            for (int w = w0; w < min(words, w0 + per); ++w) {
                s_scan[w] = rr;
                rr += __popcll(s_words[w]);
            }
        }
        const int nhot = a.rows[0];
        const int wh = nhot / 64;
        if (nhot >= a.n) {
            if (tid == 0) s_cnt[0] = T;
        } else if (wh >= w0 && wh < w0 + per) {
            int h = run0;
            for (int w = w0; w < wh; ++w) h += __popcll(s_words[w]);
            s_cnt[0] = h + __popcll(s_words[wh] & ((1ull << (nhot % 64)) - 1ull));
        }
        if (tid < UR) s_row[tid] = -1;
        __syncthreads();
        H = s_cnt[0];
        C = T - H;
        if (lists_out && blockIdx.x == 0 && tid == 0) {
            a.out_counts[0] = H;
            a.out_counts[1] = C;
        }
        dense = crosses_to_dense(a, T);
        // the set bits of ranks [i0, i0 + UR): this workgroup's list entries and,
        // unless the step crosses to dense, its items.  Thread t < UR finds the
        // bit of rank i0 + t by a binary search over the words' first ranks (a
        // serial walk by the threads owning the words took one entry per
        // iteration on a few lanes: 7-10 us of the prologue at batch 8)
        if (tid < UR && i0 + tid < T) {
            const int rank = i0 + tid;
            const int id = kth_active(s_words, s_scan, words, rank);
            const int part = rank < H ? 0 : 1;
            const int row = part == 0 ? id : id - nhot;
            if (!dense) {
                s_row[tid] = (unsigned)row < (unsigned)by_part(a.rows, part) ? row : -1;
                s_part[tid] = part;
            }
            if (lists_out) by_part(a.out_idx, part)[part == 0 ? rank : rank - H] = row;
        }
        if (dense) {
            H = a.rows[0];
            C = a.nparts > 1 ? a.rows[1] : 0;
        }
        __syncthreads();
    } else {
        dense = item_counts(a, H, C);
    }
    if (i0 >= H + C) return false;                        // whole workgroup, uniformly
    if (!a.mask || dense) {
        if (tid < UR) {
            const int item = min(i0 + tid, H + C - 1);
            int part, row;
            item_row(a, item, H, dense, part, row);
            if ((unsigned)row >= (unsigned)by_part(a.rows, part)) row = -1;
            s_row[tid] = i0 + tid < H + C ? row : -1;
            s_part[tid] = part;
        }
        __syncthreads();
    }
    return true;
}

// The part of an up tile (16 MT tokens x 64 NT items) one wave computes.  With 64
// tokens and 64 items the four waves take 2 x 2 quarters (32 tokens x 32 items
// each), so a wave reads 2 + 2 operand fragments per K slice instead of 4 + 1;
// otherwise each wave takes all tokens and 16 NT items.
template <int MT, int NT> struct WaveTile {
    static constexpr bool QUAD = MT == 4 && NT == 1;
    static constexpr int MW = QUAD ? 2 : MT;          // token tiles of 16 per wave
    static constexpr int NW = QUAD ? 2 : NT;          // item tiles of 16 per wave
    __device__ static int tok0(int wv) { return QUAD ? 32 * (wv & 1) : 0; }
    __device__ static int item0(int wv) { return QUAD ? 32 * (wv >> 1) : 16 * NT * wv; }
};

// Bias, activation and the f16 h write of an up tile: lane holds
// acc[g][jn][mt][i] = D[token tok0 + 16 mt + 4 q + i][item item0 + 16 jn + c].
template <int ACT, int NM, int NT, int MT>
__device__ __forceinline__ void up_epilogue(const FfnArgs& a,
                                            const f4m (&acc)[NM][WaveTile<MT, NT>::NW][WaveTile<MT, NT>::MW],
                                            const int* s_row, const int* s_part, int i0, int H, int T,
                                            _Float16* __restrict__ h16) {
    using WT_ = WaveTile<MT, NT>;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int q = lane >> 4, c = lane & 15;
#pragma unroll
    for (int jn = 0; jn < WT_::NW; ++jn) {
        const int r = WT_::item0(wv) + 16 * jn + c;
        const int row = s_row[r], part = s_part[r];
        const int item = i0 + r;
        if (item < T) {
            const int hp = h_pos(item, H);
            const float* pbu = by_part(a.bup, part);
            const float* pbg = by_part(a.bgate, part);
            const float bu = (row >= 0 && pbu) ? pbu[row] : 0.0f;
            const float bg = (ACT == REGLU && row >= 0 && pbg) ? pbg[row] : 0.0f;
#pragma unroll
            for (int mt = 0; mt < WT_::MW; ++mt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = WT_::tok0(wv) + 16 * mt + 4 * q + i;
                    if (tok < a.B) {
                        const float up = acc[0][jn][mt][i] + bu;
                        float hv;
                        if (ACT == RELU) {
                            hv = up > 0.0f ? up : 0.0f;
                        } else if (ACT == SQRELU) {
                            const float r = up > 0.0f ? up : 0.0f;
                            hv = r * r;
                        } else {
                            const float gt = acc[NM - 1][jn][mt][i] + bg;
                            hv = (gt > 0.0f ? gt : 0.0f) * up;
                        }
                        if (row < 0) hv = 0.0f;
                        h16[(int64_t)tok * a.h_ld + hp] = (_Float16)hv;
                    }
                }
            }
        }
    }
}

// Split over K: this slice's fp32 pre-activations of the tile (slice 0 adds
// the biases), for k_up_finish.  Same lane mapping as up_epilogue.
template <int NM, int NT, int MT>
__device__ __forceinline__ void up_partials(const FfnArgs& a,
                                            const f4m (&acc)[NM][WaveTile<MT, NT>::NW][WaveTile<MT, NT>::MW],
                                            const int* s_row, const int* s_part, int i0, int T, int slice) {
    using WT_ = WaveTile<MT, NT>;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int q = lane >> 4, c = lane & 15;
#pragma unroll
    for (int jn = 0; jn < WT_::NW; ++jn) {
        const int r = WT_::item0(wv) + 16 * jn + c;
        const int row = s_row[r], part = s_part[r];
        const int item = i0 + r;
        if (item < T) {
            float bias[NM];
            const float* pbu = by_part(a.bup, part);
            const float* pbg = by_part(a.bgate, part);
            bias[0] = (slice == 0 && row >= 0 && pbu) ? pbu[row] : 0.0f;
            if (NM == 2) bias[NM - 1] = (slice == 0 && row >= 0 && pbg) ? pbg[row] : 0.0f;
#pragma unroll
            for (int g = 0; g < NM; ++g)
#pragma unroll
                for (int mt = 0; mt < WT_::MW; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int tok = WT_::tok0(wv) + 16 * mt + 4 * q + i;
                        if (tok < a.B)
                            a.upart[((int64_t)(slice * NM + g) * a.B + tok) * a.upart_ld + item] =
                                acc[g][jn][mt][i] + bias[g];
                    }
        }
    }
}

// The slices' sum, the activation and the f16 h write of every (token, item)
// of the step (fixed slice order).  grid (x: item blocks, y: tokens).  A
// thread's first slice values are loaded before the item count, whose load
// they do not depend on (items below ld are inside the slices' buffer).
constexpr int UP_FINISH_MAX_S = 4;    // most K slices the split up kernel writes
template <int ACT, int NM>
__global__ __launch_bounds__(THREADS) void k_up_finish(const float* __restrict__ upart, int S, int ld, int B,
                                                       const int* __restrict__ ht, _Float16* __restrict__ h16,
                                                       int h_ld) {
    const int tok = blockIdx.y;
    const int stride = gridDim.x * THREADS;
    const int item0 = blockIdx.x * THREADS + threadIdx.x;
    float p[UP_FINISH_MAX_S][NM];
    auto load = [&](int item) {
        const int64_t ic = min(item, ld - 1);
#pragma unroll
        for (int k = 0; k < UP_FINISH_MAX_S; ++k)
            if (k < S)
#pragma unroll
                for (int g = 0; g < NM; ++g) p[k][g] = upart[((int64_t)(k * NM + g) * B + tok) * ld + ic];
    };
    load(item0);
    const int H = ht[0], T = ht[1];
    for (int item = item0; item < T; item += stride) {
        float v[NM];
#pragma unroll
        for (int g = 0; g < NM; ++g) v[g] = 0.0f;
#pragma unroll
        for (int k = 0; k < UP_FINISH_MAX_S; ++k)
            if (k < S)
#pragma unroll
                for (int g = 0; g < NM; ++g) v[g] += p[k][g];
        if (item + stride < T) load(item + stride);
        float hv;
        if (ACT == RELU) {
            hv = v[0] > 0.0f ? v[0] : 0.0f;
        } else if (ACT == SQRELU) {
            const float r = v[0] > 0.0f ? v[0] : 0.0f;
            hv = r * r;
        } else {
            hv = (v[NM - 1] > 0.0f ? v[NM - 1] : 0.0f) * v[0];
        }
        h16[(int64_t)tok * h_ld + h_pos(item, H)] = (_Float16)hv;
    }
}

template <int WT, int ACT, int MT, int NT>
__global__ __launch_bounds__(MFMA_WG) void k_mfma_up(FfnArgs a, _Float16* __restrict__ h16) {
    constexpr int NM = ACT == REGLU ? 2 : 1;
    using S = UpShape<WT, MT, NT>;
    constexpr int J = S::J, XN = S::XN, XJ = S::XJ, D = S::D, UR = S::UR;
    __shared__ __attribute__((aligned(16))) uint8_t s_x[16 * MT * 256];
    __shared__ __attribute__((aligned(16))) uint8_t s_w[NM][UR * 256];
    __shared__ int s_row[UR];
    __shared__ int s_part[UR];
    extern __shared__ uint64_t s_words[];        // mask words (mask mode only)
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int q = lane >> 4, c = lane & 15;
    const int i0 = blockIdx.x * UR;

    const int slice = blockIdx.y, nsl = a.ksplit;
    int H, C;
    const bool any = up_resolve<UR>(a, i0, s_row, s_part, s_words, H, C, slice == 0);
    if (nsl > 1 && blockIdx.x == 0 && slice == 0 && tid == 0) {
        a.up_ht[0] = H;
        a.up_ht[1] = H + C;
    }
    if (!any) return;
    const int T = H + C;

    // per-thread weight sources (a row that is not one, an out-of-range id,
    // reads row 0 of a partition that has rows, and its weights are zeroed)
    const uint8_t* src[NM][J];
    bool live[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        int r, ch;
        up_task<WT>(tid + MFMA_WG * j, r, ch);
        const int row = s_row[r], part = s_part[r];
        live[j] = row >= 0;
        const int rr = row >= 0 ? row : 0;
        const int pp = row >= 0 ? part : (a.rows[0] > 0 ? 0 : 1);
        src[0][j] = a.up[pp] + (int64_t)rr * a.rb;
        if (NM == 2) src[NM - 1][j] = a.gate[pp] + (int64_t)rr * a.rb;
    }
    struct Stage {
        u4 w[NM][J];
        _Float16 sc[NM][J];
        u4 xv[XJ];
    };
    auto load = [&](Stage& R, int s) {
        const int k0 = s * KS;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            int r, ch;
            up_task<WT>(tid + MFMA_WG * j, r, ch);
#pragma unroll
            for (int g = 0; g < NM; ++g) {
                if (WT == Q4) {
                    const int blk = k0 / 32 + ch;
                    R.w[g][j] = ld16_up(src[g][j] + 16 * (int64_t)blk);
                    R.sc[g][j] = __builtin_bit_cast(
                        _Float16, *reinterpret_cast<const uint16_t*>(src[g][j] + a.d / 2 + 2 * (int64_t)blk));
                } else {
                    R.w[g][j] = ld16_up(src[g][j] + 2 * (int64_t)(k0 + 8 * ch));
                }
            }
        }
#pragma unroll
        for (int j = 0; j < XJ; ++j) {
            const int t = min(tid + MFMA_WG * j, XN - 1), m = t >> 4, kb = t & 15;
            R.xv[j] = ld16(a.x + ((int64_t)min(m, a.B - 1) * a.d + k0 + 8 * kb) * 2);
        }
    };
    // (zeroing of padding tokens and of non-rows happens here, where the data
    // are consumed: a select right after a load would make the load wait)
    auto store = [&](const Stage& R, bool act) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            int r, ch;
            up_task<WT>(tid + MFMA_WG * j, r, ch);
#pragma unroll
            for (int g = 0; g < NM; ++g) {
                if (WT == Q4) {
                    u4 o[4];
                    deq_block(R.w[g][j], live[j] ? R.sc[g][j] : (_Float16)0.0f, o);
#pragma unroll
                    for (int p = 0; p < 4; ++p) *reinterpret_cast<u4*>(s_w[g] + swz(r, 4 * ch + p)) = o[p];
                } else {
                    *reinterpret_cast<u4*>(s_w[g] + swz(r, ch)) = live[j] ? R.w[g][j] : u4{0u, 0u, 0u, 0u};
                }
            }
        }
#pragma unroll
        for (int j = 0; j < XJ; ++j) {
            const int t = tid + MFMA_WG * j, m = t >> 4, kb = t & 15;
            // (token rows past B hold copies of row B - 1; their output rows are
            // never stored)
            if (t < XN) *reinterpret_cast<u4*>(s_x + swz(m, kb)) = act ? R.xv[j] : u4{0u, 0u, 0u, 0u};
        }
    };
    using WTL = WaveTile<MT, NT>;
    constexpr int MW = WTL::MW, NW = WTL::NW;
    const int tok0 = WTL::tok0(wv), item0 = WTL::item0(wv);
    f4m acc[NM][NW][MW];
#pragma unroll
    for (int g = 0; g < NM; ++g)
#pragma unroll
        for (int jn = 0; jn < NW; ++jn)
#pragma unroll
            for (int mt = 0; mt < MW; ++mt) acc[g][jn][mt] = f4m{0.f, 0.f, 0.f, 0.f};
    // every fragment of the step is read before the first product: the LDS
    // latency is paid once per step, not once per 32-wide K slice
    auto compute = [&]() {
        constexpr int NKS = KS / 32;
        h8 ax[NKS][MW], bw[NKS][NM][NW];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int kb = 4 * ks + q;
#pragma unroll
            for (int mt = 0; mt < MW; ++mt)
                ax[ks][mt] = *reinterpret_cast<const h8*>(s_x + swz(tok0 + 16 * mt + c, kb));
#pragma unroll
            for (int g = 0; g < NM; ++g)
#pragma unroll
                for (int jn = 0; jn < NW; ++jn)
                    bw[ks][g][jn] = *reinterpret_cast<const h8*>(s_w[g] + swz(item0 + 16 * jn + c, kb));
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int g = 0; g < NM; ++g)
#pragma unroll
                for (int jn = 0; jn < NW; ++jn)
#pragma unroll
                    for (int mt = 0; mt < MW; ++mt)
                        acc[g][jn][mt] = mfma32(ax[ks][mt], bw[ks][g][jn], acc[g][jn][mt]);
        // keep the order: the compiler's scheduler would interleave each product
        // with its own fragment reads again
        __builtin_amdgcn_sched_group_barrier(0x100, NKS * (MW + NM * NW), 0);   // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, NKS * NM * NW * MW, 0);     // matrix-core ops
    };
    const int steps = a.d / KS;
    run_pipeline<D, Stage>(steps * slice / nsl, steps * (slice + 1) / nsl, load, store, compute);
    if (nsl > 1) up_partials<NM, NT, MT>(a, acc, s_row, s_part, i0, T, slice);
    else up_epilogue<ACT, NM, NT, MT>(a, acc, s_row, s_part, i0, H, T, h16);
}

// Split of one partition's items over chunks, chunk starts on multiples of 8.
__device__ __forceinline__ void chunk_range8(int nch, int H, int C, int k, int& part, int& lo,
                                             int& hi) {
    int nh0, lo0, hi0, p;
    chunk_range(nch, H, C, k, p, lo0, hi0, nh0);
    const int N = p == 0 ? H : C;
    const int nk = p == 0 ? nh0 : nch - nh0;          // chunks of this partition
    const int kk = p == 0 ? k : k - nh0;
    const int per = round8((N + nk - 1) / max(nk, 1));
    part = p;
    lo = min(N, kk * per);
    hi = min(N, lo + per);
}

// ===========================================================================
// Down, split over K (the active rows): grid (d / 128 column tiles, chunks);
// chunk k covers the items chunk_range8 gives it (one partition).  A step
// stages 128 rows x 128 columns of W_downT and the token x 128 tile of h.
// Each thread loads an 8 x 8 block of weights (8 rows x 16 bytes; the 16
// lanes of a load group read 256 contiguous bytes of one row) and transposes
// it in registers, so every LDS column (a 256-byte row of the tile) holds the
// step's 128 rows.  4 waves, each owning 32 columns.
// ===========================================================================
// Byte offset of 16-byte block kb of column col in the transposed weight tile:
// the block index is XOR-ed with the column and its column group, so the
// stores (16 lanes = 16 column groups of one row block) and the fragment reads
// (16 consecutive columns) both spread over the banks.
__device__ __forceinline__ int wt_off(int col, int kb) {
    return col * 256 + 16 * (kb ^ ((col & 15) ^ ((col >> 3) & 15)));
}

template <int WT, int MT> struct DownShape {
    static constexpr int HN = 16 * MT * 16;                    // 16-byte pieces of the h tile
    static constexpr int HJ = (HN + DOWN_WG - 1) / DOWN_WG;    // per thread
    static constexpr int D = WT == Q4 ? 3 : 2;                 // steps in flight
};

template <int WT, bool LISTS, int MT>
__global__ __launch_bounds__(DOWN_WG) void k_mfma_down(FfnArgs a, DownOut o, const _Float16* __restrict__ h16) {
    using S = DownShape<WT, MT>;
    constexpr int HN = S::HN, HJ = S::HJ, D = S::D;
    __shared__ __attribute__((aligned(16))) uint8_t s_h[16 * MT * 256];
    __shared__ __attribute__((aligned(16))) uint8_t s_wt[DC * 256];      // [column][k], swizzled
    __shared__ __attribute__((aligned(16))) int s_ids[D + 1][DK];        // row ids of upcoming steps
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int q = lane >> 4, c = lane & 15;
    // XCD-aware placement: workgroups are dealt to the 8 XCDs round-robin by their
    // linear id, so workgroup L runs on XCD L % 8.  Chunk k = (L % 8) + 8 m puts
    // every column tile of one chunk on the same XCD: the chunk's weight rows (each
    // read by all column tiles, 64-byte pieces of shared 128-byte lines, and the
    // shared scale lines of Q4_0 rows) and its h slice then come from that XCD's
    // L2 after the first touch instead of once per XCD from memory.
    const int tiles = a.d / DC;
    const int L = blockIdx.x, j = L / NXCD;
    const int c0 = (j % tiles) * DC, k = L % NXCD + NXCD * (j / tiles);
    int H, C;
    const bool dense = item_counts(a, H, C);
    int part, lo, hi;
    chunk_range8(o.nch, H, C, k, part, lo, hi);
    const int hb = part == 0 ? 0 : round8(H);         // h buffer offset of this partition
    const uint8_t* base = part == 0 ? a.down[0] : a.down[1];
    const int32_t* idx = part == 0 ? a.idx[0] : a.idx[1];
    const int prows = part == 0 ? a.rows[0] : a.rows[1];
    const int steps = (hi - lo + DK - 1) / DK;
    // this thread's weights of a step.  f16: an 8 x 8 block, rows 8 rg .. +7,
    // columns 8 cg .. +7.  Q4_0: rows 4 rg .. +3 and the 16 columns held by 8
    // code bytes of one block (both nibbles of each byte: columns k .. k+7 and
    // k+16 .. k+23 of the block, k = 0 or 8), so no code byte is loaded twice.
    const int cg = WT == Q4 ? (tid & 7) : (tid & 15), rg = WT == Q4 ? (tid >> 3) : (tid >> 4);
    const int col0 = WT == Q4 ? c0 + 32 * (cg >> 1) + 8 * (cg & 1) : c0 + 8 * cg;
    // Q4_0 rows are addressed by 32-bit offsets from the partition base (the host
    // keeps Q4_0 partitions on this path below 2 GiB): a base in scalar registers
    // plus a 32-bit offset is one load operand, instead of 64-bit arithmetic
    // per row
    const uint64_t bu = reinterpret_cast<uint64_t>(base);
    typedef const __attribute__((address_space(1))) uint8_t gbyte;
    gbyte* const wb = (gbyte*)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(bu >> 32)) << 32) |
                               (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bu));
    const unsigned coff = 16u * (unsigned)(col0 >> 5) + (unsigned)(col0 & 15);      // 8 code bytes
    constexpr int NR = WT == Q4 ? 4 : 8;                                             // rows per thread
    const unsigned soff = (unsigned)(a.d / 2) + 2u * (unsigned)(col0 >> 5);          // the block's scale
    f4m acc[2][MT];
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[jn][mt] = f4m{0.f, 0.f, 0.f, 0.f};
    if (steps > 0) {                                  // uniform; an empty chunk writes zeros
        // row id of step-relative item tid of step s, or -1 (loads a clamped,
        // valid list entry whatever s is, so the load is unconditional)
        auto row_id = [&](int s) -> int {
            const int item = lo + s * DK + tid;
            const int ic = min(item, hi - 1);
            const int v = (LISTS && !dense) ? idx[ic] : ic;
            return (tid < DK && item < hi && (unsigned)v < (unsigned)prows) ? v : -1;
        };
        struct Stage {
            u4 w[8];                  // f16: 8 columns of each of 8 rows
            u2 cq[8];                 // Q4_0: 8 codes of each of 8 rows
            _Float16 sc[8];
            u4 hv[HJ];
            unsigned rows_ok;         // bit r: row r is a row (else its weights are zeroed)
            int hvalid[HJ];           // items of each h load that are in the chunk
            bool full;                // every item of the step is in the chunk
        };
        // loads of step s (its row ids are in s_ids[s % (D + 1)]); all unconditional
        auto load = [&](Stage& R, int s) {
            const int* ids = s_ids[s % (D + 1)];
            R.rows_ok = 0;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int row = ids[NR * rg + r];
                if (WT == Q4) {
                    // a non-row reads row 0 and gets a zero scale (zero weights)
                    R.rows_ok |= (row >= 0 ? 1u : 0u) << r;
                    const unsigned ro = (unsigned)max(row, 0) * (unsigned)a.rb;
                    R.cq[r] = *(const __attribute__((address_space(1))) u2*)(wb + (ro + coff));
                    R.sc[r] = *(const __attribute__((address_space(1))) _Float16*)(wb + (ro + soff));
                } else {
                    R.rows_ok |= (row >= 0 ? 1u : 0u) << r;
                    const uint8_t* rowp = base + (int64_t)(row >= 0 ? row : 0) * a.rb;
                    R.w[r] = ld16_stream(rowp + 2 * (int64_t)col0);
                }
            }
            const int i0 = lo + s * DK;
            const int last = round8(hi) - 8;          // last 8-item group of this chunk
#pragma unroll
            for (int j = 0; j < HJ; ++j) {
                const int t = min(tid + DOWN_WG * j, HN - 1), m = t >> 4, kb = t & 15;
                R.hv[j] = ld16(h16 + (int64_t)min(m, a.B - 1) * a.h_ld + hb + min(i0 + 8 * kb, last));
                // items past hi are zeroed (token rows past B hold copies of row B - 1
                // and give output rows that are never stored)
                R.hvalid[j] = hi - (i0 + 8 * kb);
            }
            R.full = i0 + DK <= hi;
        };
        auto store = [&](const Stage& R, bool act) {
            if constexpr (WT == Q4) {
                // V[h][r][p] = columns 2p, 2p+1 of nibble half h (0: k + e, 1: k + 16 + e) of row r
                unsigned V[2][4][4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const _Float16 sr = ((R.rows_ok >> r) & 1u) ? R.sc[r] : (_Float16)0.0f;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const u4 w = deq8(R.cq[r], sr, h == 1);
                        V[h][r][0] = w.x; V[h][r][1] = w.y; V[h][r][2] = w.z; V[h][r][3] = w.w;
                    }
                }
                // each column's 4 rows (8 bytes) into its [column][k] row: k = 4 rg .. +3,
                // the low or high half of 16-byte block rg / 2
                const int lc0 = col0 - c0;
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int cc = 0; cc < 8; ++cc) {
                        const int p = cc >> 1;
                        const unsigned sel = (cc & 1) ? 0x07060302u : 0x05040100u;
                        const u2 out{__builtin_amdgcn_perm(V[h][1][p], V[h][0][p], sel),
                                     __builtin_amdgcn_perm(V[h][3][p], V[h][2][p], sel)};
                        *reinterpret_cast<u2*>(s_wt + wt_off(lc0 + 16 * h + cc, rg >> 1) + 8 * (rg & 1)) = out;
                    }
            } else {
                unsigned V[8][4];                       // V[r][p] = columns 2p, 2p+1 of row r
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const bool ok = (R.rows_ok >> r) & 1u;
                    const u4 w = ok ? R.w[r] : u4{0u, 0u, 0u, 0u};
                    V[r][0] = w.x; V[r][1] = w.y; V[r][2] = w.z; V[r][3] = w.w;
                }
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) {
                    const int p = cc >> 1;
                    const unsigned sel = (cc & 1) ? 0x07060302u : 0x05040100u;
                    u4 out;
                    out.x = __builtin_amdgcn_perm(V[1][p], V[0][p], sel);
                    out.y = __builtin_amdgcn_perm(V[3][p], V[2][p], sel);
                    out.z = __builtin_amdgcn_perm(V[5][p], V[4][p], sel);
                    out.w = __builtin_amdgcn_perm(V[7][p], V[6][p], sel);
                    *reinterpret_cast<u4*>(s_wt + wt_off(8 * cg + cc, rg)) = out;
                }
            }
            if (act && R.full) {                        // (uniform) the usual step: no item to mask
#pragma unroll
                for (int j = 0; j < HJ; ++j) {
                    const int t = tid + DOWN_WG * j, m = t >> 4, kb = t & 15;
                    if (t < HN) *reinterpret_cast<u4*>(s_h + swz(m, kb)) = R.hv[j];
                }
            } else {
#pragma unroll
                for (int j = 0; j < HJ; ++j) {
                    const int t = tid + DOWN_WG * j, m = t >> 4, kb = t & 15;
                    const u4 v = R.hv[j];
                    const int valid = act ? R.hvalid[j] : 0;
                    if (t < HN)
                        *reinterpret_cast<u4*>(s_h + swz(m, kb)) =
                            u4{valid >= 2 ? v.x : (valid == 1 ? v.x & 0xffffu : 0u),
                               valid >= 4 ? v.y : (valid == 3 ? v.y & 0xffffu : 0u),
                               valid >= 6 ? v.z : (valid == 5 ? v.z & 0xffffu : 0u),
                               valid >= 8 ? v.w : (valid == 7 ? v.w & 0xffffu : 0u)};
                }
            }
        };
        auto compute = [&]() {
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                const int kb = 4 * ks + q;
                h8 ah[MT], bw[2];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) ah[mt] = *reinterpret_cast<const h8*>(s_h + swz(16 * mt + c, kb));
#pragma unroll
                for (int jn = 0; jn < 2; ++jn)
                    bw[jn] = *reinterpret_cast<const h8*>(s_wt + wt_off(32 * wv + 16 * jn + c, kb));
#pragma unroll
                for (int jn = 0; jn < 2; ++jn)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[jn][mt] = mfma32(ah[mt], bw[jn], acc[jn][mt]);
            }
        };
        // ids run one step ahead of the weights: the id load of step s + D + 1
        // is issued before the weight loads of step s + D, so waiting for it
        // never waits behind them
#pragma unroll
        for (int dd = 0; dd < D; ++dd) {
            const int v = row_id(dd);
            if (tid < DK) s_ids[dd][tid] = v;
        }
        __syncthreads();
        int nid = row_id(D);
        Stage R[D];
#pragma unroll
        for (int dd = 0; dd < D; ++dd) load(R[dd], min(dd, steps - 1));
        // one ring per round (measured: rounds of several rings here were slower,
        // 121 -> 157 us on the Q4_0 batch-64 layer); padding steps past the end
        // store a zero h tile and add exact zeros
        pipeline_rounds_padded<D, D>(0, steps, R, [&](Stage& St, int s, bool live) {
            __syncthreads();                          // the previous step's LDS reads are done
            store(St, live);
            if (tid < DK) s_ids[(s + D) % (D + 1)][tid] = nid;
            __syncthreads();
            nid = row_id(s + D + 1);
            load(St, min(s + D, steps - 1));
            compute();
        });
    }
    // partial of y: lane holds D[token 16 mt + 4 q + i][column 32 wv + 16 jn + c]
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
        const int col = c0 + 32 * wv + 16 * jn + c;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 16 * mt + 4 * q + i;
                if (tok < a.B) o.partials[((int64_t)k * a.B + tok) * a.d + col] = acc[jn][mt][i];
            }
    }
}

// ===========================================================================
// Predictor on matrix cores (batches of 16..64 tokens, f16 P1t / P2t, f16 x).
//
// First layer: u = ReLU(x P1), a [B x d] by [d x r] product with small r, so
// the K dimension (d) is split over P1_KS slices to give the chip enough
// workgroups; k_mfma_pred1 writes fp32 partial sums per slice and k_u_relu
// adds them in slice order and applies the ReLU (u stays fp32, never rounded).
// ===========================================================================
constexpr int P1_ROWS = 64;     // P1t rows per workgroup (16 per wave)
constexpr int P1_KS = 16;       // K slices

template <int MT>
__global__ __launch_bounds__(MFMA_WG) void k_mfma_pred1(const uint8_t* __restrict__ P1t,
                                                       const uint8_t* __restrict__ x, int d, int r,
                                                       int B, float* __restrict__ part) {
    constexpr int J = P1_ROWS * 16 / MFMA_WG;         // 16-byte weight loads per thread
    constexpr int XN = 16 * MT * 16;                  // 16-byte pieces of the x slice
    constexpr int XJ = (XN + MFMA_WG - 1) / MFMA_WG;  // per thread
    constexpr int D = 3;
    __shared__ __attribute__((aligned(16))) uint8_t s_x[16 * MT * 256];
    __shared__ __attribute__((aligned(16))) uint8_t s_w[P1_ROWS * 256];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int q = lane >> 4, c = lane & 15;
    const int j0 = blockIdx.x * P1_ROWS, ky = blockIdx.y;
    const int64_t rb = (int64_t)d * 2;
    const uint8_t* src[J];
    bool live[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int row = j0 + ((tid + MFMA_WG * j) >> 4);
        live[j] = row < r;
        src[j] = P1t + (int64_t)(row < r ? row : 0) * rb;
    }
    struct Stage {
        u4 w[J];
        u4 xv[XJ];
    };
    auto load = [&](Stage& R, int s) {
        const int k0 = s * KS;
#pragma unroll
        for (int j = 0; j < J; ++j) R.w[j] = ld16_stream(src[j] + 2 * (int64_t)(k0 + 8 * ((tid + MFMA_WG * j) & 15)));
#pragma unroll
        for (int j = 0; j < XJ; ++j) {
            const int t = min(tid + MFMA_WG * j, XN - 1), m = t >> 4, kb = t & 15;
            R.xv[j] = ld16(x + ((int64_t)min(m, B - 1) * d + k0 + 8 * kb) * 2);
        }
    };
    auto store = [&](const Stage& R, bool act) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int t = tid + MFMA_WG * j;
            *reinterpret_cast<u4*>(s_w + swz(t >> 4, t & 15)) = live[j] ? R.w[j] : u4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < XJ; ++j) {
            const int t = tid + MFMA_WG * j, m = t >> 4, kb = t & 15;
            if (t < XN) *reinterpret_cast<u4*>(s_x + swz(m, kb)) = (act && m < B) ? R.xv[j] : u4{0u, 0u, 0u, 0u};
        }
    };
    f4m acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f4m{0.f, 0.f, 0.f, 0.f};
    auto compute = [&]() {
#pragma unroll
        for (int ks = 0; ks < KS / 32; ++ks) {
            const int kb = 4 * ks + q;
            const h8 bw = *reinterpret_cast<const h8*>(s_w + swz(16 * wv + c, kb));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt] = mfma32(*reinterpret_cast<const h8*>(s_x + swz(16 * mt + c, kb)), bw, acc[mt]);
        }
    };
    const int steps = d / KS;
    run_pipeline<D, Stage>(ky * steps / P1_KS, (ky + 1) * steps / P1_KS, load, store, compute);
    // lane holds D[token 16 mt + 4 q + i][row 16 wv + c]
    const int row = j0 + 16 * wv + c;
    if (row < r) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 16 * mt + 4 * q + i;
                if (tok < B) part[((int64_t)ky * B + tok) * r + row] = acc[mt][i];
            }
    }
}

// u = ReLU(sum of the P1_KS slice partials, in slice order), one workgroup per
// token (r <= 4096: at most 16 values per thread).  The workgroup also finds the
// token's largest u and the power of two uscale[b] = 2^(14 - e), e =
// floor(log2(max u)), that maps that maximum into [2^14, 2^15), and writes the
// second layer's operand once for every workgroup of that layer: u * uscale
// split into two f16 parts, uh = f16(u s) and ul = f16(u s - uh) ([B][r] each,
// uh then ul).  The power of two keeps the high part finite and normal whatever
// the magnitude of u.
constexpr int UR_MAX = 16;      // u values per thread of k_u_relu (r <= 16 * 256)
__global__ __launch_bounds__(THREADS) void k_u_relu(const float* __restrict__ part, int B, int r,
                                                    _Float16* __restrict__ uhl, float* __restrict__ uscale) {
    __shared__ float s_max[NWAVES];
    __shared__ float s_scale;
    const int b = blockIdx.x;
    const int64_t len = (int64_t)B * r;
    float vmax = 0.0f;
    float uv[UR_MAX];
    // four values at a time, their 4 x P1_KS loads issued together (clamped
    // addresses, unconditional) before any of them is summed
    constexpr int UG = 4;
#pragma unroll
    for (int t0 = 0; t0 < UR_MAX; t0 += UG) {
        if (threadIdx.x + THREADS * t0 >= r) break;       // this thread has no values left
        float v[UG][P1_KS];
#pragma unroll
        for (int g = 0; g < UG; ++g) {
            const int j = min(threadIdx.x + THREADS * (t0 + g), r - 1);
            const int64_t at = (int64_t)b * r + j;
#pragma unroll
            for (int k = 0; k < P1_KS; ++k) v[g][k] = part[k * len + at];
        }
#pragma unroll
        for (int g = 0; g < UG; ++g) {
            const int j = threadIdx.x + THREADS * (t0 + g);
            float sum = v[g][0];
#pragma unroll
            for (int k = 1; k < P1_KS; ++k) sum += v[g][k];
            const float u1 = (j < r && sum > 0.0f) ? sum : 0.0f;
            uv[t0 + g] = u1;
            vmax = fmaxf(vmax, u1);
        }
    }
    // largest u of the token (max is exact, so the order does not matter)
#pragma unroll
    for (int o = WAVE / 2; o > 0; o >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, o, WAVE));
    if ((threadIdx.x & (WAVE - 1)) == 0) s_max[threadIdx.x / WAVE] = vmax;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = s_max[0];
#pragma unroll
        for (int w = 1; w < NWAVES; ++w) m = fmaxf(m, s_max[w]);
        // m == 0 (every u zero) or not finite: no scaling
        const int e = (m > 0.0f && m <= 3.0e38f) ? ilogbf(m) : 14;
        const float sc = ldexpf(1.0f, 14 - e);
        uscale[b] = sc;
        s_scale = sc;
    }
    __syncthreads();
    const float sc = s_scale;
#pragma unroll
    for (int t = 0; t < UR_MAX; ++t) {
        const int j = threadIdx.x + THREADS * t;
        if (j >= r) break;
        const int64_t at = (int64_t)b * r + j;
        const float a = uv[t] * sc;
        const _Float16 hi = (_Float16)a;
        uhl[at] = hi;
        uhl[len + at] = (_Float16)(a - (float)hi);
    }
}

// ===========================================================================
// Second layer + threshold + union over tokens: logits = u P2 + b2 on matrix
// cores, 128 neurons (two mask words) per workgroup.  u is fp32; per token it is
// scaled by the power of two uscale[b] (exact) and enters the matrix cores as
// the sum of two f16 parts, hi = f16(u s) and lo = f16(u s - hi), whose
// products with the f16 weights are exact in the fp32 accumulation.  hi + lo
// carries u s to about 22 significant bits (lo is rounded too), so the logits
// come within ~2^-22 relative of the fp32 path, far inside the 1e-5 decision
// band; the scale keeps hi finite for any u and keeps hi + lo away from the
// f16 subnormals for every u above 2^-28 of the token's largest.  The epilogue
// multiplies the accumulator by 1 / uscale[b] (exact) before adding b2.
// ===========================================================================
constexpr int P2_ROWS = 128;    // neurons per workgroup (32 per wave)

template <int MT>
__global__ __launch_bounds__(MFMA_WG) __attribute__((amdgpu_waves_per_eu(2))) void k_mfma_pred2(
                                                       const uint8_t* __restrict__ P2t,
                                                       const float* __restrict__ b2, float thr,
                                                       const _Float16* __restrict__ uhl,
                                                       const float* __restrict__ uscale, int n, int r,
                                                       int B, uint64_t* __restrict__ mask,
                                                       float* __restrict__ logits) {
    constexpr int J = P2_ROWS * 16 / MFMA_WG;         // 16-byte weight loads per thread
    constexpr int UN = 16 * MT * 16;                  // 8-element pieces of the u slice
    constexpr int UJ = (UN + MFMA_WG - 1) / MFMA_WG;  // per thread
    constexpr int D = 2;
    __shared__ __attribute__((aligned(16))) uint8_t s_uh[16 * MT * 256];
    __shared__ __attribute__((aligned(16))) uint8_t s_ul[16 * MT * 256];
    __shared__ __attribute__((aligned(16))) uint8_t s_w[P2_ROWS * 256];
    __shared__ unsigned s_flag[P2_ROWS];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int q = lane >> 4, c = lane & 15;
    const int i0 = blockIdx.x * P2_ROWS;
    const int64_t rb = (int64_t)r * 2;
    const uint8_t* src[J];
    bool live[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int row = i0 + ((tid + MFMA_WG * j) >> 4);
        live[j] = row < n;
        src[j] = P2t + (int64_t)(row < n ? row : 0) * rb;
    }
    struct Stage {
        u4 w[J];
        u4 uh[UJ], ul[UJ];
    };
    const int64_t ulen = (int64_t)B * r;
    auto load = [&](Stage& R, int s) {
        const int k0 = s * KS;
#pragma unroll
        for (int j = 0; j < J; ++j) R.w[j] = ld16_stream(src[j] + 2 * (int64_t)(k0 + 8 * ((tid + MFMA_WG * j) & 15)));
#pragma unroll
        for (int j = 0; j < UJ; ++j) {
            const int t = min(tid + MFMA_WG * j, UN - 1), m = t >> 4, kb = t & 15;
            const int64_t at = (int64_t)min(m, B - 1) * r + k0 + 8 * kb;
            R.uh[j] = ld16(uhl + at);
            R.ul[j] = ld16(uhl + ulen + at);
        }
    };
    auto store = [&](const Stage& R, bool act) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int t = tid + MFMA_WG * j;
            *reinterpret_cast<u4*>(s_w + swz(t >> 4, t & 15)) = live[j] ? R.w[j] : u4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < UJ; ++j) {
            const int t = tid + MFMA_WG * j, m = t >> 4, kb = t & 15;
            if (t < UN) {
                const bool ok = act && m < B;
                *reinterpret_cast<u4*>(s_uh + swz(m, kb)) = ok ? R.uh[j] : u4{0u, 0u, 0u, 0u};
                *reinterpret_cast<u4*>(s_ul + swz(m, kb)) = ok ? R.ul[j] : u4{0u, 0u, 0u, 0u};
            }
        }
    };
    f4m acc[2][MT];
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[jn][mt] = f4m{0.f, 0.f, 0.f, 0.f};
    auto compute = [&]() {
#pragma unroll
        for (int ks = 0; ks < KS / 32; ++ks) {
            const int kb = 4 * ks + q;
            h8 bw[2];
#pragma unroll
            for (int jn = 0; jn < 2; ++jn) bw[jn] = *reinterpret_cast<const h8*>(s_w + swz(32 * wv + 16 * jn + c, kb));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const h8 ah = *reinterpret_cast<const h8*>(s_uh + swz(16 * mt + c, kb));
                const h8 al = *reinterpret_cast<const h8*>(s_ul + swz(16 * mt + c, kb));
#pragma unroll
                for (int jn = 0; jn < 2; ++jn) {
                    acc[jn][mt] = mfma32(ah, bw[jn], acc[jn][mt]);
                    acc[jn][mt] = mfma32(al, bw[jn], acc[jn][mt]);
                }
            }
        }
    };
    run_pipeline<D, Stage, 8, true>(0, r / KS, load, store, compute);     // r = 1024: one round
    // lane holds D[token 16 mt + 4 q + i][neuron 32 wv + 16 jn + c]
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
        const int loc = 32 * wv + 16 * jn + c, i = i0 + loc;
        const float bias = (i < n && b2) ? b2[i] : 0.0f;
        unsigned fire = 0;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tok = 16 * mt + 4 * q + e;
                // 1 / uscale is a power of two: the product is exact, one rounding in the add
                const float inv = tok < B ? ldexpf(1.0f, -ilogbf(uscale[tok])) : 1.0f;
                const float lg = fmaf(acc[jn][mt][e], inv, bias);
                if (tok < B) {
                    fire |= lg > thr;
                    if (logits && i < n) logits[(int64_t)tok * n + i] = lg;
                }
            }
        fire |= __shfl_xor(fire, 16, 64);
        fire |= __shfl_xor(fire, 32, 64);
        if (q == 0) s_flag[loc] = (i < n) ? fire : 0u;
    }
    __syncthreads();
    if (wv < P2_ROWS / 64) {
        const int w = blockIdx.x * (P2_ROWS / 64) + wv;
        const uint64_t word = __ballot(s_flag[64 * wv + lane] != 0);
        if (lane == 0 && w < (n + 63) / 64) mask[w] = word;
    }
}

}  // namespace pi
