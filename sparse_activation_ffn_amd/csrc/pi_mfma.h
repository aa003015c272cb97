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
// Both kernels are software-pipelined: the global loads of step s + D are
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

constexpr int MM = 64;          // tokens per tile (batch padded to 64)
constexpr int UR = 128;         // active rows per up workgroup (32 per wave)
constexpr int DC = 128;         // output columns per down workgroup (32 per wave)
constexpr int DK = 128;         // active rows (K) per down step
constexpr int LP = 8;           // LDS row padding in halves (keeps 16-byte alignment)
constexpr int MFMA_WG = 256;    // threads of both kernels (4 waves)

__device__ __forceinline__ f4m mfma32(h8 a, h8 b, f4m c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Two 4-bit codes (bits 0..3 and 16..19 of v) -> two f16 values (q - 8) * s,
// each rounded once: 0x6400 | q is the f16 1024 + q, and 1024 + q - 1032 is exact.
__device__ __forceinline__ unsigned q4_pair(unsigned v, h2v s2) {
    const unsigned bits = (v & 0x000f000fu) | 0x64006400u;
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
        const unsigned a01 = __builtin_amdgcn_perm(0u, w[p], 0x0c010c00u);   // bytes 0, 1
        const unsigned a23 = __builtin_amdgcn_perm(0u, w[p], 0x0c030c02u);   // bytes 2, 3
        lo[2 * p] = q4_pair(a01, s2);
        lo[2 * p + 1] = q4_pair(a23, s2);
        hi[2 * p] = q4_pair(a01 >> 4, s2);
        hi[2 * p + 1] = q4_pair(a23 >> 4, s2);
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
        o[2 * p] = q4_pair(__builtin_amdgcn_perm(0u, w[p], 0x0c010c00u), s2);
        o[2 * p + 1] = q4_pair(__builtin_amdgcn_perm(0u, w[p], 0x0c030c02u), s2);
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
// the freed registers while the matrix cores work on step s.
template <int D, typename Stage, typename Load, typename Store, typename Compute>
__device__ __forceinline__ void run_pipeline(int s0, int s1, Load load, Store store, Compute compute) {
    Stage R[D];
#pragma unroll
    for (int dd = 0; dd < D; ++dd)
        if (s0 + dd < s1) load(R[dd], s0 + dd);
    for (int sb = s0; sb < s1; sb += D) {
#pragma unroll
        for (int dd = 0; dd < D; ++dd) {
            const int s = sb + dd;
            if (s < s1) {
                __syncthreads();                      // the previous step's LDS reads are done
                store(R[dd]);
                if (s + D < s1) load(R[dd], s + D);
                __syncthreads();
                compute();
            }
        }
    }
}

// ===========================================================================
// Up/gate.  Workgroup = 4 waves; tile = 64 tokens x 128 items (32 per wave).
// A step stages K = CH chunks of every row (Q4_0: CH blocks of 32; f16: CH x 8
// elements) and the matching 64 x K slice of x.  With a mask the workgroup
// scans it (all of it, in LDS) and resolves its own 128 items; workgroup 0
// writes the counts and every workgroup its items of the ascending lists.
// Writes h (f16) [B][h_ld] at h_pos(item).
// ===========================================================================
template <int WT, int NM> struct UpShape {
    static constexpr int EPC = WT == Q4 ? 32 : 8;      // weights per 16-byte chunk
    static constexpr int CH = WT == Q4 ? 4 : 8;        // chunks per row per step
    static constexpr int UK = CH * EPC;                // K per step (128 or 64)
    static constexpr int J = UR * CH / MFMA_WG;        // chunks per thread per matrix
    static constexpr int XJ = MM * UK / 8 / MFMA_WG;   // 16-byte x loads per thread
    static constexpr int D = 3;                        // steps in flight
};

template <int WT, int ACT>
__global__ __launch_bounds__(MFMA_WG) void k_mfma_up(FfnArgs a, _Float16* __restrict__ h16) {
    constexpr int NM = ACT == REGLU ? 2 : 1;
    using S = UpShape<WT, NM>;
    constexpr int UK = S::UK, CH = S::CH, J = S::J, XJ = S::XJ, D = S::D;
    __shared__ __attribute__((aligned(16))) _Float16 s_x[MM][UK + LP];
    __shared__ __attribute__((aligned(16))) _Float16 s_w[NM][UR][UK + LP];
    __shared__ int s_row[UR];
    __shared__ int s_part[UR];
    __shared__ int s_cnt[2];
    extern __shared__ uint64_t s_words[];        // mask words (mask mode only)
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int q = lane >> 4, c = lane & 15;
    const int i0 = blockIdx.x * UR;

    int H, C;
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
        int inc = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(inc, o, 64);
            if (lane >= o) inc += v;
        }
        if (lane == 63) s_wtot[wv] = inc;
        __syncthreads();
        int before = 0, T = 0;
#pragma unroll
        for (int w = 0; w < MFMA_WG / 64; ++w) {
            before += w < wv ? s_wtot[w] : 0;
            T += s_wtot[w];
        }
        const int run0 = before + inc - tot;              // rank of this thread's first set bit
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
        if (blockIdx.x == 0 && tid == 0) {
            a.out_counts[0] = H;
            a.out_counts[1] = C;
        }
        // emit the set bits with ranks in [i0, i0 + UR)
        const int ge = min(T, i0 + UR);
        int r0 = run0;
        for (int w = w0; w < min(words, w0 + per); ++w) {
            uint64_t v = s_words[w];
            const int pc = __popcll(v);
            if (pc > 0 && r0 < ge && r0 + pc > i0) {
                const int skip = max(0, i0 - r0);
                if (skip > 0) v &= ~((1ull << select_bit(v, skip)) - 1ull);
                for (int rank = r0 + skip; v != 0 && rank < ge; ++rank) {
                    const int id = 64 * w + __builtin_ctzll(v);
                    v &= v - 1ull;
                    const int part = rank < H ? 0 : 1;
                    const int row = part == 0 ? id : id - nhot;
                    const bool ok = (unsigned)row < (unsigned)a.rows[part];
                    s_row[rank - i0] = ok ? row : -1;
                    s_part[rank - i0] = part;
                    a.out_idx[part][part == 0 ? rank : rank - H] = row;
                }
            }
            r0 += pc;
        }
        __syncthreads();
    } else {
        item_counts(a, H, C);
        if (i0 >= H + C) return;                          // whole workgroup, uniformly
        if (tid < UR) {
            const int item = min(i0 + tid, H + C - 1);
            int part, row;
            item_row(a, item, H, part, row);
            if ((unsigned)row >= (unsigned)a.rows[part]) row = -1;
            s_row[tid] = i0 + tid < H + C ? row : -1;
            s_part[tid] = part;
        }
        __syncthreads();
    }
    const int T = H + C;
    if (i0 >= T) return;                                  // whole workgroup, uniformly

    // per-thread weight sources: chunk j of matrix g is (row r = t / CH, chunk t % CH)
    const uint8_t* src[NM][J];
    bool live[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int t = tid + MFMA_WG * j, r = t / CH;
        const int row = s_row[r], part = s_part[r];
        live[j] = row >= 0;
        // a row that is not one (an out-of-range id) reads row 0 of a partition
        // that has rows, and its weights are zeroed
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
        const int k0 = s * UK;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int ch = (tid + MFMA_WG * j) % CH;
#pragma unroll
            for (int g = 0; g < NM; ++g) {
                if (WT == Q4) {
                    const int blk = k0 / 32 + ch;
                    R.w[g][j] = ld16_stream(src[g][j] + 16 * (int64_t)blk);
                    R.sc[g][j] = __builtin_bit_cast(
                        _Float16, *reinterpret_cast<const uint16_t*>(src[g][j] + a.d / 2 + 2 * (int64_t)blk));
                } else {
                    R.w[g][j] = ld16_stream(src[g][j] + 2 * (int64_t)(k0 + 8 * ch));
                }
            }
        }
#pragma unroll
        for (int j = 0; j < XJ; ++j) {
            const int t = tid + MFMA_WG * j, m = t / (UK / 8), e = (t % (UK / 8)) * 8;
            R.xv[j] = m < a.B ? ld16(a.x + ((int64_t)m * a.d + k0 + e) * 2) : u4{0u, 0u, 0u, 0u};
        }
    };
    auto store = [&](const Stage& R) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int t = tid + MFMA_WG * j, r = t / CH, ch = t % CH;
#pragma unroll
            for (int g = 0; g < NM; ++g) {
                if (WT == Q4) {
                    u4 o[4];
                    deq_block(R.w[g][j], live[j] ? R.sc[g][j] : (_Float16)0.0f, o);
#pragma unroll
                    for (int p = 0; p < 4; ++p) *reinterpret_cast<u4*>(&s_w[g][r][32 * ch + 8 * p]) = o[p];
                } else {
                    *reinterpret_cast<u4*>(&s_w[g][r][8 * ch]) = live[j] ? R.w[g][j] : u4{0u, 0u, 0u, 0u};
                }
            }
        }
#pragma unroll
        for (int j = 0; j < XJ; ++j) {
            const int t = tid + MFMA_WG * j, m = t / (UK / 8), e = (t % (UK / 8)) * 8;
            *reinterpret_cast<u4*>(&s_x[m][e]) = R.xv[j];
        }
    };
    f4m acc[NM][2][4];
#pragma unroll
    for (int g = 0; g < NM; ++g)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) acc[g][jn][mt] = f4m{0.f, 0.f, 0.f, 0.f};
    auto compute = [&]() {
#pragma unroll
        for (int ks = 0; ks < UK / 32; ++ks) {
            const int kk = 32 * ks + 8 * q;
            h8 ax[4], bw[NM][2];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) ax[mt] = *reinterpret_cast<const h8*>(&s_x[16 * mt + c][kk]);
#pragma unroll
            for (int g = 0; g < NM; ++g)
#pragma unroll
                for (int jn = 0; jn < 2; ++jn)
                    bw[g][jn] = *reinterpret_cast<const h8*>(&s_w[g][32 * wv + 16 * jn + c][kk]);
#pragma unroll
            for (int g = 0; g < NM; ++g)
#pragma unroll
                for (int jn = 0; jn < 2; ++jn)
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) acc[g][jn][mt] = mfma32(ax[mt], bw[g][jn], acc[g][jn][mt]);
        }
    };
    run_pipeline<D, Stage>(0, a.d / UK, load, store, compute);
    // epilogue: lane holds D[token 16 mt + 4 q + i][item 32 wv + 16 jn + c]
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
        const int r = 32 * wv + 16 * jn + c;
        const int row = s_row[r], part = s_part[r];
        const int item = i0 + r;
        if (item < T) {
            const int hp = h_pos(item, H);
            const float bu = (row >= 0 && a.bup[part]) ? a.bup[part][row] : 0.0f;
            const float bg = (ACT == REGLU && row >= 0 && a.bgate[part]) ? a.bgate[part][row] : 0.0f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = 16 * mt + 4 * q + i;
                    if (tok < a.B) {
                        const float up = acc[0][jn][mt][i] + bu;
                        float hv;
                        if (ACT == RELU) {
                            hv = up > 0.0f ? up : 0.0f;
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
// stages 128 rows x 128 columns of W_downT and the 64 x 128 tile of h.  Each
// thread loads an 8 x 8 block of weights (8 rows x 16 bytes) and transposes it
// in registers, so every LDS column holds 8 consecutive rows in 16 bytes; the
// column's 16-byte blocks are XOR-swizzled so both the stores and the MFMA
// reads are free of bank conflicts.
// ===========================================================================
__device__ __forceinline__ int wt_off(int col, int kb) {          // halves
    return col * DK + 8 * (kb ^ ((col & 15) ^ ((col >> 3) & 15)));
}

template <int WT> struct DownShape {
    static constexpr int HJ = MM * DK / 8 / MFMA_WG;  // 16-byte h loads per thread
    static constexpr int D = WT == Q4 ? 3 : 2;        // steps in flight
};

template <int WT>
__global__ __launch_bounds__(MFMA_WG) void k_mfma_down(FfnArgs a, DownOut o, const _Float16* __restrict__ h16) {
    using S = DownShape<WT>;
    constexpr int HJ = S::HJ, D = S::D;
    __shared__ __attribute__((aligned(16))) _Float16 s_h[MM][DK + LP];
    __shared__ __attribute__((aligned(16))) _Float16 s_wt[DC * DK];       // [column][k], swizzled
    __shared__ __attribute__((aligned(16))) int s_ids[D + 1][DK];        // row ids of upcoming steps
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int q = lane >> 4, c = lane & 15;
    const int c0 = blockIdx.x * DC, k = blockIdx.y;
    int H, C;
    item_counts(a, H, C);
    int part, lo, hi;
    chunk_range8(o.nch, H, C, k, part, lo, hi);
    const int hb = part == 0 ? 0 : round8(H);         // h buffer offset of this partition
    const uint8_t* base = part == 0 ? a.down[0] : a.down[1];
    const int32_t* idx = part == 0 ? a.idx[0] : a.idx[1];
    const int prows = part == 0 ? a.rows[0] : a.rows[1];
    const int steps = (hi - lo + DK - 1) / DK;
    // this thread's 8 x 8 weight block: rows 8 rg .. +7 of the step, columns 8 cg .. +7
    const int cg = tid & 15, rg = tid >> 4;
    const int col0 = c0 + 8 * cg;
    // row id of step-relative item tid of step s (threads tid < DK), or -1
    auto row_id = [&](int s) -> int {
        const int item = lo + s * DK + tid;
        if (tid >= DK || item >= hi) return -1;
        const int row = idx ? idx[item] : item;
        return (unsigned)row < (unsigned)prows ? row : -1;
    };
    struct Stage {
        u4 w[8];                      // f16: 8 columns of each of 8 rows
        u2 cq[8];                     // Q4_0: 8 codes of each of 8 rows
        _Float16 sc[8];
        u4 hv[HJ];
    };
    // loads of step s; its row ids are in s_ids[s % (D + 1)]
    auto load = [&](Stage& R, int s) {
        const int* ids = s_ids[s % (D + 1)];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int row = ids[8 * rg + r];
            const uint8_t* rowp = base + (int64_t)(row >= 0 ? row : 0) * a.rb;
            if (WT == Q4) {
                const int blk = col0 >> 5, t0 = col0 & 31;
                R.cq[r] = *reinterpret_cast<const u2*>(rowp + 16 * (int64_t)blk + (t0 & 15));
                const _Float16 sv = __builtin_bit_cast(
                    _Float16, *reinterpret_cast<const uint16_t*>(rowp + a.d / 2 + 2 * (int64_t)blk));
                R.sc[r] = row >= 0 ? sv : (_Float16)0.0f;
            } else {
                const u4 v = ld16_stream(rowp + 2 * (int64_t)col0);
                R.w[r] = row >= 0 ? v : u4{0u, 0u, 0u, 0u};
            }
        }
        const int i0 = lo + s * DK;
#pragma unroll
        for (int j = 0; j < HJ; ++j) {
            const int t = tid + MFMA_WG * j, m = t / (DK / 8), e = (t % (DK / 8)) * 8;
            u4 v = u4{0u, 0u, 0u, 0u};
            if (m < a.B && i0 + e < hi) {
                v = ld16(h16 + (int64_t)m * a.h_ld + hb + i0 + e);
                const int valid = hi - (i0 + e);           // items past hi are zero
                if (valid < 8) {
                    unsigned w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        if (2 * p >= valid) w4[p] = 0u;
                        else if (2 * p + 1 >= valid) w4[p] &= 0xffffu;
                    }
                    v = u4{w4[0], w4[1], w4[2], w4[3]};
                }
            }
            R.hv[j] = v;
        }
    };
    auto store = [&](const Stage& R) {
        unsigned V[8][4];                               // V[r][p] = columns 2p, 2p+1 of row r
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            u4 w;
            if (WT == Q4) w = deq8(R.cq[r], R.sc[r], (col0 & 31) >= 16);
            else w = R.w[r];
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
            *reinterpret_cast<u4*>(&s_wt[wt_off(8 * cg + cc, rg)]) = out;
        }
#pragma unroll
        for (int j = 0; j < HJ; ++j) {
            const int t = tid + MFMA_WG * j, m = t / (DK / 8), e = (t % (DK / 8)) * 8;
            *reinterpret_cast<u4*>(&s_h[m][e]) = R.hv[j];
        }
    };
    f4m acc[2][4];
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[jn][mt] = f4m{0.f, 0.f, 0.f, 0.f};
    auto compute = [&]() {
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
            h8 ah[4], bw[2];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                ah[mt] = *reinterpret_cast<const h8*>(&s_h[16 * mt + c][32 * ks + 8 * q]);
#pragma unroll
            for (int jn = 0; jn < 2; ++jn)
                bw[jn] = *reinterpret_cast<const h8*>(&s_wt[wt_off(32 * wv + 16 * jn + c, 4 * ks + q)]);
#pragma unroll
            for (int jn = 0; jn < 2; ++jn)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) acc[jn][mt] = mfma32(ah[mt], bw[jn], acc[jn][mt]);
        }
    };
    // prologue: ids of the first D steps, then their loads; the id of step D is
    // loaded into a register (ids run one step ahead of the weights, and each id
    // load is issued before the weight loads it must not wait behind)
#pragma unroll
    for (int dd = 0; dd < D; ++dd)
        if (tid < DK) s_ids[dd][tid] = row_id(dd);
    __syncthreads();
    int nid = row_id(D);
    Stage R[D];
#pragma unroll
    for (int dd = 0; dd < D; ++dd)
        if (dd < steps) load(R[dd], dd);
    for (int s0 = 0; s0 < steps; s0 += D) {
#pragma unroll
        for (int dd = 0; dd < D; ++dd) {
            const int s = s0 + dd;
            if (s < steps) {
                __syncthreads();                      // the previous step's LDS reads are done
                store(R[dd]);
                if (tid < DK) s_ids[(s + D) % (D + 1)][tid] = nid;
                __syncthreads();
                if (s + D < steps) {
                    nid = row_id(s + D + 1);
                    load(R[dd], s + D);
                }
                compute();
            }
        }
    }
    // partial of y: lane holds D[token 16 mt + 4 q + i][column 32 wv + 16 jn + c]
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
        const int col = c0 + 32 * wv + 16 * jn + c;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
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
constexpr int PUK = 64;         // K per step (8 chunks of 8 f16 per row)

__global__ __launch_bounds__(MFMA_WG) void k_mfma_pred1(const uint8_t* __restrict__ P1t,
                                                       const uint8_t* __restrict__ x, int d, int r,
                                                       int B, float* __restrict__ part) {
    constexpr int J = P1_ROWS * (PUK / 8) / MFMA_WG;  // 16-byte weight loads per thread
    constexpr int XJ = MM * PUK / 8 / MFMA_WG;        // 16-byte x loads per thread
    constexpr int D = 3;
    __shared__ __attribute__((aligned(16))) _Float16 s_x[MM][PUK + LP];
    __shared__ __attribute__((aligned(16))) _Float16 s_w[P1_ROWS][PUK + LP];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int q = lane >> 4, c = lane & 15;
    const int j0 = blockIdx.x * P1_ROWS, ky = blockIdx.y;
    const int64_t rb = (int64_t)d * 2;
    const uint8_t* src[J];
    bool live[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int row = j0 + (tid + MFMA_WG * j) / (PUK / 8);
        live[j] = row < r;
        src[j] = P1t + (int64_t)(row < r ? row : 0) * rb;
    }
    struct Stage {
        u4 w[J];
        u4 xv[XJ];
    };
    auto load = [&](Stage& R, int s) {
        const int k0 = s * PUK;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int ch = (tid + MFMA_WG * j) % (PUK / 8);
            R.w[j] = ld16_stream(src[j] + 2 * (int64_t)(k0 + 8 * ch));
        }
#pragma unroll
        for (int j = 0; j < XJ; ++j) {
            const int t = tid + MFMA_WG * j, m = t / (PUK / 8), e = (t % (PUK / 8)) * 8;
            R.xv[j] = m < B ? ld16(x + ((int64_t)m * d + k0 + e) * 2) : u4{0u, 0u, 0u, 0u};
        }
    };
    auto store = [&](const Stage& R) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int t = tid + MFMA_WG * j, rr = t / (PUK / 8), ch = t % (PUK / 8);
            *reinterpret_cast<u4*>(&s_w[rr][8 * ch]) = live[j] ? R.w[j] : u4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < XJ; ++j) {
            const int t = tid + MFMA_WG * j, m = t / (PUK / 8), e = (t % (PUK / 8)) * 8;
            *reinterpret_cast<u4*>(&s_x[m][e]) = R.xv[j];
        }
    };
    f4m acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = f4m{0.f, 0.f, 0.f, 0.f};
    auto compute = [&]() {
#pragma unroll
        for (int ks = 0; ks < PUK / 32; ++ks) {
            const int kk = 32 * ks + 8 * q;
            const h8 bw = *reinterpret_cast<const h8*>(&s_w[16 * wv + c][kk]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc[mt] = mfma32(*reinterpret_cast<const h8*>(&s_x[16 * mt + c][kk]), bw, acc[mt]);
        }
    };
    const int steps = d / PUK;
    run_pipeline<D, Stage>(ky * steps / P1_KS, (ky + 1) * steps / P1_KS, load, store, compute);
    // lane holds D[token 16 mt + 4 q + i][row 16 wv + c]
    const int row = j0 + 16 * wv + c;
    if (row < r) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 16 * mt + 4 * q + i;
                if (tok < B) part[((int64_t)ky * B + tok) * r + row] = acc[mt][i];
            }
    }
}

// u = ReLU(sum of the P1_KS slice partials, in slice order); 4 outputs per thread.
__global__ __launch_bounds__(THREADS) void k_u_relu(const float* __restrict__ part, int64_t len,
                                                    float* __restrict__ u) {
    const int64_t len4 = len / 4;
    const f4* P = reinterpret_cast<const f4*>(part);
    for (int64_t t = (int64_t)blockIdx.x * THREADS + threadIdx.x; t < len4; t += (int64_t)gridDim.x * THREADS) {
        f4 v[P1_KS];
#pragma unroll
        for (int k = 0; k < P1_KS; ++k) v[k] = P[k * len4 + t];
        f4 sum = v[0];
#pragma unroll
        for (int k = 1; k < P1_KS; ++k) {
            sum.x += v[k].x; sum.y += v[k].y; sum.z += v[k].z; sum.w += v[k].w;
        }
        reinterpret_cast<f4*>(u)[t] = f4{sum.x > 0.f ? sum.x : 0.f, sum.y > 0.f ? sum.y : 0.f,
                                         sum.z > 0.f ? sum.z : 0.f, sum.w > 0.f ? sum.w : 0.f};
    }
}

// ===========================================================================
// Second layer + threshold + union over tokens: logits = u P2 + b2 on matrix
// cores, 128 neurons (two mask words) per workgroup.  u is fp32; it enters the
// matrix cores as the sum of two f16 parts (hi = f16(u), lo = f16(u - hi)),
// whose products with the f16 weights are exact, so the logits keep fp32
// accuracy and the threshold decisions match the fp32 path.
// ===========================================================================
constexpr int P2_ROWS = 128;    // neurons per workgroup (32 per wave)

__global__ __launch_bounds__(MFMA_WG) void k_mfma_pred2(const uint8_t* __restrict__ P2t,
                                                       const float* __restrict__ b2, float thr,
                                                       const float* __restrict__ u, int n, int r,
                                                       int B, uint64_t* __restrict__ mask,
                                                       float* __restrict__ logits) {
    constexpr int J = P2_ROWS * (PUK / 8) / MFMA_WG;  // 16-byte weight loads per thread
    constexpr int UJ = MM * PUK / 4 / MFMA_WG;        // 16-byte (4 float) u loads per thread
    constexpr int D = 3;
    __shared__ __attribute__((aligned(16))) _Float16 s_uh[MM][PUK + LP];
    __shared__ __attribute__((aligned(16))) _Float16 s_ul[MM][PUK + LP];
    __shared__ __attribute__((aligned(16))) _Float16 s_w[P2_ROWS][PUK + LP];
    __shared__ unsigned s_flag[P2_ROWS];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int q = lane >> 4, c = lane & 15;
    const int i0 = blockIdx.x * P2_ROWS;
    const int64_t rb = (int64_t)r * 2;
    const uint8_t* src[J];
    bool live[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int row = i0 + (tid + MFMA_WG * j) / (PUK / 8);
        live[j] = row < n;
        src[j] = P2t + (int64_t)(row < n ? row : 0) * rb;
    }
    struct Stage {
        u4 w[J];
        f4 uv[UJ];
    };
    auto load = [&](Stage& R, int s) {
        const int k0 = s * PUK;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int ch = (tid + MFMA_WG * j) % (PUK / 8);
            R.w[j] = ld16_stream(src[j] + 2 * (int64_t)(k0 + 8 * ch));
        }
#pragma unroll
        for (int j = 0; j < UJ; ++j) {
            const int t = tid + MFMA_WG * j, m = t / (PUK / 4), e = (t % (PUK / 4)) * 4;
            R.uv[j] = m < B ? *reinterpret_cast<const f4*>(u + (int64_t)m * r + k0 + e) : f4{0.f, 0.f, 0.f, 0.f};
        }
    };
    auto store = [&](const Stage& R) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int t = tid + MFMA_WG * j, rr = t / (PUK / 8), ch = t % (PUK / 8);
            *reinterpret_cast<u4*>(&s_w[rr][8 * ch]) = live[j] ? R.w[j] : u4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < UJ; ++j) {
            const int t = tid + MFMA_WG * j, m = t / (PUK / 4), e = (t % (PUK / 4)) * 4;
            const float v[4] = {R.uv[j].x, R.uv[j].y, R.uv[j].z, R.uv[j].w};
            _Float16 hi[4], lo[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                hi[p] = (_Float16)v[p];
                lo[p] = (_Float16)(v[p] - (float)hi[p]);
            }
            *reinterpret_cast<u2*>(&s_uh[m][e]) =
                u2{(unsigned)__builtin_bit_cast(uint16_t, hi[0]) | ((unsigned)__builtin_bit_cast(uint16_t, hi[1]) << 16),
                   (unsigned)__builtin_bit_cast(uint16_t, hi[2]) | ((unsigned)__builtin_bit_cast(uint16_t, hi[3]) << 16)};
            *reinterpret_cast<u2*>(&s_ul[m][e]) =
                u2{(unsigned)__builtin_bit_cast(uint16_t, lo[0]) | ((unsigned)__builtin_bit_cast(uint16_t, lo[1]) << 16),
                   (unsigned)__builtin_bit_cast(uint16_t, lo[2]) | ((unsigned)__builtin_bit_cast(uint16_t, lo[3]) << 16)};
        }
    };
    f4m acc[2][4];
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[jn][mt] = f4m{0.f, 0.f, 0.f, 0.f};
    auto compute = [&]() {
#pragma unroll
        for (int ks = 0; ks < PUK / 32; ++ks) {
            const int kk = 32 * ks + 8 * q;
            h8 bw[2];
#pragma unroll
            for (int jn = 0; jn < 2; ++jn) bw[jn] = *reinterpret_cast<const h8*>(&s_w[32 * wv + 16 * jn + c][kk]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const h8 ah = *reinterpret_cast<const h8*>(&s_uh[16 * mt + c][kk]);
                const h8 al = *reinterpret_cast<const h8*>(&s_ul[16 * mt + c][kk]);
#pragma unroll
                for (int jn = 0; jn < 2; ++jn) {
                    acc[jn][mt] = mfma32(ah, bw[jn], acc[jn][mt]);
                    acc[jn][mt] = mfma32(al, bw[jn], acc[jn][mt]);
                }
            }
        }
    };
    run_pipeline<D, Stage>(0, r / PUK, load, store, compute);
    // lane holds D[token 16 mt + 4 q + i][neuron 32 wv + 16 jn + c]
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
        const int loc = 32 * wv + 16 * jn + c, i = i0 + loc;
        const float bias = (i < n && b2) ? b2[i] : 0.0f;
        unsigned fire = 0;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tok = 16 * mt + 4 * q + e;
                const float lg = acc[jn][mt][e] + bias;
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
