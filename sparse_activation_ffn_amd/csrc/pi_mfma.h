// pi_mfma.h -- matrix-core (MFMA) path of the sparse FFN for batches of 16..64
// tokens on gfx950.
//
// At a prompt-sized batch the union of the tokens' active sets is most of the
// layer, and the gathered FFN is a real contraction: up = X [B x d] . W[rows]^T,
// then y = h [B x T] . W_downT[rows].  Both run on v_mfma_f32_16x16x16_f16 with
// fp32 accumulation; operands are staged in LDS as f16 (Q4_0 weights are
// dequantised to f16 on the way in, h is rounded to f16 once).
//
// MFMA 16x16x16 operand layout (wave64): lane l supplies A[m = l%16][k = 4(l/16)+i]
// and B[k = 4(l/16)+i][n = l%16] for i = 0..3, and receives D[m = 4(l/16)+i][n = l%16].
//
// PowerInfer pages: CSDN article, section on sparse activation (only predicted
// neurons are computed; over a batch the union of the tokens' sets).
#pragma once
#include "pi_kernels.h"

namespace pi {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4m __attribute__((ext_vector_type(4)));

constexpr int MM = 64;          // tokens per tile (batch padded to 64)
constexpr int UR = 64;          // active rows per up workgroup (16 per wave)
constexpr int UK = 128;         // K (model width) staged per up iteration
constexpr int DC = 256;         // output columns per down workgroup (64 per wave)
constexpr int DK = 64;          // active rows (K) staged per down iteration
constexpr int LP = 8;           // LDS row padding in halves (keeps 16-byte alignment)

__device__ __forceinline__ f4m mfma16(h4 a, h4 b, f4m c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// 8 consecutive weights of a row starting at element e (e % 8 == 0), as f16
// (Q4_0: dequantised (q - 8) * s, rounded to f16 once).
template <int WT> struct Deq8;
template <> struct Deq8<F16> {
    __device__ static u4 run(const uint8_t* row, int64_t d, int e) {
        return ld16_stream(row + 2 * (int64_t)e);
    }
};
template <> struct Deq8<Q4> {
    __device__ static u4 run(const uint8_t* row, int64_t d, int e) {
        const int j = e >> 5, t0 = e & 31;               // block, first element in block
        const int byte0 = t0 & 15;                       // code bytes byte0..byte0+7
        const bool hi = t0 >= 16;
        const u2 c = *reinterpret_cast<const u2*>(row + 16 * (int64_t)j + byte0);
        const _Float16 s = __builtin_bit_cast(_Float16,
                                              *reinterpret_cast<const uint16_t*>(row + d / 2 + 2 * (int64_t)j));
        unsigned out[4];
        const unsigned cw[2] = {c.x, c.y};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const unsigned w = cw[p >> 1] >> (16 * (p & 1));      // two code bytes
            const unsigned q0 = hi ? (w >> 4) & 15u : w & 15u;
            const unsigned q1 = hi ? (w >> 12) & 15u : (w >> 8) & 15u;
            const _Float16 v0 = (_Float16)((int)q0 - 8) * s;
            const _Float16 v1 = (_Float16)((int)q1 - 8) * s;
            out[p] = (unsigned)__builtin_bit_cast(uint16_t, v0) |
                     ((unsigned)__builtin_bit_cast(uint16_t, v1) << 16);
        }
        return u4{out[0], out[1], out[2], out[3]};
    }
};

// Up/gate on matrix cores.  Workgroup = 4 waves; tile = 64 tokens x 64 items.
// Writes h (f16) [B][T] token-major for the down kernel.
template <int WT, int ACT>
__global__ __launch_bounds__(256) void k_mfma_up(FfnArgs a, _Float16* __restrict__ h16) {
    constexpr int NM = ACT == REGLU ? 2 : 1;
    __shared__ __attribute__((aligned(16))) _Float16 s_x[MM][UK + LP];
    __shared__ __attribute__((aligned(16))) _Float16 s_w[NM][UR][UK + LP];
    __shared__ int s_row[UR];
    __shared__ int s_part[UR];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int H, C;
    item_counts(a, H, C);
    const int T = H + C;
    const int i0 = blockIdx.x * UR;
    if (i0 >= T) return;
    if (tid < UR) {
        const int item = min(i0 + tid, T - 1);
        int part, row;
        item_row(a, item, H, part, row);
        if ((unsigned)row >= (unsigned)a.rows[part]) row = -1;
        s_row[tid] = i0 + tid < T ? row : -1;
        s_part[tid] = part;
    }
    __syncthreads();
    f4m acc[NM][4];
#pragma unroll
    for (int g = 0; g < NM; ++g)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[g][mt] = f4m{0.f, 0.f, 0.f, 0.f};
    const int q = lane >> 4, nl = lane & 15;
    for (int k0 = 0; k0 < a.d; k0 += UK) {
        // stage x [64 tokens][UK] (tokens >= B are zero) and the rows' weights
        for (int t = tid; t < MM * UK / 8; t += 256) {
            const int m = t / (UK / 8), e = (t % (UK / 8)) * 8;
            u4 v = u4{0u, 0u, 0u, 0u};
            if (m < a.B) v = ld16(a.x + ((int64_t)m * a.d + k0 + e) * 2);
            *reinterpret_cast<u4*>(&s_x[m][e]) = v;
        }
        for (int t = tid; t < UR * UK / 8; t += 256) {
            const int r = t / (UK / 8), e = (t % (UK / 8)) * 8;
            const int row = s_row[r], part = s_part[r];
            const int64_t rr = row < 0 ? 0 : row;
            u4 v = Deq8<WT>::run(a.up[part] + rr * a.rb, a.d, k0 + e);
            if (row < 0) v = u4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u4*>(&s_w[0][r][e]) = v;
            if (ACT == REGLU) {
                u4 g = Deq8<WT>::run(a.gate[part] + rr * a.rb, a.d, k0 + e);
                if (row < 0) g = u4{0u, 0u, 0u, 0u};
                *reinterpret_cast<u4*>(&s_w[NM - 1][r][e]) = g;
            }
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < UK / 16; ++ks) {
            const int kk = ks * 16 + 4 * q;
            h4 bw[NM];
#pragma unroll
            for (int g = 0; g < NM; ++g) bw[g] = *reinterpret_cast<const h4*>(&s_w[g][16 * wv + nl][kk]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const h4 ax = *reinterpret_cast<const h4*>(&s_x[16 * mt + nl][kk]);
#pragma unroll
                for (int g = 0; g < NM; ++g) acc[g][mt] = mfma16(ax, bw[g], acc[g][mt]);
            }
        }
        __syncthreads();
    }
    // epilogue: lane holds D[token 16 mt + 4 q + i][row 16 wv + nl]
    const int r = 16 * wv + nl;
    const int row = s_row[r], part = s_part[r];
    const int item = i0 + r;
    if (row >= 0) {
        const float bu = a.bup[part] ? a.bup[part][row] : 0.0f;
        const float bg = (ACT == REGLU && a.bgate[part]) ? a.bgate[part][row] : 0.0f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 16 * mt + 4 * q + i;
                if (tok < a.B) {
                    const float up = acc[0][mt][i] + bu;
                    float hv;
                    if (ACT == RELU) {
                        hv = up > 0.0f ? up : 0.0f;
                    } else {
                        const float gt = acc[NM - 1][mt][i] + bg;
                        hv = (gt > 0.0f ? gt : 0.0f) * up;
                    }
                    h16[(int64_t)tok * a.h_ld + item] = (_Float16)hv;
                }
            }
        }
    } else if (item < T) {
        for (int tok = q; tok < a.B; tok += 4) h16[(int64_t)tok * a.h_ld + item] = (_Float16)0.0f;
    }
}

// Down on matrix cores, split over K (the active rows): grid (d / 256 column
// tiles, chunks); chunk k covers the items chunk_range gives it (one partition).
// Each wave owns 64 columns (4 n-tiles) for all 64 tokens (4 m-tiles).
template <int WT>
__global__ __launch_bounds__(256) void k_mfma_down(FfnArgs a, DownOut o, const _Float16* __restrict__ h16) {
    __shared__ __attribute__((aligned(16))) _Float16 s_h[MM][DK + LP];
    __shared__ __attribute__((aligned(16))) _Float16 s_wt[DC][DK + LP];   // [column][k]
    __shared__ int s_row[DK];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int q = lane >> 4, nl = lane & 15;
    const int c0 = blockIdx.x * DC, k = blockIdx.y;
    int H, C;
    item_counts(a, H, C);
    int part, lo, hi, nh;
    chunk_range(o.nch, H, C, k, part, lo, hi, nh);
    const int hbase = part == 0 ? 0 : H;
    const uint8_t* base = part == 0 ? a.down[0] : a.down[1];
    const int32_t* idx = part == 0 ? a.idx[0] : a.idx[1];
    const int prows = part == 0 ? a.rows[0] : a.rows[1];
    f4m acc[4][4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[nt][mt] = f4m{0.f, 0.f, 0.f, 0.f};
    for (int s0 = lo; s0 < hi; s0 += DK) {
        const int len = min(DK, hi - s0);
        if (tid < DK) {
            int row = -1;
            if (tid < len) {
                row = idx ? idx[s0 + tid] : s0 + tid;
                if ((unsigned)row >= (unsigned)prows) row = -1;
            }
            s_row[tid] = row;
        }
        // h tile [64 tokens][DK items] (zero past B, past len, and for invalid rows)
        for (int t = tid; t < MM * DK / 8; t += 256) {
            const int m = t / (DK / 8), e = (t % (DK / 8)) * 8;
            u4 v = u4{0u, 0u, 0u, 0u};
            if (m < a.B) {
                const _Float16* src = h16 + (int64_t)m * a.h_ld + hbase + s0 + e;
                unsigned w[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int e0 = e + 2 * p;
                    const uint16_t x0 = e0 < len ? __builtin_bit_cast(uint16_t, src[2 * p]) : 0;
                    const uint16_t x1 = e0 + 1 < len ? __builtin_bit_cast(uint16_t, src[2 * p + 1]) : 0;
                    w[p] = (unsigned)x0 | ((unsigned)x1 << 16);
                }
                v = u4{w[0], w[1], w[2], w[3]};
            }
            *reinterpret_cast<u4*>(&s_h[m][e]) = v;
        }
        __syncthreads();
        // weights [DK rows][DC columns], stored transposed [column][row]
        for (int t = tid; t < DK * DC / 8; t += 256) {
            const int r = t / (DC / 8), e = (t % (DC / 8)) * 8;
            const int row = s_row[r];
            const int col = c0 + e;
            u4 v = u4{0u, 0u, 0u, 0u};
            if (row >= 0 && col < a.d) v = Deq8<WT>::run(base + (int64_t)row * a.rb, a.d, col);
            const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                s_wt[e + 2 * p][r] = __builtin_bit_cast(_Float16, (uint16_t)(w[p] & 0xffffu));
                s_wt[e + 2 * p + 1][r] = __builtin_bit_cast(_Float16, (uint16_t)(w[p] >> 16));
            }
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < DK / 16; ++ks) {
            const int kk = ks * 16 + 4 * q;
            h4 ah[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) ah[mt] = *reinterpret_cast<const h4*>(&s_h[16 * mt + nl][kk]);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const h4 bw = *reinterpret_cast<const h4*>(&s_wt[64 * wv + 16 * nt + nl][kk]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) acc[nt][mt] = mfma16(ah[mt], bw, acc[nt][mt]);
            }
        }
        __syncthreads();
    }
    // partial of y: lane holds D[token 16 mt + 4 q + i][column 64 wv + 16 nt + nl]
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int col = c0 + 64 * wv + 16 * nt + nl;
        if (col < a.d) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = 16 * mt + 4 * q + i;
                    if (tok < a.B) o.partials[((int64_t)k * a.B + tok) * a.d + col] = acc[nt][mt][i];
                }
        }
    }
}

}  // namespace pi
