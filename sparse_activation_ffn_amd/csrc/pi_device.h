// pi_device.h -- device helpers of the sparse-FFN kernels for gfx950 (CDNA4, wave64).
//
// A weight row is read in 16-byte "chunks" with one 16-byte load per lane, so a
// wave moves 1 KiB per load instruction and every 128-byte line it touches is
// used whole.  Elements per chunk: f32 4, f16 8, Q4_0 32 (16 code bytes plus
// the block's fp16 scale, which sits in the row's scale plane).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pi {

constexpr int WAVE = 64;
enum { F32 = 0, F16 = 1, Q4 = 2 };
enum { RELU = 0, REGLU = 1, SQRELU = 2 };   // activations (SQRELU: max(0, a)^2)

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

// Weight streams are read once per step: non-temporal loads by default.
#ifndef PI_WEIGHT_NT
#define PI_WEIGHT_NT 1
#endif
__device__ __forceinline__ u4 ld16_stream(const void* p) {
#if PI_WEIGHT_NT
    return __builtin_nontemporal_load(reinterpret_cast<const u4*>(p));
#else
    return *reinterpret_cast<const u4*>(p);
#endif
}
__device__ __forceinline__ u4 ld16(const void* p) { return *reinterpret_cast<const u4*>(p); }
__device__ __forceinline__ u2 ld8_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u2*>(p));
}
__device__ __forceinline__ float bits_f(unsigned v) { return __builtin_bit_cast(float, v); }
__device__ __forceinline__ h2 bits_h2(unsigned v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ float half_lo(unsigned v) { return (float)bits_h2(v).x; }
__device__ __forceinline__ float half_hi(unsigned v) { return (float)bits_h2(v).y; }
__device__ __forceinline__ float half_f(uint16_t v) { return (float)__builtin_bit_cast(_Float16, v); }

// Row bytes of one neuron's row of d elements.
__host__ __device__ __forceinline__ int64_t row_bytes(int wt, int64_t d) {
    return wt == F32 ? 4 * d : wt == F16 ? 2 * d : d / 2 + d / 16;
}

// ---- dot products of one weight chunk with the matching x elements ---------
//
// x is read from `xp`, which points at the chunk's first x element of one
// token (global or LDS memory), stored as float (XT == F32) or half (XT == F16).

template <int WT> struct Chunk;
template <> struct Chunk<F32> { static constexpr int EPC = 4; };
template <> struct Chunk<F16> { static constexpr int EPC = 8; };
template <> struct Chunk<Q4> { static constexpr int EPC = 32; };

template <int WT, int XT> struct Dot;

template <> struct Dot<F32, F32> {
    __device__ static float run(u4 w, float, const void* xp, float acc) {
        f4 x = *reinterpret_cast<const f4*>(xp);
        acc = fmaf(bits_f(w.x), x.x, acc);
        acc = fmaf(bits_f(w.y), x.y, acc);
        acc = fmaf(bits_f(w.z), x.z, acc);
        acc = fmaf(bits_f(w.w), x.w, acc);
        return acc;
    }
};

template <> struct Dot<F32, F16> {
    __device__ static float run(u4 w, float, const void* xp, float acc) {
        u2 x = *reinterpret_cast<const u2*>(xp);
        acc = fmaf(bits_f(w.x), half_lo(x.x), acc);
        acc = fmaf(bits_f(w.y), half_hi(x.x), acc);
        acc = fmaf(bits_f(w.z), half_lo(x.y), acc);
        acc = fmaf(bits_f(w.w), half_hi(x.y), acc);
        return acc;
    }
};

template <> struct Dot<F16, F16> {
    // half x half products are exact in fp32; v_dot2 adds two of them per op
    __device__ static float run(u4 w, float, const void* xp, float acc) {
        u4 x = *reinterpret_cast<const u4*>(xp);
        acc = __builtin_amdgcn_fdot2(bits_h2(w.x), bits_h2(x.x), acc, false);
        acc = __builtin_amdgcn_fdot2(bits_h2(w.y), bits_h2(x.y), acc, false);
        acc = __builtin_amdgcn_fdot2(bits_h2(w.z), bits_h2(x.z), acc, false);
        acc = __builtin_amdgcn_fdot2(bits_h2(w.w), bits_h2(x.w), acc, false);
        return acc;
    }
};

template <> struct Dot<F16, F32> {
    __device__ static float run(u4 w, float, const void* xp, float acc) {
        const f4* x = reinterpret_cast<const f4*>(xp);
        f4 a = x[0], b = x[1];
        acc = fmaf(half_lo(w.x), a.x, acc);
        acc = fmaf(half_hi(w.x), a.y, acc);
        acc = fmaf(half_lo(w.y), a.z, acc);
        acc = fmaf(half_hi(w.y), a.w, acc);
        acc = fmaf(half_lo(w.z), b.x, acc);
        acc = fmaf(half_hi(w.z), b.y, acc);
        acc = fmaf(half_lo(w.w), b.z, acc);
        acc = fmaf(half_hi(w.w), b.w, acc);
        return acc;
    }
};

// Q4_0 block: code byte t holds element t (low nibble) and t + 16 (high nibble).
// Two codes go into one half2 as 1024 + q (exponent 10, so the integer is exact),
// and subtracting 1032 leaves q - 8 exactly; v_dot2 then takes two products.
// This integer-to-half conversion by OR-ing codes into the mantissa of a
// power-of-two constant is the published "magic number" method for 4-bit
// weights (Kim et al., arXiv 2211.10017, fast int4-to-fp16 conversion).
// q4_pair takes the two halves already as 0x640q.
__device__ __forceinline__ h2 q4_pair(unsigned halves_0x640q) {
    return bits_h2(halves_0x640q) - h2{(_Float16)1032.0f, (_Float16)1032.0f};
}

template <> struct Dot<Q4, F16> {
    // w: 16 code bytes of one block; s: the block's scale; xp: 32 halves
    __device__ static float run(u4 w, float s, const void* xp, float acc) {
        const u4* xv = reinterpret_cast<const u4*>(xp);
        u4 xl0 = xv[0], xl1 = xv[1], xh0 = xv[2], xh1 = xv[3];
        unsigned cw[4] = {w.x, w.y, w.z, w.w};
        unsigned xl[8] = {xl0.x, xl0.y, xl0.z, xl0.w, xl1.x, xl1.y, xl1.z, xl1.w};
        unsigned xh[8] = {xh0.x, xh0.y, xh0.z, xh0.w, xh1.x, xh1.y, xh1.z, xh1.w};
        float blk = 0.0f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            // bytes (0,1) and (2,3) of code dword m into the two halves, each as
            // 0x64 above its byte (one permute: the 0x64 bytes come from the
            // constant operand), then the low nibble kept; the high nibbles the
            // same way from the dword shifted by 4
            const unsigned ws = cw[m] >> 4;
            const unsigned l01 = __builtin_amdgcn_perm(0x64646464u, cw[m], 0x04010400u) & 0xff0fff0fu;
            const unsigned l23 = __builtin_amdgcn_perm(0x64646464u, cw[m], 0x04030402u) & 0xff0fff0fu;
            const unsigned h01 = __builtin_amdgcn_perm(0x64646464u, ws, 0x04010400u) & 0xff0fff0fu;
            const unsigned h23 = __builtin_amdgcn_perm(0x64646464u, ws, 0x04030402u) & 0xff0fff0fu;
            blk = __builtin_amdgcn_fdot2(q4_pair(l01), bits_h2(xl[2 * m]), blk, false);
            blk = __builtin_amdgcn_fdot2(q4_pair(l23), bits_h2(xl[2 * m + 1]), blk, false);
            blk = __builtin_amdgcn_fdot2(q4_pair(h01), bits_h2(xh[2 * m]), blk, false);
            blk = __builtin_amdgcn_fdot2(q4_pair(h23), bits_h2(xh[2 * m + 1]), blk, false);
        }
        return fmaf(blk, s, acc);
    }
};

template <> struct Dot<Q4, F32> {
    __device__ static float run(u4 w, float s, const void* xp, float acc) {
        const float* x = reinterpret_cast<const float*>(xp);
        unsigned cw[4] = {w.x, w.y, w.z, w.w};
        float blk = 0.0f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            unsigned byte = (cw[t >> 2] >> (8 * (t & 3))) & 0xffu;
            blk = fmaf((float)(int)(byte & 15u) - 8.0f, x[t], blk);
            blk = fmaf((float)(int)(byte >> 4) - 8.0f, x[t + 16], blk);
        }
        return fmaf(blk, s, acc);
    }
};

// ---- axpy of one weight chunk into per-lane accumulators (down projection) --
//
// The down kernel gives each lane DCH consecutive columns of a row:
// f32 4 (16 B), f16 8 (16 B), Q4_0 16 (8 code bytes = half a block: elements
// k0..k0+7 and k0+16..k0+23 of the block, k0 = 0 or 8, plus the block scale).

template <int WT> struct Down;

template <> struct Down<F32> {
    static constexpr int DCH = 4;     // columns per lane
    static constexpr int COLS = 256;  // columns per wave-wide slice
    typedef u4 raw;
    __device__ static raw load(const uint8_t* row, int64_t d, int col0) {
        return ld16_stream(row + 4 * (int64_t)col0);
    }
    __device__ static void axpy(raw w, float h, float* acc) {
        acc[0] = fmaf(h, bits_f(w.x), acc[0]);
        acc[1] = fmaf(h, bits_f(w.y), acc[1]);
        acc[2] = fmaf(h, bits_f(w.z), acc[2]);
        acc[3] = fmaf(h, bits_f(w.w), acc[3]);
    }
    // a value whose axpy adds exact zeros whatever h is
    __device__ static raw zero() { return u4{0u, 0u, 0u, 0u}; }
    // column of accumulator e, relative to the lane's first column
    __device__ static int col(int e) { return e; }
};

template <> struct Down<F16> {
    static constexpr int DCH = 8;
    static constexpr int COLS = 512;
    typedef u4 raw;
    __device__ static raw load(const uint8_t* row, int64_t d, int col0) {
        return ld16_stream(row + 2 * (int64_t)col0);
    }
    __device__ static void axpy(raw w, float h, float* acc) {
        acc[0] = fmaf(h, half_lo(w.x), acc[0]);
        acc[1] = fmaf(h, half_hi(w.x), acc[1]);
        acc[2] = fmaf(h, half_lo(w.y), acc[2]);
        acc[3] = fmaf(h, half_hi(w.y), acc[3]);
        acc[4] = fmaf(h, half_lo(w.z), acc[4]);
        acc[5] = fmaf(h, half_hi(w.z), acc[5]);
        acc[6] = fmaf(h, half_lo(w.w), acc[6]);
        acc[7] = fmaf(h, half_hi(w.w), acc[7]);
    }
    __device__ static raw zero() { return u4{0u, 0u, 0u, 0u}; }
    __device__ static int col(int e) { return e; }
};

struct Q4Half { u2 codes; float scale; };

template <> struct Down<Q4> {
    static constexpr int DCH = 16;
    static constexpr int COLS = 1024;   // 32 blocks, two lanes per block
    typedef Q4Half raw;
    // col0 = first column of this lane's half block: 32*j + k0 with k0 in {0, 8}
    __device__ static raw load(const uint8_t* row, int64_t d, int col0) {
        int j = col0 >> 5, k0 = col0 & 31;
        Q4Half r;
        r.codes = ld8_stream(row + 16 * (int64_t)j + k0);
        r.scale = half_f(*reinterpret_cast<const uint16_t*>(row + d / 2 + 2 * (int64_t)j));
        return r;
    }
    __device__ static void axpy(raw w, float h, float* acc) {
        float hs = h * w.scale;
        unsigned cw[2] = {w.codes.x, w.codes.y};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            unsigned byte = (cw[t >> 2] >> (8 * (t & 3))) & 0xffu;
            acc[t] = fmaf(hs, (float)(int)(byte & 15u) - 8.0f, acc[t]);
            acc[8 + t] = fmaf(hs, (float)(int)(byte >> 4) - 8.0f, acc[8 + t]);
        }
    }
    // codes of 8 (weight 0) with a zero scale
    __device__ static raw zero() {
        Q4Half r;
        r.codes = u2{0x88888888u, 0x88888888u};
        r.scale = 0.0f;
        return r;
    }
    // accumulators 0..7 -> columns k0..k0+7, 8..15 -> columns k0+16..k0+23
    __device__ static int col(int e) { return e < 8 ? e : e + 8; }
};

// ---- reductions ------------------------------------------------------------
//
// Cross-lane sums use DPP (data-parallel primitives: a VALU operand read from
// another lane of the same row of 16 lanes, or broadcast from the last lane of
// a row), so a 64-lane sum is six dependent VALU adds instead of six LDS
// permute round trips.  The order of the additions is fixed: results are
// bit-identical from run to run.

// DPP controls of the GFX9 family (gfx950 included)
constexpr int DPP_QUAD_1032 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_ROW_SHR1 = 0x111;   // row_shr:1 (row_shr:k = 0x110 + k)
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_BCAST15 = 0x142;
constexpr int DPP_ROW_BCAST31 = 0x143;

// v + (v of the lane CTRL selects); rows outside ROW_MASK, and lanes whose
// source lies outside their row, add 0
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float add_dpp(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false);
    return v + __builtin_bit_cast(float, t);
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int add_dpp(int v) {
    return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, false);
}

// sum over each row of 16 lanes, in every lane of the row
template <typename T>
__device__ __forceinline__ T row_sum16(T v) {
    v = add_dpp<DPP_QUAD_1032>(v);            // pairs
    v = add_dpp<DPP_QUAD_2301>(v);            // quads
    v = add_dpp<DPP_ROW_HALF_MIRROR>(v);      // the other quad of the half row
    v = add_dpp<DPP_ROW_MIRROR>(v);           // the other half of the row
    return v;
}

// sum over the wave, in lane 63 only
template <typename T>
__device__ __forceinline__ T wave_sum_last(T v) {
    v = row_sum16(v);
    v = add_dpp<DPP_ROW_BCAST15, 0xA>(v);     // rows 1, 3 += rows 0, 2
    v = add_dpp<DPP_ROW_BCAST31, 0xC>(v);     // rows 2, 3 += rows 0 + 1
    return v;
}

template <int W>
__device__ __forceinline__ float group_sum(float v) {
    // sum over aligned groups of W lanes (W a power of two <= 64), in every lane
    if constexpr (W == 16) {
        return row_sum16(v);
    } else if constexpr (W == WAVE) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_sum_last(v)), WAVE - 1));
    } else {
#pragma unroll
        for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
        return v;
    }
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<WAVE>(v); }

__device__ __forceinline__ int wave_sum_int(int v) {
    return __builtin_amdgcn_readlane(wave_sum_last(v), WAVE - 1);
}

// inclusive prefix sum over the wave (lane i gets lanes 0..i)
__device__ __forceinline__ int wave_incl_scan(int v) {
    v = add_dpp<DPP_ROW_SHR1>(v);             // row_shr 1, 2, 4, 8: Hillis-Steele in each row
    v = add_dpp<DPP_ROW_SHR1 + 1>(v);
    v = add_dpp<DPP_ROW_SHR1 + 3>(v);
    v = add_dpp<DPP_ROW_SHR1 + 7>(v);
    v = add_dpp<DPP_ROW_BCAST15, 0xA>(v);     // rows 1, 3 += last lane of rows 0, 2
    v = add_dpp<DPP_ROW_BCAST31, 0xC>(v);     // rows 2, 3 += last lane of row 1
    return v;
}

}  // namespace pi
