// Storage formats of the KV pools, as seen by the decode kernels.
//
// Both formats keep the same pool layouts (keys [blocks][K][16][H], values
// [blocks][K][H][16]) and hand the kernels the same matrix-core operands:
// bf16 key rows for the score tiles and bf16 value columns for the P.V
// tiles.  A format fixes the element type, how one 32-token chunk is loaded
// into registers, and how those registers become the bf16 operands.
//
//   KvBf16  the pools hold bf16: operands are the loaded bits.
//   KvFp8   the pools hold OCP FP8 E4M3 codes (the 8-bit cache quantisation
//           named in "Week 11. Inference", step 2, and in the lesson's
//           exercises on FP8 cache capacity), one scale per pool.  Codes are
//           widened to bf16 just before the products; every E4M3 value is a
//           bf16 value, so the widening is exact and the pool scales are
//           applied outside the products (k_scale in the softmax scale,
//           v_scale in the output normalisation).
//
// Chunk geometry shared by both (lane = 16 * quad + col):
//   score tile a (a = 0, 1), row m = col  -> token 8 * (col / 4) + 4a + col % 4
//   P.V tile c, row col                    -> head dim 16c + col,
//                                             tokens 8 * quad .. 8 * quad + 7
// The key dims a lane contributes at k-step s (32 dims per step) are given by
// dim_offset(s, quad); the query fragment uses the same map, so any
// assignment of dims to steps is valid as long as it covers each once.
#pragma once

#include "common.hpp"

namespace pkv {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// p = hi + lo with hi = bf16(p) and lo = bf16(p - hi), for eight values.  hi
// is rounded in pairs; its fp32 value is read back from the packed bits (the
// low half shifted up, the high half masked), not converted value by value.
__device__ __forceinline__ void split_bf16(const float (&p)[8], bf16x8 &hi, bf16x8 &lo)
{
#pragma unroll
    for (int e = 0; e < 8; ++e)
        hi[e] = (__bf16)p[e];
    const u32x4 bits = __builtin_bit_cast(u32x4, hi);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        lo[2 * w] = (__bf16)(p[2 * w] - __uint_as_float(bits[w] << 16));
        lo[2 * w + 1] = (__bf16)(p[2 * w + 1] - __uint_as_float(bits[w] & 0xFFFF0000u));
    }
}

// 8-byte load with the non-temporal hint.
__device__ __forceinline__ u32x2 load8_stream(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
}

struct KvBf16 {
    using Elem = uint16_t;
    // Register-ring depths (chunks resident per wave) of the fixed-partition
    // and token-balanced kernels: a bf16 chunk is 64 registers per lane.
    static constexpr int kRing = 4;
    static constexpr int kBalancedRing = 3;

    template <int H>
    struct Regs {
        u32x4 k[2][H / 32];   // score tile a, k-step s: 8 bf16 of one key row
        u32x4 v[H / 16];      // value tile c: 8 bf16 of one value column
    };

    __device__ static __forceinline__ int dim_offset(int s, int quad) { return 32 * s + 8 * quad; }

    // k_lo / v_lo: the chunk's first 16 tokens (their first key row, their
    // first element of every value row); k_hi / v_hi: its last 16 (key_hi,
    // value_hi).  BS, the tokens per block, is the value rows' length.
    template <int H, int BS = kBlockSize>
    __device__ static __forceinline__ void load(Regs<H> &r, const Elem *k_lo, const Elem *k_hi,
                                                const Elem *v_lo, const Elem *v_hi, int col,
                                                int quad)
    {
        const Elem *kb = (col >> 3) ? k_hi : k_lo;
        const int krow = 8 * ((col >> 2) & 1) + (col & 3);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int s = 0; s < H / 32; ++s)
                r.k[a][s] = load16_stream(kb + (krow + 4 * a) * H + dim_offset(s, quad));
        const Elem *vb = (quad >> 1) ? v_hi : v_lo;
#pragma unroll
        for (int c = 0; c < H / 16; ++c)
            r.v[c] = load16_stream(vb + (16 * c + col) * BS + 8 * (quad & 1));
    }

    template <int H>
    __device__ static __forceinline__ bf16x8 key(const Regs<H> &r, int a, int s)
    {
        return as_bf16x8(r.k[a][s]);
    }
    // Bits of the 8 bf16 values (masked by the caller in a tail chunk).
    template <int H>
    __device__ static __forceinline__ u32x4 value(const Regs<H> &r, int c)
    {
        return r.v[c];
    }
    // value() for a kernel that consumes the operand in several places: the
    // loaded bits need no widening, so it is value() itself.
    template <int H>
    __device__ static __forceinline__ u32x4 value_fresh(const Regs<H> &r, int c)
    {
        return r.v[c];
    }
    // Zeroes the lane's value elements from token `valid` (0..8) on, in place.
    template <int H>
    __device__ static __forceinline__ void zero_values(Regs<H> &r, int valid)
    {
        u32x4 mask;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            mask[w] = (2 * w < valid ? 0x0000FFFFu : 0u) | (2 * w + 1 < valid ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int c = 0; c < H / 16; ++c)
            r.v[c] &= mask;
    }
};

// Four E4M3 codes (bytes of w, lowest first) as four bf16, exactly.
__device__ __forceinline__ void widen4(uint32_t w, __bf16 *dst)
{
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    dst[0] = lo[0];
    dst[1] = lo[1];
    dst[2] = hi[0];
    dst[3] = hi[1];
}

__device__ __forceinline__ bf16x8 widen8(uint32_t w0, uint32_t w1)
{
    __bf16 t[8];
    widen4(w0, t);
    widen4(w1, t + 4);
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        r[e] = t[e];
    return r;
}

struct KvFp8 {
    using Elem = uint8_t;
    // An FP8 chunk is 32 registers per lane.  The fixed-partition ring of 5
    // (32 KiB in flight per wave) measured as fast as deeper ones (up to 8);
    // the token-balanced kernel runs at least as fast with 2 (one chunk in
    // flight while one is computed) as with 3 or 4.
    static constexpr int kRing = 5;
    static constexpr int kBalancedRing = 2;

    template <int H>
    struct Regs {
        u32x4 k[2][H / 64];   // score tile a, k-steps 2j and 2j+1: 16 codes of one key row
        u32x2 v[H / 16];      // value tile c: 8 codes of one value column
    };

    // Steps 2j and 2j+1 take the two halves of one 16-byte run of the key row,
    // so a lane's key bytes for both steps are one load.
    __device__ static __forceinline__ int dim_offset(int s, int quad)
    {
        return 64 * (s >> 1) + 16 * quad + 8 * (s & 1);
    }

    template <int H, int BS = kBlockSize>
    __device__ static __forceinline__ void load(Regs<H> &r, const Elem *k_lo, const Elem *k_hi,
                                                const Elem *v_lo, const Elem *v_hi, int col,
                                                int quad)
    {
        const Elem *kb = (col >> 3) ? k_hi : k_lo;
        const int krow = 8 * ((col >> 2) & 1) + (col & 3);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int j = 0; j < H / 64; ++j)
                r.k[a][j] = load16_stream(kb + (krow + 4 * a) * H + 64 * j + 16 * quad);
        const Elem *vb = (quad >> 1) ? v_hi : v_lo;
#pragma unroll
        for (int c = 0; c < H / 16; ++c)
            r.v[c] = load8_stream(vb + (16 * c + col) * BS + 8 * (quad & 1));
    }

    template <int H>
    __device__ static __forceinline__ bf16x8 key(const Regs<H> &r, int a, int s)
    {
        const u32x4 w = r.k[a][s >> 1];
        return (s & 1) ? widen8(w[2], w[3]) : widen8(w[0], w[1]);
    }
    template <int H>
    __device__ static __forceinline__ u32x4 value(const Regs<H> &r, int c)
    {
        return __builtin_bit_cast(u32x4, widen8(r.v[c][0], r.v[c][1]));
    }
    // value() widened anew at each call: the compiler cannot reuse the widened
    // operand of an earlier call, so a kernel that takes the same value tile
    // for several query tiles keeps 8 widened registers live instead of 32.
    template <int H>
    __device__ static __forceinline__ u32x4 value_fresh(const Regs<H> &r, int c)
    {
        u32x2 w = r.v[c];
        asm volatile("" : "+v"(w));
        return __builtin_bit_cast(u32x4, widen8(w[0], w[1]));
    }
    // Zeroes the lane's value codes from token `valid` (0..8) on, in place
    // (code 0 is +0).
    template <int H>
    __device__ static __forceinline__ void zero_values(Regs<H> &r, int valid)
    {
        u32x2 mask;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            uint32_t mw = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b)
                mw |= (4 * w + b < valid ? 0xFFu : 0u) << (8 * b);
            mask[w] = mw;
        }
#pragma unroll
        for (int c = 0; c < H / 16; ++c)
            r.v[c] &= mask;
    }
};

}  // namespace pkv
