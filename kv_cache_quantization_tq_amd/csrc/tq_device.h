// tq_device.h -- device code of the TurboQuant KV-cache codec for AMD MI355X
// (gfx950): tables, transform, bin search, packing and the kernel templates.
// Each kernel translation unit includes it and instantiates the kernels of one
// head_dim; the host side (tq_api.hip) includes it for the shared tables.
//
// The codec is the one on the page "@mlx-bun/inference 0.0.0-stage -> 1.0.0",
// package/src/kernels/turboquant/ops.ts (fwht, searchsorted, encodeKeys,
// decodeKeys, encodeValues, dequantScaled, decodeValues,
// decodeValuesRotated, unrotateValues, packBits/unpackBits), with the tables
// of "mlx-bun 0.0.9 -> 0.0.11", turboquant-tables.ts.
//
// Work mapping. One lane owns one 32-element group of one row (a row is one
// (token, head) vector of head_dim elements), so a row is a team of
// G = head_dim/32 adjacent lanes and a wavefront holds 64/G rows. Within a
// lane the group is 32 registers: the key path (min/max, affine code) needs
// no communication, the RMS of a value group is a sequential in-register
// sum, and the Walsh-Hadamard butterflies of span 1..16 are register
// operations. The butterflies of span 32..256 pair lanes g and g^1, g^2, g^4,
// g^8 of the team and run as DPP (or ds_swizzle) cross-lane adds. Each lane
// loads its group as 16-byte vectors and writes exactly 4*bits bytes of
// packed codes plus one fp16 scale (and zero point).
//
// Exactness. Every arithmetic step that feeds a stored plane rounds exactly
// as the plain binary32 definition does: butterflies in span order 1, 2, 4,
// ..., the single multiply by binary32(1/sqrt(d)) at the end, sequential
// sums of squares, no contraction (built with -ffp-contract=off), IEEE
// square root per group, and quotients a/b obtained as
//   q0 = a*r, e = fma(-q0, b, a), q = fma(e, r, q0),  r = RN(1/b),
// which equals the correctly rounded a/b whenever nothing overflows or
// underflows (reciprocal refinement, Markstein 1990); groups outside that
// range take the IEEE division instead. So key codes, key scales and zero
// points and value scales are bit-exact. The one exception is the value
// bin's argument z = y / (rms + 1e-8): it is taken as the single product
// y * RN(1/(rms + 1e-8)), within 1.5 ulp of the quotient (|z| < 6, so
// within 5e-7), which can move a code by one bin only for a z that close to
// a boundary -- inside the codec's tolerance of an off-by-one bin within
// 1e-5 of a boundary. The value bin (number of boundaries strictly below z)
// comes from a uniform-grid table built at compile time whose cells are
// narrower than the closest pair of boundaries, so one final comparison
// against the single boundary a cell may hold gives the count for that z.
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>


#include "tq_tables.h"

namespace {

// Compile-time tuning knobs (defaults are the measured best on MI355X):
//   TQ_ENCODE_WAVES, TQ_DECODE_WAVES  if > 0, target this many wavefronts
//                         per SIMD (caps the registers the kernel may use).
#ifndef TQ_ENCODE_WAVES
#define TQ_ENCODE_WAVES 0
#endif
#ifndef TQ_DECODE_WAVES
#define TQ_DECODE_WAVES 0
#endif

constexpr int kGroup = 32;
constexpr int kWave = 64;
constexpr int kBlockThreads = 256;
constexpr int kWavesPerBlock = kBlockThreads / kWave;

// ---------------------------------------------------------------------------
// Constant tables
// ---------------------------------------------------------------------------

template <int B> struct LM;
template <> struct LM<2> { static constexpr const float *c = kCentroids2; static constexpr const float *b = kBoundaries2; static constexpr int cell_exp = -1; };
template <> struct LM<3> { static constexpr const float *c = kCentroids3; static constexpr const float *b = kBoundaries3; static constexpr int cell_exp = -2; };
template <> struct LM<4> { static constexpr const float *c = kCentroids4; static constexpr const float *b = kBoundaries4; static constexpr int cell_exp = -3; };
template <> struct LM<5> { static constexpr const float *c = kCentroids5; static constexpr const float *b = kBoundaries5; static constexpr int cell_exp = -4; };
template <> struct LM<8> { static constexpr const float *c = kCentroids8; static constexpr const float *b = kBoundaries8; static constexpr int cell_exp = -6; };

constexpr double pow2(int e) { double r = 1.0; for (; e > 0; --e) r *= 2.0; for (; e < 0; ++e) r *= 0.5; return r; }

// Uniform grid over [-6, 6] for the B-bit table. The cell of z is
// round-to-nearest-even(z*A + C), A = 1/W a power of two: z*A is exact and
// one fma rounds, so the computed cell of any z is within 2^-14 cells of
// its true position. On the device the fma adds 2^23 as well, which leaves
// the cell index in the low mantissa bits of the result (floats in
// [2^23, 2^24) are spaced by 1), so the LDS address is one shift-add of the
// result's bit pattern. Each cell stores the number of boundaries below its
// (widened) lower edge and the one boundary, if any, inside the widened
// cell (+inf when none); W is below the smallest gap between adjacent
// boundaries, so a widened cell never holds two. The kernels need no clamp:
// a normalised value z = y / (rms + 1e-8) of a 32-element group satisfies
// |z| <= sqrt(32) < 5.66 (each |y_j| is at most the group's root-sum-square),
// and the first and last cells extend to -inf and +inf for the host
// evaluation, which clamps.
struct BinCell {
    float bnd;
    uint32_t base;
};

template <int B> struct BinGrid {
    static constexpr int NB = (1 << B) - 1;
    static constexpr float W = (float)pow2(LM<B>::cell_exp);
    static constexpr float A = (float)pow2(-LM<B>::cell_exp);
    static constexpr float LO = -6.0f;
    static constexpr float C = 6.0f * A;                 // cell c is centred at LO + c*W
    static constexpr float C_MAGIC = C + 8388608.0f;     // + 2^23
    static constexpr int N = (int)(12.0 * (double)A) + 2;
    static_assert(LM<B>::b[0] > -5.9f && LM<B>::b[NB - 1] < 5.9f, "boundaries inside the grid");
    static_assert(C_MAGIC - 8388608.0f == C, "grid offset exact");
};

template <int B> struct BinLut {
    BinCell cell[BinGrid<B>::N];
    bool ok;
    constexpr BinLut() : cell{}, ok(true)
    {
        using Gr = BinGrid<B>;
        constexpr double margin = 1.0 / 1024.0;
        for (int c = 0; c < Gr::N; ++c) {
            const double lo = (c == 0) ? -1e300 : (double)Gr::LO + ((double)c - 0.5 - margin) * (double)Gr::W;
            const double hi = (c == Gr::N - 1) ? 1e300 : (double)Gr::LO + ((double)c + 0.5 + margin) * (double)Gr::W;
            uint32_t base = 0;
            int inside = 0;
            float bnd = __builtin_huge_valf();
            for (int j = 0; j < Gr::NB; ++j) {
                const double bj = (double)LM<B>::b[j];
                if (bj < lo) {
                    ++base;
                } else if (bj <= hi) {
                    bnd = LM<B>::b[j];
                    ++inside;
                }
            }
            if (inside > 1) ok = false;
            cell[c].bnd = bnd;
            cell[c].base = base;
        }
    }
};

template <int B> struct CentTab {
    float c[1 << B];
    constexpr CentTab() : c{} { for (int i = 0; i < (1 << B); ++i) c[i] = LM<B>::c[i]; }
};

template <int D> struct SignTab;
template <> struct SignTab<64> { static constexpr const uint32_t *m = kSignMask64; };
template <> struct SignTab<128> { static constexpr const uint32_t *m = kSignMask128; };
template <> struct SignTab<256> { static constexpr const uint32_t *m = kSignMask256; };
template <> struct SignTab<512> { static constexpr const uint32_t *m = kSignMask512; };

template <int D> struct SignWords {
    uint32_t m[D / kGroup];
    constexpr SignWords() : m{} { for (int g = 0; g < D / kGroup; ++g) m[g] = SignTab<D>::m[g]; }
};

static_assert(BinLut<2>().ok && BinLut<3>().ok && BinLut<4>().ok && BinLut<5>().ok && BinLut<8>().ok,
              "a grid cell holds more than one Lloyd-Max boundary");

// binary32(1/sqrt(d)), the normalisation of the transform
template <int D> struct HadScale;
template <> struct HadScale<64> { static constexpr float v = 0x1p-3f; };
template <> struct HadScale<128> { static constexpr float v = 0x1.6a09e6p-4f; };
template <> struct HadScale<256> { static constexpr float v = 0x1p-4f; };
template <> struct HadScale<512> { static constexpr float v = 0x1.6a09e6p-5f; };

__constant__ BinLut<2> dLut2 = BinLut<2>();
__constant__ BinLut<3> dLut3 = BinLut<3>();
__constant__ BinLut<4> dLut4 = BinLut<4>();
__constant__ BinLut<5> dLut5 = BinLut<5>();
__constant__ BinLut<8> dLut8 = BinLut<8>();
__constant__ CentTab<2> dCent2 = CentTab<2>();
__constant__ CentTab<3> dCent3 = CentTab<3>();
__constant__ CentTab<4> dCent4 = CentTab<4>();
__constant__ CentTab<5> dCent5 = CentTab<5>();
__constant__ CentTab<8> dCent8 = CentTab<8>();
__constant__ SignWords<64> dSign64 = SignWords<64>();
__constant__ SignWords<128> dSign128 = SignWords<128>();
__constant__ SignWords<256> dSign256 = SignWords<256>();
__constant__ SignWords<512> dSign512 = SignWords<512>();

template <int B> __device__ __forceinline__ const BinCell *dev_lut();
template <> __device__ __forceinline__ const BinCell *dev_lut<2>() { return dLut2.cell; }
template <> __device__ __forceinline__ const BinCell *dev_lut<3>() { return dLut3.cell; }
template <> __device__ __forceinline__ const BinCell *dev_lut<4>() { return dLut4.cell; }
template <> __device__ __forceinline__ const BinCell *dev_lut<5>() { return dLut5.cell; }
template <> __device__ __forceinline__ const BinCell *dev_lut<8>() { return dLut8.cell; }

template <int B> __device__ __forceinline__ const float *dev_cent();
template <> __device__ __forceinline__ const float *dev_cent<2>() { return dCent2.c; }
template <> __device__ __forceinline__ const float *dev_cent<3>() { return dCent3.c; }
template <> __device__ __forceinline__ const float *dev_cent<4>() { return dCent4.c; }
template <> __device__ __forceinline__ const float *dev_cent<5>() { return dCent5.c; }
template <> __device__ __forceinline__ const float *dev_cent<8>() { return dCent8.c; }

template <int D> __device__ __forceinline__ uint32_t dev_sign(int g);
template <> __device__ __forceinline__ uint32_t dev_sign<64>(int g) { return dSign64.m[g]; }
template <> __device__ __forceinline__ uint32_t dev_sign<128>(int g) { return dSign128.m[g]; }
template <> __device__ __forceinline__ uint32_t dev_sign<256>(int g) { return dSign256.m[g]; }
template <> __device__ __forceinline__ uint32_t dev_sign<512>(int g) { return dSign512.m[g]; }

// The sign vector as XOR masks in the layout of a loaded group: for bf16
// data one dword per element pair (bit 15 flips the even element, bit 31
// the odd one), for binary32 data one dword per element (bit 31). The
// encoder copies its head_dim's table to LDS once per block and each lane
// reads the masks of its group there, which costs no arithmetic per tile.
template <int D, bool BF16> struct SignXor {
    static constexpr int W = BF16 ? kGroup / 2 : kGroup; // dwords per group
    uint32_t m[D / kGroup][W];
    constexpr SignXor() : m{}
    {
        for (int g = 0; g < D / kGroup; ++g) {
            const uint32_t s = SignTab<D>::m[g];
            for (int k = 0; k < W; ++k)
                m[g][k] = BF16 ? ((((s >> (2 * k)) & 1u) << 15) | (((s >> (2 * k + 1)) & 1u) << 31))
                               : (((s >> k) & 1u) << 31);
        }
    }
};

__constant__ SignXor<64, true> dSx64b = SignXor<64, true>();
__constant__ SignXor<128, true> dSx128b = SignXor<128, true>();
__constant__ SignXor<256, true> dSx256b = SignXor<256, true>();
__constant__ SignXor<512, true> dSx512b = SignXor<512, true>();
__constant__ SignXor<64, false> dSx64f = SignXor<64, false>();
__constant__ SignXor<128, false> dSx128f = SignXor<128, false>();
__constant__ SignXor<256, false> dSx256f = SignXor<256, false>();
__constant__ SignXor<512, false> dSx512f = SignXor<512, false>();

template <int D, bool BF16> __device__ __forceinline__ const uint32_t *dev_sign_xor()
{
    if constexpr (BF16) {
        if constexpr (D == 64) return &dSx64b.m[0][0];
        else if constexpr (D == 128) return &dSx128b.m[0][0];
        else if constexpr (D == 256) return &dSx256b.m[0][0];
        else return &dSx512b.m[0][0];
    } else {
        if constexpr (D == 64) return &dSx64f.m[0][0];
        else if constexpr (D == 128) return &dSx128f.m[0][0];
        else if constexpr (D == 256) return &dSx256f.m[0][0];
        else return &dSx512f.m[0][0];
    }
}

// ---------------------------------------------------------------------------
// Scalar helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// two binary32 -> packed bf16 pair, round to nearest even
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x)
{
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

// xor mask flipping the signs of the bf16 pair held in dword k (elements
// 2k and 2k+1 of the group) according to the group's sign word
__device__ __forceinline__ uint32_t sign_pair_mask(uint32_t smask, int k)
{
    return (((smask >> (2 * k)) & 1u) << 15) | (((smask >> (2 * k + 1)) & 1u) << 31);
}

// ---------------------------------------------------------------------------
// Walsh-Hadamard transform of one row held as 32 registers per lane
// ---------------------------------------------------------------------------

// butterflies of span 1, 2, 4, 8, 16 inside the group
__device__ __forceinline__ void fwht_in_lane(float (&y)[kGroup])
{
#pragma unroll
    for (int h = 1; h < kGroup; h <<= 1) {
#pragma unroll
        for (int i = 0; i < kGroup; i += 2 * h) {
#pragma unroll
            for (int j = i; j < i + h; ++j) {
                const float a = y[j];
                const float b = y[j + h];
                y[j] = a + b;
                y[j + h] = a - b;
            }
        }
    }
}

// Butterflies of span 32*M between the groups g and g^M of a row team.
//
// Each lane keeps its values multiplied by a carried sign c = +-1 (the same
// for all 32 registers of the lane), so that one fused multiply-add per
// element does the butterfly: own + sigma * partner, where sigma = +1 in
// the lower group and -1 in the upper one. The lower group then holds
// c * (a + b) and the upper one -c * (a - b); since partners differ only in
// bit M, which no earlier stage has touched, they carry equal signs, and the
// fma (exact product by +-1, one rounding) rounds exactly as a + b or a - b.
// After all stages c = (-1)^popcount(g), which the caller folds into the
// final multiply by 1/sqrt(d).
//
// M = 1, 2, 8 read the partner through DPP (quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row_ror:8, all inside a 16-lane row, hence inside
// the team); M = 4 fetches it with ds_swizzle (bitmask mode, xor 4). The
// DPP forms are written as inline assembly because the compiler does not
// fold a DPP move into v_fmac; the leading s_nop 1 provides the two wait
// states a DPP read needs after a VALU write of its source register (the
// eight registers of one block are distinct, so no hazard arises inside).
#define TQ_FMAC_DPP(k, ctrl) "v_fmac_f32_dpp %" #k ", %" #k ", %8 " ctrl " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
#define TQ_FMAC_DPP8(ctrl)                                                                                    \
    "s_nop 1\n\t" TQ_FMAC_DPP(0, ctrl) TQ_FMAC_DPP(1, ctrl) TQ_FMAC_DPP(2, ctrl) TQ_FMAC_DPP(3, ctrl)            \
        TQ_FMAC_DPP(4, ctrl) TQ_FMAC_DPP(5, ctrl) TQ_FMAC_DPP(6, ctrl) TQ_FMAC_DPP(7, ctrl)

template <int M> __device__ __forceinline__ void fwht_cross(float (&y)[kGroup], float sigma)
{
    if constexpr (M == 4) {
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            const float p = as_f((uint32_t)__builtin_amdgcn_ds_swizzle((int)as_u(y[j]), 0x101F));
            y[j] = __builtin_fmaf(p, sigma, y[j]);
        }
    } else {
#pragma unroll
        for (int b = 0; b < kGroup; b += 8) {
            if constexpr (M == 1) {
                asm volatile(TQ_FMAC_DPP8("quad_perm:[1,0,3,2]")
                             : "+v"(y[b]), "+v"(y[b + 1]), "+v"(y[b + 2]), "+v"(y[b + 3]), "+v"(y[b + 4]),
                               "+v"(y[b + 5]), "+v"(y[b + 6]), "+v"(y[b + 7])
                             : "v"(sigma));
            } else if constexpr (M == 2) {
                asm volatile(TQ_FMAC_DPP8("quad_perm:[2,3,0,1]")
                             : "+v"(y[b]), "+v"(y[b + 1]), "+v"(y[b + 2]), "+v"(y[b + 3]), "+v"(y[b + 4]),
                               "+v"(y[b + 5]), "+v"(y[b + 6]), "+v"(y[b + 7])
                             : "v"(sigma));
            } else {
                static_assert(M == 8, "cross-lane span");
                asm volatile(TQ_FMAC_DPP8("row_ror:8")
                             : "+v"(y[b]), "+v"(y[b + 1]), "+v"(y[b + 2]), "+v"(y[b + 3]), "+v"(y[b + 4]),
                               "+v"(y[b + 5]), "+v"(y[b + 6]), "+v"(y[b + 7])
                             : "v"(sigma));
            }
        }
    }
}

// Per-lane constants of the transform for group g of a D-wide row.
template <int D> struct Rot {
    float sig1, sig2, sig4, sig8; // +1 in the lower group of each span, -1 in the upper one
    float scale;                  // (-1)^popcount(g) * binary32(1/sqrt(D))
    __device__ __forceinline__ explicit Rot(int g)
    {
        sig1 = (g & 1) ? -1.0f : 1.0f;
        sig2 = (g & 2) ? -1.0f : 1.0f;
        sig4 = (g & 4) ? -1.0f : 1.0f;
        sig8 = (g & 8) ? -1.0f : 1.0f;
        scale = (__builtin_popcount((unsigned)g & (D / kGroup - 1)) & 1) ? -HadScale<D>::v : HadScale<D>::v;
    }
};

// normalised transform: butterflies of every span in increasing order, then
// one multiply by binary32(1/sqrt(D)) (which also removes the carried sign)
template <int D> __device__ __forceinline__ void hadamard(float (&y)[kGroup], const Rot<D> &rt)
{
    fwht_in_lane(y);
    if constexpr (D >= 64) fwht_cross<1>(y, rt.sig1);
    if constexpr (D >= 128) fwht_cross<2>(y, rt.sig2);
    if constexpr (D >= 256) fwht_cross<4>(y, rt.sig4);
    if constexpr (D >= 512) fwht_cross<8>(y, rt.sig8);
#pragma unroll
    for (int j = 0; j < kGroup; ++j) y[j] = y[j] * rt.scale;
}

// ---------------------------------------------------------------------------
// Bin search and bit packing
// ---------------------------------------------------------------------------

// Number of boundaries strictly below z: base of z's cell plus one if z is
// above the cell's boundary. bin_index_any accepts any z (infinities and
// NaN included; NaN lands in cell 0) and is what the host evaluation runs;
// bin_index_bounded needs |z| <= 6 and no NaN, which holds for every value
// of a group whose sum of squares is finite.
template <int B>
__host__ __device__ __forceinline__ uint32_t bin_index_any(float z, const BinCell *lut)
{
    using Gr = BinGrid<B>;
    const float zc = fminf(fmaxf(z, -3.0e38f), 3.0e38f);
    const float t = fminf(fmaxf(rintf(__builtin_fmaf(zc, Gr::A, Gr::C)), 0.0f), (float)(Gr::N - 1));
    const BinCell e = lut[(uint32_t)t];
    return e.base + (zc > e.bnd ? 1u : 0u);
}

template <int B>
__host__ __device__ __forceinline__ uint32_t bin_index_bounded(float z, const BinCell *lut)
{
    using Gr = BinGrid<B>;
    const float t = __builtin_fmaf(z, Gr::A, Gr::C_MAGIC);
    // bits(t) = bits(2^23) + cell; byte address = 8 * cell
    const uint32_t addr = (__builtin_bit_cast(uint32_t, t) << 3) - (0x4B000000u << 3);
    const BinCell e = *reinterpret_cast<const BinCell *>(reinterpret_cast<const char *>(lut) + addr);
    return e.base + (z > e.bnd ? 1u : 0u);
}

// 32 codes of B bits -> B dwords, element j at bits [j*B, j*B+B). Codes
// must be below 2^B, except for B == 8 where only the low byte of each
// value is used (signed codes arrive as negative integers).
template <int B> __device__ __forceinline__ void pack32(const uint32_t (&q)[kGroup], uint32_t (&w)[B])
{
    if constexpr (B == 8) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            // v_perm_b32 selector bytes: 4 = byte 0 of the first operand, 0 = byte 0 of the second
            const uint32_t lo = __builtin_amdgcn_perm(q[4 * k + 1], q[4 * k], 0x0c0c0400u);
            const uint32_t hi = __builtin_amdgcn_perm(q[4 * k + 3], q[4 * k + 2], 0x0c0c0400u);
            w[k] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
        }
    } else {
#pragma unroll
        for (int k = 0; k < B; ++k) w[k] = 0;
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            const int pos = j * B, k = pos >> 5, s = pos & 31;
            w[k] |= q[j] << s;
            if (s + B > 32) w[k + 1] |= q[j] >> (32 - s);
        }
    }
}

template <int B> __device__ __forceinline__ uint32_t unpack1(const uint32_t (&w)[B], int j)
{
    const int pos = j * B, k = pos >> 5, s = pos & 31;
    constexpr uint32_t mask = (1u << B) - 1u;
    if (s + B <= 32) return (w[k] >> s) & mask;
    return __builtin_amdgcn_alignbit(w[k + 1], w[k], s) & mask;
}

template <int B> __device__ __forceinline__ void store_codes(uint8_t *p, const uint32_t (&w)[B])
{
    if constexpr (B == 2) {
        *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
    } else if constexpr (B == 4) {
        *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if constexpr (B == 8) {
        reinterpret_cast<uint4 *>(p)[0] = make_uint4(w[0], w[1], w[2], w[3]);
        reinterpret_cast<uint4 *>(p)[1] = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
        uint32_t *d = reinterpret_cast<uint32_t *>(p);
#pragma unroll
        for (int k = 0; k < B; ++k) d[k] = w[k];
    }
}

template <int B> __device__ __forceinline__ void load_codes(const uint8_t *p, uint32_t (&w)[B])
{
    if constexpr (B == 2) {
        const uint2 a = *reinterpret_cast<const uint2 *>(p);
        w[0] = a.x; w[1] = a.y;
    } else if constexpr (B == 4) {
        const uint4 a = *reinterpret_cast<const uint4 *>(p);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    } else if constexpr (B == 8) {
        const uint4 a = reinterpret_cast<const uint4 *>(p)[0];
        const uint4 b = reinterpret_cast<const uint4 *>(p)[1];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else {
        const uint32_t *s = reinterpret_cast<const uint32_t *>(p);
#pragma unroll
        for (int k = 0; k < B; ++k) w[k] = s[k];
    }
}

// load_codes with the non-temporal hint: the decoder reads each packed row
// once, so its lines need not stay in the caches
template <int B> __device__ __forceinline__ void load_codes_stream(const uint8_t *p, uint32_t (&w)[B])
{
    if constexpr (B == 2) {
        const u32x2_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
        w[0] = a.x; w[1] = a.y;
    } else if constexpr (B == 4 || B == 8) {
#pragma unroll
        for (int h = 0; h < B / 4; ++h) {
            const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p) + h);
            w[4 * h] = a.x; w[4 * h + 1] = a.y; w[4 * h + 2] = a.z; w[4 * h + 3] = a.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < B; ++k) w[k] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p) + k);
    }
}

// one 16-byte store with the non-temporal hint
__device__ __forceinline__ void store16_stream(uint8_t *p, const uint4 &v)
{
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t *>(p));
}

// ---------------------------------------------------------------------------
// Group loads and stores (32 elements, 16-byte vectors)
// ---------------------------------------------------------------------------


// ---------------------------------------------------------------------------
// Key path (per lane, no communication)
// ---------------------------------------------------------------------------

// Minimum and maximum of a group, equal to a scan with strict comparisons
// that keeps the first of equal values. v_min3/v_max3 give the extreme
// values (two new elements per instruction; inline assembly because the
// compiler would first canonicalise every operand loaded as raw bits); only
// the sign of a zero extreme can differ from the scan's, so when an extreme
// is zero it is replaced by the first element equal to zero.
__device__ __forceinline__ float min3f(float a, float b, float c)
{
    float r;
    asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float max3f(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ __forceinline__ void group_min_max(const float (&x)[kGroup], float &mn, float &mx)
{
    float a = min3f(x[0], x[1], x[2]);
    float b = max3f(x[0], x[1], x[2]);
#pragma unroll
    for (int j = 3; j < kGroup; j += 2) {
        if (j + 1 < kGroup) {
            a = min3f(a, x[j], x[j + 1]);
            b = max3f(b, x[j], x[j + 1]);
        } else {
            a = min3f(a, x[j], x[j]);
            b = max3f(b, x[j], x[j]);
        }
    }
    if (a == 0.0f || b == 0.0f) {
        float first_zero = 0.0f;
        bool found = false;
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            const bool z = !found && x[j] == 0.0f;
            first_zero = z ? x[j] : first_zero;
            found = found || z;
        }
        if (a == 0.0f) a = first_zero;
        if (b == 0.0f) b = first_zero;
    }
    mn = a;
    mx = b;
}

// quotient a / b rounded to nearest, from r = RN(1/b) (see file header);
// a zero quotient may come out as +0 for a = -0 (the last fma adds +0 and
// -0), which does not matter where the result is rounded to an integer code
__host__ __device__ __forceinline__ float quot(float a, float b, float r)
{
    const float q0 = a * r;
    const float e = __builtin_fmaf(-q0, b, a);
    return __builtin_fmaf(e, r, q0);
}

// the same quotient with the sign of a zero result kept, for b > 0: equal
// to the IEEE a / b whenever quot is exact (a stored zero point or scale of
// -0 stays -0)
__host__ __device__ __forceinline__ float quot_signed(float a, float b, float r)
{
    return __builtin_copysignf(quot(a, b, r), a);
}

// x / se - zp for element j (IEEE division on the slow path)
__device__ __forceinline__ float key_shifted(float x, float se, float r, float zp, bool ieee)
{
    return (ieee ? x / se : quot(x, se, r)) - zp;
}

// Codes of one key group, packed (element j at bits [j*KB, j*KB+KB)).
// Unsigned codes: clip(rint(d), 0, maxv) = rint(clip(d, 0, maxv)) for the
// integer bounds, and v_cvt_pk_u8_f32 rounds to nearest even, saturates to
// [0, 255] and inserts the byte in one instruction; for 2-, 4- and 8-bit
// codes the bytes are laid out so that shifting whole dwords interleaves
// them into the bit stream (4-bit: even elements in one dword, odd ones in
// another shifted by 4; 2-bit: four dwords shifted by 0, 2, 4, 6). Signed
// 8-bit codes round, clip to [-127, 127] and take the low byte of each.
template <int KB, bool KS>
__device__ __forceinline__ void key_codes(const float (&x)[kGroup], float se, float r, float zp, uint32_t (&w)[KB],
                                          bool ieee)
{
    constexpr float maxv = KS ? 127.0f : (float)((1 << KB) - 1);
    if constexpr (KS) {
        uint32_t q[kGroup];
#pragma unroll
        for (int j = 0; j < kGroup; ++j)
            q[j] = (uint32_t)(int32_t)__builtin_amdgcn_fmed3f(rintf(key_shifted(x[j], se, r, zp, ieee)), -maxv, maxv);
        pack32<KB>(q, w);
    } else if constexpr (KB == 8) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint32_t b = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) b = __builtin_amdgcn_cvt_pk_u8_f32(key_shifted(x[4 * k + t], se, r, zp, ieee), t, b);
            w[k] = b;
        }
    } else if constexpr (KB == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t ev = 0, od = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float de = __builtin_amdgcn_fmed3f(key_shifted(x[8 * k + 2 * t], se, r, zp, ieee), 0.0f, maxv);
                const float dd = __builtin_amdgcn_fmed3f(key_shifted(x[8 * k + 2 * t + 1], se, r, zp, ieee), 0.0f, maxv);
                ev = __builtin_amdgcn_cvt_pk_u8_f32(de, t, ev);
                od = __builtin_amdgcn_cvt_pk_u8_f32(dd, t, od);
            }
            w[k] = ev | (od << 4);
        }
    } else if constexpr (KB == 2) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            uint32_t d4[4] = {0, 0, 0, 0};
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float d = __builtin_amdgcn_fmed3f(key_shifted(x[16 * k + 4 * t + rr], se, r, zp, ieee), 0.0f, maxv);
                    d4[rr] = __builtin_amdgcn_cvt_pk_u8_f32(d, t, d4[rr]);
                }
            }
            w[k] = d4[0] | (d4[1] << 2) | (d4[2] << 4) | (d4[3] << 6);
        }
    } else {
        uint32_t q[kGroup];
#pragma unroll
        for (int j = 0; j < kGroup; ++j)
            q[j] = __builtin_amdgcn_cvt_pk_u8_f32(
                __builtin_amdgcn_fmed3f(key_shifted(x[j], se, r, zp, ieee), 0.0f, maxv), 0, 0u);
        pack32<KB>(q, w);
    }
}

// Codes of one key group when every element's rounded value is known to be
// in the code range: the same arithmetic as key_codes without the clamp
// (the unsigned byte conversion still saturates at 0). Used for 2- and
// 4-bit unsigned and 8-bit signed codes.
template <int KB, bool KS>
__device__ __forceinline__ void key_codes_in_range(const float (&x)[kGroup], float se, float r, float zp,
                                                   uint32_t (&w)[KB])
{
    if constexpr (KS) {
        uint32_t q[kGroup];
#pragma unroll
        for (int j = 0; j < kGroup; ++j) q[j] = (uint32_t)(int32_t)rintf(quot(x[j], se, r) - zp);
        pack32<KB>(q, w);
    } else if constexpr (KB == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t ev = 0, od = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                ev = __builtin_amdgcn_cvt_pk_u8_f32(quot(x[8 * k + 2 * t], se, r) - zp, t, ev);
                od = __builtin_amdgcn_cvt_pk_u8_f32(quot(x[8 * k + 2 * t + 1], se, r) - zp, t, od);
            }
            w[k] = ev | (od << 4);
        }
    } else {
        static_assert(KB == 2, "in-range key codes: 2-bit, 4-bit or signed 8-bit");
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            uint32_t d4[4] = {0, 0, 0, 0};
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    d4[rr] = __builtin_amdgcn_cvt_pk_u8_f32(quot(x[16 * k + 4 * t + rr], se, r) - zp, t, d4[rr]);
            }
            w[k] = d4[0] | (d4[1] << 2) | (d4[2] << 4) | (d4[3] << 6);
        }
    }
}

// One key group: scale = (max - min) / maxv (signed: / (2 maxv)), zero point
// rint(min / (scale + eps)) (signed: rint((max + min) / (2 (scale + eps)))),
// codes clip(rint(x / (scale + eps) - zero)). The divisions by the constant
// and by scale + eps are exact quotients from a reciprocal (file header);
// IEEE division is kept for the reciprocal itself and for groups whose
// magnitudes leave the range where the quotient is exact. Rounding is
// monotone in x, so the codes of the group's minimum and maximum bound
// every element's code: when both are in range the clamp is skipped.
template <int KB, bool KS>
__device__ __forceinline__ void key_encode_group(const float (&x)[kGroup], uint8_t *codes,
                                                 uint16_t *scale_out, uint16_t *zero_out)
{
    float mn, mx;
    group_min_max(x, mn, mx);
    const float eps = 1e-8f;
    constexpr int maxv = KS ? 127 : (1 << KB) - 1;
    constexpr float dv = (float)(KS ? 2 * maxv : maxv);
    constexpr float rdv = 1.0f / dv; // RN(1/dv), rounded by the compiler
    const float range = mx - mn;
    const bool range_ok = range >= 0x1p-100f && range < 0x1p100f; // quotient exact and normal
    const float scale = range_ok ? quot_signed(range, dv, rdv) : range / dv;
    const float se = scale + eps;
    const float r = 1.0f / se;
    const float amax = fmaxf(fabsf(mn), fabsf(mx));
    const bool fast = (se < 1e30f) && (amax * r < 1e30f);
    float zp;
    if constexpr (KS) {
        const float num = mx + mn;
        // 2 * se and r / 2 are exact: the quotient by 2 * se from RN(1/(2 se))
        zp = rintf(fast ? quot_signed(num, 2.0f * se, 0.5f * r) : num / (2.0f * se));
    } else {
        zp = rintf(fast ? quot_signed(mn, se, r) : mn / se);
    }
    uint32_t w[KB];
    if (fast) {
        constexpr bool has_in_range = KS || KB == 2 || KB == 4;
        const float hi = rintf(quot(mx, se, r) - zp);
        const float lo = rintf(quot(mn, se, r) - zp);
        const bool in_range = KS ? (hi <= (float)maxv && lo >= -(float)maxv) : (hi <= (float)maxv);
        if (has_in_range && in_range) {
            if constexpr (has_in_range) key_codes_in_range<KB, KS>(x, se, r, zp, w);
        } else {
            key_codes<KB, KS>(x, se, r, zp, w, /*ieee=*/false);
        }
    } else {
        key_codes<KB, KS>(x, se, r, zp, w, /*ieee=*/true);
    }
    store_codes<KB>(codes, w);
    *scale_out = f32_to_f16_bits(scale);
    *zero_out = f32_to_f16_bits(zp);
}


// ---------------------------------------------------------------------------
// Coalesced output through LDS
// ---------------------------------------------------------------------------

// A wavefront's 64 lanes hold 64 consecutive 32-element groups, i.e. one
// contiguous tile of the output (4 KB in bf16, 8 KB in f32), but each lane
// owns a 64 B (128 B) piece of it. Written directly, every store
// instruction would touch 64 pieces 64 B apart. Instead each lane writes its
// piece to a per-wavefront LDS area (pieces padded by 16 B, which keeps the
// 16-byte LDS accesses free of bank conflicts) and the wavefront then
// stores the tile so that each instruction covers a contiguous 1 KB. The
// stores carry the non-temporal hint: decoded rows are written once and
// not read back by this kernel, and without the hint the dirty lines they
// leave in the caches are written back during whatever kernel runs next.
template <bool BF16> struct Stage {
    static constexpr int CH = BF16 ? 4 : 8;   // 16-byte chunks per lane
    static constexpr int STRIDE = CH + 1;     // padded piece, in 16-byte units
    static constexpr int LPI = kWave / CH;    // pieces covered by one store instruction
    static constexpr int WORDS = kWave * STRIDE;
};

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Store the tile whose first row is row0 (rows_per_wave rows of D elements),
// converting to the output type and flipping signs per `smask`; rows at or
// beyond `rows` are not written.
template <int D, bool BF16>
__device__ __forceinline__ void store_tile(void *base, int64_t row0, int64_t rows, uint32_t smask,
                                           const float (&y)[kGroup], uint4 *stage)
{
    using S = Stage<BF16>;
    constexpr int G = D / kGroup;
    const int lane = threadIdx.x & (kWave - 1);
    uint4 w[S::CH];
    if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t q[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int k = 4 * i + t;
                q[t] = pack_bf16x2(y[2 * k], y[2 * k + 1]) ^ sign_pair_mask(smask, k);
            }
            w[i] = make_uint4(q[0], q[1], q[2], q[3]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t q[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int j = 4 * i + t;
                q[t] = as_u(y[j]) ^ (((smask >> j) & 1u) << 31);
            }
            w[i] = make_uint4(q[0], q[1], q[2], q[3]);
        }
    }
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < S::CH; ++i) stage[lane * S::STRIDE + i] = w[i];
    wave_lds_sync();
    constexpr int elem_bytes = BF16 ? 2 : 4;
    uint8_t *tile = reinterpret_cast<uint8_t *>(base) + row0 * (int64_t)(D * elem_bytes);
    const int c_lo = lane % S::LPI;
    const int sub = lane / S::LPI;
    uint4 v[S::CH];
#pragma unroll
    for (int i = 0; i < S::CH; ++i) v[i] = stage[(S::LPI * i + c_lo) * S::STRIDE + sub];
    if (row0 + kWave / G <= rows) {
        // whole tile in range (wave-uniform branch)
#pragma unroll
        for (int i = 0; i < S::CH; ++i) store16_stream(tile + (uint32_t)(((S::LPI * i + c_lo) * S::CH + sub) * 16), v[i]);
    } else {
#pragma unroll
        for (int i = 0; i < S::CH; ++i) {
            const int c = S::LPI * i + c_lo; // piece = writer lane
            if (row0 + c / G < rows) store16_stream(tile + (uint32_t)((c * S::CH + sub) * 16), v[i]);
        }
    }
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

// key modes: bits | (signed << 4); 0 = no key side
enum { KMODE_NONE = 0 };

// One group as loaded: 32 elements in 16-byte vectors.
template <bool BF16> struct RawGroup {
    uint4 v[BF16 ? 4 : 8];
};

template <bool BF16> __device__ __forceinline__ void load_raw(const void *base, int64_t e0, RawGroup<BF16> &r)
{
    const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint8_t *>(base) + e0 * (BF16 ? 2 : 4));
#pragma unroll
    for (int i = 0; i < (BF16 ? 4 : 8); ++i) r.v[i] = p[i];
}

// binary32 values of a raw group, multiplied by the signs in `smask`
template <bool BF16>
__device__ __forceinline__ void raw_to_f32(const RawGroup<BF16> &r, uint32_t smask, float (&x)[kGroup])
{
    if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w[4] = {r.v[i].x, r.v[i].y, r.v[i].z, r.v[i].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int k = 4 * i + t;
                const uint32_t u = w[t] ^ sign_pair_mask(smask, k);
                x[2 * k] = as_f(u << 16);
                x[2 * k + 1] = as_f(u & 0xffff0000u);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t w[4] = {r.v[i].x, r.v[i].y, r.v[i].z, r.v[i].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int j = 4 * i + t;
                x[j] = as_f(w[t] ^ (((smask >> j) & 1u) << 31));
            }
        }
    }
}

// binary32 values of a raw group, each element's sign flipped by the XOR
// masks `m` (layout of SignXor)
template <bool BF16>
__device__ __forceinline__ void raw_to_f32_xor(const RawGroup<BF16> &r, const uint4 *m, float (&x)[kGroup])
{
#pragma unroll
    for (int i = 0; i < (BF16 ? 4 : 8); ++i) {
        const uint4 mi = m[i];
        const uint32_t w[4] = {r.v[i].x ^ mi.x, r.v[i].y ^ mi.y, r.v[i].z ^ mi.z, r.v[i].w ^ mi.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if constexpr (BF16) {
                const int k = 4 * i + t;
                x[2 * k] = as_f(w[t] << 16);
                x[2 * k + 1] = as_f(w[t] & 0xffff0000u);
            } else {
                x[4 * i + t] = as_f(w[t]);
            }
        }
    }
}

// Bins of the 32 values z_j = y_j * r (r = RN(1/(rms + 1e-8)), so
// |z_j| < 6), packed as they are found: code j at bits [j*B, j*B+B).
template <int B>
__device__ __forceinline__ void bin_pack(const float (&y)[kGroup], float r, const BinCell *lut, uint32_t (&w)[B])
{
#pragma unroll
    for (int k = 0; k < B; ++k) w[k] = 0;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
        const uint32_t q = bin_index_bounded<B>(y[j] * r, lut);
        const int pos = j * B, k = pos >> 5, sh = pos & 31;
        w[k] |= q << sh;
        if (sh + B > 32) w[k + 1] |= q >> (32 - sh);
    }
}

// Tile loop of the encoder for one key mode (KB = 0: values only): a
// wavefront walks tiles t, t + stride, ... Loads always read a valid row
// (rows past the end read the last row, whose results are not stored), so
// they need no branch. The value side runs first: it is the longer one,
// and the key group's raw words wait in registers meanwhile.
template <int D, int VB, int KB, bool KS, bool BF16IN>
__device__ __forceinline__ void encode_loop(const void *__restrict__ kin, const void *__restrict__ vin, int64_t rows,
                                            uint8_t *__restrict__ kc, uint16_t *__restrict__ ks,
                                            uint16_t *__restrict__ kz, uint8_t *__restrict__ vc,
                                            uint16_t *__restrict__ vs, const BinCell *lut, const uint32_t *sxor)
{
    constexpr int G = D / kGroup;
    constexpr int RPW = kWave / G;
    constexpr bool HASK = KB != 0;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); // wavefront-uniform
    const int g = lane % G;
    const int rl = lane / G;
    const uint4 *smask = reinterpret_cast<const uint4 *>(sxor + g * SignXor<D, BF16IN>::W);
    const Rot<D> rot(g);
    const bool hasv = vin != nullptr;
    const int64_t tiles = (rows + RPW - 1) / RPW;
    const int64_t stride = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave; t < tiles; t += stride) {
        const int64_t row = t * RPW + rl;
        const bool act = row < rows;
        const int64_t grp = row * G + g;
        const int64_t e0 = (act ? row : rows - 1) * D + (int64_t)g * kGroup;
        RawGroup<BF16IN> kraw, vraw;
        if constexpr (HASK) load_raw<BF16IN>(kin, e0, kraw);
        if (hasv) load_raw<BF16IN>(vin, e0, vraw);
        if (hasv) {
            float y[kGroup];
            raw_to_f32_xor<BF16IN>(vraw, smask, y);
            hadamard<D>(y, rot);
            float ss = 0.0f;
#pragma unroll
            for (int j = 0; j < kGroup; ++j) {
                const float sq = y[j] * y[j];
                ss = ss + sq;
            }
            const float s = sqrtf(ss / (float)kGroup);
            const float se = s + 1e-8f;
            uint32_t w[VB];
            if (se < 1e30f) {
                // ss finite: every y finite and |y / se| <= sqrt(32)
                bin_pack<VB>(y, 1.0f / se, lut, w);
            } else {
                uint32_t q[kGroup];
#pragma unroll
                for (int j = 0; j < kGroup; ++j) q[j] = bin_index_any<VB>(y[j] / se, lut);
                pack32<VB>(q, w);
            }
            if (act) {
                store_codes<VB>(vc + grp * (4 * VB), w);
                vs[grp] = f32_to_f16_bits(s);
            }
        }
        if constexpr (HASK) {
            float x[kGroup];
            raw_to_f32<BF16IN>(kraw, 0u, x);
            if (act) key_encode_group<KB, KS>(x, kc + grp * (4 * KB), ks + grp, kz + grp);
        }
    }
}

// Wavefronts per SIMD asked of the register allocator: five where the
// encoder's state fits in 96 VGPRs without spilling (bf16 inputs, every value
// width but 3 bits up to head_dim 128, 2- and 8-bit values above; one more
// wavefront in flight hides more of the loads' latency), else no constraint
// (1). TQ_ENCODE_WAVES, when defined, overrides it for every configuration.
template <int D, int VB, bool BF16IN>
constexpr int kEncodeWaves = BF16IN && VB != 3 && (D <= 128 || VB == 8 || (D == 256 && VB == 2)) ? 5 : 1;
#if TQ_ENCODE_WAVES > 0
#define TQ_ENCODE_ATTR __launch_bounds__(kBlockThreads) __attribute__((amdgpu_waves_per_eu(TQ_ENCODE_WAVES)))
#else
#define TQ_ENCODE_ATTR __launch_bounds__(kBlockThreads) __attribute__((amdgpu_waves_per_eu(kEncodeWaves<D, VB, BF16IN>)))
#endif

template <int D, int VB, bool BF16IN>
__global__ void TQ_ENCODE_ATTR
encode_kernel(const void *__restrict__ kin, const void *__restrict__ vin, int64_t rows, int32_t kmode,
              uint8_t *__restrict__ kc, uint16_t *__restrict__ ks, uint16_t *__restrict__ kz,
              uint8_t *__restrict__ vc, uint16_t *__restrict__ vs)
{
    constexpr int NCELL = BinGrid<VB>::N;
    constexpr int NSX = (D / kGroup) * SignXor<D, BF16IN>::W;
    __shared__ BinCell lut[NCELL];
    __shared__ __attribute__((aligned(16))) uint32_t sxor[NSX];
    if (vin != nullptr) {
        const BinCell *src = dev_lut<VB>();
        for (int i = threadIdx.x; i < NCELL; i += kBlockThreads) lut[i] = src[i];
        const uint32_t *sx = dev_sign_xor<D, BF16IN>();
        for (int i = threadIdx.x; i < NSX; i += kBlockThreads) sxor[i] = sx[i];
        __syncthreads();
    }
    switch (kmode) {
    case 2: encode_loop<D, VB, 2, false, BF16IN>(kin, vin, rows, kc, ks, kz, vc, vs, lut, sxor); break;
    case 3: encode_loop<D, VB, 3, false, BF16IN>(kin, vin, rows, kc, ks, kz, vc, vs, lut, sxor); break;
    case 4: encode_loop<D, VB, 4, false, BF16IN>(kin, vin, rows, kc, ks, kz, vc, vs, lut, sxor); break;
    case 5: encode_loop<D, VB, 5, false, BF16IN>(kin, vin, rows, kc, ks, kz, vc, vs, lut, sxor); break;
    case 8: encode_loop<D, VB, 8, false, BF16IN>(kin, vin, rows, kc, ks, kz, vc, vs, lut, sxor); break;
    case 8 | 16: encode_loop<D, VB, 8, true, BF16IN>(kin, vin, rows, kc, ks, kz, vc, vs, lut, sxor); break;
    default: encode_loop<D, VB, 0, false, BF16IN>(kin, vin, rows, kc, ks, kz, vc, vs, lut, sxor); break;
    }
}

// Packed input of one group for the decoder: code words and fp16 bits.
template <int KB, int VB> struct GroupCodes {
    uint32_t kw[KB > 0 ? KB : 1];
    uint32_t vw[VB];
    uint32_t ks, kz, vs;
};

template <int D, int VB, int KB>
__device__ __forceinline__ void load_group_codes(const uint8_t *__restrict__ kc, const uint16_t *__restrict__ ks,
                                                 const uint16_t *__restrict__ kz, const uint8_t *__restrict__ vc,
                                                 const uint16_t *__restrict__ vs, int64_t row, int64_t rows, int g,
                                                 bool hasv, GroupCodes<KB, VB> &c)
{
    // always a valid row (rows past the end read the last row, whose
    // results are not stored): branch-free loads keep wait counts exact
    constexpr int G = D / kGroup;
    const int64_t grp = (row < rows ? row : rows - 1) * G + g;
    if constexpr (KB != 0) {
        load_codes_stream<KB>(kc + grp * (4 * KB), c.kw);
        c.ks = __builtin_nontemporal_load(ks + grp);
        c.kz = __builtin_nontemporal_load(kz + grp);
    } else {
        c.kw[0] = 0;
        c.ks = c.kz = 0;
    }
    if (hasv) {
        load_codes_stream<VB>(vc + grp * (4 * VB), c.vw);
        c.vs = __builtin_nontemporal_load(vs + grp);
    } else {
#pragma unroll
        for (int k = 0; k < VB; ++k) c.vw[k] = 0;
        c.vs = 0;
    }
}

// Tile loop of the decoder for one key mode (KB = 0: values only). setup()
// puts the block's centroid table into LDS and waits for the block; every
// wavefront calls it once, after its first tile's loads.
template <int D, int VB, int KB, bool KS, bool BF16OUT, typename Setup>
__device__ __forceinline__ void decode_loop(const uint8_t *__restrict__ kc, const uint16_t *__restrict__ ks,
                                            const uint16_t *__restrict__ kz, const uint8_t *__restrict__ vc,
                                            const uint16_t *__restrict__ vs, int64_t rows, int32_t rotated,
                                            void *__restrict__ kout, void *__restrict__ vout, const float *cent,
                                            uint4 *stage, Setup &&setup)
{
    constexpr int G = D / kGroup;
    constexpr int RPW = kWave / G;
    constexpr bool HASK = KB != 0;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); // wavefront-uniform
    const int g = lane % G;
    const int rl = lane / G;
    const uint32_t smask = rotated ? 0u : dev_sign<D>(g);
    const Rot<D> rot(g);
    const bool hasv = vout != nullptr;
    const int64_t tiles = (rows + RPW - 1) / RPW;
    const int64_t stride = (int64_t)gridDim.x * kWavesPerBlock;
    auto tile = [&](int64_t t, const GroupCodes<KB, VB> &cur) {
        const int64_t row0 = t * RPW;
        if constexpr (HASK) {
            float y[kGroup];
            const float scale = f16_bits_to_f32((uint16_t)cur.ks);
            const float zero = f16_bits_to_f32((uint16_t)cur.kz);
#pragma unroll
            for (int j = 0; j < kGroup; ++j) {
                const uint32_t u = unpack1<KB>(cur.kw, j);
                const float qf = KS ? (float)(int32_t)(int8_t)(uint8_t)u : (float)u;
                const float sum = qf + zero;
                y[j] = sum * scale;
            }
            store_tile<D, BF16OUT>(kout, row0, rows, 0u, y, stage);
        }
        if (hasv) {
            float y[kGroup];
            const float s = f16_bits_to_f32((uint16_t)cur.vs);
#pragma unroll
            for (int j = 0; j < kGroup; ++j) y[j] = cent[unpack1<VB>(cur.vw, j)] * s;
            if (!rotated) hadamard<D>(y, rot);
            store_tile<D, BF16OUT>(vout, row0, rows, smask, y, stage);
        }
    };
    // the first tile's codes are requested before the block's table reaches
    // LDS (setup() stores it and waits for the block), so that the two
    // latencies overlap (long-context decode 266-269 against 278 us); a
    // wavefront without a tile loads the last row and stores nothing
    const int64_t t0 = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    {
        GroupCodes<KB, VB> cur;
        load_group_codes<D, VB, KB>(kc, ks, kz, vc, vs, t0 * RPW + rl, rows, g, hasv, cur);
        setup();
        if (t0 < tiles) tile(t0, cur);
    }
    for (int64_t t = t0 + stride; t < tiles; t += stride) {
        GroupCodes<KB, VB> cur;
        load_group_codes<D, VB, KB>(kc, ks, kz, vc, vs, t * RPW + rl, rows, g, hasv, cur);
        tile(t, cur);
    }
}

#if TQ_DECODE_WAVES > 0
#define TQ_DECODE_ATTR __launch_bounds__(kBlockThreads) __attribute__((amdgpu_waves_per_eu(TQ_DECODE_WAVES)))
#else
#define TQ_DECODE_ATTR __launch_bounds__(kBlockThreads)
#endif

template <int D, int VB, bool BF16OUT>
__global__ void TQ_DECODE_ATTR
decode_kernel(const uint8_t *__restrict__ kc, const uint16_t *__restrict__ ks, const uint16_t *__restrict__ kz,
              const uint8_t *__restrict__ vc, const uint16_t *__restrict__ vs, int64_t rows, int32_t kmode,
              int32_t rotated, void *__restrict__ kout, void *__restrict__ vout)
{
    constexpr int NC = 1 << VB;
    using S = Stage<BF16OUT>;
    constexpr int NL = (NC + kBlockThreads - 1) / kBlockThreads;
    __shared__ float cent[NC];
    __shared__ uint4 stage_all[kWavesPerBlock * S::WORDS];
    // the centroids go to registers first (their loads leave before the
    // first tile's), then to LDS in setup()
    const bool tables = vout != nullptr; // uniform over the block
    float cv[NL];
    if (tables) {
        const float *src = dev_cent<VB>();
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int i = threadIdx.x + k * kBlockThreads;
            cv[k] = src[i < NC ? i : NC - 1];
        }
    }
    auto setup = [&] {
        if (tables) {
#pragma unroll
            for (int k = 0; k < NL; ++k) {
                const int i = threadIdx.x + k * kBlockThreads;
                if (i < NC) cent[i] = cv[k];
            }
            __syncthreads();
        }
    };
    uint4 *stage = stage_all + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave) * S::WORDS;
    switch (kmode) {
    case 2:
        decode_loop<D, VB, 2, false, BF16OUT>(kc, ks, kz, vc, vs, rows, rotated, kout, vout, cent, stage, setup);
        break;
    case 3:
        decode_loop<D, VB, 3, false, BF16OUT>(kc, ks, kz, vc, vs, rows, rotated, kout, vout, cent, stage, setup);
        break;
    case 4:
        decode_loop<D, VB, 4, false, BF16OUT>(kc, ks, kz, vc, vs, rows, rotated, kout, vout, cent, stage, setup);
        break;
    case 5:
        decode_loop<D, VB, 5, false, BF16OUT>(kc, ks, kz, vc, vs, rows, rotated, kout, vout, cent, stage, setup);
        break;
    case 8:
        decode_loop<D, VB, 8, false, BF16OUT>(kc, ks, kz, vc, vs, rows, rotated, kout, vout, cent, stage, setup);
        break;
    case 8 | 16:
        decode_loop<D, VB, 8, true, BF16OUT>(kc, ks, kz, vc, vs, rows, rotated, kout, vout, cent, stage, setup);
        break;
    default:
        decode_loop<D, VB, 0, false, BF16OUT>(kc, ks, kz, vc, vs, rows, rotated, kout, vout, cent, stage, setup);
        break;
    }
}

// inverse rotation of attention outputs (rows of D elements, f32 or bf16);
// x and out may be the same buffer
template <int D, bool BF16>
__global__ void __launch_bounds__(kBlockThreads)
unrotate_kernel(const void *x, void *out, int64_t rows)
{
    constexpr int G = D / kGroup;
    constexpr int RPW = kWave / G;
    using S = Stage<BF16>;
    __shared__ uint4 stage_all[kWavesPerBlock * S::WORDS];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); // wavefront-uniform
    uint4 *stage = stage_all + wave * S::WORDS;
    const int g = lane % G;
    const int rl = lane / G;
    const uint32_t smask = dev_sign<D>(g);
    const Rot<D> rot(g);
    const int64_t tiles = (rows + RPW - 1) / RPW;
    for (int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave; t < tiles;
         t += (int64_t)gridDim.x * kWavesPerBlock) {
        const int64_t row0 = t * RPW;
        const int64_t row = row0 + rl;
        const int64_t e0 = (row < rows ? row : rows - 1) * D + (int64_t)g * kGroup;
        float y[kGroup];
        RawGroup<BF16> raw;
        load_raw<BF16>(x, e0, raw);
        raw_to_f32<BF16>(raw, 0u, y);
        hadamard<D>(y, rot);
        store_tile<D, BF16>(out, row0, rows, smask, y, stage);
    }
}

} // namespace
