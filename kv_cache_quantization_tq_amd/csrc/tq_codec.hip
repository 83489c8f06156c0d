// tq_codec.hip -- TurboQuant KV-cache codec for AMD MI355X (gfx950): kernels
// and the C ABI declared in include/tq.h.
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
// Exactness. Every arithmetic step rounds exactly as the plain binary32
// definition does: butterflies in span order 1, 2, 4, ..., the single
// multiply by binary32(1/sqrt(d)) at the end, sequential sums of squares,
// no contraction (built with -ffp-contract=off), IEEE division and square
// root per group, and per element a quotient a/b obtained as
//   q0 = a*r, e = fma(-q0, b, a), q = fma(e, r, q0),  r = RN(1/b),
// which equals the correctly rounded a/b whenever nothing overflows or
// underflows (reciprocal refinement, Markstein 1990); groups outside that
// range take the IEEE division instead. The value bin (number of boundaries
// strictly below z) comes from a uniform-grid table built at compile time
// whose cells are narrower than the closest pair of boundaries, so one
// final comparison against the single boundary a cell may hold gives the
// exact count.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "tq.h"
#include "tq_tables.h"

namespace {

constexpr int kGroup = 32;
constexpr int kWave = 64;
constexpr int kBlockThreads = 256;
constexpr int kWavesPerBlock = kBlockThreads / kWave;
constexpr int64_t kMaxBlocks = 8192;

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

// Uniform grid over the boundaries of the B-bit table. The cell of z is
// clamp(floor(fma(z, A, C)), 0, N-1) with A = 1/W a power of two and
// C = -LO*A, so z*A is exact and the fma rounds once; the computed cell of
// any z lies within 2^-14 cells of its true position. Each cell stores the
// number of boundaries below its (widened) lower edge and the one boundary,
// if any, inside the widened cell; +inf when none.
struct BinCell {
    float bnd;
    uint32_t base;
};

template <int B> struct BinGrid {
    static constexpr int NB = (1 << B) - 1;
    static constexpr float W = (float)pow2(LM<B>::cell_exp);
    static constexpr float A = (float)pow2(-LM<B>::cell_exp);
    static constexpr float LO = LM<B>::b[0] - 0.5f * W;
    static constexpr float C = -LO * A;
    static constexpr int N = (int)((double)(LM<B>::b[NB - 1] - LO) * (double)A) + 2;
};

template <int B> struct BinLut {
    BinCell cell[BinGrid<B>::N];
    bool ok;
    constexpr BinLut() : cell{}, ok(true)
    {
        using Gr = BinGrid<B>;
        constexpr double margin = 1.0 / 1024.0;
        for (int c = 0; c < Gr::N; ++c) {
            const double lo = (c == 0) ? -1e300 : (double)Gr::LO + ((double)c - margin) * (double)Gr::W;
            const double hi = (c == Gr::N - 1) ? 1e300 : (double)Gr::LO + ((double)c + 1.0 + margin) * (double)Gr::W;
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

// ---------------------------------------------------------------------------
// Scalar helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

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

// value of lane (lane ^ M) for M in {1,2,4,8}; all patterns stay inside a
// 16-lane DPP row, hence inside one row team
template <int M> __device__ __forceinline__ float lane_xor(float v);
template <> __device__ __forceinline__ float lane_xor<1>(float v)
{
    return as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(v), 0xB1, 0xF, 0xF, true)); // quad_perm [1,0,3,2]
}
template <> __device__ __forceinline__ float lane_xor<2>(float v)
{
    return as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(v), 0x4E, 0xF, 0xF, true)); // quad_perm [2,3,0,1]
}
template <> __device__ __forceinline__ float lane_xor<4>(float v)
{
    return as_f((uint32_t)__builtin_amdgcn_ds_swizzle((int)as_u(v), 0x101F)); // bitmask mode, xor 4
}
template <> __device__ __forceinline__ float lane_xor<8>(float v)
{
    return as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(v), 0x128, 0xF, 0xF, true)); // row_ror:8
}

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

// butterfly of span 32*M between group g and group g^M: the lower group
// keeps a + b, the upper one b's partner minus itself, i.e. a - b
template <int M> __device__ __forceinline__ void fwht_cross(float (&y)[kGroup], int g)
{
    const uint32_t neg = (g & M) ? 0x80000000u : 0u;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
        const float own = as_f(as_u(y[j]) ^ neg);
        y[j] = lane_xor<M>(y[j]) + own;
    }
}

// normalised transform (butterflies of every span in increasing order,
// then one multiply by binary32(1/sqrt(D)))
template <int D> __device__ __forceinline__ void hadamard(float (&y)[kGroup], int g)
{
    fwht_in_lane(y);
    if constexpr (D >= 64) fwht_cross<1>(y, g);
    if constexpr (D >= 128) fwht_cross<2>(y, g);
    if constexpr (D >= 256) fwht_cross<4>(y, g);
    if constexpr (D >= 512) fwht_cross<8>(y, g);
    const float r = HadScale<D>::v;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) y[j] = y[j] * r;
}

// ---------------------------------------------------------------------------
// Bin search and bit packing
// ---------------------------------------------------------------------------

template <int B>
__host__ __device__ __forceinline__ uint32_t bin_index(float z, const BinCell *lut)
{
    using Gr = BinGrid<B>;
    float t = __builtin_fmaf(z, Gr::A, Gr::C);
#if defined(__HIP_DEVICE_COMPILE__)
    t = __builtin_amdgcn_fmed3f(t, 0.0f, (float)(Gr::N - 1));
#else
    t = fminf(fmaxf(t, 0.0f), (float)(Gr::N - 1));
#endif
    const BinCell e = lut[(uint32_t)t];
    return e.base + (z > e.bnd ? 1u : 0u);
}

// 32 codes of B bits -> B dwords, element j at bits [j*B, j*B+B)
template <int B> __device__ __forceinline__ void pack32(const uint32_t (&q)[kGroup], uint32_t (&w)[B])
{
#pragma unroll
    for (int k = 0; k < B; ++k) w[k] = 0;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
        const int pos = j * B, k = pos >> 5, s = pos & 31;
        w[k] |= q[j] << s;
        if (s + B > 32) w[k + 1] |= q[j] >> (32 - s);
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

// ---------------------------------------------------------------------------
// Group loads and stores (32 elements, 16-byte vectors)
// ---------------------------------------------------------------------------

// load a group and multiply by the signs when `smask` is not zero
template <bool BF16>
__device__ __forceinline__ void load_group(const void *base, int64_t e0, uint32_t smask, float (&x)[kGroup])
{
    if constexpr (BF16) {
        const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(base) + e0);
        uint32_t w[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 a = p[i];
            w[4 * i + 0] = a.x; w[4 * i + 1] = a.y; w[4 * i + 2] = a.z; w[4 * i + 3] = a.w;
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const uint32_t u = w[k] ^ sign_pair_mask(smask, k);
            x[2 * k] = as_f(u << 16);
            x[2 * k + 1] = as_f(u & 0xffff0000u);
        }
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + e0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 a = p[i];
            x[4 * i + 0] = a.x; x[4 * i + 1] = a.y; x[4 * i + 2] = a.z; x[4 * i + 3] = a.w;
        }
#pragma unroll
        for (int j = 0; j < kGroup; ++j) x[j] = as_f(as_u(x[j]) ^ (((smask >> j) & 1u) << 31));
    }
}

// store a group, multiplying by the signs given by `smask` (0: none)
template <bool BF16>
__device__ __forceinline__ void store_group(void *base, int64_t e0, uint32_t smask, const float (&y)[kGroup])
{
    if constexpr (BF16) {
        uint4 *p = reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(base) + e0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t w[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int k = 4 * i + t;
                w[t] = pack_bf16x2(y[2 * k], y[2 * k + 1]) ^ sign_pair_mask(smask, k);
            }
            p[i] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else {
        float4 *p = reinterpret_cast<float4 *>(reinterpret_cast<float *>(base) + e0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int j = 4 * i + t;
                v[t] = as_f(as_u(y[j]) ^ (((smask >> j) & 1u) << 31));
            }
            p[i] = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
}

// ---------------------------------------------------------------------------
// Key path (per lane, no communication)
// ---------------------------------------------------------------------------

// quotient a / b rounded to nearest, from r = RN(1/b) (see file header)
__device__ __forceinline__ float quot(float a, float b, float r)
{
    const float q0 = a * r;
    const float e = __builtin_fmaf(-q0, b, a);
    return __builtin_fmaf(e, r, q0);
}

template <int KB, bool KS>
__device__ __forceinline__ void key_encode_group(const float (&x)[kGroup], uint8_t *codes,
                                                 uint16_t *scale_out, uint16_t *zero_out)
{
    // sequential min / max, keeping the first of equal values (as a scan
    // with strict comparisons does)
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int j = 1; j < kGroup; ++j) {
        mn = (x[j] < mn) ? x[j] : mn;
        mx = (x[j] > mx) ? x[j] : mx;
    }
    const float eps = 1e-8f;
    constexpr int maxv = KS ? 127 : (1 << KB) - 1;
    float scale, zp;
    if constexpr (KS) {
        scale = (mx - mn) / (float)(2 * maxv);
        const float denom = 2.0f * (scale + eps);
        zp = rintf((mx + mn) / denom);
    } else {
        scale = (mx - mn) / (float)maxv;
        zp = rintf(mn / (scale + eps));
    }
    const float se = scale + eps;
    const float r = 1.0f / se;
    const float amax = fmaxf(fabsf(mn), fabsf(mx));
    const bool fast = (se < 1e30f) && (amax * r < 1e30f);
    const float lo = KS ? -(float)maxv : 0.0f;
    const float hi = (float)maxv;
    uint32_t q[kGroup];
    if (fast) {
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            const float o = quot(x[j], se, r);
            const float c = __builtin_amdgcn_fmed3f(rintf(o - zp), lo, hi);
            q[j] = (uint32_t)(int32_t)c & 0xffu;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            const float o = x[j] / se;
            const float c = __builtin_amdgcn_fmed3f(rintf(o - zp), lo, hi);
            q[j] = (uint32_t)(int32_t)c & 0xffu;
        }
    }
    uint32_t w[KB];
    pack32<KB>(q, w);
    store_codes<KB>(codes, w);
    *scale_out = f32_to_f16_bits(scale);
    *zero_out = f32_to_f16_bits(zp);
}

template <int KB, bool KS, bool BF16>
__device__ __forceinline__ void key_decode_group(const uint8_t *codes, uint16_t scale16, uint16_t zero16,
                                                 void *out, int64_t e0)
{
    uint32_t w[KB];
    load_codes<KB>(codes, w);
    const float scale = f16_bits_to_f32(scale16);
    const float zero = f16_bits_to_f32(zero16);
    float y[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
        const uint32_t u = unpack1<KB>(w, j);
        const float qf = KS ? (float)(int32_t)(int8_t)(uint8_t)u : (float)u;
        const float s = qf + zero;
        y[j] = s * scale;
    }
    store_group<BF16>(out, e0, 0u, y);
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

// key modes: bits | (signed << 4); 0 = no key side
enum { KMODE_NONE = 0 };

template <int D, int VB, bool BF16IN>
__global__ void __launch_bounds__(kBlockThreads)
encode_kernel(const void *__restrict__ kin, const void *__restrict__ vin, int64_t rows, int32_t kmode,
              uint8_t *__restrict__ kc, uint16_t *__restrict__ ks, uint16_t *__restrict__ kz,
              uint8_t *__restrict__ vc, uint16_t *__restrict__ vs)
{
    constexpr int G = D / kGroup;
    constexpr int RPW = kWave / G;
    constexpr int NCELL = BinGrid<VB>::N;
    __shared__ BinCell lut[NCELL];
    if (vin != nullptr) {
        const BinCell *src = dev_lut<VB>();
        for (int i = threadIdx.x; i < NCELL; i += kBlockThreads) lut[i] = src[i];
        __syncthreads();
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int g = lane % G;
    const int rl = lane / G;
    const uint32_t smask = dev_sign<D>(g);
    const int64_t tiles = (rows + RPW - 1) / RPW;
    for (int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave; t < tiles;
         t += (int64_t)gridDim.x * kWavesPerBlock) {
        const int64_t row = t * RPW + rl;
        const bool act = row < rows;
        const int64_t e0 = row * D + (int64_t)g * kGroup;
        const int64_t grp = row * G + g;
        if (kmode != KMODE_NONE && act) {
            float x[kGroup];
            load_group<BF16IN>(kin, e0, 0u, x);
            switch (kmode) {
            case 2: key_encode_group<2, false>(x, kc + grp * 8, ks + grp, kz + grp); break;
            case 3: key_encode_group<3, false>(x, kc + grp * 12, ks + grp, kz + grp); break;
            case 4: key_encode_group<4, false>(x, kc + grp * 16, ks + grp, kz + grp); break;
            case 5: key_encode_group<5, false>(x, kc + grp * 20, ks + grp, kz + grp); break;
            case 8: key_encode_group<8, false>(x, kc + grp * 32, ks + grp, kz + grp); break;
            case 8 | 16: key_encode_group<8, true>(x, kc + grp * 32, ks + grp, kz + grp); break;
            default: break;
            }
        }
        if (vin != nullptr) {
            float y[kGroup];
            if (act) {
                load_group<BF16IN>(vin, e0, smask, y);
            } else {
#pragma unroll
                for (int j = 0; j < kGroup; ++j) y[j] = 0.0f;
            }
            hadamard<D>(y, g);
            float ss = 0.0f;
#pragma unroll
            for (int j = 0; j < kGroup; ++j) {
                const float sq = y[j] * y[j];
                ss = ss + sq;
            }
            const float s = sqrtf(ss / (float)kGroup);
            const float se = s + 1e-8f;
            const float r = 1.0f / se;
            uint32_t q[kGroup];
            if (se < 1e30f) {
#pragma unroll
                for (int j = 0; j < kGroup; ++j) q[j] = bin_index<VB>(quot(y[j], se, r), lut);
            } else {
#pragma unroll
                for (int j = 0; j < kGroup; ++j) q[j] = bin_index<VB>(y[j] / se, lut);
            }
            if (act) {
                uint32_t w[VB];
                pack32<VB>(q, w);
                store_codes<VB>(vc + grp * (4 * VB), w);
                vs[grp] = f32_to_f16_bits(s);
            }
        }
    }
}

template <int D, int VB, bool BF16OUT>
__global__ void __launch_bounds__(kBlockThreads)
decode_kernel(const uint8_t *__restrict__ kc, const uint16_t *__restrict__ ks, const uint16_t *__restrict__ kz,
              const uint8_t *__restrict__ vc, const uint16_t *__restrict__ vs, int64_t rows, int32_t kmode,
              int32_t rotated, void *__restrict__ kout, void *__restrict__ vout)
{
    constexpr int G = D / kGroup;
    constexpr int RPW = kWave / G;
    constexpr int NC = 1 << VB;
    __shared__ float cent[NC];
    if (vout != nullptr) {
        const float *src = dev_cent<VB>();
        for (int i = threadIdx.x; i < NC; i += kBlockThreads) cent[i] = src[i];
        __syncthreads();
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int g = lane % G;
    const int rl = lane / G;
    const uint32_t smask = rotated ? 0u : dev_sign<D>(g);
    const int64_t tiles = (rows + RPW - 1) / RPW;
    for (int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave; t < tiles;
         t += (int64_t)gridDim.x * kWavesPerBlock) {
        const int64_t row = t * RPW + rl;
        const bool act = row < rows;
        const int64_t e0 = row * D + (int64_t)g * kGroup;
        const int64_t grp = row * G + g;
        if (kmode != KMODE_NONE && act) {
            const uint16_t s16 = ks[grp], z16 = kz[grp];
            switch (kmode) {
            case 2: key_decode_group<2, false, BF16OUT>(kc + grp * 8, s16, z16, kout, e0); break;
            case 3: key_decode_group<3, false, BF16OUT>(kc + grp * 12, s16, z16, kout, e0); break;
            case 4: key_decode_group<4, false, BF16OUT>(kc + grp * 16, s16, z16, kout, e0); break;
            case 5: key_decode_group<5, false, BF16OUT>(kc + grp * 20, s16, z16, kout, e0); break;
            case 8: key_decode_group<8, false, BF16OUT>(kc + grp * 32, s16, z16, kout, e0); break;
            case 8 | 16: key_decode_group<8, true, BF16OUT>(kc + grp * 32, s16, z16, kout, e0); break;
            default: break;
            }
        }
        if (vout != nullptr) {
            float y[kGroup];
            uint32_t w[VB];
            float s = 0.0f;
            if (act) {
                load_codes<VB>(vc + grp * (4 * VB), w);
                s = f16_bits_to_f32(vs[grp]);
            } else {
#pragma unroll
                for (int k = 0; k < VB; ++k) w[k] = 0;
            }
#pragma unroll
            for (int j = 0; j < kGroup; ++j) y[j] = cent[unpack1<VB>(w, j)] * s;
            if (!rotated) hadamard<D>(y, g);
            if (act) store_group<BF16OUT>(vout, e0, smask, y);
        }
    }
}

// inverse rotation of attention outputs (rows of D elements, f32 or bf16)
template <int D, bool BF16>
__global__ void __launch_bounds__(kBlockThreads)
unrotate_kernel(const void *__restrict__ x, void *__restrict__ out, int64_t rows)
{
    constexpr int G = D / kGroup;
    constexpr int RPW = kWave / G;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int g = lane % G;
    const int rl = lane / G;
    const uint32_t smask = dev_sign<D>(g);
    const int64_t tiles = (rows + RPW - 1) / RPW;
    for (int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave; t < tiles;
         t += (int64_t)gridDim.x * kWavesPerBlock) {
        const int64_t row = t * RPW + rl;
        const bool act = row < rows;
        const int64_t e0 = row * D + (int64_t)g * kGroup;
        float y[kGroup];
        if (act) {
            load_group<BF16>(x, e0, 0u, y);
        } else {
#pragma unroll
            for (int j = 0; j < kGroup; ++j) y[j] = 0.0f;
        }
        hadamard<D>(y, g);
        if (act) store_group<BF16>(out, e0, smask, y);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

bool valid_head_dim(int32_t d) { return d == 64 || d == 128 || d == 256 || d == 512; }
bool valid_bits(int32_t b) { return b == 2 || b == 3 || b == 4 || b == 5 || b == 8; }
bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
uintptr_t code_align(int32_t bits) { return (bits == 4 || bits == 8) ? 16 : 8; }

int64_t grid_for(int64_t rows, int32_t d)
{
    const int64_t rpw = kWave / (d / kGroup);
    const int64_t tiles = (rows + rpw - 1) / rpw;
    int64_t blocks = (tiles + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    return blocks < 1 ? 1 : blocks;
}

int32_t check_rows(int64_t tokens, int32_t heads, int64_t *rows)
{
    if (tokens < 0 || heads < 1) return TQ_E_SHAPE;
    if (tokens > (int64_t)1 << 40 || heads > (1 << 20)) return TQ_E_SHAPE;
    *rows = tokens * heads;
    return TQ_OK;
}

int32_t key_mode(const tq_config *cfg) { return cfg->k_bits | (cfg->k_signed ? 16 : 0); }

typedef void (*EncodeFn)(const void *, const void *, int64_t, int32_t, uint8_t *, uint16_t *, uint16_t *,
                         uint8_t *, uint16_t *);
typedef void (*DecodeFn)(const uint8_t *, const uint16_t *, const uint16_t *, const uint8_t *,
                         const uint16_t *, int64_t, int32_t, int32_t, void *, void *);
typedef void (*UnrotateFn)(const void *, void *, int64_t);

template <int D, bool BF> EncodeFn pick_encode_vb(int32_t vb)
{
    switch (vb) {
    case 2: return encode_kernel<D, 2, BF>;
    case 3: return encode_kernel<D, 3, BF>;
    case 4: return encode_kernel<D, 4, BF>;
    case 5: return encode_kernel<D, 5, BF>;
    case 8: return encode_kernel<D, 8, BF>;
    default: return nullptr;
    }
}

template <bool BF> EncodeFn pick_encode(int32_t d, int32_t vb)
{
    switch (d) {
    case 64: return pick_encode_vb<64, BF>(vb);
    case 128: return pick_encode_vb<128, BF>(vb);
    case 256: return pick_encode_vb<256, BF>(vb);
    case 512: return pick_encode_vb<512, BF>(vb);
    default: return nullptr;
    }
}

template <int D, bool BF> DecodeFn pick_decode_vb(int32_t vb)
{
    switch (vb) {
    case 2: return decode_kernel<D, 2, BF>;
    case 3: return decode_kernel<D, 3, BF>;
    case 4: return decode_kernel<D, 4, BF>;
    case 5: return decode_kernel<D, 5, BF>;
    case 8: return decode_kernel<D, 8, BF>;
    default: return nullptr;
    }
}

template <bool BF> DecodeFn pick_decode(int32_t d, int32_t vb)
{
    switch (d) {
    case 64: return pick_decode_vb<64, BF>(vb);
    case 128: return pick_decode_vb<128, BF>(vb);
    case 256: return pick_decode_vb<256, BF>(vb);
    case 512: return pick_decode_vb<512, BF>(vb);
    default: return nullptr;
    }
}

template <bool BF> UnrotateFn pick_unrotate(int32_t d)
{
    switch (d) {
    case 64: return unrotate_kernel<64, BF>;
    case 128: return unrotate_kernel<128, BF>;
    case 256: return unrotate_kernel<256, BF>;
    case 512: return unrotate_kernel<512, BF>;
    default: return nullptr;
    }
}

int32_t launch_status()
{
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_E_HIP;
}


} // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

int64_t tq_packed_dim(int32_t dim, int32_t bits)
{
    if (dim < 1 || bits < 1 || bits > 8) return -TQ_E_BITS;
    if (((int64_t)dim * bits) % 8 != 0) return -TQ_E_ALIGN;
    return ((int64_t)dim * bits) / 8;
}

const char *tq_status_string(int32_t status)
{
    switch (status) {
    case TQ_OK: return "ok";
    case TQ_E_NULL: return "a required pointer is NULL";
    case TQ_E_HEAD_DIM: return "head_dim must be 64, 128, 256 or 512";
    case TQ_E_BITS: return "bits must be 2, 3, 4, 5 or 8 (signed keys: 8 only)";
    case TQ_E_ALIGN: return "misaligned pointer or dim*bits not a whole number of bytes";
    case TQ_E_DTYPE: return "dtype must be TQ_F32 or TQ_BF16";
    case TQ_E_SHAPE: return "tokens must be >= 0 and heads >= 1 (row count within range)";
    case TQ_E_HIP: return "HIP runtime error at kernel launch";
    default: return "unknown status";
    }
}

int32_t tq_encode_kv(const void *k, const void *v, int32_t in_dtype, int64_t tokens, int32_t heads,
                     const tq_config *cfg, const tq_packed_kv *out, void *stream)
{
    if (cfg == nullptr || out == nullptr) return TQ_E_NULL;
    if (k == nullptr && v == nullptr) return TQ_E_NULL;
    if (!valid_head_dim(cfg->head_dim)) return TQ_E_HEAD_DIM;
    if (in_dtype != TQ_F32 && in_dtype != TQ_BF16) return TQ_E_DTYPE;
    if (k != nullptr) {
        if (!valid_bits(cfg->k_bits) || (cfg->k_signed != 0 && cfg->k_bits != 8) ||
            (cfg->k_signed != 0 && cfg->k_signed != 1))
            return TQ_E_BITS;
        if (out->k_codes == nullptr || out->k_scale == nullptr || out->k_zero == nullptr) return TQ_E_NULL;
        if (!aligned(k, 16) || !aligned(out->k_codes, code_align(cfg->k_bits)) || !aligned(out->k_scale, 2) ||
            !aligned(out->k_zero, 2))
            return TQ_E_ALIGN;
    }
    if (v != nullptr) {
        if (!valid_bits(cfg->v_bits)) return TQ_E_BITS;
        if (out->v_codes == nullptr || out->v_scale == nullptr) return TQ_E_NULL;
        if (!aligned(v, 16) || !aligned(out->v_codes, code_align(cfg->v_bits)) || !aligned(out->v_scale, 2))
            return TQ_E_ALIGN;
    }
    int64_t rows = 0;
    const int32_t st = check_rows(tokens, heads, &rows);
    if (st != TQ_OK) return st;
    if (rows == 0) return TQ_OK;
    const int32_t vb = (v != nullptr) ? cfg->v_bits : 4;
    EncodeFn fn = (in_dtype == TQ_BF16) ? pick_encode<true>(cfg->head_dim, vb) : pick_encode<false>(cfg->head_dim, vb);
    const int32_t kmode = (k != nullptr) ? key_mode(cfg) : KMODE_NONE;
    hipLaunchKernelGGL(fn, dim3((uint32_t)grid_for(rows, cfg->head_dim)), dim3(kBlockThreads), 0,
                       (hipStream_t)stream, k, v, rows, kmode, (uint8_t *)out->k_codes, (uint16_t *)out->k_scale,
                       (uint16_t *)out->k_zero, (uint8_t *)out->v_codes, (uint16_t *)out->v_scale);
    return launch_status();
}

int32_t tq_decode_kv(const tq_packed_kv *in, int64_t tokens, int32_t heads, const tq_config *cfg, void *k_out,
                     void *v_out, int32_t out_dtype, int32_t flags, void *stream)
{
    if (cfg == nullptr || in == nullptr) return TQ_E_NULL;
    if (k_out == nullptr && v_out == nullptr) return TQ_E_NULL;
    if (!valid_head_dim(cfg->head_dim)) return TQ_E_HEAD_DIM;
    if (out_dtype != TQ_F32 && out_dtype != TQ_BF16) return TQ_E_DTYPE;
    if ((flags & ~TQ_DECODE_ROTATED_V) != 0) return TQ_E_SHAPE;
    if (k_out != nullptr) {
        if (!valid_bits(cfg->k_bits) || (cfg->k_signed != 0 && cfg->k_bits != 8) ||
            (cfg->k_signed != 0 && cfg->k_signed != 1))
            return TQ_E_BITS;
        if (in->k_codes == nullptr || in->k_scale == nullptr || in->k_zero == nullptr) return TQ_E_NULL;
        if (!aligned(k_out, 16) || !aligned(in->k_codes, code_align(cfg->k_bits)) || !aligned(in->k_scale, 2) ||
            !aligned(in->k_zero, 2))
            return TQ_E_ALIGN;
    }
    if (v_out != nullptr) {
        if (!valid_bits(cfg->v_bits)) return TQ_E_BITS;
        if (in->v_codes == nullptr || in->v_scale == nullptr) return TQ_E_NULL;
        if (!aligned(v_out, 16) || !aligned(in->v_codes, code_align(cfg->v_bits)) || !aligned(in->v_scale, 2))
            return TQ_E_ALIGN;
    }
    int64_t rows = 0;
    const int32_t st = check_rows(tokens, heads, &rows);
    if (st != TQ_OK) return st;
    if (rows == 0) return TQ_OK;
    const int32_t vb = (v_out != nullptr) ? cfg->v_bits : 4;
    DecodeFn fn = (out_dtype == TQ_BF16) ? pick_decode<true>(cfg->head_dim, vb) : pick_decode<false>(cfg->head_dim, vb);
    const int32_t kmode = (k_out != nullptr) ? key_mode(cfg) : KMODE_NONE;
    hipLaunchKernelGGL(fn, dim3((uint32_t)grid_for(rows, cfg->head_dim)), dim3(kBlockThreads), 0,
                       (hipStream_t)stream, (const uint8_t *)in->k_codes, (const uint16_t *)in->k_scale,
                       (const uint16_t *)in->k_zero, (const uint8_t *)in->v_codes, (const uint16_t *)in->v_scale,
                       rows, kmode, (int32_t)((flags & TQ_DECODE_ROTATED_V) != 0), k_out, v_out);
    return launch_status();
}

int32_t tq_unrotate_values(const void *x, void *out, int32_t dtype, int64_t rows, int32_t head_dim, void *stream)
{
    if (x == nullptr || out == nullptr) return TQ_E_NULL;
    if (!valid_head_dim(head_dim)) return TQ_E_HEAD_DIM;
    if (dtype != TQ_F32 && dtype != TQ_BF16) return TQ_E_DTYPE;
    if (rows < 0 || rows > ((int64_t)1 << 44)) return TQ_E_SHAPE;
    if (!aligned(x, 16) || !aligned(out, 16)) return TQ_E_ALIGN;
    if (rows == 0) return TQ_OK;
    UnrotateFn fn = (dtype == TQ_BF16) ? pick_unrotate<true>(head_dim) : pick_unrotate<false>(head_dim);
    hipLaunchKernelGGL(fn, dim3((uint32_t)grid_for(rows, head_dim)), dim3(kBlockThreads), 0, (hipStream_t)stream, x,
                       out, rows);
    return launch_status();
}

int32_t tq_lloyd_max_table(int32_t bits, float *centroids, float *boundaries)
{
    if (!valid_bits(bits)) return TQ_E_BITS;
    const float *c = nullptr, *b = nullptr;
    switch (bits) {
    case 2: c = LM<2>::c; b = LM<2>::b; break;
    case 3: c = LM<3>::c; b = LM<3>::b; break;
    case 4: c = LM<4>::c; b = LM<4>::b; break;
    case 5: c = LM<5>::c; b = LM<5>::b; break;
    default: c = LM<8>::c; b = LM<8>::b; break;
    }
    const int n = 1 << bits;
    if (centroids != nullptr)
        for (int i = 0; i < n; ++i) centroids[i] = c[i];
    if (boundaries != nullptr)
        for (int i = 0; i < n - 1; ++i) boundaries[i] = b[i];
    return TQ_OK;
}

int32_t tq_sign_vector(int32_t head_dim, float *signs)
{
    if (!valid_head_dim(head_dim)) return TQ_E_HEAD_DIM;
    if (signs == nullptr) return TQ_E_NULL;
    const uint32_t *m = head_dim == 64 ? kSignMask64 : head_dim == 128 ? kSignMask128
                      : head_dim == 256 ? kSignMask256 : kSignMask512;
    for (int i = 0; i < head_dim; ++i) signs[i] = ((m[i / 32] >> (i % 32)) & 1u) ? -1.0f : 1.0f;
    return TQ_OK;
}

int32_t tq_value_bin_host(int32_t bits, const float *z, int64_t n, uint8_t *idx)
{
    if (!valid_bits(bits)) return TQ_E_BITS;
    if (n < 0) return TQ_E_SHAPE;
    if (n > 0 && (z == nullptr || idx == nullptr)) return TQ_E_NULL;
    static constexpr BinLut<2> l2{};
    static constexpr BinLut<3> l3{};
    static constexpr BinLut<4> l4{};
    static constexpr BinLut<5> l5{};
    static constexpr BinLut<8> l8{};
    for (int64_t i = 0; i < n; ++i) {
        uint32_t r = 0;
        switch (bits) {
        case 2: r = bin_index<2>(z[i], l2.cell); break;
        case 3: r = bin_index<3>(z[i], l3.cell); break;
        case 4: r = bin_index<4>(z[i], l4.cell); break;
        case 5: r = bin_index<5>(z[i], l5.cell); break;
        default: r = bin_index<8>(z[i], l8.cell); break;
        }
        idx[i] = (uint8_t)r;
    }
    return TQ_OK;
}

} // extern "C"
