// tq_attn.hip -- attention of one query token per sequence over a packed
// cache, decoding inside the attention kernel.
//
// The page "@mlx-bun/inference 0.0.0-stage -> 1.0.0", ops.ts
// (decodeValuesRotated, unrotateValues) describes the read path: keys are
// decoded (decodeKeys: (q + zero) * scale, bf16), values only to the
// rotated domain (centroid * scale, bf16), attention runs on those, and --
// attention being linear in V -- the output is un-rotated once per query
// row instead of every cached token being un-rotated. Here the decoding
// happens in registers inside the attention kernel, so the cache is read
// in its packed form (152 bytes per token and KV head at head_dim 128 with
// 4-bit keys and values, against 512 for a decoded bf16 cache).
//
// Split over the token axis (flash decoding). attn_partial_kernel: one
// block per (sequence, KV head, split of 4 * wave_tokens tokens), each of
// its wavefronts an independent range of wave_tokens tokens, merged at the
// end of the block; the contractions run on the matrix cores. The number
// of splits fills the GPU with one round of resident blocks.
// attn_combine_kernel merges the splits' (max, sum, output) triples of a
// row and applies the inverse rotation (the codec's transform, then the
// sign vector).
#include <hip/hip_runtime.h>

#include <math.h>

#include <map>
#include <mutex>
#include <tuple>

#include "tq.h"
#include "tq_device.h"
#include "tq_host.h"

namespace {

constexpr int kAttnMaxG = 8;         // query heads per KV head
constexpr int kAttnMaxTargetBlocks = 2048; // blocks per launch aimed at, at most
constexpr int kAttnMaxSplits = kAttnMaxTargetBlocks; // splits per (sequence, KV head), at most
constexpr int kAttnMinWaveTokens = 32;

struct AttnParams {
    const void *q;
    const uint8_t *kc;
    const uint16_t *ks;
    const uint16_t *kz;
    const uint8_t *vc;
    const uint16_t *vs;
    const int32_t *left_pad;
    float *part;
    int64_t width;
    int32_t batch, hkv, g, nsplit, q_bf16, q_terms;
    int32_t wave_tokens; // tokens per wavefront; a block (split) covers 4 wavefronts' worth
    float scale;
};

// partial results: per (sequence, query head, split = block) D outputs,
// then the running max and sum (stride D + 4 keeps rows 16-byte aligned)
template <int D> __device__ __forceinline__ float *part_row(const AttnParams &p, int b, int h, int sp)
{
    const int hq = p.hkv * p.g;
    return p.part + (((int64_t)b * hq + h) * p.nsplit + sp) * (D + 4);
}

// max and sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 with the lane
// swaps of gfx950 (v_permlane16_swap exchanges 16-lane rows 1 and 3 of its
// first operand with rows 0 and 2 of its second, v_permlane32_swap the upper
// half of the first with the lower half of the second; with both operands
// equal to x, each lane ends up holding x from itself and from its partner).
// The second operand goes through an empty asm so that the compiler cannot
// treat the two results as equal.
template <bool MAX> __device__ __forceinline__ float swap_combine(float x, bool wide)
{
    uint32_t a = as_u(x), c = a;
    asm("" : "+v"(c));
    uint32_t r0, r1;
    if (wide) {
        const auto r = __builtin_amdgcn_permlane32_swap(a, c, false, false);
        r0 = r[0];
        r1 = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane16_swap(a, c, false, false);
        r0 = r[0];
        r1 = r[1];
    }
    return MAX ? fmaxf(as_f(r0), as_f(r1)) : as_f(r0) + as_f(r1);
}

__device__ __forceinline__ float rows_max(float x) { return swap_combine<true>(swap_combine<true>(x, false), true); }
__device__ __forceinline__ float rows_sum(float x) { return swap_combine<false>(swap_combine<false>(x, false), true); }

// ---------------------------------------------------------------------------
// Matrix-core operands. One wavefront tile is 16 tokens of one (sequence, KV
// head). Lane l = 16 g + h (h = l % 16, g = l / 16):
//
//   scores  S[16 tokens x 16 heads] += K[tokens x 32] * Q^T[32 x heads]
//           (v_mfma_f32_16x16x32_bf16, one per 32 of the head_dim): lane l
//           supplies the key of token h and the query of head h, 8 elements
//           each, elements s * D/4 + 8 c + [0, 8) for s = g (so a lane decodes
//           one quarter of its token's key row); it receives S[tokens 4 g ..
//           4 g + 3][head h].
//   output  O[16 dims x 16 heads] += V^T[dims x 16 tokens] * P^T[tokens x heads]
//           (v_mfma_f32_16x16x16_bf16, one per output slice and weight term;
//           slice n, n < W = D / 16, holds the 16 dims W m + n, m = 0 .. 15):
//           lane l supplies V[tokens 4 g .. 4 g + 3][dim W h + n] and the
//           weights of those same tokens for head h -- exactly the scores it
//           received, so the softmax needs no data movement; it accumulates
//           O[dims W (4 g + i) + n, i = 0 .. 3][head h]. Over all slices a
//           lane's value operands are the W consecutive dims [W h, W h + W)
//           of its four tokens, which it decodes itself from the packed rows
//           (no transposition through LDS).
//
// Query heads beyond the KV head's group read an all-zero row and their
// results are never used. Keys and values are bf16 (the decoders' output
// type), so their products are exact; the binary32 query and weights enter
// as sums of three bf16 terms (t0 = bf16(x), t1 = bf16(x - t0), t2 =
// bf16(x - t0 - t1), each difference exact), which keeps the contraction
// within the rounding of binary32 arithmetic. The matrix cores accumulate
// in binary32.
// ---------------------------------------------------------------------------

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;                 // tokens per wavefront tile
constexpr int kQRows = kAttnMaxG + 1;     // query rows in LDS; the last is zeros
constexpr int kMaxQTerms = 3;

template <int D> constexpr int kQueryRow = D + 8; // elements per query row in LDS

// One lane's quarter of a packed row: elements [s D/4, (s+1) D/4), held as
// the code words of the groups it covers (a half group at D = 64, shifted so
// that its first code is code 0) and their fp16 scales (and key zeros),
// packed two to a word when the quarter covers several groups.
template <int D, int B> struct Quarter {
    static constexpr int E = D / 4;
    static constexpr int NG = E >= kGroup ? E / kGroup : 1;
    static constexpr int NSW = (NG + 1) / 2; // scale words
    uint32_t w[NG][B];
    uint32_t sc[NSW], zr[NSW];
    __device__ __forceinline__ uint16_t scale(int gi) const { return (uint16_t)(sc[gi / 2] >> (16 * (gi & 1))); }
    __device__ __forceinline__ uint16_t zero(int gi) const { return (uint16_t)(zr[gi / 2] >> (16 * (gi & 1))); }
};

template <int NSW> __device__ __forceinline__ void load_scales(const uint8_t *p, uint32_t (&s)[NSW], bool pair)
{
    if constexpr (NSW == 1) {
        s[0] = pair ? *reinterpret_cast<const uint32_t *>(p) : (uint32_t)*reinterpret_cast<const uint16_t *>(p);
    } else {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        s[0] = v.x;
        s[1] = v.y;
    }
}

// codes from the tile's first row `codes` (uniform) at lane byte offset
// `off` (the lane's token row plus, at D >= 128, its quarter); scales from
// `scale` (+ `zero`) at lane byte offset `soff`. Loads only: at D = 64 the
// half group still has to be moved into place by finish_quarter, so that a
// prefetched tile's loads stay in flight until the tile is used.
template <int D, int B, bool ZERO>
__device__ __forceinline__ void load_quarter(const uint8_t *codes, const uint8_t *scale, const uint8_t *zero,
                                             uint32_t off, uint32_t soff, Quarter<D, B> &q)
{
    using Q = Quarter<D, B>;
    if constexpr (Q::E >= kGroup) {
#pragma unroll
        for (int gi = 0; gi < Q::NG; ++gi) {
            const uint32_t o = off + gi * (4 * B);
            load_codes<B>(codes + o, q.w[gi]);
        }
    } else {
        load_codes<B>(codes + off, q.w[0]);
    }
    load_scales<Q::NSW>(scale + soff, q.sc, Q::NG == 2);
    if constexpr (ZERO) load_scales<Q::NSW>(zero + soff, q.zr, Q::NG == 2);
}

// at D = 64 a lane with odd s holds the upper half of its group: shift it
// down so that its first code is code 0
template <int D, int B> __device__ __forceinline__ void finish_quarter(Quarter<D, B> &q, int s)
{
    using Q = Quarter<D, B>;
    if constexpr (Q::E < kGroup) {
        uint32_t t[B];
#pragma unroll
        for (int i = 0; i < B; ++i) t[i] = q.w[0][i];
        constexpr int sh_bits = kGroup / 2 * B, wo = sh_bits / 32, bs = sh_bits % 32;
        const bool upper = (s & 1) != 0;
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const uint32_t lo = i + wo < B ? t[i + wo] : 0u;
            const uint32_t hi = i + wo + 1 < B ? t[i + wo + 1] : 0u;
            const uint32_t sh = bs != 0 ? __builtin_amdgcn_alignbit(hi, lo, bs) : lo;
            q.w[0][i] = upper ? sh : t[i];
        }
    }
}

// the 8 codes first .. first + 7 (first a multiple of 8) of a group's words
// as integers; 4-bit codes are split into bytes with two masks, 8-bit codes
// are bytes already
template <int B> __device__ __forceinline__ void codes8(const uint32_t (&w)[B], int first, uint32_t (&c)[8])
{
    if constexpr (B == 4) {
        const uint32_t x = w[first / 8];
        uint32_t lo = x & 0x0f0f0f0fu, hi = (x >> 4) & 0x0f0f0f0fu;
        // hide the masks from the optimiser, which would otherwise fold
        // them into a shift and mask per code instead of byte selects
        asm("" : "+v"(lo));
        asm("" : "+v"(hi));
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            c[2 * m] = (lo >> (8 * m)) & 0xffu;
            c[2 * m + 1] = (hi >> (8 * m)) & 0xffu;
        }
    } else if constexpr (B == 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = (w[(first + u) / 4] >> (8 * ((first + u) % 4))) & 0xffu;
    } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = unpack1<B>(w, first + u);
    }
}

// 4-bit key codes are converted two at a time by reading them as FP8 (E4M3)
// bytes: a byte 0 .. 15 has exponent field 0 or 1 and so encodes the integer
// times the format's smallest subnormal, a power of two (2^-9 in the OCP
// encoding). kKeyUnit(KB) is the factor a code's float carries: that power
// of two for 4-bit unsigned codes, 1 otherwise (plain integer conversion).
template <int KB, bool KS> constexpr bool kFp8Codes = KB == 4 && !KS;
__device__ __forceinline__ float fp8_code_unit()
{
    return __builtin_amdgcn_cvt_pk_f32_fp8(0x0101, false)[0];
}

// elements 8 c .. 8 c + 7 of the quarter's key codes as floats, each the
// code times the unit above (exact: the codes have at most 8 bits)
template <int D, int KB, bool KS>
__device__ __forceinline__ void key_code_floats(const Quarter<D, KB> &k, int c, float (&f)[8])
{
    const int gi = Quarter<D, KB>::NG > 1 ? 8 * c / kGroup : 0;
    if constexpr (kFp8Codes<KB, KS>) {
        // nibbles 0 .. 7 of the word are codes 8 c .. 8 c + 7; masks put the
        // even codes in the bytes of lo and the odd ones in those of hi
        const uint32_t x = k.w[gi][(8 * c) % kGroup / 8];
        const uint32_t lo = x & 0x0f0f0f0fu, hi = (x >> 4) & 0x0f0f0f0fu;
        const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false), b = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
        const auto e = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false), o = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
        f[0] = a[0], f[2] = a[1], f[4] = b[0], f[6] = b[1];
        f[1] = e[0], f[3] = e[1], f[5] = o[0], f[7] = o[1];
    } else {
        uint32_t q[8];
        codes8<KB>(k.w[gi], (8 * c) % kGroup, q);
#pragma unroll
        for (int u = 0; u < 8; ++u) f[u] = KS ? (float)(int32_t)(int8_t)(uint8_t)q[u] : (float)q[u];
    }
}

// decodeKeys ((q + zero) * scale, rounded to bf16) of elements 8 c .. 8 c + 7
// of the quarter, as packed bf16 pairs, from the codes as floats f (code
// times unit). FMA: as fma(f, scale / unit, zero * scale) (su = scale / unit,
// zs = zero * scale), used when every group of the wavefront's tile has a
// finite nonzero scale and a finite zero point: a code has at most 8
// significant bits and an fp16 scale or zero at most 11, so both products
// are exact in binary32 (unit being a power of two), q + zero is an exact
// integer, and the fma's single rounding is that of (q + zero) * scale.
// Otherwise the two-step form on q = f / unit (which also fixes the sign of
// a zero result).
template <int D, int KB, bool FMA>
__device__ __forceinline__ u32x4_t key_chunk(const float (&f)[8], int c, float inv_unit, const Quarter<D, KB> &k,
                                             const float (&su)[Quarter<D, KB>::NG],
                                             const float (&zs)[Quarter<D, KB>::NG])
{
    const int gi = Quarter<D, KB>::NG > 1 ? 8 * c / kGroup : 0;
    const float sc = FMA ? 0.0f : f16_bits_to_f32(k.scale(gi)), zr = FMA ? 0.0f : f16_bits_to_f32(k.zero(gi));
    u32x4_t r;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        float y[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const float x = f[2 * w + u];
            y[u] = FMA ? __builtin_fmaf(x, su[gi], zs[gi]) : (x * inv_unit + zr) * sc;
        }
        r[w] = pack_bf16x2(y[0], y[1]);
    }
    return r;
}

// One lane's values of a tile: tokens 4 g + i (i = 0 .. 3), dims [W h, W h
// + W), W = D / 16 (inside one group, W dividing 32): per token the window's
// code bits shifted to start at bit 0, and the group's fp16 scale.
template <int D, int VB> struct VWin {
    static constexpr int W = D / 16;          // dims of a window
    static constexpr int WB = W * VB;         // its code bits
    static constexpr int NW = (WB + 31) / 32; // words of a window from bit 0
    // words covering lane h's window, which starts at bit WB h of the row
    static constexpr int need(int h) { return ((WB * h) % 32 + WB + 31) / 32; }
    static constexpr int most_words()
    {
        int m = 0;
        for (int h = 0; h < 16; ++h) m = need(h) > m ? need(h) : m;
        return m;
    }
    static constexpr bool same_for_all()
    {
        for (int h = 0; h < 16; ++h)
            if (need(h) != most_words()) return false;
        return true;
    }
    static constexpr int RW = most_words(); // words loaded per token, at most
    static constexpr bool ALL = same_for_all(); // every lane loads RW words
    uint32_t w[4][NW];
    uint32_t sc[2]; // fp16 scales, token 2 k + u in bits 16 u of word k
    __device__ __forceinline__ float scale(int i) const { return f16_bits_to_f32((uint16_t)(sc[i / 2] >> (16 * (i & 1)))); }
};

// the words covering the windows of the lane's four tokens, from the tile's
// first code row `codes`, and their group scales from the first scale row
// `scales`; voff[i] and soff[i]: the byte offsets of token i's first word
// and of its scale. A lane loads only the words its window covers, so that
// no read passes the end of the last row. Loads only (see finish_vwin).
template <int D, int VB> struct VRaw {
    uint32_t r[4][VWin<D, VB>::RW];
    uint32_t s[4];
};
template <int D, int VB>
__device__ __forceinline__ void load_vwin(const uint8_t *codes, const uint8_t *scales, const uint32_t (&voff)[4],
                                          const uint32_t (&soff)[4], int h, VRaw<D, VB> &v)
{
    using V = VWin<D, VB>;
    const uint32_t sh = (uint32_t)(V::WB * h) % 32;
    const uint32_t nw = (sh + V::WB + 31) / 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(codes + voff[i]);
#pragma unroll
        for (int k = 0; k < V::RW; ++k) v.r[i][k] = (V::ALL || k == 0 || (uint32_t)k < nw) ? src[k] : 0u;
        v.s[i] = *reinterpret_cast<const uint16_t *>(scales + soff[i]);
    }
}

// the windows shifted to start at bit 0, and the scales two to a word
template <int D, int VB> __device__ __forceinline__ void finish_vwin(const VRaw<D, VB> &raw, int h, VWin<D, VB> &v)
{
    using V = VWin<D, VB>;
    const uint32_t sh = (uint32_t)(V::WB * h) % 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int k = 0; k < V::NW; ++k)
            v.w[i][k] = __builtin_amdgcn_alignbit(k + 1 < V::RW ? raw.r[i][k + 1] : 0u, raw.r[i][k], sh);
    }
    v.sc[0] = raw.s[0] | (raw.s[1] << 16);
    v.sc[1] = raw.s[2] | (raw.s[3] << 16);
}

// byte offsets within a tile of the lane's value windows and scales for
// tokens t0 + i, i = 0 .. 3, clamped to the tile's last valid token nv - 1
template <int D, int VB>
__device__ __forceinline__ void vwin_offsets(int t0, int h, int nv, uint32_t vstride, uint32_t sstride,
                                             uint32_t (&voff)[4], uint32_t (&soff)[4])
{
    using V = VWin<D, VB>;
    const uint32_t wo = (uint32_t)(V::WB * h) / 32 * 4, so = (uint32_t)(V::W * h / kGroup) * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t t = (uint32_t)(t0 + i < nv ? t0 + i : nv - 1);
        voff[i] = t * vstride + wo;
        soff[i] = t * sstride + so;
    }
}

// Value lookup table in LDS. With pairs (VB < 8), entry (c1 << VB) | c0
// holds the centroids of c0 and c1 (8 bytes), so that two consecutive codes
// -- one 2 VB-bit field of a window -- are looked up at once; otherwise the
// centroids themselves (4 bytes each).
template <int VB> constexpr bool kPairTable = VB < 8;
template <int VB> constexpr int kVTabBytes = kPairTable<VB> ? (8 << (2 * VB)) : (4 << VB);

// byte offset in the table of field i of a window: pair i (codes 2 i,
// 2 i + 1) with pairs, else code i
template <int VB, int NW> __device__ __forceinline__ uint32_t vtab_offset(const uint32_t (&w)[NW], int i)
{
    constexpr int FB = kPairTable<VB> ? 2 * VB : VB; // bits of a field
    constexpr int LS = kPairTable<VB> ? 3 : 2;       // log2 of an entry's bytes
    constexpr uint32_t M = ((1u << FB) - 1) << LS;
    const int p = FB * i - LS;                       // where the scaled field starts
    if (p < 0) return (w[0] << LS) & M;
    const int k = p / 32, s = p % 32;
    const uint32_t x = (s + FB + LS <= 32) ? (w[k] >> s) : __builtin_amdgcn_alignbit(w[k + 1], w[k], s);
    return x & M;
}

// the centroids of the lane's operands of output slices 2 i and 2 i + 1:
// c0[t], c1[t] for dims W h + 2 i and W h + 2 i + 1 of token 4 g + t
struct VLook {
    float c0[4], c1[4];
};
template <int D, int VB>
__device__ __forceinline__ void value_lookup(const VWin<D, VB> &v, int i, const uint8_t *tab, VLook &l)
{
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        if constexpr (kPairTable<VB>) {
            const float2 c = *reinterpret_cast<const float2 *>(tab + vtab_offset<VB>(v.w[t], i));
            l.c0[t] = c.x;
            l.c1[t] = c.y;
        } else {
            l.c0[t] = *reinterpret_cast<const float *>(tab + vtab_offset<VB>(v.w[t], 2 * i));
            l.c1[t] = *reinterpret_cast<const float *>(tab + vtab_offset<VB>(v.w[t], 2 * i + 1));
        }
    }
}

// decodeValuesRotated (centroid * scale, rounded to bf16) of those
// operands: V[token 4 g + t][dim W h + n], t = 0 .. 3, for n = 2 i (a0) and
// n = 2 i + 1 (a1)
__device__ __forceinline__ void value_operands(const VLook &l, const float (&sc)[4], s16x4_t &a0, s16x4_t &a1)
{
    float x[4], y[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        x[t] = l.c0[t] * sc[t];
        y[t] = l.c1[t] * sc[t];
    }
    a0 = __builtin_bit_cast(s16x4_t, u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])});
    a1 = __builtin_bit_cast(s16x4_t, u32x2_t{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])});
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return as_f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return as_f(w & 0xffff0000u); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyMax = 8.0f; // see the softmax in wave_tiles

// The tiles of one wavefront: tokens [t_lo, t_end) of (sequence b, KV
// head j), 16 at a time, with an online softmax per query head in base 2
// (scores scaled by scale * log2(e) and exponentiated with exp2, so the
// running maximum is a base-2 logarithm). QT is the number of bf16 terms of
// the query. Per tile: the packed keys are loaded and their 32-element
// chunks decoded straight into the matrix cores; then the value windows are
// loaded, and after the softmax decoded, slice pair by slice pair, into the
// operands of the weighted sum. tab: the value lookup table.
template <int D, int VB, int KB, bool KS, int QT>
__device__ __forceinline__ void wave_tiles(const AttnParams &p, int b, int j, int64_t t_lo, int64_t t_end,
                                           const uint8_t *tab, const uint16_t *qrow, f32x4_t (&acc)[D / 16],
                                           float &m_run, float &l_run)
{
    using KQ = Quarter<D, KB>;
    using VW = VWin<D, VB>;
    constexpr int G = D / kGroup;
    constexpr int NC = D / 32;  // 32-element chunks of the contraction (and 8-element chunks of a quarter)
    constexpr int NS = D / 16;  // output slices
    constexpr int QR = kQueryRow<D>;
    constexpr uint32_t KROW = D * KB / 8, VROW = D * VB / 8; // code bytes per row
    const int lane = threadIdx.x & (kWave - 1);
    const int h = lane & 15, g = lane >> 4;
    // per-token strides of the planes (a token's rows of all KV heads are
    // adjacent) and the lanes' offsets within a token row
    const uint32_t kstride = (uint32_t)p.hkv * KROW, vstride = (uint32_t)p.hkv * VROW;
    const uint32_t sstride = (uint32_t)p.hkv * G * 2;
    const uint32_t kq_off = KQ::E >= kGroup ? g * (KROW / 4) : (g >> 1) * (4 * KB);
    const uint32_t ks_off = KQ::E >= kGroup ? g * KQ::NG * 2 : (g >> 1) * 2;
    const float sl2 = p.scale * kLog2e;
    // 1 / (the factor a key code's float carries), an exact power of two
    const float inv_unit = kFp8Codes<KB, KS> ? 1.0f / fp8_code_unit() : 1.0f;

    // the lanes' byte offsets within a full tile (key token h, value tokens
    // 4 g + i: the first, plus i token strides); a partial tile clamps them
    // to its last valid token
    const uint32_t koff_full = h * kstride + kq_off, ksoff_full = h * sstride + ks_off;
    uint32_t voff0, vsoff0;
    {
        uint32_t vo[4], so[4];
        vwin_offsets<D, VB>(4 * g, h, kTile, vstride, sstride, vo, so);
        voff0 = vo[0];
        vsoff0 = so[0];
    }

    // the packed key rows of the tile at t0
    auto load_keys = [&](int64_t t0, KQ &kq) {
        const int64_t row0 = ((int64_t)b * p.width + t0) * p.hkv + j;
        const int nv = (int)(t_end - t0 < kTile ? t_end - t0 : kTile);
        uint32_t koff = koff_full, ksoff = ksoff_full;
        if (nv < kTile) { // wavefront-uniform: the wavefront's last tile
            const uint32_t tk = (uint32_t)(h < nv ? h : nv - 1);
            koff = tk * kstride + kq_off;
            ksoff = tk * sstride + ks_off;
        }
        load_quarter<D, KB, true>(p.kc + row0 * KROW, reinterpret_cast<const uint8_t *>(p.ks + row0 * G),
                                  reinterpret_cast<const uint8_t *>(p.kz + row0 * G), koff, ksoff, kq);
    };

    // one tile, from its loaded key rows
    auto tile = [&](int64_t t0, KQ &kq, VRaw<D, VB> &vr) {
        const int nv = (int)(t_end - t0 < kTile ? t_end - t0 : kTile);
        finish_quarter<D, KB>(kq, g);

        // scores of the tile's 16 tokens
        float ksu[KQ::NG], kzs[KQ::NG];
        bool fma_ok = true;
#pragma unroll
        for (int gi = 0; gi < KQ::NG; ++gi) {
            const float ksc = f16_bits_to_f32(kq.scale(gi));
            ksu[gi] = ksc * inv_unit;
            kzs[gi] = f16_bits_to_f32(kq.zero(gi)) * ksc;
            fma_ok = fma_ok && ksc != 0.0f && __builtin_isfinite(kzs[gi]);
        }
        const bool tile_fma = __all(fma_ok);
        f32x4_t S = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
            float kf[8];
            key_code_floats<D, KB, KS>(kq, cc, kf);
            u32x4_t kc;
            if (tile_fma) // wavefront-uniform; the other form is rare
                kc = key_chunk<D, KB, true>(kf, cc, inv_unit, kq, ksu, kzs);
            else
                kc = key_chunk<D, KB, false>(kf, cc, inv_unit, kq, ksu, kzs);
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, kc);
#pragma unroll
            for (int t = 0; t < QT; ++t) {
                const u32x4_t qv = *reinterpret_cast<const u32x4_t *>(qrow + t * (kQRows * QR) + 8 * cc);
                S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, qv), S, 0, 0, 0);
            }
        }

        // the value windows are loaded only now, so that their registers are
        // not held through the key contraction (four wavefronts per SIMD at
        // d = 256)
        {
            const int64_t row0 = ((int64_t)b * p.width + t0) * p.hkv + j;
            uint32_t voff[4], vsoff[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) voff[i] = voff0 + i * vstride, vsoff[i] = vsoff0 + i * sstride;
            if (nv < kTile) vwin_offsets<D, VB>(4 * g, h, nv, vstride, sstride, voff, vsoff);
            load_vwin<D, VB>(p.vc + row0 * VROW, reinterpret_cast<const uint8_t *>(p.vs + row0 * G), voff, vsoff, h, vr);
        }
        VW vw;
        finish_vwin<D, VB>(vr, h, vw);
        // the first slice pair's value lookups, in flight during the softmax
        VLook look;
        value_lookup<D, VB>(vw, 0, tab, look);

        // online softmax: lane (h, g) holds tokens 4 g .. 4 g + 3 for head h
        float s4[4];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s4[i] = 4 * g + i < nv ? S[i] * sl2 : -INFINITY;
            mx = fmaxf(mx, s4[i]);
        }
        mx = rows_max(mx);
        // the reference maximum m_run moves only when the tile's maximum
        // passes it by more than kLazyMax (base 2), so that the accumulators
        // are rescaled rarely; meanwhile the weights exp2(s - m_run) stay
        // below 2^kLazyMax (their three-term split is as exact at any size)
        const bool grow = !(mx <= m_run + kLazyMax);
        const float m_ref = grow ? fmaxf(m_run, mx) : m_run;
        const bool live = m_ref != -INFINITY;
        const float alpha = live ? __builtin_amdgcn_exp2f(m_run - m_ref) : 1.0f;
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = live ? __builtin_amdgcn_exp2f(s4[i] - m_ref) : 0.0f;
        l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
        m_run = m_ref;
        s16x4_t pt[kMaxQTerms];
#pragma unroll
        for (int t = 0; t < kMaxQTerms; ++t) {
            const uint32_t w01 = pack_bf16x2(pr[0], pr[1]), w23 = pack_bf16x2(pr[2], pr[3]);
            pt[t] = __builtin_bit_cast(s16x4_t, u32x2_t{w01, w23});
            pr[0] -= bf16_lo(w01);
            pr[1] -= bf16_hi(w01);
            pr[2] -= bf16_lo(w23);
            pr[3] -= bf16_hi(w23);
        }
        if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
            for (int n = 0; n < NS; ++n) acc[n] *= alpha;
        }

        // weighted values
        float vsc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) vsc[i] = vw.scale(i);
#pragma unroll
        for (int i = 0; i < NS / 2; ++i) {
            // the next pair's lookups go out before this pair's arithmetic
            VLook next;
            if (i + 1 < NS / 2) value_lookup<D, VB>(vw, i + 1, tab, next);
            s16x4_t a0, a1;
            value_operands(look, vsc, a0, a1);
#pragma unroll
            for (int t = 0; t < kMaxQTerms; ++t) {
                acc[2 * i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a0, pt[t], acc[2 * i], 0, 0, 0);
                acc[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a1, pt[t], acc[2 * i + 1], 0, 0, 0);
            }
            look = next;
            // one pair ahead at most: the scheduler would otherwise hoist
            // every pair's lookups to the top (registers for all at once)
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Issue priority falls as the wavefront gets through its range (at 1/2,
    // 3/4 and 7/8 of its tiles). Each SIMD holds one wavefront of each of
    // the blocks on its CU, all with equal work, and the arbiter otherwise
    // favours the oldest: the first blocks dispatched ran ahead and finished
    // early, leaving the last ones to run with fewer wavefronts to hide
    // their loads. A wavefront with more tiles left now wins the arbitration
    // over one further on, so they finish closer together.
    const int n = (int)((t_end - t_lo + kTile - 1) / kTile);
    const int q1 = n / 2, q2 = 3 * n / 4, q3 = 7 * n / 8;
    int i = 0;
    for (int64_t t0 = t_lo; t0 < t_end; t0 += kTile, ++i) {
        if (i == 0)
            __builtin_amdgcn_s_setprio(3);
        else if (i == q1)
            __builtin_amdgcn_s_setprio(2);
        else if (i == q2)
            __builtin_amdgcn_s_setprio(1);
        else if (i == q3)
            __builtin_amdgcn_s_setprio(0);
        KQ kq;
        VRaw<D, VB> vr;
        load_keys(t0, kq);
        tile(t0, kq, vr);
    }
    __builtin_amdgcn_s_setprio(0);
}

// Dynamic LDS of a partial block: the query terms [q_terms][kQRows][D + 8]
// bf16; after the tiles the same bytes hold the merge area, two slots of
// [g][D + 4] floats.
template <int D> constexpr int kMergeRow = D + 4;
int64_t partial_lds_bytes(int d, int q_terms, int g)
{
    const int64_t query = (int64_t)q_terms * kQRows * (d + 8) * 2;
    const int64_t merge = (int64_t)2 * g * (d + 4) * 4;
    return query > merge ? query : merge;
}

// Register budget: four wavefronts per SIMD where the tile state fits in 128
// VGPRs without spilling (every d <= 128; d = 256 below 8-bit codes); three
// otherwise at d = 256; whatever d = 512 needs (its accumulators alone take
// 128).
template <int D, int VB, int KB> constexpr int kAttnWaves = D >= 512 ? 1 : (D == 256 && (VB == 8 || KB == 8)) ? 3 : 4;

// Blocks are ordered so that the KV heads of one (sequence, chunk) are
// dispatched to the same XCD one after another (dispatch deals block ids
// to the 8 XCDs in turn): block id -> XCD x = id % 8, slot r = id / 8,
// head j = r % hkv, chunk group (r / hkv) * 8 + x. The heads' rows of a
// token are adjacent in the planes, so they share cache lines. Each
// wavefront of a block is an independent range of wave_tokens tokens (see
// wave_tiles); the four are merged at the end of the block.
template <int D, int VB, int KB, bool KS>
__global__ void __launch_bounds__(kBlockThreads) __attribute__((amdgpu_waves_per_eu(kAttnWaves<D, VB, KB>)))
attn_partial_kernel(AttnParams p)
{
    constexpr int NS = D / 16;  // output slices
    constexpr int W = D / 16;   // slice n holds dims W m + n
    constexpr int QR = kQueryRow<D>;
    constexpr int SR = kMergeRow<D>;
    __shared__ __align__(16) uint8_t tab[kVTabBytes<VB>];
    __shared__ float ml[kWavesPerBlock][kAttnMaxG][2];
    extern __shared__ __align__(16) uint8_t lds[];
    uint16_t *qlds = reinterpret_cast<uint16_t *>(lds);

    const int id = blockIdx.x;
    const int x = id % 8, r = id / 8;
    const int j = r % p.hkv;
    const int cg = (r / p.hkv) * 8 + x;
    if (cg >= p.batch * p.nsplit) return;
    const int b = cg / p.nsplit, c = cg % p.nsplit;
    const int gq = p.g, hq = p.hkv * p.g;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int h = lane & 15, g = lane >> 4;
    const int64_t pad = p.left_pad != nullptr ? p.left_pad[b] : 0;
    const int64_t w0 = ((int64_t)c * kWavesPerBlock + wave) * p.wave_tokens;
    const int64_t t_lo = w0 > pad ? w0 : pad;
    const int64_t t_end = w0 + p.wave_tokens < p.width ? w0 + p.wave_tokens : p.width;
    // The loads of the block's table copy, then those of its query copy, are
    // issued in groups ahead of their LDS writes (loops that wrote each
    // load's data before the next load took a memory round trip per step).
    const float *cent = dev_cent<VB>();
    constexpr int NT = kPairTable<VB> ? 1 << (2 * VB) : 1 << VB; // table entries
    constexpr int TK = (NT + kBlockThreads - 1) / kBlockThreads;
    float c0[TK], c1[TK];
#pragma unroll
    for (int k = 0; k < TK; ++k) {
        const int i = tid + k * kBlockThreads < NT ? tid + k * kBlockThreads : 0;
        c0[k] = cent[kPairTable<VB> ? i & ((1 << VB) - 1) : i];
        c1[k] = kPairTable<VB> ? cent[i >> VB] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < TK; ++k) {
        const int i = tid + k * kBlockThreads;
        if (i < NT) {
            if constexpr (kPairTable<VB>)
                reinterpret_cast<float2 *>(tab)[i] = make_float2(c0[k], c1[k]);
            else
                reinterpret_cast<float *>(tab)[i] = c0[k];
        }
    }
    // the query rows of the group (zeros beyond it), 8 elements per thread
    // and step
    constexpr int D8 = D / 8, QN = kQRows * D8, QK = (QN + kBlockThreads - 1) / kBlockThreads;
    uint4 qw[QK][2];
#pragma unroll
    for (int k = 0; k < QK; ++k) {
        const int i = tid + k * kBlockThreads, e = i / D8, k8 = (i % D8) * 8;
        qw[k][0] = qw[k][1] = make_uint4(0u, 0u, 0u, 0u);
        if (i < QN && e < gq) {
            const int64_t qi = ((int64_t)b * hq + j * gq + e) * D + k8;
            if (p.q_bf16) {
                qw[k][0] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p.q) + qi);
            } else {
                qw[k][0] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(p.q) + qi);
                qw[k][1] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(p.q) + qi + 4);
            }
        }
    }
    // as q_terms bf16 terms (a bf16 query is its one term)
#pragma unroll
    for (int k = 0; k < QK; ++k) {
        const int i = tid + k * kBlockThreads, e = i / D8, k8 = (i % D8) * 8;
        if (i >= QN) continue;
        float xq[8];
        if (p.q_bf16) {
            const uint32_t w[4] = {qw[k][0].x, qw[k][0].y, qw[k][0].z, qw[k][0].w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                xq[2 * u] = bf16_lo(w[u]);
                xq[2 * u + 1] = bf16_hi(w[u]);
            }
        } else {
            const uint32_t w[8] = {qw[k][0].x, qw[k][0].y, qw[k][0].z, qw[k][0].w,
                                   qw[k][1].x, qw[k][1].y, qw[k][1].z, qw[k][1].w};
#pragma unroll
            for (int u = 0; u < 8; ++u) xq[u] = as_f(w[u]);
        }
        for (int t = 0; t < p.q_terms; ++t) {
            uint32_t w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                w[u] = pack_bf16x2(xq[2 * u], xq[2 * u + 1]);
                xq[2 * u] -= bf16_lo(w[u]);
                xq[2 * u + 1] -= bf16_hi(w[u]);
            }
            *reinterpret_cast<uint4 *>(&qlds[(t * kQRows + e) * QR + k8]) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
    __syncthreads();

    const uint16_t *qrow = qlds + (h < gq ? h : kAttnMaxG) * QR + g * (D / 4);

    f32x4_t acc[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) acc[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;
    if (p.q_terms == 1)
        wave_tiles<D, VB, KB, KS, 1>(p, b, j, t_lo, t_end, tab, qrow, acc, m_run, l_run);
    else
        wave_tiles<D, VB, KB, KS, kMaxQTerms>(p, b, j, t_lo, t_end, tab, qrow, acc, m_run, l_run);

    // merge the block's four wavefront splits: each scales its sums to the
    // block's maximum, wavefronts 2 and 3 hand theirs to 0 and 1 through two
    // slots of [head][dim] floats (dim W m + n at n * 16 + m) over the query
    // terms, which the tiles no longer use, 0 and 1 leave their sums there,
    // and the block writes the row (a0 + a2) + (a1 + a3) from both slots
    l_run = rows_sum(l_run);
    if (h < gq && g == 0) {
        ml[wave][h][0] = m_run;
        ml[wave][h][1] = l_run;
    }
    __syncthreads();
    const bool mine = h < gq;
    if (mine) {
        float M = ml[0][h][0];
#pragma unroll
        for (int v = 1; v < kWavesPerBlock; ++v) M = fmaxf(M, ml[v][h][0]);
        const float f = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - M);
#pragma unroll
        for (int n = 0; n < NS; ++n) acc[n] *= f;
    }
    float *slot0 = reinterpret_cast<float *>(lds), *slot1 = slot0 + gq * SR;
    float *own = (wave & 1) ? slot1 : slot0; // the slot of wavefronts 1 and 3 / 0 and 2
    if (wave >= 2 && mine) {
#pragma unroll
        for (int n = 0; n < NS; ++n) *reinterpret_cast<f32x4_t *>(&own[h * SR + n * 16 + 4 * g]) = acc[n];
    }
    __syncthreads();
    if (wave < 2 && mine) {
        // each lane reads and rewrites only its own positions
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            f32x4_t *q = reinterpret_cast<f32x4_t *>(&own[h * SR + n * 16 + 4 * g]);
            *q = acc[n] + *q;
        }
    }
    __syncthreads();
    for (int i = tid; i < gq * D; i += kBlockThreads) {
        const int e = i / D, k = i % D;
        float *row = part_row<D>(p, b, j * gq + e, c);
        const int at = e * SR + (k % W) * 16 + k / W;
        row[k] = slot0[at] + slot1[at];
        if (k == 0) {
            float M = ml[0][e][0];
#pragma unroll
            for (int v = 1; v < kWavesPerBlock; ++v) M = fmaxf(M, ml[v][e][0]);
            float L = 0.0f;
#pragma unroll
            for (int v = 0; v < kWavesPerBlock; ++v) {
                const float f = ml[v][e][0] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml[v][e][0] - M);
                L = fmaf(ml[v][e][1], f, L);
            }
            row[D] = M;
            row[D + 1] = L;
        }
    }
}

// One block per output row (sequence, query head): the row's split
// partials (weighted sum o_s, base-2 maximum m_s and normaliser l_s per
// split) merged -- the splits' maxima and normalisers are staged in LDS,
// M = max m_s and L = sum l_s 2^(m_s - M) reduced over the block, then
// thread (4-dim column c, split group k) sums o_s 2^(m_s - M) over splits
// k, k + KS, ... (independent loads), the groups are added through LDS and
// o_rot = o / L -- and the inverse rotation (the codec's transform, then
// the sign vector) applied by the first wavefront, written as out_dtype.
template <int D>
__global__ void __launch_bounds__(kBlockThreads) attn_combine_kernel(const float *part, int32_t nsplit, void *out,
                                                                     int32_t out_bf16)
{
    constexpr int C4 = D / 4;              // float4 columns of a row
    constexpr int KS = kBlockThreads / C4; // split groups
    constexpr int G = D / kGroup;
    __shared__ f32x4_t acc_s[KS][C4];
    __shared__ float fs[kAttnMaxSplits];   // split maxima, then their weights 2^(m_s - M)
    __shared__ float red[2][kWavesPerBlock];
    __shared__ __align__(16) float orow[D];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, c = tid % C4, k = tid / C4;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const float *base = part + row * nsplit * (int64_t)(D + 4);

    float m = -INFINITY;
    for (int sp = tid; sp < nsplit; sp += kBlockThreads) {
        fs[sp] = base[(int64_t)sp * (D + 4) + D];
        m = fmaxf(m, fs[sp]);
    }
    for (int o = kWave / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) red[0][wave] = m;
    __syncthreads();
    float M = red[0][0];
#pragma unroll
    for (int v = 1; v < kWavesPerBlock; ++v) M = fmaxf(M, red[0][v]);
    float l = 0.0f;
    for (int sp = tid; sp < nsplit; sp += kBlockThreads) {
        const float f = fs[sp] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(fs[sp] - M);
        fs[sp] = f;
        l = fmaf(base[(int64_t)sp * (D + 4) + D + 1], f, l);
    }
    for (int o = kWave / 2; o > 0; o >>= 1) l += __shfl_xor(l, o);
    if (lane == 0) red[1][wave] = l;
    __syncthreads();
    f32x4_t a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
    for (int sp = k; sp < nsplit; sp += KS) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t *>(base + (int64_t)sp * (D + 4) + 4 * c);
        a += v * fs[sp];
    }
    acc_s[k][c] = a;
    __syncthreads();
    if (tid < C4) {
        float L = 0.0f;
#pragma unroll
        for (int v = 0; v < kWavesPerBlock; ++v) L += red[1][v];
        f32x4_t o = acc_s[0][tid];
#pragma unroll
        for (int kk = 1; kk < KS; ++kk) o += acc_s[kk][tid];
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        *reinterpret_cast<f32x4_t *>(&orow[4 * tid]) = o * inv;
    }
    __syncthreads();
    if (tid >= kWave) return;
    // every G-lane group of the first wavefront transforms the row; group 0 writes it
    const int grp = tid % G;
    float y[kGroup];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) y[u] = orow[grp * kGroup + u];
    const Rot<D> rot(grp);
    hadamard<D>(y, rot);
    const uint32_t smask = dev_sign<D>(grp);
    if (tid >= G) return;
    if (out_bf16) {
        uint32_t *o = reinterpret_cast<uint32_t *>(out) + (row * D + grp * kGroup) / 2;
#pragma unroll
        for (int w = 0; w < kGroup / 2; ++w) o[w] = pack_bf16x2(y[2 * w], y[2 * w + 1]) ^ sign_pair_mask(smask, w);
    } else {
        float *o = reinterpret_cast<float *>(out) + row * D + grp * kGroup;
#pragma unroll
        for (int u = 0; u < kGroup; ++u) o[u] = ((smask >> u) & 1u) ? -y[u] : y[u];
    }
}

__global__ void __launch_bounds__(kBlockThreads) attn_zero_kernel(uint32_t *out, int64_t words)
{
    const int64_t i = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
    if (i < words) out[i] = 0u;
}

template <int D, int VB> const void *partial_kernel_k(int kmode)
{
    switch (kmode) {
    case 2: return reinterpret_cast<const void *>(&attn_partial_kernel<D, VB, 2, false>);
    case 3: return reinterpret_cast<const void *>(&attn_partial_kernel<D, VB, 3, false>);
    case 4: return reinterpret_cast<const void *>(&attn_partial_kernel<D, VB, 4, false>);
    case 5: return reinterpret_cast<const void *>(&attn_partial_kernel<D, VB, 5, false>);
    case 8: return reinterpret_cast<const void *>(&attn_partial_kernel<D, VB, 8, false>);
    default: return reinterpret_cast<const void *>(&attn_partial_kernel<D, VB, 8, true>);
    }
}

template <int D> const void *partial_kernel_for(int vb, int kmode)
{
    switch (vb) {
    case 2: return partial_kernel_k<D, 2>(kmode);
    case 3: return partial_kernel_k<D, 3>(kmode);
    case 4: return partial_kernel_k<D, 4>(kmode);
    case 5: return partial_kernel_k<D, 5>(kmode);
    default: return partial_kernel_k<D, 8>(kmode);
    }
}

// Splits (blocks) per (sequence, KV head): about `target` blocks in all,
// each wavefront taking at least kAttnMinWaveTokens tokens (non-decreasing
// in `target`, so the workspace sized for kAttnMaxTargetBlocks covers every
// launch).
int64_t n_splits(int32_t batch, int32_t kv_heads, int64_t width, int64_t target)
{
    if (width <= 0 || batch <= 0 || kv_heads <= 0) return 0;
    int64_t n = (target + (int64_t)batch * kv_heads - 1) / ((int64_t)batch * kv_heads);
    const int64_t most = (width + kWavesPerBlock * kAttnMinWaveTokens - 1) / (kWavesPerBlock * kAttnMinWaveTokens);
    if (n > most) n = most;
    return n < 1 ? 1 : n;
}

// Blocks of a partial kernel resident at once on the current device (its
// occupancy per CU times the CU count), capped at kAttnMaxTargetBlocks: one
// full round of blocks, so that no block waits for another to finish.
int64_t resident_blocks(const void *fn, size_t lds_bytes)
{
    static std::mutex mu;
    static std::map<std::tuple<int, const void *, size_t>, int64_t> known;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return kAttnMaxTargetBlocks;
    const auto key = std::make_tuple(dev, fn, lds_bytes);
    std::lock_guard<std::mutex> lock(mu);
    const auto it = known.find(key);
    if (it != known.end()) return it->second;
    int cus = 0, per_cu = 0;
    int64_t n = kAttnMaxTargetBlocks;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kBlockThreads, lds_bytes) == hipSuccess &&
        cus > 0 && per_cu > 0)
        n = (int64_t)cus * per_cu < kAttnMaxTargetBlocks ? (int64_t)cus * per_cu : kAttnMaxTargetBlocks;
    known[key] = n;
    return n;
}

int64_t wave_tokens(int64_t width, int64_t nsplit)
{
    return nsplit > 0 ? (width + nsplit * kWavesPerBlock - 1) / (nsplit * kWavesPerBlock) : 0;
}

// Split partials of tq_attention_decode_static, for callers that cannot
// allocate: a fixed array in the library's device image (each GPU the
// library runs on holds its own copy until the process ends). Host code
// must not pass `scratch` itself to a kernel (on the host the name is a
// stand-in, not a device address): it uses the address that
// hipGetSymbolAddress returns for the current device.
constexpr int64_t kAttnScratchBytes = (int64_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kAttnScratchBytes];

// The device address of `scratch` on the current device, looked up once per
// device; nullptr if the runtime reports an error.
void *scratch_address()
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        addr[dev] = ptr;
    }
    return addr[dev];
}

// Every argument check of tq_attention_decode except those of the
// workspace, in the order the pages' operations would throw.
int32_t attention_args_status(const void *q, int32_t q_dtype, const tq_packed_kv *cache, int32_t batch,
                              int64_t width, int32_t kv_heads, int32_t q_heads, const tq_config *cfg, float scale,
                              const void *out, int32_t out_dtype)
{
    if (cfg == nullptr || cache == nullptr) return TQ_E_NULL;
    if (!tq_host::valid_head_dim(cfg->head_dim)) return TQ_E_HEAD_DIM;
    if (!tq_host::valid_key_cfg(cfg) || !tq_host::valid_bits(cfg->v_bits)) return TQ_E_BITS;
    if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_E_DTYPE;
    if (out_dtype != TQ_F32 && out_dtype != TQ_BF16) return TQ_E_DTYPE;
    if (batch < 0 || width < 0 || width > ((int64_t)1 << 40) || kv_heads < 1 || q_heads < kv_heads ||
        q_heads % kv_heads != 0 || q_heads / kv_heads > kAttnMaxG || !(scale == scale))
        return TQ_E_SHAPE;
    if (((q_heads / kv_heads) & (q_heads / kv_heads - 1)) != 0) // 1, 2, 4 or 8 query heads per KV head
        return TQ_E_SHAPE;
    if ((int64_t)batch * width * kv_heads > ((int64_t)1 << 40)) return TQ_E_SHAPE;
    if ((int64_t)batch * q_heads > 0x7fffffff) return TQ_E_SHAPE; // one combine block per output row
    if (batch == 0) return TQ_OK;
    if (q == nullptr || out == nullptr) return TQ_E_NULL;
    if (!tq_host::aligned(q, 16) || !tq_host::aligned(out, 16)) return TQ_E_ALIGN;
    if (width > 0) {
        if (cache->k_codes == nullptr || cache->k_scale == nullptr || cache->k_zero == nullptr ||
            cache->v_codes == nullptr || cache->v_scale == nullptr)
            return TQ_E_NULL;
        if (!tq_host::aligned(cache->k_codes, tq_host::code_align(cfg->k_bits)) ||
            !tq_host::aligned(cache->v_codes, tq_host::code_align(cfg->v_bits)) ||
            !tq_host::aligned(cache->k_scale, 8) || !tq_host::aligned(cache->k_zero, 8) ||
            !tq_host::aligned(cache->v_scale, 8))
            return TQ_E_ALIGN;
    }
    return TQ_OK;
}

} // namespace

extern "C" {

int64_t tq_attention_workspace_bytes(int32_t batch, int32_t kv_heads, int32_t q_heads, int32_t head_dim,
                                     int64_t width)
{
    if (batch < 0 || kv_heads < 1 || q_heads < 0 || width < 0 || !tq_host::valid_head_dim(head_dim))
        return -TQ_E_SHAPE;
    if (width == 0) return 0;
    // split partials: D outputs, the maximum and the normaliser per (row, split)
    return (int64_t)batch * q_heads * n_splits(batch, kv_heads, width, kAttnMaxTargetBlocks) * (head_dim + 4) *
           (int64_t)sizeof(float);
}

int32_t tq_attention_decode(const void *q, int32_t q_dtype, const tq_packed_kv *cache, int32_t batch, int64_t width,
                            const int32_t *left_pad, int32_t kv_heads, int32_t q_heads, const tq_config *cfg,
                            float scale, void *out, int32_t out_dtype, void *workspace, int64_t workspace_bytes,
                            void *stream)
{
    const tq_host::TimingScope timing;
    const int32_t st = attention_args_status(q, q_dtype, cache, batch, width, kv_heads, q_heads, cfg, scale, out,
                                             out_dtype);
    if (st != TQ_OK) return st;
    if (batch == 0) return TQ_OK;
    const int32_t d = cfg->head_dim;
    int64_t nch = 0;
    if (width > 0) {
        if (workspace == nullptr) return TQ_E_NULL;
        if (workspace_bytes < tq_attention_workspace_bytes(batch, kv_heads, q_heads, d, width)) return TQ_E_SHAPE;
        if (!tq_host::aligned(workspace, 16)) return TQ_E_ALIGN;
        AttnParams p;
        p.q = q;
        p.kc = static_cast<const uint8_t *>(cache->k_codes);
        p.ks = static_cast<const uint16_t *>(cache->k_scale);
        p.kz = static_cast<const uint16_t *>(cache->k_zero);
        p.vc = static_cast<const uint8_t *>(cache->v_codes);
        p.vs = static_cast<const uint16_t *>(cache->v_scale);
        p.left_pad = left_pad;
        p.part = static_cast<float *>(workspace);
        p.width = width;
        p.batch = batch;
        p.hkv = kv_heads;
        p.g = q_heads / kv_heads;
        p.q_bf16 = q_dtype == TQ_BF16;
        p.q_terms = q_dtype == TQ_BF16 ? 1 : kMaxQTerms;
        p.scale = scale;
        const int kmode = cfg->k_signed ? (8 | 16) : cfg->k_bits;
        const void *fn = d == 64 ? partial_kernel_for<64>(cfg->v_bits, kmode)
                       : d == 128 ? partial_kernel_for<128>(cfg->v_bits, kmode)
                       : d == 256 ? partial_kernel_for<256>(cfg->v_bits, kmode)
                                  : partial_kernel_for<512>(cfg->v_bits, kmode);
        const size_t lds_bytes = (size_t)partial_lds_bytes(d, p.q_terms, p.g);
        nch = n_splits(batch, kv_heads, width, resident_blocks(fn, lds_bytes));
        if (nch > kAttnMaxSplits || wave_tokens(width, nch) > 0x7fffffff) return TQ_E_SHAPE;
        p.nsplit = (int32_t)nch;
        p.wave_tokens = (int32_t)wave_tokens(width, nch);
        const int64_t groups = ((int64_t)batch * nch + 7) / 8;
        const int64_t blocks = groups * 8 * kv_heads;
        if (blocks > 0x7fffffff) return TQ_E_SHAPE;
        void *args[] = {&p};
        const int32_t ls = tq_host::launch_kernel(fn, dim3((uint32_t)blocks), dim3(kBlockThreads), args, lds_bytes,
                                                  (hipStream_t)stream, true, false);
        if (ls != TQ_OK) return ls;
    }
    // merge (rows with no split are zeros) and the inverse rotation
    const int64_t rows = (int64_t)batch * q_heads;
    if (width == 0) {
        // no workspace needed: every row is zero (a fill kernel, not a
        // memset, so that the call can be captured in a graph)
        uint32_t *o32 = static_cast<uint32_t *>(out);
        int64_t words = rows * d * (out_dtype == TQ_BF16 ? 2 : 4) / 4;
        void *argsz[] = {&o32, &words};
        return tq_host::launch_kernel(reinterpret_cast<const void *>(&attn_zero_kernel),
                                      dim3((uint32_t)((words + kBlockThreads - 1) / kBlockThreads)),
                                      dim3(kBlockThreads), argsz, 0, (hipStream_t)stream, true, true);
    }
    const float *cpart = static_cast<const float *>(workspace);
    int32_t nsp = (int32_t)nch;
    int32_t obf = out_dtype == TQ_BF16;
    void *args2[] = {&cpart, &nsp, &out, &obf};
    const void *fn2 = d == 64 ? reinterpret_cast<const void *>(&attn_combine_kernel<64>)
                    : d == 128 ? reinterpret_cast<const void *>(&attn_combine_kernel<128>)
                    : d == 256 ? reinterpret_cast<const void *>(&attn_combine_kernel<256>)
                    : reinterpret_cast<const void *>(&attn_combine_kernel<512>);
    return tq_host::launch_kernel(fn2, dim3((uint32_t)rows), dim3(kBlockThreads), args2, 0, (hipStream_t)stream,
                                  false, true);
}

int32_t tq_attention_decode_static(const void *q, int32_t q_dtype, const tq_packed_kv *cache, int32_t batch,
                                   int64_t width, const int32_t *left_pad, int32_t kv_heads, int32_t q_heads,
                                   const tq_config *cfg, float scale, void *out, int32_t out_dtype, void *stream)
{
    const tq_host::TimingScope timing;
    if (cfg == nullptr) return TQ_E_NULL;
    if (!tq_host::valid_head_dim(cfg->head_dim)) return TQ_E_HEAD_DIM;
    const int64_t need = tq_attention_workspace_bytes(batch, kv_heads, q_heads, cfg->head_dim, width);
    if (need < 0) return (int32_t)-need;
    if (need > kAttnScratchBytes) return TQ_E_SCRATCH;
    const int32_t st = attention_args_status(q, q_dtype, cache, batch, width, kv_heads, q_heads, cfg, scale, out,
                                             out_dtype);
    if (st != TQ_OK) return st;
    void *ws = nullptr;
    if (need > 0 && (ws = scratch_address()) == nullptr) return TQ_E_HIP;
    return tq_attention_decode(q, q_dtype, cache, batch, width, left_pad, kv_heads, q_heads, cfg, scale, out,
                               out_dtype, ws, kAttnScratchBytes, stream);
}

} // extern "C"
