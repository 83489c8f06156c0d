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
// its wavefronts an independent range of wave_tokens tokens (see
// attn_wave), merged at the end of the block.
// attn_merge_kernel merges the splits' (max, sum, output) triples;
// attn_rotate_kernel applies the inverse rotation (the codec's transform,
// then the sign vector). All arithmetic after decoding is binary32.
#include <hip/hip_runtime.h>

#include <math.h>

#include "tq.h"
#include "tq_device.h"
#include "tq_host.h"

namespace {

constexpr int kAttnMaxG = 8;         // query heads per KV head
constexpr int kAttnTargetBlocks = 2048; // about two rounds of resident blocks on 256 CUs
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
    int32_t batch, hkv, g, nsplit, q_bf16, kmode;
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

__device__ __forceinline__ float bf16_round(float x) { return as_f(pack_bf16x2(x, 0.0f) << 16); }

// v from the lane whose index differs in bit O (lanes exchange in pairs):
// DPP for O = 1, 2, ds_swizzle (xor within 32 lanes) for O = 4, 8, 16,
// ds_bpermute for O = 32
template <int O> __device__ __forceinline__ float xor_shuffle(float v)
{
    if constexpr (O == 1)
        return as_f((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u(v), 0xB1, 0xF, 0xF, false)); // quad_perm [1,0,3,2]
    else if constexpr (O == 2)
        return as_f((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u(v), 0x4E, 0xF, 0xF, false)); // quad_perm [2,3,0,1]
    else if constexpr (O == 4 || O == 8 || O == 16)
        return as_f((uint32_t)__builtin_amdgcn_ds_swizzle((int)as_u(v), 0x1F | (O << 10)));
    else
        return __shfl_xor(v, O);
}

// sum over the lanes whose index differs from this one's only in bits
// [log2 LO, log2 HI) (e.g. LO = 1, HI = G: the G lanes of a token)
template <int LO, int HI> __device__ __forceinline__ float xor_sum(float v)
{
    if constexpr (LO < HI) {
        v += xor_shuffle<LO>(v);
        return xor_sum<2 * LO, HI>(v);
    } else {
        return v;
    }
}

template <int LO, int HI> __device__ __forceinline__ float xor_max(float v)
{
    if constexpr (LO < HI) {
        v = fmaxf(v, xor_shuffle<LO>(v));
        return xor_max<2 * LO, HI>(v);
    } else {
        return v;
    }
}

// decodeKeys of one group, rounded to bf16
template <int KB, bool KS>
__device__ __forceinline__ void key_group(const AttnParams &p, int64_t grow, float (&kx)[kGroup])
{
    uint32_t w[KB];
    load_codes<KB>(p.kc + grow * (4 * KB), w);
    const float scale = f16_bits_to_f32(p.ks[grow]);
    const float zero = f16_bits_to_f32(p.kz[grow]);
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
        const uint32_t q = unpack1<KB>(w, u);
        const float qf = KS ? (float)(int32_t)(int8_t)(uint8_t)q : (float)q;
        const float sum = qf + zero;
        kx[u] = bf16_round(sum * scale);
    }
}

__device__ __forceinline__ void key_group_any(const AttnParams &p, int64_t grow, float (&kx)[kGroup])
{
    switch (p.kmode) { // wavefront-uniform
    case 2: key_group<2, false>(p, grow, kx); break;
    case 3: key_group<3, false>(p, grow, kx); break;
    case 4: key_group<4, false>(p, grow, kx); break;
    case 5: key_group<5, false>(p, grow, kx); break;
    case 8: key_group<8, false>(p, grow, kx); break;
    default: key_group<8, true>(p, grow, kx); break;
    }
}

// LDS of a partial block: the query heads (shared), and per wavefront the
// rotated values and softmax weights of its current tile
// (rows of vt are padded by 16 bytes and the query's 32-element groups by
// 4 floats, which spreads the 16-byte accesses of a wavefront over the LDS
// banks)
template <int D, int GQ> struct AttnShared {
    static constexpr int G = D / kGroup;
    static constexpr int RPW = kWave / G; // tokens per wavefront tile
    static constexpr int VROW = D + 8;    // bf16 elements per padded vt row
    static constexpr int QG = kGroup + 4; // floats per padded query group
    __align__(16) float qs[GQ][G][QG];
    __align__(16) uint16_t vt[kWavesPerBlock][RPW][VROW]; // bf16 bits (the values are bf16)
    __align__(16) float pw[kWavesPerBlock][RPW][GQ];
    float ml[kWavesPerBlock][2];
    // the end-of-block merge reuses vt as [4][D] floats
    static_assert(sizeof(uint16_t) * kWavesPerBlock * RPW * D >= sizeof(float) * kWavesPerBlock * D, "merge area");
};

// Each wavefront of a block is an independent range of wave_tokens tokens
// of one (sequence, KV head): tiles of RPW = 64 / G tokens, lane (t, grp)
// decoding group grp of token t as the codec's decoder does; scores from
// the lane's 32 key values against each query head (query from LDS),
// summed over the token's G lanes; online softmax over the wavefront's
// tokens; the tile's rotated values and weights go through the
// wavefront's LDS area, where lane l accumulates dims l, l + 64, ... of
// every query head. Only wavefront-level synchronisation per tile.
template <int D, int VB, int GQ>
__device__ __forceinline__ void attn_wave(const AttnParams &p, int b, int c, int j, const float *cent,
                                          AttnShared<D, GQ> &sh)
{
    constexpr int G = D / kGroup;
    constexpr int RPW = AttnShared<D, GQ>::RPW;
    constexpr int VROW = AttnShared<D, GQ>::VROW;
    constexpr int DPL = D / kWave; // output dims per lane
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int grp = lane % G, rl = lane / G;
    const int hq = p.hkv * GQ;
    const int64_t pad = p.left_pad != nullptr ? p.left_pad[b] : 0;
    const int64_t w0 = ((int64_t)c * kWavesPerBlock + wave) * p.wave_tokens;
    const int64_t t_lo = w0 > pad ? w0 : pad;
    const int64_t t_end = w0 + p.wave_tokens < p.width ? w0 + p.wave_tokens : p.width;
    uint16_t (&vt)[RPW][VROW] = sh.vt[wave];
    float (&pw)[RPW][GQ] = sh.pw[wave];

    float acc[DPL][GQ];
    float m_run[GQ], l_run[GQ];
#pragma unroll
    for (int m = 0; m < DPL; ++m)
#pragma unroll
        for (int e = 0; e < GQ; ++e) acc[m][e] = 0.0f;
#pragma unroll
    for (int e = 0; e < GQ; ++e) {
        m_run[e] = -INFINITY;
        l_run[e] = 0.0f;
    }

    for (int64_t t0 = t_lo; t0 < t_end; t0 += RPW) {
        const int64_t t = t0 + rl;
        const bool valid = t < t_end;
        const int64_t row = ((int64_t)b * p.width + (valid ? t : t_lo)) * p.hkv + j;
        const int64_t grow = row * G + grp;
        float kx[kGroup];
        key_group_any(p, grow, kx);
        // values: decodeValuesRotated (centroid * scale, bf16)
        {
            uint32_t w[VB];
            load_codes<VB>(p.vc + grow * (4 * VB), w);
            const float s = f16_bits_to_f32(p.vs[grow]);
#pragma unroll
            for (int u = 0; u < kGroup; u += 8) {
                uint4 w4;
                uint32_t *wp = &w4.x;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float a = cent[unpack1<VB>(w, u + 2 * k)] * s;
                    const float b2 = cent[unpack1<VB>(w, u + 2 * k + 1)] * s;
                    wp[k] = valid ? pack_bf16x2(a, b2) : 0u;
                }
                *reinterpret_cast<uint4 *>(&vt[rl][grp * kGroup + u]) = w4;
            }
        }
        // scores, tile maximum and weights per query head
        float alpha[GQ];
#pragma unroll
        for (int e = 0; e < GQ; ++e) {
            float a = 0.0f;
            const float4 *q4 = reinterpret_cast<const float4 *>(&sh.qs[e][grp][0]);
#pragma unroll
            for (int u = 0; u < kGroup / 4; ++u) {
                const float4 qv = q4[u];
                a = fmaf(kx[4 * u], qv.x, a);
                a = fmaf(kx[4 * u + 1], qv.y, a);
                a = fmaf(kx[4 * u + 2], qv.z, a);
                a = fmaf(kx[4 * u + 3], qv.w, a);
            }
            a = xor_sum<1, G>(a);
            const float sc = valid ? a * p.scale : -INFINITY;
            const float mx = xor_max<G, kWave>(sc);
            const float m_new = fmaxf(m_run[e], mx);
            alpha[e] = m_new == -INFINITY ? 1.0f : expf(m_run[e] - m_new);
            const float pe = (m_new == -INFINITY || !valid) ? 0.0f : expf(sc - m_new);
            const float ps = xor_sum<G, kWave>(pe);
            l_run[e] = l_run[e] * alpha[e] + ps;
            m_run[e] = m_new;
            if (grp == 0) pw[rl][e] = pe;
        }
        wave_lds_sync();
        // weighted values of the tile
#pragma unroll
        for (int m = 0; m < DPL; ++m)
#pragma unroll
            for (int e = 0; e < GQ; ++e) acc[m][e] *= alpha[e];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            float pr[GQ];
#pragma unroll
            for (int e = 0; e < GQ; ++e) pr[e] = pw[r][e];
#pragma unroll
            for (int m = 0; m < DPL; ++m) {
                const float v = as_f((uint32_t)vt[r][lane + kWave * m] << 16);
#pragma unroll
                for (int e = 0; e < GQ; ++e) acc[m][e] = fmaf(pr[e], v, acc[m][e]);
            }
        }
        wave_lds_sync();
    }

    // merge the block's four wavefront splits, one query head at a time,
    // through the (now free) value area, and write the block's partial
    float *scratch = reinterpret_cast<float *>(&sh.vt[0][0][0]); // [4][D] floats
#pragma unroll
    for (int e = 0; e < GQ; ++e) {
        __syncthreads();
#pragma unroll
        for (int m = 0; m < DPL; ++m) scratch[wave * D + lane + kWave * m] = acc[m][e];
        if (lane == 0) {
            sh.ml[wave][0] = m_run[e];
            sh.ml[wave][1] = l_run[e];
        }
        __syncthreads();
        float M = sh.ml[0][0];
#pragma unroll
        for (int v = 1; v < kWavesPerBlock; ++v) M = fmaxf(M, sh.ml[v][0]);
        float f[kWavesPerBlock], L = 0.0f;
#pragma unroll
        for (int v = 0; v < kWavesPerBlock; ++v) {
            f[v] = sh.ml[v][0] == -INFINITY ? 0.0f : expf(sh.ml[v][0] - M);
            L = fmaf(sh.ml[v][1], f[v], L);
        }
        float *r = part_row<D>(p, b, j * GQ + e, c);
        for (int i = threadIdx.x; i < D; i += kBlockThreads) {
            float a = 0.0f;
#pragma unroll
            for (int v = 0; v < kWavesPerBlock; ++v) a = fmaf(scratch[v * D + i], f[v], a);
            r[i] = a;
        }
        if (threadIdx.x == 0) {
            r[D] = M;
            r[D + 1] = L;
        }
    }
    (void)hq;
}

// Blocks are ordered so that the KV heads of one (sequence, chunk) are
// dispatched to the same XCD one after another (dispatch deals block ids
// to the 8 XCDs in turn): block id -> XCD x = id % 8, slot r = id / 8,
// head j = r % hkv, chunk group (r / hkv) * 8 + x. The heads' rows of a
// token are adjacent in the planes, so they share cache lines.
template <int D, int VB, int GQ>
__global__ void __launch_bounds__(kBlockThreads) attn_partial_kernel(AttnParams p)
{
    __shared__ float cent[1 << VB];
    __shared__ AttnShared<D, GQ> sh;
    const int id = blockIdx.x;
    const int x = id % 8, r = id / 8;
    const int j = r % p.hkv;
    const int nchunks = p.nsplit;
    const int cg = (r / p.hkv) * 8 + x;
    if (cg >= p.batch * nchunks) return;
    const int b = cg / nchunks, c = cg % nchunks;
    const int hq = p.hkv * GQ;
    for (int i = threadIdx.x; i < (1 << VB); i += kBlockThreads) cent[i] = dev_cent<VB>()[i];
    for (int e = 0; e < GQ; ++e)
        for (int i = threadIdx.x; i < D; i += kBlockThreads) {
            const int64_t qi = ((int64_t)b * hq + j * GQ + e) * D + i;
            sh.qs[e][i / kGroup][i % kGroup] = p.q_bf16 ? as_f((uint32_t)reinterpret_cast<const uint16_t *>(p.q)[qi] << 16)
                                                        : reinterpret_cast<const float *>(p.q)[qi];
        }
    __syncthreads();
    attn_wave<D, VB, GQ>(p, b, c, j, cent, sh);
}

// Merge of the splits of one output row (sequence, query head), one block
// per (row, 64 dims): the largest split maximum M, the normaliser L = sum
// l_s exp(m_s - M), and o_rot = sum o_s exp(m_s - M) / L for its dims
// (thread (4 dims, k) sums splits k, k + 16, ...), written to `orot`.
__global__ void __launch_bounds__(kBlockThreads) attn_merge_kernel(const float *part, int32_t nsplit, int32_t d,
                                                                   float *orot)
{
    __shared__ float red[kBlockThreads];
    __shared__ float4 acc4[16][16];
    const int row = blockIdx.x, sl = blockIdx.y, tid = threadIdx.x;
    const int64_t stride = d + 4;
    const float *base = part + (int64_t)row * nsplit * stride;
    float m = -INFINITY;
    for (int s = tid; s < nsplit; s += kBlockThreads) m = fmaxf(m, base[s * stride + d]);
    red[tid] = m;
    __syncthreads();
    for (int h = kBlockThreads / 2; h > 0; h >>= 1) {
        if (tid < h) red[tid] = fmaxf(red[tid], red[tid + h]);
        __syncthreads();
    }
    const float M = red[0];
    __syncthreads();
    float l = 0.0f;
    if (M != -INFINITY)
        for (int s = tid; s < nsplit; s += kBlockThreads) {
            const float ms = base[s * stride + d];
            if (ms != -INFINITY) l = fmaf(base[s * stride + d + 1], expf(ms - M), l);
        }
    red[tid] = l;
    __syncthreads();
    for (int h = kBlockThreads / 2; h > 0; h >>= 1) {
        if (tid < h) red[tid] += red[tid + h];
        __syncthreads();
    }
    const float L = red[0];
    const int q4 = tid % 16, k = tid / 16; // dims 64 sl + 4 q4 .. + 3
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (M != -INFINITY)
        for (int s = k; s < nsplit; s += 16) {
            const float *ps = base + s * stride;
            const float ms = ps[d];
            if (ms == -INFINITY) continue;
            const float f = expf(ms - M);
            const float4 v = *reinterpret_cast<const float4 *>(ps + 64 * sl + 4 * q4);
            a.x = fmaf(v.x, f, a.x);
            a.y = fmaf(v.y, f, a.y);
            a.z = fmaf(v.z, f, a.z);
            a.w = fmaf(v.w, f, a.w);
        }
    acc4[k][q4] = a;
    __syncthreads();
    if (tid < 16) {
        float4 t = acc4[0][tid];
        for (int kk = 1; kk < 16; ++kk) {
            const float4 u = acc4[kk][tid];
            t.x += u.x;
            t.y += u.y;
            t.z += u.z;
            t.w += u.w;
        }
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        t.x *= inv;
        t.y *= inv;
        t.z *= inv;
        t.w *= inv;
        *reinterpret_cast<float4 *>(orot + (int64_t)row * d + 64 * sl + 4 * tid) = t;
    }
}

__global__ void __launch_bounds__(kBlockThreads) attn_zero_kernel(uint32_t *out, int64_t words)
{
    const int64_t i = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
    if (i < words) out[i] = 0u;
}

// The inverse rotation of merged rows (transform, then sign vector), G
// lanes per row, written as out_dtype.
template <int D>
__global__ void __launch_bounds__(kBlockThreads) attn_rotate_kernel(const float *orot, int32_t rows, void *out,
                                                                    int32_t out_bf16)
{
    constexpr int G = D / kGroup;
    const int grp = threadIdx.x % G;
    const int row = (int)blockIdx.x * (kBlockThreads / G) + (int)threadIdx.x / G;
    const int rr = row < rows ? row : rows - 1;
    float y[kGroup];
    const float4 *src = reinterpret_cast<const float4 *>(orot + (int64_t)rr * D + grp * kGroup);
#pragma unroll
    for (int u = 0; u < kGroup / 4; ++u) {
        const float4 v = src[u];
        y[4 * u] = v.x;
        y[4 * u + 1] = v.y;
        y[4 * u + 2] = v.z;
        y[4 * u + 3] = v.w;
    }
    const Rot<D> rot(grp);
    hadamard<D>(y, rot);
    const uint32_t smask = dev_sign<D>(grp);
    if (row >= rows) return;
    if (out_bf16) {
        uint32_t *o = reinterpret_cast<uint32_t *>(out) + ((int64_t)row * D + grp * kGroup) / 2;
#pragma unroll
        for (int k = 0; k < kGroup / 2; ++k) o[k] = pack_bf16x2(y[2 * k], y[2 * k + 1]) ^ sign_pair_mask(smask, k);
    } else {
        float *o = reinterpret_cast<float *>(out) + (int64_t)row * D + grp * kGroup;
#pragma unroll
        for (int u = 0; u < kGroup; ++u) o[u] = ((smask >> u) & 1u) ? -y[u] : y[u];
    }
}

template <int D, int VB> const void *partial_kernel_g(int gq)
{
    switch (gq) {
    case 1: return reinterpret_cast<const void *>(&attn_partial_kernel<D, VB, 1>);
    case 2: return reinterpret_cast<const void *>(&attn_partial_kernel<D, VB, 2>);
    case 4: return reinterpret_cast<const void *>(&attn_partial_kernel<D, VB, 4>);
    default: return reinterpret_cast<const void *>(&attn_partial_kernel<D, VB, 8>);
    }
}

template <int D> const void *partial_kernel_for(int vb, int gq)
{
    switch (vb) {
    case 2: return partial_kernel_g<D, 2>(gq);
    case 3: return partial_kernel_g<D, 3>(gq);
    case 4: return partial_kernel_g<D, 4>(gq);
    case 5: return partial_kernel_g<D, 5>(gq);
    default: return partial_kernel_g<D, 8>(gq);
    }
}

// Splits (blocks) per (sequence, KV head): about kAttnTargetBlocks blocks in
// all, each wavefront taking at least kAttnMinWaveTokens tokens.
int64_t n_splits(int32_t batch, int32_t kv_heads, int64_t width)
{
    if (width <= 0 || batch <= 0 || kv_heads <= 0) return 0;
    int64_t n = (kAttnTargetBlocks + (int64_t)batch * kv_heads - 1) / ((int64_t)batch * kv_heads);
    const int64_t most = (width + kWavesPerBlock * kAttnMinWaveTokens - 1) / (kWavesPerBlock * kAttnMinWaveTokens);
    if (n > most) n = most;
    return n < 1 ? 1 : n;
}

int64_t wave_tokens(int64_t width, int64_t nsplit)
{
    return nsplit > 0 ? (width + nsplit * kWavesPerBlock - 1) / (nsplit * kWavesPerBlock) : 0;
}

} // namespace

extern "C" {

int64_t tq_attention_workspace_bytes(int32_t batch, int32_t kv_heads, int32_t q_heads, int32_t head_dim,
                                     int64_t width)
{
    if (batch < 0 || kv_heads < 1 || q_heads < 0 || width < 0 || !tq_host::valid_head_dim(head_dim))
        return -TQ_E_SHAPE;
    if (width == 0) return 0;
    // split partials, then the merged rows
    return (int64_t)batch * q_heads * (n_splits(batch, kv_heads, width) * (head_dim + 4) + head_dim) *
           (int64_t)sizeof(float);
}

int32_t tq_attention_decode(const void *q, int32_t q_dtype, const tq_packed_kv *cache, int32_t batch, int64_t width,
                            const int32_t *left_pad, int32_t kv_heads, int32_t q_heads, const tq_config *cfg,
                            float scale, void *out, int32_t out_dtype, void *workspace, int64_t workspace_bytes,
                            void *stream)
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

    if (batch == 0) return TQ_OK;
    const int32_t d = cfg->head_dim;
    if (q == nullptr || out == nullptr) return TQ_E_NULL;
    if (!tq_host::aligned(q, 16) || !tq_host::aligned(out, 16)) return TQ_E_ALIGN;
    const int64_t nch = n_splits(batch, kv_heads, width);
    if (width > 0) {
        if (workspace == nullptr) return TQ_E_NULL;
        if (workspace_bytes < tq_attention_workspace_bytes(batch, kv_heads, q_heads, d, width)) return TQ_E_SHAPE;
        if (!tq_host::aligned(workspace, 16)) return TQ_E_ALIGN;
        if (cache->k_codes == nullptr || cache->k_scale == nullptr || cache->k_zero == nullptr ||
            cache->v_codes == nullptr || cache->v_scale == nullptr)
            return TQ_E_NULL;
        if (!tq_host::aligned(cache->k_codes, tq_host::code_align(cfg->k_bits)) ||
            !tq_host::aligned(cache->v_codes, tq_host::code_align(cfg->v_bits)) ||
            !tq_host::aligned(cache->k_scale, 2) || !tq_host::aligned(cache->k_zero, 2) ||
            !tq_host::aligned(cache->v_scale, 2))
            return TQ_E_ALIGN;
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
        if (wave_tokens(width, nch) > 0x7fffffff) return TQ_E_SHAPE;
        p.nsplit = (int32_t)nch;
        p.wave_tokens = (int32_t)wave_tokens(width, nch);
        p.q_bf16 = q_dtype == TQ_BF16;
        p.kmode = cfg->k_signed ? (8 | 16) : cfg->k_bits;
        p.scale = scale;
        const int gq = p.g;
        const void *fn = d == 64 ? partial_kernel_for<64>(cfg->v_bits, gq)
                       : d == 128 ? partial_kernel_for<128>(cfg->v_bits, gq)
                       : d == 256 ? partial_kernel_for<256>(cfg->v_bits, gq)
                                  : partial_kernel_for<512>(cfg->v_bits, gq);
        const int64_t groups = ((int64_t)batch * nch + 7) / 8;
        const int64_t blocks = groups * 8 * kv_heads;
        if (blocks > 0x7fffffff) return TQ_E_SHAPE;
        void *args[] = {&p};
        if (hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(kBlockThreads), args, 0, (hipStream_t)stream) !=
            hipSuccess)
            return TQ_E_HIP;
    }
    // merge (rows with no split are zeros), then the inverse rotation
    const int32_t rows = batch * q_heads;
    float *part = static_cast<float *>(workspace);
    float *orot = part + (int64_t)rows * nch * (d + 4);
    if (width == 0) {
        // no workspace needed: every row is zero (a fill kernel, not a
        // memset, so that the call can be captured in a graph)
        uint32_t *o32 = static_cast<uint32_t *>(out);
        int64_t words = (int64_t)rows * d * (out_dtype == TQ_BF16 ? 2 : 4) / 4;
        void *argsz[] = {&o32, &words};
        if (hipLaunchKernel(reinterpret_cast<const void *>(&attn_zero_kernel),
                            dim3((uint32_t)((words + kBlockThreads - 1) / kBlockThreads)), dim3(kBlockThreads), argsz,
                            0, (hipStream_t)stream) != hipSuccess)
            return TQ_E_HIP;
        return hipGetLastError() == hipSuccess ? TQ_OK : TQ_E_HIP;
    }
    int32_t nsp = (int32_t)nch;
    const float *cpart = part;
    int32_t dd = d;
    void *args2[] = {&cpart, &nsp, &dd, &orot};
    if (hipLaunchKernel(reinterpret_cast<const void *>(&attn_merge_kernel), dim3((uint32_t)rows, (uint32_t)(d / 64)),
                        dim3(kBlockThreads), args2, 0, (hipStream_t)stream) != hipSuccess)
        return TQ_E_HIP;
    const float *corot = orot;
    int32_t rows32 = rows;
    int32_t obf = out_dtype == TQ_BF16;
    void *args3[] = {&corot, &rows32, &out, &obf};
    const int32_t rpb = kBlockThreads / (d / kGroup);
    const void *fn3 = d == 64 ? reinterpret_cast<const void *>(&attn_rotate_kernel<64>)
                    : d == 128 ? reinterpret_cast<const void *>(&attn_rotate_kernel<128>)
                    : d == 256 ? reinterpret_cast<const void *>(&attn_rotate_kernel<256>)
                    : reinterpret_cast<const void *>(&attn_rotate_kernel<512>);
    if (hipLaunchKernel(fn3, dim3((uint32_t)((rows + rpb - 1) / rpb)), dim3(kBlockThreads), args3, 0,
                        (hipStream_t)stream) != hipSuccess)
        return TQ_E_HIP;
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_E_HIP;
}

} // extern "C"
