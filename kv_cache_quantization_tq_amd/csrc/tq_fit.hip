// tq_fit.hip -- Lloyd-Max fitting of value tables on the GPU.
//
// The page "mlx-bun 0.0.9 -> 0.0.11", src/mlx/turboquant-tables.ts (the
// header of LLOYD_MAX) states how the tables for widths other than 3 bits
// were made: an iterative Lloyd-Max fit to samples of a unit normal source,
// 500 iterations. One Lloyd iteration on a sample set:
//   boundaries  b_j = (c_j + c_{j+1}) / 2                  (j < L - 1)
//   assignment  k(x) = #{ j : b_j < x }   (the codec's bin rule: ties go to
//                                          the lower level)
//   centroids   c_k = mean of the samples with k(x) = k    (a level with no
//                                          sample keeps its centroid)
// This file runs the iterations on the device with no host round trip (per
// iteration an assignment launch writing per-block partial sums and an
// update launch with one block per level).
//
// Determinism: each sample enters the per-level sums as the exact integer
// rint(x * 2^s), with s chosen from the sample count and the largest
// magnitude so that no sum can overflow 63 bits; integer addition does not
// depend on order, so the result is the same for any grid and equals a
// sequential evaluation of the same rule (the centroid is then
// double(sum) * 2^-s / count in binary64).
#include <hip/hip_runtime.h>

#include <math.h>
#include <string.h>

#include "tq.h"

namespace {

constexpr int kMaxLevels = 256;
constexpr int kFitThreads = 256;
constexpr int kFitBlocks = 1024; // most blocks of a pass (per-block partials below)

// Device workspace (caller-owned). Each pass writes one partial result per
// block (no contended atomics: a handful of addresses hit by every block
// of every XCD would serialise), reduced by the next step.
struct FitWork {
    double cent[kMaxLevels];
    unsigned long long part_sum[kMaxLevels][kFitBlocks]; // two's complement int64, level-major
    unsigned int part_cnt[kMaxLevels][kFitBlocks];
    unsigned int part_max[kFitBlocks];                   // largest |x| bits per block
    int shift;                                           // s, or -1 when the samples cannot be fitted
    int emax;                                            // |x| < 2^emax for every sample
};

// largest |x| of a block's samples as the bit pattern of a non-negative
// float (its integer order is the float order; NaN patterns order above
// +inf)
__global__ void __launch_bounds__(kFitThreads) fit_absmax_kernel(const float *x, int64_t n, FitWork *w)
{
    unsigned int m = 0;
    const int64_t tid = (int64_t)blockIdx.x * kFitThreads + threadIdx.x, nt = (int64_t)gridDim.x * kFitThreads;
    if ((reinterpret_cast<uintptr_t>(x) & 15) == 0) {
        // whole 16-byte vectors, then the last n % 4 samples
        const float4 *x4 = reinterpret_cast<const float4 *>(x);
        for (int64_t v = tid; v < n / 4; v += nt) {
            const float4 a = x4[v];
            m = max(max(m, __float_as_uint(a.x) & 0x7fffffffu), __float_as_uint(a.y) & 0x7fffffffu);
            m = max(max(m, __float_as_uint(a.z) & 0x7fffffffu), __float_as_uint(a.w) & 0x7fffffffu);
        }
        if (tid < n % 4) m = max(m, __float_as_uint(x[n / 4 * 4 + tid]) & 0x7fffffffu);
    } else {
        for (int64_t i = tid; i < n; i += nt) m = max(m, __float_as_uint(x[i]) & 0x7fffffffu);
    }
    for (int o = 32; o > 0; o >>= 1) m = max(m, (unsigned int)__shfl_xor((int)m, o));
    __shared__ unsigned int wm[kFitThreads / 64];
    if ((threadIdx.x & 63) == 0) wm[threadIdx.x / 64] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < kFitThreads / 64; ++i) m = max(m, wm[i]);
        w->part_max[blockIdx.x] = m;
    }
}

// s = min(40, 62 - bitlen(n) - e) with |x| < 2^e for every sample: every
// |rint(x * 2^s)| <= 2^(62 - bitlen(n)) and n of them sum below 2^62
__device__ int fit_shift(unsigned int absmax_bits, int64_t n)
{
    if (absmax_bits >= 0x7f800000u) return -1; // inf or NaN
    int e = 0;
    if (absmax_bits != 0) frexpf(__uint_as_float(absmax_bits), &e); // |x| < 2^e
    int bl = 0;
    for (uint64_t v = (uint64_t)n; v != 0; v >>= 1) ++bl;
    int s = 62 - bl - e;
    return s > 40 ? 40 : s;
}

// one block: the largest magnitude over the absmax blocks, then the shift
__global__ void __launch_bounds__(kFitThreads) fit_init_kernel(FitWork *w, int blocks, int64_t n)
{
    __shared__ unsigned int red[kFitThreads];
    unsigned int m = 0;
    for (int b = threadIdx.x; b < blocks; b += kFitThreads) m = max(m, w->part_max[b]);
    red[threadIdx.x] = m;
    __syncthreads();
    for (int h = kFitThreads / 2; h > 0; h >>= 1) {
        if (threadIdx.x < h) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + h]);
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        w->shift = fit_shift(red[0], n);
        int e = 0;
        if (red[0] != 0 && red[0] < 0x7f800000u) frexpf(__uint_as_float(red[0]), &e);
        w->emax = e;
    }
}

// Assignment and per-level integer sums of one pass. The block computes the
// boundaries from the current centroids, keeps R replicas of the L-level
// histogram in LDS (R = the largest power of two <= 64 with R * L <=
// kHistEntries), lane l of every wavefront adding into replica l % R so
// that lanes of one wavefront rarely contend for an address, folds the
// replicas pairwise and writes the block's totals as its partial. The
// search compares the float32 sample with each boundary rounded down to
// float32, which decides b < x exactly (no float32 lies strictly between a
// binary64 value and its round-down).
constexpr int kHistEntries = 1024;

__host__ __device__ inline int fit_replicas(int levels)
{
    int r = 64;
    while (r > 1 && r * levels > kHistEntries) r >>= 1;
    return r;
}

// Number of boundaries below v (levels <= 2^NS; bnd padded with +inf):
// a binary search of NS steps, step t comparing with boundary k + 2^(NS-1-t)
// - 1. The first RS steps select their boundary from registers (rb holds
// the 2^RS - 1 boundaries they can need, rb[2^t - 1 + j] for step t and
// j = k >> (NS - t)); later steps read LDS.
template <int NS, int RS>
__device__ __forceinline__ int search_bins(float v, const float *bnd, const float (&rb)[(1 << RS) - 1])
{
    int k = 0;
#pragma unroll
    for (int t = 0; t < NS; ++t) {
        const int st = 1 << (NS - 1 - t);
        float bb;
        if (t < RS) {
            const int j = k >> (NS - t);
            bb = rb[(1 << t) - 1];
#pragma unroll
            for (int c = 1; c < (1 << t); ++c) bb = j == c ? rb[(1 << t) - 1 + c] : bb;
        } else {
            bb = bnd[k + st - 1];
        }
        k += bb < v ? st : 0;
    }
    return k;
}

// rint(x * 2^s) as an int64. With MAGIC (every |x * 2^s| < 2^51, which the
// shift rule guarantees for n >= 2^11): x * 2^s + 1.5 * 2^52 in binary64 is
// rounded to an integer, half to even, in one fma (the product is exact),
// and the integer is the difference of the bit patterns.
template <bool MAGIC> __device__ __forceinline__ long long fixed_point(float x, int s)
{
    if constexpr (MAGIC) {
        constexpr double kMagic = 6755399441055744.0; // 1.5 * 2^52
        const double t = __builtin_fma((double)x, ldexp(1.0, s), kMagic);
        return (long long)(__builtin_bit_cast(unsigned long long, t) - __builtin_bit_cast(unsigned long long, kMagic));
    } else {
        return (long long)rint(ldexp((double)x, s));
    }
}

// Bin lookup on a uniform grid (the codec's value-bin method, with a table
// built by each block from the current boundaries). Cells have width
// W = 2^(emax - 6) and cover (-2^emax, 2^emax), where every sample lies:
// cell c = round(x / W + 64) is the low bits of one fma with 2^23 added
// (x / W is exact, W a power of two). Each cell stores the number of
// boundaries below its lower edge widened by 1/1024 of a cell and the one
// boundary inside the widened cell (+inf if none), so base + (x > bnd) is
// exactly #{j : b_j < x}. If some widened cell holds two boundaries the
// block uses the binary search instead (every block reaches the same
// decision: it depends only on the boundaries and emax).
constexpr int kGridCells = 130;   // c = 0 .. 128, one per thread

struct FitCell {
    float bnd;
    unsigned int base;
};

// number of entries of the ascending array a[0..kMaxLevels) below v (<=
// v when INCL)
template <bool INCL> __device__ __forceinline__ int count_below(const float *a, double v)
{
    int lo = 0;
#pragma unroll
    for (int st = kMaxLevels / 2; st > 0; st >>= 1)
        if (INCL ? (double)a[lo + st - 1] <= v : (double)a[lo + st - 1] < v) lo += st;
    return lo;
}

// Fills lut (one cell per thread) and returns, to every thread, whether
// every widened cell holds at most one boundary.
__device__ bool build_grid(const float *bnd, int emax, FitCell *lut)
{
    bool bad = emax > 100 || emax < -100;  // keep 2^-(emax-6) and the cell edges in range
    const int c = threadIdx.x;
    if (!bad && c < kGridCells) {
        const double W = ldexp(1.0, emax - 6), LO = -ldexp(1.0, emax);
        constexpr double margin = 1.0 / 1024.0;
        const double lo = LO + ((double)c - 0.5 - margin) * W, hi = LO + ((double)c + 0.5 + margin) * W;
        const int below = count_below<false>(bnd, lo), upto = count_below<true>(bnd, hi);
        bad = upto - below > 1;
        lut[c].base = (unsigned int)below;
        lut[c].bnd = upto > below ? bnd[below] : INFINITY;
    }
    return __syncthreads_or(bad) == 0;
}

__device__ __forceinline__ int grid_bin(float v, float a, float cmag, const FitCell *lut)
{
    const float t = __builtin_fmaf(v, a, cmag);
    const FitCell e = lut[__builtin_bit_cast(unsigned int, t) - 0x4B000000u];
    return (int)e.base + (v > e.bnd ? 1 : 0);
}

template <int NS, bool MAGIC>
__global__ void __launch_bounds__(kFitThreads) fit_assign_kernel(const float *x, int64_t n, int levels, FitWork *w)
{
    constexpr int RS = NS < 2 ? NS : 2;
    __shared__ float bnd[kMaxLevels];
    __shared__ unsigned long long hsum[kHistEntries];
    __shared__ unsigned int hcnt[kHistEntries];
    const int s = w->shift;
    if (s < 0) return;
    const int R = fit_replicas(levels);
    for (int j = threadIdx.x; j < kMaxLevels; j += kFitThreads)
        bnd[j] = j < levels - 1 ? __double2float_rd((w->cent[j] + w->cent[j + 1]) * 0.5) : INFINITY;
    for (int j = threadIdx.x; j < levels * R; j += kFitThreads) {
        hsum[j] = 0;
        hcnt[j] = 0;
    }
    __syncthreads();
    __shared__ FitCell lut[kGridCells];
    const int emax = w->emax;
    const bool grid = build_grid(bnd, emax, lut);
    const float ga = ldexpf(1.0f, 6 - emax), gc = 64.0f + 8388608.0f;
    float rb[(1 << RS) - 1];
#pragma unroll
    for (int t = 0; t < RS; ++t)
#pragma unroll
        for (int j = 0; j < (1 << t); ++j) rb[(1 << t) - 1 + j] = bnd[(2 * j + 1) * (1 << (NS - 1 - t)) - 1];
    const int rep = (threadIdx.x & 63) % R;
    // four samples at a time (one 16-byte vector per thread and step when
    // the samples are 16-byte aligned), so that their searches overlap
    auto add4 = [&](const float (&v)[4], int valid) {
        int k[4];
        if (grid) {
#pragma unroll
            for (int u = 0; u < 4; ++u) k[u] = grid_bin(v[u], ga, gc, lut);
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) k[u] = search_bins<NS, RS>(v[u], bnd, rb);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (u < valid) {
                const long long q = fixed_point<MAGIC>(v[u], s);
                atomicAdd(&hsum[k[u] * R + rep], (unsigned long long)q);
                atomicAdd(&hcnt[k[u] * R + rep], 1u);
            }
        }
    };
    const int64_t tid = (int64_t)blockIdx.x * kFitThreads + threadIdx.x, nt = (int64_t)gridDim.x * kFitThreads;
    if ((reinterpret_cast<uintptr_t>(x) & 15) == 0) {
        const float4 *x4 = reinterpret_cast<const float4 *>(x);
        for (int64_t vi = tid; vi < n / 4; vi += nt) {
            const float4 a = x4[vi];
            const float v[4] = {a.x, a.y, a.z, a.w};
            add4(v, 4);
        }
        if (tid == 0 && n % 4 != 0) {
            float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int u = 0; u < (int)(n % 4); ++u) v[u] = x[n / 4 * 4 + u];
            add4(v, (int)(n % 4));
        }
    } else {
        for (int64_t i0 = tid; i0 < n; i0 += 4 * nt) {
            float v[4];
            int valid = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t i = i0 + u * nt;
                v[u] = i < n ? x[i] : 0.0f;
                valid += i < n ? 1 : 0;
            }
            add4(v, valid);
        }
    }
    __syncthreads();
    for (int half = R / 2; half > 0; half >>= 1) {
        for (int j = threadIdx.x; j < levels * half; j += kFitThreads) {
            const int kk = j / half, r = j % half;
            hsum[kk * R + r] += hsum[kk * R + r + half];
            hcnt[kk * R + r] += hcnt[kk * R + r + half];
        }
        __syncthreads();
    }
    for (int kk = threadIdx.x; kk < levels; kk += kFitThreads) {
        w->part_sum[kk][blockIdx.x] = hsum[kk * R];
        w->part_cnt[kk][blockIdx.x] = hcnt[kk * R];
    }
}

// one block per level: the level's total over the pass's block partials
// (contiguous, level-major; each thread loads its few independently), then
// its new centroid (a level with no sample keeps its value)
__global__ void __launch_bounds__(kFitThreads) fit_update_kernel(FitWork *w, int blocks)
{
    __shared__ unsigned long long rs[kFitThreads / 64][2];
    const int s = w->shift;
    if (s < 0) return;
    const int k = blockIdx.x, tid = threadIdx.x;
    unsigned long long sm = 0, c = 0;
#pragma unroll
    for (int i = 0; i < kFitBlocks / kFitThreads; ++i) {
        const int b = tid + i * kFitThreads;
        if (b < blocks) {
            sm += w->part_sum[k][b];
            c += w->part_cnt[k][b];
        }
    }
    for (int o = 32; o > 0; o >>= 1) {
        sm += __shfl_xor(sm, o);
        c += __shfl_xor(c, o);
    }
    if ((tid & 63) == 0) {
        rs[tid / 64][0] = sm;
        rs[tid / 64][1] = c;
    }
    __syncthreads();
    if (tid == 0) {
        for (int v = 1; v < kFitThreads / 64; ++v) {
            sm += rs[v][0];
            c += rs[v][1];
        }
        if (c != 0) w->cent[k] = ldexp((double)(long long)sm, -s) / (double)c;
    }
}

template <bool MAGIC> const void *assign_kernel(int ns)
{
    switch (ns) {
    case 1: return reinterpret_cast<const void *>(&fit_assign_kernel<1, MAGIC>);
    case 2: return reinterpret_cast<const void *>(&fit_assign_kernel<2, MAGIC>);
    case 3: return reinterpret_cast<const void *>(&fit_assign_kernel<3, MAGIC>);
    case 4: return reinterpret_cast<const void *>(&fit_assign_kernel<4, MAGIC>);
    case 5: return reinterpret_cast<const void *>(&fit_assign_kernel<5, MAGIC>);
    case 6: return reinterpret_cast<const void *>(&fit_assign_kernel<6, MAGIC>);
    case 7: return reinterpret_cast<const void *>(&fit_assign_kernel<7, MAGIC>);
    default: return reinterpret_cast<const void *>(&fit_assign_kernel<8, MAGIC>);
    }
}

int32_t hip_ok(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_E_HIP; }

} // namespace

extern "C" {

int64_t tq_lloyd_max_workspace_bytes(void) { return (int64_t)sizeof(FitWork); }

int32_t tq_lloyd_max_fit(const float *samples, int64_t n, int32_t levels, const double *init, int32_t iterations,
                         double *centroids, double *boundaries, void *workspace, int64_t workspace_bytes,
                         void *stream)
{
    if (levels < 2 || levels > kMaxLevels) return TQ_E_BITS;
    if (n < 1 || n > ((int64_t)1 << 40) || iterations < 0) return TQ_E_SHAPE;
    if (samples == nullptr || init == nullptr || centroids == nullptr || workspace == nullptr) return TQ_E_NULL;
    if (workspace_bytes < (int64_t)sizeof(FitWork)) return TQ_E_SHAPE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 7) != 0 || (reinterpret_cast<uintptr_t>(samples) & 3) != 0)
        return TQ_E_ALIGN;
    for (int j = 1; j < levels; ++j)
        if (!(init[j - 1] < init[j])) return TQ_E_SHAPE; // strictly ascending, finite order
    hipStream_t st = (hipStream_t)stream;
    FitWork *w = static_cast<FitWork *>(workspace);
    int32_t r = TQ_OK;
    if ((r = hip_ok(hipMemcpyAsync(w->cent, init, sizeof(double) * levels, hipMemcpyHostToDevice, st))) != TQ_OK)
        return r;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || cus <= 0)
        cus = 256;
    const int64_t want = (n / 4 + kFitThreads) / kFitThreads;
    const int64_t cap = 4LL * cus < kFitBlocks ? 4LL * cus : kFitBlocks;
    const int grid = (int)(want < cap ? want : cap);
    hipLaunchKernelGGL(fit_absmax_kernel, dim3(grid), dim3(kFitThreads), 0, st, samples, n, w);
    hipLaunchKernelGGL(fit_init_kernel, dim3(1), dim3(kFitThreads), 0, st, w, grid, n);
    int ns = 1;
    while ((1 << ns) < levels) ++ns; // levels <= 2^ns
    const void *assign = n >= (1 << 11) ? assign_kernel<true>(ns) : assign_kernel<false>(ns);
    int lv = levels;
    for (int32_t it = 0; it < iterations; ++it) {
        const float *xs = samples;
        int64_t nn = n;
        void *args[] = {&xs, &nn, &lv, &w};
        if ((r = hip_ok(hipLaunchKernel(assign, dim3(grid), dim3(kFitThreads), args, 0, st))) != TQ_OK) return r;
        hipLaunchKernelGGL(fit_update_kernel, dim3(levels), dim3(kFitThreads), 0, st, w, grid);
    }
    if ((r = hip_ok(hipGetLastError())) != TQ_OK) return r;
    int shift = 0;
    if ((r = hip_ok(hipMemcpyAsync(centroids, w->cent, sizeof(double) * levels, hipMemcpyDeviceToHost, st))) != TQ_OK)
        return r;
    if ((r = hip_ok(hipMemcpyAsync(&shift, &w->shift, sizeof(int), hipMemcpyDeviceToHost, st))) != TQ_OK) return r;
    if ((r = hip_ok(hipStreamSynchronize(st))) != TQ_OK) return r;
    if (boundaries != nullptr)
        for (int j = 0; j < levels - 1; ++j) boundaries[j] = (centroids[j] + centroids[j + 1]) * 0.5;
    return shift < 0 ? TQ_E_SHAPE : TQ_OK;
}

} // extern "C"
