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
// This file runs the iterations on the device with no host round trip.
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
constexpr int kFitWaves = kFitThreads / 64;

// Device workspace (caller-owned).
struct FitWork {
    double cent[kMaxLevels];
    double bnd[kMaxLevels];          // L - 1 boundaries, then +inf
    unsigned long long sum[kMaxLevels]; // two's complement int64
    unsigned long long cnt[kMaxLevels];
    unsigned int absmax_bits;        // largest |x| as float bits (NaN bits if any sample is NaN)
    int shift;                       // s, or -1 when the samples cannot be fitted
};

// largest |x| (as the bit pattern of a non-negative float, whose integer
// order is the float order; NaN patterns order above +inf)
__global__ void __launch_bounds__(kFitThreads) fit_absmax_kernel(const float *x, int64_t n, FitWork *w)
{
    unsigned int m = 0;
    for (int64_t i = (int64_t)blockIdx.x * kFitThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kFitThreads)
        m = max(m, __float_as_uint(x[i]) & 0x7fffffffu);
    for (int o = 32; o > 0; o >>= 1) m = max(m, (unsigned int)__shfl_xor((int)m, o));
    if ((threadIdx.x & 63) == 0) atomicMax(&w->absmax_bits, m);
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

__device__ void fit_boundaries(FitWork *w, int levels)
{
    for (int j = threadIdx.x; j < kMaxLevels; j += kFitThreads)
        w->bnd[j] = j < levels - 1 ? (w->cent[j] + w->cent[j + 1]) * 0.5 : (double)INFINITY;
}

// one block: the shift, the first boundaries, cleared accumulators
__global__ void __launch_bounds__(kFitThreads) fit_init_kernel(FitWork *w, int levels, int64_t n)
{
    if (threadIdx.x == 0) w->shift = fit_shift(w->absmax_bits, n);
    for (int j = threadIdx.x; j < kMaxLevels; j += kFitThreads) {
        w->sum[j] = 0;
        w->cnt[j] = 0;
    }
    fit_boundaries(w, levels);
}

// assignment and per-level integer sums; per-wavefront LDS histograms,
// merged into the workspace with integer atomics
__global__ void __launch_bounds__(kFitThreads) fit_assign_kernel(const float *x, int64_t n, FitWork *w)
{
    __shared__ double bnd[kMaxLevels];
    __shared__ unsigned long long hsum[kFitWaves][kMaxLevels];
    __shared__ unsigned int hcnt[kFitWaves][kMaxLevels];
    const int s = w->shift;
    if (s < 0) return;
    for (int j = threadIdx.x; j < kMaxLevels; j += kFitThreads) {
        bnd[j] = w->bnd[j];
        for (int v = 0; v < kFitWaves; ++v) {
            hsum[v][j] = 0;
            hcnt[v][j] = 0;
        }
    }
    __syncthreads();
    const int wave = threadIdx.x / 64;
    for (int64_t i = (int64_t)blockIdx.x * kFitThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kFitThreads) {
        const double xd = (double)x[i];
        // k = #{ j : bnd[j] < x } over 255 sorted entries padded with +inf
        int k = 0;
#pragma unroll
        for (int step = 128; step > 0; step >>= 1)
            if (bnd[k + step - 1] < xd) k += step;
        const long long q = (long long)rint(ldexp(xd, s));
        atomicAdd(&hsum[wave][k], (unsigned long long)q);
        atomicAdd(&hcnt[wave][k], 1u);
    }
    __syncthreads();
    for (int j = threadIdx.x; j < kMaxLevels; j += kFitThreads) {
        unsigned long long sm = 0, c = 0;
        for (int v = 0; v < kFitWaves; ++v) {
            sm += hsum[v][j];
            c += hcnt[v][j];
        }
        if (c != 0) {
            atomicAdd(&w->sum[j], sm);
            atomicAdd(&w->cnt[j], c);
        }
    }
}

// one block: new centroids from the sums, new boundaries, cleared sums
__global__ void __launch_bounds__(kFitThreads) fit_update_kernel(FitWork *w, int levels)
{
    const int s = w->shift;
    if (s < 0) return;
    for (int j = threadIdx.x; j < levels; j += kFitThreads) {
        const unsigned long long c = w->cnt[j];
        if (c != 0) w->cent[j] = ldexp((double)(long long)w->sum[j], -s) / (double)c;
        w->sum[j] = 0;
        w->cnt[j] = 0;
    }
    __syncthreads();
    fit_boundaries(w, levels);
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
    const unsigned int zero = 0;
    if ((r = hip_ok(hipMemcpyAsync(w->cent, init, sizeof(double) * levels, hipMemcpyHostToDevice, st))) != TQ_OK)
        return r;
    if ((r = hip_ok(hipMemcpyAsync(&w->absmax_bits, &zero, sizeof(zero), hipMemcpyHostToDevice, st))) != TQ_OK)
        return r;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || cus <= 0)
        cus = 256;
    const int64_t want = (n + kFitThreads - 1) / kFitThreads;
    const unsigned int grid = (unsigned int)(want < 4LL * cus ? want : 4LL * cus);
    hipLaunchKernelGGL(fit_absmax_kernel, dim3(grid), dim3(kFitThreads), 0, st, samples, n, w);
    hipLaunchKernelGGL(fit_init_kernel, dim3(1), dim3(kFitThreads), 0, st, w, (int)levels, n);
    for (int32_t it = 0; it < iterations; ++it) {
        hipLaunchKernelGGL(fit_assign_kernel, dim3(grid), dim3(kFitThreads), 0, st, samples, n, w);
        hipLaunchKernelGGL(fit_update_kernel, dim3(1), dim3(kFitThreads), 0, st, w, (int)levels);
    }
    if ((r = hip_ok(hipGetLastError())) != TQ_OK) return r;
    int shift = 0;
    if ((r = hip_ok(hipMemcpyAsync(centroids, w->cent, sizeof(double) * levels, hipMemcpyDeviceToHost, st))) != TQ_OK)
        return r;
    if (boundaries != nullptr &&
        (r = hip_ok(hipMemcpyAsync(boundaries, w->bnd, sizeof(double) * (levels - 1), hipMemcpyDeviceToHost, st))) !=
            TQ_OK)
        return r;
    if ((r = hip_ok(hipMemcpyAsync(&shift, &w->shift, sizeof(int), hipMemcpyDeviceToHost, st))) != TQ_OK) return r;
    if ((r = hip_ok(hipStreamSynchronize(st))) != TQ_OK) return r;
    return shift < 0 ? TQ_E_SHAPE : TQ_OK;
}

} // extern "C"
