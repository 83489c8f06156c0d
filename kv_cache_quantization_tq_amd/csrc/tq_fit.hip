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
//
// Method. k(x) depends only on the multiset of boundaries: with them in
// ascending order b'_0 <= b'_1 <= ..., level k holds exactly the samples in
// (b'_{k-1}, b'_k]. An iteration therefore needs, per boundary, only the
// number of samples at or below it and their sum. The samples are sorted
// once (a least-significant-digit radix sort of a 32-bit key whose order is
// the order of the values) and their fixed-point values prefix-summed in
// that order; every iteration then locates each boundary in the sorted keys
// (a splitter table in LDS, then one segment of keys) and reads counts and
// sums as differences of positions and prefix sums. All iterations run in
// one launch of a single block. The set-up reads the samples three times
// and the keys eight times, whatever the number of iterations; an
// iteration reads a few windows of keys and sums, none when the boundaries
// stay inside the windows already held.
//
// Determinism: each sample enters the sums as the exact integer
// rint(x * 2^s), with s chosen from the sample count and the largest
// magnitude so that no partial sum can overflow 63 bits; integer sums do
// not depend on order, so the centroids equal a sequential evaluation of
// the same rule (the centroid is double(sum) * 2^-s / count in binary64).
#include <hip/hip_runtime.h>

#include <math.h>
#include <string.h>

#include "tq.h"
#include "tq_host.h"

namespace {

constexpr int kMaxLevels = 256;
constexpr int kThreads = 256;                // block size of the set-up kernels
constexpr int kMaxBlocks = 1024;             // most blocks of the magnitude pass
constexpr int kItems = 16;                   // keys per thread of a sort tile
constexpr int kTile = kThreads * kItems;     // keys per sort tile
constexpr int kDigits = 256;                 // 8-bit digits, four passes
constexpr int kIterThreads = 1024;           // the iteration kernel's block
constexpr int kSplit = 32768;                // splitter keys held in LDS (128 KB)
constexpr int kSegMax = 512;                 // keys one wavefront counts in one round
constexpr int64_t kMaxSamples = ((int64_t)1 << 31) - 1;

// Start of the caller's workspace; the sample-sized arrays follow it (see
// fit_layout).
struct FitHead {
    double cent[kMaxLevels];
    unsigned int part_max[kMaxBlocks];  // largest |x| bits per block of the magnitude pass
    unsigned int digit_total[kDigits];  // keys per digit in the current sort pass
    int shift;                          // s, or -1 when the samples cannot be fitted
};

struct FitLayout {
    int64_t keys_a, keys_b, prefix, hist, tile_sum, total; // byte offsets; total = size
};

constexpr int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

// keys_a, keys_b: n sort keys each; prefix: n + 1 prefix sums (int64);
// hist: per-digit, per-tile key counts; tile_sum: per-tile sums (int64)
FitLayout fit_layout(int64_t n)
{
    const int64_t tiles = (n + kTile - 1) / kTile;
    FitLayout l;
    int64_t o = align256((int64_t)sizeof(FitHead));
    l.keys_a = o;
    o = align256(o + 4 * n);
    l.keys_b = o;
    o = align256(o + 4 * n);
    l.prefix = o;
    o = align256(o + 8 * (n + 1));
    l.hist = o;
    o = align256(o + 4 * (int64_t)kDigits * tiles);
    l.tile_sum = o;
    o = align256(o + 8 * tiles);
    l.total = o;
    return l;
}

// ---------------------------------------------------------------------------
// Keys and fixed-point values
// ---------------------------------------------------------------------------

// A 32-bit key per float whose unsigned order is the order of the values
// (for finite values; -0 sorts just below +0), and its inverse.
__device__ __forceinline__ unsigned int float_key(float x)
{
    const unsigned int u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_float(unsigned int k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Key of the last value equal to b: x <= b exactly when float_key(x) <=
// bound_key(b) (both zeros are <= a zero boundary).
__device__ __forceinline__ unsigned int bound_key(float b)
{
    return b == 0.0f ? 0x80000000u : float_key(b);
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

// ---------------------------------------------------------------------------
// Block and wavefront helpers (kThreads threads)
// ---------------------------------------------------------------------------

__device__ __forceinline__ unsigned long long lanes_below()
{
    return (1ull << (threadIdx.x & 63)) - 1ull;
}

// Exclusive prefix of v over the block's threads in thread order; `total`
// receives the sum over all threads.
template <typename T> __device__ T block_exclusive_scan(T v, T &total)
{
    __shared__ T wsum[kThreads / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    T x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const T y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    T base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
        base += w < wave ? wsum[w] : (T)0;
        tot += wsum[w];
    }
    __syncthreads(); // wsum is reused by the next call
    total = tot;
    return base + x - v;
}

// Lanes of the wavefront, among those with `valid`, whose digit equals this
// lane's (eight votes, one per digit bit). Per bit and 32-bit half of the
// mask: m &= ~(vote ^ x) with x = all ones where this lane's bit is set,
// one three-input bitwise instruction.
__device__ __forceinline__ unsigned long long match_digit(unsigned int d, bool valid)
{
    const unsigned long long v0 = __ballot(valid);
    unsigned int lo = (unsigned int)v0, hi = (unsigned int)(v0 >> 32);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const unsigned int x = 0u - ((d >> b) & 1u);
        const unsigned long long v = __ballot(x != 0u);
        lo &= ~((unsigned int)v ^ x);
        hi &= ~((unsigned int)(v >> 32) ^ x);
    }
    return ((unsigned long long)hi << 32) | lo;
}

// ---------------------------------------------------------------------------
// Largest magnitude and the fixed-point shift
// ---------------------------------------------------------------------------

// largest |x| of a block's samples as the bit pattern of a non-negative
// float (its integer order is the float order; NaN patterns order above
// +inf)
__global__ void __launch_bounds__(kThreads) fit_absmax_kernel(const float *x, int64_t n, FitHead *h)
{
    unsigned int m = 0;
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x, nt = (int64_t)gridDim.x * kThreads;
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
    __shared__ unsigned int wm[kThreads / 64];
    if ((threadIdx.x & 63) == 0) wm[threadIdx.x / 64] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < kThreads / 64; ++i) m = max(m, wm[i]);
        h->part_max[blockIdx.x] = m;
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
    const int s = 62 - bl - e;
    return s > 40 ? 40 : s;
}

// one block: the largest magnitude over the magnitude pass's blocks, then
// the shift
__global__ void __launch_bounds__(kThreads) fit_init_kernel(FitHead *h, int blocks, int64_t n)
{
    __shared__ unsigned int red[kThreads];
    unsigned int m = 0;
    for (int b = threadIdx.x; b < blocks; b += kThreads) m = max(m, h->part_max[b]);
    red[threadIdx.x] = m;
    __syncthreads();
    for (int half = kThreads / 2; half > 0; half >>= 1) {
        if (threadIdx.x < half) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + half]);
        __syncthreads();
    }
    if (threadIdx.x == 0) h->shift = fit_shift(red[0], n);
}

// ---------------------------------------------------------------------------
// Radix sort of the keys: per pass a count, a scan and a stable scatter
// ---------------------------------------------------------------------------
// A tile is kTile consecutive keys; thread t holds keys t, t + kThreads,
// ... of its tile, so step i of a tile covers kThreads consecutive keys in
// thread order. The first pass reads the samples and forms their keys.

// The tile a block processes. Blocks are dispatched to the XCDs in turn
// (block b to XCD b % 8), so tiles are dealt out in contiguous runs, one
// run per XCD: neighbouring tiles then write neighbouring bytes (histogram
// entries, runs of one digit, prefix sums) through the same L2, where
// partly written lines merge instead of being written back from several.
constexpr int kXcds = 8;

__device__ __forceinline__ int64_t block_tile(int64_t tiles)
{
    const int64_t b = blockIdx.x, x = b % kXcds, k = b / kXcds;
    const int64_t q = tiles / kXcds, r = tiles % kXcds;
    return x * q + (x < r ? x : r) + k;
}

template <bool FROM_SAMPLES> __device__ __forceinline__ unsigned int load_key(const void *src, int64_t i)
{
    if constexpr (FROM_SAMPLES) return float_key(static_cast<const float *>(src)[i]);
    else return static_cast<const unsigned int *>(src)[i];
}

template <bool FROM_SAMPLES>
__device__ __forceinline__ void load_tile(const void *src, int64_t n, int64_t tile, unsigned int (&key)[kItems])
{
    const int64_t t0 = tile * kTile + threadIdx.x;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int64_t idx = t0 + (int64_t)i * kThreads;
        key[i] = idx < n ? load_key<FROM_SAMPLES>(src, idx) : 0u;
    }
}

// keys of each digit in each tile, digit-major: hist[d * tiles + tile]
template <bool FROM_SAMPLES>
__global__ void __launch_bounds__(kThreads)
fit_digit_count_kernel(const void *src, int64_t n, int sh, unsigned int *hist, int64_t tiles, const FitHead *h)
{
    if (h->shift < 0) return;
    __shared__ unsigned int cnt[kDigits];
    cnt[threadIdx.x] = 0;
    const int64_t tile = block_tile(tiles);
    unsigned int key[kItems];
    load_tile<FROM_SAMPLES>(src, n, tile, key);
    __syncthreads();
    const int64_t t0 = tile * kTile + threadIdx.x;
    // counting needs no order: one LDS add per key (lanes adding to the
    // same digit are serialised by the LDS, which costs less than matching
    // the lanes' digits first)
#pragma unroll
    for (int i = 0; i < kItems; ++i)
        if (t0 + (int64_t)i * kThreads < n) atomicAdd(&cnt[(key[i] >> sh) & 255u], 1u);
    __syncthreads();
    hist[(int64_t)threadIdx.x * tiles + tile] = cnt[threadIdx.x];
}

// one block per digit: the digit's per-tile counts become exclusive
// prefixes within the digit, and the digit's total goes to the head
__global__ void __launch_bounds__(kThreads) fit_digit_scan_kernel(unsigned int *hist, int64_t tiles, FitHead *h)
{
    if (h->shift < 0) return;
    unsigned int *row = hist + (int64_t)blockIdx.x * tiles;
    const int64_t chunk = (tiles + kThreads - 1) / kThreads;
    const int64_t lo = min((int64_t)threadIdx.x * chunk, tiles), hi = min(lo + chunk, tiles);
    unsigned int s = 0;
    for (int64_t j = lo; j < hi; ++j) s += row[j];
    unsigned int total;
    unsigned int off = block_exclusive_scan<unsigned int>(s, total);
    for (int64_t j = lo; j < hi; ++j) {
        const unsigned int v = row[j];
        row[j] = off;
        off += v;
    }
    if (threadIdx.x == 0) h->digit_total[blockIdx.x] = total;
}

// Stable scatter of a tile: a key goes to (keys of smaller digits) + (keys
// of its digit in earlier tiles) + (keys of its digit earlier in this
// tile). Within a step the earlier keys of the same digit are those of
// lower lanes of the same wavefront and of lower wavefronts. The tile is
// first arranged in LDS in that order (digit by digit), then written out
// with consecutive threads writing consecutive positions of each digit's
// run, rather than each key on its own.
template <bool FROM_SAMPLES>
__global__ void __launch_bounds__(kThreads)
fit_digit_scatter_kernel(const void *src, int64_t n, int sh, const unsigned int *hist, int64_t tiles,
                         const FitHead *h, unsigned int *dst)
{
    if (h->shift < 0) return;
    __shared__ unsigned int start[kDigits];  // destination of the tile's first key of each digit
    __shared__ unsigned int lbase[kDigits];  // place of that key in the arranged tile
    __shared__ unsigned int run[kDigits];    // keys of each digit arranged so far
    __shared__ unsigned int wcnt[kThreads / 64][kDigits];
    __shared__ unsigned int arranged[kTile];
    const int t = threadIdx.x, wave = t >> 6;
    const int64_t tile = block_tile(tiles);
    const int64_t t0 = tile * kTile + t;
    const int nvalid = (int)min((int64_t)kTile, n - tile * kTile);
    run[t] = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) wcnt[w][t] = 0;
    unsigned int key[kItems];
    load_tile<FROM_SAMPLES>(src, n, tile, key);
    __syncthreads();
    // the tile's keys per digit, then where each digit's keys begin in the
    // arranged tile and in the destination
#pragma unroll
    for (int i = 0; i < kItems; ++i)
        if (t0 + (int64_t)i * kThreads < n) atomicAdd(&run[(key[i] >> sh) & 255u], 1u);
    __syncthreads();
    unsigned int total;
    lbase[t] = block_exclusive_scan<unsigned int>(run[t], total);
    const unsigned int base = block_exclusive_scan<unsigned int>(h->digit_total[t], total);
    start[t] = base + hist[(int64_t)t * tiles + tile];
    run[t] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const bool valid = t0 + (int64_t)i * kThreads < n;
        const unsigned int d = (key[i] >> sh) & 255u;
        const unsigned long long peers = match_digit(d, valid);
        const unsigned int rank = (unsigned int)__popcll(peers & lanes_below());
        if (valid && rank == 0) wcnt[wave][d] = (unsigned int)__popcll(peers);
        __syncthreads();
        if (valid) {
            unsigned int p = lbase[d] + run[d] + rank;
            for (int w = 0; w < wave; ++w) p += wcnt[w][d];
            arranged[p] = key[i];
        }
        __syncthreads();
        unsigned int step = 0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) {
            step += wcnt[w][t];
            wcnt[w][t] = 0;
        }
        run[t] += step;
        __syncthreads();
    }
    // key j of the arranged tile goes to start[d] + (j - lbase[d])
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int jj = i * kThreads + t;
        if (jj < nvalid) {
            const unsigned int k = arranged[jj];
            const unsigned int d = (k >> sh) & 255u;
            dst[start[d] + (unsigned int)jj - lbase[d]] = k;
        }
    }
}

// ---------------------------------------------------------------------------
// Prefix sums of the fixed-point values in sorted order
// ---------------------------------------------------------------------------

// sum of each tile's fixed-point values
template <bool MAGIC>
__global__ void __launch_bounds__(kThreads)
fit_tile_sum_kernel(const unsigned int *keys, int64_t n, const FitHead *h, long long *tile_sum)
{
    const int s = h->shift;
    if (s < 0) return;
    const int64_t tile = block_tile((n + kTile - 1) / kTile);
    const int64_t t0 = tile * kTile + threadIdx.x;
    long long acc = 0;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int64_t idx = t0 + (int64_t)i * kThreads;
        if (idx < n) acc += fixed_point<MAGIC>(key_float(keys[idx]), s);
    }
    long long total;
    block_exclusive_scan<long long>(acc, total);
    if (threadIdx.x == 0) tile_sum[tile] = total;
}

// one block: the tile sums become exclusive prefixes
__global__ void __launch_bounds__(kThreads) fit_tile_scan_kernel(long long *tile_sum, int64_t tiles, const FitHead *h)
{
    if (h->shift < 0) return;
    const int64_t chunk = (tiles + kThreads - 1) / kThreads;
    const int64_t lo = min((int64_t)threadIdx.x * chunk, tiles), hi = min(lo + chunk, tiles);
    long long s = 0;
    for (int64_t j = lo; j < hi; ++j) s += tile_sum[j];
    long long total;
    long long off = block_exclusive_scan<long long>(s, total);
    for (int64_t j = lo; j < hi; ++j) {
        const long long v = tile_sum[j];
        tile_sum[j] = off;
        off += v;
    }
}

// prefix[i] = sum of the fixed-point values of sorted keys 0 .. i-1. A tile
// is staged in LDS (one padding entry per 16, so that each thread's run of
// 16 consecutive entries falls in distinct banks), each thread sums a run,
// and the block scan of the runs gives every prefix.
template <bool MAGIC>
__global__ void __launch_bounds__(kThreads)
fit_prefix_kernel(const unsigned int *keys, int64_t n, const FitHead *h, const long long *tile_sum, long long *prefix)
{
    const int s = h->shift;
    if (s < 0) return;
    __shared__ long long q[kTile + kTile / kItems];
    auto slot = [](int j) { return j + (j >> 4); };
    const int t = threadIdx.x;
    const int64_t tile = block_tile((n + kTile - 1) / kTile);
    const int64_t t0 = tile * kTile;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int j = i * kThreads + t;
        q[slot(j)] = t0 + j < n ? fixed_point<MAGIC>(key_float(keys[t0 + j]), s) : 0;
    }
    __syncthreads();
    long long run = 0;
#pragma unroll
    for (int k = 0; k < kItems; ++k) run += q[slot(t * kItems + k)];
    long long total;
    long long acc = block_exclusive_scan<long long>(run, total) + tile_sum[tile];
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        acc += q[slot(t * kItems + k)];
        q[slot(t * kItems + k)] = acc; // inclusive prefix of entry t * kItems + k
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int j = i * kThreads + t;
        if (t0 + j < n) prefix[t0 + j + 1] = q[slot(j)];
    }
    if (tile == 0 && t == 0) prefix[0] = 0;
}

// ---------------------------------------------------------------------------
// The iterations
// ---------------------------------------------------------------------------

// the value of v in lane `src` (uniform), through the scalar unit
__device__ __forceinline__ long long lane_value(long long v, int src)
{
    const unsigned long long u = (unsigned long long)v;
    const unsigned int lo = (unsigned int)__builtin_amdgcn_readlane((int)(unsigned int)u, src);
    const unsigned int hi = (unsigned int)__builtin_amdgcn_readlane((int)(unsigned int)(u >> 32), src);
    return (long long)(((unsigned long long)hi << 32) | lo);
}

// The last window of sorted keys a wavefront counted for one boundary:
// keys[glo .. glo + glen) (glen <= kSegMax) with keys[glo] <= K and the first
// key above K in (glo, glo + glen]. Lane l holds keys glo + 64 e + l and
// the prefix sums at those positions; the window is reused while it still
// brackets the boundary (boundaries move little between late iterations),
// which costs no memory access at all.
constexpr int kWinR = kSegMax / 64; // keys (and prefix sums) per lane in a window

struct Window {
    int64_t glo;
    int glen;
    unsigned int first;  // keys[glo]
    unsigned int next;   // keys[glo + glen], or 0xffffffff (above every key) at the end
    bool ok;
    unsigned int kv[kWinR];  // 0xffffffff past the window
    long long pv[kWinR + 1]; // prefix[glo + 64 e + l] for 64 e + l <= glen
};

// Position of boundary key K in the sorted keys (the number of keys <= K)
// and the prefix sum there, computed by one wavefront (K is uniform).
// spl[i] = keys[i * seg] for i < nsp. Each narrowing round probes 64
// evenly spaced candidates and keeps the interval after the last one <= K.
__device__ __forceinline__ void locate(const unsigned int *__restrict__ keys, const long long *__restrict__ prefix,
                                       int64_t n, int64_t seg, int nsp, const unsigned int *spl, unsigned int K,
                                       Window &w, int64_t &pos, long long &psum)
{
    constexpr int R = kWinR;
    const int lane = threadIdx.x & 63;
    if (!(w.ok && w.first <= K && K < w.next)) {
        // last splitter <= K, in LDS
        int lo = 0, len = nsp;
        bool none = false;
        while (len > 64) {
            const int stride = (len + 63) / 64;
            const int i = lo + lane * stride;
            const int c = __popcll(__ballot(i < lo + len && spl[i] <= K));
            if (c == 0) { // only possible in the first round (spl[lo] <= K after it)
                none = true;
                break;
            }
            lo += (c - 1) * stride;
            len = min(stride, len - (c - 1) * stride);
        }
        if (!none) {
            const int c = __popcll(__ballot(lane < len && spl[lo + lane] <= K));
            none = c == 0;
            lo += c - 1;
        }
        if (none) { // every key is above K
            w.ok = false;
            pos = 0;
            psum = 0;
            return;
        }
        // keys[glo] <= K, and the first key above K is in (glo, glo + glen]
        int64_t glo = (int64_t)lo * seg, glen = min(seg, n - glo);
        while (glen > kSegMax) {
            const int64_t stride = (glen + 63) / 64;
            const int64_t i = glo + lane * stride;
            const int c = __popcll(__ballot(i < glo + glen && keys[i] <= K));
            glo += (c - 1) * stride;
            glen = min(stride, glen - (c - 1) * stride);
        }
        const int64_t wlo = glo, wlen = glen;
        // the window's keys and the prefix sums at every candidate position,
        // in one round of loads
#pragma unroll
        for (int e = 0; e < R; ++e) {
            const int64_t j = e * 64 + lane;
            w.kv[e] = j < wlen ? keys[wlo + j] : 0xffffffffu;
            w.pv[e] = j <= wlen ? prefix[wlo + j] : 0;
        }
        w.pv[R] = lane == 0 && R * 64 <= wlen ? prefix[wlo + R * 64] : 0;
        w.next = wlo + wlen < n ? keys[wlo + wlen] : 0xffffffffu;
        w.first = (unsigned int)__builtin_amdgcn_readfirstlane((int)w.kv[0]);
        w.glo = wlo;
        w.glen = (int)wlen;
        w.ok = true;
    }
    // the keys <= K are a prefix of the window
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < R; ++e) cnt += __popcll(__ballot(w.kv[e] <= K));
    // the prefix sum at the position: entry cnt >> 6 of lane cnt & 63,
    // broadcast entry by entry (a select over the entries with the uniform
    // index would be compiled to an indexed copy in scratch memory)
    long long v = 0;
#pragma unroll
    for (int e = 0; e <= R; ++e) {
        const long long x = lane_value(w.pv[e], cnt & 63);
        v = (cnt >> 6) == e ? x : v;
    }
    pos = w.glo + cnt;
    psum = v;
}

// All iterations in one block. An iteration: one wavefront per boundary
// locates it (wavefront w takes boundaries w, w + 16, ...; the windows of
// the first kCached of them stay in its registers); then thread k forms the
// new centroids of levels k .. k + 2 from the counts and sums (a level with
// no sample keeps its value; centroids are double-buffered so that every
// thread reads the old values) and the key of boundary k for the next
// iteration, rounded down to float32 (which decides b < x exactly for
// float32 samples: no float32 lies strictly between a binary64 value and
// its round-down). Boundaries out of ascending order are sorted.
constexpr int kCached = 1;

__device__ __forceinline__ unsigned int boundary_key(double lo, double hi)
{
    return bound_key(__double2float_rd((lo + hi) * 0.5));
}

__global__ void __launch_bounds__(kIterThreads)
fit_iterate_kernel(const unsigned int *__restrict__ keys, const long long *__restrict__ prefix, int64_t n,
                   int levels, int iterations, FitHead *h)
{
    const int s = h->shift;
    if (s < 0) return;
    __shared__ unsigned int spl[kSplit];
    __shared__ double cent[2][kMaxLevels];
    __shared__ unsigned int bkey[kMaxLevels];
    __shared__ int64_t pos[kMaxLevels];
    __shared__ long long psum[kMaxLevels];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    constexpr int kWaves = kIterThreads / 64;
    const int64_t seg = (n + kSplit - 1) / kSplit;
    const int nsp = (int)((n + seg - 1) / seg);
    for (int i = t; i < nsp; i += kIterThreads) spl[i] = keys[(int64_t)i * seg];
    for (int k = t; k < levels; k += kIterThreads) cent[0][k] = h->cent[k];
    const long long total = prefix[n];
    const int nb = levels - 1;
    __syncthreads();
    auto sort_keys = [&](bool down) {
        if (__syncthreads_or(down)) {
            // ascending order by rank, equal keys by index
            unsigned int mine = 0;
            int r = 0;
            if (t < nb) {
                mine = bkey[t];
                for (int j = 0; j < nb; ++j) {
                    const unsigned int o = bkey[j];
                    r += (o < mine || (o == mine && j < t)) ? 1 : 0;
                }
            }
            __syncthreads();
            if (t < nb) bkey[r] = mine;
            __syncthreads();
        }
    };
    unsigned int k0 = 0, k1 = 0;
    if (t < nb) k0 = bkey[t] = boundary_key(cent[0][t], cent[0][t + 1]);
    __syncthreads();
    if (t + 1 < nb) k1 = bkey[t + 1];
    sort_keys(t + 1 < nb && k0 > k1);
    Window win[kCached];
#pragma unroll
    for (int m = 0; m < kCached; ++m) win[m].ok = false;
    int cur = 0;
    for (int it = 0; it < iterations; ++it) {
#pragma unroll
        for (int m = 0; m < kCached; ++m) {
            const int j = wave + m * kWaves;
            if (j < nb) {
                int64_t p;
                long long ps;
                locate(keys, prefix, n, seg, nsp, spl, bkey[j], win[m], p, ps);
                if (lane == 0) {
                    pos[j] = p;
                    psum[j] = ps;
                }
            }
        }
        for (int j = wave + kCached * kWaves; j < nb; j += kWaves) {
            Window tmp;
            tmp.ok = false;
            int64_t p;
            long long ps;
            locate(keys, prefix, n, seg, nsp, spl, bkey[j], tmp, p, ps);
            if (lane == 0) {
                pos[j] = p;
                psum[j] = ps;
            }
        }
        __syncthreads();
        auto newc = [&](int k) {
            const int64_t hi = k < nb ? pos[k] : n, lo = k > 0 ? pos[k - 1] : 0;
            const long long shi = k < nb ? psum[k] : total, slo = k > 0 ? psum[k - 1] : 0;
            return hi > lo ? ldexp((double)(shi - slo), -s) / (double)(hi - lo) : cent[cur][k];
        };
        bool down = false;
        if (t < levels) {
            const double c0 = newc(t);
            cent[cur ^ 1][t] = c0;
            if (t < nb) {
                const double c1 = newc(t + 1);
                k0 = boundary_key(c0, c1);
                if (t + 1 < nb) {
                    k1 = boundary_key(c1, newc(t + 2));
                    down = k0 > k1;
                }
                bkey[t] = k0; // every wavefront has read bkey before the barrier above
            }
        }
        sort_keys(down);
        cur ^= 1;
    }
    for (int k = t; k < levels; k += kIterThreads) h->cent[k] = cent[cur][k];
}

// Tables of up to 17 levels (one boundary per wavefront): every wavefront
// holds all centroids (level k in lane k) and recomputes the new centroids
// and boundary keys itself from the positions and sums the wavefronts
// published, so an iteration needs one barrier. Positions and sums are
// double-buffered by iteration parity: a wavefront can only start writing
// a buffer again after every wavefront has passed the barrier of the
// iteration in between.
constexpr int kSmallLevels = kIterThreads / 64 + 1;

// lane j: the key of boundary j (ascending), from the centroids in lanes
// 0 .. levels - 1; lanes from levels - 1 on get 0xffffffff
__device__ __forceinline__ unsigned int wave_boundary_keys(double c, int levels, unsigned int *sortbuf)
{
    const int lane = threadIdx.x & 63, nb = levels - 1;
    const double cn = __shfl_down(c, 1);
    unsigned int k = lane < nb ? boundary_key(c, cn) : 0xffffffffu;
    const unsigned int kn = __shfl_down(k, 1);
    if (__ballot(lane + 1 < nb && k > kn) != 0) {
        // out of order (possible only through rounding): rank sort, equal
        // keys by lane
        int r = 0;
        for (int i = 0; i < nb; ++i) {
            const unsigned int o = (unsigned int)__builtin_amdgcn_readlane((int)k, i);
            r += (o < k || (o == k && i < lane)) ? 1 : 0;
        }
        if (lane < nb) sortbuf[r] = k;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        k = lane < nb ? sortbuf[lane] : 0xffffffffu;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    return k;
}

__global__ void __launch_bounds__(kIterThreads)
fit_iterate_small_kernel(const unsigned int *__restrict__ keys, const long long *__restrict__ prefix, int64_t n,
                         int levels, int iterations, FitHead *h)
{
    const int s = h->shift;
    if (s < 0) return;
    constexpr int kWaves = kIterThreads / 64;
    __shared__ unsigned int spl[kSplit];
    __shared__ int64_t pos[2][kSmallLevels];
    __shared__ long long psum[2][kSmallLevels];
    __shared__ unsigned int sortbuf[kWaves][kSmallLevels];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t seg = (n + kSplit - 1) / kSplit;
    const int nsp = (int)((n + seg - 1) / seg);
    for (int i = t; i < nsp; i += kIterThreads) spl[i] = keys[(int64_t)i * seg];
    const long long total = prefix[n];
    const int nb = levels - 1;
    double c = lane < levels ? h->cent[lane] : 0.0;
    __syncthreads();
    unsigned int K = wave_boundary_keys(c, levels, sortbuf[wave]);
    Window win; // wavefront w's window for boundary w
    win.ok = false;
    for (int it = 0; it < iterations; ++it) {
        const int b = it & 1;
        if (wave < nb) {
            const unsigned int Kw = (unsigned int)__builtin_amdgcn_readlane((int)K, wave);
            int64_t p;
            long long ps;
            locate(keys, prefix, n, seg, nsp, spl, Kw, win, p, ps);
            if (lane == 0) {
                pos[b][wave] = p;
                psum[b][wave] = ps;
            }
        }
        __syncthreads();
        if (lane < levels) {
            const int64_t hi = lane < nb ? pos[b][lane] : n, lo = lane > 0 ? pos[b][lane - 1] : 0;
            const long long shi = lane < nb ? psum[b][lane] : total, slo = lane > 0 ? psum[b][lane - 1] : 0;
            if (hi > lo) c = ldexp((double)(shi - slo), -s) / (double)(hi - lo);
        }
        K = wave_boundary_keys(c, levels, sortbuf[wave]);
    }
    if (wave == 0 && lane < levels) h->cent[lane] = c;
}

int32_t hip_ok(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_E_HIP; }

} // namespace

extern "C" {

int64_t tq_lloyd_max_workspace_bytes(int64_t n)
{
    if (n < 1 || n > kMaxSamples) return -TQ_E_SHAPE;
    return fit_layout(n).total;
}

int32_t tq_lloyd_max_fit(const float *samples, int64_t n, int32_t levels, const double *init, int32_t iterations,
                         double *centroids, double *boundaries, void *workspace, int64_t workspace_bytes,
                         void *stream)
{
    const tq_host::TimingScope timing;
    if (levels < 2 || levels > kMaxLevels) return TQ_E_BITS;
    if (n < 1 || n > kMaxSamples || iterations < 0) return TQ_E_SHAPE;
    if (samples == nullptr || init == nullptr || centroids == nullptr || workspace == nullptr) return TQ_E_NULL;
    const FitLayout lay = fit_layout(n);
    if (workspace_bytes < lay.total) return TQ_E_SHAPE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 7) != 0 || (reinterpret_cast<uintptr_t>(samples) & 3) != 0)
        return TQ_E_ALIGN;
    for (int j = 1; j < levels; ++j)
        if (!(init[j - 1] < init[j])) return TQ_E_SHAPE; // strictly ascending, finite order
    hipStream_t st = (hipStream_t)stream;
    char *ws = static_cast<char *>(workspace);
    FitHead *h = reinterpret_cast<FitHead *>(ws);
    unsigned int *keys_a = reinterpret_cast<unsigned int *>(ws + lay.keys_a);
    unsigned int *keys_b = reinterpret_cast<unsigned int *>(ws + lay.keys_b);
    long long *prefix = reinterpret_cast<long long *>(ws + lay.prefix);
    unsigned int *hist = reinterpret_cast<unsigned int *>(ws + lay.hist);
    long long *tile_sum = reinterpret_cast<long long *>(ws + lay.tile_sum);
    int32_t r = TQ_OK;
    if ((r = hip_ok(hipMemcpyAsync(h->cent, init, sizeof(double) * levels, hipMemcpyHostToDevice, st))) != TQ_OK)
        return r;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || cus <= 0)
        cus = 256;
    const int64_t want = (n / 4 + kThreads) / kThreads;
    const int64_t cap = 4LL * cus < kMaxBlocks ? 4LL * cus : kMaxBlocks;
    const int grid = (int)(want < cap ? want : cap);
    {
        const float *a0 = samples;
        int64_t a1 = n;
        FitHead *a2 = h;
        void *args[] = {&a0, &a1, &a2};
        if ((r = tq_host::launch_kernel(reinterpret_cast<const void *>(&fit_absmax_kernel), dim3(grid),
                                        dim3(kThreads), args, 0, st, true, false)) != TQ_OK)
            return r;
    }
    {
        FitHead *a0 = h;
        int a1 = grid;
        int64_t a2 = n;
        void *args[] = {&a0, &a1, &a2};
        if ((r = tq_host::launch_kernel(reinterpret_cast<const void *>(&fit_init_kernel), dim3(1), dim3(kThreads),
                                        args, 0, st, false, iterations == 0)) != TQ_OK)
            return r;
    }
    if (iterations > 0) {
        const int64_t tiles = (n + kTile - 1) / kTile;
        // four passes: samples -> b -> a -> b -> a
        for (int pass = 0; pass < 4; ++pass) {
            const int sh = 8 * pass;
            const void *src = pass == 0 ? static_cast<const void *>(samples) : (pass & 1 ? keys_b : keys_a);
            unsigned int *dst = pass & 1 ? keys_a : keys_b;
            if (pass == 0) {
                hipLaunchKernelGGL(fit_digit_count_kernel<true>, dim3(tiles), dim3(kThreads), 0, st, src, n, sh, hist,
                                   tiles, h);
            } else {
                hipLaunchKernelGGL(fit_digit_count_kernel<false>, dim3(tiles), dim3(kThreads), 0, st, src, n, sh, hist,
                                   tiles, h);
            }
            hipLaunchKernelGGL(fit_digit_scan_kernel, dim3(kDigits), dim3(kThreads), 0, st, hist, tiles, h);
            if (pass == 0) {
                hipLaunchKernelGGL(fit_digit_scatter_kernel<true>, dim3(tiles), dim3(kThreads), 0, st, src, n, sh,
                                   hist, tiles, h, dst);
            } else {
                hipLaunchKernelGGL(fit_digit_scatter_kernel<false>, dim3(tiles), dim3(kThreads), 0, st, src, n, sh,
                                   hist, tiles, h, dst);
            }
        }
        if (n >= (1 << 11)) {
            hipLaunchKernelGGL(fit_tile_sum_kernel<true>, dim3(tiles), dim3(kThreads), 0, st, keys_a, n, h, tile_sum);
        } else {
            hipLaunchKernelGGL(fit_tile_sum_kernel<false>, dim3(tiles), dim3(kThreads), 0, st, keys_a, n, h, tile_sum);
        }
        hipLaunchKernelGGL(fit_tile_scan_kernel, dim3(1), dim3(kThreads), 0, st, tile_sum, tiles, h);
        if (n >= (1 << 11)) {
            hipLaunchKernelGGL(fit_prefix_kernel<true>, dim3(tiles), dim3(kThreads), 0, st, keys_a, n, h, tile_sum,
                               prefix);
        } else {
            hipLaunchKernelGGL(fit_prefix_kernel<false>, dim3(tiles), dim3(kThreads), 0, st, keys_a, n, h, tile_sum,
                               prefix);
        }
        const unsigned int *a0 = keys_a;
        const long long *a1 = prefix;
        int64_t a2 = n;
        int a3 = levels, a4 = iterations;
        FitHead *a5 = h;
        void *args[] = {&a0, &a1, &a2, &a3, &a4, &a5};
        const void *fn = levels <= kSmallLevels ? reinterpret_cast<const void *>(&fit_iterate_small_kernel)
                                                : reinterpret_cast<const void *>(&fit_iterate_kernel);
        if ((r = tq_host::launch_kernel(fn, dim3(1), dim3(kIterThreads), args, 0, st, false, true)) != TQ_OK) return r;
    }
    if ((r = hip_ok(hipGetLastError())) != TQ_OK) return r;
    int shift = 0;
    if ((r = hip_ok(hipMemcpyAsync(centroids, h->cent, sizeof(double) * levels, hipMemcpyDeviceToHost, st))) != TQ_OK)
        return r;
    if ((r = hip_ok(hipMemcpyAsync(&shift, &h->shift, sizeof(int), hipMemcpyDeviceToHost, st))) != TQ_OK) return r;
    if ((r = hip_ok(hipStreamSynchronize(st))) != TQ_OK) return r;
    if (boundaries != nullptr)
        for (int j = 0; j < levels - 1; ++j) boundaries[j] = (centroids[j] + centroids[j + 1]) * 0.5;
    return shift < 0 ? TQ_E_SHAPE : TQ_OK;
}

} // extern "C"
