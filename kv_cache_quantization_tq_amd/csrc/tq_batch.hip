// tq_batch.hip -- token-axis batching of packed caches: merge, extend,
// extract and filter over the five codec planes (include/tq.h).
//
// The page "mlx-bun 0.0.9 -> 0.0.11", src/model/batched-quant.ts
// (mergeQuantRows, extendQuantRows, extractQuantRow, filterQuantRows)
// defines these operations for left-padded batches of quantised caches and
// notes why they are byte-exact: quantisation groups run along head_dim
// only, so every token of every plane is a self-contained run of bytes and
// re-arranging tokens never touches a group. Here a batch of b sequences of
// width W tokens is the planes of b * W tokens (sequence-major, then token,
// then head), sequence s occupying tokens [s * W, (s + 1) * W). Every
// operation is therefore a list of contiguous byte segments per plane,
// each either copied from a source or zero-filled (left padding); one
// kernel performs a list of segments.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <vector>

#include "tq.h"
#include "tq_host.h"

namespace {

using tq_host::valid_bits;
using tq_host::valid_head_dim;
using tq_host::valid_key_cfg;

// One contiguous run of bytes: copied from src, or zero-filled when src is
// NULL.
struct Seg {
    const uint8_t *src;
    uint8_t *dst;
    int64_t bytes;
};

constexpr int kMaxSegs = 120;           // per launch (kernel arguments stay under 4 KB)
constexpr int kThreads = 256;
constexpr int64_t kChunk = 64 * 1024;   // bytes per block (a multiple of 16)

struct SegList {
    int32_t count;
    int32_t pad;
    Seg s[kMaxSegs];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Block (x, y) moves bytes [x * kChunk, (x + 1) * kChunk) of segment y. Whole
// 16-byte vectors when the segment's ends allow, else 4-byte words, else
// single bytes (code rows of 3-bit values at head_dim 64 are 24 bytes).
// Every byte is read once and written once, so loads and stores carry the
// non-temporal hint.
__global__ void __launch_bounds__(kThreads) segment_copy_kernel(SegList L)
{
    const int si = blockIdx.y;
    if (si >= L.count) return;
    const Seg sg = L.s[si];
    const int64_t b0 = (int64_t)blockIdx.x * kChunk;
    if (b0 >= sg.bytes) return;
    const int64_t b1 = b0 + kChunk < sg.bytes ? b0 + kChunk : sg.bytes;
    const uintptr_t al = reinterpret_cast<uintptr_t>(sg.src) | reinterpret_cast<uintptr_t>(sg.dst) |
                         static_cast<uintptr_t>(b1);
    const int t = threadIdx.x;
    if ((al & 15) == 0) {
        const u32x4 *s4 = reinterpret_cast<const u32x4 *>(sg.src);
        u32x4 *d4 = reinterpret_cast<u32x4 *>(sg.dst);
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const int64_t e = b1 / 16;
        int64_t i = b0 / 16 + t;
        // four loads in flight per thread before their stores
        for (; i + 3 * kThreads < e; i += 4 * kThreads) {
            u32x4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = s4 != nullptr ? __builtin_nontemporal_load(s4 + i + u * kThreads) : zero;
#pragma unroll
            for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], d4 + i + u * kThreads);
        }
        for (; i < e; i += kThreads)
            __builtin_nontemporal_store(s4 != nullptr ? __builtin_nontemporal_load(s4 + i) : zero, d4 + i);
    } else if ((al & 3) == 0) {
        const uint32_t *s1 = reinterpret_cast<const uint32_t *>(sg.src);
        uint32_t *d1 = reinterpret_cast<uint32_t *>(sg.dst);
        for (int64_t i = b0 / 4 + t; i < b1 / 4; i += kThreads)
            __builtin_nontemporal_store(s1 != nullptr ? __builtin_nontemporal_load(s1 + i) : 0u, d1 + i);
    } else {
        for (int64_t i = b0 + t; i < b1; i += kThreads) sg.dst[i] = sg.src != nullptr ? sg.src[i] : 0;
    }
}

// The planes in a fixed order, with the bytes one token occupies in each
// (heads rows of the plane's row size).
constexpr int kPlanes = 5;

void plane_ptrs(const tq_packed_kv *p, uint8_t *out[kPlanes])
{
    out[0] = static_cast<uint8_t *>(p->k_codes);
    out[1] = static_cast<uint8_t *>(p->k_scale);
    out[2] = static_cast<uint8_t *>(p->k_zero);
    out[3] = static_cast<uint8_t *>(p->v_codes);
    out[4] = static_cast<uint8_t *>(p->v_scale);
}

// Checks the configuration for the planes `dst` has, and fills the bytes
// per token of each plane (0 for a plane dst does not have).
int32_t token_bytes(const tq_config *cfg, int32_t heads, const tq_packed_kv *dst, int64_t tb[kPlanes])
{
    if (cfg == nullptr || dst == nullptr) return TQ_E_NULL;
    if (!valid_head_dim(cfg->head_dim)) return TQ_E_HEAD_DIM;
    if (heads < 1 || heads > (1 << 20)) return TQ_E_SHAPE;
    uint8_t *p[kPlanes];
    plane_ptrs(dst, p);
    const bool has_k = p[0] || p[1] || p[2], has_v = p[3] || p[4];
    if (!has_k && !has_v) return TQ_E_NULL;
    if (has_k && !valid_key_cfg(cfg)) return TQ_E_BITS;
    if (has_v && !valid_bits(cfg->v_bits)) return TQ_E_BITS;
    const int64_t d = cfg->head_dim, g2 = 2 * (d / 32);
    const int64_t rb[kPlanes] = {d * cfg->k_bits / 8, g2, g2, d * cfg->v_bits / 8, g2};
    for (int i = 0; i < kPlanes; ++i) tb[i] = p[i] != nullptr ? rb[i] * heads : 0;
    return TQ_OK;
}

// every plane dst has must be present in src too
int32_t check_src(const tq_packed_kv *src, const tq_packed_kv *dst)
{
    if (src == nullptr) return TQ_E_NULL;
    uint8_t *s[kPlanes], *d[kPlanes];
    plane_ptrs(src, s);
    plane_ptrs(dst, d);
    for (int i = 0; i < kPlanes; ++i)
        if (d[i] != nullptr && s[i] == nullptr) return TQ_E_NULL;
    return TQ_OK;
}

// Collects segments and launches them in batches of kMaxSegs. Every
// segment is checked against the extents of its source and destination
// (in tokens, as the call's arguments define them); a call that would build
// one outside them launches nothing and returns TQ_E_SHAPE.
class Segments {
  public:
    // copy `tokens` tokens from src token s0 (of src_tokens) to dst token d0
    // (of dst_tokens) (src NULL: zero-fill), in every plane dst has
    void add(const tq_packed_kv *src, int64_t s0, int64_t src_tokens, const tq_packed_kv *dst, int64_t d0,
             int64_t dst_tokens, int64_t tokens, const int64_t tb[kPlanes])
    {
        if (tokens <= 0) return;
        if (d0 < 0 || d0 > dst_tokens - tokens || (src != nullptr && (s0 < 0 || s0 > src_tokens - tokens))) {
            outside_ = true;
            return;
        }
        for (int i = 0; i < kPlanes; ++i)
            if (tb[i] > 0 && tokens > INT64_MAX / tb[i]) {
                outside_ = true;
                return;
            }
        uint8_t *s[kPlanes] = {nullptr, nullptr, nullptr, nullptr, nullptr}, *d[kPlanes];
        if (src != nullptr) plane_ptrs(src, s);
        plane_ptrs(dst, d);
        for (int i = 0; i < kPlanes; ++i) {
            if (d[i] == nullptr) continue;
            segs_.push_back(Seg{src != nullptr ? s[i] + s0 * tb[i] : nullptr, d[i] + d0 * tb[i], tokens * tb[i]});
        }
    }

    int32_t launch(void *stream) const
    {
        if (outside_) return TQ_E_SHAPE;
        // A graph replay of calls making several launches each faulted on
        // MI355X (cause not established): such calls refuse capture before
        // launching anything.
        if (segs_.size() > (size_t)kMaxSegs) {
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            if (hipStreamIsCapturing((hipStream_t)stream, &cs) != hipSuccess) return TQ_E_HIP;
            if (cs != hipStreamCaptureStatusNone) return TQ_E_CAPTURE;
        }
        for (size_t a = 0; a < segs_.size(); a += kMaxSegs) {
            SegList L{};
            L.count = (int32_t)std::min<size_t>(kMaxSegs, segs_.size() - a);
            int64_t most = 0;
            for (int i = 0; i < L.count; ++i) {
                L.s[i] = segs_[a + i];
                most = std::max(most, L.s[i].bytes);
            }
            const int64_t gx = (most + kChunk - 1) / kChunk;
            if (gx > 0x7fffffff) return TQ_E_SHAPE;
            void *args[] = {&L};
            const int32_t ls = tq_host::launch_kernel(reinterpret_cast<const void *>(&segment_copy_kernel),
                                                      dim3((uint32_t)gx, L.count), dim3(kThreads), args, 0,
                                                      (hipStream_t)stream, a == 0, a + (size_t)kMaxSegs >= segs_.size());
            if (ls != TQ_OK) return ls;
        }
        return TQ_OK;
    }

  private:
    std::vector<Seg> segs_;
    bool outside_ = false;
};

bool token_count_ok(int64_t t) { return t >= 0 && t <= ((int64_t)1 << 40); }

// checks for a call whose output holds no tokens: it touches no pointer
int32_t empty_output_ok(const tq_config *cfg, int32_t heads)
{
    if (cfg == nullptr) return TQ_E_NULL;
    if (!valid_head_dim(cfg->head_dim)) return TQ_E_HEAD_DIM;
    if (heads < 1 || heads > (1 << 20)) return TQ_E_SHAPE;
    return TQ_OK;
}

} // namespace

extern "C" {

int32_t tq_merge_rows(const tq_packed_kv *srcs, const int64_t *lens, int32_t n, int64_t width, int32_t heads,
                      const tq_config *cfg, const tq_packed_kv *dst, int64_t *left_pad, void *stream)
{
    const tq_host::TimingScope timing;
    if (n < 0 || !token_count_ok(width)) return TQ_E_SHAPE;
    if ((int64_t)n * width > ((int64_t)1 << 40)) return TQ_E_SHAPE;
    if (n > 0 && lens == nullptr) return TQ_E_NULL;
    for (int32_t i = 0; i < n; ++i)
        if (lens[i] < 0 || lens[i] > width) return TQ_E_SHAPE;
    if ((int64_t)n * width == 0) {
        int32_t st = empty_output_ok(cfg, heads);
        if (st == TQ_OK && left_pad != nullptr)
            for (int32_t i = 0; i < n; ++i) left_pad[i] = 0;
        return st;
    }
    int64_t tb[kPlanes];
    int32_t st = token_bytes(cfg, heads, dst, tb);
    if (st != TQ_OK) return st;
    if (srcs == nullptr) return TQ_E_NULL;
    for (int32_t i = 0; i < n; ++i)
        if (lens[i] > 0 && (st = check_src(&srcs[i], dst)) != TQ_OK) return st;
    Segments sg;
    for (int32_t i = 0; i < n; ++i) {
        const int64_t pad = width - lens[i];
        sg.add(nullptr, 0, 0, dst, i * width, (int64_t)n * width, pad, tb);
        sg.add(&srcs[i], 0, lens[i], dst, i * width + pad, (int64_t)n * width, lens[i], tb);
    }
    if ((st = sg.launch(stream)) != TQ_OK) return st;
    if (left_pad != nullptr)
        for (int32_t i = 0; i < n; ++i) left_pad[i] = width - lens[i];
    return TQ_OK;
}

int32_t tq_extend_rows(const tq_packed_kv *batch, int32_t b, int64_t width, const int64_t *left_pad_in,
                       const tq_packed_kv *row, int64_t row_len, int64_t new_width, int32_t heads,
                       const tq_config *cfg, const tq_packed_kv *dst, int64_t *left_pad_out, void *stream)
{
    const tq_host::TimingScope timing;
    if (b < 0 || !token_count_ok(width) || !token_count_ok(row_len) || !token_count_ok(new_width))
        return TQ_E_SHAPE;
    if (new_width < width || new_width < row_len) return TQ_E_SHAPE;
    if ((int64_t)(b + 1) * new_width > ((int64_t)1 << 40)) return TQ_E_SHAPE;
    if (left_pad_out != nullptr && b > 0 && left_pad_in == nullptr) return TQ_E_NULL;
    int32_t st = TQ_OK;
    int64_t tb[kPlanes];
    if (new_width == 0) {
        st = empty_output_ok(cfg, heads);
    } else {
        if ((st = token_bytes(cfg, heads, dst, tb)) != TQ_OK) return st;
        if (row_len > 0 && (st = check_src(row, dst)) != TQ_OK) return st;
        if (b > 0 && width > 0 && (st = check_src(batch, dst)) != TQ_OK) return st;
    }
    if (st != TQ_OK) return st;
    const int64_t shift = new_width - width;
    if (new_width > 0) {
        Segments sg;
        const int64_t out_tokens = (int64_t)(b + 1) * new_width, in_tokens = (int64_t)b * width;
        for (int32_t i = 0; i < b; ++i) {
            sg.add(nullptr, 0, 0, dst, i * new_width, out_tokens, shift, tb);
            sg.add(batch, i * width, in_tokens, dst, i * new_width + shift, out_tokens, width, tb);
        }
        sg.add(nullptr, 0, 0, dst, (int64_t)b * new_width, out_tokens, new_width - row_len, tb);
        sg.add(row, 0, row_len, dst, (int64_t)b * new_width + new_width - row_len, out_tokens, row_len, tb);
        if ((st = sg.launch(stream)) != TQ_OK) return st;
    }
    if (left_pad_out != nullptr) {
        for (int32_t i = 0; i < b; ++i) left_pad_out[i] = left_pad_in[i] + shift;
        left_pad_out[b] = new_width - row_len;
    }
    return TQ_OK;
}

int32_t tq_extract_row(const tq_packed_kv *batch, int32_t b, int64_t width, int32_t i, int64_t left_pad,
                       int32_t heads, const tq_config *cfg, const tq_packed_kv *dst, void *stream)
{
    const tq_host::TimingScope timing;
    if (b < 1 || i < 0 || i >= b || !token_count_ok(width) || left_pad < 0 || left_pad > width) return TQ_E_SHAPE;
    if ((int64_t)b * width > ((int64_t)1 << 40)) return TQ_E_SHAPE;
    if (width - left_pad == 0) return empty_output_ok(cfg, heads);
    int64_t tb[kPlanes];
    int32_t st = token_bytes(cfg, heads, dst, tb);
    if (st != TQ_OK) return st;
    if ((st = check_src(batch, dst)) != TQ_OK) return st;
    Segments sg;
    sg.add(batch, (int64_t)i * width + left_pad, (int64_t)b * width, dst, 0, width - left_pad, width - left_pad, tb);
    return sg.launch(stream);
}

int32_t tq_filter_rows(const tq_packed_kv *batch, int32_t b, int64_t width, const int32_t *keep, int32_t n,
                       int32_t heads, const tq_config *cfg, const tq_packed_kv *dst, void *stream)
{
    const tq_host::TimingScope timing;
    if (b < 0 || n < 0 || !token_count_ok(width)) return TQ_E_SHAPE;
    if ((int64_t)b * width > ((int64_t)1 << 40) || (int64_t)n * width > ((int64_t)1 << 40)) return TQ_E_SHAPE;
    if (n > 0 && keep == nullptr) return TQ_E_NULL;
    for (int32_t j = 0; j < n; ++j)
        if (keep[j] < 0 || keep[j] >= b) return TQ_E_SHAPE;
    if ((int64_t)n * width == 0) return empty_output_ok(cfg, heads);
    int64_t tb[kPlanes];
    int32_t st = token_bytes(cfg, heads, dst, tb);
    if (st != TQ_OK) return st;
    if ((st = check_src(batch, dst)) != TQ_OK) return st;
    Segments sg;
    for (int32_t j = 0; j < n; ++j)
        sg.add(batch, (int64_t)keep[j] * width, (int64_t)b * width, dst, (int64_t)j * width, (int64_t)n * width, width,
               tb);
    return sg.launch(stream);
}

} // extern "C"
