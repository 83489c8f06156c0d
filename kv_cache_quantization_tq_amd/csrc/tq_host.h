// tq_host.h -- host-side argument checks and the kernel launch shared by the
// C ABI translation units (tq_api.hip, tq_attn.hip, tq_batch.hip, tq_fit.hip).
#ifndef TQ_HOST_H
#define TQ_HOST_H

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "tq.h"

namespace tq_host {

inline bool valid_head_dim(int32_t d) { return d == 64 || d == 128 || d == 256 || d == 512; }
inline bool valid_bits(int32_t b) { return b == 2 || b == 3 || b == 4 || b == 5 || b == 8; }
inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline uintptr_t code_align(int32_t bits) { return (bits == 4 || bits == 8) ? 16 : 8; }

// key side settings: bits in the table widths, signed only with 8 bits
inline bool valid_key_cfg(const tq_config *cfg)
{
    return valid_bits(cfg->k_bits) && (cfg->k_signed == 0 || cfg->k_signed == 1) &&
           (cfg->k_signed == 0 || cfg->k_bits == 8);
}

inline int32_t check_rows(int64_t tokens, int32_t heads, int64_t *rows)
{
    if (tokens < 0 || heads < 1) return TQ_E_SHAPE;
    if (tokens > (int64_t)1 << 40 || heads > (1 << 20)) return TQ_E_SHAPE;
    *rows = tokens * heads;
    return TQ_OK;
}

// Kernel timing armed by tq_time_next_call on the calling host thread; the
// storage lives in tq_api.hip.
struct Timing {
    hipEvent_t start = nullptr, stop = nullptr;
};
Timing &armed_timing();

// Disarms the timing when an entry point returns, whatever it returns.
struct TimingScope {
    TimingScope() = default;
    TimingScope(const TimingScope &) = delete;
    TimingScope &operator=(const TimingScope &) = delete;
    ~TimingScope() { armed_timing() = Timing{}; }
};

// Launches fn. With timing armed, the start event is bound to this dispatch's
// start when `first` and the stop event to its end when `last`
// (hipExtLaunchKernel takes both from the dispatch's own timestamps). With
// any event armed, a capturing stream is refused with TQ_E_CAPTURE at the
// entry point's first launch (a `first` one), before anything launches.
inline int32_t launch_kernel(const void *fn, dim3 grid, dim3 block, void **args, size_t lds, hipStream_t s,
                             bool first, bool last)
{
    const Timing &t = armed_timing();
    if (first && (t.start != nullptr || t.stop != nullptr)) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) != hipSuccess) return TQ_E_HIP;
        if (cs != hipStreamCaptureStatusNone) return TQ_E_CAPTURE;
    }
    hipEvent_t a = first ? t.start : nullptr, b = last ? t.stop : nullptr;
    const hipError_t e = (a == nullptr && b == nullptr) ? hipLaunchKernel(fn, grid, block, args, lds, s)
                                                        : hipExtLaunchKernel(fn, grid, block, args, lds, s, a, b, 0);
    if (e != hipSuccess) return TQ_E_HIP;
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_E_HIP;
}

} // namespace tq_host

#endif
