// tq_host.h -- host-side argument checks shared by the C ABI translation
// units (tq_api.hip, tq_batch.hip).
#ifndef TQ_HOST_H
#define TQ_HOST_H

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

} // namespace tq_host

#endif
