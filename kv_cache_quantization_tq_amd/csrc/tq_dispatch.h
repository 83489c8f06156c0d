// tq_dispatch.h -- kernel entry addresses for one head_dim, defined in
// tq_kernels_d<head_dim>.hip and launched by the C ABI in tq_api.hip.
// Each returns nullptr for an unsupported value width.
#pragma once

#include <stdint.h>

#define TQ_DECLARE_KERNELS(D)                                                \
    const void *tq_encode_kernel_d##D(int32_t v_bits, bool bf16_in);         \
    const void *tq_decode_kernel_d##D(int32_t v_bits, bool bf16_out);        \
    const void *tq_unrotate_kernel_d##D(bool bf16);

TQ_DECLARE_KERNELS(64)
TQ_DECLARE_KERNELS(128)
TQ_DECLARE_KERNELS(256)
TQ_DECLARE_KERNELS(512)

#undef TQ_DECLARE_KERNELS
