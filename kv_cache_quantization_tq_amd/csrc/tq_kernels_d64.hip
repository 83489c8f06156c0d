// tq_kernels_d64.hip -- codec kernels for head_dim 64 (one translation unit per
// head_dim so the kernels compile in parallel).
#include "tq_device.h"
#include "tq_dispatch.h"

namespace {
template <bool BF> const void *encode_for(int32_t vb)
{
    switch (vb) {
    case 2: return reinterpret_cast<const void *>(&encode_kernel<64, 2, BF>);
    case 3: return reinterpret_cast<const void *>(&encode_kernel<64, 3, BF>);
    case 4: return reinterpret_cast<const void *>(&encode_kernel<64, 4, BF>);
    case 5: return reinterpret_cast<const void *>(&encode_kernel<64, 5, BF>);
    case 8: return reinterpret_cast<const void *>(&encode_kernel<64, 8, BF>);
    default: return nullptr;
    }
}
template <bool BF> const void *decode_for(int32_t vb)
{
    switch (vb) {
    case 2: return reinterpret_cast<const void *>(&decode_kernel<64, 2, BF>);
    case 3: return reinterpret_cast<const void *>(&decode_kernel<64, 3, BF>);
    case 4: return reinterpret_cast<const void *>(&decode_kernel<64, 4, BF>);
    case 5: return reinterpret_cast<const void *>(&decode_kernel<64, 5, BF>);
    case 8: return reinterpret_cast<const void *>(&decode_kernel<64, 8, BF>);
    default: return nullptr;
    }
}
} // namespace

const void *tq_encode_kernel_d64(int32_t v_bits, bool bf16_in)
{
    return bf16_in ? encode_for<true>(v_bits) : encode_for<false>(v_bits);
}

const void *tq_decode_kernel_d64(int32_t v_bits, bool bf16_out)
{
    return bf16_out ? decode_for<true>(v_bits) : decode_for<false>(v_bits);
}

const void *tq_unrotate_kernel_d64(bool bf16)
{
    return bf16 ? reinterpret_cast<const void *>(&unrotate_kernel<64, true>)
                : reinterpret_cast<const void *>(&unrotate_kernel<64, false>);
}
