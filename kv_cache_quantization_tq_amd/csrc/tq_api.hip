// tq_api.hip -- host side of the TurboQuant KV-cache codec: the codec part of
// the C ABI declared in include/tq.h (argument validation, grid sizing,
// launches) and the host copies of the tables. The kernels live in
// tq_kernels_d<head_dim>.hip; the token-axis batching operations in
// tq_batch.hip.
#include <hip/hip_runtime.h>

#include <stdlib.h>

#include <mutex>

#include "tq.h"
#include "tq_device.h"
#include "tq_dispatch.h"
#include "tq_host.h"

namespace {

using tq_host::aligned;
using tq_host::check_rows;
using tq_host::code_align;
using tq_host::valid_bits;
using tq_host::valid_head_dim;
using tq_host::valid_key_cfg;

// One wavefront per tile: a block for every four tiles, which the hardware
// dispatches as earlier blocks retire. Measured faster than a persistent grid
// (one round of resident blocks walking the tiles with a stride) on every
// codec workload, most on the large decodes (long-context cache 286 -> 239 us,
// large-head joint decode 1218 -> 1050 us), whose HBM streams run closer to
// the device's rate when the tiles in flight are the ones dispatched last.
// The kernels keep their stride loop, so a grid capped below the tile count
// still covers every tile: the cap is the largest grid the launch accepts, or
// TQ_BLOCKS_PER_CU blocks per compute unit when that is set (tuning sweeps).
int64_t grid_for(int64_t rows, int32_t d)
{
    static std::mutex mu;
    static int cus[64] = {0};
    static int env_per_cu = -1;
    int64_t cap = 0x7fffffff;
    {
        std::lock_guard<std::mutex> lock(mu);
        if (env_per_cu < 0) {
            const char *e = getenv("TQ_BLOCKS_PER_CU");
            env_per_cu = (e != nullptr && atoi(e) > 0) ? atoi(e) : 0;
        }
        if (env_per_cu > 0) {
            int dev = 0;
            if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
            if (cus[dev] == 0) {
                int n = 0;
                if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
                    n = 256;
                cus[dev] = n;
            }
            cap = (int64_t)env_per_cu * cus[dev];
        }
    }
    const int64_t rpw = kWave / (d / kGroup);
    const int64_t tiles = (rows + rpw - 1) / rpw;
    int64_t blocks = (tiles + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > cap) blocks = cap;
    return blocks < 1 ? 1 : blocks;
}

int32_t key_mode(const tq_config *cfg) { return cfg->k_bits | (cfg->k_signed ? 16 : 0); }

const void *encode_kernel_for(int32_t d, int32_t vb, bool bf16)
{
    switch (d) {
    case 64: return tq_encode_kernel_d64(vb, bf16);
    case 128: return tq_encode_kernel_d128(vb, bf16);
    case 256: return tq_encode_kernel_d256(vb, bf16);
    case 512: return tq_encode_kernel_d512(vb, bf16);
    default: return nullptr;
    }
}

const void *decode_kernel_for(int32_t d, int32_t vb, bool bf16)
{
    switch (d) {
    case 64: return tq_decode_kernel_d64(vb, bf16);
    case 128: return tq_decode_kernel_d128(vb, bf16);
    case 256: return tq_decode_kernel_d256(vb, bf16);
    case 512: return tq_decode_kernel_d512(vb, bf16);
    default: return nullptr;
    }
}

const void *unrotate_kernel_for(int32_t d, bool bf16)
{
    switch (d) {
    case 64: return tq_unrotate_kernel_d64(bf16);
    case 128: return tq_unrotate_kernel_d128(bf16);
    case 256: return tq_unrotate_kernel_d256(bf16);
    case 512: return tq_unrotate_kernel_d512(bf16);
    default: return nullptr;
    }
}

// launch `fn` with its argument array on the grid for `rows` (the codec's
// calls launch one kernel each)
int32_t launch(const void *fn, int64_t rows, int32_t d, void **args, void *stream)
{
    if (fn == nullptr) return TQ_E_BITS;
    const dim3 grid((uint32_t)grid_for(rows, d));
    return tq_host::launch_kernel(fn, grid, dim3(kBlockThreads), args, 0, (hipStream_t)stream, true, true);
}

thread_local tq_host::Timing t_timing;


} // namespace

tq_host::Timing &tq_host::armed_timing() { return t_timing; }

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

int64_t tq_packed_dim(int32_t dim, int32_t bits)
{
    if (dim < 1 || bits < 1 || bits > 8) return -TQ_E_BITS;
    if (((int64_t)dim * bits) % 8 != 0) return -TQ_E_ALIGN;
    return ((int64_t)dim * bits) / 8;
}

const char *tq_status_string(int32_t status)
{
    switch (status) {
    case TQ_OK: return "ok";
    case TQ_E_NULL: return "a required pointer is NULL";
    case TQ_E_HEAD_DIM: return "head_dim must be 64, 128, 256 or 512";
    case TQ_E_BITS: return "bits must be 2, 3, 4, 5 or 8 (signed keys: 8 only)";
    case TQ_E_ALIGN: return "misaligned pointer or dim*bits not a whole number of bytes";
    case TQ_E_DTYPE: return "dtype must be TQ_F32 or TQ_BF16";
    case TQ_E_SHAPE: return "tokens must be >= 0 and heads >= 1 (row count within range)";
    case TQ_E_HIP: return "HIP runtime error at kernel launch";
    case TQ_E_CAPTURE: return "the stream is capturing a graph (a batching call needing more than one launch, or "
                              "kernel timing armed)";
    case TQ_E_SCRATCH: return "the call needs more scratch than the library's static buffer (64 MiB) holds";
    default: return "unknown status";
    }
}

int32_t tq_encode_kv(const void *k, const void *v, int32_t in_dtype, int64_t tokens, int32_t heads,
                     const tq_config *cfg, const tq_packed_kv *out, void *stream)
{
    const tq_host::TimingScope timing;
    if (cfg == nullptr || out == nullptr) return TQ_E_NULL;
    if (!valid_head_dim(cfg->head_dim)) return TQ_E_HEAD_DIM;
    if (in_dtype != TQ_F32 && in_dtype != TQ_BF16) return TQ_E_DTYPE;
    int64_t rows = 0;
    const int32_t st = check_rows(tokens, heads, &rows);
    if (st != TQ_OK) return st;
    if (rows == 0) return TQ_OK;
    if (k == nullptr && v == nullptr) return TQ_E_NULL;
    if (k != nullptr) {
        if (!valid_key_cfg(cfg)) return TQ_E_BITS;
        if (out->k_codes == nullptr || out->k_scale == nullptr || out->k_zero == nullptr) return TQ_E_NULL;
        if (!aligned(k, 16) || !aligned(out->k_codes, code_align(cfg->k_bits)) || !aligned(out->k_scale, 2) ||
            !aligned(out->k_zero, 2))
            return TQ_E_ALIGN;
    }
    if (v != nullptr) {
        if (!valid_bits(cfg->v_bits)) return TQ_E_BITS;
        if (out->v_codes == nullptr || out->v_scale == nullptr) return TQ_E_NULL;
        if (!aligned(v, 16) || !aligned(out->v_codes, code_align(cfg->v_bits)) || !aligned(out->v_scale, 2))
            return TQ_E_ALIGN;
    }
    const int32_t vb = (v != nullptr) ? cfg->v_bits : 4;
    const void *fn = encode_kernel_for(cfg->head_dim, vb, in_dtype == TQ_BF16);
    int32_t kmode = (k != nullptr) ? key_mode(cfg) : KMODE_NONE;
    const void *kin = k, *vin = v;
    uint8_t *kc = (uint8_t *)out->k_codes, *vc = (uint8_t *)out->v_codes;
    uint16_t *ks = (uint16_t *)out->k_scale, *kz = (uint16_t *)out->k_zero, *vs = (uint16_t *)out->v_scale;
    void *args[] = {&kin, &vin, &rows, &kmode, &kc, &ks, &kz, &vc, &vs};
    return launch(fn, rows, cfg->head_dim, args, stream);
}

int32_t tq_decode_kv(const tq_packed_kv *in, int64_t tokens, int32_t heads, const tq_config *cfg, void *k_out,
                     void *v_out, int32_t out_dtype, int32_t flags, void *stream)
{
    const tq_host::TimingScope timing;
    if (cfg == nullptr || in == nullptr) return TQ_E_NULL;
    if (!valid_head_dim(cfg->head_dim)) return TQ_E_HEAD_DIM;
    if (out_dtype != TQ_F32 && out_dtype != TQ_BF16) return TQ_E_DTYPE;
    if ((flags & ~TQ_DECODE_ROTATED_V) != 0) return TQ_E_SHAPE;
    int64_t rows = 0;
    const int32_t st = check_rows(tokens, heads, &rows);
    if (st != TQ_OK) return st;
    if (rows == 0) return TQ_OK;
    if (k_out == nullptr && v_out == nullptr) return TQ_E_NULL;
    if (k_out != nullptr) {
        if (!valid_key_cfg(cfg)) return TQ_E_BITS;
        if (in->k_codes == nullptr || in->k_scale == nullptr || in->k_zero == nullptr) return TQ_E_NULL;
        if (!aligned(k_out, 16) || !aligned(in->k_codes, code_align(cfg->k_bits)) || !aligned(in->k_scale, 2) ||
            !aligned(in->k_zero, 2))
            return TQ_E_ALIGN;
    }
    if (v_out != nullptr) {
        if (!valid_bits(cfg->v_bits)) return TQ_E_BITS;
        if (in->v_codes == nullptr || in->v_scale == nullptr) return TQ_E_NULL;
        if (!aligned(v_out, 16) || !aligned(in->v_codes, code_align(cfg->v_bits)) || !aligned(in->v_scale, 2))
            return TQ_E_ALIGN;
    }
    const int32_t vb = (v_out != nullptr) ? cfg->v_bits : 4;
    const void *fn = decode_kernel_for(cfg->head_dim, vb, out_dtype == TQ_BF16);
    int32_t kmode = (k_out != nullptr) ? key_mode(cfg) : KMODE_NONE;
    int32_t rotated = (flags & TQ_DECODE_ROTATED_V) != 0;
    const uint8_t *kc = (const uint8_t *)in->k_codes, *vc = (const uint8_t *)in->v_codes;
    const uint16_t *ks = (const uint16_t *)in->k_scale, *kz = (const uint16_t *)in->k_zero;
    const uint16_t *vs = (const uint16_t *)in->v_scale;
    void *args[] = {&kc, &ks, &kz, &vc, &vs, &rows, &kmode, &rotated, &k_out, &v_out};
    return launch(fn, rows, cfg->head_dim, args, stream);
}

int32_t tq_unrotate_values(const void *x, void *out, int32_t dtype, int64_t rows, int32_t head_dim, void *stream)
{
    const tq_host::TimingScope timing;
    if (!valid_head_dim(head_dim)) return TQ_E_HEAD_DIM;
    if (dtype != TQ_F32 && dtype != TQ_BF16) return TQ_E_DTYPE;
    if (rows < 0 || rows > ((int64_t)1 << 44)) return TQ_E_SHAPE;
    if (rows == 0) return TQ_OK;
    if (x == nullptr || out == nullptr) return TQ_E_NULL;
    if (!aligned(x, 16) || !aligned(out, 16)) return TQ_E_ALIGN;
    const void *fn = unrotate_kernel_for(head_dim, dtype == TQ_BF16);
    void *args[] = {&x, &out, &rows};
    return launch(fn, rows, head_dim, args, stream);
}

int32_t tq_time_next_call(void *start, void *stop)
{
    if (start != nullptr && stop == nullptr) return TQ_E_NULL;
    t_timing.start = static_cast<hipEvent_t>(start);
    t_timing.stop = static_cast<hipEvent_t>(stop);
    return TQ_OK;
}

int32_t tq_lloyd_max_table(int32_t bits, float *centroids, float *boundaries)
{
    if (!valid_bits(bits)) return TQ_E_BITS;
    const float *c = nullptr, *b = nullptr;
    switch (bits) {
    case 2: c = LM<2>::c; b = LM<2>::b; break;
    case 3: c = LM<3>::c; b = LM<3>::b; break;
    case 4: c = LM<4>::c; b = LM<4>::b; break;
    case 5: c = LM<5>::c; b = LM<5>::b; break;
    default: c = LM<8>::c; b = LM<8>::b; break;
    }
    const int n = 1 << bits;
    if (centroids != nullptr)
        for (int i = 0; i < n; ++i) centroids[i] = c[i];
    if (boundaries != nullptr)
        for (int i = 0; i < n - 1; ++i) boundaries[i] = b[i];
    return TQ_OK;
}

int32_t tq_sign_vector(int32_t head_dim, float *signs)
{
    if (!valid_head_dim(head_dim)) return TQ_E_HEAD_DIM;
    if (signs == nullptr) return TQ_E_NULL;
    const uint32_t *m = head_dim == 64 ? kSignMask64 : head_dim == 128 ? kSignMask128
                      : head_dim == 256 ? kSignMask256 : kSignMask512;
    for (int i = 0; i < head_dim; ++i) signs[i] = ((m[i / 32] >> (i % 32)) & 1u) ? -1.0f : 1.0f;
    return TQ_OK;
}

int32_t tq_quotient_host(const float *a, const float *b, int64_t n, float *q)
{
    if (n < 0) return TQ_E_SHAPE;
    if (n > 0 && (a == nullptr || b == nullptr || q == nullptr)) return TQ_E_NULL;
    for (int64_t i = 0; i < n; ++i) q[i] = quot_signed(a[i], b[i], 1.0f / b[i]);
    return TQ_OK;
}

int32_t tq_value_bin_host(int32_t bits, const float *z, int64_t n, uint8_t *idx)
{
    if (!valid_bits(bits)) return TQ_E_BITS;
    if (n < 0) return TQ_E_SHAPE;
    if (n > 0 && (z == nullptr || idx == nullptr)) return TQ_E_NULL;
    static constexpr BinLut<2> l2{};
    static constexpr BinLut<3> l3{};
    static constexpr BinLut<4> l4{};
    static constexpr BinLut<5> l5{};
    static constexpr BinLut<8> l8{};
    for (int64_t i = 0; i < n; ++i) {
        // the kernels' fast path for |z| <= 6, the general path otherwise
        const bool bounded = fabsf(z[i]) <= 6.0f;
        uint32_t r = 0;
        switch (bits) {
        case 2: r = bounded ? bin_index_bounded<2>(z[i], l2.cell) : bin_index_any<2>(z[i], l2.cell); break;
        case 3: r = bounded ? bin_index_bounded<3>(z[i], l3.cell) : bin_index_any<3>(z[i], l3.cell); break;
        case 4: r = bounded ? bin_index_bounded<4>(z[i], l4.cell) : bin_index_any<4>(z[i], l4.cell); break;
        case 5: r = bounded ? bin_index_bounded<5>(z[i], l5.cell) : bin_index_any<5>(z[i], l5.cell); break;
        default: r = bounded ? bin_index_bounded<8>(z[i], l8.cell) : bin_index_any<8>(z[i], l8.cell); break;
        }
        idx[i] = (uint8_t)r;
    }
    return TQ_OK;
}

} // extern "C"
