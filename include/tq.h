/*
 * tq.h -- C ABI of the TurboQuant KV-cache codec for AMD MI355X (gfx950).
 *
 * The codec is the one shown on the page "@mlx-bun/inference 0.0.0-stage ->
 * 1.0.0", package/src/kernels/turboquant/ops.ts, with the constant tables of
 * the page "mlx-bun 0.0.9 -> 0.0.11", src/mlx/turboquant-tables.ts:
 *
 *   values  (ops.ts encodeValues / decodeValues): multiply by the fixed +-1
 *           sign vector, normalised fast Walsh-Hadamard transform along
 *           head_dim, per-32-element RMS scale (stored fp16), divide by
 *           (scale + 1e-8), Lloyd-Max bin index = number of boundaries below
 *           the value, bit-packed. Decode: centroid * scale, inverse
 *           transform, sign multiply.
 *   keys    (ops.ts encodeKeys / decodeKeys): per-32-element min/max affine
 *           quantisation in binary32 with fp16 scale and zero point, round
 *           half to even, clip, bit-packed. Decode: (q + zero) * scale.
 *   packing (ops.ts packBits / bit-packing section): element i of a row
 *           occupies bits [i*bits, i*bits + bits) of the row's byte stream,
 *           least significant bit first; 8-bit codes are plain bytes.
 *
 * Data layout. K and V are row-major [tokens, heads, head_dim]; batches fold
 * into tokens. With R = tokens * heads and G = head_dim / 32 the codec
 * reads and writes five planes, each row-major and contiguous:
 *   k_codes [R, head_dim * k_bits / 8]  u8  (two's complement int8 codes when
 *                                            k_signed, otherwise unsigned)
 *   k_scale [R, G]  fp16 bits           k_zero [R, G]  fp16 bits
 *   v_codes [R, head_dim * v_bits / 8]  u8
 *   v_scale [R, G]  fp16 bits
 * Because groups never cross a row, appending at token t is a call on
 * pointers advanced by t * heads rows of each plane.
 *
 * A call with zero rows (tokens == 0) validates the configuration and
 * returns TQ_OK without touching any pointer.
 *
 * Ownership and execution. Every pointer except `cfg`, `out`/`in`
 * (host structs read during the call) is device memory owned by the caller.
 * The library allocates nothing and keeps no per-call state (beyond the
 * events tq_time_next_call arms for the calling thread). Calls enqueue
 * kernels on `stream` (a hipStream_t; NULL is the default stream) and return
 * without waiting. Argument errors are detected on the host before any
 * launch and leave every buffer untouched; a failed launch returns
 * TQ_E_HIP. Faults during execution surface at the caller's next
 * synchronisation.
 *
 * Alignment (TQ_E_ALIGN otherwise): K/V inputs and decoded outputs 16
 * bytes; code planes 16 bytes for 4- and 8-bit codes, 8 bytes for 2-, 3-
 * and 5-bit codes; fp16 planes 2 bytes.
 */
#ifndef TQ_H
#define TQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. The pages' operations throw on invalid arguments
 * (ops.ts packedDim, fwht, encodeKeys, encodeValues, packBits); here each
 * such case returns a code instead. */
enum {
    TQ_OK = 0,
    TQ_E_NULL = 1,     /* a required pointer is NULL                          */
    TQ_E_HEAD_DIM = 2, /* head_dim not in {64, 128, 256, 512}                 */
    TQ_E_BITS = 3,     /* bits not in {2,3,4,5,8}, or k_signed with k_bits!=8 */
    TQ_E_ALIGN = 4,    /* misaligned pointer, or dim * bits not a whole byte  */
    TQ_E_DTYPE = 5,    /* dtype not TQ_F32 / TQ_BF16                          */
    TQ_E_SHAPE = 6,    /* negative tokens, heads < 1, or row count overflow   */
    TQ_E_HIP = 7,      /* the HIP runtime reported an error at launch         */
    TQ_E_CAPTURE = 8,  /* a batching call needing more than one launch, or a  */
                       /* call with kernel timing armed, was made on a stream */
                       /* that is capturing a graph                           */
    TQ_E_SCRATCH = 9   /* the call needs more scratch than the library's      */
                       /* static buffer holds                                 */
};

/* Element types of K/V inputs and decoded outputs. */
enum { TQ_F32 = 0, TQ_BF16 = 1 };

/* Decode flags. */
enum {
    /* Return V still in the rotated domain, centroid * scale with no
     * inverse transform (ops.ts decodeValuesRotated: attention is linear
     * in V, so the caller may un-rotate the attention output instead). */
    TQ_DECODE_ROTATED_V = 1
};

/* Codec configuration (ops.ts: head_dim, key bits and signedness, value
 * bits). k_signed is only valid with k_bits == 8 (ops.ts encodeKeys doc). */
typedef struct tq_config {
    int32_t head_dim; /* 64, 128, 256 or 512                     */
    int32_t k_bits;   /* 2, 3, 4, 5 or 8                          */
    int32_t v_bits;   /* 2, 3, 4, 5 or 8 (Lloyd-Max table widths) */
    int32_t k_signed; /* 0 or 1                                   */
} tq_config;

/* The five device planes (layout above). Members for a side that is not
 * encoded or decoded may be NULL. */
typedef struct tq_packed_kv {
    void *k_codes;
    void *k_scale;
    void *k_zero;
    void *v_codes;
    void *v_scale;
} tq_packed_kv;

/* ops.ts packedDim: bytes per row for `dim` elements of `bits` each, i.e.
 * dim * bits / 8. Returns -TQ_E_ALIGN when dim * bits is not a multiple of
 * 8 and -TQ_E_BITS when bits is outside 1..8 or dim < 1. Host only. */
int64_t tq_packed_dim(int32_t dim, int32_t bits);

/* Static, NUL-terminated message for a status code (never NULL). */
const char *tq_status_string(int32_t status);

/* Kernel timing, for callers that measure the kernels (benchmarks): not an
 * operation of the pages. Arms the calling host thread so that the next
 * call of this library that takes a `stream` binds `stop` to the end of the
 * last kernel it launches and, if `start` is not NULL, `start` to the
 * start of the first one (hipExtLaunchKernel's stop and start events).
 * hipEventElapsedTime(e, stop) from an event e on the same stream then
 * ends exactly at the call's last kernel; a stop event alone adds nothing
 * to the launch, while a start event makes the HIP runtime enqueue a marker
 * ahead of the first kernel (measured: launches a few microseconds further
 * apart). `start` and `stop` are hipEvent_t handles created and owned by
 * the caller (timing enabled); both NULL disarms. The next such call
 * disarms whatever it returns; if it launches nothing, the events are left
 * as they were. With timing armed, a call on a stream that is capturing a
 * graph returns TQ_E_CAPTURE before launching anything. Returns TQ_E_NULL
 * when `start` is given without `stop`. Host only: records nothing by
 * itself. */
int32_t tq_time_next_call(void *start, void *stop);

/* Encode K and V [tokens, heads, head_dim] of dtype `in_dtype` into the
 * planes of `out` (ops.ts encodeKeys + packBits for K, encodeValues +
 * packBits for V). Either `k` or `v` may be NULL to encode one side only;
 * the planes of the other side are then not touched. tokens == 0 is a
 * no-op. One launch covers both sides. */
int32_t tq_encode_kv(const void *k, const void *v, int32_t in_dtype,
                     int64_t tokens, int32_t heads, const tq_config *cfg,
                     const tq_packed_kv *out, void *stream);

/* Decode the planes of `in` back to K and V [tokens, heads, head_dim] of
 * dtype `out_dtype` (ops.ts unpackBits + decodeKeys, unpackBits +
 * decodeValues; TQ_BF16 is the pages' output dtype, TQ_F32 returns the
 * binary32 value before that rounding). Either output may be NULL to skip
 * that side. `flags` is 0 or TQ_DECODE_ROTATED_V. One launch decodes K and
 * V of the same rows together (ops.ts tryDecodePackedKv). */
int32_t tq_decode_kv(const tq_packed_kv *in, int64_t tokens, int32_t heads,
                     const tq_config *cfg, void *k_out, void *v_out,
                     int32_t out_dtype, int32_t flags, void *stream);

/* ops.ts unrotateValues: apply the inverse rotation (normalised transform,
 * then sign multiply) in binary32 to `rows` rows of `head_dim` elements
 * and write them back in `dtype`. x and out may alias. */
int32_t tq_unrotate_values(const void *x, void *out, int32_t dtype, int64_t rows,
                           int32_t head_dim, void *stream);

/* Host copies of the constant tables the kernels use, for callers that
 * fuse decoding into their own kernels (turboquant-tables.ts LLOYD_MAX and
 * SIGN_VECTORS). centroids receives 2^bits floats, boundaries 2^bits - 1;
 * signs receives head_dim floats of +-1. Host only. */
int32_t tq_lloyd_max_table(int32_t bits, float *centroids, float *boundaries);
int32_t tq_sign_vector(int32_t head_dim, float *signs);

/* Host evaluation of the quotient the kernels use for key scales, zero
 * points and key codes, compiled from the same source: q[i] = a[i] / b[i]
 * from r = RN(1/b[i]) by one refinement step (q0 = a r, e = fma(-q0, b, a),
 * q = fma(e, r, q0)), the sign of a zero result taken from a[i]. For b[i] > 0
 * it equals the IEEE quotient wherever the kernels take it (|a r| < 1e30,
 * b < 1e30; outside that they divide). For checking the quotient on the
 * CPU. Host only. */
int32_t tq_quotient_host(const float *a, const float *b, int64_t n, float *q);

/* Host evaluation of the value bin search exactly as the kernels run it
 * (same code, compiled for the host: the table-driven search of the fast
 * path for |z| <= 6, the clamped general search otherwise): idx[i] = number
 * of Lloyd-Max boundaries strictly below z[i] (ops.ts searchsorted). For
 * checking the search on the CPU. Host only. */
int32_t tq_value_bin_host(int32_t bits, const float *z, int64_t n, uint8_t *idx);

/* ---------------------------------------------------------------------
 * Token-axis batching of packed caches (page "mlx-bun 0.0.9 -> 0.0.11",
 * src/model/batched-quant.ts: mergeQuantRows, extendQuantRows,
 * extractQuantRow, filterQuantRows). Codec groups run along head_dim only,
 * so moving whole tokens is byte-exact: a sequence's bytes come out exactly
 * as they were encoded.
 *
 * A batch of b sequences of width W is a plane set of b * W tokens (each
 * token `heads` rows of every plane), sequence-major: sequence s occupies
 * tokens [s * W, (s + 1) * W). Sequences are left-padded: a sequence of L
 * tokens sits in the last L token slots of its W and the W - L slots before
 * it hold zero bytes in every plane (they decode to zeros; callers mask
 * them out of attention). left_pad[s] = W - L.
 *
 * The planes handled are the members of `dst` that are not NULL (keys only,
 * values only, or all five); every source must have those planes. `cfg`
 * gives the row sizes (head_dim, k_bits, v_bits; k_signed as for the
 * codec). Source and destination must not overlap. Any alignment is
 * accepted. Arrays named lens / left_pad* / keep are host memory; planes
 * are device memory; `srcs`, `batch`, `row`, `dst` are host structs. A
 * call whose output holds no tokens touches no plane pointer; planes of a
 * source that contributes no tokens may be NULL. Errors (TQ_E_*) are
 * returned before any launch and leave dst untouched.
 *
 * Each launch carries up to 120 plane segments (source, destination,
 * bytes) as a kernel argument; a call needs one segment per plane and
 * per contiguous run of tokens. Graph capture: a call that fits in one
 * launch may be captured (checked by replaying such graphs); a call that
 * needs more than one launch returns TQ_E_CAPTURE, before launching
 * anything, when `stream` is capturing, because the replay of a graph of
 * such calls (32 merged caches, three launches per call) faulted on
 * MI355X with no cause established in this library's code. Launch those
 * calls directly.
 * --------------------------------------------------------------------- */

/* mergeQuantRows: stack n caches (srcs[i] holds lens[i] tokens) into dst,
 * a batch of n sequences of width `width` >= max(lens) (the page uses the
 * maximum; a larger width pads every sequence further). Writes
 * left_pad[i] = width - lens[i] when left_pad is not NULL. */
int32_t tq_merge_rows(const tq_packed_kv *srcs, const int64_t *lens, int32_t n, int64_t width, int32_t heads,
                      const tq_config *cfg, const tq_packed_kv *dst, int64_t *left_pad, void *stream);

/* extendQuantRows: append one cache `row` of row_len tokens to `batch`
 * (b sequences of width `width`, left pads left_pad_in) as sequence b of
 * dst, a batch of b + 1 sequences of width new_width >= max(width,
 * row_len). Existing pads grow by new_width - width; the new sequence's pad
 * is new_width - row_len (written to left_pad_out when it is not NULL;
 * left_pad_in is then required if b > 0). b may be 0 (batch unused). */
int32_t tq_extend_rows(const tq_packed_kv *batch, int32_t b, int64_t width, const int64_t *left_pad_in,
                       const tq_packed_kv *row, int64_t row_len, int64_t new_width, int32_t heads,
                       const tq_config *cfg, const tq_packed_kv *dst, int64_t *left_pad_out, void *stream);

/* extractQuantRow: copy sequence i of `batch` (b sequences of width
 * `width`) past its left pad into dst, a cache of width - left_pad tokens. */
int32_t tq_extract_row(const tq_packed_kv *batch, int32_t b, int64_t width, int32_t i, int64_t left_pad,
                       int32_t heads, const tq_config *cfg, const tq_packed_kv *dst, void *stream);

/* filterQuantRows: dst sequence j = batch sequence keep[j] (0 <= keep[j] <
 * b), j < n; widths unchanged. The page keeps sorted indices; any valid
 * indices are accepted here. */
int32_t tq_filter_rows(const tq_packed_kv *batch, int32_t b, int64_t width, const int32_t *keep, int32_t n,
                       int32_t heads, const tq_config *cfg, const tq_packed_kv *dst, void *stream);

/* ---------------------------------------------------------------------
 * Attention of one query token per sequence over a packed cache (page
 * "@mlx-bun/inference 0.0.0-stage -> 1.0.0", ops.ts decodeValuesRotated and
 * unrotateValues: attention is linear in V, so it may run on values still
 * in the rotated domain and un-rotate its output once per query row).
 * Keys are decoded as decodeKeys does (bf16), values as
 * decodeValuesRotated does (bf16); both inside the kernel, so the cache is
 * read packed. With valid tokens t of sequence b and query head h reading
 * KV head h / (q_heads / kv_heads):
 *   s_t = scale * <q[b,h], K_t>,  p = softmax(s),  o_rot = sum_t p_t Vrot_t,
 *   out[b,h] = unrotate(o_rot)   (normalised transform, then sign vector)
 * in binary32 after decoding: the two contractions run on the matrix cores
 * with binary32 accumulation, a binary32 query and the softmax weights
 * entering as sums of three bf16 terms. A sequence with no valid token
 * gives zeros.
 * --------------------------------------------------------------------- */

/* Bytes of device workspace tq_attention_decode needs (host only; <0 on
 * invalid arguments). */
int64_t tq_attention_workspace_bytes(int32_t batch, int32_t kv_heads, int32_t q_heads, int32_t head_dim,
                                     int64_t width);

/* q: [batch, q_heads, head_dim] of q_dtype (16-byte aligned). cache: a
 * batch of `batch` sequences of width `width` in the layout of the batching
 * operations above (all five planes, codes aligned as for tq_decode_kv,
 * scale and zero planes 8-byte aligned);
 * left_pad: device int32 [batch] (tokens [left_pad[b], width) of sequence
 * b are attended) or NULL for none. q_heads / kv_heads must be 1, 2, 4 or
 * 8. out: [batch, q_heads, head_dim] of out_dtype (16-byte aligned).
 * workspace: caller-owned device memory of tq_attention_workspace_bytes()
 * (16-byte aligned; may be NULL when width is 0; its size covers every
 * split count the call may choose); calls sharing a workspace must not
 * overlap. Two launches on `stream` (one when width is 0). */
int32_t tq_attention_decode(const void *q, int32_t q_dtype, const tq_packed_kv *cache, int32_t batch, int64_t width,
                            const int32_t *left_pad, int32_t kv_heads, int32_t q_heads, const tq_config *cfg,
                            float scale, void *out, int32_t out_dtype, void *workspace, int64_t workspace_bytes,
                            void *stream);

/* tq_attention_decode without a workspace argument, for callers that
 * cannot allocate device memory (code under graph capture, serving loops
 * that forbid allocation). The split partials go to a static buffer of 64
 * MiB in the library's device image, one per GPU, held until the process
 * ends; this call allocates nothing. Arguments, results and errors are
 * those of tq_attention_decode, plus TQ_E_SCRATCH (returned before any
 * launch) when tq_attention_workspace_bytes() for the call exceeds 64 MiB.
 * All calls on one GPU share its buffer and each call leaves its partials
 * there: calls that may overlap on one GPU (concurrent streams, or host
 * threads) race and must be ordered by the caller. The first call on a
 * device with width > 0 looks up the buffer's device address (a runtime
 * query, not an allocation); callers that capture graphs make that first
 * call outside the capture. */
int32_t tq_attention_decode_static(const void *q, int32_t q_dtype, const tq_packed_kv *cache, int32_t batch,
                                   int64_t width, const int32_t *left_pad, int32_t kv_heads, int32_t q_heads,
                                   const tq_config *cfg, float scale, void *out, int32_t out_dtype, void *stream);

/* ---------------------------------------------------------------------
 * Lloyd-Max table fitting (page "mlx-bun 0.0.9 -> 0.0.11",
 * src/mlx/turboquant-tables.ts, header of LLOYD_MAX: the tables are an
 * iterative Lloyd-Max fit to unit-normal samples, 500 iterations).
 * --------------------------------------------------------------------- */

/* Bytes of device workspace tq_lloyd_max_fit needs for n samples (host
 * only; 16 * n plus about 1 KB per 4096 samples). Returns -TQ_E_SHAPE
 * when n is outside 1 .. 2^31 - 1. */
int64_t tq_lloyd_max_workspace_bytes(int64_t n);

/* Fit `levels` (2..256) reconstruction levels to n (1 .. 2^31 - 1)
 * samples (device float32, finite, 4-byte aligned) by `iterations` Lloyd
 * iterations starting from init (host, `levels` strictly ascending
 * binary64 values).
 * One iteration: boundaries b_j = (c_j + c_{j+1}) / 2; each sample goes to
 * level k = #{j : b_j < x} (ties to the lower level, the codec's bin
 * rule); c_k = mean of its samples (a level with none keeps its value).
 * Samples are summed as exact integers rint(x * 2^s) with s = min(40, 62 -
 * bitlen(n) - e), |x| < 2^e for every sample, so the result does not depend
 * on summation order: c_k = double(sum_k) * 2^-s / count_k. The samples
 * are sorted once in the workspace, so an iteration costs a search per
 * boundary rather than a pass over the samples.
 * Writes the final centroids (levels) and boundaries (levels - 1, if not
 * NULL) to host memory and waits for the stream before returning.
 * `workspace` is caller-owned device memory of at least
 * tq_lloyd_max_workspace_bytes(n), 8-byte aligned; calls sharing a
 * workspace must not overlap. Returns TQ_E_SHAPE if a sample is not finite
 * or magnitudes are too large for the integer sums (s < 0). */
int32_t tq_lloyd_max_fit(const float *samples, int64_t n, int32_t levels, const double *init, int32_t iterations,
                         double *centroids, double *boundaries, void *workspace, int64_t workspace_bytes,
                         void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
