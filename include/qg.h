/*
 * qg.h -- C ABI of libqg: dequantize-fused low-bit weight matrix-vector
 * product (batch-1 LLM decode), its small-batch and prefill matrix-matrix
 * form, a fused greedy (argmax) output head, and the embedding-row gather
 * from the same 4-bit matrix, for AMD MI355X (gfx950).
 *
 * Notation. W is M x K (M outputs, K inputs). Activations x are float32
 * [rows][K], outputs y are float32 [rows][M]; every array is row-major and
 * contiguous. For every output,
 *
 *     y[n][m] = sum over k of w[m][k] * x[n][k]
 *
 * where w[m][k] is the real weight decoded from the packed format below,
 * and the sum is carried in float32 (any order; the result is within
 * 1e-5 * sum_k |w[m][k] * x[n][k]| of the exact value).
 *
 * Weight formats
 *
 *   QG_I8_ROW   codes  int8  [M][K]      two's complement, any value
 *               scales fp32  [M]         w = scales[m] * q
 *               biases must be NULL.  K must be a multiple of 16.
 *     (MiniCPM-V-4.6 on a Tesla C2075, academ.us 2607.14568, section 2.3
 *     "Quantization and residency" and section 3.3 "Decode, and why 4-bit
 *     is slower": symmetric 8-bit weights with an FP32 scale, read without
 *     unpacking; here the scale is per row.)
 *
 *   QG_I8_G64   codes  int8  [M][K]      two's complement, any value
 *               scales fp32  [M][K/64]   w = scales[m][k/64] * q
 *               biases must be NULL.  K must be a multiple of 64.
 *     (MiniCPM-V-4.6 on a Tesla C2075, section 2.3: symmetric 8-bit codes,
 *     each run of 64 sharing an FP32 factor, as that backbone ships them.)
 *
 *   QG_U4_G64   codes  uint8 [M][K/2]    byte j of a row: k=2j in bits 0..3,
 *                                        k=2j+1 in bits 4..7, q in 0..15
 *               scales bf16  [M][K/64]   (uint16 bit patterns)
 *               biases bf16  [M][K/64]
 *               w = scales[m][k/64] * q + biases[m][k/64].  K multiple of 64.
 *     (Pushing the limits of legacy hardware, "Start with the machine that
 *     actually exists": group-64 affine 4-bit codes with bf16 scale and bias;
 *     I Built an LLM Inference Engine on a 15 year old GPU..., "Quantization:
 *     The Model Doesn't Run on INT4": code times scale plus the minimum.)
 *
 *   QG_B1_G128  codes  uint8 [M][K/8]    bit (k mod 8) of byte k/8, least
 *                                        significant bit first
 *               scales fp16  [M][K/128]  (uint16 bit patterns)
 *               w = +scales[m][k/128] if the bit is 1, -scales[..] if 0.
 *               biases must be NULL.  K multiple of 128.
 *     (A 27B model on two 4GB Maxwell GPUs: inference tuning, "Why this
 *     machine is awkward": binary weights with FP16 scales.)
 *
 * Conventions shared by every entry point
 *
 *   Ownership   The caller owns every buffer. All data pointers are device
 *               pointers (hipMalloc'd or equivalent) and stay resident; the
 *               library never allocates, frees, copies to or from the host,
 *               or synchronizes. (I Built an LLM Inference Engine..., "The
 *               memory movement problem" and "Cost 2": weights live on the
 *               device, and nothing is allocated on the hot path.)
 *   Streams     Work is enqueued on `stream` (0 = the null stream) and the
 *               call returns without waiting for it.
 *   Alignment   codes, scales, biases, x, y / logits / out and ws must be
 *               16-byte aligned; idx and ids 4-byte aligned.
 *   Aliasing    The written buffers (y or logits, idx, out, ws) must not overlap
 *               each other or any input.
 *   Errors      Every argument error is detected on the host before
 *               anything is enqueued; the outputs are then left untouched
 *               and a negative QG_ERR_* code is returned. QG_ERR_LAUNCH
 *               reports a failed kernel launch (hipGetLastError).
 *               (Pushing the limits of legacy hardware, "Build the execution
 *               path, then share the weights": a request that cannot be
 *               served fails before changing live state.)
 *   Threads     The library keeps no mutable state; calls are reentrant.
 *               Calls that share a workspace must not overlap in time; two
 *               that do (on different streams) may both return wrong
 *               results, but the calls after them are not affected.
 *   Workspace   `ws` is device memory of at least qg_workspace_bytes(...)
 *               bytes for the same (op, fmt, M, K, rows); it may be NULL
 *               when that size is 0. Its contents on entry do not matter,
 *               so freshly allocated memory serves. Its first
 *               QG_WS_CONTROL_BYTES bytes are completion words (counters of
 *               finished workgroups, for the greedy head and for combining
 *               partial sums of K chunks), each tagged by the kernel launch
 *               that counts on it and claimed afresh by every launch, so a
 *               call that was cut short, or stale or uninitialised words,
 *               cannot disturb a later call. The rest is scratch (partial
 *               sums, parked argmax keys). The workspace is caller-owned
 *               device memory because the library allocates nothing on the
 *               hot path (I Built an LLM Inference Engine on a 15 year old
 *               GPU..., "Cost 2").
 */
#ifndef QG_H
#define QG_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QG_ABI_VERSION 2

typedef enum {
    QG_I8_ROW = 1,
    QG_U4_G64 = 2,
    QG_B1_G128 = 3,
    QG_I8_G64 = 4
} qg_format;

typedef enum {
    QG_OP_GEMV = 1,
    QG_OP_GEMM = 2,
    QG_OP_GEMV_ARGMAX = 3
} qg_op;

enum {
    QG_OK = 0,
    QG_ERR_NULL = -1,        /* a required pointer is NULL, or biases given where none belong */
    QG_ERR_FORMAT = -2,      /* unknown format */
    QG_ERR_SHAPE = -3,       /* M, K or rows out of range, or K not a multiple of the format's unit */
    QG_ERR_ALIGN = -4,       /* a pointer is not aligned as required */
    QG_ERR_WORKSPACE = -5,   /* ws_bytes smaller than qg_workspace_bytes(...) */
    QG_ERR_ALIAS = -6,       /* a written buffer overlaps another buffer */
    QG_ERR_LAUNCH = -7,      /* the kernel launch failed */
    QG_ERR_UNSUPPORTED = -8, /* a known format this entry point does not implement
                                (only qembed returns it: 4-bit rows only) */
    QG_ERR_SCRATCH = -9      /* the call needs more than QG_STATIC_SCRATCH_BYTES of
                                the library's own scratch (qgemv_argmax_noalloc) */
};

/* Control words at the start of every workspace (see Workspace above). */
#define QG_WS_CONTROL_BYTES 8192

/* Largest batch of qgemv / qgemv_argmax. */
#define QG_MAX_GEMV_BATCH 16
/* Largest batch of the greedy head (qgemv_argmax); above QG_MAX_GEMV_BATCH
 * it runs as the prefill product with per-tile argmax keys. */
#define QG_MAX_ARGMAX_BATCH 256

/*
 * qgemv -- batch-1 (up to QG_MAX_GEMV_BATCH) quantized matrix-vector product.
 *   y[n][m] = sum_k w[m][k] * x[n][k],  0 <= n < batch, 0 <= m < M.
 * Every packed weight is read once per call (4-bit, 9 to 16 rows on the
 * small-batch matrix-core kernel: once per launch of up to 8 rows),
 * dequantized in registers and never written out. Batches of 2 to 16 rows
 * may run on the prefill kernel (see qgemm) where that is expected to be
 * faster; the result contract is the same. (MiniCPM-V-4.6 on a Tesla
 * C2075, section 3.3: decode reads each weight once and is bandwidth-bound;
 * I Built an LLM Inference Engine..., "Optimization 4: Quantized Kernels":
 * dequantization is fused into the product.)
 *   x  float32 [batch][K];  y  float32 [batch][M] (overwritten).
 *   1 <= M <= 2^31-1, 1 <= K <= 2^30, 1 <= batch <= QG_MAX_GEMV_BATCH.
 */
int qgemv(int fmt, const void *codes, const void *scales, const void *biases,
          const float *x, float *y, int64_t M, int64_t K, int batch,
          void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * qgemm -- prefill form: the same product over N token rows.
 *   Y[n][m] = sum_k w[m][k] * X[n][k],  0 <= n < N.
 * (MiniCPM-V-4.6 on a Tesla C2075, section 3.1 "Prefill projections": the
 * prompt's projections contract whole matrices, not vectors; A 27B model on two
 * 4GB Maxwell GPUs, "A packed Q1 prefill kernel with a narrow dispatch
 * window": the weights may be consumed packed.)
 *   X  float32 [N][K];  Y  float32 [N][M] (overwritten).  1 <= N <= 2^31-1;
 *   above QG_MAX_GEMV_BATCH rows (the matrix-core kernel) K <= 2^21.
 *   All four formats; for QG_U4_G64 the bias term sum_g b[m][g] * (sum of
 *   X[n][k] over group g) is added per group beside the scaled code sums.
 *   Needs a workspace when qg_workspace_bytes(QG_OP_GEMM, ...) is nonzero:
 *   up to QG_MAX_GEMV_BATCH rows as qgemv, and above that whenever the
 *   output has too few tiles to fill the chip (fewer than one per compute
 *   unit; two for the 8-bit formats, four for the 1-bit format) or a short
 *   last round of tiles, since K is then cut into pieces whose float32
 *   partial products are added in a fixed order by a second launch (the
 *   result does not depend on the stream or the schedule). 17..48 rows of the 4-bit format at K = 1024 or 2048 may
 *   run as launches of up to QG_MAX_GEMV_BATCH rows of the matrix-vector
 *   product where that reads the weights for less than the prefill kernel's
 *   padded work costs.
 */
int qgemm(int fmt, const void *codes, const void *scales, const void *biases,
          const float *x, float *y, int64_t M, int64_t K, int64_t N,
          void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * qgemv_argmax -- qgemv followed by greedy selection, fused.
 *   logits[n][m] = y[n][m] as qgemv computes it (float32, written),
 *   idx[n]       = the lowest m whose logits[n][m] is the maximum of row n
 *                  (ties go to the lowest index; -0 equals +0).
 * (Pushing the limits of legacy hardware, "Build the execution path, then
 * share the weights": for greedy decoding the head only has to report, per
 * tile of logits, the largest value and where it sits, and the choice of
 * token is made on the device.)
 *   logits  float32 [batch][M], or NULL: then no logits are written (the
 *           greedy-only head; the maxima still come from the same float32
 *           values a non-NULL call writes).
 *   idx     int32 [batch].
 *   1 <= batch <= QG_MAX_ARGMAX_BATCH; other limits as qgemv, and K <= 2^21
 *   above QG_MAX_GEMV_BATCH rows. Up to
 *   QG_MAX_GEMV_BATCH rows use the matrix-vector kernels; more rows use the
 *   prefill kernels, which keep one (value, index) key per tile (or part of
 *   one) and token row in the workspace and reduce them in a second launch
 *   (the per-tile reduction of the page above), except 17..48 rows of the
 *   4-bit format at K = 1024 or 2048, which may run as launches of up to
 *   QG_MAX_GEMV_BATCH rows on the matrix-vector kernels. Needs a workspace.
 */
int qgemv_argmax(int fmt, const void *codes, const void *scales,
                 const void *biases, const float *x, float *logits,
                 int32_t *idx, int64_t M, int64_t K, int batch,
                 void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * qgemv_argmax_noalloc -- qgemv_argmax without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). Same arguments,
 * results and limits as qgemv_argmax; the workspace it would need comes from
 * a static array of QG_STATIC_SCRATCH_BYTES bytes that the library keeps on
 * each GPU it runs on until the process ends. The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); its first call on
 * a device looks up that device's array (the device must be current, as
 * for every call). Calls that need more scratch than the array holds return
 * QG_ERR_SCRATCH before anything is enqueued. Every call on a GPU shares
 * that GPU's array: calls that overlap in time on one GPU (different
 * streams or host threads) race and may return wrong results, though calls
 * after them are not affected. Nothing in the array has to be cleared
 * between calls (its completion words are claimed by each launch).
 */
#define QG_STATIC_SCRATCH_BYTES (8u << 20)
int qgemv_argmax_noalloc(int fmt, const void *codes, const void *scales,
                         const void *biases, const float *x, float *logits,
                         int32_t *idx, int64_t M, int64_t K, int batch,
                         hipStream_t stream);

/*
 * qembed -- embedding rows gathered from the (tied) 4-bit weight matrix.
 *   out[t][k] = e(ids[t], k),  0 <= t < n, 0 <= k < K, where for a row m
 *   inside the table e(m, k) is decoded as three rounded steps:
 *     p = scales[m][k/64] * q        (float32; exact, 8 x 4 significant bits)
 *     a = p + biases[m][k/64]        (float32, round to nearest even; the
 *                                     product and the sum are not fused)
 *     e = a rounded to IEEE binary16 (nearest even, subnormals kept,
 *         overflow to infinity) and widened back to float32.
 *   A zero sum is -0 only when both terms are -0 (IEEE 754 sums under
 *   nearest-even), and a negative sum too small for binary16 becomes -0,
 *   not +0. A row id outside [0, M) gives a row of quiet NaNs.
 * (Pushing the limits of legacy hardware, "Half a billion values, and one
 * negative zero": that row decoder multiplies and adds in two steps and
 * passes each value through FP16 on its way to FP32, and the lookup on the
 * GPU had to reproduce denormals, the sign of zero and round-to-nearest-even
 * exactly; I Built an LLM Inference Engine..., "Cost 1: the embedding lookup
 * still runs on the CPU": the quantized rows are decoded on the device from
 * token ids instead of crossing PCIe.)
 *   fmt     QG_U4_G64 only; the other known formats give QG_ERR_UNSUPPORTED.
 *   ids     int32 [n], device memory (4-byte aligned); any values.
 *   out     float32 [n][K] (overwritten).
 *   1 <= n <= 2^31-1; M and K as qgemv. No workspace.
 */
int qembed(int fmt, const void *codes, const void *scales, const void *biases,
           const int32_t *ids, float *out, int64_t M, int64_t K, int64_t n,
           hipStream_t stream);

/* Bytes of device workspace the call (op, fmt, M, K, rows) needs; rows is
 * the batch for QG_OP_GEMV / QG_OP_GEMV_ARGMAX and N for QG_OP_GEMM.
 * Returns 0 when no workspace is needed, and also for arguments the entry
 * point would reject (the entry point then reports the error). The caller
 * allocates it once, off the hot path, and may reuse it for every call of
 * the same or a smaller size (I Built an LLM Inference Engine..., "Cost 2":
 * nothing is allocated per call; Pushing the limits of legacy hardware,
 * "Build the execution path, then share the weights": the greedy head
 * keeps per-tile (value, index) pairs instead of whole logits, which is
 * what the argmax part of the workspace holds). */
size_t qg_workspace_bytes(int op, int fmt, int64_t M, int64_t K, int64_t rows);

/* Static text for a status code. */
const char *qg_status_str(int status);

/* QG_ABI_VERSION of the built library. */
int qg_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QG_H */
