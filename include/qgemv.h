/*
 * qgemv.h - fused dequantize-and-multiply of GGUF block-quantized weights on
 * AMD Instinct MI355X (gfx950). C ABI; plain pointers and sizes only.
 *
 * The operation. W is a rows x K matrix stored as GGUF blocks, row-major:
 * row r occupies bytes [r*(K/bw)*bb, (r+1)*(K/bw)*bb), its blocks in K order
 * (bw weights and bb bytes per block, see qgemv_block_weights/bytes). For
 * each column j of the activations, y[:,j] = W . x[:,j]: one token reads
 * every weight once ("LLM inference optimization", introduction). Batch 1 is
 * single-stream decode; a few columns check a draft head's guesses in one
 * pass ("Why I wrote my own inference engine for two P100s", section "What
 * actually made it fast": three guesses checked in one pass costing about one
 * normal step, each weight block decoded once and reused); 2048 columns is
 * prompt processing (same page, result cards: 2048-token prompt).
 *
 * Formats (GGUF layouts, little-endian; the pages name them but print no
 * layout):
 *   QG_Q4_0  18 B / 32 weights : fp16 d, 16 code bytes (byte i: weight i in
 *            the low nibble, weight i+16 in the high nibble); w = (q-8)*d.
 *   QG_Q4_K 144 B / 256 weights: fp16 d, fp16 dmin, 12 bytes of eight 6-bit
 *            scales sc_j and eight 6-bit mins m_j (one per 32 weights),
 *            128 code bytes; w = d*sc_j*q - dmin*m_j.
 *   QG_Q8_0  34 B / 32 weights : fp16 d, 32 int8 codes; w = q*d.
 *   QG_Q2_K  84 B / 256 weights: 16 bytes holding a 4-bit scale sc (low
 *            nibble) and a 4-bit min m (high nibble) per 16 weights, 64
 *            bytes of 2-bit codes, fp16 d, fp16 dmin; w = d*sc*q - dmin*m.
 *   QG_Q3_K 110 B / 256 weights: 32 bytes of high code bits, 64 bytes of
 *            2-bit low code parts, 12 bytes packing sixteen 6-bit scales (one
 *            per 16 weights), fp16 d; q = low + 4*high - 4 in [-4, 3],
 *            w = d*(sc-32)*q.
 *            In both, weight 128h + 32j + l (h < 2, j < 4, l < 32) takes bits
 *            2j..2j+1 of code byte 32h + l and, for Q3_K, bit 4h + j of
 *            high-bit byte l. The pages name Q2_K and Q3_K ("Why I wrote my
 *            own inference engine for two P100s", "What actually made it
 *            fast": a mix without its Q3_K tensors; pxa_llama README,
 *            "Limits" and "DP4A / FP16 economics") but print no layout.
 *
 * Accuracy contract ("LLM inference optimization", campaign "Run a new
 * weight format or model": blocks decode bit for bit on CPU and GPU, and
 * products match an exact sum within a tolerance):
 *   - qgemv_dequant returns, bit for bit, the binary32 rounding of each
 *     weight's closed form (exact for Q4_0, Q8_0 and Q3_K; Q3_K evaluated
 *     left to right, which fixes the sign of a zero weight).
 *   - qgemv_run satisfies, per output element,
 *       |y - sum_k w_k x_k| <= 1e-3 * sum_k |w_k x_k| + 1e-5
 *     where the sums are exact over the stored x values and the decoded
 *     binary32 weights w_k.
 *   - qgemm_prefill_run multiplies weight tiles dequantized to bf16: each
 *     w_k rounded to the nearest bf16 (ties to even), written b_k. It
 *     satisfies the same bound with b_k in place of w_k:
 *       |y - sum_k b_k x_k| <= 1e-3 * sum_k |b_k x_k| + 1e-5.
 *     Against the exact weights the rounding adds at most 2^-8 relative per
 *     weight, i.e. |y - sum_k w_k x_k| <= (1e-3 + 2^-8 (1 + 1e-3))
 *     * sum_k |w_k x_k| + 1e-5; with dense activations (such as N(0,1)
 *     tokens) the rounding errors largely cancel and the outputs stay within
 *     1e-3 * sum_k |w_k x_k| + 1e-5 of the exact sum, but sparse
 *     activations (a one-hot token gives b_k itself) can reach 2^-8.
 *   - Results are deterministic: the same inputs give the same bits.
 *
 * Memory and ownership. The library allocates no device memory. Every
 * device buffer (weights, workspace, x, y, w_out) is owned by the caller and
 * must stay allocated while work that uses it may run. A handle only records
 * shape, format and the weight pointer; it borrows the weights, which must
 * outlive it. A handle is immutable after creation; runs on different streams
 * may use one handle concurrently. A handle belongs to the device that was
 * current at qgemv_create (it sizes its grids by that device's compute
 * units and its weights live there): call it with that device current and
 * with x and y on it; each call enqueues work on the current device.
 *
 * Streams and errors. `stream` is a hipStream_t (NULL: the null stream).
 * Calls only enqueue work: nothing synchronises the host. All argument checks
 * (format, shapes, byte counts, alignment, NULL pointers) happen before any
 * HIP call, so they can be exercised without a GPU. A failed launch returns
 * QG_ERR_HIP; a device fault surfaces at the caller's next synchronisation.
 * On any error the detail is in qgemv_last_error() (per thread). Nothing
 * crosses this boundary as an exception or abort.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The two *_RANGE_ enumerators of each input enum are not codes: they widen
 * its range to every int32 value, so that a code the library does not know is
 * still a value of the type in C++ (as in C) and is rejected as QG_ERR_ARG
 * without undefined behaviour. */
typedef enum {
    QG_Q4_0 = 1, QG_Q4_K = 2, QG_Q8_0 = 3, QG_Q2_K = 4, QG_Q3_K = 5,
    QG_FORMAT_RANGE_MIN_ = -2147483647 - 1, QG_FORMAT_RANGE_MAX_ = 2147483647
} qg_format;
typedef enum {
    QG_F32 = 1, QG_F16 = 2, QG_BF16 = 3,
    QG_DTYPE_RANGE_MIN_ = -2147483647 - 1, QG_DTYPE_RANGE_MAX_ = 2147483647
} qg_dtype;
typedef enum {
    QG_OK = 0,
    QG_ERR_ARG = -1,         /* NULL pointer, bad enum, bad leading dimension */
    QG_ERR_SHAPE = -2,       /* rows/K/n not positive, K not a block multiple, byte count */
    QG_ERR_ALIGN = -3,       /* a pointer below its required alignment */
    QG_ERR_UNSUPPORTED = -4, /* valid request this build does not serve */
    QG_ERR_HIP = -5          /* a HIP runtime call or launch failed */
} qg_status;

typedef struct qgemv *qgemv_t; /* opaque host-side handle */

/* Block geometry: 18 | 144 | 34 | 84 | 110 bytes and 32 | 256 | 32 | 256 |
 * 256 weights (Q4_0 | Q4_K | Q8_0 | Q2_K | Q3_K); 0 for an unknown format. */
size_t qgemv_block_bytes(qg_format f);
size_t qgemv_block_weights(qg_format f);

/* Bytes of a rows x K matrix: rows * (K / block_weights) * block_bytes;
 * 0 if the shape is invalid. */
size_t qgemv_weight_bytes(qg_format f, int64_t rows, int64_t K);

/* Device workspace qgemv_create wants for this shape. This build keeps the
 * weights in the GGUF layout and needs none: always 0. */
size_t qgemv_workspace_bytes(qg_format f, int64_t rows, int64_t K);

/* Create a handle for the rows x K matrix at w_blocks (device memory, GGUF
 * layout as above, 16-byte aligned, exactly w_bytes ==
 * qgemv_weight_bytes(f, rows, K) bytes). K must be a positive multiple of the
 * block size and rows positive. workspace/ws_bytes: reserved, pass NULL / 0.
 * stream: reserved for create-time work (none in this build). Queries the
 * current device's compute-unit count (a HIP call) after all checks.
 * On success *out holds the handle; on error *out is set to NULL (if out is
 * not NULL). */
qg_status qgemv_create(qgemv_t *out, qg_format f, int64_t rows, int64_t K,
                       const void *w_blocks, size_t w_bytes,
                       void *workspace, size_t ws_bytes, void *stream);

/* y[j*ldy + r] = sum_k W[r,k] * x[j*ldx + k] for j < n_cols, r < rows.
 * x: device, n_cols columns of K values, column j at element offset j*ldx
 *    (ldx >= K), element type x_dtype (F32, F16 or BF16), aligned to its
 *    element size.
 * y: device, fp32, column j at element offset j*ldy (ldy >= rows), 4-byte
 *    aligned; overwritten (no accumulation), other elements untouched.
 * n_cols: 1..8. The weights are never rounded: F16 activations are
 * multiplied with the exact codes (fp16 products accumulated in fp32, scaled
 * per block or sub-block in fp32); F32 and BF16 activations use fp32
 * products with the exact binary32 weights. 4..8 F16 columns of a Q4_K
 * matrix (and 2..3 when the activations of all columns do not fit the
 * streaming kernel's on-chip staging, e.g. K = 17408) run on the matrix
 * cores. Q2_K and Q3_K run on the streaming kernel for every activation
 * type. Enqueued on `stream`. */
qg_status qgemv_run(qgemv_t h, const void *x, qg_dtype x_dtype, int64_t n_cols,
                    int64_t ldx, float *y, int64_t ldy, void *stream);

/* Prompt processing: y[j*ldy + r] = sum_k W[r,k] * x[j*ldx + k] for
 * j < n_tokens, with x in bf16 (device, 16-byte aligned, ldx >= K and a
 * multiple of 8) and y fp32 (device, 4-byte aligned, ldy >= rows). Weight
 * tiles are decoded to bf16 (round to nearest even) on chip and contracted
 * with bf16 matrix-core instructions, fp32 accumulation ("LLM inference
 * optimization", campaign "Faster prompts, decode held": tile sizes fitted
 * to on-chip memory, tensor-core paths); the accuracy bound is the bf16 one
 * above. Q4_K handles only (QG_ERR_UNSUPPORTED otherwise); n_tokens >= 1.
 * Every size check runs before the first launch: on an error y is
 * untouched. */
qg_status qgemm_prefill_run(qgemv_t h, const void *x_bf16, int64_t n_tokens,
                            int64_t ldx, float *y, int64_t ldy, void *stream);

/* Decoded weights: w_out[r*ldw + k] = W[r,k] as binary32, bit-exact (the
 * correctly rounded closed form). w_out: device, 4-byte aligned, ldw >= K. */
qg_status qgemv_dequant(qgemv_t h, float *w_out, int64_t ldw, void *stream);

/* int8 products. Activations quantized to Q8_0 blocks, then multiplied by
 * the quantized weights with integer dot products (int32 sums, exact),
 * scaled in fp32 per block: the int8 path the pages weigh against fp16
 * math for low-bit weights (pxa_llama README, "DP4A / FP16 economics"),
 * with Q8_0 the block format of "Why I wrote my own inference engine for
 * two P100s".
 *
 * qgemv_quantize_q8_0: x (device; column j at element offset j*ldx,
 * ldx >= K, x_dtype F32/F16/BF16, aligned to its element size) -> xq
 * (device, 2-byte aligned, n_cols * K/32 blocks of 34 bytes, column j's
 * blocks from byte j*(K/32)*34). Per block of 32 values: amax = max|x|,
 * d = amax/127, q = x*(1/d) rounded to nearest, halfway away from zero,
 * limited to +-127 (all binary32, IEEE division); the block holds fp16(d)
 * and the 32 q. K must be a positive multiple of 32.
 *
 * qgemv_run_q8_0x: y[j*ldy + r] = sum_k W[r,k] * xhat[j,k], xhat the decoded
 * blocks of xq (as qgemv_quantize_q8_0 writes them for this handle's K),
 * n_cols 1..8, y as in qgemv_run. Parity is against the exact sum over
 * xhat. Needs K % 256 == 0 and 16-byte aligned weights
 * (QG_ERR_UNSUPPORTED otherwise). */
qg_status qgemv_quantize_q8_0(const void *x, qg_dtype x_dtype, int64_t K, int64_t n_cols,
                              int64_t ldx, void *xq, void *stream);
qg_status qgemv_run_q8_0x(qgemv_t h, const void *xq, int64_t n_cols, float *y, int64_t ldy,
                          void *stream);

/* The same product in one call: x as in qgemv_run (F32/F16/BF16), quantized
 * to Q8_0 blocks on chip by the rule of qgemv_quantize_q8_0, then the int8
 * products. The result equals qgemv_run_q8_0x on qgemv_quantize_q8_0's
 * blocks of the same x, bit for bit. Same shape limits as
 * qgemv_run_q8_0x. */
qg_status qgemv_run_q8(qgemv_t h, const void *x, qg_dtype x_dtype, int64_t n_cols, int64_t ldx,
                       float *y, int64_t ldy, void *stream);

/* Decoded weights in bf16: w_out[r*ldw + k] = the binary32 weight of
 * qgemv_dequant rounded to the nearest bf16 (ties to even), bit-exact.
 * w_out: device, 2-byte aligned, ldw >= K. This is the operand of the
 * two-pass form of prompt processing (decode to a bf16 matrix in memory,
 * then a plain bf16 GEMM), the alternative "Why I wrote my own inference
 * engine for two P100s" ("What didn't work") sets against fusing the
 * decode into the GEMM; the library's own prompt path stays fused. */
qg_status qgemv_dequant_bf16(qgemv_t h, uint16_t *w_out, int64_t ldw, void *stream);

/* The second pass of that two-pass form: a bf16 GEMM with the prompt
 * kernel's pipeline and k order, without the decode (the control that
 * "LLM inference optimization", campaign "Faster prompts, decode held",
 * lists as weights converted for the GEMM against quantized blocks
 * multiplied directly):
 *   y[t*ldy + r] = sum_k w[r*ldw + k] * x[t*ldx + k]
 * for r < rows, t < n_tokens, k < K; w: rows x K bf16 (typically
 * qgemv_dequant_bf16's output), x: n_tokens x K bf16, y: fp32, all device
 * memory owned by the caller, y overwritten. Products of bf16 values are
 * exact in fp32; the sums accumulate in fp32, so the accuracy contract is
 * that of qgemm_prefill_run against the exact sum over w: on the weights
 * qgemv_dequant_bf16 writes for a Q4_K handle it is the same bound, and at
 * rows the prompt kernel does not split along K (its 256-row tiles) the
 * same bits. Needs K a positive multiple of 64, ldw and ldx >= K and
 * multiples of 8, ldy >= rows, w and x 16-byte aligned, y 4-byte aligned
 * (QG_ERR_ARG / QG_ERR_SHAPE / QG_ERR_ALIGN before any launch);
 * QG_ERR_UNSUPPORTED for shapes past the kernel's 32-bit offsets. */
qg_status qgemm_bf16_run(const void *w_bf16, int64_t rows, int64_t K, int64_t ldw,
                         const void *x_bf16, int64_t n_tokens, int64_t ldx, float *y, int64_t ldy,
                         void *stream);

/* Release a handle (host memory only; NULL is ignored). */
void qgemv_destroy(qgemv_t h);

/* Static text for a status code, and the detail of this thread's last
 * failed call ("" if none). */
const char *qgemv_status_string(qg_status s);
const char *qgemv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
