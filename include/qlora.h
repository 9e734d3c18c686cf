/*
 * qlora.h -- C ABI of the MI355X (gfx950) NF4 double-quantized QLoRA linear.
 *
 * Page legend for the citations below:
 *   [P1] "QLoRA, in depth: when a 4-bit base is worth it for small language
 *        models, and how to ship the result"
 *   [P2] "What is QLoRA, and how does 4-bit training make consumer-hardware
 *        fine-tuning possible?"
 *   [P4] "QLoRA and Fine-Tuning on One Consumer GPU"
 *   [P5] "QLoRA"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Device pointers unless stated otherwise; all buffers are caller-owned.
 *   The library never allocates, frees or retains memory.
 * - Row-major storage.  bf16 values are passed as their uint16_t bit
 *   patterns.
 * - W is the frozen weight in nn.Linear layout: n_out rows by k_in columns.
 *   k_in must be a multiple of 64 (a block never straddles a row) and n_out
 *   a multiple of 8 (16-byte aligned rows of Y and dY).
 * - Every device pointer must be 16-byte aligned.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *   the call returns without waiting for it.  Nothing is synchronised.  Calls
 *   are re-entrant: no state is kept between calls (the NF4 table is
 *   computed once on the host under std::call_once and passed to kernels by
 *   value), except the thread-local measurement request of
 *   qlora_time_next_gemm.
 * - Inputs are never written.  Outputs are fully overwritten (never
 *   accumulated into).
 * - Return value: QLORA_OK or a negative status; qlora_last_error() gives a
 *   thread-local message for the most recent failure on the calling thread.
 *   Arguments are checked on the host before anything is enqueued, so an
 *   argument error leaves every buffer untouched.
 *
 * Stored weight format (NF4 with double-quantized block scales; [P1] "The
 * mechanism in brief", [P2] "The three QLoRA ideas", [P4] "NF4 and double
 * quantisation"):
 *   nw = n_out*k_in weights, nb = nw/64 blocks, ng = ceil(nb/256) groups,
 *   flattened row-major.
 *   codes        uint8[nw/2]  two 4-bit level indices per byte; element 2j in
 *                              the low nibble, 2j+1 in the high nibble.
 *   absmax_q8    uint8[nb]     8-bit code of each block's absmax.
 *   absmax_scale float[ng]     fp32 step of the 8-bit absmax code for each
 *                              group of 256 consecutive blocks.
 *   Decode: a' = fp32(q8[b] * s2[b/256]);  w = fp32(T[code] * a');
 *           W_bf16 = round-to-nearest-even bf16 of w.
 *   T is the 16-level NF4 table from qlora_nf4_table().
 *   Cost: 4 + 8/64 + 32/16384 = 4.126953125 bits per weight.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  QLORA_OK = 0,
  QLORA_ERR_INVALID_ARG = -1, /* NULL required pointer, negative size, r < 0 */
  QLORA_ERR_SHAPE = -2,       /* k_in % 64 != 0, n_out % 8 != 0, r > 64, n_out*k_in >= 2^32, M*max(n_out,k_in) > 2^30 */
  QLORA_ERR_ALIGN = -3,       /* a device pointer not 16-byte aligned */
  QLORA_ERR_WORKSPACE = -4,   /* workspace pointer NULL or ws_bytes too small */
  QLORA_ERR_HIP = -5          /* a HIP launch or runtime error */
};

/* Largest adapter rank the kernels accept (the pages use 8 to 32). */
#define QLORA_MAX_RANK 64

/* Operation ids for qlora_workspace_bytes. */
enum { QLORA_OP_FWD = 1, QLORA_OP_BWD = 2 };

/* Storage formats of qlora_quantize_format / qlora_dequant_format.  The
 * products use QLORA_FORMAT_NF4_DQ (the format above); the others are the
 * alternatives the pages weigh it against. */
enum {
  QLORA_FORMAT_NF4_DQ = 0,   /* NF4 levels, q8 block scales + fp32 step per 256 blocks */
  QLORA_FORMAT_NF4 = 1,      /* NF4 levels, one fp32 absmax per block (4.5 bits/weight) */
  QLORA_FORMAT_INT4_DQ = 2,  /* evenly spaced levels -1 + 2i/15, double-quantized scales */
  QLORA_FORMAT_INT4 = 3      /* evenly spaced levels, fp32 absmax per block */
};

/* The frozen weight: borrowed device pointers, never written. */
typedef struct {
  int64_t n_out;              /* rows of W (output features) */
  int64_t k_in;               /* columns of W (input features), % 64 == 0 */
  const uint8_t *codes;       /* [n_out*k_in/2] */
  const uint8_t *absmax_q8;   /* [n_out*k_in/64] */
  const float *absmax_scale;  /* [ceil(n_out*k_in/64/256)] */
} qlora_nf4_weight;

/*
 * Quantize an fp32 weight into the stored format above
 * ([P1] "The mechanism in brief"; [P4] "NF4 and double quantisation").
 *   W            device fp32 [n_out, k_in], read only.
 *   codes        device uint8 [n_out*k_in/2], written.
 *   absmax_q8    device uint8 [nb], written.
 *   absmax_scale device fp32 [ng], written.
 * Per block of 64: a = max|w| (fp32); x = fp32(w / a) (IEEE division;
 * a == 0 gives x = 0); code = nearest NF4 level to x, exact ties to the lower
 * level.  Codes use the fp32 absmax before double quantization.
 * Per group of 256 blocks (the last one may be partial): s2 = fp32(max a / 255);
 * q8 = round-half-even(fp32(a / s2)) clamped to [0, 255]; a zero group gives
 * s2 = 0 and q8 = 0.  Non-finite weights give unspecified codes.
 * Needs no workspace.  n_out == 0 is a no-op.
 */
int qlora_quantize_nf4_dq(const float *W, int64_t n_out, int64_t k_in,
                          uint8_t *codes, uint8_t *absmax_q8, float *absmax_scale,
                          hipStream_t stream);

/*
 * Same as qlora_quantize_nf4_dq for a bf16 weight (widened exactly to fp32
 * first): re-quantizes a merged weight for serving ([P1] "Shipping: merge,
 * re-quantize, verify").
 *   W  device bf16 (uint16 bits) [n_out, k_in].
 */
int qlora_quantize_nf4_dq_bf16(const uint16_t *W, int64_t n_out, int64_t k_in,
                               uint8_t *codes, uint8_t *absmax_q8, float *absmax_scale,
                               hipStream_t stream);

/*
 * Merge the adapter into the frozen weight ([P1] "Shipping: merge,
 * re-quantize, verify"; [P5] "QLoRA", "Walking through the tooling": at
 * inference W' = W + scaled B A):
 *   W_merged  device bf16 [n_out, k_in], written:
 *               W_merged = bf16(W_bf16 + s * (B A)),  s = fp32(alpha / r)
 *             with W_bf16 the decoded weight, B A summed in fp32, and one
 *             rounding to bf16 (round to nearest even).
 *   A, B, r, alpha as in qlora_linear_fwd; r == 0 gives the decoded weight.
 * Re-quantizing the result (qlora_quantize_nf4_dq_bf16) gives the single
 * 4-bit weight file of the merged model; its difference from W_merged is
 * the re-quantization drift the pages warn about.
 */
int qlora_merge(const qlora_nf4_weight *w, const uint16_t *A, const uint16_t *B, int32_t r,
                float alpha, uint16_t *W_merged, hipStream_t stream);

/*
 * Dequantize the whole weight to bf16 ([P1] "The mechanism in brief": the
 * layer dequantizes W to the compute dtype, usually bf16).
 *   W_bf16  device uint16 [n_out, k_in], written.
 * Bit-exact with the decode rule above.
 */
int qlora_dequant(const qlora_nf4_weight *w, uint16_t *W_bf16, hipStream_t stream);

/*
 * Forward of the adapted linear ([P1] "The mechanism in brief": W x plus
 * (alpha / r) B A x; [P4] "The idea in one line": each weight tile is
 * dequantized to bf16 only for the matmul that uses it).
 *   X      device bf16 [M, k_in].
 *   A      device bf16 [r, k_in]     (LoRA down-projection).
 *   B      device bf16 [n_out, r]    (LoRA up-projection).
 *   Y      device bf16 [M, n_out], written:
 *            Y = X W_bf16^T + U~ B^T,  U~ = bf16(s * X A^T),  s = fp32(alpha / r)
 *          accumulated in fp32, rounded once to bf16.
 *   U_out  optional device bf16 [M, r]: receives U~ (the scaled adapter
 *          activation) for the backward pass; NULL to discard.
 *   ws     device workspace, 16-byte aligned, of qlora_workspace_bytes(
 *          QLORA_OP_FWD, ...) bytes (always enough; may be NULL when that is
 *          0).  It holds U~ when U_out is NULL, followed by fp32 split-K
 *          partial sums of X A^T for large M * k_in; with U_out given the
 *          partials alone are needed (with r == 0, nothing).  When the
 *          output tiles of the main product are too few to fill the GPU
 *          (or, with 8 to 16 tokens, the few-token kernel has at most 2
 *          output tiles per compute unit over a long reduction), the same
 *          region after U~ also holds fp32 partial products of a reduction
 *          split; a workspace too small for them is not an error: the
 *          product then runs unsplit (same contract; only the fp32
 *          summation order differs).
 * r == 0 (or A/B NULL with r == 0) gives Y = X W_bf16^T.  M == 0 is a no-op.
 * The dequantized weight is never written to memory.  M <= 16 runs a
 * dedicated few-token kernel (bound by reading the packed weight); the
 * result contract is the same, only the fp32 summation order differs.
 */
int qlora_linear_fwd(const qlora_nf4_weight *w, const uint16_t *X, int64_t M,
                     const uint16_t *A, const uint16_t *B, int32_t r, float alpha,
                     uint16_t *Y, uint16_t *U_out, void *ws, size_t ws_bytes,
                     hipStream_t stream);

/*
 * Backward of the adapted linear: gradients for the activations and the
 * adapter, never for the frozen weight ([P1] "The mechanism in brief";
 * [P4] "The idea in one line").
 *   X, A, B  as in the forward.   dY device bf16 [M, n_out].
 *   U        optional device bf16 [M, r]: the U~ the forward returned in
 *            U_out; NULL recomputes it from X and A.
 *   dX       device bf16 [M, k_in], written:
 *              dX = dY W_bf16 + V~ A,  V~ = bf16(s * dY B)
 *   dA       device fp32 [r, k_in], written:  dA = V~^T X   (= s V^T X)
 *   dB       device fp32 [n_out, r], written: dB = dY^T U~  (= s dY^T U)
 *   ws       device workspace of qlora_workspace_bytes(QLORA_OP_BWD, ...),
 *            16-byte aligned.  With r > 0 the part for U~, V~ and the token
 *            reductions is required; the rest (fp32 partial products of a
 *            reduction split of dX, used when its output tiles are too few
 *            to fill the GPU) is optional, as in the forward: without it dX
 *            is computed unsplit.  With r == 0 ws may be NULL.
 * Token reductions are deterministic (fixed-order partial sums, no float
 * atomics): repeated calls give bitwise-identical results.
 * r == 0 gives dX = dY W_bf16 and touches neither dA nor dB.  An empty
 * token or feature dimension (M, n_out or k_in zero) makes the token
 * reductions empty sums: dA and dB are zero-filled (when r > 0), dX is
 * zero-filled when n_out == 0 (and M, k_in > 0), and nothing else is written.
 */
int qlora_linear_bwd(const qlora_nf4_weight *w, const uint16_t *X, const uint16_t *dY,
                     int64_t M, const uint16_t *A, const uint16_t *B, int32_t r,
                     float alpha, const uint16_t *U, uint16_t *dX, float *dA, float *dB,
                     void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * qlora_linear_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, results and
 * errors as qlora_linear_fwd given a workspace of qlora_workspace_bytes
 * (bit for bit: the same kernels and work splits),
 * with the workspace taken from a fixed 64 MiB array the library holds on
 * each GPU it runs on (until the process ends).  Sizes whose forward needs
 * more (qlora_workspace_bytes(QLORA_OP_FWD, ...) > 64 MiB, e.g. more than
 * about 2.9 M tokens-times-k_in elements) return QLORA_ERR_WORKSPACE before
 * anything is enqueued.  The call allocates nothing and issues only kernel
 * launches.  Every call on one GPU shares that GPU's array and nothing in it
 * needs to start at zero; calls that overlap on one GPU (concurrent streams
 * or threads) race on it, so serialise them.
 */
int qlora_linear_fwd_noalloc(const qlora_nf4_weight *w, const uint16_t *X, int64_t M,
                             const uint16_t *A, const uint16_t *B, int32_t r, float alpha,
                             uint16_t *Y, uint16_t *U_out, hipStream_t stream);

/*
 * fp16 instance of the path: the same operations with every 16-bit
 * quantity in IEEE binary16 instead of bf16 -- the decoded weight
 * (W_f16 = RNE_fp16(level[c] * fp32(q8 * s2))), X, A, B, Y, U~, dY, V~ and
 * dX -- on v_mfma_f32_*_f16.  The pages compute in bf16 and name fp16 for
 * GPUs without bf16 ([P1] "A complete run on a 12 GB-class GPU", the
 * bnb_4bit_compute_dtype line).  The weight triple, dA, dB, the workspace
 * sizes and every check and error are exactly those of qlora_dequant,
 * qlora_linear_fwd and qlora_linear_bwd; the 16-bit arguments are binary16
 * bit patterns.  A separate instantiation of the kernels, not a runtime
 * switch inside them.
 */
int qlora_dequant_f16(const qlora_nf4_weight *w, uint16_t *W_f16, hipStream_t stream);
int qlora_linear_fwd_f16(const qlora_nf4_weight *w, const uint16_t *X, int64_t M,
                         const uint16_t *A, const uint16_t *B, int32_t r, float alpha,
                         uint16_t *Y, uint16_t *U_out, void *ws, size_t ws_bytes,
                         hipStream_t stream);
int qlora_linear_bwd_f16(const qlora_nf4_weight *w, const uint16_t *X, const uint16_t *dY,
                         int64_t M, const uint16_t *A, const uint16_t *B, int32_t r,
                         float alpha, const uint16_t *U, uint16_t *dX, float *dA, float *dB,
                         void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Forward and backward with LoRA dropout of the adapter input.  The pages'
 * adapter configurations set lora_dropout = 0.05 ([P1] "A complete run on a
 * 12 GB-class GPU"; [P5] "Walking through the tooling") without defining
 * it; this is inverted dropout of the adapter's input x (x is dropped before
 * A; the frozen path W x sees the undropped x):
 *   keep(m, k)  element (m, k) of X, flat index e = m k_in + k, is kept iff
 *               word (e & 3) of Philox4x32-10(counter (lo32(e >> 2),
 *               hi32(e >> 2), 0, 0), key (lo32(seed), hi32(seed))) is
 *               >= floor(dropout_p 2^32)  (Salmon et al., SC'11).
 *   s_d         fp32(alpha / (r (1 - dropout_p)))  (1 / (1 - p) folded in).
 *   forward     U~ = bf16(s_d (keep * X) A^T);  Y = X W_bf16^T + U~ B^T.
 *   backward    V~ = bf16(s_d dY B);  dX = dY W_bf16 + keep * (V~ A);
 *               dA = V~^T (keep * X);  dB = dY^T U~.
 * The mask depends only on (seed, element position), so the backward
 * regenerates it: pass the forward's seed.  U may be the forward's U_out
 * (it already holds the mask) or NULL (recomputed with the mask).  Every
 * other argument, the workspace size and the error behaviour are those of
 * qlora_linear_fwd / qlora_linear_bwd; dropout_p outside [0, 1) (or NaN)
 * returns QLORA_ERR_INVALID_ARG.  dropout_p == 0 gives exactly the results
 * of qlora_linear_fwd / qlora_linear_bwd.
 */
int qlora_linear_fwd_dropout(const qlora_nf4_weight *w, const uint16_t *X, int64_t M,
                             const uint16_t *A, const uint16_t *B, int32_t r, float alpha,
                             double dropout_p, uint64_t seed, uint16_t *Y, uint16_t *U_out,
                             void *ws, size_t ws_bytes, hipStream_t stream);
int qlora_linear_bwd_dropout(const qlora_nf4_weight *w, const uint16_t *X, const uint16_t *dY,
                             int64_t M, const uint16_t *A, const uint16_t *B, int32_t r,
                             float alpha, double dropout_p, uint64_t seed, const uint16_t *U,
                             uint16_t *dX, float *dA, float *dB, void *ws, size_t ws_bytes,
                             hipStream_t stream);
/* The same two operations in the fp16 instance (see qlora_linear_fwd_f16):
 * every 16-bit argument is a binary16 bit pattern, U~ and V~ are rounded to
 * binary16; the mask, s_d, the workspace and the errors are as above. */
int qlora_linear_fwd_dropout_f16(const qlora_nf4_weight *w, const uint16_t *X, int64_t M,
                                 const uint16_t *A, const uint16_t *B, int32_t r, float alpha,
                                 double dropout_p, uint64_t seed, uint16_t *Y, uint16_t *U_out,
                                 void *ws, size_t ws_bytes, hipStream_t stream);
int qlora_linear_bwd_dropout_f16(const qlora_nf4_weight *w, const uint16_t *X, const uint16_t *dY,
                                 int64_t M, const uint16_t *A, const uint16_t *B, int32_t r,
                                 float alpha, double dropout_p, uint64_t seed, const uint16_t *U,
                                 uint16_t *dX, float *dA, float *dB, void *ws, size_t ws_bytes,
                                 hipStream_t stream);

/* Workspace bytes needed by qlora_linear_fwd (op = QLORA_OP_FWD) or
 * qlora_linear_bwd (op = QLORA_OP_BWD) for these sizes: enough for any
 * U_out / U argument (U_out == NULL, U == NULL is the worst case), including
 * the optional room for a reduction split.  Returns 0 for invalid arguments
 * and when no workspace is used (M == 0; r == 0 with output tiles enough to
 * fill the GPU). */
size_t qlora_workspace_bytes(int op, int64_t M, int64_t n_out, int64_t k_in, int32_t r);

/* Host function: the work split the library chooses for the main product
 * of op at these sizes on a device with `compute_units` compute units
 * (<= 0: the calling thread's current device; 256 when none can be
 * queried).  op = QLORA_OP_FWD: the forward product; QLORA_OP_BWD: the dX
 * product.  Writes out[0] = the kernel (1: fused GEMM, reduction in 64-deep
 * steps; 2: few-token forward, reduction in 128-wide chunks), out[1] = the
 * splits of the reduction across workgroups (1: unsplit), out[2] = steps or
 * chunks per split, out[3] = steps or chunks in all; every split is
 * non-empty: (out[1] - 1) * out[2] < out[3] <= out[1] * out[2].  The split
 * runs only when the workspace has room for its partial sums
 * (qlora_workspace_bytes counts them).  Returns QLORA_OK, or
 * QLORA_ERR_INVALID_ARG for an unknown op, negative sizes or out == NULL. */
int qlora_plan(int op, int64_t M, int64_t n_out, int64_t k_in, int compute_units, int64_t out[4]);

/* Measurement aid.  The next fused-GEMM kernel launch made by the calling
 * thread (the forward kernel inside qlora_linear_fwd -- the GEMM, or for
 * M <= 16 the few-token kernel -- or the dX GEMM inside qlora_linear_bwd)
 * is bracketed by hipEventRecord(start) and
 * hipEventRecord(stop) on that call's stream, so hipEventElapsedTime gives
 * the duration of that one kernel.  The request is then cleared.  Passing
 * NULL for either event clears a pending request.  Events are caller-owned;
 * the setting is thread-local, so concurrent threads do not interfere. */
void qlora_time_next_gemm(hipEvent_t start, hipEvent_t stop);

/* Diagnostic of the bounds-checked build (libqlora_checked.so, compiled with
 * QLORA_BOUNDS_CHECK; same entry points, same arithmetic).  There every raw
 * global store, and every raw global load of caller-sized data, first checks
 * its element index against the size of the buffer it addresses (as the
 * layouts above define it); an access outside is skipped (a load reads
 * zeros) and counted on the device.  Writes the number of such accesses
 * since the last reset to *count (synchronising the device) and clears it
 * when `reset` is nonzero.  Returns QLORA_OK; QLORA_ERR_INVALID_ARG for
 * count == NULL or in the normal build, which has no checks; QLORA_ERR_HIP
 * if the counters cannot be read. */
int qlora_debug_oob_count(uint64_t *count, int reset);

/* Host function: copies the 16 fp32 NF4 levels the kernels use into out[16]
 * (ascending; 7 negative, an exact 0, 8 positive, extremes -1 and +1: 16
 * levels at normal quantiles, [P1] "The mechanism in brief"). */
void qlora_nf4_table(float out[16]);

/*
 * Storage-format variants, for measuring what NF4 and double quantization
 * buy ([P1] "The mechanism in brief" and [P4] "NF4 and double
 * quantisation": one fp32 absmax per 64 weights costs 0.5 bit, double
 * quantization brings the overhead to about 0.127; [P2] "Follow-up
 * questions to expect": evenly spaced int4 levels waste levels on rare
 * large values, so NF4's error is lower).  Every format uses blocks of 64,
 * x = fp32(w / max|w|) by IEEE division, the nearest level with exact ties
 * to the lower one, and the low nibble for the even element.
 *   format         QLORA_FORMAT_*; anything else -> QLORA_ERR_INVALID_ARG.
 *   codes          device uint8 [n_out*k_in/2].
 *   scales         *_DQ formats: device uint8 q8 [nb], as absmax_q8 above;
 *                  plain formats: device fp32 absmax [nb] (stored exactly).
 *   absmax_scale   *_DQ formats: device fp32 [ng] (s2 as above); plain
 *                  formats: unused, may be NULL.
 * qlora_quantize_format writes codes, scales (and absmax_scale); decoding
 * is W_bf16 = bf16(level[c] * a') with a' = fp32(q8 * s2) or the fp32
 * absmax.  QLORA_FORMAT_NF4_DQ gives exactly the results of
 * qlora_quantize_nf4_dq / qlora_dequant.  Shapes, alignment and errors as
 * for those two.  qlora_format_table copies the format's 16 fp32 levels to
 * host memory out[16] (QLORA_ERR_INVALID_ARG for an unknown format).
 */
int qlora_quantize_format(int format, const float *W, int64_t n_out, int64_t k_in,
                          uint8_t *codes, void *scales, float *absmax_scale, hipStream_t stream);
int qlora_dequant_format(int format, int64_t n_out, int64_t k_in, const uint8_t *codes,
                         const void *scales, const float *absmax_scale, uint16_t *W_bf16,
                         hipStream_t stream);
int qlora_format_table(int format, float out[16]);

/* Host function: static description of a status code. */
const char *qlora_status_string(int status);

/* Host function: thread-local detail of the last failure on this thread
 * ("" if none). */
const char *qlora_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
