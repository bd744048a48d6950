/*
 * qlinear.h - C ABI of the weight-only quantized linear library for AMD Instinct MI355X (gfx950).
 *
 * Operations (cited by page title and section):
 *   - MLX affine storage: packed uint32 codes plus one scale and one ADDITIVE bias per group of
 *     k-values, value = code*scale + bias (GPTQModel wiki "MLX Apple Silicon", Concepts table;
 *     tinygpt PRD "Quantized inference ... QuantizedLinear", Problem; gguf2mlx-stream, section 01).
 *   - Packing: each row of codes is one little-endian bitstream, code i of the row at stream
 *     bits [bits*i, bits*(i+1)) and stream bit j in bit j % 32 of word j / 32: whole codes per
 *     uint32 at 2, 4 and 8 bits (code c of a word at bits [bits*c, bits*(c+1))), codes crossing
 *     words at 3, 5 and 6 bits; scales/biases laid out [out, groups] (GPTQModel wiki "MLX Apple
 *     Silicon", Packed layouts and exact transcoding).
 *   - dequant / apply / apply_experts and the MXFP4 and Q8_0 block formats
 *     (Nx_quant API docs, Weights and Products).
 *
 * Conventions for every entry point:
 *   - W is [n, k]: n outputs by k inputs, quantized along k.  x is [m, k], y is [m, n], row-major,
 *     contiguous.  Integer sizes are element counts.
 *   - Every pointer except the host problem list of qlinear_gemv_batched is DEVICE memory on the
 *     current HIP device, owned by the caller.  The library allocates nothing and keeps no state
 *     between calls (no decoded or dense weight cache).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls are asynchronous on it; none
 *     synchronizes.  Results are deterministic: the same inputs give the same bits.
 *   - Validation is host-only and runs before any launch.  On error the call returns a status,
 *     launches nothing, and qlinear_last_error() names the offending argument.
 *   - Zero-size outputs (m == 0 or n == 0) return QL_OK without a launch.
 *   - Alignment (QL_ERR_ALIGN otherwise): w, packed words, x, MXFP4 codes, dequant outputs and
 *     workspaces 16-byte aligned; scales, biases, layer_bias and Q8_0 blocks 2-byte aligned;
 *     y aligned to its element size; ids 8-byte, offsets/perm 4-byte aligned.
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QL_OK = 0,
  QL_ERR_NULL = 1,        /* a required pointer is NULL */
  QL_ERR_SHAPE = 2,       /* a size is negative or the shapes do not agree */
  QL_ERR_DTYPE = 3,       /* a dtype outside the supported table */
  QL_ERR_ALIGN = 4,       /* a pointer is not aligned as required */
  QL_ERR_UNSUPPORTED = 5, /* bits / group_size / format not supported */
  QL_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the *_workspace_size query */
  QL_ERR_LAUNCH = 7       /* the HIP runtime rejected a launch or copy */
} ql_status;

typedef enum { QL_F32 = 0, QL_F16 = 1, QL_BF16 = 2 } ql_dtype;
typedef enum { QL_AFFINE = 0, QL_MXFP4 = 1, QL_Q8_0 = 2, QL_MXFP4_BLOCKS = 3, QL_Q4_K = 4, QL_Q6_K = 5 } ql_format;

/* One GEMV of a problem list: y[m,n] = x[m,k] . dequant(W[n,k])^T (+ layer_bias[n]).
 * All pointers are device memory; layer_bias may be NULL. */
typedef struct {
  const void* x;
  const uint32_t* packed;
  const void* scales;
  const void* biases;
  const void* layer_bias;
  void* y;
  int64_t m, n, k;
  int32_t bits, group_size;
} ql_problem;

/* Affine group quantizer (the step that produces the affine storage; gguf2mlx-stream section 01
 * and the MLX affine storage of the GPTQModel wiki Concepts table).
 * w [n,k] fp32 -> packed [n, k*bits/32] uint32, scales and biases [n, k/group_size] in
 * param_dtype (QL_F16 or QL_BF16).  Per (row, group): mn/mx = min/max in fp32 under the total
 * order (-0 < +0); scale = RNE(fl32(mx - mn) / (2^bits - 1)); bias = RNE(mn);
 * code = clamp(round-half-even(fl32(v - bias) / scale), 0, 2^bits - 1), 0 where scale == 0.
 * IEEE fp32 arithmetic, correctly rounded division.  w must be finite (otherwise the
 * outputs are unspecified).  bits in {2, 3, 4, 5, 6, 8}; group_size in {32, 64, 128} dividing k;
 * k % 32 == 0. */
ql_status qlinear_quantize(const float* w, int64_t n, int64_t k, int bits, int group_size,
                           ql_dtype param_dtype, uint32_t* packed, void* scales, void* biases,
                           void* stream);

/* quantize_q8_0 (Nx_quant API docs, quantize_q8_0): w [rows, k] fp32 -> blocks [rows, k/32*34].
 * Per block of 32 values: d = amax/127 in fp32 stored as fp16 (round to nearest even: +inf past
 * fp16's largest); quants = round(v * (1/d)) half away from zero, 1/d from the fp32 d, products
 * in fp32.  Non-finite rules of the page: a block with d == 0 or 1/d infinite (amax below about
 * 127 * 2^-128) is zero bytes; a block holding an infinity and no NaN stores d = +inf and zero
 * quants; a block holding a NaN stores d = NaN (the fp16 quiet NaN 0x7E00) and zero quants.
 * k % 32 == 0 (QL_ERR_SHAPE); w 16-byte aligned, blocks 2-byte aligned.  qlinear_dequant with
 * QL_Q8_0 decodes the result. */
ql_status qlinear_quantize_q8_0(const float* w, int64_t rows, int64_t k, uint8_t* blocks, void* stream);

/* take (Nx_quant API docs, take): dst row i = src row pos[i] for 0 <= pos[i] < src_rows, else
 * row_bytes zero bytes (which decode to zeros in every format).  Bytes are copied with no value
 * decoded; gather each part of a weight with its own row size: affine packed k*bits/8, scales and
 * biases k/group_size*2, MXFP4 codes k/2 and scales k/32, Q8_0 blocks k/32*34, or whole matrices
 * (n times those) to gather experts.  pos: int64 [n_pos], 8-byte aligned, device memory; src
 * [src_rows, row_bytes], dst [n_pos, row_bytes]. */
ql_status qlinear_take(const int64_t* pos, int64_t n_pos, const void* src, int64_t src_rows,
                       int64_t row_bytes, void* dst, void* stream);

/* GPTQ -> MLX affine rows (GPTQModel wiki "MLX Apple Silicon", Packed layouts and exact
 * transcoding; GPTQModel "Packing Formats and Compatibility", GPTQ and GPTQ_V2), continuous
 * layout with contiguous groups (g_idx[k] = k / group_size):
 *   in:  qweight [k*bits/32, n] uint32 (output column j's codes as one little-endian bits-wide
 *        stream down the input axis), qzeros [k/group_size, n*bits/32] uint32 (each group's zeros
 *        as one stream along the outputs), scales [k/group_size, n] in scale_dtype; the GPTQ value
 *        is scale * (code - zero), and v1_zeros != 0 means the stored zeros are zero - 1.
 *   out: packed [n, k*bits/32] (the affine row streams: qweight transposed word for word),
 *        scales_out [n, k/group_size] (transposed), biases_out [n, k/group_size] =
 *        RNE(-zero * scale) in scale_dtype (the product is exact in fp32).
 * bits in {2, 3, 4, 8}; group_size in {32, 64, 128}; k % 32 == 0, k % group_size == 0 and
 * n*bits % 32 == 0 (QL_ERR_SHAPE).  Word arrays 4-byte aligned, 16-bit arrays 2-byte aligned. */
ql_status qlinear_transcode_gptq(const uint32_t* qweight, const uint32_t* qzeros, const void* scales,
                                 ql_dtype scale_dtype, int64_t k, int64_t n, int bits, int group_size,
                                 int v1_zeros, uint32_t* packed, void* scales_out, void* biases_out,
                                 void* stream);

/* GPTQ_P (planar GPTQ) -> MLX affine rows (GPTQModel "Packing Formats and Compatibility",
 * GPTQ_P; GPTQModel wiki "MLX Apple Silicon", Packed layouts and exact transcoding):
 *   in:  qweight [k*bits/32, n] uint32 (output column j's codes down the input axis as planar
 *        blocks: every 32 codes take bits adjacent words holding the bit planes, low plane first,
 *        plane widths the powers of two in bits (3 = 2+1, 5 = 4+1, 6 = 4+2, 7 = 4+2+1), fields
 *        least significant first), qzeros [k/group_size, n*bits/32] (each group's true zero
 *        points as planar blocks along the outputs; no v1 form), scales [k/group_size, n] in
 *        scale_dtype; the value is scale * (code - zero).
 *   out: packed [n, k*tb/32] (tb = 8 for bits = 7, else bits), scales_out [n, k/group_size],
 *        biases_out [n, k/group_size] = RNE(-zero * scale) in scale_dtype.
 * bits in 2..8 (at 2, 4 and 8 the words equal GPTQ's continuous ones); group_size in {32, 64,
 * 128}; k and n multiples of 32, k a multiple of group_size (QL_ERR_SHAPE).  Word arrays 4-byte
 * aligned, 16-bit arrays 2-byte aligned, all device memory; outputs must not overlap inputs. */
ql_status qlinear_transcode_gptq_planar(const uint32_t* qweight, const uint32_t* qzeros, const void* scales,
                                        ql_dtype scale_dtype, int64_t k, int64_t n, int bits, int group_size,
                                        uint32_t* packed, void* scales_out, void* biases_out, void* stream);

/* Host-side check of a GPTQ / GPTQ_P g_idx (GPTQModel "Packing Formats and Compatibility",
 * g_idx: the input-channel-to-group map, and the exact affine holder's contract that it be
 * arange(k) / group_size, activation order not dropped silently): g_idx is int32 [k] in HOST
 * memory.  Returns QL_OK when g_idx[i] == i / group_size for every i, QL_ERR_UNSUPPORTED
 * (naming the first row that differs) for an activation-order map, which the transcoders cannot
 * express; launches nothing and touches no device. */
ql_status qlinear_gptq_check_g_idx(const int32_t* g_idx, int64_t k, int group_size);

/* AWQ GEMM -> MLX affine rows (GPTQModel wiki "MLX Apple Silicon", Packed layouts and exact
 * transcoding, the AWQ GEMM and seven-bit rows, and ParoQuant for the lane order; GPTQModel
 * "Packing Formats and Compatibility", AWQ GEMM):
 *   in:  qweight [k, n*bits/32] uint32 (input row i's codes as one little-endian bits-wide stream
 *        along the outputs; at 4 bits the nibbles of each word hold, from the low one up, columns
 *        0, 2, 4, 6, 1, 3, 5, 7 of its 8), qzeros [k/group_size, n*bits/32] (true zero points,
 *        packed the same way), scales [k/group_size, n] in scale_dtype; the AWQ value is
 *        scale * (code - zero).
 *   out: packed [n, k*tb/32] (the affine row streams, tb = 8 for bits = 7 (the code values kept
 *        in 8-bit rows), tb = bits otherwise), scales_out [n, k/group_size] (transposed),
 *        biases_out [n, k/group_size] = RNE(-zero * scale) in scale_dtype.
 * bits in {2, 3, 4, 5, 6, 7, 8}; group_size in {32, 64, 128}; k and n multiples of 32, k a
 * multiple of group_size (QL_ERR_SHAPE).  Word arrays 4-byte aligned, 16-bit arrays 2-byte
 * aligned, all device memory; the outputs must not overlap the inputs. */
ql_status qlinear_transcode_awq(const uint32_t* qweight, const uint32_t* qzeros, const void* scales,
                                ql_dtype scale_dtype, int64_t k, int64_t n, int bits, int group_size,
                                uint32_t* packed, void* scales_out, void* biases_out, void* stream);

/* dequant (Nx_quant Products, dequant): every value of W as a float32 value, rounded once to
 * out_dtype (QL_F32, QL_F16 or QL_BF16).  out is [rows, k].
 *   QL_AFFINE: w0 = packed [rows, k*bits/32], w1 = scales, w2 = biases [rows, k/group_size] in
 *              param_dtype; value = fl32(code*scale + bias).
 *   QL_MXFP4:  w0 = codes [rows, k/2] (value 2i in byte i's low nibble, 2i+1 in its high one),
 *              w1 = E8M0 scale bytes [rows, k/32]; value = e2m1(code) * 2^(s-127), NaN for
 *              s == 255, -0 for code 8 (Nx_quant Weights, Mxfp4).  bits/group_size/param_dtype
 *              are ignored; w2 must be NULL.
 *   QL_Q8_0:   w0 = blocks [rows, k/32*34] (little-endian fp16 d, then 32 int8), value = d*q
 *              (Nx_quant Weights, Q8_0).  w1 and w2 must be NULL.
 *   QL_MXFP4_BLOCKS: w0 = GGUF blocks [rows, k/32*17]: per 32 values the E8M0 scale byte, then
 *              16 bytes, byte j holding value j in its low nibble and value j + 16 in its high one
 *              (Nx_quant Weights, Mxfp4_blocks); values as QL_MXFP4.  w1 and w2 must be NULL; w0
 *              needs no alignment.
 *   QL_Q4_K:   w0 = blocks [rows, k/256*144] (Nx_quant Weights, Q4_K: fp16 d and dmin, 12 bytes of
 *              6-bit sub-block scales and mins, 128 bytes of 4-bit quants, placed as ggml's
 *              block_q4_K), value = d*sc*q - dmin*m with exact products and one rounding at the
 *              subtraction.  w0 16-byte aligned; w1 and w2 must be NULL.
 *   QL_Q6_K:   w0 = blocks [rows, k/256*210] (Nx_quant Weights, Q6_K: 128 bytes of low 4 bits, 64
 *              of high 2 bits, 16 int8 scales, fp16 d, placed as ggml's block_q6_K), value =
 *              d*sc*(q - 32), exact (-0 from a zero block).  w0 2-byte aligned; w1, w2 NULL.
 *              For both, k % 256 == 0.
 * For the block formats, `rows` may count the rows of a whole expert stack ([e*n]). */
ql_status qlinear_dequant(ql_format fmt, const void* w0, const void* w1, const void* w2,
                          ql_dtype param_dtype, int64_t rows, int64_t k, int bits,
                          int group_size, void* out, ql_dtype out_dtype, void* stream);

/* Decode GEMV (Nx_quant Products, apply; GPTQModel wiki "MLX Apple Silicon", Executing MLX
 * qlinear kernels: FP32 accumulation, output in the activation dtype):
 * y[m,n] = RNE_y( sum_k x[m,k]*(code*scale + bias) [+ layer_bias[n]] ), summed in fp32 straight
 * from the packed words (no stored decoded weight).  Built for small m (1..8); any m >= 0 works
 * (m > 8 runs in slices of 8).  x_dtype in {QL_F16, QL_BF16}; layer_bias (nullable) has x_dtype;
 * y_dtype in {QL_F32, QL_F16, QL_BF16}.  bits in {2, 3, 4, 5, 6, 8}; group_size in {32, 64, 128}. */
ql_status qlinear_gemv(const void* x, ql_dtype x_dtype, int64_t m, int64_t k,
                       const uint32_t* packed, const void* scales, const void* biases,
                       ql_dtype param_dtype, int64_t n, int bits, int group_size,
                       const void* layer_bias, void* y, ql_dtype y_dtype, void* stream);

/* Prefill GEMM: the same product as qlinear_gemv (Nx_quant Products, apply: fp32 accumulation,
 * one rounding to y_dtype), for large m, on the matrix cores.  Each weight is dequantized in
 * registers and rounded once to fp16, and x enters as fp16 after an exact power-of-two scaling
 * per row; the fp16 MFMA accumulates in fp32 (error ~1.5e-4 relative per output row, from the
 * fp16 rounding of the weights).  Needs a device workspace of
 * qlinear_gemm_workspace_size(m, n, k, bits, group_size) bytes (16-byte aligned), overwritten by the
 * call: the fp16 copy of x (m rows of k rounded up to a multiple of 64 values), its m row factors
 * (floats), per-group records of the weight's scales and biases (n * k/group_size pairs of
 * floats) and n row factors, each padded to 256 bytes, and, when the output has too few 256 x 128
 * tiles to fill the chip (fewer than 128), fp32 partial products of the k-ranges the call splits
 * the sum into (2 to 4 ranges: that many m x n floats), summed by a second pass in a fixed order
 * (results do not depend on timing).  At 2, 3, 5 and 6 bits the workspace also holds the codes
 * re-packed as one byte each (n * k bytes, the 8-bit layout), which the 8-bit kernel then reads.
 * The fp16 copy of x, the packed words and those bytes must each be smaller than 2 GiB
 * (QL_ERR_UNSUPPORTED otherwise).  bits in {2, 3, 4, 5, 6, 8}; group_size in {32, 64, 128}. */
size_t qlinear_gemm_workspace_size(int64_t m, int64_t n, int64_t k, int bits, int group_size);
ql_status qlinear_gemm(const void* x, ql_dtype x_dtype, int64_t m, int64_t k,
                       const uint32_t* packed, const void* scales, const void* biases,
                       ql_dtype param_dtype, int64_t n, int bits, int group_size,
                       const void* layer_bias, void* y, ql_dtype y_dtype, void* workspace,
                       size_t ws_bytes, void* stream);

/* One weight of qlinear_gemm_grouped: its own packed words, scales, biases (device memory), optional
 * layer bias, output y [m, n] and row count n.  The weights share k, bits, group_size and dtypes. */
typedef struct {
  const uint32_t* packed;
  const void* scales;
  const void* biases;
  const void* layer_bias;
  void* y;
  int64_t n;
} ql_gemm_weight;

/* Prefill GEMM of up to four weights that read the same x (the projections one layer input feeds,
 * such as q, k and v, or gate and up): y_j = x . dequant(W_j)^T for each, the product of
 * qlinear_gemm (Nx_quant Products, apply), with x converted once and one launch over the tiles of
 * every weight, so that small weights do not need a launch of their own (at 2, 3, 5 and 6 bits
 * each weight's codes are first written as bytes into the workspace and the launch takes them as
 * 8-bit codes).  Each y_j equals what qlinear_gemm gives for W_j alone whenever that call runs on
 * the same kernel (enough output tiles: then the grouped call always does); at other shapes the
 * call runs qlinear_gemm once per weight.  Arguments as qlinear_gemm; count in [0, 4]; the
 * workspace is qlinear_gemm_grouped_workspace_size bytes, 16-byte aligned. */
size_t qlinear_gemm_grouped_workspace_size(int64_t m, int64_t k, const ql_gemm_weight* weights, int count,
                                           int bits, int group_size);
ql_status qlinear_gemm_grouped(const void* x, ql_dtype x_dtype, int64_t m, int64_t k,
                               const ql_gemm_weight* weights, int count, ql_dtype param_dtype, int bits,
                               int group_size, ql_dtype y_dtype, void* workspace, size_t ws_bytes,
                               void* stream);

/* A list of independent GEMVs (each m <= 8) in one launch per class of (row-count template
 * 1/2/4/8, bits); bits and group_size may differ between problems (a problem at 2, 3, 5 or 6 bits
 * whose k is not a positive multiple of 128 runs in a launch of its own, as qlinear_gemv runs it,
 * with no table entry).  `probs` is HOST memory
 * (count entries), validated on the host like qlinear_gemv; the device table built from it (the
 * problems and their row tiles) is written to `workspace` (device memory of at least
 * qlinear_gemv_batched_workspace_size(probs, count) bytes, which depends on the shapes).
 * upload != 0 enqueues the copy of the table to the workspace on `stream` (it travels inside the
 * arguments of small copy launches, so the call neither waits nor keeps any host memory, and it
 * may be captured into a graph); upload == 0 reuses the table an earlier call with the SAME list
 * left in the same workspace (the caller guarantees it is unchanged), so only the product
 * launches are enqueued.  The dtypes are shared by the whole list.
 * No page defines a list form: each problem is the product of qlinear_gemv (Nx_quant Products,
 * apply), and the list is this library's way to run a whole decode step's projections in one
 * launch per class instead of one short launch each. */
size_t qlinear_gemv_batched_workspace_size(const ql_problem* probs, int count);
ql_status qlinear_gemv_batched(const ql_problem* probs, int count, ql_dtype x_dtype,
                               ql_dtype param_dtype, ql_dtype y_dtype, void* workspace,
                               size_t ws_bytes, int upload, void* stream);

/* Routing (Nx_quant Products, apply_experts): group positions p of ids[n_pos] (int64) by expert.
 * offsets[e+1] (int32) gets the exclusive prefix of the per-expert counts; perm[n_pos] (int32)
 * gets, expert by expert, the positions with that id in increasing p (a stable counting sort);
 * ids outside [0, e) are dropped and perm[offsets[e] .. n_pos) is left unwritten.
 * Requires e <= 4096 and n_pos < 2^31. */
ql_status qlinear_route(const int64_t* ids, int64_t n_pos, int64_t e, int32_t* offsets,
                        int32_t* perm, void* stream);

/* Routed apply (Nx_quant Products, apply_experts): for each position p of ids[n_pos],
 * y[p, :] = RNE_y( x[p / pos_per_row, :] . W_{ids[p]}^T ) summed in fp32, or zeros when
 * ids[p] is not in [0, e).  A row's bits do not depend on the other positions' experts.
 *   QL_MXFP4: w0 = codes [e, n, k/2], w1 = scales [e, n, k/32].
 *   QL_MXFP4_BLOCKS: w0 = GGUF blocks [e, n, k/32*17] (any alignment), w1 = NULL; values as QL_MXFP4.
 *   QL_Q8_0:  w0 = blocks [e, n, k/32*34], w1 = NULL.
 *   QL_Q4_K:  w0 = blocks [e, n, k/256*144] (16-byte aligned), w1 = NULL; k % 256 == 0.
 *   QL_Q6_K:  w0 = blocks [e, n, k/256*210] (2-byte aligned), w1 = NULL; k % 256 == 0.
 *             (Nx_quant Weights, Q4_K / Q6_K; the codes enter the products exactly and each
 *             sub-block's fp32 sum is scaled by d*sc, plus -dmin*m times its sum of x for Q4_K.)
 * x is [n_pos / pos_per_row, k] (pos_per_row divides n_pos; a token's top-k slots share its row);
 * x_dtype is QL_BF16 or QL_F16 (Nx_quant Products, apply_experts: any float x).  MXFP4 values are
 * exact in bf16 and meet bf16 x directly; fp16 x enters as the exact sum of two bf16 parts (top 8
 * significant bits, then the other 3), each through the bf16 products.  Q8_0 takes fp16 products
 * (bf16 x converted after an exact power-of-two scaling per row, fp16 x as it is); Q4_K and Q6_K
 * codes are exact in both 16-bit types and meet x in its own dtype's products; y is
 * [n_pos, n] in y_dtype.  k % 32 == 0; 0 <= e <= 4096.  Needs a workspace of
 * qlinear_apply_experts_workspace_size(n_pos, e) bytes (routing scratch: offsets then perm,
 * as qlinear_route writes them, each padded to 16 bytes, then the e experts in decreasing order
 * of their position counts, padded to 16 bytes, then two floats per x row: the power-of-two
 * factors of its f16 conversion for Q8_0). */
size_t qlinear_apply_experts_workspace_size(int64_t n_pos, int64_t e);
ql_status qlinear_apply_experts(ql_format fmt, const void* w0, const void* w1, int64_t e,
                                int64_t n, int64_t k, const int64_t* ids, int64_t n_pos,
                                const void* x, ql_dtype x_dtype, int64_t pos_per_row, void* y,
                                ql_dtype y_dtype, void* workspace, size_t ws_bytes, void* stream);

/* qlinear_apply_experts for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments and results,
 * but the routing scratch (offsets, permutation, expert order, x row factors: the workspace of
 * qlinear_apply_experts_workspace_size(n_pos, e) bytes) lives in a device array built into the
 * library, QL_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends.  The call allocates
 * nothing.  Sizes that need more scratch than that return QL_ERR_UNSUPPORTED (about 87,000
 * positions with 32 experts).  Every call on one GPU shares that GPU's array: calls that overlap on
 * one GPU (on different streams, or from several threads) race and must be ordered by the
 * caller; calls on one stream are ordered by it. */
#define QL_NOALLOC_SCRATCH_BYTES (1u << 20)
ql_status qlinear_apply_experts_noalloc(ql_format fmt, const void* w0, const void* w1, int64_t e,
                                        int64_t n, int64_t k, const int64_t* ids, int64_t n_pos,
                                        const void* x, ql_dtype x_dtype, int64_t pos_per_row, void* y,
                                        ql_dtype y_dtype, void* stream);

/* Message of the last failing call on this thread ("" after a successful call).  Errors name the
 * offending argument, as the Nx_quant API docs' constructors and products name the part they
 * reject (Weights; Products, "Raises Invalid_argument ... naming the part"). */
const char* qlinear_last_error(void);
/* Library version string. */
const char* qlinear_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QLINEAR_H */
