/*
 * mxq.h -- C ABI of the MI355X (gfx950) microscaling quantize + block-scaled
 * GEMM library (libmxq.so).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers owned by the caller. The library never
 *    allocates, frees or synchronizes; every call validates its arguments on the
 *    host, enqueues its kernels on `stream` (a hipStream_t; NULL = the default
 *    stream) and returns. Scratch memory, where a call needs it, is a
 *    caller-provided device `workspace` of at least mxq_workspace_bytes(...).
 *  - Argument errors are detected before anything is launched and returned as an
 *    mxq_status; nothing is written then. MXQ_ERR_HIP reports a failed launch.
 *  - Zero-sized work (rows, cols, M, N or a group of size 0) is a successful no-op.
 *  - Pointers to element data must be 16-byte aligned; leading dimensions are in
 *    elements and must keep every row 16-byte aligned.
 *  - Inputs must be finite; the bytes produced for NaN/Inf inputs are unspecified.
 *  - Calls on different streams may run concurrently; calls that share an
 *    output or workspace buffer must be ordered by the caller.
 *
 * Formats (all bit-exact against the definitions below)
 * -----------------------------------------------------
 *  E4M3 : OCP FP8 "fn" (bias 7, max 448, no Inf, S.1111.111 = NaN, never produced).
 *  E8M0 : unsigned exponent byte, value 2^(s-127); 0xFF (NaN) is never produced.
 *  E2M1 : 4-bit float, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}, bit 3 = sign;
 *         two per byte, element 2j in the low nibble of byte j.
 *  Rounding: round-to-nearest-even onto the target grid, saturating at the largest
 *  finite magnitude, sign of zero kept. All FP32 arithmetic is IEEE binary32 with
 *  correctly rounded division and no flush-to-zero (no fast math).
 *
 *  Scale layouts are canonical row-major matrices (no swizzle): the scale of the
 *  block holding element (r, c) sits at s[r * (cols / B) + c / B], B = 32 (MXFP8,
 *  MXFP4) or 16 (NVFP4). mxq_scale_bytes() returns that size.
 *
 * Sources: "Miles Blackwell RL Cambia la Uniformidad BF16 por MXFP8 y NVFP4
 * Nativos" (remio.ai); "NVIDIA presenta una metodologia de preentrenamiento de 4
 * bits utilizando NVFP4" (7minutos.es); "Miles Blackwell MXFP8/NVFP4 RL recipes"
 * (aib.vote). Each declaration names the passage that defines its operation.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXQ_ABI_VERSION 1

typedef enum {
  MXQ_OK = 0,
  MXQ_ERR_NULL = 1,      /* a required pointer is NULL                        */
  MXQ_ERR_SHAPE = 2,     /* negative size, or a size not a multiple of a block */
  MXQ_ERR_ALIGN = 3,     /* pointer or leading dimension misaligned            */
  MXQ_ERR_FORMAT = 4,    /* unsupported format / scope / option combination    */
  MXQ_ERR_WORKSPACE = 5, /* workspace NULL or smaller than required            */
  MXQ_ERR_HIP = 6        /* a HIP launch failed                                */
} mxq_status;

/* MXQ_BF16_NVFP4T: grouped GEMMs only -- BF16 activations times the stacked NVFP4 expert
 * weights of the forward pass, read transposed (see grouped_gemm_block_scaled). */
typedef enum { MXQ_MXFP8 = 1, MXQ_NVFP4 = 2, MXQ_BF16 = 3, MXQ_MXFP4 = 4, MXQ_BF16_NVFP4T = 5 } mxq_format;
typedef enum { MXQ_OUT_BF16 = 0, MXQ_OUT_F32 = 1 } mxq_out_dtype;

/* Scope of an NVFP4 FP32 (second-level) scale.
 *  ROW    : one scale per row (per token for activations), t has `rows` entries;
 *  TENSOR : one scale for the whole tensor, t has 1 entry;
 *  GROUP  : one scale per group of `group_rows` consecutive rows (one expert
 *           matrix of a stacked (G, N, K) weight), t has rows / group_rows entries. */
typedef enum { MXQ_SCOPE_ROW = 0, MXQ_SCOPE_TENSOR = 1, MXQ_SCOPE_GROUP = 2 } mxq_scope;

/* ---------------------------------------------------------------------------
 * quantize_mxfp8 -- MXFP8 quantization of a BF16 (rows, cols) row-major tensor
 * into a rowwise 1x32 copy and/or a columnwise 32x1 copy, both made from the
 * original BF16 values in one pass over HBM.
 *   Defined by: every 32 consecutive E4M3 values share one E8M0 scale ("Miles
 *   Blackwell RL", remio.ai, section "La Compatibilidad de Miles Blackwell Ahora
 *   Abarca Todo el Ciclo de RL"); rowwise and columnwise copies, because the
 *   blocks must follow each GEMM's reduction dimension (same page, section "Un
 *   Cuantizador Compartido Es el Mecanismo Real"; aib.vote, MXFP8 paragraph).
 *   Scale rule: s = clamp(e + 127, 0, 254) with e the smallest integer such that
 *   amax <= 448 * 2^e (s = 0 for an all-zero block); q = RNE_sat_E4M3(x * 2^(127-s)).
 *
 *   x      : BF16, element (r, c) at x[r * ld_x + c]; ld_x >= cols, ld_x % 8 == 0.
 *   q_row  : E4M3 (rows, cols) row-major;  s_row : E8M0 (rows, cols/32).
 *   q_colT : E4M3 (cols, rows): q_colT[c * rows + r] encodes x(r, c) -- the
 *            columnwise copy stored transposed, so it is K-contiguous for dgrad
 *            and wgrad;  s_colT : E8M0 (cols, rows/32).
 *   Either output pair may be NULL to skip that copy (not both).
 *   Requires cols % 32 == 0, and rows % 32 == 0 when the columnwise copy is
 *   requested.
 * ------------------------------------------------------------------------- */
mxq_status quantize_mxfp8(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                          void* q_row, void* s_row, void* q_colT, void* s_colT,
                          void* stream);

/* ---------------------------------------------------------------------------
 * quantize_mxfp8_multi -- quantize_mxfp8 over several tensors in one launch (e.g.
 * the input, weight and output gradient of a linear layer, whose fprop, dgrad and
 * wgrad GEMMs need all six copies): the same operation and output bytes as
 * `count` calls of quantize_mxfp8, with one kernel launch instead of `count`.
 *   Defined by: as quantize_mxfp8 (remio.ai, sections "La Compatibilidad ..." and
 *   "Un Cuantizador Compartido Es el Mecanismo Real").
 *   tensors : HOST array of `count` descriptors (1 <= count <= MXQ_MXFP8_MULTI_MAX);
 *             each descriptor's fields follow quantize_mxfp8's arguments. All
 *             tensors must request the same copies (rowwise, columnwise or both),
 *             else MXQ_ERR_FORMAT. Any invalid descriptor fails the whole call
 *             before anything is launched; empty tensors (rows or cols 0) are
 *             skipped without looking at their pointers.
 * ------------------------------------------------------------------------- */
#define MXQ_MXFP8_MULTI_MAX 8
typedef struct {
  const void* x;
  int64_t rows, cols, ld_x;
  void* q_row;
  void* s_row;
  void* q_colT;
  void* s_colT;
} mxq_mxfp8_tensor;
mxq_status quantize_mxfp8_multi(const mxq_mxfp8_tensor* tensors, int count, void* stream);

/* ---------------------------------------------------------------------------
 * quantize_mxfp4 -- MXFP4 quantization (E2M1 elements, one E8M0 scale per 32) of a
 * BF16 (rows, cols) tensor into a rowwise 1x32 and/or a columnwise 32x1 copy, in
 * one pass over HBM.
 *   Defined by: MXFP4 blocks of 32 E2M1 values sharing a power-of-two UE8M0 scale,
 *   the format NVFP4 is compared with (7minutos.es, sections "Que es realmente
 *   NVFP4" and "NVFP4 frente a MXFP4").
 *   Scale rule (as for MXFP8, with the E2M1 maximum 6): s = clamp(e + 127, 0, 254),
 *   e the smallest integer with amax <= 6 * 2^e (s = 0 for an all-zero block);
 *   q = RNE_sat_E2M1(x * 2^(127-s)).
 *
 *   x      : BF16, element (r, c) at x[r * ld_x + c]; ld_x >= cols, ld_x % 8 == 0.
 *   q_row  : packed E2M1 (rows, cols/2);  s_row : E8M0 (rows, cols/32).
 *   q_colT : packed E2M1 (cols, rows/2), the columnwise copy stored transposed
 *            (element (r, c) of x is element r of row c);  s_colT : E8M0 (cols, rows/32).
 *   Either output pair may be NULL to skip that copy (not both). Requires
 *   cols % 32 == 0, and rows % 32 == 0 when the columnwise copy is requested.
 * ------------------------------------------------------------------------- */
mxq_status quantize_mxfp4(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                          void* q_row, void* s_row, void* q_colT, void* s_colT,
                          void* stream);

/* ---------------------------------------------------------------------------
 * quantize_mxfp4_multi -- quantize_mxfp4 over several tensors in one launch (the
 * same bytes as `count` calls of quantize_mxfp4).
 *   Defined by: as quantize_mxfp4 (7minutos.es, sections "Que es realmente NVFP4" and
 *   "NVFP4 frente a MXFP4").
 *   tensors : HOST array of `count` mxq_mxfp8_tensor descriptors (the descriptor of
 *             quantize_mxfp8_multi; q_row and q_colT receive packed E2M1), with the
 *             same rules: 1 <= count <= MXQ_MXFP8_MULTI_MAX, one set of copies for
 *             all tensors, validation before any launch, empty tensors skipped.
 * ------------------------------------------------------------------------- */
mxq_status quantize_mxfp4_multi(const mxq_mxfp8_tensor* tensors, int count, void* stream);

/* ---------------------------------------------------------------------------
 * quantize_fp8_block_act -- blockwise FP8 (DeepSeek-V3 style) of an activation or
 * gradient: E4M3 elements with one FP32 scale per 1 x 128 tile.
 *   Defined by: E4M3 elements, 1 x 128 activation tiles and 128 x 128 weight blocks
 *   with FP32 scales applied in software around the matrix product ("Miles Blackwell
 *   MXFP8/NVFP4 RL recipes", aib.vote, second paragraph; "Miles Blackwell RL",
 *   remio.ai, section "NVFP4 por token cuestiona ..."); gradients in the same 1 x 128
 *   tiles (7minutos.es NVFP4 page, the 12B results paragraph).
 *   Arithmetic (binary32): s = amax / 448 over the tile (s = 0 for an all-zero tile);
 *   q = RNE_sat_E4M3(x / s) (a signed zero when s = 0). Dequantized value q * s.
 *
 *   x      : BF16 (rows, cols), row stride ld_x (ld_x % 8 == 0, cols % 8 == 0).
 *   q_row  : E4M3 (rows, cols), s_row : FP32 (rows, cols/128) -- 1 x 128 tiles along each
 *            row (the operand of fprop / dgrad); requires cols % 128 == 0.
 *   q_colT : E4M3 (cols, rows), s_colT : FP32 (cols, rows/128) -- tiles of 128 down each
 *            column, stored transposed (the operand of a GEMM that reduces over rows,
 *            e.g. wgrad); requires rows % 128 == 0.
 *   Either pair may be NULL (not both); both copies come from one read of x.
 * ------------------------------------------------------------------------- */
mxq_status quantize_fp8_block_act(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                  void* q_row, float* s_row, void* q_colT, float* s_colT, void* stream);

/* ---------------------------------------------------------------------------
 * quantize_fp8_block_weight -- blockwise FP8 of a weight: E4M3 elements with one FP32
 * scale per 128 x 128 block, as a row copy and/or a transposed copy with the same
 * codes (the forward GEMM and the transposed backward GEMM read one quantized weight).
 *   Defined by: as quantize_fp8_block_act (aib.vote, second paragraph; remio.ai,
 *   section "NVFP4 por token cuestiona ...").
 *   Arithmetic as quantize_fp8_block_act with the amax over the 128 x 128 block.
 *
 *   x      : BF16 (rows, cols), row stride ld_x; rows % 128 == cols % 128 == 0.
 *   q_row  : E4M3 (rows, cols);  s_row : FP32 (rows/128, cols/128).
 *   q_colT : E4M3 (cols, rows) = the transpose;  s_colT : FP32 (cols/128, rows/128).
 *   Either pair may be NULL (not both).
 * ------------------------------------------------------------------------- */
mxq_status quantize_fp8_block_weight(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                     void* q_row, float* s_row, void* q_colT, float* s_colT, void* stream);

/* ---------------------------------------------------------------------------
 * quantize_nvfp4_per_token -- NVFP4 with one FP32 scale per token (row),
 * computed online in the same kernel that emits the packed E2M1 values and the
 * E4M3 block scales.
 *   Defined by: E2M1 values with an E4M3 scale per 16 values plus an FP32 scale
 *   ("Miles Blackwell RL", remio.ai, section "La Compatibilidad ..."; 7minutos.es,
 *   section "Que es realmente NVFP4"); the FP32 scale taken per token so a token's
 *   bits never depend on the rest of the batch, and one fused operation emitting
 *   packed FP4, block scales and token scales (remio.ai, section "Un Cuantizador
 *   Compartido Es el Mecanismo Real"; aib.vote, per-token paragraph).
 *   Arithmetic (binary32): A = max|x| over the row; s_enc = 2688 / A (1 if A = 0,
 *   FLT_MAX on overflow); t = 1 / s_enc; per 16-block S = RNE_sat_E4M3((a_b / 6)
 *   * s_enc); r = min(s_enc / S, FLT_MAX) (0 if S = 0); q = RNE_sat_E2M1(x * r).
 *
 *   x       : BF16 (tokens, hidden), row stride ld_x elements (ld_x % 8 == 0).
 *   q_packed: uint8 (tokens, hidden/2);  s_block: E4M3 (tokens, hidden/16);
 *   s_token : float (tokens) -- the decode scale t (dequantized x = q * S * t).
 *   Requires hidden % 16 == 0 and hidden <= 16384 (a row is held in the registers of
 *   one wavefront); MXQ_ERR_SHAPE otherwise.
 * ------------------------------------------------------------------------- */
mxq_status quantize_nvfp4_per_token(const void* x, int64_t tokens, int64_t hidden, int64_t ld_x,
                                    void* q_packed, void* s_block, float* s_token,
                                    void* stream);

/* ---------------------------------------------------------------------------
 * quantize_nvfp4 -- general NVFP4 quantizer: any FP32-scale scope, optional
 * transposed (columnwise) blocking and an optional 16-point random Hadamard
 * transform along the quantized axis.
 *   Defined by: the two-level NVFP4 scaling with an FP32 tensor scale (7minutos.es,
 *   section "Que es realmente NVFP4"); joint gate/up scale for SwiGLU experts, i.e.
 *   one scale over the fused gate_up matrix of an expert (remio.ai, section "Un
 *   Cuantizador Compartido ..."); a 16x16 Hadamard matrix times a random +-1 sign
 *   vector applied to the weight-gradient GEMM inputs before quantization
 *   (7minutos.es, section "La metodologia de formacion de cuatro partes").
 *   RHT of a 16-chunk v: w = signs * v; Sylvester-order fast Walsh-Hadamard
 *   transform in binary32 (stages 1, 2, 4, 8; (a, b) -> (a + b, a - b)); u = w / 4.
 *   Scope amax is taken over the transformed values.
 *
 *   x          : BF16 (rows, cols), row stride ld_x. The input is BF16 only: the
 *                tensors this path quantizes (activations, weights, gradients, the
 *                SwiGLU output) are all BF16 on it, so no FP32-input variant exists.
 *   scope      : ROW / TENSOR / GROUP (group_rows consecutive rows share a scale;
 *                with transpose = 1 a group is group_rows consecutive COLUMNS of x,
 *                i.e. rows of the transposed output).
 *   transpose  : 0 -> blocks along each row; outputs (rows, cols/2), (rows, cols/16).
 *                1 -> blocks along each column, stored transposed; outputs
 *                (cols, rows/2), (cols, rows/16).
 *   rht_signs16: HOST pointer to 16 int8 values, each +1 or -1; NULL = no transform.
 *   q, s, t    : packed E2M1, E4M3 block scales, FP32 decode scales (count per scope).
 *   workspace  : device scratch of mxq_workspace_bytes(MXQ_OP_QUANTIZE_NVFP4,
 *                rows, cols, scope-count) bytes (TENSOR and GROUP scopes; NULL
 *                allowed for ROW).
 *   Requires the blocked axis % 16 == 0; with transpose = 1 also cols % 8 == 0;
 *   with transpose = 0 and scope ROW, cols <= 16384 (as quantize_nvfp4_per_token).
 * ------------------------------------------------------------------------- */
mxq_status quantize_nvfp4(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                          mxq_scope scope, int64_t group_rows, int transpose,
                          const int8_t* rht_signs16,
                          void* q, void* s, float* t,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * quantize_nvfp4_stochastic -- quantize_nvfp4 with the E2M1 elements rounded
 * stochastically (for gradient tensors); scales are computed exactly as there.
 *   Defined by: stochastic rounding of gradients -- rounding probabilistically by
 *   the distance to the two nearest representable values removes the bias of
 *   round-to-nearest-even; it is applied to gradients only (7minutos.es, section
 *   "La metodologia de formacion de cuatro partes").
 *   Rounding of p = x * r: m = |p| lies between E2M1 neighbours lo < hi (m >= 6
 *   gives 6); f = (m - lo) / (hi - lo); the element rounds up iff
 *   (word >> 8) < f * 2^24, where word is the 32-bit random word of the element:
 *   element idx of the OUTPUT tensor (row-major, idx = r_out * cols_out + c_out)
 *   takes word idx % 4 of Philox4x32-10 (Salmon et al., SC 2011) with counter
 *   (idx / 4 low 32 bits, high 32 bits, 0, 0) and key (seed low, seed high).
 *   Same seed and shape => same bytes. Arguments otherwise as quantize_nvfp4.
 * ------------------------------------------------------------------------- */
mxq_status quantize_nvfp4_stochastic(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                     mxq_scope scope, int64_t group_rows, int transpose,
                                     const int8_t* rht_signs16, uint64_t seed,
                                     void* q, void* s, float* t,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * quantize_nvfp4_2d -- NVFP4 for weights with one E4M3 scale per 16x16 block
 * (plus the FP32 scope scale), so that the forward pass and the transposed
 * backward pass consume the same quantized weight.
 *   Defined by: 2D block scaling of the weights -- 1x16 blocks along the dot
 *   product would give the forward and the transposed backward different
 *   quantized weights; 16x16 blocks make both use one representation, while
 *   activations and gradients keep 1x16 blocks (7minutos.es, section "La
 *   metodologia de formacion de cuatro partes").
 *   Arithmetic: as quantize_nvfp4 with the block amax taken over each 16x16
 *   block: A = scope amax; s_enc = 2688 / A (1 if A = 0, FLT_MAX on overflow);
 *   t = 1 / s_enc; S = RNE_sat_E4M3((a_b / 6) * s_enc); r = min(s_enc / S,
 *   FLT_MAX) (0 if S = 0); q = RNE_sat_E2M1(x * r). Two passes over x.
 *
 *   x      : BF16 (rows, cols), row stride ld_x; rows % 16 == cols % 16 == 0,
 *            cols <= 16384.
 *   scope  : TENSOR, or GROUP (group_rows consecutive rows = one expert matrix,
 *            group_rows % 16 == 0).
 *   q_row, s_row   : packed (rows, cols/2) and E4M3 (rows, cols/16) -- the 1x16
 *                    form a K-contiguous GEMM reads (each 16x16 block's code
 *                    repeated on its 16 rows); both NULL = skip.
 *   q_colT, s_colT : the transposed weight of each scope group in the same form,
 *                    (groups, cols, group_rows/2) and (groups, cols, group_rows/16)
 *                    (TENSOR: (cols, rows/2), (cols, rows/16)), holding the
 *                    identical codes -- the stacked per-expert layout the grouped
 *                    GEMM reads for dgrad; both NULL = skip.
 *   t      : FP32 decode scale per scope; workspace: mxq_workspace_bytes(
 *            MXQ_OP_QUANTIZE_NVFP4, rows, cols, scopes) bytes.
 * ------------------------------------------------------------------------- */
mxq_status quantize_nvfp4_2d(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                             mxq_scope scope, int64_t group_rows,
                             void* q_row, void* s_row, void* q_colT, void* s_colT, float* t,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * dequantize -- reconstruct BF16 or FP32 values from MXFP8, NVFP4 or MXFP4 data, e.g.
 * the BF16 operands of the dequantized-backward GEMMs.
 *   Defined by: the dequantized-backward mode, whose backward GEMMs run in BF16 on
 *   dequantizations of the exact low-precision forward operands ("Miles Blackwell
 *   RL", remio.ai, section "La Compatibilidad ..."; aib.vote, backward-modes
 *   paragraph).
 *   FP32 output: v = (q * S) * t, one binary32 rounding (q * S is exact; MXFP8 and
 *   MXFP4 have no t). BF16 output: that FP32 value rounded to BF16 (RNE). Overflow
 *   gives Inf.
 *
 *   fmt   : MXQ_MXFP8 (q (rows, cols) E4M3, s (rows, cols/32) E8M0, t unused),
 *           MXQ_NVFP4 (q (rows, cols/2), s (rows, cols/16) E4M3, t per t_scope) or
 *           MXQ_MXFP4 (q (rows, cols/2), s (rows, cols/32) E8M0, t unused).
 *   out   : (rows, cols) row-major, BF16 or FP32.
 * ------------------------------------------------------------------------- */
mxq_status dequantize(mxq_format fmt, const void* q, const void* s, const float* t,
                      mxq_scope t_scope, int64_t group_rows, int64_t rows, int64_t cols,
                      void* out, mxq_out_dtype out_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * dequantize_transposed -- dequantize to BF16 and transpose per group, with an
 * optional row gather: the K-contiguous BF16 operands that the dequantized-
 * backward GEMMs consume (dgrad reads each expert weight transposed, wgrad reads
 * gradients and activations with the slots along K).
 *   Defined by: the dequantized-backward mode ("Miles Blackwell RL", remio.ai,
 *   section "La Compatibilidad ..."; aib.vote, backward-modes paragraph); the value
 *   of every element is that of dequantize(..., MXQ_OUT_BF16) above.
 *
 *   out[(g * cols + c) * ld_out + j] = BF16 of input element (g * group_rows + src(j), c)
 *   for g < groups, c < cols, j < out_cols, where src(j) = src_row[j] (DEVICE int32,
 *   out_cols entries; an index outside [0, group_rows) gives a zero element) or j
 *   when src_row is NULL (then out_cols <= group_rows).
 *   fmt  : MXQ_MXFP8, MXQ_NVFP4 (t per t_scope; GROUP uses group_rows) or MXQ_BF16
 *          (q is BF16 data, s and t unused: a plain transpose).
 *   Input rows are (groups * group_rows, cols) in the layouts of dequantize().
 *   Requires cols % 32 (MXFP8) / % 16 (others) == 0, out_cols % 8 == 0,
 *   ld_out >= out_cols with ld_out % 8 == 0, groups <= 65535.
 * ------------------------------------------------------------------------- */
mxq_status dequantize_transposed(mxq_format fmt, const void* q, const void* s, const float* t,
                                 mxq_scope t_scope, int64_t groups, int64_t group_rows, int64_t cols,
                                 const int32_t* src_row, int64_t out_cols, void* out_bf16,
                                 int64_t ld_out, void* stream);

/* ---------------------------------------------------------------------------
 * gemm_block_scaled -- C = (A_hat) (B_hat)^T with FP32 output, both operands
 * K-contiguous ("TN"), scaling blocks along K.
 *   Defined by: microscaling blocks must follow the reduction dimension of the
 *   matrix product, with forward and backward using different orientations
 *   ("Miles Blackwell RL", remio.ai, section "Un Cuantizador Compartido ...");
 *   fprop, dgrad and wgrad GEMMs of linear layers run in the low-precision format
 *   (remio.ai, section "La Compatibilidad ..."; 7minutos.es, section "Que esta
 *   cuantificado y que no").
 *   MXQ_MXFP8: A (M, K) E4M3 + sA (M, K/32) E8M0; B (N, K) + sB (N, K/32); tA/tB unused.
 *              Every E4M3 * 2^(s-127) operand value is formed exactly in BF16 and the
 *              products are accumulated at FP32 precision (see
 *              gemm_mxfp8_matrix_core for the native scaled-FP8 MFMA variant).
 *              Range: a value is exact when its magnitude is below 2^128 and it is a
 *              multiple of 2^-133 (BF16's smallest subnormal). Every operand that
 *              quantize_mxfp8 makes from finite BF16 data below 2^128 meets both (its
 *              codes times 2^(s-127) are multiples of the input's own 2^-133 grid).
 *              Bytes made elsewhere can break the lower bound only with scale codes
 *              s <= 2 and E4M3 subnormal codes (e.g. s = 0, code 0x01 = 2^-136): such
 *              values are rounded to the BF16 grid before the products, and the
 *              accuracy bound below does not cover them.
 *   MXQ_NVFP4: A (M, K/2) packed E2M1 + sA (M, K/16) E4M3 + tA (ROW: M, TENSOR: 1);
 *              B likewise with tB (ROW: N, TENSOR: 1);
 *              C = tA[m] tB[n] * sum_k (qA SA)(qB SB) -- the E4M3-per-16 block
 *              products are formed exactly, then accumulated in FP32.
 *   MXQ_MXFP4: A (M, K/2) packed E2M1 + sA (M, K/32) E8M0; B (N, K/2) + sB (N, K/32);
 *              tA/tB unused. Operand values E2M1 * 2^(s-127) formed exactly (scale
 *              codes s <= 252), products accumulated at FP32 precision.
 *   MXQ_BF16 : A (M, K) BF16, B (N, K) BF16; scales unused.
 *   C[m * ldc + n], ldc >= N, C 4-byte aligned. Accuracy: normwise relative error
 *   <= 2e-5 against the FP64 product of the exact dequantized operands.
 *   Requires K % 32 == 0 (MXFP8, NVFP4, MXFP4), K % 8 == 0 (BF16), and
 *   K <= 2^22 (32-bit operand offsets); MXQ_ERR_SHAPE otherwise.
 * ------------------------------------------------------------------------- */
mxq_status gemm_block_scaled(mxq_format fmt, int64_t M, int64_t N, int64_t K,
                             const void* A, const void* sA, const float* tA, mxq_scope tA_scope,
                             const void* B, const void* sB, const float* tB, mxq_scope tB_scope,
                             float* C, int64_t ldc, void* stream);

/* ---------------------------------------------------------------------------
 * gemm_block_scaled_batch -- up to MXQ_GEMM_BATCH_MAX independent gemm_block_scaled
 * problems of one format in one launch (e.g. the fprop, dgrad and wgrad GEMMs of a
 * linear layer, which all read the quantized copies made once by the quantizer).
 *   Defined by: as gemm_block_scaled (remio.ai, sections "Un Cuantizador Compartido ..."
 *   and "La Compatibilidad ..."; 7minutos.es, section "Que esta cuantificado y que no").
 *   Each problem's C is bit-identical to what gemm_block_scaled writes for it (same
 *   accumulation order). The problems share one launch, longest K first, so one
 *   problem's output stores overlap another's main loop; a problem too small for the
 *   batch's 256 x 256 tiles (fewer than 128 of them) runs as its own launch on the same
 *   stream instead.
 *   problems : HOST array of `count` descriptors (1 <= count <= MXQ_GEMM_BATCH_MAX); each
 *              field follows gemm_block_scaled's argument of the same name (tA/tB and
 *              their scopes are used for MXQ_NVFP4 only, scopes ROW or TENSOR). Problems
 *              with M or N = 0 are skipped; any invalid descriptor fails the whole call
 *              before anything is launched. Output buffers must not overlap.
 * ------------------------------------------------------------------------- */
#define MXQ_GEMM_BATCH_MAX 8
typedef struct {
  int64_t M, N, K;
  const void* A;
  const void* sA;
  const float* tA;
  mxq_scope tA_scope;
  const void* B;
  const void* sB;
  const float* tB;
  mxq_scope tB_scope;
  float* C;
  int64_t ldc;
} mxq_gemm_problem;
mxq_status gemm_block_scaled_batch(mxq_format fmt, const mxq_gemm_problem* problems, int count, void* stream);

/* ---------------------------------------------------------------------------
 * gemm_fp8_blockwise -- C = A_hat B_hat^T (FP32 output, "TN") for blockwise FP8
 * operands, the FP32 scales applied in software around the matrix product.
 *   Defined by: DeepSeek-V3-style FP8 with 128 x 128 weight blocks, 1 x 128 activation
 *   tiles and FP32 scales applied outside the matrix hardware (aib.vote, second
 *   paragraph; remio.ai, section "NVFP4 por token cuestiona ...").
 *   C[m, n] = sum over 128-K blocks kb of sA[m, kb] sB(n, kb) sum_{k in kb} qA[m, k] qB[n, k]:
 *   each block's code products are summed at FP32 precision, scaled by the two FP32
 *   scales and accumulated in FP32.
 *   A  : E4M3 (M, K) + sA FP32 (M, K/128)        (quantize_fp8_block_act layout)
 *   B  : E4M3 (N, K) + sB FP32:
 *          b_blocks = 1: (ceil(N/128), K/128), one per 128 x 128 block (a weight, or the
 *                        transposed copy of one);
 *          b_blocks = 0: (N, K/128), one per row and 128-K tile (an activation).
 *   C[m * ldc + n], ldc >= N. Accuracy: normwise relative error <= 2e-5 against the
 *   FP64 product of the dequantized operands. Requires K % 128 == 0 and K <= 2^22.
 * ------------------------------------------------------------------------- */
mxq_status gemm_fp8_blockwise(int64_t M, int64_t N, int64_t K, const void* A, const float* sA,
                              const void* B, const float* sB, int b_blocks, float* C, int64_t ldc,
                              void* stream);

/* ---------------------------------------------------------------------------
 * gemm_fp8_blockwise_batch -- up to MXQ_GEMM_BATCH_MAX independent gemm_fp8_blockwise
 * problems in one launch (e.g. the fprop, dgrad and wgrad GEMMs of a blockwise-FP8
 * linear layer).
 *   Defined by: as gemm_fp8_blockwise (aib.vote, second paragraph; remio.ai, section
 *   "NVFP4 por token cuestiona ...").
 *   Each problem's C is bit-identical to what gemm_fp8_blockwise writes for it (same
 *   tiles and accumulation order). The problems share one launch, longest K first, so
 *   a problem with few long tiles (a layer's dgrad) runs beside the others' tiles.
 *   problems : HOST array of `count` descriptors (1 <= count <= MXQ_GEMM_BATCH_MAX);
 *              each field follows gemm_fp8_blockwise's argument of the same name.
 *              Problems with M or N = 0 are skipped; any invalid descriptor fails the
 *              whole call before anything is launched (MXQ_ERR_SHAPE / NULL / FORMAT /
 *              ALIGN as for gemm_fp8_blockwise). Output buffers must not overlap.
 * ------------------------------------------------------------------------- */
typedef struct {
  int64_t M, N, K;
  const void* A;
  const float* sA;
  const void* B;
  const float* sB;
  int b_blocks;
  float* C;
  int64_t ldc;
} mxq_fp8_block_problem;
mxq_status gemm_fp8_blockwise_batch(const mxq_fp8_block_problem* problems, int count, void* stream);

/* ---------------------------------------------------------------------------
 * gemm_mxfp8_matrix_core -- MXFP8 GEMM C = A_hat B_hat^T on the gfx950 scaled FP8
 * MFMA, which consumes the E8M0 block scales natively (one byte per row and
 * 32-K block of each operand).
 *   Defined by: block scales along the reduction dimension consumed by the
 *   matrix hardware ("Miles Blackwell RL", remio.ai, section "Un Cuantizador
 *   Compartido Es el Mecanismo Real").
 *   Accumulation (measured on MI355X): each group of 8 consecutive K products is
 *   summed in a fixed-point window ~13 bits below the group's largest product
 *   (lower bits dropped); group sums accumulate at FP32 precision. Within 2e-5
 *   normwise on Gaussian-like blocks; outlier-heavy blocks can exceed it -- use
 *   gemm_block_scaled(MXQ_MXFP8, ...) where the bound must hold for any data.
 *   Operands, layout and alignment as gemm_block_scaled(MXQ_MXFP8, ...).
 * ------------------------------------------------------------------------- */
mxq_status gemm_mxfp8_matrix_core(int64_t M, int64_t N, int64_t K,
                                  const void* A, const void* sA, const void* B, const void* sB,
                                  float* C, int64_t ldc, void* stream);

/* ---------------------------------------------------------------------------
 * grouped_gemm_block_scaled -- one GEMM per routed expert, scheduled on the device
 * from the expert offsets (no host synchronisation on the group sizes).
 *   Defined by: NVFP4 applied to the routed experts' weights and activations of
 *   the MoE layers ("Miles Blackwell RL", remio.ai, section "La Compatibilidad
 *   ..."; aib.vote, NVFP4 paragraph), where moving expert weights through memory
 *   can bind harder than arithmetic (remio.ai, section "NVFP4 por token ...").
 *
 *   vary_k = 0 (fprop / dgrad):  for every group g and slot s in
 *       [offsets[g], offsets[g+1]):  C[s, :] = A_hat[row(s), :] B_hat_g^T
 *     A      : (a_rows, K) operand; row(s) = a_row_index[s] when a_row_index is
 *              non-NULL (gather of token rows into expert order), else s. A gather
 *              index outside [0, a_rows) contributes a zero row (never read).
 *     B      : stacked (groups, N, K) operand; C : (total_slots, N) FP32.
 *     tA     : per A row (ROW) or one (TENSOR); tB : per group (GROUP with
 *              group_rows = N) or per B row (ROW).
 *   vary_k = 1 (wgrad): for every group g:  C_g = sum over k in [offsets[g],
 *       offsets[g+1]) of A[:, k] B[:, k]^T
 *     A : (M, total_k) K-contiguous; B : (N, total_k); C : (groups, M, N).
 *     Group boundaries must be multiples of 32 (MXFP8, MXFP4) or 8 (BF16); MXQ_NVFP4
 *     is not supported with vary_k = 1 in ABI version 1.
 *   vary_k = 2 (wgrad, MXQ_BF16 only): as vary_k = 1, with A given K-major: A is the
 *     (total_k, M) row-major tensor whose transpose vary_k = 1 takes -- the slot-major
 *     output gradient of the expert layer itself, so no transposed copy is needed. M % 8
 *     == 0. Same values bit for bit as vary_k = 1 on the transposed A.
 *   offsets  : DEVICE int64 (groups + 1), non-decreasing, offsets[0] = 0,
 *              offsets[groups] = total (total_slots or total_k, passed as `total`);
 *              with vary_k = 1 every offset is a multiple of 32 (MXFP8, MXFP4) or 8 (BF16).
 *              The device checks this before any tile runs; offsets that break it
 *              make the call a no-op that leaves C unwritten.
 *   fmt = MXQ_BF16_NVFP4T (vary_k = 0, no a_row_index): the dequantized-backward dgrad
 *     straight from the forward's quantized expert weights. A : BF16 (total_slots, K);
 *     B : the stacked NVFP4 weights W_g (K, N) exactly as quantize_nvfp4 (GROUP scope,
 *     group_rows = K) stores them for the forward GEMM -- packed (groups * K, N/2), E4M3
 *     sB (groups * K, N/16), tB (groups) with tB_scope GROUP -- and used transposed:
 *       C[s, n] = sum_k A[s, k] * RNE_bf16(fl32(fl32(q S) t_g))[k, n],
 *     the same BF16 operand values dequantize_transposed writes, built in the GEMM loader
 *     instead of being stored (remio.ai, section "La Compatibilidad ...": backward GEMMs
 *     in BF16 on BF16 dequantizations of the exact forward operands). sA / tA unused.
 *     Requires K % 8 == 0, N % 16 == 0 and K * N / 2 < 2^31.
 *   Limits     : K <= 2^22 (vary_k = 1: total <= 2^22); with a_row_index, a_rows times
 *              the bytes of one A row must stay below 2^31. MXQ_ERR_SHAPE otherwise.
 *   workspace: device scratch of mxq_workspace_bytes(MXQ_OP_GROUPED_GEMM, groups, 0, 0).
 * ------------------------------------------------------------------------- */
mxq_status grouped_gemm_block_scaled(mxq_format fmt, int64_t groups, const int64_t* offsets,
                                     int vary_k, int64_t total, int64_t M, int64_t N, int64_t K,
                                     const int32_t* a_row_index, int64_t a_rows,
                                     const void* A, const void* sA, const float* tA, mxq_scope tA_scope,
                                     const void* B, const void* sB, const float* tB, mxq_scope tB_scope,
                                     float* C, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * grouped_gemm_block_scaled_noalloc -- grouped_gemm_block_scaled without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, and harnesses that forbid allocation.
 *   Same operation, arguments (minus workspace), checks and bytes of C as
 *   grouped_gemm_block_scaled: the same kernels run; only the scratch of the device
 *   tile scheduler ((groups + 1) int64 tile offsets, rewritten in full by every call)
 *   lives in a static device array of the library, one per GPU, held until the
 *   process ends (64 KiB).
 *   groups <= MXQ_NOALLOC_MAX_GROUPS, else MXQ_ERR_WORKSPACE (nothing launched).
 *   The array of the CURRENT device (hipGetDevice) is used: `stream` must belong to
 *   it. Its address is looked up on the first call on each device (MXQ_ERR_HIP if
 *   that fails). No call allocates or frees.
 *   Every call on one GPU shares that GPU's array: calls that can overlap on one GPU
 *   (different streams, or several host threads) race on it and must be ordered by
 *   the caller; calls on one stream are ordered by the stream.
 * ------------------------------------------------------------------------- */
#define MXQ_NOALLOC_MAX_GROUPS 8191
mxq_status grouped_gemm_block_scaled_noalloc(mxq_format fmt, int64_t groups, const int64_t* offsets,
                                             int vary_k, int64_t total, int64_t M, int64_t N, int64_t K,
                                             const int32_t* a_row_index, int64_t a_rows,
                                             const void* A, const void* sA, const float* tA, mxq_scope tA_scope,
                                             const void* B, const void* sB, const float* tB, mxq_scope tB_scope,
                                             float* C, void* stream);

/* ---------------------------------------------------------------------------
 * moe_swiglu_quantize_nvfp4 -- SwiGLU of the gate_up GEMM output followed by
 * per-row NVFP4 quantization of the result (input of the down projection).
 *   Defined by: SwiGLU experts whose gate and up projections enter one fused GEMM
 *   ("Miles Blackwell RL", remio.ai, section "Un Cuantizador Compartido ..."), and
 *   per-token NVFP4 on the expert activations (same page, section "La
 *   Compatibilidad ..."). Each slot row (token, expert) is one scale scope.
 *   h = silu(g) * u = g u / (1 + e^(-g)) (g = row[0:inter], u = row[inter:2*inter]),
 *   rounded once to BF16 (nearest, ties to even) from its exact value, so that no
 *   approximate exponential reaches the FP4 quantizer (remio.ai, section "Un
 *   Cuantizador Compartido ..."): computed in binary64 (relative error below 2^-50)
 *   and rounded to BF16 through a round-to-odd binary32 step; then the per-token
 *   quantizer above on the BF16 row. Both h and the quantized bytes are bit-exact
 *   against the correctly rounded definition (a value within 2^-50 of a BF16 rounding
 *   midpoint is the only case the binary64 evaluation could misplace).
 *
 *   gate_up : FP32 (rows, 2*inter); h_bf16 : optional BF16 (rows, inter) copy of h
 *   (NULL = not written); q (rows, inter/2), s (rows, inter/16), t (rows).
 *   Requires inter % 16 == 0 and inter <= 16384; MXQ_ERR_SHAPE otherwise.
 * ------------------------------------------------------------------------- */
mxq_status moe_swiglu_quantize_nvfp4(const float* gate_up, int64_t rows, int64_t inter,
                                     void* h_bf16, void* q, void* s, float* t, void* stream);

/* ---------------------------------------------------------------------------
 * moe_combine -- y[t, :] = sum_j w[t, j] * O[slot_of[t, j], :] in FP32, j ascending.
 *   The weighted top-k combine that closes a routed-expert layer (remio.ai,
 *   section "NVFP4 por token ...": experts routed per token).
 *   o_slots : FP32 (total_slots, hidden); slot_of : DEVICE int64 (tokens, topk), entries
 *   in [0, total_slots) (others contribute nothing); weights : FP32 (tokens, topk);
 *   y : FP32 (tokens, hidden). hidden % 4 == 0.
 * ------------------------------------------------------------------------- */
mxq_status moe_combine(const float* o_slots, int64_t total_slots, int64_t tokens, int64_t topk,
                       int64_t hidden, const int64_t* slot_of, const float* weights, float* y,
                       void* stream);

/* ---------------------------------------------------------------------------
 * Queries.
 * ------------------------------------------------------------------------- */
/* Bytes of the scale matrix for a (rows, cols) tensor blocked along cols
 * (MXFP8, MXFP4: rows * cols/32, NVFP4: rows * cols/16); 0 for BF16 or bad shapes. */
size_t mxq_scale_bytes(mxq_format fmt, int64_t rows, int64_t cols);

enum { MXQ_OP_QUANTIZE_NVFP4 = 1, MXQ_OP_GROUPED_GEMM = 2 };
/* Workspace bytes for an op:
 *   MXQ_OP_QUANTIZE_NVFP4 (a = rows, b = cols, c = number of FP32 scales);
 *   MXQ_OP_GROUPED_GEMM   (a = groups). */
size_t mxq_workspace_bytes(int op, int64_t a, int64_t b, int64_t c);

const char* mxq_status_string(mxq_status s);
int mxq_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MXQ_H */
