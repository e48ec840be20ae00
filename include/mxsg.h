/*
 * mxsg.h - C ABI of the MI355X (gfx950) quantized MoE expert grouped GEMM.
 *
 * What it computes. The float8 MoE training pages describe one hot path:
 * quantize the routed-row activations, the expert weights and the output
 * gradients to FP8 at run time from their current amax (torchao float8 MoE
 * training PR, Summary), then run a scaled grouped matmul over per-expert
 * token groups for the forward pass and both backward products (the same
 * PR's Testing section checks outputs, input gradients and parameter
 * gradients).
 * Recipes: tensorwise dynamic; delayed with an amax history and the "max"
 * algorithm (Megatron-LM FP8-vs-BF16 MoE bug report, reproduction flags);
 * DeepSeek-style 1x128 / 128x1 / 128x128 blockwise with fp32 scales
 * (Transformer Engine "FP8BlockQuantizer not work" issue, design note);
 * MXFP8 with 32-element blocks and E8M0 scales (Megatron-LM single grouped
 * weight PR, coverage table); the same table's 4-bit rows: MXFP4 (e2m1
 * elements, E8M0 scales) and NVFP4 (e2m1 elements, an e4m3 scale per 16
 * elements and an fp32 scale per tensor). Formats are OCP e4m3, e5m2, e2m1.
 *
 * Shape of the interface. Every call takes a flat argument list (device
 * pointers, sizes, enums) instead of descriptor structs, so that each
 * argument's meaning and ownership is stated where it is declared. The
 * quantization is four calls (token tensors; tokens gathered through a
 * routing index; the SwiGLU activation of a gate/up output; the grouped
 * weight), and the buffer sizes are two pure host queries, one for token
 * tensors and one for weights. One rule is stricter than the MX block size
 * needs: MX feature dimensions must be multiples of 128, not 32, so that
 * one GEMM tile shape serves every recipe.
 *
 * Conventions for every call.
 *  - All array pointers are DEVICE pointers of the current HIP device, owned
 *    by the caller. The library never allocates, frees, copies between host
 *    and device, or synchronizes. Work is enqueued on `stream` (a
 *    hipStream_t passed as void*; NULL = the default stream) and runs in
 *    stream order. Offsets stay on the device; no call reads them on the host.
 *  - bf16 tensors are row-major uint16 bit patterns; FP8 codes are uint8 bit
 *    patterns; fp32 scales are float; E8M0 scales are uint8 (2^(c-127)).
 *  - Return value: MXSG_OK, or an error code and nothing enqueued. Argument
 *    errors are detected on the host before any HIP call; mxsg_last_error()
 *    then gives a message (per thread). A failed launch returns
 *    MXSG_HIP_ERROR.
 *  - Shapes: every feature dimension (C of a token tensor, K and N of a
 *    weight) must be a positive multiple of 128. The token dimension M may
 *    be any value >= 0, and groups may be empty or of any size. (The
 *    blockwise issue's shape rule: the blocked dimension must divide by the
 *    block; its correction: the other dimension is free.)
 *  - Groups: `group_ends` is int32[E] of cumulative row ends, non-decreasing,
 *    with group_ends[E-1] == M (group g = rows [group_ends[g-1],
 *    group_ends[g]), group_ends[-1] = 0). Values outside [0, M] are clamped
 *    on the device and a decreasing end makes that group empty, so malformed
 *    offsets give wrong numbers but never out-of-bounds accesses.
 *
 * Layouts.
 *  - Scale of a scaling unit: s = fp32(amax / fmax) (stored, the multiplier
 *    that dequantizes), codes = sat_rne(fp32(x * inv)), inv = fp32(fmax /
 *    amax); amax == 0 gives s = inv = 1. fmax = 448 (e4m3), 57344 (e5m2).
 *    MX: E8M0 code k+127 with k the smallest integer such that amax <=
 *    fmax * 2^k (clamped to [-127, 127]; 0 for amax == 0), inv = 2^-k.
 *  - 4-bit e2m1 codes (MXFP4) sit two per byte along a row: element 2i in
 *    the low nibble of byte i, element 2i + 1 in the high nibble; a row of
 *    L elements is L/2 code bytes. Sign in bit 3; magnitudes 0, 0.5, 1,
 *    1.5, 2, 3, 4, 6 (OCP MX v1.0 element formats); the MX exponent uses
 *    fmax = 6.
 *  - NVFP4: per tensor (per expert for weights) s_t = fp32(amax / (6 *
 *    448)), or 1 when amax = 0; per 16 consecutive elements along a row,
 *    the block scale code b = e4m3 sat_rne(fp32(fp32(amax_16 / 6) / s_t)),
 *    its multiplier m = fp32(e4m3(b) * s_t), and the element codes
 *    e2m1 sat_rne(fp32(x * inv)) with inv = fp32(1 / m) (0 when m = 0 or
 *    the quotient overflows); the value is e2m1(code) * e4m3(b) * s_t. Element codes sit two per byte
 *    like MXFP4 codes, but inside each 128-element (64-byte) piece of a row
 *    the 8 elements 16 s + 8 h .. 16 s + 8 h + 7 (s = 0..7, h = 0..1) form
 *    the little-endian dword at byte 32 (s / 4) + 16 h + 4 (s % 4) of the
 *    piece (element order within the dword as for MXFP4); pair interleaving
 *    then applies to the code bytes as for every code matrix. A scale
 *    buffer of R rows of L elements holds the R * L/16 block codes
 *    piece-major, byte ((l / 128) * R + r) * 8 + (l % 128) / 16 for element
 *    (r, l), then the fp32 tensor scale (little-endian) at byte R * L/16; a
 *    weight's buffer holds the E experts' block codes one after another,
 *    then the E fp32 tensor scales.
 *  - Code matrices are pair-interleaved: a matrix of R rows of L code bytes
 *    (L a multiple of 64) stores byte (r, l) at offset
 *      (r / 2) * 2L + (l / 64) * 128 + (r % 2) * 64 + (l % 64),
 *    i.e. rows 2p and 2p+1 share 2L bytes as 128-byte lines that each hold
 *    64 bytes of row 2p followed by the same 64 bytes of row 2p+1. R is
 *    rounded up to even: a buffer holds 2 * ceil(R / 2) rows; for odd R the
 *    last row of the last pair is not written and never reaches a result.
 *    This holds for row-wise token codes [M, C], column-wise codes [C, ld]
 *    and each expert's weight codes ([N, K] k-major, [K, N] n-major). The
 *    grouped GEMM reads a 64-byte contraction slice of a run of row pairs
 *    as whole 128-byte lines.
 *  - Column-wise (transposed) token layout, the wgrad operand: codes
 *    [C, ld] where group g's tokens sit at columns [P_g, P_g + m_g),
 *    P_0 = 0, P_{g+1} = P_g + ceil(m_g / 128) * 128, and columns
 *    [P_g + m_g, P_{g+1}) hold code 0x00 (zero fill of partial blocks).
 *    ld must be a multiple of 128 and >= mxsg_padded_capacity(M, E).
 *    Columns >= P_E are not written.
 *  - MX (E8M0) scale matrices are word-major: a matrix of R rows of B
 *    blocks (B = 4 * words, one 32-element block per byte) stores the
 *    scale of (row r, block b) at byte offset
 *      ((b / 4) * R + r) * 4 + (b % 4),
 *    i.e. word w (the four blocks of contraction elements [128w, 128w+128))
 *    of every row, rows consecutive, then word w + 1. The shapes below are
 *    logical [R, B]; each expert's matrix of a weight is its own [R, B]
 *    in this order. The grouped GEMM reads one word for a run of rows as
 *    contiguous memory.
 */
#ifndef MXSG_H
#define MXSG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mxsg_status;
#define MXSG_OK 0
#define MXSG_INVALID_ARGUMENT 1 /* null pointer, bad enum, negative size */
#define MXSG_BAD_SHAPE 2        /* feature dim not a multiple of 128, ld too small, ... */
#define MXSG_UNSUPPORTED 3      /* a recipe / format / mode combination not built */
#define MXSG_HIP_ERROR 4        /* a HIP launch failed */

/*
 * Device status word bits. The quantize and grouped-GEMM calls take an
 * optional `status_word` (device int32, NULL = no checks); the kernels OR
 * these bits into it when they meet a violation that only the device can
 * see. The library never clears the word (the caller zeroes it and reads it
 * whenever it likes, e.g. once per step). A violation never causes an
 * out-of-bounds access: offsets are clamped, non-finite inputs give
 * non-finite scales.
 */
#define MXSG_STATUS_ENDS_DECREASING 1 /* group_ends[g] < group_ends[g-1] for some g (group_ends[-1] = 0) */
#define MXSG_STATUS_ENDS_RANGE 2      /* some group end outside [0, M] */
#define MXSG_STATUS_ENDS_TOTAL 4      /* group_ends[E-1] != M (rows not covered exactly) */
#define MXSG_STATUS_NONFINITE 8       /* an amax reduction met a NaN or Inf input element */
#define MXSG_STATUS_BAD_EXPERT 16     /* mxsg_route met an expert id outside [0, E) */

/* recipes */
#define MXSG_RECIPE_TENSORWISE 0 /* one unit per 2-D tensor (per expert for weights), dynamic amax */
#define MXSG_RECIPE_DELAYED 1    /* as tensorwise, scale taken from a delayed-scaling state */
#define MXSG_RECIPE_BLOCKWISE 2  /* tokens 1x128 rows / 128x1 columns; weights 128x128 tiles */
#define MXSG_RECIPE_MX 3         /* 32-element blocks, E8M0 scales */
#define MXSG_RECIPE_NVFP4 4      /* e2m1 elements; e4m3 scale per 16 elements; fp32 scale per tensor */

/* element formats */
#define MXSG_FMT_E4M3 0
#define MXSG_FMT_E5M2 1
#define MXSG_FMT_E2M1 2 /* OCP MX 4-bit element (MXFP4); MX recipe only, two codes per byte */

/* grouped GEMM modes */
#define MXSG_MODE_FWD 0   /* Y[M,N]    = A[M,K]  x W_g[K,N]   (bf16 out) */
#define MXSG_MODE_DGRAD 1 /* dA[M,K]   = dY[M,N] x W_g[K,N]^T (bf16 out) */
#define MXSG_MODE_WGRAD 2 /* dW[E,K,N] = A_g^T x dY_g         (fp32 out) */

typedef void *mxsg_stream_t; /* hipStream_t */

/* Static text of a status code. */
const char *mxsg_status_str(mxsg_status s);
/* Message of the last error returned on this thread ("" if none). */
const char *mxsg_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int32_t mxsg_version(void);

/* Columns needed by the column-wise layout of M tokens in E groups:
 * the smallest multiple of 128 that is >= max over group sizes of P_E,
 * i.e. 128 * ceil((M + 127 * E) / 128). Pure host function. */
int64_t mxsg_padded_capacity(int64_t M, int32_t E);

/*
 * Byte sizes of the buffers mxsg_quantize_act writes for tokens x [M, C]
 * under `recipe` and element format `fmt`, with the column-wise output laid
 * out for E groups (ld = mxsg_padded_capacity(M, E)); E = 0 asks for the
 * row-wise sizes only. Pure host function: applies the same shape and
 * recipe/format rules as mxsg_quantize_act (C a multiple of 128, M < 2^31,
 * e2m1 only with MX) and returns their status. With b = 1 code byte per
 * element (e4m3, e5m2) or 1/2 (e2m1):
 *   bytes[0] row_codes      (M + (M & 1)) * C * b
 *   bytes[1] row_scales     BLOCKWISE 4 * M * C/128, MX M * C/32 (word-major),
 *                           NVFP4 M * C/16 + 4, else 4
 *   bytes[2] col_codes      C * ld * b               (0 when E = 0)
 *   bytes[3] col_scales     BLOCKWISE 4 * C * ld/128, MX C * ld/32 (word-major),
 *                           NVFP4 C * ld/16 + 4, else 4
 *   bytes[4] padded_starts  4 * (E + 1)              (0 when E = 0)
 * Units and shape rule: the Transformer Engine "FP8BlockQuantizer not
 * work" issue, design note (1x128 units; the blocked dimension divides by
 * the block). The padded token layout of the column-wise output is that
 * note's zero fill of partial blocks.
 */
mxsg_status mxsg_quantize_act_sizes(int64_t M, int64_t C, int32_t recipe, int32_t fmt, int32_t E,
                                    int64_t bytes[5]);

/*
 * Byte sizes of the buffers mxsg_quantize_weight writes for w [E, K, N]
 * (b as above):
 *   bytes[0] kmajor_codes, bytes[2] nmajor_codes   E * K * N * b each
 *   bytes[1] kmajor_scales, bytes[3] nmajor_scales BLOCKWISE 4 * E * K/128 * N/128,
 *                                                  MX E * K * N / 32,
 *                                                  NVFP4 E * K * N / 16 + 4 * E, else 4 * E
 * Pure host function with the shape rules of mxsg_quantize_weight (K, N
 * multiples of 128; 128x128 weight blocks of the same issue's design note).
 */
mxsg_status mxsg_quantize_weight_sizes(int32_t E, int64_t K, int64_t N, int32_t recipe,
                                       int32_t fmt, int64_t bytes[4]);

/*
 * Routing permutation of the MoE dispatch, on the device. expert_ids is
 * int32 [T, k] (device): the k experts token t was routed to (top-k
 * choices, in choice order). Writes
 *   group_ends int32 [E]: cumulative row ends of the expert groups, i.e.
 *     group_ends[e] = number of choices with an id <= e (ids in [0, E));
 *   row_index  int32 [T * k]: routed row i -> its token, rows grouped by
 *     expert in ascending id and, within an expert, in (token, choice)
 *     order (a stable order of the choices by expert id);
 *   slot_row   int32 [T * k] (optional, NULL = not written): choice
 *     t * k + j -> its routed row (the inverse map, for returning expert
 *     outputs to their tokens).
 * The result is the input the grouped GEMM and mxsg_quantize_act_gather
 * take (row_index, group_ends with M = T * k): the pages hand the grouped
 * matmul rows grouped by routed expert with cumulative offsets (torchao
 * float8 MoE training PR, Summary and Limitations; Megatron-LM FP8-vs-BF16
 * MoE bug report, additional context on TEGroupedMLP's per-expert inputs).
 * A choice with an id outside [0, E) is not routed: it sets
 * MXSG_STATUS_BAD_EXPERT in status_word (optional), its slot_row entry is
 * -1, and the rows past group_ends[E-1] are filled with -1 (which the
 * gather quantizer clamps to token 0; those rows lie outside every group).
 * Limits: T * k < 2^31, 1 <= E <= 2^20. Uses no scratch memory.
 */
mxsg_status mxsg_route(const int32_t *expert_ids, int64_t T, int32_t k, int32_t E, int32_t *group_ends,
                       int32_t *row_index, int32_t *slot_row, int32_t *status_word, mxsg_stream_t stream);

/*
 * Quantize a token-major tensor x [M, C] (routed-row activations or output
 * gradients), producing the row-wise operand (forward / dgrad) and/or the
 * column-wise operand (wgrad).
 *
 *  recipe TENSORWISE: amax = max|x| is computed first (written to amax[0],
 *    required), then s and inv. row_scales / col_scales (fp32[1], each
 *    optional) receive s.
 *  recipe DELAYED: quantizes with s = dl_scale[0], inv = dl_inv[0] (state of
 *    mxsg_delayed_update) and max-reduces max|x| into amax[0] (required;
 *    the caller or mxsg_delayed_update must have zeroed it). row_scales /
 *    col_scales (optional) receive a copy of s.
 *  recipe BLOCKWISE: row_scales fp32 [M, C/128] (1x128 units along C);
 *    col_scales fp32 [C, ld/128] (128x1 units along the padded tokens,
 *    restarting at each group). amax, dl_* unused.
 *  recipe MX: row_scales uint8 [M, C/32]; col_scales uint8 [C, ld/32]
 *    (both word-major, R = M resp. C); a
 *    32-block made only of padding gets code 127. fmt e2m1 (MXFP4): the
 *    same scales; code rows hold C/2 resp. ld/2 bytes.
 *  recipe NVFP4 (fmt e2m1 only): amax = max|x| is computed first (amax[0],
 *    required); row_scales / col_scales are NVFP4 scale buffers (Layouts)
 *    of R = M rows of C elements resp. R = C rows of ld elements, the
 *    column-wise 16x1 blocks along the padded tokens starting at each
 *    group's first token (a block of padding only gets block code 0).
 *
 *  row_codes uint8 [2 * ceil(M/2), C] (C/2 for e2m1), pair-interleaved (NULL: no row-wise
 *    output).
 *  col_codes uint8 [C, ld] (ld/2 for e2m1), pair-interleaved (NULL: no column-wise output).
 *    When given, E >= 1,
 *    group_ends and padded_starts (int32 [E+1], receives P_0..P_E) are required.
 *  At least one of row_codes / col_codes must be non-NULL.
 *  status_word (optional, see the status bits): group_ends are checked when
 *    given (E >= 1); every input element passes an amax reduction, which
 *    flags NaN / Inf inputs (out of contract: their codes are undefined).
 */
mxsg_status mxsg_quantize_act(const void *x, int64_t M, int64_t C, int32_t recipe, int32_t fmt,
                              int32_t E, const int32_t *group_ends, void *row_codes,
                              void *row_scales, void *col_codes, void *col_scales, int64_t ld,
                              int32_t *padded_starts, float *amax, const float *dl_scale,
                              const float *dl_inv, int32_t *status_word, mxsg_stream_t stream);

/*
 * mxsg_quantize_act applied to the SwiGLU activation of a gate/up GEMM
 * output, fused so the activation is never written: x is bf16 [M, 2C]
 * (device, row stride 2C); for columns c < C the quantized element is the
 * bf16 value nearest to silu(x[m, c]) * x[m, C + c] (ties to even; the
 * exact real value, so the result is correctly rounded), with
 * silu(g) = g / (1 + exp(-g)): the SwiGLU that Mixtral's experts apply
 * between the two GEMMs (the Megatron-LM FP8-vs-BF16 MoE bug report's
 * model, reproduction steps; the pages print no formula). That bf16 tensor
 * [M, C] is then quantized exactly as mxsg_quantize_act quantizes a bf16
 * tensor: every output, layout, size (mxsg_quantize_act_sizes with C) and
 * rule is that call's. Tensorwise scaling first reads gate and up once to
 * take the activation's amax (written to amax[0]). NaN / Inf inputs follow
 * the formula in IEEE arithmetic (g = -inf gives NaN); the status word's
 * MXSG_STATUS_NONFINITE bit reports a NaN or Inf activation (a non-finite
 * gate/up input, or a product past the bf16 range).
 */
mxsg_status mxsg_quantize_act_swiglu(const void *x, int64_t M, int64_t C, int32_t recipe,
                                     int32_t fmt, int32_t E, const int32_t *group_ends,
                                     void *row_codes, void *row_scales, void *col_codes,
                                     void *col_scales, int64_t ld, int32_t *padded_starts,
                                     float *amax, const float *dl_scale, const float *dl_inv,
                                     int32_t *status_word, mxsg_stream_t stream);

/*
 * mxsg_quantize_act on routed rows gathered from a token tensor: x is
 * [T, C] (one row per token) and routed row i, i < M, is x row
 * row_index[i] (int32 [M], device). This is the MoE dispatch permutation
 * that puts each token's copies in expert order in front of the grouped
 * GEMM (the torchao float8 MoE training PR overrides grouped_mm for the
 * routed experts, Limitations; its offsets imply rows contiguous per
 * expert), fused with the quantization so the permuted bf16 copy is never
 * written. Results equal mxsg_quantize_act on the tensor x[row_index];
 * tensorwise amax is taken over the routed rows only. Indices outside
 * [0, T) are clamped on the device (wrong rows, never out-of-bounds
 * reads); a token may appear any number of times or not at all. Every
 * other argument, output and rule is that of mxsg_quantize_act with
 * M = routed rows; mxsg_quantize_act_sizes gives the output sizes.
 */
mxsg_status mxsg_quantize_act_gather(const void *x, int64_t T, const int32_t *row_index, int64_t M,
                                     int64_t C, int32_t recipe, int32_t fmt, int32_t E,
                                     const int32_t *group_ends, void *row_codes, void *row_scales,
                                     void *col_codes, void *col_scales, int64_t ld,
                                     int32_t *padded_starts, float *amax, const float *dl_scale,
                                     const float *dl_inv, int32_t *status_word, mxsg_stream_t stream);

/*
 * Quantize expert weights w [E, K, N] (the single contiguous grouped weight
 * of the Megatron-LM PR), into the forward operand (k-major codes
 * [E, N, K], contiguous along K) and/or the dgrad operand (n-major codes
 * [E, K, N], contiguous along N). Either code pointer may be NULL.
 *
 *  TENSORWISE: one unit per expert; amax fp32 [E] (required) receives
 *    max|W_e|; scales fp32 [E] (same values for both layouts).
 *  DELAYED: s = dl_scale[e], inv = dl_inv[e]; max|W_e| is max-reduced into
 *    amax[e] (required, zeroed beforehand); scales fp32 [E] receive s.
 *  BLOCKWISE: 128x128 tiles of each [K, N]; one code set in two layouts;
 *    scales fp32 [E, K/128, N/128] (same array content for both layouts).
 *  MX: two code sets. k-major: blocks of 32 along K, kmajor_scales uint8
 *    [E, N, K/32]; n-major: blocks of 32 along N, nmajor_scales uint8
 *    [E, K, N/32] (each expert's matrix word-major, R = N resp. K). fmt
 *    e2m1: code rows of K/2 resp. N/2 bytes, same scales.
 *  NVFP4 (fmt e2m1): one tensor scale per expert; amax fp32 [E] (required)
 *    receives max|W_e|; 16-element blocks along K (k-major) resp. N
 *    (n-major); each scale buffer is the NVFP4 buffer of the E experts'
 *    matrices (R = N, L = K resp. R = K, L = N), tensor scales last.
 *  Scale pointers belonging to a non-NULL code pointer are required.
 *  status_word (optional): NaN / Inf weights set MXSG_STATUS_NONFINITE.
 */
mxsg_status mxsg_quantize_weight(const void *w, int32_t E, int64_t K, int64_t N, int32_t recipe,
                                 int32_t fmt, void *kmajor_codes, void *kmajor_scales,
                                 void *nmajor_codes, void *nmajor_scales, float *amax,
                                 const float *dl_scale, const float *dl_inv, int32_t *status_word,
                                 mxsg_stream_t stream);

/*
 * Delayed-scaling update for `units` scaling units (the "max" amax algorithm
 * with a history of length L, as in the Megatron-LM bug report's flags).
 * State, all device arrays owned by the caller (zero-initialized history,
 * pos, amax; scale = inv = 1 initially):
 *   history fp32 [units, L], pos int32 [units], amax fp32 [units],
 *   scale fp32 [units], inv fp32 [units].
 * Per unit: history[pos] = amax; pos = (pos + 1) % L; a = max(history);
 * if a is finite and > 0: scale = fp32(a / fmax), inv = fp32(fmax / a),
 * otherwise both are kept; finally amax = 0 (ready for the next step).
 * Margin is 0. fmt selects fmax.
 */
mxsg_status mxsg_delayed_update(float *history, int32_t *pos, float *amax, float *scale,
                                float *inv, int32_t units, int32_t L, int32_t fmt,
                                mxsg_stream_t stream);

/*
 * Grouped GEMM over per-expert token groups with FP8 operands and fp32
 * accumulation. C[i, j] = sum_l A[i, l] * B[j, l]: both code operands are
 * contiguous along the contraction index l.
 *
 *  Code operands are pair-interleaved (see Layouts) with row length lda
 *  resp. ldb; A of FWD / DGRAD holds 2 * ceil(M/2) rows.
 *  FWD:   A = row-wise codes of x  [M, K] (row length lda >= K, a multiple
 *         of 64), B = k-major weight codes [E, N, K] (ldb = K),
 *         out = Y bf16 [M, N] (row stride N).
 *  DGRAD: A = row-wise codes of dY [M, N] (lda >= N, a multiple of 64),
 *         B = n-major weight codes [E, K, N] (ldb = N),
 *         out = dA bf16 [M, K] (row stride K).
 *  WGRAD: A = column-wise codes of x  [K, lda], B = column-wise codes of dY
 *         [N, ldb] (both in the padded layout of the same groups),
 *         padded_starts int32 [E+1] from mxsg_quantize_act,
 *         out = dW fp32 [E, K, N]; accumulate != 0 adds into out.
 *
 *  Scales, by recipe (each operand's scales come from its quantize call):
 *   TENSORWISE / DELAYED: a_scales fp32 [1]; b_scales fp32 [E] for weights
 *     (FWD / DGRAD) or fp32 [1] (WGRAD). out = acc * sA * sB.
 *   BLOCKWISE: FWD a_scales [M, K/128], b_scales [E, K/128, N/128];
 *     DGRAD a_scales [M, N/128], same b_scales; WGRAD a_scales [K, lda/128],
 *     b_scales [N, ldb/128]. Partial sums of each 128-long contraction block
 *     are scaled by sA * sB and accumulated in fp32.
 *   MX: uint8 E8M0 scales with one byte per 32 contraction elements:
 *     FWD a [M, K/32], b [E, N, K/32]; DGRAD a [M, N/32], b [E, K, N/32];
 *     WGRAD a [K, lda/32], b [N, ldb/32], all word-major (the layout
 *     mxsg_quantize_act / mxsg_quantize_weight write); applied inside the
 *     MFMA.
 *   NVFP4: each operand's NVFP4 scale buffer as its quantize call wrote it
 *     (FWD: the row-wise buffer of x and the k-major weight buffer; DGRAD:
 *     of dY and the n-major weight buffer; WGRAD: the column-wise buffers of
 *     x and dY, whose rows hold ld elements). Each lane decodes its codes
 *     and multiplies by the block scale exactly in f16 (e2m1 x e4m3 products
 *     lie in [2^-10, 2688]); the f16 MFMA accumulates in fp32, and the
 *     epilogue multiplies by the two tensor scales.
 *  fmt_a / fmt_b: element formats of A and B (e4m3 x e4m3, e5m2 x e4m3 and
 *  e4m3 x e5m2 are supported; hybrid training uses e5m2 gradients; e2m1 x
 *  e2m1 with the MX recipe is MXFP4, with the NVFP4 recipe NVFP4).
 *  4-bit operands (e2m1): rows hold two codes per byte, so every row length
 *  above is in code bytes: FWD lda >= K/2 and ldb = K/2, DGRAD lda >= N/2
 *  and ldb = N/2, WGRAD lda, ldb = column-wise code bytes per row (ld/2 of
 *  the quantize call, >= mxsg_padded_capacity(M, E) / 2, a multiple of 64);
 *  scale shapes count contraction elements as for 8-bit codes. The MFMA
 *  consumes 64 contraction elements (32 bytes) per instruction, so each
 *  64-byte stage of a row is two MFMAs at the 4-bit rate.
 *
 *  Rows of FWD / DGRAD outputs belong to exactly one group and are all
 *  written. WGRAD: an empty group's dW_g is written with zeros (left
 *  unchanged when accumulating).
 *  Limits: lda, ldb < 2^23 (BAD_SHAPE); blockwise FWD / DGRAD contraction
 *  (K resp. N) <= 65536 (UNSUPPORTED).
 *  status_word (optional): group_ends are checked (status bits ENDS_*).
 */
mxsg_status mxsg_grouped_mm(int32_t mode, int32_t recipe, int32_t fmt_a, int32_t fmt_b, int32_t E,
                            int64_t M, int64_t K, int64_t N, const int32_t *group_ends,
                            const int32_t *padded_starts, const void *a_codes,
                            const void *a_scales, int64_t lda, const void *b_codes,
                            const void *b_scales, int64_t ldb, void *out, int32_t accumulate,
                            int32_t *status_word, mxsg_stream_t stream);

/*
 * Validation of a mxsg_grouped_mm call without its pointers: the mode,
 * recipe, formats, E, M, K, N, lda, ldb and accumulate rules documented
 * above, returning the status (and mxsg_last_error text) mxsg_grouped_mm
 * would return for them. Pure host function; launches nothing. The
 * accumulate flag is the wgrad accumulation into an fp32 main gradient
 * (Megatron-LM single grouped weight PR, gradient-accumulation-fusion
 * coverage table).
 */
mxsg_status mxsg_grouped_mm_check(int32_t mode, int32_t recipe, int32_t fmt_a, int32_t fmt_b,
                                  int32_t E, int64_t M, int64_t K, int64_t N, int64_t lda,
                                  int64_t ldb, int32_t accumulate);

/*
 * The device cast used by every quantizer (saturating round to nearest
 * even), applied to the n consecutive fp32 bit patterns start_bits,
 * start_bits + 1, ... (wrapping modulo 2^32): out[i] = code(float(start_bits
 * + i)). out uint8 [n] (e2m1: one 4-bit code per byte). NaN patterns give an
 * unspecified code. Lets a caller check the cast exhaustively over all 2^32
 * inputs.
 */
mxsg_status mxsg_cast_sweep(uint32_t start_bits, int64_t n, int32_t fmt, void *out,
                            mxsg_stream_t stream);

/*
 * The SwiGLU activation on its own: y[m, c] = the bf16 value nearest to
 * silu(x[m, c]) * x[m, C + c] (the activation mxsg_quantize_act_swiglu
 * quantizes), for x bf16 [M, 2C] and y bf16 [M, C], both row-major device
 * arrays, 16-byte aligned, C a positive multiple of 8. For callers that
 * keep the bf16 activation (e.g. for the backward pass of the SwiGLU).
 */
mxsg_status mxsg_swiglu(const void *x, int64_t M, int64_t C, void *y, mxsg_stream_t stream);

/*
 * The fp32 sigmoid that the SwiGLU kernels evaluate first, for every bf16
 * bit pattern g: out[g] (fp32 [65536], device) = that value for the gate
 * g. The kernels rely on its relative error being at most 2^-21 for
 * |g| <= 64 (they recompute in fp64 elsewhere and near bf16 rounding
 * midpoints); this call lets a caller check that bound on every input.
 * Outputs for |g| > 64 or non-finite g are unspecified.
 */
mxsg_status mxsg_sigmoid_sweep(float *out, mxsg_stream_t stream);

/*
 * Device-to-device copy of `bytes` (a multiple of 16; both pointers 16-byte
 * aligned) with one 16-byte streaming load and store per thread. Not a step
 * of the method: it is the HBM reference rate the quantization passes are
 * measured against, next to the datasheet bandwidth.
 */
mxsg_status mxsg_stream_copy(const void *src, void *dst, int64_t bytes, mxsg_stream_t stream);

/*
 * Clock probe, also not a step of the method: `blocks` workgroups of 256
 * threads keep the matrix cores busy with bf16 MFMAs for `iters` rounds (a
 * round is 4 MFMAs of 32x32x16 per wave); lane 0 of each workgroup writes
 * out[4 b + 0] = core clock cycles and out[4 b + 1] = wall-clock ticks
 * elapsed over its rounds, out[4 b + 2..3] = 0 (out: uint64 [4 blocks],
 * device). cycles / (ticks / wall rate) is the engine clock under matrix
 * load, which the dense MFMA peaks (quoted at 2.4 GHz) can be scaled by.
 * blocks in [0, 2^20], iters >= 0.
 */
mxsg_status mxsg_clock_probe(int32_t blocks, int32_t iters, uint64_t *out, mxsg_stream_t stream);

/* The constant rate of the wall clock the probe reads, in kHz, of the
 * current device. */
mxsg_status mxsg_wall_clock_rate_khz(int32_t *khz);

#ifdef __cplusplus
}
#endif

#endif /* MXSG_H */
