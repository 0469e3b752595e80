/*
 * salr.h - C ABI of the MI355X (gfx950) SALR linear-layer library.
 *
 * SALR ("Sparsity-Aware Low-Rank Representation for Efficient Fine-Tuning of
 * Large Language Models") serves a linear layer as
 *
 *     Y = X * W_s^T + (X * A_cat) * B_cat
 *
 * where W_s is the frozen base weight with a static per-row magnitude mask
 * applied, stored as a bitmap plus a compact array of the kept bf16 values,
 * and A_cat / B_cat stack the truncated-SVD residual adapter and the LoRA
 * adapters along the rank dimension so that all of them run as one low-rank
 * product.  Sources: the authors' abstract, and the gist.science technical
 * summary of the paper, section "Methodology" parts 1-4.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or from a torch
 *     CUDA tensor) unless a comment says "host".  bf16 tensors are passed as
 *     uint16_t bit patterns.  All matrices are row-major and dense (no
 *     leading-dimension arguments).
 *   - The caller allocates every buffer, including workspaces; the library
 *     allocates no device memory and keeps no global state.  Calls on
 *     different streams with different workspaces may run concurrently.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *   - Return value: SALR_OK (0) or a negative salr_status_t.  Argument
 *     validation happens on the host before any device work is queued; on a
 *     validation error nothing is launched and no output is touched.
 *   - Pointer alignment: every device pointer must be 16-byte aligned.
 *   - Shape limits: 1 <= N, 1 <= K <= 2^20, K % 8 == 0, N*K < 2^40,
 *     0 <= n_keep <= K, 0 <= r_cat <= 256.
 *
 * Encoded layer layout (what salr_encode writes, what the forward reads)
 *   masks   uint64 [N][ceil(K/64)]  bit b of word w set iff column 64w+b of
 *           row n is KEPT (a kept zero still sets its bit); bits past K are 0.
 *           ("bitmap indicating the non-zero elements": summary, Methodology 4)
 *   values  bf16   [N][n_keep]      each row's kept values in ascending
 *           column order, bit-exact copies of W ("compact array of dense
 *           values": summary, Methodology 4).  The buffer must be
 *           sizes.values_bytes long: the kernels may read up to 256 bytes
 *           past the last value (never used), so the tail is padding.
 *   offsets uint32 [N][ceil(K/1024)] running kept count before every 1024th
 *           column: offsets[n][g] = #kept columns < 1024*g.  This is the
 *           lookup table read beside the bitmap (summary, Methodology 4,
 *           stage 1); it locates a row's values for any 1024-column block.
 *   a_cat   bf16   [r_cat][K]       A_cat TRANSPOSED: row j is rank
 *           component j's input projection.  Rows [0, r_svd) are the residual
 *           adapter sqrt(S_r) V_r^T, then each LoRA down-projection in call
 *           order (summary, Methodology 2 and 3).
 *   b_cat   bf16   [N][r_cat]       B_cat TRANSPOSED: row n holds output n's
 *           coefficients on the r_cat components; columns [0, r_svd) are the
 *           residual adapter U_r sqrt(S_r), then each LoRA up-projection.  The
 *           buffer must be sizes.b_cat_bytes long (tail padding, as for
 *           values).
 */
#ifndef SALR_H_
#define SALR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum salr_status {
  SALR_OK = 0,
  SALR_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad dimension      */
  SALR_ERR_UNSUPPORTED = -2, /* valid request outside the supported limits  */
  SALR_ERR_WORKSPACE = -3,   /* workspace pointer null or too small         */
  SALR_ERR_NONFINITE = -4,   /* W holds Inf or NaN (salr_encode)            */
  SALR_ERR_NUMERICAL = -5,   /* SVD subspace lost rank (salr_encode)        */
  SALR_ERR_HIP = -6          /* a HIP runtime call or launch failed         */
} salr_status_t;

/* One encoded layer: plain pointers into caller-owned device buffers. */
typedef struct salr_layer {
  int64_t N;        /* out_features (rows of W)                             */
  int64_t K;        /* in_features  (columns of W)                          */
  int32_t n_keep;   /* kept weights per row                                 */
  int32_t r_cat;    /* total adapter rank (residual + all LoRA ranks)       */
  uint64_t* masks;  /* [N][ceil(K/64)]                                      */
  uint16_t* values; /* [N][n_keep] (+ padding, see values_bytes)            */
  uint32_t* offsets;/* [N][ceil(K/1024)]                                    */
  uint16_t* a_cat;  /* [r_cat][K]                                           */
  uint16_t* b_cat;  /* [N][r_cat]                                           */
  /* Parts of a fused layer (salr_fuse_layers fills these; salr_encode
   * sets n_parts = 0 and zeroes both arrays).
   * Part p owns rows part_rows[0] + ... + part_rows[p-1] onward and the
   * adapter ranks part_ranks[0] + ... + part_ranks[p-1] onward.  The
   * forward TRUSTS b_cat to be zero outside each part's block: it then reads
   * and multiplies only a row tile's own block (when every part has a
   * multiple of 16 rows and of 8 ranks), so a record that does not match a
   * block-diagonal b_cat gives a wrong Y without an error. */
  int32_t n_parts;  /* 0 (set it so for an encoded layer) or 1: one part;
                     * at most SALR_MAX_PARTS; the parts' rows must sum to
                     * N and their ranks to r_cat (else INVALID_ARG)        */
  int32_t part_rows[8];
  int32_t part_ranks[8];
  /* Value format (QSALR): SALR_VALUES_BF16 (0: `values` holds the kept
   * values) or SALR_VALUES_NF4 (1: `codes` and `scales` hold them, see
   * salr_quantize_nf4; `values` is not read by the forward).              */
  int32_t value_format;
  uint8_t* codes;   /* NF4: uint8 [N][32 * ceil(n_keep/64)] (+ padding)      */
  uint16_t* scales; /* NF4: bf16 [N][ceil(n_keep/64)] (+ padding)            */
} salr_layer_t;
#define SALR_VALUES_BF16 0
#define SALR_VALUES_NF4 1
#define SALR_MAX_PARTS 8

/* Byte sizes of every caller-allocated buffer. */
typedef struct salr_sizes {
  size_t masks_bytes;
  size_t values_bytes;     /* includes tail padding                         */
  size_t offsets_bytes;
  size_t a_cat_bytes;
  size_t b_cat_bytes;
  size_t encode_ws_bytes;  /* workspace of salr_encode                      */
  size_t forward_ws_bytes; /* workspace of salr_linear_forward for M<=M_max */
  size_t codes_bytes;      /* NF4 codes (includes tail padding)             */
  size_t scales_bytes;     /* NF4 scales (includes tail padding)            */
  size_t forward_ws_nf4_bytes; /* forward workspace of the NF4 layer        */
} salr_sizes_t;

/* Options of the residual truncated SVD inside salr_encode (NULL = the
 * defaults below).  The SVD is computed by randomized subspace iteration:
 * `oversample` extra basis vectors (default 32, at most 64; the basis width
 * r_svd + oversample is capped at min(N, K, 320)), `iters` power iterations
 * (default 40, at most 1000), starting block drawn from a counter-based
 * generator keyed by `seed` (default 0).  encode_ws_bytes from
 * salr_query_sizes covers every allowed oversample. */
typedef struct salr_encode_opts {
  int32_t oversample;
  int32_t iters;
  uint64_t seed;
} salr_encode_opts_t;

/*
 * salr_query_sizes - byte sizes of the buffers for an N x K layer that keeps
 * n_keep weights per row, with a residual adapter of rank r_svd and total
 * adapter rank r_cat, run with at most M_max input rows per forward call.
 * `out` is a host pointer.  Pure host arithmetic; no device is touched.
 * Errors: SALR_ERR_INVALID_ARG for null `out` or dimensions outside the
 * limits above (r_svd must satisfy 0 <= r_svd <= min(N, K, r_cat)).
 */
int salr_query_sizes(int64_t N, int64_t K, int32_t n_keep, int32_t r_svd,
                     int32_t r_cat, int64_t M_max, salr_sizes_t* out);

/*
 * salr_encode - offline SALR compression of one frozen weight (summary,
 * Methodology 1-4; authors' abstract):
 *   1. per output row, keep the n_keep entries of largest |w| (magnitude =
 *      the 15 low bits of the bf16 pattern; equal magnitudes at the cut are
 *      kept in ascending column order), write masks/values/offsets;
 *   2. residual R = W - W_s (the pruned entries);
 *   3. rank-r_svd truncated SVD of R, split evenly into A' = V_r sqrt(S_r),
 *      B' = sqrt(S_r) U_r^T and rounded to bf16;
 *   4. stack [A' | A_1 | ... | A_L] and [B'; B_1; ...; B_L] into a_cat/b_cat.
 *
 * W        device bf16 [N][K].
 * lora_A   host array of n_lora device pointers, lora_A[i] bf16 [lora_r[i]][K]
 *          (nn.Linear weight of the adapter's down projection, = A_i^T).
 * lora_B   host array of n_lora device pointers, lora_B[i] bf16 [N][lora_r[i]]
 *          (nn.Linear weight of the adapter's up projection, = B_i^T).
 * lora_r   host array of n_lora ranks (each >= 1).
 * opts     host pointer or NULL.
 * out      host pointer; N, K, n_keep, r_cat and the five buffer pointers must
 *          be filled in by the caller (r_cat = r_svd + sum(lora_r)); the
 *          buffers are overwritten.
 * sigma    host pointer to r_svd doubles receiving the estimated leading
 *          singular values of R, or NULL.
 * ws       device workspace of at least encode_ws_bytes.
 * Synchronous: returns after all device work has finished.  The singular
 * values are estimates (the method is iterative); masks, values, offsets and
 * the LoRA blocks are exact.
 * Errors: INVALID_ARG (shapes, nulls, alignment, r_cat mismatch),
 * WORKSPACE, NONFINITE (W holds Inf/NaN; outputs undefined), NUMERICAL
 * (the subspace basis became rank deficient; outputs undefined), HIP.
 */
int salr_encode(const uint16_t* W, int64_t N, int64_t K, int32_t n_keep,
                int32_t r_svd, int32_t n_lora, const uint16_t* const* lora_A,
                const uint16_t* const* lora_B, const int32_t* lora_r,
                const salr_encode_opts_t* opts, salr_layer_t* out,
                double* sigma, void* ws, size_t ws_bytes, void* stream);

/*
 * salr_nf4_levels - the 16 levels of the NF4 value codec (QSALR: summary,
 * Experimental Results, Ablation Studies, "Quantization"), ascending, as
 * float32: the NormalFloat definition of QLoRA (Dettmers et al. 2023) -- 8
 * positive normal quantiles at probabilities evenly spaced from 1 - d down
 * to 1/2 (exclusive), 7 negative ones mirrored likewise, and 0, with
 * d = (1/30 + 1/32) / 2, divided by the largest.  `out` is a host pointer.
 * Pure host arithmetic.  Errors: INVALID_ARG (null).
 */
int salr_nf4_levels(float* out);

/*
 * salr_quantize_nf4 - QSALR value codec: code the kept values of an encoded
 * layer (L->values, bf16) as NF4, in blocks of 64 consecutive values of a
 * row (a row's last block may be shorter): the block's scale is its largest
 * |value| (bf16, exact); each value's code is the index of the level nearest
 * to value / scale in float32 (the lower level on a tie; a zero block codes
 * 0.0, level 7); codes are nibble-packed, value 2b in the low nibble of byte
 * b of the row, rows of 32 bytes per block.  Decoded values are
 * bf16(level * scale) computed in float32.
 *
 * L   host pointer; L->values, L->codes (codes_bytes) and L->scales
 *     (scales_bytes from salr_query_sizes) must be set; on success
 *     L->value_format becomes SALR_VALUES_NF4.  The bitmap, lookup table and
 *     adapters are not touched (the forward then reads codes and scales).
 * Asynchronous on `stream`.  Errors: INVALID_ARG (nulls, alignment,
 * dimensions, a layer already in NF4), HIP.
 */
int salr_quantize_nf4(salr_layer_t* L, void* stream);

/*
 * salr_linear_forward - Y = X W_s^T + (X A_cat) B_cat for one encoded layer
 * (summary, Methodology 3 and 4: bitmap decode feeding matrix-core tiles,
 * one concatenated low-rank product).
 *
 * L   host pointer to the encoded layer.
 * X   device bf16 [M][K];  Y device bf16 [M][N] (written; may not alias X).
 * M   rows of X, 0 <= M; M == 0 is a no-op returning SALR_OK.
 * ws  device workspace of at least forward_ws_bytes for some M_max >= M.
 *     It must be zero-filled before its first use; every completed call
 *     leaves it ready for the next one.  Two calls that share a workspace
 *     must be ordered (same stream or synchronised).  Workgroups of one
 *     call hand partial results to each other through the workspace and
 *     every such wait is bounded: should one time out, the uint32 at byte
 *     offset 8 of ws becomes nonzero (and Y is unreliable); the library
 *     never clears it.
 * Products accumulate in fp32; X*A_cat is rounded to bf16 before it meets
 * B_cat; Y is rounded to bf16 (nearest-even).  An NF4 layer
 * (value_format == SALR_VALUES_NF4) computes the same with every kept value
 * replaced by its decoded value; its workspace is forward_ws_nf4_bytes.
 * Asynchronous on `stream`: returns after queueing.  Errors: INVALID_ARG,
 * WORKSPACE, UNSUPPORTED, HIP (launch failure).
 */
int salr_linear_forward(const salr_layer_t* L, const uint16_t* X, int64_t M,
                        uint16_t* Y, void* ws, size_t ws_bytes, void* stream);

/*
 * salr_linear_forward_noalloc - salr_linear_forward without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * The workspace is a fixed device array inside the library,
 * SALR_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library runs on
 * holds until the process ends.  The first call on a device (with that
 * device current) looks the array up and zero-fills it on `stream`,
 * waiting for the fill; that first call must not be under graph capture
 * (SALR_ERR_UNSUPPORTED).  Later calls allocate nothing, call no hipMalloc /
 * hipFree / allocating routine and may be captured.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (different streams
 * or threads without ordering) race and give wrong results.
 *
 * L, X, M, Y, stream: as for salr_linear_forward (same kernels, same
 * results).  wait_err: device pointer to a uint32 (4-byte aligned) that a
 * timed-out bounded wait sets nonzero (the caller clears it; Y is then
 * unreliable, and so are later calls on this GPU), or NULL to not report
 * timeouts.  Errors: those of salr_linear_forward; SALR_ERR_WORKSPACE when
 * the layer and M need more workspace than the array holds (the bytes
 * salr_query_sizes reports as forward_ws_bytes for M_max = M); SALR_ERR_HIP
 * when the array cannot be set up.
 */
#define SALR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int salr_linear_forward_noalloc(const salr_layer_t* L, const uint16_t* X, int64_t M, uint16_t* Y,
                                uint32_t* wait_err, void* stream);

/*
 * salr_fuse_layers - one encoded layer from n_parts encoded layers that read
 * the same input (q/k/v, or gate/up): a single forward call on the result
 * computes every part.  This applies the pages' single low-rank product on
 * a shared input (summary, Methodology 3) across projections:
 *   masks, values, offsets  rows of part 0, then part 1, ... (along N);
 *   a_cat                   ranks of part 0, then part 1, ... (along r_cat);
 *   b_cat                   block diagonal: row n of part p holds part p's
 *                           coefficients at columns [R_p, R_p + r_cat_p),
 *                           R_p = r_cat_0 + ... + r_cat_{p-1}, and 0
 *                           elsewhere.
 * A forward on the fused layer returns Y = [Y_0 | Y_1 | ...] along N (part
 * p's outputs are columns [N_0 + ... + N_{p-1}, + N_p)).  The zero blocks of
 * b_cat are real bytes and multiplies: the price of one launch instead of
 * n_parts.
 *
 * parts    host array of n_parts (>= 1) host pointers to encoded layers, all
 *          with the same K and n_keep.
 * out      host pointer; the caller fills N = sum N_p, K, n_keep,
 *          r_cat = sum r_cat_p (<= 256) and the five buffer pointers, sized
 *          by salr_query_sizes(N, K, n_keep, 0, r_cat, ...); its buffers must
 *          not overlap any part's.  They are overwritten.
 * The parts' rows and ranks are recorded in out->n_parts, part_rows and
 * part_ranks.  Asynchronous on `stream` (device-to-device copies and one
 * small kernel per part).  Errors: INVALID_ARG (nulls, alignment, mismatched
 * K or n_keep, sums that disagree with `out`, more than 8 parts, limits),
 * HIP.
 */
int salr_fuse_layers(const salr_layer_t* const* parts, int32_t n_parts,
                     salr_layer_t* out, void* stream);

/*
 * Backward pass, for fine-tuning the adapters while the base weight stays
 * frozen (summary, Methodology 2: the SVD residual adapter is trained
 * together with the LoRA adapters; Methodology 1: the mask belongs to the
 * frozen base weight only).  For Y = X W_s^T + (X A_cat) B_cat and the
 * upstream gradient dY = dL/dY:
 *     dX     = dY W_s + (dY B_cat^T) A_cat^T
 *     dA_cat = X^T (dY B_cat^T)          dB_cat = (X A_cat)^T dY
 * W_s itself gets no gradient.  dX is a forward of the TRANSPOSED layer:
 * W_s^T (K rows of N columns) in the encoded-layer layout, with adapters
 * B_cat^T and A_cat^T.  Its encoding is built once per frozen weight by
 * salr_transpose_layer; a row of it (a column of W_s) may keep fewer than
 * n_keep columns: its kept values come first, +0.0 fills the rest of the
 * row, and the forward kernels accept such rows.  Limits: the layer's own,
 * plus N % 8 == 0 and N <= 2^20 (W_s^T's column limits), else
 * SALR_ERR_UNSUPPORTED.
 */

/* Workspace bytes of salr_transpose_count / salr_transpose_layer for an
 * N x K layer (`out` host).  Errors: INVALID_ARG. */
int salr_transpose_ws_bytes(int64_t N, int64_t K, size_t* out);

/*
 * salr_transpose_count - the largest number of kept entries in one column of
 * W_s (host `*n_keep_t`), which is the n_keep of the transposed layer: size
 * its buffers with salr_query_sizes(K, N, n_keep_t, 0, r_cat, M_max, ...).
 * Reads L->masks only.  ws: device, salr_transpose_ws_bytes long (contents
 * on entry do not matter).  SYNCHRONOUS (waits for `stream`).
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
int salr_transpose_count(const salr_layer_t* L, int32_t* n_keep_t, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * salr_transpose_layer - the encoding of W_s^T from that of W_s (a bf16
 * layer).  LT: host pointer; the caller fills N = L->K, K = L->N,
 * n_keep >= the count from salr_transpose_count, and the masks, values and
 * offsets buffers (sizes from salr_query_sizes as above; not overlapping
 * L's).  Written: LT->masks (bit n of word w of row k set iff W_s keeps
 * (64w + n, k)), LT->values (row k: column k's kept values in ascending row
 * order, bit-exact, then +0.0 up to n_keep), LT->offsets (kept rows of
 * column k before every 1024th row), and the fields r_cat = L->r_cat,
 * n_parts = 0, value_format = SALR_VALUES_BF16, codes = scales = NULL.
 * LT->a_cat and LT->b_cat are neither read nor written (the backward supplies
 * the transposed adapters).  ws as for salr_transpose_count.  SYNCHRONOUS.
 * Errors: INVALID_ARG (shapes, nulls, alignment, LT->n_keep below the
 * largest column count), UNSUPPORTED (limits, an NF4 layer), WORKSPACE, HIP.
 */
int salr_transpose_layer(const salr_layer_t* L, salr_layer_t* LT, void* ws,
                         size_t ws_bytes, void* stream);

/* Workspace bytes of salr_linear_backward for an N x K layer whose
 * transposed layer keeps n_keep_t per row, adapter rank r_cat, at most M_max
 * tokens per call (`out` host).  Errors: INVALID_ARG, UNSUPPORTED. */
int salr_backward_ws_bytes(int64_t N, int64_t K, int32_t n_keep_t,
                           int32_t r_cat, int64_t M_max, size_t* out);

/*
 * salr_linear_backward - dX, dA_cat and dB_cat of one layer for M tokens.
 *
 * L    host pointer to the layer (its a_cat and b_cat are read; any value
 *      format, the base weight is read through LT).
 * LT   host pointer to its transposed layer from salr_transpose_layer.
 * X    device bf16 [M][K] (the forward's input); dY device bf16 [M][N].
 * dX   device bf16 [M][K], or NULL to skip it (a first layer).  Computed
 *      exactly as salr_linear_forward computes Y for LT and input dY: fp32
 *      accumulation, dY B_cat^T rounded to bf16 before it meets A_cat^T, dX
 *      rounded to bf16.  May not alias dY.
 * dA   device float [r_cat][K]: the gradient of a_cat AS STORED
 *      (dA[j][k] = sum_m G[m][j] X[m][k], G = bf16(dY B_cat^T)).
 * dB   device float [N][r_cat]: the gradient of b_cat as stored
 *      (dB[n][j] = sum_m dY[m][n] T[m][j], T = bf16(X A_cat)).  For a fused
 *      layer it covers b_cat's zero blocks too (keep them at zero).
 *      dA and dB are required when r_cat > 0; they are overwritten (not
 *      accumulated into), fp32 accumulation over the tokens; M == 0 writes
 *      zeros.
 * ws   device workspace of at least salr_backward_ws_bytes for some
 *      M_max >= M; zero-filled before its first use, then left ready by
 *      every completed call; calls that share it must be ordered.  As for
 *      the forward, a timed-out bounded wait sets the uint32 at byte 8.
 * Asynchronous on `stream`.  Errors: INVALID_ARG (shapes, nulls, alignment,
 * LT not matching L), UNSUPPORTED, WORKSPACE, HIP.
 */
int salr_linear_backward(const salr_layer_t* L, const salr_layer_t* LT,
                         const uint16_t* X, const uint16_t* dY, int64_t M,
                         uint16_t* dX, float* dA, float* dB, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * Grouped (mixture-of-experts) layer: E experts of one shape, each its own
 * encoded layer (summary, Experimental Results: SALR applied to the MoE
 * models Mixtral-8x7B and DeepSeek-V2-Lite), held in five stacked buffers,
 * expert e's arrays at fixed element strides (each a multiple of 256 bytes,
 * reported by salr_moe_query_sizes):
 *   masks   uint64 [E][masks_stride]    expert e: its [N][ceil(K/64)]
 *   values  bf16   [E][values_stride]   expert e: its [N][n_keep]
 *   offsets uint32 [E][offsets_stride]  expert e: its [N][ceil(K/1024)]
 *   a_cat   bf16   [E][a_cat_stride]    expert e: its [r_cat][K]
 *   b_cat   bf16   [E][b_cat_stride]    expert e: its [N][r_cat]
 * (values and b_cat with tail padding: use the *_bytes sizes).  All experts
 * share N, K, n_keep and r_cat (a smaller LoRA rank pads with zero ranks).
 */
typedef struct salr_moe_layer {
  int32_t E;
  int64_t N;
  int64_t K;
  int32_t n_keep;
  int32_t r_cat;
  uint64_t* masks;
  uint16_t* values;
  uint32_t* offsets;
  uint16_t* a_cat;
  uint16_t* b_cat;
} salr_moe_layer_t;

typedef struct salr_moe_sizes {
  size_t masks_bytes, values_bytes, offsets_bytes, a_cat_bytes, b_cat_bytes;
  size_t masks_stride, values_stride, offsets_stride, a_cat_stride, b_cat_stride;  /* elements */
  size_t forward_ws_bytes;  /* salr_moe_forward workspace for T_max rows    */
} salr_moe_sizes_t;

/* Sizes and strides of an E-expert layer (1 <= E <= 4096; the layer limits
 * above per expert), forward workspace for at most T_max rows (`out` host).
 * Pure host arithmetic.  Errors: INVALID_ARG. */
int salr_moe_query_sizes(int32_t E, int64_t N, int64_t K, int32_t n_keep,
                         int32_t r_cat, int64_t T_max, salr_moe_sizes_t* out);

/* The layer descriptor of expert e (views into the stacked buffers; n_parts
 * 0, bf16 values): pass it to salr_encode to encode that expert in place,
 * or to salr_linear_forward to run it alone.  `out` host; host arithmetic.
 * Errors: INVALID_ARG. */
int salr_moe_expert(const salr_moe_layer_t* G, int32_t e, salr_layer_t* out);

/*
 * salr_moe_forward - for every expert e:
 *   Y[off[e]:off[e+1]] = X[off[e]:off[e+1]] W_s,e^T
 *                        + (X[off[e]:off[e+1]] A_cat,e) B_cat,e
 * in one grouped pair of launches.
 *
 * G    host pointer to the grouped layer.
 * X    device bf16 [T][K], rows grouped by expert; Y device bf16 [T][N]
 *      (may not alias X).
 * expert_offsets  DEVICE int32 [E + 1], read by the kernels (routing needs
 *      no host round trip): off[0] = 0, nondecreasing, off[E] = T.  The
 *      kernels clamp each boundary into [0, T] and never leave X or Y, but
 *      rows outside every valid group are then not written.
 * m_cap  the expected most rows of one expert (0: T); it only sizes the
 *      low-rank grid: any distribution is computed correctly.
 * ws   device workspace, forward_ws_bytes for some T_max >= T (contents on
 *      entry do not matter; no zero fill needed).
 * Numerics as salr_linear_forward (fp32 accumulation, X A_cat rounded to
 * bf16, Y rounded to bf16).  An expert with no rows reads none of its
 * weight.  Asynchronous on `stream`.  Errors: INVALID_ARG, WORKSPACE, HIP.
 */
int salr_moe_forward(const salr_moe_layer_t* G, const uint16_t* X, int64_t T,
                     const int32_t* expert_offsets, int64_t m_cap, uint16_t* Y,
                     void* ws, size_t ws_bytes, void* stream);

/* Static English text for a status code (never NULL). */
const char* salr_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int salr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SALR_H_ */
