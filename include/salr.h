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
  /* Parts of a fused layer (salr_fuse_layers fills these; 0 = one part).
   * Part p owns rows part_rows[0] + ... + part_rows[p-1] onward and the
   * adapter ranks part_ranks[0] + ... + part_ranks[p-1] onward; b_cat is
   * zero outside each part's block.  The forward then reads and multiplies
   * only a row tile's own block (when every part has a multiple of 16 rows
   * and of 8 ranks); results are the same either way. */
  int32_t n_parts;  /* 0 (set it so for an encoded layer) or 1: one part;
                     * at most SALR_MAX_PARTS; the parts' rows must sum to
                     * N and their ranks to r_cat (else INVALID_ARG)        */
  int32_t part_rows[8];
  int32_t part_ranks[8];
} salr_layer_t;
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
} salr_sizes_t;

/* Options of the residual truncated SVD inside salr_encode (NULL = the
 * defaults below).  The SVD is computed by randomized subspace iteration:
 * `oversample` extra basis vectors (default 32, at most 64; the basis width
 * r_svd + oversample is capped at min(N, K, 320)), `iters` power iterations
 * (default 24, at most 1000), starting block drawn from a counter-based
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
 * B_cat; Y is rounded to bf16 (nearest-even).
 * Asynchronous on `stream`: returns after queueing.  Errors: INVALID_ARG,
 * WORKSPACE, UNSUPPORTED, HIP (launch failure).
 */
int salr_linear_forward(const salr_layer_t* L, const uint16_t* X, int64_t M,
                        uint16_t* Y, void* ws, size_t ws_bytes, void* stream);

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

/* Static English text for a status code (never NULL). */
const char* salr_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int salr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SALR_H_ */
