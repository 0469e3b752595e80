// Launch interfaces of the SALR HIP kernels (host side of each .hip file).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace salr {

void nf4_levels(float out[16]);  // (QSALR value codec, see below)

constexpr int kMaxRangeCols = 4096;  // columns per few-row workgroup
// Launch-tag ticket words in the forward workspace (see salr_device.hpp).
constexpr uint32_t kTicketGroups = 16;
constexpr uint32_t kTicketStride = 32;  // uint64 words between ticket words

// ----------------------------------------------------------------------------
// Forward, M <= 16: one fused launch.  Extra workgroups at the front of the
// grid compute the pieces of T = X * A_cat; every other workgroup decodes 16
// rows x one column range of W_s, multiplies, and adds its share of the
// low-rank term; range partials meet in each row tile's finishing workgroup.
// ----------------------------------------------------------------------------
struct SmallFwdArgs {
  const uint64_t* masks;
  const uint16_t* values;
  const uint32_t* offsets;
  const uint16_t* b_cat;   // [N][r_cat] (+ tail padding)
  const uint16_t* X;       // [M][K]
  uint16_t* Y;             // [M][N]
  const uint16_t* a_cat;   // [r_cat][K]
  uint64_t* tpiece;        // [r_tiles * t_pieces][256] tagged fp32 pieces of T
  uint64_t* tfinal;        // [r_tiles][128] tagged bf16 pairs: T per rank tile
  uint32_t* tcount;        // [r_tiles] pieces published per rank tile
  int64_t N;
  int32_t K, n_keep, r_cat, M;
  int32_t kw, ng;          // words / lookup entries per row
  int32_t n_tiles;         // ceil(N/16) row tiles
  int32_t splits;          // column ranges per row (1 = whole rows)
  int32_t range;           // columns per range (K when splits == 1, else 1024/2048/4096)
  int32_t vcap;            // 16-byte chunks of LDS per row
  int32_t r_tiles;         // ceil(r_cat/16)
  int32_t r_pad;           // ranks of T rounded up to a multiple of 32
  int32_t t_pieces;        // K ranges of T pieces, t_chunks * 1024 columns each
  int32_t t_chunks;
  int32_t vals_bytes;      // LDS bytes of the values area
  int32_t tl_bytes;        // bytes of the T operands (r_pad / 32 chunks x 1 KB, in the bitmap-word area)
  int32_t bl_bytes;        // LDS bytes of the B_cat rows (16 * r_cat * 2, rounded up to 16)
  // fused layers (0 parts: one block of r_cat ranks): part p owns the row
  // tiles below part_tile_end[p] and the ranks [part_rank0[p], + part_nrank[p])
  int32_t nparts;
  int32_t part_tile_end[8], part_rank0[8], part_nrank[8];
  uint64_t* tickets;       // {count, epoch} ticket words of the launch tags
  uint32_t* err;           // set nonzero when a wait times out
  uint32_t* ycount;        // [n_tiles]
  uint64_t* ypart;         // [n_tiles][splits][256] tagged fp32
  // NF4 values (nf4 != 0): codes and scales go to the end of each row's LDS
  // area (chunk offsets cofs and sofs) and are dequantized into the bf16
  // stream the decode reads
  int32_t nf4;
  const uint8_t* codes;    // [N][cb_row]
  const uint16_t* scales;  // [N][nblk]
  int32_t cb_row, nblk, cofs, sofs;
  float levels[16];        // the NF4 levels (set by launch_fwd_small)
};
// Groups of 8 values per thread of the few-row dequantization pass (32
// threads per row).
constexpr int kNf4Groups = 9;
hipError_t launch_fwd_small(const SmallFwdArgs& a, hipStream_t s);
size_t fwd_small_vals_bytes(int vcap);
// Dynamic LDS bytes of one few-row workgroup.
size_t fwd_small_lds_bytes(int vcap, int bl_bytes);
// LDS chunks per row for rows whose staged values never exceed `cap`.  The
// first value sits at slot 0..7 of the first chunk (always 0 when
// `aligned_start`), and a decode window reads at most 5 slots past one past
// the last value; rounded to a stride of 1 mod 8 chunks so consecutive rows
// start 4 banks apart.  (Two whole-row workgroups of 4096 columns with a
// low-rank term fit on one CU only with this tight count.)
inline int fwd_small_vcap(int64_t cap, bool aligned_start) {
  const int v = (int)(((aligned_start ? 0 : 7) + cap + 5) / 8 + 1);
  return v + ((1 - v % 8) + 8) % 8;
}

// ----------------------------------------------------------------------------
// Forward, M <= 16, layers with more than one round of 16-row work: one
// launch of persistent workgroups (one per CU), each streaming a run of
// whole row tiles through two LDS buffers in chunks of kChunk columns; the
// first r_tiles * t_pieces workgroups also compute the pieces of T (same
// pieces, tagged words and counters as the one-round kernel).
// ----------------------------------------------------------------------------
constexpr int kChunk = 2048;  // columns per streamed chunk (a multiple of 1024)
struct StreamFwdArgs {
  const uint64_t* masks;
  const uint16_t* values;
  const uint32_t* offsets;
  const uint16_t* b_cat;   // [N][r_cat]
  const uint16_t* X;       // [M][K]
  uint16_t* Y;             // [M][N]
  const uint16_t* a_cat;   // [r_cat][K]
  uint64_t* tpiece;        // [r_tiles * t_pieces][256] tagged fp32 pieces of T
  uint64_t* tfinal;        // [r_tiles][128] tagged bf16 pairs: T per rank tile
  uint32_t* tcount;        // [r_tiles] pieces published per rank tile
  int64_t N;
  int32_t K, n_keep, r_cat, M;
  int32_t kw, ng;          // words / lookup entries per row (ng <= 64)
  int32_t n_tiles;         // ceil(N/16)
  int32_t tiles_per_wg;    // run of row tiles per workgroup
  int32_t vcap;            // 16-byte LDS chunks per row per buffer
  int32_t r_tiles, r_pad;  // ceil(r_cat/16); ranks rounded up to a multiple of 32
  int32_t t_pieces, t_chunks;
  uint64_t* tickets;
  uint32_t* err;
};
hipError_t launch_fwd_stream(const StreamFwdArgs& a, hipStream_t s);
// Dynamic LDS bytes of one streaming workgroup.
size_t fwd_stream_lds_bytes(int vcap);

// ----------------------------------------------------------------------------
// Forward, M > 16: T = X * A_cat (bf16, [M][r_pad]) then the tiled
// decode + MFMA kernel with the low-rank term as extra K steps.
// ----------------------------------------------------------------------------
struct LowRankTArgs {
  const uint16_t* X;       // [M][K]
  const uint16_t* a_cat;   // [r_cat][K]
  float* tpart;            // [splits][M][r_pad] fp32 partial sums of X A_cat
  uint16_t* t16;           // [M][r_pad] bf16 T (their sum, written after them)
  int32_t M, K, r_cat, r_pad;
  int32_t splits, k_chunk; // K-splits, columns per split (multiple of 64)
};
hipError_t launch_lowrank_t(const LowRankTArgs& a, hipStream_t s);

struct LargeFwdArgs {
  const uint64_t* masks;
  const uint16_t* values;
  const uint16_t* b_cat;   // [N][r_cat]
  const uint16_t* X;       // [M][K]
  const float* tpart;      // [t_splits][M][r_pad] partial T, null when r_cat == 0
  const uint16_t* t16;     // [M][r_pad] bf16 T (sum of the partials), null when r_cat == 0
  uint16_t* Y;             // [M][N]
  int64_t N;
  int32_t K, n_keep, r_cat, r_pad, M;
  int32_t t_splits;
  int32_t kw;
  int64_t vchunks;         // ceil(N * n_keep / 8): 16-byte chunks of values
  // K splits (1 = none): split s covers 64-column tiles [s*kt_per, +kt_per)
  // and, when ksplit > 1, writes fp32 partials to ypart[s][M][N], summed in
  // split order by a second launch
  const uint32_t* offsets; // [N][ng] kept counts before every 1024th column
  int32_t ng;
  int32_t ksplit, kt_per;
  float* ypart;
  int32_t x_off32;         // 1 when M * K * 2 < 2^32 (X tile loads from 32-bit offsets)
  // Fused layer whose parts all have whole 256-row blocks (else nparts = 0):
  // rows [part_row_end[p-1], part_row_end[p]) use adapter ranks
  // [part_rank0[p], part_rank0[p] + part_nrank[p]) only.
  int32_t nparts;
  int32_t part_row_end[8], part_rank0[8], part_nrank[8];
};
hipError_t launch_fwd_large(const LargeFwdArgs& a, hipStream_t s);
// Output tiles of the many-row kernel and the K splits it takes for M rows
// (more workgroups when the tiles alone cannot fill the GPU).
int64_t fwd_large_tiles(int64_t N, int64_t M);
int fwd_large_ksplit(int64_t N, int64_t K, int64_t M);
// Bytes of fp32 split partials the many-row kernel may need for up to M_max rows.
size_t fwd_large_part_bytes(int64_t N, int64_t K, int64_t M_max);

// ----------------------------------------------------------------------------
// Multi-projection fusion: rows [0, rows) of a fused B_cat (row stride r_dst)
// from one part's B_cat [rows][r_src], placed at columns [col0, col0 + r_src),
// zeros elsewhere.
hipError_t launch_fuse_b(const uint16_t* src, int64_t rows, int r_src, uint16_t* dst, int r_dst, int col0,
                         hipStream_t s);

// ----------------------------------------------------------------------------
// QSALR value codec (NF4): 16 levels, 64-value blocks with a bf16 absmax
// scale, codes nibble-packed (value 2b low, 2b + 1 high nibble of byte b),
// rows of 32 bytes per block.
struct Nf4Levels {
  float v[16];
};
constexpr uint32_t kNf4ZeroCode = 7;  // the level 0.0
void nf4_levels(float out[16]);
hipError_t launch_quantize_nf4(const uint16_t* values, int64_t N, int32_t n_keep, uint8_t* codes, uint16_t* scales,
                               hipStream_t s);
hipError_t launch_dequantize_nf4(const uint8_t* codes, const uint16_t* scales, int64_t N, int32_t n_keep,
                                 uint16_t* values, hipStream_t s);

// ----------------------------------------------------------------------------
// Backward: the transposed encoding of W_s and the adapter-gradient GEMMs.
// Transposed encoding: rowpre [N][kw] (kept before each word), cnt [nb][K]
// (per 64-row block column counts, scanned in place to the kept rows before
// each block), maxcount (one word, zeroed by the caller), offsets_t
// [K][ceil(N/1024)] (or null).
hipError_t launch_transpose_count(const uint64_t* masks, int64_t N, int32_t K, uint32_t* rowpre, uint32_t* cnt,
                                  uint32_t* maxcount, uint32_t* offsets_t, int32_t ng_t, hipStream_t s);
hipError_t launch_transpose_scatter(const uint64_t* masks, const uint16_t* values, const uint32_t* rowpre,
                                    const uint32_t* colpre, int64_t N, int32_t K, int32_t n_keep, int32_t n_keep_t,
                                    uint64_t* masks_t, uint16_t* values_t, hipStream_t s);
// dst[c][r] = src[r][c] (bf16), dst rows of ld_dst >= R entries, zero past R.
hipError_t launch_transpose_bf16_pair(const uint16_t* src0, int64_t R0, int64_t C0, int64_t ld_src0, uint16_t* dst0,
                                      int64_t ld_dst0, const uint16_t* src1, int64_t R1, int64_t C1, int64_t ld_src1,
                                      uint16_t* dst1, int64_t ld_dst1, hipStream_t s);
// out[p][q] = sum over m < M of A[m][p] B[m][q] (bf16, row strides lda /
// ldb; up to pa / qa columns readable, multiples of 8, zero past P / Q),
// fp32, the rows cut into `splits` partials (part: splits * P * Q floats)
// summed in order.
hipError_t launch_gemm_tn(const uint16_t* A, int64_t lda, int64_t pa, const uint16_t* B, int64_t ldb, int64_t qa,
                          int64_t P, int64_t Q, int64_t M, int splits, float* part, float* out, hipStream_t s);

// ----------------------------------------------------------------------------
// Grouped (mixture-of-experts) forward: E experts stacked at fixed strides
// (elements of each array per expert), rows [eoff[e], eoff[e+1]) of X go to
// expert e; t16 is the bf16 T = X_e A_cat,e scratch [T][r_pad], r_pad a
// multiple of 32.
struct MoeArgs {
  const uint64_t* masks;
  const uint16_t* values;
  const uint32_t* offsets;
  const uint16_t* a_cat;
  const uint16_t* b_cat;
  size_t mstride, vstride, ostride, astride, bstride;
  const uint16_t* X;
  uint16_t* Y;
  const int32_t* eoff;
  uint16_t* t16;
  float* tpart;            // fp32 partials of T over K ranges [ksplits][T][r_pad]
  int64_t N;
  int32_t E, T, K, n_keep, r_cat, r_pad, kw, ng;
  int32_t ksplits, kspan;  // K ranges of the low-rank partials, columns per range (multiple of 128)
};
// K ranges of the grouped low-rank partials for T rows, and workspace bytes
// that hold their partials for any T' <= T (bf16 T follows them).
int moe_lowrank_splits(int64_t T, int64_t K, int r_pad);
size_t moe_lowrank_part_bytes(int64_t T, int64_t K, int r_pad);
// m_cap: the expected most rows of one expert (sets the low-rank grid; any
// count is computed correctly).
hipError_t launch_moe_forward(const MoeArgs& a, int32_t m_cap, hipStream_t s);

// ----------------------------------------------------------------------------
// Encode kernels.
// ----------------------------------------------------------------------------
struct PrunePackArgs {
  const uint16_t* W;       // [N][K]
  uint64_t* masks;
  uint16_t* values;
  uint32_t* offsets;
  uint16_t* R;             // [N][K] residual (bf16), may be null
  uint32_t* nonfinite;     // set to 1 if W holds Inf/NaN
  int64_t N;
  int32_t K, n_keep, kw, ng;
};
hipError_t launch_prune_pack(const PrunePackArgs& a, hipStream_t s);

}  // namespace salr
