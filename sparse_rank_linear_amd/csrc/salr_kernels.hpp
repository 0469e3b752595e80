// Launch interfaces of the SALR HIP kernels (host side of each .hip file).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace salr {

constexpr int kMaxRangeCols = 4096;  // columns per few-row workgroup

// ----------------------------------------------------------------------------
// Forward, M <= 16: one fused launch.  Each workgroup decodes 16 rows x one
// column range of W_s and multiplies; the first workgroups also compute the
// pieces of T = X * A_cat; range partials and T meet in each row tile's
// finishing workgroup, which adds the low-rank term.
// ----------------------------------------------------------------------------
struct SmallFwdArgs {
  const uint64_t* masks;
  const uint16_t* values;
  const uint32_t* offsets;
  const uint16_t* b_cat;   // [N][r_cat] (+ tail padding)
  const uint16_t* X;       // [M][K]
  uint16_t* Y;             // [M][N]
  const float* tsum;       // [t_pieces][16][r_pad] partial T (when r_cat > 0)
  int64_t N;
  int32_t K, n_keep, r_cat, M;
  int32_t kw, ng;          // words / lookup entries per row
  int32_t n_tiles;         // ceil(N/16) row tiles
  int32_t splits;          // column ranges per row (1 = whole rows)
  int32_t range;           // columns per range (K when splits == 1, else 1024/2048/4096)
  int32_t vcap;            // 16-byte chunks of LDS per row
  int32_t r_tiles;         // ceil(r_cat/16)
  int32_t r_pad;           // rank stride of tsum (multiple of 32)
  int32_t t_pieces;        // K ranges of tsum
  int32_t vals_bytes;      // LDS bytes of the values area
  int32_t tl_bytes;        // LDS bytes of the T partials (t_pieces * 16 * r_pad * 4)
  int32_t bl_bytes;        // LDS bytes of the B_cat rows (16 * r_cat * 2, rounded up to 16)
  int32_t done_groups;     // groups of the two-level completion count
  uint32_t* sync;          // [0] epoch, [1] finished groups, [2] error
  uint32_t* gdone;         // [done_groups] finished workgroups per group
  uint32_t* ycount;        // [n_tiles]
  uint64_t* ypart;         // [n_tiles][splits][256] tagged fp32
};
hipError_t launch_fwd_small(const SmallFwdArgs& a, hipStream_t s);
size_t fwd_small_vals_bytes(int vcap);
// Dynamic LDS bytes of one few-row workgroup.
size_t fwd_small_lds_bytes(int vcap, int tl_bytes, int bl_bytes);
// LDS chunks per row for rows whose staged values never exceed `cap`: room
// for the misaligned start and the decode window's overrun, rounded to a
// stride of 1 mod 8 chunks so consecutive rows start 4 banks apart.
inline int fwd_small_vcap(int64_t cap) {
  const int v = (int)((cap + 16) / 8 + 2);
  return v + ((1 - v % 8) + 8) % 8;
}

// T = X * A_cat for M <= 16, as t_pieces partial sums over K ranges.
struct SmallTArgs {
  const uint16_t* X;       // [M][K]
  const uint16_t* a_cat;   // [r_cat][K]
  float* tsum;             // [t_pieces][16][r_pad]
  int32_t M, K, r_cat, r_pad, r_tiles;
  int32_t t_pieces, k_range;  // K ranges (k_range columns each, <= 2048)
};
hipError_t launch_lowrank_t_small(const SmallTArgs& a, hipStream_t s);

// ----------------------------------------------------------------------------
// Forward, M > 16: T = X * A_cat (bf16, [M][r_pad]) then the tiled
// decode + MFMA kernel with the low-rank term as extra K steps.
// ----------------------------------------------------------------------------
struct LowRankTArgs {
  const uint16_t* X;       // [M][K]
  const uint16_t* a_cat;   // [r_cat][K]
  float* tpart;            // [splits][M][r_pad] fp32 partial sums of X A_cat
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
  uint16_t* Y;             // [M][N]
  int64_t N;
  int32_t K, n_keep, r_cat, r_pad, M;
  int32_t t_splits;
  int32_t kw;
  int64_t vchunks;         // ceil(N * n_keep / 8): 16-byte chunks of values
};
hipError_t launch_fwd_large(const LargeFwdArgs& a, hipStream_t s);

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
