// Launch interfaces of the SALR HIP kernels (host side of each .hip file).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace salr {

// ----------------------------------------------------------------------------
// Forward, M <= 16: one fused launch.  Producer workgroups compute
// T = X * A_cat; consumer workgroups decode 16 rows x 1024 columns of W_s
// each, multiply, reduce their K-splits and finish with the low-rank term.
// ----------------------------------------------------------------------------
struct SmallFwdArgs {
  const uint64_t* masks;
  const uint16_t* values;
  const uint32_t* offsets;
  const uint16_t* a_cat;   // [r_cat][K]
  const uint16_t* b_cat;   // [N][r_cat]
  const uint16_t* X;       // [M][K]
  uint16_t* Y;             // [M][N]
  int64_t N;
  int32_t K, n_keep, r_cat, M;
  int32_t kw, ng;          // words / lookup entries per row
  int32_t n_tiles;         // ceil(N/16) row tiles
  int32_t splits;          // consumer K-splits (= ng, 1024 columns each)
  int32_t r_tiles;         // ceil(r_cat/16)
  int32_t t_splits;        // producer K-splits
  int32_t t_chunk;         // producer K columns per split (multiple of 128)
  int32_t r_pad;           // row stride of tbuf (multiple of 32)
  uint32_t* sync;          // [0] T tiles ready, [1] finished row tiles, [2] error
  uint32_t* tcount;        // [r_tiles]
  uint32_t* ycount;        // [n_tiles]
  uint16_t* tbuf;          // [16][r_pad] bf16 T
  float* tpart;            // [r_tiles][t_splits][256]
  float* ypart;            // [n_tiles][splits][256]
};
hipError_t launch_fwd_small(const SmallFwdArgs& a, hipStream_t s);

// ----------------------------------------------------------------------------
// Forward, M > 16: T = X * A_cat (bf16, [M][r_pad]) then the tiled
// decode + MFMA kernel with the low-rank term as extra K steps.
// ----------------------------------------------------------------------------
struct LowRankTArgs {
  const uint16_t* X;       // [M][K]
  const uint16_t* a_cat;   // [r_cat][K]
  uint16_t* T;             // [M][r_pad]
  float* tpart;            // [ceil(M/64)][splits][64][r_pad]
  uint32_t* count;         // [ceil(M/64)]
  int32_t M, K, r_cat, r_pad;
  int32_t splits, k_chunk; // K-splits, columns per split (multiple of 64)
};
hipError_t launch_lowrank_t(const LowRankTArgs& a, hipStream_t s);

struct LargeFwdArgs {
  const uint64_t* masks;
  const uint16_t* values;
  const uint16_t* b_cat;   // [N][r_cat]
  const uint16_t* X;       // [M][K]
  const uint16_t* T;       // [M][r_pad] or null when r_cat == 0
  uint16_t* Y;             // [M][N]
  int64_t N;
  int32_t K, n_keep, r_cat, r_pad, M;
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
