// Host orchestration of salr_encode (selection/packing, residual truncated
// SVD, adapter concatenation).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace salr {

struct EncodeParams {
  const uint16_t* W;
  int64_t N, K;
  int32_t n_keep, r_svd, r_cat;
  int32_t n_lora;
  const uint16_t* const* lora_A;  // host array of device pointers
  const uint16_t* const* lora_B;
  const int32_t* lora_r;          // host
  int32_t oversample, iters;
  uint64_t seed;
  uint64_t* masks;
  uint16_t* values;
  uint32_t* offsets;
  uint16_t* a_cat;
  uint16_t* b_cat;
  double* sigma;                  // host, r_svd entries or null
  void* ws;
  size_t ws_bytes;
  hipStream_t stream;
};

// Basis width of the subspace iteration for a rank-r truncation.
int32_t svd_basis(int64_t N, int64_t K, int32_t r_svd, int32_t oversample);
size_t encode_ws_bytes(int64_t N, int64_t K, int32_t r_svd, int32_t oversample);
// Returns a salr_status_t value.
int encode_run(const EncodeParams& p);

}  // namespace salr
