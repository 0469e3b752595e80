// Multi-projection fusion: several encoded layers that read the same input
// become one encoded layer.
//
// Method: gist.science summary of "Sparsity-Aware Low-Rank Representation
// ...", Methodology 3 (every adapter runs as one low-rank product on the
// shared input), applied across projections that share an input (q/k/v,
// gate/up): their W_s rows are stacked, their A_cat rows are stacked, and
// B_cat becomes block diagonal, so one forward call computes all of them.
#include <algorithm>

#include "salr_kernels.hpp"

namespace salr {
namespace {

// dst rows [0, rows) of the fused B_cat (row stride r_dst): columns
// [col0, col0 + r_src) take the part's coefficients, every other column is 0.
__global__ __launch_bounds__(256) void fuse_b_kernel(const uint16_t* src, int64_t rows, int r_src, uint16_t* dst,
                                                     int r_dst, int col0) {
  const int64_t total = rows * r_dst;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = e / r_dst;
    const int j = (int)(e - n * r_dst) - col0;
    dst[e] = (j >= 0 && j < r_src) ? src[n * r_src + j] : (uint16_t)0;
  }
}

}  // namespace

hipError_t launch_fuse_b(const uint16_t* src, int64_t rows, int r_src, uint16_t* dst, int r_dst, int col0,
                         hipStream_t s) {
  const int64_t total = rows * r_dst;
  if (total == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(fuse_b_kernel, dim3(grid), dim3(256), 0, s, src, rows, r_src, dst, r_dst, col0);
  return hipGetLastError();
}

}  // namespace salr
