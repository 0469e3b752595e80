// QSALR value codec: 4-bit NormalFloat (NF4) codes for the packed kept
// values of W_s (gist.science summary of "Sparsity-Aware Low-Rank
// Representation ...", Experimental Results, Ablation Studies,
// "Quantization": SALR combined with NF4 quantization).
//
// NF4 is the NormalFloat data type of "QLoRA: Efficient Finetuning of
// Quantized LLMs" (Dettmers et al., 2023): 16 levels at quantiles of the
// standard normal distribution with an exact zero, scaled into [-1, 1], used
// per block with the block's absolute maximum as scale.  Here a block is 64
// consecutive kept values of one row (a row's last block may be shorter),
// its scale the largest |value| (a bf16 value itself, stored exactly), a
// value's code the level nearest to value / scale in float32 (ties to the
// lower level), and the decoded value bf16(level * scale) in float32.
#include <hip/hip_runtime.h>

#include <cmath>

#include "salr_device.hpp"
#include "salr_kernels.hpp"

namespace salr {
namespace {

// Standard normal quantile by bisection on the CDF 0.5 erfc(-x / sqrt 2),
// to the last representable double.
double normal_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 4096; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (0.5 * std::erfc(-mid / std::sqrt(2.0)) < p)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

// Evenly spaced probabilities from `start` towards 0.5 (step (0.5 - start) /
// div), as start + k * step with no fused multiply-add.
double spaced(double start, int k, int div) {
#pragma clang fp contract(off)
  const double step = (0.5 - start) / (double)div;
  const double t = (double)k * step;
  return t + start;
}

constexpr int kQThreads = 256;  // 4 waves, one 64-value block each

__global__ __launch_bounds__(kQThreads) void quantize_nf4_kernel(const uint16_t* values, int64_t N, int32_t n_keep,
                                                                 int32_t nblk, int32_t cb_row, Nf4Levels lv,
                                                                 uint8_t* codes, uint16_t* scales) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * (kQThreads / 64) + (threadIdx.x >> 6);
  if (blk >= N * nblk) return;
  const int64_t row = blk / nblk;
  const int b = (int)(blk - row * nblk);
  const int j = b * 64 + lane;
  const bool live = j < n_keep;
  const uint32_t bits = live ? values[row * n_keep + j] : 0u;
  // scale: the largest magnitude (bf16 magnitudes order like integers)
  uint32_t mag = bits & 0x7FFFu;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mag = max(mag, (uint32_t)__shfl_xor((int)mag, o));
  const float s = bf16_to_f32((uint16_t)mag);
  uint32_t code = kNf4ZeroCode;
  if (mag != 0u) {
    const float x = __fdiv_rn(bf16_to_f32((uint16_t)bits), s);
    float best = fabsf(x - lv.v[0]);
    code = 0;
#pragma unroll
    for (int c = 1; c < 16; ++c) {
      const float d = fabsf(x - lv.v[c]);
      if (d < best) {  // (strict: the lower level keeps a tie)
        best = d;
        code = (uint32_t)c;
      }
    }
  }
  if (!live) code = 0u;  // (padding codes of a row's last block)
  const uint32_t hi = (uint32_t)__shfl_down((int)code, 1);
  if ((lane & 1) == 0) codes[row * cb_row + b * 32 + (lane >> 1)] = (uint8_t)(code | (hi << 4));
  if (lane == 0) scales[row * nblk + b] = (uint16_t)mag;
}

// bf16 values [N][n_keep] from codes and scales (8 values a thread).
__global__ __launch_bounds__(256) void dequantize_nf4_kernel(const uint8_t* codes, const uint16_t* scales, int64_t N,
                                                             int32_t n_keep, int32_t nblk, int32_t cb_row,
                                                             Nf4Levels lv, uint16_t* values) {
  const int64_t groups = (n_keep + 7) / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= N * groups) return;
  const int64_t row = t / groups;
  const int j0 = (int)(t - row * groups) * 8;
  const uint32_t cw = *reinterpret_cast<const uint32_t*>(codes + row * cb_row + j0 / 2);  // (j0 % 8 == 0)
  const float s = bf16_to_f32(scales[row * nblk + j0 / 64]);  // (8 values never straddle a block)
  uint16_t* dst = values + row * n_keep + j0;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (j0 + e < n_keep) dst[e] = f32_to_bf16(lv.v[(cw >> (4 * e)) & 15u] * s);
}

}  // namespace

void nf4_levels(float out[16]) {
  const double top = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0);
  double lev[16];
  int n = 0;
  for (int k = 0; k < 7; ++k) lev[n++] = -normal_quantile(spaced(top, k, 7));  // 7 below zero
  lev[n++] = 0.0;
  for (int k = 7; k >= 0; --k) lev[n++] = normal_quantile(spaced(top, k, 8));  // 8 above zero
  const double big = lev[15];
  for (int c = 0; c < 16; ++c) out[c] = (float)(lev[c] / big);
}

hipError_t launch_quantize_nf4(const uint16_t* values, int64_t N, int32_t n_keep, uint8_t* codes, uint16_t* scales,
                               hipStream_t s) {
  Nf4Levels lv;
  nf4_levels(lv.v);
  const int32_t nblk = (n_keep + 63) / 64;
  const int64_t blocks = N * nblk;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_nf4_kernel, dim3((unsigned)((blocks + 3) / 4)), dim3(kQThreads), 0, s, values, N, n_keep,
                     nblk, nblk * 32, lv, codes, scales);
  return hipGetLastError();
}

hipError_t launch_dequantize_nf4(const uint8_t* codes, const uint16_t* scales, int64_t N, int32_t n_keep,
                                 uint16_t* values, hipStream_t s) {
  Nf4Levels lv;
  nf4_levels(lv.v);
  const int32_t nblk = (n_keep + 63) / 64;
  const int64_t threads = N * ((n_keep + 7) / 8);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(dequantize_nf4_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, codes, scales,
                     N, n_keep, nblk, nblk * 32, lv, values);
  return hipGetLastError();
}

}  // namespace salr
