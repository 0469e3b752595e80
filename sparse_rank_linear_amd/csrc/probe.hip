// Measurement probes (include/salr_probe.h): the achievable HBM read rate
// and bf16 matrix-core rate of this GPU, against which the forward kernels'
// roofline fractions are also reported.
#include "salr_probe.h"

#include <hip/hip_runtime.h>

#include "salr.h"
#include "salr_device.hpp"

namespace salr {
namespace {

constexpr int kReadThreads = 512;
constexpr int kReadUnroll = 4;  // 16-byte loads in flight per thread per step

// Workgroup w reads the 8 KB blocks w, w + G, w + 2G, ... (G workgroups),
// kReadUnroll blocks per step; lanes read consecutive 16-byte chunks.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4_t* src, int64_t chunks,
                                                                   uint32_t* sink) {
  const int64_t G = gridDim.x;
  const int64_t blk_chunks = kReadThreads;
  u32x4_t acc = zero_u4();
  int64_t b = blockIdx.x;
  const int64_t nblk = (chunks + blk_chunks - 1) / blk_chunks;
  for (; b + (kReadUnroll - 1) * G < nblk; b += kReadUnroll * G) {
    u32x4_t v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const int64_t c = (b + u * G) * blk_chunks + threadIdx.x;
      v[u] = c < chunks ? src[c] : zero_u4();
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  for (; b < nblk; b += G) {
    const int64_t c = b * blk_chunks + threadIdx.x;
    if (c < chunks) acc ^= src[c];
  }
  __shared__ uint32_t red[kReadThreads / 64];
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int w = 0; w < kReadThreads / 64; ++w) s ^= red[w];
    sink[blockIdx.x] = s;
  }
}

// Independent matrix-core chains per wave; operands depend on the lane so
// nothing folds at compile time.
template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_peak_kernel(float* out, int iters) {
  const uint32_t lane = threadIdx.x & 63;
  const u32x4_t a = u32x4_t{0x3F803F80u ^ lane, 0x3F803F81u, 0x3F823F80u, 0x3F803F83u ^ (lane << 1)};
  const u32x4_t b = u32x4_t{0x3C003C00u, 0x3C013C00u ^ lane, 0x3C003C02u, 0x3C033C00u};
  float sum = 0.f;
  if constexpr (SHAPE == 0) {
    f32x4_t acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = zero4();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = mfma_16x16x32(a, b, acc[c]);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) sum += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  } else {
    f32x16_t acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = mfma_32x32x16(a, b, acc[c]);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += acc[c][e];
  }
  __shared__ float red[4];
  if (lane == 0) red[threadIdx.x >> 6] = sum;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

}  // namespace
}  // namespace salr

extern "C" {

int salr_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups, void* stream) {
  if (!src || !sink || (reinterpret_cast<uintptr_t>(src) & 15u) || (bytes & 15u) || bytes == 0)
    return SALR_ERR_INVALID_ARG;
  if (workgroups < 1 || workgroups > 65536) return SALR_ERR_INVALID_ARG;
  hipLaunchKernelGGL(salr::stream_read_kernel, dim3((unsigned)workgroups), dim3(salr::kReadThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const salr::u32x4_t*>(src),
                     (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? SALR_OK : SALR_ERR_HIP;
}

int salr_probe_mfma(float* out, int32_t workgroups, int32_t iters, int32_t shape, void* stream) {
  if (!out || workgroups < 1 || workgroups > 65536 || iters < 1 || iters > (1 << 24) || (shape != 0 && shape != 1))
    return SALR_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (shape == 0)
    hipLaunchKernelGGL(salr::mfma_peak_kernel<0>, dim3((unsigned)workgroups), dim3(256), 0, s, out, iters);
  else
    hipLaunchKernelGGL(salr::mfma_peak_kernel<1>, dim3((unsigned)workgroups), dim3(256), 0, s, out, iters);
  return hipGetLastError() == hipSuccess ? SALR_OK : SALR_ERR_HIP;
}

}  // extern "C"
