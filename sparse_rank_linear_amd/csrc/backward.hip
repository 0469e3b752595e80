// Backward pass of the SALR layer for fine-tuning the adapters with the base
// weight frozen (gist.science summary of "Sparsity-Aware Low-Rank
// Representation ...", Methodology 2: the SVD residual adapter is trained
// together with the LoRA adapters; Methodology 1: the mask applies to the
// frozen base weight only).  For Y = X W_s^T + (X A_cat) B_cat and dY:
//   dX = dY W_s + (dY B_cat^T) A_cat^T,  dA_cat = X^T (dY B_cat^T),
//   dB_cat = (X A_cat)^T dY.
// dX is a forward of the transposed layer (W_s^T with adapters B_cat^T,
// A_cat^T), run by the forward kernels on a column-major copy of W_s's
// encoding built here once; the adapter gradients contract over the tokens
// straight from the token-major X, dY, G and T (tiles transposed in LDS).
//
// Transposed encoding (W_s^T, K rows of N columns), built tile-parallel:
//   1. rowpre[n][w]: kept values of row n before bitmap word w;
//   2. per 64-row block b and word w, one wave transposes the 64 x 64 bit
//      tile with 64 ballots (ballot k collects bit k of the 64 rows' words,
//      i.e. column k's word for the block) and counts each column's bits;
//   3. colpre[b][k]: kept rows of column k before block b (a scan over b),
//      the column counts, their maximum and the lookup table of W_s^T;
//   4. the same waves scatter the values: column k's kept rows in block b
//      land at colpre[b][k] onward, in row order.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "salr_device.hpp"
#include "salr_kernels.hpp"

namespace salr {
namespace {

// 1. one thread per row: exclusive running counts of the row's words
__global__ __launch_bounds__(256) void row_prefix_kernel(const uint64_t* masks, int64_t N, int32_t kw,
                                                         uint32_t* rowpre) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  uint32_t run = 0;
  for (int w = 0; w < kw; ++w) {
    rowpre[n * kw + w] = run;
    run += (uint32_t)__popcll(masks[n * kw + w]);
  }
}

// 2. wave per (block b, word w): column counts of the tile (and, with
// masks_t, the transposed bitmap words)
__device__ __forceinline__ uint64_t tile_column_word(uint64_t rw, int lane) {
  uint64_t mine = 0;
#pragma unroll 8
  for (int k = 0; k < 64; ++k) {
    const uint64_t b = __ballot((rw >> k) & 1ull);
    if (lane == k) mine = b;
  }
  return mine;
}

__global__ __launch_bounds__(256) void tile_counts_kernel(const uint64_t* masks, int64_t N, int32_t K, int32_t kw,
                                                          int32_t nb, uint32_t* cnt) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // tile id = b * kw + w
  if (t >= (int64_t)nb * kw) return;
  const int b = (int)(t / kw), w = (int)(t % kw);
  const int64_t n = (int64_t)b * 64 + lane;
  const uint64_t rw = n < N ? masks[n * kw + w] : 0ull;
  const uint64_t mine = tile_column_word(rw, lane);
  const int k = w * 64 + lane;
  if (k < K) cnt[(size_t)b * K + k] = (uint32_t)__popcll(mine);
}

// 3. thread per column: exclusive scan of the block counts (in place), the
// column's total, the lookup table of W_s^T and the largest count
__global__ __launch_bounds__(256) void column_scan_kernel(uint32_t* cnt, int32_t nb, int32_t K, uint32_t* offsets_t,
                                                          int32_t ng_t, uint32_t* maxcount) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  uint32_t run = 0;
  for (int b = 0; b < nb; ++b) {
    // (entry g of the table: kept rows before row 1024 g = 16 blocks of 64)
    if (offsets_t && (b & 15) == 0) offsets_t[(size_t)k * ng_t + (b >> 4)] = run;
    const uint32_t c = cnt[(size_t)b * K + k];
    cnt[(size_t)b * K + k] = run;
    run += c;
  }
  atomicMax(maxcount, run);
}

// 4. wave per (block b, word w): transposed bitmap word and value scatter
__global__ __launch_bounds__(256) void transpose_scatter_kernel(const uint64_t* masks, const uint16_t* values,
                                                                const uint32_t* rowpre, const uint32_t* colpre,
                                                                int64_t N, int32_t K, int32_t kw, int32_t n_keep,
                                                                int32_t nb, int32_t kw_t, int32_t n_keep_t,
                                                                uint64_t* masks_t, uint16_t* values_t) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= (int64_t)nb * kw) return;
  const int b = (int)(t / kw), w = (int)(t % kw);
  const int64_t n = (int64_t)b * 64 + lane;
  const uint64_t rw = n < N ? masks[n * kw + w] : 0ull;
  const uint32_t rp = n < N ? rowpre[n * kw + w] : 0u;
  const uint64_t mine = tile_column_word(rw, lane);  // column (w, lane)'s bits over the block's rows
  const int k = w * 64 + lane;
  const bool live = k < K;
  if (live) masks_t[(size_t)k * kw_t + b] = mine;
  uint32_t pos = live ? colpre[(size_t)b * K + k] : 0u;
  const uint64_t below = (1ull << lane) - 1ull;
  // rows of the block in order (all lanes active: row j's word and running
  // count are read from lane j); a lane whose column row j keeps copies that
  // value to the next slot of its column
  for (int j = 0; j < 64; ++j) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)rw, j);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(rw >> 32), j);
    const uint64_t wj = ((uint64_t)hi << 32) | lo;
    if (wj == 0ull) continue;
    const uint32_t rpj = (uint32_t)__builtin_amdgcn_readlane((int)rp, j);
    if (live && ((wj >> lane) & 1ull)) {
      values_t[(size_t)k * n_keep_t + pos] = values[((int64_t)b * 64 + j) * n_keep + rpj + __popcll(wj & below)];
      ++pos;
    }
  }
}

// bf16 [R][C] -> [C][ld_dst] transposes through LDS, 64 x 64 tiles; the
// destination row stride is ld_dst (>= R; the columns past R are zero).  One
// launch does two of them (blockIdx.z picks the job; blocks past a job's
// tiles leave).  A tile whose 64 columns lie inside C and whose rows start
// on 16 bytes is read with 16-byte loads, others element by element.
struct TransposeJob {
  const uint16_t* src;
  int64_t R, C, ld_src;
  uint16_t* dst;
  int64_t ld_dst;
};
__global__ __launch_bounds__(256) void transpose_bf16_tiles(TransposeJob j0, TransposeJob j1) {
  __shared__ uint16_t tile[64][65];
  const TransposeJob j = blockIdx.z == 0 ? j0 : j1;
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  if (c0 >= j.C || r0 >= (j.R > j.ld_dst ? j.R : j.ld_dst)) return;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const bool vec = c0 + 64 <= j.C && (j.ld_src & 7) == 0 && ((uintptr_t)j.src & 15) == 0;
  if (vec) {
    const int ch = threadIdx.x & 7, y0 = threadIdx.x >> 3;  // 8 chunks of a row, 32 rows a pass
    for (int y = y0; y < 64; y += 32) {
      const int64_t r = r0 + y;
      const u32x4_t v = r < j.R ? load16(j.src + r * j.ld_src + c0 + 8 * ch) : zero_u4();
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tile[y][8 * ch + 2 * e] = (uint16_t)v[e];
        tile[y][8 * ch + 2 * e + 1] = (uint16_t)(v[e] >> 16);
      }
    }
  } else {
    for (int y = ty; y < 64; y += 4) {
      const int64_t r = r0 + y, c = c0 + tx;
      tile[y][tx] = (r < j.R && c < j.C) ? j.src[r * j.ld_src + c] : (uint16_t)0;
    }
  }
  __syncthreads();
  for (int y = ty; y < 64; y += 4) {
    const int64_t c = c0 + y, r = r0 + tx;
    if (c < j.C && r < j.ld_dst) j.dst[c * j.ld_dst + r] = tile[tx][y];
  }
}

// Token contraction: part[split][p][q] = sum over rows m of the split of
// A[m][p] B[m][q] (bf16, rows of lda / ldb elements, fp32 products).  A
// workgroup owns 64 x 64 outputs, 4 waves of 32 x 32 (2 x 2 MFMA tiles; a
// 16-row tile past P or Q is skipped).  Per 64 rows of m it stages both
// 64 x 64 tiles in LDS transposed (k = m contiguous, the MFMA operand
// layout): each thread loads two consecutive rows of 8 columns with 16-byte
// loads and stores each column's pair of values as one 32-bit word; the
// next 64 rows' loads are requested before the current rows are multiplied.
// Loads read up to pa / qa columns (multiples of 8; the caller guarantees
// they exist, zero past P / Q).
constexpr int kTnPitch = 72;  // LDS row: 64 values of m + 8 (16-row operand reads on distinct banks)
__global__ __launch_bounds__(256) void gemm_tn_kernel(const uint16_t* A, int64_t lda, int64_t pa, const uint16_t* B,
                                                      int64_t ldb, int64_t qa, int64_t P, int64_t Q, int64_t M,
                                                      int64_t m_split, float* part) {
  __shared__ __attribute__((aligned(16))) uint16_t at[64 * kTnPitch];
  __shared__ __attribute__((aligned(16))) uint16_t bt[64 * kTnPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int64_t p0 = (int64_t)blockIdx.y * 64, q0 = (int64_t)blockIdx.x * 64;
  const int64_t mb = (int64_t)blockIdx.z * m_split, me = min(M, mb + m_split);
  const int wp = (wave >> 1) * 32, wq = (wave & 1) * 32;
  // staging role: rows 2 rp, 2 rp + 1 of the 64, 8 columns from c = 8 (tid % 8)
  const int rp = tid >> 3, c = 8 * (tid & 7);
  const bool pa_ok = p0 + c < pa, qa_ok = q0 + c < qa;
  f32x4_t acc[2][2] = {{zero4(), zero4()}, {zero4(), zero4()}};
  u32x4_t va[2], vb[2];
  const auto load_rows = [&](int64_t m0) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t m = m0 + 2 * rp + h;
      va[h] = (m < me && pa_ok) ? load16(A + m * lda + p0 + c) : zero_u4();
      vb[h] = (m < me && qa_ok) ? load16(B + m * ldb + q0 + c) : zero_u4();
    }
  };
  // 32-bit view of the tiles: column j's values for rows 2 rp, 2 rp + 1
  uint32_t* const at32 = reinterpret_cast<uint32_t*>(at);
  uint32_t* const bt32 = reinterpret_cast<uint32_t*>(bt);
  const bool live_x[2] = {p0 + wp < P, p0 + wp + 16 < P};
  const bool live_y[2] = {q0 + wq < Q, q0 + wq + 16 < Q};
  if (mb < me) load_rows(mb);
  for (int64_t m0 = mb; m0 < me; m0 += 64) {
    __syncthreads();  // (the previous step's operand reads are done)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // columns c + 2e (low halves) and c + 2e + 1 (high halves)
      at32[(c + 2 * e) * (kTnPitch / 2) + rp] = __builtin_amdgcn_perm(va[1][e], va[0][e], 0x05040100u);
      at32[(c + 2 * e + 1) * (kTnPitch / 2) + rp] = __builtin_amdgcn_perm(va[1][e], va[0][e], 0x07060302u);
      bt32[(c + 2 * e) * (kTnPitch / 2) + rp] = __builtin_amdgcn_perm(vb[1][e], vb[0][e], 0x05040100u);
      bt32[(c + 2 * e + 1) * (kTnPitch / 2) + rp] = __builtin_amdgcn_perm(vb[1][e], vb[0][e], 0x07060302u);
    }
    __syncthreads();
    if (m0 + 64 < me) load_rows(m0 + 64);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      u32x4_t a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = *reinterpret_cast<const u32x4_t*>(&at[(wp + 16 * t + i) * kTnPitch + 32 * kh + 8 * g]);
        b[t] = *reinterpret_cast<const u32x4_t*>(&bt[(wq + 16 * t + i) * kTnPitch + 32 * kh + 8 * g]);
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
          if (live_x[x] && live_y[y]) acc[x][y] = mfma_16x16x32(a[x], b[y], acc[x][y]);
    }
  }
  // lane holds C[p0 + wp + 16x + 4g + e][q0 + wq + 16y + i]
  float* out = part + (size_t)blockIdx.z * P * Q;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t p = p0 + wp + 16 * x + 4 * g + e, q = q0 + wq + 16 * y + i;
        const float v = acc[x][y][e];
        if (p < P && q < Q) out[p * Q + q] = v;
      }
}

__global__ __launch_bounds__(256) void sum_parts_kernel(const float* part, int splits, int64_t n, float* out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float s = 0.f;
  for (int sp = 0; sp < splits; ++sp) s += part[(size_t)sp * n + e];
  out[e] = s;
}

}  // namespace

hipError_t launch_transpose_count(const uint64_t* masks, int64_t N, int32_t K, uint32_t* rowpre, uint32_t* cnt,
                                  uint32_t* maxcount, uint32_t* offsets_t, int32_t ng_t, hipStream_t s) {
  const int32_t kw = (K + 63) / 64, nb = (int32_t)((N + 63) / 64);
  hipLaunchKernelGGL(row_prefix_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, masks, N, kw, rowpre);
  const int64_t tiles = (int64_t)nb * kw;
  hipLaunchKernelGGL(tile_counts_kernel, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, s, masks, N, K, kw, nb,
                     cnt);
  hipLaunchKernelGGL(column_scan_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, s, cnt, nb, K, offsets_t,
                     ng_t, maxcount);
  return hipGetLastError();
}

hipError_t launch_transpose_scatter(const uint64_t* masks, const uint16_t* values, const uint32_t* rowpre,
                                    const uint32_t* colpre, int64_t N, int32_t K, int32_t n_keep, int32_t n_keep_t,
                                    uint64_t* masks_t, uint16_t* values_t, hipStream_t s) {
  const int32_t kw = (K + 63) / 64, nb = (int32_t)((N + 63) / 64);
  const int64_t tiles = (int64_t)nb * kw;
  hipLaunchKernelGGL(transpose_scatter_kernel, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, s, masks, values,
                     rowpre, colpre, N, K, kw, n_keep, nb, nb, n_keep_t, masks_t, values_t);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16_pair(const uint16_t* src0, int64_t R0, int64_t C0, int64_t ld_src0, uint16_t* dst0,
                                      int64_t ld_dst0, const uint16_t* src1, int64_t R1, int64_t C1, int64_t ld_src1,
                                      uint16_t* dst1, int64_t ld_dst1, hipStream_t s) {
  const TransposeJob j0{src0, R0, C0, ld_src0, dst0, ld_dst0}, j1{src1, R1, C1, ld_src1, dst1, ld_dst1};
  const auto tiles_x = [](const TransposeJob& j) { return (j.C + 63) / 64; };
  const auto tiles_y = [](const TransposeJob& j) { return (std::max<int64_t>(j.R, j.ld_dst) + 63) / 64; };
  const int64_t gx = std::max(tiles_x(j0), tiles_x(j1)), gy = std::max(tiles_y(j0), tiles_y(j1));
  if (gx == 0 || gy == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_bf16_tiles, dim3((unsigned)gx, (unsigned)gy, 2), dim3(256), 0, s, j0, j1);
  return hipGetLastError();
}

hipError_t launch_gemm_tn(const uint16_t* A, int64_t lda, int64_t pa, const uint16_t* B, int64_t ldb, int64_t qa,
                          int64_t P, int64_t Q, int64_t M, int splits, float* part, float* out, hipStream_t s) {
  if (P == 0 || Q == 0) return hipSuccess;
  const int64_t n = P * Q;
  if (M <= 0) {  // (an empty sum: zeros)
    hipLaunchKernelGGL(sum_parts_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, 0, n, out);
    return hipGetLastError();
  }
  const int64_t m_split = ((M + splits - 1) / splits + 63) / 64 * 64;
  splits = (int)((M + m_split - 1) / m_split);
  if (splits < 1) splits = 1;
  const dim3 grid((unsigned)((Q + 63) / 64), (unsigned)((P + 63) / 64), (unsigned)splits);
  // (one split: straight into the output)
  hipLaunchKernelGGL(gemm_tn_kernel, grid, dim3(256), 0, s, A, lda, pa, B, ldb, qa, P, Q, M, m_split,
                     splits == 1 ? out : part);
  if (splits > 1)
    hipLaunchKernelGGL(sum_parts_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, splits, n, out);
  return hipGetLastError();
}

}  // namespace salr
