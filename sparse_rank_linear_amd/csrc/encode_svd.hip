// SALR encode, residual truncated SVD and adapter concatenation.
//
// Method: gist.science summary of "Sparsity-Aware Low-Rank Representation
// ...", Methodology 2 (rank-r truncated SVD of the pruning residual, used as
// an extra low-rank adapter) and Methodology 3 (all adapters stacked along
// the rank dimension).  The factor split is balanced: A' = V_r sqrt(S_r),
// B' = sqrt(S_r) U_r^T.
//
// The pages fix neither the SVD algorithm nor its precision.  On the GPU the
// leading singular subspace of R (N x K, bf16-exact) is found by randomized
// subspace iteration (Halko, Martinsson and Tropp, "Finding structure with
// randomness", 2011, Algorithm 4.4) with a basis of l = r + p columns:
//     Y = R Omega;  repeat q times: Q = orth(Y), Z = orth(R^T Q), Y = R Z;
//     Q = orth(Y);  Bt = R^T Q;  eig(Bt^T Bt) = U diag(lambda) U^T;
//     sigma = sqrt(lambda),  A'^T = diag(sigma^-1/2) U_r^T Bt^T,
//     B'^T = Q U_r diag(sigma^1/2).
// orth() is Cholesky QR: once per half-step inside the iteration (only the
// span matters there; the next product and orth() carry on from any
// well-conditioned basis), twice for the final Q, whose orthonormality the
// small eigenproblem relies on (the second pass repairs the first one's
// loss of orthogonality).  The products with R run on bf16 matrix cores
// with the fp32 basis split into two bf16 parts (v_mfma_f32_16x16x32_bf16),
// the basis' own products on fp32 ones (v_mfma_f32_16x16x4_f32); the l x l
// Cholesky and the symmetric eigen
// problem run in fp64 inside one workgroup (cyclic Jacobi, round-robin
// pairing).  Omega is Gaussian from a counter-based generator (SplitMix64,
// Steele, Lea and Flood 2014, fed to the Box-Muller transform).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "salr.h"
#include "salr_device.hpp"
#include "salr_encode.hpp"
#include "salr_kernels.hpp"

namespace salr {
namespace {

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// Generic strided fp32 GEMM: C(i,j) = alpha * sum_k A(i,k) B(k,j)
//   A(i,k) = A[i*sa0 + k*sa1] (bf16 or fp32), B(k,j) = B[k*sb0 + j*sb1] (fp32)
//   C(i,j) = C[i*sc0 + j*sc1]; with k_split > 1 the K range is split over
//   blockIdx.z and partial sums are added atomically (C must start at 0).
// 64x64 tile, 16-deep K tile, 4 waves of 32x32 (2x2 MFMA 16x16x4 tiles).
// ---------------------------------------------------------------------------
struct GemmArgs {
  int64_t M, N, K;
  const void* A;
  int a_bf16;
  int64_t sa0, sa1;
  const float* B;
  int64_t sb0, sb1;
  float* C;
  int64_t sc0, sc1;
  float alpha;
  int k_split;
  int64_t k_chunk;
};

__device__ __forceinline__ float load_a(const GemmArgs& g, int64_t off) {
  return g.a_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(g.A)[off]) : static_cast<const float*>(g.A)[off];
}

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t i0 = (int64_t)blockIdx.y * 64, j0 = (int64_t)blockIdx.x * 64;
  const int64_t kb = (int64_t)blockIdx.z * g.k_chunk;
  const int64_t ke = std::min<int64_t>(g.K, kb + g.k_chunk);
  const bool a_kcontig = g.sa1 == 1;
  const bool b_jcontig = g.sb1 == 1;
  f32x4_t acc[2][2] = {{zero4(), zero4()}, {zero4(), zero4()}};

  for (int64_t k0 = kb; k0 < ke; k0 += 16) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int ii, kk;
      if (a_kcontig) { ii = tid >> 2; kk = (tid & 3) * 4 + u; }
      else           { kk = tid >> 4; ii = (tid & 15) * 4 + u; }
      const int64_t gi = i0 + ii, gk = k0 + kk;
      As[kk][ii] = (gi < g.M && gk < ke) ? load_a(g, gi * g.sa0 + gk * g.sa1) : 0.f;
      int jj, k2;
      if (b_jcontig) { k2 = tid >> 4; jj = (tid & 15) * 4 + u; }
      else           { jj = tid >> 2; k2 = (tid & 3) * 4 + u; }
      const int64_t gj = j0 + jj, gk2 = k0 + k2;
      Bs[k2][jj] = (gj < g.N && gk2 < ke) ? g.B[gk2 * g.sb0 + gj * g.sb1] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = As[4 * ks + lg][wm * 32 + 16 * t + li];
        b[t] = Bs[4 * ks + lg][wn * 32 + 16 * t + li];
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[x], b[y], acc[x][y], 0, 0, 0);
    }
    __syncthreads();
  }
  // lane holds C(wm*32 + 16x + 4lg + e, wn*32 + 16y + li)
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t gi = i0 + wm * 32 + 16 * x + 4 * lg + e;
        const int64_t gj = j0 + wn * 32 + 16 * y + li;
        if (gi < g.M && gj < g.N) {
          float* dst = &g.C[gi * g.sc0 + gj * g.sc1];
          const float v = g.alpha * acc[x][y][e];
          if (g.k_split > 1) atomicAdd(dst, v);
          else *dst = v;
        }
      }
}

// ---------------------------------------------------------------------------
// Products with the residual on the bf16 matrix cores.  R is exact in bf16;
// the fp32 basis B is split into two bf16 parts, B = B_hi + B_lo + e with
// |e| <= 2^-17 |B|, and C = R B_hi + R B_lo accumulates in fp32
// (v_mfma_f32_16x16x32_bf16, exact products).  Both operands are read
// k-contiguous: A row-major [M][Kd] (R, or R^T materialised once), B as
// transposed parts Bh/Bl [l_pad][ld] with zeros past l and past Kd.
// ---------------------------------------------------------------------------

// dst[c][r] = src[r][c] for a rows x cols bf16 matrix (64 x 64 tiles via LDS);
// the 32 elements after dst's end (its tail room) are zeroed, so that a
// product reading past the last row meets finite values.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* src, int64_t rows, int64_t cols,
                                                             uint16_t* dst) {
  __shared__ uint16_t t[64][66];
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 32) dst[rows * cols + threadIdx.x] = 0;
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int y = ty; y < 64; y += 4) {
    const int64_t r = r0 + y, c = c0 + tx;
    t[y][tx] = (r < rows && c < cols) ? src[r * cols + c] : (uint16_t)0;
  }
  __syncthreads();
  for (int y = ty; y < 64; y += 4) {
    const int64_t c = c0 + y, r = r0 + tx;
    if (c < cols && r < rows) dst[c * rows + r] = t[tx][y];
  }
}

// Bh[c][k] = bf16(B[k][c]), Bl[c][k] = bf16(B[k][c] - Bh[c][k]) (both
// round to nearest even); zero for c >= l or k >= kd.  B fp32 [kd][l];
// tiles of 64 k x 32 c via LDS.
__global__ __launch_bounds__(256) void split_t_kernel(const float* B, int64_t kd, int l, uint16_t* Bh, uint16_t* Bl,
                                                      int64_t ld) {
  __shared__ float t[64][33];
  const int64_t k0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int y = ty; y < 64; y += 8) {
    const int64_t k = k0 + y;
    const int c = c0 + tx;
    t[y][tx] = (k < kd && c < l) ? B[k * l + c] : 0.f;
  }
  __syncthreads();
  const int kx = threadIdx.x & 63, cy = threadIdx.x >> 6;
  for (int y = cy; y < 32; y += 4) {
    const float v = t[kx][y];
    const uint16_t hi = f32_to_bf16(v);
    const uint16_t lo = f32_to_bf16(v - bf16_to_f32(hi));
    const int64_t o = (int64_t)(c0 + y) * ld + k0 + kx;
    Bh[o] = hi;
    Bl[o] = lo;
  }
}

// C[m][c] (+)= sum_k A[m][k] (Bh[c][k] + Bl[c][k]) over this workgroup's K
// range [blockIdx.y * k_chunk, +k_chunk).  Workgroup: 4 waves in CG column
// groups x 4/CG row groups of 64 rows (4 MFMA row tiles each); wave w takes
// row group w / CG and the column tiles w % CG, w % CG + CG, ... (CT of
// them).  Waves of one row group share its row tiles' loads in L1, and the
// basis is read once per 64 x 4/CG rows.  Rows past M read row M-1
// and columns past Kd read a group ending at most 7 past the row (their B
// is zero); neither is
// stored.  With split K the partial sums are added atomically (C zeroed
// first).  A needs 16 bytes of readable room past its last row.
template <int CT, int CG>
__global__ __launch_bounds__(256) void gemm_bf16x2_kernel(const uint16_t* A, int64_t lda, const uint16_t* Bh,
                                                          const uint16_t* Bl, int64_t ldb, float* C, int64_t M, int l,
                                                          int64_t Kd, int64_t k_chunk, int atomic) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int lt = (l + 15) / 16;
  constexpr int RG = 4 / CG;
  const int cg = wave % CG;
  const int64_t m0 = (int64_t)blockIdx.x * 64 * RG + 64 * (wave / CG);
  const int64_t kb = (int64_t)blockIdx.y * k_chunk, ke = std::min<int64_t>(Kd, kb + k_chunk);
  const int64_t kd8 = (Kd + 7) / 8 * 8;
  const uint16_t* arow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) arow[t] = A + std::min<int64_t>(m0 + 16 * t + i, M - 1) * lda;
  const uint16_t* bhr[CT];
  const uint16_t* blr[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int ct = std::min(cg + CG * c, lt - 1);
    bhr[c] = Bh + (int64_t)(16 * ct + i) * ldb + 8 * g;
    blr[c] = Bl + (int64_t)(16 * ct + i) * ldb + 8 * g;
  }
  f32x4_t acc[4][CT];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[t][c] = zero4();
  for (int64_t k = kb; k < ke; k += 32) {
    // (Kd need not be a multiple of 8: the last group may read up to 7
    // elements past a row, which meet B's zeros; the buffers have tail room)
    const int64_t ka = std::min<int64_t>(k + 8 * g, kd8 - 8);
    u32x4_t a[4], bh[CT], bl[CT];
#pragma unroll
    for (int t = 0; t < 4; ++t) a[t] = load16(arow[t] + ka);
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      bh[c] = load16(bhr[c] + k);
      bl[c] = load16(blr[c] + k);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        acc[t][c] = mfma_16x16x32(a[t], bh[c], acc[t][c]);
        acc[t][c] = mfma_16x16x32(a[t], bl[c], acc[t][c]);
      }
  }
  // lane holds C[m0 + 16t + 4g + e][16 ct + i]
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int ct = cg + CG * c;
    const int col = 16 * ct + i;
    if (ct >= lt || col >= l) continue;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t m = m0 + 16 * t + 4 * g + e;
        if (m >= M) continue;
        const float v = acc[t][c][e];  // (scalar copy first: see the few-row forward)
        if (atomic) atomicAdd(&C[m * l + col], v);
        else C[m * l + col] = v;
      }
  }
}

__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

// SplitMix64 finaliser: a bijective mix of a 64-bit counter.
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

__global__ void gaussian_kernel(float* p, int64_t n, uint64_t seed) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const uint64_t h = splitmix64(seed * 0x100000001B3ull + (uint64_t)i);
    const float u1 = ((float)(uint32_t)(h >> 40) + 1.0f) * (1.0f / 16777216.0f);  // (0, 1]
    const float u2 = (float)(uint32_t)(h & 0xFFFFFFu) * (1.0f / 16777216.0f);     // [0, 1)
    p[i] = sqrtf(-2.0f * logf(u1)) * cosf(6.28318530717958647692f * u2);
  }
}

// ---------------------------------------------------------------------------
// One-workgroup fp64 Cholesky of G (l x l, fp32, symmetric PSD) followed by
// the upper-triangular C = L^{-T}, so that Y C has orthonormal columns when
// G = Y^T Y.  A pivot below tol * max(diag) marks a direction Y does not
// span (to working precision); its row and column of C are zero.
// ---------------------------------------------------------------------------
constexpr int kSmallThreads = 1024;

__global__ __launch_bounds__(kSmallThreads) void chol_inv_kernel(const float* G, float* C, double* L, double* Li,
                                                                 int l, double tol_rel) {
  __shared__ double piv_sh;
  __shared__ double maxd_sh;
  const int tid = threadIdx.x;
  for (int e = tid; e < l * l; e += kSmallThreads) L[e] = (double)G[e];
  __syncthreads();
  if (tid == 0) {
    double m = 0.0;
    for (int d = 0; d < l; ++d) m = fmax(m, L[d * l + d]);
    maxd_sh = m;
  }
  __syncthreads();
  const double tol = tol_rel * maxd_sh;
  for (int j = 0; j < l; ++j) {
    if (tid == 0) {
      const double p = L[j * l + j];
      piv_sh = (p > tol && p > 0.0) ? sqrt(p) : 0.0;
    }
    __syncthreads();
    const double d = piv_sh;
    // column j below the diagonal
    for (int i = j + 1 + tid; i < l; i += kSmallThreads) L[i * l + j] = d > 0.0 ? L[i * l + j] / d : 0.0;
    if (tid == 0) L[j * l + j] = d;
    __syncthreads();
    // trailing update of the lower triangle
    const int rem = l - j - 1;
    for (int e = tid; e < rem * rem; e += kSmallThreads) {
      const int i = j + 1 + e / rem, k = j + 1 + e % rem;
      if (k <= i) L[i * l + k] -= L[i * l + j] * L[k * l + j];
    }
    __syncthreads();
  }
  // Li = L^{-1}: eliminate column k from all rows below it, k ascending
  // (right-looking forward substitution on the identity, rows of a dropped
  // pivot are zero).
  for (int e = tid; e < l * l; e += kSmallThreads) Li[e] = (e / l == e % l) ? 1.0 : 0.0;
  __syncthreads();
  for (int k = 0; k < l; ++k) {
    const double d = L[k * l + k];
    for (int c = tid; c <= k; c += kSmallThreads) Li[k * l + c] = d > 0.0 ? Li[k * l + c] / d : 0.0;
    __syncthreads();
    const int rem = l - k - 1;
    for (int e = tid; e < rem * (k + 1); e += kSmallThreads) {
      const int i = k + 1 + e / (k + 1), c = e % (k + 1);
      Li[i * l + c] -= L[i * l + k] * Li[k * l + c];
    }
    __syncthreads();
  }
  // C = Li^T
  for (int e = tid; e < l * l; e += kSmallThreads) {
    const int i = e / l, k = e % l;
    C[e] = (float)Li[k * l + i];
  }
}

// The same factorization with the matrix in registers (l <= kRegChol):
// thread (ty, tx) of a 32 x 32 grid holds the entries (ty + 32x, tx + 32y),
// x, y < NB.  Cholesky step j: the holders of column j publish it (pivot
// included) to LDS, the holder of the pivot also its square root and
// reciprocal, then after one barrier every thread applies the rank-1 update
// to its own entries.  The published columns stay in LDS (packed, column j
// at pk(j) = j*l - j*(j-1)/2) and give L for the inverse, which runs the same
// way over the rows of Li = L^{-1} (one published row per step, two row
// buffers in turn).  Every LDS access of a step is a broadcast or
// consecutive doubles, so no bank conflicts.  A zero pivot gives a zero
// column of L and a zero row of Li, as in chol_inv_kernel; the arithmetic
// differs from it only in multiplying by the reciprocal of the pivot.
constexpr int kRegChol = 160;

__device__ inline int packed_col(int j, int l) { return j * l - (j * (j - 1)) / 2; }

template <int NB>
__global__ __launch_bounds__(kSmallThreads) void chol_inv_reg_kernel(const float* G, float* C, int l, double tol_rel) {
  extern __shared__ double sm[];
  double* Lt = sm;                          // packed columns of L before scaling
  double* rowb = Lt + (l * (l + 1)) / 2;    // [2][l] published rows of Li
  double* dv = rowb + 2 * l;                // pivots' square roots (diagonal of L)
  double* rdv = dv + l;                     // their reciprocals (0 for a zero pivot)
  __shared__ double wmax[kSmallThreads / 64];
  const int tid = threadIdx.x;
  const int tx = tid & 31, ty = tid >> 5;
  double a[NB][NB];
#pragma unroll
  for (int x = 0; x < NB; ++x)
#pragma unroll
    for (int y = 0; y < NB; ++y) {
      const int i = ty + 32 * x, k = tx + 32 * y;
      a[x][y] = (i < l && k < l) ? (double)G[(int64_t)i * l + k] : 0.0;
    }
  // tolerance from the largest diagonal entry
  double m = 0.0;
#pragma unroll
  for (int x = 0; x < NB; ++x)
#pragma unroll
    for (int y = 0; y < NB; ++y)
      if (ty + 32 * x == tx + 32 * y && ty + 32 * x < l) m = fmax(m, a[x][y]);
  for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  double maxd = 0.0;
  for (int w = 0; w < kSmallThreads / 64; ++w) maxd = fmax(maxd, wmax[w]);
  const double tol = tol_rel * maxd;

  for (int j = 0; j < l; ++j) {
    const int pj = packed_col(j, l);
    if (tx == (j & 31)) {
#pragma unroll
      for (int y = 0; y < NB; ++y) {
        if (y != (j >> 5)) continue;
#pragma unroll
        for (int x = 0; x < NB; ++x) {
          const int i = ty + 32 * x;
          if (i < j || i >= l) continue;
          Lt[pj + i - j] = a[x][y];
          if (i == j) {
            const double p = a[x][y];
            const double d = (p > tol && p > 0.0) ? sqrt(p) : 0.0;
            dv[j] = d;
            rdv[j] = d > 0.0 ? 1.0 / d : 0.0;
          }
        }
      }
    }
    __syncthreads();
    const double rd = rdv[j];
    double li[NB], lk[NB];
#pragma unroll
    for (int x = 0; x < NB; ++x) {
      const int i = ty + 32 * x;
      li[x] = (i > j && i < l) ? Lt[pj + i - j] * rd : 0.0;
      const int k = tx + 32 * x;
      lk[x] = (k > j && k < l) ? Lt[pj + k - j] * rd : 0.0;
    }
#pragma unroll
    for (int x = 0; x < NB; ++x)
#pragma unroll
      for (int y = 0; y < NB; ++y) a[x][y] -= li[x] * lk[y];
  }

  // Li by rows: row k is final once divided by L[k][k]; rows below take
  // X[i][c] -= L[i][k] * Li[k][c] (c <= k)
#pragma unroll
  for (int x = 0; x < NB; ++x)
#pragma unroll
    for (int y = 0; y < NB; ++y) a[x][y] = (ty + 32 * x == tx + 32 * y) ? 1.0 : 0.0;
  for (int k = 0; k < l; ++k) {
    double* rb = rowb + (k & 1) * l;
    const double rk = rdv[k];
    if (ty == (k & 31)) {
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        if (x != (k >> 5)) continue;
#pragma unroll
        for (int y = 0; y < NB; ++y) {
          const int c = tx + 32 * y;
          if (c > k) continue;
          a[x][y] *= rk;
          rb[c] = a[x][y];
        }
      }
    }
    __syncthreads();
    const int pk = packed_col(k, l);
    double lik[NB], xr[NB];
#pragma unroll
    for (int x = 0; x < NB; ++x) {
      const int i = ty + 32 * x;
      lik[x] = (i > k && i < l) ? Lt[pk + i - k] * rk : 0.0;
      const int c = tx + 32 * x;
      xr[x] = c <= k ? rb[c] : 0.0;
    }
#pragma unroll
    for (int x = 0; x < NB; ++x)
#pragma unroll
      for (int y = 0; y < NB; ++y) a[x][y] -= lik[x] * xr[y];
  }
  // C = Li^T
#pragma unroll
  for (int x = 0; x < NB; ++x)
#pragma unroll
    for (int y = 0; y < NB; ++y) {
      const int i = ty + 32 * x, c = tx + 32 * y;
      if (i < l && c < l) C[(int64_t)c * l + i] = (float)a[x][y];
    }
}

size_t chol_reg_lds_bytes(int l) { return ((size_t)l * (l + 1) / 2 + 4 * (size_t)l) * 8; }

void launch_chol_inv_reg(hipStream_t s, const float* G, float* C, int l, double tol_rel) {
  const size_t sh = chol_reg_lds_bytes(l);
  switch ((l + 31) / 32) {
    case 1: hipLaunchKernelGGL(chol_inv_reg_kernel<1>, dim3(1), dim3(kSmallThreads), sh, s, G, C, l, tol_rel); break;
    case 2: hipLaunchKernelGGL(chol_inv_reg_kernel<2>, dim3(1), dim3(kSmallThreads), sh, s, G, C, l, tol_rel); break;
    case 3: hipLaunchKernelGGL(chol_inv_reg_kernel<3>, dim3(1), dim3(kSmallThreads), sh, s, G, C, l, tol_rel); break;
    case 4: hipLaunchKernelGGL(chol_inv_reg_kernel<4>, dim3(1), dim3(kSmallThreads), sh, s, G, C, l, tol_rel); break;
    default: hipLaunchKernelGGL(chol_inv_reg_kernel<5>, dim3(1), dim3(kSmallThreads), sh, s, G, C, l, tol_rel); break;
  }
}

// ---------------------------------------------------------------------------
// One-workgroup fp64 cyclic Jacobi eigensolver of a symmetric l x l matrix
// (fp32 input S).  Rotations of one round act on disjoint index pairs from
// the round-robin (circle) schedule, so a round is: compute all rotations,
// rotate rows, rotate columns (of the matrix and of the eigenvector
// matrix).  Output: eigenvalues in descending order (fp64) and the matching
// eigenvectors as columns of U (fp32).
// ---------------------------------------------------------------------------
constexpr int kMaxPairs = 256;

__global__ __launch_bounds__(kSmallThreads) void jacobi_kernel(const float* S, double* A, double* V, double* evals,
                                                               float* U, int l, int max_sweeps) {
  __shared__ double cs[kMaxPairs], sn[kMaxPairs];
  __shared__ int pp[kMaxPairs], qq[kMaxPairs];
  __shared__ double red[kSmallThreads];
  __shared__ int order[512];
  const int tid = threadIdx.x;
  const int n = l + (l & 1);  // even number of players; index l (if any) is a dummy
  const int npairs = n / 2;
  for (int e = tid; e < l * l; e += kSmallThreads) {
    const int i = e / l, j = e % l;
    A[e] = 0.5 * ((double)S[i * l + j] + (double)S[j * l + i]);
    V[e] = (i == j) ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int sweep = 0; sweep < max_sweeps; ++sweep) {
    // convergence: off-diagonal mass vs diagonal mass
    double off = 0.0, dia = 0.0;
    for (int e = tid; e < l * l; e += kSmallThreads) {
      const int i = e / l, j = e % l;
      const double v = A[e] * A[e];
      if (i == j) dia += v; else off += v;
    }
    red[tid] = off;
    __syncthreads();
    for (int s = kSmallThreads / 2; s > 0; s >>= 1) {
      if (tid < s) red[tid] += red[tid + s];
      __syncthreads();
    }
    const double off_t = red[0];
    __syncthreads();
    red[tid] = dia;
    __syncthreads();
    for (int s = kSmallThreads / 2; s > 0; s >>= 1) {
      if (tid < s) red[tid] += red[tid + s];
      __syncthreads();
    }
    const double dia_t = red[0];
    __syncthreads();
    if (off_t <= 1e-30 * (dia_t + 1e-300) || off_t == 0.0) break;

    for (int round = 0; round < n - 1; ++round) {
      if (tid < npairs) {
        int p, q;
        if (tid == 0) { p = n - 1; q = round; }
        else { p = (round + tid) % (n - 1); q = (round - tid + (n - 1)) % (n - 1); }
        if (p > q) { const int t = p; p = q; q = t; }
        double c = 1.0, s = 0.0;
        if (q < l) {
          const double apq = A[p * l + q];
          if (fabs(apq) > 1e-300) {
            const double theta = (A[q * l + q] - A[p * l + p]) / (2.0 * apq);
            const double t = (theta >= 0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
            c = 1.0 / sqrt(t * t + 1.0);
            s = t * c;
          }
        }
        pp[tid] = p; qq[tid] = q; cs[tid] = c; sn[tid] = s;
      }
      __syncthreads();
      // rows: A <- J^T A
      for (int e = tid; e < npairs * l; e += kSmallThreads) {
        const int k = e / l, j = e % l;
        const int p = pp[k], q = qq[k];
        if (q >= l) continue;
        const double c = cs[k], s = sn[k];
        const double ap = A[p * l + j], aq = A[q * l + j];
        A[p * l + j] = c * ap - s * aq;
        A[q * l + j] = s * ap + c * aq;
      }
      __syncthreads();
      // columns: A <- A J, V <- V J
      for (int e = tid; e < npairs * l; e += kSmallThreads) {
        const int k = e / l, i = e % l;
        const int p = pp[k], q = qq[k];
        if (q >= l) continue;
        const double c = cs[k], s = sn[k];
        const double ap = A[i * l + p], aq = A[i * l + q];
        A[i * l + p] = c * ap - s * aq;
        A[i * l + q] = s * ap + c * aq;
        const double vp = V[i * l + p], vq = V[i * l + q];
        V[i * l + p] = c * vp - s * vq;
        V[i * l + q] = s * vp + c * vq;
      }
      __syncthreads();
    }
  }
  // sort eigenvalues descending (rank by counting)
  for (int i = tid; i < l; i += kSmallThreads) {
    const double di = A[i * l + i];
    int rank = 0;
    for (int j = 0; j < l; ++j) {
      const double dj = A[j * l + j];
      rank += (dj > di) || (dj == di && j < i);
    }
    order[rank] = i;
  }
  __syncthreads();
  for (int r = tid; r < l; r += kSmallThreads) evals[r] = A[order[r] * l + order[r]];
  for (int e = tid; e < l * l; e += kSmallThreads) {
    const int i = e / l, r = e % l;
    U[i * l + r] = (float)V[i * l + order[r]];
  }
}

// The same eigensolver with A and V in LDS (l <= kLdsJacobi) and the row and
// column updates on a 32 x 32 thread grid (no index division): same
// rotations, same order per element, as jacobi_kernel.  Rows are l + 1
// doubles apart, so the column updates (32 lanes down one column) fall in
// distinct banks.
constexpr int kLdsJacobi = 96;

__global__ __launch_bounds__(kSmallThreads) void jacobi_lds_kernel(const float* S, double* evals, float* U, int l,
                                                                   int max_sweeps) {
  extern __shared__ double sm[];
  double* A = sm;           // [l][l + 1]
  double* V = sm + l * (l + 1);   // [l][l + 1]
  __shared__ double cs[kMaxPairs], sn[kMaxPairs];
  __shared__ int pp[kMaxPairs], qq[kMaxPairs];
  __shared__ double red[2 * (kSmallThreads / 64)];  // per-wave sums (off, diagonal)
  __shared__ int order[512];
  const int tid = threadIdx.x;
  const int ld = l + 1;
  const int tx = tid & 31, ty = tid >> 5;
  const int n = l + (l & 1);  // even number of players; index l (if any) is a dummy
  const int npairs = n / 2;
  for (int i = ty; i < l; i += 32)
    for (int j = tx; j < l; j += 32) {
      A[i * ld + j] = 0.5 * ((double)S[i * l + j] + (double)S[j * l + i]);
      V[i * ld + j] = (i == j) ? 1.0 : 0.0;
    }
  __syncthreads();
  for (int sweep = 0; sweep < max_sweeps; ++sweep) {
    // convergence: off-diagonal mass vs diagonal mass
    double off = 0.0, dia = 0.0;
    for (int i = ty; i < l; i += 32)
      for (int j = tx; j < l; j += 32) {
        const double v = A[i * ld + j] * A[i * ld + j];
        if (i == j) dia += v; else off += v;
      }
    for (int o = 32; o > 0; o >>= 1) {
      off += __shfl_xor(off, o);
      dia += __shfl_xor(dia, o);
    }
    if ((tid & 63) == 0) {
      red[2 * (tid >> 6)] = off;
      red[2 * (tid >> 6) + 1] = dia;
    }
    __syncthreads();
    double off_t = 0.0, dia_t = 0.0;
    for (int w = 0; w < kSmallThreads / 64; ++w) {
      off_t += red[2 * w];
      dia_t += red[2 * w + 1];
    }
    __syncthreads();
    if (off_t <= 1e-30 * (dia_t + 1e-300) || off_t == 0.0) break;

    for (int round = 0; round < n - 1; ++round) {
      if (tid < npairs) {
        int p, q;
        if (tid == 0) { p = n - 1; q = round; }
        else { p = (round + tid) % (n - 1); q = (round - tid + (n - 1)) % (n - 1); }
        if (p > q) { const int t = p; p = q; q = t; }
        double c = 1.0, sv = 0.0;
        if (q < l) {
          const double apq = A[p * ld + q];
          if (fabs(apq) > 1e-300) {
            const double theta = (A[q * ld + q] - A[p * ld + p]) / (2.0 * apq);
            const double t = (theta >= 0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
            c = 1.0 / sqrt(t * t + 1.0);
            sv = t * c;
          }
        }
        pp[tid] = p; qq[tid] = q; cs[tid] = c; sn[tid] = sv;
      }
      __syncthreads();
      // rows: A <- J^T A
      for (int k = ty; k < npairs; k += 32) {
        const int p = pp[k], q = qq[k];
        if (q >= l) continue;
        const double c = cs[k], sv = sn[k];
        for (int j = tx; j < l; j += 32) {
          const double ap = A[p * ld + j], aq = A[q * ld + j];
          A[p * ld + j] = c * ap - sv * aq;
          A[q * ld + j] = sv * ap + c * aq;
        }
      }
      __syncthreads();
      // columns: A <- A J, V <- V J
      for (int k = ty; k < npairs; k += 32) {
        const int p = pp[k], q = qq[k];
        if (q >= l) continue;
        const double c = cs[k], sv = sn[k];
        for (int i = tx; i < l; i += 32) {
          const double ap = A[i * ld + p], aq = A[i * ld + q];
          A[i * ld + p] = c * ap - sv * aq;
          A[i * ld + q] = sv * ap + c * aq;
          const double vp = V[i * ld + p], vq = V[i * ld + q];
          V[i * ld + p] = c * vp - sv * vq;
          V[i * ld + q] = sv * vp + c * vq;
        }
      }
      __syncthreads();
    }
  }
  // sort eigenvalues descending (rank by counting)
  for (int i = tid; i < l; i += kSmallThreads) {
    const double di = A[i * ld + i];
    int rank = 0;
    for (int j = 0; j < l; ++j) {
      const double dj = A[j * ld + j];
      rank += (dj > di) || (dj == di && j < i);
    }
    order[rank] = i;
  }
  __syncthreads();
  for (int r = tid; r < l; r += kSmallThreads) evals[r] = A[order[r] * ld + order[r]];
  for (int i = ty; i < l; i += 32)
    for (int r = tx; r < l; r += 32) U[i * l + r] = (float)V[i * ld + order[r]];
}

// The same eigensolver for bases too wide for two fp64 matrices in LDS
// (l <= kMidJacobi): A in LDS as fp32 (its input, the Gram matrix, is fp32
// already), the eigenvectors in global memory (fp32, L2-resident), and a
// stopping test suited to fp32 entries.
constexpr int kMidJacobi = 190;  // 4 l (l + 1) bytes of LDS
__global__ __launch_bounds__(kSmallThreads) void jacobi_mid_kernel(const float* S, double* evals, float* U, float* V, int l,
                                                                   int max_sweeps) {
  extern __shared__ float smf[];
  float* A = smf;           // [l][l + 1] in LDS; V [l][l + 1] in global memory
  __shared__ double cs[kMaxPairs], sn[kMaxPairs];
  __shared__ int pp[kMaxPairs], qq[kMaxPairs];
  __shared__ double red[2 * (kSmallThreads / 64)];  // per-wave sums (off, diagonal)
  __shared__ int order[512];
  const int tid = threadIdx.x;
  const int ld = l + 1;
  const int tx = tid & 31, ty = tid >> 5;
  const int n = l + (l & 1);  // even number of players; index l (if any) is a dummy
  const int npairs = n / 2;
  for (int i = ty; i < l; i += 32)
    for (int j = tx; j < l; j += 32) {
      A[i * ld + j] = 0.5f * (S[i * l + j] + S[j * l + i]);
      V[i * ld + j] = (i == j) ? 1.f : 0.f;
    }
  __syncthreads();
  for (int sweep = 0; sweep < max_sweeps; ++sweep) {
    // convergence: off-diagonal mass vs diagonal mass
    double off = 0.0, dia = 0.0;
    for (int i = ty; i < l; i += 32)
      for (int j = tx; j < l; j += 32) {
        const double v = (double)A[i * ld + j] * (double)A[i * ld + j];
        if (i == j) dia += v; else off += v;
      }
    for (int o = 32; o > 0; o >>= 1) {
      off += __shfl_xor(off, o);
      dia += __shfl_xor(dia, o);
    }
    if ((tid & 63) == 0) {
      red[2 * (tid >> 6)] = off;
      red[2 * (tid >> 6) + 1] = dia;
    }
    __syncthreads();
    double off_t = 0.0, dia_t = 0.0;
    for (int w = 0; w < kSmallThreads / 64; ++w) {
      off_t += red[2 * w];
      dia_t += red[2 * w + 1];
    }
    __syncthreads();
    // (fp32 entries: stop once the off-diagonal norm is 1e-6 of the diagonal's)
    if (off_t <= 1e-12 * (dia_t + 1e-300) || off_t == 0.0) break;

    for (int round = 0; round < n - 1; ++round) {
      if (tid < npairs) {
        int p, q;
        if (tid == 0) { p = n - 1; q = round; }
        else { p = (round + tid) % (n - 1); q = (round - tid + (n - 1)) % (n - 1); }
        if (p > q) { const int t = p; p = q; q = t; }
        double c = 1.0, sv = 0.0;
        if (q < l) {
          const double apq = A[p * ld + q];
          if (fabs(apq) > 1e-30) {
            const double theta = ((double)A[q * ld + q] - (double)A[p * ld + p]) / (2.0 * apq);
            const double t = (theta >= 0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
            c = 1.0 / sqrt(t * t + 1.0);
            sv = t * c;
          }
        }
        pp[tid] = p; qq[tid] = q; cs[tid] = c; sn[tid] = sv;
      }
      __syncthreads();
      // rows: A <- J^T A
      for (int k = ty; k < npairs; k += 32) {
        const int p = pp[k], q = qq[k];
        if (q >= l) continue;
        const float c = (float)cs[k], sv = (float)sn[k];
        for (int j = tx; j < l; j += 32) {
          const float ap = A[p * ld + j], aq = A[q * ld + j];
          A[p * ld + j] = c * ap - sv * aq;
          A[q * ld + j] = sv * ap + c * aq;
        }
      }
      __syncthreads();
      // columns: A <- A J, V <- V J
      for (int k = ty; k < npairs; k += 32) {
        const int p = pp[k], q = qq[k];
        if (q >= l) continue;
        const float c = (float)cs[k], sv = (float)sn[k];
        for (int i = tx; i < l; i += 32) {
          const float ap = A[i * ld + p], aq = A[i * ld + q];
          A[i * ld + p] = c * ap - sv * aq;
          A[i * ld + q] = sv * ap + c * aq;
          const float vp = V[i * ld + p], vq = V[i * ld + q];
          V[i * ld + p] = c * vp - sv * vq;
          V[i * ld + q] = sv * vp + c * vq;
        }
      }
      __syncthreads();
    }
  }
  // sort eigenvalues descending (rank by counting)
  for (int i = tid; i < l; i += kSmallThreads) {
    const float di = A[i * ld + i];
    int rank = 0;
    for (int j = 0; j < l; ++j) {
      const float dj = A[j * ld + j];
      rank += (dj > di) || (dj == di && j < i);
    }
    order[rank] = i;
  }
  __syncthreads();
  for (int r = tid; r < l; r += kSmallThreads) evals[r] = (double)A[order[r] * ld + order[r]];
  for (int i = ty; i < l; i += 32)
    for (int r = tx; r < l; r += 32) U[i * l + r] = V[i * ld + order[r]];
}

// a_cat rows [0, r): a_cat[i][k] = bf16(P[k][i] / sqrt(sigma_i)), P = Bt U_r.
__global__ void write_a_kernel(const float* P, const double* evals, uint16_t* a_cat, int64_t K, int r) {
  const int i = blockIdx.y;
  const double lam = evals[i];
  const double sg = lam > 0 ? sqrt(lam) : 0.0;
  const float scale = sg > 1e-30 ? (float)(1.0 / sqrt(sg)) : 0.f;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < K; k += (int64_t)gridDim.x * blockDim.x)
    a_cat[(int64_t)i * K + k] = f32_to_bf16(P[k * r + i] * scale);
}

// b_cat columns [0, r): b_cat[n][i] = bf16(S2[n][i] * sqrt(sigma_i)), S2 = Q U_r.
__global__ void write_b_kernel(const float* S2, const double* evals, uint16_t* b_cat, int64_t N, int r, int r_cat) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < N * r; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = e / r;
    const int i = (int)(e % r);
    const double lam = evals[i];
    const double sg = lam > 0 ? sqrt(lam) : 0.0;
    b_cat[n * r_cat + i] = f32_to_bf16(S2[e] * (float)sqrt(sg));
  }
}

// LoRA blocks: a_cat rows [row0, row0 + q) <- lora_A [q][K]; b_cat columns
// [row0, row0 + q) <- lora_B [N][q].  Bit copies.
__global__ void copy_lora_kernel(const uint16_t* la, const uint16_t* lb, uint16_t* a_cat, uint16_t* b_cat,
                                 int64_t N, int64_t K, int q, int row0, int r_cat) {
  const int64_t na = (int64_t)q * K, nb = N * q;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < na + nb; e += (int64_t)gridDim.x * blockDim.x) {
    if (e < na) {
      a_cat[(int64_t)row0 * K + e] = la[e];
    } else {
      const int64_t f = e - na, n = f / q;
      const int j = (int)(f % q);
      b_cat[n * r_cat + row0 + j] = lb[f];
    }
  }
}

struct EncodeLayout {
  int l;
  int64_t ldb;  // row stride of the split basis parts (max(N, K) rounded up to 64)
  size_t R, Rt, Bh, Bl, Y, Q, Z, Z2, G, C, dA, dB, dC, evals, U, flags, total;
};

EncodeLayout encode_layout(int64_t N, int64_t K, int32_t r_svd, int32_t oversample) {
  EncodeLayout L{};
  L.l = svd_basis(N, K, r_svd, oversample);
  const size_t l = (size_t)std::max(L.l, 1);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes, 256); return o; };
  L.flags = take(64);
  L.R = take((size_t)N * K * 2 + 64);   // (+ tail room for the product's last group)
  L.Rt = take((size_t)N * K * 2 + 64);
  L.ldb = (std::max(N, K) + 63) / 64 * 64;
  const size_t lp = (l + 31) / 32 * 32;
  L.Bh = take(lp * (size_t)L.ldb * 2);
  L.Bl = take(lp * (size_t)L.ldb * 2);
  L.Y = take((size_t)N * l * 4);
  L.Q = take((size_t)N * l * 4);
  L.Z = take((size_t)K * l * 4);
  L.Z2 = take((size_t)K * l * 4);
  L.G = take(l * l * 4);
  L.C = take(l * l * 4);
  L.dA = take(l * l * 8);
  L.dB = take(l * l * 8);
  L.dC = take(l * l * 8);
  L.evals = take(l * 8);
  L.U = take(l * l * 4);
  L.total = off;
  return L;
}

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

hipError_t gemm(hipStream_t s, int64_t M, int64_t N, int64_t K, const void* A, bool a_bf16, int64_t sa0, int64_t sa1,
                const float* B, int64_t sb0, int64_t sb1, float* C, int64_t sc0, int64_t sc1, int k_split = 1) {
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.a_bf16 = a_bf16 ? 1 : 0; g.sa0 = sa0; g.sa1 = sa1;
  g.B = B; g.sb0 = sb0; g.sb1 = sb1;
  g.C = C; g.sc0 = sc0; g.sc1 = sc1;
  g.alpha = 1.0f;
  g.k_chunk = align_up((size_t)cdiv(K, k_split), 16);
  g.k_split = (int)cdiv(K, g.k_chunk);
  if (g.k_split > 1) {
    hipLaunchKernelGGL(fill_f32_kernel, dim3(256), dim3(256), 0, s, C, M * N, 0.0f);  // C is dense here
  }
  dim3 grid((unsigned)cdiv(N, 64), (unsigned)cdiv(M, 64), (unsigned)g.k_split);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

// C [M][l] = A [M][Kd] (bf16, row-major, row stride lda) * B [Kd][l] (fp32)
// on the bf16 matrix cores (B split into two bf16 parts).
hipError_t gemm_r(hipStream_t s, const uint16_t* A, int64_t lda, int64_t M, int64_t Kd, const float* B, int l, float* C,
                  const EncodeLayout& E, void* ws) {
  uint16_t* Bh = at<uint16_t>(ws, E.Bh);
  uint16_t* Bl = at<uint16_t>(ws, E.Bl);
  const int lp = (l + 31) / 32;
  hipLaunchKernelGGL(split_t_kernel, dim3((unsigned)cdiv(Kd, 64), (unsigned)lp), dim3(256), 0, s, B, Kd, l, Bh, Bl,
                     E.ldb);
  // two column groups (128-row workgroups) while a wave's share of the
  // basis fits its registers (l <= 160), else four (64-row workgroups)
  const int lt = (l + 15) / 16;
  const int cg = cdiv(lt, 2) <= 5 ? 2 : 4;
  const int64_t rows_wg = 64 * (4 / cg);
  const int64_t mb = cdiv(M, rows_wg);
  const int64_t splits = std::max<int64_t>(1, std::min<int64_t>(cdiv(256, mb), Kd / 512));
  const int64_t k_chunk = align_up((size_t)cdiv(Kd, splits), 32);
  const int64_t ks = cdiv(Kd, k_chunk);
  const int atomic = ks > 1 ? 1 : 0;
  if (atomic) hipLaunchKernelGGL(fill_f32_kernel, dim3(256), dim3(256), 0, s, C, M * l, 0.0f);
  const dim3 grid((unsigned)mb, (unsigned)ks);
#define SALR_GEMM_R(CT, CG)                                                                                  \
  hipLaunchKernelGGL((gemm_bf16x2_kernel<CT, CG>), grid, dim3(256), 0, s, A, lda, Bh, Bl, E.ldb, C, M, l, Kd, \
                     k_chunk, atomic)
  if (cg == 2) {
    switch (cdiv(lt, 2)) {
      case 1: SALR_GEMM_R(1, 2); break;
      case 2: SALR_GEMM_R(2, 2); break;
      case 3: SALR_GEMM_R(3, 2); break;
      case 4: SALR_GEMM_R(4, 2); break;
      default: SALR_GEMM_R(5, 2); break;
    }
  } else {
    switch (cdiv(lt, 4)) {
      case 3: SALR_GEMM_R(3, 4); break;
      case 4: SALR_GEMM_R(4, 4); break;
      default: SALR_GEMM_R(5, 4); break;
    }
  }
#undef SALR_GEMM_R
  return hipGetLastError();
}

// Split count so that a skinny product (few output tiles) still fills the GPU.
int skinny_split(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = cdiv(M, 64) * cdiv(N, 64);
  int64_t s = std::max<int64_t>(1, 512 / tiles);
  return (int)std::min<int64_t>(s, std::max<int64_t>(1, K / 256));
}

// Y (rows x l, row-major) <- orthonormal basis of its column span; `tmp` has
// the same shape.  Cholesky QR `passes` times (the second pass repairs the
// first one's loss of orthogonality).
hipError_t orth(hipStream_t s, float* Y, float* tmp, int64_t rows, int l, const EncodeLayout& E, void* ws,
                int passes) {
  float* G = at<float>(ws, E.G);
  float* C = at<float>(ws, E.C);
  for (int pass = 0; pass < passes; ++pass) {
    // G = Y^T Y
    hipError_t e = gemm(s, l, l, rows, Y, false, 1, l, Y, l, 1, G, l, 1, skinny_split(l, l, rows));
    if (e != hipSuccess) return e;
    if (l <= kRegChol)
      launch_chol_inv_reg(s, G, C, l, 1e-10);
    else
      hipLaunchKernelGGL(chol_inv_kernel, dim3(1), dim3(kSmallThreads), 0, s, G, C, at<double>(ws, E.dA),
                         at<double>(ws, E.dB), l, 1e-10);
    // tmp = Y C, then copy back
    e = gemm(s, rows, l, l, Y, false, l, 1, C, l, 1, tmp, l, 1);
    if (e != hipSuccess) return e;
    e = hipMemcpyAsync(Y, tmp, (size_t)rows * l * 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace

int32_t svd_basis(int64_t N, int64_t K, int32_t r_svd, int32_t oversample) {
  if (r_svd <= 0) return 0;
  const int64_t cap = std::min<int64_t>(std::min(N, K), 320);
  return (int32_t)std::min<int64_t>((int64_t)r_svd + std::max(oversample, 0), cap);
}

size_t encode_ws_bytes(int64_t N, int64_t K, int32_t r_svd, int32_t oversample) {
  return encode_layout(N, K, r_svd, oversample).total;
}

#define CK(x)                              \
  do {                                     \
    if ((x) != hipSuccess) return SALR_ERR_HIP; \
  } while (0)

namespace {
// The encode steps.  `ev` and `hflags` receive asynchronous device-to-host
// copies; encode_run owns them and synchronizes the stream before any
// return, so no copy can land after they are gone.
int encode_steps(const EncodeParams& p, std::vector<double>& ev, uint32_t (&hflags)[4]) {
  hipStream_t s = p.stream;
  const EncodeLayout E = encode_layout(p.N, p.K, p.r_svd, p.oversample);
  if (p.ws_bytes < E.total) return SALR_ERR_WORKSPACE;
  void* ws = p.ws;
  uint32_t* flags = at<uint32_t>(ws, E.flags);
  uint16_t* R = at<uint16_t>(ws, E.R);
  if (hipMemsetAsync(flags, 0, 64, s) != hipSuccess) return SALR_ERR_HIP;

  // 1. selection, bitmap, values, lookup table, residual
  PrunePackArgs pa{};
  pa.W = p.W;
  pa.masks = p.masks;
  pa.values = p.values;
  pa.offsets = p.offsets;
  pa.R = p.r_svd > 0 ? R : nullptr;
  pa.nonfinite = flags;
  pa.N = p.N;
  pa.K = (int32_t)p.K;
  pa.n_keep = p.n_keep;
  pa.kw = (int32_t)cdiv(p.K, 64);
  pa.ng = (int32_t)cdiv(p.K, 1024);
  if (launch_prune_pack(pa, s) != hipSuccess) return SALR_ERR_HIP;

  // 2. residual truncated SVD
  const int r = p.r_svd;
  const int l = E.l;
  ev.assign(std::max(l, 1), 0.0);
  if (r > 0) {
    const int64_t N = p.N, K = p.K;
    float* Y = at<float>(ws, E.Y);
    float* Q = at<float>(ws, E.Q);
    float* Z = at<float>(ws, E.Z);
    float* Z2 = at<float>(ws, E.Z2);
    uint16_t* Rt = at<uint16_t>(ws, E.Rt);
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)cdiv(K, 64), (unsigned)cdiv(N, 64)), dim3(256), 0, s, R,
                       N, K, Rt);
    hipLaunchKernelGGL(gaussian_kernel, dim3(1024), dim3(256), 0, s, Z, K * l, p.seed);
    // Y = R Z
    CK(gemm_r(s, R, K, N, K, Z, l, Y, E, ws));
    for (int it = 0; it < p.iters; ++it) {
      CK(orth(s, Y, Q, N, l, E, ws, 1));
      // Z = R^T Y
      CK(gemm_r(s, Rt, N, K, N, Y, l, Z, E, ws));
      CK(orth(s, Z, Z2, K, l, E, ws, 1));
      // Y = R Z
      CK(gemm_r(s, R, K, N, K, Z, l, Y, E, ws));
    }
    CK(orth(s, Y, Q, N, l, E, ws, 2));
    // Bt = R^T Q  (K x l), in Z
    CK(gemm_r(s, Rt, N, K, N, Y, l, Z, E, ws));
    // G = Bt^T Bt
    float* G = at<float>(ws, E.G);
    CK(gemm(s, l, l, K, Z, false, 1, l, Z, l, 1, G, l, 1, skinny_split(l, l, K)));
    double* evals = at<double>(ws, E.evals);
    float* U = at<float>(ws, E.U);
    if (l <= kLdsJacobi)
      hipLaunchKernelGGL(jacobi_lds_kernel, dim3(1), dim3(kSmallThreads), (size_t)2 * l * (l + 1) * 8, s, G, evals, U, l,
                         30);
    else if (l <= kMidJacobi)
      hipLaunchKernelGGL(jacobi_mid_kernel, dim3(1), dim3(kSmallThreads), (size_t)4 * l * (l + 1), s, G, evals, U,
                         at<float>(ws, E.dA), l, 30);
    else
      hipLaunchKernelGGL(jacobi_kernel, dim3(1), dim3(kSmallThreads), 0, s, G, at<double>(ws, E.dA),
                         at<double>(ws, E.dB), evals, U, l, 30);
    // P = Bt U_r (K x r) in Z2; S2 = Q U_r (N x r) in Q
    CK(gemm(s, K, r, l, Z, false, l, 1, U, l, 1, Z2, r, 1));
    CK(gemm(s, N, r, l, Y, false, l, 1, U, l, 1, Q, r, 1));
    hipLaunchKernelGGL(write_a_kernel, dim3((unsigned)std::min<int64_t>(cdiv(K, 256), 64), r), dim3(256), 0, s, Z2,
                       evals, p.a_cat, K, r);
    hipLaunchKernelGGL(write_b_kernel, dim3(1024), dim3(256), 0, s, Q, evals, p.b_cat, N, r, p.r_cat);
    if (hipMemcpyAsync(ev.data(), evals, (size_t)l * 8, hipMemcpyDeviceToHost, s) != hipSuccess) return SALR_ERR_HIP;
  }

  // 3. LoRA blocks after the residual block, in call order
  int row0 = r;
  for (int a = 0; a < p.n_lora; ++a) {
    hipLaunchKernelGGL(copy_lora_kernel, dim3(1024), dim3(256), 0, s, p.lora_A[a], p.lora_B[a], p.a_cat, p.b_cat,
                       p.N, p.K, p.lora_r[a], row0, p.r_cat);
    row0 += p.lora_r[a];
  }
  if (hipGetLastError() != hipSuccess) return SALR_ERR_HIP;

  if (hipMemcpyAsync(hflags, flags, sizeof(hflags), hipMemcpyDeviceToHost, s) != hipSuccess) return SALR_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return SALR_ERR_HIP;
  if (hflags[0]) return SALR_ERR_NONFINITE;
  for (int i = 0; i < r; ++i) {
    if (!std::isfinite(ev[i])) return SALR_ERR_NUMERICAL;
    if (p.sigma) p.sigma[i] = ev[i] > 0 ? std::sqrt(ev[i]) : 0.0;
  }
  return SALR_OK;
}
}  // namespace

int encode_run(const EncodeParams& p) {
  std::vector<double> ev;
  uint32_t hflags[4] = {0, 0, 0, 0};
  const int st = encode_steps(p, ev, hflags);
  // (on an error return, copies into ev / hflags may still be queued)
  if (st != SALR_OK) (void)hipStreamSynchronize(p.stream);
  return st;
}

}  // namespace salr
