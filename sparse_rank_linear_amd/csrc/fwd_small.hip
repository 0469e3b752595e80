// SALR forward for few input rows (M <= 16): memory-bound bitmap decode on
// the matrix cores, fused with the concatenated low-rank product.
//
// Method: gist.science summary of "Sparsity-Aware Low-Rank Representation
// ...", Methodology 4 (stage 1 rebuilds dense blocks from bitmap + packed
// values, stage 2 multiplies them on matrix units) and Methodology 3 (all
// adapters run as one product on the shared input).
//
// With M <= 16 the layer streams ~1.1 bytes per weight and does at most 32
// flops per byte, far below the matrix-core ridge, so the design goal is to
// keep HBM busy and spend as few vector instructions per weight as possible:
//   * the product is computed transposed, Y^T = W_s X^T, so the 16-row MFMA
//     side holds W rows and the 16-column side holds the (zero-padded) M
//     tokens; decoded weights never leave registers;
//   * each consumer workgroup owns 16 rows x one 1024-column block (the
//     granularity of the per-row lookup table, which gives the block's first
//     value index without scanning the bitmap); it stages the block's
//     packed values with 16-byte loads into LDS and its four waves each
//     decode and multiply a quarter of the block;
//   * decode of an 8-column operand slice is two nibble expansions (3 LDS
//     words, 2 funnel shifts, 2 byte permutes each);
//   * K-split partial tiles are combined by the last workgroup of each row
//     tile, in split order, so results do not depend on scheduling;
//   * producer workgroups (lowest IDs, hence dispatched first) compute
//     T = X A_cat and publish it; the finishing workgroup of each row tile
//     waits for T, then adds T B_cat as extra matrix-core steps.
#include "salr_device.hpp"
#include "salr_kernels.hpp"

namespace salr {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 16;
constexpr int kBlock = 1024;              // columns per consumer workgroup
constexpr int kWordsPerBlock = kBlock / 64;
constexpr int kStepsPerWave = kBlock / 32 / 4;
// Staged values per row: at most 1024 values starting anywhere inside a
// 16-byte chunk -> 129 chunks (516 words); the decode window may read two
// words past the last value.
constexpr int kRowBufWords = 520;
constexpr int kChunksPerLane = 3;         // ceil(129 / 64)
constexpr uint32_t kSpinLimit = 1u << 20;

__device__ __forceinline__ u32x4_t load_x_frag(const uint16_t* X, int M, int K, int m, int col) {
  if (m < M && col < K) return load16(X + (size_t)m * K + col);
  return zero_u4();
}

// Sum the four waves' accumulators into wave 0 (fixed order).  Waves 1-3
// return false and must exit; wave 0 returns true with the total in acc.
__device__ __forceinline__ bool reduce_waves(f32x4_t& acc, f32x4_t* red, int wave, int lane) {
  __syncthreads();
  if (wave > 0) red[(wave - 1) * 64 + lane] = acc;
  __syncthreads();
  if (wave > 0) return false;
  acc += red[lane];
  acc += red[64 + lane];
  acc += red[128 + lane];
  return true;
}

// Publish a partial 16x16 tile and return true in the workgroup that arrives
// last; that one gets the sum over all parts in index order.
__device__ __forceinline__ bool last_arrival_sum(f32x4_t& acc, f32x4_t* parts, int nparts, int self,
                                                 uint32_t* counter, int lane) {
  parts[self * 64 + lane] = acc;
  __threadfence();
  uint32_t old = 0;
  if (lane == 0) old = atomic_add_acq_rel(counter, 1u);
  old = __shfl(old, 0);
  if (old != (uint32_t)(nparts - 1)) return false;
  __threadfence();
  f32x4_t sum = zero4();
  for (int p = 0; p < nparts; ++p) sum += parts[p * 64 + lane];
  acc = sum;
  if (lane == 0) atomic_store_release(counter, 0u);
  return true;
}

__global__ __launch_bounds__(kThreads) void fwd_small_kernel(SmallFwdArgs a) {
  __shared__ uint32_t vbuf[kRows * kRowBufWords];
  __shared__ uint64_t mbuf[kRows * kWordsPerBlock];
  __shared__ u32x2_t lut[16];
  __shared__ uint32_t seg[kRows][2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int n_producers = a.r_tiles * a.t_splits;
  f32x4_t acc = zero4();
  f32x4_t* red = reinterpret_cast<f32x4_t*>(vbuf);

  if ((int)blockIdx.x < n_producers) {
    // ---------------- producer: Tpart = A_cat[16 ranks] x X^T over a K range
    const int j = blockIdx.x / a.t_splits, ts = blockIdx.x % a.t_splits;
    const int k0 = ts * a.t_chunk;
    const int k1 = min(a.K, k0 + a.t_chunk);
    const int steps = (k1 - k0 + 31) / 32;
    const int per_wave = (steps + 3) / 4;
    const int s0 = wave * per_wave, s1 = min(steps, s0 + per_wave);
    const int rank = 16 * j + i;
    for (int st = s0; st < s1; ++st) {
      const int col = k0 + 32 * st + 8 * g;
      u32x4_t av = (rank < a.r_cat && col < a.K) ? load16(a.a_cat + (size_t)rank * a.K + col) : zero_u4();
      u32x4_t xv = load_x_frag(a.X, a.M, a.K, i, col);
      acc = mfma_16x16x32(av, xv, acc);
    }
    if (!reduce_waves(acc, red, wave, lane)) return;
    if (a.t_splits > 1) {
      f32x4_t* parts = reinterpret_cast<f32x4_t*>(a.tpart) + (size_t)j * a.t_splits * 64;
      if (!last_arrival_sum(acc, parts, a.t_splits, ts, &a.tcount[j], lane)) return;
    }
    // lane holds T^T[rank 16j+4g+e][token i]
#pragma unroll
    for (int e = 0; e < 4; ++e) a.tbuf[i * a.r_pad + 16 * j + 4 * g + e] = f32_to_bf16(acc[e]);
    __threadfence();
    if (lane == 0) atomic_add_acq_rel(&a.sync[0], 1u);
    return;
  }

  // ---------------- consumer: 16 rows x one 1024-column block
  const int c = blockIdx.x - n_producers;
  const int tile = c / a.splits, blk = c % a.splits;
  const int64_t row0 = (int64_t)tile * kRows;
  const int col0 = blk * kBlock;
  const int ncols = min(kBlock, a.K - col0);
  const int steps = (ncols + 31) / 32;

  // X operand slices for this wave's quarter of the block (independent of
  // the weights, issued first).
  const int s0 = wave * kStepsPerWave;
  u32x4_t xf[kStepsPerWave];
#pragma unroll
  for (int q = 0; q < kStepsPerWave; ++q) xf[q] = load_x_frag(a.X, a.M, a.K, i, col0 + 32 * (s0 + q) + 8 * g);

  if (tid < 16) lut[tid] = nibble_selectors(tid);
  if (tid < kRows) {
    const int64_t row = row0 + tid;
    uint32_t lo = 0, hi = 0;
    if (row < a.N) {
      // clamped so that even an inconsistent table stays inside the row
      hi = (blk + 1 < a.ng) ? a.offsets[row * a.ng + blk + 1] : (uint32_t)a.n_keep;
      hi = min(hi, (uint32_t)a.n_keep);
      lo = min(a.offsets[row * a.ng + blk], hi);
      lo = max(lo, hi > kBlock ? hi - kBlock : 0u);
    }
    seg[tid][0] = lo;
    seg[tid][1] = hi;
  }
  {
    const int r = tid >> 4, wi = tid & 15;
    const int64_t row = row0 + r;
    uint64_t m = 0;
    if (row < a.N && wi * 64 < ncols) m = a.masks[row * a.kw + (col0 >> 6) + wi];
    mbuf[r * kWordsPerBlock + wi] = m;
  }
  __syncthreads();

  // Stage packed values: wave w copies rows 4w..4w+3, each as the 16-byte
  // chunks that cover its value segment.  All loads are issued before any
  // LDS store.
  u32x4_t vv[4][kChunksPerLane];
  int64_t q0s[4];
  int nch[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = wave * 4 + rr;
    const int64_t row = row0 + r;
    int64_t q0 = 0;
    int n = 0;
    if (row < a.N) {
      const int64_t va = row * a.n_keep + seg[r][0];
      const int64_t vb = row * a.n_keep + seg[r][1];
      if (vb > va) {
        q0 = va >> 3;
        n = (int)(((vb + 7) >> 3) - q0);
      }
    }
    q0s[rr] = q0;
    nch[rr] = n;
#pragma unroll
    for (int t = 0; t < kChunksPerLane; ++t) {
      const int ch = lane + 64 * t;
      vv[rr][t] = (ch < n) ? load16(a.values + (q0 + ch) * 8) : zero_u4();
    }
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = wave * 4 + rr;
#pragma unroll
    for (int t = 0; t < kChunksPerLane; ++t) {
      const int ch = lane + 64 * t;
      if (ch < nch[rr]) *reinterpret_cast<u32x4_t*>(&vbuf[r * kRowBufWords + ch * 4]) = vv[rr][t];
    }
  }
  __syncthreads();

  // Decode + multiply this wave's steps.
  {
    const int64_t row = row0 + i;
    const uint32_t lead = (row < a.N) ? (uint32_t)((row * a.n_keep + seg[i][0]) & 7) : 0u;
    uint32_t run = 0;
    // kept values of this row in the block before the wave's first step
    // (two steps per 64-bit word)
    for (int wi = 0; wi < s0 / 2; ++wi) run += __popcll(mbuf[i * kWordsPerBlock + wi]);
    const uint32_t* rowbuf = &vbuf[i * kRowBufWords];
    const uint32_t below = (1u << (8 * g)) - 1u;
#pragma unroll
    for (int q = 0; q < kStepsPerWave; ++q) {
      const int st = s0 + q;
      if (st < steps) {
        const uint64_t mw = mbuf[i * kWordsPerBlock + (st >> 1)];
        const uint32_t h = (st & 1) ? (uint32_t)(mw >> 32) : (uint32_t)mw;
        const uint32_t byte = (h >> (8 * g)) & 0xFFu;
        const uint32_t idx = lead + run + __popc(h & below);
        const u32x4_t wf = expand_byte(rowbuf, idx, byte, lut);
        run += __popc(h);
        acc = mfma_16x16x32(wf, xf[q], acc);
      }
    }
  }
  if (!reduce_waves(acc, red, wave, lane)) return;
  if (a.splits > 1) {
    f32x4_t* parts = reinterpret_cast<f32x4_t*>(a.ypart) + (size_t)tile * a.splits * 64;
    if (!last_arrival_sum(acc, parts, a.splits, blk, &a.ycount[tile], lane)) return;
  }

  // Low-rank term: acc += B_cat^T[rows, :] T^T, as extra K steps.
  if (a.r_tiles > 0) {
    uint32_t spins = 0;
    while (atomic_load_acquire(&a.sync[0]) < (uint32_t)a.r_tiles) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins >= kSpinLimit) {
        if (lane == 0) atomic_store_release(&a.sync[2], 1u);
        break;
      }
    }
    const int64_t row = row0 + i;
    const int tcols = a.r_tiles * 16;
    for (int r0 = 0; r0 < a.r_pad; r0 += 32) {
      const int rb = r0 + 8 * g;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ra = rb + 2 * e;
        const uint32_t lo = (row < a.N && ra < a.r_cat) ? a.b_cat[row * a.r_cat + ra] : 0u;
        const uint32_t hi = (row < a.N && ra + 1 < a.r_cat) ? a.b_cat[row * a.r_cat + ra + 1] : 0u;
        w[e] = lo | (hi << 16);
      }
      const u32x4_t bv = u32x4_t{w[0], w[1], w[2], w[3]};
      const u32x4_t tv = (rb < tcols) ? load16(a.tbuf + i * a.r_pad + rb) : zero_u4();
      acc = mfma_16x16x32(bv, tv, acc);
    }
  }

  // lane holds Y^T[row0 + 4g + e][token i]
  if (i < a.M) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t n = row0 + 4 * g + e;
      if (n < a.N) a.Y[(size_t)i * a.N + n] = f32_to_bf16(acc[e]);
    }
  }
  if (a.r_tiles > 0 && lane == 0) {
    const uint32_t d = atomic_add_acq_rel(&a.sync[1], 1u);
    if (d == (uint32_t)(a.n_tiles - 1)) {
      atomic_store_release(&a.sync[0], 0u);
      atomic_store_release(&a.sync[1], 0u);
    }
  }
}

}  // namespace

hipError_t launch_fwd_small(const SmallFwdArgs& a, hipStream_t s) {
  const int grid = a.r_tiles * a.t_splits + a.n_tiles * a.splits;
  hipLaunchKernelGGL(fwd_small_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace salr
