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
// keep HBM busy and spend as few instructions per weight as possible:
//   * the product is computed transposed, Y^T = W_s X^T, so the 16-row MFMA
//     side holds W rows and the 16-column side holds the (zero-padded) M
//     tokens; decoded weights go straight from LDS into operand registers;
//   * a consumer workgroup (8 waves) owns 16 W rows x a column range of up
//     to 4096 columns.  When the range is the whole row, the workgroup's
//     values are one contiguous block of 16 * n_keep bf16 whose address is
//     known at launch, so every load (values, bitmap, X) is issued at once,
//     values and bitmap straight into LDS (global_load_lds), with no
//     dependent round trip.  Longer rows are cut into ranges located by the
//     per-row lookup table (one extra round trip);
//   * decode of an 8-column operand slice is two nibble expansions (three
//     aligned LDS words, 2 funnel shifts, 2 byte permutes each); a wave's
//     bitmap words
//     sit in registers and its steps' LDS reads are issued in batches so
//     their latencies overlap;
//   * range partials of one row tile are combined by the last workgroup to
//     finish, in range order (results do not depend on scheduling);
//   * T = X A_cat comes from a small preceding launch (lowrank_t_small
//     below, a few K-pieces of fp32 partial sums); the main launch copies
//     those partials and the tile's B_cat rows into LDS together with the
//     weights, so the low-rank term T B_cat is a few LDS reads and extra
//     matrix-core steps at the end;
//   * range partials handed between workgroups travel as tagged words (see
//     salr_device.hpp), so no cache-wide fence is ever executed; with whole
//     rows there is no cross-workgroup traffic at all.
#include "salr_device.hpp"
#include "salr_kernels.hpp"

namespace salr {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = 16;
constexpr int kMaxSteps = kMaxRangeCols / 32 / kWaves;  // 32-column steps per wave
constexpr int kMaxWaveWords = kMaxSteps / 2;           // bitmap words per wave
// Bitmap words per row in LDS: one word of padding puts the 16 rows' words
// in 16 distinct bank pairs.
constexpr int kMaskRowWords = kMaxRangeCols / 64 + 1;
constexpr int kPollBatch = 8;
constexpr int kBatch = 4;  // decode steps whose LDS reads are issued together

// LDS carve-up (dynamic shared memory): a fixed part, then the values area.
struct Lds {
  u32x2_t lut[16];
  uint32_t seg[kRows][2];  // per-row range of kept-value indices (within the row)
  int64_t vorg[kRows];     // global value index = LDS value slot + vorg (per row)
  uint64_t masks[kRows * kMaskRowWords];
};
static_assert(sizeof(Lds) % 16 == 0, "values area must stay 16-byte aligned");

__device__ __forceinline__ u32x4_t load_x_frag(const uint16_t* X, int M, int K, int m, int col) {
  if (m < M && col < K) return load16(X + (size_t)m * K + col);
  return zero_u4();
}

// Sum the waves' accumulators into wave 0 (fixed order).  Other waves return
// false and must leave; wave 0 returns true with the total.
__device__ __forceinline__ bool reduce_waves(f32x4_t& acc, f32x4_t* red, int wave, int lane) {
  __syncthreads();
  if (wave > 0) red[(wave - 1) * 64 + lane] = acc;
  __syncthreads();
  if (wave > 0) return false;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w) acc += red[w * 64 + lane];
  return true;
}

// Publish a partial 16x16 tile (the lane's 4 floats as tagged words) and
// return true in the workgroup elected to reduce (the last to arrive); that
// one waits for every part's words and sums them in part order.  The words of
// up to kPollBatch parts are requested together.
__device__ __forceinline__ bool reduce_parts(f32x4_t& acc, uint64_t* parts, int nparts, int self,
                                             uint32_t* counter, uint32_t tag, uint32_t* err, int lane) {
  uint64_t* mine = parts + ((size_t)self * 64 + lane) * 4;
  // (each element is copied to a scalar first: bit-casting a vector element
  // in place is miscompiled by this toolchain into four copies of element 0)
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float v = acc[e];
    store_tagged(mine + e, __float_as_uint(v), tag);
  }
  uint32_t old = 0;
  if (lane == 0) old = atomic_add_relaxed(counter, 1u);
  old = __shfl(old, 0);
  if (old != (uint32_t)(nparts - 1)) return false;
  if (lane == 0) store_coherent(counter, 0u);
  f32x4_t sum = zero4();
  for (int p0 = 0; p0 < nparts; p0 += kPollBatch) {
    uint64_t v[kPollBatch][4];
#pragma unroll
    for (int b = 0; b < kPollBatch; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[b][e] = (p0 + b < nparts) ? load_tagged_raw(parts + ((size_t)(p0 + b) * 64 + lane) * 4 + e) : 0ull;
#pragma unroll
    for (int b = 0; b < kPollBatch; ++b) {
      if (p0 + b >= nparts) break;
      bool ok = true;
#pragma unroll
      for (int e = 0; e < 4; ++e) ok &= (uint32_t)(v[b][e] >> 32) == tag;
      uint32_t w[4];
      if (ok) {
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (uint32_t)v[b][e];
      } else {
        poll_tagged<4>(parts + ((size_t)(p0 + b) * 64 + lane) * 4, tag, w, err);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sum[e] += __uint_as_float(w[e]);
    }
  }
  acc = sum;
  return true;
}

// Copy n 16-byte chunks from global src (16-byte aligned) to LDS dst as
// whole-wave direct-to-LDS loads (lane l of a block carries chunk 64b + l to
// dst + 16 (64b + l)); this wave takes blocks first, first + stride, ...
__device__ __forceinline__ void copy_chunks_to_lds(const uint32_t* src, uint32_t* dst, int64_t n, int first,
                                                   int stride, int lane) {
  for (int64_t b = first; b * 64 < n; b += stride) {
    const int64_t c = b * 64 + lane;
    if (c < n) __builtin_amdgcn_global_load_lds(src + c * 4, dst + b * 256, 16, 0, 0);
  }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_small_kernel(SmallFwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  Lds& L = *reinterpret_cast<Lds*>(smem);
  uint32_t* const vals = reinterpret_cast<uint32_t*>(smem + sizeof(Lds));
  f32x4_t* const red = reinterpret_cast<f32x4_t*>(vals);
  // after the values area: the T partials [t_pieces][16][r_pad] fp32, then
  // the tile's B_cat rows [16][r_cat] bf16
  float* const tl = reinterpret_cast<float*>(smem + sizeof(Lds) + a.vals_bytes);
  uint16_t* const bl = reinterpret_cast<uint16_t*>(smem + sizeof(Lds) + a.vals_bytes + a.tl_bytes);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const uint32_t n_wgs = gridDim.x;
  const bool talk = a.splits > 1;  // any cross-workgroup data?
  uint32_t* const epoch = &a.sync[0];
  uint32_t* const done = &a.sync[1];
  uint32_t* const err = &a.sync[2];
  const uint32_t ngroups = (uint32_t)a.done_groups;
  const uint32_t tag = load_coherent(epoch) + 1u;
  f32x4_t acc = zero4();

  // ---------------- this workgroup's weights: 16 rows x one column range
  const int c = blockIdx.x;
  const int tile = c / a.splits, rng = c % a.splits;
  const int64_t row0 = (int64_t)tile * kRows;
  const int col0 = rng * a.range;
  const int ncols = min(a.range, a.K - col0);
  const int nsteps = (ncols + 31) / 32;
  // steps per wave, even so that every wave starts on a bitmap word (<= kMaxSteps)
  const int spw = 2 * ((nsteps + 2 * kWaves - 1) / (2 * kWaves));
  const int s0 = wave * spw;
  const int nwords = (ncols + 63) / 64;            // bitmap words in the range
  const int rows_here = (int)min<int64_t>(kRows, a.N - row0);

  // X operand slices of this wave's steps (independent of the weights).
  u32x4_t xf[kMaxSteps];
#pragma unroll
  for (int q = 0; q < kMaxSteps; ++q)
    xf[q] = (q < spw) ? load_x_frag(a.X, a.M, a.K, i, col0 + 32 * (s0 + q) + 8 * g) : zero_u4();

  if (tid < 16) L.lut[tid] = nibble_selectors(tid);
  // Bitmap words of the range, per row 2*nwords dwords direct to LDS; rows
  // past N read as zero.
  for (int r = wave; r < kRows; r += kWaves) {
    uint32_t* dst = reinterpret_cast<uint32_t*>(&L.masks[r * kMaskRowWords]);
    if (r < rows_here) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(a.masks + (row0 + r) * a.kw + (col0 >> 6));
      for (int b = 0; b * 64 < 2 * nwords; ++b)
        if (b * 64 + lane < 2 * nwords) __builtin_amdgcn_global_load_lds(src + b * 64 + lane, dst + b * 64, 4, 0, 0);
    } else {
      for (int w = lane; w < 2 * kMaskRowWords; w += 64) dst[w] = 0u;
    }
  }
  if (a.splits == 1) {
    // Whole rows: row r's values start at (row0 + r) * n_keep, known without
    // reading anything.  Each row gets its own LDS area (vcap chunks, the
    // stride chosen so that row areas start in different LDS banks).
    if (tid < kRows) L.seg[tid][0] = 0;
    for (int r = wave; r < kRows; r += kWaves) {
      const int64_t va = (row0 + r) * a.n_keep, vb = va + a.n_keep;
      const int64_t q0 = va >> 3, nch = (r < rows_here && vb > va) ? ((vb + 7) >> 3) - q0 : 0;
      copy_chunks_to_lds(reinterpret_cast<const uint32_t*>(a.values) + q0 * 4, vals + (size_t)r * a.vcap * 4, nch,
                         0, 1, lane);
      if (lane == 0) L.vorg[r] = q0 * 8 - (int64_t)r * a.vcap * 8;
    }
  } else {
    // A range of a longer row: locate each row's values with the lookup
    // table (one round trip), then copy each row's chunks.
    if (tid < kRows) {
      const int64_t row = row0 + tid;
      uint32_t lo = 0, hi = 0;
      if (tid < rows_here) {
        const int g0 = col0 >> 10, g1 = (col0 + ncols + 1023) >> 10;  // lookup-table entries
        hi = (g1 < a.ng) ? a.offsets[row * a.ng + g1] : (uint32_t)a.n_keep;
        hi = min(hi, (uint32_t)a.n_keep);
        lo = min(a.offsets[row * a.ng + g0], hi);
        lo = max(lo, hi > (uint32_t)a.range ? hi - (uint32_t)a.range : 0u);  // inside the row's LDS area
      }
      L.seg[tid][0] = lo;
      L.seg[tid][1] = hi;
    }
    __syncthreads();
    for (int r = wave; r < kRows; r += kWaves) {
      const int64_t va = (row0 + r) * a.n_keep + L.seg[r][0];
      const int64_t vb = (row0 + r) * a.n_keep + L.seg[r][1];
      const int64_t q0 = va >> 3, nch = (r < rows_here && vb > va) ? ((vb + 7) >> 3) - q0 : 0;
      copy_chunks_to_lds(reinterpret_cast<const uint32_t*>(a.values) + q0 * 4, vals + (size_t)r * a.vcap * 4, nch,
                         0, 1, lane);
      if (lane == 0) L.vorg[r] = q0 * 8 - (int64_t)r * a.vcap * 8;
    }
  }

  // Low-rank operands for the epilogue, fetched with the weights: the T
  // partials of the preceding launch and this tile's B_cat rows.
  if (a.r_cat > 0) {
    copy_chunks_to_lds(reinterpret_cast<const uint32_t*>(a.tsum), reinterpret_cast<uint32_t*>(tl),
                       (int64_t)a.tl_bytes / 16, wave, kWaves, lane);
    const int64_t bbytes = (int64_t)rows_here * a.r_cat * 2;
    copy_chunks_to_lds(reinterpret_cast<const uint32_t*>(a.b_cat + row0 * a.r_cat), reinterpret_cast<uint32_t*>(bl),
                       (bbytes + 15) / 16, (wave + 3) % kWaves, kWaves, lane);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Decode + multiply this wave's steps.  The wave's bitmap words come to
  // registers first; then each batch of kBatch steps issues all its LDS
  // reads (two value windows and two selector words per step) before any of
  // them is used.
  {
    const bool live = i < rows_here;
    const uint64_t* mrow = &L.masks[i * kMaskRowWords];
    const uint16_t* vals16 = reinterpret_cast<const uint16_t*>(vals);
    // LDS slot of the row's first value in the range, plus the kept bits of
    // the range before this wave's first word
    const uint32_t base = live ? (uint32_t)((row0 + i) * a.n_keep + L.seg[i][0] - L.vorg[i]) : 0u;
    const int w0 = s0 >> 1;
    uint32_t part = 0;
    for (int w = g; w < w0; w += 4) part += __popcll(mrow[w]);
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    uint64_t mw[kMaxWaveWords];
#pragma unroll
    for (int q = 0; q < kMaxWaveWords; ++q) mw[q] = (2 * q < spw && w0 + q < nwords) ? mrow[w0 + q] : 0ull;
    uint32_t run = base + part;
    const uint32_t below = (1u << (8 * g)) - 1u;
#pragma unroll
    for (int q0 = 0; q0 < kMaxSteps; q0 += kBatch) {
      if (q0 < spw && s0 + q0 < nsteps) {
        Window3 wa[kBatch], wb[kBatch];
        uint32_t ia[kBatch], ib[kBatch];
        u32x2_t la[kBatch], lb[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const int q = q0 + b;
          const uint32_t h = (q & 1) ? (uint32_t)(mw[q >> 1] >> 32) : (uint32_t)mw[q >> 1];
          const uint32_t byte = (q < spw && s0 + q < nsteps) ? (h >> (8 * g)) & 0xFFu : 0u;
          const uint32_t lo = byte & 15u, hi = byte >> 4;
          ia[b] = run + __popc(h & below);
          ib[b] = ia[b] + __popc(lo);
          wa[b] = lds_window_words(vals16, ia[b]);
          wb[b] = lds_window_words(vals16, ib[b]);
          la[b] = L.lut[lo];
          lb[b] = L.lut[hi];
          run += __popc(h);
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const int q = q0 + b;
          if (q < spw && s0 + q < nsteps) {
            const u32x2_t x0 = expand_nibble(window_values(wa[b], ia[b]), la[b]);
            const u32x2_t x1 = expand_nibble(window_values(wb[b], ib[b]), lb[b]);
            acc = mfma_16x16x32(u32x4_t{x0.x, x0.y, x1.x, x1.y}, xf[q], acc);
          }
        }
      }
    }
  }
  if (!reduce_waves(acc, red, wave, lane)) return;
  if (a.splits > 1) {
    if (!reduce_parts(acc, a.ypart + (size_t)tile * a.splits * 256, a.splits, rng, &a.ycount[tile], tag, err,
                      lane)) {
      if (lane == 0) finish_launch(epoch, done, a.gdone, blockIdx.x, n_wgs, ngroups);
      return;
    }
  }

  // Low-rank term: acc += B_cat^T[rows, :] T^T, as extra K steps.  T is the
  // sum of the partials, rounded to bf16 before it meets B_cat.
  if (a.r_cat > 0) {
    const int tcols = a.r_tiles * 16;
    for (int r0 = 0; r0 < a.r_pad; r0 += 32) {
      const int rb = r0 + 8 * g;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ra = rb + 2 * e;
        const uint32_t lo = (i < rows_here && ra < a.r_cat) ? bl[i * a.r_cat + ra] : 0u;
        const uint32_t hi = (i < rows_here && ra + 1 < a.r_cat) ? bl[i * a.r_cat + ra + 1] : 0u;
        w[e] = lo | (hi << 16);
      }
      u32x4_t tv = zero_u4();
      if (rb < tcols) {
        f32x4_t s0v = zero4(), s1v = zero4();
        for (int p = 0; p < a.t_pieces; ++p) {
          const float* src = tl + ((size_t)p * 16 + i) * a.r_pad + rb;
          s0v += *reinterpret_cast<const f32x4_t*>(src);
          s1v += *reinterpret_cast<const f32x4_t*>(src + 4);
        }
        const float t0 = s0v[0], t1 = s0v[1], t2 = s0v[2], t3 = s0v[3];
        const float t4 = s1v[0], t5 = s1v[1], t6 = s1v[2], t7 = s1v[3];
        tv = u32x4_t{(uint32_t)f32_to_bf16(t0) | ((uint32_t)f32_to_bf16(t1) << 16),
                     (uint32_t)f32_to_bf16(t2) | ((uint32_t)f32_to_bf16(t3) << 16),
                     (uint32_t)f32_to_bf16(t4) | ((uint32_t)f32_to_bf16(t5) << 16),
                     (uint32_t)f32_to_bf16(t6) | ((uint32_t)f32_to_bf16(t7) << 16)};
      }
      acc = mfma_16x16x32(u32x4_t{w[0], w[1], w[2], w[3]}, tv, acc);
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
  if (talk && lane == 0) finish_launch(epoch, done, a.gdone, blockIdx.x, n_wgs, ngroups);
}

// ---------------------------------------------------------------------------
// T pieces for the few-row path: tsum[p][token][rank] = sum over the p-th
// K range of X[token][k] A_cat[rank][k], fp32, for 16 tokens (rows past M
// are zero) and all r_pad ranks (ranks past r_cat are zero).  One workgroup
// per (16-rank tile, K range); its 8 waves split the range and add up in
// LDS.
// ---------------------------------------------------------------------------
constexpr int kTWaves = 8;
constexpr int kTMaxSteps = 8;  // 32-column steps per wave (K range <= 2048)

__global__ __launch_bounds__(kTWaves * 64) void lowrank_t_small_kernel(SmallTArgs a) {
  __shared__ f32x4_t red[(kTWaves - 1) * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int j = blockIdx.x, p = blockIdx.y;
  const int k0 = p * a.k_range, k1 = min(a.K, k0 + a.k_range);
  const int nsteps = (k1 - k0 + 31) / 32;
  const int spw = (nsteps + kTWaves - 1) / kTWaves;
  const int rank = 16 * j + i;
  u32x4_t av[kTMaxSteps], xv[kTMaxSteps];
#pragma unroll
  for (int q = 0; q < kTMaxSteps; ++q) {
    const int st = wave * spw + q;
    const int col = k0 + 32 * st + 8 * g;
    const bool ok = q < spw && st < nsteps && col < k1;
    av[q] = (ok && rank < a.r_cat) ? load16(a.a_cat + (size_t)rank * a.K + col) : zero_u4();
    xv[q] = (ok && i < a.M) ? load16(a.X + (size_t)i * a.K + col) : zero_u4();
  }
  f32x4_t acc = zero4();
#pragma unroll
  for (int q = 0; q < kTMaxSteps; ++q) acc = mfma_16x16x32(av[q], xv[q], acc);
  if (wave > 0) red[(wave - 1) * 64 + lane] = acc;
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < kTWaves - 1; ++w) acc += red[w * 64 + lane];
  // lane holds T^T[rank 16j + 4g + e][token i]
  float* dst = a.tsum + ((size_t)p * 16 + i) * a.r_pad + 16 * j + 4 * g;
  *reinterpret_cast<f32x4_t*>(dst) = acc;
}

}  // namespace

size_t fwd_small_vals_bytes(int vcap) {
  const size_t vals = (size_t)kRows * vcap * 16;
  const size_t red = (size_t)(kWaves - 1) * 64 * 16;
  return ((vals > red ? vals : red) + 15) / 16 * 16;
}

size_t fwd_small_lds_bytes(int vcap, int tl_bytes, int bl_bytes) {
  return sizeof(Lds) + fwd_small_vals_bytes(vcap) + (size_t)tl_bytes + (size_t)bl_bytes;
}

hipError_t launch_fwd_small(const SmallFwdArgs& a, hipStream_t s) {
  const int grid = a.n_tiles * a.splits;
  hipLaunchKernelGGL(fwd_small_kernel, dim3(grid), dim3(kThreads), fwd_small_lds_bytes(a.vcap, a.tl_bytes, a.bl_bytes),
                     s, a);
  return hipGetLastError();
}

hipError_t launch_lowrank_t_small(const SmallTArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(lowrank_t_small_kernel, dim3(a.r_tiles, a.t_pieces), dim3(kTWaves * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace salr
