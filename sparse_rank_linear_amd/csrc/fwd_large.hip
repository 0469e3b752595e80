// SALR forward for many input rows (M > 16): tiled bitmap decode into LDS,
// double-buffered against bf16 matrix-core tiles, with the concatenated
// low-rank product folded in as extra K steps.
//
// Method: gist.science summary of "Sparsity-Aware Low-Rank Representation
// ...", Methodology 4 (two-stage pipeline: stage 1 rebuilds dense sub-blocks
// of W_s from the bitmap and the packed values, stage 2 feeds them to
// matrix-core GEMM tiles, the stages decoupled so decode does not stall the
// multiply) and Methodology 3 (one GEMM for all stacked adapters).
//
// Layout of one workgroup (template WM x WN waves): a BM = 64*WM token by
// BN = 64*WN output tile, K walked in 64-column tiles (one bitmap word per W
// row).  Each wave owns 64 outputs x 64 tokens (4x4 MFMA 16x16 tiles).  The
// product is computed as Y^T = W_s X^T so that a lane's four accumulator
// rows are four consecutive outputs of one token (8-byte stores).
//
// Pipeline per K tile kt (one barrier):
//   X of tile kt+1 straight to LDS (global_load_lds), the packed values of
//   tile kt+2 and the bitmap word of kt+3 into registers;
//   MFMA on tile kt  ||  decode of tile kt+1 (LDS values -> LDS dense W);
//   the values of kt+2 into the buffer freed by tile kt; barrier.
// W rows are streams of packed values: a row's running kept count gives the
// first value of each tile, so no lookup table is needed when K is walked
// from column 0.
#include <algorithm>

#include "salr_device.hpp"
#include "salr_kernels.hpp"

namespace salr {
namespace {

constexpr int kDies = 8;         // XCDs of the GPU, each with its own L2
constexpr int64_t kFillItems = 256;  // work items wanted to occupy the CUs
constexpr int kLdsRow = 36;      // words per 64-column bf16 tile row (+16 B pad)
constexpr int kVRow = 40;        // words per row of staged values (9 chunks + window)

template <int WM, int WN>
struct Cfg {
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int BM = 64 * WM;
  static constexpr int BN = 64 * WN;
  static constexpr int TPR = kThreads / BN;         // decode threads per W row
  static constexpr int CPT = 64 / TPR;              // columns per decode thread
  static constexpr int VCH = (9 + TPR - 1) / TPR;   // value chunks per thread
  static constexpr int XDMA = BM * 8 / kThreads;    // X chunks (direct-to-LDS loads) per thread
};

// A 64-column bf16 tile row is 8 chunks of 16 bytes, stored without padding
// at chunk slot (c ^ (row & 7)): a 16-row MFMA operand read (one chunk per
// row) then hits every bank once per pass, and a whole-wave direct-to-LDS
// load (64 lanes x 16 bytes, contiguous) fills 8 rows by choosing which
// chunk each lane fetches.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

// X tile (rows m0.., columns k0..) straight to LDS: load j of this wave
// covers tile rows 8 (XDMA * wave + j) .. +7.  Rows past M and columns past
// K read clamped (in-bounds) addresses: such rows only reach outputs that
// are never stored, such columns meet zero weights.
template <class C>
__device__ __forceinline__ void dma_x_tile(u32x4_t* xt, const uint16_t* X, int M, int K, int m0, int k0, int wave,
                                           int lane) {
#pragma unroll
  for (int j = 0; j < C::XDMA; ++j) {
    const int blk = C::XDMA * wave + j;  // 8-row block
    const int row = 8 * blk + (lane >> 3);
    const int chunk = (lane & 7) ^ (row & 7);
    const int m = min(m0 + row, M - 1), k = min(k0 + 8 * chunk, K - 8);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(X + (size_t)m * K + k),
                                     reinterpret_cast<uint32_t*>(xt + blk * 64), 16, 0, 0);
  }
}

// The same loads from per-thread byte offsets into X (row clamped, chunk
// column within the tile) formed once, plus the tile's column offset: a few
// instructions per tile instead of a 64-bit multiply per load.  Only for
// tiles wholly inside K (the last tile of a ragged K takes dma_x_tile).
template <class C>
__device__ __forceinline__ void dma_x_tile_fast(u32x4_t* xt, const uint16_t* X, int k0, const uint32_t (&xoff)[C::XDMA],
                                                int wave) {
  const char* const xb = reinterpret_cast<const char*>(X + k0);
#pragma unroll
  for (int j = 0; j < C::XDMA; ++j)
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(xb + xoff[j]),
                                     reinterpret_cast<uint32_t*>(xt + (C::XDMA * wave + j) * 64), 16, 0, 0);
}

template <int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void fwd_large_kernel(LargeFwdArgs a) {
  using C = Cfg<WM, WN>;
  // (each buffer its own array, so the compiler can tell a load in flight
  // into one from reads of the other)
  __shared__ u32x4_t xl0[C::BM * 8], xl1[C::BM * 8];
  __shared__ u32x4_t wl0[C::BN * 8], wl1[C::BN * 8];
  __shared__ uint32_t vl0[C::BN * kVRow], vl1[C::BN * kVRow];
  __shared__ u32x2_t lut[16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int wn = wave % WN, wm = wave / WN;
  // Tile of this workgroup.  Workgroups are dealt to the 8 dies (XCDs) in
  // turn (id % 8); tiles are numbered token-block-major and each die gets a
  // contiguous run of them, so the workgroups on one die share the same X
  // slab (read into that die's L2 once) instead of every die streaming every
  // slab.
  // With K splits, consecutive work items of a die take the same split of
  // neighbouring tiles.
  const int nb = (int)((a.N + C::BN - 1) / C::BN);
  const int total = nb * ((a.M + C::BM - 1) / C::BM);
  const int items = total * a.ksplit;
  const int per_die = (items + kDies - 1) / kDies;
  const int id = (int)blockIdx.x;  // grid: per_die * kDies workgroups
  const int item = (id % kDies) * per_die + id / kDies;
  if (item >= items) return;
  const int tile = item % total, split = item / total;
  const int64_t n0 = (int64_t)(tile % nb) * C::BN;
  const int m0 = (tile / nb) * C::BM;
  const int kt0 = split * a.kt_per;                        // this split's first K tile
  const int nk = min((a.K + 63) / 64, kt0 + a.kt_per);    // one past its last

  if (tid < 16) lut[tid] = nibble_selectors(tid);

  // byte offsets of this thread's X tile loads (see dma_x_tile_fast; used
  // when M * K * 2 < 2^32)
  uint32_t xoff[C::XDMA];
#pragma unroll
  for (int j = 0; j < C::XDMA; ++j) {
    const int row = 8 * (C::XDMA * wave + j) + (lane >> 3);
    const int chunk = (lane & 7) ^ (row & 7);
    xoff[j] = ((uint32_t)min(m0 + row, a.M - 1) * (uint32_t)a.K + 8u * (uint32_t)chunk) * 2u;
  }
  const auto load_x_tile = [&](u32x4_t* xt, int kt) {
    if (a.x_off32 && (kt + 1) * 64 <= a.K) dma_x_tile_fast<C>(xt, a.X, kt * 64, xoff, wave);
    else dma_x_tile<C>(xt, a.X, a.M, a.K, m0, kt * 64, wave, lane);
  };

  // this thread's decode row and column part
  const int drow = tid / C::TPR, dpart = tid % C::TPR;
  const int64_t grow = n0 + drow;
  const bool row_ok = grow < a.N;
  const int64_t row_base = row_ok ? grow * a.n_keep : 0;
  const uint64_t* mrow = a.masks + (row_ok ? grow * a.kw : 0);
  // (the raw word of a clamped, unconditional load; mask_ok() applies the
  // bounds where the word is used, so that it is not waited for at once)
  auto mask_raw = [&](int kt) -> uint64_t { return mrow[min(kt, a.kw - 1)]; };
  auto mask_ok = [&](uint64_t w, int kt) -> uint64_t { return (row_ok && kt < nk) ? w : 0ull; };

  // Stage the packed values of one tile of this row: chunks covering
  // [row_base + run, + popcount(mask)); returns how many.  The loads are
  // unconditional: the first chunk starts at most at the end of the values,
  // and the 9 chunks read from there stay inside the values buffer's
  // 256-byte tail padding.  Their registers are not touched until stored,
  // so the compiler counts them exactly and waits only at the store.
  auto load_v = [&](u32x4_t (&r)[C::VCH], uint32_t run, uint64_t mk) -> int {
    const int64_t va = row_base + run;
    const int cnt = __popcll(mk);
    const int64_t q0 = va >> 3;
    const int64_t q1 = min((va + cnt + 7) >> 3, a.vchunks);
    const uint16_t* const vq = a.values + q0 * 8;
#pragma unroll
    for (int u = 0; u < C::VCH; ++u) r[u] = load16(vq + (dpart + C::TPR * u) * 8);
    return cnt ? (int)(q1 - q0) : 0;
  };
  // (chunks past the row's count hold other values: the decode never
  // selects them, a zero selector byte stands for every pruned column)
  auto store_v = [&](uint32_t* vb, const u32x4_t (&r)[C::VCH], int) {
#pragma unroll
    for (int u = 0; u < C::VCH; ++u) {
      const int ch = dpart + C::TPR * u;
      if (ch < 9) *reinterpret_cast<u32x4_t*>(&vb[drow * kVRow + ch * 4]) = r[u];
    }
  };
  // Decode this thread's columns of one tile into dense bf16 in LDS.
  auto decode = [&](u32x4_t* wt, const uint32_t* vb, uint32_t run, uint64_t mk) {
    const uint32_t lead = (uint32_t)((row_base + run) & 7);
    const uint16_t* rowbuf = reinterpret_cast<const uint16_t*>(&vb[drow * kVRow]);
    const int cbeg = dpart * C::CPT;
    uint32_t idx = lead + (cbeg ? (uint32_t)__popcll(mk & ((1ull << cbeg) - 1ull)) : 0u);
#pragma unroll
    for (int b = 0; b < C::CPT / 8; ++b) {
      const uint32_t byte = (uint32_t)(mk >> (cbeg + 8 * b)) & 0xFFu;
      wt[swz(drow, cbeg / 8 + b)] = expand_byte(rowbuf, idx, byte, lut);
      idx += __popc(byte);
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = zero4();

  auto mfma_tile = [&](const u32x4_t* xt, const u32x4_t* wt) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4_t av[4], bv[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        av[t] = wt[swz(wn * 64 + t * 16 + i, ks * 4 + g)];
        bv[t] = xt[swz(wm * 64 + t * 16 + i, ks * 4 + g)];
      }
#pragma unroll
      for (int tn = 0; tn < 4; ++tn)
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) acc[tn][tm] = mfma_16x16x32(av[tn], bv[tm], acc[tn][tm]);
    }
  };

  // ---- prologue: X tile 0 and the values of tiles 0 and 1 in LDS, tile 0
  // decoded
  // kept values of the row before this split: the lookup table entry at the
  // last 1024-column boundary, plus the bitmap words after it
  uint32_t run0 = 0;
  if (kt0 > 0) {
    // (all loads issued together: fixed count, clamped indices, masked sums)
    const int w0 = kt0 & ~15;
    uint64_t wd[15];
#pragma unroll
    for (int u = 0; u < 15; ++u) wd[u] = mrow[min(w0 + u, a.kw - 1)];
    const uint32_t base = a.offsets[(row_ok ? grow : 0) * a.ng + (kt0 >> 4)];
    uint32_t sum = 0;
#pragma unroll
    for (int u = 0; u < 15; ++u) sum += (w0 + u < kt0) ? (uint32_t)__popcll(wd[u]) : 0u;
    run0 = row_ok ? base + sum : 0u;
  }
  const uint64_t mk0 = mask_ok(mask_raw(kt0), kt0);
  uint64_t mk1 = mask_ok(mask_raw(kt0 + 1), kt0 + 1);
  uint64_t mk2raw = mask_raw(kt0 + 2);
  {
    load_x_tile(xl0, kt0);
    u32x4_t vr[C::VCH];
    int n = load_v(vr, run0, mk0);
    store_v(vl0, vr, n);
    n = load_v(vr, run0 + (uint32_t)__popcll(mk0), mk1);
    store_v(vl1, vr, n);
    __syncthreads();
    decode(wl0, vl0, run0, mk0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  uint32_t run1 = run0 + (uint32_t)__popcll(mk0);  // first value of tile kt+1

  // One K tile, one barrier: X of tile kt+1 goes straight to LDS and the
  // values of tile kt+2 to registers while the matrix cores work on tile kt
  // and the decode builds tile kt+1; the values land in the buffer tile kt's
  // values just left.  (Unrolled by two so that every buffer is named.)
  auto step = [&](int kt, u32x4_t* xc, u32x4_t* xn, u32x4_t* wc, u32x4_t* wn_, uint32_t* vc, uint32_t* vn) {
    if (kt + 1 < nk) load_x_tile(xn, kt + 1);
    const uint64_t mk2 = mask_ok(mk2raw, kt + 2);
    const uint32_t run2 = run1 + (uint32_t)__popcll(mk1);
    u32x4_t vr[C::VCH];
    const int n2 = load_v(vr, run2, mk2);
    const uint64_t mk3raw = mask_raw(kt + 3);

    mfma_tile(xc, wc);
    if (kt + 1 < nk) decode(wn_, vn, run1, mk1);
    store_v(vc, vr, n2);
    __builtin_amdgcn_s_waitcnt(0);  // (this wave's X loads into LDS)
    __syncthreads();
    mk1 = mk2;
    mk2raw = mk3raw;
    run1 = run2;
  };
  for (int kt = kt0; kt < nk; kt += 2) {
    step(kt, xl0, xl1, wl0, wl1, vl0, vl1);
    if (kt + 1 < nk) step(kt + 1, xl1, xl0, wl1, wl0, vl1, vl0);
  }

  // ---- low-rank term as extra K tiles: Y^T += B_cat^T[n, :] T[m, :]^T, where
  // T = X A_cat is the sum of the K-split partials (written by the previous
  // launch), rounded to bf16 before it meets B_cat.
  // (a fused layer: only the ranks of the part that owns rows n0.., B_cat
  // being zero outside them; every part holds whole tiles)
  int rlo = 0, rhi = a.r_cat;
  for (int p = 0; p < a.nparts; ++p)
    if (n0 < a.part_row_end[p]) {
      rlo = a.part_rank0[p];
      rhi = rlo + a.part_nrank[p];
      break;
    }
  if (rhi > rlo && split == 0) {
    const size_t split_stride = (size_t)a.M * a.r_pad;
    for (int r0 = rlo; r0 < rhi; r0 += 64) {
#pragma unroll
      for (int u = 0; u < C::XDMA; ++u) {
        const int c = tid + C::kThreads * u;
        const int row = c >> 3, ch = c & 7;
        const int m = m0 + row, k = r0 + 8 * ch;
        u32x4_t v = zero_u4();
        if (m < a.M && k < a.r_pad) {
          f32x4_t lo = zero4(), hi = zero4();
          const float* src = a.tpart + (size_t)m * a.r_pad + k;
#pragma unroll 4
          for (int sp = 0; sp < a.t_splits; ++sp) {
            lo += *reinterpret_cast<const f32x4_t*>(src + sp * split_stride);
            hi += *reinterpret_cast<const f32x4_t*>(src + sp * split_stride + 4);
          }
          v = u32x4_t{(uint32_t)f32_to_bf16(lo[0]) | ((uint32_t)f32_to_bf16(lo[1]) << 16),
                      (uint32_t)f32_to_bf16(lo[2]) | ((uint32_t)f32_to_bf16(lo[3]) << 16),
                      (uint32_t)f32_to_bf16(hi[0]) | ((uint32_t)f32_to_bf16(hi[1]) << 16),
                      (uint32_t)f32_to_bf16(hi[2]) | ((uint32_t)f32_to_bf16(hi[3]) << 16)};
        }
        xl0[swz(row, ch)] = v;
      }
      const int cbeg = dpart * C::CPT;
#pragma unroll
      for (int c8 = 0; c8 < C::CPT; c8 += 8) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ra = r0 + cbeg + c8 + 2 * e;
          const uint32_t lo = (row_ok && ra < rhi) ? a.b_cat[grow * a.r_cat + ra] : 0u;
          const uint32_t hi = (row_ok && ra + 1 < rhi) ? a.b_cat[grow * a.r_cat + ra + 1] : 0u;
          w[e] = lo | (hi << 16);
        }
        wl0[swz(drow, (cbeg + c8) / 8)] = u32x4_t{w[0], w[1], w[2], w[3]};
      }
      __syncthreads();
      mfma_tile(xl0, wl0);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds Y[m][n .. n+3]
  if (a.ksplit > 1) {
    float* part = a.ypart + (size_t)split * a.M * a.N;
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
      const int64_t n = n0 + wn * 64 + tn * 16 + 4 * g;
#pragma unroll
      for (int tm = 0; tm < 4; ++tm) {
        const int m = m0 + wm * 64 + tm * 16 + i;
        if (m >= a.M) continue;
        float* dst = part + (size_t)m * a.N + n;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = acc[tn][tm][e];  // (scalar copy first: see the few-row kernel)
          if (n + e < a.N) dst[e] = v;
        }
      }
    }
    return;
  }
#pragma unroll
  for (int tn = 0; tn < 4; ++tn) {
    const int64_t n = n0 + wn * 64 + tn * 16 + 4 * g;
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
      const int m = m0 + wm * 64 + tm * 16 + i;
      if (m >= a.M) continue;
      uint16_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = f32_to_bf16(acc[tn][tm][e]);
      uint16_t* dst = a.Y + (size_t)m * a.N + n;
      if ((a.N & 3) == 0 && n + 3 < a.N) {
        *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{(uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                                   (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < a.N) dst[e] = h[e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Partial T = X * A_cat over one K range per workgroup, fp32, written to
// tpart[split][M][r_pad] (columns >= r_cat are zero).  A workgroup owns 64
// tokens (one 16-token MFMA tile per wave); the A_cat slice of each
// 64-column tile is shared through LDS.  The splits are summed by the
// consumer (the next launch), so no workgroup waits for another.
// ---------------------------------------------------------------------------
constexpr int kTThreads = 256;
constexpr int kMaxRTiles = 16;   // r_pad <= 256

__global__ __launch_bounds__(kTThreads) void lowrank_t_kernel(LowRankTArgs a) {
  __shared__ uint32_t al[kMaxRTiles * 16 * kLdsRow];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int mb = blockIdx.x, ks = blockIdx.y;
  const int token = mb * 64 + wave * 16 + i;
  const int rt = a.r_pad / 16;
  const int k0 = ks * a.k_chunk, k1 = min(a.K, k0 + a.k_chunk);

  f32x4_t acc[kMaxRTiles];
#pragma unroll
  for (int j = 0; j < kMaxRTiles; ++j) acc[j] = zero4();

  for (int kt = k0; kt < k1; kt += 64) {
    // stage A_cat[0..r_pad)[kt .. kt+64)
    for (int c = tid; c < a.r_pad * 8; c += kTThreads) {
      const int r = c >> 3, k = kt + 8 * (c & 7);
      const u32x4_t v = (r < a.r_cat && k < k1) ? load16(a.a_cat + (size_t)r * a.K + k) : zero_u4();
      *reinterpret_cast<u32x4_t*>(&al[r * kLdsRow + (c & 7) * 4]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int k = kt + 32 * s + 8 * g;
      const u32x4_t xv = (token < a.M && k < k1) ? load16(a.X + (size_t)token * a.K + k) : zero_u4();
#pragma unroll
      for (int j = 0; j < kMaxRTiles; ++j)
        if (j < rt) {
          const u32x4_t av = *reinterpret_cast<const u32x4_t*>(&al[(16 * j + i) * kLdsRow + s * 16 + g * 4]);
          acc[j] = mfma_16x16x32(av, xv, acc[j]);
        }
    }
    __syncthreads();
  }

  // lane holds T[token][16j + 4g + e]
  if (token < a.M) {
    float* dst = a.tpart + ((size_t)ks * a.M + token) * a.r_pad;
#pragma unroll
    for (int j = 0; j < kMaxRTiles; ++j)
      if (j < rt) *reinterpret_cast<f32x4_t*>(&dst[16 * j + 4 * g]) = acc[j];
  }
}

}  // namespace

hipError_t launch_lowrank_t(const LowRankTArgs& a, hipStream_t s) {
  dim3 grid((a.M + 63) / 64, a.splits);
  hipLaunchKernelGGL(lowrank_t_kernel, grid, dim3(kTThreads), 0, s, a);
  return hipGetLastError();
}

int64_t fwd_large_tiles(int64_t N, int64_t M) {
  using C = Cfg<4, 2>;
  return ((N + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM);
}

int fwd_large_ksplit(int64_t N, int64_t K, int64_t M) {
  // enough work items for every CU, each split at least 8 K tiles, at most 8
  const int64_t tiles = fwd_large_tiles(N, M), nk = (K + 63) / 64;
  int64_t s = std::min<int64_t>({kFillItems / std::max<int64_t>(tiles, 1), nk / 8, 8});
  return (int)std::max<int64_t>(s, 1);
}

size_t fwd_large_part_bytes(int64_t N, int64_t K, int64_t M_max) {
  // ksplit * tiles <= kFillItems, so the partials never exceed kFillItems
  // whole tiles; nothing when no M <= M_max splits
  using C = Cfg<4, 2>;
  size_t most = 0;
  for (int64_t M = C::BM; M - C::BM < M_max; M += C::BM) {
    const int s = fwd_large_ksplit(N, K, std::min<int64_t>(M, M_max));
    if (s > 1) most = std::max(most, (size_t)s * std::min<int64_t>(M, M_max) * N * 4);
    if (fwd_large_tiles(N, M) >= kFillItems) break;
  }
  return most;
}

namespace {
// Y = bf16(sum of the K-split partials, in split order): 8 outputs a thread
// (16-byte loads and store when MN is a multiple of 8, as it is whenever N is).
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* part, uint16_t* Y, int64_t MN, int ksplit) {
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (e0 >= MN) return;
  if ((MN & 7) == 0) {
    f32x4_t lo = zero4(), hi = zero4();
    for (int s = 0; s < ksplit; ++s) {
      const float* src = part + (size_t)s * MN + e0;
      lo += *reinterpret_cast<const f32x4_t*>(src);
      hi += *reinterpret_cast<const f32x4_t*>(src + 4);
    }
    *reinterpret_cast<u32x4_t*>(Y + e0) =
        u32x4_t{(uint32_t)f32_to_bf16(lo[0]) | ((uint32_t)f32_to_bf16(lo[1]) << 16),
                (uint32_t)f32_to_bf16(lo[2]) | ((uint32_t)f32_to_bf16(lo[3]) << 16),
                (uint32_t)f32_to_bf16(hi[0]) | ((uint32_t)f32_to_bf16(hi[1]) << 16),
                (uint32_t)f32_to_bf16(hi[2]) | ((uint32_t)f32_to_bf16(hi[3]) << 16)};
    return;
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int n = (int)min<int64_t>(8, MN - e0);
  for (int s = 0; s < ksplit; ++s) {
    const float* src = part + (size_t)s * MN + e0;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e < n) acc[e] += src[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (e < n) Y[e0 + e] = f32_to_bf16(acc[e]);
}
}  // namespace

hipError_t launch_fwd_large(const LargeFwdArgs& a, hipStream_t s) {
  // 256 tokens x 128 outputs per workgroup, 8 waves.
  using C = Cfg<4, 2>;
  // (ceil(work items / 8) workgroups per die: see the tile mapping)
  const int64_t items = fwd_large_tiles(a.N, a.M) * a.ksplit;
  const dim3 grid((unsigned)((items + kDies - 1) / kDies * kDies));
  hipLaunchKernelGGL((fwd_large_kernel<4, 2>), grid, dim3(C::kThreads), 0, s, a);
  if (a.ksplit > 1) {
    const int64_t mn = a.N * (int64_t)a.M;
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((mn + 2047) / 2048)), dim3(256), 0, s, a.ypart, a.Y, mn,
                       a.ksplit);
  }
  return hipGetLastError();
}

}  // namespace salr
