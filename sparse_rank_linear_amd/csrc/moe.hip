// Grouped (mixture-of-experts) SALR linear: E experts of one shape, each its
// own encoding, applied in one pair of launches to token rows grouped by
// expert (gist.science summary of "Sparsity-Aware Low-Rank Representation
// ...", Experimental Results: SALR on the mixture-of-experts models
// Mixtral-8x7B and DeepSeek-V2-Lite; Methodology 1-4 for the layer itself).
//
// Rows [off[e], off[e+1]) of X go to expert e; off is read on the device, so
// routing needs no host round trip, and an expert with no rows costs one
// early exit per workgroup and none of its weight bytes.
//
//   1. moe_lowrank_kernel: partials of T = X_e A_cat,e for every expert's
//      rows over K ranges (many workgroups per expert, each with all of a
//      step's loads in flight), then moe_tsum_kernel: their sum in range
//      order rounded to bf16 [T][r_pad] (the same rounding as the
//      single-layer forward).
//   2. moe_fwd_kernel: one workgroup per (16-row tile, expert).  It streams
//      the tile's compressed rows in 1024-column chunks (bitmap words to
//      LDS, each row's kept-value segment -- located by the lookup table --
//      to an LDS row buffer), the four waves decode 32-column MFMA operands
//      from LDS (nibble selectors) and multiply them by up to 64 of the
//      expert's tokens read straight from X, the waves' partial sums meet in
//      LDS, the low-rank product T B_cat,e^T joins as extra K steps, and Y is
//      rounded to bf16.  More than 64 rows for one expert: the tile is
//      streamed again per 64 rows (the decode regime has a few rows per
//      expert).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "salr_device.hpp"
#include "salr_kernels.hpp"

namespace salr {
namespace {

constexpr int kMoeThreads = 256;
constexpr int kMoeRows = 16;        // W rows per workgroup
constexpr int kMoeChunk = 1024;     // columns per streamed chunk (one lookup entry)
constexpr int kMoeWords = kMoeChunk / 64;
constexpr int kMoeTok = 64;         // tokens per pass (4 MFMA column blocks)
constexpr int kMoeRowStride = 1048; // bf16 per LDS row buffer: 7 lead + 1024 + window overrun
constexpr int kMoePieces = (kMoeChunk + 7 + 7) / 8;  // 16-byte pieces per row segment, at most
constexpr int kMoeMaxRT = 16;       // rank tiles of 16 (r_cat <= 256)
constexpr int kMoeTK = 128;         // A_cat columns per low-rank step
constexpr int64_t kMoeTPartCap = int64_t(32) << 20;  // bytes of fp32 T partials (more K splits while under it)
constexpr int kMoeTLds = kMoeTK + 8;  // bf16 per LDS row of the A_cat stage

// Expert e's token rows [s, t), clamped into [0, T] so that malformed
// boundaries can never send a workgroup out of X or Y.
__device__ __forceinline__ void expert_rows(const int32_t* eoff, int e, int32_t T, int32_t& s, int32_t& t) {
  s = min(max(eoff[e], 0), T);
  t = min(max(eoff[e + 1], s), T);
}

// 1a. Partial T of one expert over one K range: workgroup (e, ks, cb)
// takes the columns [ks kspan, + kspan) in steps of kMoeTK (all of a step's
// A_cat loads issued at once) and the expert's 64-row blocks cb, cb + CB,
// ...; fp32 partials tpart[ks][token][r_pad].
__global__ __launch_bounds__(kMoeThreads) void moe_lowrank_kernel(MoeArgs a) {
  __shared__ uint16_t al[kMoeMaxRT * 16 * kMoeTLds];
  const int e = blockIdx.x, ks = blockIdx.y;
  int32_t s, t;
  expert_rows(a.eoff, e, a.T, s, t);
  if (s >= t) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int rt = a.r_pad / 16;
  const int k0 = ks * a.kspan, k1 = min(a.K, k0 + a.kspan);
  const uint16_t* A = a.a_cat + (size_t)e * a.astride;
  constexpr int kPer = kMoeMaxRT * 16 * (kMoeTK / 8) / kMoeThreads;  // 16-byte chunks per thread, at most
  for (int32_t base = s + kMoeTok * (int32_t)blockIdx.z; base < t; base += kMoeTok * (int32_t)gridDim.z) {
    const int32_t token = base + wave * 16 + i;
    const bool live = token < t;
    f32x4_t acc[kMoeMaxRT];
#pragma unroll
    for (int j = 0; j < kMoeMaxRT; ++j) acc[j] = zero4();
    for (int kt = k0; kt < k1; kt += kMoeTK) {
      u32x4_t av[kPer], xv[kMoeTK / 32];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int c = tid + kMoeThreads * u;
        const int r = c / (kMoeTK / 8), k = kt + 8 * (c % (kMoeTK / 8));
        av[u] = (r < a.r_cat && k < k1) ? load16(A + (size_t)r * a.K + k) : zero_u4();
      }
#pragma unroll
      for (int h = 0; h < kMoeTK / 32; ++h) {
        const int k = kt + 32 * h + 8 * g;
        xv[h] = (live && k < k1) ? load16(a.X + (size_t)token * a.K + k) : zero_u4();
      }
      __syncthreads();  // (the previous step's reads of al are done)
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int c = tid + kMoeThreads * u;
        const int r = c / (kMoeTK / 8);
        if (r < a.r_pad) *reinterpret_cast<u32x4_t*>(&al[r * kMoeTLds + 8 * (c % (kMoeTK / 8))]) = av[u];
      }
      __syncthreads();
#pragma unroll
      for (int h = 0; h < kMoeTK / 32; ++h)
#pragma unroll
        for (int j = 0; j < kMoeMaxRT; ++j)
          if (j < rt) {
            const u32x4_t w = *reinterpret_cast<const u32x4_t*>(&al[(16 * j + i) * kMoeTLds + 32 * h + 8 * g]);
            acc[j] = mfma_16x16x32(w, xv[h], acc[j]);
          }
    }
    // lane holds T[token i][rank 16j + 4g + e'] (e' = 0..3)
    if (live) {
      float* dst = a.tpart + ((size_t)ks * a.T + token) * a.r_pad;
#pragma unroll
      for (int j = 0; j < kMoeMaxRT; ++j)
        if (j < rt) *reinterpret_cast<f32x4_t*>(dst + 16 * j + 4 * g) = acc[j];
    }
  }
}

// 1b. T = bf16(sum of the K-range partials, in range order): 4 entries a
// thread (rows of tokens outside every expert's range are never read).
__global__ __launch_bounds__(256) void moe_tsum_kernel(const float* tpart, int splits, int64_t n, uint16_t* t16) {
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e0 >= n) return;
  f32x4_t v = zero4();
  for (int sp = 0; sp < splits; ++sp) v += *reinterpret_cast<const f32x4_t*>(tpart + (size_t)sp * n + e0);
  *reinterpret_cast<u32x2_t*>(t16 + e0) = u32x2_t{(uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                                                  (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16)};
}

struct MoeLds {
  uint16_t vals[kMoeRows][kMoeRowStride];  // each row's value segment (from an 8-aligned start)
  uint64_t masks[kMoeRows][kMoeWords];
  uint32_t wpre[kMoeRows][kMoeWords];      // kept values of the row's chunk before each word (+ lead)
  u32x2_t lut[16];
};
static_assert(sizeof(MoeLds) <= 48 * 1024, "MoE workgroup LDS");
static_assert(kMoeRows * kMoeTok * 4 * 4 <= sizeof(uint16_t) * kMoeRows * kMoeRowStride, "partial sums fit");

// 2. Y rows of one expert for one 16-row tile.
__global__ __launch_bounds__(kMoeThreads) __attribute__((amdgpu_waves_per_eu(3))) void moe_fwd_kernel(MoeArgs a) {
  __shared__ MoeLds L;
  const int e = blockIdx.y;
  int32_t s, t;
  expert_rows(a.eoff, e, a.T, s, t);
  if (s >= t) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kMoeRows;
  const uint64_t* masks = a.masks + (size_t)e * a.mstride;
  const uint16_t* values = a.values + (size_t)e * a.vstride;
  const uint32_t* offs = a.offsets + (size_t)e * a.ostride;
  const uint16_t* bcat = a.b_cat + (size_t)e * a.bstride;
  if (tid < 16) L.lut[tid] = nibble_selectors(tid);

  // staging roles: thread (row sr, lane sl of 16)
  const int sr = tid >> 4, sl = tid & 15;
  const int64_t srow = n0 + sr;
  const bool srow_ok = srow < a.N;
  const int nchunks = (a.K + kMoeChunk - 1) / kMoeChunk;

  // a chunk's bitmap word and value range [lo, hi) (requested one chunk
  // ahead, so a chunk's value loads wait for no lookup-table round trip)
  const auto load_meta = [&](int ch, uint64_t& mw, uint32_t& lo, uint32_t& hi) __attribute__((always_inline)) {
    const int w = ch * kMoeWords + sl;
    mw = (srow_ok && ch < nchunks && w < a.kw) ? masks[srow * a.kw + w] : 0ull;
    lo = hi = 0u;
    if (srow_ok && ch < nchunks) {
      lo = offs[srow * a.ng + ch];
      hi = ch + 1 < a.ng ? offs[srow * a.ng + ch + 1] : (uint32_t)a.n_keep;
    }
  };

  for (int32_t base = s; base < t; base += kMoeTok) {
    const int nq = min(kMoeTok, t - base + 15) / 16;  // live 16-token blocks (1..4)
    f32x4_t acc[4] = {zero4(), zero4(), zero4(), zero4()};
    uint64_t mw_next;
    uint32_t lo_next, hi_next;
    load_meta(0, mw_next, lo_next, hi_next);
    for (int ch = 0; ch < nchunks; ++ch) {
      // ---- stage chunk ch: masks, per-word prefix counts, value segments
      const uint64_t mw = mw_next;
      const uint32_t lo = lo_next, hi = hi_next;
      const int64_t vfirst = srow * (int64_t)a.n_keep + lo;  // global index of the segment's first value
      const int64_t vstart = vfirst & ~int64_t(7);
      const int lead = (int)(vfirst - vstart);
      const int pieces = srow_ok && hi > lo ? (int)((vfirst + (hi - lo) - vstart + 7) >> 3) : 0;
      u32x4_t pv[(kMoePieces + 15) / 16];
#pragma unroll
      for (int u = 0; u < (kMoePieces + 15) / 16; ++u) {
        const int p = sl + 16 * u;
        pv[u] = p < pieces ? load16(values + vstart + 8 * p) : zero_u4();
      }
      load_meta(ch + 1, mw_next, lo_next, hi_next);
      // exclusive prefix of the row's word popcounts across its 16 lanes
      const uint32_t pc = (uint32_t)__popcll(mw);
      uint32_t incl = pc;
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) {
        const uint32_t o = (uint32_t)__shfl_up((int)incl, d, 16);
        if (sl >= d) incl += o;
      }
      __syncthreads();  // (the previous chunk's decode is done with the buffers)
      L.masks[sr][sl] = mw;
      L.wpre[sr][sl] = incl - pc + (uint32_t)lead;
#pragma unroll
      for (int u = 0; u < (kMoePieces + 15) / 16; ++u) {
        const int p = sl + 16 * u;
        if (p < pieces) *reinterpret_cast<u32x4_t*>(&L.vals[sr][8 * p]) = pv[u];
      }
      __syncthreads();
      // ---- decode and multiply: wave takes 32-column steps wave, wave + 4, ...
      const int cbase = ch * kMoeChunk;
      if (nq == 1) {
        // (one token block, the decode regime: X of all the wave's steps
        // requested at once, so the steps wait for one L2 round trip)
        u32x4_t xf[kMoeChunk / 32 / 4];
#pragma unroll
        for (int k = 0; k < kMoeChunk / 32 / 4; ++k) {
          const int col = cbase + 32 * (wave + 4 * k) + 8 * g;
          const int32_t tok = base + i;
          xf[k] = (tok < t && col < a.K) ? load16(a.X + (size_t)tok * a.K + col) : zero_u4();
        }
#pragma unroll
        for (int k = 0; k < kMoeChunk / 32 / 4; ++k) {
          const int ks = wave + 4 * k;
          if (cbase + 32 * ks >= a.K) break;
          const uint64_t mk = L.masks[i][ks >> 1];
          const int bit = 32 * (ks & 1) + 8 * g;
          const uint32_t byte = (uint32_t)(mk >> bit) & 0xFFu;
          const uint32_t idx = L.wpre[i][ks >> 1] + (uint32_t)__popcll(mk & ((1ull << bit) - 1ull));
          acc[0] = mfma_16x16x32(expand_byte(&L.vals[i][0], idx, byte, L.lut), xf[k], acc[0]);
        }
        continue;
      }
      for (int ks = wave; ks < kMoeChunk / 32; ks += 4) {
        const int col = cbase + 32 * ks + 8 * g;
        if (cbase + 32 * ks >= a.K) break;
        const uint64_t mk = L.masks[i][ks >> 1];
        const int bit = 32 * (ks & 1) + 8 * g;
        const uint32_t byte = (uint32_t)(mk >> bit) & 0xFFu;
        const uint32_t idx = L.wpre[i][ks >> 1] + (uint32_t)__popcll(mk & ((1ull << bit) - 1ull));
        const u32x4_t wop = expand_byte(&L.vals[i][0], idx, byte, L.lut);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q < nq) {
            const int32_t tok = base + 16 * q + i;
            const u32x4_t xop = (tok < t && col < a.K) ? load16(a.X + (size_t)tok * a.K + col) : zero_u4();
            acc[q] = mfma_16x16x32(wop, xop, acc[q]);
          }
      }
    }
    // ---- the waves' partial sums meet in LDS; wave q finishes block q
    __syncthreads();
    float* red = reinterpret_cast<float*>(&L.vals[0][0]);  // [wave][q][lane][4]
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q < nq) *reinterpret_cast<f32x4_t*>(&red[((wave * 4 + q) * 64 + lane) * 4]) = acc[q];
    __syncthreads();
    if (wave < nq) {
      const int q = wave;
      f32x4_t y = zero4();
#pragma unroll
      for (int v = 0; v < 4; ++v) y += *reinterpret_cast<const f32x4_t*>(&red[((v * 4 + q) * 64 + lane) * 4]);
      const int32_t tok = base + 16 * q + i;
      const bool tok_ok = tok < t;
      // low-rank K steps: A operand B_cat,e rows [16 x 32 ranks], B operand T [32 ranks x 16 tokens]
      const int64_t brow = n0 + i;
      for (int r0 = 0; r0 < a.r_pad; r0 += 32) {
        const int ra = r0 + 8 * g;
        u32x4_t bop = zero_u4();
        if (brow < a.N && ra < a.r_cat) {
          const uint16_t* bp = bcat + (size_t)brow * a.r_cat + ra;
          if (ra + 8 <= a.r_cat && (((size_t)brow * a.r_cat + ra) & 7) == 0) {
            bop = load16(bp);
          } else {
            uint32_t wv[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const uint32_t l0 = ra + 2 * c < a.r_cat ? bp[2 * c] : 0u;
              const uint32_t l1 = ra + 2 * c + 1 < a.r_cat ? bp[2 * c + 1] : 0u;
              wv[c] = l0 | (l1 << 16);
            }
            bop = u32x4_t{wv[0], wv[1], wv[2], wv[3]};
          }
        }
        const u32x4_t top = tok_ok ? load16(a.t16 + (size_t)tok * a.r_pad + ra) : zero_u4();
        y = mfma_16x16x32(bop, top, y);
      }
      // lane holds Y[token i][n0 + 4g + c] (c = 0..3)
      if (tok_ok) {
        const int64_t n = n0 + 4 * g;
        uint16_t h[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) h[c] = f32_to_bf16(y[c]);
        uint16_t* dst = a.Y + (size_t)tok * a.N + n;
        if ((a.N & 3) == 0 && n + 3 < a.N) {
          *reinterpret_cast<u32x2_t*>(dst) =
              u32x2_t{(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (n + c < a.N) dst[c] = h[c];
        }
      }
    }
  }
}

}  // namespace

int moe_lowrank_splits(int64_t T, int64_t K, int r_pad) {
  const int64_t steps = (K + kMoeTK - 1) / kMoeTK;
  const int64_t per = std::max<int64_t>(1, T * r_pad * 4);
  return (int)std::max<int64_t>(1, std::min<int64_t>(steps, kMoeTPartCap / per));
}

size_t moe_lowrank_part_bytes(int64_t T, int64_t K, int r_pad) {
  // a bound of splits * T * r_pad * 4 that grows with T: the splits keep the
  // partials under the cap, down to one split
  const int64_t steps = (K + kMoeTK - 1) / kMoeTK;
  const size_t row = (size_t)T * r_pad * 4;
  const size_t b = std::min<size_t>((size_t)steps * row, std::max<size_t>((size_t)kMoeTPartCap, row));
  return (b + 255) / 256 * 256;
}

hipError_t launch_moe_forward(const MoeArgs& a, int32_t m_cap, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.r_cat > 0) {
    const int blocks = std::max(1, std::min(64, (m_cap + kMoeTok - 1) / kMoeTok));
    hipLaunchKernelGGL(moe_lowrank_kernel, dim3((unsigned)a.E, (unsigned)a.ksplits, (unsigned)blocks),
                       dim3(kMoeThreads), 0, s, a);
    const int64_t n = (int64_t)a.T * a.r_pad;  // (r_pad % 32 == 0)
    hipLaunchKernelGGL(moe_tsum_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s, a.tpart, a.ksplits,
                       n, a.t16);
  }
  const int64_t tiles = (a.N + kMoeRows - 1) / kMoeRows;
  hipLaunchKernelGGL(moe_fwd_kernel, dim3((unsigned)tiles, (unsigned)a.E), dim3(kMoeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace salr
