// SALR forward for many input rows (M > 16): bitmap decode in producer
// waves, double-buffered against bf16 matrix-core tiles in consumer waves,
// with the concatenated low-rank product folded in as extra K tiles.
//
// Method: gist.science summary of "Sparsity-Aware Low-Rank Representation
// ...", Methodology 4 (two-stage pipeline: stage 1 rebuilds dense sub-blocks
// of W_s from the bitmap and the packed values, stage 2 feeds them to
// matrix-core GEMM tiles, the stages decoupled so decode does not stall the
// multiply) and Methodology 3 (one GEMM for all stacked adapters).
//
// One workgroup: BM = 256 tokens x BN = 128 outputs, 8 waves, K walked in
// 64-column tiles (one bitmap word per W row).  The two stages run in
// different waves that share each SIMD:
//   * waves 0-3 (consumers) each own 128 tokens x 64 outputs (8 x 4 MFMA
//     16x16 tiles, 32 accumulators) and do nothing but read operands from
//     LDS and issue v_mfma_f32_16x16x32_bf16;
//     Each phase they also send the X tile two phases ahead straight to LDS
//     (global_load_lds, a ring of three buffers), issued after their operand
//     reads: with such a load in flight the compiler makes every later LDS
//     access of the wave wait for it, and a consumer has none left in the
//     phase;
//   * waves 4-7 (producers) decode the W tile of the next phase into LDS and
//     keep the packed values two tiles ahead in registers.
// One LDS barrier per phase.  Because the decode and the multiply are in
// different waves, a SIMD issues the producer's vector instructions while
// its consumer's matrix instructions run.
//
// The product is computed as Y^T = W_s X^T: a consumer lane's accumulator
// rows are four consecutive outputs of one token (8-byte stores).  W rows
// are streams of packed values: a row's running kept count gives the first
// value of each tile, so K is walked from the split's first column on.
#include <algorithm>

#include "salr_device.hpp"
#include "salr_kernels.hpp"

namespace salr {
namespace {

constexpr int kDies = 8;             // XCDs of the GPU, each with its own L2
constexpr int64_t kFillItems = 256;  // work items wanted to occupy the CUs
constexpr int BM = 256;              // tokens per workgroup
constexpr int BN = 128;              // outputs (W rows) per workgroup
constexpr int kThreads = 512;
constexpr int kCons = 256;           // consumer threads (waves 0-3)
constexpr int kVRow = 40;            // words per row of staged values (10 chunks)
constexpr int kVLoads = 5;           // 16-byte value chunks per producer thread per tile
constexpr int kXLoads = BM * 8 / 256;  // X chunks (direct-to-LDS loads) per consumer thread per tile

// A 64-column bf16 tile row is 8 chunks of 16 bytes at chunk slot
// (c ^ (row & 7)): a 16-row MFMA operand read (one chunk per row) hits every
// bank once per pass, and a whole-wave direct-to-LDS load (64 lanes x 16
// bytes, contiguous) fills 8 rows by choosing which chunk each lane fetches.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

// s_waitcnt with vmcnt = n (n < 64), expcnt and lgkmcnt not waited on
// (gfx9 encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14); the
// compiler fences keep every memory operation on its side of the wait.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__global__ __launch_bounds__(kThreads) void fwd_mm_kernel(LargeFwdArgs a) {
  __shared__ u32x4_t xl0[BM * 8], xl1[BM * 8], xl2[BM * 8];  // X ring (or bf16 T for the low-rank tiles)
  __shared__ u32x4_t wl0[BN * 8], wl1[BN * 8];  // decoded W tiles (or B_cat^T slices)
  __shared__ uint32_t vl[BN * kVRow];     // packed values of the tile being decoded
  __shared__ u32x2_t luts[4][16];  // the nibble selectors, one copy per producer wave

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;

  // Tile of this workgroup.  Workgroups are dealt to the 8 dies in turn
  // (id % 8); tiles are numbered token-block-major and each die gets a
  // contiguous run of them, so the workgroups on one die share an X slab in
  // that die's L2.  With K splits, consecutive work items of a die take the
  // same split of neighbouring tiles.
  const int nb = (int)((a.N + BN - 1) / BN);
  const int total = nb * ((a.M + BM - 1) / BM);
  const int items = total * a.ksplit;
  const int per_die = (items + kDies - 1) / kDies;
  const int id = (int)blockIdx.x;
  const int item = (id % kDies) * per_die + id / kDies;
  if (item >= items) return;
  const int tile = item % total, split = item / total;
  const int64_t n0 = (int64_t)(tile % nb) * BN;
  const int m0 = (tile / nb) * BM;
  const int kt0 = split * a.kt_per;
  const int nk = min((a.K + 63) / 64, kt0 + a.kt_per);
  const int n_main = nk - kt0;

  // Low-rank tiles: ranks [rlo, rhi) in 64-rank tiles, tile j taken by K
  // split j mod ksplit (the split sums add them like any other K tile), so
  // no split carries all of them; a fused layer's row block takes only its
  // part's ranks (b_cat is zero outside them; every part holds whole
  // 256-row blocks).
  // (static indices: a runtime index into the argument's arrays would move
  // the whole argument block to private memory)
  int rlo = 0, rhi = a.r_cat;
  bool found = false;
#pragma unroll
  for (int p = 0; p < 8; ++p)
    if (!found && p < a.nparts && n0 < a.part_row_end[p]) {
      rlo = a.part_rank0[p];
      rhi = rlo + a.part_nrank[p];
      found = true;
    }
  const int n_lr_all = rhi > rlo ? (rhi - rlo + 63) / 64 : 0;
  const int n_lr = n_lr_all > split ? (n_lr_all - split + a.ksplit - 1) / a.ksplit : 0;
  const int phases = n_main + n_lr;

  // X buffer of phase p (a ring of three) and W buffer (two)
  const auto xbuf = [&](int p) __attribute__((always_inline)) -> u32x4_t* {
    const int b = p % 3;
    return b == 0 ? xl0 : (b == 1 ? xl1 : xl2);
  };

  if (wave < 4) {
    // ------------------------------------------------------------ consumer
    const int wm = wave >> 1, wn = wave & 1;  // 128-token half, 64-output half
    // X tile loads: load j of this wave fills tile rows 8 (8 wave + j) ..
    // +7, lane l fetching chunk (l & 7) ^ (row & 7) of row 8 (8 wave + j) +
    // l / 8 (the swizzled layout), from byte offsets formed once (used when
    // M * K * 2 < 2^32).  Rows past M and columns past K read clamped
    // (in-bounds) addresses: such rows reach outputs that are never stored,
    // such columns meet zero weights.
    const int nk_all = (a.K + 63) / 64;
    uint32_t xoff[kXLoads];
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) {
      const int row = 8 * (kXLoads * wave + j) + (lane >> 3);
      const int chunk = (lane & 7) ^ (row & 7);
      xoff[j] = ((uint32_t)min(m0 + row, a.M - 1) * (uint32_t)a.K + 8u * (uint32_t)chunk) * 2u;
    }
    const auto dma_x = [&](u32x4_t* xt, int kt) __attribute__((always_inline)) {
      kt = min(kt, nk_all - 1);
      const int k0 = kt * 64;
      if (a.x_off32 && k0 + 64 <= a.K) {
        const char* const xb = reinterpret_cast<const char*>(a.X + k0);
#pragma unroll
        for (int j = 0; j < kXLoads; ++j)
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(xb + xoff[j]),
                                           reinterpret_cast<uint32_t*>(xt + (kXLoads * wave + j) * 64), 16, 0, 0);
      } else {
#pragma unroll
        for (int j = 0; j < kXLoads; ++j) {
          const int row = 8 * (kXLoads * wave + j) + (lane >> 3);
          const int chunk = (lane & 7) ^ (row & 7);
          const int m = min(m0 + row, a.M - 1), k = min(k0 + 8 * chunk, a.K - 8);
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(a.X + (size_t)m * a.K + k),
                                           reinterpret_cast<uint32_t*>(xt + (kXLoads * wave + j) * 64), 16, 0, 0);
        }
      }
    };
    f32x4_t acc[4][8];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 8; ++y) acc[x][y] = zero4();
    // prologue: X of the first two tiles
    if (n_main > 0) dma_x(xl0, kt0);
    if (n_main > 1) dma_x(xl1, kt0 + 1);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();  // (and tile 0's W staged by the producers)
    for (int p = 0; p < phases; ++p) {
      const u32x4_t* xt = xbuf(p);
      const u32x4_t* wt = (p & 1) ? wl1 : wl0;
      const bool more = p + 2 < n_main;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4_t av[4], bv[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) av[t] = wt[swz(wn * 64 + t * 16 + i, ks * 4 + g)];
#pragma unroll
        for (int t = 0; t < 8; ++t) bv[t] = xt[swz(wm * 128 + t * 16 + i, ks * 4 + g)];
        // after the phase's last operand reads: X two tiles ahead into the
        // buffer freed a phase ago (every wave's reads of it ended at the
        // last barrier)
        if (ks == 1 && more) dma_x(xbuf(p + 2), kt0 + p + 2);
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
          for (int tm = 0; tm < 8; ++tm) acc[tn][tm] = mfma_16x16x32(av[tn], bv[tm], acc[tn][tm]);
      }
      // X of the next phase (issued a phase ago) has landed once at most
      // this phase's loads are outstanding
      if (more)
        wait_vmcnt<kXLoads>();
      else
        __builtin_amdgcn_s_waitcnt(0);
      lds_barrier();
    }

    // epilogue: lane holds Y[m][n .. n+3]
    if (a.ksplit > 1) {
      float* part = a.ypart + (size_t)split * a.M * a.N;
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) {
        const int64_t n = n0 + wn * 64 + tn * 16 + 4 * g;
#pragma unroll
        for (int tm = 0; tm < 8; ++tm) {
          const int m = m0 + wm * 128 + tm * 16 + i;
          if (m >= a.M) continue;
          float* dst = part + (size_t)m * a.N + n;
          if ((a.N & 3) == 0 && n + 3 < a.N) {
            *reinterpret_cast<f32x4_t*>(dst) = acc[tn][tm];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < a.N) dst[e] = acc[tn][tm][e];
          }
        }
      }
      return;
    }
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
      const int64_t n = n0 + wn * 64 + tn * 16 + 4 * g;
#pragma unroll
      for (int tm = 0; tm < 8; ++tm) {
        const int m = m0 + wm * 128 + tm * 16 + i;
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
    return;
  }

  // -------------------------------------------------------------- producer
  const int ptid = tid - kCons;          // 0..255
  const int pwave = ptid >> 6;           // 0..3
  // (this wave's own copy: its decode starts before the first barrier, and
  // a wave's LDS operations complete in order)
  u32x2_t* const lut = luts[pwave];
  if (lane < 16) lut[lane] = nibble_selectors(lane);
  const int prow = ptid >> 1, phalf = ptid & 1;  // W row of the tile, column half
  const int64_t grow = n0 + prow;
  const bool row_ok = grow < a.N;
  const int64_t row_base = row_ok ? grow * a.n_keep : 0;
  const uint64_t* mrow = a.masks + (row_ok ? grow * a.kw : 0);
  // (raw word of a clamped, unconditional load; bounds applied at use)
  auto mask_raw = [&](int kt) __attribute__((always_inline)) -> uint64_t { return mrow[min(kt, a.kw - 1)]; };
  auto mask_ok = [&](uint64_t w, int kt) __attribute__((always_inline)) -> uint64_t { return (row_ok && kt < nk) ? w : 0ull; };

  // The packed values of one tile of this row: the 10 chunks from the one
  // holding its first value (value index row_base + run) cover up to 64
  // values and the decode window's overrun; this thread loads every other
  // one.  Unconditional: the first chunk starts at most at the end of the
  // values, and 10 chunks from there stay inside the buffer's 256-byte tail
  // padding.
  auto load_v = [&](u32x4_t (&r)[kVLoads], uint32_t run) __attribute__((always_inline)) {
    const uint16_t* const vq = a.values + ((row_base + run) >> 3) * 8;
#pragma unroll
    for (int u = 0; u < kVLoads; ++u) r[u] = load16(vq + (phalf + 2 * u) * 8);
  };
  auto store_v = [&](const u32x4_t (&r)[kVLoads]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kVLoads; ++u) *reinterpret_cast<u32x4_t*>(&vl[prow * kVRow + (phalf + 2 * u) * 4]) = r[u];
  };
  // Decode this thread's 32 columns of the row's tile into dense bf16 (the
  // row's staged values come from this thread and its neighbour lane, whose
  // LDS stores precede these reads in the wave's order).
  auto decode = [&](u32x4_t* wt, uint32_t run, uint64_t mk) __attribute__((always_inline)) {
    const uint16_t* rowbuf = reinterpret_cast<const uint16_t*>(&vl[prow * kVRow]);
    uint32_t idx = (uint32_t)((row_base + run) & 7) + (phalf ? (uint32_t)__popc((uint32_t)mk) : 0u);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t byte = (uint32_t)(mk >> (32 * phalf + 8 * b)) & 0xFFu;
      wt[swz(prow, 4 * phalf + b)] = expand_byte(rowbuf, idx, byte, lut);
      idx += __popc(byte);
    }
  };
  // Low-rank tile l of this split into buffers xt (bf16 T, the sum of the
  // K-split partials of X A_cat made by the previous launch) and wt (B_cat^T
  // slices); ranks at or past rhi meet zero B_cat columns below.
  auto stage_lowrank = [&](int l, u32x4_t* xt, u32x4_t* wt) __attribute__((always_inline)) {
    const int r0 = rlo + 64 * (split + l * a.ksplit);  // this split's l-th low-rank tile
    u32x4_t tv[BM * 8 / 256];
#pragma unroll
    for (int u = 0; u < BM * 8 / 256; ++u) {
      const int c = ptid + 256 * u;
      const int row = c >> 3, ch = c & 7;
      const int m = m0 + row, k = r0 + 8 * ch;
      tv[u] = (m < a.M && k < rhi) ? load16(a.t16 + (size_t)m * a.r_pad + k) : zero_u4();
    }
#pragma unroll
    for (int u = 0; u < BM * 8 / 256; ++u) {
      const int c = ptid + 256 * u;
      xt[swz(c >> 3, c & 7)] = tv[u];
    }
    // B_cat^T row grow, ranks [r0 + 32 phalf, + 32): 16-byte loads when the
    // chunk lies inside [rlo, rhi) and is 16-byte aligned
    const uint16_t* brow = a.b_cat + (row_ok ? grow * a.r_cat : 0);
#pragma unroll
    for (int c8 = 0; c8 < 4; ++c8) {
      const int ra = r0 + 32 * phalf + 8 * c8;
      u32x4_t v = zero_u4();
      if (row_ok && ra < rhi) {
        if (ra + 8 <= rhi && (((size_t)grow * a.r_cat + ra) & 7) == 0) {
          v = load16(brow + ra);
        } else {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = ra + 2 * e < rhi ? brow[ra + 2 * e] : 0u;
            const uint32_t hi = ra + 2 * e + 1 < rhi ? brow[ra + 2 * e + 1] : 0u;
            w[e] = lo | (hi << 16);
          }
          v = u32x4_t{w[0], w[1], w[2], w[3]};
        }
      }
      wt[swz(prow, 4 * phalf + c8)] = v;
    }
  };

  // kept values of the row before this split: the lookup table entry at the
  // last 1024-column boundary, plus the bitmap words after it
  uint32_t run0 = 0;
  if (kt0 > 0) {
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

  // ---- prologue: tile kt0 decoded; the values of kt0+1, kt0+2 on their way
  const uint64_t mk0 = mask_ok(mask_raw(kt0), kt0);
  uint64_t mk1 = mask_ok(mask_raw(kt0 + 1), kt0 + 1);
  uint64_t mk2 = mask_ok(mask_raw(kt0 + 2), kt0 + 2);
  uint64_t mk3raw = mask_raw(kt0 + 3);
  uint32_t run1 = run0 + (uint32_t)__popcll(mk0);   // first value of tile kt+1
  uint32_t run2 = run1 + (uint32_t)__popcll(mk1);   // of tile kt+2
  u32x4_t va[kVLoads], vb[kVLoads];
  if (n_main > 0) {
    load_v(va, run0);
    load_v(vb, run1);
    store_v(va);
    decode(wl0, run0, mk0);
    load_v(va, run2);
  } else {
    stage_lowrank(0, xl0, wl0);
  }
  lds_barrier();

  // ---- phases: the consumers multiply the tile of phase p (kt = kt0 + p)
  // while this wave prepares the W tile of phase p + 1 and issues the loads
  // of later tiles.  Main phases are unrolled by two so that the W buffers
  // and the two value register sets are named.
  auto main_phase = [&](int p, u32x4_t(&vnext)[kVLoads], u32x4_t* wnext) __attribute__((always_inline)) {
    const int kt = kt0 + p;
    // tile kt+1: its values (loaded two phases ago) to LDS, decoded; the
    // values of kt+3 requested into the set just stored, and the bitmap
    // word of kt+4
    store_v(vnext);
    decode(wnext, run1, mk1);
    const uint64_t mk3 = mask_ok(mk3raw, kt + 3);
    const uint32_t run3 = run2 + (uint32_t)__popcll(mk2);
    load_v(vnext, run3);
    mk3raw = mask_raw(kt + 4);
    mk1 = mk2;
    mk2 = mk3;
    run1 = run2;
    run2 = run3;
    lds_barrier();
  };
  int p = 0;
  for (; p + 2 < n_main; p += 2) {
    main_phase(p, vb, wl1);
    main_phase(p + 1, va, wl0);
  }
  if (p + 1 < n_main) main_phase(p++, vb, wl1);
  // the last main phase and the low-rank phases: stage the next low-rank
  // tile (its X buffer got no direct-to-LDS load: the consumers load X only
  // for main tiles)
  for (; p < phases; ++p) {
    if (p + 1 < phases) stage_lowrank(p + 1 - n_main, xbuf(p + 1), ((p + 1) & 1) ? wl1 : wl0);
    lds_barrier();
  }
}

// ---------------------------------------------------------------------------
// Partial T = X * A_cat over one K range per workgroup, fp32, written to
// tpart[split][M][r_pad] (columns >= r_cat are zero).  A workgroup owns
// 16 kTT tokens and one K range; its four waves take the range's 32-column
// steps in turn (wave w: steps w, w + 4, ...), each wave loading its A_cat
// operands straight from memory once for all kTT token tiles (a batch of
// steps at a time, every load of the batch issued before the first
// multiply), and the waves' sums are added in wave order at the end.  The
// splits are summed by the next launch in split order, so the result does
// not depend on scheduling.
// ---------------------------------------------------------------------------
constexpr int kTThreads = 256;
constexpr int kTWaves = kTThreads / 64;
constexpr int kMaxRTiles = 16;   // r_pad <= 256
// kRT: rank tiles the instance holds (at least r_pad / 16); kTT: 16-token
// tiles per workgroup; kTBatch: steps whose loads are issued together.
template <int kRT, int kTT, int kTBatch>
__global__ __launch_bounds__(kTThreads) void lowrank_t_kernel(LowRankTArgs a) {
  __shared__ f32x4_t red[kTWaves - 1][kRT][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int tok0 = blockIdx.x * 16 * kTT + i, ks = blockIdx.y;
  const int rt = a.r_pad / 16;
  const int k0 = ks * a.k_chunk, k1 = min(a.K, k0 + a.k_chunk);
  const int nsteps = (k1 - k0 + 31) / 32;

  f32x4_t acc[kTT][kRT];
#pragma unroll
  for (int t = 0; t < kTT; ++t)
#pragma unroll
    for (int j = 0; j < kRT; ++j) acc[t][j] = zero4();
  for (int s0 = wave; s0 < nsteps; s0 += kTWaves * kTBatch) {
    u32x4_t xv[kTBatch][kTT], av[kTBatch][kRT];
#pragma unroll
    for (int b = 0; b < kTBatch; ++b) {
      const int k = k0 + 32 * (s0 + kTWaves * b) + 8 * g;  // (k >= k1 past the last step)
#pragma unroll
      for (int j = 0; j < kRT; ++j) {
        const int r = 16 * j + i;
        av[b][j] = (j < rt && r < a.r_cat && k < k1) ? load16(a.a_cat + (size_t)r * a.K + k) : zero_u4();
      }
#pragma unroll
      for (int t = 0; t < kTT; ++t) {
        const int token = tok0 + 16 * t;
        xv[b][t] = (token < a.M && k < k1) ? load16(a.X + (size_t)token * a.K + k) : zero_u4();
      }
    }
#pragma unroll
    for (int b = 0; b < kTBatch; ++b)
#pragma unroll
      for (int j = 0; j < kRT; ++j)
        if (j < rt)
#pragma unroll
          for (int t = 0; t < kTT; ++t) acc[t][j] = mfma_16x16x32(av[b][j], xv[b][t], acc[t][j]);
  }
  // the waves' sums, in wave order, one token tile at a time; lane holds
  // T[token][16j + 4g + e]
#pragma unroll
  for (int t = 0; t < kTT; ++t) {
    if (t > 0) __syncthreads();  // (wave 0 has read the previous tile's sums)
    if (wave > 0)
#pragma unroll
      for (int j = 0; j < kRT; ++j)
        if (j < rt) red[wave - 1][j][lane] = acc[t][j];
    __syncthreads();
    const int token = tok0 + 16 * t;
    if (wave == 0 && token < a.M) {
      float* dst = a.tpart + ((size_t)ks * a.M + token) * a.r_pad;
#pragma unroll
      for (int j = 0; j < kRT; ++j)
        if (j < rt) {
          f32x4_t v = acc[t][j];
#pragma unroll
          for (int w = 0; w < kTWaves - 1; ++w) v += red[w][j][lane];
          *reinterpret_cast<f32x4_t*>(&dst[16 * j + 4 * g]) = v;
        }
    }
  }
}

template <int kRT, int kTT>
void launch_lowrank_t_one(const LowRankTArgs& a, hipStream_t s) {
  // (64-token workgroups run one wave per SIMD anyway: four steps a batch,
  // so that a split of 512 columns is one round trip)
  constexpr int kB = kTT == 4 ? 4 : 2;
  const dim3 grid((a.M + 16 * kTT - 1) / (16 * kTT), a.splits);
  hipLaunchKernelGGL((lowrank_t_kernel<kRT, kTT, kB>), grid, dim3(kTThreads), 0, s, a);
}

// Sum over `splits` partial arrays `stride` floats apart of the 8 floats at
// p, in split order.  The loads of 8 splits at a time are issued together
// (clamped to split 0 past the end, those terms not added), so a thread
// waits for one memory round trip per 8 splits rather than per split.
__device__ __forceinline__ void sum_split_partials(const float* p, int64_t stride, int splits, f32x4_t& lo,
                                                   f32x4_t& hi) {
  constexpr int kU = 8;
  lo = zero4();
  hi = zero4();
  for (int s0 = 0; s0 < splits; s0 += kU) {
    f32x4_t l[kU], h[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float* src = p + (size_t)(s0 + u < splits ? s0 + u : 0) * stride;
      l[u] = *reinterpret_cast<const f32x4_t*>(src);
      h[u] = *reinterpret_cast<const f32x4_t*>(src + 4);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (s0 + u < splits) {
        lo += l[u];
        hi += h[u];
      }
  }
}

// T = bf16(sum of the K-split partials of X A_cat, in split order), [M][r_pad]
// with r_pad a multiple of 16: 8 ranks a thread.
__global__ __launch_bounds__(256) void reduce_t_kernel(const float* tpart, int splits, int64_t MR, uint16_t* t16) {
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (e0 >= MR) return;
  f32x4_t lo, hi;
  sum_split_partials(tpart + e0, MR, splits, lo, hi);
  *reinterpret_cast<u32x4_t*>(t16 + e0) =
      u32x4_t{(uint32_t)f32_to_bf16(lo[0]) | ((uint32_t)f32_to_bf16(lo[1]) << 16),
              (uint32_t)f32_to_bf16(lo[2]) | ((uint32_t)f32_to_bf16(lo[3]) << 16),
              (uint32_t)f32_to_bf16(hi[0]) | ((uint32_t)f32_to_bf16(hi[1]) << 16),
              (uint32_t)f32_to_bf16(hi[2]) | ((uint32_t)f32_to_bf16(hi[3]) << 16)};
}

// Y = bf16(sum of the K-split partials, in split order): 8 outputs a thread
// (16-byte loads and store when MN is a multiple of 8, as it is whenever N is).
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* part, uint16_t* Y, int64_t MN, int ksplit) {
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (e0 >= MN) return;
  if ((MN & 7) == 0) {
    f32x4_t lo, hi;
    sum_split_partials(part + e0, MN, ksplit, lo, hi);
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

hipError_t launch_lowrank_t(const LowRankTArgs& a, hipStream_t s) {
  const int rt = a.r_pad / 16;
  if (rt < 1 || rt > kMaxRTiles) return hipErrorInvalidValue;
  // 64 tokens a workgroup (each A_cat operand used for four token tiles;
  // 32 above 128 ranks, for registers) while that still gives a workgroup
  // per CU, else 16; the smallest instance that holds rt rank tiles
  const bool big = (int64_t)((a.M + 63) / 64) * a.splits >= 256;
  if (rt <= 2)
    big ? launch_lowrank_t_one<2, 4>(a, s) : launch_lowrank_t_one<2, 1>(a, s);
  else if (rt <= 4)
    big ? launch_lowrank_t_one<4, 4>(a, s) : launch_lowrank_t_one<4, 1>(a, s);
  else if (rt <= 6)
    big ? launch_lowrank_t_one<6, 4>(a, s) : launch_lowrank_t_one<6, 1>(a, s);
  else if (rt <= 8)
    big ? launch_lowrank_t_one<8, 4>(a, s) : launch_lowrank_t_one<8, 1>(a, s);
  else if (rt <= 12)
    big ? launch_lowrank_t_one<12, 2>(a, s) : launch_lowrank_t_one<12, 1>(a, s);
  else
    big ? launch_lowrank_t_one<16, 2>(a, s) : launch_lowrank_t_one<16, 1>(a, s);
  const int64_t mr = (int64_t)a.M * a.r_pad;  // (r_pad % 16 == 0)
  hipLaunchKernelGGL(reduce_t_kernel, dim3((unsigned)((mr + 2047) / 2048)), dim3(256), 0, s, a.tpart, a.splits, mr,
                     a.t16);
  return hipGetLastError();
}

int64_t fwd_large_tiles(int64_t N, int64_t M) { return ((N + BN - 1) / BN) * ((M + BM - 1) / BM); }

int fwd_large_ksplit(int64_t N, int64_t K, int64_t M) {
  // enough work items for every CU, each split at least 8 K tiles, at most 8
  const int64_t tiles = fwd_large_tiles(N, M), nk = (K + 63) / 64;
  int64_t s = std::min<int64_t>({kFillItems / std::max<int64_t>(tiles, 1), nk / 8, 8});
  return (int)std::max<int64_t>(s, 1);
}

size_t fwd_large_part_bytes(int64_t N, int64_t K, int64_t M_max) {
  // ksplit * tiles <= kFillItems, so the partials never exceed kFillItems
  // whole tiles; nothing when no M <= M_max splits
  size_t most = 0;
  for (int64_t M = BM; M - BM < M_max; M += BM) {
    const int s = fwd_large_ksplit(N, K, std::min<int64_t>(M, M_max));
    if (s > 1) most = std::max(most, (size_t)s * std::min<int64_t>(M, M_max) * N * 4);
    if (fwd_large_tiles(N, M) >= kFillItems) break;
  }
  return most;
}

hipError_t launch_fwd_large(const LargeFwdArgs& a, hipStream_t s) {
  // (ceil(work items / 8) workgroups per die: see the tile mapping)
  const int64_t items = fwd_large_tiles(a.N, a.M) * a.ksplit;
  const dim3 grid((unsigned)((items + kDies - 1) / kDies * kDies));
  hipLaunchKernelGGL(fwd_mm_kernel, grid, dim3(kThreads), 0, s, a);
  if (a.ksplit > 1) {
    const int64_t mn = a.N * (int64_t)a.M;
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((mn + 2047) / 2048)), dim3(256), 0, s, a.ypart, a.Y, mn,
                       a.ksplit);
  }
  return hipGetLastError();
}

}  // namespace salr
