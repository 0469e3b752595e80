// SALR forward for few input rows (M <= 16) on layers with more than one
// round of 16-row work: persistent workgroups that stream their weights
// through two LDS buffers.
//
// Method: gist.science summary of "Sparsity-Aware Low-Rank Representation
// ...", Methodology 4 (stage 1 rebuilds dense blocks from bitmap + packed
// values, stage 2 multiplies them on matrix units; the stages decoupled) and
// Methodology 3 (all adapters run as one product on the shared input).
//
// One workgroup (16 waves) per CU owns a run of whole 16-row tiles and walks
// each tile's K in chunks of kChunk columns.  A chunk of a row is its bitmap
// words plus its kept values, whose bounds are lookup-table entries (one
// every 1024 columns), so every load of a chunk is issued at once, straight
// into LDS.  While the waves decode chunk q from one buffer, the bitmap and
// values of chunk q + 1 stream into the other, so HBM is never idle between
// chunks (a workgroup that loads everything and then decodes leaves the
// memory system idle half the time once the layer needs several rounds of
// workgroups).  Per chunk, wave w issues row w's loads and decodes 4
// 32-column steps of all 16 rows (the same decode as the one-round kernel:
// register-held bitmap words, nibble expansion through a 16-entry selector
// table, swap-AB MFMA with the tokens on the 16-column side).  Tiles
// complete inside one workgroup, so partial sums never leave it.
//
// The low-rank term: the first n_pieces workgroups each compute one piece
// of T = X A_cat (16 ranks x t_chunks * 1024 columns) on their upper 8
// waves, whose operand loads go out before their first chunk's loads, so the
// piece waits for nothing else; it is published as tagged words, and the
// last of a rank tile sums the tile's pieces (fixed order) into bf16 T (the
// protocol of the one-round kernel; every workgroup is resident, so these
// waits end).
// At a tile's end, wave k adds B_cat^T[rows, 32k..] T^T[32k.., tokens] to
// its accumulator (T read once per workgroup, B_cat rows fetched with the
// tile's last chunk), then the 16 waves' sums meet in LDS.
#include "salr_device.hpp"
#include "salr_kernels.hpp"

namespace salr {
namespace {

constexpr int kSThreads = 1024;
constexpr int kSWaves = kSThreads / 64;
constexpr int kSRows = 16;
constexpr int kCSteps = kChunk / 32 / kSWaves;   // 32-column steps per wave per chunk
constexpr int kCWords = kChunk / 64;             // bitmap words per row per chunk
constexpr int kCMaskRow = kCWords + 1;           // (one word of padding: rows in distinct bank pairs)
constexpr int kPieceWave0 = 8;                    // waves kPieceWave0.. compute a T piece
constexpr int kSPieceSteps = 1024 / 32 / (kSWaves - kPieceWave0);
constexpr int kSFinBatch = 4;
static_assert(kSWaves == kSRows, "wave w issues the loads of row w");
static_assert(kCSteps % 2 == 0, "a wave's steps start on a bitmap word");

struct alignas(16) SHead {
  u32x2_t lut[16];
  uint32_t vbase[2][kSRows];  // LDS value slot of each row's first value in the buffer's chunk
  uint32_t tag;
  uint32_t pad[3];
};
static_assert(sizeof(SHead) % 16 == 0, "buffers must stay 16-byte aligned");

__device__ __forceinline__ size_t buf_bytes(int vcap) {
  return (size_t)kSRows * kCMaskRow * 8 + (size_t)kSRows * vcap * 16;
}

__device__ __forceinline__ u32x4_t load_x_frag_s(const uint16_t* X, int M, int K, int m, int col) {
  if (m < M && col < K) return load16(X + (size_t)m * K + col);
  return zero_u4();
}

__global__ __launch_bounds__(kSThreads) void fwd_stream_kernel(StreamFwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  SHead& H = *reinterpret_cast<SHead*>(smem);
  unsigned char* const buf0 = smem + sizeof(SHead);
  const size_t bbytes = buf_bytes(a.vcap);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const uint32_t n_wgs = gridDim.x;
  const uint32_t wg = blockIdx.x;
  uint32_t* const err = a.err;

  // this workgroup's tiles [t_begin, t_end), walked chunk by chunk
  const int t_begin = (int)wg * a.tiles_per_wg;
  const int t_end = min(a.n_tiles, t_begin + a.tiles_per_wg);
  const int nc = (a.K + kChunk - 1) / kChunk;  // chunks per tile
  const int n_q = (t_end - t_begin) * nc;

  // launch tag (drawn now, resolved by wave 0 where first needed)
  uint64_t drawn = 0;
  if (a.r_cat > 0 && tid == 0) drawn = draw_ticket(a.tickets, wg, n_wgs);
  uint32_t tag = 0;
  const auto resolve_tag = [&]() {
    uint32_t t = 0;
    if (lane == 0) t = tag_from_ticket(a.tickets, drawn, wg, n_wgs);
    tag = __shfl(t, 0);
  };
  if (tid < 16) H.lut[tid] = nibble_selectors(tid);

  // ---- per-chunk loads: wave w carries row w (bitmap words and values to
  // LDS); every wave its X operand slices for the chunk (registers); waves
  // with a low-rank chunk its B_cat operand when the chunk ends a tile.
  // Lookup-table row of the tile being issued (lane e holds entry e), and of
  // the next tile (requested one tile ahead).
  const int n_chunks32 = a.r_pad / 32;
  uint32_t lut_cur = 0, lut_nxt = 0;
  const auto load_lut = [&](int t) -> uint32_t {
    const int64_t row = (int64_t)t * kSRows + wave;
    return (t < t_end && row < a.N && lane < a.ng) ? a.offsets[row * a.ng + lane] : 0u;
  };
  // B_cat operand of this wave's rank chunk for tile t: lane (i, g) holds
  // B_cat[row 16t + i][32 wave + 8g .. +7]
  u32x4_t bc = zero_u4();
  const auto load_bc = [&](int t) {
    if (wave >= n_chunks32) return;
    const int64_t brow = (int64_t)t * kSRows + i;
    const int rb = 32 * wave + 8 * g;
    if (a.r_cat % 8 == 0) {
      bc = (brow < a.N && rb < a.r_cat) ? load16(a.b_cat + brow * a.r_cat + rb) : zero_u4();
    } else {
      uint32_t w4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ra = rb + 2 * e;
        const uint32_t l0 = (brow < a.N && ra < a.r_cat) ? a.b_cat[brow * a.r_cat + ra] : 0u;
        const uint32_t l1 = (brow < a.N && ra + 1 < a.r_cat) ? a.b_cat[brow * a.r_cat + ra + 1] : 0u;
        w4[e] = l0 | (l1 << 16);
      }
      bc = u32x4_t{w4[0], w4[1], w4[2], w4[3]};
    }
  };
  // (a tile of several chunks takes its B_cat operand with its last chunk,
  // after the previous tile's end; one-chunk tiles take it after the
  // previous tile's epilogue)
  const auto issue = [&](int qn, unsigned char* buf, int bsel, u32x4_t (&xd)[kCSteps]) {
    const int t = t_begin + qn / nc, c = qn % nc;
    const int64_t row = (int64_t)t * kSRows + wave;
    const bool live = row < a.N;
    const int col0 = c * kChunk;
    const int ncols = min(kChunk, a.K - col0);
    const int nwords = (ncols + 63) / 64;
    uint64_t* const mdst = reinterpret_cast<uint64_t*>(buf) + wave * kCMaskRow;
    uint32_t* const vdst = reinterpret_cast<uint32_t*>(buf + (size_t)kSRows * kCMaskRow * 8) + (size_t)wave * a.vcap * 4;
    // bitmap words (no dependence on the table), B_cat operand
    if (live) {
      const uint32_t* msrc = reinterpret_cast<const uint32_t*>(a.masks + row * a.kw + c * kCWords);
      if (lane < 2 * nwords) __builtin_amdgcn_global_load_lds(msrc + lane, reinterpret_cast<uint32_t*>(mdst), 4, 0, 0);
    } else {
      for (int w = lane; w < 2 * kCMaskRow; w += 64) reinterpret_cast<uint32_t*>(mdst)[w] = 0u;
    }
    if (nc > 1 && c == nc - 1) load_bc(t);
    // the row's kept values of the chunk: bounds from the table row
    if (c == 0) {
      if (qn > 0) lut_cur = lut_nxt;
      lut_nxt = load_lut(t + 1);
    }
    const int e0 = c * (kChunk / 1024), e1 = e0 + kChunk / 1024;
    const uint32_t lo = (uint32_t)__shfl((int)lut_cur, min(e0, 63));
    const uint32_t hi = e1 < a.ng ? (uint32_t)__shfl((int)lut_cur, min(e1, 63)) : (uint32_t)a.n_keep;
    if (live) {
      const int64_t va = row * a.n_keep + lo, vb = row * a.n_keep + hi;
      const int64_t q0 = va >> 3;
      const int64_t nch = vb > va ? ((vb + 7) >> 3) - q0 : 0;
      const uint32_t* vsrc = reinterpret_cast<const uint32_t*>(a.values) + q0 * 4;
      for (int64_t b = 0; b * 64 < nch; ++b) {
        const int64_t ch = b * 64 + lane;
        if (ch < nch) __builtin_amdgcn_global_load_lds(vsrc + ch * 4, vdst + b * 256, 16, 0, 0);
      }
      if (lane == 0) H.vbase[bsel][wave] = (uint32_t)(wave * a.vcap * 8) + (uint32_t)(va & 7);
    } else {
      if (lane == 0) H.vbase[bsel][wave] = (uint32_t)(wave * a.vcap * 8);
    }
    // X slices last: they come from L2, the values from HBM
#pragma unroll
    for (int s = 0; s < kCSteps; ++s)
      xd[s] = load_x_frag_s(a.X, a.M, a.K, i, col0 + 32 * (wave * kCSteps + s) + 8 * g);
  };

  // ---- T pieces: workgroup p < n_pieces computes piece p = (rank tile j,
  // K range kp) on waves kPieceWave0.., whose operand loads go out before
  // their first chunk's loads (so the piece waits for them alone); the last
  // piece of a rank tile to arrive sums the tile (in K order) into bf16 T.
  const int n_pieces = a.r_tiles * a.t_pieces;
  const bool producer = (int)wg < n_pieces;
  const bool pwave = producer && wave >= kPieceWave0;
  const int piece = (int)wg;
  const int pj = piece / max(a.t_pieces, 1), pkp = piece % max(a.t_pieces, 1);
  const int prank = 16 * pj + i;
  u32x4_t pav[kSPieceSteps], pxv[kSPieceSteps];
  const auto load_piece = [&](int ch) {
#pragma unroll
    for (int s = 0; s < kSPieceSteps; ++s) {
      const int col = (pkp * a.t_chunks + ch) * 1024 + 32 * ((wave - kPieceWave0) * kSPieceSteps + s) + 8 * g;
      pav[s] = (prank < a.r_cat && col < a.K) ? load16(a.a_cat + (size_t)prank * a.K + col) : zero_u4();
      pxv[s] = load_x_frag_s(a.X, a.M, a.K, i, col);
    }
  };
  if (pwave) load_piece(0);

  u32x4_t xf0[kCSteps], xf1[kCSteps];
#pragma unroll
  for (int s = 0; s < kCSteps; ++s) xf0[s] = xf1[s] = zero_u4();
  lut_cur = load_lut(t_begin);
  issue(0, buf0, 0, xf0);
  if (nc == 1) load_bc(t_begin);

  f32x4_t* const red = reinterpret_cast<f32x4_t*>(buf0 + bbytes + (size_t)kSRows * kCMaskRow * 8);
  if (producer) {
    const int j = pj;
    f32x4_t t = zero4();
    if (pwave) {
      for (int ch = 0; ch < a.t_chunks; ++ch) {
        if (ch > 0) load_piece(ch);
#pragma unroll
        for (int s = 0; s < kSPieceSteps; ++s) t = mfma_16x16x32(pav[s], pxv[s], t);
      }
    }
    // waves' sums in the second buffer's values area (no chunk there yet)
    lds_barrier();
    if (wave > 0) red[(wave - 1) * 64 + lane] = t;
    lds_barrier();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < kSWaves - 1; ++w) t += red[w * 64 + lane];
      resolve_tag();
      if (lane == 0) H.tag = tag;
      uint64_t* dst = a.tpiece + ((size_t)piece * 64 + lane) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = t[e];  // (scalar copy first: see the one-round kernel)
        store_tagged(dst + e, __float_as_uint(v), tag);
      }
      uint32_t old = 0;
      if (lane == 0) old = atomic_add_relaxed(&a.tcount[j], 1u);
      old = __shfl(old, 0);
      if (old == (uint32_t)(a.t_pieces - 1)) {
        if (lane == 0) store_coherent(&a.tcount[j], 0u);
        float sum[4] = {0.f, 0.f, 0.f, 0.f};
        for (int kp0 = 0; kp0 < a.t_pieces; kp0 += kSFinBatch) {
          uint64_t v[kSFinBatch][4];
#pragma unroll
          for (int b = 0; b < kSFinBatch; ++b)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[b][e] = (kp0 + b < a.t_pieces)
                            ? load_tagged_raw(a.tpiece + ((size_t)(j * a.t_pieces + kp0 + b) * 64 + lane) * 4 + e)
                            : 0ull;
#pragma unroll
          for (int b = 0; b < kSFinBatch; ++b) {
            if (kp0 + b < a.t_pieces) {
              bool ok = true;
#pragma unroll
              for (int e = 0; e < 4; ++e) ok &= (uint32_t)(v[b][e] >> 32) == tag;
              uint32_t w4[4];
              if (ok) {
#pragma unroll
                for (int e = 0; e < 4; ++e) w4[e] = (uint32_t)v[b][e];
              } else {
                poll_tagged<4>(a.tpiece + ((size_t)(j * a.t_pieces + kp0 + b) * 64 + lane) * 4, tag, w4, err);
              }
#pragma unroll
              for (int e = 0; e < 4; ++e) sum[e] += __uint_as_float(w4[e]);
            }
          }
        }
        uint64_t* fin = a.tfinal + ((size_t)j * 64 + lane) * 2;
        store_tagged(fin, (uint32_t)f32_to_bf16(sum[0]) | ((uint32_t)f32_to_bf16(sum[1]) << 16), tag);
        store_tagged(fin + 1, (uint32_t)f32_to_bf16(sum[2]) | ((uint32_t)f32_to_bf16(sum[3]) << 16), tag);
      }
    }
  }

  // ---- the chunk loop
  // T operand of this wave's rank chunk: lane (i, g) needs T[token i][32k +
  // 8g .. +7], held by tile 2k + g/2, lanes i + 16 g' (g' = 2(g % 2), +1).
  const int tj = 2 * wave + (g >> 1);
  const bool t_live = a.r_cat > 0 && wave < n_chunks32 && tj < a.r_tiles;
  const uint64_t* tsrc = a.tfinal + ((size_t)tj * 64 + i + 32 * (g & 1)) * 2;
  u32x4_t tv = zero_u4();
  bool t_have = false;
  f32x4_t acc = zero4();
  const uint32_t below = (1u << (8 * g)) - 1u;

  const auto step = [&](int q, unsigned char* bcur, unsigned char* bnxt, int bsel, const u32x4_t (&xc)[kCSteps],
                        u32x4_t (&xn)[kCSteps]) {
    const int t = t_begin + q / nc, c = q % nc;
    const bool tile_end = c == nc - 1;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of chunk q (and everything before) have landed
    // (LDS-only barriers throughout: __syncthreads would also wait for the
    // next chunk's loads, which must stay in flight across the tile-end and
    // T-piece barriers)
    lds_barrier();
    if (q + 1 < n_q) issue(q + 1, bnxt, bsel ^ 1, xn);

    // decode + multiply this wave's steps of chunk q
    const int col0 = c * kChunk;
    const int ncols = min(kChunk, a.K - col0);
    const int nsteps = (ncols + 31) / 32;
    const int s0 = wave * kCSteps;
    if (s0 < nsteps) {
      const uint64_t* mrow = reinterpret_cast<const uint64_t*>(bcur) + i * kCMaskRow;
      const uint16_t* vals16 = reinterpret_cast<const uint16_t*>(bcur + (size_t)kSRows * kCMaskRow * 8);
      const int w0 = s0 >> 1;
      // every bitmap read is issued before any is used, and the prefix words
      // are pinned in registers: a count that uses its word only under a lane
      // condition is otherwise compiled as a branch around the read and its
      // wait, one LDS round trip per word
      uint64_t pm[kCWords / 4], mw[kCSteps / 2];
#pragma unroll
      for (int k = 0; k < kCWords / 4; ++k) pm[k] = mrow[g + 4 * k];
#pragma unroll
      for (int u = 0; u < kCSteps / 2; ++u) mw[u] = mrow[w0 + u];
      static_assert(kCWords / 4 == 8, "operand list below");
      asm volatile(""
                   : "+v"(pm[0]), "+v"(pm[1]), "+v"(pm[2]), "+v"(pm[3]), "+v"(pm[4]), "+v"(pm[5]), "+v"(pm[6]),
                     "+v"(pm[7]));
      uint32_t part = 0;
#pragma unroll
      for (int k = 0; k < kCWords / 4; ++k) part += g + 4 * k < w0 ? (uint32_t)__popcll(pm[k]) : 0u;
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      uint32_t run = H.vbase[bsel][i] + part;
      // two steps (one bitmap word) per batch: all LDS reads of a batch are
      // issued before any is used
#pragma unroll
      for (int u = 0; u < kCSteps / 2; ++u) {
        Window3 wa[2], wb[2];
        uint32_t ia[2], ib[2];
        u32x2_t la[2], lb[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int s = 2 * u + b;
          const uint32_t h = b ? (uint32_t)(mw[u] >> 32) : (uint32_t)mw[u];
          const uint32_t byte = (s0 + s < nsteps) ? (h >> (8 * g)) & 0xFFu : 0u;
          const uint32_t lo = byte & 15u, hi = byte >> 4;
          ia[b] = run + __popc(h & below);
          ib[b] = ia[b] + __popc(lo);
          wa[b] = lds_window_words(vals16, ia[b]);
          wb[b] = lds_window_words(vals16, ib[b]);
          la[b] = H.lut[lo];
          lb[b] = H.lut[hi];
          run += __popc(h);
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int s = 2 * u + b;
          if (s0 + s < nsteps) {
            const u32x2_t x0 = expand_nibble(window_values(wa[b], ia[b]), la[b]);
            const u32x2_t x1 = expand_nibble(window_values(wb[b], ib[b]), lb[b]);
            acc = mfma_16x16x32(u32x4_t{x0.x, x0.y, x1.x, x1.y}, xc[s], acc);
          }
        }
      }
    }

    if (tile_end) {
      // low-rank chunk of this wave, then the waves' sums (in the values
      // area of the buffer just decoded)
      if (!t_have && a.r_cat > 0) {
        if (wave == 0 && !producer) {
          resolve_tag();
          if (lane == 0) H.tag = tag;
        }
      }
      lds_barrier();
      // (T is read once, at the first tile's end; its loads queue behind the
      // next chunk's, a one-time wait)
      if (!t_have) {
        tag = H.tag;
        if (t_live) {
          uint32_t d0[2], d1[2];
          poll_tagged<2>(tsrc, tag, d0, err);
          poll_tagged<2>(tsrc + 32, tag, d1, err);
          tv = u32x4_t{d0[0], d0[1], d1[0], d1[1]};
        }
        t_have = true;
      }
      if (wave < n_chunks32 && a.r_cat > 0) acc = mfma_16x16x32(bc, tv, acc);
      f32x4_t* const rsum = reinterpret_cast<f32x4_t*>(bcur + (size_t)kSRows * kCMaskRow * 8);
      if (wave > 0) rsum[(wave - 1) * 64 + lane] = acc;
      lds_barrier();
      if (wave == 0) {
#pragma unroll
        for (int w = 0; w < kSWaves - 1; ++w) acc += rsum[w * 64 + lane];
        // lane holds Y^T[row0 + 4g + e][token i]
        if (i < a.M) {
          const int64_t row0 = (int64_t)t * kSRows;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t n = row0 + 4 * g + e;
            const float v = acc[e];
            if (n < a.N) a.Y[(size_t)i * a.N + n] = f32_to_bf16(v);
          }
        }
      }
      acc = zero4();
      if (nc == 1 && q + 1 < n_q) load_bc(t + 1);
    }
  };

  unsigned char* const buf1 = buf0 + bbytes;
  for (int q = 0; q < n_q; q += 2) {
    step(q, buf0, buf1, 0, xf0, xf1);
    if (q + 1 < n_q) step(q + 1, buf1, buf0, 1, xf1, xf0);
  }
}

}  // namespace

size_t fwd_stream_lds_bytes(int vcap) {
  return sizeof(SHead) + 2 * ((size_t)kSRows * kCMaskRow * 8 + (size_t)kSRows * vcap * 16);
}

hipError_t launch_fwd_stream(const StreamFwdArgs& a, hipStream_t s) {
  const int grid = (a.n_tiles + a.tiles_per_wg - 1) / a.tiles_per_wg;
  hipLaunchKernelGGL(fwd_stream_kernel, dim3(grid), dim3(kSThreads), fwd_stream_lds_bytes(a.vcap), s, a);
  return hipGetLastError();
}

}  // namespace salr
