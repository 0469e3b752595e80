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
//   * T = X A_cat is cut into pieces of 16 ranks x (a multiple of 512 or
//     1024) columns.  Extra workgroups at the front of the grid each compute one
//     piece and nothing else, so T is complete long before any weight tile
//     needs it; the last producer of a rank tile sums its pieces in a fixed
//     order.  After its decode every weight workgroup reads T for its share
//     of the ranks and adds T B_cat for those ranks (B_cat rows fetched with
//     the weights) as extra matrix-core steps.  With whole rows a workgroup takes all ranks; with
//     ranges, range r takes the 32-rank chunks r, r + ranges, ..., so the
//     low-rank work and its gather traffic are spread over the ranges;
//   * pieces and range partials handed between workgroups travel as tagged
//     words (see salr_device.hpp), so no cache-wide fence is ever executed.
#include <cstddef>

#include "salr_device.hpp"
#include "salr_kernels.hpp"

namespace salr {
namespace {

constexpr int kThreads = 512;
constexpr int64_t kCus = 256;  // compute units of the GPU
constexpr int kWaves = kThreads / 64;
constexpr int kRows = 16;
constexpr int kMaxSteps = kMaxRangeCols / 32 / kWaves;  // 32-column steps per wave
constexpr int kMaxWaveWords = kMaxSteps / 2;           // bitmap words per wave
// Bitmap words per row in LDS: one word of padding puts the 16 rows' words
// in 16 distinct bank pairs.
constexpr int kMaskRowWords = kMaxRangeCols / 64 + 1;
constexpr int kPrefixReads = (kMaskRowWords - 1) / 4;  // bitmap words per lane for a row's prefix
constexpr int kPollBatch = 8;
constexpr int kBatch = 4;  // decode steps whose LDS reads are issued together
static_assert(kMaxSteps % kBatch == 0, "X operands are requested a batch at a time");

// LDS carve-up (dynamic shared memory): the selector table, the values area
// (at a small constant offset, which the decode's reads take as an immediate
// offset), the rest of the fixed part, then the tile's B_cat rows.
struct alignas(16) LdsHead {
  u32x2_t lut[16];
  u32x4_t zero16;  // sixteen zero bytes (reads outside an operand)
};
struct alignas(16) Lds {
  float levels[16];        // NF4 levels (NF4 layers)
  uint32_t seg[kRows][2];  // per-row range of kept-value indices (within the row)
  int64_t vorg[kRows];     // global value index = LDS value slot + vorg (per row)
  uint64_t masks[kRows * kMaskRowWords];
  uint32_t tag;
};
// T pieces are cut into chunks of piece_cols<kOneRound> columns (see the
// producer section); steps per wave of one chunk:
template <bool kOneRound>
constexpr int piece_cols() { return kOneRound ? 512 : 1024; }
template <bool kOneRound>
constexpr int piece_steps() { return piece_cols<kOneRound>() / 32 / kWaves; }
constexpr int kFinBatch = 8;                      // pieces requested together when finishing T
constexpr int kMaxLoadRows = kRows / kWaves;      // rows per load-issuing wave
static_assert(sizeof(LdsHead) % 16 == 0 && sizeof(Lds) % 16 == 0, "areas must stay 16-byte aligned");
static_assert(offsetof(Lds, masks) % 16 == 0, "bitmap rows must stay 16-byte aligned");

// Decode reads address LDS with plain byte offsets: the dynamic area starts at
// byte 0 (these kernels declare no static LDS; the kernel checks), so the
// constant part of an address folds into the read's immediate offset.
typedef __attribute__((address_space(3))) const uint32_t lds_u32_t;
typedef __attribute__((address_space(3))) const u32x2_t lds_u32x2_t;
constexpr uint32_t kValsOff = sizeof(LdsHead);  // byte offset of the values area
// The 4-value window at value index idx of the values area (see
// lds_window_words) and the selector pair of nibble q.
__device__ __forceinline__ Window3 vals_window(uint32_t idx) {
  lds_u32_t* w = reinterpret_cast<lds_u32_t*>((size_t)(kValsOff + ((idx >> 1) << 2)));
  return Window3{w[0], w[1], w[2]};
}
__device__ __forceinline__ u32x2_t lut_entry(uint32_t q) {
  return *reinterpret_cast<lds_u32x2_t*>((size_t)(offsetof(LdsHead, lut) + (q << 3)));
}

// Make the compiler hold every word in a register here (one wait for all the
// reads before it; see the decode).
__device__ __forceinline__ void pin_words(uint64_t (&p)[kPrefixReads], uint64_t (&m)[kMaxWaveWords]) {
  static_assert(kPrefixReads == 16 && kMaxWaveWords == 8, "operand list below");
  asm volatile(""
               : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]), "+v"(p[4]), "+v"(p[5]), "+v"(p[6]), "+v"(p[7]),
                 "+v"(p[8]), "+v"(p[9]), "+v"(p[10]), "+v"(p[11]), "+v"(p[12]), "+v"(p[13]), "+v"(p[14]),
                 "+v"(p[15]), "+v"(m[0]), "+v"(m[1]), "+v"(m[2]), "+v"(m[3]), "+v"(m[4]), "+v"(m[5]), "+v"(m[6]),
                 "+v"(m[7]));
}

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

// NF4 dequantization pass (kNF4 instances): the row segments' codes and
// scales were loaded to the end of each row's LDS area; 32 threads per row
// each read the codes and scales of up to kNf4Groups groups of 8 values
// (value group g of a row is LDS chunk g of its area, as in the bf16 layout),
// and after a barrier write their bf16 values, level[code] * scale rounded
// in float32, over the same area.
// Whole rows of a multiple of 8 values (one column range): value group g of
// a row is code word g of the row's codes (the codes start on a 16-byte
// boundary) and lies in scale block g / 8, so the indices are plain 32-bit
// offsets.
__device__ __forceinline__ void nf4_dequantize_rows(const SmallFwdArgs& a, const Lds& L, uint32_t* vals,
                                                    int64_t row0, int rows_here, int tid) {
  const int r = tid >> 5, p = tid & 31;
  const int nch = r < rows_here ? a.n_keep >> 3 : 0;
  const uint32_t* cw32 = vals + (size_t)r * a.vcap * 4 + a.cofs * 4;
  const uint16_t* sl = reinterpret_cast<const uint16_t*>(vals + (size_t)r * a.vcap * 4 + a.sofs * 4) +
                       (((row0 + r) * a.nblk) & 7);  // (the scales' copy starts at a 16-byte boundary)
  const int gmax = nch > 0 ? nch - 1 : 0;
  uint32_t cw[kNf4Groups], sc[kNf4Groups];
#pragma unroll
  for (int q = 0; q < kNf4Groups; ++q) {
    const int g = min(p + 32 * q, gmax);  // (clamped, read unconditionally)
    cw[q] = cw32[g];
    sc[q] = sl[g >> 3];
  }
  static_assert(kNf4Groups == 9, "operand list below");
  asm volatile("" : "+v"(cw[0]), "+v"(cw[1]), "+v"(cw[2]), "+v"(cw[3]), "+v"(cw[4]), "+v"(cw[5]), "+v"(cw[6]),
               "+v"(cw[7]), "+v"(cw[8]), "+v"(sc[0]), "+v"(sc[1]), "+v"(sc[2]), "+v"(sc[3]), "+v"(sc[4]),
               "+v"(sc[5]), "+v"(sc[6]), "+v"(sc[7]), "+v"(sc[8]));
  lds_barrier();  // every thread has its codes and scales: the area is free
#pragma unroll
  for (int q = 0; q < kNf4Groups; ++q) {
    const int g = p + 32 * q;
    if (g < nch) {
      const float s = __uint_as_float(sc[q] << 16);
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float f0 = L.levels[(cw[q] >> (4 * e)) & 15u] * s;
        const float f1 = L.levels[(cw[q] >> (4 * e + 4)) & 15u] * s;
        w[e / 2] = (uint32_t)f32_to_bf16(f0) | ((uint32_t)f32_to_bf16(f1) << 16);
      }
      reinterpret_cast<u32x4_t*>(vals)[(size_t)r * a.vcap + g] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
  }
}

__device__ __forceinline__ void nf4_dequantize(const SmallFwdArgs& a, const Lds& L, uint32_t* vals, int64_t row0,
                                               int rows_here, int tid) {
  if (a.splits == 1 && (a.n_keep & 7) == 0) {
    nf4_dequantize_rows(a, L, vals, row0, rows_here, tid);
    return;
  }
  const int r = tid >> 5, p = tid & 31;
  const uint32_t lo = L.seg[r][0], hi = L.seg[r][1];
  const bool live = r < rows_here && hi > lo;
  const int64_t rowv = (row0 + r) * a.n_keep;  // global index of the row's value 0
  const int64_t q0 = (rowv + lo) >> 3;          // first 8-value group (global)
  const int nch = live ? (int)(((rowv + hi + 7) >> 3) - q0) : 0;
  const int64_t cbyte0 = (((row0 + r) * a.cb_row + (lo >> 1)) >> 4) * 16;              // first loaded code byte
  const int64_t sbyte0 = ((((row0 + r) * a.nblk + (lo >> 6)) * 2) >> 4) * 16;         // first loaded scale byte
  const unsigned char* cl = reinterpret_cast<const unsigned char*>(vals + ((size_t)r * a.vcap + a.cofs) * 4);
  const unsigned char* sl = reinterpret_cast<const unsigned char*>(vals + ((size_t)r * a.vcap + a.sofs) * 4);
  const int64_t blo = lo >> 6, bhi = hi > 0 ? (int64_t)(hi - 1) >> 6 : 0;
  uint32_t cw[kNf4Groups];
  uint32_t sc[kNf4Groups];  // the two bf16 scales of the group (first | second << 16)
  // values of a group from this index on take the second scale
  const auto split_of = [&](int64_t j0) {
    int64_t b0 = (j0 > (int64_t)lo ? j0 : (int64_t)lo) >> 6, b1 = (j0 + 7) >> 6;
    b0 = b0 < blo ? blo : (b0 > bhi ? bhi : b0);
    b1 = b1 < blo ? blo : (b1 > bhi ? bhi : b1);
    return b1 != b0 ? (int)(64 * b1 - j0) : 8;
  };
#pragma unroll
  for (int q = 0; q < kNf4Groups; ++q) {
    const int g = p + 32 * q;
    cw[q] = 0u;
    sc[q] = 0u;
    if (g < nch) {
      // the group's 8 codes from row-local value j0 on (values before the
      // segment, never selected, read as code 0)
      const int64_t j0 = (q0 + g) * 8 - rowv;
      const int64_t jc = j0 > (int64_t)(lo & ~1u) ? j0 : (int64_t)(lo & ~1u);
      const int64_t byte = (row0 + r) * a.cb_row + (jc >> 1) - cbyte0;
      const uint32_t* w = reinterpret_cast<const uint32_t*>(cl + (byte & ~3ll));
      const uint32_t c = __builtin_amdgcn_alignbit(w[1], w[0], (uint32_t)((byte & 3) * 8 + (jc & 1) * 4));
      cw[q] = c << (4 * (uint32_t)(jc - j0));
      // scales of the group's first and last value (clamped to the segment)
      int64_t b0 = (j0 > (int64_t)lo ? j0 : (int64_t)lo) >> 6;
      int64_t b1 = (j0 + 7) >> 6;
      b0 = b0 < blo ? blo : (b0 > bhi ? bhi : b0);
      b1 = b1 < blo ? blo : (b1 > bhi ? bhi : b1);
      const uint16_t* sp = reinterpret_cast<const uint16_t*>(sl);
      sc[q] = (uint32_t)sp[((row0 + r) * a.nblk + b0) - sbyte0 / 2] |
              ((uint32_t)sp[((row0 + r) * a.nblk + b1) - sbyte0 / 2] << 16);
    }
  }
  lds_barrier();  // every thread has its codes and scales: the area is free
#pragma unroll
  for (int q = 0; q < kNf4Groups; ++q) {
    const int g = p + 32 * q;
    if (g < nch) {
      const int split = split_of((q0 + g) * 8 - rowv);
      const float s0 = __uint_as_float(sc[q] << 16), s1 = __uint_as_float(sc[q] & 0xFFFF0000u);
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float f0 = L.levels[(cw[q] >> (4 * e)) & 15u] * (e < split ? s0 : s1);
        const float f1 = L.levels[(cw[q] >> (4 * e + 4)) & 15u] * (e + 1 < split ? s0 : s1);
        w[e / 2] = (uint32_t)f32_to_bf16(f0) | ((uint32_t)f32_to_bf16(f1) << 16);
      }
      reinterpret_cast<u32x4_t*>(vals)[(size_t)r * a.vcap + g] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
  }
}

// kOneRound: every weight workgroup is resident at once, so the T producers
// sit on CUs beside some of them (see the producer section).
// kWin: a fused layer's parts bound each row tile's adapter ranks (a.nparts
// > 0); the plain instance keeps the whole-r_cat code.
// kNF4: the kept values are NF4 codes (QSALR), dequantized in LDS.
template <bool kOneRound, bool kWin, bool kNF4>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void fwd_small_kernel(SmallFwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  LdsHead& H = *reinterpret_cast<LdsHead*>(smem);
  uint32_t* const vals = reinterpret_cast<uint32_t*>(smem + sizeof(LdsHead));
  Lds& L = *reinterpret_cast<Lds*>(smem + sizeof(LdsHead) + a.vals_bytes);
  f32x4_t* const red = reinterpret_cast<f32x4_t*>(vals);
  // After the fixed part: the tile's B_cat rows [16][r_cat].
  uint16_t* const bl = reinterpret_cast<uint16_t*>(smem + sizeof(LdsHead) + a.vals_bytes + sizeof(Lds));

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  // (the decode's reads assume the dynamic area at LDS byte 0)
  if ((uint32_t)(size_t)(__attribute__((address_space(3))) unsigned char*)smem != 0u) {
    if (tid == 0) store_coherent(a.err, 2u);
    return;
  }
  const int i = lane & 15, g = lane >> 4;
  const uint32_t n_wgs = gridDim.x;
  const bool talk = a.splits > 1 || a.r_cat > 0;  // any cross-workgroup data?
  uint32_t* const err = a.err;
  // This launch's tag: a ticket drawn by thread 0 and resolved by wave 0
  // where first needed (producers: first thing; weight workgroups: after
  // their decode).
  uint64_t drawn = 0;
  uint32_t tag = 0;
  const auto resolve_tag = [&]() {
    uint32_t t = 0;
    if (lane == 0) t = tag_from_ticket(a.tickets, drawn, blockIdx.x, n_wgs);
    tag = __shfl(t, 0);
  };
  f32x4_t acc = zero4();

  // ---------------- this workgroup's role: the first n_pieces workgroups
  // compute T pieces and nothing else; the rest own 16 W rows x one column
  // range
  const int n_pieces = a.r_tiles * a.t_pieces;
  const bool producer = (int)blockIdx.x < n_pieces;
  const int c = producer ? (int)blockIdx.x : (int)blockIdx.x - n_pieces;
  const int tile = c / a.splits, rng = c % a.splits;
  const int64_t row0 = (int64_t)tile * kRows;
  const int col0 = rng * a.range;
  const int ncols = min(a.range, a.K - col0);
  // This tile's adapter ranks [rlo, rlo + rn): all of them, or in a fused
  // layer the block of the part that owns the tile (B_cat is zero outside
  // it); its B_cat rows sit in LDS with row stride bstride.
  int rlo = 0, rn = a.r_cat;
  if (kWin)
    for (int p = 0; p < a.nparts; ++p)
      if (tile < a.part_tile_end[p]) {
        rlo = a.part_rank0[p];
        rn = a.part_nrank[p];
        break;
      }
  const int bstride = kWin ? rn : a.r_cat;
  const int nsteps = (ncols + 31) / 32;
  // steps per wave, even so that every wave starts on a bitmap word (<= kMaxSteps)
  const int spw = 2 * ((nsteps + 2 * kWaves - 1) / (2 * kWaves));
  const int s0 = wave * spw;
  const int nwords = (ncols + 63) / 64;            // bitmap words in the range
  const int rows_here = (int)min<int64_t>(kRows, a.N - row0);

  // X operands of this wave's steps: those of the first decode batch are
  // requested right after the weights, each later batch's at the start of the
  // batch before it (so X is not in the way of the weight stream, and only
  // two batches of it are held in registers).
  u32x4_t xf[kMaxSteps];
  const auto load_x_batch = [&](int q0) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int q = q0 + b;
      xf[q] = (q < spw) ? load_x_frag(a.X, a.M, a.K, i, col0 + 32 * (s0 + q) + 8 * g) : zero_u4();
    }
  };

  if (!producer) {
    // (beside a T producer, this workgroup's waves take every issue slot
    // first)
    if (kOneRound) __builtin_amdgcn_s_setprio(3);
    if (tid < 16) H.lut[tid] = nibble_selectors(tid);
    if (tid == 16) H.zero16 = zero_u4();
    if (kNF4 && tid >= 64 && tid < 80) L.levels[tid - 64] = a.levels[tid - 64];
    const int lw = wave, lws = kWaves;
    // Bitmap words of the range, per row 2*nwords dwords direct to LDS; rows
    // past N read as zero.
    for (int r = lw; r < kRows; r += lws) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(&L.masks[r * kMaskRowWords]);
      if (r < rows_here) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(a.masks + (row0 + r) * a.kw + (col0 >> 6));
        for (int b = 0; b * 64 < 2 * nwords; ++b)
          if (b * 64 + lane < 2 * nwords) __builtin_amdgcn_global_load_lds(src + b * 64 + lane, dst + b * 64, 4, 0, 0);
      } else {
        for (int w = lane; w < 2 * kMaskRowWords; w += 64) dst[w] = 0u;
      }
    }
    // Values: row r's kept values [lo, hi) (indices within the row) go to
    // the row's own LDS area (vcap chunks, a stride that starts row areas in
    // different banks).  Whole rows need nothing read first; a range reads
    // its bounds from the per-row lookup table (entries every 1024 columns).
    uint32_t seg_lo[kMaxLoadRows], seg_hi[kMaxLoadRows];
#pragma unroll
    for (int k = 0; k < kMaxLoadRows; ++k) {
      const int r = lw + k * lws;
      uint32_t lo = 0, hi = (uint32_t)a.n_keep;
      if (a.splits > 1 && r < rows_here) {
        const uint32_t* orow = a.offsets + (row0 + r) * a.ng;
        const int g0 = col0 >> 10, g1 = (col0 + ncols + 1023) >> 10;
        hi = min(g1 < a.ng ? orow[g1] : (uint32_t)a.n_keep, (uint32_t)a.n_keep);
        lo = min(orow[g0], hi);
        lo = max(lo, hi > (uint32_t)a.range ? hi - (uint32_t)a.range : 0u);  // inside the row's LDS area
      }
      seg_lo[k] = lo;
      seg_hi[k] = hi;
    }
#pragma unroll
    for (int k = 0; k < kMaxLoadRows; ++k) {
      const int r = lw + k * lws;
      if (r < kRows) {
        const int64_t va = (row0 + r) * a.n_keep + seg_lo[k], vb = (row0 + r) * a.n_keep + seg_hi[k];
        const int64_t q0 = va >> 3, nch = (r < rows_here && vb > va) ? ((vb + 7) >> 3) - q0 : 0;
        if (kNF4) {
          // the segment's codes (+ 8 bytes for the last group's window) and
          // the scales of its blocks, to the end of the row's area
          const bool seg_live = r < rows_here && seg_hi[k] > seg_lo[k];
          const int64_t cb0 = (row0 + r) * a.cb_row + (seg_lo[k] >> 1);
          const int64_t cb1 = (row0 + r) * a.cb_row + ((seg_hi[k] + 1) >> 1) + 8;
          const int64_t ncc = seg_live ? ((cb1 + 15) >> 4) - (cb0 >> 4) : 0;
          copy_chunks_to_lds(reinterpret_cast<const uint32_t*>(a.codes) + (cb0 >> 4) * 4,
                             vals + ((size_t)r * a.vcap + a.cofs) * 4, ncc, 0, 1, lane);
          const int64_t sb0 = ((row0 + r) * a.nblk + (seg_lo[k] >> 6)) * 2;
          const int64_t sb1 = ((row0 + r) * a.nblk + (seg_live ? ((seg_hi[k] - 1) >> 6) + 1 : 0)) * 2;
          const int64_t nsc = seg_live ? ((sb1 + 15) >> 4) - (sb0 >> 4) : 0;
          copy_chunks_to_lds(reinterpret_cast<const uint32_t*>(a.scales) + (sb0 >> 4) * 4,
                             vals + ((size_t)r * a.vcap + a.sofs) * 4, nsc, 0, 1, lane);
        } else {
          copy_chunks_to_lds(reinterpret_cast<const uint32_t*>(a.values) + q0 * 4, vals + (size_t)r * a.vcap * 4,
                             nch, 0, 1, lane);
        }
        if (lane == 0) {
          L.vorg[r] = q0 * 8 - (int64_t)r * a.vcap * 8;
          L.seg[r][0] = seg_lo[k];
          L.seg[r][1] = seg_hi[k];
        }
      }
    }
    // This tile's B_cat rows (in a fused layer only its part's ranks, 16-byte
    // chunks: every part's rank count and offset is a multiple of 8).
    if (kWin) {
      const int cpr = rn / 8;
      const int nch = rows_here * cpr;
      const uint32_t* src0 = reinterpret_cast<const uint32_t*>(a.b_cat + row0 * a.r_cat + rlo);
      for (int b = lw; b * 64 < nch; b += lws) {
        const int cc = b * 64 + lane;
        if (cc < nch) {
          const int r = cc / cpr, q = cc - r * cpr;
          __builtin_amdgcn_global_load_lds(src0 + ((size_t)r * a.r_cat + 8 * q) / 2,
                                           reinterpret_cast<uint32_t*>(bl) + b * 256, 16, 0, 0);
        }
      }
    } else if (a.r_cat > 0) {
      const int64_t bbytes = (int64_t)rows_here * a.r_cat * 2;
      copy_chunks_to_lds(reinterpret_cast<const uint32_t*>(a.b_cat + row0 * a.r_cat), reinterpret_cast<uint32_t*>(bl),
                         (bbytes + 15) / 16, lw, lws, lane);
    }
  }

  // (the first batch's X after the weights: it comes from L2, the weights
  // from HBM)
  if (!producer) load_x_batch(0);

  // ---------------- T pieces (producer workgroups)
  // Piece p = (rank tile j, K range kp) is T^T[16 ranks][16 tokens] summed
  // over t_chunks chunks of piece_cols columns (512 when every weight
  // workgroup is resident at once: smaller pieces, spread over more
  // producers, hold up the weight loads of the CUs they share less; 1024
  // otherwise); producer workgroup p computes piece p with
  // all its waves (partials summed in LDS in wave order).  Wave 0 publishes
  // it as tagged words (lane (i, g) holds ranks 16j + 4g + e of token i) and
  // counts it; the producer that completes a rank tile's count sums the
  // tile's pieces in K order and publishes T for the tile as bf16 pairs.
  // Producers wait on nothing but each other's pieces, which are published
  // before any wait, and carry no weights, so T is ready early and no weight
  // tile is held up by it.
  if (producer) {
    if (tid == 0) drawn = draw_ticket(a.tickets, blockIdx.x, n_wgs);
    const int piece = c;
    const int j = piece / a.t_pieces, kp = piece % a.t_pieces;
    const int rank = 16 * j + i;
    f32x4_t t = zero4();
    for (int ch = 0; ch < a.t_chunks; ++ch) {
      constexpr int kPS = piece_steps<kOneRound>();
      u32x4_t pav[kPS], pxv[kPS];
#pragma unroll
      for (int q = 0; q < kPS; ++q) {
        const int col = (kp * a.t_chunks + ch) * piece_cols<kOneRound>() + 32 * (wave * kPS + q) + 8 * g;
        pav[q] = (rank < a.r_cat && col < a.K) ? load16(a.a_cat + (size_t)rank * a.K + col) : zero_u4();
        pxv[q] = load_x_frag(a.X, a.M, a.K, i, col);
      }
#pragma unroll
      for (int q = 0; q < kPS; ++q) t = mfma_16x16x32(pav[q], pxv[q], t);
    }
    if (!reduce_waves(t, red, wave, lane)) return;
    resolve_tag();
    uint64_t* dst = a.tpiece + ((size_t)piece * 64 + lane) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = t[e];  // (scalar copy first: see reduce_parts)
      store_tagged(dst + e, __float_as_uint(v), tag);
    }
    uint32_t old = 0;
    if (lane == 0) old = atomic_add_relaxed(&a.tcount[j], 1u);
    old = __shfl(old, 0);
    if (old != (uint32_t)(a.t_pieces - 1)) return;
    if (lane == 0) store_coherent(&a.tcount[j], 0u);
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
    for (int kp0 = 0; kp0 < a.t_pieces; kp0 += kFinBatch) {
      uint64_t v[kFinBatch][4];
#pragma unroll
      for (int b = 0; b < kFinBatch; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[b][e] = (kp0 + b < a.t_pieces)
                        ? load_tagged_raw(a.tpiece + ((size_t)(j * a.t_pieces + kp0 + b) * 64 + lane) * 4 + e)
                        : 0ull;
#pragma unroll
      for (int b = 0; b < kFinBatch; ++b) {
        if (kp0 + b < a.t_pieces) {
          bool ok = true;
#pragma unroll
          for (int e = 0; e < 4; ++e) ok &= (uint32_t)(v[b][e] >> 32) == tag;
          uint32_t w[4];
          if (ok) {
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (uint32_t)v[b][e];
          } else {
            poll_tagged<4>(a.tpiece + ((size_t)(j * a.t_pieces + kp0 + b) * 64 + lane) * 4, tag, w, err);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) sum[e] += __uint_as_float(w[e]);
        }
      }
    }
    uint64_t* fin = a.tfinal + ((size_t)j * 64 + lane) * 2;
    store_tagged(fin, (uint32_t)f32_to_bf16(sum[0]) | ((uint32_t)f32_to_bf16(sum[1]) << 16), tag);
    store_tagged(fin + 1, (uint32_t)f32_to_bf16(sum[2]) | ((uint32_t)f32_to_bf16(sum[3]) << 16), tag);
    return;
  }

  __builtin_amdgcn_s_waitcnt(0);  // every load of this wave has landed
  lds_barrier();
  if (kNF4) {
    nf4_dequantize(a, L, vals, row0, rows_here, tid);
    lds_barrier();
  }

  // This workgroup's share of the low-rank term: the 32-rank chunks rng,
  // rng + splits, ...; wave k reads chunk k's T operand after the decode.
  // Lane (i, g) needs T[token i][32q + 8g .. +7]: tile 2q + g/2, i.e. the
  // words of lanes i + 16 g' (g' = 2(g % 2), +1) there.
  // 32-rank chunks of [rlo, rlo + rn)
  const int clo = kWin ? rlo / 32 : 0, n_chunks = kWin ? (rlo + rn + 31) / 32 - clo : a.r_pad / 32;
  const int n_own = rn > 0 && rng < n_chunks ? (n_chunks - rng + a.splits - 1) / a.splits : 0;
  const int my_chunk = clo + rng + wave * a.splits;
  const int tj = 2 * my_chunk + (g >> 1);
  const bool t_live = wave < n_own && tj < a.r_tiles;
  const uint64_t* tsrc = a.tfinal + ((size_t)tj * 64 + i + 32 * (g & 1)) * 2;

  // Decode + multiply this wave's steps.  The wave's bitmap words come to
  // registers first; then each batch of kBatch steps issues all its LDS
  // reads (two value windows and two selector words per step) before any of
  // them is used.
  {
    const bool live = i < rows_here;
    const uint64_t* mrow = &L.masks[i * kMaskRowWords];
    // LDS slot of the row's first value in the range, plus the kept bits of
    // the range before this wave's first word
    const uint32_t base = live ? (uint32_t)((row0 + i) * a.n_keep + L.seg[i][0] - L.vorg[i]) : 0u;
    const int w0 = s0 >> 1;
    // Every bitmap read of the prefix and of this wave's words is issued
    // before any is used (clamped in-row indices), and the words are then
    // pinned in registers: a count that uses its word only under a lane
    // condition is otherwise compiled as a branch around the read and its
    // wait, one LDS round trip per word.
    uint64_t pm[kPrefixReads], mw[kMaxWaveWords];
#pragma unroll
    for (int k = 0; k < kPrefixReads; ++k) pm[k] = mrow[min(g + 4 * k, kMaskRowWords - 1)];
#pragma unroll
    for (int q = 0; q < kMaxWaveWords; ++q) mw[q] = mrow[min(w0 + q, kMaskRowWords - 1)];
    pin_words(pm, mw);
    uint32_t part = 0;
#pragma unroll
    for (int k = 0; k < kPrefixReads; ++k) part += g + 4 * k < w0 ? (uint32_t)__popcll(pm[k]) : 0u;
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
#pragma unroll
    for (int q = 0; q < kMaxWaveWords; ++q) mw[q] = (2 * q < spw && w0 + q < nwords) ? mw[q] : 0ull;
    uint32_t run = base + part;
    const uint32_t below = (1u << (8 * g)) - 1u;
#pragma unroll
    for (int q0 = 0; q0 < kMaxSteps; q0 += kBatch) {
      if (q0 + kBatch < kMaxSteps) load_x_batch(q0 + kBatch);
      if (q0 < spw && s0 + q0 < nsteps) {
        Window3 wa[kBatch], wb[kBatch];
        uint32_t ia[kBatch], ib[kBatch];
        u32x2_t la[kBatch], lb[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const int q = q0 + b;
          // (no step guard: a word outside the wave's range was zeroed above,
          // and a bitmap word has no bits past K or past a column range)
          const uint32_t h = (q & 1) ? (uint32_t)(mw[q >> 1] >> 32) : (uint32_t)mw[q >> 1];
          const uint32_t byte = (h >> (8 * g)) & 0xFFu;
          const uint32_t lo = byte & 15u, hi = byte >> 4;
          ia[b] = run + __popc(h & below);
          ib[b] = ia[b] + __popc(lo);
          wa[b] = vals_window(ia[b]);
          wb[b] = vals_window(ib[b]);
          la[b] = lut_entry(lo);
          lb[b] = lut_entry(hi);
          run += __popc(h);
        }
        // (a step past the wave's range multiplies zeros: its byte is 0,
        // which selects no value)
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const u32x2_t x0 = expand_nibble(window_values(wa[b], ia[b]), la[b]);
          const u32x2_t x1 = expand_nibble(window_values(wb[b], ib[b]), lb[b]);
          acc = mfma_16x16x32(u32x4_t{x0.x, x0.y, x1.x, x1.y}, xf[q0 + b], acc);
        }
      }
    }
  }

  // The launch tag, then the T operand of this wave's chunk.  Both are
  // requested only now: a load in flight holds up every later wait of its
  // wave (the weights must not wait for the ticket), and T is published
  // about when the decodes end.  The first barrier also ends every wave's
  // reads of the values area, which the wave sums then reuse.
  if (talk && tid == 0) drawn = draw_ticket(a.tickets, blockIdx.x, n_wgs);
  uint64_t tw[4] = {0ull, 0ull, 0ull, 0ull};
  if (t_live) {
    tw[0] = load_tagged_raw(tsrc);
    tw[1] = load_tagged_raw(tsrc + 1);
    tw[2] = load_tagged_raw(tsrc + 32);
    tw[3] = load_tagged_raw(tsrc + 33);
  }
  if (talk && wave == 0) {
    resolve_tag();
    if (lane == 0) L.tag = tag;
  }
  // B_cat operand of this wave's chunk (read before the barrier; a read
  // outside the tile's ranks or rows is pointed at the zero chunk)
  u32x4_t wv = zero_u4();
  if (wave < n_own) {
    const int rb = 32 * my_chunk + 8 * g;
    if (kWin) {
      // eight ranks in one aligned 16-byte read (ranks outside the tile's
      // block: zero)
      const int rr = rb - rlo;
      wv = *(i < rows_here && rr >= 0 && rr < rn ? reinterpret_cast<const u32x4_t*>(bl + i * bstride + rr)
                                                  : &H.zero16);
    } else if (a.r_cat % 8 == 0) {
      // eight ranks in one aligned 16-byte read (ranks past r_cat: zero)
      wv = *(i < rows_here && rb < a.r_cat ? reinterpret_cast<const u32x4_t*>(bl + i * a.r_cat + rb) : &H.zero16);
    } else {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ra = rb + 2 * e;
        const uint16_t* zh = reinterpret_cast<const uint16_t*>(&H.zero16);
        const uint32_t lo = *(i < rows_here && ra < a.r_cat ? bl + i * a.r_cat + ra : zh);
        const uint32_t hi = *(i < rows_here && ra + 1 < a.r_cat ? bl + i * a.r_cat + ra + 1 : zh);
        w[e] = lo | (hi << 16);
      }
      wv = u32x4_t{w[0], w[1], w[2], w[3]};
    }
  }
  lds_barrier();
  if (talk) tag = L.tag;
  // Low-rank term of this wave's chunk, in its own accumulator:
  // acc += B_cat^T[rows, chunk] T^T[chunk, :] as one more K step (T already
  // rounded to bf16); the waves' sums below then carry it.
  if (wave < n_own) {
    uint32_t d[4] = {0u, 0u, 0u, 0u};
    if (t_live) {
      bool ok = true;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d[e] = (uint32_t)tw[e];
        ok &= (uint32_t)(tw[e] >> 32) == tag;
      }
      if (!ok) {
        uint32_t d0[2], d1[2];
        poll_tagged<2>(tsrc, tag, d0, err);
        poll_tagged<2>(tsrc + 32, tag, d1, err);
        d[0] = d0[0], d[1] = d0[1], d[2] = d1[0], d[3] = d1[1];
      }
    }
    acc = mfma_16x16x32(wv, u32x4_t{d[0], d[1], d[2], d[3]}, acc);
  }
  // sum the waves' accumulators into wave 0 (fixed order)
  if (wave > 0) red[(wave - 1) * 64 + lane] = acc;
  lds_barrier();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w) acc += red[w * 64 + lane];
  if (a.splits > 1) {
    if (!reduce_parts(acc, a.ypart + (size_t)tile * a.splits * 256, a.splits, rng, &a.ycount[tile], tag, err,
                      lane))
      return;
  }

  // lane holds Y^T[row0 + 4g + e][token i]: four consecutive outputs of
  // token i, one 8-byte store when they are aligned and inside the layer
  if (i < a.M) {
    const int64_t n0 = row0 + 4 * g;
    uint16_t* yp = a.Y + (size_t)i * a.N + n0;
    if (n0 + 3 < a.N && (reinterpret_cast<uintptr_t>(yp) & 7) == 0) {
      const float v0 = acc[0], v1 = acc[1], v2 = acc[2], v3 = acc[3];  // (scalar copies: see reduce_parts)
      *reinterpret_cast<u32x2_t*>(yp) = u32x2_t{(uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16),
                                                (uint32_t)f32_to_bf16(v2) | ((uint32_t)f32_to_bf16(v3) << 16)};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n0 + e < a.N) yp[e] = f32_to_bf16(acc[e]);
    }
  }
}

}  // namespace

size_t fwd_small_vals_bytes(int vcap) {
  const size_t vals = (size_t)kRows * vcap * 16;
  const size_t red = (size_t)(kWaves - 1) * 64 * 16;
  return ((vals > red ? vals : red) + 15) / 16 * 16;
}

size_t fwd_small_lds_bytes(int vcap, int bl_bytes) {
  return sizeof(LdsHead) + fwd_small_vals_bytes(vcap) + sizeof(Lds) + (size_t)bl_bytes;
}

template <bool kNF4>
void launch_small(const SmallFwdArgs& a, int grid, size_t lds, bool one_round, hipStream_t s) {
  if (a.nparts > 0) {
    if (one_round)
      hipLaunchKernelGGL((fwd_small_kernel<true, true, kNF4>), dim3(grid), dim3(kThreads), lds, s, a);
    else
      hipLaunchKernelGGL((fwd_small_kernel<false, true, kNF4>), dim3(grid), dim3(kThreads), lds, s, a);
  } else if (one_round) {
    hipLaunchKernelGGL((fwd_small_kernel<true, false, kNF4>), dim3(grid), dim3(kThreads), lds, s, a);
  } else {
    hipLaunchKernelGGL((fwd_small_kernel<false, false, kNF4>), dim3(grid), dim3(kThreads), lds, s, a);
  }
}

hipError_t launch_fwd_small(const SmallFwdArgs& a, hipStream_t s) {
  const int grid = a.n_tiles * a.splits + a.r_tiles * a.t_pieces;
  // (r_cat <= 256: at most 8 rank chunks, one per wave)
  if (a.tl_bytes > 8 * 1024) return hipErrorInvalidValue;
  const size_t lds = fwd_small_lds_bytes(a.vcap, a.bl_bytes);
  // one weight workgroup per CU at most: all resident in one round
  const bool one_round = (int64_t)a.n_tiles * a.splits <= kCus;
  if (a.nf4) {
    SmallFwdArgs b = a;
    nf4_levels(b.levels);
    launch_small<true>(b, grid, lds, one_round, s);
  } else {
    launch_small<false>(a, grid, lds, one_round, s);
  }
  return hipGetLastError();
}

}  // namespace salr
