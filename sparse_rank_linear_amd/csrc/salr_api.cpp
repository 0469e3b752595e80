// C ABI of the SALR library: argument validation, workspace layout and
// kernel dispatch.  See include/salr.h for the contract of every entry point.
#include "salr.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "salr_encode.hpp"
#include "salr_kernels.hpp"

namespace {

using salr::LargeFwdArgs;
using salr::LowRankTArgs;
using salr::SmallFwdArgs;
using salr::StreamFwdArgs;

constexpr int64_t kMaxK = int64_t(1) << 20;
constexpr int64_t kMaxNK = int64_t(1) << 40;
constexpr int32_t kMaxRank = 256;
constexpr int64_t kSmallM = 16;      // M <= kSmallM takes the fused few-row kernel
constexpr size_t kSmallLdsBudget = 150 * 1024;  // one few-row workgroup per CU
constexpr int64_t kFillWgs = 256;               // few-row consumers wanted to fill the GPU
constexpr size_t kValuesPad = 256;   // tail bytes kernels may over-read
constexpr int32_t kDefaultOversample = 32;
constexpr int32_t kMaxOversample = 64;
constexpr int32_t kDefaultIters = 24;
constexpr int32_t kMaxIters = 1000;

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte layout of the forward workspace.  A fixed-size counter header comes
// first, at the same offsets for every layer shape and every M, so one
// workspace can serve many layers; every completed call leaves all counters
// at zero.  Scratch regions follow and are written before they are read.
constexpr size_t kCounterSync = 0;                       // [8, 12): the error word
constexpr size_t kCounterT = 16;                         // 16 words (few-row T rank tiles)
constexpr size_t kCounterM = kCounterT + 16 * 4;         // 256 words (T token blocks)
constexpr size_t kCounterY = kCounterM + 256 * 4;        // 65536 words (row tiles)
constexpr int64_t kMaxRowTiles = 65536;
constexpr size_t kCounterTickets = 384 * 1024;             // launch-tag ticket words
constexpr size_t kHeaderBytes = 512 * 1024;
static_assert(kCounterY + kMaxRowTiles * 4 <= kCounterTickets, "counter header overflow");
static_assert(kCounterTickets + salr::kTicketGroups * salr::kTicketStride * 8 <= kHeaderBytes, "counter header overflow");

bool dims_ok(int64_t N, int64_t K, int32_t n_keep, int32_t r_cat) {
  if (N < 1 || K < 1 || K > kMaxK || (K % 8) != 0) return false;
  if (N > kMaxNK / K || N > kMaxRowTiles * 16) return false;
  if (n_keep < 0 || n_keep > K) return false;
  if (r_cat < 0 || r_cat > kMaxRank) return false;
  return true;
}

// Large-path K-split count of the T = X A_cat kernel for M rows.
int t_splits_large(int64_t M, int64_t K) {
  const int64_t mblocks = cdiv(M, 64);
  const int64_t nk = cdiv(K, 64);
  // splits only while mblocks * splits <= 256 (bounded partial buffer and
  // counter block), and each at least 4 tiles of 64 columns: the forward
  // kernel sums the splits for every T element it reads
  int64_t s = std::max<int64_t>(1, 256 / mblocks);
  return (int)std::min<int64_t>(s, std::max<int64_t>(1, nk / 4));
}

struct FwdLayout {
  // few-row path
  int n_tiles, splits, range, vcap, r_tiles, r_pad_small, t_pieces, t_chunks;
  int vals_bytes, tl_bytes, bl_bytes;
  // few-row streaming path (layers with more than one round of 16-row work)
  bool stream;
  int tiles_per_wg, svcap;
  // many-row path
  int64_t m_max;
  int r_pad_large;
  // offsets (bytes)
  size_t tsum, tfinal, ypart, T, ltpart, ylarge, total;
};

// r_win: the most adapter ranks one row tile multiplies (r_cat, or a fused
// layer's largest part block); it sizes the few-row B_cat rows in LDS.
FwdLayout fwd_layout(int64_t N, int64_t K, int32_t n_keep, int32_t r_cat, int64_t M_max, int32_t r_win = -1) {
  if (r_win < 0) r_win = r_cat;
  FwdLayout L{};
  L.n_tiles = (int)cdiv(N, 16);
  L.r_tiles = (int)cdiv(r_cat, 16);
  L.r_pad_small = (int)align_up((size_t)std::max(L.r_tiles, 1) * 16, 32);
  L.tl_bytes = r_cat > 0 ? (L.r_pad_small / 32) * 1024 : 0;
  L.bl_bytes = r_win > 0 ? (int)align_up((size_t)16 * r_win * 2, 16) : 0;
  // Few-row column ranges: whole rows when they fit (no lookup-table round
  // trip), else the widest range that fits; narrower ranges while there are
  // too few workgroups to occupy the GPU.
  // (whole rows start on a chunk when n_keep is a multiple of 8)
  const auto vcap_for = [&](int64_t range) {
    return salr::fwd_small_vcap(std::min<int64_t>(range, n_keep), range >= K && n_keep % 8 == 0);
  };
  const auto lds_for = [&](int64_t range) { return salr::fwd_small_lds_bytes(vcap_for(range), L.bl_bytes); };
  L.range = 0;
  if (K <= salr::kMaxRangeCols && lds_for(K) <= kSmallLdsBudget && (L.n_tiles >= kFillWgs || K <= 1024)) {
    L.range = (int)K;
  } else {
    for (int range = salr::kMaxRangeCols; range >= 1024; range /= 2) {
      if (lds_for(range) > kSmallLdsBudget) continue;
      L.range = range;
      if ((int64_t)L.n_tiles * cdiv(K, range) >= kFillWgs) break;
    }
    if (L.range == 0) L.range = 1024;
    if (L.range >= K) L.range = (int)K;
  }
  L.splits = (int)cdiv(K, L.range);
  L.vcap = vcap_for(L.range);
  L.vals_bytes = (int)salr::fwd_small_vals_bytes(L.vcap);
  // Few-row T pieces: 16 ranks x t_chunks 1024-column chunks, at most 8
  // pieces per rank tile (bounds the work of the workgroup that sums them);
  // workgroups take more than one piece only when there are fewer
  // workgroups than pieces.
  {
    const int64_t chunks = cdiv(K, 1024);
    L.t_chunks = (int)cdiv(chunks, 8);
    L.t_pieces = (int)cdiv(chunks, L.t_chunks);
  }
  // More 16-row work than one round of workgroups, with rows cut into
  // column ranges: persistent streaming workgroups, one per CU, each with a
  // run of whole row tiles (needs every T piece to have a workgroup and at
  // most 64 lookup entries per row).  Whole-row layers keep the one-round
  // kernel in several rounds: two of its workgroups per CU have both tiles'
  // loads in flight at once, more than the streaming kernel's one chunk.
  // So do layers whose tile runs would leave more than 15% of the CUs idle
  // (the streaming kernel does not split a tile's K).
  {
    L.tiles_per_wg = (int)cdiv(L.n_tiles, kFillWgs);
    const int64_t n_wg = cdiv(L.n_tiles, L.tiles_per_wg);
    L.svcap = std::max(salr::fwd_small_vcap(std::min<int64_t>(salr::kChunk, n_keep), false), 65);
    const bool fills = (int64_t)L.n_tiles * 100 >= (int64_t)L.tiles_per_wg * kFillWgs * 85;
    L.stream = L.splits > 1 && fills && (int64_t)L.n_tiles * L.splits > kFillWgs && cdiv(K, 1024) <= 64 &&
               (int64_t)L.r_tiles * L.t_pieces <= n_wg && salr::fwd_stream_lds_bytes(L.svcap) <= 160 * 1024;
  }
  // The one-round few-row kernel (every weight workgroup resident at once)
  // cuts its T pieces from 512-column chunks, at most 16 per rank tile.
  if (!L.stream && (int64_t)L.n_tiles * L.splits <= kFillWgs) {
    const int64_t pchunks = cdiv(K, 512);
    L.t_chunks = (int)cdiv(pchunks, 16);
    L.t_pieces = (int)cdiv(pchunks, L.t_chunks);
  }
  L.m_max = std::max<int64_t>(M_max, 0);
  L.r_pad_large = (int)align_up((size_t)r_cat, 16);

  size_t off = kHeaderBytes;
  // few-row path: tagged T pieces and tagged range partials
  L.tsum = off;    off = align_up(off + (size_t)L.r_tiles * L.t_pieces * 256 * 8, 256);
  L.tfinal = off;  off = align_up(off + (size_t)L.r_tiles * 128 * 8, 256);
  L.ypart = off;   off = align_up(off + (L.splits > 1 ? (size_t)L.n_tiles * L.splits * 256 * 8 : 0), 256);
  // many-row path: fp32 split-K partials of T = X A_cat
  L.T = L.ltpart = off;
  if (L.m_max > kSmallM && r_cat > 0) {
    // splits * M <= 64 * max(256, ceil(M/64)) for every M <= m_max
    const size_t rows = (size_t)std::max<int64_t>(64 * 256, cdiv(L.m_max, 64) * 64);
    off = align_up(off + rows * L.r_pad_large * 4, 256);
  }
  // many-row path: fp32 K-split partials of Y (few output tiles only)
  L.ylarge = off;
  if (L.m_max > kSmallM) off = align_up(off + salr::fwd_large_part_bytes(N, K, L.m_max), 256);
  L.total = off;
  return L;
}

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

}  // namespace

extern "C" {

int salr_fuse_layers(const salr_layer_t* const* parts, int32_t n_parts, salr_layer_t* out, void* stream) {
  if (!parts || !out || n_parts < 1) return SALR_ERR_INVALID_ARG;
  int64_t N = 0;
  int32_t r_cat = 0, n_rec = 0;  // n_rec: parts recorded (a fused part counts its own)
  for (int32_t p = 0; p < n_parts; ++p) {
    const salr_layer_t* L = parts[p];
    if (!L || !dims_ok(L->N, L->K, L->n_keep, L->r_cat)) return SALR_ERR_INVALID_ARG;
    if (L->K != out->K || L->n_keep != out->n_keep) return SALR_ERR_INVALID_ARG;
    if (!L->masks || !L->offsets || (L->n_keep > 0 && !L->values)) return SALR_ERR_INVALID_ARG;
    if (L->r_cat > 0 && (!L->a_cat || !L->b_cat)) return SALR_ERR_INVALID_ARG;
    const void* ptrs[] = {L->masks, L->values, L->offsets, L->a_cat, L->b_cat};
    for (const void* q : ptrs)
      if (q && !aligned16(q)) return SALR_ERR_INVALID_ARG;
    N += L->N;
    r_cat += L->r_cat;
    if (r_cat > kMaxRank) return SALR_ERR_INVALID_ARG;
    if (L->n_parts < 0 || L->n_parts > SALR_MAX_PARTS) return SALR_ERR_INVALID_ARG;
    n_rec += L->n_parts > 1 ? L->n_parts : 1;
  }
  if (n_rec > SALR_MAX_PARTS) return SALR_ERR_INVALID_ARG;
  if (out->N != N || out->r_cat != r_cat || !dims_ok(N, out->K, out->n_keep, r_cat)) return SALR_ERR_INVALID_ARG;
  if (!out->masks || !out->offsets || (out->n_keep > 0 && !out->values)) return SALR_ERR_INVALID_ARG;
  if (r_cat > 0 && (!out->a_cat || !out->b_cat)) return SALR_ERR_INVALID_ARG;
  const void* optrs[] = {out->masks, out->values, out->offsets, out->a_cat, out->b_cat};
  for (const void* q : optrs)
    if (q && !aligned16(q)) return SALR_ERR_INVALID_ARG;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t K = out->K, kw = cdiv(K, 64), ng = cdiv(K, 1024);
  int64_t row0 = 0;
  int32_t rank0 = 0;
  for (int32_t p = 0; p < n_parts; ++p) {
    const salr_layer_t* L = parts[p];
    const auto copy = [&](void* dst, const void* src, size_t bytes) {
      return bytes == 0 || hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s) == hipSuccess;
    };
    bool ok = copy(out->masks + row0 * kw, L->masks, (size_t)L->N * kw * 8) &&
              copy(out->offsets + row0 * ng, L->offsets, (size_t)L->N * ng * 4);
    if (ok && out->n_keep > 0) ok = copy(out->values + row0 * out->n_keep, L->values, (size_t)L->N * out->n_keep * 2);
    if (ok && L->r_cat > 0) ok = copy(out->a_cat + (int64_t)rank0 * K, L->a_cat, (size_t)L->r_cat * K * 2);
    if (!ok) return SALR_ERR_HIP;
    if (r_cat > 0 &&
        salr::launch_fuse_b(L->b_cat, L->N, L->r_cat, out->b_cat + row0 * r_cat, r_cat, rank0, s) != hipSuccess)
      return SALR_ERR_HIP;
    row0 += L->N;
    rank0 += L->r_cat;
  }
  // record the parts (a fused part's own parts in its place)
  int32_t q = 0;
  for (int32_t p = 0; p < n_parts; ++p) {
    const salr_layer_t* L = parts[p];
    if (L->n_parts > 1) {
      for (int32_t e = 0; e < L->n_parts; ++e, ++q) {
        out->part_rows[q] = L->part_rows[e];
        out->part_ranks[q] = L->part_ranks[e];
      }
    } else {
      out->part_rows[q] = (int32_t)L->N;
      out->part_ranks[q] = L->r_cat;
      ++q;
    }
  }
  for (int32_t e = q; e < SALR_MAX_PARTS; ++e) out->part_rows[e] = out->part_ranks[e] = 0;
  out->n_parts = q;
  return hipGetLastError() == hipSuccess ? SALR_OK : SALR_ERR_HIP;
}

const char* salr_status_string(int status) {
  switch (status) {
    case SALR_OK: return "ok";
    case SALR_ERR_INVALID_ARG: return "invalid argument";
    case SALR_ERR_UNSUPPORTED: return "unsupported shape or option";
    case SALR_ERR_WORKSPACE: return "workspace missing or too small";
    case SALR_ERR_NONFINITE: return "weight matrix holds Inf or NaN";
    case SALR_ERR_NUMERICAL: return "truncated SVD lost rank";
    case SALR_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int salr_version(void) { return 10000; }

int salr_query_sizes(int64_t N, int64_t K, int32_t n_keep, int32_t r_svd, int32_t r_cat, int64_t M_max,
                     salr_sizes_t* out) {
  if (!out) return SALR_ERR_INVALID_ARG;
  if (!dims_ok(N, K, n_keep, r_cat)) return SALR_ERR_INVALID_ARG;
  if (r_svd < 0 || r_svd > r_cat || r_svd > std::min<int64_t>(N, K)) return SALR_ERR_INVALID_ARG;
  if (M_max < 0) return SALR_ERR_INVALID_ARG;
  std::memset(out, 0, sizeof(*out));
  out->masks_bytes = (size_t)N * cdiv(K, 64) * 8;
  out->values_bytes = align_up((size_t)N * n_keep * 2, 256) + kValuesPad;
  out->offsets_bytes = (size_t)N * cdiv(K, 1024) * 4;
  out->a_cat_bytes = (size_t)r_cat * K * 2;
  out->b_cat_bytes = align_up((size_t)N * r_cat * 2, 256) + kValuesPad;
  out->encode_ws_bytes = salr::encode_ws_bytes(N, K, r_svd, kMaxOversample);
  out->forward_ws_bytes = fwd_layout(N, K, n_keep, r_cat, M_max).total;
  return SALR_OK;
}

int salr_encode(const uint16_t* W, int64_t N, int64_t K, int32_t n_keep, int32_t r_svd, int32_t n_lora,
                const uint16_t* const* lora_A, const uint16_t* const* lora_B, const int32_t* lora_r,
                const salr_encode_opts_t* opts, salr_layer_t* out, double* sigma, void* ws, size_t ws_bytes,
                void* stream) {
  if (!out || !W) return SALR_ERR_INVALID_ARG;
  if (out->N != N || out->K != K || out->n_keep != n_keep) return SALR_ERR_INVALID_ARG;
  if (!dims_ok(N, K, n_keep, out->r_cat)) return SALR_ERR_INVALID_ARG;
  if (r_svd < 0 || r_svd > std::min<int64_t>(N, K)) return SALR_ERR_INVALID_ARG;
  if (n_lora < 0 || (n_lora > 0 && (!lora_A || !lora_B || !lora_r))) return SALR_ERR_INVALID_ARG;
  int64_t r_cat = r_svd;
  for (int i = 0; i < n_lora; ++i) {
    if (lora_r[i] < 1 || !lora_A[i] || !lora_B[i]) return SALR_ERR_INVALID_ARG;
    if (!aligned16(lora_A[i]) || !aligned16(lora_B[i])) return SALR_ERR_INVALID_ARG;
    r_cat += lora_r[i];
    if (r_cat > kMaxRank) return SALR_ERR_INVALID_ARG;
  }
  if (r_cat != out->r_cat) return SALR_ERR_INVALID_ARG;
  if (!out->masks || !out->offsets || (n_keep > 0 && !out->values)) return SALR_ERR_INVALID_ARG;
  if (r_cat > 0 && (!out->a_cat || !out->b_cat)) return SALR_ERR_INVALID_ARG;
  const void* ptrs[] = {W, out->masks, out->values, out->offsets, out->a_cat, out->b_cat};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SALR_ERR_INVALID_ARG;
  salr::EncodeParams p{};
  p.oversample = opts ? opts->oversample : kDefaultOversample;
  p.iters = opts ? opts->iters : kDefaultIters;
  p.seed = opts ? opts->seed : 0;
  if (p.oversample < 0 || p.oversample > kMaxOversample || p.iters < 0 || p.iters > kMaxIters)
    return SALR_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws)) return SALR_ERR_WORKSPACE;
  if (ws_bytes < salr::encode_ws_bytes(N, K, r_svd, p.oversample)) return SALR_ERR_WORKSPACE;
  p.W = W;
  p.N = N;
  p.K = K;
  p.n_keep = n_keep;
  p.r_svd = r_svd;
  p.r_cat = (int32_t)r_cat;
  p.n_lora = n_lora;
  p.lora_A = lora_A;
  p.lora_B = lora_B;
  p.lora_r = lora_r;
  p.masks = out->masks;
  p.values = out->values;
  p.offsets = out->offsets;
  p.a_cat = out->a_cat;
  p.b_cat = out->b_cat;
  p.sigma = sigma;
  p.ws = ws;
  p.ws_bytes = ws_bytes;
  p.stream = static_cast<hipStream_t>(stream);
  return salr::encode_run(p);
}

int salr_linear_forward(const salr_layer_t* L, const uint16_t* X, int64_t M, uint16_t* Y, void* ws, size_t ws_bytes,
                        void* stream) {
  if (!L) return SALR_ERR_INVALID_ARG;
  if (!dims_ok(L->N, L->K, L->n_keep, L->r_cat)) return SALR_ERR_INVALID_ARG;
  if (M < 0 || M > (int64_t(1) << 31) - 1) return SALR_ERR_INVALID_ARG;
  if (M == 0) return SALR_OK;
  if (!X || !Y || !L->masks || !L->offsets) return SALR_ERR_INVALID_ARG;
  if (L->n_keep > 0 && !L->values) return SALR_ERR_INVALID_ARG;
  if (L->r_cat > 0 && (!L->a_cat || !L->b_cat)) return SALR_ERR_INVALID_ARG;
  const void* ptrs[] = {X, Y, L->masks, L->values, L->offsets, L->a_cat, L->b_cat};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SALR_ERR_INVALID_ARG;
  if (static_cast<const void*>(X) == static_cast<const void*>(Y)) return SALR_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws)) return SALR_ERR_WORKSPACE;
  // A fused layer's parts: each row tile multiplies only its part's block
  // of ranks when every part has whole row tiles and 8-aligned ranks.
  if (L->n_parts < 0 || L->n_parts > SALR_MAX_PARTS) return SALR_ERR_INVALID_ARG;
  bool windows = L->n_parts > 1;
  int32_t r_win = L->r_cat;
  if (L->n_parts > 1) {
    int64_t rows = 0, ranks = 0;
    int32_t widest = 0;
    for (int p = 0; p < L->n_parts; ++p) {
      if (L->part_rows[p] < 1 || L->part_ranks[p] < 0) return SALR_ERR_INVALID_ARG;
      rows += L->part_rows[p];
      ranks += L->part_ranks[p];
      widest = std::max(widest, L->part_ranks[p]);
      windows = windows && L->part_rows[p] % 16 == 0 && L->part_ranks[p] % 8 == 0;
    }
    if (rows != L->N || ranks != L->r_cat) return SALR_ERR_INVALID_ARG;
    if (windows) r_win = widest;
  }
  const FwdLayout W = fwd_layout(L->N, L->K, L->n_keep, L->r_cat, M, r_win);
  if (ws_bytes < W.total) return SALR_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);

  hipError_t err;
  if (M <= kSmallM && W.stream) {
    StreamFwdArgs a{};
    a.masks = L->masks;
    a.values = L->values;
    a.offsets = L->offsets;
    a.b_cat = L->b_cat;
    a.X = X;
    a.Y = Y;
    a.a_cat = L->a_cat;
    a.tpiece = at<uint64_t>(ws, W.tsum);
    a.tfinal = at<uint64_t>(ws, W.tfinal);
    a.tcount = at<uint32_t>(ws, kCounterT);
    a.N = L->N;
    a.K = (int32_t)L->K;
    a.n_keep = L->n_keep;
    a.r_cat = L->r_cat;
    a.M = (int32_t)M;
    a.kw = (int32_t)cdiv(L->K, 64);
    a.ng = (int32_t)cdiv(L->K, 1024);
    a.n_tiles = W.n_tiles;
    a.tiles_per_wg = W.tiles_per_wg;
    a.vcap = W.svcap;
    a.r_tiles = L->r_cat > 0 ? W.r_tiles : 0;
    a.r_pad = L->r_cat > 0 ? W.r_pad_small : 0;
    a.t_pieces = W.t_pieces;
    a.t_chunks = W.t_chunks;
    a.tickets = at<uint64_t>(ws, kCounterTickets);
    a.err = at<uint32_t>(ws, kCounterSync + 8);
    err = salr::launch_fwd_stream(a, s);
  } else if (M <= kSmallM) {
    SmallFwdArgs a{};
    a.masks = L->masks;
    a.values = L->values;
    a.offsets = L->offsets;
    a.b_cat = L->b_cat;
    a.X = X;
    a.Y = Y;
    a.a_cat = L->a_cat;
    a.tpiece = at<uint64_t>(ws, W.tsum);
    a.tfinal = at<uint64_t>(ws, W.tfinal);
    a.tcount = at<uint32_t>(ws, kCounterT);
    a.N = L->N;
    a.K = (int32_t)L->K;
    a.n_keep = L->n_keep;
    a.r_cat = L->r_cat;
    a.M = (int32_t)M;
    a.kw = (int32_t)cdiv(L->K, 64);
    a.ng = (int32_t)cdiv(L->K, 1024);
    a.n_tiles = W.n_tiles;
    a.splits = W.splits;
    a.range = W.range;
    a.vcap = W.vcap;
    a.r_tiles = W.r_tiles;
    a.r_pad = W.r_pad_small;
    a.t_pieces = W.t_pieces;
    a.t_chunks = W.t_chunks;
    a.vals_bytes = W.vals_bytes;
    a.tl_bytes = W.tl_bytes;
    a.bl_bytes = W.bl_bytes;
    // (about 1 us with up to 48 producers; with more, T is on the critical
    // path and they start at once: measured on 4096 x 4096 at r_cat 80 / 112)
    a.psleep = W.r_tiles * W.t_pieces <= 48 ? 40 : 0;
    a.nparts = 0;
    if (windows) {
      int32_t tile_end = 0, rank0 = 0;
      for (int p = 0; p < L->n_parts; ++p) {
        tile_end += L->part_rows[p] / 16;
        a.part_tile_end[p] = tile_end;
        a.part_rank0[p] = rank0;
        a.part_nrank[p] = L->part_ranks[p];
        rank0 += L->part_ranks[p];
      }
      a.nparts = L->n_parts;
    }
    a.tickets = at<uint64_t>(ws, kCounterTickets);
    a.err = at<uint32_t>(ws, kCounterSync + 8);
    a.ycount = at<uint32_t>(ws, kCounterY);
    a.ypart = at<uint64_t>(ws, W.ypart);
    err = salr::launch_fwd_small(a, s);
  } else {
    int t_splits = 0;
    if (L->r_cat > 0) {
      LowRankTArgs t{};
      t.X = X;
      t.a_cat = L->a_cat;
      t.tpart = at<float>(ws, W.ltpart);
      t.M = (int32_t)M;
      t.K = (int32_t)L->K;
      t.r_cat = L->r_cat;
      t.r_pad = W.r_pad_large;
      t.splits = t_splits_large(M, L->K);
      t.k_chunk = (int32_t)(cdiv(cdiv(L->K, 64), t.splits) * 64);
      t.splits = (int32_t)cdiv(L->K, t.k_chunk);
      t_splits = t.splits;
      err = salr::launch_lowrank_t(t, s);
      if (err != hipSuccess) return SALR_ERR_HIP;
    }
    LargeFwdArgs a{};
    a.masks = L->masks;
    a.values = L->values;
    a.b_cat = L->b_cat;
    a.X = X;
    a.tpart = L->r_cat > 0 ? at<float>(ws, W.ltpart) : nullptr;
    a.t_splits = t_splits;
    a.Y = Y;
    a.N = L->N;
    a.K = (int32_t)L->K;
    a.n_keep = L->n_keep;
    a.r_cat = L->r_cat;
    a.r_pad = W.r_pad_large;
    a.M = (int32_t)M;
    a.kw = (int32_t)cdiv(L->K, 64);
    a.vchunks = cdiv(L->N * (int64_t)L->n_keep, 8);
    a.offsets = L->offsets;
    a.ng = (int32_t)cdiv(L->K, 1024);
    a.ksplit = salr::fwd_large_ksplit(L->N, L->K, M);
    const int64_t nk = cdiv(L->K, 64);
    a.kt_per = (int32_t)(cdiv(cdiv(nk, a.ksplit), 8) * 8);  // (whole groups of 8 tiles)
    a.ksplit = (int32_t)cdiv(nk, a.kt_per);
    a.ypart = at<float>(ws, W.ylarge);
    a.x_off32 = M * L->K * 2 < (int64_t(1) << 32) ? 1 : 0;
    a.nparts = 0;
    if (windows) {
      bool whole = true;
      for (int p = 0; p < L->n_parts; ++p) whole = whole && L->part_rows[p] % 256 == 0;
      if (whole) {
        int32_t row_end = 0, rank0 = 0;
        for (int p = 0; p < L->n_parts; ++p) {
          row_end += L->part_rows[p];
          a.part_row_end[p] = row_end;
          a.part_rank0[p] = rank0;
          a.part_nrank[p] = L->part_ranks[p];
          rank0 += L->part_ranks[p];
        }
        a.nparts = L->n_parts;
      }
    }
    err = salr::launch_fwd_large(a, s);
  }
  return err == hipSuccess ? SALR_OK : SALR_ERR_HIP;
}

}  // extern "C"
