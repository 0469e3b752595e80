// C ABI of the SALR library: argument validation, workspace layout and
// kernel dispatch.  See include/salr.h for the contract of every entry point.
#include "salr.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "salr_api_internal.hpp"
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
constexpr int32_t kDefaultIters = 40;
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
  int nf4_cofs, nf4_sofs;  // NF4: LDS chunk offsets of the codes and scales in a row's area
  int vals_bytes, tl_bytes, bl_bytes;
  // few-row streaming path (layers with more than one round of 16-row work)
  bool stream;
  int tiles_per_wg, svcap;
  // many-row path
  int64_t m_max;
  int r_pad_large;
  // offsets (bytes)
  size_t tsum, tfinal, ypart, T, ltpart, t16, ylarge, dq, total;
};

// NF4 layers: the few-row kernel's dequantization pass gives each of 32
// threads per row at most kNf4Groups groups of 8 values, so a row segment
// holds at most this many kept values.
constexpr int64_t kNf4MaxSeg = 2048;
static_assert(kNf4MaxSeg / 8 + 1 <= 32 * salr::kNf4Groups, "NF4 segment too long for the dequantization pass");

// r_win: the most adapter ranks one row tile multiplies (r_cat, or a fused
// layer's largest part block); it sizes the few-row B_cat rows in LDS.
// nf4: the layer's values are NF4 codes (QSALR): few-row segments of at most
// kNf4MaxSeg values with room for codes and scales at the end of each row's
// LDS area, no streaming kernel, and (M_max > 16) a workspace region for the
// dequantized values of the many-row kernel.
FwdLayout fwd_layout(int64_t N, int64_t K, int32_t n_keep, int32_t r_cat, int64_t M_max, int32_t r_win = -1,
                     bool nf4 = false) {
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
  // (NF4: codes of cap values + a window's 8 bytes, and the scales of its
  // blocks, in whole chunks behind the values)
  const auto nf4_code_chunks = [](int64_t cap) { return (int)((cap / 2 + 1 + 8 + 15) / 16 + 1); };
  const auto nf4_scale_chunks = [](int64_t cap) { return (int)((((cap + 63) / 64 + 1) * 2 + 15) / 16 + 1); };
  const auto vcap_for = [&](int64_t range) {
    const int64_t cap = std::min<int64_t>(range, n_keep);
    int v = salr::fwd_small_vcap(cap, range >= K && n_keep % 8 == 0);
    if (nf4) {
      const int need = nf4_code_chunks(cap) + nf4_scale_chunks(cap) + 1;
      while (v < need) v += 8;  // (stride stays 1 mod 8 chunks)
    }
    return v;
  };
  const auto lds_for = [&](int64_t range) { return salr::fwd_small_lds_bytes(vcap_for(range), L.bl_bytes); };
  L.range = 0;
  const int max_range = nf4 ? (int)kNf4MaxSeg : salr::kMaxRangeCols;
  if (K <= salr::kMaxRangeCols && lds_for(K) <= kSmallLdsBudget && (L.n_tiles >= kFillWgs || K <= 1024) &&
      (!nf4 || n_keep <= kNf4MaxSeg)) {
    L.range = (int)K;
  } else {
    for (int range = max_range; range >= 1024; range /= 2) {
      if (lds_for(range) > kSmallLdsBudget) continue;
      L.range = range;
      if ((int64_t)L.n_tiles * cdiv(K, range) >= kFillWgs) break;
    }
    if (L.range == 0) L.range = 1024;
    if (L.range >= K) L.range = (int)K;
  }
  L.splits = (int)cdiv(K, L.range);
  L.vcap = vcap_for(L.range);
  if (nf4) {
    const int64_t cap = std::min<int64_t>(L.range, n_keep);
    L.nf4_sofs = L.vcap - nf4_scale_chunks(cap);
    L.nf4_cofs = L.nf4_sofs - nf4_code_chunks(cap);
  }
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
    L.stream = !nf4 && L.splits > 1 && fills && (int64_t)L.n_tiles * L.splits > kFillWgs && cdiv(K, 1024) <= 64 &&
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
  // many-row path: fp32 split-K partials of T = X A_cat, then their bf16 sum
  L.T = L.ltpart = off;
  L.t16 = off;
  if (L.m_max > kSmallM && r_cat > 0) {
    // splits * M <= 64 * max(256, ceil(M/64)) for every M <= m_max
    const size_t rows = (size_t)std::max<int64_t>(64 * 256, cdiv(L.m_max, 64) * 64);
    off = align_up(off + rows * L.r_pad_large * 4, 256);
    L.t16 = off;
    off = align_up(off + (size_t)L.m_max * L.r_pad_large * 2, 256);
  }
  // many-row path: fp32 K-split partials of Y (few output tiles only)
  L.ylarge = off;
  if (L.m_max > kSmallM) off = align_up(off + salr::fwd_large_part_bytes(N, K, L.m_max), 256);
  // NF4, many-row path: the dequantized values (the bf16 layout, with its
  // tail padding)
  L.dq = off;
  if (nf4 && L.m_max > kSmallM) off = align_up(off + align_up((size_t)N * n_keep * 2, 256) + kValuesPad, 256);
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
    if (L->value_format != SALR_VALUES_BF16) return SALR_ERR_INVALID_ARG;  // (fusion copies bf16 values)
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
  const int64_t nblk = cdiv(n_keep, 64);
  out->codes_bytes = (size_t)N * nblk * 32 + kValuesPad;
  out->scales_bytes = align_up((size_t)N * nblk * 2, 256) + kValuesPad;
  out->forward_ws_nf4_bytes = fwd_layout(N, K, n_keep, r_cat, M_max, -1, true).total;
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
  // an encoded layer is one part: a stale record from an earlier fusion
  // into this descriptor would make the forward skip adapter ranks; its
  // values are bf16
  out->n_parts = 0;
  out->value_format = SALR_VALUES_BF16;
  for (int e = 0; e < SALR_MAX_PARTS; ++e) out->part_rows[e] = out->part_ranks[e] = 0;
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

int salr_nf4_levels(float* out) {
  if (!out) return SALR_ERR_INVALID_ARG;
  salr::nf4_levels(out);
  return SALR_OK;
}

int salr_quantize_nf4(salr_layer_t* L, void* stream) {
  if (!L || !dims_ok(L->N, L->K, L->n_keep, L->r_cat)) return SALR_ERR_INVALID_ARG;
  if (L->value_format != SALR_VALUES_BF16) return SALR_ERR_INVALID_ARG;
  if ((L->n_keep > 0 && !L->values) || !L->codes || !L->scales) return SALR_ERR_INVALID_ARG;
  if ((L->values && !aligned16(L->values)) || !aligned16(L->codes) || !aligned16(L->scales))
    return SALR_ERR_INVALID_ARG;
  if (salr::launch_quantize_nf4(L->values, L->N, L->n_keep, L->codes, L->scales, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return SALR_ERR_HIP;
  L->value_format = SALR_VALUES_NF4;
  return SALR_OK;
}

int salr_linear_forward(const salr_layer_t* L, const uint16_t* X, int64_t M, uint16_t* Y, void* ws, size_t ws_bytes,
                        void* stream) {
  // (a null ws is rejected by forward_impl before the error word is used)
  return salr::forward_impl(L, X, M, Y, ws, ws_bytes, ws ? at<uint32_t>(ws, kCounterSync + 8) : nullptr,
                            static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ----------------------------------------------------------------------------
// Backward: the transposed encoding of W_s and the gradient pass.
namespace {

// Workspace of the transposed-encoding build: rowpre [N][kw], the block
// column counts [nb][K], then the largest column count.
struct TrLayout {
  size_t rowpre, cnt, maxc, total;
};
TrLayout tr_layout(int64_t N, int64_t K) {
  TrLayout T{};
  const int64_t kw = cdiv(K, 64), nb = cdiv(N, 64);
  T.rowpre = 0;
  T.cnt = align_up((size_t)N * kw * 4, 256);
  T.maxc = align_up(T.cnt + (size_t)nb * K * 4, 256);
  T.total = T.maxc + 256;
  return T;
}

// Runs the count pass and returns (host) the largest column count.
int transpose_count_run(const salr_layer_t* L, uint32_t* offsets_t, void* ws, size_t ws_bytes, hipStream_t s,
                        uint32_t* maxc) {
  const TrLayout T = tr_layout(L->N, L->K);
  if (!ws || !aligned16(ws)) return SALR_ERR_WORKSPACE;
  if (ws_bytes < T.total) return SALR_ERR_WORKSPACE;
  uint32_t* dmax = at<uint32_t>(ws, T.maxc);
  if (hipMemsetAsync(dmax, 0, 4, s) != hipSuccess) return SALR_ERR_HIP;
  if (salr::launch_transpose_count(L->masks, L->N, (int32_t)L->K, at<uint32_t>(ws, T.rowpre), at<uint32_t>(ws, T.cnt),
                                   dmax, offsets_t, (int32_t)cdiv(L->N, 1024), s) != hipSuccess)
    return SALR_ERR_HIP;
  if (hipMemcpyAsync(maxc, dmax, 4, hipMemcpyDeviceToHost, s) != hipSuccess) return SALR_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return SALR_ERR_HIP;
  return SALR_OK;
}

// Checks shared by the transposed-encoding calls.
int transpose_check(const salr_layer_t* L) {
  if (!L || !dims_ok(L->N, L->K, L->n_keep, L->r_cat)) return SALR_ERR_INVALID_ARG;
  if (!L->masks || !aligned16(L->masks)) return SALR_ERR_INVALID_ARG;
  // W_s^T has N columns: the layer limits apply with N and K swapped
  if (L->N % 8 != 0 || L->N > kMaxK || L->K > kMaxRowTiles * 16) return SALR_ERR_UNSUPPORTED;
  return SALR_OK;
}

// Gradient-GEMM splits over the M tokens: about kGemmItems workgroups, each
// split at least 128 tokens.
constexpr int64_t kGemmItems = 512;
int gemm_splits(int64_t P, int64_t Q, int64_t M) {
  const int64_t tiles = cdiv(P, 64) * cdiv(Q, 64);
  const int64_t s = std::min<int64_t>(std::max<int64_t>(1, kGemmItems / std::max<int64_t>(tiles, 1)), cdiv(M, 128));
  return (int)std::max<int64_t>(s, 1);
}

// Backward workspace: the forward workspace of the transposed layer first
// (its counter header at offset 0), then the transposed adapters, the
// low-rank activations G and T (bf16 [M][r_pad]) and the gradient GEMMs'
// split partials.  Every region grows with M.
struct BwdLayout {
  int r_pad;
  int splits_a, splits_b;
  size_t fwd, bt, at_, tpart, g16, t16, part, total;
};
BwdLayout bwd_layout(int64_t N, int64_t K, int32_t n_keep_t, int32_t r_cat, int64_t M) {
  BwdLayout B{};
  B.r_pad = (int)align_up((size_t)r_cat, 16);
  B.fwd = fwd_layout(K, N, n_keep_t, r_cat, M).total;
  size_t off = align_up(B.fwd, 256);
  B.bt = off;   off = align_up(off + (size_t)r_cat * N * 2, 256);
  B.at_ = off;  off = align_up(off + (size_t)K * r_cat * 2, 256) + kValuesPad;
  B.tpart = off;
  B.g16 = B.t16 = B.part = off;
  if (r_cat > 0 && M > 0) {
    const size_t rows = (size_t)std::max<int64_t>(64 * 256, cdiv(M, 64) * 64);
    off = align_up(off + rows * B.r_pad * 4, 256);
    B.g16 = off;  off = align_up(off + (size_t)M * B.r_pad * 2, 256);
    B.t16 = off;  off = align_up(off + (size_t)M * B.r_pad * 2, 256);
    B.splits_a = gemm_splits(r_cat, K, M);
    B.splits_b = gemm_splits(N, r_cat, M);
    B.part = off;
    off = align_up(off + std::max((size_t)B.splits_a * r_cat * K, (size_t)B.splits_b * N * r_cat) * 4, 256);
  }
  B.total = off;
  return B;
}

}  // namespace

extern "C" {

int salr_transpose_ws_bytes(int64_t N, int64_t K, size_t* out) {
  if (!out || !dims_ok(N, K, 0, 0)) return SALR_ERR_INVALID_ARG;
  *out = tr_layout(N, K).total;
  return SALR_OK;
}

int salr_transpose_count(const salr_layer_t* L, int32_t* n_keep_t, void* ws, size_t ws_bytes, void* stream) {
  if (!n_keep_t) return SALR_ERR_INVALID_ARG;
  const int rc = transpose_check(L);
  if (rc != SALR_OK) return rc;
  uint32_t maxc = 0;
  const int e = transpose_count_run(L, nullptr, ws, ws_bytes, static_cast<hipStream_t>(stream), &maxc);
  if (e != SALR_OK) return e;
  *n_keep_t = (int32_t)maxc;
  return SALR_OK;
}

int salr_transpose_layer(const salr_layer_t* L, salr_layer_t* LT, void* ws, size_t ws_bytes, void* stream) {
  const int rc = transpose_check(L);
  if (rc != SALR_OK) return rc;
  if (!LT) return SALR_ERR_INVALID_ARG;
  if (L->value_format != SALR_VALUES_BF16) return SALR_ERR_UNSUPPORTED;
  if (L->n_keep > 0 && (!L->values || !aligned16(L->values))) return SALR_ERR_INVALID_ARG;
  if (LT->N != L->K || LT->K != L->N || !dims_ok(LT->N, LT->K, LT->n_keep, L->r_cat)) return SALR_ERR_INVALID_ARG;
  if (!LT->masks || !LT->offsets || (LT->n_keep > 0 && !LT->values)) return SALR_ERR_INVALID_ARG;
  const void* ptrs[] = {LT->masks, LT->values, LT->offsets};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return SALR_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t maxc = 0;
  int e = transpose_count_run(L, LT->offsets, ws, ws_bytes, s, &maxc);
  if (e != SALR_OK) return e;
  if ((int64_t)maxc > LT->n_keep) return SALR_ERR_INVALID_ARG;
  const TrLayout T = tr_layout(L->N, L->K);
  if (LT->n_keep > 0 && hipMemsetAsync(LT->values, 0, (size_t)LT->N * LT->n_keep * 2, s) != hipSuccess)
    return SALR_ERR_HIP;
  if (salr::launch_transpose_scatter(L->masks, L->values, at<uint32_t>(ws, T.rowpre), at<uint32_t>(ws, T.cnt), L->N,
                                     (int32_t)L->K, L->n_keep, LT->n_keep, LT->masks, LT->values, s) != hipSuccess)
    return SALR_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return SALR_ERR_HIP;
  LT->r_cat = L->r_cat;
  LT->n_parts = 0;
  for (int q = 0; q < SALR_MAX_PARTS; ++q) LT->part_rows[q] = LT->part_ranks[q] = 0;
  LT->value_format = SALR_VALUES_BF16;
  LT->codes = nullptr;
  LT->scales = nullptr;
  return SALR_OK;
}

int salr_backward_ws_bytes(int64_t N, int64_t K, int32_t n_keep_t, int32_t r_cat, int64_t M_max, size_t* out) {
  if (!out || !dims_ok(N, K, 0, r_cat) || M_max < 0) return SALR_ERR_INVALID_ARG;
  if (N % 8 != 0 || N > kMaxK || K > kMaxRowTiles * 16) return SALR_ERR_UNSUPPORTED;
  if (!dims_ok(K, N, n_keep_t, r_cat)) return SALR_ERR_INVALID_ARG;
  *out = bwd_layout(N, K, n_keep_t, r_cat, M_max).total;
  return SALR_OK;
}

int salr_linear_backward(const salr_layer_t* L, const salr_layer_t* LT, const uint16_t* X, const uint16_t* dY,
                         int64_t M, uint16_t* dX, float* dA, float* dB, void* ws, size_t ws_bytes, void* stream) {
  if (!L || !LT) return SALR_ERR_INVALID_ARG;
  if (!dims_ok(L->N, L->K, L->n_keep, L->r_cat)) return SALR_ERR_INVALID_ARG;
  if (L->N % 8 != 0 || L->N > kMaxK || L->K > kMaxRowTiles * 16) return SALR_ERR_UNSUPPORTED;
  if (LT->N != L->K || LT->K != L->N || LT->r_cat != L->r_cat || !dims_ok(LT->N, LT->K, LT->n_keep, LT->r_cat))
    return SALR_ERR_INVALID_ARG;
  if (LT->value_format != SALR_VALUES_BF16 || LT->n_parts != 0) return SALR_ERR_INVALID_ARG;
  if (M < 0 || M > (int64_t(1) << 31) - 1) return SALR_ERR_INVALID_ARG;
  const int32_t r = L->r_cat;
  if (r > 0 && (!L->a_cat || !L->b_cat)) return SALR_ERR_INVALID_ARG;
  if (M > 0 && (!X || !dY)) return SALR_ERR_INVALID_ARG;
  if (dX && (!LT->masks || !LT->offsets || (LT->n_keep > 0 && !LT->values))) return SALR_ERR_INVALID_ARG;
  if (r > 0 && (!dA || !dB)) return SALR_ERR_INVALID_ARG;
  const void* ptrs[] = {X, dY, dX, dA, dB, L->a_cat, L->b_cat, LT->masks, LT->values, LT->offsets};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return SALR_ERR_INVALID_ARG;
  if (dX && (static_cast<const void*>(dX) == static_cast<const void*>(dY))) return SALR_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws)) return SALR_ERR_WORKSPACE;
  const BwdLayout B = bwd_layout(L->N, L->K, LT->n_keep, r, M);
  if (ws_bytes < B.total) return SALR_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t N = L->N, K = L->K;
  if (M == 0) {
    // an empty token sum: zero adapter gradients (no dX rows)
    if (r > 0 && (salr::launch_gemm_tn(nullptr, 0, 0, nullptr, 0, 0, r, K, 0, 1, nullptr, dA, s) != hipSuccess ||
                  salr::launch_gemm_tn(nullptr, 0, 0, nullptr, 0, 0, N, r, 0, 1, nullptr, dB, s) != hipSuccess))
      return SALR_ERR_HIP;
    return SALR_OK;
  }
  uint16_t* bt = at<uint16_t>(ws, B.bt);   // B_cat [r][N]: the transposed layer's a_cat
  uint16_t* att = at<uint16_t>(ws, B.at_); // A_cat [K][r]: the transposed layer's b_cat
  if (r > 0) {
    if (salr::launch_transpose_bf16_pair(L->b_cat, N, r, r, bt, N, L->a_cat, r, K, K, att, r, s) != hipSuccess)
      return SALR_ERR_HIP;
  }
  if (dX) {
    salr_layer_t lt = *LT;
    lt.a_cat = r > 0 ? bt : nullptr;
    lt.b_cat = r > 0 ? att : nullptr;
    const int e = salr::forward_impl(&lt, dY, M, dX, ws, B.fwd, at<uint32_t>(ws, kCounterSync + 8), s);
    if (e != SALR_OK) return e;
  }
  if (r == 0) return SALR_OK;
  // G = dY B_cat^T and T = X A_cat, each rounded to bf16 [M][r_pad] (ranks
  // past r_cat zero)
  const auto lowrank = [&](const uint16_t* in, const uint16_t* rows, int64_t Kin, uint16_t* out16) {
    LowRankTArgs t{};
    t.X = in;
    t.a_cat = rows;
    t.tpart = at<float>(ws, B.tpart);
    t.t16 = out16;
    t.M = (int32_t)M;
    t.K = (int32_t)Kin;
    t.r_cat = r;
    t.r_pad = B.r_pad;
    t.splits = t_splits_large(M, Kin);
    t.k_chunk = (int32_t)(cdiv(cdiv(Kin, 64), t.splits) * 64);
    t.splits = (int32_t)cdiv(Kin, t.k_chunk);
    return salr::launch_lowrank_t(t, s) == hipSuccess;
  };
  // (with dX over many rows the forward of the transposed layer has just
  // made G the same way, as its own X A_cat: it is read from its workspace)
  const uint16_t* g16 = at<uint16_t>(ws, B.g16);
  if (dX && M > kSmallM) {
    g16 = at<uint16_t>(ws, fwd_layout(K, N, LT->n_keep, r, M).t16);
  } else if (!lowrank(dY, bt, N, at<uint16_t>(ws, B.g16))) {
    return SALR_ERR_HIP;
  }
  uint16_t* t16 = at<uint16_t>(ws, B.t16);
  if (!lowrank(X, L->a_cat, K, t16)) return SALR_ERR_HIP;
  float* part = at<float>(ws, B.part);
  const int64_t r8 = (int64_t)align_up((size_t)r, 8);  // (<= r_pad, zeros past r)
  // dA_cat (stored [r][K]) [j][k] = sum_m G[m][j] X[m][k]
  if (salr::launch_gemm_tn(g16, B.r_pad, r8, X, K, K, r, K, M, B.splits_a, part, dA, s) != hipSuccess)
    return SALR_ERR_HIP;
  // dB_cat (stored [N][r]) [n][j] = sum_m dY[m][n] T[m][j]
  if (salr::launch_gemm_tn(dY, N, N, t16, B.r_pad, r8, N, r, M, B.splits_b, part, dB, s) != hipSuccess)
    return SALR_ERR_HIP;
  return SALR_OK;
}

}  // extern "C"

// ----------------------------------------------------------------------------
// Grouped (mixture-of-experts) layers.
namespace {

constexpr int32_t kMaxExperts = 4096;

struct MoeLayout {
  size_t ms, vs, os, as, bs;       // per-expert strides (elements)
  size_t mb, vb, ob, ab, bb;       // buffer bytes
  int r_pad;
};
MoeLayout moe_layout(int32_t E, int64_t N, int64_t K, int32_t n_keep, int32_t r_cat) {
  MoeLayout G{};
  G.ms = align_up((size_t)N * cdiv(K, 64), 32);
  G.vs = align_up((size_t)N * n_keep, 128);
  G.os = align_up((size_t)N * cdiv(K, 1024), 64);
  G.as = align_up((size_t)r_cat * K, 128);
  G.bs = align_up((size_t)N * r_cat, 128);
  G.mb = G.ms * E * 8;
  G.vb = G.vs * E * 2 + kValuesPad;
  G.ob = G.os * E * 4;
  G.ab = G.as * E * 2;
  G.bb = G.bs * E * 2 + kValuesPad;
  G.r_pad = (int)align_up((size_t)r_cat, 32);
  return G;
}

bool moe_dims_ok(const salr_moe_layer_t* G) {
  return G && G->E >= 1 && G->E <= kMaxExperts && dims_ok(G->N, G->K, G->n_keep, G->r_cat) &&
         G->N <= kMaxNK / G->K / G->E;
}

}  // namespace

extern "C" {

int salr_moe_query_sizes(int32_t E, int64_t N, int64_t K, int32_t n_keep, int32_t r_cat, int64_t T_max,
                         salr_moe_sizes_t* out) {
  salr_moe_layer_t g{};
  g.E = E;
  g.N = N;
  g.K = K;
  g.n_keep = n_keep;
  g.r_cat = r_cat;
  if (!out || !moe_dims_ok(&g) || T_max < 0 || T_max > (int64_t(1) << 31) - 1) return SALR_ERR_INVALID_ARG;
  const MoeLayout G = moe_layout(E, N, K, n_keep, r_cat);
  std::memset(out, 0, sizeof(*out));
  out->masks_bytes = G.mb;
  out->values_bytes = G.vb;
  out->offsets_bytes = G.ob;
  out->a_cat_bytes = G.ab;
  out->b_cat_bytes = G.bb;
  out->masks_stride = G.ms;
  out->values_stride = G.vs;
  out->offsets_stride = G.os;
  out->a_cat_stride = G.as;
  out->b_cat_stride = G.bs;
  out->forward_ws_bytes =
      r_cat > 0 ? salr::moe_lowrank_part_bytes(T_max, K, G.r_pad) + align_up((size_t)T_max * G.r_pad * 2, 256) : 256;
  return SALR_OK;
}

int salr_moe_expert(const salr_moe_layer_t* G, int32_t e, salr_layer_t* out) {
  if (!out || !moe_dims_ok(G) || e < 0 || e >= G->E) return SALR_ERR_INVALID_ARG;
  if (!G->masks || !G->offsets || (G->n_keep > 0 && !G->values)) return SALR_ERR_INVALID_ARG;
  if (G->r_cat > 0 && (!G->a_cat || !G->b_cat)) return SALR_ERR_INVALID_ARG;
  const MoeLayout L = moe_layout(G->E, G->N, G->K, G->n_keep, G->r_cat);
  std::memset(out, 0, sizeof(*out));
  out->N = G->N;
  out->K = G->K;
  out->n_keep = G->n_keep;
  out->r_cat = G->r_cat;
  out->masks = G->masks + L.ms * e;
  out->values = G->values ? G->values + L.vs * e : nullptr;
  out->offsets = G->offsets + L.os * e;
  out->a_cat = G->r_cat > 0 ? G->a_cat + L.as * e : nullptr;
  out->b_cat = G->r_cat > 0 ? G->b_cat + L.bs * e : nullptr;
  out->value_format = SALR_VALUES_BF16;
  return SALR_OK;
}

int salr_moe_forward(const salr_moe_layer_t* G, const uint16_t* X, int64_t T, const int32_t* expert_offsets,
                     int64_t m_cap, uint16_t* Y, void* ws, size_t ws_bytes, void* stream) {
  if (!moe_dims_ok(G)) return SALR_ERR_INVALID_ARG;
  if (T < 0 || T > (int64_t(1) << 31) - 1 || m_cap < 0) return SALR_ERR_INVALID_ARG;
  if (T == 0) return SALR_OK;
  if (!X || !Y || !expert_offsets) return SALR_ERR_INVALID_ARG;
  if (!G->masks || !G->offsets || (G->n_keep > 0 && !G->values)) return SALR_ERR_INVALID_ARG;
  if (G->r_cat > 0 && (!G->a_cat || !G->b_cat)) return SALR_ERR_INVALID_ARG;
  const void* ptrs[] = {X, Y, G->masks, G->values, G->offsets, G->a_cat, G->b_cat};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return SALR_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(expert_offsets) & 3u) != 0) return SALR_ERR_INVALID_ARG;
  if (static_cast<const void*>(X) == static_cast<const void*>(Y)) return SALR_ERR_INVALID_ARG;
  const MoeLayout L = moe_layout(G->E, G->N, G->K, G->n_keep, G->r_cat);
  if (!ws || !aligned16(ws)) return SALR_ERR_WORKSPACE;
  const size_t part_bytes = G->r_cat > 0 ? salr::moe_lowrank_part_bytes(T, G->K, L.r_pad) : 0;
  if (G->r_cat > 0 && ws_bytes < part_bytes + (size_t)T * L.r_pad * 2) return SALR_ERR_WORKSPACE;
  salr::MoeArgs a{};
  a.masks = G->masks;
  a.values = G->values;
  a.offsets = G->offsets;
  a.a_cat = G->a_cat;
  a.b_cat = G->b_cat;
  a.mstride = L.ms;
  a.vstride = L.vs;
  a.ostride = L.os;
  a.astride = L.as;
  a.bstride = L.bs;
  a.X = X;
  a.Y = Y;
  a.eoff = expert_offsets;
  a.tpart = static_cast<float*>(ws);
  a.t16 = at<uint16_t>(ws, part_bytes);
  a.N = G->N;
  a.E = G->E;
  a.T = (int32_t)T;
  a.K = (int32_t)G->K;
  a.n_keep = G->n_keep;
  a.r_cat = G->r_cat;
  a.r_pad = G->r_cat > 0 ? L.r_pad : 0;
  a.kw = (int32_t)cdiv(G->K, 64);
  a.ng = (int32_t)cdiv(G->K, 1024);
  if (G->r_cat > 0) {
    const int64_t steps = cdiv(G->K, 128);
    const int64_t splits = salr::moe_lowrank_splits(T, G->K, L.r_pad);
    a.kspan = (int32_t)(cdiv(steps, splits) * 128);
    a.ksplits = (int32_t)cdiv(G->K, a.kspan);
  }
  const int32_t cap = (int32_t)(m_cap > 0 ? std::min<int64_t>(m_cap, T) : T);
  return salr::launch_moe_forward(a, cap, static_cast<hipStream_t>(stream)) == hipSuccess ? SALR_OK : SALR_ERR_HIP;
}

}  // extern "C"

// The forward behind both entry points: `ws` is the workspace (caller's, or
// the library's fixed array), `err` the word a timed-out wait sets.
int salr::forward_impl(const salr_layer_t* L, const uint16_t* X, int64_t M, uint16_t* Y, void* ws, size_t ws_bytes,
                       uint32_t* err_word, hipStream_t s) {
  if (!L) return SALR_ERR_INVALID_ARG;
  if (!dims_ok(L->N, L->K, L->n_keep, L->r_cat)) return SALR_ERR_INVALID_ARG;
  if (M < 0 || M > (int64_t(1) << 31) - 1) return SALR_ERR_INVALID_ARG;
  if (M == 0) return SALR_OK;
  if (!X || !Y || !L->masks || !L->offsets) return SALR_ERR_INVALID_ARG;
  if (L->value_format != SALR_VALUES_BF16 && L->value_format != SALR_VALUES_NF4) return SALR_ERR_INVALID_ARG;
  const bool nf4 = L->value_format == SALR_VALUES_NF4;
  if (!nf4 && L->n_keep > 0 && !L->values) return SALR_ERR_INVALID_ARG;
  if (nf4 && L->n_keep > 0 && (!L->codes || !L->scales)) return SALR_ERR_INVALID_ARG;
  if (L->r_cat > 0 && (!L->a_cat || !L->b_cat)) return SALR_ERR_INVALID_ARG;
  const void* ptrs[] = {X, Y, L->masks, nf4 ? nullptr : L->values, L->offsets, L->a_cat, L->b_cat,
                        nf4 ? L->codes : nullptr, nf4 ? L->scales : nullptr};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SALR_ERR_INVALID_ARG;
  if (static_cast<const void*>(X) == static_cast<const void*>(Y)) return SALR_ERR_INVALID_ARG;
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
  // (every argument check above comes before the workspace's)
  if (!ws || !aligned16(ws)) return SALR_ERR_WORKSPACE;
  const FwdLayout W = fwd_layout(L->N, L->K, L->n_keep, L->r_cat, M, r_win, nf4);
  if (ws_bytes < W.total) return SALR_ERR_WORKSPACE;
  const int32_t nblk = (int32_t)cdiv(L->n_keep, 64);

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
    a.err = err_word;
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
    a.err = err_word;
    a.ycount = at<uint32_t>(ws, kCounterY);
    a.ypart = at<uint64_t>(ws, W.ypart);
    if (nf4) {
      a.nf4 = 1;
      a.codes = L->codes;
      a.scales = L->scales;
      a.cb_row = nblk * 32;
      a.nblk = nblk;
      a.cofs = W.nf4_cofs;
      a.sofs = W.nf4_sofs;
    }
    err = salr::launch_fwd_small(a, s);
  } else {
    int t_splits = 0;
    if (L->r_cat > 0) {
      LowRankTArgs t{};
      t.X = X;
      t.a_cat = L->a_cat;
      t.tpart = at<float>(ws, W.ltpart);
      t.t16 = at<uint16_t>(ws, W.t16);
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
    // NF4: the values decoded to bf16 first (the many-row kernel is bound by
    // its matrix cores, not by the bytes of the values)
    const uint16_t* values = L->values;
    if (nf4) {
      uint16_t* dq = at<uint16_t>(ws, W.dq);
      if (salr::launch_dequantize_nf4(L->codes, L->scales, L->N, L->n_keep, dq, s) != hipSuccess) return SALR_ERR_HIP;
      values = dq;
    }
    LargeFwdArgs a{};
    a.masks = L->masks;
    a.values = values;
    a.b_cat = L->b_cat;
    a.X = X;
    a.tpart = L->r_cat > 0 ? at<float>(ws, W.ltpart) : nullptr;
    a.t16 = L->r_cat > 0 ? at<uint16_t>(ws, W.t16) : nullptr;
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
