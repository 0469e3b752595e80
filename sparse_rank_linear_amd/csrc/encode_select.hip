// SALR encode, selection and packing: per output row keep the n_keep
// entries of largest magnitude, write the bitmap, the packed values, the
// per-1024-column running counts and (optionally) the dense residual.
//
// Method: gist.science summary of "Sparsity-Aware Low-Rank Representation
// ...", Methodology 1 (static magnitude mask on the frozen weight),
// Methodology 2 (residual of the pruning) and Methodology 4 (bitmap plus a
// compact array of the kept values).
//
// Magnitude is the 15-bit key |bits| = bits & 0x7FFF, which orders bf16
// magnitudes exactly (and makes +0 and -0 equal).  One workgroup per row:
//   1. 256-bin histogram of key >> 7, pick the bin holding the n_keep-th
//      largest key;
//   2. 128-bin histogram of the low 7 bits inside that bin -> exact
//      threshold key t, count of keys > t, and the quota of keys == t that
//      are kept (the lowest columns first);
//   3. walk the row in 64-column words: wave ballots give "key > t" and
//      "key == t" masks; per-word counts are scanned across the row (in
//      segments of 256 words, carrying the totals) to get each tie's rank
//      and each kept value's slot; a second ballot gives the bitmap word and
//      mbcnt gives each kept lane's slot inside the word.
#include "salr_device.hpp"
#include "salr_kernels.hpp"

namespace salr {
namespace {

constexpr int kThreads = 256;
constexpr int kSegWords = 256;   // words scanned per segment

__device__ __forceinline__ uint32_t key_of(uint16_t b) { return b & 0x7FFFu; }

// Inclusive prefix sum of v over the 256 threads of the block (uses sh[256]).
__device__ __forceinline__ uint32_t block_scan_incl(uint32_t v, uint32_t* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int d = 1; d < kThreads; d <<= 1) {
    const uint32_t add = tid >= d ? sh[tid - d] : 0u;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  return sh[tid];
}

__global__ __launch_bounds__(kThreads) void prune_pack_kernel(PrunePackArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan_sh[kThreads];
  __shared__ uint32_t wtie[kSegWords], wgt[kSegWords];
  __shared__ uint32_t sel[4];  // threshold key, quota, bad flag
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int K = a.K;
  const uint16_t* w = a.W + row * K;

  // 1. coarse histogram + non-finite check
  hist[tid] = 0;
  if (tid == 0) sel[2] = 0;
  __syncthreads();
  bool bad = false;
  for (int c = tid; c < K; c += kThreads) {
    const uint16_t b = w[c];
    bad |= (b & 0x7F80u) == 0x7F80u;
    atomicAdd(&hist[key_of(b) >> 7], 1u);
  }
  if (bad) sel[2] = 1;
  __syncthreads();
  if (tid == 0) {
    uint32_t above = 0, b1 = 0;
    for (int b = 255; b >= 0; --b) {
      if (above + hist[b] >= (uint32_t)a.n_keep) { b1 = b; break; }
      above += hist[b];
    }
    sel[0] = b1;
    sel[1] = (uint32_t)a.n_keep - above;  // still needed from bin b1
  }
  __syncthreads();
  const uint32_t b1 = sel[0], need1 = sel[1];
  __syncthreads();

  // 2. fine histogram inside bin b1
  if (tid < 128) hist[tid] = 0;
  __syncthreads();
  for (int c = tid; c < K; c += kThreads) {
    const uint32_t k = key_of(w[c]);
    if ((k >> 7) == b1) atomicAdd(&hist[k & 127u], 1u);
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t above = 0, b2 = 0;
    for (int b = 127; b >= 0; --b) {
      if (above + hist[b] >= need1) { b2 = b; break; }
      above += hist[b];
    }
    sel[0] = (b1 << 7) | b2;     // threshold key
    sel[1] = need1 - above;      // ties at the threshold that are kept
  }
  __syncthreads();
  const uint32_t t = sel[0], quota = sel[1];
  if (tid == 0 && sel[2]) atomicOr(a.nonfinite, 1u);

  // 3. pack, one segment of kSegWords words at a time
  const int kw = a.kw;
  uint32_t tie_carry = 0, kept_carry = 0;
  for (int s0 = 0; s0 < kw; s0 += kSegWords) {
    const int nws = min(kSegWords, kw - s0);
    // 3a. per-word counts of "key > t" and "key == t"
    for (int wi = wave; wi < nws; wi += kThreads / 64) {
      const int col = (s0 + wi) * 64 + lane;
      const uint32_t k = col < K ? key_of(w[col]) : 0u;
      const bool live = col < K;
      const uint64_t gt = __ballot(live && k > t);
      const uint64_t eq = __ballot(live && k == t);
      if (lane == 0) {
        wgt[wi] = __popcll(gt);
        wtie[wi] = __popcll(eq);
      }
    }
    __syncthreads();
    // 3b. exclusive scans over the segment's words
    const uint32_t my_tie = tid < nws ? wtie[tid] : 0u;
    const uint32_t tie_incl = block_scan_incl(my_tie, scan_sh);
    const uint32_t tie_excl = tie_carry + tie_incl - my_tie;
    uint32_t my_kept = 0;
    if (tid < nws) {
      const uint32_t room = quota > tie_excl ? quota - tie_excl : 0u;
      my_kept = wgt[tid] + min(room, my_tie);
    }
    const uint32_t seg_ties = scan_sh[kThreads - 1];
    __syncthreads();
    const uint32_t kept_incl = block_scan_incl(my_kept, scan_sh);
    const uint32_t seg_kept = scan_sh[kThreads - 1];
    __syncthreads();
    if (tid < nws) {
      wtie[tid] = tie_excl;
      wgt[tid] = kept_carry + kept_incl - my_kept;  // first value slot of the word
    }
    __syncthreads();
    // 3c. bitmap words, values, offsets, residual
    for (int wi = wave; wi < nws; wi += kThreads / 64) {
      const int word = s0 + wi;
      const int col = word * 64 + lane;
      const bool live = col < K;
      const uint16_t b = live ? w[col] : (uint16_t)0;
      const uint32_t k = key_of(b);
      const uint64_t eq = __ballot(live && k == t);
      const uint32_t tie_rank = wtie[wi] + (uint32_t)__builtin_amdgcn_mbcnt_hi(
                                               (uint32_t)(eq >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)eq, 0u));
      const bool keep = live && (k > t || (k == t && tie_rank < quota));
      const uint64_t km = __ballot(keep);
      const uint32_t slot = wgt[wi] + (uint32_t)__builtin_amdgcn_mbcnt_hi(
                                          (uint32_t)(km >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)km, 0u));
      if (keep) a.values[row * a.n_keep + slot] = b;
      if (lane == 0) {
        a.masks[row * kw + word] = km;
        if ((word & 15) == 0) a.offsets[row * a.ng + (word >> 4)] = wgt[wi];
      }
      if (a.R && live) a.R[row * K + col] = keep ? (uint16_t)0 : b;
    }
    tie_carry += seg_ties;
    kept_carry += seg_kept;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_prune_pack(const PrunePackArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(prune_pack_kernel, dim3((unsigned)a.N), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace salr
