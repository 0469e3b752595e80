// Device-side building blocks shared by the SALR kernels (gfx950 / CDNA4).
//
// Matrix-core operand layouts used throughout (v_mfma_f32_16x16x32_bf16,
// wave64): for lane l, let i = l % 16 and g = l / 16.
//   A operand (16 x 32): lane holds A[i][8g .. 8g+7]      (8 bf16, 16 bytes)
//   B operand (32 x 16): lane holds B[8g .. 8g+7][i]      (8 bf16, 16 bytes)
//   D (16 x 16, fp32):   lane holds D[4g + e][i], e=0..3   (4 floats)
// Both inputs run along k inside a lane, so a row-major matrix with k
// contiguous loads straight into either operand.
//
// v_mfma_f32_32x32x16_bf16 (twice the work per instruction; in loops of
// independent instructions on MI355X it sustains 1.7x the 16x16x32 form's
// rate with four waves per SIMD and 2.5x with one): for lane l, let
// r = l % 32 and h = l / 32.
//   A operand (32 x 16): lane holds A[r][8h .. 8h+7]
//   B operand (16 x 32): lane holds B[8h .. 8h+7][r]
//   D (32 x 32, fp32):   element 4j + e of the lane is D[8j + 4h + e][r],
//                        j, e = 0..3
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "salr_kernels.hpp"

namespace salr {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// fp32 -> bf16 bit pattern, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// ---------------------------------------------------------------------------
// Nibble expansion: the core of the bitmap decode.
//
// Four consecutive columns whose keep-bits form the nibble q take their
// values, in order, from a packed stream u[0], u[1], ... (bf16).  Given the
// stream window e0 = u0 | u1<<16, e1 = u2 | u3<<16 (the 4 values from the
// group's first kept value on), the dense 4-column group is two v_perm_b32
// byte selections of {e1, e0}: column c reads u[popcount of q's bits below
// c] when its bit is set, and 0x00 bytes (selector 12) otherwise.
// nibble_selectors(q) gives the two selector words; kernels keep the 16
// entries in LDS.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x2_t nibble_selectors(uint32_t q) {
  uint32_t sel[4];
  uint32_t c = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if ((q >> s) & 1u) {
      sel[s] = (2u * c) | ((2u * c + 1u) << 8);
      ++c;
    } else {
      sel[s] = 0x0C0Cu;
    }
  }
  return u32x2_t{sel[0] | (sel[1] << 16), sel[2] | (sel[3] << 16)};
}

// Window of the 4 stream values starting at value index idx of a bf16
// stream in LDS, as two 32-bit words: three aligned words are read (one
// 8-byte read of an even word pair plus one word; unaligned 8-byte LDS reads
// are correct on CDNA but slower) and a funnel shift drops an odd leading
// value.  Words past the live values may be read; they are never selected.
struct Window3 {
  uint32_t d0, d1, d2;
};
__device__ __forceinline__ Window3 lds_window_words(const uint16_t* vals, uint32_t idx) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(vals) + (idx >> 1);
  return Window3{w[0], w[1], w[2]};
}
__device__ __forceinline__ u32x2_t window_values(Window3 w, uint32_t idx) {
  const uint32_t sh = (idx & 1u) << 4;
  return u32x2_t{__builtin_amdgcn_alignbit(w.d1, w.d0, sh), __builtin_amdgcn_alignbit(w.d2, w.d1, sh)};
}

// Dense 4-column group from the window of the 4 stream values starting at the
// group's first kept value.
__device__ __forceinline__ u32x2_t expand_nibble(u32x2_t win, u32x2_t sel) {
  return u32x2_t{__builtin_amdgcn_perm(win.y, win.x, sel.x), __builtin_amdgcn_perm(win.y, win.x, sel.y)};
}

// Dense 8-column group (one MFMA operand slice) for keep-bits `byte` whose
// first kept value is stream index `idx` (two windows: one per nibble).
__device__ __forceinline__ u32x4_t expand_byte(const uint16_t* vals, uint32_t idx, uint32_t byte, const u32x2_t* lut) {
  const uint32_t lo = byte & 15u, hi = byte >> 4;
  const uint32_t idx2 = idx + __builtin_popcount(lo);
  const u32x2_t a = expand_nibble(window_values(lds_window_words(vals, idx), idx), lut[lo]);
  const u32x2_t b = expand_nibble(window_values(lds_window_words(vals, idx2), idx2), lut[hi]);
  return u32x4_t{a.x, a.y, b.x, b.y};
}

// ---------------------------------------------------------------------------
// Passing data between workgroups of one launch.
//
// On a multi-die GPU an agent-scope fence writes back or invalidates the
// whole L2 of the die, which is far too slow to do per workgroup.  So no
// such fence is used.  Instead every word one workgroup hands to another is
// a 64-bit "tagged" word: 32 data bits and, in the high half, the launch's
// tag, written with one device-coherent 64-bit store.  Readers poll each
// word with device-coherent loads until its tag equals the current launch's
// tag, so they can never consume a stale or torn value, whatever order the
// stores become visible in.  Counters (device-coherent atomics) only elect
// which workgroup performs a reduction; they order nothing.
//
// The tag comes from kTicketGroups 64-bit ticket words {count (low half),
// epoch (high half)} in the workspace, one per group of workgroups (wg mod
// kTicketGroups), each in its own 256-byte slot so that draws on different
// words do not queue behind each other.  Every workgroup adds 1 to its
// group's word as it starts; its tag is the returned epoch + 1.  The
// workgroup that draws its group's last ticket folds the count into an epoch
// increment, and workgroup 0 advances the words of groups that have no
// members in this launch, so every word's epoch advances exactly once per
// launch and all groups agree on the tag; the next launch (stream-ordered
// after this one) runs with the next tag.  All of this happens while the
// loads of the launch's start are in flight; nothing is left to do when
// workgroups finish.
// ---------------------------------------------------------------------------
constexpr uint32_t kSpinLimit = 1u << 22;

__device__ __forceinline__ uint32_t atomic_add_relaxed(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t atomic_add_relaxed64(uint64_t* p, uint64_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_coherent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_tagged(uint64_t* p, uint32_t data, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | data, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_tagged_raw(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until all n (<= 4) consecutive tagged words at p carry `tag`; return
// their data halves.  Bounded: after kSpinLimit polls the error word is set
// and the (stale) data returned, so a kernel can never hang here.
template <int n>
__device__ __forceinline__ void poll_tagged(const uint64_t* p, uint32_t tag, uint32_t (&out)[n], uint32_t* err) {
  uint32_t spins = 0;
  while (true) {
    bool ok = true;
#pragma unroll
    for (int k = 0; k < n; ++k) {
      const uint64_t v = load_tagged_raw(p + k);
      out[k] = (uint32_t)v;
      ok &= (uint32_t)(v >> 32) == tag;
    }
    if (ok) return;
    if (++spins >= kSpinLimit) {
      store_coherent(err, 1u);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Draw workgroup wg's ticket (one lane; see above).
__device__ __forceinline__ uint64_t draw_ticket(uint64_t* tickets, uint32_t wg, uint32_t n_wgs) {
  if (wg == 0)
    for (uint32_t g = n_wgs; g < kTicketGroups; ++g)
      atomic_add_relaxed64(tickets + g * kTicketStride, uint64_t(1) << 32);
  return atomic_add_relaxed64(tickets + (wg % kTicketGroups) * kTicketStride, 1);
}
// The launch tag from a drawn ticket; the drawer of its group's last ticket
// also advances the group's epoch.  The lane that drew calls this.
__device__ __forceinline__ uint32_t tag_from_ticket(uint64_t* tickets, uint64_t drawn, uint32_t wg, uint32_t n_wgs) {
  const uint32_t g = wg % kTicketGroups;
  const uint32_t gsize = n_wgs / kTicketGroups + (g < n_wgs % kTicketGroups ? 1u : 0u);
  if ((uint32_t)drawn == gsize - 1u) atomic_add_relaxed64(tickets + g * kTicketStride, (uint64_t(1) << 32) - gsize);
  return (uint32_t)(drawn >> 32) + 1u;
}

// Workgroup barrier that waits for the wave's LDS operations but not for its
// outstanding global ones (__syncthreads waits for both, which would also
// wait for direct-to-LDS loads meant to stay in flight across it).
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ u32x4_t load16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ u32x4_t zero_u4() { return u32x4_t{0u, 0u, 0u, 0u}; }

}  // namespace salr
