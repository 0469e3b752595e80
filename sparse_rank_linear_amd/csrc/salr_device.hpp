// Device-side building blocks shared by the SALR kernels (gfx950 / CDNA4).
//
// Matrix-core operand layouts used throughout (v_mfma_f32_16x16x32_bf16,
// wave64): for lane l, let i = l % 16 and g = l / 16.
//   A operand (16 x 32): lane holds A[i][8g .. 8g+7]      (8 bf16, 16 bytes)
//   B operand (32 x 16): lane holds B[8g .. 8g+7][i]      (8 bf16, 16 bytes)
//   D (16 x 16, fp32):   lane holds D[4g + e][i], e=0..3   (4 floats)
// Both inputs run along k inside a lane, so a row-major matrix with k
// contiguous loads straight into either operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace salr {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
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
// stream window e0 = u0 | u1<<16, e1 = u2 | u3<<16, the dense 4-column group
// is two v_perm_b32 byte selections of {e1, e0}: column c reads u[popcount
// of q's bits below c] when its bit is set, and 0x00 bytes (selector 12)
// otherwise.  nibble_selectors(q) gives the two selector words; kernels keep
// the 16 entries in LDS.
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

// Dense 4-column group from packed values starting at value index `idx` of a
// row buffer in LDS (`buf32` = the buffer as 32-bit words, 4-byte aligned).
// Reads three words at the word holding value idx; a funnel shift drops the
// odd leading value.  Words past the live values may be read; they are never
// selected because their keep-bits are clear.
__device__ __forceinline__ u32x2_t expand_nibble(const uint32_t* buf32, uint32_t idx, u32x2_t sel) {
  const uint32_t w = idx >> 1;
  const uint32_t sh = (idx & 1u) << 4;
  const uint32_t d0 = buf32[w], d1 = buf32[w + 1], d2 = buf32[w + 2];
  const uint32_t e0 = __builtin_amdgcn_alignbit(d1, d0, sh);
  const uint32_t e1 = __builtin_amdgcn_alignbit(d2, d1, sh);
  return u32x2_t{__builtin_amdgcn_perm(e1, e0, sel.x), __builtin_amdgcn_perm(e1, e0, sel.y)};
}

// Dense 8-column group (one MFMA operand slice) for byte pattern `byte` whose
// first kept value is stream index `idx`.
__device__ __forceinline__ u32x4_t expand_byte(const uint32_t* buf32, uint32_t idx, uint32_t byte,
                                               const u32x2_t* lut) {
  const uint32_t lo = byte & 15u, hi = byte >> 4;
  const u32x2_t a = expand_nibble(buf32, idx, lut[lo]);
  const u32x2_t b = expand_nibble(buf32, idx + __builtin_popcount(lo), lut[hi]);
  return u32x4_t{a.x, a.y, b.x, b.y};
}

// ---------------------------------------------------------------------------
// Agent-scope synchronisation between workgroups of one launch.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t atomic_add_acq_rel(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_load_acquire(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_release(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ u32x4_t load16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ u32x4_t zero_u4() { return u32x4_t{0u, 0u, 0u, 0u}; }

}  // namespace salr
