// Matrix-core building blocks shared by the low-bit read paths (the token-wise decode and the
// per-channel decode): operand construction from packed codes, the bf16 hi/lo split of
// softmax weights, wave-level helpers. Device code only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

inline constexpr float kNegInf = -__builtin_inff();

// Page table and context lengths are read-only for the whole call: reading them through the
// constant address space lets the compiler use scalar loads (waited on with lgkmcnt), so looking
// up the next pages never waits for the tile loads already in flight (vmcnt).
typedef __attribute__((address_space(4))) const int32_t const_i32;
__device__ __forceinline__ int32_t ro_load(const int32_t* p, int64_t i) {
  return ((const_i32*)(p))[i];
}

// Maximum over the four 16-lane rows (lanes n, n+16, n+32, n+48), in every lane: gfx950's row
// swaps exchange rows 0<->1, 2<->3 and then the two halves, without going through LDS.
__device__ __forceinline__ float max_over_rows(float v) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Maximum of two values that are finite or -inf (scores), as the median of (a, b, +inf): one
// instruction, where fmaxf of values fresh from a lane exchange first quiets both operands.
__device__ __forceinline__ float max_nc(float a, float b) {
  return __builtin_amdgcn_fmed3f(a, b, __builtin_inff());
}

// max_over_rows for scores (finite or -inf).
__device__ __forceinline__ float max_over_rows_nc(float v) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max_nc(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_nc(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

__device__ __forceinline__ float min_over_rows(float v) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fminf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fminf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Orders this wave's LDS writes before its later LDS reads (one-wave workgroups: no s_barrier,
// and no wait on the global loads in flight).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
inline constexpr float kLazyRescale = 8.0f;  // log2 units
__device__ __forceinline__ v8bf as_bf(v4u x) { return __builtin_bit_cast(v8bf, x); }

// V operand values: bf16(B + c). For INT4, B = 16 (bits 0x4180) and c sits at mantissa bits
// 3..6 of the low byte; for INT2, B = 4 (bits 0x4080) and c sits at bits 5..6.
template <int BITS> struct VBias;
template <> struct VBias<4> {
  static constexpr float value = 16.0f;
  static constexpr uint32_t high_bytes = 0x41414141u;
};
template <> struct VBias<2> {
  static constexpr float value = 4.0f;
  static constexpr uint32_t high_bytes = 0x40404040u;
};

// Low bytes (0x80 | c << shift) of four tokens -> two dwords of bf16 (B + c), tokens in byte order.
template <int BITS>
__device__ __forceinline__ uint32_t bias_bf16_lo(uint32_t lo_bytes) {
  return __builtin_amdgcn_perm(lo_bytes, VBias<BITS>::high_bytes, 0x00050004u);
}
template <int BITS>
__device__ __forceinline__ uint32_t bias_bf16_hi(uint32_t lo_bytes) {
  return __builtin_amdgcn_perm(lo_bytes, VBias<BITS>::high_bytes, 0x00070006u);
}

// Split four floats into bf16 hi (truncated) + lo (rounded remainder), packed in pairs.
__device__ __forceinline__ void split_bf16(const float (&w)[4], uint32_t& hi01, uint32_t& hi23, uint32_t& lo01,
                                           uint32_t& lo23) {
  uint32_t hb[4];
  float lf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hb[i] = __float_as_uint(w[i]) & 0xFFFF0000u;
    lf[i] = w[i] - __uint_as_float(hb[i]);
  }
  hi01 = __builtin_amdgcn_perm(hb[1], hb[0], 0x07060302u);
  hi23 = __builtin_amdgcn_perm(hb[3], hb[2], 0x07060302u);
  // the remainders rounded to bf16 two at a time (one packed conversion per pair)
  lo01 = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){lf[0], lf[1]}, v2bf));
  lo23 = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){lf[2], lf[3]}, v2bf));
}

// K-code operand of one tile for MFMA j from the bytes this lane loaded (32 channels of one token).
template <int BITS>
__device__ __forceinline__ v4i k_operand(const uint4 w, int j) {
  v4i a;
  if constexpr (BITS == 4) {
    const uint32_t w0 = j ? w.z : w.x, w1 = j ? w.w : w.y;
    a[0] = static_cast<int>(w0 & 0x0F0F0F0Fu);
    a[1] = static_cast<int>((w0 >> 4) & 0x0F0F0F0Fu);
    a[2] = static_cast<int>(w1 & 0x0F0F0F0Fu);
    a[3] = static_cast<int>((w1 >> 4) & 0x0F0F0F0Fu);
  } else {
    const uint32_t w0 = j ? w.y : w.x;
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = static_cast<int>((w0 >> (2 * r)) & 0x03030303u);
  }
  return a;
}

// Channel 8n + m of the four tokens of this lane group as bf16 low bytes 0x80 | c << shift
// (shift 3 for INT4, 5 for INT2), one token per byte. `c80` holds 0x80808080 in a VGPR, so each
// byte costs two VOP3 operations (shift/mask + or) instead of three.
template <int BITS>
__device__ __forceinline__ uint32_t v_bf16_low_bytes(const uint4 w, int m, uint32_t c80) {
  if constexpr (BITS == 4) {
    const uint32_t d = (m >> 1) == 0 ? w.x : (m >> 1) == 1 ? w.y : (m >> 1) == 2 ? w.z : w.w;
    if (m & 1) return ((d >> 1) & 0x78787878u) | c80;  // high nibble: bits 4..7 -> 3..6
    return ((d & 0x0F0F0F0Fu) << 3) | c80;              // low nibble: bits 0..3 -> 3..6
  } else {
    const uint32_t d = (m >> 2) ? w.y : w.x;
    const int sh = 2 * (m & 3);  // crumb position; target bits 5..6
    if (sh == 0) return ((d & 0x03030303u) << 5) | c80;
    return (((sh <= 5) ? (d << (5 - sh)) : (d >> (sh - 5))) & 0x60606060u) | c80;
  }
}

// A constant kept in a VGPR (the empty register-only asm makes it opaque to the compiler).
__device__ __forceinline__ uint32_t vgpr_const(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Buffer resource over one page-head tile (base and size are wave-uniform, so they live in
// SGPRs; loads outside the tile would return zero). The last word is the raw-buffer format used
// for untyped loads on CDNA.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

}  // namespace kvq
