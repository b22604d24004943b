// The block-diagonal Hadamard rotation of 16 tokens on the matrix cores, shared by the write
// paths (the token-wise append and the per-channel page writer). The inputs are bf16 and the
// entries of R are +-1 (or 0) times a power of two, so the operands are exact in bf16 and the
// products accumulate in float32 (the bookkeeping of channels, k-steps and operand tables is
// described in kvq_append.hip). Device code only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_device.h"
#include "kvq_mfma.h"

namespace kvq {

// Factor of the block-diagonal Sylvester matrix (blocks of 2^LB) for bit position p, input bit a,
// output bit o.
template <int LB>
__host__ __device__ constexpr int bit_factor(int p, int a, int o) {
  return (p < LB) ? (((a & o) != 0) ? -1 : 1) : (a == o ? 1 : 0);
}

// Sign (+1 / -1) or absence (0) of k-step s in the MFMA of output tile n: bits 0 and 1.
template <int LB>
__host__ __device__ constexpr int step_sign(int s, int n) {
  return bit_factor<LB>(0, s & 1, n & 1) * bit_factor<LB>(1, (s >> 1) & 1, (n >> 1) & 1);
}

// 1/sqrt(b) splits into 2^-(LB/2), folded into the B operand exactly, times 1/sqrt(2) for odd LB.
template <int LB>
constexpr uint32_t b_entry(int f) {
  constexpr uint32_t exp_bits = 127u - static_cast<uint32_t>(LB / 2);  // bf16 exponent of 2^-(LB/2)
  return f == 0 ? 0u : (((f < 0) ? 0x8000u : 0u) | (exp_bits << 7));
}

// B operand for the output tiles with n >> 2 == n2: lane (G, c) holds rows k = 8G + r, r = 2q + e.
template <int LB>
constexpr uint32_t b_word(int lane, int n2, int q) {
  const int G = lane >> 4, c = lane & 15;
  const int f = bit_factor<LB>(3, G & 1, c & 1) * bit_factor<LB>(4, G >> 1, (c >> 1) & 1) *
                bit_factor<LB>(5, q & 1, (c >> 2) & 1) * bit_factor<LB>(6, q >> 1, c >> 3);
  return b_entry<LB>(f * bit_factor<LB>(2, 0, n2)) | (b_entry<LB>(f * bit_factor<LB>(2, 1, n2)) << 16);
}

// All B operands, built at compile time: [n2][lane][q] for each block size.
template <int LB>
struct BTable {
  uint32_t w[2][64][4];
  constexpr BTable() : w() {
    for (int n2 = 0; n2 < 2; ++n2)
      for (int l = 0; l < 64; ++l)
        for (int q = 0; q < 4; ++q) w[n2][l][q] = b_word<LB>(l, n2, q);
  }
};
template <int LB>
__device__ constexpr BTable<LB> kBTable{};

template <int LB>
__device__ __forceinline__ v4u load_b(int lane, int n2) {
  const uint4 x = *reinterpret_cast<const uint4*>(kBTable<LB>.w[n2][lane]);
  return v4u{x.x, x.y, x.z, x.w};
}

// A operand of k-step s from the four 16-byte loads of one token (load q holds input channels
// 32q + 8G + 0..7): register q = {channel s, channel s + 4} of load q.
__device__ __forceinline__ v4u make_a(const uint4 (&x)[4], int s) {
  const uint32_t sel = (s & 1) ? 0x07060302u : 0x05040100u;
  v4u a;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t d[4] = {x[q].x, x[q].y, x[q].z, x[q].w};
    a[q] = __builtin_amdgcn_perm(d[(s >> 1) + 2], d[s >> 1], sel);
  }
  return a;
}

// y[n][i] = (R x)[token 4G + i][channel 8c + n] for the wave's 16 tokens (before 1/sqrt(2)).
template <int LB>
__device__ __forceinline__ void rotate_tile(const uint4 (&x)[4], const v4u (&bop)[2], v4f (&y)[8]) {
  v4u a[4], na[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    a[s] = make_a(x, s);
    na[s] = a[s] ^ v4u{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    y[n] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int sg = step_sign<LB>(s, n);
      if (sg > 0) y[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a[s]), as_bf(bop[n >> 2]), y[n], 0, 0, 0);
      if (sg < 0) y[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(na[s]), as_bf(bop[n >> 2]), y[n], 0, 0, 0);
    }
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Value of quad lane I (every quad holds the same per-token values in its lane I).
template <int I>
__device__ __forceinline__ float quad_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), I * 0x55, 0xF, 0xF, true));
}

template <typename T>
__device__ __forceinline__ T pick4(int i, T v0, T v1, T v2, T v3) {
  return i == 0 ? v0 : i == 1 ? v1 : i == 2 ? v2 : v3;
}

// V words of four consecutive tokens: word jj = byte jj of tokens 0, 1, 2, 3 (a 4x4 byte transpose).
__device__ __forceinline__ uint4 interleave4(const uint32_t (&p)[4]) {
  const uint32_t x01_lo = __builtin_amdgcn_perm(p[1], p[0], 0x05010400u);
  const uint32_t x01_hi = __builtin_amdgcn_perm(p[1], p[0], 0x07030602u);
  const uint32_t x23_lo = __builtin_amdgcn_perm(p[3], p[2], 0x05010400u);
  const uint32_t x23_hi = __builtin_amdgcn_perm(p[3], p[2], 0x07030602u);
  return make_uint4(__builtin_amdgcn_perm(x23_lo, x01_lo, 0x05040100u), __builtin_amdgcn_perm(x23_lo, x01_lo, 0x07060302u),
                    __builtin_amdgcn_perm(x23_hi, x01_hi, 0x05040100u), __builtin_amdgcn_perm(x23_hi, x01_hi, 0x07060302u));
}

}  // namespace kvq
