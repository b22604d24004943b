// Write path: block-diagonal Hadamard rotation + token-wise asymmetric INT4/INT2 quantization
// + packing + paged store, one fused kernel (SAW-INT4 abstract, fugumt.com paper page: a fused
// rotation-quantization kernel writing straight into a paged cache; OScaR summary, zhichai.net,
// "The OScaR Framework": Quant(S (R V)) with a per-token scale S).
//
// Mapping: a 16-lane row group owns one (token, head) and does both its K and its V vector;
// lane i holds channels 8i..8i+7 (one 16-byte bf16 load per tensor). A wave covers four
// consecutive tokens of one KV head and a 256-thread workgroup sixteen, so a page-aligned run of
// sixteen tokens - one page-head tile of the cache - is written by one workgroup, i.e. through
// one XCD's L2, which merges the V tile's byte-interleaved stores into whole lines before they
// reach HBM.
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {
namespace {

// Rotate, optionally scale per token, quantize and pack the 8 channels this lane holds (output
// block lf.pos of the rotated vector). Returns the packed codes (INT4: 32 bits, INT2: low 16
// bits); scale/zero are the stored values, identical in all 16 lanes of the group.
template <int BITS, bool TOKEN_SCALE>
__device__ __forceinline__ uint32_t rotate_quantize8(float (&x)[8], const RowFwhtPlan& rot, const LaneFwht& lf,
                                                     float& scale, float& zero) {
  fwht_row16_planned(x, rot, lf);

  float s = 1.0f;
  if constexpr (TOKEN_SCALE) {
    // RMS in double precision, rounded once to float (so the stored scale does not depend
    // on the summation order), 1 for an all-zero vector.
    double ss = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) ss += static_cast<double>(x[k]) * static_cast<double>(x[k]);
    ss = row16_sum_f64(ss);
    s = static_cast<float>(sqrt(ss * (1.0 / kHeadDim)));
    if (s == 0.0f) s = 1.0f;
    const float rs = 1.0f / s;
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = div_rn(x[k], s, rs);
  }

  float mn = fminf(fminf(fminf(x[0], x[1]), fminf(x[2], x[3])), fminf(fminf(x[4], x[5]), fminf(x[6], x[7])));
  float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  mn = row16_min(mn);
  mx = row16_max(mx);
  constexpr float kQmax = static_cast<float>((1 << BITS) - 1);
  const float delta = (mx - mn) / kQmax;  // IEEE division (the build uses correctly rounded f32 divide)

  uint32_t packed = 0;
  if (delta != 0.0f) {
    const float r = 1.0f / delta;
    float c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = fminf(fmaxf(rintf(div_rn(x[k] - mn, delta, r)), 0.0f), kQmax);
    if constexpr (BITS == 4) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
        packed = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(c[2 * m + 1], 16.0f, c[2 * m]), m, packed);
    } else {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const float b = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(c[4 * m + 3], 4.0f, c[4 * m + 2]), 4.0f,
                                                      c[4 * m + 1]), 4.0f, c[4 * m]);
        packed = __builtin_amdgcn_cvt_pk_u8_f32(b, m, packed);
      }
    }
  }
  scale = delta * s;
  zero = mn * s;
  return packed;
}

template <int BITS>
__device__ __forceinline__ void store_k(uint8_t* tile_row, int li, uint32_t packed) {
  if constexpr (BITS == 4) {
    *reinterpret_cast<uint32_t*>(tile_row + li * 4) = packed;
  } else {
    *reinterpret_cast<uint16_t*>(tile_row + li * 2) = static_cast<uint16_t>(packed);
  }
}

// V tile: byte j of token t at ((t / 4) * row + j) * 4 + t % 4.
template <int BITS>
__device__ __forceinline__ void store_v(uint8_t* tile, int off, int li, uint32_t packed) {
  constexpr int kRow = kHeadDim * BITS / 8;
  constexpr int kBytesPerLane = 8 * BITS / 8;
  uint8_t* base = tile + ((off >> 2) * kRow) * 4 + (off & 3);
#pragma unroll
  for (int m = 0; m < kBytesPerLane; ++m) {
    const int j = li * kBytesPerLane + m;
    base[j * 4] = static_cast<uint8_t>(packed >> (8 * m));
  }
}

template <int BITS, bool TOKEN_SCALE>
__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a) {
  constexpr int kRow = kHeadDim * BITS / 8;
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4;
  const int li = lane & 15;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 6) * 4 + grp;
  const int h = blockIdx.y;

  int64_t slot = -1;
  if (t < a.num_tokens) slot = a.slots[t];
  const bool live = slot >= 0 && slot < a.num_slots;

  uint4 kw = make_uint4(0, 0, 0, 0), vw = make_uint4(0, 0, 0, 0);
  if (live) {
    kw = *reinterpret_cast<const uint4*>(a.k + t * a.k_stride + h * kHeadDim + li * 8);
    vw = *reinterpret_cast<const uint4*>(a.v + t * a.v_stride + h * kHeadDim + li * 8);
  }
  float kx[8], vx[8];
  bf16x8_to_f32(kw, kx);
  bf16x8_to_f32(vw, vx);

  // Every lane runs the transform (the DPP exchanges need all 64 lanes); dead rows store nothing.
  const LaneFwht lf = lane_fwht(a.rot, li);
  float ks, kz, vs, vz;
  const uint32_t kp = rotate_quantize8<BITS, TOKEN_SCALE>(kx, a.rot, lf, ks, kz);
  const uint32_t vp = rotate_quantize8<BITS, TOKEN_SCALE>(vx, a.rot, lf, vs, vz);

  if (live) {
    const int64_t page = slot / a.page_size;
    const int off = static_cast<int>(slot - page * a.page_size);
    const int64_t tile_index = page * a.num_kv_heads + h;     // (page, head) tile
    const int64_t row_index = tile_index * a.page_size + off;  // (page, head, offset) row
    store_k<BITS>(a.k_codes + row_index * kRow, lf.pos, kp);
    store_v<BITS>(a.v_codes + tile_index * a.page_size * kRow, off, lf.pos, vp);
    if (li == 0) {
      reinterpret_cast<float2*>(a.k_sz)[row_index] = make_float2(ks, kz);
      reinterpret_cast<float2*>(a.v_sz)[row_index] = make_float2(vs, vz);
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((a.num_tokens + 15) / 16), static_cast<unsigned>(a.num_kv_heads));
  const dim3 block(256);
  if (a.bits == 4 && !a.token_scale) {
    hipLaunchKernelGGL((append_kernel<4, false>), grid, block, 0, stream, a);
  } else if (a.bits == 4) {
    hipLaunchKernelGGL((append_kernel<4, true>), grid, block, 0, stream, a);
  } else if (!a.token_scale) {
    hipLaunchKernelGGL((append_kernel<2, false>), grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL((append_kernel<2, true>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace kvq
