// Per-channel page writer: the per-channel reading of OScaR (OScaR abstract on the openalex
// page: the rotation and the per-token scaling let the per-channel quantization paradigm hold up
// under extreme compression; zhichai.net summary, "Root Cause: Token Norm Imbalance" and "The
// OScaR Framework": V-hat = Quant(S (R V))), a whole page at a time. Each token of the page is
// rotated (y = R x), divided by its RMS s (u = y / s, so every token has unit RMS), and the page's
// ps normalised tokens share one asymmetric (scale, zero) per channel:
//   scale_c = (max_t u_tc - min_t u_tc) / qmax,  zero_c = min_t u_tc,
//   code_tc = clamp(rint((u_tc - zero_c) / scale_c), 0, qmax).
// Stored: codes (in the token-wise cache's layout), s per token, (scale, zero) per channel.
//
// The rotation runs on the matrix cores as in the token-wise append (kvq_rotate_mfma.h): one
// workgroup per (input page, KV head), one wave per 16-token tile of the page, K and V in the
// same wave. Lane (G, c) ends with channels 8c .. 8c + 7 of tokens 4G .. 4G + 3 of its tile; a
// token's RMS is a 16-lane row sum, a channel's minimum and maximum run over the lane's four
// tokens, the four row groups (row swaps) and the page's waves (LDS). Divisions are Markstein-
// corrected (bit-exact with IEEE division) on a fast path that every ordinary page takes.
#include "kvq_device.h"
#include "kvq_launch.h"
#include "kvq_mfma.h"
#include "kvq_rotate_mfma.h"

namespace kvq {
namespace {

constexpr float kPcFastMinScale = 0x1p-100f;  // below this (or 0) a channel takes the guarded path

template <int BITS>
__device__ __forceinline__ void pc_quantize_tile(v4f (&y)[8], bool odd_lb, int c, int G, int wave, int waves,
                                                 float (&mm)[kPcMaxPage / 16][2][kHeadDim], uint32_t (&packed)[4],
                                                 float (&s)[4], float (&delta)[8], float (&zero)[8]) {
  constexpr float kQmax = static_cast<float>((1 << BITS) - 1);
  if (odd_lb) {
    constexpr float kInvSqrt2 = 0.70710678118654752440f;
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) y[n][i] *= kInvSqrt2;
  }
  // u = y / s per token, s = RMS (double precision across the 16-lane row, rounded once). The row
  // sums are equal in the row's 16 lanes, so lane c takes the square root and the reciprocal of
  // token c & 3 only and the quads broadcast them.
  double ss[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    double v = 0.0;
#pragma unroll
    for (int n = 0; n < 8; ++n) v += static_cast<double>(y[n][i]) * static_cast<double>(y[n][i]);
    ss[i] = row16_sum_f64(v);
  }
  float s_own = static_cast<float>(sqrt(pick4(c & 3, ss[0], ss[1], ss[2], ss[3]) * (1.0 / kHeadDim)));
  if (s_own == 0.0f) s_own = 1.0f;
  const bool plain_own = s_own >= 0x1p-100f && s_own <= 0x1p100f;
  const float rs_own = rcp_rn(plain_own ? s_own : 1.0f);
  s[0] = quad_bcast<0>(s_own);
  s[1] = quad_bcast<1>(s_own);
  s[2] = quad_bcast<2>(s_own);
  s[3] = quad_bcast<3>(s_own);
  // every token of the wave is some lane's own token
  if (__builtin_expect(__all(plain_own), 1)) {
    const float rs[4] = {quad_bcast<0>(rs_own), quad_bcast<1>(rs_own), quad_bcast<2>(rs_own), quad_bcast<3>(rs_own)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int n = 0; n < 8; ++n) y[n][i] = div_rn(y[n][i], s[i], rs[i]);
    }
  } else {
    // an extreme s and y are first brought near 1 by the same power of two (exact), so that the
    // reciprocal stays a normal number
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float m2 = (s[i] < 0x1p-100f) ? 0x1p100f : ((s[i] > 0x1p100f) ? 0x1p-100f : 1.0f);
      const float sm = s[i] * m2;
      const float rs = 1.0f / sm;
#pragma unroll
      for (int n = 0; n < 8; ++n) y[n][i] = div_rn(y[n][i] * m2, sm, rs);
    }
  }
  // minimum and maximum of channel 8c + n over the tile (four tokens in-lane, the four row groups)
  float mn[8], mx[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    mn[n] = min_over_rows(fminf(fminf(y[n][0], y[n][1]), fminf(y[n][2], y[n][3])));
    mx[n] = max_over_rows(fmaxf(fmaxf(y[n][0], y[n][1]), fmaxf(y[n][2], y[n][3])));
  }
  // ... and over the page's tiles
  if (G == 0) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      mm[wave][0][8 * c + n] = mn[n];
      mm[wave][1][8 * c + n] = mx[n];
    }
  }
  __syncthreads();
  for (int w = 0; w < waves; ++w) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      mn[n] = fminf(mn[n], mm[w][0][8 * c + n]);
      mx[n] = fmaxf(mx[n], mm[w][1][8 * c + n]);
    }
  }
  __syncthreads();  // the LDS block is reused by the next tensor
  // scale RN(d / qmax) by the correction step with RN(1 / qmax) (equal to IEEE division for every
  // normal d); codes by the corrected quotient, rint without clamp (q <= qmax (1 + 2^-23))
  constexpr float kInvQmax = 1.0f / kQmax;
  // |u| <= sqrt(128) (unit RMS), so a scale is below 2^5 and the fast reciprocal holds
  float r[8];
  bool fast = true;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    delta[n] = div_rn(mx[n] - mn[n], kQmax, kInvQmax);
    zero[n] = mn[n];
    fast = fast && delta[n] >= kPcFastMinScale;
  }
  if (__builtin_expect(__all(fast), 1)) {
#pragma unroll
    for (int n = 0; n < 8; ++n) r[n] = rcp_rn(delta[n]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float cd[8];
#pragma unroll
      for (int n = 0; n < 8; ++n) cd[n] = div_rn(y[n][i] - mn[n], delta[n], r[n]);
      packed[i] = pack_codes<BITS>(cd);
    }
  } else {
    // guarded path: IEEE division, the clamp, zero codes for a constant channel
#pragma unroll
    for (int n = 0; n < 8; ++n) delta[n] = (mx[n] - mn[n]) / kQmax;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float cd[8];
#pragma unroll
      for (int n = 0; n < 8; ++n)
        cd[n] = (delta[n] != 0.0f) ? fminf(fmaxf(rintf((y[n][i] - mn[n]) / delta[n]), 0.0f), kQmax) : 0.0f;
      uint32_t p = 0;
      if constexpr (BITS == 4) {
#pragma unroll
        for (int m = 0; m < 4; ++m) p = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(cd[2 * m + 1], 16.0f, cd[2 * m]), m, p);
      } else {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const float bv = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(cd[4 * m + 3], 4.0f, cd[4 * m + 2]), 4.0f,
                                                         cd[4 * m + 1]), 4.0f, cd[4 * m]);
          p = __builtin_amdgcn_cvt_pk_u8_f32(bv, m, p);
        }
      }
      packed[i] = p;
    }
  }
}

template <int BITS, int LB>
__global__ __launch_bounds__(64 * (kPcMaxPage / 16)) void pc_write_mfma_kernel(const PcWriteArgs a) {
  constexpr int kRow = kHeadDim * BITS / 8;
  constexpr int kLaneBytes = 8 * BITS / 8;
  __shared__ float mm[kPcMaxPage / 16][2][kHeadDim];
  // workgroups numbered head-fastest: the ones that run together read whole token rows (all heads)
  const int ip = static_cast<int>(blockIdx.x / static_cast<uint32_t>(a.num_kv_heads));
  const int h = static_cast<int>(blockIdx.x % static_cast<uint32_t>(a.num_kv_heads));
  const int32_t page = a.page_ids[ip];
  if (page < 0 || page >= a.num_pages) return;  // uniform per workgroup
  const int ps = a.page_size;
  const int waves = ps / 16;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = lane >> 4, c = lane & 15;
  const v4u bop[2] = {load_b<LB>(lane, 0), load_b<LB>(lane, 1)};
  // lane (G, c) loads bytes 64q + 16G of token c of the tile (input channels 32q + 8G + 0..7)
  const int64_t tok = static_cast<int64_t>(ip) * ps + 16 * wave + c;
  uint4 kx[4], vx[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    kx[q] = *reinterpret_cast<const uint4*>(a.k + tok * a.k_stride + h * kHeadDim + 8 * G + 32 * q);
    vx[q] = *reinterpret_cast<const uint4*>(a.v + tok * a.v_stride + h * kHeadDim + 8 * G + 32 * q);
  }
  __builtin_amdgcn_sched_barrier(0);  // issue every load before any arithmetic
  uint32_t kp[4], vp[4];
  float ks[4], vs[4], kd[8], kz[8], vd[8], vz[8];
  {
    v4f y[8];
    rotate_tile<LB>(kx, bop, y);
    pc_quantize_tile<BITS>(y, (LB & 1) != 0, c, G, wave, waves, mm, kp, ks, kd, kz);
  }
  {
    v4f y[8];
    rotate_tile<LB>(vx, bop, y);
    pc_quantize_tile<BITS>(y, (LB & 1) != 0, c, G, wave, waves, mm, vp, vs, vd, vz);
  }
  // stores: token rows (page, head, 16 wave + 4G + i); codes as in the token-wise cache
  const int64_t tile = static_cast<int64_t>(page) * a.num_kv_heads + h;
  const int64_t row0 = tile * ps + 16 * wave + 4 * G;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint8_t* kdst = a.k_codes + (row0 + i) * kRow + kLaneBytes * c;
    if constexpr (BITS == 4) {
      *reinterpret_cast<uint32_t*>(kdst) = kp[i];
    } else {
      *reinterpret_cast<uint16_t*>(kdst) = static_cast<uint16_t>(kp[i]);
    }
    if (c == i) a.k_s[row0 + i] = ks[i];
    if (c == 4 + i) a.v_s[row0 + i] = vs[i];
  }
  {
    uint8_t* vdst = a.v_codes + row0 * kRow + 4 * kLaneBytes * c;  // the four tokens' interleaved words
    const uint4 w = interleave4(vp);
    if constexpr (BITS == 4) {
      *reinterpret_cast<uint4*>(vdst) = w;
    } else {
      *reinterpret_cast<uint2*>(vdst) = make_uint2(w.x, w.y);
    }
  }
  if (wave == 0 && G == 0) {  // the page's channel parameters, 8 channels per lane
    float4* kc = reinterpret_cast<float4*>(a.k_cp + tile * 2 * kHeadDim);
    float4* vc = reinterpret_cast<float4*>(a.v_cp + tile * 2 * kHeadDim);
    kc[2 * c] = make_float4(kd[0], kd[1], kd[2], kd[3]);
    kc[2 * c + 1] = make_float4(kd[4], kd[5], kd[6], kd[7]);
    kc[32 + 2 * c] = make_float4(kz[0], kz[1], kz[2], kz[3]);
    kc[32 + 2 * c + 1] = make_float4(kz[4], kz[5], kz[6], kz[7]);
    vc[2 * c] = make_float4(vd[0], vd[1], vd[2], vd[3]);
    vc[2 * c + 1] = make_float4(vd[4], vd[5], vd[6], vd[7]);
    vc[32 + 2 * c] = make_float4(vz[0], vz[1], vz[2], vz[3]);
    vc[32 + 2 * c + 1] = make_float4(vz[4], vz[5], vz[6], vz[7]);
  }
}

template <int BITS>
hipError_t launch_pc_write_mfma(const PcWriteArgs& a, int lb, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.num_input_pages) * static_cast<unsigned>(a.num_kv_heads));
  const dim3 block(static_cast<unsigned>(64 * (a.page_size / 16)));
  switch (lb) {
    case 0: hipLaunchKernelGGL((pc_write_mfma_kernel<BITS, 0>), grid, block, 0, stream, a); break;
    case 1: hipLaunchKernelGGL((pc_write_mfma_kernel<BITS, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((pc_write_mfma_kernel<BITS, 2>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((pc_write_mfma_kernel<BITS, 3>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((pc_write_mfma_kernel<BITS, 4>), grid, block, 0, stream, a); break;
    case 5: hipLaunchKernelGGL((pc_write_mfma_kernel<BITS, 5>), grid, block, 0, stream, a); break;
    case 6: hipLaunchKernelGGL((pc_write_mfma_kernel<BITS, 6>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((pc_write_mfma_kernel<BITS, 7>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pc_write(const PcWriteArgs& a, hipStream_t stream) {
  int lb = 0;
  while ((1 << lb) < a.rot.hb) ++lb;
  return a.bits == 4 ? launch_pc_write_mfma<4>(a, lb, stream) : launch_pc_write_mfma<2>(a, lb, stream);
}

}  // namespace kvq
