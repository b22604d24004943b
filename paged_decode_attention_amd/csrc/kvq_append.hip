// Write path: block-diagonal Hadamard rotation + token-wise asymmetric INT4/INT2 quantization
// + packing + paged store, one fused kernel (SAW-INT4 abstract, fugumt.com paper page: a fused
// rotation-quantization kernel writing straight into a paged cache; OScaR summary, zhichai.net,
// "The OScaR Framework": Quant(S (R V)) with a per-token scale S).
//
// One wave rotates and quantizes 16 consecutive tokens of one KV head, K and V. The rotation
// y = R x is a dense contraction over the 128 channels, done on the matrix cores
// (v_mfma_f32_16x16x32_bf16): the bf16 inputs and the +-1 (or 0) entries of R are exact bf16
// operands, and the products accumulate in float32.
//
// Channel bookkeeping. Input channel m = s + 4 e + 8 G + 32 q (s: MFMA k-step 0..3, e: 0..1,
// G: lane row 0..3, q: 16-byte load 0..3) and output channel o = n + 8 c (n: MFMA 0..7, c: lane
// column 0..15). For the Sylvester matrix, H[m][o] is a product over the seven bit positions:
// inside a block of b = 2^LB channels each bit contributes (-1)^(m_p o_p), outside it the
// block-diagonal structure asks m_p == o_p. Bits 0-1 pair s with n, so that factor is uniform
// over the wave and becomes the sign (or absence) of a whole k-step; bit 2 pairs e with n >> 2
// and bits 3-6 pair (G, q) with c, all of which is baked into two constant B operands (one per
// n >> 2). Each lane then ends with 8 consecutive output channels (8c .. 8c + 7) of 4 tokens
// (rows 4G .. 4G + 3 of the MFMA output), which is exactly what the packed stores need: 4 code
// bytes of a K row per token, and - when the 4 tokens are the 4 consecutive slots that share the
// V tile's interleaved words - one 16-byte V store per lane.
//
// Quantization of the 32 values a lane holds per tensor: min / max in-lane and across the 16-lane
// row (DPP), scale and its reciprocal computed once per token (lane c & 3 does token c & 3, then
// quad broadcasts), codes by Markstein-corrected division (bit-exact with IEEE division), round
// half to even inside the byte conversion of the packing. Tokens whose scale is 0 or tiny take a slower path with IEEE division and the
// clamp; it is wave-uniform and never taken for ordinary data.
#include <algorithm>

#include "kvq_device.h"
#include "kvq_launch.h"
#include "kvq_mfma.h"
#include "kvq_rotate_mfma.h"

namespace kvq {
namespace {

// A token whose scale lies outside [2^-100, 2^101) (0, tiny, huge or not finite) takes the guarded
// path; inside it the reciprocal from rcp_rn is the correctly rounded one that div_rn needs.
constexpr float kFastMinScale = 0x1p-100f;
constexpr float kFastMaxScale = 0x1p101f;

// Quantize and pack the 32 values y[n][i] (token i, channel 8c + n) of one tensor. Returns the
// packed codes of each token (INT4: 4 bytes, INT2: 2 bytes) and its stored scale and zero.
template <int BITS, bool TOKEN_SCALE, bool ODD_LB>
__device__ __forceinline__ void quantize_tile(v4f (&y)[8], int c, uint32_t (&packed)[4], float (&scale)[4],
                                              float (&zero)[4]) {
  constexpr float kQmax = static_cast<float>((1 << BITS) - 1);
  if constexpr (ODD_LB) {
    constexpr float kInvSqrt2 = 0.70710678118654752440f;
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) y[n][i] *= kInvSqrt2;
  }
  float s[4] = {1.f, 1.f, 1.f, 1.f};
  if constexpr (TOKEN_SCALE) {
    // RMS in double precision across the 128 channels (16 lanes x 8), rounded once to float. The
    // row sums are equal in the row's 16 lanes (butterfly of commutative adds), so lane c takes the
    // square root and the reciprocal of token c & 3 only, and the quads broadcast them.
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
    const bool plain_own = s_own >= kFastMinScale && s_own < kFastMaxScale;
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
      // a subnormal, tiny or huge RMS somewhere in the wave: IEEE division for the whole wave (the
      // reciprocal would overflow, or the correction step's residual underflow; inside the range
      // both give the correctly rounded quotient)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < 8; ++n) y[n][i] = y[n][i] / s[i];
    }
  }
  float mn[4], mx[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // chains of three-input min / max: 8 values in 4 instructions each
    float a = fminf(fminf(y[0][i], y[1][i]), y[2][i]);
    float b = fmaxf(fmaxf(y[0][i], y[1][i]), y[2][i]);
    a = fminf(fminf(a, y[3][i]), y[4][i]);
    b = fmaxf(fmaxf(b, y[3][i]), y[4][i]);
    a = fminf(fminf(a, y[5][i]), y[6][i]);
    b = fmaxf(fmaxf(b, y[5][i]), y[6][i]);
    a = fminf(a, y[7][i]);
    b = fmaxf(b, y[7][i]);
    a = fminf(a, dpp_row<kDppQuadXor1>(a));
    b = fmaxf(b, dpp_row<kDppQuadXor1>(b));
    a = fminf(a, dpp_row<kDppQuadXor2>(a));
    b = fmaxf(b, dpp_row<kDppQuadXor2>(b));
    a = fminf(a, dpp_row<kDppHalfMirror>(a));
    b = fmaxf(b, dpp_row<kDppHalfMirror>(b));
    a = fminf(a, dpp_row<kDppRowRor8>(a));
    b = fmaxf(b, dpp_row<kDppRowRor8>(b));
    mn[i] = a;
    mx[i] = b;
  }
  // Scale and its reciprocal: lane c computes token c & 3, then quads broadcast. The scale
  // RN(d / qmax) comes from Markstein's correction with the constant RN(1 / qmax) - equal to IEEE
  // division for every normal d (checked exhaustively over all significands); smaller scales take
  // the guarded path, which divides again.
  const int own = c & 3;
  const float d_own = pick4(own, mx[0] - mn[0], mx[1] - mn[1], mx[2] - mn[2], mx[3] - mn[3]);
  constexpr float kInvQmax = 1.0f / kQmax;
  const float delta_own = div_rn(d_own, kQmax, kInvQmax);
  const bool fast_own = delta_own >= kFastMinScale && delta_own < kFastMaxScale;
  const float r_own = rcp_rn(fast_own ? delta_own : 1.0f);
  float delta[4], r[4];
  delta[0] = quad_bcast<0>(delta_own); r[0] = quad_bcast<0>(r_own);
  delta[1] = quad_bcast<1>(delta_own); r[1] = quad_bcast<1>(r_own);
  delta[2] = quad_bcast<2>(delta_own); r[2] = quad_bcast<2>(r_own);
  delta[3] = quad_bcast<3>(delta_own); r[3] = quad_bcast<3>(r_own);

  // every token of the wave is some lane's own token
  if (__builtin_expect(__all(fast_own), 1)) {
    // q = RN((y - mn) / delta) exactly; q <= qmax (1 + 2^-23) and q >= 0, so the rounding to an
    // integer in the packing needs no clamp.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float cd[8];
#pragma unroll
      for (int n = 0; n < 8; ++n) cd[n] = div_rn(y[n][i] - mn[i], delta[i], r[i]);
      packed[i] = pack_codes<BITS>(cd);
    }
  } else {
    // Guarded path: IEEE division, the clamp, and all-zero codes for a zero scale.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      delta[i] = (mx[i] - mn[i]) / kQmax;
      float cd[8];
#pragma unroll
      for (int n = 0; n < 8; ++n)
        cd[n] = (delta[i] != 0.0f) ? fminf(fmaxf(rintf((y[n][i] - mn[i]) / delta[i]), 0.0f), kQmax) : 0.0f;
      packed[i] = pack_codes<BITS>(cd);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    scale[i] = delta[i] * s[i];
    zero[i] = mn[i] * s[i];
  }
}

// Inputs of one work item (16 tokens of one KV head): lane (G, t) holds bytes 64q + 16G .. + 15
// of token t's K and V head vectors, and the slots of tokens 4G .. 4G + 3.
struct TileInputs {
  uint4 kx[4], vx[4];
  int64_t slot[4];
};

__device__ __forceinline__ void load_tile(const AppendArgs& a, int64_t tile0, int h, int G, int c, TileInputs& in) {
  // Rows past the last token re-read the last one: MFMA rows are independent tokens, and those
  // rows are never stored.
  const int64_t last = a.num_tokens - 1;
  const int64_t tok_in = min(tile0 + c, last);
  const uint16_t* kp = a.k + tok_in * a.k_stride + h * kHeadDim + 8 * G;
  const uint16_t* vp = a.v + tok_in * a.v_stride + h * kHeadDim + 8 * G;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    in.kx[q] = *reinterpret_cast<const uint4*>(kp + 32 * q);
    in.vx[q] = *reinterpret_cast<const uint4*>(vp + 32 * q);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) in.slot[i] = a.slots[min(tile0 + 4 * G + i, last)];
}

template <int BITS, bool TOKEN_SCALE, int LB>
__device__ __forceinline__ void process_tile(const AppendArgs& a, int64_t tile0, int h, int c, const v4u (&bop)[2],
                                             const TileInputs& in) {
  constexpr int kRow = kHeadDim * BITS / 8;   // code bytes per token row
  constexpr int kLaneBytes = 8 * BITS / 8;    // code bytes per lane per token (8 channels)
  const int G = (threadIdx.x & 63) >> 4;
  uint32_t kp[4], vp[4];
  float ks[4], kz[4], vs[4], vz[4];
  {
    v4f y[8];
    rotate_tile<LB>(in.kx, bop, y);
    quantize_tile<BITS, TOKEN_SCALE, (LB & 1) != 0>(y, c, kp, ks, kz);
  }
  {
    v4f y[8];
    rotate_tile<LB>(in.vx, bop, y);
    quantize_tile<BITS, TOKEN_SCALE, (LB & 1) != 0>(y, c, vp, vs, vz);
  }

  // ---- stores. Row r = (page * H + h) * ps + off of the cache; a K row starts at r * kRow, the
  // V word group of offsets off & ~3 at (r - (off & 3)) * kRow, the scale/zero pair at 8 r.
  const uint32_t ps = static_cast<uint32_t>(a.page_size);
  const uint32_t page_rows = static_cast<uint32_t>(a.num_kv_heads) * ps;  // rows per page (< 2^32: checked)
  const uint32_t head_row = static_cast<uint32_t>(h) * ps;
  bool live[4];
  uint64_t row[4];
  uint32_t off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    live[i] = tile0 + 4 * G + i < a.num_tokens && in.slot[i] >= 0 && in.slot[i] < a.num_slots;
    const uint32_t s = live[i] ? static_cast<uint32_t>(in.slot[i]) : 0u;  // live slots are < 2^32
    const uint32_t t = __umulhi(s, a.ps_magic);
    const uint32_t page = (t + ((s - t) >> 1)) >> a.ps_shift;
    off[i] = s - page * ps;
    row[i] = static_cast<uint64_t>(page) * page_rows + (head_row + off[i]);
  }
  uint8_t* const k_lane = a.k_codes + kLaneBytes * c;
  uint8_t* const v_lane = a.v_codes + 4 * kLaneBytes * c;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!live[i]) continue;
    if constexpr (BITS == 4) {
      *reinterpret_cast<uint32_t*>(k_lane + row[i] * kRow) = kp[i];
    } else {
      *reinterpret_cast<uint16_t*>(k_lane + row[i] * kRow) = static_cast<uint16_t>(kp[i]);
    }
    if (c == i) reinterpret_cast<float2*>(a.k_sz)[row[i]] = make_float2(ks[i], kz[i]);
    if (c == 4 + i) reinterpret_cast<float2*>(a.v_sz)[row[i]] = make_float2(vs[i], vz[i]);
  }
  // V: whole interleaved words when the four tokens fill one word group of a tile, else bytes.
  const bool group = live[0] && live[1] && live[2] && live[3] && (in.slot[0] & 3) == 0 &&
                     in.slot[1] == in.slot[0] + 1 && in.slot[2] == in.slot[0] + 2 && in.slot[3] == in.slot[0] + 3;
  if (group) {
    uint8_t* dst = v_lane + row[0] * kRow;
    const uint4 w = interleave4(vp);
    if constexpr (BITS == 4) {
      *reinterpret_cast<uint4*>(dst) = w;
    } else {
      *reinterpret_cast<uint2*>(dst) = make_uint2(w.x, w.y);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!live[i]) continue;
      const uint32_t sub = off[i] & 3;
      uint8_t* base = v_lane + (row[i] - sub) * kRow + sub;
#pragma unroll
      for (int m = 0; m < kLaneBytes; ++m) base[4 * m] = static_cast<uint8_t>(vp[i] >> (8 * m));
    }
  }
}

// One wave per work item of 16 tokens x one KV head, all loads issued before any arithmetic.
// Items are numbered head-fastest (w = tile * H + h), so the waves that run together read the
// same tokens' rows of all heads (one contiguous stretch of the K/V inputs) and write the
// neighbouring page-head tiles of the cache.
#ifndef KVQ_APPEND_MIN_WAVES
#define KVQ_APPEND_MIN_WAVES 1   // waves per SIMD the register allocation must allow
#endif

template <int BITS, bool TOKEN_SCALE, int LB>
__global__ __launch_bounds__(256, KVQ_APPEND_MIN_WAVES) void append_kernel(const AppendArgs a, int64_t num_tiles) {
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4;
  const int c = lane & 15;
  // work item w = (16-token tile, head), uniform per wave: scalar index arithmetic
  const uint32_t w = blockIdx.x * 4u + static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)));
  const uint32_t tq = fast_div(w, a.div_heads);
  const int64_t tile = tq;
  const int h = static_cast<int>(w - tq * a.div_heads.d);
  if (tile >= num_tiles || h >= a.num_kv_heads) return;  // uniform per wave
  const v4u bop[2] = {load_b<LB>(lane, 0), load_b<LB>(lane, 1)};
  TileInputs in;
  load_tile(a, tile * 16, h, G, c, in);
  __builtin_amdgcn_sched_barrier(0);  // issue every load (K, V, slots) before any arithmetic
  process_tile<BITS, TOKEN_SCALE, LB>(a, tile * 16, h, c, bop, in);
}

template <int BITS, bool TS, int LB>
hipError_t launch_one(const AppendArgs& a, hipStream_t stream) {
  const int64_t tiles = (a.num_tokens + 15) / 16;
  const int64_t items = tiles * a.num_kv_heads;  // < 2^31 (checked by the caller)
  hipLaunchKernelGGL((append_kernel<BITS, TS, LB>), dim3(static_cast<unsigned>((items + 3) / 4)), dim3(256), 0, stream,
                     a, tiles);
  return hipGetLastError();
}

template <int BITS, bool TS>
hipError_t launch_lb(const AppendArgs& a, int lb, hipStream_t stream) {
  switch (lb) {
    case 0: return launch_one<BITS, TS, 0>(a, stream);
    case 1: return launch_one<BITS, TS, 1>(a, stream);
    case 2: return launch_one<BITS, TS, 2>(a, stream);
    case 3: return launch_one<BITS, TS, 3>(a, stream);
    case 4: return launch_one<BITS, TS, 4>(a, stream);
    case 5: return launch_one<BITS, TS, 5>(a, stream);
    case 6: return launch_one<BITS, TS, 6>(a, stream);
    default: return launch_one<BITS, TS, 7>(a, stream);
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& args, hipStream_t stream) {
  AppendArgs a = args;
  a.div_heads = make_fast_div(static_cast<uint32_t>(a.num_kv_heads));
  int lb = 0;
  while ((1 << lb) < a.rot.hb) ++lb;
  if (a.bits == 4 && !a.token_scale) return launch_lb<4, false>(a, lb, stream);
  if (a.bits == 4) return launch_lb<4, true>(a, lb, stream);
  if (!a.token_scale) return launch_lb<2, false>(a, lb, stream);
  return launch_lb<2, true>(a, lb, stream);
}

}  // namespace kvq
