// Read path on the matrix cores: paged decode attention over the rotated INT4/INT2 cache with
// QK^T and PV on MFMA (sources as in kvq_decode.hip: dequantization fused into attention, ainews.cool
// "Technical Deep Dive"; a paged low-bit attention kernel, OSCAR abstract on thelatestinai.com;
// split decoding after FlashDecoding-v2, named in the OScaR abstract).
//
// One wave per (split, KV head, sequence); the split's pages are walked as 16-token tiles, two
// tiles per step. Dequantization is folded around the contractions instead of materialised:
//   score_j = q~ . (delta_j c_j + z_j 1) = delta_j (q~ . c_j) + z_j sum(q~)
//   sum_j p_j v_j = sum_j (p_j delta_j) c_j + sum_j p_j z_j 1
// so the integer codes c_j enter the MFMAs directly.
//
// QK^T  (v_mfma_i32_16x16x64_i8): A = K codes of one tile (row = token, lane (G, t) holds 32
//   channels of token t as bytes), B = the query of the group's heads as a 21-bit fixed-point
//   integer split into three signed int8 limbs (column = head). The three limb products are
//   combined by Horner's rule (x 128 between limbs) in exact int32 arithmetic; the output lane
//   (G, n) holds heads n, tokens 4G..4G+3.
// PV    (v_mfma_f32_16x16x32_bf16): A = p_j delta_j for head n and tokens 4G..4G+3 of both tiles -
//   already in the lanes the QK output left them in - split into bf16 hi + lo parts (two MFMAs);
//   B = V codes as bf16 values B + c (B = 16 for INT4, 4 for INT2: with that exponent the code
//   lands in the low mantissa bits, so two shifts/masks and one byte permute per two codes build
//   the operand from the token-interleaved V tile); the offset is folded into the zero term
//   (z - B delta). A small B keeps the hi/lo split error of p delta (about 2^-17 relative) from
//   being amplified by the offset.
//   Output lane (G, n) holds heads 4G..4G+3, channels 8n..8n+7.
// Online softmax in base 2 with a lazy maximum: the accumulators are rescaled only when a tile's
// maximum exceeds the running one by more than 8 (so p <= 2^8 in between).
#include <algorithm>

#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLazyRescale = 8.0f;  // log2 units
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
  __bf16 lb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hb[i] = __float_as_uint(w[i]) & 0xFFFF0000u;
    lb[i] = static_cast<__bf16>(w[i] - __uint_as_float(hb[i]));
  }
  hi01 = __builtin_amdgcn_perm(hb[1], hb[0], 0x07060302u);
  hi23 = __builtin_amdgcn_perm(hb[3], hb[2], 0x07060302u);
  lo01 = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lb[0])) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lb[1])) << 16);
  lo23 = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lb[2])) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lb[3])) << 16);
}

// Channel of the query that MFMA j, register slot r, byte k of lane group G multiplies (it must
// match the byte the K-code operand puts there).
template <int BITS>
__device__ __forceinline__ int qk_channel(int G, int j, int r, int k) {
  if constexpr (BITS == 4) {
    return 32 * G + 16 * j + 8 * (r >> 1) + 2 * k + (r & 1);
  } else {
    return 32 * G + 16 * j + 4 * k + r;
  }
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
// (shift 3 for INT4, 5 for INT2), one token per byte.
template <int BITS>
__device__ __forceinline__ uint32_t v_bf16_low_bytes(const uint4 w, int m) {
  if constexpr (BITS == 4) {
    const uint32_t d = (m >> 1) == 0 ? w.x : (m >> 1) == 1 ? w.y : (m >> 1) == 2 ? w.z : w.w;
    return (((m & 1) ? (d >> 1) : (d << 3)) & 0x78787878u) | 0x80808080u;
  } else {
    const uint32_t d = (m >> 2) ? w.y : w.x;
    const int sh = 2 * (m & 3);  // crumb position; target bits 5..6
    return (((sh <= 5) ? (d << (5 - sh)) : (d >> (sh - 5))) & 0x60606060u) | 0x80808080u;
  }
}

struct TileLoad {
  uint4 k;        // K codes: token n, channels 32G..32G+31
  uint4 v;        // V codes: tokens 4G..4G+3, channels 8n..8n+7
  float4 ksz01, ksz23;  // (scale, zero) of tokens 4G..4G+3
  float4 vsz01, vsz23;
};

template <int BITS>
__device__ __forceinline__ TileLoad load_tile(const DecodeArgs& a, int64_t page, int sub, int kvh, int G, int n) {
  constexpr int kRow = kHeadDim * BITS / 8;
  const int64_t tile = page * a.num_kv_heads + kvh;
  const uint8_t* kt = a.k_codes + (tile * a.page_size + 16 * sub) * kRow;
  const uint8_t* vt = a.v_codes + (tile * a.page_size + 16 * sub) * kRow;
  const float4* ks = reinterpret_cast<const float4*>(a.k_sz + (tile * a.page_size + 16 * sub + 4 * G) * 2);
  const float4* vs = reinterpret_cast<const float4*>(a.v_sz + (tile * a.page_size + 16 * sub + 4 * G) * 2);
  TileLoad t;
  if constexpr (BITS == 4) {
    t.k = *reinterpret_cast<const uint4*>(kt + n * kRow + 16 * G);
    t.v = *reinterpret_cast<const uint4*>(vt + G * 4 * kRow + 16 * n);
  } else {
    const uint2 k2 = *reinterpret_cast<const uint2*>(kt + n * kRow + 8 * G);
    const uint2 v2 = *reinterpret_cast<const uint2*>(vt + G * 4 * kRow + 8 * n);
    t.k = make_uint4(k2.x, k2.y, 0, 0);
    t.v = make_uint4(v2.x, v2.y, 0, 0);
  }
  t.ksz01 = ks[0];
  t.ksz23 = ks[1];
  t.vsz01 = vs[0];
  t.vsz23 = vs[1];
  return t;
}

template <int BITS>
__global__ __launch_bounds__(64) void decode_mfma_kernel(const DecodeArgs a) {
  __shared__ float qs[8][kHeadDim];

  const int lane = threadIdx.x;
  const int G = lane >> 4;
  const int n = lane & 15;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int g = a.num_q_heads / a.num_kv_heads;
  const int ps = a.page_size;
  const int tiles_per_page = ps / 16;
  const int len = min(max(a.context_lens[b], 0), a.max_context_len);
  const int n_pages = (len + ps - 1) / ps;
  const int p_begin = split * a.pages_per_split;
  const int p_end = min(n_pages, p_begin + a.pages_per_split);
  const int64_t q_row0 = (static_cast<int64_t>(b) * a.num_q_heads + static_cast<int64_t>(kvh) * g) * kHeadDim;

  if (p_begin >= p_end) {
    if (a.num_splits == 1) {  // empty sequence, unsplit: zero output
      for (int h = G; h < g; h += 4) {
        float4* o = reinterpret_cast<float4*>(a.out + q_row0 + h * kHeadDim + n * 8);
        o[0] = make_float4(0.f, 0.f, 0.f, 0.f);
        o[1] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    return;
  }

  // ---- query: rotate (R q), scale by softmax_scale * log2(e), stage in LDS in natural order
  const LaneFwht lf = lane_fwht(a.rot, n);
  for (int h0 = 0; h0 < g; h0 += 4) {
    const int h = h0 + G;
    float x[8];
    const uint4 w = (h < g) ? *reinterpret_cast<const uint4*>(a.q + q_row0 + h * kHeadDim + n * 8) : make_uint4(0, 0, 0, 0);
    bf16x8_to_f32(w, x);
    int pos = n;
    if (!a.q_prerotated) {
      fwht_row16_planned(x, a.rot, lf);
      pos = lf.pos;
    }
    if (h < g) {
#pragma unroll
      for (int k = 0; k < 8; ++k) qs[h][8 * pos + k] = x[k] * a.qk_scale_log2;
    }
  }
  __syncthreads();

  // ---- query as 21-bit fixed point x = rint(q' 2^E), |x| <= 2^20, in three int8 limbs
  float qv[32];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int k = 0; k < 4; ++k) qv[(j * 4 + r) * 4 + k] = (n < g) ? qs[n][qk_channel<BITS>(G, j, r, k)] : 0.f;
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(qv[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  int e2 = 0;
  (void)frexpf(amax, &e2);
  const int E = (amax > 0.f) ? 20 - e2 : 0;
  v4i L0[2], L1[2], L2[2];
  int sx = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t d0 = 0, d1 = 0, d2 = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int x = static_cast<int>(rintf(ldexpf(qv[(j * 4 + r) * 4 + k], E)));
        sx += x;
        const int l2 = ((x + 64) & 127) - 64;
        const int x1 = (x - l2) >> 7;
        const int l1 = ((x1 + 64) & 127) - 64;
        const int l0 = (x1 - l1) >> 7;
        d0 |= (static_cast<uint32_t>(l0) & 0xFFu) << (8 * k);
        d1 |= (static_cast<uint32_t>(l1) & 0xFFu) << (8 * k);
        d2 |= (static_cast<uint32_t>(l2) & 0xFFu) << (8 * k);
      }
      L0[j][r] = static_cast<int>(d0);
      L1[j][r] = static_cast<int>(d1);
      L2[j][r] = static_cast<int>(d2);
    }
  }
  sx += __shfl_xor(sx, 16, 64);
  sx += __shfl_xor(sx, 32, 64);
  const float inv_scale = ldexpf(1.0f, -E);     // q' = x 2^-E
  const float sum_q = static_cast<float>(sx);   // sum of x over the 128 channels

  // ---- walk the split's tiles two at a time
  const int tile_begin = p_begin * tiles_per_page;
  const int tile_end = min(p_end * tiles_per_page, (len + 15) / 16);
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.max_pages_per_seq;

  v4f acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;   // running maximum of head n (log2 units), equal in the 4 lanes of head n
  float l_part = 0.f;      // this lane's share of sum p (head n)
  float z_part = 0.f;      // this lane's share of sum p (z - B delta) (head n)

  auto page_of = [&](int tile) -> int64_t {
    const int32_t p = bt[tile / tiles_per_page];
    return (p >= 0 && p < a.num_pages) ? p : -1;
  };
  // Loads of tiles (t, t+1) into (x, y); a missing or invalid tile re-reads a valid one and is
  // masked out through its page flag.
  auto fetch = [&](int t, TileLoad& x, TileLoad& y, int64_t& px, int64_t& py) {
    px = page_of(t);
    py = (t + 1 < tile_end) ? page_of(t + 1) : -1;
    const int64_t sx = px < 0 ? 0 : px;
    x = load_tile<BITS>(a, sx, t % tiles_per_page, kvh, G, n);
    y = load_tile<BITS>(a, py < 0 ? sx : py, (t + 1) % tiles_per_page, kvh, G, n);
  };

  auto step = [&](const TileLoad& ca, const TileLoad& cb, int64_t pa, int64_t pb, int tile) {
    const bool a_ok = pa >= 0;
    const bool b_ok = (tile + 1 < tile_end) && pb >= 0;
    // QK^T for both tiles: exact int32 dot products of the codes with the fixed-point query
    v4i sa = v4i{0, 0, 0, 0}, sb = v4i{0, 0, 0, 0};
    const v4i ka0 = k_operand<BITS>(ca.k, 0), ka1 = k_operand<BITS>(ca.k, 1);
    const v4i kb0 = k_operand<BITS>(cb.k, 0), kb1 = k_operand<BITS>(cb.k, 1);
    sa = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka0, L0[0], sa, 0, 0, 0);
    sb = __builtin_amdgcn_mfma_i32_16x16x64_i8(kb0, L0[0], sb, 0, 0, 0);
    sa = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka1, L0[1], sa, 0, 0, 0);
    sb = __builtin_amdgcn_mfma_i32_16x16x64_i8(kb1, L0[1], sb, 0, 0, 0);
    sa = sa << 7;
    sb = sb << 7;
    sa = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka0, L1[0], sa, 0, 0, 0);
    sb = __builtin_amdgcn_mfma_i32_16x16x64_i8(kb0, L1[0], sb, 0, 0, 0);
    sa = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka1, L1[1], sa, 0, 0, 0);
    sb = __builtin_amdgcn_mfma_i32_16x16x64_i8(kb1, L1[1], sb, 0, 0, 0);
    sa = sa << 7;
    sb = sb << 7;
    sa = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka0, L2[0], sa, 0, 0, 0);
    sb = __builtin_amdgcn_mfma_i32_16x16x64_i8(kb0, L2[0], sb, 0, 0, 0);
    sa = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka1, L2[1], sa, 0, 0, 0);
    sb = __builtin_amdgcn_mfma_i32_16x16x64_i8(kb1, L2[1], sb, 0, 0, 0);

    // scores (log2 units) of head n, tokens 4G+i of tile a (s[i]) and tile b (s[4+i])
    const int tok_a = tile * 16 + 4 * G, tok_b = tok_a + 16;
    const float kd[8] = {ca.ksz01.x, ca.ksz01.z, ca.ksz23.x, ca.ksz23.z, cb.ksz01.x, cb.ksz01.z, cb.ksz23.x, cb.ksz23.z};
    const float kz[8] = {ca.ksz01.y, ca.ksz01.w, ca.ksz23.y, ca.ksz23.w, cb.ksz01.y, cb.ksz01.w, cb.ksz23.y, cb.ksz23.w};
    const float vd[8] = {ca.vsz01.x, ca.vsz01.z, ca.vsz23.x, ca.vsz23.z, cb.vsz01.x, cb.vsz01.z, cb.vsz23.x, cb.vsz23.z};
    const float vz[8] = {ca.vsz01.y, ca.vsz01.w, ca.vsz23.y, ca.vsz23.w, cb.vsz01.y, cb.vsz01.w, cb.vsz23.y, cb.vsz23.w};
    float s[8];
    bool ok[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int acc_i = i < 4 ? sa[i] : sb[i - 4];
      ok[i] = (i < 4 ? (a_ok && tok_a + i < len) : (b_ok && tok_b + i - 4 < len));
      const float sc = inv_scale * __builtin_fmaf(kd[i], static_cast<float>(acc_i), kz[i] * sum_q);
      s[i] = ok[i] ? sc : kNegInf;
    }
    float mt = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    if (__any(mt > m_run + kLazyRescale)) {
      const float m_new = (mt > m_run + kLazyRescale) ? mt : m_run;
      const float alpha = (m_run == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_part *= alpha;
      z_part *= alpha;
      // accumulator rows are heads 4G+i; their factors live in lane 4G+i (head n = 4G+i)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * G + i, 64);
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[m][i] *= ai;
      }
    }
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = ok[i] ? __builtin_amdgcn_exp2f(s[i] - m_run) : 0.f;
      l_part += p;
      z_part = __builtin_fmaf(p, ok[i] ? __builtin_fmaf(-VBias<BITS>::value, vd[i], vz[i]) : 0.f, z_part);
      w[i] = ok[i] ? p * vd[i] : 0.f;
    }
    uint32_t h01a, h23a, l01a, l23a, h01b, h23b, l01b, l23b;
    split_bf16({w[0], w[1], w[2], w[3]}, h01a, h23a, l01a, l23a);
    split_bf16({w[4], w[5], w[6], w[7]}, h01b, h23b, l01b, l23b);
    const v8bf p_hi = as_bf(v4u{h01a, h23a, h01b, h23b});
    const v8bf p_lo = as_bf(v4u{l01a, l23a, l01b, l23b});
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint32_t na = v_bf16_low_bytes<BITS>(ca.v, m);
      const uint32_t nb = v_bf16_low_bytes<BITS>(cb.v, m);
      const v8bf vb = as_bf(v4u{bias_bf16_lo<BITS>(na), bias_bf16_hi<BITS>(na), bias_bf16_lo<BITS>(nb),
                                bias_bf16_hi<BITS>(nb)});
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p_hi, vb, acc[m], 0, 0, 0);
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p_lo, vb, acc[m], 0, 0, 0);
    }
  };

  // Double-buffered walk: buffer 0 holds tiles (t, t+1) while tiles (t+2, t+3) load into buffer 1.
  TileLoad x0, y0, x1, y1;
  int64_t px0, py0, px1 = -1, py1 = -1;
  fetch(tile_begin, x0, y0, px0, py0);
  for (int tile = tile_begin; tile < tile_end; tile += 4) {
    if (tile + 2 < tile_end) fetch(tile + 2, x1, y1, px1, py1);
    step(x0, y0, px0, py0, tile);
    if (tile + 2 >= tile_end) break;
    if (tile + 4 < tile_end) fetch(tile + 4, x0, y0, px0, py0);
    step(x1, y1, px1, py1, tile + 2);
  }

  // ---- finish: totals of head n, then moved to the accumulator rows (heads 4G+i)
  l_part += __shfl_xor(l_part, 16, 64);
  l_part += __shfl_xor(l_part, 32, 64);
  z_part += __shfl_xor(z_part, 16, 64);
  z_part += __shfl_xor(z_part, 32, 64);
  float lrow[4], zrow[4], mrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lrow[i] = __shfl(l_part, 4 * G + i, 64);
    zrow[i] = __shfl(z_part, 4 * G + i, 64);
    mrow[i] = __shfl(m_run, 4 * G + i, 64);
  }

  if (a.num_splits == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * G + i;
      float o[8];
      const float inv_l = (lrow[i] > 0.f) ? 1.0f / lrow[i] : 0.f;
#pragma unroll
      for (int m = 0; m < 8; ++m) o[m] = (acc[m][i] + zrow[i]) * inv_l;
      fwht_row16_planned(o, a.rot, lf);  // R^T = R: back to the original basis
      if (h < g) {
        float4* dst = reinterpret_cast<float4*>(a.out + q_row0 + h * kHeadDim + 8 * lf.pos);
        dst[0] = make_float4(o[0], o[1], o[2], o[3]);
        dst[1] = make_float4(o[4], o[5], o[6], o[7]);
      }
    }
  } else {
    const int64_t base = (static_cast<int64_t>(split) * a.batch + b) * a.num_q_heads + static_cast<int64_t>(kvh) * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * G + i;
      if (h < g) {
        float4* dst = reinterpret_cast<float4*>(a.ws_acc + (base + h) * kHeadDim + 8 * n);
        dst[0] = make_float4(acc[0][i] + zrow[i], acc[1][i] + zrow[i], acc[2][i] + zrow[i], acc[3][i] + zrow[i]);
        dst[1] = make_float4(acc[4][i] + zrow[i], acc[5][i] + zrow[i], acc[6][i] + zrow[i], acc[7][i] + zrow[i]);
        if (n == 0) reinterpret_cast<float2*>(a.ws_ml)[base + h] = make_float2(mrow[i], lrow[i]);
      }
    }
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.num_splits), static_cast<unsigned>(a.num_kv_heads),
                  static_cast<unsigned>(a.batch));
  if (a.bits == 4) {
    hipLaunchKernelGGL(decode_mfma_kernel<4>, grid, dim3(64), 0, stream, a);
  } else {
    hipLaunchKernelGGL(decode_mfma_kernel<2>, grid, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace kvq
