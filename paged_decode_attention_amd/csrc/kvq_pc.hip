// Per-channel pages, read path: the per-channel reading of OScaR (OScaR abstract on the openalex
// page: the rotation and the per-token scaling let the per-channel quantization paradigm hold up
// under extreme compression; zhichai.net summary, "Root Cause: Token Norm Imbalance" and "The
// OScaR Framework": V-hat = Quant(S (R V))). The pages are written by kvq_pc_write.hip: codes in
// the token-wise cache's layout, s per token, (scale, zero) per channel of the page's u = y / s.
//
// Read path (pc_decode_kernel): k^_t = s_t (scale (.) c_t + zero) in the rotated basis, so
//   q~ . k^_t = s_t (sum_c (q~_c scale_c) c_tc + sum_c q~_c zero_c):
// per page, the query is multiplied by the page's K channel scales and split into int8 limbs for
// the integer matrix-core product with the codes (the token-wise decode's scheme, redone per
// page), and sum_c q~_c zero_c is one dot product per page. For V,
//   sum_t p_t v^_t = scale (.) sum_t (p_t s_t) c_t + zero sum_t p_t s_t,
// so the PV product of a page accumulates with weights w_t = p_t s_t and is folded into the
// output with the page's V channel scales and zeros when the page ends. The last split of every
// sequence attends to the bf16 tokens of its unfinished page instead (the residual window). Every
// split writes its partial in the original basis, and the split merge combines them.
#include <algorithm>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_launch.h"
#include "kvq_mfma.h"

namespace kvq {
namespace {

// ---------------------------------------------------------------------------- read path
constexpr int kNT = 2;  // 16-token tiles per step (a page holds a whole number of steps)

// One tile as a lane loads it: K codes of token n (channels 32G .. 32G + 31), V codes of tokens
// 4G .. 4G + 3 (channels 8n .. 8n + 7), and one token scale (lanes 0..15: K, 16..31: V; the
// upper half repeats them).
struct PcTile {
  uint4 k;
  uint4 v;
  float s;
};

// The query's int8 limbs for one page: x = rint(q' 2^E), q' = q~ (.) the page's K channel scales,
// |x| < 2^20, split as in the token-wise decode (bytes of x + 0x808080 with the top bit flipped).
struct QueryLimbs {
  v4i l0[2], l1[2], l2[2];
  float inv_scale;  // 2^-E
};

template <int BITS>
__device__ __forceinline__ QueryLimbs page_limbs(const float (&qv)[32]) {
  QueryLimbs L;
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(qv[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  int e2 = 0;
  (void)frexpf(amax, &e2);
  const int E = (amax > 0.f) ? 20 - e2 : 0;
  const float two_e = ldexpf(1.0f, E);
  constexpr float kRoundMagic = 12582912.0f;                 // 1.5 * 2^23
  constexpr uint32_t kOffsetBits = 0x4B400000u - 0x808080u;  // bits(magic + x) - this = x + 0x808080
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t xb[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        xb[k] = __float_as_uint(__builtin_fmaf(qv[(j * 4 + r) * 4 + k], two_e, kRoundMagic)) - kOffsetBits;
      const uint32_t lo01 = __builtin_amdgcn_perm(xb[1], xb[0], 0x05010400u);
      const uint32_t lo23 = __builtin_amdgcn_perm(xb[3], xb[2], 0x05010400u);
      const uint32_t hi01 = __builtin_amdgcn_perm(xb[1], xb[0], 0x07030602u);
      const uint32_t hi23 = __builtin_amdgcn_perm(xb[3], xb[2], 0x07030602u);
      L.l0[j][r] = static_cast<int>(__builtin_amdgcn_perm(lo23, lo01, 0x05040100u) ^ 0x80808080u);
      L.l1[j][r] = static_cast<int>(__builtin_amdgcn_perm(lo23, lo01, 0x07060302u) ^ 0x80808080u);
      L.l2[j][r] = static_cast<int>(__builtin_amdgcn_perm(hi23, hi01, 0x05040100u) ^ 0x80808080u);
    }
  }
  L.inv_scale = ldexpf(1.0f, -E);
  return L;
}

// The residual window: softmax partial of each query head of one (sequence, KV head) over the
// n_tail bf16 tokens of the unfinished page (lane t scores token t; lane l then accumulates
// channels 2l, 2l + 1), in the original basis.
__device__ __forceinline__ void pc_tail(const PcDecodeArgs& a, int b, int kvh, int g, int n_tail, float (&qs)[8][kHeadDim],
                        float (&pw)[8][kPcMaxPage]) {
  const int lane = threadIdx.x;
  // raw query rows (scaled to log2 units)
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if (c < g) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(
          a.q + (static_cast<int64_t>(b) * a.num_q_heads + static_cast<int64_t>(kvh) * g + c) * kHeadDim + 2 * lane);
      qs[c][2 * lane] = bf16_lo(w) * a.qk_scale_log2;
      qs[c][2 * lane + 1] = bf16_hi(w) * a.qk_scale_log2;
    }
  }
  wave_lds_sync();
  const int64_t tok_stride = static_cast<int64_t>(a.num_kv_heads) * kHeadDim;
  const uint16_t* kt = a.tail_k + static_cast<int64_t>(b) * a.page_size * tok_stride + kvh * kHeadDim;
  const uint16_t* vt = a.tail_v + static_cast<int64_t>(b) * a.page_size * tok_stride + kvh * kHeadDim;
  // lane l scores tokens l and l + 64
  constexpr int kRounds = kPcMaxPage / 64;
  float s[kRounds][8];
#pragma unroll
  for (int rd = 0; rd < kRounds; ++rd) {
#pragma unroll
    for (int c = 0; c < 8; ++c) s[rd][c] = kNegInf;
    const int t = lane + 64 * rd;
    if (t < n_tail) {
#pragma unroll
      for (int c = 0; c < 8; ++c) s[rd][c] = 0.f;
      const uint16_t* kr = kt + t * tok_stride;
      for (int j = 0; j < kHeadDim / 8; ++j) {
        float x[8];
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(kr + 8 * j), x);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          if (c < g) {
#pragma unroll
            for (int k = 0; k < 8; ++k) s[rd][c] = __builtin_fmaf(qs[c][8 * j + k], x[k], s[rd][c]);
          }
        }
      }
    }
  }
  float m[8], l[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float mx = s[0][c];
#pragma unroll
    for (int rd = 1; rd < kRounds; ++rd) mx = fmaxf(mx, s[rd][c]);
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float sum = 0.f;
#pragma unroll
    for (int rd = 0; rd < kRounds; ++rd) {
      const float p = (s[rd][c] != kNegInf) ? __builtin_amdgcn_exp2f(s[rd][c] - mx) : 0.f;  // no token: 0
      sum += p;
      pw[c][lane + 64 * rd] = p;
    }
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
    m[c] = mx;
    l[c] = sum;
  }
  wave_lds_sync();
  float acc[8][2];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c][0] = acc[c][1] = 0.f;
  for (int t = 0; t < n_tail; ++t) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(vt + t * tok_stride + 2 * lane);
    const float v0 = bf16_lo(w), v1 = bf16_hi(w);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (c < g) {
        acc[c][0] = __builtin_fmaf(pw[c][t], v0, acc[c][0]);
        acc[c][1] = __builtin_fmaf(pw[c][t], v1, acc[c][1]);
      }
    }
  }
  const int64_t pairs = static_cast<int64_t>(a.batch) * a.num_q_heads;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if (c < g) {
      const int64_t row = a.num_splits * pairs + static_cast<int64_t>(b) * a.num_q_heads + static_cast<int64_t>(kvh) * g + c;
      *reinterpret_cast<float2*>(a.ws_acc + row * kHeadDim + 2 * lane) = make_float2(acc[c][0], acc[c][1]);
      if (lane == 0) reinterpret_cast<float2*>(a.ws_ml)[row] = make_float2(m[c], l[c]);
    }
  }
}

// One wave per (split, KV head, sequence); split num_splits takes the residual window. Column n
// of the QK output is query head n (n < g used), as in the token-wise decode.
template <int BITS>
__global__ __launch_bounds__(64, 2) void pc_decode_kernel(const PcDecodeArgs a) {
  __shared__ float qs[8][kHeadDim];            // rotated query rows (log2 units); raw ones for the tail
  __shared__ float4 szs[2][kNT][16];           // token scales of a step's tiles: [buf][tile][K 0..3 | V 4..7]
  __shared__ float cps[2][4][kHeadDim];        // page parameters: [page parity][K scale, K zero, V scale, V zero]
  __shared__ float pw[8][kPcMaxPage];          // tail softmax weights

  const int lane = threadIdx.x;
  const int G = lane >> 4;
  const int n = lane & 15;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int g = a.num_q_heads / a.num_kv_heads;
  const int ps = a.page_size;
  const int tpp = ps / 16;  // tiles per page: 2, 4 or 8 (page sizes 32, 64, 128)
  const int tpp_shift = (ps == 32) ? 1 : ((ps == 64) ? 2 : 3);  // tile indices are >= 0: shift and mask
  const int len = min(max(ro_load(a.context_lens, b), 0), a.max_context_len);
  const int n_full = len / ps;
  const int64_t pairs = static_cast<int64_t>(a.batch) * a.num_q_heads;

  if (split == a.num_splits) {
    pc_tail(a, b, kvh, g, len - n_full * ps, qs, pw);
    return;
  }
  const int p_begin = split * a.pages_per_split;
  const int p_end = (split == a.num_splits - 1) ? n_full : min(n_full, p_begin + a.pages_per_split);
  if (p_begin >= p_end) {  // no page: an empty partial (weight 0 in the merge)
    for (int c = G; c < g; c += 4) {
      const int64_t row = split * pairs + static_cast<int64_t>(b) * a.num_q_heads + static_cast<int64_t>(kvh) * g + c;
      float4* o = reinterpret_cast<float4*>(a.ws_acc + row * kHeadDim + 8 * n);
      o[0] = make_float4(0.f, 0.f, 0.f, 0.f);
      o[1] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (n == 0) reinterpret_cast<float2*>(a.ws_ml)[row] = make_float2(kNegInf, 0.f);
    }
    return;
  }
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.max_pages_per_seq;
  const int64_t page_rows = static_cast<int64_t>(a.num_kv_heads) * ps;
  const int64_t head_rows = static_cast<int64_t>(kvh) * ps;
  auto page_id = [&](int p) -> int32_t {
    const int32_t id = ro_load(bt, p);
    return (id >= 0 && id < a.num_pages) ? id : -1;
  };
  // page parameters: lanes 0..31 take the K (scale, zero) block, 32..63 the V block, 8 floats each
  struct Params {
    float4 lo, hi;
  };
  auto load_params = [&](int32_t id) -> Params {
    const int64_t base = (static_cast<int64_t>(id < 0 ? 0 : id) * a.num_kv_heads + kvh) * 2 * kHeadDim + 8 * (lane & 31);
    const float* src = (lane < 32 ? a.k_cp : a.v_cp) + base;
    return Params{*reinterpret_cast<const float4*>(src), *reinterpret_cast<const float4*>(src + 4)};
  };
  auto stage_params = [&](int parity, const Params& r) {
    float* dst = &cps[parity][0][0] + 8 * lane;  // lanes 0..15 K scale, 16..31 K zero, 32..47 V scale, 48..63 V zero
    reinterpret_cast<float4*>(dst)[0] = r.lo;
    reinterpret_cast<float4*>(dst)[1] = r.hi;
  };

  // per-lane byte offsets inside a tile's K and V code blocks
  const uint32_t lo_k = (BITS == 4) ? (n * (kHeadDim / 2) + 16 * G) : (n * (kHeadDim / 4) + 8 * G);
  const uint32_t lo_v = (BITS == 4) ? (G * 4 * (kHeadDim / 2) + 16 * n) : (G * 4 * (kHeadDim / 4) + 8 * n);
  const float* s_src = ((lane & 31) < 16 ? a.k_s : a.v_s) + (lane & 15);
  const int tile_begin = p_begin * tpp;
  const int tile_end = p_end * tpp;
  const int last_tile = tile_end - 1;
  auto fetch = [&](int t, PcTile (&x)[kNT], int64_t (&pg)[kNT]) {
#pragma unroll
    for (int u = 0; u < kNT; ++u) {
      const int tt = min(t + u, last_tile);
      const int32_t p = page_id(tt >> tpp_shift);
      pg[u] = (p >= 0 && t + u <= last_tile) ? p : -1;
      const int64_t row0 = (p >= 0 ? p : 0) * page_rows + head_rows + 16 * (tt & (tpp - 1));
      constexpr int kRowShift = (BITS == 4) ? 6 : 5;
      const __amdgpu_buffer_rsrc_t kr = tile_rsrc(a.k_codes + (row0 << kRowShift), 16 << kRowShift);
      const __amdgpu_buffer_rsrc_t vr = tile_rsrc(a.v_codes + (row0 << kRowShift), 16 << kRowShift);
      if constexpr (BITS == 4) {
        x[u].k = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, lo_k, 0, 2));
        x[u].v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, lo_v, 0, 2));
      } else {
        const uint2 k2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(kr, lo_k, 0, 2));
        const uint2 v2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(vr, lo_v, 0, 2));
        x[u].k = make_uint4(k2.x, k2.y, 0, 0);
        x[u].v = make_uint4(v2.x, v2.y, 0, 0);
      }
      x[u].s = s_src[row0];
    }
  };

  // query rows (row group G: heads G and G + 4), the first page's parameters and the first two
  // steps' tiles start loading before the query is prepared
  uint4 qw[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int c = min(4 * r + G, g - 1);
    qw[r] = *reinterpret_cast<const uint4*>(
        a.q + (static_cast<int64_t>(b) * a.num_q_heads + static_cast<int64_t>(kvh) * g + c) * kHeadDim + n * 8);
  }
  Params prm = load_params(page_id(p_begin));
  __builtin_amdgcn_sched_barrier(0);
  PcTile x0[kNT], x1[kNT], x2[kNT];
  int64_t pg0[kNT], pg1[kNT], pg2[kNT];
  fetch(tile_begin, x0, pg0);
  fetch(tile_begin + kNT, x1, pg1);

  const LaneFwht lf = lane_fwht(a.rot, n);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int c = 4 * r + G;
    if (4 * r >= g) break;
    float x[8];
    bf16x8_to_f32(qw[r], x);
    fwht_row16_planned(x, a.rot, lf);
    if (c < g) {
#pragma unroll
      for (int k = 0; k < 8; ++k) qs[c][8 * lf.pos + k] = x[k] * a.qk_scale_log2;
    }
  }
  stage_params(p_begin & 1, prm);
  prm = load_params(page_id(min(p_begin + 1, p_end - 1)));  // the next page's, in flight
#pragma unroll
  for (int u = 0; u < kNT; ++u) reinterpret_cast<float*>(szs[0][u])[lane] = x0[u].s;
  wave_lds_sync();

  v4f acc[8], accp[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
    accp[m] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  float m_run = kNegInf;  // running maximum of head n (log2 units)
  float l_part = 0.f;     // this lane's share of sum p (head n)
  float sw = 0.f;         // this lane's share of the page's sum of p s_V (head n)
  QueryLimbs L{};
  float zq = 0.f;          // sum_c q~_c zero_c of the current page (head n)
  float dv[8], zv[8];      // V channel scale and (zero - B scale) of channels 8n .. 8n + 7
  const uint32_t c80 = vgpr_const(0x80808080u);

  auto page_begin = [&](int p) {
    const int par = p & 1;
    float qv[32];
    float zp = 0.f;
    // the lane's 32 channels are 32G .. 32G + 31: read them four at a time and place each
    // in the operand slot (j, r, k) whose channel it is
    const float4* qrow = reinterpret_cast<const float4*>(&qs[n < g ? n : 0][32 * G]);
    const float4* krow = reinterpret_cast<const float4*>(&cps[par][0][32 * G]);
    const float4* zrow = reinterpret_cast<const float4*>(&cps[par][1][32 * G]);
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const float4 q4 = qrow[f], k4 = krow[f], z4 = zrow[f];
      const float qq[4] = {q4.x, q4.y, q4.z, q4.w};
      const float kk[4] = {k4.x, k4.y, k4.z, k4.w};
      const float zz[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int off = 4 * f + e;  // channel 32G + off
        int slot;
        if constexpr (BITS == 4) {  // off = 16 j + 8 (r >> 1) + 2 k + (r & 1)
          const int j = off >> 4, rh = (off >> 3) & 1, k = (off >> 1) & 3, rl = off & 1;
          slot = (j * 4 + 2 * rh + rl) * 4 + k;
        } else {                    // off = 16 j + 4 k + r
          const int j = off >> 4, k = (off >> 2) & 3, r = off & 3;
          slot = (j * 4 + r) * 4 + k;
        }
        const float q = (n < g) ? qq[e] : 0.f;
        qv[slot] = q * kk[e];
        zp = __builtin_fmaf(q, zz[e], zp);
      }
      if (f & 1) __builtin_amdgcn_sched_barrier(0);  // bound the reads in flight (registers)
    }
    zp += __shfl_xor(zp, 16, 64);
    zp += __shfl_xor(zp, 32, 64);
    zq = zp;
    L = page_limbs<BITS>(qv);
    const float4* vrow = reinterpret_cast<const float4*>(&cps[par][2][8 * n]);
    const float4* vzrow = reinterpret_cast<const float4*>(&cps[par][3][8 * n]);
    const float4 d0 = vrow[0], d1 = vrow[1], e0 = vzrow[0], e1 = vzrow[1];
    const float dd[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
    const float ee[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      dv[m] = dd[m];
      zv[m] = __builtin_fmaf(-VBias<BITS>::value, dd[m], ee[m]);
    }
  };
  auto page_end = [&](int p) {
    // fold the page's PV product into the output: scale (.) accp + (zero - B scale) sum_t p_t s_t
    float swc = sw;
    swc += __shfl_xor(swc, 16, 64);
    swc += __shfl_xor(swc, 32, 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float swi = __shfl(swc, 4 * G + i, 64);
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m][i] = __builtin_fmaf(dv[m], accp[m][i], __builtin_fmaf(zv[m], swi, acc[m][i]));
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) accp[m] = v4f{0.f, 0.f, 0.f, 0.f};
    sw = 0.f;
    // the next page's parameters (loaded a page ago) into the other buffer; the one after starts loading
    if (p + 1 < p_end) stage_params((p + 1) & 1, prm);
    prm = load_params(page_id(min(p + 2, p_end - 1)));
  };

  auto step = [&](const PcTile (&c)[kNT], const int64_t (&pg)[kNT], int tile, const PcTile (&next)[kNT], int buf) {
    const int p = tile >> tpp_shift;
    if ((tile & (tpp - 1)) == 0) page_begin(p);
    v4i sc[kNT];
    {
      v4i s0[kNT], s1[kNT], s2[kNT];
#pragma unroll
      for (int u = 0; u < kNT; ++u) {
        const v4i k0 = k_operand<BITS>(c[u].k, 0);
        s0[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(k0, L.l0[0], v4i{0, 0, 0, 0}, 0, 0, 0);
        s1[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(k0, L.l1[0], v4i{0, 0, 0, 0}, 0, 0, 0);
        s2[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(k0, L.l2[0], v4i{0, 0, 0, 0}, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kNT; ++u) {
        const v4i k1 = k_operand<BITS>(c[u].k, 1);
        s0[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(k1, L.l0[1], s0[u], 0, 0, 0);
        s1[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(k1, L.l1[1], s1[u], 0, 0, 0);
        s2[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(k1, L.l2[1], s2[u], 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kNT; ++u) sc[u] = (((s2[u] << 8) + s1[u]) << 8) + s0[u];
    }
    // scores in log2 units: s_K,t (x 2^-E + sum_c q~_c zero_c); tokens 4G + i of tile u
    float sr[4 * kNT], sv[4 * kNT];
#pragma unroll
    for (int u = 0; u < kNT; ++u) {
      const float4 ks = szs[buf][u][G], vs = szs[buf][u][4 + G];
      const float kk[4] = {ks.x, ks.y, ks.z, ks.w};
      const float vv[4] = {vs.x, vs.y, vs.z, vs.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float t = kk[i] * __builtin_fmaf(static_cast<float>(sc[u][i]), L.inv_scale, zq);
        sr[4 * u + i] = pg[u] >= 0 ? t : kNegInf;
        sv[4 * u + i] = vv[i];
      }
    }
    float mt = sr[0];
#pragma unroll
    for (int i = 1; i < 4 * kNT; ++i) mt = fmaxf(mt, sr[i]);
    mt = max_over_rows(mt);
    if (__any(mt > m_run + kLazyRescale)) {
      const float m_new = (mt > m_run + kLazyRescale) ? mt : m_run;
      const float alpha = (m_run == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_part *= alpha;
      sw *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * G + i, 64);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          acc[m][i] *= ai;
          accp[m][i] *= ai;
        }
      }
    }
    const float m_ref = (m_run == kNegInf) ? 0.f : m_run;
    float w[4 * kNT];
#pragma unroll
    for (int i = 0; i < 4 * kNT; ++i) {
      const float pv = __builtin_amdgcn_exp2f(sr[i] - m_ref);  // -inf -> 0
      l_part += pv;
      w[i] = (sr[i] == kNegInf) ? 0.f : pv * sv[i];
      sw += w[i];
    }
    uint32_t h01a, h23a, l01a, l23a, h01b, h23b, l01b, l23b;
    split_bf16({w[0], w[1], w[2], w[3]}, h01a, h23a, l01a, l23a);
    split_bf16({w[4], w[5], w[6], w[7]}, h01b, h23b, l01b, l23b);
    const v8bf p_hi = as_bf(v4u{h01a, h23a, h01b, h23b});
    const v8bf p_lo = as_bf(v4u{l01a, l23a, l01b, l23b});
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint32_t na = v_bf16_low_bytes<BITS>(c[0].v, m, c80);
      const uint32_t nb = v_bf16_low_bytes<BITS>(c[1].v, m, c80);
      const v8bf vb = as_bf(v4u{bias_bf16_lo<BITS>(na), bias_bf16_hi<BITS>(na), bias_bf16_lo<BITS>(nb),
                                bias_bf16_hi<BITS>(nb)});
      accp[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p_hi, vb, accp[m], 0, 0, 0);
      accp[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p_lo, vb, accp[m], 0, 0, 0);
    }
    if (((tile + kNT) & (tpp - 1)) == 0) page_end(p);
#pragma unroll
    for (int u = 0; u < kNT; ++u) reinterpret_cast<float*>(szs[buf ^ 1][u])[lane] = next[u].s;
    wave_lds_sync();
  };

  for (int tile = tile_begin;; tile += 6 * kNT) {
    fetch(tile + 2 * kNT, x2, pg2);
    step(x0, pg0, tile, x1, 0);
    if (tile + kNT >= tile_end) break;
    fetch(tile + 3 * kNT, x0, pg0);
    step(x1, pg1, tile + kNT, x2, 1);
    if (tile + 2 * kNT >= tile_end) break;
    fetch(tile + 4 * kNT, x1, pg1);
    step(x2, pg2, tile + 2 * kNT, x0, 0);
    if (tile + 3 * kNT >= tile_end) break;
    fetch(tile + 5 * kNT, x2, pg2);
    step(x0, pg0, tile + 3 * kNT, x1, 1);
    if (tile + 4 * kNT >= tile_end) break;
    fetch(tile + 6 * kNT, x0, pg0);
    step(x1, pg1, tile + 4 * kNT, x2, 0);
    if (tile + 5 * kNT >= tile_end) break;
    fetch(tile + 7 * kNT, x1, pg1);
    step(x2, pg2, tile + 5 * kNT, x0, 1);
    if (tile + 6 * kNT >= tile_end) break;
  }

  // ---- partial of this split in the original basis: R acc (R is its own inverse)
  l_part += __shfl_xor(l_part, 16, 64);
  l_part += __shfl_xor(l_part, 32, 64);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 4 * G + i;
    const float lr = __shfl(l_part, c, 64);
    const float mr = __shfl(m_run, c, 64);
    float o[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) o[m] = acc[m][i];
    fwht_row16_planned(o, a.rot, lf);
    if (c < g) {
      const int64_t row = split * pairs + static_cast<int64_t>(b) * a.num_q_heads + static_cast<int64_t>(kvh) * g + c;
      float4* dst = reinterpret_cast<float4*>(a.ws_acc + row * kHeadDim + 8 * lf.pos);
      dst[0] = make_float4(o[0], o[1], o[2], o[3]);
      dst[1] = make_float4(o[4], o[5], o[6], o[7]);
      if (n == 0) reinterpret_cast<float2*>(a.ws_ml)[row] = make_float2(mr, lr);
    }
  }
}

}  // namespace

hipError_t launch_pc_decode(const PcDecodeArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.num_splits + 1), static_cast<unsigned>(a.num_kv_heads),
                  static_cast<unsigned>(a.batch));
  if (a.bits == 4) hipLaunchKernelGGL(pc_decode_kernel<4>, grid, dim3(64), 0, stream, a);
  else hipLaunchKernelGGL(pc_decode_kernel<2>, grid, dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // merge every split (empty ones weigh nothing); the partials are already in the original basis
  DecodeArgs m{};
  m.rot = make_row_fwht_plan(1);
  m.page_size = a.page_size;
  m.context_lens = a.context_lens;
  m.max_context_len = a.max_context_len;
  m.batch = a.batch;
  m.num_q_heads = a.num_q_heads;
  m.num_kv_heads = a.num_kv_heads;
  m.num_splits = a.num_splits + 1;
  m.pages_per_split = a.pages_per_split;
  m.all_splits = 1;
  m.ws_acc = a.ws_acc;
  m.ws_ml = a.ws_ml;
  m.out = a.out;
  return launch_decode_merge(m, stream);
}

}  // namespace kvq
