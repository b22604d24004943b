// Read path: paged decode attention over the rotated INT4/INT2 cache, dequantized on the fly,
// split over pages with an online-softmax (log-sum-exp) merge, one inverse Hadamard on the output.
//
// Sources: dequantization fused into the attention kernel (ainews.cool "Technical Deep Dive",
// third phase); a paged low-bit attention kernel (OSCAR abstract, thelatestinai.com page); split
// decoding as in FlashDecoding-v2, the baseline the OScaR abstract compares against. Scores are
// taken in the rotated basis: (R q) . (R k) = q . k because R is orthonormal, and sum_j p_j R v_j =
// R (sum_j p_j v_j), so a single R^T (= R) on the output undoes the V rotation.
//
// This is the VALU kernel: one wave per (split, kv head, sequence); a 16-lane row group takes one
// token at a time (lane i: channels 8i..8i+7), four tokens per wave step, each row group keeping
// its own running (max, sum, accumulator) per query head; the four are merged at the end.
#include <algorithm>

#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {
namespace {

constexpr float kNegInf = -__builtin_inff();

template <int BITS>
__device__ __forceinline__ uint32_t load_k_codes(const uint8_t* tile, int off, int li) {
  constexpr int kRow = kHeadDim * BITS / 8;
  if constexpr (BITS == 4) {
    return *reinterpret_cast<const uint32_t*>(tile + off * kRow + li * 4);
  } else {
    return *reinterpret_cast<const uint16_t*>(tile + off * kRow + li * 2);
  }
}

// V tile: byte j of token t at ((t / 4) * row + j) * 4 + t % 4. Returns the packed codes of
// channels 8 li .. 8 li + 7 of token t (same packing as a K row word).
template <int BITS>
__device__ __forceinline__ uint32_t load_v_codes(const uint8_t* tile, int t, int li) {
  constexpr int kRow = kHeadDim * BITS / 8;
  const int sh = 8 * (t & 3);
  const uint8_t* p = tile + ((t >> 2) * kRow) * 4;
  if constexpr (BITS == 4) {
    const uint4 w = *reinterpret_cast<const uint4*>(p + li * 16);
    return ((w.x >> sh) & 0xFFu) | (((w.y >> sh) & 0xFFu) << 8) | (((w.z >> sh) & 0xFFu) << 16) |
           (((w.w >> sh) & 0xFFu) << 24);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(p + li * 8);
    return ((w.x >> sh) & 0xFFu) | (((w.y >> sh) & 0xFFu) << 8);
  }
}

template <int BITS>
__device__ __forceinline__ void dequant8(uint32_t codes, float2 sz, float (&x)[8]) {
  constexpr uint32_t kMask = (1u << BITS) - 1u;
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = __builtin_fmaf(static_cast<float>((codes >> (BITS * k)) & kMask), sz.x, sz.y);
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

template <int BITS, int G>
__global__ __launch_bounds__(64) void decode_valu_kernel(const DecodeArgs a) {
  const int lane = threadIdx.x;
  const int grp = lane >> 4;
  const int li = lane & 15;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int ps = a.page_size;
  const int len = min(max(a.context_lens[b], 0), a.max_context_len);
  const int n_pages = (len + ps - 1) / ps;
  const int p_begin = split * a.pages_per_split;
  // the last split also takes the pages past num_splits * pages_per_split (see plan_splits)
  const int p_end = (split == a.num_splits - 1) ? n_pages : min(n_pages, p_begin + a.pages_per_split);
  const int64_t q_row0 = (static_cast<int64_t>(b) * a.num_q_heads + kvh * G) * kHeadDim;

  if (p_begin >= p_end) {
    // Nothing to attend in this split. Unsplit calls own the output row: an empty sequence
    // attends to nothing and yields zeros. Split calls leave it to the merge kernel.
    if (a.num_splits == 1 && grp == 0) {
      for (int h = 0; h < G; ++h) {
        float4* o = reinterpret_cast<float4*>(a.out + q_row0 + h * kHeadDim + li * 8);
        o[0] = make_float4(0.f, 0.f, 0.f, 0.f);
        o[1] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    return;
  }

  // Rotated, pre-scaled query (log2 domain): q~ = R q * softmax_scale * log2(e).
  float q[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 w = *reinterpret_cast<const uint4*>(a.q + q_row0 + h * kHeadDim + li * 8);
    bf16x8_to_f32(w, q[h]);
    if (!a.q_prerotated) {
      fwht_row16(q[h], a.hb, li);
#pragma unroll
      for (int k = 0; k < 8; ++k) q[h][k] *= a.inv_sqrt_hb;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) q[h][k] *= a.qk_scale_log2;
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[h][k] = 0.f;
  }

  constexpr int kRow = kHeadDim * BITS / 8;
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.max_pages_per_seq;
  for (int pi = p_begin; pi < p_end; ++pi) {
    const int32_t page = bt[pi];
    if (page < 0 || page >= a.num_pages) continue;  // a corrupt table entry reads nothing
    const int64_t tile = static_cast<int64_t>(page) * a.num_kv_heads + kvh;
    const uint8_t* kt = a.k_codes + tile * ps * kRow;
    const uint8_t* vt = a.v_codes + tile * ps * kRow;
    const float2* ksz = reinterpret_cast<const float2*>(a.k_sz) + tile * ps;
    const float2* vsz = reinterpret_cast<const float2*>(a.v_sz) + tile * ps;
    const int tok0 = pi * ps;
    for (int it = 0; it < ps / 4; ++it) {
      const int off = it * 4 + grp;
      const bool valid = tok0 + off < len;
      float kf[8], vf[8];
      dequant8<BITS>(load_k_codes<BITS>(kt, off, li), ksz[off], kf);
      dequant8<BITS>(load_v_codes<BITS>(vt, off, li), vsz[off], vf);
      if (!valid) {
#pragma unroll
        for (int k = 0; k < 8; ++k) vf[k] = 0.f;  // rows past the end may hold anything
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) d = __builtin_fmaf(q[h][k], kf[k], d);
        d = row16_sum(d);
        const float s = valid ? d : kNegInf;
        const float mn = fmaxf(m[h], s);
        const float alpha = (mn == kNegInf) ? 1.f : exp2f(m[h] - mn);
        const float p = (mn == kNegInf) ? 0.f : exp2f(s - mn);
        l[h] = __builtin_fmaf(l[h], alpha, p);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[h][k] = __builtin_fmaf(acc[h][k], alpha, p * vf[k]);
        m[h] = mn;
      }
    }
  }

  // Merge the four row groups (lanes xor 16, xor 32).
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mo = fmaxf(m[h], shfl_xor_f(m[h], 16));
    mo = fmaxf(mo, shfl_xor_f(mo, 32));
    const float sc = (m[h] == kNegInf) ? 0.f : exp2f(m[h] - mo);
    float lh = l[h] * sc;
    lh += shfl_xor_f(lh, 16);
    lh += shfl_xor_f(lh, 32);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float v = acc[h][k] * sc;
      v += shfl_xor_f(v, 16);
      v += shfl_xor_f(v, 32);
      acc[h][k] = v;
    }
    m[h] = mo;
    l[h] = lh;
  }

  if (a.num_splits == 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float o[8];
      const float inv_l = 1.0f / l[h];
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = acc[h][k] * inv_l;
      fwht_row16(o, a.hb, li);
      if (grp == 0) {
        float4* dst = reinterpret_cast<float4*>(a.out + q_row0 + h * kHeadDim + li * 8);
        dst[0] = make_float4(o[0] * a.inv_sqrt_hb, o[1] * a.inv_sqrt_hb, o[2] * a.inv_sqrt_hb, o[3] * a.inv_sqrt_hb);
        dst[1] = make_float4(o[4] * a.inv_sqrt_hb, o[5] * a.inv_sqrt_hb, o[6] * a.inv_sqrt_hb, o[7] * a.inv_sqrt_hb);
      }
    }
  } else if (grp == 0) {
    const int64_t base = (static_cast<int64_t>(split) * a.batch + b) * a.num_q_heads + kvh * G;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float4* dst = reinterpret_cast<float4*>(a.ws_acc + (base + h) * kHeadDim + li * 8);
      dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
      if (li == 0) reinterpret_cast<float2*>(a.ws_ml)[base + h] = make_float2(m[h], l[h]);
    }
  }
}

// Log-sum-exp merge of the splits of one (sequence, query head) per 16-lane row group, then
// the inverse rotation and the store.
__global__ __launch_bounds__(64) void decode_merge_kernel(const DecodeArgs a) {
  const int lane = threadIdx.x;
  const int grp = lane >> 4;
  const int li = lane & 15;
  const int64_t pairs = static_cast<int64_t>(a.batch) * a.num_q_heads;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 4 + grp;
  const bool live = idx < pairs;
  const int b = live ? static_cast<int>(idx / a.num_q_heads) : 0;
  const int len = live ? min(max(a.context_lens[b], 0), a.max_context_len) : 0;
  const int n_pages = (len + a.page_size - 1) / a.page_size;
  const int n_used = min(a.num_splits, (n_pages + a.pages_per_split - 1) / a.pages_per_split);

  float mo = kNegInf;
  for (int s = 0; s < n_used; ++s) {
    mo = fmaxf(mo, reinterpret_cast<const float2*>(a.ws_ml)[s * pairs + idx].x);
  }
  float lsum = 0.f, o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = 0.f;
  for (int s = 0; s < n_used; ++s) {
    const float2 ml = reinterpret_cast<const float2*>(a.ws_ml)[s * pairs + idx];
    const float sc = exp2f(ml.x - mo);
    lsum = __builtin_fmaf(ml.y, sc, lsum);
    const float4* src = reinterpret_cast<const float4*>(a.ws_acc + (s * pairs + idx) * kHeadDim + li * 8);
    const float4 x0 = src[0], x1 = src[1];
    o[0] = __builtin_fmaf(x0.x, sc, o[0]); o[1] = __builtin_fmaf(x0.y, sc, o[1]);
    o[2] = __builtin_fmaf(x0.z, sc, o[2]); o[3] = __builtin_fmaf(x0.w, sc, o[3]);
    o[4] = __builtin_fmaf(x1.x, sc, o[4]); o[5] = __builtin_fmaf(x1.y, sc, o[5]);
    o[6] = __builtin_fmaf(x1.z, sc, o[6]); o[7] = __builtin_fmaf(x1.w, sc, o[7]);
  }
  const float inv_l = (n_used > 0) ? 1.0f / lsum : 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] *= inv_l;
  fwht_row16(o, a.hb, li);
  if (live) {
    float4* dst = reinterpret_cast<float4*>(a.out + idx * kHeadDim + li * 8);
    dst[0] = make_float4(o[0] * a.inv_sqrt_hb, o[1] * a.inv_sqrt_hb, o[2] * a.inv_sqrt_hb, o[3] * a.inv_sqrt_hb);
    dst[1] = make_float4(o[4] * a.inv_sqrt_hb, o[5] * a.inv_sqrt_hb, o[6] * a.inv_sqrt_hb, o[7] * a.inv_sqrt_hb);
  }
}

template <int BITS>
hipError_t launch_valu_bits(const DecodeArgs& a, int g, dim3 grid, hipStream_t stream) {
  const dim3 block(64);
  switch (g) {
    case 1: hipLaunchKernelGGL((decode_valu_kernel<BITS, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_valu_kernel<BITS, 2>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((decode_valu_kernel<BITS, 3>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_valu_kernel<BITS, 4>), grid, block, 0, stream, a); break;
    case 5: hipLaunchKernelGGL((decode_valu_kernel<BITS, 5>), grid, block, 0, stream, a); break;
    case 6: hipLaunchKernelGGL((decode_valu_kernel<BITS, 6>), grid, block, 0, stream, a); break;
    case 7: hipLaunchKernelGGL((decode_valu_kernel<BITS, 7>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((decode_valu_kernel<BITS, 8>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

SplitPlan plan_splits(int32_t batch, int32_t num_kv_heads, int32_t max_context_len, int32_t page_size,
                      int32_t pages_per_split_request) {
  const int64_t max_pages = (static_cast<int64_t>(max_context_len) + page_size - 1) / page_size;
  SplitPlan p{1, static_cast<int32_t>(max_pages > 0 ? max_pages : 1)};
  if (max_pages <= 0) return p;
  int64_t pps;
  if (pages_per_split_request > 0) {
    pps = pages_per_split_request;
  } else {
    // Aim for about 2048 waves (8 per CU on 256 CUs) so every CU has several waves of loads
    // in flight; never split below 8 pages (128 tokens) per wave.
    const int64_t items = static_cast<int64_t>(batch) * num_kv_heads;
    int64_t splits = (2048 + items - 1) / items;
    splits = std::max<int64_t>(1, std::min<int64_t>(splits, (max_pages + 7) / 8));
    // Split size rounded down to an even number of pages (the matrix-core kernel walks two pages
    // per step, so only the last split can end in a half-empty step). The pages left over after
    // the last full split go to that split when they are at most half a split (e.g. the page
    // of the newest token); only a larger remainder gets a split of its own.
    pps = std::max<int64_t>(1, max_pages / splits);
    if (splits > 1 && pps > 8) pps &= ~int64_t{1};
    const int64_t full = max_pages / pps, rem = max_pages % pps;
    p.pages_per_split = static_cast<int32_t>(pps);
    p.num_splits = static_cast<int32_t>(std::max<int64_t>(1, full + (2 * rem > pps ? 1 : 0)));
    return p;
  }
  pps = std::max<int64_t>(1, std::min<int64_t>(pps, max_pages));
  p.pages_per_split = static_cast<int32_t>(pps);
  p.num_splits = static_cast<int32_t>((max_pages + pps - 1) / pps);
  return p;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const int g = a.num_q_heads / a.num_kv_heads;
  const dim3 grid(static_cast<unsigned>(a.num_splits), static_cast<unsigned>(a.num_kv_heads),
                  static_cast<unsigned>(a.batch));
  if (!a.use_valu) return launch_decode_mfma(a, stream);  // launches its own merge
  hipError_t e = (a.bits == 4) ? launch_valu_bits<4>(a, g, grid, stream) : launch_valu_bits<2>(a, g, grid, stream);
  if (e != hipSuccess || a.num_splits == 1) return e;
  const int64_t pairs = static_cast<int64_t>(a.batch) * a.num_q_heads;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(static_cast<unsigned>((pairs + 3) / 4)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
