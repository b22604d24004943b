// Baseline for the low-bit path: paged decode attention over an unquantized bf16 cache - the
// kind of BF16 split decode (FlashDecoding-v2, named in the OScaR abstract on the thelatestinai.com
// page) against which the pages state their decode speed-ups. Same split-K structure, softmax and
// merge as the INT4/INT2 read path, so that the two differ only in what a token costs to read:
// 512 bytes of bf16 K+V per token and head here against 144 (INT4) or 80 (INT2).
//
// Cache (per page and KV head): K [page_size][128] bf16, token-major; V [page_size / 16][128][16]
// bf16, channel-major inside each run of 16 tokens, so that the PV matrix-core operand (16
// channels x 8 tokens per lane group) is two contiguous 8-byte loads per lane.
//
// QK^T (v_mfma_f32_16x16x32_bf16): A = 16 tokens x 32 channels of K, B = the query (bf16, exact)
// of up to 16 heads; four k-steps cover the 128 channels. Output lane (G, n) holds head n, tokens
// 4G..4G+3. PV (same instruction): A = p of head n for tokens 4G..4G+3 of two tiles, split into bf16
// hi + lo; B = V of 16 channels for the same 8 tokens. Output lane (G, c) holds heads 4G..4G+3,
// channel 16m + c of block m.
#include <type_traits>

#include "kvq_device.h"
#include "kvq_launch.h"
#include "kvq_mfma.h"

namespace kvq {
namespace {

// Loads of one 16-token tile for one lane: K rows (A operand of the four QK k-steps) and the V
// words of the lane's channel in each of the eight 16-channel blocks.
struct Bf16Tile {
  uint4 k[4];
  uint2 v[8];
};

// ---------------------------------------------------------------------------- cache write

__global__ __launch_bounds__(256) void bf16_cache_write_kernel(const Bf16WriteArgs a) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int h = blockIdx.y;
  const int oct = threadIdx.x & 15;  // channels 8 oct .. 8 oct + 7
  if (t >= a.num_tokens) return;
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t page = slot / a.page_size;
  const int off = static_cast<int>(slot - page * a.page_size);
  const int64_t tile = page * a.num_kv_heads + h;
  const uint4 kw = *reinterpret_cast<const uint4*>(a.k + t * a.k_stride + h * kHeadDim + 8 * oct);
  const uint4 vw = *reinterpret_cast<const uint4*>(a.v + t * a.v_stride + h * kHeadDim + 8 * oct);
  *reinterpret_cast<uint4*>(a.k_cache + (tile * a.page_size + off) * kHeadDim + 8 * oct) = kw;
  uint16_t* vdst = a.v_cache + ((tile * (a.page_size / 16) + off / 16) * kHeadDim + 8 * oct) * 16 + (off & 15);
  const uint32_t w[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) vdst[16 * j] = static_cast<uint16_t>(w[j >> 1] >> (16 * (j & 1)));
}

// ---------------------------------------------------------------------------- decode

__global__ __launch_bounds__(64, 2) void decode_bf16_kernel(const DecodeBf16Args a) {
  const int lane = threadIdx.x;
  const int G = lane >> 4;
  const int n = lane & 15;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int g = a.num_q_heads / a.num_kv_heads;
  const int ps = a.page_size;
  const int tiles_per_page = ps / 16;
  const int len = min(max(ro_load(a.context_lens, b), 0), a.max_context_len);
  const int n_pages = (len + ps - 1) / ps;
  const int p_begin = split * a.pages_per_split;
  const int p_end = (split == a.num_splits - 1) ? n_pages : min(n_pages, p_begin + a.pages_per_split);
  const int64_t head0 = static_cast<int64_t>(b) * a.num_q_heads + static_cast<int64_t>(kvh) * g;

  if (p_begin >= p_end) {
    if (a.num_splits == 1) {
      for (int h = G; h < g; h += 4) {
        float4* o = reinterpret_cast<float4*>(a.out + (head0 + h) * kHeadDim + n * 8);
        o[0] = make_float4(0.f, 0.f, 0.f, 0.f);
        o[1] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    return;
  }
  const int tile_begin = p_begin * tiles_per_page;
  const int tile_end = min(p_end * tiles_per_page, (len + 15) / 16);
  const int last_tile = tile_end - 1;
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.max_pages_per_seq;

  // query (B operand of QK): head n, channels 32 s + 8 G .. + 7
  v4u qb[4];
  {
    const int h = min(n, g - 1);
    const uint16_t* qp = a.q + (head0 + h) * kHeadDim + 8 * G;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 x = *reinterpret_cast<const uint4*>(qp + 32 * s);
      qb[s] = (n < g) ? v4u{x.x, x.y, x.z, x.w} : v4u{0u, 0u, 0u, 0u};
    }
  }

  // Tile t of the split: page and position of its 16 tokens; past the split's end the last tile
  // is read again (masked), an invalid page id reads page 0 (masked).
  auto tile_page = [&](int t, int& valid) -> int64_t {
    const int tt = min(t, last_tile);
    const int32_t p = ro_load(bt, tt / tiles_per_page);
    const bool ok = p >= 0 && p < a.num_pages;
    valid = (ok && t <= last_tile) ? 1 : 0;
    return (static_cast<int64_t>(ok ? p : 0) * a.num_kv_heads + kvh) * tiles_per_page + tt % tiles_per_page;
  };
  auto load = [&](int t, Bf16Tile& x, int& valid) {
    const int64_t sub = tile_page(t, valid);  // (page, head, 16-token run) index
    const uint16_t* kp = a.k_cache + (sub * 16 + n) * kHeadDim + 8 * G;  // lane (G, t=n): token n
#pragma unroll
    for (int s = 0; s < 4; ++s) x.k[s] = *reinterpret_cast<const uint4*>(kp + 32 * s);
    const uint16_t* vp = a.v_cache + sub * (kHeadDim * 16) + n * 16 + 4 * G;  // channel 16m + n, tokens 4G..
#pragma unroll
    for (int m = 0; m < 8; ++m) x.v[m] = *reinterpret_cast<const uint2*>(vp + 16 * 16 * m);
  };

  v4f acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;  // running maximum of head n (log2 units)
  float l_part = 0.f;     // this lane's share of sum p for head n

  auto step = [&](const Bf16Tile (&x)[2], const int (&valid)[2], int t0) {
    float sr[8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      v4f s4 = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 kk = x[u].k[s];
        s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(v4u{kk.x, kk.y, kk.z, kk.w}), as_bf(qb[s]), s4, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = valid[u] && (t0 + u) * 16 + 4 * G + i < len;
        sr[4 * u + i] = ok ? s4[i] * a.qk_scale_log2 : kNegInf;
      }
    }
    float mt = sr[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sr[i]);
    mt = max_over_rows(mt);
    if (__any(mt > m_run + kLazyRescale)) {
      const float m_new = (mt > m_run + kLazyRescale) ? mt : m_run;
      const float alpha = (m_run == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * G + i, 64);
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[m][i] *= ai;
      }
    }
    const float m_ref = (m_run == kNegInf) ? 0.f : m_run;
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = __builtin_amdgcn_exp2f(sr[i] - m_ref);  // 0 for masked tokens
      l_part += p[i];
    }
    uint32_t h0[2], l0[2], h1[2], l1[2];
    split_bf16({p[0], p[1], p[2], p[3]}, h0[0], h0[1], l0[0], l0[1]);
    split_bf16({p[4], p[5], p[6], p[7]}, h1[0], h1[1], l1[0], l1[1]);
    const v8bf p_hi = as_bf(v4u{h0[0], h0[1], h1[0], h1[1]});
    const v8bf p_lo = as_bf(v4u{l0[0], l0[1], l1[0], l1[1]});
    // masked tokens may hold anything in the cache (even NaN): zero their V entries
    uint32_t keep[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int w = 0; w < 2; ++w)
        keep[u][w] = (sr[4 * u + 2 * w] == kNegInf ? 0u : 0xFFFFu) | (sr[4 * u + 2 * w + 1] == kNegInf ? 0u : 0xFFFF0000u);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const v4u vb = v4u{x[0].v[m].x & keep[0][0], x[0].v[m].y & keep[0][1], x[1].v[m].x & keep[1][0],
                         x[1].v[m].y & keep[1][1]};
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p_hi, as_bf(vb), acc[m], 0, 0, 0);
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p_lo, as_bf(vb), acc[m], 0, 0, 0);
    }
  };

  // double-buffered walk over steps of two tiles
  Bf16Tile xa[2], xb[2];
  int va[2], vb[2];
  load(tile_begin, xa[0], va[0]);
  load(tile_begin + 1, xa[1], va[1]);
  for (int t = tile_begin;; t += 4) {
    load(t + 2, xb[0], vb[0]);
    load(t + 3, xb[1], vb[1]);
    step(xa, va, t);
    if (t + 2 >= tile_end) break;
    load(t + 4, xa[0], va[0]);
    load(t + 5, xa[1], va[1]);
    step(xb, vb, t + 2);
    if (t + 4 >= tile_end) break;
  }

  // ---- finish: totals of head n, moved to the accumulator rows (heads 4G + i)
  l_part += __shfl_xor(l_part, 16, 64);
  l_part += __shfl_xor(l_part, 32, 64);
  float lrow[4], mrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lrow[i] = __shfl(l_part, 4 * G + i, 64);
    mrow[i] = __shfl(m_run, 4 * G + i, 64);
  }
  const int64_t pairs = static_cast<int64_t>(a.batch) * a.num_q_heads;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * G + i;
    if (h >= g) continue;
    if (a.num_splits == 1) {
      const float inv_l = 1.0f / lrow[i];
      float* o = a.out + (head0 + h) * kHeadDim + n;
#pragma unroll
      for (int m = 0; m < 8; ++m) o[16 * m] = acc[m][i] * inv_l;
    } else {
      const int64_t row = static_cast<int64_t>(split) * pairs + head0 + h;
      float* o = a.ws_acc + row * kHeadDim + n;
#pragma unroll
      for (int m = 0; m < 8; ++m) o[16 * m] = acc[m][i];
      if (n == 0) reinterpret_cast<float2*>(a.ws_ml)[row] = make_float2(mrow[i], lrow[i]);
    }
  }
}

}  // namespace

hipError_t launch_bf16_write(const Bf16WriteArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((a.num_tokens + 15) / 16), static_cast<unsigned>(a.num_kv_heads));
  hipLaunchKernelGGL(bf16_cache_write_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_bf16(const DecodeBf16Args& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.num_splits), static_cast<unsigned>(a.num_kv_heads),
                  static_cast<unsigned>(a.batch));
  hipLaunchKernelGGL(decode_bf16_kernel, grid, dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_splits == 1) return e;
  DecodeArgs m{};
  m.page_size = a.page_size;
  m.context_lens = a.context_lens;
  m.max_context_len = a.max_context_len;
  m.batch = a.batch;
  m.num_q_heads = a.num_q_heads;
  m.num_kv_heads = a.num_kv_heads;
  m.rot = make_row_fwht_plan(1);  // no rotation to undo
  m.out = a.out;
  m.num_splits = a.num_splits;
  m.pages_per_split = a.pages_per_split;
  m.ws_acc = a.ws_acc;
  m.ws_ml = a.ws_ml;
  return launch_decode_merge(m, stream);
}

}  // namespace kvq
