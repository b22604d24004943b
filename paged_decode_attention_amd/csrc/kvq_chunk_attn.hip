// Several queries per sequence, large chunks (chunked prefill): the causal attention of a
// sequence's last q_len tokens over its paged low-bit cache, with every cache tile staged once per
// workgroup in LDS and shared by the workgroup's 256 (query, head) columns (the paged low-bit
// attention of the OSCAR abstract on thelatestinai.com, with dequantization fused into the
// attention as in ainews.cool "Technical Deep Dive", phase 3).
//
// A workgroup of eight waves takes 256 columns of one (sequence, KV head) item - column c is
// query c / g, head c % g - and walks the sequence in 64-token tiles. Each of the first four waves
// loads one 16-token sub-tile (K and V codes, scale/zero) a tile ahead and stages it in LDS; the
// other four only compute, so on each SIMD one wave starts its matrix work on a tile while the
// other still stages the next one:
//   K: the codes themselves as fp16 integers (exact), token-major, with each token's scale and zero
//      beside them;
//   V: dequantized to fp16 (d c + z, rounded once), channel-major, scaled by a power of two E that
//      only grows along the walk: the largest of the V magnitudes seen so far, this tile's
//      included (each wave publishes its sub-tile's a tile ahead), sits in [2^13, 2^14).
// Every wave computes, for its 32 columns, on the matrix cores (v_mfma_f32_16x16x32_f16):
//   score = scale_j (q . c_j) + zero_j sum(q)
// with q split into fp16 hi + lo parts (two passes, about 22 significant bits: with the long-tailed
// token norms of the OScaR workload, logits reach hundreds of log2 units, and fp16 alone would move
// the weights of near-tied tokens), the zero term in fp32; then the base-2 online softmax with a
// lazy maximum, and O^T += V^T P with P in fp16; the accumulators are scaled down when E grows.
// At the end each column is normalised, rotated back (the Hadamard transform is its own inverse)
// and stored. No workspace, no split of the context: a workgroup per 256 columns per item already
// fills the chip many times over for a large chunk.
#include <algorithm>

#include "kvq_chunk.h"
#include "kvq_device.h"
#include "kvq_mfma.h"

namespace kvq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;                     // waves that stage the tiles (a 16-token sub-tile each)
constexpr int kGroups = 2;                    // groups of kWaves waves computing on the same tiles
constexpr int kWavesWg = kWaves * kGroups;
constexpr int kColsWave = 32;                 // two 16-column blocks per wave
constexpr int kColsWg = kColsWave * kWavesWg; // 256
constexpr int kColsSel = 128;                 // the unit of the large-chunk selection rule
constexpr int kTile = 16 * kWaves;            // tokens per tile: one 16-token sub-tile per wave
constexpr int kKStride = 136;                 // halves per K row in LDS (272 B: 16 rows hit distinct banks)
constexpr int kVStride = kTile + 8;           // halves per V^T row (the tile plus 16 B)
constexpr int kKBytes = kTile * kKStride * 2;
constexpr int kVBytes = kHeadDim * kVStride * 2;
constexpr int kBufBytes = kKBytes + kVBytes;  // one tile: 35,840 B; two buffers
constexpr int kQStride = 132;                 // floats per staged query row (prologue)
constexpr int kOStride = 132;                 // floats per output row (epilogue)
constexpr int kLdsBytes = (kColsWg * kQStride * 4 > 2 * kBufBytes) ? kColsWg * kQStride * 4 : 2 * kBufBytes;
static_assert(kColsWg * kOStride * 4 <= kLdsBytes, "the output rows fit");
constexpr float kLazy = 8.0f;                 // rescale when the maximum grows by more than 2^8
constexpr float kNoMag = -1000.0f;            // V exponent before any nonzero V
constexpr _Float16 kOne16 = static_cast<_Float16>(1.0f);

// Exponent e with |x| 2^-e in [2^13, 2^14) for the largest magnitude x of a block (0 for an empty
// or non-finite block), clamped so that 2^-e stays a normal float.
__device__ __forceinline__ int block_exponent(float mag) {
  if (!(mag > 0.f) || !(mag < __builtin_inff())) return 0;
  int e = 0;
  (void)frexpf(mag, &e);  // mag < 2^e
  return min(max(e - 14, -100), 100);
}

__device__ __forceinline__ float wave_max(float v) { return max_over_rows(row16_max(v)); }

// One sub-tile as this lane loads it: K codes of token l / 4 (channels 32 (l % 4) ..), V codes of
// the 4-token group l / 16 (bytes 8 l.. or 16 l.. of the sub-tile's token-interleaved V block),
// the scale/zero of K token l / 4 and of V token 4 (l / 16) + l % 4 (the lane's quad shares them).
struct SubTile {
  uint4 k, v;
  float2 ksz, vsz;
};

template <int BITS>
__device__ __forceinline__ SubTile load_subtile(const DecodeArgs& a, int64_t row0, bool ok, int lane) {
  constexpr int kRow = kHeadDim * BITS / 8;   // bytes per token row
  const uint32_t code_bytes = ok ? 16u * kRow : 0u;
  const uint32_t sz_bytes = ok ? 16u * 8u : 0u;
  const __amdgpu_buffer_rsrc_t kr = tile_rsrc(a.k_codes + row0 * kRow, code_bytes);
  const __amdgpu_buffer_rsrc_t vr = tile_rsrc(a.v_codes + row0 * kRow, code_bytes);
  const __amdgpu_buffer_rsrc_t ks = tile_rsrc(a.k_sz + row0 * 2, sz_bytes);
  const __amdgpu_buffer_rsrc_t vs = tile_rsrc(a.v_sz + row0 * 2, sz_bytes);
  SubTile s;
  // V scale/zero first: they are waited for a tile before the codes
  s.vsz = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(vs, 8 * (4 * (lane >> 4) + (lane & 3)), 0, 0));
  if constexpr (BITS == 4) {
    s.k = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, 16 * lane, 0, 2));
    s.v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, 16 * lane, 0, 2));
  } else {
    const uint2 k2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(kr, 8 * lane, 0, 2));
    const uint2 v2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(vr, 8 * lane, 0, 2));
    s.k = make_uint4(k2.x, k2.y, 0u, 0u);
    s.v = make_uint4(v2.x, v2.y, 0u, 0u);
  }
  s.ksz = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(ks, 8 * (lane >> 2), 0, 0));
  return s;
}

// Codes in four bytes (0..15) -> two dwords of fp16 integers c, bytes 0,1 and bytes 2,3: the bit
// pattern 0x6400 | c is 1024 + c, and subtracting 1024 is exact. (Normal operands: the matrix
// cores' dot products over fp16 subnormals, c 2^-24, came out about 30 times less precise.)
__device__ __forceinline__ uint32_t code_pair(uint32_t bytes, int hi) {
  const h2 x = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, bytes, hi ? 0x05030402u : 0x05010400u));
  return __builtin_bit_cast(uint32_t, x - h2{static_cast<_Float16>(1024.f), static_cast<_Float16>(1024.f)});
}

// Codes in four bytes -> fp16 of d c + z for two tokens (d0, b0) and (d1, b1), computed in fp32 as
// fma(1024 + c, d, z - 1024 d) (b holds z - 1024 d) and rounded once.
__device__ __forceinline__ uint32_t dequant_pair(uint32_t bytes, int hi, float d0, float b0, float d1, float b1) {
  const h2 x = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, bytes, hi ? 0x05030402u : 0x05010400u));
  h2 r;
  r[0] = static_cast<_Float16>(__builtin_fmaf(static_cast<float>(x[0]), d0, b0));
  r[1] = static_cast<_Float16>(__builtin_fmaf(static_cast<float>(x[1]), d1, b1));
  return __builtin_bit_cast(uint32_t, r);
}

// Position in a K row of LDS of each channel: the staging writes a code word's channels in the
// order its shifts produce them. INT4: channel 8u + 2k + h sits at 8u + 4h + k; INT2: channel
// 16u + 4k + r at 16u + 4r + k. The query is staged in the same order.
template <int BITS>
__device__ __forceinline__ int k_position(int ch) {
  if constexpr (BITS == 4) {
    return (ch & ~7) + 4 * (ch & 1) + ((ch & 7) >> 1);
  } else {
    return (ch & ~15) + 4 * (ch & 3) + ((ch & 15) >> 2);
  }
}

// V^T position of the 4-token group T (tokens 4T..4T+3 of the tile): the PV operand of lane group
// G for 32-token step s holds tokens 32s + 4G..4G+3 and 32s + 16 + 4G..4G+3 (the QK output rows of
// that lane group in the step's two 16-token blocks), so they are stored side by side.
__device__ __forceinline__ int vt_group_pos(int T) {
  const int s = T >> 3, gi = T & 7;
  return 32 * s + 8 * (gi & 3) + 4 * (gi >> 2);
}

// A V^T row's 8-half groups are stored XOR-swizzled by the row's channel bits 3..5: the staging
// lanes of a wave write channels 8 apart (rows 1,152 B apart, all on one bank otherwise), the PV
// operand reads take whole groups.
__device__ __forceinline__ int vt_swizzle(int ch, int pos) {
  return pos ^ (8 * ((ch >> 3) & 7));
}

template <int BITS>
__global__ __launch_bounds__(64 * kWavesWg, 1) void chunk_attention_kernel(const DecodeArgs a) {
  constexpr int kQmax = (1 << BITS) - 1;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  __shared__ __attribute__((aligned(16))) float2 mz[2][kTile];  // per K token: (scale 2^eQ, zero)
  __shared__ float pvalid[2][kWaves];     // per buffer and sub-tile: page valid
  __shared__ float vexp[3][kWaves];       // per tile (mod 3) and sub-tile: V exponent, published ahead
  __shared__ float qmax_w[kWavesWg];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const bool stager = w < kWaves;
  const int G = lane >> 4;
  const int n = lane & 15;
  const int g = a.num_q_heads / a.num_kv_heads;
  // Workgroups go to the eight XCDs in turn. With a multiple of eight, workgroup w takes the logical
  // block (w % 8) (n / 8) + w / 8, so each XCD runs consecutive column blocks of the same
  // (sequence, KV head) items at the same time and their tiles are read once into its L2.
  const uint32_t n_cb = static_cast<uint32_t>((a.q_len_max * g + kColsWg - 1) / kColsWg);
  const uint32_t n_wg = gridDim.x;
  const uint32_t wg = (n_wg % 8 == 0) ? (blockIdx.x % 8) * (n_wg / 8) + blockIdx.x / 8 : blockIdx.x;
  const uint32_t item = wg / n_cb;
  const int kvh = static_cast<int>(item % static_cast<uint32_t>(a.num_kv_heads));
  const int b = static_cast<int>(item / static_cast<uint32_t>(a.num_kv_heads));
  const int c0 = kColsWg * static_cast<int>(wg % n_cb);
  const int ps = a.page_size;
  const int len = min(max(ro_load(a.context_lens, b), 0), a.max_context_len);
  const int qlen = min(min(max(ro_load(a.q_lens, b), 0), a.q_len_max), len);
  const int rows_cols = a.q_len_max * g;  // columns that are rows of out
  const int valid_cols = qlen * g;        // columns with a query
  auto col_row = [&](int c) -> int64_t {
    return (static_cast<int64_t>(b) * a.q_len_max + c / g) * a.num_q_heads + static_cast<int64_t>(kvh) * g + c % g;
  };

  if (c0 >= valid_cols) {  // no query in this workgroup: its rows of out are zero
    for (int cl = 4 * w + G; cl < kColsWg; cl += 4 * kWavesWg) {
      const int c = c0 + cl;
      if (c < rows_cols) {
        float4* o = reinterpret_cast<float4*>(a.out + col_row(c) * kHeadDim + 8 * n);
        o[0] = make_float4(0.f, 0.f, 0.f, 0.f);
        o[1] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    return;
  }
  // causal limits: column c sees tokens 0 .. len - qlen + c / g
  const int lim_lo = len - qlen + c0 / g;
  const int lim_hi = len - qlen + (min(c0 + kColsWg, valid_cols) - 1) / g;
  const int n_tiles = (lim_hi + kTile) / kTile;
  const int full_tiles = (lim_lo + 1) / kTile;  // tiles every column sees whole
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.max_pages_per_seq;
  const int64_t page_rows = static_cast<int64_t>(a.num_kv_heads) * ps;

  // ---- tile loads: wave w takes tokens 64 i + 16 w .. + 15
  auto fetch = [&](int i, bool& ok) -> SubTile {
    const int tok0 = kTile * i + 16 * w;
    ok = false;
    int64_t row0 = 0;
    if (tok0 < len) {
      const int32_t p = ro_load(bt, tok0 / ps);
      ok = p >= 0 && p < a.num_pages;
      row0 = (ok ? p : 0) * page_rows + static_cast<int64_t>(kvh) * ps + tok0 % ps;
    }
    return load_subtile<BITS>(a, row0, ok, lane);
  };
  bool ok_a = false, ok_b = false;
  SubTile ta = {};
  if (stager) ta = fetch(0, ok_a);

  // ---- query: rotated (R q) and times softmax_scale * log2(e), staged as fp32 rows (buffer area,
  // K-row channel order), with the workgroup's largest magnitude; then split into fp16 hi + lo
  // with one power of two for the workgroup, and each column's sum kept in fp32
  float* const qs = reinterpret_cast<float*>(lds);
  float am = 0.f;
#pragma unroll 2
  for (int pass = 0; pass < kColsWave / 4; ++pass) {
    const int cl = kColsWave * w + 4 * pass + G;
    const int c = c0 + cl;
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (c < valid_cols) bf16x8_to_f32(*reinterpret_cast<const uint4*>(a.q + col_row(c) * kHeadDim + 8 * n), x);
    int pos = n;
    if (!a.q_prerotated) {
      const LaneFwht lf = lane_fwht(a.rot, n);
      fwht_row16_planned(x, a.rot, lf);
      pos = lf.pos;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x[k] *= a.qk_scale_log2;
      am = fmaxf(am, fabsf(x[k]));
      qs[cl * kQStride + k_position<BITS>(8 * pos + k)] = x[k];
    }
  }
  am = wave_max(am);
  if (lane == 0) qmax_w[w] = am;
  __syncthreads();
  float qm = qmax_w[0];
#pragma unroll
  for (int v = 1; v < kWavesWg; ++v) qm = fmaxf(qm, qmax_w[v]);
  const int eq = block_exponent(qm);
  const float sq = ldexpf(1.f, -eq);
  v8h qhi[2][4], qlo[2][4];
  float qsum[2];
  int lim[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int cl = kColsWave * w + 16 * cb + n;
    float s = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const float4 xa = *reinterpret_cast<const float4*>(qs + cl * kQStride + 32 * ks + 8 * G);
      const float4 xb = *reinterpret_cast<const float4*>(qs + cl * kQStride + 32 * ks + 8 * G + 4);
      const float x[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        s += x[k];
        const float y = x[k] * sq;
        const _Float16 h = static_cast<_Float16>(y);
        qhi[cb][ks][k] = h;
        qlo[cb][ks][k] = static_cast<_Float16>(y - static_cast<float>(h));
      }
    }
    s += __shfl_xor(s, 16, 64);
    s += __shfl_xor(s, 32, 64);
    qsum[cb] = s;
    lim[cb] = (c0 + cl < valid_cols) ? len - qlen + (c0 + cl) / g : -1;
  }
  const float k_mul = ldexpf(1.f, eq);  // the fp16 query is q 2^-eQ
  SubTile tb_ = ta;
  if (stager && n_tiles > 1) tb_ = fetch(1, ok_b);

  // ---- publish the V exponent of this wave's sub-tile of tile i: the largest magnitude of its
  // dequantized values (rows past the sequence excluded)
  auto publish = [&](int i, const SubTile& s, bool ok) {
    const bool vv = ok && kTile * i + 16 * w + 4 * (lane >> 4) + (lane & 3) < len;
    const float vd = vv ? s.vsz.x : 0.f, vz = vv ? s.vsz.y : 0.f;
    const float mv = wave_max(fmaxf(fabsf(vz), fabsf(__builtin_fmaf(static_cast<float>(kQmax), vd, vz))));
    if (lane == 0) vexp[i % 3][w] = (mv > 0.f) ? static_cast<float>(block_exponent(mv)) : kNoMag;
  };
  if (stager) {
    publish(0, ta, ok_a);
    if (n_tiles > 1) publish(1, tb_, ok_b);
  }
  __syncthreads();  // every wave has its query and published its first V exponents: tiles go to the buffers

  // ---- stage this wave's sub-tile of tile i in buffer buf
  auto stage = [&](int i, const SubTile& s, bool ok, int buf, float e_tile) {
    uint8_t* const kb = lds + buf * kBufBytes;
    uint8_t* const vb = kb + kKBytes;
    const int tok0 = kTile * i + 16 * w;
    // K: token tk, channels 32 qq ..; rows past the sequence may hold anything: zero scale/zero
    const int tk = lane >> 2, qq = lane & 3;
    const bool kv = ok && tok0 + tk < len;
    if (qq == 0) mz[buf][16 * w + tk] = make_float2(kv ? s.ksz.x * k_mul : 0.f, kv ? s.ksz.y : 0.f);
    _Float16* krow = reinterpret_cast<_Float16*>(kb) + (16 * w + tk) * kKStride + 32 * qq;
    if constexpr (BITS == 4) {
      const uint32_t words[4] = {s.k.x, s.k.y, s.k.z, s.k.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t t0 = words[j] & 0x0F0F0F0Fu, t1 = (words[j] >> 4) & 0x0F0F0F0Fu;
        *reinterpret_cast<uint4*>(krow + 8 * j) =
            make_uint4(code_pair(t0, 0), code_pair(t0, 1), code_pair(t1, 0), code_pair(t1, 1));
      }
    } else {
      const uint32_t words[2] = {s.k.x, s.k.y};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint32_t o[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t t = (words[j] >> (2 * r)) & 0x03030303u;
          o[2 * r] = code_pair(t, 0);
          o[2 * r + 1] = code_pair(t, 1);
        }
        *reinterpret_cast<uint4*>(krow + 16 * j) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(krow + 16 * j + 8) = make_uint4(o[4], o[5], o[6], o[7]);
      }
    }
    // V: tokens 4 tg .. 4 tg + 3, dequantized with the power of two 2^-E of this tile
    const int tg = lane >> 4;
    const bool vv = ok && tok0 + 4 * tg + (lane & 3) < len;
    const float vd_l = vv ? s.vsz.x : 0.f, vz_l = vv ? s.vsz.y : 0.f;
    // the group's four tokens from the lanes of this quad
    const float vd[4] = {dpp_f32<0x00>(vd_l), dpp_f32<0x55>(vd_l), dpp_f32<0xAA>(vd_l), dpp_f32<0xFF>(vd_l)};
    const float vz[4] = {dpp_f32<0x00>(vz_l), dpp_f32<0x55>(vz_l), dpp_f32<0xAA>(vz_l), dpp_f32<0xFF>(vz_l)};
    const float sv = (e_tile == kNoMag) ? 1.f : ldexpf(1.f, -static_cast<int>(e_tile));
    float vd2[4], vb2[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      vd2[t] = vd[t] * sv;
      vb2[t] = __builtin_fmaf(-1024.f, vd2[t], vz[t] * sv);
    }
    if (lane == 0) pvalid[buf][w] = ok ? 1.f : 0.f;
    const int vpos = vt_group_pos(4 * w + tg);
    auto put_v = [&](int ch, uint32_t bytes) {
      const uint32_t lo = dequant_pair(bytes, 0, vd2[0], vb2[0], vd2[1], vb2[1]);
      const uint32_t hi = dequant_pair(bytes, 1, vd2[2], vb2[2], vd2[3], vb2[3]);
      *reinterpret_cast<uint2*>(reinterpret_cast<_Float16*>(vb) + ch * kVStride + vt_swizzle(ch, vpos)) =
          make_uint2(lo, hi);
    };
    if constexpr (BITS == 4) {
      const uint32_t words[4] = {s.v.x, s.v.y, s.v.z, s.v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rb = (4 * lane + j) & 63;  // row byte: channels 2 rb, 2 rb + 1
        put_v(2 * rb, words[j] & 0x0F0F0F0Fu);
        put_v(2 * rb + 1, (words[j] >> 4) & 0x0F0F0F0Fu);
      }
    } else {
      const uint32_t words[2] = {s.v.x, s.v.y};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int rb = (2 * lane + j) & 31;  // row byte: channels 4 rb .. 4 rb + 3
#pragma unroll
        for (int r = 0; r < 4; ++r) put_v(4 * rb + r, (words[j] >> (2 * r)) & 0x03030303u);
      }
    }
  };

  v4f acc[2][8];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[cb][m] = v4f{0.f, 0.f, 0.f, 0.f};
  // Running maximum per column, kept as nbase = -(reference maximum) (0 before the first score)
  // and the threshold thr on a step's maximum relative to it above which the reference is raised:
  // -inf before the first score (any finite score raises it), kLazy after.
  float nbase[2] = {0.f, 0.f};
  float thr[2] = {kNegInf, kNegInf};
  float l_part[2] = {0.f, 0.f};
  float e_acc = kNoMag;  // V exponent E the accumulators are kept in (uniform)

  // ---- one tile from buffer buf, its V staged with exponent e_tile (>= e_acc)
  auto compute = [&](int i, int buf, float e_tile) {
    const uint8_t* const kb = lds + buf * kBufBytes;
    const uint8_t* const vb = kb + kKBytes;
    bool pok[kWaves], all_ok = true;
#pragma unroll
    for (int t = 0; t < kWaves; ++t) {
      pok[t] = pvalid[buf][t] != 0.f;
      all_ok = all_ok && pok[t];
    }
    // every column sees every token of the tile and every page is valid: no masks
    const bool full = all_ok && i < full_tiles;
    // E grew with this tile: the accumulators scaled down (a factor below 2^-149 is zero:
    // contributions that far below the new ones)
    if (e_tile > e_acc) {
      const float f = ldexpf(1.f, static_cast<int>(e_acc - e_tile));
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[cb][m] *= f;
      e_acc = e_tile;
    }

    // 32-token steps. Scores of 16-token blocks t = 2 st, 2 st + 1 x 16-column block cb: q . c
    // on the matrix cores (hi and lo query parts, four 32-channel steps each), then
    // x = scale (q . c) + zero sum(q) - m with the running maximum (row group G holds tokens
    // 16 t + 4 G + r of lane n's column), the maximum raised when the step's exceeds it by kLazy,
    // P = 2^x in fp16 and O^T += V^T P.
    // q . c of one step on the matrix cores: d[cb][u] for 16-token block 2 st + u
    auto qk = [&](int st, v4f (&d)[2][2]) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const _Float16* krow = reinterpret_cast<const _Float16*>(kb) + (16 * (2 * st + u) + n) * kKStride + 8 * G;
        v8h kf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kf[ks] = *reinterpret_cast<const v8h*>(krow + 32 * ks);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          v4f e = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) e = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[ks], qhi[cb][ks], e, 0, 0, 0);
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) e = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[ks], qlo[cb][ks], e, 0, 0, 0);
          d[cb][u] = e;
        }
      }
    };
    // The next step's products are issued before this step's softmax: the matrix cores work on
    // them while the vector units run the softmax.
    v4f dq[kTile / 32][2][2];
    qk(0, dq[0]);
#pragma unroll
    for (int st = 0; st < kTile / 32; ++st) {
      if (st + 1 < kTile / 32) qk(st + 1, dq[st + 1]);
      float x[2][2][4];  // [cb][block of the step][r]
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = 2 * st + u;
        const float4 u0 = *reinterpret_cast<const float4*>(&mz[buf][16 * t + 4 * G]);
        const float4 u1 = *reinterpret_cast<const float4*>(&mz[buf][16 * t + 4 * G + 2]);
        const float km[4] = {u0.x, u0.z, u1.x, u1.z};
        const float kz[4] = {u0.y, u0.w, u1.y, u1.w};
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            x[cb][u][r] = __builtin_fmaf(dq[st][cb][u][r], km[r], __builtin_fmaf(kz[r], qsum[cb], nbase[cb]));
      }

      if (!full) {  // tokens past a column's causal limit or on an invalid page
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = 2 * st + u;
              const int tok = kTile * i + 16 * t + 4 * G + r;
              x[cb][u][r] = (pok[t] && tok <= lim[cb]) ? x[cb][u][r] : kNegInf;
            }
      }

      // Step maxima per lane. Only a step whose scores pass the rescale threshold somewhere needs
      // the column maxima (over the four row groups, so that a column's lanes agree); most steps
      // skip that reduction and the rescale, for both column blocks in one branch.
      float mt[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        mt[cb] = kNegInf;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) mt[cb] = fmaxf(mt[cb], x[cb][u][r]);
      }
      if (__any(!(mt[0] <= thr[0]) || !(mt[1] <= thr[1]))) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const float mc = max_over_rows(mt[cb]);
          const bool raise = !(mc <= thr[cb]);
          const float dm = raise ? mc : 0.f;
          const float alpha = (thr[cb] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(-dm);
          nbase[cb] -= dm;
          thr[cb] = raise ? kLazy : thr[cb];
          l_part[cb] *= alpha;
#pragma unroll
          for (int m = 0; m < 8; ++m) acc[cb][m] *= alpha;
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) x[cb][u][r] -= dm;
        }
      }
      v8h pf[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        float p[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) p[u][r] = __builtin_amdgcn_exp2f(x[cb][u][r]);
        pf[cb] = v8h{static_cast<_Float16>(p[0][0]), static_cast<_Float16>(p[0][1]),
                     static_cast<_Float16>(p[0][2]), static_cast<_Float16>(p[0][3]),
                     static_cast<_Float16>(p[1][0]), static_cast<_Float16>(p[1][1]),
                     static_cast<_Float16>(p[1][2]), static_cast<_Float16>(p[1][3])};
        // the row sum takes the fp16 weights the products use, two per dot instruction (fp32 sum)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          l_part[cb] = __builtin_amdgcn_fdot2(h2{pf[cb][2 * k], pf[cb][2 * k + 1]}, h2{kOne16, kOne16}, l_part[cb], false);
      }

      // O^T += V^T P: 16-channel block m of this 32-token step
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const v8h vf = *reinterpret_cast<const v8h*>(reinterpret_cast<const _Float16*>(vb) + (16 * m + n) * kVStride +
                                                     vt_swizzle(16 * m + n, 32 * st + 8 * G));
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[cb][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[cb], acc[cb][m], 0, 0, 0);
      }
    }
  };

  // ---- the walk: tile i + 1 is staged in the buffer the previous step has released, with E from
  // the V exponents its waves published a tile earlier; tile i + 2's loads are issued, tile i
  // computes from buffer i & 1, and tile i + 2's exponents are published. Staging before the
  // compute leaves only one tile of loads in registers across it. (The loop is not unrolled: the
  // tile step is a large block of code, and instruction fetch matters.)
  auto tile_exponent = [&](int i, float e_prev) {
    const float* ve = vexp[i % 3];
#pragma unroll
    for (int v = 0; v < kWaves; ++v) e_prev = fmaxf(e_prev, ve[v]);
    return e_prev;
  };
  float e_stg = tile_exponent(0, kNoMag);  // E of the last staged tile
  if (stager) stage(0, ta, ok_a, 0, e_stg);
  __syncthreads();
#pragma unroll 1
  for (int i = 0;; ++i) {
    const float e_tile = e_stg;
    if (i + 1 < n_tiles) {
      e_stg = tile_exponent(i + 1, e_stg);
      if (stager) stage(i + 1, tb_, ok_b, (i + 1) & 1, e_stg);
    }
    SubTile tc = {};
    bool ok_c = false;
    if (stager && i + 2 < n_tiles) tc = fetch(i + 2, ok_c);
    compute(i, i & 1, e_tile);
    if (i + 1 >= n_tiles) break;
    if (stager && i + 2 < n_tiles) publish(i + 2, tc, ok_c);
    __syncthreads();
    tb_ = tc;
    ok_b = ok_c;
  }

  // ---- finish: sums over the row groups, normalise, rotate back, store
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    l_part[cb] += __shfl_xor(l_part[cb], 16, 64);
    l_part[cb] += __shfl_xor(l_part[cb], 32, 64);
  }
  __syncthreads();  // every wave is done with the tile buffers
  float* const os = reinterpret_cast<float*>(lds);
  // the lane's transform plan, rebuilt from the lane id rather than kept in registers over the walk
  const LaneFwht lf_out = lane_fwht(a.rot, static_cast<int>(__lane_id()) & 15);
  const float ev_scale = (e_acc == kNoMag) ? 0.f : ldexpf(1.f, static_cast<int>(e_acc));
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int cl = kColsWave * w + 16 * cb + n;
    // columns without a query (past q_lens) saw a zero query in the full tiles: zero output
    const float f = (lim[cb] >= 0 && l_part[cb] > 0.f) ? ev_scale / l_part[cb] : 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m)
      *reinterpret_cast<float4*>(os + cl * kOStride + 16 * m + 4 * G) =
          make_float4(acc[cb][m][0] * f, acc[cb][m][1] * f, acc[cb][m][2] * f, acc[cb][m][3] * f);
  }
  wave_lds_sync();
#pragma unroll 2
  for (int pass = 0; pass < kColsWave / 4; ++pass) {
    const int cl = kColsWave * w + 4 * pass + G;
    const int c = c0 + cl;
    const float4 xa = *reinterpret_cast<const float4*>(os + cl * kOStride + 8 * n);
    const float4 xb = *reinterpret_cast<const float4*>(os + cl * kOStride + 8 * n + 4);
    float x[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
    fwht_row16_planned(x, a.rot, lf_out);  // R^T = R: back to the original basis
    if (c < rows_cols) {
      float4* dst = reinterpret_cast<float4*>(a.out + col_row(c) * kHeadDim + 8 * lf_out.pos);
      dst[0] = make_float4(x[0], x[1], x[2], x[3]);
      dst[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
  }
}

}  // namespace

bool chunk_attention_shape(int64_t batch, int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads) {
  const int64_t cols = static_cast<int64_t>(max_q_len) * (num_q_heads / num_kv_heads);
  const int64_t blocks = (cols + kColsSel - 1) / kColsSel * num_kv_heads * batch;
  return cols >= kColsSel && blocks >= 256 && blocks * 64 * kWavesWg < (int64_t{1} << 31);
}

bool chunk_attention_applies(const DecodeArgs& a) {
  return a.q_lens && chunk_attention_shape(a.batch, a.q_len_max, a.num_q_heads, a.num_kv_heads);
}

hipError_t launch_chunk_attention(const DecodeArgs& a, hipStream_t stream) {
  const int64_t cols = static_cast<int64_t>(a.q_len_max) * (a.num_q_heads / a.num_kv_heads);
  const int64_t n_wg = (cols + kColsWg - 1) / kColsWg * a.num_kv_heads * a.batch;  // < 2^31: checked by the caller
  const dim3 grid(static_cast<unsigned>(n_wg));
  if (a.bits == 4) hipLaunchKernelGGL(chunk_attention_kernel<4>, grid, dim3(64 * kWavesWg), 0, stream, a);
  else hipLaunchKernelGGL(chunk_attention_kernel<2>, grid, dim3(64 * kWavesWg), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
