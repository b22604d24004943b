// Read path on the matrix cores: paged decode attention over the rotated INT4/INT2 cache with
// QK^T and PV on MFMA (sources as in kvq_decode.hip: dequantization fused into attention, ainews.cool
// "Technical Deep Dive"; a paged low-bit attention kernel, OSCAR abstract on thelatestinai.com;
// split decoding after FlashDecoding-v2, named in the OScaR abstract).
//
// One wave per (split, KV head, sequence) - four splits of one (sequence, KV head) to a workgroup
// when a sequence has 16 splits or more; the split's pages are walked as 16-token tiles, two
// tiles per step (four for INT2). Dequantization is folded around the contractions instead of materialised:
//   score_j = q~ . (delta_j c_j + z_j 1) = delta_j (q~ . c_j) + z_j sum(q~)
//   sum_j p_j v_j = sum_j (p_j delta_j) c_j + sum_j p_j z_j 1
// so the integer codes c_j enter the MFMAs directly.
//
// QK^T  (v_mfma_i32_16x16x64_i8): A = K codes of one tile (row = token, lane (G, t) holds 32
//   channels of token t as bytes), B = the query of the group's heads as a 21-bit fixed-point
//   integer split into three signed int8 limbs (column = head). The three limb products are
//   combined by Horner's rule (x 256 between limbs) in exact int32 arithmetic; the output lane
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
#include <type_traits>

#include "kvq_device.h"
#include "kvq_launch.h"
#include "kvq_mfma.h"

#ifndef KVQ_DECODE_NT2
#define KVQ_DECODE_NT2 4      // tiles per step of the INT2 decode (one query per sequence)
#endif
#ifndef KVQ_DECODE_MIN_WAVES
#define KVQ_DECODE_MIN_WAVES 2    // waves per SIMD the register allocation must allow
#endif

namespace kvq {
namespace {

// One 16-token tile as this lane loads it: K codes of token n (channels 32G..32G+31), V codes of
// tokens 4G..4G+3 (channels 8n..8n+7), and one float of the tile's scale/zero block (lanes 0..31:
// the 32 K floats, lanes 32..63: the 32 V floats), staged through LDS before use.
struct TileCodes {
  uint4 k;
  uint4 v;
  float sz;
};

// Per-lane byte offsets of the tile loads (constant for the whole walk).
struct LaneOffsets {
  uint32_t k, v;       // inside the K / V tile
  const float* sz;     // this lane's scale/zero array (K for lanes 0..31, V for 32..63) + lane offset
};

// The code and scale/zero loads are non-temporal (cache policy nt): every byte of the cache is
// read once per call, so it should not displace the page table, queries and partials in L2.
constexpr int kCodeAux = 2;

// Loads one tile whose first token row (in the [page][head][token] row numbering shared by the
// code and scale/zero arrays) is row0. A tile that is not live (past the split's end, or on a page
// id outside the pool) loads its codes through a zero-size buffer resource: the same instructions
// issue (fixed wait counts) and return zeros without touching memory.
template <int BITS>
__device__ __forceinline__ TileCodes load_tile(const DecodeArgs& a, int64_t row0, const LaneOffsets& lo, bool live) {
  constexpr int kRowShift = (BITS == 4) ? 6 : 5;  // log2(bytes per token row)
  const int64_t off = row0 << kRowShift;
  const uint32_t bytes = live ? (16u << kRowShift) : 0u;
  const __amdgpu_buffer_rsrc_t kr = tile_rsrc(a.k_codes + off, bytes);
  const __amdgpu_buffer_rsrc_t vr = tile_rsrc(a.v_codes + off, bytes);
  TileCodes t;
  if constexpr (BITS == 4) {
    t.k = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, lo.k, 0, kCodeAux));
    t.v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, lo.v, 0, kCodeAux));
  } else {
    const uint2 k2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(kr, lo.k, 0, kCodeAux));
    const uint2 v2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(vr, lo.v, 0, kCodeAux));
    t.k = make_uint4(k2.x, k2.y, 0, 0);
    t.v = make_uint4(v2.x, v2.y, 0, 0);
  }
  t.sz = __builtin_nontemporal_load(lo.sz + row0 * 2);
  return t;
}

// ---------------------------------------------------------------------------- fused decode step
// Rotate, optionally scale, quantize and pack the 8 channels this lane holds of one head vector
// (a 16-lane row group holds the vector): the write path for a single token, with the in-register
// butterfly instead of the matrix cores. Returns the packed codes of output block lf.pos (INT4:
// 4 bytes, INT2: 2 bytes) and the stored scale and zero (equal in the row group's 16 lanes).
template <int BITS, bool TOKEN_SCALE>
__device__ __forceinline__ uint32_t rotate_quantize_row(float (&x)[8], const RowFwhtPlan& rot, const LaneFwht& lf,
                                                        float& scale, float& zero) {
  fwht_row16_planned(x, rot, lf);
  float s = 1.0f;
  if constexpr (TOKEN_SCALE) {
    double ss = 0.0;  // RMS in double precision, rounded once to float; 1 for an all-zero vector
#pragma unroll
    for (int k = 0; k < 8; ++k) ss += static_cast<double>(x[k]) * static_cast<double>(x[k]);
    ss = row16_sum_f64(ss);
    s = static_cast<float>(sqrt(ss * (1.0 / kHeadDim)));
    if (s == 0.0f) s = 1.0f;
    if (s >= 0x1p-100f && s < 0x1p101f) {
      const float rs = rcp_rn(s);
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = div_rn(x[k], s, rs);
    } else {
      // a subnormal, tiny or huge RMS: IEEE division (its reciprocal would overflow, or the
      // correction step's residual underflow)
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = x[k] / s;
    }
  }
  float mn = fminf(fminf(fminf(x[0], x[1]), fminf(x[2], x[3])), fminf(fminf(x[4], x[5]), fminf(x[6], x[7])));
  float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  mn = row16_min(mn);
  mx = row16_max(mx);
  constexpr float kQmax = static_cast<float>((1 << BITS) - 1);
  const float delta = (mx - mn) / kQmax;  // IEEE division
  uint32_t packed = 0;
  if (delta != 0.0f) {
    // clamped to [0, qmax] before the packing rounds to an integer: the same codes as rounding first,
    // since both bounds are integers
    float c[8];
    if (delta >= 0x1p-100f && delta < 0x1p101f) {
      const float r = rcp_rn(delta);
#pragma unroll
      for (int k = 0; k < 8; ++k) c[k] = fminf(fmaxf(div_rn(x[k] - mn, delta, r), 0.0f), kQmax);
    } else {
      // a tiny or huge scale: IEEE division (see above)
#pragma unroll
      for (int k = 0; k < 8; ++k) c[k] = fminf(fmaxf((x[k] - mn) / delta, 0.0f), kQmax);
    }
    packed = pack_codes<BITS>(c);
  }
  scale = delta * s;
  zero = mn * s;
  return packed;
}

// The new token of sequence b (position len - 1) for KV head kvh: row group 0 writes K, row group
// 1 writes V (groups 2 and 3 repeat the work and store nothing). Waits until the stores are done,
// so that this wave's later loads of the same page see them (no other wave reads this page-head
// tile in the call).
template <int BITS>
__device__ __forceinline__ void append_new_token(const DecodeArgs& a, int b, int kvh, int pos, int32_t page, int lane) {
  constexpr int kRow = kHeadDim * BITS / 8;
  constexpr int kLaneBytes = 8 * BITS / 8;
  const int G = lane >> 4;
  const int li = lane & 15;
  const bool is_v = (G & 1) != 0;
  const uint16_t* src = is_v ? a.v_new + static_cast<int64_t>(b) * a.v_new_stride
                             : a.k_new + static_cast<int64_t>(b) * a.k_new_stride;
  float x[8];
  bf16x8_to_f32(*reinterpret_cast<const uint4*>(src + kvh * kHeadDim + 8 * li), x);
  const LaneFwht lf = lane_fwht(a.rot, li);
  float scale, zero;
  const uint32_t packed = a.token_scale ? rotate_quantize_row<BITS, true>(x, a.rot, lf, scale, zero)
                                        : rotate_quantize_row<BITS, false>(x, a.rot, lf, scale, zero);
  const int ps = a.page_size;
  const int off = pos % ps;
  const int64_t tile = static_cast<int64_t>(page) * a.num_kv_heads + kvh;  // (page, head) tile
  const int64_t row = tile * ps + off;
  if (G == 0) {
    uint8_t* k = a.k_codes_w + row * kRow + kLaneBytes * lf.pos;
    if constexpr (BITS == 4) {
      *reinterpret_cast<uint32_t*>(k) = packed;
    } else {
      *reinterpret_cast<uint16_t*>(k) = static_cast<uint16_t>(packed);
    }
    if (li == 0) reinterpret_cast<float2*>(a.k_sz_w)[row] = make_float2(scale, zero);
  } else if (G == 1) {
    uint8_t* v = a.v_codes_w + tile * ps * kRow + ((off >> 2) * kRow + kLaneBytes * lf.pos) * 4 + (off & 3);
#pragma unroll
    for (int m = 0; m < kLaneBytes; ++m) v[4 * m] = static_cast<uint8_t>(packed >> (8 * m));
    if (li == 0) reinterpret_cast<float2*>(a.v_sz_w)[row] = make_float2(scale, zero);
  }
  // the stores complete before any later load is issued (and the compiler moves no load above)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Rotation inside each 16-lane row (DPP row_ror): every lane takes the value of the lane R places
// along its row, wrapping around.
template <int R>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x120 + R, 0xF, 0xF, false));
}

__device__ __forceinline__ void lse_combine(float& m, float& l, float (&o)[8], int xor_mask) {
  const float m2 = __shfl_xor(m, xor_mask);
  const float l2 = __shfl_xor(l, xor_mask);
  const float mn = fmaxf(m, m2);
  const float fa = (m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
  const float fb = (m2 == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
  l = l * fa + l2 * fb;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = o[i] * fa + __shfl_xor(o[i], xor_mask) * fb;
  m = mn;
}

// MQ = false: decode, one query per sequence. The 16 columns of the QK output are F = 2 tile slots
// of W = 8 columns: column n holds query head n % W (used while below g <= 8) against the tokens
// of tile n / W of the step, so one output carries the scores of both of the step's tiles and
// every lane's softmax work is useful. The PV product then keeps one accumulator row per (tile
// slot, head); the slots are summed once, at the end. (Four slots of four columns need four-tile
// steps, which fit in registers only double-buffered; that was slower on every workload shape.)
// MQ = true: several queries per sequence (F = 1); a wave takes a tile of 16 columns out of the
// (query token, head) pairs of one KV head, column c meaning query c / g, head c % g, each with
// its own causal length.
// NT = 2 tiles per step (INT4, and several queries per sequence) or 4 (INT2 with one query per
// sequence: its tiles are half the registers, and the per-step softmax bookkeeping - the maximum
// across rows, the rescale test, the scale/zero staging - is spent once per 64 tokens), three step
// buffers.
// WG = 4 (one query per sequence, a sequence in many splits): a workgroup holds the WG splits
// 4 j .. 4 j + 3 of one (sequence, KV head) item, one per wave. Each wave walks its own pages as
// above; at the end the waves combine their (maximum, sum, accumulator) rows in LDS (log-sum-exp),
// so one partial per group reaches memory for the merge. WG = 1: one wave per workgroup, one
// partial per split.
template <int BITS, bool PS16, int NT, bool MQ, int F, int WG>
__global__ __launch_bounds__(64 * WG, KVQ_DECODE_MIN_WAVES) void decode_mfma_kernel(const DecodeArgs a) {
  static_assert(F == 1 || F == 2, "pack factor");
  static_assert(NT == 2 || (NT == 4 && !MQ), "a step is one or two PV chunks of two tiles");
  static_assert(!MQ || F == 1, "several queries fill the 16 columns themselves");
  static_assert(WG == 1 || (!MQ && F == 2 && WG == 4), "split groups: one query per sequence");
  constexpr int W = 16 / F;   // columns per tile slot
  constexpr int KG = NT / F;  // packed score groups per step
  constexpr int P = 4 * KG;   // scores per lane per step
  constexpr int kQRows = MQ ? 16 : 8;  // query vectors staged per wave
  // Per wave of the workgroup: the query rows (prologue only) and the accumulator rows (epilogue
  // only) share one block; the scale/zero staging of the walk has its own.
  constexpr int kRedRows = F > 1 ? 16 : 1;
  constexpr int kQsRedBytes = std::max(kQRows * kHeadDim * 4, kRedRows * kHeadDim * 4);
  __shared__ __attribute__((aligned(16))) uint8_t qsred_all[WG][kQsRedBytes];
  __shared__ float4 szs_all[WG][2][NT][16];  // scale/zero of a step's tiles, two steps: [buf][tile][K 0..31 | V 32..63]
  __shared__ float2 cml[WG][8];  // split groups: each wave's (maximum, sum) per head

  const int lane = threadIdx.x & 63;
  // the wave index is uniform across the wave: kept in a scalar register
  const int wv = (WG == 1) ? 0 : __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  float (&qs)[kQRows][kHeadDim] = *reinterpret_cast<float (*)[kQRows][kHeadDim]>(&qsred_all[wv][0]);
  float4 (&szs)[2][NT][16] = szs_all[wv];
  // accumulator rows, for the sum over tile slots (and, in split groups, the rows to combine)
  float4 (&red)[kRedRows][kHeadDim / 4] = *reinterpret_cast<float4 (*)[kRedRows][kHeadDim / 4]>(&qsred_all[wv][0]);
  const int G = lane >> 4;
  const int n = lane & 15;
  const int u_l = n / W;  // tile slot of this lane's column
  const int h_l = n % W;  // query column of this lane
  // One query per sequence: a one-dimensional grid numbered (sequence, KV head) item fastest, so
  // that with a multiple of 8 items every split of an item lands on the same XCD (workgroups go to
  // the eight XCDs in turn) - and the merge of its partials, numbered alike, reads them from that
  // XCD's L2.
  // (scalar divisions by invariant divisors, see FastDiv)
  const uint32_t gq = MQ ? 0u : fast_div(blockIdx.x, a.div_items);          // split group (WG = 4) or split
  const uint32_t item = MQ ? 0u : blockIdx.x - gq * a.div_items.d;
  const int group = static_cast<int>(gq);
  const int split = MQ ? static_cast<int>(blockIdx.x) : group * WG + wv;
  const uint32_t hsel = MQ ? blockIdx.y : item;  // MQ: (column tile, KV head); else (sequence, KV head)
  const uint32_t hq = fast_div(hsel, a.div_kvh);
  const int kvh = static_cast<int>(hsel - hq * a.div_kvh.d);
  const int c0 = MQ ? 16 * static_cast<int>(hq) : 0;  // first column of the tile
  const int b = MQ ? static_cast<int>(blockIdx.z) : static_cast<int>(hq);
  const int g = a.group;
  const int ps = PS16 ? 16 : a.page_size;
  const int tiles_per_page = PS16 ? 1 : ps / 16;
  const int len = min(max(ro_load(a.context_lens, b), 0), a.max_context_len);
  const int n_pages = (len + ps - 1) / ps;
  // The pages past num_splits * pages_per_split (see plan_splits) go to the last split, or, in the
  // fused step, to the first: the split that writes the new token (the last page's) is then not
  // also the longest one.
  const int extra = max(0, n_pages - a.num_splits * a.pages_per_split);
  const bool extra_first = a.fused && extra > 0 && a.num_splits > 1;
  const int p_begin = split * a.pages_per_split + ((extra_first && split > 0) ? extra : 0);
  const int p_end = (split >= a.num_splits) ? p_begin  // a group's waves past the last split: no pages
                    : extra_first ? min(n_pages, (split + 1) * a.pages_per_split + extra)
                                  : ((split == a.num_splits - 1) ? n_pages : min(n_pages, p_begin + a.pages_per_split));
  // queries of this sequence (MQ; never more than its tokens) and the tile's valid columns
  const int qlen = MQ ? min(min(max(ro_load(a.q_lens, b), 0), a.q_len_max), len) : 1;
  const int ncols = MQ ? min(16, qlen * g - c0) : g;
  const int ncols_rows = MQ ? min(16, a.q_len_max * g - c0) : g;  // columns that are rows of out
  // row (in head vectors) of q / out for local column c
  auto col_row = [&](int c) -> int64_t {
    if constexpr (MQ) {
      const int cc = c0 + c;
      return (static_cast<int64_t>(b) * a.q_len_max + cc / g) * a.num_q_heads + static_cast<int64_t>(kvh) * g + cc % g;
    } else {
      return static_cast<int64_t>(b) * a.num_q_heads + static_cast<int64_t>(kvh) * g + c;
    }
  };
  // causal length of this lane's column (MQ), else the sequence length
  const int len_col = MQ ? ((n < ncols) ? len - qlen + (c0 + n) / g + 1 : 0) : len;

  if (a.fused && len > 0) {
    // this split owns the last page: write the new token first
    const int pos = len - 1;
    const int last_page = pos / ps;
    if (last_page >= p_begin && last_page < p_end) {
      const int32_t page = ro_load(a.block_table, static_cast<int64_t>(b) * a.max_pages_per_seq + last_page);
      if (page >= 0 && page < a.num_pages) append_new_token<BITS>(a, b, kvh, pos, page, lane);
    }
  }

  const LaneFwht lf = lane_fwht(a.rot, n);
  // ---- split groups: the waves' rows combined in LDS - each wave's (max, sum) per head and its
  // accumulator rows (zero term included) in its own accumulator block - then a log-sum-exp over
  // the group's splits: wave wv takes heads wv, wv + 4, row group G the row of wave G, combined
  // across the four row groups; the group's partial goes to the workspace for the merge.
  constexpr int S = (F == 1) ? 4 : W / 4;  // output heads per lane at the end of the walk
  auto group_finish = [&](const float (&ov)[S][8], const float (&lrow)[S], const float (&zrow)[S],
                          const float (&mrow)[S]) {
    float* const mine = reinterpret_cast<float*>(&red[0][0]);  // rows [head][128] (after the slot sums)
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int c = G + 4 * s;
      float4* dst = reinterpret_cast<float4*>(mine + c * kHeadDim + 8 * n);
      const float zr = zrow[s];
      dst[0] = make_float4(ov[s][0] + zr, ov[s][1] + zr, ov[s][2] + zr, ov[s][3] + zr);
      dst[1] = make_float4(ov[s][4] + zr, ov[s][5] + zr, ov[s][6] + zr, ov[s][7] + zr);
      if (n == 0) cml[wv][c] = make_float2(mrow[s], lrow[s]);
    }
    __syncthreads();
    const int64_t pairs = static_cast<int64_t>(a.batch) * a.num_q_heads;
    for (int c = wv; c < g; c += WG) {
      const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(&qsred_all[G][0]) +
                                                          c * kHeadDim + 8 * n);
      const float4 ra = src[0], rb = src[1];
      float o[8] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
      float mm = cml[G][c].x, ll = cml[G][c].y;
      lse_combine(mm, ll, o, 16);
      lse_combine(mm, ll, o, 32);
      if (G == 0) {
        const int64_t row = group * pairs + col_row(c);
        float4* dst = reinterpret_cast<float4*>(a.ws_acc + row * kHeadDim + 8 * n);
        dst[0] = make_float4(o[0], o[1], o[2], o[3]);
        dst[1] = make_float4(o[4], o[5], o[6], o[7]);
        if (n == 0) reinterpret_cast<float2*>(a.ws_ml)[row] = make_float2(mm, ll);
      }
    }
  };

  if (p_begin >= p_end || ncols <= 0) {
    if constexpr (WG > 1) {  // no pages for this wave: an empty row (maximum -inf) in its group
      float ov[S][8], lrow[S], zrow[S], mrow[S];
#pragma unroll
      for (int s = 0; s < S; ++s) {
#pragma unroll
        for (int m = 0; m < 8; ++m) ov[s][m] = 0.f;
        lrow[s] = 0.f;
        zrow[s] = 0.f;
        mrow[s] = kNegInf;
      }
      group_finish(ov, lrow, zrow, mrow);
      return;
    }
    if (a.num_splits == 1) {  // empty sequence (or no valid query in the tile): zero output
      for (int c = G; c < ncols_rows; c += 4) {
        float4* o = reinterpret_cast<float4*>(a.out + col_row(c) * kHeadDim + n * 8);
        o[0] = make_float4(0.f, 0.f, 0.f, 0.f);
        o[1] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    return;
  }

  // ---- walk the split's tiles, NT per step, the next NT to 2 NT tiles loading meanwhile
  const int tile_begin = p_begin * tiles_per_page;
  const int tile_end = min(p_end * tiles_per_page, (len + 15) / 16);
  // tiles before full_end are valid for every column (MQ: the tile's first query is the most limited)
  const int full_end = min(tile_end, (MQ ? len - qlen + c0 / g + 1 : len) / 16);
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.max_pages_per_seq;

  v4f acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;   // running maximum of head h_l (log2 units), equal in every lane of the head
  float l_part = 0.f;      // this lane's share of sum p (head h_l)
  float z_part = 0.f;      // this lane's share of sum p (z - B delta) (head h_l)
  const float lazy = kLazyRescale;

  // Page of a tile (scalar load). Tiles past the split's end issue the same loads as the others
  // (zero-size resources: no memory traffic, masked out through pg = -1), so that the wait for a
  // buffer never has to drain the loads of the next one.
  LaneOffsets lo;
  lo.k = (BITS == 4) ? (n * (kHeadDim / 2) + 16 * G) : (n * (kHeadDim / 4) + 8 * G);
  lo.v = (BITS == 4) ? (G * 4 * (kHeadDim / 2) + 16 * n) : (G * 4 * (kHeadDim / 4) + 8 * n);
  lo.sz = (lane < 32) ? a.k_sz + lane : a.v_sz + (lane - 32);
  const int last_tile = tile_end - 1;
  const int64_t page_rows = static_cast<int64_t>(a.num_kv_heads) * ps;  // token rows per page (all heads)
  const int64_t head_rows = static_cast<int64_t>(kvh) * ps;
  auto fetch = [&](int t, TileCodes (&x)[NT], int64_t (&pg)[NT]) {
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int tt = min(t + u, last_tile);
      const int32_t p = ro_load(bt, PS16 ? tt : tt / tiles_per_page);
      const bool ok = (p >= 0 && p < a.num_pages);
      const bool live = ok && t + u <= last_tile;
      pg[u] = live ? p : -1;
      const int64_t row0 = (ok ? p : 0) * page_rows + head_rows + (PS16 ? 0 : 16 * (tt % tiles_per_page));
      x[u] = load_tile<BITS>(a, row0, lo, live);
    }
  };

  // The query rows (row group G: heads G and G + 4) and then the first two steps' tiles start
  // loading before the query is prepared; every lane loads (heads past the group re-read the last one).
  constexpr int kQPerGroup = kQRows / 4;
  uint4 qw[kQPerGroup];
#pragma unroll
  for (int r = 0; r < kQPerGroup; ++r) {
    const int c = min(4 * r + G, ncols - 1);
    qw[r] = *reinterpret_cast<const uint4*>(a.q + col_row(c) * kHeadDim + n * 8);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the query loads ahead of the tile loads (in-order vmcnt)
  TileCodes x0[NT], x1[NT];
  int64_t pg0[NT], pg1[NT];
  fetch(tile_begin, x0, pg0);
  fetch(tile_begin + NT, x1, pg1);

  // ---- query: rotate (R q), scale by softmax_scale * log2(e), stage in LDS in natural order
#pragma unroll
  for (int r = 0; r < kQPerGroup; ++r) {
    const int c = 4 * r + G;
    if (4 * r >= ncols) break;
    float x[8];
    bf16x8_to_f32(qw[r], x);
    int pos = n;
    if (!a.q_prerotated) {
      fwht_row16_planned(x, a.rot, lf);
      pos = lf.pos;
    }
    if (c < ncols) {
#pragma unroll
      for (int k = 0; k < 8; ++k) qs[c][8 * pos + k] = x[k] * a.qk_scale_log2;
    }
  }
  wave_lds_sync();

  // ---- query as 21-bit fixed point x = rint(q' 2^E), |x| <= 2^20, in three int8 limbs: with the
  // offset x + 0x808080 (in [0x708080, 0x908080]) its three bytes b_i are x's base-256 digits
  // shifted by 128, so limb l_i = b_i - 128 is byte b_i with the top bit flipped, and
  // x = (l2 * 256 + l1) * 256 + l0. Column n takes head h_l: the F tile slots share the query.
  // qv[(j * 4 + r) * 4 + k] is the channel that MFMA j, register slot r, byte k of lane group G
  // multiplies: the byte the K-code operand puts there (INT4: 32 G + 16 j + 8 (r >> 1) + 2 k + (r & 1),
  // INT2: 32 G + 16 j + 4 k + r). Those are 16-byte runs of the staged row: eight 16-byte LDS reads.
  // Columns past the group's heads take the last head's query (finite scores that are never stored).
  float qv[32];
  {
    const float* qrow = &qs[min(h_l, ncols - 1)][0];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (BITS == 4) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // channels 32 G + 16 j + 8 h + 2 k + (r & 1), r = 2 h + (r & 1)
          const float4 lo = *reinterpret_cast<const float4*>(qrow + 32 * G + 16 * j + 8 * h);
          const float4 hi = *reinterpret_cast<const float4*>(qrow + 32 * G + 16 * j + 8 * h + 4);
          const float c[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
          for (int rr = 0; rr < 2; ++rr)
#pragma unroll
            for (int k = 0; k < 4; ++k) qv[(j * 4 + 2 * h + rr) * 4 + k] = c[2 * k + rr];
        }
      } else {  // channels 32 G + 16 j + 4 k + r
        float c[16];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float4 x = *reinterpret_cast<const float4*>(qrow + 32 * G + 16 * j + 4 * e);
          c[4 * e] = x.x;
          c[4 * e + 1] = x.y;
          c[4 * e + 2] = x.z;
          c[4 * e + 3] = x.w;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int k = 0; k < 4; ++k) qv[(j * 4 + r) * 4 + k] = c[4 * k + r];
      }
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(qv[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  int e2 = 0;
  (void)frexpf(amax, &e2);
  const int E = (amax > 0.f) ? 20 - e2 : 0;
  const float two_e = ldexpf(1.0f, E);  // exact: |q' 2^E| < 2^20
  // RN(v + 1.5 * 2^23) holds rint(v) in its low mantissa bits (|v| < 2^22, ties to even)
  constexpr float kRoundMagic = 12582912.0f;
  constexpr uint32_t kOffsetBits = 0x4B400000u - 0x808080u;  // bits(magic + x) - this = x + 0x808080
  v4i L0[2], L1[2], L2[2];
  uint32_t sxb = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t xb[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        xb[k] = __float_as_uint(__builtin_fmaf(qv[(j * 4 + r) * 4 + k], two_e, kRoundMagic)) - kOffsetBits;
        sxb += xb[k];
      }
      // byte i of the four values -> one dword per limb (byte k = value k), top bits flipped
      const uint32_t lo01 = __builtin_amdgcn_perm(xb[1], xb[0], 0x05010400u);  // b0(x0) b0(x1) b1(x0) b1(x1)
      const uint32_t lo23 = __builtin_amdgcn_perm(xb[3], xb[2], 0x05010400u);
      const uint32_t hi01 = __builtin_amdgcn_perm(xb[1], xb[0], 0x07030602u);  // b2(x0) b2(x1) b3 b3
      const uint32_t hi23 = __builtin_amdgcn_perm(xb[3], xb[2], 0x07030602u);
      L0[j][r] = static_cast<int>(__builtin_amdgcn_perm(lo23, lo01, 0x05040100u) ^ 0x80808080u);
      L1[j][r] = static_cast<int>(__builtin_amdgcn_perm(lo23, lo01, 0x07060302u) ^ 0x80808080u);
      L2[j][r] = static_cast<int>(__builtin_amdgcn_perm(hi23, hi01, 0x05040100u) ^ 0x80808080u);
    }
  }
  // sum of x over this lane's 32 values, then over the four row groups (128 channels)
  int sx = static_cast<int>(sxb - 32u * 0x808080u);
  sx += __shfl_xor(sx, 16, 64);
  sx += __shfl_xor(sx, 32, 64);
  const float inv_scale = ldexpf(1.0f, -E);     // q' = x 2^-E
  const float sum_q = static_cast<float>(sx);   // sum of x over the 128 channels

  const uint32_t c80 = vgpr_const(0x80808080u);
  // One step over NT tiles. full (all 16 NT tokens valid, all pages valid) drops every mask.
  auto step_impl = [&](auto full_tag, const TileCodes (&c)[NT], const int64_t (&pg)[NT], int tile,
                       const TileCodes (&next)[NT], int buf) {
    constexpr bool full = decltype(full_tag)::value;

    // QK^T, two tiles at a time: one exact int32 dot product per query limb (six independent
    // MFMA chains of depth two), then x = ((s2 * 256) + s1) * 256 + s0 - Horner's rule on the
    // finished products, every partial sum below 2^31. Tile t's scores then go to packed group
    // t / F, in the columns of slot t % F.
    v4i sc[KG];
#pragma unroll
    for (int t0 = 0; t0 < NT; t0 += 2) {
      v4i s0[2], s1[2], s2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const v4i k0 = k_operand<BITS>(c[t0 + u].k, 0);
        s0[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(k0, L0[0], v4i{0, 0, 0, 0}, 0, 0, 0);
        s1[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(k0, L1[0], v4i{0, 0, 0, 0}, 0, 0, 0);
        s2[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(k0, L2[0], v4i{0, 0, 0, 0}, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const v4i k1 = k_operand<BITS>(c[t0 + u].k, 1);
        s0[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(k1, L0[1], s0[u], 0, 0, 0);
        s1[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(k1, L1[1], s1[u], 0, 0, 0);
        s2[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(k1, L2[1], s2[u], 0, 0, 0);
      }
      if constexpr (F == 1) {
#pragma unroll
        for (int u = 0; u < 2; ++u) sc[t0 + u] = (((s2[u] << 8) + s1[u]) << 8) + s0[u];
      } else {  // F = 2: the lane's own tile (slot u_l) picked limb by limb, then one combination
        const bool second = u_l == 1;
        v4i a0, a1, a2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a0[i] = second ? s0[1][i] : s0[0][i];
          a1[i] = second ? s1[1][i] : s1[0][i];
          a2[i] = second ? s2[1][i] : s2[0][i];
        }
        sc[t0 / 2] = (((a2 << 8) + a1) << 8) + a0;
      }
    }

    // raw scores t = delta (q~.c) + z sum(q~), in units of 2^E * log2; value 4k + i is token
    // 4G + i of tile k F + u_l
    float sr[P], vd[P], vzz[P];
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      const float4* zb = szs[buf][k * F + (F > 1 ? u_l : 0)];
      const float4 k01 = zb[2 * G], k23 = zb[2 * G + 1];
      const float4 v01 = zb[8 + 2 * G], v23 = zb[8 + 2 * G + 1];
      const float kd[4] = {k01.x, k01.z, k23.x, k23.z};
      const float kz[4] = {k01.y, k01.w, k23.y, k23.w};
      const float vdd[4] = {v01.x, v01.z, v23.x, v23.z};
      const float vz[4] = {v01.y, v01.w, v23.y, v23.w};
      int64_t pgl = pg[k * F];
#pragma unroll
      for (int u = 1; u < F; ++u) pgl = (u_l == u) ? pg[k * F + u] : pgl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float t = __builtin_fmaf(kd[i], static_cast<float>(sc[k][i]), kz[i] * sum_q);
        if constexpr (!full) {
          const bool ok = pgl >= 0 && (tile + k * F + u_l) * 16 + 4 * G + i < len_col;
          t = ok ? t : kNegInf;
        }
        sr[4 * k + i] = t;
        vd[4 * k + i] = vdd[i];
        vzz[4 * k + i] = __builtin_fmaf(-VBias<BITS>::value, vdd[i], vz[i]);
      }
    }
    // step maximum of each head: over the lane's values, the four row groups and the F slots
    float mt = sr[0];
#pragma unroll
    for (int i = 1; i < P; ++i) mt = fmaxf(mt, sr[i]);
    mt = max_over_rows_nc(mt);
    if constexpr (F == 2) mt = max_nc(mt, row_ror<8>(mt));
    mt *= inv_scale;  // log2 units
    if (__any(mt > m_run + lazy)) {
      const float m_new = (mt > m_run + lazy) ? mt : m_run;
      const float alpha = (m_run == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_part *= alpha;
      z_part *= alpha;
      // accumulator row 4G + i is (slot, head (4G + i) % W); that head's factor lives in lane
      // (4G + i) % W
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, (4 * G + i) & (W - 1), 64);
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[m][i] *= ai;
      }
    }
    const float m_ref = (m_run == kNegInf) ? 0.f : m_run;  // only a step with no valid token leaves -inf
    float w[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
      // p = 2^(t 2^-E - m); invalid tokens have t = -inf and so p = 0
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(inv_scale, sr[i], -m_ref));
      l_part += p;
      if constexpr (full) {
        z_part = __builtin_fmaf(p, vzz[i], z_part);
        w[i] = p * vd[i];
      } else {  // rows past the end may hold anything, even NaN: select, do not multiply
        z_part = __builtin_fmaf(p, (sr[i] == kNegInf) ? 0.f : vzz[i], z_part);
        w[i] = (sr[i] == kNegInf) ? 0.f : p * vd[i];
      }
    }
    // PV over chunks of two tiles (32 tokens). A row r = QK column r; with F > 1 a row carries
    // only the tokens of its own slot's tile, zero for the chunk's other tile.
#pragma unroll
    for (int ch = 0; ch < NT / 2; ++ch) {
      const int t0 = 2 * ch, t1 = t0 + 1;
      v8bf p_hi, p_lo;
      if constexpr (F == 1) {
        uint32_t h01a, h23a, l01a, l23a, h01b, h23b, l01b, l23b;
        split_bf16({w[4 * t0], w[4 * t0 + 1], w[4 * t0 + 2], w[4 * t0 + 3]}, h01a, h23a, l01a, l23a);
        split_bf16({w[4 * t1], w[4 * t1 + 1], w[4 * t1 + 2], w[4 * t1 + 3]}, h01b, h23b, l01b, l23b);
        p_hi = as_bf(v4u{h01a, h23a, h01b, h23b});
        p_lo = as_bf(v4u{l01a, l23a, l01b, l23b});
      } else {
        const int k = t0 / F;
        uint32_t h01, h23, l01, l23;
        split_bf16({w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]}, h01, h23, l01, l23);
        const uint32_t m0 = (u_l == t0 % F) ? ~0u : 0u;
        const uint32_t m1 = (u_l == t1 % F) ? ~0u : 0u;
        p_hi = as_bf(v4u{h01 & m0, h23 & m0, h01 & m1, h23 & m1});
        p_lo = as_bf(v4u{l01 & m0, l23 & m0, l01 & m1, l23 & m1});
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint32_t na = v_bf16_low_bytes<BITS>(c[t0].v, m, c80);
        const uint32_t nb = v_bf16_low_bytes<BITS>(c[t1].v, m, c80);
        const v8bf vb = as_bf(v4u{bias_bf16_lo<BITS>(na), bias_bf16_hi<BITS>(na), bias_bf16_lo<BITS>(nb),
                                  bias_bf16_hi<BITS>(nb)});
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p_hi, vb, acc[m], 0, 0, 0);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p_lo, vb, acc[m], 0, 0, 0);
      }
    }
    // stage the next step's scale/zero blocks in the other buffer
#pragma unroll
    for (int u = 0; u < NT; ++u) reinterpret_cast<float*>(szs[buf ^ 1][u])[lane] = next[u].sz;
    wave_lds_sync();
  };
  auto step = [&](const TileCodes (&c)[NT], const int64_t (&pg)[NT], int tile, const TileCodes (&next)[NT],
                  int buf) {
    bool pages_ok = true;
#pragma unroll
    for (int u = 0; u < NT; ++u) pages_ok = pages_ok && pg[u] >= 0;
    if ((tile + NT - 1 < full_end) && pages_ok) {
      step_impl(std::true_type{}, c, pg, tile, next, buf);
    } else {
      step_impl(std::false_type{}, c, pg, tile, next, buf);
    }
  };

#pragma unroll
  for (int u = 0; u < NT; ++u) reinterpret_cast<float*>(szs[0][u])[lane] = x0[u].sz;
  wave_lds_sync();
  // Triple-buffered walk: while the tiles of one buffer are processed, the next two steps'
  // tiles are already loading. Step k reads scale/zero buffer k & 1; the six-step cycle keeps
  // the parity aligned.
  TileCodes x2[NT];
  int64_t pg2[NT];
  for (int tile = tile_begin;; tile += 6 * NT) {
    fetch(tile + 2 * NT, x2, pg2);
    step(x0, pg0, tile, x1, 0);
    if (tile + NT >= tile_end) break;
    fetch(tile + 3 * NT, x0, pg0);
    step(x1, pg1, tile + NT, x2, 1);
    if (tile + 2 * NT >= tile_end) break;
    fetch(tile + 4 * NT, x1, pg1);
    step(x2, pg2, tile + 2 * NT, x0, 0);
    if (tile + 3 * NT >= tile_end) break;
    fetch(tile + 5 * NT, x2, pg2);
    step(x0, pg0, tile + 3 * NT, x1, 1);
    if (tile + 4 * NT >= tile_end) break;
    fetch(tile + 6 * NT, x0, pg0);
    step(x1, pg1, tile + 4 * NT, x2, 0);
    if (tile + 5 * NT >= tile_end) break;
    fetch(tile + 7 * NT, x1, pg1);
    step(x2, pg2, tile + 5 * NT, x0, 1);
    if (tile + 6 * NT >= tile_end) break;
  }

  // ---- finish: each head's totals over the row groups and the tile slots (then equal in every
  // lane of the head; lane h < W holds head h)
  l_part += __shfl_xor(l_part, 16, 64);
  l_part += __shfl_xor(l_part, 32, 64);
  z_part += __shfl_xor(z_part, 16, 64);
  z_part += __shfl_xor(z_part, 32, 64);
  if constexpr (F == 2) {
    l_part += row_ror<8>(l_part);
    z_part += row_ror<8>(z_part);
  }
  // S output heads per lane: F = 1: heads 4G + s, straight from the accumulator rows; F > 1:
  // heads G + 4s, the sum of their F slot rows, exchanged through LDS.
  float ov[S][8];
  int hh[S];
  if constexpr (F == 1) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      hh[s] = 4 * G + s;
#pragma unroll
      for (int m = 0; m < 8; ++m) ov[s][m] = acc[m][s];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      red[4 * G + i][2 * n] = make_float4(acc[0][i], acc[1][i], acc[2][i], acc[3][i]);
      red[4 * G + i][2 * n + 1] = make_float4(acc[4][i], acc[5][i], acc[6][i], acc[7][i]);
    }
    wave_lds_sync();
#pragma unroll
    for (int s = 0; s < S; ++s) {
      hh[s] = G + 4 * s;
#pragma unroll
      for (int m = 0; m < 8; ++m) ov[s][m] = 0.f;
#pragma unroll
      for (int u = 0; u < F; ++u) {
        const float4 ra = red[u * W + hh[s]][2 * n], rb = red[u * W + hh[s]][2 * n + 1];
        ov[s][0] += ra.x; ov[s][1] += ra.y; ov[s][2] += ra.z; ov[s][3] += ra.w;
        ov[s][4] += rb.x; ov[s][5] += rb.y; ov[s][6] += rb.z; ov[s][7] += rb.w;
      }
    }
  }
  float lrow[S], zrow[S], mrow[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    lrow[s] = __shfl(l_part, hh[s], 64);
    zrow[s] = __shfl(z_part, hh[s], 64);
    mrow[s] = __shfl(m_run, hh[s], 64);
  }

  if (a.num_splits == 1) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int c = hh[s];
      float o[8];
      const float inv_l = (lrow[s] > 0.f) ? 1.0f / lrow[s] : 0.f;
#pragma unroll
      for (int m = 0; m < 8; ++m) o[m] = (c < ncols) ? (ov[s][m] + zrow[s]) * inv_l : 0.f;
      fwht_row16_planned(o, a.rot, lf);  // R^T = R: back to the original basis
      if (c < ncols_rows) {
        float4* dst = reinterpret_cast<float4*>(a.out + col_row(c) * kHeadDim + 8 * lf.pos);
        dst[0] = make_float4(o[0], o[1], o[2], o[3]);
        dst[1] = make_float4(o[4], o[5], o[6], o[7]);
      }
    }
    return;
  }

  if constexpr (WG > 1) {
    group_finish(ov, lrow, zrow, mrow);
    return;
  }

  // Split: publish this split's partial (un-normalised accumulator with its zero term, running
  // maximum and sum) for the merge kernel.
  const int64_t pairs = static_cast<int64_t>(a.batch) * (MQ ? a.q_len_max : 1) * a.num_q_heads;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int c = hh[s];
    if (c < ncols) {
      const int64_t row = split * pairs + col_row(c);
      float4* dst = reinterpret_cast<float4*>(a.ws_acc + row * kHeadDim + 8 * n);
      const float zr = zrow[s];
      dst[0] = make_float4(ov[s][0] + zr, ov[s][1] + zr, ov[s][2] + zr, ov[s][3] + zr);
      dst[1] = make_float4(ov[s][4] + zr, ov[s][5] + zr, ov[s][6] + zr, ov[s][7] + zr);
      if (n == 0) reinterpret_cast<float2*>(a.ws_ml)[row] = make_float2(mrow[s], lrow[s]);
    }
  }
}

// Log-sum-exp merge of the split partials of one (sequence, query head) per wave. Row group G
// takes splits G, G + 4, G + 8, ...; lane n holds channels 8n..8n+7. NB splits per row group (1, 2,
// 4 or 8: as many as the call's partial rows need, at most eight) are loaded with independent loads
// before any is combined, so up to 4 NB splits cost one memory round trip.
// The four groups' running (max, sum, vector) are then combined across rows, rotated back and
// stored by row group 0.
template <int NB>
__global__ __launch_bounds__(64) void decode_merge_splits_kernel(const DecodeArgs a) {
  const int lane = threadIdx.x;
  const int G = lane >> 4;
  const int n = lane & 15;
  // one query per sequence: numbered like the decode's items (item fastest, then the group's head)
  uint32_t pair = blockIdx.x;  // (b * q_len_max + j) * num_q_heads + h  (decode: q_len_max = 1)
  uint32_t bb = 0;             // the sequence (decode)
  if (!a.q_lens) {
    const uint32_t j = fast_div(blockIdx.x, a.div_items);
    const uint32_t item = blockIdx.x - j * a.div_items.d;
    bb = fast_div(item, a.div_kvh);
    const uint32_t kk = item - bb * a.div_kvh.d;
    pair = bb * static_cast<uint32_t>(a.num_q_heads) + kk * static_cast<uint32_t>(a.group) + j;
  }
  const int q_len_max = a.q_lens ? a.q_len_max : 1;
  const int64_t pairs = static_cast<int64_t>(a.batch) * q_len_max * a.num_q_heads;
  const float2* ml_all = reinterpret_cast<const float2*>(a.ws_ml);
  // One batch of 4 NB splits: row group G loads splits s0 + G + 4j (past s_last: s_last again).
  struct Batch {
    float2 ml[NB];
    float4 xa[NB], xb[NB];
  };
  auto load_batch = [&](int s0, int s_last, Batch& bt) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int sp = min(s0 + G + 4 * j, s_last);
      const int64_t row = sp * pairs + pair;
      bt.ml[j] = ml_all[row];
      const float4* src = reinterpret_cast<const float4*>(a.ws_acc + row * kHeadDim + 8 * n);
      bt.xa[j] = src[0];
      bt.xb[j] = src[1];
    }
  };
  // The first batch is loaded before the sequence length (and so the number of splits it uses)
  // is known: the workspace holds num_splits rows, and the rows this call did not write (stale,
  // possibly NaN) are dropped by selection below, never multiplied by a zero weight.
  Batch bt;
  load_batch(0, a.num_splits - 1, bt);
  __builtin_amdgcn_sched_barrier(0);

  const int b = a.q_lens ? static_cast<int>(pair / static_cast<uint32_t>(q_len_max * a.num_q_heads))
                         : static_cast<int>(bb);
  const int len = min(max(ro_load(a.context_lens, b), 0), a.max_context_len);
  const int n_pages = (len + a.page_size - 1) / a.page_size;
  int nu = a.all_splits ? a.num_splits : min(a.num_splits, (n_pages + a.pages_per_split - 1) / a.pages_per_split);
  if (a.q_lens) {  // a query row past the sequence's queries has no partials: zero output
    const int j = static_cast<int>((pair / static_cast<uint32_t>(a.num_q_heads)) % static_cast<uint32_t>(q_len_max));
    if (j >= min(min(max(ro_load(a.q_lens, b), 0), a.q_len_max), len)) nu = 0;
  }
  const LaneFwht lf = lane_fwht(a.rot, n);
  float mo = kNegInf, lsum = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0;;) {
    bool use[NB];
    float mc = mo;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      // a split with no token for this row (several queries: past a query's causal limit) has
      // maximum -inf and weighs nothing (even when every split so far is such a split)
      use[j] = s0 + G + 4 * j < nu && bt.ml[j].x != kNegInf;
      mc = use[j] ? fmaxf(mc, bt.ml[j].x) : mc;
    }
    const float r = (mo == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(mo - mc);
    lsum *= r;
#pragma unroll
    for (int m = 0; m < 8; ++m) o[m] *= r;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (!use[j]) continue;
      const float f = __builtin_amdgcn_exp2f(bt.ml[j].x - mc);
      lsum = __builtin_fmaf(bt.ml[j].y, f, lsum);
      o[0] = __builtin_fmaf(bt.xa[j].x, f, o[0]); o[1] = __builtin_fmaf(bt.xa[j].y, f, o[1]);
      o[2] = __builtin_fmaf(bt.xa[j].z, f, o[2]); o[3] = __builtin_fmaf(bt.xa[j].w, f, o[3]);
      o[4] = __builtin_fmaf(bt.xb[j].x, f, o[4]); o[5] = __builtin_fmaf(bt.xb[j].y, f, o[5]);
      o[6] = __builtin_fmaf(bt.xb[j].z, f, o[6]); o[7] = __builtin_fmaf(bt.xb[j].w, f, o[7]);
    }
    mo = mc;
    s0 += 4 * NB;
    if (s0 >= nu) break;
    load_batch(s0, nu - 1, bt);
  }
  lse_combine(mo, lsum, o, 16);
  lse_combine(mo, lsum, o, 32);
  const float inv_l = (nu > 0 && lsum > 0.f) ? 1.0f / lsum : 0.f;  // an empty sequence yields zeros
#pragma unroll
  for (int m = 0; m < 8; ++m) o[m] *= inv_l;
  fwht_row16_planned(o, a.rot, lf);
  if (G == 0) {
    float4* dst = reinterpret_cast<float4*>(a.out + pair * kHeadDim + 8 * lf.pos);
    dst[0] = make_float4(o[0], o[1], o[2], o[3]);
    dst[1] = make_float4(o[4], o[5], o[6], o[7]);
  }
}

constexpr int kMinSplitsGrouped = 16;

template <bool MQ, int F, int NT, int WG, int NT2 = NT>
hipError_t launch_kernel(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
  const bool ps16 = a.page_size == 16;
  const dim3 block(64 * WG);
  if (a.bits == 4) {
    if (ps16) hipLaunchKernelGGL((decode_mfma_kernel<4, true, NT, MQ, F, WG>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_mfma_kernel<4, false, NT, MQ, F, WG>), grid, block, 0, stream, a);
  } else {
    if (ps16) hipLaunchKernelGGL((decode_mfma_kernel<2, true, NT2, MQ, F, WG>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_mfma_kernel<2, false, NT2, MQ, F, WG>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

// Column tiles of 16 (query, head) pairs per KV head for several queries per sequence.
int32_t mq_column_tiles(int32_t q_len_max, int32_t group) { return (q_len_max * group + 15) / 16; }

static void set_index_divisors(DecodeArgs& a) {
  a.div_items = make_fast_div(static_cast<uint32_t>(a.batch) * static_cast<uint32_t>(a.num_kv_heads));
  a.div_kvh = make_fast_div(static_cast<uint32_t>(a.num_kv_heads));
  a.group = a.num_q_heads / a.num_kv_heads;
}

hipError_t launch_decode_mfma(const DecodeArgs& args, hipStream_t stream) {
  DecodeArgs a = args;
  set_index_divisors(a);
  const unsigned tiles = a.q_lens ? static_cast<unsigned>(mq_column_tiles(a.q_len_max, a.num_q_heads / a.num_kv_heads)) : 1u;
  const dim3 grid = a.q_lens ? dim3(static_cast<unsigned>(a.num_splits), static_cast<unsigned>(a.num_kv_heads) * tiles,
                                    static_cast<unsigned>(a.batch))
                             : dim3(static_cast<unsigned>(a.num_splits) * static_cast<unsigned>(a.batch) *
                                    static_cast<unsigned>(a.num_kv_heads));
  if (a.q_lens) {
    const hipError_t e = launch_kernel<true, 1, 2, 1>(a, grid, stream);
    if (e != hipSuccess || a.num_splits == 1) return e;
    return launch_decode_merge(a, stream);
  }
  // One query per sequence (g <= 8, checked by the caller: two tile slots). A split sequence runs in
  // groups of four splits per workgroup, which combine their partials in LDS (while the grid of
  // 256-thread workgroups stays below 2^32 work-items; otherwise one split per workgroup).
  // Only items with many splits are grouped: a group's workgroup keeps its LDS until its slowest wave
  // ends, so with few splits per item (a large or ragged batch, where many of a group's waves would
  // have no pages) one split per workgroup keeps more waves busy.
  const uint64_t items = static_cast<uint64_t>(a.batch) * static_cast<uint64_t>(a.num_kv_heads);
  const uint64_t groups = (static_cast<uint64_t>(a.num_splits) + 3) / 4;
  if (a.num_splits >= kMinSplitsGrouped && groups * items * 256 < (uint64_t{1} << 32)) {
    const hipError_t e = launch_kernel<false, 2, 2, 4, KVQ_DECODE_NT2>(a, dim3(static_cast<unsigned>(groups * items)), stream);
    if (e != hipSuccess) return e;
    // the merge sees one partial per group, every group's row written (an empty one with maximum -inf)
    DecodeArgs m = a;
    m.num_splits = static_cast<int32_t>(groups);
    m.all_splits = 1;
    return launch_decode_merge(m, stream);
  }
  const hipError_t e = launch_kernel<false, 2, 2, 1, KVQ_DECODE_NT2>(a, grid, stream);
  if (e != hipSuccess || a.num_splits == 1) return e;
  return launch_decode_merge(a, stream);
}

hipError_t launch_decode_merge(const DecodeArgs& args, hipStream_t stream) {
  DecodeArgs a = args;
  set_index_divisors(a);
  const int64_t pairs = static_cast<int64_t>(a.batch) * (a.q_lens ? a.q_len_max : 1) * a.num_q_heads;
  const dim3 grid(static_cast<unsigned>(pairs));
  // the loads of one batch cover every partial row when there are at most 4 NB of them
  if (a.num_splits <= 4) hipLaunchKernelGGL(decode_merge_splits_kernel<1>, grid, dim3(64), 0, stream, a);
  else if (a.num_splits <= 8) hipLaunchKernelGGL(decode_merge_splits_kernel<2>, grid, dim3(64), 0, stream, a);
  else if (a.num_splits <= 16) hipLaunchKernelGGL(decode_merge_splits_kernel<4>, grid, dim3(64), 0, stream, a);
  else hipLaunchKernelGGL(decode_merge_splits_kernel<8>, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
