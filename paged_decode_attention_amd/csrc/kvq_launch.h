// Internal launch interface between the C ABI (kvq_api.hip) and the kernels. Arguments have
// already been validated by the caller of these functions.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvq_fastdiv.h"

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kTileTokens = 16;   // tokens handled per page sub-tile; page_size % 16 == 0

// Cross-lane part of the Walsh-Hadamard transform of one 16-lane row (8 channels per lane).
// The lane butterflies use the lane masks 1, 2, 7 and 8 - each a single DPP move (quad_perm,
// quad_perm, row_half_mirror, row_ror:8) - and every lane keeps its value multiplied by a
// known sign, so each stage is one fused multiply-add: x = c_stage * x[lane ^ mask] + x. After
// the last stage lane l holds sign(l) * (Sylvester output block pos(l)). Built on the host by
// make_row_fwht_plan() for a block size b (b <= 8: no lane stages).
struct RowFwhtPlan {
  int32_t hb;            // block size b
  int32_t lane_stages;   // log2(b / 8) for b >= 16, else 0
  float inv_sqrt_hb;     // float32(1 / sqrt(b))
  uint32_t neg[4];       // bit l: stage coefficient of lane l is -1
  uint32_t sign;         // bit l: lane l ends with the negated output
  uint64_t pos;          // 4 bits per lane: output channel block (channels 8 pos .. 8 pos + 7)
};
RowFwhtPlan make_row_fwht_plan(int32_t hb);

struct AppendArgs {
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_stride, v_stride;     // elements between tokens
  int64_t num_tokens;
  int32_t num_kv_heads;
  const int64_t* slots;
  uint8_t* k_codes;
  uint8_t* v_codes;
  float* k_sz;
  float* v_sz;
  int64_t num_slots;              // num_pages * page_size (< 2^32)
  int32_t page_size;
  uint32_t ps_magic;              // slot / page_size = (hi + ((slot - hi) >> 1)) >> ps_shift,
  int32_t ps_shift;               //   hi = umulhi(slot, ps_magic)  (32-bit slots)
  RowFwhtPlan rot;                // the rotation (Hadamard block size and lane plan)
  int32_t bits;
  int32_t token_scale;
  FastDiv div_heads;              // division by num_kv_heads (set by launch_append)
};

struct DecodeArgs {
  const uint16_t* q;
  int32_t q_prerotated;
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const float* k_sz;
  const float* v_sz;
  int32_t page_size;
  const int32_t* block_table;
  int32_t max_pages_per_seq;
  const int32_t* context_lens;
  int32_t max_context_len;        // lengths are clamped to this (the grid was sized for it)
  int32_t num_pages;              // page ids outside [0, num_pages) are skipped
  int32_t batch, num_q_heads, num_kv_heads;
  int32_t hb;
  float inv_sqrt_hb;
  RowFwhtPlan rot;                // lane plan of the rotation (MFMA kernel)
  int32_t bits;
  float qk_scale_log2;            // softmax_scale * log2(e)
  float* out;
  int32_t num_splits;             // splits of the page range per (sequence, kv head)
  int32_t pages_per_split;
  // Partials: [num_splits][batch][num_q_heads][128] and [..][2] (max, sum) in log2 units; with one
  // query per sequence and 16 or more splits only the first ceil(num_splits / 4) rows are used
  // (one per group of four splits, combined in the decode's workgroup).
  float* ws_acc;
  float* ws_ml;
  // Several queries per sequence (chunked prefill, speculative verification): q and out are
  // [batch][q_len_max][num_q_heads][128]; sequence b's q_lens[b] queries are its last q_lens[b]
  // tokens, causal. nullptr for the decode (one query per sequence).
  const int32_t* q_lens;
  int32_t q_len_max;
  // Fused decode step: before attending, the wave that owns a sequence's last page rotates,
  // quantizes and writes that sequence's new token (position context_lens[b] - 1) for its KV head.
  int32_t fused;
  const uint16_t* k_new;          // bf16 [batch][num_kv_heads][128], token stride k_new_stride
  const uint16_t* v_new;
  int64_t k_new_stride, v_new_stride;
  int32_t token_scale;
  uint8_t* k_codes_w;             // the same cache as k_codes ... v_sz, writable
  uint8_t* v_codes_w;
  float* k_sz_w;
  float* v_sz_w;
  // Merge: every split of every row holds a partial (an empty one has maximum -inf), instead of
  // the splits that cover the row's pages.
  int32_t all_splits;
  // Set by the launchers from the fields above (callers leave them): division by batch *
  // num_kv_heads and by num_kv_heads, and the query heads per KV head.
  FastDiv div_items, div_kvh;
  int32_t group;
};

// Per-channel pages (the per-channel reading of OScaR): codes as in the token-wise cache, a
// float32 scale per token, a float32 (scale, zero) per channel per page-head.
constexpr int kPcMaxPage = 128;   // page sizes 32, 64 and 128

struct PcWriteArgs {
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_stride, v_stride;     // elements between tokens
  int32_t num_input_pages;        // input page i = tokens i * page_size .. + page_size - 1
  const int32_t* page_ids;        // destination page of input page i (out of range: skipped)
  int32_t num_kv_heads;
  uint8_t* k_codes;
  uint8_t* v_codes;
  float* k_s;                     // [num_pages][num_kv_heads][page_size]
  float* v_s;
  float* k_cp;                    // [num_pages][num_kv_heads][2][128] = {scale[128], zero[128]}
  float* v_cp;
  int32_t num_pages;
  int32_t page_size;
  RowFwhtPlan rot;
  int32_t bits;
};

struct PcDecodeArgs {
  const uint16_t* q;              // bf16 [batch][num_q_heads][128]
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const float* k_s;
  const float* v_s;
  const float* k_cp;
  const float* v_cp;
  int32_t page_size;
  const int32_t* block_table;     // complete pages of each sequence
  int32_t max_pages_per_seq;
  const int32_t* context_lens;
  int32_t max_context_len;
  int32_t num_pages;
  const uint16_t* tail_k;         // bf16 [batch][page_size][num_kv_heads][128]: the unfinished page
  const uint16_t* tail_v;
  int32_t batch, num_q_heads, num_kv_heads;
  RowFwhtPlan rot;
  int32_t bits;
  float qk_scale_log2;
  int32_t num_splits;             // page splits; split num_splits attends the tail
  int32_t pages_per_split;
  float* ws_acc;                  // [num_splits + 1][batch][num_q_heads][128], original basis
  float* ws_ml;
  float* out;
};
hipError_t launch_pc_write(const PcWriteArgs& a, hipStream_t stream);
hipError_t launch_pc_decode(const PcDecodeArgs& a, hipStream_t stream);

struct DequantArgs {
  const uint8_t* codes;
  const float* sz;
  int32_t tensor;                 // 0 = K layout, 1 = V layout
  int32_t page;
  int32_t num_kv_heads;
  int32_t page_size;
  int32_t hb;
  float inv_sqrt_hb;
  int32_t bits;
  int32_t unrotate;
  float* out;
};

// Baseline: unquantized bf16 paged cache (K token-major, V channel-major per 16 tokens).
struct Bf16WriteArgs {
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_stride, v_stride;     // elements between tokens
  int64_t num_tokens;
  int32_t num_kv_heads;
  const int64_t* slots;
  uint16_t* k_cache;
  uint16_t* v_cache;
  int64_t num_slots;
  int32_t page_size;
};

struct DecodeBf16Args {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  int32_t page_size;
  const int32_t* block_table;
  int32_t max_pages_per_seq;
  const int32_t* context_lens;
  int32_t max_context_len;
  int32_t num_pages;
  int32_t batch, num_q_heads, num_kv_heads;
  float qk_scale_log2;            // softmax_scale * log2(e)
  float* out;
  int32_t num_splits;
  int32_t pages_per_split;
  float* ws_acc;                  // same layout as DecodeArgs
  float* ws_ml;
};

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_bf16_write(const Bf16WriteArgs& a, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeBf16Args& a, hipStream_t stream);
// Log-sum-exp merge of the split partials (ws_acc, ws_ml) into out, then the inverse rotation
// given by a.rot (the identity plan for block size 1); reads a.context_lens, a.max_context_len,
// a.page_size, a.pages_per_split, a.num_splits, a.batch, a.num_q_heads.
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream);
// Column tiles (16 (query, head) pairs each) per KV head when a sequence has q_len_max queries.
int32_t mq_column_tiles(int32_t q_len_max, int32_t group);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_dequant(const DequantArgs& a, hipStream_t stream);

// Split plan used by both the workspace query and the launch. one_query: one query per sequence
// (decode), where a split of a large batch is capped in length; several queries per sequence
// fill the waves with column tiles, and their partials grow with the queries, so no cap there.
struct SplitPlan {
  int32_t num_splits;
  int32_t pages_per_split;
};
SplitPlan plan_splits(int32_t batch, int32_t num_kv_heads, int32_t max_context_len, int32_t page_size,
                      int32_t pages_per_split_request, bool one_query);

}  // namespace kvq
