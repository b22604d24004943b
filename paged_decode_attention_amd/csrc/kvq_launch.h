// Internal launch interface between the C ABI (kvq_api.hip) and the kernels. Arguments have
// already been validated by the caller of these functions.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kTileTokens = 16;   // tokens handled per page sub-tile; page_size % 16 == 0

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
  int64_t num_slots;              // num_pages * page_size
  int32_t page_size;
  int32_t hb;                     // Hadamard block
  float inv_sqrt_hb;              // float32(1 / sqrt(hb))
  int32_t bits;
  int32_t token_scale;
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
  int32_t bits;
  float qk_scale_log2;            // softmax_scale * log2(e)
  float* out;
  int32_t num_splits;             // splits of the page range per (sequence, kv head)
  int32_t pages_per_split;
  float* ws_acc;                  // [num_splits][batch][num_q_heads][128]
  float* ws_ml;                   // [num_splits][batch][num_q_heads][2]  (max, sum) in log2 units
};

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

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_dequant(const DequantArgs& a, hipStream_t stream);

// Split plan used by both the workspace query and the launch.
struct SplitPlan {
  int32_t num_splits;
  int32_t pages_per_split;
};
SplitPlan plan_splits(int32_t batch, int32_t num_kv_heads, int32_t max_context_len, int32_t page_size,
                      int32_t pages_per_split_request);

}  // namespace kvq
