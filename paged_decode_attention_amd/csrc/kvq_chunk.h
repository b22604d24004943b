// Launch interface of the large-chunk attention (kvq_chunk_attn.hip): several queries per sequence
// with at least 128 (query, head) columns per KV head, and enough of them to fill the chip - one
// launch, each cache tile dequantized once per 256 columns, no split partials, no workspace.
#pragma once

#include "kvq_launch.h"

namespace kvq {

// Whether kvq_paged_prefill_attention takes the large-chunk kernel for these (validated) arguments.
bool chunk_attention_applies(const DecodeArgs& a);
// The same rule on the sizes alone (num_q_heads a multiple of num_kv_heads, all positive).
bool chunk_attention_shape(int64_t batch, int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads);
hipError_t launch_chunk_attention(const DecodeArgs& a, hipStream_t stream);

}  // namespace kvq
