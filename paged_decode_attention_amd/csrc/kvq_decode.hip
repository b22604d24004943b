// Read path, host side: the split plan of the paged decode (how a sequence's pages are divided
// among waves for split decoding, FlashDecoding-v2 style, the baseline named in the OScaR abstract
// on the thelatestinai.com page) and the decode launch. The kernels are in kvq_decode_mfma.hip.
#include <algorithm>

#include "kvq_launch.h"

namespace kvq {

constexpr int64_t kMaxPagesFewSplits = 48;

SplitPlan plan_splits(int32_t batch, int32_t num_kv_heads, int32_t max_context_len, int32_t page_size,
                      int32_t pages_per_split_request, bool one_query) {
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
    // With few splits per sequence (a large batch fills the waves by itself), the longest
    // sequences' waves set the tail when lengths differ; 48 pages (768 tokens of 16) per split
    // bounds a wave's walk at one more partial per 48 pages.
    if (one_query && splits <= 8 && pps > kMaxPagesFewSplits) pps = kMaxPagesFewSplits;
    if (pps < max_pages && pps > 8) pps &= ~int64_t{1};
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
  return launch_decode_mfma(a, stream);  // launches its own merge
}

}  // namespace kvq
