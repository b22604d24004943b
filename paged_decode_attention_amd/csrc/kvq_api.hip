// C ABI of libkvq: argument validation, workspace sizing and kernel launches. Host code only;
// the kernels live in kvq_append.hip, kvq_decode_mfma.hip, kvq_dequant.hip, kvq_baseline_bf16.hip,
// kvq_pc_write.hip and kvq_pc.hip.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/kvq.h"
#include "kvq_chunk.h"
#include "kvq_launch.h"

namespace {

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// A launch dimension holds fewer than 2^32 work-items (blocks x threads per block).
bool grid_fits(int64_t blocks, int64_t threads_per_block) {
  return blocks >= 0 && blocks <= (int64_t{0xFFFFFFFF} / threads_per_block);
}

kvq_status check_common(int32_t head_dim, int32_t page_size, int32_t hadamard_block, int32_t bits) {
  if (page_size <= 0 || hadamard_block <= 0) return KVQ_ERR_SHAPE;
  if (bits != 2 && bits != 4) return KVQ_ERR_UNSUPPORTED;
  if (head_dim != kvq::kHeadDim) return KVQ_ERR_UNSUPPORTED;
  if (page_size % kvq::kTileTokens) return KVQ_ERR_UNSUPPORTED;
  if (!is_pow2(hadamard_block) || head_dim % hadamard_block) return KVQ_ERR_SHAPE;
  return KVQ_OK;
}

float inv_sqrt(int32_t b) { return static_cast<float>(1.0 / std::sqrt(static_cast<double>(b))); }

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace of a split call: the partial accumulators of every (split, sequence, query head),
// then their (max, sum) pairs. Every entry a merge reads is written by the same call first, so
// the contents on entry do not matter.
struct WorkspaceLayout {
  size_t acc_bytes, ml_offset, total;
};

WorkspaceLayout workspace_layout(int32_t num_splits, int32_t batch, int32_t num_q_heads, int32_t q_len_max = 1) {
  WorkspaceLayout w{0, 0, 0};
  if (num_splits <= 1) return w;
  const size_t rows = static_cast<size_t>(num_splits) * batch * q_len_max * num_q_heads;
  w.acc_bytes = rows * kvq::kHeadDim * sizeof(float);
  w.ml_offset = round_up(w.acc_bytes);
  w.total = w.ml_offset + round_up(rows * 2 * sizeof(float));
  return w;
}

}  // namespace

namespace kvq {

// Builds the lane plan of the cross-lane Walsh-Hadamard stages by running the butterfly network
// symbolically on the unit vectors of one block of lanes (see RowFwhtPlan).
RowFwhtPlan make_row_fwht_plan(int32_t hb) {
  RowFwhtPlan p{};
  p.hb = hb;
  p.inv_sqrt_hb = inv_sqrt(hb);
  uint64_t identity = 0;
  for (int l = 0; l < 16; ++l) identity |= static_cast<uint64_t>(l) << (4 * l);
  p.pos = identity;
  const int nl = hb >= 16 ? hb / 8 : 1;  // lanes per block
  int n = 0;
  while ((1 << n) < nl) ++n;
  p.lane_stages = n;
  if (n == 0) return p;
  auto parity = [](int x) { return __builtin_popcount(static_cast<unsigned>(x)) & 1; };
  static const int kMasks[4] = {1, 2, 7, 8};
  int dual[4] = {0, 0, 0, 0};  // functional f_k with f_k(m_j) = [j == k]: lane l is an "a" lane iff f_k(l) = 0
  for (int k = 0; k < n; ++k) {
    for (int f = 0; f < nl; ++f) {
      bool ok = true;
      for (int j = 0; j < n; ++j) ok = ok && (parity(f & kMasks[j]) == (j == k ? 1 : 0));
      if (ok) {
        dual[k] = f;
        break;
      }
    }
  }
  int v[16][16] = {};  // true value of lane l as +-1 coefficients over the block's inputs
  int sig[16];
  for (int l = 0; l < nl; ++l) {
    v[l][l] = 1;
    sig[l] = 1;
  }
  for (int k = 0; k < n; ++k) {
    const int m = kMasks[k];
    int nv[16][16], nsig[16];
    for (int l = 0; l < nl; ++l) {
      const bool a = parity(dual[k] & l) == 0;
      const int c = (a ? 1 : -1) * sig[l] * sig[l ^ m];
      if (c < 0)
        for (int blk = 0; blk < 16; blk += nl) p.neg[k] |= 1u << (blk + l);
      nsig[l] = a ? sig[l] : -sig[l];
      for (int i = 0; i < nl; ++i) nv[l][i] = (c * sig[l ^ m] * v[l ^ m][i] + sig[l] * v[l][i]) * nsig[l];
    }
    for (int l = 0; l < nl; ++l) {
      sig[l] = nsig[l];
      for (int i = 0; i < nl; ++i) v[l][i] = nv[l][i];
    }
  }
  p.pos = 0;
  for (int l = 0; l < nl; ++l) {
    int row = -1;
    for (int r = 0; r < nl && row < 0; ++r) {
      bool eq = true;
      for (int i = 0; i < nl; ++i) eq = eq && (v[l][i] == (parity(r & i) ? -1 : 1));
      if (eq) row = r;
    }
    for (int blk = 0; blk < 16; blk += nl) {
      p.pos |= static_cast<uint64_t>(blk + row) << (4 * (blk + l));
      if (sig[l] < 0) p.sign |= 1u << (blk + l);
    }
  }
  return p;
}

}  // namespace kvq

extern "C" {

int32_t kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char* kvq_status_string(int32_t status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "a required pointer is NULL";
    case KVQ_ERR_SHAPE: return "invalid or inconsistent size, stride, block size or alignment";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration (bits must be 2 or 4, head_dim 128, page_size a multiple of 16 (per-channel pages: 32, 64 or 128), at most 8 query heads per KV head for a single query)";
    case KVQ_ERR_WORKSPACE: return "decode workspace missing or too small (allocation-free decode: the split partials exceed its fixed scratch)";
    case KVQ_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

kvq_status kvq_rotate_quantize_append(
    const uint16_t* k, const uint16_t* v, int64_t k_token_stride, int64_t v_token_stride,
    int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
    const int64_t* slot_mapping,
    uint8_t* k_codes, uint8_t* v_codes, float* k_sz, float* v_sz,
    int32_t num_pages, int32_t page_size,
    int32_t hadamard_block, int32_t bits, int32_t token_scale,
    hipStream_t stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_pages < 0) return KVQ_ERR_SHAPE;
  if (kvq_status s = check_common(head_dim, page_size, hadamard_block, bits)) return s;
  if (token_scale != 0 && token_scale != 1) return KVQ_ERR_SHAPE;
  const int64_t row_elems = static_cast<int64_t>(num_kv_heads) * head_dim;
  if (k_token_stride < row_elems || v_token_stride < row_elems) return KVQ_ERR_SHAPE;
  if (k_token_stride % 8 || v_token_stride % 8) return KVQ_ERR_SHAPE;
  // one 64-lane wave per 16 tokens x one KV head, four per 256-thread workgroup
  if (num_kv_heads > 65535 || num_tokens > (int64_t{1} << 36) ||
      !grid_fits((((num_tokens + 15) / 16) * num_kv_heads + 3) / 4, 256))
    return KVQ_ERR_UNSUPPORTED;
  // 32-bit slots and rows per page
  if (static_cast<int64_t>(num_pages) * page_size > 0xFFFFFFFFll ||
      static_cast<int64_t>(num_kv_heads) * page_size > 0xFFFFFFFFll)
    return KVQ_ERR_UNSUPPORTED;
  if (num_tokens == 0) return KVQ_OK;
  if (!k || !v || !slot_mapping || !k_codes || !v_codes || !k_sz || !v_sz) return KVQ_ERR_NULL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(slot_mapping, 8) || !aligned(k_codes, 16) ||
      !aligned(v_codes, 16) || !aligned(k_sz, 8) || !aligned(v_sz, 8))
    return KVQ_ERR_SHAPE;

  kvq::AppendArgs a{};
  a.k = k;
  a.v = v;
  a.k_stride = k_token_stride;
  a.v_stride = v_token_stride;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.slots = slot_mapping;
  a.k_codes = k_codes;
  a.v_codes = v_codes;
  a.k_sz = k_sz;
  a.v_sz = v_sz;
  a.num_slots = static_cast<int64_t>(num_pages) * page_size;
  a.page_size = page_size;
  // Division by the invariant page size for 32-bit slots (Granlund-Montgomery, round-up
  // multiplier): l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1, then
  // n / d = (t + ((n - t) >> 1)) >> (l - 1) with t = umulhi(m, n), for every n < 2^32.
  {
    int l = 0;
    while ((int64_t{1} << l) < page_size) ++l;
    const uint64_t d = static_cast<uint64_t>(page_size);
    a.ps_magic = static_cast<uint32_t>(((uint64_t{1} << 32) * ((uint64_t{1} << l) - d)) / d + 1);
    a.ps_shift = l - 1;
  }
  a.rot = kvq::make_row_fwht_plan(hadamard_block);
  a.bits = bits;
  a.token_scale = token_scale;
  return kvq::launch_append(a, stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

size_t kvq_paged_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t max_context_len, int32_t page_size, int32_t pages_per_split) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim != kvq::kHeadDim || page_size <= 0 ||
      max_context_len < 0 || pages_per_split < 0)
    return 0;
  const kvq::SplitPlan p = kvq::plan_splits(batch, num_kv_heads, max_context_len, page_size, pages_per_split, true);
  return workspace_layout(p.num_splits, batch, num_q_heads).total;
}

size_t kvq_paged_decode_bf16_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t max_context_len, int32_t page_size,
                                            int32_t pages_per_split) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim != kvq::kHeadDim || page_size <= 0 ||
      max_context_len < 0 || pages_per_split < 0)
    return 0;
  const kvq::SplitPlan p = kvq::plan_splits(batch, num_kv_heads, max_context_len, page_size, pages_per_split, true);
  return workspace_layout(p.num_splits, batch, num_q_heads).total;
}

}  // extern "C"

namespace {

// Validation and argument set-up shared by the decode and the fused decode step.
kvq_status decode_args(
    kvq::DecodeArgs& a, const uint16_t* q, int32_t q_prerotated,
    const uint8_t* k_codes, const uint8_t* v_codes, const float* k_sz, const float* v_sz,
    int32_t num_pages, int32_t page_size, const int32_t* block_table, int32_t max_pages_per_seq,
    const int32_t* context_lens, int32_t max_context_len,
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t hadamard_block, int32_t bits, float softmax_scale,
    float* out, void* workspace, size_t workspace_bytes, int32_t pages_per_split, int32_t q_len_max = 0,
    bool uses_workspace = true) {
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_pages < 0 || max_context_len < 0 ||
      max_pages_per_seq < 0 || pages_per_split < 0 || q_len_max < 0)
    return KVQ_ERR_SHAPE;
  if (kvq_status s = check_common(head_dim, page_size, hadamard_block, bits)) return s;
  if (num_q_heads % num_kv_heads) return KVQ_ERR_SHAPE;
  if (q_prerotated != 0 && q_prerotated != 1) return KVQ_ERR_SHAPE;
  // one query per sequence: the heads of a KV head are the columns of one wave (at most 8);
  // several: columns are (query, head) pairs in tiles of 16, any group size
  if (q_len_max == 0 && num_q_heads / num_kv_heads > 8) return KVQ_ERR_UNSUPPORTED;
  const int32_t tiles = q_len_max > 0 ? kvq::mq_column_tiles(q_len_max, num_q_heads / num_kv_heads) : 1;
  if (num_kv_heads > 65535 || batch > 65535 || static_cast<int64_t>(num_kv_heads) * tiles > 65535)
    return KVQ_ERR_UNSUPPORTED;
  const int64_t need_pages = (static_cast<int64_t>(max_context_len) + page_size - 1) / page_size;
  if (max_pages_per_seq < need_pages) return KVQ_ERR_SHAPE;
  // a page table with entries to read needs a pool to point into
  if (need_pages > 0 && num_pages == 0) return KVQ_ERR_SHAPE;
  if (batch == 0) return KVQ_OK;
  const kvq::SplitPlan plan =
      kvq::plan_splits(batch * tiles, num_kv_heads, max_context_len, page_size, pages_per_split, q_len_max == 0);
  // one 64-lane wave per split and (sequence, KV head) item (one grid dimension with one query per
  // sequence), and per merged (query row, head) pair
  if (!grid_fits(static_cast<int64_t>(plan.num_splits) * (q_len_max > 0 ? 1 : static_cast<int64_t>(batch) * num_kv_heads), 64) ||
      !grid_fits(static_cast<int64_t>(batch) * (q_len_max > 0 ? q_len_max : 1) * num_q_heads, 64))
    return KVQ_ERR_UNSUPPORTED;
  if (!q || !k_codes || !v_codes || !k_sz || !v_sz || !block_table || !context_lens || !out) return KVQ_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(k_sz, 8) ||
      !aligned(v_sz, 8) || !aligned(block_table, 4) || !aligned(context_lens, 4))
    return KVQ_ERR_SHAPE;

  const WorkspaceLayout ws = workspace_layout(plan.num_splits, batch, num_q_heads, q_len_max > 0 ? q_len_max : 1);
  if (uses_workspace && ws.total > 0 && (!workspace || workspace_bytes < ws.total || !aligned(workspace, 16)))
    return KVQ_ERR_WORKSPACE;

  a = kvq::DecodeArgs{};
  a.q_len_max = q_len_max;
  a.q = q;
  a.q_prerotated = q_prerotated;
  a.k_codes = k_codes;
  a.v_codes = v_codes;
  a.k_sz = k_sz;
  a.v_sz = v_sz;
  a.page_size = page_size;
  a.block_table = block_table;
  a.max_pages_per_seq = max_pages_per_seq;
  a.context_lens = context_lens;
  a.max_context_len = max_context_len;
  a.num_pages = num_pages;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.hb = hadamard_block;
  a.inv_sqrt_hb = inv_sqrt(hadamard_block);
  a.rot = kvq::make_row_fwht_plan(hadamard_block);
  a.bits = bits;
  const double scale = softmax_scale > 0.f ? static_cast<double>(softmax_scale) : 1.0 / std::sqrt(static_cast<double>(head_dim));
  a.qk_scale_log2 = static_cast<float>(scale * 1.4426950408889634);  // log2(e)
  a.out = out;
  a.num_splits = plan.num_splits;
  a.pages_per_split = plan.pages_per_split;
  a.ws_acc = (uses_workspace && ws.total) ? static_cast<float*>(workspace) : nullptr;
  a.ws_ml = (uses_workspace && ws.total) ? reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.ml_offset) : nullptr;
  return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_paged_decode_attention(
    const uint16_t* q, int32_t q_prerotated,
    const uint8_t* k_codes, const uint8_t* v_codes, const float* k_sz, const float* v_sz,
    int32_t num_pages, int32_t page_size,
    const int32_t* block_table, int32_t max_pages_per_seq,
    const int32_t* context_lens, int32_t max_context_len,
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t hadamard_block, int32_t bits, float softmax_scale,
    float* out, void* workspace, size_t workspace_bytes, int32_t pages_per_split,
    hipStream_t stream) {
  kvq::DecodeArgs a;
  if (kvq_status s = decode_args(a, q, q_prerotated, k_codes, v_codes, k_sz, v_sz, num_pages, page_size, block_table,
                                 max_pages_per_seq, context_lens, max_context_len, batch, num_q_heads, num_kv_heads,
                                 head_dim, hadamard_block, bits, softmax_scale, out, workspace, workspace_bytes,
                                 pages_per_split))
    return s;
  if (batch == 0) return KVQ_OK;
  return kvq::launch_decode(a, stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------- allocation-free decode
//
// The split partials of kvq_paged_decode_attention_noalloc live in this array: one copy per GPU,
// placed by the runtime when the library's code is loaded there. Host code never uses its name as
// an address (on the host it is only a stand-in for the symbol): each GPU's copy is looked up once
// with hipGetSymbolAddress, with that GPU current, and the kernels take that address.
static __device__ __align__(256) uint8_t scratch[KVQ_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch` per device (null until looked up)

// The current device's copy of `scratch`.
kvq_status scratch_address(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return KVQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_paged_decode_attention_noalloc(
    const uint16_t* q, int32_t q_prerotated,
    const uint8_t* k_codes, const uint8_t* v_codes, const float* k_sz, const float* v_sz,
    int32_t num_pages, int32_t page_size,
    const int32_t* block_table, int32_t max_pages_per_seq,
    const int32_t* context_lens, int32_t max_context_len,
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t hadamard_block, int32_t bits, float softmax_scale,
    float* out, int32_t pages_per_split,
    hipStream_t stream) {
  // Validate every argument, and that the partials fit the scratch, against an aligned non-null
  // stand-in for the scratch's address (never dereferenced): nothing touches the device before
  // the call is known to be valid.
  void* const stand_in = reinterpret_cast<void*>(uintptr_t{256});
  kvq::DecodeArgs a;
  if (kvq_status s = decode_args(a, q, q_prerotated, k_codes, v_codes, k_sz, v_sz, num_pages, page_size, block_table,
                                 max_pages_per_seq, context_lens, max_context_len, batch, num_q_heads, num_kv_heads,
                                 head_dim, hadamard_block, bits, softmax_scale, out, stand_in,
                                 KVQ_DECODE_NOALLOC_SCRATCH_BYTES, pages_per_split))
    return s;
  if (batch == 0) return KVQ_OK;
  if (a.ws_acc) {  // split: point the partials at this GPU's scratch, at the same offsets
    char* base = nullptr;
    if (kvq_status s = scratch_address(&base)) return s;
    const char* const si = static_cast<const char*>(stand_in);
    a.ws_acc = reinterpret_cast<float*>(base + (reinterpret_cast<const char*>(a.ws_acc) - si));
    a.ws_ml = reinterpret_cast<float*>(base + (reinterpret_cast<const char*>(a.ws_ml) - si));
  }
  return kvq::launch_decode(a, stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

kvq_status kvq_decode_step(
    const uint16_t* q, int32_t q_prerotated,
    const uint16_t* k_new, const uint16_t* v_new, int64_t k_new_stride, int64_t v_new_stride,
    uint8_t* k_codes, uint8_t* v_codes, float* k_sz, float* v_sz,
    int32_t num_pages, int32_t page_size,
    const int32_t* block_table, int32_t max_pages_per_seq,
    const int32_t* context_lens, int32_t max_context_len,
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t hadamard_block, int32_t bits, int32_t token_scale, float softmax_scale,
    float* out, void* workspace, size_t workspace_bytes, int32_t pages_per_split,
    hipStream_t stream) {
  // shape checks of the new tokens first, as every entry point checks shapes before pointers
  if (token_scale != 0 && token_scale != 1) return KVQ_ERR_SHAPE;
  const int64_t row_elems = static_cast<int64_t>(num_kv_heads) * head_dim;
  if (num_kv_heads > 0 && (k_new_stride < row_elems || v_new_stride < row_elems || k_new_stride % 8 ||
                           v_new_stride % 8))
    return KVQ_ERR_SHAPE;
  kvq::DecodeArgs a;
  if (kvq_status s = decode_args(a, q, q_prerotated, k_codes, v_codes, k_sz, v_sz, num_pages, page_size, block_table,
                                 max_pages_per_seq, context_lens, max_context_len, batch, num_q_heads, num_kv_heads,
                                 head_dim, hadamard_block, bits, softmax_scale, out, workspace, workspace_bytes,
                                 pages_per_split))
    return s;
  if (batch == 0) return KVQ_OK;
  if (!k_new || !v_new) return KVQ_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return KVQ_ERR_SHAPE;
  a.fused = 1;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_new_stride = k_new_stride;
  a.v_new_stride = v_new_stride;
  a.token_scale = token_scale;
  a.k_codes_w = k_codes;
  a.v_codes_w = v_codes;
  a.k_sz_w = k_sz;
  a.v_sz_w = v_sz;
  return kvq::launch_decode_mfma(a, stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

kvq_status kvq_dequant_page(
    const uint8_t* codes, const float* sz, int32_t tensor, int32_t page, int32_t num_pages,
    int32_t num_kv_heads, int32_t page_size, int32_t head_dim,
    int32_t hadamard_block, int32_t bits, int32_t unrotate,
    float* out, hipStream_t stream) {
  if (num_kv_heads <= 0 || num_pages <= 0 || page < 0 || page >= num_pages) return KVQ_ERR_SHAPE;
  if (kvq_status s = check_common(head_dim, page_size, hadamard_block, bits)) return s;
  if ((tensor != 0 && tensor != 1) || (unrotate != 0 && unrotate != 1)) return KVQ_ERR_SHAPE;
  if (num_kv_heads > 65535) return KVQ_ERR_UNSUPPORTED;
  if (!codes || !sz || !out) return KVQ_ERR_NULL;
  if (!aligned(codes, 4) || !aligned(sz, 8) || !aligned(out, 16)) return KVQ_ERR_SHAPE;
  kvq::DequantArgs a{};
  a.codes = codes;
  a.sz = sz;
  a.tensor = tensor;
  a.page = page;
  a.num_kv_heads = num_kv_heads;
  a.page_size = page_size;
  a.hb = hadamard_block;
  a.inv_sqrt_hb = inv_sqrt(hadamard_block);
  a.bits = bits;
  a.unrotate = unrotate;
  a.out = out;
  return kvq::launch_dequant(a, stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}


// ---------------------------------------------------------------------------- several queries

int32_t kvq_paged_prefill_kernel(int32_t batch, int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads) {
  if (batch <= 0 || max_q_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads) return -1;
  return kvq::chunk_attention_shape(batch, max_q_len, num_q_heads, num_kv_heads) ? 1 : 0;
}

size_t kvq_paged_prefill_workspace_size(int32_t batch, int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t max_context_len, int32_t page_size,
                                        int32_t pages_per_split) {
  if (batch <= 0 || max_q_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
      head_dim != kvq::kHeadDim || page_size <= 0 || max_context_len < 0 || pages_per_split < 0)
    return 0;
  const int32_t tiles = kvq::mq_column_tiles(max_q_len, num_q_heads / num_kv_heads);
  const kvq::SplitPlan p =
      kvq::plan_splits(batch * tiles, num_kv_heads, max_context_len, page_size, pages_per_split, false);
  return workspace_layout(p.num_splits, batch, num_q_heads, max_q_len).total;
}

kvq_status kvq_paged_prefill_attention(
    const uint16_t* q, int32_t q_prerotated, const int32_t* q_lens, int32_t max_q_len,
    const uint8_t* k_codes, const uint8_t* v_codes, const float* k_sz, const float* v_sz,
    int32_t num_pages, int32_t page_size,
    const int32_t* block_table, int32_t max_pages_per_seq,
    const int32_t* context_lens, int32_t max_context_len,
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t hadamard_block, int32_t bits, float softmax_scale,
    float* out, void* workspace, size_t workspace_bytes, int32_t pages_per_split,
    hipStream_t stream) {
  if (max_q_len <= 0) return KVQ_ERR_SHAPE;
  if (static_cast<int64_t>(batch) * max_q_len > 0x7FFFFFFF / 128) return KVQ_ERR_UNSUPPORTED;
  // the large-chunk kernel takes no workspace (decode_args rejects the other sizes first)
  const bool chunk = kvq_paged_prefill_kernel(batch, max_q_len, num_q_heads, num_kv_heads) == 1;
  kvq::DecodeArgs a;
  if (kvq_status s = decode_args(a, q, q_prerotated, k_codes, v_codes, k_sz, v_sz, num_pages, page_size, block_table,
                                 max_pages_per_seq, context_lens, max_context_len, batch, num_q_heads, num_kv_heads,
                                 head_dim, hadamard_block, bits, softmax_scale, out, workspace, workspace_bytes,
                                 pages_per_split, max_q_len, !chunk))
    return s;
  if (batch == 0) return KVQ_OK;
  if (!q_lens) return KVQ_ERR_NULL;
  if (!aligned(q_lens, 4)) return KVQ_ERR_SHAPE;
  a.q_lens = q_lens;
  if (chunk) return kvq::launch_chunk_attention(a, stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
  return kvq::launch_decode_mfma(a, stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

// ---------------------------------------------------------------------------- bf16 baseline

kvq_status kvq_bf16_cache_write(
    const uint16_t* k, const uint16_t* v, int64_t k_token_stride, int64_t v_token_stride,
    int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
    const int64_t* slot_mapping, uint16_t* k_cache, uint16_t* v_cache,
    int32_t num_pages, int32_t page_size, hipStream_t stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_pages < 0 || page_size <= 0) return KVQ_ERR_SHAPE;
  if (head_dim != kvq::kHeadDim || page_size % kvq::kTileTokens) return KVQ_ERR_UNSUPPORTED;
  const int64_t row_elems = static_cast<int64_t>(num_kv_heads) * head_dim;
  if (k_token_stride < row_elems || v_token_stride < row_elems || k_token_stride % 8 || v_token_stride % 8)
    return KVQ_ERR_SHAPE;
  if (num_kv_heads > 65535 || !grid_fits((num_tokens + 15) / 16, 256)) return KVQ_ERR_UNSUPPORTED;
  if (num_tokens == 0) return KVQ_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return KVQ_ERR_NULL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(slot_mapping, 8) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16))
    return KVQ_ERR_SHAPE;
  kvq::Bf16WriteArgs a{};
  a.k = k;
  a.v = v;
  a.k_stride = k_token_stride;
  a.v_stride = v_token_stride;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.slots = slot_mapping;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_slots = static_cast<int64_t>(num_pages) * page_size;
  a.page_size = page_size;
  return kvq::launch_bf16_write(a, stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

kvq_status kvq_paged_decode_attention_bf16(
    const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
    int32_t num_pages, int32_t page_size,
    const int32_t* block_table, int32_t max_pages_per_seq,
    const int32_t* context_lens, int32_t max_context_len,
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
    float* out, void* workspace, size_t workspace_bytes, int32_t pages_per_split, hipStream_t stream) {
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_pages < 0 || max_context_len < 0 ||
      max_pages_per_seq < 0 || pages_per_split < 0 || page_size <= 0)
    return KVQ_ERR_SHAPE;
  if (head_dim != kvq::kHeadDim || page_size % kvq::kTileTokens) return KVQ_ERR_UNSUPPORTED;
  if (num_q_heads % num_kv_heads) return KVQ_ERR_SHAPE;
  if (num_q_heads / num_kv_heads > 16) return KVQ_ERR_UNSUPPORTED;
  if (num_kv_heads > 65535 || batch > 65535) return KVQ_ERR_UNSUPPORTED;
  const int64_t need_pages = (static_cast<int64_t>(max_context_len) + page_size - 1) / page_size;
  if (max_pages_per_seq < need_pages) return KVQ_ERR_SHAPE;
  if (need_pages > 0 && num_pages == 0) return KVQ_ERR_SHAPE;  // nothing for the page table to point into
  if (batch == 0) return KVQ_OK;
  const kvq::SplitPlan plan = kvq::plan_splits(batch, num_kv_heads, max_context_len, page_size, pages_per_split, true);
  if (!grid_fits(plan.num_splits, 64) || !grid_fits(static_cast<int64_t>(batch) * num_q_heads, 64))
    return KVQ_ERR_UNSUPPORTED;
  if (!q || !k_cache || !v_cache || !block_table || !context_lens || !out) return KVQ_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_table, 4) || !aligned(context_lens, 4))
    return KVQ_ERR_SHAPE;
  const WorkspaceLayout ws = workspace_layout(plan.num_splits, batch, num_q_heads);
  if (ws.total > 0 && (!workspace || workspace_bytes < ws.total || !aligned(workspace, 16))) return KVQ_ERR_WORKSPACE;
  kvq::DecodeBf16Args a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.page_size = page_size;
  a.block_table = block_table;
  a.max_pages_per_seq = max_pages_per_seq;
  a.context_lens = context_lens;
  a.max_context_len = max_context_len;
  a.num_pages = num_pages;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  const double scale = softmax_scale > 0.f ? static_cast<double>(softmax_scale) : 1.0 / std::sqrt(static_cast<double>(head_dim));
  a.qk_scale_log2 = static_cast<float>(scale * 1.4426950408889634);
  a.out = out;
  a.num_splits = plan.num_splits;
  a.pages_per_split = plan.pages_per_split;
  a.ws_acc = ws.total ? static_cast<float*>(workspace) : nullptr;
  a.ws_ml = ws.total ? reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.ml_offset) : nullptr;
  return kvq::launch_decode_bf16(a, stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------- per-channel pages

namespace {

kvq_status check_pc(int32_t head_dim, int32_t page_size, int32_t hadamard_block, int32_t bits) {
  if (kvq_status s = check_common(head_dim, page_size, hadamard_block, bits)) return s;
  if (page_size != 32 && page_size != 64 && page_size != kvq::kPcMaxPage) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

// Page splits over the complete pages, plus the split of the unfinished page.
kvq::SplitPlan pc_plan(int32_t batch, int32_t num_kv_heads, int32_t max_context_len, int32_t page_size,
                       int32_t pages_per_split) {
  const int32_t full_tokens = max_context_len / page_size * page_size;
  return kvq::plan_splits(batch, num_kv_heads, full_tokens, page_size, pages_per_split, true);
}

}  // namespace

extern "C" {

kvq_status kvq_pc_write_pages(
    const uint16_t* k, const uint16_t* v, int64_t k_token_stride, int64_t v_token_stride,
    int32_t num_input_pages, const int32_t* page_ids, int32_t num_kv_heads, int32_t head_dim,
    uint8_t* k_codes, uint8_t* v_codes, float* k_s, float* v_s, float* k_cp, float* v_cp,
    int32_t num_pages, int32_t page_size, int32_t hadamard_block, int32_t bits, hipStream_t stream) {
  if (num_input_pages < 0 || num_kv_heads <= 0 || num_pages < 0) return KVQ_ERR_SHAPE;
  if (kvq_status s = check_pc(head_dim, page_size, hadamard_block, bits)) return s;
  // one workgroup of 4 page_size threads per (input page, KV head), in one grid dimension
  if (!grid_fits(static_cast<int64_t>(num_input_pages) * num_kv_heads, 4 * page_size)) return KVQ_ERR_UNSUPPORTED;
  const int64_t row_elems = static_cast<int64_t>(num_kv_heads) * head_dim;
  if (k_token_stride < row_elems || v_token_stride < row_elems || k_token_stride % 8 || v_token_stride % 8)
    return KVQ_ERR_SHAPE;
  if (num_input_pages == 0) return KVQ_OK;
  if (!k || !v || !page_ids || !k_codes || !v_codes || !k_s || !v_s || !k_cp || !v_cp) return KVQ_ERR_NULL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(page_ids, 4) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
      !aligned(k_s, 4) || !aligned(v_s, 4) || !aligned(k_cp, 16) || !aligned(v_cp, 16))
    return KVQ_ERR_SHAPE;
  kvq::PcWriteArgs a{};
  a.k = k;
  a.v = v;
  a.k_stride = k_token_stride;
  a.v_stride = v_token_stride;
  a.num_input_pages = num_input_pages;
  a.page_ids = page_ids;
  a.num_kv_heads = num_kv_heads;
  a.k_codes = k_codes;
  a.v_codes = v_codes;
  a.k_s = k_s;
  a.v_s = v_s;
  a.k_cp = k_cp;
  a.v_cp = v_cp;
  a.num_pages = num_pages;
  a.page_size = page_size;
  a.rot = kvq::make_row_fwht_plan(hadamard_block);
  a.bits = bits;
  return kvq::launch_pc_write(a, stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

size_t kvq_pc_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t max_context_len, int32_t page_size, int32_t pages_per_split) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim != kvq::kHeadDim || page_size <= 0 ||
      max_context_len < 0 || pages_per_split < 0)
    return 0;
  const kvq::SplitPlan p = pc_plan(batch, num_kv_heads, max_context_len, page_size, pages_per_split);
  return workspace_layout(p.num_splits + 1, batch, num_q_heads).total;
}

kvq_status kvq_pc_decode_attention(
    const uint16_t* q,
    const uint8_t* k_codes, const uint8_t* v_codes, const float* k_s, const float* v_s,
    const float* k_cp, const float* v_cp, int32_t num_pages, int32_t page_size,
    const int32_t* block_table, int32_t max_pages_per_seq,
    const int32_t* context_lens, int32_t max_context_len,
    const uint16_t* tail_k, const uint16_t* tail_v,
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t hadamard_block, int32_t bits, float softmax_scale,
    float* out, void* workspace, size_t workspace_bytes, int32_t pages_per_split, hipStream_t stream) {
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_pages < 0 || max_context_len < 0 ||
      max_pages_per_seq < 0 || pages_per_split < 0)
    return KVQ_ERR_SHAPE;
  if (kvq_status s = check_pc(head_dim, page_size, hadamard_block, bits)) return s;
  if (num_q_heads % num_kv_heads) return KVQ_ERR_SHAPE;
  if (num_q_heads / num_kv_heads > 8) return KVQ_ERR_UNSUPPORTED;
  if (num_kv_heads > 65535 || batch > 65535) return KVQ_ERR_UNSUPPORTED;
  if (max_pages_per_seq < max_context_len / page_size) return KVQ_ERR_SHAPE;
  // complete pages to read need a pool to point into
  if (max_context_len / page_size > 0 && num_pages == 0) return KVQ_ERR_SHAPE;
  if (batch == 0) return KVQ_OK;
  const kvq::SplitPlan plan = pc_plan(batch, num_kv_heads, max_context_len, page_size, pages_per_split);
  // one wave per page split plus the tail's, and per merged (sequence, head) pair
  if (!grid_fits(static_cast<int64_t>(plan.num_splits) + 1, 64) ||
      !grid_fits(static_cast<int64_t>(batch) * num_q_heads, 64))
    return KVQ_ERR_UNSUPPORTED;
  if (!q || !k_codes || !v_codes || !k_s || !v_s || !k_cp || !v_cp || !block_table || !context_lens || !tail_k ||
      !tail_v || !out)
    return KVQ_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(k_s, 4) ||
      !aligned(v_s, 4) || !aligned(k_cp, 16) || !aligned(v_cp, 16) || !aligned(block_table, 4) ||
      !aligned(context_lens, 4) || !aligned(tail_k, 16) || !aligned(tail_v, 16))
    return KVQ_ERR_SHAPE;
  const WorkspaceLayout ws = workspace_layout(plan.num_splits + 1, batch, num_q_heads);
  if (!workspace || workspace_bytes < ws.total || !aligned(workspace, 16)) return KVQ_ERR_WORKSPACE;
  kvq::PcDecodeArgs a{};
  a.q = q;
  a.k_codes = k_codes;
  a.v_codes = v_codes;
  a.k_s = k_s;
  a.v_s = v_s;
  a.k_cp = k_cp;
  a.v_cp = v_cp;
  a.page_size = page_size;
  a.block_table = block_table;
  a.max_pages_per_seq = max_pages_per_seq;
  a.context_lens = context_lens;
  a.max_context_len = max_context_len;
  a.num_pages = num_pages;
  a.tail_k = tail_k;
  a.tail_v = tail_v;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.rot = kvq::make_row_fwht_plan(hadamard_block);
  a.bits = bits;
  const double scale = softmax_scale > 0.f ? static_cast<double>(softmax_scale) : 1.0 / std::sqrt(static_cast<double>(head_dim));
  a.qk_scale_log2 = static_cast<float>(scale * 1.4426950408889634);
  a.num_splits = plan.num_splits;
  a.pages_per_split = plan.pages_per_split;
  a.ws_acc = static_cast<float*>(workspace);
  a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.ml_offset);
  a.out = out;
  return kvq::launch_pc_decode(a, stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // extern "C"
