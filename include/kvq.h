/*
 * kvq.h - C ABI of the rotated low-bit paged KV cache for AMD Instinct MI355X (gfx950).
 *
 * Two hot paths and one inspection call, all asynchronous on a caller-supplied HIP stream:
 *
 *   kvq_rotate_quantize_append   write path: block-diagonal Hadamard rotation of every new
 *                                K/V head vector, token-wise asymmetric INT4 (or INT2)
 *                                quantization with a float32 scale and zero per token per
 *                                head, nibble packing, paged store through a slot mapping.
 *                                (SAW-INT4 abstract: "SAW-INT4: System-Aware 4-Bit KV-Cache
 *                                Quantization for Real-World LLM Serving", fugumt.com paper
 *                                page, Abstract - token-wise INT4 after a block-diagonal
 *                                Hadamard rotation, fused into a paged cache layout. The
 *                                optional per-token scaling step before quantization is the
 *                                S of the OScaR formula V-hat = Quant(S (R V)), zhichai.net
 *                                "OScaR: Occam's Razor for Extreme KV Cache Quantization in
 *                                LLMs", section "The OScaR Framework", used at INT2.)
 *   kvq_paged_decode_attention   read path: one decode query per head attends over its
 *                                sequence's quantized pages, dequantizing on the fly in the
 *                                rotated basis (the query is rotated by the same matrix),
 *                                split over pages with an online-softmax merge; one inverse
 *                                rotation of the output undoes the rotation of V.
 *                                (Dequantization fused into attention: ainews.cool
 *                                "Technical Deep Dive", third phase; a paged low-bit
 *                                attention kernel: the OSCAR abstract on the
 *                                thelatestinai.com page; split decoding against which OScaR
 *                                compares: FlashDecoding-v2, named in the OScaR abstract on
 *                                the same page.)
 *   kvq_dequant_page             codes of one page back to float32, optionally un-rotated
 *                                (inspection and test surface).
 *
 * Conventions shared by every entry point
 *   - Every pointer is DEVICE memory owned by the caller; the library allocates nothing,
 *     keeps no global state and may be called from several host threads at once.
 *   - Each call validates its arguments on the host, enqueues its kernels on `stream` and
 *     returns; results are valid once the caller synchronises the stream. No call blocks.
 *   - bf16 values cross the ABI as their 16-bit patterns (uint16_t).
 *   - Return value: KVQ_OK, or the first failed check (nothing is launched then), or
 *     KVQ_ERR_HIP if the launch itself failed. No C++ exception crosses the ABI.
 *   - head_dim must be 128 and page_size a multiple of 16 (KVQ_ERR_UNSUPPORTED otherwise).
 *   - Sizes whose launch would need 2^32 or more work-items in one grid dimension return
 *     KVQ_ERR_UNSUPPORTED: an append of more than 2^26 - 4 (16-token tile, KV head) items
 *     (about a billion token-heads), 2^26 or more (split, sequence, KV head) waves in a decode
 *     (splits of one sequence times sequences times KV heads), or 2^26 or more (query row, head)
 *     pairs in one attention call.
 *   - An attention call whose max_context_len needs a page (> 0) with num_pages == 0 returns
 *     KVQ_ERR_SHAPE: the page table would have nothing to point into.
 *   - Alignment (KVQ_ERR_SHAPE otherwise): k, v, q, out, k_codes and v_codes 16 bytes (the
 *     codes argument of kvq_dequant_page 4); slot_mapping, k_sz, v_sz 8; block_table and
 *     context_lens 4; token strides a multiple of 8 elements.
 *
 * Rotation R (block size b, a power of two dividing head_dim; b = 1 is no rotation, i.e.
 * plain INT4): R = blockdiag(H_b, ..., H_b) / sqrt(b), H_b the Sylvester Hadamard matrix
 * H_b[i][j] = (-1)^popcount(i & j), blocks over contiguous channels. R is symmetric and its
 * own inverse.
 *
 * Quantizer (per token, per KV head, per tensor): y = R x in float32; with token_scale,
 * s = RMS(y) (1 if 0) and u = y / s, else u = y, s = 1; scale_u = (max u - min u) / (2^bits - 1);
 * code = clamp(rint((u - min u) / scale_u), 0, 2^bits - 1) (round half to even, IEEE divide;
 * all codes 0 when scale_u = 0). Stored: scale = scale_u * s, zero = min u * s, so that
 * dequant = code * scale + zero in the rotated basis.
 *
 * Cache layout (row = head_dim * bits / 8 bytes; codes packed low bits first, i.e. for INT4
 * channel 2j is the low nibble of byte j, for INT2 channel 4j + k sits at bits 2k..2k+1):
 *   K codes  uint8 [num_pages][num_kv_heads][page_size][row]            token-major rows
 *   V codes  uint8 [num_pages][num_kv_heads][page_size / 4][row][4]     byte j of token t of a
 *            page-head tile sits at ((t / 4) * row + j) * 4 + t % 4: four consecutive tokens
 *            are interleaved byte by byte, so a 32-bit word holds one byte of four tokens
 *   K/V sz   float [num_pages][num_kv_heads][page_size][2] = {scale, zero}
 *   slot     = page * page_size + offset inside the page.
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 3

typedef int32_t kvq_status;
enum {
  KVQ_OK = 0,
  KVQ_ERR_NULL = 1,         /* a required pointer is NULL */
  KVQ_ERR_SHAPE = 2,        /* a size is negative or inconsistent (e.g. q heads not a multiple of kv heads) */
  KVQ_ERR_UNSUPPORTED = 3,  /* valid but not implemented: bits not 2/4, head_dim != 128, page_size % 16 */
  KVQ_ERR_WORKSPACE = 4,    /* decode workspace missing or smaller than kvq_paged_decode_workspace_size */
  KVQ_ERR_HIP = 5           /* the HIP runtime rejected a launch */
};

/* KVQ_ABI_VERSION of the loaded library. */
int32_t kvq_abi_version(void);

/* Static English text for a status code (never NULL). */
const char* kvq_status_string(int32_t status);

/*
 * Write path: rotate, quantize, pack and append num_tokens new tokens for every KV head.
 *
 *   k, v             bf16 [num_tokens][num_kv_heads][head_dim], head vectors contiguous;
 *                    token i starts at element i * k_token_stride (v_token_stride), both
 *                    >= num_kv_heads * head_dim.
 *   slot_mapping     int64 [num_tokens]: destination slot of token i; a negative slot skips
 *                    the token; slots >= num_pages * page_size are ignored as well. Two
 *                    tokens with the same slot in one call race (undefined result).
 *                    num_pages * page_size must stay below 2^32 (KVQ_ERR_UNSUPPORTED).
 *   k_codes, v_codes, k_sz, v_sz   the cache, layout above; only the addressed rows change.
 *   hadamard_block   b: power of two dividing head_dim (1 = no rotation).
 *   bits             4 (INT4) or 2 (INT2).
 *   token_scale      0: SAW-INT4 (rotate, quantize); 1: OScaR (rotate, scale per token, quantize).
 *
 * num_tokens == 0 is a no-op returning KVQ_OK.
 */
kvq_status kvq_rotate_quantize_append(
    const uint16_t* k, const uint16_t* v, int64_t k_token_stride, int64_t v_token_stride,
    int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
    const int64_t* slot_mapping,
    uint8_t* k_codes, uint8_t* v_codes, float* k_sz, float* v_sz,
    int32_t num_pages, int32_t page_size,
    int32_t hadamard_block, int32_t bits, int32_t token_scale,
    hipStream_t stream);

/*
 * Bytes of device workspace kvq_paged_decode_attention (and kvq_decode_step) needs for these
 * sizes (0 when the call runs unsplit). pages_per_split: 0 = the library's choice, else the
 * number of pages each split covers. Pass the same values to both calls.
 */
size_t kvq_paged_decode_workspace_size(
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t max_context_len, int32_t page_size, int32_t pages_per_split);

/*
 * Read path: one decode step of attention for every (sequence, query head).
 *
 *   q                bf16 [batch][num_q_heads][head_dim].
 *   q_prerotated     0: the kernel forms R q in float32 (the bf16 q is never re-rounded);
 *                    1: q already holds R q.
 *   k_codes ... v_sz the cache written by kvq_rotate_quantize_append (same bits, b).
 *   block_table      int32 [batch][max_pages_per_seq]: physical page of each logical page;
 *                    only the first ceil(context_lens[i] / page_size) entries are read.
 *   context_lens     int32 [batch] (device): tokens to attend per sequence, each in
 *                    [0, max_context_len]; 0 gives a zero output row.
 *   max_context_len  host-side upper bound of context_lens, used to size the grid.
 *   num_q_heads      multiple of num_kv_heads; query head h reads KV head h / (num_q_heads / num_kv_heads),
 *                    at most 8 query heads per KV head.
 *   softmax_scale    <= 0 selects 1 / sqrt(head_dim).
 *   out              float32 [batch][num_q_heads][head_dim], un-rotated (R applied once).
 *   workspace        device scratch of at least kvq_paged_decode_workspace_size(...) bytes
 *                    (may be NULL when that size is 0) for the partial results of split
 *                    sequences; its contents on entry do not matter and on return are
 *                    unspecified. Calls sharing a workspace must not overlap (e.g. run them on
 *                    one stream).
 *   pages_per_split  0 = library's choice; > 0 forces the split size (tuning and tests).
 *
 * batch == 0 is a no-op returning KVQ_OK.
 */
kvq_status kvq_paged_decode_attention(
    const uint16_t* q, int32_t q_prerotated,
    const uint8_t* k_codes, const uint8_t* v_codes, const float* k_sz, const float* v_sz,
    int32_t num_pages, int32_t page_size,
    const int32_t* block_table, int32_t max_pages_per_seq,
    const int32_t* context_lens, int32_t max_context_len,
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t hadamard_block, int32_t bits, float softmax_scale,
    float* out, void* workspace, size_t workspace_bytes, int32_t pages_per_split,
    hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): kvq_paged_decode_attention with the split partials in
 * a fixed scratch array inside the library instead of a caller workspace. Arguments, layouts,
 * results and error behaviour are those of kvq_paged_decode_attention without workspace and
 * workspace_bytes; the same kernels run. The call allocates nothing.
 *
 * The scratch is KVQ_DECODE_NOALLOC_SCRATCH_BYTES (16 MiB) of device memory per GPU, taken when the
 * library's code is loaded on that GPU and held until the process ends. Sizes whose partials
 * (kvq_paged_decode_workspace_size with the same arguments) exceed it return KVQ_ERR_WORKSPACE
 * before anything is launched. Every call on one GPU shares that GPU's scratch, and its contents
 * are those of the last call: calls that overlap on one GPU (other streams, other threads) race
 * and give undefined results; serialize them (e.g. one stream). The first call on a GPU looks up
 * that GPU's scratch address (a HIP runtime query, no allocation): callers that capture graphs make
 * one call on each GPU before capturing, so that the query does not fall inside the capture.
 */
#define KVQ_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

kvq_status kvq_paged_decode_attention_noalloc(
    const uint16_t* q, int32_t q_prerotated,
    const uint8_t* k_codes, const uint8_t* v_codes, const float* k_sz, const float* v_sz,
    int32_t num_pages, int32_t page_size,
    const int32_t* block_table, int32_t max_pages_per_seq,
    const int32_t* context_lens, int32_t max_context_len,
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t hadamard_block, int32_t bits, float softmax_scale,
    float* out, int32_t pages_per_split,
    hipStream_t stream);

/*
 * Several queries per sequence - chunked prefill, speculative verification: the causal attention
 * of each sequence's last q_lens[b] tokens, already appended to the cache, over its context (the
 * paged low-bit attention of the decode, with query tiles of more than one token).
 *
 *   q                bf16 [batch][max_q_len][num_q_heads][head_dim]; query j of sequence b sits at
 *                    position context_lens[b] - q_lens[b] + j and attends to tokens 0 .. that position.
 *   q_lens           int32 [batch] (device), each in [0, max_q_len]; clamped to context_lens[b].
 *   out              float32 [batch][max_q_len][num_q_heads][head_dim], un-rotated; rows with
 *                    j >= q_lens[b] are zero.
 *   workspace        at least kvq_paged_prefill_workspace_size(...) bytes (same arguments); unused (may
 *                    be NULL, 0 bytes) when kvq_paged_prefill_kernel(...) returns 1.
 *   Any number of query heads per KV head. All other arguments as for kvq_paged_decode_attention;
 *   with max_q_len = 1 and q_lens = 1 it computes the same attention.
 *   Large chunks (kvq_paged_prefill_kernel returns 1) run a kernel that stages each cache tile once
 *   per 256 (query, head) columns and takes both products on the fp16 matrix cores: the codes and
 *   the query (split into fp16 hi + lo parts) exactly enough for logits of hundreds of log2 units,
 *   V and the softmax weights in fp16 (relative error about 2^-12 each); it splits no context and
 *   leaves the workspace untouched.
 */
size_t kvq_paged_prefill_workspace_size(
    int32_t batch, int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t max_context_len, int32_t page_size, int32_t pages_per_split);

kvq_status kvq_paged_prefill_attention(
    const uint16_t* q, int32_t q_prerotated, const int32_t* q_lens, int32_t max_q_len,
    const uint8_t* k_codes, const uint8_t* v_codes, const float* k_sz, const float* v_sz,
    int32_t num_pages, int32_t page_size,
    const int32_t* block_table, int32_t max_pages_per_seq,
    const int32_t* context_lens, int32_t max_context_len,
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t hadamard_block, int32_t bits, float softmax_scale,
    float* out, void* workspace, size_t workspace_bytes, int32_t pages_per_split,
    hipStream_t stream);

/*
 * Which kernel kvq_paged_prefill_attention runs for these sizes: 1 for the large-chunk kernel -
 * max_q_len * (num_q_heads / num_kv_heads) >= 128 (query, head) columns per KV head and at least
 * 256 blocks of 128 columns over the batch and KV heads - 0 for the split kernel of the
 * decode with 16-column query tiles, -1 for sizes the call rejects (a size not positive,
 * num_q_heads not a multiple of num_kv_heads). Host only, no GPU call.
 */
int32_t kvq_paged_prefill_kernel(int32_t batch, int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads);

/*
 * Fused decode step: append each sequence's new token and attend, in one launch (the fused
 * pipeline of the OSCAR abstract on the thelatestinai.com page; one launch per layer per step).
 * Equivalent to kvq_rotate_quantize_append of k_new[b], v_new[b] at the slot of position
 * context_lens[b] - 1 (block_table[b][(L - 1) / page_size] * page_size + (L - 1) % page_size), followed by
 * kvq_paged_decode_attention over context_lens[b] tokens - so the new token is attended.
 *
 *   k_new, v_new     bf16 [batch][num_kv_heads][head_dim], token stride k_new_stride / v_new_stride
 *                    (elements, >= num_kv_heads * head_dim, a multiple of 8): the new token of each
 *                    sequence. Sequences with context_lens[b] == 0 append nothing (zero output); an
 *                    invalid page id at position L - 1 skips the append and masks the page.
 *   token_scale      as for kvq_rotate_quantize_append.
 *   All other arguments and the workspace as for kvq_paged_decode_attention (the cache arrays are
 *   written, so they are not const here). Only the query heads' outputs and the new tokens' cache
 *   rows change.
 */
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
    hipStream_t stream);

/*
 * Dequantize every token of one page of the K (tensor = 0) or V (tensor = 1) half of the
 * cache: out float32 [num_kv_heads][page_size][head_dim] = code * scale + zero (a single
 * rounding), multiplied by R^T when unrotate = 1. page must lie in [0, num_pages).
 */
kvq_status kvq_dequant_page(
    const uint8_t* codes, const float* sz, int32_t tensor, int32_t page, int32_t num_pages,
    int32_t num_kv_heads, int32_t page_size, int32_t head_dim,
    int32_t hadamard_block, int32_t bits, int32_t unrotate,
    float* out, hipStream_t stream);

/*
 * Baseline (for measurements side by side with the low-bit path): an unquantized bf16 paged
 * cache and split decode attention over it - the kind of BF16 split decode (FlashDecoding-v2,
 * named in the OScaR abstract on the thelatestinai.com page) the pages compare their speed-ups
 * against. Same block table, context lengths, GQA rule, softmax scale and error behaviour as
 * kvq_paged_decode_attention; no rotation. Its workspace (size from
 * kvq_paged_decode_bf16_workspace_size with the same arguments) holds only split partials, so
 * its contents on entry do not matter.
 *
 * Cache layout (bf16 bit patterns, caller-owned device memory):
 *   k_cache  uint16 [num_pages][num_kv_heads][page_size][head_dim]            token-major rows
 *   v_cache  uint16 [num_pages][num_kv_heads][page_size / 16][head_dim][16]   channel-major inside
 *            each run of 16 tokens: token t, channel c at [.., t / 16, c, t % 16]
 */

/* Copy bf16 K/V [num_tokens][num_kv_heads][head_dim] (token strides as for
 * kvq_rotate_quantize_append) to their slots; negative or out-of-pool slots are skipped. */
kvq_status kvq_bf16_cache_write(
    const uint16_t* k, const uint16_t* v, int64_t k_token_stride, int64_t v_token_stride,
    int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
    const int64_t* slot_mapping, uint16_t* k_cache, uint16_t* v_cache,
    int32_t num_pages, int32_t page_size, hipStream_t stream);

/* Bytes of workspace kvq_paged_decode_attention_bf16 needs (0 when it runs unsplit). */
size_t kvq_paged_decode_bf16_workspace_size(
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t max_context_len, int32_t page_size, int32_t pages_per_split);

/* Decode attention over the bf16 cache: out float32 [batch][num_q_heads][head_dim];
 * at most 16 query heads per KV head. */
kvq_status kvq_paged_decode_attention_bf16(
    const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
    int32_t num_pages, int32_t page_size,
    const int32_t* block_table, int32_t max_pages_per_seq,
    const int32_t* context_lens, int32_t max_context_len,
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
    float* out, void* workspace, size_t workspace_bytes, int32_t pages_per_split, hipStream_t stream);

/*
 * Per-channel pages - the per-channel reading of OScaR (OScaR abstract on the openalex page: the
 * rotation and a per-token scaling make per-channel quantization hold up at INT2; zhichai.net
 * "OScaR: Occam's Razor for Extreme KV Cache Quantization in LLMs", sections "Root Cause: Token
 * Norm Imbalance" and "The OScaR Framework", V-hat = Quant(S (R V))). Each token is rotated,
 * y = R x, and divided by its RMS s (1 if 0): u = y / s. The page_size tokens of one page and KV
 * head then share one asymmetric (scale, zero) per channel c over their u:
 *   scale_c = (max_t u_tc - min_t u_tc) / (2^bits - 1), zero_c = min_t u_tc,
 *   code_tc = clamp(rint((u_tc - zero_c) / scale_c), 0, 2^bits - 1)   (0 where scale_c = 0),
 * and dequant = s_t (code_tc * scale_c + zero_c) in the rotated basis. A page is quantized once all
 * its tokens exist; until then they stay in bf16 in the caller's residual window (tail).
 *
 * Layout (caller-owned device memory, row = head_dim * bits / 8 bytes):
 *   K codes, V codes   as the token-wise cache (see the top of this file)
 *   k_s, v_s           float [num_pages][num_kv_heads][page_size]         per-token s
 *   k_cp, v_cp         float [num_pages][num_kv_heads][2][head_dim]       {scale[head_dim], zero[head_dim]}
 *   tail_k, tail_v     bf16 [batch][page_size][num_kv_heads][head_dim]    sequence b's newest
 *                      context_lens[b] % page_size tokens, oldest first
 * page_size must be 32, 64 or 128 (KVQ_ERR_UNSUPPORTED otherwise). Alignment: k, v, codes, k_cp, v_cp,
 * tail_k, tail_v, q, out 16 bytes; k_s, v_s, page_ids, block_table, context_lens 4.
 */

/* Quantize whole pages: input page i is tokens i * page_size .. i * page_size + page_size - 1 of
 * k and v (bf16 [num_input_pages * page_size][num_kv_heads][head_dim], token strides as for
 * kvq_rotate_quantize_append) and is written to cache page page_ids[i] (int32 [num_input_pages]);
 * ids outside [0, num_pages) are skipped, and two inputs with the same id race. Writes the codes,
 * s and (scale, zero) of every KV head of those pages. num_input_pages == 0 is a no-op;
 * num_input_pages * num_kv_heads * page_size >= 2^30 gives KVQ_ERR_UNSUPPORTED. */
kvq_status kvq_pc_write_pages(
    const uint16_t* k, const uint16_t* v, int64_t k_token_stride, int64_t v_token_stride,
    int32_t num_input_pages, const int32_t* page_ids, int32_t num_kv_heads, int32_t head_dim,
    uint8_t* k_codes, uint8_t* v_codes, float* k_s, float* v_s, float* k_cp, float* v_cp,
    int32_t num_pages, int32_t page_size, int32_t hadamard_block, int32_t bits, hipStream_t stream);

/* Workspace bytes of kvq_pc_decode_attention (never 0 for batch > 0; same arguments). */
size_t kvq_pc_decode_workspace_size(
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t max_context_len, int32_t page_size, int32_t pages_per_split);

/* Decode attention over per-channel pages and the residual window: sequence b attends to its
 * context_lens[b] / page_size complete pages (block_table[b][0 ..], only those entries are read)
 * followed by its context_lens[b] % page_size tail tokens. q bf16 [batch][num_q_heads][head_dim]
 * (un-rotated; the kernel rotates it), at most 8 query heads per KV head; out float32
 * [batch][num_q_heads][head_dim] in the original basis; a sequence of length 0 gives zeros. The
 * workspace (kvq_pc_decode_workspace_size bytes) is required; its contents on entry do not
 * matter. Other arguments as for kvq_paged_decode_attention. */
kvq_status kvq_pc_decode_attention(
    const uint16_t* q,
    const uint8_t* k_codes, const uint8_t* v_codes, const float* k_s, const float* v_s,
    const float* k_cp, const float* v_cp, int32_t num_pages, int32_t page_size,
    const int32_t* block_table, int32_t max_pages_per_seq,
    const int32_t* context_lens, int32_t max_context_len,
    const uint16_t* tail_k, const uint16_t* tail_v,
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t hadamard_block, int32_t bits, float softmax_scale,
    float* out, void* workspace, size_t workspace_bytes, int32_t pages_per_split, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H_ */
