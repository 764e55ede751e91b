/*
 * sad.h - C ABI of libsad.so, the MI355X (gfx950) sparse-attention decode step.
 *
 * The step (DeepSeek-V4 style sparse MLA decode) has five parts:
 *   1. indexer scoring of each query token against MXFP4 keys of its request's
 *      compressed rows,
 *   2. per-token top-k over those scores,
 *   3. local->global slot mapping through paged block tables, merged with the
 *      sliding-window (SWA) slot ids into one sparse_indices row + a length,
 *   4. dequantize-and-gather of the selected rows of a paged FP8 latent cache,
 *   5. MLA attention of all query heads over the gathered rows.
 * Parts 1+2 are indexer_score_topk, part 3 is build_sparse_indices, part 4 is
 * gather_dequant_kv (standalone; also fused into part 5), part 5 is
 * sparse_mla_decode.
 *
 * Sources (web pages; cited by page and function):
 *   [ops]     tokenspeed "DeepSeek V4 attention kernel boundaries" page
 *             (runtime/layers/attention/deepseek_v4_ops.py)
 *   [model]   tokenspeed DeepSeek V4 model page (runtime/models/deepseek_v4.py)
 *   [backend] tokenspeed DeepSeek V4 attention backend page
 *   [vllm]    vLLM vllm.models.deepseek_v41.common.ops API page
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked "host".  Structs are passed
 *     by host pointer and read on the host during the call only.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream).  No call allocates device memory, copies,
 *     synchronizes or reads device data on the host, so every call may be
 *     captured into a HIP graph.
 *   - The caller owns every buffer; outputs and workspaces are caller
 *     preallocated (the pages never allocate under graph capture: [model]
 *     top-k buffer, [backend] SWA metadata).  The library keeps no state but
 *     a thread-local error string.
 *   - Return codes: SAD_OK; SAD_EINVAL (null required pointer, negative or
 *     inconsistent size); SAD_EUNSUPPORTED (a dimension or block size outside
 *     the supported set); SAD_EWORKSPACE (workspace too small); SAD_ELAUNCH
 *     (the HIP launch failed).  sad_last_error() describes the last non-OK
 *     return on the calling thread.  num_tokens == 0 returns SAD_OK and
 *     launches nothing ([ops] empty-input early returns).
 *   - Device data the host cannot check without a sync (stale ids, -1 pages,
 *     ids past a table or past the pool) is handled fail closed ([model]
 *     SWA slot sanitizing): any id that does not resolve to a row of the pool
 *     becomes -1 and is masked; -1 means "no row" everywhere ([vllm] "-1 = skip").
 *
 * Cache formats:
 *   sad_kv_cache (latent rows; [ops] dequantize_deepseek_v4_fp8_ds_mla_cache
 *   page addressing with fp32 instead of ue8m0 scales): page g starts at
 *   pool + g*page_stride and holds block_size rows.  Row o's values are at
 *   byte o*(d_nope + 2*d_rope): d_nope FP8 e4m3fn (OCP) bytes then d_rope
 *   bf16.  Row o's scales are at byte block_size*(d_nope + 2*d_rope) + o*4*(d_nope/64):
 *   d_nope/64 fp32, one per 64 nope elements.  Row value: nope[d] =
 *   bf16_rne(float(e4m3(v[d])) * scale[d/64]), rope copied.  A slot is
 *   page*block_size + row.  In the pages' native form (SAD_KV_SCALE_UE8M0,
 *   d_nope 448, d_rope 64: a 576-byte value row) row o's scales are 8 bytes at
 *   block_size*(d_nope + 2*d_rope) + o*8: 7 ue8m0 bytes, scale 2^(b-127), and
 *   one pad byte ([ops] deepseek_v4_swa_scale_dim); the product is exact.
 *
 *   sad_mxfp4_cache (indexer keys; [ops] read_deepseek_v4_indexer_mxfp4_cache):
 *   page g holds block_size rows: first block_size*dim/2 bytes of packed E2M1
 *   (row-major, low nibble = even element), then block_size*dim/32 e8m0
 *   exponents (value 2^(b-127), one per 32 elements).
 */
#ifndef SAD_H
#define SAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SAD_OK = 0,
  SAD_EINVAL = 1,
  SAD_EUNSUPPORTED = 2,
  SAD_EWORKSPACE = 3,
  SAD_ELAUNCH = 4
};

/* Scale forms of sad_kv_cache (see "Cache formats"). */
enum { SAD_KV_SCALE_F32 = 0, SAD_KV_SCALE_UE8M0 = 1 };

/* Paged FP8 latent KV cache (see "Cache formats").  Supported (d_nope, d_rope,
 * scale_format): (128, 32, F32), (512, 64, F32) and the pages' native record
 * (448, 64, UE8M0); block_size 16 or 64; page_stride a multiple of 16 and
 * >= block_size*(d_nope + 2*d_rope + scale bytes per row); num_pages*block_size < 2^31. */
typedef struct {
  const void* pool;     /* device, uint8 [num_pages * page_stride] */
  int64_t page_stride;  /* bytes between consecutive pages */
  int64_t num_pages;    /* page ids outside [0, num_pages) are invalid */
  int32_t block_size;   /* rows per page */
  int32_t d_nope;       /* FP8 part of the row */
  int32_t d_rope;       /* bf16 part of the row */
  int32_t scale_format; /* SAD_KV_SCALE_F32 or SAD_KV_SCALE_UE8M0 */
} sad_kv_cache;

/* Paged MXFP4 indexer-key cache.  dim 64 or 128; block_size 16 or 64;
 * page_stride a multiple of 16 and >= block_size*(dim/2 + dim/32). */
typedef struct {
  const void* pool;
  int64_t page_stride;
  int64_t num_pages;
  int32_t block_size;
  int32_t dim;
} sad_mxfp4_cache;

/* Ragged batch ([backend] init_forward_metadata / _decode_positions_from_metadata).
 * Token t belongs to request r = token_to_req[t] with query_start_loc[r] <= t <
 * query_start_loc[r+1]; seq_lens[r] counts this step's query tokens, so the
 * token's position is p = seq_lens[r] - (qsl[r+1]-qsl[r]) + (t - qsl[r]) and it
 * sees n_c = floor((p+1)/compress_ratio) compressed rows ([model] indexer
 * row_lens).  A token whose request id is out of range, or whose position is
 * negative, sees nothing. */
typedef struct {
  const int32_t* query_start_loc; /* device [num_reqs + 1] */
  const int32_t* seq_lens;        /* device [num_reqs] */
  const int32_t* token_to_req;    /* device [num_tokens] */
  int32_t num_reqs;
  int32_t num_tokens;
} sad_batch;

/*
 * build_sparse_indices - one sparse_indices row per token plus sparse_topk_lens.
 *
 * Defined by [vllm] build_flashinfer_mixed_sparse_indices (window columns first,
 * then compressed columns; replay_start lower-bounds the window) and
 * compute_global_topk_indices_and_lens (local id -> page*B + row, count of
 * valid entries), [backend] _update_decode_swa_metadata (window = last
 * window_size positions) and the dense branch of
 * _decode_compressed_attention_indices_and_lens (ratio-128 layers attend to
 * every compressed row).
 *
 * Row t of sparse_indices ([num_tokens, window_size + padded_topk] int32, row
 * stride window_size + padded_topk):
 *   columns [0, window_size): the slots of positions lo..p in ascending order,
 *     lo = max(p - window_size + 1, replay_start[r], 0), mapped through
 *     swa_bt[r][pos / swa_block_size]; then -1.  A position whose page is
 *     unbacked (< 0, past swa_bt_cols or past swa_num_pages) gives -1 in its column.
 *   columns [window_size, window_size + padded_topk): candidates are
 *     topk_local[t][0..topk) (local compressed-row ids, -1 = none), or, when
 *     topk_local is NULL (dense mode), 0..min(n_c, padded_topk)-1.  A candidate
 *     l is kept when 0 <= l < n_c and comp_bt[r][l / comp_block_size] is a valid
 *     page; kept candidates are written in candidate order as page*B + l%B,
 *     packed to the left; the rest of the segment is -1.
 *   sparse_topk_lens[t] = number of kept candidates.
 * Integer-only; bit-exact.  padded_topk must be >= topk and a multiple of 64;
 * topk_stride >= topk.  Block tables are int32 [num_reqs, cols] with row stride
 * *_bt_stride (elements).  replay_start may be NULL (all 0).
 */
int build_sparse_indices(const sad_batch* batch, const int32_t* replay_start,
                         const int32_t* swa_bt, int64_t swa_bt_stride, int32_t swa_bt_cols,
                         int32_t swa_block_size, int64_t swa_num_pages,
                         const int32_t* comp_bt, int64_t comp_bt_stride, int32_t comp_bt_cols,
                         int32_t comp_block_size, int64_t comp_num_pages,
                         const int32_t* topk_local, int64_t topk_stride, int32_t topk,
                         int32_t window_size, int32_t compress_ratio, int32_t padded_topk,
                         int32_t* sparse_indices, int32_t* sparse_topk_lens, void* stream);

/*
 * indexer_score_topk - indexer scores and per-token top-k local ids.
 *
 * Defined by [model] _deepseek_v4_indexer_topk_from_cache_deepgemm_decode (per
 * token, MXFP4 query heads against every paged MXFP4 key of the token's
 * request, weighted into one fp32 logit per compressed row) and
 * _deepseek_v4_indexer_topk_from_logits (top-k over the first n_c logits,
 * output prefilled with -1); weights are pre-folded as w * Di^-1/2 * Hi^-1/2
 * ([vllm] fused_indexer_q_rope_quant, MXFP4 path).
 *
 * For token t of request r and each compressed row s < n_c(t) whose key page
 * idx_bt[r][s / block_size] is valid:
 *     score[s] = sum_h weights[t,h] * max(dot(q[t,h], key[s]), 0)
 * (the per-head ReLU is this library's reading of the unprinted combination).
 * q·key products are exact in fp32; the head sum is fp32.
 * topk_local[t][0..m) = the m = min(topk, #valid rows) highest-scoring row ids
 * in ASCENDING id order (ties at the threshold go to the lower id);
 * topk_local[t][m..topk) = -1.
 *
 *   q_values  [num_tokens, num_idx_heads, dim/2] u8 packed E2M1 (low nibble even)
 *   q_scales  [num_tokens, num_idx_heads, dim/32] u8 e8m0
 *   weights   [num_tokens, num_idx_heads] fp32 (pre-folded)
 *   idx_bt    int32 [num_reqs, idx_bt_cols], row stride idx_bt_stride
 *   topk_local out int32 [num_tokens, topk]
 *   logits_debug NULL, or out fp32 [num_tokens, logits_stride]: score[s] for
 *     valid rows s < n_c(t), -inf for invalid rows s < n_c(t) (others untouched);
 *     requires logits_stride >= idx_bt_cols*block_size.
 *   workspace  >= indexer_score_topk_workspace_size(num_tokens, idx_bt_cols*block_size, topk)
 * num_idx_heads in [1, 64]; topk in [1, 65536].  Up to 32768 rows
 * (idx_bt_cols*block_size) one workgroup per token selects the top-k; past that the
 * rows go in chunks of 32768 whose own top-k are merged, which needs
 * ceil(rows / 32768) * topk <= 32768 (else SAD_EUNSUPPORTED; e.g. topk 2048 allows
 * 524288 rows, a 2M-token context at compress_ratio 4).
 */
int indexer_score_topk(const sad_batch* batch, const uint8_t* q_values, const uint8_t* q_scales,
                       const float* weights, int32_t num_idx_heads, const sad_mxfp4_cache* keys,
                       const int32_t* idx_bt, int64_t idx_bt_stride, int32_t idx_bt_cols,
                       int32_t compress_ratio, int32_t topk, int32_t* topk_local,
                       float* logits_debug, int64_t logits_stride, void* workspace,
                       size_t workspace_bytes, void* stream);
size_t indexer_score_topk_workspace_size(int32_t num_tokens, int32_t max_ctx_rows, int32_t topk);

/*
 * indexer_topk_sparse_indices - indexer_score_topk and build_sparse_indices in one call
 * (up to 32768 rows the index build runs inside the top-k kernel, so the step takes one
 * launch fewer; past that the call runs the build as its own launch).
 *
 * Exactly indexer_score_topk(batch, q_values, ..., topk, topk_local, NULL, 0, workspace,
 * workspace_bytes) followed by build_sparse_indices(batch, replay_start, swa_bt, ...,
 * comp_num_pages, topk_local, topk_stride = topk, topk, window_size, compress_ratio,
 * padded_topk, sparse_indices, sparse_topk_lens): the same outputs, bit for bit, and
 * the union of both calls' argument rules and errors, plus comp_block_size a power of
 * two >= 16 (else SAD_EUNSUPPORTED).  Each argument means what it means there (see
 * both declarations above and below).
 */
int indexer_topk_sparse_indices(
    const sad_batch* batch, const uint8_t* q_values, const uint8_t* q_scales, const float* weights,
    int32_t num_idx_heads, const sad_mxfp4_cache* keys, const int32_t* idx_bt, int64_t idx_bt_stride,
    int32_t idx_bt_cols, int32_t compress_ratio, int32_t topk, int32_t* topk_local,
    const int32_t* replay_start, const int32_t* swa_bt, int64_t swa_bt_stride, int32_t swa_bt_cols,
    int32_t swa_block_size, int64_t swa_num_pages, const int32_t* comp_bt, int64_t comp_bt_stride,
    int32_t comp_bt_cols, int32_t comp_block_size, int64_t comp_num_pages, int32_t window_size,
    int32_t padded_topk, int32_t* sparse_indices, int32_t* sparse_topk_lens, void* workspace,
    size_t workspace_bytes, void* stream);

/*
 * prepare_indexer_q_mxfp4 - the indexer query in the form indexer_score_topk takes.
 *
 * Defined by [ops] deepseek_v4_prepare_indexer_q_mxfp4 with
 * _apply_gptj_rope_tail_rows and _deepseek_v4_hadamard_rotate, and by [vllm]
 * fused_indexer_q_rope_quant (MXFP4 path).  Per (token t, head h) row x of
 * idx_dim bf16 values:
 *   1. RoPE, GPT-J style, on the last rope_dim elements: with n = idx_dim - rope_dim,
 *      c_i = cos_sin_cache[p][i], s_i = cos_sin_cache[p][rope_dim/2 + i] and
 *      p = positions[t], the pair (e, o) = (x[n+2i], x[n+2i+1]) becomes
 *      (e*c_i - o*s_i, e*s_i + o*c_i), each product and sum one fp32 operation;
 *      the row is then rounded to bf16 (nearest even);
 *   2. y = bf16(fp32(H x) * fp32(idx_dim^-1/2)) with H the Sylvester Hadamard
 *      matrix (H[i][j] = (-1)^popcount(i & j)); H x is the fp32 radix-2 fast
 *      transform: stages over the element-index bits, bit 0 first, each pair
 *      (i, i + s) becoming (x_i + x_{i+s}, x_i - x_{i+s}) in fp32;
 *   3. MXFP4 per 32 elements: e = the smallest integer with 6 * 2^e >= max|y|
 *      (-127 for a block below 2^-126), clamped to [-127, 127]; scale byte e + 127;
 *      each element's E2M1 code is the grid value nearest |y| / 2^e (a tie goes to
 *      the even code) with bit 3 = the sign bit of y (-0.0 gives 0x8); the even
 *      element is the low nibble;
 *   4. weights_out = fp32(fp32(weights * softmax_scale) * head_scale).
 * A token whose position is outside [0, max_pos) is failed closed: its codes and
 * scale bytes are 0 and its folded weights 0.  Inputs are finite.
 *
 *   index_q        [num_tokens, num_idx_heads, idx_dim] bf16, 16-byte aligned
 *   positions      [num_tokens] int32
 *   cos_sin_cache  [max_pos, rope_dim] fp32 (cos columns, then sin), 16-byte aligned
 *   weights        [num_tokens, num_idx_heads] fp32
 *   q_values       out [num_tokens, num_idx_heads, idx_dim/2] u8, 16-byte aligned
 *   q_scales       out [num_tokens, num_idx_heads, idx_dim/32] u8 (e8m0)
 *   weights_out    out [num_tokens, num_idx_heads] fp32
 * idx_dim in {64, 128} (else SAD_EUNSUPPORTED); rope_dim a multiple of 8 in
 * (0, idx_dim) and max_pos >= 1 (else SAD_EINVAL).  num_tokens == 0 is a no-op.
 */
int prepare_indexer_q_mxfp4(const uint16_t* index_q, const int32_t* positions,
                            const float* cos_sin_cache, int32_t max_pos, int32_t rope_dim,
                            const float* weights, float softmax_scale, float head_scale,
                            int32_t num_tokens, int32_t num_idx_heads, int32_t idx_dim,
                            uint8_t* q_values, uint8_t* q_scales, float* weights_out,
                            void* stream);

/*
 * gather_dequant_kv - dequantized rows of every attended column.
 *
 * Defined by [ops] dequantize_deepseek_v4_fp8_ds_mla_cache (slot -> page row,
 * one fp32 multiply per FP8 element, bf16 rounding, slot -1 -> zero row) and
 * [vllm] dequantize_and_gather_k_cache.
 * out[t][c] ([num_tokens, window_size + padded_topk, d_nope + d_rope] bf16) is
 * the dequantized row at slot sparse_indices[t][c] for window columns
 * c < window_size (read from `swa`) and for compressed columns
 * window_size <= c < window_size + sparse_topk_lens[t] (read from `comp`); it
 * is all zeros for slot -1, for slots that do not resolve to a row of the pool,
 * and for compressed columns past sparse_topk_lens[t].  Bit-exact.
 * `swa` and `comp` must have the same (d_nope, d_rope); they may share a pool.
 */
int gather_dequant_kv(const sad_kv_cache* swa, const sad_kv_cache* comp,
                      const int32_t* sparse_indices, const int32_t* sparse_topk_lens,
                      int32_t num_tokens, int32_t window_size, int32_t padded_topk,
                      uint16_t* out_bf16, void* stream);

/*
 * sparse_mla_decode - attention of every query head over the attended rows.
 *
 * Defined by [backend] forward_deepseek_v4_decode (FlashMLA sparse decode over
 * window ids bounded by their lengths plus compressed ids bounded by
 * extra_topk_length, FP8 cache, head_dim_v = head_dim, per-head attention
 * sink) and [model] DeepseekV4Attention (softmax scale = head_dim^-1/2).
 * For token t and head h, over the attended columns j (window columns with a
 * valid slot, compressed columns < sparse_topk_lens[t] with a valid slot) with
 * x_j the dequantized row (d_nope + d_rope values, as in gather_dequant_kv):
 *     l_j = softmax_scale * dot(q[t,h], x_j)
 *     out[t,h] = sum_j exp(l_j) x_j / (sum_j exp(l_j) + exp(attn_sink[h]))
 *     lse[t,h] = log(sum_j exp(l_j) + exp(attn_sink[h]))      (natural log)
 * (sink terms absent when attn_sink is NULL).  With nothing attended and no
 * sink, out = 0 and lse = -inf.  fp32 softmax and accumulation (bf16 MFMA
 * operands), bf16 out.
 *   q_bf16  [num_tokens, num_heads, d_nope + d_rope] bf16
 *   out_bf16 [num_tokens, num_heads, d_nope + d_rope] bf16
 *   lse      NULL or fp32 [num_tokens, num_heads]
 *   sparse_indices [num_tokens, window_size + padded_topk] int32 (may be NULL
 *            when window_size + padded_topk = 0); sparse_topk_lens [num_tokens]
 *   workspace >= sparse_mla_decode_workspace_size(num_tokens, num_heads,
 *                window_size + padded_topk, d_nope + d_rope)
 * num_heads in {8, 16, ..., 128} (a multiple of 8, <= 128); (d_nope, d_rope,
 * scale_format) = (512, 64, F32), (128, 32, F32) or the pages' native (448, 64, UE8M0),
 * the same for both caches; page sizes (block_size) of both caches are powers of two
 * and may differ (the window cache and the compressed cache are separate pools).
 * With fewer (token, 64-head group) pairs than compute units a token's columns are
 * split over several workgroups (as many as keep one workgroup per compute unit, each
 * with at least 4 tiles of 32 columns, at most 256); the fp32 partial results are
 * merged through the workspace.
 */
int sparse_mla_decode(const uint16_t* q_bf16, int32_t num_tokens, int32_t num_heads,
                      const sad_kv_cache* swa, const sad_kv_cache* comp,
                      const int32_t* sparse_indices, const int32_t* sparse_topk_lens,
                      int32_t window_size, int32_t padded_topk, float softmax_scale,
                      const float* attn_sink, uint16_t* out_bf16, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream);
size_t sparse_mla_decode_workspace_size(int32_t num_tokens, int32_t num_heads,
                                        int32_t max_row_width, int32_t dv);

/*
 * sparse_mla_decode_noalloc - sparse_mla_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, the same outputs and errors.
 *
 * The split partials go to a static 32 MiB scratch array inside the library, one per
 * GPU, held until the process ends; its device address is resolved on the first call on
 * each device that splits a token's columns (make such a first call outside graph
 * capture).  No call allocates or frees memory.  When the partials of the column splits
 * that sparse_mla_decode would use exceed 32 MiB, fewer splits are used (outputs then
 * differ from sparse_mla_decode's only by the fp32 summation order), so no input is
 * refused for its size.  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (on different streams or threads) race and must be
 * serialized by the caller.  SAD_ELAUNCH if the array has no device address on the
 * current device.
 */
int sparse_mla_decode_noalloc(const uint16_t* q_bf16, int32_t num_tokens, int32_t num_heads,
                              const sad_kv_cache* swa, const sad_kv_cache* comp,
                              const int32_t* sparse_indices, const int32_t* sparse_topk_lens,
                              int32_t window_size, int32_t padded_topk, float softmax_scale,
                              const float* attn_sink, uint16_t* out_bf16, float* lse, void* stream);

/*
 * inv_rope_fp8_quant - the attention output in the form the output projection takes.
 *
 * Defined by [vllm] fused_inv_rope_fp8_quant and [model] _project_attention_output
 * (attention RoPE: GPT-J style, is_neox_style=False; cos/sin table with the cos half
 * first) and by [ops] _fp8_e4m3_pow2_bytes (power-of-two FP8 block scales).  With
 * G = n_groups, hpg = num_heads / G and D = hpg * head_dim:
 *   1. in every head, with n = head_dim - rope_dim, c_i = cos_sin_cache[p][i],
 *      s_i = cos_sin_cache[p][rope_dim/2 + i] and p = positions[t], the pair
 *      (e, o) = (x[n+2i], x[n+2i+1]) becomes (e*c_i + o*s_i, o*c_i - e*s_i), each
 *      product and sum one fp32 operation (the inverse of the forward rotation);
 *   2. row (g, t) is heads g*hpg .. g*hpg + hpg - 1 of token t, heads then dims (D
 *      values); it is cut into blocks of 128 consecutive values (a block may span two
 *      heads);
 *   3. per block: e = the smallest integer with 448 * 2^e >= max|x|, at least -33
 *      (= ceil(log2(max(amax / 448, 1e-10)))); out_scales = 2^e (fp32); each code is
 *      the e4m3fn value nearest x / 2^e (a tie goes to the even code, the sign bit is
 *      copied) - the rotated fp32 values are quantized directly.
 * A token whose position is outside [0, max_pos) is failed closed: zero codes and
 * zero scales.  Inputs are finite.
 *
 *   attn_out      [num_tokens, num_heads, head_dim] bf16, 16-byte aligned
 *   positions     [num_tokens] int32
 *   cos_sin_cache [max_pos, rope_dim] fp32, 16-byte aligned
 *   out_fp8       out [n_groups, num_tokens, D] u8 (e4m3fn), 16-byte aligned
 *   out_scales    out [n_groups, num_tokens, D/128] fp32
 * num_heads a multiple of n_groups; head_dim (>= 32) and rope_dim multiples of 8
 * with 0 < rope_dim <= head_dim; D a multiple of 128; max_pos >= 1 (else SAD_EINVAL).
 * num_tokens == 0 is a no-op.
 */
int inv_rope_fp8_quant(const uint16_t* attn_out, const int32_t* positions,
                       const float* cos_sin_cache, int32_t max_pos, int32_t rope_dim,
                       int32_t num_tokens, int32_t num_heads, int32_t head_dim,
                       int32_t n_groups, uint8_t* out_fp8, float* out_scales, void* stream);

/*
 * insert_kv_rows - compressed KV rows into the paged FP8 latent cache (the write side
 * of the rows sparse_mla_decode reads).
 *
 * Defined by [ops] _write_fp8_ds_mla_cache_rows_capturable and _fp8_ds_mla_cache_rows,
 * with the fp32 scale form of the cache (sad_kv_cache): for row i with slot
 * s = slot_mapping[i] and compressed position c = floor(positions[i] / ratio) * ratio:
 *   - rope part: GPT-J rotation at c ((e, o) -> (e*cos - o*sin, e*sin + o*cos), each
 *     product and sum one fp32 operation), stored bf16 (nearest even);
 *   - nope part, per 64 values: scale = fp32(max(amax, 1e-4)) / 448 and code =
 *     e4m3fn(clamp(x / scale, +-448)) (correctly rounded fp32 divisions, nearest even);
 *   - row s % B of page s / B: values at page*page_stride + (s % B)*(Dn + 2*Dr), scales
 *     at page*page_stride + B*(Dn + 2*Dr) + (s % B)*4*Dn/64.
 * In the native form (SAD_KV_SCALE_UE8M0, 448 + 64) the nope part takes the pages' own
 * rule ([ops] _fp8_ds_mla_cache_rows): per 64 values e = the smallest integer with
 * 448 * 2^e >= max(amax, 1e-4), code = e4m3fn(x * 2^-e), scale byte e + 127, and the
 * row's 8th scale byte is a zero pad.
 * A negative slot, a page past num_pages or c outside [0, max_pos) writes nothing.  The
 * cache's pool is written in place; two rows with the same slot race.
 *
 *   rows           [num_rows, Dn + Dr] bf16 (before RoPE), 16-byte aligned
 *   positions      [num_rows] int32 token positions
 *   cos_sin_cache  [max_pos, Dr] fp32 (cos columns, then sin), 16-byte aligned
 *   slot_mapping   [num_rows] int32
 * (Dn, Dr) and the page geometry as for sparse_mla_decode; compress_ratio >= 1 and
 * max_pos >= 1 (else SAD_EINVAL).  num_rows == 0 is a no-op.
 */
int insert_kv_rows(const uint16_t* rows, const int32_t* positions, const float* cos_sin_cache,
                   int32_t max_pos, int32_t compress_ratio, const int32_t* slot_mapping,
                   int32_t num_rows, const sad_kv_cache* cache, void* stream);

/*
 * insert_index_keys - compressed indexer keys into the paged MXFP4 cache (the write side
 * of the keys indexer_score_topk reads).
 *
 * Defined by the [ops] compressor path (_apply_gptj_rope_tail_rows at the compressed
 * position, then _deepseek_v4_hadamard_rotate, then the quantizer) and
 * write_deepseek_v4_indexer_mxfp4_cache (page = [B x dim/2 values] then
 * [B x dim/32 e8m0]).  Each key takes exactly the steps 1-3 of prepare_indexer_q_mxfp4
 * (RoPE on the last rope_dim values at c = floor(positions[i] / ratio) * ratio, bf16,
 * the fp32 fast Hadamard transform with scale dim^-1/2, bf16, MXFP4) and is stored at
 * row s % B of page s / B, s = slot_mapping[i].  A negative slot, a page past
 * num_pages or c outside [0, max_pos) writes nothing; the pool is written in place.
 *
 *   keys           [num_rows, dim] bf16 (before RoPE), 16-byte aligned
 *   positions      [num_rows] int32; cos_sin_cache [max_pos, rope_dim] fp32, 16-byte aligned
 *   slot_mapping   [num_rows] int32
 * dim in {64, 128} and block_size in {16, 64} (else SAD_EUNSUPPORTED); rope_dim a
 * multiple of 8 in (0, dim); page_stride >= block_size*(dim/2 + dim/32), a multiple of
 * 16; the pool 16-byte aligned (else SAD_EINVAL).  num_rows == 0 is a no-op.
 */
int insert_index_keys(const uint16_t* keys, const int32_t* positions, const float* cos_sin_cache,
                      int32_t max_pos, int32_t rope_dim, int32_t compress_ratio,
                      const int32_t* slot_mapping, int32_t num_rows, const sad_mxfp4_cache* cache,
                      void* stream);

/* Description of the last non-OK return on the calling thread ("" if none). */
const char* sad_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SAD_H */
