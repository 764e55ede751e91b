// build_sparse_indices: window slots + compressed slots per token (integer only).
//
// [vllm] build_flashinfer_mixed_sparse_indices / compute_global_topk_indices_and_lens,
// [backend] _update_decode_swa_metadata and the dense branch of
// _decode_compressed_attention_indices_and_lens.  One workgroup per token row;
// kept compressed candidates are compacted in candidate order with a ballot scan.
#include "sad_internal.h"

namespace sad {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 8;  // consecutive compressed candidates per thread and chunk

__global__ __launch_bounds__(kThreads) void build_sparse_indices_kernel(
    sad_batch b, const int32_t* __restrict__ replay, const int32_t* __restrict__ swa_bt,
    int64_t swa_stride, int swa_cols, int swa_block, int64_t swa_pages,
    const int32_t* __restrict__ comp_bt, int64_t comp_stride, int comp_cols, int comp_block,
    int64_t comp_pages, const int32_t* __restrict__ topk_local, int64_t topk_stride, int topk,
    int window, int ratio, int padded, int32_t* __restrict__ out, int32_t* __restrict__ lens) {
  __shared__ int wave_count[kThreads / 64];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int32_t* row = out + (int64_t)t * (window + padded);

  TokenGeom g;
  const bool ok = token_geometry_uniform(b, t, ratio, g);  // scalar-cache loads

  // Window columns: positions lo..pos ascending, then -1.
  int lo = 0;
  if (ok) {
    lo = g.pos - window + 1;
    if (replay != nullptr) lo = max(lo, uniform_ro_load(replay + g.req));
    lo = max(lo, 0);
  }
  const int32_t* swa_row = ok ? swa_bt + (int64_t)g.req * swa_stride : nullptr;
  for (int j = tid; j < window; j += kThreads) {
    const int p = lo + j;
    int s = -1;
    if (ok && p <= g.pos) s = page_slot(swa_row, swa_cols, swa_block, swa_pages, p);
    row[j] = s;
  }

  // Compressed columns: kept candidates packed left in candidate order.  Each thread
  // takes kPerThread consecutive candidates of a chunk: their id and table loads go out
  // together, and one workgroup scan places the kept ones.
  const int ncand = !ok ? 0 : (topk_local != nullptr ? topk : min(g.n_comp, padded));
  const int32_t* comp_row = ok ? comp_bt + (int64_t)g.req * comp_stride : nullptr;
  const int32_t* cand_row = topk_local != nullptr ? topk_local + (int64_t)t * topk_stride : nullptr;
  int base = 0;
  for (int c0 = 0; c0 < ncand; c0 += kThreads * kPerThread) {
    const int cb = c0 + tid * kPerThread;
    // Loads take clamped in-range addresses and are masked afterwards, so all of a
    // thread's loads of one kind are in flight together.
    int l[kPerThread];
    if (cand_row != nullptr) {
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) l[i] = cand_row[min(cb + i, ncand - 1)];
    } else {
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) l[i] = cb + i;
    }
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
      if (cb + i >= ncand || l[i] < 0 || l[i] >= g.n_comp || l[i] / comp_block >= comp_cols) l[i] = -1;
    int pg[kPerThread];
    if (comp_cols > 0) {
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) pg[i] = comp_row[l[i] < 0 ? 0 : l[i] / comp_block];
    } else {
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) pg[i] = -1;
    }
    int sl[kPerThread];
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const bool keep = l[i] >= 0 && pg[i] >= 0 && (int64_t)pg[i] < comp_pages;
      sl[i] = keep ? pg[i] * comp_block + l[i] % comp_block : -1;
      cnt += keep;
    }
    // exclusive scan of the per-thread counts
    const int incl = wave_incl_scan(cnt);
    if (lane == 63) wave_count[wave] = incl;
    __syncthreads();
    int off = base + incl - cnt;
    int total = base;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
      const int cw = wave_count[w];
      if (w < wave) off += cw;
      total += cw;
    }
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
      if (sl[i] >= 0) row[window + off++] = sl[i];
    base = total;
    __syncthreads();
  }
  for (int j = base + tid; j < padded; j += kThreads) row[window + j] = -1;
  if (tid == 0) lens[t] = base;
}

}  // namespace

int check_build_args(const char* what, const sad_batch* batch, const int32_t* swa_bt,
                     int64_t swa_bt_stride, int32_t swa_bt_cols, int32_t swa_block_size,
                     int64_t swa_num_pages, const int32_t* comp_bt, int64_t comp_bt_stride,
                     int32_t comp_bt_cols, int32_t comp_block_size, int64_t comp_num_pages,
                     bool has_topk, int64_t topk_stride, int32_t topk, int32_t window_size,
                     int32_t compress_ratio, int32_t padded_topk, const int32_t* sparse_indices,
                     const int32_t* sparse_topk_lens) {
  SAD_CHECK(batch != nullptr, SAD_EINVAL, "%s: batch is NULL", what);
  const int T = batch->num_tokens;
  SAD_CHECK(T >= 0 && batch->num_reqs >= 0, SAD_EINVAL, "%s: negative num_tokens/num_reqs", what);
  SAD_CHECK(window_size >= 0 && padded_topk >= 0 && topk >= 0, SAD_EINVAL,
            "%s: negative window_size/padded_topk/topk", what);
  SAD_CHECK(padded_topk % 64 == 0, SAD_EINVAL, "%s: padded_topk (%d) must be a multiple of 64", what,
            padded_topk);
  SAD_CHECK(compress_ratio >= 1, SAD_EINVAL, "%s: compress_ratio must be >= 1", what);
  SAD_CHECK(!has_topk || (topk <= padded_topk && topk_stride >= topk), SAD_EINVAL,
            "%s: need topk <= padded_topk and topk_stride >= topk", what);
  SAD_CHECK(swa_block_size >= 1 && comp_block_size >= 1, SAD_EINVAL, "%s: block sizes must be >= 1",
            what);
  SAD_CHECK(swa_bt_cols >= 0 && comp_bt_cols >= 0 && swa_num_pages >= 0 && comp_num_pages >= 0,
            SAD_EINVAL, "%s: negative table/pool size", what);
  SAD_CHECK(swa_num_pages * (int64_t)swa_block_size <= INT32_MAX &&
                comp_num_pages * (int64_t)comp_block_size <= INT32_MAX,
            SAD_EINVAL, "%s: slots must fit int32 (num_pages*block_size)", what);
  SAD_CHECK(swa_bt_stride >= swa_bt_cols && comp_bt_stride >= comp_bt_cols, SAD_EINVAL,
            "%s: table stride smaller than its column count", what);
  SAD_CHECK((int64_t)T * (window_size + padded_topk) < ((int64_t)1 << 40), SAD_EINVAL,
            "%s: output too large", what);
  if (T == 0) return SAD_OK;
  SAD_CHECK(batch->query_start_loc && batch->seq_lens && batch->token_to_req, SAD_EINVAL,
            "%s: batch arrays must be non-NULL", what);
  SAD_CHECK(swa_bt != nullptr && comp_bt != nullptr, SAD_EINVAL, "%s: block tables must be non-NULL",
            what);
  SAD_CHECK(sparse_indices != nullptr && sparse_topk_lens != nullptr, SAD_EINVAL,
            "%s: outputs must be non-NULL", what);
  return SAD_OK;
}

}  // namespace sad

using namespace sad;

extern "C" int build_sparse_indices(const sad_batch* batch, const int32_t* replay_start,
                                    const int32_t* swa_bt, int64_t swa_bt_stride,
                                    int32_t swa_bt_cols, int32_t swa_block_size,
                                    int64_t swa_num_pages, const int32_t* comp_bt,
                                    int64_t comp_bt_stride, int32_t comp_bt_cols,
                                    int32_t comp_block_size, int64_t comp_num_pages,
                                    const int32_t* topk_local, int64_t topk_stride, int32_t topk,
                                    int32_t window_size, int32_t compress_ratio,
                                    int32_t padded_topk, int32_t* sparse_indices,
                                    int32_t* sparse_topk_lens, void* stream) {
  clear_error();
  const int rc = check_build_args("build_sparse_indices", batch, swa_bt, swa_bt_stride, swa_bt_cols,
                                  swa_block_size, swa_num_pages, comp_bt, comp_bt_stride, comp_bt_cols,
                                  comp_block_size, comp_num_pages, topk_local != nullptr, topk_stride,
                                  topk, window_size, compress_ratio, padded_topk, sparse_indices,
                                  sparse_topk_lens);
  if (rc != SAD_OK || batch->num_tokens == 0) return rc;
  const int T = batch->num_tokens;
  hipLaunchKernelGGL(build_sparse_indices_kernel, dim3(T), dim3(kThreads), 0,
                     (hipStream_t)stream, *batch, replay_start, swa_bt, swa_bt_stride, swa_bt_cols,
                     swa_block_size, swa_num_pages, comp_bt, comp_bt_stride, comp_bt_cols,
                     comp_block_size, comp_num_pages, topk_local, topk_stride, topk, window_size,
                     compress_ratio, padded_topk, sparse_indices, sparse_topk_lens);
  return check_launch("build_sparse_indices");
}
