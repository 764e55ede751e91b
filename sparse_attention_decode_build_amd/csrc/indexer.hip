// indexer_score_topk: MXFP4 indexer scores and per-token top-k local row ids.
//
// [model] _deepseek_v4_indexer_topk_from_cache_deepgemm_decode (per token, every
// indexer head's MXFP4 query against each paged MXFP4 key of the request, weighted
// into one fp32 logit per compressed row) and _deepseek_v4_indexer_topk_from_logits
// (top-k of the first n_c logits, -1 prefilled).  The head combination
// sum_h w_h * ReLU(q_h . k) is this library's reading of the unprinted formula.
//
// Scoring: v_mfma_scale_f32_16x16x128_f8f6f4 with both operands E2M1 and the e8m0
// block exponents as the hardware scales: one lane carries 32 elements of one row
// together with that block's exponent, which is exactly the MXFP4 block of the
// cache, so a 128-dim key is one MFMA per 16 heads x 16 keys.  FP4 x FP4 products
// scaled by powers of two are exact in fp32, so every per-head dot is exact.
//
// Top-k: one 1024-thread workgroup per token holds the token's keys in registers
// (order-preserving uint32 transform), finds the exact k-th largest key with radix
// passes of 12, 12 and 8 bits over one LDS histogram (the later passes only when more
// than k rows are candidates), then compacts the winners in row order (ties at the
// threshold go to the lower row id), so the output is ascending.
#include <type_traits>
#include <utility>

#include "sad_internal.h"

namespace sad {
namespace {

// Compile-time loop: f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>).
template <typename F, int... J>
__device__ inline void static_for_impl(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ------------------------------------------------------------------ scoring

constexpr int kScoreThreads = 256;
constexpr int kRowsPerWave = 512;                                  // 32 groups of 16 rows
constexpr int kScoreChunk = kRowsPerWave * (kScoreThreads / 64);  // compressed rows per workgroup
// 16-row groups whose key loads are in flight together: small batches and short waves
// keep the registers low, so more waves per SIMD hide the random page reads
constexpr int kGroupBatch = 4;

typedef int gi32x4_t __attribute__((__vector_size__(4 * sizeof(int))));

// Buffer-resource flags word for raw (unformatted, unswizzled) loads on gfx9-family GPUs.
constexpr int kRawBufferFlags = 0x00020000;

struct IdxDesc {
  const uint8_t* pool;
  int64_t stride;
  int64_t num_pages;
  int block;
};

// Keys of one batch of row groups: lane (m = lane%16, grp = lane/16) holds 16 packed
// bytes (dims 32*grp .. +32) and the e8m0 exponent of row 16*u + m.
struct KeyBatch {
  gi32x4_t v[kGroupBatch];
  int e[kGroupBatch];
};

// One wave scores 512 consecutive compressed rows of one token, 4 groups of 16 rows at
// a time; the loads of the next batch are issued before the current one is scored.  The
// page ids of the wave's rows are loaded once up front (one per lane, at most 64 pages),
// with a wave mask of the ones that are pool pages.  BLOCK (rows per page, 16 or 64) is
// a template argument, so a row's page column is a shift.
template <int DIM, int BLOCK>
__global__ __launch_bounds__(kScoreThreads) void indexer_score_kernel(
    sad_batch b, const uint8_t* __restrict__ qv, const uint8_t* __restrict__ qs,
    const float* __restrict__ wts, int num_heads, IdxDesc kc, const int32_t* __restrict__ bt,
    int64_t bt_stride, int bt_cols, int ratio, float* __restrict__ logits, int64_t logits_stride,
    float* __restrict__ dbg, int64_t dbg_stride) {
  constexpr int VB = DIM / 2;    // packed value bytes per row
  constexpr int SB = DIM / 32;   // exponent bytes per row
  constexpr int LGB = BLOCK == 16 ? 4 : 6;
  static_assert(BLOCK == 16 || BLOCK == 64, "16 or 64 rows per page");
  static_assert(kRowsPerWave % BLOCK == 0, "every wave starts on a page boundary");
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int m = lane & 15;
  const int grp = lane >> 4;
  // A operands: 16 heads x 128 dims per tile; lane (m, grp) holds dims [32*grp, 32*grp+32)
  // of head 16*ht + m and that block's exponent.  They need only the token, so they are
  // loaded first, together with the token's request.
  gi32x4_t qa[4];
  int qsc[4];
  float wl[4][4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const int h = ht * 16 + m;
    qa[ht] = gi32x4_t{0, 0, 0, 0};
    qsc[ht] = 127;
    if (h < num_heads && grp < SB) {
      qa[ht] = *reinterpret_cast<const gi32x4_t*>(qv + ((int64_t)t * num_heads + h) * VB + 16 * grp);
      qsc[ht] = qs[((int64_t)t * num_heads + h) * SB + grp];
    }
    // this lane's outputs are heads 16*ht + 4*grp + j
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ho = ht * 16 + 4 * grp + j;
      wl[ht][j] = ho < num_heads ? wts[(int64_t)t * num_heads + ho] : 0.0f;
    }
  }
  const int req = uniform_ro_load(b.token_to_req + t);  // scalar load: not behind the Q loads
  if (req < 0 || req >= b.num_reqs || bt_cols <= 0) return;
  // Page ids of this wave's rows: lane i holds table column col0 + i (a 16-row group
  // never straddles a page, since 16 divides the page size).  The load needs only the
  // request, so it goes out with the loads of the token's length (column clamped into
  // the table; lanes past the wave's columns are cleared below).
  const int w_begin = blockIdx.x * kScoreChunk + wave * kRowsPerWave;
  const int32_t* bt_row = bt + (int64_t)req * bt_stride;
  const int col0 = w_begin >> LGB;
  const int pid_any = bt_row[min(col0 + lane, bt_cols - 1)];
  TokenGeom g;
  if (!token_geometry_uniform(b, t, ratio, g)) return;
  const int n_rows = min(g.n_comp, bt_cols * BLOCK);
  if (w_begin >= n_rows) return;  // no barriers in this kernel: waves may leave early
  const int w_rows = min(kRowsPerWave, n_rows - w_begin);
  const int n_groups = (w_rows + 15) / 16;
  const int ncol = ((w_begin + w_rows - 1) >> LGB) - col0 + 1;  // <= 64
  const int pid = lane < ncol ? pid_any : -1;
  const uint64_t pool_cols = __ballot(pid >= 0 && (int64_t)pid < kc.num_pages);  // bit i: column col0 + i
  // Issue the loads of the batch's groups as buffer loads: a wave-uniform resource per
  // page (zero records for an absent or unbacked group, so its loads return zeros and
  // touch no memory), the group's first row as the scalar offset and a per-lane
  // constant offset.  Every load goes out unconditionally.
  // (lanes past the key's dims, grp >= SB, read out of range: zeros)
  const uint32_t lane_voff = grp < SB ? (uint32_t)(m * VB + 16 * grp) : (1u << 30);
  const uint32_t lane_soff = grp < SB ? (uint32_t)(m * SB + grp) : (1u << 30);
  auto load = [&](int gb, KeyBatch& kb) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kGroupBatch; ++u) {
      // the wave starts on a page boundary, so the group's table column (minus col0)
      // and its first row in the page are constants
      const int ci = (16 * (gb + u)) >> LGB;
      const int r0 = (16 * (gb + u)) & (BLOCK - 1);
      const int page = __builtin_amdgcn_readlane(pid, ci);  // wave-uniform
      const bool page_ok = (pool_cols >> ci) & 1ull;
      const bool ok = gb + u < n_groups && page_ok;
      // the base depends on the page only (shared by its groups); a group past the
      // wave's rows gets zero records instead
      const uint8_t* pg = kc.pool + (int64_t)(page_ok ? page : 0) * kc.stride;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)pg, (short)0, ok ? (int)kc.stride : 0, kRawBufferFlags);
      kb.v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane_voff, r0 * VB, 0);
      kb.e[u] = __builtin_amdgcn_raw_buffer_load_b8(rs, lane_soff, BLOCK * VB + r0 * SB, 0);
    }
  };
  // this lane's first logit (lanes 0..15 store row w_begin + 16 g + lane of group g)
  float* lrow = logits + (int64_t)t * logits_stride + w_begin + lane;
  float* drow = dbg != nullptr ? dbg + (int64_t)t * dbg_stride + w_begin + lane : nullptr;
  // the ReLU's upper clamp, kept opaque so the clamp stays one med3 instruction
  float fmax_big = 3.402823466e+38f;
  asm volatile("" : "+s"(fmax_big));

  // Score the batch's groups from kb (absent groups are scored too, on the zero key;
  // only rows before the end are stored).  The MFMAs of group u+1 are issued before the
  // results of group u are combined.
  auto mma = [&](const KeyBatch& kb, int u, f32x4_t (&acc)[4]) __attribute__((always_inline)) {
    const i32x8_t kv = {kb.v[u][0], kb.v[u][1], kb.v[u][2], kb.v[u][3], 0, 0, 0, 0};
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const i32x8_t qv8 = {qa[ht][0], qa[ht][1], qa[ht][2], qa[ht][3], 0, 0, 0, 0};
      // format 4 = E2M1 for both operands; scales are e8m0 in byte 0
      acc[ht] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qv8, kv, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 4, 4,
                                                                 0, qsc[ht], 0, kb.e[u]);
      asm volatile("" : "+v"(acc[ht]));  // results in VGPRs: the combine reads them directly
    }
  };
  auto combine = [&](int gb, int u, const f32x4_t (&acc)[4]) __attribute__((always_inline)) {
    const bool ok = (pool_cols >> ((16 * (gb + u)) >> LGB)) & 1ull;
    float part = 0.0f;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int j = 0; j < 4; ++j)  // ReLU as one med3 (clamp to [0, FLT_MAX])
        part = __builtin_fmaf(wl[ht][j], __builtin_amdgcn_fmed3f(acc[ht][j], 0.0f, fmax_big), part);
    // lanes m, m+16, m+32, m+48 hold the 4 head groups of the group's row m: the row swaps of
    // v_permlane16_swap / v_permlane32_swap hand each lane the value of lane ^ 16, then
    // of lane ^ 32 (the same sums as two xor shuffles, without the LDS)
    const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(part), __float_as_uint(part), false, false);
    part = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
    const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
    part = __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
    if (lane < 16 && 16 * (gb + u) + lane < w_rows) {
      const float v = ok ? part : -INFINITY;
      lrow[16 * (gb + u)] = v;
      if (drow != nullptr) drow[16 * (gb + u)] = v;
    }
  };
  auto score = [&](int gb, const KeyBatch& kb) __attribute__((always_inline)) {
    f32x4_t acc[2][4];
    mma(kb, 0, acc[0]);
    static_for<kGroupBatch>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      if constexpr (u + 1 < kGroupBatch) mma(kb, u + 1, acc[(u + 1) & 1]);
      combine(gb, u, acc[u & 1]);
    });
  };

  // Straight-line schedule (so the memory waits are exact): the loads of batch b+1 are
  // in flight while batch b is scored.
  constexpr int kBatches = kRowsPerWave / 16 / kGroupBatch;
  KeyBatch kbuf[2];
  load(0, kbuf[0]);
  static_for<kBatches>([&](auto bc) {
    constexpr int bi = decltype(bc)::value;
    if constexpr (bi + 1 < kBatches) load((bi + 1) * kGroupBatch, kbuf[(bi + 1) & 1]);
    score(bi * kGroupBatch, kbuf[bi & 1]);
  });
}

// ------------------------------------------------------------------ top-k

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kDigitBins = 4096;  // radix digits of 12 bits (then 12, then 8)

__device__ inline uint32_t order_key(float f) {
  // -inf and NaN mark rows that are not candidates
  if (!(f > -INFINITY)) return 0u;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the workgroup (every thread calls it, all lanes active), in
// uint32 (sums wrap modulo 2^32); returns the exclusive prefix and writes the total to
// *total.  It holds one barrier:
// callers alternate between two `sh` buffers, so the reads of one scan are done before
// the next-but-one scan writes the same buffer (the scan between them has a barrier).
__device__ inline uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
  static_assert(kTopkWaves == 16, "the wave totals fill one 16-lane DPP row");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  // the wave totals, scanned within each 16-lane row (every row holds all 16)
  uint32_t w = sh[lane & 15];
  w += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, 0x111, 0xF, 0xF, false);  // row_shr:1
  w += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, 0x112, 0xF, 0xF, false);  // row_shr:2
  w += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, 0x114, 0xF, 0xF, false);  // row_shr:4
  w += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, 0x118, 0xF, 0xF, false);  // row_shr:8
  *total = (uint32_t)__builtin_amdgcn_readlane((int)w, 15);
  const uint32_t before = (uint32_t)__builtin_amdgcn_readlane((int)w, max(wave - 1, 0));
  return (wave == 0 ? 0u : before) + incl - v;
}

// The digit bin holding the kk-th largest counted key (1-based), scanning the bins
// from the top: returns it, the number of keys in higher bins (*above) and in the bin
// itself (*count), and the number of counted keys (*total).  Thread t owns bins 4095-4t .. 4092-4t; it clears
// them after reading, so the histogram is zero for the next pass (the barriers of the
// scan and of the pick order the clear before that pass's adds).
__device__ inline int select_bin(int* hist, int kk, uint32_t* sh, int* pick, int* above, int* count,
                                 int* total) {
  static_assert(kDigitBins == 4 * kTopkThreads, "four bins per thread");
  const int tid = threadIdx.x;
  int4* h4 = reinterpret_cast<int4*>(hist) + (kTopkThreads - 1 - tid);
  const int4 hv = *h4;
  *h4 = make_int4(0, 0, 0, 0);
  const int c[4] = {hv.w, hv.z, hv.y, hv.x};  // bins 4095-4t, 4094-4t, 4093-4t, 4092-4t
  uint32_t tot;
  const int a0 = (int)block_excl_scan((uint32_t)(c[0] + c[1] + c[2] + c[3]), sh, &tot);
  *total = (int)tot;
  const int a1 = a0 + c[0], a2 = a1 + c[1], a3 = a2 + c[2], a4 = a3 + c[3];
  if (a0 < kk && kk <= a4) {  // the one thread whose bins hold the kk-th key
    const int q = kk <= a1 ? 0 : kk <= a2 ? 1 : kk <= a3 ? 2 : 3;
    pick[0] = kDigitBins - 1 - (4 * tid + q);
    pick[1] = q == 0 ? a0 : q == 1 ? a1 : q == 2 ? a2 : a3;
    pick[2] = c[q];
  }
  __syncthreads();
  *above = pick[1];
  *count = pick[2];
  return pick[0];
}

// Index-build arguments of the fused path (build_sparse_indices on the top-k output).
struct BuildArgs {
  const int32_t* replay;
  const int32_t* swa_bt;
  int64_t swa_stride;
  int swa_cols;
  int swa_block;
  int64_t swa_pages;
  const int32_t* comp_bt;
  int64_t comp_stride;
  int comp_cols;
  int comp_block;
  int64_t comp_pages;
  int window;
  int padded;
  int32_t* si;
  int32_t* lens;
};

// Rows past one workgroup's reach (32 keys per thread) go through chunks: each chunk
// of kTopkChunk rows keeps its own top-k (value and row id, k slots per chunk, padded
// with -inf / -1), then one workgroup per token selects the top-k of those candidates.
// Every row of the token's top-k is in its chunk's top-k (fewer than k rows of the
// chunk precede it in the order value desc, row asc), and the candidates keep row
// order (chunks in order, each ascending), so the result equals the one-pass top-k.
constexpr int kTopkChunk = 32 * kTopkThreads;
struct ChunkIO {
  float* vals;    // [T][nch * k]
  int32_t* ids;   // [T][nch * k]
  int nch;
};
enum TopkMode { kDirect = 0, kDirectBuild = 1, kChunk = 2, kMerge = 3 };

// Mode kDirect: top-k of the token's first n_c logits.  kDirectBuild: the same, and the
// workgroup also writes the token's sparse_indices row and length, as
// build_sparse_indices would from this top-k row: window columns lo..p through the
// window table, then the winners' slots through the compressed table (ascending, the
// ones whose page is not in the pool dropped), then -1.  kChunk: chunk blockIdx.y of
// the logits -> its k candidates.  kMerge: the candidates -> the token's top-k.
template <int KPT, int MODE>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    sad_batch b, int ratio, int max_rows, const float* __restrict__ logits, int64_t logits_stride,
    int k, int32_t* __restrict__ out, BuildArgs ba, ChunkIO cio) {
  constexpr bool BUILD = MODE == kDirectBuild;
  // logits staged in row order (coalesced global loads), then read back thread-contiguous
  constexpr int kStride = KPT <= 16 ? KPT + 4 : KPT;  // padded rows: conflict-free 16-byte reads
  __shared__ __align__(16) float stage[kTopkThreads * kStride];
  __shared__ __align__(16) int hist[kDigitBins];
  __shared__ __align__(16) uint32_t scan_sh[2][kTopkWaves];
  __shared__ int pick[3];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int base = tid * KPT;  // the thread's rows after staging: base .. base + KPT - 1

  // The workspace row holds max_rows logits (a chunk: its part of them; the merge: the
  // token's nch * k candidates), so they are loaded before the token's length is known
  // (at an index clamped into the row: none is conditional); rows past n become -inf
  // below.  The token's geometry comes through scalar loads, which the wait for them
  // does not serialize behind the logits loads.
  const int chunk = MODE == kChunk ? (int)blockIdx.y : 0;
  const int row_off = chunk * kTopkChunk;
  const int span = MODE == kMerge ? cio.nch * k : max_rows - row_off;  // positions in the row
  const float* lrow = MODE == kMerge ? cio.vals + (int64_t)t * cio.nch * k
                                     : logits + (int64_t)t * logits_stride + row_off;
  float lv[KPT];
  if (span > 0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) lv[i] = lrow[min(i * kTopkThreads + tid, span - 1)];
  }
  TokenGeom g;
  const bool ok = token_geometry_uniform(b, t, ratio, g);
  const int n = MODE == kMerge ? span
                : MODE == kChunk ? (ok ? max(0, min(min(g.n_comp, max_rows) - row_off, kTopkChunk)) : 0)
                : (ok ? min(g.n_comp, max_rows) : 0);
  int32_t* orow = out + (int64_t)t * k;
  // chunk outputs: k candidate slots of this chunk
  float* cvals = MODE == kChunk ? cio.vals + ((int64_t)t * cio.nch + chunk) * k : nullptr;
  int32_t* cids = MODE == kChunk ? cio.ids + ((int64_t)t * cio.nch + chunk) * k : nullptr;

  // Index-build loads that need only the token, issued now and used at the end: the
  // compressed-table page ids of the thread's rows (its KPT consecutive rows lie in at
  // most two columns: the block size is a power of two >= 16), the replay bound, and
  // the window page of position lo0 + tid (lo0 = max(p - window + 1, 0) is a lower
  // bound of the window's first position).
  int pg0 = -1, pg1 = -1, replay = 0, lo0 = 0, win_slot = -1;
  int32_t* si_row = BUILD ? ba.si + (int64_t)t * (ba.window + ba.padded) : nullptr;
  const int32_t* swa_row = nullptr;
  if constexpr (BUILD) {
    if (n > 0 && ba.comp_cols > 0) {
      const int32_t* comp_row = ba.comp_bt + (int64_t)g.req * ba.comp_stride;
      const int c0 = base / ba.comp_block;
      pg0 = comp_row[min(c0, ba.comp_cols - 1)];
      pg1 = comp_row[min(c0 + 1, ba.comp_cols - 1)];
    }
    if (ok) {
      lo0 = max(g.pos - ba.window + 1, 0);
      if (ba.replay != nullptr) replay = uniform_ro_load(ba.replay + g.req);
      swa_row = ba.swa_bt + (int64_t)g.req * ba.swa_stride;
      if (tid < ba.window && lo0 + tid <= g.pos)
        win_slot = page_slot(swa_row, ba.swa_cols, ba.swa_block, ba.swa_pages, lo0 + tid);
    }
  }
  // Window columns: the slots of positions lo..p, lo = max(lo0, replay), then -1.
  // Position lo0 + j goes to column lo0 + j - lo.
  auto window_stores = [&]() __attribute__((always_inline)) {
    const int lo = max(lo0, replay);
    for (int j = tid; j < ba.window; j += kTopkThreads) {
      const int p0 = lo0 + j;
      int slot = win_slot;
      if (j >= kTopkThreads)
        slot = ok && p0 <= g.pos ? page_slot(swa_row, ba.swa_cols, ba.swa_block, ba.swa_pages, p0) : -1;
      if (ok && p0 >= lo && p0 <= g.pos) si_row[p0 - lo] = slot;
      if (j > g.pos - lo) si_row[j] = -1;  // columns past p - lo (all of them when !ok)
    }
  };

  if (n == 0) {
    if constexpr (MODE == kChunk) {
      for (int j = tid; j < k; j += kTopkThreads) {
        cvals[j] = -INFINITY;
        cids[j] = -1;
      }
      return;
    }
    for (int j = tid; j < k; j += kTopkThreads) orow[j] = -1;
    if constexpr (BUILD) {
      window_stores();
      for (int j = tid; j < ba.padded; j += kTopkThreads) si_row[ba.window + j] = -1;
      if (tid == 0) ba.lens[t] = 0;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int r = i * kTopkThreads + tid;  // row; thread r / KPT holds it
    stage[(r / KPT) * kStride + r % KPT] = r < n ? lv[i] : -INFINITY;
  }
  reinterpret_cast<int4*>(hist)[tid] = make_int4(0, 0, 0, 0);
  __syncthreads();
  uint32_t key[KPT];
#pragma unroll
  for (int i = 0; i < KPT; i += 4) {
    const float4 v = *reinterpret_cast<const float4*>(&stage[tid * kStride + i]);
    key[i + 0] = order_key(v.x);
    key[i + 1] = order_key(v.y);
    key[i + 2] = order_key(v.z);
    key[i + 3] = order_key(v.w);
  }

  // Pass 1: top 12 bits of every candidate key (this also counts the candidates).
  // Each select_bin leaves the histogram cleared for the next pass.
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (key[i] != 0u) atomicAdd(&hist[key[i] >> 20], 1);
  __syncthreads();
  int above, count, nvalid;
  const int d1 = select_bin(hist, k, scan_sh[0], pick, &above, &count, &nvalid);

  // Keys > thr are taken, plus `need` keys == thr in row order.  When every key of the
  // selected bin is taken, the threshold is just below the bin and the later passes are
  // skipped (the smallest candidate key, that of the most negative float, is in bin 8 of
  // the first digit, so thr stays above 0, the mark of the non-candidates).
  uint32_t thr = 0u;
  int need = 0;
  if (nvalid > k) {
    int kk = k - above;
    if (kk == count) {
      thr = ((uint32_t)d1 << 20) - 1u;
    } else {
      // Pass 2: next 12 bits of the keys in digit d1.
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        if ((int)(key[i] >> 20) == d1) atomicAdd(&hist[(key[i] >> 8) & 4095u], 1);
      __syncthreads();
      int dummy;
      const int d2 = select_bin(hist, kk, scan_sh[1], pick, &above, &count, &dummy);
      kk -= above;
      const uint32_t prefix = ((uint32_t)d1 << 20) | ((uint32_t)d2 << 8);
      if (kk == count) {
        thr = prefix - 1u;
      } else {
        // Pass 3: last 8 bits of the keys in digits (d1, d2).
#pragma unroll
        for (int i = 0; i < KPT; ++i)
          if ((key[i] >> 8) == (prefix >> 8)) atomicAdd(&hist[key[i] & 255u], 1);
        __syncthreads();
        const int d3 = select_bin(hist, kk, scan_sh[0], pick, &above, &count, &dummy);
        kk -= above;
        thr = prefix | (uint32_t)d3;
        need = kk;
      }
    }
  }
  const bool ties = thr != 0u;  // with thr == 0 every candidate is taken

  // One scan gives both the keys above the threshold and the keys equal to it in the
  // threads before this one (packed 16 + 16 bits; each count is at most 32768 and the
  // equal-key count below 65536, so no carry crosses).  Equal keys are taken in row
  // order, so min(equal before, need) of them precede this thread's winners.
  uint32_t gt_local = 0, eq_local = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    gt_local += key[i] > thr;
    eq_local += ties && key[i] == thr;
  }
  uint32_t packed_total;
  const uint32_t packed = block_excl_scan((gt_local << 16) | eq_local, scan_sh[1], &packed_total);
  const int eq_before = (int)(packed & 0xFFFFu);
  const int total = (int)(packed_total >> 16) + min((int)(packed_total & 0xFFFFu), need);
  int pos = (int)(packed >> 16) + min(eq_before, need);
  // The winners go to LDS in output order (the staging buffer is free since pass 1:
  // total <= n fits), then out as whole rows with coalesced stores.  The LDS stores
  // are unconditional, losers writing to a word of the histogram (no longer read), so
  // the loop has no branches.
  int32_t* ostage = reinterpret_cast<int32_t*>(stage);
  int32_t* trash = hist + tid;
  uint32_t sel_bits = 0;  // bit i: row base + i is a winner
  {
    int run = eq_before;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const bool eq = ties && key[i] == thr;
      const bool s = key[i] > thr || (eq && run < need);
      run += eq ? 1 : 0;
      *(s ? ostage + pos : trash) = base + i;
      pos += s ? 1 : 0;
      sel_bits |= (s ? 1u : 0u) << i;
    }
  }
  constexpr int kCap = kTopkThreads * kStride;  // words of the staging buffer
  if constexpr (MODE == kChunk) {
    __syncthreads();
    for (int j = tid; j < k; j += kTopkThreads) {
      const int v = ostage[min(j, kCap - 1)];
      cvals[j] = j < total ? lrow[v] : -INFINITY;
      cids[j] = j < total ? row_off + v : -1;
    }
  } else if constexpr (MODE == kMerge) {
    __syncthreads();
    const int32_t* crow = cio.ids + (int64_t)t * cio.nch * k;
    for (int j = tid; j < k; j += kTopkThreads) {
      const int v = ostage[min(j, kCap - 1)];
      orow[j] = j < total ? crow[v] : -1;
    }
  } else if constexpr (!BUILD) {
    __syncthreads();
    for (int j = tid; j < k; j += kTopkThreads) {
      const int v = ostage[min(j, kCap - 1)];
      orow[j] = j < total ? v : -1;
    }
  } else {
    // The winners' slots in row order; those whose compressed page is not in the pool
    // are dropped (fail closed), the rest packed left.  Rows base + i with i < split lie
    // in column c0, the others in column c0 + 1; slot = column's page * B + row % B.
    const int lg_b = 31 - __builtin_clz(ba.comp_block);
    const int c0 = base >> lg_b;
    const int split = ((c0 + 1) << lg_b) - base;  // >= 1
    const uint32_t in_first = split >= 32 ? 0xFFFFFFFFu : (1u << split) - 1u;
    const bool ok0 = c0 < ba.comp_cols && pg0 >= 0 && (int64_t)pg0 < ba.comp_pages;
    const bool ok1 = c0 + 1 < ba.comp_cols && pg1 >= 0 && (int64_t)pg1 < ba.comp_pages;
    const uint32_t vbits = sel_bits & ((ok0 ? in_first : 0u) | (ok1 ? ~in_first : 0u));
    const uint32_t d0 = ((uint32_t)pg0 << lg_b) - ((uint32_t)c0 << lg_b) + (uint32_t)base;
    const uint32_t d1s = ((uint32_t)pg1 << lg_b) - ((uint32_t)(c0 + 1) << lg_b) + (uint32_t)base;
    uint32_t vtotal_u;
    int vpos = (int)block_excl_scan((uint32_t)__builtin_popcount(vbits), scan_sh[0], &vtotal_u);  // also orders ostage
    const int vtotal = (int)vtotal_u;
    for (int j = tid; j < k; j += kTopkThreads) {
      const int v = ostage[min(j, kCap - 1)];
      orow[j] = j < total ? v : -1;
    }
    __syncthreads();  // the winners are read out before their slots overwrite them
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const bool v = (vbits >> i) & 1u;
      *(v ? ostage + vpos : trash) = (int)((i >= split ? d1s : d0) + (uint32_t)i);
      vpos += v ? 1 : 0;
    }
    __syncthreads();
    for (int j = tid; j < ba.padded; j += kTopkThreads) {
      const int v = ostage[min(j, kCap - 1)];
      si_row[ba.window + j] = j < vtotal ? v : -1;
    }
    if (tid == 0) ba.lens[t] = vtotal;
    window_stores();
  }
}

}  // namespace
}  // namespace sad

using namespace sad;

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Chunks of the top-k for rows past one workgroup's reach (1 when it needs none).
static int topk_chunks(int64_t max_rows) { return (int)((max_rows + kTopkChunk - 1) / kTopkChunk); }

extern "C" size_t indexer_score_topk_workspace_size(int32_t num_tokens, int32_t max_ctx_rows,
                                                    int32_t topk) {
  if (num_tokens <= 0 || max_ctx_rows <= 0) return 0;
  const size_t stride = (size_t)((max_ctx_rows + 3) / 4 * 4);
  size_t bytes = align256((size_t)num_tokens * stride * sizeof(float));
  const int nch = topk_chunks(max_ctx_rows);
  if (nch > 1 && topk > 0)  // the chunks' candidates: a value and a row id each
    bytes += 2 * align256((size_t)num_tokens * nch * topk * sizeof(float));
  return bytes;
}

namespace {

// Scoring + top-k (+ the index build when ba != nullptr; its arguments already checked).
int run_indexer(const sad_batch* batch, const uint8_t* q_values, const uint8_t* q_scales,
                const float* weights, int32_t num_idx_heads, const sad_mxfp4_cache* keys,
                const int32_t* idx_bt, int64_t idx_bt_stride, int32_t idx_bt_cols,
                int32_t compress_ratio, int32_t topk, int32_t* topk_local, float* logits_debug,
                int64_t logits_stride, void* workspace, size_t workspace_bytes, void* stream,
                const BuildArgs* ba) {
  SAD_CHECK(batch != nullptr && keys != nullptr, SAD_EINVAL, "indexer_score_topk: NULL batch/keys");
  const int T = batch->num_tokens;
  SAD_CHECK(T >= 0 && batch->num_reqs >= 0, SAD_EINVAL, "indexer_score_topk: negative sizes");
  SAD_CHECK(keys->dim == 64 || keys->dim == 128, SAD_EUNSUPPORTED,
            "indexer_score_topk: dim %d unsupported (64 or 128)", keys->dim);
  SAD_CHECK(keys->block_size == 16 || keys->block_size == 64, SAD_EUNSUPPORTED,
            "indexer_score_topk: block_size %d unsupported (16 or 64)", keys->block_size);
  SAD_CHECK(num_idx_heads >= 1 && num_idx_heads <= 64, SAD_EUNSUPPORTED,
            "indexer_score_topk: num_idx_heads %d unsupported (1..64)", num_idx_heads);
  SAD_CHECK(topk >= 1 && topk <= 65536, SAD_EINVAL, "indexer_score_topk: topk must be in [1, 65536]");
  SAD_CHECK(compress_ratio >= 1, SAD_EINVAL, "indexer_score_topk: compress_ratio must be >= 1");
  SAD_CHECK(idx_bt_cols >= 0 && idx_bt_stride >= idx_bt_cols, SAD_EINVAL,
            "indexer_score_topk: bad table shape");
  const int64_t need_stride = (int64_t)keys->block_size * (keys->dim / 2 + keys->dim / 32);
  SAD_CHECK(keys->page_stride >= need_stride && keys->page_stride % 16 == 0, SAD_EINVAL,
            "indexer_score_topk: page_stride must be a multiple of 16 and >= %lld",
            (long long)need_stride);
  SAD_CHECK(keys->num_pages >= 0, SAD_EINVAL, "indexer_score_topk: negative num_pages");
  const int64_t max_rows64 = (int64_t)idx_bt_cols * keys->block_size;
  SAD_CHECK(max_rows64 <= INT32_MAX / 2, SAD_EINVAL, "indexer_score_topk: idx_bt_cols*block_size too large");
  const int nch = topk_chunks(max_rows64);
  SAD_CHECK(nch <= 1 || (int64_t)nch * topk <= kTopkChunk, SAD_EUNSUPPORTED,
            "indexer_score_topk: %lld rows need %d chunks of the top-k, and %d x topk %d candidates "
            "exceed %d",
            (long long)max_rows64, nch, nch, topk, kTopkChunk);
  const int max_rows = (int)max_rows64;
  SAD_CHECK(logits_debug == nullptr || logits_stride >= max_rows, SAD_EINVAL,
            "indexer_score_topk: logits_stride must be >= idx_bt_cols*block_size");
  if (T == 0) return SAD_OK;
  SAD_CHECK(batch->query_start_loc && batch->seq_lens && batch->token_to_req, SAD_EINVAL,
            "indexer_score_topk: batch arrays must be non-NULL");
  SAD_CHECK(q_values && q_scales && weights && idx_bt && topk_local && keys->pool, SAD_EINVAL,
            "indexer_score_topk: NULL pointer argument");
  SAD_CHECK(((uintptr_t)q_values & 15) == 0 && ((uintptr_t)keys->pool & 15) == 0, SAD_EINVAL,
            "indexer_score_topk: q_values and the key pool must be 16-byte aligned");
  const size_t ws_need = indexer_score_topk_workspace_size(T, max_rows, topk);
  SAD_CHECK(workspace_bytes >= ws_need && (ws_need == 0 || workspace != nullptr), SAD_EWORKSPACE,
            "indexer_score_topk: workspace needs %zu bytes, got %zu", ws_need, workspace_bytes);
  SAD_CHECK(((uintptr_t)workspace & 15) == 0, SAD_EINVAL,
            "indexer_score_topk: workspace must be 16-byte aligned");
  const int64_t ws_stride = (max_rows + 3) / 4 * 4;
  float* logits = reinterpret_cast<float*>(workspace);
  IdxDesc kd{(const uint8_t*)keys->pool, keys->page_stride, keys->num_pages, keys->block_size};
  hipStream_t st = (hipStream_t)stream;
  if (max_rows > 0) {
    const dim3 grid((max_rows + kScoreChunk - 1) / kScoreChunk, T);
    auto score = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, grid, dim3(kScoreThreads), 0, st, *batch, q_values, q_scales, weights,
                         num_idx_heads, kd, idx_bt, idx_bt_stride, idx_bt_cols, compress_ratio, logits,
                         ws_stride, logits_debug, logits_stride);
    };
    if (keys->dim == 128)
      keys->block_size == 64 ? score(indexer_score_kernel<128, 64>) : score(indexer_score_kernel<128, 16>);
    else
      keys->block_size == 64 ? score(indexer_score_kernel<64, 64>) : score(indexer_score_kernel<64, 16>);
    int rc = check_launch("indexer_score_topk(score)");
    if (rc != SAD_OK) return rc;
  }
  const BuildArgs bargs = ba != nullptr ? *ba : BuildArgs{};
  if (nch <= 1) {
    auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3(T), dim3(kTopkThreads), 0, st, *batch, compress_ratio, max_rows,
                         logits, ws_stride, topk, topk_local, bargs, ChunkIO{});
    };
    if (max_rows <= 4 * kTopkThreads)
      ba != nullptr ? go(topk_kernel<4, kDirectBuild>) : go(topk_kernel<4, kDirect>);
    else if (max_rows <= 16 * kTopkThreads)
      ba != nullptr ? go(topk_kernel<16, kDirectBuild>) : go(topk_kernel<16, kDirect>);
    else
      ba != nullptr ? go(topk_kernel<32, kDirectBuild>) : go(topk_kernel<32, kDirect>);
    return check_launch("indexer_score_topk(topk)");
  }
  // chunks, then the merge of their candidates (then the index build, as its own call)
  uint8_t* cand = reinterpret_cast<uint8_t*>(workspace) + align256((size_t)T * ws_stride * sizeof(float));
  const ChunkIO cio{reinterpret_cast<float*>(cand),
                    reinterpret_cast<int32_t*>(cand + align256((size_t)T * nch * topk * sizeof(float))), nch};
  hipLaunchKernelGGL((topk_kernel<32, kChunk>), dim3(T, nch), dim3(kTopkThreads), 0, st, *batch, compress_ratio,
                     max_rows, logits, ws_stride, topk, topk_local, bargs, cio);
  int rc = check_launch("indexer_score_topk(topk chunks)");
  if (rc != SAD_OK) return rc;
  auto merge = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(T), dim3(kTopkThreads), 0, st, *batch, compress_ratio, max_rows, logits,
                       ws_stride, topk, topk_local, bargs, cio);
  };
  const int ncand = nch * topk;
  if (ncand <= 4 * kTopkThreads)
    merge(topk_kernel<4, kMerge>);
  else if (ncand <= 16 * kTopkThreads)
    merge(topk_kernel<16, kMerge>);
  else
    merge(topk_kernel<32, kMerge>);
  rc = check_launch("indexer_score_topk(topk merge)");
  if (rc != SAD_OK || ba == nullptr) return rc;
  return build_sparse_indices(batch, ba->replay, ba->swa_bt, ba->swa_stride, ba->swa_cols, ba->swa_block,
                              ba->swa_pages, ba->comp_bt, ba->comp_stride, ba->comp_cols, ba->comp_block,
                              ba->comp_pages, topk_local, topk, topk, ba->window, compress_ratio, ba->padded,
                              ba->si, ba->lens, stream);
}

}  // namespace

extern "C" int indexer_score_topk(const sad_batch* batch, const uint8_t* q_values,
                                  const uint8_t* q_scales, const float* weights,
                                  int32_t num_idx_heads, const sad_mxfp4_cache* keys,
                                  const int32_t* idx_bt, int64_t idx_bt_stride, int32_t idx_bt_cols,
                                  int32_t compress_ratio, int32_t topk, int32_t* topk_local,
                                  float* logits_debug, int64_t logits_stride, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  clear_error();
  return run_indexer(batch, q_values, q_scales, weights, num_idx_heads, keys, idx_bt, idx_bt_stride,
                     idx_bt_cols, compress_ratio, topk, topk_local, logits_debug, logits_stride,
                     workspace, workspace_bytes, stream, nullptr);
}

extern "C" int indexer_topk_sparse_indices(
    const sad_batch* batch, const uint8_t* q_values, const uint8_t* q_scales, const float* weights,
    int32_t num_idx_heads, const sad_mxfp4_cache* keys, const int32_t* idx_bt, int64_t idx_bt_stride,
    int32_t idx_bt_cols, int32_t compress_ratio, int32_t topk, int32_t* topk_local,
    const int32_t* replay_start, const int32_t* swa_bt, int64_t swa_bt_stride, int32_t swa_bt_cols,
    int32_t swa_block_size, int64_t swa_num_pages, const int32_t* comp_bt, int64_t comp_bt_stride,
    int32_t comp_bt_cols, int32_t comp_block_size, int64_t comp_num_pages, int32_t window_size,
    int32_t padded_topk, int32_t* sparse_indices, int32_t* sparse_topk_lens, void* workspace,
    size_t workspace_bytes, void* stream) {
  clear_error();
  const int rc = check_build_args("indexer_topk_sparse_indices", batch, swa_bt, swa_bt_stride,
                                  swa_bt_cols, swa_block_size, swa_num_pages, comp_bt, comp_bt_stride,
                                  comp_bt_cols, comp_block_size, comp_num_pages, true, topk, topk,
                                  window_size, compress_ratio, padded_topk, sparse_indices,
                                  sparse_topk_lens);
  if (rc != SAD_OK) return rc;
  SAD_CHECK(comp_block_size >= 16 && (comp_block_size & (comp_block_size - 1)) == 0, SAD_EUNSUPPORTED,
            "indexer_topk_sparse_indices: comp_block_size must be a power of two >= 16 (got %d)",
            comp_block_size);
  const BuildArgs ba{replay_start, swa_bt, swa_bt_stride, swa_bt_cols, swa_block_size, swa_num_pages,
                     comp_bt, comp_bt_stride, comp_bt_cols, comp_block_size, comp_num_pages,
                     window_size, padded_topk, sparse_indices, sparse_topk_lens};
  return run_indexer(batch, q_values, q_scales, weights, num_idx_heads, keys, idx_bt, idx_bt_stride,
                     idx_bt_cols, compress_ratio, topk, topk_local, nullptr, 0, workspace,
                     workspace_bytes, stream, &ba);
}
