// sparse_mla_decode: fused gather + FP8 dequant + MLA attention over sparse rows.
//
// [backend] forward_deepseek_v4_decode (FlashMLA sparse decode: window ids bounded by
// their lengths plus compressed ids bounded by extra_topk_length, FP8 cache,
// head_dim_v = head_dim, per-head attention sink); [model] DeepseekV4Attention
// (softmax scale head_dim^-1/2).  K and V are the same dequantized latent row.
//
// Work decomposition (gfx950, 64-lane waves, bf16 MFMA 32x32x16, fp32 accumulate):
//   * one workgroup = one token x one group of 64 heads x one split of the token's
//     attended columns, 4 waves (one per SIMD).  Wave w owns heads 32*(w/2) .. +32 of
//     the group and half of the latent dims (w%2): its Q^T fragments for those dims stay
//     in AGPRs, and its O^T accumulator for those output dims in AGPRs, for the whole
//     split.  The two waves of a head block add their partial S^T through LDS;
//   * the workgroups of one token's head groups are numbered 8 apart so they run on the
//     same XCD at the same time and the second read of each row hits that XCD's L2;
//   * columns are taken 32 at a time (a tile); wave w carries rows 8w..8w+7 of every
//     tile.  The raw cache bytes of tiles j+2 .. j+4 are in flight HBM -> LDS as direct
//     global-to-LDS loads of whole 128-byte lines (no VGPRs) while tile j is computed,
//     and the slot ids of a tile arrive the same way three steps before its rows;
//   * step j: (A) S^T = K Q^T on tile j's K tile; barrier.  (B) each wave stores its
//     rows of tile j+1, dequantized in registers during the previous step, into the
//     other K buffer (key-major, rows padded by one 16-byte chunk); both dim halves of
//     S^T summed, row maximum, weights; phase C's first LDS reads issued.  (C) O^T +=
//     V^T P^T, with V^T read from the same K tile through ds_read_b64_tr_b16 (no
//     transposed copy), while the wave's rows of tile j+2 (read from LDS in B) are
//     dequantized into registers (fp32 multiply by the row's block scale, bf16
//     rounding) and the loads of tile j+5 are issued between the MFMAs; barrier.  Each
//     MFMA slot's companions are fixed in source order;
//   * S^T puts one head per lane, so the online softmax needs only a swap with lane^32,
//     and the probabilities already sit in the B-operand layout of the PV MFMA;
//   * splits of one token write (o / l, log2-sum-exp) partials that a second kernel
//     merges, with the sink, when more than one split is used.
// Barriers are raw s_barrier with explicit LDS waits so that the in-flight LDS DMA of
// the next tiles is only waited for when a tile is consumed.
#include <math.h>

#include <algorithm>
#include <type_traits>
#include <utility>

#include "lds_dma.h"
#include "sad_internal.h"

namespace sad {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;              // attended columns per tile
constexpr int kRawSlots = 3;           // raw tiles in LDS: the one being dequantized + two in flight
constexpr float kRescaleSlack = 8.0f;  // keep the running max until exceeded by 2^8
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// s_waitcnt immediate (gfx9 encoding) waiting for lgkmcnt(0) only.
constexpr int kWaitLgkm0 = 0xC07F;

__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
}

// Source of the DMA for columns that are not attended: reading zeros makes their
// dequantized rows exactly zero with no masking in the dequant.
__device__ __align__(16) uint8_t kZeroRow[1024];

// Scheduling hint for a chain of N MFMAs that each consume R LDS reads: keep
// kLdsAhead reads in flight ahead of the chain, then one MFMA per R reads.
constexpr int kLdsAhead = 8;
template <int N, int R>
__device__ inline void sched_reads_ahead() {
  constexpr int kDsRead = 0x100, kMfma = 0x008;
  __builtin_amdgcn_sched_group_barrier(kDsRead, kLdsAhead, 0);
  constexpr int body = N - kLdsAhead / R;
#pragma unroll
  for (int i = 0; i < body; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMfma, kLdsAhead / R, 0);
}

// Compile-time loop: f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>).
template <typename F, int... J>
__device__ inline void static_for_impl(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}


typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

__device__ inline uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

template <int DN, int DR>
struct Shape {
  // Rows with fp32 scales and whole 128-byte fp8 lines (the pages' native 448 + 64 row
  // runs on the dim-split kernel).
  static constexpr int DQK = DN + DR;
  static constexpr int ROWB = DN + 2 * DR;  // value bytes per cached row
  static constexpr int NSC = DN / 64;       // scale blocks per row
  static constexpr int SCB = 4 * NSC;       // scale bytes per row
  static constexpr int MT = DQK / 32;       // PV MFMA m-tiles (output dims / 32)
  static constexpr int MT0 = (MT + 1) / 2;  // m-tiles of dim half 0 (half 1 gets the rest)
  static constexpr int MT1 = MT - MT0;
  static constexpr int KS0 = 2 * MT0;       // QK k-steps (16 dims) of dim half 0
  static constexpr int KS1 = 2 * MT1;
  static constexpr int KCH = DQK / 8 + 1;  // 16-byte chunks per K row in LDS (odd: one pad chunk)
  static constexpr int FP8_LINES = (DN + 127) / 128;  // 128-byte lines holding fp8 values
  static constexpr int FP8_TAIL = DN % 128 == 0 ? 8 : (DN % 128) / 16;  // fp8 chunks of the last one
  static constexpr int ROPE_CH = DR / 8;              // 16-byte bf16 chunks of the rope part
  // fp8 lines, then one line read from byte DN of the row: the rope part
  static constexpr int LINES = FP8_LINES + 1;
  static constexpr int DMA_PER_TILE = LINES + 1;  // value loads + one scale load per wave
  static constexpr int RAW_V = kWaves * LINES * 1024;  // [wave][line][row%8][chunk%8][16 B]
  static constexpr int RAW_S = kThreads;               // [row][32 bytes] of scales, padded
  static_assert(ROWB % 16 == 0 && DN % 64 == 0, "rows are whole chunks, fp8 part whole scale blocks");
  static_assert(128 * FP8_LINES <= ROWB, "every fp8 line lies inside the row");
  static_assert(ROPE_CH <= 8 && SCB <= 32, "rope part within one line, scales within 32 bytes");
  static_assert(kTile == 8 * kWaves, "each wave carries 8 rows of a tile");
  static_assert(DQK % 32 == 0, "output dims in 32-row MFMA tiles");
};

// Element offset of (key, dim) in the K tile.  Rows hold an odd number of 16-byte
// chunks (one pad chunk), so consecutive keys start 16 bytes apart modulo 128: the QK
// fragment reads (8 keys, same chunk) and the transposing PV reads (8 keys x 64 bytes)
// both spread over all LDS banks, and every fragment address is a per-lane base plus
// a compile-time offset.
template <int KCH>
__device__ inline int kt_off(int key, int dim) {
  return key * KCH * 8 + dim;
}

// Row values / scales of one attended column, or the zero row when the column is not
// attended (past ncols, slot -1, page outside the pool).  ONE: the window and the
// compressed columns read the same cache (wave-uniform descriptor).
template <bool ONE>
__device__ inline void slot_row(int slot, int col, int window, const KvDesc& swa, const KvDesc& comp, int rowb,
                                int scb, const uint8_t* zrow, const uint8_t** vals, const uint8_t** scales) {
  const KvDesc& kv = (ONE || col < window) ? swa : comp;
  // branch-free, so it can sit between other work without splitting it into blocks
  const bool ok = slot >= 0 && (slot >> kv.block_shift) < (int)kv.num_pages;  // num_pages * block fits in int32
  const int s2 = ok ? slot : 0;
  const int page = s2 >> kv.block_shift;
  const int ro = s2 & (kv.block - 1);
  const uint8_t* pg = kv.pool + (int64_t)page * kv.stride;
  const uint8_t* v = pg + ro * rowb;
  const uint8_t* sc = pg + (kv.block * rowb + ro * scb);
  asm("" : "+v"(v), "+v"(sc));  // computed on every lane (no branch around them)
  *vals = ok ? v : zrow;
  *scales = ok ? sc : zrow;
}

// Copy one tile's raw rows HBM -> LDS.  Wave w carries rows 8w..8w+7 of the tile:
// lane l handles row 8w + l/8 (address vrow/srow, from slot_row) and 16-byte chunk l%8 of
// each 128-byte line, so every load reads whole lines (8 rows x 128 contiguous bytes).
// Values land as [wave][line][row%8][chunk%8] (16 B each): the fp8 lines, then the rope
// part read from byte DN of the row; scales as [row][32 bytes].
// Every wave issues exactly DMA_PER_TILE loads with all lanes active (lanes past the
// row read the zero row into padding LDS), so a wave's vmcnt advances by a known
// amount per tile.  Returns the wave's 8-bit validity (bit r: row 8w + r attended).
template <int DN, int DR>
__device__ inline uint32_t dma_issue(int lane, int wave, uint8_t (&raw_v)[Shape<DN, DR>::RAW_V],
                                     float (&raw_s)[Shape<DN, DR>::RAW_S], const uint8_t* vrow,
                                     const uint8_t* srow, const uint8_t* zrow) {
  using S = Shape<DN, DR>;
  const int c = lane & 7;
  const uint32_t vbase = lds_addr(raw_v) + wave * S::LINES * 1024;
  const uint8_t* vsrc = vrow + 16 * c;
  static_for<S::LINES>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(vbase + j * 1024);
    if constexpr (j < S::FP8_LINES)
      dma_x4_off<128 * j>(vsrc, dst);  // inside the row (a half fp8 line reads rope bytes too)
    else if constexpr (S::ROPE_CH == 8)
      dma_x4_off<DN>(vsrc, dst);
    else
      dma_x4_off<0>(c < S::ROPE_CH ? vsrc + DN : zrow, dst);
  });
  dma_x1(c < S::SCB / 4 ? srow + 4 * c : zrow, __builtin_amdgcn_readfirstlane(lds_addr(raw_s) + wave * 256));
  // lane 8r carries row 8w + r: gather ballot bits 0, 8, .., 56 into one byte
  const uint64_t b = __ballot(vrow != zrow) & 0x0101010101010101ull;
  return (uint32_t)((b * 0x0102040810204080ull) >> 56);
}

// Load J of dma_issue on its own (J < LINES: value line J; J == LINES: the scales), so
// the loads of one tile can be spread between other work in the same order.
template <int DN, int DR, int J>
__device__ inline void dma_one(int lane, int wave, uint8_t (&raw_v)[Shape<DN, DR>::RAW_V],
                               float (&raw_s)[Shape<DN, DR>::RAW_S], const uint8_t* vrow, const uint8_t* srow,
                               const uint8_t* zrow) {
  using S = Shape<DN, DR>;
  const int c = lane & 7;
  if constexpr (J < S::LINES) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(raw_v) + wave * S::LINES * 1024 + J * 1024);
    if constexpr (J < S::FP8_LINES)
      dma_x4_off<128 * J>(vrow + 16 * c, dst);
    else if constexpr (S::ROPE_CH == 8)
      dma_x4_off<DN>(vrow + 16 * c, dst);
    else
      dma_x4_off<0>(c < S::ROPE_CH ? vrow + 16 * c + DN : zrow, dst);
  } else {
    dma_x1(c < S::SCB / 4 ? srow + 4 * c : zrow, __builtin_amdgcn_readfirstlane(lds_addr(raw_s) + wave * 256));
  }
}
__device__ inline uint32_t row_mask(const uint8_t* vrow, const uint8_t* zrow) {
  const uint64_t b = __ballot(vrow != zrow) & 0x0101010101010101ull;
  return (uint32_t)((b * 0x0102040810204080ull) >> 56);
}
template <int N>
__device__ inline void wait_lgkm() {
  asm volatile("s_waitcnt lgkmcnt(%0)" :: "n"(N) : "memory");
}

// Scale (fp32) of block `blk` of tile row `key` from the raw scale slot.
template <int DN, int DR>
__device__ inline float scale_at(const float (&raw_s)[Shape<DN, DR>::RAW_S], int key, int blk) {
  return raw_s[key * 8 + blk];
}

// Dequantize fp8 lines [J0, J1) (and the rope line when ROPE) of this wave's 8 rows of
// the raw tile into the padded bf16 K tile: fp8 elements become
// bf16_rne(float(e4m3) * scale), rope elements are copied.  Lane (row 8w + l/8, chunk
// l%8) converts 16 elements per line.  It reads only the wave's own DMA, so only this
// wave's vmcnt guards it.  All LDS reads are issued before the arithmetic.
template <int DN, int DR, int J0, int J1, bool ROPE>
__device__ inline void dequant_lines(int lane, int wave, const uint8_t (&raw_v)[Shape<DN, DR>::RAW_V],
                                     const float (&raw_s)[Shape<DN, DR>::RAW_S],
                                     uint16_t (&kt)[kTile * Shape<DN, DR>::KCH * 8]) {
  using S = Shape<DN, DR>;
  constexpr int NJ = J1 - J0;
  const int c = lane & 7;
  const int key = 8 * wave + (lane >> 3);
  const uint8_t* src = raw_v + wave * S::LINES * 1024 + (lane >> 3) * 128 + 16 * c;
  uint4 raw[NJ > 0 ? NJ : 1];
  float sc[NJ > 0 ? NJ : 1];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    raw[j] = *reinterpret_cast<const uint4*>(src + (J0 + j) * 1024);
    sc[j] = scale_at<DN, DR>(raw_s, key, 2 * (J0 + j) + (c >> 2));  // dims 128j + 16c .. +16: block 2j + c/4
  }
  uint4 rope = make_uint4(0u, 0u, 0u, 0u);
  if (ROPE && c < S::ROPE_CH) rope = *reinterpret_cast<const uint4*>(src + S::FP8_LINES * 1024);
  uint16_t* dst = kt + kt_off<S::KCH>(key, 16 * c);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const uint32_t wv[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
    uint32_t o[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[q], false) * sc[j];
      const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[q], true) * sc[j];
      o[2 * q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2_t));
      o[2 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2_t));
    }
    // the chunks of a half fp8 line past the fp8 part hold rope bytes: not stored
    if (J0 + j < S::FP8_LINES - 1 || c < S::FP8_TAIL) {
      *reinterpret_cast<uint4*>(dst + 128 * (J0 + j)) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4*>(dst + 128 * (J0 + j) + 8) = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
  if (ROPE && c < S::ROPE_CH) *reinterpret_cast<uint4*>(kt + kt_off<S::KCH>(key, DN + 8 * c)) = rope;
}

// This wave's 8 rows of one raw tile held in registers between their LDS reads and the
// store into a K tile: lane (row 8w + l/8, chunk l%8) keeps 16 fp8 values and their
// block scale per fp8 line, and one 16-byte chunk of the rope line (zero-row padding
// for chunks past the rope part).
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

template <int DN, int DR>
struct RawRows {
  u32x4_t v[Shape<DN, DR>::FP8_LINES];
  float sc[Shape<DN, DR>::FP8_LINES];
  u32x4_t rope;
};

template <int DN, int DR>
__device__ inline void raw_load(int lane, int wave, const uint8_t (&raw_v)[Shape<DN, DR>::RAW_V],
                                const float (&raw_s)[Shape<DN, DR>::RAW_S], RawRows<DN, DR>& r) {
  using S = Shape<DN, DR>;
  const int c = lane & 7;
  const int key = 8 * wave + (lane >> 3);
  const uint8_t* src = raw_v + wave * S::LINES * 1024 + (lane >> 3) * 128 + 16 * c;
#pragma unroll
  for (int j = 0; j < S::FP8_LINES; ++j) {
    r.v[j] = *reinterpret_cast<const u32x4_t*>(src + j * 1024);
    r.sc[j] = scale_at<DN, DR>(raw_s, key, 2 * j + (c >> 2));  // dims 128j + 16c .. +16: block 2j + c/4
  }
  r.rope = *reinterpret_cast<const u32x4_t*>(src + S::FP8_LINES * 1024);
}

// max(x of this lane, x of lane ^ 32): the two lane halves swapped in one VALU op.
__device__ inline float max_xor32(float x) {
  float a = x, b = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

template <int DN, int DR, bool ONE, bool LSE>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(1, 1)))
sparse_mla_kernel(const uint16_t* __restrict__ q, int num_tokens, int num_heads, KvDesc swa,
                  KvDesc comp, const int32_t* __restrict__ si, const int32_t* __restrict__ lens,
                  int window, int padded, float scale_log2, const float* __restrict__ sink,
                  uint16_t* __restrict__ out, float* __restrict__ lse_out,
                  float* __restrict__ part_o, float* __restrict__ part_lse, int num_splits,
                  int head_groups) {
  static_assert(DN % 128 == 0, "whole fp8 lines with fp32 scales (the native row runs on the dim-split kernel)");
  using S = Shape<DN, DR>;
  constexpr int DQK = S::DQK;
  constexpr int KSMAX = S::KS0;
  constexpr int MTMAX = S::MT0;
  constexpr int NV = S::DMA_PER_TILE;
  // Three raw slots (this wave's rows of tiles i+2, i+3 and i+4 arrive there) and two K
  // tiles (tile i, read by PV, and tile i+1, read by QK; tile i+2 is written into the
  // first one once every wave's PV is done with it).
  __shared__ __align__(16) uint8_t raw_v[kRawSlots][S::RAW_V];
  __shared__ __align__(16) float raw_s[kRawSlots][S::RAW_S];
  __shared__ __align__(16) uint16_t kt[2][kTile * S::KCH * 8];
  __shared__ uint32_t kt_mask[2];  // validity of the tile in each K buffer (bit j: column j)
  __shared__ int32_t ids_lds[4][kWaves][64];  // slot ids of tiles j+5 .. j+8 (lanes 0..7 of each wave)
  __shared__ __align__(16) float xbuf[kWaves * 64 * 16];  // [wave][q4][lane] float4: partial S

  // Block -> (token, split, head group): the head groups of one (token, split) are
  // 8 blocks apart, i.e. on the same XCD and dispatched together.
  const int L = blockIdx.x;
  const int grp = L / (8 * head_groups);
  const int off = L - grp * 8 * head_groups;
  const int pair = grp * 8 + (off & 7);
  const int hg = off >> 3;
  if (pair >= num_tokens * num_splits) return;
  const int t = pair / num_splits;
  const int split = pair - t * num_splits;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  __builtin_assume(wave >= 0 && wave < kWaves);
  const int n = lane & 31;    // head within the wave's block / key row within a fragment
  const int h = lane >> 5;    // lane half
  const int hb = wave >> 1;   // head block of this wave
  const int dh = wave & 1;    // dim half of this wave
  const int head = hg * 64 + hb * 32 + n;
  const bool block_active = hg * 64 + hb * 32 < num_heads;
  const int ks_n = dh == 0 ? S::KS0 : S::KS1;  // k-steps of this wave's dims
  const int mt_n = dh == 0 ? S::MT0 : S::MT1;  // m-tiles of this wave's dims
  const int dim0 = dh == 0 ? 0 : 32 * S::MT0;  // first dim of this wave's half
  // the zero row's address, kept opaque so it is not reloaded in the loop
  const uint8_t* zrow = kZeroRow;
  asm volatile("" : "+s"(zrow));

  const int width = window + padded;
  const int32_t* si_row = si + (int64_t)t * width;
  const int ncols = window + min(max(lens[t], 0), padded);
  const int ntiles = (ncols + kTile - 1) / kTile;
  const int per = (ntiles + num_splits - 1) / num_splits;
  const int tile_begin = split * per;
  const int tile_end = min(ntiles, tile_begin + per);
  const int col_end = min(ncols, tile_end * kTile);
  const uint16_t* qrow = q + ((int64_t)t * num_heads + min(head, num_heads - 1)) * DQK;

  // Q^T fragments: lane (head n, half h) holds dims dim0 + [16kk + 8h, 16kk + 8h + 8).
  bf16x8_t qf[KSMAX];
#pragma unroll
  for (int kk = 0; kk < KSMAX; ++kk) {
    qf[kk] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    // qrow is clamped to an existing head: the lanes of heads past num_heads load a copy
    // (their outputs are never written), so no load is conditional
    if (kk < ks_n) qf[kk] = *reinterpret_cast<const bf16x8_t*>(qrow + dim0 + 16 * kk + 8 * h);
  }
  f32x16_t acc_o[MTMAX];
#pragma unroll
  for (int mt = 0; mt < MTMAX; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[mt][r] = 0.0f;
  float m_run = -INFINITY;
  float l_run = 0.0f;  // sum of the bf16-rounded weights (normalizes O)
  float l_lse = 0.0f;  // sum of the fp32 weights (log-sum-exp)


  // Slot id of this lane's row (8*wave + lane/8) of a tile.  For the first five tiles the
  // wave's 8 ids are one scalar load (a window past the end of the sparse_indices row is
  // moved back inside it; the ids of such columns are unused).  Later tiles' ids arrive
  // three steps ahead as a direct global -> LDS load in the row DMAs' vmcnt stream, so
  // no scalar load is outstanding at a barrier's lgkmcnt wait.
  struct SlotIds {
    int v[8];  // sparse_indices[c .. c+8) of the wave's rows (c = lc, wave-uniform)
    int c0;    // first column of the wave's rows
    int lc;    // first column loaded
  };
  auto load_slots = [&](int tile) __attribute__((always_inline)) -> SlotIds {
    SlotIds ids;
    ids.c0 = tile * kTile + 8 * wave;  // wave-uniform
    if (width >= 8) {
      ids.lc = max(0, min(ids.c0, width - 8));
      const int32_t* p = si_row + ids.lc;
#pragma unroll
      for (int j = 0; j < 8; ++j) ids.v[j] = p[j];  // always inside the row; unused past col_end
    } else {  // a row of fewer than 8 ids: only the ids that exist are read
      ids.lc = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) ids.v[j] = j < width ? si_row[j] : -1;
    }
    return ids;
  };
  auto pick_slot = [&](const SlotIds& ids) __attribute__((always_inline)) -> int {
    // lanes 0..7 take the 8 ids, then every lane fetches its row's id with one shuffle
    int w8 = 0;
#define SAD_WRITELANE(j) asm("v_writelane_b32 %0, %1, " #j : "+v"(w8) : "s"(__builtin_amdgcn_readfirstlane(ids.v[j])))
    SAD_WRITELANE(0);
    SAD_WRITELANE(1);
    SAD_WRITELANE(2);
    SAD_WRITELANE(3);
    SAD_WRITELANE(4);
    SAD_WRITELANE(5);
    SAD_WRITELANE(6);
    SAD_WRITELANE(7);
#undef SAD_WRITELANE
    const int r = lane >> 3;
    const int idx = min(ids.c0 + r - ids.lc, 7);
    const int x = __builtin_amdgcn_ds_bpermute(idx << 2, w8);
    return ids.c0 + r < col_end ? x : -1;
  };
  auto row_addr_of = [&](int tile, int slot, const uint8_t** vrow, const uint8_t** srow)
      __attribute__((always_inline)) {
    slot_row<ONE>(slot, tile * kTile + 8 * wave + (lane >> 3), window, swa, comp, S::ROWB, S::SCB, zrow, vrow,
                  srow);
  };
  // ids of the wave's 8 rows of a tile -> the LDS ring (lanes 0..7; the others read the
  // zero row into the unused part of the wave's 256 bytes)
  auto id_fetch = [&](int tile) __attribute__((always_inline)) {
    const int col = tile * kTile + 8 * wave + lane;
    const void* src = lane < 8 && col < width ? static_cast<const void*>(si_row + col) : static_cast<const void*>(zrow);
    dma_x1(src, __builtin_amdgcn_readfirstlane(lds_addr(ids_lds[(tile - tile_begin) & 3][wave])));
  };
  auto slot_of = [&](int tile) __attribute__((always_inline)) -> int {
    const int r = lane >> 3;
    const int x = ids_lds[(tile - tile_begin) & 3][wave][r];
    return tile * kTile + 8 * wave + r < col_end ? x : -1;
  };
  // Wait until at most `after` tiles' DMAs issued after the awaited one are in flight.
  auto wait_tiles = [&](int after) __attribute__((always_inline)) {
    if (after >= 2)
      wait_vmem<2 * NV>();
    else if (after == 1)
      wait_vmem<NV>();
    else
      wait_vmem<0>();
  };
  RawRows<DN, DR> rr;             // this wave's raw rows of the tile being dequantized
  u32x4_t rope_keep;  // rope chunk of the tile whose K rows are stored in phase C
  u32x4_t dq[2 * S::FP8_LINES];  // ... and their fp8 part as bf16 (rope part: rr.rope)
  // One fp8 word of the raw rows (4 e4m3 values) -> 4 bf16 in dq: word w of line j holds
  // elements 16c + 4(w%4) .. +4 of that line.
  auto convert_word = [&](auto wc) __attribute__((always_inline)) {
    constexpr int w = decltype(wc)::value;
    constexpr int j = w >> 2;
    constexpr int qw = w & 3;
    const uint32_t word = rr.v[j][qw];
    const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false) * rr.sc[j];
    const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true) * rr.sc[j];
    dq[2 * j + (qw >> 1)][2 * (qw & 1)] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2_t));
    dq[2 * j + (qw >> 1)][2 * (qw & 1) + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2_t));
  };
  constexpr int NWORD = 4 * S::FP8_LINES;

  // Prologue: DMA of tiles 0, 1, 2 (raw slots 0, 1, 2); tile 0 dequantized into K buffer
  // 0 and tile 1 into registers; DMA of tiles 3 and 4 into slots 0 and 1.  Tile j uses
  // raw slot j % 3 and K buffer j % 2.  A wave's mask byte of a tile is kept from its DMA
  // until it writes it beside that tile's K buffer.
  uint32_t mask_a = 0, mask_b = 0, mask_c = 0, mask_d = 0;  // this wave's bytes for tiles j+1 .. j+4
  {
    // The slot ids of tiles 0..4 are all loaded and picked before the first row DMA, so
    // no id load waits behind a row DMA in the vmcnt stream.
    int sl[5];
    if (width >= 8) {
      SlotIds ids[5];
#pragma unroll
      for (int k = 0; k < 5; ++k) {
        ids[k].c0 = (tile_begin + k) * kTile + 8 * wave;
        ids[k].lc = max(0, min(ids[k].c0, width - 8));
#pragma unroll
        for (int j = 0; j < 8; ++j) ids[k].v[j] = si_row[ids[k].lc + j];
      }
#pragma unroll
      for (int k = 0; k < 5; ++k) sl[k] = pick_slot(ids[k]);
    } else {
#pragma unroll
      for (int k = 0; k < 5; ++k) sl[k] = pick_slot(load_slots(tile_begin + k));
    }
    // Q fragments landed together with the ids (a wait the compiler sees, so it does not
    // re-check the Q loads inside the tile loop); Q^T lives in AGPRs from here on (an
    // MFMA operand only), leaving the VGPRs for fragments in flight
    __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
    for (int kk = 0; kk < KSMAX; ++kk) asm volatile("" : "+a"(qf[kk]));
    auto dma_at = [&](int tile, int slot, int slot_index) __attribute__((always_inline)) -> uint32_t {
      const uint8_t* vr;
      const uint8_t* sr;
      row_addr_of(tile, slot, &vr, &sr);
      return dma_issue<DN, DR>(lane, wave, raw_v[slot_index], raw_s[slot_index], vr, sr, zrow);
    };
    id_fetch(tile_begin + 5);
    id_fetch(tile_begin + 6);
    id_fetch(tile_begin + 7);
    uint32_t m0 = 0;
    if (tile_begin < tile_end) m0 = dma_at(tile_begin, sl[0], 0);
    if (tile_begin + 1 < tile_end) mask_a = dma_at(tile_begin + 1, sl[1], 1);
    if (tile_begin + 2 < tile_end) mask_b = dma_at(tile_begin + 2, sl[2], 2);
    if (tile_begin < tile_end) {
      wait_tiles(min(2, tile_end - 1 - tile_begin));
      dequant_lines<DN, DR, 0, S::FP8_LINES, true>(lane, wave, raw_v[0], raw_s[0], kt[0]);
      if (lane == 0) reinterpret_cast<uint8_t*>(&kt_mask[0])[wave] = (uint8_t)m0;
    }
    wait_tiles(min(1, tile_end - 2 - tile_begin));
    raw_load<DN, DR>(lane, wave, raw_v[1], raw_s[1], rr);  // stale past the last tile (unused)
    static_for<NWORD>(convert_word);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // raw reads of slots 0 and 1 done before their refill
    if (tile_begin + 3 < tile_end) mask_c = dma_at(tile_begin + 3, sl[3], 0);
    if (tile_begin + 4 < tile_end) mask_d = dma_at(tile_begin + 4, sl[4], 1);
  }

  // Phase A of step j (after a barrier: K buffer b holds tile j, the other one is free):
  // S^T = K Q^T over this wave's dims on the MFMAs; the partial S^T is published for the
  // partner wave (same head block, other dim half); barrier.
  auto phase_a = [&](int b, f32x16_t& s) __attribute__((always_inline)) {
    int lane_s = lane;
    asm volatile("" : "+v"(lane_s));
    lds_barrier();
    const uint16_t* kbase = kt[b] + kt_off<S::KCH>(lane_s & 31, dim0 + 8 * (lane_s >> 5));
    bf16x8_t af[KSMAX];
    static_for<(kLdsAhead < KSMAX ? kLdsAhead : KSMAX)>([&](auto kc) {
      constexpr int kk = decltype(kc)::value;
      if (kk < ks_n) af[kk] = *reinterpret_cast<const bf16x8_t*>(kbase + 16 * kk);
    });
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.0f;
    __builtin_amdgcn_sched_barrier(0);
    static_for<KSMAX>([&](auto kc) {
      constexpr int kk = decltype(kc)::value;
      if (kk < ks_n) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk], qf[kk], s, 0, 0, 0);
      if constexpr (kk + kLdsAhead < KSMAX) {
        if (kk + kLdsAhead < ks_n) af[kk + kLdsAhead] = *reinterpret_cast<const bf16x8_t*>(kbase + 16 * (kk + kLdsAhead));
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    float4* xw = reinterpret_cast<float4*>(xbuf) + wave * 4 * 64 + lane_s;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) xw[64 * q4] = make_float4(s[4 * q4], s[4 * q4 + 1], s[4 * q4 + 2], s[4 * q4 + 3]);
    lds_barrier();
  };

  // Weights of one pair of this lane's S^T values (r, r+1) relative to the running
  // maximum, into the PV B operand; O is normalized by the sum of the same rounded
  // weights the PV MFMA multiplies with.
  float sv[16];       // this lane's S^T values of the current tile (both dim halves)
  float m_use = 0.0f;  // the maximum the weights are relative to (log2 domain)
  auto weight_pair = [&](auto rc, bf16x8_t (&pb)[2]) __attribute__((always_inline)) {
    constexpr int r = decltype(rc)::value;
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], scale_log2, -m_use));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r + 1], scale_log2, -m_use));
    const bf16x2_t w = __builtin_convertvector(f32x2_t{p0, p1}, bf16x2_t);
    pb[r >> 3][r & 7] = w[0];
    pb[r >> 3][(r & 7) + 1] = w[1];
    l_run = __builtin_amdgcn_fdot2_f32_bf16(w, bf16x2_t{(__bf16)1.0f, (__bf16)1.0f}, l_run, false);
    if (LSE) l_lse += p0 + p1;
  };

  // ---- Phase C's LDS reads, issued during phase B (which leaves LDS idle otherwise).
  //      The V^T fragment (lane: dim 32mt + lane%32, 8 keys) comes from the key-major
  //      tile through two transposing reads: in each 16-lane group, lane (a = i/4,
  //      b = i%4) points at key a of the 4-key set and dims 4b..4b+3, and lane j
  //      receives dim j of all 4 keys.  Read (mt, q4) covers keys 8*q4 + 4*(g/2) + ia of
  //      m-tile mt.  The PV MFMAs run keys 0..15 of every m-tile first (ks = 0), then
  //      keys 16..31: MFMA i = ks*MT + mt takes reads 2i and 2i+1 = (mt, 2ks) and
  //      (mt, 2ks+1), issued kLdsAhead reads earlier.
  constexpr int NREAD = 4 * MTMAX;
  s16x4_t vf[NREAD];
  int slot5 = -1;  // slot id of this lane's row of tile j+5
  auto v_base = [&](int b, int lane_s) __attribute__((always_inline)) -> const uint16_t* {
    const int g = lane_s >> 4;
    const int ia = (lane_s & 15) >> 2;
    const int ib = lane_s & 3;
    return kt[b] + kt_off<S::KCH>(4 * (g >> 1) + ia, dim0 + 16 * (g & 1) + 4 * ib);
  };
  auto vread = [&](auto jc, const uint16_t* vbase) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    constexpr int i = j >> 1;  // MFMA
    constexpr int mt = i % MTMAX;
    constexpr int q4 = 2 * (i / MTMAX) + (j & 1);
    if (mt < mt_n)
      vf[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(vbase + kt_off<S::KCH>(8 * q4, 32 * mt)));
  };
  // this wave's DMA of tile j+2 and the ids of tile j+5 landed, then the raw rows of
  // tile j+2, the slot ids of tile j+5 and the first V^T fragments of tile j
  auto c_reads = [&](int tile, int b, int rs2, int lane_s) __attribute__((always_inline)) {
    // From the second step on, every step issues the DMA of tile j+5 (zero rows past the
    // last tile) and the id load of tile j+8, so the loads issued after them are
    // counted exactly.
    const int k = tile - tile_begin;
    if (k >= 2) {
      wait_vmem<2 * NV + 2>();
    } else if (k == 1) {
      if (tile_begin + 4 < tile_end)
        wait_vmem<2 * NV + 1>();
      else
        wait_vmem<NV + 1>();
    } else {
      wait_tiles(min(2, tile_end - 3 - tile));
    }
    slot5 = slot_of(tile + 5);
    raw_load<DN, DR>(lane_s, wave, raw_v[rs2], raw_s[rs2], rr);
    const uint16_t* vbase = v_base(b, lane_s);
    static_for<(kLdsAhead < NREAD ? kLdsAhead : NREAD)>([&](auto jc) { vread(jc, vbase); });
  };

  // Phase B: both dim halves of S^T summed, unattended columns -inf, row maximum, lazy
  // rescale decision, phase C's first LDS reads, and the weights of keys 0..15 (pb[0];
  // keys 16..31 follow between the first PV MFMAs).  Returns whether any head of the
  // wave needs its O rescaled.
  auto phase_b = [&](int tile, int b, int rs2, const f32x16_t& s, bf16x8_t (&pb)[2], float& alpha)
                     __attribute__((always_inline)) -> bool {
    int lane_s = lane;
    asm volatile("" : "+v"(lane_s));
    const float4* xr = reinterpret_cast<const float4*>(xbuf) + (wave ^ 1) * 4 * 64 + lane_s;
    float4 ox[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) ox[q4] = xr[64 * q4];
    // this wave's mask byte of tile j+1 beside the other K buffer (its rows go there
    // during phase C)
    {
      if (lane_s == 0) reinterpret_cast<uint8_t*>(&kt_mask[b ^ 1])[wave] = (uint8_t)mask_a;
      mask_a = mask_b;
      mask_b = mask_c;
      mask_c = mask_d;
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 o = ox[q4];
      sv[4 * q4] = s[4 * q4] + o.x;
      sv[4 * q4 + 1] = s[4 * q4 + 1] + o.y;
      sv[4 * q4 + 2] = s[4 * q4 + 2] + o.z;
      sv[4 * q4 + 3] = s[4 * q4 + 3] + o.w;
    }
    const uint32_t vm = __builtin_amdgcn_readfirstlane(kt_mask[b]);
    if (vm != 0xFFFFFFFFu) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * (lane_s >> 5) + (r & 3);
        sv[r] = ((vm >> key) & 1u) ? sv[r] : -INFINITY;
      }
    }
    float tmax = sv[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, sv[r]);
    tmax = max_xor32(tmax) * scale_log2;
    // the running maximum is kept until a tile exceeds it by 2^slack (also true when it
    // is still -inf)
    const bool upd = tmax > m_run + kRescaleSlack;
    const float m_new = upd ? tmax : m_run;
    alpha = upd ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // exp2(-inf) = 0
    m_use = m_new == -INFINITY ? 0.0f : m_new;
    m_run = m_new;
    l_run *= alpha;
    if (LSE) l_lse *= alpha;
    rope_keep = rr.rope;
    c_reads(tile, b, rs2, lane_s);
    static_for<4>([&](auto pc) { weight_pair(std::integral_constant<int, 2 * decltype(pc)::value>{}, pb); });
    return __ballot(upd) != 0ull;
  };

  // Phase C: O^T += V^T P^T on tile j while this wave's rows of tile j+1 (dequantized in
  // registers during the previous step) are stored into the other K buffer, free since
  // the step began, each 16-byte chunk just before the words that overwrite its registers
  // with tile j+2 (read from its raw slot in phase B) are converted, and this wave's DMA
  // of tile j+5 into that raw slot is issued.
  auto phase_c = [&](int tile, int b, int rs2, bf16x8_t (&pb)[2]) __attribute__((always_inline)) {
    int lane_s = lane;
    asm volatile("" : "+v"(lane_s));
    // Between the PV MFMAs go the weights of keys 16..31 (before the first ks = 1
    // MFMA), the V^T reads kLdsAhead ahead, one 4-byte word of the raw rows at a time
    // dequantized, and the DMA loads of tile j+5.
    const uint16_t* vbase = v_base(b, lane_s);
    // slots of the DMA loads: every second slot, ending with the last one (a burst of
    // loads in consecutive slots stalled on a full memory pipeline), and the V^T reads
    // issued after the raw reads by then when both dim halves have the same m-tiles
    // (else 0: wait for all)
    constexpr int DSTEP = 2 * MTMAX - 1 - 2 * (NV - 1) >= 1 ? 2 : 1;
    constexpr int DSLOT0 = 2 * MTMAX - 1 - DSTEP * (NV - 1) >= 1 ? 2 * MTMAX - 1 - DSTEP * (NV - 1) : 1;
    static_assert(DSLOT0 + DSTEP * (NV - 1) < 2 * MTMAX, "every DMA load has a slot");
    constexpr int V_BEFORE = kLdsAhead + 2 * DSLOT0 < NREAD ? kLdsAhead + 2 * DSLOT0 : NREAD;
    constexpr int RAW_AFTER = S::MT0 == S::MT1 ? (V_BEFORE < 15 ? V_BEFORE : 15) : 0;
    const uint8_t* vr5 = zrow;
    const uint8_t* sr5 = zrow;
    __builtin_amdgcn_sched_barrier(0);
    static_for<2 * MTMAX>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int mt = i % MTMAX;
      constexpr int ks = i / MTMAX;
      if (mt < mt_n) {
        const bf16x8_t a = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(vf[2 * i], vf[2 * i + 1], 0, 1, 2, 3, 4, 5, 6, 7));
        acc_o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks], acc_o[mt], 0, 0, 0);
      }
      // pair p of keys 16..31 in slot min(p, MT-1): all before the first ks = 1 MFMA
      static_for<4>([&](auto pc) {
        constexpr int p = decltype(pc)::value;
        if constexpr ((p < MTMAX - 1 ? p : MTMAX - 1) == i) weight_pair(std::integral_constant<int, 8 + 2 * p>{}, pb);
      });
      if constexpr (2 * i + kLdsAhead < NREAD) {
        vread(std::integral_constant<int, 2 * i + kLdsAhead>{}, vbase);
        vread(std::integral_constant<int, 2 * i + kLdsAhead + 1>{}, vbase);
      }
      // word w in slot min(w, last): more words than MFMAs go to the last slot
      static_for<NWORD>([&](auto wc) {
        constexpr int w = decltype(wc)::value;
        constexpr int slot = w < 2 * MTMAX ? w : 2 * MTMAX - 1;
        if constexpr (slot == i) {
          if constexpr (w % 2 == 0) {
            constexpr int kk = w >> 1;
            const int key = 8 * wave + (lane_s >> 3);
            const int c = lane_s & 7;
            uint16_t* sdst = kt[b ^ 1] + kt_off<S::KCH>(key, 16 * c) + 128 * (kk >> 1) + 8 * (kk & 1);
            if ((kk >> 1) < S::FP8_LINES - 1 || S::FP8_TAIL == 8 || c < S::FP8_TAIL)
              *reinterpret_cast<u32x4_t*>(sdst) = dq[kk];
          }
          convert_word(wc);
        }
      });
      if constexpr (i == 0) {
        const int key = 8 * wave + (lane_s >> 3);
        const int c = lane_s & 7;
        if (c < S::ROPE_CH) *reinterpret_cast<u32x4_t*>(kt[b ^ 1] + kt_off<S::KCH>(key, DN + 8 * c)) = rope_keep;
      }
      // the DMA of tile j+5 into the raw slot just read, one load per second slot, so a stall
      // of the memory pipeline overlaps the MFMAs already issued
      if constexpr (i == DSLOT0 - 1) {
        row_addr_of(tile + 5, slot5, &vr5, &sr5);
        mask_d = row_mask(vr5, zrow);
      }
      if constexpr (i >= DSLOT0 && (i - DSLOT0) % DSTEP == 0 && (i - DSLOT0) / DSTEP < NV) {
        // this wave's reads of the raw slot are complete before its refill: at most
        // RAW_AFTER LDS reads issued after them are still outstanding
        if constexpr (i == DSLOT0) wait_lgkm<RAW_AFTER>();
        dma_one<DN, DR, (i - DSLOT0) / DSTEP>(lane_s, wave, raw_v[rs2], raw_s[rs2], vr5, sr5, zrow);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    id_fetch(tile + 8);
  };

  // Tile loop.  A step whose tile raises some head's running maximum leaves the inner
  // loop so that the (rare) rescale of O runs outside it and the O accumulators stay in
  // place across the steps of the inner loop.
  int tile = tile_begin;
  int rs2 = 2;  // raw slot of tile j+2
  for (;;) {
    f32x16_t s;
    bf16x8_t pb[2];
    float alpha = 1.0f;
    bool rescale = false;
    for (; tile < tile_end; ++tile, rs2 = rs2 == kRawSlots - 1 ? 0 : rs2 + 1) {
      const int b = (tile - tile_begin) & 1;
      phase_a(b, s);
      if (phase_b(tile, b, rs2, s, pb, alpha)) {
        rescale = true;
        break;
      }
      phase_c(tile, b, rs2, pb);
    }
    if (!rescale) break;
#pragma unroll
    for (int mt = 0; mt < MTMAX; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[mt][r] *= alpha;
    phase_c(tile, (tile - tile_begin) & 1, rs2, pb);
    ++tile;
    rs2 = rs2 == kRawSlots - 1 ? 0 : rs2 + 1;
  }
  // the direct-to-LDS loads issued past the last tile land before the workgroup ends
  wait_vmem<0>();

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float l_exp = LSE ? l_lse + __shfl_xor(l_lse, 32, 64) : l_tot;
  const bool lane_active = block_active && head < num_heads;
  // lane (n, h) holds O^T rows (dims) dim0 + 32mt + 8(r/4) + 4h + r%4 for head n
  if (num_splits == 1) {
    // O goes through LDS (the two K buffers: 64 head rows of DQK bf16 plus one 16-byte
    // chunk of padding, the K tiles' own row pitch) so that the workgroup's 64 heads,
    // which are contiguous in out, leave as one linear copy of whole lines.
    constexpr int RP = 2 * DQK + 16;  // bytes per staged head row
    static_assert(64 * RP <= (int)sizeof(kt), "the staged output fits the K buffers");
    uint8_t* ostage = reinterpret_cast<uint8_t*>(&kt[0][0]);
    lds_barrier();  // every wave's last PV reads of the K buffers are done
    if (lane_active) {
      const float s2 = sink != nullptr ? sink[head] * kLog2e : -INFINITY;
      const float mm = fmaxf(m_run, s2);
      const float mref = mm == -INFINITY ? 0.0f : mm;
      const float so = exp2f(m_run - mref);
      const float es = exp2f(s2 - mref);
      const float den = l_tot * so + es;
      const float den_lse = l_exp * so + es;
      const float f = den > 0.0f ? so / den : 0.0f;
      uint8_t* srow = ostage + (hb * 32 + n) * RP + 2 * dim0;
#pragma unroll
      for (int mt = 0; mt < MTMAX; ++mt)
        if (mt < mt_n) {
#pragma unroll
          for (int gg = 0; gg < 4; ++gg) {
            uint2 w;
            w.x = pack_bf16(acc_o[mt][4 * gg + 0] * f, acc_o[mt][4 * gg + 1] * f);
            w.y = pack_bf16(acc_o[mt][4 * gg + 2] * f, acc_o[mt][4 * gg + 3] * f);
            *reinterpret_cast<uint2*>(srow + 2 * (32 * mt + 8 * gg + 4 * h)) = w;
          }
        }
      if (lse_out != nullptr && h == 0 && dh == 0)
        lse_out[(int64_t)t * num_heads + head] = den_lse > 0.0f ? (mref + log2f(den_lse)) * kLn2 : -INFINITY;
    }
    lds_barrier();
    constexpr int CPR = DQK / 8;  // 16-byte chunks per head row
    const int rows = min(64, num_heads - hg * 64);
    uint8_t* obase = reinterpret_cast<uint8_t*>(out + ((int64_t)t * num_heads + hg * 64) * DQK);
    for (int i = tid; i < rows * CPR; i += kThreads) {
      const int r = i / CPR;
      *reinterpret_cast<uint4*>(obase + 16 * (int64_t)i) =
          *reinterpret_cast<const uint4*>(ostage + r * RP + 16 * (i - r * CPR));
    }
  } else {
    if (!lane_active) return;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    float* prow = part_o + (((int64_t)split * num_tokens + t) * num_heads + head) * DQK + dim0;
#pragma unroll
    for (int mt = 0; mt < MTMAX; ++mt)
      if (mt < mt_n) {
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const float4 w = make_float4(acc_o[mt][4 * gg + 0] * inv, acc_o[mt][4 * gg + 1] * inv,
                                       acc_o[mt][4 * gg + 2] * inv, acc_o[mt][4 * gg + 3] * inv);
          *reinterpret_cast<float4*>(prow + 32 * mt + 8 * gg + 4 * h) = w;
        }
      }
    if (h == 0 && dh == 0)
      part_lse[((int64_t)split * num_tokens + t) * num_heads + head] =
          l_exp > 0.0f ? m_run + log2f(l_exp) : -INFINITY;
  }
}

// Most column splits of one (token, head group): the combine stages the splits' weights
// in LDS.
constexpr int kMaxSplits = 256;

// Merge split partials: out = sum_s 2^(lse_s - M) o_s / (sum_s 2^(lse_s - M) + 2^(sink2 - M)).
template <int DQK>
__global__ __launch_bounds__(DQK) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse,
                                                      int num_splits, int T, int num_heads,
                                                      const float* __restrict__ sink,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ lse_out) {
  __shared__ float lse_s[kMaxSplits];
  const int head = blockIdx.x;
  const int t = blockIdx.y;
  const int d = threadIdx.x;
  const int64_t th = (int64_t)t * num_heads + head;
  const int64_t plane = (int64_t)T * num_heads;
  // the splits' log2-sum-exp values, one load per thread, then read from LDS
  for (int s = d; s < num_splits; s += DQK) lse_s[s] = part_lse[s * plane + th];
  __syncthreads();
  const float s2 = sink != nullptr ? sink[head] * kLog2e : -INFINITY;
  float mm = s2;
  for (int s = 0; s < num_splits; ++s) mm = fmaxf(mm, lse_s[s]);
  const float mref = mm == -INFINITY ? 0.0f : mm;
  float den = exp2f(s2 - mref);
  float acc = 0.0f;
  // unrolled so that several splits' loads are in flight at once
#pragma unroll 8
  for (int s = 0; s < num_splits; ++s) {
    const float w = exp2f(lse_s[s] - mref);
    den += w;
    acc += w * part_o[(s * plane + th) * DQK + d];
  }
  out[th * DQK + d] = f32_to_bf16_bits(den > 0.0f ? acc / den : 0.0f);
  if (lse_out != nullptr && d == 0)
    lse_out[th] = den > 0.0f ? (mref + log2f(den)) * kLn2 : -INFINITY;
}

int choose_splits(int T, int num_heads, int max_cols, int dqk) {
  const int cus = num_cus();
  const int units = T * ((num_heads + 63) / 64);  // workgroups without splitting
  if (units <= 0 || units >= cus) return 1;
  (void)dqk;
  const int tiles = (max_cols + kTile - 1) / kTile;
  // as many splits as keep one workgroup per compute unit, each with at least 4 tiles:
  // with fewer workgroups than compute units the extra partials' traffic costs less
  // than the idle units do
  int s = std::min(cus / units, tiles / 4);
  return std::max(1, std::min(s, kMaxSplits));
}

// Workspace bytes of `splits` column splits (0 without splitting): the partials o / l
// (fp32 [splits, T, H, dqk]) and log2-sum-exp (fp32 [splits, T, H]).
size_t split_workspace_bytes(int splits, int T, int H, int dqk) {
  if (splits <= 1) return 0;
  const size_t n = (size_t)splits * T * H;
  return (n * dqk + n) * sizeof(float);
}

template <int DN, int DR>
int launch(const uint16_t* q, int T, int H, const KvDesc& s, const KvDesc& c, const int32_t* si,
           const int32_t* lens, int W, int P, float scale, const float* sink, uint16_t* out,
           float* lse, void* ws, size_t ws_bytes, int splits, hipStream_t st) {
  using Sh = Shape<DN, DR>;
  float* part_o = nullptr;
  float* part_lse = nullptr;
  if (splits > 1) {
    const size_t po = (size_t)splits * T * H * Sh::DQK * sizeof(float);
    const size_t need = po + (size_t)splits * T * H * sizeof(float);
    SAD_CHECK(ws != nullptr && ws_bytes >= need, SAD_EWORKSPACE,
              "sparse_mla_decode: workspace needs %zu bytes, got %zu", need, ws_bytes);
    part_o = reinterpret_cast<float*>(ws);
    part_lse = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + po);
  }
  int rc;
  if constexpr (DN == 512 || DN == 448) {
    // the 512 + 64 row and the pages' native 448 + 64 row: the dim-split kernel
    rc = launch_mla_dsplit(q, T, H, s, c, si, lens, W, P, scale, sink, out, lse, part_o, part_lse, splits,
                           DN == 448, st);
  } else {
    const int head_groups = (H + 63) / 64;
    const int pairs = T * splits;
    const int blocks = (pairs + 7) / 8 * 8 * head_groups;
    // one cache for both segments (the usual case): wave-uniform row descriptors
    const bool one = s.pool == c.pool && s.stride == c.stride && s.num_pages == c.num_pages && s.block == c.block;
    // the fp32 sum of the weights is only kept for the log-sum-exp outputs
    const bool want_lse = lse != nullptr || splits > 1;
    auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3(blocks), dim3(kThreads), 0, st, q, T, H, s, c, si, lens, W, P,
                         scale * kLog2e, sink, out, lse, part_o, part_lse, splits, head_groups);
    };
    if (one)
      want_lse ? go(sparse_mla_kernel<DN, DR, true, true>) : go(sparse_mla_kernel<DN, DR, true, false>);
    else
      want_lse ? go(sparse_mla_kernel<DN, DR, false, true>) : go(sparse_mla_kernel<DN, DR, false, false>);
    rc = check_launch("sparse_mla_decode(attention)");
  }
  if (rc != SAD_OK || splits == 1) return rc;
  hipLaunchKernelGGL((combine_kernel<Sh::DQK>), dim3(H, T), dim3(Sh::DQK), 0, st, part_o, part_lse,
                     splits, T, H, sink, out, lse);
  return check_launch("sparse_mla_decode(combine)");
}

// The scratch buffer of sparse_mla_decode_noalloc: one per GPU the library runs on (each
// device holds its own copy of this array, at its own address, until the process ends).
constexpr size_t kNoAllocScratchBytes = 32ull << 20;
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// The device address of this device's copy of `scratch` (resolved once per device, with
// that device current; the array's name is only a host-side stand-in), or NULL.
void* noalloc_scratch() {
  static void* ptrs[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* p = __atomic_load_n(&ptrs[dev], __ATOMIC_ACQUIRE);
  if (p != nullptr) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  __atomic_store_n(&ptrs[dev], p, __ATOMIC_RELEASE);
  return p;
}

// Shared body of sparse_mla_decode and sparse_mla_decode_noalloc.  With static_ws the
// workspace is this device's copy of `scratch` (resolved only when splits need it) and
// the column splits are reduced until their partials fit in it.
int mla_decode_entry(const char* name, const uint16_t* q_bf16, int32_t num_tokens, int32_t num_heads,
                     const sad_kv_cache* swa, const sad_kv_cache* comp, const int32_t* sparse_indices,
                     const int32_t* sparse_topk_lens, int32_t window_size, int32_t padded_topk,
                     float softmax_scale, const float* attn_sink, uint16_t* out_bf16, float* lse,
                     void* workspace, size_t workspace_bytes, bool static_ws, void* stream) {
  clear_error();
  int rc = check_kv_cache(swa, "sparse_mla_decode(swa)");
  if (rc != SAD_OK) return rc;
  rc = check_kv_cache(comp, "sparse_mla_decode(comp)");
  if (rc != SAD_OK) return rc;
  SAD_CHECK(swa->d_nope == comp->d_nope && swa->d_rope == comp->d_rope &&
                swa->scale_format == comp->scale_format,
            SAD_EINVAL, "%s: swa and comp caches must share (d_nope, d_rope, scale_format)", name);
  SAD_CHECK(num_tokens >= 0 && window_size >= 0 && padded_topk >= 0, SAD_EINVAL, "%s: negative size", name);
  SAD_CHECK(num_heads >= 8 && num_heads <= 128 && num_heads % 8 == 0, SAD_EUNSUPPORTED,
            "%s: num_heads %d unsupported (multiple of 8, <= 128)", name, num_heads);
  SAD_CHECK(num_tokens < 65536, SAD_EINVAL, "%s: num_tokens must be < 65536", name);
  if (num_tokens == 0) return SAD_OK;
  SAD_CHECK(q_bf16 && (sparse_indices || window_size + padded_topk == 0) && sparse_topk_lens && out_bf16,
            SAD_EINVAL, "%s: NULL pointer argument", name);
  SAD_CHECK(((uintptr_t)q_bf16 & 15) == 0 && ((uintptr_t)out_bf16 & 15) == 0, SAD_EINVAL,
            "%s: q and out must be 16-byte aligned", name);
  SAD_CHECK(((uintptr_t)workspace & 15) == 0, SAD_EINVAL, "%s: workspace must be 16-byte aligned", name);
  const int dqk = swa->d_nope + swa->d_rope;
  int splits = choose_splits(num_tokens, num_heads, window_size + padded_topk, dqk);
  if (static_ws) {
    while (splits > 1 && split_workspace_bytes(splits, num_tokens, num_heads, dqk) > kNoAllocScratchBytes)
      --splits;
    workspace = nullptr;
    workspace_bytes = 0;
    if (splits > 1) {
      workspace = noalloc_scratch();
      SAD_CHECK(workspace != nullptr, SAD_ELAUNCH, "%s: the static scratch has no device address", name);
      workspace_bytes = kNoAllocScratchBytes;
    }
  }
  const size_t need = split_workspace_bytes(splits, num_tokens, num_heads, dqk);
  SAD_CHECK(need == 0 || (workspace != nullptr && workspace_bytes >= need), SAD_EWORKSPACE,
            "%s: workspace needs %zu bytes, got %zu", name, need, workspace_bytes);
  KvDesc s{(const uint8_t*)swa->pool, swa->page_stride, swa->num_pages, swa->block_size,
           __builtin_ctz(swa->block_size)};
  KvDesc c{(const uint8_t*)comp->pool, comp->page_stride, comp->num_pages, comp->block_size,
           __builtin_ctz(comp->block_size)};
  hipStream_t st = (hipStream_t)stream;
  if (swa->d_nope == 512)
    return launch<512, 64>(q_bf16, num_tokens, num_heads, s, c, sparse_indices, sparse_topk_lens,
                           window_size, padded_topk, softmax_scale, attn_sink, out_bf16, lse,
                           workspace, workspace_bytes, splits, st);
  if (swa->d_nope == 448)
    return launch<448, 64>(q_bf16, num_tokens, num_heads, s, c, sparse_indices, sparse_topk_lens,
                           window_size, padded_topk, softmax_scale, attn_sink, out_bf16, lse,
                           workspace, workspace_bytes, splits, st);
  return launch<128, 32>(q_bf16, num_tokens, num_heads, s, c, sparse_indices, sparse_topk_lens,
                         window_size, padded_topk, softmax_scale, attn_sink, out_bf16, lse,
                         workspace, workspace_bytes, splits, st);
}

}  // namespace
}  // namespace sad

using namespace sad;

extern "C" size_t sparse_mla_decode_workspace_size(int32_t num_tokens, int32_t num_heads,
                                                   int32_t max_row_width, int32_t dv) {
  if (num_tokens <= 0 || num_heads <= 0 || max_row_width <= 0 || dv <= 0) return 0;
  return split_workspace_bytes(choose_splits(num_tokens, num_heads, max_row_width, dv), num_tokens, num_heads,
                               dv);
}

extern "C" int sparse_mla_decode(const uint16_t* q_bf16, int32_t num_tokens, int32_t num_heads,
                                 const sad_kv_cache* swa, const sad_kv_cache* comp,
                                 const int32_t* sparse_indices, const int32_t* sparse_topk_lens,
                                 int32_t window_size, int32_t padded_topk, float softmax_scale,
                                 const float* attn_sink, uint16_t* out_bf16, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return mla_decode_entry("sparse_mla_decode", q_bf16, num_tokens, num_heads, swa, comp, sparse_indices,
                          sparse_topk_lens, window_size, padded_topk, softmax_scale, attn_sink, out_bf16, lse,
                          workspace, workspace_bytes, false, stream);
}

extern "C" int sparse_mla_decode_noalloc(const uint16_t* q_bf16, int32_t num_tokens, int32_t num_heads,
                                         const sad_kv_cache* swa, const sad_kv_cache* comp,
                                         const int32_t* sparse_indices, const int32_t* sparse_topk_lens,
                                         int32_t window_size, int32_t padded_topk, float softmax_scale,
                                         const float* attn_sink, uint16_t* out_bf16, float* lse,
                                         void* stream) {
  return mla_decode_entry("sparse_mla_decode_noalloc", q_bf16, num_tokens, num_heads, swa, comp,
                          sparse_indices, sparse_topk_lens, window_size, padded_topk, softmax_scale, attn_sink,
                          out_bf16, lse, nullptr, 0, true, stream);
}
