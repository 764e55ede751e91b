// sparse_mla_decode for the 512 fp8 + 64 bf16 latent row with fp32 block scales, and
// for the pages' native 448 fp8 + 64 bf16 row with ue8m0 scales: the dim-split kernel.
//
// [backend] forward_deepseek_v4_decode (FlashMLA sparse decode: window ids bounded by
// their lengths plus compressed ids bounded by extra_topk_length, FP8 cache,
// head_dim_v = head_dim, per-head attention sink); [model] DeepseekV4Attention
// (softmax scale head_dim^-1/2).  K and V are the same dequantized latent row.
//
// Work decomposition (gfx950, 64-lane waves, one wave per SIMD):
//   * one workgroup = one token x one group of 64 heads x one split of the token's
//     attended columns.  Wave w owns a 144-dim slice of the 576 latent dims for all 64
//     heads: nope dims 128w .. 128w+127 and rope dims 512+16w .. 512+16w+15.  Its Q^T
//     fragments for that slice (72 registers) and its O^T accumulator (144) stay in
//     AGPRs for the whole split;
//   * per tile of 32 attended columns, every wave's slice of each row (64 fp8 bytes and
//     8 rope values per lane, and the scale of those 64 bytes) comes from HBM into an LDS
//     ring by direct global -> LDS loads two steps ahead; the wave reads its own bytes
//     back and dequantizes them in registers into the A operand of the QK MFMA
//     (v_mfma_f32_32x32x16_bf16), so no K fragment is read from a shared tile.  The same
//     registers are stored once into the wave's own K tile, from which the transposing
//     LDS read (ds_read_b64_tr_b16) gives the V^T operand of the PV MFMA
//     (v_mfma_f32_16x16x32_bf16);
//   * each wave's partial S^T (its 144 dims) goes to LDS; wave w adds the four partials
//     of heads 16w .. 16w+15 and runs their online softmax; the bf16 weights go back
//     through LDS to every wave for PV.  Two barriers per tile;
//   * software pipeline (step j): phase 1 runs the QK MFMAs of tile j+1 with the dequant
//     of tile j+2 and, one by one, the row loads of tile j+4 between them; phase 2 runs
//     the PV MFMAs of tile j with the softmax of tile j+1 between them.  The weights, their
//     rescale factors and the K tiles are double-buffered so that the two phases of one
//     step never wait on each other's data;
//   * the two head groups of one (token, split) are numbered 8 workgroups apart, so
//     they run on the same XCD at the same time and the second read of each row hits
//     that XCD's L2;
//   * the native 448 + 64 row keeps the same slices, with nope dims 448..511 (wave 3's
//     lane half 1) as zeros: those lanes load the zero row and a zero Q fragment, and
//     their output dims are not written; its power-of-two scales dequantize with the
//     scaled conversion instruction.
// LDS layouts keep every store and read of the loop free of bank conflicts (with 32 or
// 64 banks): a K tile row is 288 bytes and the two 16-byte halves of each of its
// 32-byte blocks are swapped in the rows with fb(key) = 1 (fb below); the lane groups
// of the transposing read take their keys in the order that pairs rows 4 apart modulo
// 8 in each pass.
#include <math.h>

#include <type_traits>
#include <utility>

#include "lds_dma.h"
#include "sad_internal.h"

namespace sad {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;                  // attended columns per tile
constexpr int DN = 512, DR = 64, DQK = DN + DR;
constexpr int SCB = 4 * DN / 64;           // scale bytes per cached row (8 fp32)
constexpr int KS = 9;                      // QK k-steps (16 dims) of a wave's slice
constexpr int MT = 9;                      // PV m-tiles (16 dims) of a wave's slice
constexpr int NRAW = 2;                    // raw tiles in the LDS ring (tiles j+2 and j+3)
constexpr int KPITCH = 2 * (DQK / kWaves);  // bytes per key row of a wave's K tile (288)
constexpr int KT_WAVE = kTile * KPITCH;    // one wave's K tile
constexpr int KT_BUF = kWaves * KT_WAVE;   // one K buffer (all waves)
constexpr int XB_OFF = 2 * KT_BUF;         // partial S^T exchange
constexpr int XB_BYTES = kWaves * 2 * 4 * 64 * 16;
constexpr int PB_OFF = XB_OFF + XB_BYTES;  // bf16 weights exchange
constexpr int PB_BYTES = 4 * 64 * 16;       // one buffer (two: the weights of tiles j and j+1)
constexpr int MISC_OFF = PB_OFF + 2 * PB_BYTES;  // per-head rescale factors, flags, final factors
constexpr int MISC_BYTES = 2 * 64 * 4 + 2 * 16 + 64 * 4 + 64 * 4;
// raw ring: per slot and wave, the four 1 KB chunks of nope bytes, 1 KB of rope values
// and 256 bytes of scales, each in lane order (lane i's 16 or 4 bytes at 16i or 4i)
constexpr int RAW_OFF = (MISC_OFF + MISC_BYTES + 255) / 256 * 256;
constexpr int RAW_WAVE = 4 * 1024 + 1024 + 256;
constexpr int RAW_SLOT = kWaves * RAW_WAVE;
// slot-id ring: per slot and wave, the 32 ids of a tile (twice: lanes 32..63 repeat them)
constexpr int IDS_OFF = RAW_OFF + NRAW * RAW_SLOT;
constexpr int IDS_SLOT = kWaves * 256;
constexpr int LDS_BYTES = IDS_OFF + 2 * IDS_SLOT;
constexpr int OPITCH = 2 * DQK + 16;       // bytes per staged output head row
constexpr float kRescaleSlack = 8.0f;      // keep the running max until exceeded by 2^8
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
static_assert(64 * OPITCH <= XB_OFF + XB_BYTES, "the staged output fits the K and exchange buffers");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// Source of the loads of columns that are not attended: their rows dequantize to zero
// and their logits are masked.
__device__ __align__(16) uint8_t kZeroRow[1024];

template <typename F, int... J>
__device__ inline void static_for_impl(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Instruction classes of the scheduler's group barriers
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedDsRead = 0x100;
#define SCHED_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// A load through the global address space (a plain pointer to a row or to the zero row
// would compile to a flat load, which also counts against lgkmcnt and so would be
// drained by every barrier's LDS wait).
template <typename T>
__device__ inline T gload(const uint8_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(1))) T*>(
      (const __attribute__((address_space(1))) uint8_t*)p);
}

template <typename T>
__device__ inline T* lds_ptr(uint8_t* base, int off) {
  return reinterpret_cast<T*>(base + off);
}

__device__ inline uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// bf16_rne(float(e4m3) * scale) of the 4 fp8 values in `word` -> 2 words of bf16 pairs.
__device__ inline void dequant_word(uint32_t word, float sc, uint32_t& lo, uint32_t& hi) {
  const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false) * sc;
  const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true) * sc;
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf16x2_t));
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(b, bf16x2_t));
}

// max over the four 16-lane rows holding the same head
__device__ inline float max_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float sum_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <bool ONE, bool LSE, bool NAT>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
mla_dsplit_kernel(const uint16_t* __restrict__ q, int num_tokens, int num_heads, KvDesc swa, KvDesc comp,
                  const int32_t* __restrict__ si, const int32_t* __restrict__ lens, int window, int padded,
                  float scale_log2, const float* __restrict__ sink, uint16_t* __restrict__ out,
                  float* __restrict__ lse_out, float* __restrict__ part_o, float* __restrict__ part_lse,
                  int num_splits, int head_groups) {
  __shared__ __align__(16) uint8_t smem[LDS_BYTES];

  // Block -> (token, split, head group): the head groups of one (token, split) are 8
  // blocks apart, i.e. on the same XCD and dispatched together.
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
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(w >= 0 && w < kWaves);
  const int key = lane & 31;  // load / QK role: the tile row of this lane
  const int hf = lane >> 5;   // lane half: nope bytes 64hf.., rope values 8hf.. of the slice
  // The cached record: 512 fp8 + 64 bf16 with 8 fp32 scales, or (NAT) the pages' native
  // 448 fp8 + 64 bf16 with 8 ue8m0 bytes (7 used).  The slices keep the 576-dim layout
  // either way; in the native form nope dims 448..511 (wave 3's lane half 1) are zero.
  constexpr int R_NOPE = NAT ? 448 : DN;  // fp8 bytes of a row, and its rope's offset
  constexpr int R_ROWB = R_NOPE + 2 * DR;  // value bytes per row
  constexpr int R_SCB = NAT ? 8 : SCB;     // scale bytes per row
  constexpr int IO_D = R_NOPE + DR;        // dims of a q and of an out row
  const bool pad_lane = NAT && w == 3 && hf == 1;
  const int c16 = lane & 15;  // softmax / PV role: head (within 16) ...
  const int g = lane >> 4;    // ... and lane group (which 8 keys of the tile)
  // keys of the lane group's k-slots: slot 4r + a <-> key 8g + 4(r ^ (g & 1)) + a (the
  // transposing read of r = 0 and r = 1 then covers 8 rows with distinct row % 8 in each
  // of its passes over two lane groups)
  const int kq0 = 8 * g + 4 * (g & 1);        // keys of slots 0..3
  const int kq1 = 8 * g + 4 * (1 - (g & 1));  // keys of slots 4..7

  const int width = window + padded;
  const int32_t* si_row = si + (int64_t)t * width;
  const int ncols = window + min(max(lens[t], 0), padded);
  const int ntiles = (ncols + kTile - 1) / kTile;
  const int per = (ntiles + num_splits - 1) / num_splits;
  const int tile_begin = min(ntiles, split * per);
  const int tile_end = min(ntiles, tile_begin + per);
  const int col_end = min(ncols, tile_end * kTile);

  const uint8_t* zrow = kZeroRow;
  asm volatile("" : "+s"(zrow));

  // the slot ids of the first four tiles, requested before Q: the rows they name go out
  // (in the prologue) while Q is still in flight
  const int b0 = tile_begin;
  const bool any_tile = b0 < tile_end;
  int id0[4] = {0, 0, 0, 0};
  if (any_tile) {
#pragma unroll
    for (int k = 0; k < 4; ++k) id0[k] = si_row[min((b0 + k) * kTile + key, width - 1)];
  }

  // ---- Q^T fragments of this wave's slice: B operand of the 32x32x16 MFMA, lane (head
  // n = key, half hf) holds 8 dims of k-step s: nope 128w + 64hf + 8s (s < 8), rope
  // 512 + 16w + 8hf (s = 8) of the 576-dim layout (q's rope starts at R_NOPE).  Heads
  // past num_heads load a copy of the last head (their outputs are not written), so
  // every load is unconditional; the native form's padding dims load dim 0 and are zeroed.
  bf16x8_t qf[2][KS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int head = min(hg * 64 + 32 * nt + key, num_heads - 1);
    const uint16_t* qrow = q + ((int64_t)t * num_heads + head) * IO_D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int d = s < 8 ? (pad_lane ? 0 : 128 * w + 64 * hf + 8 * s) : R_NOPE + 16 * w + 8 * hf;
      const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qrow + d);
      qf[nt][s] = s < 8 && pad_lane ? bf16x8_t{} : v;
    }
  }

  // ---- row addressing and the LDS rings.  Every vector-memory operation of the tile
  // loop is a direct global -> LDS load issued here, so vmcnt counts exactly these:
  // per step the six row loads of one tile, then the slot ids of a later tile.
  const uint32_t lds_w = __builtin_amdgcn_readfirstlane(lds_addr(smem) + w * RAW_WAVE);
  const uint32_t ids_w = __builtin_amdgcn_readfirstlane(lds_addr(smem) + IDS_OFF + w * 256);
  const uint8_t* raw_w = smem + RAW_OFF + w * RAW_WAVE;
  const int32_t* ids_lds = reinterpret_cast<const int32_t*>(smem + IDS_OFF + w * 256);
  auto id_src = [&](int tile) __attribute__((always_inline)) -> const int32_t* {
    const int col = tile * kTile + key;
    return si_row + min(col, width - 1);  // in the row; columns past col_end are masked
  };
  // slot ids of `tile` -> id slot b (lane i: the id of key i % 32)
  auto issue_ids = [&](int tile, int b) __attribute__((always_inline)) {
    dma_x1(id_src(tile), ids_w + b * IDS_SLOT);
  };
  auto read_id = [&](int b) __attribute__((always_inline)) -> int { return ids_lds[b * (IDS_SLOT / 4) + lane]; };
  struct RowAddr {
    const uint8_t* vrow;
    const uint8_t* srow;
  };
  // the row and scale addresses of this lane's key in `tile` (slot id `id`); the tile's
  // validity mask in *mask (bit k: key k)
  auto row_addr = [&](int tile, int id, uint32_t* mask) __attribute__((always_inline)) -> RowAddr {
    const int col = tile * kTile + key;
    const bool inside = col < col_end;
    const bool is_swa = ONE || col < window;
    // two caches: the per-lane choice between the descriptors is made here, from SGPR
    // copies pinned at this point (else per-lane copies of both descriptors are hoisted
    // out of the tile loop and spilled)
    KvDesc sw = swa, cp = comp;
    if (!ONE) {
      asm volatile("" : "+s"(sw.pool), "+s"(sw.stride), "+s"(sw.num_pages), "+s"(sw.block), "+s"(sw.block_shift));
      asm volatile("" : "+s"(cp.pool), "+s"(cp.stride), "+s"(cp.num_pages), "+s"(cp.block), "+s"(cp.block_shift));
    } else if (LSE) {
      asm volatile("" : "+s"(sw.pool));
    }
    const uint8_t* pool = is_swa ? sw.pool : cp.pool;
    const int64_t stride = is_swa ? sw.stride : cp.stride;
    const int64_t npages = is_swa ? sw.num_pages : cp.num_pages;
    const int blk = is_swa ? sw.block : cp.block;
    const int shift = is_swa ? sw.block_shift : cp.block_shift;
    const int slot = inside ? id : -1;
    const bool ok = slot >= 0 && (int64_t)(slot >> shift) < npages;
    const int s2 = ok ? slot : 0;
    const int page = s2 >> shift;
    const int ro = s2 & (blk - 1);
    const uint8_t* pg = pool + (int64_t)page * stride;
    *mask = (uint32_t)__ballot(ok);
    return RowAddr{ok ? pg + ro * R_ROWB : zrow, ok ? pg + (blk * R_ROWB + ro * R_SCB) : zrow};
  };
  // load i (0..5) of a tile's rows into raw slot b
  auto issue_load = [&](const RowAddr& ra, int i, int b) __attribute__((always_inline)) {
    const uint32_t dst = lds_w + RAW_OFF + b * RAW_SLOT;
    const uint8_t* vn = pad_lane ? zrow : ra.vrow + 128 * w + 64 * hf;
    if (i == 0) dma_x4_off<0>(vn, dst);
    if (i == 1) dma_x4_off<16>(vn, dst + 1024);
    if (i == 2) dma_x4_off<32>(vn, dst + 2048);
    if (i == 3) dma_x4_off<48>(vn, dst + 3072);
    if (i == 4) dma_x4_off<0>(ra.vrow + R_NOPE + 32 * w + 16 * hf, dst + 4096);
    // the scale of nope block 2w + hf: its fp32 word, or (native) the word holding its byte
    if (i == 5) dma_x1(NAT ? (pad_lane ? zrow : ra.srow + 4 * (w >> 1)) : ra.srow + 8 * w + 4 * hf, dst + 5120);
  };
  // all six loads of `tile` into raw slot b; returns the tile's validity mask
  auto issue_raw = [&](int tile, int id, int b) __attribute__((always_inline)) -> uint32_t {
    uint32_t m;
    const RowAddr ra = row_addr(tile, id, &m);
#pragma unroll
    for (int i = 0; i < 6; ++i) issue_load(ra, i, b);
    return m;
  };
  constexpr int kLoadsPerStep = 6 + 1;  // row loads of one tile + one tile's slot ids

  // ---- dequant: raw slot b -> the QK A operand (k-step s: 8 nope values 8s .. of the
  // lane half's 64, k-step 8: its 8 rope values); each lane reads back its own bytes
  bf16x8_t kf[2][KS];  // two tiles: the one the QK reads and the one being dequantized
  struct RawRegs {
    u32x4_t v[4];
    u32x4_t rope;
    float sc;
  };
  auto read_raw = [&](int b, RawRegs& x) __attribute__((always_inline)) {
    const uint8_t* r = raw_w + b * RAW_SLOT;
#pragma unroll
    for (int i = 0; i < 4; ++i) x.v[i] = *reinterpret_cast<const u32x4_t*>(r + 1024 * i + 16 * lane);
    x.rope = *reinterpret_cast<const u32x4_t*>(r + 4096 + 16 * lane);
    x.sc = *reinterpret_cast<const float*>(r + 5120 + 4 * lane);
    if (NAT) {  // ue8m0 byte b -> the fp32 2^(b - 127) (b = 0: the denormal 2^-127)
      const uint32_t b = (__float_as_uint(x.sc) >> (8 * (2 * (w & 1) + hf))) & 255u;
      x.sc = __uint_as_float(b != 0 ? b << 23 : 0x00400000u);
    }
  };
  // one k-step (s < 8: nope values 8s..; s = 8: the rope values).  The native form's
  // power-of-two scales take the scaled conversion (v_cvt_scalef32_pk_bf16_fp8): the
  // multiply and the bf16 rounding in one instruction per pair, with the same result as
  // bf16_rne(float(e4m3) * 2^(b - 127)) for every code and scale byte 0 .. 254.  (Byte
  // 255, which the pages' writer never produces and ue8m0 reserves for NaN, decodes as
  // NaN here instead of inf; a row holding it makes the output non-finite either way.)
  auto dequant_ks = [&](const RawRegs& x, bf16x8_t (&k)[KS], int s) __attribute__((always_inline)) {
    if (s < 8) {
      uint32_t o[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t word = x.v[s >> 1][2 * (s & 1) + h];
        if (NAT) {
          o[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, x.sc, false));
          o[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, x.sc, true));
        } else {
          dequant_word(word, x.sc, o[2 * h], o[2 * h + 1]);
        }
      }
      k[s] = __builtin_bit_cast(bf16x8_t, u32x4_t{o[0], o[1], o[2], o[3]});
    } else {
      k[8] = __builtin_bit_cast(bf16x8_t, x.rope);
    }
  };
  auto dequant_regs = [&](const RawRegs& x, bf16x8_t (&k)[KS]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < KS; ++s) dequant_ks(x, k, s);
  };
  auto dequant = [&](int b, bf16x8_t (&k)[KS]) __attribute__((always_inline)) {
    RawRegs x;
    read_raw(b, x);
    dequant_regs(x, k);
  };

  // ---- LDS regions
  uint8_t* kt0 = smem + w * KT_WAVE;          // this wave's K tile, buffer 0 (+KT_BUF: buffer 1)
  uint8_t* xb = smem + XB_OFF;
  uint8_t* pb = smem + PB_OFF;
  float* alpha_lds = lds_ptr<float>(smem, MISC_OFF);          // [2][64] rescale factors
  uint32_t* flags = lds_ptr<uint32_t>(smem, MISC_OFF + 512);  // [2][4]: byte w of [b][0]: wave w rescaled
  float* fin_lds = lds_ptr<float>(smem, MISC_OFF + 544);      // [64] final factors
  float* lse_lds = lds_ptr<float>(smem, MISC_OFF + 800);      // [64] log2-sum-exp

  // Row key of a K tile keeps its 32-byte blocks with the 16-byte halves swapped when
  // fb(key) = 1: rows k and k+8 (and k and k+4 within 8) then fill different halves of
  // the banks in each pass of the stores, which all write one 16-byte chunk of 16 (or 8)
  // consecutive rows.
  auto fb = [](int k) __attribute__((always_inline)) -> int { return ((k >> 2) ^ (k >> 3)) & 1; };
  // store this lane's K operand into K buffer b (row `key`, the lane half's bytes: nope
  // chunks 8hf + s are the halves s%2 of blocks 4hf + s/2, the rope chunk the half hf of
  // block 8)
  const int fbk = fb(key);
  const int st_e = key * KPITCH + 128 * hf + 16 * fbk;        // even chunks
  const int st_o = key * KPITCH + 128 * hf + 16 * (1 - fbk);  // odd chunks
  const int st_r = key * KPITCH + 256 + 16 * (hf ^ fbk);      // rope chunk
  auto store_k = [&](int b, const bf16x8_t (&k)[KS]) __attribute__((always_inline)) {
    uint8_t* kt = kt0 + b * KT_BUF;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      *reinterpret_cast<bf16x8_t*>(kt + ((s & 1) ? st_o : st_e) + 32 * (s >> 1)) = k[s];
    *reinterpret_cast<bf16x8_t*>(kt + st_r) = k[8];
  };

  // ---- QK: S^T[nt] (32 keys x 32 heads) over the wave's slice
  f32x16_t sacc[2];
  auto qk = [&](const bf16x8_t (&k)[KS]) __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[nt][r] = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[s], qf[0][s], sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[s], qf[1][s], sacc[1], 0, 0, 0);
    }
  };
  // partial S^T -> LDS as [wave][nt][reg group j][lane][4 floats]: reg group j of lane
  // (head col, half h') holds keys 8j + 4h' + 0..3, which the lane group g = j of the
  // owner wave reads
  auto store_s = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x4_t* dst = reinterpret_cast<f32x4_t*>(xb) + ((w * 2 + nt) * 4) * 64 + lane;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dst[j * 64] = f32x4_t{sacc[nt][4 * j], sacc[nt][4 * j + 1], sacc[nt][4 * j + 2], sacc[nt][4 * j + 3]};
    }
  };

  // ---- online softmax of heads 16w .. 16w+15 (lane: head 16w + c16, 8 keys of group g)
  // the lane's partial S^T chunks: reg group g of source lane col + 32(g & 1) (keys kq0..)
  // and of lane col + 32(1 - (g & 1)) (keys kq1..), nt = w / 2, col = 16(w % 2) + c16
  const int sr_off = ((w >> 1) * 4 + g) * 64 + 16 * (w & 1) + c16 + 32 * (g & 1);
  float m_run = -INFINITY;
  float l_run = 0.0f;  // sum of the bf16-rounded weights the PV MFMA multiplies with
  float l_lse = 0.0f;  // sum of the fp32 weights (log-sum-exp)
  // the four partials of this lane's 8 keys, summed (k-slot order: slots 0..3 are keys
  // kq0 + 0..3, slots 4..7 keys kq1 + 0..3)
  auto s_read = [&](f32x4_t (&pa)[kWaves], f32x4_t (&pb2)[kWaves]) __attribute__((always_inline)) {
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(xb) + sr_off;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      pa[v] = src[v * 2 * 4 * 64];
      pb2[v] = src[v * 2 * 4 * 64 + 32 - 64 * (g & 1)];
    }
  };
  auto s_sum = [&](const f32x4_t (&pa)[kWaves], const f32x4_t (&pb2)[kWaves], float (&sv)[8])
      __attribute__((always_inline)) {
    f32x4_t a = pa[0], b = pb2[0];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) {
      a += pa[v];
      b += pb2[v];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = a[i];
      sv[4 + i] = b[i];
    }
  };
  auto s_reduce = [&](float (&sv)[8]) __attribute__((always_inline)) {
    f32x4_t pa[kWaves], pb2[kWaves];
    s_read(pa, pb2);
    s_sum(pa, pb2, sv);
  };
  // unattended columns of the tile (bit k of vm clear) -> -inf
  auto s_mask = [&](float (&sv)[8], uint32_t vm) __attribute__((always_inline)) {
    const uint32_t m0 = vm >> kq0, m1 = vm >> kq1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = ((m0 >> i) & 1u) ? sv[i] : -INFINITY;
      sv[4 + i] = ((m1 >> i) & 1u) ? sv[4 + i] : -INFINITY;
    }
  };
  auto softmax = [&](const float (&sv)[8], int b) __attribute__((always_inline)) {
    float tmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    tmax = max_rows(tmax) * scale_log2;
    // the running maximum is kept until a tile exceeds it by 2^slack (also true while it
    // is -inf); O needs rescaling only when it already holds weights (a finite maximum)
    const bool upd = tmax > m_run + kRescaleSlack;
    const bool resc = upd && m_run != -INFINITY;
    const float m_new = upd ? tmax : m_run;
    const float alpha = resc ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    m_run = m_new;
    l_run *= alpha;
    if (LSE) l_lse *= alpha;
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], scale_log2, -m_use));
    // (scalars, not elements of a vector: a bit_cast of a vector element compiled to the
    // first element every time)
    uint32_t pw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2_t w2 = __builtin_convertvector(f32x2_t{p[2 * i], p[2 * i + 1]}, bf16x2_t);
      pw[i] = __builtin_bit_cast(uint32_t, w2);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(w2, bf16x2_t{(__bf16)1.0f, (__bf16)1.0f}, l_run, false);
    }
    if (LSE) {
#pragma unroll
      for (int i = 0; i < 8; ++i) l_lse += p[i];
    }
    reinterpret_cast<u32x4_t*>(pb + b * PB_BYTES)[w * 64 + lane] = u32x4_t{pw[0], pw[1], pw[2], pw[3]};
    // every lane stores (the four lanes of a head store the same value): no branch
    const bool any = __ballot(resc) != 0ull;
    alpha_lds[64 * b + 16 * w + c16] = alpha;
    reinterpret_cast<uint8_t*>(flags + b)[w] = any ? 1 : 0;
  };

  // ---- PV: O^T (144 dims x 64 heads) += V^T P^T; tile (m, n): lane (c16, g) holds head
  // 16n + c16, dims 16m + 4g .. +3 of the slice
  f32x4_t acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // per-lane V^T read offsets within a K tile: lane (g, 4a + b) of read r reads row
  // kq_r + a, the 8-byte piece b of each 32-byte block m (halves swapped as stored)
  const int ka = (lane & 15) >> 2;
  const int kb = lane & 3;
  const int vrd0 = (kq0 + ka) * KPITCH + 8 * (kb ^ (2 * fb(kq0 + ka)));
  const int vrd1 = (kq1 + ka) * KPITCH + 8 * (kb ^ (2 * fb(kq1 + ka)));
  // the PV operands of K buffer b: P^T fragments of the four head tiles and the V^T
  // fragments of the nine dim tiles
  auto pv_read = [&](int b, bf16x8_t (&pf)[4], bf16x8_t (&vf)[MT]) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < 4; ++n) pf[n] = reinterpret_cast<const bf16x8_t*>(pb + b * PB_BYTES)[n * 64 + lane];
    const uint8_t* kt = kt0 + b * KT_BUF;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
      const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kt + vrd0 + 32 * m));
      const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kt + vrd1 + 32 * m));
      vf[m] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto pv_mma = [&](const bf16x8_t (&pf)[4], const bf16x8_t (&vf)[MT]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[m], pf[n], acc[m][n], 0, 0, 0);
  };
  // The O^T accumulators live in AGPRs (MFMA accumulators only): the rare rescale reads,
  // multiplies and writes each of them back explicitly, so that no other code needs them
  // in VGPRs.
  auto rescale = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const float al = alpha_lds[64 * b + 16 * n + c16];
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m][n] *= al;
    }
  };
  // (no instruction is scheduled across it: the phases' instruction mixes stay as
  // interleaved above)
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: the state every step starts from (step j, R = (j - b0) % 2):
  //   K buffer R holds tile j, P buffer R its weights (their rescale factor in slot R);
  //   kf[R ^ 1] holds tile j+1 dequantized; in flight, in this order: the rows of tile
  //   j+2 (raw slot R), the ids of j+4 (id slot R), the rows of j+3, the ids of j+5.
  uint32_t mask_ring[NRAW];  // validity of the tile in each raw slot
  uint32_t mask_cur = 0;   // scratch: validity of tile j+2 while step j runs
  uint32_t mask_prev = 0;  // validity of tile j+1 (the tile of step j's softmax)
  // The Q and id loads are the only loads the compiler tracks.  The rows of the first two
  // tiles go out as soon as the ids are in (the compiler waits for those), with Q still in
  // flight; then everything lands (vmcnt(0)) before the tile loop, so none of the
  // compiler's own waits ever counts a direct load after that.
  if (any_tile) {
    mask_ring[0] = issue_raw(b0, id0[0], 0);
    mask_ring[1] = issue_raw(b0 + 1, id0[1], 1);
  }
  // Q^T is an MFMA operand only: it lives in AGPRs, leaving the VGPRs to the rows in flight
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q and the first two tiles landed
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" : "+a"(qf[nt][s]));
  if (any_tile) {
    dequant(0, kf[0]);
    wait_lds();  // raw slot 0 read before it is refilled
    const uint32_t mask_b0 = mask_ring[0];
    mask_ring[0] = issue_raw(b0 + 2, id0[2], 0);
    issue_ids(b0 + 4, 0);
    qk(kf[0]);
    store_k(0, kf[0]);
    store_s();
    dequant(1, kf[1]);  // (tile b0+1 landed with Q)
    wait_lds();
    mask_prev = mask_ring[1];
    mask_ring[1] = issue_raw(b0 + 3, id0[3], 1);
    issue_ids(b0 + 5, 1);
    barrier();  // partial S^T of tile b0 published
    float sv[8];
    s_reduce(sv);
    s_mask(sv, mask_b0);
    softmax(sv, 0);
    barrier();  // weights of tile b0 published
  }

  // ---- tile loop, step j (R = (j - b0) % 2):
  // P1: QK of tile j+1 (kf[R ^ 1]), tile j+1 -> K buffer R ^ 1 and its partial S^T
  //     published; tile j+2 dequantized into kf[R] and the rows of tile j+4 and the ids
  //     of j+6 requested, all under the QK MFMAs; the PV operands of tile j read; barrier.
  // P2: PV of tile j (K buffer R, P buffer R, after the rescale its softmax asked for)
  //     with the softmax of tile j+1 -> P buffer R ^ 1 under the PV MFMAs; barrier.
  // Each phase is one scheduling region whose VALU and LDS work is spread between its
  // MFMAs (one wave per SIMD: its MFMAs hide nothing unless its own VALU instructions
  // sit between them); the steps past the last tile load zero rows and compute
  // unattended (fully masked) tiles.
  auto step = [&](int j, auto rc) __attribute__((always_inline)) {
    constexpr int R = decltype(rc)::value;
    // P1: the QK MFMAs of tile j+1, with the dequant of tile j+2 and the stores between
    // them, and the seven loads of the rows of tile j+4 and the ids of tile j+6 spread
    // between MFMA pairs (issued in a burst they stall the wave until the memory
    // pipeline drains)
    wait_vmem<kLoadsPerStep>();  // rows of tile j+2 and ids of tile j+4 landed
    RawRegs x;
    read_raw(R, x);
    const int id4 = read_id(R);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[nt][r] = 0.0f;
    const bf16x8_t (&k1)[KS] = kf[R ^ 1];
    auto qk_pair = [&](int s2) __attribute__((always_inline)) {
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1[s2], qf[0][s2], sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1[s2], qf[1][s2], sacc[1], 0, 0, 0);
    };
    qk_pair(0);
    qk_pair(1);
    wait_lds();  // raw slot R and id slot R read (their data is in x and id4)
    uint32_t mask_j4;
    const RowAddr ra = row_addr(j + 4, id4, &mask_j4);
    // seven sub-phases, each ending in one load: an MFMA pair, a k-step of the dequant
    // and K-tile stores between them
    qk_pair(2);
    dequant_ks(x, kf[R], 0);
    __builtin_amdgcn_sched_barrier(0);
    issue_load(ra, 0, R);
    __builtin_amdgcn_sched_barrier(0);
    qk_pair(3);
    dequant_ks(x, kf[R], 1);
    __builtin_amdgcn_sched_barrier(0);
    issue_load(ra, 1, R);
    __builtin_amdgcn_sched_barrier(0);
    qk_pair(4);
    dequant_ks(x, kf[R], 2);
    store_k(R ^ 1, kf[R ^ 1]);
    __builtin_amdgcn_sched_barrier(0);
    issue_load(ra, 2, R);
    __builtin_amdgcn_sched_barrier(0);
    qk_pair(5);
    dequant_ks(x, kf[R], 3);
    __builtin_amdgcn_sched_barrier(0);
    issue_load(ra, 3, R);
    __builtin_amdgcn_sched_barrier(0);
    qk_pair(6);
    dequant_ks(x, kf[R], 4);
    __builtin_amdgcn_sched_barrier(0);
    issue_load(ra, 4, R);
    __builtin_amdgcn_sched_barrier(0);
    qk_pair(7);
    dequant_ks(x, kf[R], 5);
    __builtin_amdgcn_sched_barrier(0);
    issue_load(ra, 5, R);
    __builtin_amdgcn_sched_barrier(0);
    qk_pair(8);
    dequant_ks(x, kf[R], 6);
    __builtin_amdgcn_sched_barrier(0);
    issue_ids(j + 6, R);
    __builtin_amdgcn_sched_barrier(0);
    dequant_ks(x, kf[R], 7);
    dequant_ks(x, kf[R], 8);
    store_s();
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" : "+v"(kf[R][s]));
    mask_cur = mask_ring[R];  // tile j+2
    mask_ring[R] = mask_j4;
    // the PV operands of tile j (K buffer R and P buffer R, complete since the previous
    // step): requested here so that their LDS latency passes under the barrier (the
    // dequant registers of tile j+2 are dead by now, which leaves room for them)
    bf16x8_t pf[4], vf[MT];
    pv_read(R, pf, vf);
    const uint32_t rescale_flags = flags[R];  // set by tile j's softmax, in the previous step
    barrier();
    // P2
    if (__builtin_amdgcn_readfirstlane(rescale_flags) != 0u) rescale(R);
    f32x4_t spa[kWaves], spb[kWaves];
    s_read(spa, spb);
    pv_mma(pf, vf);
    float sv[8];
    s_sum(spa, spb, sv);
    s_mask(sv, mask_prev);
    softmax(sv, R ^ 1);  // tile j+1
    SCHED_GROUP(kSchedDsRead, 2 * kWaves);
    static_for<MT * 4>([&](auto) {
      SCHED_GROUP(kSchedMfma, 1);
      SCHED_GROUP(kSchedValu, 3);
    });
    mask_prev = mask_cur;
    barrier();
  };
  // An even number of steps, so that the loop body has no exit in its middle: a tile
  // past the split's end is all unattended columns (zero rows, -inf logits, no weight).
  const int tile_stop = b0 + ((tile_end - b0 + 1) & ~1);
  for (int j = b0; j < tile_stop; j += 2) {
    step(j, std::integral_constant<int, 0>{});
    step(j + 1, std::integral_constant<int, 1>{});
  }
  // the direct loads still in flight write LDS: they land before the epilogue reuses it
  // and before the workgroup's LDS is released
  wait_vmem<0>();

  // ---- epilogue: per-head totals from the owner waves, then the output
  const bool lane_head_ok = hg * 64 + 16 * w + c16 < num_heads;
  {
    const float l_tot = sum_rows(l_run);
    const float l_exp = LSE ? sum_rows(l_lse) : l_tot;
    const int head = hg * 64 + 16 * w + c16;
    if (g == 0) {
      if (num_splits == 1) {
        const float s2 = (sink != nullptr && lane_head_ok) ? sink[head] * kLog2e : -INFINITY;
        const float mm = fmaxf(m_run, s2);
        const float mref = mm == -INFINITY ? 0.0f : mm;
        const float so = exp2f(m_run - mref);
        const float es = exp2f(s2 - mref);
        const float den = l_tot * so + es;
        const float den_lse = l_exp * so + es;
        fin_lds[16 * w + c16] = den > 0.0f ? so / den : 0.0f;
        lse_lds[16 * w + c16] = den_lse > 0.0f ? (mref + log2f(den_lse)) * kLn2 : -INFINITY;
      } else {
        fin_lds[16 * w + c16] = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        lse_lds[16 * w + c16] = l_exp > 0.0f ? m_run + log2f(l_exp) : -INFINITY;
      }
    }
  }
  barrier();  // final factors published; every wave's last PV reads of the K buffers done
  const int rows = min(64, num_heads - hg * 64);
  float f[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) f[n] = fin_lds[16 * n + c16];
  if (lse_out != nullptr && num_splits == 1 && tid < rows)
    lse_out[(int64_t)t * num_heads + hg * 64 + tid] = lse_lds[tid];
  // slice dim d of m-tile m: nope 128w + 16m + 4g (m < 8), rope 512 + 16w + 4g (m = 8)
  if (num_splits == 1) {
    // O goes through LDS (the K buffers: 64 head rows of IO_D bf16, padded by 16 bytes)
    // so that the workgroup's heads, contiguous in out, leave as one linear copy.
    constexpr int OP = 2 * IO_D + 16;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (NAT && m >= 4 && m < 8 && w == 3) continue;  // the native form's padding dims
      const int d = m < 8 ? 128 * w + 16 * m + 4 * g : R_NOPE + 16 * w + 4 * g;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        uint2 v;
        v.x = pack2(acc[m][n][0] * f[n], acc[m][n][1] * f[n]);
        v.y = pack2(acc[m][n][2] * f[n], acc[m][n][3] * f[n]);
        *reinterpret_cast<uint2*>(smem + (16 * n + c16) * OP + 2 * d) = v;
      }
    }
    barrier();
    constexpr int CPR = IO_D / 8;  // 16-byte chunks per head row
    uint8_t* obase = reinterpret_cast<uint8_t*>(out + ((int64_t)t * num_heads + hg * 64) * IO_D);
    for (int i = tid; i < rows * CPR; i += kThreads) {
      const int r = i / CPR;
      *reinterpret_cast<uint4*>(obase + 16 * (int64_t)i) =
          *reinterpret_cast<const uint4*>(smem + r * OP + 16 * (i - r * CPR));
    }
  } else {
    const int64_t base = ((int64_t)split * num_tokens + t) * num_heads;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int head = hg * 64 + 16 * n + c16;
      if (head >= num_heads) continue;
      float* prow = part_o + (base + head) * IO_D;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (NAT && m >= 4 && m < 8 && w == 3) continue;
        const int d = m < 8 ? 128 * w + 16 * m + 4 * g : R_NOPE + 16 * w + 4 * g;
        *reinterpret_cast<float4*>(prow + d) =
            make_float4(acc[m][n][0] * f[n], acc[m][n][1] * f[n], acc[m][n][2] * f[n], acc[m][n][3] * f[n]);
      }
    }
    if (tid < rows) part_lse[base + hg * 64 + tid] = lse_lds[tid];
  }
}

}  // namespace

int launch_mla_dsplit(const uint16_t* q, int T, int H, const KvDesc& s, const KvDesc& c, const int32_t* si,
                      const int32_t* lens, int W, int P, float scale, const float* sink, uint16_t* out,
                      float* lse, float* part_o, float* part_lse, int splits, bool native, hipStream_t st) {
  const int head_groups = (H + 63) / 64;
  const int pairs = T * splits;
  const int blocks = (pairs + 7) / 8 * 8 * head_groups;
  const bool one = s.pool == c.pool && s.stride == c.stride && s.num_pages == c.num_pages && s.block == c.block;
  const bool want_lse = lse != nullptr || splits > 1;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(kThreads), 0, st, q, T, H, s, c, si, lens, W, P,
                       scale * kLog2e, sink, out, lse, part_o, part_lse, splits, head_groups);
  };
  auto pick = [&](auto nat) {
    constexpr bool N = decltype(nat)::value;
    if (one)
      want_lse ? go(mla_dsplit_kernel<true, true, N>) : go(mla_dsplit_kernel<true, false, N>);
    else
      want_lse ? go(mla_dsplit_kernel<false, true, N>) : go(mla_dsplit_kernel<false, false, N>);
  };
  native ? pick(std::true_type{}) : pick(std::false_type{});
  return check_launch("sparse_mla_decode(attention)");
}

}  // namespace sad
