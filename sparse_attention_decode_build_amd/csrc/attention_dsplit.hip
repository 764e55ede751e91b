// sparse_mla_decode for the 512 fp8 + 64 bf16 latent row with fp32 block scales, and
// for the pages' native 448 fp8 + 64 bf16 row with ue8m0 scales: the dim-split kernel.
//
// [backend] forward_deepseek_v4_decode (FlashMLA sparse decode: window ids bounded by
// their lengths plus compressed ids bounded by extra_topk_length, FP8 cache,
// head_dim_v = head_dim, per-head attention sink); [model] DeepseekV4Attention
// (softmax scale head_dim^-1/2).  K and V are the same dequantized latent row.
//
// Work decomposition (gfx950, 64-lane waves, two waves per SIMD):
//   * one workgroup = one token x one group of 64 heads x one split of the token's
//     attended columns, eight waves.  The 576 latent dims are cut into four 144-dim
//     slices (slice w: nope dims 128w .. 128w+127 and rope dims 512+16w .. 512+16w+15);
//     each slice has a QK wave (wave w) and a PV wave (wave 4+w) on the same SIMD.
//   * QK wave w holds its slice of Q^T for all 64 heads in registers (the B operand of
//     v_mfma_f32_32x32x16_bf16).  Per tile of 32 attended columns it reads its slice of
//     each row (64 fp8 bytes and 8 rope values per lane, and the fp32 scale of those 64
//     bytes) from an LDS ring, dequantizes it in registers into the A operand (the
//     oracle's arithmetic: float(e4m3) * scale rounded to bf16), runs QK, stores the
//     dequantized rows into its slice's K tile and its partial S^T (its 144 dims, 64
//     heads) into LDS.  It also owns the online softmax of heads 16w .. 16w+15: it adds
//     the four partials of those heads, masks unattended columns and publishes the bf16
//     weights, the rescale factors and a rescale flag (lazy rescale: the running max is
//     kept until a tile exceeds it by 2^8).
//   * PV wave 4+w holds O^T of slice w for all 64 heads (144 accumulator registers).  It
//     reads V^T from its slice's K tile with the transposing LDS read
//     (ds_read_b64_tr_b16), the weights from LDS, and runs v_mfma_f32_16x16x32_bf16.  It
//     also issues every row load of its slice: direct global -> LDS loads
//     (global_load_lds_dwordx4 / _dword) of the rows two tiles ahead into a three-slot
//     ring, and of the slot ids four tiles ahead into a ring of their own; it alone
//     waits for them (exact vmcnt counts) before the barrier that hands them over.
//   * two barriers per tile step.  Step s: phase A = the softmax of tile s-1 (QK waves)
//     beside the 36 PV MFMAs of tile s-2 and the V^T reads of tile s-1 (PV waves);
//     phase B = the dequant and QK of tile s (QK waves) beside the weights of tile s-1,
//     its rescale and the loads of tile s+2 (PV waves).  So each SIMD always has one
//     wave of MFMAs and one of VALU work, which the hardware interleaves; a single wave
//     per SIMD holding both roles left the MFMA and VALU work serialized by its own
//     dependencies.  Every exchange (K tile, partial S^T, weights, rescale factors) has
//     one buffer: its writer and its readers are always separated by a barrier.
//   * the two head groups of one (token, split) are numbered 8 workgroups apart, so
//     they run on the same XCD at the same time and the second read of each row hits
//     that XCD's L2;
//   * the native 448 + 64 row keeps the same slices, with nope dims 448..511 (slice 3's
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

constexpr int kSlices = 4;                  // latent dim slices (one QK and one PV wave each)
constexpr int kWaves = 2 * kSlices;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;                   // attended columns per tile
constexpr int DN = 512, DR = 64, DQK = DN + DR;
constexpr int SCB = 4 * DN / 64;            // scale bytes per cached row (8 fp32)
constexpr int KS = 9;                       // QK k-steps (16 dims) of a slice
constexpr int MT = 9;                       // PV m-tiles (16 dims) of a slice
constexpr int NRAW = 3;                     // raw ring slots: tiles s (QK), s+1 (landed), s+2 (in flight)
constexpr int KPITCH = 2 * (DQK / kSlices);  // bytes per key row of a slice's K tile (288)
constexpr int KT_WAVE = kTile * KPITCH;      // one slice's K tile
constexpr int KT_BYTES = kSlices * KT_WAVE;
constexpr int XB_OFF = KT_BYTES;             // partial S^T exchange
constexpr int XB_BYTES = kSlices * 2 * 4 * 64 * 16;
constexpr int PB_OFF = XB_OFF + XB_BYTES;    // bf16 weights
constexpr int PB_BYTES = 4 * 64 * 16;
// raw ring: per slot and slice, the four 1 KB chunks of nope bytes, 1 KB of rope values
// and 256 bytes of scales, each in lane order (lane i's 16 or 4 bytes at 16i or 4i)
constexpr int RAW_OFF = PB_OFF + PB_BYTES;
constexpr int RAW_WAVE = 4 * 1024 + 1024 + 256;
constexpr int RAW_SLOT = kSlices * RAW_WAVE;
// slot-id ring: per slot and slice, the 32 ids of a tile (twice: lanes 32..63 repeat them)
constexpr int IDS_OFF = RAW_OFF + NRAW * RAW_SLOT;
constexpr int IDS_SLOT = kSlices * 256;
constexpr int MISC_OFF = IDS_OFF + 2 * IDS_SLOT;  // rescale factors, flags, final factors, lse, masks
constexpr int MISC_BYTES = 64 * 4 + 16 + 64 * 4 + 64 * 4 + 16;
constexpr int LDS_BYTES = MISC_OFF + MISC_BYTES;
constexpr float kRescaleSlack = 8.0f;       // keep the running max until exceeded by 2^8
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
static_assert(64 * (2 * DQK + 16) <= MISC_OFF, "the staged output fits below the misc words");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// Source of the loads of columns that are not attended: their rows dequantize to zero
// and their logits are masked.
__device__ __align__(16) uint8_t kZeroRow[1024];

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

// (no instruction is scheduled across it)
__device__ inline void barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

template <bool ONE, bool LSE, bool NAT>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
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
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool qk_role = wv < kSlices;
  const int w = wv & (kSlices - 1);  // the dim slice of this wave
  __builtin_assume(w >= 0 && w < kSlices);
  const int key = lane & 31;  // load / QK role: the tile row of this lane
  const int hf = lane >> 5;   // lane half: nope bytes 64hf.., rope values 8hf.. of the slice
  // The cached record: 512 fp8 + 64 bf16 with 8 fp32 scales, or (NAT) the pages' native
  // 448 fp8 + 64 bf16 with 8 ue8m0 bytes (7 used).  The slices keep the 576-dim layout
  // either way; in the native form nope dims 448..511 (slice 3's lane half 1) are zero.
  constexpr int R_NOPE = NAT ? 448 : DN;
  constexpr int R_ROWB = R_NOPE + 2 * DR;
  constexpr int R_SCB = NAT ? 8 : SCB;
  constexpr int IO_D = R_NOPE + DR;
  const bool pad_lane = NAT && w == 3 && hf == 1;
  const int c16 = lane & 15;  // softmax / PV role: head (within 16) ...
  const int g = lane >> 4;    // ... and lane group (which 8 keys of the tile)
  // keys of the lane group's k-slots: slot 4r + a <-> key 8g + 4(r ^ (g & 1)) + a (the
  // transposing read of r = 0 and r = 1 then covers 8 rows with distinct row % 8 in each
  // of its passes over two lane groups)
  const int kq0 = 8 * g + 4 * (g & 1);
  const int kq1 = 8 * g + 4 * (1 - (g & 1));

  const int width = window + padded;
  const int32_t* si_row = si + (int64_t)t * width;
  const int ncols = window + min(max(lens[t], 0), padded);
  const int ntiles = (ncols + kTile - 1) / kTile;
  const int per = (ntiles + num_splits - 1) / num_splits;
  const int tile_begin = min(ntiles, split * per);
  const int tile_end = min(ntiles, tile_begin + per);
  const int col_end = min(ncols, tile_end * kTile);
  const int b0 = tile_begin;
  const int nt = tile_end - b0;  // tiles of this split

  uint8_t* kt_w = smem + w * KT_WAVE;  // this slice's K tile
  uint8_t* xb = smem + XB_OFF;
  uint8_t* pb = smem + PB_OFF;
  float* alpha_lds = lds_ptr<float>(smem, MISC_OFF);            // [64]
  uint32_t* flags = lds_ptr<uint32_t>(smem, MISC_OFF + 256);    // byte w: slice w's heads rescaled
  float* fin_lds = lds_ptr<float>(smem, MISC_OFF + 272);        // [64]
  float* lse_lds = lds_ptr<float>(smem, MISC_OFF + 528);        // [64]
  uint32_t* mask_lds = lds_ptr<uint32_t>(smem, MISC_OFF + 784);  // [4] tile validity ring
  auto fb = [](int k) __attribute__((always_inline)) -> int { return ((k >> 2) ^ (k >> 3)) & 1; };

  // ---- row loads: the PV wave of slice w issues every load of slice w's raw ring
  // slice and id ring; each is a direct global -> LDS load, so vmcnt counts exactly these
  const uint8_t* zrow = kZeroRow;
  asm volatile("" : "+s"(zrow));
  const uint32_t lds_w = __builtin_amdgcn_readfirstlane(lds_addr(smem) + w * RAW_WAVE);
  const uint32_t ids_w = __builtin_amdgcn_readfirstlane(lds_addr(smem) + IDS_OFF + w * 256);
  const int32_t* ids_lds = reinterpret_cast<const int32_t*>(smem + IDS_OFF + w * 256);
  auto issue_ids = [&](int tile, int b) __attribute__((always_inline)) {
    const int col = tile * kTile + key;
    dma_x1(si_row + min(col, width - 1), ids_w + b * IDS_SLOT);
  };
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
    // out of the tile loop)
    KvDesc sw = swa, cp = comp;
    if (!ONE) {
      asm volatile("" : "+s"(sw.pool), "+s"(sw.stride), "+s"(sw.num_pages), "+s"(sw.block), "+s"(sw.block_shift));
      asm volatile("" : "+s"(cp.pool), "+s"(cp.stride), "+s"(cp.num_pages), "+s"(cp.block), "+s"(cp.block_shift));
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
  auto issue_raw = [&](int tile, int id, int b) __attribute__((always_inline)) -> uint32_t {
    uint32_t m;
    const RowAddr ra = row_addr(tile, id, &m);
#pragma unroll
    for (int i = 0; i < 6; ++i) issue_load(ra, i, b);
    return m;
  };
  constexpr int kLoadsPerStep = 6 + 1;  // row loads of one tile + one tile's slot ids
  if (qk_role) {
    // ===================== QK waves: dequant, QK, K tile, softmax =====================
    // Q^T fragments of the slice: B operand of the 32x32x16 MFMA, lane (head n = key,
    // half hf) holds 8 dims of k-step s: nope 128w + 64hf + 8s (s < 8), rope
    // 512 + 16w + 8hf (s = 8) of the 576-dim layout (q's rope starts at R_NOPE).  Heads
    // past num_heads load a copy of the last head (their outputs are not written), so
    // every load is unconditional; the native form's padding dims load dim 0 and are zeroed.
    bf16x8_t qf[2][KS];
#pragma unroll
    for (int n2 = 0; n2 < 2; ++n2) {
      const int head = min(hg * 64 + 32 * n2 + key, num_heads - 1);
      const uint16_t* qrow = q + ((int64_t)t * num_heads + head) * IO_D;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int d = s < 8 ? (pad_lane ? 0 : 128 * w + 64 * hf + 8 * s) : R_NOPE + 16 * w + 8 * hf;
        const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qrow + d);
        qf[n2][s] = s < 8 && pad_lane ? bf16x8_t{} : v;
      }
    }
    const uint8_t* raw_w = smem + RAW_OFF + w * RAW_WAVE;
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
      if (NAT) {
        const uint32_t b8 = (__float_as_uint(x.sc) >> (8 * (2 * (w & 1) + hf))) & 255u;
        x.sc = __uint_as_float(b8 != 0 ? b8 << 23 : 0x00400000u);
      }
    };
    // one k-step (s < 8: nope values 8s.. of the lane half's 64, s = 8: the rope values).
    // The native form's power-of-two scales take the scaled conversion
    // (v_cvt_scalef32_pk_bf16_fp8): the multiply and the bf16 rounding in one instruction
    // per pair, with the same result as bf16_rne(float(e4m3) * 2^(b - 127)) for every code
    // and scale byte 0 .. 254.  (Byte 255, which the pages' writer never produces and
    // ue8m0 reserves for NaN, decodes as NaN here instead of inf; a row holding it makes
    // the output non-finite either way.)
    auto dequant_ks = [&](const RawRegs& x, int s) __attribute__((always_inline)) -> bf16x8_t {
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
        return __builtin_bit_cast(bf16x8_t, u32x4_t{o[0], o[1], o[2], o[3]});
      }
      return __builtin_bit_cast(bf16x8_t, x.rope);
    };
    // store k-step s of this lane's K operand into the slice's K tile (row `key`, the
    // lane half's bytes: nope chunks 8hf + s are the halves s%2 of blocks 4hf + s/2, the
    // rope chunk the half hf of block 8)
    const int fbk = fb(key);
    const int st_e = key * KPITCH + 128 * hf + 16 * fbk;
    const int st_o = key * KPITCH + 128 * hf + 16 * (1 - fbk);
    const int st_r = key * KPITCH + 256 + 16 * (hf ^ fbk);
    auto store_k = [&](int s, const bf16x8_t& k) __attribute__((always_inline)) {
      const int o = s < 8 ? ((s & 1) ? st_o : st_e) + 32 * (s >> 1) : st_r;
      *reinterpret_cast<bf16x8_t*>(kt_w + o) = k;
    };
    // QK result: S^T[n2] (32 keys x 32 heads) over the slice; partial S^T -> LDS as
    // [slice][n2][reg group j][lane][4 floats]: reg group j of lane (head col, half h')
    // holds keys 8j + 4h' + 0..3, which the lane group g = j of the owner wave reads
    f32x16_t sacc[2];
    auto store_s = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int n2 = 0; n2 < 2; ++n2) {
        f32x4_t* dst = reinterpret_cast<f32x4_t*>(xb) + ((w * 2 + n2) * 4) * 64 + lane;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          dst[j * 64] = f32x4_t{sacc[n2][4 * j], sacc[n2][4 * j + 1], sacc[n2][4 * j + 2], sacc[n2][4 * j + 3]};
      }
    };
    // ---- online softmax of heads 16w .. 16w+15 (lane: head 16w + c16, 8 keys of group g):
    // the lane's partial S^T chunks are reg group g of source lane col + 32(g & 1) (keys
    // kq0..) and of lane col + 32(1 - (g & 1)) (keys kq1..), n2 = w / 2, col = 16(w % 2) + c16
    const int sr_off = ((w >> 1) * 4 + g) * 64 + 16 * (w & 1) + c16 + 32 * (g & 1);
    float m_run = -INFINITY;
    float l_run = 0.0f;  // sum of the bf16-rounded weights the PV MFMA multiplies with
    float l_lse = 0.0f;  // sum of the fp32 weights (log-sum-exp)
    // the four partials of this lane's 8 keys, summed (k-slot order)
    auto s_reduce = [&](float (&sv)[8]) __attribute__((always_inline)) {
      const f32x4_t* src = reinterpret_cast<const f32x4_t*>(xb) + sr_off;
      f32x4_t pa[kSlices], pb2[kSlices];
#pragma unroll
      for (int v = 0; v < kSlices; ++v) {
        pa[v] = src[v * 2 * 4 * 64];
        pb2[v] = src[v * 2 * 4 * 64 + 32 - 64 * (g & 1)];
      }
      f32x4_t a = pa[0], b = pb2[0];
#pragma unroll
      for (int v = 1; v < kSlices; ++v) {
        a += pa[v];
        b += pb2[v];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = a[i];
        sv[4 + i] = b[i];
      }
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
    auto softmax = [&](const float (&sv)[8]) __attribute__((always_inline)) {
      // the running maximum is kept until a tile exceeds it by 2^slack (also true while it
      // is -inf); O needs rescaling only when it already holds weights (a finite maximum).
      // A head's maximum moves iff one of its keys has sv * scale_log2 > m_run + slack:
      // rounding is monotone, so that is the test max(sv) * scale_log2 > m_run + slack
      // key by key.  When no lane of the wave has such a key (the usual tile) the
      // maximum, its cross-lane reduction and the rescale are skipped.
      float p[8];
      bool resc = false;
      float alpha = 1.0f;
      bool over = false;
      const float thr = m_run + kRescaleSlack;
#pragma unroll
      for (int i = 0; i < 8; ++i) over = over || sv[i] * scale_log2 > thr;
      if (__ballot(over) == 0ull) {
        const float m_use = m_run == -INFINITY ? 0.0f : m_run;
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], scale_log2, -m_use));
      } else {
        float tmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
        tmax = max_rows(tmax) * scale_log2;
        const bool upd = tmax > thr;
        resc = upd && m_run != -INFINITY;
        const float m_new = upd ? tmax : m_run;
        alpha = resc ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        m_run = m_new;
        l_run *= alpha;
        if (LSE) l_lse *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], scale_log2, -m_use));
      }
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
      reinterpret_cast<u32x4_t*>(pb)[w * 64 + lane] = u32x4_t{pw[0], pw[1], pw[2], pw[3]};
      // every lane stores (the four lanes of a head store the same value): no branch
      const bool any = __ballot(resc) != 0ull;
      alpha_lds[16 * w + c16] = alpha;
      reinterpret_cast<uint8_t*>(flags)[w] = any ? 1 : 0;
    };

    int slot = 0;  // raw slot of tile s: (s - b0) % 3
    // step s: A = the softmax of tile s-1; B = the dequant and QK of tile s, its K tile
    // and partial S^T.  The loop is peeled so that every step is straight-line code.
    auto qk_step = [&](int s, auto doA, auto doB) __attribute__((always_inline)) {
      if constexpr (decltype(doA)::value) {
        float sv[8];
        s_reduce(sv);
        // (most tiles have every column attended: no mask to apply)
        const uint32_t vm = __builtin_amdgcn_readfirstlane(mask_lds[(s - 1 - b0) & 3]);
        if (vm != 0xFFFFFFFFu) s_mask(sv, vm);
        softmax(sv);
      }
      barrier();  // A: weights of tile s-1 published; V^T of tile s-1 read
      if constexpr (decltype(doB)::value) {
        RawRegs x;
        read_raw(slot, x);
#pragma unroll
        for (int n2 = 0; n2 < 2; ++n2)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[n2][r] = 0.0f;
        // k-step by k-step: the dequant, its K-tile store and its MFMA pair, in this order
        // (the scheduler otherwise sinks the K-tile stores behind the last MFMAs, where
        // they lengthen the burst of stores the barrier waits for); the MFMAs of one
        // k-step run while the next k-step's dequant issues
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8_t k = dequant_ks(x, ks);
          store_k(ks, k);
          sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, qf[0][ks], sacc[0], 0, 0, 0);
          sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, qf[1][ks], sacc[1], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        store_s();
        slot = slot == NRAW - 1 ? 0 : slot + 1;
      }
      barrier();  // B: partial S^T and K tile of tile s published
    };
    constexpr std::true_type kT{};
    constexpr std::false_type kF{};
    if (nt > 0) {
      qk_step(b0, kF, kT);
      for (int s = b0 + 1; s < tile_end; ++s) qk_step(s, kT, kT);
      qk_step(tile_end, kT, kF);
      qk_step(tile_end + 1, kF, kF);
    }
    // ---- epilogue: final factors of heads 16w .. 16w+15
    const bool lane_head_ok = hg * 64 + 16 * w + c16 < num_heads;
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
    barrier();  // E1: final factors published
    const int rows = min(64, num_heads - hg * 64);
    if (lse_out != nullptr && num_splits == 1 && tid < rows)
      lse_out[(int64_t)t * num_heads + hg * 64 + tid] = lse_lds[tid];
    if (num_splits > 1 && tid < rows) {
      const int64_t base = ((int64_t)split * num_tokens + t) * num_heads;
      part_lse[base + hg * 64 + tid] = lse_lds[tid];
    }
    if (num_splits == 1) barrier();  // E2: output staged
  } else {
    // ===================== PV waves: O^T (slice w, 64 heads) += V^T P^T =====================
    // tile (m, n): lane (c16, g) holds head 16n + c16, dims 16m + 4g .. +3 of the slice
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
    bf16x8_t pf[4], vf[MT];
    auto read_v = [&](int m) __attribute__((always_inline)) {
      typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
      const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kt_w + vrd0 + 32 * m));
      const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kt_w + vrd1 + 32 * m));
      vf[m] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // prologue: rows of tiles b0 and b0+1 (raw slots 0, 1), ids of b0+2 and b0+3 (id
    // slots 0, 1), their validity in the mask ring; all landed before the first barrier.
    // The two id loads are the only vector loads the compiler tracks.
    if (nt > 0) {
      const int ida = si_row[min(b0 * kTile + key, width - 1)];
      const int idb = si_row[min((b0 + 1) * kTile + key, width - 1)];
      const uint32_t m0 = issue_raw(b0, ida, 0);
      const uint32_t m1 = issue_raw(b0 + 1, idb, 1);
      issue_ids(b0 + 2, 0);
      issue_ids(b0 + 3, 1);
      if (w == 0) {
        mask_lds[0] = m0;
        mask_lds[1] = m1;
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    int rslot = 2;  // raw slot of tile s+2 at step s
    // step s: A = PV MFMAs of tile s-2 (operands in registers) and the V^T reads of tile
    // s-1; B = the weights of tile s-1 and its rescale, then the rows of tile s+2 and the
    // ids of tile s+4 requested (s < tile_end)
    auto pv_step = [&](int s, auto mma_c, auto rd_c) __attribute__((always_inline)) {
      constexpr bool mma = decltype(mma_c)::value, rd = decltype(rd_c)::value;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if constexpr (mma) {
#pragma unroll
          for (int n = 0; n < 4; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[m], pf[n], acc[m][n], 0, 0, 0);
        }
        if constexpr (rd) read_v(m);
      }
      wait_vmem<kLoadsPerStep>();  // rows of tile s (requested at step s-2) landed
      barrier();  // A
      if constexpr (rd) {
#pragma unroll
        for (int n = 0; n < 4; ++n) pf[n] = reinterpret_cast<const bf16x8_t*>(pb)[n * 64 + lane];
        // the rescale tile s-1's softmax asked for, before any of its weights are added
        const uint32_t fl = flags[0];
        if (__builtin_amdgcn_readfirstlane(fl) != 0u) {
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            const float al = alpha_lds[16 * n + c16];
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m][n] *= al;
          }
        }
      }
      if (s < tile_end) {
        const int R = (s - b0) & 1;
        const int id2 = ids_lds[R * (IDS_SLOT / 4) + lane];
        wait_lds();
        uint32_t mnew;
        const RowAddr ra = row_addr(s + 2, id2, &mnew);
#pragma unroll
        for (int i = 0; i < 6; ++i) issue_load(ra, i, rslot);
        issue_ids(s + 4, R);
        if (w == 0) mask_lds[(s + 2 - b0) & 3] = mnew;
        rslot = rslot == NRAW - 1 ? 0 : rslot + 1;
      }
      barrier();  // B
    };
    constexpr std::true_type kT{};
    constexpr std::false_type kF{};
    if (nt > 0) {
      pv_step(b0, kF, kF);
      pv_step(b0 + 1, kF, kT);  // V^T of tile b0
      for (int s = b0 + 2; s < tile_end + 1; ++s) pv_step(s, kT, kT);
      pv_step(tile_end + 1, kT, kF);  // PV of the last tile
    }
    // the direct loads still in flight write LDS: they land before the epilogue reuses it
    wait_vmem<0>();
    barrier();  // E1
    const int rows = min(64, num_heads - hg * 64);
    float f[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) f[n] = fin_lds[16 * n + c16];
    // slice dim d of m-tile m: nope 128w + 16m + 4g (m < 8), rope 512 + 16w + 4g (m = 8)
    if (num_splits == 1) {
      // O goes through LDS (64 head rows of IO_D bf16, padded by 16 bytes) so that the
      // workgroup's heads, contiguous in out, leave as one linear copy
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
      barrier();  // E2
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
    }
  }
  if (num_splits == 1) {
    constexpr int OP = 2 * IO_D + 16;
    constexpr int CPR = IO_D / 8;
    const int rows = min(64, num_heads - hg * 64);
    uint8_t* obase = reinterpret_cast<uint8_t*>(out + ((int64_t)t * num_heads + hg * 64) * IO_D);
    for (int i = tid; i < rows * CPR; i += kThreads) {
      const int r = i / CPR;
      *reinterpret_cast<uint4*>(obase + 16 * (int64_t)i) =
          *reinterpret_cast<const uint4*>(smem + r * OP + 16 * (i - r * CPR));
    }
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
