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
//     in VGPRs, and its O^T accumulator for those output dims in AGPRs, for the whole
//     split.  The two waves of a head block add their partial S^T through LDS;
//   * the workgroups of one token's head groups are numbered 8 apart so they run on the
//     same XCD at the same time and the second read of each row hits that XCD's L2;
//   * columns are taken 32 at a time.  The raw cache bytes of tile i+1 are copied
//     HBM -> LDS by direct global-to-LDS loads (no VGPRs) while tile i is computed;
//     the row addresses of tile i+2 are resolved meanwhile;
//   * tile i is dequantized from LDS (fp32 multiply by the row's block scale, bf16
//     rounding) into two LDS copies: key-major K[32][D] for S^T = K Q^T, dim-major
//     V^T[D][32] for O^T += V^T P^T;
//   * S^T puts one head per lane, so the online softmax needs only a swap with lane^32,
//     and the probabilities already sit in the B-operand layout of the PV MFMA (the key
//     order inside V^T rows is permuted to match);
//   * splits of one token write (o / l, log2-sum-exp) partials that a second kernel
//     merges, with the sink, when more than one split is used.
// Barriers are raw s_barrier with explicit LDS waits so that the in-flight LDS DMA of
// the next tile is only waited for when that tile is consumed.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "sad_internal.h"

namespace sad {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;              // attended columns per tile
constexpr float kRescaleSlack = 8.0f;  // keep the running max until exceeded by 2^8
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// s_waitcnt immediates (gfx9 encoding): lgkmcnt(0) only; vmcnt(0) only.
constexpr int kWaitLgkm0 = 0xC07F;
constexpr int kWaitVm0 = 0x0F70;

__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
}

struct KvDesc {
  const uint8_t* pool;
  int64_t stride;
  int64_t num_pages;
  int block;
};

template <int DN, int DR>
struct Shape {
  static constexpr int DQK = DN + DR;
  static constexpr int ROWB = DN + 2 * DR;  // value bytes per cached row
  static constexpr int NSC = DN / 64;       // fp32 scales per row
  static constexpr int MT = DQK / 32;       // PV MFMA m-tiles (output dims / 32)
  static constexpr int MT0 = (MT + 1) / 2;  // m-tiles of dim half 0 (half 1 gets the rest)
  static constexpr int MT1 = MT - MT0;
  static constexpr int KS0 = 2 * MT0;       // QK k-steps (16 dims) of dim half 0
  static constexpr int KS1 = 2 * MT1;
  static constexpr int KROW = DQK + 8;      // padded K-major row (bf16 elements)
  static constexpr int CPR = ROWB / 16;     // 16-byte chunks per row
  static constexpr int VAL_LOADS = (kTile * CPR + kThreads - 1) / kThreads;  // per wave
  static constexpr int NOPE_UNITS = (kTile / 8) * (DN / 4);  // 8 keys x 4 fp8 dims
  static constexpr int NU = (NOPE_UNITS + kThreads - 1) / kThreads;
  static constexpr int ROPE_UNITS = (kTile / 4) * (DR / 4);  // 4 keys x 4 bf16 dims
  static_assert(ROWB % 16 == 0, "rows are whole 16-byte chunks");
  static_assert(kTile * NSC <= kThreads, "one scale dword per thread");
  static_assert(ROPE_UNITS <= kThreads, "one rope unit per thread");
  static_assert(DQK % 32 == 0, "output dims in 32-row MFMA tiles");
};


// Keys of the 8-key V^T chunk c (chunk c = 2*ks + h feeds k-step ks, lane half h):
// position e (0..7) holds key 16*(c/2) + 8*(e/4) + 4*(c%2) + e%4, which is the key the
// S^T accumulator register 8*ks + e of a lane in half h belongs to.
__device__ inline int chunk_key(int c, int e) {
  return 16 * (c >> 1) + 8 * (e >> 2) + 4 * (c & 1) + (e & 3);
}

// Physical 16-byte chunk of V^T row d holding logical chunk c (the rotation spreads LDS
// banks for both the fragment reads (8 consecutive rows) and the dequant writes).
__device__ inline int vt_chunk(int d, int c) { return (c + (d >> 1) + (d >> 3)) & 3; }

__device__ inline uint32_t pack_bf16(float a, float b) {
  return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
}

// Row base pointers of one tile (values, scales); nullptr = column not attended.
__device__ inline void resolve_rows(const uint8_t** rowv, const uint8_t** rows, int tile0,
                                    int ncols, int window, const int32_t* si_row,
                                    const KvDesc& swa, const KvDesc& comp, int rowb, int nsc) {
  const int r = threadIdx.x;
  if (r >= kTile) return;
  const int col = tile0 + r;
  const uint8_t* pv = nullptr;
  const uint8_t* ps = nullptr;
  if (col < ncols) {
    const int slot = si_row[col];
    const KvDesc& kv = col < window ? swa : comp;
    if (slot_ok(slot, kv.block, kv.num_pages)) {
      const int page = slot / kv.block;
      const int ro = slot - page * kv.block;
      const uint8_t* pg = kv.pool + (int64_t)page * kv.stride;
      pv = pg + (int64_t)ro * rowb;
      ps = pg + (int64_t)kv.block * rowb + (int64_t)ro * 4 * nsc;
    }
  }
  rowv[r] = pv;
  rows[r] = ps;
}

// Copy one tile's raw rows (values and fp32 scales) HBM -> LDS with direct loads.
// Unattended rows read a harmless dummy address; their data is zeroed on dequant.
template <int DN, int DR>
__device__ inline void dma_tile(uint8_t* raw_v, float* raw_s, const uint8_t* const* rowv,
                                const uint8_t* const* rows, const void* dummy) {
  using S = Shape<DN, DR>;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < S::VAL_LOADS; ++j) {
    const int q0 = (j * kWaves + wave) * 64;
    const int q = q0 + lane;
    if (q0 < kTile * S::CPR) {
      if (q < kTile * S::CPR) {
        const int row = q / S::CPR;
        const int c16 = q - row * S::CPR;
        const uint8_t* base = rowv[row];
        const void* src = base != nullptr ? (const void*)(base + 16 * c16) : dummy;
        __builtin_amdgcn_global_load_lds(src, raw_v + q0 * 16, 16, 0, 0);
      }
    }
  }
  {
    const int q0 = wave * 64;
    const int q = q0 + lane;
    if (q0 < kTile * S::NSC) {
      if (q < kTile * S::NSC) {
        const int row = q / S::NSC;
        const uint8_t* base = rows[row];
        const void* src = base != nullptr ? (const void*)(base + 4 * (q - row * S::NSC)) : dummy;
        __builtin_amdgcn_global_load_lds(src, raw_s + q0, 4, 0, 0);
      }
    }
  }
}

// Dequantize the raw tile in LDS into the K-major and V^T copies.
template <int DN, int DR>
__device__ inline void dequant_tile(const uint8_t* raw_v, const float* raw_s, uint32_t valid,
                                    uint16_t* kt, uint16_t* vt) {
  using S = Shape<DN, DR>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < S::NU; ++u) {
    const int unit = tid + u * kThreads;
    if (unit < S::NOPE_UNITS) {
      const int c = unit / (DN / 4);
      const int dg = unit - c * (DN / 4);
      uint32_t packed[8][2];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = chunk_key(c, e);
        const bool ok = (valid >> key) & 1u;
        const uint32_t w = ok ? *reinterpret_cast<const uint32_t*>(raw_v + key * S::ROWB + 4 * dg) : 0u;
        const float sc = ok ? raw_s[key * S::NSC + (4 * dg) / 64] : 0.0f;
        packed[e][0] = pack_bf16(e4m3_to_f32<0>(w) * sc, e4m3_to_f32<1>(w) * sc);
        packed[e][1] = pack_bf16(e4m3_to_f32<2>(w) * sc, e4m3_to_f32<3>(w) * sc);
        *reinterpret_cast<uint2*>(kt + key * S::KROW + 4 * dg) = make_uint2(packed[e][0], packed[e][1]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 4 * dg + j;
        // bf16 of dim j for keys e = 0..7: low or high half of packed[e][j/2]
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        uint4 w;
        w.x = __builtin_amdgcn_perm(packed[1][j >> 1], packed[0][j >> 1], sel);
        w.y = __builtin_amdgcn_perm(packed[3][j >> 1], packed[2][j >> 1], sel);
        w.z = __builtin_amdgcn_perm(packed[5][j >> 1], packed[4][j >> 1], sel);
        w.w = __builtin_amdgcn_perm(packed[7][j >> 1], packed[6][j >> 1], sel);
        *reinterpret_cast<uint4*>(vt + d * kTile + 8 * vt_chunk(d, c)) = w;
      }
    }
  }
  if (tid < S::ROPE_UNITS) {
    const int kq = tid / (DR / 4);
    const int dg = tid - kq * (DR / 4);
    // keys 4kq..4kq+3 = chunk c = 2*(kq/4) + kq%2, positions 4*((kq/2)%2) .. +3
    const int c = 2 * (kq >> 2) + (kq & 1);
    const int pos0 = 4 * ((kq >> 1) & 1);
    uint2 r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = 4 * kq + j;
      r[j] = ((valid >> key) & 1u) ? *reinterpret_cast<const uint2*>(raw_v + key * S::ROWB + DN + 8 * dg)
                                   : make_uint2(0u, 0u);
      *reinterpret_cast<uint2*>(kt + key * S::KROW + DN + 4 * dg) = r[j];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d = DN + 4 * dg + e;
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t a0 = (e < 2) ? r[0].x : r[0].y;
      const uint32_t a1 = (e < 2) ? r[1].x : r[1].y;
      const uint32_t a2 = (e < 2) ? r[2].x : r[2].y;
      const uint32_t a3 = (e < 2) ? r[3].x : r[3].y;
      uint2 w;
      w.x = __builtin_amdgcn_perm(a1, a0, sel);
      w.y = __builtin_amdgcn_perm(a3, a2, sel);
      *reinterpret_cast<uint2*>(vt + d * kTile + 8 * vt_chunk(d, c) + pos0) = w;
    }
  }
}

template <int DN, int DR>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(1, 1)))
sparse_mla_kernel(const uint16_t* __restrict__ q, int num_tokens, int num_heads, KvDesc swa,
                  KvDesc comp, const int32_t* __restrict__ si, const int32_t* __restrict__ lens,
                  int window, int padded, float scale_log2, const float* __restrict__ sink,
                  uint16_t* __restrict__ out, float* __restrict__ lse_out,
                  float* __restrict__ part_o, float* __restrict__ part_lse, int num_splits,
                  int head_groups) {
  using S = Shape<DN, DR>;
  constexpr int DQK = S::DQK;
  constexpr int KSMAX = S::KS0;
  constexpr int MTMAX = S::MT0;
  // Distinct LDS objects, so the compiler can tell the DMA targets from the buffers
  // that are read while a DMA is in flight.
  __shared__ __align__(16) uint8_t raw_v0[kTile * S::ROWB];
  __shared__ __align__(16) uint8_t raw_v1[kTile * S::ROWB];
  __shared__ __align__(16) float raw_s0[kTile * S::NSC];
  __shared__ __align__(16) float raw_s1[kTile * S::NSC];
  __shared__ __align__(16) uint16_t kt[kTile * S::KROW];
  __shared__ __align__(16) uint16_t vt[DQK * kTile];
  __shared__ __align__(16) float xbuf[kWaves * 16 * 64];
  __shared__ const uint8_t* rowv0[kTile];
  __shared__ const uint8_t* rowv1[kTile];
  __shared__ const uint8_t* rows0[kTile];
  __shared__ const uint8_t* rows1[kTile];

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
  const int wave = tid >> 6;
  const int n = lane & 31;  // head within the wave's block / key row within a fragment
  const int h = lane >> 5;  // lane half
  const int hb = wave >> 1;  // head block of this wave
  const int dh = wave & 1;   // dim half of this wave
  const int head = hg * 64 + hb * 32 + n;
  const bool block_active = hg * 64 + hb * 32 < num_heads;
  const int ks_n = dh == 0 ? S::KS0 : S::KS1;  // k-steps of this wave's dims
  const int mt_n = dh == 0 ? S::MT0 : S::MT1;  // m-tiles of this wave's dims
  const int dim0 = dh == 0 ? 0 : 32 * S::MT0;  // first dim of this wave's half

  const int width = window + padded;
  const int32_t* si_row = si + (int64_t)t * width;
  const int ncols = window + min(max(lens[t], 0), padded);
  const int ntiles = (ncols + kTile - 1) / kTile;
  const int per = (ntiles + num_splits - 1) / num_splits;
  const int tile_begin = split * per;
  const int tile_end = min(ntiles, tile_begin + per);
  const uint16_t* qrow = q + ((int64_t)t * num_heads + min(head, num_heads - 1)) * DQK;
  const void* dummy = q + (int64_t)t * num_heads * DQK;  // >= 16 readable bytes

  // Q^T fragments: lane (head n, half h) holds dims dim0 + [16kk + 8h, 16kk + 8h + 8).
  bf16x8_t qf[KSMAX];
#pragma unroll
  for (int kk = 0; kk < KSMAX; ++kk) {
    qf[kk] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    if (kk < ks_n && head < num_heads)
      qf[kk] = *reinterpret_cast<const bf16x8_t*>(qrow + dim0 + 16 * kk + 8 * h);
  }

  f32x16_t acc_o[MTMAX];
#pragma unroll
  for (int mt = 0; mt < MTMAX; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[mt][r] = 0.0f;
  float m_run = -INFINITY;
  float l_run = 0.0f;  // sum of the bf16-rounded weights (normalizes O)
  float l_lse = 0.0f;  // sum of the fp32 weights (log-sum-exp)

  // Prologue: rows of the first two tiles, DMA of the first.
  if (tile_begin < tile_end) {
    resolve_rows(rowv0, rows0, tile_begin * kTile, ncols, window, si_row, swa, comp, S::ROWB, S::NSC);
    resolve_rows(rowv1, rows1, (tile_begin + 1) * kTile, ncols, window, si_row, swa, comp, S::ROWB,
                 S::NSC);
    lds_barrier();
    dma_tile<DN, DR>(raw_v0, raw_s0, rowv0, rows0, dummy);
  }

  // One tile step; the tag selects the LDS staging buffer holding this tile.
  auto step = [&](int tile, auto cur_tag) __attribute__((always_inline)) {
    constexpr bool CUR1 = decltype(cur_tag)::value;
    uint8_t* raw_v = CUR1 ? raw_v1 : raw_v0;
    float* raw_s = CUR1 ? raw_s1 : raw_s0;
    uint8_t* nraw_v = CUR1 ? raw_v0 : raw_v1;
    float* nraw_s = CUR1 ? raw_s0 : raw_s1;
    const uint8_t** rowv = CUR1 ? rowv1 : rowv0;
    const uint8_t** rows = CUR1 ? rows1 : rows0;
    const uint8_t** nrowv = CUR1 ? rowv0 : rowv1;
    const uint8_t** nrows = CUR1 ? rows0 : rows1;
    const int tile0 = tile * kTile;

    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's DMA of this tile landed
    lds_barrier();  // all waves' DMA landed; the previous tile's compute is done
    if (tile + 1 < tile_end) dma_tile<DN, DR>(nraw_v, nraw_s, nrowv, nrows, dummy);
    if (tile + 2 < tile_end)
      resolve_rows(rowv, rows, tile0 + 2 * kTile, ncols, window, si_row, swa, comp, S::ROWB, S::NSC);
    // validity of this tile's 32 columns, one bit per key
    uint32_t valid_mask;
    {
      bool ok = false;
      const int col = tile0 + n;
      if (col < ncols) {
        const int slot = si_row[col];
        const KvDesc& kv = col < window ? swa : comp;
        ok = slot_ok(slot, kv.block, kv.num_pages);
      }
      valid_mask = (uint32_t)__ballot(ok);
    }
    dequant_tile<DN, DR>(raw_v, raw_s, valid_mask, kt, vt);
    lds_barrier();  // K / V^T copies complete

    // ---- partial S^T = K Q^T over this wave's dims: lane (head n, half h) gets
    //      keys 8*(r/4) + 4h + r%4, r = 0..15
    f32x16_t s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.0f;
    if (block_active) {
#pragma unroll
      for (int kk = 0; kk < KSMAX; ++kk) {
        if (kk < ks_n) {
          const bf16x8_t a =
              *reinterpret_cast<const bf16x8_t*>(kt + n * S::KROW + dim0 + 16 * kk + 8 * h);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s, 0, 0, 0);
        }
      }
    }
    // ---- add the partner wave's half: S = S(dims half 0) + S(dims half 1)
#pragma unroll
    for (int r = 0; r < 16; ++r) xbuf[(wave * 16 + r) * 64 + lane] = s[r];
    lds_barrier();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float other = xbuf[((wave ^ 1) * 16 + r) * 64 + lane];
      s[r] = dh == 0 ? s[r] + other : other + s[r];
    }
    if (!block_active) return;
    // ---- online softmax (log2 domain, lazy rescaling); identical in both dim halves
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * h + (r & 3);
      s[r] = ((valid_mask >> key) & 1u) ? s[r] * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, s[r]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const bool upd = tmax > m_run + kRescaleSlack;  // also true when m_run is -inf
    if (__ballot(upd) != 0ull) {
      const float alpha = upd ? exp2f(m_run - tmax) : 1.0f;  // exp2(-inf) = 0
      if (upd) m_run = tmax;
      l_run *= alpha;
      l_lse *= alpha;
#pragma unroll
      for (int mt = 0; mt < MTMAX; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[mt][r] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.0f : m_run;
    bf16x8_t pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // normalize by the same rounded weights the PV MFMA multiplies with
      const float pf = exp2f(s[r] - m_use);
      const __bf16 p = (__bf16)pf;
      l_run += (float)p;
      l_lse += pf;
      pb[r >> 3][r & 7] = p;
    }
    // ---- O^T += V^T P^T over this wave's output dims
#pragma unroll
    for (int mt = 0; mt < MTMAX; ++mt) {
      if (mt < mt_n) {
        const int d = dim0 + 32 * mt + n;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8_t a =
              *reinterpret_cast<const bf16x8_t*>(vt + d * kTile + 8 * vt_chunk(d, 2 * ks + h));
          acc_o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks], acc_o[mt], 0, 0, 0);
        }
      }
    }
  };

  for (int tile = tile_begin; tile < tile_end; tile += 2) {
    step(tile, std::false_type{});
    if (tile + 1 < tile_end) step(tile + 1, std::true_type{});
  }

  if (!block_active || head >= num_heads) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float l_exp = l_lse + __shfl_xor(l_lse, 32, 64);
  // lane (n, h) holds O^T rows (dims) dim0 + 32mt + 8(r/4) + 4h + r%4 for head n
  if (num_splits == 1) {
    const float s2 = sink != nullptr ? sink[head] * kLog2e : -INFINITY;
    const float mm = fmaxf(m_run, s2);
    const float mref = mm == -INFINITY ? 0.0f : mm;
    const float so = exp2f(m_run - mref);
    const float es = exp2f(s2 - mref);
    const float den = l_tot * so + es;
    const float den_lse = l_exp * so + es;
    const float f = den > 0.0f ? so / den : 0.0f;
    uint16_t* orow = out + ((int64_t)t * num_heads + head) * DQK + dim0;
#pragma unroll
    for (int mt = 0; mt < MTMAX; ++mt)
      if (mt < mt_n) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint2 w;
          w.x = pack_bf16(acc_o[mt][4 * g + 0] * f, acc_o[mt][4 * g + 1] * f);
          w.y = pack_bf16(acc_o[mt][4 * g + 2] * f, acc_o[mt][4 * g + 3] * f);
          *reinterpret_cast<uint2*>(orow + 32 * mt + 8 * g + 4 * h) = w;
        }
      }
    if (lse_out != nullptr && h == 0 && dh == 0)
      lse_out[(int64_t)t * num_heads + head] = den_lse > 0.0f ? (mref + log2f(den_lse)) * kLn2 : -INFINITY;
  } else {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    float* prow = part_o + (((int64_t)split * num_tokens + t) * num_heads + head) * DQK + dim0;
#pragma unroll
    for (int mt = 0; mt < MTMAX; ++mt)
      if (mt < mt_n) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 w = make_float4(acc_o[mt][4 * g + 0] * inv, acc_o[mt][4 * g + 1] * inv,
                                       acc_o[mt][4 * g + 2] * inv, acc_o[mt][4 * g + 3] * inv);
          *reinterpret_cast<float4*>(prow + 32 * mt + 8 * g + 4 * h) = w;
        }
      }
    if (h == 0 && dh == 0)
      part_lse[((int64_t)split * num_tokens + t) * num_heads + head] =
          l_exp > 0.0f ? m_run + log2f(l_exp) : -INFINITY;
  }
}

// Merge split partials: out = sum_s 2^(lse_s - M) o_s / (sum_s 2^(lse_s - M) + 2^(sink2 - M)).
template <int DQK>
__global__ __launch_bounds__(DQK) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse,
                                                      int num_splits, int T, int num_heads,
                                                      const float* __restrict__ sink,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ lse_out) {
  const int head = blockIdx.x;
  const int t = blockIdx.y;
  const int d = threadIdx.x;
  const int64_t th = (int64_t)t * num_heads + head;
  const int64_t plane = (int64_t)T * num_heads;
  const float s2 = sink != nullptr ? sink[head] * kLog2e : -INFINITY;
  float mm = s2;
  for (int s = 0; s < num_splits; ++s) mm = fmaxf(mm, part_lse[s * plane + th]);
  const float mref = mm == -INFINITY ? 0.0f : mm;
  float den = exp2f(s2 - mref);
  float acc = 0.0f;
  for (int s = 0; s < num_splits; ++s) {
    const float w = exp2f(part_lse[s * plane + th] - mref);
    den += w;
    acc += w * part_o[(s * plane + th) * DQK + d];
  }
  out[th * DQK + d] = f32_to_bf16_bits(den > 0.0f ? acc / den : 0.0f);
  if (lse_out != nullptr && d == 0)
    lse_out[th] = den > 0.0f ? (mref + log2f(den)) * kLn2 : -INFINITY;
}

int choose_splits(int T, int num_heads, int max_cols, int dqk, int rowb) {
  const int units = T * ((num_heads + 63) / 64);  // workgroups without splitting
  if (units <= 0 || units >= kNumCUs) return 1;
  const int tiles = (max_cols + kTile - 1) / kTile;
  int s = (kNumCUs + units - 1) / units;
  s = std::min(s, std::max(1, tiles / 4));
  // keep the partials' traffic (write + read of 128 heads x dqk fp32) below the rows'
  const int64_t row_bytes = (int64_t)max_cols * rowb;
  const int64_t part_bytes = 2LL * 128 * dqk * 4;
  s = (int)std::min<int64_t>(s, std::max<int64_t>(1, row_bytes / part_bytes));
  return std::max(1, s);
}

template <int DN, int DR>
int launch(const uint16_t* q, int T, int H, const KvDesc& s, const KvDesc& c, const int32_t* si,
           const int32_t* lens, int W, int P, float scale, const float* sink, uint16_t* out,
           float* lse, void* ws, size_t ws_bytes, hipStream_t st) {
  using Sh = Shape<DN, DR>;
  const int splits = choose_splits(T, H, W + P, Sh::DQK, Sh::ROWB);
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
  const int head_groups = (H + 63) / 64;
  const int pairs = T * splits;
  const int blocks = (pairs + 7) / 8 * 8 * head_groups;
  hipLaunchKernelGGL((sparse_mla_kernel<DN, DR>), dim3(blocks), dim3(kThreads), 0, st, q, T, H, s, c,
                     si, lens, W, P, scale * kLog2e, sink, out, lse, part_o, part_lse, splits,
                     head_groups);
  int rc = check_launch("sparse_mla_decode(attention)");
  if (rc != SAD_OK || splits == 1) return rc;
  hipLaunchKernelGGL((combine_kernel<Sh::DQK>), dim3(H, T), dim3(Sh::DQK), 0, st, part_o, part_lse,
                     splits, T, H, sink, out, lse);
  return check_launch("sparse_mla_decode(combine)");
}

}  // namespace
}  // namespace sad

using namespace sad;

extern "C" size_t sparse_mla_decode_workspace_size(int32_t num_tokens, int32_t num_heads,
                                                   int32_t max_row_width, int32_t dv) {
  if (num_tokens <= 0 || num_heads <= 0 || max_row_width <= 0 || dv <= 0) return 0;
  // value bytes per cached row for the supported latent shapes
  const int rowb = dv == 576 ? 640 : (dv == 160 ? 192 : 2 * dv);
  const int splits = choose_splits(num_tokens, num_heads, max_row_width, dv, rowb);
  if (splits <= 1) return 0;
  const size_t n = (size_t)splits * num_tokens * num_heads;
  return (n * dv + n) * sizeof(float);
}

extern "C" int sparse_mla_decode(const uint16_t* q_bf16, int32_t num_tokens, int32_t num_heads,
                                 const sad_kv_cache* swa, const sad_kv_cache* comp,
                                 const int32_t* sparse_indices, const int32_t* sparse_topk_lens,
                                 int32_t window_size, int32_t padded_topk, float softmax_scale,
                                 const float* attn_sink, uint16_t* out_bf16, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  int rc = check_kv_cache(swa, "sparse_mla_decode(swa)");
  if (rc != SAD_OK) return rc;
  rc = check_kv_cache(comp, "sparse_mla_decode(comp)");
  if (rc != SAD_OK) return rc;
  SAD_CHECK(swa->d_nope == comp->d_nope && swa->d_rope == comp->d_rope, SAD_EINVAL,
            "sparse_mla_decode: swa and comp caches must share (d_nope, d_rope)");
  SAD_CHECK(num_tokens >= 0 && window_size >= 0 && padded_topk >= 0, SAD_EINVAL,
            "sparse_mla_decode: negative size");
  SAD_CHECK(num_heads >= 8 && num_heads <= 128 && num_heads % 8 == 0, SAD_EUNSUPPORTED,
            "sparse_mla_decode: num_heads %d unsupported (multiple of 8, <= 128)", num_heads);
  SAD_CHECK(num_tokens < 65536, SAD_EINVAL, "sparse_mla_decode: num_tokens must be < 65536");
  if (num_tokens == 0) return SAD_OK;
  SAD_CHECK(q_bf16 && sparse_indices && sparse_topk_lens && out_bf16, SAD_EINVAL,
            "sparse_mla_decode: NULL pointer argument");
  SAD_CHECK(((uintptr_t)q_bf16 & 15) == 0 && ((uintptr_t)out_bf16 & 15) == 0, SAD_EINVAL,
            "sparse_mla_decode: q and out must be 16-byte aligned");
  SAD_CHECK(((uintptr_t)workspace & 15) == 0, SAD_EINVAL,
            "sparse_mla_decode: workspace must be 16-byte aligned");
  KvDesc s{(const uint8_t*)swa->pool, swa->page_stride, swa->num_pages, swa->block_size};
  KvDesc c{(const uint8_t*)comp->pool, comp->page_stride, comp->num_pages, comp->block_size};
  hipStream_t st = (hipStream_t)stream;
  if (swa->d_nope == 512)
    return launch<512, 64>(q_bf16, num_tokens, num_heads, s, c, sparse_indices, sparse_topk_lens,
                           window_size, padded_topk, softmax_scale, attn_sink, out_bf16, lse,
                           workspace, workspace_bytes, st);
  return launch<128, 32>(q_bf16, num_tokens, num_heads, s, c, sparse_indices, sparse_topk_lens,
                         window_size, padded_topk, softmax_scale, attn_sink, out_bf16, lse,
                         workspace, workspace_bytes, st);
}
