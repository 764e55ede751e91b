// prepare_indexer_q_mxfp4: indexer query -> the scorer's MXFP4 inputs.
//
// [ops] deepseek_v4_prepare_indexer_q_mxfp4 (GPT-J RoPE on the last rope_dim elements,
// then the Hadamard rotation of the bf16 row with scale D^-1/2, then MXFP4 values with one
// ue8m0 scale per 32 elements) and _deepseek_v4_hadamard_rotate; [vllm]
// fused_indexer_q_rope_quant (MXFP4 path: two E2M1 nibbles per byte, the even element in
// the low nibble; weights_out = weights * softmax_scale * head_scale).
//
// One row (token, head) of D elements is held by the 4 lanes of a quad, D/4 consecutive
// elements each (16 rows per wave):
//   * 16-byte loads; a RoPE pair of the tail never straddles two lanes;
//   * the Hadamard transform is the fp32 radix-2 fast transform, index bit 0 first: the
//     bits inside a lane's slice in registers, the two top bits across the quad (DPP
//     quad permutes, no LDS);
//   * a 32-element scale block lies in one lane (D = 128) or a lane pair (D = 64);
//   * codes come from the gfx950 FP4 conversion of bf16 pairs with the block scale (it
//     divides by the scale's power of two, rounds to nearest even, saturates and copies
//     the sign bit), two elements per instruction; each lane stores its codes as one 16-
//     or 8-byte word.
// The kernel streams: 2*D bytes in, D/2 + D/32 bytes out per row, plus the weights.
#include <cmath>

#include "sad_internal.h"

namespace sad {
namespace {

constexpr int kQThreads = 256;
constexpr int kRowsPerBlock = kQThreads / 4;

typedef __attribute__((__vector_size__(16))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// Two floats rounded to bf16 (nearest even), packed (a in the low half).
__device__ inline uint32_t bf16_pack(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Both floats rounded to bf16 (nearest even) and widened back.
__device__ inline void bf16_round2(float& a, float& b) {
  const uint32_t u = bf16_pack(a, b);
  a = __uint_as_float(u << 16);
  b = __uint_as_float(u & 0xFFFF0000u);
}

// Shared exponent of a block whose largest magnitude is `a` (a bf16 value held in a
// float): the smallest e with 6 * 2^e >= a, -127 for a zero (or subnormal) block.
// With a = m * 2^k, m in [1, 2): 6 * 2^e >= a  <=>  2^(e-k) >= m / 6, which is
// 2^-2 for m <= 1.5 and 2^-1 above.
__device__ inline int block_exponent(float a) {
  const uint32_t bits = __float_as_uint(a);
  const int biased = (int)((bits >> 23) & 0xFFu);
  if (biased == 0) return -127;
  const int e = (biased - 127) - ((bits & 0x7FFFFFu) <= 0x400000u ? 2 : 1);
  return min(max(e, -127), 127);
}

// Lane l of a quad reads lane l ^ M (M = 1 or 2) with a DPP quad permute.
template <int M>
__device__ inline uint32_t quad_xor(uint32_t v) {
  constexpr int ctrl = M == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, ctrl, 0xF, 0xF, false);
}

template <int M>
__device__ inline float quad_xor(float v) {
  return __uint_as_float(quad_xor<M>(__float_as_uint(v)));
}

// The lane's part of one row's transform: RoPE on the tail at cos/sin row `cs`, bf16,
// the fp32 fast Hadamard transform (Sylvester order), the scale and bf16, and the
// MXFP4 codes of the lane's D/4 values (word[D/32], the even value in the low nibble).
// Returns the exponent of the lane's scale block.  All four lanes of the quad call it
// (the top transform stages are quad permutes).
template <int D>
__device__ inline int quad_row_mxfp4(const uint16_t* __restrict__ row, const float* __restrict__ cs,
                                     int rope_dim, int sub, float rot_scale, uint32_t* word) {
#pragma clang fp contract(off)
  constexpr int EPL = D / 4;   // elements per lane
  constexpr int NG = EPL / 8;  // 8-element (16-byte) groups per lane
  static_assert(EPL == 16 || EPL == 32, "a lane holds 16 or 32 elements");
  const int d_lane = sub * EPL;
  const int nope = D - rope_dim;

  // Every load of the lane is issued before the first use.
  u32x4_t raw[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) raw[g] = *reinterpret_cast<const u32x4_t*>(row + d_lane + 8 * g);
  float4 cg[NG], sg[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int i0 = max(d_lane + 8 * g - nope, 0) >> 1;  // clamped: groups of the head read pair 0
    cg[g] = *reinterpret_cast<const float4*>(cs + i0);
    sg[g] = *reinterpret_cast<const float4*>(cs + (rope_dim >> 1) + i0);
  }

  float x[EPL];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[8 * g + 2 * k] = __uint_as_float(raw[g][k] << 16);
      x[8 * g + 2 * k + 1] = __uint_as_float(raw[g][k] & 0xFFFF0000u);
    }

  // RoPE on the tail (a group of 8 elements is all head or all tail), each product and
  // sum a separately rounded float operation; then the row is rounded to bf16.
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const bool tail = d_lane + 8 * g >= nope;
    const float cv[4] = {cg[g].x, cg[g].y, cg[g].z, cg[g].w};
    const float sv[4] = {sg[g].x, sg[g].y, sg[g].z, sg[g].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float e = x[8 * g + 2 * k], o = x[8 * g + 2 * k + 1];
      const float re = e * cv[k] - o * sv[k];
      const float ro = e * sv[k] + o * cv[k];
      x[8 * g + 2 * k] = tail ? re : e;
      x[8 * g + 2 * k + 1] = tail ? ro : o;
    }
  }
#pragma unroll
  for (int j = 0; j < EPL; j += 2) bf16_round2(x[j], x[j + 1]);

  // Hadamard (Sylvester order), fp32: at each index bit, low' = low + high and
  // high' = low - high.  Across the quad a lane gets its partner's value p and forms
  // p + h (low lane) or p - h (high lane) as one exactly rounded fma with +-1.
  float* h = x;
#pragma unroll
  for (int s = 1; s < EPL; s <<= 1) {
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      if (j & s) continue;
      const float a = h[j], b = h[j + s];
      h[j] = a + b;
      h[j + s] = a - b;
    }
  }
  {
    const float s1 = (sub & 1) ? -1.0f : 1.0f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) h[j] = __builtin_fmaf(h[j], s1, quad_xor<1>(h[j]));
    const float s2 = (sub & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) h[j] = __builtin_fmaf(h[j], s2, quad_xor<2>(h[j]));
  }
  // Scale, round to bf16 (packed pairs), and the block's largest magnitude from the
  // bf16 bits (magnitudes order like unsigned integers).
  uint32_t yb[EPL / 2];
  uint32_t mx = 0;
#pragma unroll
  for (int j = 0; j < EPL; j += 2) {
    yb[j / 2] = bf16_pack(h[j] * rot_scale, h[j + 1] * rot_scale);
    const uint32_t m = yb[j / 2] & 0x7FFF7FFFu;
    mx = max(mx, max(m & 0xFFFFu, m >> 16));
  }
  if (EPL == 16) mx = max(mx, quad_xor<1>(mx));  // D = 64: a block is a lane pair

  // MXFP4 codes: the conversion divides by the scale's power of two (exponent field
  // e + 127; 0 means 2^-127), rounds to nearest even, saturates, copies the sign bit.
  const int e = block_exponent(__uint_as_float(mx << 16));
  const float scale = __uint_as_float((uint32_t)(e + 127) << 23);
#pragma unroll
  for (int wd = 0; wd < EPL / 8; ++wd) {
    const uint32_t* p = yb + 4 * wd;
    uint32_t v = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(bf16x2_t, p[0]), scale, 0);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(v, __builtin_bit_cast(bf16x2_t, p[1]), scale, 1);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(v, __builtin_bit_cast(bf16x2_t, p[2]), scale, 2);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(v, __builtin_bit_cast(bf16x2_t, p[3]), scale, 3);
    word[wd] = v;
  }
  return e;
}

// The lane's codes (D/4 values) and, from one lane per 32-value block, its scale byte.
template <int D>
__device__ inline void store_quad_row(uint8_t* vout, uint8_t* sout, int sub, const uint32_t* word,
                                      int e, bool ok) {
  constexpr int EPL = D / 4;
  uint8_t* v = vout + sub * (EPL / 2);
  if constexpr (EPL == 32) {
    *reinterpret_cast<u32x4_t*>(v) = ok ? u32x4_t{word[0], word[1], word[2], word[3]} : u32x4_t{0, 0, 0, 0};
    sout[sub] = ok ? (uint8_t)(e + 127) : 0;
  } else {
    *reinterpret_cast<uint2*>(v) = ok ? make_uint2(word[0], word[1]) : make_uint2(0u, 0u);
    if ((sub & 1) == 0) sout[sub >> 1] = ok ? (uint8_t)(e + 127) : 0;
  }
}

template <int D>
__global__ __launch_bounds__(kQThreads) void prepare_indexer_q_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ positions,
    const float* __restrict__ cos_sin, int max_pos, int rope_dim,
    const float* __restrict__ weights, float softmax_scale, float head_scale, float rot_scale,
    int rows, int heads, uint8_t* __restrict__ q_values, uint8_t* __restrict__ q_scales,
    float* __restrict__ weights_out) {
#pragma clang fp contract(off)
  const int sub = threadIdx.x & 3;
  const int row = (int)blockIdx.x * kRowsPerBlock + ((int)threadIdx.x >> 2);
  const bool live = row < rows;
  const int r = live ? row : rows - 1;  // dead lanes still join the quad permutes
  const int t = r / heads;
  const int pos = positions[t];
  const float w = weights[r];
  const bool ok = pos >= 0 && pos < max_pos;
  uint32_t word[D / 32];
  const int e = quad_row_mxfp4<D>(q + (int64_t)r * D, cos_sin + (int64_t)(ok ? pos : 0) * rope_dim,
                                  rope_dim, sub, rot_scale, word);
  if (!live) return;
  store_quad_row<D>(q_values + (int64_t)r * (D / 2), q_scales + (int64_t)r * (D / 32), sub, word, e, ok);
  if (sub == 0) weights_out[r] = ok ? (w * softmax_scale) * head_scale : 0.0f;
}

// Key rows written into the paged MXFP4 cache at their slots (RoPE at the compressed
// position); a negative slot, a page past the pool or a position outside the table
// writes nothing.
template <int D>
__global__ __launch_bounds__(kQThreads) void insert_index_keys_kernel(
    const uint16_t* __restrict__ keys, const int32_t* __restrict__ positions,
    const float* __restrict__ cos_sin, int max_pos, int rope_dim, int ratio, float rot_scale,
    const int32_t* __restrict__ slots, int rows, uint8_t* __restrict__ pool, int64_t page_stride,
    int64_t num_pages, int block) {
  const int sub = threadIdx.x & 3;
  const int row = (int)blockIdx.x * kRowsPerBlock + ((int)threadIdx.x >> 2);
  const bool live = row < rows;
  const int r = live ? row : rows - 1;
  const int slot = slots[r];
  const int pos = positions[r];
  const int cp = pos >= 0 ? (pos / ratio) * ratio : -1;
  const bool ok = slot >= 0 && (int64_t)(slot / block) < num_pages && cp >= 0 && cp < max_pos;
  uint32_t word[D / 32];
  const int e = quad_row_mxfp4<D>(keys + (int64_t)r * D, cos_sin + (int64_t)(cp >= 0 && cp < max_pos ? cp : 0) * rope_dim,
                                  rope_dim, sub, rot_scale, word);
  if (!live || !ok) return;
  uint8_t* page = pool + (int64_t)(slot / block) * page_stride;
  const int ro = slot % block;
  store_quad_row<D>(page + (int64_t)ro * (D / 2), page + (int64_t)block * (D / 2) + (int64_t)ro * (D / 32),
                    sub, word, e, true);
}

}  // namespace
}  // namespace sad

using namespace sad;

extern "C" int prepare_indexer_q_mxfp4(const uint16_t* index_q, const int32_t* positions,
                                       const float* cos_sin_cache, int32_t max_pos,
                                       int32_t rope_dim, const float* weights,
                                       float softmax_scale, float head_scale,
                                       int32_t num_tokens, int32_t num_idx_heads,
                                       int32_t idx_dim, uint8_t* q_values, uint8_t* q_scales,
                                       float* weights_out, void* stream) {
  clear_error();
  SAD_CHECK(num_tokens >= 0 && num_idx_heads >= 0 && max_pos >= 0, SAD_EINVAL,
            "prepare_indexer_q_mxfp4: negative size");
  SAD_CHECK(idx_dim == 64 || idx_dim == 128, SAD_EUNSUPPORTED,
            "prepare_indexer_q_mxfp4: idx_dim must be 64 or 128 (got %d)", idx_dim);
  SAD_CHECK(rope_dim > 0 && rope_dim < idx_dim && rope_dim % 8 == 0, SAD_EINVAL,
            "prepare_indexer_q_mxfp4: rope_dim must be a multiple of 8 in (0, idx_dim) (got %d)",
            rope_dim);
  if (num_tokens == 0 || num_idx_heads == 0) return SAD_OK;
  SAD_CHECK(max_pos >= 1, SAD_EINVAL, "prepare_indexer_q_mxfp4: the cos/sin table has no row");
  SAD_CHECK(index_q && positions && cos_sin_cache && weights && q_values && q_scales &&
                weights_out,
            SAD_EINVAL, "prepare_indexer_q_mxfp4: NULL pointer argument");
  SAD_CHECK(((uintptr_t)index_q & 15) == 0 && ((uintptr_t)cos_sin_cache & 15) == 0 &&
                ((uintptr_t)q_values & 15) == 0,
            SAD_EINVAL,
            "prepare_indexer_q_mxfp4: index_q and cos_sin_cache must be 16-byte aligned, "
            "q_values 16-byte aligned");
  const int64_t rows = (int64_t)num_tokens * num_idx_heads;
  const int rpb = kRowsPerBlock;
  const int64_t blocks = (rows + rpb - 1) / rpb;
  SAD_CHECK(rows + rpb < ((int64_t)1 << 31), SAD_EINVAL,
            "prepare_indexer_q_mxfp4: num_tokens * num_idx_heads must be below 2^31");
  const float rot_scale = (float)(1.0 / std::sqrt((double)idx_dim));
  if (idx_dim == 128) {
    hipLaunchKernelGGL((prepare_indexer_q_kernel<128>), dim3((unsigned)blocks), dim3(kQThreads), 0,
                       (hipStream_t)stream, index_q, positions, cos_sin_cache, max_pos, rope_dim,
                       weights, softmax_scale, head_scale, rot_scale, (int)rows, num_idx_heads,
                       q_values, q_scales, weights_out);
  } else {
    hipLaunchKernelGGL((prepare_indexer_q_kernel<64>), dim3((unsigned)blocks), dim3(kQThreads), 0,
                       (hipStream_t)stream, index_q, positions, cos_sin_cache, max_pos, rope_dim,
                       weights, softmax_scale, head_scale, rot_scale, (int)rows, num_idx_heads,
                       q_values, q_scales, weights_out);
  }
  return check_launch("prepare_indexer_q_mxfp4");
}

extern "C" int insert_index_keys(const uint16_t* keys, const int32_t* positions,
                                 const float* cos_sin_cache, int32_t max_pos, int32_t rope_dim,
                                 int32_t compress_ratio, const int32_t* slot_mapping,
                                 int32_t num_rows, const sad_mxfp4_cache* cache, void* stream) {
  clear_error();
  SAD_CHECK(cache != nullptr, SAD_EINVAL, "insert_index_keys: cache is NULL");
  const int D = cache->dim;
  SAD_CHECK(D == 64 || D == 128, SAD_EUNSUPPORTED,
            "insert_index_keys: dim must be 64 or 128 (got %d)", D);
  SAD_CHECK(cache->block_size == 16 || cache->block_size == 64, SAD_EUNSUPPORTED,
            "insert_index_keys: block_size must be 16 or 64 (got %d)", cache->block_size);
  SAD_CHECK(num_rows >= 0 && max_pos >= 0 && compress_ratio >= 1 && cache->num_pages >= 0,
            SAD_EINVAL, "insert_index_keys: bad size");
  SAD_CHECK(rope_dim > 0 && rope_dim < D && rope_dim % 8 == 0, SAD_EINVAL,
            "insert_index_keys: rope_dim must be a multiple of 8 in (0, dim) (got %d)", rope_dim);
  SAD_CHECK(cache->page_stride >= (int64_t)cache->block_size * (D / 2 + D / 32), SAD_EINVAL,
            "insert_index_keys: page_stride below block_size * (dim/2 + dim/32)");
  if (num_rows == 0) return SAD_OK;
  SAD_CHECK(max_pos >= 1, SAD_EINVAL, "insert_index_keys: the cos/sin table has no row");
  SAD_CHECK(keys && positions && cos_sin_cache && slot_mapping && cache->pool, SAD_EINVAL,
            "insert_index_keys: NULL pointer argument");
  SAD_CHECK(((uintptr_t)keys & 15) == 0 && ((uintptr_t)cos_sin_cache & 15) == 0 &&
                ((uintptr_t)cache->pool & 15) == 0 && cache->page_stride % 16 == 0,
            SAD_EINVAL,
            "insert_index_keys: keys, cos_sin_cache and the pool must be 16-byte aligned, "
            "page_stride a multiple of 16");
  SAD_CHECK(cache->num_pages * (int64_t)cache->block_size <= INT32_MAX, SAD_EINVAL,
            "insert_index_keys: pool too large for int32 slots");
  SAD_CHECK((int64_t)num_rows + kRowsPerBlock < ((int64_t)1 << 31), SAD_EINVAL,
            "insert_index_keys: too many rows");
  const unsigned grid = (unsigned)(((int64_t)num_rows + kRowsPerBlock - 1) / kRowsPerBlock);
  const float rot_scale = (float)(1.0 / std::sqrt((double)D));
  uint8_t* pool = (uint8_t*)const_cast<void*>(cache->pool);
  if (D == 128) {
    hipLaunchKernelGGL((insert_index_keys_kernel<128>), dim3(grid), dim3(kQThreads), 0,
                       (hipStream_t)stream, keys, positions, cos_sin_cache, max_pos, rope_dim,
                       compress_ratio, rot_scale, slot_mapping, num_rows, pool, cache->page_stride,
                       cache->num_pages, cache->block_size);
  } else {
    hipLaunchKernelGGL((insert_index_keys_kernel<64>), dim3(grid), dim3(kQThreads), 0,
                       (hipStream_t)stream, keys, positions, cos_sin_cache, max_pos, rope_dim,
                       compress_ratio, rot_scale, slot_mapping, num_rows, pool, cache->page_stride,
                       cache->num_pages, cache->block_size);
  }
  return check_launch("insert_index_keys");
}
