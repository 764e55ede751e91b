// prepare_indexer_q_mxfp4: indexer query -> the scorer's MXFP4 inputs.
//
// [ops] deepseek_v4_prepare_indexer_q_mxfp4 (GPT-J RoPE on the last rope_dim elements,
// then the Hadamard rotation of the bf16 row with scale D^-1/2, then MXFP4 values with one
// ue8m0 scale per 32 elements) and _deepseek_v4_hadamard_rotate; [vllm]
// fused_indexer_q_rope_quant (MXFP4 path: two E2M1 nibbles per byte, the even element in
// the low nibble; weights_out = weights * softmax_scale * head_scale).
//
// One row (token, head) of D elements is held by D/8 lanes, 8 consecutive elements each:
//   * one 16-byte load per lane; a RoPE pair of the tail never straddles two lanes;
//   * the Hadamard butterflies over element-index bits 0..2 run inside the lane, the
//     higher bits across lanes (xor shuffles), in double precision, where every partial
//     sum of bf16 values is exact; the sum is then rounded once to float;
//   * a 32-element scale block is 4 lanes, so its largest magnitude takes two shuffles;
//   * each lane writes its 8 codes as one 4-byte word, every 4th lane its block's scale.
// The kernel streams: 2*D bytes in, D/2 + D/32 bytes out per row, plus the weights.
#include <cmath>

#include "sad_internal.h"

namespace sad {
namespace {

constexpr int kQThreads = 256;

typedef __attribute__((__vector_size__(16))) uint32_t u32x4_t;

__device__ inline float bf16_round(float x) { return bf16_bits_to_f32(f32_to_bf16_bits(x)); }

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

// E2M1 code of a magnitude already divided by the block scale: the count of grid
// midpoints it passes; at a midpoint the even code wins (">" above an even code,
// ">=" above an odd one).
__device__ inline uint32_t e2m1_code(float m) {
  return (uint32_t)(m > 0.25f) + (uint32_t)(m >= 0.75f) + (uint32_t)(m > 1.25f) +
         (uint32_t)(m >= 1.75f) + (uint32_t)(m > 2.5f) + (uint32_t)(m >= 3.5f) +
         (uint32_t)(m > 5.0f);
}

template <int D>
__global__ __launch_bounds__(kQThreads) void prepare_indexer_q_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ positions,
    const float* __restrict__ cos_sin, int max_pos, int rope_dim,
    const float* __restrict__ weights, float softmax_scale, float head_scale, float rot_scale,
    int rows, int heads, uint8_t* __restrict__ q_values, uint8_t* __restrict__ q_scales,
    float* __restrict__ weights_out) {
#pragma clang fp contract(off)
  constexpr int LPR = D / 8;                 // lanes per row
  constexpr int RPB = kQThreads / LPR;       // rows per workgroup
  static_assert(LPR % 4 == 0 && 64 % LPR == 0, "a row is 4..64 lanes of one wave");
  const int sub = threadIdx.x % LPR;
  const int row = (int)blockIdx.x * RPB + (int)threadIdx.x / LPR;
  const bool live = row < rows;
  const int r = live ? row : rows - 1;  // dead lanes still join the shuffles
  const int t = r / heads;

  const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(q + (int64_t)r * D + sub * 8);
  const int pos = positions[t];
  const float w = weights[r];
  const bool ok = pos >= 0 && pos < max_pos;

  float x[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = bf16_bits_to_f32(raw[k] & 0xFFFFu);
    x[2 * k + 1] = bf16_bits_to_f32(raw[k] >> 16);
  }

  // RoPE on the tail, each product and sum a separately rounded float operation (the
  // kernel body is compiled without multiply-add contraction).
  const int nope = D - rope_dim;
  const int d0 = sub * 8;
  if (d0 >= nope) {
    const int i0 = (d0 - nope) >> 1;
    const float* cs = cos_sin + (int64_t)(ok ? pos : 0) * rope_dim;
    const float4 c = *reinterpret_cast<const float4*>(cs + i0);
    const float4 s = *reinterpret_cast<const float4*>(cs + (rope_dim >> 1) + i0);
    const float cv[4] = {c.x, c.y, c.z, c.w};
    const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float e = x[2 * k], o = x[2 * k + 1];
      x[2 * k] = e * cv[k] - o * sv[k];
      x[2 * k + 1] = e * sv[k] + o * cv[k];
    }
  }

  // Hadamard (Sylvester order): at each index bit, low' = low + high, high' = low - high.
  double h[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) h[j] = (double)bf16_round(x[j]);
#pragma unroll
  for (int s = 1; s < 8; s <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j & s) continue;
      const double a = h[j], b = h[j + s];
      h[j] = a + b;
      h[j + s] = a - b;
    }
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) {
    const bool high = (sub & m) != 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double p = __shfl_xor(h[j], m, 64);
      h[j] = high ? p - h[j] : h[j] + p;
    }
  }
  float y[8];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    y[j] = bf16_round((float)h[j] * rot_scale);
    amax = fmaxf(amax, fabsf(y[j]));
  }

  // MXFP4: a 32-element block is lanes 4b .. 4b+3 of the row.
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const int e = block_exponent(amax);
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t code = e2m1_code(ldexpf(fabsf(y[j]), -e)) | (y[j] < 0.0f ? 8u : 0u);
    word |= code << (4 * j);
  }
  if (!live) return;
  *reinterpret_cast<uint32_t*>(q_values + (int64_t)r * (D / 2) + sub * 4) = ok ? word : 0u;
  if ((sub & 3) == 0) q_scales[(int64_t)r * (D / 32) + (sub >> 2)] = ok ? (uint8_t)(e + 127) : 0;
  if (sub == 0) weights_out[r] = ok ? (w * softmax_scale) * head_scale : 0.0f;
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
                ((uintptr_t)q_values & 3) == 0,
            SAD_EINVAL,
            "prepare_indexer_q_mxfp4: index_q and cos_sin_cache must be 16-byte aligned, "
            "q_values 4-byte aligned");
  const int64_t rows = (int64_t)num_tokens * num_idx_heads;
  const int rpb = kQThreads / (idx_dim / 8);
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
