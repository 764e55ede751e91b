// inv_rope_fp8_quant: attention output -> the output projection's grouped FP8 input.
//
// [vllm] fused_inv_rope_fp8_quant and [model] _project_attention_output: inverse GPT-J
// RoPE on the last rope_dim elements of every head (the model's attention RoPE has
// is_neox_style=False; the cos/sin table holds the cos half first), heads taken in
// groups, each group's row of D = heads_per_group * head_dim values quantized to FP8
// e4m3 in blocks of 128 with power-of-two scales ([ops] _fp8_e4m3_pow2_bytes:
// scale = 2^ceil(log2(max(amax / 448, 1e-10)))).  Output is group major, [G, T, D].
//
// One 128-value block per 4 lanes (32 values, four 16-byte loads per lane; 64 blocks
// per workgroup): consecutive blocks are consecutive bytes of a group's row, so loads
// and stores are whole lines, and the per-lane index work is spread over 32 values.
// The block maximum takes two DPP quad permutes; the codes come from the gfx950 FP8
// conversion with the block scale (it divides by the scale's power of two and rounds
// to nearest even), two per instruction.
// The kernel streams: 2 bytes in and 1 byte out per value, 4 bytes per block scale.
#include "sad_internal.h"

namespace sad {
namespace {

constexpr int kOThreads = 256;
constexpr int kBlock = 128;                          // values per FP8 scale block
constexpr int kVals = 32;                            // values per lane
constexpr int kLanesPerBlock = kBlock / kVals;       // 4: one quad
constexpr int kBlocksPerWg = kOThreads / kLanesPerBlock;

typedef __attribute__((__vector_size__(16))) uint32_t u32x4_t;
typedef short __attribute__((ext_vector_type(2))) s16x2_t;

__device__ inline float quad_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  return fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
}

// Exponent of the block scale: the smallest e with 448 * 2^e >= a, at least -33.
// With a = m * 2^k, m in [1, 2) and 448 = 1.75 * 2^8: e = k - 8, plus one when m > 1.75.
__device__ inline int fp8_block_exponent(float a) {
  const uint32_t bits = __float_as_uint(a);
  const int biased = (int)((bits >> 23) & 0xFFu);
  if (biased == 0) return -33;
  const int e = (biased - 127) - 8 + ((bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return max(e, -33);
}

__global__ __launch_bounds__(kOThreads) void inv_rope_fp8_kernel(
    const uint16_t* __restrict__ o, const int32_t* __restrict__ positions,
    const float* __restrict__ cos_sin, int max_pos, int rope_dim, int T, int H, int Dh,
    int hpg, int nblk, int total_blocks, uint8_t* __restrict__ out, float* __restrict__ scales) {
#pragma clang fp contract(off)
  const int lb = threadIdx.x & 3;  // lane within the block's quad
  const int blk = (int)blockIdx.x * kBlocksPerWg + ((int)threadIdx.x >> 2);
  const bool live = blk < total_blocks;
  const int b = live ? blk : total_blocks - 1;  // dead lanes still join the DPP steps
  const int row = b / nblk;                     // g * T + t
  const int k = b - row * nblk;
  const int g = row / T;
  const int t = row - g * T;
  const int d_row = k * kBlock + kVals * lb;  // position in the group's row of D values
  const int hl = d_row / Dh;
  const int dh0 = d_row - hl * Dh;  // head dim of the lane's first value

  const uint16_t* src = o + ((int64_t)t * H + (int64_t)g * hpg) * Dh + d_row;
  u32x4_t raw[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) raw[q] = *reinterpret_cast<const u32x4_t*>(src + 8 * q);
  const int pos = positions[t];
  const bool ok = pos >= 0 && pos < max_pos;
  const int nope = Dh - rope_dim;
  const float* cs = cos_sin + (int64_t)(ok ? pos : 0) * rope_dim;
  // Each 8-value group is all head or all tail (head_dim and rope_dim are multiples of
  // 8); a lane's 32 values may run into the next head.
  bool tail[4];
  float4 c[4], s[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int dh = dh0 + 8 * q;
    dh = dh >= Dh ? dh - Dh : dh;
    tail[q] = dh >= nope;
    const int i0 = max(dh - nope, 0) >> 1;  // clamped: head groups read pair 0 and ignore it
    c[q] = *reinterpret_cast<const float4*>(cs + i0);
    s[q] = *reinterpret_cast<const float4*>(cs + (rope_dim >> 1) + i0);
  }

  float x[kVals];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[8 * q + 2 * w] = __uint_as_float(raw[q][w] << 16);
      x[8 * q + 2 * w + 1] = __uint_as_float(raw[q][w] & 0xFFFF0000u);
    }
  // Inverse RoPE (rotation by -angle) on the tail groups.
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float cv[4] = {c[q].x, c[q].y, c[q].z, c[q].w};
    const float sv[4] = {s[q].x, s[q].y, s[q].z, s[q].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float e = x[8 * q + 2 * w], od = x[8 * q + 2 * w + 1];
      const float re = e * cv[w] + od * sv[w];
      const float ro = od * cv[w] - e * sv[w];
      x[8 * q + 2 * w] = tail[q] ? re : e;
      x[8 * q + 2 * w + 1] = tail[q] ? ro : od;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < kVals; ++j) amax = fmaxf(amax, fabsf(x[j]));
  amax = quad_max(amax);
  const int e = fp8_block_exponent(amax);
  const float scale = __uint_as_float((uint32_t)(e + 127) << 23);
  uint32_t words[kVals / 4];
#pragma unroll
  for (int wd = 0; wd < kVals / 4; ++wd) {
    s16x2_t v = {0, 0};
    v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v, x[4 * wd], x[4 * wd + 1], scale, false);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v, x[4 * wd + 2], x[4 * wd + 3], scale, true);
    words[wd] = ok ? __builtin_bit_cast(uint32_t, v) : 0u;
  }
  if (!live) return;
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + (int64_t)row * (nblk * kBlock) + d_row);
  dst[0] = u32x4_t{words[0], words[1], words[2], words[3]};
  dst[1] = u32x4_t{words[4], words[5], words[6], words[7]};
  if (lb == 0) scales[(int64_t)row * nblk + k] = ok ? scale : 0.0f;
}

}  // namespace
}  // namespace sad

using namespace sad;

extern "C" int inv_rope_fp8_quant(const uint16_t* attn_out, const int32_t* positions,
                                  const float* cos_sin_cache, int32_t max_pos, int32_t rope_dim,
                                  int32_t num_tokens, int32_t num_heads, int32_t head_dim,
                                  int32_t n_groups, uint8_t* out_fp8, float* out_scales,
                                  void* stream) {
  clear_error();
  SAD_CHECK(num_tokens >= 0 && num_heads >= 1 && head_dim >= 1 && n_groups >= 1 && max_pos >= 0,
            SAD_EINVAL, "inv_rope_fp8_quant: bad size");
  SAD_CHECK(num_heads % n_groups == 0, SAD_EINVAL,
            "inv_rope_fp8_quant: num_heads (%d) must be a multiple of n_groups (%d)", num_heads,
            n_groups);
  SAD_CHECK(head_dim % 8 == 0 && head_dim >= 32 && rope_dim % 8 == 0 && rope_dim > 0 &&
                rope_dim <= head_dim,
            SAD_EINVAL,
            "inv_rope_fp8_quant: head_dim (>= 32) and rope_dim must be multiples of 8, "
            "0 < rope_dim <= head_dim (got %d, %d)",
            head_dim, rope_dim);
  const int64_t D = (int64_t)(num_heads / n_groups) * head_dim;
  SAD_CHECK(D % kBlock == 0, SAD_EINVAL,
            "inv_rope_fp8_quant: heads_per_group * head_dim must be a multiple of 128");
  if (num_tokens == 0) return SAD_OK;
  SAD_CHECK(max_pos >= 1, SAD_EINVAL, "inv_rope_fp8_quant: the cos/sin table has no row");
  SAD_CHECK(attn_out && positions && cos_sin_cache && out_fp8 && out_scales, SAD_EINVAL,
            "inv_rope_fp8_quant: NULL pointer argument");
  SAD_CHECK(((uintptr_t)attn_out & 15) == 0 && ((uintptr_t)cos_sin_cache & 15) == 0 &&
                ((uintptr_t)out_fp8 & 15) == 0,
            SAD_EINVAL,
            "inv_rope_fp8_quant: attn_out, cos_sin_cache and out_fp8 must be 16-byte aligned");
  const int64_t nblk = D / kBlock;
  const int64_t total = (int64_t)num_tokens * n_groups * nblk;
  SAD_CHECK(total + kBlocksPerWg < ((int64_t)1 << 31), SAD_EINVAL,
            "inv_rope_fp8_quant: too many blocks");
  const int64_t grid = (total + kBlocksPerWg - 1) / kBlocksPerWg;
  hipLaunchKernelGGL(inv_rope_fp8_kernel, dim3((unsigned)grid), dim3(kOThreads), 0,
                     (hipStream_t)stream, attn_out, positions, cos_sin_cache, max_pos, rope_dim,
                     num_tokens, num_heads, head_dim, num_heads / n_groups, (int)nblk, (int)total,
                     out_fp8, out_scales);
  return check_launch("inv_rope_fp8_quant");
}
