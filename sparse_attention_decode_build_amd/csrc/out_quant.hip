// inv_rope_fp8_quant: attention output -> the output projection's grouped FP8 input.
//
// [vllm] fused_inv_rope_fp8_quant and [model] _project_attention_output: inverse GPT-J
// RoPE on the last rope_dim elements of every head (the model's attention RoPE has
// is_neox_style=False; the cos/sin table holds the cos half first), heads taken in
// groups, each group's row of D = heads_per_group * head_dim values quantized to FP8
// e4m3 in blocks of 128 with power-of-two scales ([ops] _fp8_e4m3_pow2_bytes:
// scale = 2^ceil(log2(max(amax / 448, 1e-10)))).  Output is group major, [G, T, D].
//
// One 128-value block per 16 lanes (8 values, one 16-byte load per lane; 16 blocks
// per workgroup): consecutive blocks are consecutive bytes of a group's row, so loads
// and stores are whole lines.  The block maximum takes four DPP steps inside the
// 16-lane row; the codes come from the gfx950 FP8 conversion with the block scale (it
// divides by the scale's power of two and rounds to nearest even), two per instruction.
// The kernel streams: 2 bytes in and 1 byte out per value, 4 bytes per block scale.
#include "sad_internal.h"

namespace sad {
namespace {

constexpr int kOThreads = 256;
constexpr int kBlock = 128;                        // values per FP8 scale block
constexpr int kBlocksPerWg = kOThreads / 16;       // one block per 16 lanes

typedef __attribute__((__vector_size__(16))) uint32_t u32x4_t;
typedef short __attribute__((ext_vector_type(2))) s16x2_t;

// Maximum over the 16 lanes of a DPP row (quad swaps, then half-row and row mirrors).
__device__ inline float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
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
  const int lb = threadIdx.x & 15;  // lane within the block
  const int blk = (int)blockIdx.x * kBlocksPerWg + ((int)threadIdx.x >> 4);
  const bool live = blk < total_blocks;
  const int b = live ? blk : total_blocks - 1;  // dead lanes still join the DPP steps
  const int row = b / nblk;                     // g * T + t
  const int k = b - row * nblk;
  const int g = row / T;
  const int t = row - g * T;
  const int d_row = k * kBlock + 8 * lb;  // position in the group's row of D values
  const int hl = d_row / Dh;
  const int dh = d_row - hl * Dh;  // head dim of the lane's first value

  const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(
      o + ((int64_t)t * H + (int64_t)g * hpg) * Dh + d_row);
  const int pos = positions[t];
  const bool ok = pos >= 0 && pos < max_pos;
  const int nope = Dh - rope_dim;
  const int i0 = max(dh - nope, 0) >> 1;  // clamped: head values read pair 0 and ignore it
  const float* cs = cos_sin + (int64_t)(ok ? pos : 0) * rope_dim;
  const float4 c = *reinterpret_cast<const float4*>(cs + i0);
  const float4 s = *reinterpret_cast<const float4*>(cs + (rope_dim >> 1) + i0);

  float x[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    x[2 * q] = __uint_as_float(raw[q] << 16);
    x[2 * q + 1] = __uint_as_float(raw[q] & 0xFFFF0000u);
  }
  // Inverse RoPE (rotation by -angle) on the tail; 8 values are all head or all tail.
  const bool tail = dh >= nope;
  const float cv[4] = {c.x, c.y, c.z, c.w};
  const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float e = x[2 * q], od = x[2 * q + 1];
    const float re = e * cv[q] + od * sv[q];
    const float ro = od * cv[q] - e * sv[q];
    x[2 * q] = tail ? re : e;
    x[2 * q + 1] = tail ? ro : od;
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
  amax = row16_max(amax);
  const int e = fp8_block_exponent(amax);
  const float scale = __uint_as_float((uint32_t)(e + 127) << 23);
  s16x2_t lo = {0, 0}, hi = {0, 0};
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, x[0], x[1], scale, false);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, x[2], x[3], scale, true);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, x[4], x[5], scale, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, x[6], x[7], scale, true);
  if (!live) return;
  const uint2 codes = ok ? make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi))
                         : make_uint2(0u, 0u);
  *reinterpret_cast<uint2*>(out + (int64_t)row * (nblk * kBlock) + d_row) = codes;
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
  SAD_CHECK(head_dim % 8 == 0 && rope_dim % 8 == 0 && rope_dim > 0 && rope_dim <= head_dim,
            SAD_EINVAL,
            "inv_rope_fp8_quant: head_dim and rope_dim must be multiples of 8, 0 < rope_dim <= "
            "head_dim (got %d, %d)",
            head_dim, rope_dim);
  const int64_t D = (int64_t)(num_heads / n_groups) * head_dim;
  SAD_CHECK(D % kBlock == 0, SAD_EINVAL,
            "inv_rope_fp8_quant: heads_per_group * head_dim must be a multiple of 128");
  if (num_tokens == 0) return SAD_OK;
  SAD_CHECK(max_pos >= 1, SAD_EINVAL, "inv_rope_fp8_quant: the cos/sin table has no row");
  SAD_CHECK(attn_out && positions && cos_sin_cache && out_fp8 && out_scales, SAD_EINVAL,
            "inv_rope_fp8_quant: NULL pointer argument");
  SAD_CHECK(((uintptr_t)attn_out & 15) == 0 && ((uintptr_t)cos_sin_cache & 15) == 0 &&
                ((uintptr_t)out_fp8 & 7) == 0,
            SAD_EINVAL,
            "inv_rope_fp8_quant: attn_out and cos_sin_cache must be 16-byte aligned, out_fp8 "
            "8-byte aligned");
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
