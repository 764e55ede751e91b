// insert_kv_rows: compressed KV rows into the paged FP8 latent cache.
//
// [ops] _write_fp8_ds_mla_cache_rows_capturable and _fp8_ds_mla_cache_rows: the rope
// tail of each row is rotated GPT-J style at the compressed position
// floor(p / ratio) * ratio and stored bf16; the nope part is stored FP8 e4m3 with one
// scale per 64 values, here in the fp32 scale form of these caches:
// scale = fp32(max(amax, 1e-4)) / 448 and code = e4m3(clamp(x / scale, +-448)), both
// divisions correctly rounded fp32.  Row o of page g: values at g*stride + o*(Dn + 2*Dr),
// scales at g*stride + B*(Dn + 2*Dr) + o*4*Dn/64.
//
// The pages' native record (448 + 64) is written with their own rule instead: per 64
// values e = ceil(log2(max(amax, 1e-4) / 448)), computed exactly as the smallest e with
// 448 * 2^e >= max(amax, 1e-4); codes e4m3(x * 2^-e); one scale byte e + 127 per block
// and a zero pad byte (8 per row, after the page's rows).
//
// One wave per row: lane l holds nope values 8l .. 8l+7 (a scale block is 8 lanes, its
// maximum three DPP steps) and, for l < Dr/8, rope values 8l .. 8l+7.
#include "sad_internal.h"

namespace sad {
namespace {

constexpr int kKThreads = 256;
constexpr int kRowsPerWg = kKThreads / 64;

typedef __attribute__((__vector_size__(16))) uint32_t u32x4_t;
typedef short __attribute__((ext_vector_type(2))) s16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// Maximum over the 8 lanes of a half DPP row (quad swaps, then the half-row mirror).
__device__ inline float lane8_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  return fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
}

// Exponent of a native block scale: the smallest e with 448 * 2^e >= a (a >= 1e-4).
// With a = m * 2^k, m in [1, 2) and 448 = 1.75 * 2^8: e = k - 8, plus one when m > 1.75.
__device__ inline int native_exponent(float a) {
  const uint32_t bits = __float_as_uint(a);
  return (int)((bits >> 23) & 0xFFu) - 127 - 8 + ((bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
}

template <int DN, int DR>
__global__ __launch_bounds__(kKThreads) void insert_kv_rows_kernel(
    const uint16_t* __restrict__ rows, const int32_t* __restrict__ positions,
    const float* __restrict__ cos_sin, int max_pos, int ratio, const int32_t* __restrict__ slots,
    int num_rows, uint8_t* __restrict__ pool, int64_t page_stride, int64_t num_pages, int block) {
#pragma clang fp contract(off)
  constexpr int ROWB = DN + 2 * DR;
  constexpr int NSC = DN / 64;
  constexpr bool NATIVE = DN % 128 != 0;
  constexpr int SCB = NATIVE ? 8 : 4 * NSC;  // scale bytes per row
  static_assert(DN / 8 <= 64 && DR / 8 <= 64, "a row fits one wave");
  const int lane = threadIdx.x & 63;
  const int row = (int)blockIdx.x * kRowsPerWg + ((int)threadIdx.x >> 6);
  if (row >= num_rows) return;  // whole waves
  const int slot = slots[row];
  const int pos = positions[row];
  const int cp = pos >= 0 ? (pos / ratio) * ratio : -1;
  if (slot < 0 || (int64_t)(slot / block) >= num_pages || cp < 0 || cp >= max_pos) return;
  uint8_t* page = pool + (int64_t)(slot / block) * page_stride;
  const int ro = slot % block;
  const uint16_t* src = rows + (int64_t)row * (DN + DR);

  if (lane < DN / 8) {
    const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(src + 8 * lane);
    float x[8];
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(raw[k] << 16);
      x[2 * k + 1] = __uint_as_float(raw[k] & 0xFFFF0000u);
      amax = fmaxf(amax, fmaxf(fabsf(x[2 * k]), fabsf(x[2 * k + 1])));
    }
    amax = lane8_max(amax);
    float y[8];
    float cvt_scale = 1.0f;  // the conversion divides by this power of two
    int e = 0;
    if constexpr (NATIVE) {
      e = native_exponent(fmaxf(amax, 1.0e-4f));
      cvt_scale = __uint_as_float((uint32_t)(e + 127) << 23);
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = x[j];  // |x| / 2^e <= 448 by the choice of e
    } else {
      const float scale = fmaxf(amax, 1.0e-4f) / 448.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = fminf(fmaxf(x[j] / scale, -448.0f), 448.0f);
      if ((lane & 7) == 0)
        *reinterpret_cast<float*>(page + (int64_t)block * ROWB + (int64_t)ro * SCB + 4 * (lane >> 3)) = scale;
    }
    s16x2_t lo = {0, 0}, hi = {0, 0};
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, y[0], y[1], cvt_scale, false);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, y[2], y[3], cvt_scale, true);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, y[4], y[5], cvt_scale, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, y[6], y[7], cvt_scale, true);
    *reinterpret_cast<uint2*>(page + (int64_t)ro * ROWB + 8 * lane) =
        make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    if (NATIVE && (lane & 7) == 0)
      page[(int64_t)block * ROWB + (int64_t)ro * SCB + (lane >> 3)] = (uint8_t)min(max(e + 127, 0), 255);
  }
  if (NATIVE && lane == DN / 8) page[(int64_t)block * ROWB + (int64_t)ro * SCB + NSC] = 0;  // pad byte
  if (lane < DR / 8) {
    const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(src + DN + 8 * lane);
    const float* cs = cos_sin + (int64_t)cp * DR;
    const float4 c = *reinterpret_cast<const float4*>(cs + 4 * lane);
    const float4 s = *reinterpret_cast<const float4*>(cs + DR / 2 + 4 * lane);
    const float cv[4] = {c.x, c.y, c.z, c.w};
    const float sv[4] = {s.x, s.y, s.z, s.w};
    u32x4_t outv;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float e = __uint_as_float(raw[k] << 16), o = __uint_as_float(raw[k] & 0xFFFF0000u);
      const float re = e * cv[k] - o * sv[k];
      const float rv = e * sv[k] + o * cv[k];
      outv[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{re, rv}, bf16x2_t));
    }
    *reinterpret_cast<u32x4_t*>(page + (int64_t)ro * ROWB + DN + 16 * lane) = outv;
  }
}

}  // namespace
}  // namespace sad

using namespace sad;

extern "C" int insert_kv_rows(const uint16_t* rows, const int32_t* positions,
                              const float* cos_sin_cache, int32_t max_pos, int32_t compress_ratio,
                              const int32_t* slot_mapping, int32_t num_rows,
                              const sad_kv_cache* cache, void* stream) {
  clear_error();
  const int rc = check_kv_cache(cache, "insert_kv_rows");
  if (rc != SAD_OK) return rc;
  SAD_CHECK(num_rows >= 0 && max_pos >= 0 && compress_ratio >= 1, SAD_EINVAL,
            "insert_kv_rows: bad size");
  if (num_rows == 0) return SAD_OK;
  SAD_CHECK(max_pos >= 1, SAD_EINVAL, "insert_kv_rows: the cos/sin table has no row");
  SAD_CHECK(rows && positions && cos_sin_cache && slot_mapping, SAD_EINVAL,
            "insert_kv_rows: NULL pointer argument");
  SAD_CHECK(((uintptr_t)rows & 15) == 0 && ((uintptr_t)cos_sin_cache & 15) == 0 &&
                ((uintptr_t)cache->pool & 15) == 0 && cache->page_stride % 16 == 0,
            SAD_EINVAL,
            "insert_kv_rows: rows, cos_sin_cache and the pool must be 16-byte aligned, "
            "page_stride a multiple of 16");
  SAD_CHECK((int64_t)num_rows + kRowsPerWg < ((int64_t)1 << 31), SAD_EINVAL,
            "insert_kv_rows: too many rows");
  const unsigned grid = (unsigned)(((int64_t)num_rows + kRowsPerWg - 1) / kRowsPerWg);
  uint8_t* pool = (uint8_t*)const_cast<void*>(cache->pool);
  if (cache->d_nope == 512) {
    hipLaunchKernelGGL((insert_kv_rows_kernel<512, 64>), dim3(grid), dim3(kKThreads), 0,
                       (hipStream_t)stream, rows, positions, cos_sin_cache, max_pos, compress_ratio,
                       slot_mapping, num_rows, pool, cache->page_stride, cache->num_pages,
                       cache->block_size);
  } else if (cache->d_nope == 448) {
    hipLaunchKernelGGL((insert_kv_rows_kernel<448, 64>), dim3(grid), dim3(kKThreads), 0,
                       (hipStream_t)stream, rows, positions, cos_sin_cache, max_pos, compress_ratio,
                       slot_mapping, num_rows, pool, cache->page_stride, cache->num_pages,
                       cache->block_size);
  } else {
    hipLaunchKernelGGL((insert_kv_rows_kernel<128, 32>), dim3(grid), dim3(kKThreads), 0,
                       (hipStream_t)stream, rows, positions, cos_sin_cache, max_pos, compress_ratio,
                       slot_mapping, num_rows, pool, cache->page_stride, cache->num_pages,
                       cache->block_size);
  }
  return check_launch("insert_kv_rows");
}
