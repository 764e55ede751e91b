// gather_dequant_kv: dequantized bf16 rows of every attended column (bit-exact).
//
// [ops] dequantize_deepseek_v4_fp8_ds_mla_cache: row o of page g has its values at
// g*stride + o*(Dn + 2*Dr) (Dn e4m3fn bytes, then Dr bf16) and its Dn/64 fp32 scales at
// g*stride + B*(Dn + 2*Dr) + o*4*(Dn/64); nope[d] = bf16_rne(float(e4m3) * scale[d/64]),
// rope copied, slot -1 -> zero row.  One wave per output row: lanes read 8 (or 2)
// consecutive FP8 bytes each, so a row's nope values are one coalesced 512-byte read.
#include "sad_internal.h"

namespace sad {
namespace {

constexpr int kThreads = 256;

// 2^(b - 127) for a ue8m0 byte (byte 0 is the subnormal 2^-127).
__device__ inline float ue8m0_scale(uint32_t b) {
  return b != 0 ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

template <int DN, int DR>
__global__ __launch_bounds__(kThreads) void gather_dequant_kernel(
    KvDesc swa, KvDesc comp, const int32_t* __restrict__ si, const int32_t* __restrict__ lens,
    int64_t num_rows, int window, int padded, uint16_t* __restrict__ out) {
  constexpr int ROWB = DN + 2 * DR;       // value bytes per row
  constexpr bool NATIVE = DN % 128 != 0;  // the native record (448 + 64): ue8m0 scale bytes
  constexpr int EPL = NATIVE ? 8 : DN / 64;  // FP8 elements per lane (8 or 2)
  constexpr int NLANES = DN / EPL;           // lanes holding nope values
  constexpr int SCB = NATIVE ? 8 : 4 * (DN / 64);  // scale bytes per row
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (r >= num_rows) return;
  const int width = window + padded;
  const int64_t t = r / width;
  const int c = (int)(r - t * width);
  int slot = si[r];
  const bool is_comp = c >= window;
  if (is_comp) {
    const int n = lens[t];
    if (c - window >= n) slot = -1;
  }
  const KvDesc kv = is_comp ? comp : swa;
  const bool valid = slot_ok(slot, kv.block, kv.num_pages);
  uint16_t* o = out + r * (DN + DR);

  uint16_t res[EPL];
  if (valid) {
    const int page = slot / kv.block;
    const int ro = slot - page * kv.block;
    const uint8_t* pg = kv.pool + (int64_t)page * kv.stride;
    const uint8_t* vals = pg + (int64_t)ro * ROWB;
    const uint8_t* srow = pg + (int64_t)kv.block * ROWB + (int64_t)ro * SCB;
    if (lane < NLANES) {
      float sc;
      if constexpr (NATIVE)
        sc = ue8m0_scale(srow[(lane * EPL) / 64]);
      else
        sc = reinterpret_cast<const float*>(srow)[(lane * EPL) / 64];
      if constexpr (EPL == 8) {
        const uint2 w = *reinterpret_cast<const uint2*>(vals + lane * 8);
        res[0] = f32_to_bf16_bits(e4m3_to_f32<0>(w.x) * sc);
        res[1] = f32_to_bf16_bits(e4m3_to_f32<1>(w.x) * sc);
        res[2] = f32_to_bf16_bits(e4m3_to_f32<2>(w.x) * sc);
        res[3] = f32_to_bf16_bits(e4m3_to_f32<3>(w.x) * sc);
        res[4] = f32_to_bf16_bits(e4m3_to_f32<0>(w.y) * sc);
        res[5] = f32_to_bf16_bits(e4m3_to_f32<1>(w.y) * sc);
        res[6] = f32_to_bf16_bits(e4m3_to_f32<2>(w.y) * sc);
        res[7] = f32_to_bf16_bits(e4m3_to_f32<3>(w.y) * sc);
      } else {
        const uint32_t w = *reinterpret_cast<const uint16_t*>(vals + lane * 2);
        res[0] = f32_to_bf16_bits(e4m3_to_f32<0>(w) * sc);
        res[1] = f32_to_bf16_bits(e4m3_to_f32<1>(w) * sc);
      }
    }
    // rope: DR bf16 = 2*DR bytes copied by the first DR/2 lanes (4 bytes each)
    if (lane < DR / 2) {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(vals + DN + lane * 4);
      *reinterpret_cast<uint32_t*>(o + DN + lane * 2) = v;
    }
  } else {
#pragma unroll
    for (int i = 0; i < EPL; ++i) res[i] = 0;
    if (lane < DR / 2) *reinterpret_cast<uint32_t*>(o + DN + lane * 2) = 0u;
  }
  if (lane >= NLANES) return;
  if constexpr (EPL == 8) {
    uint4 v;
    v.x = res[0] | ((uint32_t)res[1] << 16);
    v.y = res[2] | ((uint32_t)res[3] << 16);
    v.z = res[4] | ((uint32_t)res[5] << 16);
    v.w = res[6] | ((uint32_t)res[7] << 16);
    *reinterpret_cast<uint4*>(o + lane * 8) = v;
  } else {
    *reinterpret_cast<uint32_t*>(o + lane * 2) = res[0] | ((uint32_t)res[1] << 16);
  }
}

}  // namespace

int kv_scale_bytes(const sad_kv_cache* c) {
  return c->scale_format == SAD_KV_SCALE_UE8M0 ? 8 : 4 * (c->d_nope / 64);
}

int check_kv_cache(const sad_kv_cache* c, const char* what) {
  SAD_CHECK(c != nullptr && c->pool != nullptr, SAD_EINVAL, "%s: cache or pool is NULL", what);
  const bool f32 = c->scale_format == SAD_KV_SCALE_F32;
  const bool native = c->scale_format == SAD_KV_SCALE_UE8M0;
  SAD_CHECK((f32 && c->d_nope == 512 && c->d_rope == 64) || (f32 && c->d_nope == 128 && c->d_rope == 32) ||
                (native && c->d_nope == 448 && c->d_rope == 64),
            SAD_EUNSUPPORTED, "%s: (d_nope, d_rope, scale_format) = (%d, %d, %d) unsupported", what,
            c->d_nope, c->d_rope, c->scale_format);
  SAD_CHECK(c->block_size == 16 || c->block_size == 64, SAD_EUNSUPPORTED,
            "%s: block_size %d unsupported", what, c->block_size);
  const int64_t need = (int64_t)c->block_size * (c->d_nope + 2 * c->d_rope + kv_scale_bytes(c));
  SAD_CHECK(c->page_stride >= need && c->page_stride % 16 == 0, SAD_EINVAL,
            "%s: page_stride %lld must be a multiple of 16 and >= %lld", what,
            (long long)c->page_stride, (long long)need);
  SAD_CHECK(c->num_pages >= 0 && c->num_pages * (int64_t)c->block_size <= INT32_MAX, SAD_EINVAL,
            "%s: num_pages*block_size must fit int32", what);
  SAD_CHECK(((uintptr_t)c->pool & 15) == 0, SAD_EINVAL, "%s: pool must be 16-byte aligned", what);
  return SAD_OK;
}

}  // namespace sad

using namespace sad;

extern "C" int gather_dequant_kv(const sad_kv_cache* swa, const sad_kv_cache* comp,
                                 const int32_t* sparse_indices, const int32_t* sparse_topk_lens,
                                 int32_t num_tokens, int32_t window_size, int32_t padded_topk,
                                 uint16_t* out_bf16, void* stream) {
  clear_error();
  int rc = check_kv_cache(swa, "gather_dequant_kv(swa)");
  if (rc != SAD_OK) return rc;
  rc = check_kv_cache(comp, "gather_dequant_kv(comp)");
  if (rc != SAD_OK) return rc;
  SAD_CHECK(swa->d_nope == comp->d_nope && swa->d_rope == comp->d_rope &&
                swa->scale_format == comp->scale_format,
            SAD_EINVAL, "gather_dequant_kv: swa and comp caches must share (d_nope, d_rope, scale_format)");
  SAD_CHECK(num_tokens >= 0 && window_size >= 0 && padded_topk >= 0, SAD_EINVAL,
            "gather_dequant_kv: negative size");
  if (num_tokens == 0 || window_size + padded_topk == 0) return SAD_OK;
  SAD_CHECK(sparse_indices && sparse_topk_lens && out_bf16, SAD_EINVAL,
            "gather_dequant_kv: NULL pointer argument");
  SAD_CHECK(((uintptr_t)out_bf16 & 15) == 0, SAD_EINVAL,
            "gather_dequant_kv: out must be 16-byte aligned");
  const int64_t rows = (int64_t)num_tokens * (window_size + padded_topk);
  const int64_t blocks = (rows + 3) / 4;
  SAD_CHECK(blocks < ((int64_t)1 << 31), SAD_EINVAL, "gather_dequant_kv: too many rows");
  KvDesc s{(const uint8_t*)swa->pool, swa->page_stride, swa->num_pages, swa->block_size,
           __builtin_ctz(swa->block_size)};
  KvDesc c{(const uint8_t*)comp->pool, comp->page_stride, comp->num_pages, comp->block_size,
           __builtin_ctz(comp->block_size)};
  if (swa->d_nope == 512) {
    hipLaunchKernelGGL((gather_dequant_kernel<512, 64>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       (hipStream_t)stream, s, c, sparse_indices, sparse_topk_lens, rows,
                       window_size, padded_topk, out_bf16);
  } else if (swa->d_nope == 448) {
    hipLaunchKernelGGL((gather_dequant_kernel<448, 64>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       (hipStream_t)stream, s, c, sparse_indices, sparse_topk_lens, rows,
                       window_size, padded_topk, out_bf16);
  } else {
    hipLaunchKernelGGL((gather_dequant_kernel<128, 32>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       (hipStream_t)stream, s, c, sparse_indices, sparse_topk_lens, rows,
                       window_size, padded_topk, out_bf16);
  }
  return check_launch("gather_dequant_kv");
}
