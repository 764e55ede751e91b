// Internal helpers shared by the libsad.so translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sad.h"

namespace sad {

// ---- host-side error reporting -------------------------------------------------

void set_error(const char* fmt, ...);
void clear_error();
int check_launch(const char* what);
// Host-side validation of a latent KV cache descriptor (SAD_OK or an error code).
int check_kv_cache(const sad_kv_cache* c, const char* what);
// Bytes of one row's scales: 4*d_nope/64 (fp32 form) or 8 (native ue8m0 form).
int kv_scale_bytes(const sad_kv_cache* c);
// Host-side checks of build_sparse_indices' arguments (SAD_OK or an error code, the
// message naming `what`); shared with the fused indexer + index build entry point.
int check_build_args(const char* what, const sad_batch* batch, const int32_t* swa_bt,
                     int64_t swa_bt_stride, int32_t swa_bt_cols, int32_t swa_block_size,
                     int64_t swa_num_pages, const int32_t* comp_bt, int64_t comp_bt_stride,
                     int32_t comp_bt_cols, int32_t comp_block_size, int64_t comp_num_pages,
                     bool has_topk, int64_t topk_stride, int32_t topk, int32_t window_size,
                     int32_t compress_ratio, int32_t padded_topk, const int32_t* sparse_indices,
                     const int32_t* sparse_topk_lens);

#define SAD_CHECK(cond, code, ...)   \
  do {                               \
    if (!(cond)) {                   \
      ::sad::set_error(__VA_ARGS__); \
      return (code);                 \
    }                                \
  } while (0)

// Compute units of the current device (read once per device; 256, MI355X's count, if the
// query fails).  The launch heuristics size their grids with it.
int num_cus();

// A paged latent KV cache as the attention kernels address it.
struct KvDesc {
  const uint8_t* pool;
  int64_t stride;
  int64_t num_pages;
  int block;
  int block_shift;  // log2(block)
};

// The dim-split attention kernel of the (512 fp8 + 64 bf16, fp32 scales) row, or with
// native = true of the pages' (448 fp8 + 64 bf16, ue8m0 scales) row: out (or, with
// splits > 1, the split partials part_o / part_lse) for every token and head.
int launch_mla_dsplit(const uint16_t* q, int T, int H, const KvDesc& swa, const KvDesc& comp,
                      const int32_t* si, const int32_t* lens, int W, int P, float scale, const float* sink,
                      uint16_t* out, float* lse, float* part_o, float* part_lse, int splits, bool native,
                      hipStream_t st);

// ---- vector types -----------------------------------------------------------------

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2_t;

// ---- token geometry ---------------------------------------------------------------

// Request, position and number of visible compressed rows of token t.
// ([backend] _decode_positions_from_metadata; [model] indexer row_lens.)
struct TokenGeom {
  int req;
  int pos;
  int n_comp;
};

// A read of a batch word at a workgroup-uniform index through the constant address
// space: a scalar-cache load (these arrays are inputs no kernel writes during a launch),
// counted apart from the vector memory loads, so a vector load issued earlier is not
// waited for when its value is needed.
__device__ inline int uniform_ro_load(const int32_t* p) {
  typedef const __attribute__((address_space(4))) int32_t const_i32;
  return *(const_i32*)p;
}

// Geometry of a workgroup-uniform token t, read with scalar-cache loads.  Returns false
// when the token sees nothing (bad request id or negative position).
__device__ inline bool token_geometry_uniform(const sad_batch& b, int t, int ratio, TokenGeom& g) {
  const int r = uniform_ro_load(b.token_to_req + t);
  g.req = r;
  g.pos = -1;
  g.n_comp = 0;
  if (r < 0 || r >= b.num_reqs) return false;
  const int q0 = uniform_ro_load(b.query_start_loc + r);
  const int q1 = uniform_ro_load(b.query_start_loc + r + 1);
  const int p = uniform_ro_load(b.seq_lens + r) - (q1 - q0) + (t - q0);
  if (p < 0) return false;
  g.pos = p;
  g.n_comp = (p + 1) / ratio;
  return true;
}

// Paged lookup: logical row -> slot, or -1 when the page is not a valid pool page.
__device__ inline int page_slot(const int32_t* bt_row, int cols, int block, int64_t num_pages,
                                int logical) {
  if (logical < 0) return -1;
  const int col = logical / block;
  if (col >= cols) return -1;
  const int page = bt_row[col];
  if (page < 0 || (int64_t)page >= num_pages) return -1;
  return page * block + (logical - col * block);
}

// A slot resolves to a row of the pool iff 0 <= slot / block < num_pages.
__device__ inline bool slot_ok(int slot, int block, int64_t num_pages) {
  return slot >= 0 && (int64_t)(slot / block) < num_pages;
}

// ---- wave / block reductions ------------------------------------------------------

__device__ inline int wave_lane() { return __lane_id(); }

// Inclusive prefix sum across the 64 lanes of a wave.
// Inclusive prefix sum over the 64 lanes of a wave (all lanes active), modulo 2^32: DPP
// row shifts by 1, 2, 4 and 8 scan each row of 16 lanes (lanes shifted in from outside
// the row add zero), then the row broadcasts of lane 15 (into rows 1 and 3) and of
// lane 31 (into rows 2 and 3) carry the row totals.
__device__ inline uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ inline int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ---- element conversions ------------------------------------------------------------

// Round a float to bf16 bits, nearest-even (finite inputs).
__device__ inline uint16_t f32_to_bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ inline float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// OCP e4m3fn byte -> float (exact).  gfx950's conversion instruction decodes OCP
// FP8; byte selects which of the 4 bytes of `word` is converted.
template <int kByte>
__device__ inline float e4m3_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8((int)word, kByte);
}

}  // namespace sad
