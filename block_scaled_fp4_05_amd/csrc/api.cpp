// C ABI of the NVFP4 MoE grouped GEMM library (declared in include/moe_fp4.h).
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime, so an argument that fails here never reaches a launch, and one
// that passes here always launches: there is no second check that could reject
// a configuration the first one accepted (the failure mode described on
// "Peering into the CUTLASS SharedStorage", section "Why This Message Was
// Written", where can_implement passed and initialize then failed).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "../../include/moe_fp4.h"
#include "launch.h"

using moe_fp4::GemmArgs;
using moe_fp4::GemmTile;

namespace {

constexpr int kAbiVersion = 2;
// The work-list tables (8 bytes per expert) live in LDS beside each kernel's
// own buffers (at most 68 KB); 8192 experts keep every kernel within 160 KB.
constexpr int32_t kMaxExperts = 8192;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Whether the byte ranges [p, p + pb) and [q, q + qb) share a byte.
bool overlap(const void* p, int64_t pb, const void* q, int64_t qb) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return pb > 0 && qb > 0 && a < b + (uintptr_t)qb && b < a + (uintptr_t)pb;
}

int check_gemm_shape(int32_t num_experts, int64_t m_total, int64_t n, int64_t k) {
  if (num_experts < 1 || m_total < 0 || n < 1 || k < 1) return MOE_FP4_ERR_SHAPE;
  if (num_experts > kMaxExperts) return MOE_FP4_ERR_UNSUPPORTED;
  if (n % 16 != 0 || k % moe_fp4::kKStep != 0) return MOE_FP4_ERR_UNSUPPORTED;
  // Row-index entries are addressed with 32-bit byte offsets.
  if (n > INT32_MAX / 2 || m_total > INT32_MAX / 4 - 1024) return MOE_FP4_ERR_UNSUPPORTED;
  // One expert's packed weights are addressed with 32-bit buffer offsets.
  if (k / 2 > ((int64_t)INT32_MAX - 4096) / n) return MOE_FP4_ERR_UNSUPPORTED;
  // The work-list counts items in int32: bound the largest possible count.
  const int64_t max_mtiles = m_total / 16 + (m_total < num_experts ? m_total : num_experts);
  const int64_t n_tiles = (n + 31) / 32;
  // Items and items x pipeline stages are counted in int32.
  if (max_mtiles * n_tiles * (k / moe_fp4::kKStep) >= (int64_t)INT32_MAX)
    return MOE_FP4_ERR_UNSUPPORTED;
  return MOE_FP4_OK;
}

}  // namespace

extern "C" {

int moe_fp4_abi_version(void) { return kAbiVersion; }

const char* moe_fp4_status_string(int status) {
  switch (status) {
    case MOE_FP4_OK: return "ok";
    case MOE_FP4_ERR_NULL: return "a required pointer is NULL";
    case MOE_FP4_ERR_SHAPE: return "a size is out of range or sizes are inconsistent";
    case MOE_FP4_ERR_ALIGN: return "a pointer or leading dimension is misaligned";
    case MOE_FP4_ERR_UNSUPPORTED: return "valid arguments outside what the kernels support";
    case MOE_FP4_ERR_HIP: return "the HIP runtime reported an error";
    case MOE_FP4_ERR_ARG: return "an enumerated argument has an unknown value, or buffers overlap";
    default: return "unknown status";
  }
}

int64_t moe_fp4_stage_bytes(int64_t bm, int64_t bn, int64_t bk) {
  if (bm < 1 || bn < 1 || bk < 16 || bk % 16 != 0) return -1;
  // Packed FP4 (half a byte per element) plus one E4M3 byte per 16 elements,
  // for the A tile (bm x bk) and the B tile (bn x bk).
  const int64_t a = bm * bk / 2 + bm * (bk / 16);
  const int64_t b = bn * bk / 2 + bn * (bk / 16);
  return a + b;
}

int moe_fp4_quantize(const void* x, int in_dtype, int64_t rows, int64_t k, int64_t ld_x,
                     uint8_t* q, uint8_t* sf, float* tensor_scale, int scale_mode,
                     void* stream) {
  if (in_dtype != MOE_FP4_IN_BF16 && in_dtype != MOE_FP4_IN_FP32) return MOE_FP4_ERR_ARG;
  if (scale_mode != MOE_FP4_SCALE_STATIC && scale_mode != MOE_FP4_SCALE_DYNAMIC)
    return MOE_FP4_ERR_ARG;
  if (!tensor_scale) return MOE_FP4_ERR_NULL;
  if (rows < 0 || k <= 0 || k % 16 != 0 || ld_x < k) return MOE_FP4_ERR_SHAPE;
  if (rows > 0 && (!x || !q || !sf)) return MOE_FP4_ERR_NULL;
  const int64_t esize = in_dtype == MOE_FP4_IN_BF16 ? 2 : 4;
  if (!aligned(tensor_scale, 4)) return MOE_FP4_ERR_ALIGN;
  if (rows > 0 && (!aligned(x, 16) || (ld_x * esize) % 16 != 0 || !aligned(q, 8)))
    return MOE_FP4_ERR_ALIGN;
  if (rows > 0 && (rows > INT64_MAX / k)) return MOE_FP4_ERR_SHAPE;
  // x's extent, ((rows - 1) * ld_x + k) * esize bytes, must be representable.
  if (rows > 1 && (ld_x > (INT64_MAX / esize - k) / (rows - 1))) return MOE_FP4_ERR_SHAPE;
  // The four buffers must be distinct: the dynamic mode hands the amax pass's
  // partial values to the quantise pass inside q while x is still being read,
  // and writes the tensor scale while q is being read.
  if (rows > 0) {
    const int64_t xb = ((rows - 1) * ld_x + k) * esize, qb = rows * (k / 2), sb = rows * (k / 16);
    if (overlap(x, xb, q, qb) || overlap(x, xb, sf, sb) || overlap(x, xb, tensor_scale, 4) ||
        overlap(q, qb, sf, sb) || overlap(q, qb, tensor_scale, 4) ||
        overlap(sf, sb, tensor_scale, 4))
      return MOE_FP4_ERR_ARG;
  }
  hipError_t err = moe_fp4::launch_quantize(x, in_dtype, rows, k, ld_x, q, sf, tensor_scale,
                                            scale_mode == MOE_FP4_SCALE_DYNAMIC ? 1 : 0,
                                            reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? MOE_FP4_OK : MOE_FP4_ERR_HIP;
}

size_t moe_grouped_gemm_fp4_workspace_size(int32_t num_experts, int64_t m_total, int64_t n,
                                           int64_t k) {
  (void)num_experts, (void)m_total, (void)n, (void)k;
  // Every kernel builds its work list in LDS from the device offsets.
  return 0;
}

int moe_grouped_gemm_fp4_plan(int32_t num_experts, int64_t m_total, int64_t n, int64_t k,
                              moe_fp4_gemm_plan* plan) {
  if (!plan) return MOE_FP4_ERR_NULL;
  const int s = check_gemm_shape(num_experts, m_total, n, k);
  if (s != MOE_FP4_OK) return s;
  const GemmTile t = moe_fp4::choose_tile(num_experts, m_total, n, k, getenv("MOE_FP4_TILE"));
  plan->tile_m = 16 * t.m_blocks;
  plan->tile_n = 16 * t.n_blocks;
  plan->k_step = (t.tiled == 4 || t.tiled == 6) ? 256 : t.tiled ? 64 : moe_fp4::kKStep * t.k_sub;
  plan->waves_per_group = t.waves;
  plan->lds_bytes = moe_fp4::gemm_lds_bytes(t, num_experts);
  return MOE_FP4_OK;
}

}  // extern "C"

namespace {

int grouped_gemm(const uint8_t* a_q, const uint8_t* a_sf, const float* a_scale, int64_t a_rows,
                 const int32_t* a_row_index, const uint8_t* w_q, const uint8_t* w_sf,
                 const float* w_scale, const int32_t* expert_offsets, int32_t num_experts,
                 int64_t m_total, int64_t n, int64_t k, uint16_t* out, int64_t ldo,
                 void* stream, bool packed) {
  if (!a_q || !a_sf || !a_scale || !w_q || !w_sf || !w_scale || !expert_offsets || !out)
    return MOE_FP4_ERR_NULL;
  if (num_experts < 1 || m_total < 0 || n < 1 || k < 1 || ldo < n || a_rows < 0)
    return MOE_FP4_ERR_SHAPE;
  if (!a_row_index && a_rows < m_total) return MOE_FP4_ERR_SHAPE;
  if (m_total > 0 && a_rows < 1) return MOE_FP4_ERR_SHAPE;
  const int s = check_gemm_shape(num_experts, m_total, n, k);
  if (s != MOE_FP4_OK) return s;
  if (!aligned(a_q, 16) || !aligned(a_sf, 16) || !aligned(w_q, 16) || !aligned(w_sf, 16) ||
      !aligned(out, 16) || !aligned(a_scale, 4) || !aligned(w_scale, 4) ||
      !aligned(expert_offsets, 4) || (a_row_index && !aligned(a_row_index, 4)) || ldo % 8 != 0)
    return MOE_FP4_ERR_ALIGN;
  // Activations and one item's output rows are addressed with 32-bit buffer
  // offsets as well.
  if (a_rows > ((int64_t)INT32_MAX - 4096) / (k / 2) || ldo > (1 << 23))
    return MOE_FP4_ERR_UNSUPPORTED;
  const GemmTile t = moe_fp4::fit_output_range(
      moe_fp4::choose_tile(num_experts, m_total, n, k, getenv("MOE_FP4_TILE")), k, ldo);
  // Packed weights fix the per-wavefront K step to the layout's granule.
  if (packed && !t.tiled &&
      (t.n_blocks != 4 || t.k_sub != moe_fp4::packed_granule(k) / moe_fp4::kKStep))
    return MOE_FP4_ERR_UNSUPPORTED;
  moe_fp4::log_tile(packed ? "moe_grouped_gemm_fp4_packed" : "moe_grouped_gemm_fp4", num_experts,
                    m_total, n, k, ldo, t);
  if (m_total == 0) return MOE_FP4_OK;
  GemmArgs p = {};
  p.a_q = a_q;
  p.a_sf = a_sf;
  p.a_scale = a_scale;
  p.a_row_index = a_row_index;
  p.w_q = w_q;
  p.w_sf = w_sf;
  p.w_scale = w_scale;
  p.offsets = expert_offsets;
  p.out = out;
  p.a_rows = a_rows;
  p.m_total = m_total;
  p.n = n;
  p.k = k;
  p.ldo = ldo;
  p.num_experts = num_experts;
  p.n_tiles = (int32_t)((n + 16 * t.n_blocks - 1) / (16 * t.n_blocks));
  p.w_packed = packed ? 1 : 0;
  hipError_t err = moe_fp4::launch_grouped_gemm(p, t, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? MOE_FP4_OK : MOE_FP4_ERR_HIP;
}

int grouped_gemm_finalize(const uint8_t* a_q, const uint8_t* a_sf, const float* a_scale,
                          int64_t a_rows, const int32_t* a_row_index, const uint8_t* w_q,
                          const uint8_t* w_sf, const float* w_scale, int w_packed,
                          const int32_t* expert_offsets, int32_t num_experts, int64_t m_total,
                          int64_t n, int64_t k, const int32_t* out_token,
                          const float* row_weight, float* out, int64_t ldo, int64_t num_tokens,
                          void* stream) {
  if (!a_q || !a_sf || !a_scale || !w_q || !w_sf || !w_scale || !expert_offsets || !out ||
      !out_token || !row_weight)
    return MOE_FP4_ERR_NULL;
  if (w_packed != 0 && w_packed != 1) return MOE_FP4_ERR_ARG;
  if (num_experts < 1 || m_total < 0 || n < 1 || k < 1 || ldo < n || a_rows < 0 || num_tokens < 1)
    return MOE_FP4_ERR_SHAPE;
  if (!a_row_index && a_rows < m_total) return MOE_FP4_ERR_SHAPE;
  if (m_total > 0 && a_rows < 1) return MOE_FP4_ERR_SHAPE;
  const int s = check_gemm_shape(num_experts, m_total, n, k);
  if (s != MOE_FP4_OK) return s;
  if (!aligned(a_q, 16) || !aligned(a_sf, 16) || !aligned(w_q, 16) || !aligned(w_sf, 16) ||
      !aligned(out, 4) || !aligned(a_scale, 4) || !aligned(w_scale, 4) ||
      !aligned(expert_offsets, 4) || (a_row_index && !aligned(a_row_index, 4)) ||
      !aligned(out_token, 4) || !aligned(row_weight, 4))
    return MOE_FP4_ERR_ALIGN;
  if (a_rows > ((int64_t)INT32_MAX - 4096) / (k / 2)) return MOE_FP4_ERR_UNSUPPORTED;
  // The token rows are addressed with 32-bit byte offsets.
  if (num_tokens > (int64_t)INT32_MAX / 4 || ldo > ((int64_t)INT32_MAX - 4096) / 4 / num_tokens)
    return MOE_FP4_ERR_UNSUPPORTED;
  GemmTile t = moe_fp4::choose_tile(num_experts, m_total, n, k, getenv("MOE_FP4_TILE"));
  // The finalize epilogue runs in the per-wave kernel with 64-column items;
  // experts large enough for the workgroup tile take four row blocks per item.
  if (t.tiled) t = GemmTile{4, 4, 4, k % 512 == 0 ? 2 : 1, k % 2048 == 0 ? 1 : 0, 0};
  if (t.n_blocks != 4 || t.k_sub > 2) return MOE_FP4_ERR_UNSUPPORTED;
  if (w_packed && t.k_sub != moe_fp4::packed_granule(k) / moe_fp4::kKStep)
    return MOE_FP4_ERR_UNSUPPORTED;
  moe_fp4::log_tile("moe_grouped_gemm_fp4_finalize", num_experts, m_total, n, k, ldo, t);
  if (m_total == 0) return MOE_FP4_OK;
  GemmArgs p = {};
  p.a_q = a_q;
  p.a_sf = a_sf;
  p.a_scale = a_scale;
  p.a_row_index = a_row_index;
  p.w_q = w_q;
  p.w_sf = w_sf;
  p.w_scale = w_scale;
  p.offsets = expert_offsets;
  p.out = nullptr;
  p.a_rows = a_rows;
  p.m_total = m_total;
  p.n = n;
  p.k = k;
  p.ldo = n;
  p.num_experts = num_experts;
  p.n_tiles = (int32_t)((n + 63) / 64);
  p.w_packed = w_packed;
  p.out_token = out_token;
  p.row_weight = row_weight;
  p.fin_out = out;
  p.fin_ldo = ldo;
  p.num_tokens = num_tokens;
  hipError_t err =
      moe_fp4::launch_grouped_gemm_finalize(p, t, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? MOE_FP4_OK : MOE_FP4_ERR_HIP;
}

int grouped_gemm_swiglu(const uint8_t* a_q, const uint8_t* a_sf, const float* a_scale,
                        int64_t a_rows, const int32_t* a_row_index, const uint8_t* w_q,
                        const uint8_t* w_sf, const float* w_scale, int w_packed,
                        const int32_t* expert_offsets, int32_t num_experts, int64_t m_total,
                        int64_t n, int64_t k, const float* h_scale, uint8_t* h_q, uint8_t* h_sf,
                        void* stream) {
  if (!a_q || !a_sf || !a_scale || !w_q || !w_sf || !w_scale || !expert_offsets || !h_scale ||
      !h_q || !h_sf)
    return MOE_FP4_ERR_NULL;
  if (w_packed != 0 && w_packed != 1) return MOE_FP4_ERR_ARG;
  if (num_experts < 1 || m_total < 0 || n < 1 || k < 1 || a_rows < 0) return MOE_FP4_ERR_SHAPE;
  if (!a_row_index && a_rows < m_total) return MOE_FP4_ERR_SHAPE;
  if (m_total > 0 && a_rows < 1) return MOE_FP4_ERR_SHAPE;
  const int s = check_gemm_shape(num_experts, m_total, n, k);
  if (s != MOE_FP4_OK) return s;
  if (!aligned(a_q, 16) || !aligned(a_sf, 16) || !aligned(w_q, 16) || !aligned(w_sf, 16) ||
      !aligned(h_q, 16) || !aligned(h_sf, 16) || !aligned(a_scale, 4) || !aligned(w_scale, 4) ||
      !aligned(h_scale, 4) || !aligned(expert_offsets, 4) ||
      (a_row_index && !aligned(a_row_index, 4)))
    return MOE_FP4_ERR_ALIGN;
  if (a_rows > ((int64_t)INT32_MAX - 4096) / (k / 2)) return MOE_FP4_ERR_UNSUPPORTED;
  // The intermediate has n/2 columns in whole 16-element blocks; packed weights
  // are read in whole 64-row groups, which must not straddle the gate/up halves.
  if (n % 32 != 0 || (w_packed && (n / 2) % 64 != 0)) return MOE_FP4_ERR_UNSUPPORTED;
  // The outputs are written while the inputs are still being read.
  const int64_t hq_bytes = m_total * (n / 4), hs_bytes = m_total * (n / 32);
  if (overlap(h_q, hq_bytes, h_sf, hs_bytes) || overlap(h_q, hq_bytes, a_q, a_rows * (k / 2)) ||
      overlap(h_q, hq_bytes, a_sf, a_rows * (k / 16)) ||
      overlap(h_sf, hs_bytes, a_q, a_rows * (k / 2)) ||
      overlap(h_sf, hs_bytes, a_sf, a_rows * (k / 16)))
    return MOE_FP4_ERR_ARG;
  GemmTile t = moe_fp4::choose_tile(num_experts, m_total, n, k, getenv("MOE_FP4_TILE"));
  // Per-wave kernels with 4 row blocks (32 gate + 32 up rows) per item;
  // experts large enough for the workgroup tile take four row blocks of rows.
  if (t.tiled) t = GemmTile{4, 4, 4, k % 512 == 0 ? 2 : 1, k % 2048 == 0 ? 1 : 0, 0};
  if (t.n_blocks != 4 || t.k_sub > 2) return MOE_FP4_ERR_UNSUPPORTED;
  if (w_packed && t.k_sub != moe_fp4::packed_granule(k) / moe_fp4::kKStep)
    return MOE_FP4_ERR_UNSUPPORTED;
  moe_fp4::log_tile("moe_grouped_gemm_fp4_swiglu", num_experts, m_total, n, k, n, t);
  if (m_total == 0) return MOE_FP4_OK;
  GemmArgs p = {};
  p.a_q = a_q;
  p.a_sf = a_sf;
  p.a_scale = a_scale;
  p.a_row_index = a_row_index;
  p.w_q = w_q;
  p.w_sf = w_sf;
  p.w_scale = w_scale;
  p.offsets = expert_offsets;
  p.a_rows = a_rows;
  p.m_total = m_total;
  p.n = n;
  p.k = k;
  p.ldo = n;
  p.num_experts = num_experts;
  p.n_tiles = (int32_t)((n / 2 + 31) / 32);
  p.w_packed = w_packed;
  p.h_q = h_q;
  p.h_sf = h_sf;
  p.h_scale = h_scale;
  hipError_t err =
      moe_fp4::launch_grouped_gemm_swiglu(p, t, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? MOE_FP4_OK : MOE_FP4_ERR_HIP;
}

int repack(const uint8_t* src, uint8_t* dst, int32_t num_experts, int64_t n, int64_t k,
           void* stream, bool to_packed) {
  if (!src || !dst) return MOE_FP4_ERR_NULL;
  if (num_experts < 1 || n < 1 || k < 1) return MOE_FP4_ERR_SHAPE;
  if (n % 16 != 0 || k % moe_fp4::kKStep != 0) return MOE_FP4_ERR_UNSUPPORTED;
  if (n > INT32_MAX / 2 || k / 2 > ((int64_t)INT32_MAX - 4096) / n) return MOE_FP4_ERR_UNSUPPORTED;
  if (!aligned(src, 16) || !aligned(dst, 16)) return MOE_FP4_ERR_ALIGN;
  const uintptr_t bytes = (uintptr_t)num_experts * (uintptr_t)n * (uintptr_t)(k / 2);
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + bytes && b < a + bytes) return MOE_FP4_ERR_ARG;  // overlapping buffers
  hipError_t err = moe_fp4::launch_repack(src, dst, num_experts, n, k, to_packed,
                                          reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? MOE_FP4_OK : MOE_FP4_ERR_HIP;
}

}  // namespace

extern "C" {

int moe_grouped_gemm_fp4(const uint8_t* a_q, const uint8_t* a_sf, const float* a_scale,
                         int64_t a_rows, const int32_t* a_row_index,
                         const uint8_t* w_q, const uint8_t* w_sf, const float* w_scale,
                         const int32_t* expert_offsets, int32_t num_experts,
                         int64_t m_total, int64_t n, int64_t k,
                         uint16_t* out, int64_t ldo, void* stream) {
  return grouped_gemm(a_q, a_sf, a_scale, a_rows, a_row_index, w_q, w_sf, w_scale,
                      expert_offsets, num_experts, m_total, n, k, out, ldo, stream, false);
}

int moe_grouped_gemm_fp4_packed(const uint8_t* a_q, const uint8_t* a_sf, const float* a_scale,
                                int64_t a_rows, const int32_t* a_row_index,
                                const uint8_t* w_packed, const uint8_t* w_sf,
                                const float* w_scale, const int32_t* expert_offsets,
                                int32_t num_experts, int64_t m_total, int64_t n, int64_t k,
                                uint16_t* out, int64_t ldo, void* stream) {
  return grouped_gemm(a_q, a_sf, a_scale, a_rows, a_row_index, w_packed, w_sf, w_scale,
                      expert_offsets, num_experts, m_total, n, k, out, ldo, stream, true);
}

int moe_grouped_gemm_fp4_finalize(const uint8_t* a_q, const uint8_t* a_sf, const float* a_scale,
                                  int64_t a_rows, const int32_t* a_row_index,
                                  const uint8_t* w_q, const uint8_t* w_sf, const float* w_scale,
                                  int w_packed, const int32_t* expert_offsets,
                                  int32_t num_experts, int64_t m_total, int64_t n, int64_t k,
                                  const int32_t* out_token, const float* row_weight, float* out,
                                  int64_t ldo, int64_t num_tokens, void* stream) {
  return grouped_gemm_finalize(a_q, a_sf, a_scale, a_rows, a_row_index, w_q, w_sf, w_scale,
                               w_packed, expert_offsets, num_experts, m_total, n, k, out_token,
                               row_weight, out, ldo, num_tokens, stream);
}

int moe_grouped_gemm_fp4_swiglu(const uint8_t* a_q, const uint8_t* a_sf, const float* a_scale,
                                int64_t a_rows, const int32_t* a_row_index,
                                const uint8_t* w_q, const uint8_t* w_sf, const float* w_scale,
                                int w_packed, const int32_t* expert_offsets, int32_t num_experts,
                                int64_t m_total, int64_t n, int64_t k, const float* h_scale,
                                uint8_t* h_q, uint8_t* h_sf, void* stream) {
  return grouped_gemm_swiglu(a_q, a_sf, a_scale, a_rows, a_row_index, w_q, w_sf, w_scale,
                             w_packed, expert_offsets, num_experts, m_total, n, k, h_scale, h_q,
                             h_sf, stream);
}

int moe_fp4_combine(const uint16_t* rows, int64_t ld_rows, int64_t m_total,
                    const int32_t* token_rows, const float* token_weights, int32_t topk,
                    int64_t num_tokens, int64_t n, const float* residual, int64_t ld_res,
                    void* out, int out_dtype, int64_t ldo, void* stream) {
  if (out_dtype != MOE_FP4_OUT_BF16 && out_dtype != MOE_FP4_OUT_FP32) return MOE_FP4_ERR_ARG;
  if (!token_rows || !token_weights || !out || (m_total > 0 && !rows)) return MOE_FP4_ERR_NULL;
  if (m_total < 0 || num_tokens < 0 || topk < 1 || n < 1 || ldo < n || (m_total > 0 && ld_rows < n) ||
      (residual && ld_res < n))
    return MOE_FP4_ERR_SHAPE;
  const int64_t esize = out_dtype == MOE_FP4_OUT_FP32 ? 4 : 2;
  if ((m_total > 0 && (!aligned(rows, 16) || ld_rows % 8 != 0)) || !aligned(out, 16) ||
      (ldo * esize) % 16 != 0 || !aligned(token_rows, 4) || !aligned(token_weights, 4) ||
      (residual && (!aligned(residual, 16) || ld_res % 4 != 0)))
    return MOE_FP4_ERR_ALIGN;
  if (n % 16 != 0) return MOE_FP4_ERR_UNSUPPORTED;
  const int64_t lim = (int64_t)INT32_MAX - 4096;
  if (m_total > lim / 2 / (ld_rows > 0 ? ld_rows : 1) || num_tokens > lim / esize / ldo ||
      (residual && num_tokens > lim / 4 / ld_res) || num_tokens > lim / topk)
    return MOE_FP4_ERR_UNSUPPORTED;
  if (num_tokens == 0) return MOE_FP4_OK;
  moe_fp4::CombineArgs a;
  a.rows = rows;
  a.ld_rows = ld_rows;
  a.m_total = m_total;
  a.token_rows = token_rows;
  a.token_weights = token_weights;
  a.topk = topk;
  a.num_tokens = num_tokens;
  a.n = n;
  a.residual = residual;
  a.ld_res = ld_res;
  a.out = out;
  a.ldo = ldo;
  a.f32_out = out_dtype == MOE_FP4_OUT_FP32 ? 1 : 0;
  hipError_t err = moe_fp4::launch_combine(a, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? MOE_FP4_OK : MOE_FP4_ERR_HIP;
}

int moe_fp4_pack_weights(const uint8_t* w_q, uint8_t* w_packed, int32_t num_experts,
                         int64_t n, int64_t k, void* stream) {
  return repack(w_q, w_packed, num_experts, n, k, stream, true);
}

int moe_fp4_unpack_weights(const uint8_t* w_packed, uint8_t* w_q, int32_t num_experts,
                           int64_t n, int64_t k, void* stream) {
  return repack(w_packed, w_q, num_experts, n, k, stream, false);
}

}  // extern "C"
