// Internal interface between the C-ABI layer (api.cpp) and the kernel
// launchers.  Arguments reaching a launcher have been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_fp4 {

// Quantiser: enqueue the kernels of moe_fp4_quantize on `stream`.
hipError_t launch_quantize(const void* x, int in_dtype, int64_t rows, int64_t k, int64_t ld_x,
                           uint8_t* q, uint8_t* sf, float* tensor_scale, int dynamic,
                           hipStream_t stream);

// Tile shapes of the grouped GEMM.  Rows per work item = 16 * m_blocks; output
// columns per wavefront = 16 * n_blocks; a workgroup holds `waves` wavefronts,
// each working on its own item; one pipeline stage covers 256 * k_sub
// elements of K.
struct GemmTile {
  int m_blocks;
  int n_blocks;
  int waves;
  int k_sub;
  int lds_scales;  // weight block scales staged through LDS (needs k % 2048 == 0)
  int tiled;       // workgroup-tiled kernel, operands shared in LDS: 1 = 128 x 128
                   // items (grouped_gemm_tiled.hip); 2 = 256 x 256 items
                   // (grouped_gemm_big.hip) for experts of kBigRows rows or more
                   // and the per-wave kernel for the rest; 3 = 256 x 256 for all;
                   // 4 = 48 x 512 items (grouped_gemm_mid.hip) for every expert;
                   // 5, 6, 7 = splits by expert size over the large tile, the
                   // 48 x 512 items and the per-wave items (launch_grouped_gemm)
  int f8 = 0;      // 256 x 256 items: split K by scale block on the FP8 MFMA
                   // instead of dequantising to FP16 (MOE_FP4_TILE "256x256f8")
};

constexpr int kKStep = 256;  // K granularity the kernels require

// Packed weight layout (moe_fp4_pack_weights): K elements per granule, and the
// bytes of one 16-row x granule block.  Rows are grouped by 64.
__host__ __device__ constexpr int32_t packed_granule(int64_t k) { return k % 512 == 0 ? 512 : 256; }
__host__ __device__ constexpr int32_t packed_block_bytes(int32_t granule) { return 8 * granule; }
constexpr int kPackRows = 64;

// Token-order combine of routed rows (combine.hip).
struct CombineArgs {
  const uint16_t* rows;  // BF16 [m_total][ld_rows]
  int64_t ld_rows;
  int64_t m_total;
  const int32_t* token_rows;     // [num_tokens][topk], row index or < 0
  const float* token_weights;    // [num_tokens][topk]
  int32_t topk;
  int64_t num_tokens;
  int64_t n;
  const float* residual;  // FP32 [num_tokens][ld_res] or NULL
  int64_t ld_res;
  void* out;              // BF16 or FP32 [num_tokens][ldo]
  int64_t ldo;
  int32_t f32_out;
};
hipError_t launch_combine(const CombineArgs& args, hipStream_t stream);

// Rearrange weight codes between the row-major and the packed layout.
hipError_t launch_repack(const uint8_t* src, uint8_t* dst, int32_t num_experts, int64_t n,
                         int64_t k, bool to_packed, hipStream_t stream);

// The tile used for a problem with these sizes; `env` (may be NULL) is the
// value of MOE_FP4_TILE ("MxN" or "MxNxK": M rows per item, N columns per
// wave, K elements per pipeline stage; a trailing 'r' keeps the weight block
// scales in registers instead of staging them through LDS).
GemmTile choose_tile(int32_t num_experts, int64_t m_total, int64_t n, int64_t k, const char* env);

// LDS bytes a workgroup of the grouped GEMM uses for `num_experts` experts.
int64_t gemm_lds_bytes(const GemmTile& t, int32_t num_experts);

// The tile `t`, or the per-wave tile of 64-row items when t is a workgroup
// tile whose output rows (128 or 256 of them, ldo BF16 values apart) would not
// fit one store resource: every kernel addresses one item's output rows with
// 32-bit buffer offsets below 2^31 - 4096 bytes.
GemmTile fit_output_range(const GemmTile& t, int64_t k, int64_t ldo);

// Rows of output one item of tile t covers.
int32_t item_rows(const GemmTile& t);

// With MOE_FP4_LOG set (to anything but "0"), print the tile an entry point
// chose to stderr, once per change of entry point, sizes or tile.
void log_tile(const char* entry, int32_t num_experts, int64_t m_total, int64_t n, int64_t k,
              int64_t ldo, const GemmTile& t);

struct GemmArgs {
  const uint8_t* a_q;
  const uint8_t* a_sf;
  const float* a_scale;
  const int32_t* a_row_index;
  const uint8_t* w_q;
  const uint8_t* w_sf;
  const float* w_scale;
  const int32_t* offsets;
  uint16_t* out;
  int64_t a_rows;
  int64_t m_total;
  int64_t n;
  int64_t k;
  int64_t ldo;
  int32_t num_experts;
  int32_t n_tiles;   // ceil(n / (16 * n_blocks))
  int32_t w_packed;  // w_q is in the packed layout
  // Experts this launch covers, by row count: rows_lo <= rows, and rows <
  // rows_hi unless rows_hi is 0 (so a zeroed GemmArgs covers every expert).
  // Launches over disjoint ranges write disjoint output rows.
  int32_t rows_lo;
  int32_t rows_hi;
  // Finalize epilogue only (moe_grouped_gemm_fp4_finalize): routed row r adds
  // row_weight[r] * its result into FP32 row out_token[r] of fin_out.
  const int32_t* out_token;
  const float* row_weight;
  float* fin_out;
  int64_t fin_ldo;
  int64_t num_tokens;
  // SwiGLU epilogue only (moe_grouped_gemm_fp4_swiglu): the NVFP4 intermediate
  // h_q [m_total][n/4], h_sf [m_total][n/32] at the static tensor scale *h_scale.
  uint8_t* h_q;
  uint8_t* h_sf;
  const float* h_scale;
};

hipError_t launch_grouped_gemm(const GemmArgs& args, const GemmTile& tile, hipStream_t stream);

// The same GEMM with the finalize epilogue (grouped_gemm_finalize.hip): per-wave
// kernels with 64-column items only.
hipError_t launch_grouped_gemm_finalize(const GemmArgs& args, const GemmTile& tile,
                                        hipStream_t stream);

// The same GEMM with the SwiGLU + NVFP4 epilogue (grouped_gemm_swiglu.hip):
// per-wave kernels, items of 32 intermediate columns (4 row blocks).
hipError_t launch_grouped_gemm_swiglu(const GemmArgs& args, const GemmTile& tile,
                                      hipStream_t stream);

// Workgroup-tiled kernel (grouped_gemm_tiled.hip): 128 x 128 items, 4 waves.
hipError_t launch_grouped_gemm_tiled(const GemmArgs& args, hipStream_t stream);
size_t tiled_lds(int32_t num_experts);

// Large-tile kernel (grouped_gemm_big.hip): 256 x 256 items, 8 waves of 128 x 64;
// f8: the split-K-by-scale-block FP8 variant.
hipError_t launch_grouped_gemm_big(const GemmArgs& args, bool f8, hipStream_t stream);
size_t big_lds(int32_t num_experts);

// Workgroup kernel for experts of a few dozen rows (grouped_gemm_mid.hip): 48 x 512
// items, 8 waves of 64 columns each, activations shared in LDS; needs k % 512 == 0.
// Sets its own n_tiles.
hipError_t launch_grouped_gemm_mid(const GemmArgs& args, hipStream_t stream);
size_t mid_lds(int32_t num_experts);

// LDS a workgroup may use on gfx950.
constexpr size_t kLdsBytes = 160 * 1024;

// Rows from which an expert takes the 256 x 256 tile when the problem is split
// by expert size (GemmTile.tiled == 2).  Measured on the Zipf prefill shard
// (256 experts, 4096 tokens top-8): 64 -> 397 us, 96 -> 303, 128 -> 316,
// 256 -> 352, 384 -> 359.
constexpr int32_t kBigRows = 96;

// Rows from which an expert takes the 48 x 512 items when per-wave items take
// the smaller experts (GemmTile.tiled 6 and 7): one 16-row block gains nothing
// from sharing the weight conversion.
constexpr int32_t kMidRows = 17;

}  // namespace moe_fp4
