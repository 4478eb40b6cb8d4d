// NVFP4 grouped GEMM with the finalize epilogue: every routed row's result,
// times its routing weight, is added into its token's FP32 output row (the
// final output write of the Mixture-of-Experts down projection; "Peering into
// the CUTLASS Kernel", section "Input Knowledge Required", item 5).  The same
// per-wavefront kernel as the plain GEMM (grouped_gemm_kernel.h) with the
// epilogue swapped; instantiated for 64-column items with one, two or four row
// blocks, 256- or 512-element stages, weight scales through registers or LDS,
// and either weight layout.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "grouped_gemm_kernel.h"

namespace moe_fp4 {
namespace {

template <int KSUB, bool SL, bool PK>
hipError_t launch_fin_mb(const GemmArgs& p, int m_blocks, hipStream_t stream) {
  switch (m_blocks) {
    case 1: return launch_tile<1, 4, KSUB, 4, SL, PK, kEpiFinalize>(p, stream);
    case 2: return launch_tile<2, 4, KSUB, 4, SL, PK, kEpiFinalize>(p, stream);
    case 4: return launch_tile<4, 4, KSUB, 4, SL, PK, kEpiFinalize>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool SL, bool PK>
hipError_t launch_fin_k(const GemmArgs& p, const GemmTile& t, hipStream_t stream) {
  if (t.k_sub == 2) return launch_fin_mb<2, SL, PK>(p, t.m_blocks, stream);
  if (t.k_sub == 1) return launch_fin_mb<1, SL, PK>(p, t.m_blocks, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_grouped_gemm_finalize(const GemmArgs& p, const GemmTile& t, hipStream_t stream) {
  if (t.tiled || t.n_blocks != 4 || t.waves != 4 || p.k % (256 * t.k_sub) != 0)
    return hipErrorInvalidValue;
  if (t.lds_scales) {
    if (p.k % 2048 != 0) return hipErrorInvalidValue;
    return p.w_packed ? launch_fin_k<true, true>(p, t, stream) : launch_fin_k<true, false>(p, t, stream);
  }
  return p.w_packed ? launch_fin_k<false, true>(p, t, stream) : launch_fin_k<false, false>(p, t, stream);
}

}  // namespace moe_fp4
