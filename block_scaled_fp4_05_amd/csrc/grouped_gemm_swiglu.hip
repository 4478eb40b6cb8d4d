// NVFP4 grouped GEMM for the gate+up projection with the SwiGLU + NVFP4
// epilogue: each routed row's gate and up results meet in registers, pass
// through the gated SiLU and are quantised to NVFP4 at a static tensor scale,
// so the down projection reads 0.5625 bytes per intermediate element instead
// of a BF16 round trip ("Peering into the CUTLASS Kernel", section "Input
// Knowledge Required", item 5: the final-write epilogue, possibly with an
// activation and a quantisation).  The same per-wavefront kernel as the plain
// GEMM (grouped_gemm_kernel.h) with items of 32 intermediate columns (the 32
// gate rows and the 32 matching up rows of the weights); instantiated for one,
// two or four row blocks, 256- or 512-element stages, weight scales through
// registers or LDS, and either weight layout.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "grouped_gemm_kernel.h"

namespace moe_fp4 {
namespace {

template <int KSUB, bool SL, bool PK>
hipError_t launch_sw_mb(const GemmArgs& p, int m_blocks, hipStream_t stream) {
  switch (m_blocks) {
    case 1: return launch_tile<1, 4, KSUB, 4, SL, PK, kEpiSwiglu>(p, stream);
    case 2: return launch_tile<2, 4, KSUB, 4, SL, PK, kEpiSwiglu>(p, stream);
    case 4: return launch_tile<4, 4, KSUB, 4, SL, PK, kEpiSwiglu>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool SL, bool PK>
hipError_t launch_sw_k(const GemmArgs& p, const GemmTile& t, hipStream_t stream) {
  if (t.k_sub == 2) return launch_sw_mb<2, SL, PK>(p, t.m_blocks, stream);
  if (t.k_sub == 1) return launch_sw_mb<1, SL, PK>(p, t.m_blocks, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_grouped_gemm_swiglu(const GemmArgs& p, const GemmTile& t, hipStream_t stream) {
  if (t.tiled || t.n_blocks != 4 || t.waves != 4 || p.k % (256 * t.k_sub) != 0 || p.n % 32 != 0)
    return hipErrorInvalidValue;
  if (p.w_packed && (p.n / 2) % 64 != 0) return hipErrorInvalidValue;
  if (t.lds_scales) {
    if (p.k % 2048 != 0) return hipErrorInvalidValue;
    return p.w_packed ? launch_sw_k<true, true>(p, t, stream) : launch_sw_k<true, false>(p, t, stream);
  }
  return p.w_packed ? launch_sw_k<false, true>(p, t, stream) : launch_sw_k<false, false>(p, t, stream);
}

}  // namespace moe_fp4
