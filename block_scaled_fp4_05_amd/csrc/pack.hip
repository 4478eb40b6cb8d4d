// Weight-code repacking between the row-major layout and the packed layout
// the grouped GEMM's wavefronts load in (layout defined in moe_fp4.h).
//
// Expert weights are constant across calls, so they are rearranged once: in
// the packed layout every load instruction of the GEMM reads 1 KB of
// consecutive bytes and one pipeline stage of a 64-column work item reads one
// consecutive block, where the row-major layout spreads a stage over 64 row
// segments a row pitch apart.  A pure byte permutation, HBM-bound: one thread
// per 16-byte piece, walking the packed side in order so that side is read or
// written in full consecutive lines.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace moe_fp4 {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Row-major byte offset (within one expert) of the 16-byte piece at packed
// byte offset `off`.
__host__ __device__ inline uint32_t rowmajor_offset(uint32_t off, uint32_t n, uint32_t kb,
                                                    uint32_t granule) {
  const uint32_t gb = granule / 2;                  // code bytes per row per granule
  const uint32_t bb = packed_block_bytes(granule);  // 16 rows x gb
  const uint32_t group_bytes = kPackRows * kb;
  const uint32_t q = off / group_bytes;
  const uint32_t o1 = off - q * group_bytes;
  const uint32_t left = n / 16 - 4 * q;
  const uint32_t rg = left < 4 ? left : 4;          // 16-row blocks in this group
  const uint32_t t = o1 / (rg * bb);                // granule
  const uint32_t o2 = o1 - t * rg * bb;
  const uint32_t j = o2 / bb;                       // row block in the group
  const uint32_t piece = (o2 - j * bb) / 16;
  const uint32_t r = piece & 15, g = (piece >> 4) & 3, h = (piece >> 6) & 1, s = piece >> 7;
  const uint32_t row = kPackRows * q + 16 * j + r;
  return row * kb + t * gb + (gb / 4) * g + 32 * s + 16 * h;
}

template <bool TO_PACKED>
__global__ __launch_bounds__(256) void k_repack(const uint8_t* __restrict__ src,
                                                uint8_t* __restrict__ dst, uint32_t n,
                                                uint32_t kb, uint32_t granule) {
  const uint32_t bytes = n * kb;  // one expert; < 2^31 (checked on the host)
  const size_t base = (size_t)blockIdx.y * bytes;
  const uint8_t* s = src + base;
  uint8_t* d = dst + base;
  for (uint32_t off = (blockIdx.x * 256u + threadIdx.x) * 16u; off < bytes;
       off += gridDim.x * 256u * 16u) {
    const uint32_t rm = rowmajor_offset(off, n, kb, granule);
    if (TO_PACKED) {
      *reinterpret_cast<u32x4_t*>(d + off) = *reinterpret_cast<const u32x4_t*>(s + rm);
    } else {
      *reinterpret_cast<u32x4_t*>(d + rm) = *reinterpret_cast<const u32x4_t*>(s + off);
    }
  }
}

}  // namespace

hipError_t launch_repack(const uint8_t* src, uint8_t* dst, int32_t num_experts, int64_t n,
                         int64_t k, bool to_packed, hipStream_t stream) {
  const uint32_t kb = (uint32_t)(k / 2);
  const uint32_t pieces = (uint32_t)(n * kb / 16);
  // About 2048 workgroups in all, at least one per expert.
  uint32_t gx = (2048u + (uint32_t)num_experts - 1) / (uint32_t)num_experts;
  const uint32_t need = (pieces + 255u) / 256u;
  if (gx > need) gx = need;
  if (gx < 1) gx = 1;
  const dim3 grid(gx, (unsigned)num_experts);
  if (to_packed)
    hipLaunchKernelGGL(k_repack<true>, grid, dim3(256), 0, stream, src, dst, (uint32_t)n, kb,
                       (uint32_t)packed_granule(k));
  else
    hipLaunchKernelGGL(k_repack<false>, grid, dim3(256), 0, stream, src, dst, (uint32_t)n, kb,
                       (uint32_t)packed_granule(k));
  return hipGetLastError();
}

}  // namespace moe_fp4
