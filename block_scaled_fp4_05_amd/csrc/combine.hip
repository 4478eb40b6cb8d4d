// MoE finalize as a token-order pass (moe_fp4_combine): each token's output row is
// the routing-weighted sum of its top-k routed rows, read from the grouped GEMM's
// BF16 output through the token -> rows map, summed in FP32 in slot order and
// written once (the final output write of the Mixture-of-Experts down
// projection, "Peering into the CUTLASS Kernel", section "Input Knowledge
// Required", item 5).
//
// Why a pass of its own on MI355X: a token's rows come from different experts,
// so the GEMM's work items that produce them run on all 8 XCDs, whose L2 caches
// are separate; adding them in the GEMM's epilogue takes device-wide atomics that
// resolve beyond the L2, one per element (moe_grouped_gemm_fp4_finalize).  Here
// every output element is read k times and written once with plain coalesced
// accesses, in a fixed order, so the result is reproducible bit for bit.
//
// Layout: one wavefront per (token, 512-column chunk): lane l owns columns
// 8l .. 8l+7 of the chunk, reads 16 bytes of each routed row and keeps eight
// FP32 sums.  HBM-bound: k * 2 bytes read (+ 4 of residual) and 2 or 4 written
// per output element.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_device.h"
#include "gemm_common.h"
#include "launch.h"

namespace moe_fp4 {
namespace {

constexpr int kCombineThreads = 256;
constexpr int kChunk = 512;  // output columns per wavefront

template <bool F32_OUT, bool RES>
__global__ __launch_bounds__(kCombineThreads) void k_combine(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t chunks = (a.n + kChunk - 1) / kChunk;
  const int64_t total = a.num_tokens * chunks;
  const rsrc_t rows_rs = make_rsrc(a.rows, (uint32_t)(a.m_total * a.ld_rows * 2));
  const rsrc_t out_rs = make_rsrc(a.out, (uint32_t)(a.num_tokens * a.ldo * (F32_OUT ? 4 : 2)));
  const rsrc_t res_rs = make_rsrc(a.residual, RES ? (uint32_t)(a.num_tokens * a.ld_res * 4) : 0u);
  const int64_t waves = (int64_t)gridDim.x * (kCombineThreads / 64);
  for (int64_t wv = (int64_t)blockIdx.x * (kCombineThreads / 64) + uniform(threadIdx.x >> 6);
       wv < total; wv += waves) {
    const int64_t t = wv / chunks;
    const int32_t col = (int32_t)(wv - t * chunks) * kChunk + 8 * lane;
    const bool col_ok = col < a.n;  // n % 16 == 0: a lane's 8 columns are all in or all out
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int32_t s = 0; s < a.topk; ++s) {
      const int32_t r = uniform(a.token_rows[t * a.topk + s]);
      const float w = __builtin_bit_cast(float, uniform(__builtin_bit_cast(int32_t, a.token_weights[t * a.topk + s])));
      if (r < 0 || r >= a.m_total) continue;  // uniform: no row in this slot
      const uint32_t off = col_ok ? (uint32_t)(((int64_t)r * a.ld_rows + col) * 2) : kOutOfRange;
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rows_rs, off, 0, 0);
      const uint32_t vv[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = __builtin_bit_cast(float, vv[i] << 16);
        const float hi = __builtin_bit_cast(float, vv[i] & 0xFFFF0000u);
        acc[2 * i] = acc[2 * i] + w * lo;
        acc[2 * i + 1] = acc[2 * i + 1] + w * hi;
      }
    }
    if (RES) {
      const uint32_t roff = col_ok ? (uint32_t)((t * a.ld_res + col) * 4) : kOutOfRange;
      const u32x4_t r0 = __builtin_amdgcn_raw_buffer_load_b128(res_rs, roff, 0, 0);
      const u32x4_t r1 = __builtin_amdgcn_raw_buffer_load_b128(res_rs, roff + 16u, 0, 0);
      // Copy the elements to scalars before the bit cast: a bit cast applied to a
      // vector-element expression does not read the selected element.
      const uint32_t rr[8] = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_bit_cast(float, rr[i]) + acc[i];
    }
    if (F32_OUT) {
      const uint32_t ooff = col_ok ? (uint32_t)((t * a.ldo + col) * 4) : kOutOfRange;
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4_t{__builtin_bit_cast(uint32_t, acc[0]), __builtin_bit_cast(uint32_t, acc[1]),
                  __builtin_bit_cast(uint32_t, acc[2]), __builtin_bit_cast(uint32_t, acc[3])},
          out_rs, ooff, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4_t{__builtin_bit_cast(uint32_t, acc[4]), __builtin_bit_cast(uint32_t, acc[5]),
                  __builtin_bit_cast(uint32_t, acc[6]), __builtin_bit_cast(uint32_t, acc[7])},
          out_rs, ooff + 16u, 0, 0);
    } else {
      typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
      const bf16x8_t b = {(__bf16)acc[0], (__bf16)acc[1], (__bf16)acc[2], (__bf16)acc[3],
                          (__bf16)acc[4], (__bf16)acc[5], (__bf16)acc[6], (__bf16)acc[7]};
      const uint32_t ooff = col_ok ? (uint32_t)((t * a.ldo + col) * 2) : kOutOfRange;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, b), out_rs, ooff, 0, 0);
    }
  }
}

template <bool F32_OUT>
hipError_t launch_res(const CombineArgs& a, hipStream_t stream, int grid) {
  if (a.residual)
    hipLaunchKernelGGL((k_combine<F32_OUT, true>), dim3(grid), dim3(kCombineThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((k_combine<F32_OUT, false>), dim3(grid), dim3(kCombineThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  const int64_t chunks = (a.n + kChunk - 1) / kChunk;
  const int64_t waves = a.num_tokens * chunks;
  int64_t grid = (waves + kCombineThreads / 64 - 1) / (kCombineThreads / 64);
  if (grid > 65536) grid = 65536;
  if (grid < 1) grid = 1;
  return a.f32_out ? launch_res<true>(a, stream, (int)grid) : launch_res<false>(a, stream, (int)grid);
}

}  // namespace moe_fp4
