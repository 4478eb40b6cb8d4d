// NVFP4 activation quantiser for gfx950.
//
// Packing (two 4-bit values per byte) and the 16-element FP8 block scale come
// from "Peering into the CUTLASS SharedStorage", section "Input Knowledge",
// item 3; the recipe (tensor scale amax / 2688, round-to-nearest-even block
// scale, IEEE division, round-to-nearest-even E2M1 code) is this library's
// definition, stated in moe_fp4.h.
//
// Kernels, in stream order:
//   DYNAMIC: amax -> quantize      STATIC: quantize
// The dynamic tensor scale needs the whole matrix's amax before any block can
// be encoded, so it takes two launches; it needs no scratch memory, no atomics
// and no reset launch.  Since g = fl(amax / 2688) is a non-decreasing function
// of amax, the maximum of the per-workgroup values fl(amax_wg / 2688) is g
// itself (0 for an all-zero matrix, for which g = 1).  The quantise launch is
// laid out so that its workgroup w writes, in its first pass, the codes of
// blocks [256 w, 256 w + 256): 2 KB of q that no other workgroup touches (the
// other blocks of that pass lie past the first `pieces` pieces).  The amax
// launch writes its P partial values into the first P floats of every such
// 2 KB piece (P <= 256 workgroups, at most 512 pieces); each quantise
// workgroup reduces the copy in its own piece, and only after a barrier that
// follows the reduction does it overwrite the piece with codes.  Workgroup 0
// also publishes g to the caller's tensor_scale.  A matrix of fewer than 256
// blocks takes one workgroup in each launch and one partial value.  The copies
// are scattered 4-byte stores, P per piece: with 512 partial values and 2048
// pieces they took 7 us of the amax launch on 4096 x 6144 BF16 values, hence
// the lower caps.
//
// One thread quantises one 16-element block at a time: 32 (BF16) or 64 (FP32)
// bytes in, 8 bytes of codes and 1 scale byte out, consecutive threads on
// consecutive blocks of a row, so every access is coalesced; each pass loads
// kQuantBlocks blocks per thread before encoding them.  The pass is HBM-bound:
// (2 or 4) + 0.5625 bytes per element.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "fp4_device.h"
#include "launch.h"

namespace moe_fp4 {
namespace {

constexpr int kThreads = 256;

// Sixteen consecutive input elements as floats (BF16 widens exactly).
template <int DT, typename I>
__device__ __forceinline__ void load_block16(const void* x, I row, int64_t ld_x, I b,
                                             float (&v)[16]) {
  if (DT == 0) {  // BF16
    const uint8_t* p = reinterpret_cast<const uint8_t*>(x) + ((int64_t)row * ld_x + (int64_t)b * 16) * 2;
    u32x4_t w0 = load_16B(p), w1 = load_16B(p + 16);
    uint32_t w[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    }
  } else {  // FP32
    const uint8_t* p = reinterpret_cast<const uint8_t*>(x) + ((int64_t)row * ld_x + (int64_t)b * 16) * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4_t w = load_16B(p + 16 * j);
      // Copy each lane to a scalar before the bit cast: a bit cast applied to
      // a vector-element expression does not read the selected lane.
      const uint32_t u[4] = {w[0], w[1], w[2], w[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * j + i] = __builtin_bit_cast(float, u[i]);
    }
  }
}

__global__ void k_set_one(float* ts) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *ts = 1.0f;
}

// Blocks per thread per iteration of the amax pass: all their loads are in
// flight before the reduction.  Measured on the 512 x 6144 BF16 decode
// activations (one pass per thread): 96 workgroups of 8 blocks per thread run
// the two launches in 8.4 us, against 8.8 us for 192 of 4, 9.7 for 384 of 2
// and 9.7 for 48 of 16.
constexpr int kAmaxBlocks = 8;
// Blocks per thread per iteration of the quantise pass.
constexpr int kQuantBlocks = 4;
// Blocks of one quantise workgroup's first pass, and the floats of q they
// cover (8 bytes of codes per block): room for this many partial values.
constexpr int kPiece = kThreads;
constexpr int kPieceFloats = kPiece * 8 / 4;
// Launch limits of the dynamic path: at most kMaxPartials amax workgroups and
// kMaxPieces quantise workgroups, so the amax launch writes at most
// kMaxPartials * kMaxPieces floats of partial values.  Measured on 4096 x 6144
// and 8192 x 8192 BF16 values (amax + quantise): 256 and 512, 24.2 and 51.9 us;
// 512 and 2048 with 4 amax blocks and 1 quantise block per thread, 29.4 and
// 57.3 us; 512 and 512, 24.9 and 53.0; 512 and 256, 26.0 and 57.4.
constexpr int kMaxPartials = kPieceFloats / 2;
constexpr int kMaxPieces = 512;

// Block-wide maximum of one float per thread (all threads must call it).
__device__ __forceinline__ float block_max(float m, float* wave_max) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = wave_max[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, wave_max[w]);
  return r;
}

// I: the index type (32-bit whenever rows * k/16 fits, which avoids 64-bit
// division in the index arithmetic).  Workgroup p reduces its share of the
// blocks to fl(amax / 2688) (0 if all its elements are 0) and stores it as
// float p of each of the `pieces` 2 KB pieces at the start of q.
template <int DT, typename I, int NB>
__global__ __launch_bounds__(kThreads) void k_amax(const void* x, int64_t rows, int64_t k,
                                                   int64_t ld_x, float* partials, int pieces) {
  __shared__ float wave_max[kThreads / 64];
  const I nb = (I)(k / 16);
  const I total = (I)rows * nb;
  const I stride = (I)gridDim.x * kThreads;
  float m = 0.0f;
  for (I blk = (I)blockIdx.x * kThreads + threadIdx.x; blk < total; blk += NB * stride) {
    float v[NB][16];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      // Past the end, re-read the last block: a duplicate leaves the max as it is.
      I bj = blk + (I)j * stride;
      bj = bj < total ? bj : total - 1;
      const I row = bj / nb;
      load_block16<DT, I>(x, row, ld_x, bj - row * nb, v[j]);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[j][i]));
  }
  const float wg = block_max(m, wave_max);
  const float g = wg / 2688.0f;  // IEEE division, rounded to nearest even (0 stays 0)
  for (int w = threadIdx.x; w < pieces; w += kThreads)
    partials[(int64_t)w * kPieceFloats + blockIdx.x] = g;
}

template <int DT, bool DYN, typename I>
__global__ __launch_bounds__(kThreads) void k_quantize(const void* x, int64_t rows, int64_t k,
                                                       int64_t ld_x, uint8_t* q, uint8_t* sf,
                                                       float* ts, int nparts) {
  float g;
  if constexpr (DYN) {
    // The amax launch's partial values, from this workgroup's own piece of q
    // (nparts <= kPieceFloats = 2 floats per thread).  block_max's barrier
    // orders these reads before any thread of the workgroup overwrites the
    // piece with codes.
    __shared__ float wave_max[kThreads / 64];
    const float* part = reinterpret_cast<const float*>(q) + (int64_t)blockIdx.x * kPieceFloats;
    const int t = threadIdx.x;
    float m = 0.0f;
    if (t < nparts) m = part[t];
    if (t + kThreads < nparts) m = fmaxf(m, part[t + kThreads]);
    const float mx = block_max(m, wave_max);
    g = mx > 0.0f ? mx : 1.0f;  // all-zero matrix: g = 1
    if (blockIdx.x == 0 && t == 0) *ts = g;
  } else {
    g = *ts;
  }
  const float six_g = 6.0f * g;
  const I nb = (I)(k / 16);
  const I total = (I)rows * nb;
  const I stride = (I)gridDim.x * kThreads;
  for (I blk0 = (I)blockIdx.x * kThreads + threadIdx.x; blk0 < total;
       blk0 += (I)kQuantBlocks * stride) {
    // All kQuantBlocks loads first (past the end, the last block again, unused).
    float vb[kQuantBlocks][16];
    I rowj[kQuantBlocks], bj[kQuantBlocks];
#pragma unroll
    for (int j = 0; j < kQuantBlocks; ++j) {
      I blk = blk0 + (I)j * stride;
      blk = blk < total ? blk : total - 1;
      rowj[j] = blk / nb;
      bj[j] = blk - rowj[j] * nb;
      load_block16<DT, I>(x, rowj[j], ld_x, bj[j], vb[j]);
    }
#pragma unroll
    for (int j = 0; j < kQuantBlocks; ++j) {
    if (blk0 + (I)j * stride >= total) break;
    const I row = rowj[j], b = bj[j];
    const float (&v)[16] = vb[j];
    float amax_b = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax_b = fmaxf(amax_b, fabsf(v[i]));
    // Block scale: E4M3 with round-to-nearest-even.  The hardware conversion
    // rounds to nearest even; clamping to 448 first makes it saturate.
    const float r = fminf(amax_b / six_g, 448.0f);
    const uint32_t sfb = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r, r, 0, false) & 0xFFu;
    const float s = __builtin_amdgcn_cvt_f32_fp8(sfb, 0) * g;
    uint32_t packed[2] = {0u, 0u};
    if (s >= 0x1p-100f && s <= 0x1p125f) {
      // The 16 quotients x / s share their divisor: one IEEE division gives
      // rs = RN(1/s), and each quotient is q = RN(x * rs) corrected once with
      // the exact residual, y = RN(q + RN(x - q s) * rs), Markstein's
      // correction, which equals RN(x / s) when rs = RN(1/s) and the residual
      // is exact.  With s >= 2^-100 the residual is exact for every quotient
      // of magnitude 2^-3 or more, the only ones whose E2M1 code is not zero;
      // smaller ones stay smaller and keep x's sign (s > 0, so the quotient's
      // sign is x's), which is all their code depends on.  q is clamped to
      // [-8, 8] first: from 8 up the code saturates anyway, and a quotient
      // that overflows (a static scale far below the data) then stays finite.
      // Checked on the CPU against the IEEE quotient's code on 2.1e9 pairs.
      const float rs = 1.0f / s;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float y[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float x = v[2 * i + h];
          const float q = __builtin_fminf(__builtin_fmaxf(x * rs, -8.0f), 8.0f);
          y[h] = __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q, s, x), rs, q), x);
        }
        // The hardware E2M1 conversion: nearest even, saturating, sign kept.
        const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0], y[1], 1.0f, 0) & 0xFFu;
        packed[i >> 2] |= c << (8 * (i & 3));
      }
    } else if (s != 0.0f) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // IEEE division (the compiler's correctly rounded sequence), then the
        // hardware E2M1 conversion: nearest even, saturating, sign kept.
        const float y0 = v[2 * i] / s, y1 = v[2 * i + 1] / s;
        const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y0, y1, 1.0f, 0) & 0xFFu;
        packed[i >> 2] |= c << (8 * (i & 3));
      }
    }
    *reinterpret_cast<u32x2_t*>(q + (int64_t)row * (k / 2) + (int64_t)b * 8) =
        u32x2_t{packed[0], packed[1]};
    sf[(int64_t)row * nb + b] = (uint8_t)sfb;
    }
  }
}


template <int DT, typename I>
hipError_t launch_dt(const void* x, int64_t rows, int64_t k, int64_t ld_x, uint8_t* q, uint8_t* sf,
                     float* ts, int dynamic, hipStream_t stream) {
  const int64_t total = rows * (k / 16);
  const int64_t want = (total + kThreads - 1) / kThreads;
  if (dynamic) {
    if (total > 0) {
      // Quantise workgroups: one whole 256-block piece each in the first pass
      // (the rest of the blocks follow in grid-stride passes), at most
      // kMaxPieces.  Amax workgroups: each thread covers kAmaxBlocks blocks
      // per pass, at most kMaxPartials; a matrix below one piece takes one.
      int64_t pieces = total / kPiece;
      if (pieces > kMaxPieces) pieces = kMaxPieces;
      int64_t parts = (want + kAmaxBlocks - 1) / kAmaxBlocks;
      if (parts > kMaxPartials) parts = kMaxPartials;
      if (pieces < 1) pieces = parts = 1;
      hipLaunchKernelGGL((k_amax<DT, I, kAmaxBlocks>), dim3((unsigned)parts), dim3(kThreads), 0,
                         stream, x, rows, k, ld_x, reinterpret_cast<float*>(q), (int)pieces);
      hipLaunchKernelGGL((k_quantize<DT, true, I>), dim3((unsigned)pieces), dim3(kThreads), 0,
                         stream, x, rows, k, ld_x, q, sf, ts, (int)parts);
    } else {
      hipLaunchKernelGGL(k_set_one, dim3(1), dim3(64), 0, stream, ts);
    }
  } else if (total > 0) {
    const int64_t groups = (want + kQuantBlocks - 1) / kQuantBlocks;
    const int grid = (int)(groups < 65536 ? groups : 65536);
    hipLaunchKernelGGL((k_quantize<DT, false, I>), dim3(grid), dim3(kThreads), 0, stream, x, rows,
                       k, ld_x, q, sf, ts, 0);
  }
  return hipGetLastError();
}

// 32-bit block indices when every index (including one stride past the last
// block) fits, 64-bit otherwise.  MOE_FP4_INDEX64=1 takes the 64-bit build at
// any size: the two builds must give the same bits, and only this switch lets a
// test run the 64-bit one on a matrix that fits in memory many times over.
template <int DT>
hipError_t launch_idx(const void* x, int64_t rows, int64_t k, int64_t ld_x, uint8_t* q, uint8_t* sf,
                      float* ts, int dynamic, hipStream_t stream) {
  const int64_t total = rows * (k / 16);
  const int64_t reach = total + (int64_t)kAmaxBlocks * kMaxPartials * kThreads +
                        (int64_t)kQuantBlocks * 65536LL * kThreads;
  const char* force = getenv("MOE_FP4_INDEX64");
  const bool wide = force && force[0] == '1' && force[1] == '\0';
  if (reach < INT32_MAX && !wide)
    return launch_dt<DT, int32_t>(x, rows, k, ld_x, q, sf, ts, dynamic, stream);
  return launch_dt<DT, int64_t>(x, rows, k, ld_x, q, sf, ts, dynamic, stream);
}

}  // namespace

hipError_t launch_quantize(const void* x, int in_dtype, int64_t rows, int64_t k, int64_t ld_x,
                           uint8_t* q, uint8_t* sf, float* tensor_scale, int dynamic,
                           hipStream_t stream) {
  if (in_dtype == 0) return launch_idx<0>(x, rows, k, ld_x, q, sf, tensor_scale, dynamic, stream);
  return launch_idx<1>(x, rows, k, ld_x, q, sf, tensor_scale, dynamic, stream);
}

}  // namespace moe_fp4
