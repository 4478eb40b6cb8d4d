// NVFP4 grouped GEMM for gfx950, workgroup-tiled variant for experts with many
// rows (prefill-sized experts, the dense case): the compute-bound end of the
// same grouped problem ("Peering into the CUTLASS Kernel", section "Input
// Knowledge Required", item 4), where the pages' large-GEMM figures apply
// ("Peering into the CUTLASS Kernel Cache", section "The Scene") and larger
// tiles raise data reuse ("Peering into the CUTLASS SharedStorage", section
// "Why This Matters").
//
// Design: a workgroup of 4 wavefronts computes a 128 x 128 output tile of one
// expert, each wavefront a 64 x 64 quarter.  Per 64-element K stage every
// thread loads one operand row's 32 code bytes and 4 block-scale bytes,
// dequantises them exactly to FP16 (the same exact map as the decode kernel)
// and writes them to a double-buffered LDS stage; after one barrier every
// wavefront reads its MFMA operands from LDS.  So each element is dequantised
// once per workgroup instead of once per wavefront that uses it, which is what
// bounds the per-wave kernel when experts are large.  The next stage's global
// loads are issued right after the current stage is written to LDS, so they
// are in flight during the MFMAs.  Work items (expert, 128-row M-tile, 128-
// column N-tile) come from the same device-side work list, one per workgroup
// per round.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_device.h"
#include "gemm_common.h"
#include "launch.h"

namespace moe_fp4 {
namespace {

constexpr int kTM = 128;              // output rows per item
constexpr int kTN = 128;              // output columns per item
constexpr int kTK = 64;               // K elements per stage
constexpr int kThreads = 256;         // 4 wavefronts, 2 x 2 over the tile
constexpr int kRowBytes = kTK * 2;    // one operand row of a stage in FP16
constexpr int kStageBytes = (kTM + kTN) * kRowBytes;  // 32 KB

// LDS: the work-list tables, then two stages.  A stage holds the 128 activation
// rows, then the 128 weight rows, each row as 8 chunks of 16 bytes (8 FP16
// values); chunk q of row r is stored at position q ^ (r % 8), so the 8 lanes
// writing one chunk index and the 16 lanes reading one MFMA K slice spread
// over the LDS banks.
__host__ __device__ constexpr size_t tiled_lds_bytes(int num_experts) {
  return worklist_bytes(num_experts) + 2 * (size_t)kStageBytes;
}

// Write one thread's 64 dequantised values (row r of the stage) to LDS.
__device__ __forceinline__ void write_row(uint8_t* stage, int row, const half8_t (&v)[8]) {
  uint8_t* base = stage + row * kRowBytes;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    *reinterpret_cast<half8_t*>(base + 16 * (q ^ (row & 7))) = v[q];
}

// MFMA operand of a 16-row block: lane (c, g) reads row `row0 + c`, K values
// 32*kk + 8g .. +7 of the stage.
__device__ __forceinline__ half8_t read_frag(const uint8_t* stage, int row0, int c, int g, int kk) {
  const int row = row0 + c;
  const int q = 4 * kk + g;
  return *reinterpret_cast<const half8_t*>(stage + row * kRowBytes + 16 * (q ^ (row & 7)));
}

template <int PD>
__global__ __launch_bounds__(kThreads) void k_grouped_gemm_tiled(const GemmArgs p) {
  static_assert(PD % 2 == 0, "stage ring must be even (LDS buffers alternate)");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int32_t* prefix = reinterpret_cast<int32_t*>(smem);
  int32_t* offl = prefix + (p.num_experts + 1);
  __shared__ int32_t wave_sum[kThreads / 64];
  uint8_t* const stages = smem + worklist_bytes(p.num_experts);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;   // this wave's 64 x 64 quarter
  // Loader role: waves 0-1 load activation rows, waves 2-3 weight rows (taken
  // from the uniform wave number so the resource choice stays scalar).
  const bool is_w = wave >= kTM / 64;
  const int lrow = tid & (kTM - 1);

  const int32_t total_items = build_worklist<kThreads>(p, kTM, prefix, offl, wave_sum);
  const WorkList wl{prefix, offl};

  const int nblk = gridDim.x, b = blockIdx.x;
  const int32_t rounds = (total_items + nblk - 1) / nblk;
  if (rounds == 0) return;
  const int32_t last_items = total_items - (rounds - 1) * nblk;
  const int32_t lb_full = logical_block(b, nblk, nblk);
  const int32_t lb_last = logical_block(b, nblk, last_items);
  const int32_t my_items = (rounds - 1) + (lb_last < last_items ? 1 : 0);

  const int32_t n = (int32_t)p.n, kb = (int32_t)(p.k >> 1), nbk = (int32_t)(p.k >> 4);
  const int32_t nst = (int32_t)(p.k / kTK);
  const rsrc_t a_rs = make_rsrc(p.a_q, (uint32_t)(p.a_rows * kb));
  const rsrc_t as_rs = make_rsrc(p.a_sf, (uint32_t)(p.a_rows * nbk));
  const int32_t a_last = (int32_t)p.a_rows - 1;
  // Packed weight layout: bytes of a 16-row block, and log2 of the stages per
  // granule (a granule of 256 or 512 elements holds 4 or 8 stages of 64).
  const int32_t pk_block = packed_block_bytes(packed_granule(p.k));
  const int32_t pk_lg = packed_granule(p.k) == 512 ? 3 : 2;

  int32_t from = 0;
  for (int32_t j = 0; j < my_items; ++j) {
    const int32_t item = j * nblk + (j == rounds - 1 ? lb_last : lb_full);
    const ItemPos it = locate(item, from, wl, p, kTM, kTN, lane);
    from = it.e;

    // This thread's operand row: a gathered activation row (rows past the
    // expert's end repeat its first row; never stored) or a weight row (past
    // n: out of range, reads zeros).
    rsrc_t rq, rs;
    uint32_t voff_q, voff_s;
    uint32_t half = 16;  // bytes from a stage's first 16 code bytes to its second
    int32_t wrg = 0;     // packed weights: 16-row blocks in this wave's 64-row group
    if (is_w) {
      rq = make_rsrc(p.w_q + (int64_t)it.e * n * kb, (uint32_t)(n * kb));
      rs = make_rsrc(p.w_sf + (int64_t)it.e * n * nbk, (uint32_t)(n * nbk));
      const int32_t row = it.n0 + lrow;
      if (p.w_packed) {
        // This wave's 64 rows are one group of the packed layout; a thread's
        // row is piece r of each 16-row block j of the group.
        const int32_t grp0 = uniform(it.n0 + (lrow & ~(kPackRows - 1)));
        // (A group wholly past n has no blocks: its rows read out of range and
        // its stage offsets stay small and non-negative.)
        const int32_t left = grp0 < n ? (n - grp0) / 16 : 0;
        wrg = left < 4 ? left : 4;
        const int32_t j = (row - grp0) >> 4, r = row & 15;
        voff_q = row < n ? (uint32_t)(grp0 * kb + j * pk_block + 16 * r) : kOutOfRange;
        half = 1024;
      } else {
        voff_q = row < n ? (uint32_t)(row * kb) : kOutOfRange;
      }
      voff_s = row < n ? (uint32_t)(row * nbk) : kOutOfRange;
    } else {
      const int32_t r = it.row0 + (lrow < it.rows_valid ? lrow : 0);
      int32_t src = p.a_row_index ? p.a_row_index[r] : r;
      src = src < 0 ? 0 : (src > a_last ? a_last : src);
      rq = a_rs;
      rs = as_rs;
      voff_q = (uint32_t)(src * kb);
      voff_s = (uint32_t)(src * nbk);
    }

    float4_t acc[4][4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) acc[jb][ib] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // A ring of PD register stages: stage st's 64 codes and 4 block scales are
    // loaded PD stages before they are dequantised, so the loads have PD
    // stages of MFMA work to arrive.  Stages past the last one are loaded out
    // of range (no traffic).
    u32x4_t q0[PD], q1[PD];
    uint32_t sc[PD];
    // Byte offset of stage st's codes: row-major, 32 bytes per stage along the
    // row; packed (weight waves), the stage's 32 bytes of a row are two
    // 16-byte pieces 1 KB apart in block j of granule t, at the position of
    // sub-step s and lane group g of the packed order.
    const bool wpk = is_w && p.w_packed;
    auto stage_off = [&](int32_t st) -> int32_t {
      if (!wpk) return st * (kTK / 2);
      const int32_t t = st >> pk_lg, m = st & ((1 << pk_lg) - 1);
      const int32_t g = m >> (pk_lg - 2), sub = m & ((1 << (pk_lg - 2)) - 1);
      return t * wrg * pk_block + sub * 2048 + g * 256;
    };
    auto load_stage = [&](int slot, int32_t st) {
      const bool in = st < nst;
      const uint32_t oq = in ? voff_q : kOutOfRange, os = in ? voff_s : kOutOfRange;
      const int32_t kq = uniform(stage_off(st)), ks = uniform(st * (kTK / 16));
      q0[slot] = __builtin_amdgcn_raw_buffer_load_b128(rq, oq, kq, 0);
      q1[slot] = __builtin_amdgcn_raw_buffer_load_b128(rq, oq + half, kq, 0);
      sc[slot] = __builtin_amdgcn_raw_buffer_load_b32(rs, os, ks, 0);
    };
    // Issue the ring in slot order (kept by the scheduling barriers) so the
    // oldest loads are the ones the first dequantisation needs.
#pragma unroll
    for (int d = 0; d < PD; ++d) {
      load_stage(d, d);
      __builtin_amdgcn_sched_barrier(0);
    }

    for (int32_t st0 = 0; st0 < nst; st0 += PD) {
#pragma unroll
      for (int d = 0; d < PD; ++d) {
        const int32_t st = st0 + d;
        uint8_t* const stage = stages + (d & 1) * kStageBytes;  // PD is even: d & 1 == st & 1
        // Dequantise this stage's row into LDS.
        {
          const half2_t s01 = scale_pair_x2m8<false>(sc[d]), s23 = scale_pair_x2m8<true>(sc[d]);
          const _Float16 bs[4] = {s01[0], s01[1], s23[0], s23[1]};
          half8_t v[8];
#pragma unroll
          for (int w = 0; w < 4; ++w) v[w] = dequant8(q0[d][w], bs[w >> 1]);
#pragma unroll
          for (int w = 0; w < 4; ++w) v[4 + w] = dequant8(q1[d][w], bs[2 + (w >> 1)]);
          write_row(stage, (is_w ? kTM : 0) + lrow, v);
        }
        load_stage(d, st + PD);
        __syncthreads();
        // 16 MFMAs per K32 slice over this wave's 64 x 64 quarter.
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          half8_t af[4], wf[4];
#pragma unroll
          for (int ib = 0; ib < 4; ++ib) af[ib] = read_frag(stage, 64 * wm + 16 * ib, c, g, kk);
#pragma unroll
          for (int jb = 0; jb < 4; ++jb) wf[jb] = read_frag(stage, kTM + 64 * wn + 16 * jb, c, g, kk);
#pragma unroll
          for (int jb = 0; jb < 4; ++jb)
#pragma unroll
            for (int ib = 0; ib < 4; ++ib)
              acc[jb][ib] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[jb], af[ib], acc[jb][ib], 0, 0, 0);
        }
      }
    }

    // Epilogue: rows 64*wm + 16*ib + c of the item, columns 64*wn + 16*jb +
    // 4g .. +3.  The store resource covers exactly the item's valid rows, so
    // rows past the expert's end are dropped; column blocks past n are skipped.
    {
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      // The host picks this tile only when 128 rows of ldo BF16 values stay
      // below 2^31 - 4096 bytes, so the resource size and every offset fit 31 bits.
      const uint32_t ldo = (uint32_t)p.ldo;
      const rsrc_t o = make_rsrc(p.out + (int64_t)it.row0 * ldo,
                                 (uint32_t)it.rows_valid * ldo * 2u);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        const int32_t col = it.n0 + 64 * wn + 16 * jb;
        if (col < n) {
#pragma unroll
          for (int ib = 0; ib < 4; ++ib) {
            const float4_t v = acc[jb][ib];
            const bf16x4_t bv = {(__bf16)(v[0] * it.alpha), (__bf16)(v[1] * it.alpha),
                                 (__bf16)(v[2] * it.alpha), (__bf16)(v[3] * it.alpha)};
            const uint32_t off = ((uint32_t)(64 * wm + 16 * ib + c) * ldo + (uint32_t)(col + 4 * g)) * 2u;
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, bv), o, off, 0, 0);
          }
        }
      }
    }
    // The next item's first stage writes stage buffer 0 while waves may still
    // be reading the last stage (buffer 1): order them.
    __syncthreads();
  }
}

size_t tiled_lds_of(int32_t num_experts) { return tiled_lds_bytes(num_experts); }

template <int PD>
hipError_t launch_pd(const GemmArgs& p, hipStream_t stream) {
  auto kern = k_grouped_gemm_tiled<PD>;
  const size_t lds = tiled_lds_bytes(p.num_experts);
  int resident = 0;
  hipError_t err = resident_groups(kern, kThreads, lds, &resident);
  if (err != hipSuccess) return err;
  // Upper bound on the number of items: the host does not see the offsets.
  const int64_t max_mtiles = p.m_total / kTM + (p.m_total < p.num_experts ? p.m_total : p.num_experts);
  const int64_t max_items = max_mtiles * p.n_tiles;
  int64_t grid = resident;
  if (max_items < grid) grid = max_items;
  if (grid < 1) grid = 1;
  grid = (grid + kXcds - 1) / kXcds * kXcds;  // whole rounds over the XCDs
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t tiled_lds(int32_t num_experts) { return tiled_lds_of(num_experts); }

hipError_t launch_grouped_gemm_tiled(const GemmArgs& p, hipStream_t stream) {
  // K is a multiple of 256, so the stage count (K / 64) is a multiple of the
  // ring depth.  A deeper ring (8) would take more than 256 VGPRs and halve
  // the waves per SIMD.
  return launch_pd<4>(p, stream);
}

}  // namespace moe_fp4
