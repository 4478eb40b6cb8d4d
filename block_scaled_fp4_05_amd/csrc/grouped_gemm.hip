// NVFP4 block-scaled MoE grouped GEMM for gfx950.
//
// The problem: one GEMM per expert over the rows routed to it, all experts in
// one launch ("Peering into the CUTLASS Kernel Cache", section "Knowledge
// Required", MoE item; "Peering into the CUTLASS Kernel", section "Input
// Knowledge Required", item 4).  At decode an expert sees 16-64 rows, far
// below what makes a GEMM compute-bound (same page, "Context"), so the kernel
// is built to stream the weights once at HBM speed; the pages' SM120 tiles,
// TMA and warp-specialised schedules are not reused.
//
// Design (one MI355X = 256 CUs in 8 XCDs, 64-lane wavefronts):
//  * Work list.  An item is (expert e, M-tile of 16*MB rows, N-tile of 16*NBW
//    columns).  Each workgroup scans the expert offsets once into an LDS
//    prefix array of item counts; empty experts own no items and their
//    weights are never read.  Items are numbered expert-major, N-tile, then
//    M-tile fastest, so the M-tiles of one (expert, N-tile) run side by side
//    and share that weight tile through L2.
//  * Persistent wavefronts.  Every wavefront walks its own items (stride =
//    number of wavefronts); no inter-wave synchronisation after the prefix.
//    Workgroup ids are remapped so consecutive items land on the same XCD
//    (the hardware deals workgroups round-robin over the 8 XCDs), keeping an
//    expert's activation rows in one L2.
//  * Loads.  K advances 256 elements per step.  For a 16-row block, lane
//    (c = lane % 16, g = lane / 16) loads 32 contiguous bytes (64 codes) of row
//    c at byte 32g of the step's 128-byte span, plus the 4 scale bytes of those
//    64 codes: every 16-byte global load is a full-lane vector load straight
//    into registers, already in MFMA operand order.  The contraction order
//    over K is free, so MFMA t (0..7) of the step takes codes 8t..8t+7 of every
//    lane; weights and activations use the same K order.
//  * Pipelining.  The next (item, K-step) unit's loads are issued before the
//    current unit is computed, across item boundaries too, so a wave keeps a
//    step of loads in flight while it dequantises and multiplies.
//  * Math.  Codes are dequantised exactly to FP16 (fp4_device.h) and fed to
//    v_mfma_f32_16x16x32_f16 with FP32 accumulation: weights are the A operand
//    (16 output columns), activations the B operand (16 rows).  The 16-element
//    E4M3 block scales are applied during dequantisation, exactly, so CDNA4's
//    scaled FP4 MFMA (32-element E8M0 scales) is not used.
//  * Epilogue.  acc * a_scale * w_scale[e] -> BF16 (round to nearest even),
//    each lane storing 4 consecutive columns (8 bytes) of one row; rows past the
//    expert's end and column blocks past n are not written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_device.h"
#include "launch.h"

namespace moe_fp4 {
namespace {

constexpr int kXcds = 8;

__device__ __forceinline__ int64_t clamp_off(int32_t v, int64_t m_total) {
  int64_t x = v;
  return x < 0 ? 0 : (x > m_total ? m_total : x);
}

// Register image of one K-step for one wavefront: per 16-row block, 32 code
// bytes and 4 scale bytes per lane.
template <int MB, int NBW>
struct Stage {
  u32x4_t w[NBW][2];
  uint32_t ws[NBW];
  u32x4_t a[MB][2];
  uint32_t as[MB];
};

// Where a wavefront's current item lives.
struct Item {
  int32_t e;
  int32_t rows_valid;  // rows of this M-tile that belong to the expert (1..16*MB)
  int64_t row0;        // first output row of the M-tile
  int32_t n0;          // first output column of the N-tile
};

template <int MB, int NBW>
__device__ __forceinline__ Item decode_item(int32_t i, const int32_t* prefix, const GemmArgs& p) {
  constexpr int BM = 16 * MB;
  int lo = 0, hi = p.num_experts;  // prefix[lo] <= i < prefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= i) lo = mid; else hi = mid;
  }
  const int64_t r_lo = clamp_off(p.offsets[lo], p.m_total);
  const int64_t r_hi = clamp_off(p.offsets[lo + 1], p.m_total);
  const int32_t cnt = (int32_t)(r_hi - r_lo);
  const int32_t mts = (cnt + BM - 1) / BM;
  const int32_t local = i - prefix[lo];
  const int32_t nt = local / mts, mt = local - nt * mts;
  Item it;
  it.e = lo;
  it.row0 = r_lo + (int64_t)mt * BM;
  const int32_t left = cnt - mt * BM;
  it.rows_valid = left < BM ? left : BM;
  it.n0 = nt * 16 * NBW;
  return it;
}

// Source activation row (gathered, clamped) of each 16-row block for this lane.
template <int MB>
__device__ __forceinline__ void source_rows(const Item& it, int c, const GemmArgs& p,
                                            int64_t (&src)[MB]) {
#pragma unroll
  for (int ib = 0; ib < MB; ++ib) {
    const int rr = 16 * ib + c;
    const int64_t r = it.row0 + (rr < it.rows_valid ? rr : 0);
    int64_t s = p.a_row_index ? (int64_t)p.a_row_index[r] : r;
    s = s < 0 ? 0 : (s >= p.a_rows ? p.a_rows - 1 : s);
    src[ib] = s;
  }
}

template <int MB, int NBW>
__device__ __forceinline__ void issue_loads(Stage<MB, NBW>& st, const Item& it,
                                            const int64_t (&src)[MB], int ks, int c, int g,
                                            const GemmArgs& p) {
  const int64_t kb = p.k >> 1, nbk = p.k >> 4;
  const int64_t qoff = (int64_t)ks * 128 + 32 * g;
  const int64_t soff = (int64_t)ks * 16 + 4 * g;
#pragma unroll
  for (int jb = 0; jb < NBW; ++jb) {
    if (it.n0 + 16 * jb < p.n) {
      const int64_t wrow = (int64_t)it.e * p.n + it.n0 + 16 * jb + c;
      const uint8_t* wq = p.w_q + wrow * kb + qoff;
      st.w[jb][0] = load_16B(wq);
      st.w[jb][1] = load_16B(wq + 16);
      st.ws[jb] = load_4B(p.w_sf + wrow * nbk + soff);
    }
  }
#pragma unroll
  for (int ib = 0; ib < MB; ++ib) {
    if (16 * ib < it.rows_valid) {
      const uint8_t* aq = p.a_q + src[ib] * kb + qoff;
      st.a[ib][0] = load_16B(aq);
      st.a[ib][1] = load_16B(aq + 16);
      st.as[ib] = load_4B(p.a_sf + src[ib] * nbk + soff);
    }
  }
}

template <int MB, int NBW>
__device__ __forceinline__ void compute_stage(const Stage<MB, NBW>& st, const Item& it,
                                              const GemmArgs& p, float4_t (&acc)[NBW][MB]) {
  // Block scales of this step, as FP16 value * 2^-8: scale t/2 serves MFMA t.
  half2_t wsc[NBW][2], asc[MB][2];
#pragma unroll
  for (int jb = 0; jb < NBW; ++jb) {
    wsc[jb][0] = scale_pair_x2m8<false>(st.ws[jb]);
    wsc[jb][1] = scale_pair_x2m8<true>(st.ws[jb]);
  }
#pragma unroll
  for (int ib = 0; ib < MB; ++ib) {
    asc[ib][0] = scale_pair_x2m8<false>(st.as[ib]);
    asc[ib][1] = scale_pair_x2m8<true>(st.as[ib]);
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int half = t >> 2, word = t & 3, sidx = (t >> 1) & 1, spair = t >> 2;
    half8_t af[MB];
#pragma unroll
    for (int ib = 0; ib < MB; ++ib) {
      if (16 * ib < it.rows_valid) af[ib] = dequant8(st.a[ib][half][word], asc[ib][spair][sidx]);
    }
#pragma unroll
    for (int jb = 0; jb < NBW; ++jb) {
      if (it.n0 + 16 * jb < p.n) {
        const half8_t wf = dequant8(st.w[jb][half][word], wsc[jb][spair][sidx]);
#pragma unroll
        for (int ib = 0; ib < MB; ++ib) {
          if (16 * ib < it.rows_valid)
            acc[jb][ib] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf, af[ib], acc[jb][ib], 0, 0, 0);
        }
      }
    }
  }
}

template <int MB, int NBW>
__device__ __forceinline__ void epilogue(float4_t (&acc)[NBW][MB], const Item& it, int c, int g,
                                         const GemmArgs& p) {
  const float alpha = p.a_scale[0] * p.w_scale[it.e];
#pragma unroll
  for (int jb = 0; jb < NBW; ++jb) {
#pragma unroll
    for (int ib = 0; ib < MB; ++ib) {
      const int rr = 16 * ib + c;
      if (it.n0 + 16 * jb < p.n && rr < it.rows_valid) {
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        const float4_t v = acc[jb][ib];
        const bf16x4_t b = {(__bf16)(v[0] * alpha), (__bf16)(v[1] * alpha),
                            (__bf16)(v[2] * alpha), (__bf16)(v[3] * alpha)};
        uint16_t* o = p.out + (it.row0 + rr) * p.ldo + it.n0 + 16 * jb + 4 * g;
        *reinterpret_cast<u32x2_t*>(o) = __builtin_bit_cast(u32x2_t, b);
      }
      acc[jb][ib] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }
}

template <int MB, int NBW, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_grouped_gemm(const GemmArgs p) {
  constexpr int BM = 16 * MB;
  constexpr int NTHR = WAVES * 64;
  extern __shared__ int32_t prefix[];  // [num_experts + 1] item prefix
  __shared__ int32_t wave_sum[WAVES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.num_experts;

  // ---- work list: exclusive prefix over experts of (M-tiles * N-tiles) ----
  {
    const int per = (E + NTHR - 1) / NTHR;
    const int beg = tid * per < E ? tid * per : E;
    const int end = beg + per < E ? beg + per : E;
    int32_t local = 0;
    for (int e = beg; e < end; ++e) {
      const int64_t cnt = clamp_off(p.offsets[e + 1], p.m_total) - clamp_off(p.offsets[e], p.m_total);
      local += cnt > 0 ? (int32_t)((cnt + BM - 1) / BM) * p.n_tiles : 0;
    }
    int32_t incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t t = __shfl_up(incl, d, 64);
      if (lane >= d) incl += t;
    }
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    int32_t base = 0;
    for (int w = 0; w < wave; ++w) base += wave_sum[w];
    int32_t run = base + incl - local;
    for (int e = beg; e < end; ++e) {
      prefix[e] = run;
      const int64_t cnt = clamp_off(p.offsets[e + 1], p.m_total) - clamp_off(p.offsets[e], p.m_total);
      run += cnt > 0 ? (int32_t)((cnt + BM - 1) / BM) * p.n_tiles : 0;
    }
    if (tid == NTHR - 1) prefix[E] = base + incl;
    __syncthreads();
  }
  const int32_t total_items = prefix[E];

  // ---- XCD-aware wavefront numbering ----
  const int nblk = gridDim.x, b = blockIdx.x;
  const int xcd = b % kXcds, slot = b / kXcds;
  const int per_xcd = nblk / kXcds, rem = nblk % kXcds;
  const int lblk = xcd * per_xcd + (xcd < rem ? xcd : rem) + slot;
  const int32_t lw = lblk * WAVES + wave;
  const int32_t nw = nblk * WAVES;
  if (lw >= total_items) return;

  const int c = lane & 15, g = lane >> 4;
  const int nks = (int)(p.k / kKStep);
  const int32_t my_items = (total_items - lw + nw - 1) / nw;
  const int64_t units = (int64_t)my_items * nks;

  float4_t acc[NBW][MB];
#pragma unroll
  for (int jb = 0; jb < NBW; ++jb)
#pragma unroll
    for (int ib = 0; ib < MB; ++ib) acc[jb][ib] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  Stage<MB, NBW> s0, s1;
  // Item of the unit being loaded (ld_*) and of the unit being computed (cp_*).
  int32_t ld_item = lw;
  int ld_ks = 0;
  Item ld_it = decode_item<MB, NBW>(ld_item, prefix, p);
  int64_t ld_src[MB];
  source_rows<MB>(ld_it, c, p, ld_src);
  Item cp_it = ld_it;

  auto advance = [&]() {
    if (++ld_ks == nks) {
      ld_ks = 0;
      ld_item += nw;
      ld_it = decode_item<MB, NBW>(ld_item, prefix, p);
      source_rows<MB>(ld_it, c, p, ld_src);
    }
  };

  issue_loads<MB, NBW>(s0, ld_it, ld_src, ld_ks, c, g, p);
  int cp_ks = 0;
  for (int64_t u = 0; u < units; u += 2) {
    // even unit: prefetch u+1 into s1, compute s0
    const bool has1 = u + 1 < units;
    if (has1) {
      advance();
      issue_loads<MB, NBW>(s1, ld_it, ld_src, ld_ks, c, g, p);
    }
    compute_stage<MB, NBW>(s0, cp_it, p, acc);
    if (++cp_ks == nks) {
      epilogue<MB, NBW>(acc, cp_it, c, g, p);
      cp_ks = 0;
      if (has1) cp_it = ld_it;
    }
    if (!has1) break;
    // odd unit: prefetch u+2 into s0, compute s1
    const bool has2 = u + 2 < units;
    if (has2) {
      advance();
      issue_loads<MB, NBW>(s0, ld_it, ld_src, ld_ks, c, g, p);
    }
    compute_stage<MB, NBW>(s1, cp_it, p, acc);
    if (++cp_ks == nks) {
      epilogue<MB, NBW>(acc, cp_it, c, g, p);
      cp_ks = 0;
      if (has2) cp_it = ld_it;
    }
  }
}

template <int MB, int NBW, int WAVES>
hipError_t launch_tile(const GemmArgs& p, hipStream_t stream) {
  auto kern = k_grouped_gemm<MB, NBW, WAVES>;
  const size_t lds = sizeof(int32_t) * ((size_t)p.num_experts + 1);
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  int cus = 0;
  err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  int per_cu = 0;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, WAVES * 64, lds);
  if (err != hipSuccess) return err;
  if (per_cu < 1) per_cu = 1;
  // Upper bound on the number of items: the host does not see the offsets.
  constexpr int BM = 16 * MB;
  const int64_t max_mtiles = p.m_total / BM + (p.m_total < p.num_experts ? p.m_total : p.num_experts);
  const int64_t max_items = max_mtiles * p.n_tiles;
  int64_t grid = (int64_t)cus * per_cu;
  const int64_t need = (max_items + WAVES - 1) / WAVES;
  if (need < grid) grid = need;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WAVES * 64), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

GemmTile choose_tile(int32_t num_experts, int64_t m_total, int64_t n, int64_t k, const char* env) {
  (void)n;
  (void)k;
  GemmTile t{1, 4, 4};
  const int64_t avg = num_experts > 0 ? (m_total + num_experts - 1) / num_experts : m_total;
  if (avg > 32) t.m_blocks = 4;
  else if (avg > 16) t.m_blocks = 2;
  if (env && *env) {
    int bm = 0, bn = 0;
    const char* s = env;
    while (*s >= '0' && *s <= '9') bm = bm * 10 + (*s++ - '0');
    if (*s == 'x' || *s == 'X') {
      ++s;
      while (*s >= '0' && *s <= '9') bn = bn * 10 + (*s++ - '0');
      if ((bm == 16 || bm == 32 || bm == 64) && (bn == 32 || bn == 64) && *s == '\0') {
        t.m_blocks = bm / 16;
        t.n_blocks = bn / 16;
      }
    }
  }
  return t;
}

int64_t gemm_lds_bytes(const GemmTile& t, int32_t num_experts) {
  return (int64_t)sizeof(int32_t) * ((int64_t)num_experts + 1 + t.waves);
}

hipError_t launch_grouped_gemm(const GemmArgs& p, const GemmTile& t, hipStream_t stream) {
  if (t.waves != 4) return hipErrorInvalidValue;
  if (t.n_blocks == 4) {
    switch (t.m_blocks) {
      case 1: return launch_tile<1, 4, 4>(p, stream);
      case 2: return launch_tile<2, 4, 4>(p, stream);
      case 4: return launch_tile<4, 4, 4>(p, stream);
      default: break;
    }
  } else if (t.n_blocks == 2) {
    switch (t.m_blocks) {
      case 1: return launch_tile<1, 2, 4>(p, stream);
      case 2: return launch_tile<2, 2, 4>(p, stream);
      case 4: return launch_tile<4, 2, 4>(p, stream);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace moe_fp4
