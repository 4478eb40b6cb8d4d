// NVFP4 grouped GEMM for gfx950, large-tile variant for the compute-bound end
// of the grouped problem (prefill-sized experts and the dense case; "Peering
// into the CUTLASS Kernel", section "Input Knowledge Required", item 4, with
// the reuse argument of "Peering into the CUTLASS SharedStorage", section
// "Why This Matters": larger tiles re-read less data per multiply-add).
//
// The exact path multiplies dequantised FP16 values on the FP16 MFMA.  A
// workgroup of 8 wavefronts (two per SIMD) computes a 256 x 256 tile, each
// wavefront a 128 x 64 piece with v_mfma_f32_32x32x16_f16 (8 accumulator tiles
// of 32 x 32).  Per 64-element K stage every thread loads one operand row's 32
// code bytes and 4 block-scale bytes (waves 0-3 activation rows, waves 4-7
// weight rows; a register ring keeps PD stages of loads in flight), dequantises
// it exactly to FP16 (fp4_device.h) and writes it to the next of two 64 KB LDS
// stages while the MFMAs of the current stage run.  Each element is
// dequantised once per workgroup; what the MFMAs read from LDS per stage (192
// KB) and what the threads write (64 KB) stay under the MFMA time at 256 bytes
// per clock, and the second wavefront of each SIMD issues while the first waits.
// Items (expert, 256-row M-tile, 256-column N-tile) come from the device-side
// work list, one per workgroup per round.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_device.h"
#include "gemm_common.h"
#include "launch.h"

namespace moe_fp4 {
namespace {

constexpr int kBM = 256;                 // output rows per item
constexpr int kBN = 256;                 // output columns per item
constexpr int kBK = 64;                  // K elements per stage
constexpr int kBThreads = 512;           // 8 wavefronts: 2 (rows) x 4 (columns)
constexpr int kBRow = kBK * 2;           // one operand row of a stage in FP16
constexpr int kBStage = (kBM + kBN) * kBRow;  // 64 KB

__host__ __device__ constexpr size_t big_lds_bytes(int num_experts) {
  return worklist_bytes(num_experts) + 2 * (size_t)kBStage;
}

// Row r of a stage is 8 chunks of 16 bytes (8 FP16 values); chunk q is stored at
// position q ^ swz(r).  The lanes of one LDS access touch 8 or 16 consecutive
// rows with one chunk index; swz is a bijection on every 8 aligned rows, and
// with the row's parity (which half of a 256-byte bank line it lands in) on
// every 16, so those lanes hit distinct banks either way.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ void put_chunk(uint8_t* stage, int row, int q, const half8_t& v) {
  *reinterpret_cast<half8_t*>(stage + row * kBRow + 16 * (q ^ swz(row))) = v;
}

// Operand of v_mfma_f32_32x32x16_f16 for a 32-row block and K slice sl (16
// elements): lane l reads row `row0 + l % 32`, K values 16*sl + 8*(l / 32) .. +7.
__device__ __forceinline__ half8_t frag32(const uint8_t* stage, int row0, int lane, int sl) {
  const int row = row0 + (lane & 31);
  const int q = 2 * sl + (lane >> 5);
  return *reinterpret_cast<const half8_t*>(stage + row * kBRow + 16 * (q ^ swz(row)));
}

typedef float float16_t __attribute__((ext_vector_type(16)));

// One operand row's raw stage: 64 codes in two 16-byte pieces and 4 scale bytes.
struct RowStage {
  u32x4_t q0, q1;
  uint32_t s;
};

// Dequantise chunk w (8 values) of a row's stage into LDS row `row`.
__device__ __forceinline__ void dequant_chunk(uint8_t* stage, int row, const RowStage& r, int w) {
  const half2_t sp = (w < 4) ? scale_pair_x2m8<false>(r.s) : scale_pair_x2m8<true>(r.s);
  const _Float16 sc = sp[(w >> 1) & 1];
  put_chunk(stage, row, w, dequant8(w < 4 ? r.q0[w & 3] : r.q1[w & 3], sc));
}

// Items of one expert in banded order: its M-tiles are taken in bands of
// kBand, and a band's items run N-tile by N-tile, M-tile fastest.  Workgroups
// with consecutive logical numbers share an XCD and its L2 (logical_block), so
// the 32 items an XCD runs side by side form a kBand x 8 block of the output:
// 4 activation strips and 8 weight strips read through one L2, where an N-tile
// per XCD (the plain N-major order) reads 32 activation strips and 1 weight
// strip.  On the dense 8192^3 case that cuts the strips fetched per round from
// 33 to 12 per XCD.  A bijection on the expert's items; experts of kBand
// M-tiles or fewer keep the plain order.
constexpr int kBand = 4;

__device__ __forceinline__ ItemPos locate_banded(int32_t i, int32_t from, const WorkList& wl,
                                                 const GemmArgs& p, int lane) {
  const int32_t e = find_expert(i, from, wl, p.num_experts, lane);
  const int32_t r_lo = uniform(wl.off[e]);
  const int32_t cnt = uniform(wl.off[e + 1]) - r_lo;
  const int32_t mts = (cnt + kBM - 1) / kBM;
  const int32_t local = i - uniform(wl.prefix[e]);
  const int32_t band_items = kBand * p.n_tiles;
  const int32_t band = local / band_items, within = local - band * band_items;
  const int32_t left = mts - band * kBand;
  const int32_t tall = left < kBand ? left : kBand;  // M-tiles in this band
  const int32_t nt = within / tall, mt = band * kBand + (within - nt * tall);
  ItemPos it;
  it.e = e;
  it.row0 = r_lo + mt * kBM;
  const int32_t rows_left = cnt - mt * kBM;
  it.rows_valid = rows_left < kBM ? rows_left : kBM;
  it.n0 = nt * kBN;
  it.alpha = ((sconst_f32)p.a_scale)[0] * ((sconst_f32)p.w_scale)[e];
  return it;
}

// One operand row of an item for one loader thread: its buffer resources and
// byte offsets, and where stage st's codes start.
struct OperandRow {
  rsrc_t rq, rs;
  uint32_t vq, vs;
  uint32_t half;    // bytes between the row's two 16-byte code pieces of a stage
  int32_t wrg;      // packed weights: 16-row blocks in this wave's 64-row group
  int32_t pk_block, pk_lg;
  bool wpk;         // packed weight row

  // Byte offset of stage st's codes: row-major, 32 bytes per stage; packed
  // (weight waves), two 16-byte pieces 1 KB apart in block j of granule t, at
  // the position of sub-step s and lane group g of the packed order.
  __device__ __forceinline__ int32_t q_off(int32_t st) const {
    if (!wpk) return st * (kBK / 2);
    const int32_t t = st >> pk_lg, m = st & ((1 << pk_lg) - 1);
    const int32_t gg = m >> (pk_lg - 2), sub = m & ((1 << (pk_lg - 2)) - 1);
    return t * wrg * pk_block + sub * 2048 + gg * 256;
  }
};

// This thread's operand row of item `it`: activation row `lrow` of the item,
// gathered through the row index (rows past the expert's end repeat its first
// row: computed, never stored), or weight row `lrow` (past n: out of range,
// reads zeros).  Waves 4-7 load weight rows.
__device__ __forceinline__ OperandRow operand_row(const GemmArgs& p, const ItemPos& it, bool is_w,
                                                  int wave, int lrow) {
  const int32_t n = (int32_t)p.n, kb = (int32_t)(p.k >> 1), nbk = (int32_t)(p.k >> 4);
  OperandRow o;
  // Packed weight layout: bytes of a 16-row block, and log2 of the stages per
  // granule (a granule of 256 or 512 elements holds 4 or 8 stages of 64).
  o.pk_block = packed_block_bytes(packed_granule(p.k));
  o.pk_lg = packed_granule(p.k) == 512 ? 3 : 2;
  o.half = 16;
  o.wrg = 0;
  o.wpk = is_w && p.w_packed;
  if (is_w) {
    o.rq = make_rsrc(p.w_q + (int64_t)it.e * n * kb, (uint32_t)(n * kb));
    o.rs = make_rsrc(p.w_sf + (int64_t)it.e * n * nbk, (uint32_t)(n * nbk));
    const int32_t row = it.n0 + lrow;
    if (p.w_packed) {
      // This wave's 64 rows are one group of the packed layout; a thread's
      // row is piece r of each 16-row block j of the group.  (A group wholly
      // past n has no blocks: its rows read out of range.)
      const int32_t grp0 = uniform(it.n0 + 64 * (wave - 4));
      const int32_t left = grp0 < n ? (n - grp0) / 16 : 0;
      o.wrg = left < 4 ? left : 4;
      const int32_t jb = (row - grp0) >> 4, r = row & 15;
      o.vq = row < n ? (uint32_t)(grp0 * kb + jb * o.pk_block + 16 * r) : kOutOfRange;
      o.half = 1024;
    } else {
      o.vq = row < n ? (uint32_t)(row * kb) : kOutOfRange;
    }
    o.vs = row < n ? (uint32_t)(row * nbk) : kOutOfRange;
  } else {
    const int32_t a_last = (int32_t)p.a_rows - 1;
    const int32_t r = it.row0 + (lrow < it.rows_valid ? lrow : 0);
    int32_t src = p.a_row_index ? p.a_row_index[r] : r;
    src = src < 0 ? 0 : (src > a_last ? a_last : src);
    o.rq = make_rsrc(p.a_q, (uint32_t)(p.a_rows * kb));
    o.rs = make_rsrc(p.a_sf, (uint32_t)(p.a_rows * nbk));
    o.vq = (uint32_t)(src * kb);
    o.vs = (uint32_t)(src * nbk);
  }
  return o;
}

// Issue the loads of stage st of an operand row (out of range, so no traffic,
// when !in).
__device__ __forceinline__ void load_row_stage(RowStage& r, const OperandRow& o, int32_t st, bool in) {
  const int32_t kq = uniform(o.q_off(st)), ks = uniform(st * (kBK / 16));
  const uint32_t oq = in ? o.vq : kOutOfRange, os = in ? o.vs : kOutOfRange;
  r.q0 = __builtin_amdgcn_raw_buffer_load_b128(o.rq, oq, kq, 0);
  r.q1 = __builtin_amdgcn_raw_buffer_load_b128(o.rq, oq + o.half, kq, 0);
  r.s = __builtin_amdgcn_raw_buffer_load_b32(o.rs, os, ks, 0);
}

// The epilogue of a 256 x 256 item, staged through LDS (`tile`: 128 KB, free
// after the item's last barrier).  Lane l holds activation row 128*wm + 32*ab +
// l % 32 and, per accumulator quad q, the 4 output columns 64*wn + 32*wb + 8q
// + 4*(l / 32) .. +3: written to LDS row by row (512 bytes, 16-byte chunk c at
// position c ^ (row % 32)), then read back so that each wave stores two whole
// 512-byte row segments per instruction.  Rows past the expert's end fall
// outside the store resource; 8-column chunks past n get an out-of-range
// offset.  Ends with a barrier (the next item's first stage rewrites `tile`).
__device__ __forceinline__ void store_tile(float16_t (&acc)[2][4], const ItemPos& it,
                                           const GemmArgs& p, uint8_t* tile, int tid, int lane,
                                           int wm, int wn) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  constexpr int kTileRow = 2 * kBN;  // bytes
  const int32_t n = (int32_t)p.n;
  const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int wb = 0; wb < 2; ++wb) {
#pragma unroll
    for (int ab = 0; ab < 4; ++ab) {
      const int row = 128 * wm + 32 * ab + r32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float16_t& v = acc[wb][ab];
        const bf16x4_t bv = {(__bf16)(v[4 * q] * it.alpha), (__bf16)(v[4 * q + 1] * it.alpha),
                             (__bf16)(v[4 * q + 2] * it.alpha), (__bf16)(v[4 * q + 3] * it.alpha)};
        const int chunk = 8 * wn + 4 * wb + q;
        *reinterpret_cast<u32x2_t*>(tile + row * kTileRow + 16 * (chunk ^ (row & 31)) + 8 * h) =
            __builtin_bit_cast(u32x2_t, bv);
      }
    }
  }
  __syncthreads();
  // The host picks this tile only when 256 rows of ldo BF16 values stay below
  // 2^31 - 4096 bytes, so the resource size and every offset fit 31 bits.
  const uint32_t ldo = (uint32_t)p.ldo;
  const rsrc_t o = make_rsrc(p.out + (int64_t)it.row0 * ldo, (uint32_t)it.rows_valid * ldo * 2u);
  const int chunk = tid & 31, r0 = tid >> 5;  // 16 rows per pass of the workgroup
  const bool col_ok = it.n0 + 8 * chunk < n;
#pragma unroll
  for (int i = 0; i < kBM / 16; ++i) {
    const int row = r0 + 16 * i;
    const u32x4_t d = *reinterpret_cast<const u32x4_t*>(tile + row * kTileRow + 16 * (chunk ^ (row & 31)));
    const uint32_t off =
        col_ok ? ((uint32_t)row * ldo + (uint32_t)(it.n0 + 8 * chunk)) * 2u : kOutOfRange;
    __builtin_amdgcn_raw_buffer_store_b128(d, o, off, 0, 0);
  }
  // The next item's first stage rewrites these buffers.
  __syncthreads();
}

template <int PD>
__global__ __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_grouped_gemm_big(const GemmArgs p) {
  static_assert(PD % 2 == 0, "stage ring must be even (LDS buffers alternate)");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int32_t* prefix = reinterpret_cast<int32_t*>(smem);
  int32_t* offl = prefix + (p.num_experts + 1);
  __shared__ int32_t wave_sum[kBThreads / 64];
  uint8_t* const stages = smem + worklist_bytes(p.num_experts);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // this wave's piece: rows 128*wm.., columns 64*wn..
  // Loader role (uniform per wave): waves 0-3 load activation rows, 4-7 weight rows.
  const bool is_w = wave >= 4;
  const int lrow = tid & 255;
  const int srow = (is_w ? kBM : 0) + lrow;  // the row this thread writes in a stage

  const int32_t total_items = build_worklist<kBThreads>(p, kBM, prefix, offl, wave_sum);
  const WorkList wl{prefix, offl};

  const int nblk = gridDim.x, b = blockIdx.x;
  const int32_t rounds = (total_items + nblk - 1) / nblk;
  if (rounds == 0) return;
  const int32_t last_items = total_items - (rounds - 1) * nblk;
  const int32_t lb_full = logical_block(b, nblk, nblk);
  const int32_t lb_last = logical_block(b, nblk, last_items);
  const int32_t my_items = (rounds - 1) + (lb_last < last_items ? 1 : 0);

  const int32_t nst = (int32_t)(p.k / kBK);

  int32_t from = 0;
  for (int32_t j = 0; j < my_items; ++j) {
    const int32_t item = j * nblk + (j == rounds - 1 ? lb_last : lb_full);
    const ItemPos it = locate_banded(item, from, wl, p, lane);
    from = it.e;

    const OperandRow orow = operand_row(p, it, is_w, wave, lrow);

    // 2 x 4 accumulator tiles of 32 x 32: acc[wb][ab] holds weight rows (output
    // columns) 32*wb .. +31 and activation rows 32*ab .. +31 of this wave's piece.
    float16_t acc[2][4];
#pragma unroll
    for (int wb = 0; wb < 2; ++wb)
#pragma unroll
      for (int ab = 0; ab < 4; ++ab)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[wb][ab][i] = 0.0f;

    // The ring: slot d holds the raw stage loaded PD stages before it is
    // dequantised.  Stages past the last one load out of range (no traffic).
    RowStage ring[PD];
    auto load_stage = [&](int slot, int32_t st) {
      const bool in = st < nst;
      load_row_stage(ring[slot], orow, st, in);
    };

    // MFMA operands of one 16-element K slice: fw[2] weight and fa[4] activation
    // blocks of 32 rows of this wave's piece; two slices in flight.
    half8_t fw[2][2], fa[2][4];
    // Operand read i (0..5) of slice sl, in the order the slice's MFMAs first
    // need them: fw[0], fa[0..3], fw[1].
    auto read_one = [&](const uint8_t* stage, int sl, int i) {
      const int sk = sl & 3, f = sl & 1;
      if (i == 0) fw[f][0] = frag32(stage, kBM + 64 * wn, lane, sk);
      else if (i < 5) fa[f][i - 1] = frag32(stage, 128 * wm + 32 * (i - 1), lane, sk);
      else fw[f][1] = frag32(stage, kBM + 64 * wn + 32, lane, sk);
    };
    // MFMA i (0..7) of slice sl: weight block i / 4, activation block i % 4.
    auto mfma_one = [&](int sl, int i) {
      const int wb = i >> 2, ab = i & 3, f = sl & 1;
      acc[wb][ab] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fw[f][wb], fa[f][ab], acc[wb][ab], 0, 0, 0);
    };

#pragma unroll
    for (int d = 0; d < PD; ++d) {
      load_stage(d, d);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) dequant_chunk(stages, srow, ring[0], w);
    load_stage(0, PD);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 6; ++i) read_one(stages, 0, i);

    // Stage st (data in buffer `cur`, slice 0's operands already in registers),
    // issued in a fixed order, one MFMA per step:
    //   slices 0-2 (steps 0-23): step m issues MFMA m % 8 of slice m / 8; the
    //       first 6 steps of each slice also read one operand of the next slice,
    //       and every third step dequantises one 16-byte chunk of stage st+1
    //       (from the ring) into `nxt`; then the ring slot is reloaded with stage
    //       st+1+PD;
    //   barrier: stage st+1 is in `nxt`, and every read of `cur` is done;
    //   slice 3 (steps 24-31): the same, reading stage st+1's slice 0 from `nxt`.
    // `cur` is rewritten (with stage st+2) only in the next stage, after this
    // barrier, so one barrier per stage orders every LDS access.  The last stage
    // dequantises the ring's out-of-range loads (zeros) into `nxt`, unused.
    for (int32_t st0 = 0; st0 < nst; st0 += PD) {
#pragma unroll
      for (int d = 0; d < PD; ++d) {
        const int32_t st = st0 + d;
        const uint8_t* cur = stages + (d & 1) * kBStage;  // PD is even: d & 1 == st & 1
        uint8_t* nxt = stages + ((d + 1) & 1) * kBStage;
        const int kSlot = (d + 1) % PD;  // holds stage st + 1
#pragma unroll
        for (int m = 0; m < 24; ++m) {
          const int sl = m >> 3, i = m & 7;
          mfma_one(sl, i);
          if (i < 6) read_one(cur, sl + 1, i);
          if (m % 3 == 0) dequant_chunk(nxt, srow, ring[kSlot], m / 3);
          __builtin_amdgcn_sched_barrier(0);
        }
        load_stage(kSlot, st + 1 + PD);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          mfma_one(3, i);
          if (i < 6) read_one(nxt, 4, i);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // The next item's first stage rewrites buffer 0, which the last slice 3
    // read from.
    __syncthreads();

    store_tile(acc, it, p, stages, tid, lane, wm, wn);
  }
}


// ---- Split K by scale block on the FP8 MFMA (MOE_FP4_TILE "256x256f8") ----
//
// The alternative to dequantising into FP16 that CDNA4's matrix cores allow
// without losing exactness.  Their native block-scaled FP4 product takes one
// power-of-two scale per 32 elements, where NVFP4 has an E4M3 scale per 16
// ("Peering into the CUTLASS SharedStorage", section "Input Knowledge", item 3),
// so here each 16-element block is its own product: the E2M1 codes are
// re-encoded as E4M3 bytes (every E2M1 value is an E4M3 value, so this is
// exact), one v_mfma_f32_32x32x16_fp8_fp8 per block and 32 x 32 tile gives the
// block's unscaled sums P_b (exact in FP32: multiples of 1/4 below 2^10), and
// the VALU applies the scales, acc = fma(sa * sw, P_b, acc): sa * sw (two E4M3
// values) and its product with P_b are exact, so every block adds one exactly
// known term with one rounding, as the FP16 path's MFMA accumulation does.
//
// Stage layout in LDS (two stages of 40 KB; the 128 KB epilogue tile reuses
// them): 512 operand rows of 64 E4M3 bytes (8-byte chunk c of row r at position
// c ^ ((r >> 2) & 7), so the 32 rows one ds_read_b64 touches hit distinct banks),
// then the rows' block scales as FP32, [4 blocks][512 rows].  Per 16-element
// slice a wave reads 2 weight and 4 activation operands (8 bytes per lane), its
// 32 weight-row scales (8 reads of 16 bytes, two addresses per instruction) and
// 4 activation-row scales, issues 8 MFMAs and 256 FMAs (plus 256 multiplies for
// the scale products): the VALU work per MFMA is what bounds this variant.
constexpr int kF8Row = kBK;                          // bytes per operand row per stage
constexpr int kF8Codes = (kBM + kBN) * kF8Row;       // 32 KB
constexpr int kF8Stage = kF8Codes + (kBM + kBN) * (kBK / 16) * 4;  // + 8 KB of scales
static_assert(2 * kF8Stage <= 2 * kBStage, "FP8 stages fit in the FP16 stages' LDS");

typedef long fp8x8_t;  // eight E4M3 bytes, the operand of one lane

__device__ __forceinline__ int swz8(int row) { return (row >> 2) & 7; }

// Eight packed E2M1 codes (element 0 in the low nibble) as eight E4M3 bytes
// (element 0 in the low byte).  The magnitude bits index a table of the eight
// E4M3 encodings of 0, 0.5, 1, 1.5, 2, 3, 4, 6 (v_perm_b32 selects bytes of a
// 64-bit operand); the sign moves from bit 3 to bit 7.
__device__ __forceinline__ u32x2_t e2m1x8_to_e4m3(uint32_t c) {
  constexpr uint32_t kTabHi = 0x4C484440u, kTabLo = 0x3C383000u;  // codes 4-7, 0-3
  const uint32_t lo = c & 0x0F0F0F0Fu, hi = (c >> 4) & 0x0F0F0F0Fu;  // even, odd elements
  const uint32_t elo = __builtin_amdgcn_perm(kTabHi, kTabLo, lo & 0x07070707u) | ((lo & 0x08080808u) << 4);
  const uint32_t ehi = __builtin_amdgcn_perm(kTabHi, kTabLo, hi & 0x07070707u) | ((hi & 0x08080808u) << 4);
  // Interleave: bytes (even0, odd0, even1, odd1) and (even2, odd2, even3, odd3).
  return u32x2_t{__builtin_amdgcn_perm(ehi, elo, 0x05010400u), __builtin_amdgcn_perm(ehi, elo, 0x07030602u)};
}

// Write one operand row's stage into LDS: its 64 codes as E4M3 bytes and its 4
// block scales as FP32.
__device__ __forceinline__ void put_row_f8(uint8_t* stage, int row, const RowStage& r) {
  uint8_t* base = stage + row * kF8Row;
  const int sw = swz8(row);
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const uint32_t c = d < 4 ? r.q0[d] : r.q1[d - 4];
    *reinterpret_cast<u32x2_t*>(base + 8 * (d ^ sw)) = e2m1x8_to_e4m3(c);
  }
  float* sc = reinterpret_cast<float*>(stage + kF8Codes);
  sc[0 * (kBM + kBN) + row] = __builtin_amdgcn_cvt_f32_fp8(r.s, 0);
  sc[1 * (kBM + kBN) + row] = __builtin_amdgcn_cvt_f32_fp8(r.s, 1);
  sc[2 * (kBM + kBN) + row] = __builtin_amdgcn_cvt_f32_fp8(r.s, 2);
  sc[3 * (kBM + kBN) + row] = __builtin_amdgcn_cvt_f32_fp8(r.s, 3);
}

// Operand of v_mfma_f32_32x32x16_fp8_fp8 for the 32-row block at row0, slice
// (block) sl: lane l reads row row0 + l % 32, elements 16 sl + 8 (l / 32) .. +7.
__device__ __forceinline__ fp8x8_t frag_f8(const uint8_t* stage, int row0, int lane, int sl) {
  const int row = row0 + (lane & 31);
  const int c = 2 * sl + (lane >> 5);
  return *reinterpret_cast<const fp8x8_t*>(stage + row * kF8Row + 8 * (c ^ swz8(row)));
}

template <int PD>
__global__ __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_grouped_gemm_big_f8(const GemmArgs p) {
  static_assert(PD % 2 == 0, "stage ring must be even (LDS buffers alternate)");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int32_t* prefix = reinterpret_cast<int32_t*>(smem);
  int32_t* offl = prefix + (p.num_experts + 1);
  __shared__ int32_t wave_sum[kBThreads / 64];
  uint8_t* const stages = smem + worklist_bytes(p.num_experts);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // this wave's piece: rows 128*wm.., columns 64*wn..
  const bool is_w = wave >= 4;               // loader role, as in the FP16 kernel
  const int lrow = tid & 255;
  const int srow = (is_w ? kBM : 0) + lrow;
  const int h = lane >> 5;

  const int32_t total_items = build_worklist<kBThreads>(p, kBM, prefix, offl, wave_sum);
  const WorkList wl{prefix, offl};
  const int nblk = gridDim.x, b = blockIdx.x;
  const int32_t rounds = (total_items + nblk - 1) / nblk;
  if (rounds == 0) return;
  const int32_t last_items = total_items - (rounds - 1) * nblk;
  const int32_t lb_full = logical_block(b, nblk, nblk);
  const int32_t lb_last = logical_block(b, nblk, last_items);
  const int32_t my_items = (rounds - 1) + (lb_last < last_items ? 1 : 0);
  const int32_t nst = (int32_t)(p.k / kBK);

  int32_t from = 0;
  for (int32_t j = 0; j < my_items; ++j) {
    const int32_t item = j * nblk + (j == rounds - 1 ? lb_last : lb_full);
    const ItemPos it = locate_banded(item, from, wl, p, lane);
    from = it.e;
    const OperandRow orow = operand_row(p, it, is_w, wave, lrow);

    // Scalar accumulators (the VALU updates them element by element; a
    // 16-wide vector updated that way is rebuilt for every element).
    float acc[2][4][16];
#pragma unroll
    for (int wb = 0; wb < 2; ++wb)
#pragma unroll
      for (int ab = 0; ab < 4; ++ab)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[wb][ab][i] = 0.0f;

    RowStage ring[PD];
#pragma unroll
    for (int d = 0; d < PD; ++d) load_row_stage(ring[d], orow, d, d < nst);
    put_row_f8(stages, srow, ring[0]);
    load_row_stage(ring[0], orow, PD, PD < nst);
    __syncthreads();

    for (int32_t st0 = 0; st0 < nst; st0 += PD) {
#pragma unroll
      for (int d = 0; d < PD; ++d) {
        const int32_t st = st0 + d;
        const uint8_t* cur = stages + (d & 1) * kF8Stage;  // PD is even: d & 1 == st & 1
        uint8_t* nxt = stages + ((d + 1) & 1) * kF8Stage;
        const int kSlot = (d + 1) % PD;                      // holds stage st + 1
        const float* sc = reinterpret_cast<const float*>(cur + kF8Codes);
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          // Tile t = (wb, ab) = (t / 4, t % 4) of slice sl.  Only the block
          // products of tiles t and t + 1 are live: step t issues MFMA t + 1
          // (its operands read from LDS in the same step) and then scales and
          // adds tile t on the VALU.  The compiler barrier at the end of each
          // step keeps the next step's LDS reads, and with them its MFMA,
          // from being hoisted above this step's VALU work, which would make
          // all eight products live at once; the barrier also uses the tile's
          // sums, so the VALU work cannot sink below it either.
          const float* scl = sc + sl * (kBM + kBN);
          float sa[4];
#pragma unroll
          for (int ab = 0; ab < 4; ++ab) sa[ab] = scl[128 * wm + 32 * ab + (lane & 31)];
          fp8x8_t fw = frag_f8(cur, kBM + 64 * wn, lane, sl);
          float4_t sw[4];
          float16_t pb[2];
          const float16_t zero = {};
          pb[0] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(fw, frag_f8(cur, 128 * wm, lane, sl), zero,
                                                             0, 0, 0);
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int wb = t >> 2, ab = t & 3;
            if (ab == 0) {
              // This lane's 16 weight rows of block wb: 8q + 4h .. +3, q < 4.
              const int r0 = kBM + 64 * wn + 32 * wb;
#pragma unroll
              for (int q = 0; q < 4; ++q)
                sw[q] = *reinterpret_cast<const float4_t*>(scl + r0 + 8 * q + 4 * h);
            }
            if (t + 1 < 8) {
              const int wb1 = (t + 1) >> 2, ab1 = (t + 1) & 3;
              if (ab1 == 0) fw = frag_f8(cur, kBM + 64 * wn + 32 * wb1, lane, sl);
              pb[(t + 1) & 1] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(
                  fw, frag_f8(cur, 128 * wm + 32 * ab1, lane, sl), zero, 0, 0, 0);
            }
            // The next stage's conversion, spread over the steps of slice 1.
            if (sl == 1 && t == 3) put_row_f8(nxt, srow, ring[kSlot]);
            const float16_t& P = pb[t & 1];
#pragma unroll
            for (int v = 0; v < 16; ++v)
              acc[wb][ab][v] = __builtin_fmaf(sa[ab], sw[v >> 2][v & 3] * P[v], acc[wb][ab][v]);
            const float* a = acc[wb][ab];
            asm volatile("" ::"v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]),
                         "v"(a[6]), "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]),
                         "v"(a[12]), "v"(a[13]), "v"(a[14]), "v"(a[15])
                         : "memory");
          }
        }
        load_row_stage(ring[kSlot], orow, st + 1 + PD, st + 1 + PD < nst);
        // Stage st+1 is in `nxt` and every read of `cur` is done; `cur` is
        // rewritten (stage st+2) only after this barrier.
        __syncthreads();
      }
    }
    float16_t out[2][4];
#pragma unroll
    for (int wb = 0; wb < 2; ++wb)
#pragma unroll
      for (int ab = 0; ab < 4; ++ab)
#pragma unroll
        for (int i = 0; i < 16; ++i) out[wb][ab][i] = acc[wb][ab][i];
    store_tile(out, it, p, stages, tid, lane, wm, wn);
  }
}

}  // namespace

size_t big_lds(int32_t num_experts) { return big_lds_bytes(num_experts); }

hipError_t launch_grouped_gemm_big(const GemmArgs& p, bool f8, hipStream_t stream) {
  // K is a multiple of 256, so the stage count (K / 64) is a multiple of the ring.
  constexpr int PD = 2;
  auto kern = f8 ? k_grouped_gemm_big_f8<PD> : k_grouped_gemm_big<PD>;
  const size_t lds = big_lds_bytes(p.num_experts);
  if (lds > kLdsBytes) return hipErrorInvalidValue;  // the host picks this tile only if it fits
  int resident = 0;
  hipError_t err = resident_groups(kern, kBThreads, lds, &resident);
  if (err != hipSuccess) return err;
  // Upper bound on the number of items: the host does not see the offsets.
  const int64_t max_mtiles = p.m_total / kBM + (p.m_total < p.num_experts ? p.m_total : p.num_experts);
  const int64_t max_items = max_mtiles * p.n_tiles;
  int64_t grid = resident;
  if (max_items < grid) grid = max_items;
  if (grid < 1) grid = 1;
  grid = (grid + kXcds - 1) / kXcds * kXcds;  // whole rounds over the XCDs
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace moe_fp4
