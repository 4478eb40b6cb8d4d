// The per-wavefront NVFP4 grouped-GEMM kernel template and its launcher, shared by
// the translation units that instantiate it (grouped_gemm.hip: plain BF16 store;
// grouped_gemm_finalize.hip: the routing-weighted token-order epilogue;
// grouped_gemm_swiglu.hip: the SwiGLU + NVFP4 epilogue of the gate+up projection).
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
//  * Persistent wavefronts.  Every wavefront walks its own items in rounds of
//    one item per wavefront, with no inter-wave synchronisation after the
//    prefix; the workgroups active in a round are spread evenly over the XCDs.
//  * Loads.  A pipeline stage covers 256*KSUB K elements.  Lane (c = lane %
//    16, g = lane / 16) loads row c of each 16-row block, K run g of the stage,
//    with 16-byte buffer loads that land in registers already in MFMA operand
//    order.  Every load is unconditional (rows past n read zeros, a masked
//    store is an out-of-range buffer offset), so the compiler's count of
//    outstanding loads is exact and one stage stays in flight while the
//    previous one is computed.
//  * Weight block scales (SL).  For K a multiple of 2048, each wave copies the
//    128-byte scale line of every weight row (one line = 2048 K elements) into
//    its own LDS buffer with full-line buffer-to-LDS loads, double-buffered by
//    span, and reads each stage's scales from there.  Loading the line in the
//    per-stage pieces the MFMA needs would fetch every line in several pieces
//    far apart in time, which costs several DRAM fetches per line.
//  * Math.  Codes are dequantised exactly to FP16 (fp4_device.h) and fed to
//    v_mfma_f32_16x16x32_f16 with FP32 accumulation: weights are the A operand
//    (16 output columns), activations the B operand (16 rows).  The 16-element
//    E4M3 block scales are applied during dequantisation, exactly, so CDNA4's
//    scaled FP4 MFMA (32-element E8M0 scales) is not used.
//  * Epilogue.  acc * a_scale * w_scale[e] -> BF16 (round to nearest even),
//    each lane storing 4 consecutive columns (8 bytes) of one row; rows past the
//    expert's end and column blocks past n are not written.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_device.h"
#include "gemm_common.h"
#include "launch.h"

namespace moe_fp4 {
namespace {

// K elements whose block scales fill one 128-byte line of a row.
constexpr int kSpan = 2048;

// What a finished item's epilogue does with its FP32 tile.
enum Epilogue : int {
  kEpiStore = 0,     // BF16 store of the routed rows (the plain GEMM)
  kEpiFinalize = 1,  // routing-weighted FP32 adds into token rows
  kEpiSwiglu = 2,    // SwiGLU of gate and up columns, NVFP4-quantised
};

// Weight rows of row block jb of an item at column n0.  With the SwiGLU
// epilogue an item covers 32 columns of the intermediate: blocks 0 and 1 are
// gate rows n0 .. n0+31, blocks 2 and 3 the matching up rows n/2 + n0 ..
// (the first half of the weight rows is the gate, the second the up
// projection); otherwise block jb is rows n0 + 16*jb ...
template <bool SW>
__device__ __forceinline__ int32_t block_row0(int32_t n0, int32_t n, int jb) {
  if constexpr (SW) return (jb < 2 ? 0 : (n >> 1)) + n0 + 16 * (jb & 1);
  else return n0 + 16 * jb;
}
// Whether row block jb holds weight rows (n % 16 == 0, so a block is all in or all out).
template <bool SW>
__device__ __forceinline__ bool block_in(int32_t n0, int32_t n, int jb) {
  if constexpr (SW) return n0 + 16 * (jb & 1) < (n >> 1);
  else return n0 + 16 * jb < n;
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// LDS bytes per wave for staged weight scales: two span buffers of 16*NBW
// rows x 128 bytes, and a 1 KB sink for the copies issued by stages that start
// no span (see issue_loads).
template <int NBW>
constexpr int scale_lds_per_wave() {
  return 2 * 16 * NBW * 128 + 1024;
}

// Register image of one pipeline stage (KSUB sub-steps of 256 K elements) for
// one wavefront.  Within a stage, lane group g (lanes 16g .. 16g+15, one row
// each) owns the contiguous K run [64*KSUB*g, 64*KSUB*(g+1)) of the stage: per
// 16-row block and sub-step s, 32 code bytes (elements 64s .. 64s+63 of its
// run) and one scale dword; the KSUB scale dwords of a lane are adjacent in
// memory and arrive in one load.  Weights and activations use the same K
// order, so every product pairs the same K element.  With SL the weight scales
// come from LDS instead (ws is then filled by compute_stage).
template <int MB, int NBW, int KSUB>
struct Stage {
  u32x4_t w[NBW][KSUB][2];
  uint32_t ws[NBW][KSUB];
  u32x4_t a[MB][KSUB][2];
  uint32_t as[MB][KSUB];
};

// The loads of a work item: this expert's weight resources and each lane's
// byte offsets into them and into the activations.
template <int MB, int NBW>
struct ItemLoads {
  rsrc_t w, ws;
  uint32_t w_voff[NBW], ws_voff[NBW];  // lane's weight row, or out of range past n
  uint32_t a_voff[MB], as_voff[MB];    // lane's (gathered, clamped) activation row
  uint32_t sl_voff;                    // lane's 16-byte piece of a scale-line copy
  int32_t n0;
};

// An empty use of the lane offsets: keeps their registers allocated until the
// loads that read them have completed (it is placed after the wait for those
// loads), so decoding the next item never overwrites an address operand of a
// load still in flight and needs no wait of its own.
template <int MB, int NBW>
__device__ __forceinline__ void hold(const ItemLoads<MB, NBW>& l) {
#pragma unroll
  for (int jb = 0; jb < NBW; ++jb) asm volatile("" ::"v"(l.w_voff[jb]), "v"(l.ws_voff[jb]));
#pragma unroll
  for (int ib = 0; ib < MB; ++ib) asm volatile("" ::"v"(l.a_voff[ib]), "v"(l.as_voff[ib]));
  asm volatile("" ::"v"(l.sl_voff));
}

// The same loads with every offset out of range: they return zeros without a
// memory request (used for the one surplus issue at the end of a wave's work).
template <int MB, int NBW>
__device__ __forceinline__ ItemLoads<MB, NBW> nowhere(const ItemLoads<MB, NBW>& l) {
  ItemLoads<MB, NBW> z = l;
#pragma unroll
  for (int jb = 0; jb < NBW; ++jb) z.w_voff[jb] = z.ws_voff[jb] = kOutOfRange;
#pragma unroll
  for (int ib = 0; ib < MB; ++ib) z.a_voff[ib] = z.as_voff[ib] = kOutOfRange;
  z.sl_voff = kOutOfRange;
  z.n0 = 0x40000000;  // no scale-line copy either
  return z;
}

// Lane (c, g)'s entry of the row index for row block ib of an item: a vector
// load issued an item ahead of its use (so its latency is hidden behind a
// unit of work, where scalar loads would stall the wave when it is needed).
// Rows past the expert's end repeat its first row: their products are
// computed and never stored.  Without a row index the resource is empty, the
// load returns nothing and the caller takes the row itself.
__device__ __forceinline__ uint32_t row_index_load(const rsrc_t& idx_rs, const ItemPos& it, int ib,
                                                   int c) {
  const int32_t rr = 16 * ib + c;
  const int32_t r = it.row0 + (rr < it.rows_valid ? rr : 0);
  return __builtin_amdgcn_raw_buffer_load_b32(idx_rs, (uint32_t)(4 * r), 0, 0);
}

// The per-lane loads of a located item: this expert's weight resources and
// each lane's byte offsets.  `rows[ib]` is the lane's row-index entry for row
// block ib (row_index_load).
// Row x pitch for lane offsets.  The host bounds rows * (k/2) below 2^31 with
// k/2 >= 128, so both factors are below 2^24 and the 24-bit multiply is exact;
// it also keeps the compiler from a 64-bit multiply-add whose unused high half
// would wait on loads still in flight in that register.
__device__ __forceinline__ uint32_t mul24(int32_t a, int32_t b) {
  return __umul24((uint32_t)a, (uint32_t)b);
}

// Weight half of item_loads: the expert's weight resources and the lane's
// weight and scale-line offsets (no dependence on the row index).
template <int MB, int NBW, int KSUB, bool PK, bool SW>
__device__ __forceinline__ void item_loads_w(const ItemPos& it, const GemmArgs& p, int lane,
                                             ItemLoads<MB, NBW>& ld) {
  const int c = lane & 15, g = lane >> 4;
  // 32-bit offsets: the host guarantees n * k/2 and a_rows * k/2 < 2^31.
  const int32_t n = (int32_t)p.n, kb = (int32_t)(p.k >> 1), nbk = (int32_t)(p.k >> 4);
  ld.w = make_rsrc(p.w_q + (int64_t)it.e * n * kb, (uint32_t)(n * kb));
  ld.ws = make_rsrc(p.w_sf + (int64_t)it.e * n * nbk, (uint32_t)(n * nbk));
  ld.n0 = it.n0;
  // Packed codes (PK, 64-column items): a row block of 16 rows starting at
  // rb sits in the 64-row group rb / 64, at block (rb % 64) / 16 of each
  // granule, in this kernel's lane order.  (For the plain mapping the item is
  // one whole group; for SwiGLU every group is whole, n/2 % 64 == 0.)
  constexpr int32_t kBlock = 16 * 128 * KSUB;
#pragma unroll
  for (int jb = 0; jb < NBW; ++jb) {
    if constexpr (SW) {
      const int32_t rb = block_row0<SW>(it.n0, n, jb);
      const int32_t row = rb + c;
      const bool ok = block_in<SW>(it.n0, n, jb);
      const uint32_t wv = PK ? (uint32_t)((rb & ~63) * kb + ((rb & 63) >> 4) * kBlock + 16 * lane)
                             : mul24(row, kb) + 32 * KSUB * g;
      ld.w_voff[jb] = ok ? wv : kOutOfRange;
      ld.ws_voff[jb] = ok ? mul24(row, nbk) + 4 * KSUB * g : kOutOfRange;
    } else {
      const int32_t row = it.n0 + 16 * jb + c;
      const bool ok = row < n;
      const uint32_t wv = PK ? (uint32_t)(it.n0 * kb + jb * kBlock + 16 * lane)
                             : mul24(row, kb) + 32 * KSUB * g;
      ld.w_voff[jb] = ok ? wv : kOutOfRange;
      ld.ws_voff[jb] = ok ? mul24(row, nbk) + 4 * KSUB * g : kOutOfRange;
    }
  }
  // Scale-line copies move 8 rows x 128 bytes per instruction: lane l takes
  // row l/8 and stores the row's 16-byte chunk (l%8) ^ (row%8) in LDS slot l%8,
  // a swizzle that spreads the later per-stage reads over the LDS banks.
  {
    const int r8 = lane >> 3, slot = lane & 7;
    ld.sl_voff = mul24(it.n0 + r8, nbk) + 16 * (slot ^ r8);
  }
}

// Activation half of item_loads: the lane's activation row offsets, from its
// row-index entries `rows`.
template <int MB, int NBW, int KSUB>
__device__ __forceinline__ void item_loads_a(const ItemPos& it, const GemmArgs& p, int lane,
                                             const uint32_t (&rows)[MB], ItemLoads<MB, NBW>& ld) {
  const int c = lane & 15, g = lane >> 4;
  const int32_t kb = (int32_t)(p.k >> 1), nbk = (int32_t)(p.k >> 4);
  const int32_t a_last = (int32_t)p.a_rows - 1;
#pragma unroll
  for (int ib = 0; ib < MB; ++ib) {
    const int32_t rr = 16 * ib + c;
    int32_t mine = p.a_row_index ? (int32_t)rows[ib] : it.row0 + (rr < it.rows_valid ? rr : 0);
    mine = mine < 0 ? 0 : (mine > a_last ? a_last : mine);
    ld.a_voff[ib] = mul24(mine, kb) + 32 * KSUB * g;
    ld.as_voff[ib] = mul24(mine, nbk) + 4 * KSUB * g;
  }
}

template <int MB, int NBW, int KSUB, bool PK, bool SW>
__device__ __forceinline__ void item_loads(const ItemPos& it, const GemmArgs& p, int lane,
                                           const uint32_t (&rows)[MB], ItemLoads<MB, NBW>& ld) {
  item_loads_w<MB, NBW, KSUB, PK, SW>(it, p, lane, ld);
  item_loads_a<MB, NBW, KSUB>(it, p, lane, rows, ld);
}

// The KSUB scale dwords of one lane, in one load.
template <int KSUB>
__device__ __forceinline__ void load_scales(uint32_t (&d)[KSUB], const rsrc_t& rs, uint32_t voff,
                                            int32_t soff) {
  if constexpr (KSUB == 1) {
    d[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0);
  } else if constexpr (KSUB == 2) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0);
    d[0] = v[0];
    d[1] = v[1];
  } else {
    static_assert(KSUB == 4, "stages of 256, 512 or 1024 K elements");
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
    d[0] = v[0];
    d[1] = v[1];
    d[2] = v[2];
    d[3] = v[3];
  }
}

// Where the scale-line copy of a stage goes: the buffer of its span when the
// stage starts a span (sl_span >= 0), else the sink, with no data moved.
struct LineCopy {
  uint8_t* dst;     // LDS: span buffer or sink (wavefront-uniform)
  int32_t span;     // span of the item the copy reads, or -1 for none
};

// Issue every load of stage `kst` of the current item.  Unconditional, so the
// compiler can count outstanding loads exactly; weight rows past n read
// zeros.  The per-lane offsets stay fixed for a whole item and the stage's K
// position goes in the scalar offset, so the loop writes no VGPR that an
// in-flight load still reads.  With SL, the stage first copies the 128-byte
// scale lines of the item's 16*NBW weight rows for its span into LDS, or, if
// it starts no span, issues the same copies out of range into the sink.
// PART 0 issues everything; 1 only the weight side (line copies, codes, scales),
// 2 only the activation side (the kernel's first stage issues 1, then 2, so the
// weight loads need not wait for the row index).
template <int MB, int NBW, int KSUB, bool SL, bool PK, bool SW, int PART = 0>
__device__ __forceinline__ void issue_loads(Stage<MB, NBW, KSUB>& st, const ItemLoads<MB, NBW>& it,
                                            const rsrc_t& a_rs, const rsrc_t& as_rs, int32_t kst,
                                            const LineCopy& lc, int32_t n, int32_t nbk) {
  // Packed codes: a stage is granule kst of the item's 64-row group, rg blocks
  // of 16 rows one after another (rg < 4 only in a last, partial group).
  constexpr int32_t kBlock = 16 * 128 * KSUB;
  const int32_t left = (n - it.n0) >> 4;
  const int32_t wk = PK ? (left < NBW ? left : NBW) * kBlock : 0;
  if constexpr (SL && PART != 2) {
    const bool on = lc.span >= 0;
    const int32_t soff = uniform(on ? lc.span * 128 : 0);
#pragma unroll
    for (int i = 0; i < 2 * NBW; ++i) {
      // Rows 8i .. 8i+7 of the tile (half i%2 of row block i/2): all inside n
      // or all outside (n % 16 == 0).
      const int32_t rows_at = SW ? block_row0<SW>(it.n0, n, i >> 1) + 8 * (i & 1) - it.n0 : 8 * i;
      const bool rows_ok = on && (SW ? block_in<SW>(it.n0, n, i >> 1) : it.n0 + 8 * i < n);
      const uint32_t voff = rows_ok ? it.sl_voff + (uint32_t)(rows_at * nbk) : kOutOfRange;
      uint8_t* dst = on ? lc.dst + 1024 * i : lc.dst;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(it.ws, (lds_ptr)dst, 16, voff, soff, 0, 0);
    }
  }
  const int32_t qk = uniform(kst * 128 * KSUB), sk = uniform(kst * 16 * KSUB);
  const int32_t qw = PK ? uniform(kst * wk) : qk;
  // Byte steps between a lane's pieces: sub-step s and half h.  Row-major:
  // consecutive bytes of the row; packed: 1 KB apart (one load instruction
  // of the wavefront reads 1 KB of consecutive bytes).
  constexpr uint32_t kS = PK ? 2048u : 32u, kH = PK ? 1024u : 16u;
  if constexpr (PART != 2) {
#pragma unroll
    for (int jb = 0; jb < NBW; ++jb) {
#pragma unroll
      for (int s = 0; s < KSUB; ++s) {
        st.w[jb][s][0] =
            __builtin_amdgcn_raw_buffer_load_b128(it.w, it.w_voff[jb] + kS * s, qw, kLoadStreamOnce);
        st.w[jb][s][1] = __builtin_amdgcn_raw_buffer_load_b128(it.w, it.w_voff[jb] + kS * s + kH,
                                                               qw, kLoadStreamOnce);
      }
      if constexpr (!SL) load_scales<KSUB>(st.ws[jb], it.ws, it.ws_voff[jb], sk);
    }
  }
  if constexpr (PART != 1) {
#pragma unroll
    for (int ib = 0; ib < MB; ++ib) {
#pragma unroll
      for (int s = 0; s < KSUB; ++s) {
        st.a[ib][s][0] = __builtin_amdgcn_raw_buffer_load_b128(a_rs, it.a_voff[ib] + 32u * s, qk, 0);
        st.a[ib][s][1] = __builtin_amdgcn_raw_buffer_load_b128(a_rs, it.a_voff[ib] + 32u * s + 16u, qk, 0);
      }
      load_scales<KSUB>(st.as[ib], as_rs, it.as_voff[ib], sk);
    }
  }
}

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const uint8_t*)p);
}

// NBW LDS reads of one width at `addr` + 2048 * jb (row blocks are 16 rows x
// 128 bytes apart), then a wait for all of them, in one asm statement: the
// compiler sees neither an LDS read it would order after the in-flight
// buffer-to-LDS copies nor outputs it could use before the wait.  `dep` is a
// register of the stage's last load, so the compiler waits for that load
// first (and with it, in issue order, for the stage's own line copy).
#define MOE_FP4_LDS_READ2(OP, T)                                                      \
  {                                                                                 \
    T r0, r1;                                                                       \
    asm volatile(OP " %0, %2\n\t" OP " %1, %2 offset:2048\n\ts_waitcnt lgkmcnt(0)"  \
                 : "=&v"(r0), "=&v"(r1)                                             \
                 : "v"(addr), "v"(dep));                                            \
    out[0] = r0;                                                                    \
    out[1] = r1;                                                                    \
  }
#define MOE_FP4_LDS_READ4(OP, T)                                                    \
  {                                                                                 \
    T r0, r1, r2, r3;                                                               \
    asm volatile(OP " %0, %4\n\t" OP " %1, %4 offset:2048\n\t" OP                   \
                    " %2, %4 offset:4096\n\t" OP                                    \
                    " %3, %4 offset:6144\n\ts_waitcnt lgkmcnt(0)"                   \
                 : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)                       \
                 : "v"(addr), "v"(dep));                                            \
    out[0] = r0;                                                                    \
    out[1] = r1;                                                                    \
    out[2] = r2;                                                                    \
    out[3] = r3;                                                                    \
  }

template <int NBW, typename T>
__device__ __forceinline__ void lds_read_rows(T (&out)[NBW], uint32_t addr, uint32_t dep) {
  if constexpr (sizeof(T) == 4) {
    if constexpr (NBW == 2) MOE_FP4_LDS_READ2("ds_read_b32", T) else MOE_FP4_LDS_READ4("ds_read_b32", T)
  } else if constexpr (sizeof(T) == 8) {
    if constexpr (NBW == 2) MOE_FP4_LDS_READ2("ds_read_b64", T) else MOE_FP4_LDS_READ4("ds_read_b64", T)
  } else {
    if constexpr (NBW == 2) MOE_FP4_LDS_READ2("ds_read_b128", T) else MOE_FP4_LDS_READ4("ds_read_b128", T)
  }
}
#undef MOE_FP4_LDS_READ2
#undef MOE_FP4_LDS_READ4

// Weight scales of one stage from the LDS span buffer `buf` (stage j of its
// span): lane (c, g) of block jb reads row 16*jb + c, bytes 16*KSUB*j +
// 4*KSUB*g .. +4*KSUB of the line, which the copy stored with its 16-byte
// chunks swizzled by row.
template <int NBW, int KSUB>
__device__ __forceinline__ void read_line_scales(uint32_t (&ws)[NBW][KSUB], const uint8_t* buf,
                                                 int32_t j, int c, int g, uint32_t dep) {
  const int o = 16 * KSUB * j + 4 * KSUB * g;
  const int chunk = (o >> 4) ^ (c & 7), within = o & 15;
  const uint32_t addr = lds_addr(buf) + (uint32_t)(c * 128 + 16 * chunk + within);
  if constexpr (KSUB == 1) {
    uint32_t r[NBW];
    lds_read_rows<NBW>(r, addr, dep);
#pragma unroll
    for (int jb = 0; jb < NBW; ++jb) ws[jb][0] = r[jb];
  } else if constexpr (KSUB == 2) {
    u32x2_t r[NBW];
    lds_read_rows<NBW>(r, addr, dep);
#pragma unroll
    for (int jb = 0; jb < NBW; ++jb) {
      ws[jb][0] = r[jb][0];
      ws[jb][1] = r[jb][1];
    }
  } else {
    u32x4_t r[NBW];
    lds_read_rows<NBW>(r, addr, dep);
#pragma unroll
    for (int jb = 0; jb < NBW; ++jb) {
      ws[jb][0] = r[jb][0];
      ws[jb][1] = r[jb][1];
      ws[jb][2] = r[jb][2];
      ws[jb][3] = r[jb][3];
    }
  }
}

template <int MB, int NBW, int KSUB, bool SKIP>
__device__ __forceinline__ void compute_stage(const Stage<MB, NBW, KSUB>& st,
                                              const uint32_t (&wsd)[NBW][KSUB], int32_t rows_valid,
                                              float4_t (&acc)[NBW][MB]) {
#pragma unroll
  for (int s = 0; s < KSUB; ++s) {
    // Block scales of this sub-step, as FP16 value * 2^-8: scale t/2 serves MFMA t.
    half2_t wsc[NBW][2], asc[MB][2];
#pragma unroll
    for (int jb = 0; jb < NBW; ++jb) {
      wsc[jb][0] = scale_pair_x2m8<false>(wsd[jb][s]);
      wsc[jb][1] = scale_pair_x2m8<true>(wsd[jb][s]);
    }
#pragma unroll
    for (int ib = 0; ib < MB; ++ib) {
      asc[ib][0] = scale_pair_x2m8<false>(st.as[ib][s]);
      asc[ib][1] = scale_pair_x2m8<true>(st.as[ib][s]);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int half = t >> 2, word = t & 3, sidx = (t >> 1) & 1, spair = t >> 2;
      half8_t af[MB];
#pragma unroll
      for (int ib = 0; ib < MB; ++ib)
        af[ib] = dequant8(st.a[ib][s][half][word], asc[ib][spair][sidx]);
      // Column blocks past n hold zeros and rows past the expert repeat its
      // first row; neither is stored.  With SKIP, row blocks wholly past the
      // expert skip their MFMAs (a uniform branch).  Without it every loaded
      // register is consumed on every path: a load whose result some path
      // skipped would look pending to the compiler on the next iteration and
      // cost a wait there, which matters when items end every stage or two.
#pragma unroll
      for (int jb = 0; jb < NBW; ++jb) {
        const half8_t wf = dequant8(st.w[jb][s][half][word], wsc[jb][spair][sidx]);
#pragma unroll
        for (int ib = 0; ib < MB; ++ib) {
          if (!SKIP || 16 * ib < rows_valid)
            acc[jb][ib] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf, af[ib], acc[jb][ib], 0, 0, 0);
        }
      }
    }
  }
}

// Registers the stores of the last finished item read: kept allocated (see
// hold_stores) until a later wait shows the stores complete, so no following
// instruction overwrites them while a store may still be reading them.
template <int MB, int NBW>
struct PendingStores {
  u32x2_t data[NBW][MB];
  uint32_t voff[MB];
  u32x4_t rows[2 * MB];  // staged epilogue: 8 rows x 128 bytes per store
  uint32_t rvoff;
};

template <int MB, int NBW, bool STAGED, bool SW = false>
__device__ __forceinline__ void hold_stores(const PendingStores<MB, NBW>& ps) {
  if constexpr (SW) {
    // SwiGLU epilogue: per row block one code dword, one scale byte and their offsets.
#pragma unroll
    for (int ib = 0; ib < MB; ++ib) asm volatile("" ::"v"(ps.voff[ib]), "v"(ps.data[0][ib]), "v"(ps.data[1][ib]));
  } else if constexpr (STAGED) {
    asm volatile("" ::"v"(ps.rvoff));
#pragma unroll
    for (int k = 0; k < 2 * MB; ++k) asm volatile("" ::"v"(ps.rows[k]));
  } else {
#pragma unroll
    for (int ib = 0; ib < MB; ++ib) {
      asm volatile("" ::"v"(ps.voff[ib]));
#pragma unroll
      for (int jb = 0; jb < NBW; ++jb) asm volatile("" ::"v"(ps.data[jb][ib]));
    }
  }
}

// LDS bytes of a wave's output tile for the staged epilogue: 16*MB rows of
// 32*NBW bytes, padded by 16 bytes per row against bank conflicts.
template <int MB, int NBW>
constexpr int out_tile_pitch() { return 32 * NBW + 16; }
template <int MB, int NBW>
constexpr int out_tile_bytes() { return 16 * MB * out_tile_pitch<MB, NBW>(); }

// Staged BF16 store of a finished 64-column item: the wave writes its tile to
// LDS in the accumulator layout (lane (c, g): row 16*ib + c, columns 16*jb +
// 4g .. +3), reads it back row-major (lane l: row 8k + l/8, columns 8*(l%8)
// .. +7) and stores 16 bytes per lane, so every store instruction writes 8
// whole 128-byte row segments instead of 16 rows x 32 bytes.  A wave's LDS
// operations execute in order, so no barrier is needed, and the next item's
// writes cannot overtake these reads.  Rows past the expert's end fall
// outside the store resource; a column chunk past n gets an out-of-range
// offset.
template <int MB, int NBW>
__device__ __forceinline__ void epilogue_staged(float4_t (&acc)[NBW][MB], const ItemPos& it,
                                                int lane, const GemmArgs& p,
                                                PendingStores<MB, NBW>& ps, uint8_t* tile) {
  static_assert(NBW == 4, "row segments of 64 columns");
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  constexpr int kPitch = out_tile_pitch<MB, NBW>();
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int jb = 0; jb < NBW; ++jb) {
#pragma unroll
    for (int ib = 0; ib < MB; ++ib) {
      const float4_t v = acc[jb][ib];
      const bf16x4_t b = {(__bf16)(v[0] * it.alpha), (__bf16)(v[1] * it.alpha),
                          (__bf16)(v[2] * it.alpha), (__bf16)(v[3] * it.alpha)};
      *reinterpret_cast<u32x2_t*>(tile + (16 * ib + c) * kPitch + 32 * jb + 8 * g) =
          __builtin_bit_cast(u32x2_t, b);
      acc[jb][ib] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }
  const int32_t ldo = (int32_t)p.ldo;
  const rsrc_t o = make_rsrc(p.out + (int64_t)it.row0 * ldo,
                             (uint32_t)((int64_t)it.rows_valid * ldo * 2));
  const int r8 = lane >> 3, q = lane & 7;
  const bool col_ok = it.n0 + 8 * q < (int32_t)p.n;
  ps.rvoff = col_ok ? (uint32_t)((r8 * ldo + it.n0 + 8 * q) * 2) : kOutOfRange;
#pragma unroll
  for (int k = 0; k < 2 * MB; ++k)
    ps.rows[k] = *reinterpret_cast<const u32x4_t*>(tile + (8 * k + r8) * kPitch + 16 * q);
#pragma unroll
  for (int k = 0; k < 2 * MB; ++k)
    __builtin_amdgcn_raw_buffer_store_b128(ps.rows[k], o, ps.rvoff, uniform(16 * k * ldo), 0);
}

// BF16 store of a finished item.  Lane (c, g) holds rows 16*ib + c, columns
// 16*jb + 4g .. +3.  Stores go through a buffer resource covering exactly the
// item's valid rows, so rows past the expert's end fall outside it and are
// dropped; a column block past n (uniform) is skipped.
template <int MB, int NBW>
__device__ __forceinline__ void epilogue(float4_t (&acc)[NBW][MB], const ItemPos& it,
                                         int c, int g, const GemmArgs& p,
                                         PendingStores<MB, NBW>& ps) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  const int32_t ldo = (int32_t)p.ldo;
  const rsrc_t o = make_rsrc(p.out + (int64_t)it.row0 * ldo,
                             (uint32_t)((int64_t)it.rows_valid * ldo * 2));
#pragma unroll
  for (int ib = 0; ib < MB; ++ib)
    ps.voff[ib] = (uint32_t)(((16 * ib + c) * ldo + it.n0 + 4 * g) * 2);
#pragma unroll
  for (int jb = 0; jb < NBW; ++jb) {
#pragma unroll
    for (int ib = 0; ib < MB; ++ib) {
      const float4_t v = acc[jb][ib];
      const bf16x4_t b = {(__bf16)(v[0] * it.alpha), (__bf16)(v[1] * it.alpha),
                          (__bf16)(v[2] * it.alpha), (__bf16)(v[3] * it.alpha)};
      ps.data[jb][ib] = __builtin_bit_cast(u32x2_t, b);
      acc[jb][ib] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    if (it.n0 + 16 * jb < (int32_t)p.n) {
#pragma unroll
      for (int ib = 0; ib < MB; ++ib)
        __builtin_amdgcn_raw_buffer_store_b64(ps.data[jb][ib], o, ps.voff[ib] + 32u * jb, 0, 0);
    }
  }
}

// Finalize epilogue: routed row r of the item adds row_weight[r] * alpha *
// acc into FP32 row out_token[r] of fin_out, one atomic add per element, so the
// top-k rows of a token, which belong to different experts and therefore to
// different work items, meet in token order without a BF16 round trip
// ("Peering into the CUTLASS Kernel", section "Input Knowledge Required", item
// 5: the epilogue that performs the final output write).  The order in which a
// token's rows arrive is not fixed.  Lane (c, g) holds rows 16*ib + c, columns
// 16*jb + 4g .. +3; rows past the expert's end, and tokens outside
// [0, num_tokens), get an out-of-range offset; a column block past n
// (uniform) is skipped.
template <int MB, int NBW>
__device__ __forceinline__ void epilogue_finalize(float4_t (&acc)[NBW][MB], const ItemPos& it,
                                                  int c, int g, const GemmArgs& p,
                                                  const int32_t (&tok)[MB],
                                                  const float (&wt)[MB]) {
  const int32_t ldt = (int32_t)p.fin_ldo, ntok = (int32_t)p.num_tokens;
  const rsrc_t o = make_rsrc(p.fin_out, (uint32_t)((int64_t)ntok * ldt * 4));
  uint32_t base[MB];
#pragma unroll
  for (int ib = 0; ib < MB; ++ib) {
    const bool ok = 16 * ib + c < it.rows_valid && tok[ib] >= 0 && tok[ib] < ntok;
    base[ib] = ok ? (uint32_t)(tok[ib] * ldt + it.n0 + 4 * g) * 4u : kOutOfRange;
  }
#pragma unroll
  for (int jb = 0; jb < NBW; ++jb) {
    if (it.n0 + 16 * jb < (int32_t)p.n) {
#pragma unroll
      for (int ib = 0; ib < MB; ++ib) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = (acc[jb][ib][i] * it.alpha) * wt[ib];
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v, o, base[ib] + 64u * jb + 4u * i, 0, 0);
        }
      }
    }
#pragma unroll
    for (int ib = 0; ib < MB; ++ib) acc[jb][ib] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
}

// SiLU in FP32: x / (1 + e^-x), with the device library's expf and an IEEE
// division; very negative x gives e^-x = inf and the limit -0.
__device__ __forceinline__ float silu_f32(float x) { return x / (1.0f + expf(-x)); }

// SwiGLU + NVFP4 epilogue of the gate+up projection: the FINALIZE epilogue
// with an activation and a quantisation ("Peering into the CUTLASS Kernel",
// section "Input Knowledge Required", item 5), read as the gated SiLU between
// the two projections of a Mixture-of-Experts FFN.  An item covers 32
// intermediate columns i0 .. i0+31 (i0 = it.n0): acc[0..1] hold the gate
// columns, acc[2..3] the up columns, so lane (c, g) holds, for row 16*ib + c,
// elements 4g .. 4g+3 of intermediate blocks i0/16 (b = 0) and i0/16 + 1
// (b = 1).  Per element, in FP32: gate and up = fl(acc * alpha) (the value the
// plain path rounds to BF16), h = fl(silu(gate) * up).  Per 16-element block,
// with the caller's static tensor scale gt: amax over the block (the 4 lanes
// of a row exchange their maxima), scale = E4M3_RNE(fl(amax / fl(6 gt))),
// s = fl(E4M3 value * gt), code = E2M1_RNE(fl(h / s)) (all zero when s = 0):
// the activation quantiser's recipe with a static scale.  Output rows are the
// routed rows (h_q [m_total][n/4], h_sf [m_total][n/32]), which the down
// projection reads as its activations.  Lane g stores bytes 4g .. 4g+3 of the
// row's 16 code bytes (gathered from two lanes) and lanes g = 0, 1 the scale
// byte of block g; rows past the expert's end fall outside the item's store
// resources and blocks past n/2 get an out-of-range offset.
template <int MB, int NBW>
__device__ __forceinline__ void epilogue_swiglu(float4_t (&acc)[NBW][MB], const ItemPos& it,
                                                const GemmArgs& p, PendingStores<MB, NBW>& ps) {
  static_assert(NBW == 4, "gate and up blocks of 32 intermediate columns");
  // The lane number, read here rather than taken from the caller: the values
  // derived from it below are then computed per epilogue instead of being
  // hoisted out of the main loop, where they would hold registers (or spill)
  // across every stage.
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  const int c = lane & 15, g = lane >> 4;
  const int32_t inter = (int32_t)(p.n >> 1);
  const int32_t qrow = inter >> 1, srow = inter >> 4;  // bytes per row: codes, scales
  const float gt = ((sconst_f32)p.h_scale)[0];
  const float six_g = 6.0f * gt;
  const rsrc_t oq = make_rsrc(p.h_q + (int64_t)it.row0 * qrow, (uint32_t)(it.rows_valid * qrow));
  const rsrc_t os = make_rsrc(p.h_sf + (int64_t)it.row0 * srow, (uint32_t)(it.rows_valid * srow));
  const bool q_ok = it.n0 + 16 * (g >> 1) < inter;
  const bool s_ok = g < 2 && it.n0 + 16 * g < inter;
  // Lane g's code bytes 4g .. 4g+3 are the 16-bit halves of lanes 2g and
  // 2g+1 (mod 4) of the same row, for block g / 2.
  const int src0 = c + 16 * ((2 * g) & 3), src1 = c + 16 * ((2 * g + 1) & 3);
  const int sh = 16 * (g >> 1);
#pragma unroll
  for (int ib = 0; ib < MB; ++ib) {
    uint32_t half[2], sfb[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float4_t gv = acc[b][ib], uv = acc[2 + b][ib];
      float h[4];
      float m = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float gate = gv[v] * it.alpha, up = uv[v] * it.alpha;
        h[v] = silu_f32(gate) * up;
        m = fmaxf(m, fabsf(h[v]));
      }
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      // E4M3 block scale, nearest even; clamping to 448 first makes it saturate.
      const float r = fminf(m / six_g, 448.0f);
      sfb[b] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r, r, 0, false) & 0xFFu;
      const float sc = __builtin_amdgcn_cvt_f32_fp8(sfb[b], 0) * gt;
      const bool live = sc != 0.0f;
      const float y0 = live ? h[0] / sc : 0.0f, y1 = live ? h[1] / sc : 0.0f;
      const float y2 = live ? h[2] / sc : 0.0f, y3 = live ? h[3] / sc : 0.0f;
      // E2M1 codes: nearest even, saturating, sign kept (element 2i low nibble).
      const uint32_t c01 = (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y0, y1, 1.0f, 0) & 0xFFu;
      const uint32_t c23 = (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y2, y3, 1.0f, 0) & 0xFFu;
      half[b] = c01 | (c23 << 8);
      acc[b][ib] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
      acc[2 + b][ib] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const uint32_t both = half[0] | (half[1] << 16);
    const uint32_t v0 = (uint32_t)__shfl((int)both, src0, 64);
    const uint32_t v1 = (uint32_t)__shfl((int)both, src1, 64);
    const int32_t row = 16 * ib + c;
    ps.data[0][ib][0] = ((v0 >> sh) & 0xFFFFu) | (((v1 >> sh) & 0xFFFFu) << 16);
    ps.data[0][ib][1] = g == 0 ? sfb[0] : sfb[1];
    ps.voff[ib] = q_ok ? (uint32_t)(row * qrow + (it.n0 >> 1) + 4 * g) : kOutOfRange;
    ps.data[1][ib][0] = s_ok ? (uint32_t)(row * srow + (it.n0 >> 4) + g) : kOutOfRange;
    __builtin_amdgcn_raw_buffer_store_b32(ps.data[0][ib][0], oq, ps.voff[ib], 0, 0);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)ps.data[0][ib][1], os, ps.data[1][ib][0], 0, 0);
  }
}

// Tiles of one or two row blocks with 256-element stages, and one-row-block
// tiles with 512-element stages whose weight scales come through LDS, fit two
// wavefronts per SIMD (at most 256 registers): ask for that, or the allocator
// drifts past it and halves the wavefronts in flight.
template <int MB, int NBW, int KSUB, int WAVES, bool SL, bool PK, int R, int EPI>
__global__ __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu((MB <= 2 && KSUB == 1) || (MB == 1 && KSUB == 2 && SL) ? 2 : 1)))
void k_grouped_gemm(const GemmArgs p) {
  static_assert(R == 2 || (R == 3 && !SL), "a third register stage only without scale lines");
  constexpr bool FIN = EPI == kEpiFinalize, SW = EPI == kEpiSwiglu;
  // Kernels without scale lines stage the plain store through a per-wave LDS
  // tile (the other epilogues need none).
  constexpr bool STAGED = !SL && NBW == 4 && EPI == kEpiStore;
  static_assert(EPI == kEpiStore || NBW == 4, "finalize and SwiGLU kernels use 4 row blocks");
  // Output columns (intermediate columns with SwiGLU) per item.
  constexpr int kItemCols = SW ? 32 : 16 * NBW;
  static_assert(!PK || NBW == 4, "packed weights are read by 64-column items");
  constexpr int BM = 16 * MB;
  constexpr int NTHR = WAVES * 64;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int32_t* prefix = reinterpret_cast<int32_t*>(smem);  // [num_experts + 1] item prefix
  int32_t* offl = prefix + (p.num_experts + 1);         // [num_experts + 1] clamped offsets
  __shared__ int32_t wave_sum[WAVES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);  // the compiler cannot see that this is wave-uniform
  const int E = p.num_experts;
  const int32_t m_total = (int32_t)p.m_total;

  const int32_t total_items = build_worklist<NTHR>(p, BM, prefix, offl, wave_sum);


  // ---- XCD-aware wavefront numbering ----
  // Items are dealt in rounds of nw (one per wavefront).  Within a round, the
  // active workgroups (those whose waves have an item) are spread evenly over
  // the 8 XCDs, and consecutive items go to consecutive waves of one XCD.  The
  // hardware places workgroup b on XCD b % 8; the grid is a multiple of 8.
  const int nblk = gridDim.x, b = blockIdx.x;
  const int32_t nw = nblk * WAVES;
  const int32_t rounds = (total_items + nw - 1) / nw;
  if (rounds == 0) return;
  const int32_t last_items = total_items - (rounds - 1) * nw;
  const int32_t lw_full = logical_block(b, nblk, nblk) * WAVES + wave;
  const int32_t lw_last =
      logical_block(b, nblk, (last_items + WAVES - 1) / WAVES) * WAVES + wave;
  const int32_t my_items = (rounds - 1) + (lw_last < last_items ? 1 : 0);
  if (my_items == 0) return;
  auto item_of = [&](int32_t j) -> int32_t {
    return j * nw + (j == rounds - 1 ? lw_last : lw_full);
  };

  const int c = lane & 15, g = lane >> 4;
  const int32_t nsub = (int32_t)(p.k / 256);    // 256-element sub-steps per row
  const int32_t nst = nsub / KSUB;              // stages per item
  const int32_t units = my_items * nst;         // < 2^31 (host bound on items * stages)
  const rsrc_t a_rs = make_rsrc(p.a_q, (uint32_t)(p.a_rows * (p.k >> 1)));
  const rsrc_t as_rs = make_rsrc(p.a_sf, (uint32_t)(p.a_rows * (p.k >> 4)));
  const int32_t n = (int32_t)p.n, nbk = (int32_t)(p.k >> 4);

  // This wave's scale-line buffers (SL): span buffers 0 and 1, then the sink.
  constexpr int kSpanStages = kSpan / (256 * KSUB);  // stages per span
  constexpr int kBufBytes = 16 * NBW * 128;
  uint8_t* const sl_base = smem + worklist_bytes(E) + (size_t)wave * scale_lds_per_wave<NBW>();
  uint8_t* const out_tile = smem + worklist_bytes(E) + (size_t)wave * out_tile_bytes<MB, NBW>();
  auto line_copy = [&](int32_t round, int32_t st) -> LineCopy {
    LineCopy lc;
    const bool start = st % kSpanStages == 0;
    const int32_t span = st / kSpanStages;
    const int32_t nsp = nst / kSpanStages;
    const int32_t buf = (round * nsp + span) & 1;
    lc.dst = start ? sl_base + buf * kBufBytes : sl_base + 2 * kBufBytes;
    lc.span = start ? span : -1;
    return lc;
  };

  float4_t acc[NBW][MB];
#pragma unroll
  for (int jb = 0; jb < NBW; ++jb)
#pragma unroll
    for (int ib = 0; ib < MB; ++ib) acc[jb][ib] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // A ring of R register stages.  Unit v (stage ld_st of the wave's item
  // round ld_round) goes to slot v % R with its own lane offsets l[slot] and
  // item position pos[slot]; the loads run R-1 units ahead of the unit being
  // computed.  cp_round / cp_st count the unit being computed.
  // nx: the item after ld's, located and with its scalar loads in flight.
  const WorkList wl{prefix, offl};
  ItemPos ld_pos, nx, pos[R];
  ItemLoads<MB, NBW> l[R];
  int32_t ld_round = 0, ld_st = 0, cp_round = 0, cp_st = 0;
  // Row-index entries: of the item being started (first item), then of nx.
  const rsrc_t idx_rs = make_rsrc(p.a_row_index, p.a_row_index ? (uint32_t)(4 * m_total) : 0u);
  uint32_t nrow[MB], frow[MB];  // frow: the first item's entries, for its first stage
  ld_pos = locate(item_of(0), 0, wl, p, 16 * MB, kItemCols, lane);
#pragma unroll
  for (int ib = 0; ib < MB; ++ib) frow[ib] = row_index_load(idx_rs, ld_pos, ib, c);
  item_loads_w<MB, NBW, KSUB, PK, SW>(ld_pos, p, lane, l[0]);
  // Finalize: each row's destination token and routing weight, fetched like
  // the row-index entries (ntok/nwt: of the item being started, then of nx)
  // and carried per register stage to the item's epilogue (ftok/fwt).
  const rsrc_t tok_rs = make_rsrc(p.out_token, FIN ? (uint32_t)(4 * m_total) : 0u);
  const rsrc_t wt_rs = make_rsrc(p.row_weight, FIN ? (uint32_t)(4 * m_total) : 0u);
  int32_t ntok[MB], ftok[R][MB];
  float nwt[MB], fwt[R][MB];
  if constexpr (FIN) {
#pragma unroll
    for (int ib = 0; ib < MB; ++ib) {
      ntok[ib] = (int32_t)row_index_load(tok_rs, ld_pos, ib, c);
      nwt[ib] = __builtin_bit_cast(float, row_index_load(wt_rs, ld_pos, ib, c));
      ftok[0][ib] = ntok[ib];
      fwt[0][ib] = nwt[ib];
    }
  }
  // nx: the item after ld's, located a stage or more before it is needed
  // (the last item repeats itself; that copy is never used).
  auto locate_next = [&](int32_t round) {
    const int32_t r = round + 1 < my_items ? round + 1 : round;
    nx = locate(item_of(r), ld_pos.e, wl, p, 16 * MB, kItemCols, lane);
  };
  locate_next(0);
  pos[0] = ld_pos;
  // Fetch nx's row-index entries now; every later issue refetches them for
  // the current nx, unconditionally (no load behind a branch), so they are a
  // unit or more old when an item change consumes them.
  auto prefetch_rows = [&]() {
#pragma unroll
    for (int ib = 0; ib < MB; ++ib) nrow[ib] = row_index_load(idx_rs, nx, ib, c);
    if constexpr (FIN) {
#pragma unroll
      for (int ib = 0; ib < MB; ++ib) {
        ntok[ib] = (int32_t)row_index_load(tok_rs, nx, ib, c);
        nwt[ib] = __builtin_bit_cast(float, row_index_load(wt_rs, nx, ib, c));
      }
    }
  };
  prefetch_rows();
  // Move the load position to the next unit: a new item (already located)
  // gets its lane offsets in dst, otherwise dst takes src's offsets.
  auto advance = [&](ItemLoads<MB, NBW>& dst, const ItemLoads<MB, NBW>& src) -> bool {
    if (++ld_st == nst) {
      ld_st = 0;
      ++ld_round;
      ld_pos = nx;
      item_loads<MB, NBW, KSUB, PK, SW>(ld_pos, p, lane, nrow, dst);
      locate_next(ld_round);
      return true;
    }
    dst = src;
    return false;
  };
  PendingStores<MB, NBW> ps;
#pragma unroll
  for (int ib = 0; ib < MB; ++ib) {
    ps.voff[ib] = 0;
#pragma unroll
    for (int jb = 0; jb < NBW; ++jb) ps.data[jb][ib] = u32x2_t{0u, 0u};
  }
  ps.rvoff = 0;
#pragma unroll
  for (int k = 0; k < 2 * MB; ++k) ps.rows[k] = u32x4_t{0u, 0u, 0u, 0u};
  auto retire = [&](const ItemPos& it, const int32_t (&tok)[MB], const float (&wt)[MB]) {
    if (++cp_st == nst) {
      if constexpr (FIN) epilogue_finalize<MB, NBW>(acc, it, c, g, p, tok, wt);
      else if constexpr (SW) epilogue_swiglu<MB, NBW>(acc, it, p, ps);
      else if constexpr (STAGED) epilogue_staged<MB, NBW>(acc, it, lane, p, ps, out_tile);
      else epilogue<MB, NBW>(acc, it, c, g, p, ps);
      cp_st = 0;
      ++cp_round;
    }
  };
  // Weight scales of the stage about to be computed.
  auto stage_scales = [&](const Stage<MB, NBW, KSUB>& st, uint32_t (&wsd)[NBW][KSUB]) {
    if constexpr (SL) {
      const int32_t nsp = nst / kSpanStages;
      const int32_t buf = (cp_round * nsp + cp_st / kSpanStages) & 1;
      // The stage's last load (the activation scales) orders the read after
      // the stage's line copy: loads complete in issue order.
      read_line_scales<NBW, KSUB>(wsd, sl_base + buf * kBufBytes, cp_st % kSpanStages, c, g,
                                  st.as[MB - 1][KSUB - 1]);
    } else {
#pragma unroll
      for (int jb = 0; jb < NBW; ++jb)
#pragma unroll
        for (int s = 0; s < KSUB; ++s) wsd[jb][s] = st.ws[jb][s];
    }
  };
  // Issue unit v's loads into slot `to` (lane offsets advanced from slot
  // `from`).  Past the last unit the issue still happens, keeping the code
  // free of branches around loads, but with out-of-range offsets: no data.
  Stage<MB, NBW, KSUB> s[R];
  auto issue = [&](int to, int from, int32_t v) {
    const bool more = v < units;
    bool fresh = false;
    if (more) fresh = advance(l[to], l[from]); else l[to] = nowhere<MB, NBW>(l[from]);
    pos[to] = ld_pos;
    if constexpr (FIN) {
#pragma unroll
      for (int ib = 0; ib < MB; ++ib) {
        ftok[to][ib] = fresh ? ntok[ib] : ftok[from][ib];
        fwt[to][ib] = fresh ? nwt[ib] : fwt[from][ib];
      }
    }
    prefetch_rows();
    issue_loads<MB, NBW, KSUB, SL, PK, SW>(s[to], l[to], a_rs, as_rs, ld_st,
                                       more ? line_copy(ld_round, ld_st)
                                            : LineCopy{sl_base + 2 * kBufBytes, -1},
                                       n, nbk);
  };

  uint32_t wsd[NBW][KSUB];
  // The first stage: the weight side at once; the activation side once the row
  // index has arrived (the weight loads must not wait for it).
  issue_loads<MB, NBW, KSUB, SL, PK, SW, 1>(s[0], l[0], a_rs, as_rs, ld_st, line_copy(ld_round, ld_st), n, nbk);
  __builtin_amdgcn_sched_barrier(0);
  item_loads_a<MB, NBW, KSUB>(ld_pos, p, lane, frow, l[0]);
  issue_loads<MB, NBW, KSUB, SL, PK, SW, 2>(s[0], l[0], a_rs, as_rs, ld_st, line_copy(ld_round, ld_st), n, nbk);
#pragma unroll
  for (int r = 1; r < R - 1; ++r) issue(r, r - 1, r);
  bool done = false;
  for (int32_t u = 0; !done; u += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (done) break;
      // Every step issues the unit R-1 ahead before computing this one, so
      // R-1 units are always in flight.
      issue((r + R - 1) % R, (r + R - 2) % R, u + r + R - 1);
      // Without the uniform branches of SL kernels, keep the scheduler from
      // sinking the next stage's loads into (or below) this stage's computation.
      if constexpr (!SL) __builtin_amdgcn_sched_barrier(0);
      stage_scales(s[r], wsd);
      compute_stage<MB, NBW, KSUB, SL>(s[r], wsd, pos[r].rows_valid, acc);
      hold<MB, NBW>(l[r]);
      if constexpr (!SL) hold_stores<MB, NBW, STAGED, SW>(ps);
      retire(pos[r], ftok[r], fwt[r]);
      done = u + r + 1 >= units;
    }
  }
}


// Register stages per wave.  Two (one unit in flight while one computes).
// A third was measured on the 32-row, 256-element-stage kernel: its extra
// registers spill, and the spill code's waits on in-flight loads cost more
// than the deeper prefetch gained.
template <int MB, int NBW, int KSUB, bool SL>
constexpr int register_stages() { return 2; }

template <int MB, int NBW, int KSUB, int WAVES, bool SL, bool PK = false, int EPI = kEpiStore>
hipError_t launch_tile(const GemmArgs& p, hipStream_t stream) {
  auto kern = k_grouped_gemm<MB, NBW, KSUB, WAVES, SL, PK, register_stages<MB, NBW, KSUB, SL>(), EPI>;
  const size_t lds = worklist_bytes(p.num_experts) +
                     (SL ? (size_t)WAVES * scale_lds_per_wave<NBW>()
                         : (NBW == 4 && EPI == kEpiStore ? (size_t)WAVES * out_tile_bytes<MB, NBW>() : 0));
  int resident = 0;
  hipError_t err = resident_groups(kern, WAVES * 64, lds, &resident);
  if (err != hipSuccess) return err;
  // Upper bound on the number of items: the host does not see the offsets.
  constexpr int BM = 16 * MB;
  const int64_t max_mtiles = p.m_total / BM + (p.m_total < p.num_experts ? p.m_total : p.num_experts);
  const int64_t max_items = max_mtiles * p.n_tiles;
  int64_t grid = resident;
  const int64_t need = (max_items + WAVES - 1) / WAVES;
  if (need < grid) grid = need;
  if (grid < 1) grid = 1;
  grid = (grid + kXcds - 1) / kXcds * kXcds;  // whole rounds over the XCDs
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WAVES * 64), lds, stream, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace moe_fp4
