// NVFP4 grouped GEMM for gfx950, workgroup items for experts of a few dozen
// rows: the prefill end of a skewed routing, where an expert owns more rows
// than one 16-row block but far fewer than the 256 that make the large tile
// pay ("Peering into the CUTLASS Kernel", section "Input Knowledge Required",
// item 4: one GEMM per expert over its routed rows; "Peering into the CUTLASS
// Kernel Scheduler", section "The Context": tile geometry decides the reuse at
// small per-expert M).
//
// The per-wave kernel dequantises its 64 weight rows once per 16-row item, so
// an expert of 48 rows converts every weight code three times, and the vector
// ALU, not HBM, bounds it.  Here a workgroup of 8 wavefronts (one per CU, two
// per SIMD) takes an item of up to 48 rows x 512 columns and converts each
// operand once:
//  * activations: per 256-element K stage the item's rows are dequantised
//    exactly to FP16 by the workgroup (one thread per row and 32-element run)
//    into one of two LDS buffers, and every wave reads its MFMA operands from
//    there;
//  * weights: each wave streams its own 64 weight rows (4 blocks of 16) into a
//    three-stage register ring (two stages in flight while one computes),
//    dequantises each fragment once and uses it for every 16-row block of the
//    item;
//  * weight scales: each wave copies the scale bytes of its 64 rows for 1024
//    K elements at a time (64 contiguous bytes per row) into a double-buffered
//    LDS area with buffer-to-LDS loads, and reads each stage's scales there.
//    Loading them per stage would read 16 bytes of 16 different rows' lines
//    per instruction; measured, that cost a fifth of the kernel's time.
// Products run on v_mfma_f32_16x16x32_f16 (weights as the A operand, 16 output
// columns; activations as B, 16 rows) with FP32 accumulation, and the tile
// leaves through LDS in 16-byte stores of whole row segments.  Row blocks past
// the item's rows issue no MFMAs (the K loop is instantiated per live block
// count).  One barrier per stage orders the activation buffers.
//
// K order: a stage is half of a 512-element granule (the packed weight
// layout's unit), and lane group g of a wave owns elements 128 g + 64 s ..
// +63 of granule half s, for weights and activations alike, so each product
// pairs the same element and packed and row-major weights give identical
// results.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "fp4_device.h"
#include "gemm_common.h"
#include "launch.h"

namespace moe_fp4 {
namespace {

typedef __attribute__((address_space(3))) void* mid_lds_ptr;

constexpr int kMWaves = 8;
constexpr int kMThreads = 64 * kMWaves;
constexpr int kMCols = 64 * kMWaves;  // output columns per item, 64 per wavefront
constexpr int kMK = 256;              // K elements per stage
constexpr int kMRow = 2 * kMK;        // bytes of one activation row of a stage in FP16
// LDS pitch of a stage row: 16 bytes of padding put the 16 rows one 16-byte
// access touches (same chunk, consecutive rows) in distinct banks, and every
// per-step and per-block position stays an immediate offset.
constexpr int kMPitch = kMRow + 16;
constexpr int kMGranule = 512;        // K elements per granule (two stages)
// Weight scales: K elements per LDS copy (4 stages), bytes per row of one copy,
// and the LDS of one wave: two copies of 64 rows, then a 1 KB sink for the
// copies of stages that start none.
constexpr int kMScaleK = 1024;
constexpr int kMScaleRow = kMScaleK / 16;
constexpr int kMScaleBuf = 64 * kMScaleRow;
constexpr int kMScaleWave = 2 * kMScaleBuf + 1024;

template <int MB>
__host__ __device__ constexpr size_t mid_stage_bytes() {
  return (size_t)16 * MB * kMPitch;
}
// Dynamic LDS of a workgroup (the scale copies' kMWaves * kMScaleWave bytes are
// a static array beside it).
template <int MB>
__host__ __device__ constexpr size_t mid_lds_bytes(int num_experts) {
  return worklist_bytes(num_experts) + 2 * mid_stage_bytes<MB>();
}

// Calls f(integral_constant<int, 0>) .. f(integral_constant<int, N-1>), unrolled.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// One stage of raw loads: a wave's 4 weight row blocks (the lane's 64 codes of
// each), and the loader thread's 32 activation codes and their scale dword.
struct MidStage {
  u32x4_t w[4][2];
  u32x4_t a;
  uint32_t as;
};

// Per-item buffer resources and lane offsets (bytes), fixed for the item; the
// stage position goes in the scalar offset.
struct MidLoads {
  rsrc_t w, ws;
  uint32_t wq[4];    // weight codes, per row block
  uint32_t sl;       // scale copy: row grp0 + lane % 16 (+ 16 per row block), chunk lane / 16
  uint32_t aq, asc;  // loader thread's activation codes and scales
  int32_t wk;        // packed: bytes of one granule of the wave's 64-row group
};

// Issue stage st's loads into `s`: the scale copy of the 1024-element span the
// stage starts (st % 4 == 0; the other stages copy nothing, out of range into
// the wave's sink), then the activations (the end of the previous stage waits
// for them), then the weight codes.  Past the last stage (`past`) every offset
// is pushed out of range, so the loads return zeros without memory traffic and
// every issue stays unconditional.  The activation offsets, scalar part
// included, stay far below 2^32 even then (rows of at most 2^31 - 4097 bytes
// in all, a few hundred bytes past a row's end), so a past stage's activations
// are zero, and its products add exact zeros whatever its weight loads return
// (a dequantised weight is always finite).
template <bool PK, int SUB>
__device__ __forceinline__ void mid_issue(MidStage& s, const MidLoads& l, const rsrc_t& a_rs,
                                          const rsrc_t& as_rs, int32_t st, bool past,
                                          uint8_t* sl_base, int32_t nbk) {
  const uint32_t kill = past ? kOutOfRange : 0u;
  const int32_t granule = st >> 1;
  {
    const bool on = (st & 3) == 0 && !past;
    uint8_t* dst = on ? sl_base + ((st >> 2) & 1) * kMScaleBuf : sl_base + 2 * kMScaleBuf;
    const int32_t soff = uniform(on ? (st >> 2) * kMScaleRow : 0);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const uint32_t v = on ? l.sl + (uint32_t)(16 * jb * nbk) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(l.ws, (mid_lds_ptr)(on ? dst + 1024 * jb : dst), 16, v,
                                               soff, 0, 0);
    }
  }
  const int32_t q = uniform(granule * (kMGranule / 2) + 32 * SUB);
  const int32_t sc = uniform(granule * (kMGranule / 16) + 4 * SUB);
  s.a = __builtin_amdgcn_raw_buffer_load_b128(a_rs, l.aq | kill, q, 0);
  s.as = __builtin_amdgcn_raw_buffer_load_b32(as_rs, l.asc | kill, sc, 0);
  // Packed: granule t of block j is 4 KB, its halves s 2 KB apart and the two
  // 16-byte pieces of a lane 1 KB apart (one load of the wave reads 1 KB).
  const int32_t qw = PK ? uniform(granule * l.wk + 2048 * SUB) : q;
  constexpr uint32_t kHalf = PK ? 1024u : 16u;
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    s.w[jb][0] = __builtin_amdgcn_raw_buffer_load_b128(l.w, l.wq[jb] | kill, qw, kLoadStreamOnce);
    s.w[jb][1] =
        __builtin_amdgcn_raw_buffer_load_b128(l.w, (l.wq[jb] + kHalf) | kill, qw, kLoadStreamOnce);
  }
}

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t mid_lds_addr(const uint8_t* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)p);
}

// The loader thread's 32 activation values of a stage (half ah of lane group
// ag's 64-element run), dequantised exactly to FP16 into LDS row `ar` of
// `buf`: 16-byte chunk 8 ag + 4 ah + w holds values 8w .. 8w+7 of the half.
__device__ __forceinline__ void mid_put_act(uint8_t* buf, int ar, int ag, int ah, const MidStage& s) {
  const half2_t sp = ah ? scale_pair_x2m8<true>(s.as) : scale_pair_x2m8<false>(s.as);
  uint8_t* run = buf + ar * kMPitch + 128 * ag + 64 * ah;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    *reinterpret_cast<half8_t*>(run + 16 * w) = dequant8(s.a[w], sp[w >> 1]);
}

// The workgroup barrier of the K loop, without the memory fence of
// __syncthreads: a workgroup-scope fence makes the compiler wait for every
// buffer-to-LDS copy in flight (and, loads completing in order, for every load
// before it), which drained the prefetch ring at each stage.  The activation
// stages need no more than their LDS writes completed before the barrier; the
// scale copies are read only by the wave that made them.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void mid_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left open
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// This stage's weight scale dwords of the wave's 4 row blocks, from the LDS
// copy at `sl` (this stage's span): lane (c, g) of block jb takes row 16 jb +
// c, bytes 32 gh + 8 g + 4 sub of the row's 64 (gh: the stage's granule in
// the span).  A copy instruction stored block jb's rows at 1 KB x jb, row r's
// 16-byte chunk u at 16 (r + 16 u).  `dep` is a register of a load issued
// after the copy, so waiting for it (loads complete in issue order) orders
// the reads after the copy; the reads and their wait are one asm statement,
// so the compiler sees no LDS read it could move ahead of that.
__device__ __forceinline__ void mid_read_scales(uint32_t (&wsd)[4], const uint8_t* sl, int c, int g,
                                                int gh, int sub, uint32_t dep) {
  const int b = 32 * gh + 8 * g + 4 * sub;
  const uint32_t addr = mid_lds_addr(sl) + (uint32_t)(16 * (c + 16 * (b >> 4)) + (b & 15));
  uint32_t r0, r1, r2, r3;
  asm volatile(
      "ds_read_b32 %0, %4\n\tds_read_b32 %1, %4 offset:1024\n\tds_read_b32 %2, %4 offset:2048\n\t"
      "ds_read_b32 %3, %4 offset:3072\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(addr), "v"(dep));
  wsd[0] = r0;
  wsd[1] = r1;
  wsd[2] = r2;
  wsd[3] = r3;
}

// The MFMAs of one stage for a wave: per 32-element step t, lane (c, g) reads
// activation row 16 ib + c, values 8t .. 8t+7 of lane group g's run, for the
// LIVE row blocks, and dequantises its weight fragment of each row block jb
// once for all of them.
template <int MB, int LIVE>
__device__ __forceinline__ void mid_compute(const MidStage& s, const uint32_t (&wsd)[4],
                                            const uint8_t* buf, int c, int g,
                                            float4_t (&acc)[4][MB]) {
  half2_t wsc[4][2];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    wsc[jb][0] = scale_pair_x2m8<false>(wsd[jb]);
    wsc[jb][1] = scale_pair_x2m8<true>(wsd[jb]);
  }
  const uint8_t* rbase = buf + c * kMPitch + 128 * g;
  // Step t + 1's activation reads are issued before step t's MFMAs; the
  // scheduling fence after each step keeps the compiler from hoisting every
  // read of the stage at once (which would not fit the registers).
  half8_t af[2][LIVE];
  auto read_af = [&](half8_t (&dst)[LIVE], int t) {
#pragma unroll
    for (int ib = 0; ib < LIVE; ++ib)
      dst[ib] = *reinterpret_cast<const half8_t*>(rbase + 16 * ib * kMPitch + 16 * t);
  };
  read_af(af[0], 0);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (t < 7) read_af(af[(t + 1) & 1], t + 1);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const half8_t wf = dequant8(s.w[jb][t >> 2][t & 3], wsc[jb][t >> 2][(t >> 1) & 1]);
#pragma unroll
      for (int ib = 0; ib < LIVE; ++ib)
        acc[jb][ib] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf, af[t & 1][ib], acc[jb][ib], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Where a thread and its wave sit (fixed for the kernel).
struct MidThread {
  int tid, lane, wave, c, g;
  int ar, ag, ah;   // activation loader: row, lane group, half of the group's run
  bool loader;
  uint8_t* stages;  // the two activation stages (the epilogue tile reuses them)
  uint8_t* sl;      // this wave's scale copies
};

// The K loop of one item with LIVE row blocks and a ring of R register
// stages: stage st reads its weight scales, computes from ring slot st % R
// and LDS buffer st % 2, then writes stage st+1's activations (loaded R-1
// stages earlier) into the other buffer, reloads its slot with stage st+R and
// meets the workgroup at the barrier, so R-1 stages of loads stay in flight
// while one computes.  The caller has issued stages 0 .. R-1 and filled
// buffer 0.  Unrolled by a multiple of R and 2, so every slot, buffer and
// granule half is a constant.  Every stage of the unrolled group runs, also
// past the last one (K / 256 not a multiple of the group): its loads are out
// of range, so its weights are zeros and its MFMAs add exact zeros to the
// accumulators (which start at +0 and so never hold -0).  A guard around the
// stages instead would make the compiler's count of loads in flight a lower
// bound on every path, and its waits drained the ring.
template <int MB, int LIVE, bool PK, int R>
__device__ __forceinline__ void mid_k_loop(float4_t (&acc)[4][MB], MidStage (&ring)[R],
                                           const MidLoads& l, const rsrc_t& a_rs,
                                           const rsrc_t& as_rs, const MidThread& th, int32_t nst,
                                           int32_t nbk) {
  constexpr int U = R % 2 == 0 ? R : 2 * R;
  uint8_t* const buf[2] = {th.stages, th.stages + mid_stage_bytes<MB>()};
  for (int32_t st0 = 0; st0 < nst; st0 += U) {
    static_for<U>([&](auto dd) {
      constexpr int D = decltype(dd)::value;
      const int32_t st = st0 + D;
      {
        uint32_t wsd[4];
        // The stage's scale copy was issued before its activation loads.
        mid_read_scales(wsd, th.sl + ((st >> 2) & 1) * kMScaleBuf, th.c, th.g, (st >> 1) & 1, D & 1,
                        ring[D % R].as);
        mid_compute<MB, LIVE>(ring[D % R], wsd, buf[D & 1], th.c, th.g, acc);
        if (th.loader && st + 1 < nst)
          mid_put_act(buf[(D + 1) & 1], th.ar, th.ag, th.ah, ring[(D + 1) % R]);
        const int32_t nxt = st + R;  // st0 is even: nxt's granule half is (D + R) % 2
        mid_issue<PK, (D + R) & 1>(ring[D % R], l, a_rs, as_rs, nxt, nxt >= nst, th.sl, nbk);
        mid_barrier();
      }
    });
  }
}

// BF16 epilogue of an item through LDS (`tile`: 16 MB rows of 1 KB over the two
// activation stages, free after the K loop's last barrier).  Lane (c, g) of wave wv holds, for row 16 ib +
// c, columns 64 wv + 16 jb + 4 g .. +3; those 8 bytes go to 16-byte chunk
// 8 wv + 2 jb + g / 2 of the row (position chunk ^ (row % 32)).  The
// workgroup then stores 16-byte chunks of whole rows.  Rows past the expert's
// end fall outside the store resource; chunks past n get an out-of-range
// offset.  Ends with a barrier (the next item rewrites `tile`).
template <int MB>
__device__ __forceinline__ void mid_store(float4_t (&acc)[4][MB], const ItemPos& it,
                                          const GemmArgs& p, uint8_t* tile, const MidThread& th) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  constexpr int kTileRow = 2 * kMCols;
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
#pragma unroll
    for (int ib = 0; ib < MB; ++ib) {
      const float4_t v = acc[jb][ib];
      const bf16x4_t b = {(__bf16)(v[0] * it.alpha), (__bf16)(v[1] * it.alpha),
                          (__bf16)(v[2] * it.alpha), (__bf16)(v[3] * it.alpha)};
      const int row = 16 * ib + th.c, chunk = 8 * th.wave + 2 * jb + (th.g >> 1);
      *reinterpret_cast<u32x2_t*>(tile + row * kTileRow + 16 * (chunk ^ (row & 31)) + 8 * (th.g & 1)) =
          __builtin_bit_cast(u32x2_t, b);
    }
  }
  __syncthreads();
  // The host picks this kernel only when 48 rows of ldo BF16 values stay below
  // 2^31 - 4096 bytes, so the resource size and every offset fit 31 bits.
  const uint32_t ldo = (uint32_t)p.ldo;
  const rsrc_t o = make_rsrc(p.out + (int64_t)it.row0 * ldo, (uint32_t)it.rows_valid * ldo * 2u);
  constexpr int kChunks = kTileRow / 16, kPass = kMThreads / kChunks;
  const int chunk = th.tid % kChunks, r0 = th.tid / kChunks;  // kPass rows per pass
  const bool col_ok = it.n0 + 8 * chunk < (int32_t)p.n;
#pragma unroll
  for (int i = 0; i < 16 * MB / kPass; ++i) {
    const int row = r0 + kPass * i;
    const u32x4_t d = *reinterpret_cast<const u32x4_t*>(tile + row * kTileRow + 16 * (chunk ^ (row & 31)));
    const uint32_t off = col_ok ? ((uint32_t)row * ldo + (uint32_t)(it.n0 + 8 * chunk)) * 2u : kOutOfRange;
    __builtin_amdgcn_raw_buffer_store_b128(d, o, off, 0, 0);
  }
  __syncthreads();
}

// One item with LIVE row blocks: lane offsets, the first R stages, the K loop
// and the epilogue.  Instantiated per LIVE, with every register the item
// needs declared inside, so the branches of the caller share none.
template <int MB, int LIVE, bool PK, int R>
__device__ __forceinline__ void mid_item(const GemmArgs& p, const ItemPos& it, const MidThread& th,
                                         const rsrc_t& a_rs, const rsrc_t& as_rs) {
  // 32-bit offsets: the host guarantees n * k/2 and a_rows * k/2 < 2^31.
  const int32_t n = (int32_t)p.n, kb = (int32_t)(p.k >> 1), nbk = (int32_t)(p.k >> 4);
  const int32_t nst = (int32_t)(p.k / kMK);  // even: K is a multiple of 512
  const int32_t a_last = (int32_t)p.a_rows - 1;
  MidLoads l;
  l.w = make_rsrc(p.w_q + (int64_t)it.e * n * kb, (uint32_t)(n * kb));
  l.ws = make_rsrc(p.w_sf + (int64_t)it.e * n * nbk, (uint32_t)(n * nbk));
  const int32_t grp0 = uniform(it.n0 + 64 * th.wave);  // this wave's 64 weight rows
  {
    const int32_t left = grp0 < n ? (n - grp0) >> 4 : 0;
    l.wk = uniform((left < 4 ? left : 4) * packed_block_bytes(kMGranule));
  }
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    const int32_t row = grp0 + 16 * jb + th.c;
    const uint32_t wv = PK ? (uint32_t)(grp0 * kb + jb * packed_block_bytes(kMGranule) + 16 * th.lane)
                           : (uint32_t)(row * kb + (kMGranule / 8) * th.g);
    l.wq[jb] = row < n ? wv : kOutOfRange;
  }
  {
    // Block jb's copy adds 16 jb rows to this offset; a block lies wholly
    // inside n or wholly past it (n % 16 == 0), and past n its copy reads
    // nothing: the offset then stays at or above the resource's size.
    const int32_t row = grp0 + th.c;
    l.sl = row < n ? (uint32_t)(row * nbk + 16 * th.g) : kOutOfRange;
  }
  {
    // Rows past the expert's end load nothing (zeros): their products are
    // computed in a partly live row block and never stored.
    const bool a_ok = th.loader && th.ar < it.rows_valid;
    int32_t src = it.row0 + (a_ok ? th.ar : 0);
    if (p.a_row_index) src = p.a_row_index[src];
    src = src < 0 ? 0 : (src > a_last ? a_last : src);
    l.aq = a_ok ? (uint32_t)(src * kb + (kMGranule / 8) * th.ag + 16 * th.ah) : kOutOfRange;
    l.asc = a_ok ? (uint32_t)(src * nbk + (kMGranule / 64) * th.ag) : kOutOfRange;
  }

  float4_t acc[4][MB];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
#pragma unroll
    for (int ib = 0; ib < MB; ++ib) acc[jb][ib] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  MidStage ring[R];
  static_for<R>([&](auto dd) {
    constexpr int D = decltype(dd)::value;
    mid_issue<PK, D & 1>(ring[D], l, a_rs, as_rs, D, D >= nst, th.sl, nbk);
  });
  if (th.loader) mid_put_act(th.stages, th.ar, th.ag, th.ah, ring[0]);
  mid_barrier();
  mid_k_loop<MB, LIVE, PK, R>(acc, ring, l, a_rs, as_rs, th, nst, nbk);
  mid_store<MB>(acc, it, p, th.stages, th);
}

template <int MB, int R, bool PK>
__global__ __launch_bounds__(kMThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_grouped_gemm_mid(const GemmArgs p) {
  constexpr int BM = 16 * MB;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int32_t* prefix = reinterpret_cast<int32_t*>(smem);
  int32_t* offl = prefix + (p.num_experts + 1);
  __shared__ int32_t wave_sum[kMWaves];

  MidThread th;
  th.tid = threadIdx.x;
  th.lane = th.tid & 63;
  th.wave = uniform(th.tid >> 6);
  th.c = th.lane & 15;
  th.g = th.lane >> 4;
  // Activation loader role: thread (ar, part) converts row ar, half part % 2
  // of lane group part / 2's run; 16 consecutive lanes take 16 consecutive
  // rows of one half run.
  th.ar = th.tid % BM;
  const int part = th.tid / BM;
  th.ag = (part >> 1) & 3;
  th.ah = part & 1;
  th.loader = th.tid < 8 * BM;
  th.stages = smem + worklist_bytes(p.num_experts);
  // The scale copies get an LDS array of their own: the compiler then knows
  // that the activation stages' reads and writes cannot touch what a copy in
  // flight writes, and does not wait for the copies before them.
  __shared__ __attribute__((aligned(16))) uint8_t sl_area[kMWaves * kMScaleWave];
  th.sl = sl_area + (size_t)th.wave * kMScaleWave;

  const int32_t total_items = build_worklist<kMThreads>(p, BM, prefix, offl, wave_sum);
  const WorkList wl{prefix, offl};

  const int nblk = gridDim.x, b = blockIdx.x;
  const int32_t rounds = (total_items + nblk - 1) / nblk;
  if (rounds == 0) return;
  const int32_t last_items = total_items - (rounds - 1) * nblk;
  const int32_t lb_full = logical_block(b, nblk, nblk);
  const int32_t lb_last = logical_block(b, nblk, last_items);
  const int32_t my_items = (rounds - 1) + (lb_last < last_items ? 1 : 0);

  const rsrc_t a_rs = make_rsrc(p.a_q, (uint32_t)(p.a_rows * (p.k >> 1)));
  const rsrc_t as_rs = make_rsrc(p.a_sf, (uint32_t)(p.a_rows * (p.k >> 4)));

  int32_t from = 0;
  for (int32_t j = 0; j < my_items; ++j) {
    const int32_t item = j * nblk + (j == rounds - 1 ? lb_last : lb_full);
    const ItemPos it = locate(item, from, wl, p, BM, kMCols, th.lane);
    from = it.e;
    const int live = (it.rows_valid + 15) >> 4;
    if (live <= 1) {
      mid_item<MB, 1, PK, R>(p, it, th, a_rs, as_rs);
    } else if (live == 2 && MB > 2) {
      if constexpr (MB > 2) mid_item<MB, 2, PK, R>(p, it, th, a_rs, as_rs);
    } else if (live == 3 && MB > 3) {
      if constexpr (MB > 3) mid_item<MB, 3, PK, R>(p, it, th, a_rs, as_rs);
    } else {
      mid_item<MB, MB, PK, R>(p, it, th, a_rs, as_rs);
    }
  }
}

// 48-row items with three register stages (two in flight while one
// computes): the in-flight bytes, not the arithmetic, bound this kernel.
constexpr int kMidBlocks = 3;
constexpr int kMidRing = 3;
static_assert(8 * 16 * kMidBlocks <= kMThreads, "one activation loader per row and half run");
static_assert(2 * mid_stage_bytes<kMidBlocks>() >= (size_t)16 * kMidBlocks * 2 * kMCols,
              "the epilogue tile fits the two activation stages");

}  // namespace

// Dynamic plus static LDS of a workgroup.
size_t mid_lds(int32_t num_experts) {
  return mid_lds_bytes<kMidBlocks>(num_experts) + (size_t)kMWaves * kMScaleWave;
}

hipError_t launch_grouped_gemm_mid(const GemmArgs& args, hipStream_t stream) {
  if (args.k % kMGranule != 0) return hipErrorInvalidValue;
  GemmArgs p = args;
  p.n_tiles = (int32_t)((p.n + kMCols - 1) / kMCols);
  auto kern = p.w_packed ? k_grouped_gemm_mid<kMidBlocks, kMidRing, true>
                         : k_grouped_gemm_mid<kMidBlocks, kMidRing, false>;
  const size_t lds = mid_lds_bytes<kMidBlocks>(p.num_experts);
  if (mid_lds(p.num_experts) > kLdsBytes) return hipErrorInvalidValue;  // the host picks this tile only if it fits
  int resident = 0;
  hipError_t err = resident_groups(kern, kMThreads, lds, &resident);
  if (err != hipSuccess) return err;
  // Upper bound on the number of items: the host does not see the offsets.
  constexpr int BM = 16 * kMidBlocks;
  const int64_t max_mtiles = p.m_total / BM + (p.m_total < p.num_experts ? p.m_total : p.num_experts);
  const int64_t max_items = max_mtiles * p.n_tiles;
  int64_t grid = resident;
  if (max_items < grid) grid = max_items;
  if (grid < 1) grid = 1;
  grid = (grid + kXcds - 1) / kXcds * kXcds;  // whole rounds over the XCDs
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kMThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace moe_fp4
