// Pieces shared by the grouped-GEMM kernels for gfx950: buffer resources, the
// device-side work list over (expert, M-tile, N-tile) items, XCD-aware
// workgroup numbering, and the host's occupancy cache.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace moe_fp4 {

constexpr int kXcds = 8;
// Word 3 of a raw buffer resource on gfx9-class GPUs: 32-bit data format,
// no swizzle, range checking on (an access at or past num_records reads 0 and
// a store there is dropped).
constexpr int kRawBufferWord3 = 0x00020000;
// A buffer offset past every resource built here (each covers < 2^31 bytes).
constexpr uint32_t kOutOfRange = 0x80000000u;
// Cache-policy operand of a buffer load on gfx950: bit 1 is the non-temporal
// hint, which lets the caches drop the line first.  The decode and 48-row
// kernels load their weight codes with it: a weight tile streams through once
// (or twice, close together), and without the hint those streams push the
// activation rows, which every N-tile of an expert reads again, out of the
// caches.  Measured on the decode gate+up shard (256 experts x 16 rows, K 6144,
// N 512): 86.4 -> 77.5 us; on the down projection 66 -> 61.5 us; on the Zipf
// experts below 96 rows 278 -> 271 us for the whole GEMM.  The hint on the
// activation loads made the decode shard slower (91.4 us).
constexpr int kLoadStreamOnce = 2;

typedef __amdgpu_buffer_rsrc_t rsrc_t;
// Pointers the compiler reads through the scalar cache (uniform addresses).
typedef const int32_t __attribute__((address_space(4)))* sconst_i32;
typedef const float __attribute__((address_space(4)))* sconst_f32;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRawBufferWord3);
}

__device__ __forceinline__ int32_t uniform(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int32_t clamp_off(int32_t v, int32_t m_total) {
  return v < 0 ? 0 : (v > m_total ? m_total : v);
}

// Logical number of workgroup b in a grid of nblk (a multiple of 8) when only
// the first `active` logical workgroups have work: those are split evenly over
// the 8 XCDs (workgroup b runs on XCD b % 8), consecutive logical numbers on
// one XCD; the rest follow.  A bijection of [0, nblk).
__device__ __forceinline__ int logical_block(int b, int nblk, int active) {
  const int per_xcd = nblk / kXcds;
  int pxa = (active + kXcds - 1) / kXcds;
  pxa = pxa < per_xcd ? pxa : per_xcd;
  const int xcd = b % kXcds, slot = b / kXcds;
  if (slot < pxa) return xcd * pxa + slot;
  return kXcds * pxa + xcd * (per_xcd - pxa) + (slot - pxa);
}

// Bytes of the work-list tables in LDS: the item prefix and the clamped
// offsets, E+1 ints each.
__host__ __device__ constexpr size_t worklist_bytes(int num_experts) {
  return ((size_t)(num_experts + 1) * 8 + 15) / 16 * 16;
}

// Work-list tables in LDS: prefix[e] = items of experts before e (prefix[E] =
// all items) and off[e] = expert offsets clamped into [0, m_total].
struct WorkList {
  const int32_t* prefix;
  const int32_t* off;
};

// Items of an expert with cnt rows in this launch: ceil(cnt / bm) * n_tiles if
// cnt is in the launch's row range, else none (an empty expert, or a
// decreasing offset pair, a violated precondition, owns none either).
__device__ __forceinline__ int32_t expert_items(const GemmArgs& p, int32_t cnt, int32_t bm) {
  const bool take = cnt > 0 && cnt >= p.rows_lo && (p.rows_hi == 0 || cnt < p.rows_hi);
  return take ? ((cnt + bm - 1) / bm) * p.n_tiles : 0;
}

// Fill the work-list tables (all NTHR threads of the workgroup take part; two
// barriers inside).  Returns the total item count.
template <int NTHR>
__device__ __forceinline__ int32_t build_worklist(const GemmArgs& p, int32_t bm, int32_t* prefix,
                                                  int32_t* offl, int32_t* wave_sum) {
  constexpr int WAVES = NTHR / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.num_experts;
  const int32_t m_total = (int32_t)p.m_total;
  const int per = (E + NTHR - 1) / NTHR;
  const int beg = tid * per < E ? tid * per : E;
  const int end = beg + per < E ? beg + per : E;
  int32_t local = 0;
  for (int e = beg; e < end; ++e) {
    const int32_t cnt = clamp_off(p.offsets[e + 1], m_total) - clamp_off(p.offsets[e], m_total);
    local += expert_items(p, cnt, bm);
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
    const int32_t lo = clamp_off(p.offsets[e], m_total), hi = clamp_off(p.offsets[e + 1], m_total);
    offl[e] = lo;
    const int32_t cnt = hi - lo;
    run += expert_items(p, cnt, bm);
  }
  if (tid == NTHR - 1) {
    int32_t total = 0;
    for (int w = 0; w < WAVES; ++w) total += wave_sum[w];
    prefix[E] = total;
    offl[E] = clamp_off(p.offsets[E], m_total);
  }
  __syncthreads();
  return uniform(prefix[E]);
}

// The expert owning item i, searching forward from expert `from` (which owns
// an item <= i): 64 experts per step, one LDS read and a ballot.  prefix is
// non-decreasing, so the experts e with prefix[e] <= i form a prefix of the
// range and their count locates the owner (empty experts are passed over).
__device__ __forceinline__ int32_t find_expert(int32_t i, int32_t from, const WorkList& wl,
                                               int32_t E, int lane) {
  int32_t lo = from;
  for (;;) {
    const int32_t e = lo + 1 + lane;
    const int32_t v = e <= E ? wl.prefix[e] : INT32_MAX;
    const int32_t t = (int32_t)__popcll(__ballot(v <= i));
    if (t < 64) return uniform(lo + t);
    lo += 64;
  }
}

// Where a work item lives; every field is wavefront-uniform.
struct ItemPos {
  int32_t e;
  int32_t rows_valid;  // rows of this M-tile that belong to the expert (1..bm)
  int32_t row0;        // first output row of the M-tile
  int32_t n0;          // first output column of the N-tile
  float alpha;         // a_scale * w_scale[e]
};

// Locate item i (search from expert `from`): LDS reads, plus scalar loads of
// the two tensor scales (consumed only by the item's epilogue).
__device__ __forceinline__ ItemPos locate(int32_t i, int32_t from, const WorkList& wl,
                                          const GemmArgs& p, int32_t bm, int32_t bn, int lane) {
  const int32_t e = find_expert(i, from, wl, p.num_experts, lane);
  const int32_t r_lo = uniform(wl.off[e]);
  const int32_t cnt = uniform(wl.off[e + 1]) - r_lo;
  const int32_t mts = (cnt + bm - 1) / bm;
  const int32_t local = i - uniform(wl.prefix[e]);
  const int32_t nt = local / mts, mt = local - nt * mts;
  ItemPos it;
  it.e = e;
  it.row0 = r_lo + mt * bm;
  const int32_t left = cnt - mt * bm;
  it.rows_valid = left < bm ? left : bm;
  it.n0 = nt * bn;
  it.alpha = ((sconst_f32)p.a_scale)[0] * ((sconst_f32)p.w_scale)[e];
  return it;
}

// Resident workgroups the device can hold for one kernel (host; cached per
// device, kernel and LDS size, since the query costs more host time than a
// small decode GEMM takes on the GPU).
hipError_t resident_groups_of(const void* kern, int threads, size_t lds, int* out);

template <typename K>
hipError_t resident_groups(K kern, int threads, size_t lds, int* out) {
  return resident_groups_of(reinterpret_cast<const void*>(kern), threads, lds, out);
}

}  // namespace moe_fp4
