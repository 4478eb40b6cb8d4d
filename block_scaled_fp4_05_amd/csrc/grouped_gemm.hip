// NVFP4 block-scaled MoE grouped GEMM for gfx950: host-side tile choice and the
// launchers of the plain (BF16 store) kernels.  The kernel itself and its design
// notes are in grouped_gemm_kernel.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

#include "grouped_gemm_kernel.h"

namespace moe_fp4 {

hipError_t resident_groups_of(const void* kern, int threads, size_t lds, int* out) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t>, int> groups;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const auto key = std::make_tuple(dev, kern, lds);
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = groups.find(key);
    if (it != groups.end()) {
      *out = it->second;
      return hipSuccess;
    }
  }
  int cus = 0;
  err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  int per_cu = 0;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, lds);
  if (err != hipSuccess) return err;
  if (per_cu < 1) per_cu = 1;
  std::lock_guard<std::mutex> g(mu);
  groups[key] = cus * per_cu;
  *out = cus * per_cu;
  return hipSuccess;
}

GemmTile choose_tile(int32_t num_experts, int64_t m_total, int64_t n, int64_t k, const char* env) {
  (void)n;
  GemmTile t{1, 4, 4, 1, 0, 0};
  const int64_t avg = num_experts > 0 ? (m_total + num_experts - 1) / num_experts : m_total;
  if (avg > 32) t.m_blocks = 4;
  else if (avg > 16) t.m_blocks = 2;
  // Experts this large are compute-bound: share dequantised operands in LDS.
  // When the work list leaves room for two 64 KB stages, experts with at least
  // kBigRows rows take 256 x 256 items and the rest 48 x 512 items (K a
  // multiple of 512) or per-wave items (two launches over disjoint experts,
  // chosen on the device from the offsets); else every expert takes 128 x 128
  // items.  A single expert takes the large tile in one launch (the second
  // launch of the split would find no expert to run and still cost its few
  // microseconds).  Measured on the Zipf prefill shard (256 experts, 4096
  // tokens top-8): 48 x 512 items for the experts below 96 rows 284-288 us,
  // per-wave items 298-302 us.
  if (avg >= 96) {
    const bool mid = k % 512 == 0 && mid_lds(num_experts) <= kLdsBytes;
    t = big_lds(num_experts) > kLdsBytes ? GemmTile{8, 8, 4, 1, 0, 1}
        : num_experts == 1              ? GemmTile{16, 16, 8, 1, 0, 3}
                                        : GemmTile{16, 16, 8, 1, 0, mid ? 5 : 2};
  }
  if (k % 512 == 0) t.k_sub = 2;
  t.lds_scales = k % kSpan == 0 ? 1 : 0;
  // "256x256!": every expert in 256 x 256 items, however few its rows.
  // "256x256f8" and "256x256f8!": the same with the split-K FP8 inner product.
  if (env && std::strncmp(env, "256x256", 7) == 0 && env[7] != '\0') {
    const char* rest = env + 7;
    const bool f8 = rest[0] == 'f' && rest[1] == '8';
    if (f8) rest += 2;
    const bool all = rest[0] == '!' && rest[1] == '\0';
    if ((all || (f8 && rest[0] == '\0')) && big_lds(num_experts) <= kLdsBytes) {
      t = GemmTile{16, 16, 8, 1, 0, all ? 3 : 2};
      t.f8 = f8 ? 1 : 0;
    }
    if (all || f8) return t;
  }
  // Splits by expert size: "256x256m" (large tile from kBigRows rows, 48 x 512
  // items below), "48x512p" (48 x 512 items from kMidRows rows, per-wave items
  // below), "256x256mp" (all three).
  if (env && k % 512 == 0 && mid_lds(num_experts) <= kLdsBytes && big_lds(num_experts) <= kLdsBytes) {
    if (std::strcmp(env, "256x256m") == 0) return GemmTile{16, 16, 8, 1, 0, 5};
    if (std::strcmp(env, "48x512p") == 0) return GemmTile{3, 32, 8, 2, 0, 6};
    if (std::strcmp(env, "256x256mp") == 0) return GemmTile{16, 16, 8, 1, 0, 7};
  }
  if (env && *env) {
    // "MxN" or "MxNxK", optionally followed by 'r' (weight scales through
    // registers rather than LDS): M rows per item, N columns per wave, K
    // elements per stage.
    int v[3] = {0, 0, 0};
    int nv = 0;
    const char* s = env;
    bool ok = true;
    while (ok && nv < 3) {
      if (*s < '0' || *s > '9') { ok = false; break; }
      while (*s >= '0' && *s <= '9') v[nv] = v[nv] * 10 + (*s++ - '0');
      ++nv;
      if (*s == '\0' || *s == 'r') break;
      if (*s == 'x' || *s == 'X') ++s; else ok = false;
    }
    const bool regs = ok && *s == 'r';
    if (regs) ++s;
    ok = ok && *s == '\0' && nv >= 2;
    if (ok && nv == 2 && v[0] == 128 && v[1] == 128 && !regs) {
      t = GemmTile{8, 8, 4, 1, 0, 1};
      return t;
    }
    if (ok && nv == 2 && v[0] == 48 && v[1] == 512 && !regs) {
      if (k % 512 == 0 && mid_lds(num_experts) <= kLdsBytes) t = GemmTile{3, 32, 8, 2, 0, 4};
      return t;
    }
    if (ok && nv == 2 && v[0] == 256 && v[1] == 256 && !regs) {
      if (big_lds(num_experts) <= kLdsBytes) t = GemmTile{16, 16, 8, 1, 0, 2};
      return t;
    }
    ok = ok && (v[0] == 16 || v[0] == 32 || v[0] == 64) && (v[1] == 32 || v[1] == 64);
    if (nv == 3)
      ok = ok && (v[2] == 256 || (v[2] == 512 && k % 512 == 0) ||
                  (v[2] == 1024 && k % 1024 == 0 && v[1] == 32 && v[0] <= 32));
    if (ok) {
      t.tiled = 0;
      t.lds_scales = k % kSpan == 0 ? 1 : 0;
      t.k_sub = k % 512 == 0 ? 2 : 1;
      t.m_blocks = v[0] / 16;
      t.n_blocks = v[1] / 16;
      if (nv == 3) t.k_sub = v[2] / 256;
      if (regs) t.lds_scales = 0;
    }
  }
  return t;
}

int32_t item_rows(const GemmTile& t) {
  if (t.tiled == 4 || t.tiled == 6) return 48;
  if (t.tiled >= 2) return 256;
  if (t.tiled) return 128;
  return 16 * t.m_blocks;
}

GemmTile fit_output_range(const GemmTile& t, int64_t k, int64_t ldo) {
  if (!t.tiled || (int64_t)item_rows(t) * ldo * 2 <= (int64_t)INT32_MAX - 4096) return t;
  return GemmTile{4, 4, 4, k % 512 == 0 ? 2 : 1, k % kSpan == 0 ? 1 : 0, 0};
}

void log_tile(const char* entry, int32_t num_experts, int64_t m_total, int64_t n, int64_t k,
              int64_t ldo, const GemmTile& t) {
  const char* env = getenv("MOE_FP4_LOG");
  if (!env || !*env || (env[0] == '0' && env[1] == '\0')) return;
  static std::mutex mu;
  static std::string last;
  char line[320];
  const char* kind = t.tiled == 7 ? "256x256 workgroup tile for experts of >= 96 rows, 48x512 "
                                    "workgroup items for 17-95 rows, 16x64 per-wave items below"
                     : t.tiled == 6 ? "48x512 workgroup items for experts of >= 17 rows, 16x64 "
                                      "per-wave items below"
                     : t.tiled == 5 ? "256x256 workgroup tile for experts of >= 96 rows, 48x512 "
                                      "workgroup items for the rest"
                     : t.tiled == 4 ? "48x512 workgroup items for every expert"
                     : t.tiled == 3 ? (t.f8 ? "256x256 workgroup tile (FP8 split-K) for every expert"
                                           : "256x256 workgroup tile for every expert")
                     : t.tiled == 2 ? (t.f8 ? "256x256 workgroup tile (FP8 split-K) for experts of "
                                              ">= 96 rows, 16x64 per-wave items for the rest"
                                            : "256x256 workgroup tile for experts of >= 96 rows, "
                                              "16x64 per-wave items for the rest")
                     : t.tiled == 1 ? "128x128 workgroup tile" : "per-wave items";
  snprintf(line, sizeof line,
           "moe_fp4: %s E=%d m_total=%lld n=%lld k=%lld ldo=%lld: %s (tile %dx%d, k step %d, "
           "weight scales %s)\n",
           entry, (int)num_experts, (long long)m_total, (long long)n, (long long)k, (long long)ldo,
           kind, item_rows(t), t.tiled >= 2 ? 256 : t.tiled ? 128 : 16 * t.n_blocks,
           t.tiled == 4 ? 256 : t.tiled ? 64 : 256 * t.k_sub,
           t.tiled == 4 ? "in registers" : t.tiled ? "in LDS stages" : t.lds_scales ? "via LDS lines" : "in registers");
  std::lock_guard<std::mutex> g(mu);
  if (last == line) return;
  last = line;
  fputs(line, stderr);
}

int64_t gemm_lds_bytes(const GemmTile& t, int32_t num_experts) {
  if (t.tiled == 4 || t.tiled == 6) return (int64_t)mid_lds(num_experts) + 16;
  if (t.tiled >= 2) return (int64_t)big_lds(num_experts) + 16;
  if (t.tiled) return (int64_t)tiled_lds(num_experts) + 16;
  int64_t b = (int64_t)worklist_bytes(num_experts) + (int64_t)sizeof(int32_t) * t.waves;
  if (t.lds_scales) b += (int64_t)t.waves * (2 * 16 * 16 * t.n_blocks * 8 + 1024);
  else if (t.n_blocks == 4) b += (int64_t)t.waves * 16 * t.m_blocks * (32 * t.n_blocks + 16);
  return b;
}

template <int NBW, int KSUB, bool SL, bool PK = false>
hipError_t launch_mb(const GemmArgs& p, int m_blocks, hipStream_t stream) {
  switch (m_blocks) {
    case 1: return launch_tile<1, NBW, KSUB, 4, SL, PK>(p, stream);
    case 2: return launch_tile<2, NBW, KSUB, 4, SL, PK>(p, stream);
    case 4: return launch_tile<4, NBW, KSUB, 4, SL, PK>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

// 1024-element stages: only for tiles whose two register stages still fit.
template <bool SL>
hipError_t launch_mb_k1024(const GemmArgs& p, int m_blocks, hipStream_t stream) {
  switch (m_blocks) {
    case 1: return launch_tile<1, 2, 4, 4, SL>(p, stream);
    case 2: return launch_tile<2, 2, 4, 4, SL>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool SL>
hipError_t launch_sl(const GemmArgs& p, const GemmTile& t, hipStream_t stream) {
  if (p.w_packed) {
    // The packed layout's granule fixes the stage: k_sub = 2 iff k % 512 == 0.
    if (t.n_blocks != 4 || t.k_sub != packed_granule(p.k) / kKStep) return hipErrorInvalidValue;
    return t.k_sub == 2 ? launch_mb<4, 2, SL, true>(p, t.m_blocks, stream)
                        : launch_mb<4, 1, SL, true>(p, t.m_blocks, stream);
  }
  if (t.n_blocks == 4) {
    if (t.k_sub == 4) return hipErrorInvalidValue;
    return t.k_sub == 2 ? launch_mb<4, 2, SL>(p, t.m_blocks, stream)
                        : launch_mb<4, 1, SL>(p, t.m_blocks, stream);
  }
  if (t.n_blocks == 2) {
    if (t.k_sub == 4) return launch_mb_k1024<SL>(p, t.m_blocks, stream);
    return t.k_sub == 2 ? launch_mb<2, 2, SL>(p, t.m_blocks, stream)
                        : launch_mb<2, 1, SL>(p, t.m_blocks, stream);
  }
  return hipErrorInvalidValue;
}

// Per-wave tile for the experts below kBigRows rows when the large tile takes
// the rest: 16-row items, 64 columns, the K step of the packed granule.  One
// row block keeps two waves per SIMD (measured on the Zipf prefill shard:
// 16-row items 12% faster than 32-row items, which run one wave per SIMD).
GemmTile small_expert_tile(int64_t k) {
  return GemmTile{1, 4, 4, k % 512 == 0 ? 2 : 1, k % kSpan == 0 ? 1 : 0, 0};
}

hipError_t launch_grouped_gemm(const GemmArgs& p, const GemmTile& t, hipStream_t stream) {
  if (t.tiled == 4) return launch_grouped_gemm_mid(p, stream);
  if (t.tiled >= 5) {
    // Launches over disjoint expert-size ranges: the large tile from kBigRows
    // rows (5, 7), 48 x 512 items in between, per-wave items below kMidRows (6, 7).
    const bool use_big = t.tiled != 6, use_pw = t.tiled != 5;
    hipError_t err = hipSuccess;
    if (use_big) {
      GemmArgs big = p;
      big.rows_lo = kBigRows;
      big.n_tiles = (int32_t)((p.n + 255) / 256);
      err = launch_grouped_gemm_big(big, false, stream);
      if (err != hipSuccess) return err;
    }
    GemmArgs mid = p;
    mid.rows_lo = use_pw ? kMidRows : 0;
    mid.rows_hi = use_big ? kBigRows : 0;
    err = launch_grouped_gemm_mid(mid, stream);
    if (err != hipSuccess || !use_pw) return err;
    GemmArgs small = p;
    const GemmTile s = small_expert_tile(p.k);
    small.rows_hi = kMidRows;
    small.n_tiles = (int32_t)((p.n + 16 * s.n_blocks - 1) / (16 * s.n_blocks));
    return s.lds_scales ? launch_sl<true>(small, s, stream) : launch_sl<false>(small, s, stream);
  }
  if (t.tiled == 3) return launch_grouped_gemm_big(p, t.f8 != 0, stream);
  if (t.tiled == 2) {
    // Experts with kBigRows rows or more in 256 x 256 items, the rest per wave.
    GemmArgs big = p, small = p;
    big.rows_lo = kBigRows;
    big.n_tiles = (int32_t)((p.n + 255) / 256);
    hipError_t err = launch_grouped_gemm_big(big, t.f8 != 0, stream);
    if (err != hipSuccess) return err;
    const GemmTile s = small_expert_tile(p.k);
    small.rows_hi = kBigRows;
    small.n_tiles = (int32_t)((p.n + 16 * s.n_blocks - 1) / (16 * s.n_blocks));
    return s.lds_scales ? launch_sl<true>(small, s, stream) : launch_sl<false>(small, s, stream);
  }
  if (t.tiled) return launch_grouped_gemm_tiled(p, stream);
  if (t.waves != 4 || p.k % (256 * t.k_sub) != 0) return hipErrorInvalidValue;
  if (t.lds_scales) {
    if (p.k % kSpan != 0) return hipErrorInvalidValue;
    return launch_sl<true>(p, t, stream);
  }
  return launch_sl<false>(p, t, stream);
}

}  // namespace moe_fp4
