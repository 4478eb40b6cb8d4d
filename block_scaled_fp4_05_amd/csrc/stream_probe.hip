// Streaming-read probe for gfx950: a measurement aid for the roofline context of
// the grouped GEMM, not part of the method and not behind the library's C ABI.
// It reads a device buffer with the access pattern of the decode GEMM's weight
// stream and no arithmetic, so that bench.py can report what that pattern
// streams at on this part, with and without the non-temporal load hint.
//
// Each wavefront reads `stages` stages of 16 KB: every load instruction of the
// wavefront covers 1 KB of consecutive bytes (16 bytes per lane), 16 of them
// per stage, with two stages in flight (the decode GEMM's register ring).
//   layout 0 (regions): wavefront w reads its own contiguous region of
//     `per_wave` bytes, stage s at offset 16 KB * s of it, as the decode GEMM
//     streams its 64-row weight group;
//   layout 1 (interleaved): stage s of wavefront w is the 16 KB piece
//     s * waves + w of the buffer, so the wavefronts sweep the buffer together.
// The loaded words are folded with XOR and one word is stored only when the
// fold equals a value the caller's data never produce (the sink stays
// untouched in practice); the store keeps the loads from being removed.
// Every load goes through a buffer resource that covers the caller's buffer,
// so an offset past its end reads zeros instead of faulting.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kLoadsPerStage = 16;  // 1 KB each per wavefront
constexpr uint32_t kStageBytes = 1024u * kLoadsPerStage;
constexpr uint32_t kNeverFolded = 0x9E3779B9u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

template <int NT>
__device__ __forceinline__ void load_stage(u32x4_t (&r)[kLoadsPerStage], __amdgpu_buffer_rsrc_t rs,
                                           uint32_t off) {
#pragma unroll
  for (int i = 0; i < kLoadsPerStage; ++i)
    r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 1024u * i, 0, NT ? 2 : 0);
}

template <int LAYOUT, int NT>
__global__ __launch_bounds__(256) void k_stream_probe(const uint8_t* buf, uint32_t buf_bytes,
                                                      uint32_t per_wave, int stages, int waves,
                                                      uint32_t* sink) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t w = blockIdx.x * 4 + (threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(buf, buf_bytes);
  auto stage_off = [&](int s) -> uint32_t {
    const uint32_t piece = LAYOUT == 0 ? 0u : (uint32_t)s * (uint32_t)waves + w;
    return LAYOUT == 0 ? w * per_wave + kStageBytes * (uint32_t)s + 16u * lane
                       : piece * kStageBytes + 16u * lane;
  };
  u32x4_t ring[2][kLoadsPerStage];
  load_stage<NT>(ring[0], rs, stage_off(0));
  load_stage<NT>(ring[1], rs, stage_off(stages > 1 ? 1 : 0));
  uint32_t fold = 0;
  for (int s = 0; s < stages; s += 2) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
#pragma unroll
      for (int i = 0; i < kLoadsPerStage; ++i)
        fold ^= ring[d][i].x ^ ring[d][i].y ^ ring[d][i].z ^ ring[d][i].w;
      const int nx = s + d + 2;
      load_stage<NT>(ring[d], rs, stage_off(nx < stages ? nx : stages - 1));
    }
  }
  if (fold == kNeverFolded) sink[0] = fold;
}

}  // namespace

// Returns 0 on success, 1 for arguments the probe does not accept, 2 for a
// launch error.  buf: device buffer of buf_bytes (< 2^31) bytes; per_wave: bytes
// of each wavefront's region (layout 0; a multiple of 16 KB is not required);
// stages >= 2 of 16 KB per wavefront; waves a positive multiple of 4; nt 0 or 1;
// sink: one device word; stream: a hipStream_t (0 = the null stream).
extern "C" int moe_fp4_stream_probe(const void* buf, uint64_t buf_bytes, uint64_t per_wave,
                                    int stages, int waves, int layout, int nt, void* sink,
                                    void* stream) {
  if (!buf || !sink || buf_bytes == 0 || buf_bytes >= (1ull << 31) || stages < 2 || waves < 4 ||
      waves % 4 != 0 || (layout != 0 && layout != 1) || (nt != 0 && nt != 1))
    return 1;
  const uint64_t need = layout == 0 ? (uint64_t)waves * per_wave
                                    : (uint64_t)waves * (uint64_t)stages * kStageBytes;
  if (layout == 0 && per_wave < (uint64_t)stages * kStageBytes) return 1;
  if (need > buf_bytes) return 1;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(waves / 4)), block(256);
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  uint32_t* s = static_cast<uint32_t*>(sink);
  const uint32_t bb = (uint32_t)buf_bytes, pw = (uint32_t)per_wave;
  if (layout == 0 && nt == 0)
    hipLaunchKernelGGL((k_stream_probe<0, 0>), grid, block, 0, st, b, bb, pw, stages, waves, s);
  else if (layout == 0)
    hipLaunchKernelGGL((k_stream_probe<0, 1>), grid, block, 0, st, b, bb, pw, stages, waves, s);
  else if (nt == 0)
    hipLaunchKernelGGL((k_stream_probe<1, 0>), grid, block, 0, st, b, bb, pw, stages, waves, s);
  else
    hipLaunchKernelGGL((k_stream_probe<1, 1>), grid, block, 0, st, b, bb, pw, stages, waves, s);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
