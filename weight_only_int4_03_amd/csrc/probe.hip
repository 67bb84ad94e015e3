// Measurement probes: the GPU's own streaming-read and MFMA ceilings.
//
// The Swordfish page (blog.alpindale.net, section "Decode, counting
// memory-pipe slots") rates decode kernels against the platform's practical
// DRAM ceiling; these kernels measure that ceiling and the dense fp16 MFMA
// rate on the machine at hand, so that the GEMMs can be rated against both
// the data-sheet peaks and what the chip sustains.
#include "common.h"

namespace w4a16 {

constexpr uint32_t kProbeTag = 0x9e3779b9u;

// Streaming read: each wave owns a contiguous chunk (16 KiB; 4 KiB for
// buffers under 256 MiB, so that small reads still spread over many more
// waves than the CUs hold) and walks it in 1 KiB wave-wide rows, four
// 128-bit non-temporal loads in flight per lane, folding everything into a
// running XOR.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4_t *buf, int64_t n16,
                                                          int chunk, uint32_t *sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  const int64_t begin = wave * chunk;
  const int64_t end = begin + chunk < n16 ? begin + chunk : n16;
  uint4_t x = {0u, 0u, 0u, 0u};
  if (end - begin == chunk) {
#pragma unroll 1
    for (int64_t o = begin + lane; o < end; o += 256) {
      const uint4_t a = load_nt(buf + o), b = load_nt(buf + o + 64);
      const uint4_t c = load_nt(buf + o + 128), d = load_nt(buf + o + 192);
      x ^= a ^ b ^ c ^ d;
    }
  } else {
    for (int64_t o = begin + lane; o < end; o += 64) x ^= load_nt(buf + o);
  }
  const uint32_t r = x[0] ^ x[1] ^ x[2] ^ x[3];
  if (r == kProbeTag) sink[0] = r;
}

// Four independent accumulator chains of v_mfma_f32_32x32x16_f16 per wave.
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iterations, float *sink) {
  const int lane = threadIdx.x & 63;
  const _Float16 a0 = (_Float16)(lane * 0.001f), b0 = (_Float16)(1.0f - lane * 0.0005f);
  const half8_t a = {a0, a0, a0, a0, a0, a0, a0, a0};
  const half8_t b = {b0, b0, b0, b0, b0, b0, b0, b0};
  float16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iterations; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  if (__builtin_bit_cast(uint32_t, s) == kProbeTag) sink[0] = s;
}

hipError_t launch_stream_read(const void *buf, int64_t bytes, void *sink, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int chunk = bytes >= ((int64_t)256 << 20) ? 1024 : 256;  // 16-byte words per wave
  const int64_t blocks = ceil_div(ceil_div(n16, (int64_t)chunk), (int64_t)4);
  if (blocks > ((int64_t)1 << 31) - 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     (const uint4_t *)buf, n16, chunk, (uint32_t *)sink);
  return hipGetLastError();
}

hipError_t launch_mfma_peak(int iterations, int64_t workgroups, void *sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)workgroups), dim3(256), 0, s, iterations,
                     (float *)sink);
  return hipGetLastError();
}

}  // namespace w4a16
