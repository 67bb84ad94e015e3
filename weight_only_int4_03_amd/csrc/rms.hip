// RMSNorm row factors for a projection whose weights carry the folded gain.
//
// FuTransformer (arXiv 2610.23796), section 3.2.2: with the frozen RMSNorm
// gain gamma folded into the projection weights (W' = gamma * W, done by the
// packer), the GEMM reads the raw activations x and multiplies output row m
// by rho_m = (q_m / H + eps)^(-1/2), q_m = sum_h x_mh^2, H the row length
// (here K).  This kernel computes rho; the GEMM epilogues apply it.
//
// One workgroup per row: each thread sums the squares of a strided slice in
// FP32 (16-byte loads), then a fixed-shape tree through LDS combines the 256
// partial sums, so the result is the same on every run.  rho uses correctly
// rounded division and square root.
#include "common.h"

namespace w4a16 {

template <bool BF>
__global__ __launch_bounds__(256) void rms_rowscale_kernel(const uint16_t *__restrict__ A,
                                                           int64_t K, float eps,
                                                           float *__restrict__ rho) {
  __shared__ float part[256];
  const int64_t m = blockIdx.x;
  const uint4_t *row = (const uint4_t *)(A + m * K);
  const int64_t nvec = K / 8;
  float acc = 0.0f;
  for (int64_t i = threadIdx.x; i < nvec; i += 256) {
    const uint4_t v = row[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float lo, hi;
      if constexpr (BF) {
        lo = bitcast<float>(v[j] << 16);
        hi = bitcast<float>(v[j] & 0xFFFF0000u);
      } else {
        const half2_t h = bitcast<half2_t>(v[j]);
        lo = (float)h[0];
        hi = (float)h[1];
      }
      acc = __builtin_fmaf(lo, lo, acc);
      acc = __builtin_fmaf(hi, hi, acc);
    }
  }
  part[threadIdx.x] = acc;
  __syncthreads();
#pragma unroll
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float mean = __fdiv_rn(part[0], (float)K);
    rho[m] = __fdiv_rn(1.0f, __fsqrt_rn(mean + eps));
  }
}

hipError_t launch_rms_rowscale(const uint16_t *A, int64_t M, int64_t K, float eps, bool bf16,
                               float *rho, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(rms_rowscale_kernel<true>, dim3((unsigned)M), dim3(256), 0, s, A, K, eps,
                       rho);
  else
    hipLaunchKernelGGL(rms_rowscale_kernel<false>, dim3((unsigned)M), dim3(256), 0, s, A, K, eps,
                       rho);
  return hipGetLastError();
}

}  // namespace w4a16
