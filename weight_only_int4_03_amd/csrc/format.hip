// Format kernels: quantize+pack, repack/unrepack, dequantize.
//
// Quantize+pack and dequantize follow the page "GPU Kernels for INT4
// Inference, in depth" (aicassindra.com), section "The data contract"
// (quantize_pack and dequantize); the repacked layout is described in
// common.h.
#include "common.h"

namespace w4a16 {

// ---------------------------------------------------------------------------
// Quantize + pack.  One thread per (group g, column n): adjacent threads take
// adjacent columns, so every row access of W and of the packed output is a
// coalesced run.  The scale is an IEEE fp32 division, the rounding of W/s is
// round-half-to-even (v_rndne_f32), and fp16(s) is the round-to-nearest-even
// conversion -- the same decisions, in the same precision, as the definition.
// With a gain vector (FuTransformer, arXiv 2610.23796, section 3.2.2: the
// frozen RMSNorm gain folded into the next projection), the matrix quantized
// is W'[k,n] = fp32(gamma[k] * W[k,n]).
__global__ __launch_bounds__(256) void pack_kernel(const float *__restrict__ W,
                                                   const float *__restrict__ gamma, int64_t N,
                                                   int G, int32_t *__restrict__ packed,
                                                   uint16_t *__restrict__ scales) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t g = blockIdx.y;
  if (n >= N) return;
  const float *colw = W + g * G * N + n;
  const float *gam = gamma != nullptr ? gamma + g * G : nullptr;
  auto col = [&](int k) { return gam != nullptr ? __fmul_rn(gam[k], colw[k * N]) : colw[k * N]; };
  float amax = 0.0f;
#pragma unroll 16
  for (int k = 0; k < G; ++k) amax = fmaxf(amax, fabsf(col(k)));
  float s = __fdiv_rn(amax, 7.0f);
  s = s < 1e-8f ? 1e-8f : s;
#pragma unroll 2
  for (int r = 0; r < G / 8; ++r) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float q = __builtin_rintf(__fdiv_rn(col(8 * r + i), s));
      q = fminf(fmaxf(q, -8.0f), 7.0f);
      word |= (uint32_t)((int)q + 8) << (4 * i);
    }
    packed[(g * (G / 8) + r) * N + n] = (int32_t)word;
  }
  scales[g * N + n] = to_half_bits(s);
}

hipError_t launch_pack(const float *W, const float *gamma, int64_t K, int64_t N, int G,
                       int32_t *packed, uint16_t *scales, hipStream_t s) {
  dim3 grid((unsigned)ceil_div(N, 256), (unsigned)(K / G));
  hipLaunchKernelGGL(pack_kernel, grid, dim3(256), 0, s, W, gamma, N, G, packed, scales);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Repack / unrepack.  Blocks [0, wblocks) move weight words: one thread per
// (strip t, tile q, lane position l) writes the 16-byte lane vector of the
// tile.  The remaining blocks move scales: one thread per (strip, group octet,
// column) writes eight consecutive groups' scales.

__device__ __forceinline__ uint32_t permute_nibbles(uint32_t w) {
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) out |= ((w >> (4 * i)) & 0xFu) << (4 * nibble_pos(i));
  return out;
}

__device__ __forceinline__ uint32_t unpermute_nibbles(uint32_t w) {
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) out |= ((w >> (4 * nibble_pos(i))) & 0xFu) << (4 * i);
  return out;
}

template <bool FORWARD>
__global__ __launch_bounds__(256) void repack_kernel(const int32_t *__restrict__ packed,
                                                     const uint16_t *__restrict__ scales,
                                                     uint4_t *__restrict__ rw,
                                                     uint16_t *__restrict__ rs,
                                                     int32_t *__restrict__ packed_out,
                                                     uint16_t *__restrict__ scales_out,
                                                     int64_t N, int64_t KT, int64_t KG,
                                                     int64_t KG8, int64_t NS,
                                                     int64_t wblocks) {
  if ((int64_t)blockIdx.x < wblocks) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (t*KT + q)*64 + l
    if (idx >= NS * KT * 64) return;
    const int l = (int)(idx & 63);
    const int64_t tq = idx >> 6;
    const int64_t q = tq % KT, t = tq / KT;
    const int h = l >> 5, c = l & 31;
    const int64_t n = t * kStrip + c;
    const int64_t r0 = 8 * q + 4 * h;
    if (FORWARD) {
      uint4_t v;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = n < N ? permute_nibbles((uint32_t)packed[(r0 + j) * N + n]) : 0x88888888u;
      rw[idx] = v;
    } else {
      if (n >= N) return;
      uint4_t v = rw[idx];
#pragma unroll
      for (int j = 0; j < 4; ++j) packed_out[(r0 + j) * N + n] = (int32_t)unpermute_nibbles(v[j]);
    }
  } else {
    const int64_t idx = ((int64_t)blockIdx.x - wblocks) * 256 + threadIdx.x;  // (t*KG8+o)*32+c
    if (idx >= NS * KG8 * 32) return;
    const int c = (int)(idx & 31);
    const int64_t to = idx >> 5;
    const int64_t o = to % KG8, t = to / KG8;
    const int64_t n = t * kStrip + c;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t g = 8 * o + e;
      if (FORWARD)
        rs[idx * 8 + e] = (g < KG && n < N) ? scales[g * N + n] : (uint16_t)0;
      else if (g < KG && n < N)
        scales_out[g * N + n] = rs[idx * 8 + e];
    }
  }
}

static void repack_geometry(int64_t K, int64_t N, int G, int64_t &KT, int64_t &KG, int64_t &KG8,
                            int64_t &NS) {
  KT = K / kTileK;
  KG = groups_of(K, G);
  KG8 = ceil_div(KG, 8);
  NS = ceil_div(N, kStrip);
}

hipError_t launch_repack(const int32_t *packed, const uint16_t *scales, int64_t K, int64_t N,
                         int G, void *rw, void *rs, hipStream_t s) {
  int64_t KT, KG, KG8, NS;
  repack_geometry(K, N, G, KT, KG, KG8, NS);
  const int64_t wblocks = ceil_div(NS * KT * 64, 256);
  const int64_t sblocks = ceil_div(NS * KG8 * 32, 256);
  hipLaunchKernelGGL(repack_kernel<true>, dim3((unsigned)(wblocks + sblocks)), dim3(256), 0, s,
                     packed, scales, (uint4_t *)rw, (uint16_t *)rs, (int32_t *)nullptr,
                     (uint16_t *)nullptr, N, KT, KG, KG8, NS, wblocks);
  return hipGetLastError();
}

hipError_t launch_unrepack(const void *rw, const void *rs, int64_t K, int64_t N, int G,
                           int32_t *packed, uint16_t *scales, hipStream_t s) {
  int64_t KT, KG, KG8, NS;
  repack_geometry(K, N, G, KT, KG, KG8, NS);
  const int64_t wblocks = ceil_div(NS * KT * 64, 256);
  const int64_t sblocks = ceil_div(NS * KG8 * 32, 256);
  hipLaunchKernelGGL(repack_kernel<false>, dim3((unsigned)(wblocks + sblocks)), dim3(256), 0, s,
                     (const int32_t *)nullptr, (const uint16_t *)nullptr, (uint4_t *)rw,
                     (uint16_t *)rs, packed, scales, N, KT, KG, KG8, NS, wblocks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// INT8 weights.  Quantize + pack: the int4 kernel's steps with 8-bit codes
// (s = max|W| / 127 as an IEEE fp32 division, round half to even, clamp to
// [-128, 127], stored offset by 128), four codes per int32 along K.
__global__ __launch_bounds__(256) void pack8_kernel(const float *__restrict__ W, int64_t N, int G,
                                                    int32_t *__restrict__ packed,
                                                    uint16_t *__restrict__ scales) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t g = blockIdx.y;
  if (n >= N) return;
  const float *col = W + g * G * N + n;
  float amax = 0.0f;
#pragma unroll 16
  for (int k = 0; k < G; ++k) amax = fmaxf(amax, fabsf(col[k * N]));
  float s = __fdiv_rn(amax, 127.0f);
  s = s < 1e-8f ? 1e-8f : s;
#pragma unroll 2
  for (int r = 0; r < G / 4; ++r) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float q = __builtin_rintf(__fdiv_rn(col[(4 * r + i) * N], s));
      q = fminf(fmaxf(q, -128.0f), 127.0f);
      word |= (uint32_t)((int)q + 128) << (8 * i);
    }
    packed[(g * (G / 4) + r) * N + n] = (int32_t)word;
  }
  scales[g * N + n] = to_half_bits(s);
}

hipError_t launch_pack8(const float *W, int64_t K, int64_t N, int G, int32_t *packed,
                        uint16_t *scales, hipStream_t s) {
  dim3 grid((unsigned)ceil_div(N, 256), (unsigned)(K / G));
  hipLaunchKernelGGL(pack8_kernel, grid, dim3(256), 0, s, W, N, G, packed, scales);
  return hipGetLastError();
}

// Bytes (k0, k1, k2, k3) of a canonical word go to byte slots (0, 2, 1, 3):
// swapping the middle two bytes, its own inverse.
__device__ __forceinline__ uint32_t swap_mid_bytes(uint32_t w) {
  return (w & 0xFF0000FFu) | ((w & 0x0000FF00u) << 8) | ((w & 0x00FF0000u) >> 8);
}

// One thread per repacked 16-byte vector (t, q, j, l): canonical rows
// r = 16q + 8h + 4j + i (i = 0..3) of column 32t + c, l = 32h + c.
template <bool FORWARD>
__global__ __launch_bounds__(256) void repack8_kernel(const int32_t *__restrict__ packed,
                                                      uint4_t *__restrict__ rw,
                                                      int32_t *__restrict__ packed_out,
                                                      int64_t N, int64_t KT, int64_t NS) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // ((t*KT + q)*2 + j)*64 + l
  if (idx >= NS * KT * 128) return;
  const int l = (int)(idx & 63);
  const int j = (int)((idx >> 6) & 1);
  const int64_t tq = idx >> 7;
  const int64_t q = tq % KT, t = tq / KT;
  const int h = l >> 5, c = l & 31;
  const int64_t n = t * kStrip + c;
  const int64_t r0 = 16 * q + 8 * h + 4 * j;
  if (FORWARD) {
    uint4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = n < N ? swap_mid_bytes((uint32_t)packed[(r0 + i) * N + n]) : 0x80808080u;
    rw[idx] = v;
  } else {
    if (n >= N) return;
    const uint4_t v = rw[idx];
#pragma unroll
    for (int i = 0; i < 4; ++i) packed_out[(r0 + i) * N + n] = (int32_t)swap_mid_bytes(v[i]);
  }
}

hipError_t launch_repack8(const int32_t *packed, const uint16_t *scales, int64_t K, int64_t N,
                          int G, void *rw, void *rs, hipStream_t s) {
  int64_t KT, KG, KG8, NS;
  repack_geometry(K, N, G, KT, KG, KG8, NS);
  hipLaunchKernelGGL(repack8_kernel<true>, dim3((unsigned)ceil_div(NS * KT * 128, 256)),
                     dim3(256), 0, s, packed, (uint4_t *)rw, (int32_t *)nullptr, N, KT, NS);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // The scales are laid out as for INT4 weights: the scale half of repack_kernel.
  const int64_t sblocks = ceil_div(NS * KG8 * 32, 256);
  hipLaunchKernelGGL(repack_kernel<true>, dim3((unsigned)sblocks), dim3(256), 0, s,
                     (const int32_t *)nullptr, scales, (uint4_t *)nullptr, (uint16_t *)rs,
                     (int32_t *)nullptr, (uint16_t *)nullptr, N, KT, KG, KG8, NS, (int64_t)0);
  return hipGetLastError();
}

hipError_t launch_unrepack8(const void *rw, const void *rs, int64_t K, int64_t N, int G,
                            int32_t *packed, uint16_t *scales, hipStream_t s) {
  int64_t KT, KG, KG8, NS;
  repack_geometry(K, N, G, KT, KG, KG8, NS);
  hipLaunchKernelGGL(repack8_kernel<false>, dim3((unsigned)ceil_div(NS * KT * 128, 256)),
                     dim3(256), 0, s, (const int32_t *)nullptr, (uint4_t *)rw, packed, N, KT, NS);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t sblocks = ceil_div(NS * KG8 * 32, 256);
  hipLaunchKernelGGL(repack_kernel<false>, dim3((unsigned)sblocks), dim3(256), 0, s,
                     (const int32_t *)nullptr, (const uint16_t *)nullptr, (uint4_t *)nullptr,
                     (uint16_t *)rs, (int32_t *)nullptr, scales, N, KT, KG, KG8, NS, (int64_t)0);
  return hipGetLastError();
}

// Dequantize INT8 weights: one thread per lane position (t, q, l), its two
// vectors = 32 consecutive k of one column; weights fp16((u - 128) s) or
// bf16((u - 128) s), each rounded once.  CANONICAL writes W [K, N]; otherwise
// the fragment order of dequant_kernel (the dense tier's operand layout).
template <bool CANONICAL, bool BF>
__global__ __launch_bounds__(256) void dequant8_kernel(const uint4_t *__restrict__ rw,
                                                       const uint16_t *__restrict__ rs,
                                                       uint16_t *__restrict__ W16, int64_t N,
                                                       int64_t KT, int64_t KG8, int64_t NS,
                                                       int gshift) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (t*KT + q)*64 + l
  if (idx >= NS * KT * 64) return;
  const int l = (int)(idx & 63);
  const int64_t tq = idx >> 6;
  const int64_t q = tq % KT, t = tq / KT;
  const int h = l >> 5, c = l & 31;
  const int64_t n = t * kStrip + c;
  const int g = (int)((64 * q + 32 * h) >> gshift);
  const uint16_t s16 = rs[scale_index(t, KG8, c, g)];
  const uint4_t v0 = rw[tq * 128 + l], v1 = rw[tq * 128 + 64 + l];
  const Dequant dq;
  auto run = [&](int jj) {  // k offsets 8 jj .. +7 of the lane's 32
    const uint4_t &v = jj < 2 ? v0 : v1;
    const int w = (jj & 1) * 2;
    return dq.scaled8_bits<BF>(v[w], v[w + 1], s16);
  };
  if (CANONICAL) {
    if (n >= N) return;
    const int64_t k0 = 64 * q + 32 * h;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint4_t w = run(jj);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        W16[(k0 + 8 * jj + i) * N + n] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
    }
  } else {
    uint4_t *out = (uint4_t *)W16 + idx * 4;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) out[jj] = run(jj);
  }
}

template <bool CANONICAL>
static hipError_t launch_dequant8(const void *rw, const void *rs, int64_t K, int64_t N, int G,
                                  bool bf16, uint16_t *W, hipStream_t s) {
  int64_t KT, KG, KG8, NS;
  repack_geometry(K, N, G, KT, KG, KG8, NS);
  const int gshift = group_shift(K, G);
  const dim3 grid((unsigned)ceil_div(NS * KT * 64, 256));
  if (bf16)
    hipLaunchKernelGGL((dequant8_kernel<CANONICAL, true>), grid, dim3(256), 0, s,
                       (const uint4_t *)rw, (const uint16_t *)rs, W, N, KT, KG8, NS, gshift);
  else
    hipLaunchKernelGGL((dequant8_kernel<CANONICAL, false>), grid, dim3(256), 0, s,
                       (const uint4_t *)rw, (const uint16_t *)rs, W, N, KT, KG8, NS, gshift);
  return hipGetLastError();
}

hipError_t launch_dequant8_canonical(const void *rw, const void *rs, int64_t K, int64_t N, int G,
                                     bool bf16, uint16_t *W, hipStream_t s) {
  return launch_dequant8<true>(rw, rs, K, N, G, bf16, W, s);
}

hipError_t launch_dequant8_fragment(const void *rw, const void *rs, int64_t K, int64_t N, int G,
                                    bool bf16, uint16_t *Wf, hipStream_t s) {
  return launch_dequant8<false>(rw, rs, K, N, G, bf16, Wf, s);
}

// ---------------------------------------------------------------------------
// Prescaled zero rows (Swordfish page, blog.alpindale.net, section "The packed
// format": AWQ zero points enter as rows shaped like the scales holding
// (8 - zp) * s).  One thread per (strip, group octet, column), as the scale
// half of repack_kernel, writing z = fp16((8 - zp) s) into the repacked scale
// layout; padding entries are zero.  (8 - zp) s is an integer of at most 9
// bits times an fp16 value, exact in fp32, so the conversion is the one
// rounding.
__global__ __launch_bounds__(256) void zero_rows_kernel(const uint16_t *__restrict__ scales,
                                                        const uint8_t *__restrict__ zeros,
                                                        uint16_t *__restrict__ rz, int64_t N,
                                                        int64_t KG, int64_t KG8, int64_t NS) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (t*KG8+o)*32+c
  if (idx >= NS * KG8 * 32) return;
  const int c = (int)(idx & 31);
  const int64_t to = idx >> 5;
  const int64_t o = to % KG8, t = to / KG8;
  const int64_t n = t * kStrip + c;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t g = 8 * o + e;
    uint16_t z = 0;
    if (g < KG && n < N) {
      const float s = (float)bitcast<_Float16>(scales[g * N + n]);
      z = to_half_bits(__fmul_rn((float)(8 - (int)zeros[g * N + n]), s));
    }
    rz[idx * 8 + e] = z;
  }
}

hipError_t launch_zero_rows(const uint16_t *scales, const uint8_t *zeros, int64_t K, int64_t N,
                            int G, void *rz, hipStream_t s) {
  int64_t KT, KG, KG8, NS;
  repack_geometry(K, N, G, KT, KG, KG8, NS);
  hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)ceil_div(NS * KG8 * 32, 256)), dim3(256),
                     0, s, scales, zeros, (uint16_t *)rz, N, KG, KG8, NS);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dequantize.  One thread per repacked lane vector (four words = 32 weights of
// one column).  Each weight is fp16((q - 8) * s): the fp16 product of the
// exact value q - 8 and the fp16 scale rounds the exact product once.  With
// BF the weights are bf16((q - 8) * s), the exact product rounded once to
// bf16 (the operand the bf16-activation kernels feed their MFMAs).  With
// zero rows rz (null: none) each weight is the single rounding of
// (q - 8) * s + z, as the GEMM kernels compute it.
//
// CANONICAL writes W16 [K, N] row-major (the definition's layout).
// Otherwise the output is fragment-ordered for the dense GEMM: the lane
// vector (t, q, l) expands to four 16-byte runs at uint4 index
// ((t*KT + q)*64 + l)*4 + j, run j holding k = 64q + 32h + 8j .. +7.
template <bool CANONICAL, bool BF>
__global__ __launch_bounds__(256) void dequant_kernel(const uint4_t *__restrict__ rw,
                                                      const uint16_t *__restrict__ rs,
                                                      const uint16_t *__restrict__ rz,
                                                      uint16_t *__restrict__ W16, int64_t N,
                                                      int64_t KT, int64_t KG8, int64_t NS,
                                                      int gshift) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= NS * KT * 64) return;
  const int l = (int)(idx & 63);
  const int64_t tq = idx >> 6;
  const int64_t q = tq % KT, t = tq / KT;
  const int h = l >> 5, c = l & 31;
  const int64_t n = t * kStrip + c;
  const int g = (int)((64 * q + 32 * h) >> gshift);
  const int64_t si = scale_index(t, KG8, c, g);
  const uint16_t s16 = rs[si];
  const uint16_t z16 = rz != nullptr ? rz[si] : (uint16_t)0;
  const _Float16 sh = bitcast<_Float16>(s16), zh = bitcast<_Float16>(z16);
  const half2_t s2 = {sh, sh}, z2 = {zh, zh};
  const Dequant::BScale bs = rz != nullptr ? Dequant::BScale(s16, z16) : Dequant::BScale(s16);
  const uint4_t v = rw[idx];
  const Dequant dq;
  auto word = [&](uint32_t x) {
    if constexpr (BF)
      return bitcast<uint4_t>(dq.scaled_bf16(x, bs));
    else
      return rz != nullptr ? bitcast<uint4_t>(dq.scaled_zp(x, s2, z2))
                           : bitcast<uint4_t>(dq.scaled(x, s2));
  };
  if (CANONICAL) {
    if (n >= N) return;
    const int64_t k0 = 64 * q + 32 * h;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4_t w = word(v[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        W16[(k0 + 8 * j + i) * N + n] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
    }
  } else {
    uint4_t *out = (uint4_t *)W16 + idx * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = word(v[j]);
  }
}

template <bool CANONICAL>
static hipError_t launch_dequant(const void *rw, const void *rs, const void *rz, int64_t K,
                                 int64_t N, int G, bool bf16, uint16_t *W, hipStream_t s) {
  int64_t KT, KG, KG8, NS;
  repack_geometry(K, N, G, KT, KG, KG8, NS);
  const int gshift = group_shift(K, G);
  const dim3 grid((unsigned)ceil_div(NS * KT * 64, 256));
  if (bf16)
    hipLaunchKernelGGL((dequant_kernel<CANONICAL, true>), grid, dim3(256), 0, s,
                       (const uint4_t *)rw, (const uint16_t *)rs, (const uint16_t *)rz, W, N, KT,
                       KG8, NS, gshift);
  else
    hipLaunchKernelGGL((dequant_kernel<CANONICAL, false>), grid, dim3(256), 0, s,
                       (const uint4_t *)rw, (const uint16_t *)rs, (const uint16_t *)rz, W, N, KT,
                       KG8, NS, gshift);
  return hipGetLastError();
}

hipError_t launch_dequant_canonical(const void *rw, const void *rs, const void *rz, int64_t K,
                                    int64_t N, int G, bool bf16, uint16_t *W, hipStream_t s) {
  return launch_dequant<true>(rw, rs, rz, K, N, G, bf16, W, s);
}

hipError_t launch_dequant_fragment(const void *rw, const void *rs, const void *rz, int64_t K,
                                   int64_t N, int G, bool bf16, uint16_t *Wf, hipStream_t s) {
  return launch_dequant<false>(rw, rs, rz, K, N, G, bf16, Wf, s);
}

}  // namespace w4a16
