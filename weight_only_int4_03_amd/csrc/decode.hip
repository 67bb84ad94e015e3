// Decode path (small M): a weight-streaming W4A16 GEMM.
//
// What it computes is the page "GPU Kernels for INT4 Inference, in depth"
// (aicassindra.com), section "The job, stated precisely": C = A * dequant(W),
// FP32 accumulation.  The page's section "What this simple kernel leaves on
// the table" names the decode problems this kernel answers: too few programs
// at M = 1 (hence split-K, reduced afterwards), dequantization in the loop,
// and a layout not tuned for the hardware (hence the repacked layout).  The
// scale is applied after each group's accumulation, as FuTransformer
// (arXiv 2610.23796) section 3.3.4 does.
//
// Mapping on gfx950 (wave64, MFMA):
//   * M <= 16: v_mfma_f32_16x16x32_f16, activation rows padded to 16;
//     M <= 32: v_mfma_f32_32x32x16_f16, rows padded to 32.  MFMA is far from
//     the bound here; it replaces ~8 VALU MACs per weight with one issue slot.
//   * A workgroup owns SPW column strips (32 columns each; for SwiGLU the
//     gate strips and the matching up strips) and a slice of K.  Its WAVES
//     waves split that slice by whole groups of 128; every packed word is read
//     exactly once, with 16-byte non-temporal loads (each wave-wide load is a
//     contiguous 1 KiB tile), D groups ahead of use.
//   * Nibbles become fp16 (u - 8) in registers (shift, and-or with the 0x6400
//     exponent, one packed subtract).  Each group of 128 k accumulates into a
//     zeroed MFMA tile; the tile times the column's fp16 scale is then added
//     to the FP32 accumulator (one FMA per accumulator per group).
//   * Waves reduce through LDS.  With KS > 1 workgroups on one strip group,
//     each writes its partial tile to the workspace; the last one to arrive
//     (agent-scope counter) sums the KS partials in split order and runs the
//     epilogue, then resets the counter.  The order is fixed, so results are
//     bit-identical from run to run.
#include <type_traits>

#include "common.h"

namespace w4a16 {

struct DecodeArgs {
  const uint16_t *A;
  int M, K;
  const uint4_t *rw;
  const uint16_t *rs;
  int N, NS, KT, KG, KG8;
  uint16_t *out;
  int ldo;
  int KS;            // workgroups per strip group (K splits)
  int nsg;           // strip groups
  int up_off;        // SwiGLU: strip offset from a gate strip to its up strip
  int valid_strips;  // plain: NS; SwiGLU: number of gate strips
  float *ws;
  unsigned *counters;
};

template <int MT, int SPW, int D>
struct DecodeFrag {
  static constexpr int NB = 2;               // 16-byte weight vectors per strip per group
  static constexpr int NA = MT == 16 ? 4 : 8;  // 16-byte activation vectors per group
  uint4_t b[SPW][NB];
  uint4_t a[NA];
  uint16_t sc[SPW][MT == 16 ? 2 : 1];
};

template <int MT, int SPW, int WAVES, int D, bool SWIGLU>
__global__ __launch_bounds__(WAVES * 64) void decode_kernel(DecodeArgs p) {
  extern __shared__ float lds[];  // [WAVES][SPW][M][32]
  __shared__ int last_flag;
  constexpr int SH = SWIGLU ? SPW / 2 : SPW;
  constexpr int NPART = MT == 16 ? 2 : 1;  // 16-column halves (MT=16) or whole strip
  typedef typename std::conditional<MT == 16, float4_t, float16_t>::type acc_t;
  typedef DecodeFrag<MT, SPW, D> Frag;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sg = blockIdx.x % p.nsg, split = blockIdx.x / p.nsg;
  const int M = p.M;

  int strip[SPW];
  bool sval[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int base = sg * SH + (s % SH);
    strip[s] = SWIGLU && s >= SH ? base + p.up_off : base;
    sval[s] = base < p.valid_strips;
  }

  const int unit = split * WAVES + wave, nunits = p.KS * WAVES;
  const int g0 = (int)((int64_t)p.KG * unit / nunits);
  const int g1 = (int)((int64_t)p.KG * (unit + 1) / nunits);

  // Lane roles.  MT=16: lane = 16*g4 + c16; row of A = c16; lane group g4
  // covers k offsets 32*g4 .. +31 of the group.  MT=32: lane = 32*h + c;
  // row of A = c; lane half h covers k offsets 64x + 32h .. +31 of X-tile x.
  const int mrow = MT == 16 ? (lane & 15) : (lane & 31);
  const bool arow = mrow < M;
  const uint4_t *Arow = (const uint4_t *)(p.A + (int64_t)(arow ? mrow : 0) * p.K);
  const int g4 = lane >> 4, c16 = lane & 15;
  const int h = lane >> 5, c32 = lane & 31;

  auto load = [&](Frag &f, int g) {
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const uint4_t *tile = p.rw + ((int64_t)strip[s] * p.KT + 2 * g) * 64;
      if constexpr (MT == 16) {
#pragma unroll
        for (int part = 0; part < 2; ++part)
          f.b[s][part] = sval[s] ? load_nt(tile + (g4 >> 1) * 64 + (g4 & 1) * 32 + 16 * part + c16)
                                 : uint4_t{0, 0, 0, 0};
      } else {
#pragma unroll
        for (int x = 0; x < 2; ++x)
          f.b[s][x] = sval[s] ? load_nt(tile + x * 64 + lane) : uint4_t{0, 0, 0, 0};
      }
      const uint16_t *sp = p.rs + (((int64_t)strip[s] * p.KG8 + (g >> 3)) * 32) * 8 + (g & 7);
#pragma unroll
      for (int part = 0; part < NPART; ++part)
        f.sc[s][part] = sval[s] ? sp[(MT == 16 ? 16 * part + c16 : c32) * 8] : (uint16_t)0;
    }
    if constexpr (MT == 16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) f.a[j] = arow ? Arow[16 * g + 4 * g4 + j] : uint4_t{0, 0, 0, 0};
    } else {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          f.a[4 * x + j] = arow ? Arow[16 * g + 8 * x + 4 * h + j] : uint4_t{0, 0, 0, 0};
    }
  };

  acc_t acc[SPW][NPART];
#pragma unroll
  for (int s = 0; s < SPW; ++s)
#pragma unroll
    for (int part = 0; part < NPART; ++part) acc[s][part] = acc_t{};

  auto compute = [&](const Frag &f) {
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
#pragma unroll
      for (int part = 0; part < NPART; ++part) {
        acc_t t = acc_t{};
        if constexpr (MT == 16) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            t = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(f.a[j]),
                                                       nibbles_to_half8(f.b[s][part][j]), t, 0, 0,
                                                       0);
        } else {
#pragma unroll
          for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              t = __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<half8_t>(f.a[4 * x + j]),
                                                         nibbles_to_half8(f.b[s][x][j]), t, 0, 0,
                                                         0);
        }
        const float sc = (float)bitcast<_Float16>(f.sc[s][part]);
        acc[s][part] += t * sc;
      }
    }
  };

  // D-deep register pipeline over this wave's groups [g0, g1).
  Frag f[D];
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (g0 + d < g1) load(f[d], g0 + d);
  for (int g = g0; g < g1; g += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (g + d < g1) {
        compute(f[d]);
        if (g + d + D < g1) load(f[d], g + d + D);
      }
    }
  }

  // Cross-wave reduction through LDS: lds[((wave*SPW + s)*M + m)*32 + col].
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
#pragma unroll
    for (int part = 0; part < NPART; ++part) {
#pragma unroll
      for (int r = 0; r < (MT == 16 ? 4 : 16); ++r) {
        const int m = MT == 16 ? 4 * g4 + r : 8 * (r >> 2) + 4 * h + (r & 3);
        const int col = MT == 16 ? 16 * part + c16 : c32;
        if (m < M) lds[((wave * SPW + s) * M + m) * 32 + col] = acc[s][part][r];
      }
    }
  }
  __syncthreads();

  const int tileE = SPW * M * 32;
  const int nthreads = WAVES * 64;
  auto wave_sum = [&](int e) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += lds[w * tileE + e];
    return v;
  };
  auto epilogue = [&](auto value_at) {
    if constexpr (SWIGLU) {
      for (int e = threadIdx.x; e < SH * M * 32; e += nthreads) {
        const int s = e / (M * 32), rem = e - s * M * 32;
        const int m = rem >> 5, c = rem & 31;
        const int gstrip = sg * SH + s;
        if (gstrip < p.valid_strips) {
          const float gv = value_at(e), uv = value_at(e + SH * M * 32);
          p.out[(int64_t)m * p.ldo + gstrip * 32 + c] = to_half_bits(silu_mul(gv, uv));
        }
      }
    } else {
      for (int e = threadIdx.x; e < tileE; e += nthreads) {
        const int s = e / (M * 32), rem = e - s * M * 32;
        const int m = rem >> 5, c = rem & 31;
        const int col = (sg * SPW + s) * 32 + c;
        if (col < p.N) p.out[(int64_t)m * p.ldo + col] = to_half_bits(value_at(e));
      }
    }
  };

  if (p.KS == 1) {
    epilogue(wave_sum);
    return;
  }

  float *mine = p.ws + ((int64_t)sg * p.KS + split) * tileE;
  for (int e = threadIdx.x; e < tileE; e += nthreads) mine[e] = wave_sum(e);
  __threadfence();  // release this wave's partial stores at agent scope
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(p.counters + sg, 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    const int is_last = prev == (unsigned)(p.KS - 1);
    if (is_last)
      __hip_atomic_store(p.counters + sg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = is_last;
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();  // acquire the other workgroups' partials
  const float *all = p.ws + (int64_t)sg * p.KS * tileE;
  epilogue([&](int e) {
    float v = 0.0f;
    for (int sp = 0; sp < p.KS; ++sp) v += all[(int64_t)sp * tileE + e];
    return v;
  });
}

// ---------------------------------------------------------------------------
// Host side: configuration choice and launch.

struct DecodeConfig {
  int MT, SPW, WAVES, D, KS, nsg;
};

static DecodeConfig decode_config(const Problem &p) {
  DecodeConfig c;
  c.MT = p.M <= 16 ? 16 : 32;
  c.WAVES = 4;
  c.D = 2;
  const int64_t NS = ceil_div(p.N, kStrip);
  const int64_t KG = p.K / kGroup;
  c.SPW = p.swiglu ? 2 : 1;
  c.nsg = (int)(p.swiglu ? (p.N / 2 / kStrip) : ceil_div(NS, c.SPW));
  // Enough workgroups to cover the 256 CUs several times over, but never
  // fewer than one group per wave.
  int64_t ks = ceil_div(1024, c.nsg);
  const int64_t ks_max = KG / c.WAVES > 0 ? KG / c.WAVES : 1;
  if (ks > ks_max) ks = ks_max;
  if (ks < 1) ks = 1;
  if (ks > 64) ks = 64;
  c.KS = (int)ks;
  return c;
}

int64_t decode_workspace_bytes(const Problem &p) {
  const DecodeConfig c = decode_config(p);
  if (c.KS == 1) return 0;
  return (int64_t)c.nsg * c.KS * c.SPW * p.M * 32 * (int64_t)sizeof(float);
}

template <int MT, int SPW, int WAVES, int D, bool SWIGLU>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t s) {
  const size_t lds = (size_t)WAVES * SPW * a.M * 32 * sizeof(float);
  hipLaunchKernelGGL((decode_kernel<MT, SPW, WAVES, D, SWIGLU>), dim3(a.nsg * a.KS),
                     dim3(WAVES * 64), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const Problem &p, void *workspace, hipStream_t s) {
  const DecodeConfig c = decode_config(p);
  DecodeArgs a;
  a.A = p.A;
  a.M = (int)p.M;
  a.K = (int)p.K;
  a.rw = (const uint4_t *)p.rw;
  a.rs = (const uint16_t *)p.rs;
  a.N = (int)p.N;
  a.NS = (int)ceil_div(p.N, kStrip);
  a.KT = (int)(p.K / kTileK);
  a.KG = (int)(p.K / kGroup);
  a.KG8 = (int)ceil_div(a.KG, 8);
  a.out = p.out;
  a.ldo = (int)(p.swiglu ? p.N / 2 : p.N);
  a.KS = c.KS;
  a.nsg = c.nsg;
  a.up_off = (int)(p.N / 2 / kStrip);
  a.valid_strips = p.swiglu ? a.up_off : a.NS;
  a.counters = (unsigned *)workspace;
  a.ws = (float *)((char *)workspace + kCounterBytes);
  if (c.KS > 1 && (workspace == nullptr || c.nsg * 4 > kCounterBytes)) return hipErrorInvalidValue;
  if (c.MT == 16) {
    return p.swiglu ? launch_decode_t<16, 2, 4, 2, true>(a, s) : launch_decode_t<16, 1, 4, 2, false>(a, s);
  }
  return p.swiglu ? launch_decode_t<32, 2, 4, 2, true>(a, s) : launch_decode_t<32, 1, 4, 2, false>(a, s);
}

}  // namespace w4a16
