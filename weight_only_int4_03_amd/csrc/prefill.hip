// Prefill path (large M) and the dense fallback's GEMM.
//
// The product is the page "GPU Kernels for INT4 Inference, in depth"
// (aicassindra.com), section "The job, stated precisely"; the page's tiled
// kernel (section "A W4A16 kernel in Triton") is the plainest form: a BM x BN
// output tile per program, a K loop that loads an activation tile and the
// packed rows, unpacks, centres and scales in registers, and feeds the matrix
// unit with FP32 accumulation.  Swordfish (blog.alpindale.net, "A single
// layout with three consumers") runs a fused prefill mainloop and a dense tier
// (dequantize once into fp16 scratch, then a dense GEMM) over one prepacked
// tensor; this file provides both mainloops for gfx950.
//
// gfx950 mapping:
//   * 256 threads = 4 waves per workgroup; the workgroup tile is BM x 256
//     (BM = 32 * MI rows; each wave owns all BM rows and 64 columns = two
//     32-column strips).  v_mfma_f32_32x32x16_f16 with the weights as the
//     A operand (32 columns of a strip) and the activations as the B operand
//     (32 rows), so each lane ends with runs of 4 consecutive output columns.
//   * A [BM x 64] tiles go global -> registers -> LDS, double buffered (one
//     barrier per 64-k step), with the 16-byte chunks XOR-swizzled by row so
//     that ds_read_b128 of 32 rows spreads over the banks.
//   * Packed weights are not staged in LDS: each wave alone consumes its two
//     strips, so each lane loads its 16-byte lane vector (4 words = 32 k of
//     one column) straight from global memory one step ahead, and
//     dequantizes it directly into MFMA operand registers (shift / and-or /
//     packed subtract / packed multiply by the fp16 group scale: exactly the
//     fp16 dequantized weight).  No dequantized tile is ever materialised.
//   * DENSE reads instead the fp16 weights that the fallback's dequant kernel
//     wrote in the same fragment order (four 16-byte vectors per lane and step).
//   * Workgroup ids are remapped so that each XCD (ids are dealt round-robin
//     over the 8 XCDs) works on one contiguous range of tiles, walked in
//     groups of 4 row tiles so that concurrently running tiles share weight
//     columns and activation rows in that XCD's L2.
#include <cstdio>
#include <cstdlib>

#include "common.h"

namespace w4a16 {

struct PrefillArgs {
  const uint16_t *A;
  int M, K;
  const uint4_t *rw;    // packed (fused) or fragment-ordered fp16 (DENSE)
  const uint16_t *rs;
  int N, NS, KT, KG8;
  uint16_t *out;
  int ldo;
  int tiles_m, tiles_n;
  int up_off, valid_strips;
};

template <int WN, bool DENSE>
struct PrefillB {
  uint4_t v[WN][DENSE ? 4 : 1];
  uint16_t sc[WN];
};

template <int MI, int WN, bool DENSE, bool SWIGLU>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_kernel(PrefillArgs p) {
  constexpr int BM = 32 * MI;
  constexpr int GM = 4;  // row tiles per group in the tile walk
  __shared__ uint4_t lds[2][BM * 8];
  typedef PrefillB<WN, DENSE> BRegs;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c = lane & 31;
  const int M = p.M;
  const Dequant dq;

  // XCD-aware tile walk.
  const int T = p.tiles_m * p.tiles_n;
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int per = T >> 3, extra = T & 7;
  const int tau = xcd * per + (xcd < extra ? xcd : extra) + local;
  const int group = tau / (GM * p.tiles_n);
  const int first_m = group * GM;
  const int gsize = p.tiles_m - first_m < GM ? p.tiles_m - first_m : GM;
  const int in_group = tau - group * GM * p.tiles_n;
  const int tm = first_m + in_group % gsize;
  const int tn = in_group / gsize;
  const int m0 = tm * BM;

  int strip[WN];
  bool sval[WN];
#pragma unroll
  for (int w = 0; w < WN; ++w) {
    if constexpr (SWIGLU) {
      constexpr int HW = WN / 2;
      const int base = (tn * 4 + wave) * HW + (w % HW);
      strip[w] = w >= HW ? base + p.up_off : base;
      sval[w] = base < p.valid_strips;
    } else {
      strip[w] = (tn * 4 + wave) * WN + w;
      sval[w] = strip[w] < p.NS;
    }
  }

  // Activation staging: thread tid moves chunk (tid & 7) of rows (tid >> 3) + 32 i.
  const int arow = tid >> 3, achunk = tid & 7;
  const uint4_t *Ag = (const uint4_t *)p.A;
  uint4_t areg[MI];
  auto load_a = [&](int q) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = m0 + arow + 32 * i;
      areg[i] = row < M ? Ag[((int64_t)row * p.K + 64 * q) / 8 + achunk] : uint4_t{0, 0, 0, 0};
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = arow + 32 * i;
      lds[buf][row * 8 + (achunk ^ (row & 7))] = areg[i];
    }
  };
  auto load_b = [&](int q, BRegs &r) {
#pragma unroll
    for (int w = 0; w < WN; ++w) {
      const int64_t vec = ((int64_t)strip[w] * p.KT + q) * 64 + lane;
      if constexpr (DENSE) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          r.v[w][j] = sval[w] ? load_nt(p.rw + vec * 4 + j) : uint4_t{0, 0, 0, 0};
      } else {
        r.v[w][0] = sval[w] ? load_nt(p.rw + vec) : uint4_t{0, 0, 0, 0};
        const int g = q >> 1;
        r.sc[w] = sval[w] ? p.rs[(((int64_t)strip[w] * p.KG8 + (g >> 3)) * 32 + c) * 8 + (g & 7)]
                          : (uint16_t)0;
      }
    }
  };

  float16_t acc[WN][MI];
#pragma unroll
  for (int w = 0; w < WN; ++w)
#pragma unroll
    for (int i = 0; i < MI; ++i) acc[w][i] = float16_t{};

  auto compute = [&](int buf, const BRegs &r) {
    half2_t s2[WN];
#pragma unroll
    for (int w = 0; w < WN; ++w) {
      const _Float16 sh = bitcast<_Float16>(r.sc[w]);
      s2[w] = half2_t{sh, sh};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half8_t bf[WN];
#pragma unroll
      for (int w = 0; w < WN; ++w) {
        if constexpr (DENSE)
          bf[w] = bitcast<half8_t>(r.v[w][j]);
        else
          bf[w] = dq.scaled(r.v[w][0][j], s2[w]);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const half8_t af =
            bitcast<half8_t>(lds[buf][(32 * i + c) * 8 + ((4 * h + j) ^ (c & 7))]);
#pragma unroll
        for (int w = 0; w < WN; ++w)
          acc[w][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[w], af, acc[w][i], 0, 0, 0);
      }
    }
  };

  BRegs bcur, bnext;
  load_a(0);
  load_b(0, bcur);
  store_a(0);
  __syncthreads();
  for (int q = 0; q < p.KT; ++q) {
    const bool more = q + 1 < p.KT;
    if (more) {
      load_a(q + 1);
      load_b(q + 1, bnext);
    }
    compute(q & 1, bcur);
    if (more) store_a((q + 1) & 1);
    __syncthreads();
    bcur = bnext;
  }

  // Epilogue.  acc[w][i][4*rg + e] is the output at row m0 + 32 i + c and
  // column 32 strip[w] + 8 rg + 4 h + e: four consecutive columns per store.
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int m = m0 + 32 * i + c;
    if (m >= M) continue;
    uint16_t *orow = p.out + (int64_t)m * p.ldo;
    if constexpr (SWIGLU) {
      constexpr int HW = WN / 2;
#pragma unroll
      for (int w = 0; w < HW; ++w) {
        if (!sval[w]) continue;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          half2_t lo, hi;
          lo.x = (_Float16)silu_mul(acc[w][i][4 * rg + 0], acc[w + HW][i][4 * rg + 0]);
          lo.y = (_Float16)silu_mul(acc[w][i][4 * rg + 1], acc[w + HW][i][4 * rg + 1]);
          hi.x = (_Float16)silu_mul(acc[w][i][4 * rg + 2], acc[w + HW][i][4 * rg + 2]);
          hi.y = (_Float16)silu_mul(acc[w][i][4 * rg + 3], acc[w + HW][i][4 * rg + 3]);
          const int n = strip[w] * 32 + 8 * rg + 4 * h;
          *(uint2 *)(orow + n) = uint2{bitcast<uint32_t>(lo), bitcast<uint32_t>(hi)};
        }
      }
    } else {
#pragma unroll
      for (int w = 0; w < WN; ++w) {
        if (!sval[w]) continue;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int n = strip[w] * 32 + 8 * rg + 4 * h;
          if (n >= p.N) continue;
          half2_t lo, hi;
          lo.x = (_Float16)acc[w][i][4 * rg + 0];
          lo.y = (_Float16)acc[w][i][4 * rg + 1];
          hi.x = (_Float16)acc[w][i][4 * rg + 2];
          hi.y = (_Float16)acc[w][i][4 * rg + 3];
          *(uint2 *)(orow + n) = uint2{bitcast<uint32_t>(lo), bitcast<uint32_t>(hi)};
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Second mainloop: WM x WNW waves, two waves per SIMD.  Each wave owns
// 32*MI rows and two strips (64 columns; for SwiGLU a gate strip and its up
// strip); the workgroup tile is (32*MI*WM) x (64*WNW).  With two waves on
// each SIMD the hardware overlaps one wave's MFMAs with the other's LDS
// reads and dequantization, which a single wave per SIMD cannot do across
// its own dependency chains.
template <int MI, int WM, int WNW, int TPS, bool DENSE, bool SWIGLU>
__global__ __launch_bounds__(64 * WM * WNW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill2_kernel(PrefillArgs p) {
  // TPS: 64-k tiles per pipeline step (2 = one whole 128-k scale group).
  constexpr int BM = 32 * MI * WM;
  constexpr int NT = 64 * WM * WNW;
  constexpr int GM = 4;  // row tiles per group in the tile walk
  constexpr int CH = 8 * TPS;  // 16-byte chunks per staged activation row
  constexpr int AV = BM * CH / NT;
  static_assert(BM * CH % NT == 0, "activation tile split");
  __shared__ uint4_t lds[2][BM * CH];
  struct BRegs {
    uint4_t v[2][TPS][DENSE ? 4 : 1];
    uint16_t sc[2];
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WNW, wn = wave % WNW;
  const int h = lane >> 5, c = lane & 31;
  const int M = p.M;
  const Dequant dq;

  // XCD-aware tile walk (as in prefill_kernel).
  const int T = p.tiles_m * p.tiles_n;
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int per = T >> 3, extra = T & 7;
  const int tau = xcd * per + (xcd < extra ? xcd : extra) + local;
  const int group = tau / (GM * p.tiles_n);
  const int first_m = group * GM;
  const int gsize = p.tiles_m - first_m < GM ? p.tiles_m - first_m : GM;
  const int in_group = tau - group * GM * p.tiles_n;
  const int tm = first_m + in_group % gsize;
  const int tn = in_group / gsize;
  const int m0 = tm * BM;

  int strip[2];
  bool sval[2];
  if constexpr (SWIGLU) {
    const int base = tn * WNW + wn;
    strip[0] = base;
    strip[1] = base + p.up_off;
    sval[0] = sval[1] = base < p.valid_strips;
  } else {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      strip[w] = (tn * WNW + wn) * 2 + w;
      sval[w] = strip[w] < p.NS;
    }
  }

  // LDS swizzle: 16 consecutive rows read at one k land in 16 distinct
  // 16-byte bank groups (the 64 banks x 4 bytes), so the 16 lanes that an
  // ds_read_b128 serves together never collide.  Rows are CH*16 bytes long.
  auto swz = [](int row) {
    return CH == 16 ? (row & 15) : ((row >> 1) & 7);
  };
  // Activation staging: thread tid moves chunk (tid % CH) of rows tid / CH + (NT/CH) i.
  const int arow = tid / CH, achunk = tid % CH;
  const uint4_t *Ag = (const uint4_t *)p.A;
  uint4_t areg[AV];
  auto load_a = [&](int q) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      int row = m0 + arow + (NT / CH) * i;
      row = row < M ? row : M - 1;  // rows past M are computed and never stored
      areg[i] = Ag[((int64_t)row * p.K + 64 * TPS * q) / 8 + achunk];
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int row = arow + (NT / CH) * i;
      lds[buf][row * CH + (achunk ^ swz(row))] = areg[i];
    }
  };
  auto load_b = [&](int q, BRegs &r) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int st = sval[w] ? strip[w] : 0;   // invalid strips read strip 0, never stored
#pragma unroll
      for (int t = 0; t < TPS; ++t) {
        const int64_t vec = ((int64_t)st * p.KT + TPS * q + t) * 64 + lane;
        if constexpr (DENSE) {
#pragma unroll
          for (int j = 0; j < 4; ++j) r.v[w][t][j] = load_nt(p.rw + vec * 4 + j);
        } else {
          r.v[w][t][0] = load_nt(p.rw + vec);
        }
      }
      if constexpr (!DENSE) {
        const int g = (TPS * q) >> 1;
        r.sc[w] = p.rs[(((int64_t)st * p.KG8 + (g >> 3)) * 32 + c) * 8 + (g & 7)];
      }
    }
  };

  float16_t acc[2][MI];
#pragma unroll
  for (int w = 0; w < 2; ++w)
#pragma unroll
    for (int i = 0; i < MI; ++i) acc[w][i] = float16_t{};

  const int rbase = wm * 32 * MI;
  auto compute = [&](int buf, const BRegs &r) {
    half2_t s2[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const _Float16 sh = bitcast<_Float16>(r.sc[w]);
      s2[w] = half2_t{sh, sh};
    }
#pragma unroll
    for (int jj = 0; jj < 4 * TPS; ++jj) {
      const int t = jj >> 2, j = jj & 3;
      half8_t bf[2];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        if constexpr (DENSE)
          bf[w] = bitcast<half8_t>(r.v[w][t][j]);
        else
          bf[w] = dq.scaled(r.v[w][t][0][j], s2[w]);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int row = rbase + 32 * i + c;
        const half8_t af =
            bitcast<half8_t>(lds[buf][row * CH + ((8 * t + 4 * h + j) ^ swz(row))]);
#pragma unroll
        for (int w = 0; w < 2; ++w)
          acc[w][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[w], af, acc[w][i], 0, 0, 0);
      }
    }
  };

  BRegs bcur, bnext;
  load_a(0);
  load_b(0, bcur);
  store_a(0);
  __syncthreads();
  const int nsteps = p.KT / TPS;
  for (int q = 0; q < nsteps; ++q) {
    const bool more = q + 1 < nsteps;
    if (more) {
      load_a(q + 1);
      load_b(q + 1, bnext);
    }
    compute(q & 1, bcur);
    if (more) store_a((q + 1) & 1);
    __syncthreads();
    bcur = bnext;
  }

  // Epilogue: acc[w][i][4*rg + e] is the output at row m0 + rbase + 32 i + c
  // and column 32 strip[w] + 8 rg + 4 h + e.
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int m = m0 + rbase + 32 * i + c;
    if (m >= M) continue;
    uint16_t *orow = p.out + (int64_t)m * p.ldo;
    if constexpr (SWIGLU) {
      if (!sval[0]) continue;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        half2_t lo, hi;
        lo.x = (_Float16)silu_mul(acc[0][i][4 * rg + 0], acc[1][i][4 * rg + 0]);
        lo.y = (_Float16)silu_mul(acc[0][i][4 * rg + 1], acc[1][i][4 * rg + 1]);
        hi.x = (_Float16)silu_mul(acc[0][i][4 * rg + 2], acc[1][i][4 * rg + 2]);
        hi.y = (_Float16)silu_mul(acc[0][i][4 * rg + 3], acc[1][i][4 * rg + 3]);
        const int n = strip[0] * 32 + 8 * rg + 4 * h;
        *(uint2 *)(orow + n) = uint2{bitcast<uint32_t>(lo), bitcast<uint32_t>(hi)};
      }
    } else {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        if (!sval[w]) continue;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int n = strip[w] * 32 + 8 * rg + 4 * h;
          if (n >= p.N) continue;
          half2_t lo, hi;
          lo.x = (_Float16)acc[w][i][4 * rg + 0];
          lo.y = (_Float16)acc[w][i][4 * rg + 1];
          hi.x = (_Float16)acc[w][i][4 * rg + 2];
          hi.y = (_Float16)acc[w][i][4 * rg + 3];
          *(uint2 *)(orow + n) = uint2{bitcast<uint32_t>(lo), bitcast<uint32_t>(hi)};
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side.

static PrefillArgs prefill_args(const Problem &p, int BM, const void *weights) {
  PrefillArgs a;
  a.A = p.A;
  a.M = (int)p.M;
  a.K = (int)p.K;
  a.rw = (const uint4_t *)weights;
  a.rs = (const uint16_t *)p.rs;
  a.N = (int)p.N;
  a.NS = (int)ceil_div(p.N, kStrip);
  a.KT = (int)(p.K / kTileK);
  a.KG8 = (int)ceil_div(p.K / kGroup, 8);
  a.out = p.out;
  a.ldo = (int)(p.swiglu ? p.N / 2 : p.N);
  a.up_off = (int)(p.N / 2 / kStrip);
  a.valid_strips = p.swiglu ? a.up_off : a.NS;
  a.tiles_m = (int)ceil_div(p.M, BM);
  // Each workgroup covers 8 strips (plain) or 4 gate strips + their up strips.
  a.tiles_n = (int)(p.swiglu ? ceil_div(a.up_off, 4) : ceil_div(a.NS, 8));
  return a;
}

template <int MI, bool DENSE, bool SWIGLU>
static hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((prefill_kernel<MI, 2, DENSE, SWIGLU>), dim3(a.tiles_m * a.tiles_n),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

template <bool DENSE>
static hipError_t launch_tiled(const Problem &p, const void *weights, hipStream_t s) {
  // Row tile: 256 rows once M is large, smaller tiles for the transition range.
  const int MI = p.M > 128 ? 8 : (p.M > 64 ? 4 : 2);
  const PrefillArgs a = prefill_args(p, 32 * MI, weights);
  if (MI == 8)
    return p.swiglu ? launch_prefill_t<8, DENSE, true>(a, s) : launch_prefill_t<8, DENSE, false>(a, s);
  if (MI == 4)
    return p.swiglu ? launch_prefill_t<4, DENSE, true>(a, s) : launch_prefill_t<4, DENSE, false>(a, s);
  return p.swiglu ? launch_prefill_t<2, DENSE, true>(a, s) : launch_prefill_t<2, DENSE, false>(a, s);
}

template <int MI, int WM, int WNW, int TPS, bool DENSE, bool SWIGLU>
static hipError_t launch_prefill2_t(const Problem &p, const void *weights, hipStream_t s) {
  PrefillArgs a = prefill_args(p, 32 * MI * WM, weights);
  a.tiles_n = (int)(p.swiglu ? ceil_div(a.up_off, WNW) : ceil_div(a.NS, 2 * WNW));
  hipLaunchKernelGGL((prefill2_kernel<MI, WM, WNW, TPS, DENSE, SWIGLU>), dim3(a.tiles_m * a.tiles_n),
                     dim3(64 * WM * WNW), 0, s, a);
  return hipGetLastError();
}

template <bool DENSE>
static hipError_t launch_tiled2(const Problem &p, const void *weights, hipStream_t s) {
  const char *v = std::getenv("W4A16_PREFILL_TPS");
  if constexpr (!DENSE) {
    if (v != nullptr && *v == '2')
      return p.swiglu ? launch_prefill2_t<4, 2, 4, 2, DENSE, true>(p, weights, s)
                      : launch_prefill2_t<4, 2, 4, 2, DENSE, false>(p, weights, s);
  }
  return p.swiglu ? launch_prefill2_t<4, 2, 4, 1, DENSE, true>(p, weights, s)
                  : launch_prefill2_t<4, 2, 4, 1, DENSE, false>(p, weights, s);
}

static bool prefill_v2() {
  const char *v = std::getenv("W4A16_PREFILL_V2");
  return v != nullptr && *v == '1';
}

hipError_t launch_prefill(const Problem &p, hipStream_t s) {
  if (prefill_v2() && p.M > 256) return launch_tiled2<false>(p, p.rw, s);
  return launch_tiled<false>(p, p.rw, s);
}

int tiled_describe(const Problem &p, bool dense, char *buf, size_t n) {
  const int MI = p.M > 128 ? 8 : (p.M > 64 ? 4 : 2);
  const PrefillArgs a = prefill_args(p, 32 * MI, nullptr);
  return snprintf(buf, n, "%sprefill_kernel<%d, 2, %s, %s> workgroups=%d threads=256",
                  dense ? "dequant_kernel<false>; " : "", MI, dense ? "true" : "false",
                  p.swiglu ? "true" : "false", a.tiles_m * a.tiles_n);
}

int64_t dense_workspace_bytes(const Problem &p) {
  // fp16 weights in fragment order: 64 columns x 64 k x 2 bytes per (strip, tile) half.
  return ceil_div(p.N, kStrip) * (p.K / kTileK) * 64 * 4 * 16;
}

hipError_t launch_dense(const Problem &p, void *workspace, hipStream_t s) {
  if (workspace == nullptr) return hipErrorInvalidValue;
  void *w16f = workspace;
  hipError_t e = launch_dequant_fragment(p.rw, p.rs, p.K, p.N, (uint16_t *)w16f, s);
  if (e != hipSuccess) return e;
  if (prefill_v2() && p.M > 256) return launch_tiled2<true>(p, w16f, s);
  return launch_tiled<true>(p, w16f, s);
}

}  // namespace w4a16
