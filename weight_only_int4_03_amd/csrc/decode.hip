// Decode path (small M): a weight-streaming W4A16 GEMM.
//
// What it computes is the page "GPU Kernels for INT4 Inference, in depth"
// (aicassindra.com), section "The job, stated precisely": C = A * dequant(W),
// FP32 accumulation.  The page's section "What this simple kernel leaves on
// the table" names the decode problems this kernel answers: too few programs
// at M = 1 (hence the K split, reduced afterwards), dequantization in the
// loop, and a layout not tuned for the hardware (hence the repacked layout).
// The scale is applied after each group's accumulation, as FuTransformer
// (arXiv 2610.23796) section 3.3.4 does.
//
// Mapping on gfx950 (wave64, MFMA):
//   * M <= 16: v_mfma_f32_16x16x32_f16, activation rows padded to 16;
//     M <= 32: v_mfma_f32_32x32x16_f16, rows padded to 32.  MFMA is far from
//     the bound here; it replaces ~8 VALU MACs per weight with one issue slot.
//   * A workgroup owns SPW column strips (32 columns each; for SwiGLU a gate
//     strip and the matching up strip) and a slice of K.  Its WAVES waves
//     split that slice by whole groups of 128; every packed word is read
//     exactly once, with 16-byte non-temporal loads (each wave-wide load is a
//     contiguous 1 KiB tile), D groups ahead of use.
//   * Nibbles become fp16 (u - 8) in registers (shift, and-or with the 0x6400
//     exponent, one packed subtract).  Each group of 128 k accumulates into a
//     zeroed MFMA tile; the tile times the column's fp16 scale is then added
//     to the FP32 accumulator (one FMA per accumulator per group).
//   * Waves reduce through LDS.  With KS = 1 the workgroup then runs the
//     epilogue.  With KS > 1 workgroups on one strip group, each writes its
//     partial tile to the workspace and a second kernel sums the KS partials
//     in split order and runs the epilogue.  No workgroup waits on another:
//     on gfx950 an agent-scope fence writes back and invalidates the XCD's
//     L2, so a per-workgroup fence (the "last workgroup finishes" pattern)
//     serialises the whole grid; the kernel boundary publishes the partials
//     once instead.  The order is fixed, so results are bit-identical from
//     run to run.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <vector>

#include "common.h"
#include "decode_args.h"

namespace w4a16 {

template <int MT, int SPW, int BITS = 4>
struct DecodeFrag {
  static constexpr int NB = 2;                 // 16-byte weight vectors per strip per group
  static constexpr int NV = BITS == 8 ? 2 : 1;  // vectors per lane and MFMA unit (INT8: two)
  static constexpr int NA = MT == 16 ? 4 : 8;  // 16-byte activation vectors per group
  uint4_t b[SPW][NB][NV];
  uint4_t a[NA];
  int gi;  // group held (one-row instances read its activations from LDS)
  // Scales per strip, 16-column half (MT=16) and 64-k tile (MT=32, which
  // can span two groups when G < 128), and the zero rows likewise (16-bit
  // values held in 32-bit words, which keeps the arrays in registers).
  uint32_t sc[SPW][MT == 16 ? 2 : 1][MT == 16 ? 1 : 2];
  uint32_t zs[SPW][MT == 16 ? 2 : 1][MT == 16 ? 1 : 2];
};

// PRE: the weights are scaled before the MFMA (bf16 activations, whose
// weights are rounded to bf16, and groups shorter than the 128-k unit, whose
// lanes meet different scales within one MFMA); otherwise each 128-k unit is
// accumulated unscaled and its tile scaled once afterwards.
// ZP: zero rows (AWQ zero points prescaled as fp16((8 - zp) s)); each weight
// is then the one rounding of (u - 8) s + z, so it is scaled before the MFMA.
// HALF (MT=16 only): the workgroup owns one 16-column half of each of its
// strips (workgroups 2b and 2b+1 share strip group b), which doubles the
// workgroups of a narrow projection without splitting K.
// BITS: 4 (INT4 codes offset by 8) or 8 (INT8 codes offset by 128, the
// repacked INT8 layout: twice the bytes per tile, two vectors per lane).
template <int MT, int SPW, int WAVES, int D, int RPL, bool SWIGLU, bool BF, bool PRE, bool ZP,
          bool HALF, int BITS = 4>
__global__ __launch_bounds__(WAVES * 64) void decode_kernel(DecodeArgs p) {
  static_assert(PRE || !BF, "bf16 weights are always scaled before the MFMA");
  static_assert(PRE || !ZP, "weights with zero points are scaled before the MFMA");
  static_assert(!HALF || MT == 16, "half strips need the 16-column MFMA");
  static_assert(BITS == 4 || (BITS == 8 && !ZP), "INT8 weights have no zero rows");
  static_assert(MT == 16 ? (RPL >= 0 && RPL <= 4) : RPL == 16, "rows per lane");
  // RPL = 0: the one-row (M = 1) instance without the matrix unit: each lane
  // takes v_dot2_f32_f16 products of its 32 k of the activation row with the
  // exact u - 8 weights, and the four lanes that share a column are summed at
  // the end by a ds_swizzle and a v_permlane32_swap.
  constexpr bool DOT = RPL == 0;
  static_assert(!DOT || (!PRE && !BF && !ZP && BITS == 4), "dot instances: fp16 INT4, G >= 128");
  // LDS: the cross-wave reduction [WAVES][SPW][M][32] floats; one-row
  // instances (M = 1) add the workgroup's activation slice after it.
  extern __shared__ float lds[];
  constexpr int SH = SWIGLU ? SPW / 2 : SPW;
  // 16-column halves per workgroup (MT=16) or the whole strip (MT=32).
  constexpr int NPART = MT == 16 ? (HALF ? 1 : 2) : 1;
  typedef typename std::conditional<MT == 16, float4_t, float16_t>::type acc_t;
  typedef DecodeFrag<MT, SPW, BITS> Frag;
  constexpr int NV = Frag::NV;
  constexpr uint32_t TILE = 1024u * NV;   // bytes per 64-k tile of a strip
  constexpr uint32_t GROUP = 2u * TILE;   // bytes per 128-k unit of a strip

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int half = HALF ? (int)(blockIdx.x & 1) : 0;  // first 16-column half owned
  const int bid = HALF ? (int)(blockIdx.x >> 1) : (int)blockIdx.x;
  const int sg = bid % p.nsg, split = bid / p.nsg;
  const int M = p.M;
  const Dequant dq;

  // The grid covers exactly the strip groups that exist, so every strip a
  // workgroup names is a real one (the repacked buffer pads N to 32 columns).
  const char *wbase[SPW];
  const char *sbase[SPW];
  const char *zbase[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int base = sg * SH + (s % SH);
    const int strip = SWIGLU && s >= SH ? base + p.up_off : base;
    wbase[s] = (const char *)(p.rw + (int64_t)strip * p.KT * 64 * NV);
    sbase[s] = (const char *)(p.rs + (int64_t)strip * p.KG8 * 256);
    zbase[s] = ZP ? (const char *)(p.rz + (int64_t)strip * p.KG8 * 256) : nullptr;
  }

  const int unit = split * WAVES + wave, nunits = p.KS * WAVES;
  const int g0 = (int)((int64_t)p.KG * unit / nunits);
  const int g1 = (int)((int64_t)p.KG * (unit + 1) / nunits);
  // One-row instances (M = 1): the MFMA activation operand is 16 copies of
  // one row; loaded from global memory per group that is four 16-byte loads
  // per 1 KiB of weights, which occupy the wave's memory requests (measured
  // on MI355X: the one-row GEMMs ran 13-22% faster with those loads
  // removed).  Each wave instead copies its own K range of the row into a
  // private LDS region with one 16-byte load per lane and KiB, and reads each
  // group's fragment from there one group ahead of its use; no other wave
  // touches the region, so no workgroup barrier is
  // needed.
  constexpr bool AL = MT == 16 && RPL <= 1;
  const int wslice = (int)ceil_div((int64_t)p.KG, (int64_t)nunits) * 256;  // bytes per wave
  char *lds_a = (char *)lds + WAVES * SPW * 32 * 4 + wave * wslice;  // after the reduction tile

  // Lane roles.  MT=16: lane = 16*g4 + c16; row of A = c16; lane group g4
  // covers k offsets 32*g4 .. +31 of the group.  MT=32: lane = 32*h + c;
  // row of A = c; lane half h covers k offsets 64x + 32h .. +31 of X-tile x.
  // Rows of the MFMA tile beyond M read row M-1 again: output row m depends
  // only on activation row m, and rows >= M are never stored.
  const int g4 = lane >> 4, c16 = lane & 15;
  const int h = lane >> 5, c32 = lane & 31;
  const int mrow = MT == 16 ? c16 : c32;
  const uint32_t arow_off = (uint32_t)(mrow < M ? mrow : M - 1) * (uint32_t)p.K * 2u;
  // Byte offsets inside one group's bytes of a strip (two 64-k tiles; an
  // INT8 tile holds a lane's second vector 1 KiB after its first).
  const uint32_t wlane = MT == 16 ? (uint32_t)((g4 >> 1) * TILE + ((g4 & 1) * 32 + c16) * 16)
                                  : (uint32_t)(lane * 16);
  const uint32_t slane = (uint32_t)((MT == 16 ? c16 : c32) * 16);
  // k offset, within a 128-k unit, of the lane's first weight (tile x = 0).
  const int klane = MT == 16 ? 32 * g4 : 32 * h;
  const uint32_t alane = MT == 16 ? (uint32_t)(g4 * 64) : (uint32_t)(h * 64);
  const char *Ab = (const char *)p.A;

  // Every address is a uniform base plus one 32-bit lane offset (plus a
  // constant), which maps onto the scalar-base form of the global loads.
  auto soff = [&](int grp) { return (uint32_t)(grp >> 3) * 512u + (uint32_t)(grp & 7) * 2u + slane; };
  auto load = [&](Frag &f, int g) {
    const uint32_t ow = (uint32_t)g * GROUP + wlane;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const char *wp = wbase[s] + ow;
      if constexpr (MT == 16) {
#pragma unroll
        for (int part = 0; part < NPART; ++part)
#pragma unroll
          for (int v = 0; v < NV; ++v)
            f.b[s][part][v] = load_nt((const uint4_t *)(wp + (half + part) * 256 + v * 1024));
      } else {
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int v = 0; v < NV; ++v)
            f.b[s][x][v] = load_nt((const uint4_t *)(wp + x * TILE + v * 1024));
      }
      if constexpr (PRE) {
        if constexpr (MT == 16) {
          const uint32_t so = soff((128 * g + klane) >> p.gshift) + half * 256;
#pragma unroll
          for (int part = 0; part < NPART; ++part) {
            f.sc[s][part][0] = *(const uint16_t *)(sbase[s] + so + part * 256);
            if constexpr (ZP) f.zs[s][part][0] = *(const uint16_t *)(zbase[s] + so + part * 256);
          }
        } else {
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const uint32_t so = soff((128 * g + 64 * x + klane) >> p.gshift);
            f.sc[s][0][x] = *(const uint16_t *)(sbase[s] + so);
            if constexpr (ZP) f.zs[s][0][x] = *(const uint16_t *)(zbase[s] + so);
          }
        }
      } else {
        const char *sp = sbase[s] + soff((128 * g) >> p.gshift) + half * 256;
#pragma unroll
        for (int part = 0; part < NPART; ++part)
          f.sc[s][part][0] = *(const uint16_t *)(sp + part * 256);
      }
    }
    const char *ag = Ab + (uint32_t)(arow_off + (uint32_t)g * 256u + alane);
    if constexpr (AL) {
      f.gi = g;  // activations are read from LDS just ahead of use
    } else if constexpr (MT == 16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) f.a[j] = *(const uint4_t *)(ag + j * 16);
    } else {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int j = 0; j < 4; ++j) f.a[4 * x + j] = *(const uint4_t *)(ag + x * 128 + j * 16);
    }
  };

  acc_t acc[SPW][NPART];
#pragma unroll
  for (int s = 0; s < SPW; ++s)
#pragma unroll
    for (int part = 0; part < NPART; ++part) acc[s][part] = acc_t{};

  // MFMA weight operand j (k offsets 8j .. 8j+7 of the lane's 32) of one
  // strip part: unscaled (exact code minus offset, fp16) or scaled.
  auto wq = [&](const uint4_t(&v)[NV], int j) {
    if constexpr (BITS == 8)
      return dq.bytes8(v[j >> 1][(j & 1) * 2], v[j >> 1][(j & 1) * 2 + 1]);
    else
      return dq(v[0][j]);
  };
  auto wsc = [&](const uint4_t(&v)[NV], int j, uint16_t sc, uint16_t zs) {
    if constexpr (BITS == 8)
      return dq.scaled8_bits<BF>(v[j >> 1][(j & 1) * 2], v[j >> 1][(j & 1) * 2 + 1], sc);
    else
      return dq.scaled_bits<BF, ZP>(v[0][j], sc, zs);
  };

  auto compute = [&](const Frag &f) {
    if constexpr (PRE) {
      // Scaled weights (rounded to fp16 or bf16) into the MFMA, which
      // accumulates straight into the FP32 accumulator.
#pragma unroll
      for (int s = 0; s < SPW; ++s) {
#pragma unroll
        for (int part = 0; part < NPART; ++part) {
          if constexpr (MT == 16) {
            const uint16_t sc = (uint16_t)f.sc[s][part][0], zs = (uint16_t)f.zs[s][part][0];
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[s][part] = mfma16<BF>(f.a[j], wsc(f.b[s][part], j, sc, zs), acc[s][part]);
          } else {
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                acc[s][part] = mfma32<BF>(
                    f.a[4 * x + j],
                    wsc(f.b[s][x], j, (uint16_t)f.sc[s][0][x], (uint16_t)f.zs[s][0][x]),
                    acc[s][part]);
          }
        }
      }
      return;
    }
    if constexpr (DOT) {
      // k offsets 32 g4 + 8 j .. + 7 of the group: the lane's activation
      // fragment f.a[j] and its weight word j, paired by v_dot2_f32_f16.
#pragma unroll
      for (int s = 0; s < SPW; ++s) {
#pragma unroll
        for (int part = 0; part < NPART; ++part) {
          float t = 0.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const half8_t w = dq(f.b[s][part][0][j]);
            const half8_t a = bitcast<half8_t>(f.a[j]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              t = __builtin_amdgcn_fdot2(half2_t{a[2 * q], a[2 * q + 1]},
                                         half2_t{w[2 * q], w[2 * q + 1]}, t, false);
          }
          acc[s][part][0] += t * (float)bitcast<_Float16>((uint16_t)f.sc[s][part][0]);
        }
      }
      return;
    }
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
#pragma unroll
      for (int part = 0; part < NPART; ++part) {
        acc_t t = acc_t{};
        if constexpr (MT == 16) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            t = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(f.a[j]),
                                                       wq(f.b[s][part], j), t, 0, 0, 0);
        } else {
#pragma unroll
          for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              t = __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<half8_t>(f.a[4 * x + j]),
                                                         wq(f.b[s][x], j), t, 0, 0, 0);
        }
        const float sc = (float)bitcast<_Float16>((uint16_t)f.sc[s][part][0]);
        // Element r of a lane's tile holds row 4*g4 + r (MT=16), so with
        // M < 4 only elements r < RPL can hold real rows.
#pragma unroll
        for (int r = 0; r < RPL; ++r) acc[s][part][r] += t[r] * sc;
      }
    }
  };

  // D-deep register pipeline over this wave's groups [g0, g1): buffer d
  // holds group g + d.  The steady-state loop is branch-free, so each buffer
  // keeps its registers and the loads of groups g + D .. g + 2D - 1 stay in
  // flight while groups g .. g + D - 1 are consumed.
  // The prologue loads are unconditional (a wave with fewer than D groups
  // loads its last group again) so that the loop is always entered with the
  // same loads outstanding and the compiler's wait counts stay exact.
  // After each reload the next buffer's weight registers pass through an
  // empty asm statement that is ordered after the reload's loads: left free,
  // the compiler hoists the next buffer's dequantization above the reload,
  // waits there for that buffer, and the loads then arrive in batches of D
  // instead of streaming.
  auto after_reload = [&](Frag &f) {
#pragma unroll
    for (int s = 0; s < SPW; ++s)
#pragma unroll
      for (int x = 0; x < (MT == 16 ? NPART : 2); ++x)
#pragma unroll
        for (int v = 0; v < NV; ++v) asm volatile("" : "+v"(f.b[s][x][v]) : : "memory");
  };
  // Rotated order (p.stagger): loop index g reads group gmap(g), so that the
  // waves of different workgroups are not at the same offset of their
  // strips at the same time.  Only the order of the per-group additions to
  // the FP32 accumulators changes.
  const int ng = g1 - g0;
  const int rot = (p.stagger != 0 && ng > 0)
                      ? (int)(((uint32_t)blockIdx.x * 2654435761u >> 8) % (uint32_t)ng) : 0;
  auto gmap = [&](int g) { int t = g - g0 + rot; return g0 + (t >= ng ? t - ng : t); };
  auto load_g = [&](Frag &f, int g) { load(f, gmap(g)); };
  // One-row instances: the MFMA activation operand of the group f holds.
  auto fill_a = [&](Frag &f) {
    if constexpr (AL) {
      const char *src = lds_a + (f.gi - g0) * 256 + alane;
#pragma unroll
      for (int j = 0; j < 4; ++j) f.a[j] = *(const uint4_t *)(src + j * 16);
    }
  };
  // The wave's range [g0, g1) of activation row 0: its first 16 groups are
  // loaded into registers before the first weight loads and stored to LDS
  // after them, so the stores wait only for the activations (loads complete
  // in issue order) while the weights stay in flight; longer ranges copy the
  // rest afterwards.  A wave-scope fence orders the lanes' LDS writes before
  // any lane's reads.
  constexpr int AV = AL ? 4 : 1;  // 16-byte activation vectors per lane (16 groups)
  uint4_t av[AV];
  const uint4_t *asrc = (const uint4_t *)p.A + (int64_t)g0 * 16;
  const int n16 = (g1 - g0) * 16;
  if constexpr (AL) {
    if (n16 > 0) {
#pragma unroll
      for (int t = 0; t < AV; ++t) {
        const int e = lane + 64 * t;
        av[t] = asrc[e < n16 ? e : n16 - 1];
      }
    }
  }
  Frag f[D];
  if (g1 > g0) {
#pragma unroll
    for (int d = 0; d < D; ++d) load_g(f[d], g0 + d < g1 ? g0 + d : g1 - 1);
  }
  if constexpr (AL) {
    uint4_t *dst = (uint4_t *)lds_a;
#pragma unroll
    for (int t = 0; t < AV; ++t) {
      const int e = lane + 64 * t;
      if (e < n16) dst[e] = av[t];
    }
    for (int e = lane + 64 * AV; e < n16; e += 64) dst[e] = asrc[e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  if (g1 > g0) {
    fill_a(f[0]);
    int g = g0;
    for (; g + 2 * D <= g1; g += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        fill_a(f[(d + 1) % D]);
        compute(f[d]);
        load_g(f[d], g + d + D);
        after_reload(f[(d + 1) % D]);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (g + d < g1) {
        fill_a(f[d]);
        compute(f[d]);
        if (g + d + D < g1) load_g(f[d], g + d + D);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (g + D + d < g1) {
        fill_a(f[d]);
        compute(f[d]);
      }
  }

  if constexpr (DOT) {
    // Each lane holds its quarter (k offsets 32 g4 ..) of its column's sum:
    // add the quarters of lanes c16, c16 + 16 (ds_swizzle, swap of 16-lane
    // groups) and of the two 32-lane halves (v_permlane32_swap), leaving the
    // column sum as row 0 in every lane.
#pragma unroll
    for (int s = 0; s < SPW; ++s)
#pragma unroll
      for (int part = 0; part < NPART; ++part) {
        float v = acc[s][part][0];
        v += bitcast<float>(__builtin_amdgcn_ds_swizzle(bitcast<int>(v), 0x401F));
        const auto x = __builtin_amdgcn_permlane32_swap(bitcast<unsigned>(v),
                                                        bitcast<unsigned>(v), false, false);
        acc[s][part][0] = bitcast<float>((unsigned)x[0]) + bitcast<float>((unsigned)x[1]);
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
        const int col = MT == 16 ? 16 * (half + part) + c16 : c32;
        if (m < M) lds[((wave * SPW + s) * M + m) * 32 + col] = acc[s][part][r];
      }
    }
  }
  __syncthreads();

  const int tileE = SPW * M * 32;
  constexpr int nthreads = WAVES * 64;
  auto wave_sum = [&](int e) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += lds[w * tileE + e];
    return v;
  };

  // Tile element e of the columns this workgroup owns, in the [s][m][32]
  // order of the tile (with HALF: 16 of each 32).
  auto owned = [&](int e) { return HALF ? ((e >> 4) << 5) + 16 * half + (e & 15) : e; };
  constexpr int OWN = HALF ? 16 : 32;
  if (p.KS == 1) {
    const int E = SH * M * OWN;
    for (int e = threadIdx.x; e < E; e += nthreads)
      decode_epilogue<SPW, SWIGLU, BF>(p, sg, owned(e), wave_sum);
    return;
  }
  if (p.xs != nullptr) {
    // The KS workgroups of a strip group finish it here (split_exchange).
    constexpr int EPT = (SH * MT * OWN + nthreads - 1) / nthreads;
    const int E = SH * M * 32;
    int64_t el[EPT];
    bool live[EPT];
    float v[EPT], u[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int x = threadIdx.x + i * nthreads;
      const int e = owned(x);
      live[i] = x < SH * M * OWN;
      el[i] = (int64_t)sg * E + e;
      v[i] = live[i] ? wave_sum(e) : 0.0f;
      u[i] = live[i] && SWIGLU ? wave_sum(e + E) : 0.0f;
    }
    split_exchange<EPT>(p.xs, p.KS, split, (int64_t)p.nsg * E, el, live, v, u);
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      if (!live[i]) continue;
      const int e = owned(threadIdx.x + i * nthreads);
      decode_epilogue<SPW, SWIGLU, BF>(p, sg, e, [&](int y) { return y == e ? v[i] : u[i]; });
    }
    return;
  }
  if (p.sync != nullptr) {
    float *mine = p.ws + ((int64_t)sg * p.KS + split) * tileE;
    for (int e = threadIdx.x; e < SPW * M * OWN; e += nthreads)
      store_partial(mine + owned(e), wave_sum(owned(e)));
    if (!split_last(p.sync + sg * (HALF ? 2 : 1) + half, p.KS, (int *)lds)) return;
    const float *all = p.ws + (int64_t)sg * p.KS * tileE;
    for (int e = threadIdx.x; e < SH * M * OWN; e += nthreads)
      decode_epilogue<SPW, SWIGLU, BF>(p, sg, owned(e), [&](int y) {
        return sum_partials(all + y, tileE, p.KS);
      });
    return;
  }
  float *mine = p.ws + ((int64_t)sg * p.KS + split) * tileE;
  for (int e = threadIdx.x; e < SPW * M * OWN; e += nthreads) mine[owned(e)] = wave_sum(owned(e));
}

// Second stage for KS > 1: one thread per output element sums the KS partial
// tiles of its strip group in split order (starting from the first partial,
// so two partials give p0 + p1 exactly as split_exchange does), then runs
// the epilogue.  The partials of up to eight splits are loaded before any is
// added, so their memory latencies overlap instead of adding up.
template <int SPW, bool SWIGLU, bool BF>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs p) {
  constexpr int SH = SWIGLU ? SPW / 2 : SPW;
  const int E = SH * p.M * 32;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)p.nsg * E) return;
  const int sg = (int)(idx / E), e = (int)(idx - (int64_t)sg * E);
  const int tileE = SPW * p.M * 32;
  const float *all = p.ws + (int64_t)sg * p.KS * tileE;
  decode_epilogue<SPW, SWIGLU, BF>(p, sg, e, [&](int x) {
    float v = 0.0f;
    for (int sp0 = 0; sp0 < p.KS; sp0 += 8) {
      float t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        t[i] = sp0 + i < p.KS ? all[(int64_t)(sp0 + i) * tileE + x] : 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (sp0 + i < p.KS) v = sp0 + i == 0 ? t[i] : v + t[i];
    }
    return v;
  });
}

// ---------------------------------------------------------------------------
// Host side: configuration choice and launch.

struct DecodeConfig {
  int MT, SPW, WAVES, D, KS, nsg;
  bool half;  // one 16-column half of each strip per workgroup (MT=16)
};

static int env_int(const char *name, int fallback) {
  const char *v = std::getenv(name);
  if (v == nullptr || *v == 0) return fallback;
  const int x = std::atoi(v);
  return x > 0 ? x : fallback;
}

// Waves per workgroup and K splits.  The aim is enough waves in flight to
// cover HBM latency (several per SIMD on all 256 CUs) without splitting K
// across workgroups unless the strip groups alone leave CUs idle.  Half
// strips (M <= 16) double the workgroups of a narrow projection; measured on
// MI355X they pay off where the doubled grid is at most one workgroup per CU
// and K is short (or M <= 4): each half-strip workgroup reads the whole
// activation slice for half the weights, so at larger M and long K the
// activation loads dominate, and a grid of 1.5 workgroups per CU leaves half
// the CUs with twice the work.  Two groups in flight per wave, four for
// one-row GEMVs with long per-wave K ranges (at M = 1 the activation row is
// staged per wave in LDS; eight waves replaced four waves of four for the
// half-strip GEMVs: Llama-8B down 10.4 -> 8.5 us, the 4096 x 4096 GEMV
// unchanged at 4.7 us).
// W4A16_DECODE_HALF (0 or 1), W4A16_DECODE_WAVES (4 or 8),
// W4A16_DECODE_KS and W4A16_DECODE_DEPTH (groups loaded ahead: 2 or 4)
// override the choice.
static DecodeConfig decode_config(const Problem &p) {
  DecodeConfig c;
  c.MT = p.M <= 16 ? 16 : 32;
  const int64_t NS = ceil_div(p.N, kStrip);
  const int64_t KG = p.K / kGroup;
  c.SPW = p.swiglu ? 2 : 1;
  c.nsg = (int)(p.swiglu ? (p.N / 2 / kStrip) : NS);
  const char *hv = std::getenv("W4A16_DECODE_HALF");
  // One-row GEMMs whose strip groups are more than 256 and not a multiple of
  // it also take half strips (Llama-70B QKV, 320 strip groups: 640
  // workgroups spread over the CUs more evenly than 320).
  const bool uneven_row = p.M == 1 && c.nsg > 256 && c.nsg % 256 != 0 && !p.swiglu;
  const bool half_fits = (2 * (int64_t)c.nsg <= 256 && (KG <= 64 || p.M <= 4)) || uneven_row;
  c.half = c.MT == 16 && (hv != nullptr && *hv != 0 ? *hv == '1' : half_fits);
  const int64_t units = (int64_t)c.nsg * (c.half ? 2 : 1);
  int waves = (units < 384 || KG >= 128) ? 8 : 4;
  waves = env_int("W4A16_DECODE_WAVES", waves) >= 8 ? 8 : 4;
  // LDS for the cross-wave reduction: WAVES * SPW * M * 32 floats < 64 KiB.
  while (waves > 4 && (int64_t)waves * c.SPW * p.M * 32 * 4 >= 65536) waves /= 2;
  c.WAVES = waves;

  // A second launch (the reduction) costs more than idle CUs unless each
  // wave still streams a long K slice: split K only for narrow, deep shapes.
  int64_t ks = (units < 256 && KG / c.WAVES >= 8) ? 2 : 1;
  ks = env_int("W4A16_DECODE_KS", (int)ks);
  if (ks > KG) ks = KG;
  if (ks > 64) ks = 64;
  if (ks < 1) ks = 1;
  c.KS = (int)ks;
  // Four groups in flight for the one-row GEMVs whose waves stream at least
  // 12 groups (Llama-8B down: 9.2 -> 8.5 us); shorter ranges lose more to
  // the deeper prologue than they gain (4096 x 4096: 4.8 -> 5.0 us), and so
  // do the fused gate/up instances, with two strips' registers per group
  // (Llama-70B gate/up: 42.7 us two deep, 45.4 us four deep).
  const bool deep_row = p.M == 1 && !p.swiglu && KG / (c.KS * c.WAVES) >= 12;
  c.D = env_int("W4A16_DECODE_DEPTH", deep_row ? 4 : 2) >= 4 ? 4 : 2;
  return c;
}

// LDS of the one-row instances' activation slices: one region per wave,
// each the longest per-wave K range.
static size_t one_row_slice_bytes(int KG, int KS, int WAVES) {
  return (size_t)WAVES * ceil_div(KG, KS * WAVES) * 256;
}

// One-row instances (activation row staged per wave in LDS) serve M = 1
// when the slices fit; otherwise M = 1 runs the four-rows-per-lane
// instances.
static bool one_row(const Problem &p, const DecodeConfig &c) {
  return c.MT == 16 && p.M == 1 &&
         (size_t)c.WAVES * c.SPW * 32 * 4 + one_row_slice_bytes((int)(p.K / kGroup), c.KS, c.WAVES) <=
             kMaxLdsPerWorkgroup;
}

// The one-row instances without the matrix unit (v_dot2_f32_f16 products,
// ds_swizzle / v_permlane32_swap lane sums) for fp16 INT4 weights with
// groups of at least 128 k, when W4A16_DECODE_DOT=1.  Measured against the
// MFMA instances (activation row padded to 16 rows) on MI355X; off unless
// forced.
static bool dot_row(const Problem &p, const DecodeConfig &c) {
  const char *v = std::getenv("W4A16_DECODE_DOT");
  return v != nullptr && *v == '1' && one_row(p, c) && !p.bf16 && !p.zp && p.bits == 4 &&
         p.G >= kGroup;
}

// Rotated K order (each wave starts its K range, or the coop kernel its
// sequence of rounds, at an offset hashed from the workgroup index).  Strips
// are contiguous in K, so without it the concurrently running waves read
// addresses that agree modulo the strip stride.  Measured on MI355X: where
// that stride is a multiple of 128 KiB (INT4 at K = 8192: the Llama-70B QKV,
// O and gate/up projections) rotating gains up to 13% (gate/up M = 4, 16:
// 46.5 -> 40.5 us, 48.8 -> 42.7 us; QKV M = 1: 18.5 -> 15.0 us); at other
// strides it changes nothing or costs 1-3% (Llama-8B gate/up, 64 KiB), so it
// is off there.  W4A16_DECODE_STAGGER (0 or 1) overrides the choice.
static bool decode_stagger(const Problem &p) {
  const int64_t strip_bytes = p.K * kStrip * p.bits / 8;
  bool on = strip_bytes % (128 * 1024) == 0;
  const char *v = std::getenv("W4A16_DECODE_STAGGER");
  if (v != nullptr && *v != 0) on = *v == '1';
  return on;
}

// Split-K finish inside the launch (split_exchange).  Measured on MI355X
// (bench.py --sweep splitk): with two K splits and a small output the
// exchange beats the reduction launch (Llama-8B down at M = 8: 10.9 against
// 12.2 us; Llama-70B down at M = 4 and 16: 24.3 and 26.9 against 25.5 and
// 27.8 us); with more splits or rows its one memory transaction per 8 bytes
// of partial values costs more than the launch it saves (M = 32, four splits:
// 14.4 against 9.6 us).  The exchange slots live in this fixed array, zero
// when the library loads and left zero by every call; so the exchange runs
// only for calls on the library's own workspace or fixed scratch, whose calls
// must not overlap in time on one device anyway.  A call with a caller's
// workspace keeps the reduction launch, which gives the same bits (two
// partials: p0 + p1 either way), except where the cooperative kernel's
// configuration itself takes two K splits only because they can be finished
// in the launch (coop_config: Llama-8B O and down at M = 9-16); a caller's
// workspace then keeps the unsplit layout, and the two calls differ by FP32
// summation order.  W4A16_SPLIT_FINISH=exchange, =last (the
// last workgroup of a tile sums partial tiles written through to the point of
// coherence: split_last) or =reduce overrides the choice for measurement;
// with it set, calls that overlap in time on one device race.
static __device__ __align__(256) unsigned long long split_sync[1 << 20];  // 8 MiB
constexpr int64_t kExchangeMaxElems = 16 * 8192;  // M * output columns

static std::mutex g_split_sync_mutex;
static std::vector<void *> g_split_sync;  // device address of split_sync, per device

static void *split_sync_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(g_split_sync_mutex);
  if ((int)g_split_sync.size() <= dev) g_split_sync.resize(dev + 1, nullptr);
  if (g_split_sync[dev] == nullptr) {
    void *q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(split_sync)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_split_sync[dev] = q;
  }
  return g_split_sync[dev];
}

int split_finish(const Problem &p, int KS) {
  if (KS <= 1) return 0;
  const int64_t el = (p.swiglu ? p.N / 2 : ceil_div(p.N, kStrip) * kStrip) * p.M;
  int mode = p.own_ws && KS == 2 && el <= kExchangeMaxElems ? 1 : 0;
  const char *v = std::getenv("W4A16_SPLIT_FINISH");
  if (v != nullptr && std::strcmp(v, "exchange") == 0) mode = 1;
  if (v != nullptr && std::strcmp(v, "last") == 0) mode = 2;
  if (v != nullptr && std::strcmp(v, "reduce") == 0) mode = 0;
  if (mode == 1 && split_exchange_bytes(KS, el) > (int64_t)sizeof(split_sync)) mode = 0;
  // (last: one counter per strip group and half strip, or column group)
  if (mode == 2 && 2 * ceil_div(p.N, kStrip) * (int64_t)sizeof(unsigned) > (int64_t)sizeof(split_sync))
    mode = 0;
  return mode;
}

static int describe_finish(const Problem &p, int KS, int spw, const char *sw, const char *bf,
                           char *buf, size_t n) {
  switch (split_finish(p, KS)) {
    case 1: return snprintf(buf, n, "; K splits finished in the launch (exchange)");
    case 2: return snprintf(buf, n, "; K splits finished in the launch (last workgroup)");
    default: return snprintf(buf, n, "; decode_reduce_kernel<%d, %s, %s>", spw, sw, bf);
  }
}

int decode_describe(const Problem &p, char *buf, size_t n) {
  int WC, WK, KS;
  const char *sw = p.swiglu ? "true" : "false", *bf = p.bf16 ? "true" : "false";
  if (coop_config(p, WC, WK, KS)) {
    const int mt = p.M <= 16 ? 16 : 32;
    const int rpl = mt == 16 ? (p.M == 1 ? 1 : 4) : 16;
    const int spw = p.swiglu ? 2 : 1;
    const int nsg = (int)(p.swiglu ? (p.N / 2 / kStrip) : ceil_div(p.N, kStrip));
    int k = snprintf(buf, n,
                     "decode_coop_kernel<%d, %d, %d, %d, %d, %s, %s, %s, %d> workgroups=%d "
                     "threads=%d ks=%d",
                     mt, spw, WC, WK, rpl, sw, bf, p.zp ? "true" : "false", p.bits,
                     (int)ceil_div(nsg, WC) * KS, WC * WK * 64, KS);
    if (decode_stagger(p) && k > 0 && (size_t)k < n) k += snprintf(buf + k, n - k, " stagger");
    if (KS > 1 && k > 0 && (size_t)k < n) k += describe_finish(p, KS, spw, sw, bf, buf + k, n - k);
    return k;
  }
  const DecodeConfig c = decode_config(p);
  const int rpl = c.MT == 16 ? (dot_row(p, c) ? 0 : one_row(p, c) ? 1 : 4) : 16;
  const char *pre = (p.bf16 || p.G < kGroup || p.zp) ? "true" : "false";
  const char *zp = p.zp ? "true" : "false", *hf = c.half ? "true" : "false";
  int k = snprintf(buf, n,
                   "decode_kernel<%d, %d, %d, %d, %d, %s, %s, %s, %s, %s, %d> workgroups=%d "
                   "threads=%d ks=%d",
                   c.MT, c.SPW, c.WAVES, c.D, rpl, sw, bf, pre, zp, hf, p.bits,
                   c.nsg * c.KS * (c.half ? 2 : 1), c.WAVES * 64, c.KS);
  if (decode_stagger(p) && k > 0 && (size_t)k < n) k += snprintf(buf + k, n - k, " stagger");
  if (c.KS > 1 && k > 0 && (size_t)k < n) k += describe_finish(p, c.KS, c.SPW, sw, bf, buf + k, n - k);
  return k;
}

int64_t decode_workspace_bytes(const Problem &p) {
  int WC, WK, KS;
  if (coop_config(p, WC, WK, KS)) {
    const int64_t nsg = p.swiglu ? p.N / 2 / kStrip : ceil_div(p.N, kStrip);
    const int64_t spw = p.swiglu ? 2 : 1;
    return KS == 1 ? 0 : nsg * KS * spw * p.M * 32 * (int64_t)sizeof(float);
  }
  const DecodeConfig c = decode_config(p);
  if (c.KS == 1) return 0;
  return (int64_t)c.nsg * c.KS * c.SPW * p.M * 32 * (int64_t)sizeof(float);
}

template <int MT, int SPW, int WAVES, int D, int RPL, bool SWIGLU, bool BF, bool PRE, bool ZP,
          bool HALF, int BITS>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t s) {
  const size_t lds = (size_t)WAVES * SPW * a.M * 32 * sizeof(float) +
                     (MT == 16 && RPL <= 1 ? one_row_slice_bytes(a.KG, a.KS, WAVES) : 0);
  hipLaunchKernelGGL((decode_kernel<MT, SPW, WAVES, D, RPL, SWIGLU, BF, PRE, ZP, HALF, BITS>),
                     dim3(a.nsg * a.KS * (HALF ? 2 : 1)), dim3(WAVES * 64), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.KS == 1 || a.xs != nullptr || a.sync != nullptr) return e;
  return launch_decode_reduce(a, SWIGLU, BF, s);
}

template <int MT, int SPW, int RPL, bool SWIGLU, bool BF, bool PRE, bool ZP, bool HALF, int BITS>
static hipError_t launch_decode_h(const DecodeArgs &a, const DecodeConfig &c, hipStream_t s) {
  if (c.D == 4)
    return c.WAVES == 8 ? launch_decode_t<MT, SPW, 8, 4, RPL, SWIGLU, BF, PRE, ZP, HALF, BITS>(a, s)
                        : launch_decode_t<MT, SPW, 4, 4, RPL, SWIGLU, BF, PRE, ZP, HALF, BITS>(a, s);
  return c.WAVES == 8 ? launch_decode_t<MT, SPW, 8, 2, RPL, SWIGLU, BF, PRE, ZP, HALF, BITS>(a, s)
                      : launch_decode_t<MT, SPW, 4, 2, RPL, SWIGLU, BF, PRE, ZP, HALF, BITS>(a, s);
}

template <int MT, int SPW, int RPL, bool SWIGLU, bool BF, bool PRE, bool ZP, int BITS>
static hipError_t launch_decode_w(const DecodeArgs &a, const DecodeConfig &c, hipStream_t s) {
  if constexpr (MT == 16) {
    if (c.half) return launch_decode_h<MT, SPW, RPL, SWIGLU, BF, PRE, ZP, true, BITS>(a, c, s);
  }
  return launch_decode_h<MT, SPW, RPL, SWIGLU, BF, PRE, ZP, false, BITS>(a, c, s);
}

template <bool BF, bool PRE, bool ZP, int BITS = 4>
static hipError_t launch_decode_bf(const Problem &p, const DecodeArgs &a, const DecodeConfig &c,
                                   hipStream_t s) {
  if constexpr (!BF && !PRE && !ZP && BITS == 4) {
    if (dot_row(p, c))
      return p.swiglu ? launch_decode_w<16, 2, 0, true, BF, PRE, ZP, BITS>(a, c, s)
                      : launch_decode_w<16, 1, 0, false, BF, PRE, ZP, BITS>(a, c, s);
  }
  if (one_row(p, c))
    return p.swiglu ? launch_decode_w<16, 2, 1, true, BF, PRE, ZP, BITS>(a, c, s)
                    : launch_decode_w<16, 1, 1, false, BF, PRE, ZP, BITS>(a, c, s);
  if (c.MT == 16)
    return p.swiglu ? launch_decode_w<16, 2, 4, true, BF, PRE, ZP, BITS>(a, c, s)
                    : launch_decode_w<16, 1, 4, false, BF, PRE, ZP, BITS>(a, c, s);
  return p.swiglu ? launch_decode_w<32, 2, 16, true, BF, PRE, ZP, BITS>(a, c, s)
                  : launch_decode_w<32, 1, 16, false, BF, PRE, ZP, BITS>(a, c, s);
}

DecodeArgs decode_args(const Problem &p, int KS, void *workspace) {
  DecodeArgs a;
  a.xs = nullptr;
  a.sync = nullptr;
  const int finish = split_finish(p, KS);
  if (finish == 1) a.xs = (unsigned long long *)split_sync_address();
  if (finish == 2 && workspace != nullptr) a.sync = (unsigned *)split_sync_address();
  a.A = p.A;
  a.M = (int)p.M;
  a.K = (int)p.K;
  a.rw = (const uint4_t *)p.rw;
  a.rs = (const uint16_t *)p.rs;
  a.rz = (const uint16_t *)p.rz;
  a.N = (int)p.N;
  a.NS = (int)ceil_div(p.N, kStrip);
  a.KT = (int)(p.K / kTileK);
  a.KG = (int)(p.K / kGroup);
  a.KG8 = (int)ceil_div(groups_of(p.K, p.G), 8);
  a.gshift = p.gshift;
  a.out = p.out;
  a.ldo = (int)(p.swiglu ? p.N / 2 : p.N);
  a.KS = KS;
  a.up_off = (int)(p.N / 2 / kStrip);
  a.valid_strips = p.swiglu ? a.up_off : a.NS;
  a.nsg = p.swiglu ? a.up_off : a.NS;
  a.ws = (float *)workspace;
  a.rowscale = p.rowscale;
  a.stagger = decode_stagger(p) ? 1 : 0;
  return a;
}

hipError_t launch_decode_reduce(const DecodeArgs &a, bool swiglu, bool bf16, hipStream_t s) {
  const int64_t total = (int64_t)a.nsg * a.M * 32;
  const dim3 grid((unsigned)ceil_div(total, 256));
  if (swiglu) {
    if (bf16)
      hipLaunchKernelGGL((decode_reduce_kernel<2, true, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((decode_reduce_kernel<2, true, false>), grid, dim3(256), 0, s, a);
  } else {
    if (bf16)
      hipLaunchKernelGGL((decode_reduce_kernel<1, false, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((decode_reduce_kernel<1, false, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const Problem &p, void *workspace, hipStream_t s) {
  int WC, WK, KS;
  if (coop_config(p, WC, WK, KS)) return launch_decode_coop(p, workspace, WC, WK, KS, s);
  const DecodeConfig c = decode_config(p);
  DecodeArgs a = decode_args(p, c.KS, workspace);
  if (c.KS > 1 && workspace == nullptr) return hipErrorInvalidValue;
  if (p.bits == 8) {
    if (p.bf16) return launch_decode_bf<true, true, false, 8>(p, a, c, s);
    return p.G < kGroup ? launch_decode_bf<false, true, false, 8>(p, a, c, s)
                        : launch_decode_bf<false, false, false, 8>(p, a, c, s);
  }
  if (p.zp)
    return p.bf16 ? launch_decode_bf<true, true, true>(p, a, c, s)
                  : launch_decode_bf<false, true, true>(p, a, c, s);
  if (p.bf16) return launch_decode_bf<true, true, false>(p, a, c, s);
  return p.G < kGroup ? launch_decode_bf<false, true, false>(p, a, c, s)
                      : launch_decode_bf<false, false, false>(p, a, c, s);
}

}  // namespace w4a16
