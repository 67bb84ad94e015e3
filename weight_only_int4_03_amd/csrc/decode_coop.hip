// Decode path, cooperative form: activations and scales staged once per
// workgroup in LDS and shared by waves that own different columns.
//
// Same product as decode.hip (page "GPU Kernels for INT4 Inference, in
// depth", section "The job, stated precisely"; scale after each group's
// accumulation as in FuTransformer, arXiv 2610.23796, section 3.3.4).  The
// difference is where the activation fragments and the group scales come
// from.  In decode.hip every wave loads its own activation fragments and
// scales from global memory, so each workgroup re-reads A once per wave and
// the vector-memory path carries as many activation bytes as weight bytes
// at M = 16 (twice as many at M = 32).  The Swordfish page (section
// "Decode, counting memory-pipe slots") makes the same observation: load
// slots, not arithmetic, are the scarce resource of a decode kernel.
//
// Workgroup layout: WC x WK waves.  Wave (wc, wk) owns strip group
// cg*WC + wc (SPW strips of 32 columns: one strip, or a gate strip and its
// up strip) and, in every round of WK consecutive groups of 128 k, the
// group with index wk.  Per round the workgroup stages the activation rows
// of those WK groups and the scales of its WC*SPW strips into LDS (global
// -> registers -> LDS, double buffered, one barrier per round); weights
// stream per wave straight into registers, D rounds ahead, and are
// dequantized in registers into MFMA operands.  At the end the WK partial
// tiles of each column are summed through LDS; with KS > 1 the partial
// tiles go to the workspace and decode_reduce_kernel finishes them (or, as a
// measurement switch, the launch finishes them itself: split_exchange,
// split_last).
#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "common.h"
#include "decode_args.h"

namespace w4a16 {

template <int MT, int SPW, int BITS>
struct CoopFrag {
  static constexpr int NV = BITS == 8 ? 2 : 1;  // 16-byte vectors per lane and MFMA unit
  uint4_t b[SPW][2][NV];  // weight vectors of the wave's strips for one group
};

template <int MT, int SPW, int WC, int WK, int RPL, bool SWIGLU, bool BF, bool ZP, int BITS>
__global__ __launch_bounds__(WC * WK * 64) void decode_coop_kernel(DecodeArgs p) {
  constexpr int NW = WC * WK, NT = NW * 64, D = 2;
  constexpr int SH = SWIGLU ? SPW / 2 : SPW;
  constexpr int NPART = MT == 16 ? 2 : 1;
  typedef typename std::conditional<MT == 16, float4_t, float16_t>::type acc_t;
  typedef CoopFrag<MT, SPW, BITS> Frag;
  constexpr int NV = Frag::NV;
  constexpr uint32_t TILE = 1024u * NV;   // bytes per 64-k tile of a strip
  constexpr uint32_t GROUP = 2u * TILE;   // bytes per 128-k unit of a strip
  static_assert(MT == 16 ? (RPL >= 1 && RPL <= 4) : RPL == 16, "rows per lane");
  static_assert(BITS == 4 || (BITS == 8 && !ZP), "INT8 weights have no zero rows");

  extern __shared__ uint4_t smem[];
  const int M = p.M;
  const int ars = WK * 256 + 16;               // bytes per staged activation row
  const int abuf = M * ars;                    // bytes per activation buffer
  const int sbuf = (ZP ? 2 : 1) * WC * SPW * 32 * WK * 2;  // bytes per scale (+ zero row) buffer
  char *lds = (char *)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wc = wave % WC, wk = wave / WC;
  const int ncg = (p.nsg + WC - 1) / WC;
  const int cg = blockIdx.x % ncg, split = blockIdx.x / ncg;
  const int sg_raw = cg * WC + wc;
  const bool active = sg_raw < p.nsg;          // inactive waves mirror the last group
  const int sg = active ? sg_raw : p.nsg - 1;
  const Dequant dq;

  const char *wbase[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int base = sg * SH + (s % SH);
    const int strip = SWIGLU && s >= SH ? base + p.up_off : base;
    wbase[s] = (const char *)(p.rw + (int64_t)strip * p.KT * 64 * NV);
  }

  const int gb = (int)((int64_t)p.KG * split / p.KS);
  const int ge = (int)((int64_t)p.KG * (split + 1) / p.KS);
  const int R = (ge - gb + WK - 1) / WK;      // rounds
  // Rotation of the order of the full rounds: loop round r works on round
  // rm(r); a partial last round stays last (the steady-state loop computes
  // every wave's group unconditionally).
  const int RF = (ge - gb) / WK;              // full rounds
  const int rot = (p.stagger != 0 && RF > 0)
                      ? (int)(((uint32_t)blockIdx.x * 2654435761u >> 8) % (uint32_t)RF) : 0;
  auto rm = [&](int r) {
    if (r >= RF) return r;
    const int t = r + rot;
    return t >= RF ? t - RF : t;
  };

  const int g4 = lane >> 4, c16 = lane & 15;
  const int h = lane >> 5, c32 = lane & 31;
  const int mrow = MT == 16 ? c16 : c32;
  // An INT8 tile holds a lane's second vector 1 KiB after its first.
  const uint32_t wlane = MT == 16 ? (uint32_t)((g4 >> 1) * TILE + ((g4 & 1) * 32 + c16) * 16)
                                  : (uint32_t)(lane * 16);
  // LDS byte offset of this lane's activation fragment (row min(mrow, M-1)).
  const int a_lane = (mrow < M ? mrow : M - 1) * ars + wk * 256 + (MT == 16 ? g4 * 64 : h * 64);

  // ---- cooperative staging of round r into registers, then into LDS ------
  // Activations: M rows x WK groups = M * WK * 16 vectors of 16 bytes.
  // Scales: WC*SPW strips x 32 columns x WK groups, 2 bytes each.
  constexpr int AROWS = RPL == 1 ? 1 : MT;     // activation rows staged (M <= AROWS)
  constexpr int AV_MAX = (AROWS * WK * 16 + NT - 1) / NT;
  constexpr int SC_N = (WC * SPW * 32 * WK + NT - 1) / NT;
  struct Stage {
    uint4_t av[AV_MAX];
    uint16_t scv[SC_N];
    uint16_t zsv[ZP ? SC_N : 1];
  };
  const int nav = M * WK * 16;
  // Loads are unconditional (indices clamped into range) so that no register
  // is conditionally rewritten while weight loads are still in flight;
  // staged groups past the end of the K range are never consumed.
  auto stage_load = [&](Stage &st, int r) {
    const int g0 = gb + rm(r) * WK;
#pragma unroll
    for (int t = 0; t < AV_MAX; ++t) {
      int e = tid + t * NT;
      e = e < nav ? e : nav - 1;
      const int row = e / (WK * 16), c = e - row * (WK * 16);
      int gg = g0 + c / 16;
      gg = gg < ge ? gg : ge - 1;
      st.av[t] = *(const uint4_t *)((const char *)p.A +
                                    ((int64_t)row * p.K + (int64_t)gg * 128) * 2 + (c & 15) * 16);
    }
#pragma unroll
    for (int t = 0; t < SC_N; ++t) {
      int e = tid + t * NT;
      e = e < WC * SPW * 32 * WK ? e : WC * SPW * 32 * WK - 1;
      const int wkk = e % WK, c = (e / WK) & 31, sl = e / (WK * 32);
      const int wcc = sl / SPW, s = sl % SPW;
      int sgg = cg * WC + wcc;
      sgg = sgg < p.nsg ? sgg : p.nsg - 1;
      const int base = sgg * SH + (s % SH);
      const int strip = SWIGLU && s >= SH ? base + p.up_off : base;
      int gg = g0 + wkk;
      gg = gg < ge ? gg : ge - 1;
      const int64_t si = scale_index(strip, p.KG8, c, (gg * 128) >> p.gshift);
      st.scv[t] = p.rs[si];
      if constexpr (ZP) st.zsv[t] = p.rz[si];
    }
  };
  // Stores are unconditional too: threads past the end repeat the last
  // element, writing the same value to the same place.  (A conditional store
  // lets the compiler sink the global load next to it, where waiting for it
  // also waits for the weight loads issued in between.)
  auto stage_store = [&](const Stage &st, int buf) {
    char *ab = lds + buf * abuf;
#pragma unroll
    for (int t = 0; t < AV_MAX; ++t) {
      int e = tid + t * NT;
      e = e < nav ? e : nav - 1;
      const int row = e / (WK * 16), c = e - row * (WK * 16);
      *(uint4_t *)(ab + row * ars + c * 16) = st.av[t];
    }
    uint16_t *sb = (uint16_t *)(lds + 2 * abuf + buf * sbuf);
#pragma unroll
    for (int t = 0; t < SC_N; ++t) {
      int e = tid + t * NT;
      e = e < WC * SPW * 32 * WK ? e : WC * SPW * 32 * WK - 1;
      sb[e] = st.scv[t];
      if constexpr (ZP) sb[WC * SPW * 32 * WK + e] = st.zsv[t];
    }
  };

  // ---- per-wave weight stream --------------------------------------------
  // The wave's group in round r is gb + r*WK + wk; past the end of the K
  // range it re-reads the last group (never consumed).
  auto group_of = [&](int r) {
    const int g = gb + rm(r) * WK + wk;
    return g < ge ? g : ge - 1;
  };
  auto wload = [&](Frag &f, int r) {
    const uint32_t ow = (uint32_t)group_of(r) * GROUP + wlane;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const char *wp = wbase[s] + ow;
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int v = 0; v < NV; ++v)
          f.b[s][x][v] =
              load_nt((const uint4_t *)(wp + (MT == 16 ? x * 256 : x * TILE) + v * 1024));
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
  auto wsc = [&](const uint4_t(&v)[NV], int j, uint16_t s16, uint16_t z16) {
    if constexpr (BITS == 8)
      return dq.scaled8_bits<BF>(v[j >> 1][(j & 1) * 2], v[j >> 1][(j & 1) * 2 + 1], s16);
    else
      return dq.scaled_bits<BF, ZP>(v[0][j], s16, z16);
  };

  auto compute = [&](const Frag &f, int buf) {
    const char *ab = lds + buf * abuf + a_lane;
    const uint16_t *sb = (const uint16_t *)(lds + 2 * abuf + buf * sbuf);
    uint4_t a[MT == 16 ? 4 : 8];
    if constexpr (MT == 16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = *(const uint4_t *)(ab + j * 16);
    } else {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int j = 0; j < 4; ++j) a[4 * x + j] = *(const uint4_t *)(ab + x * 128 + j * 16);
    }
    if constexpr (BF || ZP) {
      // bf16, and weights with zero rows: scaled (and shifted) and rounded
      // before the MFMA, which accumulates straight into the FP32 tile.
#pragma unroll
      for (int s = 0; s < SPW; ++s) {
#pragma unroll
        for (int part = 0; part < NPART; ++part) {
          const int col = MT == 16 ? 16 * part + c16 : c32;
          const int si = ((wc * SPW + s) * 32 + col) * WK + wk;
          const uint16_t s16 = sb[si];
          const uint16_t z16 = ZP ? sb[WC * SPW * 32 * WK + si] : 0;
          if constexpr (MT == 16) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[s][part] = mfma16<BF>(a[j], wsc(f.b[s][part], j, s16, z16), acc[s][part]);
          } else {
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                acc[s][part] = mfma32<BF>(a[4 * x + j], wsc(f.b[s][x], j, s16, z16), acc[s][part]);
          }
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
            t = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(a[j]), wq(f.b[s][part], j),
                                                       t, 0, 0, 0);
        } else {
#pragma unroll
          for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              t = __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<half8_t>(a[4 * x + j]),
                                                         wq(f.b[s][x], j), t, 0, 0, 0);
        }
        const int col = MT == 16 ? 16 * part + c16 : c32;
        const float sc = (float)bitcast<_Float16>(sb[((wc * SPW + s) * 32 + col) * WK + wk]);
#pragma unroll
        for (int r = 0; r < RPL; ++r) acc[s][part][r] += t[r] * sc;
      }
    }
  };

  // ---- main loop: rounds r, two per iteration (buffers 0 and 1) ----------
  // Round r's activations and scales are loaded two rounds ahead, just
  // before its weights, and reach LDS one round ahead.  Loads complete in
  // issue order, so waiting for a round's staged values never waits for the
  // weights of that round or the next, and at every barrier two rounds of
  // weights stay in flight.  Scheduling barriers keep that issue order and
  // keep the next round's dequantization below the workgroup barrier (hoisted
  // above it, it would wait there for that round's weights).
  auto round_barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  Frag f0, f1;
  Stage s0, s1;
  stage_load(s0, 0);
  __builtin_amdgcn_sched_barrier(0);
  wload(f0, 0);
  stage_load(s1, 1);
  __builtin_amdgcn_sched_barrier(0);
  wload(f1, 1);
  stage_store(s0, 0);
  round_barrier();
  int r = 0;
  // Steady state: rounds r, r+1 are loaded, round r is in LDS buffer 0 and
  // round r+1 in s1; rounds r+2, r+3 exist.
  for (; r + 4 <= R; r += 2) {
    compute(f0, 0);
    stage_load(s0, r + 2);
    __builtin_amdgcn_sched_barrier(0);
    wload(f0, r + 2);
    stage_store(s1, 1);
    round_barrier();
    compute(f1, 1);
    stage_load(s1, r + 3);
    __builtin_amdgcn_sched_barrier(0);
    wload(f1, r + 3);
    stage_store(s0, 0);
    round_barrier();
  }
  // Tail: at most three rounds left (r .. R-1), in the same state.
  if (r < R) {
    if (gb + rm(r) * WK + wk < ge) compute(f0, 0);
    if (r + 2 < R) {
      stage_load(s0, r + 2);
      __builtin_amdgcn_sched_barrier(0);
      wload(f0, r + 2);
    }
    if (r + 1 < R) stage_store(s1, 1);
    round_barrier();
  }
  if (r + 1 < R) {
    if (gb + rm(r + 1) * WK + wk < ge) compute(f1, 1);
    if (r + 2 < R) stage_store(s0, 0);
    round_barrier();
  }
  if (r + 2 < R) {
    if (gb + rm(r + 2) * WK + wk < ge) compute(f0, 0);
    round_barrier();
  }

  // ---- cross-wave sum over wk, then epilogue or partial tile -------------
  float *red = (float *)lds;  // [WK][WC][SPW][M][32]; the staging buffers are free now
  const int tileE = SPW * M * 32;
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
#pragma unroll
    for (int part = 0; part < NPART; ++part) {
#pragma unroll
      for (int rr = 0; rr < (MT == 16 ? 4 : 16); ++rr) {
        const int m = MT == 16 ? 4 * g4 + rr : 8 * (rr >> 2) + 4 * h + (rr & 3);
        const int col = MT == 16 ? 16 * part + c16 : c32;
        if (m < M) red[((wk * WC + wc) * SPW + s) * M * 32 + m * 32 + col] = acc[s][part][rr];
      }
    }
  }
  __syncthreads();
  auto sum_wk = [&](int wcc, int e) {
    float v = 0.0f;
#pragma unroll
    for (int k = 0; k < WK; ++k) v += red[(k * WC + wcc) * tileE + e];
    return v;
  };
  if (p.KS == 1) {
    const int E = SH * M * 32;
    for (int x = tid; x < WC * E; x += NT) {
      const int wcc = x / E, e = x - wcc * E;
      const int sgg = cg * WC + wcc;
      if (sgg < p.nsg)
        decode_epilogue<SPW, SWIGLU, BF>(p, sgg, e, [&](int y) { return sum_wk(wcc, y); });
    }
    return;
  }
  if (p.xs != nullptr) {
    // The KS workgroups of a strip group finish it here (split_exchange):
    // each element's partials meet pairwise; the last holder runs the epilogue.
    constexpr int EPT = (WC * SH * MT * 32 + NT - 1) / NT;
    const int E = SH * M * 32;
    int64_t el[EPT];
    bool live[EPT];
    float v[EPT], u[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int x = tid + i * NT;
      const int wcc = x / E, e = x - wcc * E;
      live[i] = x < WC * E && cg * WC + wcc < p.nsg;
      el[i] = (int64_t)(cg * WC + wcc) * E + e;
      v[i] = live[i] ? sum_wk(wcc, e) : 0.0f;
      u[i] = live[i] && SWIGLU ? sum_wk(wcc, e + E) : 0.0f;
    }
    split_exchange<EPT>(p.xs, p.KS, split, (int64_t)p.nsg * E, el, live, v, u);
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      if (!live[i]) continue;
      const int x = tid + i * NT;
      const int wcc = x / E, e = x - wcc * E;
      decode_epilogue<SPW, SWIGLU, BF>(p, cg * WC + wcc, e,
                                       [&](int y) { return y == e ? v[i] : u[i]; });
    }
    return;
  }
  if (p.sync != nullptr) {
    for (int x = tid; x < WC * tileE; x += NT) {
      const int wcc = x / tileE, e = x - wcc * tileE;
      const int sgg = cg * WC + wcc;
      if (sgg < p.nsg) store_partial(p.ws + ((int64_t)sgg * p.KS + split) * tileE + e, sum_wk(wcc, e));
    }
    if (!split_last(p.sync + cg, p.KS, (int *)lds)) return;
    const int E = SH * M * 32;
    for (int x = tid; x < WC * E; x += NT) {
      const int wcc = x / E, e = x - wcc * E;
      const int sgg = cg * WC + wcc;
      if (sgg < p.nsg)
        decode_epilogue<SPW, SWIGLU, BF>(p, sgg, e, [&](int y) {
          return sum_partials(p.ws + (int64_t)sgg * p.KS * tileE + y, tileE, p.KS);
        });
    }
    return;
  }
  for (int x = tid; x < WC * tileE; x += NT) {
    const int wcc = x / tileE, e = x - wcc * tileE;
    const int sgg = cg * WC + wcc;
    if (sgg < p.nsg) p.ws[((int64_t)sgg * p.KS + split) * tileE + e] = sum_wk(wcc, e);
  }
  (void)active;
}

// ---------------------------------------------------------------------------
// Host side.

size_t coop_lds_bytes(int M, int WC, int WK, int SPW, bool zp) {
  const size_t stage =
      2 * (size_t)M * (WK * 256 + 16) + 2 * (size_t)(zp ? 2 : 1) * WC * SPW * 32 * WK * 2;
  const size_t red = (size_t)WK * WC * SPW * M * 32 * 4;
  return stage > red ? stage : red;
}

template <int MT, int SPW, int WC, int WK, int RPL, bool SWIGLU, bool BF, bool ZP, int BITS>
static hipError_t launch_coop_t(const DecodeArgs &a, hipStream_t s) {
  const size_t lds = coop_lds_bytes(a.M, WC, WK, SPW, ZP);
  const int ncg = (a.nsg + WC - 1) / WC;
  hipLaunchKernelGGL((decode_coop_kernel<MT, SPW, WC, WK, RPL, SWIGLU, BF, ZP, BITS>), dim3(ncg * a.KS),
                     dim3(WC * WK * 64), lds, s, a);
  return hipGetLastError();
}

template <int MT, int SPW, int RPL, bool SWIGLU, bool BF, bool ZP, int BITS>
static hipError_t launch_coop_w(const DecodeArgs &a, int WC, int WK, hipStream_t s) {
  if (WC == 4 && WK == 1) return launch_coop_t<MT, SPW, 4, 1, RPL, SWIGLU, BF, ZP, BITS>(a, s);
  if (WC == 8 && WK == 1) return launch_coop_t<MT, SPW, 8, 1, RPL, SWIGLU, BF, ZP, BITS>(a, s);
  if (WC == 2 && WK == 2) return launch_coop_t<MT, SPW, 2, 2, RPL, SWIGLU, BF, ZP, BITS>(a, s);
  if (WC == 4 && WK == 2) return launch_coop_t<MT, SPW, 4, 2, RPL, SWIGLU, BF, ZP, BITS>(a, s);
  if (WC == 2 && WK == 4) return launch_coop_t<MT, SPW, 2, 4, RPL, SWIGLU, BF, ZP, BITS>(a, s);
  if constexpr (SPW == 1)  // (the fused form would spill at 32 rows)
    if (WC == 1 && WK == 8) return launch_coop_t<MT, SPW, 1, 8, RPL, SWIGLU, BF, ZP, BITS>(a, s);
  return launch_coop_t<MT, SPW, 1, 4, RPL, SWIGLU, BF, ZP, BITS>(a, s);
}

template <bool BF, bool ZP, int BITS>
static hipError_t launch_coop_bf(const Problem &p, const DecodeArgs &a, int WC, int WK,
                                 hipStream_t s) {
  if (p.M == 1)
    return p.swiglu ? launch_coop_w<16, 2, 1, true, BF, ZP, BITS>(a, WC, WK, s)
                    : launch_coop_w<16, 1, 1, false, BF, ZP, BITS>(a, WC, WK, s);
  if (p.M <= 16)
    return p.swiglu ? launch_coop_w<16, 2, 4, true, BF, ZP, BITS>(a, WC, WK, s)
                    : launch_coop_w<16, 1, 4, false, BF, ZP, BITS>(a, WC, WK, s);
  return p.swiglu ? launch_coop_w<32, 2, 16, true, BF, ZP, BITS>(a, WC, WK, s)
                  : launch_coop_w<32, 1, 16, false, BF, ZP, BITS>(a, WC, WK, s);
}

// -1 if unset, else the integer value.
static int coop_env_raw(const char *name) {
  const char *v = std::getenv(name);
  if (v == nullptr || *v == 0) return -1;
  return std::atoi(v);
}

static int coop_env(const char *name, int fallback) {
  const char *v = std::getenv(name);
  if (v == nullptr || *v == 0) return fallback;
  const int x = std::atoi(v);
  return x > 0 ? x : fallback;
}

// Where the cooperative kernel wins (measured on MI355X, sweeping both
// kernels' configurations over the Llama-8B and -70B projections):
//  * 32-row tiles (M > 16): every shape.  Four waves per column group along
//    K and two column groups per workgroup (the fused projections with at
//    least 512 strip groups and plain ones with K >= 24576: four column
//    groups, two waves along K; plain ones with 129-255 strip groups: one
//    column group and eight waves along K, Llama-8B QKV 10.56 -> 9.90 us
//    against four); K is split (power of two) while the grid stays within
//    256 workgroups.  Measured at M = 32 against two waves along K with two
//    column groups: Llama-8B QKV 11.4 -> 10.6 us, gate/up 20.8 -> 19.6 us,
//    down 15.9 -> 15.1 us; Llama-70B QKV 21.3 -> 19.6 us, O 17.0 -> 15.9 us,
//    gate/up 63.2 -> 54.7 us (the 70B down projection, K = 28672: 37.5 us
//    with four column groups against 38.0 us with two).
//  * M <= 16: wide shapes (>= 384 strip groups: the fused gate/up
//    projections), deep ones (K >= 24576), grids that the per-wave kernel
//    would spread unevenly (more than 256 strip groups, not a multiple of
//    256), and at M > 8 shapes with >= 192 strip groups or K >= 12288.  Four
//    waves per column group along K (two when four column groups share a
//    workgroup); the fewest column groups per workgroup that keep the grid
//    within 256 workgroups.  M = 1 on wide shapes keeps one column group;
//    the widest fused ones (>= 512 strip groups, fp16 INT4) take the
//    per-wave kernel.  Narrow plain shapes with short K (K < 12288) and
//    192-255 strip groups at M > 8, or 128-255 at M = 16: one strip per
//    workgroup with eight waves along K (and two K splits at M = 16 where the
//    split grid fits and the launch can finish it); the same layout with two
//    splits for plain projections of medium depth (12288 <= K < 24576) and
//    97-128 strip groups at M = 9-16.
// Other narrow, short-K shapes at small M keep the per-wave kernel (its
// half-strip grid fills the CUs without sharing activations).  W4A16_DECODE_COOP=0/1
// forces the choice; W4A16_COOP_WC / _WK / _KS override the configuration.
bool coop_config(const Problem &p, int &WC, int &WK, int &KS) {
  const int nsg = (int)(p.swiglu ? (p.N / 2 / kStrip) : ceil_div(p.N, kStrip));
  const int KG = (int)(p.K / kGroup);
  const int SPW = p.swiglu ? 2 : 1;
  const int force = coop_env_raw("W4A16_DECODE_COOP");
  if (p.G < kGroup) return false;  // one scale per column and 128-k unit
  if (p.bits == 8 && p.zp) return false;  // INT8 weights have no zero rows
  const bool wide = nsg >= 384, deep = KG >= 192;
  const bool uneven = nsg > 256 && nsg % 256 != 0;
  bool use;
  if (p.M > 16) {
    // Eight waves per workgroup, four groups of 128 k per round (67 KiB of
    // LDS at M = 32), except for the widest fused projections and the
    // deepest plain ones (four column groups, two groups per round) and
    // mid-width plain ones that fill the CUs with one column group per
    // workgroup, eight groups per round (133 KiB) and no K split.
    use = true;
    if (p.swiglu) {
      WC = nsg >= 512 ? 4 : 2;
      WK = nsg >= 512 ? 2 : 4;
    } else if (KG >= 192) {
      WC = 4;
      WK = 2;
    } else {
      WC = nsg > 128 && nsg < 256 ? 1 : 2;
      WK = WC == 1 ? 8 : 4;
    }
    KS = 1;
    if (WC > 1)
      while ((int64_t)ceil_div(nsg, WC) * KS * 2 <= 256 && KG / (KS * 2) >= 8) KS *= 2;
  } else if (p.M == 1 && !p.swiglu && (deep || uneven) && p.bits == 4 && !p.zp && !p.bf16) {
    // One-row plain projections that are deep or spread unevenly over the
    // CUs (Llama-70B down and QKV): the per-wave kernel with the activation
    // row staged per wave, measured on MI355X at 22.7 against 24.7 us (down,
    // K = 28672) and, with half strips, 11.2 against 12.8 us (QKV, 320 strip
    // groups).
    use = false;
    WC = 1; WK = 4; KS = 1;
  } else if (p.M == 1 && p.swiglu && nsg >= 512 && p.bits == 4 && !p.zp && !p.bf16) {
    // The widest fused projections at M = 1 (Llama-70B gate/up): the
    // per-wave kernel, which stages the activation row per wave without
    // workgroup barriers, measured 42.7 us against 46.5 us.
    use = false;
    WC = 1; WK = 4; KS = 1;
  } else if (!p.swiglu && KG < 96 && nsg < 256 &&
             ((p.M > 8 && nsg >= 192) || (p.M == 16 && nsg >= 128))) {
    // Narrow, short-K plain projections (Llama-8B QKV at M > 8, O at
    // M = 16): one strip per workgroup, eight waves along K, no K split.
    // Measured at M = 16: QKV 7.56 (four waves along K) -> 7.09 us, O 7.09
    // (per-wave kernel, half strips) -> 6.91 us; at M = 8-12 the O
    // projection stays faster on the per-wave kernel (M = 8: 5.66 against
    // 6.57 us) and QKV ties with it at M = 8.
    use = true;
    WC = 1; WK = 8; KS = 1;
    // Two K splits where the doubled grid still fits one workgroup per CU
    // and the launch finishes them itself (exchange): O at M = 16, 7.05 ->
    // 6.37 us; with the reduction launch instead (a caller's workspace) the
    // split measured 7.95 us, so that keeps one split.
    if (p.M == 16 && 2 * nsg <= 256 && split_finish(p, 2) == 1) KS = 2;
  } else if (!p.swiglu && p.M > 8 && KG >= 96 && KG < 192 && nsg > 96 && 2 * nsg <= 256 &&
             split_finish(p, 2) == 1) {
    // Narrow plain projections of medium depth at M = 9-16 (Llama-8B down):
    // one strip per workgroup, eight waves along K and two K splits finished
    // in the launch, 11.77 -> 11.50 us against two column groups with four
    // splits and the reduction launch (which a caller's workspace keeps:
    // this layout with the reduction launch measured 13.0 us).
    use = true;
    WC = 1; WK = 8; KS = 2;
  } else if (p.M == 1 && wide) {
    use = true;
    WC = 1; WK = 4; KS = 1;
  } else {
    use = wide || deep || uneven || (p.M > 8 && (nsg >= 192 || KG >= 96));
    KS = deep ? 2 : (KG >= 96 && p.M > 8 ? 4 : 1);
    WC = 1;
    while (WC < 4 && (int64_t)ceil_div(nsg, WC) * KS > 256) WC *= 2;
    WK = WC == 4 ? 2 : 4;
  }
  if (force == 0) return false;
  if (force == 1) use = true;
  if (!use) return false;
  WC = coop_env("W4A16_COOP_WC", WC);
  WK = coop_env("W4A16_COOP_WK", WK);
  KS = coop_env("W4A16_COOP_KS", KS);
  static const int allowed[7][2] = {{4, 1}, {8, 1}, {2, 2}, {4, 2}, {2, 4}, {1, 4}, {1, 8}};
  bool ok = false;
  for (auto &c : allowed) ok |= (c[0] == WC && c[1] == WK);
  if (!ok || (SPW == 2 && WC == 1 && WK == 8)) return false;
  if (KS > KG) KS = KG;
  if (KS < 1) KS = 1;
  if (coop_lds_bytes((int)p.M, WC, WK, SPW, p.zp) > kMaxLdsPerWorkgroup) return false;
  return true;
}

hipError_t launch_decode_coop(const Problem &p, void *workspace, int WC, int WK, int KS,
                              hipStream_t s) {
  DecodeArgs a = decode_args(p, KS, workspace);
  if (KS > 1 && workspace == nullptr) return hipErrorInvalidValue;
  const hipError_t e =
      p.bits == 8 ? (p.bf16 ? launch_coop_bf<true, false, 8>(p, a, WC, WK, s)
                            : launch_coop_bf<false, false, 8>(p, a, WC, WK, s))
      : p.zp      ? (p.bf16 ? launch_coop_bf<true, true, 4>(p, a, WC, WK, s)
                            : launch_coop_bf<false, true, 4>(p, a, WC, WK, s))
                  : (p.bf16 ? launch_coop_bf<true, false, 4>(p, a, WC, WK, s)
                            : launch_coop_bf<false, false, 4>(p, a, WC, WK, s));
  if (e != hipSuccess || KS == 1 || a.xs != nullptr || a.sync != nullptr) return e;
  return launch_decode_reduce(a, p.swiglu, p.bf16, s);
}

}  // namespace w4a16
