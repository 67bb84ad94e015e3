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
  // prefill2_kernel split-K: the nsteps pipeline steps are cut into KS
  // slices (slice j: steps [j nsteps / KS, (j+1) nsteps / KS)); with KS > 1
  // every slice writes FP32 partials ws[KS][M][N] (gate and up columns alike)
  // and prefill_reduce_kernel finishes the output.
  int KS, nsteps;
  float *ws;
  const float *rowscale;  // per-row output factor, or null
  int gshift;             // group of k = k >> gshift
  const uint16_t *rz;     // prescaled zero rows (laid out as rs), or null
};

template <int WN, bool DENSE>
struct PrefillB {
  uint4_t v[WN][DENSE ? 4 : 1];
  uint16_t sc[WN];
  uint16_t zs[WN];  // zero row of the group (0 without zero points)
};

template <int MI, int WN, bool DENSE, bool SWIGLU, bool BF>
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
        const int g = (64 * q + 32 * h) >> p.gshift;
        const int64_t si = scale_index(strip[w], p.KG8, c, g);
        r.sc[w] = sval[w] ? p.rs[si] : (uint16_t)0;
        r.zs[w] = sval[w] && p.rz != nullptr ? p.rz[si] : (uint16_t)0;
      }
    }
  };

  float16_t acc[WN][MI];
#pragma unroll
  for (int w = 0; w < WN; ++w)
#pragma unroll
    for (int i = 0; i < MI; ++i) acc[w][i] = float16_t{};

  auto compute = [&](int buf, const BRegs &r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4_t bf[WN];
#pragma unroll
      for (int w = 0; w < WN; ++w) {
        if constexpr (DENSE) {
          bf[w] = r.v[w][j];
        } else {
          // A zero row of 0 leaves every weight as the plain scaled value.
          bf[w] = dq.scaled_bits<BF, true>(r.v[w][0][j], r.sc[w], r.zs[w]);
        }
      }
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const uint4_t af = lds[buf][(32 * i + c) * 8 + ((4 * h + j) ^ (c & 7))];
#pragma unroll
        for (int w = 0; w < WN; ++w) acc[w][i] = mfma32<BF>(bf[w], af, acc[w][i]);
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
    const float rs = p.rowscale != nullptr ? p.rowscale[m] : 1.0f;
    if constexpr (SWIGLU) {
      constexpr int HW = WN / 2;
#pragma unroll
      for (int w = 0; w < HW; ++w) {
        if (!sval[w]) continue;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const float16_t &g = acc[w][i], &u = acc[w + HW][i];
          const int n = strip[w] * 32 + 8 * rg + 4 * h;
          *(uint2 *)(orow + n) =
              uint2{pack_out2<BF>(silu_mul(rs * g[4 * rg + 0], rs * u[4 * rg + 0]),
                                  silu_mul(rs * g[4 * rg + 1], rs * u[4 * rg + 1])),
                    pack_out2<BF>(silu_mul(rs * g[4 * rg + 2], rs * u[4 * rg + 2]),
                                  silu_mul(rs * g[4 * rg + 3], rs * u[4 * rg + 3]))};
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
          const float16_t &v = acc[w][i];
          *(uint2 *)(orow + n) = uint2{pack_out2<BF>(rs * v[4 * rg + 0], rs * v[4 * rg + 1]),
                                       pack_out2<BF>(rs * v[4 * rg + 2], rs * v[4 * rg + 3])};
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
// its own dependency chains.  Two waves per SIMD leave 256 registers per
// wave, so nothing is staged in registers that need not be: activations go
// from memory straight into LDS (buffer loads with the LDS destination), and
// all operands are addressed with fixed 32-bit lane offsets plus a scalar k
// offset.  Each step issues the next step's loads, then runs its MFMAs
// (a scheduling barrier keeps the loads first), then meets the workgroup
// barrier, which also waits for the loads.
template <int MI, int WM, int WNW, int TPS, bool DENSE, bool SWIGLU, bool BF, bool ZP, int BITS>
__global__ __launch_bounds__(64 * WM * WNW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill2_kernel(PrefillArgs p) {
  // TPS: 64-k tiles per pipeline step (2 = one whole 128-k scale group).
  // ZP: zero rows (AWQ zero points prescaled as fp16((8 - zp) s)), loaded
  // beside the scales.
  // All global reads are buffer loads: a per-lane 32-bit offset fixed for the
  // whole k loop plus a scalar offset that advances with k, so the loop does
  // no address arithmetic and holds no 64-bit pointers.  Buffer reads past the
  // end of a resource return zero, which also covers activation rows past M.
  constexpr int BM = 32 * MI * WM;
  constexpr int NW = WM * WNW;
  constexpr int NT = 64 * NW;
  // Row tiles per group in the tile walk: the workgroups of one XCD walk GM
  // row tiles of a column tile before the next column tile, so that many
  // row tiles share each weight tile while it is in the XCD's L2 (8 measured
  // 1-4% faster than 4 with 128-row tiles at M = 4096 and 8191).
  constexpr int GM = 8;
  constexpr int CH = 8 * TPS;  // 16-byte chunks per staged activation row
  constexpr int AV = BM * CH / NT;  // activation copies per lane and step
  // BITS: 4 (INT4 codes) or 8 (INT8 codes in the repacked INT8 layout, whose
  // two vectors per lane and tile lie 1 KiB apart).
  static_assert(BITS == 4 || (BITS == 8 && !DENSE && !ZP), "INT8: fused, no zero rows");
  constexpr int NV = DENSE ? 4 : (BITS == 8 ? 2 : 1);  // 16-byte vectors per lane, strip, tile
  constexpr int VSTEP = BITS == 8 ? 1024 : 16;          // bytes between a lane's vectors
  static_assert(BM * CH % NT == 0, "activation tile split");
  static_assert((NT / CH) % 16 == 0, "swizzle period must divide the rows per copy");
  // The two activation stages are separate arrays so that the compiler can
  // tell the stage being filled from the stage being read.
  __shared__ uint4_t lds0[BM * CH];
  __shared__ uint4_t lds1[BM * CH];
  static_assert(!(DENSE && ZP), "the dense tier's weights are already dequantized");
  struct BRegs {
    uint4_t v[2][TPS][NV];
    uint32_t sc[2][TPS];  // per strip and 64-k tile (tiles may lie in different groups):
                          // scale bits
    // Zero-row bits, in registers of their own: merged into the scale
    // register right after the load, they would make the wave wait there for
    // every load of the step (loads complete in issue order).
    uint32_t zc[ZP ? 2 : 1][TPS];
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WNW, wn = wave % WNW;
  const int h = lane >> 5, c = lane & 31;
  const Dequant dq;

  // XCD-aware tile walk (as in prefill_kernel) over KS slices of T tiles:
  // each XCD takes a contiguous range of the KS * T (slice, tile) pairs.
  const int T = p.tiles_m * p.tiles_n;
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int per = (T * p.KS) >> 3, extra = (T * p.KS) & 7;
  const int tau_all = xcd * per + (xcd < extra ? xcd : extra) + local;
  const int ks = tau_all / T;
  const int tau = tau_all - ks * T;
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

  // Buffer resources.  The activation resource starts at this tile's first
  // row and ends at row M, so rows past M read as zero.
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(p.A + (int64_t)m0 * p.K), (short)0, (p.M - m0) * p.K * 2, kBufferConfig);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void *)p.rw, (short)0, p.NS * p.KT * 64 * 16 * NV, kBufferConfig);
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)p.rs, (short)0, p.NS * p.KG8 * 512, kBufferConfig);
  const __amdgpu_buffer_rsrc_t rzr = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(ZP ? p.rz : p.rs), (short)0, p.NS * p.KG8 * 512, kBufferConfig);

  // LDS swizzle: 16 consecutive rows read at one k land in 16 distinct
  // 16-byte bank groups (the 64 banks x 4 bytes), so the 16 lanes that an
  // ds_read_b128 serves together never collide.  Rows are CH*16 bytes long.
  auto swz = [](int row) {
    return CH == 16 ? (row & 15) : ((row >> 1) & 7);
  };
  // Activation staging goes straight from memory into LDS: copy i of wave
  // `wave` fills the 64 consecutive 16-byte LDS slots starting at slot
  // (i * NW + wave) * 64, one per lane.  Slot s holds row s / CH, physical
  // chunk s % CH, which is logical chunk (s % CH) ^ swz(row); the rows a lane
  // fills advance by NT / CH per copy, a multiple of the swizzle period, so
  // the lane's logical chunk is the same for every copy.
  const int slot0 = wave * 64 + lane;
  const int arow0 = slot0 / CH;
  const int a_off = (arow0 * p.K + ((slot0 % CH) ^ swz(arow0)) * 8) * 2;
  const int a_rows = (NT / CH) * p.K * 2;  // bytes between successive copies
  typedef __attribute__((address_space(3))) void *lds_ptr;
  // The row advance of copy i goes into the lane offset, which the buffer's
  // range check covers (rows past M read as zero); the k offset, always
  // inside the row, is the scalar offset.
  auto load_a = [&](int q, uint4_t *stage) {
    const int k_off = 128 * TPS * q;
#pragma unroll
    for (int i = 0; i < AV; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr)(stage + (i * NW + wave) * 64), 16,
                                               a_off + a_rows * i, k_off, 0, 0);
  };
  // Weights: invalid strips read strip 0 and are never stored.
  int w_off[2], s_off[2];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const int st = sval[w] ? strip[w] : 0;
    w_off[w] = st * p.KT * 64 * 16 * NV + lane * (BITS == 8 ? 16 : 16 * NV);
    s_off[w] = (st * p.KG8 * 32 + c) * 16;
  }
  auto load_b = [&](int q, BRegs &r) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
#pragma unroll
      for (int t = 0; t < TPS; ++t)
#pragma unroll
        for (int j = 0; j < NV; ++j)
          r.v[w][t][j] = bitcast<uint4_t>(__builtin_amdgcn_raw_buffer_load_b128(
              rw, w_off[w] + VSTEP * j, (TPS * q + t) * 1024 * NV, kBufferNT));
    }
    if constexpr (!DENSE) {
#pragma unroll
      for (int t = 0; t < TPS; ++t) {
        const int g = (64 * (TPS * q + t) + 32 * h) >> p.gshift;
        const int g_off = (g >> 3) * 512 + (g & 7) * 2;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          r.sc[w][t] = __builtin_amdgcn_raw_buffer_load_b16(rsc, s_off[w] + g_off, 0, 0);
          if constexpr (ZP)
            r.zc[w][t] = __builtin_amdgcn_raw_buffer_load_b16(rzr, s_off[w] + g_off, 0, 0);
        }
      }
    }
  };

  float16_t acc[2][MI];
#pragma unroll
  for (int w = 0; w < 2; ++w)
#pragma unroll
    for (int i = 0; i < MI; ++i) acc[w][i] = float16_t{};

  const int rbase = wm * 32 * MI;
  auto compute = [&](const uint4_t *stage, const BRegs &r) {
    auto frag = [&](int jj, int w) -> uint4_t {
      const int t = jj >> 2, j = jj & 3;
      if constexpr (DENSE) {
        return r.v[w][t][j];
      } else if constexpr (BITS == 8) {
        const uint4_t &v = r.v[w][t][j >> 1];
        return dq.scaled8_bits<BF>(v[(j & 1) * 2], v[(j & 1) * 2 + 1], (uint16_t)r.sc[w][t]);
      } else if constexpr (ZP) {
        return dq.scaled_bits<BF, true>(r.v[w][t][0][j], (uint16_t)r.sc[w][t],
                                        (uint16_t)r.zc[w][t]);
      } else if constexpr (BF) {
        return bitcast<uint4_t>(
            dq.scaled_bf16(r.v[w][t][0][j], Dequant::BScale((uint16_t)r.sc[w][t])));
      } else {
        const _Float16 sh = bitcast<_Float16>((uint16_t)r.sc[w][t]);
        return bitcast<uint4_t>(dq.scaled(r.v[w][t][0][j], half2_t{sh, sh}));
      }
    };
    if constexpr (BITS == 8 || DENSE || BM == 256) {
      // Fragment by fragment (the pipelined form below would spill with the
      // 8-bit weights' second vector per lane, and in the 256-row tile).
#pragma unroll
      for (int jj = 0; jj < 4 * TPS; ++jj) {
        const int t = jj >> 2, j = jj & 3;
        const uint4_t bw[2] = {frag(jj, 0), frag(jj, 1)};
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int row = rbase + 32 * i + c;
          const uint4_t af = stage[row * CH + ((8 * t + 4 * h + j) ^ swz(row))];
#pragma unroll
          for (int w = 0; w < 2; ++w) acc[w][i] = mfma32<BF>(bw[w], af, acc[w][i]);
        }
      }
      return;
    }
    // Software-pipelined by one fragment: fragment jj + 1 is dequantized
    // while fragment jj's MFMAs run.
    uint4_t bf[2] = {frag(0, 0), frag(0, 1)};
#pragma unroll
    for (int jj = 0; jj < 4 * TPS; ++jj) {
      const int t = jj >> 2, j = jj & 3;
      uint4_t af[MI];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int row = rbase + 32 * i + c;
        af[i] = stage[row * CH + ((8 * t + 4 * h + j) ^ swz(row))];
      }
      uint4_t nb[2] = {bf[0], bf[1]};
      if (jj + 1 < 4 * TPS) {
        nb[0] = frag(jj + 1, 0);
        nb[1] = frag(jj + 1, 1);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int w = 0; w < 2; ++w) acc[w][i] = mfma32<BF>(bf[w], af[i], acc[w][i]);
      // Interleave the MFMAs with the next fragment's dequantization, one
      // MFMA then three VALU instructions (measured 1% faster than the
      // compiler's own order; one and two, or two and five, were slower).
#pragma unroll
      for (int k = 0; k < 2 * MI; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three VALU
      }
      bf[0] = nb[0];
      bf[1] = nb[1];
    }
  };


  // Two register sets for the weights and two LDS stages for the activations,
  // used in turn (the loop is unrolled by two so that nothing is copied).
  // Every step loads the next step's operands unconditionally (the last step
  // reloads its own k range into the idle buffers), so the loop has no
  // conditional loads; the barrier that ends a step waits for those loads.
  const int q0 = (int)((int64_t)ks * p.nsteps / p.KS);
  const int q1 = (int)((int64_t)(ks + 1) * p.nsteps / p.KS);
  BRegs b0, b1;
  load_a(q0, lds0);
  load_b(q0, b0);
  __syncthreads();
  auto step = [&](int q, const uint4_t *stage, const BRegs &cur, uint4_t *nstage, BRegs &next) {
    const int qn = q + 1 < q1 ? q + 1 : q;
    load_a(qn, nstage);
    load_b(qn, next);
    // Keep the loads ahead of the step's MFMAs, so that their latency is
    // spent under the math rather than at the barrier.
    __builtin_amdgcn_sched_barrier(0);
    compute(stage, cur);
    __syncthreads();
  };
  int q = q0;
  for (; q + 1 < q1; q += 2) {
    step(q, lds0, b0, lds1, b1);
    step(q + 1, lds1, b1, lds0, b0);
  }
  if (q < q1) step(q, lds0, b0, lds1, b1);

  if (p.KS > 1) {
    // Split K: FP32 partials of this slice, columns as in the weights.
    float *slice = p.ws + (int64_t)ks * p.M * p.N;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = m0 + rbase + 32 * i + c;
      if (m >= p.M) continue;
      float *prow = slice + (int64_t)m * p.N;
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        if (!sval[w]) continue;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int n = strip[w] * 32 + 8 * rg + 4 * h;
          if (n >= p.N) continue;
          *(float4_t *)(prow + n) = float4_t{acc[w][i][4 * rg + 0], acc[w][i][4 * rg + 1],
                                             acc[w][i][4 * rg + 2], acc[w][i][4 * rg + 3]};
        }
      }
    }
    return;
  }

  // Epilogue: acc[w][i][4*rg + e] is the output at row m0 + rbase + 32 i + c
  // and column 32 strip[w] + 8 rg + 4 h + e.
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int m = m0 + rbase + 32 * i + c;
    if (m >= p.M) continue;
    uint16_t *orow = p.out + (int64_t)m * p.ldo;
    const float rs = p.rowscale != nullptr ? p.rowscale[m] : 1.0f;
    if constexpr (SWIGLU) {
      if (!sval[0]) continue;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const float16_t &g = acc[0][i], &u = acc[1][i];
        const int n = strip[0] * 32 + 8 * rg + 4 * h;
        *(uint2 *)(orow + n) = uint2{pack_out2<BF>(silu_mul(rs * g[4 * rg + 0], rs * u[4 * rg + 0]),
                                                   silu_mul(rs * g[4 * rg + 1], rs * u[4 * rg + 1])),
                                     pack_out2<BF>(silu_mul(rs * g[4 * rg + 2], rs * u[4 * rg + 2]),
                                                   silu_mul(rs * g[4 * rg + 3], rs * u[4 * rg + 3]))};
      }
    } else {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        if (!sval[w]) continue;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int n = strip[w] * 32 + 8 * rg + 4 * h;
          if (n >= p.N) continue;
          const float16_t &v = acc[w][i];
          *(uint2 *)(orow + n) = uint2{pack_out2<BF>(rs * v[4 * rg + 0], rs * v[4 * rg + 1]),
                                       pack_out2<BF>(rs * v[4 * rg + 2], rs * v[4 * rg + 3])};
        }
      }
    }
  }
}

// Second stage of a split-K prefill: sums the KS FP32 partial slices in
// slice order and applies the epilogue.  One thread per 4 consecutive
// outputs of a row.
template <bool SWIGLU, bool BF>
__global__ __launch_bounds__(256) void prefill_reduce_kernel(const float *ws, int KS, int M,
                                                             int N, uint16_t *out, int ldo,
                                                             const float *rowscale) {
  const int per_row = ldo >> 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)M * per_row) return;
  const int m = (int)(idx / per_row), n = (int)(idx - (int64_t)m * per_row) * 4;
  const int64_t slice = (int64_t)M * N;
  const float *src = ws + (int64_t)m * N + n;
  // Slices are added in order; the partials of up to eight slices are loaded
  // before any is added, so their memory latencies overlap.
  float4_t g = {0.0f, 0.0f, 0.0f, 0.0f}, u = {0.0f, 0.0f, 0.0f, 0.0f};
  constexpr int B = 8;
  for (int k0 = 0; k0 < KS; k0 += B) {
    float4_t tg[B], tu[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      if (k0 + i < KS) {
        tg[i] = *(const float4_t *)(src + (k0 + i) * slice);
        if constexpr (SWIGLU) tu[i] = *(const float4_t *)(src + (k0 + i) * slice + N / 2);
      }
    }
#pragma unroll
    for (int i = 0; i < B; ++i) {
      if (k0 + i < KS) {
        g += tg[i];
        if constexpr (SWIGLU) u += tu[i];
      }
    }
  }
  if (rowscale != nullptr) {
    g *= rowscale[m];
    u *= rowscale[m];
  }
  uint2 o;
  if constexpr (SWIGLU)
    o = uint2{pack_out2<BF>(silu_mul(g[0], u[0]), silu_mul(g[1], u[1])),
              pack_out2<BF>(silu_mul(g[2], u[2]), silu_mul(g[3], u[3]))};
  else
    o = uint2{pack_out2<BF>(g[0], g[1]), pack_out2<BF>(g[2], g[3])};
  *(uint2 *)(out + (int64_t)m * ldo + n) = o;
}

// ---------------------------------------------------------------------------
// Host side.

hipError_t launch_prefill_reduce(const float *ws, int KS, const Problem &p, hipStream_t s) {
  const int ldo = (int)(p.swiglu ? p.N / 2 : p.N);
  const dim3 grid((unsigned)ceil_div(p.M * (ldo / 4), 256));
  if (p.swiglu) {
    if (p.bf16)
      hipLaunchKernelGGL((prefill_reduce_kernel<true, true>), grid, dim3(256), 0, s, ws, KS,
                         (int)p.M, (int)p.N, p.out, ldo, p.rowscale);
    else
      hipLaunchKernelGGL((prefill_reduce_kernel<true, false>), grid, dim3(256), 0, s, ws, KS,
                         (int)p.M, (int)p.N, p.out, ldo, p.rowscale);
  } else {
    if (p.bf16)
      hipLaunchKernelGGL((prefill_reduce_kernel<false, true>), grid, dim3(256), 0, s, ws, KS,
                         (int)p.M, (int)p.N, p.out, ldo, p.rowscale);
    else
      hipLaunchKernelGGL((prefill_reduce_kernel<false, false>), grid, dim3(256), 0, s, ws, KS,
                         (int)p.M, (int)p.N, p.out, ldo, p.rowscale);
  }
  return hipGetLastError();
}

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
  a.KG8 = (int)ceil_div(groups_of(p.K, p.G), 8);
  a.gshift = p.gshift;
  a.out = p.out;
  a.ldo = (int)(p.swiglu ? p.N / 2 : p.N);
  a.up_off = (int)(p.N / 2 / kStrip);
  a.valid_strips = p.swiglu ? a.up_off : a.NS;
  a.tiles_m = (int)ceil_div(p.M, BM);
  // Each workgroup covers 8 strips (plain) or 4 gate strips + their up strips.
  a.tiles_n = (int)(p.swiglu ? ceil_div(a.up_off, 4) : ceil_div(a.NS, 8));
  a.KS = 1;
  a.nsteps = a.KT;
  a.ws = nullptr;
  a.rowscale = p.rowscale;
  a.rz = (const uint16_t *)p.rz;
  return a;
}

template <int MI, bool DENSE, bool SWIGLU, bool BF>
static hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((prefill_kernel<MI, 2, DENSE, SWIGLU, BF>), dim3(a.tiles_m * a.tiles_n),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int MI, bool DENSE>
static hipError_t launch_prefill_mi(const Problem &p, const PrefillArgs &a, hipStream_t s) {
  if (p.bf16)
    return p.swiglu ? launch_prefill_t<MI, DENSE, true, true>(a, s)
                    : launch_prefill_t<MI, DENSE, false, true>(a, s);
  return p.swiglu ? launch_prefill_t<MI, DENSE, true, false>(a, s)
                  : launch_prefill_t<MI, DENSE, false, false>(a, s);
}

template <bool DENSE>
static hipError_t launch_tiled(const Problem &p, const void *weights, hipStream_t s) {
  // Row tile: 256 rows once M is large, smaller tiles for the transition range.
  const int MI = p.M > 128 ? 8 : (p.M > 64 ? 4 : 2);
  const PrefillArgs a = prefill_args(p, 32 * MI, weights);
  if (MI == 8) return launch_prefill_mi<8, DENSE>(p, a, s);
  if (MI == 4) return launch_prefill_mi<4, DENSE>(p, a, s);
  return launch_prefill_mi<2, DENSE>(p, a, s);
}

static int env_int(const char *name, int fallback) {
  const char *v = std::getenv(name);
  if (v == nullptr || *v == 0) return fallback;
  const int x = std::atoi(v);
  return x > 0 ? x : fallback;
}

// prefill2_kernel addresses every operand with 32-bit buffer offsets.
static bool fits_buffer_offsets(const Problem &p, bool dense) {
  const int64_t limit = (int64_t)1 << 31;
  const int64_t ns = ceil_div(p.N, kStrip);
  return p.M * p.K * 2 < limit &&
         ns * (p.K / kTileK) * 1024 * (dense ? 4 : (p.bits == 8 ? 2 : 1)) < limit &&
         ns * ceil_div(groups_of(p.K, p.G), 8) * 512 < limit && p.M * p.N * 4 < limit;
}

// Compute units of the current device (256 on MI355X), cached per device.
static int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Launch shape of prefill2_kernel: rows per workgroup tile (64, 128 or 256),
// 64-k tiles per pipeline step, and K slices.
struct Prefill2Config {
  int bm, tps, ks, tiles;
  int wm;  // waves along the rows: 2 (4 along the columns) or 1 (8 along the columns)
  int mi() const { return bm / (32 * wm); }   // 32-row MFMA blocks per wave
  int wnw() const { return 8 / wm; }          // waves along the columns
};

// K slices for a grid of `tiles` workgroups: halve each workgroup's k range
// while the doubled grid still fits one workgroup per CU (at most 16 slices,
// at least 4 pipeline steps each; slices may differ by one step).
static int k_slices(int64_t tiles, int nsteps, int cus) {
  int ks = 1;
  while (tiles * ks * 2 <= cus && ks < 16 && nsteps / (2 * ks) >= 4) ks *= 2;
  return ks;
}

// false: the one-wave kernel (prefill_kernel) runs instead.  The fused path
// takes prefill2_kernel unless an operand is too large for 32-bit offsets (a
// logged fallback) or W4A16_PREFILL_V2=0.  The dense tier keeps the one-wave
// kernel unless W4A16_PREFILL_V2=1: on its fp16 weights (four 16-byte vectors
// per lane and 64-k tile) the 8-wave mainloop measured 482-488 TFLOP/s at
// M = 16384 on MI355X against 700 or more for the one-wave mainloop, whose
// 512 registers hold those vectors.
//
// Tile rows (64, 128 or 256) come from a small time model fitted to
// measurements on MI355X: a workgroup of a BM-row tile over a k range of
// K/ks runs at eff(BM) x 4.5 TFLOP/s (eff = 0.6, 0.85, 1.0: smaller tiles
// reuse each dequantized weight fragment less), the grid runs in
// ceil(workgroups / CUs) rounds, and a split K adds the round trip of the
// FP32 partials through memory (2 ks M N 4 bytes at 5 TB/s) plus ~3 us.  Two
// 64-k tiles (one scale group) per pipeline step: half the barriers of one
// 64-k tile, measured 0-5% faster.  Up to M = 256 the tile is 64 rows with
// the waves as 1 x 8 instead of 2 x 4 (W4A16_PREFILL_WM): two waves then no
// longer dequantize the same weight fragment, which halves the
// dequantization work per MFMA; its 512-column tiles need more K slices to
// fill the GPU.  W4A16_PREFILL_BM, W4A16_PREFILL_TPS and W4A16_PREFILL_KS
// override.
static bool prefill2_config(const Problem &p, bool dense, Prefill2Config &c) {
  const char *v = std::getenv("W4A16_PREFILL_V2");
  const bool on = v != nullptr && *v != 0 ? *v == '1' : !dense;
  if (!on || !fits_buffer_offsets(p, dense)) return false;
  const int cus = device_cus();
  const int64_t NS = ceil_div(p.N, kStrip);
  const int bm_env = env_int("W4A16_PREFILL_BM", 0);
  bool side = false;  // the eight waves side by side along the columns (WM = 1)
  if (dense) {
    c.bm = 256;  // the dense tier always runs the 256-row tile, unsplit
  } else if (bm_env == 64 || bm_env == 128 || bm_env == 256) {
    c.bm = bm_env;
  } else if (p.M > 256) {
    // Large batches: 128 x 512 tiles, each wave 128 rows x 64 columns, so
    // every weight fragment is dequantized once per workgroup and feeds four
    // row blocks.  Measured on MI355X against 256 x 256 tiles with 2 x 4
    // waves (which dequantize each fragment twice), Llama-8B gate/up and down
    // at M = 384-16384: 2-10% faster (M = 4096: 813 against 847 us and 397
    // against 414 us); 64-row tiles side by side and 128-row tiles with 2 x 4
    // waves were slower than both.
    c.bm = 128;
    side = true;
  } else if (p.K <= 8192 || p.M > 128) {
    // Transition batches: 64-row tiles with the eight waves side by side
    // (each wave's dequantized fragments feed all 64 rows), measured 3-16%
    // faster on the K = 4096 projections and at M = 256; the deep, narrow
    // down projection at M <= 128 keeps the 2 x 4 layout, whose smaller tiles
    // need fewer K slices.
    c.bm = 64;
    side = true;
  } else {
    static const double eff[3] = {0.6, 0.85, 1.0};
    const int64_t tn = p.swiglu ? ceil_div(NS / 2, 4) : ceil_div(NS, 8);
    double best = 0.0;
    for (int i = 0; i < 3; ++i) {
      const int bm = 64 << i;
      const int tps = 2;
      const int64_t tiles = ceil_div(p.M, bm) * tn;
      const int ks = k_slices(tiles, (int)(p.K / kTileK / tps), cus);
      const double rounds = (double)ceil_div(tiles * ks, (int64_t)cus);
      double t = rounds * 2.0 * bm * 256.0 * ((double)p.K / ks) / (4.5e12 * eff[i]);
      if (ks > 1) t += 2.0 * ks * (double)p.M * (double)p.N * 4.0 / 5e12 + 3e-6;
      if (i == 0 || t < best) {
        best = t;
        c.bm = bm;
      }
    }
  }
  c.tps = dense ? 1 : env_int("W4A16_PREFILL_TPS", 2) == 2 ? 2 : 1;
  c.wm = side ? 1 : 2;
  const int wm_env = env_int("W4A16_PREFILL_WM", 0);
  if (!dense && c.bm <= 128 && (wm_env == 1 || wm_env == 2)) c.wm = wm_env;
  const int64_t tiles_n = p.swiglu ? ceil_div(NS / 2, c.wnw()) : ceil_div(NS, 2 * c.wnw());
  c.tiles = (int)(ceil_div(p.M, c.bm) * tiles_n);
  const int nsteps = (int)(p.K / kTileK / c.tps);
  int ks = dense ? 1 : k_slices(c.tiles, nsteps, cus);
  const int ks_env = env_int("W4A16_PREFILL_KS", 0);
  if (!dense && ks_env > 0 && ks_env <= nsteps) ks = ks_env;
  c.ks = ks;
  return true;
}

template <int MI, int WM, int TPS, bool DENSE, bool SWIGLU, bool BF, bool ZP, int BITS>
static hipError_t launch_prefill2_t(const Problem &p, const void *weights, const Prefill2Config &c,
                                    void *workspace, hipStream_t s) {
  constexpr int WNW = 8 / WM;
  PrefillArgs a = prefill_args(p, 32 * MI * WM, weights);
  a.tiles_n = (int)(p.swiglu ? ceil_div(a.up_off, WNW) : ceil_div(a.NS, 2 * WNW));
  a.KS = c.ks;
  a.nsteps = a.KT / TPS;
  a.ws = (float *)workspace;
  hipLaunchKernelGGL((prefill2_kernel<MI, WM, WNW, TPS, DENSE, SWIGLU, BF, ZP, BITS>),
                     dim3(a.tiles_m * a.tiles_n * c.ks), dim3(64 * WM * WNW), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || c.ks == 1) return e;
  return launch_prefill_reduce((const float *)workspace, c.ks, p, s);
}

template <int MI, int WM, int TPS, bool DENSE, bool ZP, int BITS>
static hipError_t launch_prefill2_z(const Problem &p, const void *weights,
                                    const Prefill2Config &c, void *ws, hipStream_t s) {
  if (p.bf16)
    return p.swiglu
               ? launch_prefill2_t<MI, WM, TPS, DENSE, true, true, ZP, BITS>(p, weights, c, ws, s)
               : launch_prefill2_t<MI, WM, TPS, DENSE, false, true, ZP, BITS>(p, weights, c, ws, s);
  return p.swiglu
             ? launch_prefill2_t<MI, WM, TPS, DENSE, true, false, ZP, BITS>(p, weights, c, ws, s)
             : launch_prefill2_t<MI, WM, TPS, DENSE, false, false, ZP, BITS>(p, weights, c, ws, s);
}

template <int MI, int WM, int TPS, bool DENSE>
static hipError_t launch_prefill2_tps(const Problem &p, const void *weights,
                                      const Prefill2Config &c, void *ws, hipStream_t s) {
  if constexpr (!DENSE) {
    if (p.bits == 8) return launch_prefill2_z<MI, WM, TPS, DENSE, false, 8>(p, weights, c, ws, s);
    if (p.zp) return launch_prefill2_z<MI, WM, TPS, DENSE, true, 4>(p, weights, c, ws, s);
  }
  return launch_prefill2_z<MI, WM, TPS, DENSE, false, 4>(p, weights, c, ws, s);
}

template <int MI, int WM, bool DENSE>
static hipError_t launch_prefill2_m(const Problem &p, const void *weights, const Prefill2Config &c,
                                    void *ws, hipStream_t s) {
  if constexpr (!DENSE) {
    if (c.tps == 2) return launch_prefill2_tps<MI, WM, 2, DENSE>(p, weights, c, ws, s);
  }
  return launch_prefill2_tps<MI, WM, 1, DENSE>(p, weights, c, ws, s);
}

bool prefill_fused_available(const Problem &p) {
  Prefill2Config c;
  return p.bits == 4 || prefill2_config(p, false, c);
}

int64_t prefill_workspace_bytes(const Problem &p) {
  TransConfig tc;
  if (transition_config(p, tc)) return transition_workspace_bytes(p);
  Prefill2Config c;
  if (!prefill2_config(p, false, c) || c.ks == 1) return 0;
  return (int64_t)c.ks * p.M * p.N * (int64_t)sizeof(float);
}

static const char *kOneWaveFallback =
    "prefill-one-wave: operands beyond the 8-wave kernel's 32-bit offsets (or "
    "W4A16_PREFILL_V2=0), running the one-wave kernel";

hipError_t launch_prefill(const Problem &p, void *workspace, hipStream_t s) {
  TransConfig tc;
  if (transition_config(p, tc)) return launch_transition(p, tc, workspace, s);
  Prefill2Config c;
  if (!prefill2_config(p, false, c)) {
    note_fallback(kOneWaveFallback, "fused prefill");
    return launch_tiled<false>(p, p.rw, s);
  }
  if (c.ks > 1 && workspace == nullptr) return hipErrorInvalidValue;
  if (c.wm == 1)
    return c.bm == 64 ? launch_prefill2_m<2, 1, false>(p, p.rw, c, workspace, s)
                      : launch_prefill2_m<4, 1, false>(p, p.rw, c, workspace, s);
  if (c.bm == 64) return launch_prefill2_m<1, 2, false>(p, p.rw, c, workspace, s);
  if (c.bm == 128) return launch_prefill2_m<2, 2, false>(p, p.rw, c, workspace, s);
  return launch_prefill2_m<4, 2, false>(p, p.rw, c, workspace, s);
}

int tiled_describe(const Problem &p, bool dense, char *buf, size_t n) {
  const char *pre = !dense ? ""
                   : p.bits == 8 ? (p.bf16 ? "dequant8_kernel<false, true>; "
                                           : "dequant8_kernel<false, false>; ")
                                 : (p.bf16 ? "dequant_kernel<false, true>; "
                                           : "dequant_kernel<false, false>; ");
  const char *d = dense ? "true" : "false", *sw = p.swiglu ? "true" : "false";
  const char *bf = p.bf16 ? "true" : "false";
  const char *zp = p.zp && !dense ? "true" : "false";
  TransConfig tc;
  if (!dense && transition_config(p, tc)) return transition_describe(p, tc, buf, n);
  Prefill2Config c;
  if (prefill2_config(p, dense, c)) {
    int k = snprintf(buf, n,
                     "%sprefill2_kernel<%d, %d, %d, %d, %s, %s, %s, %s, %d> workgroups=%d "
                     "threads=512 ks=%d",
                     pre, c.mi(), c.wm, c.wnw(), c.tps, d, sw, bf, zp, dense ? 4 : p.bits,
                     c.tiles * c.ks, c.ks);
    if (c.ks > 1 && k > 0 && (size_t)k < n)
      k += snprintf(buf + k, n - k, "; prefill_reduce_kernel<%s, %s>", sw, bf);
    return k;
  }
  const int MI = p.M > 128 ? 8 : (p.M > 64 ? 4 : 2);
  const PrefillArgs a = prefill_args(p, 32 * MI, nullptr);
  return snprintf(buf, n, "%sprefill_kernel<%d, 2, %s, %s, %s> workgroups=%d threads=256", pre, MI,
                  d, sw, bf, a.tiles_m * a.tiles_n);
}

int64_t dense_workspace_bytes(const Problem &p) {
  // fp16 weights in fragment order: 64 columns x 64 k x 2 bytes per (strip, tile) half.
  return ceil_div(p.N, kStrip) * (p.K / kTileK) * 64 * 4 * 16;
}

hipError_t launch_dense(const Problem &p, void *workspace, hipStream_t s) {
  if (workspace == nullptr) return hipErrorInvalidValue;
  void *w16f = workspace;
  hipError_t e =
      p.bits == 8
          ? launch_dequant8_fragment(p.rw, p.rs, p.K, p.N, p.G, p.bf16, (uint16_t *)w16f, s)
          : launch_dequant_fragment(p.rw, p.rs, p.rz, p.K, p.N, p.G, p.bf16, (uint16_t *)w16f, s);
  if (e != hipSuccess) return e;
  Prefill2Config c;
  if (prefill2_config(p, true, c)) return launch_prefill2_m<4, 2, true>(p, w16f, c, nullptr, s);
  return launch_tiled<true>(p, w16f, s);
}

}  // namespace w4a16
