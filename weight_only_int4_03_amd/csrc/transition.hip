// Transition regime (M from 33 to a few hundred rows): a skinny-tile fused
// W4A16 GEMM.
//
// The product is the page "GPU Kernels for INT4 Inference, in depth"
// (aicassindra.com), section "The job, stated precisely".  The Swordfish page
// (blog.alpindale.net, section "Decode, counting memory-pipe slots") singles
// out the batches between decode and prefill (its M >= 49 regime) as needing
// a scheme of their own: too many rows for a weight-streaming GEMV, too few
// for a prefill tile to fill the GPU without splitting K across workgroups
// (whose FP32 partials then cost as much memory traffic as a good part of
// the weights).
//
// gfx950 mapping.  A workgroup owns BM = 32 * MI rows and WC strip pairs
// (64 columns each: two adjacent strips, or a gate strip and its up strip for
// the SwiGLU epilogue), and 8 waves: WC along the columns times WK along K.
// The K range is walked in rounds of WK groups of 128 k; in each round wave
// (wc, wk) takes group wk of its strip pair, so every weight of the
// workgroup's columns is dequantized exactly once per row tile and the
// workgroup covers its whole K range without splitting it across
// workgroups.  Per round:
//   * the BM x (WK * 128) activation tile goes from memory straight into LDS
//     (buffer loads with an LDS destination, one round ahead, two stages);
//     16-byte chunks are XOR-swizzled by row so that the ds_read_b128 of 16
//     rows never share a bank group;
//   * each wave streams its two strips' packed words (16-byte buffer loads)
//     two rounds ahead into a ring of three register sets, and dequantizes
//     them into MFMA operands in registers (the fp16 group scale applied:
//     exactly the dequantized weight);
//   * v_mfma_f32_32x32x16_f16 with the weights as the first operand (32
//     columns) and the activations as the second (32 rows), MI row blocks per
//     dequantized fragment.
// At the end the WK partial tiles of a column are summed through LDS in wk
// order and wave wk = 0 runs the epilogue.  Where the tiles alone leave CUs
// idle K is still split across workgroups (FP32 partials and the prefill
// path's slice-order reduction kernel), but over far fewer slices than a
// prefill tile needs.
#include <cstdio>
#include <cstdlib>

#include "common.h"

namespace w4a16 {

struct TransArgs {
  const uint16_t *A;
  int M, K;
  const uint4_t *rw;
  const uint16_t *rs;
  const uint16_t *rz;     // prescaled zero rows (laid out as rs), or null
  int N, NS, KT, KG, KG8;
  uint16_t *out;
  int ldo;
  int up_off;             // SwiGLU: strip offset from a gate strip to its up strip
  int npairs;             // strip pairs (SwiGLU: gate strips; plain: ceil(NS / 2))
  int row_tiles, col_groups, KS;
  // Stream-K (upw > 0): the flat work is `units` (tile, round) units, tile by
  // tile (row tile fastest) and round by round; each workgroup takes upw
  // consecutive units.  A tile covered by several workgroups is finished by
  // transition_sk_reduce_kernel from their partials.
  int upw, units, rt_rounds;
  float *ws;              // FP32 partials [slice][M][N]: K slice, or a tile's part in Stream-K
  const float *rowscale;  // per-row output factor, or null
  int gshift;             // group of k = k >> gshift
};

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8) that waits until at most n vector-memory loads are
// outstanding and for nothing else.
constexpr int vm_wait(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// One tile of the transition GEMM: row tile rt, column group cg, over the
// groups [gb, ge) of K, into the output or (slice >= 0) into FP32 partial
// slice `slice` of the workspace.
template <int MI, int WC, int WK, bool SWIGLU, bool BF, bool ZP, int BITS>
__device__ __forceinline__ void transition_tile(const TransArgs &p, const int rt, const int cg,
                                                const int gb, const int ge, const int slice) {
  constexpr int NW = WC * WK, NT = NW * 64;
  static_assert(NW == 8 || NW == 4, "eight or four waves per workgroup");
  constexpr int BM = 32 * MI;
  constexpr int CH = WK * 16;          // 16-byte chunks per staged activation row
  constexpr int AV = BM * CH / NT;     // activation copies per lane and round
  static_assert(BM * CH % NT == 0, "activation tile split");
  constexpr int NV = BITS == 8 ? 2 : 1;               // 16-byte vectors per lane, strip, tile
  constexpr int VSTEP = BITS == 8 ? 1024 : 16;        // bytes between a lane's vectors
  static_assert(BITS == 4 || (BITS == 8 && !ZP), "INT8 weights have no zero rows");
  // The two activation stages are separate arrays so that the compiler can
  // tell the stage being filled from the stage being read; after the main
  // loop they hold the cross-wave reduction.
  __shared__ uint4_t lds0[BM * CH];
  __shared__ uint4_t lds1[BM * CH];
  struct BRegs {
    uint4_t v[2][2][NV];  // [strip][64-k tile][vector]
    uint32_t sc[2][2];    // [strip][tile]: scale bits
    // Zero-row bits, in registers of their own: combined with the scale right
    // after the load, they would make the wave wait for the load there.
    uint32_t zc[ZP ? 2 : 1][2];
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wc = wave % WC, wk = wave / WC;
  const int h = lane >> 5, c = lane & 31;
  const Dequant dq;

  const int m0 = rt * BM;

  const int pair = cg * WC + wc;
  int strip[2];
  bool sval[2];
  if constexpr (SWIGLU) {
    strip[0] = pair;
    strip[1] = pair + p.up_off;
    sval[0] = sval[1] = pair < p.npairs;
  } else {
    strip[0] = 2 * pair;
    strip[1] = 2 * pair + 1;
    sval[0] = strip[0] < p.NS;
    sval[1] = strip[1] < p.NS;
  }

  // R rounds of WK groups.
  const int R = (ge - gb + WK - 1) / WK;

  // Buffer resources.  The activation resources (one per round, below) start
  // at this tile's first row and end at row M, so rows past M read as zero.
  const int arows = p.M - m0 < BM ? p.M - m0 : BM;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void *)p.rw, (short)0, p.NS * p.KT * 1024 * NV, kBufferConfig);
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)p.rs, (short)0, p.NS * p.KG8 * 512, kBufferConfig);
  const __amdgpu_buffer_rsrc_t rzr = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(ZP ? p.rz : p.rs), (short)0, p.NS * p.KG8 * 512, kBufferConfig);

  // Activation staging: copy i of wave `wave` fills the 64 consecutive
  // 16-byte LDS slots from (i * NW + wave) * 64, one per lane.  Slot s holds
  // row s / CH, physical chunk s % CH, which is the logical chunk
  // (s % CH) ^ (row & 15) of the round's WK * 128 k; the XOR stays inside the
  // 16 chunks of one group.  A lane's physical chunk is the same in every
  // copy and its row advances by RPC = NT / CH rows per copy, so its
  // logical chunk takes at most two values (even and odd copies when RPC is
  // 8).  The whole offset (row, k and chunk) goes into the lane offset, which
  // the buffer's range check covers: rows past M, and the k past the end of
  // the last row that a partial last round stages (never consumed), read as
  // zero.
  constexpr int RPC = NT / CH;
  static_assert(RPC == 8 || RPC == 16, "rows per copy");
  const int row0 = (wave * 64 + lane) / CH, ph = (wave * 64 + lane) % CH;
  const int a_even = row0 * p.K * 2 + ((ph ^ (row0 & 15)) * 16);
  const int a_odd = row0 * p.K * 2 + ((ph ^ ((row0 + RPC) & 15)) * 16);
  // The round's k offset moves the resource's base instead of the lane
  // offsets (which stay fixed for the whole loop, so no per-round address
  // registers are written while loads are in flight); the resource shrinks by
  // the same amount, so its range check still ends at row M.
  typedef __attribute__((address_space(3))) void *lds_ptr;
  const char *a_tile = (const char *)(p.A + (int64_t)m0 * p.K);
  const int a_bytes = arows * p.K * 2;
  auto load_a = [&](int r, uint4_t *stage) {
    const int kbyte = (gb + r * WK) * 256;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a_tile + kbyte), (short)0, a_bytes - kbyte, kBufferConfig);
#pragma unroll
    for (int i = 0; i < AV; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (lds_ptr)(stage + (i * NW + wave) * 64), 16,
          ((i & 1) ? a_odd : a_even) + i * RPC * p.K * 2, 0, 0, 0);
  };

  // Weights and scales: invalid strips read strip 0 and are never stored; a
  // wave past the end of the K range reloads its last group (never consumed).
  int w_off[2], s_off[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int st = sval[s] ? strip[s] : 0;
    w_off[s] = st * p.KT * 1024 * NV + lane * 16;
    // Lane half h reads the scale of k + 32 h: with 32-k groups the next
    // group (2 bytes on, never across an octet: the group of the half's
    // first k is even), else the same one; the rest of the offset is the
    // same for the whole wave and goes into the scalar offset.
    s_off[s] = (st * p.KG8 * 32 + c) * 16 + (p.gshift == 5 ? 2 * h : 0);
  }
  auto load_b = [&](int r, BRegs &regs) {
    int grp = gb + r * WK + wk;
    grp = grp < ge ? grp : ge - 1;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < NV; ++j)
          regs.v[s][t][j] = bitcast<uint4_t>(__builtin_amdgcn_raw_buffer_load_b128(
              rw, w_off[s] + VSTEP * j, (2 * grp + t) * 1024 * NV, kBufferNT));
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int g = (128 * grp + 64 * t) >> p.gshift;
      const int g_off = (g >> 3) * 512 + (g & 7) * 2;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        regs.sc[s][t] = __builtin_amdgcn_raw_buffer_load_b16(rsc, s_off[s], g_off, 0);
        if constexpr (ZP)
          regs.zc[s][t] = __builtin_amdgcn_raw_buffer_load_b16(rzr, s_off[s], g_off, 0);
      }
    }
  };

  float16_t acc[2][MI];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < MI; ++i) acc[s][i] = float16_t{};

  auto compute = [&](const uint4_t *stage, const BRegs &regs) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4_t bf[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const uint16_t s16 = (uint16_t)regs.sc[s][t];
          if constexpr (BITS == 8) {
            const uint4_t &v = regs.v[s][t][j >> 1];
            bf[s] = dq.scaled8_bits<BF>(v[(j & 1) * 2], v[(j & 1) * 2 + 1], s16);
          } else if constexpr (ZP) {
            bf[s] = dq.scaled_bits<BF, true>(regs.v[s][t][0][j], s16,
                                             (uint16_t)regs.zc[s][t]);
          } else if constexpr (BF) {
            bf[s] = bitcast<uint4_t>(dq.scaled_bf16(regs.v[s][t][0][j], Dequant::BScale(s16)));
          } else {
            const _Float16 sh = bitcast<_Float16>(s16);
            bf[s] = bitcast<uint4_t>(dq.scaled(regs.v[s][t][0][j], half2_t{sh, sh}));
          }
        }
        const int chunk = 16 * wk + 8 * t + 4 * h + j;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int row = 32 * i + c;
          const uint4_t af = stage[row * CH + (chunk ^ (row & 15))];
#pragma unroll
          for (int s = 0; s < 2; ++s) acc[s][i] = mfma32<BF>(bf[s], af, acc[s][i]);
        }
      }
    }
  };

  // Round r: issue the activations of round r + 1 (into the idle stage) and
  // the weights of round r + 2 (into the register set that round r - 1
  // used), keep those loads ahead of the round's MFMAs, compute, then meet
  // the workgroup barrier, which waits for the activation loads (issued
  // before the weights, so the weights stay in flight for two rounds).
  // Loads past the last round reload the last round (never consumed).
  auto round = [&](int r, const uint4_t *cur_stage, uint4_t *next_stage, const BRegs &cur,
                   BRegs &ahead) {
    load_a(r + 1 < R ? r + 1 : R - 1, next_stage);
    load_b(r + 2 < R ? r + 2 : R - 1, ahead);
    __builtin_amdgcn_sched_barrier(0);
    if (gb + r * WK + wk < ge) compute(cur_stage, cur);
    __syncthreads();
  };
  BRegs b0, b1, b2;
  load_a(0, lds0);
  load_b(0, b0);
  __builtin_amdgcn_sched_barrier(0);
  load_b(R > 1 ? 1 : 0, b1);
  __builtin_amdgcn_sched_barrier(0);
  // Enter the loop in its steady state: round 0's activations and weights
  // complete, only round 1's weights (the last eight loads) in flight.  (Left
  // to itself the compiler merges the entry state, with round 0's weights
  // still pending, into every iteration and then waits inside each round for
  // loads issued a round early.)
  __builtin_amdgcn_s_waitcnt(vm_wait(4 * NV + (ZP ? 8 : 4)));
  __syncthreads();
  // Three register sets and two stages: six rounds per iteration, then up to
  // five more after the loop.  (With the early exits inside the loop the
  // compiler merges their pending loads into the loop head and waits there,
  // every iteration, for weights issued a round early.)
  int r = 0;
  for (; r + 6 <= R; r += 6) {
    round(r, lds0, lds1, b0, b2);
    round(r + 1, lds1, lds0, b1, b0);
    round(r + 2, lds0, lds1, b2, b1);
    round(r + 3, lds1, lds0, b0, b2);
    round(r + 4, lds0, lds1, b1, b0);
    round(r + 5, lds1, lds0, b2, b1);
  }
  if (r < R) {
    round(r, lds0, lds1, b0, b2);
    if (r + 1 < R) {
      round(r + 1, lds1, lds0, b1, b0);
      if (r + 2 < R) {
        round(r + 2, lds0, lds1, b2, b1);
        if (r + 3 < R) {
          round(r + 3, lds1, lds0, b0, b2);
          if (r + 4 < R) round(r + 4, lds0, lds1, b1, b0);
        }
      }
    }
  }

  // Cross-wave sum over wk: waves wk >= 1 write their tiles (one float4 per
  // lane and instruction, 1 KiB contiguous per wave-wide store), wave wk = 0
  // adds them in wk order.  Slot q = (wk - 1) * WC + wc holds MI * 8 KiB;
  // the first SPS slots go to stage 0, the rest to stage 1.
  constexpr int SLOT = 2 * MI * 4 * 64;               // float4 per slot
  constexpr int SPS = BM * CH / SLOT;                 // slots per stage
  static_assert((WK - 1) * WC <= 2 * SPS, "reduction fits in the two stages");
  auto slot_ptr = [&](int q) {
    return (float4_t *)(q < SPS ? lds0 : lds1) + (q % SPS) * SLOT;
  };
  if (wk > 0) {
    float4_t *dst = slot_ptr((wk - 1) * WC + wc);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dst[((s * MI + i) * 4 + e) * 64 + lane] =
              float4_t{acc[s][i][4 * e], acc[s][i][4 * e + 1], acc[s][i][4 * e + 2],
                       acc[s][i][4 * e + 3]};
  }
  __syncthreads();
  if (wk > 0) return;
#pragma unroll
  for (int k = 1; k < WK; ++k) {
    const float4_t *src = slot_ptr((k - 1) * WC + wc);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float4_t v = src[((s * MI + i) * 4 + e) * 64 + lane];
#pragma unroll
          for (int x = 0; x < 4; ++x) acc[s][i][4 * e + x] += v[x];
        }
  }

  // acc[s][i][4*rg + e] is the output at row m0 + 32 i + c and column
  // 32 strip[s] + 8 rg + 4 h + e.
  if (slice >= 0) {
    float *part = p.ws + (int64_t)slice * p.M * p.N;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = m0 + 32 * i + c;
      if (m >= p.M) continue;
      float *prow = part + (int64_t)m * p.N;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (!sval[s]) continue;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int n = strip[s] * 32 + 8 * rg + 4 * h;
          if (n >= p.N) continue;
          *(float4_t *)(prow + n) = float4_t{acc[s][i][4 * rg + 0], acc[s][i][4 * rg + 1],
                                             acc[s][i][4 * rg + 2], acc[s][i][4 * rg + 3]};
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int m = m0 + 32 * i + c;
    if (m >= p.M) continue;
    uint16_t *orow = p.out + (int64_t)m * p.ldo;
    const float rs = p.rowscale != nullptr ? p.rowscale[m] : 1.0f;
    if constexpr (SWIGLU) {
      if (!sval[0]) continue;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const float16_t &g = acc[0][i], &u = acc[1][i];
        const int n = strip[0] * 32 + 8 * rg + 4 * h;
        *(uint2 *)(orow + n) =
            uint2{pack_out2<BF>(silu_mul(rs * g[4 * rg + 0], rs * u[4 * rg + 0]),
                                silu_mul(rs * g[4 * rg + 1], rs * u[4 * rg + 1])),
                  pack_out2<BF>(silu_mul(rs * g[4 * rg + 2], rs * u[4 * rg + 2]),
                                silu_mul(rs * g[4 * rg + 3], rs * u[4 * rg + 3]))};
      }
    } else {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (!sval[s]) continue;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int n = strip[s] * 32 + 8 * rg + 4 * h;
          if (n >= p.N) continue;
          const float16_t &v = acc[s][i];
          *(uint2 *)(orow + n) = uint2{pack_out2<BF>(rs * v[4 * rg + 0], rs * v[4 * rg + 1]),
                                       pack_out2<BF>(rs * v[4 * rg + 2], rs * v[4 * rg + 3])};
        }
      }
    }
  }
}

template <int MI, int WC, int WK, bool SWIGLU, bool BF, bool ZP, int BITS>
__global__ __launch_bounds__(WC * WK * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void transition_kernel(TransArgs p) {
  // XCD-aware walk: workgroup ids are dealt round-robin over the 8 XCDs; each
  // XCD takes a contiguous range of (row tile, column group, K slice) triples
  // with the row tile fastest, so the row tiles that read the same weights
  // run together on one XCD's L2.
  const int T = p.row_tiles * p.col_groups * p.KS;
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int per = T >> 3, extra = T & 7;
  const int tau = xcd * per + (xcd < extra ? xcd : extra) + local;
  const int rt = tau % p.row_tiles;
  const int rest = tau / p.row_tiles;
  const int cg = rest % p.col_groups, ks = rest / p.col_groups;
  // K slice of this workgroup: groups [gb, ge).
  transition_tile<MI, WC, WK, SWIGLU, BF, ZP, BITS>(
      p, rt, cg, (int)((int64_t)p.KG * ks / p.KS), (int)((int64_t)p.KG * (ks + 1) / p.KS),
      p.KS > 1 ? ks : -1);
}

// Stream-K form (the Swordfish page, "Decode, counting memory-pipe slots": a
// persistent kernel over flat (tile, k-slice) units for the batches above
// M = 48): one workgroup per CU, each taking p.upw consecutive (tile, round)
// units, tile by tile.  A tile whose units all fall in one workgroup's range
// is finished there; otherwise each workgroup's share goes to partial slice
// (workgroup - the tile's first workgroup) and transition_sk_reduce_kernel
// adds the slices in that order.  The pages flush with atomic adds into the
// output instead; the slices keep the sum deterministic.
template <int MI, int WC, int WK, bool SWIGLU, bool BF, bool ZP, int BITS>
__global__ __launch_bounds__(WC * WK * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void transition_sk_kernel(TransArgs p) {
  // The workgroups' unit ranges are dealt by the same XCD-aware walk.
  const int T = (int)gridDim.x;
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int per = T >> 3, extra = T & 7;
  const int tau = xcd * per + (xcd < extra ? xcd : extra) + local;
  const int u0 = tau * p.upw;
  const int u1 = u0 + p.upw < p.units ? u0 + p.upw : p.units;
  for (int u = u0; u < u1;) {
    const int t = u / p.rt_rounds, r0 = u - t * p.rt_rounds;
    const int len = p.rt_rounds - r0 < u1 - u ? p.rt_rounds - r0 : u1 - u;
    const int first = t * p.rt_rounds / p.upw, last = ((t + 1) * p.rt_rounds - 1) / p.upw;
    const int ge = (r0 + len) * WK < p.KG ? (r0 + len) * WK : p.KG;
    // The previous tile's cross-wave sum (in the stages) has been read.
    if (u != u0) __syncthreads();
    transition_tile<MI, WC, WK, SWIGLU, BF, ZP, BITS>(p, t % p.row_tiles, t / p.row_tiles,
                                                      r0 * WK, ge,
                                                      first == last ? -1 : tau - first);
    u += len;
  }
}

// Second stage of a Stream-K launch: the tiles that several workgroups
// shared.  Each thread takes 4 consecutive outputs of a row, finds its tile
// and the workgroups that covered it, and (if more than one) sums their
// partial slices in order (the tile's first K units first) and runs the
// epilogue; a tile one workgroup covered was finished by that workgroup.
template <bool SWIGLU, bool BF>
__global__ __launch_bounds__(256) void transition_sk_reduce_kernel(TransArgs p, int BM, int WC) {
  const int per_row = p.ldo >> 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)p.M * per_row) return;
  const int m = (int)(idx / per_row), n = (int)(idx - (int64_t)m * per_row) * 4;
  const int pair = SWIGLU ? n / 32 : n / 64;
  const int t = (pair / WC) * p.row_tiles + m / BM;
  const int first = t * p.rt_rounds / p.upw, last = ((t + 1) * p.rt_rounds - 1) / p.upw;
  if (first == last) return;
  const int parts = last - first + 1;
  const int64_t slice = (int64_t)p.M * p.N;
  const float *src = p.ws + (int64_t)m * p.N + n;
  // The partials of up to eight parts are loaded before any is added, so
  // their memory latencies overlap; they are added in part order.
  float4_t g = {0.0f, 0.0f, 0.0f, 0.0f}, u = {0.0f, 0.0f, 0.0f, 0.0f};
  constexpr int B = 8;
  for (int k0 = 0; k0 < parts; k0 += B) {
    float4_t tg[B], tu[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      if (k0 + i < parts) {
        tg[i] = *(const float4_t *)(src + (k0 + i) * slice);
        if constexpr (SWIGLU) tu[i] = *(const float4_t *)(src + (k0 + i) * slice + p.N / 2);
      }
    }
#pragma unroll
    for (int i = 0; i < B; ++i) {
      if (k0 + i < parts) {
        g = k0 + i == 0 ? tg[i] : g + tg[i];
        if constexpr (SWIGLU) u = k0 + i == 0 ? tu[i] : u + tu[i];
      }
    }
  }
  if (p.rowscale != nullptr) {
    g *= p.rowscale[m];
    u *= p.rowscale[m];
  }
  uint2 o;
  if constexpr (SWIGLU)
    o = uint2{pack_out2<BF>(silu_mul(g[0], u[0]), silu_mul(g[1], u[1])),
              pack_out2<BF>(silu_mul(g[2], u[2]), silu_mul(g[3], u[3]))};
  else
    o = uint2{pack_out2<BF>(g[0], g[1]), pack_out2<BF>(g[2], g[3])};
  *(uint2 *)(p.out + (int64_t)m * p.ldo + n) = o;
}

static hipError_t launch_sk_reduce(const Problem &p, const TransArgs &a, int BM, int WC,
                                   hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(p.M * (a.ldo / 4), 256));
  const dim3 block(256);
  if (p.swiglu) {
    if (p.bf16)
      hipLaunchKernelGGL((transition_sk_reduce_kernel<true, true>), grid, block, 0, s, a, BM, WC);
    else
      hipLaunchKernelGGL((transition_sk_reduce_kernel<true, false>), grid, block, 0, s, a, BM, WC);
  } else {
    if (p.bf16)
      hipLaunchKernelGGL((transition_sk_reduce_kernel<false, true>), grid, block, 0, s, a, BM, WC);
    else
      hipLaunchKernelGGL((transition_sk_reduce_kernel<false, false>), grid, block, 0, s, a, BM, WC);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host side.

static int env_int(const char *name, int fallback) {
  const char *v = std::getenv(name);
  if (v == nullptr || *v == 0) return fallback;
  const int x = std::atoi(v);
  return x > 0 ? x : fallback;
}

static int device_cus_t() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Rows above which the prefill tiles take over from the transition kernel.
constexpr int64_t kTransitionMaxM = 256;

// Launch shape: MI (rows per tile / 32), the wave split, row tiles, column
// groups and K slices.  Measured on MI355X over M = 48 .. 512 on the
// Llama-8B gate/up (4096 x 28672) and down (14336 x 4096) projections:
// 64-row tiles (MI = 2, four waves along K) wherever their grid fits one
// workgroup per CU, else 128-row tiles (MI = 4, two waves along K: the
// 64 KiB activation stage holds 128 rows of two groups); K is then split
// while the split grid still fits one workgroup per CU and each slice keeps
// at least two rounds (a larger grid runs in two passes and was slower in
// every measured case, despite the partial traffic it avoids).  Up to
// M = 256 this beats the prefill tiles (gate/up M = 64: 27.5 against
// 36.6 us; down M = 64: 24.5 against 26.9 us; down M = 256: 44.1 against
// 48.5 us); above it the prefill tiles win.
// W4A16_TRANSITION (0 or 1), W4A16_TRANSITION_MI (2 or 4) and
// W4A16_TRANSITION_KS override; any W4A16_PREFILL_* override (V2, BM, WM,
// TPS, KS) selects the prefill kernels unless W4A16_TRANSITION=1.
bool transition_config(const Problem &p, TransConfig &c) {
  const char *v = std::getenv("W4A16_TRANSITION");
  const bool forced = v != nullptr && *v == '1';
  if (v != nullptr && *v == '0') return false;
  if (!forced && (p.M <= 32 || p.M > kTransitionMaxM)) return false;
  // An override of the prefill kernel's configuration selects that kernel.
  if (!forced)
    for (const char *name : {"W4A16_PREFILL_V2", "W4A16_PREFILL_BM", "W4A16_PREFILL_WM",
                             "W4A16_PREFILL_TPS", "W4A16_PREFILL_KS"}) {
      const char *x = std::getenv(name);
      if (x != nullptr && *x != 0) return false;
    }
  // 32-bit buffer offsets of every operand.
  const int64_t limit = (int64_t)1 << 31;
  const int64_t ns = ceil_div(p.N, kStrip);
  if (!(p.M * p.K * 2 < limit && ns * (p.K / kTileK) * 1024 * (p.bits == 8 ? 2 : 1) < limit &&
        ns * ceil_div(groups_of(p.K, p.G), 8) * 512 < limit && p.M * p.N * 4 < limit))
    return false;
  const int cus = device_cus_t();
  const int64_t npairs = p.swiglu ? p.N / 64 : ceil_div(ns, 2);
  const int64_t tiles2 = ceil_div(p.M, 64) * ceil_div(npairs, 2);
  c.mi = tiles2 <= cus ? 2 : 4;
  const int mi_env = env_int("W4A16_TRANSITION_MI", 0);
  if (mi_env == 2 || mi_env == 4) c.mi = mi_env;
  // The 128-row tile fills the registers with INT4 weights and symmetric
  // scales; INT8 weights (two vectors per lane and tile) and zero rows take
  // the 64-row tile, and leave to the prefill tiles the batches whose 64-row
  // grid would exceed two workgroups per CU (INT8 gate/up at M = 256: 106.6
  // against 84.3 us for the eight-wave tiles; at M = 192 the four-wave tiles
  // tie with the prefill tile for INT8 and lose 4% with zero rows).
  if (p.bits == 8 || p.zp) {
    if (!forced && tiles2 > 2 * cus) return false;
    c.mi = 2;
  }
  c.wk = c.mi == 2 ? 4 : 2;
  c.wc = 8 / c.wk;
  // Four-wave workgroups (64-row tiles): two waves along N and two along K
  // and a 32 KiB activation stage, so two workgroups share a CU and one
  // computes while the other waits at its round barrier; the grid then fills
  // two slots per CU.  Taken where the 64-row grid exceeds one workgroup per
  // CU but fits two, with no K split: measured on MI355X (bench.py --sweep
  // transition, transition_int8, transition_zp) on the Llama-8B gate/up
  // projection at M = 96 and 128, INT4: 41.6 and 44.4 against 46.9 and
  // 51.4 us for the 128-row tiles (prefill tile 47.7 and 50.0); INT8: 51.6 and 54.2 against 55.5 and
  // 59.3 us, zero rows: 45.9 and 48.5 against 50.8 and 53.2 us for the
  // prefill tile.  Where the four-wave grid needs a K split (down
  // projections, gate/up at M <= 64) or two passes (M >= 192) it was 3-21%
  // slower.  W4A16_TRANSITION_WAVES (4 or 8) forces the choice.
  int slots = cus;
  const int waves_env = env_int("W4A16_TRANSITION_WAVES", 0);
  const bool four = waves_env == 4 || (waves_env == 0 && mi_env == 0 && tiles2 > cus &&
                                       tiles2 <= 2 * cus);
  if (four) {
    c.mi = 2;
    c.wk = 2;
    c.wc = 2;
    slots = 2 * cus;
  }
  c.col_groups = (int)ceil_div(npairs, c.wc);
  c.row_tiles = (int)ceil_div(p.M, 32 * c.mi);
  const int64_t tiles = (int64_t)c.row_tiles * c.col_groups;
  const int64_t KG = p.K / kGroup;
  c.ks = 1;
  while (c.ks < 16 && tiles * c.ks * 2 <= slots && KG / (c.ks * 2) >= 2 * c.wk) c.ks *= 2;
  const int ks_env = env_int("W4A16_TRANSITION_KS", 0);
  if (ks_env > 0) c.ks = (int)(ks_env < KG ? ks_env : KG);
  c.tiles = (int)(tiles * c.ks);
  c.sk_upw = 0;
  c.sk_parts = 1;
  // Stream-K (W4A16_TRANSITION_SK=1; INT4 weights without zero rows): the
  // (tile, round) units dealt evenly, upw consecutive units per workgroup,
  // one workgroup per CU.  Not the default: measured on MI355X (bench.py
  // --sweep transition, three runs on two boxes) it wins only on the
  // Llama-8B down projection at M = 128 (1.0-1.4 us of 31) and within
  // 0.1-0.5 us at M = 48 and 64; with the same K partition as the tiles'
  // split (M = 96, 256) its walk order costs 0.4-1.7 us, where it shares
  // tiles among more workgroups than the split (M = 192) 7 us, and where the
  // tiles need no split (gate/up: every tile then writes two partial slices)
  // 8-11 us.
  if (p.bits == 4 && !p.zp) {
    const int64_t rounds = ceil_div(KG, c.wk), units = tiles * rounds;
    const int64_t upw = ceil_div(units, cus);
    int parts = 1;
    for (int64_t t = 0; t < tiles; ++t) {
      const int64_t n = ((t + 1) * rounds - 1) / upw - t * rounds / upw + 1;
      if (n > parts) parts = (int)n;
    }
    const char *sk = std::getenv("W4A16_TRANSITION_SK");
    if (sk != nullptr && *sk == '1') {
      c.ks = 1;
      c.sk_rounds = (int)rounds;
      c.sk_units = (int)units;
      c.sk_upw = (int)upw;
      c.sk_parts = parts;
      c.tiles = (int)ceil_div(units, upw);
    }
  }
  return true;
}

int64_t transition_workspace_bytes(const Problem &p) {
  TransConfig c;
  if (!transition_config(p, c)) return 0;
  const int64_t slices = c.sk_upw > 0 ? c.sk_parts : c.ks;
  return slices > 1 ? slices * p.M * p.N * (int64_t)sizeof(float) : 0;
}

int transition_describe(const Problem &p, const TransConfig &c, char *buf, size_t n) {
  const char *sw = p.swiglu ? "true" : "false", *bf = p.bf16 ? "true" : "false";
  int k = snprintf(buf, n,
                   "%s<%d, %d, %d, %s, %s, %s, %d> workgroups=%d threads=%d ks=%d",
                   c.sk_upw > 0 ? "transition_sk_kernel" : "transition_kernel", c.mi, c.wc,
                   c.wk, sw, bf, p.zp ? "true" : "false", p.bits, c.tiles, c.wc * c.wk * 64, c.ks);
  if (c.sk_upw > 0 && k > 0 && (size_t)k < n) {
    k += snprintf(buf + k, n - k, " stream-k units=%d per_workgroup=%d", c.sk_units, c.sk_upw);
    if (c.sk_parts > 1 && k > 0 && (size_t)k < n)
      k += snprintf(buf + k, n - k, "; transition_sk_reduce_kernel<%s, %s>", sw, bf);
    return k;
  }
  if (c.ks > 1 && k > 0 && (size_t)k < n)
    k += snprintf(buf + k, n - k, "; prefill_reduce_kernel<%s, %s>", sw, bf);
  return k;
}

template <int MI, int WC, int WK, bool SWIGLU, bool BF, bool ZP, int BITS>
static hipError_t launch_transition_t(const Problem &p, const TransConfig &c, void *ws,
                                      hipStream_t s) {
  TransArgs a;
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
  a.out = p.out;
  a.ldo = (int)(p.swiglu ? p.N / 2 : p.N);
  a.up_off = (int)(p.N / 2 / kStrip);
  a.npairs = (int)(p.swiglu ? p.N / 64 : ceil_div(a.NS, 2));
  a.row_tiles = c.row_tiles;
  a.col_groups = c.col_groups;
  a.KS = c.ks;
  a.upw = c.sk_upw;
  a.units = c.sk_units;
  a.rt_rounds = c.sk_rounds;
  a.ws = (float *)ws;
  a.rowscale = p.rowscale;
  a.gshift = p.gshift;
  if constexpr (BITS == 4 && !ZP) {
    if (c.sk_upw > 0) {
      hipLaunchKernelGGL((transition_sk_kernel<MI, WC, WK, SWIGLU, BF, ZP, BITS>),
                         dim3(c.tiles), dim3(WC * WK * 64), 0, s, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess || c.sk_parts == 1) return e;
      return launch_sk_reduce(p, a, 32 * MI, WC, s);
    }
  }
  if (c.sk_upw > 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((transition_kernel<MI, WC, WK, SWIGLU, BF, ZP, BITS>), dim3(c.tiles),
                     dim3(WC * WK * 64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || c.ks == 1) return e;
  return launch_prefill_reduce((const float *)ws, c.ks, p, s);
}

template <int MI, bool BF, bool ZP, int BITS>
static hipError_t launch_transition_sw(const Problem &p, const TransConfig &c, void *ws,
                                       hipStream_t s) {
  constexpr int WK = MI == 2 ? 4 : 2, WC = 8 / WK;
  return p.swiglu ? launch_transition_t<MI, WC, WK, true, BF, ZP, BITS>(p, c, ws, s)
                  : launch_transition_t<MI, WC, WK, false, BF, ZP, BITS>(p, c, ws, s);
}

template <int MI>
static hipError_t launch_transition_mi(const Problem &p, const TransConfig &c, void *ws,
                                       hipStream_t s) {
  if (p.bits == 8)
    return p.bf16 ? launch_transition_sw<MI, true, false, 8>(p, c, ws, s)
                  : launch_transition_sw<MI, false, false, 8>(p, c, ws, s);
  if (p.zp)
    return p.bf16 ? launch_transition_sw<MI, true, true, 4>(p, c, ws, s)
                  : launch_transition_sw<MI, false, true, 4>(p, c, ws, s);
  return p.bf16 ? launch_transition_sw<MI, true, false, 4>(p, c, ws, s)
                : launch_transition_sw<MI, false, false, 4>(p, c, ws, s);
}

hipError_t launch_transition(const Problem &p, const TransConfig &c, void *ws, hipStream_t s) {
  if ((c.ks > 1 || c.sk_parts > 1) && ws == nullptr) return hipErrorInvalidValue;
  if (c.wc * c.wk == 4) {
    if (c.mi != 2) return hipErrorInvalidValue;
    if (p.bits == 8)
      return p.swiglu ? (p.bf16 ? launch_transition_t<2, 2, 2, true, true, false, 8>(p, c, ws, s)
                                : launch_transition_t<2, 2, 2, true, false, false, 8>(p, c, ws, s))
                      : (p.bf16 ? launch_transition_t<2, 2, 2, false, true, false, 8>(p, c, ws, s)
                                : launch_transition_t<2, 2, 2, false, false, false, 8>(p, c, ws, s));
    if (p.zp)
      return p.swiglu ? (p.bf16 ? launch_transition_t<2, 2, 2, true, true, true, 4>(p, c, ws, s)
                                : launch_transition_t<2, 2, 2, true, false, true, 4>(p, c, ws, s))
                      : (p.bf16 ? launch_transition_t<2, 2, 2, false, true, true, 4>(p, c, ws, s)
                                : launch_transition_t<2, 2, 2, false, false, true, 4>(p, c, ws, s));
    if (p.swiglu)
      return p.bf16 ? launch_transition_t<2, 2, 2, true, true, false, 4>(p, c, ws, s)
                    : launch_transition_t<2, 2, 2, true, false, false, 4>(p, c, ws, s);
    return p.bf16 ? launch_transition_t<2, 2, 2, false, true, false, 4>(p, c, ws, s)
                  : launch_transition_t<2, 2, 2, false, false, false, 4>(p, c, ws, s);
  }
  if (c.mi == 4 && p.bits == 4 && !p.zp)
    return p.bf16 ? launch_transition_sw<4, true, false, 4>(p, c, ws, s)
                  : launch_transition_sw<4, false, false, 4>(p, c, ws, s);
  if (c.mi != 2) return hipErrorInvalidValue;
  return launch_transition_mi<2>(p, c, ws, s);
}

}  // namespace w4a16
