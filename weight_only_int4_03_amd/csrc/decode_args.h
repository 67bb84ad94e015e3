// Decode-path definitions shared by decode.hip and decode_coop.hip
// (internal, not part of the ABI).
#pragma once

#include "common.h"

namespace w4a16 {

// LDS one workgroup may allocate on gfx950 (the CU's 160 KiB).
constexpr size_t kMaxLdsPerWorkgroup = 160 * 1024;

struct DecodeArgs {
  const uint16_t *A;
  int M, K;
  const uint4_t *rw;
  const uint16_t *rs;
  const uint16_t *rz;  // prescaled zero rows (laid out as rs), or null
  int N, NS, KT, KG, KG8;
  uint16_t *out;
  int ldo;
  int KS;            // workgroups per strip group (K splits)
  int nsg;           // strip groups
  int up_off;        // SwiGLU: strip offset from a gate strip to its up strip
  int valid_strips;  // plain: NS; SwiGLU: number of gate strips
  float *ws;         // KS > 1: partial tiles [nsg][KS][SPW][M][32]
  unsigned long long *xs;  // KS > 1, finished in the launch: exchange slots (all zero), or null
  unsigned *sync;    // KS > 1, finished in the launch by the last workgroup: counters (zero)
  const float *rowscale;  // per-row output factor, or null
  int gshift;        // group of k = k >> gshift (KG counts 128-k units, KG8 scale octets)
  int stagger;       // nonzero: K order rotated by an offset hashed from the workgroup index
};

// Epilogue of one element e of strip group sg's tile (tile element order
// [s][m][c]; for SwiGLU e covers the gate half only and e + SH*M*32 is the
// matching up element).  value_at(e) is the complete FP32 dot product.
template <int SPW, bool SWIGLU, bool BF, typename F>
__device__ __forceinline__ void decode_epilogue(const DecodeArgs &p, int sg, int e, F value_at) {
  constexpr int SH = SWIGLU ? SPW / 2 : SPW;
  const int M = p.M;
  const int s = e / (M * 32), rem = e - s * M * 32;
  const int m = rem >> 5, c = rem & 31;
  const float rs = p.rowscale != nullptr ? p.rowscale[m] : 1.0f;
  if constexpr (SWIGLU) {
    const int gstrip = sg * SH + s;
    if (gstrip < p.valid_strips) {
      const float gv = value_at(e) * rs, uv = value_at(e + SH * M * 32) * rs;
      p.out[(int64_t)m * p.ldo + gstrip * 32 + c] = to_out_bits<BF>(silu_mul(gv, uv));
    }
  } else {
    const int col = (sg * SPW + s) * 32 + c;
    if (col < p.N) p.out[(int64_t)m * p.ldo + col] = to_out_bits<BF>(value_at(e) * rs);
  }
}

// Split-K finish inside the launch.  The KS partial sums of one output
// element meet in a fixed binary tree: at each level the two partners swap
// their value into the same 64-bit slot with one device-scope atomic
// exchange.  The partner that finds the slot empty (zero) is done; the other
// one now holds both values, adds them (fp32 addition is commutative, so
// the sum has the same bits whichever partner came second), clears the slot
// for the next call, and goes up a level.  No workgroup waits for another and
// no fence is needed: the value travels inside the atomic.  Each thread
// carries up to EPT elements (live[i]); on return live[i] is true where this
// thread ends with the complete sum in v[i] (and u[i]).  A slot holds
// (~v, u): v is made a canonical NaN if it is any NaN, so the low word is
// never zero.  Slots: level by level, floor(n/2) per level for n partners;
// element elem of slot j lives at xs[j * stride + elem].
template <int EPT>
__device__ __forceinline__ void split_exchange(unsigned long long *xs, int KS, int split,
                                               int64_t stride, const int64_t (&elem)[EPT],
                                               bool (&live)[EPT], float (&v)[EPT],
                                               float (&u)[EPT]) {
  int idx = split, n = KS;
  int64_t base = 0;
  while (n > 1) {
    const int pairs = n >> 1;
    if (idx < 2 * pairs) {
      // All of this thread's exchanges are in flight before any is waited for.
      unsigned long long got[EPT];
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        if (!live[i]) continue;
        v[i] = v[i] == v[i] ? v[i] : __builtin_nanf("");
        const unsigned long long mine =
            ((unsigned long long)__builtin_bit_cast(uint32_t, u[i]) << 32) |
            (uint32_t)~__builtin_bit_cast(uint32_t, v[i]);
        got[i] = __hip_atomic_exchange(xs + (base + (idx >> 1)) * stride + elem[i], mine,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        if (!live[i]) continue;
        if (got[i] == 0) {
          live[i] = false;
          continue;
        }
        v[i] = v[i] + __builtin_bit_cast(float, ~(uint32_t)got[i]);
        u[i] = u[i] + __builtin_bit_cast(float, (uint32_t)(got[i] >> 32));
        __hip_atomic_store(xs + (base + (idx >> 1)) * stride + elem[i], 0ull, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    base += pairs;
    idx >>= 1;
    n = (n + 1) >> 1;
  }
}

// Split-K finish by the last workgroup of a tile.  Every workgroup stores
// its partial tile with device-scope stores (written through to the point of
// coherence), waits until they are complete, and one thread counts the
// arrival; the workgroup that brings the count to KS is the last, resets the
// counter for the next call, and sums the KS partials in split order with
// device-scope loads (the same sums, in the same order, as the reduction
// kernel).  Returns true in the last workgroup (uniform over the workgroup).
// `flag` is one word of LDS no thread is still reading.
__device__ __forceinline__ bool split_last(unsigned *counter, int KS, int *flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == (unsigned)(KS - 1);
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last ? 1 : 0;
  }
  __syncthreads();
  return *flag != 0;
}

__device__ __forceinline__ void store_partial(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum of KS partials at p, p + step, ... in split order; eight loads are in
// flight before any is added.
__device__ __forceinline__ float sum_partials(const float *p, int64_t step, int KS) {
  float v = 0.0f;
  for (int s0 = 0; s0 < KS; s0 += 8) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      t[i] = s0 + i < KS ? __hip_atomic_load(p + (int64_t)(s0 + i) * step, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)
                         : 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (s0 + i < KS) v = s0 + i == 0 ? t[i] : v + t[i];
  }
  return v;
}

// Exchange slots a split-K launch needs: KS - 1 per output element (SwiGLU:
// per gate element), 8 bytes each.
inline int64_t split_exchange_bytes(int64_t KS, int64_t elems) {
  return KS > 1 ? (KS - 1) * elems * 8 : 0;
}

// Argument block for a decode launch with KS splits of K (workspace holds
// the split partial tiles when KS > 1).
DecodeArgs decode_args(const Problem &p, int KS, void *workspace);

// How a decode launch with KS > 1 K splits is finished: 0 reduction launch,
// 1 in-launch exchange, 2 last workgroup (the library's choice, or the
// W4A16_SPLIT_FINISH override).
int split_finish(const Problem &p, int KS);

// Second stage of a split-K decode launch: sums the KS partial tiles of each
// strip group in split order and runs the epilogue.
hipError_t launch_decode_reduce(const DecodeArgs &a, bool swiglu, bool bf16, hipStream_t s);

// Cooperative decode kernel (decode_coop.hip): configuration from the
// environment (W4A16_COOP_WC, W4A16_COOP_WK, W4A16_COOP_KS); false if the
// configuration does not fit.
bool coop_config(const Problem &p, int &WC, int &WK, int &KS);
size_t coop_lds_bytes(int M, int WC, int WK, int SPW, bool zp);
hipError_t launch_decode_coop(const Problem &p, void *workspace, int WC, int WK, int KS,
                              hipStream_t s);

}  // namespace w4a16
