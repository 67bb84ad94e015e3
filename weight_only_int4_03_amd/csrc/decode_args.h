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

// Argument block for a decode launch with KS splits of K (workspace holds
// the split partial tiles when KS > 1).
DecodeArgs decode_args(const Problem &p, int KS, void *workspace);

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
