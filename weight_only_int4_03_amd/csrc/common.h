// Internal definitions shared by the library's HIP sources (not part of the ABI).
//
// Repacked weight layout.  The canonical [K/8, N] int32 words are grouped into
// tiles of 32 columns x 64 k (1 KiB).  Strip t (columns 32t .. 32t+31) holds
// its K/64 tiles contiguously, strip after strip:
//     word offset of (t, q, l, j) = ((t * KT + q) * 64 + l) * 4 + j,  KT = K/64
// Lane position l = 32h + c holds the four words of column 32t + c with
// canonical rows r = 8q + 4h + j (k = 64q + 32h + 8j .. +7), so one 16-byte
// load per lane brings 32 consecutive k of one column, and one wave-wide load
// brings a whole contiguous 1 KiB tile.
//
// Inside each word the nibbles are permuted so that the four shift-and-mask
// steps (w >> 4j) & 0x000F000F yield the fp16 pairs (k0,k1), (k2,k3), (k4,k5),
// (k6,k7) in register order: k offset i sits at nibble position
// (i % 2) * 4 + i / 2.  Pad columns (n >= N) hold 0x88888888 (all zero weights).
//
// INT8 weights (8-bit codes offset by 128, canonical [K/4, N] int32 with
// byte k at bits 8(k mod 4)) use the same strips and 64-k tiles at twice the
// bytes: a tile is 2 KiB, two 1 KiB halves; in half j lane position
// l = 32h + c holds four words of column 32t + c with k = 64q + 32h + 16j +
// 4i .. +3 in word i, so a lane's two 16-byte vectors bring its 32
// consecutive k and every wave-wide load is still one contiguous KiB:
//     uint4 offset of (t, q, j, l) = ((t * KT + q) * 2 + j) * 64 + l.
// Inside each word the bytes hold k offsets (0, 2, 1, 3), so
// w & 0x00FF00FF and (w >> 8) & 0x00FF00FF yield the pairs (k0,k1), (k2,k3).
// Pad columns hold 0x80808080 (all zero weights).
//
// Repacked scale layout: fp16 [NS][KG8][32][8], NS = ceil(N/32),
// KG8 = ceil(K/128 / 8): entry ((t*KG8 + o)*32 + c)*8 + e is the scale of group
// 8o + e and column 32t + c (zero in padding), so a lane reads eight
// consecutive groups' scales of its column with one 16-byte load.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

constexpr int kGroup = 128;   // k per decode unit and per prefill step (the default group)
constexpr int kTileK = 64;    // k per repacked tile
constexpr int kStrip = 32;    // columns per strip
constexpr int kTileWords = 256;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Nibble position of k offset i (0..7) inside a repacked word.
__host__ __device__ inline int nibble_pos(int i) { return (i & 1) * 4 + (i >> 1); }

template <typename To, typename From>
__device__ __forceinline__ To bitcast(From v) { return __builtin_bit_cast(To, v); }

// Nibble -> fp16 conversion (the magic-number idiom of FuTransformer, arXiv
// 2610.23796, section 3.3.4, and of the Swordfish page, section "The packed
// format": place the nibble in the mantissa of a power-of-two 16-bit float
// and subtract the power plus the offset 8).  For fp16 the exponent pattern
// 0x6400 is 1024.0 with a mantissa step of 1, so
//   (w & 0x000F000F) | 0x64006400  = the pair (1024 + u, 1024 + u'),
//   (w & 0x00F000F0) | 0x64006400  = the pair (1024 + 16u, 1024 + 16u'),
// both exact.  One packed add of -1032 turns the first into u - 8; one packed
// FMA (x / 16 - 72) turns the second into u - 8; both results are exact.  The
// other four nibbles come the same way from w >> 8.  With the repacked in-word
// order (k offset i at nibble (i % 2) * 4 + i / 2) the four pairs are
// (k0,k1), (k2,k3), (k4,k5), (k6,k7): 9 VALU instructions per 8 weights
// (1 shift, 4 v_and_or_b32, 2 v_pk_add_f16, 2 v_pk_fma_f16).
struct Dequant {
  uint32_t mask_lo, mask_hi, magic;
  half2_t bias, sixteenth, bias16;

  __device__ __forceinline__ Dequant() {
    mask_lo = 0x000F000Fu;
    mask_hi = 0x00F000F0u;
    magic = 0x64006400u;
    // Keep the masks in SGPRs and the exponent pattern in a VGPR, so that the
    // compiler emits the three-operand v_and_or_b32 (VOP3 on gfx950 takes no
    // literal and at most one SGPR).
    asm volatile("" : "+s"(mask_lo), "+s"(mask_hi));
    asm volatile("" : "+v"(magic));
    bias = half2_t{(_Float16)-1032.0f, (_Float16)-1032.0f};
    sixteenth = half2_t{(_Float16)0.0625f, (_Float16)0.0625f};
    bias16 = half2_t{(_Float16)-72.0f, (_Float16)-72.0f};
  }

  // Eight fp16 values u - 8 of one repacked word, in k order.
  __device__ __forceinline__ half8_t operator()(uint32_t w) const {
    const uint32_t t = w >> 8;
    const half2_t p0 = bitcast<half2_t>((w & mask_lo) | magic) + bias;
    const half2_t p1 =
        __builtin_elementwise_fma(bitcast<half2_t>((w & mask_hi) | magic), sixteenth, bias16);
    const half2_t p2 = bitcast<half2_t>((t & mask_lo) | magic) + bias;
    const half2_t p3 =
        __builtin_elementwise_fma(bitcast<half2_t>((t & mask_hi) | magic), sixteenth, bias16);
    const uint4_t r = {bitcast<uint32_t>(p0), bitcast<uint32_t>(p1), bitcast<uint32_t>(p2),
                       bitcast<uint32_t>(p3)};
    return bitcast<half8_t>(r);
  }

  // The dequantized weights fp16((u - 8) * s): the exact u - 8 times the fp16
  // scale, rounded once -- bit-equal to the format's definition.
  __device__ __forceinline__ half8_t scaled(uint32_t w, half2_t s2) const {
    const half8_t v = (*this)(w);
    const half2_t q0 = half2_t{v[0], v[1]} * s2, q1 = half2_t{v[2], v[3]} * s2;
    const half2_t q2 = half2_t{v[4], v[5]} * s2, q3 = half2_t{v[6], v[7]} * s2;
    return half8_t{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
  }

  // INT8: the eight codes of two repacked words (k order) as fp16 u - 128,
  // exact: (w & 0x00FF00FF) | 0x64006400 is the pair (1024 + u, 1024 + u'),
  // and one packed add of -1152 leaves u - 128 (Swordfish page, "The packed
  // format": the same idiom over byte lanes with a bias of 128).  5 VALU
  // instructions per 4 weights.
  __device__ __forceinline__ half8_t bytes8(uint32_t w0, uint32_t w1) const {
    const half2_t b = half2_t{(_Float16)-1152.0f, (_Float16)-1152.0f};
    const uint32_t m = 0x00FF00FFu;
    const half2_t p0 = bitcast<half2_t>((w0 & m) | magic) + b;
    const half2_t p1 = bitcast<half2_t>(((w0 >> 8) & m) | magic) + b;
    const half2_t p2 = bitcast<half2_t>((w1 & m) | magic) + b;
    const half2_t p3 = bitcast<half2_t>(((w1 >> 8) & m) | magic) + b;
    return half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  }
  // fp16((u - 128) * s), one rounding.
  __device__ __forceinline__ half8_t scaled8(uint32_t w0, uint32_t w1, half2_t s2) const {
    const half8_t v = bytes8(w0, w1);
    const half2_t q0 = half2_t{v[0], v[1]} * s2, q1 = half2_t{v[2], v[3]} * s2;
    const half2_t q2 = half2_t{v[4], v[5]} * s2, q3 = half2_t{v[6], v[7]} * s2;
    return half8_t{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
  }
  // bf16((u - 128) * s): (1024 + u) s - 1152 s in one exact mixed-precision
  // FMA (19-bit product, 15-bit constant), then one rounding to bf16.
  __device__ __forceinline__ bf16x8_t scaled8_bf16(uint32_t w0, uint32_t w1, float s) const {
    const uint32_t m = 0x00FF00FFu;
    const float c = -1152.0f * s;
    const half2_t x0 = bitcast<half2_t>((w0 & m) | magic);
    const half2_t x1 = bitcast<half2_t>(((w0 >> 8) & m) | magic);
    const half2_t x2 = bitcast<half2_t>((w1 & m) | magic);
    const half2_t x3 = bitcast<half2_t>(((w1 >> 8) & m) | magic);
    auto f = [&](_Float16 x) { return (__bf16)__builtin_fmaf((float)x, s, c); };
    return bf16x8_t{f(x0[0]), f(x0[1]), f(x1[0]), f(x1[1]),
                    f(x2[0]), f(x2[1]), f(x3[0]), f(x3[1])};
  }
  template <bool BF>
  __device__ __forceinline__ uint4_t scaled8_bits(uint32_t w0, uint32_t w1, uint16_t s16) const {
    if constexpr (BF) {
      return bitcast<uint4_t>(scaled8_bf16(w0, w1, (float)bitcast<_Float16>(s16)));
    } else {
      const _Float16 sh = bitcast<_Float16>(s16);
      return bitcast<uint4_t>(scaled8(w0, w1, half2_t{sh, sh}));
    }
  }

  // With a zero row (AWQ zero points prescaled as z = fp16((8 - zp) s)):
  // fp16((u - 8) * s + z), one fused multiply-add per pair, rounded once.
  __device__ __forceinline__ half8_t scaled_zp(uint32_t w, half2_t s2, half2_t z2) const {
    const half8_t v = (*this)(w);
    const half2_t q0 = __builtin_elementwise_fma(half2_t{v[0], v[1]}, s2, z2);
    const half2_t q1 = __builtin_elementwise_fma(half2_t{v[2], v[3]}, s2, z2);
    const half2_t q2 = __builtin_elementwise_fma(half2_t{v[4], v[5]}, s2, z2);
    const half2_t q3 = __builtin_elementwise_fma(half2_t{v[6], v[7]}, s2, z2);
    return half8_t{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
  }

  // bf16 activations.  The dequantized weight is then bf16((u - 8) * s): the
  // exact product of u - 8 and the fp16 scale, rounded once to bf16.  The
  // magic-number pairs (1024 + u, or 1024 + 16u) go straight into a
  // mixed-precision FMA (fp16 x fp32 + fp32 -> fp32, v_fma_mix_f32) with
  // per-column constants of the group: (1024 + u) s - 1032 s, and
  // (1024 + 16u) (s / 16) - 72 s.  Every product and constant has at most 22
  // significant bits and the sum is (u - 8) s itself, so the FMA is exact; one
  // v_cvt_pk_bf16_f32 per pair then rounds.  17 VALU instructions per word.
  //
  // A zero row z (fp16) joins the constants: (1024 + u) s + (z - 1032 s) and
  // (1024 + 16u) (s / 16) + (z - 72 s).  z is 0 or at least |s| in magnitude,
  // so it is a multiple of the fp16 spacing of s, and so are both constants
  // (below 2^22 of those spacings: exact in fp32); the FMA result
  // (u - 8) s + z is exact as well, and the conversion is the one rounding.
  struct BScale {
    float s, c_lo, s_hi, c_hi;
    __device__ __forceinline__ explicit BScale(uint16_t s16) {
      s = (float)bitcast<_Float16>(s16);
      c_lo = -1032.0f * s;
      s_hi = s * 0.0625f;
      c_hi = -72.0f * s;
    }
    __device__ __forceinline__ BScale(uint16_t s16, uint16_t z16) {
      s = (float)bitcast<_Float16>(s16);
      const float z = (float)bitcast<_Float16>(z16);
      c_lo = __builtin_fmaf(-1032.0f, s, z);
      s_hi = s * 0.0625f;
      c_hi = __builtin_fmaf(-72.0f, s, z);
    }
  };
  // The scaled weights of either type as a raw 16-byte MFMA operand (ZP: with
  // the zero row z16).
  template <bool BF>
  __device__ __forceinline__ uint4_t scaled_bits(uint32_t w, uint16_t s16) const;
  template <bool BF, bool ZP>
  __device__ __forceinline__ uint4_t scaled_bits(uint32_t w, uint16_t s16, uint16_t z16) const;

  __device__ __forceinline__ bf16x8_t scaled_bf16(uint32_t w, const BScale &b) const {
    const uint32_t t = w >> 8;
    const half2_t x0 = bitcast<half2_t>((w & mask_lo) | magic);
    const half2_t x1 = bitcast<half2_t>((w & mask_hi) | magic);
    const half2_t x2 = bitcast<half2_t>((t & mask_lo) | magic);
    const half2_t x3 = bitcast<half2_t>((t & mask_hi) | magic);
    auto lo = [&](_Float16 x) { return (__bf16)__builtin_fmaf((float)x, b.s, b.c_lo); };
    auto hi = [&](_Float16 x) { return (__bf16)__builtin_fmaf((float)x, b.s_hi, b.c_hi); };
    return bf16x8_t{lo(x0[0]), lo(x0[1]), hi(x1[0]), hi(x1[1]),
                    lo(x2[0]), lo(x2[1]), hi(x3[0]), hi(x3[1])};
  }
};

__device__ __forceinline__ uint4_t load_nt(const uint4_t *p) {
  return __builtin_nontemporal_load(p);
}

// Buffer resource word 3 for raw (stride 0, untyped 32-bit) buffers on gfx9
// class parts, and the cache-policy operand of a streaming (non-temporal)
// buffer read.
constexpr int kBufferConfig = 0x00020000;
constexpr int kBufferNT = 2;

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

__device__ __forceinline__ uint16_t to_half_bits(float v) {
  return bitcast<uint16_t>((_Float16)v);
}

template <bool BF>
__device__ __forceinline__ uint4_t Dequant::scaled_bits(uint32_t w, uint16_t s16) const {
  if constexpr (BF) {
    return bitcast<uint4_t>(scaled_bf16(w, BScale(s16)));
  } else {
    const _Float16 sh = bitcast<_Float16>(s16);
    return bitcast<uint4_t>(scaled(w, half2_t{sh, sh}));
  }
}

template <bool BF, bool ZP>
__device__ __forceinline__ uint4_t Dequant::scaled_bits(uint32_t w, uint16_t s16,
                                                        uint16_t z16) const {
  if constexpr (!ZP) {
    return scaled_bits<BF>(w, s16);
  } else if constexpr (BF) {
    return bitcast<uint4_t>(scaled_bf16(w, BScale(s16, z16)));
  } else {
    const _Float16 sh = bitcast<_Float16>(s16), zh = bitcast<_Float16>(z16);
    return bitcast<uint4_t>(scaled_zp(w, half2_t{sh, sh}, half2_t{zh, zh}));
  }
}

// Output element bits: fp16, or bf16 (round to nearest even) for bf16
// activations.
template <bool BF>
__device__ __forceinline__ uint16_t to_out_bits(float v) {
  if constexpr (BF)
    return bitcast<uint16_t>((__bf16)v);
  else
    return bitcast<uint16_t>((_Float16)v);
}

// A packed pair of output elements (lo in the low half).
template <bool BF>
__device__ __forceinline__ uint32_t pack_out2(float lo, float hi) {
  if constexpr (BF)
    return bitcast<uint32_t>(bf16x2_t{(__bf16)lo, (__bf16)hi});
  else
    return bitcast<uint32_t>(half2_t{(_Float16)lo, (_Float16)hi});
}

// One MFMA step, fp16 or bf16 operands (raw 16-byte vectors of 8 elements:
// x is the instruction's first operand, y its second).
template <bool BF>
__device__ __forceinline__ float16_t mfma32(uint4_t x, uint4_t y, float16_t c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8_t>(x), bitcast<bf16x8_t>(y), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<half8_t>(x), bitcast<half8_t>(y), c, 0,
                                                  0, 0);
}
template <bool BF>
__device__ __forceinline__ float4_t mfma16(uint4_t x, uint4_t y, float4_t c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(x), bitcast<bf16x8_t>(y), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(x), bitcast<half8_t>(y), c, 0,
                                                  0, 0);
}

// ---------------------------------------------------------------------------
// Host-side launch descriptions (defined in decode.hip / prefill.hip /
// format.hip, called from api.hip).

struct Problem {
  const uint16_t *A;
  int64_t M, K, N;
  const void *rw;
  const void *rs;
  uint16_t *out;   // C [M,N] or Z [M,N/2]
  bool swiglu;
  bool bf16;       // A and the output are bf16 (else fp16)
  const float *rowscale;  // per-row output factor [M], or null
  int G = kGroup;  // quantization group along K
  int gshift = 7;  // group of k = k >> gshift (see group_shift)
  const void *rz = nullptr;  // prescaled zero rows, laid out as rs, or null
  bool zp = false;           // zero rows in use (rz != null when launching)
  int bits = 4;              // weight code width: 4 (INT4) or 8 (INT8)
  bool own_ws = true;        // runs on the library's workspace or fixed scratch, not a caller's
};

// Group sizes: a power of two >= 32 that divides K, or K itself
// (channelwise).  The kernels find the group of k as k >> gshift; for a
// channelwise G that is not a power of two gshift is 31, so every k maps to
// group 0.
inline int group_shift(int64_t K, int G) {
  if ((G & (G - 1)) == 0) {
    int s = 0;
    while ((1 << s) < G) ++s;
    return s;
  }
  return G == K ? 31 : -1;
}

// Groups per column and its octets (the repacked scale layout holds eight
// consecutive groups of a column in one 16-byte run).
inline int64_t groups_of(int64_t K, int G) { return K / G; }

// Index of the scale of group g, strip st, column c of the strip in the
// repacked scale buffer [NS][KG8][32][8].
__host__ __device__ inline int64_t scale_index(int64_t st, int64_t KG8, int c, int g) {
  return ((st * KG8 + (g >> 3)) * 32 + c) * 8 + (g & 7);
}

hipError_t launch_pack(const float *W, const float *gamma, int64_t K, int64_t N, int G,
                       int32_t *packed, uint16_t *scales, hipStream_t s);
// RMSNorm row factors rho[m] = (sum_k A[m,k]^2 / K + eps)^(-1/2) (rms.hip).
hipError_t launch_rms_rowscale(const uint16_t *A, int64_t M, int64_t K, float eps, bool bf16,
                               float *rho, hipStream_t s);
hipError_t launch_repack(const int32_t *packed, const uint16_t *scales, int64_t K, int64_t N,
                         int G, void *rw, void *rs, hipStream_t s);
hipError_t launch_unrepack(const void *rw, const void *rs, int64_t K, int64_t N, int G,
                           int32_t *packed, uint16_t *scales, hipStream_t s);
// INT8 weights: quantize + pack ([K/4, N] words), repack / unrepack, dequantize.
hipError_t launch_pack8(const float *W, int64_t K, int64_t N, int G, int32_t *packed,
                        uint16_t *scales, hipStream_t s);
hipError_t launch_repack8(const int32_t *packed, const uint16_t *scales, int64_t K, int64_t N,
                          int G, void *rw, void *rs, hipStream_t s);
hipError_t launch_unrepack8(const void *rw, const void *rs, int64_t K, int64_t N, int G,
                            int32_t *packed, uint16_t *scales, hipStream_t s);
hipError_t launch_dequant8_canonical(const void *rw, const void *rs, int64_t K, int64_t N, int G,
                                     bool bf16, uint16_t *W, hipStream_t s);
hipError_t launch_dequant8_fragment(const void *rw, const void *rs, int64_t K, int64_t N, int G,
                                    bool bf16, uint16_t *Wf, hipStream_t s);

// Prescaled zero rows fp16((8 - zp) s) in the repacked scale layout.
hipError_t launch_zero_rows(const uint16_t *scales, const uint8_t *zeros, int64_t K, int64_t N,
                            int G, void *rz, hipStream_t s);
// rz: prescaled zero rows (repacked layout) or null.
hipError_t launch_dequant_canonical(const void *rw, const void *rs, const void *rz, int64_t K,
                                    int64_t N, int G, bool bf16, uint16_t *W, hipStream_t s);
hipError_t launch_dequant_fragment(const void *rw, const void *rs, const void *rz, int64_t K,
                                   int64_t N, int G, bool bf16, uint16_t *Wf, hipStream_t s);

// Reports a fallback (a slower kernel taking a shape the selected one cannot):
// once per kind `what` on stderr, and as w4a16_last_fallback (api.hip).
void note_fallback(const char *what, const char *who);

// Decode path: workspace bytes (split-K partials), the launch, and a text
// description of the launch (kernel instances and grid).
int64_t decode_workspace_bytes(const Problem &p);
int decode_describe(const Problem &p, char *buf, size_t n);
hipError_t launch_decode(const Problem &p, void *workspace, hipStream_t s);

// Prefill path (fused dequant) and dense path (fp16 fragment-ordered weights).
int64_t prefill_workspace_bytes(const Problem &p);
hipError_t launch_prefill(const Problem &p, void *workspace, hipStream_t s);
// False when the fused path cannot take the problem (INT8 weights outside the
// 8-wave kernel's limits: the one-wave kernel reads INT4 codes only).
bool prefill_fused_available(const Problem &p);
int64_t dense_workspace_bytes(const Problem &p);
hipError_t launch_dense(const Problem &p, void *workspace, hipStream_t s);
int tiled_describe(const Problem &p, bool dense, char *buf, size_t n);

// Transition-regime kernel (transition.hip): launch shape, workspace (FP32
// partials when K is split), description and launch.  transition_config
// returns false where the kernel does not take the problem.
struct TransConfig {
  int mi, wc, wk, ks, tiles, row_tiles, col_groups;
  // Stream-K: units per workgroup (0: one tile or K slice per workgroup),
  // (tile, round) units, rounds per tile, most workgroups sharing a tile.
  int sk_upw = 0, sk_units = 0, sk_rounds = 0, sk_parts = 1;
};
bool transition_config(const Problem &p, TransConfig &c);
int64_t transition_workspace_bytes(const Problem &p);
int transition_describe(const Problem &p, const TransConfig &c, char *buf, size_t n);
hipError_t launch_transition(const Problem &p, const TransConfig &c, void *ws, hipStream_t s);
// Second stage of a split-K tiled GEMM: sums KS FP32 partial slices
// ws[KS][M][N] in slice order and runs the epilogue into p.out (prefill.hip).
hipError_t launch_prefill_reduce(const float *ws, int KS, const Problem &p, hipStream_t s);

// Measurement probes (probe.hip).
hipError_t launch_stream_read(const void *buf, int64_t bytes, void *sink, hipStream_t s);
hipError_t launch_mfma_peak(int iterations, int64_t workgroups, void *sink, hipStream_t s);

}  // namespace w4a16
