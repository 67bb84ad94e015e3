/*
 * w4a16.h -- C ABI of the MI355X (gfx950) W4A16 weight-only INT4 GEMM.
 *
 * The operation (page "GPU Kernels for INT4 Inference, in depth",
 * aicassindra.com, section "The job, stated precisely"): C = A * W with A the
 * fp16 activations [M,K] and W [K,N] stored as 4-bit integers with one fp16
 * scale per group of G = 128 consecutive values along K; the weight is
 * w = (q - 8) * s; accumulation is FP32; the result must equal A times the
 * dequantized weights up to floating-point rounding.
 *
 * Canonical packed format (same page, section "The data contract"):
 *   packed  int32 [K/8, N]  row-major; value k of column n is the nibble at
 *                           bits 4(k mod 8) .. 4(k mod 8)+3 of word [k/8, n],
 *                           stored offset by 8 (0..15);
 *   scales  fp16  [K/G, N]  row-major, passed as uint16_t bit patterns.
 * The GEMM consumes a device-friendly permutation of that format built once
 * at load time by w4a16_repack (the same page, section "Integrating a kernel
 * into serving", advises repacking at load time only, not on every call).
 *
 * Conventions shared by every call:
 *   - Return value: W4A16_OK (0) or a negative W4A16_ERR_* code; no exception
 *     crosses the ABI.  w4a16_last_error() gives a readable message for the
 *     calling thread's last failure.
 *   - Pointers named *_d are device pointers (hipMalloc or equivalent); the
 *     others are host pointers.  All buffers are owned by the caller; the
 *     library keeps no reference to them after the call returns.
 *   - Device work is enqueued on `stream` (a hipStream_t; NULL is the null
 *     stream) and is asynchronous: a fault inside a kernel surfaces at the
 *     caller's next synchronisation.  Launch errors are checked right after
 *     each launch and reported as W4A16_ERR_HIP.
 *   - fp16 values cross the ABI as uint16_t bit patterns.
 *   - Group size G: the GPU paths take G a power of two >= 32 that divides
 *     K (G = 128 is the data contract's default) or G == K (channelwise: one
 *     scale per column), else W4A16_ERR_UNSUPPORTED; the GPU packer takes any
 *     G with G % 8 == 0.  Repacked buffers are built for one G, which every
 *     call on them must pass again.
 *   - K % 128 == 0, N % 8 == 0, and 16-byte aligned device pointers are
 *     required (else W4A16_ERR_INVALID).  M is arbitrary (M == 0 is a no-op).
 *   - Launch configurations are the library's measured choices.  For tests
 *     and measurement, environment variables read at every call override
 *     them (W4A16_DECODE_COOP, _HALF, _WAVES, _DEPTH, _KS, _STAGGER, _DOT;
 *     W4A16_COOP_WC, _WK, _KS; W4A16_TRANSITION, _MI, _KS, _SK, _WAVES;
 *     W4A16_PREFILL_V2,
 *     _BM, _WM, _TPS, _KS, any of which selects the prefill kernels over the
 *     transition kernel); a value no kernel supports is clamped to a
 *     supported one or ignored.  The result of a GEMM does not depend on them
 *     beyond FP32 summation order.  W4A16_SPLIT_FINISH=exchange or =last
 *     finishes a decode launch's K splits inside the launch instead of a
 *     second, reduction launch (slots and counters in a fixed array per
 *     device, so with it set, calls that overlap in time on one device race).
 */
#ifndef W4A16_H
#define W4A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_OK 0
#define W4A16_ERR_INVALID (-1)     /* null pointer, bad size or shape, misalignment */
#define W4A16_ERR_UNSUPPORTED (-2) /* valid in the format, not handled here (G != 128) */
#define W4A16_ERR_NONFINITE (-3)   /* host pack: W holds a NaN or an infinity */
#define W4A16_ERR_HIP (-4)         /* a HIP runtime call or kernel launch failed */
#define W4A16_ERR_WORKSPACE (-5)   /* workspace too small, or its allocation failed */

/* Kernel paths (see w4a16_select_path). */
#define W4A16_PATH_AUTO 0
#define W4A16_PATH_DECODE 1  /* weight-streaming split-K kernel, small M */
#define W4A16_PATH_PREFILL 2 /* LDS-tiled MFMA kernel with in-register dequant */
#define W4A16_PATH_DENSE 3   /* dequantize to fp16 scratch, then dense fp16 GEMM */

/* Flags for w4a16_gemm_ex: a path in the low 4 bits, OR'ed with: */
#define W4A16_FLAG_SWIGLU 0x10 /* fused SwiGLU epilogue (see w4a16_gemm_swiglu) */
#define W4A16_FLAG_BF16 0x20   /* bf16 activations and output (see w4a16_gemm_ex) */
#define W4A16_FLAG_ZP 0x40     /* zero rows in use: for w4a16_describe,
                                  w4a16_gemm_workspace_bytes (w4a16_gemm_zp
                                  implies it) */
#define W4A16_FLAG_INT8 0x80   /* INT8 weights: for w4a16_describe,
                                  w4a16_gemm_workspace_bytes, w4a16_select_path
                                  (w4a16_gemm_int8 implies it) */

typedef void *w4a16_stream_t; /* a hipStream_t */

/* ---------------------------------------------------------------------------
 * Quantize and pack (data contract, quantize_pack).  For each group g of G
 * rows and column n: s = max|W[gG:(g+1)G, n]| / 7 in fp32, s = max(s, 1e-8),
 * q = clamp(round_half_even(W / s), -8, 7) + 8 with an fp32 division, scale
 * stored as fp16(s) (round to nearest even).
 *   W_d       fp32 [K, N] row-major, device, read only
 *   packed_d  int32 [K/8, N], device, written
 *   scales_d  fp16 bits [K/G, N], device, written
 * Runs one kernel on `stream`.  Non-finite W produces unspecified nibbles for
 * that group (use w4a16_pack_host to have them rejected).
 * Errors: W4A16_ERR_INVALID (null pointer, K % G, K % 8, N < 1, G < 1),
 * W4A16_ERR_HIP.
 * ------------------------------------------------------------------------- */
int w4a16_pack(const float *W_d, int64_t K, int64_t N, int G, int32_t *packed_d,
               uint16_t *scales_d, w4a16_stream_t stream);

/* Quantize and pack with a folded RMSNorm gain (FuTransformer, arXiv
 * 2610.23796, section 3.2.2: the frozen gain gamma of the RMSNorm before a
 * projection is folded into its weights once, before quantizing, so the GEMM
 * reads the raw activations).  Same as w4a16_pack applied to
 * W'[k,n] = fp32(gamma[k] * W[k,n]) (one fp32 rounding per element).
 *   gamma_d  fp32 [K], device, read only; NULL means w4a16_pack itself.
 * Pair the packed weights with w4a16_rms_rowscale and w4a16_gemm_rowscale. */
int w4a16_pack_gain(const float *W_d, const float *gamma_d, int64_t K, int64_t N, int G,
                    int32_t *packed_d, uint16_t *scales_d, w4a16_stream_t stream);

/* Same computation on host memory, for loaders that quantize on the CPU.
 * nthreads <= 0 uses every hardware thread.  Returns W4A16_ERR_NONFINITE if W
 * holds a NaN or an infinity (outputs are then unspecified). */
int w4a16_pack_host(const float *W, int64_t K, int64_t N, int G, int32_t *packed,
                    uint16_t *scales, int nthreads);

/* ---------------------------------------------------------------------------
 * Repacked layout, built once at load (the data contract section notes that
 * production kernels often permute the canonical layout at load time).
 * Columns are padded to a multiple of 32 (the pad dequantizes to zero).
 * Byte sizes of the two buffers, or a negative error code for an invalid
 * shape.
 * ------------------------------------------------------------------------- */
int64_t w4a16_repacked_weight_bytes(int64_t K, int64_t N, int G);
int64_t w4a16_repacked_scale_bytes(int64_t K, int64_t N, int G);

/* Permute canonical (packed_d, scales_d) into the repacked buffers
 * (rw_d: w4a16_repacked_weight_bytes, rs_d: w4a16_repacked_scale_bytes, both
 * device, 16-byte aligned).  A bijection on the data: w4a16_unrepack inverts
 * it exactly.  One kernel on `stream`.
 * Errors: W4A16_ERR_INVALID, W4A16_ERR_UNSUPPORTED (G != 128), W4A16_ERR_HIP. */
int w4a16_repack(const int32_t *packed_d, const uint16_t *scales_d, int64_t K, int64_t N,
                 int G, void *rw_d, void *rs_d, w4a16_stream_t stream);

/* Inverse of w4a16_repack, for checking a load after repacking (the same
 * page's serving section recommends checking one layer).  Writes canonical
 * packed_d [K/8,N] and scales_d [K/G,N]. */
int w4a16_unrepack(const void *rw_d, const void *rs_d, int64_t K, int64_t N, int G,
                   int32_t *packed_d, uint16_t *scales_d, w4a16_stream_t stream);

/* Dequantize (data contract, dequantize): W16_d[k,n] = fp16((q - 8) * s),
 * canonical fp16 [K, N] row-major, device.  Bit-exact with the definition. */
int w4a16_dequant(const void *rw_d, const void *rs_d, int64_t K, int64_t N, int G,
                  uint16_t *W16_d, w4a16_stream_t stream);

/* The same dequantization for bf16 models: Wb_d[k,n] = bf16((q - 8) * s), the
 * exact product of q - 8 and the fp16 scale rounded once to bf16 (nearest
 * even), bf16 bits [K, N] row-major, device.  The data contract's dequantize
 * casts to the activation type (.half() for fp16 activations); this is its
 * bf16 reading, and it is the weight operand of every bf16-activation GEMM. */
int w4a16_dequant_bf16(const void *rw_d, const void *rs_d, int64_t K, int64_t N, int G,
                       uint16_t *Wb_d, w4a16_stream_t stream);

/* ---------------------------------------------------------------------------
 * Zero points (Swordfish page, blog.alpindale.net, section "The packed
 * format"): asymmetric (AWQ) weights are w = (q - zp) * s with a 4-bit zero
 * point zp per group and column.  The kernels take them as a third tensor
 * shaped like the scales, the prescaled zero rows z = fp16((8 - zp) * s), and
 * form each weight as one fused multiply-add, round((q - 8) * s + z), rounded
 * once to the activation type.  The nibbles q are stored as they are (0..15,
 * the same packed format and w4a16_repack as the symmetric weights).
 *
 * Build the zero rows of repacked weights:
 *   scales_d  fp16 bits [K/G, N] canonical, device (the same scales given to
 *             w4a16_repack)
 *   zeros_d   uint8 [K/G, N] row-major, device: zp (AWQ checkpoints hold
 *             0..15; any byte value is computed as given)
 *   rz_d      device, 16-byte aligned, w4a16_repacked_scale_bytes(K, N, G)
 *             bytes, written in the repacked scales' layout (padding zero)
 * One kernel on `stream`.  Errors: W4A16_ERR_INVALID, W4A16_ERR_UNSUPPORTED
 * (G), W4A16_ERR_HIP. */
int w4a16_zero_rows(const uint16_t *scales_d, const uint8_t *zeros_d, int64_t K, int64_t N,
                    int G, void *rz_d, w4a16_stream_t stream);

/* Dequantize weights with zero rows: W_d[k,n] = round((q - 8) * s + z), fp16
 * bits [K, N] row-major (bf16 with flags = W4A16_FLAG_BF16), bit-exact with
 * that definition.  rz_d as written by w4a16_zero_rows (not NULL). */
int w4a16_dequant_zp(const void *rw_d, const void *rs_d, const void *rz_d, int64_t K, int64_t N,
                     int G, int flags, uint16_t *W_d, w4a16_stream_t stream);

/* ---------------------------------------------------------------------------
 * INT8 weights (W8A16).  The Swordfish page (blog.alpindale.net, section "The
 * packed format") runs an int8 variant whose unsigned 8-bit codes carry a
 * bias of 128, dequantized with the same idiom; "Making a Single GPU Go Fast"
 * (arunshar.com, chapter 9, section 9.3.2) recommends weight-only INT8 with
 * per-output-channel scales (G = K here).  Format, by analogy with the int4
 * data contract: per group of G rows along K and column n,
 * s = max|W| / 127 (fp32), s = max(s, 1e-8), q = clamp(round_half_even(W / s),
 * -128, 127) + 128, scale stored as fp16(s); four codes consecutive along K
 * share one int32, code k at bits 8(k mod 4) .. 8(k mod 4)+7:
 *   packed  int32 [K/4, N];  scales fp16 bits [K/G, N];  w = (q - 128) * s.
 * Group sizes, alignment and errors as for INT4 weights; the packer needs
 * G % 4 == 0. */
int w4a16_pack_int8(const float *W_d, int64_t K, int64_t N, int G, int32_t *packed_d,
                    uint16_t *scales_d, w4a16_stream_t stream);

/* Repacked INT8 weights: 1 byte per weight, N padded to 32 (the pad
 * dequantizes to zero); the scale buffer is w4a16_repacked_scale_bytes. */
int64_t w4a16_repacked_weight_bytes_int8(int64_t K, int64_t N, int G);

/* Permute canonical INT8 (packed_d [K/4,N], scales_d) into the repacked
 * buffers; w4a16_unrepack_int8 inverts it exactly. */
int w4a16_repack_int8(const int32_t *packed_d, const uint16_t *scales_d, int64_t K, int64_t N,
                      int G, void *rw_d, void *rs_d, w4a16_stream_t stream);
int w4a16_unrepack_int8(const void *rw_d, const void *rs_d, int64_t K, int64_t N, int G,
                        int32_t *packed_d, uint16_t *scales_d, w4a16_stream_t stream);

/* W_d[k,n] = round((q - 128) * s), fp16 bits [K, N] (bf16 with
 * flags = W4A16_FLAG_BF16), rounded once; bit-exact with that definition. */
int w4a16_dequant_int8(const void *rw_d, const void *rs_d, int64_t K, int64_t N, int G, int flags,
                       uint16_t *W_d, w4a16_stream_t stream);

/* GEMM on INT8 weights: out[m,n] = r_m * sum_k A[m,k] * w[k,n], FP32
 * accumulation, with w = (q - 128) * s (fp16 activations: the product with
 * the exact weight; bf16 activations: with bf16((q - 128) * s)) and r_m =
 * rowscale_d[m] or 1 when rowscale_d is NULL.  The same paths as INT4
 * weights: M <= 32 streams the weights (decode), larger M runs the fused
 * MFMA kernel (prefill; operands beyond its 32-bit offsets fall back to the
 * dense tier), W4A16_PATH_DENSE dequantizes into the workspace first.
 * Flags, workspace, outputs and errors as w4a16_gemm_ex (W4A16_FLAG_INT8 is
 * implied and may be given). */
int w4a16_gemm_int8(const uint16_t *A_d, int64_t M, int64_t K, const void *rw_d, const void *rs_d,
                    int64_t N, int G, const float *rowscale_d, uint16_t *out_d, int flags,
                    void *workspace_d, int64_t workspace_bytes, w4a16_stream_t stream);

/* ---------------------------------------------------------------------------
 * GEMM (the job, stated precisely): C_d[m,n] = sum_k A_d[m,k] * w[k,n], FP32
 * accumulation, one fp16 rounding (nearest even) at the end.
 *   A_d  fp16 bits [M, K] row-major, device
 *   rw_d, rs_d  repacked weights of a [K, N] matrix (w4a16_repack)
 *   C_d  fp16 bits [M, N] row-major, device, written
 * The kernel path is chosen from (M, K, N) by a fixed table (decode for small
 * M, prefill for large M, dense fallback for very large M).  Deterministic:
 * the same call gives the same bits on every run.  Uses the library's
 * per-device workspace (split-K partials): the call never synchronises and
 * never frees; when the workspace is too small it allocates a larger one,
 * except under stream capture (HIP graphs), where it returns
 * W4A16_ERR_WORKSPACE instead -- size it beforehand with
 * w4a16_reserve_workspace(w4a16_gemm_workspace_bytes(...)).  Calls that
 * overlap in time on one device (different streams) must use w4a16_gemm_ex
 * with separate workspaces.  A decode launch that splits K in two with a
 * small output (M times output columns <= 131072) finishes the splits inside
 * the launch, exchanging the two partial values of each output through slots
 * the library holds per device (8 MiB with the library's code object, zero
 * whenever no call runs; the first such call on a device looks up their
 * address: make it outside stream capture); with a caller's workspace
 * (w4a16_gemm_ex) a second launch sums them instead, with the same bits.
 * Where the library's layout takes two K splits only because it finishes
 * them itself (narrow plain projections at M = 9-16, e.g. Llama-8B O and
 * down), a caller's workspace keeps the unsplit layout instead: the two
 * calls then differ by FP32 summation order only.
 * A shape the selected kernel cannot take (operands beyond a kernel's 32-bit
 * offsets) runs a slower kernel instead; each such fallback is reported once
 * per process on stderr and by w4a16_last_fallback (the INT4 kernels page,
 * section "Integrating a kernel into serving", keeps a logged
 * dequantize-then-matmul fallback).
 * Errors: W4A16_ERR_INVALID, W4A16_ERR_UNSUPPORTED, W4A16_ERR_WORKSPACE,
 * W4A16_ERR_HIP.
 * ------------------------------------------------------------------------- */
int w4a16_gemm(const uint16_t *A_d, int64_t M, int64_t K, const void *rw_d, const void *rs_d,
               int64_t N, int G, uint16_t *C_d, w4a16_stream_t stream);

/* GEMM with the SwiGLU epilogue of a concatenated gate/up projection
 * (FuTransformer, arXiv 2610.23796, section 2.1: Z = SiLU(X W_g) * (X W_u),
 * gate and up sharing one GEMM).  Columns [0, N/2) of the weight are the gate
 * projection and [N/2, N) the up projection; N % 64 == 0.  Writes
 * Z_d[m,j] = fp16(silu(c[m,j]) * c[m,j+N/2]) computed from the FP32
 * accumulators, Z_d fp16 bits [M, N/2] row-major. */
int w4a16_gemm_swiglu(const uint16_t *A_d, int64_t M, int64_t K, const void *rw_d,
                      const void *rs_d, int64_t N, int G, uint16_t *Z_d,
                      w4a16_stream_t stream);

/* Explicit form of the two calls above.  `flags` = path (W4A16_PATH_*, AUTO
 * to use the table) | W4A16_FLAG_SWIGLU | W4A16_FLAG_BF16.  `workspace_d`
 * (device, 256-byte aligned, at least w4a16_gemm_workspace_bytes) is owned by
 * the caller and needs no initialisation: it carries nothing from one call to
 * the next.  workspace_d may be NULL to use the library's per-device
 * workspace.
 * W4A16_FLAG_BF16 (bf16 models: FuTransformer and the Swordfish page run
 * bf16 activations): A_d and out_d hold bf16 bits instead of fp16; the same
 * repacked weights and fp16 scales are used, each weight entering the product
 * as bf16((q - 8) * s) (see w4a16_dequant_bf16); FP32 accumulation; the output
 * (and the SwiGLU epilogue's) is rounded once to bf16, nearest even. */
int w4a16_gemm_ex(const uint16_t *A_d, int64_t M, int64_t K, const void *rw_d,
                  const void *rs_d, int64_t N, int G, uint16_t *out_d, int flags,
                  void *workspace_d, int64_t workspace_bytes, w4a16_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops, harnesses that forbid allocation): w4a16_gemm_ex
 * with the split-K partials in a fixed scratch array that the library holds
 * per GPU (w4a16_noalloc_scratch_bytes() bytes, 64 MiB, allocated with the
 * library's code object and held until the process ends) instead of a
 * workspace.  Same flags (path | W4A16_FLAG_SWIGLU | W4A16_FLAG_BF16),
 * arguments and outputs as w4a16_gemm_ex, and the results (bits) of
 * w4a16_gemm_ex on the library's workspace (workspace_d NULL); the call makes no
 * allocation, free or synchronisation of any kind.  A problem whose
 * workspace (w4a16_gemm_workspace_bytes) exceeds the scratch returns
 * W4A16_ERR_WORKSPACE before any launch (e.g. the dense tier of a large
 * weight).  All calls on one GPU share its scratch: calls that overlap in
 * time on one GPU (different streams) race and must not be issued; calls on
 * one stream are safe.  The first call on each device looks up the scratch's
 * device address (make it outside capture).  Like w4a16_gemm it finishes two
 * K splits of a small decode output inside the launch, through the library's
 * per-device exchange slots. */
int w4a16_gemm_noalloc(const uint16_t *A_d, int64_t M, int64_t K, const void *rw_d,
                       const void *rs_d, int64_t N, int G, uint16_t *out_d, int flags,
                       w4a16_stream_t stream);
int64_t w4a16_noalloc_scratch_bytes(void);

/* GEMM with a per-row output factor (FuTransformer, section 3.2.2: the
 * RMSNorm row factor rho_m of the raw activations, applied in the GEMM's
 * epilogue): out[m,n] = rowscale[m] * sum_k A[m,k] * w[k,n], and with
 * W4A16_FLAG_SWIGLU the factor multiplies both the gate and the up value
 * before the epilogue, Z = silu(r g) * (r u).  Everything else as
 * w4a16_gemm_ex (same flags, workspace and errors).
 *   rowscale_d  fp32 [M], device, read only (W4A16_ERR_INVALID if NULL and
 *               M > 0) */
int w4a16_gemm_rowscale(const uint16_t *A_d, int64_t M, int64_t K, const void *rw_d,
                        const void *rs_d, int64_t N, int G, const float *rowscale_d,
                        uint16_t *out_d, int flags, void *workspace_d, int64_t workspace_bytes,
                        w4a16_stream_t stream);

/* GEMM on weights with zero points: out[m,n] = r_m * sum_k A[m,k] * w[k,n]
 * with w = round((q - 8) * s + z) in the activation type (w4a16_dequant_zp)
 * and r_m = rowscale_d[m], or 1 when rowscale_d is NULL.  rz_d (not NULL when
 * M > 0) as written by w4a16_zero_rows; flags, workspace, outputs and errors
 * as w4a16_gemm_ex (W4A16_FLAG_ZP is implied and may be given). */
int w4a16_gemm_zp(const uint16_t *A_d, int64_t M, int64_t K, const void *rw_d, const void *rs_d,
                  const void *rz_d, int64_t N, int G, const float *rowscale_d, uint16_t *out_d,
                  int flags, void *workspace_d, int64_t workspace_bytes, w4a16_stream_t stream);

/* RMSNorm row factors of the raw activations (FuTransformer, section 3.2.2):
 * rho_d[m] = (sum_k A[m,k]^2 / K + eps)^(-1/2), sums in FP32 (fixed order,
 * deterministic), correctly rounded division and square root.
 *   A_d    fp16 bits [M, K] (bf16 with flags = W4A16_FLAG_BF16), device,
 *          16-byte aligned; K % 8 == 0
 *   eps    finite, >= 0
 *   rho_d  fp32 [M], device, written
 * Errors: W4A16_ERR_INVALID, W4A16_ERR_HIP. */
int w4a16_rms_rowscale(const uint16_t *A_d, int64_t M, int64_t K, float eps, int flags,
                       float *rho_d, w4a16_stream_t stream);

/* Workspace bytes that w4a16_gemm_ex (w4a16_gemm_zp: add W4A16_FLAG_ZP) needs
 * for this problem and flags; the figure also covers the launch on the
 * library's own workspace, so it serves w4a16_reserve_workspace too. */
int64_t w4a16_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N, int G, int flags);

/* The path (W4A16_PATH_DECODE / PREFILL / DENSE) that AUTO picks for this
 * problem (after fallbacks), or a negative error code. */
int w4a16_select_path(int64_t M, int64_t K, int64_t N, int G, int flags);

/* The library's per-device workspace (used by the GEMM calls given no
 * workspace).  Host calls on the calling thread's current device; they may
 * synchronise the device, so make them at load time, outside stream capture.
 *   w4a16_reserve_workspace(bytes): grow the workspace to at least `bytes`
 *     (bytes >= 0; a smaller request keeps the current buffer), freeing any
 *     buffers that earlier GEMM calls replaced.  Errors: W4A16_ERR_INVALID,
 *     W4A16_ERR_WORKSPACE (allocation failed), W4A16_ERR_HIP.
 *   w4a16_workspace_reserved(): bytes the current workspace holds (or a
 *     negative error code).
 *   w4a16_release_workspace(): synchronise the device and free its workspace
 *     buffers (a later GEMM call allocates again). */
int w4a16_reserve_workspace(int64_t bytes);
int64_t w4a16_workspace_reserved(void);
int w4a16_release_workspace(void);

/* The most recent fallback of any thread ("" if none): the calling entry
 * point or tier, then what ran instead and why.  Each kind of fallback is also
 * written once per process to stderr. */
const char *w4a16_last_fallback(void);

/* Writes into buf (len bytes, NUL-terminated, truncated if short) a text
 * description of the launches w4a16_gemm_ex would make for this problem and
 * flags on the library's workspace (workspace_d NULL; a caller's workspace
 * can change the decode layout, see w4a16_gemm): each kernel instance as it
 * is named in profiler output, with its grid.  Host only; touches no device.  Returns the length written or a
 * negative error code (W4A16_ERR_INVALID for a bad shape, flag or buffer). */
int w4a16_describe(int64_t M, int64_t K, int64_t N, int G, int flags, char *buf, int64_t len);

/* ---- Measurement probes ------------------------------------------------
 * The machine's own ceilings, against which the GEMM's roofline fractions are
 * also reported: the Swordfish page (blog.alpindale.net, section "Decode,
 * counting memory-pipe slots") rates its decode kernels against the
 * platform's practical DRAM ceiling rather than the data-sheet figure, and
 * the INT4 kernels page (aicassindra.com, section "Benchmarking against the
 * roofline") asks for measurements on one's own GPU. */

/* Streaming read: every 16-byte word of buf_d[0 .. bytes) is read exactly
 * once with 128-bit non-temporal loads spread over the whole GPU; nothing is
 * written except, in the unlikely case that the XOR of everything read equals
 * a fixed tag, one 32-bit word at sink_d (so the reads cannot be removed).
 * bytes > 0 and a multiple of 16; buf_d 16-byte aligned; sink_d a device
 * buffer of at least 4 bytes.  Time it with events on `stream`. */
int w4a16_probe_stream_read(const void *buf_d, int64_t bytes, void *sink_d,
                            w4a16_stream_t stream);

/* Dense fp16 MFMA loop: `workgroups` workgroups of 256 threads (4 waves)
 * each run `iterations` rounds of 4 independent v_mfma_f32_32x32x16_f16
 * (operands held in registers, FP32 accumulators), with no memory traffic
 * but one conditional 4-byte store to sink_d.  *flops_out (host pointer, may
 * be NULL) receives the floating-point operations performed:
 * workgroups * 4 * iterations * 4 * 32768.  1 <= iterations <= 2^24,
 * 1 <= workgroups <= 2^20. */
int w4a16_probe_mfma(int64_t iterations, int64_t workgroups, void *sink_d, int64_t *flops_out,
                     w4a16_stream_t stream);

/* Thread-local message for the calling thread's last error ("" if none). */
const char *w4a16_last_error(void);

/* Library version string. */
const char *w4a16_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
