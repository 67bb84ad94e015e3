// C ABI of the W4A16 library: argument checks, path dispatch, workspace.
// The operations and their citations are documented in include/w4a16.h.
#include "w4a16.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <set>
#include <string>
#include <thread>
#include <vector>

#include "common.h"

namespace w4a16 {
namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(W4A16_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }  // null passes

// Shape rules of the canonical format (data contract) plus this library's.
int check_shape(int64_t K, int64_t N, int G, const char *who) {
  if (G <= 0) return fail(W4A16_ERR_INVALID, "%s: G must be positive (got %d)", who, G);
  if (K <= 0 || N <= 0) return fail(W4A16_ERR_INVALID, "%s: K and N must be positive", who);
  if (K % 8 != 0 || K % G != 0)
    return fail(W4A16_ERR_INVALID, "%s: K (%lld) must be a multiple of 8 and of G (%d)", who,
                (long long)K, G);
  return W4A16_OK;
}

int check_gpu_shape(int64_t K, int64_t N, int G, const char *who) {
  int rc = check_shape(K, N, G, who);
  if (rc != W4A16_OK) return rc;
  if (K % kGroup != 0)
    return fail(W4A16_ERR_INVALID, "%s: K (%lld) must be a multiple of 128", who, (long long)K);
  if (G < 32 || group_shift(K, G) < 0)
    return fail(W4A16_ERR_UNSUPPORTED,
                "%s: G must be a power of two >= 32 dividing K, or K itself (got %d)", who, G);
  if (N % 8 != 0)
    return fail(W4A16_ERR_INVALID, "%s: N (%lld) must be a multiple of 8", who, (long long)N);
  if (K > (int64_t)1 << 30 || N > (int64_t)1 << 30)
    return fail(W4A16_ERR_INVALID, "%s: K or N too large", who);
  return W4A16_OK;
}

// ---------------------------------------------------------------------------
// Library-owned per-device workspace (split-K partials, dense-tier scratch).
// It holds no state between calls: every call writes what it later reads.
//
// A GEMM call never synchronises and never frees: when a call needs more than
// the device's workspace holds, a larger buffer is allocated (outside stream
// capture only) and the old one is retired, to be freed by the next
// w4a16_reserve_workspace or w4a16_release_workspace, which synchronise the
// device first.  Under capture a call that needs more returns
// W4A16_ERR_WORKSPACE: size the workspace with w4a16_reserve_workspace
// before capturing.

struct DeviceWorkspace {
  void *ptr = nullptr;
  int64_t bytes = 0;
  std::vector<void *> retired;  // replaced buffers, possibly still in use by queued kernels
};

std::mutex g_ws_mutex;
std::vector<DeviceWorkspace> g_ws;

int current_device(int *dev) {
  hipError_t e = hipGetDevice(dev);
  return e == hipSuccess ? W4A16_OK : hip_fail(e, "hipGetDevice");
}

DeviceWorkspace &workspace_of(int dev) {
  if ((int)g_ws.size() <= dev) g_ws.resize(dev + 1);
  return g_ws[dev];
}

// True when `stream` is recording into a HIP graph.
bool capturing(hipStream_t stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &st) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return st != hipStreamCaptureStatusNone;
}

int device_workspace(int64_t need, hipStream_t stream, void **out) {
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != W4A16_OK) return rc;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  DeviceWorkspace &w = workspace_of(dev);
  if (w.bytes < need) {
    if (capturing(stream))
      return fail(W4A16_ERR_WORKSPACE,
                  "the library workspace holds %lld bytes and this call needs %lld; a call under "
                  "stream capture does not allocate: call w4a16_reserve_workspace(%lld) first",
                  (long long)w.bytes, (long long)need, (long long)need);
    const int64_t bytes = need + need / 4;  // some headroom for later, larger calls
    void *p = nullptr;
    hipError_t e = hipMalloc(&p, (size_t)bytes);
    if (e != hipSuccess)
      return fail(W4A16_ERR_WORKSPACE, "workspace allocation of %lld bytes failed: %s",
                  (long long)bytes, hipGetErrorString(e));
    if (w.ptr != nullptr) w.retired.push_back(w.ptr);
    w.ptr = p;
    w.bytes = bytes;
  }
  *out = w.ptr;
  return W4A16_OK;
}

// Synchronise the device and free its retired buffers (and, with all, the
// current one).  Called with g_ws_mutex held.
int drain_workspace(DeviceWorkspace &w, bool all) {
  if (w.retired.empty() && !(all && w.ptr != nullptr)) return W4A16_OK;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  for (void *p : w.retired) (void)hipFree(p);
  w.retired.clear();
  if (all && w.ptr != nullptr) {
    (void)hipFree(w.ptr);
    w.ptr = nullptr;
    w.bytes = 0;
  }
  return W4A16_OK;
}

// ---------------------------------------------------------------------------
// Fixed scratch of w4a16_gemm_noalloc, for callers that cannot allocate (code
// under stream capture, serving loops that forbid allocation): the split-K
// partials of a call live in this array, one copy per GPU, held until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
// Every call on a GPU shares that GPU's copy, so calls that overlap in time on
// one GPU race.  Nothing in it needs clearing: each call writes every element
// it later reads.
constexpr int64_t kScratchBytes = (int64_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
std::vector<void *> g_scratch;  // device address of `scratch`, per device (null: not looked up)

int scratch_address(void **out) {
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != W4A16_OK) return rc;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if ((int)g_scratch.size() <= dev) g_scratch.resize(dev + 1, nullptr);
  if (g_scratch[dev] == nullptr) {
    void *p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr || ((uintptr_t)p & 255u) != 0)
      return fail(W4A16_ERR_HIP, "scratch symbol has no 256-byte aligned device address");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return W4A16_OK;
}

// ---------------------------------------------------------------------------
// Fallbacks.  A shape that the selected kernel cannot take runs a slower
// kernel instead; each kind is reported once per process on stderr (the INT4
// kernels page, section "Integrating a kernel into serving", keeps a logged
// dequantize-then-matmul fallback), and the most recent one is kept for
// w4a16_last_fallback.

std::mutex g_fb_mutex;
std::set<std::string> g_fb_seen;
std::string g_fb_last;

}  // namespace

void note_fallback(const char *what, const char *who) {
  std::lock_guard<std::mutex> lock(g_fb_mutex);
  g_fb_last = std::string(who) + ": " + what;
  if (g_fb_seen.insert(what).second)
    fprintf(stderr, "w4a16: fallback in %s: %s (reported once per process)\n", who, what);
}

namespace {

// ---------------------------------------------------------------------------
// Dispatch.  Decode streams the weights once per call and wins while the
// product is weight-bound; the tiled MFMA kernel takes over when the
// activation rows make it compute-bound; the dense tier (dequantize once, then
// a dense fp16 GEMM) is kept for very large M.  Thresholds from measurement
// on MI355X.
constexpr int64_t kDecodeMaxM = 32;
constexpr int64_t kDenseMinM = 1 << 30;  // the fused kernel is kept at every M measured so far

int select_path(int64_t M, int64_t K, int64_t N, int bits = 4) {
  (void)K;
  (void)N;
  (void)bits;
  if (M <= kDecodeMaxM) return W4A16_PATH_DECODE;
  if (M >= kDenseMinM) return W4A16_PATH_DENSE;
  return W4A16_PATH_PREFILL;
}

// The decode kernels form activation and weight offsets in 32 bits: the
// activation rows of one call (M * K * 2 bytes) and one strip's weights
// (K / 2 bytes, K for INT8, times 32 columns) must stay below 4 GiB.
bool decode_fits(const Problem &p) {
  const int64_t limit = (int64_t)1 << 32;
  const int64_t m = p.M < kDecodeMaxM ? p.M : kDecodeMaxM;
  return m * p.K * 2 < limit && p.K * 16 * (p.bits == 8 ? 2 : 1) < limit;
}

// The path a call takes: the requested (or automatic) path with the
// fallbacks applied.  *why names the fallback when one replaced the path
// (nullptr otherwise); a forced decode path that the decode kernels cannot
// take gives -1.
int resolve_path(const Problem &p, int requested, const char **why) {
  *why = nullptr;
  int path = requested == W4A16_PATH_AUTO ? select_path(p.M, p.K, p.N, p.bits) : requested;
  if (path == W4A16_PATH_DECODE && !decode_fits(p)) {
    if (requested == W4A16_PATH_DECODE) return -1;
    path = W4A16_PATH_PREFILL;
    *why = "decode-offsets: M*K or K beyond the decode kernels' 32-bit offsets, running the "
           "prefill path";
  }
  if (path == W4A16_PATH_PREFILL && !prefill_fused_available(p)) {
    path = W4A16_PATH_DENSE;
    *why = "int8-prefill-dense: INT8 operands beyond the fused kernel's 32-bit offsets, running "
           "the dense tier (dequantize, then dense GEMM)";
  }
  return path;
}

// Workspace of a call on `path`.  The decode path runs M > 32 in 32-row
// slices; a trailing slice of M % 32 rows may take another configuration,
// so the need is the larger of the two slice sizes'.
int64_t workspace_for(int path, const Problem &p) {
  if (path == W4A16_PATH_DENSE) return dense_workspace_bytes(p);
  if (path == W4A16_PATH_PREFILL) return prefill_workspace_bytes(p);
  if (path == W4A16_PATH_DECODE) {
    Problem q = p;
    q.M = p.M < kDecodeMaxM ? p.M : kDecodeMaxM;
    int64_t need = decode_workspace_bytes(q);
    if (p.M > kDecodeMaxM && p.M % kDecodeMaxM != 0) {
      q.M = p.M % kDecodeMaxM;
      const int64_t tail = decode_workspace_bytes(q);
      if (tail > need) need = tail;
    }
    return need;
  }
  return 0;
}

int run_gemm(const uint16_t *A, int64_t M, int64_t K, const void *rw, const void *rs, int64_t N,
             int G, uint16_t *out, int flags, void *workspace, int64_t ws_bytes,
             hipStream_t stream, const float *rowscale = nullptr, const void *rz = nullptr,
             const char *who = nullptr, int bits = 4, bool no_alloc = false) {
  if (who == nullptr) who = (flags & W4A16_FLAG_SWIGLU) ? "w4a16_gemm_swiglu" : "w4a16_gemm";
  const bool bf16 = (flags & W4A16_FLAG_BF16) != 0;
  int rc = check_gpu_shape(K, N, G, who);
  if (rc != W4A16_OK) return rc;
  if (M < 0) return fail(W4A16_ERR_INVALID, "%s: M must be >= 0", who);
  if (M > ((int64_t)1 << 30)) return fail(W4A16_ERR_INVALID, "%s: M too large", who);
  const bool swiglu = (flags & W4A16_FLAG_SWIGLU) != 0;
  if (swiglu && N % 64 != 0)
    return fail(W4A16_ERR_INVALID, "%s: N (%lld) must be a multiple of 64", who, (long long)N);
  if (M == 0) return W4A16_OK;
  if (!A || !rw || !rs || !out) return fail(W4A16_ERR_INVALID, "%s: null pointer", who);
  if (!aligned16(A) || !aligned16(rw) || !aligned16(rs) || !aligned16(out) || !aligned16(rz))
    return fail(W4A16_ERR_INVALID, "%s: device pointers must be 16-byte aligned", who);
  const int requested = flags & 0xF;
  if (requested > W4A16_PATH_DENSE)
    return fail(W4A16_ERR_INVALID, "%s: unknown path %d", who, requested);
  Problem p{A, M, K, N, rw, rs, out, swiglu, bf16, rowscale, G, group_shift(K, G), rz,
            rz != nullptr, bits, workspace == nullptr || no_alloc};
  const char *why = nullptr;
  const int path = resolve_path(p, requested, &why);
  if (path < 0)
    return fail(W4A16_ERR_UNSUPPORTED,
                "%s: the decode path takes M*K*2 and 16*K (32*K for INT8) below 2^32", who);
  const int64_t need = workspace_for(path, p);
  void *ws = workspace;
  if (need > 0) {
    if (ws == nullptr && !no_alloc) {
      rc = device_workspace(need, stream, &ws);
      if (rc != W4A16_OK) return rc;
    } else if (ws_bytes < need || ((uintptr_t)ws & 255u) != 0) {
      return fail(W4A16_ERR_WORKSPACE, "%s: workspace needs %lld bytes, 256-byte aligned%s", who,
                  (long long)need, no_alloc ? " (beyond this entry point's fixed scratch)" : "");
    }
  }
  if (why != nullptr) note_fallback(why, who);

  hipError_t e = hipSuccess;
  if (path == W4A16_PATH_DECODE) {
    // The decode kernels take up to 32 rows; larger M runs in 32-row slices.
    const int64_t ldo = swiglu ? N / 2 : N;
    for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += kDecodeMaxM) {
      Problem q = p;
      q.A = A + m0 * K;
      q.out = out + m0 * ldo;
      if (rowscale != nullptr) q.rowscale = rowscale + m0;
      q.M = M - m0 < kDecodeMaxM ? M - m0 : kDecodeMaxM;
      e = launch_decode(q, ws, stream);
    }
  } else if (path == W4A16_PATH_PREFILL) {
    e = launch_prefill(p, ws, stream);
  } else {
    e = launch_dense(p, ws, stream);
  }
  if (e != hipSuccess) return hip_fail(e, who);
  return W4A16_OK;
}

}  // namespace
}  // namespace w4a16

using namespace w4a16;

extern "C" {

int w4a16_probe_stream_read(const void *buf_d, int64_t bytes, void *sink_d,
                            w4a16_stream_t stream) {
  const char *who = "w4a16_probe_stream_read";
  if (!buf_d || !sink_d) return fail(W4A16_ERR_INVALID, "%s: null pointer", who);
  if (bytes <= 0 || bytes % 16 != 0)
    return fail(W4A16_ERR_INVALID, "%s: bytes must be a positive multiple of 16", who);
  if (!aligned16(buf_d)) return fail(W4A16_ERR_INVALID, "%s: buffer must be 16-byte aligned", who);
  hipError_t e = launch_stream_read(buf_d, bytes, sink_d, (hipStream_t)stream);
  return e == hipSuccess ? W4A16_OK : hip_fail(e, who);
}

int w4a16_probe_mfma(int64_t iterations, int64_t workgroups, void *sink_d, int64_t *flops_out,
                     w4a16_stream_t stream) {
  const char *who = "w4a16_probe_mfma";
  if (!sink_d) return fail(W4A16_ERR_INVALID, "%s: null pointer", who);
  if (iterations < 1 || iterations > ((int64_t)1 << 24) || workgroups < 1 ||
      workgroups > ((int64_t)1 << 20))
    return fail(W4A16_ERR_INVALID, "%s: iterations or workgroups out of range", who);
  hipError_t e = launch_mfma_peak((int)iterations, workgroups, sink_d, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, who);
  if (flops_out) *flops_out = workgroups * 4 * iterations * 4 * 32768;
  return W4A16_OK;
}

const char *w4a16_last_error(void) { return g_last_error.c_str(); }

const char *w4a16_version(void) { return "w4a16-gfx950 0.1"; }

int w4a16_pack(const float *W_d, int64_t K, int64_t N, int G, int32_t *packed_d,
               uint16_t *scales_d, w4a16_stream_t stream) {
  return w4a16_pack_gain(W_d, nullptr, K, N, G, packed_d, scales_d, stream);
}

int w4a16_pack_gain(const float *W_d, const float *gamma_d, int64_t K, int64_t N, int G,
                    int32_t *packed_d, uint16_t *scales_d, w4a16_stream_t stream) {
  const char *who = gamma_d != nullptr ? "w4a16_pack_gain" : "w4a16_pack";
  int rc = check_shape(K, N, G, who);
  if (rc != W4A16_OK) return rc;
  if (G % 8 != 0)
    return fail(W4A16_ERR_UNSUPPORTED, "%s: the GPU packer needs G % 8 == 0 (got %d)", who, G);
  if (K / G > 65535) return fail(W4A16_ERR_INVALID, "%s: K too large", who);
  if (!W_d || !packed_d || !scales_d) return fail(W4A16_ERR_INVALID, "%s: null pointer", who);
  hipError_t e = launch_pack(W_d, gamma_d, K, N, G, packed_d, scales_d, (hipStream_t)stream);
  return e == hipSuccess ? W4A16_OK : hip_fail(e, who);
}

// Host quantize+pack: threads split the columns.  fp32 IEEE division,
// round-half-to-even (nearbyintf in the default rounding mode) and the
// compiler's round-to-nearest-even float -> _Float16 conversion.
int w4a16_pack_host(const float *W, int64_t K, int64_t N, int G, int32_t *packed,
                    uint16_t *scales, int nthreads) {
  int rc = check_shape(K, N, G, "w4a16_pack_host");
  if (rc != W4A16_OK) return rc;
  if (!W || !packed || !scales) return fail(W4A16_ERR_INVALID, "w4a16_pack_host: null pointer");
  int nt = nthreads > 0 ? nthreads : (int)std::thread::hardware_concurrency();
  if (nt < 1) nt = 1;
  const int64_t chunk = 64;
  const int64_t nchunks = ceil_div(N, chunk);
  if (nt > nchunks) nt = (int)nchunks;
  std::vector<int> bad(nt, 0);
  auto work = [&](int id) {
    std::vector<float> scale(chunk);
    for (int64_t cb = id; cb < nchunks; cb += nt) {
      const int64_t n0 = cb * chunk, n1 = n0 + chunk < N ? n0 + chunk : N;
      for (int64_t g = 0; g < K / G; ++g) {
        for (int64_t n = n0; n < n1; ++n) scale[n - n0] = 0.0f;
        for (int64_t k = g * G; k < (g + 1) * G; ++k) {
          const float *row = W + k * N;
          for (int64_t n = n0; n < n1; ++n) {
            const float a = std::fabs(row[n]);
            if (!std::isfinite(row[n])) bad[id] = 1;
            if (a > scale[n - n0]) scale[n - n0] = a;
          }
        }
        for (int64_t n = n0; n < n1; ++n) {
          float s = scale[n - n0] / 7.0f;
          scale[n - n0] = s < 1e-8f ? 1e-8f : s;
          _Float16 hs = (_Float16)scale[n - n0];
          std::memcpy(&scales[g * N + n], &hs, 2);
        }
        for (int64_t r = g * G / 8; r < (g + 1) * G / 8; ++r) {
          for (int64_t n = n0; n < n1; ++n) packed[r * N + n] = 0;
          for (int i = 0; i < 8; ++i) {
            const float *row = W + (8 * r + i) * N;
            for (int64_t n = n0; n < n1; ++n) {
              float q = std::nearbyint(row[n] / scale[n - n0]);
              q = q < -8.0f ? -8.0f : (q > 7.0f ? 7.0f : q);
              packed[r * N + n] |= (int32_t)((uint32_t)((int)q + 8) << (4 * i));
            }
          }
        }
      }
    }
  };
  std::vector<std::thread> pool;
  for (int i = 1; i < nt; ++i) pool.emplace_back(work, i);
  work(0);
  for (auto &t : pool) t.join();
  for (int i = 0; i < nt; ++i)
    if (bad[i]) return fail(W4A16_ERR_NONFINITE, "w4a16_pack_host: W holds NaN or Inf");
  return W4A16_OK;
}

int64_t w4a16_repacked_weight_bytes(int64_t K, int64_t N, int G) {
  int rc = check_gpu_shape(K, N, G, "w4a16_repacked_weight_bytes");
  if (rc != W4A16_OK) return rc;
  return ceil_div(N, kStrip) * (K / kTileK) * kTileWords * 4;
}

int64_t w4a16_repacked_scale_bytes(int64_t K, int64_t N, int G) {
  int rc = check_gpu_shape(K, N, G, "w4a16_repacked_scale_bytes");
  if (rc != W4A16_OK) return rc;
  return ceil_div(N, kStrip) * ceil_div(groups_of(K, G), 8) * 32 * 8 * 2;
}

int w4a16_repack(const int32_t *packed_d, const uint16_t *scales_d, int64_t K, int64_t N, int G,
                 void *rw_d, void *rs_d, w4a16_stream_t stream) {
  int rc = check_gpu_shape(K, N, G, "w4a16_repack");
  if (rc != W4A16_OK) return rc;
  if (!packed_d || !scales_d || !rw_d || !rs_d)
    return fail(W4A16_ERR_INVALID, "w4a16_repack: null pointer");
  if (!aligned16(rw_d) || !aligned16(rs_d))
    return fail(W4A16_ERR_INVALID, "w4a16_repack: repacked buffers must be 16-byte aligned");
  hipError_t e = launch_repack(packed_d, scales_d, K, N, G, rw_d, rs_d, (hipStream_t)stream);
  return e == hipSuccess ? W4A16_OK : hip_fail(e, "w4a16_repack");
}

int w4a16_unrepack(const void *rw_d, const void *rs_d, int64_t K, int64_t N, int G,
                   int32_t *packed_d, uint16_t *scales_d, w4a16_stream_t stream) {
  int rc = check_gpu_shape(K, N, G, "w4a16_unrepack");
  if (rc != W4A16_OK) return rc;
  if (!packed_d || !scales_d || !rw_d || !rs_d)
    return fail(W4A16_ERR_INVALID, "w4a16_unrepack: null pointer");
  if (!aligned16(rw_d) || !aligned16(rs_d))
    return fail(W4A16_ERR_INVALID, "w4a16_unrepack: repacked buffers must be 16-byte aligned");
  hipError_t e = launch_unrepack(rw_d, rs_d, K, N, G, packed_d, scales_d, (hipStream_t)stream);
  return e == hipSuccess ? W4A16_OK : hip_fail(e, "w4a16_unrepack");
}

static int dequant_common(const void *rw_d, const void *rs_d, const void *rz_d, int64_t K,
                          int64_t N, int G, uint16_t *W_d, bool bf16, hipStream_t stream,
                          const char *who) {
  int rc = check_gpu_shape(K, N, G, who);
  if (rc != W4A16_OK) return rc;
  if (!rw_d || !rs_d || !W_d) return fail(W4A16_ERR_INVALID, "%s: null pointer", who);
  if (!aligned16(rw_d) || !aligned16(rs_d) || !aligned16(rz_d))
    return fail(W4A16_ERR_INVALID, "%s: repacked buffers must be 16-byte aligned", who);
  hipError_t e = launch_dequant_canonical(rw_d, rs_d, rz_d, K, N, G, bf16, W_d, stream);
  return e == hipSuccess ? W4A16_OK : hip_fail(e, who);
}

int w4a16_dequant(const void *rw_d, const void *rs_d, int64_t K, int64_t N, int G,
                  uint16_t *W16_d, w4a16_stream_t stream) {
  return dequant_common(rw_d, rs_d, nullptr, K, N, G, W16_d, false, (hipStream_t)stream,
                        "w4a16_dequant");
}

int w4a16_dequant_bf16(const void *rw_d, const void *rs_d, int64_t K, int64_t N, int G,
                       uint16_t *Wb_d, w4a16_stream_t stream) {
  return dequant_common(rw_d, rs_d, nullptr, K, N, G, Wb_d, true, (hipStream_t)stream,
                        "w4a16_dequant_bf16");
}

int w4a16_zero_rows(const uint16_t *scales_d, const uint8_t *zeros_d, int64_t K, int64_t N,
                    int G, void *rz_d, w4a16_stream_t stream) {
  const char *who = "w4a16_zero_rows";
  int rc = check_gpu_shape(K, N, G, who);
  if (rc != W4A16_OK) return rc;
  if (!scales_d || !zeros_d || !rz_d) return fail(W4A16_ERR_INVALID, "%s: null pointer", who);
  if (!aligned16(rz_d))
    return fail(W4A16_ERR_INVALID, "%s: the zero-row buffer must be 16-byte aligned", who);
  hipError_t e = launch_zero_rows(scales_d, zeros_d, K, N, G, rz_d, (hipStream_t)stream);
  return e == hipSuccess ? W4A16_OK : hip_fail(e, who);
}

int w4a16_dequant_zp(const void *rw_d, const void *rs_d, const void *rz_d, int64_t K, int64_t N,
                     int G, int flags, uint16_t *W_d, w4a16_stream_t stream) {
  const char *who = "w4a16_dequant_zp";
  if (flags & ~W4A16_FLAG_BF16) return fail(W4A16_ERR_INVALID, "%s: unknown flags 0x%x", who, flags);
  if (!rz_d) return fail(W4A16_ERR_INVALID, "%s: null pointer", who);
  return dequant_common(rw_d, rs_d, rz_d, K, N, G, W_d, (flags & W4A16_FLAG_BF16) != 0,
                        (hipStream_t)stream, who);
}

int w4a16_pack_int8(const float *W_d, int64_t K, int64_t N, int G, int32_t *packed_d,
                    uint16_t *scales_d, w4a16_stream_t stream) {
  const char *who = "w4a16_pack_int8";
  int rc = check_shape(K, N, G, who);
  if (rc != W4A16_OK) return rc;
  if (G % 4 != 0)
    return fail(W4A16_ERR_UNSUPPORTED, "%s: the GPU packer needs G % 4 == 0 (got %d)", who, G);
  if (K / G > 65535) return fail(W4A16_ERR_INVALID, "%s: K too large", who);
  if (!W_d || !packed_d || !scales_d) return fail(W4A16_ERR_INVALID, "%s: null pointer", who);
  hipError_t e = launch_pack8(W_d, K, N, G, packed_d, scales_d, (hipStream_t)stream);
  return e == hipSuccess ? W4A16_OK : hip_fail(e, who);
}

int64_t w4a16_repacked_weight_bytes_int8(int64_t K, int64_t N, int G) {
  int rc = check_gpu_shape(K, N, G, "w4a16_repacked_weight_bytes_int8");
  if (rc != W4A16_OK) return rc;
  return ceil_div(N, kStrip) * (K / kTileK) * 2 * kTileWords * 4;
}

int w4a16_repack_int8(const int32_t *packed_d, const uint16_t *scales_d, int64_t K, int64_t N,
                      int G, void *rw_d, void *rs_d, w4a16_stream_t stream) {
  const char *who = "w4a16_repack_int8";
  int rc = check_gpu_shape(K, N, G, who);
  if (rc != W4A16_OK) return rc;
  if (!packed_d || !scales_d || !rw_d || !rs_d) return fail(W4A16_ERR_INVALID, "%s: null pointer", who);
  if (!aligned16(rw_d) || !aligned16(rs_d))
    return fail(W4A16_ERR_INVALID, "%s: repacked buffers must be 16-byte aligned", who);
  hipError_t e = launch_repack8(packed_d, scales_d, K, N, G, rw_d, rs_d, (hipStream_t)stream);
  return e == hipSuccess ? W4A16_OK : hip_fail(e, who);
}

int w4a16_unrepack_int8(const void *rw_d, const void *rs_d, int64_t K, int64_t N, int G,
                        int32_t *packed_d, uint16_t *scales_d, w4a16_stream_t stream) {
  const char *who = "w4a16_unrepack_int8";
  int rc = check_gpu_shape(K, N, G, who);
  if (rc != W4A16_OK) return rc;
  if (!packed_d || !scales_d || !rw_d || !rs_d) return fail(W4A16_ERR_INVALID, "%s: null pointer", who);
  if (!aligned16(rw_d) || !aligned16(rs_d))
    return fail(W4A16_ERR_INVALID, "%s: repacked buffers must be 16-byte aligned", who);
  hipError_t e = launch_unrepack8(rw_d, rs_d, K, N, G, packed_d, scales_d, (hipStream_t)stream);
  return e == hipSuccess ? W4A16_OK : hip_fail(e, who);
}

int w4a16_dequant_int8(const void *rw_d, const void *rs_d, int64_t K, int64_t N, int G, int flags,
                       uint16_t *W_d, w4a16_stream_t stream) {
  const char *who = "w4a16_dequant_int8";
  if (flags & ~W4A16_FLAG_BF16) return fail(W4A16_ERR_INVALID, "%s: unknown flags 0x%x", who, flags);
  int rc = check_gpu_shape(K, N, G, who);
  if (rc != W4A16_OK) return rc;
  if (!rw_d || !rs_d || !W_d) return fail(W4A16_ERR_INVALID, "%s: null pointer", who);
  if (!aligned16(rw_d) || !aligned16(rs_d))
    return fail(W4A16_ERR_INVALID, "%s: repacked buffers must be 16-byte aligned", who);
  hipError_t e = launch_dequant8_canonical(rw_d, rs_d, K, N, G, (flags & W4A16_FLAG_BF16) != 0,
                                           W_d, (hipStream_t)stream);
  return e == hipSuccess ? W4A16_OK : hip_fail(e, who);
}

int w4a16_gemm_int8(const uint16_t *A_d, int64_t M, int64_t K, const void *rw_d, const void *rs_d,
                    int64_t N, int G, const float *rowscale_d, uint16_t *out_d, int flags,
                    void *workspace_d, int64_t workspace_bytes, w4a16_stream_t stream) {
  if (flags & ~(0xF | W4A16_FLAG_SWIGLU | W4A16_FLAG_BF16 | W4A16_FLAG_INT8))
    return fail(W4A16_ERR_INVALID, "w4a16_gemm_int8: unknown flags 0x%x", flags);
  return run_gemm(A_d, M, K, rw_d, rs_d, N, G, out_d, flags & ~W4A16_FLAG_INT8, workspace_d,
                  workspace_bytes, (hipStream_t)stream, rowscale_d, nullptr, "w4a16_gemm_int8", 8);
}

int w4a16_gemm(const uint16_t *A_d, int64_t M, int64_t K, const void *rw_d, const void *rs_d,
               int64_t N, int G, uint16_t *C_d, w4a16_stream_t stream) {
  return run_gemm(A_d, M, K, rw_d, rs_d, N, G, C_d, W4A16_PATH_AUTO, nullptr, 0,
                  (hipStream_t)stream);
}

int w4a16_gemm_swiglu(const uint16_t *A_d, int64_t M, int64_t K, const void *rw_d,
                      const void *rs_d, int64_t N, int G, uint16_t *Z_d, w4a16_stream_t stream) {
  return run_gemm(A_d, M, K, rw_d, rs_d, N, G, Z_d, W4A16_PATH_AUTO | W4A16_FLAG_SWIGLU, nullptr,
                  0, (hipStream_t)stream);
}

int w4a16_gemm_ex(const uint16_t *A_d, int64_t M, int64_t K, const void *rw_d, const void *rs_d,
                  int64_t N, int G, uint16_t *out_d, int flags, void *workspace_d,
                  int64_t workspace_bytes, w4a16_stream_t stream) {
  if (flags & ~(0xF | W4A16_FLAG_SWIGLU | W4A16_FLAG_BF16))
    return fail(W4A16_ERR_INVALID, "w4a16_gemm_ex: unknown flags 0x%x", flags);
  return run_gemm(A_d, M, K, rw_d, rs_d, N, G, out_d, flags, workspace_d, workspace_bytes,
                  (hipStream_t)stream);
}

int w4a16_gemm_noalloc(const uint16_t *A_d, int64_t M, int64_t K, const void *rw_d,
                       const void *rs_d, int64_t N, int G, uint16_t *out_d, int flags,
                       w4a16_stream_t stream) {
  const char *who = "w4a16_gemm_noalloc";
  if (flags & ~(0xF | W4A16_FLAG_SWIGLU | W4A16_FLAG_BF16))
    return fail(W4A16_ERR_INVALID, "%s: unknown flags 0x%x", who, flags);
  void *ws = nullptr;
  int rc = scratch_address(&ws);
  if (rc != W4A16_OK) return rc;
  return run_gemm(A_d, M, K, rw_d, rs_d, N, G, out_d, flags, ws, kScratchBytes,
                  (hipStream_t)stream, nullptr, nullptr, who, 4, true);
}

int64_t w4a16_noalloc_scratch_bytes(void) { return kScratchBytes; }

int w4a16_gemm_rowscale(const uint16_t *A_d, int64_t M, int64_t K, const void *rw_d,
                        const void *rs_d, int64_t N, int G, const float *rowscale_d,
                        uint16_t *out_d, int flags, void *workspace_d, int64_t workspace_bytes,
                        w4a16_stream_t stream) {
  if (flags & ~(0xF | W4A16_FLAG_SWIGLU | W4A16_FLAG_BF16))
    return fail(W4A16_ERR_INVALID, "w4a16_gemm_rowscale: unknown flags 0x%x", flags);
  if (M > 0 && rowscale_d == nullptr)
    return fail(W4A16_ERR_INVALID, "w4a16_gemm_rowscale: null row scale");
  return run_gemm(A_d, M, K, rw_d, rs_d, N, G, out_d, flags, workspace_d, workspace_bytes,
                  (hipStream_t)stream, rowscale_d);
}

int w4a16_gemm_zp(const uint16_t *A_d, int64_t M, int64_t K, const void *rw_d, const void *rs_d,
                  const void *rz_d, int64_t N, int G, const float *rowscale_d, uint16_t *out_d,
                  int flags, void *workspace_d, int64_t workspace_bytes, w4a16_stream_t stream) {
  if (flags & ~(0xF | W4A16_FLAG_SWIGLU | W4A16_FLAG_BF16 | W4A16_FLAG_ZP))
    return fail(W4A16_ERR_INVALID, "w4a16_gemm_zp: unknown flags 0x%x", flags);
  if (M > 0 && rz_d == nullptr) return fail(W4A16_ERR_INVALID, "w4a16_gemm_zp: null zero rows");
  return run_gemm(A_d, M, K, rw_d, rs_d, N, G, out_d, flags & ~W4A16_FLAG_ZP, workspace_d,
                  workspace_bytes, (hipStream_t)stream, rowscale_d, rz_d, "w4a16_gemm_zp");
}

int w4a16_rms_rowscale(const uint16_t *A_d, int64_t M, int64_t K, float eps, int flags,
                       float *rho_d, w4a16_stream_t stream) {
  const char *who = "w4a16_rms_rowscale";
  if (flags & ~W4A16_FLAG_BF16) return fail(W4A16_ERR_INVALID, "%s: unknown flags 0x%x", who, flags);
  if (M < 0 || K <= 0 || K % 8 != 0)
    return fail(W4A16_ERR_INVALID, "%s: need M >= 0 and K a positive multiple of 8", who);
  if (M > ((int64_t)1 << 30) || K > ((int64_t)1 << 30))
    return fail(W4A16_ERR_INVALID, "%s: M or K too large", who);
  if (!(eps >= 0.0f) || !std::isfinite(eps))
    return fail(W4A16_ERR_INVALID, "%s: eps must be finite and >= 0", who);
  if (M == 0) return W4A16_OK;
  if (!A_d || !rho_d) return fail(W4A16_ERR_INVALID, "%s: null pointer", who);
  if (!aligned16(A_d)) return fail(W4A16_ERR_INVALID, "%s: A must be 16-byte aligned", who);
  hipError_t e = launch_rms_rowscale(A_d, M, K, eps, (flags & W4A16_FLAG_BF16) != 0, rho_d,
                                     (hipStream_t)stream);
  return e == hipSuccess ? W4A16_OK : hip_fail(e, who);
}

int64_t w4a16_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N, int G, int flags) {
  int rc = check_gpu_shape(K, N, G, "w4a16_gemm_workspace_bytes");
  if (rc != W4A16_OK) return rc;
  if (M <= 0) return 0;
  const int bits = (flags & W4A16_FLAG_INT8) ? 8 : 4;
  Problem p{nullptr, M, K, N, nullptr, nullptr, nullptr, (flags & W4A16_FLAG_SWIGLU) != 0,
            (flags & W4A16_FLAG_BF16) != 0, nullptr, G, group_shift(K, G), nullptr,
            (flags & W4A16_FLAG_ZP) != 0, bits};
  const char *why = nullptr;
  const int path = resolve_path(p, flags & 0xF, &why);
  if (path < 0)
    return fail(W4A16_ERR_UNSUPPORTED, "w4a16_gemm_workspace_bytes: beyond the decode path");
  // The launch on a caller's workspace can differ from the one on the
  // library's (K splits that only a launch on the library's workspace finishes
  // itself): the size covers both, for w4a16_gemm_ex and for
  // w4a16_reserve_workspace alike.
  const int64_t own = workspace_for(path, p);
  p.own_ws = false;
  const int64_t caller = workspace_for(path, p);
  return own > caller ? own : caller;
}

int w4a16_describe(int64_t M, int64_t K, int64_t N, int G, int flags, char *buf, int64_t len) {
  int rc = check_gpu_shape(K, N, G, "w4a16_describe");
  if (rc != W4A16_OK) return rc;
  if (M < 1) return fail(W4A16_ERR_INVALID, "w4a16_describe: M must be >= 1");
  if (buf == nullptr || len < 1) return fail(W4A16_ERR_INVALID, "w4a16_describe: no buffer");
  if (flags & ~(0xF | W4A16_FLAG_SWIGLU | W4A16_FLAG_BF16 | W4A16_FLAG_ZP | W4A16_FLAG_INT8))
    return fail(W4A16_ERR_INVALID, "w4a16_describe: unknown flags 0x%x", flags);
  if ((flags & W4A16_FLAG_ZP) && (flags & W4A16_FLAG_INT8))
    return fail(W4A16_ERR_UNSUPPORTED, "w4a16_describe: INT8 weights have no zero points");
  const int bits = (flags & W4A16_FLAG_INT8) ? 8 : 4;
  const bool swiglu = (flags & W4A16_FLAG_SWIGLU) != 0;
  if (swiglu && N % 64 != 0)
    return fail(W4A16_ERR_INVALID, "w4a16_describe: N (%lld) must be a multiple of 64",
                (long long)N);
  if ((flags & 0xF) > W4A16_PATH_DENSE)
    return fail(W4A16_ERR_INVALID, "w4a16_describe: unknown path %d", flags & 0xF);
  Problem p{nullptr, M, K, N, nullptr, nullptr, nullptr, swiglu, (flags & W4A16_FLAG_BF16) != 0,
            nullptr, G, group_shift(K, G), nullptr, (flags & W4A16_FLAG_ZP) != 0, bits};
  const char *why = nullptr;
  const int path = resolve_path(p, flags & 0xF, &why);
  if (path < 0)
    return fail(W4A16_ERR_UNSUPPORTED, "w4a16_describe: beyond the decode kernels' offsets");
  char tmp[1024];
  int k;
  if (path == W4A16_PATH_DECODE) {
    Problem q = p;
    q.M = M < kDecodeMaxM ? M : kDecodeMaxM;
    k = decode_describe(q, tmp, sizeof tmp);
    const int64_t slices = ceil_div(M, kDecodeMaxM);
    if (slices > 1 && k > 0 && k < (int)sizeof tmp)
      k += snprintf(tmp + k, sizeof tmp - k, " (x%lld row slices of 32)", (long long)(M / 32));
    if (slices > 1 && M % kDecodeMaxM != 0 && k > 0 && k < (int)sizeof tmp) {
      // The trailing slice may take another configuration.
      q.M = M % kDecodeMaxM;
      k += snprintf(tmp + k, sizeof tmp - k, "; last %lld rows: ", (long long)q.M);
      if (k > 0 && k < (int)sizeof tmp) {
        const int t = decode_describe(q, tmp + k, sizeof tmp - k);
        if (t < 0) return fail(W4A16_ERR_INVALID, "w4a16_describe: formatting failed");
        k += t;
      }
    }
  } else {
    k = tiled_describe(p, path == W4A16_PATH_DENSE, tmp, sizeof tmp);
  }
  if (why != nullptr && k > 0 && k < (int)sizeof tmp)
    k += snprintf(tmp + k, sizeof tmp - k, " (fallback %s)", why);
  if (k < 0) return fail(W4A16_ERR_INVALID, "w4a16_describe: formatting failed");
  snprintf(buf, (size_t)len, "%s", tmp);
  return k < len ? k : (int)(len - 1);
}

int w4a16_select_path(int64_t M, int64_t K, int64_t N, int G, int flags) {
  int rc = check_gpu_shape(K, N, G, "w4a16_select_path");
  if (rc != W4A16_OK) return rc;
  if (M < 0) return fail(W4A16_ERR_INVALID, "w4a16_select_path: M must be >= 0");
  Problem p{nullptr, M, K, N, nullptr, nullptr, nullptr, (flags & W4A16_FLAG_SWIGLU) != 0,
            (flags & W4A16_FLAG_BF16) != 0, nullptr, G, group_shift(K, G), nullptr,
            (flags & W4A16_FLAG_ZP) != 0, (flags & W4A16_FLAG_INT8) ? 8 : 4};
  const char *why = nullptr;
  return resolve_path(p, W4A16_PATH_AUTO, &why);
}

int w4a16_reserve_workspace(int64_t bytes) {
  if (bytes < 0) return fail(W4A16_ERR_INVALID, "w4a16_reserve_workspace: bytes must be >= 0");
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != W4A16_OK) return rc;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  DeviceWorkspace &w = workspace_of(dev);
  if (w.bytes >= bytes) return drain_workspace(w, false);
  if (w.ptr != nullptr) w.retired.push_back(w.ptr);
  w.ptr = nullptr;
  w.bytes = 0;
  rc = drain_workspace(w, false);
  if (rc != W4A16_OK) return rc;
  if (bytes == 0) return W4A16_OK;
  void *p = nullptr;
  hipError_t e = hipMalloc(&p, (size_t)bytes);
  if (e != hipSuccess)
    return fail(W4A16_ERR_WORKSPACE, "w4a16_reserve_workspace: allocation of %lld bytes failed: %s",
                (long long)bytes, hipGetErrorString(e));
  w.ptr = p;
  w.bytes = bytes;
  return W4A16_OK;
}

int64_t w4a16_workspace_reserved(void) {
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != W4A16_OK) return rc;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  return workspace_of(dev).bytes;
}

int w4a16_release_workspace(void) {
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != W4A16_OK) return rc;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  return drain_workspace(workspace_of(dev), true);
}

const char *w4a16_last_fallback(void) {
  static thread_local std::string copy;
  std::lock_guard<std::mutex> lock(g_fb_mutex);
  copy = g_fb_last;
  return copy.c_str();
}

}  // extern "C"
