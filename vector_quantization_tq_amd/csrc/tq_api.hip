// C ABI of libtq (declared in include/tq.h): argument checks, the quantizer
// object and its device tables, and kernel launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/tq.h"
#include "tq_internal.h"
#include "tq_kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(TQ_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Walsh masks in the order the kernels use (odd subsets of the index bits).
const int kMasks[4][8] = {{1}, {1, 2}, {1, 2, 4, 7}, {1, 2, 4, 8, 7, 11, 13, 14}};

bool fill_codebook(int d, int bp, tq::Codebook& cb) {
  const int K = 1 << bp;
  std::vector<double> c(K), t(K - 1);
  if (tq::codebook(d, K, c.data(), t.data()) != 0) return false;
  cb.bp = bp;
  cb.levels = K;
  cb.nterms = K / 2;
  for (int k = 0; k < K; ++k) cb.c[k] = static_cast<float>(c[k]);
  for (int k = 0; k < K - 1; ++k) cb.t[k] = static_cast<float>(t[k]);
  // coefficients in the +-1 basis: coef_S = mean_idx c[idx] prod_{p in S} s_p
  double csum = 0;
  for (int i = 0; i < cb.nterms; ++i) {
    const int mk = kMasks[bp - 1][i];
    double a = 0;
    for (int idx = 0; idx < K; ++idx) {
      double sgn = 1;
      for (int p = 0; p < bp; ++p)
        if (mk & (1 << p)) sgn *= ((idx >> p) & 1) ? 1.0 : -1.0;
      a += c[idx] * sgn;
    }
    a /= K;
    cb.mask[i] = mk;
    cb.coef[i] = static_cast<float>(a);
    csum += a;
  }
  cb.coef_sum = static_cast<float>(csum);
  // the expansion must reproduce the codebook (symmetric => odd subsets only)
  for (int idx = 0; idx < K; ++idx) {
    double v = 0;
    for (int i = 0; i < cb.nterms; ++i) {
      double sgn = 1;
      for (int p = 0; p < bp; ++p)
        if (cb.mask[i] & (1 << p)) sgn *= ((idx >> p) & 1) ? 1.0 : -1.0;
      v += static_cast<double>(cb.coef[i]) * sgn;
    }
    if (std::fabs(v - c[idx]) > 1e-6 * (std::fabs(c[idx]) + 1e-3)) return false;
  }
  return true;
}

struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

int check_quantizer(const tq_quantizer* q) {
  if (!q) return fail(TQ_EINVAL, "quantizer is NULL");
  return TQ_OK;
}

int check_mode(const tq_quantizer* q, int mode) {
  if (mode != TQ_PROD && mode != TQ_MSE && mode != TQ_MSE_KEYS)
    return fail(TQ_EINVAL, "mode must be TQ_PROD, TQ_MSE or TQ_MSE_KEYS");
  if (q->cb[mode == TQ_PROD ? 0 : 1].bp < 1) return fail(TQ_EINVAL, "prod mode needs bits >= 2 (bits=%d)", q->bits);
  return TQ_OK;
}

// the quantizer's key encoding is readable by the scoring kernels
int check_keys(const tq_quantizer* q) {
  if (tq::key_codebook(q).bp < 1) return fail(TQ_EINVAL, "prod keys need bits >= 2 (bits=%d)", q->bits);
  return TQ_OK;
}

// Library-owned workspace of tq_attend_decode_noalloc: one copy per device,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, taken once per device (with that device current) when
// a quantizer is made there, and only that address is ever passed on.
static __device__ __align__(256) uint8_t scratch[TQ_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// with device `dev` current
int scratch_setup(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return fail(TQ_EUNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev]) return TQ_OK;
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  g_scratch[dev] = p;
  return TQ_OK;
}

void* scratch_of(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch[dev];
}

}  // namespace

extern "C" {

int tq_version(void) { return 1; }

const char* tq_last_error(void) { return g_last_error.c_str(); }

int tq_host_normals(uint64_t seed, int tag, int64_t n, double* out) {
  if (n < 0 || (n > 0 && !out)) return fail(TQ_EINVAL, "bad n or NULL output");
  tq::normals(seed, tag, n, out);
  return TQ_OK;
}

int tq_host_rotation(int d, uint64_t seed, double* pi_out) {
  if (d < 3 || d > 1024 || !pi_out) return fail(TQ_EINVAL, "need 3 <= d <= 1024 and an output array");
  tq::rotation(d, seed, pi_out);
  return TQ_OK;
}

int tq_host_rotation_hadamard(int d, uint64_t seed, double* pi_out) {
  if (d < 4 || d > 1024 || (d & (d - 1)) || !pi_out)
    return fail(TQ_EINVAL, "need d a power of two in [4, 1024] and an output array");
  tq::rotation_hadamard(d, seed, pi_out);
  return TQ_OK;
}

int tq_host_qjl_matrix(int m, int d, uint64_t seed, double* s_out) {
  if (m < 1 || d < 1 || !s_out) return fail(TQ_EINVAL, "need m, d >= 1 and an output array");
  tq::qjl_matrix(m, d, seed, s_out);
  return TQ_OK;
}

int tq_host_codebook(int d, int levels, double* centroids, double* thresholds) {
  if (d < 3 || d > 1024) return fail(TQ_EINVAL, "need 3 <= d <= 1024");
  if (levels != 2 && levels != 4 && levels != 8 && levels != 16) return fail(TQ_EINVAL, "levels must be 2, 4, 8 or 16");
  if (!centroids || !thresholds) return fail(TQ_EINVAL, "NULL output");
  if (tq::codebook(d, levels, centroids, thresholds) != 0) return fail(TQ_EINVAL, "codebook failed");
  return TQ_OK;
}

tq_quantizer* tq_make_quantizer(int d, int bits, uint64_t seed) { return tq_make_quantizer_ex(d, bits, seed, TQ_ROT_HAAR); }

tq_quantizer* tq_make_quantizer_ex(int d, int bits, uint64_t seed, int rotation) {
  if (d < 3 || d > 1024) { fail(TQ_EINVAL, "d=%d out of [3, 1024]", d); return nullptr; }
  if (bits < 1 || bits > 4) { fail(TQ_EINVAL, "bits=%d out of [1, 4]", bits); return nullptr; }
  if (rotation != TQ_ROT_HAAR && rotation != TQ_ROT_HADAMARD) {
    fail(TQ_EINVAL, "rotation must be TQ_ROT_HAAR or TQ_ROT_HADAMARD");
    return nullptr;
  }
  if (rotation == TQ_ROT_HADAMARD && (d < 4 || (d & (d - 1)))) {
    fail(TQ_EINVAL, "the Hadamard rotation needs d a power of two >= 4 (d=%d)", d);
    return nullptr;
  }
  tq_quantizer* q = new (std::nothrow) tq_quantizer();
  if (!q) { fail(TQ_ENOMEM, "host allocation failed"); return nullptr; }
  q->d = d;
  q->bits = bits;
  q->m = d;
  q->seed = seed;
  q->rotation = rotation;
  q->pi.resize(static_cast<size_t>(d) * d);
  q->s.resize(static_cast<size_t>(q->m) * d);
  if (rotation == TQ_ROT_HADAMARD)
    tq::rotation_hadamard(d, seed, q->pi.data());
  else
    tq::rotation(d, seed, q->pi.data());
  tq::qjl_matrix(q->m, d, seed, q->s.data());
  if (bits >= 2 && !fill_codebook(d, bits - 1, q->cb[TQ_PROD])) { fail(TQ_EINVAL, "prod codebook failed"); delete q; return nullptr; }
  if (!fill_codebook(d, bits, q->cb[TQ_MSE])) { fail(TQ_EINVAL, "mse codebook failed"); delete q; return nullptr; }

  std::vector<float> pi32(q->pi.size()), s32(q->s.size()), sp32(q->s.size());
  for (size_t i = 0; i < q->pi.size(); ++i) pi32[i] = static_cast<float>(q->pi[i]);
  for (size_t i = 0; i < q->s.size(); ++i) s32[i] = static_cast<float>(q->s[i]);
  for (int r = 0; r < q->m; ++r)
    for (int j = 0; j < d; ++j) {   // S' = S Pi^T: S'[r][j] = sum_k S[r][k] Pi[j][k]
      double a = 0;
      for (int k = 0; k < d; ++k) a += q->s[static_cast<size_t>(r) * d + k] * q->pi[static_cast<size_t>(j) * d + k];
      sp32[static_cast<size_t>(r) * d + j] = static_cast<float>(a);
    }
  std::vector<float> spt32(sp32.size());   // S' k-major for the general-d encoder
  for (int r = 0; r < q->m; ++r)
    for (int j = 0; j < d; ++j) spt32[static_cast<size_t>(j) * q->m + r] = sp32[static_cast<size_t>(r) * d + j];
  const int dm = d + q->m;
  std::vector<float> qt32(static_cast<size_t>(d) * dm);
  for (int k = 0; k < d; ++k) {
    for (int j = 0; j < d; ++j) qt32[static_cast<size_t>(k) * dm + j] = pi32[static_cast<size_t>(j) * d + k];
    for (int r = 0; r < q->m; ++r) qt32[static_cast<size_t>(k) * dm + d + r] = s32[static_cast<size_t>(r) * d + k];
  }
  hipError_t e = hipGetDevice(&q->device);
  if (e != hipSuccess) { hip_fail(e, "hipGetDevice"); delete q; return nullptr; }
  // raise the dynamic-LDS limit of the large encode tiles; if the runtime
  // refuses, launches that need more than the default report the error
  if (tq::set_kernel_attributes() != hipSuccess) (void)hipGetLastError();
  // device address of the allocation-free entry point's scratch array on this
  // device (a failure here is retried, and reported, by that entry point)
  if (scratch_setup(q->device) != TQ_OK) (void)hipGetLastError();
  const size_t bp = pi32.size() * sizeof(float), bs = s32.size() * sizeof(float);
  if ((e = hipMalloc(&q->d_pi, bp)) != hipSuccess || (e = hipMalloc(&q->d_s, bs)) != hipSuccess ||
      (e = hipMalloc(&q->d_sp, bs)) != hipSuccess ||
      (e = hipMalloc(&q->d_qt, qt32.size() * sizeof(float))) != hipSuccess ||
      (e = hipMalloc(&q->d_spt, bs)) != hipSuccess) {
    hip_fail(e, "hipMalloc");
    tq_free_quantizer(q);
    return nullptr;
  }
  if ((e = hipMemcpy(q->d_pi, pi32.data(), bp, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(q->d_s, s32.data(), bs, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(q->d_sp, sp32.data(), bs, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(q->d_qt, qt32.data(), qt32.size() * sizeof(float), hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(q->d_spt, spt32.data(), bs, hipMemcpyHostToDevice)) != hipSuccess) {
    hip_fail(e, "hipMemcpy");
    tq_free_quantizer(q);
    return nullptr;
  }
  if (d > 128 && d <= 256) {
    // the eight-wave encoder's operands: Pi and S' scaled by 2^8 and split into
    // fp16 hi + lo (rounded to nearest), rows j < d, columns k < d, zero padded
    // to 256 x 256
    constexpr int W = 256;
    std::vector<_Float16> wide(static_cast<size_t>(4) * W * W, static_cast<_Float16>(0.f));
    for (int j = 0; j < d; ++j)
      for (int k = 0; k < d; ++k) {
        const float vp = pi32[static_cast<size_t>(j) * d + k] * 256.f;
        const float vs = sp32[static_cast<size_t>(j) * d + k] * 256.f;
        const _Float16 ph = static_cast<_Float16>(vp), sh = static_cast<_Float16>(vs);
        const size_t o = static_cast<size_t>(j) * W + k;
        wide[o] = ph;
        wide[static_cast<size_t>(W) * W + o] = static_cast<_Float16>(vp - static_cast<float>(ph));
        wide[static_cast<size_t>(2) * W * W + o] = sh;
        wide[static_cast<size_t>(3) * W * W + o] = static_cast<_Float16>(vs - static_cast<float>(sh));
      }
    const size_t bw = wide.size() * sizeof(_Float16);
    if ((e = hipMalloc(&q->d_wide, bw)) != hipSuccess ||
        (e = hipMemcpy(q->d_wide, wide.data(), bw, hipMemcpyHostToDevice)) != hipSuccess) {
      hip_fail(e, "wide encoder tables");
      tq_free_quantizer(q);
      return nullptr;
    }
  }
  return q;
}

void tq_free_quantizer(tq_quantizer* q) {
  if (!q) return;
  if (q->d_pi || q->d_s || q->d_sp || q->d_qt || q->d_spt || q->d_wide) {
    DeviceGuard g(q->device);
    if (q->d_wide) (void)hipFree(q->d_wide);
    if (q->d_pi) (void)hipFree(q->d_pi);
    if (q->d_s) (void)hipFree(q->d_s);
    if (q->d_sp) (void)hipFree(q->d_sp);
    if (q->d_qt) (void)hipFree(q->d_qt);
    if (q->d_spt) (void)hipFree(q->d_spt);
  }
  delete q;
}

int tq_quantizer_info(const tq_quantizer* q, int* d, int* bits, int* m) {
  if (int r = check_quantizer(q)) return r;
  if (d) *d = q->d;
  if (bits) *bits = q->bits;
  if (m) *m = q->m;
  return TQ_OK;
}

int tq_set_key_mode(tq_quantizer* q, int key_mode) {
  if (int r = check_quantizer(q)) return r;
  if (key_mode != TQ_PROD && key_mode != TQ_MSE_KEYS) return fail(TQ_EINVAL, "key mode must be TQ_PROD or TQ_MSE_KEYS");
  if (key_mode == TQ_PROD && q->cb[TQ_PROD].bp < 1) return fail(TQ_EINVAL, "prod keys need bits >= 2 (bits=%d)", q->bits);
  q->key_mode = key_mode;
  return TQ_OK;
}

int64_t tq_code_words(const tq_quantizer* q, int mode, int64_t nseq, int64_t n) {
  if (check_quantizer(q) || check_mode(q, mode)) return -1;
  if (nseq < 0 || n < 0) return fail(TQ_EINVAL, "negative size");
  if (mode == TQ_PROD) return nseq * n * ((q->d + 31) / 32) * (q->cb[0].bp + 1);
  if (mode == TQ_MSE_KEYS) return nseq * n * ((q->d + 31) / 32) * q->cb[1].bp;
  return nseq * ((n + 31) / 32) * q->cb[1].bp * q->d;
}

int tq_encode(const tq_quantizer* q, int mode, const void* x, int dtype, int64_t nseq, int64_t n, uint32_t* codes,
              float* norms, float* gammas, void* stream) {
  if (int r = check_quantizer(q)) return r;
  if (int r = check_mode(q, mode)) return r;
  if (dtype != TQ_F32 && dtype != TQ_BF16) return fail(TQ_EINVAL, "dtype must be TQ_F32 or TQ_BF16");
  if (nseq < 0 || n < 0) return fail(TQ_EINVAL, "negative size");
  if (nseq * n == 0) return TQ_OK;
  if (!x || !codes || !norms || (mode == TQ_PROD && !gammas)) return fail(TQ_EINVAL, "NULL array argument");
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(norms, 16) || (gammas && !aligned(gammas, 16)))
    return fail(TQ_EINVAL, "device pointers must be 16-byte aligned");
  if (q->d > tq::kMaxEncodeD) return fail(TQ_EUNSUPPORTED, "encode supports d <= %d (d=%d)", tq::kMaxEncodeD, q->d);
  if (nseq > 65535) return fail(TQ_EUNSUPPORTED, "nseq > 65535");
  DeviceGuard g(q->device);
  if (!g.ok) return fail(TQ_EHIP, "cannot select the quantizer's device");
  hipError_t e = tq::launch_encode(q, mode, x, dtype, nseq, n, codes, norms, gammas, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e, "encode launch");
}

int tq_decode(const tq_quantizer* q, int mode, const uint32_t* codes, const float* norms, const float* gammas,
              int64_t nseq, int64_t n, float* x_out, void* stream) {
  if (int r = check_quantizer(q)) return r;
  if (int r = check_mode(q, mode)) return r;
  if (nseq < 0 || n < 0) return fail(TQ_EINVAL, "negative size");
  if (nseq * n == 0) return TQ_OK;
  if (!codes || !norms || !x_out || (mode == TQ_PROD && !gammas)) return fail(TQ_EINVAL, "NULL array argument");
  if (!aligned(codes, 16) || !aligned(norms, 16) || !aligned(x_out, 16) || (gammas && !aligned(gammas, 16)))
    return fail(TQ_EINVAL, "device pointers must be 16-byte aligned");
  if (nseq > 65535) return fail(TQ_EUNSUPPORTED, "nseq > 65535");
  DeviceGuard g(q->device);
  if (!g.ok) return fail(TQ_EHIP, "cannot select the quantizer's device");
  hipError_t e = tq::launch_decode(q, mode, codes, norms, gammas, nseq, n, x_out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e, "decode launch");
}

static int check_heads(int B, int Hq, int Hkv) {
  if (B < 1 || Hq < 1 || Hkv < 1) return fail(TQ_EINVAL, "B, Hq, Hkv must be >= 1");
  if (Hq % Hkv) return fail(TQ_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  return TQ_OK;
}

int64_t tq_scores_workspace_bytes(const tq_quantizer* q, int B, int Hq, int Hkv, int64_t n, int topk) {
  if (check_quantizer(q) || check_heads(B, Hq, Hkv)) return -1;
  if (int r = check_keys(q)) return r;
  if (topk > 0) return tq::topk_ws_bytes(q, B, Hq, Hkv, n, topk);
  return tq::scores_ws_bytes(q, B, Hq, Hkv);
}

int tq_scores(const tq_quantizer* q, const void* queries, int q_dtype, int B, int Hq, int Hkv, const uint32_t* codes,
              const float* norms, const float* gammas, int64_t n, int topk, float* out, int64_t* out_idx,
              void* workspace, int64_t ws_bytes, void* stream) {
  if (int r = check_quantizer(q)) return r;
  if (int r = check_heads(B, Hq, Hkv)) return r;
  if (int r = check_keys(q)) return r;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return fail(TQ_EINVAL, "q_dtype must be TQ_F32 or TQ_BF16");
  if (n < 0) return fail(TQ_EINVAL, "negative n");
  if (topk < 0 || topk > 32) return fail(TQ_EINVAL, "topk must be in [0, 32]");
  if (topk > 0 && n < topk) return fail(TQ_EINVAL, "topk (%d) larger than n (%lld)", topk, static_cast<long long>(n));
  if (n == 0) return TQ_OK;
  if (!tq::key_qjl(q)) gammas = nullptr;   // MSE-only keys carry no gamma
  if (!queries || !codes || !norms || (tq::key_qjl(q) && !gammas) || !out || (topk > 0 && !out_idx))
    return fail(TQ_EINVAL, "NULL array argument");
  if (!aligned(queries, 16) || !aligned(codes, 16) || !aligned(norms, 16) || (gammas && !aligned(gammas, 16)) ||
      !aligned(out, 16) || (out_idx && !aligned(out_idx, 16)))
    return fail(TQ_EINVAL, "device pointers must be 16-byte aligned");
  if (q->d > tq::kMaxEncodeD) return fail(TQ_EUNSUPPORTED, "scores support d <= %d (d=%d)", tq::kMaxEncodeD, q->d);
  if (q->d > 256 && topk > 0) return fail(TQ_EUNSUPPORTED, "top-k supports d <= 256 (d=%d)", q->d);
  const int64_t need = tq_scores_workspace_bytes(q, B, Hq, Hkv, n, topk);
  if (need < 0) return TQ_EINVAL;
  if (!workspace || ws_bytes < need)
    return fail(TQ_EWORKSPACE, "workspace of %lld bytes needed", static_cast<long long>(need));
  if (!aligned(workspace, 256)) return fail(TQ_EINVAL, "workspace must be 256-byte aligned");
  if (static_cast<int64_t>(B) * Hkv * ((Hq / Hkv + 3) / 4) > 65535) return fail(TQ_EUNSUPPORTED, "too many groups");
  DeviceGuard g(q->device);
  if (!g.ok) return fail(TQ_EHIP, "cannot select the quantizer's device");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = topk > 0 ? tq::launch_topk(q, queries, q_dtype, B, Hq, Hkv, codes, norms, gammas, n, topk, out, out_idx,
                                            workspace, st)
                          : tq::launch_scores(q, queries, q_dtype, B, Hq, Hkv, codes, norms, gammas, n, out, workspace, st);
  if (e == hipErrorNotSupported) return fail(TQ_EUNSUPPORTED, "shape not supported by the scores kernels");
  return e == hipSuccess ? TQ_OK : hip_fail(e, "scores launch");
}

int tq_query_prep(const tq_quantizer* q, const void* queries, int q_dtype, int B, int Hq, int Hkv, void* workspace,
                  int64_t ws_bytes, void* stream) {
  if (int r = check_quantizer(q)) return r;
  if (int r = check_heads(B, Hq, Hkv)) return r;
  if (int r = check_keys(q)) return r;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return fail(TQ_EINVAL, "q_dtype must be TQ_F32 or TQ_BF16");
  if (!queries) return fail(TQ_EINVAL, "NULL queries");
  if (!aligned(queries, 16)) return fail(TQ_EINVAL, "device pointers must be 16-byte aligned");
  if (q->d > 256) return fail(TQ_EUNSUPPORTED, "the split query-prep path supports d <= 256 (d=%d)", q->d);
  const int64_t need = tq::scores_ws_bytes(q, B, Hq, Hkv);
  if (!workspace || ws_bytes < need)
    return fail(TQ_EWORKSPACE, "workspace of %lld bytes needed", static_cast<long long>(need));
  if (!aligned(workspace, 256)) return fail(TQ_EINVAL, "workspace must be 256-byte aligned");
  if (static_cast<int64_t>(B) * Hkv * ((Hq / Hkv + 3) / 4) * 4 > 0x7fffffff) return fail(TQ_EUNSUPPORTED, "too many queries");
  DeviceGuard g(q->device);
  if (!g.ok) return fail(TQ_EHIP, "cannot select the quantizer's device");
  hipError_t e = tq::launch_query_prep_ws(q, queries, q_dtype, B, Hq, Hkv, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e, "query prep launch");
}

int tq_scores_from_prep(const tq_quantizer* q, int B, int Hq, int Hkv, const uint32_t* codes, const float* norms,
                        const float* gammas, int64_t n, float* logits, const void* workspace, int64_t ws_bytes,
                        void* stream) {
  if (int r = check_quantizer(q)) return r;
  if (int r = check_heads(B, Hq, Hkv)) return r;
  if (int r = check_keys(q)) return r;
  if (n < 0) return fail(TQ_EINVAL, "negative n");
  if (n == 0) return TQ_OK;
  if (!tq::key_qjl(q)) gammas = nullptr;   // MSE-only keys carry no gamma
  if (!codes || !norms || (tq::key_qjl(q) && !gammas) || !logits) return fail(TQ_EINVAL, "NULL array argument");
  if (!aligned(codes, 16) || !aligned(norms, 16) || (gammas && !aligned(gammas, 16)) || !aligned(logits, 16))
    return fail(TQ_EINVAL, "device pointers must be 16-byte aligned");
  if (q->d > 256) return fail(TQ_EUNSUPPORTED, "the split query-prep path supports d <= 256 (d=%d)", q->d);
  const int64_t need = tq::scores_ws_bytes(q, B, Hq, Hkv);
  if (!workspace || ws_bytes < need)
    return fail(TQ_EWORKSPACE, "workspace of %lld bytes needed", static_cast<long long>(need));
  if (!aligned(workspace, 256)) return fail(TQ_EINVAL, "workspace must be 256-byte aligned");
  if (static_cast<int64_t>(B) * Hkv * ((Hq / Hkv + 3) / 4) > 65535) return fail(TQ_EUNSUPPORTED, "too many groups");
  DeviceGuard g(q->device);
  if (!g.ok) return fail(TQ_EHIP, "cannot select the quantizer's device");
  hipError_t e = tq::launch_scores_scan(q, B, Hq, Hkv, codes, norms, gammas, n, logits, workspace,
                                        static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return fail(TQ_EUNSUPPORTED, "shape not supported by the scores kernels");
  return e == hipSuccess ? TQ_OK : hip_fail(e, "scores launch");
}

int64_t tq_attend_workspace_bytes(const tq_quantizer* kq, const tq_quantizer* vq, int B, int Hq, int Hkv, int64_t n_comp,
                                  int n_tail) {
  if (check_quantizer(kq) || check_quantizer(vq) || check_heads(B, Hq, Hkv)) return -1;
  if (kq->d != vq->d) return fail(TQ_EINVAL, "key and value quantizers differ in d");
  if (n_comp < 0 || n_tail < 0) return fail(TQ_EINVAL, "negative size");
  return tq::attend_ws_bytes(kq, vq, B, Hq, Hkv, n_comp, n_tail);
}

}  // extern "C"

// Argument checks and launch of decode attention.  With `noalloc` the
// workspace is the device's scratch array (workspace/ws_bytes unused): the
// call then allocates nothing and rejects shapes whose workspace exceeds it.
static int attend_checked(const tq_quantizer* kq, const tq_quantizer* vq, const void* queries, int q_dtype, int B,
                          int Hq, int Hkv, const uint32_t* kcodes, const float* knorms, const float* kgammas,
                          const uint32_t* vcodes, const float* vnorms, int64_t n_comp, const uint16_t* k_tail,
                          const uint16_t* v_tail, int n_tail, float scale, float v_threshold, float* out,
                          void* workspace, int64_t ws_bytes, bool noalloc, void* stream) {
  if (!(v_threshold >= 0.f && v_threshold < 1.f)) return fail(TQ_EINVAL, "v_threshold must lie in [0, 1)");
  if (int r = check_quantizer(kq)) return r;
  if (int r = check_quantizer(vq)) return r;
  if (int r = check_heads(B, Hq, Hkv)) return r;
  if (kq->d != vq->d) return fail(TQ_EINVAL, "key and value quantizers differ in d");
  if (int r = check_keys(kq)) return r;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return fail(TQ_EINVAL, "q_dtype must be TQ_F32 or TQ_BF16");
  if (n_comp < 0 || n_tail < 0) return fail(TQ_EINVAL, "negative size");
  if (n_comp + n_tail < 1) return fail(TQ_EINVAL, "empty cache (n_comp + n_tail == 0)");
  if (!queries || !out) return fail(TQ_EINVAL, "NULL queries or output");
  if (!tq::key_qjl(kq)) kgammas = nullptr;   // MSE-only keys carry no gamma
  if (n_comp > 0 && (!kcodes || !knorms || (tq::key_qjl(kq) && !kgammas) || !vcodes || !vnorms))
    return fail(TQ_EINVAL, "NULL cache array");
  if (n_tail > 0 && (!k_tail || !v_tail)) return fail(TQ_EINVAL, "NULL tail array");
  const void* ptrs[] = {queries, out, kcodes, knorms, kgammas, vcodes, vnorms, k_tail, v_tail};
  for (const void* p : ptrs)
    if (p && !aligned(p, 16)) return fail(TQ_EINVAL, "device pointers must be 16-byte aligned");
  if (!tq::attend_supports_d(kq->d))
    return fail(TQ_EUNSUPPORTED, "attend supports d in {64, 96, 128, 256} (d=%d)", kq->d);
  if (v_threshold > 0.f && kq->d != 128) return fail(TQ_EUNSUPPORTED, "sparse V (v_threshold > 0) needs d = 128");
  const int64_t need = tq_attend_workspace_bytes(kq, vq, B, Hq, Hkv, n_comp, n_tail);
  if (need < 0) return TQ_EINVAL;
  if (noalloc) {
    if (need > static_cast<int64_t>(TQ_NOALLOC_SCRATCH_BYTES))
      return fail(TQ_EWORKSPACE, "this shape needs %lld bytes of workspace, more than the %lld-byte scratch of the "
                  "allocation-free call; use tq_attend_decode with a caller workspace",
                  static_cast<long long>(need), static_cast<long long>(TQ_NOALLOC_SCRATCH_BYTES));
  } else {
    if (!workspace || ws_bytes < need)
      return fail(TQ_EWORKSPACE, "workspace of %lld bytes needed", static_cast<long long>(need));
    if (!aligned(workspace, 256)) return fail(TQ_EINVAL, "workspace must be 256-byte aligned");
  }
  if (!(scale > 0.f)) scale = 1.f / std::sqrt(static_cast<float>(kq->d));
  DeviceGuard g(kq->device);
  if (!g.ok) return fail(TQ_EHIP, "cannot select the quantizer's device");
  if (noalloc) {
    workspace = scratch_of(kq->device);
    if (!workspace) {
      if (int r = scratch_setup(kq->device)) return r;
      workspace = scratch_of(kq->device);
    }
  }
  hipError_t e = tq::launch_attend(kq, vq, queries, q_dtype, B, Hq, Hkv, kcodes, knorms, kgammas, vcodes, vnorms, n_comp,
                                   k_tail, v_tail, n_tail, scale, v_threshold, out, workspace,
                                   static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return fail(TQ_EUNSUPPORTED, "shape not supported by the attention kernels");
  return e == hipSuccess ? TQ_OK : hip_fail(e, "attend launch");
}

extern "C" {

int tq_attend_decode_sparse(const tq_quantizer* kq, const tq_quantizer* vq, const void* queries, int q_dtype, int B,
                            int Hq, int Hkv, const uint32_t* kcodes, const float* knorms, const float* kgammas,
                            const uint32_t* vcodes, const float* vnorms, int64_t n_comp, const uint16_t* k_tail,
                            const uint16_t* v_tail, int n_tail, float scale, float v_threshold, float* out,
                            void* workspace, int64_t ws_bytes, void* stream) {
  return attend_checked(kq, vq, queries, q_dtype, B, Hq, Hkv, kcodes, knorms, kgammas, vcodes, vnorms, n_comp, k_tail,
                        v_tail, n_tail, scale, v_threshold, out, workspace, ws_bytes, false, stream);
}

int tq_attend_decode(const tq_quantizer* kq, const tq_quantizer* vq, const void* queries, int q_dtype, int B, int Hq,
                     int Hkv, const uint32_t* kcodes, const float* knorms, const float* kgammas, const uint32_t* vcodes,
                     const float* vnorms, int64_t n_comp, const uint16_t* k_tail, const uint16_t* v_tail, int n_tail,
                     float scale, float* out, void* workspace, int64_t ws_bytes, void* stream) {
  return attend_checked(kq, vq, queries, q_dtype, B, Hq, Hkv, kcodes, knorms, kgammas, vcodes, vnorms, n_comp, k_tail,
                        v_tail, n_tail, scale, 0.f, out, workspace, ws_bytes, false, stream);
}

int64_t tq_attend_segments_workspace_bytes(const tq_segment* segs, int nseg, int B, int Hq, int Hkv, int n_tail) {
  if (!segs || nseg < 1 || nseg > TQ_MAX_SEGMENTS) return fail(TQ_EINVAL, "need 1 <= nseg <= %d segments", TQ_MAX_SEGMENTS);
  if (check_heads(B, Hq, Hkv)) return -1;
  if (n_tail < 0) return fail(TQ_EINVAL, "negative n_tail");
  tq::AttendSegment sg[TQ_MAX_SEGMENTS];
  for (int i = 0; i < nseg; ++i) {
    if (!segs[i].kq || !segs[i].vq) return fail(TQ_EINVAL, "segment %d: NULL quantizer", i);
    if (segs[i].n < 0) return fail(TQ_EINVAL, "segment %d: negative n", i);
    sg[i] = {segs[i].kq, segs[i].vq, nullptr, nullptr, nullptr, nullptr, nullptr, segs[i].n};
  }
  return tq::attend_segments_ws_bytes(sg, nseg, B, Hq, Hkv);
}

int tq_attend_decode_segments(const tq_segment* segs, int nseg, const void* queries, int q_dtype, int B, int Hq,
                              int Hkv, const uint16_t* k_tail, const uint16_t* v_tail, int n_tail, float scale,
                              float* out, void* workspace, int64_t ws_bytes, void* stream) {
  if (!segs || nseg < 1 || nseg > TQ_MAX_SEGMENTS) return fail(TQ_EINVAL, "need 1 <= nseg <= %d segments", TQ_MAX_SEGMENTS);
  if (int r = check_heads(B, Hq, Hkv)) return r;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return fail(TQ_EINVAL, "q_dtype must be TQ_F32 or TQ_BF16");
  if (n_tail < 0) return fail(TQ_EINVAL, "negative n_tail");
  if (!queries || !out) return fail(TQ_EINVAL, "NULL queries or output");
  if (n_tail > 0 && (!k_tail || !v_tail)) return fail(TQ_EINVAL, "NULL tail array");
  const tq_quantizer* v0 = segs[0].vq;
  int64_t total = n_tail;
  tq::AttendSegment sg[TQ_MAX_SEGMENTS];
  for (int i = 0; i < nseg; ++i) {
    const tq_segment& g = segs[i];
    if (!g.kq || !g.vq) return fail(TQ_EINVAL, "segment %d: NULL quantizer", i);
    if (g.n < 0) return fail(TQ_EINVAL, "segment %d: negative n", i);
    if (int r = check_keys(g.kq)) return r;
    if (g.kq->d != v0->d || g.vq->d != v0->d) return fail(TQ_EINVAL, "segment %d: quantizers differ in d", i);
    // the merge rotates the summed values back with one Pi^T
    if (g.vq->seed != v0->seed || g.vq->rotation != v0->rotation)
      return fail(TQ_EINVAL, "segment %d: value quantizers must share seed and rotation (one Pi)", i);
    const float* kg = tq::key_qjl(g.kq) ? g.kgammas : nullptr;   // MSE-only keys carry no gamma
    if (g.n > 0 && (!g.kcodes || !g.knorms || (tq::key_qjl(g.kq) && !kg) || !g.vcodes || !g.vnorms))
      return fail(TQ_EINVAL, "segment %d: NULL cache array", i);
    const void* ptrs[] = {g.kcodes, g.knorms, kg, g.vcodes, g.vnorms};
    for (const void* p : ptrs)
      if (p && !aligned(p, 16)) return fail(TQ_EINVAL, "device pointers must be 16-byte aligned");
    sg[i] = {g.kq, g.vq, g.kcodes, g.knorms, kg, g.vcodes, g.vnorms, g.n};
    total += g.n;
  }
  if (total < 1) return fail(TQ_EINVAL, "empty cache");
  const void* ptrs[] = {queries, out, k_tail, v_tail};
  for (const void* p : ptrs)
    if (p && !aligned(p, 16)) return fail(TQ_EINVAL, "device pointers must be 16-byte aligned");
  if (!tq::attend_supports_d(v0->d))
    return fail(TQ_EUNSUPPORTED, "attend supports d in {64, 96, 128, 256} (d=%d)", v0->d);
  const int64_t need = tq::attend_segments_ws_bytes(sg, nseg, B, Hq, Hkv);
  if (!workspace || ws_bytes < need)
    return fail(TQ_EWORKSPACE, "workspace of %lld bytes needed", static_cast<long long>(need));
  if (!aligned(workspace, 256)) return fail(TQ_EINVAL, "workspace must be 256-byte aligned");
  if (!(scale > 0.f)) scale = 1.f / std::sqrt(static_cast<float>(v0->d));
  DeviceGuard dg(v0->device);
  if (!dg.ok) return fail(TQ_EHIP, "cannot select the quantizer's device");
  hipError_t e = tq::launch_attend_segments(sg, nseg, queries, q_dtype, B, Hq, Hkv, k_tail, v_tail, n_tail, scale, 0.f,
                                            out, workspace, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return fail(TQ_EUNSUPPORTED, "shape not supported by the attention kernels");
  return e == hipSuccess ? TQ_OK : hip_fail(e, "attend launch");
}

int tq_requantize(const tq_quantizer* from, const tq_quantizer* to, int mode, const uint32_t* codes_in,
                  const float* norms_in, const float* gammas_in, int64_t nseq, int64_t n, uint32_t* codes_out,
                  float* norms_out, float* gammas_out, void* workspace, int64_t ws_bytes, void* stream) {
  if (int r = check_quantizer(from)) return r;
  if (int r = check_quantizer(to)) return r;
  if (int r = check_mode(from, mode)) return r;
  if (int r = check_mode(to, mode)) return r;
  if (from->d != to->d) return fail(TQ_EINVAL, "quantizers differ in d");
  if (nseq < 0 || n < 0) return fail(TQ_EINVAL, "negative size");
  if (nseq * n == 0) return TQ_OK;
  if (!codes_in || !norms_in || !codes_out || !norms_out || (mode == TQ_PROD && (!gammas_in || !gammas_out)))
    return fail(TQ_EINVAL, "NULL array argument");
  const void* ptrs[] = {codes_in, norms_in, gammas_in, codes_out, norms_out, gammas_out, workspace};
  for (const void* p : ptrs)
    if (p && !aligned(p, 16)) return fail(TQ_EINVAL, "device pointers must be 16-byte aligned");
  if (to->d > 256) return fail(TQ_EUNSUPPORTED, "encode supports d <= 256 (d=%d)", to->d);
  if (nseq > 65535) return fail(TQ_EUNSUPPORTED, "nseq > 65535");
  const int64_t need = nseq * n * from->d * static_cast<int64_t>(sizeof(float));
  if (!workspace || ws_bytes < need)
    return fail(TQ_EWORKSPACE, "workspace of %lld bytes needed", static_cast<long long>(need));
  DeviceGuard g(to->device);
  if (!g.ok) return fail(TQ_EHIP, "cannot select the quantizer's device");
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* x = static_cast<float*>(workspace);
  hipError_t e = tq::launch_decode(from, mode, codes_in, norms_in, gammas_in, nseq, n, x, st);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  e = tq::launch_encode(to, mode, x, TQ_F32, nseq, n, codes_out, norms_out, gammas_out, st);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "encode launch");
}

int tq_attend_decode_noalloc(const tq_quantizer* kq, const tq_quantizer* vq, const void* queries, int q_dtype, int B,
                             int Hq, int Hkv, const uint32_t* kcodes, const float* knorms, const float* kgammas,
                             const uint32_t* vcodes, const float* vnorms, int64_t n_comp, const uint16_t* k_tail,
                             const uint16_t* v_tail, int n_tail, float scale, float* out, void* stream) {
  return attend_checked(kq, vq, queries, q_dtype, B, Hq, Hkv, kcodes, knorms, kgammas, vcodes, vnorms, n_comp, k_tail,
                        v_tail, n_tail, scale, 0.f, out, nullptr, 0, true, stream);
}

}  // extern "C"
