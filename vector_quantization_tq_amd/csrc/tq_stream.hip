// Streaming ceiling for the logits scan: a kernel that moves exactly the
// scan's bytes with no arithmetic in between, so that its time is what plain
// streaming of that traffic costs on this part.
//
// The layout and launch follow the scan of prod keys at d = 128, 3 bits: a
// key is 48 bytes of packed words plus a norm and a gamma (4 bytes each), and
// four query heads share it, so the scan writes 16 bytes of logits per key.
// Waves take batches of 64 consecutive keys of one sequence (about 4096 waves
// over all sequences, batches dealt round-robin as in the scan).  Per batch a
// lane loads 3 x 16 bytes of words (non-temporal, as the scan's staging copies)
// and its key's norm and gamma, folds them into 4 floats and stores one
// 16-byte run of the output: 3584 bytes read and 1024 written per batch, the
// scan's mix.  The fold keeps every load live; the output values mean nothing.
//
// Built into its own library (libtq_stream.so), used only by the benchmark.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kBatch = 64;
constexpr int kWordsPerKey = 12;   // 48 bytes
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) stream_scan_mix(const u4* __restrict__ codes, const float* __restrict__ norms,
                                                       const float* __restrict__ gammas, int64_t n, int64_t nseq,
                                                       f4* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t grp = blockIdx.y;
  const int64_t nbatch = n / kBatch;   // n a multiple of 64 (checked by the host)
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 4;
  const u4* cb = codes + grp * n * (kWordsPerKey / 4);
  const float* nb = norms + grp * n;
  const float* gb = gammas + grp * n;
  f4* ob = out + grp * n;          // 4 floats per key
  for (int64_t bt = static_cast<int64_t>(blockIdx.x) * 4 + wave; bt < nbatch; bt += stride) {
    const int64_t k0 = bt * kBatch;
    const u4* src = cb + k0 * (kWordsPerKey / 4);
    const u4 a = __builtin_nontemporal_load(src + lane);
    const u4 b = __builtin_nontemporal_load(src + 64 + lane);
    const u4 c = __builtin_nontemporal_load(src + 128 + lane);
    const float nv = __builtin_nontemporal_load(nb + k0 + lane);
    const float gv = __builtin_nontemporal_load(gb + k0 + lane);
    const uint32_t x = a.x ^ b.y ^ c.z, y = a.y ^ b.z ^ c.w, z = a.z ^ b.w ^ c.x, w = a.w ^ b.x ^ c.y;
    const f4 o = {__uint_as_float(x) + nv, __uint_as_float(y) + gv, __uint_as_float(z) * nv, __uint_as_float(w) * gv};
    ob[k0 + lane] = o;
  }
}

}  // namespace

extern "C" {

// codes: nseq * n * 12 uint32 words, norms/gammas: nseq * n floats, out:
// nseq * n * 4 floats; n a multiple of 64.  Returns 0 or a hipError_t.
int tq_stream_scan_mix(const void* codes, const float* norms, const float* gammas, int64_t n, int64_t nseq, float* out,
                       void* stream) {
  if (n <= 0 || n % kBatch || nseq <= 0 || nseq > 65535 || !codes || !norms || !gammas || !out)
    return static_cast<int>(hipErrorInvalidValue);
  const int64_t nbatch = n / kBatch;
  int64_t bx = (1024 + nseq - 1) / nseq;           // about 4096 waves in all, as the scan
  const int64_t need = (nbatch + 3) / 4;
  if (bx > need) bx = need;
  if (bx < 1) bx = 1;
  hipLaunchKernelGGL(stream_scan_mix, dim3(static_cast<unsigned>(bx), static_cast<unsigned>(nseq)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u4*>(codes), norms, gammas, n, nseq,
                     reinterpret_cast<f4*>(out));
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
