// Internal declarations shared by the libtq sources (not part of the ABI).
#pragma once

#include <cstdint>
#include <vector>

namespace tq {

// host precompute (tq_host.cpp)
void normals(uint64_t seed, int tag, int64_t n, double* out);
void rotation(int d, uint64_t seed, double* pi);
void signs(uint64_t seed, int d, double* out);
void rotation_hadamard(int d, uint64_t seed, double* pi);
void qjl_matrix(int m, int d, uint64_t seed, double* s);
int codebook(int d, int K, double* centroids, double* thresholds);

constexpr int kMaxLevels = 16;
constexpr int kMaxEncodeD = 1024;   // largest d of encode and logits (the host quantizer's bound)
constexpr int kMaxTerms = 8;

// One codebook as the kernels see it (passed by value as a kernel argument).
// The centroid of an index is also written in the +-1 (Walsh) basis of its
// bits: with s_p = 2*bit_p - 1, c[idx] = sum_t coef[t] * prod_{p in mask[t]} s_p,
// and prod_{p in mask} s_p = 2*XOR_{p in mask} bit_p - 1 for odd |mask|.  A
// symmetric codebook has only odd-size masks, 2^(bp-1) of them.
struct Codebook {
  int bp = 0;      // index bits (0 = codebook unavailable)
  int levels = 0;  // 2^bp
  int nterms = 0;  // 2^(bp-1)
  float c[kMaxLevels] = {};
  float t[kMaxLevels] = {};   // thresholds, levels-1 used
  int mask[kMaxTerms] = {};
  float coef[kMaxTerms] = {};
  float coef_sum = 0.f;       // sum of coef (the centroid of "all bits 0" is -coef_sum)
};

}  // namespace tq

struct tq_quantizer {
  int d = 0, bits = 0, m = 0, device = 0, rotation = 0;   // rotation: TQ_ROT_HAAR (0) or TQ_ROT_HADAMARD (1)
  uint64_t seed = 0;
  std::vector<double> pi, s;          // host float64 copies (row major)
  tq::Codebook cb[2];                 // [TQ_PROD] b-1 bits, [TQ_MSE] b bits (values and MSE-only keys)
  float* d_pi = nullptr;              // [d][d]   y = Pi x
  float* d_s = nullptr;               // [m][d]   QJL matrix
  float* d_sp = nullptr;              // [m][d]   S' = S Pi^T (acts on rotated residuals)
  float* d_qt = nullptr;              // [d][d+m] column k of Pi then of S (query transform, k-major)
  float* d_spt = nullptr;             // [d][m]   S' k-major (d_spt[k * m + r] = S'[r][k]), general-d encoder
  uint16_t* d_wide = nullptr;         // 128 < d <= 256: fp16 [4][256][256] = Pi hi, Pi lo, S' hi, S' lo (x 2^8,
                                      // zero past d), the eight-wave encoder's operands
  int key_mode = 0;                   // key layout the scoring calls read: TQ_PROD (0) or TQ_MSE_KEYS (2)
};

namespace tq {
// codebook and term count of the keys the scoring calls read
inline bool key_qjl(const tq_quantizer* q) { return q->key_mode != 2; }
inline const Codebook& key_codebook(const tq_quantizer* q) { return q->cb[key_qjl(q) ? 0 : 1]; }
inline int key_terms(const tq_quantizer* q) { return key_codebook(q).nterms + (key_qjl(q) ? 1 : 0); }
}  // namespace tq
