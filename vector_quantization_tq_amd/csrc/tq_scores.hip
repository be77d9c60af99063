// Attention logits straight from the packed key codes.
//
// The query is rotated and projected once (a2a-mcp.org "什麼是TurboQuant？",
// how-to-implement section: fused kernel that pre-rotates the query and
// reads indices directly), then for every key
//   logit = n <Pi q, c[idx]> + gamma sqrt(pi/2)/m <S q, sigma>
// (blog.hotdry.top "TurboQuant vector-search compression", QJL section: the
// unbiased inner-product estimate).
//
// Both inner products are written over bit planes.  With s_p = 2 bit_p - 1,
// c[idx] = sum_t coef_t * (2 XOR_{p in mask_t} bit_p - 1), so
//   <q^, c[idx]> = sum_t <2 coef_t q^, b_t> - coef_sum * sum(q^),
//   <s, sigma>   = <2 s, b_qjl> - sum(s),
// where every b is a 0/1 vector read straight out of the packed words.  The
// <value, 0/1 bits> products run on the 16x16x128 f8f6f4 MFMA: the key bits
// are the fp4 B operand (a mask per nibble, no table lookup), the query side
// is the fp8 A operand split into 4 limbs (rows), each limb carrying the
// next 4 bits of the value, so the sum over limbs is float-accurate.
// A 16-row tile holds 4 queries x 4 limbs; one MFMA covers 16 keys and 128
// coordinates.  The kernel is bound by HBM reads of the packed codes.
#include "tq_device.h"
#include "tq_kernels.h"

namespace tq {

namespace {

template <int BP>
__device__ __forceinline__ uint32_t walsh_word(const uint32_t (&w)[5], int t) {
  // Walsh masks of the odd subsets of the index bits, in the order the host
  // computes the coefficients
  constexpr int masks[4][8] = {{1}, {1, 2}, {1, 2, 4, 7}, {1, 2, 4, 8, 7, 11, 13, 14}};
  const int mk = masks[BP - 1][t];
  uint32_t r = 0u;
#pragma unroll
  for (int p = 0; p < BP; ++p)
    if (mk & (1 << p)) r ^= w[p];
  return r;
}

}  // namespace

// ---------------------------------------------------------------------------
// Query prep: one workgroup per query slot (group, row tile, query-in-tile).
// Writes the fp8 A operands [group*RT + rt][term][chunk][lane][32 bytes] and
// per-query constants [group*RT + rt][qi][16 floats]:
//   {cM, cQ, sM0..3, sQ0..3}: logit = n (sum_k sM_k C_M,k + cM) + gamma (sum_k sQ_k C_Q,k + cQ)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) query_prep_kernel(const void* __restrict__ queries, int q_dtype, int Hq, int Hkv,
                                                         int G, int RT, int d, int m, const float* __restrict__ pi,
                                                         const float* __restrict__ s, Codebook cb, int C,
                                                         uint8_t* __restrict__ wsA, float* __restrict__ wsC) {
  extern __shared__ float sm[];
  float* qv = sm;           // [d]
  float* qh = qv + d;       // [d]   Pi q
  float* sq = qh + d;       // [m]   S q
  const int tid = threadIdx.x;
  const int slot = blockIdx.x;
  const int gy = slot >> 2, qi = slot & 3;
  const int grp = gy / RT, rt = gy - grp * RT;
  const int b = grp / Hkv, kvh = grp - b * Hkv;
  const int qg = rt * 4 + qi;                 // query index inside the KV group
  const bool valid = qg < G;
  const int T = cb.nterms + 1;

  if (valid) {
    const int64_t qoff = (static_cast<int64_t>(b) * Hq + kvh * G + qg) * d;
    for (int j = tid; j < d; j += blockDim.x) qv[j] = load_elem(queries, q_dtype, qoff + j);
  }
  __syncthreads();
  float lmax_h = 0.f, lmax_s = 0.f, lsum_h = 0.f, lsum_s = 0.f;
  if (valid) {
    for (int j = tid; j < d; j += blockDim.x) {
      float a = 0.f;
      for (int k = 0; k < d; ++k) a = fmaf(pi[static_cast<int64_t>(j) * d + k], qv[k], a);
      qh[j] = a;
      lmax_h = fmaxf(lmax_h, fabsf(a));
      lsum_h += a;
    }
    for (int r = tid; r < m; r += blockDim.x) {
      float a = 0.f;
      for (int k = 0; k < d; ++k) a = fmaf(s[static_cast<int64_t>(r) * d + k], qv[k], a);
      sq[r] = a;
      lmax_s = fmaxf(lmax_s, fabsf(a));
      lsum_s += a;
    }
  }
  // block reductions (max and sum of both vectors)
  for (int off = 32; off > 0; off >>= 1) {
    lmax_h = fmaxf(lmax_h, __shfl_xor(lmax_h, off));
    lmax_s = fmaxf(lmax_s, __shfl_xor(lmax_s, off));
    lsum_h += __shfl_xor(lsum_h, off);
    lsum_s += __shfl_xor(lsum_s, off);
  }
  __shared__ float wred[4][4];
  if ((tid & 63) == 0) {
    wred[tid >> 6][0] = lmax_h;
    wred[tid >> 6][1] = lmax_s;
    wred[tid >> 6][2] = lsum_h;
    wred[tid >> 6][3] = lsum_s;
  }
  __syncthreads();
  float max_h = 0.f, max_s = 0.f, sum_h = 0.f, sum_s = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    max_h = fmaxf(max_h, wred[w][0]);
    max_s = fmaxf(max_s, wred[w][1]);
    sum_h += wred[w][2];
    sum_s += wred[w][3];
  }
  const float alpha2 = 2.f * 1.2533141373155003f / static_cast<float>(m);   // 2 sqrt(pi/2)/m
  float amax = 0.f;
  for (int t = 0; t < cb.nterms; ++t) amax = fmaxf(amax, fabsf(cb.coef[t]));
  // values are divided by the fp4 slot value (>= 0.5): bound by 2 * max
  const float vmax_m = 2.f * 2.f * amax * max_h;
  const float vmax_q = 2.f * alpha2 * max_s;
  const int E_m = vmax_m > 0.f ? 7 - ilogbf(vmax_m) : 0;
  const int E_q = vmax_q > 0.f ? 7 - ilogbf(vmax_q) : 0;

  // A operand bytes of this query: rows 4*qi .. 4*qi+3 (limbs), lane-groups 0..3
  const int64_t tile_bytes = 64 * 32;
  uint8_t* base = wsA + static_cast<int64_t>(gy) * T * C * tile_bytes;
  for (int t = 0; t < T; ++t) {
    const bool is_q = t == T - 1;
    const float coef = is_q ? alpha2 : 2.f * cb.coef[t];
    const int E = is_q ? E_q : E_m;
    for (int c = 0; c < C; ++c) {
      for (int e2 = tid; e2 < 16 * 32; e2 += blockDim.x) {
        const int li = e2 >> 5, e = e2 & 31;        // li: 4 limbs x 4 lane-groups
        const int limb = li & 3, g = li >> 2;
        const int lane = 4 * qi + limb + 16 * g;
        uint32_t byte = 0u;
        if (valid) {
          const int k = a_elem_to_k(g, e);
          const int coord = c * 128 + 32 * (k >> 5) + k_to_bit(k);
          const int lim = is_q ? m : d;
          if (coord < lim) {
            const float v = coef * (is_q ? sq[coord] : qh[coord]) / fp4_slot_value((k & 31) >> 3);
            byte = e4m3_limb(ldexpf(v, E), limb);
          }
        }
        base[(static_cast<int64_t>(t) * C + c) * tile_bytes + lane * 32 + e] = static_cast<uint8_t>(byte);
      }
    }
  }
  if (tid < 16) {
    float val = 0.f;
    if (valid) {
      if (tid == 0) val = -cb.coef_sum * sum_h;
      else if (tid == 1) val = -0.5f * alpha2 * sum_s;
      else if (tid < 6) val = ldexpf(1.f, -E_m - 4 * (tid - 2));
      else if (tid < 10) val = ldexpf(1.f, -E_q - 4 * (tid - 6));
    }
    wsC[(static_cast<int64_t>(gy) * 4 + qi) * 16 + tid] = val;
  }
}

// ---------------------------------------------------------------------------
// Scores: grid (key blocks, groups * row tiles); 4 waves, each wave handles
// kTilesPerWave tiles of 16 keys.  Lane l: key (l & 15) of the tile, word
// group (l >> 4) of each 128-coordinate chunk.
// ---------------------------------------------------------------------------
constexpr int kTilesPerWave = 8;
constexpr int kKeysPerBlock = 4 * kTilesPerWave * 16;

template <int BP, int C>
__global__ void __launch_bounds__(256) scores_kernel(const uint32_t* __restrict__ codes, const float* __restrict__ norms,
                                                     const float* __restrict__ gammas, int64_t n, int d, int Hq,
                                                     int Hkv, int G, int RT, const uint8_t* __restrict__ wsA,
                                                     const float* __restrict__ wsC, float* __restrict__ out) {
  constexpr int T = (1 << (BP - 1)) + 1;
  constexpr int W = BP + 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gy = blockIdx.y;
  const int grp = gy / RT, rt = gy - grp * RT;
  const int b = grp / Hkv, kvh = grp - b * Hkv;
  const int qi = lane >> 4;
  const int Gw = (d + 31) >> 5;

  v8i A[T][C];
  const v8i* ap = reinterpret_cast<const v8i*>(wsA + static_cast<int64_t>(gy) * T * C * 2048);
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < C; ++c) A[t][c] = ap[(t * C + c) * 64 + lane];
  const float* cs = wsC + (static_cast<int64_t>(gy) * 4 + qi) * 16;
  const float cM = cs[0], cQ = cs[1];
  const float sM0 = cs[2], sM1 = cs[3], sM2 = cs[4], sM3 = cs[5];
  const float sQ0 = cs[6], sQ1 = cs[7], sQ2 = cs[8], sQ3 = cs[9];
  const int qg = rt * 4 + qi;
  float* orow = (qg < G) ? out + (static_cast<int64_t>(b) * Hq + kvh * G + qg) * n : nullptr;

  const uint32_t* cbase = codes + static_cast<int64_t>(grp) * n * Gw * W;
  const float* nb = norms + static_cast<int64_t>(grp) * n;
  const float* gb = gammas + static_cast<int64_t>(grp) * n;
  const int64_t kstart = static_cast<int64_t>(blockIdx.x) * kKeysPerBlock + wave * (kTilesPerWave * 16);

  for (int tile = 0; tile < kTilesPerWave; ++tile) {
    const int64_t k0 = kstart + tile * 16;
    if (k0 >= n) break;
    const int64_t key = k0 + (lane & 15);
    const bool kv = key < n;
    v4f accM = {0.f, 0.f, 0.f, 0.f}, accQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int gg = 4 * c + (lane >> 4);
      uint32_t w[5] = {0u, 0u, 0u, 0u, 0u};
      if (kv && gg < Gw) {
        const uint32_t* wp = cbase + (key * Gw + gg) * W;
#pragma unroll
        for (int p = 0; p < W; ++p) w[p] = wp[p];
      }
#pragma unroll
      for (int t = 0; t < T - 1; ++t) {
        accM = mfma_fp8_fp4(A[t][c], bits_to_fp4(walsh_word<BP>(w, t)), accM);
      }
      accQ = mfma_fp8_fp4(A[T - 1][c], bits_to_fp4(w[BP]), accQ);
    }
    pin(accM);
    pin(accQ);
    const float mse = fmaf(accM[0], sM0, fmaf(accM[1], sM1, fmaf(accM[2], sM2, fmaf(accM[3], sM3, cM))));
    const float qjl = fmaf(accQ[0], sQ0, fmaf(accQ[1], sQ1, fmaf(accQ[2], sQ2, fmaf(accQ[3], sQ3, cQ))));
    if (kv && orow) orow[key] = fmaf(nb[key], mse, gb[key] * qjl);
  }
}

int64_t scores_ws_bytes(const tq_quantizer* q, int B, int Hq, int Hkv) {
  const int G = Hq / Hkv;
  const int RT = (G + 3) / 4;
  const int T = q->cb[0].nterms + 1;
  const int C = (q->d + 127) / 128;
  const int64_t groups = static_cast<int64_t>(B) * Hkv * RT;
  return groups * T * C * 2048 + groups * 4 * 16 * 4;
}

hipError_t launch_query_prep(const tq_quantizer* q, const void* queries, int q_dtype, int B, int Hq, int Hkv,
                             uint8_t* wsA, float* wsC, hipStream_t st) {
  const int G = Hq / Hkv;
  const int RT = (G + 3) / 4;
  const int C = (q->d + 127) / 128;
  const size_t lds = sizeof(float) * (2 * q->d + q->m);
  dim3 grid(static_cast<unsigned>(static_cast<int64_t>(B) * Hkv * RT * 4));
  hipLaunchKernelGGL(query_prep_kernel, grid, dim3(256), lds, st, queries, q_dtype, Hq, Hkv, G, RT, q->d, q->m, q->d_pi,
                     q->d_s, q->cb[0], C, wsA, wsC);
  return hipGetLastError();
}

hipError_t launch_scores(const tq_quantizer* q, const void* queries, int q_dtype, int B, int Hq, int Hkv,
                         const uint32_t* codes, const float* norms, const float* gammas, int64_t n, float* out,
                         void* ws, hipStream_t st) {
  const int G = Hq / Hkv;
  const int RT = (G + 3) / 4;
  const int T = q->cb[0].nterms + 1;
  const int C = (q->d + 127) / 128;
  const int64_t groups = static_cast<int64_t>(B) * Hkv * RT;
  uint8_t* wsA = static_cast<uint8_t*>(ws);
  float* wsC = reinterpret_cast<float*>(wsA + groups * T * C * 2048);
  hipError_t e = launch_query_prep(q, queries, q_dtype, B, Hq, Hkv, wsA, wsC, st);
  if (e != hipSuccess) return e;
  dim3 grid(static_cast<unsigned>((n + kKeysPerBlock - 1) / kKeysPerBlock), static_cast<unsigned>(groups));
  const int bp = q->cb[0].bp;
#define TQ_SC(BPV, CV)                                                                                           \
  if (bp == BPV && C == CV) {                                                                                    \
    hipLaunchKernelGGL((scores_kernel<BPV, CV>), grid, dim3(256), 0, st, codes, norms, gammas, n, q->d, Hq, Hkv, G, \
                       RT, wsA, wsC, out);                                                                       \
    return hipGetLastError();                                                                                    \
  }
  TQ_SC(1, 1) TQ_SC(2, 1) TQ_SC(3, 1) TQ_SC(1, 2) TQ_SC(2, 2) TQ_SC(3, 2)
#undef TQ_SC
  return hipErrorInvalidValue;
}

}  // namespace tq
