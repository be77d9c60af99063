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
// are the fp4 B operand (a mask per nibble, no table lookup; the fourth of
// every 4 coordinates is read as 1 - 2 bit, its A element negated and halved,
// so that its half of the -1 rides in the MFMA and the constants above sum
// the other coordinates only), the query side
// is the fp8 A operand split into 4 limbs (rows), each limb carrying the
// next 4 bits of the value with its own exponent, so the sum over limbs is
// float-accurate per coordinate.  (The matrix core adds the products of a
// row in groups of 8 aligned to the largest, keeping about 12 bits; after
// the rotation the coordinates of one query are of similar size, so this
// costs nothing measurable here -- unlike the softmax weights of the
// attention kernel, which span many decades and use fixed-point limbs.)
// A 16-row tile holds 4 queries x 4 limbs; one MFMA covers 16 keys and 128
// coordinates.  The kernel is bound by HBM reads of the packed codes.
#include "tq_device.h"
#include "tq_kernels.h"

namespace tq {

// ---------------------------------------------------------------------------
// Query prep: one workgroup per query slot (group, row tile, query-in-tile).
// Writes the fp8 A operands [group*RT + rt][term][chunk][lane][32 bytes] and
// per-query constants [group*RT + rt][qi][16 floats]:
//   {cM, cQ, sM0..3, sQ0..3}: logit = n (sum_k sM_k C_M,k + cM) + gamma (sum_k sQ_k C_Q,k + cQ)
// The terms are the Walsh terms of the key codebook, then (prod keys) the
// QJL term; MSE-only keys have no QJL term.
// ---------------------------------------------------------------------------
// BOUND (the bounded top-k scan): also writes, in constants 10 and 11, bounds
// of what limbs 2 and 3 add to the MSE and QJL sums of any key, so that a
// scan over limbs 0 and 1 alone brackets the full score
// (n (sum_k<2 sM_k C_M,k + cM +- E_M) + gamma (... +- E_Q)).
template <bool QBF16, bool ONE, bool BOUND = false>
__device__ __forceinline__ void query_prep_body(const void* __restrict__ queries, int q_dtype, int Hq, int Hkv, int G,
                                                int RT, int d, int m, const float* __restrict__ qt, const Codebook& cb,
                                                int qjl, int C, uint8_t* __restrict__ wsA, float* __restrict__ wsC) {
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
  const int T = cb.nterms + (qjl ? 1 : 0);   // Walsh terms (+ the QJL term)

  // [Pi q, S q] from the k-major table: wave w takes the contraction slice
  // k in [w KQ, (w+1) KQ), lane the 4 consecutive outputs 4 lane + 256 r;
  // the loads of a slice are independent 16-byte reads (indices clamped, no
  // branches), partial sums meet in LDS
  float lmax_h = 0.f, lmax_s = 0.f, lsum_h = 0.f, lsum_s = 0.f;
  const int dm = d + m;
  float* pw = sq + m;   // [4][dm] partial sums
  const int wave = tid >> 6, lane = tid & 63;
  const int KQ = (d + 3) / 4;
  const int k0 = min(d, wave * KQ), k1 = min(d, k0 + KQ);
  // ONE (d <= 128, d + m <= 256 and a multiple of 4, checked by the host):
  // a wave's whole slice is one batch of 32 loads per lane, issued right
  // after the query element so that both are in flight together.  The query
  // load has no branch (row and index clamped) and its value is stored
  // unconditionally, so it stays ahead of the table loads and the wait for it
  // leaves them outstanding (vector loads retire in issue order).
  float qe;
  {
    const int64_t qi0 = (static_cast<int64_t>(b) * Hq + kvh * G + (valid ? qg : 0)) * d + min(tid, d - 1);
    if constexpr (QBF16) qe = bf16_to_f32(static_cast<const uint16_t*>(queries)[qi0]);
    else qe = static_cast<const float*>(queries)[qi0];
  }
  __builtin_amdgcn_sched_barrier(0);
  float4 v1[32];
  if constexpr (ONE) {
    const int oc = min(4 * lane, dm - 4);
#pragma unroll
    for (int u = 0; u < 32; ++u)
      v1[u] = *reinterpret_cast<const float4*>(qt + static_cast<int64_t>(min(k0 + u, k1 - 1)) * dm + oc);
  }
  __shared__ float qstage[256];   // element tid of the query (clamped duplicates past d)
  qstage[tid] = qe;
  if constexpr (!ONE) {
    if (valid) {
      if (tid < d) qv[tid] = qe;
      for (int j = tid + blockDim.x; j < d; j += blockDim.x)
        qv[j] = load_elem(queries, q_dtype, (static_cast<int64_t>(b) * Hq + kvh * G + qg) * d + j);
    }
  }
  __syncthreads();
  if constexpr (ONE) {
    const int o = 4 * lane;
    float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const float qk = (valid && k0 + u < k1) ? qstage[min(k0 + u, k1 - 1)] : 0.f;
      a[0] = fmaf(v1[u].x, qk, a[0]);
      a[1] = fmaf(v1[u].y, qk, a[1]);
      a[2] = fmaf(v1[u].z, qk, a[2]);
      a[3] = fmaf(v1[u].w, qk, a[3]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (o + e < dm) pw[wave * dm + o + e] = a[e];
  } else {
    for (int ob = 0; ob < dm; ob += 256) {
      const int o = ob + 4 * lane;
      float a[4] = {0.f, 0.f, 0.f, 0.f};
      if (valid && (dm & 3) == 0) {
        const int oc = min(o, dm - 4);
        for (int kk = k0; kk < k1; kk += 16) {
          // 16 loads in flight before the first use
          float4 v[16];
#pragma unroll
          for (int u = 0; u < 16; ++u)
            v[u] = *reinterpret_cast<const float4*>(qt + static_cast<int64_t>(min(kk + u, k1 - 1)) * dm + oc);
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const float qk = kk + u < k1 ? qv[min(kk + u, k1 - 1)] : 0.f;
            a[0] = fmaf(v[u].x, qk, a[0]);
            a[1] = fmaf(v[u].y, qk, a[1]);
            a[2] = fmaf(v[u].z, qk, a[2]);
            a[3] = fmaf(v[u].w, qk, a[3]);
          }
        }
      } else if (valid) {
#pragma unroll 4
        for (int kk = k0; kk < k1; ++kk) {
          const float qk = qv[kk];
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e] = fmaf(qt[static_cast<int64_t>(kk) * dm + min(o + e, dm - 1)], qk, a[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (o + e < dm) pw[wave * dm + o + e] = a[e];
    }
  }
  __syncthreads();
  if (valid) {
    for (int o = tid; o < dm; o += blockDim.x) {
      const float a = (pw[o] + pw[dm + o]) + (pw[2 * dm + o] + pw[3 * dm + o]);
      // the constant terms sum the coordinates outside slot 3 (the MFMA's
      // 1 - 2 bit slot carries its own half)
      if (o < d) {
        qh[o] = a;
        lmax_h = fmaxf(lmax_h, fabsf(a));
        if (!key_slot3_coord(o)) lsum_h += a;
      } else {
        sq[o - d] = a;
        lmax_s = fmaxf(lmax_s, fabsf(a));
        if (!key_slot3_coord(o - d)) lsum_s += a;
      }
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

  // A operand bytes of this query: rows 4*qi .. 4*qi+3 (limbs), lane-groups
  // 0..3.  One thread per (term, chunk, lane-group, element) writes the 4 limbs
  // of its value: limb k carries the next 4 significant bits, each rounded to
  // fp8 E4M3 by the hardware conversion (round to nearest even), so every
  // residual is exact in float.
  const int64_t tile_bytes = 64 * 32;
  uint8_t* base = wsA + static_cast<int64_t>(gy) * T * C * tile_bytes;
  // BOUND: per thread, sum over its elements of |limb value| x the largest
  // |B| of the element's slot (0.5, 1, 2, 1), limbs 2-3 and all limbs, in
  // the scaled units of limb 0 (each limb 16x finer than the one before)
  float lo_m = 0.f, lo_q = 0.f, all_m = 0.f, all_q = 0.f;
  for (int idx = tid; idx < T * C * 128; idx += blockDim.x) {
    const int t = idx / (C * 128), c = (idx >> 7) - t * C, ge = idx & 127;
    const int g = ge >> 5, e = ge & 31;
    const bool is_q = qjl && t == T - 1;
    const int k = a_elem_to_k(g, e);
    const int coord = c * 128 + 32 * (k >> 5) + k_to_bit(k);
    float x = 0.f;
    if (valid && coord < (is_q ? m : d)) {
      const float coef = is_q ? alpha2 : 2.f * cb.coef[t];
      const float v = coef * (is_q ? sq[coord] : qh[coord]) / key_slot_value((k & 31) >> 3);
      x = ldexpf(v, is_q ? E_q : E_m);
    }
    uint8_t* dst = base + (static_cast<int64_t>(t) * C + c) * tile_bytes + (4 * qi + 16 * g) * 32 + e;
    float lo = 0.f, all = 0.f;
#pragma unroll
    for (int limb = 0; limb < 4; ++limb) {
      const uint32_t byte = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false)) & 0xFFu;
      dst[limb * 32] = static_cast<uint8_t>(byte);
      const float lv = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(byte), 0);
      x = (x - lv) * 16.f;
      if constexpr (BOUND) {
        const float a = fabsf(lv) * ldexpf(1.f, -4 * limb);
        all += a;
        if (limb >= 2) lo += a;
      }
    }
    if constexpr (BOUND) {
      const int sl = (k & 31) >> 3;
      const float bm = sl == 0 ? 0.5f : (sl == 2 ? 2.f : 1.f);
      if (is_q) {
        lo_q = fmaf(lo, bm, lo_q);
        all_q = fmaf(all, bm, all_q);
      } else {
        lo_m = fmaf(lo, bm, lo_m);
        all_m = fmaf(all, bm, all_m);
      }
    }
  }
  float e_m = 0.f, e_q = 0.f;
  if constexpr (BOUND) {
    for (int off = 32; off > 0; off >>= 1) {
      lo_m += __shfl_xor(lo_m, off);
      lo_q += __shfl_xor(lo_q, off);
      all_m += __shfl_xor(all_m, off);
      all_q += __shfl_xor(all_q, off);
    }
    __shared__ float bred[4][4];
    if ((tid & 63) == 0) {
      bred[tid >> 6][0] = lo_m;
      bred[tid >> 6][1] = lo_q;
      bred[tid >> 6][2] = all_m;
      bred[tid >> 6][3] = all_q;
    }
    __syncthreads();
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w)
      for (int j = 0; j < 4; ++j) s4[j] += bred[w][j];
    // In real units (limb 0's scale 2^-E): the limbs 2-3 part of an MSE (QJL)
    // sum is at most lo (the matrix core's own rounding only shrinks the
    // products it truncates; 1% covers its aligned adds), and the float
    // evaluation of either bracket differs from the full chain's by a few
    // roundings of magnitudes below |constant| + all.
    const float cm = valid ? fabsf(cb.coef_sum * sum_h) : 0.f;
    const float cq = valid && qjl ? fabsf(0.5f * alpha2 * sum_s) : 0.f;
    e_m = 1.01f * ldexpf(s4[0], -E_m) + 0x1p-17f * (cm + ldexpf(s4[2], -E_m));
    e_q = 1.01f * ldexpf(s4[1], -E_q) + 0x1p-17f * (cq + ldexpf(s4[3], -E_q));
  }
  if (tid < 16) {
    float val = 0.f;
    if (valid) {
      if (tid == 0) val = -cb.coef_sum * sum_h;
      else if (tid == 1) val = qjl ? -0.5f * alpha2 * sum_s : 0.f;
      else if (tid < 6) val = ldexpf(1.f, -E_m - 4 * (tid - 2));
      else if (tid < 10) val = ldexpf(1.f, -E_q - 4 * (tid - 6));
      else if (tid == 10) val = e_m;
      else if (tid == 11) val = e_q;
    }
    wsC[(static_cast<int64_t>(gy) * 4 + qi) * 16 + tid] = val;
  }
}

template <bool QBF16, bool ONE, bool BOUND>
__global__ void __launch_bounds__(256) query_prep_kernel(const void* __restrict__ queries, int q_dtype, int Hq, int Hkv,
                                                         int G, int RT, int d, int m, const float* __restrict__ qt,
                                                         Codebook cb, int qjl, int C, uint8_t* __restrict__ wsA,
                                                         float* __restrict__ wsC) {
  query_prep_body<QBF16, ONE, BOUND>(queries, q_dtype, Hq, Hkv, G, RT, d, m, qt, cb, qjl, C, wsA, wsC);
}

// The query operands of several quantizers (the segments of one cache) in
// one launch: blockIdx.y picks the quantizer.
template <bool QBF16, bool ONE>
__global__ void __launch_bounds__(256) query_prep_multi_kernel(const void* __restrict__ queries, int q_dtype, int Hq,
                                                               int Hkv, int G, int RT, int d, int m, int C,
                                                               PrepSet set) {
  const int k = blockIdx.y;
  query_prep_body<QBF16, ONE>(queries, q_dtype, Hq, Hkv, G, RT, d, m, set.qt[k], set.cb[k], set.qjl[k], C, set.wsA[k],
                              set.wsC[k]);
}

// ---------------------------------------------------------------------------
// Scores: grid (blocks per group, groups * row tiles), 4 independent waves
// per block.  A wave takes batches of 64 consecutive keys (4 MFMA tiles of
// 16): batch k of the group goes to wave (k mod waves-per-group).  The packed
// words of a batch are one contiguous run; they travel from HBM straight into
// a ring of kRing LDS slots owned by the wave (global_load_lds, no registers
// held while in flight), together with the batch's norms and gammas.  The
// wave consumes slot i while the next kRing-1 batches are in flight, reading
// the words back in the MFMA operand layout.  The 4 x 64 logits of a batch are
// staged in LDS and leave as one 256-byte run per query row.
//
// Vector-memory waits are explicit: the counter (vmcnt) retires in issue
// order, so waiting for batch i means allowing every younger load and store
// of this wave to stay outstanding.
// ---------------------------------------------------------------------------
#ifndef TQ_SCORES_WAVES
#define TQ_SCORES_WAVES 4096
#endif
#ifndef TQ_SCORES_RING
#define TQ_SCORES_RING 2
#endif
constexpr int kTargetWaves = TQ_SCORES_WAVES;   // resident waves aimed at (256 CUs x 4 SIMDs x 4)
constexpr int kRing = TQ_SCORES_RING;
constexpr int kBatchKeys = 64;
// cache policy of the staging copies: non-temporal (nt).  Every packed key is
// read once per call; marking the stream non-temporal keeps it from
// displacing other lines and measured 5% faster (30.4 -> 28.9 us back to back)
constexpr int kNt = 2;

template <int WPK, bool QJL>
struct DmaPlan {
  // bytes per lane per load; the 12-byte form places lanes 16 bytes apart in LDS, so it is not used
  static constexpr int SZ = (WPK % 4 == 0) ? 16 : 4;
  static constexpr int WPL = SZ / 4;                                            // words per lane per load
  static constexpr int NC = WPK / WPL;                                          // loads for the packed words
  static constexpr int L = NC + (QJL ? 2 : 1);                                  // + norms (+ gammas)
};

// issue the loads of one batch (keys k0 .. k0+63 of a sequence of n keys) into an LDS slot
template <int WPK, bool QJL>
__device__ __forceinline__ void issue_batch(uint32_t* slot, const uint32_t* __restrict__ cbase,
                                            const float* __restrict__ nb, const float* __restrict__ gb, int64_t k0,
                                            int64_t n, int lane) {
  using P = DmaPlan<WPK, QJL>;
  // valid words from this batch's start (> 0), at most the batch's own; the
  // offsets are 32-bit bytes from the batch's uniform start, so each copy
  // addresses as scalar base + vector offset
  const uint32_t limit = static_cast<uint32_t>(min((n - k0) * WPK, static_cast<int64_t>(kBatchKeys * WPK)));
  const char* base = reinterpret_cast<const char*>(cbase + k0 * WPK);
#pragma unroll
  for (int i = 0; i < P::NC; ++i) {
    uint32_t off = static_cast<uint32_t>(i * 64 * P::WPL) + static_cast<uint32_t>(lane * P::WPL);
    if (off + P::WPL > limit) off = limit - P::WPL;   // past the end: re-read the last valid words
    const uint32_t* src = reinterpret_cast<const uint32_t*>(base + 4u * off);
    lds_ptr_t* dst = as_lds(slot + i * 64 * P::WPL);
    if constexpr (P::SZ == 16) {
      __builtin_amdgcn_global_load_lds(src, dst, 16, 0, kNt);
    } else {
      __builtin_amdgcn_global_load_lds(src, dst, 4, 0, kNt);
    }
  }
  // key k0 + lane, clamped to n - 1 (k0 < n)
  const uint32_t kb = 4u * static_cast<uint32_t>(min(static_cast<int64_t>(lane), n - 1 - k0));
  float* ng = reinterpret_cast<float*>(slot + kBatchKeys * WPK);
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const float*>(reinterpret_cast<const char*>(nb + k0) + kb), as_lds(ng),
                                   4, 0, kNt);
  if constexpr (QJL)
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const float*>(reinterpret_cast<const char*>(gb + k0) + kb),
                                     as_lds(ng + kBatchKeys), 4, 0, kNt);
}

// QJL: prod keys (BP index planes + the QJL plane, gamma per key); without
// it MSE-only keys (BP index planes, norms only).
template <int BP, int GW, bool QJL>
__global__ void __launch_bounds__(256) scores_kernel(const uint32_t* __restrict__ codes, const float* __restrict__ norms,
                                                     const float* __restrict__ gammas, int64_t n, int Hq, int Hkv,
                                                     int G, int RT, const uint8_t* __restrict__ wsA,
                                                     const float* __restrict__ wsC, float* __restrict__ out) {
  constexpr int T = (1 << (BP - 1)) + (QJL ? 1 : 0);
  constexpr int W = BP + (QJL ? 1 : 0);
  constexpr int C = (GW + 3) / 4;
  constexpr int WPK = GW * W;                                   // packed words per key
  constexpr int SLOTW = kBatchKeys * WPK + 2 * kBatchKeys;      // words per ring slot
  constexpr int WAVEW = kRing * SLOTW + 4 * kBatchKeys;         // + logit staging
  using P = DmaPlan<WPK, QJL>;
  constexpr int L = P::L;
  __shared__ __attribute__((aligned(16))) uint32_t lds[4 * WAVEW];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t* ring = lds + wave * WAVEW;
  float* lout = reinterpret_cast<float*>(ring + kRing * SLOTW);

  const int gy = blockIdx.y;
  const int grp = gy / RT, rt = gy - grp * RT;
  const int b = grp / Hkv, kvh = grp - b * Hkv;
  const int qi = lane >> 4, j = lane & 15, g = lane >> 4;

  const uint32_t* cbase = codes + static_cast<int64_t>(grp) * n * WPK;
  const float* nb = norms + static_cast<int64_t>(grp) * n;
  const float* gb = QJL ? gammas + static_cast<int64_t>(grp) * n : nullptr;
  const int64_t nbatch = (n + kBatchKeys - 1) / kBatchKeys;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 4;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (first >= nbatch) return;
  const int nbw = static_cast<int>((nbatch - first + stride - 1) / stride);   // batches of this wave

  // prologue: fill the ring
#pragma unroll
  for (int s2 = 0; s2 < kRing; ++s2)
    if (s2 < nbw) issue_batch<WPK, QJL>(ring + s2 * SLOTW, cbase, nb, gb, (first + s2 * stride) * kBatchKeys, n, lane);

  // query-side operands (L2 resident)
  v8i A[T][C];
  const v8i* ap = reinterpret_cast<const v8i*>(wsA + static_cast<int64_t>(gy) * T * C * 2048);
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < C; ++c) A[t][c] = ap[(t * C + c) * 64 + lane];
  float cs[10];
  {
    const float* cp = wsC + (static_cast<int64_t>(gy) * 4 + qi) * 16;
#pragma unroll
    for (int i = 0; i < 10; ++i) cs[i] = cp[i];
  }
  // output row of lane l in the store phase: query (l >> 4), keys 4*(l & 15) .. +3
  const int sqg = rt * 4 + (lane >> 4);
  float* srow = (sqg < G) ? out + (static_cast<int64_t>(b) * Hq + kvh * G + sqg) * n : nullptr;
  const bool vec_store = (n & 3) == 0;
  const int S = vec_store ? 1 : 4;   // store instructions per batch (all but the last batch)

  for (int i = 0; i < nbw; ++i) {
    const int64_t k0 = (first + static_cast<int64_t>(i) * stride) * kBatchKeys;
    uint32_t* slot = ring + (i % kRing) * SLOTW;
    const float* lng = reinterpret_cast<const float*>(slot + kBatchKeys * WPK);
    // wait for this batch: younger ops are the loads of later batches already issued
    // and the stores of the previous kRing-1 iterations
    {
      const int cl = min(kRing - 1, nbw - 1 - i);
      const int cst = min(i, kRing - 1);
      wait_vm_upto<(kRing - 1) * (L + 4)>(cl * L + cst * S);
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kk = 16 * u + j;   // key of this lane within the batch
      v4f accM = {0.f, 0.f, 0.f, 0.f}, accQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int gg = 4 * c + g;
        uint32_t w[5] = {0u, 0u, 0u, 0u, 0u};
        if (gg < GW) {
#pragma unroll
          for (int p = 0; p < W; ++p) w[p] = slot[(kk * GW + gg) * W + p];
        }
#pragma unroll
        for (int t = 0; t < (1 << (BP - 1)); ++t)
          accM = mfma_fp8_fp4(A[t][c], key_bits_to_fp4(walsh_word<BP>(w, t)), accM);
        if constexpr (QJL) accQ = mfma_fp8_fp4(A[T - 1][c], key_bits_to_fp4(w[BP]), accQ);
      }
      pin(accM);
      const float mse = fmaf(accM[0], cs[2], fmaf(accM[1], cs[3], fmaf(accM[2], cs[4], fmaf(accM[3], cs[5], cs[0]))));
      if constexpr (QJL) {
        pin(accQ);
        const float qjl = fmaf(accQ[0], cs[6], fmaf(accQ[1], cs[7], fmaf(accQ[2], cs[8], fmaf(accQ[3], cs[9], cs[1]))));
        lout[qi * kBatchKeys + kk] = fmaf(lng[kk], mse, lng[kBatchKeys + kk] * qjl);
      } else {
        lout[qi * kBatchKeys + kk] = lng[kk] * mse;
      }
    }
    __builtin_amdgcn_wave_barrier();
    {
      typedef float f4 __attribute__((ext_vector_type(4)));
      const f4 v = *reinterpret_cast<const f4*>(lout + (lane >> 4) * kBatchKeys + 4 * (lane & 15));
      const int64_t key = k0 + 4 * (lane & 15);
      if (srow) {
        if (vec_store && key + 4 <= n) {
          *reinterpret_cast<f4*>(srow + key) = v;   // write-back: the next consumer reads it from cache
        } else {
          if (key + 0 < n) srow[key + 0] = v.x;
          if (key + 1 < n) srow[key + 1] = v.y;
          if (key + 2 < n) srow[key + 2] = v.z;
          if (key + 3 < n) srow[key + 3] = v.w;
        }
      }
    }
    // every LDS read of this slot (and of the staging area) has returned before
    // the slot is refilled and the staging area rewritten
    wait_lgkm0();
    __builtin_amdgcn_wave_barrier();
    if (i + kRing < nbw)
      issue_batch<WPK, QJL>(slot, cbase, nb, gb, (first + static_cast<int64_t>(i + kRing) * stride) * kBatchKeys, n, lane);
  }
}

int64_t scores_ws_bytes(const tq_quantizer* q, int B, int Hq, int Hkv) {
  // 256 < d: the float [Pi q; S q] of every query
  if (q->d > 256) return static_cast<int64_t>(B) * Hq * (q->d + q->m) * 4 + 256;
  const int G = Hq / Hkv;
  const int RT = (G + 3) / 4;
  const int T = key_terms(q);
  const int C = (q->d + 127) / 128;
  const int64_t groups = static_cast<int64_t>(B) * Hkv * RT;
  return groups * T * C * 2048 + groups * 4 * 16 * 4;
}

hipError_t launch_query_prep(const tq_quantizer* q, const void* queries, int q_dtype, int B, int Hq, int Hkv,
                             uint8_t* wsA, float* wsC, hipStream_t st, bool bound) {
  const int G = Hq / Hkv;
  const int RT = (G + 3) / 4;
  const int C = (q->d + 127) / 128;
  const size_t lds = sizeof(float) * (2 * q->d + q->m + 4 * (q->d + q->m));
  dim3 grid(static_cast<unsigned>(static_cast<int64_t>(B) * Hkv * RT * 4));
  const int dm = q->d + q->m;
  const bool one = dm % 4 == 0 && dm <= 256 && q->d <= 128;
#define TQ_QP(BF, ONE, BD)                                                                                            \
  hipLaunchKernelGGL((query_prep_kernel<BF, ONE, BD>), grid, dim3(256), lds, st, queries, q_dtype, Hq, Hkv, G, RT, q->d, \
                     q->m, q->d_qt, key_codebook(q), key_qjl(q) ? 1 : 0, C, wsA, wsC)
  if (bound) {
    if (q_dtype == 1) {
      if (one) TQ_QP(true, true, true); else TQ_QP(true, false, true);
    } else {
      if (one) TQ_QP(false, true, true); else TQ_QP(false, false, true);
    }
  } else {
    if (q_dtype == 1) {
      if (one) TQ_QP(true, true, false); else TQ_QP(true, false, false);
    } else {
      if (one) TQ_QP(false, true, false); else TQ_QP(false, false, false);
    }
  }
#undef TQ_QP
  return hipGetLastError();
}

hipError_t launch_query_prep_multi(const tq_quantizer* const* qs, void* const* ws, int nq, const void* queries,
                                   int q_dtype, int B, int Hq, int Hkv, hipStream_t st) {
  if (nq < 1 || nq > kPrepSetMax) return hipErrorInvalidValue;
  const tq_quantizer* q0 = qs[0];
  const int G = Hq / Hkv;
  const int RT = (G + 3) / 4;
  const int C = (q0->d + 127) / 128;
  const int64_t groups = static_cast<int64_t>(B) * Hkv * RT;
  PrepSet set = {};
  for (int k = 0; k < nq; ++k) {
    if (qs[k]->d != q0->d || qs[k]->m != q0->m) return hipErrorInvalidValue;
    set.qt[k] = qs[k]->d_qt;
    set.cb[k] = key_codebook(qs[k]);
    set.qjl[k] = key_qjl(qs[k]) ? 1 : 0;
    set.wsA[k] = static_cast<uint8_t*>(ws[k]);
    set.wsC[k] = reinterpret_cast<float*>(set.wsA[k] + groups * key_terms(qs[k]) * C * 2048);
  }
  const size_t lds = sizeof(float) * (2 * q0->d + q0->m + 4 * (q0->d + q0->m));
  dim3 grid(static_cast<unsigned>(groups * 4), static_cast<unsigned>(nq));
  const int dm = q0->d + q0->m;
  const bool one = dm % 4 == 0 && dm <= 256 && q0->d <= 128;
#define TQ_QPM(BF, ONE)                                                                                            \
  hipLaunchKernelGGL((query_prep_multi_kernel<BF, ONE>), grid, dim3(256), lds, st, queries, q_dtype, Hq, Hkv, G, RT, \
                     q0->d, q0->m, C, set)
  if (q_dtype == 1) {
    if (one) TQ_QPM(true, true); else TQ_QPM(true, false);
  } else {
    if (one) TQ_QPM(false, true); else TQ_QPM(false, false);
  }
#undef TQ_QPM
  return hipGetLastError();
}

hipError_t launch_query_prep_ws(const tq_quantizer* q, const void* queries, int q_dtype, int B, int Hq, int Hkv,
                                void* ws, hipStream_t st, bool bound) {
  const int G = Hq / Hkv;
  const int RT = (G + 3) / 4;
  const int T = key_terms(q);
  const int C = (q->d + 127) / 128;
  const int64_t groups = static_cast<int64_t>(B) * Hkv * RT;
  uint8_t* wsA = static_cast<uint8_t*>(ws);
  float* wsC = reinterpret_cast<float*>(wsA + groups * T * C * 2048);
  return launch_query_prep(q, queries, q_dtype, B, Hq, Hkv, wsA, wsC, st, bound);
}

hipError_t launch_scores_scan(const tq_quantizer* q, int B, int Hq, int Hkv, const uint32_t* codes, const float* norms,
                              const float* gammas, int64_t n, float* out, const void* ws, hipStream_t st) {
  const int G = Hq / Hkv;
  const int RT = (G + 3) / 4;
  const int T = key_terms(q);
  const int C = (q->d + 127) / 128;
  const int64_t groups = static_cast<int64_t>(B) * Hkv * RT;
  const uint8_t* wsA = static_cast<const uint8_t*>(ws);
  const float* wsC = reinterpret_cast<const float*>(wsA + groups * T * C * 2048);
  const int64_t nbatch = (n + kBatchKeys - 1) / kBatchKeys;
  int64_t bx = (kTargetWaves / 4 + groups - 1) / groups;
  const int64_t need = (nbatch + 3) / 4;
  if (bx > need) bx = need;
  if (bx < 1) bx = 1;
  dim3 grid(static_cast<unsigned>(bx), static_cast<unsigned>(groups));
  const int bp = key_codebook(q).bp;
  const bool qjl = key_qjl(q);
  const int gw = (q->d + 31) / 32;
#define TQ_SC(BPV, GWV, QV)                                                                                       \
  if (bp == BPV && gw == GWV && qjl == QV) {                                                                      \
    hipLaunchKernelGGL((scores_kernel<BPV, GWV, QV>), grid, dim3(256), 0, st, codes, norms, gammas, n, Hq, Hkv, G, \
                       RT, wsA, wsC, out);                                                                        \
    return hipGetLastError();                                                                                     \
  }
#define TQ_SC_ALL(GWV)                                                                                  \
  TQ_SC(1, GWV, true) TQ_SC(2, GWV, true) TQ_SC(3, GWV, true) TQ_SC(1, GWV, false) TQ_SC(2, GWV, false) \
  TQ_SC(3, GWV, false) TQ_SC(4, GWV, false)
  TQ_SC_ALL(1) TQ_SC_ALL(2) TQ_SC_ALL(3) TQ_SC_ALL(4) TQ_SC_ALL(5) TQ_SC_ALL(6) TQ_SC_ALL(7) TQ_SC_ALL(8)
#undef TQ_SC_ALL
#undef TQ_SC
  return hipErrorNotSupported;
}

// ---------------------------------------------------------------------------
// Logits for 256 < d <= 1024, on the vector ALU: the operand layout of the
// matrix-core scan holds at most 8 words per key in registers.  The prep
// writes q^ = Pi q and s = S q of every query in float; the scan gives a
// thread to a key, walks its packed words and accumulates
//   logit = n <q^, c[idx]> + gamma sqrt(pi/2)/m <s, sigma>
// (blog.hotdry.top "TurboQuant vector-search compression", QJL section) for
// up to 4 queries of its KV group per pass, with their vectors in LDS.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) big_prep_kernel(const void* __restrict__ queries, int q_dtype, int d, int m,
                                                       const float* __restrict__ qt, float* __restrict__ qs) {
  __shared__ float qv[kMaxEncodeD];
  const int64_t qh = blockIdx.x;   // b * Hq + h
  const int tid = threadIdx.x;
  for (int k = tid; k < d; k += 256) qv[k] = load_elem(queries, q_dtype, qh * d + k);
  __syncthreads();
  const int dm = d + m;
  for (int o = tid; o < dm; o += 256) {
    float a = 0.f;
    for (int k = 0; k < d; ++k) a = fmaf(qt[static_cast<int64_t>(k) * dm + o], qv[k], a);
    qs[qh * dm + o] = a;
  }
}

constexpr int kBigQ = 4;   // queries per pass of the scan

template <bool QJL>
__global__ void __launch_bounds__(256) big_scores_kernel(const uint32_t* __restrict__ codes,
                                                         const float* __restrict__ norms,
                                                         const float* __restrict__ gammas, int64_t n, int d, int m,
                                                         int Hq, int Hkv, const float* __restrict__ qs, Codebook cb,
                                                         float* __restrict__ out) {
  __shared__ float qsh[kBigQ][2 * kMaxEncodeD];
  __shared__ float cen[kMaxLevels];
  const int tid = threadIdx.x;
  const int G = Hq / Hkv;
  const int64_t seq = blockIdx.y;
  const int64_t b = seq / Hkv;
  const int kvh = static_cast<int>(seq - b * Hkv);
  const int64_t key = static_cast<int64_t>(blockIdx.x) * 256 + tid;
  const int dm = d + m;
  const int GW = (d + 31) / 32, bp = cb.bp, W = bp + (QJL ? 1 : 0);
  const float alpha = 1.2533141373155003f / static_cast<float>(m);   // sqrt(pi/2) / m
  if (tid < kMaxLevels) cen[tid] = tid < cb.levels ? cb.c[tid] : 0.f;
  for (int q0 = 0; q0 < G; q0 += kBigQ) {
    const int nq = min(kBigQ, G - q0);
    const int64_t qrow = b * Hq + static_cast<int64_t>(kvh) * G + q0;   // first query of the pass
    __syncthreads();
    for (int e = tid; e < nq * dm; e += 256) {
      const int t = e / dm, o = e - t * dm;
      qsh[t][o] = qs[(qrow + t) * dm + o];
    }
    __syncthreads();
    if (key >= n) continue;
    float am[kBigQ] = {0.f, 0.f, 0.f, 0.f}, aq[kBigQ] = {0.f, 0.f, 0.f, 0.f};
    const uint32_t* kw = codes + (seq * n + key) * GW * W;
    for (int gw = 0; gw < GW; ++gw) {
      uint32_t w[5] = {0u, 0u, 0u, 0u, 0u};
      for (int p = 0; p < W; ++p) w[p] = kw[gw * W + p];
      const int nb = min(32, d - 32 * gw);
      for (int bit = 0; bit < nb; ++bit) {
        const int j = 32 * gw + bit;
        int idx = 0;
        for (int p = 0; p < bp; ++p) idx |= static_cast<int>((w[p] >> bit) & 1u) << p;
        const float c = cen[idx];
        const float sg = QJL ? (((w[bp] >> bit) & 1u) ? 1.f : -1.f) : 0.f;
#pragma unroll
        for (int t = 0; t < kBigQ; ++t) {
          am[t] = fmaf(c, qsh[t][j], am[t]);
          if constexpr (QJL) aq[t] = fmaf(sg, qsh[t][d + j], aq[t]);
        }
      }
    }
    const float nv = norms[seq * n + key];
    const float gv = QJL ? gammas[seq * n + key] : 0.f;
    for (int t = 0; t < nq; ++t)
      out[(qrow + t) * n + key] = QJL ? fmaf(nv, am[t], gv * alpha * aq[t]) : nv * am[t];
  }
}

static hipError_t launch_scores_big(const tq_quantizer* q, const void* queries, int q_dtype, int B, int Hq, int Hkv,
                                    const uint32_t* codes, const float* norms, const float* gammas, int64_t n,
                                    float* out, void* ws, hipStream_t st) {
  if (q->d > kMaxEncodeD || q->m > kMaxEncodeD) return hipErrorNotSupported;
  float* qs = static_cast<float*>(ws);
  hipLaunchKernelGGL(big_prep_kernel, dim3(static_cast<unsigned>(static_cast<int64_t>(B) * Hq)), dim3(256), 0, st,
                     queries, q_dtype, q->d, q->m, q->d_qt, qs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<unsigned>((n + 255) / 256), static_cast<unsigned>(static_cast<int64_t>(B) * Hkv));
  if (key_qjl(q))
    hipLaunchKernelGGL((big_scores_kernel<true>), grid, dim3(256), 0, st, codes, norms, gammas, n, q->d, q->m, Hq, Hkv,
                       qs, key_codebook(q), out);
  else
    hipLaunchKernelGGL((big_scores_kernel<false>), grid, dim3(256), 0, st, codes, norms, gammas, n, q->d, q->m, Hq,
                       Hkv, qs, key_codebook(q), out);
  return hipGetLastError();
}

hipError_t launch_scores(const tq_quantizer* q, const void* queries, int q_dtype, int B, int Hq, int Hkv,
                         const uint32_t* codes, const float* norms, const float* gammas, int64_t n, float* out,
                         void* ws, hipStream_t st) {
  if (q->d > 256) return launch_scores_big(q, queries, q_dtype, B, Hq, Hkv, codes, norms, gammas, n, out, ws, st);
  hipError_t e = launch_query_prep_ws(q, queries, q_dtype, B, Hq, Hkv, ws, st);
  if (e != hipSuccess) return e;
  return launch_scores_scan(q, B, Hq, Hkv, codes, norms, gammas, n, out, ws, st);
}

}  // namespace tq
