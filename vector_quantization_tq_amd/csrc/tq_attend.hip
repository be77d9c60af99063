// Decode attention over the packed cache, and top-k search over packed keys.
//
// Attention (decode step, one query per head): logits from the packed keys as
// in tq_scores (a2a-mcp.org "什麼是TurboQuant？", how-to-implement: fused kernel
// from indices with the query pre-rotated once), softmax over them (scaled dot
// product, max-subtracted), and the weighted sum of MSE-decoded values
// (friday-blog "TurboQuant 深度解析（二）", section 1: values take the
// rotation + scalar-quantiser stage).  The most recent tokens may stay in
// bf16 (blog.hotdry.top "TurboQuant vector-search compression", engineering
// configuration: keep the latest 128-256 tokens in full precision).
//
// Split over token chunks (flash-decoding): one workgroup per (KV group,
// row tile of 4 queries, chunk).  Per step of 128 tokens:
//   K phase   each wave scores 2 tiles of 16 keys on the f8f6f4 MFMA
//             (fp8 query limbs x fp4 key bit planes, as the logits kernel);
//   softmax   one wave per query: running max m, sum l (base 2), weights
//             w_t = p_t * ||v_t||, split into 4 fp8 limbs in the MFMA A layout;
//   V phase   sum_t w_t c[idx_t] in the value quantizer's rotated frame, again
//             on the f8f6f4 MFMA: tokens are the contraction dimension, the
//             32-token value words are the fp4 B operand, c[idx] is written in
//             the +-1 basis of the index bits (Walsh terms), each wave owns
//             32 output coordinates.
// A merge kernel combines the chunks, adds the exact bf16 tail, applies
// Pi_v^T once per query and divides by the softmax sum.
#include "tq_device.h"
#include "tq_kernels.h"

namespace tq {

namespace {

constexpr int kStep = 128;          // tokens per step
constexpr float kLog2e = 1.4426950408889634f;

// Fixed-point limbs of x in [0, 16): x ~ l0 + l1/16 + l2/256 + l3/4096 with
// every limb a small integer (|l| <= 16), exact in fp8 E4M3.  Byte k of the
// result is limb k.  The matrix core sums the products of a row in groups of 8,
// aligned to the largest product of the group, so limbs that are integers on
// one common scale keep those group sums exact whatever the spread of the
// weights (per-element floating limbs would lose the small ones).
__device__ __forceinline__ uint32_t fixed_limbs4(float x) {
  const float l0 = rintf(x);
  float r = (x - l0) * 16.f;
  const float l1 = rintf(r);
  r = (r - l1) * 16.f;
  const float l2 = rintf(r);
  r = (r - l2) * 16.f;
  const float l3 = rintf(r);
  const int b01 = __builtin_amdgcn_cvt_pk_fp8_f32(l0, l1, 0, false);
  const int b23 = __builtin_amdgcn_cvt_pk_fp8_f32(l2, l3, 0, false);
  return (static_cast<uint32_t>(b01) & 0xFFFFu) | (static_cast<uint32_t>(b23) << 16);
}

}  // namespace

// partial record of one (group row tile, chunk, query): acc[128] then m, l
constexpr int kPartStride = 128 + 4;

// chunk length (a multiple of the step): the largest power-of-two multiple of
// 128 tokens, up to 4096, that still leaves about 2048 workgroups
static int64_t attend_chunk_len(int64_t n_comp, int64_t groups) {
  int64_t ch = kStep;
  while (ch < 4096 && (n_comp + 2 * ch - 1) / (2 * ch) * groups >= 2048) ch *= 2;
  return ch;
}

static int64_t attend_chunks(int64_t n_comp, int64_t groups) {
  if (n_comp <= 0) return 0;
  const int64_t ch = attend_chunk_len(n_comp, groups);
  return (n_comp + ch - 1) / ch;
}

int64_t attend_ws_bytes(const tq_quantizer* kq, const tq_quantizer*, int B, int Hq, int Hkv, int64_t n_comp, int) {
  const int G = Hq / Hkv;
  const int RT = (G + 3) / 4;
  const int64_t groups = static_cast<int64_t>(B) * Hkv * RT;
  const int64_t nch = attend_chunks(n_comp, groups);
  const int64_t prep = (scores_ws_bytes(kq, B, Hq, Hkv) + 255) / 256 * 256;
  return prep + groups * nch * 4 * kPartStride * 4 + 256;
}

template <int BPK, int BPV>
__global__ void __launch_bounds__(256) attend_chunk_kernel(
    const uint32_t* __restrict__ kcodes, const float* __restrict__ knorms, const float* __restrict__ kgammas,
    const uint32_t* __restrict__ vcodes, const float* __restrict__ vnorms, int64_t n, int64_t chunk, int G, int RT,
    float scale_log2, const uint8_t* __restrict__ wsA, const float* __restrict__ wsC, Codebook vcb,
    float* __restrict__ part) {
  constexpr int d = 128;
  constexpr int TK = (1 << (BPK - 1)) + 1;   // key MFMA terms (Walsh + QJL)
  constexpr int WK = BPK + 1;                // key words per 32-coordinate group
  constexpr int NV = 1 << (BPV - 1);         // value Walsh terms
  __shared__ float sc[4][kStep];             // scaled logits (base 2)
  __shared__ __attribute__((aligned(16))) uint32_t av[64 * 8];   // value A operand (fp8 limbs)
  __shared__ float qst[4][4];                // per query: rescale factor, E

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gy = blockIdx.y;
  const int grp = gy / RT, rt = gy - grp * RT;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t c1 = min(n, c0 + chunk);
  const int qi = lane >> 4, j = lane & 15, g = lane >> 4;

  v8i AK[TK];
  {
    const v8i* ap = reinterpret_cast<const v8i*>(wsA + static_cast<int64_t>(gy) * TK * 2048);
#pragma unroll
    for (int t = 0; t < TK; ++t) AK[t] = ap[t * 64 + lane];
  }
  float cs[10];
  {
    const float* cp = wsC + (static_cast<int64_t>(gy) * 4 + qi) * 16;
#pragma unroll
    for (int i = 0; i < 10; ++i) cs[i] = cp[i];
  }
  const uint32_t* kb = kcodes + static_cast<int64_t>(grp) * n * 4 * WK;
  const float* knb = knorms + static_cast<int64_t>(grp) * n;
  const float* kgb = kgammas + static_cast<int64_t>(grp) * n;
  const int64_t nbk = (n + 31) >> 5;
  const uint32_t* vb = vcodes + static_cast<int64_t>(grp) * nbk * BPV * d;
  const float* vnb = vnorms + static_cast<int64_t>(grp) * n;

  // running softmax state of query `wave` (softmax phase) -- kept by every lane of that wave
  float m_run = -INFINITY, l_run = 0.f, w_run = 0.f;
  int e_run = 0;
  // value accumulators: [Walsh term][column tile of this wave]; rows 4q+limb, column 16ct+j
  v4f acc[NV][2];
#pragma unroll
  for (int t = 0; t < NV; ++t) acc[t][0] = acc[t][1] = (v4f){0.f, 0.f, 0.f, 0.f};
  int e_acc = 0;   // scale exponent the accumulators are in (per query, same in every wave)

  for (int64_t t0 = c0; t0 < c1; t0 += kStep) {
    // ---------------- K phase: logits of tokens t0 + 32*wave .. +31 ----------------
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tt = 32 * wave + 16 * u + j;   // token within the step
      const int64_t key = t0 + tt;
      const bool kv = key < c1;
      uint32_t w[5] = {0u, 0u, 0u, 0u, 0u};
      if (kv) {
        const uint32_t* wp = kb + (key * 4 + g) * WK;
#pragma unroll
        for (int p = 0; p < WK; ++p) w[p] = wp[p];
      }
      v4f aM = {0.f, 0.f, 0.f, 0.f}, aQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < TK - 1; ++t) aM = mfma_fp8_fp4(AK[t], bits_to_fp4(walsh_word<BPK>(w, t)), aM);
      aQ = mfma_fp8_fp4(AK[TK - 1], bits_to_fp4(w[BPK]), aQ);
      pin(aM);
      pin(aQ);
      const float mse = fmaf(aM[0], cs[2], fmaf(aM[1], cs[3], fmaf(aM[2], cs[4], fmaf(aM[3], cs[5], cs[0]))));
      const float qjl = fmaf(aQ[0], cs[6], fmaf(aQ[1], cs[7], fmaf(aQ[2], cs[8], fmaf(aQ[3], cs[9], cs[1]))));
      float s = -INFINITY;
      if (kv) s = fmaf(knb[key], mse, kgb[key] * qjl) * scale_log2;
      sc[qi][tt] = s;
    }
    __syncthreads();
    // ---------------- softmax phase: wave q handles query q ----------------
    {
      const int q = wave;
      const int ta = 2 * lane, tb = 2 * lane + 1;
      const float sa = sc[q][ta], sb = sc[q][tb];
      float mx = fmaxf(sa, sb);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);   // 0 on the first step
      const float pa = exp2f(sa - m_new), pb = exp2f(sb - m_new);
      const float na = (t0 + ta < c1) ? vnb[t0 + ta] : 0.f;
      const float nb2 = (t0 + tb < c1) ? vnb[t0 + tb] : 0.f;
      const float wa = pa * na, wb = pb * nb2;
      float ps = pa + pb, wm = fmaxf(wa, wb);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        ps += __shfl_xor(ps, off);
        wm = fmaxf(wm, __shfl_xor(wm, off));
      }
      l_run = fmaf(l_run, alpha, ps);
      m_run = m_new;
      // the A values are w / (fp4 slot value >= 0.5): 2 * max lands in [8, 16)
      const int e_new = wm > 0.f ? 3 - ilogbf(2.f * wm) : e_run;
      if (lane == 0) {
        qst[q][0] = ldexpf(alpha, e_new - e_run);   // accumulator rescale for this query
        qst[q][1] = static_cast<float>(e_new);
      }
      e_run = e_new;
      // A operand of the value MFMA: rows 4q + limb, K = token slot.  The
      // weight sum that enters the Walsh constant term is taken over the
      // quantised weights, so that sum_t w_t (2 b_t - 1) is exact for them.
      float wq_sum = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tk = 2 * lane + h;
        const float wt = h ? wb : wa;
        // token -> K: token = 32(K/32) + 4(K%8) + (K%32)/8; K -> (lane-group, element)
        const int hh = tk >> 5, rem = tk & 31;
        const int K = 32 * hh + 8 * (rem & 3) + (rem >> 2);
        const int gg = (K & 63) >> 4, e = 16 * (K >> 6) + (K & 15);
        const float v = ldexpf(wt / fp4_slot_value((K & 31) >> 3), e_new);
        const uint32_t limbs = fixed_limbs4(v);
        {
          float rec = 0.f;
#pragma unroll
          for (int lb = 3; lb >= 0; --lb)
            rec = fmaf(rec, 1.f / 16.f, __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(limbs >> (8 * lb)), 0));
          wq_sum = fmaf(ldexpf(rec, -e_new), fp4_slot_value((K & 31) >> 3), wq_sum);
        }
        uint8_t* avb = reinterpret_cast<uint8_t*>(av);
#pragma unroll
        for (int lb = 0; lb < 4; ++lb) avb[(4 * q + lb + 16 * gg) * 32 + e] = static_cast<uint8_t>(limbs >> (8 * lb));
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) wq_sum += __shfl_xor(wq_sum, off);
      w_run = fmaf(w_run, alpha, wq_sum);
    }
    __syncthreads();
    // ---------------- V phase: wave owns coordinates 32*wave .. +31 ----------------
    {
      const v8i A = *reinterpret_cast<const v8i*>(av + lane * 8);
      const float rs = qst[qi][0];
      e_acc = static_cast<int>(qst[qi][1]);
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        acc[t][0] *= rs;
        acc[t][1] *= rs;
      }
      const int64_t blk = (t0 >> 5) + g;   // 32-token block of this lane group
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int col = 32 * wave + 16 * ct + j;
        uint32_t w[5] = {0u, 0u, 0u, 0u, 0u};
        if (blk < nbk) {
          const uint32_t* wp = vb + (blk * BPV) * d + col;
#pragma unroll
          for (int p = 0; p < BPV; ++p) w[p] = wp[p * d];
        }
#pragma unroll
        for (int t = 0; t < NV; ++t) acc[t][ct] = mfma_fp8_fp4(A, bits_to_fp4(walsh_word<BPV>(w, t)), acc[t][ct]);
      }
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        pin(acc[t][0]);
        pin(acc[t][1]);
      }
    }
    __syncthreads();
  }

  // ---------------- chunk result ----------------
  // value part: sum_t w_t c[idx] = sum_S coef_S (2 sum_t w_t b_S - sum_t w_t);
  // the softmax state of query q lives in wave q: publish it
  if (lane == 0) {
    qst[wave][2] = w_run;
    qst[wave][3] = l_run;
    qst[wave][0] = m_run;
  }
  __syncthreads();
  const float wq = qst[qi][2];
  float* pbase = part + ((static_cast<int64_t>(gy) * gridDim.x + blockIdx.x) * 4) * kPartStride;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    float v = 0.f;
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      const v4f a = acc[t][ct];
      const float sum = ldexpf(fmaf(a[3], 1.f / 4096.f, fmaf(a[2], 1.f / 256.f, fmaf(a[1], 1.f / 16.f, a[0]))), -e_acc);
      v = fmaf(vcb.coef[t], fmaf(2.f, sum, -wq), v);
    }
    pbase[qi * kPartStride + 32 * wave + 16 * ct + j] = v;
  }
  if (threadIdx.x < 4) {
    pbase[threadIdx.x * kPartStride + 128] = qst[threadIdx.x][0];
    pbase[threadIdx.x * kPartStride + 129] = qst[threadIdx.x][3];
  }
}

// one workgroup (128 threads) per (batch, query head)
__global__ void __launch_bounds__(256) attend_merge_kernel(const void* __restrict__ queries, int q_dtype, int Hq,
                                                           int Hkv, int G, int RT, int64_t nchunk,
                                                           const float* __restrict__ part,
                                                           const uint16_t* __restrict__ k_tail,
                                                           const uint16_t* __restrict__ v_tail, int n_tail,
                                                           float scale_log2, const float* __restrict__ piv,
                                                           float* __restrict__ out) {
  constexpr int d = 128;
  __shared__ float qv[d];
  __shared__ float accs[d];
  __shared__ float red[8];
  __shared__ float ts[512];   // tail logits (n_tail <= 512)
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / Hq, h = bh - b * Hq;
  const int kvh = h / G, qg = h - kvh * G;
  const int rt = qg >> 2, qi = qg & 3;
  const int64_t gy = (static_cast<int64_t>(b) * Hkv + kvh) * RT + rt;
  if (tid < d) qv[tid] = load_elem(queries, q_dtype, static_cast<int64_t>(bh) * d + tid);
  // global max over chunks and tail
  float mloc = -INFINITY;
  for (int64_t c = tid; c < nchunk; c += blockDim.x)
    mloc = fmaxf(mloc, part[((gy * nchunk + c) * 4 + qi) * kPartStride + 128]);
  __syncthreads();
  const int64_t toff = (static_cast<int64_t>(b) * Hkv + kvh) * n_tail;
  for (int t = tid; t < n_tail; t += blockDim.x) {
    const uint16_t* kt = k_tail + (toff + t) * d;
    float s = 0.f;
    for (int k = 0; k < d; ++k) s = fmaf(qv[k], bf16_to_f32(kt[k]), s);
    ts[t] = s * scale_log2;
    mloc = fmaxf(mloc, ts[t]);
  }
  for (int off = 32; off > 0; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
  if ((tid & 63) == 0) red[tid >> 6] = mloc;
  __syncthreads();
  float M = -INFINITY;
  for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) M = fmaxf(M, red[w]);
  __syncthreads();
  // denominators
  float lsum = 0.f;
  for (int64_t c = tid; c < nchunk; c += blockDim.x) {
    const float* pc = part + ((gy * nchunk + c) * 4 + qi) * kPartStride;
    lsum += pc[129] * exp2f(pc[128] - M);
  }
  for (int t = tid; t < n_tail; t += blockDim.x) {
    const float p = exp2f(ts[t] - M);
    ts[t] = p;
    lsum += p;
  }
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off);
  if ((tid & 63) == 0) red[tid >> 6] = lsum;
  __syncthreads();
  float L = 0.f;
  for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) L += red[w];
  // rotated-frame accumulator of the compressed part
  if (tid < d) {
    float a = 0.f;
    for (int64_t c = 0; c < nchunk; ++c) {
      const float* pc = part + ((gy * nchunk + c) * 4 + qi) * kPartStride;
      a = fmaf(pc[tid], exp2f(pc[128] - M), a);
    }
    accs[tid] = a;
  }
  __syncthreads();
  if (tid < d) {
    float o = 0.f;
    for (int jj = 0; jj < d; ++jj) o = fmaf(piv[static_cast<int64_t>(jj) * d + tid], accs[jj], o);   // Pi^T acc
    for (int t = 0; t < n_tail; ++t) o = fmaf(ts[t], bf16_to_f32(v_tail[(toff + t) * d + tid]), o);
    out[static_cast<int64_t>(bh) * d + tid] = o / L;
  }
}

hipError_t launch_attend(const tq_quantizer* kq, const tq_quantizer* vq, const void* queries, int q_dtype, int B, int Hq,
                         int Hkv, const uint32_t* kcodes, const float* knorms, const float* kgammas,
                         const uint32_t* vcodes, const float* vnorms, int64_t n_comp, const uint16_t* k_tail,
                         const uint16_t* v_tail, int n_tail, float scale, float* out, void* ws, hipStream_t st) {
  if (kq->d != 128 || n_tail > 512) return hipErrorNotSupported;
  const int G = Hq / Hkv;
  const int RT = (G + 3) / 4;
  const int64_t groups = static_cast<int64_t>(B) * Hkv * RT;
  const int64_t nch = attend_chunks(n_comp, groups);
  const int64_t prep = (scores_ws_bytes(kq, B, Hq, Hkv) + 255) / 256 * 256;
  float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + prep);
  const float sl = scale * kLog2e;
  hipError_t e;
  if (nch > 0) {
    e = launch_query_prep_ws(kq, queries, q_dtype, B, Hq, Hkv, ws, st);
    if (e != hipSuccess) return e;
    const int T = kq->cb[0].nterms + 1;
    const uint8_t* wsA = static_cast<const uint8_t*>(ws);
    const float* wsC = reinterpret_cast<const float*>(wsA + groups * T * 2048);
    const int64_t ch = attend_chunk_len(n_comp, groups);
    dim3 grid(static_cast<unsigned>(nch), static_cast<unsigned>(groups));
    const int bpk = kq->cb[0].bp, bpv = vq->cb[1].bp;
#define TQ_AT(K, V)                                                                                              \
  if (bpk == K && bpv == V) {                                                                                    \
    hipLaunchKernelGGL((attend_chunk_kernel<K, V>), grid, dim3(256), 0, st, kcodes, knorms, kgammas, vcodes, vnorms, \
                       n_comp, ch, G, RT, sl, wsA, wsC, vq->cb[1], part);                                       \
  } else
    TQ_AT(1, 1) TQ_AT(1, 2) TQ_AT(1, 3) TQ_AT(1, 4) TQ_AT(2, 1) TQ_AT(2, 2) TQ_AT(2, 3) TQ_AT(2, 4)
    TQ_AT(3, 1) TQ_AT(3, 2) TQ_AT(3, 3) TQ_AT(3, 4) { return hipErrorNotSupported; }
#undef TQ_AT
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attend_merge_kernel, dim3(static_cast<unsigned>(B * Hq)), dim3(128), 0, st, queries, q_dtype, Hq, Hkv,
                     G, RT, nch, part, k_tail, v_tail, n_tail, sl, vq->d_pi, out);
  return hipGetLastError();
}

}  // namespace tq
