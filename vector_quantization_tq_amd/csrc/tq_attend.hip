// Decode attention over the packed cache: chunking, workspace, the merge
// kernel and the launch sequence (the chunk kernel is in tq_attend_impl.h).
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
//             d/64 tiles of 16 output coordinates (32 coordinates at d = 128).
// A merge kernel combines the chunks, adds the exact bf16 tail, applies
// Pi_v^T once per query and divides by the softmax sum.  Head dimensions 64,
// 96, 128 and 256 each have their chunk-kernel instantiations.
#include "tq_attend_impl.h"

namespace tq {
namespace attn {
// compiled in their own sources (tq_attend_d64.hip, tq_attend_d96.hip, tq_attend_d256.hip)
#define TQ_EXTERN_CHUNKS(DV)                                                                                         \
  extern template hipError_t launch_chunks_d<DV, false>(const AttendSegment&, int64_t, int, int, float, float,      \
                                                       const uint8_t*, const float*, float*, int64_t, int64_t, int64_t, \
                                                       int64_t, hipStream_t);
TQ_EXTERN_CHUNKS(64)
TQ_EXTERN_CHUNKS(96)
TQ_EXTERN_CHUNKS(256)
#undef TQ_EXTERN_CHUNKS
}  // namespace attn

bool attend_supports_d(int d) { return d == 64 || d == 96 || d == 128 || d == 256; }

using attn::kStep;
using attn::kLog2e;

// partial record of one (group row tile, chunk, query): acc[d] then m, l
static int64_t part_stride(int d) { return d + 4; }

static int64_t device_cus() {
  static int64_t cus = [] {
    int dev = 0, c = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        c < 1)
      c = 256;
    return static_cast<int64_t>(c);
  }();
  return cus;
}

// chunk length (a multiple of the step): the largest power-of-two multiple of
// 128 tokens, up to 1024, that still leaves at least 768 workgroups (three
// resident per CU, or three quarters of the slots where four fit); shorter
// ones add partial records and pipeline fills.  `bpc` is the dense kernel's
// residency (attend_blocks_per_cu): the chunking never depends on whether
// sparse V is on, so the workspace size does not either.
static int64_t attend_chunk_len(int64_t n_comp, int64_t groups, int bpc, bool segmented = false) {
  // a cache in several segments: each segment's launch gets the shortest
  // multiple of the step whose chunks fill one round of the resident
  // workgroups, at least 128 and at most 2048 tokens (the launches run one
  // after the other, and one merge reads every segment's records)
  if (segmented && bpc > 0) {
    const int64_t per = max(static_cast<int64_t>(1), bpc * device_cus() / groups);
    const int64_t c = ((n_comp + per - 1) / per + kStep - 1) / kStep * kStep;
    return min(static_cast<int64_t>(2048), max(static_cast<int64_t>(kStep), c));
  }
  int64_t ch = kStep;
  while (ch < 1024 && (n_comp + 2 * ch - 1) / (2 * ch) * groups >= 768) ch *= 2;
  // few long sequences: no more than 64 partial records per query (the merge
  // reads them with one workgroup per query, and there it, not the chunk
  // kernel, is the longer part) ...
  if (ch == 1024 && (n_comp + ch - 1) / ch > 64) {
    ch = 2048;
    // ... unless 2048-token chunks fill less than one round of the resident
    // workgroups: then the shortest multiple of the step whose chunks fill at
    // most one round, with at most 96 records per query (4-bit long context,
    // 8 groups of 130816 tokens at three per CU: 93 chunks of 1408 tokens,
    // 60.1 -> 56.2 us)
    const int64_t slots = bpc * device_cus();
    if (bpc > 0 && (n_comp + ch - 1) / ch * groups < slots) {
      const int64_t per = min(static_cast<int64_t>(96), max(static_cast<int64_t>(1), slots / groups));
      const int64_t c = ((n_comp + per - 1) / per + kStep - 1) / kStep * kStep;
      ch = min(static_cast<int64_t>(2048), max(static_cast<int64_t>(1024), c));
    }
  }
  return ch;
}

static int attend_bpc(const tq_quantizer* kq, const tq_quantizer* vq) {
  return kq->d == 128 ? attn::attend_blocks_per_cu(key_codebook(kq).bp, vq->cb[1].bp, key_qjl(kq), false) : 0;
}

static int64_t attend_chunks(int64_t n_comp, int64_t groups, int bpc, bool segmented = false) {
  if (n_comp <= 0) return 0;
  const int64_t ch = attend_chunk_len(n_comp, groups, bpc, segmented);
  return (n_comp + ch - 1) / ch;
}

// segments with tokens in a call (the chunking of a segment depends on it)
static int live_segments(const AttendSegment* segs, int nseg) {
  int k = 0;
  for (int i = 0; i < nseg; ++i) k += segs[i].n > 0 ? 1 : 0;
  return k;
}

// Workspace of a cache in segments: the query operands of each segment (its
// key quantizer's, 256-byte aligned, only for segments with tokens), then the
// partial records of all segments' chunks.  For one segment this is the
// layout of tq_attend_decode.
int64_t attend_segments_ws_bytes(const AttendSegment* segs, int nseg, int B, int Hq, int Hkv) {
  const int G = Hq / Hkv;
  const int RT = (G + 3) / 4;
  const int64_t groups = static_cast<int64_t>(B) * Hkv * RT;
  int64_t prep = 0, nrec = 0;
  const bool multi = live_segments(segs, nseg) > 1;
  for (int i = 0; i < nseg; ++i) {
    const int64_t nch = attend_chunks(segs[i].n, groups, attend_bpc(segs[i].kq, segs[i].vq), multi);
    if (nch == 0) continue;
    prep += (scores_ws_bytes(segs[i].kq, B, Hq, Hkv) + 255) / 256 * 256;
    nrec += nch;
  }
  if (nrec == 0)   // only a tail: keep the single-segment size rule
    prep = (scores_ws_bytes(segs[0].kq, B, Hq, Hkv) + 255) / 256 * 256;
  return prep + groups * nrec * 4 * part_stride(segs[0].kq->d) * 4 + 256;
}

int64_t attend_ws_bytes(const tq_quantizer* kq, const tq_quantizer* vq, int B, int Hq, int Hkv, int64_t n_comp, int) {
  const AttendSegment seg = {kq, vq, nullptr, nullptr, nullptr, nullptr, nullptr, n_comp};
  return attend_segments_ws_bytes(&seg, 1, B, Hq, Hkv);
}

// One workgroup (256 threads) per (batch, query head): combine the chunk
// partials (max-shifted), add the exact bf16 tail, rotate back once and
// normalise.  The kernel is a short chain of dependent steps over a few
// hundred kilobytes, so its time is memory latency: every load that does not
// depend on the softmax maximum -- the records' maxima and sums, the first MR
// records of each slice, the first tail key rows and tail values -- is issued
// at the start, and the columns of Pi (read from L2) all at once before the
// rotation back.  Record and tail-value sums are spread over NSL slices of
// D/4 threads (4 consecutive coordinates each); a tail token's logit is taken
// by 4 threads (D/4 coordinates each, joined by row shuffles).  Longer caches
// take further rounds of the same loops.
constexpr int kMergeRec = 12;   // records per slice loaded at the start
template <int D>
__global__ void __launch_bounds__(256) attend_merge_kernel(const void* __restrict__ queries, int q_dtype, int Hq,
                                                           int Hkv, int G, int RT, int64_t nchunk,
                                                           const float* __restrict__ part,
                                                           const uint16_t* __restrict__ k_tail,
                                                           const uint16_t* __restrict__ v_tail, int n_tail,
                                                           float scale_log2, const float* __restrict__ piv,
                                                           float* __restrict__ out) {
  constexpr int d = D;
  constexpr int MR = kMergeRec;
  constexpr int PS = D + 4;                       // record stride
  constexpr int TPS = D / 4;                      // threads per slice
  constexpr int NSL = 256 / TPS;                  // slices
  constexpr int KT = 256 / NSL < 32 ? 256 / NSL : 32;   // tail values per slice loaded at the start
  constexpr int QU = D / 32;                      // 16-byte key pieces per thread (a quarter row)
  constexpr int R0 = D <= 128 ? 4 : 2;            // rounds of 64 tail keys loaded at the start
  constexpr int KP = 256 / D;                     // threads per output coordinate in Pi^T acc
  constexpr int JP = D / KP;                      // inner indices per such thread
  __shared__ __attribute__((aligned(16))) float qv[d];
  __shared__ float accs[d];
  __shared__ __attribute__((aligned(16))) float sl8[NSL][d];
  __shared__ __attribute__((aligned(16))) float tl8[NSL][d];
  __shared__ float pp[KP][d];
  __shared__ float red[8];
  __shared__ float ts[512];   // tail logits, then tail weights (n_tail <= 512)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slc = tid / TPS, u4 = 4 * (tid - slc * TPS);   // slice, first coordinate of this thread's quad
  const bool sact = slc < NSL;                              // thread takes part in the slice sums
  const int kq4 = tid & 3, kt64 = tid >> 2;                 // tail logits: quarter row, token within a round
  const int bh = blockIdx.x;
  const int b = bh / Hq, h = bh - b * Hq;
  const int kvh = h / G, qg = h - kvh * G;
  const int rt = qg >> 2, qi = qg & 3;
  const int64_t gy = (static_cast<int64_t>(b) * Hkv + kvh) * RT + rt;
  const float* pq = part + (gy * nchunk * 4 + qi) * PS;   // chunk c at pq + c * 4 * PS
  const int64_t cstride = 4 * PS;
  const int64_t toff = (static_cast<int64_t>(b) * Hkv + kvh) * n_tail;
  const int64_t clast = nchunk > 0 ? nchunk - 1 : 0;
  const int tlast = n_tail > 0 ? n_tail - 1 : 0;

  // ---------------- loads issued together ----------------
  const float qe = tid < d ? load_elem(queries, q_dtype, static_cast<int64_t>(bh) * d + tid) : 0.f;
  // records' maxima and sums, one per thread (first 256 records)
  const bool rec0 = tid < nchunk;
  const float m0 = rec0 ? pq[static_cast<int64_t>(tid) * cstride + D] : -INFINITY;
  const float l0 = rec0 ? pq[static_cast<int64_t>(tid) * cstride + D + 1] : 0.f;
  // the first MR records of this thread's slice (record c = slc + NSL k)
  float mc[MR];
  float4 pc[MR];
  if (nchunk > 0 && sact) {
#pragma unroll
    for (int k = 0; k < MR; ++k) {
      const int64_t c = min(static_cast<int64_t>(slc + NSL * k), clast);
      mc[k] = pq[c * cstride + D];
      pc[k] = *reinterpret_cast<const float4*>(pq + c * cstride + u4);
    }
  }
  // tail keys: token 64 r + kt64, coordinates D/4 kq4 .. +D/4-1 (R0 rounds of 64 tokens)
  uint4 kr[R0][QU];
  // tail values: token slc + NSL k (k < KT), coordinates u4 .. u4 + 3
  uint2 vr[KT];
  if (n_tail > 0) {
#pragma unroll
    for (int r = 0; r < R0; ++r) {
      const uint4* kt = reinterpret_cast<const uint4*>(k_tail + (toff + min(64 * r + kt64, tlast)) * d + (D / 4) * kq4);
#pragma unroll
      for (int c = 0; c < QU; ++c) kr[r][c] = kt[c];
    }
    if (sact) {
#pragma unroll
      for (int k = 0; k < KT; ++k)
        vr[k] = *reinterpret_cast<const uint2*>(v_tail + (toff + min(slc + NSL * k, tlast)) * d + u4);
    }
  }
  if (tid < d) qv[tid] = qe;
  __syncthreads();

  // ---------------- the softmax maximum ----------------
  float mloc = m0;
  for (int64_t c = tid + 256; c < nchunk; c += 256) mloc = fmaxf(mloc, pq[c * cstride + D]);
  // logit of token 64 r + kt64 from its quarter rows (4 consecutive lanes)
  auto tail_logit = [&](const uint4 (&row)[QU]) {
    float s0 = 0.f, s1 = 0.f;
    const float4* q4 = reinterpret_cast<const float4*>(qv + (D / 4) * kq4);
#pragma unroll
    for (int c = 0; c < QU; ++c) {
      const float4 qa = q4[2 * c], qb = q4[2 * c + 1];
      const float qq[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
      const uint32_t wv[4] = {row[c].x, row[c].y, row[c].z, row[c].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s0 = fmaf(qq[2 * e], __uint_as_float(wv[e] << 16), s0);
        s1 = fmaf(qq[2 * e + 1], __uint_as_float(wv[e] & 0xFFFF0000u), s1);
      }
    }
    float sv = s0 + s1;
    sv += dpp_f<0xB1>(sv);   // quad_perm [1,0,3,2]
    sv += dpp_f<0x4E>(sv);   // quad_perm [2,3,0,1]
    return sv * scale_log2;
  };
  if (n_tail > 0) {
#pragma unroll
    for (int r = 0; r < R0; ++r) {
      const int t = 64 * r + kt64;
      const float sl = tail_logit(kr[r]);
      if (t < n_tail) {
        if (kq4 == 0) ts[t] = sl;
        mloc = fmaxf(mloc, sl);
      }
    }
  }
  for (int t0 = 64 * R0; t0 < n_tail; t0 += 64) {
    const int t = t0 + kt64;
    uint4 row[QU];
    const uint4* kt = reinterpret_cast<const uint4*>(k_tail + (toff + min(t, tlast)) * d + (D / 4) * kq4);
#pragma unroll
    for (int c = 0; c < QU; ++c) row[c] = kt[c];
    const float sl = tail_logit(row);
    if (t < n_tail) {
      if (kq4 == 0) ts[t] = sl;
      mloc = fmaxf(mloc, sl);
    }
  }
  mloc = wave_max(mloc);
  if (lane == 0) red[wave] = mloc;
  __syncthreads();   // the maxima, and every tail logit in ts[]
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  // ---------------- denominators and tail weights ----------------
  float lsum = rec0 ? l0 * exp2f(m0 - M) : 0.f;
  for (int64_t c = tid + 256; c < nchunk; c += 256) lsum = fmaf(pq[c * cstride + D + 1], exp2f(pq[c * cstride + D] - M), lsum);
  for (int t = tid; t < n_tail; t += 256) {
    const float pt = exp2f(ts[t] - M);
    ts[t] = pt;
    lsum += pt;
  }
  lsum = wave_sum(lsum);
  if (lane == 0) red[4 + wave] = lsum;

  // ---------------- records: rotated-frame accumulator ----------------
  if (sact) {
    float4 a = {0.f, 0.f, 0.f, 0.f};
    if (nchunk > 0) {
#pragma unroll
      for (int k = 0; k < MR; ++k) {
        const float wk = slc + NSL * k < nchunk ? exp2f(mc[k] - M) : 0.f;
        a.x = fmaf(pc[k].x, wk, a.x);
        a.y = fmaf(pc[k].y, wk, a.y);
        a.z = fmaf(pc[k].z, wk, a.z);
        a.w = fmaf(pc[k].w, wk, a.w);
      }
    }
    for (int64_t c0 = slc + NSL * MR; c0 < nchunk; c0 += 8 * NSL) {
      float mm[8];
      float4 pr[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t c = min(c0 + NSL * k, clast);
        mm[k] = pq[c * cstride + D];
        pr[k] = *reinterpret_cast<const float4*>(pq + c * cstride + u4);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float wk = c0 + NSL * k < nchunk ? exp2f(mm[k] - M) : 0.f;
        a.x = fmaf(pr[k].x, wk, a.x);
        a.y = fmaf(pr[k].y, wk, a.y);
        a.z = fmaf(pr[k].z, wk, a.z);
        a.w = fmaf(pr[k].w, wk, a.w);
      }
    }
    *reinterpret_cast<float4*>(&sl8[slc][u4]) = a;
  }
  __syncthreads();   // tail weights in ts[], slice sums in sl8
  if (tid < d) {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < NSL; ++k) v += sl8[k][tid];
    accs[tid] = v;
  }
  // ---------------- tail values (original frame) ----------------
  if (sact) {
    float4 a = {0.f, 0.f, 0.f, 0.f};
    auto add = [&](float pt, uint2 raw) {
      a.x = fmaf(pt, __uint_as_float(raw.x << 16), a.x);
      a.y = fmaf(pt, __uint_as_float(raw.x & 0xFFFF0000u), a.y);
      a.z = fmaf(pt, __uint_as_float(raw.y << 16), a.z);
      a.w = fmaf(pt, __uint_as_float(raw.y & 0xFFFF0000u), a.w);
    };
    if (n_tail > 0) {
#pragma unroll
      for (int k = 0; k < KT; ++k) add(slc + NSL * k < n_tail ? ts[min(slc + NSL * k, tlast)] : 0.f, vr[k]);
    }
    for (int t0 = slc + NSL * KT; t0 < n_tail; t0 += 8 * NSL) {
      uint2 raw[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        raw[k] = *reinterpret_cast<const uint2*>(v_tail + (toff + min(t0 + NSL * k, tlast)) * d + u4);
#pragma unroll
      for (int k = 0; k < 8; ++k) add(t0 + NSL * k < n_tail ? ts[min(t0 + NSL * k, tlast)] : 0.f, raw[k]);
    }
    *reinterpret_cast<float4*>(&tl8[slc][u4]) = a;
  }
  __syncthreads();   // accs and the tail slice sums complete
  // ---------------- Pi^T acc (the inner index split over KP threads) ----------------
  if (tid < KP * D) {
    const int i = tid % D, part = tid / D;
    const int j0 = part * JP;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    constexpr int PJ = JP < 64 ? JP : 64;   // columns of Pi loaded together (JP is a multiple of PJ)
    static_assert(JP % PJ == 0, "inner split");
    for (int jj = 0; jj < JP; jj += PJ) {
      float pv[PJ];
#pragma unroll
      for (int k = 0; k < PJ; ++k) pv[k] = piv[static_cast<int64_t>(j0 + jj + k) * d + i];
#pragma unroll
      for (int k = 0; k < PJ; ++k) o[k & 3] = fmaf(pv[k], accs[j0 + jj + k], o[k & 3]);
    }
    pp[part][i] = (o[0] + o[1]) + (o[2] + o[3]);
  }
  __syncthreads();
  if (tid < d) {
    const float L = (red[4] + red[5]) + (red[6] + red[7]);
    float tv = 0.f, ov = 0.f;
#pragma unroll
    for (int k = 0; k < NSL; ++k) tv += tl8[k][tid];
#pragma unroll
    for (int k = 0; k < KP; ++k) ov += pp[k][tid];
    out[static_cast<int64_t>(bh) * d + tid] = (ov + tv) / L;
  }
}

static hipError_t launch_chunks(const AttendSegment& sg, int64_t groups, int G, int RT, float sl, float vtau,
                                const uint8_t* wsA, const float* wsC, float* part, int64_t nrec, int64_t rec0,
                                int64_t nch, bool multi, hipStream_t st) {
  const int64_t ch = attend_chunk_len(sg.n, groups, attend_bpc(sg.kq, sg.vq), multi);
  switch (sg.kq->d) {
    case 64: return attn::launch_chunks_d<64, false>(sg, groups, G, RT, sl, vtau, wsA, wsC, part, nrec, rec0, nch, ch, st);
    case 96: return attn::launch_chunks_d<96, false>(sg, groups, G, RT, sl, vtau, wsA, wsC, part, nrec, rec0, nch, ch, st);
    case 128: return attn::launch_chunks_d<128, true>(sg, groups, G, RT, sl, vtau, wsA, wsC, part, nrec, rec0, nch, ch, st);
    case 256: return attn::launch_chunks_d<256, false>(sg, groups, G, RT, sl, vtau, wsA, wsC, part, nrec, rec0, nch, ch, st);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_attend_segments(const AttendSegment* segs, int nseg, const void* queries, int q_dtype, int B, int Hq,
                                  int Hkv, const uint16_t* k_tail, const uint16_t* v_tail, int n_tail, float scale,
                                  float vtau, float* out, void* ws, hipStream_t st) {
  if (nseg < 1 || n_tail > 512) return hipErrorNotSupported;
  const int d = segs[0].kq->d;
  if (!attend_supports_d(d)) return hipErrorNotSupported;
  for (int i = 0; i < nseg; ++i)
    if (segs[i].kq->d != d || segs[i].vq->d != d) return hipErrorNotSupported;
  const int G = Hq / Hkv;
  const int RT = (G + 3) / 4;
  const int64_t groups = static_cast<int64_t>(B) * Hkv * RT;
  int64_t nrec = 0, prep = 0;
  const bool multi = live_segments(segs, nseg) > 1;
  for (int i = 0; i < nseg; ++i) {
    const int64_t nch = attend_chunks(segs[i].n, groups, attend_bpc(segs[i].kq, segs[i].vq), multi);
    if (nch == 0) continue;
    prep += (scores_ws_bytes(segs[i].kq, B, Hq, Hkv) + 255) / 256 * 256;
    nrec += nch;
  }
  if (nrec == 0) prep = (scores_ws_bytes(segs[0].kq, B, Hq, Hkv) + 255) / 256 * 256;
  float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + prep);
  const float sl = scale * kLog2e;
  hipError_t e;
  // the query operands of every segment with tokens, up to kPrepSetMax per launch
  {
    const tq_quantizer* pq[kPrepSetMax];
    void* pws[kPrepSetMax];
    int np = 0;
    uint8_t* pw = static_cast<uint8_t*>(ws);
    for (int i = 0; i < nseg; ++i) {
      if (attend_chunks(segs[i].n, groups, attend_bpc(segs[i].kq, segs[i].vq), multi) == 0) continue;
      pq[np] = segs[i].kq;
      pws[np] = pw;
      ++np;
      pw += (scores_ws_bytes(segs[i].kq, B, Hq, Hkv) + 255) / 256 * 256;
      if (np == kPrepSetMax) {
        if ((e = launch_query_prep_multi(pq, pws, np, queries, q_dtype, B, Hq, Hkv, st)) != hipSuccess) return e;
        np = 0;
      }
    }
    if (np > 0 && (e = launch_query_prep_multi(pq, pws, np, queries, q_dtype, B, Hq, Hkv, st)) != hipSuccess) return e;
  }
  uint8_t* pw = static_cast<uint8_t*>(ws);
  int64_t rec0 = 0;
  for (int i = 0; i < nseg; ++i) {
    const AttendSegment& sg = segs[i];
    const int64_t nch = attend_chunks(sg.n, groups, attend_bpc(sg.kq, sg.vq), multi);
    if (nch == 0) continue;
    const uint8_t* wsA = pw;
    const float* wsC = reinterpret_cast<const float*>(wsA + groups * key_terms(sg.kq) * ((d + 127) / 128) * 2048);
    e = launch_chunks(sg, groups, G, RT, sl, vtau, wsA, wsC, part, nrec, rec0, nch, multi, st);
    if (e != hipSuccess) return e;
    pw += (scores_ws_bytes(sg.kq, B, Hq, Hkv) + 255) / 256 * 256;
    rec0 += nch;
  }
  // every value quantizer shares Pi (checked by the caller): one rotation back
#define TQ_MERGE(DV)                                                                                             \
  hipLaunchKernelGGL(attend_merge_kernel<DV>, dim3(static_cast<unsigned>(B * Hq)), dim3(256), 0, st, queries, q_dtype, \
                     Hq, Hkv, G, RT, nrec, part, k_tail, v_tail, n_tail, sl, segs[0].vq->d_pi, out)
  switch (d) {
    case 64: TQ_MERGE(64); break;
    case 96: TQ_MERGE(96); break;
    case 128: TQ_MERGE(128); break;
    default: TQ_MERGE(256); break;
  }
#undef TQ_MERGE
  return hipGetLastError();
}

hipError_t launch_attend(const tq_quantizer* kq, const tq_quantizer* vq, const void* queries, int q_dtype, int B, int Hq,
                         int Hkv, const uint32_t* kcodes, const float* knorms, const float* kgammas,
                         const uint32_t* vcodes, const float* vnorms, int64_t n_comp, const uint16_t* k_tail,
                         const uint16_t* v_tail, int n_tail, float scale, float vtau, float* out, void* ws,
                         hipStream_t st) {
  const AttendSegment seg = {kq, vq, kcodes, knorms, kgammas, vcodes, vnorms, n_comp};
  return launch_attend_segments(&seg, 1, queries, q_dtype, B, Hq, Hkv, k_tail, v_tail, n_tail, scale, vtau, out, ws, st);
}

}  // namespace tq
