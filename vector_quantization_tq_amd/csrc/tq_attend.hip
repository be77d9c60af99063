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
// the staging copies are non-temporal (nt): each packed token is read once
// per call (measured 2-3% faster than the default policy)
constexpr int kNtPolicy = 2;
constexpr float kLog2e = 1.4426950408889634f;

// Fixed-point limbs of x in [0, 16): x ~ l0 + l1/16 + l2/256 + l3/4096 with
// every limb a small integer (|l0| <= 16, |l1..3| <= 8), returned in xq.  Byte
// k of the result is limb k divided by sv in {0.5, 1, 2}, the fp4 slot value
// the B operand gives this token, so each product of the value MFMA is l_k
// times a 0/1 bit on one grid for all tokens.  l / sv stays exact in fp8 E4M3
// (4 significant bits: even numbers up to 32, halves up to 8).  The scaled
// conversion divides by its scale operand (checked bit for bit against
// multiplying the limbs by 1 / sv first), which saves those products.  The
// matrix core sums the products of a row in groups of 8, aligned to the
// largest product of the group, so limbs that are integers on one common
// scale keep those group sums exact whatever the spread of the weights
// (per-element floating limbs would lose the small ones).
__device__ __forceinline__ uint32_t fixed_limbs4(float x, float sv, float& xq) {
  const float l0 = rintf(x);
  float r = (x - l0) * 16.f;
  const float l1 = rintf(r);
  r = (r - l1) * 16.f;
  const float l2 = rintf(r);
  r = (r - l2) * 16.f;
  const float l3 = rintf(r);
  xq = l0 + (l1 + (l2 + l3 * (1.f / 16.f)) * (1.f / 16.f)) * (1.f / 16.f);   // exact: 16-bit fixed point
  typedef short v2s __attribute__((ext_vector_type(2)));
  v2s pk = {0, 0};
  pk = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pk, l0, l1, sv, false);   // bytes 0, 1
  pk = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pk, l2, l3, sv, true);    // bytes 2, 3
  return __builtin_bit_cast(uint32_t, pk);
}

}  // namespace

// partial record of one (group row tile, chunk, query): acc[128] then m, l
constexpr int kPartStride = 128 + 4;

// Residency of the chunk kernel (workgroups per CU it is built for; 0: the
// compiler's choice with a 3-step staging ring, 2 or 3 per CU by its VGPRs
// and LDS).  With a 2-step ring and at most 128 VGPRs four workgroups share
// a CU (4 waves per SIMD): the extra waves hide each other's ALU phases
// better than the deeper ring hides memory latency (GQA layer, 3-bit: 78 ->
// 72 us).  That budget holds the query terms and the value accumulators
// without spilling where the key's MSE bits and the value bits are at most 3
// each and the key and value bits sum to at most 6.  4-bit prod keys with
// 4-bit values need 190 VGPRs and 58 KB of LDS with the 3-step ring (two per
// CU); with the 2-step ring they fit 168 VGPRs, three per CU.  The sparse-V
// kernels keep the compiler's choice.
constexpr int attend_blocks_per_cu(int bpk, int bpv, bool qjl, bool sparse) {
  return sparse ? 0
         : (bpk <= 3 && bpv <= 3 && bpk + (qjl ? 1 : 0) + bpv <= 6) ? 4
         : (qjl && bpk == 3 && bpv == 4) ? 3
                                         : 0;
}

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
  return attend_blocks_per_cu(key_codebook(kq).bp, vq->cb[1].bp, key_qjl(kq), false);
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
  return prep + groups * nrec * 4 * kPartStride * 4 + 256;
}

int64_t attend_ws_bytes(const tq_quantizer* kq, const tq_quantizer* vq, int B, int Hq, int Hkv, int64_t n_comp, int) {
  const AttendSegment seg = {kq, vq, nullptr, nullptr, nullptr, nullptr, nullptr, n_comp};
  return attend_segments_ws_bytes(&seg, 1, B, Hq, Hkv);
}

// Copy `words` 32-bit words (a multiple of 4) from src to LDS dst by 16-byte
// DMA loads (global -> LDS, no registers), spread over the 4 waves; words at
// or past `limit` (a multiple of 4, > 0) re-read the last valid 16 bytes.
// `wave` is wave-uniform; offsets are 32-bit bytes from the uniform source,
// so each copy addresses as scalar base + vector offset.
__device__ __forceinline__ void dma16(uint32_t* dst, const uint32_t* src, int words, int limit, int wave, int lane) {
  const char* s8 = reinterpret_cast<const char*>(src);
  for (int i = wave; i * 256 < words; i += 4) {
    uint32_t off = static_cast<uint32_t>(i * 256) + 4u * static_cast<uint32_t>(lane);
    if (off + 4u > static_cast<uint32_t>(limit)) off = static_cast<uint32_t>(limit) - 4u;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(s8 + 4u * off), as_lds(dst + i * 256), 16, 0,
                                     kNtPolicy);
  }
}
// 64 floats of a per-token array, one per lane, index clamped to [0, n-1]
// (t0 >= 0, n >= 1)
__device__ __forceinline__ void dma_tok(float* dst, const float* src, int64_t t0, int64_t n, int lane) {
  const int64_t tb = min(t0, n - 1);                                    // uniform
  const uint32_t l = static_cast<uint32_t>(min(static_cast<int64_t>(lane), n - 1 - tb));
  const char* s8 = reinterpret_cast<const char*>(src + tb);
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const float*>(s8 + 4u * l), as_lds(dst), 4, 0, kNtPolicy);
}

// QJL: prod keys (QJL plane + gammas); without it MSE-only keys.  SPARSE:
// the sparse-V threshold vtau is applied (a separate instantiation, so that
// the dense kernel carries none of its cost).
template <int BPK, int BPV, int NSLOT, bool QJL, bool SPARSE>
__device__ __forceinline__ void attend_chunk_body(
    const uint32_t* __restrict__ kcodes, const float* __restrict__ knorms, const float* __restrict__ kgammas,
    const uint32_t* __restrict__ vcodes, const float* __restrict__ vnorms, int64_t n, int64_t chunk, int G, int RT,
    float scale_log2, float vtau, const uint8_t* __restrict__ wsA, const float* __restrict__ wsC, const Codebook& vcb,
    float* __restrict__ part, int64_t nrec, int64_t rec0) {
  constexpr int d = 128;
  constexpr int TK = (1 << (BPK - 1)) + (QJL ? 1 : 0);   // key MFMA terms (Walsh + QJL)
  constexpr int WK = BPK + (QJL ? 1 : 0);                // key words per 32-coordinate group
  constexpr int WPK = 4 * WK;                // key words per token
  constexpr int NV = 1 << (BPV - 1);         // value Walsh terms
  constexpr int KW = kStep * WPK;            // key words of a step
  constexpr int VW = 4 * BPV * d;            // value words of a step (4 blocks of 32 tokens)
  constexpr int SLOT = KW + VW + 3 * kStep;  // + key norms, key gammas, value norms
  static_assert(NSLOT == 2 || NSLOT == 3, "staging ring of 2 or 3 steps");
  __shared__ __attribute__((aligned(16))) uint32_t stage[NSLOT][SLOT];
  __shared__ float sc[4][kStep];             // scaled logits (base 2)
  __shared__ __attribute__((aligned(16))) uint32_t av[64 * 8];   // value A operand (fp8 limbs)
  __shared__ float qst[4][4];                // per query: rescale factor, E, value work left in the step

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gy = blockIdx.y;
  const int grp = gy / RT;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t c1 = min(n, c0 + chunk);
  const int qi = lane >> 4, j = lane & 15, g = lane >> 4;

  const uint32_t* kb = kcodes + static_cast<int64_t>(grp) * n * WPK;
  const float* knb = knorms + static_cast<int64_t>(grp) * n;
  const float* kgb = QJL ? kgammas + static_cast<int64_t>(grp) * n : nullptr;
  const int64_t nbk = (n + 31) >> 5;
  const uint32_t* vb = vcodes + static_cast<int64_t>(grp) * nbk * BPV * d;
  const float* vnb = vnorms + static_cast<int64_t>(grp) * n;

  // stage the packed keys, values and per-token norms of the step at t0
  auto issue = [&](int64_t t0, int buf) {
    uint32_t* sl = stage[buf];
    const int kv = static_cast<int>(min(static_cast<int64_t>(kStep), n - t0)) * WPK;
    dma16(sl, kb + t0 * WPK, KW, kv, wave, lane);
    const int64_t b0 = t0 >> 5;
    const int vv = static_cast<int>(min(static_cast<int64_t>(4), nbk - b0)) * BPV * d;
    dma16(sl + KW, vb + b0 * BPV * d, VW, vv, wave, lane);
    float* nz = reinterpret_cast<float*>(sl + KW + VW);
    if (wave < 2) {
      dma_tok(nz + 64 * wave, knb, t0 + 64 * wave, n, lane);
      if constexpr (QJL) dma_tok(nz + kStep + 64 * wave, kgb, t0 + 64 * wave, n, lane);
    } else {
      dma_tok(nz + 2 * kStep + 64 * (wave - 2), vnb, t0 + 64 * (wave - 2), n, lane);
    }
  };

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

  // running softmax state of query `wave` (softmax phase), uniform over that wave
  // m_run: running max logit; wmax: largest weight p n so far (relative to
  // m_run), which sets the limb exponent e_run; the sums of p and of the
  // quantised weights stay per lane and are reduced once at the end
  float m_run = -INFINITY, wmax = 0.f, l_lane = 0.f, w_lane = 0.f;
  int e_run = 0;
  // value accumulators: [Walsh term][column tile of this wave]; rows 4q+limb, column 16ct+j
  v4f acc[NV][2];
#pragma unroll
  for (int t = 0; t < NV; ++t) acc[t][0] = acc[t][1] = (v4f){0.f, 0.f, 0.f, 0.f};
  int e_acc = 0;   // scale exponent the accumulators are in (per query, same in every wave)

  // DMA instructions this wave issues per step (the same for every step)
  constexpr int KI = KW / 256, VI = VW / 256;
  const int per_step = (KI + 3 - wave) / 4 + (VI + 3 - wave) / 4 + (wave < 2 ? (QJL ? 2 : 1) : 1);
  // softmax tokens of this lane: tA and tB = tA + 4, whose value-MFMA A bytes
  // are adjacent (K and K + 1 in the same fp4 slot), so each limb of the pair
  // is one 16-bit LDS write.  token = 32(K/32) + 4(K%8) + (K%32)/8.
  const int tA = 8 * (lane >> 2) + (lane & 3), tB = tA + 4;
  int a_off;       // byte offset of tA's limb 0 in the A tile, minus 32 * 4q
  float a_sv;
  {
    const int hh = tA >> 5, rem = tA & 31;
    const int K = 32 * hh + 8 * (rem & 3) + (rem >> 2);
    const int gg = (K & 63) >> 4, e = 16 * (K >> 6) + (K & 15);
    a_off = 16 * gg * 32 + e;
    a_sv = fp4_slot_value((K & 31) >> 3);   // 0.5, 1 or 2
  }
  // prefetch depth NSLOT - 1: steps s+1 .. s+NSLOT-1 are in flight while step s is used
  constexpr int P = NSLOT - 1;
#pragma unroll
  for (int k = 0; k < P; ++k)
    if (c0 + k * kStep < c1) issue(c0 + k * kStep, k);
  int buf = 0;
  for (int64_t t0 = c0; t0 < c1; t0 += kStep, buf = buf == NSLOT - 1 ? 0 : buf + 1) {
    // this wave's part of step t0 has landed once at most the loads of the
    // later steps already issued are outstanding (the counter retires in
    // issue order) ...
    {
      const int64_t later = (c1 - t0 - 1) / kStep;   // steps after t0 in this chunk
      const int ahead = static_cast<int>(min(static_cast<int64_t>(P - 1), later));
      wait_vm_upto<8>(ahead * per_step);
    }
    __syncthreads();   // ... and every wave's; the slot of step t0 - kStep is free again
    if (t0 + P * kStep < c1) issue(t0 + P * kStep, buf == 0 ? NSLOT - 1 : buf - 1);
    const uint32_t* sl = stage[buf];
    const float* kns = reinterpret_cast<const float*>(sl + KW + VW);
    const int live = static_cast<int>(min(static_cast<int64_t>(kStep), c1 - t0));   // tokens of the step in the chunk
    // ---------------- K phase: logits of tokens t0 + 32*wave .. +31 ----------------
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tt = 32 * wave + 16 * u + j;   // token within the step
      uint32_t w[5] = {0u, 0u, 0u, 0u, 0u};
#pragma unroll
      for (int p = 0; p < WK; ++p) w[p] = sl[(tt * 4 + g) * WK + p];
      v4f aM = {0.f, 0.f, 0.f, 0.f}, aQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < (1 << (BPK - 1)); ++t) aM = mfma_fp8_fp4(AK[t], bits_to_fp4(walsh_word<BPK>(w, t)), aM);
      if constexpr (QJL) aQ = mfma_fp8_fp4(AK[TK - 1], bits_to_fp4(w[BPK]), aQ);
      pin(aM);
      const float mse = fmaf(aM[0], cs[2], fmaf(aM[1], cs[3], fmaf(aM[2], cs[4], fmaf(aM[3], cs[5], cs[0]))));
      float logit = kns[tt] * mse;
      if constexpr (QJL) {
        pin(aQ);
        const float qjl = fmaf(aQ[0], cs[6], fmaf(aQ[1], cs[7], fmaf(aQ[2], cs[8], fmaf(aQ[3], cs[9], cs[1]))));
        logit = fmaf(kns[tt], mse, kns[kStep + tt] * qjl);
      }
      float s = -INFINITY;
      if (tt < live) s = logit * scale_log2;
      sc[qi][tt] = s;
    }
    __syncthreads();
    // ---------------- softmax phase: wave q handles query q ----------------
    {
      const int q = wave;
      const float sa = sc[q][tA], sb = sc[q][tB];
      // the max is reduced over the wave only when some logit exceeds it
      float m_new = m_run;
      if (__ballot(sa > m_run || sb > m_run) != 0ull) m_new = fmaxf(m_run, wave_max(fmaxf(sa, sb)));
      const float alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first step
      const float pa = __builtin_amdgcn_exp2f(sa - m_new), pb = __builtin_amdgcn_exp2f(sb - m_new);
      const float* vns = kns + 2 * kStep;
      // past the chunk's end p is exactly 0 (logit -inf) and the staged norm a
      // finite re-read, so the weight is 0 without a mask
      const float na = vns[tA];
      const float nb2 = vns[tB];
      float wa = pa * na, wb = pb * nb2;
      l_lane = fmaf(l_lane, alpha, pa + pb);
      m_run = m_new;
      // the limb exponent follows the running max weight, so the accumulator
      // rescale alpha 2^(e_new - e_run) stays bounded (about 2 at most) and is
      // exactly 1 in steps that set no new maximum
      wmax *= alpha;
      if (__ballot(wa > wmax || wb > wmax) != 0ull) wmax = fmaxf(wmax, wave_max(fmaxf(wa, wb)));
      // the weights are quantised on the grid 2^(-12 - e): wmax 2^e lands in [8, 16)
      const int e_new = wmax > 0.f ? 3 - ilogb_pos(wmax) : e_run;
      // sparse V: a token whose weight is below vtau times the largest weight
      // of the chunk so far leaves the value sum (its p stays in the
      // normaliser); a step with no weight left skips the value MFMAs
      if constexpr (SPARSE) {
        const float thr = vtau * wmax;
        wa = wa < thr ? 0.f : wa;
        wb = wb < thr ? 0.f : wb;
        const bool vwork = __ballot(wa > 0.f || wb > 0.f) != 0ull;
        if (lane == 0) qst[q][2] = vwork ? 1.f : 0.f;
      }
      if (lane == 0) {
        qst[q][0] = ldexpf(alpha, e_new - e_run);   // accumulator rescale for this query
        qst[q][1] = static_cast<float>(e_new);
      }
      e_run = e_new;
      // A operand of the value MFMA: rows 4q + limb, K = token slot.  The
      // weight sum that enters the Walsh constant term is taken over the
      // quantised weights, so that sum_t w_t (2 b_t - 1) is exact for them.
      float qa, qb;
      const uint32_t la = fixed_limbs4(ldexpf(wa, e_new), a_sv, qa);
      const uint32_t lb = fixed_limbs4(ldexpf(wb, e_new), a_sv, qb);
      w_lane = fmaf(w_lane, alpha, ldexpf(qa + qb, -e_new));
      // limb k of tokens tA and tB are adjacent bytes: one 16-bit write per limb
      const uint32_t p01 = __builtin_amdgcn_perm(lb, la, 0x05010400u);   // la0 lb0 la1 lb1
      const uint32_t p23 = __builtin_amdgcn_perm(lb, la, 0x07030602u);   // la2 lb2 la3 lb3
      uint16_t* avh = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(av) + 4 * q * 32 + a_off);
      avh[0] = static_cast<uint16_t>(p01);
      avh[16] = static_cast<uint16_t>(p01 >> 16);
      avh[32] = static_cast<uint16_t>(p23);
      avh[48] = static_cast<uint16_t>(p23 >> 16);
    }
    __syncthreads();
    // ---------------- V phase: wave owns coordinates 32*wave .. +31 ----------------
    {
      const v8i A = *reinterpret_cast<const v8i*>(av + lane * 8);
      const float rs = qst[qi][0];
      e_acc = static_cast<int>(qst[qi][1]);
      if (__ballot(rs != 1.f) != 0ull) {
#pragma unroll
        for (int t = 0; t < NV; ++t) {
          acc[t][0] *= rs;
          acc[t][1] *= rs;
        }
      }
      // lane group g reads the 32-token block g of the step; blocks past the
      // end hold re-read words, which meet zero weights
      bool vwork = true;
      if constexpr (SPARSE) vwork = qst[0][2] != 0.f || qst[1][2] != 0.f || qst[2][2] != 0.f || qst[3][2] != 0.f;
#pragma unroll
      for (int ct = 0; ct < 2 && vwork; ++ct) {
        const int col = 32 * wave + 16 * ct + j;
        uint32_t w[5] = {0u, 0u, 0u, 0u, 0u};
#pragma unroll
        for (int p = 0; p < BPV; ++p) w[p] = sl[KW + (g * BPV + p) * d + col];
#pragma unroll
        for (int t = 0; t < NV; ++t) acc[t][ct] = mfma_fp8_fp4(A, bits_to_fp4(walsh_word<BPV>(w, t)), acc[t][ct]);
      }
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        pin(acc[t][0]);
        pin(acc[t][1]);
      }
    }
  }

  // ---------------- chunk result ----------------
  // value part: sum_t w_t c[idx] = sum_S coef_S (2 sum_t w_t b_S - sum_t w_t);
  // the softmax state of query q lives in wave q: publish it
  __syncthreads();
  {
    const float w_run = wave_sum(w_lane), l_run = wave_sum(l_lane);
    if (lane == 0) {
      qst[wave][2] = w_run;
      qst[wave][3] = l_run;
      qst[wave][0] = m_run;
    }
  }
  __syncthreads();
  const float wq = qst[qi][2];
  // record rec0 + chunk of the nrec records of this row tile (a cache kept in
  // several segments writes each segment's chunks to its own range)
  float* pbase = part + ((static_cast<int64_t>(gy) * nrec + rec0 + blockIdx.x) * 4) * kPartStride;
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

template <int BPK, int BPV, bool QJL, bool SPARSE>
struct AttendResidency {
  static constexpr int kBlocks = attend_blocks_per_cu(BPK, BPV, QJL, SPARSE);
  static constexpr int kSlots = kBlocks > 0 ? 2 : 3;
  static constexpr int kBlocksPerCu = kBlocks > 0 ? kBlocks : 1;
};

template <int BPK, int BPV, bool QJL, bool SPARSE>
__global__ void __launch_bounds__(256, (AttendResidency<BPK, BPV, QJL, SPARSE>::kBlocksPerCu)) attend_chunk_kernel(
    const uint32_t* __restrict__ kcodes, const float* __restrict__ knorms, const float* __restrict__ kgammas,
    const uint32_t* __restrict__ vcodes, const float* __restrict__ vnorms, int64_t n, int64_t chunk, int G, int RT,
    float scale_log2, float vtau, const uint8_t* __restrict__ wsA, const float* __restrict__ wsC, Codebook vcb,
    float* __restrict__ part, int64_t nrec, int64_t rec0) {
  attend_chunk_body<BPK, BPV, AttendResidency<BPK, BPV, QJL, SPARSE>::kSlots, QJL, SPARSE>(kcodes, knorms, kgammas, vcodes, vnorms, n, chunk, G, RT, scale_log2, vtau,
                                              wsA, wsC, vcb, part, nrec, rec0);
}

// One workgroup (256 threads) per (batch, query head): combine the chunk
// partials (max-shifted), add the exact bf16 tail, rotate back once and
// normalise.  The kernel is a short chain of dependent steps over a few
// hundred kilobytes, so its time is memory latency: every load that does not
// depend on the softmax maximum -- the records' maxima and sums, the first MR
// records of each slice, the first 256 tail key rows and the first 256 tail
// values -- is issued at the start, and the half columns of Pi (read from L2)
// all at once before the rotation back.  Record sums are spread over 8
// slices of 32 threads (4 consecutive coordinates each, 16-byte loads); a
// tail token's logit is taken by 4 threads (32 coordinates each, joined by
// row shuffles) and its value by the 32 threads of its slice.  Longer caches
// take further rounds of the same loops.
constexpr int kMergeRec = 12;   // records per slice loaded at the start (96 records)
__global__ void __launch_bounds__(256) attend_merge_kernel(const void* __restrict__ queries, int q_dtype, int Hq,
                                                           int Hkv, int G, int RT, int64_t nchunk,
                                                           const float* __restrict__ part,
                                                           const uint16_t* __restrict__ k_tail,
                                                           const uint16_t* __restrict__ v_tail, int n_tail,
                                                           float scale_log2, const float* __restrict__ piv,
                                                           float* __restrict__ out) {
  constexpr int d = 128;
  constexpr int MR = kMergeRec;
  __shared__ __attribute__((aligned(16))) float qv[d];
  __shared__ float accs[d];
  __shared__ __attribute__((aligned(16))) float sl8[8][d];
  __shared__ __attribute__((aligned(16))) float tl8[8][d];
  __shared__ float half2[2][d];
  __shared__ float red[8];
  __shared__ float ts[512];   // tail logits, then tail weights (n_tail <= 512)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = tid & (d - 1), hf = tid >> 7;
  const int slc = tid >> 5, u4 = 4 * (tid & 31);   // slice, first coordinate of this thread's quad
  const int kq4 = tid & 3, kt64 = tid >> 2;          // tail logits: quarter row, token within a round of 64
  const int bh = blockIdx.x;
  const int b = bh / Hq, h = bh - b * Hq;
  const int kvh = h / G, qg = h - kvh * G;
  const int rt = qg >> 2, qi = qg & 3;
  const int64_t gy = (static_cast<int64_t>(b) * Hkv + kvh) * RT + rt;
  const float* pq = part + (gy * nchunk * 4 + qi) * kPartStride;   // chunk c at pq + c * 4 * kPartStride
  const int64_t cstride = 4 * kPartStride;
  const int64_t toff = (static_cast<int64_t>(b) * Hkv + kvh) * n_tail;
  const int64_t clast = nchunk > 0 ? nchunk - 1 : 0;
  const int tlast = n_tail > 0 ? n_tail - 1 : 0;

  // ---------------- loads issued together ----------------
  const float qe = tid < d ? load_elem(queries, q_dtype, static_cast<int64_t>(bh) * d + tid) : 0.f;
  // records' maxima and sums, one per thread (first 256 records)
  const bool rec0 = tid < nchunk;
  const float m0 = rec0 ? pq[static_cast<int64_t>(tid) * cstride + 128] : -INFINITY;
  const float l0 = rec0 ? pq[static_cast<int64_t>(tid) * cstride + 129] : 0.f;
  // the first MR records of this thread's slice (record c = slc + 8 k)
  float mc[MR];
  float4 pc[MR];
  if (nchunk > 0) {
#pragma unroll
    for (int k = 0; k < MR; ++k) {
      const int64_t c = min(static_cast<int64_t>(slc + 8 * k), clast);
      mc[k] = pq[c * cstride + 128];
      pc[k] = *reinterpret_cast<const float4*>(pq + c * cstride + u4);
    }
  }
  // tail keys: token 64 r + kt64, coordinates 32 kq4 .. +31 (4 rounds of 64 tokens)
  uint4 kr[4][4];
  // tail values: token slc + 8 k (k < 32), coordinates u4 .. u4 + 3
  uint2 vr[32];
  if (n_tail > 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint4* kt = reinterpret_cast<const uint4*>(k_tail + (toff + min(64 * r + kt64, tlast)) * d + 32 * kq4);
#pragma unroll
      for (int c = 0; c < 4; ++c) kr[r][c] = kt[c];
    }
#pragma unroll
    for (int k = 0; k < 32; ++k)
      vr[k] = *reinterpret_cast<const uint2*>(v_tail + (toff + min(slc + 8 * k, tlast)) * d + u4);
  }
  if (tid < d) qv[tid] = qe;
  __syncthreads();

  // ---------------- the softmax maximum ----------------
  float mloc = m0;
  for (int64_t c = tid + 256; c < nchunk; c += 256) mloc = fmaxf(mloc, pq[c * cstride + 128]);
  // logit of token 64 r + kt64 from its quarter rows (4 consecutive lanes)
  auto tail_logit = [&](const uint4 (&row)[4]) {
    float s0 = 0.f, s1 = 0.f;
    const float4* q4 = reinterpret_cast<const float4*>(qv + 32 * kq4);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
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
    for (int r = 0; r < 4; ++r) {
      const int t = 64 * r + kt64;
      const float sl = tail_logit(kr[r]);
      if (t < n_tail) {
        if (kq4 == 0) ts[t] = sl;
        mloc = fmaxf(mloc, sl);
      }
    }
  }
  for (int t0 = 256; t0 < n_tail; t0 += 64) {
    const int t = t0 + kt64;
    uint4 row[4];
    const uint4* kt = reinterpret_cast<const uint4*>(k_tail + (toff + min(t, tlast)) * d + 32 * kq4);
#pragma unroll
    for (int c = 0; c < 4; ++c) row[c] = kt[c];
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
  for (int64_t c = tid + 256; c < nchunk; c += 256) lsum = fmaf(pq[c * cstride + 129], exp2f(pq[c * cstride + 128] - M), lsum);
  for (int t = tid; t < n_tail; t += 256) {
    const float pt = exp2f(ts[t] - M);
    ts[t] = pt;
    lsum += pt;
  }
  lsum = wave_sum(lsum);
  if (lane == 0) red[4 + wave] = lsum;

  // ---------------- records: rotated-frame accumulator ----------------
  {
    float4 a = {0.f, 0.f, 0.f, 0.f};
    if (nchunk > 0) {
#pragma unroll
      for (int k = 0; k < MR; ++k) {
        const float wk = slc + 8 * k < nchunk ? exp2f(mc[k] - M) : 0.f;
        a.x = fmaf(pc[k].x, wk, a.x);
        a.y = fmaf(pc[k].y, wk, a.y);
        a.z = fmaf(pc[k].z, wk, a.z);
        a.w = fmaf(pc[k].w, wk, a.w);
      }
    }
    for (int64_t c0 = slc + 8 * MR; c0 < nchunk; c0 += 64) {
      float mm[8];
      float4 pp[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t c = min(c0 + 8 * k, clast);
        mm[k] = pq[c * cstride + 128];
        pp[k] = *reinterpret_cast<const float4*>(pq + c * cstride + u4);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float wk = c0 + 8 * k < nchunk ? exp2f(mm[k] - M) : 0.f;
        a.x = fmaf(pp[k].x, wk, a.x);
        a.y = fmaf(pp[k].y, wk, a.y);
        a.z = fmaf(pp[k].z, wk, a.z);
        a.w = fmaf(pp[k].w, wk, a.w);
      }
    }
    *reinterpret_cast<float4*>(&sl8[slc][u4]) = a;
  }
  __syncthreads();   // tail weights in ts[], slice sums in sl8
  if (tid < d) {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) v += sl8[k][i];
    accs[i] = v;
  }
  // ---------------- tail values (original frame) ----------------
  {
    float4 a = {0.f, 0.f, 0.f, 0.f};
    auto add = [&](float pt, uint2 raw) {
      a.x = fmaf(pt, __uint_as_float(raw.x << 16), a.x);
      a.y = fmaf(pt, __uint_as_float(raw.x & 0xFFFF0000u), a.y);
      a.z = fmaf(pt, __uint_as_float(raw.y << 16), a.z);
      a.w = fmaf(pt, __uint_as_float(raw.y & 0xFFFF0000u), a.w);
    };
    if (n_tail > 0) {
#pragma unroll
      for (int k = 0; k < 32; ++k) add(slc + 8 * k < n_tail ? ts[min(slc + 8 * k, tlast)] : 0.f, vr[k]);
    }
    for (int t0 = slc + 256; t0 < n_tail; t0 += 64) {
      uint2 raw[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        raw[k] = *reinterpret_cast<const uint2*>(v_tail + (toff + min(t0 + 8 * k, tlast)) * d + u4);
#pragma unroll
      for (int k = 0; k < 8; ++k) add(t0 + 8 * k < n_tail ? ts[min(t0 + 8 * k, tlast)] : 0.f, raw[k]);
    }
    *reinterpret_cast<float4*>(&tl8[slc][u4]) = a;
  }
  __syncthreads();   // accs and the tail slice sums complete
  // ---------------- Pi^T acc (inner index split between the two halves) ----------------
  {
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    const int j0 = hf * (d / 2);
    float pv[d / 2];
#pragma unroll
    for (int k = 0; k < d / 2; ++k) pv[k] = piv[static_cast<int64_t>(j0 + k) * d + i];
#pragma unroll
    for (int k = 0; k < d / 2; ++k) o[k & 3] = fmaf(pv[k], accs[j0 + k], o[k & 3]);
    half2[hf][i] = (o[0] + o[1]) + (o[2] + o[3]);
  }
  __syncthreads();
  if (tid < d) {
    const float L = (red[4] + red[5]) + (red[6] + red[7]);
    float tv = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) tv += tl8[k][i];
    out[static_cast<int64_t>(bh) * d + i] = (half2[0][i] + half2[1][i] + tv) / L;
  }
}

static hipError_t launch_chunks(const AttendSegment& sg, int64_t groups, int G, int RT, float sl, float vtau,
                                const uint8_t* wsA, const float* wsC, float* part, int64_t nrec, int64_t rec0,
                                int64_t nch, bool multi, hipStream_t st) {
  const int bpc = attend_bpc(sg.kq, sg.vq);
  const int64_t ch = attend_chunk_len(sg.n, groups, bpc, multi);
  dim3 grid(static_cast<unsigned>(nch), static_cast<unsigned>(groups));
  const int bpk = key_codebook(sg.kq).bp, bpv = sg.vq->cb[1].bp;
  const bool qjl = key_qjl(sg.kq);
#define TQ_AT(K, V, QV)                                                                                       \
  if (bpk == K && bpv == V && qjl == QV) {                                                                    \
    if (vtau > 0.f)                                                                                           \
      hipLaunchKernelGGL((attend_chunk_kernel<K, V, QV, true>), grid, dim3(256), 0, st, sg.kcodes, sg.knorms,  \
                         sg.kgammas, sg.vcodes, sg.vnorms, sg.n, ch, G, RT, sl, vtau, wsA, wsC, sg.vq->cb[1],  \
                         part, nrec, rec0);                                                                   \
    else                                                                                                      \
      hipLaunchKernelGGL((attend_chunk_kernel<K, V, QV, false>), grid, dim3(256), 0, st, sg.kcodes, sg.knorms, \
                         sg.kgammas, sg.vcodes, sg.vnorms, sg.n, ch, G, RT, sl, 0.f, wsA, wsC, sg.vq->cb[1],   \
                         part, nrec, rec0);                                                                   \
  } else
#define TQ_AT4(K, QV) TQ_AT(K, 1, QV) TQ_AT(K, 2, QV) TQ_AT(K, 3, QV) TQ_AT(K, 4, QV)
  TQ_AT4(1, true) TQ_AT4(2, true) TQ_AT4(3, true)
  TQ_AT4(1, false) TQ_AT4(2, false) TQ_AT4(3, false) TQ_AT4(4, false) { return hipErrorNotSupported; }
#undef TQ_AT4
#undef TQ_AT
  return hipGetLastError();
}

hipError_t launch_attend_segments(const AttendSegment* segs, int nseg, const void* queries, int q_dtype, int B, int Hq,
                                  int Hkv, const uint16_t* k_tail, const uint16_t* v_tail, int n_tail, float scale,
                                  float vtau, float* out, void* ws, hipStream_t st) {
  if (nseg < 1 || n_tail > 512) return hipErrorNotSupported;
  for (int i = 0; i < nseg; ++i)
    if (segs[i].kq->d != 128 || segs[i].vq->d != 128) return hipErrorNotSupported;
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
    const float* wsC = reinterpret_cast<const float*>(wsA + groups * key_terms(sg.kq) * 2048);
    e = launch_chunks(sg, groups, G, RT, sl, vtau, wsA, wsC, part, nrec, rec0, nch, multi, st);
    if (e != hipSuccess) return e;
    pw += (scores_ws_bytes(sg.kq, B, Hq, Hkv) + 255) / 256 * 256;
    rec0 += nch;
  }
  // every value quantizer shares Pi (checked by the caller): one rotation back
  hipLaunchKernelGGL(attend_merge_kernel, dim3(static_cast<unsigned>(B * Hq)), dim3(256), 0, st, queries, q_dtype, Hq, Hkv,
                     G, RT, nrec, part, k_tail, v_tail, n_tail, sl, segs[0].vq->d_pi, out);
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
