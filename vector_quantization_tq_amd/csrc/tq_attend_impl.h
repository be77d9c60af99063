// Decode-attention chunk kernel (internal to libtq): the template over the
// head dimension D, the key and value widths and the sparse-V switch.  Every
// D has its own source file that instantiates launch_chunks_d<D>, so that the
// widths compile in parallel.  What the kernel computes is described in
// tq_attend.hip.
#pragma once

#include "tq_device.h"
#include "tq_kernels.h"

namespace tq {
namespace attn {

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
// As dma16 with 4-byte copies (words need not come in 16-byte runs): 64
// words per instruction; words at or past `limit` (> 0) re-read the last
// valid word.
__device__ __forceinline__ void dma4(uint32_t* dst, const uint32_t* src, int words, int limit, int wave, int lane) {
  const char* s8 = reinterpret_cast<const char*>(src);
  for (int i = wave; i * 64 < words; i += 4) {
    uint32_t off = static_cast<uint32_t>(i * 64) + static_cast<uint32_t>(lane);
    if (off + 1u > static_cast<uint32_t>(limit)) off = static_cast<uint32_t>(limit) - 1u;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(s8 + 4u * off), as_lds(dst + i * 64), 4, 0,
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
template <int D, int BPK, int BPV, int NSLOT, bool QJL, bool SPARSE>
__device__ __forceinline__ void attend_chunk_body(
    const uint32_t* __restrict__ kcodes, const float* __restrict__ knorms, const float* __restrict__ kgammas,
    const uint32_t* __restrict__ vcodes, const float* __restrict__ vnorms, int64_t n, int64_t chunk, int G, int RT,
    float scale_log2, float vtau, const uint8_t* __restrict__ wsA, const float* __restrict__ wsC, const Codebook& vcb,
    float* __restrict__ part, int64_t nrec, int64_t rec0) {
  static_assert(D % 32 == 0 && D >= 32 && D <= 256, "head dimension: a multiple of 32 up to 256");
  constexpr int d = D;
  constexpr int NG = D / 32;                 // 32-coordinate groups
  constexpr int KC = (NG + 3) / 4;           // 128-coordinate MFMA chunks of a key
  constexpr int NT16 = D / 16;               // 16-coordinate value tiles
  constexpr int CTW = (NT16 + 3) / 4;        // value tiles per wave (waves own consecutive tiles)
  constexpr int PS = D + 4;                  // partial record stride: acc[D], m, l
  constexpr int TK = (1 << (BPK - 1)) + (QJL ? 1 : 0);   // key MFMA terms (Walsh + QJL)
  constexpr int WK = BPK + (QJL ? 1 : 0);                // key words per 32-coordinate group
  constexpr int WPK = NG * WK;               // key words per token
  constexpr int NV = 1 << (BPV - 1);         // value Walsh terms
  constexpr bool K16 = WPK % 4 == 0;         // key runs are 16-byte aligned: 16-byte copies
  constexpr int KW = kStep * WPK;            // key words of a step
  constexpr int KWP = (KW + (K16 ? 255 : 63)) / (K16 ? 256 : 64) * (K16 ? 256 : 64);   // whole copy rounds
  constexpr int VW = 4 * BPV * d;            // value words of a step (4 blocks of 32 tokens)
  constexpr int VWP = (VW + 255) / 256 * 256;
  constexpr int SLOT = KWP + VWP + 3 * kStep;   // + key norms, key gammas, value norms
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
    if constexpr (K16) dma16(sl, kb + t0 * WPK, KW, kv, wave, lane);
    else dma4(sl, kb + t0 * WPK, KW, kv, wave, lane);
    const int64_t b0 = t0 >> 5;
    const int vv = static_cast<int>(min(static_cast<int64_t>(4), nbk - b0)) * BPV * d;
    dma16(sl + KWP, vb + b0 * BPV * d, VW, vv, wave, lane);
    float* nz = reinterpret_cast<float*>(sl + KWP + VWP);
    if (wave < 2) {
      dma_tok(nz + 64 * wave, knb, t0 + 64 * wave, n, lane);
      if constexpr (QJL) dma_tok(nz + kStep + 64 * wave, kgb, t0 + 64 * wave, n, lane);
    } else {
      dma_tok(nz + 2 * kStep + 64 * (wave - 2), vnb, t0 + 64 * (wave - 2), n, lane);
    }
  };

  v8i AK[TK][KC];
  {
    const v8i* ap = reinterpret_cast<const v8i*>(wsA + static_cast<int64_t>(gy) * TK * KC * 2048);
#pragma unroll
    for (int t = 0; t < TK; ++t)
#pragma unroll
      for (int c = 0; c < KC; ++c) AK[t][c] = ap[(t * KC + c) * 64 + lane];
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
  v4f acc[NV][CTW];
#pragma unroll
  for (int t = 0; t < NV; ++t)
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) acc[t][ct] = (v4f){0.f, 0.f, 0.f, 0.f};
  int e_acc = 0;   // scale exponent the accumulators are in (per query, same in every wave)

  // DMA instructions this wave issues per step (the same for every step)
  constexpr int KI = KWP / (K16 ? 256 : 64), VI = VWP / 256;
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
    const float* kns = reinterpret_cast<const float*>(sl + KWP + VWP);
    const int live = static_cast<int>(min(static_cast<int64_t>(kStep), c1 - t0));   // tokens of the step in the chunk
    // ---------------- K phase: logits of tokens t0 + 32*wave .. +31 ----------------
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tt = 32 * wave + 16 * u + j;   // token within the step
      v4f aM = {0.f, 0.f, 0.f, 0.f}, aQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        // lane group g reads group 4c + g; groups past the key (d < 128) give
        // zero bits, which meet zero query limbs
        const int gg = 4 * c + g;
        uint32_t w[5] = {0u, 0u, 0u, 0u, 0u};
        if (NG % 4 == 0 || gg < NG) {
#pragma unroll
          for (int p = 0; p < WK; ++p) w[p] = sl[(tt * NG + gg) * WK + p];
        }
#pragma unroll
        for (int t = 0; t < (1 << (BPK - 1)); ++t)
          aM = mfma_fp8_fp4(AK[t][c], key_bits_to_fp4(walsh_word<BPK>(w, t)), aM);
        if constexpr (QJL) aQ = mfma_fp8_fp4(AK[TK - 1][c], key_bits_to_fp4(w[BPK]), aQ);
      }
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
        for (int t = 0; t < NV; ++t)
#pragma unroll
          for (int ct = 0; ct < CTW; ++ct) acc[t][ct] *= rs;
      }
      // lane group g reads the 32-token block g of the step; blocks past the
      // end hold re-read words, which meet zero weights
      bool vwork = true;
      if constexpr (SPARSE) vwork = qst[0][2] != 0.f || qst[1][2] != 0.f || qst[2][2] != 0.f || qst[3][2] != 0.f;
#pragma unroll
      for (int ct = 0; ct < CTW && vwork; ++ct) {
        if (NT16 % 4 != 0 && CTW * wave + ct >= NT16) break;   // d not a multiple of 64: the last wave has fewer tiles
        const int col = 16 * (CTW * wave + ct) + j;
        uint32_t w[5] = {0u, 0u, 0u, 0u, 0u};
#pragma unroll
        for (int p = 0; p < BPV; ++p) w[p] = sl[KWP + (g * BPV + p) * d + col];
#pragma unroll
        for (int t = 0; t < NV; ++t) acc[t][ct] = mfma_fp8_fp4(A, bits_to_fp4(walsh_word<BPV>(w, t)), acc[t][ct]);
      }
#pragma unroll
      for (int t = 0; t < NV; ++t)
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) pin(acc[t][ct]);
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
  float* pbase = part + ((static_cast<int64_t>(gy) * nrec + rec0 + blockIdx.x) * 4) * PS;
#pragma unroll
  for (int ct = 0; ct < CTW; ++ct) {
    if (NT16 % 4 != 0 && CTW * wave + ct >= NT16) break;
    float v = 0.f;
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      const v4f a = acc[t][ct];
      const float sum = ldexpf(fmaf(a[3], 1.f / 4096.f, fmaf(a[2], 1.f / 256.f, fmaf(a[1], 1.f / 16.f, a[0]))), -e_acc);
      v = fmaf(vcb.coef[t], fmaf(2.f, sum, -wq), v);
    }
    pbase[qi * PS + 16 * (CTW * wave + ct) + j] = v;
  }
  if (threadIdx.x < 4) {
    pbase[threadIdx.x * PS + D] = qst[threadIdx.x][0];
    pbase[threadIdx.x * PS + D + 1] = qst[threadIdx.x][3];
  }
}

template <int D, int BPK, int BPV, bool QJL, bool SPARSE>
struct AttendResidency {
  // d = 128: the tuned residency above; other widths: the compiler's choice,
  // with a 2-step ring where a 3-step one would not leave room for two
  // workgroups per CU (d = 256)
  static constexpr int kBlocks = D == 128 ? attend_blocks_per_cu(BPK, BPV, QJL, SPARSE) : 0;
  static constexpr int kSlots = (kBlocks > 0 || D > 128) ? 2 : 3;
  static constexpr int kBlocksPerCu = kBlocks > 0 ? kBlocks : 1;
};

template <int D, int BPK, int BPV, bool QJL, bool SPARSE>
__global__ void __launch_bounds__(256, (AttendResidency<D, BPK, BPV, QJL, SPARSE>::kBlocksPerCu)) attend_chunk_kernel(
    const uint32_t* __restrict__ kcodes, const float* __restrict__ knorms, const float* __restrict__ kgammas,
    const uint32_t* __restrict__ vcodes, const float* __restrict__ vnorms, int64_t n, int64_t chunk, int G, int RT,
    float scale_log2, float vtau, const uint8_t* __restrict__ wsA, const float* __restrict__ wsC, Codebook vcb,
    float* __restrict__ part, int64_t nrec, int64_t rec0) {
  attend_chunk_body<D, BPK, BPV, AttendResidency<D, BPK, BPV, QJL, SPARSE>::kSlots, QJL, SPARSE>(
      kcodes, knorms, kgammas, vcodes, vnorms, n, chunk, G, RT, scale_log2, vtau, wsA, wsC, vcb, part, nrec, rec0);
}

// Launch the chunk kernel of head dimension D for one segment: the
// instantiation of its key and value widths (sparse V only where SPARSE_OK).
template <int D, bool SPARSE_OK>
hipError_t launch_chunks_d(const AttendSegment& sg, int64_t groups, int G, int RT, float sl, float vtau,
                           const uint8_t* wsA, const float* wsC, float* part, int64_t nrec, int64_t rec0, int64_t nch,
                           int64_t ch, hipStream_t st) {
  dim3 grid(static_cast<unsigned>(nch), static_cast<unsigned>(groups));
  const int bpk = key_codebook(sg.kq).bp, bpv = sg.vq->cb[1].bp;
  const bool qjl = key_qjl(sg.kq);
  if (vtau > 0.f && !SPARSE_OK) return hipErrorNotSupported;
#define TQ_AT(K, V, QV)                                                                                          \
  if (bpk == K && bpv == V && qjl == QV) {                                                                       \
    if constexpr (SPARSE_OK) {                                                                                   \
      if (vtau > 0.f) {                                                                                          \
        hipLaunchKernelGGL((attend_chunk_kernel<D, K, V, QV, true>), grid, dim3(256), 0, st, sg.kcodes, sg.knorms,  \
                           sg.kgammas, sg.vcodes, sg.vnorms, sg.n, ch, G, RT, sl, vtau, wsA, wsC, sg.vq->cb[1],   \
                           part, nrec, rec0);                                                                    \
        return hipGetLastError();                                                                                \
      }                                                                                                          \
    }                                                                                                            \
    hipLaunchKernelGGL((attend_chunk_kernel<D, K, V, QV, false>), grid, dim3(256), 0, st, sg.kcodes, sg.knorms,     \
                       sg.kgammas, sg.vcodes, sg.vnorms, sg.n, ch, G, RT, sl, 0.f, wsA, wsC, sg.vq->cb[1], part,  \
                       nrec, rec0);                                                                              \
    return hipGetLastError();                                                                                    \
  }
#define TQ_AT4(K, QV) TQ_AT(K, 1, QV) TQ_AT(K, 2, QV) TQ_AT(K, 3, QV) TQ_AT(K, 4, QV)
  TQ_AT4(1, true) TQ_AT4(2, true) TQ_AT4(3, true)
  TQ_AT4(1, false) TQ_AT4(2, false) TQ_AT4(3, false) TQ_AT4(4, false)
#undef TQ_AT4
#undef TQ_AT
  return hipErrorNotSupported;
}

}  // namespace attn
}  // namespace tq
