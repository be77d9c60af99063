// Top-k inner-product search straight from packed keys: the unbiased score of
// blog.hotdry.top "TurboQuant vector-search compression" (QJL section) for
// every (query, key) pair, of which only the k best per query leave the chip
// (a2a-mcp.org "什麼是TurboQuant？", benchmark section: top-k recall of a
// vector search over d = 200 embeddings).
//
// With hundreds of queries sharing every key this is bound by the matrix core,
// not by HBM.  A workgroup owns up to 16 queries of one key sequence (4 row
// tiles of the query-operand layout, one per wave, held in registers) and a
// slice of that sequence's keys.  Keys pass through LDS 64 at a time, read
// once from memory for all four waves, with the next batch in flight in
// registers while the current one is scored.  Each lane scores one key of a
// 16-key tile for one query and keeps the KK best (score, index) pairs it has
// seen in registers, ordered by score descending, then index ascending.  At
// the end the 16 lanes of a query hand their sorted lists to a tournament
// (shuffles within the 16 lanes) that emits the slice's top k.  Workgroups
// that share a key slice sit on one XCD so the slice is reused from that
// XCD's L2.  A second kernel merges the slices of each query the same way.
//
// The arithmetic of a score is the logits kernel's, term for term, so a top-k
// score equals the corresponding logit bit for bit.
#include "tq_device.h"
#include "tq_kernels.h"

namespace tq {

namespace {

constexpr int kTopBlockKeys = 64;
// Candidates a lane may queue before the lists take them (see the scan loop)
constexpr int kQueue = 8;

// (s, i) ranks before (t, j): higher score, ties to the lower index
// (bitwise, so that no operand is evaluated under a branch)
__device__ __forceinline__ bool ranks_before(float s, int i, float t, int j) {
  return static_cast<bool>(static_cast<int>(s > t) | (static_cast<int>(s == t) & static_cast<int>(i < j)));
}

// insert into a list sorted by ranks_before; the last entry falls off
template <int KK>
__device__ __forceinline__ void list_insert(float s, int i, float (&ls)[KK], int (&li)[KK]) {
#pragma unroll
  for (int k = 0; k < KK; ++k) {
    const bool b = ranks_before(s, i, ls[k], li[k]);
    const float ts = b ? ls[k] : s;
    const int ti = b ? li[k] : i;
    ls[k] = b ? s : ls[k];
    li[k] = b ? i : li[k];
    s = ts;
    i = ti;
  }
}

template <int KK>
__device__ __forceinline__ void list_init(float (&ls)[KK], int (&li)[KK]) {
#pragma unroll
  for (int k = 0; k < KK; ++k) {
    ls[k] = -INFINITY;
    li[k] = 0x7fffffff;
  }
}

// Tournament over the sorted lists of WIDTH consecutive lanes (a power of two
// <= 64, aligned): round r finds the r-th best pair of their union on every
// lane of the group; the writer lane stores it at position r.
template <int KK, int WIDTH>
__device__ __forceinline__ void tournament(const float (&ls)[KK], const int (&li)[KK], int topk, bool writer,
                                           float* out_s, int* out_i, int64_t* out_i64) {
  int head = 0;
  for (int r = 0; r < topk; ++r) {
    float s = -INFINITY;
    int i = 0x7fffffff;
#pragma unroll
    for (int k = 0; k < KK; ++k) {
      if (k == head) {
        s = ls[k];
        i = li[k];
      }
    }
    float bs = s;
    int bi = i;
#pragma unroll
    for (int off = WIDTH / 2; off > 0; off >>= 1) {
      const float os = __shfl_xor(bs, off);
      const int oi = __shfl_xor(bi, off);
      if (ranks_before(os, oi, bs, bi)) {
        bs = os;
        bi = oi;
      }
    }
    // the lane whose head won moves on (a key sits in one list only, so one
    // lane matches, unless all that is left are fillers)
    if (s == bs && i == bi) ++head;
    if (writer) {
      if (out_s) out_s[r] = bs;
      if (out_i) out_i[r] = bi;
      if (out_i64) out_i64[r] = bi;
    }
  }
}

}  // namespace

struct TopkPlan {
  int RT;               // row tiles (4 queries each) per key sequence
  int64_t rg_per_seq;   // row groups (4 row tiles) per key sequence
  int64_t rg_count;     // all row groups
  int64_t slices;       // key slices per sequence
  int64_t slice_keys;   // keys per slice (a multiple of the batch)
};

static int64_t topk_resident_blocks() {
  static int64_t blocks = [] {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    return static_cast<int64_t>(3) * cus;
  }();
  return blocks;
}

static TopkPlan topk_plan(int B, int Hq, int Hkv, int64_t n) {
  TopkPlan p;
  const int G = Hq / Hkv;
  p.RT = (G + 3) / 4;
  p.rg_per_seq = (p.RT + 3) / 4;
  p.rg_count = static_cast<int64_t>(B) * Hkv * p.rg_per_seq;
  // about three rounds of resident workgroups (three per CU): fewer, longer
  // slices spend less of their time filling the lists (measured on the
  // 10^6-key search: 2331 workgroups 6.5 ms, 4158 6.7 ms, 1512 7.4 ms)
  int64_t s = (3 * topk_resident_blocks() + p.rg_count - 1) / p.rg_count;
  const int64_t max_s = (n + kTopBlockKeys - 1) / kTopBlockKeys;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  const int64_t per = n > 0 ? (n + s - 1) / s : 1;
  p.slice_keys = (per + kTopBlockKeys - 1) / kTopBlockKeys * kTopBlockKeys;
  p.slices = (n + p.slice_keys - 1) / p.slice_keys;
  return p;
}

static int64_t topk_prep_bytes(const tq_quantizer* q, int B, int Hq, int Hkv) {
  return (scores_ws_bytes(q, B, Hq, Hkv) + 255) / 256 * 256;
}

int64_t topk_ws_bytes(const tq_quantizer* q, int B, int Hq, int Hkv, int64_t n, int topk) {
  const TopkPlan p = topk_plan(B, Hq, Hkv, n);
  // candidates [row group][slice][16 queries][topk]: float scores, then int indices
  return topk_prep_bytes(q, B, Hq, Hkv) + p.rg_count * p.slices * 16 * topk * 8 + 256;
}

// QJL: prod keys (with the QJL plane and gammas); without it MSE-only keys.
// Three workgroups per CU where the query operands leave room (the
// compiler would otherwise take a few more registers and drop to two).
template <int BP, int GW, int KK, bool QJL>
__global__ void __launch_bounds__(256, (KK <= 16 && ((1 << (BP - 1)) + QJL) * ((GW + 3) / 4) <= 10) ? 3 : 1)
    topk_scan_kernel(const uint32_t* __restrict__ codes, const float* __restrict__ norms,
                     const float* __restrict__ gammas, int64_t n, int RT, int64_t rg_per_seq, int64_t rg_count,
                     int64_t slices, int64_t slice_keys, int topk, const uint8_t* __restrict__ wsA,
                     const float* __restrict__ wsC, float* __restrict__ cand_s, int* __restrict__ cand_i) {
  constexpr int T = (1 << (BP - 1)) + (QJL ? 1 : 0);
  constexpr int W = BP + (QJL ? 1 : 0);
  constexpr int C = (GW + 3) / 4;
  constexpr int WPK = GW * W;                      // packed words per key
  constexpr int BW = kTopBlockKeys * WPK;          // words of a batch
  constexpr int BUFW = BW + 2 * kTopBlockKeys;     // + norms + gammas
  constexpr int NS = 3;                            // batches b, b+1, b+2 staged at once
  __shared__ __attribute__((aligned(16))) uint32_t buf[NS][BUFW];
  // candidate queue: entry e of thread tid at cq[e][tid] (score bits, key)
  __shared__ uint2 cq[kQueue][256];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup -> (row group, slice); consecutive workgroups go round-robin over
  // the 8 XCDs, so XCD x takes slices x, x+8, ... with all row groups of each
  const int64_t L = blockIdx.x;
  const int64_t x = L & 7, jx = L >> 3;
  const int64_t rg = jx % rg_count;
  const int64_t slice = x + 8 * (jx / rg_count);
  if (slice >= slices) return;   // uniform over the workgroup
  const int64_t seq = rg / rg_per_seq;
  const int rt = static_cast<int>((rg - seq * rg_per_seq) * 4) + wave;
  const bool active = rt < RT;   // uniform over the wave
  const int64_t gy = seq * RT + rt;
  const int qi = lane >> 4, jj = lane & 15, g = lane >> 4;

  v8i A[T][C];
  float cs[10];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < C; ++c) A[t][c] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 10; ++i) cs[i] = 0.f;
  if (active) {
    const v8i* ap = reinterpret_cast<const v8i*>(wsA + gy * T * C * 2048);
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int c = 0; c < C; ++c) A[t][c] = ap[(t * C + c) * 64 + lane];
    const float* cp = wsC + (gy * 4 + qi) * 16;
#pragma unroll
    for (int i = 0; i < 10; ++i) cs[i] = cp[i];
  }

  float ls[KK];
  int li[KK];
  list_init<KK>(ls, li);
  // Keys that pass the pruning bounds are queued per lane in LDS and enter the
  // sorted list in bulk, when some lane of the wave has a full queue and at
  // the end of the slice.  The insertion runs under a wave-wide gate, so
  // inserting every candidate as it arrives costs the whole wave an insertion
  // whenever any of its 64 lanes has one; batched, it costs about as many
  // insertion rounds as the fullest queue holds.  The bounds a queued key
  // passed only rise until the lists take it, so the filter stays valid.
  int qn = 0;
  // A key can only enter the query's top k if it ranks at least level with
  // the query's current k-th best.  The largest of the 16 lanes' own k-th
  // best scores is a lower bound of that (the lane alone holds k scores at
  // least as large), so keys below it are skipped without touching the
  // lists: insertions become rare.  A second bound: each of the 16 lanes
  // holds j + 1 scores at least its entry j, so the smallest entry j over the
  // lanes is at most the query's k-th best when 16 (j + 1) >= k.  With
  // j = (k - 1) / 16 this takes the lanes' best scores, which rank near the
  // query's top k (the first bound, a single lane's k-th best, ranks near its
  // 16 k-th).  The bound changes only when the lists do, so it is refreshed
  // after each bulk insertion (wave-uniform: the row reductions need every
  // lane).
  float tau = -INFINITY;
  auto refresh = [&]() {
    float kth = ls[0];
#pragma unroll
    for (int k = 1; k < KK; ++k)
      if (k == topk - 1) kth = ls[k];
    const float topj = (KK > 16 && topk > 16) ? ls[1] : ls[0];
    tau = fmaxf(row_max16(kth), row_min16(topj));
  };
  auto drain = [&]() {
#pragma unroll 1
    for (int e = 0; e < kQueue; ++e) {
      if (__ballot(e < qn) == 0ull) break;
      if (e < qn) {
        const uint2 c = cq[e][tid];
        list_insert<KK>(__uint_as_float(c.x), static_cast<int>(c.y), ls, li);
      }
    }
    qn = 0;
    refresh();
  };

  const uint32_t* cbase = codes + seq * n * WPK;
  const float* nb = norms + seq * n;
  const float* gb = QJL ? gammas + seq * n : nullptr;
  const int64_t k_begin = slice * slice_keys;
  const int64_t k_end = min(n, k_begin + slice_keys);
  const int nbat = static_cast<int>((k_end - k_begin + kTopBlockKeys - 1) / kTopBlockKeys);

  // batch bi of the slice goes HBM -> LDS by dword DMA (no registers, no
  // alignment assumptions); past the slice end the last valid word is re-read
  // DMA instructions per batch: words round-robin, norms by wave 2, gammas by wave 3
  const int wave_dma = (WPK + 3 - wave) / 4 + ((wave == 2 || (QJL && wave == 3)) ? 1 : 0);
  auto issue = [&](int bi, int slot) {
    const int64_t k0 = k_begin + static_cast<int64_t>(bi) * kTopBlockKeys;
    const int valid = static_cast<int>(min(k_end, k0 + kTopBlockKeys) - k0);
    uint32_t* dst = buf[slot];
    // 32-bit byte offsets from the batch's uniform start: scalar base + vector offset
    const char* src = reinterpret_cast<const char*>(cbase + k0 * WPK);
    const uint32_t vw = static_cast<uint32_t>(valid * WPK);
    for (int i = wave; i < WPK; i += 4) {
      uint32_t off = static_cast<uint32_t>(i * 64 + lane);
      if (off >= vw) off = vw - 1;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(src + 4u * off), as_lds(dst + i * 64), 4, 0, 0);
    }
    if (wave == 2 || (QJL && wave == 3)) {
      const char* arr = reinterpret_cast<const char*>((wave == 2 ? nb : gb) + k0);
      const uint32_t t = 4u * static_cast<uint32_t>(min(lane, valid - 1));
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const float*>(arr + t),
                                       as_lds(dst + BW + (wave - 2) * kTopBlockKeys), 4, 0, 0);
    }
  };

  constexpr int P = NS - 1;   // batches in flight ahead of the one being scored
#pragma unroll
  for (int k = 0; k < P; ++k)
    if (k < nbat) issue(k, k);
  int slot = 0;
  for (int bi = 0; bi < nbat; ++bi, slot = slot == NS - 1 ? 0 : slot + 1) {
    wait_vm_upto<16>(min(P - 1, nbat - 1 - bi) * wave_dma);   // this wave's loads of batch bi landed
    __syncthreads();                                          // ... and every wave's; slot of bi-1 free
    if (bi + P < nbat) issue(bi + P, slot == 0 ? NS - 1 : slot - 1);
    if (active) {
      const uint32_t* kw = buf[slot];
      const float* kn = reinterpret_cast<const float*>(kw + BW);
      const int64_t k0 = k_begin + static_cast<int64_t>(bi) * kTopBlockKeys;
      const int nk = static_cast<int>(min(static_cast<int64_t>(kTopBlockKeys), k_end - k0));
#pragma unroll
      for (int u = 0; u < kTopBlockKeys / 16; ++u) {
        const int kk = 16 * u + jj;
        v4f aM = {0.f, 0.f, 0.f, 0.f}, aQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < C; ++c) {
          // groups past the key's last one (gg >= GW) read the next key's
          // words or the batch's norms, inside the slot: their fp4 values
          // are finite and meet query coordinates >= 32 GW >= d, which the
          // query operand holds as 0, so they add exactly 0
          const int gg = 4 * c + g;
          uint32_t w[5] = {0u, 0u, 0u, 0u, 0u};
#pragma unroll
          for (int p = 0; p < W; ++p) w[p] = kw[(kk * GW + gg) * W + p];
#pragma unroll
          for (int t = 0; t < (1 << (BP - 1)); ++t)
            aM = mfma_fp8_fp4(A[t][c], key_bits_to_fp4(walsh_word<BP>(w, t)), aM);
          if constexpr (QJL) aQ = mfma_fp8_fp4(A[T - 1][c], key_bits_to_fp4(w[BP]), aQ);
        }
        pin(aM);
        const float mse = fmaf(aM[0], cs[2], fmaf(aM[1], cs[3], fmaf(aM[2], cs[4], fmaf(aM[3], cs[5], cs[0]))));
        float s = kn[kk] * mse;
        if constexpr (QJL) {
          pin(aQ);
          const float qjl = fmaf(aQ[0], cs[6], fmaf(aQ[1], cs[7], fmaf(aQ[2], cs[8], fmaf(aQ[3], cs[9], cs[1]))));
          s = fmaf(kn[kk], mse, kn[kTopBlockKeys + kk] * qjl);
        }
        const int key = static_cast<int>(k0) + kk;
        const bool ins = kk < nk && s >= tau && ranks_before(s, key, ls[KK - 1], li[KK - 1]);
        if (ins) {
          cq[qn][tid] = make_uint2(__float_as_uint(s), static_cast<uint32_t>(key));
          ++qn;
        }
        // a queue is full: every lane's queued keys enter its list
        if (__ballot(qn == kQueue) != 0ull) drain();
      }
    }
  }

  if (!active) return;   // no barrier follows
  drain();
  const int64_t q16 = wave * 4 + qi;
  const int64_t base = ((rg * slices + slice) * 16 + q16) * topk;
  tournament<KK, 16>(ls, li, topk, jj == 0, cand_s + base, cand_i + base, nullptr);
}

// One wave per query: merge the slices' candidate lists into the final top k.
template <int KK>
__global__ void __launch_bounds__(64) topk_merge_kernel(const float* __restrict__ cand_s,
                                                        const int* __restrict__ cand_i, int64_t slices, int Hq,
                                                        int Hkv, int64_t rg_per_seq, int topk,
                                                        float* __restrict__ out, int64_t* __restrict__ out_idx) {
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x;   // b * Hq + h
  const int G = Hq / Hkv;
  const int64_t b = bh / Hq;
  const int h = static_cast<int>(bh - b * Hq);
  const int kvh = h / G, qg = h - kvh * G;
  const int rt = qg >> 2, qi = qg & 3;
  const int64_t seq = b * Hkv + kvh;
  const int64_t rg = seq * rg_per_seq + (rt >> 2);
  const int64_t q16 = (rt & 3) * 4 + qi;
  float ls[KK];
  int li[KK];
  list_init<KK>(ls, li);
  for (int64_t sl = lane; sl < slices; sl += 64) {
    const int64_t base = ((rg * slices + sl) * 16 + q16) * topk;
    for (int k = 0; k < topk; ++k) {
      const float s = cand_s[base + k];
      const int i = cand_i[base + k];
      if (!ranks_before(s, i, ls[KK - 1], li[KK - 1])) break;   // the slice's list is sorted
      list_insert<KK>(s, i, ls, li);
    }
  }
  tournament<KK, 64>(ls, li, topk, lane == 0, out + bh * topk, nullptr, out_idx + bh * topk);
}

hipError_t launch_topk(const tq_quantizer* q, const void* queries, int q_dtype, int B, int Hq, int Hkv,
                       const uint32_t* codes, const float* norms, const float* gammas, int64_t n, int topk, float* out,
                       int64_t* out_idx, void* ws, hipStream_t st) {
  if (topk < 1 || topk > 32 || n >= 0x7fffffff) return hipErrorNotSupported;
  const TopkPlan p = topk_plan(B, Hq, Hkv, n);
  const int T = key_terms(q);
  const int Cc = (q->d + 127) / 128;
  const int64_t row_tiles = static_cast<int64_t>(B) * Hkv * p.RT;
  // whole rounds of 8 slices so that each XCD's workgroups share slices
  const int64_t blocks = (p.slices + 7) / 8 * 8 * p.rg_count;
  if (blocks > 0x7fffffff) return hipErrorNotSupported;
  hipError_t e = launch_query_prep_ws(q, queries, q_dtype, B, Hq, Hkv, ws, st);
  if (e != hipSuccess) return e;
  const uint8_t* wsA = static_cast<const uint8_t*>(ws);
  const float* wsC = reinterpret_cast<const float*>(wsA + row_tiles * T * Cc * 2048);
  float* cs = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + topk_prep_bytes(q, B, Hq, Hkv));
  int* ci = reinterpret_cast<int*>(cs + p.rg_count * p.slices * 16 * topk);
  const int bp = key_codebook(q).bp;
  const bool qjl = key_qjl(q);
  const int gw = (q->d + 31) / 32;
  // per-lane list length: the shortest of 12, 16, 32 that holds k entries
  // (the insertion cost grows with it)
  const int kk = topk <= 12 ? 12 : (topk <= 16 ? 16 : 32);
  bool launched = false;
#define TQ_TK_L(BPV, GWV, KKV, QV)                                                                              \
  hipLaunchKernelGGL((topk_scan_kernel<BPV, GWV, KKV, QV>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, \
                     codes, norms, gammas, n, p.RT, p.rg_per_seq, p.rg_count, p.slices, p.slice_keys, topk, wsA, wsC,   \
                     cs, ci)
#define TQ_TK(BPV, GWV, QV)                                           \
  if (!launched && bp == BPV && gw == GWV && qjl == QV) {             \
    if (kk == 32)                                                     \
      TQ_TK_L(BPV, GWV, 32, QV);                                      \
    else if (kk == 16)                                                \
      TQ_TK_L(BPV, GWV, 16, QV);                                      \
    else                                                              \
      TQ_TK_L(BPV, GWV, 12, QV);                                      \
    launched = true;                                                  \
  }
#define TQ_TK_ALL(GWV)                                                                                  \
  TQ_TK(1, GWV, true) TQ_TK(2, GWV, true) TQ_TK(3, GWV, true) TQ_TK(1, GWV, false) TQ_TK(2, GWV, false) \
  TQ_TK(3, GWV, false) TQ_TK(4, GWV, false)
  TQ_TK_ALL(1) TQ_TK_ALL(2) TQ_TK_ALL(3) TQ_TK_ALL(4) TQ_TK_ALL(5) TQ_TK_ALL(6) TQ_TK_ALL(7) TQ_TK_ALL(8)
#undef TQ_TK_ALL
#undef TQ_TK
#undef TQ_TK_L
  if (!launched) return hipErrorNotSupported;
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 mgrid(static_cast<unsigned>(static_cast<int64_t>(B) * Hq));
  if (kk == 32)
    hipLaunchKernelGGL((topk_merge_kernel<32>), mgrid, dim3(64), 0, st, cs, ci, p.slices, Hq, Hkv, p.rg_per_seq, topk,
                       out, out_idx);
  else if (kk == 16)
    hipLaunchKernelGGL((topk_merge_kernel<16>), mgrid, dim3(64), 0, st, cs, ci, p.slices, Hq, Hkv, p.rg_per_seq, topk,
                       out, out_idx);
  else
    hipLaunchKernelGGL((topk_merge_kernel<12>), mgrid, dim3(64), 0, st, cs, ci, p.slices, Hq, Hkv, p.rg_per_seq, topk,
                       out, out_idx);
  return hipGetLastError();
}

}  // namespace tq
