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
// The bounded search: row tiles (32 queries) per row group of its scan, and
// the candidates one merge wave rescores (more: the exact path)
constexpr int kLbRowTiles = 8;
constexpr int kLbCand = 512;

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
// lane of the group; the writer lane stores it at position r < topk.  Runs
// `rounds` >= topk rounds and returns the last one's score (-inf once only
// fillers are left).
template <int KK, int WIDTH>
__device__ __forceinline__ float tournament(const float (&ls)[KK], const int (&li)[KK], int topk, bool writer,
                                            float* out_s, int* out_i, int64_t* out_i64, int rounds = -1) {
  if (rounds < topk) rounds = topk;
  int head = 0;
  float last = -INFINITY;
  for (int r = 0; r < rounds; ++r) {
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
    if (writer && r < topk) {
      if (out_s) out_s[r] = bs;
      if (out_i) out_i[r] = bi;
      if (out_i64) out_i64[r] = bi;
    }
    last = bs;
  }
  return last;
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

// the bounded scan: row groups of 8 row tiles, two workgroups per CU
static TopkPlan topk_lb_plan(int B, int Hq, int Hkv, int64_t n) {
  TopkPlan p;
  const int G = Hq / Hkv;
  p.RT = (G + 3) / 4;
  p.rg_per_seq = (p.RT + kLbRowTiles - 1) / kLbRowTiles;
  p.rg_count = static_cast<int64_t>(B) * Hkv * p.rg_per_seq;
  int64_t s = (3 * (topk_resident_blocks() / 3 * 2) + p.rg_count - 1) / p.rg_count;
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

// The bounded search serves k <= 12 (one 12-entry list per query) with query
// operands of at most 10 MFMA tiles (two lists per lane fit beside them)
static bool topk_bounded(const tq_quantizer* q, int topk) {
  const int C = (q->d + 127) / 128;
  return topk <= 12 && key_terms(q) * C <= 10;
}

struct TopkLayout {
  int64_t exact_cand, lb_cand, lb_ceil, flags, total;   // byte offsets after the prep, and the size
};
static TopkLayout topk_layout(const tq_quantizer* q, int B, int Hq, int Hkv, int64_t n, int topk) {
  const TopkPlan p = topk_plan(B, Hq, Hkv, n);
  TopkLayout l;
  int64_t o = topk_prep_bytes(q, B, Hq, Hkv);
  // exact candidates [row group][slice][16 queries][topk]: float scores, then int indices
  l.exact_cand = o;
  o += (p.rg_count * p.slices * 16 * topk * 8 + 255) / 256 * 256;
  l.lb_cand = l.lb_ceil = l.flags = o;
  if (topk_bounded(q, topk)) {
    const TopkPlan pl = topk_lb_plan(B, Hq, Hkv, n);
    // bounded candidates [row group][slice][32 queries][topk] (lower bounds, indices),
    // then one ceiling per cell, then one flag per query
    l.lb_cand = o;
    o += (pl.rg_count * pl.slices * 32 * topk * 8 + 255) / 256 * 256;
    l.lb_ceil = o;
    o += (pl.rg_count * pl.slices * 32 * 4 + 255) / 256 * 256;
    l.flags = o;
    o += (static_cast<int64_t>(B) * Hq + 255) / 256 * 256;
  }
  l.total = o + 256;
  return l;
}

int64_t topk_ws_bytes(const tq_quantizer* q, int B, int Hq, int Hkv, int64_t n, int topk) {
  return topk_layout(q, B, Hq, Hkv, n, topk).total;
}

// QJL: prod keys (with the QJL plane and gammas); without it MSE-only keys.
// Three workgroups per CU where the query operands leave room (the
// compiler would otherwise take a few more registers and drop to two).
template <int BP, int GW, int KK, bool QJL>
__global__ void __launch_bounds__(256, (KK <= 16 && ((1 << (BP - 1)) + QJL) * ((GW + 3) / 4) <= 10) ? 3 : 1)
    topk_scan_kernel(const uint32_t* __restrict__ codes, const float* __restrict__ norms,
                     const float* __restrict__ gammas, int64_t n, int RT, int64_t rg_per_seq, int64_t rg_count,
                     int64_t slices, int64_t slice_keys, int topk, const uint8_t* __restrict__ wsA,
                     const float* __restrict__ wsC, float* __restrict__ cand_s, int* __restrict__ cand_i,
                     const uint8_t* __restrict__ flags, int Hq, int Hkv) {
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
  if (flags) {
    // the fallback of the bounded search: only row groups holding a query
    // whose bound could not be certified run (uniform over the workgroup)
    const int G = Hq / Hkv;
    const int64_t qbase = (seq / Hkv) * Hq + (seq % Hkv) * G;
    const int qg0 = static_cast<int>((rg - seq * rg_per_seq) * 16);
    bool any = false;
    for (int j = 0; j < 16; ++j)
      if (qg0 + j < G && flags[qbase + qg0 + j]) any = true;
    if (!any) return;
  }
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
                                                        float* __restrict__ out, int64_t* __restrict__ out_idx,
                                                        const uint8_t* __restrict__ flags) {
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x;   // b * Hq + h
  if (flags && !flags[bh]) return;   // certified by the bounded search
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

// ---------------------------------------------------------------------------
// Bounded search (k <= 12).  The exact scan spends its matrix-core time on 4
// limbs of every query; a scan over limbs 0 and 1 alone carries 8 queries
// per 16-row operand (2 limbs each) and halves it.  Its sums bracket the full
// score: the query prep bounds what limbs 2 and 3 add (E_M, E_Q per query),
// so for every key
//   lo = n (C_M,0-1 + cM - E_M) + gamma (C_Q,0-1 + cQ - E_Q) <= s <= lo + 2 B,
//   B = n E_M + gamma E_Q.
// Pass 1 keeps, per query and key slice, the keys with the best lower bounds
// (pruned by upper bound against the running k-th lower bound), emits the
// slice's top k of them and a ceiling of every upper bound it does not emit.
// The merge takes tau = the query's k-th lower bound: every key whose upper
// bound stays below tau ranks below k keys, so if every slice's ceiling is
// below tau the top k lies among the emitted keys with an upper bound >= tau,
// and those are scored again with the exact scan's operands and arithmetic
// (the logits' bits) and ranked.  A query whose ceiling reaches tau (ties,
// repeated keys) is flagged and served by the exact scan and merge.
// ---------------------------------------------------------------------------
template <int BP, int GW, bool QJL, int KK>
__global__ void __launch_bounds__(256, 2)
    topk_lb_scan_kernel(const uint32_t* __restrict__ codes, const float* __restrict__ norms,
                        const float* __restrict__ gammas, int64_t n, int RT, int64_t rg_per_seq, int64_t rg_count,
                        int64_t slices, int64_t slice_keys, int topk, const uint8_t* __restrict__ wsA,
                        const float* __restrict__ wsC, float* __restrict__ cand_l, int* __restrict__ cand_i,
                        float* __restrict__ cand_f) {
  static_assert(KK >= 10 && KK <= 12, "lists of 10 or 12 entries (k <= KK)");
  constexpr int T = (1 << (BP - 1)) + (QJL ? 1 : 0);
  constexpr int W = BP + (QJL ? 1 : 0);
  constexpr int C = (GW + 3) / 4;
  constexpr int WPK = GW * W;
  constexpr int BW = kTopBlockKeys * WPK;
  constexpr int BUFW = BW + 2 * kTopBlockKeys;
  constexpr int NS = 3;
  __shared__ __attribute__((aligned(16))) uint32_t buf[NS][BUFW];
  __shared__ uint2 cq[2][kQueue][256];   // candidate queues of the lane's two queries

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t L = blockIdx.x;
  const int64_t x = L & 7, jx = L >> 3;
  const int64_t rg = jx % rg_count;
  const int64_t slice = x + 8 * (jx / rg_count);
  if (slice >= slices) return;   // uniform over the workgroup
  const int64_t seq = rg / rg_per_seq;
  const int rt0 = static_cast<int>((rg - seq * rg_per_seq) * kLbRowTiles) + 2 * wave;   // this wave's row tiles
  const bool active = rt0 < RT;                                                            // uniform over the wave
  const int jj = lane & 15, g = lane >> 4;

  // A operand row r = lane & 15: limb r & 1 of the wave's query r >> 1,
  // gathered from the 4-limb operands of its row tile
  v8i A[T][C];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < C; ++c) A[t][c] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
  {
    const int r = lane & 15, ql = r >> 1;
    const int rta = rt0 + (ql >> 2);
    if (active && rta < RT) {
      const v8i* ap = reinterpret_cast<const v8i*>(wsA + (seq * RT + rta) * T * C * 2048);
      const int src = 4 * (ql & 3) + (r & 1) + 16 * g;
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int c = 0; c < C; ++c) A[t][c] = ap[(t * C + c) * 64 + src];
    }
  }
  // output rows 4g .. 4g+3: limbs 0, 1 of query 2g, then of query 2g + 1
  // (row tile rt0 + g / 2, in-tile 2 (g % 2) + h); per query the lower
  // bracket's constants and 2 E
  const int rtq = rt0 + (g >> 1);
  float sM[2][2], sQ[2][2], cMl[2], cQl[2], e2M[2], e2Q[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float cv[12] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (active && rtq < RT) {
      const float* cp = wsC + ((seq * RT + rtq) * 4 + 2 * (g & 1) + h) * 16;
#pragma unroll
      for (int j = 0; j < 12; ++j) cv[j] = cp[j];
    }
    sM[h][0] = cv[2];
    sM[h][1] = cv[3];
    sQ[h][0] = cv[6];
    sQ[h][1] = cv[7];
    cMl[h] = cv[0] - cv[10];
    cQl[h] = cv[1] - cv[11];
    e2M[h] = 2.f * cv[10];
    e2Q[h] = 2.f * cv[11];
  }

  float ls[2][KK];
  int li[2][KK];
  list_init<KK>(ls[0], li[0]);
  list_init<KK>(ls[1], li[1]);
  int qn[2] = {0, 0};
  float tau[2] = {-INFINITY, -INFINITY};
  float nmax = 0.f, gmax = 0.f;   // the largest norm and gamma among this lane's keys
  // the running k-th best lower bound of each query (the exact scan's two
  // bounds, over lower bounds), refreshed when its list changes
  auto refresh = [&](int h) {
    float kth = ls[h][0];
#pragma unroll
    for (int k = 1; k < KK; ++k)
      if (k == topk - 1) kth = ls[h][k];
    tau[h] = fmaxf(row_max16(kth), row_min16(ls[h][0]));
  };
  auto drain = [&]() {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll 1
      for (int e = 0; e < kQueue; ++e) {
        if (__ballot(e < qn[h]) == 0ull) break;
        if (e < qn[h]) {
          const uint2 c = cq[h][e][tid];
          list_insert<KK>(__uint_as_float(c.x), static_cast<int>(c.y), ls[h], li[h]);
        }
      }
      qn[h] = 0;
      refresh(h);
    }
  };

  const uint32_t* cbase = codes + seq * n * WPK;
  const float* nb = norms + seq * n;
  const float* gb = QJL ? gammas + seq * n : nullptr;
  const int64_t k_begin = slice * slice_keys;
  const int64_t k_end = min(n, k_begin + slice_keys);
  const int nbat = static_cast<int>((k_end - k_begin + kTopBlockKeys - 1) / kTopBlockKeys);
  const int wave_dma = (WPK + 3 - wave) / 4 + ((wave == 2 || (QJL && wave == 3)) ? 1 : 0);
  auto issue = [&](int bi, int slot) {
    const int64_t k0 = k_begin + static_cast<int64_t>(bi) * kTopBlockKeys;
    const int valid = static_cast<int>(min(k_end, k0 + kTopBlockKeys) - k0);
    uint32_t* dst = buf[slot];
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

  constexpr int P = NS - 1;
#pragma unroll
  for (int k = 0; k < P; ++k)
    if (k < nbat) issue(k, k);
  int slot = 0;
  for (int bi = 0; bi < nbat; ++bi, slot = slot == NS - 1 ? 0 : slot + 1) {
    wait_vm_upto<16>(min(P - 1, nbat - 1 - bi) * wave_dma);
    __syncthreads();
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
          // groups past the key's last (gg >= GW) read inside the slot and
          // meet query coordinates the operand holds as 0
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
        if constexpr (QJL) pin(aQ);
        const float nv = kn[kk];
        const float gv = QJL ? kn[kTopBlockKeys + kk] : 0.f;
        const bool kin = kk < nk;
        nmax = fmaxf(nmax, kin ? nv : 0.f);
        gmax = fmaxf(gmax, kin ? gv : 0.f);
        const int key = static_cast<int>(k0) + kk;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float ml = fmaf(aM[2 * h], sM[h][0], fmaf(aM[2 * h + 1], sM[h][1], cMl[h]));
          float lo = nv * ml, up;
          if constexpr (QJL) {
            const float ql = fmaf(aQ[2 * h], sQ[h][0], fmaf(aQ[2 * h + 1], sQ[h][1], cQl[h]));
            lo = fmaf(nv, ml, gv * ql);
            up = fmaf(nv, e2M[h], fmaf(gv, e2Q[h], lo));
          } else {
            up = fmaf(nv, e2M[h], lo);
          }
          const bool ins = kin && up >= tau[h] && ranks_before(lo, key, ls[h][KK - 1], li[h][KK - 1]);
          if (ins) {
            cq[h][qn[h]][tid] = make_uint2(__float_as_uint(lo), static_cast<uint32_t>(key));
            ++qn[h];
          }
        }
        if (__ballot(qn[0] == kQueue || qn[1] == kQueue) != 0ull) drain();
      }
    }
  }

  if (!active) return;   // no barrier follows
  drain();
  // every key of the slice left out of the emitted top k has a lower bound
  // at most its lane list's last entry or the (k+1)-th entry of the union,
  // and an upper bound at most that plus 2 (nmax E_M + gmax E_Q)
  const float nm = row_max16(nmax), gm = row_max16(gmax);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t q32 = wave * 8 + 2 * g + h;
    const int64_t cell = (rg * slices + slice) * 32 + q32;
    const float next = tournament<KK, 16>(ls[h], li[h], topk, jj == 0, cand_l + cell * topk, cand_i + cell * topk,
                                          nullptr, topk + 1);
    const float fl = fmaxf(row_max16(ls[h][KK - 1]), next);
    float fu = fmaf(nm, e2M[h], fmaf(gm, e2Q[h], fl));
    if (fu > -INFINITY) fu += fabsf(fu) * 0x1p-20f;   // the two roundings above, upward
    if (jj == 0) cand_f[cell] = fu;
  }
}

// One wave per query: certify the bounded scan's result and rescore its
// candidates exactly, or flag the query for the exact scan.
template <int BP, int GW, bool QJL>
__global__ void __launch_bounds__(64)
    topk_lb_merge_kernel(const uint32_t* __restrict__ codes, const float* __restrict__ norms,
                         const float* __restrict__ gammas, int64_t n, int Hq, int Hkv, int RT, int64_t rg_per_seq,
                         int64_t slices, int topk, const uint8_t* __restrict__ wsA, const float* __restrict__ wsC,
                         const float* __restrict__ cand_l, const int* __restrict__ cand_i,
                         const float* __restrict__ cand_f, float* __restrict__ out, int64_t* __restrict__ out_idx,
                         uint8_t* __restrict__ flags) {
  constexpr int KK = 12;
  constexpr int T = (1 << (BP - 1)) + (QJL ? 1 : 0);
  constexpr int W = BP + (QJL ? 1 : 0);
  constexpr int C = (GW + 3) / 4;
  constexpr int WPK = GW * W;
  __shared__ int cand[kLbCand];
  __shared__ int ncand;

  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x;   // b * Hq + h
  const int G = Hq / Hkv;
  const int64_t b = bh / Hq;
  const int h = static_cast<int>(bh - b * Hq);
  const int kvh = h / G, qg = h - kvh * G;
  const int rt = qg >> 2, qi = qg & 3;
  const int64_t seq = b * Hkv + kvh;
  const int64_t rg = seq * rg_per_seq + rt / kLbRowTiles;
  const int64_t q32 = (rt % kLbRowTiles) * 4 + qi;
  const int64_t gy = seq * RT + rt;
  const float* cq = wsC + (gy * 4 + qi) * 16;
  const float eM = cq[10], eQ = QJL ? cq[11] : 0.f;

  // tau = the k-th best lower bound; the ceiling of what the slices left out
  float ls[KK];
  int li[KK];
  list_init<KK>(ls, li);
  float ceil_u = -INFINITY;
  for (int64_t sl = lane; sl < slices; sl += 64) {
    const int64_t cell = (rg * slices + sl) * 32 + q32;
    ceil_u = fmaxf(ceil_u, cand_f[cell]);
    for (int k = 0; k < topk; ++k) {
      const float s = cand_l[cell * topk + k];
      const int i = cand_i[cell * topk + k];
      if (!ranks_before(s, i, ls[KK - 1], li[KK - 1])) break;   // the slice's list is sorted
      list_insert<KK>(s, i, ls, li);
    }
  }
  const float tau = tournament<KK, 64>(ls, li, topk, false, nullptr, nullptr, nullptr);
  ceil_u = wave_max(ceil_u);
  if (lane == 0) ncand = 0;
  __syncthreads();
  bool ok = tau > -INFINITY && ceil_u < tau;
  // candidates: emitted keys whose upper bound reaches tau
  if (ok) {
    for (int64_t sl = lane; sl < slices; sl += 64) {
      const int64_t cell = (rg * slices + sl) * 32 + q32;
      for (int k = 0; k < topk; ++k) {
        const float s = cand_l[cell * topk + k];
        if (!(s > -INFINITY)) break;
        const int i = cand_i[cell * topk + k];
        const float bk = fmaf(norms[seq * n + i], eM, QJL ? gammas[seq * n + i] * eQ : 0.f);
        float up = fmaf(2.f, bk, s);
        up += fabsf(up) * 0x1p-20f;
        if (up >= tau) {
          const int pos = atomicAdd(&ncand, 1);
          if (pos < kLbCand) cand[pos] = i;
        }
      }
    }
  }
  __syncthreads();
  const int nc = ncand;
  if (nc > kLbCand) ok = false;
  if (lane == 0) flags[bh] = ok ? 0 : 1;
  if (!ok) return;   // uniform

  // exact scores: the exact scan's operands and arithmetic, 16 candidates
  // per round, the query's rows 4 qi .. 4 qi + 3 on lanes 16 qi .. 16 qi + 15
  const int jj = lane & 15, g = lane >> 4;
  v8i A[T][C];
  {
    const v8i* ap = reinterpret_cast<const v8i*>(wsA + gy * T * C * 2048);
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int c = 0; c < C; ++c) A[t][c] = ap[(t * C + c) * 64 + lane];
  }
  float cs[10];
  {
    const float* cp = wsC + (gy * 4 + g) * 16;
#pragma unroll
    for (int i = 0; i < 10; ++i) cs[i] = cp[i];
  }
  list_init<KK>(ls, li);
  for (int c0 = 0; c0 < nc; c0 += 16) {
    const bool cv = c0 + jj < nc;
    const int key = cand[cv ? c0 + jj : 0];
    const uint32_t* kw = codes + (seq * n + key) * WPK;
    v4f aM = {0.f, 0.f, 0.f, 0.f}, aQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int gg = 4 * c + g;
      uint32_t w[5] = {0u, 0u, 0u, 0u, 0u};
      if (gg < GW) {
#pragma unroll
        for (int p = 0; p < W; ++p) w[p] = kw[gg * W + p];
      }
#pragma unroll
      for (int t = 0; t < (1 << (BP - 1)); ++t)
        aM = mfma_fp8_fp4(A[t][c], key_bits_to_fp4(walsh_word<BP>(w, t)), aM);
      if constexpr (QJL) aQ = mfma_fp8_fp4(A[T - 1][c], key_bits_to_fp4(w[BP]), aQ);
    }
    pin(aM);
    const float mse = fmaf(aM[0], cs[2], fmaf(aM[1], cs[3], fmaf(aM[2], cs[4], fmaf(aM[3], cs[5], cs[0]))));
    const float kn = norms[seq * n + key];
    float s = kn * mse;
    if constexpr (QJL) {
      pin(aQ);
      const float qjl = fmaf(aQ[0], cs[6], fmaf(aQ[1], cs[7], fmaf(aQ[2], cs[8], fmaf(aQ[3], cs[9], cs[1]))));
      s = fmaf(kn, mse, gammas[seq * n + key] * qjl);
    }
    if (cv && g == qi && ranks_before(s, key, ls[KK - 1], li[KK - 1])) list_insert<KK>(s, key, ls, li);
  }
  tournament<KK, 16>(ls, li, topk, lane == 16 * qi, out + bh * topk, nullptr, out_idx + bh * topk);
}

// the bounded scan and its merge for one (BP, GW, QJL), where the operands fit
template <int BPV, int GWV, bool QV>
static hipError_t launch_topk_bounded(const TopkPlan& pl, const uint32_t* codes, const float* norms,
                                      const float* gammas, int64_t n, int B, int Hq, int Hkv, int topk,
                                      const uint8_t* wsA, const float* wsC, float* ll, int* lix, float* lc, float* out,
                                      int64_t* out_idx, uint8_t* flags, hipStream_t st) {
  constexpr int T = (1 << (BPV - 1)) + (QV ? 1 : 0);
  if constexpr (T * ((GWV + 3) / 4) > 10) {
    return hipErrorNotSupported;
  } else {
    const int64_t blocks = (pl.slices + 7) / 8 * 8 * pl.rg_count;
    if (blocks > 0x7fffffff) return hipErrorNotSupported;
    // 10-entry lists where they hold k (fewer registers, cheaper insertions)
    if (topk <= 10)
      hipLaunchKernelGGL((topk_lb_scan_kernel<BPV, GWV, QV, 10>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                         codes, norms, gammas, n, pl.RT, pl.rg_per_seq, pl.rg_count, pl.slices, pl.slice_keys, topk,
                         wsA, wsC, ll, lix, lc);
    else
      hipLaunchKernelGGL((topk_lb_scan_kernel<BPV, GWV, QV, 12>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                         codes, norms, gammas, n, pl.RT, pl.rg_per_seq, pl.rg_count, pl.slices, pl.slice_keys, topk,
                         wsA, wsC, ll, lix, lc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((topk_lb_merge_kernel<BPV, GWV, QV>), dim3(static_cast<unsigned>(static_cast<int64_t>(B) * Hq)),
                       dim3(64), 0, st, codes, norms, gammas, n, Hq, Hkv, pl.RT, pl.rg_per_seq, pl.slices, topk, wsA,
                       wsC, ll, lix, lc, out, out_idx, flags);
    return hipGetLastError();
  }
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
  const bool bounded = topk_bounded(q, topk);
  const TopkLayout lay = topk_layout(q, B, Hq, Hkv, n, topk);
  hipError_t e = launch_query_prep_ws(q, queries, q_dtype, B, Hq, Hkv, ws, st, bounded);
  if (e != hipSuccess) return e;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  const uint8_t* wsA = w8;
  const float* wsC = reinterpret_cast<const float*>(wsA + row_tiles * T * Cc * 2048);
  float* cs = reinterpret_cast<float*>(w8 + lay.exact_cand);
  int* ci = reinterpret_cast<int*>(cs + p.rg_count * p.slices * 16 * topk);
  const int bp = key_codebook(q).bp;
  const bool qjl = key_qjl(q);
  const int gw = (q->d + 31) / 32;
  // Bounded search first; the exact scan and merge below then run only for
  // the queries it flags (their workgroups and waves exit at once otherwise)
  uint8_t* flags = nullptr;
  if (bounded) {
    const TopkPlan pl = topk_lb_plan(B, Hq, Hkv, n);
    float* ll = reinterpret_cast<float*>(w8 + lay.lb_cand);
    int* lix = reinterpret_cast<int*>(ll + pl.rg_count * pl.slices * 32 * topk);
    float* lc = reinterpret_cast<float*>(w8 + lay.lb_ceil);
    uint8_t* fl = w8 + lay.flags;
    e = hipErrorNotSupported;
    bool matched = false;
#define TQ_LB(BPV, GWV, QV)                                                                                   \
  if (!matched && bp == BPV && gw == GWV && qjl == QV) {                                                      \
    matched = true;                                                                                           \
    e = launch_topk_bounded<BPV, GWV, QV>(pl, codes, norms, gammas, n, B, Hq, Hkv, topk, wsA, wsC, ll, lix, lc, \
                                          out, out_idx, fl, st);                                              \
  }
#define TQ_LB_ALL(GWV)                                                                                  \
  TQ_LB(1, GWV, true) TQ_LB(2, GWV, true) TQ_LB(3, GWV, true) TQ_LB(1, GWV, false) TQ_LB(2, GWV, false) \
  TQ_LB(3, GWV, false) TQ_LB(4, GWV, false)
    TQ_LB_ALL(1) TQ_LB_ALL(2) TQ_LB_ALL(3) TQ_LB_ALL(4) TQ_LB_ALL(5) TQ_LB_ALL(6) TQ_LB_ALL(7) TQ_LB_ALL(8)
#undef TQ_LB_ALL
#undef TQ_LB
    if (e == hipSuccess) flags = fl;
    else if (e != hipErrorNotSupported) return e;
  }
  // per-lane list length: the shortest of 12, 16, 32 that holds k entries
  // (the insertion cost grows with it)
  const int kk = topk <= 12 ? 12 : (topk <= 16 ? 16 : 32);
  bool launched = false;
#define TQ_TK_L(BPV, GWV, KKV, QV)                                                                              \
  hipLaunchKernelGGL((topk_scan_kernel<BPV, GWV, KKV, QV>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, \
                     codes, norms, gammas, n, p.RT, p.rg_per_seq, p.rg_count, p.slices, p.slice_keys, topk, wsA, wsC,   \
                     cs, ci, flags, Hq, Hkv)
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
                       out, out_idx, flags);
  else if (kk == 16)
    hipLaunchKernelGGL((topk_merge_kernel<16>), mgrid, dim3(64), 0, st, cs, ci, p.slices, Hq, Hkv, p.rg_per_seq, topk,
                       out, out_idx, flags);
  else
    hipLaunchKernelGGL((topk_merge_kernel<12>), mgrid, dim3(64), 0, st, cs, ci, p.slices, Hq, Hkv, p.rg_per_seq, topk,
                       out, out_idx, flags);
  return hipGetLastError();
}

}  // namespace tq
