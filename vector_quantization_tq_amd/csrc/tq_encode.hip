// Encode and decode kernels.
//
// Encode follows the two stages on the pages (blog.hotdry.top "TurboQuant
// vector-search compression", random rotation + scalar quantisation and QJL
// residual correction sections; a2a-mcp.org "什麼是TurboQuant？", stage 1
// and stage 2): n = ||x||, y = Pi x / n, nearest Lloyd-Max centroid per
// coordinate, rho = y - c[idx], gamma = n ||rho||, QJL bits = sign(S' rho)
// with S' = S Pi^T (so S' rho = S r / n for the residual r = x - x_hat).
//
// Both products by a d x d matrix run on the fp32 MFMA (16x16x4): the code
// decisions are taken on fp32-accurate values.  One workgroup encodes a tile
// of 64 vectors; each of its 4 waves owns 16 vectors (rows) and all output
// columns, so a wave only ever reads back its own rows from LDS.
#include <algorithm>

#include "tq_device.h"
#include "tq_kernels.h"

namespace tq {

namespace {

constexpr int kTileRows = 64;
constexpr int kThreads = 256;

// Y[16 rows of this wave][DP] = X[rows][0:d] * M^T, with M given k-major:
// Mt[k * ldm + j] = M[j][k] (row j of M gives output column j), so that the
// 16 lanes of a column tile read 16 consecutive floats.  X in LDS with row
// stride `ld`.  acc[ct] holds output column tile ct (16 columns) in MFMA C
// layout.
// acc[rt][j] = rows 16 rt .. 16 rt + 15 of xs (64 rows, row stride ld) times
// column tile ct = w + 4 j of the k-major matrix Mt (column j of the product
// = row j of the matrix), for the column tiles ct < NT that wave w owns.  The
// 16x16x4 fp32 MFMA: lane (r, kq) holds A[row r][k0 + kq] and B[k0 + kq][col
// r]; each matrix load feeds the four row tiles, and no two waves load the
// same matrix elements.
template <int NT, int NTW>
__device__ __forceinline__ void gemm_tile64(const float* xs, int ld, const float* __restrict__ Mt, int ldm, int rows_m,
                                           int d, int w, v4f (&acc)[4][NTW]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[rt][j] = (v4f){0.f, 0.f, 0.f, 0.f};
  // Loads at clamped (always valid) addresses and no branches around the
  // loads or the MFMAs.  Only A is zeroed past k = d (a select on the LDS
  // value); B is not masked: a product column past d (or a column tile past
  // NT) holds values that nothing reads.
  int colc[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) colc[j] = min((w + 4 * j) * 16 + r, rows_m - 1);
  for (int k0 = 0; k0 < d; k0 += 4) {
    const int k = k0 + kq;
    const bool kin = k < d;
    const int kc = min(k, d - 1);
    float b[NTW], a[4];
#pragma unroll
    for (int j = 0; j < NTW; ++j) b[j] = Mt[static_cast<int64_t>(kc) * ldm + colc[j]];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const float v = xs[(16 * rt + r) * ld + kc];
      a[rt] = kin ? v : 0.f;
    }
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt][j] = mfma_f32(a[rt], b[j], acc[rt][j]);
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int j = 0; j < NTW; ++j) pin(acc[rt][j]);
}

template <int NT>
__global__ void __launch_bounds__(kThreads) encode_kernel(const void* __restrict__ x, int dtype, int64_t n, int d, int mode,
                                                          const float* __restrict__ pit, int ldp,
                                                          const float* __restrict__ spt,
                                                          Codebook cb, uint32_t* __restrict__ codes,
                                                          float* __restrict__ norms, float* __restrict__ gammas) {
  constexpr int DP = NT * 16;
  constexpr int LD = DP + 1;
  constexpr int NTW = (NT + 3) / 4;   // column tiles per wave
  extern __shared__ float smem[];
  float* xs = smem;                                               // [64][LD] floats: x, then rho
  float* nrm = xs + kTileRows * LD;                               // [64]
  float* cen = nrm + kTileRows;                                   // [16]
  uint8_t* idxb = reinterpret_cast<uint8_t*>(cen + kMaxLevels);   // [64][DP]
  uint8_t* sgnb = idxb + kTileRows * DP;                          // [64][DP]
  __shared__ float part2[4][kTileRows];                           // per wave: partial ||rho||^2 of each row

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int64_t seq = blockIdx.y;
  const int64_t v0 = static_cast<int64_t>(blockIdx.x) * kTileRows;
  const int rows = static_cast<int>(n - v0 < kTileRows ? n - v0 : kTileRows);
  const int64_t base = seq * n + v0;   // first vector of the tile

  if (tid < kMaxLevels) cen[tid] = tid < cb.levels ? cb.c[tid] : 0.f;
  // ---- load the tile, zero rows past n and columns past d ----
  if (dtype == 0 && (d & 3) == 0) {   // fp32 rows of whole 16-byte chunks
    // four threads per row, 16-byte chunks c = part, part + 4, ...: every
    // load of a thread is issued before the first store
    constexpr int CPT = (DP / 4 + 3) / 4;   // chunks per thread
    const int row = tid >> 2, part = tid & 3, cpr = d >> 2;
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(x) + (base + row) * d);
    float4 v[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = part + 4 * u;
      v[u] = (row < rows && c < cpr) ? src[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = part + 4 * u;
      if (4 * c < DP) {
        float* dst = xs + row * LD + 4 * c;
        dst[0] = v[u].x;
        dst[1] = v[u].y;
        dst[2] = v[u].z;
        dst[3] = v[u].w;
      }
    }
  } else {
    for (int e = tid; e < kTileRows * DP; e += kThreads) {
      const int row = e / DP, col = e - row * DP;
      float v = 0.f;
      if (row < rows && col < d) v = load_elem(x, dtype, (base + row) * d + col);
      xs[row * LD + col] = v;
    }
  }
  __syncthreads();
  // ---- norms: 4 threads per row ----
  {
    const int row = tid >> 2, part = tid & 3;
    float s = 0.f;
    for (int col = part; col < d; col += 4) {
      const float v = xs[row * LD + col];
      s = fmaf(v, v, s);
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (part == 0) nrm[row] = sqrtf(s);
  }
  __syncthreads();

  // ---- rotation: y = Pi x / n; wave w takes column tiles w, w + 4, ... of all 64 rows ----
  v4f acc[4][NTW];
  gemm_tile64<NT, NTW>(xs, LD, pit, ldp, d, d, wave, acc);

  const int col_in = lane & 15, rq = lane >> 4;   // C layout: rows 16 rt + 4 rq + i, column 16 ct + col_in
  float inv_n[4][4], rho2[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float nv = nrm[16 * rt + 4 * rq + i];
      inv_n[rt][i] = nv > 0.f ? 1.f / nv : 0.f;
      rho2[rt][i] = 0.f;
    }
  const int kh = cb.levels >> 1;   // centroids per half of the codebook
  // bucketize, residual (rho stays in acc until every wave has read x)
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int col = (wave + 4 * j) * 16 + col_in;
    if (wave + 4 * j < NT) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * rt + 4 * rq + i;
          const float y = acc[rt][j][i] * inv_n[rt][i];
          // idx = #{t_k < y} on the symmetric codebook (middle threshold 0,
          // t[K/2 + k] = -t[K/2 - 2 - k]): K/2 + j for y > 0, K/2 - 1 - j
          // otherwise, j = #{positive thresholds below |y|}
          const float ay = fabsf(y);
          int jm = 0;
#pragma unroll
          for (int k = 0; k + 1 < kMaxLevels / 2; ++k)
            if (k + 1 < kh) jm += (cb.t[kh + k] < ay) ? 1 : 0;
          const int idx = y > 0.f ? kh + jm : kh - 1 - jm;
          const float rho = col < d ? y - cen[idx] : 0.f;
          rho2[rt][i] = fmaf(rho, rho, rho2[rt][i]);
          idxb[row * DP + col] = col < d ? static_cast<uint8_t>(idx) : 0;
          acc[rt][j][i] = rho;
        }
    }
  }
  __syncthreads();   // all waves finished reading x before rho overwrites it
#pragma unroll
  for (int j = 0; j < NTW; ++j)
    if (wave + 4 * j < NT) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) xs[(16 * rt + 4 * rq + i) * LD + (wave + 4 * j) * 16 + col_in] = acc[rt][j][i];
    }

  if (mode == 0) {
    // this wave's part of ||rho||^2 per row (a sum over its 16 column lanes)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sum = rho2[rt][i];
        sum += __shfl_xor(sum, 1);
        sum += __shfl_xor(sum, 2);
        sum += __shfl_xor(sum, 4);
        sum += __shfl_xor(sum, 8);
        if (col_in == 0) part2[wave][16 * rt + 4 * rq + i] = sum;
      }
    __syncthreads();
    // ---- QJL projection z = S' rho; bit = [z >= 0] (all ones for n = 0) ----
    gemm_tile64<NT, NTW>(xs, LD, spt, d, d, d, wave, acc);
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int col = (wave + 4 * j) * 16 + col_in;
      if (wave + 4 * j < NT) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * rt + 4 * rq + i;
            const bool bit = (acc[rt][j][i] >= 0.f) || (inv_n[rt][i] == 0.f);
            sgnb[row * DP + col] = (col < d && bit) ? 1 : 0;
          }
      }
    }
    if (tid < rows) {
      const float nv = nrm[tid];
      norms[base + tid] = nv;
      gammas[base + tid] = nv * sqrtf((part2[0][tid] + part2[1][tid]) + (part2[2][tid] + part2[3][tid]));
    }
  } else {
    if (tid < rows) norms[base + tid] = nrm[tid];
  }
  __syncthreads();

  // ---- bit packing ----
  const int bp = cb.bp;
  if (mode != 1) {
    // keys: words [vec][g][W], W = bp + 1 with the QJL plane, bp without
    const int G = (d + 31) >> 5;
    const int W = bp + (mode == 0 ? 1 : 0);
    for (int task = tid; task < kTileRows * G; task += kThreads) {
      const int row = task / G, g = task - row * G;
      if (row >= rows) continue;
      uint32_t w[5] = {0u, 0u, 0u, 0u, 0u};
      const uint8_t* ib = idxb + row * DP + 32 * g;
      const uint8_t* sb = sgnb + row * DP + 32 * g;
      for (int i = 0; i < 32; ++i) {
        if (32 * g + i >= DP) break;
        const uint32_t iv = ib[i];
        for (int p = 0; p < bp; ++p) w[p] |= ((iv >> p) & 1u) << i;
        if (mode == 0) w[bp] |= static_cast<uint32_t>(sb[i]) << i;
      }
      uint32_t* out = codes + ((base + row) * G + g) * W;
      for (int p = 0; p < W; ++p) out[p] = w[p];
    }
  } else {
    // mse: words [seq][blk][bp][d]; this tile holds blocks 2*bx and 2*bx+1
    const int64_t nb = (n + 31) >> 5;
    for (int task = tid; task < 2 * d; task += kThreads) {
      const int half = task / d, j = task - half * d;
      const int64_t blk = (v0 >> 5) + half;
      if (blk >= nb) continue;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      for (int i = 0; i < 32; ++i) {
        const int row = 32 * half + i;
        if (row >= rows) break;
        const uint32_t iv = idxb[row * DP + j];
        for (int p = 0; p < bp; ++p) w[p] |= ((iv >> p) & 1u) << i;
      }
      uint32_t* out = codes + ((seq * nb + blk) * bp) * d + j;
      for (int p = 0; p < bp; ++p) out[static_cast<int64_t>(p) * d] = w[p];
    }
  }
}

// ---------------------------------------------------------------------------
// Tile encoder for d <= 128 (the head dimensions of attention caches), on the
// fp16 16x16x32 MFMA with split operands.
//
// The matrix core accumulates fp16 products at fp32 accuracy, so a float
// operand written as hi + lo (two fp16 numbers, 22 significant bits)
// reproduces a float product to about 2^-22.  The rotation is
// x . (Pi_hi + Pi_lo) (bf16 keys are exact in fp16 after a power-of-two row
// scale; fp32 keys add x_lo . Pi_hi), the QJL projection is
// rho_hi . S'_hi + rho_lo . S'_hi + rho_hi . S'_lo.  Pi is scaled by 2^8 and
// rho by 2^14 before splitting so that the lo parts stay normal numbers.
//
// Wave w owns the 32-coordinate group w: its rows of Pi_hi/lo and S'_hi/lo
// stay in registers as B operands for the whole kernel; the x (or rho) tile
// sits once in LDS for all four waves, and each lane reads its 8 consecutive
// contraction values as one 16-byte load.  Workgroups are persistent over
// 64-vector tiles and fetch the next tile into registers while the current
// one is encoded.
//
// prod (keys): C[vector][coordinate]; an index bit plane of 16 coordinates of
// 4 vectors is one ballot, so a packed word is assembled from two ballots.
// mse (values): the operands are swapped, C[coordinate][vector], so a ballot
// gives 16 tokens of 4 coordinates: the token-major value words come out the
// same way.
// ---------------------------------------------------------------------------
constexpr int kEncRows = 64;
constexpr float kPiScale = 256.f;       // 2^8
constexpr float kRhoScale = 16384.f;    // 2^14

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// rs - hh rounded once to fp16, for hh = rs rounded to fp16 (so rs - hh is
// exact in fp32): v_fma_mixlo_f16 reads hh as an fp16 source and rs as fp32
// (one instruction in place of a convert, a subtract and a convert)
__device__ __forceinline__ _Float16 f16_remainder(float rs, _Float16 hh) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(hh), "v"(rs));
  return __builtin_bit_cast(_Float16, static_cast<uint16_t>(r));
}

__device__ __forceinline__ v4f mfma_f16(const v8h& a, const v8h& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Binary search of the sorted thresholds: bit L of idx = #{t_k < y} is
// decided by one comparison against the threshold that splits the cells
// still possible, picked from the candidates by the bits above L with
// branch-free selects.  Each comparison is also that bit plane's lane mask.
template <int BP, int L>
__device__ __forceinline__ float pick_threshold(const float (&th)[(1 << BP) - 1], const bool (&bit)[BP]) {
  constexpr int NC = 1 << (BP - 1 - L);
  float c[NC];
#pragma unroll
  for (int u = 0; u < NC; ++u) c[u] = th[u * (2 << L) + (1 << L) - 1];
#pragma unroll
  for (int j = 0; (1 << j) < NC; ++j)
#pragma unroll
    for (int u = 0; u < (NC >> (j + 1)); ++u) c[u] = bit[L + 1 + j] ? c[2 * u + 1] : c[2 * u];
  return c[0];
}

template <int BP, int L>
__device__ __forceinline__ void decide_bits(float y, const float (&th)[(1 << BP) - 1], bool (&bit)[BP]) {
  bit[L] = pick_threshold<BP, L>(th, bit) < y;
  if constexpr (L > 0) decide_bits<BP, L - 1>(y, th, bit);
}

// c[idx] from the bits, by a select tree over the 2^BP centroids
template <int BP>
__device__ __forceinline__ float pick_centroid(const float (&cen)[1 << BP], const bool (&bit)[BP]) {
  float c[1 << BP];
#pragma unroll
  for (int u = 0; u < (1 << BP); ++u) c[u] = cen[u];
#pragma unroll
  for (int j = 0; j < BP; ++j)
#pragma unroll
    for (int u = 0; u < ((1 << BP) >> (j + 1)); ++u) c[u] = bit[j] ? c[2 * u + 1] : c[2 * u];
  return c[0];
}

// LK: how a tile is loaded: 0 element by element (any d, either dtype),
// 1 bf16 and 2 fp32 in 16-byte chunks fetched one tile ahead.  BP: index
// bits.  MODE: 0 keys with the QJL sketch (token-major words + rho, gamma),
// 1 values (coordinate-major 32-token words), 2 MSE-only keys (token-major
// words, no QJL plane).  FULL: d == 32 KS, so every wave owns 32 existing
// coordinates and the coordinate guards compile away.
template <int KS, int LK, int MODE, int BP, bool FULL>
__global__ void __launch_bounds__(256, 2) encode_tile_kernel(const void* __restrict__ x, int dtype, int64_t nseq,
                                                             int64_t n, int d, const float* __restrict__ pi,
                                                             const float* __restrict__ sp, Codebook cb,
                                                             uint32_t* __restrict__ codes, float* __restrict__ norms,
                                                             float* __restrict__ gammas) {
  constexpr bool PROD = MODE != 1;       // token-major words, C[vector][coordinate]
  constexpr bool QJL = MODE == 0;        // residual, QJL plane and gamma
  constexpr int KP = 32 * KS;            // padded contraction length
  constexpr int LDH = KP + 8;            // LDS row stride in halves (16-byte rows, conflict-free reads)
  constexpr bool XLO = LK != 1;          // fp32 keys need x_lo (bf16 keys are exact in fp16)
  constexpr int PREN = LK == 2 ? KS * 2 : LK == 1 ? KS : 1;   // 16-byte chunks per loader thread
  constexpr int EPT = KP / 4;            // elements per loader thread (scalar path)
  __shared__ __attribute__((aligned(16))) _Float16 xh[kEncRows * LDH];
  __shared__ __attribute__((aligned(16))) _Float16 xl[XLO ? kEncRows * LDH : 8];
  __shared__ __attribute__((aligned(16))) _Float16 rh[QJL ? kEncRows * LDH : 8];
  __shared__ __attribute__((aligned(16))) _Float16 rl[QJL ? kEncRows * LDH : 8];
  __shared__ __attribute__((aligned(16))) float scl2[2][kEncRows];   // 2^(6 - row scale) / n, by tile parity
  __shared__ float nrm2[2][kEncRows];    // n, by tile parity
  __shared__ float part2[4][kEncRows];
  __shared__ uint32_t ost[2][1024];

  static_assert(KS == 4, "four waves own 32 coordinates each");
  if constexpr (FULL) d = 32 * KS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int r16 = lane & 15, q = lane >> 4;
  constexpr int bp = BP;
  constexpr int NT = (1 << BP) - 1;      // thresholds
  const int G = (d + 31) >> 5;
  const int W = bp + (QJL ? 1 : 0);      // token-major words per group
  const int WPK = G * W;
  const int64_t tps = (n + kEncRows - 1) / kEncRows;   // tiles per sequence
  const int64_t total = nseq * tps;
  const int64_t nb = (n + 31) >> 5;                      // mse blocks per sequence

  // stationary operands: lane (r16, q) holds row 32w + 16ct + r16, columns
  // 32s + 8q .. +7 of Pi (and S'), split into hi + lo
  v8h bPh[2][KS], bPl[2][KS], bSh[2][QJL ? KS : 1], bSl[2][QJL ? KS : 1];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int j = 32 * w + 16 * ct + r16;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = 32 * s2 + 8 * q + e;
        const bool in = j < d && k < d;
        const float vp = in ? pi[static_cast<int64_t>(j) * d + k] * kPiScale : 0.f;
        const _Float16 ph = static_cast<_Float16>(vp);
        bPh[ct][s2][e] = ph;
        bPl[ct][s2][e] = static_cast<_Float16>(vp - static_cast<float>(ph));
        if constexpr (QJL) {
          const float vs = in ? sp[static_cast<int64_t>(j) * d + k] * kPiScale : 0.f;
          const _Float16 sh = static_cast<_Float16>(vs);
          bSh[ct][s2][e] = sh;
          bSl[ct][s2][e] = static_cast<_Float16>(vs - static_cast<float>(sh));
        }
      }
  }
  for (int e = tid; e < kEncRows * LDH; e += 256) {
    xh[e] = static_cast<_Float16>(0.f);
    if constexpr (XLO) xl[e] = static_cast<_Float16>(0.f);
    if constexpr (QJL) {
      rh[e] = static_cast<_Float16>(0.f);
      rl[e] = static_cast<_Float16>(0.f);
    }
  }

  // loader role: row = tid / 4, four threads per row
  const int lrow = tid >> 2, part = tid & 3;
  constexpr int esz = LK == 1 ? 2 : 4;
  const int CH = d * esz / 16;           // 16-byte chunks per row (vector paths)
  uint4 pre[PREN];
  // tile t = seq * tps + r; the loop steps t by the grid size, so the next
  // tile's (seq, r) comes from the current one without a division in the
  // common cases
  struct TileAt { int64_t seq, r; };
  auto advance = [&](TileAt a) {
    a.r += gridDim.x;
    if (a.r >= tps) {
      if (a.r < 2 * tps) {
        a.r -= tps;
        ++a.seq;
      } else {
        const int64_t k = a.r / tps;
        a.seq += k;
        a.r -= k * tps;
      }
    }
    return a;
  };
  auto tile_of = [&](TileAt a, int64_t& seq, int64_t& v0, int& rows) {
    seq = a.seq;
    v0 = a.r * kEncRows;
    rows = static_cast<int>(min(static_cast<int64_t>(kEncRows), n - v0));
  };
  auto fetch = [&](TileAt t) {
    if constexpr (LK != 0) {
      int64_t seq, v0;
      int rows;
      tile_of(t, seq, v0, rows);
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(x) +
                                                        ((seq * n + v0 + lrow) * d) * esz);
#pragma unroll
      for (int j = 0; j < PREN; ++j) {
        const int c = part + 4 * j;
        pre[j] = make_uint4(0u, 0u, 0u, 0u);   // rows past n and chunks past d read as 0
        if (lrow < rows && c < CH) pre[j] = src[c];
      }
    }
  };
  // element e of this thread's share of the row (column col(e)), as float
  auto commit = [&](TileAt t, float* scl, float* nrm) {
    int64_t seq, v0;
    int rows;
    tile_of(t, seq, v0, rows);
    float v[EPT];
    int cols[EPT];
    int cnt = 0;
    if constexpr (LK == 1) {
#pragma unroll
      for (int j = 0; j < PREN; ++j) {
        const int c = part + 4 * j;
        const uint32_t u[4] = {pre[j].x, pre[j].y, pre[j].z, pre[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[8 * j + 2 * e] = __uint_as_float(u[e] << 16);
          v[8 * j + 2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
          cols[8 * j + 2 * e] = 8 * c + 2 * e;
          cols[8 * j + 2 * e + 1] = 8 * c + 2 * e + 1;
        }
      }
      cnt = EPT;
    } else if constexpr (LK == 2) {
#pragma unroll
      for (int j = 0; j < PREN; ++j) {
        const int c = part + 4 * j;
        const uint32_t u[4] = {pre[j].x, pre[j].y, pre[j].z, pre[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[4 * j + e] = __uint_as_float(u[e]);
          cols[4 * j + e] = 4 * c + e;
        }
      }
      cnt = EPT;
    } else {
      const int64_t off = (seq * n + v0 + lrow) * d;
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const int col = part + 4 * j;
        v[j] = (lrow < rows && col < d) ? load_elem(x, dtype, off + col) : 0.f;
        cols[j] = col;
      }
      cnt = EPT;
    }
    float ss = 0.f, mx = 0.f;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      ss = fmaf(v[j], v[j], ss);
      mx = fmaxf(mx, fabsf(v[j]));
    }
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    // power-of-two row scale putting the largest element in [2^14, 2^15)
    const int sig = mx > 0.f ? 14 - ilogb_pos(mx) : 0;
    _Float16* hr = xh + lrow * LDH;
    _Float16* lr = xl + lrow * LDH;
    if constexpr (LK == 1) {
      // a 16-byte chunk of 8 bf16 values becomes one 16-byte row segment
#pragma unroll
      for (int j = 0; j < PREN; ++j) {
        const int c = part + 4 * j;
        if (c < CH) {
          v8h hv;
#pragma unroll
          for (int e = 0; e < 8; ++e) hv[e] = static_cast<_Float16>(ldexpf(v[8 * j + e], sig));
          *reinterpret_cast<v8h*>(hr + 8 * c) = hv;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        if (j < cnt && cols[j] < d) {
          const float sv = ldexpf(v[j], sig);
          const _Float16 h = static_cast<_Float16>(sv);
          hr[cols[j]] = h;
          if constexpr (XLO) lr[cols[j]] = static_cast<_Float16>(sv - static_cast<float>(h));
        }
      }
    }
    if (part == 0) {
      const float nv = lrow < rows ? sqrtf(ss) : 0.f;
      nrm[lrow] = nv;
      // y 2^14 = acc * scl: the rotation of u, times 2^14 (Pi carries 2^8, the row 2^sig)
      scl[lrow] = nv > 0.f ? ldexpf(1.f / nv, 6 - sig) : 0.f;
    }
  };
  auto store = [&](TileAt t, int buf) {
    int64_t seq, v0;
    int rows;
    tile_of(t, seq, v0, rows);
    if constexpr (PROD) {
      uint32_t* dst = codes + (seq * n + v0) * WPK;
      for (int e = tid; e < rows * WPK; e += 256) dst[e] = ost[buf][e];
    } else {
      const int nblk = (rows + 31) >> 5;
      uint32_t* dst = codes + ((seq * nb + (v0 >> 5)) * bp) * d;
      for (int e = tid; e < nblk * bp * d; e += 256) dst[e] = ost[buf][e];
    }
  };
  // acc[h2][ct] (+)= rows 32h + 16h2 .. of src times this wave's columns;
  // SWAP puts the stationary operand first (C[coordinate][vector])
  auto contract = [&](const _Float16* src, const v8h (&bm)[2][KS], int h, bool swap, v4f (&acc)[2][2]) {
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      v8h a[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        a[h2] = *reinterpret_cast<const v8h*>(src + (32 * h + 16 * h2 + r16) * LDH + 32 * s2 + 8 * q);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          acc[h2][ct] = swap ? mfma_f16(bm[ct][s2], a[h2], acc[h2][ct]) : mfma_f16(a[h2], bm[ct][s2], acc[h2][ct]);
    }
  };
  auto zero_acc = [&](v4f (&acc)[2][2]) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) acc[h2][ct] = (v4f){0.f, 0.f, 0.f, 0.f};
  };
  auto pin_acc = [&](v4f (&acc)[2][2]) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) pin(acc[h2][ct]);
  };
  // packed word of row 4q + i of a ballot pair (low 16 bits, high 16 bits)
  auto halves = [&](uint64_t m0, uint64_t m1) {
    // bytes 0-1 of m0 >> 16q, then bytes 0-1 of m1 >> 16q (one byte permute)
    return __builtin_amdgcn_perm(static_cast<uint32_t>(m1 >> (16 * q)), static_cast<uint32_t>(m0 >> (16 * q)),
                                 0x05040100u);
  };
  // The codebook is symmetric (the middle threshold is 0 and c[K-1-i] = -c[i]
  // exactly), so idx = #{t_k < y} is K/2 + j for y > 0 and K/2 - 1 - j
  // otherwise, with j = #{positive t_k < |y|}: the top bit is the sign and the
  // low bits are j, complemented for y <= 0.  Only the positive halves of the
  // tables are kept; the centroids pre-scaled for the residual.
  constexpr int KH = 1 << (BP - 1);      // centroids per half
  float thp[KH > 1 ? KH - 1 : 1], cenS[KH];
#pragma unroll
  for (int k2 = 0; k2 + 1 < KH; ++k2) thp[k2] = cb.t[KH + k2] * kRhoScale;   // compared with y 2^14
#pragma unroll
  for (int k2 = 0; k2 < KH; ++k2) cenS[k2] = cb.c[KH + k2] * kRhoScale;
  // sign and magnitude bits of y from a (the accumulator, y 2^14 = a * scl):
  // pos = [y > 0] = [a > 0] (the scale is positive, or 0 with a = 0), jb =
  // bits of j from |y 2^14| against the thresholds times 2^14 (power-of-two
  // scaling: the same decisions)
  auto classify = [&](float a, float ys, bool& pos, bool (&jb)[BP > 1 ? BP - 1 : 1]) {
    pos = a > 0.f;
    if constexpr (BP > 1) decide_bits<BP - 1, BP - 2>(fabsf(ys), thp, jb);
    else jb[0] = false;
  };
  // lanes whose coordinate exists (token-major layouts): 32w + 16ct + r16 < d
  const uint64_t okm0 = FULL ? ~0ull : __ballot(32 * w + r16 < d);
  const uint64_t okm1 = FULL ? ~0ull : __ballot(32 * w + 16 + r16 < d);

  int64_t t = blockIdx.x;
  TileAt cur = {static_cast<int64_t>(blockIdx.x) / tps, static_cast<int64_t>(blockIdx.x) % tps}, prev = cur;
  if (t < total) fetch(cur);
  __syncthreads();   // zero fill done before the first commit
  int it = 0;
  for (; t < total; t += gridDim.x, ++it) {
    const int buf = it & 1;
    float* scl = scl2[buf];
    float* nrm = nrm2[buf];
    commit(cur, scl, nrm);
    const TileAt nxt = advance(cur);
    if (t + gridDim.x < total) fetch(nxt);   // in flight while this tile is encoded
    __syncthreads();
    if (it > 0) store(prev, buf ^ 1);

    int64_t seq, v0;
    int rows;
    tile_of(cur, seq, v0, rows);
    prev = cur;
    cur = nxt;

    if constexpr (PROD) {
#pragma unroll 1
      for (int h = 0; h < 2; ++h) {
        v4f acc[2][2];
        zero_acc(acc);
        contract(xh, bPh, h, false, acc);
        contract(xh, bPl, h, false, acc);
        if constexpr (XLO) contract(xl, bPh, h, false, acc);
        pin_acc(acc);
        // lane holds vector 32h + 16h2 + 4q + i, coordinate 32w + 16ct + r16
        float r2v[2][4];   // partial ||rho||^2 (x 2^28) of this lane's two coordinates
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int vbase = 32 * h + 16 * h2 + 4 * q;
          const float4 sc4 = *reinterpret_cast<const float4*>(scl + vbase);   // one LDS read for 4 rows
          const float scv[4] = {sc4.x, sc4.y, sc4.z, sc4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float scS = scv[i];
            // lane masks of the sign and the magnitude bits, taken as soon as
            // each is decided (no per-lane booleans kept alive)
            uint64_t ms[2], mj[2][BP > 1 ? BP - 1 : 1];
            float r2 = 0.f;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
              const int c = 32 * w + 16 * ct + r16;
              const float a = acc[h2][ct][i];
              bool pos, jb[BP > 1 ? BP - 1 : 1];
              classify(a, a * scS, pos, jb);
              ms[ct] = __ballot(pos);
#pragma unroll
              for (int p = 0; p + 1 < BP; ++p) mj[ct][p] = __ballot(jb[p]);
              if constexpr (QJL) {
                // rho * 2^14 = y 2^14 - c[idx] 2^14 in one rounding
                float cabs;
                if constexpr (BP > 1) cabs = pick_centroid<BP - 1>(cenS, jb);
                else cabs = cenS[0];
                const float rs = (FULL || c < d) ? fmaf(a, scS, pos ? -cabs : cabs) : 0.f;
                r2 = fmaf(rs, rs, r2);
                // hi + lo split
                const _Float16 hh = static_cast<_Float16>(rs);   // c < KP: four waves of 32
                rh[(vbase + i) * LDH + c] = hh;
                rl[(vbase + i) * LDH + c] = f16_remainder(rs, hh);
              }
            }
            // plane words: the sign plane is [y > 0], the low planes are
            // [bit of j == sign] (complemented for y <= 0)
            uint32_t wd[BP];
            const uint64_t s0 = ms[0] & okm0, s1 = ms[1] & okm1;
            wd[BP - 1] = halves(s0, s1);
#pragma unroll
            for (int p = 0; p + 1 < BP; ++p) wd[p] = halves(~(mj[0][p] ^ s0) & okm0, ~(mj[1][p] ^ s1) & okm1);
            if constexpr (QJL) r2v[h2][i] = r2;
            if (r16 == 0 && (FULL || w < G)) {
#pragma unroll
              for (int p = 0; p < BP; ++p) ost[buf][(vbase + i) * WPK + w * W + p] = wd[p];
            }
          }
        }
        if constexpr (QJL) {
          // ||rho||^2 over this wave's 32 coordinates: the 8 rows' partial sums
          // reduced over the 16 lanes of a row by a transposing butterfly (each
          // stage halves the values a lane keeps); lane r16 ends with the row
          // 16 b3 + 2 b2 + b0 (bits of r16) of its h2 = b3 half, summed over all
          // 16 lanes, and lanes r16 and r16 ^ 2 hold the same sum
          const bool b3 = (r16 & 8) != 0, b2 = (r16 & 4) != 0, b0 = (r16 & 1) != 0;
          float a4[4], a2[2];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float lo = r2v[0][k], hi = r2v[1][k];
            a4[k] = (b3 ? hi : lo) + dpp_f<0x128>(b3 ? lo : hi);   // partner r16 ^ 8 (row_ror:8)
          }
#pragma unroll
          for (int k = 0; k < 2; ++k)
            a2[k] = (b2 ? a4[k + 2] : a4[k]) + dpp_f<0x141>(b2 ? a4[k] : a4[k + 2]);   // partner r16 ^ 7 (row_half_mirror)
          float t = (b0 ? a2[1] : a2[0]) + dpp_f<0xB1>(b0 ? a2[0] : a2[1]);         // partner r16 ^ 1
          t += dpp_f<0x4E>(t);                                                        // partner r16 ^ 2
          if ((r16 & 2) == 0) part2[w][32 * h + 16 * (b3 ? 1 : 0) + 4 * q + 2 * (b2 ? 1 : 0) + (b0 ? 1 : 0)] = t;
        }
      }
      __syncthreads();   // rho complete; every wave done with the x tile

      // ---- QJL: z = S' rho (scaled), bit = [z >= 0] (all ones for a zero vector) ----
      if constexpr (QJL) {
#pragma unroll 1
        for (int h = 0; h < 2; ++h) {
          v4f acc[2][2];
          zero_acc(acc);
          contract(rh, bSh, h, false, acc);
          contract(rl, bSh, h, false, acc);
          contract(rh, bSl, h, false, acc);
          pin_acc(acc);
          if (FULL || w < G) {
            uint32_t wd[2][4];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const int vbase = 32 * h + 16 * h2 + 4 * q;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const uint64_t zm = __ballot(!(nrm[vbase + i] > 0.f));   // zero vectors: all bits 1
                const uint64_t m0 = (__ballot(acc[h2][0][i] >= 0.f) | zm) & okm0;
                const uint64_t m1 = (__ballot(acc[h2][1][i] >= 0.f) | zm) & okm1;
                wd[h2][i] = halves(m0, m1);
              }
            }
            if (r16 == 0) {
#pragma unroll
              for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < 4; ++i) ost[buf][(32 * h + 16 * h2 + 4 * q + i) * WPK + w * W + bp] = wd[h2][i];
            }
          }
        }
      }
      if (tid < rows) {
        const float nv = nrm[tid];
        norms[seq * n + v0 + tid] = nv;
        if constexpr (QJL)
          gammas[seq * n + v0 + tid] =
              nv * sqrtf(part2[0][tid] + part2[1][tid] + part2[2][tid] + part2[3][tid]) * (1.f / kRhoScale);
      }
    } else {
      // lane holds coordinate 32w + 16ct + 4q + i, token 32h + 16h2 + r16;
      // half h is the 32-token block h of the tile
#pragma unroll 1
      for (int h = 0; h < 2; ++h) {
        v4f acc[2][2];
        zero_acc(acc);
        contract(xh, bPh, h, true, acc);
        contract(xh, bPl, h, true, acc);
        if constexpr (XLO) contract(xl, bPh, h, true, acc);
        pin_acc(acc);
        // lane holds coordinate 32w + 16ct + 4q + i, token 32h + 16h2 + r16
        const float sc0 = scl[32 * h + r16], sc1 = scl[32 * h + 16 + r16];
        const uint64_t tm0 = __ballot(32 * h + r16 < rows), tm1 = __ballot(32 * h + 16 + r16 < rows);
        if (FULL || w < G) {
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int c = 32 * w + 16 * ct + 4 * q + i;
              bool p0, p1, j0[BP > 1 ? BP - 1 : 1], j1[BP > 1 ? BP - 1 : 1];
              classify(acc[0][ct][i], acc[0][ct][i] * sc0, p0, j0);
              classify(acc[1][ct][i], acc[1][ct][i] * sc1, p1, j1);
              // sign plane [y > 0]; low planes [bit of j == sign]; padding tokens 0.
              // Every ballot is taken before the one branch that writes the words.
              const uint64_t s0 = __ballot(p0) & tm0, s1 = __ballot(p1) & tm1;
              uint32_t wd[BP];
#pragma unroll
              for (int p = 0; p < BP; ++p) {
                const uint64_t m0 = p == BP - 1 ? s0 : ~(__ballot(j0[p < BP - 1 ? p : 0]) ^ s0) & tm0;
                const uint64_t m1 = p == BP - 1 ? s1 : ~(__ballot(j1[p < BP - 1 ? p : 0]) ^ s1) & tm1;
                wd[p] = halves(m0, m1);
              }
              if (r16 == 0 && (FULL || c < d)) {
#pragma unroll
                for (int p = 0; p < BP; ++p) ost[buf][(h * bp + p) * d + c] = wd[p];
              }
            }
        }
      }
      if (tid < rows) norms[seq * n + v0 + tid] = nrm[tid];
      __syncthreads();   // every wave is done with the x tile before the next commit
    }
  }
  __syncthreads();
  if (it > 0) store(prev, (it - 1) & 1);
}

// Decode: one workgroup per 8 vectors; plain fp32 FMAs (not on the hot path).
__global__ void __launch_bounds__(256) decode_kernel(const uint32_t* __restrict__ codes, const float* __restrict__ norms,
                                                     const float* __restrict__ gammas, int64_t n, int d, int m, int mode,
                                                     const float* __restrict__ pi, const float* __restrict__ s,
                                                     Codebook cb, float* __restrict__ out) {
  constexpr int V = 8;
  extern __shared__ float sm[];
  float* cv = sm;            // [V][d]   n * c[idx]
  float* sg = cv + V * d;    // [V][m]   gamma * sqrt(pi/2)/m * sigma
  const int tid = threadIdx.x;
  const int64_t seq = blockIdx.y;
  const int64_t v0 = static_cast<int64_t>(blockIdx.x) * V;
  const int bp = cb.bp;
  const float qjl = 1.2533141373155003f / static_cast<float>(m);   // sqrt(pi/2)/m
  for (int e = tid; e < V * d; e += blockDim.x) {
    const int v = e / d, j = e - v * d;
    const int64_t t = v0 + v;
    float val = 0.f;
    if (t < n) {
      uint32_t idx = 0;
      if (mode != 1) {
        const int G = (d + 31) >> 5;
        const uint32_t* w = codes + ((seq * n + t) * G + (j >> 5)) * (bp + (mode == 0 ? 1 : 0));
        for (int p = 0; p < bp; ++p) idx |= ((w[p] >> (j & 31)) & 1u) << p;
      } else {
        const int64_t nb = (n + 31) >> 5;
        const uint32_t* w = codes + ((seq * nb + (t >> 5)) * bp) * d + j;
        for (int p = 0; p < bp; ++p) idx |= ((w[static_cast<int64_t>(p) * d] >> (t & 31)) & 1u) << p;
      }
      val = norms[seq * n + t] * cb.c[idx];
    }
    cv[e] = val;
  }
  if (mode == 0) {
    const int G = (d + 31) >> 5;
    for (int e = tid; e < V * m; e += blockDim.x) {
      const int v = e / m, r = e - v * m;
      const int64_t t = v0 + v;
      float val = 0.f;
      if (t < n) {
        const uint32_t w = codes[((seq * n + t) * G + (r >> 5)) * (bp + 1) + bp];
        val = gammas[seq * n + t] * qjl * (((w >> (r & 31)) & 1u) ? 1.f : -1.f);
      }
      sg[e] = val;
    }
  }
  __syncthreads();
  for (int e = tid; e < V * d; e += blockDim.x) {
    const int v = e / d, i = e - v * d;
    const int64_t t = v0 + v;
    if (t >= n) continue;
    float acc = 0.f;
    for (int j = 0; j < d; ++j) acc = fmaf(pi[static_cast<int64_t>(j) * d + i], cv[v * d + j], acc);
    if (mode == 0)
      for (int r = 0; r < m; ++r) acc = fmaf(s[static_cast<int64_t>(r) * d + i], sg[v * m + r], acc);
    out[(seq * n + t) * d + i] = acc;
  }
}

template <int NT>
hipError_t launch_encode_nt(const tq_quantizer* q, int mode, const void* x, int dtype, int64_t nseq, int64_t n,
                            uint32_t* codes, float* norms, float* gammas, hipStream_t st) {
  constexpr int DP = NT * 16;
  const size_t lds = sizeof(float) * (kTileRows * (DP + 1) + kTileRows + kMaxLevels) + 2 * kTileRows * DP;
  dim3 grid(static_cast<unsigned>((n + kTileRows - 1) / kTileRows), static_cast<unsigned>(nseq));
  // Pi k-major = the first d columns of the query table (row stride d + m); S' k-major
  hipLaunchKernelGGL((encode_kernel<NT>), grid, dim3(kThreads), lds, st, x, dtype, n, q->d, mode, q->d_qt, q->d + q->m,
                     q->d_spt,
                     q->cb[mode == 0 ? 0 : 1], codes, norms, gammas);
  return hipGetLastError();
}

}  // namespace

size_t encode_lds_bytes(int d) {
  const int DP = ((d + 15) / 16) * 16;
  return sizeof(float) * (kTileRows * (DP + 1) + kTileRows + kMaxLevels) + 2 * kTileRows * DP;
}

static int encode_tile_blocks() {
  static int blocks = [] {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    return 2 * cus;   // two resident workgroups per CU (LDS and registers)
  }();
  return blocks;
}

template <int LK, int MODE, bool FULL>
hipError_t launch_encode_tile_m(const tq_quantizer* q, const void* x, int dtype, int64_t nseq, int64_t n,
                                uint32_t* codes, float* norms, float* gammas, hipStream_t st) {
  const int64_t tiles = nseq * ((n + kEncRows - 1) / kEncRows);
  const dim3 grid(static_cast<unsigned>(std::min<int64_t>(tiles, encode_tile_blocks())));
  const Codebook& cb = q->cb[MODE == 0 ? 0 : 1];
#define TQ_ENC(BPV)                                                                                                 \
  case BPV:                                                                                                         \
    hipLaunchKernelGGL((encode_tile_kernel<4, LK, MODE, BPV, FULL>), grid, dim3(256), 0, st, x, dtype, nseq, n, q->d,     \
                       q->d_pi, q->d_sp, cb, codes, norms, gammas);                                               \
    break;
  switch (cb.bp) {
    TQ_ENC(1) TQ_ENC(2) TQ_ENC(3)
    case 4:
      if constexpr (MODE != 0) {
        hipLaunchKernelGGL((encode_tile_kernel<4, LK, MODE, 4, FULL>), grid, dim3(256), 0, st, x, dtype, nseq, n, q->d,
                           q->d_pi, q->d_sp, cb, codes, norms, gammas);
        break;
      }
      return hipErrorNotSupported;
    default: return hipErrorNotSupported;
  }
#undef TQ_ENC
  return hipGetLastError();
}

template <int LK>
hipError_t launch_encode_tile_lk(const tq_quantizer* q, int mode, const void* x, int dtype, int64_t nseq, int64_t n,
                                 uint32_t* codes, float* norms, float* gammas, hipStream_t st) {
  // d = 128 (the usual head dimension) takes the variant without coordinate guards
  constexpr bool F = LK != 0;
  if (F && q->d == 128) {
    if (mode == 0) return launch_encode_tile_m<LK, 0, F>(q, x, dtype, nseq, n, codes, norms, gammas, st);
    if (mode == 1) return launch_encode_tile_m<LK, 1, F>(q, x, dtype, nseq, n, codes, norms, gammas, st);
    return launch_encode_tile_m<LK, 2, F>(q, x, dtype, nseq, n, codes, norms, gammas, st);
  }
  if (mode == 0) return launch_encode_tile_m<LK, 0, false>(q, x, dtype, nseq, n, codes, norms, gammas, st);
  if (mode == 1) return launch_encode_tile_m<LK, 1, false>(q, x, dtype, nseq, n, codes, norms, gammas, st);
  return launch_encode_tile_m<LK, 2, false>(q, x, dtype, nseq, n, codes, norms, gammas, st);
}

hipError_t launch_encode_tile(const tq_quantizer* q, int mode, const void* x, int dtype, int64_t nseq, int64_t n,
                              uint32_t* codes, float* norms, float* gammas, hipStream_t st) {
  const int esz = dtype == 1 ? 2 : 4;
  if ((q->d * esz) % 16 != 0) return launch_encode_tile_lk<0>(q, mode, x, dtype, nseq, n, codes, norms, gammas, st);
  if (dtype == 1) return launch_encode_tile_lk<1>(q, mode, x, dtype, nseq, n, codes, norms, gammas, st);
  return launch_encode_tile_lk<2>(q, mode, x, dtype, nseq, n, codes, norms, gammas, st);
}

hipError_t launch_encode(const tq_quantizer* q, int mode, const void* x, int dtype, int64_t nseq, int64_t n,
                         uint32_t* codes, float* norms, float* gammas, hipStream_t st) {
  if (q->d <= 128) {
    return launch_encode_tile(q, mode, x, dtype, nseq, n, codes, norms, gammas, st);
  }
  const int nt = (q->d + 15) / 16;
  switch (nt) {
#define TQ_NT_CASE(N) \
  case N: return launch_encode_nt<N>(q, mode, x, dtype, nseq, n, codes, norms, gammas, st);
    TQ_NT_CASE(1) TQ_NT_CASE(2) TQ_NT_CASE(3) TQ_NT_CASE(4) TQ_NT_CASE(5) TQ_NT_CASE(6) TQ_NT_CASE(7) TQ_NT_CASE(8)
    TQ_NT_CASE(9) TQ_NT_CASE(10) TQ_NT_CASE(11) TQ_NT_CASE(12) TQ_NT_CASE(13) TQ_NT_CASE(14) TQ_NT_CASE(15) TQ_NT_CASE(16)
#undef TQ_NT_CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const tq_quantizer* q, int mode, const uint32_t* codes, const float* norms, const float* gammas,
                         int64_t nseq, int64_t n, float* out, hipStream_t st) {
  const size_t lds = sizeof(float) * 8 * (q->d + (mode == 0 ? q->m : 0));
  dim3 grid(static_cast<unsigned>((n + 7) / 8), static_cast<unsigned>(nseq));
  hipLaunchKernelGGL(decode_kernel, grid, dim3(256), lds, st, codes, norms, gammas, n, q->d, q->m, mode, q->d_pi, q->d_s,
                     q->cb[mode == 0 ? 0 : 1], out);
  return hipGetLastError();
}

}  // namespace tq

namespace tq {

hipError_t set_kernel_attributes() {
  static hipError_t once = [] {
    hipError_t e = hipSuccess;
#define TQ_ATTR(N)                                                                                                  \
  if (e == hipSuccess)                                                                                              \
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&encode_kernel<N>), hipFuncAttributeMaxDynamicSharedMemorySize, \
                            static_cast<int>(encode_lds_bytes(N * 16)));
    TQ_ATTR(1) TQ_ATTR(2) TQ_ATTR(3) TQ_ATTR(4) TQ_ATTR(5) TQ_ATTR(6) TQ_ATTR(7) TQ_ATTR(8)
    TQ_ATTR(9) TQ_ATTR(10) TQ_ATTR(11) TQ_ATTR(12) TQ_ATTR(13) TQ_ATTR(14) TQ_ATTR(15) TQ_ATTR(16)
#undef TQ_ATTR
    return e;
  }();
  return once;
}

}  // namespace tq
