// Encode and decode kernels.
//
// Encode follows the two stages on the pages (blog.hotdry.top "TurboQuant
// vector-search compression", random rotation + scalar quantisation and QJL
// residual correction sections; a2a-mcp.org "什麼是TurboQuant？", stage 1
// and stage 2): n = ||x||, y = Pi x / n, nearest Lloyd-Max centroid per
// coordinate, rho = y - c[idx], gamma = n ||rho||, QJL bits = sign(S' rho)
// with S' = S Pi^T (so S' rho = S r / n for the residual r = x - x_hat).
//
// Both products by a d x d matrix (Pi x and S' rho) are taken to fp32
// accuracy, so the code decisions are taken on fp32-accurate values:
//  * prod keys at d = 128 (encode_keys_split_kernel): the split products
//    below, with the rotation and the QJL projection in different waves of
//    one workgroup, pipelined one tile apart;
//  * d <= 128 (encode_tile_kernel): the fp16 16x16x32 MFMA on split
//    operands.  A float is written as hi + lo, two fp16 numbers (22
//    significant bits), and the matrix core accumulates the products at fp32
//    accuracy: x (Pi_hi + Pi_lo) for the rotation (bf16 keys are exact in
//    fp16 after a power-of-two row scale; fp32 keys add x_lo Pi_hi) and
//    rho_hi S'_hi + rho_lo S'_hi + rho_hi S'_lo for the QJL projection.
//    Wave w keeps its 32 rows of Pi and S' (hi and lo) in registers as the
//    stationary operand; workgroups are persistent over 64-vector tiles.
//  * 128 < d <= 256 with rows in 16-byte runs (encode_tile_kernel<8, ...>):
//    the same split products with eight waves, whose rows of Pi and S' (hi
//    and lo) are read per 32-column step from the quantizer's fp16 tables in
//    L2 instead of being held in registers.
//  * otherwise (encode_kernel): the fp32 MFMA (16x16x4), one workgroup per
//    tile of 64 vectors; each wave takes a quarter of the 16-column tiles
//    for all 64 rows.
//  * the Hadamard rotation, values and MSE-only keys (encode_wht_kernel): the
//    fast Walsh-Hadamard transform in registers, no matrix core.
#include <algorithm>
#include <type_traits>

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
// Encoder for 256 < d <= 1024: the general kernel's steps on tiles of ROWS
// vectors (16 for keys; 32 for values, whose words hold 32 tokens), so that a
// tile of d floats per row fits in LDS.  Same fp32 matrix-core contraction
// (gemm_rows below), bucketize, residual, QJL projection and packing as
// encode_kernel; Pi and S' are read from the L2-resident tables once per tile.
// ---------------------------------------------------------------------------
// acc[rt][j] = rows 16 rt .. 16 rt + 15 of xs times column tile w + 4 j of the
// k-major Mt, for R row tiles and NTW column tiles per wave (column tiles at
// or past NT compute on clamped columns and are never read).
template <int R, int NTW>
__device__ __forceinline__ void gemm_rows(const float* xs, int ld, const float* __restrict__ Mt, int ldm, int rows_m,
                                          int d, int w, v4f (&acc)[R][NTW]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < R; ++rt)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[rt][j] = (v4f){0.f, 0.f, 0.f, 0.f};
  int colc[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) colc[j] = min((w + 4 * j) * 16 + r, rows_m - 1);
  for (int k0 = 0; k0 < d; k0 += 4) {
    const int k = k0 + kq;
    const bool kin = k < d;
    const int kc = min(k, d - 1);
    float b[NTW], a[R];
#pragma unroll
    for (int j = 0; j < NTW; ++j) b[j] = Mt[static_cast<int64_t>(kc) * ldm + colc[j]];
#pragma unroll
    for (int rt = 0; rt < R; ++rt) {
      const float v = xs[(16 * rt + r) * ld + kc];
      a[rt] = kin ? v : 0.f;
    }
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int rt = 0; rt < R; ++rt) acc[rt][j] = mfma_f32(a[rt], b[j], acc[rt][j]);
  }
#pragma unroll
  for (int rt = 0; rt < R; ++rt)
#pragma unroll
    for (int j = 0; j < NTW; ++j) pin(acc[rt][j]);
}

size_t encode_big_lds_bytes(int d, int rows, bool keys) {
  const int DP = ((d + 15) / 16) * 16;
  // x (then rho) [rows][DP + 1] floats, norms, centroids; keys add index and
  // sign bytes [rows][DP] each (values keep their index bytes over x)
  return sizeof(float) * (static_cast<size_t>(rows) * (DP + 1) + rows + kMaxLevels) +
         (keys ? 2 * static_cast<size_t>(rows) * DP : 0);
}

template <int ROWS, int NTW>
__global__ void __launch_bounds__(kThreads) encode_big_kernel(const void* __restrict__ x, int dtype, int64_t n, int d,
                                                              int mode, const float* __restrict__ pit, int ldp,
                                                              const float* __restrict__ spt, Codebook cb,
                                                              uint32_t* __restrict__ codes, float* __restrict__ norms,
                                                              float* __restrict__ gammas) {
  constexpr int R = ROWS / 16;
  constexpr int TPR = kThreads / ROWS;   // threads per row for the norms
  const int NT = (d + 15) / 16;
  const int DP = NT * 16, LD = DP + 1;
  extern __shared__ float smem[];
  float* xs = smem;                       // [ROWS][LD]
  float* nrm = xs + ROWS * LD;            // [ROWS]
  float* cen = nrm + ROWS;                // [kMaxLevels]
  uint8_t* idxb = mode == 1 ? reinterpret_cast<uint8_t*>(xs) : reinterpret_cast<uint8_t*>(cen + kMaxLevels);
  uint8_t* sgnb = idxb + ROWS * DP;       // keys only
  __shared__ float part2[4][ROWS];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int64_t seq = blockIdx.y;
  const int64_t v0 = static_cast<int64_t>(blockIdx.x) * ROWS;
  const int rows = static_cast<int>(n - v0 < ROWS ? n - v0 : ROWS);
  const int64_t base = seq * n + v0;

  if (tid < kMaxLevels) cen[tid] = tid < cb.levels ? cb.c[tid] : 0.f;
  for (int e = tid; e < ROWS * DP; e += kThreads) {
    const int row = e / DP, col = e - row * DP;
    float v = 0.f;
    if (row < rows && col < d) v = load_elem(x, dtype, (base + row) * d + col);
    xs[row * LD + col] = v;
  }
  __syncthreads();
  {
    const int row = tid / TPR, part = tid % TPR;
    float s = 0.f;
    for (int col = part; col < d; col += TPR) {
      const float v = xs[row * LD + col];
      s = fmaf(v, v, s);
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) s += __shfl_xor(s, o);
    if (part == 0) nrm[row] = sqrtf(s);
  }
  __syncthreads();

  v4f acc[R][NTW];
  gemm_rows<R, NTW>(xs, LD, pit, ldp, d, d, wave, acc);

  const int col_in = lane & 15, rq = lane >> 4;
  float inv_n[R][4], rho2[R][4];
#pragma unroll
  for (int rt = 0; rt < R; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float nv = nrm[16 * rt + 4 * rq + i];
      inv_n[rt][i] = nv > 0.f ? 1.f / nv : 0.f;
      rho2[rt][i] = 0.f;
    }
  const int kh = cb.levels >> 1;
  // keys: index bytes go to their own array now and rho stays in acc; values:
  // the index (as a float) stays in acc, since its bytes go over x
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int col = (wave + 4 * j) * 16 + col_in;
#pragma unroll
    for (int rt = 0; rt < R; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y = acc[rt][j][i] * inv_n[rt][i];
        const float ay = fabsf(y);
        int jm = 0;
#pragma unroll
        for (int k = 0; k + 1 < kMaxLevels / 2; ++k)
          if (k + 1 < kh) jm += (cb.t[kh + k] < ay) ? 1 : 0;
        const int idx = col < d ? (y > 0.f ? kh + jm : kh - 1 - jm) : 0;
        const float rho = col < d ? y - cen[idx] : 0.f;
        rho2[rt][i] = fmaf(rho, rho, rho2[rt][i]);
        if (mode != 1) {
          if (wave + 4 * j < NT) idxb[(16 * rt + 4 * rq + i) * DP + col] = static_cast<uint8_t>(idx);
          acc[rt][j][i] = rho;
        } else {
          acc[rt][j][i] = static_cast<float>(idx);
        }
      }
  }
  __syncthreads();   // every wave is done with x: rho (keys) or the index bytes (values) go over it
#pragma unroll
  for (int j = 0; j < NTW; ++j)
    if (wave + 4 * j < NT) {
#pragma unroll
      for (int rt = 0; rt < R; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * rt + 4 * rq + i, col = (wave + 4 * j) * 16 + col_in;
          if (mode != 1) xs[row * LD + col] = acc[rt][j][i];
          else idxb[row * DP + col] = static_cast<uint8_t>(acc[rt][j][i]);
        }
    }

  if (mode == 0) {
#pragma unroll
    for (int rt = 0; rt < R; ++rt)
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
    gemm_rows<R, NTW>(xs, LD, spt, d, d, d, wave, acc);
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int col = (wave + 4 * j) * 16 + col_in;
      if (wave + 4 * j < NT) {
#pragma unroll
        for (int rt = 0; rt < R; ++rt)
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

  const int bp = cb.bp;
  if (mode != 1) {
    const int G = (d + 31) >> 5;
    const int W = bp + (mode == 0 ? 1 : 0);
    for (int task = tid; task < ROWS * G; task += kThreads) {
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
    // values: one 32-token block per tile (ROWS = 32), words [seq][blk][bp][d]
    static_assert(ROWS == 32 || ROWS == 16, "tile rows");
    const int64_t nb = (n + 31) >> 5;
    const int64_t blk = v0 >> 5;
    if (ROWS == 32 && blk < nb) {
      for (int j = tid; j < d; j += kThreads) {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        for (int i = 0; i < rows; ++i) {
          const uint32_t iv = idxb[i * DP + j];
          for (int p = 0; p < bp; ++p) w[p] |= ((iv >> p) & 1u) << i;
        }
        uint32_t* out = codes + ((seq * nb + blk) * bp) * d + j;
        for (int p = 0; p < bp; ++p) out[static_cast<int64_t>(p) * d] = w[p];
      }
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
constexpr int kWideK = 256;             // rows and columns of the wide kernel's fp16 tables
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
// coordinates and the coordinate guards compile away.  HAD: Pi = H D / sqrt(d)
// (the structured rotation): sqrt(d) Pi has entries +-1, so the rotation's
// stationary operand is +-2^8 exactly in fp16 and needs no lo part -- one
// product per rotation term instead of two (bf16 input), with 1/sqrt(d)
// moved into the fp32 row scale.
//
// KS = 8 (128 < d <= 256): eight waves, wave w owning group w as above, but
// the rows of Pi and S' (hi and lo, 256 inputs) do not fit in registers: they
// are read per 32-input step from fp16 tables (`wt`: Pi hi, Pi lo, S' hi, S'
// lo, each [256][256], row j = output coordinate j, zero past d), which stay
// in L2, with the next step's operands in flight while the current one is
// multiplied.
template <int KS, int LK, int MODE, int BP, bool FULL, bool HAD = false>
__global__ void __launch_bounds__(64 * KS, KS == 4 ? 2 : 1)
    encode_tile_kernel(const void* __restrict__ x, int dtype, int64_t nseq, int64_t n, int d,
                       const float* __restrict__ pi, const float* __restrict__ sp, const _Float16* __restrict__ wt,
                       Codebook cb, uint32_t* __restrict__ codes, float* __restrict__ norms,
                       float* __restrict__ gammas) {
  constexpr bool PROD = MODE != 1;       // token-major words, C[vector][coordinate]
  constexpr bool QJL = MODE == 0;        // residual, QJL plane and gamma
  constexpr bool STREAM = KS == 8;       // Pi and S' rows from the L2-resident tables
  constexpr int NTH = 64 * KS;           // threads: one wave per 32-coordinate group
  constexpr int TPR = NTH / kEncRows;    // loader threads per row
  constexpr int KP = 32 * KS;            // padded contraction length
  constexpr int LDH = KP + 8;            // LDS row stride in halves (16-byte rows, conflict-free reads)
  constexpr bool XLO = LK != 1;          // fp32 keys need x_lo (bf16 keys are exact in fp16)
  constexpr int PREN = LK == 2 ? 8 : LK == 1 ? 4 : 1;   // 16-byte chunks per loader thread
  constexpr int EPT = KP / TPR;          // elements per loader thread (scalar path)
  constexpr int TAB = kWideK * kWideK;   // elements of one table (STREAM)
  __shared__ __attribute__((aligned(16))) _Float16 xh[kEncRows * LDH];
  __shared__ __attribute__((aligned(16))) _Float16 xl[XLO ? kEncRows * LDH : 8];
  __shared__ __attribute__((aligned(16))) _Float16 rh[QJL ? kEncRows * LDH : 8];
  __shared__ __attribute__((aligned(16))) _Float16 rl[QJL ? kEncRows * LDH : 8];
  __shared__ __attribute__((aligned(16))) float scl2[2][kEncRows];   // 2^(6 - row scale) / n, by tile parity
  __shared__ float nrm2[2][kEncRows];    // n, by tile parity
  __shared__ float part2[KS][kEncRows];
  __shared__ uint32_t ost[2][256 * KS];

  static_assert(KS == 4 || KS == 8, "four or eight waves own 32 coordinates each");
  static_assert(!STREAM || !HAD, "the wide kernel takes the +-1 rotation as a general one");
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

  static_assert(!HAD || FULL, "the +-1 rotation operand is built for d = 32 KS");
  // stationary operands: lane (r16, q) holds row 32w + 16ct + r16, columns
  // 32s + 8q .. +7 of Pi (and S'), split into hi + lo (HAD: sqrt(d) Pi 2^8 =
  // +-2^8, exact, no lo part); none with STREAM
  constexpr int RS = STREAM ? 1 : KS;
  v8h bPh[2][RS], bPl[2][HAD ? 1 : RS], bSh[2][QJL ? RS : 1], bSl[2][QJL ? RS : 1];
  if constexpr (!STREAM) {
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int j = 32 * w + 16 * ct + r16;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = 32 * s2 + 8 * q + e;
        const bool in = j < d && k < d;
        if constexpr (HAD) {
          const float pv = in ? pi[static_cast<int64_t>(j) * d + k] : 0.f;
          bPh[ct][s2][e] = static_cast<_Float16>(pv > 0.f ? kPiScale : pv < 0.f ? -kPiScale : 0.f);
        } else {
          const float vp = in ? pi[static_cast<int64_t>(j) * d + k] * kPiScale : 0.f;
          const _Float16 ph = static_cast<_Float16>(vp);
          bPh[ct][s2][e] = ph;
          bPl[ct][s2][e] = static_cast<_Float16>(vp - static_cast<float>(ph));
        }
        if constexpr (QJL) {
          const float vs = in ? sp[static_cast<int64_t>(j) * d + k] * kPiScale : 0.f;
          const _Float16 sh = static_cast<_Float16>(vs);
          bSh[ct][s2][e] = sh;
          bSl[ct][s2][e] = static_cast<_Float16>(vs - static_cast<float>(sh));
        }
      }
  }
  }
  for (int e = tid; e < kEncRows * LDH; e += NTH) {
    xh[e] = static_cast<_Float16>(0.f);
    if constexpr (XLO) xl[e] = static_cast<_Float16>(0.f);
    if constexpr (QJL) {
      rh[e] = static_cast<_Float16>(0.f);
      rl[e] = static_cast<_Float16>(0.f);
    }
  }

  // loader role: row = tid / TPR, TPR threads per row
  const int lrow = tid / TPR, part = tid % TPR;
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
        const int c = part + TPR * j;
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
        const int c = part + TPR * j;
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
        const int c = part + TPR * j;
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
        const int col = part + TPR * j;
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
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) {
      ss += __shfl_xor(ss, o);
      mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    // power-of-two row scale putting the largest element in [2^14, 2^15)
    const int sig = mx > 0.f ? 14 - ilogb_pos(mx) : 0;
    _Float16* hr = xh + lrow * LDH;
    _Float16* lr = xl + lrow * LDH;
    if constexpr (LK == 1) {
      // a 16-byte chunk of 8 bf16 values becomes one 16-byte row segment
#pragma unroll
      for (int j = 0; j < PREN; ++j) {
        const int c = part + TPR * j;
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
      // y 2^14 = acc * scl: the rotation of u, times 2^14 (Pi carries 2^8, the row 2^sig;
      // HAD: the operand is sqrt(d) Pi 2^8, so the scale also divides by sqrt(d))
      if constexpr (HAD)
        scl[lrow] = nv > 0.f ? ldexpf(1.f / (nv * sqrtf(static_cast<float>(32 * KS))), 6 - sig) : 0.f;
      else
        scl[lrow] = nv > 0.f ? ldexpf(1.f / nv, 6 - sig) : 0.f;
    }
  };
  auto store = [&](TileAt t, int buf) {
    int64_t seq, v0;
    int rows;
    tile_of(t, seq, v0, rows);
    if constexpr (PROD) {
      uint32_t* dst = codes + (seq * n + v0) * WPK;
      for (int e = tid; e < rows * WPK; e += NTH) dst[e] = ost[buf][e];
    } else {
      const int nblk = (rows + 31) >> 5;
      uint32_t* dst = codes + ((seq * nb + (v0 >> 5)) * bp) * d;
      for (int e = tid; e < nblk * bp * d; e += NTH) dst[e] = ost[buf][e];
    }
  };
  // acc[h2][ct] (+)= rows 32h + 16h2 .. of src times this wave's columns;
  // SWAP puts the stationary operand first (C[coordinate][vector])
  auto contract = [&](const _Float16* src, const v8h (&bm)[2][RS], int h, bool swap, v4f (&acc)[2][2]) {
#pragma unroll
    for (int s2 = 0; s2 < RS; ++s2) {
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
  // STREAM: acc[h2][ct] (+)= rows 32h + 16h2 .. of A0 times table T0, of A0
  // times T1 and of A1 times T0 (each product only where the pointers are
  // set): the B operands of step s2 are this wave's rows of the tables,
  // loaded one step ahead
  auto contract_stream = [&](const _Float16* A0, const _Float16* A1, const _Float16* T0, const _Float16* T1, int h,
                             bool swap, v4f (&acc)[2][2]) {
    // this lane's operand bytes within a table: row 32w + 16ct + r16, columns
    // 8q .. 8q + 7 of each 32-column step (uniform table base + 32-bit offset)
    auto ld = [&](const _Float16* T, int s2, int ct) {
      const uint32_t off = static_cast<uint32_t>(((32 * w + 16 * ct + r16) * kWideK + 32 * s2 + 8 * q) * 2);
      return *reinterpret_cast<const v8h*>(reinterpret_cast<const char*>(T) + off);
    };
    // SP 32-column steps per iteration, the next iteration's operands in
    // flight while these are multiplied; not unrolled further (unrolled, the
    // loop hoists every load and spills)
    constexpr int SP = 2;   // d = 256, GQA shape: 1 step 3.73 ms, 2 steps 3.35 ms, 4 steps 4.93 ms (keys)
    v8h b0[SP][2], b1[SP][2];
#pragma unroll
    for (int u = 0; u < SP; ++u)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        b0[u][ct] = ld(T0, u, ct);
        if (T1) b1[u][ct] = ld(T1, u, ct);
      }
#pragma unroll 1
    for (int s0 = 0; s0 < KS; s0 += SP) {
      v8h n0[SP][2], n1[SP][2];
      if (s0 + SP < KS) {
#pragma unroll
        for (int u = 0; u < SP; ++u)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            n0[u][ct] = ld(T0, s0 + SP + u, ct);
            if (T1) n1[u][ct] = ld(T1, s0 + SP + u, ct);
          }
      }
#pragma unroll
      for (int u = 0; u < SP; ++u) {
        const int s2 = s0 + u;
        v8h a0[2], a1[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          a0[h2] = *reinterpret_cast<const v8h*>(A0 + (32 * h + 16 * h2 + r16) * LDH + 32 * s2 + 8 * q);
          if (A1) a1[h2] = *reinterpret_cast<const v8h*>(A1 + (32 * h + 16 * h2 + r16) * LDH + 32 * s2 + 8 * q);
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            acc[h2][ct] = swap ? mfma_f16(b0[u][ct], a0[h2], acc[h2][ct]) : mfma_f16(a0[h2], b0[u][ct], acc[h2][ct]);
            if (T1)
              acc[h2][ct] = swap ? mfma_f16(b1[u][ct], a0[h2], acc[h2][ct]) : mfma_f16(a0[h2], b1[u][ct], acc[h2][ct]);
            if (A1)
              acc[h2][ct] = swap ? mfma_f16(b0[u][ct], a1[h2], acc[h2][ct]) : mfma_f16(a1[h2], b0[u][ct], acc[h2][ct]);
          }
      }
      if (s0 + SP < KS) {
#pragma unroll
        for (int u = 0; u < SP; ++u)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            b0[u][ct] = n0[u][ct];
            if (T1) b1[u][ct] = n1[u][ct];
          }
      }
    }
  };
  // the rotation (x Pi^T, split products) of rows 32h .. 32h + 31
  auto rotate = [&](int h, bool swap, v4f (&acc)[2][2]) {
    if constexpr (STREAM) {
      contract_stream(xh, XLO ? xl : nullptr, wt, wt + TAB, h, swap, acc);
    } else {
      contract(xh, bPh, h, swap, acc);
      if constexpr (!HAD) contract(xh, bPl, h, swap, acc);
      if constexpr (XLO) contract(xl, bPh, h, swap, acc);
    }
  };
  auto sum_parts = [&](int r) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k) t += part2[k][r];
    return t;
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
        rotate(h, false, acc);
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
          if constexpr (STREAM) {
            contract_stream(rh, rl, wt + 2 * TAB, wt + 3 * TAB, h, false, acc);
          } else {
            contract(rh, bSh, h, false, acc);
            contract(rl, bSh, h, false, acc);
            contract(rh, bSl, h, false, acc);
          }
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
          gammas[seq * n + v0 + tid] = nv * sqrtf(sum_parts(tid)) * (1.f / kRhoScale);
      }
    } else {
      // lane holds coordinate 32w + 16ct + 4q + i, token 32h + 16h2 + r16;
      // half h is the 32-token block h of the tile
#pragma unroll 1
      for (int h = 0; h < 2; ++h) {
        v4f acc[2][2];
        zero_acc(acc);
        rotate(h, true, acc);
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

// ---------------------------------------------------------------------------
// Key encoder for d = 128 (prod mode) with the work split
// by role between the eight waves of a workgroup, pipelined one tile apart:
//  * rotation waves 0-3: wave w keeps rows 32w .. 32w + 31 of Pi in
//    registers; for tile i it takes the rotation, decides the index bits, and
//    writes the index words, the residual rho (hi and lo) and its partial
//    ||rho||^2 to LDS;
//  * projection waves 4-7: wave 4 + w keeps rows 32w .. 32w + 31 of S' (hi
//    and lo); it puts tile i + 1 into LDS and fetches tile i + 2, stores the
//    finished words, norms and gammas of tile i - 2, then projects the
//    residual of tile i - 1 and writes its QJL words.
// One barrier per tile.  A SIMD holds one wave of each role: while one
// classifies (vector ALU), the other's products occupy the matrix core; the
// projection waves do their vector work first, when the rotation waves start
// on the matrix core, and both roles issue the products of their second
// 32-key half inside the decisions on the first.  Every global access of an
// iteration (the fetch, then the stores) is issued at its start: the stores
// share the load counter, so the wait for the fetched tile one iteration
// later also waits for them, and by then they are a whole iteration old.
// Each role's stationary operands are live only in its own loop.
//
// The arithmetic per element is the tile kernel's: the same split fp16
// products (rows scaled so that the largest element lies in [2^14, 2^15);
// x (Pi_hi + Pi_lo), plus x_lo Pi_hi for fp32 keys; rho_hi S'_hi + rho_lo S'_hi
// + rho_hi S'_lo) in the same order per accumulator, and the same decisions
// and roundings.
// ---------------------------------------------------------------------------
__device__ __forceinline__ v4f mfma_x(const v8h& a, const v8h& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int LK, int BP, bool HAD>
__global__ void __launch_bounds__(512, 1)
    encode_keys_split_kernel(const void* __restrict__ x, int64_t nseq, int64_t n, const float* __restrict__ pi,
                             const float* __restrict__ sp, Codebook cb, uint32_t* __restrict__ codes,
                             float* __restrict__ norms, float* __restrict__ gammas) {
  static_assert(LK == 1 || LK == 2, "bf16 or fp32 rows in 16-byte chunks");
  constexpr int D = 128;
  constexpr int LDH = D + 8;             // LDS row stride in halves
  constexpr bool XLO = LK == 2;          // fp32 keys carry x_lo (bf16 keys are exact in fp16)
  constexpr int NSRC = XLO ? 2 : 1;      // parts of x in LDS
  // rotation products: (x_hi, Pi_hi) (x_hi, Pi_lo), and (x_lo, Pi_hi) for fp32 keys;
  // HAD (Pi = H D / sqrt(d)): the operand sqrt(d) Pi 2^8 = +-2^8 is exact, so
  // (x_hi, +-2^8), and (x_lo, +-2^8) for fp32 keys
  constexpr int NPASS = HAD ? (XLO ? 2 : 1) : (XLO ? 3 : 2);
  constexpr int W = BP + 1;              // words per 32-coordinate group: index planes + QJL
  constexpr int WPK = 4 * W;             // words per key
  constexpr int esz = LK == 1 ? 2 : 4;
  constexpr int CH = D * esz / 16;       // 16-byte chunks per row
  constexpr int PREN = CH / 4;           // chunks per loader thread (4 threads per row)
  constexpr int EPT = D / 4;             // elements per loader thread
  __shared__ __attribute__((aligned(16))) uint16_t xs16[NSRC][2][kEncRows * LDH];   // x: fp16 hi (and lo)
  __shared__ __attribute__((aligned(16))) _Float16 rh[2][kEncRows * LDH];
  __shared__ __attribute__((aligned(16))) _Float16 rl[2][kEncRows * LDH];
  __shared__ __attribute__((aligned(16))) float scl3[3][kEncRows];   // y 2^14 = acc * scl
  __shared__ float nrm3[3][kEncRows];                                // n
  __shared__ float part2[2][4][kEncRows];                            // ||rho||^2 per coordinate group
  __shared__ __attribute__((aligned(16))) uint32_t ost[3][kEncRows * WPK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int w = wv & 3;                  // coordinate group (rotation) or QJL row group (projection)
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t tps = (n + kEncRows - 1) / kEncRows;   // tiles per sequence
  const int64_t total = nseq * tps;
  // tiles of this workgroup: blockIdx.x + k gridDim.x < total (the grid never exceeds the tiles)
  const int T = static_cast<int>((total - blockIdx.x + gridDim.x - 1) / gridDim.x);

  // A operand: rows 32h + 16h2 + r16 of an LDS tile, columns 32 s2 + 8q .. + 7
  auto a_op = [&](const void* src, int h, int h2, int s2) {
    return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + (32 * h + 16 * h2 + r16) * LDH +
                                           32 * s2 + 8 * q);
  };
  auto zero_pin = [&](v4f (&acc)[2][2], bool zero) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        if (zero) acc[h2][ct] = (v4f){0.f, 0.f, 0.f, 0.f};
        else pin(acc[h2][ct]);
      }
  };
  // packed word of row 4q + i of a ballot pair (low 16 bits, high 16 bits)
  auto halves = [&](uint64_t m0, uint64_t m1) {
    return __builtin_amdgcn_perm(static_cast<uint32_t>(m1 >> (16 * q)), static_cast<uint32_t>(m0 >> (16 * q)),
                                 0x05040100u);
  };
  // element (ct, s2, e) of this lane's stationary operand: row 32w + 16ct + r16
  // of a matrix (output coordinate), column 32 s2 + 8q + e, times 2^8
  auto mat_at = [&](const float* __restrict__ m, int ct, int s2, int e) {
    return m[(32 * w + 16 * ct + r16) * D + 32 * s2 + 8 * q + e] * kPiScale;
  };

  if (wv < 4) {
    // ======================= rotation waves =======================
    v8h bP[HAD ? 1 : 2][2][4];   // Pi_hi, Pi_lo (HAD: +-2^8 only)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = mat_at(pi, ct, s2, e);
          if constexpr (HAD) {
            bP[0][ct][s2][e] = static_cast<_Float16>(v > 0.f ? kPiScale : v < 0.f ? -kPiScale : 0.f);
          } else {
            const _Float16 h0 = static_cast<_Float16>(v);
            bP[0][ct][s2][e] = h0;
            bP[HAD ? 0 : 1][ct][s2][e] = static_cast<_Float16>(v - static_cast<float>(h0));
          }
        }
    // pass k: source part (x_hi, x_lo) and Pi part (hi, lo)
    auto pass_src = [](int k) { return HAD ? k : (k == 2 ? 1 : 0); };
    auto pass_op = [](int k) { return HAD ? 0 : (k == 1 ? 1 : 0); };
    // symmetric codebook: sign = top index bit, |y| against the positive
    // thresholds gives the others (as in the tile kernel)
    constexpr int KH = 1 << (BP - 1);
    float thp[KH > 1 ? KH - 1 : 1], cenS[KH];
#pragma unroll
    for (int k2 = 0; k2 + 1 < KH; ++k2) thp[k2] = cb.t[KH + k2] * kRhoScale;
#pragma unroll
    for (int k2 = 0; k2 < KH; ++k2) cenS[k2] = cb.c[KH + k2] * kRhoScale;
    __syncthreads();   // tile 0 is in LDS
    int s3 = 0;
    for (int i = 0; i < T + 2; ++i, s3 = s3 == 2 ? 0 : s3 + 1) {
      if (i < T) {
        const int sb = i & 1;
        const float* scl = scl3[s3];
        v4f acc[2][2][2];
        // A operands of one 32-key half: [source][s2][h2]
        v8h av[NSRC][4][2];
        auto load_half = [&](int h) {
#pragma unroll
          for (int sr = 0; sr < NSRC; ++sr)
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
              for (int h2 = 0; h2 < 2; ++h2) av[sr][s2][h2] = __builtin_bit_cast(v8h, a_op(xs16[sr][sb], h, h2, s2));
        };
        // sub-step k of half h: pass k / 4, contraction step k % 4 (per
        // accumulator the products keep the order pass by pass, step by step)
        auto rot = [&](int h, int k) {
          const int ps = k >> 2, s2 = k & 3;
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
              acc[h][h2][ct] = mfma_x(av[pass_src(ps)][s2][h2], bP[pass_op(ps)][ct][s2], acc[h][h2][ct]);
        };
        load_half(0);
        zero_pin(acc[0], true);
#pragma unroll
        for (int k = 0; k < 4 * NPASS; ++k) rot(0, k);
        zero_pin(acc[0], false);
        load_half(1);
        zero_pin(acc[1], true);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h == 1) {
            zero_pin(acc[1], false);
          }
          // lane holds vector 32h + 16h2 + 4q + i, coordinate 32w + 16ct + r16
          float r2v[2][4];
          uint32_t wdall[2][4][BP];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int vbase = 32 * h + 16 * h2 + 4 * q;
            const float4 sc4 = *reinterpret_cast<const float4*>(scl + vbase);
            const float scv[4] = {sc4.x, sc4.y, sc4.z, sc4.w};
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              if (h == 0) {   // half 1's products, a few per classification step of half 0
                const int st = 4 * h2 + i4;
#pragma unroll
                for (int k = (st * 4 * NPASS) / 8; k < ((st + 1) * 4 * NPASS) / 8; ++k) rot(1, k);
              }
              const float scS = scv[i4];
              uint64_t ms[2], mj[2][BP > 1 ? BP - 1 : 1];
              float r2 = 0.f;
#pragma unroll
              for (int ct = 0; ct < 2; ++ct) {
                const int c = 32 * w + 16 * ct + r16;
                const float a = acc[h][h2][ct][i4];
                const bool pos = a > 0.f;
                bool jb[BP > 1 ? BP - 1 : 1];
                if constexpr (BP > 1) decide_bits<BP - 1, BP - 2>(fabsf(a * scS), thp, jb);
                else jb[0] = false;
                ms[ct] = __ballot(pos);
#pragma unroll
                for (int p = 0; p + 1 < BP; ++p) mj[ct][p] = __ballot(jb[p]);
                float cabs;
                if constexpr (BP > 1) cabs = pick_centroid<BP - 1>(cenS, jb);
                else cabs = cenS[0];
                // rho 2^14 = y 2^14 - c[idx] 2^14 in one rounding, split hi + lo
                const float rs = fmaf(a, scS, pos ? -cabs : cabs);
                r2 = fmaf(rs, rs, r2);
                const _Float16 hh = static_cast<_Float16>(rs);
                rh[sb][(vbase + i4) * LDH + c] = hh;
                rl[sb][(vbase + i4) * LDH + c] = f16_remainder(rs, hh);
              }
              // sign plane [y > 0]; low planes [bit of j == sign]
              const uint64_t s0 = ms[0], s1 = ms[1];
              wdall[h2][i4][BP - 1] = halves(s0, s1);
#pragma unroll
              for (int p = 0; p + 1 < BP; ++p) wdall[h2][i4][p] = halves(~(mj[0][p] ^ s0), ~(mj[1][p] ^ s1));
              r2v[h2][i4] = r2;
            }
          }
          if (r16 == 0) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
              for (int i4 = 0; i4 < 4; ++i4)
#pragma unroll
                for (int p = 0; p < BP; ++p)
                  ost[s3][(32 * h + 16 * h2 + 4 * q + i4) * WPK + w * W + p] = wdall[h2][i4][p];
          }
          // ||rho||^2 over this wave's 32 coordinates by the transposing
          // butterfly of the tile kernel: lane r16 ends with row 16 b3 + 2 b2 + b0
          // (lanes r16 and r16 ^ 2 hold the same sum and write the same word)
          const bool b3 = (r16 & 8) != 0, b2 = (r16 & 4) != 0, b0 = (r16 & 1) != 0;
          float a4[4], a2[2];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float lo = r2v[0][k], hi = r2v[1][k];
            a4[k] = (b3 ? hi : lo) + dpp_f<0x128>(b3 ? lo : hi);
          }
#pragma unroll
          for (int k = 0; k < 2; ++k) a2[k] = (b2 ? a4[k + 2] : a4[k]) + dpp_f<0x141>(b2 ? a4[k] : a4[k + 2]);
          float t = (b0 ? a2[1] : a2[0]) + dpp_f<0xB1>(b0 ? a2[0] : a2[1]);
          t += dpp_f<0x4E>(t);
          part2[sb][w][32 * h + 16 * (b3 ? 1 : 0) + 4 * q + 2 * (b2 ? 1 : 0) + (b0 ? 1 : 0)] = t;
        }
      }
      __syncthreads();
    }
  } else {
    // ======================= projection waves =======================
    const int tq = tid - 256;            // 0 .. 255
    v8h bSh[2][4], bSl[2][4];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = mat_at(sp, ct, s2, e);
          const _Float16 h0 = static_cast<_Float16>(v);
          bSh[ct][s2][e] = h0;
          bSl[ct][s2][e] = static_cast<_Float16>(v - static_cast<float>(h0));
        }
    const int lrow = tq >> 2, part = tq & 3;   // loader: 4 threads per row
    uint4 pre[PREN];
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
    auto rows_of = [&](TileAt a) { return static_cast<int>(min(static_cast<int64_t>(kEncRows), n - a.r * kEncRows)); };
    auto fetch = [&](TileAt a) {
      const int rows = rows_of(a);
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(x) +
                                                        ((a.seq * n + a.r * kEncRows + lrow) * D) * esz);
#pragma unroll
      for (int j = 0; j < PREN; ++j) {
        pre[j] = make_uint4(0u, 0u, 0u, 0u);   // rows past n read as 0
        if (lrow < rows) pre[j] = src[part + 4 * j];
      }
    };
    // the tile in `pre` -> LDS slot xsl, and its norms and scales
    auto commit = [&](TileAt a, int xsl, float* scl, float* nrm) {
      const int rows = rows_of(a);
      float v[EPT];
#pragma unroll
      for (int j = 0; j < PREN; ++j) {
        const uint32_t u[4] = {pre[j].x, pre[j].y, pre[j].z, pre[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (LK == 1) {
            v[8 * j + 2 * e] = __uint_as_float(u[e] << 16);
            v[8 * j + 2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
          } else {
            v[4 * j + e] = __uint_as_float(u[e]);
          }
        }
      }
      float ss = 0.f, mx = 0.f;
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        ss = fmaf(v[j], v[j], ss);
        mx = fmaxf(mx, fabsf(v[j]));
      }
#pragma unroll
      for (int o = 1; o < 4; o <<= 1) {
        ss += __shfl_xor(ss, o);
        mx = fmaxf(mx, __shfl_xor(mx, o));
      }
      // power-of-two row scale putting the largest element in [2^14, 2^15)
      const int sig = mx > 0.f ? 14 - ilogb_pos(mx) : 0;
      uint16_t* row = xs16[0][xsl] + lrow * LDH;
      if constexpr (LK == 1) {
        // bf16 keys are exact in fp16 after the row scale: a chunk of 8 is one 16-byte row segment
#pragma unroll
        for (int j = 0; j < PREN; ++j) {
          v8h hv;
#pragma unroll
          for (int e = 0; e < 8; ++e) hv[e] = static_cast<_Float16>(ldexpf(v[8 * j + e], sig));
          *reinterpret_cast<v8h*>(row + 8 * (part + 4 * j)) = hv;
        }
      } else {
        typedef _Float16 v4h __attribute__((ext_vector_type(4)));
        uint16_t* rowl = xs16[NSRC - 1][xsl] + lrow * LDH;
#pragma unroll
        for (int j = 0; j < PREN; ++j) {
          v4h hv, lv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sv = ldexpf(v[4 * j + e], sig);
            const _Float16 hh = static_cast<_Float16>(sv);
            hv[e] = hh;
            lv[e] = static_cast<_Float16>(sv - static_cast<float>(hh));
          }
          *reinterpret_cast<v4h*>(row + 4 * (part + 4 * j)) = hv;
          *reinterpret_cast<v4h*>(rowl + 4 * (part + 4 * j)) = lv;
        }
      }
      if (part == 0) {
        const float nv = lrow < rows ? sqrtf(ss) : 0.f;
        nrm[lrow] = nv;
        // y 2^14 = acc * scl: the rotation of u, times 2^14 (Pi carries 2^8, the row 2^sig)
        // (HAD: the operand is sqrt(d) Pi 2^8, so the scale also divides by sqrt(d))
        if constexpr (HAD)
          scl[lrow] = nv > 0.f ? ldexpf(1.f / (nv * sqrtf(static_cast<float>(D))), 6 - sig) : 0.f;
        else
          scl[lrow] = nv > 0.f ? ldexpf(1.f / nv, 6 - sig) : 0.f;
      }
    };
    TileAt p2 = {0, 0}, p1 = {0, 0}, c0 = {static_cast<int64_t>(blockIdx.x) / tps, static_cast<int64_t>(blockIdx.x) % tps};
    TileAt n1 = c0;
    fetch(c0);
    commit(c0, 0, scl3[0], nrm3[0]);
    if (T > 1) {
      n1 = advance(c0);
      fetch(n1);
    }
    __syncthreads();   // tile 0 is in LDS
    int s3 = 0;        // slot of tile i; i - 1 is s3 - 1, i - 2 and i + 1 are s3 + 1 (mod 3)
    float nv_pend = 0.f, gv_pend = 0.f;   // norm and gamma of tile i - 2, row tq
    for (int i = 0; i < T + 2; ++i, s3 = s3 == 2 ? 0 : s3 + 1) {
      const int s3m1 = s3 == 0 ? 2 : s3 - 1, s3p1 = s3 == 2 ? 0 : s3 + 1;
      TileAt nn = n1;
      if (i + 1 < T) {
        // ---- tile i + 1 into LDS; tile i + 2 in flight ----
        commit(n1, (i + 1) & 1, scl3[s3p1], nrm3[s3p1]);
        const TileAt n2 = advance(n1);
        if (i + 2 < T) fetch(n2);
        nn = n2;
      }
      if (i >= 2) {
        // ---- tile i - 2 (finished in the previous iteration): words, norms, gammas ----
        const int rows = rows_of(p2);
        uint4* dst = reinterpret_cast<uint4*>(codes + (p2.seq * n + p2.r * kEncRows) * WPK);
        const uint4* srcw = reinterpret_cast<const uint4*>(ost[s3p1]);
        for (int e = tq; e < rows * (WPK / 4); e += 256) dst[e] = srcw[e];
        if (tq < rows) {
          const int64_t o = p2.seq * n + p2.r * kEncRows + tq;
          norms[o] = nv_pend;
          gammas[o] = gv_pend;
        }
      }
      if (i >= 1 && i <= T) {
        // ---- QJL of tile i - 1: z = S' rho (scaled), bit = [z >= 0] (all ones for a zero vector) ----
        const int sbp = (i - 1) & 1;
        const float* nrm = nrm3[s3m1];
        // A operands of one 32-key half: [rho hi, rho lo][s2][h2]
        v8h ra[2][4][2];
        auto load_rho = [&](int h) {
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              ra[0][s2][h2] = __builtin_bit_cast(v8h, a_op(rh[sbp], h, h2, s2));
              ra[1][s2][h2] = __builtin_bit_cast(v8h, a_op(rl[sbp], h, h2, s2));
            }
        };
        v4f qa[2][2][2];
        // sub-step k of half h: products rho_hi S'_hi, rho_lo S'_hi, rho_hi S'_lo
        // (k / 4), contraction step k % 4; the tile kernel's order per accumulator
        auto proj = [&](int h, int k) {
          const int ps = k >> 2, s2 = k & 3;
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
              qa[h][h2][ct] = mfma_x(ra[ps == 1 ? 1 : 0][s2][h2], ps == 2 ? bSl[ct][s2] : bSh[ct][s2], qa[h][h2][ct]);
        };
        load_rho(0);
        zero_pin(qa[0], true);
#pragma unroll
        for (int k = 0; k < 12; ++k) proj(0, k);
        zero_pin(qa[0], false);
        load_rho(1);
        zero_pin(qa[1], true);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h == 1) zero_pin(qa[1], false);
          uint32_t wd[2][4];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int vbase = 32 * h + 16 * h2 + 4 * q;
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              if (h == 0) {   // half 1's products, a few per step of half 0
                const int st = 4 * h2 + i4;
#pragma unroll
                for (int k = (st * 12) / 8; k < ((st + 1) * 12) / 8; ++k) proj(1, k);
              }
              const uint64_t zm = __ballot(!(nrm[vbase + i4] > 0.f));
              const uint64_t m0 = __ballot(qa[h][h2][0][i4] >= 0.f) | zm;
              const uint64_t m1 = __ballot(qa[h][h2][1][i4] >= 0.f) | zm;
              wd[h2][i4] = halves(m0, m1);
            }
          }
          if (r16 == 0) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
              for (int i4 = 0; i4 < 4; ++i4) ost[s3m1][(32 * h + 16 * h2 + 4 * q + i4) * WPK + w * W + BP] = wd[h2][i4];
          }
        }
        // norm and gamma of row tq, stored with the words in the next iteration
        if (tq < kEncRows) {
          nv_pend = nrm[tq];
          float t = 0.f;
#pragma unroll
          for (int k = 0; k < 4; ++k) t += part2[sbp][k][tq];
          gv_pend = nv_pend * sqrtf(t) * (1.f / kRhoScale);
        }
      }
      p2 = p1;
      p1 = c0;
      c0 = n1;
      n1 = nn;
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// Walsh-Hadamard encoder for the structured rotation Pi = H D / sqrt(d)
// (TQ_ROT_HADAMARD; H the Sylvester-ordered Hadamard matrix, D the random
// signs), values and MSE-only keys, d = 32 .. 256 a power of two.
// [wiselychen] "Google TurboQuant：KV Cache 壓縮 6x…", TurboQuant+ section:
// the community implementation applies the rotation as a fast Walsh-Hadamard
// transform (O(d log d) butterflies) instead of a dense product.
//
// A lane holds one token's coordinates in registers (two lanes per token for
// d = 256, which each keep 128): the sign flips of D are one xor per bf16 pair
// on the raw bits, the log2(d) butterfly stages run in registers (the last
// one across the lane pair for d = 256), and nothing goes through LDS.  The
// decisions compare v = H D x directly with the thresholds times ||x|| sqrt(d)
// (y = v / (||x|| sqrt(d))), one compare per index bit as in the tile kernel;
// each compare is a lane mask over the wave's tokens, so for values (32-token
// words, one bit per token) a plane word is half of a ballot, collected into
// one lane per coordinate with writelane and stored 64 coordinates at a time.
// MSE-only keys (token-major words) shift each decision into the lane's own
// words.  One wave per 64 tokens (32 for d = 256), no synchronisation.
// ---------------------------------------------------------------------------
// Bits of j = #{positive thresholds < m} (m >= 0), NB of them, by the
// binary search of decide_bits, each returned as the sign bit (bit 31) of
// u[L] = threshold - m (set iff m > threshold); the next threshold is picked
// with bitfield selects on the sign masks.
template <int NB>
__device__ __forceinline__ void mag_sign_bits(float m, const float (&th)[(1 << NB) - 1], uint32_t (&u)[NB]) {
  static_assert(NB >= 1 && NB <= 3, "1 to 3 magnitude bits");
  auto f = [](float x) { return __float_as_uint(x); };
  auto sel = [](uint32_t mask, uint32_t a1, uint32_t a0) { return (mask & a1) | (~mask & a0); };   // v_bfi_b32
  auto msk = [](uint32_t x) { return static_cast<uint32_t>(static_cast<int32_t>(x) >> 31); };
  if constexpr (NB == 1) {
    u[0] = f(th[0] - m);
  } else if constexpr (NB == 2) {
    u[1] = f(th[1] - m);
    const uint32_t m1 = msk(u[1]);
    u[0] = f(__uint_as_float(sel(m1, f(th[2]), f(th[0]))) - m);
  } else {
    u[2] = f(th[3] - m);
    const uint32_t m2 = msk(u[2]);
    u[1] = f(__uint_as_float(sel(m2, f(th[5]), f(th[1]))) - m);
    const uint32_t m1 = msk(u[1]);
    const uint32_t lo = sel(m2, f(th[4]), f(th[0])), hi = sel(m2, f(th[6]), f(th[2]));
    u[0] = f(__uint_as_float(sel(m1, hi, lo)) - m);
  }
}

// lane L of acc takes the wave-uniform word val (v_writelane_b32; the lane
// select is an inline constant, so the word is the one scalar operand)
template <int L>
__device__ __forceinline__ uint32_t write_lane(uint32_t acc, uint32_t val) {
  asm("v_writelane_b32 %0, %1, %2" : "+v"(acc) : "s"(val), "n"(L));
  return acc;
}
// f(IC<I>{}) for I = B .. E-1, each I a compile-time constant
template <int V>
struct IC {
  static constexpr int value = V;
};
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IC<B>{});
    static_for<B + 1, E>(f);
  }
}

struct WhtSigns {
  uint32_t pm[128];   // bf16 pair k (coordinates 2k, 2k+1): bit 15 / bit 31 set where D is -1
};

template <int D, int BP, int MODE, bool BF16>
__global__ void __launch_bounds__(256, (BP == 1 ? 2 : 3)) encode_wht_kernel(const void* __restrict__ x, int64_t nseq, int64_t n,
                                                         WhtSigns sg, Codebook cb, uint32_t* __restrict__ codes,
                                                         float* __restrict__ norms) {
  static_assert(D >= 32 && D <= 256 && (D & (D - 1)) == 0, "d: a power of two from 32 to 256");
  static_assert(MODE == 1 || MODE == 2, "values or MSE-only keys");
  constexpr int S = D > 128 ? D / 128 : 1;   // lanes per token
  constexpr int DL = D / S;                  // coordinates per lane
  constexpr int TPW = 64 / S;                // tokens per wave
  constexpr int KH = 1 << (BP - 1);          // centroids per half of the symmetric codebook
  constexpr int NJ = BP > 1 ? BP - 1 : 1;
  const int lane = threadIdx.x & 63;
  const int64_t tiles = (n + TPW - 1) / TPW;   // per sequence
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wid >= nseq * tiles) return;   // the whole wave
  const int64_t seq = wid / tiles, r = wid - seq * tiles;
  const int64_t t0 = r * TPW;
  const int rows = static_cast<int>(min(static_cast<int64_t>(TPW), n - t0));
  const int tok = lane & (TPW - 1), part = lane / TPW;
  const bool live = tok < rows;
  const uint64_t lm = __ballot(live);

  // ---- load this lane's coordinates part*DL .. +DL-1 (rows past n re-read the last one) ----
  float v[DL];
  {
    const int64_t row = seq * n + t0 + min(tok, rows - 1);
    if constexpr (BF16) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + row * D + part * DL);
      uint4 raw[DL / 8];
#pragma unroll
      for (int j = 0; j < DL / 8; ++j) raw[j] = src[j];
#pragma unroll
      for (int j = 0; j < DL / 8; ++j) {
        const uint32_t u[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 4 * j + e;   // pair within the lane's slice
          const uint32_t xm = S == 1 ? sg.pm[k] : (part ? sg.pm[DL / 2 + k] : sg.pm[k]);
          const uint32_t w = u[e] ^ xm;
          v[2 * k] = __uint_as_float(w << 16);
          v[2 * k + 1] = __uint_as_float(w & 0xFFFF0000u);
        }
      }
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + row * D + part * DL);
      uint4 raw[DL / 4];
#pragma unroll
      for (int j = 0; j < DL / 4; ++j) raw[j] = src[j];
#pragma unroll
      for (int j = 0; j < DL / 4; ++j) {
        const uint32_t u[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 4 * j + e;
          const int k = c >> 1;
          const uint32_t pmk = S == 1 ? sg.pm[k] : (part ? sg.pm[DL / 2 + k] : sg.pm[k]);
          const uint32_t xm = (c & 1) ? (pmk & 0x80000000u) : (pmk << 16);
          v[c] = __uint_as_float(u[e] ^ xm);
        }
      }
    }
  }
  // ---- v = H (D x): butterflies over pairs (i, i + h), h = 1, 2, ..., the last across the lane pair ----
#pragma unroll
  for (int h = 1; h < DL; h <<= 1)
#pragma unroll
    for (int i = 0; i < DL; ++i)
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
  if constexpr (S == 2) {
    // coordinate c of part 0 pairs with c + 128 of part 1: part 0 keeps a + b, part 1 a - b
    const float sgn = part ? -1.f : 1.f;
#pragma unroll
    for (int c = 0; c < DL; ++c) v[c] = fmaf(sgn, v[c], __shfl_xor(v[c], 32));
  }
  // ---- ||x||: H H^T = d I, so ||v||^2 = d ||x||^2 (taken from v, so that x
  // need not stay live through the butterflies) ----
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < DL; ++c) ss = fmaf(v[c], v[c], ss);
  if constexpr (S == 2) ss += __shfl_xor(ss, 32);
  const float nv = sqrtf(ss * (1.f / static_cast<float>(D)));
  // ---- thresholds of |y| scaled to v: y > t  <=>  v > t ||x|| sqrt(d) ----
  const float tsc = nv * sqrtf(static_cast<float>(D));
  float thr[KH > 1 ? KH - 1 : 1];
#pragma unroll
  for (int k = 0; k + 1 < KH; ++k) thr[k] = cb.t[KH + k] * tsc;

  if constexpr (MODE == 1) {
    // ---- values: plane words of 32 tokens, coordinate-major ----
    const int64_t nb = (n + 31) >> 5;
    // word (block, plane p, coordinate c) of the low / high half of a mask
    const int64_t blk0 = S == 1 ? 2 * r : r;
    const bool has1 = S == 2 || blk0 + 1 < nb;
    uint32_t acc0[BP], acc1[BP];
#pragma unroll
    for (int p = 0; p < BP; ++p) acc0[p] = acc1[p] = 0u;
    static_for<0, DL>([&](auto ci) {
      constexpr int c = decltype(ci)::value;
      const float a = v[c];
      bool jb[NJ];
      if constexpr (BP > 1) decide_bits<BP - 1, BP - 2>(fabsf(a), thr, jb);
      else jb[0] = false;
      // sign plane [y > 0]; low planes [bit of j == sign]; padding tokens 0
      const uint64_t sm = __ballot(a > 0.f) & lm;
#pragma unroll
      for (int p = 0; p < BP; ++p) {
        const uint64_t m = p == BP - 1 ? sm : ~(__ballot(jb[p < BP - 1 ? p : 0]) ^ sm) & lm;
        acc0[p] = write_lane<(c & 63)>(acc0[p], static_cast<uint32_t>(m));
        acc1[p] = write_lane<(c & 63)>(acc1[p], static_cast<uint32_t>(m >> 32));
      }
      if constexpr ((c & 63) == 63 || c == DL - 1) {
        const int cb0 = c & ~63;
        if (lane <= (c & 63)) {
#pragma unroll
          for (int p = 0; p < BP; ++p) {
            const int64_t w0 = ((seq * nb + blk0) * BP + p) * D + cb0 + lane;
            codes[w0] = acc0[p];
            if (S == 2) codes[w0 + DL] = acc1[p];                                   // coordinate 128 + c
            else if (has1) codes[w0 + static_cast<int64_t>(BP) * D] = acc1[p];     // block blk0 + 1
          }
        }
      }
    });
  } else {
    // ---- MSE-only keys: this lane's groups of 32 coordinates, token-major words ----
    constexpr int GL = DL / 32;
    constexpr int G = D / 32;
    uint32_t* dst = codes + ((seq * n + t0 + tok) * G + part * GL) * BP;
    // Each decision is the sign bit of a difference (exact: a difference of
    // distinct floats is never zero): [y > 0] of 0 - v, [|y| > t] of t - |v|.
    // alignbit(w, u, 31) = (w << 1) | (u >> 31) shifts it into the word, so
    // the decisions stay vector bits (no lane masks held in scalar registers).
    // Words are built from coordinate 32 g + 31 down, so bit c ends at c.
#pragma unroll
    for (int g = 0; g < GL; ++g) {
      uint32_t ws = 0u, wj[NJ];
#pragma unroll
      for (int p = 0; p < NJ; ++p) wj[p] = 0u;
#pragma unroll
      for (int c = 31; c >= 0; --c) {
        const float a = v[32 * g + c];
        ws = __builtin_amdgcn_alignbit(ws, __float_as_uint(0.f - a), 31);
        if constexpr (BP > 1) {
          uint32_t u[NJ];
          mag_sign_bits<BP - 1>(fabsf(a), thr, u);
#pragma unroll
          for (int p = 0; p < NJ; ++p) wj[p] = __builtin_amdgcn_alignbit(wj[p], u[p], 31);
        }
      }
      if (live) {
        // sign plane [y > 0]; low planes [bit of j == sign]
        dst[g * BP + BP - 1] = ws;
#pragma unroll
        for (int p = 0; p + 1 < BP; ++p) dst[g * BP + p] = ~(wj[p] ^ ws);
      }
    }
  }
  if (part == 0 && live) norms[seq * n + t0 + tok] = nv;
}

template <int D, int MODE, bool BF16>
hipError_t launch_encode_wht_d(const tq_quantizer* q, const void* x, int64_t nseq, int64_t n, uint32_t* codes,
                               float* norms, hipStream_t st) {
  WhtSigns sg;
  // row 0 of Pi is D / sqrt(d) (row 0 of H is all ones)
  for (int k = 0; k < D / 2; ++k)
    sg.pm[k] = (q->pi[2 * k] < 0 ? 0x8000u : 0u) | (q->pi[2 * k + 1] < 0 ? 0x80000000u : 0u);
  for (int k = D / 2; k < 128; ++k) sg.pm[k] = 0u;
  constexpr int TPW = D > 128 ? 64 / (D / 128) : 64;
  const int64_t waves = nseq * ((n + TPW - 1) / TPW);
  if ((waves + 3) / 4 > 0x7FFFFFFFll) return hipErrorNotSupported;
  const dim3 grid(static_cast<unsigned>((waves + 3) / 4));
  const Codebook& cb = q->cb[1];
  switch (cb.bp) {
#define TQ_WHT(BPV)                                                                                       \
  case BPV:                                                                                               \
    hipLaunchKernelGGL((encode_wht_kernel<D, BPV, MODE, BF16>), grid, dim3(256), 0, st, x, nseq, n, sg, cb, \
                       codes, norms);                                                                     \
    break;
    TQ_WHT(1) TQ_WHT(2) TQ_WHT(3) TQ_WHT(4)
#undef TQ_WHT
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

template <int MODE, bool BF16>
hipError_t launch_encode_wht_m(const tq_quantizer* q, const void* x, int64_t nseq, int64_t n, uint32_t* codes,
                               float* norms, hipStream_t st) {
  switch (q->d) {
    case 32: return launch_encode_wht_d<32, MODE, BF16>(q, x, nseq, n, codes, norms, st);
    case 64: return launch_encode_wht_d<64, MODE, BF16>(q, x, nseq, n, codes, norms, st);
    case 128: return launch_encode_wht_d<128, MODE, BF16>(q, x, nseq, n, codes, norms, st);
    case 256: return launch_encode_wht_d<256, MODE, BF16>(q, x, nseq, n, codes, norms, st);
    default: return hipErrorNotSupported;
  }
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

static int device_cu_count() {
  static int cus = [] {
    int dev = 0, c = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1)
      c = 256;
    return c;
  }();
  return cus;
}

// Persistent grid of the tile encoder: as many workgroups as fit on the chip
// at once for this instantiation (its registers and LDS decide: two per CU
// for prod keys, three or four for values and MSE-only keys; one for the
// eight-wave kernel with prod keys), so that every resident slot loops over
// tiles.
template <int KS, int LK, int MODE, int BPV, bool FULL, bool HAD>
int encode_tile_grid() {
  static const int blocks = [] {
    int per = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per, reinterpret_cast<const void*>(&encode_tile_kernel<KS, LK, MODE, BPV, FULL, HAD>), 64 * KS, 0) !=
            hipSuccess ||
        per < 1) {
      (void)hipGetLastError();
      per = KS == 4 ? 2 : 1;
    }
    return std::min(per, 4) * device_cu_count();
  }();
  return blocks;
}

template <int KS, int LK, int MODE, bool FULL, bool HAD = false>
hipError_t launch_encode_tile_m(const tq_quantizer* q, const void* x, int dtype, int64_t nseq, int64_t n,
                                uint32_t* codes, float* norms, float* gammas, hipStream_t st) {
  const int64_t tiles = nseq * ((n + kEncRows - 1) / kEncRows);
  const Codebook& cb = q->cb[MODE == 0 ? 0 : 1];
  const _Float16* wt = reinterpret_cast<const _Float16*>(q->d_wide);
  if (KS == 8 && !wt) return hipErrorNotSupported;
#define TQ_ENC(BPV)                                                                                                  \
  {                                                                                                                  \
    const dim3 grid(static_cast<unsigned>(std::min<int64_t>(tiles, encode_tile_grid<KS, LK, MODE, BPV, FULL, HAD>()))); \
    hipLaunchKernelGGL((encode_tile_kernel<KS, LK, MODE, BPV, FULL, HAD>), grid, dim3(64 * KS), 0, st, x, dtype, nseq, \
                       n, q->d, q->d_pi, q->d_sp, wt, cb, codes, norms, gammas);                                     \
  }
  switch (cb.bp) {
    case 1: TQ_ENC(1) break;
    case 2: TQ_ENC(2) break;
    case 3: TQ_ENC(3) break;
    case 4:
      if constexpr (MODE != 0) {
        TQ_ENC(4)
        break;
      }
      return hipErrorNotSupported;
    default: return hipErrorNotSupported;
  }
#undef TQ_ENC
  return hipGetLastError();
}

// Prod keys at d = 128 (rows in 16-byte runs; HAD: the Hadamard rotation): the
// role-split key encoder, one eight-wave workgroup per CU (its LDS holds two
// tiles of x and of rho and three of words)
template <int LK, bool HAD>
hipError_t launch_encode_keys_split(const tq_quantizer* q, const void* x, int64_t nseq, int64_t n, uint32_t* codes,
                                    float* norms, float* gammas, hipStream_t st) {
  const int64_t tiles = nseq * ((n + kEncRows - 1) / kEncRows);
  if (tiles == 0) return hipSuccess;
  const Codebook& cb = q->cb[0];
  const dim3 grid(static_cast<unsigned>(std::min<int64_t>(tiles, device_cu_count())));
#define TQ_SPLIT(B)                                                                                                \
  hipLaunchKernelGGL((encode_keys_split_kernel<LK, B, HAD>), grid, dim3(512), 0, st, x, nseq, n, q->d_pi, q->d_sp, cb, \
                     codes, norms, gammas)
  switch (cb.bp) {
    case 1: TQ_SPLIT(1); break;
    case 2: TQ_SPLIT(2); break;
    case 3: TQ_SPLIT(3); break;
    default: return hipErrorNotSupported;
  }
#undef TQ_SPLIT
  return hipGetLastError();
}

template <int LK>
hipError_t launch_encode_tile_lk(const tq_quantizer* q, int mode, const void* x, int dtype, int64_t nseq, int64_t n,
                                 uint32_t* codes, float* norms, float* gammas, hipStream_t st) {
  // d = 128 (the usual head dimension) takes the variant without coordinate guards
  constexpr bool F = LK != 0;
  if constexpr (F) {
    if (q->d == 128 && q->rotation == 1) {   // TQ_ROT_HADAMARD: the exact +-1 rotation operand
#ifndef TQ_NO_SPLIT_ENCODE
      if (mode == 0) return launch_encode_keys_split<LK, true>(q, x, nseq, n, codes, norms, gammas, st);
#endif
      if (mode == 0) return launch_encode_tile_m<4, LK, 0, true, true>(q, x, dtype, nseq, n, codes, norms, gammas, st);
      if (mode == 1) return launch_encode_tile_m<4, LK, 1, true, true>(q, x, dtype, nseq, n, codes, norms, gammas, st);
      return launch_encode_tile_m<4, LK, 2, true, true>(q, x, dtype, nseq, n, codes, norms, gammas, st);
    }
  }
  if (F && q->d == 128) {
#ifndef TQ_NO_SPLIT_ENCODE
    if constexpr (F) {
      if (mode == 0) return launch_encode_keys_split<LK, false>(q, x, nseq, n, codes, norms, gammas, st);
    }
#endif
    if (mode == 0) return launch_encode_tile_m<4, LK, 0, F>(q, x, dtype, nseq, n, codes, norms, gammas, st);
    if (mode == 1) return launch_encode_tile_m<4, LK, 1, F>(q, x, dtype, nseq, n, codes, norms, gammas, st);
    return launch_encode_tile_m<4, LK, 2, F>(q, x, dtype, nseq, n, codes, norms, gammas, st);
  }
  if (mode == 0) return launch_encode_tile_m<4, LK, 0, false>(q, x, dtype, nseq, n, codes, norms, gammas, st);
  if (mode == 1) return launch_encode_tile_m<4, LK, 1, false>(q, x, dtype, nseq, n, codes, norms, gammas, st);
  return launch_encode_tile_m<4, LK, 2, false>(q, x, dtype, nseq, n, codes, norms, gammas, st);
}

// 128 < d <= 256 with rows in 16-byte runs: the eight-wave tile kernel
// (operands streamed from the quantizer's fp16 tables)
template <int LK>
hipError_t launch_encode_wide_lk(const tq_quantizer* q, int mode, const void* x, int dtype, int64_t nseq, int64_t n,
                                 uint32_t* codes, float* norms, float* gammas, hipStream_t st) {
  if (q->d == 256) {
    if (mode == 0) return launch_encode_tile_m<8, LK, 0, true>(q, x, dtype, nseq, n, codes, norms, gammas, st);
    if (mode == 1) return launch_encode_tile_m<8, LK, 1, true>(q, x, dtype, nseq, n, codes, norms, gammas, st);
    return launch_encode_tile_m<8, LK, 2, true>(q, x, dtype, nseq, n, codes, norms, gammas, st);
  }
  if (mode == 0) return launch_encode_tile_m<8, LK, 0, false>(q, x, dtype, nseq, n, codes, norms, gammas, st);
  if (mode == 1) return launch_encode_tile_m<8, LK, 1, false>(q, x, dtype, nseq, n, codes, norms, gammas, st);
  return launch_encode_tile_m<8, LK, 2, false>(q, x, dtype, nseq, n, codes, norms, gammas, st);
}

hipError_t launch_encode_tile(const tq_quantizer* q, int mode, const void* x, int dtype, int64_t nseq, int64_t n,
                              uint32_t* codes, float* norms, float* gammas, hipStream_t st) {
  const int esz = dtype == 1 ? 2 : 4;
  if ((q->d * esz) % 16 != 0) return launch_encode_tile_lk<0>(q, mode, x, dtype, nseq, n, codes, norms, gammas, st);
  if (dtype == 1) return launch_encode_tile_lk<1>(q, mode, x, dtype, nseq, n, codes, norms, gammas, st);
  return launch_encode_tile_lk<2>(q, mode, x, dtype, nseq, n, codes, norms, gammas, st);
}

// The Walsh-Hadamard encoder takes the structured rotation wherever it
// applies (values and MSE-only keys, d a power of two from 32 to 256); prod
// keys need the dense S' contraction anyway and stay on the tile kernel.
bool encode_uses_wht(const tq_quantizer* q, int mode) {
#ifndef TQ_NO_WHT_ENCODE
  return q->rotation == 1 && mode != 0 && q->d >= 32 && q->d <= 256 && (q->d & (q->d - 1)) == 0;
#else
  (void)q;
  (void)mode;
  return false;
#endif
}

hipError_t launch_encode(const tq_quantizer* q, int mode, const void* x, int dtype, int64_t nseq, int64_t n,
                         uint32_t* codes, float* norms, float* gammas, hipStream_t st) {
  if (encode_uses_wht(q, mode)) {
    if (mode == 1)
      return dtype == 1 ? launch_encode_wht_m<1, true>(q, x, nseq, n, codes, norms, st)
                        : launch_encode_wht_m<1, false>(q, x, nseq, n, codes, norms, st);
    return dtype == 1 ? launch_encode_wht_m<2, true>(q, x, nseq, n, codes, norms, st)
                      : launch_encode_wht_m<2, false>(q, x, nseq, n, codes, norms, st);
  }
  if (q->d <= 128) {
    return launch_encode_tile(q, mode, x, dtype, nseq, n, codes, norms, gammas, st);
  }
  if (q->d <= kWideK && q->d_wide && (q->d * (dtype == 1 ? 2 : 4)) % 16 == 0) {
    return dtype == 1 ? launch_encode_wide_lk<1>(q, mode, x, dtype, nseq, n, codes, norms, gammas, st)
                      : launch_encode_wide_lk<2>(q, mode, x, dtype, nseq, n, codes, norms, gammas, st);
  }
  if (q->d > kWideK) {
    if (q->d > kMaxEncodeD) return hipErrorNotSupported;
    // values: tiles of 32 (one token word); keys: 16
    const int rows = mode == 1 ? 32 : 16;
    const size_t lds = encode_big_lds_bytes(q->d, rows, mode != 1);
    dim3 grid(static_cast<unsigned>((n + rows - 1) / rows), static_cast<unsigned>(nseq));
    const float* spt = q->d_spt;
    const Codebook& cb = q->cb[mode == 0 ? 0 : 1];
    const int ntw = ((q->d + 15) / 16 + 3) / 4;
#define TQ_BIG(ROWS, NTWV)                                                                                      \
  hipLaunchKernelGGL((encode_big_kernel<ROWS, NTWV>), grid, dim3(kThreads), lds, st, x, dtype, n, q->d, mode, q->d_qt, \
                     q->d + q->m, spt, cb, codes, norms, gammas)
    if (rows == 32) {
      if (ntw <= 8) TQ_BIG(32, 8); else TQ_BIG(32, 16);
    } else {
      if (ntw <= 8) TQ_BIG(16, 8); else TQ_BIG(16, 16);
    }
#undef TQ_BIG
    return hipGetLastError();
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
#define TQ_ATTR_BIG(ROWS, NTWV, KEYS)                                                                        \
  if (e == hipSuccess)                                                                                       \
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&encode_big_kernel<ROWS, NTWV>),                   \
                            hipFuncAttributeMaxDynamicSharedMemorySize,                                     \
                            static_cast<int>(encode_big_lds_bytes(kMaxEncodeD, ROWS, KEYS)));
    TQ_ATTR_BIG(16, 8, true) TQ_ATTR_BIG(16, 16, true) TQ_ATTR_BIG(32, 8, false) TQ_ATTR_BIG(32, 16, false)
#undef TQ_ATTR_BIG
    return e;
  }();
  return once;
}

}  // namespace tq

