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
#include "tq_device.h"
#include "tq_kernels.h"

namespace tq {

namespace {

constexpr int kTileRows = 64;
constexpr int kThreads = 256;

// Y[16 rows of this wave][DP] = X[rows][0:d] * M^T, with M [rows_m][d] row
// major (row j of M gives output column j).  X in LDS with row stride `ld`.
// acc[ct] holds output column tile ct (16 columns) in MFMA C layout.
template <int NT>
__device__ __forceinline__ void gemm_rows_16(const float* xs, int ld, const float* __restrict__ M, int rows_m, int d,
                                             v4f (&acc)[NT]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) acc[ct] = (v4f){0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < d; k0 += 4) {
    const int k = k0 + kq;
    const float a = k < d ? xs[r * ld + k] : 0.f;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      const int j = ct * 16 + r;
      const float b = (k < d && j < rows_m) ? M[static_cast<int64_t>(j) * d + k] : 0.f;
      acc[ct] = mfma_f32(a, b, acc[ct]);
    }
  }
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) pin(acc[ct]);
}

template <int NT>
__global__ void __launch_bounds__(kThreads) encode_kernel(const void* __restrict__ x, int dtype, int64_t n, int d, int mode,
                                                          const float* __restrict__ pi, const float* __restrict__ sp,
                                                          Codebook cb, uint32_t* __restrict__ codes,
                                                          float* __restrict__ norms, float* __restrict__ gammas) {
  constexpr int DP = NT * 16;
  constexpr int LD = DP + 1;
  extern __shared__ float smem[];
  float* xs = smem;                                               // [64][LD] floats: x, then rho
  float* nrm = xs + kTileRows * LD;                               // [64]
  float* cen = nrm + kTileRows;                                   // [16]
  uint8_t* idxb = reinterpret_cast<uint8_t*>(cen + kMaxLevels);   // [64][DP]
  uint8_t* sgnb = idxb + kTileRows * DP;                          // [64][DP]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int64_t seq = blockIdx.y;
  const int64_t v0 = static_cast<int64_t>(blockIdx.x) * kTileRows;
  const int rows = static_cast<int>(n - v0 < kTileRows ? n - v0 : kTileRows);
  const int64_t base = seq * n + v0;   // first vector of the tile

  if (tid < kMaxLevels) cen[tid] = tid < cb.levels ? cb.c[tid] : 0.f;
  // ---- load the tile (coalesced), zero rows past n and columns past d ----
  for (int e = tid; e < kTileRows * DP; e += kThreads) {
    const int row = e / DP, col = e - row * DP;
    float v = 0.f;
    if (row < rows && col < d) v = load_elem(x, dtype, (base + row) * d + col);
    xs[row * LD + col] = v;
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

  // ---- rotation: y = Pi x / n ----
  const float* xw = xs + wave * 16 * LD;   // this wave's 16 rows
  v4f acc[NT];
  gemm_rows_16<NT>(xw, LD, pi, d, d, acc);

  const int col_in = lane & 15, rq = lane >> 4;   // C layout: rows 4*rq+i, column ct*16+col_in
  float inv_n[4], rho2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float nv = nrm[wave * 16 + 4 * rq + i];
    inv_n[i] = nv > 0.f ? 1.f / nv : 0.f;
    rho2[i] = 0.f;
  }
  // bucketize, residual; write rho back over this wave's rows of x
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    const int col = ct * 16 + col_in;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wave * 16 + 4 * rq + i;
      const float y = acc[ct][i] * inv_n[i];
      int idx = 0;
      for (int k = 0; k < cb.levels - 1; ++k) idx += (cb.t[k] < y) ? 1 : 0;
      const float rho = col < d ? y - cen[idx] : 0.f;
      if (col < d) rho2[i] = fmaf(rho, rho, rho2[i]);
      idxb[row * DP + col] = col < d ? static_cast<uint8_t>(idx) : 0;
      acc[ct][i] = rho;
    }
  }
  __syncthreads();   // all waves finished reading x before rho overwrites it
#pragma unroll
  for (int ct = 0; ct < NT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) xs[(wave * 16 + 4 * rq + i) * LD + ct * 16 + col_in] = acc[ct][i];

  if (mode == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float s = rho2[i];
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      s += __shfl_xor(s, 8);
      rho2[i] = s;
    }
    __syncthreads();
    // ---- QJL projection z = S' rho; bit = [z >= 0] (all ones for n = 0) ----
    gemm_rows_16<NT>(xw, LD, sp, d, d, acc);
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      const int col = ct * 16 + col_in;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wave * 16 + 4 * rq + i;
        const bool bit = (acc[ct][i] >= 0.f) || (inv_n[i] == 0.f);
        sgnb[row * DP + col] = (col < d && bit) ? 1 : 0;
      }
    }
    if (col_in == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wave * 16 + 4 * rq + i;
        if (row < rows) {
          const float nv = nrm[row];
          norms[base + row] = nv;
          gammas[base + row] = nv * sqrtf(rho2[i]);
        }
      }
    }
  } else {
    if (col_in == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wave * 16 + 4 * rq + i;
        if (row < rows) norms[base + row] = nrm[row];
      }
    }
  }
  __syncthreads();

  // ---- bit packing ----
  const int bp = cb.bp;
  if (mode == 0) {
    // prod: words [vec][g][bp+1]
    const int G = (d + 31) >> 5;
    const int W = bp + 1;
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
        w[bp] |= static_cast<uint32_t>(sb[i]) << i;
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
      if (mode == 0) {
        const int G = (d + 31) >> 5;
        const uint32_t* w = codes + ((seq * n + t) * G + (j >> 5)) * (bp + 1);
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
  hipLaunchKernelGGL((encode_kernel<NT>), grid, dim3(kThreads), lds, st, x, dtype, n, q->d, mode, q->d_pi, q->d_sp,
                     q->cb[mode], codes, norms, gammas);
  return hipGetLastError();
}

}  // namespace

size_t encode_lds_bytes(int d) {
  const int DP = ((d + 15) / 16) * 16;
  return sizeof(float) * (kTileRows * (DP + 1) + kTileRows + kMaxLevels) + 2 * kTileRows * DP;
}

hipError_t launch_encode(const tq_quantizer* q, int mode, const void* x, int dtype, int64_t nseq, int64_t n,
                         uint32_t* codes, float* norms, float* gammas, hipStream_t st) {
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
                     q->cb[mode], out);
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
