// Kernel launchers (internal).  Arguments are validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "tq_internal.h"

namespace tq {

size_t encode_lds_bytes(int d);
hipError_t launch_encode(const tq_quantizer* q, int mode, const void* x, int dtype, int64_t nseq, int64_t n,
                         uint32_t* codes, float* norms, float* gammas, hipStream_t st);
hipError_t launch_decode(const tq_quantizer* q, int mode, const uint32_t* codes, const float* norms, const float* gammas,
                         int64_t nseq, int64_t n, float* out, hipStream_t st);

int64_t scores_ws_bytes(const tq_quantizer* q, int B, int Hq, int Hkv);

// query operands of up to kPrepSetMax quantizers of one d in one launch
constexpr int kPrepSetMax = 4;
struct PrepSet {
  const float* qt[kPrepSetMax];
  Codebook cb[kPrepSetMax];
  int qjl[kPrepSetMax];
  uint8_t* wsA[kPrepSetMax];
  float* wsC[kPrepSetMax];
};
hipError_t launch_query_prep_multi(const tq_quantizer* const* qs, void* const* ws, int nq, const void* queries,
                                   int q_dtype, int B, int Hq, int Hkv, hipStream_t st);
// bound: also the limb bounds the bounded top-k scan reads (constants 10, 11)
hipError_t launch_query_prep_ws(const tq_quantizer* q, const void* queries, int q_dtype, int B, int Hq, int Hkv,
                                void* ws, hipStream_t st, bool bound = false);
hipError_t launch_scores_scan(const tq_quantizer* q, int B, int Hq, int Hkv, const uint32_t* codes, const float* norms,
                              const float* gammas, int64_t n, float* out, const void* ws, hipStream_t st);
hipError_t launch_scores(const tq_quantizer* q, const void* queries, int q_dtype, int B, int Hq, int Hkv,
                         const uint32_t* codes, const float* norms, const float* gammas, int64_t n, float* out,
                         void* ws, hipStream_t st);

int64_t topk_ws_bytes(const tq_quantizer* q, int B, int Hq, int Hkv, int64_t n, int topk);
hipError_t launch_topk(const tq_quantizer* q, const void* queries, int q_dtype, int B, int Hq, int Hkv,
                       const uint32_t* codes, const float* norms, const float* gammas, int64_t n, int topk,
                       float* out, int64_t* out_idx, void* ws, hipStream_t st);

// one segment of a compressed cache (its quantizers, packed arrays, tokens per sequence)
struct AttendSegment {
  const tq_quantizer* kq;
  const tq_quantizer* vq;
  const uint32_t* kcodes;
  const float* knorms;
  const float* kgammas;
  const uint32_t* vcodes;
  const float* vnorms;
  int64_t n;
};

int64_t attend_ws_bytes(const tq_quantizer* kq, const tq_quantizer* vq, int B, int Hq, int Hkv, int64_t n_comp,
                        int n_tail);
int64_t attend_segments_ws_bytes(const AttendSegment* segs, int nseg, int B, int Hq, int Hkv);
bool attend_supports_d(int d);   // head dimensions the attention kernels are built for
hipError_t launch_attend_segments(const AttendSegment* segs, int nseg, const void* queries, int q_dtype, int B, int Hq,
                                  int Hkv, const uint16_t* k_tail, const uint16_t* v_tail, int n_tail, float scale,
                                  float vtau, float* out, void* ws, hipStream_t st);
hipError_t launch_attend(const tq_quantizer* kq, const tq_quantizer* vq, const void* queries, int q_dtype, int B, int Hq,
                         int Hkv, const uint32_t* kcodes, const float* knorms, const float* kgammas,
                         const uint32_t* vcodes, const float* vnorms, int64_t n_comp, const uint16_t* k_tail,
                         const uint16_t* v_tail, int n_tail, float scale, float vtau, float* out, void* ws,
                         hipStream_t st);

hipError_t set_kernel_attributes();

}  // namespace tq
