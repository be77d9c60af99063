/*
 * tq.h -- C ABI of libtq, the TurboQuant hot path for AMD Instinct MI355X
 * (gfx950).
 *
 * The method (TurboQuant) is described on these pages; citations below name
 * the page by site and title and the section on it:
 *   [hotdry]  blog.hotdry.top, "TurboQuant vector-search compression":
 *             sections "随机旋转与标量量化" (random rotation + scalar
 *             quantisation), "QJL 残差校正" (QJL residual correction),
 *             "工程配置参数清单" (engineering configuration), "精度调优与
 *             监控要点" (accuracy tuning and monitoring: an MSE-only mode
 *             without the QJL correction, for workloads where it ranks better)
 *   [a2a]     a2a-mcp.org, "什麼是TurboQuant？": sections "第一階段" (stage 1:
 *             rotation + Lloyd-Max), "第二階段" (stage 2: QJL), "如何實作
 *             TurboQuant" (how to implement: precompute codebooks, quantise at
 *             every cache update, fused logits from indices with the query
 *             rotated once)
 *   [friday]  friday-blog, "TurboQuant 深度解析（二）": section "1. 三步壓縮的
 *             數學細節" (rotation, QJL, residual correction)
 *   [wiselychen] ai-coding.wiselychen.com, "Google TurboQuant：KV Cache 壓縮
 *             6x…": section "最猛的社群實作：TurboQuant+" (a Walsh-Hadamard
 *             rotation in a community implementation; near-Gaussian rotated
 *             coordinates; "Sparse V": the value work of low-weight tokens
 *             skipped)
 *
 * Conventions
 *   - Every array argument of the compute calls (tq_encode, tq_decode,
 *     tq_scores, tq_attend_decode) is a DEVICE pointer on the device that was
 *     current when the quantizer was made; the caller owns all of them.  The
 *     library owns only the quantizer and its device tables.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Compute calls
 *     are asynchronous on that stream; they never allocate device memory and
 *     never synchronise.
 *   - Calls return TQ_OK (0) or a negative status; they never abort.  A
 *     description of the last failure on the calling thread is available from
 *     tq_last_error().  Arguments are checked on the host before any launch;
 *     NaN/Inf input values are not checked (their codes are unspecified).
 *   - Device pointers must be 16-byte aligned.
 *
 * Packed layouts (ours; the pages fix the bit budget -- b-1 index bits and one
 * QJL bit per coordinate for keys, plus the norms -- not a byte order):
 *   prod (keys):  uint32 words [nseq][n][G][b], G = ceil(d/32).  Word (g, p)
 *                 for p < b-1 holds bit p of the Lloyd-Max index of coordinates
 *                 32g..32g+31 (bit i <-> coordinate 32g+i); word (g, b-1) holds
 *                 the QJL sign bits of projections 32g..32g+31 (1 = non-negative).
 *                 Plus float norms [nseq][n] and float gammas [nseq][n].
 *   mse keys:     uint32 words [nseq][n][G][b]: the prod layout with all b
 *                 words holding index bits (word (g, p) = bit p of the b-bit
 *                 index), no QJL plane.  Plus float norms [nseq][n] only.
 *   mse (values): uint32 words [nseq][ceil(n/32)][b][d].  Word (blk, p, j)
 *                 holds bit p of the index of coordinate j of tokens
 *                 32blk..32blk+31 (bit i <-> token 32blk+i); bits of padding
 *                 tokens are 0.  Plus float norms [nseq][n].
 *   Index 0 is the most negative centroid.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  TQ_OK = 0,
  TQ_EINVAL = -1,        /* bad argument (null pointer, size, mode, alignment) */
  TQ_EUNSUPPORTED = -2,  /* valid but not implemented for this shape */
  TQ_EHIP = -3,          /* a HIP runtime call failed */
  TQ_ENOMEM = -4,        /* host or device allocation failed (tq_make_quantizer only) */
  TQ_EWORKSPACE = -5     /* workspace smaller than the size query returned */
};

enum { TQ_PROD = 0,     /* keys: (bits-1)-bit Lloyd-Max index + 1-bit QJL sketch */
       TQ_MSE = 1,      /* values: bits-bit Lloyd-Max index only */
       TQ_MSE_KEYS = 2  /* keys without QJL: bits-bit index, token-major ([hotdry] accuracy tuning) */ };

enum { TQ_F32 = 0, TQ_BF16 = 1 };

enum { TQ_ROT_HAAR = 0,      /* dense Haar rotation: QR of a Gaussian matrix ([a2a] stage 1) */
       TQ_ROT_HADAMARD = 1   /* structured: H D / sqrt(d) ([wiselychen] community implementation) */ };

typedef struct tq_quantizer tq_quantizer;

/* Layout/ABI version of this header. */
int tq_version(void);

/* Description of the last failure on this thread ("" if none). */
const char* tq_last_error(void);

/* ------------------------------------------------------------------------
 * Host-only precompute (no GPU needed).  All outputs are host arrays the
 * caller allocates.
 * ------------------------------------------------------------------------ */

/* n standard normals of stream `tag` (1 = rotation, 2 = QJL) of quantizer
 * seed `seed`: SplitMix64 (Steele, Lea & Flood 2014) from state
 * seed XOR (tag << 56), uniforms ((z >> 11) + 0.5) * 2^-53, Box-Muller on
 * consecutive pairs (cos first).  The pages name no generator. */
int tq_host_normals(uint64_t seed, int tag, int64_t n, double* out);

/* Random orthogonal rotation Pi (d x d, row major, y = Pi x): the orthogonal
 * factor of the QR decomposition G = Pi R with positive diag(R), G filled
 * row major from stream 1 ([a2a] stage 1: rotation by QR of a Gaussian
 * matrix).  3 <= d <= 1024. */
int tq_host_rotation(int d, uint64_t seed, double* pi_out);

/* Structured rotation Pi = H D / sqrt(d) (d x d, row major): H the
 * Sylvester-Hadamard matrix, H[i][j] = (-1)^popcount(i & j); D = diag of d
 * random signs, sign j = -1 when the top bit of output j of stream 3 is set
 * ([wiselychen] community implementation: Walsh-Hadamard rotation; the signs
 * and the ordering are our reading).  d a power of two in [4, 1024]. */
int tq_host_rotation_hadamard(int d, uint64_t seed, double* pi_out);

/* QJL matrix S (m x d, row major), iid N(0,1) from stream 2 ([hotdry] QJL
 * section). */
int tq_host_qjl_matrix(int m, int d, uint64_t seed, double* s_out);

/* Lloyd-Max codebook with `levels` (2,4,8,16) cells for the law of one
 * coordinate of a uniform unit vector in R^d, density ~ (1-x^2)^((d-3)/2)
 * on [-1,1] ([a2a] stage 1: Beta((d-1)/2,(d-1)/2) on [-1,1]; [hotdry]
 * random rotation section).  centroids[levels] ascending and symmetric,
 * thresholds[levels-1] = midpoints. */
int tq_host_codebook(int d, int levels, double* centroids, double* thresholds);

/* ------------------------------------------------------------------------
 * Quantizer: everything the method precomputes offline for (d, bits, seed)
 * ([a2a] how to implement: precompute the codebooks for the head dimension
 * and bit width).  Holds Pi, S (m = d rows), S' = S Pi^T, the (bits-1)-bit
 * codebook for keys and the bits-bit codebook for values, on the current
 * HIP device.  2 <= bits <= 4 (bits = 1 allows TQ_MSE only), 3 <= d <= 1024.
 * Returns NULL on failure (see tq_last_error).
 * ------------------------------------------------------------------------ */
tq_quantizer* tq_make_quantizer(int d, int bits, uint64_t seed);

/* As tq_make_quantizer with the rotation chosen: TQ_ROT_HAAR (the default
 * above) or TQ_ROT_HADAMARD (tq_host_rotation_hadamard; d a power of two).
 * Every compute call works with either: the kernels take Pi as a dense
 * matrix, so the structured rotation changes the codes, not the cost. */
tq_quantizer* tq_make_quantizer_ex(int d, int bits, uint64_t seed, int rotation);
void tq_free_quantizer(tq_quantizer* q);

/* d, bits, m of a quantizer (any output pointer may be NULL). */
int tq_quantizer_info(const tq_quantizer* q, int* d, int* bits, int* m);

/* Which key encoding the scoring calls (tq_scores, tq_query_prep,
 * tq_scores_from_prep, tq_attend_decode as kq) read from this quantizer:
 * TQ_PROD (the default; needs bits >= 2) or TQ_MSE_KEYS ([hotdry] accuracy
 * tuning section: the MSE-only mode, logit(q, i) = n_i <Pi q, c_b[index_i]>
 * with the bits-bit codebook).  Not thread-safe against concurrent calls on
 * the same quantizer; a query-prep workspace is only valid for the key mode
 * it was written under.  Returns TQ_EINVAL for any other value. */
int tq_set_key_mode(tq_quantizer* q, int key_mode);

/* Number of uint32 code words for nseq sequences of n vectors in `mode`. */
int64_t tq_code_words(const tq_quantizer* q, int mode, int64_t nseq, int64_t n);

/* Encode ([hotdry] both stages; [a2a] stage 1 and 2; [friday] steps 1-3):
 * n_i = ||x_i||; y = Pi x_i / n_i; index_j = #{k : t_k < y_j};
 * prod only: rho = y - c[index], gamma_i = n_i ||rho||,
 * QJL bit_r = [ (S' rho)_r >= 0 ] (S' rho = S r / n_i with r = x - x_hat).
 * A zero vector gets y = 0, index = levels/2 - 1, gamma = 0, all QJL bits 1.
 *   x:      [nseq][n][d] of dtype (TQ_F32 or TQ_BF16)
 *   codes:  tq_code_words(q, mode, nseq, n) uint32 words, layout above
 *   norms:  [nseq][n] float;  gammas: [nseq][n] float (prod), NULL or
 *           ignored (TQ_MSE, TQ_MSE_KEYS: those use the bits-bit codebook)
 * nseq*n may be 0 (no launch).  Every d of a quantizer (3 <= d <= 1024);
 * above 256 a general tile kernel (slower, fp32 matrix core). */
int tq_encode(const tq_quantizer* q, int mode, const void* x, int dtype, int64_t nseq, int64_t n,
              uint32_t* codes, float* norms, float* gammas, void* stream);

/* Decode ([hotdry] QJL section): prod: x~ = n Pi^T c[index] +
 * gamma sqrt(pi/2)/m S^T sigma, sigma = +-1; mse and mse keys:
 * x^ = n Pi^T c[index].
 * x_out: [nseq][n][d] float. */
int tq_decode(const tq_quantizer* q, int mode, const uint32_t* codes, const float* norms,
              const float* gammas, int64_t nseq, int64_t n, float* x_out, void* stream);

/* Attention logits straight from prod codes, the query rotated and projected
 * once ([a2a] stage 2 and how-to-implement: fused kernel from indices with a
 * pre-rotated query; [hotdry] QJL section: unbiased inner product):
 *   logit(q, i) = n_i <Pi q, c[index_i]> + gamma_i sqrt(pi/2)/m <S q, sigma_i>
 *   queries: [B][Hq][d] (q_dtype TQ_F32 or TQ_BF16); query head h reads KV
 *            head h / (Hq/Hkv) (Hq a multiple of Hkv)
 *   codes/norms/gammas: the encoding of [B*Hkv] sequences of n keys in the
 *            quantizer's key mode (tq_set_key_mode); with TQ_MSE_KEYS the
 *            logit has no QJL term and gammas may be NULL
 *   topk == 0: out = logits [B][Hq][n] float, out_idx unused (may be NULL)
 *   topk  > 0: out = the topk largest logits per query [B][Hq][topk] float,
 *              descending, ties by lower index; out_idx [B][Hq][topk] int64
 *              (1 <= topk <= 32)
 *   workspace: device scratch of at least tq_scores_workspace_bytes(...)
 *   d <= 256: the matrix-core scan; 256 < d <= 1024: logits only (topk == 0),
 *             a vector-ALU scan; topk > 0 there returns TQ_EUNSUPPORTED */
int64_t tq_scores_workspace_bytes(const tq_quantizer* q, int B, int Hq, int Hkv, int64_t n, int topk);

/* The two halves of tq_scores (topk == 0), for callers that score several
 * caches with the same queries or time the scan alone:
 * tq_query_prep rotates and projects the queries once and writes the
 * query-side MFMA operands into `workspace` (a2a how-to-implement: the query
 * is pre-rotated once); tq_scores_from_prep streams the packed keys against
 * them.  The workspace must not change between the two calls.  d <= 256
 * (TQ_EUNSUPPORTED above: tq_scores covers those). */
int tq_query_prep(const tq_quantizer* q, const void* queries, int q_dtype, int B, int Hq, int Hkv, void* workspace,
                  int64_t ws_bytes, void* stream);
int tq_scores_from_prep(const tq_quantizer* q, int B, int Hq, int Hkv, const uint32_t* codes, const float* norms,
                        const float* gammas, int64_t n, float* logits, const void* workspace, int64_t ws_bytes,
                        void* stream);

int tq_scores(const tq_quantizer* q, const void* queries, int q_dtype, int B, int Hq, int Hkv,
              const uint32_t* codes, const float* norms, const float* gammas, int64_t n, int topk,
              float* out, int64_t* out_idx, void* workspace, int64_t ws_bytes, void* stream);

/* Decode-step attention over a packed cache with an optional exact tail
 * ([hotdry] engineering configuration: recent 128-256 tokens kept in full
 * precision, older tokens compressed).  For each query head h of batch b:
 *   s_i = scale * logit(q, i) for compressed tokens (keys of kq in its key
 *         mode; kgammas may be NULL for TQ_MSE_KEYS),
 *   s_i = scale * <q, k_tail_i> for tail tokens (bf16 keys),
 *   p = softmax(s) (max-subtracted, float),
 *   out = sum_i p_i v_i, v_i = n_i Pi_v^T c_v[index_i] (mse values of vq) or
 *         the bf16 tail value.
 *   queries [B][Hq][d]; kcodes/knorms/kgammas: key encoding of [B*Hkv]
 *   sequences of n_comp keys; vcodes/vnorms: mse encoding of the same;
 *   k_tail, v_tail: [B][Hkv][n_tail][d] bf16 (NULL if n_tail == 0);
 *   out: [B][Hq][d] float.  scale <= 0 selects 1/sqrt(d).
 *   n_comp + n_tail >= 1; kq and vq must have the same d, one of 64, 96,
 *   128 or 256 (TQ_EUNSUPPORTED otherwise); n_tail <= 512.
 *   workspace: device scratch of at least tq_attend_workspace_bytes(...) */
int64_t tq_attend_workspace_bytes(const tq_quantizer* kq, const tq_quantizer* vq, int B, int Hq, int Hkv,
                                  int64_t n_comp, int n_tail);
int tq_attend_decode(const tq_quantizer* kq, const tq_quantizer* vq, const void* queries, int q_dtype,
                     int B, int Hq, int Hkv, const uint32_t* kcodes, const float* knorms,
                     const float* kgammas, const uint32_t* vcodes, const float* vnorms, int64_t n_comp,
                     const uint16_t* k_tail, const uint16_t* v_tail, int n_tail, float scale, float* out,
                     void* workspace, int64_t ws_bytes, void* stream);

/* Sparse V ([wiselychen] TurboQuant+ table: the value work of low-weight
 * tokens is skipped).  tq_attend_decode with one more argument, v_threshold in
 * [0, 1) (TQ_EINVAL otherwise).  The weight of compressed token t is
 * w_t = p_t * n_t (softmax weight times value norm, the size of its term in
 * the output).  Tokens are visited in sequence order within chunks of at most
 * 1024 tokens; a token with w_t < v_threshold * (largest w so far in its
 * chunk, itself included) leaves the value sum, while its p_t stays in the
 * normaliser.  A 128-token step in which no weight is left (for any query of
 * the row tile) skips the value MFMAs.  Tail tokens are never dropped.
 * Because the running maximum never exceeds the overall one, the dropped set
 * lies inside D = {t : w_t < v_threshold * max_u w_u}, and each output element
 * differs from tq_attend_decode's by at most sum_{t in D} p_t |v_t[e]| / sum_t
 * p_t.  v_threshold = 0 gives tq_attend_decode's result bit for bit.
 * v_threshold > 0 needs d = 128 (TQ_EUNSUPPORTED otherwise). */
int tq_attend_decode_sparse(const tq_quantizer* kq, const tq_quantizer* vq, const void* queries, int q_dtype,
                            int B, int Hq, int Hkv, const uint32_t* kcodes, const float* knorms,
                            const float* kgammas, const uint32_t* vcodes, const float* vnorms, int64_t n_comp,
                            const uint16_t* k_tail, const uint16_t* v_tail, int n_tail, float scale,
                            float v_threshold, float* out, void* workspace, int64_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Temporal decay ([wiselychen] TurboQuant+ table: older tokens are kept at
 * a lower precision, a further 30-34% of memory at long context).  Reading:
 * the compressed cache is kept in age segments, each encoded with its own
 * quantizers (e.g. the newest tokens at 4 bits, older ones at 2); decode
 * attention runs one softmax over every segment and the exact tail; a token
 * moves to an older segment by tq_requantize.
 * ------------------------------------------------------------------------ */
#define TQ_MAX_SEGMENTS 16

/* One segment of a compressed cache: [B*Hkv] sequences of n tokens encoded
 * with kq (in its key mode; kgammas may be NULL for TQ_MSE_KEYS) and, for the
 * values, vq (TQ_MSE).  The value quantizers of all segments of one call must
 * share d, seed and rotation (hence Pi, whatever their widths): the value
 * sums of all segments are rotated back once.  Key quantizers are free. */
typedef struct tq_segment {
  const tq_quantizer* kq;
  const tq_quantizer* vq;
  const uint32_t* kcodes;
  const float* knorms;
  const float* kgammas;
  const uint32_t* vcodes;
  const float* vnorms;
  int64_t n;
} tq_segment;

/* Decode attention over nseg (1..TQ_MAX_SEGMENTS) segments plus the optional
 * bf16 tail: logits of every segment's tokens (by its own key quantizer) and
 * of the tail share one softmax; out = sum_i p_i v_i with each value decoded
 * by its segment's quantizer.  With one segment this is tq_attend_decode.
 * The order of the segments does not change the result beyond rounding.
 * queries [B][Hq][d], tails [B][Hkv][n_tail][d] bf16, out [B][Hq][d] float,
 * scale <= 0 selects 1/sqrt(d); d in {64, 96, 128, 256}.  workspace: at least
 * tq_attend_segments_workspace_bytes(...) bytes, 256-byte aligned. */
int64_t tq_attend_segments_workspace_bytes(const tq_segment* segs, int nseg, int B, int Hq, int Hkv, int n_tail);
int tq_attend_decode_segments(const tq_segment* segs, int nseg, const void* queries, int q_dtype, int B, int Hq,
                              int Hkv, const uint16_t* k_tail, const uint16_t* v_tail, int n_tail, float scale,
                              float* out, void* workspace, int64_t ws_bytes, void* stream);

/* Re-encode tokens at another width (a token ageing into an older segment):
 * decode the codes of `from` (x~ with the QJL term for TQ_PROD; x^ for TQ_MSE
 * and TQ_MSE_KEYS) and encode the result with `to` in the same mode.  The two
 * quantizers must have the same d.  codes_in/norms_in/gammas_in: the encoding
 * of [nseq][n] vectors by `from`; the outputs take `to`'s layout and sizes
 * (tq_code_words(to, mode, nseq, n) words).  workspace: nseq * n * d floats
 * (the decoded vectors), 16-byte aligned.  Asynchronous on `stream`. */
int tq_requantize(const tq_quantizer* from, const tq_quantizer* to, int mode, const uint32_t* codes_in,
                  const float* norms_in, const float* gammas_in, int64_t nseq, int64_t n, uint32_t* codes_out,
                  float* norms_out, float* gammas_out, void* workspace, int64_t ws_bytes, void* stream);

/* Allocation-free decode attention, for callers that cannot allocate device
 * memory: code under HIP graph capture, serving loops and harnesses that
 * forbid hipMalloc.  Same arguments and result as tq_attend_decode without
 * the workspace: the call uses a scratch array of TQ_NOALLOC_SCRATCH_BYTES
 * that the library holds on each device until the process ends (its address
 * is taken when the first quantizer is made on that device), and it calls no
 * allocating routine.  Shapes whose tq_attend_workspace_bytes(...) exceeds
 * TQ_NOALLOC_SCRATCH_BYTES are rejected with TQ_EWORKSPACE (16 MiB covers,
 * e.g., 8 x 8 KV heads x 32 query heads over 32768 tokens, which needs about
 * 4.7 MB).  Every call on a device shares that device's scratch: calls that
 * overlap on one device (two streams, two threads) race and give undefined
 * results; calls ordered on one stream are safe.  Nothing in the scratch
 * needs to start at zero: each call writes every byte it reads. */
#define TQ_NOALLOC_SCRATCH_BYTES (16ll << 20)
int tq_attend_decode_noalloc(const tq_quantizer* kq, const tq_quantizer* vq, const void* queries, int q_dtype,
                             int B, int Hq, int Hkv, const uint32_t* kcodes, const float* knorms,
                             const float* kgammas, const uint32_t* vcodes, const float* vnorms, int64_t n_comp,
                             const uint16_t* k_tail, const uint16_t* v_tail, int n_tail, float scale, float* out,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
