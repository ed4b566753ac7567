/*
 * tq.h -- C ABI of the TurboQuant KV-cache hot path for AMD MI355X (gfx950).
 *
 * The operations follow three public pages about TurboQuant:
 *   [P1] "TurboQuant KV 캐시 압축 for llama.cpp" (AmesianX README_KO on stig.sh)
 *   [P2] "윈도우용 터보퀀트(TurboQuant) 구현을 개선하다" (idea.jsleekr.com)
 *   [P3] "[GitHub 탐방] TurboQuant 3-bit KV 캐시 압축 — 단일 GPU 재현 기록" (velog.io)
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless marked "host".  The library never
 *     allocates, frees or synchronises inside tq_encode, tq_decode,
 *     tq_attn_decode or tq_ip_search: the caller owns every buffer.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls are asynchronous on that stream; results are valid once the
 *     stream has been synchronised.
 *   - Return value: TQ_OK (0) or a negative TQ_E* code.  All argument checks
 *     happen on the host before any launch; on an error nothing is launched
 *     and no output is touched.  TQ_EDEVICE reports a failed launch
 *     (hipGetLastError after the launch).
 *   - The library keeps no mutable global state: calls on different streams
 *     may run concurrently.
 *   - Non-finite inputs give unspecified (but in-bounds) results.
 *
 * Packed formats (all little-endian):
 *   codes  : one row of d*bits/8 bytes per vector; index i occupies bits
 *            [bits*i, bits*i + bits) of the row read as an LSB-first bit stream;
 *            index 0 is the most negative centroid.
 *   norms  : IEEE half (uint16) per vector, round to nearest even, clamped to 65504.
 *   qjl    : one row of m/8 bytes per vector; bit j (LSB-first) is 1 when the
 *            j-th projection of the residual is >= 0.
 *   gamma  : IEEE half per vector, the norm of the residual r (see tq_encode).
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    TQ_OK = 0,
    TQ_EINVAL = -1,        /* null pointer, bad size, stride or alignment      */
    TQ_EUNSUPPORTED = -2,  /* d, bits, qjl_m, k or head ratio outside support  */
    TQ_EWORKSPACE = -3,    /* workspace missing or smaller than required       */
    TQ_EDEVICE = -4,       /* the HIP runtime reported a launch failure        */
    TQ_ESCRATCH = -5       /* needs more than the no-alloc entry point's static scratch */
};

enum { TQ_F32 = 0, TQ_F16 = 1, TQ_BF16 = 2 };

/*
 * One quantiser: what the encoder and decoder of one cache (K or V) share.
 * Host struct, filled by tq_codebook and passed by pointer; the library copies
 * it by value into kernel arguments.
 *
 *   d           head dimension: 32, 64, 128, 256 or 512 (512: no residual).
 *               Attention: 128 and 256; 64 with 2- or 4-bit keys and 2..4-bit
 *               values.
 *   bits        1..4 bits per coordinate (L = 2^bits centroids).
 *   qjl_m       0, or the number of residual sign bits m (multiple of 32,
 *               <= 256; m = d for TQ_RES_SRHT and TQ_RES_SIGN).
 *   residual    TQ_RES_NONE (qjl_m = 0), or how the m residual bits are
 *               formed (K caches and search only):
 *                 TQ_RES_QJL   signs of S r for a caller-drawn Gaussian S
 *                              [m][d] ([P1] "QJL 보정 효과": TurboQuant_prod);
 *                 TQ_RES_SRHT  signs of H(D2 r), the structured projection
 *                              with the second sign basis D2 = sign_mask2
 *                              ([P1] v1.3.0: QJL is SRHT-based in the paper;
 *                              v1.4.2 item 2: its signs2);
 *                 TQ_RES_SIGN  Direct Sign: the signs of r itself, with the
 *                              mean |r_i| as the scale ([P1] v1.1.0 "Direct
 *                              Sign — 논문 QJL 대비 4.3배 낮은 분산").
 *   sign_mask   bit i (word i/32, bit i%32) set means D_ii = -1: the seeded
 *               random sign flip applied before the Walsh-Hadamard transform
 *               ([P1] v1.7.0 "핵심 설계 결정" item 4, "tbq_signs").
 *   centroid    L float32 Lloyd-Max centroids of N(0,1), ascending, exactly
 *               symmetric; entries >= L are 0.
 *   threshold   L-1 float32 midpoints; the middle one is exactly 0.
 *   sign_mask2  the second sign basis D2 of TQ_RES_SRHT (filled for every
 *               codec with d <= 256; bit i set means D2_ii = -1).
 *   rotation    the transform R after the sign flip D:
 *                 TQ_ROT_WHT     R = H, the Sylvester Walsh-Hadamard matrix;
 *                 TQ_ROT_DOUBLE  R = H D3 H / sqrt(d) with the sign flip
 *                                D3 = sign_mask3: S1 -> WHT -> S2 -> WHT per
 *                                head ([P1] v1.5.3 "핵심 변경" item 1, head_dim
 *                                64 only).  R R = d I as for H.
 *   norm_blocks 1: one norm per vector, ||x||.  2: one norm per half of the
 *               rotated vector y = R D x ([P1] v1.5.2 "핵심 변경" item 5: after
 *               the 512-point transform each 256-half has its own norm):
 *               nu_h = ||y_h|| / sqrt(d) (so nu_0^2 + nu_1^2 = ||x||^2) and
 *               z_h = y_h / (nu_h sqrt(2)).  d = 256 or 512, no residual.
 *   sign_mask3  D3 of TQ_ROT_DOUBLE (filled for every codec with d <= 256):
 *               bit i set when bit 63 of SplitMix64 output 513 + i is set.
 *   sign_mask_hi  D for dims 256..511 of a d = 512 codec (bit i of the array
 *               = dim 256 + i).
 */
enum { TQ_RES_NONE = 0, TQ_RES_QJL = 1, TQ_RES_SRHT = 2, TQ_RES_SIGN = 3 };
enum { TQ_ROT_WHT = 0, TQ_ROT_DOUBLE = 1 };
typedef struct {
    int32_t d;
    int32_t bits;
    int32_t qjl_m;
    int32_t residual;
    uint64_t seed;
    uint32_t sign_mask[8];
    float centroid[16];
    float threshold[15];
    uint32_t sign_mask2[8];
    int32_t rotation;
    int32_t norm_blocks;
    uint32_t sign_mask3[8];
    uint32_t sign_mask_hi[8];
} tq_codec;

/*
 * tq_codebook -- fill a codec (host only, deterministic, no device access).
 *
 * The scalar stage is the Lloyd-Max quantiser ([P1] page header "Walsh-Hadamard
 * Transform + Lloyd-Max 양자화"; [P3] "GPU 세대가 바뀌면": each coordinate maps to
 * one of 2^bits centroids) of the rotated unit coordinate z = H(Dx)/||x||, which
 * has unit variance, so the codebook is that of N(0,1).  It is solved in
 * double precision by the Lloyd fixed-point iteration (centroid = conditional
 * mean of its cell, threshold = midpoint) on the positive half, mirrored, then
 * rounded to float32.  Signs: D_ii = -1 when bit 63 of the (i+1)-th SplitMix64
 * output from state `seed` is set; D2_ii likewise from output 257 + i.
 * The residual kind is TQ_RES_QJL when qjl_m > 0, else TQ_RES_NONE.
 *
 * Errors: TQ_EINVAL if out is NULL; TQ_EUNSUPPORTED for d not in {32,64,128,256},
 * bits not in 1..4, qjl_m not a multiple of 32 in 0..256.
 */
int tq_codebook(int bits, int d, uint64_t seed, int qjl_m, tq_codec *out);

/*
 * tq_codebook_ex -- tq_codebook with an explicit residual kind (TQ_RES_*).
 * TQ_RES_SRHT and TQ_RES_SIGN use m = d bits (qjl_m must be 0 or d);
 * TQ_RES_QJL needs qjl_m > 0; TQ_RES_NONE needs qjl_m = 0.  Errors as
 * tq_codebook, plus TQ_EUNSUPPORTED for an unknown kind or a mismatched qjl_m.
 */
int tq_codebook_ex(int bits, int d, uint64_t seed, int residual, int qjl_m, tq_codec *out);

/*
 * tq_codebook_opts -- tq_codebook_ex with the rotation (TQ_ROT_*) and the
 * number of norm blocks (1 or 2) explicit; tq_codebook and tq_codebook_ex use
 * TQ_ROT_WHT and one norm.  Errors as tq_codebook_ex, plus TQ_EUNSUPPORTED for
 * TQ_ROT_DOUBLE at d != 64 ([P1] v1.5.3 uses it at head_dim 64 only), for
 * norm_blocks not 1 or 2, and for two norm blocks at d < 256 or with a
 * residual kind (the pages keep one norm for the residual codecs, [P1]
 * v1.5.2 item 5).
 */
int tq_codebook_opts(int bits, int d, uint64_t seed, int residual, int qjl_m, int rotation, int norm_blocks,
                     tq_codec *out);

/*
 * tq_encode -- quantise n vectors ([P1] v1.7.0 "핵심 설계 결정" item 4: sign flip +
 * butterfly WHT inside the encoder; [P2] "핵심 발견 3": bit-packed indices; [P1]
 * "약간의 비하인드": a 3-bit d=128 block is 48 B of codes + a 2 B norm).
 *
 * For each row x (d values of x_dtype, row i at x + i*x_row_stride elements):
 *   n = ||x||_2;  z = H(D x)/n (z = 0 when n = 0);  idx_i = #{j : z_i > t_j};
 *   codes = packed idx;  norms = half(n).
 * With codec->qjl_m = m > 0 (the paper's TurboQuant_prod residual correction,
 * [P1] "QJL 보정 효과", K caches only), r = (z - c[idx]) / sqrt(d) and
 *   TQ_RES_QJL:  gamma = half(||r||);  bit j = [(S r)_j >= 0];
 *   TQ_RES_SRHT: gamma = half(||r||);  bit j = [(H D2 r)_j >= 0];
 *   TQ_RES_SIGN: gamma = half(sum_i |r_i| / d);  bit i = [r_i >= 0].
 *
 *   c              codec (host pointer).
 *   x              [n][x_row_stride] elements; 16-byte aligned; x_row_stride*elem
 *                  must be a multiple of 16 bytes and x_row_stride >= d.
 *   codes          row i at codes + i*code_row_stride; code_row_stride >= d*bits/8,
 *                  multiple of 4; codes 4-byte aligned.
 *   norms_f16      [n] halves.
 *   qjl_S          [m][d] float32 row-major, 16-byte aligned (N(0,1) draws made by
 *                  the caller) for TQ_RES_QJL; NULL (unused) for the other kinds.
 *   qjl_bits       [n][m/8] bytes, 4-byte aligned; NULL when m = 0.
 *   qjl_gamma_f16  [n] halves; NULL when m = 0.
 * n = 0 is valid and launches nothing.  Vectors whose squared norm underflows
 * float32 are encoded as the zero vector.
 */
int tq_encode(const tq_codec *c, const void *x, int x_dtype, int64_t n, int64_t x_row_stride,
              uint8_t *codes, int64_t code_row_stride, uint16_t *norms_f16,
              const float *qjl_S, uint8_t *qjl_bits, uint16_t *qjl_gamma_f16, void *stream);

/*
 * tq_encode_kv -- tq_encode of a layer's keys and values in one call (one
 * launch when the K codec has no QJL; the per-call cost dominates at the sizes
 * of a prefill chunk).  Both rows sets have n rows of the same d, dtype and
 * x_row_stride; every K argument means what it means for tq_encode with kc,
 * every V argument what it means with vc.  vc must not use QJL (QJL is K-only,
 * [P1] "QJL 보정 효과"): TQ_EUNSUPPORTED, as are codecs of different d.
 */
int tq_encode_kv(const tq_codec *kc, const tq_codec *vc, const void *k, const void *v, int x_dtype,
                 int64_t n, int64_t x_row_stride,
                 uint8_t *k_codes, int64_t k_code_row_stride, uint16_t *k_norms_f16,
                 uint8_t *v_codes, int64_t v_code_row_stride, uint16_t *v_norms_f16,
                 const float *qjl_S, uint8_t *k_qjl_bits, uint16_t *k_qjl_gamma_f16, void *stream);

/*
 * tq_prefill -- chunked prefill: encode one sequence's chunk of `tokens` new
 * keys and values per head into its packed cache at token slots
 * [t0, t0 + tokens), all heads in one call (one launch unless kc uses QJL).
 * [P3] ("실험 설계") describes the prompt's K/V entering the compressed cache
 * before decoding; the chunk size is the caller's.  Same arithmetic as tq_encode.
 *
 *   k, v      [n_heads][tokens][d] elements of x_dtype, contiguous, 16-byte aligned.
 *   k_codes, v_codes    one sequence's cache planes [n_heads][ctx_cap][d*bits/8]
 *             (for sequence b of a batched cache, pass the plane pointers offset
 *             by b * n_heads * ctx_cap rows), 4-byte aligned; k_norms_f16,
 *             v_norms_f16 [n_heads][ctx_cap].
 *   qjl_S, k_qjl_bits [n_heads][ctx_cap][m/8], k_qjl_gamma_f16 [n_heads][ctx_cap]:
 *             as in tq_encode for kc, NULL when kc has no QJL.
 * Only the slots [t0, t0 + tokens) of every head are written; tokens = 0 is
 * valid and launches nothing.  Errors: TQ_EINVAL for NULL or misaligned
 * pointers, a bad x_dtype, n_heads or ctx_cap <= 0, t0 < 0, tokens < 0 or
 * t0 + tokens > ctx_cap; TQ_EUNSUPPORTED for an unsupported codec, codecs of
 * different d, or QJL on vc.
 */
int tq_prefill(const tq_codec *kc, const tq_codec *vc, const void *k, const void *v, int x_dtype,
               int n_heads, int64_t tokens, int64_t t0, int64_t ctx_cap,
               uint8_t *k_codes, uint16_t *k_norms_f16, uint8_t *v_codes, uint16_t *v_norms_f16,
               const float *qjl_S, uint8_t *k_qjl_bits, uint16_t *k_qjl_gamma_f16, void *stream);

/*
 * tq_append -- the decode-step append: encode the new key and value of every
 * (sequence, head) into the packed cache at that sequence's position.  [P3]
 * ("결과 — 피크 VRAM") describes each decode step adding the new K/V to the
 * cache before attention; with a residual window ([P3] "실험 설계") the token
 * leaving the window is the one appended.  Same arithmetic as tq_encode; one
 * launch for K and V unless kc uses QJL.
 *
 *   k, v      [batch][n_heads][d] elements of x_dtype, contiguous, 16-byte aligned.
 *   pos       [batch] int32 on the device: token slot written for sequence b
 *             (read by the kernel, not updated); a slot outside [0, ctx_cap)
 *             writes nothing for that sequence.
 *   k_codes, v_codes    cache planes [batch][n_heads][ctx_cap][d*bits/8] (the
 *             layout the attention calls read), 4-byte aligned; k_norms_f16,
 *             v_norms_f16 [batch][n_heads][ctx_cap].
 *   qjl_S, k_qjl_bits [batch][n_heads][ctx_cap][m/8], k_qjl_gamma_f16
 *             [batch][n_heads][ctx_cap]: as in tq_encode for kc, NULL when kc
 *             has no QJL.
 * Only the addressed slots are written.  Errors: TQ_EINVAL for NULL or
 * misaligned pointers, a bad x_dtype, or batch, n_heads or ctx_cap <= 0;
 * TQ_EUNSUPPORTED for an unsupported codec, codecs of different d, or QJL on vc.
 */
int tq_append(const tq_codec *kc, const tq_codec *vc, const void *k, const void *v, int x_dtype,
              int batch, int n_heads, const int32_t *pos, int64_t ctx_cap,
              uint8_t *k_codes, uint16_t *k_norms_f16, uint8_t *v_codes, uint16_t *v_norms_f16,
              const float *qjl_S, uint8_t *k_qjl_bits, uint16_t *k_qjl_gamma_f16, void *stream);

/*
 * tq_decode -- reconstruct x_hat = half_norm * D H(c[idx]) / d for n rows: the
 * dequantise step of decompress-then-attend ([P3] "결과 — 피크 VRAM": the
 * reference reconstructs the full K/V each step) with the inverse transform
 * applied per vector ([P1] v1.5.1 "핵심 기술" item 2: V WHT on encode, IWHT on
 * read).  Used to check reconstructions; decode attention never calls it.
 *   codes: row i at codes + i*code_row_stride (code_row_stride >= d*bits/8,
 *          any byte stride, so rows of a cache with padding can be read in
 *          place); norms_f16 [n]; x_hat [n][d] float32 (16-byte aligned).
 * n = 0 is valid and launches nothing.  Errors: TQ_EINVAL for NULL or
 * misaligned pointers, n < 0 or a short row stride; TQ_EUNSUPPORTED for an
 * unsupported codec.
 */
int tq_decode(const tq_codec *c, const uint8_t *codes, int64_t code_row_stride,
              const uint16_t *norms_f16, int64_t n, float *x_hat, void *stream);

/*
 * tq_attn_decode -- one decode step of grouped-query attention read straight
 * from the packed cache (compressed-domain attention, [P3] "결과 — 피크 VRAM"
 * contrasts it with decompress-then-attend).
 *
 * For batch b and query head h (kv head kh = h / (n_q_heads/n_kv_heads)):
 *   q_rot = H(D_K q) (the query is rotated once, [P1] v1.7.0 item 4: the same WHT
 *           on the Q side, so the rotation cancels by Parseval);
 *   s_t   = scale * n_t/d * <q_rot, c_K[idx_t]>
 *           (+ with QJL: scale * n_t * gamma_t * sqrt(pi/2)/m * <S q_rot/sqrt(d), 2 bit_t - 1>,
 *            [P1] "Attention Sharpening": d_qjl * sum(Q_wht2[i] * sign[i]); with
 *            TQ_RES_SRHT S = H D2; with TQ_RES_SIGN S = I and the constant
 *            sqrt(pi/2)/m is replaced by 1);
 *   p     = softmax(s) over t < ctx_len[b] (exact, float32 accumulation,
 *           [P1] v1.5.2 "핵심 변경" item 1: float, not half2);
 *   o     = D_V H( sum_t p_t nV_t c_V[vidx_t] ) / d  (V accumulated in the rotated
 *           domain, one inverse WHT per output, [P1] v1.5.1 item 2).
 *
 *   kc, vc          K and V codecs (host); independent bit widths ([P2] "핵심 발견 2":
 *                   asymmetric K/V).  kc->d == vc->d in {128, 256}; vc->qjl_m must
 *                   be 0 (QJL is K-only, [P1] "지원 K/V 조합").
 *   q               [batch][n_q_heads][d] of q_dtype, 16-byte aligned, contiguous.
 *   ctx_len         [batch] int32 on the device; values are clamped to [0, ctx_cap].
 *   k_codes         [batch][n_kv_heads][ctx_cap][d*kbits/8]   contiguous, 16-B aligned
 *   k_norms         [batch][n_kv_heads][ctx_cap] halves
 *   k_qjl, k_gamma  [batch][n_kv_heads][ctx_cap][m/8], [..][ctx_cap] halves; NULL if m = 0
 *   qjl_S           [m][d] float32 for TQ_RES_QJL keys; NULL otherwise
 *   v_codes, v_norms as k_codes / k_norms with vbits
 *   out             [batch][n_q_heads][d] float32; a sequence with ctx_len 0 gives 0.
 *   workspace       device scratch of at least tq_attn_workspace_bytes(...) bytes,
 *                   16-byte aligned (QJL query projections and split-K partials).
 * Supported: n_q_heads % n_kv_heads == 0, group size g = n_q_heads/n_kv_heads
 * with g <= 8 or g a multiple of a divisor in 1..8 (heads are processed in
 * chunks of at most 8).  ctx_cap >= 1.
 * The context is cut into splits whose count is planned per call from the
 * device; a positive integer in the environment variable TQ_ATTN_SPLITS
 * replaces that count (clamped to the capacity's 64-token tiles), which tests
 * use to show the result does not depend on it.  Query the workspace size
 * under the same setting.
 */
int tq_attn_decode(const tq_codec *kc, const tq_codec *vc,
                   const void *q, int q_dtype, int batch, int n_q_heads, int n_kv_heads,
                   const int32_t *ctx_len, int64_t ctx_cap,
                   const uint8_t *k_codes, const uint16_t *k_norms,
                   const uint8_t *k_qjl, const uint16_t *k_gamma, const float *qjl_S,
                   const uint8_t *v_codes, const uint16_t *v_norms,
                   float scale, float *out, void *workspace, size_t workspace_bytes,
                   void *stream);

/*
 * tq_attn_decode_noalloc -- tq_attn_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same computation and arguments without the
 * workspace, which comes from a static device array of the library instead.
 *
 * The array holds TQ_NOALLOC_SCRATCH_BYTES (16 MiB) per device, for as long as
 * the process runs; its device address is looked up once per device on the
 * first call made there.  A call needing more scratch than that
 * (tq_attn_workspace_bytes(...) > TQ_NOALLOC_SCRATCH_BYTES) returns
 * TQ_ESCRATCH and launches nothing.  Nothing in the scratch has to start at
 * zero: every value the kernels read is written earlier in the same call.
 * Every call on one device shares its array: calls that overlap on one device
 * (concurrent streams, or threads without ordering) race and give undefined
 * results; order them on one stream.  The call allocates and frees nothing.
 * Errors: those of tq_attn_decode, TQ_ESCRATCH, and TQ_EDEVICE when the
 * scratch address cannot be looked up.
 */
#define TQ_NOALLOC_SCRATCH_BYTES (16u << 20)
int tq_attn_decode_noalloc(const tq_codec *kc, const tq_codec *vc,
                           const void *q, int q_dtype, int batch, int n_q_heads, int n_kv_heads,
                           const int32_t *ctx_len, int64_t ctx_cap,
                           const uint8_t *k_codes, const uint16_t *k_norms,
                           const uint8_t *k_qjl, const uint16_t *k_gamma, const float *qjl_S,
                           const uint8_t *v_codes, const uint16_t *v_norms,
                           float scale, float *out, void *stream);

/*
 * tq_attn_decode_mq -- multi-query decode over the packed cache: n_cols query
 * tokens per sequence in one call, each attending causally.  [P1] runs several
 * query columns through its attention kernel at once (v1.1.0 "버그 수정": the
 * ncols = 2 prompt-evaluation path; v1.4.2 "MMA Tensor Core 가속"), the shape
 * of chunked-prefill attention and of speculative verification.
 *
 * The n_cols columns are the last n_cols tokens of each sequence, and their
 * keys and values are already in the cache (append or prefill first): column c
 * of sequence b sits at position ctx_len[b] - n_cols + c and attends over the
 * first max(0, ctx_len[b] - (n_cols - 1 - c)) tokens, exactly as
 * tq_attn_decode would with that context length.  A column that sees no token
 * gives a zero row.
 *
 *   q    [batch][n_cols][n_q_heads][d] of q_dtype, contiguous, 16-byte aligned.
 *   out  [batch][n_cols][n_q_heads][d] float32.
 *   workspace  >= tq_workspace_bytes(TQ_OP_ATTN_DECODE_MQ, ..., n_q = n_cols, ...).
 * Every other argument and error is that of tq_attn_decode; 1 <= n_cols <=
 * TQ_MAX_QUERY_COLS.  The query rows of one kv head (its g heads in each
 * column) share the scan of its cache in blocks of up to 8 rows, so with
 * g * n_cols <= 8 the cache is read once for all columns.  n_cols = 1 is
 * tq_attn_decode.
 */
#define TQ_MAX_QUERY_COLS 64
int tq_attn_decode_mq(const tq_codec *kc, const tq_codec *vc,
                      const void *q, int q_dtype, int batch, int n_cols, int n_q_heads, int n_kv_heads,
                      const int32_t *ctx_len, int64_t ctx_cap,
                      const uint8_t *k_codes, const uint16_t *k_norms,
                      const uint8_t *k_qjl, const uint16_t *k_gamma, const float *qjl_S,
                      const uint8_t *v_codes, const uint16_t *v_norms,
                      float scale, float *out, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * Optional softmax-side switches of decode attention, all off in a zeroed
 * struct (tq_attn_decode_ex with opts == NULL is tq_attn_decode_mq).
 *
 *   score_mode  TQ_SCORE_PLAIN: scores as in tq_attn_decode.
 *               TQ_SCORE_SHARPEN: every score of a query row that attends over
 *               N tokens is multiplied by alpha(N) = 1 + c sqrt(ln N),
 *               c = 1 / (2 sqnr sqrt(ln N0)) -- the dynamic attention
 *               sharpening of [P1] v1.5.2 ("핵심 변경" item 3, "Attention
 *               Sharpening — 이론 & 동적 α 공식"), which offsets the flattening
 *               of the softmax by K quantisation noise.
 *               TQ_SCORE_SOFTEN: alpha(N) = sqnr / (sqnr + sqrt(ln N / ln N0)),
 *               the MMSE softening of [P1] v1.5.2 item 11.
 *               alpha = 1 for N <= 1.  N counts the row's own tokens (its
 *               column's causal limit in multi-query calls).
 *   sqnr        SQNR_eff > 0 of the key cache (the pages print no value per
 *               type; the caller picks it); ignored when plain.
 *   ref_tokens  N0 >= 2; 0 means 2048 (the pages' reference context).
 *   sparse_v    0 = off; tau in (0, 1]: a token whose softmax weight relative to
 *               the largest weight is below tau adds nothing to the output, the
 *               denominator still counting it -- the sparse V dequantisation of
 *               [P3] "왜 이걸 보게 됐나" (weights below 1e-6 skip their V).  The
 *               kernels compare against their running maximum, which never
 *               exceeds the true one, so they drop a subset of those tokens; a
 *               32-token step whose weights are all dropped skips its V work.
 */
enum { TQ_SCORE_PLAIN = 0, TQ_SCORE_SHARPEN = 1, TQ_SCORE_SOFTEN = 2 };
typedef struct {
    int32_t score_mode;
    float sqnr;
    int32_t ref_tokens;
    float sparse_v;
} tq_attn_opts;

/*
 * tq_attn_decode_ex -- tq_attn_decode_mq with the switches above (opts may be
 * NULL).  Errors: those of tq_attn_decode_mq, and TQ_EINVAL for an unknown
 * score_mode, sqnr not finite and positive when used, ref_tokens of 1 or
 * negative, or sparse_v outside [0, 1].  Workspace: as tq_attn_decode_mq.
 */
int tq_attn_decode_ex(const tq_codec *kc, const tq_codec *vc,
                      const void *q, int q_dtype, int batch, int n_cols, int n_q_heads, int n_kv_heads,
                      const int32_t *ctx_len, int64_t ctx_cap,
                      const uint8_t *k_codes, const uint16_t *k_norms,
                      const uint8_t *k_qjl, const uint16_t *k_gamma, const float *qjl_S,
                      const uint8_t *v_codes, const uint16_t *v_norms,
                      float scale, const tq_attn_opts *opts, float *out,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * The three launches of tq_attn_decode as separate calls (same arguments, same
 * checks, same workspace, which carries the state between them), for callers
 * that time or schedule the stages themselves:
 *   tq_attn_prepare  with QJL keys: the projection S q_rot/sqrt(d) of every
 *                    rotated query into the workspace (the Q_wht2 half of the
 *                    fused Q_wht1/Q_wht2 pass of [P1] v1.4.2 item 5); without
 *                    QJL it launches nothing;
 *   tq_attn_scan     rotate the queries (q_rot = H(D_K q), the Q-side WHT of
 *                    [P1] v1.7.0 item 4), then stream the packed cache: scores,
 *                    online softmax and rotated V sums per context split, into
 *                    the workspace;
 *   tq_attn_combine  merge the splits and apply one inverse transform per head
 *                    into `out` ([P1] v1.5.1 item 2).
 * tq_attn_decode == prepare, scan, combine on one stream.
 */
int tq_attn_prepare(const tq_codec *kc, const tq_codec *vc,
                    const void *q, int q_dtype, int batch, int n_q_heads, int n_kv_heads,
                    const int32_t *ctx_len, int64_t ctx_cap,
                    const uint8_t *k_codes, const uint16_t *k_norms,
                    const uint8_t *k_qjl, const uint16_t *k_gamma, const float *qjl_S,
                    const uint8_t *v_codes, const uint16_t *v_norms,
                    float scale, float *out, void *workspace, size_t workspace_bytes,
                    void *stream);
int tq_attn_scan(const tq_codec *kc, const tq_codec *vc,
                 const void *q, int q_dtype, int batch, int n_q_heads, int n_kv_heads,
                 const int32_t *ctx_len, int64_t ctx_cap,
                 const uint8_t *k_codes, const uint16_t *k_norms,
                 const uint8_t *k_qjl, const uint16_t *k_gamma, const float *qjl_S,
                 const uint8_t *v_codes, const uint16_t *v_norms,
                 float scale, float *out, void *workspace, size_t workspace_bytes,
                 void *stream);
int tq_attn_combine(const tq_codec *kc, const tq_codec *vc,
                    const void *q, int q_dtype, int batch, int n_q_heads, int n_kv_heads,
                    const int32_t *ctx_len, int64_t ctx_cap,
                    const uint8_t *k_codes, const uint16_t *k_norms,
                    const uint8_t *k_qjl, const uint16_t *k_gamma, const float *qjl_S,
                    const uint8_t *v_codes, const uint16_t *v_norms,
                    float scale, float *out, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * tq_attn_decode_rw -- decode attention over the packed cache plus a residual
 * window of exact recent tokens.  [P3] ("실험 설계", "결과 — 피크 VRAM")
 * describes the V3 cache: the most recent rw tokens stay uncompressed and are
 * appended to the decompressed ones before attention.  Here the window tokens
 * join the same softmax as the ctx_len[b] packed tokens, with score
 * scale <q, k_win_t> (exact keys, no QJL term) and value v_win_t:
 *   o = sum over packed and window tokens of softmax(s)_t * value_t.
 *
 *   k_win, v_win  [batch][n_kv_heads][win_cap][d] in win_dtype (TQ_F32, TQ_F16
 *                 or TQ_BF16), 16-byte aligned; caller-owned, read only.
 *   win_len       [batch] int32 on the device: tokens used in each sequence's
 *                 window, clamped to [0, win_cap].
 *   win_cap       window capacity; 0 means no window (then k_win, v_win and
 *                 win_len may be NULL and the call equals tq_attn_decode).
 * Every other argument, the workspace (tq_attn_workspace_bytes covers both
 * calls) and the error behaviour are those of tq_attn_decode; additionally
 * win_cap < 0, a bad win_dtype, or NULL/misaligned window pointers with
 * win_cap > 0 give TQ_EINVAL.  A sequence with no packed and no window token
 * gives a zero output row.
 */
int tq_attn_decode_rw(const tq_codec *kc, const tq_codec *vc,
                      const void *q, int q_dtype, int batch, int n_q_heads, int n_kv_heads,
                      const int32_t *ctx_len, int64_t ctx_cap,
                      const uint8_t *k_codes, const uint16_t *k_norms,
                      const uint8_t *k_qjl, const uint16_t *k_gamma, const float *qjl_S,
                      const uint8_t *v_codes, const uint16_t *v_norms,
                      const void *k_win, const void *v_win, int win_dtype,
                      const int32_t *win_len, int win_cap,
                      float scale, float *out, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * Workspace sizes.  The workspace holds float32 staging of the rotated-domain
 * partial sums (max, sum, acc[d]) of every (query head, context split) before
 * the one inverse transform per head (the float staging of [P1] v1.5.2 "핵심
 * 변경" item 2), and with QJL keys the projected queries (Q_wht2 of [P1] v1.4.2
 * item 5); for search, the rotated queries and per-block candidate lists.  The
 * caller allocates it ([P3] "결과 — 피크 VRAM" counts the reference's peak
 * memory; here nothing is allocated inside a call).
 *
 * tq_workspace_bytes(op, ...) -- bytes needed by operation `op` (0 on bad
 * arguments or an unknown op):
 *   TQ_OP_ATTN_DECODE, TQ_OP_ATTN_DECODE_RW: kc, vc, batch, n_q_heads,
 *       n_kv_heads, ctx_cap as for tq_attn_decode (n_q, n_db, k unused);
 *   TQ_OP_IP_SEARCH: kc is the search codec (vc may be NULL), n_q, n_db, k as
 *       for tq_ip_search (batch, heads and ctx_cap unused);
 *   TQ_OP_ATTN_DECODE_MQ: as TQ_OP_ATTN_DECODE with n_q = n_cols, the query
 *       columns per sequence of tq_attn_decode_mq.
 * The codecs are arguments because the sizes depend on d, the bit widths
 * (through the split plan) and the QJL width m.  The size depends on the
 * current device (its compute-unit count sets the split count).
 * tq_attn_workspace_bytes and tq_search_workspace_bytes are the same sizes for
 * one operation each.
 */
enum { TQ_OP_ATTN_DECODE = 1, TQ_OP_ATTN_DECODE_RW = 2, TQ_OP_IP_SEARCH = 3, TQ_OP_ATTN_DECODE_MQ = 4 };
size_t tq_workspace_bytes(int op, const tq_codec *kc, const tq_codec *vc, int batch, int n_q_heads,
                          int n_kv_heads, int64_t ctx_cap, int n_q, int64_t n_db, int k);

size_t tq_attn_workspace_bytes(const tq_codec *kc, const tq_codec *vc, int batch,
                               int n_q_heads, int n_kv_heads, int64_t ctx_cap);

/*
 * tq_ip_search -- inner-product search over QJL-encoded database vectors, the
 * non-softmax use case for which the QJL estimator is unbiased and helps
 * ([P2] "핵심 발견 1 — QJL 레이어를 제거하라": vector search has no softmax).
 *
 *   est(q, t) = n_t ( <H(Dq), c[idx_t]>/d
 *                     + gamma_t sqrt(pi/2)/m <S H(Dq)/sqrt(d), 2 bit_t - 1> )
 * (S = H D2 for TQ_RES_SRHT; S = I and constant 1 for TQ_RES_SIGN), then the
 * k largest estimates per query, ordered by (estimate desc, id asc).
 *
 *   c            codec (host) with qjl_m = m (0 = MSE-only estimate); qjl_S
 *                [m][d] for TQ_RES_QJL, NULL for the other kinds.
 *   q            [n_q][d] float32, 16-byte aligned.
 *   codes, norms [n_db][d*bits/8] (16-byte aligned), [n_db]; qjl_bits [n_db][m/8]
 *                (4-byte aligned); qjl_gamma [n_db].
 *   out_scores   [n_q][k] float32;  out_ids [n_q][k] int64.  If n_db < k the tail
 *                is filled with -inf and id -1.
 *   workspace    >= tq_search_workspace_bytes(...) bytes, 16-byte aligned.
 * Supported: d in {128, 256}, 1 <= k <= 64, n_db < 2^31.
 */
int tq_ip_search(const tq_codec *c, const float *q, int n_q,
                 const uint8_t *codes, const uint16_t *norms,
                 const uint8_t *qjl_bits, const uint16_t *qjl_gamma, const float *qjl_S,
                 int64_t n_db, int k, float *out_scores, int64_t *out_ids,
                 void *workspace, size_t workspace_bytes, void *stream);

size_t tq_search_workspace_bytes(const tq_codec *c, int n_q, int64_t n_db, int k);

/*
 * Stored bytes per vector: d*bits/8 codes + 2 B norm (+ m/8 + 2 B with QJL).
 * [P1] "약간의 비하인드": a 3-bit head_dim-128 block is 50 B (48 B codes + a
 * 2 B norm); [P3] "결과 — 피크 VRAM" gives the theoretical compression the
 * reference's memory_bytes() reports (K4/V2 5.12x against fp16).  Returns 0
 * for d <= 0, bits outside 1..4 or qjl_m < 0.
 */
size_t tq_packed_bytes(int d, int bits, int qjl_m);

/*
 * tq_stream_read -- read `bytes` of device memory at `src` with 16-byte loads,
 * keeping only a running XOR (nothing is written except, with negligible
 * probability, one word at *sink).  A measurement helper: decode is bound by
 * memory bandwidth ([P1] v1.8.0 "성능 특성": decode reads its operands from
 * memory every token), and the decode scan is itself a read-only stream, so
 * this kernel's rate is the practical read ceiling the scan is compared with.
 *   src   16-byte aligned; bytes a multiple of 16 (0 launches nothing).
 *   sink  one uint32 on the device, 4-byte aligned.
 * Errors: TQ_EINVAL for NULL or misaligned pointers or a bad size.
 */
int tq_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

/*
 * Static description of an error code (never NULL).  [P1] v1.2.0 ("입력 검증")
 * handles invalid K/V type combinations by silently falling back; this
 * library reports them as TQ_EUNSUPPORTED and leaves the policy to the caller.
 */
const char *tq_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
