/*
 * csa.h -- C ABI of libcsa.so: compressed sparse attention (CSA) and heavily
 * compressed attention (HCA) for one layer on one MI355X (gfx950) GPU.
 *
 * The method (DeepSeek-V4 hybrid attention) as the pages describe it:
 *   - jiwasawa.github.io "deepseek-v4" post, section on the hybrid attention
 *     mechanism that breaks the context wall: CSA compresses the KV of m
 *     adjacent tokens into one entry, a Lightning Indexer scores the
 *     compressed entries per query token, a top-k selector keeps k of them,
 *     and shared-KV multi-query attention runs over the kept entries; HCA
 *     compresses with m' >> m and attends densely; a sliding-window branch
 *     over the newest tokens runs alongside.
 *   - hazakura.dev "DeepSeek V4とOpenCode", section "衝撃1：CSA + HCA":
 *     m = 4, m' = 128, FP4 indexer, 128-token window.
 *   - studioglobal.ai "DeepSeek V4 Flash" answer, section on the CSA/HCA
 *     breakthrough: pooling is softmax-gated, k = 512 blocks per query,
 *     the window branch is always present; section on FP4/FP8 mixed
 *     precision: MXFP4 holds two values per byte.
 *   - ai-papers.net "deepseek-v4-1m-context-window..." section on how the
 *     hybrid attention works: the indexer runs at FP4 over the already
 *     shortened sequence.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is device memory owned by the caller; the
 *     library never allocates, frees, synchronises, or keeps a pointer after
 *     the call returns.  Work is enqueued on `stream` (0 = null stream).
 *   - Tensors are row-major with the innermost index last.  The entry points
 *     of the path's core steps (hca_compress, csa_quantize_mxfp4,
 *     csa_index_topk, csa_attend, hca_attend) take their floating inputs
 *     and outputs as strided views (csa_in / csa_out): a tensor of B
 *     sequences of rows, each row contiguous, with element strides between
 *     sequences and between rows, so a slice of a larger buffer (a window
 *     of raw rows, a range of query rows) is passed without a copy.  Every
 *     other tensor is dense.
 *   - Floating tensors are fp32 or bf16 as given by `dt` (one dtype per call);
 *     arithmetic is fp32 inside the kernels.
 *   - Positions: a sequence's tokens are at positions 0,1,2,...  Query row i
 *     of every sequence is at position q_pos0 + i.  Raw row r of the raw
 *     K/V tensors is at position raw_pos0 + r.  Compressed entry j covers
 *     tokens m*j .. m*j+m-1.
 *   - Window and candidates of a query at position t: the window is the raw
 *     tokens w0..t with w0 = max(0, t-W+1); compressed entry j is a candidate
 *     iff it is complete and visible (m*j+m-1 <= t) and starts before the
 *     window (m*j < w0), so n_cand(t) = min(ceil(w0/m), floor((t+1)/m)).
 *     A token is never reached both raw and through an entry lying wholly
 *     inside the window.
 *   - Errors: arguments are checked on the host before anything is
 *     enqueued.  A failed check returns CSA_EINVAL (bad value, null or
 *     misaligned pointer, too small workspace) or CSA_EUNSUPPORTED (a valid
 *     shape the library has no kernel for), writes nothing, and sets a
 *     thread-local message read by csa_last_error().  A launch error
 *     returns CSA_EDEVICE.  Base pointers must be 16-byte aligned.
 *   - Views: strides are >= 0 and in elements; consecutive rows do not
 *     overlap (row_stride >= the row length); base and strides are
 *     16-byte multiples (a per-token gate of one logit per row excepted);
 *     an output's sequences do not overlap.  A failed check is CSA_EINVAL.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 8

typedef enum csa_dtype { CSA_F32 = 0, CSA_BF16 = 1 } csa_dtype;

typedef enum csa_status {
    CSA_OK = 0,
    CSA_EINVAL = 1,
    CSA_EUNSUPPORTED = 2,
    CSA_EDEVICE = 3
} csa_status;

/* Strided views: element (b, r, e) of a view of B sequences of rows, each
 * row of contiguous elements, is at p + b * seq_stride + r * row_stride + e
 * (elements of the tensor's dtype). */
typedef struct csa_in {
    const void *p;
    int64_t seq_stride, row_stride;
} csa_in;
typedef struct csa_out {
    void *p;
    int64_t seq_stride, row_stride;
} csa_out;

/* Version of this ABI (CSA_ABI_VERSION of the build). */
int csa_abi_version(void);

/* Message of the last failed call on this thread ("" if none). */
const char *csa_last_error(void);

/*
 * hca_compress -- softmax-gated pooling of m adjacent rows into one entry
 * (jiwasawa.github.io post, CSA token-level compression: m adjacent tokens'
 * KV become one entry, the sequence shrinks to 1/m; studioglobal.ai answer,
 * CSA bullet: the pooling is softmax-gated).  Serves both CSA (m = 4) and
 * HCA (m' = 128).
 *
 *   out[b][j][c] = sum_{i<m} softmax_i( z[b][m*j+i][g(c)] ) * x[b][m*j+i][c]
 *
 * for j < T/m (a trailing partial block is not emitted), with the softmax
 * over the block's m logits and g(c) = c if gate_channels == C, 0 if
 * gate_channels == 1 (one logit per token).
 *   x     view of B x T rows of C               dt
 *   gate  view of B x T rows of gate_channels   dt
 *   out   view of B x T/m rows of C             dt (rounded to nearest even
 *         for bf16)
 * Requires B >= 1, T >= 0, C % 8 == 0 and C <= 1024, m >= 1.
 */
csa_status hca_compress(csa_dtype dt, int64_t B, int64_t T, int64_t C, int64_t m, csa_in x,
                        csa_in gate, int64_t gate_channels, csa_out out, hipStream_t stream);

/*
 * hca_append -- one decode step of cache upkeep (jiwasawa.github.io post,
 * CSA token-level compression: every m adjacent tokens become one entry;
 * the sliding-window branch keeps the newest tokens uncompressed).  The
 * token at position t joins the raw window rows and the gate logits of its
 * block; when it completes a block (t + 1 a multiple of m), the block's m
 * rows are pooled into entry (t + 1)/m - 1 of ck, cv exactly as
 * hca_compress pools them (the same arithmetic, so the entries are
 * bit-identical to a pooling of the whole sequence).  For CSA, the new
 * entry's indexer key is encoded separately with csa_quantize_mxfp4.
 *   k_new, v_new   [B, C]                 dt   the token's K and V rows
 *   gk_new, gv_new [B, gate_channels]     dt   its gate logits for K and V
 *   rk, rv         [B, wcap, C]           dt   window buffer: row r holds
 *                  position *win_pos0 + r; on entry positions *win_pos0 ..
 *                  t - 1, on return *win_pos0 .. t (pass raw_pos0 =
 *                  *win_pos0 and raw_len = t - *win_pos0 + 1 to attention)
 *   *win_pos0      host, in/out: when the buffer is full (t - *win_pos0 ==
 *                  wcap), its newest W - 1 rows move to the front first and
 *                  *win_pos0 becomes t - W + 1
 *   gk_blk, gv_blk [B, m, gate_channels]  dt   gate logits of the block's
 *                  tokens so far (slot = position mod m); owned by the caller,
 *                  written only by this call
 *   ck, cv         [B, nc_cap, C]         dt   compressed caches
 * Passing the same buffers as K and V (k_new == v_new, rk == rv, ck == cv)
 * keeps one vector per token and entry.
 * Requires C % 8 == 0 (C <= 1024), 1 <= m <= W, wcap >= 2 W, the window
 * buffer holding the min(t, W - 1) positions before t (*win_pos0 <= t -
 * min(t, W - 1)), and nc_cap >= (t + 1)/m.  On an error nothing is written
 * and *win_pos0 is unchanged.
 */
csa_status hca_append(csa_dtype dt, int64_t B, int64_t C, int64_t m, int64_t W, int64_t t,
                      const void *k_new, const void *v_new, const void *gk_new,
                      const void *gv_new, int64_t gate_channels, void *rk, void *rv,
                      int64_t wcap, int64_t *win_pos0, void *gk_blk, void *gv_blk, void *ck,
                      void *cv, int64_t nc_cap, hipStream_t stream);

/*
 * csa_quantize_mxfp4 -- MXFP4 encoding of rows (studioglobal.ai answer,
 * FP4/FP8 mixed precision: MXFP4, two values per byte; the indexer runs at
 * FP4 per every page).  Per run of 32 values: scale exponent
 * e = floor(log2 max|x|) - 2 clamped to [-127, 127] (-127 for an all-zero
 * run), stored as the byte e + 127; each value x * 2^-e is rounded to the
 * nearest of {0, 0.5, 1, 1.5, 2, 3, 4, 6} (ties to the even code, larger
 * magnitudes saturate to 6), code = magnitude index | 8 if x's sign bit is
 * set.  Element 2i of a row is the low nibble of byte i.
 *   x       view of rows rows of d (x.seq_stride is not used)   dt, finite
 *   codes   [rows, d/2]    uint8
 *   scales  [rows, d/32]   uint8 (E8M0)
 * Requires d % 32 == 0.
 */
csa_status csa_quantize_mxfp4(csa_dtype dt, int64_t rows, int64_t d, csa_in x,
                              uint8_t *codes, uint8_t *scales, hipStream_t stream);

/*
 * csa_index_topk -- Lightning Indexer score and top-k selection per query
 * token (jiwasawa.github.io post, CSA indexer bullet: every query token
 * scores the compressed entries with a lightweight indexer and a top-k
 * selector keeps k entries; studioglobal.ai answer: k = 512 at FP4).
 *
 * q_idx is encoded to MXFP4 inside the call (same rule as
 * csa_quantize_mxfp4), then for every candidate j of the query at t
 *   I(t, j) = sum_{h < HI} max(0, qhat[t][h] . khat[j])
 * is formed in fp32 (exact for inputs whose partial sums need at most 24
 * significant bits, e.g. N(0,1) data).  The kept entries are the first
 * min(k, n_cand(t)) candidates under the order (score descending, index
 * ascending); -0 counts as +0.
 *   q_idx      view of B x Tq rows of HI * dI ([HI][dI] per query)   dt
 *   k_codes    [B, Nc, dI/2]     uint8 (csa_quantize_mxfp4 of the indexer keys)
 *   k_scales   [B, Nc, dI/32]    uint8
 *   topk       [B, Tq, k]        int32 out: kept indices in ascending order,
 *                                then -1 in the remaining slots
 *   ws         workspace of at least csa_index_topk_workspace(...) bytes
 * Requires HI in {1, 2, 4}, dI in {32, 64}, 1 <= k <= 2048, W >= 0,
 * q_pos0 >= 0 and n_cand(q_pos0 + Tq - 1) <= Nc.
 */
csa_status csa_index_topk_workspace(int64_t B, int64_t Tq, int64_t HI, int64_t dI,
                                    int64_t Nc, int64_t m, int64_t W, int64_t k,
                                    int64_t q_pos0, size_t *bytes);
csa_status csa_index_topk(csa_dtype dt, int64_t B, int64_t Tq, int64_t HI, int64_t dI,
                          int64_t Nc, int64_t m, int64_t W, int64_t k, int64_t q_pos0,
                          csa_in q_idx, const uint8_t *k_codes, const uint8_t *k_scales,
                          int32_t *topk, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * csa_index_topk_noalloc -- csa_index_topk without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  The selection
 * state lives in a static device array of CSA_NOALLOC_SCRATCH_BYTES bytes
 * per GPU, held by the library until the process ends; its address is
 * looked up once per device at the first call there.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams,
 * other host threads) race and give undefined results.  Nothing in the array
 * needs to start at any value.  Same arguments, layouts and results as
 * csa_index_topk; the call allocates and frees nothing.
 * Errors: CSA_EUNSUPPORTED when the selection needs more scratch than the
 * array holds (csa_index_topk_workspace(...) > CSA_NOALLOC_SCRATCH_BYTES,
 * e.g. many query rows over more than 32,768 candidates; decode rows and
 * prefill rows over at most 32,768 candidates fit); otherwise as
 * csa_index_topk.
 */
#define CSA_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
csa_status csa_index_topk_noalloc(csa_dtype dt, int64_t B, int64_t Tq, int64_t HI, int64_t dI,
                                  int64_t Nc, int64_t m, int64_t W, int64_t k, int64_t q_pos0,
                                  csa_in q_idx, const uint8_t *k_codes,
                                  const uint8_t *k_scales, int32_t *topk, hipStream_t stream);

/*
 * csa_attend -- shared-KV multi-query attention over the kept compressed
 * entries joined with the raw sliding window (jiwasawa.github.io post, CSA
 * "Shared Key-Value MQA" bullet and the SWA branch; hazakura.dev note, CSA
 * bullets: 128-token window).  For every sequence b, query row i at
 * t = q_pos0 + i and head h, one softmax runs over the key set
 *   S = { entries named in the first min(k, n_cand(t)) slots of topk[b][i]
 *         that are candidates of t }  U  { raw tokens w0..t },
 *   o[b][i][h] = sum_{s in S} softmax_s( scale * q[b][i][h] . key_s ) val_s
 * with key/val = ck/cv rows for entries and rk/rv rows for raw tokens.
 * Slots holding -1 or a non-candidate index contribute nothing.
 * One vector per entry and raw token may serve as both key and value (the
 * "shared key-value" reading of the same post): pass the same buffer as ck
 * and cv and as rk and rv, and each row is then read once.
 *   q, o   views of B x Tq rows of H * D ([H][D] per query token)   dt
 *   ck, cv views of B x Nc rows of D                                dt
 *   rk, rv views of B x raw_len rows of D, covering positions w0..t of
 *          every query                                              dt
 *   topk   [B, Tq, k]      int32
 *   (a sequence's rows of ck, cv, rk or rv must lie within 2 GiB of its
 *   first row)
 *   ws     workspace of at least csa_attend_workspace(...) bytes
 * bf16 requires H % 32 == 0 (H <= 256) and D in {64, 128}; fp32 requires
 * D <= 256.
 */
csa_status csa_attend_workspace(csa_dtype dt, int64_t B, int64_t Tq, int64_t H, int64_t D,
                                int64_t k, int64_t W, size_t *bytes);
csa_status csa_attend(csa_dtype dt, int64_t B, int64_t Tq, int64_t H, int64_t D,
                      int64_t Nc, int64_t m, int64_t W, int64_t k, int64_t q_pos0,
                      float scale, csa_in q, csa_in ck, csa_in cv, const int32_t *topk,
                      csa_in rk, csa_in rv, int64_t raw_pos0, int64_t raw_len, csa_out o,
                      void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * hca_attend -- dense attention over every compressed candidate joined with
 * the raw window (jiwasawa.github.io post, HCA part: no sparse selection,
 * dense attention over the heavily compressed sequence; hazakura.dev note,
 * HCA bullets: m' = 128).  Same as csa_attend with S = { all candidates of
 * t } U { raw tokens w0..t }.  Argument meaning, layouts and requirements
 * as for csa_attend.
 */
csa_status hca_attend_workspace(csa_dtype dt, int64_t B, int64_t Tq, int64_t H, int64_t D,
                                int64_t Nc, int64_t m, int64_t W, int64_t q_pos0,
                                size_t *bytes);
csa_status hca_attend(csa_dtype dt, int64_t B, int64_t Tq, int64_t H, int64_t D,
                      int64_t Nc, int64_t m, int64_t W, int64_t q_pos0, float scale, csa_in q,
                      csa_in ck, csa_in cv, csa_in rk, csa_in rv, int64_t raw_pos0,
                      int64_t raw_len, csa_out o, void *ws, size_t ws_bytes,
                      hipStream_t stream);

/*
 * csa_quantize_mxfp8 -- MXFP8 (E4M3) encoding of rows, the storage of the
 * compressed KV entries (ai-papers.net article, hybrid attention section:
 * most KV entries are kept in FP8; the block format is the OCP Microscaling
 * one of the FP4 indexer keys).  Per run of 32 values: scale exponent
 * e = floor(log2 max|x|) - 8 clamped to [-127, 127] (-127 for an all-zero
 * run), stored as the byte e + 127; each value x * 2^-e is rounded to the
 * nearest E4M3 value (bias 7, subnormals k * 2^-9, largest 448; ties to the
 * even code, larger magnitudes saturate to 448), bit 7 = x's sign bit.
 *   x       [rows, d]      dt, finite values, 16-byte aligned
 *   codes   [rows, d]      uint8, 16-byte aligned
 *   scales  [rows, d/32]   uint8 (E8M0)
 * Requires d % 32 == 0.  Caller-owned device memory; nothing is allocated.
 */
csa_status csa_quantize_mxfp8(csa_dtype dt, int64_t rows, int64_t d, const void *x,
                              void *codes, void *scales, hipStream_t stream);

/*
 * csa_attend_mxfp8 / hca_attend_mxfp8 -- csa_attend / hca_attend (bf16) with
 * the compressed entries stored as MXFP8 (ai-papers.net article, hybrid
 * attention section: most KV entries in FP8).  The key and value of entry j
 * are the exact values code * 2^(scale - 127) of csa_quantize_mxfp8 output;
 * queries, the raw window rows and the output stay bf16, and the arithmetic
 * is that of the bf16 path (every such value is exact in bf16).
 *   ck, cv               [B, Nc, 128]   uint8 E4M3 codes, 16-byte aligned
 *   ck_scales, cv_scales [B, Nc, 4]     uint8 E8M0, 4-byte aligned
 *   q, o [B, Tq, H, 128] bf16; rk, rv [B, raw_len, 128] bf16; topk as for
 *   csa_attend; ws of at least csa_attend_workspace / hca_attend_workspace
 *   (CSA_BF16, same sizes) bytes.
 * Passing the same buffers as ck and cv, ck_scales and cv_scales, and rk and
 * rv selects the one-vector key-and-value reading (each row read once).
 * Requires D = 128 and H in {32, 64, 128, 256}; other arguments and errors
 * as for csa_attend / hca_attend.
 */
csa_status csa_attend_mxfp8(int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t Nc,
                            int64_t m, int64_t W, int64_t k, int64_t q_pos0, float scale,
                            const void *q, const void *ck, const void *cv,
                            const void *ck_scales, const void *cv_scales,
                            const int32_t *topk, const void *rk, const void *rv,
                            int64_t raw_pos0, int64_t raw_len, void *o, void *ws,
                            size_t ws_bytes, hipStream_t stream);
csa_status hca_attend_mxfp8(int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t Nc,
                            int64_t m, int64_t W, int64_t q_pos0, float scale,
                            const void *q, const void *ck, const void *cv,
                            const void *ck_scales, const void *cv_scales, const void *rk,
                            const void *rv, int64_t raw_pos0, int64_t raw_len, void *o,
                            void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * csa_quantize_fp8_rows -- E4M3 encoding of rows with ONE scale exponent per
 * row: the storage of every row that the FP8-arithmetic attention reads
 * (ai-papers.net article, hybrid attention section: most KV entries in FP8).
 * The exponent rule of csa_quantize_mxfp8 is applied to the whole row:
 * e = floor(log2 max|row|) - 8, clamped to [-127, 127] (-127 for a zero row);
 * each value x * 2^-e rounded to the nearest E4M3 value, ties to the even
 * code, saturating at 448, bit 7 = x's sign bit.  The row's scale is one
 * 32-bit word: the bits of the fp32 power of two 2^e, i.e. the E8M0 byte
 * e + 127 in bits 23..30 and zeros elsewhere (all zero for a zero row).
 *   x       [rows, d]   dt, finite values, 16-byte aligned
 *   codes   [rows, d]   uint8, 16-byte aligned
 *   scales  [rows]      uint32 words, 4-byte aligned
 * Requires d in {32, 64, 128, 256} (else CSA_EUNSUPPORTED).  Caller-owned
 * device memory; nothing is allocated.
 */
csa_status csa_quantize_fp8_rows(csa_dtype dt, int64_t rows, int64_t d, const void *x,
                                 void *codes, void *scales, hipStream_t stream);

/*
 * csa_attend_fp8 / hca_attend_fp8 -- csa_attend / hca_attend with FP8
 * arithmetic (ai-papers.net article, hybrid attention section: most KV
 * entries in FP8; jiwasawa.github.io post: shared-KV MQA over the selected
 * entries, dense HCA, the SWA window).  Every key and value row, compressed
 * entries and raw window rows alike, is an FP8 row as csa_quantize_fp8_rows
 * writes it, and each query head's row is encoded the same way inside the
 * call; the scores are the exact products of those values (scaled FP8 MFMA,
 * fp32 accumulation) and the softmax runs in fp32.  The probabilities, times
 * each value row's own scale, are rounded to E4M3 for the value product (a
 * relative error of at most 2^-4 per probability while p * 2^(e_v - E) >=
 * 2^-12, E the largest value exponent among the 64 keys it is processed
 * with); the softmax denominators add the unrounded probabilities.
 *   q, o                 [B, Tq, H, 128]  bf16, 16-byte aligned
 *   ck, cv               [B, Nc, 128]     uint8 E4M3 codes, 16-byte aligned
 *   ck_scales, cv_scales [B, Nc]          uint32 scale words, 4-byte aligned
 *   rk, rv               [B, raw_len, 128] codes; rk_scales, rv_scales
 *                        [B, raw_len] words, as for the compressed rows
 *   topk as for csa_attend; ws of at least csa_attend_workspace /
 *   hca_attend_workspace (CSA_BF16, same sizes) bytes.
 * Requires D = 128 and H in {32, 64, 128, 256}; other arguments and errors
 * as for csa_attend / hca_attend.
 */
csa_status csa_attend_fp8(int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t Nc,
                          int64_t m, int64_t W, int64_t k, int64_t q_pos0, float scale,
                          const void *q, const void *ck, const void *cv,
                          const void *ck_scales, const void *cv_scales,
                          const int32_t *topk, const void *rk, const void *rv,
                          const void *rk_scales, const void *rv_scales, int64_t raw_pos0,
                          int64_t raw_len, void *o, void *ws, size_t ws_bytes,
                          hipStream_t stream);
csa_status hca_attend_fp8(int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t Nc,
                          int64_t m, int64_t W, int64_t q_pos0, float scale,
                          const void *q, const void *ck, const void *cv,
                          const void *ck_scales, const void *cv_scales, const void *rk,
                          const void *rv, const void *rk_scales, const void *rv_scales,
                          int64_t raw_pos0, int64_t raw_len, void *o, void *ws,
                          size_t ws_bytes, hipStream_t stream);

/*
 * csa_index_attend -- csa_index_topk followed by csa_attend over the same
 * query rows (jiwasawa.github.io post, CSA indexer and shared-KV MQA
 * bullets), with bit-identical results (topk and o), scheduled as a
 * pipeline: the query rows of each sequence are cut into n_chunks slices of
 * ceil(Tq / n_chunks) rows; the selection of every slice runs on
 * aux_stream, and the attention of slice c runs on stream once its
 * selection is done, so one slice's attention overlaps the next slices'
 * selection.  aux_stream first waits for the work already queued on
 * stream, and stream has waited for all of aux_stream's work of this call
 * when the call returns (use the results on stream).  aux_stream == stream
 * (or n_chunks == 1) runs the two steps in order on stream.  Arguments,
 * layouts and requirements are those of the two entry points; topk
 * [B, Tq, k] is written; ws holds csa_index_attend_workspace bytes.  The
 * library keeps 65 HIP events per host thread and device, made at the first
 * call (a stream wait takes an event's state when it is queued, so later
 * calls may record them again at once).
 */
csa_status csa_index_attend_workspace(csa_dtype dt, int64_t B, int64_t Tq, int64_t H, int64_t D,
                                      int64_t HI, int64_t dI, int64_t Nc, int64_t m, int64_t W,
                                      int64_t k, int64_t q_pos0, int64_t n_chunks,
                                      size_t *bytes);
csa_status csa_index_attend(csa_dtype dt, int64_t B, int64_t Tq, int64_t H, int64_t D,
                            int64_t HI, int64_t dI, int64_t Nc, int64_t m, int64_t W, int64_t k,
                            int64_t q_pos0, float scale, const void *q, const void *q_idx,
                            const uint8_t *k_codes, const uint8_t *k_scales, const void *ck,
                            const void *cv, const void *rk, const void *rv, int64_t raw_pos0,
                            int64_t raw_len, int32_t *topk, void *o, int64_t n_chunks, void *ws,
                            size_t ws_bytes, hipStream_t stream, hipStream_t aux_stream);

/*
 * A stack of attention layers (hazakura.dev note, CSA/HCA bullets: HCA in
 * the first two layers of V4-Pro, the two kinds interleaved layer by layer;
 * studioglobal.ai answer, CSA/HCA section: from layer 2 the even layers are
 * CSA and the odd ones HCA; ai-papers.net article, hybrid attention section:
 * the 61-layer stack alternates the two).  The attention core of every
 * layer, run in order on one stream; what lies between layers (projections,
 * norms, the rest of the model) is not part of this library, so each layer
 * brings its own queries.
 */
typedef enum csa_layer_kind { CSA_LAYER_CSA = 0, CSA_LAYER_HCA = 1 } csa_layer_kind;

typedef struct csa_layer_desc {
    int32_t kind;              /* csa_layer_kind */
    int32_t reserved;          /* 0 */
    int64_t m;                 /* compression ratio of the layer's caches */
    int64_t Nc;                /* compressed rows held per sequence */
    const void *q;             /* [B, Tq, H, D] attention queries */
    const void *ck, *cv;       /* [B, Nc, D] compressed keys and values */
    const void *rk, *rv;       /* [B, raw_len, D] raw window rows */
    const void *q_idx;         /* CSA: [B, Tq, HI, dI] indexer queries */
    const uint8_t *k_codes;    /* CSA: [B, Nc, dI/2] MXFP4 indexer keys */
    const uint8_t *k_scales;   /* CSA: [B, Nc, dI/32] their E8M0 scales */
    int32_t *topk;             /* CSA: [B, Tq, k] kept entries (written) */
    void *o;                   /* [B, Tq, H, D] output (written) */
} csa_layer_desc;

/* The schedule the pages describe, for n_layers layers: kinds[0] and
 * kinds[1] are HCA; from layer 2 on, even layers are CSA and odd ones HCA
 * (61 layers: 30 CSA, 31 HCA). */
csa_status csa_layer_schedule(int64_t n_layers, int32_t *kinds);

/*
 * csa_stack_attend -- every layer in order: a CSA layer runs csa_index_topk
 * (into its topk) and csa_attend, an HCA layer runs hca_attend, with the
 * layer's own m, Nc and buffers and the shared sizes, window, q_pos0,
 * raw_pos0, raw_len and scale.  All layers are checked before the first
 * launch: an invalid layer returns its error (message "layer l: ...") and
 * nothing runs.  One workspace of csa_stack_workspace bytes serves every
 * layer in turn (stream order).  dt is the dtype of every floating-point
 * tensor of every layer.
 */
csa_status csa_stack_workspace(csa_dtype dt, int64_t n_layers, const csa_layer_desc *layers,
                               int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t HI,
                               int64_t dI, int64_t W, int64_t k, int64_t q_pos0, size_t *bytes);
csa_status csa_stack_attend(csa_dtype dt, int64_t n_layers, const csa_layer_desc *layers,
                            int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t HI, int64_t dI,
                            int64_t W, int64_t k, int64_t q_pos0, float scale, int64_t raw_pos0,
                            int64_t raw_len, void *ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H */
