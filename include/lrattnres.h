/* liblrattnres: the LR-AttnRes depth-mix read on AMD Instinct MI355X (gfx950).
 *
 * The read (LR-AttnRes paper, §3.1 routing equation with the sliced key of §3.3; the
 * author's explainer, "A short description chooses a full-width value"): for every token t
 * at one read site with n sources o_1..o_n (each a row of d values) and the site's static
 * query q (r values, the same for every token),
 *
 *     k_i     = the last r coordinates of o_i                 (a view, no key projection)
 *     rho_i   = sqrt(mean_j k_ij^2 + eps)                      (parameter-free RMS)
 *     z_i     = q . k_i / rho_i
 *     alpha_i = exp(z_i) / sum_j exp(z_j)                      (softmax over sources)
 *     h       = sum_i alpha_i o_i                              (all d coordinates)
 *
 * With r = d this is standard AttnRes. The two-phase block schedule (AttnRes technical-report
 * summary, "Method": Phase 1 batches a block's static queries against the cached block
 * representations, Phase 2 merges each site's intra-block partial sum by an online-softmax
 * update; LR-AttnRes paper §3.4 shows the sliced key keeps both conditions) is exposed as
 * lrar_forward_stats + lrar_merge. The backward follows the paper's App. B.3 (Lemma 2 and
 * Corollary 2.1).
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument named src/out/acc/m/l/q/dout/dsrc/dq/alpha/workspace is a
 *     DEVICE pointer; arrays of pointers (src, src_ld, dsrc, dsrc_ld) are HOST arrays that
 *     are read during the call only. The caller owns all memory; the library never
 *     allocates, frees or synchronises.
 *   - Matrices are row-major with an explicit row stride in ELEMENTS of their own type
 *     (ld >= d). A source is [T, d]; several sources may be the same buffer. The row stride
 *     of a source, key, accumulator or partial sum may not exceed 256 MiB (else
 *     LRAR_ERR_UNSUPPORTED): the kernels address a tile's rows by 32-bit byte offsets.
 *   - io selects the element type of sources and of out: LRAR_BF16 (raw bfloat16 bits) or
 *     LRAR_F32. q, m, l, alpha, dout, dsrc and dq are always float32.
 *   - Arithmetic: scores, RMS and softmax in float64 (bf16 x fp32 products are exact in
 *     float64); the value mix accumulates in float32 and rounds to nearest-even on output.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and is
 *     asynchronous. Calls that overlap on one device race only on buffers they share.
 *   - Every function validates all arguments before touching the device and returns a
 *     status; nothing throws or aborts. lrar_last_error() describes the last failure on
 *     the calling thread.
 *   - Aliasing: no output may share a byte with any other buffer of the call (inputs may share
 *     bytes with each other: repeated and strided sources are legal). Buffers are compared as
 *     the rows they touch, exactly when they share one row stride, so column slices of one
 *     wide buffer may be sources and output together; a partial overlap returns
 *     LRAR_ERR_INVALID (at T > 0). The one exception is lrar_merge_accumulate's in-place update.
 *   - Rows are fully vectorised (16-byte accesses) when d is a multiple of 8 (bf16) or 4
 *     (f32) and every row start is 16-byte aligned; other shapes (e.g. d = 513, odd
 *     strides) take a scalar-element path that computes the same result more slowly.
 *   - A "register tile" holds a whole row in registers: up to 32 chunks of 64 units, i.e.
 *     d <= 16384 (bf16) / 8192 (f32) on the vector path and d <= 2048 on the element path.
 *     The one-pass reads run on such tiles; rows wider than a tile are served by a
 *     column-chunked kernel that reads the keys first, takes the softmax once and then streams
 *     the rows (the key bytes are read twice).
 */
#ifndef LRATTNRES_H_
#define LRATTNRES_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LRAR_MAX_SOURCES 64 /* sources per read (full routing needs 2L+1) */
#define LRAR_MAX_QUERIES 64 /* site queries per Phase-1 call */

typedef enum lrar_status {
  LRAR_OK = 0,
  LRAR_ERR_INVALID = 1,     /* an argument is out of range, null or aliased */
  LRAR_ERR_UNSUPPORTED = 2, /* valid, but this shape/variant combination is not built */
  LRAR_ERR_DEVICE = 3       /* the HIP runtime reported an error at launch */
} lrar_status;

typedef enum lrar_dtype { LRAR_F32 = 0, LRAR_BF16 = 1 } lrar_dtype;

typedef enum lrar_variant {
  LRAR_VARIANT_AUTO = 0,     /* pick per shape */
  LRAR_VARIANT_TWO_PASS = 1, /* key slices first, softmax once, then stream the values */
  LRAR_VARIANT_ONLINE = 2    /* one pass per source with an online-softmax accumulator */
} lrar_variant;

/* The depth-mix read (LR-AttnRes paper §3.1 routing equation, §3.3 routing keys; explainer,
 * "A short description chooses a full-width value").
 *   T, d, r, eps : tokens, width, key width (1 <= r <= d), RMS epsilon (>= 0, finite;
 *                  eps = 0 is allowed and yields NaN for an all-zero key slice).
 *   io           : element type of the sources and of out.
 *   n, src, src_ld : 1 <= n <= LRAR_MAX_SOURCES sources; src[i] is a device [T, src_ld[i]]
 *                  matrix of which the first d columns are used.
 *   q            : device float32 [r], the site query.
 *   out, out_ld  : device [T, out_ld] of type io; receives h. Overlaps no source.
 *   alpha, alpha_ld : optional device float32 [T, alpha_ld >= n]; receives the weights.
 *   variant      : lrar_variant. AUTO runs ONLINE when the row fits a register tile and
 *                  TWO_PASS otherwise; TWO_PASS serves any width; ONLINE returns
 *                  LRAR_ERR_UNSUPPORTED for rows wider than a register tile.
 * With n = 1 the output equals src[0] exactly (the embedding-only read is the identity). */
lrar_status lrar_forward(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                         int32_t n, const void* const* src, const int64_t* src_ld,
                         const float* q, void* out, int64_t out_ld, float* alpha,
                         int64_t alpha_ld, int32_t variant, void* stream);

/* lrar_forward that also saves, for the backward, each source's normalization and softmax
 * statistics (LR-AttnRes paper App. I, "Implementation": the fused kernel keeps them for its
 * backward): per row t, saved[t][i] = z_i (the score) and saved[t][n + i] = 1 / rho_i (the
 * reciprocal RMS of the key), both float64.
 *   saved, saved_ld : device float64 [T, saved_ld >= 2n]; overlaps no other buffer.
 * Other arguments as for lrar_forward (no weights output). lrar_backward_saved takes the
 * buffer. */
lrar_status lrar_forward_save(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                              int32_t n, const void* const* src, const int64_t* src_ld,
                              const float* q, void* out, int64_t out_ld, double* saved,
                              int64_t saved_ld, int32_t variant, void* stream);

/* The full-width-RMS control read (LR-AttnRes paper §4.4, Eq. 13 "control"; App. B.1): the
 * key of source i is its last r coordinates divided by the RMS of the whole row,
 *     kbar_i = tail_r(o_i) / sqrt(||o_i||^2 / d + eps),   z_i = q . kbar_i,
 * and h = sum_i softmax_i(z) o_i as in lrar_forward. Arguments as for lrar_forward. One pass
 * over the sources on a register tile; rows wider than a tile take the column-chunked kernel
 * (its key pass sums the square of every column). */
lrar_status lrar_forward_fullrms(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                                 int32_t n, const void* const* src, const int64_t* src_ld,
                                 const float* q, void* out, int64_t out_ld, float* alpha,
                                 int64_t alpha_ld, void* stream);

/* The separate-key read, the read side of Projected LR-AttnRes (LR-AttnRes paper App. C.1:
 * each source has its own r-wide key, RMS-normalised; App. C.2: a source then carries d + r
 * elements). Source i's value is src[i] (d wide) and its key the first r columns of key[i]:
 *     z_i = q . k_i / sqrt(||k_i||^2 / r + eps),   h = sum_i softmax_i(z) o_i.
 *   key, key_ld : host arrays of n device pointers [T, key_ld[i] >= r] of type io (1 <= r <= d).
 * Other arguments as for lrar_forward. One pass over the sources and keys on a register tile
 * when the row fits one and a spread key piece serves the key: r <= 64 with any key alignment,
 * or r <= 512 when r is a multiple of the per-lane piece (r / 32 or r / 64 rounded up to a power
 * of two) and the key rows are aligned to it (16 bytes at most). Every other key (any r, any
 * alignment) and rows wider than a tile take the column-chunked kernel, whose key pass reads the
 * key rows element by element. */
lrar_status lrar_forward_keys(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                              int32_t n, const void* const* src, const int64_t* src_ld,
                              const void* const* key, const int64_t* key_ld, const float* q,
                              void* out, int64_t out_ld, float* alpha, int64_t alpha_ld,
                              void* stream);

/* Phase 1 of the two-phase schedule (AttnRes technical-report summary, "Method"; LR-AttnRes
 * paper §3.4): nq site queries against the same n cached sources. For query s, token t:
 *     m[s][t]   = max_i z_si  rounded to float32,
 *     l[s][t]   = sum_i exp(z_si - m[s][t]),
 *     acc[s][t] = sum_i exp(z_si - m[s][t]) o_i     (d values, NOT normalised).
 *   q, q_ld       : device float32 [nq, q_ld >= r]; 1 <= nq <= LRAR_MAX_QUERIES.
 *   m, l, ml_ld   : device float32, element (s, t) at s * ml_ld + t, ml_ld >= T.
 *   acc           : element (s, t, j) at s * acc_qstride + t * acc_ld + j, in acc_dtype
 *                   (LRAR_F32 is exact enough for parity; LRAR_BF16 halves the bytes).
 *                   acc_ld >= d, acc_qstride >= T * acc_ld. m, l and acc overlap no other
 *                   buffer of the call. */
lrar_status lrar_forward_stats(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                               int32_t n, const void* const* src, const int64_t* src_ld,
                               int32_t nq, const float* q, int64_t q_ld, float* m, float* l,
                               int64_t ml_ld, void* acc, lrar_dtype acc_dtype, int64_t acc_ld,
                               int64_t acc_qstride, void* stream);

/* Phase 2 (AttnRes technical-report summary, "Method": Phase 2 merges each site's intra-block
 * partial sum into the Phase-1 statistics by an online-softmax update; LR-AttnRes paper §3.4:
 * the sliced key keeps that merge exact). Merges one site's (m, l, acc) with n >= 0 further
 * sources (normally the site's intra-block partial sum), and normalises:
 *     m' = max(m, max_b z_b),  l' = l e^{m-m'} + sum_b e^{z_b-m'},
 *     h  = (acc e^{m-m'} + sum_b e^{z_b-m'} o_b) / l'.
 *   m, l          : device float32 [T]; acc: device [T, acc_ld] of acc_dtype.
 *   n, src, src_ld, q : the extra sources and the site query (q may be NULL when n = 0).
 *   out, out_ld   : device [T, out_ld] of type io.
 *   m_out, l_out  : optional device float32 [T]; receive m' (rounded to float32) and l'
 *                   relative to that rounded m'.
 * Rows wider than a register tile take the column-chunked kernel. */
lrar_status lrar_merge(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                       const float* m, const float* l, const void* acc, lrar_dtype acc_dtype,
                       int64_t acc_ld, int32_t n, const void* const* src,
                       const int64_t* src_ld, const float* q, void* out, int64_t out_ld,
                       float* m_out, float* l_out, void* stream);

/* Phase 2 with the partial-sum update fused in (LR-AttnRes paper §3.3 "Partial-block routing":
 * the block's running partial sum is kept at full width, a new sub-layer output is added to it,
 * and the next read site takes the sum as a source; AttnRes technical-report summary, "Method",
 * Phase 2). In one pass:
 *     b_out = b + o                 (element type io, round to nearest even; b = 0 if NULL),
 *     then lrar_merge of (m, l, acc) with the single extra source b_out.
 * Reading b and o once and writing b_out replaces an update kernel plus a merge that reads
 * b_out again.
 *   b, b_ld       : device [T, b_ld] of type io, the block's partial sum so far, or NULL for
 *                   the block's first write.
 *   o, o_ld       : device [T, o_ld] of type io, the sub-layer output just written.
 *   b_out, b_out_ld : device [T, b_out_ld] of type io; receives b + o. It may be b or o itself
 *                   (same pointer and row stride: updated in place) but may not otherwise
 *                   overlap them, acc or out.
 *   Other arguments as for lrar_merge with n = 1. Rows wider than a register tile run as two
 *   kernels: b_out = b + o, then the column-chunked merge reads b_out. */
lrar_status lrar_merge_accumulate(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                                  const float* m, const float* l, const void* acc,
                                  lrar_dtype acc_dtype, int64_t acc_ld, const void* b,
                                  int64_t b_ld, const void* o, int64_t o_ld, void* b_out,
                                  int64_t b_out_ld, const float* q, void* out, int64_t out_ld,
                                  float* m_out, float* l_out, void* stream);

/* Backward of one read (LR-AttnRes paper App. B.3: Lemma 2 and Corollary 2.1), each source
 * slot treated as an independent input. With g = dout[t]:
 *     dz_i    = alpha_i <g, o_i - h>
 *     dsrc_i  = alpha_i g  +  on the last r coordinates: dz_i (q - z_i kbar_i / r) / rho_i
 *     dq      = sum_t sum_i dz_i kbar_i,       kbar_i = k_i / rho_i.
 *   dout, dout_ld : device float32 [T, dout_ld].
 *   dsrc, dsrc_ld : host array of n distinct device float32 [T, dsrc_ld[i]] pointers.
 *   accumulate    : 0 overwrites dsrc; 1 adds into it (a source's total gradient sums over
 *                   every read it takes part in).
 *   dq            : device float32 [r]; overwritten. The token sum is evaluated in a fixed
 *                   order, so results are bitwise reproducible.
 *   workspace     : device scratch of at least lrar_backward_workspace_size(T, d, r, n)
 *                   bytes, 8-byte aligned; its contents are not needed after the call.
 * Rows that fit a register tile (vector path: d a multiple of 8 (bf16) / 4 (f32), every row of
 * the sources, dout and dsrc 16-byte aligned, d <= 16384 / 8192) run on row tiles, with any r.
 * Other rows (the element path at any width; wider vector rows) run one wave per row and keep
 * query-gradient partials for the key's chunks of 64 units in registers: served when the key
 * spans at most 64 such chunks on the element path (r <= 4032 always) or 8 on the vector path
 * (8 x 64 units, r <= 3584 (bf16) / 1792 (f32) always); LRAR_ERR_UNSUPPORTED otherwise.
 * dsrc, dq and the workspace overlap no other buffer of the call (nor each other). */
lrar_status lrar_backward(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                          int32_t n, const void* const* src, const int64_t* src_ld,
                          const float* q, const float* dout, int64_t dout_ld,
                          float* const* dsrc, const int64_t* dsrc_ld, int32_t accumulate,
                          float* dq, void* workspace, size_t workspace_bytes, void* stream);

/* lrar_backward with the gradients in grad_dtype (the pages' own kernel writes bf16 source
 * gradients: LR-AttnRes paper App. I). dout is a device [T, dout_ld] array of grad_dtype and
 * dsrc a host array of n distinct device [T, dsrc_ld[i]] arrays of grad_dtype. Every value is
 * computed in float32 / float64 as in lrar_backward; with LRAR_BF16 the source gradient (after
 * the optional addition of the existing one) is rounded to nearest even once. dq stays float32.
 * The vector path needs every dout and dsrc row 16-byte aligned. Other arguments, limits and
 * the workspace as for lrar_backward (lrar_backward_grad with LRAR_F32 is lrar_backward). */
lrar_status lrar_backward_grad(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                               int32_t n, const void* const* src, const int64_t* src_ld,
                               const float* q, lrar_dtype grad_dtype, const void* dout,
                               int64_t dout_ld, void* const* dsrc, const int64_t* dsrc_ld,
                               int32_t accumulate, float* dq, void* workspace,
                               size_t workspace_bytes, void* stream);

/* lrar_backward_grad from the statistics lrar_forward_save kept (LR-AttnRes paper App. I,
 * "Implementation"; App. B.3): the scores z_i and reciprocal RMS 1 / rho_i are read from
 * `saved` (device float64 [T, saved_ld >= 2n], as lrar_forward_save wrote it for the same
 * sources, q and eps) instead of being recomputed from the keys, so the key pass reduces only
 * s_i = <g, o_i>. eps enters through the saved 1 / rho_i and is not an argument. A weights array
 * alone would not do: the key columns' gradient needs z_i and rho_i themselves. Other
 * arguments, limits and the workspace as for lrar_backward_grad. */
lrar_status lrar_backward_saved(int64_t T, int32_t d, int32_t r, lrar_dtype io, int32_t n,
                                const void* const* src, const int64_t* src_ld, const float* q,
                                const double* saved, int64_t saved_ld, lrar_dtype grad_dtype,
                                const void* dout, int64_t dout_ld, void* const* dsrc,
                                const int64_t* dsrc_ld, int32_t accumulate, float* dq,
                                void* workspace, size_t workspace_bytes, void* stream);

/* lrar_backward_grad with no workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the query-gradient partials go to a 32 MiB scratch array that the library holds in each
 * GPU's memory until the process ends. The call allocates and frees nothing. Arguments, results
 * and limits as for lrar_backward_grad. The workspace entry point's workgroup count is kept
 * when its partials ((grid + 32) * r float64 values) fit the scratch, so the results are the
 * same bits; otherwise fewer workgroups are used (dq then sums in another fixed order), and a
 * key so wide that fewer than min(256, that count) workgroups would fit returns
 * LRAR_ERR_UNSUPPORTED (only possible for r > 14563).
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one GPU (different
 * streams, or host threads) race, and must be ordered by the caller. Nothing in the scratch
 * needs to be cleared between calls. */
lrar_status lrar_backward_noalloc(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                                  int32_t n, const void* const* src, const int64_t* src_ld,
                                  const float* q, lrar_dtype grad_dtype, const void* dout,
                                  int64_t dout_ld, void* const* dsrc, const int64_t* dsrc_ld,
                                  int32_t accumulate, float* dq, void* stream);

/* Bytes of device workspace lrar_backward needs for this shape (0 if T = 0). */
size_t lrar_backward_workspace_size(int64_t T, int32_t d, int32_t r, int32_t n);

/* A plain streaming device-to-device copy of `bytes` bytes (both pointers 16-byte aligned,
 * bytes a multiple of 16). Not part of the read: it is the reference kernel used to
 * calibrate hardware traffic counters and to measure the achievable copy bandwidth. */
lrar_status lrar_copy(void* dst, const void* src, size_t bytes, void* stream);

/* A plain streaming read of `bytes` bytes (src 16-byte aligned, bytes a multiple of 16) that
 * folds them into one 32-bit word per thread written to `sink` (device, 4-byte aligned,
 * lrar_read_stream_sink_bytes() bytes, not overlapping src). Not part of the read: it is the
 * reference kernel for the read-bandwidth ceiling. */
lrar_status lrar_read_stream(const void* src, size_t bytes, void* sink, void* stream);

/* Bytes of the sink lrar_read_stream writes. */
size_t lrar_read_stream_sink_bytes(void);

/* A plain stream with a kernel's traffic: for each of T rows, reads the n bf16 source rows of d
 * columns (src as for lrar_forward, n in [1, LRAR_MAX_SOURCES]) and writes their mean, summed
 * in float32 in source order, to each of nout output rows: out[j] is a device [T, out_ld[j]]
 * matrix of out_dtype (LRAR_F32: the float32 sum; LRAR_BF16: rounded to nearest even),
 * 1 <= nout <= LRAR_MAX_SOURCES; out and out_ld are HOST arrays of nout entries. One bf16
 * output gives a read's traffic; more outputs or float32 ones give the write-heavy mixes of
 * Phase 1 (8 rows in, 12 accumulator rows out per token) and the backward. Not part of the
 * read: it is the reference kernel for the same-traffic bandwidth ceiling a kernel is measured
 * against. d and every src_ld are multiples of 8, every out_ld a multiple of 16 bytes, and
 * every pointer is 16-byte aligned; no output may overlap a source or another output. The
 * launch shape is the caller's: waves_per_cu (4, 8, ..., 32) waves per compute unit;
 * waves_per_row (1, 2 or 4) waves of one workgroup sharing each row, as the reads of wide
 * rows share theirs; slots (2, 4, 8 or 16) 16-byte units a lane, so the waves of a row take it
 * in passes of 64 x slots x waves_per_row units, 64-unit chunks dealt to them in turn; depth
 * (1, 2 or 4, with depth x slots <= 16) sources loaded together before any is added;
 * rows_per_wave (> 0: launches of that many rows per row group; 0: one launch); and lockstep
 * (0: none; 1 or 2: the waves of a workgroup meet at a barrier once per row, or once per
 * group of depth sources, as the reads keep their waves together). Errors as for
 * lrar_forward. */
lrar_status lrar_mix_stream(int64_t T, int32_t d, int32_t n, const void* const* src,
                            const int64_t* src_ld, int32_t nout, void* const* out,
                            const int64_t* out_ld, lrar_dtype out_dtype, int32_t waves_per_cu,
                            int32_t waves_per_row, int32_t depth, int32_t slots,
                            int32_t rows_per_wave, int32_t lockstep, void* stream);

/* Static description of a status code. */
const char* lrar_status_string(lrar_status status);

/* Thread-local description of the last non-OK status returned on this thread. */
const char* lrar_last_error(void);

/* Library version, e.g. "0.1.0". */
const char* lrar_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LRATTNRES_H_ */
