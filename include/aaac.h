/*
 * aaac.h -- C ABI of the MI355X (gfx950) activation-aware dual-codebook 4-bit weight quantizer.
 *
 * Method: the gist.science summary page "기술 요약: AAAC (활성화 인식 적응형 코드북)"
 * (arXiv 2605.08692), cited as "AAAC summary" with its section number. Each weight matrix gets two
 * learned scalar tables T0, T1 of n entries (n = 16 for INT4, 15 for NVFP4; §2 mechanism 1); every
 * group of g weights gets a positive scale; every selection group of S weights picks the table with
 * the lower activation-weighted reconstruction error (§2 mechanism 2); the tables are refined as
 * activation-weighted k-means centroids, alternating with the assignment (§2 mechanism 4); the
 * result is stored as 4-bit codes, bf16 tables, and the table choice in the sign bit of the bf16
 * scale or in a separate bitmap (§2 mechanism 3).
 *
 * Conventions for every call:
 *  - W is bf16 [R, C] row-major (out x in), passed as uint16_t bit patterns. A scale group is g
 *    consecutive weights of a row, a selection group S consecutive weights; groups never cross rows.
 *  - Supported shapes: g and S powers of two with 8 <= S <= g <= 512, C % g == 0, R >= 1,
 *    2 <= n <= 16, R * C < 2^40. Device pointers must be 16-byte aligned.
 *  - All data pointers are DEVICE pointers owned by the caller. The library never allocates, frees
 *    or synchronizes; every call checks its arguments on the host, enqueues its kernels on `stream`
 *    (a hipStream_t; NULL means the default stream) and returns. Buffers must stay alive until the
 *    stream work has completed.
 *  - A failed check returns a non-zero status BEFORE anything is launched, so nothing is written.
 *    AAAC_ERR_HIP reports a launch error seen through hipGetLastError; aaac_last_error() returns a
 *    message for the last failure on the calling thread.
 *  - Workspaces are caller-owned device buffers of at least aaac_workspace_bytes(...) bytes, 256-byte
 *    aligned, and ZERO-FILLED before their first use; every call leaves its workspace zero-filled
 *    again where that matters (the counters), so one workspace can be reused call after call on one
 *    stream. Calls that overlap on different streams need different workspaces.
 *  - Weights must be finite. Results are bitwise deterministic for given inputs and device.
 *  - Tables are fp32 [2][n] (T0 then T1) while iterating; bf16 [2][n] bit patterns when packed.
 */
#ifndef AAAC_H
#define AAAC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t aaac_status;

#define AAAC_OK 0
#define AAAC_ERR_INVALID_ARG 1          /* null pointer, misaligned pointer, bad flag */
#define AAAC_ERR_UNSUPPORTED_SHAPE 2    /* g, S, n, R, C outside the supported set */
#define AAAC_ERR_WORKSPACE_TOO_SMALL 3  /* ws_bytes below aaac_workspace_bytes(...) */
#define AAAC_ERR_HIP 4                  /* the HIP runtime reported an error */

/* Workspace query operations. */
#define AAAC_OP_IMPORTANCE 0
#define AAAC_OP_INIT 1
#define AAAC_OP_ASSIGN 2
#define AAAC_OP_REFINE 3

/* Flags of aaac_refine. */
#define AAAC_REFINE_ROUND_BF16 1        /* round the new tables to bf16 (ties to even), stored as fp32 */
#define AAAC_REFINE_W2_KNOWN 2          /* *w2 already holds sum I w^2 of this matrix (see err) */

/* Static description of a status code. Never NULL. */
const char* aaac_status_string(aaac_status status);

/* Detail of the last failure on the calling thread ("" if none). Valid until the next call on
 * this thread. */
const char* aaac_last_error(void);

/* Workspace bytes needed by one call of operation `op` on an [R, C] matrix (for IMPORTANCE, R is
 * the token count T and C the column count K). Returns 0 for an unknown op or unsupported shape. */
size_t aaac_workspace_bytes(int op, int64_t R, int64_t C, int g, int S, int n);

/*
 * Importance, AAAC summary §2 mechanism 2: I_k = sum_t X[t, k]^2 over the calibration tokens.
 *
 * X      fp32 [T, K] with row stride ldx >= K (elements); one chunk of the token stream.
 * I_acc  fp64 [K], accumulated in place: I_acc[k] += sum_t X[t, k]^2 (fp32 squares are exact in
 *        fp64). Zero it before the first chunk; chunks may follow in any number of calls.
 * I_out  fp32 [K] or NULL; if given, receives I_acc rounded to fp32 after this chunk.
 * ws     workspace of aaac_workspace_bytes(AAAC_OP_IMPORTANCE, T, K, 0, 0, 0) bytes.
 * T == 0 is allowed (I_out is still written). The sum over a chunk is taken in a fixed order.
 */
aaac_status aaac_importance(const float* X, int64_t T, int64_t K, int64_t ldx, double* I_acc,
                            float* I_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Table initialization, AAAC summary §2 mechanism 4: equally spaced quantiles of the normalized
 * weight distribution, T1 shifted half a step. With s = max |w| over the scale group,
 * u = fl32(w / s) (u = +0 when s = 0), V the ascending sort of all N = R*C values of u:
 *   T0[j] = V[floor((2j + 1) N / (2n))],  T1[j] = V[min(N - 1, floor((j + 1) N / n))].
 * Found by an exact radix select; tables fp32 [2][n] (output).
 * ws: aaac_workspace_bytes(AAAC_OP_INIT, R, C, g, 0, n) bytes.
 */
aaac_status aaac_init_quantiles(const uint16_t* W, int64_t R, int64_t C, int g, int n,
                                float* tables, void* ws, size_t ws_bytes, void* stream);

/*
 * Assign, AAAC summary §2 mechanisms 2 and 4. For every weight and table c, q_c is the entry
 * nearest to u = w / s (ties to the lower index); for every selection group H,
 *   E_c(H) = sum_{k in H} I_k (w_k - s T_c[q_c(k)])^2,   sel(H) = 1 iff E_1 < E_0,
 * and the stored code is q_sel. The nearest entry is decided on exactly rounded fp32 residuals
 * w - s T (a differing decision is only possible when the two squared distances agree to 2.4e-7
 * relative); the selection compares E_1 - E_0 accumulated in fp32 over at most four terms and in
 * fp64 beyond (a differing decision needs |E_1 - E_0| < 1e-6 max(E_0, E_1)).
 *
 * I       fp32 [C] importance (finite, >= 0).
 * tables  fp32 [2][n], any order, duplicates allowed.
 * codes   [R * C / 2] bytes, two codes per byte, the low nibble holds the even column.
 * sel     [R * C / S] bytes, 0 = T0, 1 = T1, one per selection group in row-major order.
 * err     NULL, or fp64 [R * C / S][2] receiving (E_0, E_1) per selection group (for checking).
 * err_total  NULL, or one fp64 receiving the total weighted error of the assignment,
 *         sum over H of E_sel(H) (the k-means objective that the alternation never increases, §2
 *         mechanism 4). Summed in a fixed order (lanes in row order, then waves, then workgroups
 *         in order; no floating-point atomics), so it is reproducible call after call. Needs ws.
 * ws      with err_total: aaac_workspace_bytes(AAAC_OP_ASSIGN, R, C, g, S, n) bytes, same
 *         zero-fill rule as the other workspaces; otherwise ignored (may be NULL, ws_bytes 0).
 * One kernel (the lookup structure lives in LDS).
 */
aaac_status aaac_assign(const uint16_t* W, int64_t R, int64_t C, int g, int S, int n,
                        const float* I, const float* tables, uint8_t* codes, uint8_t* sel,
                        double* err, double* err_total, void* ws, size_t ws_bytes, void* stream);

/*
 * Refine, AAAC summary §2 mechanism 4 (activation-weighted k-means). For every table c and entry j,
 * over the cell {weights with sel = c and code = j}:
 *   num = sum I_k s w_k,  den = sum I_k s^2,   T_c[j] <- num / den if den > 0, else unchanged.
 * num / den minimizes sum I (w - s t)^2 over t, i.e. it is the I s^2-weighted centroid of u.
 * Every term is exact in fp64 and is added in fp64, per thread, then across threads and workgroups
 * in a fixed order, so the result is bitwise reproducible.
 * One kernel: the last workgroup to finish a matrix (an integer ticket in the workspace) adds the
 * per-workgroup partials and writes tables_out. The ticket is reset at the end of every call; a call
 * that did not complete (a device fault) leaves the workspace to be zero-filled again.
 *
 * codes, sel   as written by aaac_assign.
 * tables_in    fp32 [2][n];  tables_out fp32 [2][n], may equal tables_in.
 * flags        0, or AAAC_REFINE_ROUND_BF16 (round the new entries to bf16; used on the last
 *              iteration so that the final assign runs against the stored tables) and/or
 *              AAAC_REFINE_W2_KNOWN (see w2; needs err).
 * err          NULL, or two fp64: err[0] receives the total weighted error of the incoming
 *              assignment under tables_in (the codes and selectors as the assign half-step left
 *              them: the quantity aaac_assign's err_total reports), err[1] the same assignment's
 *              error under the tables this call writes (after this half-step; after the bf16
 *              rounding when that flag is set). Both are formed from the cell sums as
 *              E = W2 - 2 sum_cells T num + sum_cells T^2 den with W2 = sum I_k w_k^2 (sums of
 *              exact fp64 terms). Their absolute accuracy is about 1e-15 W2, far below E except
 *              for matrices quantized almost exactly (aaac_assign's err_total has no such limit).
 * w2           with err: one fp64. Without AAAC_REFINE_W2_KNOWN the kernel sums W2 (one more fp64
 *              fma per weight) and writes it here; with the flag it reads W2 from here (the value
 *              an earlier call on the same W and I wrote), at no cost per weight. NULL without err.
 * ws           aaac_workspace_bytes(AAAC_OP_REFINE, R, C, g, S, n) bytes.
 */
aaac_status aaac_refine(const uint16_t* W, int64_t R, int64_t C, int g, int S, int n,
                        const float* I, const uint8_t* codes, const uint8_t* sel,
                        const float* tables_in, float* tables_out, int flags, double* err,
                        double* w2, void* ws, size_t ws_bytes, void* stream);

/*
 * Pack, AAAC summary §2 mechanism 3 and §4: the stored format.
 *   codes_u8  NULL, or codes given one per byte: u8 [R * C], the code of (r, c) in the low nibble
 *             of byte r * C + c (the high nibble is ignored). Then codes_out (u8 [R * C / 2], not
 *             NULL, 4-byte aligned; codes_u8 8-byte aligned) receives them two per byte, the even
 *             column in the low nibble: the layout aaac_assign writes and aaac_dequant reads. Codes
 *             from aaac_assign are already in that layout and need neither (both NULL).
 *   scales    [R * C / g] bf16 bit patterns of s = max |w| over each scale group; when S == g the
 *             sign bit holds the selector (1 = T1), when S < g it is 0.
 *   bitmap    S < g: [ceil(R * C / S / 8)] bytes, bit i (byte i >> 3, bit i & 7) = selector of the
 *             i-th selection group in row-major order (1 / S extra bits per weight). S == g: NULL.
 *   tables_bf16 [2][n] bf16 bit patterns of the tables (ties to even).
 * Errors: AAAC_ERR_INVALID_ARG for codes_u8 without codes_out (or the reverse) or a misaligned
 * pointer; shape errors as for aaac_assign.
 */
aaac_status aaac_pack(const uint16_t* W, int64_t R, int64_t C, int g, int S, int n,
                      const uint8_t* sel, const float* tables, const uint8_t* codes_u8,
                      uint8_t* codes_out, uint16_t* scales, uint8_t* bitmap,
                      uint16_t* tables_bf16, void* stream);

/*
 * Dequantize, AAAC summary §1 (the dequantized values are what inference uses) and §2 mechanism 3:
 *   W_hat = bf16(|s| * T~_sel[q])  (the product of two bf16 values is exact in fp32; one rounding,
 *   ties to even), with the selector read from the scale sign bit (bitmap == NULL, S == g) or from
 *   the bitmap (S < g).
 * W_hat  bf16 [R, C] bit patterns (output).
 */
aaac_status aaac_dequant(const uint8_t* codes, const uint16_t* scales, const uint8_t* bitmap,
                         const uint16_t* tables_bf16, int64_t R, int64_t C, int g, int S, int n,
                         uint16_t* W_hat, void* stream);

/*
 * Pack and dequantize up to AAAC_MAX_BATCH matrices that share g, S and n, in one set of launches
 * (pack: 1, or 2 with bitmaps; dequant: 1): every output as aaac_pack / aaac_dequant give for
 * matrix i, bit for bit. Arrays of count per-matrix arguments, laid out and owned as in the
 * single calls; bitmap may be NULL when S == g (else it and every bitmap[i] must be given).
 * Errors: AAAC_ERR_INVALID_ARG for count outside [1, AAAC_MAX_BATCH], a null array, or any matrix
 * the single call would reject (nothing is launched then).
 */
aaac_status aaac_pack_batch(int count, const uint16_t* const* W, const int64_t* R,
                            const int64_t* C, int g, int S, int n, const uint8_t* const* sel,
                            const float* const* tables, uint16_t* const* scales,
                            uint8_t* const* bitmap, uint16_t* const* tables_bf16, void* stream);
aaac_status aaac_dequant_batch(int count, const uint8_t* const* codes,
                               const uint16_t* const* scales, const uint8_t* const* bitmap,
                               const uint16_t* const* tables_bf16, const int64_t* R,
                               const int64_t* C, int g, int S, int n, uint16_t* const* W_hat,
                               void* stream);

/*
 * Decode GEMV on the packed format, AAAC summary §1 (4-bit weights with 16-bit activations, W4A16;
 * the dequantized values are the weights inference uses) and §2 mechanism 3 (the stored format):
 *   y[b, r] = sum_c |s(r, c)| * T~_sel(r, c)[q(r, c)] * x[b, c]      for b < B
 * The weight is the exact product of the bf16 scale and the bf16 table entry (both are bf16, so the
 * product is exact in fp32); unlike aaac_dequant it is not rounded to bf16 first. Sums run in fp32
 * in a fixed order (bitwise reproducible): within a scale group, then scaled by |s|, then across
 * groups; a code >= n reads entry 0, as in aaac_dequant.
 * codes, scales, bitmap, tables_bf16  as written by aaac_assign / aaac_pack (bitmap NULL iff S == g).
 *                                     codes 16-byte aligned, scales 8-byte aligned.
 * x   bf16 [B, C] bit patterns (row stride C), 16-byte aligned; 1 <= B <= 4.
 * y   fp32 [B, R] (output, row stride R).
 * Shapes as for the other calls, and C % 32 == 0.
 */
aaac_status aaac_gemv(const uint8_t* codes, const uint16_t* scales, const uint8_t* bitmap,
                      const uint16_t* tables_bf16, int64_t R, int64_t C, int g, int S, int n,
                      const uint16_t* x, int B, float* y, void* stream);

/* aaac_gemv over up to AAAC_MAX_BATCH matrices sharing g, S, n and B in one launch (for example
 * every linear of a decoder layer for one decode step). bitmap is an array of count pointers when
 * S < g, else NULL. Results are bitwise identical to one aaac_gemv call per matrix. */
aaac_status aaac_gemv_batch(int count, const uint8_t* const* codes, const uint16_t* const* scales,
                            const uint8_t* const* bitmap, const uint16_t* const* tables_bf16,
                            const int64_t* R, const int64_t* C, int g, int S, int n,
                            const uint16_t* const* x, int B, float* const* y, void* stream);

/*
 * AWQ composition hook, AAAC summary §4 (AAAC on weights that AWQ scaled before quantization; the
 * search for the scales is not part of this library). Given a positive finite per-column scale
 * a [C] (fp32), prepares the inputs that quantize W diag(a) against the importance that matches
 * it, the energy of the inputs x / a that the scaled matrix sees at inference:
 *   W_scaled[r, c] = bf16(W[r, c] * a[c])   exact product, one rounding (ties to even); a product
 *                                           past the bf16 range becomes infinite, so choose a that
 *                                           keeps the weights finite
 *   I_scaled[c]    = fp32(I[c] / a[c]^2)    one fp64 division of exact operands, then fp32
 * W, W_scaled  bf16 [R, C]; W_scaled may be W (in place). 16-byte aligned.
 * a            fp32 [C], 16-byte aligned.
 * I, I_scaled  fp32 [C], both NULL or both given; I_scaled may be I.
 * The rest of the pipeline then runs on (W_scaled, I_scaled) unchanged. Shapes: R >= 1, C >= 8,
 * C % 8 == 0, R * C < 2^40.
 */
aaac_status aaac_awq_prescale(const uint16_t* W, int64_t R, int64_t C, const float* a,
                              const float* I, uint16_t* W_scaled, float* I_scaled, void* stream);

/*
 * Batched assign / refine over up to AAAC_MAX_BATCH matrices that share g, S and n (for example
 * the seven linears of one decoder layer) in one launch each. Element i of every array describes
 * matrix i exactly as the single-matrix call does; the results are bitwise identical to calling
 * the single-matrix entry points one matrix at a time, except where a sum's rounding depends on
 * how the rows are split over workgroups (the refine sums and err_total: the same call gives the
 * same bits every time; against single calls they agree to rounding). refine updates tables[i] in
 * place. The host arrays are read during the call only. The refine workspace holds
 * aaac_batch_workspace_bytes(AAAC_OP_REFINE, count, R, C, g, S, n) bytes, same zero-fill rule as
 * above. assign: err_total is NULL or fp64 [count] (the total of matrix i in err_total[i]), with
 * a workspace of aaac_batch_workspace_bytes(AAAC_OP_ASSIGN, count, R, C, g, S, n) bytes.
 * refine: err is NULL or fp64 [2][count] (matrix i's error before the update at err[i], after it
 * at err[count + i]), w2 NULL or fp64 [count] (matrix i's at index i); as in aaac_refine.
 */
#define AAAC_MAX_BATCH 8

size_t aaac_batch_workspace_bytes(int op, int count, const int64_t* R, const int64_t* C, int g,
                                  int S, int n);

/*
 * Init for up to AAAC_MAX_BATCH matrices sharing g and n, in one set of launches (6 in all, not 6
 * per matrix): tables[i] as aaac_init_quantiles gives for matrix i, bit for bit. The workspace
 * holds aaac_batch_workspace_bytes(AAAC_OP_INIT, count, R, C, g, 8, n) bytes (fixed headers of
 * histograms, then the keys of every matrix), zero-filled before its first use; every call leaves
 * the headers zero again, so one workspace serves any later batch that fits in it.
 */
aaac_status aaac_init_quantiles_batch(int count, const uint16_t* const* W, const int64_t* R,
                                      const int64_t* C, int g, int n, float* const* tables,
                                      void* ws, size_t ws_bytes, void* stream);

aaac_status aaac_assign_batch(int count, const uint16_t* const* W, const int64_t* R,
                              const int64_t* C, int g, int S, int n, const float* const* I,
                              const float* const* tables, uint8_t* const* codes,
                              uint8_t* const* sel, double* err_total, void* ws, size_t ws_bytes,
                              void* stream);

aaac_status aaac_refine_batch(int count, const uint16_t* const* W, const int64_t* R,
                              const int64_t* C, int g, int S, int n, const float* const* I,
                              const uint8_t* const* codes, const uint8_t* const* sel,
                              float* const* tables, int flags, double* err, double* w2, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * aaac_refine_batch without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation). The
 * counters and per-workgroup partials live in a fixed array in the library's device memory: each
 * GPU the library runs on holds one copy, of 256 + 8 * 66 * 1024 * 8 bytes (about 4.3 MB), until
 * the process ends; its address on a device is looked up once, on the first call there. Every
 * other argument, and every result, is as for aaac_refine_batch (bit for bit the same). The call
 * allocates nothing and launches a small kernel that clears the counters before the refine.
 * All calls on one GPU share that array, so calls that overlap on one GPU (on different streams,
 * or from different threads) race and must not be issued; calls on one stream are ordered.
 * Errors: as aaac_refine_batch; AAAC_ERR_WORKSPACE_TOO_SMALL if a batch needed more scratch than
 * the array holds (not possible within AAAC_MAX_BATCH matrices); AAAC_ERR_HIP if the array's
 * address cannot be obtained.
 */
aaac_status aaac_refine_batch_noalloc(int count, const uint16_t* const* W, const int64_t* R,
                                      const int64_t* C, int g, int S, int n,
                                      const float* const* I, const uint8_t* const* codes,
                                      const uint8_t* const* sel, float* const* tables, int flags,
                                      double* err, double* w2, void* stream);

/*
 * One iteration of the alternation (AAAC summary §2 mechanism 4) in one launch: the batched assign
 * against tables[i], writing codes[i] and sel[i], then the batched refine from those codes,
 * updating tables[i] in place. flags, err and w2 are as for aaac_refine_batch: err[i] receives the
 * weighted error of the assignment this call makes under the tables it was made with, and
 * err[count + i] under the tables it writes. Codes, selectors, tables and errors are bitwise those
 * of aaac_assign_batch followed by aaac_refine_batch with the same arguments. With S >= 16 one kernel does both: each wave assigns
 * a row and adds its terms into the refine bins at once, so W is read once. With S = 8 the call
 * makes the two launches. Workspace: as aaac_refine_batch.
 * Errors: as aaac_assign_batch and aaac_refine_batch.
 */
aaac_status aaac_assign_refine_batch(int count, const uint16_t* const* W, const int64_t* R,
                                     const int64_t* C, int g, int S, int n,
                                     const float* const* I, float* const* tables,
                                     uint8_t* const* codes, uint8_t* const* sel, int flags,
                                     double* err, double* w2, void* ws, size_t ws_bytes,
                                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AAAC_H */
