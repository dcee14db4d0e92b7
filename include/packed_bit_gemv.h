/*
 * packed_bit_gemv.h - C ABI of libpackedbitgemv.so, the MI355X (gfx950)
 * decode-time matrix-vector kernels for bit-packed ternary weights and for an
 * int8 output head.
 *
 * What is computed (Neutrino-1 8B model page, English text on bittide):
 *   - every transformer linear is stored as ternary codes c in {-1, 0, +1}
 *     with a scale and a row sum per row; the kernels read the packed codes
 *     and decode them in registers, so no fp16/fp32 copy of a weight matrix
 *     exists anywhere (introduction; "Where the bytes live"; "Inside the
 *     coded lane");
 *   - the untied output head is an int8 tensor with a per-row scale
 *     ("Where the bytes live");
 *   - a speculative verify step puts several drafted positions through the
 *     same weights together ("speculative" section): the same products for
 *     M <= 8 activation rows.
 *
 * Packed layout (this library's own; the page calls its format proprietary):
 *   - 2 bits per code, 16 codes per little-endian uint32 word;
 *   - code j (0..15) of a word: pair t = j / 2, half h = j % 2;
 *       nonzero bit at 16*h + 14 - 2*t,
 *       sign bit    at 16*h + 15 - 2*t;
 *     so each 16-bit half holds 8 two-bit fields, highest first (even codes
 *     in the low half, odd codes in the high half), and a field read as a
 *     2-bit two's-complement integer is the code: +1 = 01, -1 = 11, 0 = 00;
 *     10 never occurs. Shifting a word left by 2t and masking with
 *     0xC000C000 leaves two IEEE fp16 values equal to 2*c[2t], 2*c[2t+1].
 *   - row r of an N x K matrix is pbg_words_per_row(K) = 4 * ceil(K / 64)
 *     consecutive words (a whole number of 16-byte chunks); word w holds the
 *     codes of columns 16w .. 16w+15; codes past column K-1 are 0.
 *   - per row: an fp32 scale s_r and an int32 row sum sum_j c_rj.
 *
 * Conventions for every entry point:
 *   - all array pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them. Its only global state is a
 *     per-device cache of the compute-unit count (read once, atomically), so
 *     calls from several threads are safe;
 *   - work is enqueued on the caller's `stream` (0 = the null stream) and
 *     the call returns without waiting, except where stated;
 *   - arguments are validated before any HIP call; on a validation error
 *     nothing is enqueued and a negative PBG_ERR_* code is returned;
 *   - a HIP error that earlier work left pending on the calling thread
 *     (hipPeekAtLastError) belongs to the caller: the call enqueues nothing,
 *     leaves that error in place and returns PBG_ERR_HIP (hipErrorNotReady,
 *     a completion status, is not treated as an error);
 *   - outputs must not overlap inputs;
 *   - activations x are IEEE fp16 bit patterns (uint16_t), row-major [m][k];
 *     they must be finite (the result for Inf or NaN activations is not
 *     specified; the kernels form 0 * x_j for a zero code);
 *   - outputs y are fp32, row-major [m][n]; accumulation is fp32 in an
 *     unspecified order (any order meets |y - y_exact| <= 1e-3 * s_r *
 *     sum_j |x_j| for K below about 16,000).
 */
#ifndef PACKED_BIT_GEMV_H
#define PACKED_BIT_GEMV_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PBG_ABI_VERSION 2

/* Return codes. */
#define PBG_OK 0
#define PBG_ERR_NULL (-1)    /* a required pointer is NULL */
#define PBG_ERR_SHAPE (-2)   /* n, k or m out of range */
#define PBG_ERR_ALIGN (-3)   /* a pointer lacks its required alignment */
#define PBG_ERR_CODE (-4)    /* pack input held a value outside {-1, 0, +1} */
#define PBG_ERR_HIP (-5)     /* a HIP launch or copy failed */
#define PBG_ERR_WORKSPACE (-6) /* a workspace is smaller than the call needs */

/* Limits: 1 <= n <= PBG_MAX_N, 1 <= k <= PBG_MAX_K, 1 <= m <= PBG_MAX_M. */
#define PBG_MAX_N 16777216LL
#define PBG_MAX_K 16777216LL
#define PBG_MAX_M 8

/* Version of this ABI (PBG_ABI_VERSION of the built library). */
int pbg_abi_version(void);

/* Static message for a return code; never NULL. */
const char* pbg_strerror(int code);

/* Words per packed row for k columns: 4 * ceil(k / 64); 0 if k <= 0. */
int64_t pbg_words_per_row(int64_t k);

/*
 * pack_ternary - load-time encoding of one coded linear.
 * Source: Neutrino-1 8B model page, "Where the bytes live" (ternary codes with
 * per-row scales and row sums) and "Inside the coded lane" (code occupancy).
 *
 *   codes    [n][k] int8, row-major, values -1, 0, +1 (any alignment)
 *   packed   [n][pbg_words_per_row(k)] uint32 out, 16-byte aligned
 *   row_sum  [n] int32 out: sum_j codes[r][j] over valid codes
 *   stats    [4] int64 out, device, 8-byte aligned: n_minus, n_zero, n_plus,
 *            n_invalid over the whole tensor (zeroed by this call)
 *   stats_host  NULL, or a host array of 4 int64: then the call waits for the
 *            stream, copies stats there and returns PBG_ERR_CODE if
 *            n_invalid > 0
 * An invalid code is counted and packed as 0 and adds nothing to row_sum.
 */
int pack_ternary(const int8_t* codes, int64_t n, int64_t k, uint32_t* packed, int32_t* row_sum,
                 int64_t* stats, int64_t* stats_host, hipStream_t stream);

/*
 * ternary_gemv - y[r] = scale[r] * sum_j c[r][j] * x[j], one activation row.
 * Source: Neutrino-1 8B model page, introduction (the kernels expand the
 * codes; decode speed is set by the weight bytes read per token) and "Where the bytes
 * live" (per-row scale).
 *
 *   packed  [n][pbg_words_per_row(k)] uint32, 16-byte aligned
 *   scale   [n] fp32, 4-byte aligned
 *   x       [k] fp16 bits, 2-byte aligned
 *   y       [n] fp32 out, 4-byte aligned
 */
int ternary_gemv(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                 float* y, hipStream_t stream);

/*
 * ternary_gemm_small - Y[i][r] = scale[r] * sum_j c[r][j] * X[i][j] for
 * 1 <= m <= 8 activation rows, reading each weight word once.
 * Source: Neutrino-1 8B model page, "speculative" section (the 8B scores a
 * drafted run of up to six tokens plus one in a single forward pass).
 *
 *   packed, scale  as ternary_gemv
 *   x       [m][k] fp16 bits, 2-byte aligned
 *   y       [m][n] fp32 out, 4-byte aligned
 */
int ternary_gemm_small(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                       int64_t m, float* y, hipStream_t stream);

/*
 * ternary_gemm_splitk - ternary_gemm_small (1 <= m <= 8 activation rows) with
 * the K columns also split across workgroups, for matrices whose few rows or
 * long rows would leave the plain kernels short of workgroups or re-reading
 * all of x per row block (a 1,024 x 12,288 shard of the down projection, the
 * full 4,096 x 12,288 one at m = 8). Each slice of a row block adds its
 * partial sums into one 64-bit integer per output in the workspace (exact
 * fixed point with 23 fractional bits; the low 4 bits count arrivals); the
 * slice that completes an output writes it and sets the integer back to
 * zero. No workgroup waits for another, and the result is the exact sum of
 * the slices' fp32 partials rounded once, whatever order they arrive in, so
 * it is bitwise repeatable (its summation order differs from
 * ternary_gemm_small's).
 * Source: Neutrino-1 8B model page, introduction (decode speed is set by the
 * bytes a step moves), geometry table (feed-forward width 12,288) and
 * "speculative" section (several drafted positions in one pass).
 *
 *   packed, scale, n, k, x, m, y  as ternary_gemm_small; activations must
 *              be finite with |x| <= 65,504 (any finite fp16)
 *   workspace  device, 256-byte aligned, owned by the caller, at least
 *              pbg_splitk_workspace_bytes(n, k) bytes (enough for every m),
 *              all zero before its first use (e.g. one zero fill at
 *              allocation); every call leaves it all zero again. Calls that
 *              overlap in time need separate workspaces.
 *   workspace_bytes  its size; PBG_ERR_WORKSPACE if too small
 * The split runs where it measured faster on MI355X: m >= 2 with
 * 4,096 < k <= 16,384, k % 8 == 0, x 16-byte aligned, and n <= 2,048, or
 * n <= 4,096 with k <= 12,288 and m >= 5. Other calls run ternary_gemm_small's
 * kernels and leave the workspace untouched.
 */
int64_t pbg_splitk_workspace_bytes(int64_t n, int64_t k);

int ternary_gemm_splitk(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                        int64_t m, float* y, void* workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * The 3-bit variant: five-level codes c in {-2, -1, 0, +1, +2}, 3 bits per
 * code, the size of the shipped coded lane.
 * Source: Neutrino-1 8B model page, "Where the bytes live" (the coded lane
 * is 72,351,744 bytes per layer, exactly 3 bits per coded weight) and
 * "Inside the coded lane" (codes split into zero, plus and minus). The page
 * does not say what the third bit means; this library reads it as a
 * magnitude (|c| = 2) and fixes its own layout:
 *   - a row of k codes is padded with zero codes to K128 = 128 * ceil(k/128)
 *     and holds pbg_words_per_row3(k) = 12 * ceil(k / 128) words;
 *   - words [0, K128 / 16): the sign/nonzero plane, exactly the 2-bit layout
 *     above for sign(c) (a code of magnitude 2 is written like one of 1);
 *   - words [K128 / 16, 3 * K128 / 32): the magnitude plane; magnitude word q
 *     holds codes 32q .. 32q + 31, code 32q + j with j = 16i + 2t + h
 *     (i = 0, 1; t = 0..7; h = 0, 1) at bit 16h + 8i + t, set iff |c| = 2;
 *     a magnitude bit is never set without its nonzero bit.
 *   - per row: an fp32 scale and an int32 row sum sum_j c_rj.
 */
int64_t pbg_words_per_row3(int64_t k);

/*
 * pack_ternary3 - load-time encoding of one five-level linear; as
 * pack_ternary, with
 *   codes    [n][k] int8, values -2..+2 (any alignment)
 *   packed   [n][pbg_words_per_row3(k)] uint32 out, 16-byte aligned
 *   stats    [6] int64 out, device, 8-byte aligned: counts of -2, -1, 0, +1,
 *            +2 and of invalid codes (zeroed by this call)
 *   stats_host  NULL, or a host array of 6 int64 (then the call waits and
 *            returns PBG_ERR_CODE if any code was invalid)
 * An invalid code is counted and packed as 0 and adds nothing to row_sum.
 */
int pack_ternary3(const int8_t* codes, int64_t n, int64_t k, uint32_t* packed, int32_t* row_sum,
                  int64_t* stats, int64_t* stats_host, hipStream_t stream);

/*
 * ternary3_gemv / ternary3_gemm_small - ternary_gemv and ternary_gemm_small
 * for five-level packs: y[r] = scale[r] * sum_j c[r][j] * x[j] (m = 1), or
 * Y[i][r] for 1 <= m <= 8 activation rows, each weight word read once.
 *   packed  [n][pbg_words_per_row3(k)] uint32, 16-byte aligned
 *   scale, x, y, m as the 2-bit calls
 */
int ternary3_gemv(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x, float* y,
                  hipStream_t stream);

int ternary3_gemm_small(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                        int64_t m, float* y, hipStream_t stream);

/*
 * int8_head_gemv - Y[i][v] = scale[v] * sum_j w[v][j] * X[i][j] for the int8
 * output head, 1 <= m <= 8 activation rows.
 * Source: Neutrino-1 8B model page, "Where the bytes live" (untied int8
 * output head of 151,936 x 4,096, a scale per row).
 *
 *   w       [n][k] int8, row-major, 16-byte aligned
 *   scale   [n] fp32, 4-byte aligned
 *   x       [m][k] fp16 bits, 2-byte aligned
 *   y       [m][n] fp32 out, 4-byte aligned
 */
int int8_head_gemv(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, int64_t m,
                   float* y, hipStream_t stream);

/*
 * int8_head_argmax - greedy token of each activation row through the int8
 * head without writing the logits: token[i] = argmax_v Y[i][v] with Y as in
 * int8_head_gemv, the lowest v among equal maxima; logit[i] = Y[i][token[i]].
 * Source: Neutrino-1 8B model page, "speculative" section (acceptance of a
 * drafted token compares it with the large model's greedy choice, so the
 * verify step needs only this index per row) and "Where the bytes live"
 * (int8 head).
 *
 *   w, scale, x, m  as int8_head_gemv (1 <= m <= 8); logits must be finite
 *   keys    [m * PBG_ARGMAX_KEYS_PER_ROW] uint64 device workspace, 8-byte
 *           aligned, owned by the caller and all zero before the first call
 *           (e.g. one zero fill at allocation). Partial maxima of a row sit
 *           in separate 128-byte lines so that workgroups do not queue on one
 *           address; the call leaves the entries it used at zero again, so
 *           the workspace stays ready. Calls that overlap in time need
 *           separate workspaces.
 *   token   [m] int32 out, 4-byte aligned
 *   logit   [m] fp32 out, 4-byte aligned, or NULL
 * The result does not depend on the order in which workgroups finish.
 */
#define PBG_ARGMAX_KEYS_PER_ROW 4096

int int8_head_argmax(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, int64_t m,
                     uint64_t* keys, int32_t* token, float* logit, hipStream_t stream);

/*
 * int8_head_argmax_noalloc - int8_head_argmax for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid allocation): the same computation and results, with
 * the keys workspace replaced by a device array the library owns.
 *
 *   w, scale, n, k, x, m, token, logit  as int8_head_argmax
 *   1 <= m <= PBG_MAX_M; a larger m returns PBG_ERR_SHAPE
 * The array holds the keys of PBG_MAX_M rows (PBG_NOALLOC_SCRATCH_BYTES =
 * 256 KiB) on every GPU the library runs on and is kept until the process
 * ends. It starts zeroed and every call leaves it zero again. The call
 * allocates and frees nothing. All calls on one GPU share the array: calls
 * that overlap in time (other streams, other threads) race and their tokens
 * are then unspecified; calls ordered on one stream are safe.
 */
#define PBG_NOALLOC_SCRATCH_BYTES (PBG_MAX_M * PBG_ARGMAX_KEYS_PER_ROW * 8)

int int8_head_argmax_noalloc(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                             int64_t m, int32_t* token, float* logit, hipStream_t stream);

/*
 * int8_embedding_gather - out[i][j] = scale[t] * table[t][j] with t =
 * tokens[i], formed exactly and rounded once to fp32.
 * Source: Neutrino-1 8B model page, "Where the bytes live" (untied int8 input
 * embedding, a scale per row, one row read per token).
 *
 *   table   [n][k] int8, row-major (any alignment)
 *   scale   [n] fp32, 4-byte aligned
 *   tokens  [m] int32 device, 4-byte aligned; ids outside [0, n) give a row
 *           of NaN
 *   out     [m][k] fp32 out, 4-byte aligned
 *   1 <= m; m * ceil(k / 1024) <= 2^23
 */
int int8_embedding_gather(const int8_t* table, const float* scale, int64_t n, int64_t k, const int32_t* tokens,
                          int64_t m, float* out, hipStream_t stream);

/* Largest d_model of ternary_ffn_swiglu (one 4,096-column slice per row). */
#define PBG_FFN_MAX_MODEL 4096

/*
 * ternary_swiglu_gate_up - the first half of ternary_ffn_swiglu on its own:
 * h[j] = fp16(silu(g[j]) * u[j]) with g = gate x and u = up x, in one launch
 * that reads gate and up together; g and u never reach memory.
 * Source: as ternary_ffn_swiglu. Arguments, layouts, alignment and limits
 * are those of ternary_ffn_swiglu.
 */
int ternary_swiglu_gate_up(const uint32_t* gate_packed, const float* gate_scale, const uint32_t* up_packed,
                           const float* up_scale, int64_t d_model, int64_t d_ff, const uint16_t* x, uint16_t* h,
                           hipStream_t stream);

/*
 * ternary_ffn_swiglu - the gated feed-forward block of one layer for one
 * activation row:
 *   g = gate x, u = up x              (ternary linears, d_ff x d_model)
 *   h[j] = fp16(silu(g[j]) * u[j])    (silu(z) = z / (1 + exp(-z)); rounded
 *                                      to nearest even, overflow to +-inf)
 *   y = down h                        (ternary linear, d_model x d_ff)
 * Source: Neutrino-1 8B model page, geometry table (feed-forward gated by
 * SwiGLU, three linears per layer; widths 4,096 and 12,288) and "Where the
 * bytes live" (per-row scales). The page does not write the gate out; silu
 * on the gate output times the up output is the usual SwiGLU.
 * Two launches on `stream`: ternary_swiglu_gate_up (gate and up together,
 * SwiGLU in the epilogue), then ternary_gemv of down on h.
 *
 *   gate_packed, up_packed  [d_ff][pbg_words_per_row(d_model)] uint32, 16-byte
 *                           aligned; gate_scale, up_scale [d_ff] fp32
 *   down_packed             [d_model][pbg_words_per_row(d_ff)] uint32, 16-byte
 *                           aligned; down_scale [d_model] fp32
 *   x        [d_model] fp16 bits, 16-byte aligned
 *   h        [d_ff] fp16 bits out, 16-byte aligned: the down linear's input
 *   y        [d_model] fp32 out
 *   8 <= d_model <= PBG_FFN_MAX_MODEL with d_model % 8 == 0;
 *   1 <= d_ff <= PBG_MAX_N.
 */
int ternary_ffn_swiglu(const uint32_t* gate_packed, const float* gate_scale, const uint32_t* up_packed,
                       const float* up_scale, const uint32_t* down_packed, const float* down_scale, int64_t d_model,
                       int64_t d_ff, const uint16_t* x, uint16_t* h, float* y, hipStream_t stream);

/*
 * ternary_swiglu_gate_up_small / ternary_ffn_swiglu_small - the two calls
 * above for 1 <= m <= PBG_MAX_M activation rows, the shape a speculative
 * verify step scores (Neutrino-1 8B model page, "speculative" section): every
 * weight byte is read once for all m rows.
 *   x     fp16 [m][d_model], 16-byte aligned
 *   h     out, fp16 [m][d_ff], row i = fp16(silu(g_i) * u_i) with g_i, u_i the
 *         gate and up outputs of x row i; 16-byte aligned
 *   y     out (ffn only), fp32 [m][d_model], y_i = down h_i, 4-byte aligned
 * d_model, d_ff, the packs and scales are as for the m = 1 calls (same limits
 * and alignment); m = 1 runs exactly the m = 1 kernels. Returns PBG_ERR_SHAPE
 * for m outside [1, PBG_MAX_M].
 * For 2 <= m with d_ff % 8 == 0 and 4,096 < d_ff <= 12,288, the ffn call
 * splits down over K in two slices that each add their part to y with an
 * fp32 atomic add, after the gate|up launch has set y to +0: y's earlier
 * contents are ignored, and the result is the same bits on every call (two
 * addends onto +0 give one result in either order). y must be device memory
 * of this GPU (device-scope atomics) and must not overlap h, x or the
 * weights.
 */
int ternary_swiglu_gate_up_small(const uint32_t* gate_packed, const float* gate_scale, const uint32_t* up_packed,
                                 const float* up_scale, int64_t d_model, int64_t d_ff, const uint16_t* x, int64_t m,
                                 uint16_t* h, hipStream_t stream);

int ternary_ffn_swiglu_small(const uint32_t* gate_packed, const float* gate_scale, const uint32_t* up_packed,
                             const float* up_scale, const uint32_t* down_packed, const float* down_scale,
                             int64_t d_model, int64_t d_ff, const uint16_t* x, int64_t m, uint16_t* h, float* y,
                             hipStream_t stream);

/*
 * ternary3_swiglu_gate_up, ternary3_ffn_swiglu, ternary3_swiglu_gate_up_small,
 * ternary3_ffn_swiglu_small - the four SwiGLU feed-forward calls above with
 * the three linears in the 3-bit layout (five-level codes, see
 * ternary3_gemv): the same h = fp16(silu(gate x) * up x) and y = down h, one
 * launch for gate and up together, then ternary3_gemv (m = 1) or
 * ternary3_gemm_small (m rows) of down on h.
 * Source: Neutrino-1 8B model page, geometry table (gated SwiGLU block, three
 * linears) and "Where the bytes live" (the coded lane at 3 bits per weight,
 * per-row scales).
 *
 *   gate_packed, up_packed  [d_ff][pbg_words_per_row3(d_model)] uint32,
 *                           16-byte aligned
 *   down_packed             [d_model][pbg_words_per_row3(d_ff)] uint32,
 *                           16-byte aligned
 * Everything else (scales, x, h, y, m, limits, alignment, return codes, and
 * the two K-slices of down added onto a cleared y for 2 <= m) is as for the
 * 2-bit calls of the same name without the 3.
 */
int ternary3_swiglu_gate_up(const uint32_t* gate_packed, const float* gate_scale, const uint32_t* up_packed,
                            const float* up_scale, int64_t d_model, int64_t d_ff, const uint16_t* x, uint16_t* h,
                            hipStream_t stream);

int ternary3_ffn_swiglu(const uint32_t* gate_packed, const float* gate_scale, const uint32_t* up_packed,
                        const float* up_scale, const uint32_t* down_packed, const float* down_scale, int64_t d_model,
                        int64_t d_ff, const uint16_t* x, uint16_t* h, float* y, hipStream_t stream);

int ternary3_swiglu_gate_up_small(const uint32_t* gate_packed, const float* gate_scale, const uint32_t* up_packed,
                                  const float* up_scale, int64_t d_model, int64_t d_ff, const uint16_t* x, int64_t m,
                                  uint16_t* h, hipStream_t stream);

int ternary3_ffn_swiglu_small(const uint32_t* gate_packed, const float* gate_scale, const uint32_t* up_packed,
                              const float* up_scale, const uint32_t* down_packed, const float* down_scale,
                              int64_t d_model, int64_t d_ff, const uint16_t* x, int64_t m, uint16_t* h, float* y,
                              hipStream_t stream);

/*
 * pbg_stream_read - measurement helper, not a step of the decode path: reads
 * `bytes` of device memory once with the loads the GEMV kernels use (16-byte
 * non-temporal loads, 1 KiB of consecutive bytes per wave-wide load, up to
 * 4 in flight per lane) and only folds them by XOR. Its duration is the streaming-
 * read ceiling for one launch that moves the same bytes, the reference a
 * GEMV's time is set against.
 * Source: Neutrino-1 8B model page, introduction (single-stream decode speed
 * is set by the bytes moved per token).
 *
 *   src    device, 16-byte aligned; 16 <= bytes <= PBG_STREAM_READ_MAX_BYTES,
 *          bytes % 16 == 0
 *   sink   [PBG_STREAM_READ_SINK_WORDS] uint32 device, 4-byte aligned: the
 *          call XORs into it, so with sink all zero before the call, the XOR
 *          of all its words afterwards is the XOR of all 32-bit words of src
 *          (every byte was read). Calls that overlap in time on one sink
 *          still give the XOR of both ranges.
 */
#define PBG_STREAM_READ_SINK_WORDS 8192
#define PBG_STREAM_READ_MAX_BYTES (1LL << 40)

int pbg_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PACKED_BIT_GEMV_H */
