/*
 * nf4.h -- C ABI of the MI355X (gfx950) fused NF4 dequantise-and-multiply
 * library (libnf4.so).
 *
 * What it computes.  Frozen linear layers stored as NF4: a weight W [N, K]
 * (the F.linear [out, in] layout) is kept as packed 4-bit indices into a
 * 16-entry code, one scale per block of 64 consecutive elements, and
 * optionally those scales again quantised to 8 bits in groups of 256 with a
 * mean offset ("double quantisation").  bitsandbytes issue #2034 ("MatMul4Bit
 * keeps B and quant_state on ctx instead of save_for_backward ...") shows the
 * interface this mirrors: quantize_4bit(w, blocksize=64, quant_type="nf4",
 * compress_statistics=True) and matmul_4bit(h, w.t(), quant_state=st) in
 * section "Minimal reproducer", and the QuantState tensor fields (absmax,
 * nested_absmax, nested_offset, code) in sections "Root cause" and "Why
 * save_for_backward fixes it".  Soup issue #842 ("Layer streaming: a
 * checkpoint-visible fused NF4 dequantise-and-multiply"), "Design sketch",
 * asks for every one of those fields to be an explicit tensor so an autograd
 * wrapper can route them through save_for_backward, for a backward that
 * computes only grad_x = grad_y @ W with no dense W materialised, and for a
 * deterministic reduction (no atomics, no non-deterministic split-K).
 *
 * Encoding (identical in the CPU checker):
 *   - elements are taken flattened row-major; element 2i sits in the HIGH
 *     nibble of byte i;
 *   - block b covers elements [64b, 64b + 64); absmax[b] = max |w|;
 *   - index q = number of fp32 midpoints of adjacent codes strictly below
 *     t = fp32(w / absmax[b]) (t = 0 for an all-zero block);
 *   - nested form: offset = fp32 of the fp64 mean of absmax (sequential
 *     sums over consecutive chunks of 256, then over the chunk sums);
 *     c = fp32(absmax - offset); per group g of 256 blocks s2[g] = max |c|,
 *     absmax is replaced by the u8 index of fp32(c / s2) in nested_code by the
 *     same midpoint rule;
 *   - decode: absmax_hat = fp32(fp32(nested_code[q2] * s2[b / 256]) + offset)
 *     (nested) or absmax[b]; w_hat = bf16_rne(fp32(code[q] * absmax_hat)).
 *
 * Conventions shared by every call.
 *   Memory     Every pointer argument is DEVICE memory allocated and owned by
 *              the caller, except where a comment says otherwise.  The
 *              library never allocates, frees or retains a pointer after the
 *              call returns.
 *   Streams    `stream` is a hipStream_t passed as void* (NULL = the null
 *              stream).  Work is enqueued asynchronously; no call
 *              synchronises the device or the stream.
 *   Layout     All tensors are dense row-major.  bf16 tensors are 16-bit
 *              bfloat16 bit patterns.  x, y, grad_y, grad_x and packed must be
 *              16-byte aligned.
 *   W-args     (packed, absmax, nested_absmax, nested_offset, code16,
 *              nested_code256, N, K):
 *                packed         u8[N*K/2]
 *                absmax         f32[nb] when nested_absmax == NULL, else u8[nb]
 *                               (nb = ceil(N*K/64))
 *                nested_absmax  f32[ng] (ng = ceil(nb/256)) or NULL
 *                nested_offset  f32[1]; required iff nested_absmax != NULL
 *                code16         f32[16], ascending
 *                nested_code256 f32[256], ascending; required iff nested
 *   Errors     Every call that can fail returns an int status: NF4_OK or a
 *              negative NF4_ERR_* code.  On error nothing is enqueued and no
 *              output is touched.  nf4_status_str() names each code.  No C++
 *              exception crosses this interface.
 *   Empty      M == 0 (or N*K == 0 for the codec) returns NF4_OK with no work.
 *              A product whose contraction is empty (forward K == 0, input
 *              gradient N == 0) writes zeros with a fill kernel (never a
 *              memset, so the call can be captured into a HIP graph).  An
 *              operand with no elements may be NULL (as torch gives for empty
 *              tensors).
 *   Determinism  Every kernel sums in a fixed order and uses no atomics; the
 *              tile and the split of a contraction across workgroups are a
 *              pure function of (M, N, K, compute-unit count), for the grouped
 *              calls of (total_M, E, N, K), and of the NF4_BM, NF4_BN,
 *              NF4_CONSUMERS, NF4_SPLITS, NF4_SMALL_M and NF4_GEMV_* tuning
 *              variables when they are set (read on every call; a different
 *              tile may round differently in the last bit).  Repeated calls
 *              with the same inputs and environment give bitwise identical
 *              outputs.
 */
#ifndef NF4_H_
#define NF4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define NF4_OK                0
#define NF4_ERR_NULL         -1  /* a required pointer is NULL                     */
#define NF4_ERR_SHAPE        -2  /* negative size, odd N*K, E < 1, ...             */
#define NF4_ERR_UNSUPPORTED  -3  /* e.g. K % 64 != 0 for a matmul                   */
#define NF4_ERR_ALIGN        -4  /* a pointer that must be 16-byte aligned is not  */
#define NF4_ERR_WORKSPACE    -5  /* workspace missing or smaller than required     */
#define NF4_ERR_HIP          -6  /* the HIP runtime reported an error on launch    */
#define NF4_ERR_DTYPE        -7  /* unknown dtype selector                          */
#define NF4_ERR_SCRATCH      -8  /* needs more scratch than the fixed buffer holds  */

/* ---- dtype selectors ---------------------------------------------------- */
#define NF4_DTYPE_F32  0
#define NF4_DTYPE_BF16 1

/* ---- op selectors for nf4_workspace_bytes -------------------------------- */
#define NF4_OP_QUANTIZE          0
#define NF4_OP_MATMUL_FWD        1
#define NF4_OP_MATMUL_BWD_INPUT  2
#define NF4_OP_GROUPED_FWD       3
#define NF4_OP_GROUPED_BWD_INPUT 4
#define NF4_OP_MATMUL_FWD_8BIT        5
#define NF4_OP_MATMUL_BWD_INPUT_8BIT  6

/* ---- path counters (host-side launch counts; they prove which kernel ran,
 *      as the "Acceptance criteria" of Soup issue #842 ask) ---------------- */
#define NF4_PATH_QUANTIZE       0  /* codec: quantise                           */
#define NF4_PATH_DEQUANTIZE     1  /* codec: dequantise                         */
#define NF4_PATH_FWD_TILED      2  /* fused forward, MFMA tiles                 */
#define NF4_PATH_FWD_SMALL_M    3  /* fused forward, weight-streaming small M   */
#define NF4_PATH_BWD_TILED      4  /* fused input gradient, MFMA tiles          */
#define NF4_PATH_SPLITK_REDUCE  5  /* fixed-order reduction of split partials   */
#define NF4_PATH_GROUPED_FWD    6  /* grouped (expert) forward                  */
#define NF4_PATH_GROUPED_BWD    7  /* grouped (expert) input gradient           */
#define NF4_PATH_FWD_8BIT       8  /* 8-bit blockwise forward (plain or grouped) */
#define NF4_PATH_BWD_8BIT       9  /* 8-bit blockwise input gradient            */
#define NF4_PATH_COUNT         10

/*
 * nf4_quantize -- NF4 blockwise quantisation of w [N, K] (bitsandbytes #2034,
 * "Minimal reproducer": quantize_4bit(w, blocksize=64, quant_type="nf4",
 * compress_statistics=...)).
 *   w             device, f32 or bf16 per w_dtype, N*K elements (N*K even)
 *   nested_code256  NULL: plain form, absmax is written as f32[nb];
 *                 non-NULL: nested form, absmax is written as u8[nb] and
 *                 nested_absmax f32[ng], nested_offset f32[1] are written.
 *   ws, ws_bytes  device scratch of at least
 *                 nf4_workspace_bytes(NF4_OP_QUANTIZE, 0, N, K, 1) bytes
 *                 (0 for the plain form; ws may then be NULL).
 * Output bytes are identical to the CPU checker's.
 */
int nf4_quantize(const void* w, int w_dtype, int64_t N, int64_t K,
                 const float* code16, const float* nested_code256,
                 uint8_t* packed, void* absmax, float* nested_absmax,
                 float* nested_offset, void* ws, size_t ws_bytes, void* stream);

/*
 * nf4_dequantize -- the dense weight in the compute dtype from packed data
 * and the statistics (bitsandbytes #2034 "Root cause": dequantize_4bit(B,
 * state)).  out is bf16[N*K] (bf16_rne of fp32(code[q]*absmax_hat)) or
 * f32[N*K] (fp32(code[q]*absmax_hat)) per out_dtype.  Bit-exact.
 */
int nf4_dequantize(const uint8_t* packed, const void* absmax,
                   const float* nested_absmax, const float* nested_offset,
                   const float* code16, const float* nested_code256,
                   int64_t N, int64_t K, int out_dtype, void* out, void* stream);

/*
 * nf4_matmul_fwd -- y = x . W_hat^T without materialising W_hat
 * (bitsandbytes #2034 "Minimal reproducer": matmul_4bit(h, w.t()) ==
 * F.linear(h, W_hat)).
 *   x  bf16 [M, K];  y  bf16 [M, N];  fp32 accumulation, bf16 RNE output.
 *   Requires K % 64 == 0.  ws: nf4_workspace_bytes(NF4_OP_MATMUL_FWD, M, N, K, 1)
 *   bytes (may be 0 and ws NULL).
 */
int nf4_matmul_fwd(const void* x, int64_t M,
                   const uint8_t* packed, const void* absmax,
                   const float* nested_absmax, const float* nested_offset,
                   const float* code16, const float* nested_code256,
                   int64_t N, int64_t K, void* y, void* ws, size_t ws_bytes,
                   void* stream);

/*
 * nf4_matmul_bwd_input -- grad_x = grad_y . W_hat from the same packed layout
 * (Soup #842 "Design sketch": the backward computes only grad_x = grad_y @ W
 * with a transposed fused kernel; no weight gradient, the base is frozen).
 *   grad_y bf16 [M, N];  grad_x bf16 [M, K].
 *   Requires K % 64 == 0 and N % 8 == 0.  ws as for the forward with
 *   NF4_OP_MATMUL_BWD_INPUT.
 */
int nf4_matmul_bwd_input(const void* grad_y, int64_t M,
                         const uint8_t* packed, const void* absmax,
                         const float* nested_absmax, const float* nested_offset,
                         const float* code16, const float* nested_code256,
                         int64_t N, int64_t K, void* grad_x, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * nf4_grouped_matmul_fwd -- per-expert forward over expert-sorted rows
 * (bitsandbytes fork PR "Experts trainability ...", "Commit 2": each expert
 * projection is dequantise + F.linear on that expert's slice of the stack).
 *   x        bf16 [total_M, K], rows sorted by expert
 *   offsets  device int32 [E + 1]: rows offsets[e] .. offsets[e+1]-1 belong
 *            to expert e; must be non-decreasing from 0 to total_M.  Each
 *            entry is clamped to [0, total_M] on the device, so a malformed
 *            array cannot cause out-of-range accesses (its rows' results are
 *            then unspecified).
 *   W-args   the expert stack [E, N, K] quantised as ONE tensor of E*N rows;
 *            N, K are per-expert.  Requires K % 64 == 0.
 *   y        bf16 [total_M, N]
 * Routing, gather and scatter stay with the caller.
 */
int nf4_grouped_matmul_fwd(const void* x, const int32_t* offsets, int32_t E,
                           int64_t total_M,
                           const uint8_t* packed, const void* absmax,
                           const float* nested_absmax, const float* nested_offset,
                           const float* code16, const float* nested_code256,
                           int64_t N, int64_t K, void* y, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * nf4_grouped_matmul_bwd_input -- grad_x[rows of e] = grad_y[rows of e] .
 * W_hat_e (the same "Commit 2" backward: grad_output @ W on the expert
 * slice).  grad_y bf16 [total_M, N], grad_x bf16 [total_M, K].
 * Requires K % 64 == 0 and N % 8 == 0.
 */
int nf4_grouped_matmul_bwd_input(const void* grad_y, const int32_t* offsets,
                                 int32_t E, int64_t total_M,
                                 const uint8_t* packed, const void* absmax,
                                 const float* nested_absmax,
                                 const float* nested_offset,
                                 const float* code16, const float* nested_code256,
                                 int64_t N, int64_t K, void* grad_x, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * ---- 8-bit blockwise variants --------------------------------------------
 * bitsandbytes fork PR "Experts trainability: bit-exact recompute-in-backward
 * + ExpertsNbit", "Commit 1": its quant_type table lists 8-bit blockwise
 * formats (int8 with a dynamic map, fp8 e4m3 with its codebook) beside nf4
 * and fp4.  Same blocks of 64, same plain or nested absmax, but one byte per
 * weight: the byte is an index into an ascending 256-entry fp32 table
 * `code256` passed in (the pages define neither map; any ascending table
 * works, for example the integers -128..127 over 127 or the e4m3 values over
 * their largest).  Encoding: index = number of table midpoints strictly
 * below t = fp32(w / absmax) (the 4-bit rule with 255 midpoints); decode
 * w_hat = bf16_rne(fp32(code256[q] * absmax_hat)).
 * W8-args: (packed u8[N*K], absmax, nested_absmax, nested_offset, code256,
 * nested_code256, N, K); the statistics fields are as for the 4-bit form.
 * Conventions (memory, streams, errors, determinism) as above.  The matmuls
 * run their own fused kernel (path counters NF4_PATH_FWD_8BIT /
 * NF4_PATH_BWD_8BIT), workspace from NF4_OP_MATMUL_FWD_8BIT /
 * NF4_OP_MATMUL_BWD_INPUT_8BIT; the grouped calls need none.
 */
int nf4_quantize_8bit(const void* w, int w_dtype, int64_t N, int64_t K,
                      const float* code256, const float* nested_code256,
                      uint8_t* packed, void* absmax, float* nested_absmax,
                      float* nested_offset, void* ws, size_t ws_bytes, void* stream);
int nf4_dequantize_8bit(const uint8_t* packed, const void* absmax,
                        const float* nested_absmax, const float* nested_offset,
                        const float* code256, const float* nested_code256,
                        int64_t N, int64_t K, int out_dtype, void* out, void* stream);
int nf4_matmul_fwd_8bit(const void* x, int64_t M,
                        const uint8_t* packed, const void* absmax,
                        const float* nested_absmax, const float* nested_offset,
                        const float* code256, const float* nested_code256,
                        int64_t N, int64_t K, void* y, void* ws, size_t ws_bytes,
                        void* stream);
int nf4_matmul_bwd_input_8bit(const void* grad_y, int64_t M,
                              const uint8_t* packed, const void* absmax,
                              const float* nested_absmax, const float* nested_offset,
                              const float* code256, const float* nested_code256,
                              int64_t N, int64_t K, void* grad_x, void* ws,
                              size_t ws_bytes, void* stream);
int nf4_grouped_matmul_fwd_8bit(const void* x, const int32_t* offsets, int32_t E,
                                int64_t total_M,
                                const uint8_t* packed, const void* absmax,
                                const float* nested_absmax, const float* nested_offset,
                                const float* code256, const float* nested_code256,
                                int64_t N, int64_t K, void* y, void* ws,
                                size_t ws_bytes, void* stream);
int nf4_grouped_matmul_bwd_input_8bit(const void* grad_y, const int32_t* offsets,
                                      int32_t E, int64_t total_M,
                                      const uint8_t* packed, const void* absmax,
                                      const float* nested_absmax,
                                      const float* nested_offset,
                                      const float* code256, const float* nested_code256,
                                      int64_t N, int64_t K, void* grad_x, void* ws,
                                      size_t ws_bytes, void* stream);

/*
 * nf4_matmul_fwd_noalloc -- nf4_matmul_fwd without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.
 *   Same arguments, result and kernels as nf4_matmul_fwd (bitwise identical
 *   output), minus ws / ws_bytes.  The split-contraction partials go to a
 *   fixed device array of NF4_NOALLOC_SCRATCH_BYTES inside the library; each
 *   GPU the library runs on holds its own copy until the process ends.  Its
 *   address is looked up once per device (with hipGetSymbolAddress) on the
 *   first call made while that device is current; the call runs on the
 *   current device, and `stream` must belong to it.
 *   Allocates nothing: no hipMalloc, hipFree or allocating library routine.
 *   A product whose plan needs more than NF4_NOALLOC_SCRATCH_BYTES of
 *   partials (nf4_workspace_bytes(NF4_OP_MATMUL_FWD, ...) larger than it)
 *   returns NF4_ERR_SCRATCH and enqueues nothing.
 *   All calls on one GPU share its array, and every partial is written
 *   before it is read, so nothing needs clearing between calls; two calls
 *   that overlap on one GPU (different streams, no ordering) race on it.
 */
#define NF4_NOALLOC_SCRATCH_BYTES (64u << 20)

int nf4_matmul_fwd_noalloc(const void* x, int64_t M,
                           const uint8_t* packed, const void* absmax,
                           const float* nested_absmax, const float* nested_offset,
                           const float* code16, const float* nested_code256,
                           int64_t N, int64_t K, void* y, void* stream);

/* ---- host-only helpers (no device work) --------------------------------- */

/* Workspace bytes the call `op` needs for these sizes on the current device
 * (a pure function of the sizes and the device's compute-unit count).  Returns
 * 0 when no workspace is needed, SIZE_MAX for invalid sizes. */
size_t nf4_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int32_t E);

/* Storage sizes of one quantised N x K tensor (negative on invalid sizes). */
int64_t nf4_packed_bytes(int64_t N, int64_t K);   /* N*K/2             */
int64_t nf4_absmax_count(int64_t N, int64_t K);   /* ceil(N*K/64)      */
int64_t nf4_nested_count(int64_t N, int64_t K);   /* ceil(nb/256)      */

/* Launch counters per NF4_PATH_* (process-wide, thread-safe). Returns -1 for
 * an unknown path id. */
int64_t nf4_path_count(int path);
void nf4_reset_path_counts(void);

/* Static description of a status code; never NULL. */
const char* nf4_status_str(int status);

/* Library version string; never NULL. */
const char* nf4_version(void);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* NF4_H_ */
