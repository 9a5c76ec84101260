/*
 * dbf.h -- C ABI of the MI355X (gfx950) double-binary factorized linear layer.
 *
 * The layer (one token x of M features, N outputs, inner rank R, L terms):
 *
 *   y = sum_{i=1..L} diag(alpha_i) B1_i diag(beta_i) B2_i diag(gamma_i) x
 *
 * with sign factors B1_i in {+-1}^{N x R}, B2_i in {+-1}^{R x M} and fp16
 * scale vectors alpha_i (N), beta_i (R), gamma_i (M).  This is the weight
 * update of "LoRDBA: Low-Rank Double-Binary Adaptation" (section 2,
 * "Arquitetura Central", the parametrization of Delta W, with L the envelope
 * rank); with L = 1 it is the double binary factorization of "Addition is
 * almost all you need" (technical summary, section 2:  W ~ (a . A . m^T)
 * (B . b^T) with a = alpha, A = B1, m = beta, B = B2, b = gamma); with L > 1
 * it is the sum of boolean kernels of "Highly Efficient and Effective LLMs
 * with Multi-Boolean Architectures" (technical summary, section 2, item 2),
 * here with a double-binary term per kernel.
 *
 * Conventions shared by every entry point
 *   - Every pointer except `terms` (host array) is device memory owned by the
 *     caller.  The library never allocates, frees or keeps device memory; the
 *     only state it keeps is a per-thread last-error string and a per-device
 *     record that the device is gfx950.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work on it and return; nothing synchronises.  Faults inside a kernel
 *     show up at the caller's next synchronisation.
 *   - Activations x are [T x M] row-major with row stride ldx >= M elements;
 *     outputs y are [T x N] with ldy >= N; the base weight W0 is [N x M]
 *     (PyTorch's [out, in]) with ldw >= M.
 *   - Scales are fp16 (bit patterns, `const void*` to 2-byte elements).
 *   - Every call validates all arguments before the first HIP call and
 *     returns DBF_OK (0) or a negative dbf_status; dbf_last_error() then
 *     describes the problem.  No exception crosses the ABI.
 *   - Non-finite inputs are outside the contract.
 */
#ifndef DBF_H
#define DBF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DBF_ABI_VERSION 1
#define DBF_LAYOUT_VERSION 1

/* status codes */
#define DBF_OK 0
#define DBF_EINVAL (-1)       /* a size, stride, count or NULL pointer is wrong */
#define DBF_EDTYPE (-2)       /* unsupported dtype code for this argument */
#define DBF_EALIGN (-3)       /* a device pointer is not 16-byte aligned */
#define DBF_EWORKSPACE (-4)   /* ws is NULL or smaller than dbf_workspace_bytes */
#define DBF_EDEVICE (-5)      /* current device is not gfx950, or no device */
#define DBF_EUNSUPPORTED (-6) /* valid but not supported (e.g. int overflow) */
#define DBF_ELAUNCH (-7)      /* a kernel launch failed */
#define DBF_ESTALLED (-8)     /* a handoff wait gave up (dbf_workspace_check) */

/* dtype codes */
#define DBF_F16 1
#define DBF_BF16 2
#define DBF_F32 3
#define DBF_I8 4
#define DBF_I32 5

/* execution paths for dbf_linear_forward / dbf_workspace_bytes */
#define DBF_PATH_AUTO 0   /* chosen by T and n_terms */
#define DBF_PATH_DECODE 1 /* sign-accumulate over packed bits with 16-entry
                             signed subset-sum tables (fp32 throughout) */
#define DBF_PATH_MFMA 2   /* +-1 tiles unpacked from the bits into MFMA
                             operands (fp16 operands, fp32 accumulation) */

#define DBF_MAX_TERMS 8

/* Version of this ABI and of the packed bit layout below. */
int dbf_abi_version(void);
int dbf_layout_version(void);

/* Message for the last non-OK status returned on the calling thread. */
const char *dbf_last_error(void);

/*
 * Packed sign layout (DBF_LAYOUT_VERSION 1).  One bit per sign, as LoRDBA
 * (section 2, "Eficiencia de Armazenamento") and DBF (technical summary,
 * section 2, sign matrices with fp16 scale vectors) store the factors.
 * A sign matrix S in {+-1}^{rows x K} -- B1 with rows = N, K = R; B2 with
 * rows = R, K = M -- is stored as uint32 words:
 *   bit value 1 is +1, 0 is -1; every padding bit is 0;
 *   kw  = min(4, ceil(K / 32)) words per row per tile;
 *   a tile is 64 rows x kw words (64 * kw * 4 bytes, a multiple of 128 B
 *   when kw = 4), stored row by row;
 *   tile (rt, kb) is tile number rt * nkb + kb, nkb = ceil(K / (32 kw));
 *   bit j of word w of row r of tile (rt, kb) holds S[64 rt + r,
 *   32 kw kb + 32 w + j].
 * A wavefront reading one tile row per lane moves one contiguous kw*256 B.
 * dbf_packed_bytes is the size of that buffer, padding included.
 */
size_t dbf_packed_bytes(int64_t rows, int64_t k);

/*
 * Pack the signs of src [rows x k] (row stride ld >= k elements, dtype
 * DBF_I8, DBF_F16, DBF_BF16 or DBF_F32) into `packed`
 * (dbf_packed_bytes(rows, k) bytes, 16-byte aligned).  Bit = (v >= 0):
 * 0 and -0.0 map to +1, NaN to -1 (the binarization B = sign(H) of LoRDBA
 * section 2, "Pipeline de Treinamento", leaves sign(0) open).  Every word of
 * the buffer, padding included, is written.
 */
int dbf_pack(const void *src, int src_dtype, int64_t rows, int64_t k,
             int64_t ld, uint32_t *packed, void *stream);

/* Inverse of dbf_pack for the signs only: writes +-1 as int8 to
 * dst [rows x k] with row stride ld >= k. */
int dbf_unpack(const uint32_t *packed, int64_t rows, int64_t k, int8_t *dst,
               int64_t ld, void *stream);

/*
 * One term of the sum: device pointers to the packed B1 (N x R layout),
 * the packed B2 (R x M layout) and the fp16 vectors alpha (N), beta (R),
 * gamma (M).  The array of terms is host memory and is read during the
 * call only.  Terms may alias the same packed factors.
 */
typedef struct dbf_term {
    const uint32_t *b1;
    const uint32_t *b2;
    const void *alpha;
    const void *beta;
    const void *gamma;
} dbf_term;

/* Bytes of device workspace dbf_linear_forward / dbf_linear_forward_i8 /
 * lordba_adapter_forward need for these sizes and path (the rank-R
 * intermediate of every term, and per-token scale slots for the MFMA
 * path).  The caller allocates it, 16-byte aligned.  Its first
 * DBF_WS_HEAD_BYTES bytes hold the decode path's handoff counters between
 * the workgroups of one launch: they must be zero before the first call
 * that uses the buffer (e.g. allocate it zeroed), every call leaves them
 * zero again, and no path keeps scratch there, so one buffer may serve calls
 * of every path in turn.  The rest is scratch, clobbered by every call.
 * Calls that run at the same time (on different streams) need separate
 * workspaces. */
#define DBF_WS_HEAD_BYTES 16640
size_t dbf_workspace_bytes(int64_t N, int64_t M, int64_t R, int n_terms,
                           int64_t T, int path);

/* Health of a workspace after decode-path or adapter calls.  The consumer
 * workgroups of those launches wait for the producer workgroups of the same
 * launch (dispatched first, so the wait always ends); as a safety net a wait
 * gives up after 2^26 polls (seconds), lets the kernel finish, and sets a
 * flag in the workspace head.  The output of such a call is not valid.
 *   ws      device workspace of earlier calls (not NULL, 16-byte aligned)
 *   stream  the stream those calls ran on; this call waits for it
 * Returns DBF_OK when no wait gave up.  Otherwise it zeroes the head (so the
 * buffer is usable again) and returns DBF_ESTALLED; or DBF_EINVAL when a
 * lordba_multi_adapter_forward call met an adapter index out of range.  Reads 4 bytes and
 * synchronizes the stream, so it is not for use inside graph capture. */
int dbf_workspace_check(void *ws, void *stream);

/*
 * y (+)= sum_i Delta W_i x for T tokens.
 * The forward of LoRDBA section 2 ("Kernel de Inferencia") and DBF section 2
 * ("Inferencia"): two sign-accumulate products over the packed bits,
 * interleaved with the per-channel scales, with no multiplication inside
 * the inner products on the decode path.
 *   terms[n_terms]   1 <= n_terms <= DBF_MAX_TERMS; b1, b2, alpha, beta,
 *                    gamma all non-NULL.
 *   x                [T x M], x_dtype DBF_BF16 or DBF_F16, row stride ldx.
 *   y                [T x N], y_dtype DBF_F32, DBF_BF16 or DBF_F16, ldy.
 *   accumulate       0: y = result; 1: y = y + result (in fp32).
 *   ws, ws_bytes     workspace of dbf_workspace_bytes(..., path) bytes.
 *   path             DBF_PATH_AUTO picks the decode path while T <= 4 or
 *                    n_terms * ceil(T / 4) * R * (N + M) <= 8.0e7, and the
 *                    MFMA path above; the others force one (both are
 *                    correct for every T >= 1).
 * Accumulation is fp32; the decode path keeps every intermediate in fp32,
 * the MFMA path rounds gamma*x and the rank-R intermediate to fp16 once
 * each, both multiplied by exact powers of two per token that keep them
 * inside the fp16 range (so any finite x with a finite result works at any
 * magnitude).
 * T = 0 is valid and does nothing.  Results are bitwise reproducible run
 * to run (no floating-point atomics).
 */
int dbf_linear_forward(const dbf_term *terms, int n_terms, int64_t N,
                       int64_t M, int64_t R, const void *x, int x_dtype,
                       int64_t T, int64_t ldx, void *y, int y_dtype,
                       int64_t ldy, int accumulate, void *ws, size_t ws_bytes,
                       int path, void *stream);

/*
 * dbf_linear_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The workspace is a fixed scratch array of
 * DBF_NOALLOC_SCRATCH_BYTES inside the library, one per device (each device
 * that loads the library holds it until the process ends).  The call
 * allocates nothing.
 *   Arguments, paths and results as dbf_linear_forward (the same kernels).
 *   A call whose dbf_workspace_bytes(N, M, R, n_terms, T, path) exceeds
 *   DBF_NOALLOC_SCRATCH_BYTES returns DBF_EWORKSPACE before any HIP call.
 *   Every call on a device shares that device's array: calls that overlap on
 *   one device (different streams or threads at the same time) race; order
 *   them on one stream.
 */
#define DBF_NOALLOC_SCRATCH_BYTES (16u << 20)
int dbf_linear_forward_noalloc(const dbf_term *terms, int n_terms, int64_t N,
                               int64_t M, int64_t R, const void *x, int x_dtype,
                               int64_t T, int64_t ldx, void *y, int y_dtype,
                               int64_t ldy, int accumulate, int path,
                               void *stream);

/*
 * Integer-activation variant: x is int8 [T x M] with gamma folded into it
 * upstream (terms[i].gamma must be NULL, since gamma sits on the summed
 * index and cannot be applied to integer sums).  The two sign-accumulate
 * products of LoRDBA section 2 ("Kernel de Inferencia") need only additions
 * and subtractions, so with integer activations they are exact integer sums
 * (the int32 S1 and S2 below); the per-channel scales then enter in fp32.
 *   s1 (optional, int32 [n_terms x T x R]):  S1_i = B2_i x, exact.
 *   s2 (optional, int32 [n_terms x T x N]):  S2_i = B1_i S1_i, exact;
 *       needs every beta == NULL (beta = 1).
 *   y  (optional, y_dtype DBF_F32/BF16/F16, ldy): sum_i alpha_i .
 *       B1_i (beta_i . S1_i), fp32 accumulation; a NULL alpha or beta means
 *       all ones.
 * Exactness needs |S1| < 2^31 and, for s2 or a NULL beta, R * M * 127 <
 * 2^31; larger shapes return DBF_EUNSUPPORTED.  Uses the decode path and
 * its workspace (dbf_workspace_bytes(..., DBF_PATH_DECODE)).
 */
int dbf_linear_forward_i8(const dbf_term *terms, int n_terms, int64_t N,
                          int64_t M, int64_t R, const int8_t *x, int64_t T,
                          int64_t ldx, int32_t *s1, int32_t *s2, void *y,
                          int y_dtype, int64_t ldy, void *ws, size_t ws_bytes,
                          void *stream);

/*
 * LoRDBA adapter mode: y = W0 x + sum_i Delta W_i x, the adapter kept
 * unmerged beside the frozen base (LoRDBA sections 1 and 5).  W0 [N x M]
 * bf16 row stride ldw, x bf16 [T x M].  n_terms = 0 computes the base only
 * (terms may then be NULL).  y_dtype DBF_F32, DBF_BF16 or DBF_F16.  The base
 * product and the adapter's second sign-accumulate run in one kernel over
 * the same output rows; the rank-R intermediate needs ws of
 * dbf_workspace_bytes(N, M, R, n_terms, T, DBF_PATH_DECODE) bytes (may be
 * NULL when n_terms = 0).
 */
int lordba_adapter_forward(const void *w0, int64_t ldw, const dbf_term *terms,
                           int n_terms, int64_t N, int64_t M, int64_t R,
                           const void *x, int64_t T, int64_t ldx, void *y,
                           int y_dtype, int64_t ldy, void *ws,
                           size_t ws_bytes, void *stream);

/*
 * ---- Boolean kernels (the Multi-Boolean form) ---------------------------
 * "Highly Efficient and Effective LLMs with Multi-Boolean Architectures",
 * technical summary, section 2: item 1 approximates a weight by its sign
 * matrix with a rank-one scale, W ~ sign(W) . (s_out s_in^T), item 2 sums
 * several such kernels.  So
 *
 *   y = sum_{k=1..K} s_out_k . (Wb_k (s_in_k . x)),   Wb_k in {+-1}^{N x M},
 *
 * one sign-accumulate product per kernel over a full N x M sign matrix (the
 * double-binary layer's stage S3 at R = M).  dbf_svid_extract (below)
 * extracts such kernels from a real weight.
 */
typedef struct {
    const uint32_t *w;  /* Wb_k, dbf_pack(rows = N, k = M) layout; 16-byte aligned */
    const void *s_in;   /* fp16 [M], 2-byte aligned */
    const void *s_out;  /* fp16 [N], 2-byte aligned */
} dbf_bool_kernel;

/* Bytes of workspace dbf_bool_forward needs (0 when T, N, M or n_kernels is
 * not positive).  The head rule of dbf_workspace_bytes applies: its first
 * DBF_WS_HEAD_BYTES must be zero before first use and every call leaves
 * them zero, so one buffer may serve both kinds of call in turn. */
size_t dbf_bool_workspace_bytes(int64_t N, int64_t M, int n_kernels, int64_t T,
                                int path);

/*
 * y (+)= sum_k s_out_k . (Wb_k (s_in_k . x)) for T tokens.
 *   kernels          host array of n_kernels (1..DBF_MAX_TERMS) kernels.
 *   x                [T x M], x_dtype DBF_BF16 or DBF_F16, row stride ldx.
 *   y                [T x N], y_dtype DBF_F32, DBF_BF16 or DBF_F16, ldy.
 *   accumulate       0: y = result; 1: y = y + result (in fp32).
 *   ws, ws_bytes     workspace of dbf_bool_workspace_bytes(..., path) bytes.
 *   path             DBF_PATH_AUTO picks the decode path while T <= 2 or
 *                    n_kernels * b <= 4, b the decode's token blocks
 *                    (ceil(T / 2) for T <= 4, ceil(T / 4) above), and the
 *                    MFMA path otherwise;
 *                    the others force one.
 * The decode path keeps everything in fp32; the MFMA path rounds s_in . x
 * to fp16 once (times an exact power of two per token that keeps it inside
 * the fp16 range), with fp32 accumulation.  x, y 16-byte aligned.  T = 0 is
 * valid and does nothing.  Results are bitwise reproducible run to run.
 */
int dbf_bool_forward(const dbf_bool_kernel *kernels, int n_kernels, int64_t N,
                     int64_t M, const void *x, int x_dtype, int64_t T,
                     int64_t ldx, void *y, int y_dtype, int64_t ldy,
                     int accumulate, void *ws, size_t ws_bytes, int path,
                     void *stream);

/*
 * Successive SVID extraction of boolean kernels from a real weight, the
 * conversion the same section describes: item 1 takes a kernel as the signs
 * of the matrix with a rank-one scale, W ~ sign(W) . (s_out s_in^T); item 3
 * extracts each later kernel the same way from the residual the earlier
 * ones leave.  The page leaves the rank-one fit open; here it is the
 * leading singular pair (sigma, u, v) of |r| (r the current residual),
 * which |r| >= 0 makes nonnegative, split evenly: s_out = fp16(sqrt(sigma)
 * u), s_in = fp16(sqrt(sigma) v), found by `iters` power iterations from
 * the all-ones direction in fp32; the residual is then r - sign(r) .
 * (s_out s_in^T) with the rounded scales.  sign(0) = +1 (the pack rule).
 *   w               N x M, w_dtype DBF_F32, DBF_BF16 or DBF_F16, row stride
 *                   ldw >= M (element-aligned).
 *   kernels         host array of n_kernels (1..DBF_MAX_TERMS) outputs:
 *                   w the packed signs (dbf_packed_bytes(N, M) bytes,
 *                   16-byte aligned), s_in fp16 [M], s_out fp16 [N]
 *                   (2-byte aligned); all written.  They feed
 *                   dbf_bool_forward as they are.
 *   iters           power iterations per kernel, 1..1000.
 *   residual_sq     optional device float [n_kernels]: ||W - sum_{j <= k}
 *                   kernel_j||_F^2 after kernel k.
 *   ws, ws_bytes    dbf_svid_workspace_bytes(N, M) bytes, 16-byte aligned
 *                   (scratch; holds the fp32 residual).
 * Every sum runs in a fixed order, so results are bitwise reproducible.
 */
typedef struct {
    uint32_t *w;  /* packed signs, written */
    void *s_in;   /* fp16 [M], written */
    void *s_out;  /* fp16 [N], written */
} dbf_bool_kernel_out;

size_t dbf_svid_workspace_bytes(int64_t N, int64_t M);
int dbf_svid_extract(const void *w, int w_dtype, int64_t N, int64_t M,
                     int64_t ldw, int n_kernels,
                     const dbf_bool_kernel_out *kernels, int iters,
                     float *residual_sq, void *ws, size_t ws_bytes,
                     void *stream);

/*
 * ---- Backward of dbf_linear_forward -------------------------------------
 * For a loss L with dy = dL/dy, the chain rule through the LoRDBA
 * parametrization (section 2, "Arquitetura Central"), per term i:
 *   g_i = B1_i^T (alpha_i . dy),  h_i = B2_i^T (beta_i . g_i),
 *   s_i = B2_i (gamma_i . x),     z_i = B1_i (beta_i . s_i),
 *   dx = sum_i gamma_i . h_i,
 *   dalpha_i = sum_t dy . z_i,  dbeta_i = sum_t s_i . g_i,  dgamma_i = sum_t x . h_i.
 * The four products per term are sign-accumulates over B2, B1 and their
 * transposes, which the caller packs once with dbf_transpose_packed.
 */

/* out = the packed layout of S^T (k rows x `rows` columns; dbf_packed_bytes(k,
 * rows) bytes, 16-byte aligned) for `packed`, the layout of S (rows x k).
 * Bit-exact; padding bits are 0. */
int dbf_transpose_packed(const uint32_t *packed, int64_t rows, int64_t k,
                         uint32_t *out, void *stream);

typedef struct {
    const uint32_t *b1t;  /* B1_i^T packed: rows R, k N */
    const uint32_t *b2t;  /* B2_i^T packed: rows M, k R */
} dbf_term_t;

/* Workspace bytes of dbf_linear_backward (the head rule of
 * dbf_workspace_bytes applies). */
size_t dbf_backward_workspace_bytes(int64_t N, int64_t M, int64_t R, int n_terms,
                                    int64_t T, int path);

/*
 * Gradients for T tokens.
 *   terms, tterms    n_terms forward terms (alpha, beta, gamma required) and
 *                    their packed transposes.
 *   x  [T x M], x_dtype DBF_BF16 or DBF_F16, ldx;  dy [T x N], dy_dtype
 *   DBF_BF16, DBF_F16 or DBF_F32, lddy.
 *   dx [T x M], dx_dtype DBF_F32/BF16/F16, lddx;  dalpha [n_terms x N],
 *   dbeta [n_terms x R], dgamma [n_terms x M], fp32, contiguous.  Any of
 *   the four outputs may be NULL (not computed); all are overwritten.
 *   path             DBF_PATH_AUTO: decode products while T <= 16, MFMA
 *                    products above; or forced.
 * The products keep fp32 intermediates; on the MFMA path each product rounds
 * its scaled input to fp16 once, times an exact power of two per token that
 * keeps it inside the fp16 range (fp32 sums), so small gradients keep their
 * precision.  Token sums run in fixed order,
 * so results are bitwise reproducible.  T = 0 is valid and does nothing.
 */
int dbf_linear_backward(const dbf_term *terms, const dbf_term_t *tterms, int n_terms,
                        int64_t N, int64_t M, int64_t R, const void *x, int x_dtype,
                        int64_t ldx, const void *dy, int dy_dtype, int64_t lddy,
                        int64_t T, void *dx, int dx_dtype, int64_t lddx, float *dalpha,
                        float *dbeta, float *dgamma, void *ws, size_t ws_bytes, int path,
                        void *stream);

/*
 * ---- Several adapters in one batch --------------------------------------
 * LoRDBA's adapters are small enough to keep many beside one frozen base
 * (section 1: cheap to swap and to communicate).  Each token t uses adapter
 * adapter_idx[t] of the table, or none (-1):
 *
 *   y[t] = W0 x[t] + Delta W_{adapter_idx[t]} x[t].
 */
#define DBF_MAX_ADAPTERS 32

/*
 *   w0, ldw          bf16 base [N x M], shared by every token.
 *   adapters         host array of n_adapters (1..DBF_MAX_ADAPTERS) one-term
 *                    adapters of rank R (alpha, beta, gamma required).
 *   adapter_idx      device int32 [T]: the token's adapter, or -1 for the
 *                    base alone.  An index outside [-1, n_adapters) is
 *                    treated as -1 and raises a flag that dbf_workspace_check
 *                    reports as DBF_EINVAL.
 *   x                bf16 [T x M], ldx;  y [T x N], y_dtype, ldy.
 *   ws, ws_bytes     dbf_workspace_bytes(N, M, R, 1, T, DBF_PATH_DECODE).
 * One launch: one-token workgroups run each token's adapter B2 product while
 * the row workgroups stream W0 once for every token, then add each token's
 * alpha . (B1 w) from its own adapter.
 */
int lordba_multi_adapter_forward(const void *w0, int64_t ldw, const dbf_term *adapters,
                                 int n_adapters, int64_t N, int64_t M, int64_t R,
                                 const int32_t *adapter_idx, const void *x, int64_t T,
                                 int64_t ldx, void *y, int y_dtype, int64_t ldy, void *ws,
                                 size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DBF_H */
