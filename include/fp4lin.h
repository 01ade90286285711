/*
 * fp4lin — FP4 (E2M1) quantized linear layer forward for AMD Instinct MI355X
 * (gfx950). C ABI of libfp4lin.so.
 *
 * The method (FP4 training write-up "微软首创FP4训练框架，训练效果媲美BF16", and the
 * abstract of "Optimizing Large Language Model Training Using FP4 Quantization"):
 * every linear layer Y = A W (A: M tokens x K in-features, W: K x N) is computed
 * from an activation matrix whose outliers are clamped at a per-tensor quantile
 * of |A| (outlier paragraph), a sparse compensation matrix dA = A - A_clamped
 * that is non-zero only at clamped entries (compensation paragraph), token-wise
 * (per row) quantization of A_clamped and channel-wise (per column) quantization
 * of W (granularity paragraph), both by ScaleShift to the E2M1 grid
 * (FP4-format, rounding and ScaleShift paragraphs):
 *
 *     Y = (s_A (.) Q(A_clamped)) (Q(W) (.) s_W) + dA W
 *
 * Number format and rounding, as this library fixes them where the pages are
 * silent:
 *   - E2M1 magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; a code is 4 bits,
 *     sign (bit 3) and magnitude index (bits 0..2).
 *   - For each vector (a row of A, a column of W): amax = max |x|,
 *     inv = RN32(6/amax), s = RN32(amax/6), y = RN32(|x| * inv); the magnitude
 *     index is the number of midpoints {0.25,0.75,1.25,1.75,2.5,3.5,5} with
 *     y >= midpoint (round to nearest, ties away from zero, saturating at 6).
 *     amax = 0 gives inv = +Inf, s = 0 and all-zero magnitudes.
 *   - The sign bit is the sign bit of x (so -0 encodes as 0b1000).
 *   - Threshold tau = k-th smallest |a| (0-based) over all M*K entries with
 *     k = clamp(ceil(q*M*K) - 1, 0, M*K - 1) in IEEE double; the clamped set is
 *     {|a| > tau} (strict).
 *
 * Layouts:
 *   - Dense inputs are row-major with a leading dimension in elements
 *     (lda >= K for A, ldw >= N for W); dtype float32 or bfloat16.
 *   - Packed FP4 matrices: one packed row per vector of L codes, two codes per
 *     byte with the even index in the low nibble, each row padded with zero
 *     codes to a multiple of 128 codes; the row stride is fp4lin_packed_ld(L)
 *     bytes (a multiple of 64). A is packed M x packed_ld(K); W is packed
 *     N-major, N x packed_ld(K) (column j's K codes are contiguous).
 *   - Scales are float32, one per packed row.
 *   - dA is COO in row-major order (row, col int32; val float32 =
 *     RN32(a - sign(a)*tau)) plus row_ptr[M+1] (int32, row_ptr[M] = nnz).
 *   - Y is float32, M x N row-major with leading dimension ldy >= N.
 *
 * Conventions for every call:
 *   - Pointers are device pointers owned by the caller unless marked "host".
 *     The library never allocates, frees or keeps a pointer after return, holds
 *     no global state (apart from each host thread's record of its last HIP
 *     launch result, see fp4lin_last_hip_error, and the static device scratch
 *     of fp4lin_outlier_select_noalloc) and is safe to call from several host
 *     threads.
 *   - All device work is enqueued asynchronously, in order, on `stream`
 *     (0 = the null stream). Nothing is read back and there is no host
 *     synchronisation: results are valid once the caller synchronises the
 *     stream.
 *   - Arguments are checked on the host before anything is enqueued. On error
 *     the call returns a non-zero fp4lin_status, enqueues nothing and leaves
 *     every output untouched. A launch failure reported by the HIP runtime
 *     returns FP4LIN_ERR_LAUNCH (outputs are then unspecified).
 *   - Inputs must be finite (not checked).
 *   - Packed-code pointers and workspaces must be 16-byte aligned.
 */
#ifndef FP4LIN_H
#define FP4LIN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP4LIN_OK = 0,
  FP4LIN_ERR_NULL = 1,       /* a required pointer is NULL                      */
  FP4LIN_ERR_SHAPE = 2,      /* a size < 1, a size >= 2^31, or ld < row length  */
  FP4LIN_ERR_DTYPE = 3,      /* dtype not one of fp4lin_dtype                   */
  FP4LIN_ERR_QUANTILE = 4,   /* q is NaN or outside [0, 1]                      */
  FP4LIN_ERR_CAPACITY = 5,   /* COO capacity < M*K - 1 - k                      */
  FP4LIN_ERR_ALIGN = 6,      /* a pointer that must be 16-byte aligned is not   */
  FP4LIN_ERR_WORKSPACE = 7,  /* workspace smaller than the *_workspace_bytes   */
  FP4LIN_ERR_LAUNCH = 8,     /* the HIP runtime rejected a kernel launch        */
  FP4LIN_ERR_SCRATCH = 9     /* beyond the allocation-free call's static scratch */
} fp4lin_status;

typedef enum { FP4LIN_F32 = 0, FP4LIN_BF16 = 1 } fp4lin_dtype;

/* Sparse compensation matrix dA (device arrays, caller-owned). */
typedef struct {
  int32_t* row;       /* capacity entries; row index of each non-zero          */
  int32_t* col;       /* capacity entries; column index (ascending per row)     */
  float* val;         /* capacity entries; RN32(a - sign(a)*tau)                */
  int32_t* row_ptr;   /* M+1 entries; row i owns [row_ptr[i], row_ptr[i+1])     */
  int64_t capacity;   /* host value: entries allocated in row/col/val           */
} fp4lin_coo;

/* Where fp4lin_forward keeps its intermediates inside its workspace (byte
 * offsets from the workspace base). Filled by fp4lin_forward_layout. */
typedef struct {
  size_t tau;          /* float                                                  */
  size_t coo_row;      /* int32[capacity]                                        */
  size_t coo_col;      /* int32[capacity]                                        */
  size_t coo_val;      /* float[capacity]                                        */
  size_t row_ptr;      /* int32[M+1]                                             */
  size_t Aq;           /* uint8[M * packed_ld(K)]                                */
  size_t sA;           /* float[M]                                               */
  size_t Wq;           /* uint8[N * packed_ld(K)]                                */
  size_t sW;           /* float[N]                                               */
  size_t scratch;      /* internal scratch of the select / weight passes         */
  int64_t capacity;    /* COO capacity = M*K - 1 - k                             */
  size_t total;        /* bytes the forward needs                                */
} fp4lin_forward_offsets;

/* ---- host helpers (no device work) ------------------------------------- */

/* Rank of the clamp threshold: clamp(ceil(q*n) - 1, 0, n - 1), with q*n and
 * ceil evaluated in IEEE double (outlier paragraph: quantile search).
 * Returns -1 if n < 1 or q is NaN or outside [0, 1]. */
int64_t fp4lin_quantile_rank(int64_t n, double q);

/* Bytes per packed row of L FP4 codes: roundup(L, 128) / 2. -1 if L < 1. */
int64_t fp4lin_packed_ld(int64_t L);

/* Workspace bytes fp4lin_outlier_select needs for an M x K input of dtype dt
 * (radix histograms, selection state, per-row counts: grows with M).
 * 0 on invalid arguments. */
size_t fp4lin_select_workspace_bytes(int64_t M, int64_t K, fp4lin_dtype dt);

/* Workspace bytes fp4lin_quantize_weight needs for a K x N weight (per-column
 * maxima). 0 on invalid arguments. */
size_t fp4lin_weight_workspace_bytes(int64_t K, int64_t N);

/* Workspace bytes fp4lin_forward needs, including tau, the COO (capacity
 * M*K - 1 - k for k = fp4lin_quantile_rank(M*K, q)), the packed operands and
 * scales. 0 on invalid arguments. */
size_t fp4lin_workspace_bytes(int64_t M, int64_t K, int64_t N, fp4lin_dtype dt, double q);

/* Fill *out with the forward workspace layout for these arguments. */
fp4lin_status fp4lin_forward_layout(int64_t M, int64_t K, int64_t N, fp4lin_dtype dt,
                                    double q, fp4lin_forward_offsets* out /* host */);

/* Static description of a status code. */
const char* fp4lin_status_str(fp4lin_status s);

/* The hipError_t value (as int) of the calling thread's most recent launch
 * check, and its name: after FP4LIN_ERR_LAUNCH they say what the HIP runtime
 * reported. hipSuccess (0) before any launch on the thread. */
int fp4lin_last_hip_error(void);
const char* fp4lin_last_hip_error_name(void);

/* ---- device operations ---------------------------------------------------- */

/* Outlier selection (outlier and compensation paragraphs of the FP4 training
 * write-up; the abstract's "outlier clamping and compensation").
 * Computes tau, the k-th smallest |a| over the M x K matrix A (k from q as in
 * fp4lin_quantile_rank), and the COO of dA: every entry with |a| > tau, in
 * row-major order, val = RN32(a - sign(a)*tau), and dA.row_ptr.
 *   A        device, M x K, dtype dt, leading dimension lda (elements)
 *   tau      device, 1 float (output)
 *   dA       device arrays (outputs); dA.capacity (host) >= M*K - 1 - k
 *   ws       device workspace of >= fp4lin_select_workspace_bytes(M, K, dt)
 * M*K must be below 2^32 (32-bit histogram counts) and M*K - 1 - k below 2^31
 * (int32 COO positions), else FP4LIN_ERR_SHAPE.
 * Errors: NULL, SHAPE, DTYPE, QUANTILE, CAPACITY, ALIGN (ws), WORKSPACE, LAUNCH. */
fp4lin_status fp4lin_outlier_select(const void* A, fp4lin_dtype dt, int64_t M, int64_t K,
                                    int64_t lda, double q, float* tau, fp4lin_coo dA,
                                    void* ws, size_t ws_bytes, hipStream_t stream);

/* Allocation-free variant of fp4lin_outlier_select, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same operation and outputs, with the
 * select's scratch taken from a static device array of 8 MiB that the library
 * holds on every GPU it runs on until the process ends, instead of a workspace
 * argument. The call allocates and frees nothing; on its first call for a
 * device it looks up that device's copy of the array (the device of `stream`,
 * or the current device for the null stream).
 *   A, dt, M, K, lda, q, tau, dA, stream   as in fp4lin_outlier_select
 * The select must fit the scratch: fp4lin_select_workspace_bytes(M, K, dt) at
 * most 8 MiB, i.e. M up to 1 865 152 rows for bfloat16 and 2 088 896 rows for
 * float32, else FP4LIN_ERR_SCRATCH (checked before anything is enqueued).
 * Every call on a GPU shares that GPU's scratch: calls that overlap on one GPU
 * (on different streams, or from several host threads without ordering) race
 * and give undefined results; calls ordered on one stream are safe. No kernel
 * relies on the scratch's contents from an earlier call.
 * Errors: NULL, SHAPE, DTYPE, QUANTILE, CAPACITY, SCRATCH, LAUNCH (also when
 * the device or its scratch address cannot be determined). */
fp4lin_status fp4lin_outlier_select_noalloc(const void* A, fp4lin_dtype dt, int64_t M,
                                            int64_t K, int64_t lda, double q, float* tau,
                                            fp4lin_coo dA, hipStream_t stream);

/* Token-wise activation quantization (granularity, rounding and ScaleShift
 * paragraphs): each row of X, clamped to [-tau, tau] when tau is given, is
 * scaled by its own amax and rounded to E2M1.
 *   X        device, M x K, dtype dt, leading dimension ldx
 *   tau      device, 1 float, or NULL for no clamping
 *   Xq       device, M x fp4lin_packed_ld(K) bytes (output, padding zeroed)
 *   sX       device, M floats (output): RN32(amax_i / 6)
 * Also used for dgrad operands: dY rows over N, and W rows over N.
 * Errors: NULL, SHAPE, DTYPE, ALIGN (Xq, sX), LAUNCH. */
fp4lin_status fp4lin_quantize_act(const void* X, fp4lin_dtype dt, int64_t M, int64_t K,
                                  int64_t ldx, const float* tau, uint8_t* Xq, float* sX,
                                  hipStream_t stream);

/* Channel-wise weight quantization (granularity paragraph): each column j of
 * the K x N weight is scaled by its own amax and rounded to E2M1; the codes are
 * written transposed, N-major, so the GEMM reads both operands K-contiguous.
 *   W        device, K x N, dtype dt, leading dimension ldw
 *   Wq       device, N x fp4lin_packed_ld(K) bytes (output, padding zeroed)
 *   sW       device, N floats (output): RN32(amax_j / 6)
 *   ws       device workspace of >= fp4lin_weight_workspace_bytes(K, N)
 * K must be at most 65535 * 128 = 8388480 (tiles of 128 codes along K index
 * the second grid dimension), else FP4LIN_ERR_SHAPE.
 * Errors: NULL, SHAPE, DTYPE, ALIGN, WORKSPACE, LAUNCH. */
fp4lin_status fp4lin_quantize_weight(const void* W, fp4lin_dtype dt, int64_t K, int64_t N,
                                     int64_t ldw, uint8_t* Wq, float* sW, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

/* FP4 GEMM with fused epilogue (the FP4 GeMM kernel paragraph gives the role;
 * here it runs on the gfx950 FP4 matrix cores with unit block scales):
 *   acc[i,j] = sum_k v(Aq[i,k]) v(Bq[j,k])            (exact in fp32)
 *   Y[i,j]   = RN32(RN32(acc*sA[i])*sB[j]) + s[i,j],
 *   s[i,j]   = sum_{(i,k) in dA} val*W[k,j], accumulated from 0 in ascending k
 *              with fp32 fused multiply-add, then added once to the product
 *              (rows without non-zeros: the product as it is).
 * The compensation (compensation paragraph: dA W added back) has two
 * schedules with the same bits, picked from dA.capacity: up to 10 entries per
 * row of A (capacity <= 10*M) it runs in the GEMM's epilogue and Y is written
 * once; above that the GEMM writes Y and a second kernel adds s to it (faster
 * at those densities).
 *   Aq, sA   device, M x packed_ld(K) bytes, M floats
 *   Bq, sB   device, N x packed_ld(K) bytes (N-major), N floats
 *   dA       host pointer to a COO descriptor, or NULL for no compensation;
 *            its col, val and row_ptr arrays are read (row is not) and must
 *            describe one row-major matrix, as fp4lin_outlier_select writes them
 *   W        device K x N (dtype wdt, leading dimension ldw), required exactly
 *            when dA is given (the unquantized weight dA multiplies);
 *            K*ldw*sizeof(dtype) must be below 2^31
 *   Y        device, M x N floats, leading dimension ldy (output)
 * Packed operands are addressed with 32-bit byte offsets: (M+1)*packed_ld(K)
 * and (N+1)*packed_ld(K) must be below 2^31 (else FP4LIN_ERR_SHAPE).
 * Errors: NULL, SHAPE, DTYPE, ALIGN, LAUNCH. */
fp4lin_status fp4lin_gemm(const uint8_t* Aq, const float* sA, const uint8_t* Bq,
                          const float* sB, int64_t M, int64_t N, int64_t K,
                          const fp4lin_coo* dA, const void* W, fp4lin_dtype wdt,
                          int64_t ldw, float* Y, int64_t ldy, hipStream_t stream);

/* Sparse compensation alone (compensation paragraph of the FP4 training
 * write-up): Y[i,:] = Y[i,:] + s[i,:], where s is the sum over row i's
 * non-zeros of dA, ascending k, of val * W[k,:], accumulated from 0 with fp32
 * fused multiply-add. Rows without non-zeros are not touched. fp4lin_gemm with
 * a non-NULL dA gives bit for bit what fp4lin_gemm with dA = NULL followed by
 * this call gives, with either of its schedules (in its epilogue it computes
 * the same sum without reading Y back).
 *   dA       host pointer to a COO descriptor (device arrays; row is not read)
 *   W        device K x N weight (dtype wdt, leading dimension ldw); column
 *            indices of dA must be < K
 *   Y        device M x N floats, leading dimension ldy (read and written)
 * W is addressed with 32-bit byte offsets: K*ldw*sizeof(dtype) must be below
 * 2^31 (else FP4LIN_ERR_SHAPE).
 * Errors: NULL, SHAPE, DTYPE, LAUNCH. */
fp4lin_status fp4lin_sparse_add(const fp4lin_coo* dA, const void* W, fp4lin_dtype wdt,
                                int64_t K, int64_t ldw, int64_t M, int64_t N, float* Y,
                                int64_t ldy, hipStream_t stream);

/* ---- micro-scaled (MXFP4) variant ------------------------------------------
 * Micro-scaling lecture "FP4量化训练的硬件挑战：NVIDIA Blackwell架构上的微缩放格式
 * （Micro-scaling）实现", section 3 (one scale per small group, taken from the
 * group's max, elements divided by it and rounded to FP4), with the per-block
 * E8M0 scales of the format survey "训练大型语言模型的挑战" (custom-formats
 * section). Blocks are 32 consecutive codes along K: per row of A, per column
 * of W. A block's scale is 2^e, e the least integer >= -127 with
 * 6 * 2^e >= the block's max |x| (so no element is clipped), stored as the
 * byte e + 127; each element is |x| / 2^e (exact) rounded to the nearest E2M1
 * value, ties away from zero, sign copied. Padding codes are zero and a block
 * with no non-zero element has the byte 0. Each row (of A) or column (of W)
 * has fp4lin_mx_scales_ld(K) = fp4lin_packed_ld(K) / 16 scale bytes, stored
 * step-major for the GEMM: for each K step s of 128 codes, one 32-bit word per
 * row holds the bytes of blocks 4s .. 4s+3 (low byte first), and the words of
 * consecutive rows are adjacent. With R rows, the byte of block b of row i is
 * at offset (b / 4) * 4R + 4i + b % 4 (R * mx_scales_ld(K) bytes in all). */

/* Bytes per row of E8M0 block scales for rows of L codes, or -1 if L < 1. */
int64_t fp4lin_mx_scales_ld(int64_t L);

/* Micro-scaled activation quantization: X (clamped to [-tau, tau] when tau is
 * given, as in the forward) in blocks of 32 along each row.
 *   X        device, M x K, dtype dt, leading dimension ldx
 *   tau      device, 1 float, or NULL for no clamping
 *   Xq       device, M x fp4lin_packed_ld(K) bytes (output, padding zeroed)
 *   Xs       device, M * fp4lin_mx_scales_ld(K) bytes, step-major (output)
 * Xq and Xs must be 16-byte aligned.
 * Errors: NULL, SHAPE, DTYPE, ALIGN, LAUNCH. */
fp4lin_status fp4lin_quantize_act_mx(const void* X, fp4lin_dtype dt, int64_t M, int64_t K,
                                     int64_t ldx, const float* tau, uint8_t* Xq, uint8_t* Xs,
                                     hipStream_t stream);

/* Micro-scaled weight quantization: blocks of 32 along K in each column of the
 * K x N weight, written N-major like fp4lin_quantize_weight. Needs no workspace.
 *   W        device, K x N, dtype dt, leading dimension ldw
 *   Wq       device, N x fp4lin_packed_ld(K) bytes (output, padding zeroed)
 *   Ws       device, N * fp4lin_mx_scales_ld(K) bytes, step-major (output)
 * Wq and Ws must be 16-byte aligned; K must be at most 65535 * 128 = 8388480
 * (tiles of 128 codes along K index the second grid dimension), else
 * FP4LIN_ERR_SHAPE.
 * Errors: NULL, SHAPE, DTYPE, ALIGN, LAUNCH. */
fp4lin_status fp4lin_quantize_weight_mx(const void* W, fp4lin_dtype dt, int64_t K, int64_t N,
                                        int64_t ldw, uint8_t* Wq, uint8_t* Ws,
                                        hipStream_t stream);

/* Micro-scaled FP4 GEMM: the block scales go to the matrix core's scale
 * operands, so
 *   Y[i,j] = sum over blocks b of 2^(eA[i,b] + eB[j,b]) *
 *            sum_{k in b} v(Aq[i,k]) v(Bq[j,k])       (fp32 accumulation)
 *            + s[i,j]                                  (as in fp4lin_gemm)
 * with no separate scale epilogue. Each block's dot product and its scaling
 * are exact; the sum over blocks is rounded to fp32.
 *   Aq, As   device, M x packed_ld(K) bytes; M * mx_scales_ld(K) bytes
 *   Bq, Bs   device, N x packed_ld(K) bytes (N-major); N * mx_scales_ld(K)
 *            (scales step-major, as the quantizers write them)
 *   dA, W, wdt, ldw, Y, ldy   as in fp4lin_gemm
 * Aq, Bq, As and Bs must be 16-byte aligned; the limits of fp4lin_gemm apply.
 * Errors: NULL, SHAPE, DTYPE, ALIGN, LAUNCH. */
fp4lin_status fp4lin_gemm_mx(const uint8_t* Aq, const uint8_t* As, const uint8_t* Bq,
                             const uint8_t* Bs, int64_t M, int64_t N, int64_t K,
                             const fp4lin_coo* dA, const void* W, fp4lin_dtype wdt,
                             int64_t ldw, float* Y, int64_t ldy, hipStream_t stream);

/* Workspace of fp4lin_forward_mx and where it keeps its intermediates: the
 * layout of fp4lin_forward_layout with the sA / sW offsets holding the
 * step-major E8M0 scales of A (M * mx_scales_ld(K) bytes) and of W
 * (N * mx_scales_ld(K) bytes). 0 (or an error) for invalid arguments. */
size_t fp4lin_workspace_bytes_mx(int64_t M, int64_t K, int64_t N, fp4lin_dtype dt, double q);
fp4lin_status fp4lin_forward_layout_mx(int64_t M, int64_t K, int64_t N, fp4lin_dtype dt,
                                       double q, fp4lin_forward_offsets* out /* host */);

/* The whole micro-scaled layer forward: what fp4lin_outlier_select,
 * fp4lin_quantize_act_mx (with the selected tau), fp4lin_quantize_weight_mx
 * and fp4lin_gemm_mx (with dA) compute, in that order on `stream`, keeping
 * every intermediate in `ws` at the offsets fp4lin_forward_layout_mx reports.
 * The outlier compaction also block-quantizes the rows of A it reads, and the
 * quantization of W shares the launch of the select's row count; every
 * intermediate and Y are bit-identical to those of the separate calls.
 *   A, W     device inputs (same dtype dt), leading dimensions lda, ldw
 *   Y        device output, M x N floats, leading dimension ldy
 *   ws       device workspace of >= fp4lin_workspace_bytes_mx(M, K, N, dt, q)
 * Errors: any of the calls it makes. */
fp4lin_status fp4lin_forward_mx(const void* A, const void* W, fp4lin_dtype dt, int64_t M,
                                int64_t K, int64_t N, int64_t lda, int64_t ldw, double q,
                                float* Y, int64_t ldy, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* The whole layer forward (forward-start paragraph: W and A are quantized when
 * the layer's forward begins). Computes what fp4lin_outlier_select,
 * fp4lin_quantize_act (with the selected tau), fp4lin_quantize_weight and
 * fp4lin_gemm (with dA) compute, in that order on `stream`, keeping every
 * intermediate in `ws` at the offsets fp4lin_forward_layout reports. One
 * route for every dtype, K and layout: the select's row count also takes each
 * row's amax clamped to tau, its compaction quantizes the rows of A it reads
 * with the scales that follow, and the two passes over W that
 * fp4lin_quantize_weight makes share the launches of those two row kernels;
 * every intermediate and Y are bit-identical to those of the separate calls.
 *   A, W     device inputs (same dtype dt), leading dimensions lda, ldw
 *   Y        device output, M x N floats, leading dimension ldy
 *   ws       device workspace of >= fp4lin_workspace_bytes(M, K, N, dt, q)
 * Errors: any of the above. */
fp4lin_status fp4lin_forward(const void* A, const void* W, fp4lin_dtype dt, int64_t M,
                             int64_t K, int64_t N, int64_t lda, int64_t ldw, double q,
                             float* Y, int64_t ldy, void* ws, size_t ws_bytes,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4LIN_H */
