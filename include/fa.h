/*
 * fa.h -- C ABI of the fused attention forward pass for AMD Instinct MI355X
 * (gfx950).
 *
 * What is computed (slides "Case study: FlashAttention", slide "Attention is
 * where tokens meet", the attention equation; per-row form on the slide
 * "Problem: softmax needs the whole row"):
 *
 *     S   = scale * Q K^T + mask          (mask: 0 visible, -inf excluded)
 *     O   = softmax_rows(S) V
 *     LSE = ln sum_j exp(S_ij)            (per query row, natural log)
 *
 * for every (batch, head) independently (slide "Queries, keys and values":
 * after the head split each head is an [n x d_k] problem of its own). The
 * causal mask excludes key j from query i when j > i. The kernel never
 * stores S or P; it merges key/value tiles with the online-softmax
 * recurrence of the slide "Online softmax: divide once, at the end" and
 * divides by the row sum once per row. The log-sum-exp row statistic is the
 * quantity that lets partial results over disjoint key blocks be combined
 * later ("Mastering FlashAttention: The Algebraic Foundation", deep-insight
 * takeaways).
 *
 * Layout. q, k, v and o are dense row-major [batch, heads, n, d_k] arrays
 * with d_k fastest (the [h x n x d_k] head split of the slide "Queries, keys
 * and values" with a leading batch axis). lse is dense fp32 [batch, heads,
 * n]. All pointers are device pointers on the current HIP device.
 *
 * Element types. q, k and v share one type. o has the input type for
 * FA_F32, FA_F16 and FA_BF16, and is bf16 for FA_FP8_E4M3 (OCP e4m3 "fn",
 * largest finite 448, no infinities). Accumulation is fp32.
 *
 * Supported shapes. batch, heads >= 1; n >= 1 (any n: ragged tails are
 * masked inside the kernel); d_k in {64, 128}; causal in {0, 1}; scale
 * any finite value whose product with log2(e) is finite (the method's scale
 * is 1/sqrt(d_k); the equation admits any scalar). The library folds log2(e)
 * into |scale| and evaluates exponentials as exp2; a negative scale is
 * applied by negating q inside the kernel, which is exact:
 * scale (q . k) = |scale| ((-q) . k).
 *
 * Ownership. The caller owns every buffer. The library allocates no device
 * or host memory per call and no n x n buffer; the entry points that need
 * scratch memory (fa_forward_splitkv, fa_backward) take it from the caller
 * as a workspace argument. It holds no state beyond per-process kernel
 * registration and each device's compute-unit count, read once (it decides
 * how query tiles are grouped into workgroups). Inputs are only read. Outputs are written in full (every
 * element of the valid rows) and must not overlap the inputs or each other.
 * Calls are reentrant and thread-safe.
 *
 * Errors. Every entry point returns an fa_status. Arguments are validated on
 * the host before any HIP call; on a validation error nothing is launched
 * and no output byte is written. FA_ERR_HIP means the HIP runtime refused
 * the device query or the launch (for example: no GPU); fa_last_hip_error()
 * then returns the hipError_t code for the calling thread. The call is
 * asynchronous: it returns once the kernel is enqueued on `stream` (a
 * hipStream_t; NULL means the null stream). Faults inside the kernel surface
 * at the caller's next synchronisation with that stream, and the buffers
 * must stay alive until the stream has passed the kernel.
 */
#ifndef FA_MI355X_FA_H
#define FA_MI355X_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_F32 = 0,       /* IEEE binary32                                  */
  FA_F16 = 1,       /* IEEE binary16                                  */
  FA_BF16 = 2,      /* bfloat16 (upper half of a binary32)            */
  FA_FP8_E4M3 = 3   /* OCP 8-bit E4M3 "fn" (bias 7, max 448, no inf)  */
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL                             */
  FA_ERR_SHAPE = 2,       /* batch, heads or n < 1, or a workspace too small         */
  FA_ERR_DTYPE = 3,       /* dtype is not one of fa_dtype                           */
  FA_ERR_UNSUPPORTED = 4, /* d_k not in {64, 128}, causal not in {0, 1}, or a mode  */
                          /* this entry point does not offer                       */
  FA_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned                       */
  FA_ERR_SCALE = 6,       /* scale not finite (or overflows times log2 e); a descale
                             not finite and > 0                                    */
  FA_ERR_ALIAS = 7,       /* an output or workspace overlaps an input or an output  */
  FA_ERR_OVERFLOW = 8,    /* the problem exceeds the kernel's index or grid range   */
                          /* (one head's bytes must stay below 2^31)               */
  FA_ERR_HIP = 9,         /* the HIP runtime refused a call; see fa_last_hip_error  */
  FA_ERR_SCRATCH = 10     /* fa_forward_splitkv_noalloc: partials exceed its fixed
                             scratch (fa_noalloc_scratch_bytes)                    */
} fa_status;

/*
 * fa_forward -- O and LSE of exact scaled-dot-product attention.
 *
 *   q, k, v  [batch, heads, n, d_k] of `dtype` (read only)
 *   o        [batch, heads, n, d_k] output (input type; bf16 for FP8_E4M3)
 *   lse      [batch, heads, n] fp32 output, natural-log log-sum-exp of the
 *            scaled (and masked) scores of each row; may be NULL (not written)
 *   scale    multiplier of Q K^T (typically 1/sqrt(d_k))
 *   causal   1: key j is excluded from query i when j > i; 0: no mask
 *   dtype    an fa_dtype; FA_FP8_E4M3 here means all descales are 1.0
 *   stream   hipStream_t to enqueue on (NULL: the null stream)
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int batch, int heads, int n, int d_k, float scale, int causal,
               int dtype, void* stream);

/*
 * fa_forward_fp8 -- as fa_forward for FP8_E4M3 inputs with one fp32 descale
 * per tensor: the value of an element is (its e4m3 code value) * descale.
 * The scores are scale * q_descale * k_descale * (Q8 K8^T); O is
 * v_descale * (P V8), written as bf16. LSE is in units of those scores.
 * Descales must be finite and > 0. (FP8 is the input precision that the
 * dictionary entry "FlashAttention" credits to FlashAttention-3.)
 */
int fa_forward_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                   int batch, int heads, int n, int d_k, float scale, int causal,
                   float q_descale, float k_descale, float v_descale, void* stream);

/*
 * fa_forward_strided -- fa_forward on q, k, v, o laid out with arbitrary
 * element strides (d_k contiguous): element (b, h, i, c) of q is
 *     q[b * strides[0] + h * strides[1] + i * strides[2] + c]
 * and likewise k (strides[3..5]), v (strides[6..8]) and o (strides[9..11]).
 * This takes, for example, the [batch, n, heads, d_k] rows of X Wq directly,
 * without the head transpose of the slide "Queries, keys and values" (strides
 * n*heads*d_k, d_k, heads*d_k). lse stays dense [batch, heads, n]. The result
 * is bitwise the one fa_forward gives on the same values in the dense layout.
 *   strides   12 int64 values (elements), each >= 0; a row stride must be
 *             >= d_k (FA_ERR_UNSUPPORTED otherwise); each stride times the
 *             element size must be a multiple of 16 bytes (FA_ERR_ALIGN); the
 *             rows that o addresses must be disjoint (FA_ERR_ALIAS); one
 *             head's rows must span less than 2^31 bytes (FA_ERR_OVERFLOW)
 * Other arguments and errors as fa_forward (FA_FP8_E4M3: unit descales).
 */
int fa_forward_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                       int batch, int heads, int n, int d_k, const int64_t* strides,
                       float scale, int causal, int dtype, void* stream);

/*
 * fa_forward_varlen -- fa_forward over a ragged batch: `batch` sequences of
 * different lengths packed along one row axis. Sequence b is rows
 * cu_seqlens[b] .. cu_seqlens[b+1] - 1; attention (and the causal mask, by
 * position within the sequence) never crosses sequences.
 *   q, k, v, o    [total, heads, d_k], contiguous (d_k fastest)
 *   lse           [heads, total] fp32, or NULL
 *   cu_seqlens    DEVICE pointer to batch + 1 int32 offsets, non-decreasing,
 *                 cu_seqlens[0] = 0, cu_seqlens[batch] = total, and no
 *                 sequence longer than max_seqlen. The kernels clamp every
 *                 offset to [0, total] and every length to max_seqlen, so
 *                 other contents give unspecified results but no access
 *                 outside the arrays.
 *   max_seqlen    the longest sequence (sizes the grid), >= 1
 * total = 0 returns FA_OK without launching. Other arguments and errors as
 * fa_forward (FA_FP8_E4M3: unit descales).
 */
int fa_forward_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int* cu_seqlens, int batch, int total, int max_seqlen, int heads,
                      int d_k, float scale, int causal, int dtype, void* stream);

/*
 * fa_forward_splitkv -- fa_forward with the keys of every (batch, head) cut
 * into `splits` contiguous blocks that separate workgroups process, followed
 * by the log-sum-exp merge of their partial results:
 *     LSE = ln sum_g e^{LSE_g},   O = sum_g e^{LSE_g - LSE} O_g
 * where O_g and LSE_g are the output and log-sum-exp of the row over block g
 * alone. The merge is the associative combine of per-block softmax states
 * ("Mastering FlashAttention: The Algebraic Foundation", deep-insight
 * takeaways: log-sum-exp lets blocks recombine without global
 * synchronisation). It raises the parallelism of problems with few
 * (batch, head, query tile) units. The result equals fa_forward's up to
 * rounding.
 *
 *   splits      requested number of key blocks, 1 .. 256. Block g holds
 *               keys [g*B, min(n, (g+1)*B)) with B = 128 * ceil(ceil(n /
 *               splits) / 128), so ceil(n / B) blocks are used (one block:
 *               plain fa_forward, no workspace). The workspace holds fp32
 *               O_g [blocks][batch][heads][n][d_k] from byte 0 and fp32
 *               LSE_g [blocks][batch][heads][n] from the next multiple of
 *               256 bytes.
 *   workspace   caller-owned device memory, 16-byte aligned, at least
 *               fa_splitkv_workspace_size(...) bytes, not overlapping any
 *               other argument; its contents on entry are ignored and on
 *               return are unspecified (fp32 partial outputs and LSEs)
 * Other arguments as fa_forward. Extra status codes: FA_ERR_UNSUPPORTED for
 * splits out of range, FA_ERR_NULL / FA_ERR_ALIGN / FA_ERR_ALIAS for the
 * workspace, FA_ERR_SHAPE when workspace_bytes is too small. Two kernels are
 * enqueued on `stream` (the blocks, then the merge).
 */
int fa_forward_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                       int batch, int heads, int n, int d_k, float scale, int causal, int dtype,
                       int splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_forward_splitkv_noalloc -- fa_forward_splitkv for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid allocation. Instead of a workspace argument, the
 * per-block partials go to a fixed array of fa_noalloc_scratch_bytes()
 * (128 MiB) that the library's code object holds on each GPU it runs on
 * until the process ends. The call allocates nothing (no hipMalloc, no
 * allocating library routine); the caller still passes q, k, v, o and lse.
 * The result is that of fa_forward_splitkv with the same arguments, bit for
 * bit (the same kernels on the same block count).
 *
 * The partials need fa_splitkv_workspace_size(batch, heads, n, d_k, splits)
 * bytes; a call that needs more than the scratch returns FA_ERR_SCRATCH
 * before any HIP call (use fa_forward_splitkv with a workspace then). Every
 * call on one GPU uses that GPU's one scratch array: calls that overlap on
 * one GPU (for instance on two streams at once) race on it and must be
 * ordered by the caller. The array keeps the last call's partials; nothing
 * in it needs to start at zero (every partial row is written before the
 * merge reads it). Other arguments, status codes and the asynchronous
 * contract as fa_forward_splitkv.
 */
int fa_forward_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                               int batch, int heads, int n, int d_k, float scale, int causal,
                               int dtype, int splits, void* stream);

/* Bytes of the fixed per-GPU scratch of fa_forward_splitkv_noalloc. */
size_t fa_noalloc_scratch_bytes(void);

/* Workspace bytes fa_forward_splitkv needs for these sizes; 0 when the keys
 * would not be split (or the sizes are invalid). Pure host computation. */
size_t fa_splitkv_workspace_size(int batch, int heads, int n, int d_k, int splits);

/*
 * fa_splitkv_splits -- a key-block count for fa_forward_splitkv. Splitting
 * pays only while the (batch, head, 256-row query tile) units leave compute
 * units idle; under a causal mask the longest tiles set the time, so twice
 * as many units are asked for. The count doubles from 1 while
 *     batch * heads * ceil(n / 256) * splits < compute_units * (causal ? 2 : 1)
 * and every block would still hold at least 256 keys (512 * splits <= n),
 * up to 256. Examples with 256 compute units: 2 heads, n = 4096, no mask ->
 * 8; 4 heads, n = 16384, causal -> 2; 64 (batch, head) pairs, n = 2048,
 * causal -> 1 (these are the measured best choices).
 *   compute_units  the device's compute-unit count; <= 0 reads it from the
 *                  current HIP device (256 when that query fails).
 * Returns 0 for invalid sizes (batch, heads or n < 1, causal not 0 or 1).
 * Host code only; the query of the device is its only HIP call.
 */
int fa_splitkv_splits(int batch, int heads, int n, int causal, int compute_units);

/*
 * fa_backward -- gradients of the attention of fa_forward (f16 / bf16).
 *
 * Given dO = dL/dO of a scalar loss L, with P = softmax_rows(scale Q K^T +
 * mask) as in fa_forward:
 *     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   D = rowsum(dO * O),
 *     dQ = scale dS K,   dK = scale dS^T Q
 * (the chain rule through the equation of the slide "Attention is where
 * tokens meet"). P is never stored: it is recomputed on-chip from Q, K and
 * the forward's LSE, in two passes (article "Mastering FlashAttention: The
 * Algebraic Foundation", technical deep dive): a query-major pass writes dQ,
 * a key-major pass writes dK and dV. The result is deterministic (no atomics).
 *
 *   q, k, v     the forward's inputs, [batch, heads, n, d_k] (read only)
 *   o, lse      the forward's outputs O [batch, heads, n, d_k] and fp32 LSE
 *               [batch, heads, n] for the same q, k, v, scale and causal flag
 *               (read only)
 *   dout        dO, [batch, heads, n, d_k] (read only)
 *   dq, dk, dv  outputs, [batch, heads, n, d_k], same type as q
 *   dtype       FA_F16 or FA_BF16 (others: FA_ERR_UNSUPPORTED)
 *   workspace   caller-owned device memory, 16-byte aligned, at least
 *               fa_backward_workspace_size(batch, heads, n) bytes; on return
 *               it holds fp32 D [batch, heads, n] from byte 0 and
 *               -LSE * log2(e) from the next multiple of 256 bytes
 * Other arguments as fa_forward. All pointers are required (FA_ERR_NULL) and
 * 16-byte aligned. dq, dk, dv and the workspace must not overlap any input or
 * each other (FA_ERR_ALIAS); workspace_bytes too small gives FA_ERR_SHAPE.
 * Two kernels are enqueued on `stream`.
 */
int fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, int batch, int heads, int n,
                int d_k, float scale, int causal, int dtype, void* workspace,
                size_t workspace_bytes, void* stream);

/* Workspace bytes fa_backward needs (0 for invalid sizes). Pure host code. */
size_t fa_backward_workspace_size(int batch, int heads, int n);

/*
 * fa_backward_varlen -- fa_backward over a ragged batch, the gradients of
 * fa_forward_varlen: q, k, v, o, dout, dq, dk, dv are [total, heads, d_k]
 * packed rows, lse is [heads, total] (as fa_forward_varlen writes it), and
 * cu_seqlens, batch, total and max_seqlen are as for fa_forward_varlen (the
 * same clamping applies). Packed rows with equal lengths are also the
 * [batch, n, heads, d_k] layout. The workspace must hold
 * fa_backward_workspace_size(1, heads, total) bytes; on return it holds D and
 * -LSE * log2(e) as [heads, total] fp32 arrays (the second from the next
 * multiple of 256 bytes). total = 0 returns FA_OK without launching. Other
 * arguments and errors as fa_backward.
 */
int fa_backward_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, const int* cu_seqlens,
                       int batch, int total, int max_seqlen, int heads, int d_k, float scale,
                       int causal, int dtype, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * fa_forward_unfused -- the same O and LSE as fa_forward (f16 / bf16), computed
 * step by step with S and P written to memory: S = scale Q K^T (causal
 * entries -inf) as fp32, then a row softmax writing P in the input type and
 * LSE, then O = P V. This is the computation the fused kernel replaces
 * (slides "Case study: FlashAttention", slide "FlashAttention: the idea":
 * done step by step, S and P go out to HBM and back); it exists as a measured
 * contrast, not as a fast path. Its memory traffic and workspace grow as n^2.
 *
 *   workspace   caller-owned device memory, 16-byte aligned, at least
 *               fa_unfused_workspace_size(batch, heads, n) bytes: fp32 S
 *               [batch, heads, n, n] from byte 0, P [batch, heads, n, n] in
 *               the input type from the next multiple of 256 bytes; on return
 *               it holds S and P
 * Other arguments as fa_forward. dtype must be FA_F16 or FA_BF16
 * (FA_ERR_UNSUPPORTED otherwise). Three kernels are enqueued on `stream`.
 */
int fa_forward_unfused(const void* q, const void* k, const void* v, void* o, float* lse,
                       int batch, int heads, int n, int d_k, float scale, int causal, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes fa_forward_unfused needs (0 for invalid sizes). */
size_t fa_unfused_workspace_size(int batch, int heads, int n);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_status_string(int status);

/* hipError_t of the most recent FA_ERR_HIP returned on the calling thread
 * (0 if none). */
int fa_last_hip_error(void);

/* Version of this ABI: major * 10000 + minor * 100 + patch. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_FA_H */
