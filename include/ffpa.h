/*
 * ffpa.h -- C ABI of the MI355X (gfx950) large-head-dim attention library (libffpa.so).
 *
 * The library computes fused scaled-dot-product attention for head dims D = 320..1024
 * (D % 32 == 0) in bf16 or fp16 storage with fp32 accumulation: a forward pass that returns O
 * and a float32 log-sum-exp, and a backward pass in four stages (preprocess Delta =
 * rowsum(dO * O), then dV, dK and dQ). It follows the operation the ffpa-attn user guide defines:
 *
 *   - "Backends Overview", section "Automatic SDPA fallback": the entry points keep PyTorch's
 *     scaled_dot_product_attention contract, O = softmax(scale * Q K^T) V;
 *   - "Triton Backend", section "Feature support": causal masking is tail-aligned (bottom-right),
 *     cross-attention (Nq != Nkv), GQA/MQA and non-aligned N are supported;
 *   - "CuTe-DSL Backend", section "Hard constraints": GQA/MQA is a zero-stride head broadcast, and
 *     rows with no legal key give O = 0, LSE = -inf and exactly zero gradient;
 *   - "CuTe-DSL Backend", section "Varlen (packed THD) API": packed [T, H, D] tensors with int32
 *     cu_seqlens [B+1] starting at 0, causal applied per sequence, LSE returned as float32
 *     [H_q, T_q];
 *   - "CuTe-DSL Backend", section "Blackwell status": the backward runs as preprocess, dV, dK, dQ.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers to contiguous buffers owned by the caller. The
 *     library allocates no memory and keeps no state between calls, except the fixed per-device
 *     scratch array that ffpa_decode_fwd_noalloc uses in place of a workspace.
 *   - Element (b, h, n, d) of a dense [B, H, N, D] tensor sits at ((b*H + h)*N + n)*D + d;
 *     element (t, h, d) of a packed [T, H, D] tensor sits at (t*H + h)*D + d.
 *   - Query head h reads KV head h / (Hq / Hkv).
 *   - Causal: key j is legal for query i iff j <= i + (Nkv - Nq) (per sequence for varlen).
 *   - dtype: FFPA_DTYPE_BF16 or FFPA_DTYPE_FP16; q, k, v, o, dout, dq, dk, dv all use it.
 *   - scale multiplies Q K^T before the softmax; it must be finite and > 0 (1/sqrt(D) is the
 *     SDPA default).
 *   - stream: a hipStream_t (NULL = the default stream). Work is enqueued asynchronously; results
 *     are valid once the stream has been synchronised. The backward's launches are ordered on it.
 *   - Return value: an ffpa_status_t. Arguments are validated on the host before anything is
 *     enqueued; a non-OK status means nothing was launched. FFPA_ERR_HIP reports a failed launch.
 *   - Inputs are assumed finite. Buffers may not alias each other except q/k/v among themselves.
 *
 * Optional P/dS workspace of the backward entry points (workspace, workspace_bytes)
 *   NULL: the dK, dV and dQ stages recompute S and P (and dP, dS) from q, k, v and dout (memory
 *     O(N)).
 *   Non-NULL: a P/dS stage stores the rounded P = exp(scale q k^T - lse) and
 *     dS = P * (dP - Delta) (dtype, the values the products use) into the workspace, and the dK,
 *     dV and dQ stages are products of them, dk = scale * dS^T q, dv = P^T dout and
 *     dq = scale * dS k, instead of recomputations: 4 D flops per (query, key) pair to form P and
 *     dS, then 2 D per product, instead of 6 D, 4 D and 6 D. It takes
 *     ffpa_bwd_workspace_bytes() bytes of device memory: 2 * B * Hq * Nkv * round_up(Nq, 8) * 2,
 *     the dS block, then the P block, each stored transposed (one row of round_up(Nq, 8) queries
 *     per key). The workspace is caller-owned device memory; its contents are scratch. A workspace
 *     smaller than the size function's value is FFPA_ERR_INVALID_ARGUMENT. When the size function
 *     returns 0 (a head's block would exceed 2^31 bytes) the workspace is ignored and the stages
 *     recompute.
 *   Both choices give the same result up to the order of fp32 additions and the rounding of P and
 *   dS to dtype.
 */
#ifndef FFPA_H_
#define FFPA_H_

#include <hip/hip_runtime_api.h> /* hipStream_t */
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FFPA_DTYPE_BF16 = 0,
  FFPA_DTYPE_FP16 = 1
} ffpa_dtype_t;

/* attn_mask kinds ("Triton Backend", "Feature support": boolean and additive masks). */
typedef enum {
  FFPA_MASK_ADDITIVE = 1, /* a bias in q's dtype added to the scaled scores */
  FFPA_MASK_BOOL = 2      /* one byte per element: nonzero keeps the key, 0 drops it (score -inf) */
} ffpa_mask_kind_t;

typedef enum {
  FFPA_OK = 0,
  FFPA_ERR_INVALID_ARGUMENT = 1, /* null pointer, size < 1, Hq % Hkv != 0, bad enum, causal not 0/1, scale <= 0 */
  FFPA_ERR_NOT_SUPPORTED = 2,    /* D outside [320, 1024] or D % 32 != 0 */
  FFPA_ERR_HIP = 3,              /* a HIP launch or runtime call failed */
  FFPA_ERR_TOO_LARGE = 4         /* ffpa_decode_fwd_noalloc: the call needs more than the fixed scratch */
} ffpa_status_t;

/*
 * Dense forward ("Backends Overview", "Automatic SDPA fallback"; "CuTe-DSL Backend",
 * "Hard constraints").
 *   q    [batch, hq,  nq,  d]   in
 *   k, v [batch, hkv, nkv, d]   in
 *   o    [batch, hq,  nq,  d]   out, softmax(scale q k^T) v rounded to dtype; 0 for empty rows
 *   lse  [batch, hq,  nq] fp32  out, natural-log log-sum-exp of the scaled scores; -inf for empty rows
 * Requires batch, hq, hkv, nq, nkv >= 1 and hq % hkv == 0.
 */
ffpa_status_t ffpa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
    int batch, int hq, int hkv, int nq, int nkv, int d,
    ffpa_dtype_t dtype, float scale, int causal, hipStream_t stream);

/*
 * Dense forward for grids too small to fill the GPU: same arguments and results as ffpa_fwd
 * (O and LSE equal up to fp32 summation order), plus a caller-owned device workspace of at least
 * ffpa_fwd_split_workspace_bytes() bytes. The key tiles of every query tile are split into ranges
 * (an equal share of the tile's own, causal, range each: the heavy tiles of a causal grid are
 * split too); each range writes a normalised fp32 O and its log2 LSE per row to the workspace and
 * a second pass merges them by LSE weights ("Triton Backend", "Feature support": the split-KV
 * two-stage merge). When the size function returns 0 no split helps: the call is ffpa_fwd and
 * the workspace is ignored (may be NULL). Otherwise a NULL or smaller workspace is
 * FFPA_ERR_INVALID_ARGUMENT. Workspace layout: fp32 O [batch, hq, nq, nsplit, d] then fp32 LSE
 * [batch, hq, nq, nsplit]; its contents are scratch.
 */
ffpa_status_t ffpa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
    int batch, int hq, int hkv, int nq, int nkv, int d,
    ffpa_dtype_t dtype, float scale, int causal, void* workspace, size_t workspace_bytes,
    hipStream_t stream);

/* Bytes of the ffpa_fwd_split workspace; 0 when the grid needs no split or the sizes are invalid. */
size_t ffpa_fwd_split_workspace_bytes(int batch, int hq, int hkv, int nq, int nkv, int d);

/*
 * Dense forward with an attn_mask ("Triton Backend", "Feature support": boolean and additive
 * masks, broadcast in any of the four dimensions). Arguments as ffpa_fwd plus:
 *   mask          device pointer to the mask (FFPA_MASK_ADDITIVE: q's dtype; FFPA_MASK_BOOL: one
 *                 byte per element, nonzero keeps the key)
 *   mask_kind     FFPA_MASK_ADDITIVE or FFPA_MASK_BOOL
 *   mask_strides  host int64[4]: element (b, h, i, j) of the mask, for query head h, query i and
 *                 key j, sits at b*s[0] + h*s[1] + i*s[2] + j*s[3]; a stride of 0 broadcasts that
 *                 dimension. s[3] must be 0 or 1; with s[3] == 1, s[0..2] are multiples of 8 and
 *                 the mask pointer is 16-byte (additive) / 8-byte (boolean) aligned. The mask is
 *                 read in aligned 8-key pieces: the piece holding a row's last key is read whole,
 *                 so up to 7 elements past that key (never past its aligned 16- or 8-byte piece)
 *                 are loaded and ignored.
 * The scores are scale * q k^T + bias (or -inf where a boolean mask drops the key), combined with
 * the causal mask when causal = 1; a row whose scores are all -inf is empty (O = 0, LSE = -inf).
 * Invalid mask arguments are FFPA_ERR_INVALID_ARGUMENT.
 */
ffpa_status_t ffpa_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse,
    int batch, int hq, int hkv, int nq, int nkv, int d,
    const void* mask, ffpa_mask_kind_t mask_kind, const int64_t* mask_strides,
    ffpa_dtype_t dtype, float scale, int causal, hipStream_t stream);

/*
 * FP8 dense forward ("Backends Overview", backend table and notes: FP8 attention takes fp16/bf16
 * activations and quantizes Q, K and V inside the kernel; forward only). Arguments as ffpa_fwd
 * plus a caller-owned device workspace of at least ffpa_fwd_fp8_workspace_bytes() bytes. Head dims
 * as ffpa_fwd (320..1024, multiples of 32) and batch * hq <= 65535 (else FFPA_ERR_NOT_SUPPORTED);
 * a workspace that is NULL or too small is
 * FFPA_ERR_INVALID_ARGUMENT. The guide's FP8 page is not available; the semantics implemented:
 *   - OCP e4m3 (max 448) for Q, K, V and P, rounded to nearest even from fp32;
 *   - one scale per (batch, head) and tensor: x8 = e4m3(x * (448 / amax)), amax = max |x| over the
 *     head (a zero head stays zero);
 *   - S = scale * (Q8 K8^T) * amax_q * amax_k / 448^2; P = exp(S - running row max) in [0, 1],
 *     P8 = e4m3(P * 448); O = (P8 V8) * amax_v / 448^2 / l with l = sum P (fp32), LSE = ln-sum-exp
 *     of S as in ffpa_fwd; causal, GQA and empty rows as in ffpa_fwd.
 * Workspace layout (each part 256-byte aligned): fp32 amax of Q [batch, hq], K [batch, hkv],
 * V [batch, hkv]; K8 [batch, hkv, nkv, d] bytes; V8 transposed [batch, hkv, d, np] bytes with np =
 * nkv rounded up to 64 (zero padding). It is left filled after the call.
 */
ffpa_status_t ffpa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
    int batch, int hq, int hkv, int nq, int nkv, int d,
    ffpa_dtype_t dtype, float scale, int causal, void* workspace, size_t workspace_bytes,
    hipStream_t stream);

/* Bytes of the ffpa_fwd_fp8 workspace; 0 for invalid sizes or d outside 320..1024. Host function. */
size_t ffpa_fwd_fp8_workspace_bytes(int batch, int hq, int hkv, int nq, int nkv, int d);

/*
 * Strided (zero-copy) dense forward ("Backends Overview", backend table notes: NHD zero-copy
 * consumes [B, N, H, D] or fused-QKV chunk views without a packed copy, an inference-path
 * feature). Same as ffpa_fwd, but q, k, v and o are addressed through strides instead of the
 * packed [B, H, N, D] layout: element (b, h, n, d) of tensor t sits at
 *   b * strides[3t] + h * strides[3t + 1] + n * strides[3t + 2] + d,    t = 0 q, 1 k, 2 v, 3 o,
 * with strides in elements (so [B, N, H, D] is {N H D, D, H D} and a fused [B, N, 3, H, D] tensor
 * gives q, k, v views with {3 N H D, D, 3 H D} at offsets 0, H D, 2 H D). lse stays packed
 * [batch, hq, nq]. Requirements (else FFPA_ERR_INVALID_ARGUMENT): strides non-NULL, non-negative
 * and multiples of 8; q, k, v, o 16-byte aligned; for every tensor, (rows - 1) * row stride + d
 * below 2^30 elements and head and row strides below 2^31. o must not overlap the inputs or
 * itself.
 */
ffpa_status_t ffpa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
    int batch, int hq, int hkv, int nq, int nkv, int d, const int64_t* strides,
    ffpa_dtype_t dtype, float scale, int causal, hipStream_t stream);

/*
 * Split-KV decode forward ("Triton Backend", "Feature support": decode as a two-stage split-KV
 * path; "Backends Overview", "Automatic SDPA fallback": the native decode path serves Nq in
 * [1, 8)). Same arguments, layouts and results as ffpa_fwd (o, lse), plus a caller-owned device
 * workspace of at least ffpa_decode_workspace_bytes() bytes (scratch: partial results per key
 * range). The keys are cut into ranges processed by separate workgroups, each over all
 * (query head of the KV group, query) rows, and the partial results are merged by a second
 * launch; the result equals ffpa_fwd's up to the order of fp32 additions. Meant for few queries
 * (it is correct for any nq, but each workgroup holds 32 rows). A NULL or too-small workspace is
 * FFPA_ERR_INVALID_ARGUMENT.
 */
ffpa_status_t ffpa_decode_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
    int batch, int hq, int hkv, int nq, int nkv, int d,
    ffpa_dtype_t dtype, float scale, int causal, void* workspace, size_t workspace_bytes,
    hipStream_t stream);

/* ffpa_decode_fwd with the strided layouts of ffpa_fwd_strided (same strides[12] and rules). */
ffpa_status_t ffpa_decode_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
    int batch, int hq, int hkv, int nq, int nkv, int d, const int64_t* strides,
    ffpa_dtype_t dtype, float scale, int causal, void* workspace,
    size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of the ffpa_decode_fwd workspace for these sizes: batch * hq * nq * nsplit * (d + 1) * 4,
 * where nsplit (the number of key ranges, 1..256) is the library's choice for these sizes; 0 for
 * invalid sizes. Host function; launches nothing.
 */
size_t ffpa_decode_workspace_bytes(int batch, int hq, int hkv, int nq, int nkv, int d);

/* Bytes of the library's fixed device scratch used by ffpa_decode_fwd_noalloc (32 MiB per GPU). */
#define FFPA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * ffpa_decode_fwd without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * arguments (minus the workspace), checks and results as ffpa_decode_fwd; the partial results go
 * to a fixed device array of FFPA_NOALLOC_SCRATCH_BYTES inside the library instead of a caller
 * workspace. It calls no hipMalloc/hipFree: each GPU the library runs on holds its own copy of the
 * array from the first call on that device until the process ends.
 *   - Sizes whose ffpa_decode_workspace_bytes() exceeds FFPA_NOALLOC_SCRATCH_BYTES return
 *     FFPA_ERR_TOO_LARGE (nothing launched); use ffpa_decode_fwd with a workspace for them.
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's contents (every
 *     entry a call reads is written earlier in the same call, so no clearing is needed). Calls
 *     that overlap on one GPU (on different streams, or from different threads without ordering)
 *     race on it and give undefined results: serialize them on one stream.
 */
ffpa_status_t ffpa_decode_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
    int batch, int hq, int hkv, int nq, int nkv, int d,
    ffpa_dtype_t dtype, float scale, int causal, hipStream_t stream);

/*
 * Bytes of the optional P/dS workspace of ffpa_bwd / ffpa_bwd_stage for these sizes:
 * 2 * batch * hq * nkv * round_up(nq, 8) * 2, or 0 when the stored-P/dS passes are not available
 * (a head's block above 2^31 bytes) or a size is < 1. Host function; launches nothing.
 */
size_t ffpa_bwd_workspace_bytes(int batch, int hq, int nq, int nkv);

/*
 * Dense backward ("CuTe-DSL Backend", "Blackwell status": preprocess, dV, dK, dQ) of
 * L = sum(dout * o) + sum(dlse * lse). Takes the forward's inputs, its outputs o and lse,
 * dout [batch, hq, nq, d] and optionally the gradient of the returned LSE ("CuTe-DSL Backend",
 * "Varlen (packed THD) API": the LSE is handed back to the caller, return_lse=True, so a loss may
 * use it).
 *   dlse  [batch, hq, nq] fp32   in, or NULL for zero. Since d lse_i / d s_ij = P_ij, it enters
 *                                as delta_i = rowsum(dout * o)_i - dlse_i (dS = P * (dP - delta));
 *                                ignored on rows with lse = -inf
 *   delta [batch, hq, nq] fp32   caller-owned workspace, overwritten with that delta
 *   dq    [batch, hq, nq, d]     out
 *   dk, dv [batch, hkv, nkv, d]  out; sums over the hq/hkv query heads that share a KV head
 *   workspace, workspace_bytes   optional P/dS workspace (see above), or NULL, 0
 * Gradients are accumulated in fp32 and rounded to dtype once. Rows with lse = -inf contribute
 * nothing and get dq = 0.
 */
ffpa_status_t ffpa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
    const float* lse, const float* dlse, float* delta, void* dq, void* dk, void* dv,
    int batch, int hq, int hkv, int nq, int nkv, int d,
    ffpa_dtype_t dtype, float scale, int causal, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Dense backward with the attn_mask of ffpa_fwd_masked (same mask arguments; "Triton Backend",
 * "Feature support": additive masks get a gradient reduced to their shape), through the P/dS
 * workspace, which is required here (NULL: FFPA_ERR_INVALID_ARGUMENT; sizes whose workspace is
 * not available: FFPA_ERR_NOT_SUPPORTED). The mask enters P exactly as in the forward; dlse as in
 * ffpa_bwd.
 *   dmask  NULL, or (additive masks only) the bias gradient out: dS = P * (dP - delta), the
 *          gradient with respect to the scores, summed over the broadcast dimensions (those with
 *          a 0 stride), written packed row-major in the shape [s0 ? batch : 1, s1 ? hq : 1,
 *          s2 ? nq : 1, s3 ? nkv : 1] in q's dtype (fp32 sums, one rounding).
 */
ffpa_status_t ffpa_bwd_masked(const void* q, const void* k, const void* v, const void* o, const void* dout,
    const float* lse, const float* dlse, float* delta, void* dq, void* dk, void* dv,
    int batch, int hq, int hkv, int nq, int nkv, int d,
    const void* mask, ffpa_mask_kind_t mask_kind, const int64_t* mask_strides, void* dmask,
    ffpa_dtype_t dtype, float scale, int causal, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One stage of the dense backward, with exactly the arguments of ffpa_bwd plus `stage`:
 *   0 = preprocess (writes delta), 4 = P and dS, 1 = dK, 2 = dV, 3 = dQ,
 *   5 = dK, dV and dQ in one launch (P/dS workspace required, else FFPA_ERR_INVALID_ARGUMENT).
 * ffpa_bwd is these launches in the order 0, 4, 1, 2, 3, or 0, 4, 5 when ffpa_bwd_fused_products()
 * is 1 for its sizes and it has a workspace. Stages 4 and 1 read the delta written by
 * stage 0 (and so does stage 3 without a workspace); only stage 0 reads dlse. With a P/dS
 * workspace, stage 4 writes P and dS into it and stages 1, 2 and 3 read them: pass the same
 * workspace to all of them (a stage that reads a workspace that was not filled gives undefined
 * results). Without a workspace stage 4 launches nothing and stages 1, 2
 * and 3 are independent. The pages run dV before dK; the order of the products does not matter.
 * Lets a caller time or schedule the launches individually ("CuTe-DSL Backend", "Blackwell
 * status": the backward is separate launches). Returns FFPA_ERR_INVALID_ARGUMENT for another
 * stage.
 */
ffpa_status_t ffpa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o,
    const void* dout, const float* lse, const float* dlse, float* delta, void* dq, void* dk, void* dv,
    int batch, int hq, int hkv, int nq, int nkv, int d,
    ffpa_dtype_t dtype, float scale, int causal, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * 1 when ffpa_bwd with a P/dS workspace forms dK, dV and dQ in one launch (stage 5) for these dense
 * sizes, else 0. That is the case when each product pass alone would give fewer than two
 * workgroups per compute unit: a causal grid's heaviest tiles then set each pass's time, and one
 * combined grid lets the light tiles of one pass run beside the heavy tiles of another ("CuTe-DSL
 * Backend", "Blackwell status": the dV, dK and dQ stages are independent once dS is known). The
 * result is the same as stages 1, 2 and 3 bit for bit. Host function.
 */
int ffpa_bwd_fused_products(int batch, int hq, int hkv, int nq, int nkv, int d);

/*
 * Packed (THD) varlen forward ("CuTe-DSL Backend", "Varlen (packed THD) API").
 *   q [total_q, hq, d]; k, v [total_k, hkv, d]; o [total_q, hq, d]; lse [hq, total_q] fp32.
 *   cu_seqlens_q [batch+1], cu_seqlens_k [batch+1]: device int32, start at 0, non-decreasing,
 *     end at total_q / total_k. cu_seqlens_k == NULL means cu_seqlens_k = cu_seqlens_q (then
 *     total_k must equal total_q, else FFPA_ERR_INVALID_ARGUMENT).
 *   max_seqlen_q / max_seqlen_k bound every sequence length (they size the launch grid).
 * Sequence s attends queries [cu_q[s], cu_q[s+1]) to keys [cu_k[s], cu_k[s+1]); sequences of
 * length 0 are allowed. The device contents of cu_seqlens are not read on the host: contents
 * that break the rules above are undefined behaviour.
 */
ffpa_status_t ffpa_varlen_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    int batch, int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
    int hq, int hkv, int d, ffpa_dtype_t dtype, float scale, int causal, hipStream_t stream);

/*
 * Bytes of the optional P/dS workspace of ffpa_varlen_bwd for any cu_seqlens consistent with the
 * totals and max_seqlen values: 2 * hq * total_k * round_up(max_seqlen_q, 8) * 2, two blocks
 * (dS, then P), each bounding the packed per-sequence layout (sequence by sequence, then head,
 * then key row of round_up(Lq, 8) queries); 0 when not available (see ffpa_bwd_workspace_bytes).
 * Host function.
 */
size_t ffpa_varlen_bwd_workspace_bytes(int hq, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k);

/*
 * Exact bytes of the same workspace for the given sequence lengths: 2 * hq * sum_s Lk_s *
 * round_up(Lq_s, 8) * 2, from HOST copies of cu_seqlens (cu_seqlens_k_host NULL: the q ones).
 * 0 when the copies break the cu_seqlens rules of ffpa_varlen_fwd for these totals and max
 * lengths, or when the workspace is not available. Host function.
 */
size_t ffpa_varlen_bwd_workspace_bytes_exact(int hq, int batch, const int32_t* cu_seqlens_q_host,
    const int32_t* cu_seqlens_k_host, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k);

/*
 * Packed (THD) varlen backward ("CuTe-DSL Backend", "Varlen (packed THD) API": the packed call
 * with autograd; "Blackwell status": preprocess, dV, dK, dQ). Arguments as ffpa_varlen_fwd plus
 * o, dout [total_q, hq, d], the forward's lse [hq, total_q], dlse [hq, total_q] fp32 or NULL (as
 * in ffpa_bwd), a caller-owned fp32 workspace delta [hq, total_q], the outputs dq [total_q, hq, d],
 * dk, dv [total_k, hkv, d], and the optional P/dS workspace.
 *   cu_seqlens_q_host, cu_seqlens_k_host: NULL, or host copies of the device cu_seqlens (k NULL:
 *     the q ones). With them the P/dS workspace needs only the exact size
 *     (ffpa_varlen_bwd_workspace_bytes_exact), the copies are checked on the host (a bad copy is
 *     FFPA_ERR_INVALID_ARGUMENT) and must equal the device contents (else undefined behaviour);
 *     without them it needs ffpa_varlen_bwd_workspace_bytes.
 */
ffpa_status_t ffpa_varlen_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
    const float* lse, const float* dlse, float* delta, void* dq, void* dk, void* dv,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    const int32_t* cu_seqlens_q_host, const int32_t* cu_seqlens_k_host,
    int batch, int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
    int hq, int hkv, int d, ffpa_dtype_t dtype, float scale, int causal,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Human-readable name of a status code; never NULL. */
const char* ffpa_status_string(ffpa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* FFPA_H_ */
