/*
 * xfa — fused causal flash-attention, forward and backward, for MI355X
 * (gfx950).  Plain C ABI of libxfa.so.
 *
 * The operation (xtrain T14 "Fused Flash-Attention Kernel" design doc,
 * section "What flash-attention is"): for each head bh of B*H heads,
 *   out = softmax(mask(Q K^T * scale)) V,
 * where the causal mask hides key j from query i when j > i (positions count
 * from 0 within each sequence, queries and keys share positions).  The
 * forward also returns L_i = ln(sum_j exp(s_ij)) over the unmasked scaled
 * logits s_ij (the logsumexp the backward needs; section "Key Design Decision
 * 2").  The backward gets dQ, dK, dV of the loss sum(dO * out) by recomputing
 * p_ij = exp(s_ij - L_i) and using D_i = sum_d dO_i[d] O_i[d] (sections
 * "What flash-attention is", backward part, and "Key Design Decision 3").
 * No S x S buffer is ever allocated or written.
 *
 * Conventions shared by every entry point
 *   Layout    Q, K, V, O, dO, dQ, dK, dV: contiguous row-major [B, H, S, hd]
 *             (the same as [B*H*S, hd] rows; row r is query r % S of head
 *             r / S) in the element type `dtype`.  L and D: contiguous
 *             [B, H, S] float32.
 *   dtype     XFA_DTYPE_F32: every tensor float32.  XFA_DTYPE_BF16: the
 *             [.., hd] tensors bfloat16, L and D float32; arithmetic always
 *             accumulates in float32.
 *   Sizes     B, H, S >= 0 and hd in {16, 32, 64, 128}.  If B, H or S is 0
 *             the call does nothing and returns XFA_OK (pointers unused).
 *   Pointers  device pointers (hipMalloc'ed or equivalent) of the calling
 *             process's current device, 16-byte aligned.  Outputs must not
 *             overlap inputs or each other.  The caller owns every buffer;
 *             the library never allocates, frees or synchronises.
 *   scale     finite and > 0 (typically 1/sqrt(hd)).
 *   causal    1 = causal mask (tiles wholly above the diagonal are skipped),
 *             0 = no mask.
 *   stream    a hipStream_t passed as void*; NULL is the default stream.  All
 *             work is enqueued on it and the call returns without waiting.
 *   Errors    a status is returned, nothing is thrown.  Argument checks are
 *             made before any GPU call, so an error other than XFA_ERR_HIP
 *             means nothing was enqueued.  XFA_ERR_HIP reports a failed launch;
 *             faults during execution surface at the caller's next
 *             synchronisation.
 *   Threads   the functions keep no state and may be called concurrently on
 *             different streams with disjoint buffers.
 */
#ifndef XFA_H
#define XFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  XFA_DTYPE_F32 = 0,
  XFA_DTYPE_BF16 = 1
} xfa_dtype_t;

typedef enum {
  XFA_OK = 0,
  XFA_ERR_INVALID_ARGUMENT = 1, /* null or misaligned pointer, negative size, bad scale/causal/dtype */
  XFA_ERR_UNSUPPORTED = 2,      /* hd not in {16,32,64,128}, S > 2^30, (S+256)*hd*4 >= 2^31, or B*H*ceil(S/128) >= 2^24 (workgroups of one dispatch) */
  XFA_ERR_HIP = 3               /* a kernel launch failed */
} xfa_status_t;

/* Forward (T14 design doc, "What flash-attention is": the online-softmax
 * recurrence over KV tiles, out = acc / l, L = m + log l).
 *   in : q, k, v   [B,H,S,hd] dtype
 *   out: out       [B,H,S,hd] dtype
 *        lse       [B,H,S] float32, natural-log logsumexp of each query's
 *                  scaled, masked logits                                      */
xfa_status_t xfa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                     int64_t B, int64_t H, int64_t S, int64_t hd, float scale, int causal,
                     int dtype, void* stream);

/* Backward preprocess (T14 design doc, "Key Design Decision 3": D_i =
 * sum_d dO_i[d] * O_i[d], one O(N) pass before the backward).
 *   in : out, dout [B,H,S,hd] dtype (out as returned by xfa_fwd)
 *   out: delta     [B,H,S] float32
 * scale and causal do not enter D; they are checked like everywhere else so
 * that the three calls share one argument tail.                              */
xfa_status_t xfa_bwd_preprocess(const void* out, const void* dout, float* delta,
                                int64_t B, int64_t H, int64_t S, int64_t hd, float scale,
                                int causal, int dtype, void* stream);

/* Device workspace xfa_bwd and xfa_bwd_dropout need for a shape, in bytes
 * (T14 design doc, "Module Layout": the backward FFI entry next to the
 * forward's; "Key Design Decisions" 3 and the escape hatches: dQ summed per
 * query row, dK/dV per key block).  dQ can be summed across key blocks by
 * fp32 atomics into such a workspace or formed by a separate query-outer
 * pass that owns its rows; this library ships the second (the minimum atomic
 * traffic of the first alone takes longer than the whole backward on
 * MI355X), so the result is 0 for every shape and dtype and the workspace
 * argument is never dereferenced.  Pure function of its arguments, no GPU
 * call; arguments are validated by xfa_bwd, not here.                       */
size_t xfa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t hd, int dtype);

/* Backward (T14 design doc, "What flash-attention is", backward part:
 * p = exp(s - L), dp = dO . V, ds = p (dp - D) scale; dQ += ds K,
 * dK += ds Q, dV += p dO).
 *   in : q, k, v, dout [B,H,S,hd] dtype; lse [B,H,S] from xfa_fwd;
 *        delta [B,H,S] from xfa_bwd_preprocess
 *   out: dq, dk, dv    [B,H,S,hd] dtype (fully overwritten)
 *   workspace          caller-owned device memory of at least
 *                      xfa_bwd_workspace_bytes(B, H, S, hd, dtype) bytes,
 *                      256-byte aligned, overlapping no other argument; may
 *                      be NULL when that size is 0 (always, in this build),
 *                      and is then not dereferenced.
 * Two kernels on `stream` (dK/dV, then dQ).  Each output element is produced
 * by exactly one workgroup (no atomics), so results are bitwise
 * reproducible.  On XFA_ERR_HIP the dK/dV kernel may have been enqueued
 * already; the outputs are then unspecified.                                */
xfa_status_t xfa_bwd(const void* q, const void* k, const void* v, const void* dout,
                     const float* lse, const float* delta, void* dq, void* dk, void* dv,
                     void* workspace, int64_t B, int64_t H, int64_t S, int64_t hd, float scale,
                     int causal, int dtype, void* stream);

/* Dropout on the attention probabilities (xtrain dropout design doc, section
 * "RNG: counter-based"; applied to P as inverted dropout): with
 * M_ij = keep_ij / (1 - p),  out = (P o M) V  and L unchanged.  Element
 * (head bh, query i, key j) has flat index n = (bh*S + i)*S + j and
 *   keep = (splitmix64(seed XOR (n * 0x9E3779B97F4A7C15 mod 2^64)) >> 40)
 *          >= ceil(p * 2^24),
 * which is the doc's float32 test (top 24 bits / 2^24 >= p); splitmix64(x)
 * is one step of Steele, Lea and Flood's generator from state x.  The mask
 * depends on (seed, n) only and is regenerated in the backward, never
 * stored.  The backward (same doc, "dropout node backward", by the chain
 * rule): dV = (P o M)^T dO, dP = M o (dO V^T), ds = p (dP - D) scale;
 * D = rowsum(dO * out) from xfa_bwd_preprocess on the dropped out is still
 * rowsum(P o dP), so the preprocess is unchanged.
 *   dropout_p  in [0, 1), finite; else XFA_ERR_INVALID_ARGUMENT.  p = 0
 *              runs the kernels without dropout (bitwise the plain calls).
 *   seed       any 64-bit value; the forward and the backward of one step
 *              must get the same seed, p, B, H, S.
 * Other arguments (the workspace included), layouts and errors as in xfa_fwd
 * and xfa_bwd.                                                               */
xfa_status_t xfa_fwd_dropout(const void* q, const void* k, const void* v, void* out, float* lse,
                             int64_t B, int64_t H, int64_t S, int64_t hd, float scale, int causal,
                             float dropout_p, uint64_t seed, int dtype, void* stream);

xfa_status_t xfa_bwd_dropout(const void* q, const void* k, const void* v, const void* dout,
                             const float* lse, const float* delta, void* dq, void* dk, void* dv,
                             void* workspace, int64_t B, int64_t H, int64_t S, int64_t hd,
                             float scale, int causal, float dropout_p, uint64_t seed, int dtype,
                             void* stream);

/* Static, NUL-terminated description of a status code.                       */
const char* xfa_status_string(xfa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* XFA_H */
