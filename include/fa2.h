/*
 * fa2.h -- C ABI of the MI355X (gfx950) FlashAttention-2 library, libfa2.so.
 *
 * The operation is scaled dot-product attention computed blockwise, as the
 * article "Revolutionizing Web-Based AI: How a Plain JavaScript Prototype
 * Paved the Way for High-Performance WebGPU Flash Attention 2" describes in
 * its section "Translating to WGSL and Optimizing Passes": the forward pass
 * walks K and V block by block with the online-softmax state held in
 * registers and never writes the N x N attention matrix to global memory;
 * the backward pass rebuilds the attention weights from Q, K and the saved
 * log-sum-exp instead of reading a cached matrix.
 *
 * Definitions (per batch b and head h; i, j index rows of the sequence):
 *   S_ij  = scale * q_i . k_j, with S_ij = -inf for j > i when causal
 *   LSE_i = ln sum_j exp(S_ij)          (natural log, scaled masked logits)
 *   P_ij  = exp(S_ij - LSE_i)
 *   O_i   = sum_j P_ij v_j
 *   dQ, dK, dV = gradients of L = sum(O * dO) for the upstream gradient dO.
 *
 * Layout and ownership (every call):
 *   - q, k, v, o, dO, dq, dk, dv are DEVICE pointers to contiguous row-major
 *     [B, H, N, d] arrays of the element type `dtype` (FA2_F32: float,
 *     FA2_BF16: bfloat16, FA2_F16: IEEE binary16).  lse is a device float
 *     array [B, H, N].
 *   - Every pointer must be 16-byte aligned.  Outputs must not alias inputs
 *     or each other.
 *   - The caller owns every buffer (inputs, outputs, workspace).  The library
 *     allocates nothing and keeps no state between calls, apart from the
 *     static per-GPU workspace of fa2_backward_noalloc (below).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work and return; results are valid once the stream
 *     has completed it.  Calls are reentrant and thread-safe.
 *
 * Kernel choice: the 16-bit types at d = 128 and d = 64 run tuned kernels
 * (direct loads into swizzled LDS rings); with the environment variable
 * FA2_FORCE_GENERIC set (to anything but "0") every call takes the generic
 * kernels instead, a second tiling of the same arithmetic (read at each
 * call; meant for cross-checking the two).
 *
 * Errors: every call returns an fa2_status and never aborts.  Arguments are
 * validated before any HIP call is made, so a rejected call touches no
 * device state.  B, H or N equal to 0 is a valid empty problem: FA2_OK and
 * nothing is launched.
 */
#ifndef FA2_H
#define FA2_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA2_F32 = 0, FA2_BF16 = 1, FA2_F16 = 2 } fa2_dtype;

typedef enum {
  FA2_OK = 0,
  FA2_ERR_INVALID_ARG = 1, /* null pointer, negative size, scale not finite
                              or zero, dtype not an fa2_dtype, size
                              overflow (N * d must stay below 2^31)        */
  FA2_ERR_UNSUPPORTED = 2, /* d not in {16, 32, 64, 128}, or a pointer not
                              16-byte aligned                              */
  FA2_ERR_WORKSPACE = 3,   /* backward workspace NULL or too small         */
  FA2_ERR_LAUNCH = 4,      /* a HIP launch reported an error               */
  FA2_ERR_SCRATCH = 5      /* fa2_backward_noalloc: the problem needs more
                              workspace than its static buffer holds       */
} fa2_status;

/*
 * Forward pass.  Writes o [B,H,N,d] (dtype) and lse [B,H,N] (float, natural
 * log).  Arithmetic: the two products run on MFMA with fp32 accumulation
 * (bf16 operands for FA2_BF16, fp16 for FA2_F16, fp32 for FA2_F32); the
 * softmax state is fp32; in the 16-bit modes the weights P are rounded to
 * the element type (nearest even) before the second product and o is
 * rounded to nearest even (the backward likewise rounds dS).  The article
 * names half-precision floats as a source of rounding error to watch
 * (section "Numerical Stability and Loss Drift"); FA2_F16 is that type.
 * scale: the factor on q . k (commonly 1/sqrt(d)); must be finite and
 * nonzero.  A negative factor is computed as |scale| * (-q) . k (the query
 * fragments' sign bits flipped in registers, exact in every type).  Zero is
 * rejected: the kernels fold the factor into the exponent of every logit,
 * and a masked logit (-inf) times zero is not a number.
 * causal: nonzero keeps keys j <= i (top-left aligned).
 */
int fa2_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int N, int d, float scale, int causal, int dtype,
                void* stream);

/*
 * Bytes of device workspace fa2_backward needs for this problem (0 for an
 * empty one).  The workspace holds D = rowsum(dO * O) and LSE * log2(e),
 * each float [B,H,N] padded to 256 bytes, and, in fp32 when the problem
 * leaves few workgroups for long key or query ranges, fp32 partial sums of
 * dK, dV or dQ whose ranges were split over several workgroups (added in a
 * fixed order).  Its contents on entry do not matter and on return are
 * unspecified.  Returns 0 for invalid sizes.
 */
size_t fa2_backward_workspace_size(int B, int H, int N, int d, int dtype);

/*
 * Backward pass for the loss L = sum(O * dO).  o and lse must be the outputs
 * of fa2_forward for the same q, k, v, scale and causal.  Overwrites dq, dk,
 * dv (never accumulates into them).  Kernels, in stream order:
 *   1. a query-tile-parallel kernel that computes D_i = sum_k dO_ik O_ik
 *      (fp32; a row whose keys all lie in its first 32-key block takes
 *      sum_j P_ij dP_ij from that block instead, free of O's rounding) and
 *      LSE_i * log2(e) for its rows into the workspace, then recomputes P
 *      and dP and accumulates dQ in registers;
 *   2. a key-tile-parallel kernel that recomputes P from q, k and lse and
 *      accumulates dK and dV in registers.
 * No atomics: every output element is written once by one workgroup, or
 * summed from fp32 partials in a fixed order, so the results are the same
 * bits from run to run.
 * workspace / workspace_bytes: device buffer of at least
 * fa2_backward_workspace_size(B, H, N, d, dtype) bytes, 16-byte aligned.
 */
int fa2_backward(const void* q, const void* k, const void* v, const void* o,
                 const void* dO, const float* lse, void* dq, void* dk, void* dv,
                 int B, int H, int N, int d, float scale, int causal, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * One stage of fa2_backward, with exactly fa2_backward's arguments and
 * checks: stage 1 = the dQ kernel (writes dq, and D and LSE * log2(e) of
 * every row to the workspace), 2 = the dK/dV kernel (reads them; writes dk,
 * dv).  Enqueuing stages 1 and 2 in order on one stream is fa2_backward; the
 * split lets a caller record events around each kernel.  Any other stage:
 * FA2_ERR_INVALID_ARG.
 */
int fa2_backward_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                       const void* dO, const float* lse, void* dq, void* dk, void* dv, int B,
                       int H, int N, int d, float scale, int causal, int dtype, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Grouped-query and multi-query attention.  The article "Revolutionizing
 * Web-Based AI: How a Plain JavaScript Prototype Paved the Way for
 * High-Performance WebGPU Flash Attention 2" names grouped-query attention
 * as the next primitive to build (section "Next Frontiers in WebGPU ML",
 * "Broader Opset Support") without defining it; the reading taken: the
 * H query heads form H_kv consecutive groups of G = H / H_kv, and query
 * head h uses key/value head h / G (H_kv = 1: multi-query attention;
 * H_kv = H: exactly fa2_forward / fa2_backward).
 *
 * Same arguments, layouts and behaviour as the calls above except:
 *   H_kv   number of key/value heads; 1 <= H_kv and H_kv divides H (both 0
 *          when H is 0), else FA2_ERR_INVALID_ARG.
 *   k, v   [B, H_kv, N, d]; dk, dv (backward) [B, H_kv, N, d], each the sum
 *          of the gradients of the group's query heads, written once
 *          (overwritten, never accumulated into).
 *   q, o, dO, dq [B, H, N, d] and lse [B, H, N] as before.
 *   workspace  at least fa2_backward_workspace_size_ex(B, H, H_kv, N, d,
 *          dtype) bytes (which equals fa2_backward_workspace_size when
 *          H_kv = H).
 * The dK/dV kernel walks the query heads of a group inside one workgroup
 * per key tile.  When that leaves too few workgroups to fill the device
 * (bf16, d = 128), each group is split over S workgroups (S divides G) that
 * write fp32 partial sums into the workspace, and a second kernel of stage
 * 2 adds the S partials in a fixed order and rounds once.  No atomics either
 * way, so results are the same bits from run to run.
 */
size_t fa2_backward_workspace_size_ex(int B, int H, int H_kv, int N, int d, int dtype);

int fa2_forward_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int H_kv, int N, int d, float scale, int causal, int dtype,
                   void* stream);

int fa2_backward_ex(const void* q, const void* k, const void* v, const void* o,
                    const void* dO, const float* lse, void* dq, void* dk, void* dv,
                    int B, int H, int H_kv, int N, int d, float scale, int causal, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

int fa2_backward_stage_ex(int stage, const void* q, const void* k, const void* v, const void* o,
                          const void* dO, const float* lse, void* dq, void* dk, void* dv, int B,
                          int H, int H_kv, int N, int d, float scale, int causal, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa2_backward_ex for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels, results (the same bits as
 * fa2_backward_ex) and errors, without the workspace arguments: the
 * workspace is a static device array of FA2_NOALLOC_SCRATCH_BYTES bytes
 * (64 MiB) inside the library, one per GPU, placed when the library's code
 * object is loaded onto that GPU and held until the process ends.  The call
 * allocates nothing (no hipMalloc, no hipFree, no allocating library call);
 * on the first call on a device it looks up that device's copy with
 * hipGetSymbolAddress.  The current device must be the one that `stream`
 * and the tensors belong to.
 *
 * Limit: problems whose fa2_backward_workspace_size_ex exceeds
 * FA2_NOALLOC_SCRATCH_BYTES are rejected with FA2_ERR_SCRATCH before any HIP
 * call (D and LSE * log2(e) take 8 bytes per query row, so plain multi-head
 * problems fit up to about 8 M rows B * H * N; split grouped-query and fp32
 * walks add fp32 partial sums).  The buffer keeps the last call's contents;
 * every call writes all it reads, so nothing needs clearing.  All calls on
 * one GPU share the one buffer: calls whose work overlaps in time on that GPU
 * (other streams, other threads) race and give wrong results; serialise them
 * (one stream, or events between streams).
 */
#define FA2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int fa2_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dO, const float* lse, void* dq, void* dk, void* dv,
                         int B, int H, int H_kv, int N, int d, float scale, int causal, int dtype,
                         void* stream);

/*
 * Packed ragged batches (variable-length sequences).  The article's forward
 * pass runs one workgroup per batch entry, head and query tile (section
 * "Translating to WGSL and Optimizing Passes"); these calls let each batch
 * entry have its own length.  The reading taken (the pages say nothing about
 * ragged batches): B sequences packed one after the other along the token
 * axis of each head,
 *   q, o, dO, dq  [H, T, d];  k, v, dk, dv  [H_kv, T, d];  lse  [H, T],
 * sequence b occupying rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of every head;
 * attention (and causal masking, top-left) stays inside each sequence.
 *   cu_seqlens  DEVICE int32 [B + 1]: 0 = cu[0] <= cu[1] <= ... <= cu[B] <= T,
 *               4-byte aligned.  The library does not read it on the host;
 *               offsets outside [0, T] are clamped and lengths cut to
 *               max_seqlen, so inconsistent offsets give wrong results but no
 *               access outside the tensors.  Rows not covered by any sequence
 *               are neither read for results nor written.
 *   max_seqlen  the longest sequence, 0 <= max_seqlen <= T (sizes the grid).
 * Other arguments, arithmetic and errors as the fixed-length calls (H_kv as
 * in fa2_forward_ex).  Sequences of length 0 are allowed.
 */
int fa2_forward_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                       const int* cu_seqlens, int B, int H, int H_kv, int T, int max_seqlen, int d,
                       float scale, int causal, int dtype, void* stream);

size_t fa2_backward_workspace_size_varlen(int B, int H, int H_kv, int T, int max_seqlen, int d,
                                          int dtype);

int fa2_backward_varlen(const void* q, const void* k, const void* v, const void* o, const void* dO,
                        const float* lse, void* dq, void* dk, void* dv, const int* cu_seqlens, int B,
                        int H, int H_kv, int T, int max_seqlen, int d, float scale, int causal,
                        int dtype, void* workspace, size_t workspace_bytes, void* stream);

int fa2_backward_stage_varlen(int stage, const void* q, const void* k, const void* v, const void* o,
                              const void* dO, const float* lse, void* dq, void* dk, void* dv,
                              const int* cu_seqlens, int B, int H, int H_kv, int T, int max_seqlen,
                              int d, float scale, int causal, int dtype, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * Decoding: N_q new queries against a cache of N_k keys and values.  The
 * article "Revolutionizing Web-Based AI: How a Plain JavaScript Prototype
 * Paved the Way for High-Performance WebGPU Flash Attention 2" names
 * flash-decoding as a next primitive (section "Next Frontiers in WebGPU ML",
 * "Broader Opset Support") without defining it; the reading taken: the
 * forward pass's softmax attention with a rectangular score matrix, the
 * queries being the last N_q positions of the sequence, so with causal != 0
 * query i keeps keys j <= N_k - N_q + i (no mask for N_q = 1).
 *
 *   q, o   [B, H, N_q, d] (dtype); k, v [B, H_kv, N_k, d] (dtype), H_kv
 *          dividing H, query head h reading key/value head h / (H / H_kv);
 *   lse    [B, H, N_q] float, natural log, as fa2_forward.
 * Arithmetic as fa2_forward.  For FA2_BF16 and FA2_F16 with d = 128 or 64 the
 * cache is split into chunks walked by separate workgroups, and a second
 * kernel merges their normalised partial outputs with weights
 * exp(LSE_chunk - max) and rounds O once; the split depends only on the
 * sizes, so results are the same bits from run to run.  Every other
 * supported type and head size (as fa2_forward) runs the forward kernel with
 * the cache as its keys, unsplit.
 * N_k = 0 with N_q > 0, or causal with N_q > N_k: FA2_ERR_INVALID_ARG.
 * B, H or N_q = 0: no-op.
 * workspace: device memory of at least fa2_decode_workspace_size(...) bytes,
 * 16-byte aligned (the partial results); may be NULL when that size is 0.
 * Asynchronous on stream, like the other calls.
 */
size_t fa2_decode_workspace_size(int B, int H, int H_kv, int N_q, int N_k, int d, int dtype);

int fa2_decode(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int H_kv, int N_q, int N_k, int d, float scale, int causal,
               int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* fa2_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */
