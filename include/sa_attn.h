/*
 * sa_attn.h — streaming exact attention (online softmax) for AMD MI355X (gfx950).
 *
 * C ABI of libsa_attn.so.  Every computing entry point is asynchronous on the
 * caller's HIP stream; the library never allocates, frees or synchronises
 * device memory and keeps no state between calls except a cached device
 * property (compute-unit count) per device.
 *
 * What is computed.  For batch b, query head h (reading key/value head
 * h / (H_q / H_kv): consecutive grouping of query heads over KV heads, as the
 * "Attention API" page reshapes queries to (T, H_kv, G, D) in
 * compute_hybrid_attention_store), query row i and key j:
 *
 *   s[i,j]   = scale * dot(q[b,i,h,:], k[b,j,hk,:]) - slope[h] * |i + S_k - S_q - j|
 *   visible  = (!causal || j <= i + S_k - S_q) && (mask == NULL || mask[b,j] != 0)
 *   lse[i]   = log(sum over visible j of exp(s[i,j]))            (natural log)
 *   out[i,:] = sum over visible j of exp(s[i,j] - lse[i]) * v[b,j,hk,:]
 *
 * computed in one streaming sweep over key/value tiles with running float32
 * row maximum and row sum ("StreamAttention: Fused Online Softmax Attention",
 * section "Kernel Design (Fused Online Softmax)"; "Attention API" page,
 * online_softmax_attention).  A row with no visible key yields out = 0 and
 * lse = -inf, never NaN ("flash-attn-volta" page, section "Stability").
 * Causal alignment is bottom-right (the last query row sees every key); with
 * S_q == S_k it is the usual j <= i.
 *
 * Conventions shared by all entry points:
 *  - Tensors are dense, row-major, with the shapes given per argument.
 *  - q, k, v, out and the decode workspace must be 16-byte aligned; the mask
 *    and slopes need only their natural alignment.
 *  - Supported: D in {64, 128}; dtype SA_F16 or SA_BF16 (q, k, v and out all
 *    of that type); 1 <= H_kv <= H_q with H_q % H_kv == 0.
 *  - Inputs are read-only.  out and lse must not overlap any input.
 *  - Return value: SA_OK or an sa_status code.  All arguments are validated
 *    before anything is launched; on an error nothing is launched and the
 *    outputs are untouched.  sa_last_error() then holds a description.
 *    There is no fallback path: an unsupported request fails.
 *  - Calls on one stream are ordered; calls on different streams that write
 *    the same outputs or workspace race.
 */
#ifndef SA_ATTN_H
#define SA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, negative or inconsistent size */
  SA_ERR_UNSUPPORTED = 2,  /* valid request outside what the kernels implement (D, dtype) */
  SA_ERR_WORKSPACE = 3,    /* decode workspace missing or smaller than required */
  SA_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} sa_status;

typedef enum { SA_F16 = 0, SA_BF16 = 1 } sa_dtype;

/* hipStream_t without pulling HIP headers into C callers. */
typedef struct ihipStream_t* sa_stream_t;

/*
 * Attention forward (prefill), the operation of the "StreamAttention" page's
 * API Reference, forward(query, key, value, causal, return_lse,
 * attention_mask, alibi_slopes), with a boolean key-padding mask as in its
 * Quick Start, and the flash_attn_forward(..., return_softmax_lse) of the
 * "flash-attn-volta" page, section "Use".
 *
 *   q     [B, S_q, H_q, D]   dtype, device
 *   k, v  [B, S_k, H_kv, D]  dtype, device
 *   out   [B, S_q, H_q, D]   dtype, device; every element is written
 *   lse   [B, H_q, S_q]      float32, device, natural log; NULL = not written
 *   scale  multiplies q.k in float32 (callers usually pass 1/sqrt(D))
 *   causal 0 or 1 (bottom-right aligned, see above)
 *   key_padding_mask [B, S_k] uint8 device, nonzero = keep; NULL = all keep
 *   alibi_slopes     [H_q] float32 device; NULL = no bias.  The kernels add
 *                    a bias in units of 1 / |scale|, so with slopes the scale
 *                    must be nonzero with 1 / |scale| finite in float32
 *                    (SA_ERR_INVALID_ARG otherwise)
 *
 * B == 0 or S_q == 0 is a successful no-op.  S_k == 0 writes out = 0 and
 * lse = -inf.  Errors: SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_HIP.
 */
int sa_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                int B, int S_q, int S_k, int H_q, int H_kv, int D, float scale,
                int causal, const uint8_t* key_padding_mask, const float* alibi_slopes,
                int dtype, sa_stream_t stream);

/*
 * Block-sparse attention forward: sa_attn_fwd in which each block of 128
 * query rows attends only to the blocks of 128 keys selected for it (the
 * execution step of the "Stem: Rethinking Causal Information Flow in Sparse
 * Attention" page, section 2.3, with its default block_size of 128 from
 * section 6).  Key j is visible to row i when sa_attn_fwd's rules keep it
 * (causal, padding) and block_mask[b][h][i / 128][j / 128] is nonzero; the
 * result equals dense attention with that element mask (the page's
 * "pseudo-sparse" run), and only the selected key/value tiles are read.
 *
 *   block_mask [B, H_q, ceil(S_q / 128), ceil(S_k / 128)] uint8, device,
 *              nonzero = visit; may be NULL only when S_k == 0
 *   all other arguments, layouts and rules as in sa_attn_fwd
 *
 * A row left with no visible key gets out = 0 and lse = -inf.  Supports
 * S_k <= 262144 (SA_ERR_UNSUPPORTED beyond).  B == 0 or S_q == 0 is a
 * successful no-op.  Errors: SA_ERR_INVALID_ARG (also when out or lse
 * overlaps the block mask), SA_ERR_UNSUPPORTED, SA_ERR_HIP.
 */
int sa_attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* out, float* lse,
                             int B, int S_q, int S_k, int H_q, int H_kv, int D, float scale,
                             int causal, const uint8_t* key_padding_mask,
                             const float* alibi_slopes, const uint8_t* block_mask, int dtype,
                             sa_stream_t stream);

/*
 * Attention forward with an additive float mask and dropout ("StreamAttention:
 * Fused Online Softmax Attention" page, "Recent Updates": boolean/additive
 * masks, dropout and deterministic Philox seeding; "API Reference":
 * attention_mask and dropout_p).  Arguments and rules as in sa_attn_fwd,
 * plus:
 *
 *   attn_bias  float32, device, or NULL: element (b, h, i, j) at
 *              attn_bias[b * bias_stride_b + h * bias_stride_h
 *                        + i * bias_stride_q + j],
 *              added to the scaled score of query row i and key j next to
 *              the ALiBi bias; -inf hides the key.  Strides are in elements,
 *              non-negative multiples of 4 (0 broadcasts that axis); the
 *              pointer is 16-byte aligned.  Entries must not be +inf or NaN.
 *              As for alibi_slopes, a bias needs a nonzero scale with
 *              1 / |scale| finite (SA_ERR_INVALID_ARG otherwise).
 *   dropout_p  in [0, 1); 0 turns dropout off.  A probability P[i, j] of
 *              (batch b, query head h) is kept when 16-bit half
 *              (j mod 64) / 32 (0 = low) of word (j mod 4) of
 *              Philox4x32-10 (Salmon et al., SC'11) with counter
 *              (8 (j / 64) + (j mod 32) / 4, i, b * H_q + h, offset) and key
 *              (seed low word, seed high word) is at least
 *              floor(dropout_p * 2^16), so the drop probability is dropout_p
 *              rounded down to a multiple of 2^-16; the output is
 *              sum_j P[i, j] keep[i, j] v_j / (1 - dropout_p).  lse is that
 *              of the softmax before dropout.
 *   seed, offset: the generator's key and fourth counter word (advance
 *              offset between calls that share a seed).
 *
 * Runs workgroups of four waves, or with dropout under the causal rule and
 * without ALiBi eight waves in two groups; with attn_bias NULL and dropout_p
 * 0 the call is sa_attn_fwd's.  B == 0 or S_q == 0 is a successful no-op.
 * Errors: SA_ERR_INVALID_ARG (also for a dropout_p outside [0, 1), bad bias
 * strides or alignment, out/lse overlapping the bias), SA_ERR_UNSUPPORTED,
 * SA_ERR_HIP.
 */
int sa_attn_fwd_ext(const void* q, const void* k, const void* v, void* out, float* lse,
                    int B, int S_q, int S_k, int H_q, int H_kv, int D, float scale,
                    int causal, const uint8_t* key_padding_mask, const float* alibi_slopes,
                    const float* attn_bias, int64_t bias_stride_b, int64_t bias_stride_h,
                    int64_t bias_stride_q, double dropout_p, uint64_t seed, uint32_t offset,
                    int dtype, sa_stream_t stream);

/*
 * Bytes of device workspace sa_attn_decode needs for these sizes (an upper
 * bound that holds for every H_kv dividing H_q).  Pure host arithmetic: no
 * HIP call.  Returns 0 when a size is negative or the result would overflow.
 */
size_t sa_attn_decode_workspace_size(int B, int H_q, int S_k, int D);

/*
 * Single-token attention over a key/value cache (S_q = 1), split over the key
 * axis: each split streams its keys once for up to 16 of the H_q / H_kv
 * query heads that share a KV head and writes a normalised partial output and
 * its log-sum-exp to the workspace; a second kernel merges the splits of each
 * (batch, query head) with log-sum-exp weights into out and lse
 * ("StreamAttention" page, "Engine Direction": partial online-softmax states
 * merged in a second kernel; "Distributed and Long-Context Variants":
 * log-sum-exp weighted combining).  The result equals sa_attn_fwd with
 * S_q = 1 (for which the bottom-right causal rule hides nothing).
 *
 *   q        [B, 1, H_q, D]    dtype, device
 *   k_cache  [B, S_k, H_kv, D] dtype, device
 *   v_cache  [B, S_k, H_kv, D] dtype, device
 *   out      [B, 1, H_q, D]    dtype, device
 *   lse      [B, H_q, 1]       float32, device; NULL = not written
 *   key_padding_mask [B, S_k] uint8 (nonzero = keep) or NULL
 *   alibi_slopes [H_q] float32 or NULL; the bias is -slope * (S_k - 1 - j)
 *   workspace, workspace_bytes: caller-owned device scratch of at least
 *     sa_attn_decode_workspace_size(B, H_q, S_k, D) bytes, 16-byte aligned;
 *     its contents on entry do not matter and on return are unspecified.
 *     Calls that may run at the same time must not share a workspace.
 *   The scale must be nonzero, with 1 / |scale| finite, when alibi_slopes
 *   is given.
 *
 * B == 0 is a no-op; S_k == 0 writes out = 0, lse = -inf.  Errors:
 * SA_ERR_INVALID_ARG (also when one split would span 4 GiB or more of
 * k_cache), SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP.
 */
int sa_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                   void* out, float* lse, int B, int S_k, int H_q, int H_kv, int D,
                   float scale, const uint8_t* key_padding_mask, const float* alibi_slopes,
                   int dtype, void* workspace, size_t workspace_bytes, sa_stream_t stream);

/*
 * sa_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid allocation.  Same arguments, rules, kernels and
 * results as sa_attn_decode; the decode's partial results live in a 16 MiB
 * scratch array inside this library instead (each GPU holds its own copy
 * from the library's load until the process ends).  The call allocates and
 * frees nothing.
 *
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on
 * one GPU (different streams with no ordering between them) race and must
 * not be issued.  A shape whose partial results exceed the scratch
 * (B * H_q * splits * (D + 1) * 4 bytes, splits as sa_attn_decode_num_splits)
 * returns SA_ERR_UNSUPPORTED with a message; use sa_attn_decode with a
 * workspace for it.  Other errors as sa_attn_decode.
 */
int sa_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                           void* out, float* lse, int B, int S_k, int H_q, int H_kv, int D,
                           float scale, const uint8_t* key_padding_mask, const float* alibi_slopes,
                           int dtype, sa_stream_t stream);

/*
 * Bytes of device workspace sa_attn_decode_fused needs: 65536 bytes of
 * arrival counters followed by sa_attn_decode's partial area.  Pure host
 * arithmetic; returns 0 when a size is negative or the result would overflow.
 */
size_t sa_attn_decode_fused_workspace_size(int B, int H_q, int S_k, int D);

/*
 * sa_attn_decode as a single kernel (the "StreamAttention" page, "Seed-Only
 * Serving Wedge": at small batch the second launch of a split-then-merge
 * decode costs as much as the work, and a single-kernel split design is what
 * it calls for).  The splits are the same as sa_attn_decode's; each hands its
 * partial state over through the workspace and counts itself on its head
 * group's arrival counter (a device-scope atomic add), and the last split of
 * a group to arrive merges the group's partial states with log-sum-exp
 * weights in the same launch.  No workgroup waits for another.  Same
 * arguments, layouts, rules and result as sa_attn_decode, except the
 * workspace:
 *
 *   workspace  at least sa_attn_decode_fused_workspace_size(B, H_q, S_k, D)
 *              bytes, 256-byte aligned.  Its first 65536 bytes hold the
 *              arrival counters (32-bit, one per head group): they must be
 *              zero before the first call that uses this workspace, and
 *              every call that completes leaves them zero again, so calls of
 *              any shape can reuse it.  Calls sharing a workspace must be
 *              ordered (one stream); calls that may overlap need separate
 *              ones.
 *
 * Errors: SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED (more than 16384 head groups
 * B * H_kv * ceil(H_q / H_kv / 16), or partial outputs of 4 GiB or more: use
 * sa_attn_decode), SA_ERR_WORKSPACE, SA_ERR_HIP.
 */
int sa_attn_decode_fused(const void* q, const void* k_cache, const void* v_cache, void* out,
                         float* lse, int B, int S_k, int H_q, int H_kv, int D, float scale,
                         const uint8_t* key_padding_mask, const float* alibi_slopes, int dtype,
                         void* workspace, size_t workspace_bytes, sa_stream_t stream);

/* Number of key splits sa_attn_decode uses for these sizes on a device with
 * num_cu compute units (host arithmetic only; exposed for tests and tools). */
int sa_attn_decode_num_splits(int B, int S_k, int H_q, int H_kv, int num_cu);

/* Number of key splits sa_attn_decode_fused uses: that of sa_attn_decode,
 * capped at 64 per head group (the last split of a group merges all of the
 * group's partial results alone), then rounded to whole 128-key steps. */
int sa_attn_decode_fused_num_splits(int B, int S_k, int H_q, int H_kv, int num_cu);

/*
 * Bytes of device workspace sa_attn_bwd needs: one float2 per (batch, query
 * head, row), B * H_q * S_q * 8.  Pure host arithmetic; 0 for a negative
 * size or on overflow.
 */
size_t sa_attn_bwd_workspace_size(int B, int H_q, int S_q);

/*
 * Gradients of sa_attn_fwd's output: the single-sweep backward of the
 * "StreamAttention" page ("Recent Updates": recompute the score tiles from
 * the saved lse, stream dQ, dK and dV) and the quantities the
 * "flash-attn-volta" page checks ("Backward correctness").  With P the
 * attention probabilities over the visible keys (same causal rule, mask and
 * ALiBi bias as the forward, neither of which has a gradient):
 *   dv = P^T dout,  dS = P (dout V^T - rowsum(dout * out)),
 *   dq = scale dS K,  dk = scale dS^T q,
 * each KV head receiving the sum over the query heads that read it.
 *
 *   q, out, dout  [B, S_q, H_q, D]   dtype, device (out: the forward's output)
 *   k, v          [B, S_k, H_kv, D]  dtype, device
 *   lse           [B, H_q, S_q]      float32, device: the forward's lse
 *   dq            [B, S_q, H_q, D]   dtype, device, fully written
 *   dk, dv        [B, S_k, H_kv, D]  dtype, device, fully written
 *   other arguments as for sa_attn_fwd
 *   workspace, workspace_bytes: caller-owned device scratch of at least
 *     sa_attn_bwd_workspace_size(B, H_q, S_q) bytes, 16-byte aligned, when
 *     S_q > 0; contents on entry do not matter.
 *
 * The gradients accumulate in float32 in a fixed order (no atomics): the
 * same inputs give bit-identical outputs.  B == 0, or S_q == S_k == 0, is a
 * no-op; S_q == 0 writes dk = dv = 0 and S_k == 0 writes dq = 0.  Errors as
 * for sa_attn_fwd, plus SA_ERR_WORKSPACE; outputs must not overlap inputs,
 * each other or the workspace.
 */
int sa_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, int B, int S_q, int S_k, int H_q,
                int H_kv, int D, float scale, int causal, const uint8_t* key_padding_mask,
                const float* alibi_slopes, int dtype, void* workspace, size_t workspace_bytes,
                sa_stream_t stream);

/* Static description of a status code. */
const char* sa_status_string(int status);

/* Description of the last non-OK return on the calling thread ("" if none). */
const char* sa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SA_ATTN_H */
