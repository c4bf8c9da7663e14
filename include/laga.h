/*
 * laga.h -- C ABI of the LAGA per-rank attention path on one MI355X (gfx950).
 *
 * The operations follow "A Training-Memory Regression in MLA Sequence
 * Parallelism: Why Megatron-Core Forbids Absorption, and LAGA -- a
 * Communication-Efficient Fix" (arXiv 2607.17644v1), cited as [LAGA §...].
 * A rank r of an SP group of size P owns the head shard
 * H_r = [r*h, (r+1)*h) with h = n_h / P [LAGA §3.3, Algorithm 1 input] and,
 * after the latent all-gather, holds the full-sequence latent and k_pe.  This
 * library runs everything that rank computes locally: the latent norm, the
 * head-shard up-projection, causal attention, and the backward of all three
 * [LAGA §3.3 Algorithm 1; §5.1; §5.2].  Collectives are not part of it.
 *
 * Conventions shared by every entry point
 *  - All arrays are dense, row-major, contiguous device memory owned by the
 *    caller.  The library allocates nothing, keeps no state between calls and
 *    is reentrant; calls on one stream are ordered by that stream.  The one
 *    exception is laga_attn_bwd_noalloc, whose workspace is a static device
 *    array of the library, shared by all its calls on a GPU (see there).
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *    enqueued asynchronously; device faults surface at the caller's next
 *    synchronisation.  Argument checks run on the host before any launch and
 *    enqueue nothing when they fail.
 *  - Every pointer must be non-NULL and 16-byte aligned (LAGA_ERR_ALIGN).
 *  - Outputs are overwritten, never accumulated into.
 *  - "in" dtype is dims->dtype: bfloat16 (raw 16-bit patterns) or float32.
 *    Every output that is compared with an fp64 reference is float32.
 *  - The attention mask is causal over global positions (key u <= query t),
 *    with no dropout, bias, softcap or window.
 *
 * Layouts (T = B*S tokens, h local heads, d_qk = d_nope + d_rope, C = d_nope + d_v)
 *   latent   [B, S, d_kv]  in        gathered latent (pre-norm)
 *   gamma    [d_kv]        in        RMSNorm weight
 *   latent_n [B, S, d_kv]  float32   L = gamma * latent * rstd
 *   rstd     [B, S]        float32   1 / sqrt(mean(latent^2) + eps)
 *   w_kv_b   [n_h, C, d_kv] in       full tensor; per head the d_nope K rows
 *                                    then the d_v V rows; rows of H_r are read
 *   q        [B, S, h, d_qk] in      nope part first, rope part already rotated
 *   k_pe     [B, S, d_rope] in       one band shared by every head
 *   k_nope   [B, S, h, d_nope] kv  see below
 *   v        [B, S, h, d_v]    kv
 * K/V storage ("kv"): float32 for LAGA_F32; fp16 for LAGA_BF16 +
 * LAGA_OPERANDS_FP16; for LAGA_BF16 + LAGA_OPERANDS_SPLIT an fp16 plane
 * hi = fp16(x) [B, S, h, d] followed by a byte plane [B, S, h, d] of OCP e4m3
 * values lo = e4m3((x - hi) * 2^LAGA_KV_LO_SHIFT) (round to nearest even,
 * saturated at +-448), the value being hi + lo * 2^-LAGA_KV_LO_SHIFT: about
 * 2^-15 relative for |x| < 256, fp16 accuracy beyond.
 *   o        [B, S, h, d_v]  float32
 *   lse      [B, h, S]       float32 natural-log sum of exp(scores) per query
 */
#ifndef LAGA_H
#define LAGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LAGA_OK = 0,
  LAGA_ERR_INVALID = 1,     /* NULL dims/pointer, B or S < 1, bad head split, eps <= 0 */
  LAGA_ERR_UNSUPPORTED = 2, /* head dims / dtype / precision combination not built */
  LAGA_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
  LAGA_ERR_HIP = 4,         /* the HIP runtime reported an error at launch */
  LAGA_ERR_WORKSPACE = 5    /* backward workspace missing or smaller than required */
} laga_status;

typedef enum { LAGA_F32 = 0, LAGA_BF16 = 1 } laga_dtype;

/* Scale exponent of the e4m3 low plane of split K/V storage (see above). */
#define LAGA_KV_LO_SHIFT 12

/*
 * Operand precision of the matrix-core contractions for LAGA_BF16 inputs.
 *  LAGA_OPERANDS_FP16:  K/V are stored as fp16; scores, probabilities and V
 *                       enter the MFMAs as single fp16 values (fp32 accumulate).
 *  LAGA_OPERANDS_SPLIT: K/V are stored as an fp16 hi plane plus an e4m3 low
 *                       plane, and every computed operand (L, K, V, P, dS,
 *                       and the fold operands) enters the MFMAs as a hi+lo
 *                       pair (fp16/bf16 hi; the K/V low terms of the forward
 *                       as e4m3 products), giving fp32-class results at
 *                       1.4-3x the matrix-core work.
 * LAGA_F32 inputs always use float32 MFMAs and float32 K/V (field ignored).
 * The backward needs the K/V, o and lse of a LAGA_OPERANDS_SPLIT forward.
 */
typedef enum { LAGA_OPERANDS_FP16 = 0, LAGA_OPERANDS_SPLIT = 1 } laga_precision;

/* Sizes in the paper's notation [LAGA §2.1, §3.3]. */
typedef struct {
  int64_t B;         /* batch */
  int64_t S;         /* full (gathered) sequence length */
  int32_t n_h;       /* total heads */
  int32_t sp_size;   /* P, SP degree; n_h % P == 0 */
  int32_t sp_rank;   /* r, 0 <= r < P */
  int32_t d_kv;      /* latent width */
  int32_t d_nope;    /* per-head non-positional q/k width */
  int32_t d_rope;    /* decoupled RoPE band width */
  int32_t d_v;       /* per-head value width */
  float eps;         /* RMSNorm epsilon (1e-6) */
  int32_t dtype;     /* laga_dtype of every "in" array */
  int32_t precision; /* laga_precision */
} laga_dims;

/*
 * Supported shapes: (d_kv, d_nope, d_rope, d_v) = (512, 128, 64, 128) with
 * LAGA_BF16 (DeepSeek-V3 head dims [LAGA §4.1]) and (64, 32, 16, 32) with
 * LAGA_F32.  Anything else returns LAGA_ERR_UNSUPPORTED.  Inputs must be
 * finite; bf16 inputs converted to fp16 operands must stay below 65504 in
 * magnitude.
 */

/* Bytes per logical element of k_nope / v for these dims, all planes counted:
 * 2 (fp16), 3 (fp16 + e4m3 low plane) or 4 (float32).  Returns 0 when the
 * dims are invalid or unsupported. */
size_t laga_kv_elem_bytes(const laga_dims* dims);

/*
 * Latent RMSNorm [LAGA §2.1 "kv = W_kv_b LN(latent)"; §3.3 Algorithm 1 norm
 * of the latent].  Per token t: rstd[t] = 1/sqrt(mean_j latent[t,j]^2 + eps),
 * latent_n[t,j] = gamma[j] * latent[t,j] * rstd[t].
 */
laga_status laga_latent_norm(const laga_dims* dims, const void* latent, const void* gamma,
                             float* latent_n, float* rstd, void* stream);

/*
 * Head-shard up-projection [LAGA §3.3 Algorithm 1 local up-projection; §5.1]:
 * for i in [0, h): k_nope[t,i,:] = W_kv_b[r*h+i, 0:d_nope, :] . latent_n[t,:]
 * and v[t,i,:] = W_kv_b[r*h+i, d_nope:C, :] . latent_n[t,:].  Output element
 * type is given by laga_kv_elem_bytes.
 */
laga_status laga_kv_up(const laga_dims* dims, const float* latent_n, const void* w_kv_b,
                       void* k_nope, void* v, void* stream);

/*
 * Causal attention forward of the h local heads [LAGA §3.3 Algorithm 1 scores,
 * softmax and output; §5.3 the k_pe band is shared by all heads]:
 * s[t,u] = (q_nope[t,i] || q_rope[t,i]) . (k_nope[u,i] || k_pe[u]) / sqrt(d_nope + d_rope)
 * for u <= t; o[t,i] = sum_u softmax_u(s) v[u,i]; lse[i,t] = ln sum_u exp(s[t,u]).
 */
laga_status laga_attn_fwd(const laga_dims* dims, const void* q, const void* k_nope,
                          const void* k_pe, const void* v, float* o, float* lse, void* stream);

/*
 * The forward with the up-projection fused into the attention [LAGA §4.7
 * Limitations, fused up-projection kernel; §8 Discussion, open direction (i)]:
 * o and lse as laga_latent_norm + laga_kv_up + laga_attn_fwd compute them,
 * from the raw latent, without materialising k_nope / v in their own layout.
 * Only for LAGA_BF16 inputs at the V3 head dims with LAGA_OPERANDS_FP16 (the
 * forward-only mode: the normalised latent and W_kv_b's head shard are rounded
 * to fp16, so |gamma * latent / rms| and |W_kv_b| must stay below 65504);
 * anything else returns LAGA_ERR_UNSUPPORTED.
 * Layouts: q [B,S,h,d_qk], latent [B,S,d_kv], gamma [d_kv], k_pe [B,S,d_rope],
 * w_kv_b [n_h, d_nope+d_v, d_kv] (all bfloat16; rows r*h .. r*h+h-1 of w_kv_b
 * read); o [B,S,h,d_v] and lse [B,h,S] float32.
 * workspace: device memory of at least
 * laga_attn_fwd_fused_workspace_bytes(dims) bytes (16-byte aligned), owned by
 * the caller, whose contents need no initialisation and are overwritten:
 * 672 bytes per token and local head (K, V and rope rows, padded as the
 * attention's LDS tiles) with S rounded up to 256, 1 KB per token and 256 KB
 * per local head (197 MB at S = 16384, h = 16), plus 270 KB per split
 * 256-query tile and local head (35 MB at S = 4096, h = 16): a query tile with
 * more key blocks than the even share of all tiles' work per compute unit
 * runs as two tasks over the halves of its keys, merged afterwards (short
 * sequences only).  Two launches on
 * `stream` (three when tiles are split); calls that share a workspace must not
 * overlap in time.
 */
size_t laga_attn_fwd_fused_workspace_bytes(const laga_dims* dims);
laga_status laga_attn_fwd_fused(const laga_dims* dims, const void* q, const void* latent,
                                const void* gamma, const void* k_pe, const void* w_kv_b,
                                float* o, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * Absorbed form (B2) forward of the h local heads, the baseline that the
 * pages port from inference to training [LAGA §3.2 (B2), Fig. 2; §4.3 the
 * memory it costs].  W_kv_b's K half is folded into the query, attention runs
 * against the shared latent, and the V half is applied afterwards:
 *   q_abs[t,i,c] = sum_n q_nope[t,i,n] W[i,n,c]                        (absorb)
 *   s[t,i,u]     = (q_abs[t,i] . L[u] + q_rope[t,i] . k_pe[u]) / sqrt(d_nope + d_rope), u <= t
 *   acc[t,i]     = sum_u softmax_u(s) L[u]                           (latent accumulator)
 *   o[t,i,d]     = sum_c acc[t,i,c] W[i, d_nope + d, c]              (un-absorb)
 * which equals laga_attn_fwd's o up to rounding (same scores).  Arrays:
 *   q, k_pe, w_kv_b  as for the LAGA path (bf16); latent_n from laga_latent_norm
 *   q_abs  [B,S,h,d_kv]          fp16    written: the absorbed query
 *   kx     [B,S,d_kv + d_rope]   fp16    written: fp16(L) || fp16(k_pe), shared by all heads
 *   acc    [B,S,h,d_kv]          float32 written: the normalised latent accumulator
 *   o      [B,S,h,d_v]           float32, lse [B,h,S] float32 (natural log)
 * q_abs and acc are the n_h * d_kv-wide intermediates whose activation memory
 * the pages measure; the caller owns them, as it owns LAGA's K/V.  Operands
 * enter the matrix cores as fp16 (the precision field is ignored).  LAGA_BF16
 * with the V3 head dims only; anything else returns LAGA_ERR_UNSUPPORTED.
 */
laga_status laga_absorbed_fwd(const laga_dims* dims, const void* q, const float* latent_n,
                              const void* k_pe, const void* w_kv_b, void* q_abs, void* kx,
                              float* acc, float* o, float* lse, void* stream);

/*
 * Workspace bytes laga_attn_bwd needs for these dims (0 if invalid).  It grows
 * linearly with the token count B * S (no S x S quantity is ever stored: both
 * attention-backward kernels rebuild the probabilities from lse): for
 * LAGA_BF16 at the V3 head dims about 2.2 KB per token and local head plus
 * 4.2 KB per token, and a fixed part for the dW_kv_b partial sums (at most
 * about 70 MB) -- 0.66 GiB at S = 16384, h = 16 and 4.9 GiB at S = 131072.
 */
size_t laga_attn_bwd_workspace_bytes(const laga_dims* dims);

/*
 * Backward of the rank-local path for the loss sum(d_o * o) [LAGA §5.2]:
 *   dq        [B,S,h,d_qk] float32
 *   d_latent  [B,S,d_kv]   float32  gradient w.r.t. the pre-norm gathered latent
 *                                   (this rank's partial; the cross-rank sum is a
 *                                   reduce-scatter outside this library)
 *   d_k_pe    [B,S,d_rope] float32  sum over the local heads (this rank's partial)
 *   d_w_kv_b  [n_h,C,d_kv] float32  rows of H_r written; other rows untouched
 *   d_gamma   [d_kv]       float32  this rank's partial
 * Inputs are those of the forward plus its o and lse (LAGA_OPERANDS_SPLIT for
 * LAGA_BF16), rstd from laga_latent_norm, and d_o [B,S,h,d_v] in the input
 * dtype.  workspace: device memory of at least laga_attn_bwd_workspace_bytes.
 */
laga_status laga_attn_bwd(const laga_dims* dims, const void* q, const void* latent,
                          const void* gamma, const float* rstd, const void* k_nope,
                          const void* k_pe, const void* v, const void* w_kv_b,
                          const float* o, const float* lse, const void* d_o, float* dq,
                          float* d_latent, float* d_k_pe, float* d_w_kv_b, float* d_gamma,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * laga_attn_bwd with stage timing, for tracing tools.  `events` holds
 * n_events hipEvent_t handles created by the caller; with n_events ==
 * LAGA_BWD_STAGES + 1 the library records events[i] on `stream` right before
 * stage i and events[LAGA_BWD_STAGES] after the last, so that
 * hipEventElapsedTime(events[i], events[i+1]) is the duration of stage i:
 *   0 delta = rowsum(d_o * o)     1 dK/dV attention kernel   2 dq attention kernel
 *   3 dk_pe head sum              4 fold into dL             5 fold into dW_kv_b (+ chunk sum)
 *   6 RMSNorm backward (+ dgamma reduction)
 * n_events == 0 behaves exactly like laga_attn_bwd; any other count returns
 * LAGA_ERR_INVALID.  Recording failures return LAGA_ERR_HIP.
 */
#define LAGA_BWD_STAGES 7
laga_status laga_attn_bwd_traced(const laga_dims* dims, const void* q, const void* latent,
                                 const void* gamma, const float* rstd, const void* k_nope,
                                 const void* k_pe, const void* v, const void* w_kv_b,
                                 const float* o, const float* lse, const void* d_o, float* dq,
                                 float* d_latent, float* d_k_pe, float* d_w_kv_b, float* d_gamma,
                                 void* workspace, size_t workspace_bytes, void* const* events,
                                 int n_events, void* stream);

/*
 * laga_attn_bwd without a caller workspace, for callers that cannot allocate
 * device memory (code under stream/graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a static device array
 * of LAGA_NOALLOC_SCRATCH_BYTES inside the library: one copy on every GPU the
 * library runs on, held until the process ends; its address is looked up once
 * per device (hipGetSymbolAddress) on the first call made with that device
 * current.  The call allocates nothing.  Problems whose
 * laga_attn_bwd_workspace_bytes exceeds LAGA_NOALLOC_SCRATCH_BYTES (at the V3
 * head dims: more than about 5900 tokens with 16 local heads, or about 700
 * with 128) return LAGA_ERR_WORKSPACE; that and every other argument check
 * happen on the host before anything touches the GPU.  No part of
 * the scratch needs to start at zero (every stage writes its region before it
 * is read).  All calls on one GPU share its scratch: calls that can overlap
 * in time on one GPU (different streams, or host threads) race, so the caller
 * serialises them.  Arguments and results are those of laga_attn_bwd.
 */
#define LAGA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
laga_status laga_attn_bwd_noalloc(const laga_dims* dims, const void* q, const void* latent,
                                  const void* gamma, const float* rstd, const void* k_nope,
                                  const void* k_pe, const void* v, const void* w_kv_b,
                                  const float* o, const float* lse, const void* d_o, float* dq,
                                  float* d_latent, float* d_k_pe, float* d_w_kv_b, float* d_gamma,
                                  void* stream);

/*
 * Backward of the absorbed form (B2) [LAGA §3.2 (B2), Fig. 2; the baseline
 * whose training cost §4.3-4.4 measure]: gradients of sum(d_o * o) for the o
 * of laga_absorbed_fwd, taken through B2's own steps (un-absorb, latent
 * attention, absorb):
 *   d_acc = dO W^v,  dP = d_acc L^T,  dS = P (dP - rowsum(P dP)),
 *   d_q_abs = dS L / sqrt(d_qk),  dq_rope = dS k_pe / sqrt(d_qk),
 *   dL = P^T d_acc + dS^T q_abs / sqrt(d_qk),  dk_pe = sum over heads dS^T q_rope / sqrt(d_qk),
 *   dq_nope = d_q_abs W^k^T,  dW^k = q_nope^T d_q_abs,  dW^v = dO^T acc,
 * then the RMSNorm's backward.  The outputs equal laga_attn_bwd's (the two
 * forms are the same function): dq [B,S,h,d_qk], d_latent [B,S,d_kv], d_k_pe
 * [B,S,d_rope], the rows r*h .. r*h+h-1 of d_w_kv_b [n_h,C,d_kv] (other rows
 * untouched) and d_gamma [d_kv], all float32.  Inputs (bfloat16 unless noted):
 * q, latent, gamma, rstd (float32, from laga_latent_norm), k_pe, w_kv_b and
 * d_o [B,S,h,d_v].  Every product keeps bf16 hi + lo terms (fp32-class
 * accuracy); the S x S scores, probabilities and score gradients are
 * materialised one chunk of query rows at a time, and q_abs, lse, delta and
 * acc are recomputed from that chunk's scores at this accuracy rather than
 * taken from the fp16-operand forward (whose rounding of acc alone would cost
 * the dW_kv_b bar).  LAGA_BF16 inputs at the V3 head dims only (else
 * LAGA_ERR_UNSUPPORTED).  workspace (16-byte aligned, owned by the caller,
 * contents irrelevant): laga_absorbed_bwd_workspace_bytes(dims) bytes give the
 * default chunks, about 8.7 KB per token and local head, 4.4 KB per token, and
 * up to 1 GiB of chunk buffers (3.6 GB at S = 16384, h = 16).  A smaller
 * workspace, down to laga_absorbed_bwd_min_workspace_bytes(dims) (chunks of 32
 * tokens), runs with the largest chunks that fit it: less memory, more
 * launches; below the minimum the call returns LAGA_ERR_WORKSPACE.  Results of
 * different chunkings agree to rounding (the order of the sums over chunks).
 */
size_t laga_absorbed_bwd_workspace_bytes(const laga_dims* dims);
size_t laga_absorbed_bwd_min_workspace_bytes(const laga_dims* dims);
laga_status laga_absorbed_bwd(const laga_dims* dims, const void* q, const void* latent,
                              const void* gamma, const float* rstd, const void* k_pe,
                              const void* w_kv_b, const void* d_o, float* dq, float* d_latent,
                              float* d_k_pe, float* d_w_kv_b, float* d_gamma, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Static, human-readable text of a status code. */
const char* laga_status_string(laga_status status);

#ifdef __cplusplus
}
#endif

#endif /* LAGA_H */
