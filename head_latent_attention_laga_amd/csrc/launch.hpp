// Host-side launchers of the LAGA kernels (internal; the public ABI is laga.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace laga {

// Validated sizes of one call.  h local heads start at global head `head_lo`.
struct Shape {
  int64_t B, S, T;  // T = B * S tokens
  int n_h, h, head_lo;
  int d_kv, d_nope, d_rope, d_v;
  float eps;
  bool bf16;   // inputs are bfloat16 (else float32)
  bool split;  // hi/lo split operands, float32 K/V (bf16 inputs only)
  int C() const { return d_nope + d_v; }
  int d_qk() const { return d_nope + d_rope; }
};

hipError_t launch_norm_fwd(const Shape& s, const void* latent, const void* gamma, float* L,
                           float* rstd, hipStream_t st);
hipError_t launch_kv_up(const Shape& s, const float* L, const void* w, void* k_nope, void* v,
                        hipStream_t st);
hipError_t launch_attn_fwd(const Shape& s, const void* q, const void* k_nope, const void* k_pe,
                           const void* v, float* o, float* lse, hipStream_t st);

// Fused forward (fp16 operands, bfloat16 inputs at the V3 head dims): the
// latent's RMSNorm, the head-shard up-projection and the attention in two
// launches, K/V passing through `workspace` as key-block images.  The error
// word (int at workspace + 32) is set if a consumer ever gave up waiting.
size_t fused_fwd_workspace_bytes(const Shape& s);  // 0: unsupported shape
hipError_t launch_attn_fwd_fused(const Shape& s, const void* q, const void* latent, const void* gamma,
                                 const void* k_pe, const void* w, float* o, float* lse, void* workspace,
                                 hipStream_t st);

// Backward pieces.  Workspace carving lives in the API layer.
// Copies of the bfloat16 inputs that the backward kernels read: exact fp16
// q16 [T,h,d_qk], do16 [T,h,d_v], kpe16 [T,d_rope] (taken in place of the
// inputs), and for split operands e4m3 rows q8 = e4m3(q_nope * 2^s)
// [T,h,d_nope], do8 = e4m3(dO * 2^s) [T,h,d_v] with one shift per row, whose
// E8M0 bytes 127 - s are qsc / osc [B,h,S] (int32).
// do16 holds dO * 2^g, with g (do_shift, one int) chosen from the maxima
// do_row_max [ceil(T*h / 4)] (one per delta workgroup of 4 rows) so that
// max |dO| * 2^g lies in [8, 16): the fp16
// copy keeps dO's relative precision at any gradient magnitude, and the
// attention-backward kernels undo the factor on their outputs.
struct BwdCopies {
  void* q16; void* do16; void* kpe16;
  void* q8; void* do8; int* qsc; int* osc;
  float* do_row_max; int* do_shift;
};
// delta = rowsum(dO * o) and, for bfloat16 inputs, the copies above.
hipError_t launch_bwd_prep(const Shape& s, const float* o, const void* q, const void* d_o, const void* k_pe,
                           float* delta, const BwdCopies& c, hipStream_t st);
hipError_t launch_attn_bwd_dkdv(const Shape& s, const void* q, const void* k_nope,
                                const void* k_pe, const void* v, const float* lse,
                                const float* delta, const void* d_o, const BwdCopies& c, void* dkv,
                                float* dk_pe_part, hipStream_t st);
// dq, recomputing P and dS from lse and delta.  q, k_pe, d_o: the fp16 copies
// (bfloat16 inputs) or the float32 inputs; k_nope, v: their first plane;
// do_row_scale: the E8M0 bytes of dO's e4m3 rows (BwdCopies::osc) or nullptr.
hipError_t launch_attn_bwd_dq(const Shape& s, const void* q, const void* k_nope, const void* k_pe, const void* v,
                              const float* lse, const float* delta, const void* d_o, const int* do_shift,
                              const int* do_row_scale, float* dq, hipStream_t st);
hipError_t launch_head_sum(const Shape& s, const float* part, float* out, hipStream_t st);
// dkv: [T, h, d_nope + d_v] as bf16 hi/lo planes (bf16 inputs) or one fp32 plane.
hipError_t launch_fold_dl(const Shape& s, const void* dkv, const void* w, float* dL, hipStream_t st);
size_t fold_dw_partial_floats(const Shape& s);
// lplanes: the normalised latent [T, d_kv] in the same plane format (launch_norm_planes).
hipError_t launch_fold_dw(const Shape& s, const void* dkv, const void* lplanes, float* partial, float* d_w,
                          hipStream_t st);
hipError_t launch_norm_planes(const Shape& s, const void* latent, const void* gamma, const float* rstd,
                              void* lplanes, hipStream_t st);
size_t norm_bwd_partial_floats(const Shape& s);

// Absorbed form (B2): q_abs [T, h, d_kv] fp16 = W^k^T q_nope per head; the
// latent attention over kx = fp16 [T, d_kv + d_rope] (L || k_pe) writing the
// normalised latent accumulator acc [T, h, d_kv] fp32 and lse [B, h, S]; and
// o [T, h, d_v] = W^v acc per head.
hipError_t launch_absorb_q(const Shape& s, const void* q, const void* w, void* q_abs, hipStream_t st);
hipError_t launch_absorbed_pack(const Shape& s, const float* L, const void* k_pe, void* kx, hipStream_t st);
hipError_t launch_absorbed_attn(const Shape& s, const void* q_abs, const void* q, const void* kx, float* acc,
                                float* lse, hipStream_t st);
hipError_t launch_unabsorb_o(const Shape& s, const float* acc, const void* w, float* o, hipStream_t st);
// Absorbed form (B2) backward: gradients of sum(dO * o) for laga_absorbed_fwd's
// output, every product in split (fp32-class) precision, the S x S quantities
// materialised one chunk of query rows at a time; lse, delta and acc are
// recomputed from the chunk's own scores.  Workspace: absorbed_bwd_workspace_bytes
// for the default chunks; any size down to absorbed_bwd_min_workspace_bytes
// (32-token chunks) runs with the largest chunks that fit (0: unsupported).
size_t absorbed_bwd_workspace_bytes(const Shape& s);
size_t absorbed_bwd_min_workspace_bytes(const Shape& s);
hipError_t launch_absorbed_bwd(const Shape& s, const void* q, const void* latent, const void* gamma,
                               const float* rstd, const void* k_pe, const void* w, const void* d_o, float* dq,
                               float* d_latent, float* d_k_pe, float* d_w, float* d_gamma, void* workspace,
                               size_t workspace_bytes, hipStream_t st);
// Its products (gemm.hip).
hipError_t launch_b2_planes(const Shape& s, const void* x, int64_t x_ld, int64_t x_z, int64_t w_row0,
                            const void* w, void* out, int64_t out_plane, int64_t out_ld, hipStream_t st);
hipError_t launch_b2_rows_keys(const void* rows, int64_t rows_plane, int64_t rows_ld, int64_t nrows, const void* keys,
                               int64_t keys_plane, int64_t nkeys, int64_t kdim, float* out, int64_t out_ld,
                               hipStream_t st);
// Products over rows into the key-side gradients; with few key tiles their K
// runs in up to B2_KG_SPLIT chunks into `part`, 2 b2_keygrad_chunks nkeys 576 floats.
constexpr int B2_KG_SPLIT = 8;
int b2_keygrad_chunks(int64_t nkeys, int64_t nrows);
hipError_t launch_b2_key_grads(const void* pp, const void* dsp, int64_t p_plane, int64_t ldu, int64_t nrows,
                               int64_t nkeys, const void* dacc_rows, int64_t dacc_plane, const void* qx_rows,
                               int64_t qx_plane, float* dL, float* dkpe, float* part, hipStream_t st);
// Products that contract over a chunk's keys run in at most B2_KSPLIT K
// chunks, each to its own fp32 partial, summed in a fixed order afterwards.
constexpr int B2_KSPLIT = 4;
int b2_key_chunks(int64_t nrows, int ncols, int64_t kpad);
hipError_t launch_b2_rows_by_keys(const void* ap, int64_t p_plane, int64_t ldu, int64_t nrows, int64_t kpad,
                                  const void* keys, int64_t keys_plane, int ncols, float* part, hipStream_t st);
hipError_t launch_b2_dq_nope(const Shape& s, const float* dqx, const void* w, float* dq, hipStream_t st);
size_t b2_dw_partial_floats(const Shape& s);
hipError_t launch_b2_dw(const Shape& s, const void* x, int64_t x_ld, int64_t x_z, const void* yp, int64_t y_plane,
                        float* partial, float* d_w, int64_t row0, hipStream_t st);
hipError_t launch_norm_bwd(const Shape& s, const float* dL, const void* latent, const void* gamma,
                           const float* rstd, float* d_latent, float* dgamma_part, float* d_gamma,
                           hipStream_t st);

}  // namespace laga
