// C ABI of the LAGA per-rank attention path: argument checks, workspace
// carving and kernel sequencing.  Declarations and contracts: include/laga.h.
#include "laga.h"

#include "launch.hpp"

#include <mutex>

namespace {

using laga::Shape;

constexpr int64_t kMaxTokens = int64_t(1) << 22;

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Fills `s` from `d`; returns LAGA_OK or the reason the dims are rejected.
laga_status check_dims(const laga_dims* d, Shape* s) {
  if (d == nullptr) return LAGA_ERR_INVALID;
  if (d->B < 1 || d->S < 1 || d->n_h < 1 || d->sp_size < 1) return LAGA_ERR_INVALID;
  if (d->n_h % d->sp_size != 0 || d->sp_rank < 0 || d->sp_rank >= d->sp_size) return LAGA_ERR_INVALID;
  if (!(d->eps > 0.f) || !(d->eps < 1.f)) return LAGA_ERR_INVALID;
  if (d->dtype != LAGA_F32 && d->dtype != LAGA_BF16) return LAGA_ERR_INVALID;
  if (d->precision != LAGA_OPERANDS_FP16 && d->precision != LAGA_OPERANDS_SPLIT) return LAGA_ERR_INVALID;
  if (d->B > kMaxTokens || d->S > kMaxTokens || d->B * d->S > kMaxTokens) return LAGA_ERR_UNSUPPORTED;
  const bool v3 = d->d_kv == 512 && d->d_nope == 128 && d->d_rope == 64 && d->d_v == 128;
  const bool tiny = d->d_kv == 64 && d->d_nope == 32 && d->d_rope == 16 && d->d_v == 32;
  if (!((d->dtype == LAGA_BF16 && v3) || (d->dtype == LAGA_F32 && tiny))) return LAGA_ERR_UNSUPPORTED;
  s->B = d->B;
  s->S = d->S;
  s->T = d->B * d->S;
  s->n_h = d->n_h;
  s->h = d->n_h / d->sp_size;
  s->head_lo = d->sp_rank * s->h;
  s->d_kv = d->d_kv;
  s->d_nope = d->d_nope;
  s->d_rope = d->d_rope;
  s->d_v = d->d_v;
  s->eps = d->eps;
  s->bf16 = d->dtype == LAGA_BF16;
  s->split = s->bf16 && d->precision == LAGA_OPERANDS_SPLIT;
  if (static_cast<int64_t>(s->h) * ((s->S + 127) / 128) * s->B > (int64_t(1) << 31)) return LAGA_ERR_UNSUPPORTED;
  return LAGA_OK;
}

laga_status from_hip(hipError_t e) {
  if (e == hipSuccess) return LAGA_OK;
  if (e == hipErrorNotSupported) return LAGA_ERR_UNSUPPORTED;
  return LAGA_ERR_HIP;
}

// Backward workspace regions, each 256-byte aligned, in float32 elements.
struct BwdLayout {
  size_t delta, cvt, lo8, dos, dkv, dkpe, dL, lp, dw, dg, total;  // byte offsets, total bytes
};

size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

BwdLayout bwd_layout(const Shape& s) {
  BwdLayout L;
  size_t off = 0;
  auto take = [&](size_t floats) {
    const size_t at = off;
    off += round256(floats * sizeof(float));
    return at;
  };
  L.delta = take(static_cast<size_t>(s.B) * s.h * s.S);
  // fp16 copies of q, dO and k_pe (bfloat16 inputs only), in float units.
  L.cvt = take(s.bf16 ? (static_cast<size_t>(s.T) * (s.h * (s.d_qk() + s.d_v) + s.d_rope) + 1) / 2 : 0);
  // e4m3 rows of q_nope and dO and their per-row scale bytes (split operands).
  L.lo8 = take(s.split ? (static_cast<size_t>(s.T) * s.h * (s.d_nope + s.d_v) + 3) / 4 + 2 * s.T * s.h : 0);
  // Maxima of |dO| per delta workgroup (4 rows) and the dO scale shift (bfloat16 inputs).
  L.dos = take(s.bf16 ? (static_cast<size_t>(s.T) * s.h + 3) / 4 + 64 : 0);
  L.dkv = take(static_cast<size_t>(s.T) * s.h * s.C());
  L.dkpe = take(static_cast<size_t>(s.h) * s.T * s.d_rope);
  L.dL = take(static_cast<size_t>(s.T) * s.d_kv);
  L.lp = take(static_cast<size_t>(s.T) * s.d_kv);  // bf16 hi/lo planes or fp32
  L.dw = take(laga::fold_dw_partial_floats(s));
  L.dg = take(laga::norm_bwd_partial_floats(s));
  L.total = off;
  return L;
}

// ------------------------------------------------ allocation-free backward
// Scratch of laga_attn_bwd_noalloc: a device array of fixed size, one copy per
// GPU the library runs on, held until the process ends.  Host code never uses
// the array's name as an address (in host code it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, once per
// device, and is what the kernels receive.
static __device__ __align__(256) char scratch[LAGA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (LAGA_OK), looked up on the first call
// on that device with the device current.
laga_status current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LAGA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return LAGA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LAGA_OK;
}

}  // namespace

extern "C" {

size_t laga_kv_elem_bytes(const laga_dims* dims) {
  Shape s;
  if (check_dims(dims, &s) != LAGA_OK) return 0;
  return !s.bf16 ? 4 : s.split ? 3 : 2;  // f32 | fp16 | fp16 + e4m3
}

laga_status laga_latent_norm(const laga_dims* dims, const void* latent, const void* gamma,
                             float* latent_n, float* rstd, void* stream) {
  Shape s;
  laga_status st = check_dims(dims, &s);
  if (st != LAGA_OK) return st;
  if (!latent || !gamma || !latent_n || !rstd) return LAGA_ERR_INVALID;
  if (!aligned16(latent) || !aligned16(gamma) || !aligned16(latent_n) || !aligned16(rstd)) return LAGA_ERR_ALIGN;
  return from_hip(laga::launch_norm_fwd(s, latent, gamma, latent_n, rstd, static_cast<hipStream_t>(stream)));
}

laga_status laga_kv_up(const laga_dims* dims, const float* latent_n, const void* w_kv_b, void* k_nope,
                       void* v, void* stream) {
  Shape s;
  laga_status st = check_dims(dims, &s);
  if (st != LAGA_OK) return st;
  if (!latent_n || !w_kv_b || !k_nope || !v) return LAGA_ERR_INVALID;
  if (!aligned16(latent_n) || !aligned16(w_kv_b) || !aligned16(k_nope) || !aligned16(v)) return LAGA_ERR_ALIGN;
  return from_hip(laga::launch_kv_up(s, latent_n, w_kv_b, k_nope, v, static_cast<hipStream_t>(stream)));
}

laga_status laga_attn_fwd(const laga_dims* dims, const void* q, const void* k_nope, const void* k_pe,
                          const void* v, float* o, float* lse, void* stream) {
  Shape s;
  laga_status st = check_dims(dims, &s);
  if (st != LAGA_OK) return st;
  if (!q || !k_nope || !k_pe || !v || !o || !lse) return LAGA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k_nope) || !aligned16(k_pe) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return LAGA_ERR_ALIGN;
  return from_hip(laga::launch_attn_fwd(s, q, k_nope, k_pe, v, o, lse, static_cast<hipStream_t>(stream)));
}

size_t laga_attn_fwd_fused_workspace_bytes(const laga_dims* dims) {
  Shape s;
  if (check_dims(dims, &s) != LAGA_OK) return 0;
  return laga::fused_fwd_workspace_bytes(s);
}

laga_status laga_attn_fwd_fused(const laga_dims* dims, const void* q, const void* latent, const void* gamma,
                                const void* k_pe, const void* w_kv_b, float* o, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream) {
  Shape s;
  laga_status st = check_dims(dims, &s);
  if (st != LAGA_OK) return st;
  const size_t need = laga::fused_fwd_workspace_bytes(s);
  if (need == 0) return LAGA_ERR_UNSUPPORTED;
  if (!q || !latent || !gamma || !k_pe || !w_kv_b || !o || !lse) return LAGA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(latent) || !aligned16(gamma) || !aligned16(k_pe) || !aligned16(w_kv_b) ||
      !aligned16(o) || !aligned16(lse))
    return LAGA_ERR_ALIGN;
  if (workspace == nullptr || workspace_bytes < need) return LAGA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LAGA_ERR_ALIGN;
  return from_hip(laga::launch_attn_fwd_fused(s, q, latent, gamma, k_pe, w_kv_b, o, lse, workspace,
                                              static_cast<hipStream_t>(stream)));
}

size_t laga_absorbed_bwd_workspace_bytes(const laga_dims* dims) {
  Shape s;
  if (check_dims(dims, &s) != LAGA_OK) return 0;
  return laga::absorbed_bwd_workspace_bytes(s);
}

size_t laga_absorbed_bwd_min_workspace_bytes(const laga_dims* dims) {
  Shape s;
  if (check_dims(dims, &s) != LAGA_OK) return 0;
  return laga::absorbed_bwd_min_workspace_bytes(s);
}

laga_status laga_absorbed_bwd(const laga_dims* dims, const void* q, const void* latent, const void* gamma,
                              const float* rstd, const void* k_pe, const void* w_kv_b, const void* d_o, float* dq,
                              float* d_latent, float* d_k_pe, float* d_w_kv_b, float* d_gamma, void* workspace,
                              size_t workspace_bytes, void* stream) {
  Shape s;
  laga_status st = check_dims(dims, &s);
  if (st != LAGA_OK) return st;
  const size_t need = laga::absorbed_bwd_min_workspace_bytes(s);
  if (need == 0) return LAGA_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, latent, gamma, rstd, k_pe, w_kv_b, d_o, dq, d_latent, d_k_pe, d_w_kv_b, d_gamma};
  for (const void* p : ptrs)
    if (p == nullptr) return LAGA_ERR_INVALID;
  for (const void* p : ptrs)
    if (!aligned16(p)) return LAGA_ERR_ALIGN;
  if (workspace == nullptr || workspace_bytes < need) return LAGA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LAGA_ERR_ALIGN;
  return from_hip(laga::launch_absorbed_bwd(s, q, latent, gamma, rstd, k_pe, w_kv_b, d_o, dq, d_latent, d_k_pe,
                                            d_w_kv_b, d_gamma, workspace, workspace_bytes,
                                            static_cast<hipStream_t>(stream)));
}

laga_status laga_absorbed_fwd(const laga_dims* dims, const void* q, const float* latent_n, const void* k_pe,
                              const void* w_kv_b, void* q_abs, void* kx, float* acc, float* o, float* lse,
                              void* stream) {
  Shape s;
  laga_status st = check_dims(dims, &s);
  if (st != LAGA_OK) return st;
  if (!s.bf16) return LAGA_ERR_UNSUPPORTED;  // built for the V3 head dims with bf16 inputs
  if (!q || !latent_n || !k_pe || !w_kv_b || !q_abs || !kx || !acc || !o || !lse) return LAGA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(latent_n) || !aligned16(k_pe) || !aligned16(w_kv_b) || !aligned16(q_abs) ||
      !aligned16(kx) || !aligned16(acc) || !aligned16(o) || !aligned16(lse))
    return LAGA_ERR_ALIGN;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e;
  if ((e = laga::launch_absorb_q(s, q, w_kv_b, q_abs, hs)) != hipSuccess) return from_hip(e);
  if ((e = laga::launch_absorbed_pack(s, latent_n, k_pe, kx, hs)) != hipSuccess) return from_hip(e);
  if ((e = laga::launch_absorbed_attn(s, q_abs, q, kx, acc, lse, hs)) != hipSuccess) return from_hip(e);
  return from_hip(laga::launch_unabsorb_o(s, acc, w_kv_b, o, hs));
}

size_t laga_attn_bwd_workspace_bytes(const laga_dims* dims) {
  Shape s;
  if (check_dims(dims, &s) != LAGA_OK) return 0;
  return bwd_layout(s).total;
}

}  // extern "C"

namespace {

// The backward behind laga_attn_bwd, laga_attn_bwd_traced and
// laga_attn_bwd_noalloc.  With from_scratch the workspace is the device's
// static scratch array; every argument and size is checked on the host before
// anything touches the GPU.
laga_status attn_bwd_impl(const laga_dims* dims, const void* q, const void* latent, const void* gamma,
                          const float* rstd, const void* k_nope, const void* k_pe, const void* v, const void* w_kv_b,
                          const float* o, const float* lse, const void* d_o, float* dq, float* d_latent,
                          float* d_k_pe, float* d_w_kv_b, float* d_gamma, void* workspace, size_t workspace_bytes,
                          bool from_scratch, void* const* events, int n_events, void* stream) {
  Shape s;
  laga_status st = check_dims(dims, &s);
  if (st != LAGA_OK) return st;
  if (n_events != 0 && (n_events != LAGA_BWD_STAGES + 1 || events == nullptr)) return LAGA_ERR_INVALID;
  if (n_events != 0)
    for (int i = 0; i < n_events; ++i)
      if (events[i] == nullptr) return LAGA_ERR_INVALID;
  if (s.bf16 && !s.split) return LAGA_ERR_UNSUPPORTED;  // the backward needs fp32-class K/V
  const void* ptrs[] = {q, latent, gamma, rstd, k_nope, k_pe, v, w_kv_b, o, lse, d_o,
                        dq, d_latent, d_k_pe, d_w_kv_b, d_gamma};
  for (const void* p : ptrs)
    if (p == nullptr) return LAGA_ERR_INVALID;
  for (const void* p : ptrs)
    if (!aligned16(p)) return LAGA_ERR_ALIGN;
  const BwdLayout L = bwd_layout(s);
  if (from_scratch) {
    if (L.total > LAGA_NOALLOC_SCRATCH_BYTES) return LAGA_ERR_WORKSPACE;
    if ((st = current_scratch(&workspace)) != LAGA_OK) return st;
    workspace_bytes = LAGA_NOALLOC_SCRATCH_BYTES;
  }
  if (workspace == nullptr || workspace_bytes < L.total) return LAGA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LAGA_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  float* delta = reinterpret_cast<float*>(ws + L.delta);
  void* dkv = ws + L.dkv;
  void* lp = ws + L.lp;
  float* dkpe = reinterpret_cast<float*>(ws + L.dkpe);
  float* dL = reinterpret_cast<float*>(ws + L.dL);
  float* dw = reinterpret_cast<float*>(ws + L.dw);
  float* dg = reinterpret_cast<float*>(ws + L.dg);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) -> hipError_t {
    return n_events ? hipEventRecord(static_cast<hipEvent_t>(events[i]), hs) : hipSuccess;
  };

  hipError_t e;
  if ((e = mark(0)) != hipSuccess) return from_hip(e);
  // bfloat16 inputs reach the attention kernels as exact fp16 copies.
  laga::BwdCopies cp;
  uint16_t* q16 = reinterpret_cast<uint16_t*>(ws + L.cvt);
  uint16_t* do16 = q16 + static_cast<size_t>(s.T) * s.h * s.d_qk();
  cp.q16 = q16;
  cp.do16 = do16;
  cp.kpe16 = do16 + static_cast<size_t>(s.T) * s.h * s.d_v;
  cp.q8 = ws + L.lo8;
  cp.do8 = ws + L.lo8 + static_cast<size_t>(s.T) * s.h * s.d_nope;
  cp.qsc = reinterpret_cast<int*>(ws + L.lo8 + static_cast<size_t>(s.T) * s.h * (s.d_nope + s.d_v));
  cp.osc = cp.qsc + s.T * s.h;
  cp.do_row_max = s.bf16 ? reinterpret_cast<float*>(ws + L.dos) : nullptr;
  cp.do_shift = s.bf16 ? reinterpret_cast<int*>(ws + L.dos) + (s.T * s.h + 3) / 4 : nullptr;
  if ((e = laga::launch_bwd_prep(s, o, q, d_o, k_pe, delta, cp, hs)) != hipSuccess) return from_hip(e);
  if (s.bf16) {
    q = cp.q16;
    d_o = cp.do16;
    k_pe = cp.kpe16;
  }
  if ((e = mark(1)) != hipSuccess) return from_hip(e);
  if ((e = laga::launch_attn_bwd_dkdv(s, q, k_nope, k_pe, v, lse, delta, d_o, cp, dkv, dkpe, hs)) != hipSuccess)
    return from_hip(e);
  if ((e = mark(2)) != hipSuccess) return from_hip(e);
  if ((e = laga::launch_attn_bwd_dq(s, q, k_nope, k_pe, v, lse, delta, d_o, cp.do_shift, s.split ? cp.osc : nullptr,
                                    dq, hs)) != hipSuccess)
    return from_hip(e);
  if ((e = mark(3)) != hipSuccess) return from_hip(e);
  if ((e = laga::launch_head_sum(s, dkpe, d_k_pe, hs)) != hipSuccess) return from_hip(e);
  if ((e = mark(4)) != hipSuccess) return from_hip(e);
  if ((e = laga::launch_fold_dl(s, dkv, w_kv_b, dL, hs)) != hipSuccess) return from_hip(e);
  if ((e = mark(5)) != hipSuccess) return from_hip(e);
  if ((e = laga::launch_norm_planes(s, latent, gamma, rstd, lp, hs)) != hipSuccess) return from_hip(e);
  if ((e = laga::launch_fold_dw(s, dkv, lp, dw, d_w_kv_b, hs)) != hipSuccess) return from_hip(e);
  if ((e = mark(6)) != hipSuccess) return from_hip(e);
  if ((e = laga::launch_norm_bwd(s, dL, latent, gamma, rstd, d_latent, dg, d_gamma, hs)) != hipSuccess)
    return from_hip(e);
  if ((e = mark(7)) != hipSuccess) return from_hip(e);
  return LAGA_OK;
}

}  // namespace

extern "C" {

laga_status laga_attn_bwd_traced(const laga_dims* dims, const void* q, const void* latent, const void* gamma,
                                 const float* rstd, const void* k_nope, const void* k_pe, const void* v,
                                 const void* w_kv_b, const float* o, const float* lse, const void* d_o, float* dq,
                                 float* d_latent, float* d_k_pe, float* d_w_kv_b, float* d_gamma, void* workspace,
                                 size_t workspace_bytes, void* const* events, int n_events, void* stream) {
  return attn_bwd_impl(dims, q, latent, gamma, rstd, k_nope, k_pe, v, w_kv_b, o, lse, d_o, dq, d_latent, d_k_pe,
                       d_w_kv_b, d_gamma, workspace, workspace_bytes, false, events, n_events, stream);
}

laga_status laga_attn_bwd(const laga_dims* dims, const void* q, const void* latent, const void* gamma,
                          const float* rstd, const void* k_nope, const void* k_pe, const void* v,
                          const void* w_kv_b, const float* o, const float* lse, const void* d_o,
                          float* dq, float* d_latent, float* d_k_pe, float* d_w_kv_b, float* d_gamma,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return laga_attn_bwd_traced(dims, q, latent, gamma, rstd, k_nope, k_pe, v, w_kv_b, o, lse, d_o, dq, d_latent,
                              d_k_pe, d_w_kv_b, d_gamma, workspace, workspace_bytes, nullptr, 0, stream);
}

laga_status laga_attn_bwd_noalloc(const laga_dims* dims, const void* q, const void* latent, const void* gamma,
                                  const float* rstd, const void* k_nope, const void* k_pe, const void* v,
                                  const void* w_kv_b, const float* o, const float* lse, const void* d_o, float* dq,
                                  float* d_latent, float* d_k_pe, float* d_w_kv_b, float* d_gamma, void* stream) {
  return attn_bwd_impl(dims, q, latent, gamma, rstd, k_nope, k_pe, v, w_kv_b, o, lse, d_o, dq, d_latent, d_k_pe,
                       d_w_kv_b, d_gamma, nullptr, 0, true, nullptr, 0, stream);
}

const char* laga_status_string(laga_status status) {
  switch (status) {
    case LAGA_OK: return "LAGA_OK";
    case LAGA_ERR_INVALID: return "LAGA_ERR_INVALID: invalid argument";
    case LAGA_ERR_UNSUPPORTED: return "LAGA_ERR_UNSUPPORTED: dims/dtype/precision not supported";
    case LAGA_ERR_ALIGN: return "LAGA_ERR_ALIGN: pointer not 16-byte aligned";
    case LAGA_ERR_HIP: return "LAGA_ERR_HIP: HIP launch error";
    case LAGA_ERR_WORKSPACE: return "LAGA_ERR_WORKSPACE: workspace missing or too small";
  }
  return "unknown laga_status";
}

}  // extern "C"
