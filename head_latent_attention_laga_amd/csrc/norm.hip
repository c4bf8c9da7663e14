// Latent RMSNorm forward and backward.
//
// Forward [LAGA §2.1 "kv = W_kv_b LN(latent)", §3.3 Algorithm 1 norm of the
// latent; RMS form with eps inside the square root and a learned gamma]:
//   rstd[t] = 1 / sqrt(mean_j x[t,j]^2 + eps),  L[t,j] = gamma[j] x[t,j] rstd[t]
// Backward (chain rule of the forward):
//   x_hat = x rstd, g = gamma * dL,
//   dx = rstd (g - x_hat * mean_j(g_j x_hat_j)),  dgamma = sum_t dL * x_hat.
//
// Both are HBM-bound: one 64-lane wavefront owns one token row of d_kv
// elements, each lane a contiguous run of d_kv/64 elements, so a wavefront
// reads the row with fully coalesced 16-byte loads and reduces it with
// cross-lane shuffles.  The dgamma reduction over tokens is deterministic:
// each workgroup keeps per-lane partial sums for a strided set of tokens and
// writes one partial row; a second kernel adds the partial rows in order.
#include "device.hpp"
#include "launch.hpp"

namespace laga {
namespace {

constexpr int kNormBlock = 256;
constexpr int kRowsPerBlock = kNormBlock / kWave;

template <int EPL>
__device__ __forceinline__ void load_run(const bf16_t* p, float* v) {
  if constexpr (EPL % 8 == 0) {
#pragma unroll
    for (int c = 0; c < EPL; c += 8) {
      u16x8 r = *reinterpret_cast<const u16x8*>(p + c);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[c + j] = bf16_to_f32(r[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j) v[j] = bf16_to_f32(p[j]);
  }
}

template <int EPL>
__device__ __forceinline__ void load_run(const float* p, float* v) {
  if constexpr (EPL % 4 == 0) {
#pragma unroll
    for (int c = 0; c < EPL; c += 4) {
      f32x4 r = *reinterpret_cast<const f32x4*>(p + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[c + j] = r[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j) v[j] = p[j];
  }
}

template <int EPL>
__device__ __forceinline__ void store_run(float* p, const float* v) {
  if constexpr (EPL % 4 == 0) {
#pragma unroll
    for (int c = 0; c < EPL; c += 4) {
      f32x4 r = {v[c], v[c + 1], v[c + 2], v[c + 3]};
      *reinterpret_cast<f32x4*>(p + c) = r;
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j) p[j] = v[j];
  }
}

template <class InT, int D>
__global__ __launch_bounds__(kNormBlock) void rmsnorm_fwd_kernel(const InT* __restrict__ x,
                                                                 const InT* __restrict__ gamma,
                                                                 float* __restrict__ L,
                                                                 float* __restrict__ rstd,
                                                                 int64_t T, float eps) {
  constexpr int EPL = D / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  float v[EPL], g[EPL];
  load_run<EPL>(x + t * D + lane * EPL, v);
  load_run<EPL>(gamma + lane * EPL, g);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) ss += v[j] * v[j];
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
#pragma unroll
  for (int j = 0; j < EPL; ++j) v[j] = g[j] * (v[j] * r);
  store_run<EPL>(L + t * D + lane * EPL, v);
  if (lane == 0) rstd[t] = r;
}

// Grid-strided over tokens; each workgroup writes one partial dgamma row.
template <class InT, int D>
__global__ __launch_bounds__(kNormBlock) void rmsnorm_bwd_kernel(
    const float* __restrict__ dL, const InT* __restrict__ x, const InT* __restrict__ gamma,
    const float* __restrict__ rstd, float* __restrict__ dx, float* __restrict__ dgamma_part,
    int64_t T) {
  constexpr int EPL = D / kWave;
  __shared__ float red[kRowsPerBlock][D];
  const int lane = threadIdx.x % kWave;
  const int wv = threadIdx.x / kWave;
  float g[EPL], acc[EPL];
  load_run<EPL>(gamma + lane * EPL, g);
#pragma unroll
  for (int j = 0; j < EPL; ++j) acc[j] = 0.f;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kRowsPerBlock;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wv; t < T; t += stride) {
    float xv[EPL], d[EPL];
    load_run<EPL>(x + t * D + lane * EPL, xv);
    load_run<EPL>(dL + t * D + lane * EPL, d);
    const float r = rstd[t];
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      xv[j] *= r;  // x_hat
      acc[j] += d[j] * xv[j];
      d[j] *= g[j];  // g = gamma * dL
      dot += d[j] * xv[j];
    }
    dot = wave_sum(dot) / static_cast<float>(D);
#pragma unroll
    for (int j = 0; j < EPL; ++j) d[j] = r * (d[j] - xv[j] * dot);
    store_run<EPL>(dx + t * D + lane * EPL, d);
  }
#pragma unroll
  for (int j = 0; j < EPL; ++j) red[wv][lane * EPL + j] = acc[j];
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += kNormBlock) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kRowsPerBlock; ++w) s += red[w][c];
    dgamma_part[static_cast<int64_t>(blockIdx.x) * D + c] = s;
  }
}

// out[c] = sum_p part[p, c] in a fixed order (deterministic): a workgroup owns
// kSumCols columns; thread group g adds rows g, g + kSumGroups, ... and the
// group sums are added in increasing g.
constexpr int kSumCols = 32, kSumGroups = kNormBlock / kSumCols;
__global__ __launch_bounds__(kNormBlock) void column_sum_kernel(const float* __restrict__ part,
                                                                float* __restrict__ out, int rows,
                                                                int cols) {
  __shared__ float red[kSumGroups][kSumCols];
  const int cl = threadIdx.x % kSumCols, g = threadIdx.x / kSumCols;
  const int c = blockIdx.x * kSumCols + cl;
  float s = 0.f;
  if (c < cols)
#pragma unroll 8  // the loads issue together; the sum keeps its order
    for (int p = g; p < rows; p += kSumGroups) s += part[static_cast<int64_t>(p) * cols + c];
  red[g][cl] = s;
  __syncthreads();
  if (g == 0 && c < cols) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < kSumGroups; ++i) t += red[i][cl];
    out[c] = t;
  }
}

// L = gamma * x * rstd, the normalised latent rebuilt from the saved rstd, as
// NS planes of the MFMA element type of the W_kv_b-gradient GEMM (bf16 hi + lo,
// or one fp32 plane); planes are `plane` elements apart.
template <class M, int NS, class InT, int D>
__global__ __launch_bounds__(kNormBlock) void norm_planes_kernel(const InT* __restrict__ x,
                                                                 const InT* __restrict__ gamma,
                                                                 const float* __restrict__ rstd,
                                                                 typename M::elem* __restrict__ out,
                                                                 int64_t T, int64_t plane) {
  typedef typename M::elem E;
  constexpr int EPL = D / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  float v[EPL], g[EPL];
  load_run<EPL>(x + t * D + lane * EPL, v);
  load_run<EPL>(gamma + lane * EPL, g);
  const float r = rstd[t];
  E part[NS][EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    E p[NS];
    split_to<M, NS>(g[j] * (v[j] * r), p);
#pragma unroll
    for (int s = 0; s < NS; ++s) part[s][j] = p[s];
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    E* dst = out + s * plane + t * D + lane * EPL;
    if constexpr (EPL * sizeof(E) == 16) {
      *reinterpret_cast<u16x8*>(dst) = *reinterpret_cast<const u16x8*>(part[s]);
    } else {
#pragma unroll
      for (int j = 0; j < EPL; ++j) dst[j] = part[s][j];
    }
  }
}

constexpr int kNormBwdBlocks = 512;

template <class InT, int D>
hipError_t norm_fwd_t(const Shape& s, const void* x, const void* g, float* L, float* rstd,
                      hipStream_t st) {
  const int64_t blocks = (s.T + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL((rmsnorm_fwd_kernel<InT, D>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kNormBlock), 0, st, static_cast<const InT*>(x),
                     static_cast<const InT*>(g), L, rstd, s.T, s.eps);
  return hipGetLastError();
}

int norm_bwd_blocks(const Shape& s) {
  const int64_t need = (s.T + kRowsPerBlock - 1) / kRowsPerBlock;
  return static_cast<int>(need < kNormBwdBlocks ? need : kNormBwdBlocks);
}

template <class InT, int D>
hipError_t norm_bwd_t(const Shape& s, const float* dL, const void* x, const void* g,
                      const float* rstd, float* dx, float* part, float* dgamma, hipStream_t st) {
  const int blocks = norm_bwd_blocks(s);
  hipLaunchKernelGGL((rmsnorm_bwd_kernel<InT, D>), dim3(blocks), dim3(kNormBlock), 0, st, dL,
                     static_cast<const InT*>(x), static_cast<const InT*>(g), rstd, dx, part, s.T);
  hipLaunchKernelGGL(column_sum_kernel, dim3((D + kSumCols - 1) / kSumCols), dim3(kNormBlock), 0, st, part,
                     dgamma, blocks, D);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_norm_fwd(const Shape& s, const void* x, const void* g, float* L, float* rstd,
                           hipStream_t st) {
  if (s.bf16 && s.d_kv == 512) return norm_fwd_t<bf16_t, 512>(s, x, g, L, rstd, st);
  if (!s.bf16 && s.d_kv == 64) return norm_fwd_t<float, 64>(s, x, g, L, rstd, st);
  return hipErrorInvalidValue;
}

hipError_t launch_norm_planes(const Shape& s, const void* x, const void* g, const float* rstd, void* out,
                              hipStream_t st) {
  const unsigned blocks = static_cast<unsigned>((s.T + kRowsPerBlock - 1) / kRowsPerBlock);
  const int64_t plane = s.T * s.d_kv;
  if (s.bf16 && s.d_kv == 512) {
    hipLaunchKernelGGL((norm_planes_kernel<MmaBf16, 2, bf16_t, 512>), dim3(blocks), dim3(kNormBlock), 0, st,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(g), rstd,
                       static_cast<bf16_t*>(out), s.T, plane);
  } else if (!s.bf16 && s.d_kv == 64) {
    hipLaunchKernelGGL((norm_planes_kernel<MmaF32, 1, float, 64>), dim3(blocks), dim3(kNormBlock), 0, st,
                       static_cast<const float*>(x), static_cast<const float*>(g), rstd, static_cast<float*>(out),
                       s.T, plane);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

size_t norm_bwd_partial_floats(const Shape& s) {
  return static_cast<size_t>(norm_bwd_blocks(s)) * s.d_kv;
}

hipError_t launch_norm_bwd(const Shape& s, const float* dL, const void* x, const void* g,
                           const float* rstd, float* dx, float* part, float* dgamma,
                           hipStream_t st) {
  if (s.bf16 && s.d_kv == 512) return norm_bwd_t<bf16_t, 512>(s, dL, x, g, rstd, dx, part, dgamma, st);
  if (!s.bf16 && s.d_kv == 64) return norm_bwd_t<float, 64>(s, dL, x, g, rstd, dx, part, dgamma, st);
  return hipErrorInvalidValue;
}

}  // namespace laga
