// Causal attention backward of one rank's head shard [LAGA §5.2].
#include "device.hpp"
#include "launch.hpp"

namespace laga {
namespace {

// delta[b, i, t] = sum_c d_o[b, t, i, c] * o[b, t, i, c]  (one wavefront per row).
template <class InT, int DV>
__global__ __launch_bounds__(256) void bwd_dot_kernel(const float* __restrict__ o, const InT* __restrict__ d_o,
                                                      float* __restrict__ delta, int64_t rows, int h,
                                                      int64_t S) {
  constexpr int EPL = DV / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;  // (b, t, i)
  if (row >= rows) return;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) acc += o[row * DV + lane * EPL + j] * to_f32(d_o[row * DV + lane * EPL + j]);
  acc = wave_sum(acc);
  if (lane == 0) {
    const int64_t bt = row / h;
    const int i = static_cast<int>(row % h);
    const int64_t b = bt / S, t = bt % S;
    delta[(b * h + i) * S + t] = acc;
  }
}

// out[t, c] = sum_i part[i, t, c] in increasing i (deterministic head sum).
__global__ __launch_bounds__(256) void head_sum_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                       int64_t n, int h) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (j >= n) return;
  float s = 0.f;
  for (int i = 0; i < h; ++i) s += part[i * n + j];
  out[j] = s;
}

}  // namespace

hipError_t launch_bwd_dot(const Shape& s, const float* o, const void* d_o, float* delta, hipStream_t st) {
  const int64_t rows = s.T * s.h;
  const unsigned blocks = static_cast<unsigned>((rows + 3) / 4);
  if (s.bf16)
    hipLaunchKernelGGL((bwd_dot_kernel<bf16_t, 128>), dim3(blocks), dim3(256), 0, st, o,
                       static_cast<const bf16_t*>(d_o), delta, rows, s.h, s.S);
  else
    hipLaunchKernelGGL((bwd_dot_kernel<float, 32>), dim3(blocks), dim3(256), 0, st, o,
                       static_cast<const float*>(d_o), delta, rows, s.h, s.S);
  return hipGetLastError();
}

hipError_t launch_head_sum(const Shape& s, const float* part, float* out, hipStream_t st) {
  const int64_t n = s.T * s.d_rope;
  hipLaunchKernelGGL(head_sum_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, part, out,
                     n, s.h);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv(const Shape&, const void*, const void*, const void*, const void*, const float*,
                                const float*, const void*, float*, float*, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_attn_bwd_dq(const Shape&, const void*, const void*, const void*, const void*, const float*,
                              const float*, const void*, float*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace laga
