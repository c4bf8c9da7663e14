// Matrix-core GEMMs of the path: the head-shard up-projection and the two
// folds of (dk_nope || dv) back through W_kv_b.
//
//   kv_up   [LAGA §3.3 Algorithm 1 local up-projection; §5.1]
//           C[t, n] = sum_k L[t, k] W_r[n, k],   n = i*(d_nope+d_v) + c
//           scattered into k_nope[t, i, c] (c < d_nope) and v[t, i, c - d_nope]
//   fold_dl C[t, k] = sum_n dKV[t, n] W_r[n, k]         (dL, input of the norm backward)
//   fold_dw C[n, k] = sum_t dKV[t, n] L[t, k]           (the (full_seq, H_r) shard
//           of the W_kv_b gradient [LAGA §5.2]); L is rebuilt on the fly from
//           the latent, gamma and rstd, and the reduction over t is split into
//           chunks summed by a second, deterministic kernel.
//
// One kernel template serves all three: a 128x128 output tile per 256-thread
// workgroup (four wavefronts in 2x2, each 64x64 = 2x2 MFMA atoms of 32x32),
// K staged through LDS 32 at a time.  Loaders read each operand along its
// contiguous axis with 16-byte loads and write LDS rows in the K-contiguous
// order the atoms read.  Float operands are split on the way into LDS into NS
// bf16 terms (hi, lo); the product keeps the terms with sa + sb < max(NSA, NSB),
// which makes a bf16 matrix-core GEMM accurate to about 2^-16 relative.
#include "device.hpp"
#include "launch.hpp"

namespace laga {
namespace {

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int kThreads = 256;

template <class M> struct Pad { static constexpr int v = 8; };
template <> struct Pad<MmaF32> { static constexpr int v = 1; };

// ------------------------------------------------------------------- loaders
// load4(row, k, out): four consecutive elements along the operand's contiguous
// axis (k for K-contiguous operands, row otherwise), zero outside [0,R)x[0,K).

struct LoadF32KC {  // float src[row * ld + k]
  static constexpr bool KC = true;
  const float* p; int64_t ld, R, K;
  __device__ void load4(int64_t r, int64_t k, float* o) const {
    if (r < R && k + 3 < K) {
      f32x4 v = *reinterpret_cast<const f32x4*>(p + r * ld + k);
      o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = (r < R && k + j < K) ? p[r * ld + k + j] : 0.f;
    }
  }
};

template <class InT>
struct LoadInKC {  // input-dtype src[row * ld + k]
  static constexpr bool KC = true;
  const InT* p; int64_t ld, R, K;
  __device__ void load4(int64_t r, int64_t k, float* o) const {
    if constexpr (sizeof(InT) == 2) {
      if (r < R && k + 3 < K) {
        u16x4 v = *reinterpret_cast<const u16x4*>(p + r * ld + k);
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = bf16_to_f32(v[j]);
        return;
      }
    } else {
      if (r < R && k + 3 < K) {
        f32x4 v = *reinterpret_cast<const f32x4*>(p + r * ld + k);
        o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
        return;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = (r < R && k + j < K) ? to_f32(p[r * ld + k + j]) : 0.f;
  }
};

struct LoadF32RC {  // float src[k * ld + row]
  static constexpr bool KC = false;
  const float* p; int64_t ld, R, K;
  __device__ void load4(int64_t r, int64_t k, float* o) const {
    if (k < K && r + 3 < R) {
      f32x4 v = *reinterpret_cast<const f32x4*>(p + k * ld + r);
      o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = (k < K && r + j < R) ? p[k * ld + r + j] : 0.f;
    }
  }
};

template <class InT>
struct LoadInRC {  // input-dtype src[k * ld + row]
  static constexpr bool KC = false;
  const InT* p; int64_t ld, R, K;
  __device__ void load4(int64_t r, int64_t k, float* o) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = (k < K && r + j < R) ? to_f32(p[k * ld + r + j]) : 0.f;
  }
};

// L[t, c] = gamma[c] * x[t, c] * rstd[t], read as B(row = c, k = t).
template <class InT>
struct LoadNormRC {
  static constexpr bool KC = false;
  const InT* x; const InT* gamma; const float* rstd; int64_t ld, R, K;
  __device__ void load4(int64_t r, int64_t k, float* o) const {
    const float rs = (k < K) ? rstd[k] : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = (k < K && r + j < R) ? to_f32(gamma[r + j]) * (to_f32(x[k * ld + r + j]) * rs) : 0.f;
  }
};

// ----------------------------------------------------------------- epilogues
// n = i*C + c -> k_nope[t,i,c] or v[t,i,c-d_nope]; with NS == 2 the value is
// written as an fp16 hi part in plane 0 and the fp16 rest in plane 1.
template <class KvT, int NS>
struct EpiKvUp {
  KvT* kn; KvT* v; int64_t M; int N, C, dn, dv, h; int64_t plane_k, plane_v;
  __device__ void operator()(int64_t m, int n, float val) const {
    if (m >= M || n >= N) return;
    const int i = n / C, c = n - i * C;
    KvT part[NS];
    if constexpr (NS == 1) {
      part[0] = static_cast<KvT>(val);
    } else {
      part[0] = static_cast<KvT>(val);
      part[1] = static_cast<KvT>(val - static_cast<float>(part[0]));
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (c < dn) kn[s * plane_k + (m * h + i) * dn + c] = part[s];
      else v[s * plane_v + (m * h + i) * dv + (c - dn)] = part[s];
    }
  }
};

struct EpiStore {  // out[m * ld + n] (+ chunk offset)
  float* p; int64_t M; int N; int64_t ld; int64_t chunk_stride;
  __device__ void operator()(int64_t m, int n, float val) const {
    if (m >= M || n >= N) return;
    p[blockIdx.z * chunk_stride + m * ld + n] = val;
  }
};

// ------------------------------------------------------------------- kernel
template <class M, int NS>
__device__ __forceinline__ void put(typename M::elem* base, int64_t stride_plane, float x) {
  typename M::elem part[NS];
  split_to<M, NS>(x, part);
#pragma unroll
  for (int s = 0; s < NS; ++s) base[s * stride_plane] = part[s];
}

template <class M, int NS, class L, int ROWS>
struct Stage {
  static constexpr int LD = BK + Pad<M>::v;
  static constexpr int GROUPS = ROWS * BK / 4 / kThreads;
  float reg[GROUPS][4];
  __device__ void load(const L& ld, int64_t row0, int64_t k0) {
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) {
      const int idx = g * kThreads + threadIdx.x;
      if constexpr (L::KC) {
        ld.load4(row0 + idx / (BK / 4), k0 + (idx % (BK / 4)) * 4, reg[g]);
      } else {
        ld.load4(row0 + (idx % (ROWS / 4)) * 4, k0 + idx / (ROWS / 4), reg[g]);
      }
    }
  }
  __device__ void store(typename M::elem* lds) const {
    constexpr int64_t plane = static_cast<int64_t>(ROWS) * LD;
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) {
      const int idx = g * kThreads + threadIdx.x;
      if constexpr (L::KC) {
        const int r = idx / (BK / 4), k = (idx % (BK / 4)) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) put<M, NS>(lds + r * LD + k + j, plane, reg[g][j]);
      } else {
        const int r = (idx % (ROWS / 4)) * 4, k = idx / (ROWS / 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) put<M, NS>(lds + (r + j) * LD + k, plane, reg[g][j]);
      }
    }
  }
};

template <class M, int NSA, int NSB, class LA, class LB, class EPI>
__global__ __launch_bounds__(kThreads) void gemm_kernel(LA la, LB lb, EPI epi, int64_t k_chunk,
                                                        int64_t K) {
  typedef typename M::elem E;
  constexpr int LD = BK + Pad<M>::v;
  __shared__ __attribute__((aligned(16))) E As[NSA * BM * LD];
  __shared__ __attribute__((aligned(16))) E Bs[NSB * BN * LD];

  const int lane = threadIdx.x % kWave;
  const int wv = threadIdx.x / kWave;
  const int wm = wv / 2, wn = wv % 2;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * BN;
  const int64_t kbeg = static_cast<int64_t>(blockIdx.z) * k_chunk;
  const int64_t kend = (kbeg + k_chunk < K) ? kbeg + k_chunk : K;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  Stage<M, NSA, LA, BM> sa;
  Stage<M, NSB, LB, BN> sb;
  constexpr int NSMAX = NSA > NSB ? NSA : NSB;
  const int row = lane % 32, kofs = (lane / 32) * M::KPL;

  if (kbeg < kend) {
    sa.load(la, m0, kbeg);
    sb.load(lb, n0, kbeg);
  }
  for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
    __syncthreads();
    sa.store(As);
    sb.store(Bs);
    __syncthreads();
    if (k0 + BK < kend) {
      sa.load(la, m0, k0 + BK);
      sb.load(lb, n0, k0 + BK);
    }
#pragma unroll
    for (int ks = 0; ks < BK / M::K; ++ks) {
      typename M::frag af[NSA][2], bfr[NSB][2];
#pragma unroll
      for (int s = 0; s < NSA; ++s)
#pragma unroll
        for (int a = 0; a < 2; ++a)
          af[s][a] = lds_frag<M>(As + s * BM * LD + (wm * 64 + a * 32 + row) * LD + ks * M::K + kofs);
#pragma unroll
      for (int s = 0; s < NSB; ++s)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          bfr[s][b] = lds_frag<M>(Bs + s * BN * LD + (wn * 64 + b * 32 + row) * LD + ks * M::K + kofs);
#pragma unroll
      for (int s1 = 0; s1 < NSA; ++s1)
#pragma unroll
        for (int s2 = 0; s2 < NSB; ++s2) {
          if (s1 + s2 >= NSMAX) continue;
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) acc[a][b] = M::mma(af[s1][a], bfr[s2][b], acc[a][b]);
        }
    }
  }
  // C[r]: row 8*(r/4) + 4*(lane/32) + r%4 of the atom, column lane%32.
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + a * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
        const int n = static_cast<int>(n0 + wn * 64 + b * 32 + (lane % 32));
        epi(m, n, acc[a][b][r]);
      }
}

template <class M, int NSA, int NSB, class LA, class LB, class EPI>
hipError_t run_gemm(LA la, LB lb, EPI epi, int64_t Mrows, int64_t Ncols, int64_t K, int chunks,
                    hipStream_t st) {
  const int64_t per = ((K + chunks - 1) / chunks + BK - 1) / BK * BK;
  const int nchunks = static_cast<int>((K + per - 1) / per);
  dim3 grid(static_cast<unsigned>((Ncols + BN - 1) / BN), static_cast<unsigned>((Mrows + BM - 1) / BM),
            static_cast<unsigned>(nchunks));
  hipLaunchKernelGGL((gemm_kernel<M, NSA, NSB, LA, LB, EPI>), grid, dim3(kThreads), 0, st, la, lb,
                     epi, per, K);
  return hipGetLastError();
}

// Number of K chunks for the W_kv_b gradient so that about 1024 workgroups run.
int dw_chunks(const Shape& s) {
  const int64_t tiles = ((static_cast<int64_t>(s.h) * s.C() + BM - 1) / BM) * ((s.d_kv + BN - 1) / BN);
  int64_t c = (1024 + tiles - 1) / tiles;
  const int64_t kmax = (s.T + BK - 1) / BK;
  if (c > kmax) c = kmax;
  if (c < 1) c = 1;
  // Round to the chunk count run_gemm will actually produce.
  const int64_t per = ((s.T + c - 1) / c + BK - 1) / BK * BK;
  return static_cast<int>((s.T + per - 1) / per);
}

// out[j] = sum_c part[c * n + j], rows of W_kv_b of this shard.
__global__ __launch_bounds__(256) void chunk_sum_kernel(const float* __restrict__ part,
                                                        float* __restrict__ out, int64_t n,
                                                        int chunks) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (j >= n) return;
  float s = 0.f;
  for (int c = 0; c < chunks; ++c) s += part[c * n + j];
  out[j] = s;
}

}  // namespace

hipError_t launch_kv_up(const Shape& s, const float* L, const void* w, void* k_nope, void* v,
                        hipStream_t st) {
  const int64_t N = static_cast<int64_t>(s.h) * s.C();
  LoadF32KC la{L, s.d_kv, s.T, s.d_kv};
  if (s.bf16) {
    LoadInKC<bf16_t> lb{static_cast<const bf16_t*>(w) + static_cast<int64_t>(s.head_lo) * s.C() * s.d_kv,
                        s.d_kv, N, s.d_kv};
    const int64_t pk = s.T * s.h * s.d_nope, pv = s.T * s.h * s.d_v;
    if (s.split) {
      EpiKvUp<half_t, 2> e{static_cast<half_t*>(k_nope), static_cast<half_t*>(v), s.T, static_cast<int>(N),
                           s.C(), s.d_nope, s.d_v, s.h, pk, pv};
      return run_gemm<MmaBf16, 2, 1>(la, lb, e, s.T, N, s.d_kv, 1, st);
    }
    EpiKvUp<half_t, 1> e{static_cast<half_t*>(k_nope), static_cast<half_t*>(v), s.T, static_cast<int>(N),
                         s.C(), s.d_nope, s.d_v, s.h, pk, pv};
    return run_gemm<MmaBf16, 2, 1>(la, lb, e, s.T, N, s.d_kv, 1, st);
  }
  LoadInKC<float> lb{static_cast<const float*>(w) + static_cast<int64_t>(s.head_lo) * s.C() * s.d_kv,
                     s.d_kv, N, s.d_kv};
  EpiKvUp<float, 1> e{static_cast<float*>(k_nope), static_cast<float*>(v), s.T, static_cast<int>(N),
                      s.C(), s.d_nope, s.d_v, s.h, 0, 0};
  return run_gemm<MmaF32, 1, 1>(la, lb, e, s.T, N, s.d_kv, 1, st);
}

hipError_t launch_fold_dl(const Shape& s, const float* dkv, const void* w, float* dL,
                          hipStream_t st) {
  const int64_t Kd = static_cast<int64_t>(s.h) * s.C();
  LoadF32KC la{dkv, Kd, s.T, Kd};
  EpiStore e{dL, s.T, s.d_kv, s.d_kv, 0};
  if (s.bf16) {
    LoadInRC<bf16_t> lb{static_cast<const bf16_t*>(w) + static_cast<int64_t>(s.head_lo) * s.C() * s.d_kv,
                        s.d_kv, s.d_kv, Kd};
    return run_gemm<MmaBf16, 2, 1>(la, lb, e, s.T, s.d_kv, Kd, 1, st);
  }
  LoadInRC<float> lb{static_cast<const float*>(w) + static_cast<int64_t>(s.head_lo) * s.C() * s.d_kv,
                     s.d_kv, s.d_kv, Kd};
  return run_gemm<MmaF32, 1, 1>(la, lb, e, s.T, s.d_kv, Kd, 1, st);
}

size_t fold_dw_partial_floats(const Shape& s) {
  return static_cast<size_t>(dw_chunks(s)) * s.h * s.C() * s.d_kv;
}

hipError_t launch_fold_dw(const Shape& s, const float* dkv, const void* latent, const void* gamma,
                          const float* rstd, float* partial, float* d_w, hipStream_t st) {
  const int64_t Mr = static_cast<int64_t>(s.h) * s.C();
  const int chunks = dw_chunks(s);
  LoadF32RC la{dkv, Mr, Mr, s.T};
  EpiStore e{partial, Mr, s.d_kv, s.d_kv, Mr * s.d_kv};
  hipError_t err;
  if (s.bf16) {
    LoadNormRC<bf16_t> lb{static_cast<const bf16_t*>(latent), static_cast<const bf16_t*>(gamma), rstd,
                          s.d_kv, s.d_kv, s.T};
    err = run_gemm<MmaBf16, 2, 2>(la, lb, e, Mr, s.d_kv, s.T, chunks, st);
  } else {
    LoadNormRC<float> lb{static_cast<const float*>(latent), static_cast<const float*>(gamma), rstd,
                         s.d_kv, s.d_kv, s.T};
    err = run_gemm<MmaF32, 1, 1>(la, lb, e, Mr, s.d_kv, s.T, chunks, st);
  }
  if (err != hipSuccess) return err;
  const int64_t n = Mr * s.d_kv;
  hipLaunchKernelGGL(chunk_sum_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                     partial, d_w + static_cast<int64_t>(s.head_lo) * s.C() * s.d_kv, n, chunks);
  return hipGetLastError();
}

}  // namespace laga
