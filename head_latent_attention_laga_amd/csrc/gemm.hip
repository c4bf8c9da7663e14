// Matrix-core GEMMs of the path: the head-shard up-projection and the two
// folds of (dk_nope || dv) back through W_kv_b.
//
//   kv_up   [LAGA §3.3 Algorithm 1 local up-projection; §5.1]
//           C[t, n] = sum_k L[t, k] W_r[n, k],   n = i*(d_nope+d_v) + c
//           scattered into k_nope[t, i, c] (c < d_nope) and v[t, i, c - d_nope]
//   fold_dl C[t, k] = sum_n dKV[t, n] W_r[n, k]         (dL, input of the norm backward)
//   fold_dw C[n, k] = sum_t dKV[t, n] L[t, k]           (the (full_seq, H_r) shard
//           of the W_kv_b gradient [LAGA §5.2]); the reduction over t is split
//           into chunks summed by a second, deterministic kernel.
//
// One kernel template serves all three: a 128x128 output tile per 256-thread
// workgroup (four wavefronts in 2x2, each 64x64 = 2x2 MFMA atoms of 32x32),
// K staged through double-buffered LDS 32 at a time, one barrier per step.
// Each operand slab moves global -> registers -> LDS in 16-byte chunks along
// the operand's contiguous axis:
//   KC operands (k contiguous in memory) land as LDS rows [row][k] and are
//      read with 16-byte fragment loads;
//   RC operands (row contiguous: the k axis strides memory) land as [k][row]
//      and 16-bit fragments come from gfx950's transposing LDS read.
// Operands are stored as NS planes of the MFMA element type (x ~= sum of the
// planes).  bf16 planes are written by the producing kernels, except the
// normalised latent of the up-projection, which arrives in fp32 and is split
// into bf16 hi + lo while it is staged.  The product keeps the term pairs
// (sa, sb) with sa + sb < max(NSA, NSB), which makes the bf16 GEMM accurate to
// about 2^-16 relative.
#include <type_traits>

#include "attn_common.hpp"
#include "launch.hpp"

namespace laga {
namespace {

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int kThreads = 256;

// A GEMM operand in global memory: element (row r, k) of plane s at
//   p + s * plane + r * ld + k   (KC)   or   p + s * plane + k * ld + r   (RC),
// plus zstride * z for batch z of a batched GEMM.  Rows >= R and k >= K read
// as zero.
template <class Src>
struct Operand {
  const Src* p;
  int64_t ld, plane, R, K;
  int64_t zstride = 0;
};

// ROWS x BK slab of one operand, in NS LDS planes of the MFMA element type.
template <class M, int NS, bool KC, int ROWS, class Src>
struct SlabT {
  typedef typename M::elem E;
  typedef typename M::frag F;
  static constexpr int EPC = 16 / sizeof(E);  // elements per 16-byte chunk
  static constexpr bool SPLIT = !std::is_same<Src, E>::value;
  static_assert(!SPLIT || (std::is_same<Src, float>::value && NS == 2 && EPC == 8),
                "only fp32 -> 16-bit hi/lo splitting");
  static constexpr int LD = KC ? BK + EPC : ROWS + (sizeof(E) == 2 ? 32 : 4);  // LDS pitch, elements
  static constexpr int PLANE = (KC ? ROWS : BK) * LD;
  static constexpr int BYTES = NS * PLANE * static_cast<int>(sizeof(E));
  static constexpr int CHUNKS = ROWS * BK / EPC;  // per plane
  static constexpr int PER = CHUNKS / kThreads;
  static_assert(CHUNKS % kThreads == 0, "whole chunks per thread");
  static constexpr int NP = SPLIT ? 1 : NS;  // planes read from memory
  static constexpr int WORDS = SPLIT ? 2 : 1;  // 16-byte words per chunk read

  u32x4 reg[NP][PER][WORDS];

  __device__ static void chunk_pos(int c, int& r, int& k) {
    if constexpr (KC) {
      r = c / (BK / EPC);
      k = (c % (BK / EPC)) * EPC;
    } else {
      k = c / (ROWS / EPC);
      r = (c % (ROWS / EPC)) * EPC;
    }
  }

  __device__ void load(const Operand<Src>& op, int64_t row0, int64_t k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int r, k;
      chunk_pos(i * kThreads + static_cast<int>(threadIdx.x), r, k);
      const int64_t gr = row0 + r, gk = k0 + k;
      // KC: rows are whole; K is a multiple of the chunk.  RC: R is a multiple of the chunk.
      const bool ok = gr < op.R && gk < op.K;
      const Src* src = op.p + (KC ? gr * op.ld + gk : gk * op.ld + gr);
#pragma unroll
      for (int s = 0; s < NP; ++s)
#pragma unroll
        for (int w = 0; w < WORDS; ++w)
          reg[s][i][w] = ok ? *reinterpret_cast<const u32x4*>(src + s * op.plane + w * (16 / sizeof(Src)))
                            : u32x4{0u, 0u, 0u, 0u};
    }
  }

  __device__ void store(E* lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int r, k;
      chunk_pos(i * kThreads + static_cast<int>(threadIdx.x), r, k);
      E* dst = lds + (KC ? r * LD + k : k * LD + r);
      if constexpr (SPLIT && std::is_same<M, MmaBf16>::value) {  // bf16 hi/lo planes, two values per word
        u32x4 hw, lw;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const f32x4 x = __builtin_bit_cast(f32x4, reg[0][i][w]);
          uint32_t h, l;
          split_bf16_pair(x[0], x[1], h, l);
          hw[2 * w] = h;
          lw[2 * w] = l;
          split_bf16_pair(x[2], x[3], h, l);
          hw[2 * w + 1] = h;
          lw[2 * w + 1] = l;
        }
        *reinterpret_cast<u32x4*>(dst) = hw;
        *reinterpret_cast<u32x4*>(dst + PLANE) = lw;
      } else if constexpr (SPLIT) {
        E part[NS][EPC];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const f32x4 x = __builtin_bit_cast(f32x4, reg[0][i][w]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            E t[NS];
            split_to<M, NS>(x[j], t);
#pragma unroll
            for (int s = 0; s < NS; ++s) part[s][4 * w + j] = t[s];
          }
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) *reinterpret_cast<u32x4*>(dst + s * PLANE) = *reinterpret_cast<u32x4*>(part[s]);
      } else {
#pragma unroll
        for (int s = 0; s < NS; ++s) *reinterpret_cast<u32x4*>(dst + s * PLANE) = reg[s][i][0];
      }
    }
  }

  // Fragment of atom rows n0 .. n0+31 for the MFMA step at k = kk (natural k order).
  __device__ static F frag(const E* lds, int s, int n0, int kk) {
    const int lane = threadIdx.x % kWave;
    const E* plane = lds + s * PLANE;
    if constexpr (KC) {
      return lds_frag<M>(plane + (n0 + lane % 32) * LD + kk + (lane / 32) * M::KPL);
    } else if constexpr (sizeof(E) == 2) {
      return __builtin_bit_cast(F, tr_frag(plane, LD, kk, n0));
    } else {
      return plane[(kk + lane / 32) * LD + n0 + lane % 32];
    }
  }
};

// ----------------------------------------------------------------- epilogues
// n = i*C + c -> k_nope[t,i,c] or v[t,i,c-d_nope].  With NS == 2 (fp16
// storage) the value x is written as hi = fp16(x) in a first plane and the
// rest as an e4m3 byte of (x - hi) * 2^kLoShift in a byte plane after it.
template <class KvT, int NS>
struct EpiKvUp {
  static_assert(NS == 1 || sizeof(KvT) == 2, "the split form stores fp16 + e4m3");
  static constexpr bool TRANS = true;  // takes 4 consecutive n of one row m
  KvT* kn; KvT* v; int64_t M; int N, C, dn, dv, h; int64_t plane_k, plane_v;
  // n .. n+3 lie in one head and one part (C, dn multiples of 4).
  __device__ void store4(int64_t m, int n, f32x4 val, int /*z*/) const {
    if (m >= M || n >= N) return;
    const int i = n / C, c = n - i * C;
    const bool isk = c < dn;
    const int64_t e = isk ? (m * h + i) * dn + c : (m * h + i) * dv + (c - dn);
    KvT* base = isk ? kn : v;
    KvT hi[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) hi[j] = static_cast<KvT>(val[j]);
    if constexpr (sizeof(KvT) == 2)
      *reinterpret_cast<u16x4*>(base + e) = *reinterpret_cast<const u16x4*>(hi);
    else
      *reinterpret_cast<f32x4*>(base + e) = *reinterpret_cast<const f32x4*>(hi);
    if constexpr (NS == 2) {
      constexpr float sc = static_cast<float>(1 << kLoShift);
      uint8_t* lo = reinterpret_cast<uint8_t*>(base + (isk ? plane_k : plane_v));
      *reinterpret_cast<uint32_t*>(lo + e) =
          pack_e4m3x4((val[0] - static_cast<float>(hi[0])) * sc, (val[1] - static_cast<float>(hi[1])) * sc,
                      (val[2] - static_cast<float>(hi[2])) * sc, (val[3] - static_cast<float>(hi[3])) * sc);
    }
  }
};

// out[z * zstride + m * ld + n] as fp16, four consecutive n at a time
// (z: the batch of a batched GEMM).
struct EpiHalf {
  static constexpr bool TRANS = true;
  half_t* p; int64_t M; int N; int64_t ld, zstride;
  __device__ void store4(int64_t m, int n, f32x4 val, int z) const {
    if (m >= M || n >= N) return;
    half_t h4[4] = {static_cast<half_t>(val[0]), static_cast<half_t>(val[1]), static_cast<half_t>(val[2]),
                    static_cast<half_t>(val[3])};
    *reinterpret_cast<u16x4*>(p + z * zstride + m * ld + n) = *reinterpret_cast<const u16x4*>(h4);
  }
};

struct EpiStore {  // out[z * chunk_stride + m * ld + n] (z: batch * chunks + K chunk)
  static constexpr bool TRANS = false;
  float* p; int64_t M; int N; int64_t ld; int64_t chunk_stride;
  __device__ void operator()(int64_t m, int n, float val, int z) const {
    if (m >= M || n >= N) return;
    p[z * chunk_stride + m * ld + n] = val;
  }
};

// ------------------------------------------------------------------- kernel
// Tiles (x = N tile, y = M tile, z = batch * nchunks + K chunk) come from a
// 1-D launch.  Workgroup ids are dealt round-robin to the 8 XCDs, each with
// its own L2; they are remapped so that every XCD takes one contiguous range
// of tiles in x-fastest order: the N tiles that share an A row block (and the
// M tiles that share a B block) then run on the same XCD and read those rows
// from HBM once instead of once per XCD.
template <class M, class SA, class SB, class EPI>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(Operand<typename SA::Src_t> A,
                                                           Operand<typename SB::Src_t> B, EPI epi,
                                                           int64_t k_chunk, int64_t K, int nchunks, int gx, int gy,
                                                           int gz) {
  typedef typename M::elem E;
  constexpr int STAGE = SA::BYTES + SB::BYTES;
  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

  const int total = gx * gy * gz;
  const int id = static_cast<int>(blockIdx.x);
  const int tile = total % 8 == 0 ? (id % 8) * (total / 8) + id / 8 : id;
  const int bx = tile % gx, by = (tile / gx) % gy, bz = tile / (gx * gy);
  const int wv = threadIdx.x / kWave;
  const int wm = wv / 2, wn = wv % 2;
  const int64_t m0 = static_cast<int64_t>(by) * BM;
  const int64_t n0 = static_cast<int64_t>(bx) * BN;
  // bz = batch * nchunks + K chunk (the epilogues index their output by it).
  const int chunk = bz % nchunks, batch = bz / nchunks;
  A.p += batch * A.zstride;
  B.p += batch * B.zstride;
  const int64_t kbeg = static_cast<int64_t>(chunk) * k_chunk;
  const int64_t kend = (kbeg + k_chunk < K) ? kbeg + k_chunk : K;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // Two register stages of operand slabs in flight: the loads for step k+2
  // are issued while step k computes, so about two steps of products cover
  // the global-memory latency.  The loop is unrolled by two so that each
  // stage keeps its own registers.
  typename SA::Slab sa0, sa1;
  typename SB::Slab sb0, sb1;
  constexpr int NSA = SA::Slab::NS_, NSB = SB::Slab::NS_;
  constexpr int NSMAX = NSA > NSB ? NSA : NSB;

  auto compute = [&](const E* as, const E* bs) {
#pragma unroll
    for (int kk = 0; kk < BK; kk += M::K) {
      typename M::frag af[NSA][2], bfr[NSB][2];
#pragma unroll
      for (int s = 0; s < NSA; ++s)
#pragma unroll
        for (int a = 0; a < 2; ++a) af[s][a] = SA::Slab::frag(as, s, wm * 64 + a * 32, kk);
#pragma unroll
      for (int s = 0; s < NSB; ++s)
#pragma unroll
        for (int b = 0; b < 2; ++b) bfr[s][b] = SB::Slab::frag(bs, s, wn * 64 + b * 32, kk);
#pragma unroll
      for (int s1 = 0; s1 < NSA; ++s1)
#pragma unroll
        for (int s2 = 0; s2 < NSB; ++s2) {
          if (s1 + s2 >= NSMAX) continue;
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              // EPI::TRANS: the atom holds C^T (rows n, columns m).
              if constexpr (EPI::TRANS) acc[a][b] = M::mma(bfr[s2][b], af[s1][a], acc[a][b]);
              else acc[a][b] = M::mma(af[s1][a], bfr[s2][b], acc[a][b]);
            }
        }
    }
  };
  // One step: publish the slabs of step k0 (held in sa/sb) into LDS buffer
  // `buf`, refill sa/sb with step k0 + 2*BK, compute step k0.
  auto step = [&](int64_t k0, int buf, typename SA::Slab& sa, typename SB::Slab& sb) {
    E* as = reinterpret_cast<E*>(lds + buf * STAGE);
    E* bs = reinterpret_cast<E*>(lds + buf * STAGE + SA::BYTES);
    sa.store(as);
    sb.store(bs);
    __syncthreads();  // also orders the reads of this buffer two steps ago before the stores above
    if (k0 + 2 * BK < kend) {
      sa.load(A, m0, k0 + 2 * BK);
      sb.load(B, n0, k0 + 2 * BK);
    }
    compute(as, bs);
  };

  if (kbeg < kend) {
    sa0.load(A, m0, kbeg);
    sb0.load(B, n0, kbeg);
  }
  if (kbeg + BK < kend) {
    sa1.load(A, m0, kbeg + BK);
    sb1.load(B, n0, kbeg + BK);
  }
  for (int64_t k0 = kbeg; k0 < kend; k0 += 2 * BK) {
    step(k0, 0, sa0, sb0);
    if (k0 + BK < kend) step(k0 + BK, 1, sa1, sb1);
  }
  // C[r]: row 8*(r/4) + 4*(lane/32) + r%4 of the atom, column lane%32.
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if constexpr (EPI::TRANS) {
        const int64_t m = m0 + wm * 64 + a * 32 + (lane % 32);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = static_cast<int>(n0 + wn * 64 + b * 32 + 8 * g + 4 * (lane / 32));
          const f32x4 v4 = {acc[a][b][4 * g], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2], acc[a][b][4 * g + 3]};
          epi.store4(m, n, v4, bz);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + wm * 64 + a * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
          const int n = static_cast<int>(n0 + wn * 64 + b * 32 + (lane % 32));
          epi(m, n, acc[a][b][r], bz);
        }
      }
    }
}

// Operand description: MFMA type, planes, orientation, rows per tile, source element.
template <class M, int NS, bool KC, int ROWS, class Src>
struct Side {
  struct Slab : SlabT<M, NS, KC, ROWS, Src> { static constexpr int NS_ = NS; };
  typedef Src Src_t;
  static constexpr int BYTES = Slab::BYTES;
};

template <class M, class SA, class SB, class EPI>
hipError_t run_gemm(Operand<typename SA::Src_t> A, Operand<typename SB::Src_t> B, EPI epi, int64_t Mrows,
                    int64_t Ncols, int64_t K, int chunks, hipStream_t st, int batches = 1) {
  const int64_t per = ((K + chunks - 1) / chunks + BK - 1) / BK * BK;
  const int nchunks = static_cast<int>((K + per - 1) / per);
  const int gx = static_cast<int>((Ncols + BN - 1) / BN), gy = static_cast<int>((Mrows + BM - 1) / BM),
            gz = nchunks * batches;
  hipLaunchKernelGGL((gemm_kernel<M, SA, SB, EPI>), dim3(static_cast<unsigned>(gx * gy * gz)), dim3(kThreads), 0, st,
                     A, B, epi, per, K, nchunks, gx, gy, gz);
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
#pragma unroll 8  // the loads issue together; the sum keeps its order
  for (int c = 0; c < chunks; ++c) s += part[c * n + j];
  out[j] = s;
}

}  // namespace

hipError_t launch_kv_up(const Shape& s, const float* L, const void* w, void* k_nope, void* v,
                        hipStream_t st) {
  const int64_t N = static_cast<int64_t>(s.h) * s.C();
  const int64_t w0 = static_cast<int64_t>(s.head_lo) * s.C() * s.d_kv;
  const int64_t pk = s.T * s.h * s.d_nope, pv = s.T * s.h * s.d_v;
  Operand<float> A{L, s.d_kv, 0, s.T, s.d_kv};
  if (s.bf16) {
    typedef Side<MmaBf16, 2, true, BM, float> SA;
    typedef Side<MmaBf16, 1, true, BN, bf16_t> SB;
    Operand<bf16_t> B{static_cast<const bf16_t*>(w) + w0, s.d_kv, 0, N, s.d_kv};
    if (s.split) {
      EpiKvUp<half_t, 2> e{static_cast<half_t*>(k_nope), static_cast<half_t*>(v), s.T, static_cast<int>(N),
                           s.C(), s.d_nope, s.d_v, s.h, pk, pv};
      return run_gemm<MmaBf16, SA, SB>(A, B, e, s.T, N, s.d_kv, 1, st);
    }
    EpiKvUp<half_t, 1> e{static_cast<half_t*>(k_nope), static_cast<half_t*>(v), s.T, static_cast<int>(N),
                         s.C(), s.d_nope, s.d_v, s.h, pk, pv};
    return run_gemm<MmaBf16, SA, SB>(A, B, e, s.T, N, s.d_kv, 1, st);
  }
  typedef Side<MmaF32, 1, true, BM, float> SA;
  typedef Side<MmaF32, 1, true, BN, float> SB;
  Operand<float> B{static_cast<const float*>(w) + w0, s.d_kv, 0, N, s.d_kv};
  EpiKvUp<float, 1> e{static_cast<float*>(k_nope), static_cast<float*>(v), s.T, static_cast<int>(N),
                      s.C(), s.d_nope, s.d_v, s.h, 0, 0};
  return run_gemm<MmaF32, SA, SB>(A, B, e, s.T, N, s.d_kv, 1, st);
}

// Absorbed form [LAGA §3.2 (B2)], per local head i (batch z = i):
//   absorb    q_abs[t, i, c] = sum_n q_nope[t, i, n] W[i, n, c]        (c < d_kv)
//   un-absorb o[t, i, d]     = sum_c acc[t, i, c] W[i, d_nope + d, c]  (d < d_v)
hipError_t launch_absorb_q(const Shape& s, const void* q, const void* w, void* q_abs, hipStream_t st) {
  const int64_t w0 = static_cast<int64_t>(s.head_lo) * s.C() * s.d_kv;
  typedef Side<MmaBf16, 1, true, BM, bf16_t> SA;   // q_nope rows, n contiguous
  typedef Side<MmaBf16, 1, false, BN, bf16_t> SB;  // W^k[i]: c contiguous, n strides memory
  Operand<bf16_t> A{static_cast<const bf16_t*>(q), static_cast<int64_t>(s.h) * s.d_qk(), 0, s.T, s.d_nope, s.d_qk()};
  Operand<bf16_t> B{static_cast<const bf16_t*>(w) + w0, s.d_kv, 0, s.d_kv, s.d_nope,
                    static_cast<int64_t>(s.C()) * s.d_kv};
  EpiHalf e{static_cast<half_t*>(q_abs), s.T, s.d_kv, static_cast<int64_t>(s.h) * s.d_kv, s.d_kv};
  return run_gemm<MmaBf16, SA, SB>(A, B, e, s.T, s.d_kv, s.d_nope, 1, st, s.h);
}

hipError_t launch_unabsorb_o(const Shape& s, const float* acc, const void* w, float* o, hipStream_t st) {
  const int64_t w0 = static_cast<int64_t>(s.head_lo) * s.C() * s.d_kv + static_cast<int64_t>(s.d_nope) * s.d_kv;
  typedef Side<MmaBf16, 2, true, BM, float> SA;   // acc rows in fp32, split into bf16 hi + lo while staged
  typedef Side<MmaBf16, 1, true, BN, bf16_t> SB;  // W^v[i] rows, c contiguous
  Operand<float> A{acc, static_cast<int64_t>(s.h) * s.d_kv, 0, s.T, s.d_kv, s.d_kv};
  Operand<bf16_t> B{static_cast<const bf16_t*>(w) + w0, s.d_kv, 0, s.d_v, s.d_kv, static_cast<int64_t>(s.C()) * s.d_kv};
  EpiStore e{o, s.T, s.d_v, static_cast<int64_t>(s.h) * s.d_v, s.d_v};
  return run_gemm<MmaBf16, SA, SB>(A, B, e, s.T, s.d_v, s.d_kv, 1, st, s.h);
}

hipError_t launch_fold_dl(const Shape& s, const void* dkv, const void* w, float* dL, hipStream_t st) {
  const int64_t Kd = static_cast<int64_t>(s.h) * s.C();
  const int64_t w0 = static_cast<int64_t>(s.head_lo) * s.C() * s.d_kv;
  EpiStore e{dL, s.T, s.d_kv, s.d_kv, 0};
  if (s.bf16) {
    typedef Side<MmaBf16, 2, true, BM, bf16_t> SA;    // dKV[t, n]: bf16 hi/lo planes
    typedef Side<MmaBf16, 1, false, BN, bf16_t> SB;   // W_r[n, k]: reduction over n strides memory
    Operand<bf16_t> A{static_cast<const bf16_t*>(dkv), Kd, s.T * Kd, s.T, Kd};
    Operand<bf16_t> B{static_cast<const bf16_t*>(w) + w0, s.d_kv, 0, s.d_kv, Kd};
    return run_gemm<MmaBf16, SA, SB>(A, B, e, s.T, s.d_kv, Kd, 1, st);
  }
  typedef Side<MmaF32, 1, true, BM, float> SA;
  typedef Side<MmaF32, 1, false, BN, float> SB;
  Operand<float> A{static_cast<const float*>(dkv), Kd, 0, s.T, Kd};
  Operand<float> B{static_cast<const float*>(w) + w0, s.d_kv, 0, s.d_kv, Kd};
  return run_gemm<MmaF32, SA, SB>(A, B, e, s.T, s.d_kv, Kd, 1, st);
}

size_t fold_dw_partial_floats(const Shape& s) {
  return static_cast<size_t>(dw_chunks(s)) * s.h * s.C() * s.d_kv;
}

hipError_t launch_fold_dw(const Shape& s, const void* dkv, const void* lplanes, float* partial, float* d_w,
                          hipStream_t st) {
  const int64_t Mr = static_cast<int64_t>(s.h) * s.C();
  const int chunks = dw_chunks(s);
  EpiStore e{partial, Mr, s.d_kv, s.d_kv, Mr * s.d_kv};
  hipError_t err;
  if (s.bf16) {
    typedef Side<MmaBf16, 2, false, BM, bf16_t> SA;   // dKV[t, n] read as A(row = n, k = t)
    typedef Side<MmaBf16, 2, false, BN, bf16_t> SB;   // L[t, c] read as B(row = c, k = t)
    Operand<bf16_t> A{static_cast<const bf16_t*>(dkv), Mr, s.T * Mr, Mr, s.T};
    Operand<bf16_t> B{static_cast<const bf16_t*>(lplanes), s.d_kv, s.T * s.d_kv, s.d_kv, s.T};
    err = run_gemm<MmaBf16, SA, SB>(A, B, e, Mr, s.d_kv, s.T, chunks, st);
  } else {
    typedef Side<MmaF32, 1, false, BM, float> SA;
    typedef Side<MmaF32, 1, false, BN, float> SB;
    Operand<float> A{static_cast<const float*>(dkv), Mr, 0, Mr, s.T};
    Operand<float> B{static_cast<const float*>(lplanes), s.d_kv, 0, s.d_kv, s.T};
    err = run_gemm<MmaF32, SA, SB>(A, B, e, Mr, s.d_kv, s.T, chunks, st);
  }
  if (err != hipSuccess) return err;
  const int64_t n = Mr * s.d_kv;
  hipLaunchKernelGGL(chunk_sum_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                     partial, d_w + static_cast<int64_t>(s.head_lo) * s.C() * s.d_kv, n, chunks);
  return hipGetLastError();
}

}  // namespace laga
