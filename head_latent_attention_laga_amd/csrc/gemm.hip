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
// Two kernel templates, both with a (64 TM) x (64 TN) output tile per
// 256-thread workgroup (four wavefronts in 2x2, each TM x TN MFMA atoms of
// 32x32) and K taken 32 at a time, one barrier per step:
//  * gemm_dma_kernel (every bf16 product): operand slabs go from global memory
//    straight into a ring of LDS stages (no staging registers); the fp32
//    normalised latent of the up-projection (and the absorbed form's fp32
//    accumulator) is split into bf16 hi + lo as it is read from LDS, or, for
//    fp16 K/V storage, rounded to fp16 and multiplied by W converted to fp16
//    in a single fp16 product.  Short
//    steps (K = 512 for the up-projection) make load latency the limit, so
//    the tiles are small enough for 2-3 workgroups per CU.
//  * gemm_kernel (the float32 test dims): slabs move global -> registers ->
//    LDS, one step ahead.
// Operand orientation:
//   KC operands (k contiguous in memory) land as LDS rows [row][k] and are
//      read with 16-byte fragment loads;
//   RC operands (row contiguous: the k axis strides memory) land as [k][row]
//      and 16-bit fragments come from gfx950's transposing LDS read.
// Operands are stored as NS planes of the MFMA element type (x ~= sum of the
// planes), written by the producing kernels.  The product keeps the term
// pairs (sa, sb) with sa + sb < max(NSA, NSB), which makes the bf16 GEMM
// accurate to about 2^-16 relative.
#include <type_traits>

#include "attn_common.hpp"
#include "launch.hpp"

namespace laga {
namespace {

constexpr int BK = 32;
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
  // Conversions on the way into LDS: fp32 -> 16-bit (NS == 2: hi + lo planes;
  // NS == 1: one rounded plane), or bf16 -> fp16 (one plane).
  static constexpr bool SPLIT = !std::is_same<Src, E>::value;
  static constexpr bool FROM_F32 = std::is_same<Src, float>::value;
  static_assert(!SPLIT || (EPC == 8 && (FROM_F32 || (std::is_same<Src, bf16_t>::value && NS == 1 &&
                                                     std::is_same<E, half_t>::value))),
                "fp32 -> 16-bit planes or bf16 -> fp16 only");
  static constexpr int LD = KC ? BK + EPC : ROWS + (sizeof(E) == 2 ? 32 : 4);  // LDS pitch, elements
  static constexpr int PLANE = (KC ? ROWS : BK) * LD;
  static constexpr int BYTES = NS * PLANE * static_cast<int>(sizeof(E));
  static constexpr int CHUNKS = ROWS * BK / EPC;  // per plane
  static constexpr int PER = CHUNKS / kThreads;
  static_assert(CHUNKS % kThreads == 0, "whole chunks per thread");
  static constexpr int NP = SPLIT ? 1 : NS;  // planes read from memory
  static constexpr int WORDS = SPLIT && FROM_F32 ? 2 : 1;  // 16-byte words per chunk read

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

  // Buffer loads: one descriptor per plane whose range ends with the last
  // row (KC) or k-row (RC) of the slab that exists, so chunks past it read as
  // zero with no branch.  KC operands need K to be a multiple of BK; rows of
  // an RC slab past R read neighbouring data, which only reaches output rows
  // or columns that are never stored.
  __device__ void load(const Operand<Src>& op, int64_t row0, int64_t k0) {
    constexpr int es = sizeof(Src);
    const Src* base = op.p + (KC ? row0 * op.ld + k0 : k0 * op.ld + row0);
    int64_t lim = KC ? op.R - row0 : op.K - k0;
    if (lim > (KC ? ROWS : BK)) lim = KC ? ROWS : BK;
    const int nbytes = static_cast<int>(lim * op.ld) * es;
    const int ld_b = static_cast<int>(op.ld) * es;
#pragma unroll
    for (int s = 0; s < NP; ++s) {
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<Src*>(base + s * op.plane), 0, nbytes, 0x00020000);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        int r, k;
        chunk_pos(i * kThreads + static_cast<int>(threadIdx.x), r, k);
        const int off = KC ? r * ld_b + k * es : k * ld_b + r * es;
#pragma unroll
        for (int w = 0; w < WORDS; ++w) reg[s][i][w] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * w, 0, 0);
      }
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
      } else if constexpr (SPLIT && !FROM_F32) {  // bf16 -> fp16, exact within fp16's range
        const u16x8 x = __builtin_bit_cast(u16x8, reg[0][i][0]);
        half8 h;
#pragma unroll
        for (int j = 0; j < 8; ++j) h[j] = static_cast<half_t>(bf16_to_f32(x[j]));
        *reinterpret_cast<half8*>(dst) = h;
      } else if constexpr (SPLIT && NS == 1) {  // fp32 -> one rounded 16-bit plane
        E part[EPC];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const f32x4 x = __builtin_bit_cast(f32x4, reg[0][i][w]);
#pragma unroll
          for (int j = 0; j < 4; ++j) part[4 * w + j] = M::from_f32(x[j]);
        }
        *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<u32x4*>(part);
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
template <class KvT, int NS, int DN, int DV>
struct EpiKvUp {
  static_assert(NS == 1 || sizeof(KvT) == 2, "the split form stores fp16 + e4m3");
  static constexpr bool TRANS = true;  // takes 4 consecutive n of one row m
  static constexpr int C = DN + DV;
  KvT* kn; KvT* v; int64_t M; int N, h; int64_t plane_k, plane_v;
  // n .. n+3 lie in one head and one part (C, DN multiples of 4).
  __device__ void store4(int64_t m, int n, f32x4 val, int /*z*/) const {
    if (m >= M || n >= N) return;
    const int i = n / C, c = n % C;
    // Two explicit paths rather than a selected pointer: selecting between
    // the two struct fields made the compiler index a stack copy of them.
    if (c < DN) put(kn, plane_k, (m * h + i) * DN + c, val);
    else put(v, plane_v, (m * h + i) * DV + (c - DN), val);
  }
  __device__ static void put(KvT* base, int64_t plane, int64_t e, f32x4 val) {
    KvT hi[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) hi[j] = static_cast<KvT>(val[j]);
    if constexpr (sizeof(KvT) == 2)
      *reinterpret_cast<u16x4*>(base + e) = *reinterpret_cast<const u16x4*>(hi);
    else
      *reinterpret_cast<f32x4*>(base + e) = *reinterpret_cast<const f32x4*>(hi);
    if constexpr (NS == 2) {
      constexpr float sc = static_cast<float>(1 << kLoShift);
      uint8_t* lo = reinterpret_cast<uint8_t*>(base + plane);
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

// EpiStore into K-chunk partials (its own type, so that these launches are
// told apart from other stores of the same operand shapes in a trace).
struct EpiPart : EpiStore {};

// out as bf16 hi + lo planes (x = hi + lo to about 2^-16), four consecutive n at
// a time: hi at p[z * zstride + m * ld + n], lo at the same place + plane.
struct EpiPlanes {
  static constexpr bool TRANS = true;
  bf16_t* p; int64_t plane, M; int N; int64_t ld, zstride;
  __device__ void store4(int64_t m, int n, f32x4 val, int z) const {
    if (m >= M || n >= N) return;
    uint32_t h0, l0, h1, l1;
    split_bf16_pair(val[0], val[1], h0, l0);
    split_bf16_pair(val[2], val[3], h1, l1);
    const int64_t e = z * zstride + m * ld + n;
    *reinterpret_cast<u32x2*>(p + e) = u32x2{h0, h1};
    *reinterpret_cast<u32x2*>(p + plane + e) = u32x2{l0, l1};
  }
};

// out[m * ld + n] += val; columns n >= n0 go to out1[m * ld1 + n - n0] instead
// (one product whose output spans two accumulators).
struct EpiAccum {
  static constexpr bool TRANS = false;
  float* p; int64_t ld; float* p1; int64_t ld1; int64_t M; int N, n0;
  __device__ void operator()(int64_t m, int n, float val, int /*z*/) const {
    if (m >= M || n >= N) return;
    if (n < n0) p[m * ld + n] += val;
    else p1[m * ld1 + (n - n0)] += val;
  }
};

// ------------------------------------------------------------------- kernel
// Tiles (x = N tile, y = M tile, z = batch * nchunks + K chunk) come from a
// 1-D launch.  Workgroup ids are dealt round-robin to the 8 XCDs, each with
// its own L2; they are remapped so that every XCD takes one contiguous range
// of tiles in x-fastest order: the N tiles that share an A row block (and the
// M tiles that share a B block) then run on the same XCD and read those rows
// from HBM once instead of once per XCD.
template <class M, class SA, class SB, class EPI, int TM, int TN>
__global__ __launch_bounds__(kThreads, TM * TN > 4 ? 1 : 2) void gemm_kernel(Operand<typename SA::Src_t> A,
                                                                            Operand<typename SB::Src_t> B, EPI epi,
                                                                            int64_t k_chunk, int64_t K, int nchunks,
                                                                            int gx, int gy, int gz) {
  typedef typename M::elem E;
  constexpr int BM = 64 * TM, BN = 64 * TN;
  static_assert(SA::ROWS == BM && SB::ROWS == BN, "slab rows match the tile");
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

  f32x16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // One register stage of operand slabs in flight: the loads for step k + 1
  // are issued right after the barrier of step k and stored to the other LDS
  // buffer at the start of step k + 1, so one step of products (TM TN
  // products per k16 and term pair) covers the global-memory latency.
  typename SA::Slab sa;
  typename SB::Slab sb;
  constexpr int NSA = SA::Slab::NS_, NSB = SB::Slab::NS_;
  constexpr int NSMAX = NSA > NSB ? NSA : NSB;
  auto compute = [&](const E* as, const E* bs) {
#pragma unroll
    for (int kk = 0; kk < BK; kk += M::K) {
      typename M::frag af[NSA][TM], bfr[NSB][TN];
#pragma unroll
      for (int s = 0; s < NSA; ++s)
#pragma unroll
        for (int a = 0; a < TM; ++a) af[s][a] = SA::Slab::frag(as, s, wm * 32 * TM + a * 32, kk);
#pragma unroll
      for (int s = 0; s < NSB; ++s)
#pragma unroll
        for (int b = 0; b < TN; ++b) bfr[s][b] = SB::Slab::frag(bs, s, wn * 32 * TN + b * 32, kk);
#pragma unroll
      for (int s1 = 0; s1 < NSA; ++s1)
#pragma unroll
        for (int s2 = 0; s2 < NSB; ++s2) {
          if (s1 + s2 >= NSMAX) continue;
#pragma unroll
          for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int b = 0; b < TN; ++b) {
              // EPI::TRANS: the atom holds C^T (rows n, columns m).
              if constexpr (EPI::TRANS) acc[a][b] = M::mma(bfr[s2][b], af[s1][a], acc[a][b]);
              else acc[a][b] = M::mma(af[s1][a], bfr[s2][b], acc[a][b]);
            }
        }
    }
  };
  // One step: publish the slabs of step k0 (held in sa/sb) into LDS buffer
  // `buf`, refill sa/sb with step k0 + BK, compute step k0.  A buffer is
  // written two steps after it was read; the barrier of the step in between
  // orders the two.
  auto step = [&](int64_t k0, int buf) {
    E* as = reinterpret_cast<E*>(lds + buf * STAGE);
    E* bs = reinterpret_cast<E*>(lds + buf * STAGE + SA::BYTES);
    sa.store(as);
    sb.store(bs);
    __syncthreads();
    if (k0 + BK < kend) {
      sa.load(A, m0, k0 + BK);
      sb.load(B, n0, k0 + BK);
    }
    compute(as, bs);
  };

  if (kbeg < kend) {
    sa.load(A, m0, kbeg);
    sb.load(B, n0, kbeg);
  }
  // Unrolled by two so that each step names its buffer as a constant.
  for (int64_t k0 = kbeg; k0 < kend; k0 += 2 * BK) {
    step(k0, 0);
    if (k0 + BK < kend) step(k0 + BK, 1);
  }
  // C[r]: row 8*(r/4) + 4*(lane/32) + r%4 of the atom, column lane%32.
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      if constexpr (EPI::TRANS) {
        const int64_t m = m0 + wm * 32 * TM + a * 32 + (lane % 32);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = static_cast<int>(n0 + wn * 32 * TN + b * 32 + 8 * g + 4 * (lane / 32));
          const f32x4 v4 = {acc[a][b][4 * g], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2], acc[a][b][4 * g + 3]};
          epi.store4(m, n, v4, bz);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + wm * 32 * TM + a * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
          const int n = static_cast<int>(n0 + wn * 32 * TN + b * 32 + (lane % 32));
          epi(m, n, acc[a][b][r], bz);
        }
      }
    }
}

// Operand description: MFMA type, planes, orientation, rows per tile, source element.
template <class M, int NS, bool KC_, int ROWS_, class Src>
struct Side {
  struct Slab : SlabT<M, NS, KC_, ROWS_, Src> { static constexpr int NS_ = NS; };
  typedef Src Src_t;
  static constexpr int BYTES = Slab::BYTES;
  static constexpr int ROWS = ROWS_;
  static constexpr bool KC = KC_;
};

// Launch with (64 TM) x (64 TN) tiles; SA / SB must have 64 TM / 64 TN rows.
template <class M, int TM, int TN, class SA, class SB, class EPI>
hipError_t run_gemm(Operand<typename SA::Src_t> A, Operand<typename SB::Src_t> B, EPI epi, int64_t Mrows,
                    int64_t Ncols, int64_t K, int chunks, hipStream_t st, int batches = 1) {
  if ((SA::KC || SB::KC) && K % BK != 0) return hipErrorInvalidValue;  // KC slabs take whole BK steps
  const int64_t per = ((K + chunks - 1) / chunks + BK - 1) / BK * BK;
  const int nchunks = static_cast<int>((K + per - 1) / per);
  const int gx = static_cast<int>((Ncols + 64 * TN - 1) / (64 * TN)),
            gy = static_cast<int>((Mrows + 64 * TM - 1) / (64 * TM)), gz = nchunks * batches;
  hipLaunchKernelGGL((gemm_kernel<M, SA, SB, EPI, TM, TN>), dim3(static_cast<unsigned>(gx * gy * gz)),
                     dim3(kThreads), 0, st, A, B, epi, per, K, nchunks, gx, gy, gz);
  return hipGetLastError();
}

// ------------------------------------------------------- DMA-fed GEMM kernel
// For bf16 matrix-core products (every GEMM of the path except the float32
// test dims).  With K = 512 (the up-projection) a 32-wide k step holds only a
// few hundred cycles of products per wavefront, too few to hide the latency
// of the next step's global loads when they pass through registers.  Here the
// operand slabs go from global memory straight into LDS (buffer loads with an
// LDS destination: no staging registers, no LDS store instructions), NST - 1
// steps ahead, into a ring of NST stages.  Each wavefront issues the same
// number of 1 KB loads per stage, so waiting for a stage is one
// s_waitcnt vmcnt(N) before the step's barrier.
//
// Operand layouts in a stage (16-byte slots XOR-swizzled so that the reads
// below touch every LDS bank once per 16 or 32 lanes):
//   DKC<NP, bf16>:  ROWS lines x 64 B (k contiguous), slot c of line r at c ^ ((r >> 2) & 3)
//   DKC<1, float>:  ROWS lines x 128 B, slot c of line r at c ^ ((r >> 1) & 7); the
//                   fp32 values become bf16 hi + lo terms as they are read
//   DRC<NP>:        BK k-lines x ROWS * 2 B (rows contiguous), slot c of k-line k at
//                   c ^ 4 (k % 4), read with transposing reads
// A slot's source address follows from its LDS position, so the swizzle costs
// nothing on the load side.

// 16 bytes per lane from `rs` (byte offset voff + soff) to lds + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(lds), 16, voff, soff, 0, 0);
}


// k-contiguous operand: NP planes of Src, ROWS rows per tile.  HALF: the
// operand enters fp16 products as one fp16 term (fp32 rounded, or bf16
// converted, as it is read from LDS) instead of bf16 terms.
template <int NP_, class Src, int ROWS_, bool HALF_ = false>
struct DKC {
  static constexpr int ROWS = ROWS_, NP = NP_;
  static constexpr bool HALF = HALF_;
  static constexpr bool F32 = std::is_same<Src, float>::value;
  static constexpr bool SRC_F32 = F32;  // stored as fp32 in memory
  static_assert(!F32 || NP == 1, "one fp32 plane, split when read");
  static_assert(!HALF || NP == 1, "one plane converted to fp16");
  static constexpr int NT = HALF ? 1 : (F32 ? 2 : NP);  // 16-bit terms per element
  static constexpr int LINE = BK * static_cast<int>(sizeof(Src));  // 64 or 128 bytes
  static constexpr int SPL = LINE / 16;
  static constexpr int PLANE = ROWS * LINE;
  static constexpr int BYTES = NP * PLANE;
  static constexpr int SLOTS = PLANE / 16;
  static_assert(SLOTS % (4 * kWave) == 0, "whole 1 KB loads for every wavefront");
  static constexpr int IPW = SLOTS / (4 * kWave);  // loads per wavefront and plane
  __device__ static int swz(int line) { return F32 ? (line >> 1) & 7 : (line >> 2) & 3; }
  // Source byte offset (within the step's slab) of load i of wavefront w for this lane.
  __device__ static int voff(int i, int w, int lane, int ld_bytes) {
    const int q = (i * 4 + w) * kWave + lane, line = q / SPL, c = (q % SPL) ^ swz(line);
    return line * ld_bytes + c * 16;
  }
  // Lines of the step's slab that exist: rows past R read as zero.
  __device__ static int lines(int64_t r_left, int64_t /*k_left*/) {
    return static_cast<int>(r_left < ROWS ? r_left : ROWS);
  }
  // Per-lane byte offsets of the atom at row 32 * lane-independent offset, k step kk:
  // bf16: one 16-byte slot per term; fp32: two slots.
  struct Lane { int o[2][2]; };  // [kk / 16][half]
  __device__ static Lane lane_offsets(int row0) {
    const int lane = threadIdx.x % kWave, hf = lane / 32, line = row0 + lane % 32;
    Lane L;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if constexpr (F32) {
        const int c0 = (16 * s + 8 * hf) / 4;
        L.o[s][0] = line * LINE + ((c0) ^ swz(line)) * 16;
        L.o[s][1] = line * LINE + ((c0 + 1) ^ swz(line)) * 16;
      } else {
        L.o[s][0] = line * LINE + (((16 * s + 8 * hf) / 8) ^ swz(line)) * 16;
        L.o[s][1] = 0;
      }
    }
    return L;
  }
  // The 16-bit terms of the fragment of atom `a` (rows row0 + 32 a ..) at k step s.
  __device__ static void frag(const char* st, const Lane& L, int a, int s, u16x8* out) {
    const char* base = st + a * 32 * LINE;
    if constexpr (HALF && F32) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(base + L.o[s][0]);
      const f32x4 y = *reinterpret_cast<const f32x4*>(base + L.o[s][1]);
      const half8 h = {static_cast<half_t>(x[0]), static_cast<half_t>(x[1]), static_cast<half_t>(x[2]),
                       static_cast<half_t>(x[3]), static_cast<half_t>(y[0]), static_cast<half_t>(y[1]),
                       static_cast<half_t>(y[2]), static_cast<half_t>(y[3])};
      out[0] = __builtin_bit_cast(u16x8, h);
    } else if constexpr (HALF) {  // bf16 -> fp16, exact within fp16's normal range
      const u16x8 x = *reinterpret_cast<const u16x8*>(base + L.o[s][0]);
      half8 h;
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = static_cast<half_t>(bf16_to_f32(x[j]));
      out[0] = __builtin_bit_cast(u16x8, h);
    } else if constexpr (F32) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(base + L.o[s][0]);
      const f32x4 y = *reinterpret_cast<const f32x4*>(base + L.o[s][1]);
      uint32_t h[4], l[4];
      split_bf16_pair(x[0], x[1], h[0], l[0]);
      split_bf16_pair(x[2], x[3], h[1], l[1]);
      split_bf16_pair(y[0], y[1], h[2], l[2]);
      split_bf16_pair(y[2], y[3], h[3], l[3]);
      out[0] = __builtin_bit_cast(u16x8, u32x4{h[0], h[1], h[2], h[3]});
      out[1] = __builtin_bit_cast(u16x8, u32x4{l[0], l[1], l[2], l[3]});
    } else {
#pragma unroll
      for (int p = 0; p < NP; ++p) out[p] = *reinterpret_cast<const u16x8*>(base + p * PLANE + L.o[s][0]);
    }
  }
  static constexpr bool KC = true;
};

// Row-contiguous operand (k strides memory): NP bf16 planes, ROWS rows per tile.
template <int NP_, int ROWS_>
struct DRC {
  static constexpr int ROWS = ROWS_, NP = NP_, NT = NP_;
  static constexpr bool HALF = false, SRC_F32 = false;
  static constexpr int LINE = ROWS * 2;  // one k-line
  static constexpr int SPL = LINE / 16;
  static_assert(LINE % 256 == 0, "k-lines span whole bank windows");
  static constexpr int PLANE = BK * LINE;
  static constexpr int BYTES = NP * PLANE;
  static constexpr int SLOTS = PLANE / 16;
  static_assert(SLOTS % (4 * kWave) == 0, "whole 1 KB loads for every wavefront");
  static constexpr int IPW = SLOTS / (4 * kWave);
  __device__ static int swz(int kl) { return 4 * (kl & 3); }
  __device__ static int voff(int i, int w, int lane, int ld_bytes) {
    const int q = (i * 4 + w) * kWave + lane, kl = q / SPL, c = (q % SPL) ^ swz(kl);
    return kl * ld_bytes + c * 16;
  }
  __device__ static int lines(int64_t /*r_left*/, int64_t k_left) {
    return static_cast<int>(k_left < BK ? k_left : BK);
  }
  // Transposing read of rows (k-lines) k0 + 8 hf + s/4 (+4) and columns
  // n0 + 16 (g % 2) + 4 (s % 4) of a swizzled stage (lane = 16 g + s): the
  // per-lane byte offset for the atom at column n0 (a multiple of 32);
  // k steps add 16 lines.
  struct Lane { int o[8]; };  // per atom of the wavefront (up to 8)
  template <int NA>
  __device__ static Lane lane_offsets(int col0) {
    static_assert(NA <= 8, "atoms per wavefront");
    const int lane = threadIdx.x % kWave, g = lane / 16, s = lane % 16, hf = lane / 32;
    const int kl = 8 * hf + s / 4;  // k-line within the step (% 4 == (s / 4) % 4)
    Lane L;
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      const int chunk = (col0 + 32 * a) / 8 + 2 * (g % 2) + (s % 4) / 2;
      L.o[a] = kl * LINE + (chunk ^ swz(kl)) * 16 + 8 * (s % 2);
    }
    return L;
  }
  __device__ static void frag(const char* st, const Lane& L, int a, int s, u16x8* out) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const char* b = st + p * PLANE + L.o[a] + s * 16 * LINE;
      const s16x4 x = ds_read_tr16(b);
      const s16x4 y = ds_read_tr16(b + 4 * LINE);
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      out[p] = __builtin_bit_cast(u16x8, s16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]});
    }
  }
  static constexpr bool KC = false;
};

// C[m, n] = sum_k A[m, k] B[n, k] over the term pairs (ta, tb) with
// ta + tb < max(NT_A, NT_B), bf16 MFMAs, (64 TM) x (64 TN) tiles, NST stages.
template <class OA, class OB, class EPI, int TM, int TN, int NST, int OCC>
__global__ __launch_bounds__(kThreads, OCC) void gemm_dma_kernel(Operand<bf16_t> A16, Operand<float> A32,
                                                                 Operand<bf16_t> B, EPI epi, int64_t k_chunk,
                                                                 int64_t K, int nchunks, int gx, int gy, int gz) {
  static_assert(OA::ROWS == 64 * TM && OB::ROWS == 64 * TN, "operand rows match the tile");
  static_assert(OA::HALF == OB::HALF, "both operands fp16 or both bf16 terms");
  constexpr int STAGE = OA::BYTES + OB::BYTES;
  constexpr int IPS = OA::IPW * OA::NP + OB::IPW * OB::NP;  // loads per wavefront and stage
  static_assert((NST - 2) * IPS < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char lds[NST * STAGE];
  constexpr bool A_F32 = OA::SRC_F32;  // fp32 A (split or rounded when read)

  const int total = gx * gy * gz;
  const int id = static_cast<int>(blockIdx.x);
  const int tile = total % 8 == 0 ? (id % 8) * (total / 8) + id / 8 : id;
  const int bx = tile % gx, by = (tile / gx) % gy, bz = tile / (gx * gy);
  const int lane = threadIdx.x % kWave;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int wm = wv / 2, wn = wv % 2;
  const int64_t m0 = static_cast<int64_t>(by) * 64 * TM;
  const int64_t n0 = static_cast<int64_t>(bx) * 64 * TN;
  const int chunk = bz % nchunks, batch = bz / nchunks;
  const int64_t kbeg = static_cast<int64_t>(chunk) * k_chunk;
  const int64_t kend = (kbeg + k_chunk < K) ? kbeg + k_chunk : K;
  const int nsteps = static_cast<int>((kend - kbeg + BK - 1) / BK);

  // Operand bases at the tile's first row / k, and per-lane source offsets.
  const int es_a = A_F32 ? 4 : 2;
  const int64_t lda = A_F32 ? A32.ld : A16.ld, Ra = A_F32 ? A32.R : A16.R;
  const char* abase = A_F32 ? reinterpret_cast<const char*>(A32.p + batch * A32.zstride)
                            : reinterpret_cast<const char*>(A16.p + batch * A16.zstride);
  abase += (OA::KC ? m0 * lda + kbeg : kbeg * lda + m0) * es_a;
  const int64_t aplane = (A_F32 ? 0 : A16.plane) * es_a;
  const char* bbase = reinterpret_cast<const char*>(B.p + batch * B.zstride) +
                      (OB::KC ? n0 * B.ld + kbeg : kbeg * B.ld + n0) * 2;
  const int64_t bplane = B.plane * 2;
  const int lda_b = static_cast<int>(lda) * es_a, ldb_b = static_cast<int>(B.ld) * 2;
  int va[OA::IPW], vb[OB::IPW];
#pragma unroll
  for (int i = 0; i < OA::IPW; ++i) va[i] = OA::voff(i, wv, lane, lda_b);
#pragma unroll
  for (int i = 0; i < OB::IPW; ++i) vb[i] = OB::voff(i, wv, lane, ldb_b);

  // Issue step `it` (k = kbeg + it BK) into stage `sb`; steps past the end
  // read zeros (an empty range), so every step issues the same loads.
  auto issue = [&](int it, char* sb) {
    const int64_t k0 = static_cast<int64_t>(it) * BK;
    const int64_t kl = kend - kbeg - k0;
    const int la = OA::lines(Ra - m0, kl), lb = OB::lines(B.R - n0, kl);
    const int64_t adv_a = OA::KC ? k0 * es_a : k0 * lda_b, adv_b = OB::KC ? k0 * 2 : k0 * ldb_b;
#pragma unroll
    for (int p = 0; p < OA::NP; ++p) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(abase + p * aplane + adv_a), 0, kl > 0 ? la * lda_b : 0, 0x00020000);
#pragma unroll
      for (int i = 0; i < OA::IPW; ++i) dma16(rs, sb + p * OA::PLANE + (i * 4 + wv) * 1024, va[i], 0);
    }
#pragma unroll
    for (int p = 0; p < OB::NP; ++p) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(bbase + p * bplane + adv_b), 0, kl > 0 ? lb * ldb_b : 0, 0x00020000);
#pragma unroll
      for (int i = 0; i < OB::IPW; ++i)
        dma16(rs, sb + OA::BYTES + p * OB::PLANE + (i * 4 + wv) * 1024, vb[i], 0);
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  typename OA::Lane la_off;
  typename OB::Lane lb_off;
  if constexpr (OA::KC) la_off = OA::lane_offsets(wm * 32 * TM);
  else la_off = OA::template lane_offsets<TM>(wm * 32 * TM);
  if constexpr (OB::KC) lb_off = OB::lane_offsets(wn * 32 * TN);
  else lb_off = OB::template lane_offsets<TN>(wn * 32 * TN);

  auto compute = [&](const char* st) {
    const char* as = st;
    const char* bs = st + OA::BYTES;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      u16x8 af[TM][OA::NT], bfr[TN][OB::NT];
#pragma unroll
      for (int a = 0; a < TM; ++a) OA::frag(as, la_off, a, s, af[a]);
#pragma unroll
      for (int b = 0; b < TN; ++b) OB::frag(bs, lb_off, b, s, bfr[b]);
      constexpr int NTM = OA::NT > OB::NT ? OA::NT : OB::NT;
#pragma unroll
      for (int ta = 0; ta < OA::NT; ++ta)
#pragma unroll
        for (int tb = 0; tb < OB::NT; ++tb) {
          if (ta + tb >= NTM) continue;
#pragma unroll
          for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int b = 0; b < TN; ++b) {
              if constexpr (OA::HALF) {
                const half8 x = __builtin_bit_cast(half8, af[a][ta]), y = __builtin_bit_cast(half8, bfr[b][tb]);
                if constexpr (EPI::TRANS) acc[a][b] = MmaF16::mma(y, x, acc[a][b]);
                else acc[a][b] = MmaF16::mma(x, y, acc[a][b]);
              } else if constexpr (EPI::TRANS) {
                acc[a][b] = MmaBf16::mma(bfr[b][tb], af[a][ta], acc[a][b]);
              } else {
                acc[a][b] = MmaBf16::mma(af[a][ta], bfr[b][tb], acc[a][b]);
              }
            }
        }
    }
  };

  // Prologue: NST - 1 steps in flight.
#pragma unroll
  for (int it = 0; it < NST - 1; ++it) issue(it, lds + it * STAGE);
  // Unrolled by NST so that every stage offset is a constant.
  for (int it0 = 0; it0 < nsteps; it0 += NST) {
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      const int it = it0 + j;
      if (it >= nsteps) break;
      wait_vmcnt<(NST - 2) * IPS>();  // this wavefront's loads of step `it` have landed
      __syncthreads();                // so have every wavefront's; stage (it - 1) % NST is free
      issue(it + NST - 1, lds + ((j + NST - 1) % NST) * STAGE);
      compute(lds + j * STAGE);
    }
  }
  wait_vmcnt<0>();  // no load into LDS outlives the workgroup

  // C[r]: row 8*(r/4) + 4*(lane/32) + r%4 of the atom, column lane%32.
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      if constexpr (EPI::TRANS) {
        const int64_t m = m0 + wm * 32 * TM + a * 32 + (lane % 32);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = static_cast<int>(n0 + wn * 32 * TN + b * 32 + 8 * g + 4 * (lane / 32));
          const f32x4 v4 = {acc[a][b][4 * g], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2], acc[a][b][4 * g + 3]};
          epi.store4(m, n, v4, bz);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + wm * 32 * TM + a * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
          const int n = static_cast<int>(n0 + wn * 32 * TN + b * 32 + (lane % 32));
          epi(m, n, acc[a][b][r], bz);
        }
      }
    }
}

// Launch of the DMA kernel: A either 16-bit planes (A16) or one fp32 plane (A32).
template <class OA, class OB, int TM, int TN, int NST, int OCC, class EPI>
hipError_t run_gemm_dma(Operand<bf16_t> A16, Operand<float> A32, Operand<bf16_t> B, EPI epi, int64_t Mrows,
                        int64_t Ncols, int64_t K, int chunks, hipStream_t st, int batches = 1) {
  if ((OA::KC || OB::KC) && K % BK != 0) return hipErrorInvalidValue;  // k-contiguous slabs take whole steps
  const int64_t per = ((K + chunks - 1) / chunks + BK - 1) / BK * BK;
  const int nchunks = static_cast<int>((K + per - 1) / per);
  const int gx = static_cast<int>((Ncols + 64 * TN - 1) / (64 * TN)),
            gy = static_cast<int>((Mrows + 64 * TM - 1) / (64 * TM)), gz = nchunks * batches;
  hipLaunchKernelGGL((gemm_dma_kernel<OA, OB, EPI, TM, TN, NST, OCC>), dim3(static_cast<unsigned>(gx * gy * gz)),
                     dim3(kThreads), 0, st, A16, A32, B, epi, per, K, nchunks, gx, gy, gz);
  return hipGetLastError();
}

// Tiles (in 64-row units) of the W_kv_b gradient GEMM, rows h * C and columns
// d_kv, for bfloat16 inputs (float32 inputs use 128 x 128).
constexpr int DW_TM = 2, DW_TN = 2;

// Number of K chunks for the W_kv_b gradient so that about DW_TARGET
// workgroups run.
constexpr int DW_TARGET = 512;
int dw_chunks(const Shape& s) {
  const int tm = s.bf16 ? 64 * DW_TM : 128, tn = s.bf16 ? 64 * DW_TN : 128;
  const int64_t tiles = ((static_cast<int64_t>(s.h) * s.C() + tm - 1) / tm) * ((s.d_kv + tn - 1) / tn);
  int64_t c = (DW_TARGET + tiles - 1) / tiles;
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
  if (s.bf16 && s.d_nope == 128 && s.d_v == 128) {
    // L as bf16 hi + lo (formed as it is read from LDS), W exact in bf16:
    // K / V to about 2^-16 relative, then stored as split planes.  With
    // K = 512 the steps are short, so the tiles are sized for two workgroups
    // per CU whose loads cover each other's latency (measured against 64-
    // to 256-row tiles, 2-4 stages and 1-3 workgroups per CU).
    Operand<bf16_t> B{static_cast<const bf16_t*>(w) + w0, s.d_kv, 0, N, s.d_kv};
    if (s.split) {
      EpiKvUp<half_t, 2, 128, 128> e{static_cast<half_t*>(k_nope), static_cast<half_t*>(v), s.T,
                                     static_cast<int>(N), s.h, pk, pv};
      return run_gemm_dma<DKC<1, float, 128>, DKC<1, bf16_t, 256>, 2, 4, 2, 2>(Operand<bf16_t>{}, A, B, e, s.T, N,
                                                                               s.d_kv, 1, st);
    }
    // Single fp16 storage: one fp16 product of L and W, both rounded to fp16
    // as they are read from LDS (K / V to about 2^-11 relative before their
    // own fp16 rounding), half the matrix-core work of the hi/lo form.
    EpiKvUp<half_t, 1, 128, 128> e{static_cast<half_t*>(k_nope), static_cast<half_t*>(v), s.T, static_cast<int>(N),
                                   s.h, pk, pv};
    return run_gemm_dma<DKC<1, float, 256, true>, DKC<1, bf16_t, 128, true>, 4, 2, 2, 2>(Operand<bf16_t>{}, A, B, e,
                                                                                         s.T, N, s.d_kv, 1, st);
  }
  if (s.bf16 || s.d_nope != 32 || s.d_v != 32) return hipErrorNotSupported;
  typedef Side<MmaF32, 1, true, 128, float> SA;
  typedef Side<MmaF32, 1, true, 128, float> SB;
  Operand<float> B{static_cast<const float*>(w) + w0, s.d_kv, 0, N, s.d_kv};
  EpiKvUp<float, 1, 32, 32> e{static_cast<float*>(k_nope), static_cast<float*>(v), s.T, static_cast<int>(N),
                              s.h, 0, 0};
  return run_gemm<MmaF32, 2, 2, SA, SB>(A, B, e, s.T, N, s.d_kv, 1, st);
}

// Absorbed form [LAGA §3.2 (B2)], per local head i (batch z = i):
//   absorb    q_abs[t, i, c] = sum_n q_nope[t, i, n] W[i, n, c]        (c < d_kv)
//   un-absorb o[t, i, d]     = sum_c acc[t, i, c] W[i, d_nope + d, c]  (d < d_v)
hipError_t launch_absorb_q(const Shape& s, const void* q, const void* w, void* q_abs, hipStream_t st) {
  const int64_t w0 = static_cast<int64_t>(s.head_lo) * s.C() * s.d_kv;
  typedef DKC<1, bf16_t, 128> OA;  // q_nope rows, n contiguous
  typedef DRC<1, 256> OB;          // W^k[i]: c contiguous, n strides memory
  Operand<bf16_t> A{static_cast<const bf16_t*>(q), static_cast<int64_t>(s.h) * s.d_qk(), 0, s.T, s.d_nope, s.d_qk()};
  Operand<bf16_t> B{static_cast<const bf16_t*>(w) + w0, s.d_kv, 0, s.d_kv, s.d_nope,
                    static_cast<int64_t>(s.C()) * s.d_kv};
  EpiHalf e{static_cast<half_t*>(q_abs), s.T, s.d_kv, static_cast<int64_t>(s.h) * s.d_kv, s.d_kv};
  return run_gemm_dma<OA, OB, 2, 4, 4, 1>(A, Operand<float>{}, B, e, s.T, s.d_kv, s.d_nope, 1, st, s.h);
}

hipError_t launch_unabsorb_o(const Shape& s, const float* acc, const void* w, float* o, hipStream_t st) {
  const int64_t w0 = static_cast<int64_t>(s.head_lo) * s.C() * s.d_kv + static_cast<int64_t>(s.d_nope) * s.d_kv;
  typedef DKC<1, float, 256> OA;   // acc rows in fp32, split into bf16 hi + lo as they are read
  typedef DKC<1, bf16_t, 128> OB;  // W^v[i] rows, c contiguous
  Operand<float> A{acc, static_cast<int64_t>(s.h) * s.d_kv, 0, s.T, s.d_kv, s.d_kv};
  Operand<bf16_t> B{static_cast<const bf16_t*>(w) + w0, s.d_kv, 0, s.d_v, s.d_kv, static_cast<int64_t>(s.C()) * s.d_kv};
  EpiStore e{o, s.T, s.d_v, static_cast<int64_t>(s.h) * s.d_v, s.d_v};
  return run_gemm_dma<OA, OB, 4, 2, 3, 1>(Operand<bf16_t>{}, A, B, e, s.T, s.d_v, s.d_kv, 1, st, s.h);
}

hipError_t launch_fold_dl(const Shape& s, const void* dkv, const void* w, float* dL, hipStream_t st) {
  const int64_t Kd = static_cast<int64_t>(s.h) * s.C();
  const int64_t w0 = static_cast<int64_t>(s.head_lo) * s.C() * s.d_kv;
  EpiStore e{dL, s.T, s.d_kv, s.d_kv, 0};
  if (s.bf16) {
    typedef DKC<2, bf16_t, 64> OA;  // dKV[t, n]: bf16 hi/lo planes
    typedef DRC<1, 256> OB;         // W_r[n, k]: reduction over n strides memory
    Operand<bf16_t> A{static_cast<const bf16_t*>(dkv), Kd, s.T * Kd, s.T, Kd};
    Operand<bf16_t> B{static_cast<const bf16_t*>(w) + w0, s.d_kv, 0, s.d_kv, Kd};
    return run_gemm_dma<OA, OB, 1, 4, 3, 2>(A, Operand<float>{}, B, e, s.T, s.d_kv, Kd, 1, st);
  }
  typedef Side<MmaF32, 1, true, 128, float> SA;
  typedef Side<MmaF32, 1, false, 128, float> SB;
  Operand<float> A{static_cast<const float*>(dkv), Kd, 0, s.T, Kd};
  Operand<float> B{static_cast<const float*>(w) + w0, s.d_kv, 0, s.d_kv, Kd};
  return run_gemm<MmaF32, 2, 2, SA, SB>(A, B, e, s.T, s.d_kv, Kd, 1, st);
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
    typedef DRC<2, 64 * DW_TM> OA;  // dKV[t, n] read as A(row = n, k = t)
    typedef DRC<2, 64 * DW_TN> OB;  // L[t, c] read as B(row = c, k = t)
    Operand<bf16_t> A{static_cast<const bf16_t*>(dkv), Mr, s.T * Mr, Mr, s.T};
    Operand<bf16_t> B{static_cast<const bf16_t*>(lplanes), s.d_kv, s.T * s.d_kv, s.d_kv, s.T};
    err = run_gemm_dma<OA, OB, DW_TM, DW_TN, 2, 2>(A, Operand<float>{}, B, e, Mr, s.d_kv, s.T, chunks, st);
  } else {
    typedef Side<MmaF32, 1, false, 128, float> SA;
    typedef Side<MmaF32, 1, false, 128, float> SB;
    Operand<float> A{static_cast<const float*>(dkv), Mr, 0, Mr, s.T};
    Operand<float> B{static_cast<const float*>(lplanes), s.d_kv, 0, s.d_kv, s.T};
    err = run_gemm<MmaF32, 2, 2, SA, SB>(A, B, e, Mr, s.d_kv, s.T, chunks, st);
  }
  if (err != hipSuccess) return err;
  const int64_t n = Mr * s.d_kv;
  hipLaunchKernelGGL(chunk_sum_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                     partial, d_w + static_cast<int64_t>(s.head_lo) * s.C() * s.d_kv, n, chunks);
  return hipGetLastError();
}

// ------------------------------------------------ absorbed form (B2), backward
// Products of laga_absorbed_bwd (absorbed.hip sequences them).  Every operand
// that is not exact in bf16 enters as bf16 hi + lo planes, and the products
// keep the term pairs hi.hi, hi.lo, lo.hi: fp32-class results.  Plane
// buffers: qx [2][R][576] (q_abs || q_rope, R = T h rows r = t h + i), dacc
// [2][R][512], kxp [2][Tp][576] (L || k_pe); per chunk of rows r0 .. r0 + Rc:
// P and c.dS as [2][Rc][ldu] planes, S and dP as fp32 [Rc][ldu].
namespace {
constexpr int B2_DQ = 576, B2_DL = 512;
}

hipError_t launch_b2_planes(const Shape& s, const void* x, int64_t x_ld, int64_t x_z, int64_t w_row0,
                            const void* w, void* out, int64_t out_plane, int64_t out_ld, hipStream_t st) {
  // out[t h + i][c] = sum_n x[t][i][n] W[head_lo + i][w_row0 + n][c], n < 128, as bf16 hi/lo planes
  // (x: token pitch x_ld, head pitch x_z elements; out: row pitch out_ld).
  const int64_t w0 = static_cast<int64_t>(s.head_lo) * s.C() * s.d_kv + w_row0 * s.d_kv;
  Operand<bf16_t> A{static_cast<const bf16_t*>(x), x_ld, 0, s.T, 128, x_z};
  Operand<bf16_t> B{static_cast<const bf16_t*>(w) + w0, s.d_kv, 0, s.d_kv, 128, static_cast<int64_t>(s.C()) * s.d_kv};
  EpiPlanes e{static_cast<bf16_t*>(out), out_plane, s.T, s.d_kv, static_cast<int64_t>(s.h) * out_ld, out_ld};
  return run_gemm_dma<DKC<1, bf16_t, 128>, DRC<1, 256>, 2, 4, 4, 1>(A, Operand<float>{}, B, e, s.T, s.d_kv, 128, 1,
                                                                     st, s.h);
}

hipError_t launch_b2_rows_keys(const void* rows, int64_t rows_plane, int64_t rows_ld, int64_t nrows, const void* keys,
                               int64_t keys_plane, int64_t nkeys, int64_t kdim, float* out, int64_t out_ld,
                               hipStream_t st) {
  // out[r][u] = sum_k rows[r][k] keys[u][k], k < kdim (keys' row pitch 576).
  Operand<bf16_t> A{static_cast<const bf16_t*>(rows), rows_ld, rows_plane, nrows, kdim};
  Operand<bf16_t> B{static_cast<const bf16_t*>(keys), B2_DQ, keys_plane, nkeys, kdim};
  EpiStore e{out, nrows, static_cast<int>(nkeys), out_ld, 0};
  return run_gemm_dma<DKC<2, bf16_t, 128>, DKC<2, bf16_t, 128>, 2, 2, 2, 2>(A, Operand<float>{}, B, e, nrows, nkeys,
                                                                             kdim, 1, st);
}

int b2_keygrad_chunks(int64_t nkeys, int64_t nrows) {
  // K (= rows) chunks so that the dS product (576 columns) runs about 512
  // workgroups; at most B2_KG_SPLIT, at least 256 rows each.
  const int64_t tiles = ((nkeys + 127) / 128) * ((B2_DQ + 127) / 128);
  int64_t c = (512 + tiles - 1) / tiles;
  if (c > B2_KG_SPLIT) c = B2_KG_SPLIT;
  if (c > nrows / 256) c = nrows / 256;
  if (c < 1) c = 1;
  const int64_t per = ((nrows + c - 1) / c + BK - 1) / BK * BK;  // as run_gemm_dma splits
  return static_cast<int>((nrows + per - 1) / per);
}

namespace {
// dL[u][c] += sum over k of part[k][u][c] (c < 512) and dk_pe[u][c - 512] +=
// the same for c >= 512, where k runs over the nch partials of the P product
// (columns < 512 only) and then the nch partials of the c.dS product, in that
// order.  part[g][k][u][576], g = 0 (P) / 1 (c.dS).  One thread per 4 columns.
__global__ __launch_bounds__(256) void b2_kg_sum_kernel(const float* __restrict__ part, int nch, int64_t nkeys,
                                                        float* __restrict__ dL, float* __restrict__ dkpe) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (j >= nkeys * (B2_DQ / 4)) return;
  const int64_t u = j / (B2_DQ / 4);
  const int c = static_cast<int>(j % (B2_DQ / 4)) * 4;
  const int64_t e = u * B2_DQ + c, gs = static_cast<int64_t>(nch) * nkeys * B2_DQ;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (c < B2_DL)
    for (int k = 0; k < nch; ++k) v += *reinterpret_cast<const f32x4*>(part + k * nkeys * B2_DQ + e);
  for (int k = 0; k < nch; ++k) v += *reinterpret_cast<const f32x4*>(part + gs + k * nkeys * B2_DQ + e);
  float* o = c < B2_DL ? dL + u * B2_DL + c : dkpe + u * 64 + (c - B2_DL);
  *reinterpret_cast<f32x4*>(o) += v;
}
}  // namespace

hipError_t launch_b2_key_grads(const void* pp, const void* dsp, int64_t p_plane, int64_t ldu, int64_t nrows,
                               int64_t nkeys, const void* dacc_rows, int64_t dacc_plane, const void* qx_rows,
                               int64_t qx_plane, float* dL, float* dkpe, float* part, hipStream_t st) {
  // dL[u][c] += sum_r P[r][u] dacc[r][c]; (dL || dk_pe)[u][c] += sum_r cdS[r][u] qx[r][c].
  // With few key tiles the rows (K) are split into chunks whose fp32 partials
  // (part: 2 b2_keygrad_chunks(nkeys, nrows) nkeys 576 floats) are summed in
  // a fixed order.
  typedef DRC<2, 128> OA;  // P / cdS [r][u] read as A(row = u, k = r)
  typedef DRC<2, 128> OB;  // dacc / qx [r][c] read as B(row = c, k = r)
  Operand<bf16_t> Ap{static_cast<const bf16_t*>(pp), ldu, p_plane, nkeys, nrows};
  Operand<bf16_t> Bd{static_cast<const bf16_t*>(dacc_rows), B2_DL, dacc_plane, B2_DL, nrows};
  Operand<bf16_t> As{static_cast<const bf16_t*>(dsp), ldu, p_plane, nkeys, nrows};
  Operand<bf16_t> Bq{static_cast<const bf16_t*>(qx_rows), B2_DQ, qx_plane, B2_DQ, nrows};
  const int nch = b2_keygrad_chunks(nkeys, nrows);
  if (nch == 1) {
    EpiAccum e1{dL, B2_DL, dkpe, 64, nkeys, B2_DL, B2_DL};
    hipError_t err = run_gemm_dma<OA, OB, 2, 2, 2, 2>(Ap, Operand<float>{}, Bd, e1, nkeys, B2_DL, nrows, 1, st);
    if (err != hipSuccess) return err;
    EpiAccum e2{dL, B2_DL, dkpe, 64, nkeys, B2_DQ, B2_DL};
    return run_gemm_dma<OA, OB, 2, 2, 2, 2>(As, Operand<float>{}, Bq, e2, nkeys, B2_DQ, nrows, 1, st);
  }
  const int64_t stride = nkeys * B2_DQ;
  EpiPart e1{{part, nkeys, B2_DL, B2_DQ, stride}};
  hipError_t err = run_gemm_dma<OA, OB, 2, 2, 2, 2>(Ap, Operand<float>{}, Bd, e1, nkeys, B2_DL, nrows, nch, st);
  if (err != hipSuccess) return err;
  EpiPart e2{{part + nch * stride, nkeys, B2_DQ, B2_DQ, stride}};
  err = run_gemm_dma<OA, OB, 2, 2, 2, 2>(As, Operand<float>{}, Bq, e2, nkeys, B2_DQ, nrows, nch, st);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(b2_kg_sum_kernel, dim3(static_cast<unsigned>((nkeys * (B2_DQ / 4) + 255) / 256)), dim3(256),
                     0, st, part, nch, nkeys, dL, dkpe);
  return hipGetLastError();
}

int b2_key_chunks(int64_t nrows, int ncols, int64_t kpad) {
  // K chunks so that about 512 workgroups run (two per CU at this tile's
  // occupancy), at most B2_KSPLIT and at least 256 keys each.
  const int64_t tiles = ((ncols + 127) / 128) * ((nrows + 127) / 128);
  int64_t c = (512 + tiles - 1) / tiles;
  if (c > B2_KSPLIT) c = B2_KSPLIT;
  if (c > kpad / 256) c = kpad / 256;
  if (c < 1) c = 1;
  // The count run_gemm_dma produces for this request.
  const int64_t per = ((kpad + c - 1) / c + BK - 1) / BK * BK;
  return static_cast<int>((kpad + per - 1) / per);
}

hipError_t launch_b2_rows_by_keys(const void* ap, int64_t p_plane, int64_t ldu, int64_t nrows, int64_t kpad,
                                  const void* keys, int64_t keys_plane, int ncols, float* part, hipStream_t st) {
  // part[c][r][n] = sum over u in K chunk c of A[r][u] kxp[u][n], n < ncols, u < kpad (A is P or
  // c.dS as bf16 hi/lo planes, zero past the chunk's keys); c < b2_key_chunks(nrows, ncols, kpad).
  Operand<bf16_t> A{static_cast<const bf16_t*>(ap), ldu, p_plane, nrows, kpad};
  Operand<bf16_t> B{static_cast<const bf16_t*>(keys), B2_DQ, keys_plane, ncols, kpad};
  EpiStore e{part, nrows, ncols, ncols, nrows * ncols};
  return run_gemm_dma<DKC<2, bf16_t, 128>, DRC<2, 128>, 2, 2, 2, 2>(A, Operand<float>{}, B, e, nrows, ncols, kpad,
                                                                     b2_key_chunks(nrows, ncols, kpad), st);
}

hipError_t launch_b2_dq_nope(const Shape& s, const float* dqx, const void* w, float* dq, hipStream_t st) {
  // dq[t][i][n] = sum_c d_q_abs[t h + i][c] W^k[head_lo + i][n][c].
  const int64_t w0 = static_cast<int64_t>(s.head_lo) * s.C() * s.d_kv;
  Operand<float> A{dqx, static_cast<int64_t>(s.h) * B2_DQ, 0, s.T, B2_DL, B2_DQ};
  Operand<bf16_t> B{static_cast<const bf16_t*>(w) + w0, s.d_kv, 0, s.d_nope, s.d_kv,
                    static_cast<int64_t>(s.C()) * s.d_kv};
  EpiStore e{dq, s.T, s.d_nope, static_cast<int64_t>(s.h) * s.d_qk(), s.d_qk()};
  return run_gemm_dma<DKC<1, float, 256>, DKC<1, bf16_t, 128>, 4, 2, 3, 1>(Operand<bf16_t>{}, A, B, e, s.T, s.d_nope,
                                                                             B2_DL, 1, st, s.h);
}

int b2_dw_chunks(const Shape& s) {
  const int64_t tiles = static_cast<int64_t>(s.h) * (128 / 128) * (B2_DL / 128);
  int64_t c = (DW_TARGET + tiles - 1) / tiles;
  const int64_t kmax = (s.T + BK - 1) / BK;
  if (c > kmax) c = kmax;
  if (c < 1) c = 1;
  const int64_t per = ((s.T + c - 1) / c + BK - 1) / BK * BK;
  return static_cast<int>((s.T + per - 1) / per);
}

size_t b2_dw_partial_floats(const Shape& s) {
  return static_cast<size_t>(b2_dw_chunks(s)) * s.h * 128 * B2_DL;
}

namespace {
// dW[head_lo + i][row0 + n][c] = sum over the K chunks of part[i][chunk][n][c], in order.
__global__ __launch_bounds__(256) void b2_dw_sum_kernel(const float* __restrict__ part, float* __restrict__ dw,
                                                        int h, int chunks, int64_t head_stride, int64_t row0) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  constexpr int64_t X = 128 * B2_DL;
  if (j >= h * X) return;
  const int64_t i = j / X, e = j % X;
  const float* pp = part + i * chunks * X + e;
  float acc = 0.f;
#pragma unroll 8
  for (int c = 0; c < chunks; ++c) acc += pp[c * X];
  dw[i * head_stride + row0 * B2_DL + e] = acc;
}
}  // namespace

hipError_t launch_b2_dw(const Shape& s, const void* x, int64_t x_ld, int64_t x_z, const void* yp, int64_t y_plane,
                        float* partial, float* d_w, int64_t row0, hipStream_t st) {
  // dW[head_lo + i][row0 + n][c] = sum_t x[t][i][n] y[t h + i][c] (x: q_nope or dO, bf16 exact,
  // token pitch x_ld and head pitch x_z elements; y: d_q_abs or acc as bf16 hi/lo planes
  // [2][R][512]); K split into chunks, summed in order.
  const int chunks = b2_dw_chunks(s);
  typedef DRC<1, 128> OA;  // x[t][i][n] read as A(row = n, k = t)
  typedef DRC<2, 128> OB;  // y[t h + i][c] read as B(row = c, k = t)
  Operand<bf16_t> A{static_cast<const bf16_t*>(x), x_ld, 0, 128, s.T, x_z};
  Operand<bf16_t> B{static_cast<const bf16_t*>(yp), static_cast<int64_t>(s.h) * B2_DL, y_plane, B2_DL, s.T, B2_DL};
  EpiStore e{partial, 128, B2_DL, B2_DL, 128 * B2_DL};
  hipError_t err = run_gemm_dma<OA, OB, 2, 2, 2, 2>(A, Operand<float>{}, B, e, 128, B2_DL, s.T, chunks, st, s.h);
  if (err != hipSuccess) return err;
  const int64_t n = static_cast<int64_t>(s.h) * 128 * B2_DL;
  hipLaunchKernelGGL(b2_dw_sum_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, partial,
                     d_w + static_cast<int64_t>(s.head_lo) * s.C() * s.d_kv, s.h, chunks,
                     static_cast<int64_t>(s.C()) * s.d_kv, row0);
  return hipGetLastError();
}

}  // namespace laga
