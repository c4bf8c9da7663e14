// dq of the causal attention backward of one rank's head shard [LAGA §5.2]:
//   dq = dS K / sqrt(d_qk)
// from the dS tiles the dK/dV kernel (attn_bwd.hip) writes, so no score is
// recomputed here.
//
// A workgroup of 4 wavefronts owns 128 queries (32 per wavefront) and walks
// the keys from 0 to its diagonal, 64 at a time: dq^T = K^T dS^T with one
// query per lane column.  The K^T operands come from transposing LDS reads of
// the K tile (hi plane plus the k_pe band converted to fp16 on the way;
// double-buffered, shared by the four wavefronts); the wavefront's own dS
// tiles ([key][query]) are loaded one key block ahead in 16-byte chunks,
// copied to its private LDS area and read back transposed (query = lane
// column, 8 consecutive keys) as the dS^T operands.  Every dS element is read
// once, so the kernel streams the tiles from HBM (non-temporal loads); tiles
// above the diagonal are never stored or read.
//
// This file is compiled with the matrix-core accumulators in VGPRs (see the
// build script).
#include "attn_bwd_common.hpp"

namespace laga {
namespace {
using namespace bwd;

// ================================================================ dq kernel
template <class InT, class M, int DN, int DR>
struct Dq {
  typedef typename M::elem E;
  typedef typename M::frag F;
  static constexpr int DQK = DN + DR;
  static constexpr int BM = 128, BN = 64;
  static constexpr bool TR = M::KPL == 8;
  // K tile, read transposed only: a row pitch of 64 or 192 (mod 256) bytes
  // puts the four rows a half-wavefront's transposing read touches in four
  // disjoint 64-byte bank windows.
  static constexpr int LKR = TR ? DQK + 32 : DQK + TilePad<M>::both;
  static_assert(!TR || (LKR * 2) % 256 == 64 || (LKR * 2) % 256 == 192, "conflict-free transposing reads");
  static constexpr int BUF_BYTES = BN * LKR * sizeof(E);
  static constexpr int NQT = (DQK + 31) / 32;  // dq^T row atoms (the last may run past d_qk)
  static constexpr int NKS = BN / M::K;        // k-steps (keys) per block
  // Staging chunks (16 bytes): nope part of K (hi plane), rope band (input type).
  static constexpr int EPC = 16 / sizeof(E), IPC = 16 / sizeof(InT);
  static constexpr int KCH = BN * DN / EPC, PCH = BN * DR / IPC;
  static constexpr int IK = (KCH + kThreads - 1) / kThreads, IP = (PCH + kThreads - 1) / kThreads;
  static constexpr int kAhead = 6;  // K^T operand reads in flight ahead of the products
  // dS: the wavefront's two tiles of a key block, as 16-byte chunks (NDC per
  // lane) and in its private LDS area.
  static constexpr int DS_BYTES = (BN / 32) * kDsTile * static_cast<int>(sizeof(E));
  static constexpr int NDC = DS_BYTES / 16 / kWave;
  // K tile buffers, the four dS areas, and room for the last K^T atom's
  // reads of rows past d_qk.
  static constexpr int OFF_DS = 2 * BUF_BYTES;
  static constexpr int LDS_BYTES = OFF_DS + 4 * DS_BYTES + (NQT * 32 - DQK) * static_cast<int>(sizeof(E));

  // dS tiles are loaded two key blocks ahead (into the set of the block's
  // parity), the K tile one block ahead.
  struct Regs { u32x4 k[IK]; u32x4 p[IP]; u32x4 ds[2][NDC]; };

  // Stage key block key0's K tile rows (zero past the sequence).
  __device__ static void load_k(const BwdArgs& a, int b, int head, int64_t key0, Regs& R) {
    const int nk = static_cast<int>(a.S - key0 < BN ? a.S - key0 : BN);
    const int64_t row0 = (b * a.S + key0) * a.h + head;
    const int krow_b = a.h * DN * static_cast<int>(sizeof(E));
    const int prow_b = DR * static_cast<int>(sizeof(InT));
    const auto rk = rsrc(static_cast<const E*>(a.k_nope) + row0 * DN, nk * krow_b);
    const auto rp = rsrc(static_cast<const InT*>(a.k_pe) + (b * a.S + key0) * DR, nk * prow_b);
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < IK; ++i) {
      const int c = i * kThreads + tid;
      const int r = c / (DN / EPC), j = c % (DN / EPC);
      if (KCH % kThreads == 0 || c < KCH) R.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, r * krow_b + j * 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < IP; ++i) {
      const int c = i * kThreads + tid;
      const int r = c / (DR / IPC), j = c % (DR / IPC);
      if (PCH % kThreads == 0 || c < PCH) R.p[i] = __builtin_amdgcn_raw_buffer_load_b128(rp, r * prow_b + j * 16, 0, 0);
    }
  }

  // Stage the wavefront's dS tiles (qb, key0 / 32 + t) of key block key0 into
  // `ds`, zero for tiles above the diagonal and for wavefronts past the
  // sequence.
  __device__ static void load_ds(const BwdArgs& a, int b, int head, int64_t key0, int64_t qb, bool qin,
                                 u32x4 (&ds)[NDC]) {
    const int lane = threadIdx.x % kWave;
    constexpr int CPT = NDC / (BN / 32);  // chunks per lane per tile
#pragma unroll
    for (int t = 0; t < BN / 32; ++t) {
      const int64_t kt = key0 / 32 + t;
      if (qin && kt <= qb) {
        const u32x4* tile = reinterpret_cast<const u32x4*>(static_cast<const E*>(a.ds) +
                                                           ds_tile(a, b, head, qb, kt) * kDsTile);
#pragma unroll
        for (int c = 0; c < CPT; ++c) ds[t * CPT + c] = __builtin_nontemporal_load(tile + c * kWave + lane);
      } else {
#pragma unroll
        for (int c = 0; c < CPT; ++c) ds[t * CPT + c] = u32x4{0, 0, 0, 0};
      }
    }
  }

  __device__ static void store(const Regs& R, char* buf) {
    E* Kr = reinterpret_cast<E*>(buf);
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < IK; ++i) {
      const int c = i * kThreads + tid;
      if (KCH % kThreads != 0 && c >= KCH) continue;
      const int r = c / (DN / EPC), col = (c % (DN / EPC)) * EPC;
      *reinterpret_cast<u32x4*>(Kr + r * LKR + col) = R.k[i];
    }
#pragma unroll
    for (int i = 0; i < IP; ++i) {
      const int c = i * kThreads + tid;
      if (PCH % kThreads != 0 && c >= PCH) continue;
      const int r = c / (DR / IPC), col = DN + (c % (DR / IPC)) * IPC;
      E tmp[IPC];
      convert_chunk<E, InT>(R.p[i], tmp);
#pragma unroll
      for (int j = 0; j < IPC; j += EPC) {
        *reinterpret_cast<u32x4*>(Kr + r * LKR + col + j) = *reinterpret_cast<u32x4*>(tmp + j);
      }
    }
  }

  // A operand of dq^T += K^T dS^T for k-step s of the block (keys s K ..,
  // natural order), dims n0 + lane % 32.
  __device__ static F kt_frag(const E* Kr, int s, int n0) {
    if constexpr (TR) {
      return tr_frag(Kr, LKR, s * M::K, n0);
    } else {
      const int lane = threadIdx.x % kWave;
      return Kr[(s * M::K + lane / 32) * LKR + n0 + lane % 32];
    }
  }

  // B operand of dq^T += K^T dS^T for k-step s: query lane % 32, keys
  // s K + hf KPL + [0, KPL) from the wavefront's dS area ([key][query] tiles).
  __device__ static F ds_frag(const E* D, int s) {
    const E* tile = D + (s * M::K / 32) * kDsTile;
    if constexpr (TR) {
      return tr_frag(tile, 32, (s * M::K) % 32, 0);
    } else {
      const int lane = threadIdx.x % kWave;
      return tile[((s * M::K) % 32 + lane / 32) * 32 + lane % 32];
    }
  }

  // Publish key block kb's K tile into `buf` and the wavefront's dS tiles
  // into its area (P = kb's parity), start loading the K tile of kb + 1 and
  // the dS tiles of kb + 2, accumulate.
  template <int P>
  __device__ static void step(const BwdArgs& a, char* buf, char* dsa, int kb, int nkb, int b, int head,
                              int64_t qb, bool qin, Regs& R, f32x16* dq) {
    store(R, buf);
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int c = 0; c < NDC; ++c) reinterpret_cast<u32x4*>(dsa)[c * kWave + lane] = R.ds[P][c];
    __syncthreads();
    if (kb + 1 < nkb) load_k(a, b, head, static_cast<int64_t>(kb + 1) * BN, R);
    if (kb + 2 < nkb) load_ds(a, b, head, static_cast<int64_t>(kb + 2) * BN, qb, qin, R.ds[P]);
    const E* D = reinterpret_cast<const E*>(dsa);
    F ds[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) ds[s] = ds_frag(D, s);
    const E* Kr = reinterpret_cast<const E*>(buf);
    pipelined<NKS * NQT, kAhead, F>([&](int i) { return kt_frag(Kr, i / NQT, (i % NQT) * 32); },
                                    [&](int i, const F& k) { dq[i % NQT] = M::mma(k, ds[i / NQT], dq[i % NQT]); });
  }

  __device__ static void run(const BwdArgs& a, char* lds) {
    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int hf = lane / 32, col = lane % 32;
    const int n_qt = static_cast<int>((a.S + BM - 1) / BM);
    const int nbh = a.B * a.h;
    const int qt = n_qt - 1 - static_cast<int>(blockIdx.x / nbh);  // longest first
    const int bh = blockIdx.x % nbh;
    const int b = bh / a.h, head = bh % a.h;
    const int64_t q0 = static_cast<int64_t>(qt) * BM;
    const int64_t qw = q0 + wv * 32;
    const int64_t qb = qw / 32;
    const bool qin = qw < a.S;  // the wavefront has queries (its dS tiles exist)
    const int64_t tq = qw + col;

    f32x16 dq[NQT];
#pragma unroll
    for (int n = 0; n < NQT; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[n][r] = 0.f;

    int64_t kend = q0 + BM;
    if (kend > a.S) kend = a.S;
    const int nkb = static_cast<int>((kend + BN - 1) / BN);
    Regs R;
    load_k(a, b, head, 0, R);
    load_ds(a, b, head, 0, qb, qin, R.ds[0]);
    if (nkb > 1) load_ds(a, b, head, BN, qb, qin, R.ds[1]);
    char* dsa = lds + OFF_DS + wv * DS_BYTES;  // this wavefront's dS area
    int kb = 0;
    // Unrolled by two so that each step names its buffers as constants and
    // the LDS addresses fold into immediates.
    for (; kb + 1 < nkb; kb += 2) {
      step<0>(a, lds, dsa, kb, nkb, b, head, qb, qin, R, dq);
      step<1>(a, lds + BUF_BYTES, dsa, kb + 1, nkb, b, head, qb, qin, R, dq);
    }
    if (kb < nkb) step<0>(a, lds, dsa, kb, nkb, b, head, qb, qin, R, dq);
    if (tq >= a.S) return;
    float* out = a.dq + ((b * a.S + tq) * a.h + head) * DQK;
    // dS carries dO's scale 2^g.
    const float osc = a.scale * pow2i(-do_shift_of(a));
#pragma unroll
    for (int n = 0; n < NQT; ++n)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (n * 32 + 8 * j + 4 * hf >= DQK) continue;
        f32x4 w = {dq[n][4 * j] * osc, dq[n][4 * j + 1] * osc, dq[n][4 * j + 2] * osc, dq[n][4 * j + 3] * osc};
        *reinterpret_cast<f32x4*>(out + n * 32 + 8 * j + 4 * hf) = w;
      }
  }
};

template <class InT, class M, int DN, int DR>
__global__ __launch_bounds__(kThreads) void dq_kernel(BwdArgs a) {
  typedef Dq<InT, M, DN, DR> Kn;
  __shared__ __attribute__((aligned(16))) char lds[Kn::LDS_BYTES];
  Kn::run(a, lds);
}


}  // namespace

hipError_t launch_attn_bwd_dq(const Shape& s, const void* k_nope, const void* k_pe, const void* ds,
                              const int* do_shift, float* dq, hipStream_t st) {
  BwdArgs a = make_args(s, nullptr, k_nope, k_pe, nullptr, nullptr, nullptr, nullptr);
  a.ds = const_cast<void*>(ds);
  a.dq = dq;
  a.do_shift = do_shift;
  const unsigned grid = static_cast<unsigned>(((s.S + 127) / 128) * s.B * s.h);
  if (s.bf16 && s.split && s.d_nope == 128 && s.d_rope == 64 && s.d_v == 128)
    hipLaunchKernelGGL((dq_kernel<half_t, MmaF16, 128, 64>), dim3(grid), dim3(kThreads), 0, st, a);
  else if (!s.bf16 && s.d_nope == 32 && s.d_rope == 16 && s.d_v == 32)
    hipLaunchKernelGGL((dq_kernel<float, MmaF32, 32, 16>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    return hipErrorNotSupported;
  return hipGetLastError();
}

}  // namespace laga
