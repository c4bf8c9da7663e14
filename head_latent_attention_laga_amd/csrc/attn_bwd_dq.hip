// dq of the causal attention backward of one rank's head shard [LAGA §5.2]:
//   dq = dS K / sqrt(d_qk),  dS = P * (dP - delta),  dP = dO V^T,
// with P rebuilt from the forward's lse (the dK/dV kernel and the reductions
// live in attn_bwd.hip).
//
// A workgroup of 4 wavefronts owns 128 queries (q and dO held in registers
// as B operands) and walks the keys from 0 to its diagonal, 64 at a time:
// S^T = K q^T and dP^T = V dO^T leave one query per lane column, the layout
// in which dS^T is the B operand of dq^T = K^T dS^T (K^T from transposing
// LDS reads).  K (hi plane) and the k_pe band stream through double-buffered
// LDS, the k_pe band converted to fp16 on the way.
//
// Precision: dq is a per-element output, so single fp16 K, V and dS suffice
// for its bound; the float32 instantiation uses fp32 MFMAs.
//
// This file is compiled with the matrix-core accumulators in VGPRs (see the
// build script): the loop then keeps dq and the score tiles in place instead
// of copying accumulators between register files every iteration.
#include "attn_bwd_common.hpp"

namespace laga {
namespace {
using namespace bwd;

// ================================================================ dq kernel
template <class InT, class M, int NS, int DN, int DR, int DV>
struct Dq {
  typedef typename M::elem E;
  typedef typename M::frag F;
  static constexpr int DQK = DN + DR;
  static constexpr int BM = 128, BN = 64;
  static constexpr bool TR = M::KPL == 8;
  // One K tile read both as rows (S^T) and transposed (dq^T); V rows only.
  static constexpr int LKR = DQK + TilePad<M>::both, LVR = DV + TilePad<M>::row;
  static constexpr int KR_B = BN * LKR * sizeof(E);
  static constexpr int VR_B = BN * LVR * sizeof(E);
  static constexpr int BUF_BYTES = KR_B + VR_B;
  static constexpr int KS_QK = DQK / M::K, KS_V = DV / M::K;
  static constexpr int NT = BN / 32, NQT = (DQK + 31) / 32, STEPS = 32 / M::K;
  // Staging chunks (16 bytes): nope part of K (hi plane), rope band (input type), V (hi plane).
  static constexpr int EPC = 16 / sizeof(E), IPC = 16 / sizeof(InT);
  static constexpr int KCH = BN * DN / EPC, PCH = BN * DR / IPC, VCH = BN * DV / EPC;
  static constexpr int IK = (KCH + kThreads - 1) / kThreads, IP = (PCH + kThreads - 1) / kThreads;
  static constexpr int IV = (VCH + kThreads - 1) / kThreads;

  struct Regs { u32x4 k[IK]; u32x4 p[IP]; u32x4 v[IV]; };
  static constexpr int kScoreAhead = 4, kDqAhead = 4;  // operand reads in flight ahead of the products

  __device__ static void load(const BwdArgs& a, int b, int head, int64_t key0, Regs& R) {
    const int nk = static_cast<int>(a.S - key0 < BN ? a.S - key0 : BN);
    const int64_t row0 = (b * a.S + key0) * a.h + head;
    const int krow_b = a.h * DN * static_cast<int>(sizeof(E));
    const int vrow_b = a.h * DV * static_cast<int>(sizeof(E));
    const int prow_b = DR * static_cast<int>(sizeof(InT));
    const auto rk = rsrc(static_cast<const E*>(a.k_nope) + row0 * DN, nk * krow_b);
    const auto rv = rsrc(static_cast<const E*>(a.v) + row0 * DV, nk * vrow_b);
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
#pragma unroll
    for (int i = 0; i < IV; ++i) {
      const int c = i * kThreads + tid;
      const int r = c / (DV / EPC), j = c % (DV / EPC);
      if (VCH % kThreads == 0 || c < VCH) R.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, r * vrow_b + j * 16, 0, 0);
    }
  }

  __device__ static void store(const Regs& R, char* buf) {
    E* Kr = reinterpret_cast<E*>(buf);
    E* Vr = reinterpret_cast<E*>(buf + KR_B);
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
#pragma unroll
    for (int i = 0; i < IV; ++i) {
      const int c = i * kThreads + tid;
      if (VCH % kThreads != 0 && c >= VCH) continue;
      const int r = c / (DV / EPC), col = (c % (DV / EPC)) * EPC;
      *reinterpret_cast<u32x4*>(Vr + r * LVR + col) = R.v[i];
    }
  }

  // KPL input elements at byte offset `off` of a buffer (zero outside it) as a fragment.
  __device__ static F frag_from(__amdgpu_buffer_rsrc_t r, int off) {
    if constexpr (sizeof(InT) * M::KPL == 16) {
      const u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
      E tmp[M::KPL];
      convert_chunk<E, InT>(raw, tmp);
      return *reinterpret_cast<F*>(tmp);
    } else {
      static_assert(sizeof(InT) == 4 && M::KPL == 1, "fp32 rows feed one element per lane");
      return M::from_f32(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0)));
    }
  }

  // A operand of dq^T += K^T dS^T for one MFMA step of key atom t.
  __device__ static F kt_frag(const E* Kr, int t, int st, int n0) {
    if constexpr (TR) {
      return tr_frag_acc(Kr, LKR, t * 32 + st * 16, n0);
    } else {
      const int lane = threadIdx.x % kWave;
      const int k = t * 32 + 8 * (st / 4) + 4 * (lane / 32) + (st % 4);
      return Kr[k * LKR + n0 + lane % 32];
    }
  }

  // Stationary operands of one wavefront: its 32 queries' q and dO
  // fragments (B operands) and softmax statistics.
  struct Stat { F qf[KS_QK], of[KS_V]; float lse2, dl; };

  // One block of BN keys from key0 against the wavefront's 32 queries from qw
  // (lane column = query tq).  MASK: the block may cross the diagonal, reach
  // past the sequence, or lie wholly after the wavefront's queries.
  template <bool MASK>
  __device__ static void block(const BwdArgs& a, const char* buf, int64_t key0, int64_t qw, const Stat& Q,
                               f32x16* dq) {
    const int lane = threadIdx.x % kWave;
    const int hf = lane / 32, col = lane % 32;
    if (MASK && key0 > qw + 31) return;  // every key of the block follows these queries
    const E* Kr = reinterpret_cast<const E*>(buf);
    const E* Vr = reinterpret_cast<const E*>(buf + KR_B);
    // S^T[key, q], dP^T[key, q] for the NT key atoms, chains interleaved.
    f32x16 sc[NT], dp[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) { sc[t][r] = 0.f; dp[t][r] = 0.f; }
    // Products in the order (s, t): S^T from K row s, then (s < KS_V) dP^T
    // from V row s; each operand read kScoreAhead products ahead.
    constexpr int NKV = KS_V * 2 * NT;  // products of the steps that have both
    auto item = [](int i, int& s, int& t, bool& isv) {
      if (i < NKV) {
        s = i / (2 * NT); t = (i % (2 * NT)) / 2; isv = i % 2;
      } else {
        s = KS_V + (i - NKV) / NT; t = (i - NKV) % NT; isv = false;
      }
    };
    pipelined<NKV + (KS_QK - KS_V) * NT, kScoreAhead, F>(
        [&](int i) {
          int s, t; bool isv;
          item(i, s, t, isv);
          return isv ? lds_frag<M>(Vr + (t * 32 + col) * LVR + hf * M::KPL + s * M::K)
                     : lds_frag<M>(Kr + (t * 32 + col) * LKR + hf * M::KPL + s * M::K);
        },
        [&](int i, const F& f) {
          int s, t; bool isv;
          item(i, s, t, isv);
          if (isv) dp[t] = M::mma(f, Q.of[s], dp[t]);
          else sc[t] = M::mma(f, Q.qf[s], sc[t]);
        });
    // rel = key - query of accumulator row 0 of atom t (32-bit: within a block).
    const int rel = static_cast<int>(key0 - qw) - col;
    const int kin = static_cast<int>(a.S - key0);  // keys of the block inside the sequence
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(fmaf(sc[t][r], a.scale_log2, -Q.lse2));
        if constexpr (MASK) {
          const int u = t * 32 + 8 * (r / 4) + 4 * hf + (r % 4);  // key offset in the block
          if (rel + u > 0 || u >= kin) p = 0.f;
        }
        dp[t][r] = p * (dp[t][r] - Q.dl);
      }
    // dq^T[d, q] += K^T dS^T  (k = keys of the accumulators), the K^T
    // operands read kDqAhead products ahead.
    F df[NT][STEPS];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int stp = 0; stp < STEPS; ++stp) {
        E dh[M::KPL];
#pragma unroll
        for (int j = 0; j < M::KPL; ++j) dh[j] = M::from_f32(dp[t][stp * M::KPL + j]);
        df[t][stp] = *reinterpret_cast<F*>(dh);
      }
    pipelined<NT * STEPS * NQT, kDqAhead, F>(
        [&](int i) { return kt_frag(Kr, i / NQT / STEPS, (i / NQT) % STEPS, (i % NQT) * 32); },
        [&](int i, const F& f) { dq[i % NQT] = M::mma(f, df[i / NQT / STEPS][(i / NQT) % STEPS], dq[i % NQT]); });
  }

  template <bool MASK>
  __device__ static void step(const BwdArgs& a, char* buf, int kb, int nkb, int b, int head, int64_t qw,
                              Regs& R, const Stat& Q, f32x16* dq) {
    const int64_t key0 = static_cast<int64_t>(kb) * BN;
    store(R, buf);  // `buf`: the buffer of kb's parity
    __syncthreads();
    if (kb + 1 < nkb) load(a, b, head, key0 + BN, R);
    block<MASK>(a, buf, key0, qw, Q, dq);
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
    const int64_t tq = qw + col;
    const bool qvalid = tq < a.S;

    // q / dO rows of the wavefront; rows past the sequence read as zero, which
    // with zero statistics makes their dS zero.
    const int g = do_shift_of(a);
    Stat Q;
    {
      const int nq = static_cast<int>(a.S - qw < 32 ? (a.S - qw > 0 ? a.S - qw : 0) : 32);
      const int64_t row0 = (b * a.S + qw) * a.h + head;
      const int qrb = a.h * DQK * static_cast<int>(sizeof(InT)), orb = a.h * DV * static_cast<int>(sizeof(InT));
      const auto rq = rsrc(static_cast<const InT*>(a.q) + row0 * DQK, nq * qrb);
      const auto ro = rsrc(static_cast<const InT*>(a.d_o) + row0 * DV, nq * orb);
#pragma unroll
      for (int s = 0; s < KS_QK; ++s)
        Q.qf[s] = frag_from(rq, col * qrb + (s * M::K + hf * M::KPL) * static_cast<int>(sizeof(InT)));
#pragma unroll
      for (int s = 0; s < KS_V; ++s)
        Q.of[s] = frag_from(ro, col * orb + (s * M::K + hf * M::KPL) * static_cast<int>(sizeof(InT)));
      const int64_t si0 = (static_cast<int64_t>(b) * a.h + head) * a.S + qw;
      Q.lse2 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc(a.lse + si0, nq * 4), col * 4, 0, 0)) * kLog2e;
      Q.dl = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc(a.delta + si0, nq * 4), col * 4, 0, 0)) *
             pow2i(g);  // dO enters scaled by 2^g
    }
    const int64_t qrow = (b * a.S + (qvalid ? tq : 0)) * a.h + head;

    f32x16 dq[NQT];
#pragma unroll
    for (int n = 0; n < NQT; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[n][r] = 0.f;

    // Key blocks wholly at or below the workgroup's first query need no mask.
    int64_t kend = q0 + BM;
    if (kend > a.S) kend = a.S;
    const int nkb = static_cast<int>((kend + BN - 1) / BN);
    int nfree = static_cast<int>((q0 + 1) / BN);
    if (nfree > nkb) nfree = nkb;
    Regs R;
    load(a, b, head, 0, R);
    int kb = 0;
    // Unrolled by two so that each step names its buffer as a constant offset
    // and the LDS addresses fold into immediates.
    for (; kb + 1 < nfree; kb += 2) {
      step<false>(a, lds, kb, nkb, b, head, qw, R, Q, dq);
      step<false>(a, lds + BUF_BYTES, kb + 1, nkb, b, head, qw, R, Q, dq);
    }
    for (; kb < nfree; ++kb) step<false>(a, lds + (kb & 1) * BUF_BYTES, kb, nkb, b, head, qw, R, Q, dq);
    for (; kb < nkb; ++kb) step<true>(a, lds + (kb & 1) * BUF_BYTES, kb, nkb, b, head, qw, R, Q, dq);
    if (!qvalid) return;
    float* out = a.dq + qrow * DQK;
    const float osc = a.scale * pow2i(-g);
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

template <class InT, class M, int NS, int DN, int DR, int DV>
__global__ __launch_bounds__(kThreads) void dq_kernel(BwdArgs a) {
  typedef Dq<InT, M, NS, DN, DR, DV> Kn;
  __shared__ __attribute__((aligned(16))) char lds[2 * Kn::BUF_BYTES];
  Kn::run(a, lds);
}


}  // namespace

hipError_t launch_attn_bwd_dq(const Shape& s, const void* q, const void* kn, const void* kp, const void* v,
                              const float* lse, const float* delta, const void* d_o, const int* do_shift, float* dq,
                              hipStream_t st) {
  BwdArgs a = make_args(s, q, kn, kp, v, lse, delta, d_o);
  a.dq = dq;
  a.do_shift = do_shift;
  const unsigned grid = static_cast<unsigned>(((s.S + 127) / 128) * s.B * s.h);
  if (s.bf16 && s.split && s.d_nope == 128 && s.d_rope == 64 && s.d_v == 128)
    hipLaunchKernelGGL((dq_kernel<half_t, MmaF16, 2, 128, 64, 128>), dim3(grid), dim3(kThreads), 0, st, a);
  else if (!s.bf16 && s.d_nope == 32 && s.d_rope == 16 && s.d_v == 32)
    hipLaunchKernelGGL((dq_kernel<float, MmaF32, 1, 32, 16, 32>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    return hipErrorNotSupported;
  return hipGetLastError();
}

}  // namespace laga
