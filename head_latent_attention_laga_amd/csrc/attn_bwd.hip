// Causal attention backward of one rank's head shard [LAGA §5.2: gradients of
// the rank-local computation; the k_pe band's gradient is the sum over the
// local heads; the K/V gradients are folded back through W_kv_b elsewhere].
//
// With P = softmax(s), s = q.K^T / sqrt(d_qk) (causal), and upstream dO:
//   delta[t] = sum_c dO[t,c] o[t,c]                         (bwd_dot_kernel)
//   dV  = P^T dO,  dP = dO V^T,  dS = P * (dP - delta)
//   dK  = dS^T q / sqrt(d_qk)  -> dk_nope = dK[:, :d_nope], dk_pe = sum_i dK[:, d_nope:]
//   dq  = dS K / sqrt(d_qk)
// P is rebuilt from the forward's lse, never stored.
//
// Two flash-style kernels, neither of which holds an S x S matrix:
//  * dkdv: a workgroup of 4 wavefronts owns 128 keys of one head (32 per
//    wavefront; K and V held in registers as B operands) and walks the
//    queries from its diagonal to the end, 32 at a time.  q and dO blocks
//    stream through double-buffered LDS (buffer loads in flight in registers
//    while the previous block is computed), converted to fp16 on the way and
//    stored twice: rows padded for 16-byte operand reads of S = q K^T and
//    dP = dO V^T, and rows padded for conflict-free transposing reads that
//    feed dK^T = q^T dS and dV^T = dO^T P.  The 32x32 accumulators of S / dP
//    hold one key per lane column, which is the B-operand layout of the
//    dK / dV products, so P and dS never leave registers.
//  * dq: a workgroup of 4 wavefronts owns 128 queries (q and dO in
//    registers) and walks keys 0 .. diagonal, 64 at a time, computing
//    S^T = K q^T and dP^T = V dO^T (one query per lane column) and
//    dq^T = K^T dS^T with K^T from transposing reads.
// dk_pe is written per head into a workspace and summed over heads in a fixed
// order (deterministic, no atomics).
//
// Precision (LAGA_OPERANDS_SPLIT): the products that feed dK, dV and hence
// dW_kv_b, dLatent and dgamma use K, V, P and dS as fp16 hi + lo pairs (q and
// dO are exact in fp16); dq uses the hi parts of K and V and single fp16 dS.
// The float32 instantiation uses fp32 MFMAs.
#include <type_traits>

#include "attn_common.hpp"
#include "launch.hpp"

namespace laga {
namespace {

constexpr int kThreads = 256;  // 4 wavefronts, one per SIMD
constexpr float kLog2e = 1.4426950408889634f;

struct BwdArgs {
  const void* q; const void* k_nope; const void* k_pe; const void* v;
  const float* lse; const float* delta; const void* d_o;
  void* dkv; float* dk_pe_part; float* dq;
  int64_t S, plane_k, plane_v, plane_dkv; int B, h; float scale_log2, scale;
};

// Row pitches (elements) of LDS tiles: rows read one per lane with 16-byte
// reads are padded by 16 bytes; rows read with transposing reads (4 rows x
// 64 bytes per half-wavefront) are padded to a pitch of 16 mod 64 dwords.
template <class M> struct TilePad { static constexpr int row = 8, tr = 32; };
template <> struct TilePad<MmaF32> { static constexpr int row = 4, tr = 4; };  // keeps 16-byte row alignment

// 16-byte chunk of `E` converted from a 16-byte chunk of the input type.
template <class E, class InT>
__device__ __forceinline__ void convert_chunk(u32x4 raw, E* out) {
  if constexpr (sizeof(InT) == 2 && sizeof(E) == 2) {     // bf16 -> fp16
    const u16x8 v = __builtin_bit_cast(u16x8, raw);
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = static_cast<E>(bf16_to_f32(v[j]));
  } else if constexpr (sizeof(InT) == sizeof(E)) {        // same type
    *reinterpret_cast<u32x4*>(out) = raw;
  } else {
    static_assert(sizeof(InT) == sizeof(E), "unsupported conversion");
  }
}

template <class T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const T* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), 0, bytes, 0x00020000);
}

// KPL elements of a global row as an operand fragment (zero when !valid).
template <class M, class Src>
__device__ __forceinline__ typename M::frag load_frag(const Src* p, bool valid) {
  typedef typename M::elem E;
  E tmp[M::KPL];
#pragma unroll
  for (int j = 0; j < M::KPL; ++j) tmp[j] = M::from_f32(valid ? to_f32(p[j]) : 0.f);
  return *reinterpret_cast<typename M::frag*>(tmp);
}

// ============================================================ dK / dV kernel
template <class InT, class M, int NS, int DN, int DR, int DV>
struct Dkdv {
  typedef typename M::elem E;
  typedef typename M::frag F;
  static constexpr int DQK = DN + DR, C = DN + DV;
  static constexpr int BQ = 32, BK = 128;
  static constexpr bool TR = M::KPL == 8;  // 16-bit operands: separate transposed-read tiles
  static constexpr int LQR = DQK + TilePad<M>::row, LQT = DQK + TilePad<M>::tr;
  static constexpr int LOR = DV + TilePad<M>::row, LOT = DV + TilePad<M>::tr;
  static constexpr int QR_B = BQ * LQR * sizeof(E), QT_B = TR ? BQ * LQT * sizeof(E) : 0;
  static constexpr int OR_B = BQ * LOR * sizeof(E), OT_B = TR ? BQ * LOT * sizeof(E) : 0;
  static constexpr int BUF_BYTES = QR_B + QT_B + OR_B + OT_B + 2 * BQ * 4;
  // The lo planes of the workgroup's K and V (split operands) stay in LDS for
  // the whole kernel; the hi parts live in registers.
  static constexpr int LLO = (DN > DV ? DN : DV) + TilePad<M>::row;
  static constexpr int LO_B = NS == 2 ? BK * LLO * sizeof(E) : 0;
  static constexpr int LDS_BYTES = 2 * BUF_BYTES + 2 * LO_B;
  static constexpr int KS_QK = DQK / M::K, KS_N = DN / M::K, KS_V = DV / M::K;
  static constexpr int STEPS = BQ / M::K;
  static constexpr int NKT = (DQK + 31) / 32, NVT = DV / 32;
  // Staging: 16-byte chunks of the input rows.
  static constexpr int IPC = 16 / sizeof(InT);
  static constexpr int QCH = BQ * DQK / IPC, OCH = BQ * DV / IPC;
  static constexpr int IQ = (QCH + kThreads - 1) / kThreads, IO = (OCH + kThreads - 1) / kThreads;
  static_assert(DQK % IPC == 0 && DV % IPC == 0, "rows of whole chunks");

  struct Regs { u32x4 q[IQ]; u32x4 o[IO]; float lse2, dlt; };

  __device__ static void load(const BwdArgs& a, int b, int head, int64_t q0, Regs& R) {
    const int nq = static_cast<int>(a.S - q0 < BQ ? a.S - q0 : BQ);
    const int64_t row0 = (b * a.S + q0) * a.h + head;
    const int qrow_b = a.h * DQK * static_cast<int>(sizeof(InT));
    const int orow_b = a.h * DV * static_cast<int>(sizeof(InT));
    const auto rq = rsrc(static_cast<const InT*>(a.q) + row0 * DQK, nq * qrow_b);
    const auto ro = rsrc(static_cast<const InT*>(a.d_o) + row0 * DV, nq * orow_b);
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < IQ; ++i) {
      const int c = i * kThreads + tid;
      const int r = c / (DQK / IPC), j = c % (DQK / IPC);
      R.q[i] = (c < QCH) ? __builtin_amdgcn_raw_buffer_load_b128(rq, r * qrow_b + j * 16, 0, 0) : u32x4{};
    }
#pragma unroll
    for (int i = 0; i < IO; ++i) {
      const int c = i * kThreads + tid;
      const int r = c / (DV / IPC), j = c % (DV / IPC);
      R.o[i] = (c < OCH) ? __builtin_amdgcn_raw_buffer_load_b128(ro, r * orow_b + j * 16, 0, 0) : u32x4{};
    }
    const int t = tid % BQ;
    const int64_t si = (static_cast<int64_t>(b) * a.h + head) * a.S + q0 + t;
    R.lse2 = t < nq ? a.lse[si] * kLog2e : 0.f;
    R.dlt = t < nq ? a.delta[si] : 0.f;
  }

  __device__ static void store(const Regs& R, char* buf) {
    E* Qr = reinterpret_cast<E*>(buf);
    E* Qt = reinterpret_cast<E*>(buf + QR_B);
    E* Or = reinterpret_cast<E*>(buf + QR_B + QT_B);
    E* Ot = reinterpret_cast<E*>(buf + QR_B + QT_B + OR_B);
    float* st = reinterpret_cast<float*>(buf + QR_B + QT_B + OR_B + OT_B);
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < IQ; ++i) {
      const int c = i * kThreads + tid;
      if (c >= QCH) continue;
      const int r = c / (DQK / IPC), col = (c % (DQK / IPC)) * IPC;
      E tmp[IPC];
      convert_chunk<E, InT>(R.q[i], tmp);
#pragma unroll
      for (int j = 0; j < IPC; j += 16 / sizeof(E)) {
        *reinterpret_cast<u32x4*>(Qr + r * LQR + col + j) = *reinterpret_cast<u32x4*>(tmp + j);
        if constexpr (TR) *reinterpret_cast<u32x4*>(Qt + r * LQT + col + j) = *reinterpret_cast<u32x4*>(tmp + j);
      }
    }
#pragma unroll
    for (int i = 0; i < IO; ++i) {
      const int c = i * kThreads + tid;
      if (c >= OCH) continue;
      const int r = c / (DV / IPC), col = (c % (DV / IPC)) * IPC;
      E tmp[IPC];
      convert_chunk<E, InT>(R.o[i], tmp);
#pragma unroll
      for (int j = 0; j < IPC; j += 16 / sizeof(E)) {
        *reinterpret_cast<u32x4*>(Or + r * LOR + col + j) = *reinterpret_cast<u32x4*>(tmp + j);
        if constexpr (TR) *reinterpret_cast<u32x4*>(Ot + r * LOT + col + j) = *reinterpret_cast<u32x4*>(tmp + j);
      }
    }
    if (tid < BQ) {
      st[tid] = R.lse2;
      st[BQ + tid] = R.dlt;
    }
  }

  // A operand of a product whose k index runs over the queries of the block:
  // rows n0 + lane%32 of the transposed tile (dims), queries of accumulator
  // registers st*KPL .. (see acc_key_col).
  __device__ static F tr_frag(const E* Rt, const E* Rr, int ldt, int ldr, int st, int n0) {
    if constexpr (TR) {
      return tr_frag_acc(Rt, ldt, st * 16, n0);
    } else {
      const int lane = threadIdx.x % kWave;
      const int qi = 8 * (st / 4) + 4 * (lane / 32) + (st % 4);
      return Rr[qi * ldr + n0 + lane % 32];
    }
  }

  __device__ static void run(const BwdArgs& a, char* lds) {
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    const int hf = lane / 32, col = lane % 32;
    // Longest key blocks (smallest key index: most queries) first.
    const int nbh = a.B * a.h;
    const int kb = blockIdx.x / nbh;
    const int bh = blockIdx.x % nbh;
    const int b = bh / a.h, head = bh % a.h;
    const int64_t k0 = static_cast<int64_t>(kb) * BK;
    const int64_t wk0 = k0 + wv * 32;
    const int64_t key = wk0 + col;  // this lane's key (B-operand column)
    const bool kvalid = key < a.S;
    const int64_t kc = kvalid ? key : 0;

    // Stationary K (nope hi/lo planes, rope) and V (hi/lo planes) fragments.
    const E* kn = static_cast<const E*>(a.k_nope) + ((b * a.S + kc) * a.h + head) * DN;
    const E* vg = static_cast<const E*>(a.v) + ((b * a.S + kc) * a.h + head) * DV;
    const InT* kp = static_cast<const InT*>(a.k_pe) + (b * a.S + kc) * DR;
    F kf[KS_N], kr[KS_QK - KS_N], vf[KS_V];
#pragma unroll
    for (int s = 0; s < KS_N; ++s) kf[s] = load_frag<M>(kn + s * M::K + hf * M::KPL, kvalid);
#pragma unroll
    for (int s = 0; s < KS_V; ++s) vf[s] = load_frag<M>(vg + s * M::K + hf * M::KPL, kvalid);
#pragma unroll
    for (int s = 0; s < KS_QK - KS_N; ++s) kr[s] = load_frag<M>(kp + s * M::K + hf * M::KPL, kvalid);
    E* klo = reinterpret_cast<E*>(lds + 2 * BUF_BYTES);
    E* vlo = reinterpret_cast<E*>(lds + 2 * BUF_BYTES + LO_B);
    if constexpr (NS == 2) {
      // Lo planes of this workgroup's 128 keys -> LDS rows (published by the
      // first barrier of the query loop).  Keys past the sequence read as zero.
      const int nkw = static_cast<int>(a.S - k0 < BK ? a.S - k0 : BK);
      const int krb = a.h * DN * static_cast<int>(sizeof(E)), vrb = a.h * DV * static_cast<int>(sizeof(E));
      const E* kbase = static_cast<const E*>(a.k_nope) + a.plane_k + ((b * a.S + k0) * a.h + head) * DN;
      const E* vbase = static_cast<const E*>(a.v) + a.plane_v + ((b * a.S + k0) * a.h + head) * DV;
      const auto rk = rsrc(kbase, nkw * krb), rv = rsrc(vbase, nkw * vrb);
      constexpr int EPC = 16 / sizeof(E);
#pragma unroll
      for (int i = 0; i < BK * DN / EPC / kThreads; ++i) {
        const int c = i * kThreads + static_cast<int>(threadIdx.x);
        const int r = c / (DN / EPC), j = c % (DN / EPC);
        *reinterpret_cast<u32x4*>(klo + r * LLO + j * EPC) = __builtin_amdgcn_raw_buffer_load_b128(rk, r * krb + j * 16, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < BK * DV / EPC / kThreads; ++i) {
        const int c = i * kThreads + static_cast<int>(threadIdx.x);
        const int r = c / (DV / EPC), j = c % (DV / EPC);
        *reinterpret_cast<u32x4*>(vlo + r * LLO + j * EPC) = __builtin_amdgcn_raw_buffer_load_b128(rv, r * vrb + j * 16, 0, 0);
      }
    }
    const E* klo_row = klo + (wv * 32 + col) * LLO + hf * M::KPL;  // this lane's key
    const E* vlo_row = vlo + (wv * 32 + col) * LLO + hf * M::KPL;

    f32x16 dk[NKT], dvt[NVT];
#pragma unroll
    for (int n = 0; n < NKT; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) dk[n][r] = 0.f;
#pragma unroll
    for (int n = 0; n < NVT; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) dvt[n][r] = 0.f;

    const int nqb = static_cast<int>((a.S - k0 + BQ - 1) / BQ);
    Regs R;
    load(a, b, head, k0, R);
    for (int it = 0; it < nqb; ++it) {
      const int64_t q0 = k0 + static_cast<int64_t>(it) * BQ;
      char* buf = lds + (it & 1) * BUF_BYTES;
      store(R, buf);
      __syncthreads();
      if (it + 1 < nqb) load(a, b, head, q0 + BQ, R);
      if (q0 + BQ - 1 < wk0) continue;  // every query of the block precedes this wavefront's keys

      const E* Qr = reinterpret_cast<const E*>(buf);
      const E* Qt = reinterpret_cast<const E*>(buf + QR_B);
      const E* Or = reinterpret_cast<const E*>(buf + QR_B + QT_B);
      const E* Ot = reinterpret_cast<const E*>(buf + QR_B + QT_B + OR_B);
      const float* st = reinterpret_cast<const float*>(buf + QR_B + QT_B + OR_B + OT_B);
      const int nq = static_cast<int>(a.S - q0 < BQ ? a.S - q0 : BQ);

      // S[q, key], dP[q, key]: rows = queries 8g + 4hf + i, column = key.
      f32x16 sc, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) { sc[r] = 0.f; dp[r] = 0.f; }
      const E* qrow = Qr + col * LQR + hf * M::KPL;
#pragma unroll
      for (int s = 0; s < KS_N; ++s) {
        const F qa = lds_frag<M>(qrow + s * M::K);
        sc = M::mma(qa, kf[s], sc);
        if constexpr (NS == 2) sc = M::mma(qa, lds_frag<M>(klo_row + s * M::K), sc);
      }
#pragma unroll
      for (int s = KS_N; s < KS_QK; ++s) sc = M::mma(lds_frag<M>(qrow + s * M::K), kr[s - KS_N], sc);
      const E* orow = Or + col * LOR + hf * M::KPL;
#pragma unroll
      for (int s = 0; s < KS_V; ++s) {
        const F oa = lds_frag<M>(orow + s * M::K);
        dp = M::mma(oa, vf[s], dp);
        if constexpr (NS == 2) dp = M::mma(oa, lds_frag<M>(vlo_row + s * M::K), dp);
      }

      // P = exp(s - lse) and dS = P (dP - delta), per query row of the block.
      const bool edge = q0 < wk0 + 31 || nq < BQ;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(st + 8 * g + 4 * hf);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(st + BQ + 8 * g + 4 * hf);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g + i;
          float p = __builtin_amdgcn_exp2f(fmaf(sc[r], a.scale_log2, -l4[i]));
          if (edge) {
            const int qi = 8 * g + 4 * hf + i;
            if (key > q0 + qi || qi >= nq) p = 0.f;
          }
          sc[r] = p;
          dp[r] = p * (dp[r] - d4[i]);
        }
      }

      // dV^T[dv, key] += dO^T P ; dK^T[d, key] += q^T dS   (k = queries)
#pragma unroll
      for (int stp = 0; stp < STEPS; ++stp) {
        E ph[NS][M::KPL], dh[NS][M::KPL];
#pragma unroll
        for (int j = 0; j < M::KPL; ++j) {
          E t1[NS], t2[NS];
          split_to<M, NS>(sc[stp * M::KPL + j], t1);
          split_to<M, NS>(dp[stp * M::KPL + j], t2);
#pragma unroll
          for (int p = 0; p < NS; ++p) { ph[p][j] = t1[p]; dh[p][j] = t2[p]; }
        }
#pragma unroll
        for (int n = 0; n < NVT; ++n) {
          const F oa = tr_frag(Ot, Or, LOT, LOR, stp, n * 32);
#pragma unroll
          for (int p = 0; p < NS; ++p) dvt[n] = M::mma(oa, *reinterpret_cast<F*>(ph[p]), dvt[n]);
        }
#pragma unroll
        for (int n = 0; n < NKT; ++n) {
          const F qa = tr_frag(Qt, Qr, LQT, LQR, stp, n * 32);
#pragma unroll
          for (int p = 0; p < NS; ++p) dk[n] = M::mma(qa, *reinterpret_cast<F*>(dh[p]), dk[n]);
        }
      }
    }

    if (!kvalid) return;
    // Lane holds column `key`; accumulator r is row 8(r/4) + 4hf + r%4 of its 32-row atom.
    const int64_t orow = ((b * a.S + key) * a.h + head) * C;
#pragma unroll
    for (int n = 0; n < NKT; ++n)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = n * 32 + 8 * g + 4 * hf;
        if (d >= DQK) continue;
        f32x4 w = {dk[n][4 * g] * a.scale, dk[n][4 * g + 1] * a.scale, dk[n][4 * g + 2] * a.scale,
                   dk[n][4 * g + 3] * a.scale};
        if (d < DN)
          store_dkv(a, orow + d, w);
        else
          *reinterpret_cast<f32x4*>(a.dk_pe_part + (static_cast<int64_t>(head) * a.B * a.S + b * a.S + key) * DR +
                                    (d - DN)) = w;
      }
#pragma unroll
    for (int n = 0; n < NVT; ++n)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = n * 32 + 8 * g + 4 * hf;
        f32x4 w = {dvt[n][4 * g], dvt[n][4 * g + 1], dvt[n][4 * g + 2], dvt[n][4 * g + 3]};
        store_dkv(a, orow + DN + d, w);
      }
  }

  // Four consecutive dK / dV values in the fold GEMMs' operand format: bf16 hi
  // and lo planes (16-bit operand path) or fp32.
  __device__ static void store_dkv(const BwdArgs& a, int64_t at, f32x4 w) {
    if constexpr (std::is_same<M, MmaF32>::value) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.dkv) + at) = w;
    } else {
      u16x4 hi, lo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hi[j] = f32_to_bf16(w[j]);
        lo[j] = f32_to_bf16(w[j] - bf16_to_f32(hi[j]));
      }
      bf16_t* p = static_cast<bf16_t*>(a.dkv) + at;
      *reinterpret_cast<u16x4*>(p) = hi;
      *reinterpret_cast<u16x4*>(p + a.plane_dkv) = lo;
    }
  }
};

// ================================================================ dq kernel
template <class InT, class M, int NS, int DN, int DR, int DV>
struct Dq {
  typedef typename M::elem E;
  typedef typename M::frag F;
  static constexpr int DQK = DN + DR;
  static constexpr int BM = 128, BN = 64;
  static constexpr bool TR = M::KPL == 8;
  static constexpr int LKR = DQK + TilePad<M>::row, LKT = DQK + TilePad<M>::tr, LVR = DV + TilePad<M>::row;
  static constexpr int KR_B = BN * LKR * sizeof(E), KT_B = TR ? BN * LKT * sizeof(E) : 0;
  static constexpr int VR_B = BN * LVR * sizeof(E);
  static constexpr int BUF_BYTES = KR_B + KT_B + VR_B;
  static constexpr int KS_QK = DQK / M::K, KS_V = DV / M::K;
  static constexpr int NT = BN / 32, NQT = (DQK + 31) / 32, STEPS = 32 / M::K;
  // Staging chunks (16 bytes): nope part of K (hi plane), rope band (input type), V (hi plane).
  static constexpr int EPC = 16 / sizeof(E), IPC = 16 / sizeof(InT);
  static constexpr int KCH = BN * DN / EPC, PCH = BN * DR / IPC, VCH = BN * DV / EPC;
  static constexpr int IK = (KCH + kThreads - 1) / kThreads, IP = (PCH + kThreads - 1) / kThreads;
  static constexpr int IV = (VCH + kThreads - 1) / kThreads;

  struct Regs { u32x4 k[IK]; u32x4 p[IP]; u32x4 v[IV]; };

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
      R.k[i] = (c < KCH) ? __builtin_amdgcn_raw_buffer_load_b128(rk, r * krow_b + j * 16, 0, 0) : u32x4{};
    }
#pragma unroll
    for (int i = 0; i < IP; ++i) {
      const int c = i * kThreads + tid;
      const int r = c / (DR / IPC), j = c % (DR / IPC);
      R.p[i] = (c < PCH) ? __builtin_amdgcn_raw_buffer_load_b128(rp, r * prow_b + j * 16, 0, 0) : u32x4{};
    }
#pragma unroll
    for (int i = 0; i < IV; ++i) {
      const int c = i * kThreads + tid;
      const int r = c / (DV / EPC), j = c % (DV / EPC);
      R.v[i] = (c < VCH) ? __builtin_amdgcn_raw_buffer_load_b128(rv, r * vrow_b + j * 16, 0, 0) : u32x4{};
    }
  }

  __device__ static void store(const Regs& R, char* buf) {
    E* Kr = reinterpret_cast<E*>(buf);
    E* Kt = reinterpret_cast<E*>(buf + KR_B);
    E* Vr = reinterpret_cast<E*>(buf + KR_B + KT_B);
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < IK; ++i) {
      const int c = i * kThreads + tid;
      if (c >= KCH) continue;
      const int r = c / (DN / EPC), col = (c % (DN / EPC)) * EPC;
      *reinterpret_cast<u32x4*>(Kr + r * LKR + col) = R.k[i];
      if constexpr (TR) *reinterpret_cast<u32x4*>(Kt + r * LKT + col) = R.k[i];
    }
#pragma unroll
    for (int i = 0; i < IP; ++i) {
      const int c = i * kThreads + tid;
      if (c >= PCH) continue;
      const int r = c / (DR / IPC), col = DN + (c % (DR / IPC)) * IPC;
      E tmp[IPC];
      convert_chunk<E, InT>(R.p[i], tmp);
#pragma unroll
      for (int j = 0; j < IPC; j += EPC) {
        *reinterpret_cast<u32x4*>(Kr + r * LKR + col + j) = *reinterpret_cast<u32x4*>(tmp + j);
        if constexpr (TR) *reinterpret_cast<u32x4*>(Kt + r * LKT + col + j) = *reinterpret_cast<u32x4*>(tmp + j);
      }
    }
#pragma unroll
    for (int i = 0; i < IV; ++i) {
      const int c = i * kThreads + tid;
      if (c >= VCH) continue;
      const int r = c / (DV / EPC), col = (c % (DV / EPC)) * EPC;
      *reinterpret_cast<u32x4*>(Vr + r * LVR + col) = R.v[i];
    }
  }

  // A operand of dq^T += K^T dS^T for one MFMA step of key atom t.
  __device__ static F kt_frag(const E* Kt, const E* Kr, int t, int st, int n0) {
    if constexpr (TR) {
      return tr_frag_acc(Kt, LKT, t * 32 + st * 16, n0);
    } else {
      const int lane = threadIdx.x % kWave;
      const int k = t * 32 + 8 * (st / 4) + 4 * (lane / 32) + (st % 4);
      return Kr[k * LKR + n0 + lane % 32];
    }
  }

  __device__ static void run(const BwdArgs& a, char* lds) {
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
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

    const int64_t qrow = (b * a.S + (qvalid ? tq : 0)) * a.h + head;
    const InT* qg = static_cast<const InT*>(a.q) + qrow * DQK;
    const InT* og = static_cast<const InT*>(a.d_o) + qrow * DV;
    F qf[KS_QK], of[KS_V];
#pragma unroll
    for (int s = 0; s < KS_QK; ++s) qf[s] = load_frag<M>(qg + s * M::K + hf * M::KPL, qvalid);
#pragma unroll
    for (int s = 0; s < KS_V; ++s) of[s] = load_frag<M>(og + s * M::K + hf * M::KPL, qvalid);
    const int64_t si = (static_cast<int64_t>(b) * a.h + head) * a.S + (qvalid ? tq : 0);
    const float lse2 = qvalid ? a.lse[si] * kLog2e : 0.f;
    const float dl = qvalid ? a.delta[si] : 0.f;

    f32x16 dq[NQT];
#pragma unroll
    for (int n = 0; n < NQT; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[n][r] = 0.f;

    int64_t kend = q0 + BM;
    if (kend > a.S) kend = a.S;
    const int nkb = static_cast<int>((kend + BN - 1) / BN);
    Regs R;
    load(a, b, head, 0, R);
    for (int kb = 0; kb < nkb; ++kb) {
      const int64_t key0 = static_cast<int64_t>(kb) * BN;
      char* buf = lds + (kb & 1) * BUF_BYTES;
      store(R, buf);
      __syncthreads();
      if (kb + 1 < nkb) load(a, b, head, key0 + BN, R);
      if (key0 > qw + 31) continue;  // whole block above this wavefront's diagonal

      const E* Kr = reinterpret_cast<const E*>(buf);
      const E* Kt = reinterpret_cast<const E*>(buf + KR_B);
      const E* Vr = reinterpret_cast<const E*>(buf + KR_B + KT_B);
      f32x16 sc[NT], dp[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) { sc[t][r] = 0.f; dp[t][r] = 0.f; }
        const E* krow = Kr + (t * 32 + col) * LKR + hf * M::KPL;
#pragma unroll
        for (int s = 0; s < KS_QK; ++s) sc[t] = M::mma(lds_frag<M>(krow + s * M::K), qf[s], sc[t]);
        const E* vrow = Vr + (t * 32 + col) * LVR + hf * M::KPL;
#pragma unroll
        for (int s = 0; s < KS_V; ++s) dp[t] = M::mma(lds_frag<M>(vrow + s * M::K), of[s], dp[t]);
      }
      const bool edge = key0 + BN - 1 > qw || key0 + BN > a.S;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(fmaf(sc[t][r], a.scale_log2, -lse2));
          if (edge) {
            const int64_t u = key0 + t * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
            if (u > tq || u >= a.S) p = 0.f;
          }
          dp[t][r] = p * (dp[t][r] - dl);
        }
      // dq^T[d, q] += K^T dS^T  (k = keys of the accumulators)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int stp = 0; stp < STEPS; ++stp) {
          E dh[M::KPL];
#pragma unroll
          for (int j = 0; j < M::KPL; ++j) dh[j] = M::from_f32(dp[t][stp * M::KPL + j]);
          const F df = *reinterpret_cast<F*>(dh);
#pragma unroll
          for (int n = 0; n < NQT; ++n) dq[n] = M::mma(kt_frag(Kt, Kr, t, stp, n * 32), df, dq[n]);
        }
    }
    if (!qvalid) return;
    float* out = a.dq + qrow * DQK;
#pragma unroll
    for (int n = 0; n < NQT; ++n)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (n * 32 + 8 * g + 4 * hf >= DQK) continue;
        f32x4 w = {dq[n][4 * g] * a.scale, dq[n][4 * g + 1] * a.scale, dq[n][4 * g + 2] * a.scale,
                   dq[n][4 * g + 3] * a.scale};
        *reinterpret_cast<f32x4*>(out + n * 32 + 8 * g + 4 * hf) = w;
      }
  }
};

template <class InT, class M, int NS, int DN, int DR, int DV>
__global__ __launch_bounds__(kThreads) void dkdv_kernel(BwdArgs a) {
  typedef Dkdv<InT, M, NS, DN, DR, DV> Kn;
  __shared__ __attribute__((aligned(16))) char lds[Kn::LDS_BYTES];
  Kn::run(a, lds);
}

template <class InT, class M, int NS, int DN, int DR, int DV>
__global__ __launch_bounds__(kThreads) void dq_kernel(BwdArgs a) {
  typedef Dq<InT, M, NS, DN, DR, DV> Kn;
  __shared__ __attribute__((aligned(16))) char lds[2 * Kn::BUF_BYTES];
  Kn::run(a, lds);
}

BwdArgs make_args(const Shape& s, const void* q, const void* kn, const void* kp, const void* v, const float* lse,
                  const float* delta, const void* d_o) {
  BwdArgs a;
  a.q = q; a.k_nope = kn; a.k_pe = kp; a.v = v; a.lse = lse; a.delta = delta; a.d_o = d_o;
  a.dkv = nullptr; a.dk_pe_part = nullptr; a.dq = nullptr;
  a.S = s.S; a.B = static_cast<int>(s.B); a.h = s.h;
  a.plane_k = s.T * s.h * s.d_nope;
  a.plane_v = s.T * s.h * s.d_v;
  a.plane_dkv = s.T * s.h * s.C();
  a.scale = 1.0f / sqrtf(static_cast<float>(s.d_qk()));
  a.scale_log2 = kLog2e * a.scale;
  return a;
}

// delta[b, i, t] = sum_c d_o[b, t, i, c] * o[b, t, i, c]  (one wavefront per row).
template <class InT, int DV>
__global__ __launch_bounds__(256) void bwd_dot_kernel(const float* __restrict__ o, const InT* __restrict__ d_o,
                                                      float* __restrict__ delta, int64_t rows, int h,
                                                      int64_t S) {
  const int lane = threadIdx.x % kWave;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;  // (b, t, i)
  if (row >= rows) return;
  float acc = 0.f;
#pragma unroll
  for (int c = lane; c < DV; c += kWave) acc += o[row * DV + c] * to_f32(d_o[row * DV + c]);
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

hipError_t launch_attn_bwd_dkdv(const Shape& s, const void* q, const void* kn, const void* kp, const void* v,
                                const float* lse, const float* delta, const void* d_o, void* dkv,
                                float* dk_pe_part, hipStream_t st) {
  BwdArgs a = make_args(s, q, kn, kp, v, lse, delta, d_o);
  a.dkv = dkv;
  a.dk_pe_part = dk_pe_part;
  const unsigned grid = static_cast<unsigned>(((s.S + 127) / 128) * s.B * s.h);
  if (s.bf16 && s.split && s.d_nope == 128 && s.d_rope == 64 && s.d_v == 128)
    hipLaunchKernelGGL((dkdv_kernel<bf16_t, MmaF16, 2, 128, 64, 128>), dim3(grid), dim3(kThreads), 0, st, a);
  else if (!s.bf16 && s.d_nope == 32 && s.d_rope == 16 && s.d_v == 32)
    hipLaunchKernelGGL((dkdv_kernel<float, MmaF32, 1, 32, 16, 32>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    return hipErrorNotSupported;
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dq(const Shape& s, const void* q, const void* kn, const void* kp, const void* v,
                              const float* lse, const float* delta, const void* d_o, float* dq, hipStream_t st) {
  BwdArgs a = make_args(s, q, kn, kp, v, lse, delta, d_o);
  a.dq = dq;
  const unsigned grid = static_cast<unsigned>(((s.S + 127) / 128) * s.B * s.h);
  if (s.bf16 && s.split && s.d_nope == 128 && s.d_rope == 64 && s.d_v == 128)
    hipLaunchKernelGGL((dq_kernel<bf16_t, MmaF16, 2, 128, 64, 128>), dim3(grid), dim3(kThreads), 0, st, a);
  else if (!s.bf16 && s.d_nope == 32 && s.d_rope == 16 && s.d_v == 32)
    hipLaunchKernelGGL((dq_kernel<float, MmaF32, 1, 32, 16, 32>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    return hipErrorNotSupported;
  return hipGetLastError();
}

}  // namespace laga
