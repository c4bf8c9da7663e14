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
//  * dkdv: a workgroup owns 128 keys of one head (32 per wavefront, K and V
//    held in registers as B operands) and walks the queries from its diagonal
//    to the end, 32 at a time, staging q / dO through LDS both row-major (for
//    S = q K^T and dP = dO V^T) and transposed (for dK^T = q^T dS and
//    dV^T = dO^T P).  The 32x32 accumulators of S / dP put one key per lane
//    column, which is exactly the B-operand layout of the dK / dV products.
//  * dq: a workgroup owns 128 queries (32 per wavefront, q and dO in registers)
//    and walks keys 0 .. diagonal, 64 at a time, computing S^T = K q^T and
//    dP^T = V dO^T so that one query sits per lane column, and dq^T = K^T dS^T.
// dk_pe is written per head into a workspace and summed over heads in a fixed
// order (deterministic, no atomics).
//
// Precision (LAGA_OPERANDS_SPLIT): K, V, P and dS enter the products of dK and
// dV as fp16 hi + lo pairs (q and dO are exact in fp16); dq uses single fp16 dS
// and K_hi.  The float32 instantiation uses fp32 MFMAs.
#include "device.hpp"
#include "launch.hpp"

namespace laga {
namespace {

constexpr int kThreads = 256;

template <class M> struct BPad { static constexpr int v = 8; };
template <> struct BPad<MmaF32> { static constexpr int v = 1; };

// Stage a [ROWS x COLS] tile whose row r starts at src + r*ld (rows >= nrows are
// zero) into LDS: row-major planes dst_r[s*plane_r + r*LDR + c] (NS_R parts) and/or
// transposed dst_t[c*LDT + acc_key_col(r)] (hi part only).  Each thread item is
// 4 rows x VEC columns read with 16-byte loads.
template <class M, class Src, int ROWS, int COLS, int NS_R, bool ROW, bool TRANS>
__device__ __forceinline__ void stage(const Src* __restrict__ src, int64_t ld, int nrows,
                                      typename M::elem* dst_r, int LDR, int plane_r,
                                      typename M::elem* dst_t, int LDT) {
  typedef typename M::elem E;
  constexpr int VEC = 16 / sizeof(Src);
  static_assert(COLS % VEC == 0 && ROWS % 4 == 0, "tile shape");
  typedef Src svec __attribute__((ext_vector_type(VEC)));
  constexpr int ITEMS = (ROWS / 4) * (COLS / VEC);
  for (int it = threadIdx.x; it < ITEMS; it += kThreads) {
    const int rg = it / (COLS / VEC), c = (it % (COLS / VEC)) * VEC;
    svec v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = rg * 4 + r;
      v[r] = row < nrows ? *reinterpret_cast<const svec*>(src + row * ld + c) : svec{};
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        E part[NS_R];
        split_to<M, NS_R>(to_f32(v[r][e]), part);
        if constexpr (ROW) {
#pragma unroll
          for (int s = 0; s < NS_R; ++s) dst_r[s * plane_r + (rg * 4 + r) * LDR + c + e] = part[s];
        }
        if constexpr (TRANS) dst_t[(c + e) * LDT + acc_key_col(rg * 4 + r)] = part[0];
      }
    }
  }
}

// Load a KPL-element B-operand fragment of row `row` (columns col0..) of a
// global matrix, split into SPLIT parts.
template <class M, int SPLIT, class Src>
__device__ __forceinline__ void load_frag_split(const Src* p, bool valid, typename M::frag* out) {
  typedef typename M::elem E;
  E part[SPLIT][M::KPL];
#pragma unroll
  for (int j = 0; j < M::KPL; ++j) {
    E tmp[SPLIT];
    split_to<M, SPLIT>(valid ? to_f32(p[j]) : 0.f, tmp);
#pragma unroll
    for (int s = 0; s < SPLIT; ++s) part[s][j] = tmp[s];
  }
#pragma unroll
  for (int s = 0; s < SPLIT; ++s) out[s] = *reinterpret_cast<typename M::frag*>(part[s]);
}

struct BwdArgs {
  const void* q; const void* k_nope; const void* k_pe; const void* v;
  const float* lse; const float* delta; const void* d_o;
  float* dkv; float* dk_pe_part; float* dq;
  int64_t S, plane_k, plane_v; int B, h; float scale_log2, scale;
};

// ============================================================ dK / dV kernel
template <class InT, class KvT, class M, int SPLIT, int DN, int DR, int DV>
struct DkdvKernel {
  typedef typename M::elem E;
  typedef typename M::frag F;
  static constexpr int DQK = DN + DR, C = DN + DV;
  static constexpr int BQ = 32, BK = 128;
  static constexpr int PAD = BPad<M>::v;
  static constexpr int LDQ = DQK + PAD, LDO = DV + PAD, LDT = BQ + PAD;
  static constexpr int KS_QK = DQK / M::K, KS_NOPE = DN / M::K, KS_V = DV / M::K;
  static constexpr int STEPS = BQ / M::K;
  // d_qk need not be a multiple of 32: the last dK^T atom reads padding rows of
  // q^T whose results are never stored.
  static constexpr int NKT = (DQK + 31) / 32, NVT = DV / 32;
  static constexpr int OFF_DO = BQ * LDQ, OFF_QT = OFF_DO + BQ * LDO, OFF_OT = OFF_QT + NKT * 32 * LDT;
  static constexpr int LDS_ELEMS = OFF_OT + DV * LDT;

  __device__ static void run(const BwdArgs& a, E* lds, float* stat) {
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

    const InT* qg = static_cast<const InT*>(a.q);
    const InT* og = static_cast<const InT*>(a.d_o);
    const KvT* kn = static_cast<const KvT*>(a.k_nope);
    const KvT* vg = static_cast<const KvT*>(a.v);
    const InT* kp = static_cast<const InT*>(a.k_pe);

    // Stationary K and V fragments of this lane's key.
    F kf[SPLIT][KS_QK], vf[SPLIT][KS_V];
    const int64_t krow = ((b * a.S + (kvalid ? key : 0)) * a.h + head);
#pragma unroll
    for (int s = 0; s < KS_QK; ++s) {
      const int d0 = s * M::K + hf * M::KPL;
      F tmp[SPLIT];
      if (d0 < DN) {
#pragma unroll
        for (int p = 0; p < SPLIT; ++p) load_frag_split<M, 1>(kn + p * a.plane_k + krow * DN + d0, kvalid, &tmp[p]);
      } else {
        load_frag_split<M, 1>(kp + (b * a.S + (kvalid ? key : 0)) * DR + (d0 - DN), kvalid, tmp);
        if constexpr (SPLIT == 2) tmp[1] = F{};
      }
#pragma unroll
      for (int p = 0; p < SPLIT; ++p) kf[p][s] = tmp[p];
    }
#pragma unroll
    for (int s = 0; s < KS_V; ++s) {
      F tmp[SPLIT];
#pragma unroll
      for (int p = 0; p < SPLIT; ++p)
        load_frag_split<M, 1>(vg + p * a.plane_v + krow * DV + s * M::K + hf * M::KPL, kvalid, &tmp[p]);
#pragma unroll
      for (int p = 0; p < SPLIT; ++p) vf[p][s] = tmp[p];
    }

    f32x16 dk[NKT], dvt[NVT];
#pragma unroll
    for (int n = 0; n < NKT; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) dk[n][r] = 0.f;
#pragma unroll
    for (int n = 0; n < NVT; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) dvt[n][r] = 0.f;

    E* Qs = lds;
    E* Os = lds + OFF_DO;
    E* Qt = lds + OFF_QT;
    E* Ot = lds + OFF_OT;
    float* lse2 = stat;       // [BQ] lse in log2 units
    float* dlt = stat + BQ;   // [BQ] delta

    for (int64_t q0 = k0; q0 < a.S; q0 += BQ) {
      const int nq = static_cast<int>(a.S - q0 < BQ ? a.S - q0 : BQ);
      __syncthreads();
      stage<M, InT, BQ, DQK, 1, true, true>(qg + ((b * a.S + q0) * a.h + head) * DQK, int64_t(a.h) * DQK, nq,
                                            Qs, LDQ, 0, Qt, LDT);
      stage<M, InT, BQ, DV, 1, true, true>(og + ((b * a.S + q0) * a.h + head) * DV, int64_t(a.h) * DV, nq,
                                           Os, LDO, 0, Ot, LDT);
      if (threadIdx.x < BQ) {
        const int t = threadIdx.x;
        const bool ok = t < nq;
        lse2[t] = ok ? a.lse[(static_cast<int64_t>(b) * a.h + head) * a.S + q0 + t] * 1.4426950408889634f : 0.f;
        dlt[t] = ok ? a.delta[(static_cast<int64_t>(b) * a.h + head) * a.S + q0 + t] : 0.f;
      }
      __syncthreads();
      if (q0 + BQ - 1 < wk0) continue;  // every query of the block is before this wavefront's keys

      // S[q, key] and dP[q, key]: rows = queries 8g + 4hf + i, column = key.
      f32x16 sc, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) { sc[r] = 0.f; dp[r] = 0.f; }
      const E* qrow = Qs + col * LDQ + hf * M::KPL;
#pragma unroll
      for (int s = 0; s < KS_QK; ++s) sc = M::mma(lds_frag<M>(qrow + s * M::K), kf[0][s], sc);
      if constexpr (SPLIT == 2) {
#pragma unroll
        for (int s = 0; s < KS_NOPE; ++s) sc = M::mma(lds_frag<M>(qrow + s * M::K), kf[1][s], sc);
      }
      const E* orow = Os + col * LDO + hf * M::KPL;
#pragma unroll
      for (int s = 0; s < KS_V; ++s) {
        const F of = lds_frag<M>(orow + s * M::K);
        dp = M::mma(of, vf[0][s], dp);
        if constexpr (SPLIT == 2) dp = M::mma(of, vf[1][s], dp);
      }
      const bool diag = q0 < wk0 + 31;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = 8 * (r / 4) + 4 * hf + (r % 4);
        float p = exp2f(sc[r] * a.scale_log2 - lse2[qi]);
        if ((diag && key > q0 + qi) || qi >= nq) p = 0.f;
        sc[r] = p;
        dp[r] = p * (dp[r] - dlt[qi]);
      }
      // dV^T[dv, key] += dO^T P ; dK^T[d, key] += q^T dS  (k = queries, permuted).
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        E ph[SPLIT][M::KPL], dh[SPLIT][M::KPL];
#pragma unroll
        for (int j = 0; j < M::KPL; ++j) {
          E t1[SPLIT], t2[SPLIT];
          split_to<M, SPLIT>(sc[st * M::KPL + j], t1);
          split_to<M, SPLIT>(dp[st * M::KPL + j], t2);
#pragma unroll
          for (int s = 0; s < SPLIT; ++s) { ph[s][j] = t1[s]; dh[s][j] = t2[s]; }
        }
        const int r0 = st * M::KPL;
        const int qc = acc_key_col(8 * (r0 / 4) + 4 * hf + (r0 % 4));
#pragma unroll
        for (int s = 0; s < SPLIT; ++s) {
          const F pf = *reinterpret_cast<F*>(ph[s]);
          const F df = *reinterpret_cast<F*>(dh[s]);
#pragma unroll
          for (int n = 0; n < NVT; ++n) dvt[n] = M::mma(lds_frag<M>(Ot + (n * 32 + col) * LDT + qc), pf, dvt[n]);
#pragma unroll
          for (int n = 0; n < NKT; ++n) dk[n] = M::mma(lds_frag<M>(Qt + (n * 32 + col) * LDT + qc), df, dk[n]);
        }
      }
    }

    if (!kvalid) return;
    // Lane holds column `key`; accumulator r is row 8(r/4) + 4hf + r%4 of its 32-row atom.
    float* out = a.dkv + ((b * a.S + key) * a.h + head) * C;
#pragma unroll
    for (int n = 0; n < NKT; ++n)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = n * 32 + 8 * g + 4 * hf;
        f32x4 w = {dk[n][4 * g] * a.scale, dk[n][4 * g + 1] * a.scale, dk[n][4 * g + 2] * a.scale,
                   dk[n][4 * g + 3] * a.scale};
        if (d >= DQK) continue;
        if (d < DN)
          *reinterpret_cast<f32x4*>(out + d) = w;
        else
          *reinterpret_cast<f32x4*>(a.dk_pe_part + (static_cast<int64_t>(head) * a.B * a.S + b * a.S + key) * DR + (d - DN)) = w;
      }
#pragma unroll
    for (int n = 0; n < NVT; ++n)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = n * 32 + 8 * g + 4 * hf;
        f32x4 w = {dvt[n][4 * g], dvt[n][4 * g + 1], dvt[n][4 * g + 2], dvt[n][4 * g + 3]};
        *reinterpret_cast<f32x4*>(out + DN + d) = w;
      }
  }
};

// ================================================================ dq kernel
template <class InT, class KvT, class M, int SPLIT, int DN, int DR, int DV>
struct DqKernel {
  typedef typename M::elem E;
  typedef typename M::frag F;
  static constexpr int DQK = DN + DR;
  static constexpr int BM = 128, BN = 64;
  static constexpr int PAD = BPad<M>::v;
  static constexpr int LDK = DQK + PAD, LDV = DV + PAD, LDT = BN + PAD;
  static constexpr int KS_QK = DQK / M::K, KS_NOPE = DN / M::K, KS_V = DV / M::K;
  static constexpr int NT = BN / 32, NQT = (DQK + 31) / 32, STEPS = 32 / M::K;
  static constexpr int OFF_KL = BN * LDK;
  static constexpr int OFF_V = OFF_KL + (SPLIT == 2 ? BN * LDK : 0);  // lo plane keeps the hi stride
  static constexpr int OFF_KT = OFF_V + SPLIT * BN * LDV;
  static constexpr int LDS_ELEMS = OFF_KT + NQT * 32 * LDT;  // K^T padded to whole atoms

  __device__ static void run(const BwdArgs& a, E* lds) {
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

    const InT* qg = static_cast<const InT*>(a.q);
    const InT* og = static_cast<const InT*>(a.d_o);
    F qf[KS_QK], of[KS_V];
    const int64_t qrow = (b * a.S + (qvalid ? tq : 0)) * a.h + head;
#pragma unroll
    for (int s = 0; s < KS_QK; ++s) load_frag_split<M, 1>(qg + qrow * DQK + s * M::K + hf * M::KPL, qvalid, &qf[s]);
#pragma unroll
    for (int s = 0; s < KS_V; ++s) load_frag_split<M, 1>(og + qrow * DV + s * M::K + hf * M::KPL, qvalid, &of[s]);
    const float lse2 = qvalid ? a.lse[(static_cast<int64_t>(b) * a.h + head) * a.S + tq] * 1.4426950408889634f : 0.f;
    const float dl = qvalid ? a.delta[(static_cast<int64_t>(b) * a.h + head) * a.S + tq] : 0.f;

    f32x16 dq[NQT];
#pragma unroll
    for (int n = 0; n < NQT; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[n][r] = 0.f;

    E* Ks = lds;
    E* Kl = lds + OFF_KL;
    E* Vs = lds + OFF_V;
    E* Kt = lds + OFF_KT;
    const KvT* kn = static_cast<const KvT*>(a.k_nope);
    const KvT* vg = static_cast<const KvT*>(a.v);
    const InT* kp = static_cast<const InT*>(a.k_pe);

    int64_t kend = q0 + BM;
    if (kend > a.S) kend = a.S;
    for (int64_t key0 = 0; key0 < kend; key0 += BN) {
      const int nk = static_cast<int>(a.S - key0 < BN ? a.S - key0 : BN);
      __syncthreads();
      stage<M, KvT, BN, DN, 1, true, true>(kn + ((b * a.S + key0) * a.h + head) * DN, int64_t(a.h) * DN, nk,
                                           Ks, LDK, 0, Kt, LDT);
      if constexpr (SPLIT == 2)
        stage<M, KvT, BN, DN, 1, true, false>(kn + a.plane_k + ((b * a.S + key0) * a.h + head) * DN,
                                              int64_t(a.h) * DN, nk, Kl, LDK, 0, nullptr, 0);
      stage<M, InT, BN, DR, 1, true, true>(kp + (b * a.S + key0) * DR, DR, nk, Ks + DN, LDK, 0, Kt + DN * LDT, LDT);
#pragma unroll
      for (int p = 0; p < SPLIT; ++p)
        stage<M, KvT, BN, DV, 1, true, false>(vg + p * a.plane_v + ((b * a.S + key0) * a.h + head) * DV,
                                              int64_t(a.h) * DV, nk, Vs + p * BN * LDV, LDV, 0, nullptr, 0);
      __syncthreads();
      if (key0 > qw + 31) continue;

      f32x16 sc[NT], dp[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) { sc[t][r] = 0.f; dp[t][r] = 0.f; }
        const E* krow = Ks + (t * 32 + col) * LDK + hf * M::KPL;
#pragma unroll
        for (int s = 0; s < KS_QK; ++s) sc[t] = M::mma(lds_frag<M>(krow + s * M::K), qf[s], sc[t]);
        if constexpr (SPLIT == 2) {
          const E* lrow = Kl + (t * 32 + col) * LDK + hf * M::KPL;
#pragma unroll
          for (int s = 0; s < KS_NOPE; ++s) sc[t] = M::mma(lds_frag<M>(lrow + s * M::K), qf[s], sc[t]);
        }
        const E* vrow = Vs + (t * 32 + col) * LDV + hf * M::KPL;
#pragma unroll
        for (int s = 0; s < KS_V; ++s) {
          dp[t] = M::mma(lds_frag<M>(vrow + s * M::K), of[s], dp[t]);
          if constexpr (SPLIT == 2) dp[t] = M::mma(lds_frag<M>(vrow + BN * LDV + s * M::K), of[s], dp[t]);
        }
      }
      const bool diag = key0 + BN - 1 > qw;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t u = key0 + t * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
          float p = exp2f(sc[t][r] * a.scale_log2 - lse2);
          if ((diag && u > tq) || u >= a.S) p = 0.f;
          dp[t][r] = p * (dp[t][r] - dl);
        }
      // dq^T[d, q] += K^T dS^T  (k = keys, permuted)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
          E dh[M::KPL];
#pragma unroll
          for (int j = 0; j < M::KPL; ++j) dh[j] = M::from_f32(dp[t][st * M::KPL + j]);
          const F df = *reinterpret_cast<F*>(dh);
          const int r0 = st * M::KPL;
          const int kc = acc_key_col(t * 32 + 8 * (r0 / 4) + 4 * hf + (r0 % 4));
#pragma unroll
          for (int n = 0; n < NQT; ++n) dq[n] = M::mma(lds_frag<M>(Kt + (n * 32 + col) * LDT + kc), df, dq[n]);
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

template <class InT, class KvT, class M, int SPLIT, int DN, int DR, int DV>
__global__ __launch_bounds__(kThreads) void dkdv_kernel(BwdArgs a) {
  typedef DkdvKernel<InT, KvT, M, SPLIT, DN, DR, DV> Kn;
  __shared__ __attribute__((aligned(16))) typename M::elem lds[Kn::LDS_ELEMS];
  __shared__ float stat[2 * Kn::BQ];
  Kn::run(a, lds, stat);
}

template <class InT, class KvT, class M, int SPLIT, int DN, int DR, int DV>
__global__ __launch_bounds__(kThreads) void dq_kernel(BwdArgs a) {
  typedef DqKernel<InT, KvT, M, SPLIT, DN, DR, DV> Kn;
  __shared__ __attribute__((aligned(16))) typename M::elem lds[Kn::LDS_ELEMS];
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
  a.scale = 1.0f / sqrtf(static_cast<float>(s.d_qk()));
  a.scale_log2 = 1.4426950408889634f * a.scale;
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
                                const float* lse, const float* delta, const void* d_o, float* dkv,
                                float* dk_pe_part, hipStream_t st) {
  BwdArgs a = make_args(s, q, kn, kp, v, lse, delta, d_o);
  a.dkv = dkv;
  a.dk_pe_part = dk_pe_part;
  const unsigned grid = static_cast<unsigned>(((s.S + 127) / 128) * s.B * s.h);
  if (s.bf16 && s.split && s.d_nope == 128 && s.d_rope == 64 && s.d_v == 128)
    hipLaunchKernelGGL((dkdv_kernel<bf16_t, half_t, MmaF16, 2, 128, 64, 128>), dim3(grid), dim3(kThreads), 0, st, a);
  else if (!s.bf16 && s.d_nope == 32 && s.d_rope == 16 && s.d_v == 32)
    hipLaunchKernelGGL((dkdv_kernel<float, float, MmaF32, 1, 32, 16, 32>), dim3(grid), dim3(kThreads), 0, st, a);
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
    hipLaunchKernelGGL((dq_kernel<bf16_t, half_t, MmaF16, 2, 128, 64, 128>), dim3(grid), dim3(kThreads), 0, st, a);
  else if (!s.bf16 && s.d_nope == 32 && s.d_rope == 16 && s.d_v == 32)
    hipLaunchKernelGGL((dq_kernel<float, float, MmaF32, 1, 32, 16, 32>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    return hipErrorNotSupported;
  return hipGetLastError();
}

}  // namespace laga
