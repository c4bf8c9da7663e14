// Causal attention forward of one rank's head shard.
//
// [LAGA §3.3 Algorithm 1 scores / softmax / output; §5.3 shared k_pe band]
//   s[t,u] = (q_nope || q_rope)[t,i] . (k_nope[u,i] || k_pe[u]) / sqrt(d_nope + d_rope), u <= t
//   o[t,i] = sum_u softmax_u(s) v[u,i],   lse[i,t] = ln sum_u exp(s[t,u])
//
// Flash-style: one 256-thread workgroup owns BM = 128 queries of one head and
// streams the keys 0 .. (last query of the tile) in blocks of BN = 64 through
// LDS, with an online softmax, so no S x S score matrix ever exists.  Each
// wavefront owns 32 queries and keeps them in registers as the B operand of
//     S^T[key, query] = K . Q^T          (A = K rows from LDS)
// so that the 32x32 accumulator layout puts one query per lane column: the row
// statistics (running max, running sum) are lane-local up to one exchange with
// the other half of the wavefront, and the probabilities already sit in the
// layout of the B operand of
//     O^T[dv, query] += V^T . P^T        (A = V^T from LDS, key-permuted)
// The k_pe band is staged once per key block and serves every query of the
// tile; it is never expanded per head.  Blocks that lie entirely above a
// wavefront's diagonal are skipped; only blocks crossing it are masked.
//
// Precision: SPLIT == 1 feeds fp16 operands (bf16 q / k_pe convert exactly);
// SPLIT == 2 stores K/V as float32 and feeds K, V and P as fp16 hi + lo pairs
// (S = Q.K_hi + Q.K_lo, O = P_hi V_hi + P_hi V_lo + P_lo V_hi), fp32-class.
// The float32 instantiation uses fp32 MFMAs throughout.
#include "device.hpp"
#include "launch.hpp"

namespace laga {
namespace {

constexpr int BM = 128;  // queries per workgroup (4 wavefronts x 32)
constexpr int BN = 64;   // keys per block
constexpr int kThreads = 256;

template <class M> struct AttnPad { static constexpr int v = 8; };
template <> struct AttnPad<MmaF32> { static constexpr int v = 1; };

struct FwdArgs {
  const void* q; const void* k_nope; const void* k_pe; const void* v;
  float* o; float* lse;
  int64_t S; int B, h, n_qt; float scale_log2;
};

template <class InT, class KvT, class M, int SPLIT, int DN, int DR, int DV>
struct FwdKernel {
  typedef typename M::elem E;
  static constexpr int DQK = DN + DR;
  static constexpr int PAD = AttnPad<M>::v;
  static constexpr int LDK = DQK + PAD;   // hi plane: nope + rope
  static constexpr int LDKL = DN + PAD;   // lo plane: nope only
  static constexpr int LDV = BN + PAD;    // V^T rows (one per dv)
  static constexpr int NT = BN / 32;      // S^T atoms per wavefront per block
  static constexpr int NO = DV / 32;      // O^T atoms
  static constexpr int KS_QK = DQK / M::K;
  static constexpr int KS_NOPE = DN / M::K;
  static constexpr int PV_STEPS = 32 / M::K;  // MFMA steps per 32-key atom
  static constexpr int LDS_K = BN * LDK;
  static constexpr int LDS_KL = (SPLIT == 2) ? BN * LDKL : 0;
  static constexpr int LDS_V = SPLIT * DV * LDV;
  static constexpr int LDS_ELEMS = LDS_K + LDS_KL + LDS_V;

  // Staging of one key block: global -> registers (prefetch) -> LDS.
  static constexpr int KVEC = 16 / sizeof(KvT);                 // KvT per 16-byte load
  static constexpr int PVEC = 16 / sizeof(InT);                 // k_pe per 16-byte load
  static constexpr int K_ITEMS = BN * DN / KVEC;
  static constexpr int P_ITEMS = BN * DR / PVEC;
  static constexpr int V_ITEMS = (BN / 4) * (DV / KVEC);        // 4 keys x KVEC dv each
  static constexpr int K_PER = (K_ITEMS + kThreads - 1) / kThreads;
  static constexpr int P_PER = (P_ITEMS + kThreads - 1) / kThreads;
  static constexpr int V_PER = (V_ITEMS + kThreads - 1) / kThreads;
  typedef KvT kvec __attribute__((ext_vector_type(KVEC)));
  typedef InT pvec __attribute__((ext_vector_type(PVEC)));

  struct Regs {
    kvec k[K_PER];
    pvec p[P_PER];
    kvec v[V_PER][4];
  };

  __device__ static void load_block(const FwdArgs& a, int b, int head, int64_t key0, Regs& R) {
    const KvT* kn = static_cast<const KvT*>(a.k_nope);
    const InT* kp = static_cast<const InT*>(a.k_pe);
    const KvT* vv = static_cast<const KvT*>(a.v);
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < K_PER; ++j) {
      const int it = j * kThreads + tid;
      const int key = it / (DN / KVEC), c = (it % (DN / KVEC)) * KVEC;
      const int64_t u = key0 + key;
      if (it < K_ITEMS && u < a.S)
        R.k[j] = *reinterpret_cast<const kvec*>(kn + ((b * a.S + u) * a.h + head) * DN + c);
      else
        R.k[j] = kvec{};
    }
#pragma unroll
    for (int j = 0; j < P_PER; ++j) {
      const int it = j * kThreads + tid;
      const int key = it / (DR / PVEC), c = (it % (DR / PVEC)) * PVEC;
      const int64_t u = key0 + key;
      if (it < P_ITEMS && u < a.S)
        R.p[j] = *reinterpret_cast<const pvec*>(kp + (b * a.S + u) * DR + c);
      else
        R.p[j] = pvec{};
    }
#pragma unroll
    for (int j = 0; j < V_PER; ++j) {
      const int it = j * kThreads + tid;
      const int kg = it / (DV / KVEC), c = (it % (DV / KVEC)) * KVEC;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t u = key0 + kg * 4 + r;
        if (it < V_ITEMS && u < a.S)
          R.v[j][r] = *reinterpret_cast<const kvec*>(vv + ((b * a.S + u) * a.h + head) * DV + c);
        else
          R.v[j][r] = kvec{};
      }
    }
  }

  __device__ static void store_block(const Regs& R, E* lds) {
    E* Ks = lds;
    E* Kl = lds + LDS_K;
    E* Vt = lds + LDS_K + LDS_KL;
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < K_PER; ++j) {
      const int it = j * kThreads + tid;
      if (it >= K_ITEMS) continue;
      const int key = it / (DN / KVEC), c = (it % (DN / KVEC)) * KVEC;
#pragma unroll
      for (int e = 0; e < KVEC; ++e) {
        E part[SPLIT];
        split_to<M, SPLIT>(to_f32(R.k[j][e]), part);
        Ks[key * LDK + c + e] = part[0];
        if constexpr (SPLIT == 2) Kl[key * LDKL + c + e] = part[1];
      }
    }
#pragma unroll
    for (int j = 0; j < P_PER; ++j) {
      const int it = j * kThreads + tid;
      if (it >= P_ITEMS) continue;
      const int key = it / (DR / PVEC), c = (it % (DR / PVEC)) * PVEC;
#pragma unroll
      for (int e = 0; e < PVEC; ++e) Ks[key * LDK + DN + c + e] = M::from_f32(to_f32(R.p[j][e]));
    }
#pragma unroll
    for (int j = 0; j < V_PER; ++j) {
      const int it = j * kThreads + tid;
      if (it >= V_ITEMS) continue;
      const int kg = it / (DV / KVEC), c = (it % (DV / KVEC)) * KVEC;
      const int col = acc_key_col(kg * 4);  // 4 consecutive keys stay contiguous
#pragma unroll
      for (int e = 0; e < KVEC; ++e) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          E part[SPLIT];
          split_to<M, SPLIT>(to_f32(R.v[j][r][e]), part);
#pragma unroll
          for (int s = 0; s < SPLIT; ++s) Vt[s * DV * LDV + (c + e) * LDV + col + r] = part[s];
        }
      }
    }
  }

  __device__ static void run(const FwdArgs& a, E* lds) {
    const int lane = threadIdx.x % kWave;
    const int wv = threadIdx.x / kWave;
    const int hf = lane / 32;
    const int col = lane % 32;

    // Workgroup -> (batch*head, query tile).  Heads are grouped per XCD
    // (workgroup ids are dealt round-robin to the 8 XCDs) so that the
    // workgroups sharing a head's K/V stream share one L2; within an XCD the
    // longest (latest) query tiles go first.
    const int nbh = a.B * a.h;
    int bh, qt_rank;
    if (nbh % 8 == 0) {
      const int xcd = blockIdx.x % 8, j = blockIdx.x / 8, hpx = nbh / 8;
      bh = xcd * hpx + j % hpx;
      qt_rank = j / hpx;
    } else {
      bh = blockIdx.x % nbh;
      qt_rank = blockIdx.x / nbh;
    }
    const int qt = a.n_qt - 1 - qt_rank;
    const int b = bh / a.h, head = bh % a.h;
    const int64_t q0 = static_cast<int64_t>(qt) * BM;
    const int64_t qw = q0 + wv * 32;       // first query of this wavefront
    const int64_t tq = qw + col;           // this lane's query

    // Q fragments (B operand): query tq, dims hf*KPL + s*K + [0, KPL).
    const InT* qp = static_cast<const InT*>(a.q);
    typename M::frag qf[KS_QK];
#pragma unroll
    for (int s = 0; s < KS_QK; ++s) {
      E tmp[M::KPL];
#pragma unroll
      for (int j = 0; j < M::KPL; ++j)
        tmp[j] = M::from_f32(tq < a.S ? to_f32(qp[((b * a.S + tq) * a.h + head) * DQK + s * M::K + hf * M::KPL + j]) : 0.f);
      qf[s] = *reinterpret_cast<typename M::frag*>(tmp);
    }

    f32x16 o[NO];
#pragma unroll
    for (int n = 0; n < NO; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[n][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    int64_t kend = q0 + BM;
    if (kend > a.S) kend = a.S;
    const int nkb = static_cast<int>((kend + BN - 1) / BN);

    Regs R;
    load_block(a, b, head, 0, R);
    for (int kb = 0; kb < nkb; ++kb) {
      const int64_t key0 = static_cast<int64_t>(kb) * BN;
      __syncthreads();
      store_block(R, lds);
      __syncthreads();
      if (kb + 1 < nkb) load_block(a, b, head, key0 + BN, R);
      if (key0 > qw + 31) continue;  // whole block above this wavefront's diagonal

      const E* Ks = lds;
      const E* Kl = lds + LDS_K;
      const E* Vt = lds + LDS_K + LDS_KL;

      f32x16 sc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[t][r] = 0.f;
        const E* krow = Ks + (t * 32 + col) * LDK + hf * M::KPL;
#pragma unroll
        for (int s = 0; s < KS_QK; ++s) sc[t] = M::mma(lds_frag<M>(krow + s * M::K), qf[s], sc[t]);
        if constexpr (SPLIT == 2) {
          const E* lrow = Kl + (t * 32 + col) * LDKL + hf * M::KPL;
#pragma unroll
          for (int s = 0; s < KS_NOPE; ++s) sc[t] = M::mma(lds_frag<M>(lrow + s * M::K), qf[s], sc[t]);
        }
      }

      // Scale into the log2 domain and mask keys past this lane's query.
      const bool diag = key0 + BN - 1 > qw;
      float mloc = -INFINITY;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sc[t][r] * a.scale_log2;
          if (diag) {
            const int64_t u = key0 + t * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
            if (u > tq) x = -INFINITY;
          }
          sc[t][r] = x;
          mloc = fmaxf(mloc, x);
        }
      mloc = fmaxf(mloc, swap_halves(mloc));
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = exp2f(m_run - m_new);
      float lsum = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(sc[t][r] - m_new);
          sc[t][r] = p;
          lsum += p;
        }
      lsum += swap_halves(lsum);
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int n = 0; n < NO; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[n][r] *= alpha;

      // O^T += V^T P^T, one step covers K keys; accumulator r = step*KPL + j.
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int st = 0; st < PV_STEPS; ++st) {
          E ph[M::KPL], pl[M::KPL];
#pragma unroll
          for (int j = 0; j < M::KPL; ++j) {
            E part[SPLIT];
            split_to<M, SPLIT>(sc[t][st * M::KPL + j], part);
            ph[j] = part[0];
            if constexpr (SPLIT == 2) pl[j] = part[1];
          }
          const typename M::frag pfh = *reinterpret_cast<typename M::frag*>(ph);
          const int r0 = st * M::KPL;
          const int kcol = acc_key_col(t * 32 + 8 * (r0 / 4) + 4 * hf + (r0 % 4));
#pragma unroll
          for (int n = 0; n < NO; ++n) {
            const E* vrow = Vt + (n * 32 + col) * LDV + kcol;
            o[n] = M::mma(lds_frag<M>(vrow), pfh, o[n]);
            if constexpr (SPLIT == 2) {
              const typename M::frag pfl = *reinterpret_cast<typename M::frag*>(pl);
              o[n] = M::mma(lds_frag<M>(vrow + DV * LDV), pfh, o[n]);
              o[n] = M::mma(lds_frag<M>(vrow), pfl, o[n]);
            }
          }
        }
    }

    if (tq < a.S) {
      const float inv = 1.0f / l_run;
      float* op = a.o + ((b * a.S + tq) * a.h + head) * DV;
#pragma unroll
      for (int n = 0; n < NO; ++n)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 w = {o[n][4 * g] * inv, o[n][4 * g + 1] * inv, o[n][4 * g + 2] * inv, o[n][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(op + n * 32 + 8 * g + 4 * hf) = w;
        }
      if (hf == 0) a.lse[(static_cast<int64_t>(b) * a.h + head) * a.S + tq] = (m_run + log2f(l_run)) * 0.69314718055994531f;
    }
  }
};

template <class InT, class KvT, class M, int SPLIT, int DN, int DR, int DV>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(FwdArgs a) {
  typedef FwdKernel<InT, KvT, M, SPLIT, DN, DR, DV> Kn;
  __shared__ __attribute__((aligned(16))) typename M::elem lds[Kn::LDS_ELEMS];
  Kn::run(a, lds);
}

template <class InT, class KvT, class M, int SPLIT, int DN, int DR, int DV>
hipError_t fwd_t(const Shape& s, const void* q, const void* kn, const void* kp, const void* v, float* o,
                 float* lse, hipStream_t st) {
  FwdArgs a;
  a.q = q; a.k_nope = kn; a.k_pe = kp; a.v = v; a.o = o; a.lse = lse;
  a.S = s.S; a.B = static_cast<int>(s.B); a.h = s.h;
  a.n_qt = static_cast<int>((s.S + BM - 1) / BM);
  a.scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(DN + DR));
  const int64_t grid = static_cast<int64_t>(a.n_qt) * s.B * s.h;
  hipLaunchKernelGGL((attn_fwd_kernel<InT, KvT, M, SPLIT, DN, DR, DV>), dim3(static_cast<unsigned>(grid)),
                     dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const Shape& s, const void* q, const void* kn, const void* kp, const void* v,
                           float* o, float* lse, hipStream_t st) {
  if (s.bf16 && s.d_nope == 128 && s.d_rope == 64 && s.d_v == 128) {
    if (s.split) return fwd_t<bf16_t, float, MmaF16, 2, 128, 64, 128>(s, q, kn, kp, v, o, lse, st);
    return fwd_t<bf16_t, half_t, MmaF16, 1, 128, 64, 128>(s, q, kn, kp, v, o, lse, st);
  }
  if (!s.bf16 && s.d_nope == 32 && s.d_rope == 16 && s.d_v == 32)
    return fwd_t<float, float, MmaF32, 1, 32, 16, 32>(s, q, kn, kp, v, o, lse, st);
  return hipErrorInvalidValue;
}

}  // namespace laga
