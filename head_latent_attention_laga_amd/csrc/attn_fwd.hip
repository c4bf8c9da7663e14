// Causal attention forward of one rank's head shard.
//
// [LAGA §3.3 Algorithm 1 scores / softmax / output; §5.3 shared k_pe band]
//   s[t,u] = (q_nope || q_rope)[t,i] . (k_nope[u,i] || k_pe[u]) / sqrt(d_nope + d_rope), u <= t
//   o[t,i] = sum_u softmax_u(s) v[u,i],   lse[i,t] = ln sum_u exp(s[t,u])
//
// Flash-style: a workgroup of NW wavefronts owns BM = 32*NW queries of one
// head and streams keys 0 .. (last query of the tile) in blocks of BN = 64
// through double-buffered LDS (the next block's global loads are in flight in
// registers while the current one is computed), with an online softmax, so no
// S x S matrix ever exists.  Each wavefront keeps its 32 queries in registers
// as the B operand of
//     S^T[key, query] = K . Q^T          (A = K rows, 16-byte LDS reads)
// so that the 32x32 accumulators hold one query per lane column: the running
// max / sum are lane-local up to one exchange between wavefront halves, and
// the probabilities already sit in the B-operand layout of
//     O^T[dv, query] += V^T . P^T        (A = V^T via transposing LDS reads)
// K, k_pe and V are staged as plain 16-byte copies in their storage layout:
// the rope band stays bf16 and meets q_rope in bf16 MFMAs (both exact), the
// nope part meets q_nope (converted once to fp16, exactly) in fp16 MFMAs.
// The k_pe band is staged once per key block for all queries of the tile and
// never expanded per head.  Blocks above a wavefront's diagonal are skipped;
// only blocks crossing it are masked.
//
// Precision: NS == 1 uses single fp16 K, V and P.  NS == 2 reads K and V as
// fp16 hi/lo planes (as laga_kv_up writes them) and splits P:
// S = Q.K_hi + Q.K_lo, O = P_hi V_hi + P_hi V_lo + P_lo V_hi (fp32-class).
// The float32 instantiation uses fp32 MFMAs throughout.
#include "attn_common.hpp"
#include "launch.hpp"

namespace laga {
namespace {

constexpr int BN = 64;  // keys per block

struct FwdArgs {
  const void* q; const void* k_nope; const void* k_pe; const void* v;
  float* o; float* lse;
  int64_t S, plane_k, plane_v; int B, h, n_qt; float scale_log2;
};

template <class M> struct Pads { static constexpr int k = 8, r = 8, v = 16; };
template <> struct Pads<MmaF32> { static constexpr int k = 4, r = 4, v = 4; };

// M: K/V/P operand type (fp16 or fp32); MR: rope operand type (bf16 or fp32);
// InT: storage type of q and k_pe.
template <class InT, class M, class MR, int NS, int DN, int DR, int DV, int NW>
struct Fwd {
  typedef typename M::elem E;
  typedef typename MR::elem ER;
  typedef typename M::frag F;
  typedef typename MR::frag FR;
  static constexpr int NT = NW * kWave;
  static constexpr int BM = 32 * NW;
  static constexpr int LDK = DN + Pads<M>::k, LDR = DR + Pads<M>::r, LDV = DV + Pads<M>::v;
  // LDS buffer: NS K planes | rope band | NS V planes (element offsets of E; rope in ER).
  static constexpr int K_ELEMS = NS * BN * LDK;
  static constexpr int R_BYTES = BN * LDR * sizeof(ER);
  static constexpr int V_ELEMS = NS * BN * LDV;
  static constexpr int BUF_BYTES = (K_ELEMS + V_ELEMS) * sizeof(E) + R_BYTES;
  static constexpr int LDS_BYTES = 2 * BUF_BYTES;
  // 16-byte chunks per block.
  static constexpr int EPC = 16 / sizeof(E), RPC = 16 / sizeof(ER);
  static constexpr int K_CH = NS * BN * DN / EPC, R_CH = BN * DR / RPC, V_CH = NS * BN * DV / EPC;
  static constexpr int ALL_CH = K_CH + R_CH + V_CH;
  static constexpr int CH = (ALL_CH + NT - 1) / NT;
  static constexpr int KS_N = DN / M::K, KS_R = DR / MR::K, NO = DV / 32, PV_STEPS = 32 / M::K;
  static_assert(DN % M::K == 0 && DR % MR::K == 0 && DV % 32 == 0, "head dims");

  struct Regs { u32x4 c[CH]; };

  __device__ static void load_block(const FwdArgs& a, int b, int head, int64_t key0, Regs& R) {
    const E* kn = static_cast<const E*>(a.k_nope);
    const ER* kp = static_cast<const ER*>(a.k_pe);
    const E* vg = static_cast<const E*>(a.v);
    const int nk = static_cast<int>(a.S - key0 < BN ? a.S - key0 : BN);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      int c = i * NT + static_cast<int>(threadIdx.x);
      u32x4 val{0u, 0u, 0u, 0u};
      if (c < K_CH) {
        const int p = c / (BN * DN / EPC), rem = c % (BN * DN / EPC);
        const int r = rem / (DN / EPC), j = rem % (DN / EPC);
        val = load_chunk(kn + p * a.plane_k + ((b * a.S + key0) * a.h + head) * DN, int64_t(a.h) * DN, r, j * EPC, nk);
      } else if (c < K_CH + R_CH) {
        c -= K_CH;
        const int r = c / (DR / RPC), j = c % (DR / RPC);
        val = load_chunk(kp + (b * a.S + key0) * DR, DR, r, j * RPC, nk);
      } else if (c < ALL_CH) {
        c -= K_CH + R_CH;
        const int p = c / (BN * DV / EPC), rem = c % (BN * DV / EPC);
        const int r = rem / (DV / EPC), j = rem % (DV / EPC);
        val = load_chunk(vg + p * a.plane_v + ((b * a.S + key0) * a.h + head) * DV, int64_t(a.h) * DV, r, j * EPC, nk);
      }
      R.c[i] = val;
    }
  }

  __device__ static void store_block(const Regs& R, char* buf) {
    E* Ks = reinterpret_cast<E*>(buf);
    ER* Kr = reinterpret_cast<ER*>(buf + K_ELEMS * sizeof(E));
    E* Vs = reinterpret_cast<E*>(buf + K_ELEMS * sizeof(E) + R_BYTES);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      int c = i * NT + static_cast<int>(threadIdx.x);
      if (c < K_CH) {
        const int p = c / (BN * DN / EPC), rem = c % (BN * DN / EPC);
        store_chunk(Ks + p * BN * LDK, LDK, rem / (DN / EPC), (rem % (DN / EPC)) * EPC, R.c[i]);
      } else if (c < K_CH + R_CH) {
        c -= K_CH;
        store_chunk(Kr, LDR, c / (DR / RPC), (c % (DR / RPC)) * RPC, R.c[i]);
      } else if (c < ALL_CH) {
        c -= K_CH + R_CH;
        const int p = c / (BN * DV / EPC), rem = c % (BN * DV / EPC);
        store_chunk(Vs + p * BN * LDV, LDV, rem / (DV / EPC), (rem % (DV / EPC)) * EPC, R.c[i]);
      }
    }
  }

  // A operand of O^T += V^T P^T for one MFMA step: rows dv n0 + lane%32, keys of
  // accumulator registers st*KPL .. of 32-key atom t (see acc_key_col).
  __device__ static F v_frag(const E* Vp, int t, int st, int n0) {
    if constexpr (M::KPL == 8) {
      return tr_frag_acc(Vp, LDV, t * 32 + st * 16, n0);
    } else {
      const int lane = threadIdx.x % kWave;
      const int key = t * 32 + 8 * (st / 4) + 4 * (lane / 32) + (st % 4);
      return Vp[key * LDV + n0 + lane % 32];
    }
  }

  __device__ static void run(const FwdArgs& a, char* lds) {
    const int lane = threadIdx.x % kWave;
    const int wv = threadIdx.x / kWave;
    const int hf = lane / 32;
    const int col = lane % 32;

    // Workgroup -> (batch*head, query tile).  Workgroup ids are dealt
    // round-robin to the 8 XCDs; heads are grouped per XCD so the workgroups
    // streaming one head's K/V share an L2, and within an XCD the longest
    // (latest) query tiles start first.
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
    const int64_t qw = q0 + wv * 32;
    const int64_t tq = qw + col;
    const bool qvalid = tq < a.S;

    // Q fragments (B operand): query tq, dims hf*KPL + s*K + [0, KPL).
    const InT* qp = static_cast<const InT*>(a.q) + ((b * a.S + (qvalid ? tq : 0)) * a.h + head) * (DN + DR);
    F qn[KS_N];
    FR qr[KS_R];
#pragma unroll
    for (int s = 0; s < KS_N; ++s) {
      E tmp[M::KPL];
#pragma unroll
      for (int j = 0; j < M::KPL; ++j) tmp[j] = M::from_f32(qvalid ? to_f32(qp[s * M::K + hf * M::KPL + j]) : 0.f);
      qn[s] = *reinterpret_cast<F*>(tmp);
    }
#pragma unroll
    for (int s = 0; s < KS_R; ++s) {
      ER tmp[MR::KPL];
#pragma unroll
      for (int j = 0; j < MR::KPL; ++j) tmp[j] = qvalid ? qp[DN + s * MR::K + hf * MR::KPL + j] : ER{};
      qr[s] = *reinterpret_cast<FR*>(tmp);
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
      char* buf = lds + (kb & 1) * BUF_BYTES;
      store_block(R, buf);
      __syncthreads();
      if (kb + 1 < nkb) load_block(a, b, head, key0 + BN, R);
      if (key0 > qw + 31) continue;  // whole block above this wavefront's diagonal

      const E* Ks = reinterpret_cast<const E*>(buf);
      const ER* Kr = reinterpret_cast<const ER*>(buf + K_ELEMS * sizeof(E));
      const E* Vs = reinterpret_cast<const E*>(buf + K_ELEMS * sizeof(E) + R_BYTES);

      f32x16 sc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[t][r] = 0.f;
        const int krow = t * 32 + col;
#pragma unroll
        for (int s = 0; s < KS_N; ++s) {
          sc[t] = M::mma(lds_frag<M>(Ks + krow * LDK + s * M::K + hf * M::KPL), qn[s], sc[t]);
          if constexpr (NS == 2)
            sc[t] = M::mma(lds_frag<M>(Ks + BN * LDK + krow * LDK + s * M::K + hf * M::KPL), qn[s], sc[t]);
        }
#pragma unroll
        for (int s = 0; s < KS_R; ++s)
          sc[t] = MR::mma(lds_frag<MR>(Kr + krow * LDR + s * MR::K + hf * MR::KPL), qr[s], sc[t]);
      }

      // Row max of the raw scores (scale > 0 is folded into the exponent).
      const bool diag = key0 + BN - 1 > qw;
      float mloc = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (diag) {
            const int64_t u = key0 + t * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
            if (u > tq) sc[t][r] = -INFINITY;
          }
          mloc = fmaxf(mloc, sc[t][r]);
        }
      mloc = fmaxf(mloc, swap_halves(mloc));
      const float m_new = fmaxf(m_run, mloc * a.scale_log2);
      float lsum = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(fmaf(sc[t][r], a.scale_log2, -m_new));
          sc[t][r] = p;
          lsum += p;
        }
      lsum += swap_halves(lsum);
      if (__any(m_new != m_run)) {
        const float alpha = exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int n = 0; n < NO; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[n][r] *= alpha;
      }
      l_run += lsum;
      m_run = m_new;

      // O^T += V^T P^T; one step covers K keys, accumulator r = st*KPL + j.
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int st = 0; st < PV_STEPS; ++st) {
          E ph[M::KPL], pl[M::KPL];
#pragma unroll
          for (int j = 0; j < M::KPL; ++j) {
            E part[NS];
            split_to<M, NS>(sc[t][st * M::KPL + j], part);
            ph[j] = part[0];
            if constexpr (NS == 2) pl[j] = part[1];
          }
          const F pfh = *reinterpret_cast<F*>(ph);
#pragma unroll
          for (int n = 0; n < NO; ++n) {
            const F vh = v_frag(Vs, t, st, n * 32);
            o[n] = M::mma(vh, pfh, o[n]);
            if constexpr (NS == 2) {
              const F pfl = *reinterpret_cast<F*>(pl);
              o[n] = M::mma(v_frag(Vs + BN * LDV, t, st, n * 32), pfh, o[n]);
              o[n] = M::mma(vh, pfl, o[n]);
            }
          }
        }
    }

    if (qvalid) {
      const float inv = 1.0f / l_run;
      float* op = a.o + ((b * a.S + tq) * a.h + head) * DV;
#pragma unroll
      for (int n = 0; n < NO; ++n)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 w = {o[n][4 * g] * inv, o[n][4 * g + 1] * inv, o[n][4 * g + 2] * inv, o[n][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(op + n * 32 + 8 * g + 4 * hf) = w;
        }
      if (hf == 0)
        a.lse[(static_cast<int64_t>(b) * a.h + head) * a.S + tq] = (m_run + log2f(l_run)) * 0.69314718055994531f;
    }
  }
};

template <class InT, class M, class MR, int NS, int DN, int DR, int DV, int NW>
__global__ __launch_bounds__(NW * kWave) void attn_fwd_kernel(FwdArgs a) {
  typedef Fwd<InT, M, MR, NS, DN, DR, DV, NW> Kn;
  __shared__ __attribute__((aligned(16))) char lds[Kn::LDS_BYTES];
  Kn::run(a, lds);
}

template <class InT, class M, class MR, int NS, int DN, int DR, int DV, int NW>
hipError_t fwd_t(const Shape& s, const void* q, const void* kn, const void* kp, const void* v, float* o,
                 float* lse, hipStream_t st) {
  typedef Fwd<InT, M, MR, NS, DN, DR, DV, NW> Kn;
  FwdArgs a;
  a.q = q; a.k_nope = kn; a.k_pe = kp; a.v = v; a.o = o; a.lse = lse;
  a.S = s.S; a.B = static_cast<int>(s.B); a.h = s.h;
  a.plane_k = s.T * s.h * DN;
  a.plane_v = s.T * s.h * DV;
  a.n_qt = static_cast<int>((s.S + Kn::BM - 1) / Kn::BM);
  a.scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(DN + DR));
  const int64_t grid = static_cast<int64_t>(a.n_qt) * s.B * s.h;
  hipLaunchKernelGGL((attn_fwd_kernel<InT, M, MR, NS, DN, DR, DV, NW>), dim3(static_cast<unsigned>(grid)),
                     dim3(Kn::NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const Shape& s, const void* q, const void* kn, const void* kp, const void* v,
                           float* o, float* lse, hipStream_t st) {
  if (s.bf16 && s.d_nope == 128 && s.d_rope == 64 && s.d_v == 128) {
    if (s.split) return fwd_t<bf16_t, MmaF16, MmaBf16, 2, 128, 64, 128, 8>(s, q, kn, kp, v, o, lse, st);
    return fwd_t<bf16_t, MmaF16, MmaBf16, 1, 128, 64, 128, 8>(s, q, kn, kp, v, o, lse, st);
  }
  if (!s.bf16 && s.d_nope == 32 && s.d_rope == 16 && s.d_v == 32)
    return fwd_t<float, MmaF32, MmaF32, 1, 32, 16, 32, 4>(s, q, kn, kp, v, o, lse, st);
  return hipErrorInvalidValue;
}

}  // namespace laga
