// dq of the causal attention backward of one rank's head shard [LAGA §5.2],
// recomputing the probabilities and score gradients from the forward's lse
// and the row sums delta, so that no S x S quantity ever reaches memory:
//   P = exp(s - lse),  dP = dO . V^T,  dS = P * (dP - delta),
//   dq = dS . K / sqrt(d_qk)              (K = k_nope || k_pe)
//
// Layout of the work (the forward kernel's, attn_fwd.hip): a workgroup of NW
// wavefronts owns 32*QH*NW queries of one head and streams the keys 0 .. its
// last query in blocks of 32 through double-buffered LDS (the next block's
// 16-byte buffer loads in flight in registers while the current one is
// computed).  Each wavefront holds the q rows of its QH groups of 32 queries
// in registers and their dO rows in a private LDS area (registers cannot hold
// both next to the dq accumulators) as the B operands of
//     S^T[key, query]  = K . q^T           (A = K rows, 16-byte LDS reads)
//     dP^T[key, query] = V . dO^T          (A = V rows, 16-byte LDS reads)
// so the accumulators hold one query per lane column: lse and delta are
// lane-local, and P and dS = P (dP - delta) already sit in the B-operand
// layout of
//     dq^T[d, query] += K^T . dS^T         (A = K^T, transposing LDS reads)
// With QH = 2 (one wavefront per
// SIMD, 64 queries each) every K / V operand read from LDS feeds two
// products, and the two query groups are independent chains of products and
// vector work that the wavefront interleaves; the state of two wavefronts
// per SIMD with 32 queries each does not fit the register file.  Blocks above
// a wavefront's diagonal are skipped; only blocks crossing it are masked.  K
// is staged twice per block: rows padded for conflict-free 16-byte reads, and
// rows of a 448-byte pitch, which puts the four rows of each transposing read
// in four different 64-byte bank windows.
//
// Precision: single fp16 operands (q, K's hi plane and k_pe exact or nearly;
// V's hi plane; dO scaled by 2^g into fp16's normal range by the prep pass;
// dS rounded once), fp32 accumulation: dq's error budget allows it, unlike
// the dK / dV products, which feed reductions over every token.  The float32
// instantiation uses fp32 MFMAs throughout.
#include "attn_bwd_common.hpp"

namespace laga {
namespace {
using namespace bwd;

template <class M, int DN, int DR, int DV, int NW, int QH>
struct Dq {
  typedef typename M::elem E;
  typedef typename M::frag F;
  static constexpr int DQK = DN + DR;
  static constexpr int NT = NW * kWave, WQ = 32 * QH, BM = WQ * NW, BN = 32;
  static constexpr bool TR = M::KPL == 8;  // 16-bit operands: K^T from transposing reads
  static constexpr int NQT = (DQK + 31) / 32;   // dq^T atoms (the last may run past d_qk)
  static constexpr int KS_QK = DQK / M::K, KS_V = DV / M::K, STEPS = 32 / M::K;
  // LDS pitches (elements).  Row-read tiles: 4 (mod 8) dwords, so the 16 rows
  // a 16-byte read serves at once start in 16 distinct 4-bank groups.  The
  // transposed-read K copy: 448 bytes.  fp32: one K tile wide enough for the
  // last atom's rows past d_qk (their values only reach rows of dq^T that
  // are never stored).
  static constexpr int LKR = TR ? DQK + 8 : NQT * 32 + 4;
  static constexpr int LKT = DQK + 32;
  static constexpr int LV = DV + (TR ? 8 : 4);
  static constexpr int LDO = DV + (TR ? 8 : 4);  // the wavefront's dO rows (16-byte row reads)
  static_assert(BN == 32, "one 32x32 atom of keys per block");
  static_assert(!TR || ((LKR * 2 / 4) % 8 == 4 && (LV * 2 / 4) % 8 == 4 && (LKT * 2) % 256 == 192),
                "bank-conflict-free pitches");
  static constexpr int KR_BYTES = BN * LKR * sizeof(E);
  static constexpr int KT_BYTES = TR ? BN * LKT * sizeof(E) : 0;
  static constexpr int V_BYTES = BN * LV * sizeof(E);
  static constexpr int OFF_KT = KR_BYTES, OFF_V = OFF_KT + KT_BYTES;
  static constexpr int BUF_BYTES = OFF_V + V_BYTES;
  static constexpr int DO_BYTES = WQ * LDO * sizeof(E);  // per wavefront
  static constexpr int OFF_DO = 2 * BUF_BYTES;
  static constexpr int LDS_BYTES = OFF_DO + NW * DO_BYTES;
  // Staging: 16-byte chunks of the K nope plane, the k_pe band and V.
  static constexpr int EPC = 16 / sizeof(E);
  static constexpr int CK = DN / EPC, CR = DR / EPC, CV = DV / EPC;
  static constexpr int IK = (BN * CK + NT - 1) / NT, IR = (BN * CR + NT - 1) / NT, IV = (BN * CV + NT - 1) / NT;
  static constexpr int kAhead = 2;  // operand reads in flight ahead of the products

  struct Regs { u32x4 k[IK]; u32x4 r[IR]; u32x4 v[IV]; };

  // Per query group u of the wavefront (query qw + 32 u + lane % 32).
  struct State {
    F qf[QH][KS_QK];   // q row (B operand), dims s K + hf KPL + [0, KPL)
    const E* dorow;    // the lane's dO row of group 0 (scaled by 2^g) in the wavefront's LDS area
    f32x16 dq[QH][NQT];
    float lse2[QH], dlt[QH];  // lse in log2 units; delta in the units of the scaled dO
  };

  // Chunk c = i NT + thread of a [BN][CPR chunks] region (c < BN * CPR).
  template <int CPR, int PER>
  __device__ static void load_region(const char* base, int row_bytes, int nk, u32x4* out) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(base, nk * row_bytes);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = i * NT + static_cast<int>(threadIdx.x);
      if ((BN * CPR) % NT == 0 || c < BN * CPR)
        out[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (c / CPR) * row_bytes + (c % CPR) * 16, 0, 0);
    }
  }

  // Keys key0 .. key0 + BN - 1; rows past the sequence read as zero.
  __device__ static void load_block(const BwdArgs& a, int b, int head, int64_t key0, Regs& R) {
    const int nk = static_cast<int>(a.S - key0 < BN ? a.S - key0 : BN);
    const int64_t row0 = (b * a.S + key0) * a.h + head;
    const int es = static_cast<int>(sizeof(E));
    load_region<CK, IK>(static_cast<const char*>(a.k_nope) + row0 * DN * es, a.h * DN * es, nk, R.k);
    load_region<CR, IR>(static_cast<const char*>(a.k_pe) + (b * a.S + key0) * DR * es, DR * es, nk, R.r);
    load_region<CV, IV>(static_cast<const char*>(a.v) + row0 * DV * es, a.h * DV * es, nk, R.v);
  }

  __device__ static void store_block(const Regs& R, char* buf) {
    E* Kr = reinterpret_cast<E*>(buf);
    E* Kt = reinterpret_cast<E*>(buf + OFF_KT);
    E* Vr = reinterpret_cast<E*>(buf + OFF_V);
#pragma unroll
    for (int i = 0; i < IK; ++i) {
      const int c = i * NT + static_cast<int>(threadIdx.x), r = c / CK, col = (c % CK) * EPC;
      if ((BN * CK) % NT != 0 && c >= BN * CK) continue;
      *reinterpret_cast<u32x4*>(Kr + r * LKR + col) = R.k[i];
      if constexpr (TR) *reinterpret_cast<u32x4*>(Kt + r * LKT + col) = R.k[i];
    }
#pragma unroll
    for (int i = 0; i < IR; ++i) {
      const int c = i * NT + static_cast<int>(threadIdx.x), r = c / CR, col = DN + (c % CR) * EPC;
      if ((BN * CR) % NT != 0 && c >= BN * CR) continue;
      *reinterpret_cast<u32x4*>(Kr + r * LKR + col) = R.r[i];
      if constexpr (TR) *reinterpret_cast<u32x4*>(Kt + r * LKT + col) = R.r[i];
    }
#pragma unroll
    for (int i = 0; i < IV; ++i) {
      const int c = i * NT + static_cast<int>(threadIdx.x), r = c / CV, col = (c % CV) * EPC;
      if ((BN * CV) % NT != 0 && c >= BN * CV) continue;
      *reinterpret_cast<u32x4*>(Vr + r * LV + col) = R.v[i];
    }
  }

  // A operand of dq^T += K^T dS^T: dims n0 + lane % 32, the keys of
  // accumulator registers st KPL .. st KPL + KPL - 1 of the 32-key half
  // starting at row k0 (see acc_key_col).
  __device__ static F kt_frag(const char* buf, int k0, int st, int n0) {
    if constexpr (TR) {
      return tr_frag_acc(reinterpret_cast<const E*>(buf + OFF_KT), LKT, k0 + st * 16, n0);
    } else {
      const int lane = threadIdx.x % kWave;
      const int key = k0 + 8 * (st / 4) + 4 * (lane / 32) + (st % 4);
      return reinterpret_cast<const E*>(buf)[key * LKR + n0 + lane % 32];
    }
  }

  // The 32 keys of the block in `buf` (the first at kg0) against the
  // wavefront's query groups (the first query at qw).
  __device__ static void compute(const BwdArgs& a, const char* buf, int64_t kg0, int64_t qw, State& st_) {
    constexpr int k0 = 0;
    const int lane = threadIdx.x % kWave;
    const int hf = lane / 32, col = lane % 32;
    const E* Kr = reinterpret_cast<const E*>(buf);
    const E* Vr = reinterpret_cast<const E*>(buf + OFF_V);
    f32x16 sc[QH], dp[QH];
#pragma unroll
    for (int u = 0; u < QH; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) { sc[u][r] = 0.f; dp[u][r] = 0.f; }
    // S^T and dP^T: one chain of row reads, kAhead ahead of the products,
    // each K / V read feeding every query group; the dP^T steps also read
    // the groups' dO fragments (B operands, the wavefront's LDS area) ahead.
    const E* krow = Kr + (k0 + col) * LKR + hf * M::KPL;
    const E* vrow = Vr + (k0 + col) * LV + hf * M::KPL;
    struct Ops { F a; F o[QH]; };
    pipelined<KS_QK + KS_V, kAhead, Ops>(
        [&](int i) {
          Ops r;
          if (i < KS_QK) {
            r.a = lds_frag<M>(krow + i * M::K);
          } else {
            r.a = lds_frag<M>(vrow + (i - KS_QK) * M::K);
#pragma unroll
            for (int u = 0; u < QH; ++u) r.o[u] = lds_frag<M>(st_.dorow + 32 * u * LDO + (i - KS_QK) * M::K);
          }
          return r;
        },
        [&](int i, const Ops& f) {
#pragma unroll
          for (int u = 0; u < QH; ++u) {
            if (i < KS_QK) sc[u] = M::mma(f.a, st_.qf[u][i], sc[u]);
            else dp[u] = M::mma(f.a, f.o[u], dp[u]);
          }
        });
    // P and dS = P (dP - delta) in the key order of the accumulator
    // registers: register r holds key kg0 + 8 (r / 4) + 4 hf + r % 4.  The
    // causal mask only where the block reaches past a group's first query.
    // One group at a time (a scheduling barrier between them), each packed
    // into MFMA operands right away: the group's 32 fp32 values are then the
    // only accumulator copies live in vector registers.
    F dsf[QH][STEPS];
#pragma unroll
    for (int u = 0; u < QH; ++u) {
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = __builtin_amdgcn_exp2f(fmaf(sc[u][r], a.scale_log2, -st_.lse2[u]));
      const int64_t gq = qw + 32 * u;
      if (kg0 + 31 > gq) {
        const int rel = static_cast<int>(gq + col - kg0) - 4 * hf;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r / 4) + (r % 4) > rel) ds[r] = 0.f;
      }
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        E t[M::KPL];
#pragma unroll
        for (int j = 0; j < M::KPL; ++j) t[j] = M::from_f32(ds[st * M::KPL + j] * (dp[u][st * M::KPL + j] - st_.dlt[u]));
        dsf[u][st] = *reinterpret_cast<F*>(t);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // dq^T += K^T dS^T.
    pipelined<STEPS * NQT, kAhead, F>([&](int i) { return kt_frag(buf, k0, i / NQT, (i % NQT) * 32); },
                                      [&](int i, const F& k) {
#pragma unroll
                                        for (int u = 0; u < QH; ++u)
                                          st_.dq[u][i % NQT] = M::mma(k, dsf[u][i / NQT], st_.dq[u][i % NQT]);
                                      });
  }

  // One key block: publish the prefetched block, prefetch the next one, and
  // compute if the block holds keys at or below some query of the wavefront.
  __device__ static void step(const BwdArgs& a, int kb, int nkb, int b, int head, int64_t qw, char* cur, Regs& R,
                              State& st_) {
    store_block(R, cur);
    __syncthreads();
    const int64_t key0 = static_cast<int64_t>(kb) * BN;
    if (kb + 1 < nkb) load_block(a, b, head, key0 + BN, R);
    // Blocks whose keys all follow the wavefront's queries are skipped (so
    // is everything for a wavefront past the end of the sequence).
    if (key0 > qw + WQ - 1 || qw >= a.S) return;
    compute(a, cur, key0, qw, st_);
  }

  __device__ static void run(const BwdArgs& a, char* lds) {
    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int hf = lane / 32, col = lane % 32;
    // Workgroup -> (batch * head, query tile): heads grouped per XCD (ids are
    // dealt round-robin to the 8 XCDs) so that the workgroups streaming one
    // head's K / V share an L2; the longest (latest) tiles start first.
    const int nbh = a.B * a.h;
    const int n_qt = static_cast<int>((a.S + BM - 1) / BM);
    int bh, qt_rank;
    if (nbh % 8 == 0) {
      const int xcd = blockIdx.x % 8, j = blockIdx.x / 8, hpx = nbh / 8;
      bh = xcd * hpx + j % hpx;
      qt_rank = j / hpx;
    } else {
      bh = blockIdx.x % nbh;
      qt_rank = blockIdx.x / nbh;
    }
    const int qt = n_qt - 1 - qt_rank;
    const int b = bh / a.h, head = bh % a.h;
    const int64_t q0 = static_cast<int64_t>(qt) * BM;
    const int64_t qw = q0 + wv * WQ;

    int64_t kend = q0 + BM;
    if (kend > a.S) kend = a.S;
    const int nkb = static_cast<int>((kend + BN - 1) / BN);
    Regs R;
    load_block(a, b, head, 0, R);

    // A lane past the sequence reads the first query's data instead (its
    // column of dq^T is never stored).
    State st_;
    st_.dorow = reinterpret_cast<const E*>(lds + OFF_DO + wv * DO_BYTES) + col * LDO + hf * M::KPL;
    const int g = do_shift_of(a);
    int rsh[QH];  // per-query power of two that normalises the query's dS (see below)
#pragma unroll
    for (int u = 0; u < QH; ++u) {
      const int64_t tq = qw + 32 * u + col;
      const int64_t tc = tq < a.S ? tq : 0;
      const int64_t row = (b * a.S + tc) * a.h + head;
      const E* qp = static_cast<const E*>(a.q) + row * DQK + hf * M::KPL;
      const E* op = static_cast<const E*>(a.d_o) + row * DV + hf * M::KPL;
#pragma unroll
      for (int s = 0; s < KS_QK; ++s) st_.qf[u][s] = *reinterpret_cast<const F*>(qp + s * M::K);
      // The lane's part of its dO row, in the layout it reads back.
      E* dst = reinterpret_cast<E*>(lds + OFF_DO + wv * DO_BYTES) + (32 * u + col) * LDO + hf * M::KPL;
#pragma unroll
      for (int s = 0; s < KS_V; ++s) *reinterpret_cast<F*>(dst + s * M::K) = *reinterpret_cast<const F*>(op + s * M::K);
      const int64_t si = (static_cast<int64_t>(b) * a.h + head) * a.S + tc;
      // dS of query t is linear in its dO row, whose fp16 copy carries the
      // global factor 2^g.  A row far below the largest |dO| would give dS in
      // fp16's subnormal range; scaling the row's P by 2^e (folded into the
      // exponent: P 2^e = exp2(log2 P + e)), with e from the row's own
      // magnitude (the E8M0 byte 127 - s of its e4m3 copy: max |dO| 2^s in
      // [128, 256)), brings every row's dS near unit scale; dq is divided by
      // 2^e at the end.
      rsh[u] = 0;
      if (a.osc != nullptr) {
        const int e = 120 - a.osc[si] - g;
        rsh[u] = e < -100 ? -100 : (e > 100 ? 100 : e);
      }
      st_.lse2[u] = a.lse[si] * kLog2e - static_cast<float>(rsh[u]);
      st_.dlt[u] = a.delta[si] * pow2i(g);
#pragma unroll
      for (int n = 0; n < NQT; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) st_.dq[u][n][r] = 0.f;
    }

    int kb = 0;
    // Unrolled by two so that each step names its buffer as a constant offset.
    for (; kb + 1 < nkb; kb += 2) {
      step(a, kb, nkb, b, head, qw, lds, R, st_);
      step(a, kb + 1, nkb, b, head, qw, lds + BUF_BYTES, R, st_);
    }
    if (kb < nkb) step(a, kb, nkb, b, head, qw, lds, R, st_);

    // dS carries dO's scale 2^g and the row's 2^e.
#pragma unroll
    for (int u = 0; u < QH; ++u) {
      const int64_t tq = qw + 32 * u + col;
      if (tq >= a.S) continue;
      const float osc = a.scale * pow2i(-g - rsh[u]);
      float* out = a.dq + ((b * a.S + tq) * a.h + head) * DQK;
#pragma unroll
      for (int n = 0; n < NQT; ++n)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (n * 32 + 8 * j + 4 * hf >= DQK) continue;
          const f32x4 w = {st_.dq[u][n][4 * j] * osc, st_.dq[u][n][4 * j + 1] * osc,
                           st_.dq[u][n][4 * j + 2] * osc, st_.dq[u][n][4 * j + 3] * osc};
          *reinterpret_cast<f32x4*>(out + n * 32 + 8 * j + 4 * hf) = w;
        }
    }
  }
};

template <class M, int DN, int DR, int DV, int NW, int QH>
__global__ __launch_bounds__(NW * kWave) void dq_kernel(BwdArgs a) {
  typedef Dq<M, DN, DR, DV, NW, QH> Kn;
  __shared__ __attribute__((aligned(16))) char lds[Kn::LDS_BYTES];
  Kn::run(a, lds);
}

template <class M, int DN, int DR, int DV, int NW, int QH>
hipError_t dq_t(const BwdArgs& a, const Shape& s, hipStream_t st) {
  typedef Dq<M, DN, DR, DV, NW, QH> Kn;
  const int64_t grid = ((s.S + Kn::BM - 1) / Kn::BM) * s.B * s.h;
  hipLaunchKernelGGL((dq_kernel<M, DN, DR, DV, NW, QH>), dim3(static_cast<unsigned>(grid)), dim3(Kn::NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_dq(const Shape& s, const void* q, const void* k_nope, const void* k_pe, const void* v,
                              const float* lse, const float* delta, const void* d_o, const int* do_shift,
                              const int* do_row_scale, float* dq, hipStream_t st) {
  BwdArgs a = make_args(s, q, k_nope, k_pe, v, lse, delta, d_o);
  a.dq = dq;
  a.do_shift = do_shift;
  a.osc = do_row_scale;
  if (s.bf16 && s.split && s.d_nope == 128 && s.d_rope == 64 && s.d_v == 128)
    return dq_t<MmaF16, 128, 64, 128, 4, 2>(a, s, st);
  if (!s.bf16 && s.d_nope == 32 && s.d_rope == 16 && s.d_v == 32) return dq_t<MmaF32, 32, 16, 32, 4, 1>(a, s, st);
  return hipErrorNotSupported;
}

}  // namespace laga
