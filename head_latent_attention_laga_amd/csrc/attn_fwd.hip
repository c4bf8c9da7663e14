// Causal attention forward of one rank's head shard.
//
// [LAGA §3.3 Algorithm 1 scores / softmax / output; §5.3 shared k_pe band]
//   s[t,u] = (q_nope || q_rope)[t,i] . (k_nope[u,i] || k_pe[u]) / sqrt(d_nope + d_rope), u <= t
//   o[t,i] = sum_u softmax_u(s) v[u,i],   lse[i,t] = ln sum_u exp(s[t,u])
//
// Flash-style: a workgroup of NW wavefronts owns BM = 32*NW queries of one
// head and streams keys 0 .. (last query of the tile) in blocks of BN = 64,
// with an online softmax, so no S x S matrix ever exists.  Key blocks are
// double-buffered in LDS: the next block's 16-byte global loads are in flight
// in registers while the current block is computed, then stored as plain
// 16-byte copies.  Tile rows are padded so that every LDS read below uses an
// immediate offset and hits distinct banks: K and rope rows (one row per lane,
// 16-byte reads) are 16 bytes longer than their data; V rows (transposing
// reads of 4 rows x 64 bytes per half-wavefront) are 64 bytes longer.
//
// Each wavefront keeps its 32 queries in registers as the B operand of
//     S^T[key, query] = K . Q^T          (A = K rows, 16-byte LDS reads)
// so the 32x32 accumulators hold one query per lane column: running max and
// sum are lane-local up to one exchange between the wavefront halves, and the
// probabilities already sit in the B-operand layout of
//     O^T[dv, query] += V^T . P^T        (A = V^T via transposing LDS reads)
// The rope band stays bf16 and meets q_rope in bf16 MFMAs (both exact); the
// nope part meets q_nope (converted once to fp16, exactly) in fp16 MFMAs.
// The k_pe band is loaded once per key block for all queries of the tile and
// never expanded per head.  Blocks above a wavefront's diagonal are skipped;
// only blocks crossing it are masked.
//
// Precision: NS == 1 uses single fp16 K, V and P.  NS == 2 reads K and V as
// laga_kv_up writes them for split operands, an fp16 hi plane and an e4m3
// plane of the rest scaled by 2^kLoShift: S = Q.K_hi + Q8.K_lo and
// O = P.V_hi + P8.V_lo, where the low terms run as e4m3 matrix-core products
// (K = 64 per instruction, half the cycles of fp16 per element) with q and P
// rounded to e4m3 -- harmless, as those terms are 2^-11 of the result.  P in
// fp16 rounds independently from pair to pair and averages out in O and in
// the backward's delta = sum dO o.
// The float32 instantiation uses fp32 MFMAs throughout.
#include <algorithm>
#include "attn_common.hpp"
#include "launch.hpp"

namespace laga {
namespace {

constexpr int BN = 64;          // keys per block
constexpr float kRescale = 8.f;  // lazy-rescale threshold of the running max (log2 units)


struct FwdArgs {
  const void* q; const void* k_nope; const void* k_pe; const void* v;
  float* o; float* lse;
  int64_t S, plane_k, plane_v; int B, h, n_qt; float scale_log2;
};

// Row padding (elements) of the K, rope and V tiles.  16-bit V tiles are
// read only with transposing reads and go unpadded with swizzled blocks.
template <class M, int NS> struct Pads { static constexpr int k = 8, r = 8, v = 0; static constexpr bool swz = true; };
template <int NS> struct Pads<MmaF32, NS> { static constexpr int k = 4, r = 4, v = 4; static constexpr bool swz = false; };

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
  // Chunks (16 bytes) per row, elements per chunk, padded row pitches.
  static constexpr int EPC = 16 / sizeof(E), RPC = 16 / sizeof(ER);
  static constexpr int CK = DN / EPC, CR = DR / RPC, CV = DV / EPC;
  static constexpr int LDK = DN + Pads<M, NS>::k, LDR = DR + Pads<M, NS>::r, LDV = DV + Pads<M, NS>::v;
  // NS == 2: K and V also have an e4m3 low plane (see kLoShift).
  static constexpr bool LO8 = NS == 2;
  static_assert(!LO8 || sizeof(E) == 2, "low planes complement fp16 operands");
  static constexpr int K8P = DN + 16;  // byte pitch of the e4m3 K rows (16-byte row reads)
  // LDS buffer: K | K low | rope band | V | V low.
  static constexpr int K_BYTES = BN * LDK * sizeof(E);
  static constexpr int K8_BYTES = LO8 ? BN * K8P : 0;
  static constexpr int R_BYTES = BN * LDR * sizeof(ER);
  static constexpr int V_BYTES = BN * LDV * sizeof(E);
  static constexpr int V8_BYTES = LO8 ? BN * DV : 0;
  static constexpr int OFF_K8 = K_BYTES, OFF_R = OFF_K8 + K8_BYTES, OFF_V = OFF_R + R_BYTES,
                       OFF_V8 = OFF_V + V_BYTES;
  static constexpr int BUF_BYTES = OFF_V8 + V8_BYTES;
  static_assert(OFF_V % 256 == 0 && OFF_V8 % 128 == 0 && BUF_BYTES % 256 == 0, "swizzled tiles stay aligned");
  // 16-byte chunks of data per region (the padding is never loaded).
  static constexpr int K_CH = BN * CK, K8_CH = LO8 ? BN * DN / 16 : 0, R_CH = BN * CR, V_CH = BN * CV,
                       V8_CH = LO8 ? BN * DV / 16 : 0;
  static_assert(K_CH % NT == 0 && K8_CH % NT == 0 && R_CH % NT == 0 && V_CH % NT == 0 && V8_CH % NT == 0,
                "staging passes");
  static constexpr int KS_N = DN / M::K, KS_R = DR / MR::K, NO = DV / 32, PV_STEPS = 32 / M::K;
  static constexpr int KS_8 = DN / 64;  // e4m3 atoms (K = 64) over d_nope
  static_assert(DN % M::K == 0 && DR % MR::K == 0 && DV % 32 == 0 && (!LO8 || (DN % 64 == 0 && DV == 128 && BN == 64)),
                "head dims");

  // Staging: chunk c of a plane-major [planes][BN][CPR chunks] region, read
  // from global memory in order (coalesced) and written to its padded row.
  // Each region is a whole number of workgroup passes.
  static constexpr int IK = K_CH / NT, IK8 = K8_CH / NT, IR = R_CH / NT, IV = V_CH / NT, IV8 = V8_CH / NT;
  struct Regs {
    u32x4 k[IK]; u32x4 k8[IK8 > 0 ? IK8 : 1]; u32x4 r[IR > 0 ? IR : 1]; u32x4 v[IV]; u32x4 v8[IV8 > 0 ? IV8 : 1];
  };

  // Buffer loads: one scalar descriptor per (region, plane) and block, lane
  // offsets fixed for the whole kernel.  Rows past the end of the sequence
  // lie outside the descriptor's range and read as zero (masked anyway).
  template <int CPR, int PER>
  __device__ static void load_region(const char* block_base, int64_t plane_bytes, int row_bytes, int nk,
                                     u32x4* out) {
    static_assert((BN * CPR) % NT == 0, "a pass stays inside one plane");
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = i * NT + static_cast<int>(threadIdx.x);
      const int plane = (i * NT) / (BN * CPR);
      const int r = (c % (BN * CPR)) / CPR, lc = c % CPR;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(block_base + plane * plane_bytes), 0, nk * row_bytes, 0x00020000);
      out[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, r * row_bytes + lc * 16, 0, 0);
    }
  }

  // SWZ: 0 plain rows, 1 swz_block (16-bit transposing reads), 2 swz8_chunk
  // (8-bit transposing reads).
  template <int CPR, int PER, int PITCH_BYTES, int SWZ = 0>
  __device__ static void store_region(const u32x4* in, char* lds_region) {
    static_assert(SWZ != 1 || (CPR >= 16 && PITCH_BYTES % 256 == 0), "swizzled rows span whole 256-byte windows");
    static_assert(SWZ != 2 || (CPR == 8 && PITCH_BYTES == 128), "8-bit swizzle assumes 128-byte rows");
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = i * NT + static_cast<int>(threadIdx.x);
      const int plane = c / (BN * CPR), r = (c % (BN * CPR)) / CPR, lc = c % CPR;
      const int pc = SWZ == 1 ? swz_block(r, lc) : SWZ == 2 ? swz8_chunk(r, lc) : lc;
      *reinterpret_cast<u32x4*>(lds_region + (plane * BN + r) * PITCH_BYTES + pc * 16) = in[i];
    }
  }

  __device__ static void load_block(const FwdArgs& a, int b, int head, int64_t key0, Regs& R) {
    const int nk = static_cast<int>(a.S - key0 < BN ? a.S - key0 : BN);
    const int64_t row0 = (b * a.S + key0) * a.h + head;
    const char* kg = static_cast<const char*>(a.k_nope);
    const char* vg = static_cast<const char*>(a.v);
    load_region<CK, IK>(kg + row0 * DN * sizeof(E), 0, a.h * DN * static_cast<int>(sizeof(E)), nk, R.k);
    load_region<CR, IR>(static_cast<const char*>(a.k_pe) + (b * a.S + key0) * DR * sizeof(ER), 0,
                        DR * static_cast<int>(sizeof(ER)), nk, R.r);
    load_region<CV, IV>(vg + row0 * DV * sizeof(E), 0, a.h * DV * static_cast<int>(sizeof(E)), nk, R.v);
    if constexpr (LO8) {  // byte planes after the fp16 planes
      load_region<DN / 16, IK8>(kg + a.plane_k * sizeof(E) + row0 * DN, 0, a.h * DN, nk, R.k8);
      load_region<DV / 16, IV8>(vg + a.plane_v * sizeof(E) + row0 * DV, 0, a.h * DV, nk, R.v8);
    }
  }

  __device__ static void store_block(const Regs& R, char* buf) {
    store_region<CK, IK, LDK * sizeof(E)>(R.k, buf);
    store_region<CR, IR, LDR * sizeof(ER)>(R.r, buf + OFF_R);
    store_region<CV, IV, LDV * sizeof(E), Pads<M, NS>::swz ? 1 : 0>(R.v, buf + OFF_V);
    if constexpr (LO8) {
      store_region<DN / 16, IK8, K8P>(R.k8, buf + OFF_K8);
      store_region<DV / 16, IV8, DV, 2>(R.v8, buf + OFF_V8);
    }
  }

  static constexpr int kScoreAhead = 2;  // score operand reads in flight ahead of the products
  __device__ static F k_frag(const E* Kp, int r, int c0) { return lds_frag<M>(Kp + r * LDK + c0); }
  __device__ static FR r_frag(const ER* Rp, int r, int c0) { return lds_frag<MR>(Rp + r * LDR + c0); }

  // A operand of O^T += V^T P^T for one MFMA step: rows dv n0 + lane%32, keys of
  // accumulator registers st*KPL .. of 32-key atom t (see acc_key_col).
  __device__ static F v_frag(const E* Vp, int t, int st, int n0) {
    if constexpr (M::KPL == 8) {
      return tr_frag_acc_swz(Vp, LDV, t * 32 + st * 16, n0);
    } else {
      const int lane = threadIdx.x % kWave;
      const int key = t * 32 + 8 * (st / 4) + 4 * (lane / 32) + (st % 4);
      return Vp[key * LDV + n0 + lane % 32];
    }
  }

  // A operand of S_lo^T += K_lo . Q^T, e4m3 atom s: key row krow, bytes
  // 64 s + 32 hf + [0, 32) of the row.
  __device__ static i32x8 k8_frag(const uint8_t* K8, int krow, int s, int hf) {
    const uint8_t* p = K8 + krow * K8P + 64 * s + 32 * hf;
    const u32x4 x = *reinterpret_cast<const u32x4*>(p), y = *reinterpret_cast<const u32x4*>(p + 16);
    return i32x8{static_cast<int>(x[0]), static_cast<int>(x[1]), static_cast<int>(x[2]), static_cast<int>(x[3]),
                 static_cast<int>(y[0]), static_cast<int>(y[1]), static_cast<int>(y[2]), static_cast<int>(y[3])};
  }

  struct State {
    i32x8 q8[LO8 ? KS_8 : 1];
    F qn[KS_N];
    FR qr[KS_R];
    f32x16 o[NO];
    float m_run, l_run;
  };

  __device__ static void compute_block(const FwdArgs& a, const char* buf, int64_t key0, int64_t qw, int64_t tq,
                                       State& st_) {
    const int lane = threadIdx.x % kWave;
    const int hf = lane / 32, col = lane % 32;
    const E* Ks = reinterpret_cast<const E*>(buf);
    const ER* Kr = reinterpret_cast<const ER*>(buf + OFF_R);
    const E* Vs = reinterpret_cast<const E*>(buf + OFF_V);
    const uint8_t* K8 = reinterpret_cast<const uint8_t*>(buf + OFF_K8);
    const uint8_t* V8 = reinterpret_cast<const uint8_t*>(buf + OFF_V8);

    f32x16 sc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[t][r] = 0.f;
    if constexpr (sizeof(F) == 16 && sizeof(FR) == 16) {
      // One chain of 16-byte operand reads, kScoreAhead ahead of the products:
      //   K_nope (s, t) | rope band (s, t) | e4m3 K_lo halves (s, t, half)
      // the low terms adding Q . K_lo (e4m3 K_lo * 2^kLoShift against e4m3 q).
      constexpr int NN = 2 * KS_N, NR = 2 * KS_R, N8 = LO8 ? 4 * KS_8 : 0;
      u32x4 lo;  // first half of an e4m3 fragment
      pipelined<NN + NR + N8, kScoreAhead, u32x4>(
          [&](int i) {
            if (i < NN) {
              return __builtin_bit_cast(u32x4, k_frag(Ks, (i % 2) * 32 + col, (i / 2) * M::K + hf * M::KPL));
            } else if (i < NN + NR) {
              const int j = i - NN;
              return __builtin_bit_cast(u32x4, r_frag(Kr, (j % 2) * 32 + col, (j / 2) * MR::K + hf * MR::KPL));
            } else {
              const int j = i - NN - NR;  // (s, t, half) = (j / 4, (j / 2) % 2, j % 2)
              return *reinterpret_cast<const u32x4*>(K8 + ((j / 2) % 2 * 32 + col) * K8P + 64 * (j / 4) + 32 * hf +
                                                      16 * (j % 2));
            }
          },
          [&](int i, const u32x4& f) {
            if (i < NN) {
              sc[i % 2] = M::mma(__builtin_bit_cast(F, f), st_.qn[i / 2], sc[i % 2]);
            } else if (i < NN + NR) {
              const int j = i - NN;
              sc[j % 2] = MR::mma(__builtin_bit_cast(FR, f), st_.qr[j / 2], sc[j % 2]);
            } else {
              const int j = i - NN - NR;
              if (j % 2 == 0) {
                lo = f;
              } else {
                const i32x8 k8 = {static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                                  static_cast<int>(lo[3]), static_cast<int>(f[0]), static_cast<int>(f[1]),
                                  static_cast<int>(f[2]), static_cast<int>(f[3])};
                const int t = (j / 2) % 2;
                sc[t] = mma_e4m3(k8, st_.q8[j / 4], sc[t], 127 - kLoShift, 127);
              }
            }
          });
    } else {
#pragma unroll
      for (int s = 0; s < KS_N; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int krow = t * 32 + col;
          sc[t] = M::mma(k_frag(Ks, krow, s * M::K + hf * M::KPL), st_.qn[s], sc[t]);
        }
#pragma unroll
      for (int s = 0; s < KS_R; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          sc[t] = MR::mma(r_frag(Kr, t * 32 + col, s * MR::K + hf * MR::KPL), st_.qr[s], sc[t]);
      if constexpr (LO8) {  // + Q . K_lo: e4m3 K_lo * 2^kLoShift against e4m3 q
#pragma unroll
        for (int s = 0; s < KS_8; ++s)
#pragma unroll
          for (int t = 0; t < 2; ++t)
            sc[t] = mma_e4m3(k8_frag(K8, t * 32 + col, s, hf), st_.q8[s], sc[t], 127 - kLoShift, 127);
      }
    }

    // Causal mask, only on blocks that cross this wavefront's diagonal: key
    // key0 + t*32 + 8(r/4) + 4hf + r%4 is masked when it exceeds the query.
    if (__builtin_expect(key0 + BN - 1 > qw, 0)) {
      const int rel = static_cast<int>(tq - key0) - 4 * hf;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (t * 32 + 8 * (r / 4) + (r % 4) > rel) sc[t][r] = -INFINITY;
    }
    // Row max of the raw scores (the scale > 0 is folded into the exponent).
    float mloc = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sc[t][r]);
    mloc = pair_max(mloc) * a.scale_log2;
    // The running max (log2 units) is raised only when a row's block max
    // exceeds it by more than kRescale, so unnormalised probabilities stay
    // below 2^kRescale and O / l are rescaled rarely.
    if (__any(mloc > st_.m_run + kRescale)) {
      const float m_new = fmaxf(st_.m_run, mloc);
      const float alpha = __builtin_amdgcn_exp2f(st_.m_run - m_new);
      st_.l_run *= alpha;
#pragma unroll
      for (int n = 0; n < NO; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) st_.o[n][r] *= alpha;
      st_.m_run = m_new;
    }
    float lsum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[t][r], a.scale_log2, -st_.m_run));
        sc[t][r] = p;
        lsum += p;
      }
    st_.l_run += pair_sum(lsum);

    // O^T += V^T P^T; one step covers K keys, accumulator r = st*KPL + j.
    if constexpr (sizeof(F) == 16) {
      // V^T operands read kScoreAhead products ahead; P of (t, st) converted
      // where its first product needs it.
      F pf;
      pipelined<2 * PV_STEPS * NO, kScoreAhead, F>(
          [&](int i) { return v_frag(Vs, i / NO / PV_STEPS, (i / NO) % PV_STEPS, (i % NO) * 32); },
          [&](int i, const F& v) {
            const int t = i / NO / PV_STEPS, st = (i / NO) % PV_STEPS;
            if (i % NO == 0) {
              E ph[M::KPL];
#pragma unroll
              for (int j = 0; j < M::KPL; ++j) ph[j] = M::from_f32(sc[t][st * M::KPL + j]);
              pf = *reinterpret_cast<F*>(ph);
            }
            st_.o[i % NO] = M::mma(v, pf, st_.o[i % NO]);
          });
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int st = 0; st < PV_STEPS; ++st) {
          E ph[M::KPL];
#pragma unroll
          for (int j = 0; j < M::KPL; ++j) ph[j] = M::from_f32(sc[t][st * M::KPL + j]);
          const F pf = *reinterpret_cast<F*>(ph);
#pragma unroll
          for (int n = 0; n < NO; ++n) st_.o[n] = M::mma(v_frag(Vs, t, st, n * 32), pf, st_.o[n]);
        }
    }
    if constexpr (LO8) {
      // + P . V_lo over the whole block in one e4m3 atom per 32 dv: byte
      // 16 t + r of a lane's P operand is its probability sc[t][r].  P stays
      // at or below 2^kRescale (the running max), inside e4m3's range.
      static_assert(kRescale <= 8, "unnormalised probabilities within e4m3's 448");
      i32x8 p8;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          p8[4 * t + g] = static_cast<int>(
              pack_e4m3x4_in_range(sc[t][4 * g], sc[t][4 * g + 1], sc[t][4 * g + 2], sc[t][4 * g + 3]));
#pragma unroll
      for (int n = 0; n < NO; ++n) st_.o[n] = mma_e4m3(tr8_frag_acc64(V8, n), p8, st_.o[n], 127 - kLoShift, 127);
    }
  }

  // One key block: publish the prefetched block, prefetch the next one, and
  // compute (ALL: every wavefront of the tile has keys <= its queries here).
  template <bool ALL>
  __device__ static void step(const FwdArgs& a, int kb, int nkb, int b, int head, int64_t qw, int64_t tq,
                              char* cur, Regs& R, State& st_) {
    store_block(R, cur);
    __syncthreads();
    const int64_t key0 = static_cast<int64_t>(kb) * BN;
    if (kb + 1 < nkb) load_block(a, b, head, key0 + BN, R);
    if (ALL || key0 <= qw + 31) compute_block(a, cur, key0, qw, tq, st_);
  }

  // Q fragments (B operand) of query tq -- dims hf*KPL + s*K + [0, KPL) -- and
  // an empty accumulator.
  __device__ static void begin(const FwdArgs& a, int b, int head, int64_t tq, bool qvalid, State& st_) {
    const int hf = (threadIdx.x % kWave) / 32;
    const InT* qp = static_cast<const InT*>(a.q) + ((b * a.S + (qvalid ? tq : 0)) * a.h + head) * (DN + DR);
#pragma unroll
    for (int s = 0; s < KS_N; ++s) {
      E tmp[M::KPL];
      if constexpr (M::KPL == 8 && sizeof(InT) == 2) {
        const u16x8 raw = qvalid ? *reinterpret_cast<const u16x8*>(qp + s * M::K + hf * M::KPL) : u16x8{};
#pragma unroll
        for (int j = 0; j < 8; ++j) tmp[j] = M::from_f32(to_f32(static_cast<InT>(raw[j])));
      } else {
#pragma unroll
        for (int j = 0; j < M::KPL; ++j) tmp[j] = M::from_f32(qvalid ? to_f32(qp[s * M::K + hf * M::KPL + j]) : 0.f);
      }
      st_.qn[s] = *reinterpret_cast<F*>(tmp);
    }
    if constexpr (LO8) {  // e4m3 copy of q_nope for the low-plane products: dims 64 s + 32 hf + [0, 32)
#pragma unroll
      for (int s = 0; s < KS_8; ++s)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u16x8 raw = qvalid ? *reinterpret_cast<const u16x8*>(qp + 64 * s + 32 * hf + 8 * c) : u16x8{};
          float f[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) f[j] = to_f32(static_cast<InT>(raw[j]));
          st_.q8[s][2 * c] = static_cast<int>(pack_e4m3x4(f[0], f[1], f[2], f[3]));
          st_.q8[s][2 * c + 1] = static_cast<int>(pack_e4m3x4(f[4], f[5], f[6], f[7]));
        }
    }
#pragma unroll
    for (int s = 0; s < KS_R; ++s) {
      if constexpr (MR::KPL == 8 && sizeof(InT) == 2) {
        st_.qr[s] = qvalid ? *reinterpret_cast<const FR*>(qp + DN + s * MR::K + hf * MR::KPL) : FR{};
      } else {
        ER tmp[MR::KPL];
#pragma unroll
        for (int j = 0; j < MR::KPL; ++j) tmp[j] = qvalid ? qp[DN + s * MR::K + hf * MR::KPL + j] : ER{};
        st_.qr[s] = *reinterpret_cast<FR*>(tmp);
      }
    }
#pragma unroll
    for (int n = 0; n < NO; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) st_.o[n][r] = 0.f;
    st_.m_run = -INFINITY;
    st_.l_run = 0.f;
  }

  // o = O / l and lse of query tq.
  __device__ static void finish(const FwdArgs& a, int b, int head, int64_t tq, bool qvalid, const State& st_) {
    if (!qvalid) return;
    const int hf = (threadIdx.x % kWave) / 32;
    const float inv = 1.0f / st_.l_run;
    float* op = a.o + ((b * a.S + tq) * a.h + head) * DV;
#pragma unroll
    for (int n = 0; n < NO; ++n)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 w = {st_.o[n][4 * g] * inv, st_.o[n][4 * g + 1] * inv, st_.o[n][4 * g + 2] * inv,
                   st_.o[n][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(op + n * 32 + 8 * g + 4 * hf) = w;
      }
    if (hf == 0)
      a.lse[(static_cast<int64_t>(b) * a.h + head) * a.S + tq] = (st_.m_run + log2f(st_.l_run)) * 0.69314718055994531f;
  }

  // Blocks with key0 <= q0 + 31 are computed by every wavefront; the last few
  // (above the lower wavefronts' diagonals) are skipped per wavefront.
  __device__ static int blocks_for_all(int64_t q0, int nkb) {
    const int nall = static_cast<int>((q0 + 31) / BN) + 1;
    return nall < nkb ? nall : nkb;
  }

  __device__ static void run(const FwdArgs& a, char* lds) {
    const int lane = threadIdx.x % kWave;
    const int wv = threadIdx.x / kWave;
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

    int64_t kend = q0 + BM;
    if (kend > a.S) kend = a.S;
    const int nkb = static_cast<int>((kend + BN - 1) / BN);
    Regs R;
    load_block(a, b, head, 0, R);
    State st_;
    begin(a, b, head, tq, qvalid, st_);

    const int nall = blocks_for_all(q0, nkb);
    int kb = 0;
    // Unrolled by two so that each step names its buffer as a constant offset
    // and the LDS addresses fold into immediates (single-term operands only:
    // the split instantiation has no registers to spare for it).
    if constexpr (!LO8) {
      for (; kb + 1 < nall; kb += 2) {
        step<true>(a, kb, nkb, b, head, qw, tq, lds, R, st_);
        step<true>(a, kb + 1, nkb, b, head, qw, tq, lds + BUF_BYTES, R, st_);
      }
    }
    for (; kb < nall; ++kb) step<true>(a, kb, nkb, b, head, qw, tq, lds + (kb & 1) * BUF_BYTES, R, st_);
    for (; kb < nkb; ++kb) step<false>(a, kb, nkb, b, head, qw, tq, lds + (kb & 1) * BUF_BYTES, R, st_);
    finish(a, b, head, tq, qvalid, st_);
  }

  // ------------------------------------------------ key blocks given as LDS images
  // The fused forward's attention: key block kb of (b, head) is a ready-made
  // image of the LDS buffer (K, rope band and V rows, padded and swizzled as
  // store_block leaves them) at img + kb * BUF_BYTES, so each block is one
  // contiguous global -> LDS copy (1 KB per wavefront instruction, no staging
  // registers), issued one block ahead into the other buffer.
  static constexpr int IMG_LOADS = BUF_BYTES / 1024;
  static_assert(BUF_BYTES % 1024 == 0, "whole 1 KB copies");

  __device__ static void issue_image(const char* img_block, char* buf, int wv) {
    const int lane = threadIdx.x % kWave;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(img_block), 0, BUF_BYTES, 0x00020000);
    for (int j = wv; j < IMG_LOADS; j += NW) load_lds16(rs, buf + j * 1024, j * 1024 + 16 * lane);
  }

  // Waits until this wavefront's copies of the current block have landed,
  // leaving those of the next block (if any) in flight: the copies return in
  // issue order, and a wavefront issues IMG_HI or IMG_HI - 1 of them per block.
  static constexpr int IMG_HI = (IMG_LOADS + NW - 1) / NW;
  static constexpr int IMG_NHI = IMG_LOADS % NW == 0 ? NW : IMG_LOADS % NW;  // wavefronts issuing IMG_HI
  __device__ static void wait_image(bool next_in_flight, int wv) {
    if (!next_in_flight) wait_vmcnt<0>();
    else if (wv < IMG_NHI) wait_vmcnt<IMG_HI>();
    else wait_vmcnt<IMG_HI - 1>();
  }

  // Readiness of the key tiles (kTileBlocks blocks each) when images are
  // produced by other workgroups: flags[kt] is set (release) once tile kt's
  // images are written.  Thread 0 checks a tile before the barrier of the step
  // that copies its first block; the flag's load is issued one step earlier,
  // so the step's wait for its copies also covers it and a ready tile costs no
  // stall.  Waiting is bounded: past kSpinLimit polls *ok is cleared and the
  // error word set, and the caller writes NaN instead of results.
  struct Ready { const int* flags; int* err; int* ok; };
  static constexpr int kTileBlocks = 4;                // 256 keys per produced tile
  static constexpr unsigned kSpinLimit = 1u << 20;     // polls (about 0.2 us apart)
  __device__ static int peek_tile(const Ready& rd, int blk, int nkb) {
    return blk < nkb && blk % kTileBlocks == 0
               ? __hip_atomic_load(rd.flags + blk / kTileBlocks, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
               : 1;
  }
  __device__ static void tile_ready(const Ready& rd, int kt, int fv) {
    unsigned spins = 0;
    while (fv == 0) {
      if (++spins > kSpinLimit) {
        *rd.ok = 0;
        __hip_atomic_store(rd.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
      fv = __hip_atomic_load(rd.flags + kt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the tile's images are visible to the copies below
  }

  // One key block with NBUF buffers: block kb is in `cur`; block kb + NBUF - 1
  // goes into `ahead` (the buffer of block kb - 1, free once every wavefront
  // has passed this step's barrier).
  template <bool ALL, int NBUF>
  __device__ static void image_step(const FwdArgs& a, const char* img, int kb, int nkb, int wv, int64_t qw,
                                    int64_t tq, char* cur, char* ahead, State& st_, const Ready& rd, int& fv) {
    if constexpr (NBUF == 2) wait_vmcnt<0>();
    else wait_image(kb + 1 < nkb, wv);
    const int nb = kb + NBUF - 1;  // the block this step copies
    if (rd.flags != nullptr && threadIdx.x == 0 && nb < nkb && nb % kTileBlocks == 0)
      tile_ready(rd, nb / kTileBlocks, fv);
    __syncthreads();
    if (nb < nkb) issue_image(img + static_cast<int64_t>(nb) * BUF_BYTES, ahead, wv);
    if (rd.flags != nullptr && threadIdx.x == 0) fv = peek_tile(rd, nb + 1, nkb);
    const int64_t key0 = static_cast<int64_t>(kb) * BN;
    if (ALL || key0 <= qw + 31) compute_block(a, cur, key0, qw, tq, st_);
  }

  // Query tile qt of (b, head) against the images at img (that head's block 0),
  // NBUF image buffers at lds.  part 0: every key block, o and lse written.
  // part 1 / 2: the key blocks before / from split_block(), and the
  // unnormalised partial (O, running max, sum; log2 units) written to `partial`
  // ([BM rows][PART_ROW] floats) for fused_merge_kernel.
  static constexpr int PART_ROW = DV + 4;  // 16-byte aligned rows: O, then the running max and sum
  __device__ static int split_block(int64_t q0, int nkb) { return blocks_for_all(q0, nkb) / 2; }

  template <int NBUF>
  __device__ static bool run_images(const FwdArgs& a, const char* img, int b, int head, int qt, char* lds,
                                    int part, float* partial, const Ready& rd) {
    static_assert(!LO8, "images hold single-plane K and V");
    static_assert(NBUF == 2 || NBUF == 3, "double or triple buffering");
    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int64_t q0 = static_cast<int64_t>(qt) * BM;
    const int64_t qw = q0 + wv * 32;
    const int64_t tq = qw + lane % 32;
    const bool qvalid = tq < a.S;
    int64_t kend = q0 + BM;
    if (kend > a.S) kend = a.S;
    const int nkb = static_cast<int>((kend + BN - 1) / BN);
    const int kmid = split_block(q0, nkb);
    const int kb0 = part == 2 ? kmid : 0, kb1 = part == 1 ? kmid : nkb;  // this task's key blocks
    const int nall = blocks_for_all(q0, nkb) < kb1 ? blocks_for_all(q0, nkb) : kb1;
    static_assert(NBUF == 2, "the tile flags are read one step ahead, under the step's vmcnt(0)");
    State st_;
    begin(a, b, head, tq, qvalid, st_);  // q loads first: the block waits below count only image copies after them
    int fv = 1;
    if (rd.flags != nullptr && threadIdx.x == 0)
      tile_ready(rd, kb0 / kTileBlocks,
                 __hip_atomic_load(rd.flags + kb0 / kTileBlocks, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    __syncthreads();
    issue_image(img + static_cast<int64_t>(kb0) * BUF_BYTES, lds, wv);
    if (rd.flags != nullptr && threadIdx.x == 0) fv = peek_tile(rd, kb0 + 1, kb1);
    int kb = kb0;
    // Unrolled by NBUF so that each step names its buffers as constant offsets
    // (block kb0 + j + NBUF i sits in buffer j).
    for (; kb + NBUF - 1 < nall; kb += NBUF) {
#pragma unroll
      for (int j = 0; j < NBUF; ++j)
        image_step<true, NBUF>(a, img, kb + j, kb1, wv, qw, tq, lds + j * BUF_BYTES,
                               lds + ((j + NBUF - 1) % NBUF) * BUF_BYTES, st_, rd, fv);
    }
    for (; kb < kb1; ++kb)
      image_step<false, NBUF>(a, img, kb, kb1, wv, qw, tq, lds + ((kb - kb0) % NBUF) * BUF_BYTES,
                              lds + ((kb - kb0 + NBUF - 1) % NBUF) * BUF_BYTES, st_, rd, fv);
    if (rd.flags != nullptr && !*rd.ok) return false;  // set before the last step's barrier
    if (part == 0) {
      finish(a, b, head, tq, qvalid, st_);
      return true;
    }
    if (!qvalid) return true;
    const int hf = lane / 32;
    float* pr = partial + static_cast<int64_t>(wv * 32 + lane % 32) * PART_ROW;
#pragma unroll
    for (int n = 0; n < NO; ++n)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(pr + n * 32 + 8 * g + 4 * hf) =
            f32x4{st_.o[n][4 * g], st_.o[n][4 * g + 1], st_.o[n][4 * g + 2], st_.o[n][4 * g + 3]};
    if (hf == 0) {
      pr[DV] = st_.m_run;
      pr[DV + 1] = st_.l_run;
    }
    return true;
  }
};

// Two wavefronts per SIMD: either one 8-wavefront workgroup or two independent
// 4-wavefront workgroups per CU (whose barriers do not line up).
template <class InT, class M, class MR, int NS, int DN, int DR, int DV, int NW>
__global__ __launch_bounds__(NW * kWave, 2) void attn_fwd_kernel(FwdArgs a) {
  typedef Fwd<InT, M, MR, NS, DN, DR, DV, NW> Kn;
  __shared__ __attribute__((aligned(1024))) char lds[2 * Kn::BUF_BYTES];
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

// ------------------------------------------------------------------ fused forward
// The up-projection fused with the attention, in one launch [LAGA §4.7
// Limitations, fused up-projection kernel; §8 Discussion, open direction (i)].
// Operands are fp16 (the forward-only precision mode): a prep kernel writes
// the normalised latent L (RMSNorm of §2.1, rounded to fp16) and the head
// shard W_r of W_kv_b converted to fp16; then every workgroup of the fused
// kernel takes a ticket from an atomic counter and runs one task:
//  * producer (tickets first): K/V of 256 keys x one head, C^T = W_r[head] L^T
//    (fp16 matrix-core products, both operands copied global -> LDS through a
//    ring of three stages), written -- with the keys' k_pe rows -- as four
//    images of the attention's LDS key-block buffer, then flagged as written
//    (one flag per head and key tile, release at device scope);
//  * consumer (tickets after every producer ticket): the attention of one
//    256-query tile of one head (or of one half of its key blocks, for the
//    heaviest tiles of short sequences), heaviest first, which streams the
//    images with plain global -> LDS copies, waiting (acquire) for each key
//    tile's flag before copying its first block.
// A consumer waits only for producer tasks, and every producer ticket is
// handed out before any consumer ticket, so each producer a consumer waits
// for is already running on some CU, and producers wait for nothing: every
// wait ends.  A bounded spin backs that up: past it the consumer writes NaN
// outputs and sets the error word instead of spinning on.  The tickets are
// split into 8 independent queues by workgroup id modulo 8 (when the batch
// x heads count allows), one per XCD under the round-robin dispatch, so one
// head's producers and consumers share an L2.
typedef Fwd<bf16_t, MmaF16, MmaBf16, 1, 128, 64, 128, 8> FusedAttn;
constexpr int kFusedKeys = 256;          // keys per producer task
constexpr int kMaxTasks = 64;            // consumer tasks per head when query tiles are split
constexpr int kCUs = 256;                // compute units the split rule balances over (MI355X)

struct FusedArgs {
  FwdArgs f;  // q, o, lse, sizes and the score scale of the attention
  const half_t* l16;   // [T, 512] fp16 normalised latent
  const half_t* w16;   // [h, 256, 512] fp16 head shard of W_kv_b
  const bf16_t* k_pe;  // [T, 64]
  char* img;           // [B*h][nkb_img][BUF_BYTES] key-block images
  int* tickets;        // [8]
  int* err;            // set when a consumer gave up waiting
  int* done;           // [B*h][n_kt] set when that key tile's images are written
  int n_kt, nkb_img, parts, hpp, prod_pp;
  // Consumer tasks per head in ticket order when some query tiles are split
  // (n_task > 0): qt << 2 | part (0 whole, 1 / 2 the halves of its key blocks);
  // with n_task == 0 tile n_qt - 1 - rank, whole.  Split tiles are qt >= q_split.
  int n_task, q_split;
  int task[kMaxTasks];
  float* part;  // [(qt - q_split) * B * h + bh][2][BM][PART_ROW] partials of split tiles
};

template <int BKP, int NSTP>
struct KvProducerT {
  typedef FusedAttn Kn;
  static constexpr int DKV = 512, C = 256;
  static constexpr int LINE = BKP * 2;       // bytes of one source row per step
  static constexpr int SPR = LINE / 16;      // 16-byte slots per row and step
  static constexpr int OPB = 256 * LINE;     // one operand per stage: W rows, then L rows
  static constexpr int STAGE = 2 * OPB;
  static constexpr int LDS_BYTES = NSTP * STAGE;
  static constexpr int NSTEP = DKV / BKP;
  static constexpr int ROWB = DKV * 2;       // bytes of one source row
  static constexpr int IPO = OPB / 1024 / 8; // 1 KB copies per wavefront, operand and stage
  static constexpr int IPS = 2 * IPO;
  static_assert(IPO * 8 * 1024 == OPB, "whole copies for every wavefront");
  static_assert(SPR == 4 || SPR == 8, "64- or 128-byte rows");
  // 16-byte slot c of LDS row r holds source chunk c ^ swz(r): a half-wavefront
  // reading 32 rows at one k offset then spreads over all banks.
  __device__ static int swz(int r) { return SPR == 4 ? (r >> 2) & 3 : (r >> 1) & 7; }

  __device__ static void run(const FusedArgs& a, int b, int head, int kt, char* lds) {
    const int lane = threadIdx.x % kWave, hf = lane / 32;
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int wo = wv / 4, wk = wv % 4;  // outputs wo*128 + [0,128), keys wk*64 + [0,64)
    const int64_t key_lo = static_cast<int64_t>(kt) * kFusedKeys;
    const int nvalid = static_cast<int>(a.f.S - key_lo < kFusedKeys ? a.f.S - key_lo : kFusedKeys);
    const char* wsrc = reinterpret_cast<const char*>(a.w16 + static_cast<int64_t>(head) * C * DKV);
    const char* lsrc = reinterpret_cast<const char*>(a.l16 + (static_cast<int64_t>(b) * a.f.S + key_lo) * DKV);
    int voff[IPO];
#pragma unroll
    for (int i = 0; i < IPO; ++i) {
      const int q = (i * 8 + wv) * kWave + lane, row = q / SPR;
      voff[i] = row * ROWB + ((q % SPR) ^ swz(row)) * 16;
    }
    // Step `it` into stage sb; steps past the end copy nothing (empty range)
    // so that every step issues the same number of copies.
    auto issue = [&](int it, char* sb) {
      const bool live = it < NSTEP;
      const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(wsrc + (live ? it * LINE : 0)), 0, live ? 256 * ROWB : 0, 0x00020000);
      const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(lsrc + (live ? it * LINE : 0)), 0, live ? nvalid * ROWB : 0, 0x00020000);
#pragma unroll
      for (int i = 0; i < IPO; ++i) load_lds16(rw, sb + (i * 8 + wv) * 1024, voff[i]);
#pragma unroll
      for (int i = 0; i < IPO; ++i) load_lds16(rl, sb + OPB + (i * 8 + wv) * 1024, voff[i]);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;
    // Fragment rows: W row wo*128 + 32 x + lane%32, L row wk*64 + 32 y + lane%32,
    // k = 16 s + 8 hf + [0, 8) of the step: slot 2 s + hf.
    const int sw = swz(lane % 32);
    const int oa = (wo * 128 + lane % 32) * LINE, ob = OPB + (wk * 64 + lane % 32) * LINE;
    auto compute = [&](const char* st) {
#pragma unroll
      for (int s = 0; s < BKP / 16; ++s) {
        const int slot = ((2 * s + hf) ^ sw) * 16;
        half8 af[4], bfr[2];
#pragma unroll
        for (int x = 0; x < 4; ++x) af[x] = *reinterpret_cast<const half8*>(st + oa + x * 32 * LINE + slot);
#pragma unroll
        for (int y = 0; y < 2; ++y) bfr[y] = *reinterpret_cast<const half8*>(st + ob + y * 32 * LINE + slot);
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int y = 0; y < 2; ++y) acc[x][y] = MmaF16::mma(af[x], bfr[y], acc[x][y]);
      }
    };

#pragma unroll
    for (int it = 0; it < NSTP - 1; ++it) issue(it, lds + it * STAGE);
    for (int it0 = 0; it0 < NSTEP; it0 += NSTP) {
#pragma unroll
      for (int j = 0; j < NSTP; ++j) {
        const int it = it0 + j;
        if (it >= NSTEP) break;
        wait_vmcnt<(NSTP - 2) * IPS>();  // this wavefront's copies of step `it` have landed
        __syncthreads();                 // so have every wavefront's; stage (it - 1) % NSTP is free
        issue(it + NSTP - 1, lds + ((j + NSTP - 1) % NSTP) * STAGE);
        compute(lds + j * STAGE);
      }
    }
    wait_vmcnt<0>();  // no copy into LDS outlives the task

    // acc[x][y][r]: output wo*128 + 32 x + 8 (r/4) + 4 hf + r%4, key wk*64 + 32 y + lane%32.
    // The four block images are assembled in LDS two at a time (keys
    // 128 p .. 128 p + 127): four consecutive outputs of one key go in as one
    // 8-byte write into the K rows (padded) or the V rows (16-byte chunks
    // swizzled), the keys' k_pe rows into the rope band; then the two images,
    // contiguous in global memory, leave as whole 16-byte-per-lane stores.
    static_assert(2 * Kn::BUF_BYTES <= LDS_BYTES, "two images fit in the stage ring");
    char* img = a.img + ((static_cast<int64_t>(b) * a.f.h + head) * a.nkb_img + kt * (kFusedKeys / BN)) *
                            static_cast<int64_t>(Kn::BUF_BYTES);
    const bf16_t* kp = a.k_pe + (static_cast<int64_t>(b) * a.f.S + key_lo) * 64;
    __syncthreads();  // every wavefront is done reading the stages
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (wk / 2 == p) {
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          const int key = (wk % 2) * 64 + 32 * y + lane % 32;  // within this pair of blocks
          char* blk = lds + (key / BN) * Kn::BUF_BYTES;
          const int row = key % BN;
#pragma unroll
          for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int o = 32 * x + 8 * g + 4 * hf;  // within this wavefront's 128 outputs
              typedef _Float16 half4 __attribute__((ext_vector_type(4)));
              const half4 h4 = {static_cast<half_t>(acc[x][y][4 * g]), static_cast<half_t>(acc[x][y][4 * g + 1]),
                                static_cast<half_t>(acc[x][y][4 * g + 2]), static_cast<half_t>(acc[x][y][4 * g + 3])};
              char* dst = wo == 0 ? blk + (row * Kn::LDK + o) * 2
                                  : blk + Kn::OFF_V + row * Kn::LDV * 2 + swz_block(row, o / 8) * 16 + (o % 8) * 2;
              *reinterpret_cast<half4*>(dst) = h4;
            }
        }
      }
      // The rope band of the pair: 128 keys x 8 chunks (zeros past the sequence).
#pragma unroll
      for (int i = 0; i < 128 * 8 / 512; ++i) {
        const int c = i * 512 + static_cast<int>(threadIdx.x), key = c / 8, ch = c % 8;
        const int gk = p * 128 + key;
        const u32x4 v = gk < nvalid ? *reinterpret_cast<const u32x4*>(kp + gk * 64 + ch * 8) : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(lds + (key / BN) * Kn::BUF_BYTES + Kn::OFF_R + (key % BN) * Kn::LDR * 2 + ch * 16) =
            v;
      }
      __syncthreads();
      char* gdst = img + static_cast<int64_t>(2 * p) * Kn::BUF_BYTES;
      constexpr int NCH = 2 * Kn::BUF_BYTES / 16;
      for (int c = static_cast<int>(threadIdx.x); c < NCH; c += 512)
        *reinterpret_cast<u32x4*>(gdst + c * 16) = *reinterpret_cast<const u32x4*>(lds + c * 16);
      __syncthreads();  // the LDS images are free again
    }
    // Every store of this task is complete before the tile's flag is set.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(a.done + (static_cast<int64_t>(b) * a.f.h + head) * a.n_kt + kt, 1, __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
};

typedef KvProducerT<32, 3> KvProducer;
constexpr int kImageBufs = 2;  // key-block image buffers (a third, two blocks in flight, measured no faster)
constexpr int kFusedLds = KvProducer::LDS_BYTES > kImageBufs * FusedAttn::BUF_BYTES ? KvProducer::LDS_BYTES
                                                                                   : kImageBufs * FusedAttn::BUF_BYTES;

__global__ __launch_bounds__(8 * kWave, 2) void attn_fwd_fused_kernel(FusedArgs a) {
  // One shared array for everything, the ticket words at its end: with a
  // second __shared__ object the compiler starts tracking the global -> LDS
  // copies itself and waits for each stage's copies right after issuing them
  // (the explicit waits before each barrier order them here).
  __shared__ __attribute__((aligned(1024))) char lds[kFusedLds + 16];
  int* sh = reinterpret_cast<int*>(lds + kFusedLds);
  const int part = a.parts == 8 ? static_cast<int>(blockIdx.x % 8) : 0;
  if (threadIdx.x == 0) {
    sh[0] = __hip_atomic_fetch_add(a.tickets + part, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh[1] = 1;  // cleared if a consumer gives up waiting for a key tile
  }
  __syncthreads();
  const int t = __builtin_amdgcn_readfirstlane(sh[0]);
  const int bh0 = part * a.hpp;
  // Producers in key-tile order over the queue's heads (the heads of one key
  // tile share its latent rows in L2); consumers heaviest tile first,
  // interleaved over the heads.
  if (t < a.prod_pp) {
    const int bh = bh0 + t % a.hpp;
    KvProducer::run(a, bh / a.f.h, bh % a.f.h, t / a.hpp, lds);
    return;
  }
  const int c = t - a.prod_pp;
  const int bh = bh0 + c % a.hpp, rank = c / a.hpp;
  const int e = a.n_task > 0 ? a.task[rank] : (a.f.n_qt - 1 - rank) << 2;
  const int qt = e >> 2, half = e & 3;
  const int b = bh / a.f.h, head = bh % a.f.h;
  float* partial = half == 0 ? nullptr
                             : a.part + ((static_cast<int64_t>(qt - a.q_split) * a.f.B * a.f.h + bh) * 2 + (half - 1)) *
                                            FusedAttn::BM * FusedAttn::PART_ROW;
  // Each key tile is waited for (its producer's flag) just before its first
  // block is copied, so the attention starts once the first tile is written.
  const FusedAttn::Ready rd{a.done + static_cast<int64_t>(bh) * a.n_kt, a.err, sh + 1};
  if (FusedAttn::run_images<kImageBufs>(a.f, a.img + static_cast<int64_t>(bh) * a.nkb_img * FusedAttn::BUF_BYTES, b,
                                        head, qt, lds, half, partial, rd))
    return;
  // Never expected (a producer did not finish): NaN outputs instead of a hang.
  if (half != 0) {  // a split tile: its partials are merged into o and lse, so poison them
    for (int i = threadIdx.x; i < FusedAttn::BM * FusedAttn::PART_ROW; i += 8 * kWave) partial[i] = __builtin_nanf("");
    return;
  }
  const int64_t q0 = static_cast<int64_t>(qt) * FusedAttn::BM;
  for (int i = threadIdx.x; i < FusedAttn::BM * 128; i += 8 * kWave) {
    const int64_t tq = q0 + i / 128;
    if (tq >= a.f.S) continue;
    a.f.o[((b * a.f.S + tq) * a.f.h + head) * 128 + i % 128] = __builtin_nanf("");
    if (i % 128 == 0) a.f.lse[(static_cast<int64_t>(b) * a.f.h + head) * a.f.S + tq] = __builtin_nanf("");
  }
}

// o and lse of the split query tiles from their two partials: with m = max(m1,
// m2) and a_i = 2^(m_i - m), o = (a1 O1 + a2 O2) / (a1 l1 + a2 l2) and lse =
// (m + log2(a1 l1 + a2 l2)) ln 2.  One thread per (tile, head, row, 4 columns).
__global__ __launch_bounds__(256) void fused_merge_kernel(const float* __restrict__ part, float* __restrict__ o,
                                                          float* __restrict__ lse, int q_split, int n_split, int B,
                                                          int h, int64_t S) {
  constexpr int BM = FusedAttn::BM, PR = FusedAttn::PART_ROW, DV = 128;
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per_tile = static_cast<int64_t>(BM) * (DV / 4);
  if (j >= static_cast<int64_t>(n_split) * B * h * per_tile) return;
  const int64_t tb = j / per_tile;  // (split tile, bh)
  const int r = static_cast<int>((j % per_tile) / (DV / 4)), c4 = static_cast<int>(j % (DV / 4)) * 4;
  const int bh = static_cast<int>(tb % (B * h)), qt = q_split + static_cast<int>(tb / (B * h));
  const int64_t tq = static_cast<int64_t>(qt) * BM + r;
  if (tq >= S) return;
  const float* p1 = part + (tb * 2) * BM * PR + static_cast<int64_t>(r) * PR;
  const float* p2 = p1 + static_cast<int64_t>(BM) * PR;
  const float m1 = p1[DV], l1 = p1[DV + 1], m2 = p2[DV], l2 = p2[DV + 1];
  const float m = fmaxf(m1, m2);
  const float a1 = __builtin_amdgcn_exp2f(m1 - m), a2 = __builtin_amdgcn_exp2f(m2 - m);
  const float l = a1 * l1 + a2 * l2, inv = 1.0f / l;
  const f32x4 x = *reinterpret_cast<const f32x4*>(p1 + c4), y = *reinterpret_cast<const f32x4*>(p2 + c4);
  const int b = bh / h, head = bh % h;
  *reinterpret_cast<f32x4*>(o + ((b * S + tq) * h + head) * DV + c4) =
      f32x4{(a1 * x[0] + a2 * y[0]) * inv, (a1 * x[1] + a2 * y[1]) * inv, (a1 * x[2] + a2 * y[2]) * inv,
            (a1 * x[3] + a2 * y[3]) * inv};
  if (c4 == 0) lse[(static_cast<int64_t>(b) * h + head) * S + tq] = (m + log2f(l)) * 0.69314718055994531f;
}

// The fused forward's prep: workgroups [0, nb_norm) normalise 4 latent rows
// each into fp16 (one wavefront per row, the RMSNorm of the plain forward);
// the next nb_w convert 2048 elements each of the W_kv_b head shard to fp16;
// the last one clears the tickets, the error word and the per-head counts.
__global__ __launch_bounds__(256) void fused_prep_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ gamma,
                                                         half_t* __restrict__ l16, int64_t T, float eps, int nb_norm,
                                                         const bf16_t* __restrict__ w, half_t* __restrict__ w16,
                                                         int64_t n_w8, int nb_w, int* __restrict__ counters,
                                                         int n_cnt) {
  const int blk = static_cast<int>(blockIdx.x);
  if (blk < nb_norm) {
    const int lane = threadIdx.x % kWave;
    const int64_t t = static_cast<int64_t>(blk) * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    const u16x8 xr = *reinterpret_cast<const u16x8*>(x + t * 512 + lane * 8);
    const u16x8 gr = *reinterpret_cast<const u16x8*>(gamma + lane * 8);
    float v[8];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = bf16_to_f32(xr[j]);
      ss += v[j] * v[j];
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / 512.0f + eps);
    half8 out;
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = static_cast<half_t>(bf16_to_f32(gr[j]) * (v[j] * r));
    *reinterpret_cast<half8*>(l16 + t * 512 + lane * 8) = out;
  } else if (blk < nb_norm + nb_w) {
    const int64_t i = static_cast<int64_t>(blk - nb_norm) * 256 + threadIdx.x;
    if (i >= n_w8) return;
    const u16x8 wr = *reinterpret_cast<const u16x8*>(w + i * 8);
    half8 out;
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = static_cast<half_t>(bf16_to_f32(wr[j]));
    *reinterpret_cast<half8*>(w16 + i * 8) = out;
  } else {
    for (int i = threadIdx.x; i < n_cnt; i += 256) counters[i] = 0;
  }
}

// Workspace of the fused forward: counters | L16 | W16 | images.
struct FusedLayout {
  size_t cnt, l16, w16, img, part, total;
  int n_cnt, n_kt, nkb_img;
  int n_qt, q_split, n_task;  // q_split == n_qt: no tile is split
  int task[kMaxTasks];
};

// Which query tiles run as two tasks, and the consumer task order.  Tile qt
// has nkb(qt) key blocks; with the work spread evenly each CU gets W / kCUs
// blocks (W: all tiles of all heads), and a tile larger than that would set
// the time alone.  Such tiles (qt >= 1, so both halves have blocks) are split
// at split_block() into two tasks, when the per-head task list fits kMaxTasks
// (short sequences only: at S = 16384 with 16 heads, or S = 4096 with 128, no
// tile is split).  Tasks run heaviest first.
void fused_tasks(const Shape& s, FusedLayout& L) {
  constexpr int BM = FusedAttn::BM;
  L.n_qt = static_cast<int>((s.S + BM - 1) / BM);
  L.q_split = L.n_qt;
  L.n_task = 0;
  if (2 * L.n_qt > kMaxTasks) return;
  auto nkb = [&](int qt) {
    const int64_t kend = std::min<int64_t>(static_cast<int64_t>(qt + 1) * BM, s.S);
    return static_cast<int>((kend + BN - 1) / BN);
  };
  auto nall = [&](int qt) { return std::min(static_cast<int>((static_cast<int64_t>(qt) * BM + 31) / BN) + 1, nkb(qt)); };
  int64_t W = 0;
  for (int qt = 0; qt < L.n_qt; ++qt) W += nkb(qt);
  W *= s.B * s.h;
  const double avg = static_cast<double>(W) / kCUs;
  int q = L.n_qt;
  while (q > 1 && nkb(q - 1) > avg) --q;  // nkb grows with qt
  if (q == L.n_qt) return;
  L.q_split = q;
  struct T { int w, qt, part; };
  T t[kMaxTasks];
  int n = 0;
  for (int qt = 0; qt < L.n_qt; ++qt) {
    if (qt < q) {
      t[n++] = {nkb(qt), qt, 0};
    } else {
      const int mid = nall(qt) / 2;
      t[n++] = {mid, qt, 1};
      t[n++] = {nkb(qt) - mid, qt, 2};
    }
  }
  std::sort(t, t + n, [](const T& x, const T& y) {
    return x.w != y.w ? x.w > y.w : (x.qt != y.qt ? x.qt > y.qt : x.part < y.part);
  });
  for (int i = 0; i < n; ++i) L.task[i] = t[i].qt << 2 | t[i].part;
  L.n_task = n;
}

FusedLayout fused_layout(const Shape& s);

size_t r256(size_t b) { return (b + 255) & ~size_t(255); }

FusedLayout fused_layout(const Shape& s) {
  FusedLayout L;
  L.n_kt = static_cast<int>((s.S + kFusedKeys - 1) / kFusedKeys);
  L.nkb_img = L.n_kt * (kFusedKeys / BN);
  L.n_cnt = 16 + static_cast<int>(s.B) * s.h * L.n_kt;
  size_t off = 0;
  L.cnt = off;
  off += r256(static_cast<size_t>(L.n_cnt) * 4);
  L.l16 = off;
  off += r256(static_cast<size_t>(s.T) * 512 * 2);
  L.w16 = off;
  off += r256(static_cast<size_t>(s.h) * 256 * 512 * 2);
  L.img = off;
  off += static_cast<size_t>(s.B) * s.h * L.nkb_img * FusedAttn::BUF_BYTES;
  fused_tasks(s, L);
  L.part = off;
  off += static_cast<size_t>(L.n_qt - L.q_split) * s.B * s.h * 2 * FusedAttn::BM * FusedAttn::PART_ROW * 4;
  L.total = off;
  return L;
}

bool fused_supported(const Shape& s) {
  return s.bf16 && !s.split && s.d_kv == 512 && s.d_nope == 128 && s.d_rope == 64 && s.d_v == 128;
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

namespace laga {

size_t fused_fwd_workspace_bytes(const Shape& s) { return fused_supported(s) ? fused_layout(s).total : 0; }

hipError_t launch_attn_fwd_fused(const Shape& s, const void* q, const void* latent, const void* gamma,
                                 const void* k_pe, const void* w, float* o, float* lse, void* workspace,
                                 hipStream_t st) {
  if (!fused_supported(s)) return hipErrorNotSupported;
  const FusedLayout L = fused_layout(s);
  char* ws = static_cast<char*>(workspace);
  int* counters = reinterpret_cast<int*>(ws + L.cnt);
  half_t* l16 = reinterpret_cast<half_t*>(ws + L.l16);
  half_t* w16 = reinterpret_cast<half_t*>(ws + L.w16);
  const int nb_norm = static_cast<int>((s.T + 3) / 4);
  const int64_t n_w8 = static_cast<int64_t>(s.h) * 256 * 512 / 8;
  const int nb_w = static_cast<int>((n_w8 + 255) / 256);
  const bf16_t* wr = static_cast<const bf16_t*>(w) + static_cast<int64_t>(s.head_lo) * 256 * 512;
  hipLaunchKernelGGL(fused_prep_kernel, dim3(static_cast<unsigned>(nb_norm + nb_w + 1)), dim3(256), 0, st,
                     static_cast<const bf16_t*>(latent), static_cast<const bf16_t*>(gamma), l16, s.T, s.eps, nb_norm,
                     wr, w16, n_w8, nb_w, counters, L.n_cnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  FusedArgs a;
  a.f.q = q; a.f.k_nope = nullptr; a.f.k_pe = nullptr; a.f.v = nullptr; a.f.o = o; a.f.lse = lse;
  a.f.S = s.S; a.f.B = static_cast<int>(s.B); a.f.h = s.h;
  a.f.plane_k = 0; a.f.plane_v = 0;
  a.f.n_qt = static_cast<int>((s.S + FusedAttn::BM - 1) / FusedAttn::BM);
  a.f.scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(s.d_nope + s.d_rope));
  a.l16 = l16; a.w16 = w16; a.k_pe = static_cast<const bf16_t*>(k_pe);
  a.img = ws + L.img;
  a.tickets = counters;
  a.err = counters + 8;
  a.done = counters + 16;
  a.n_kt = L.n_kt;
  a.nkb_img = L.nkb_img;
  const int nbh = static_cast<int>(s.B) * s.h;
  a.parts = nbh % 8 == 0 ? 8 : 1;
  a.hpp = nbh / a.parts;
  a.prod_pp = a.hpp * a.n_kt;
  a.n_task = L.n_task;
  a.q_split = L.q_split;
  for (int i = 0; i < kMaxTasks; ++i) a.task[i] = i < L.n_task ? L.task[i] : 0;
  a.part = reinterpret_cast<float*>(ws + L.part);
  const int tasks = L.n_task > 0 ? L.n_task : a.f.n_qt;  // consumer tasks per head
  const int64_t grid = static_cast<int64_t>(a.parts) * a.hpp * (a.n_kt + tasks);
  if (grid >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_fwd_fused_kernel, dim3(static_cast<unsigned>(grid)), dim3(8 * kWave), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess || L.n_task == 0) return e;
  const int n_split = L.n_qt - L.q_split;
  const int64_t nthr = static_cast<int64_t>(n_split) * s.B * s.h * FusedAttn::BM * 32;
  hipLaunchKernelGGL(fused_merge_kernel, dim3(static_cast<unsigned>((nthr + 255) / 256)), dim3(256), 0, st, a.part, o,
                     lse, L.q_split, n_split, static_cast<int>(s.B), s.h, s.S);
  return hipGetLastError();
}

}  // namespace laga
