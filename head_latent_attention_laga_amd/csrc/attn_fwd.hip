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

    int64_t kend = q0 + BM;
    if (kend > a.S) kend = a.S;
    const int nkb = static_cast<int>((kend + BN - 1) / BN);
    Regs R;
    load_block(a, b, head, 0, R);

    // Q fragments (B operand): query tq, dims hf*KPL + s*K + [0, KPL).
    State st_;
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

    // Blocks with key0 <= q0 + 31 are computed by every wavefront; the last
    // few (above the lower wavefronts' diagonals) are skipped per wavefront.
    int nall = static_cast<int>((q0 + 31) / BN) + 1;
    if (nall > nkb) nall = nkb;
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

    if (qvalid) {
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
        a.lse[(static_cast<int64_t>(b) * a.h + head) * a.S + tq] =
            (st_.m_run + log2f(st_.l_run)) * 0.69314718055994531f;
    }
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
