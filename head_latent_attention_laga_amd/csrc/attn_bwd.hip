// Causal attention backward of one rank's head shard [LAGA §5.2: gradients of
// the rank-local computation; the k_pe band's gradient is the sum over the
// local heads; the K/V gradients are folded back through W_kv_b elsewhere].
//
// With P = softmax(s), s = q.K^T / sqrt(d_qk) (causal), and upstream dO:
//   delta[t] = sum_c dO[t,c] o[t,c]                (bwd_prep_kernel, bwd_dot_kernel)
//   dV  = P^T dO,  dP = dO V^T,  dS = P * (dP - delta)
//   dK  = dS^T q / sqrt(d_qk)  -> dk_nope = dK[:, :d_nope], dk_pe = sum_i dK[:, d_nope:]
//   dq  = dS K / sqrt(d_qk)
// P is rebuilt from the forward's lse, never stored.
//
// Two kernels, neither of which holds or writes an S x S quantity, so the
// backward's memory grows linearly with S:
//  * dkdv: a workgroup of 4 wavefronts owns 128 keys of one head (32 per
//    wavefront; K and V held in registers as B operands) and walks the
//    queries from its diagonal to the end, 32 at a time.  q and dO blocks
//    stream through double-buffered LDS (buffer loads in flight in registers
//    while the previous block is computed), one tile each, read both as
//    16-byte rows (the A operands of S = q K^T and dP = dO V^T) and with
//    transposing reads (the A operands of dK^T = q^T dS and dV^T = dO^T P).
//    The 32x32 accumulators of S / dP hold one key per lane column, which is
//    the B-operand layout of the dK / dV products, so P and dS feed them
//    straight from registers.
//  * dq (attn_bwd_dq.hip): query-stationary, like the forward; it recomputes
//    P and dS for its queries from lse and delta.
// dk_pe is written per head into a workspace and summed over heads in a fixed
// order (deterministic, no atomics).
//
// Precision (LAGA_OPERANDS_SPLIT): the products that feed dK, dV and hence
// dW_kv_b, dLatent and dgamma use K, V, P and dS as hi + lo pairs (q and dO
// are exact in fp16): S and dP add the low planes of K and V as e4m3 products
// against e4m3 copies of q_nope and dO, each query row scaled by its own power
// of two (the row's E8M0 byte is the A operand's scale), and dK_nope, dV take P
// and dS as fp16 hi + lo (dk_pe the hi term of dS).  The float32 instantiation
// uses fp32 MFMAs.
#include "attn_bwd_common.hpp"

namespace laga {
namespace {
using namespace bwd;

// ============================================================ dK / dV kernel
template <class InT, class M, int NS, int DN, int DR, int DV>
struct Dkdv {
  typedef typename M::elem E;
  typedef typename M::frag F;
  static constexpr int DQK = DN + DR, C = DN + DV;
  static constexpr int BQ = 32, BK = 128;
  static constexpr bool TR = M::KPL == 8;  // 16-bit operands: separate transposed-read tiles
  // One q tile and one dO tile per block, read both as rows and transposed.
  // 16-bit operands: row pitches of 16 (mod 32) dwords, the 16-byte chunks
  // of row r XOR-swizzled by sw(r) = (r / 4) mod 4.  A 16-byte row read
  // serves 16 rows at once: r mod 4 picks one of four 16-dword windows of the
  // 64 banks and sw(r) one chunk inside it, so the 16 rows hit distinct
  // banks; the four consecutive rows (one sw) of a transposing read fall in
  // the four windows.  fp32: rows padded by 4 elements.
  static constexpr int sw_pitch(int n) {
    int d = n / 2;
    while (d % 32 != 16) ++d;
    return 2 * d;
  }
  static constexpr int LQR = TR ? sw_pitch(DQK) : DQK + 4, LOR = TR ? sw_pitch(DV) : DV + 4;
  static_assert(!TR || (DQK % 32 == 0 && DV % 32 == 0), "whole groups of four chunks per row");
  static constexpr int QR_B = BQ * LQR * sizeof(E), OR_B = BQ * LOR * sizeof(E);
  // Split operands: the low terms S_lo = q8 K_lo^T and dP_lo = dO8 V_lo^T run
  // as e4m3 products; e4m3 q_nope / dO rows (16-byte row reads, 16-byte pad)
  // and their per-query E8M0 scales are staged with each block.
  static constexpr bool LO8 = NS == 2;
  static constexpr int P8 = 16;  // row padding (bytes) of the e4m3 tiles
  static constexpr int Q8_B = LO8 ? BQ * (DN + P8) : 0, O8_B = LO8 ? BQ * (DV + P8) : 0;
  static constexpr int OFF_Q8 = QR_B + OR_B, OFF_O8 = OFF_Q8 + Q8_B, OFF_ST = OFF_O8 + O8_B;
  static constexpr int BUF_BYTES = OFF_ST + (LO8 ? 4 : 2) * BQ * 4;  // lse, delta [, q / dO scales]
  static constexpr int LDS_BYTES = 2 * BUF_BYTES;
  static constexpr int KS_QK = DQK / M::K, KS_N = DN / M::K, KS_V = DV / M::K;
  static constexpr int KS8_N = DN / 64, KS8_V = DV / 64;  // e4m3 atoms (K = 64)
  static_assert(!LO8 || (sizeof(E) == 2 && DN % 64 == 0 && DV % 64 == 0 && BQ * DN / 16 == kThreads &&
                         BQ * DV / 16 == kThreads), "e4m3 staging: one 16-byte chunk per thread");
  static constexpr int STEPS = BQ / M::K;
  static constexpr int NKT = (DQK + 31) / 32, NVT = DV / 32;
  // Staging: 16-byte chunks of the input rows.
  static constexpr int IPC = 16 / sizeof(InT);
  static constexpr int QCH = BQ * DQK / IPC, OCH = BQ * DV / IPC;
  static constexpr int IQ = (QCH + kThreads - 1) / kThreads, IO = (OCH + kThreads - 1) / kThreads;
  static_assert(DQK % IPC == 0 && DV % IPC == 0, "rows of whole chunks");

  struct Regs {
    u32x4 q[IQ]; u32x4 o[IO]; float lse2, dlt;  // lse2: natural-log lse until stored
    u32x4 q8, o8; int qs, os;                    // split operands only
    float dsc; int dsh;                          // 2^g and g of the dO scale (set once)
  };

  // Stationary operands of one wavefront: its 32 keys' K (nope hi plane, rope)
  // and V (hi plane) fragments, and for split operands the e4m3 low planes
  // of K_nope and V (B operands of the e4m3 products), all in registers.
  struct Stat {
    F kf[KS_N], kr[KS_QK - KS_N], vf[KS_V];
    i32x8 k8[LO8 ? KS8_N : 1], v8[LO8 ? KS8_V : 1];
  };
  struct Acc { f32x16 dk[NKT], dvt[NVT]; };

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
      if (QCH % kThreads == 0 || c < QCH) R.q[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, r * qrow_b + j * 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < IO; ++i) {
      const int c = i * kThreads + tid;
      const int r = c / (DV / IPC), j = c % (DV / IPC);
      if (OCH % kThreads == 0 || c < OCH) R.o[i] = __builtin_amdgcn_raw_buffer_load_b128(ro, r * orow_b + j * 16, 0, 0);
    }
    // Statistics of the block's queries; rows past the sequence read as zero.
    const int t = tid % BQ;
    const int64_t si0 = (static_cast<int64_t>(b) * a.h + head) * a.S + q0;
    R.lse2 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc(a.lse + si0, nq * 4), t * 4, 0, 0));
    R.dlt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc(a.delta + si0, nq * 4), t * 4, 0, 0));
    if constexpr (LO8) {
      const int r = tid / (DN / 16), j = tid % (DN / 16);
      R.q8 = __builtin_amdgcn_raw_buffer_load_b128(rsrc(a.q8 + row0 * DN, nq * a.h * DN), r * a.h * DN + j * 16, 0, 0);
      const int ro8 = tid / (DV / 16), jo8 = tid % (DV / 16);
      R.o8 = __builtin_amdgcn_raw_buffer_load_b128(rsrc(a.do8 + row0 * DV, nq * a.h * DV), ro8 * a.h * DV + jo8 * 16,
                                                   0, 0);
      R.qs = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(rsrc(a.qsc + si0, nq * 4), t * 4, 0, 0));
      R.os = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(rsrc(a.osc + si0, nq * 4), t * 4, 0, 0));
    }
  }

  // Offset in its row of row r's 16-byte chunk that starts at element el.
  __device__ static int chunk_at(int r, int el) { return TR ? 8 * ((el / 8) ^ ((r / 4) % 4)) : el; }

  __device__ static void store(const Regs& R, char* buf) {
    E* Qr = reinterpret_cast<E*>(buf);
    E* Or = reinterpret_cast<E*>(buf + QR_B);
    float* st = reinterpret_cast<float*>(buf + OFF_ST);
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < IQ; ++i) {
      const int c = i * kThreads + tid;
      if (QCH % kThreads != 0 && c >= QCH) continue;
      const int r = c / (DQK / IPC), col = (c % (DQK / IPC)) * IPC;
      E tmp[IPC];
      convert_chunk<E, InT>(R.q[i], tmp);
#pragma unroll
      for (int j = 0; j < IPC; j += 16 / sizeof(E)) {
        *reinterpret_cast<u32x4*>(Qr + r * LQR + chunk_at(r, col + j)) = *reinterpret_cast<u32x4*>(tmp + j);
      }
    }
#pragma unroll
    for (int i = 0; i < IO; ++i) {
      const int c = i * kThreads + tid;
      if (OCH % kThreads != 0 && c >= OCH) continue;
      const int r = c / (DV / IPC), col = (c % (DV / IPC)) * IPC;
      E tmp[IPC];
      convert_chunk<E, InT>(R.o[i], tmp);
#pragma unroll
      for (int j = 0; j < IPC; j += 16 / sizeof(E)) {
        *reinterpret_cast<u32x4*>(Or + r * LOR + chunk_at(r, col + j)) = *reinterpret_cast<u32x4*>(tmp + j);
      }
    }
    if (tid < BQ) {
      st[tid] = R.lse2 * kLog2e;
      st[BQ + tid] = R.dlt * R.dsc;  // delta in the units of the scaled dO
    }
    if constexpr (LO8) {
      const int r = tid / (DN / 16), j = tid % (DN / 16);
      *reinterpret_cast<u32x4*>(buf + OFF_Q8 + r * (DN + P8) + j * 16) = R.q8;
      const int ro8 = tid / (DV / 16), jo8 = tid % (DV / 16);
      *reinterpret_cast<u32x4*>(buf + OFF_O8 + ro8 * (DV + P8) + jo8 * 16) = R.o8;
      if (tid < BQ) {
        reinterpret_cast<int*>(st)[2 * BQ + tid] = R.qs;
        // dO8 * 2^-s_row feeds dP in the scaled units of the fp16 part: 2^(g - s_row).
        const int e = R.os + R.dsh;
        reinterpret_cast<int*>(st)[3 * BQ + tid] = e < 0 ? 0 : (e > 254 ? 254 : e);
      }
    }
  }

  // 32 e4m3 bytes of an LDS row (the A or B operand of one e4m3 atom).
  __device__ static i32x8 frag8(const char* p) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(p), y = *reinterpret_cast<const u32x4*>(p + 16);
    return i32x8{static_cast<int>(x[0]), static_cast<int>(x[1]), static_cast<int>(x[2]), static_cast<int>(x[3]),
                 static_cast<int>(y[0]), static_cast<int>(y[1]), static_cast<int>(y[2]), static_cast<int>(y[3])};
  }

  // A operand of a product whose k index runs over the queries of the block:
  // rows n0 + lane%32 of the transposed tile (dims), queries of accumulator
  // registers st*KPL .. (see acc_key_col).
  __device__ static F tr_frag(const E* T, int ld, int st, int n0) {
    if constexpr (TR) {
      // tr_frag_acc's lanes on the swizzled rows: rows 16 st + 4 hf + s / 4
      // (sw = hf) and the same + 8 (sw = hf ^ 2); n0 spans whole chunk groups.
      const int lane = threadIdx.x % kWave;
      const int g = lane / 16, s = lane % 16, hf = lane / 32;
      const int row = st * 16 + 4 * hf + s / 4, blk = 2 * (g % 2) + (s % 4) / 2;
      const s16x4 lo = ds_read_tr16(T + row * ld + n0 + 8 * (blk ^ hf) + 4 * (s % 2));
      const s16x4 hi = ds_read_tr16(T + (row + 8) * ld + n0 + 8 * (blk ^ hf ^ 2) + 4 * (s % 2));
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      const s16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return __builtin_bit_cast(F, r);
    } else {
      const int lane = threadIdx.x % kWave;
      const int qi = 8 * (st / 4) + 4 * (lane / 32) + (st % 4);
      return T[qi * ld + n0 + lane % 32];
    }
  }

  // Fragment of a stationary K / V row held in memory as E (16-byte loads) or
  // as the input type (converted).
  template <class Src>
  __device__ static F row_frag(const Src* p) {
    if constexpr (std::is_same<Src, E>::value && sizeof(F) == 16) {
      return *reinterpret_cast<const F*>(p);
    } else {
      E tmp[M::KPL];
#pragma unroll
      for (int j = 0; j < M::KPL; ++j) tmp[j] = M::from_f32(to_f32(p[j]));
      return *reinterpret_cast<F*>(tmp);
    }
  }

  static constexpr int kAhead = 6;  // operand reads in flight ahead of the score products

  // v (accumulator order r) as NS-term MFMA operands: out[r / KPL][q][r % KPL].
  __device__ static void split16(const float (&v)[16], E (&out)[STEPS][NS][M::KPL]) {
    if constexpr (std::is_same<E, half_t>::value && NS == 2) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        half2_t hi, lo;
        split_f16_pair(v[r], v[r + 1], hi, lo);
        out[r / M::KPL][0][r % M::KPL] = hi[0];
        out[r / M::KPL][0][r % M::KPL + 1] = hi[1];
        out[r / M::KPL][1][r % M::KPL] = lo[0];
        out[r / M::KPL][1][r % M::KPL + 1] = lo[1];
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        E t[NS];
        split_to<M, NS>(v[r], t);
#pragma unroll
        for (int q = 0; q < NS; ++q) out[r / M::KPL][q][r % M::KPL] = t[q];
      }
    }
  }

  // One block of BQ queries starting at q0 against the wavefront's 32 keys
  // from wk0 (lane column `col`).  MASK: the block may cross the causal
  // diagonal or the end of the sequence (and may lie wholly before the keys).
  template <bool MASK>
  __device__ static void block(const BwdArgs& a, const char* buf, int64_t q0, int64_t wk0, const Stat& K,
                               Acc& acc) {
    const int lane = threadIdx.x % kWave;
    const int hf = lane / 32, col = lane % 32;
    if (MASK && q0 + BQ - 1 < wk0) return;  // every query of the block precedes these keys
    const E* Qr = reinterpret_cast<const E*>(buf);
    const E* Or = reinterpret_cast<const E*>(buf + QR_B);
    const float* st = reinterpret_cast<const float*>(buf + OFF_ST);
    // The rows' lse and delta, read before the products: issued next to their
    // use they were waited for in the middle of the dP chain.
    f32x4 l4[4], d4[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      l4[g] = *reinterpret_cast<const f32x4*>(st + 8 * g + 4 * hf);
      d4[g] = *reinterpret_cast<const f32x4*>(st + BQ + 8 * g + 4 * hf);
    }

    // S[q, key], dP[q, key]: rows = queries 8g + 4hf + i, column = key.  The
    // chains run one after the other so that the vector work on each result
    // (P from S, dS from dP) overlaps the next chain of products:
    //   S | dP + P | dV + dS | dK
    f32x16 sc, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) { sc[r] = 0.f; dp[r] = 0.f; }
    if constexpr (LO8) {
      // One chain of 16-byte operand reads feeds both score products:
      //   q8 halves (2 KS8_N) | q rows (KS_QK) | dO8 halves (2 KS8_V) | dO rows (KS_V)
      // (the longer e4m3 products first, so each chain ends on a short one)
      // the low terms adding (q8 * 2^-s_q) . (K_lo * 2^-kLoShift)^T with the
      // per-query scale in the A operand (dP likewise).
      const int qs = reinterpret_cast<const int*>(st)[2 * BQ + col];
      const int os = reinterpret_cast<const int*>(st)[3 * BQ + col];
      // Row reads of 16-byte chunk 2 i + hf (K step i): chunk x ^ 2 (i % 2) of
      // group i / 2, x = hf ^ sw(col).
      static_assert(TR && M::K == 16 && M::KPL == 8, "16-bit split operands");
      const int x = hf ^ ((col / 4) % 4);
      const E* qrow[2] = {Qr + col * LQR + 8 * x, Qr + col * LQR + 8 * (x ^ 2)};
      const E* orow[2] = {Or + col * LOR + 8 * x, Or + col * LOR + 8 * (x ^ 2)};
      const char* q8row = buf + OFF_Q8 + col * (DN + P8) + 32 * hf;
      const char* o8row = buf + OFF_O8 + col * (DV + P8) + 32 * hf;
      constexpr int N8Q = 2 * KS8_N, N8O = 2 * KS8_V;
      u32x4 half8lo;  // first 16 bytes of an e4m3 fragment
      auto join = [](u32x4 x, u32x4 y) {
        return i32x8{static_cast<int>(x[0]), static_cast<int>(x[1]), static_cast<int>(x[2]), static_cast<int>(x[3]),
                     static_cast<int>(y[0]), static_cast<int>(y[1]), static_cast<int>(y[2]), static_cast<int>(y[3])};
      };
      pipelined<N8Q + KS_QK + N8O + KS_V, kAhead, u32x4>(
          [&](int i) {
            if (i < N8Q) return *reinterpret_cast<const u32x4*>(q8row + 64 * (i / 2) + 16 * (i % 2));
            i -= N8Q;
            if (i < KS_QK) return *reinterpret_cast<const u32x4*>(qrow[i % 2] + 32 * (i / 2));
            i -= KS_QK;
            if (i < N8O) return *reinterpret_cast<const u32x4*>(o8row + 64 * (i / 2) + 16 * (i % 2));
            i -= N8O;
            return *reinterpret_cast<const u32x4*>(orow[i % 2] + 32 * (i / 2));
          },
          [&](int i, const u32x4& f) {
            if (i < N8Q) {
              if (i % 2 == 0) half8lo = f;
              else sc = mma_e4m3(join(half8lo, f), K.k8[i / 2], sc, qs, 127 - kLoShift);
              return;
            }
            i -= N8Q;
            if (i < KS_QK) {
              sc = M::mma(__builtin_bit_cast(F, f), i < KS_N ? K.kf[i] : K.kr[i - KS_N], sc);
              return;
            }
            i -= KS_QK;
            if (i < N8O) {
              if (i % 2 == 0) half8lo = f;
              else dp = mma_e4m3(join(half8lo, f), K.v8[i / 2], dp, os, 127 - kLoShift);
              return;
            }
            i -= N8O;
            dp = M::mma(__builtin_bit_cast(F, f), K.vf[i], dp);
          });
    } else {
      static_assert(!TR, "16-bit operands are split");
      const E* qrow = Qr + col * LQR + hf * M::KPL;
      const E* orow = Or + col * LOR + hf * M::KPL;
#pragma unroll
      for (int s = 0; s < KS_N; ++s) sc = M::mma(lds_frag<M>(qrow + s * M::K), K.kf[s], sc);
#pragma unroll
      for (int s = KS_N; s < KS_QK; ++s) sc = M::mma(lds_frag<M>(qrow + s * M::K), K.kr[s - KS_N], sc);
#pragma unroll
      for (int s = 0; s < KS_V; ++s) dp = M::mma(lds_frag<M>(orow + s * M::K), K.vf[s], dp);
    }

    // P = exp(s - lse) per query row of the block, split into NS terms
    // grouped by MFMA step (k = queries of accumulator registers).
    const int rel = static_cast<int>(wk0 - q0) + col;  // key - q0
    const int nq = static_cast<int>(a.S - q0 < BQ ? a.S - q0 : BQ);
    float pv[16];
    E ph[STEPS][NS][M::KPL];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        float p = __builtin_amdgcn_exp2f(fmaf(sc[r], a.scale_log2, -l4[g][i]));
        if constexpr (MASK) {
          const int qi = 8 * g + 4 * hf + i;
          if (rel > qi || qi >= nq) p = 0.f;
        }
        pv[r] = p;
      }
    }
    split16(pv, ph);
    // dV^T[dv, key] += dO^T P   (k = queries)
#pragma unroll
    for (int stp = 0; stp < STEPS; ++stp) {
      F oa[NVT];
#pragma unroll
      for (int n = 0; n < NVT; ++n) oa[n] = tr_frag(Or, LOR, stp, n * 32);
#pragma unroll
      for (int q = 0; q < NS; ++q)
#pragma unroll
        for (int n = 0; n < NVT; ++n) acc.dvt[n] = M::mma(oa[n], *reinterpret_cast<F*>(ph[stp][q]), acc.dvt[n]);
    }

    // dS = P (dP - delta), split the same way.
    E dh[STEPS][NS][M::KPL];
    float dsv[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int i = 0; i < 4; ++i) dsv[4 * g + i] = pv[4 * g + i] * (dp[4 * g + i] - d4[g][i]);
    }
    split16(dsv, dh);
    // dK^T[d, key] += q^T dS   (k = queries).  The rope rows (d >= DN) give
    // dk_pe, which reaches no other gradient (not dLatent, dW_kv_b or dgamma,
    // whose bars need dS as a hi + lo pair): they take the hi term of dS only,
    // as dq does.
#pragma unroll
    for (int stp = 0; stp < STEPS; ++stp) {
      F qa[NKT];
#pragma unroll
      for (int n = 0; n < NKT; ++n) qa[n] = tr_frag(Qr, LQR, stp, n * 32);
#pragma unroll
      for (int q = 0; q < NS; ++q)
#pragma unroll
        for (int n = 0; n < NKT; ++n) {
          if (q > 0 && n * 32 >= DN) continue;
          acc.dk[n] = M::mma(qa[n], *reinterpret_cast<F*>(dh[stp][q]), acc.dk[n]);
        }
    }
  }

  // Publish the staged block `it` into `buf` (the buffer of its parity),
  // start loading the next one, compute.
  template <bool MASK>
  __device__ static void step(const BwdArgs& a, char* buf, int it, int nqb, int b, int head, int64_t k0,
                              int64_t wk0, Regs& R, const Stat& K, Acc& acc) {
    const int64_t q0 = k0 + static_cast<int64_t>(it) * BQ;
    store(R, buf);
    __syncthreads();
    if (it + 1 < nqb) load(a, b, head, q0 + BQ, R);
    block<MASK>(a, buf, q0, wk0, K, acc);
  }

  __device__ static void run(const BwdArgs& a, char* lds) {
    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
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
    // Keys past the sequence use row 0's values: every product they enter is
    // masked and their gradients are not stored.
    const int64_t kc = kvalid ? key : 0;

    Stat K;
    const E* kn = static_cast<const E*>(a.k_nope) + ((b * a.S + kc) * a.h + head) * DN;
    const E* vg = static_cast<const E*>(a.v) + ((b * a.S + kc) * a.h + head) * DV;
    const InT* kp = static_cast<const InT*>(a.k_pe) + (b * a.S + kc) * DR;
#pragma unroll
    for (int s = 0; s < KS_N; ++s) K.kf[s] = row_frag(kn + s * M::K + hf * M::KPL);
#pragma unroll
    for (int s = 0; s < KS_V; ++s) K.vf[s] = row_frag(vg + s * M::K + hf * M::KPL);
#pragma unroll
    for (int s = 0; s < KS_QK - KS_N; ++s) K.kr[s] = row_frag(kp + s * M::K + hf * M::KPL);
    if constexpr (LO8) {
      // e4m3 low planes (after the fp16 planes) of this lane's key: bytes
      // 64 s + 32 hf + [0, 32) of its K_nope and V rows.
      const uint8_t* k8 = static_cast<const uint8_t*>(a.k_nope) + a.plane_k * sizeof(E) +
                          ((b * a.S + kc) * a.h + head) * DN + 32 * hf;
      const uint8_t* v8 = static_cast<const uint8_t*>(a.v) + a.plane_v * sizeof(E) +
                          ((b * a.S + kc) * a.h + head) * DV + 32 * hf;
#pragma unroll
      for (int s = 0; s < KS8_N; ++s) K.k8[s] = *reinterpret_cast<const i32x8*>(k8 + 64 * s);
#pragma unroll
      for (int s = 0; s < KS8_V; ++s) K.v8[s] = *reinterpret_cast<const i32x8*>(v8 + 64 * s);
    }

    Acc acc;
#pragma unroll
    for (int n = 0; n < NKT; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.dk[n][r] = 0.f;
#pragma unroll
    for (int n = 0; n < NVT; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.dvt[n][r] = 0.f;

    // Query blocks from the diagonal: the first BK / BQ cross the workgroup's
    // keys, the ones after them up to the last whole block need no mask, and
    // a ragged last block is masked again.
    const int nqb = static_cast<int>((a.S - k0 + BQ - 1) / BQ);
    const int ndiag = nqb < BK / BQ ? nqb : BK / BQ;
    static_assert((BK / BQ) % 2 == 0, "the unmasked blocks start at an even index");
    const int nfull = static_cast<int>((a.S - k0) / BQ);
    const int nmid = nfull > ndiag ? nfull : ndiag;
    Regs R;
    R.dsh = do_shift_of(a);
    R.dsc = pow2i(R.dsh);
    load(a, b, head, k0, R);
    int it = 0;
    for (; it < ndiag; ++it) step<true>(a, lds + (it & 1) * BUF_BYTES, it, nqb, b, head, k0, wk0, R, K, acc);
    // The unmasked blocks start at an even index (ndiag = BK / BQ whenever
    // there are any), so unrolled by two each step names its buffer as a
    // constant offset and the LDS addresses fold into immediates.
    for (; it + 1 < nmid; it += 2) {
      step<false>(a, lds, it, nqb, b, head, k0, wk0, R, K, acc);
      step<false>(a, lds + BUF_BYTES, it + 1, nqb, b, head, k0, wk0, R, K, acc);
    }
    for (; it < nmid; ++it) step<false>(a, lds + (it & 1) * BUF_BYTES, it, nqb, b, head, k0, wk0, R, K, acc);
    for (; it < nqb; ++it) step<true>(a, lds + (it & 1) * BUF_BYTES, it, nqb, b, head, k0, wk0, R, K, acc);
    const f32x16* dk = acc.dk;
    const f32x16* dvt = acc.dvt;

    if (!kvalid) return;
    // Lane holds column `key`; accumulator r is row 8(r/4) + 4hf + r%4 of its 32-row atom.
    // dK and dV come out in the units of the scaled dO: multiply by 2^-g.
    const int64_t orow = ((b * a.S + key) * a.h + head) * C;
    const float vsc = pow2i(-R.dsh), ksc = a.scale * vsc;
#pragma unroll
    for (int n = 0; n < NKT; ++n)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = n * 32 + 8 * g + 4 * hf;
        if (d >= DQK) continue;
        f32x4 w = {dk[n][4 * g] * ksc, dk[n][4 * g + 1] * ksc, dk[n][4 * g + 2] * ksc, dk[n][4 * g + 3] * ksc};
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
        f32x4 w = {dvt[n][4 * g] * vsc, dvt[n][4 * g + 1] * vsc, dvt[n][4 * g + 2] * vsc, dvt[n][4 * g + 3] * vsc};
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

template <class InT, class M, int NS, int DN, int DR, int DV>
__global__ __launch_bounds__(kThreads) void dkdv_kernel(BwdArgs a) {
  typedef Dkdv<InT, M, NS, DN, DR, DV> Kn;
  __shared__ __attribute__((aligned(16))) char lds[Kn::LDS_BYTES];
  Kn::run(a, lds);
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

// bfloat16 inputs: delta as above, plus fp16 copies (exact) of the q and dO
// rows and of the k_pe band, which the attention-backward kernels then stage
// with plain 16-byte copies.  A wavefront takes the rows of kRowsPerWave
// consecutive tokens (b, t) of one head i, so that their delta and scale
// entries ([b, i, t] order) are consecutive and four lanes store each kind
// at once.  Per row, the first DV/8 lanes take 8 elements of dO and o each,
// the next DQK/8 lanes 8 elements of q, and on head 0 the next DR/8 lanes 8
// elements of k_pe.
constexpr int kRowsPerWave = 4;  // tokens of the delta / copy pass per wavefront

template <int DN, int DR, int DV>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const float* __restrict__ o, const bf16_t* __restrict__ q,
                                                       const bf16_t* __restrict__ d_o,
                                                       const bf16_t* __restrict__ k_pe, float* __restrict__ delta,
                                                       half_t* __restrict__ q16, half_t* __restrict__ kpe16,
                                                       uint8_t* __restrict__ q8, uint8_t* __restrict__ do8,
                                                       int* __restrict__ qsc, int* __restrict__ osc,
                                                       float* __restrict__ do_max, int64_t T, int h, int64_t S) {
  constexpr int DQK = DN + DR, NO = DV / 8, NQ = DQK / 8, NR = DR / 8;
  static_assert(NO + NQ + NR <= kWave && DV % 8 == 0 && DQK % 8 == 0 && DR % 8 == 0, "one chunk per lane");
  static_assert(NO == 16 && DN / 8 == 16, "dO and q_nope fill one 16-lane group each");
  const int lane = threadIdx.x % kWave;
  // Wavefront w: head i = w mod h, tokens bt0 .. bt0 + kRowsPerWave - 1; the
  // loads of its rows are issued together.  Tokens past the end still reach
  // the workgroup barrier below and touch no memory.
  const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  const int i = static_cast<int>(w % h);
  const int64_t bt0 = (w / h) * kRowsPerWave;
  u16x8 raw[kRowsPerWave];
  f32x4 o0[kRowsPerWave], o1[kRowsPerWave];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int64_t row = (bt0 + r) * h + i;
    raw[r] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    o0[r] = o1[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (bt0 + r >= T) continue;
    if (lane < NO) {
      const int64_t at = row * DV + lane * 8;
      raw[r] = *reinterpret_cast<const u16x8*>(d_o + at);
      o0[r] = *reinterpret_cast<const f32x4*>(o + at);
      o1[r] = *reinterpret_cast<const f32x4*>(o + at + 4);
    } else if (lane < NO + NQ) {
      raw[r] = *reinterpret_cast<const u16x8*>(q + row * DQK + (lane - NO) * 8);
    } else if (lane < NO + NQ + NR && i == 0) {
      raw[r] = *reinterpret_cast<const u16x8*>(k_pe + (bt0 + r) * DR + (lane - NO - NQ) * 8);
    }
  }
  float wave_amax = 0.f;  // largest |dO| of the wavefront's rows (dO lanes)
  float dl[kRowsPerWave];  // delta of each row (every lane)
  int esc[kRowsPerWave];   // E8M0 byte of each row: dO's in lanes 0..15, q_nope's in 16..31
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int64_t bt = bt0 + r;
    const bool live = bt < T;
    const int64_t row = bt * h + i;
    float f[8];
    half8 hv;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f[j] = bf16_to_f32(raw[r][j]);
      hv[j] = static_cast<half_t>(f[j]);
    }
    float acc = 0.f;
    if (live && lane < NO) {  // dO's fp16 copy follows the global scale (do_convert_kernel)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc += f[j] * o0[r][j] + f[4 + j] * o1[r][j];
    } else if (live && lane < NO + NQ) {
      *reinterpret_cast<half8*>(q16 + row * DQK + (lane - NO) * 8) = hv;
    } else if (live && lane < NO + NQ + NR && i == 0) {
      *reinterpret_cast<half8*>(kpe16 + bt * DR + (lane - NO - NQ) * 8) = hv;
    }
    // e4m3 copies of the dO row (lanes 0..15) and the q_nope row (lanes
    // 16..31), each scaled by the power of two 2^s that brings its largest
    // magnitude into [128, 256); the E8M0 byte 127 - s undoes it inside the
    // matrix-core product.
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(f[j]));
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
    wave_amax = fmaxf(wave_amax, amax);
    const int sh = e4m3_row_shift(amax);
    const float sc = __uint_as_float(static_cast<uint32_t>(127 + sh) << 23);
    if (live && lane < NO + DN / 8) {
      uint8_t* dst = lane < NO ? do8 + row * DV + lane * 8 : q8 + row * DN + (lane - NO) * 8;
      *reinterpret_cast<uint2*>(dst) = make_uint2(pack_e4m3x4(f[0] * sc, f[1] * sc, f[2] * sc, f[3] * sc),
                                                  pack_e4m3x4(f[4] * sc, f[5] * sc, f[6] * sc, f[7] * sc));
    }
    esc[r] = 127 - sh;
    dl[r] = wave_sum(acc);
  }
  // Lane r (dO's group) stores row r's delta and dO scale, lane NO + r q_nope's scale.
  const int r = lane % NO;
  if (r < kRowsPerWave && lane < NO + DN / 8 && bt0 + r < T) {
    float d = dl[0];
    int e = esc[0];
#pragma unroll
    for (int k = 1; k < kRowsPerWave; ++k)
      if (r == k) { d = dl[k]; e = esc[k]; }
    const int64_t bt = bt0 + r;
    const int64_t si = ((bt / S) * h + i) * S + bt % S;
    if (lane < NO) {
      delta[si] = d;
      osc[si] = e;
    } else {
      qsc[si] = e;
    }
  }
  // Largest |dO| of the workgroup's rows (lane 0's group holds dO), one value per workgroup.
  __shared__ float wmax[4];
  if (lane == 0) wmax[threadIdx.x / kWave] = wave_amax;
  __syncthreads();
  if (threadIdx.x == 0) do_max[blockIdx.x] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

// g = the shift that brings max |dO| into [8, 16) (0 for an all-zero dO),
// from the per-workgroup maxima of the delta kernel: one workgroup (a max is
// independent of the reduction order).
__global__ __launch_bounds__(1024) void do_shift_kernel(const float* __restrict__ part_max, int64_t n,
                                                        int* __restrict__ shift) {
  __shared__ float part[1024 / kWave];
  float m = 0.f;
#pragma unroll 8  // eight loads in flight per thread
  for (int64_t i = threadIdx.x; i < n; i += 1024) m = fmaxf(m, part_max[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  if (threadIdx.x % kWave == 0) part[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 1024 / kWave; ++w) m = fmaxf(m, part[w]);
    const int e = static_cast<int>((__float_as_uint(m) >> 23) & 0xff);  // m = 1.f * 2^(e - 127)
    int g = e == 0 ? 0 : 130 - e;                                       // m * 2^g in [8, 16)
    shift[0] = g < -100 ? -100 : (g > 100 ? 100 : g);
  }
}

// dO's fp16 copy, scaled by 2^g (exact: a power of two).
__global__ __launch_bounds__(256) void do_convert_kernel(const bf16_t* __restrict__ d_o, const int* __restrict__ shift,
                                                         half_t* __restrict__ do16, int64_t n8) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n8) return;
  const float sc = __uint_as_float(static_cast<uint32_t>(127 + shift[0]) << 23);
  const u16x8 v = *reinterpret_cast<const u16x8*>(d_o + i * 8);
  half8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = static_cast<half_t>(bf16_to_f32(v[j]) * sc);
  *reinterpret_cast<half8*>(do16 + i * 8) = r;
}

// out[t, c] = sum_i part[i, t, c] in increasing i (deterministic head sum).
__global__ __launch_bounds__(256) void head_sum_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                       int64_t n, int h) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (j >= n) return;
  float s = 0.f;
#pragma unroll 8  // the loads issue together; the sum keeps its order
  for (int i = 0; i < h; ++i) s += part[i * n + j];
  out[j] = s;
}

}  // namespace

hipError_t launch_bwd_prep(const Shape& s, const float* o, const void* q, const void* d_o, const void* k_pe,
                           float* delta, const BwdCopies& c, hipStream_t st) {
  const int64_t rows = s.T * s.h;
  const unsigned blocks = static_cast<unsigned>((rows + 3) / 4);
  if (s.bf16 && s.d_nope == 128 && s.d_rope == 64 && s.d_v == 128) {
    // One wavefront per kRowsPerWave tokens and head; one dO maximum per
    // workgroup (the workspace holds (T h + 3) / 4 of them: more than enough).
    const int64_t waves = (s.T + kRowsPerWave - 1) / kRowsPerWave * s.h;
    const unsigned pblocks = static_cast<unsigned>((waves + 3) / 4);
    hipLaunchKernelGGL((bwd_prep_kernel<128, 64, 128>), dim3(pblocks), dim3(256), 0, st, o,
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(d_o),
                       static_cast<const bf16_t*>(k_pe), delta, static_cast<half_t*>(c.q16),
                       static_cast<half_t*>(c.kpe16), static_cast<uint8_t*>(c.q8), static_cast<uint8_t*>(c.do8),
                       c.qsc, c.osc, c.do_row_max, s.T, s.h, s.S);
    hipLaunchKernelGGL(do_shift_kernel, dim3(1), dim3(1024), 0, st, c.do_row_max, static_cast<int64_t>(pblocks),
                       c.do_shift);
    const int64_t n8 = rows * s.d_v / 8;
    hipLaunchKernelGGL(do_convert_kernel, dim3(static_cast<unsigned>((n8 + 255) / 256)), dim3(256), 0, st,
                       static_cast<const bf16_t*>(d_o), c.do_shift, static_cast<half_t*>(c.do16), n8);
  }
  else if (!s.bf16 && s.d_v == 32)
    hipLaunchKernelGGL((bwd_dot_kernel<float, 32>), dim3(blocks), dim3(256), 0, st, o,
                       static_cast<const float*>(d_o), delta, rows, s.h, s.S);
  else
    return hipErrorNotSupported;
  return hipGetLastError();
}

hipError_t launch_head_sum(const Shape& s, const float* part, float* out, hipStream_t st) {
  const int64_t n = s.T * s.d_rope;
  hipLaunchKernelGGL(head_sum_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, part, out,
                     n, s.h);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv(const Shape& s, const void* q, const void* kn, const void* kp, const void* v,
                                const float* lse, const float* delta, const void* d_o, const BwdCopies& c,
                                void* dkv, float* dk_pe_part, hipStream_t st) {
  BwdArgs a = make_args(s, q, kn, kp, v, lse, delta, d_o);
  a.do_shift = c.do_shift;
  a.q8 = static_cast<const uint8_t*>(c.q8);
  a.do8 = static_cast<const uint8_t*>(c.do8);
  a.qsc = c.qsc;
  a.osc = c.osc;
  a.dkv = dkv;
  a.dk_pe_part = dk_pe_part;
  const unsigned grid = static_cast<unsigned>(((s.S + 127) / 128) * s.B * s.h);
  if (s.bf16 && s.split && s.d_nope == 128 && s.d_rope == 64 && s.d_v == 128)
    hipLaunchKernelGGL((dkdv_kernel<half_t, MmaF16, 2, 128, 64, 128>), dim3(grid), dim3(kThreads), 0, st, a);
  else if (!s.bf16 && s.d_nope == 32 && s.d_rope == 16 && s.d_v == 32)
    hipLaunchKernelGGL((dkdv_kernel<float, MmaF32, 1, 32, 16, 32>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    return hipErrorNotSupported;
  return hipGetLastError();
}

}  // namespace laga
