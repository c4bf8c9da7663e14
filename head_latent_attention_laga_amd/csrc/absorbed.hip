// Absorbed form (B2) of one rank's attention: latent-space attention over the
// shared latent [LAGA §3.2 (B2), Fig. 2; the scores equal the explicit ones of
// §2.1 / Algorithm 1].
//
//   kx[u]      = L[u] || k_pe[u]                           (fp16, d_kv + d_rope)
//   s[t,i,u]   = (q_abs[t,i] || q_rope[t,i]) . kx[u] / sqrt(d_nope + d_rope),  u <= t
//   acc[t,i]   = sum_u softmax_u(s) L[u]                   (fp32, d_kv wide)
//   lse[i,t]   = ln sum_u exp(s[t,i,u])
//
// q_abs (= W^k^T q_nope, d_kv wide) comes from the batched absorb GEMM and the
// output o = W^v acc from the un-absorb GEMM (gemm.hip).  This is the pages'
// B2 baseline, built to measure its cost next to LAGA's path: both n_h * d_kv
// intermediates (q_abs, acc) live in HBM, as a training forward keeps them.
//
// Every head reads the same keys and values (the latent), so a workgroup
// takes 64 consecutive (token, head) query rows - 64 / h tokens of every head -
// and streams key blocks of 32 rows of kx through LDS once for all of them.
// Two wavefronts share 32 query rows: each keeps half of the 576 score
// dimensions of its queries in registers (18 fp16 B-operand fragments of
// S^T = K . Q^T) and accumulates half of the 512 latent output columns
// (O^T[dv, query] += V^T . P^T, 8 accumulator tiles, V^T from transposing
// reads of the same tile: the score and value sides share one copy of L in
// LDS).  The two partial score tiles meet through LDS: each lane adds its
// partner's same-lane values, so both wavefronts hold bitwise the same scores
// and the same softmax.  One wavefront per SIMD.  This file is compiled with
// every matrix-core result in vector registers (a build flag): the output
// accumulators are rescaled by vector instructions whenever the running
// maximum grows, and held in accumulator registers they were copied out and
// back around that rare branch on every key block.
//
// Key blocks move HBM -> LDS with buffer loads straight into LDS (16 bytes per
// lane, no staging registers) into two separate shared arrays, the next block
// in flight while the current one is computed.  Rows are 1152 bytes, so row r
// starts at bank 32 (r & 1); 16-byte chunk c of row r is stored at c ^ f(r),
// f(r) = bit 1 of r << 2 | bits 2..3 of r (< 8): the 16 rows of a row-read
// pass and the 4 rows of a transposing read fall on different banks, and with
// 128-byte aligned rows every read is a per-lane base XOR a constant plus an
// immediate offset.
//
// Backward (launch_absorbed_bwd): B2's own steps in reverse, every product
// on bf16 hi + lo planes (three MFMA terms, fp32 accumulation) so that dW_kv_b
// and dgamma meet the same bars as LAGA's backward.  Query rows go in chunks
// (tokens s0 .. s1 of one sequence, all heads): S and dP = d_acc . L over the
// chunk's keys u < s1 are materialised in fp32, the rows' lse and delta are
// recomputed from them, P and c.dS are written as planes, and the products
// over keys (acc, d_q_abs || dq_rope) and over rows (dL || dk_pe) consume
// them.  After the chunks: dq_nope, dW^k, dW^v and the norm's backward.
#include <algorithm>

#include "attn_common.hpp"
#include "launch.hpp"

namespace laga {
namespace {

constexpr int DL = 512, DR = 64, DNQ = 128, DQ = DL + DR;  // latent, rope band, q_nope, score width
constexpr int BN = 32;                                      // keys per block
constexpr int NW = 4, NT = NW * kWave, ROWS = 16 * NW;      // query rows per workgroup (32 per pair)
constexpr int PITCH = DQ * 2;                               // bytes per kx row in LDS (1152)
constexpr int CPR = PITCH / 16;                             // 16-byte chunks per row (72)
constexpr int TILE = BN * PITCH;                            // bytes per key block (36864)
constexpr int PASSES = TILE / (NT * 16);                    // 1 KB windows per wavefront per block
constexpr int KSH = DQ / 32, NOH = DL / 64;                 // score steps (18), output tiles (8) per wavefront
constexpr int XCH = NW * kWave * 16 * 4;                    // partial-score exchange area (bytes)
constexpr float kRescale = 8.f;                             // lazy-rescale threshold (log2 units)
static_assert(TILE % (NT * 16) == 0 && CPR % 8 == 0 && PITCH % 128 == 0, "layout");

struct AbsArgs {
  const half_t* q_abs;  // [B, S, h, DL]
  const bf16_t* q;      // [B, S, h, DNQ + DR] (rope part used)
  const half_t* kx;     // [B, S, DQ]
  float* acc;           // [B, S, h, DL]
  float* lse;           // [B, h, S]
  int64_t S;
  int B, h, n_rt;
  float scale_log2;
};

__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

struct Abs {
  // Source offsets (bytes into the key block) of the lane's 16-byte chunk in
  // each pass: physical chunk P = (p NW + wavefront) 64 + lane of the tile
  // holds row P / CPR, logical chunk (P mod CPR) ^ swz(row).  They do not
  // depend on the block, so they are formed once, before the key loop, and
  // kept: each is pinned to an accumulator register where it is formed,
  // which stops the compiler from recomputing them (a division by CPR and
  // the swizzle, per pass) on every block.
  struct Src { uint32_t off[PASSES]; };

  __device__ static Src src_offsets() {
    const int lane = threadIdx.x % kWave;
    const int wv = static_cast<int>(threadIdx.x) / kWave;
    Src o;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int P = (p * NW + wv) * kWave + lane;
      const int r = P / CPR, pc = P % CPR;
      o.off[p] = static_cast<uint32_t>(r * PITCH + (pc ^ swz(r)) * 16);
      asm volatile("" : "+a"(o.off[p]));
    }
    return o;
  }

  // Issue one key block (rows key0 ..) into `buf`; rows past the sequence read as zero.
  __device__ static void issue(const AbsArgs& a, int b, int64_t key0, char* buf, const Src& so) {
    const int64_t left = a.S - key0;
    const int nk = static_cast<int>(left < BN ? (left > 0 ? left : 0) : BN);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<half_t*>(a.kx + (static_cast<int64_t>(b) * a.S + key0) * DQ), 0, nk * PITCH, 0x00020000);
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) load_lds16(rs, buf + (p * NW + wv) * 1024, so.off[p]);
  }

  struct State {
    half8 qf[KSH];   // score dims 288 hw + 16 j + 8 hf + [0, 8)
    f32x16 o[NOH];   // latent columns 256 hw + 32 n + ...
    float m_run, l_run;
  };

  // Per-lane byte offsets: row fragment of key row col, score step s = 4m + u
  // at (rb ^ 32u) + 128m; transposing fragment (st, n) at
  // (tb ^ 64 (n&1) [^ 32 for rows + 8]) + (16 st [+ 8]) * PITCH + 128 (n >> 1).
  struct Offs { uint32_t rb, tb; };

  __device__ static void compute(const AbsArgs& a, const char* buf, float* xch, int64_t key0, int64_t t_lo,
                                 int64_t tq, int hw, const Offs& of0, State& st) {
    Offs of = of0;
    asm volatile("" : "+v"(of.rb), "+v"(of.tb));  // form the addresses per block, not held across the loop
    const int lane = threadIdx.x % kWave;
    const int hf = lane / 32;
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
    // The key fragments read kAhead products ahead of their use.
    constexpr int kAhead = 3;
    pipelined<KSH, kAhead, half8>(
        [&](int j) {
          const int s = hw * KSH + j;  // score step over the 576 dims
          return lds_at<half8>(buf, (of.rb ^ (32u * (s % 4))) + 128 * (s / 4));
        },
        [&](int j, const half8& kf) { sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, st.qf[j], sc, 0, 0, 0); });
    // Partial scores meet the partner's: same lane, same (key, query) elements.
    f32x4* mine = reinterpret_cast<f32x4*>(xch) + (threadIdx.x / kWave) * kWave * 4 + lane;
    const f32x4* theirs = reinterpret_cast<const f32x4*>(xch) + ((threadIdx.x / kWave) ^ 1) * kWave * 4 + lane;
#pragma unroll
    for (int g = 0; g < 4; ++g) mine[g * kWave] = f32x4{sc[4 * g], sc[4 * g + 1], sc[4 * g + 2], sc[4 * g + 3]};
    lds_barrier();
    f32x4 o4[4];  // the partner's values, all four reads in flight together
#pragma unroll
    for (int g = 0; g < 4; ++g) o4[g] = theirs[g * kWave];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int k = 0; k < 4; ++k) sc[4 * g + k] += o4[g][k];
    // Causal mask on blocks that reach past the pair's first query token:
    // key key0 + 8(r/4) + 4hf + r%4 is masked above the lane's token.
    if (key0 + BN - 1 > t_lo) {
      const int rel = static_cast<int>(tq - key0) - 4 * hf;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r / 4) + (r % 4) > rel) sc[r] = -INFINITY;
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sc[r]);
    mloc = pair_max(mloc) * a.scale_log2;
    if (__any(mloc > st.m_run + kRescale)) {
      const float m_new = fmaxf(st.m_run, mloc);
      const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
      st.l_run *= alpha;
#pragma unroll
      for (int n = 0; n < NOH; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[n][r] *= alpha;
      st.m_run = m_new;
    }
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sc[r], a.scale_log2, -st.m_run));
      sc[r] = p;
      lsum += p;
    }
    st.l_run += pair_sum(lsum);

    // O^T += V^T P^T over the block's 32 keys for this wavefront's 256 columns,
    // the V^T fragments (transposing reads) kAhead products ahead.
    half8 pf[2];
#pragma unroll
    for (int sp = 0; sp < 2; ++sp)
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[sp][j] = static_cast<half_t>(sc[sp * 8 + j]);
    pipelined<2 * NOH, kAhead, half8>(
        [&](int i) {
          const int sp = i / NOH, n = hw * NOH + i % NOH;
          const uint32_t row0 = sp * 16 * PITCH + 128 * (n >> 1);
          const uint32_t x0 = (of.tb ^ (64u * (n & 1))) + row0;
          const uint32_t x1 = (of.tb ^ (64u * (n & 1) + 32u)) + row0 + 8 * PITCH;
          const s16x4 lo = ds_read_tr16(buf + x0), hi = ds_read_tr16(buf + x1);
          typedef short s16x8 __attribute__((ext_vector_type(8)));
          return __builtin_bit_cast(half8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        },
        [&](int i, const half8& v) {
          st.o[i % NOH] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v, pf[i / NOH], st.o[i % NOH], 0, 0, 0);
        });
  }

  // Blocks are computed by both wavefronts of a pair or by neither (skipped
  // when they lie wholly after the pair's last query token), but every
  // wavefront reaches both barriers of every step.
  __device__ static void step(const AbsArgs& a, int kb, int b, int64_t t_lo, int64_t t_hi, int64_t tq, int hw,
                              const char* cur, char* nxt, float* xch, const Offs& of, const Src& so, State& st) {
    dma_barrier();  // block kb has landed in `cur`; `nxt` (block kb-1) and the exchange area are free
    const int64_t key0 = static_cast<int64_t>(kb) * BN;
    issue(a, b, key0 + BN, nxt, so);  // on every step, so every path has the same loads in flight
    if (key0 <= t_hi) {
      compute(a, cur, xch, key0, t_lo, tq, hw, of, st);
    } else {
      lds_barrier();  // the exchange barrier of the pairs that compute
    }
  }

  __device__ static void run(const AbsArgs& a, char* lds0, char* lds1, float* xch) {
    const int lane = threadIdx.x % kWave;
    const int wv = threadIdx.x / kWave;
    const int pr = wv / 2, hw = wv % 2;  // pair, half
    const int hf = lane / 32, col = lane % 32, g = lane / 16, sl = lane % 16;
    // Row tiles longest first; every tile reads the same keys, so L2 serves them all.
    const int b = static_cast<int>(blockIdx.x) % a.B;
    const int rt = a.n_rt - 1 - static_cast<int>(blockIdx.x) / a.B;
    const int64_t rows = a.S * a.h;
    const int64_t r0 = static_cast<int64_t>(rt) * ROWS + pr * 32;  // the pair's first query row
    const int64_t row = r0 + col;
    const bool qvalid = row < rows;
    const int64_t rc = qvalid ? row : rows - 1;
    const int64_t tq = rc / a.h;  // the lane's query token
    const int i = static_cast<int>(rc % a.h);
    const int64_t t_lo = (r0 < rows ? r0 : rows - 1) / a.h;
    const int64_t t_hi = (r0 + 31 < rows ? r0 + 31 : rows - 1) / a.h;
    const int64_t last = static_cast<int64_t>(rt) * ROWS + ROWS - 1;
    const int64_t tile_hi = (last < rows ? last : rows - 1) / a.h;
    const int nkb = static_cast<int>(tile_hi / BN) + 1;

    const Src so = src_offsets();
    issue(a, b, 0, lds0, so);

    State st;
    {
      const half_t* qa = a.q_abs + (static_cast<int64_t>(b) * a.S * a.h + rc) * DL;
      const bf16_t* qr = a.q + (static_cast<int64_t>(b) * a.S * a.h + rc) * (DNQ + DR) + DNQ;
#pragma unroll
      for (int j = 0; j < KSH; ++j) {
        const int d = (hw * KSH + j) * 16 + hf * 8;  // score dim of this lane's fragment
        if (d < DL) {
          st.qf[j] = qvalid ? *reinterpret_cast<const half8*>(qa + d) : half8{};
        } else {
          const u16x8 raw = qvalid ? *reinterpret_cast<const u16x8*>(qr + (d - DL)) : u16x8{};
          half8 h;
#pragma unroll
          for (int k = 0; k < 8; ++k) h[k] = static_cast<half_t>(bf16_to_f32(raw[k]));
          st.qf[j] = h;
        }
      }
    }
#pragma unroll
    for (int n = 0; n < NOH; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[n][r] = 0.f;
    st.m_run = -INFINITY;
    st.l_run = 0.f;

    Offs of;
    of.rb = col * PITCH + 16 * (hf ^ swz(col));
    {
      const int tr = 4 * hf + sl / 4;  // + 16 st; swz() of it is the same for both halves of the block
      const int cl = 2 * (g % 2) + (sl % 4) / 2;
      of.tb = tr * PITCH + 16 * (cl ^ swz(tr)) + 8 * (sl % 2);
    }

    // Unrolled by two so that each step names its buffers statically.
    int kb = 0;
    for (; kb + 1 < nkb; kb += 2) {
      step(a, kb, b, t_lo, t_hi, tq, hw, lds0, lds1, xch, of, so, st);
      step(a, kb + 1, b, t_lo, t_hi, tq, hw, lds1, lds0, xch, of, so, st);
    }
    if (kb < nkb) step(a, kb, b, t_lo, t_hi, tq, hw, lds0, lds1, xch, of, so, st);
    // The last step's prefetch must land before the wave ends: the
    // workgroup's LDS is handed to another workgroup afterwards.
    __builtin_amdgcn_s_waitcnt(0);

    if (qvalid) {
      const float inv = 1.0f / st.l_run;
      float* op = a.acc + (static_cast<int64_t>(b) * a.S * a.h + row) * DL + hw * (DL / 2);
#pragma unroll
      for (int n = 0; n < NOH; ++n)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 w = {st.o[n][4 * q4] * inv, st.o[n][4 * q4 + 1] * inv, st.o[n][4 * q4 + 2] * inv,
                           st.o[n][4 * q4 + 3] * inv};
          *reinterpret_cast<f32x4*>(op + n * 32 + 8 * q4 + 4 * hf) = w;
        }
      if (hw == 0 && hf == 0)
        a.lse[(static_cast<int64_t>(b) * a.h + i) * a.S + tq] = (st.m_run + log2f(st.l_run)) * 0.69314718055994531f;
    }
  }
};

__global__ __launch_bounds__(NT, 1) void absorbed_attn_kernel(AbsArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds0[TILE];
  __shared__ __attribute__((aligned(1024))) char lds1[TILE];
  __shared__ __attribute__((aligned(16))) float xch[XCH / 4];
  Abs::run(a, lds0, lds1, xch);
}

// kx[t] = fp16(L[t]) || fp16(k_pe[t]); one thread per 8 elements.
__global__ __launch_bounds__(256) void absorbed_pack_kernel(const float* __restrict__ L, const bf16_t* __restrict__ k_pe,
                                                            half_t* __restrict__ kx, int64_t T) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // 8-element chunk
  if (j >= T * (DQ / 8)) return;
  const int64_t t = j / (DQ / 8);
  const int c = static_cast<int>(j % (DQ / 8)) * 8;
  half8 h;
  if (c < DL) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(L + t * DL + c);
    const f32x4 y = *reinterpret_cast<const f32x4*>(L + t * DL + c + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      h[k] = static_cast<half_t>(x[k]);
      h[4 + k] = static_cast<half_t>(y[k]);
    }
  } else {
    const u16x8 r = *reinterpret_cast<const u16x8*>(k_pe + t * DR + (c - DL));
#pragma unroll
    for (int k = 0; k < 8; ++k) h[k] = static_cast<half_t>(bf16_to_f32(r[k]));
  }
  *reinterpret_cast<half8*>(kx + t * DQ + c) = h;
}

// ------------------------------------------------------------------ backward
// Elementwise pieces of the absorbed form's backward (products in gemm.hip).
constexpr int B2_CHUNK_CAP_MB = 1024;  // per-chunk S, dP, P and c.dS buffers

__device__ __forceinline__ void split8(const float* x, u16x8& hi, u16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) split_bf16_pair(x[2 * j], x[2 * j + 1], h[j], l[j]);
  hi = __builtin_bit_cast(u16x8, u32x4{h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(u16x8, u32x4{l[0], l[1], l[2], l[3]});
}

// Row statistics of one chunk from its scores S and dP = d_acc . L (fp32,
// row pitch ldu), over the row's keys u <= its token: lse = ln sum_u exp(S c)
// and delta = sum_u P dP (= sum_j dO o for this P).  One wavefront per row,
// each lane an online (max, sum, weighted dP sum) over its 4-key groups (four
// 16-byte loads of S and of dP in flight), merged across the wavefront.
__global__ __launch_bounds__(256) void b2_rowstat_kernel(const float* __restrict__ S, const float* __restrict__ dP,
                                                         int64_t ldu, int64_t nrows, int64_t nkeys, int64_t s0, int h,
                                                         float scale, float* __restrict__ lse,
                                                         float* __restrict__ delta) {
  constexpr int UNR = 4;  // float4 loads of S and dP per lane in flight: 1024 keys per wave step
  const int64_t rr = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (rr >= nrows) return;
  const int lane = threadIdx.x % kWave;
  const int64_t st = s0 + rr / h;
  const int64_t nk = st + 1 < nkeys ? st + 1 : nkeys;
  const float c2 = scale * 1.4426950408889634f;  // log2 units
  const float* srow = S + rr * ldu;
  const float* drow = dP + rr * ldu;
  float m = -INFINITY, l = 0.f, dsum = 0.f;
  // ldu is a multiple of 32 >= nk, so a float4 that starts below nk lies inside the row;
  // its elements at or past nk (never written) are masked by selection, not arithmetic.
  for (int64_t base = 4 * lane; base < nk; base += 4 * kWave * UNR) {
    f32x4 xs[UNR], dps[UNR];
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int64_t u = base + 4 * kWave * k;
      xs[k] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      dps[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (u < nk) {
        xs[k] = *reinterpret_cast<const f32x4*>(srow + u);
        dps[k] = *reinterpret_cast<const f32x4*>(drow + u);
      }
    }
    float mx = m;
#pragma unroll
    for (int k = 0; k < UNR; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = base + 4 * kWave * k + j < nk;
        xs[k][j] = ok ? xs[k][j] * c2 : -INFINITY;
        dps[k][j] = ok ? dps[k][j] : 0.f;
        mx = fmaxf(mx, xs[k][j]);
      }
    // mx is finite: the element at base is valid.
    const float a = __builtin_amdgcn_exp2f(m - mx);
    l *= a;
    dsum *= a;
    m = mx;
#pragma unroll
    for (int k = 0; k < UNR; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = __builtin_amdgcn_exp2f(xs[k][j] - m);
        l += e;
        dsum += e * dps[k][j];
      }
  }
  float mw = m;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mw = fmaxf(mw, __shfl_xor(mw, o, kWave));
  const float a = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mw);
  l = wave_sum(l * a);
  dsum = wave_sum(dsum * a);
  if (lane == 0) {
    lse[rr] = (mw + log2f(l)) * 0.69314718055994531f;
    delta[rr] = dsum / l;
  }
}

// kxp[p][t] = L[t] || k_pe[t] as bf16 hi (p = 0) / lo (p = 1) planes, L = gamma x rstd
// (the forward's normalisation); rows t in [T, Tp) are zero.  One thread per 8 elements.
__global__ __launch_bounds__(256) void b2_kxp_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ gamma,
                                                     const float* __restrict__ rstd, const bf16_t* __restrict__ k_pe,
                                                     bf16_t* __restrict__ kxp, int64_t T, int64_t Tp) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (j >= Tp * (DQ / 8)) return;
  const int64_t t = j / (DQ / 8);
  const int c = static_cast<int>(j % (DQ / 8)) * 8;
  u16x8 hi = {}, lo = {};
  if (t < T && c < DL) {
    const u16x8 xr = *reinterpret_cast<const u16x8*>(x + t * DL + c);
    const u16x8 gr = *reinterpret_cast<const u16x8*>(gamma + c);
    const float r = rstd[t];
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = bf16_to_f32(gr[k]) * (bf16_to_f32(xr[k]) * r);
    split8(v, hi, lo);
  } else if (t < T) {
    hi = *reinterpret_cast<const u16x8*>(k_pe + t * DR + (c - DL));
  }
  *reinterpret_cast<u16x8*>(kxp + t * DQ + c) = hi;
  *reinterpret_cast<u16x8*>(kxp + Tp * DQ + t * DQ + c) = lo;
}

// qx[p][r][512 ..] = q_rope[r] (hi plane), 0 (lo plane).
__global__ __launch_bounds__(256) void b2_qrope_kernel(const bf16_t* __restrict__ q, bf16_t* __restrict__ qx,
                                                       int64_t rows) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (j >= rows * (DR / 8)) return;
  const int64_t r = j / (DR / 8);
  const int c = static_cast<int>(j % (DR / 8)) * 8;
  *reinterpret_cast<u16x8*>(qx + r * DQ + DL + c) = *reinterpret_cast<const u16x8*>(q + r * (DNQ + DR) + DNQ + c);
  *reinterpret_cast<u16x8*>(qx + rows * DQ + r * DQ + DL + c) = u16x8{};
}

// One chunk of rows (tokens s0 .. of one sequence, all heads): from the scores
// S and dP = d_acc . L (fp32, row pitch ldu) and the rows' lse and delta,
// P = exp(S c - lse) and c.dS = c P (dP - delta) on keys u <= the row's token,
// zero on the others and on u in [nkeys, kpad); written as bf16 hi / lo planes
// (plane pitch pplane).  One thread per 8 keys.
__global__ __launch_bounds__(256) void b2_pds_kernel(const float* __restrict__ S, const float* __restrict__ dP,
                                                     const float* __restrict__ lse, const float* __restrict__ delta,
                                                     bf16_t* __restrict__ pp, bf16_t* __restrict__ dsp,
                                                     int64_t pplane, int64_t ldu, int64_t nrows, int64_t nkeys,
                                                     int64_t kpad, int64_t s0, int h, float scale) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per_row = kpad / 8;
  if (j >= nrows * per_row) return;
  const int64_t rr = j / per_row;
  const int64_t u0 = (j % per_row) * 8;
  const int64_t st = s0 + rr / h;  // the row's token within its sequence
  const float lse2 = lse[rr] * 1.4426950408889634f;
  const float dl = delta[rr];
  const float sc2 = scale * 1.4426950408889634f;
  float p[8], ds[8];
  const int64_t lim = st < nkeys - 1 ? st : nkeys - 1;  // last key of the row
  if (u0 + 7 <= lim) {  // the whole group is valid: two 16-byte loads of each
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(S + rr * ldu + u0);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(S + rr * ldu + u0 + 4);
    const f32x4 d0 = *reinterpret_cast<const f32x4*>(dP + rr * ldu + u0);
    const f32x4 d1 = *reinterpret_cast<const f32x4*>(dP + rr * ldu + u0 + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      p[k] = __builtin_amdgcn_exp2f(fmaf(s0[k], sc2, -lse2));
      p[4 + k] = __builtin_amdgcn_exp2f(fmaf(s1[k], sc2, -lse2));
      ds[k] = scale * p[k] * (d0[k] - dl);
      ds[4 + k] = scale * p[4 + k] * (d1[k] - dl);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t u = u0 + k;
      p[k] = 0.f;
      ds[k] = 0.f;
      if (u <= lim) {
        p[k] = __builtin_amdgcn_exp2f(fmaf(S[rr * ldu + u], sc2, -lse2));
        ds[k] = scale * p[k] * (dP[rr * ldu + u] - dl);
      }
    }
  }
  u16x8 h8, l8;
  split8(p, h8, l8);
  *reinterpret_cast<u16x8*>(pp + rr * ldu + u0) = h8;
  *reinterpret_cast<u16x8*>(pp + pplane + rr * ldu + u0) = l8;
  split8(ds, h8, l8);
  *reinterpret_cast<u16x8*>(dsp + rr * ldu + u0) = h8;
  *reinterpret_cast<u16x8*>(dsp + pplane + rr * ldu + u0) = l8;
}

// acc planes of a chunk: out[r][c] (hi) and out[plane + r][c] (lo) from the sum over the
// K-chunk partials part[k][r][c], k = 0 .. nch - 1 in order.  One thread per 8 columns.
__global__ __launch_bounds__(256) void b2_ksum_planes_kernel(const float* __restrict__ part, int nch, int64_t nrows,
                                                             bf16_t* __restrict__ out, int64_t plane) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (j >= nrows * (DL / 8)) return;
  const int64_t e = j * 8;  // = r * 512 + c
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < nch; ++k) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(part + k * nrows * DL + e);
    const f32x4 b = *reinterpret_cast<const f32x4*>(part + k * nrows * DL + e + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] += a[i];
      v[4 + i] += b[i];
    }
  }
  u16x8 hi, lo;
  split8(v, hi, lo);
  *reinterpret_cast<u16x8*>(out + e) = hi;
  *reinterpret_cast<u16x8*>(out + plane + e) = lo;
}

// out[e] = sum over k in order of part[k * n + e], four elements per thread (n % 4 == 0).
__global__ __launch_bounds__(256) void b2_ksum_kernel(const float* __restrict__ part, int nch, int64_t n,
                                                      float* __restrict__ out) {
  const int64_t e = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (e >= n) return;
  f32x4 v = *reinterpret_cast<const f32x4*>(part + e);
  for (int k = 1; k < nch; ++k) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(part + k * n + e);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += a[i];
  }
  *reinterpret_cast<f32x4*>(out + e) = v;
}

// out planes [2][rows][512] = bf16 hi / lo of in[r][0 .. 512) (row pitch ld_in).
__global__ __launch_bounds__(256) void b2_planes_kernel(const float* __restrict__ in, int64_t ld_in,
                                                        bf16_t* __restrict__ out, int64_t rows) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (j >= rows * (DL / 8)) return;
  const int64_t r = j / (DL / 8);
  const int c = static_cast<int>(j % (DL / 8)) * 8;
  const f32x4 a = *reinterpret_cast<const f32x4*>(in + r * ld_in + c);
  const f32x4 b = *reinterpret_cast<const f32x4*>(in + r * ld_in + c + 4);
  const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  u16x8 hi, lo;
  split8(v, hi, lo);
  *reinterpret_cast<u16x8*>(out + r * DL + c) = hi;
  *reinterpret_cast<u16x8*>(out + rows * DL + r * DL + c) = lo;
}

// dq[r][128 + j] = dqx[r][512 + j] (the rope part of dq).
__global__ __launch_bounds__(256) void b2_dq_rope_kernel(const float* __restrict__ dqx, float* __restrict__ dq,
                                                         int64_t rows) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (j >= rows * (DR / 4)) return;
  const int64_t r = j / (DR / 4);
  const int c = static_cast<int>(j % (DR / 4)) * 4;
  *reinterpret_cast<f32x4*>(dq + r * (DNQ + DR) + DNQ + c) = *reinterpret_cast<const f32x4*>(dqx + r * DQ + DL + c);
}

__global__ __launch_bounds__(256) void b2_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (j < n) p[j] = 0.f;
}

unsigned blocks_for(int64_t n) { return static_cast<unsigned>((n + 255) / 256); }

// Workspace of laga_absorbed_bwd, regions 256-byte aligned.
struct B2Layout {
  int64_t R, Tp, ldu, tc, rc_max;
  size_t qx, dacc, kxp, accp, dqx, dL, sbuf, dpbuf, pp, dsp, rlse, rdelta, kpart, kgpart, dw, dg, total;
};

// tc: tokens per chunk of query rows (a multiple of 32); 0 picks the default,
// the largest whose chunk buffers fit B2_CHUNK_CAP_MB.
B2Layout b2_layout(const Shape& s, int64_t tc = 0) {
  B2Layout L;
  L.R = s.T * s.h;
  L.Tp = s.T + 32;
  L.ldu = (s.S + 31) / 32 * 32;
  if (tc <= 0) {
    const int64_t per_token = 16 * static_cast<int64_t>(s.h) * L.ldu;  // S, dP (fp32), P, c.dS (2 bf16 planes)
    tc = (static_cast<int64_t>(B2_CHUNK_CAP_MB) << 20) / per_token / 32 * 32;
  }
  if (tc < 32) tc = 32;
  if (tc > L.ldu) tc = L.ldu;
  L.tc = tc;
  L.rc_max = tc * s.h;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~size_t(255);
    return at;
  };
  L.qx = take(static_cast<size_t>(2) * L.R * DQ * 2);
  L.dacc = take(static_cast<size_t>(2) * L.R * DL * 2);
  L.kxp = take(static_cast<size_t>(2) * L.Tp * DQ * 2);
  L.accp = take(static_cast<size_t>(2) * L.R * DL * 2);
  L.dqx = take(static_cast<size_t>(L.R) * DQ * 4);
  L.dL = take(static_cast<size_t>(s.T) * DL * 4);
  L.sbuf = take(static_cast<size_t>(L.rc_max) * L.ldu * 4);
  L.dpbuf = take(static_cast<size_t>(L.rc_max) * L.ldu * 4);
  L.pp = take(static_cast<size_t>(2) * L.rc_max * L.ldu * 2);
  L.dsp = take(static_cast<size_t>(2) * L.rc_max * L.ldu * 2);
  L.rlse = take(static_cast<size_t>(L.rc_max) * 4);
  L.rdelta = take(static_cast<size_t>(L.rc_max) * 4);
  L.kpart = take(static_cast<size_t>(B2_KSPLIT) * L.rc_max * DQ * 4);
  // Key-side partials: the largest over the chunks that split their rows.
  size_t kg = 0;
  for (int64_t s0 = 0; s0 < s.S; s0 += L.tc) {
    const int64_t s1 = s0 + L.tc < s.S ? s0 + L.tc : s.S;
    const int nch = b2_keygrad_chunks(s1, (s1 - s0) * s.h);
    if (nch > 1) kg = std::max(kg, static_cast<size_t>(2) * nch * s1 * DQ);
  }
  L.kgpart = take(kg * 4);
  L.dw = take(b2_dw_partial_floats(s) * 4);
  L.dg = take(norm_bwd_partial_floats(s) * 4);
  L.total = off;
  return L;
}

bool b2_supported(const Shape& s) { return s.bf16 && s.d_kv == DL && s.d_rope == DR && s.d_nope == DNQ && s.d_v == DNQ; }

}  // namespace

size_t absorbed_bwd_workspace_bytes(const Shape& s) { return b2_supported(s) ? b2_layout(s).total : 0; }
size_t absorbed_bwd_min_workspace_bytes(const Shape& s) { return b2_supported(s) ? b2_layout(s, 32).total : 0; }

namespace {
// The layout a call runs with: the default chunk size, or for a smaller
// workspace the largest chunk (in steps of 32 tokens) whose layout fits.
B2Layout b2_layout_for(const Shape& s, size_t bytes) {
  B2Layout L = b2_layout(s);
  if (L.total <= bytes) return L;
  int64_t lo = 32, hi = L.tc;  // layout(lo) fits (checked by the caller), layout(hi) does not
  while (hi - lo > 32) {
    const int64_t mid = (lo + hi) / 64 * 32;
    if (b2_layout(s, mid).total <= bytes) lo = mid;
    else hi = mid;
  }
  return b2_layout(s, lo);
}
}  // namespace

hipError_t launch_absorbed_bwd(const Shape& s, const void* q, const void* latent, const void* gamma,
                               const float* rstd, const void* k_pe, const void* w, const void* d_o, float* dq,
                               float* d_latent, float* d_k_pe, float* d_w, float* d_gamma, void* workspace,
                               size_t workspace_bytes, hipStream_t st) {
  if (!b2_supported(s)) return hipErrorNotSupported;
  if (workspace_bytes < absorbed_bwd_min_workspace_bytes(s)) return hipErrorInvalidValue;
  const B2Layout L = b2_layout_for(s, workspace_bytes);
  char* ws = static_cast<char*>(workspace);
  bf16_t* qx = reinterpret_cast<bf16_t*>(ws + L.qx);
  bf16_t* dacc = reinterpret_cast<bf16_t*>(ws + L.dacc);
  bf16_t* kxp = reinterpret_cast<bf16_t*>(ws + L.kxp);
  bf16_t* accp = reinterpret_cast<bf16_t*>(ws + L.accp);
  float* rlse = reinterpret_cast<float*>(ws + L.rlse);
  float* rdelta = reinterpret_cast<float*>(ws + L.rdelta);
  float* kpart = reinterpret_cast<float*>(ws + L.kpart);
  float* kgpart = reinterpret_cast<float*>(ws + L.kgpart);
  float* dqx = reinterpret_cast<float*>(ws + L.dqx);
  float* dL = reinterpret_cast<float*>(ws + L.dL);
  float* sbuf = reinterpret_cast<float*>(ws + L.sbuf);
  float* dpbuf = reinterpret_cast<float*>(ws + L.dpbuf);
  bf16_t* pp = reinterpret_cast<bf16_t*>(ws + L.pp);
  bf16_t* dsp = reinterpret_cast<bf16_t*>(ws + L.dsp);
  float* dwp = reinterpret_cast<float*>(ws + L.dw);
  float* dgp = reinterpret_cast<float*>(ws + L.dg);
  const bf16_t* qb = static_cast<const bf16_t*>(q);
  const int64_t R = L.R, dq_ld = static_cast<int64_t>(s.h) * (DNQ + DR), do_ld = static_cast<int64_t>(s.h) * DNQ;
  const int64_t qx_plane = R * DQ, dacc_plane = R * DL, kxp_plane = L.Tp * DQ, pplane = L.rc_max * L.ldu;
  const float scale = 1.0f / sqrtf(static_cast<float>(DNQ + DR));
  hipError_t e;
#define B2_TRY(x) \
  if ((e = (x)) != hipSuccess) return e
  // Operands: q_abs, d_acc as planes; the rope columns of qx; L || k_pe; zeroed accumulators.
  B2_TRY(launch_b2_planes(s, q, dq_ld, DNQ + DR, 0, w, qx, qx_plane, DQ, st));
  B2_TRY(launch_b2_planes(s, d_o, do_ld, DNQ, DNQ, w, dacc, dacc_plane, DL, st));
  hipLaunchKernelGGL(b2_qrope_kernel, dim3(blocks_for(R * (DR / 8))), dim3(256), 0, st, qb, qx, R);
  hipLaunchKernelGGL(b2_kxp_kernel, dim3(blocks_for(L.Tp * (DQ / 8))), dim3(256), 0, st,
                     static_cast<const bf16_t*>(latent), static_cast<const bf16_t*>(gamma), rstd,
                     static_cast<const bf16_t*>(k_pe), kxp, s.T, L.Tp);
  hipLaunchKernelGGL(b2_zero_kernel, dim3(blocks_for(s.T * DL)), dim3(256), 0, st, dL, s.T * DL);
  hipLaunchKernelGGL(b2_zero_kernel, dim3(blocks_for(s.T * DR)), dim3(256), 0, st, d_k_pe, s.T * DR);
  B2_TRY(hipGetLastError());
  // Row chunks of tc tokens x all heads against their keys 0 .. chunk end.
  for (int64_t b = 0; b < s.B; ++b) {
    for (int64_t s0 = 0; s0 < s.S; s0 += L.tc) {
      const int64_t s1 = s0 + L.tc < s.S ? s0 + L.tc : s.S;
      const int64_t r0 = (b * s.S + s0) * s.h, nrows = (s1 - s0) * s.h;
      const int64_t nkeys = s1, kpad = (s1 + 31) / 32 * 32;
      const bf16_t* keys = kxp + b * s.S * DQ;
      B2_TRY(launch_b2_rows_keys(qx + r0 * DQ, qx_plane, DQ, nrows, keys, kxp_plane, nkeys, DQ, sbuf, L.ldu, st));
      B2_TRY(launch_b2_rows_keys(dacc + r0 * DL, dacc_plane, DL, nrows, keys, kxp_plane, nkeys, DL, dpbuf, L.ldu, st));
      hipLaunchKernelGGL(b2_rowstat_kernel, dim3(static_cast<unsigned>((nrows + 3) / 4)), dim3(256), 0, st, sbuf,
                         dpbuf, L.ldu, nrows, nkeys, s0, s.h, scale, rlse, rdelta);
      hipLaunchKernelGGL(b2_pds_kernel, dim3(blocks_for(nrows * (kpad / 8))), dim3(256), 0, st, sbuf, dpbuf, rlse,
                         rdelta, pp, dsp, pplane, L.ldu, nrows, nkeys, kpad, s0, s.h, scale);
      B2_TRY(hipGetLastError());
      // acc = P L (as planes), then dL, dk_pe from P and c.dS, then d_q_abs || dq_rope = c.dS kx.
      B2_TRY(launch_b2_rows_by_keys(pp, pplane, L.ldu, nrows, kpad, keys, kxp_plane, DL, kpart, st));
      const int nca = b2_key_chunks(nrows, DL, kpad);
      hipLaunchKernelGGL(b2_ksum_planes_kernel, dim3(blocks_for(nrows * (DL / 8))), dim3(256), 0, st, kpart, nca,
                         nrows, accp + r0 * DL, R * DL);
      B2_TRY(hipGetLastError());
      B2_TRY(launch_b2_key_grads(pp, dsp, pplane, L.ldu, nrows, nkeys, dacc + r0 * DL, dacc_plane, qx + r0 * DQ,
                                 qx_plane, dL + b * s.S * DL, d_k_pe + b * s.S * DR, kgpart, st));
      B2_TRY(launch_b2_rows_by_keys(dsp, pplane, L.ldu, nrows, kpad, keys, kxp_plane, DQ, kpart, st));
      const int ncq = b2_key_chunks(nrows, DQ, kpad);
      hipLaunchKernelGGL(b2_ksum_kernel, dim3(blocks_for(nrows * (DQ / 4))), dim3(256), 0, st, kpart, ncq,
                         nrows * DQ, dqx + r0 * DQ);
      B2_TRY(hipGetLastError());
    }
  }
  // dq = [d_q_abs W^k^T || dq_rope]; dW^k from q_nope and d_q_abs, dW^v from dO and acc; the norm's backward.
  B2_TRY(launch_b2_dq_nope(s, dqx, w, dq, st));
  hipLaunchKernelGGL(b2_dq_rope_kernel, dim3(blocks_for(R * (DR / 4))), dim3(256), 0, st, dqx, dq, R);
  hipLaunchKernelGGL(b2_planes_kernel, dim3(blocks_for(R * (DL / 8))), dim3(256), 0, st, dqx, DQ, qx, R);
  B2_TRY(hipGetLastError());
  B2_TRY(launch_b2_dw(s, q, dq_ld, DNQ + DR, qx, R * DL, dwp, d_w, 0, st));
  B2_TRY(launch_b2_dw(s, d_o, do_ld, DNQ, accp, R * DL, dwp, d_w, DNQ, st));
  B2_TRY(launch_norm_bwd(s, dL, latent, gamma, rstd, d_latent, dgp, d_gamma, st));
#undef B2_TRY
  return hipSuccess;
}

hipError_t launch_absorbed_pack(const Shape& s, const float* L, const void* k_pe, void* kx, hipStream_t st) {
  if (!(s.bf16 && s.d_kv == DL && s.d_rope == DR && s.d_nope == DNQ)) return hipErrorNotSupported;
  const int64_t n = s.T * (DQ / 8);
  hipLaunchKernelGGL(absorbed_pack_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, L,
                     static_cast<const bf16_t*>(k_pe), static_cast<half_t*>(kx), s.T);
  return hipGetLastError();
}

hipError_t launch_absorbed_attn(const Shape& s, const void* q_abs, const void* q, const void* kx, float* acc,
                                float* lse, hipStream_t st) {
  if (!(s.bf16 && s.d_kv == DL && s.d_rope == DR && s.d_nope == DNQ)) return hipErrorNotSupported;
  AbsArgs a;
  a.q_abs = static_cast<const half_t*>(q_abs);
  a.q = static_cast<const bf16_t*>(q);
  a.kx = static_cast<const half_t*>(kx);
  a.acc = acc;
  a.lse = lse;
  a.S = s.S;
  a.B = static_cast<int>(s.B);
  a.h = s.h;
  a.n_rt = static_cast<int>((s.S * s.h + ROWS - 1) / ROWS);
  a.scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(s.d_nope + s.d_rope));
  const int64_t grid = static_cast<int64_t>(a.n_rt) * s.B;
  hipLaunchKernelGGL(absorbed_attn_kernel, dim3(static_cast<unsigned>(grid)), dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace laga
