// Pieces shared by the attention kernels: LDS tile staging with 16-byte
// copies and the transposing LDS read that turns a row-major [k][n] tile
// into 32x32 MFMA operand fragments.
#pragma once

#include "device.hpp"

namespace laga {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// gfx950 transposing LDS read of 16-bit elements.  Within each group of 16
// lanes, lane i receives element (i % 4) of the 8-byte words that lanes
// 4j + i/4 (j = 0..3) addressed.  If lane s of the group addresses row
// k0 + s/4, columns c0 + 4(s%4) .. +3 of a row-major tile, lane i therefore
// gets column c0 + i, rows k0 .. k0+3.
// (The address-space cast keeps the compiler's knowledge of which shared
// array is read, which global->LDS loads into another array rely on.)
__device__ __forceinline__ s16x4 ds_read_tr16(const void* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_ptr));
}

// Runs use(i, read(i)) for i = 0 .. N-1 with each read issued D uses before
// its own, rotating over D + 1 registers; the scheduling barrier after each
// use keeps that order.  Left to itself the compiler issues a read or two at
// a time and, with one wavefront per SIMD, waits out the LDS latency before
// each product.
template <int N, int D, class Frag, class Read, class Use>
__device__ __forceinline__ void pipelined(Read rd, Use use) {
  constexpr int A = D < N ? D : N;
  Frag fr[A + 1];
#pragma unroll
  for (int i = 0; i < A; ++i) fr[i] = rd(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + A < N) fr[(i + A) % (A + 1)] = rd(i + A);
    use(i, fr[i % (A + 1)]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Fragment of an operand whose k index runs down the rows of a row-major
// 16-bit tile (k = row, n = column; row pitch `ld` elements), for a 32x32x16
// atom: lane l gets column n0 + l%32 and the 8 rows
//   k0 + 4*hf + [0,4)  and  k0 + 8 + 4*hf + [0,4)      (hf = l / 32)
// which is the key order that 32x32 accumulator registers r = 8*st .. 8*st+7
// hold (see acc_key_col), so probabilities and score gradients can be fed
// straight from accumulators against this operand.
template <class E>
__device__ __forceinline__ half8 tr_frag_acc(const E* tile, int ld, int k0, int n0) {
  static_assert(sizeof(E) == 2, "16-bit tiles only");
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, s = lane % 16, hf = lane / 32;
  const int col = n0 + 16 * (g % 2) + 4 * (s % 4);
  const int row = k0 + 4 * hf + s / 4;
  s16x4 a = ds_read_tr16(tile + row * ld + col);
  s16x4 b = ds_read_tr16(tile + (row + 8) * ld + col);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(half8, r);
}

// Same, with the natural k order of the atom: lane l gets rows k0 + 8*hf + [0,8).
template <class E>
__device__ __forceinline__ half8 tr_frag(const E* tile, int ld, int k0, int n0) {
  static_assert(sizeof(E) == 2, "16-bit tiles only");
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, s = lane % 16, hf = lane / 32;
  const int col = n0 + 16 * (g % 2) + 4 * (s % 4);
  const int row = k0 + 8 * hf + s / 4;
  s16x4 a = ds_read_tr16(tile + row * ld + col);
  s16x4 b = ds_read_tr16(tile + (row + 4) * ld + col);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(half8, r);
}

// Tiles read only with transposing reads can go unpadded with an XOR swizzle
// of their 16-byte blocks: block b of row r is stored at b ^ (4 * (r % 4)).
// A transposing read takes four consecutive rows x 64 bytes per 32 lanes;
// with a row pitch of a multiple of 256 bytes the swizzle puts those four
// 64-byte spans in four different windows of the 64 banks.
__device__ __forceinline__ int swz_block(int r, int b) { return b ^ (4 * (r & 3)); }

// tr_frag_acc on a swizzled tile (ld a multiple of 128 elements, k0 % 4 == 0).
template <class E>
__device__ __forceinline__ half8 tr_frag_acc_swz(const E* tile, int ld, int k0, int n0) {
  static_assert(sizeof(E) == 2, "16-bit tiles only");
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, s = lane % 16, hf = lane / 32;
  const int row = k0 + 4 * hf + s / 4;  // row % 4 == s / 4
  const int col = 8 * swz_block(s / 4, n0 / 8 + 2 * (g % 2) + (s % 4) / 2) + 4 * (s % 2);
  s16x4 a = ds_read_tr16(tile + row * ld + col);
  s16x4 b = ds_read_tr16(tile + (row + 8) * ld + col);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(half8, r);
}

// 8-bit tiles of 128-byte rows read with ds_read_b64_tr_b8 (tr8_frag_acc64):
// 8-byte word w of row r is stored at w ^ (4 * h(r)), h(r) = bit 1 of r | bit 3
// of r << 1, i.e. 16-byte chunk c at c ^ (2 * h(r)).  The eight rows one
// half-wavefront reads (4 consecutive, twice, 8 apart) then cover all 64 banks.
__device__ __forceinline__ int swz8_h(int r) { return ((r >> 1) & 1) | (((r >> 3) & 1) << 1); }
__device__ __forceinline__ int swz8_chunk(int r, int c) { return c ^ (2 * swz8_h(r)); }

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// gfx950 transposing LDS read of 8-bit elements.  Within each group of 16
// lanes, byte j (0..7) that lane i receives is element i % 8 of the 8-byte
// word addressed by lane 2j + i/8 of the group.
__device__ __forceinline__ i32x2 ds_read_tr8(const void* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(lds_ptr));
}

// e4m3 A operand (K = 64) of a product against 32x32 accumulators fed as B:
// from a swizzled [64 keys][128 bytes] tile, lane l gets column 32 n + l % 32
// and as byte J = 16 t + r the key 32 t + 8 (r / 4) + 4 hf + r % 4, the key
// that accumulator register r of atom t holds (hf = l / 32).  Read m covers
// J = 8m .. 8m+7, i.e. keys 16m + {0..3, 8..11} + 4hf; source lane s of a
// 16-lane group addresses key row 16m + 8 (s/8) + 4 hf + (s/2) % 4 and the
// 8 columns from 32 n + 16 (g%2) + 8 (s%2) (g = l / 16).
__device__ __forceinline__ i32x8 tr8_frag_acc64(const uint8_t* tile, int n) {
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, s = lane % 16, hf = lane / 32;
  const int row = 8 * (s / 8) + 4 * hf + (s / 2) % 4;  // + 16 m; bits 1, 3 fixed by s
  const int word = 4 * (n ^ swz8_h(row)) + 2 * (g % 2) + (s % 2);
  const uint8_t* p = tile + row * 128 + 8 * word;
  i32x8 out;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const i32x2 x = ds_read_tr8(p + m * 16 * 128);
    out[2 * m] = x[0];
    out[2 * m + 1] = x[1];
  }
  return out;
}

// Load of a T from shared memory at byte offset `off` of `base`.  Pointer
// arithmetic on the shared array (rather than integer addresses) lets the
// compiler see which array is read, so loads in flight into another array are
// not waited for.
template <class T>
__device__ __forceinline__ T lds_at(const void* base, uint32_t off) {
  return *reinterpret_cast<const T*>(static_cast<const char*>(base) + off);
}

// 16 bytes per lane from a buffer resource straight into LDS: lane l's bytes
// land at lds_window + 16 l (lds_window wave-uniform); offsets outside the
// resource's range read as zero.  The wave's later s_waitcnt on loads covers
// the LDS write.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, void* lds_window, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(lds_window), 16, voffset, 0, 0, 0);
}

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left at their maximum.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS data written by ds_write only: wait for this
// wave's LDS operations, then s_barrier, with a compiler memory barrier so no
// LDS access moves across it.  Unlike __syncthreads it does not wait for the
// global->LDS loads in flight into another buffer.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left at their maximum
  asm volatile("s_barrier" ::: "memory");
}

// Barrier after global->LDS loads: wait for this wave's loads (vmcnt(0);
// expcnt and lgkmcnt left at their maximum), then __syncthreads.  The
// compiler tracks such loads only as register writes, not as LDS writes: at a
// loop head it may issue the barrier with loads still in flight, so that a
// wave reads rows that another wave's load has not yet written.
__device__ __forceinline__ void dma_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
}

// One 16-byte chunk of a [rows x cols] tile copied from global memory:
// row r of the source starts at src + r*ld (elements), rows >= nrows read as 0.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <class T>
__device__ __forceinline__ u32x4 load_chunk(const T* src, int64_t ld, int r, int c, int nrows) {
  if (r < nrows) return *reinterpret_cast<const u32x4*>(src + r * ld + c);
  return u32x4{0u, 0u, 0u, 0u};
}

template <class T>
__device__ __forceinline__ void store_chunk(T* dst, int ld, int r, int c, u32x4 v) {
  *reinterpret_cast<u32x4*>(dst + r * ld + c) = v;
}

}  // namespace laga
