// Shared device helpers of the DSA kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTileQ = 128;  // attention tile rows (queries); the tile-class grid
constexpr int kTileK = 64;   // attention tile columns (keys); one u64 mask word

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// float -> bf16 bits, round to nearest even (NaN stays NaN): the IEEE
// narrowing conversion, which gfx950 does in hardware (v_cvt_pk_bf16_f32)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// eight floats as eight bf16 (round to nearest even): one MFMA operand fragment
__device__ __forceinline__ u32x4 pack8(const float* x) {
  return u32x4{pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), pack_bf2(x[4], x[5]), pack_bf2(x[6], x[7])};
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ void store(float* p, float x) { *p = x; }
};
template <> struct Elem<uint16_t> {
  __device__ static __forceinline__ float load(const uint16_t* p) { return bf2f(*p); }
  __device__ static __forceinline__ void store(uint16_t* p, float x) { *p = f2bf(x); }
};

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_32x32x16_bf16. Lane l supplies A[m = l%32][k = 8*(l/32) + i] and
// B[k = 8*(l/32) + i][n = l%32], i = 0..7, and holds
// C[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32] in register r = 0..15.
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// row of accumulator register r for lane-half h (h = lane / 32)
__device__ __forceinline__ constexpr int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// A-operand fragment of v_mfma_f32_32x32x16_bf16 read *transposed* from a
// natural row-major LDS tile X[k][m] (m contiguous, `pitch` elements per row)
// with ds_read_b64_tr_b16. Lane l receives A[m][k] = X[k][m] for
// m = mbase + l%32 and the eight k rows {kr0..kr0+3, kr1..kr1+3}, where kr0/kr1
// are this lane-half's rows (they may differ between halves). Within each
// 16-lane group, the instruction hands lane i element (i%4) of the 4-element
// chunk of source lane (i/4 + 4*slot). So source lane j points at row
// kr + j/4, columns m0 + 4*(j%4) .. +3, and lane i gets column m0 + i.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;
__device__ __forceinline__ u32x4 lds_tr_frag(const uint16_t* X, int pitch, int kr0, int kr1, int mbase) {
  const int lane = threadIdx.x & 63, j = lane & 15;
  const int m0 = mbase + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(X + (kr0 + (j >> 2)) * pitch + m0));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(X + (kr1 + (j >> 2)) * pitch + m0));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

// Tiles whose rows are read both ways -- b128 fragment reads of 16
// consecutive rows at one chunk, and transposing reads of 4 rows x 4 chunks --
// are stored with a padded pitch and the low two bits of each 16-byte chunk
// index XORed with bits 2-3 of the row: chunk c of row r sits at chunk
// c ^ ((r >> 2) & 3). With a pitch of 20 chunks (128-element rows) or 28
// chunks (192-element rows), both read patterns touch 16 distinct 4-bank
// groups of the 64 LDS banks.
__device__ __forceinline__ int swz_chunk(int r, int c) { return c ^ ((r >> 2) & 3); }

// b128 A/B fragment of a swizzled tile: row r, logical chunk c (8 elements)
__device__ __forceinline__ u32x4 lds_frag_x(const uint16_t* X, int pitch, int r, int c) {
  return *(const u32x4*)(X + r * pitch + swz_chunk(r, c) * 8);
}

// lds_tr_frag on a swizzled tile (kr0, kr1 multiples of 4, mbase of 32)
__device__ __forceinline__ u32x4 lds_tr_frag_x(const uint16_t* X, int pitch, int kr0, int kr1, int mbase) {
  const int lane = threadIdx.x & 63, j = lane & 15;
  const int m0 = mbase + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const int ra = kr0 + (j >> 2), rb = kr1 + (j >> 2);
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16_ptr)(X + ra * pitch + swz_chunk(ra, m0 >> 3) * 8 + (m0 & 7)));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16_ptr)(X + rb * pitch + swz_chunk(rb, m0 >> 3) * 8 + (m0 & 7)));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Inclusive prefix sum over the 64 lanes of a wave with DPP: four row shifts
// give each 16-lane row its own prefix, then row 0's total is broadcast into
// rows 1 and 3, and rows 0-1's total into rows 2 and 3. Lanes read zero past a
// row's edge. No LDS round trip (a __shfl_up scan is six ds_bpermute waits).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Asynchronous global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's bytes land at lds_base + 16*l, so one wave fills a contiguous 1 KB
// block. `lds_base` must be wave-uniform. Completion is waited for with
// wait_vmem() before the barrier that publishes the block.
__device__ __forceinline__ void g2lds16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)gsrc,
                                   (void __attribute__((address_space(3)))*)lds_base, 16, 0, 0);
}
// 4 bytes per lane (global_load_lds_dword): lane l's word lands at lds_base + 4*l
__device__ __forceinline__ void g2lds4(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)gsrc,
                                   (void __attribute__((address_space(3)))*)lds_base, 4, 0, 0);
}
// The same copies issued through inline assembly. The compiler then does not
// track them as LDS writes, so it inserts no wait for every outstanding load
// before LDS reads it cannot prove disjoint from them (with dynamically indexed
// buffers it never can). The caller waits for them explicitly (wait_vmem or
// wait_vmem_n) before the barrier that publishes them; waits the compiler
// computes for its own loads stay correct, since loads complete in issue order.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
// M0 (the LDS base of the copy) is saved and restored around it: M0 is a
// register the compiler allocates itself (LDS-parameter, readlane-index and
// message uses), and an asm statement cannot declare it clobbered, so a value
// the compiler holds there must survive the copy. The two scalar moves cost
// little beside the copy itself, whose issue stalls the wave for ~100+ cycles
// when several are queued.
__device__ __forceinline__ void g2lds16_async(const void* gsrc, void* lds_base) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
               "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(save) : "v"(gsrc), "s"(lds_addr(lds_base)) : "memory");
}
// A wave-uniform pointer moved to SGPRs (read from the first active lane).
template <typename T> __device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return (T*)(uintptr_t)((hi << 32) | lo);
}
// The same 16-byte copy from a wave-uniform base (SGPR pair) plus a per-lane
// 32-bit byte offset: no 64-bit address arithmetic per lane. `gbase` must be
// wave-uniform and held in SGPRs (see uniform_ptr).
__device__ __forceinline__ void g2lds16_async_off(const void* gbase, uint32_t off, void* lds_base) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
               "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(save) : "v"(off), "s"(gbase), "s"(lds_addr(lds_base)) : "memory");
}
// ... with the non-temporal hint, for data read exactly once
__device__ __forceinline__ void g2lds16_async_off_nt(const void* gbase, uint32_t off, void* lds_base) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
               "global_load_lds_dwordx4 %1, %2 nt\n\ts_mov_b32 m0, %0"
               : "=&s"(save) : "v"(off), "s"(gbase), "s"(lds_addr(lds_base)) : "memory");
}
// 4 bytes per lane from a wave-uniform base (SGPR pair) plus a per-lane byte offset
__device__ __forceinline__ void g2lds4_async_off(const void* gbase, uint32_t off, void* lds_base) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
               "global_load_lds_dword %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(save) : "v"(off), "s"(gbase), "s"(lds_addr(lds_base)) : "memory");
}
__device__ __forceinline__ void g2lds4_async(const void* gsrc, void* lds_base) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
               "global_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(save) : "v"(gsrc), "s"(lds_addr(lds_base)) : "memory");
}
// Wait until at most N vector-memory instructions of this wave are in flight
// (they complete in issue order). Issued through the builtin, so that the
// compiler's own wait insertion knows the loads before it are complete.
// Encoding (gfx9): vmcnt in bits 3:0 and 15:14; expcnt (bits 6:4) and lgkmcnt
// (bits 11:8) left at their maxima.
template <int N> __device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_vmem() { wait_vmem_n<0>(); }
// Workgroup barrier that publishes this wave's LDS writes (ds_write; LDS-DMA
// copies count as vector-memory instructions and are waited for separately)
// without the wait for every outstanding global load that __syncthreads()'s
// release fence adds. The memory clobber keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Workgroups of a 1-D grid are dealt round-robin to the 8 XCDs, each with
// its own L2. Remap the block id so that each XCD works through one contiguous
// range of logical blocks; blocks that share operands (same batch and head)
// then share an L2. The tail beyond a multiple of 8 keeps its id.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int NX = 8;
  const int per = nblocks / NX;
  if (bid >= per * NX) return bid;
  return (bid % NX) * per + bid / NX;
}

// Order of the query-major attention grids: logical block L -> (bh, qb) with
// nq query blocks per (batch, head) of decreasing cost (qb = nq-1 first).
// Blocks are taken in groups of two (batch, head) pairs; within a group the
// costliest blocks of both pairs come first. The pairs of a group still run
// together (they share an XCD's L2), and the last blocks dispatched anywhere
// are short ones, so the causal triangle's long blocks do not end up alone
// at the tail of the grid.
__device__ __forceinline__ void grouped_order(int L, int nq, int nbh, int& bh, int& qb) {
  constexpr int G = 2;
  const int bh0 = L / (G * nq) * G;
  const int g = min(G, nbh - bh0);
  const int r = L - bh0 * nq;
  qb = nq - 1 - r / g;
  bh = bh0 + r % g;
}

// 64-key tiles of the longest sequence: the attention kernels stage a
// workgroup's tile-class rows (one byte per tile) in LDS at start, so that
// walking the tiles reads LDS instead of waiting on global loads that would
// also wait for the tile copies in flight.
constexpr int kMaxTiles = kMaxS / kTileK;

// n bytes from global memory to LDS, by the whole workgroup; the caller
// publishes them with a barrier
__device__ __forceinline__ void stage_bytes(uint8_t* dst, const uint8_t* src, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = src[i];
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// x(l) + x(l ^ 32) and max(x(l), x(l ^ 32)) in every lane through
// v_permlane32_swap, which trades the upper half of its first operand with the
// lower half of its second: with both operands x, the first result holds the
// lower half's values in both halves and the second the upper half's.
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Wave reductions with DPP (no LDS round trips): the row shifts and row
// broadcasts of wave_incl_scan, with lanes past a row's edge or outside the
// row mask reading the identity; lane 63 ends with the whole wave's result,
// which every lane then reads.
template <int CTRL, int RMASK>
__device__ __forceinline__ int dpp_or(int identity, int x) {
  return __builtin_amdgcn_update_dpp(identity, x, CTRL, RMASK, 0xf, false);
}
template <typename Op>
__device__ __forceinline__ int wave_reduce_bits(int x, int identity, Op op) {
  x = op(x, dpp_or<0x111, 0xf>(identity, x));
  x = op(x, dpp_or<0x112, 0xf>(identity, x));
  x = op(x, dpp_or<0x114, 0xf>(identity, x));
  x = op(x, dpp_or<0x118, 0xf>(identity, x));
  x = op(x, dpp_or<0x142, 0xa>(identity, x));
  x = op(x, dpp_or<0x143, 0xc>(identity, x));
  return __builtin_amdgcn_readlane(x, 63);
}
__device__ __forceinline__ float wave_max(float x) {
  return __int_as_float(wave_reduce_bits(__float_as_int(x), __float_as_int(-INFINITY), [](int a, int b) {
    return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
  }));
}
__device__ __forceinline__ float wave_min(float x) {
  return __int_as_float(wave_reduce_bits(__float_as_int(x), __float_as_int(INFINITY), [](int a, int b) {
    return __float_as_int(fminf(__int_as_float(a), __int_as_float(b)));
  }));
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  return (uint32_t)wave_reduce_bits((int)x, 0, [](int a, int b) { return (int)((uint32_t)a + (uint32_t)b); });
}
__device__ __forceinline__ float wave_sumf(float x) {
  return __int_as_float(wave_reduce_bits(__float_as_int(x), 0, [](int a, int b) {
    return __float_as_int(__int_as_float(a) + __int_as_float(b));
  }));
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t x) {
  return (uint32_t)wave_reduce_bits((int)x, -1, [](int a, int b) { return (int)min((uint32_t)a, (uint32_t)b); });
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
  return (uint32_t)wave_reduce_bits((int)x, 0, [](int a, int b) { return (int)max((uint32_t)a, (uint32_t)b); });
}

// order-preserving map float -> u32 (larger float => larger key; -0 == +0)
__device__ __forceinline__ uint32_t fkey(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace dsa
