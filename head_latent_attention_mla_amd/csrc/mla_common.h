// Device-side helpers shared by the libmla kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mla_internal.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// Cache-policy operand of the direct-to-LDS tile loads of the bf16 latent
// scans: the nontemporal (streaming) bit of the gfx950 memory instructions.
// A scan reads each cached row once per work-group, so the lines are marked
// for early eviction and the data that is read again (the latent queries, the
// absorption weights of the next step) stays in the caches.  The E4M3 scans
// keep the default policy: their query-row groups read each tile through L2
// at different times, and with the hint 10-27% more of it came from HBM.
constexpr int CPOL_STREAM = 2;

// XOR pattern applied to the 16-byte chunk index of LDS row t.  For any 8
// consecutive rows starting at a multiple of 8 it is a permutation of 0..7
// (MFMA fragment reads: 8 lanes x 16 B on 8 rows hit distinct banks), and for
// 4 consecutive rows starting at a multiple of 4 the chunk pairs {c, c^1}
// (c even) map to 8 distinct chunks (transpose reads: 4 rows x 32 B).
__device__ __forceinline__ int chunk_swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

// gfx950 transpose read: within each group of 16 lanes, lane j reads 4
// consecutive 16-bit elements at its own address; lane i of the group then
// holds element (i % 4) of lanes 4e + i/4, e = 0..3.  Used so that a lane
// whose address points at row (base + j/4), column (cb + 4 (j%4)) receives
// the four rows base..base+3 of column cb + i.
__device__ __forceinline__ i16x4 ds_read_tr16(const char* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lds_ptr));
}

__device__ __forceinline__ bf16x8 join_tr(i16x4 lo, i16x4 hi) {
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// MFMA with the accumulator pinned to VGPRs (for accumulators that the VALU
// reads right after).  The hazard recognizer does not see inside inline asm:
// after the last of these, call mfma_v_drain() on the accumulators before any
// other instruction reads them (an MFMA result needs 12 wait states before a
// VALU read on gfx950; the drain gives 16).  Back-to-back MFMAs accumulating
// into the same registers need no wait states.
__device__ __forceinline__ void mfma32_v0(f32x16& c, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_v(f32x16& c, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_drain(f32x16& c0, f32x16& c1) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(c0), "+v"(c1));
}

// XOR pattern of the 16-byte chunk index (low 3 bits) of a bf16 latent-cache
// tile row t (tiles stored row-major, 1152 bytes per row).  A
// 128-bit LDS read is served 16 lanes per pass from 64 banks (256 bytes); a
// score-fragment read puts 16 consecutive tile rows, 1152 bytes apart (128
// mod 256), in one pass, so rows of equal parity in any aligned run of 16
// need distinct XORs: bit 1 of t selects bit 2 of the XOR and bits 2..3 of
// t its bits 0..1.  The transposed value reads (4 consecutive rows x 32
// bytes) stay conflict-free: rows 4q and 4q + 2 differ in XOR bit 2.
// tile_swz(t + 16) = tile_swz(t) and tile_swz(t + 8) = tile_swz(t) ^ 2.
__device__ __forceinline__ int tile_swz(int t) { return (((t >> 1) & 1) << 2) | ((t >> 2) & 3); }

// Compile-time loop: f(std::integral_constant<int, I>{}) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}

// LDS reads issued as inline asm.  The compiler does not track these: every
// consumer must first pass the loaded registers through wait_lgkm<N>(), which
// waits until at most N LDS operations are outstanding (LDS operations of a
// wave complete in order).  Used in the hot loops because the compiler's own
// waits are conservative while direct-to-LDS loads are in flight.
template <int OFF>
__device__ __forceinline__ void lds_read_b128(i16x8& d, uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void lds_read_tr16(i16x4& d, uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "i"(OFF));
}
template <typename R>
__device__ __forceinline__ void touch_reg(R& r) {
  asm volatile("" : "+v"(r));
}
template <int N, typename... R>
__device__ __forceinline__ void wait_lgkm(R&... regs) {
  static_assert(N >= 0 && N < 16, "lgkmcnt");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N));
  (touch_reg(regs), ...);   // consumers depend on these, so they follow the wait
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// round-to-nearest-even float -> bf16 (hardware conversion on gfx950)
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

__device__ __forceinline__ uint16_t bf16_bits(__bf16 x) { return __builtin_bit_cast(uint16_t, x); }

// Split partial outputs: four consecutive values of a partial row, stored as
// fp32 or as bf16 (rounded to nearest even).  PartRaw is what a load returns
// (the values still packed), part_vals unpacks it.
template <bool PB16>
using PartRaw = typename std::conditional<PB16, uint64_t, f32x4>::type;

template <bool PB16>
__device__ __forceinline__ PartRaw<PB16> part_load(const void* base, int64_t elem) {
  if constexpr (PB16) return *(const uint64_t*)((const uint16_t*)base + elem);
  else return *(const f32x4*)((const float*)base + elem);
}

template <bool PB16>
__device__ __forceinline__ f32x4 part_vals(PartRaw<PB16> r) {
  if constexpr (PB16) {
    const uint32_t lo = (uint32_t)r, hi = (uint32_t)(r >> 32);
    return f32x4{__builtin_bit_cast(float, lo << 16), __builtin_bit_cast(float, lo & 0xFFFF0000u),
                 __builtin_bit_cast(float, hi << 16), __builtin_bit_cast(float, hi & 0xFFFF0000u)};
  } else {
    return r;
  }
}

// (two v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint64_t pack_bf16x4(f32x4 v) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(uint64_t, __builtin_convertvector(v, bf16x4_t));
}

__device__ __forceinline__ void part_store(void* base, int64_t elem, f32x4 v, bool pb16) {
  if (pb16) *(uint64_t*)((uint16_t*)base + elem) = pack_bf16x4(v);
  else *(f32x4*)((float*)base + elem) = v;
}

// Work-group barriers that wait only for what the barrier publishes.
// __syncthreads() would also wait for the prefetch of the next tile (vmcnt).
__device__ __forceinline__ void barrier_tile_ready() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// acc *= alpha on an accumulator that lives in AGPRs, one register at a time
// (a plain vector multiply makes the register allocator move the whole block
// through VGPRs).
__device__ __forceinline__ void scale_acc(f32x16& acc, float alpha) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float x = acc[i];
    float t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(x), "=&v"(t) : "v"(alpha));
    acc[i] = x;
  }
}

// lanes l and l ^ 32 hold the same query row: combine their values.
// v_permlane32_swap exchanges the upper half of one register with the lower
// half of another, so swapping x with a copy of x leaves {x[l], x[l ^ 32]} in
// the two registers of every lane.  Issued as inline asm: the compiler's own
// builtin is treated as returning two equal values and one gets folded away.
// The s_nop padding covers the VALU-write -> permlane-read hazard and the
// permlane-write -> VALU-read hazard.
__device__ __forceinline__ void halves(float x, float& a, float& b) {
  a = x;
  b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
// max of three, without the NaN-quieting the compiler adds around fmaxf on
// values it cannot see (scores are finite or -inf)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float max_halves(float x) {
  float a, b;
  halves(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_halves(float x) {
  float a, b;
  halves(x, a, b);
  return a + b;
}

}  // namespace mla
