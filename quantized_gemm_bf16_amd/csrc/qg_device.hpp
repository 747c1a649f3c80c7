// Device primitives for gfx950 (CDNA4): vector types, buffer resources,
// global->LDS direct loads, MFMA wrappers, conversions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zero (this is how tile tails along M/N and masked K chunks read 0).
// Base and size are workgroup-uniform; readfirstlane lets the compiler keep
// the descriptor in SGPRs (a VGPR descriptor would need a waterfall loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* q = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Offset that is always outside a resource (resources are < 2^31 bytes here).
constexpr uint32_t kOOB = 0x80000000u;

// 128-bit buffer descriptor as four dwords (gfx9 layout: base address,
// stride 0, num_records, dword3 flags), for use in inline assembly.
__device__ __forceinline__ i32x4 make_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  return i32x4{(int)__builtin_amdgcn_readfirstlane((uint32_t)p),
               (int)(__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) & 0xFFFF),
               (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}

// One 16-byte chunk per lane, written to LDS at lds_wave_base + 16 * lane
// (buffer_load_dwordx4 ... lds; M0 holds the wave's LDS base). Issued from
// inline assembly on purpose: the compiler cannot tell which part of LDS an
// in-flight direct load writes, so for loads it knows about it waits for all
// of them (vmcnt 0) before every LDS read, draining a multi-stage ring. The
// callers wait for exactly the loads they need with wait_vmcnt<N>() instead.
__device__ __forceinline__ void load_lds_x4(const i32x4& rsrc, void* lds_wave_base, uint32_t voff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds_wave_base);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(m0v), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}
// One dword per lane, written to LDS at lds_wave_base + 4 * lane (inline
// assembly for the same reason as load_lds_x4).
__device__ __forceinline__ void load_lds_x1a(const i32x4& rsrc, void* lds_wave_base, uint32_t voff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds_wave_base);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(m0v), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}

// A copy of a workgroup-uniform value that the compiler cannot move out of
// the branch it is taken in (an empty volatile asm with the value tied to its
// output). Code that depends on the copy stays inside a rarely taken branch
// instead of being hoisted out of the loop around it, where its results
// would occupy registers (or spill) for the whole loop.
__device__ __forceinline__ uint32_t pinned(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}

// Zeroes, in LDS, the bytes of a 16-byte chunk from byte `keep` on
// (0 < keep < 16). When K * element size is not a multiple of 16, the chunk
// that holds the end of a row's K elements also holds bytes past K (row
// padding with undefined contents, possibly NaN); they must read as zero
// before any MFMA consumes the chunk, as out-of-range chunks do. Called by
// the lane whose direct load wrote the chunk, after waiting for that load;
// the caller's barrier (or, within one wave, LDS ordering) publishes it.
__device__ __forceinline__ void lds_chunk_trim(char* p, int keep) {
  asm volatile("" ::: "memory");
  i32x4 x = *(const i32x4*)p;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int vb = keep - 4 * d;  // bytes of dword d that lie before K
    const uint32_t m = vb >= 4 ? ~0u : (vb <= 0 ? 0u : (1u << (8 * vb)) - 1u);
    x[d] = (int)((uint32_t)x[d] & m);
  }
  *(i32x4*)p = x;
  asm volatile("" ::: "memory");
}

// 16-byte buffer store / load with the sc1 cache-policy bit (coherent at agent
// scope across the XCDs' L2s; gfx950 cache-policy encoding: sc0 = 1, nt = 2,
// sc1 = 16).
__device__ __forceinline__ void store_sc1_x4(__amdgpu_buffer_rsrc_t r, uint32_t voff, i32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, 0, 16);
}
__device__ __forceinline__ i32x4 load_sc1_x4(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 16));
}

// Plain 16-byte buffer load into registers (zero outside the resource).
__device__ __forceinline__ i32x4 load_x4(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt low 4 bits in [3:0], high 2 bits in [15:14]; expcnt [6:4] and
// lgkmcnt [11:8] left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for the LDS ring. __syncthreads() carries a workgroup
// release fence, which the compiler implements as a wait for ALL outstanding
// vector-memory operations -- that would drain every prefetched stage. Here
// the caller has already waited for exactly the loads it needs (wait_vmcnt);
// this waits for the wave's own LDS reads (lgkmcnt 0) and meets the other
// waves. The empty asm statements keep the compiler from moving LDS accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- MFMA (32x32 output tile per instruction) ------------------------------
// Operand lane layout: lane l supplies row (l % 32) of its operand and the
// k-slice selected by l / 32; the output element r of lane l is
// row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
__device__ __forceinline__ f32x16 mfma_bf16(i32x4 a, i32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(i32x4 a, i32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ i32x16 mfma_i8(i32x4 a, i32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
// OCP e4m3 x e4m3, 64-deep; unit scales (E8M0 127 = 2^0).
__device__ __forceinline__ f32x16 mfma_e4m3(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// ---- conversions ---------------------------------------------------------
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);  // RNE (v_cvt_pk_bf16_f32)
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);  // RNE
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Wave and lane ids.
__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

}  // namespace qg
