// Device-side helpers shared by the BAM attention kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bam {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// bf16 bits -> float (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Per-head SSMax factor c = s ln(n) (natural log); 1 with SSMax off.
__device__ __forceinline__ float ssmax_c(bool ssmax, float s, int n) {
  return ssmax ? s * __logf((float)n) : 1.0f;
}

// max(a, b, c).  Written in C on purpose: an inline-asm v_max3_f32 is opaque to the
// compiler's hazard checks, which then do not wait for a preceding MFMA to finish writing
// the registers it reads.
__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// Lane exchange with lane ^ 32 (the other half of a wave64).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// max(x, x of lane ^ 32) without an LDS round trip: v_permlane32_swap of x with itself
// leaves, in each lane, one copy of its own value and one of its partner's.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// XOR swizzle (Gray code of the row) of the 16-byte chunks of a row-major bf16 tile in
// LDS, so 16-byte reads of one chunk column across consecutive rows spread over banks
// (the row swizzle of head sizes other than 64, below).
__device__ __forceinline__ int swz_chunk(int r, int mask) { return (r ^ (r >> 1)) & mask; }

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define BAM_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Buffer resource for raw (unswizzled) buffer loads of `bytes` bytes from `base`; every
// field is made wave-uniform.  Loads whose VGPR offset is at or beyond `bytes` return zeros.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// Direct buffer -> LDS loads (lane l writes lds_base + size * l), written as inline
// assembly so the compiler does not track them: its own tracking of such loads makes every
// later LDS read wait for all of them, which would drain the prefetch of later tiles.  The
// caller orders them with BAM_WAIT_VMCNT / BAM_BARRIER_VMCNT (each load counts once).
// `soff` and `lds_base` must be wave-uniform.
//
// Every buffer load written as inline assembly starts with BAM_VMEM_SGPR_NOPS.  Its SGPR
// operands (the offset, the resource) are often written by v_readfirstlane just before it,
// and on this architecture a vector-memory instruction that reads an SGPR written by a VALU
// instruction needs five wait states first; the compiler enforces that for the instructions
// it emits, but not for inline assembly (a load that read a stale offset returned zeros).
// The same nops cover the one wait state between writing M0 and an LDS-direct load.
#define BAM_VMEM_SGPR_NOPS "s_nop 4\n\t"
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p);
}
__device__ __forceinline__ void lds_dma16(const i32x4& rsrc, uint32_t voff, uint32_t soff, void* lds_base) {
  asm volatile(BAM_VMEM_SGPR_NOPS "buffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)), "{m0}"(lds_addr(lds_base))
               : "memory");
}
__device__ __forceinline__ void lds_dma4(const i32x4& rsrc, uint32_t voff, uint32_t soff, void* lds_base) {
  asm volatile(BAM_VMEM_SGPR_NOPS "buffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)), "{m0}"(lds_addr(lds_base))
               : "memory");
}

// Transposing LDS read (gfx950): in each group of 16 lanes, lane i receives element i of
// the 4-element rows read by lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// Row swizzle of the 16-byte chunks of a 128-byte (Dh = 64) row in LDS: with m = row / 2,
// s = m ^ ((m & 1) << 2).  The 16 rows read by 16 lanes of a K operand read then hit 16
// distinct chunk slots of the 256-byte bank space, and the 4 rows x 4 chunks of each half
// wave of a transposing V read do too.  Other head sizes use the Gray code of the row.
template <int DH>
__device__ __forceinline__ int vswz(int r) {
  if (DH == 64) {
    const int mm = r >> 1;
    return (mm ^ ((mm & 1) << 2)) & 7;
  }
  return swz_chunk(r, DH / 8 - 1);
}

// A wave-uniform float read through the constant address space, which the compiler lowers
// to a scalar load (s_load_dword into an SGPR, waited for on lgkmcnt): it does not queue
// behind the vector loads in flight, and waiting for it does not wait for them.
__device__ __forceinline__ float uniform_load(const float* p) {
  return *(const __attribute__((address_space(4))) float*)p;
}

// s_waitcnt with only the vector-memory counter constrained (expcnt / lgkmcnt left at max)
#define BAM_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// Work-group barrier that waits only for this wave's LDS operations and for all but the
// newest `n` of its vector-memory operations (direct-to-LDS loads still in flight for
// later tiles).  __syncthreads() would drain every outstanding load at each barrier.
// The empty asm statements keep the compiler from moving memory operations across it.
#define BAM_BARRIER_VMCNT(n)                                                          \
  do {                                                                                \
    asm volatile("" ::: "memory");                                                    \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (0 << 8)); \
    __builtin_amdgcn_s_barrier();                                                     \
    asm volatile("" ::: "memory");                                                    \
  } while (0)

}  // namespace bam
