// Device-side helpers shared by the BAM attention kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bam {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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

// acc + lo + hi of a packed bf16 pair (v_dot2_f32_bf16 against (1, 1), fp32 accumulate)
__device__ __forceinline__ float sum_bf16x2(uint32_t packed, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, acc, false);
}

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Per-head SSMax factor c = s ln(n) (natural log); 1 with SSMax off.
__device__ __forceinline__ float ssmax_c(bool ssmax, float s, int n) {
  return ssmax ? s * __logf((float)n) : 1.0f;
}

// Lane exchange with lane ^ 32 (the other half of a wave64).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// max(x, x of lane ^ 32) without an LDS round trip: v_permlane32_swap of x with itself
// leaves, in each lane, one copy of its own value and one of its partner's.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace bam

namespace bam {

// XOR swizzle (Gray code of the row) of the 16-byte chunks of a row-major bf16 tile in
// LDS, so 16-byte reads of one chunk column across consecutive rows spread over banks.
__device__ __forceinline__ int swz_chunk(int r, int mask) { return (r ^ (r >> 1)) & mask; }

// Stage ROWS rows x DH bf16 (rows row0 .. row0 + ROWS - 1 of a [*, DH] tensor; rows at or
// beyond nvalid are zero) into LDS row-major with swizzled 16-byte chunks.
template <int DH, int ROWS, int NT>
__device__ __forceinline__ void stage_rows(const uint16_t* __restrict__ src, int row0, int nvalid,
                                           uint16_t* dst, int tid) {
  constexpr int KCH = DH / 8;
  for (int cidx = tid; cidx < ROWS * KCH; cidx += NT) {
    const int r = cidx / KCH;
    const int ch = cidx - r * KCH;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (row0 + r < nvalid) val = *(const u32x4*)(src + (size_t)(row0 + r) * DH + ch * 8);
    *(u32x4*)(dst + r * DH + (ch ^ swz_chunk(r, KCH - 1)) * 8) = val;
  }
}

// 16-byte read of chunk `ch` of row `r` from a tile staged by stage_rows.
template <int DH>
__device__ __forceinline__ u32x4 read_chunk(const uint16_t* tile, int r, int ch) {
  return *(const u32x4*)(tile + r * DH + (ch ^ swz_chunk(r, DH / 8 - 1)) * 8);
}

// Stage ROWS rows x DH bf16 transposed into LDS: dst[e * STRIDE + r] = src[row0 + r][e]
// (zero for rows at or beyond nvalid).  Two rows are packed per 32-bit LDS write.
template <int DH, int ROWS, int NT, int STRIDE>
__device__ __forceinline__ void stage_rows_T(const uint16_t* __restrict__ src, int row0, int nvalid,
                                             uint16_t* dst, int tid) {
  constexpr int KCH = DH / 8;
  for (int pidx = tid; pidx < (ROWS / 2) * KCH; pidx += NT) {
    const int p = pidx % (ROWS / 2);
    const int ch = pidx / (ROWS / 2);
    const int r0 = 2 * p;
    u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
    if (row0 + r0 < nvalid) v0 = *(const u32x4*)(src + (size_t)(row0 + r0) * DH + ch * 8);
    if (row0 + r0 + 1 < nvalid) v1 = *(const u32x4*)(src + (size_t)(row0 + r0 + 1) * DH + ch * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w0 = v0[e >> 1], w1 = v1[e >> 1];
      const uint32_t packed = (e & 1) ? __builtin_amdgcn_perm(w1, w0, 0x07060302u)
                                      : __builtin_amdgcn_perm(w1, w0, 0x05040100u);
      *(uint32_t*)(dst + (ch * 8 + e) * STRIDE + r0) = packed;
    }
  }
}

// MFMA operand of 8 bf16 whose contraction index runs over rows {c, c+1, c+2, c+3,
// c+8, .., c+11} of column `row` of a transposed tile (the order in which a 32x32
// accumulator holds them in one lane half).
template <int STRIDE>
__device__ __forceinline__ bf16x8 read_T_operand(const uint16_t* tileT, int row, int col) {
  const u32x2 lo = *(const u32x2*)(tileT + row * STRIDE + col);
  const u32x2 hi = *(const u32x2*)(tileT + row * STRIDE + col + 8);
  const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
  return as_bf16x8(av);
}

}  // namespace bam
