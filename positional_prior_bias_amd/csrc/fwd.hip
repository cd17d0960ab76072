// BAM attention prefill forward for gfx950.
//
// Semantics ("ALiBi: Attention with Linear Biases", "Code"; "Résumé Technique :
// Mécanisme d'Attention Bayésienne (BAM)", "Solution Proposée : GGD-BAM"):
//   logit_ij = c_i (q_i.k_j / sqrt(Dh) + b_h(i - j)),  O = softmax_j(logit) V.
// Flash-style: one pass over key tiles with an online softmax in the exp2 domain;
// the exact result of the dense definition up to float rounding.
//
// bf16 kernel design (wave64, v_mfma_f32_32x32x16_bf16):
//   * A work-group of 4 waves owns 128 query rows of one (b, h); each wave owns 32.
//   * S^T = K Q^T is computed with keys as MFMA rows and queries as columns, so each
//     lane owns one query (column) and 16 keys per 32x32 block; the row max / sum of
//     the softmax is an in-lane reduction plus one exchange with lane ^ 32.
//   * The bias enters as the MFMA accumulator's initial value: the accumulator is
//     loaded with sqrt(Dh) * b(i - j) from a window of the per-head distance table
//     staged in LDS, so the MFMA returns q.k + sqrt(Dh) b directly.  Distances the
//     causal mask forbids hold -inf in that window, so masking is free as well.
//   * O^T = V^T P^T: P^T is fed from the S^T accumulators without any lane exchange
//     by letting the MFMA's contraction index run over the keys in the order the
//     accumulator holds them; V is staged transposed in LDS to match.
//   * K tiles are staged in LDS with 16-byte chunks XOR-swizzled by row (Gray code)
//     so the 16-byte operand reads of 32 rows do not collide in banks.
#include <float.h>

#include "bam_device.h"
#include "bam_internal.h"

namespace bam {

namespace {

constexpr int kMQ = 128;   // query rows per work-group (4 waves x 32)
constexpr int kNK = 64;    // keys per tile
constexpr int kTW = kMQ + kNK;  // distance-window entries per tile

__device__ __forceinline__ int swz(int r, int mask) { return (r ^ (r >> 1)) & mask; }

template <int DH, bool CAUSAL>
__global__ void __launch_bounds__(256, 2) fwd_bf16_kernel(FwdArgs a, int nqb) {
  constexpr int KCH = DH / 8;          // 16-byte chunks per K row
  constexpr int KS = DH / 16;          // MFMA k-steps over the head dimension
  constexpr int DB = DH / 32;          // 32-row blocks of O^T
  constexpr int VTS = kNK + 4;         // bf16 per V^T row (padded against bank conflicts)

  __shared__ __attribute__((aligned(16))) uint16_t Ks[kNK * DH];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[DH * VTS];
  __shared__ float tw[kTW];

  const int BH = a.B * a.H;
  const int bid = blockIdx.x;
  int qb = bid / BH;
  const int bh = bid - qb * BH;
  if (CAUSAL) qb = nqb - 1 - qb;  // longest rows first
  const int h = bh % a.H;
  const int T = a.T;
  const size_t base = (size_t)bh * T * DH;
  const uint16_t* __restrict__ Q = (const uint16_t*)a.q + base;
  const uint16_t* __restrict__ K = (const uint16_t*)a.k + base;
  const uint16_t* __restrict__ V = (const uint16_t*)a.v + base;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ql = lane & 31;
  const int hh = lane >> 5;
  const int i0 = qb * kMQ;
  const int i = i0 + wave * 32 + ql;

  // Q^T operand: lane holds q_i[16 ks + 8 hh .. + 7]
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (i < T) w = *(const u32x4*)(Q + (size_t)i * DH + 16 * ks + 8 * hh);
    qf[ks] = as_bf16x8(w);
  }

  const float sqrtD = __builtin_sqrtf((float)DH);
  const int n_i = CAUSAL ? i + 1 : T;
  const float c = ssmax_c(a.ssmax, a.ssmax ? a.s[h] : 1.0f, n_i);
  // logit in log2 units = Cl * (q.k + sqrt(Dh) b); c = 0 only when one key is visible
  const float Cl = fmaxf(c * kLog2e / sqrtD, FLT_MIN);

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int x = 0; x < 16; ++x) oacc[db][x] = 0.f;
  float m = kNegInf, l = 0.f;

  const int kend = CAUSAL ? min(T, i0 + kMQ) : T;
  const int ntiles = (kend + kNK - 1) / kNK;
  const float* __restrict__ tabh = a.tab + (size_t)h * a.tab_stride;
  const int dlo = CAUSAL ? 0 : -(T - 1);
  const int dhi = T - 1;

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * kNK;
    __syncthreads();
    // ---- stage K (row-major, swizzled 16-byte chunks)
#pragma unroll
    for (int cidx = tid; cidx < kNK * KCH; cidx += 256) {
      const int r = cidx / KCH;
      const int ch = cidx - r * KCH;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (j0 + r < T) val = *(const u32x4*)(K + (size_t)(j0 + r) * DH + ch * 8);
      *(u32x4*)(Ks + r * DH + (ch ^ swz(r, KCH - 1)) * 8) = val;
    }
    // ---- stage V transposed: Vt[dh][key], two keys per dword
#pragma unroll
    for (int pidx = tid; pidx < (kNK / 2) * KCH; pidx += 256) {
      const int p = pidx % (kNK / 2);
      const int ch = pidx / (kNK / 2);
      const int r0 = 2 * p;
      u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
      if (j0 + r0 < T) v0 = *(const u32x4*)(V + (size_t)(j0 + r0) * DH + ch * 8);
      if (j0 + r0 + 1 < T) v1 = *(const u32x4*)(V + (size_t)(j0 + r0 + 1) * DH + ch * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w0 = v0[e >> 1], w1 = v1[e >> 1];
        // even e: low halves of w0 / w1; odd e: high halves
        const uint32_t packed = (e & 1) ? __builtin_amdgcn_perm(w1, w0, 0x07060302u)
                                        : __builtin_amdgcn_perm(w1, w0, 0x05040100u);
        *(uint32_t*)(Vt + (ch * 8 + e) * VTS + r0) = packed;
      }
    }
    // ---- stage the distance window: tw[x] = sqrt(Dh) * b(d_min + x)
    const int d_min = i0 - j0 - (kNK - 1);
    for (int x = tid; x < kTW; x += 256) {
      const int d = d_min + x;
      float val = kNegInf;
      if (d >= dlo && d <= dhi) val = sqrtD * tabh[d - a.tab_d0];
      tw[x] = val;
    }
    __syncthreads();

    // ---- S'^T = K Q^T + sqrt(Dh) b   (two 32-key blocks)
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int kl = 32 * kb + 8 * (x >> 2) + 4 * hh + (x & 3);
        sacc[kb][x] = tw[32 * wave + ql + (kNK - 1) - kl];
      }
      const int r = 32 * kb + ql;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch = 2 * ks + hh;
        const u32x4 kw = *(const u32x4*)(Ks + r * DH + (ch ^ swz(r, KCH - 1)) * 8);
        sacc[kb] = mfma32x32x16(as_bf16x8(kw), qf[ks], sacc[kb]);
      }
    }
    if (!CAUSAL && j0 + kNK > T) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int kl = 32 * kb + 8 * (x >> 2) + 4 * hh + (x & 3);
          if (j0 + kl >= T) sacc[kb][x] = kNegInf;
        }
    }

    // ---- online softmax (exp2 domain)
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int x = 0; x < 16; ++x) mx = fmaxf(mx, sacc[kb][x]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m, Cl * mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float sc = exp2_fast(m - m_use);
    m = m_new;
    l *= sc;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int x = 0; x < 16; ++x) oacc[db][x] *= sc;

    u32x4 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int x = 0; x < 16; x += 2) {
        const float p0 = exp2_fast(Cl * sacc[kb][x] - m_use);
        const float p1 = exp2_fast(Cl * sacc[kb][x + 1] - m_use);
        l += p0 + p1;
        pf[2 * kb + (x >> 3)][(x & 7) >> 1] = pack_bf16x2(p0, p1);
      }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int row = 32 * db + ql;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int col = 16 * st + 4 * hh;   // = 32 kb + 16 s' + 4 hh
        const u32x2 lo = *(const u32x2*)(Vt + row * VTS + col);
        const u32x2 hi = *(const u32x2*)(Vt + row * VTS + col + 8);
        const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
        oacc[db] = mfma32x32x16(as_bf16x8(av), as_bf16x8(pf[st]), oacc[db]);
      }
    }
  }

  // ---- epilogue
  const float lt = l + xor32(l);
  if (i < T) {
    const float inv = 1.0f / lt;
    const size_t orow = base + (size_t)i * DH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dh0 = 32 * db + 8 * g + 4 * hh;
        const float o0 = oacc[db][4 * g + 0] * inv, o1 = oacc[db][4 * g + 1] * inv;
        const float o2 = oacc[db][4 * g + 2] * inv, o3 = oacc[db][4 * g + 3] * inv;
        if (a.o_f32) {
          f32x4 w = {o0, o1, o2, o3};
          *(f32x4*)((float*)a.o + orow + dh0) = w;
        } else {
          u32x2 w = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
          *(u32x2*)((uint16_t*)a.o + orow + dh0) = w;
        }
      }
    if (hh == 0) a.lse[(size_t)bh * T + i] = (m + __log2f(lt)) * kLn2;
  }
}

// ------------------------------------------------------------------------------------
// fp32 path: one query row per lane, keys and values broadcast from LDS, fp32 FMA.
// ------------------------------------------------------------------------------------
constexpr int kMQ32 = 64;
constexpr int kNK32 = 64;

template <int DH, bool CAUSAL>
__global__ void __launch_bounds__(64) fwd_f32_kernel(FwdArgs a, int nqb) {
  __shared__ __attribute__((aligned(16))) float Ks[kNK32 * DH];
  __shared__ __attribute__((aligned(16))) float Vs[kNK32 * DH];
  __shared__ float tw[kMQ32 + kNK32];

  const int BH = a.B * a.H;
  int qb = blockIdx.x / BH;
  const int bh = blockIdx.x - qb * BH;
  if (CAUSAL) qb = nqb - 1 - qb;
  const int h = bh % a.H;
  const int T = a.T;
  const size_t base = (size_t)bh * T * DH;
  const float* __restrict__ Q = (const float*)a.q + base;
  const float* __restrict__ K = (const float*)a.k + base;
  const float* __restrict__ V = (const float*)a.v + base;
  const int lane = threadIdx.x;
  const int i0 = qb * kMQ32;
  const int i = i0 + lane;

  float qr[DH];
#pragma unroll
  for (int e = 0; e < DH; e += 4) {
    f32x4 w = {0.f, 0.f, 0.f, 0.f};
    if (i < T) w = *(const f32x4*)(Q + (size_t)i * DH + e);
    qr[e] = w[0]; qr[e + 1] = w[1]; qr[e + 2] = w[2]; qr[e + 3] = w[3];
  }
  const int n_i = CAUSAL ? i + 1 : T;
  const float c = ssmax_c(a.ssmax, a.ssmax ? a.s[h] : 1.0f, n_i);
  const float Cs = fmaxf(c * kLog2e / __builtin_sqrtf((float)DH), FLT_MIN);
  const float Cb = fmaxf(c * kLog2e, FLT_MIN);

  float o[DH];
#pragma unroll
  for (int e = 0; e < DH; ++e) o[e] = 0.f;
  float m = kNegInf, l = 0.f;
  const int kend = CAUSAL ? min(T, i0 + kMQ32) : T;
  const float* __restrict__ tabh = a.tab + (size_t)h * a.tab_stride;
  const int dlo = CAUSAL ? 0 : -(T - 1);
  const int dhi = T - 1;

  for (int j0 = 0; j0 < kend; j0 += kNK32) {
    __syncthreads();
    for (int x = lane; x < kNK32 * DH / 4; x += 64) {
      const int r = (4 * x) / DH;
      f32x4 kw = {0.f, 0.f, 0.f, 0.f}, vw = {0.f, 0.f, 0.f, 0.f};
      if (j0 + r < T) {
        kw = *(const f32x4*)(K + (size_t)j0 * DH + 4 * x);
        vw = *(const f32x4*)(V + (size_t)j0 * DH + 4 * x);
      }
      *(f32x4*)(Ks + 4 * x) = kw;
      *(f32x4*)(Vs + 4 * x) = vw;
    }
    const int d_min = i0 - j0 - (kNK32 - 1);
    for (int x = lane; x < kMQ32 + kNK32; x += 64) {
      const int d = d_min + x;
      tw[x] = (d >= dlo && d <= dhi) ? tabh[d - a.tab_d0] : kNegInf;
    }
    __syncthreads();
    const int nk = min(kNK32, kend - j0);
    float sc[kNK32];
    float mx = kNegInf;
#pragma unroll 4
    for (int jj = 0; jj < kNK32; ++jj) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < DH; ++e) dot = fmaf(qr[e], Ks[jj * DH + e], dot);
      const float bv = tw[lane + (kNK32 - 1) - jj];
      float t = fmaf(Cs, dot, Cb * bv);
      if (jj >= nk || bv == kNegInf) t = kNegInf;
      sc[jj] = t;
      mx = fmaxf(mx, t);
    }
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float s0 = exp2_fast(m - m_use);
    m = m_new;
    l *= s0;
#pragma unroll
    for (int e = 0; e < DH; ++e) o[e] *= s0;
#pragma unroll 2
    for (int jj = 0; jj < kNK32; ++jj) {
      const float p = exp2_fast(sc[jj] - m_use);
      l += p;
#pragma unroll
      for (int e = 0; e < DH; ++e) o[e] = fmaf(p, Vs[jj * DH + e], o[e]);
    }
  }
  if (i < T) {
    const float inv = 1.0f / l;
    const size_t orow = base + (size_t)i * DH;
#pragma unroll
    for (int e = 0; e < DH; e += 4) {
      const float o0 = o[e] * inv, o1 = o[e + 1] * inv, o2 = o[e + 2] * inv, o3 = o[e + 3] * inv;
      if (a.o_f32) {
        f32x4 w = {o0, o1, o2, o3};
        *(f32x4*)((float*)a.o + orow + e) = w;
      } else {
        u32x2 w = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
        *(u32x2*)((uint16_t*)a.o + orow + e) = w;
      }
    }
    a.lse[(size_t)bh * T + i] = (m + __log2f(l)) * kLn2;
  }
}

template <int DH, bool CAUSAL>
hipError_t launch_bf16_t(const FwdArgs& a, hipStream_t stream) {
  const int nqb = (a.T + kMQ - 1) / kMQ;
  const long nblocks = (long)nqb * a.B * a.H;
  hipLaunchKernelGGL((fwd_bf16_kernel<DH, CAUSAL>), dim3((unsigned)nblocks), dim3(256), 0, stream, a, nqb);
  return hipGetLastError();
}

template <int DH, bool CAUSAL>
hipError_t launch_f32_t(const FwdArgs& a, hipStream_t stream) {
  const int nqb = (a.T + kMQ32 - 1) / kMQ32;
  const long nblocks = (long)nqb * a.B * a.H;
  hipLaunchKernelGGL((fwd_f32_kernel<DH, CAUSAL>), dim3((unsigned)nblocks), dim3(64), 0, stream, a, nqb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int Dh, hipStream_t stream) {
  switch (Dh) {
    case 32: return a.causal ? launch_bf16_t<32, true>(a, stream) : launch_bf16_t<32, false>(a, stream);
    case 64: return a.causal ? launch_bf16_t<64, true>(a, stream) : launch_bf16_t<64, false>(a, stream);
    case 128: return a.causal ? launch_bf16_t<128, true>(a, stream) : launch_bf16_t<128, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_f32(const FwdArgs& a, int Dh, hipStream_t stream) {
  switch (Dh) {
    case 32: return a.causal ? launch_f32_t<32, true>(a, stream) : launch_f32_t<32, false>(a, stream);
    case 64: return a.causal ? launch_f32_t<64, true>(a, stream) : launch_f32_t<64, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bam
