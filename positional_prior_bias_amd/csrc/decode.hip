// BAM attention decode: one query row per (b, h) against a long KV cache, split-KV.
//
// The query of sequence b sits at position i = kv_len[b] - 1 and sees n = kv_len[b]
// keys; logit_j = c (q.k_j / sqrt(Dh) + b_h(i - j)), c = s_h ln(n) with SSMax
// ("Résumé Technique : Mécanisme d'Attention Bayésienne (BAM)", "Solution Proposée :
// GGD-BAM"; retrieval far beyond the training context, "Bayesian Attention
// Mechanism", "Highlights").
//
// HBM-bound streaming design:
//   * grid = (nsplit, H, B); a work-group of 4 waves owns one contiguous key range of
//     one (b, h) and each wave takes every fourth tile of it;
//   * a tile is 8 fully coalesced 1 KiB loads of K and of V per wave (16-byte loads,
//     lane l reads bytes 16 l .. 16 l + 15 of each KiB); Dh / 8 lanes share a key (4, 8 or
//     16 for Dh = 32, 64, 128), each holding 8 of its head-dimension entries;
//   * q.k is a per-lane 8-term dot plus a butterfly over the lanes of a key; the
//     online softmax keeps (m, l, o) per lane with a wave-uniform running max;
//   * the partial (m, l, o) of each range goes to the workspace and a second kernel
//     merges the ranges exactly by their log-sum-exp.
// The bias of distance d comes from the per-head table (one float per key, read
// through L2, shared by every sequence of the batch).
// Paged caches (PAGED): K and V live in pages [num_pages, H, page_size, Dh] and
// block_table[b][p] names the page that holds keys p * page_size .. of sequence b.
// page_size is a multiple of 64, so a wave tile never straddles two pages and costs one
// scalar table read; page ids are clamped to [0, num_pages) so a bad table cannot read
// outside the pages.
// Prior-aware skipping (SKIP, contiguous caches): a bound kernel first takes, per (b, h),
// the largest logit of the last 256 keys (minus a rounding margin) as a lower bound M- of
// the row's largest logit.  Each range then bounds its own logits from above, key by key,
// by c (b(d) + |q| |k|_page / sqrt(Dh)) with the caller's per-page maxima of |k|, and a
// range whose bound sits more than 160 (log2 units) below M- writes the partial of a range
// with no visible key (m = -inf, l = 0, o = 0) without reading its K and V.  In the full
// computation that range's merge weight 2^(m_s - M) is below 2^-160, i.e. exactly 0 in
// float32, so both give the same bits.
#include <float.h>

#include "bam_device.h"
#include "bam_internal.h"

namespace bam {

namespace {

constexpr int kWaves = 4;
constexpr int kRows = 8;  // 1 KiB loads per tile per tensor

template <int DH>
struct DecodeShape {
  static constexpr int LPK = DH / 8;        // lanes per key
  static constexpr int KPI = 64 / LPK;      // keys per 1 KiB load
  static constexpr int KT = kRows * KPI;    // keys per wave tile
};

__device__ __forceinline__ float dot8(const float* q, const u32x4& w) {
  float acc = q[0] * bf16_lo(w[0]);
  acc = fmaf(q[1], bf16_hi(w[0]), acc);
  acc = fmaf(q[2], bf16_lo(w[1]), acc);
  acc = fmaf(q[3], bf16_hi(w[1]), acc);
  acc = fmaf(q[4], bf16_lo(w[2]), acc);
  acc = fmaf(q[5], bf16_hi(w[2]), acc);
  acc = fmaf(q[6], bf16_lo(w[3]), acc);
  acc = fmaf(q[7], bf16_hi(w[3]), acc);
  return acc;
}

template <int DH, bool PAGED, bool SKIP>
__global__ void __launch_bounds__(256) decode_split_kernel(DecodeArgs a) {
  using S = DecodeShape<DH>;
  constexpr int LPK = S::LPK, KPI = S::KPI, KT = S::KT;
  static_assert(!(PAGED && SKIP), "skipping is for contiguous caches");
  __shared__ float red[kWaves][DH + 2];

  const int sidx = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int bh = b * a.H + h;
  int L = a.kv_len[b];
  L = L < 1 ? 1 : (L > a.Lmax ? a.Lmax : L);   // keep reads in bounds whatever the input
  const int iq = L - 1;
  const int kbeg = sidx * a.chunk;
  const int kend = min(kbeg + a.chunk, L);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int slot = lane / LPK;      // key slot inside a 1 KiB load
  const int cl = lane % LPK;        // which 8 head-dim entries this lane holds

  const float qscale = kLog2e / __builtin_sqrtf((float)DH);
  float qv[8];
  {
    const u32x4 w = *(const u32x4*)((const uint16_t*)a.q + (size_t)bh * DH + cl * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[2 * e] = bf16_lo(w[e]) * qscale;
      qv[2 * e + 1] = bf16_hi(w[e]) * qscale;
    }
  }
  const float c = ssmax_c(a.ssmax, a.ssmax ? a.s[h] : 1.0f, L);
  const float C = fmaxf(c, FLT_MIN);
  const float* __restrict__ tabh = a.tab + (size_t)h * a.tab_stride;
  const size_t kvbase = PAGED ? 0 : (size_t)bh * a.Lmax * DH;
  const uint16_t* __restrict__ Kc = (const uint16_t*)a.k + kvbase;
  const uint16_t* __restrict__ Vc = (const uint16_t*)a.v + kvbase;

  float m = kNegInf, l = 0.f;
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;

  if constexpr (SKIP) {
    // upper bound of this range's logits: c (b(i - j) + |q| |k|_page(j) / sqrt(Dh)), in
    // log2 units, over its keys; every thread takes every 256th key
    const float qn = a.bound[2 * bh + 1];
    const float* __restrict__ nrm = a.key_norms + (size_t)bh * a.npages;
    float ub = kNegInf;
    for (int key = kbeg + tid; key < kend; key += 256)
      ub = fmaxf(ub, fmaf(tabh[iq - key], kLog2e, qn * nrm[key / kNormPage]));
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) ub = fmaxf(ub, __shfl_xor(ub, off, 64));
    if (lane == 0) red[wave][0] = ub;
    __syncthreads();
    ub = fmaxf(fmaxf(red[0][0], red[1][0]), fmaxf(red[2][0], red[3][0]));
    ub = C * ub;
    if (ub != kNegInf) ub += fabsf(ub) * 0x1p-10f + 1.0f;   // covers the rounding of the logits
    const bool skip = ub < a.bound[2 * bh] - 160.0f;
    __syncthreads();                                   // red is reused below
    if (skip) {
      float* part = a.part + ((size_t)bh * a.nsplit + sidx) * (DH + 2);
      if (tid < DH) part[2 + tid] = 0.f;
      if (tid == 0) {
        part[0] = kNegInf;
        part[1] = 0.f;
      }
      return;
    }
  }

  for (int tb = kbeg + wave * KT; tb < kend; tb += kWaves * KT) {
    // rows of this tile: Kt / Vt + (tile-relative key) * DH
    const uint16_t* __restrict__ Kt = Kc + (size_t)tb * DH;
    const uint16_t* __restrict__ Vt = Vc + (size_t)tb * DH;
    if (PAGED) {
      const int lp = tb / a.page_size;
      int pg = a.block_table[(size_t)b * a.max_blocks + lp];
      pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
      const size_t pbase = (((size_t)pg * a.H + h) * a.page_size + (tb - lp * a.page_size)) * DH;
      Kt = (const uint16_t*)a.k + pbase;
      Vt = (const uint16_t*)a.v + pbase;
    }
    u32x4 kw[kRows], vw[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int kr = r * KPI + slot;
      const u32x4 z = {0u, 0u, 0u, 0u};
      kw[r] = z;
      vw[r] = z;
      if (tb + kr < kend) {
        kw[r] = __builtin_nontemporal_load((const u32x4*)(Kt + (size_t)kr * DH + cl * 8));
        vw[r] = __builtin_nontemporal_load((const u32x4*)(Vt + (size_t)kr * DH + cl * 8));
      }
    }
    float lg[kRows];
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      float d = dot8(qv, kw[r]);
#pragma unroll
      for (int off = 1; off < LPK; off <<= 1) d += __shfl_xor(d, off, 64);
      const int key = tb + r * KPI + slot;
      float t = kNegInf;
      if (key < kend) t = C * fmaf(tabh[iq - key], kLog2e, d);
      lg[r] = t;
      mx = fmaxf(mx, t);
    }
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float sc = exp2_fast(m - m_use);
    m = m_new;
    l *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= sc;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const float p = exp2_fast(lg[r] - m_use);
      l += p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = fmaf(p, bf16_lo(vw[r][e]), o[2 * e]);
        o[2 * e + 1] = fmaf(p, bf16_hi(vw[r][e]), o[2 * e + 1]);
      }
    }
  }
  // sum over the key slots of the wave (same running max everywhere in the wave)
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    l += __shfl_xor(l, off, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += __shfl_xor(o[e], off, 64);
  }
  if (lane < LPK) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][cl * 8 + e] = o[e];
    if (lane == 0) {
      red[wave][DH] = m;
      red[wave][DH + 1] = l;
    }
  }
  __syncthreads();
  if (tid < DH) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red[w][DH]);
    float Ls = 0.f, Os = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = red[w][DH];
      const float wt = (mw == kNegInf) ? 0.f : exp2_fast(mw - M);
      Ls += wt * red[w][DH + 1];
      Os += wt * red[w][tid];
    }
    float* part = a.part + ((size_t)bh * a.nsplit + sidx) * (DH + 2);
    part[2 + tid] = Os;
    if (tid == 0) {
      part[0] = M;
      part[1] = Ls;
    }
  }
}

// Per (b, h): M- = the largest logit of the last min(n, 256) keys, computed as the split
// kernel computes logits (the same scaled query, the same table entry, a different
// summation order) and lowered by a margin that covers the difference, so M- never exceeds
// the largest logit the split kernel finds; and |q| log2(e) / sqrt(Dh), rounded up.
template <int DH>
__global__ void __launch_bounds__(256) decode_bound_kernel(DecodeArgs a) {
  __shared__ float smax[4];
  __shared__ float sq;
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh - b * a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int L = a.kv_len[b];
  L = L < 1 ? 1 : (L > a.Lmax ? a.Lmax : L);
  const int iq = L - 1;
  const float qscale = kLog2e / __builtin_sqrtf((float)DH);
  const uint16_t* __restrict__ qp = (const uint16_t*)a.q + (size_t)bh * DH;
  if (tid == 0) {
    float ss = 0.f;
    for (int e = 0; e < DH; e += 2) {
      const uint32_t w = *(const uint32_t*)(qp + e);
      const float x0 = bf16_lo(w) * qscale, x1 = bf16_hi(w) * qscale;
      ss = fmaf(x0, x0, fmaf(x1, x1, ss));
    }
    // the sum of DH squares rounds by at most DH 2^-24 of itself, the root by half that
    sq = __builtin_sqrtf(ss) * (1.0f + 0x1p-14f);
  }
  const float c = ssmax_c(a.ssmax, a.ssmax ? a.s[h] : 1.0f, L);
  const float C = fmaxf(c, FLT_MIN);
  const float* __restrict__ tabh = a.tab + (size_t)h * a.tab_stride;
  float t = kNegInf;
  const int key = iq - tid;
  if (key >= 0) {
    const uint16_t* __restrict__ kp = (const uint16_t*)a.k + ((size_t)bh * a.Lmax + key) * DH;
    float d = 0.f;
    for (int e = 0; e < DH; e += 8) {
      const u32x4 w = *(const u32x4*)(kp + e);
      const u32x4 qw = *(const u32x4*)(qp + e);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        d = fmaf(bf16_lo(qw[x]) * qscale, bf16_lo(w[x]), d);
        d = fmaf(bf16_hi(qw[x]) * qscale, bf16_hi(w[x]), d);
      }
    }
    t = C * fmaf(tabh[iq - key], kLog2e, d);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) t = fmaxf(t, __shfl_xor(t, off, 64));
  if (lane == 0) smax[wave] = t;
  __syncthreads();
  if (tid == 0) {
    float mx = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
    // two fp32 dot products of the same terms in different orders differ by at most about
    // DH 2^-23 of the sum of |terms|; the margin is far wider, and -inf stays -inf
    mx -= fabsf(mx) * 0x1p-10f + 1.0f;
    a.bound[2 * bh] = mx;
    a.bound[2 * bh + 1] = sq;
  }
}

// Per-page maxima of the key norms: norms[b][h][p] = max |k_j| over keys j of page p
// (kNormPage keys; keys at or beyond Lmax count as zero), computed in fp32 and rounded up
// so that it bounds the exact norm.  One wave per page, one lane per key.
template <int DH>
__global__ void __launch_bounds__(256) decode_key_norms_kernel(const uint16_t* __restrict__ k, int H, int Lmax,
                                                               int npages, float* __restrict__ norms) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int page = blockIdx.x * 4 + wave;
  const int bh = blockIdx.y;
  if (page >= npages) return;
  const int key = page * kNormPage + lane;
  float ss = 0.f;
  if (key < Lmax) {
    const uint16_t* __restrict__ kp = k + ((size_t)bh * Lmax + key) * DH;
    for (int e = 0; e < DH; e += 8) {
      const u32x4 w = *(const u32x4*)(kp + e);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float x0 = bf16_lo(w[x]), x1 = bf16_hi(w[x]);
        ss = fmaf(x0, x0, fmaf(x1, x1, ss));
      }
    }
  }
  float n = __builtin_sqrtf(ss) * (1.0f + 0x1p-14f);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) n = fmaxf(n, __shfl_xor(n, off, 64));
  if (lane == 0) norms[(size_t)bh * npages + page] = n;
}

// Merge the per-range partials of one (b, h): M = max m_s, L = sum 2^(m_s - M) l_s,
// O = sum 2^(m_s - M) o_s / L.  Four waves take every fourth range (independent loads,
// unrolled), then combine through LDS.
template <int DH>
__global__ void __launch_bounds__(256) decode_combine_kernel(DecodeArgs a) {
  constexpr int EPL = (DH + 63) / 64;   // head-dim entries per lane (at Dh = 32 lanes 32..63 idle)
  __shared__ float smax[4];
  __shared__ float sl[4];
  __shared__ float so[4][DH];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int S = a.nsplit;
  const float* part = a.part + (size_t)bh * S * (DH + 2);
  float M = kNegInf;
  for (int s = tid; s < S; s += 256) M = fmaxf(M, part[(size_t)s * (DH + 2)]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  if (lane == 0) smax[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
  float L = 0.f, O[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) O[e] = 0.f;
#pragma unroll 4
  for (int s = wave; s < S; s += 4) {
    const float* ps = part + (size_t)s * (DH + 2);
    const float ms = ps[0];
    const float wt = (ms == kNegInf) ? 0.f : exp2_fast(ms - M);
    L = fmaf(wt, ps[1], L);
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      if (lane + 64 * e < DH) O[e] = fmaf(wt, ps[2 + lane + 64 * e], O[e]);
  }
  if (lane == 0) sl[wave] = L;
#pragma unroll
  for (int e = 0; e < EPL; ++e)
    if (lane + 64 * e < DH) so[wave][lane + 64 * e] = O[e];
  __syncthreads();
  if (tid < DH) {
    const float Ls = sl[0] + sl[1] + sl[2] + sl[3];
    const float out = (so[0][tid] + so[1][tid] + so[2][tid] + so[3][tid]) / Ls;
    if (a.o_f32) {
      ((float*)a.o)[(size_t)bh * DH + tid] = out;
    } else {
      ((__bf16*)a.o)[(size_t)bh * DH + tid] = (__bf16)out;
    }
    if (tid == 0) a.lse[bh] = (M + __log2f(Ls)) * kLn2;
  }
}

template <int DH>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  if (a.block_table) {
    hipLaunchKernelGGL((decode_split_kernel<DH, true, false>), dim3(a.nsplit, a.H, a.B), dim3(256), 0, stream, a);
  } else if (a.key_norms) {
    hipLaunchKernelGGL(decode_bound_kernel<DH>, dim3(a.B * a.H), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_split_kernel<DH, false, true>), dim3(a.nsplit, a.H, a.B), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_split_kernel<DH, false, false>), dim3(a.nsplit, a.H, a.B), dim3(256), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel<DH>, dim3(a.B * a.H), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// Keys per split: a whole number of work-group tiles, about 2K keys for long caches.
// Keys per split: 2048 for long caches; shorter when that would leave fewer than about
// 512 work-groups (2 per CU), so short caches still spread over the whole chip (measured:
// 1.8x at 2k keys, 1.4x at 4k; a higher target shortens the splits of 16k caches too far).
// Always a whole number of work-group tiles.
int decode_chunk_keys(int Lmax, int Dh, int BH) {
  const int tile = kWaves * kRows * (64 / (Dh / 8));
  constexpr int kTargetGroups = 512;
  const int min_splits = (kTargetGroups + BH - 1) / BH;
  int want = (Lmax + min_splits - 1) / min_splits;
  if (want > 2048) want = 2048;
  if (want < tile) want = tile;
  return ((want + tile - 1) / tile) * tile;
}

hipError_t launch_decode_key_norms(const void* k, int B, int H, int Lmax, int Dh, float* norms,
                                   hipStream_t stream) {
  const int npages = (Lmax + kNormPage - 1) / kNormPage;
  const dim3 grid((npages + 3) / 4, B * H);
  const uint16_t* kp = (const uint16_t*)k;
  switch (Dh) {
    case 32: hipLaunchKernelGGL(decode_key_norms_kernel<32>, grid, dim3(256), 0, stream, kp, H, Lmax, npages, norms); break;
    case 64: hipLaunchKernelGGL(decode_key_norms_kernel<64>, grid, dim3(256), 0, stream, kp, H, Lmax, npages, norms); break;
    case 128: hipLaunchKernelGGL(decode_key_norms_kernel<128>, grid, dim3(256), 0, stream, kp, H, Lmax, npages, norms); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int Dh, hipStream_t stream) {
  switch (Dh) {
    case 32: return launch_t<32>(a, stream);
    case 64: return launch_t<64>(a, stream);
    case 128: return launch_t<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bam
