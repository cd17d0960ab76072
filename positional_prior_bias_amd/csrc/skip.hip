// Prior-aware key-tile skipping for the causal bf16 prefill forward.
//
// With a positional prior that decays with distance ("Bayesian Attention Mechanism"
// README, "Implementation Details": local heads with beta > 0), the keys far behind a
// query get weights far below float32 resolution.  This file plans, for every work-group of
// the forward kernel (one query block of one (b, h)), the first key tile that can carry a
// weight that float32 can hold; the forward kernel starts its key loop there.
//
// The bound (logit l_ij = c_i (q_i.k_j / sqrt(Dh) + b(i - j)), c_i > 0):
//   upper: l_ij <= c_i (|q_i| Kmax / sqrt(Dh) + S(i - j)),  Kmax = max_j |k_j| of the (b, h),
//          S(d) = max_{d' >= d} b(d')  (the suffix maximum of the head's bias row);
//   lower: max_j l_ij >= l_ii = c_i (q_i.k_i / sqrt(Dh) + b(0))  (key i is always visible).
// Key j is skipped for row i when upper < lower - kSkipMargin, i.e. when
//   S(i - j) < R_i = (q_i.k_i - |q_i| Kmax) / sqrt(Dh) + b(0) - kSkipMargin / c_i.
// A skipped key's softmax weight is then below e^-kSkipMargin times the row's largest
// weight.  kSkipMargin = 104 > 150 ln 2, so that ratio is below 2^-150, under the smallest
// float32 subnormal: the skipped terms are zero at float32 precision, whatever order the
// online softmax meets them in.  The rounding of the bound's own float32 arithmetic is a
// few ulps of values of order 10^2, far inside the margin.  Rows with c_i <= 0 (SSMax at
// n = 1) and non-finite bounds never skip.
//
// Three small kernels, all reading what the forward reads anyway (Q, K once; the table):
//   skip_rows_kernel   per row: u_i = |q_i| / sqrt(Dh), v_i = R_i + u_i Kmax, and a per-block
//                      max of |k_j|;
//   skip_suffix_kernel per head: S(d) for d in [0, T - 1] from the forward's table;
//   skip_plan_kernel   per query block: Kmax, R = min_i R_i, the largest distance D* with
//                      S(D*) >= R (a 64-way search; S is non-increasing), and the first key
//                      tile floor((i0 - D*) / 64).
// For rows i >= i0 and keys j < i0 - D*, i - j > D*, so b(i - j) <= S(D* + 1) < R <= R_i.
#include <float.h>

#include "bam_device.h"
#include "bam_internal.h"

namespace bam {

namespace {

constexpr float kSkipMargin = 104.0f;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_min(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fminf(x, __shfl_xor(x, o, 64));
  return x;
}

// DH / 8 lanes per row, each reading 16 bytes of q_i and of k_i.
template <int DH>
__global__ void __launch_bounds__(256) skip_rows_kernel(SkipArgs a, int T, int H) {
  constexpr int LPR = DH / 8;
  constexpr int RPB = 256 / LPR;
  const int bh = blockIdx.y;
  const int h = bh % H;
  const int tid = threadIdx.x;
  const int i = blockIdx.x * RPB + tid / LPR;
  const int part = tid % LPR;
  float qq = 0.f, kk = 0.f, qk = 0.f;
  if (i < T) {
    const size_t off = ((size_t)bh * T + i) * DH + part * 8;
    const u32x4 qw = *(const u32x4*)((const uint16_t*)a.q + off);
    const u32x4 kw = *(const u32x4*)((const uint16_t*)a.k + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float q0 = __uint_as_float(qw[e] << 16), q1 = __uint_as_float(qw[e] & 0xffff0000u);
      const float k0 = __uint_as_float(kw[e] << 16), k1 = __uint_as_float(kw[e] & 0xffff0000u);
      qq = fmaf(q0, q0, fmaf(q1, q1, qq));
      kk = fmaf(k0, k0, fmaf(k1, k1, kk));
      qk = fmaf(q0, k0, fmaf(q1, k1, qk));
    }
  }
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) {
    qq += __shfl_xor(qq, o, 64);
    kk += __shfl_xor(kk, o, 64);
    qk += __shfl_xor(qk, o, 64);
  }
  const float rs = 1.0f / __builtin_sqrtf((float)DH);
  if (part == 0 && i < T) {
    const float c = ssmax_c(a.ssmax, a.ssmax ? a.s[h] : 1.0f, i + 1);
    const float b0 = a.tab[(size_t)h * a.tab_stride + a.tab_d0] * rs;   // the table holds sqrt(Dh) b
    float v = c > 0.f ? fmaf(qk, rs, b0) - kSkipMargin / c : kNegInf;
    if (!(v > kNegInf && v < __builtin_huge_valf())) v = kNegInf;
    a.rowu[(size_t)bh * T + i] = __builtin_sqrtf(qq) * rs;
    a.rowv[(size_t)bh * T + i] = v;
  }
  // block maximum of |k_j|
  __shared__ float wmax[4];
  const float kn = wave_max(__builtin_sqrtf(kk));
  if ((tid & 63) == 0) wmax[tid >> 6] = kn;
  __syncthreads();
  if (tid == 0)
    a.kpart[(size_t)bh * gridDim.x + blockIdx.x] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

// S(d) = max_{d' in [d, T - 1]} b(d') for one head; b(d) is the forward table's entry
// tab_d0 - d divided by sqrt(Dh).  Each thread owns a run of consecutive distances.
__global__ void __launch_bounds__(1024) skip_suffix_kernel(SkipArgs a, int T, float rs) {
  const int h = blockIdx.x;
  const float* th = a.tab + (size_t)h * a.tab_stride + a.tab_d0;   // th[-d] = sqrt(Dh) b(d)
  float* sh = a.smax + (size_t)h * T;
  const int tid = threadIdx.x;
  const int run = (T + 1023) / 1024;
  const int d0 = min(T, tid * run), d1 = min(T, d0 + run);
  float mx = kNegInf;
  for (int d = d0; d < d1; ++d) mx = fmaxf(mx, th[-d]);
  __shared__ float suf[1024];
  suf[tid] = mx;
  __syncthreads();
  // inclusive suffix maximum over the 1024 runs
  for (int o = 1; o < 1024; o <<= 1) {
    const float x = tid + o < 1024 ? fmaxf(suf[tid], suf[tid + o]) : suf[tid];
    __syncthreads();
    suf[tid] = x;
    __syncthreads();
  }
  float acc = tid + 1 < 1024 ? suf[tid + 1] : kNegInf;
  for (int d = d1 - 1; d >= d0; --d) {
    acc = fmaxf(acc, th[-d]);
    sh[d] = acc * rs;
  }
}

// One wave per query block of the forward kernel (block index qb * B * H + b * H + h).
__global__ void __launch_bounds__(64) skip_plan_kernel(SkipArgs a, int T, int H, int BH, int MQ, int nparts) {
  const int bid = blockIdx.x;
  const int qb = bid / BH;
  const int bh = bid - qb * BH;
  const int h = bh % H;
  const int lane = threadIdx.x;
  float km = 0.f;
  for (int p = lane; p < nparts; p += 64) km = fmaxf(km, a.kpart[(size_t)bh * nparts + p]);
  km = wave_max(km);
  const int i0 = qb * MQ;
  const int i1 = min(T, i0 + MQ);
  float r = __builtin_huge_valf();
  for (int i = i0 + lane; i < i1; i += 64) {
    float ri = a.rowv[(size_t)bh * T + i] - a.rowu[(size_t)bh * T + i] * km;
    if (!(ri > kNegInf)) ri = kNegInf;
    r = fminf(r, ri);
  }
  r = wave_min(r);
  int tile = 0;
  const float* sh = a.smax + (size_t)h * T;
  if (r > kNegInf && i0 > 0 && !(sh[i0] >= r)) {
    // invariant: S(lo) >= r or lo = 0; S(hi) < r.  S is non-increasing, so the probes that
    // pass form a prefix of the lanes.
    int lo = 0, hi = i0;
    while (hi - lo > 1) {
      const int step = (hi - lo + 63) / 64;
      const int p = lo + step * (lane + 1);
      const bool ok = p < hi && sh[p] >= r;
      const unsigned long long bal = __ballot(ok);
      const int last = bal ? 63 - __builtin_clzll(bal) : -1;   // last passing probe
      const int nlo = last >= 0 ? lo + step * (last + 1) : lo;
      hi = min(hi, lo + step * (last + 2));
      lo = nlo;
    }
    tile = (i0 - lo) / 64;
  }
  if (lane == 0) a.first_tile[bid] = tile;
}

}  // namespace

int skip_rows_per_block(int Dh) { return 256 / (Dh / 8); }

hipError_t launch_fwd_skip_plan(const SkipArgs& a, int B, int H, int T, int Dh, int MQ, hipStream_t stream) {
  const int rpb = skip_rows_per_block(Dh);
  const int nparts = (T + rpb - 1) / rpb;
  const dim3 grid_rows((unsigned)nparts, (unsigned)(B * H));
  switch (Dh) {
    case 32: hipLaunchKernelGGL(skip_rows_kernel<32>, grid_rows, dim3(256), 0, stream, a, T, H); break;
    case 64: hipLaunchKernelGGL(skip_rows_kernel<64>, grid_rows, dim3(256), 0, stream, a, T, H); break;
    case 128: hipLaunchKernelGGL(skip_rows_kernel<128>, grid_rows, dim3(256), 0, stream, a, T, H); break;
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(skip_suffix_kernel, dim3((unsigned)H), dim3(1024), 0, stream, a, T,
                     1.0f / std::sqrt((float)Dh));
  const int nqb = (T + MQ - 1) / MQ;
  hipLaunchKernelGGL(skip_plan_kernel, dim3((unsigned)(nqb * B * H)), dim3(64), 0, stream, a, T, H, B * H, MQ,
                     nparts);
  return hipGetLastError();
}

}  // namespace bam
