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
//   skip_suffix_kernel per head: C(c) = S(64 c), the suffix maximum at chunk starts, from
//                      the forward's table;
//   skip_plan_kernel   per query block: Kmax, R = min_i R_i, the largest chunk c* with
//                      C(c*) >= R (a 64-way search; C is non-increasing), and the first key
//                      tile floor((i0 - 64 c* - 63) / 64).
// For rows i >= i0 and keys j < i0 - 64 c* - 63, i - j >= 64 (c* + 1), so
// b(i - j) <= C(c* + 1) < R <= R_i.  (Chunk granularity can only keep more keys than the
// exact largest distance would; the plan is in whole tiles anyway.)
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

// C(c) = S(64 c) = max_{d >= 64 c} b(d) for one head: the maxima of the 64-distance chunks
// (one wave per chunk, coalesced), then their suffix maximum (each thread a run of chunks,
// then a scan over the runs).  The forward's table holds sqrt(Dh) b at entry tab_d0 - d.
__global__ void __launch_bounds__(1024) skip_suffix_kernel(SkipArgs a, int T, float rs) {
  const int h = blockIdx.x;
  const float* th = a.tab + (size_t)h * a.tab_stride + a.tab_d0;   // th[-d] = sqrt(Dh) b(d)
  const int nch = (T + 63) / 64;
  float* ch = a.smax + (size_t)h * nch;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int c = wave; c < nch; c += 16) {
    const int d = 64 * c + lane;
    const float mx = wave_max(d < T ? th[-d] : kNegInf);
    if (lane == 0) ch[c] = mx * rs;
  }
  __syncthreads();
  const int run = (nch + 1023) / 1024;
  const int c0 = min(nch, tid * run), c1 = min(nch, c0 + run);
  float mx = kNegInf;
  for (int c = c0; c < c1; ++c) mx = fmaxf(mx, ch[c]);
  __shared__ float suf[1024];
  suf[tid] = mx;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {   // inclusive suffix maximum over the runs
    const float x = tid + o < 1024 ? fmaxf(suf[tid], suf[tid + o]) : suf[tid];
    __syncthreads();
    suf[tid] = x;
    __syncthreads();
  }
  float acc = tid + 1 < 1024 ? suf[tid + 1] : kNegInf;
  for (int c = c1 - 1; c >= c0; --c) {
    acc = fmaxf(acc, ch[c]);
    ch[c] = acc;
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
  const int nch = (T + 63) / 64;
  const float* cs = a.smax + (size_t)h * nch;   // C(c) = S(64 c), non-increasing in c
  const int cmax = i0 / 64;
  if (r > kNegInf && i0 > 0 && !(cs[cmax] >= r)) {
    // c* = the largest chunk with C(c*) >= r (0 if none).  Invariant: C(lo) >= r or lo = 0;
    // C(hi) < r.  The probes that pass form a prefix of the lanes.
    int lo = 0, hi = cmax;
    while (hi - lo > 1) {
      const int step = (hi - lo + 63) / 64;
      const int p = lo + step * (lane + 1);
      const bool ok = p < hi && cs[p] >= r;
      const unsigned long long bal = __ballot(ok);
      const int last = bal ? 63 - __builtin_clzll(bal) : -1;   // last passing probe
      const int nlo = last >= 0 ? lo + step * (last + 1) : lo;
      hi = min(hi, lo + step * (last + 2));
      lo = nlo;
    }
    // every d >= 64 (c* + 1) has b(d) <= C(c* + 1) < r: keys j < i0 - 64 c* - 63 are out
    tile = max(0, i0 - 64 * lo - 63) / 64;
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
