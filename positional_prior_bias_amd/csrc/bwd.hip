// BAM attention backward for gfx950.
//
// Gradients of L = sum(O * dO) through logit_ij = c_i (S_ij + b_h(i - j)),
// S = q.k / sqrt(Dh), c_i = s_h ln(n_i) with SSMax:
//   dP = dO V^T, D_i = sum_e dO_ie O_ie, dZ = P * (dP - D),
//   dV = P^T dO, dQ_i = c_i / sqrt(Dh) sum_j dZ_ij k_j, dK_j = sum_i c_i / sqrt(Dh) dZ_ij q_i,
//   dalpha = sum c dZ db/dalpha, dbeta = sum c dZ db/dbeta, ds = sum dZ ln(n) (S + b).
// alpha's scale and beta are the trained per-head scalars ("Bayesian Attention
// Mechanism", "Implementation Details"); the parameter gradients are reduced in fp32.
//
// Kernels (all bf16 MFMA 32x32x16, fp32 accumulate, P recomputed from lse):
//   bwd_pre    D_i = rowsum(dO * O)
//   bwd_dkdv   a work-group owns 128 keys (32 per wave) and walks the query tiles;
//              S = Q K^T with queries as MFMA rows and keys as columns puts one key per
//              lane, so P^T and dZ^T feed dV += P^T dO and dK += dZ^T Q straight from
//              the accumulators; Q and dO are staged both row-major and transposed.
//   bwd_dq     a work-group owns 128 queries (32 per wave), shaped like the forward
//              (one query per lane), walks the key tiles: dQ^T += K^T dZ^T, and the
//              per-element parameter terms are accumulated here, one partial per
//              work-group (no atomics: the reduction order is fixed).
//   bwd_params sums the partials of each head (alpha, beta, s and, when wanted, mu).
// The bias is again the accumulator's initial value (sqrt(Dh) b from the distance
// window in LDS, -inf where the causal mask forbids the pair).
#include <float.h>

#include "bam_device.h"
#include "bam_internal.h"

namespace bam {

namespace {

constexpr int kQT = 64;      // queries per tile (dkdv)
constexpr int kKB = 128;     // keys per work-group (dkdv)
constexpr int kMQ = 128;     // queries per work-group (dq)
constexpr int kNK = 64;      // keys per tile (dq)
constexpr int kTS = 64 + 4;  // transposed-tile row stride (bf16)

// ------------------------------------------------------------------------------------
template <int DH>
__global__ void __launch_bounds__(256) bwd_pre_kernel(BwdArgs a, long nrows) {
  constexpr int LPR = DH / 8;  // lanes per row, 8 elements each
  const long gt = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gt / LPR;
  const int cl = (int)(gt % LPR);
  float acc = 0.f;
  if (row < nrows) {
    const size_t off = (size_t)row * DH + cl * 8;
    const u32x4 dw = *(const u32x4*)((const uint16_t*)a.dout + off);
    float ov[8];
    if (a.o_f32) {
      const f32x4 o0 = *(const f32x4*)((const float*)a.o + off);
      const f32x4 o1 = *(const f32x4*)((const float*)a.o + off + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { ov[e] = o0[e]; ov[4 + e] = o1[e]; }
    } else {
      const u32x4 ow = *(const u32x4*)((const uint16_t*)a.o + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) { ov[2 * e] = bf16_lo(ow[e]); ov[2 * e + 1] = bf16_hi(ow[e]); }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(bf16_lo(dw[e]), ov[2 * e], acc);
      acc = fmaf(bf16_hi(dw[e]), ov[2 * e + 1], acc);
    }
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
  if (row < nrows && cl == 0) a.Dbuf[row] = acc;
}

// ------------------------------------------------------------------------------------
template <int DH, bool CAUSAL>
__global__ void __launch_bounds__(256, 2) bwd_dkdv_kernel(BwdArgs a, int nkb) {
  constexpr int KS = DH / 16;
  constexpr int DB = DH / 32;
  constexpr int TW = kQT + kKB;   // distance window
  __shared__ __attribute__((aligned(16))) uint16_t Qs[kQT * DH];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[DH * kTS];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[kQT * DH];
  __shared__ __attribute__((aligned(16))) uint16_t dOt[DH * kTS];
  __shared__ float tw[TW];
  __shared__ __attribute__((aligned(16))) float sCl[kQT];
  __shared__ __attribute__((aligned(16))) float sL2[kQT];
  __shared__ __attribute__((aligned(16))) float sD[kQT];
  __shared__ __attribute__((aligned(16))) float sCq[kQT];

  const int BH = a.B * a.H;
  const int kb = blockIdx.x / BH;
  const int bh = blockIdx.x - kb * BH;
  const int h = bh % a.H;
  const int T = a.T;
  const size_t base = (size_t)bh * T * DH;
  const uint16_t* __restrict__ Q = (const uint16_t*)a.q + base;
  const uint16_t* __restrict__ K = (const uint16_t*)a.k + base;
  const uint16_t* __restrict__ V = (const uint16_t*)a.v + base;
  const uint16_t* __restrict__ dO = (const uint16_t*)a.dout + base;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ql = lane & 31;
  const int hh = lane >> 5;
  const int j0 = kb * kKB;
  const int jw = j0 + 32 * wave;
  const int j = jw + ql;   // this lane's key

  // K^T and V^T operands (contraction over the head dimension): lane holds key j.
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
    if (j < T) {
      kw = *(const u32x4*)(K + (size_t)j * DH + 16 * ks + 8 * hh);
      vw = *(const u32x4*)(V + (size_t)j * DH + 16 * ks + 8 * hh);
    }
    kf[ks] = as_bf16x8(kw);
    vf[ks] = as_bf16x8(vw);
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int x = 0; x < 16; ++x) { dk[db][x] = 0.f; dv[db][x] = 0.f; }

  const float sqrtD = __builtin_sqrtf((float)DH);
  const float inv_sqrtD = 1.0f / sqrtD;
  const float* __restrict__ tabh = a.tab + (size_t)h * a.tab_stride;
  const int dlo = CAUSAL ? 0 : -(T - 1);
  const int dhi = T - 1;
  const float sh = a.ssmax ? a.s[h] : 1.0f;
  const int qstart = CAUSAL ? j0 : 0;

  for (int i0 = qstart; i0 < T; i0 += kQT) {
    __syncthreads();
    stage_rows<DH, kQT, 256>(Q, i0, T, Qs, tid);
    stage_rows<DH, kQT, 256>(dO, i0, T, dOs, tid);
    stage_rows_T<DH, kQT, 256, kTS>(Q, i0, T, Qt, tid);
    stage_rows_T<DH, kQT, 256, kTS>(dO, i0, T, dOt, tid);
    const int d_min = i0 - j0 - (kKB - 1);
    for (int x = tid; x < TW; x += 256) {
      const int d = d_min + x;
      tw[x] = (d >= dlo && d <= dhi) ? sqrtD * tabh[d - a.tab_d0] : kNegInf;
    }
    if (tid < kQT) {
      const int i = i0 + tid;
      if (i < T) {
        const int n = CAUSAL ? i + 1 : T;
        const float c = ssmax_c(a.ssmax, sh, n);
        sCl[tid] = fmaxf(c * kLog2e * inv_sqrtD, FLT_MIN);
        sL2[tid] = a.lse[(size_t)bh * T + i] * kLog2e;
        sD[tid] = a.Dbuf[(size_t)bh * T + i];
        sCq[tid] = c * inv_sqrtD;
      } else {
        sCl[tid] = FLT_MIN;
        sL2[tid] = __builtin_huge_valf();
        sD[tid] = 0.f;
        sCq[tid] = 0.f;
      }
    }
    __syncthreads();
    if (CAUSAL && i0 + kQT - 1 < jw) continue;  // every query of the tile precedes this wave's keys

#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // S' = Q K^T + sqrt(Dh) b (queries as rows), dP = dO V^T
      f32x16 s, dp;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int qrow = 32 * qb + 8 * (x >> 2) + 4 * hh + (x & 3);
        s[x] = tw[qrow - 32 * wave - ql + (kKB - 1)];
        dp[x] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 qw = read_chunk<DH>(Qs, 32 * qb + ql, 2 * ks + hh);
        const u32x4 ow = read_chunk<DH>(dOs, 32 * qb + ql, 2 * ks + hh);
        s = mfma32x32x16(as_bf16x8(qw), kf[ks], s);
        dp = mfma32x32x16(as_bf16x8(ow), vf[ks], dp);
      }
      if (!CAUSAL && j >= T) {
#pragma unroll
        for (int x = 0; x < 16; ++x) s[x] = kNegInf;
      }
      u32x4 pf[2], zf[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int q4 = 32 * qb + 8 * g + 4 * hh;
        const f32x4 cl4 = *(const f32x4*)(sCl + q4);
        const f32x4 l24 = *(const f32x4*)(sL2 + q4);
        const f32x4 d4 = *(const f32x4*)(sD + q4);
        const f32x4 cq4 = *(const f32x4*)(sCq + q4);
        float pv[4], zv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int x = 4 * g + r;
          const float p = exp2_fast(cl4[r] * s[x] - l24[r]);
          pv[r] = p;
          zv[r] = p * (dp[x] - d4[r]) * cq4[r];
        }
        // register x = 8 s' + t, t = 4 (g & 1) + r  ->  operand st = s', dwords (t >> 1)
        pf[g >> 1][2 * (g & 1) + 0] = pack_bf16x2(pv[0], pv[1]);
        pf[g >> 1][2 * (g & 1) + 1] = pack_bf16x2(pv[2], pv[3]);
        zf[g >> 1][2 * (g & 1) + 0] = pack_bf16x2(zv[0], zv[1]);
        zf[g >> 1][2 * (g & 1) + 1] = pack_bf16x2(zv[2], zv[3]);
      }
      // dV += P^T dO, dK += (c dZ / sqrt(Dh))^T Q   (contraction over this block's queries)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = 32 * db + ql;
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          const int col = 32 * qb + 16 * sp + 4 * hh;
          dv[db] = mfma32x32x16(as_bf16x8(pf[sp]), read_T_operand<kTS>(dOt, row, col), dv[db]);
          dk[db] = mfma32x32x16(as_bf16x8(zf[sp]), read_T_operand<kTS>(Qt, row, col), dk[db]);
        }
      }
    }
  }

  // write dK, dV: lane holds head-dim column 32 db + ql of keys jw + 8 (x>>2) + 4 hh + (x&3)
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int key = jw + 8 * (x >> 2) + 4 * hh + (x & 3);
      if (key < T) {
        const size_t off = base + (size_t)key * DH + 32 * db + ql;
        if (a.grad_f32) {
          ((float*)a.dk)[off] = dk[db][x];
          ((float*)a.dv)[off] = dv[db][x];
        } else {
          ((__bf16*)a.dk)[off] = (__bf16)dk[db][x];
          ((__bf16*)a.dv)[off] = (__bf16)dv[db][x];
        }
      }
    }
}

// ------------------------------------------------------------------------------------
// MU: also accumulate the offset term c dZ db/dmu (db/dmu table tab_dm).
template <int DH, bool CAUSAL, bool MU>
__global__ void __launch_bounds__(256, 2) bwd_dq_kernel(BwdArgs a, int nqb) {
  constexpr int KS = DH / 16;
  constexpr int DB = DH / 32;
  constexpr int TW = kMQ + kNK;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kNK * DH];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[DH * kTS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kNK * DH];
  __shared__ float tw[TW];
  __shared__ float twa[TW];
  __shared__ float twb[TW];
  __shared__ float twm[MU ? TW : 1];
  __shared__ float red[4][4];

  const int BH = a.B * a.H;
  const int qb = blockIdx.x / BH;
  const int bh = blockIdx.x - qb * BH;
  const int h = bh % a.H;
  const int b = bh / a.H;
  const int T = a.T;
  const size_t base = (size_t)bh * T * DH;
  const uint16_t* __restrict__ Q = (const uint16_t*)a.q + base;
  const uint16_t* __restrict__ K = (const uint16_t*)a.k + base;
  const uint16_t* __restrict__ V = (const uint16_t*)a.v + base;
  const uint16_t* __restrict__ dO = (const uint16_t*)a.dout + base;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ql = lane & 31;
  const int hh = lane >> 5;
  const int i0 = qb * kMQ;
  const int i = i0 + wave * 32 + ql;

  bf16x8 qf[KS], of[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 qw = {0u, 0u, 0u, 0u}, ow = {0u, 0u, 0u, 0u};
    if (i < T) {
      qw = *(const u32x4*)(Q + (size_t)i * DH + 16 * ks + 8 * hh);
      ow = *(const u32x4*)(dO + (size_t)i * DH + 16 * ks + 8 * hh);
    }
    qf[ks] = as_bf16x8(qw);
    of[ks] = as_bf16x8(ow);
  }
  const float sqrtD = __builtin_sqrtf((float)DH);
  const float inv_sqrtD = 1.0f / sqrtD;
  const int n_i = CAUSAL ? i + 1 : T;
  const float c = ssmax_c(a.ssmax, a.ssmax ? a.s[h] : 1.0f, n_i);
  const float Cl = fmaxf(c * kLog2e * inv_sqrtD, FLT_MIN);
  const bool valid = i < T;
  const float L2 = valid ? a.lse[(size_t)bh * T + i] * kLog2e : __builtin_huge_valf();
  const float Di = valid ? a.Dbuf[(size_t)bh * T + i] : 0.f;
  const float lnn_sd = a.ssmax ? __logf((float)n_i) * inv_sqrtD : 0.f;

  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int x = 0; x < 16; ++x) dq[db][x] = 0.f;
  float ga = 0.f, gb = 0.f, gs = 0.f, gm = 0.f;

  const int kend = CAUSAL ? min(T, i0 + kMQ) : T;
  const int ntiles = (kend + kNK - 1) / kNK;
  const float* __restrict__ tabh = a.tab + (size_t)h * a.tab_stride;
  const float* __restrict__ tabah = a.tab_da + (size_t)h * a.tab_stride;
  const float* __restrict__ tabbh = a.tab_db + (size_t)h * a.tab_stride;
  const float* __restrict__ tabmh = MU ? a.tab_dm + (size_t)h * a.tab_stride : nullptr;
  const int dlo = CAUSAL ? 0 : -(T - 1);
  const int dhi = T - 1;

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * kNK;
    __syncthreads();
    stage_rows<DH, kNK, 256>(K, j0, T, Ks, tid);
    stage_rows<DH, kNK, 256>(V, j0, T, Vs, tid);
    stage_rows_T<DH, kNK, 256, kTS>(K, j0, T, Kt, tid);
    const int d_min = i0 - j0 - (kNK - 1);
    for (int x = tid; x < TW; x += 256) {
      const int d = d_min + x;
      const bool ok = d >= dlo && d <= dhi;
      tw[x] = ok ? sqrtD * tabh[d - a.tab_d0] : kNegInf;
      twa[x] = ok ? tabah[d - a.tab_d0] : 0.f;
      twb[x] = ok ? tabbh[d - a.tab_d0] : 0.f;
      if (MU) twm[x] = ok ? tabmh[d - a.tab_d0] : 0.f;
    }
    __syncthreads();

    u32x4 zf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s, dp;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int kl = 32 * kb + 8 * (x >> 2) + 4 * hh + (x & 3);
        s[x] = tw[32 * wave + ql + (kNK - 1) - kl];
        dp[x] = 0.f;
      }
      const int r = 32 * kb + ql;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32x32x16(as_bf16x8(read_chunk<DH>(Ks, r, 2 * ks + hh)), qf[ks], s);
        dp = mfma32x32x16(as_bf16x8(read_chunk<DH>(Vs, r, 2 * ks + hh)), of[ks], dp);
      }
      float zv[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int kl = 32 * kb + 8 * (x >> 2) + 4 * hh + (x & 3);
        float sx = s[x];
        if (!CAUSAL && j0 + kl >= T) sx = kNegInf;
        const float p = exp2_fast(Cl * sx - L2);
        const float z = p * (dp[x] - Di);
        zv[x] = z;
        const int widx = 32 * wave + ql + (kNK - 1) - kl;
        const float cz = c * z;
        ga = fmaf(cz, twa[widx], ga);
        gb = fmaf(cz, twb[widx], gb);
        if (MU) gm = fmaf(cz, twm[widx], gm);
        gs = fmaf(z * lnn_sd, fmaxf(sx, -FLT_MAX), gs);
      }
#pragma unroll
      for (int x = 0; x < 16; x += 2) zf[2 * kb + (x >> 3)][(x & 7) >> 1] = pack_bf16x2(zv[x], zv[x + 1]);
    }
    // dQ^T += K^T dZ^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int row = 32 * db + ql;
#pragma unroll
      for (int st = 0; st < 4; ++st)
        dq[db] = mfma32x32x16(read_T_operand<kTS>(Kt, row, 16 * st + 4 * hh), as_bf16x8(zf[st]), dq[db]);
    }
  }

  if (valid) {
    const float cq = c * inv_sqrtD;
    const size_t orow = base + (size_t)i * DH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dh0 = 32 * db + 8 * g + 4 * hh;
        const float o0 = dq[db][4 * g] * cq, o1 = dq[db][4 * g + 1] * cq;
        const float o2 = dq[db][4 * g + 2] * cq, o3 = dq[db][4 * g + 3] * cq;
        if (a.grad_f32) {
          f32x4 w = {o0, o1, o2, o3};
          *(f32x4*)((float*)a.dq + orow + dh0) = w;
        } else {
          u32x2 w = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
          *(u32x2*)((uint16_t*)a.dq + orow + dh0) = w;
        }
      }
  }
  // per-work-group parameter partials (fixed order, no atomics)
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    ga += __shfl_xor(ga, off, 64);
    gb += __shfl_xor(gb, off, 64);
    gs += __shfl_xor(gs, off, 64);
    if (MU) gm += __shfl_xor(gm, off, 64);
  }
  if (lane == 0) {
    red[0][wave] = ga;
    red[1][wave] = gb;
    red[2][wave] = gs;
    red[3][wave] = gm;
  }
  __syncthreads();
  if (tid < 4) {
    const float v = red[tid][0] + red[tid][1] + red[tid][2] + red[tid][3];
    a.param_part[(((size_t)h * a.B + b) * nqb + qb) * 4 + tid] = v;
  }
}

// ------------------------------------------------------------------------------------
__global__ void __launch_bounds__(64) bwd_params_kernel(BwdArgs a, int nper) {
  const int k = blockIdx.x;   // 0: alpha, 1: beta, 2: s, 3: mu
  const int h = blockIdx.y;
  double acc = 0.0;
  if (k == 3 && a.dmu == nullptr) return;
  for (int x = threadIdx.x; x < nper; x += 64) acc += (double)a.param_part[((size_t)h * nper + x) * 4 + k];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) acc += __shfl_xor(acc, off, 64);
  if (threadIdx.x == 0) {
    float* out = k == 0 ? a.dalpha : (k == 1 ? a.dbeta : (k == 2 ? a.ds : a.dmu));
    out[h] = (k == 2 && !a.ssmax) ? 0.f : (float)acc;
  }
}

template <int DH, bool CAUSAL>
hipError_t launch_t(const BwdArgs& a, hipStream_t stream) {
  const long nrows = (long)a.B * a.H * a.T;
  const long pre_threads = nrows * (DH / 8);
  hipLaunchKernelGGL(bwd_pre_kernel<DH>, dim3((unsigned)((pre_threads + 255) / 256)), dim3(256), 0, stream,
                     a, nrows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nkb = (a.T + kKB - 1) / kKB;
  hipLaunchKernelGGL((bwd_dkdv_kernel<DH, CAUSAL>), dim3((unsigned)(nkb * a.B * a.H)), dim3(256), 0, stream,
                     a, nkb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqb = (a.T + kMQ - 1) / kMQ;
  if (a.tab_dm)
    hipLaunchKernelGGL((bwd_dq_kernel<DH, CAUSAL, true>), dim3((unsigned)(nqb * a.B * a.H)), dim3(256), 0,
                       stream, a, nqb);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<DH, CAUSAL, false>), dim3((unsigned)(nqb * a.B * a.H)), dim3(256), 0,
                       stream, a, nqb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_params_kernel, dim3(4, a.H), dim3(64), 0, stream, a, a.B * nqb);
  return hipGetLastError();
}

}  // namespace

size_t bwd_param_partials(int B, int H, int T) { return (size_t)H * B * ((T + kMQ - 1) / kMQ) * 4; }

hipError_t launch_bwd(const BwdArgs& a, int Dh, hipStream_t stream) {
  switch (Dh) {
    case 32: return a.causal ? launch_t<32, true>(a, stream) : launch_t<32, false>(a, stream);
    case 64: return a.causal ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bam
