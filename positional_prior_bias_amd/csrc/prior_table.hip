// Per-head distance table of the Generalized-Gaussian positional prior.
//
// "Résumé Technique : Mécanisme d'Attention Bayésienne (BAM)", "Solution Proposée :
// GGD-BAM": b = -|x / alpha|^beta per head.  The offset convention is x = d - mu with
// d = i - j (query minus key).  The bias depends on the distance only, so one row of
// n values per head replaces the dense T x T matrix; it is rebuilt on every call since
// alpha and beta are trained parameters ("Bayesian Attention Mechanism",
// "Implementation Details").  One power per (head, distance): the exponent in float64,
// the final 2^fraction in float32 (pow_pos), rounded once to float32.  The value and
// derivatives at one distance come from prior_bias_at, which the short-sequence forward
// kernel also calls for its own bias window.
//
// The same table carries any other bias that depends on the head and i - j only.  The
// Sandwich bias (attention-gym "Score Mods", "Sandwich") is the inner product of two
// d_bar-dimensional sinusoidal position embeddings, sum_i cos(d w_i) / ratio_h with
// w_i = 10000^(-2 i / d_bar) over the d_bar / 2 frequencies, and has no parameters.
#include "../../include/bam.h"
#include "bam_device.h"
#include "bam_internal.h"
#include "prior_eval.h"

namespace bam {

// Entry t of head h holds distance d = d_first + step * t.  Distances outside
// [dlo, dhi] are padding: -inf in the bias table (a key never visible), 0 in the
// derivative tables.  kind kPriorAlpha: alpha-form; kPriorRef: the reference
// parameterisation ("Bayesian Attention Mechanism", "Implementation Details"), where
// alpha / beta / mu hold theta_alpha / theta_beta / theta_mu, x = (j - i) - mu = -d - mu,
// mu = e^theta_mu - e^-theta_mu and b = -e^theta_alpha (|x| + eps)^theta_beta;
// kPriorSandwich: alpha holds ratio_h and beta d_bar (d_bar above 2 kSandwichMaxFreq is
// taken as 2 kSandwichMaxFreq, and the frequency count is trunc(d_bar) / 2; a NaN d_bar
// violates the precondition of finite parameters and counts as no frequency, so every
// entry is finite), and the derivative tables are zero.
constexpr int kSandwichMaxFreq = 4096;

namespace {

__global__ void __launch_bounds__(256) prior_table_kernel(const float* __restrict__ alpha,
                                                          const float* __restrict__ beta,
                                                          const float* __restrict__ mu, int kind,
                                                          int d_first, int step, int n, int stride,
                                                          int dlo, int dhi, float scale,
                                                          float* __restrict__ tab,
                                                          float* __restrict__ ta,
                                                          float* __restrict__ tb,
                                                          float* __restrict__ tm) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int h = blockIdx.y;
  // Sandwich: the inverse frequencies 10000^(2 i / d_bar) of this head, once per block, in
  // dynamic LDS (kSandwichMaxFreq doubles; the launch gives none for the other kinds).
  extern __shared__ double inv_w[];
  int nf = 0;
  if (kind == kPriorSandwich) {
    // trunc(min(d_bar, 8192)) / 2 frequencies; a NaN d_bar (tested by its bits: the library
    // is built with -fno-honor-nans) counts as none
    const float db0 = beta[h];
    const bool nan = (__float_as_uint(db0) & 0x7fffffffu) > 0x7f800000u;
    const float db = nan ? 0.f : fminf(db0, 2.0f * kSandwichMaxFreq);   // d_bar above 8192 is taken as 8192
    nf = db < 2.0f ? 0 : (int)db / 2;
    for (int i = threadIdx.x; i < nf; i += blockDim.x) inv_w[i] = pow(10000.0, 2.0 * i / (double)db);
    __syncthreads();
  }
  if (t >= n) return;
  const int d = d_first + step * t;
  const size_t idx = (size_t)h * stride + t;
  if (d < dlo || d > dhi) {
    tab[idx] = -__builtin_huge_valf();
    if (ta) ta[idx] = 0.f;
    if (tb) tb[idx] = 0.f;
    if (tm) tm[idx] = 0.f;
    return;
  }
  const double a = alpha[h];
  const double be = beta[h];
  const double m = mu ? (double)mu[h] : 0.0;
  const bool der = ta || tb || tm;   // derivative tables wanted (the forward's table is bias only)
  double b;
  PriorDerivs D;
  if (kind == kPriorSandwich) {
    double acc = 0.0;
    for (int i = 0; i < nf; ++i) acc += cos((double)d / inv_w[i]);
    b = acc / a;
  } else {
    b = prior_bias_at(kind, a, be, m, d, der, D);
  }
  // The derivatives saturate at +-FLT_MAX: where u^beta overflows float32 the bias is -inf
  // and the weight exactly 0, and the backward's product 0 * derivative must stay 0.
  const double kFltMax = 3.4028234663852886e38;
  tab[idx] = (float)(b * scale);
  if (ta) ta[idx] = (float)fmin(kFltMax, fmax(-kFltMax, D.da));
  if (tb) tb[idx] = (float)fmin(kFltMax, fmax(-kFltMax, D.db));
  if (tm) tm[idx] = (float)fmin(kFltMax, fmax(-kFltMax, D.dm));
}

}  // namespace

hipError_t launch_prior_table(const float* alpha, const float* beta, const float* mu, int kind, int H,
                              int d0, int n, int stride, float scale, float* tab, float* dalpha,
                              float* dbeta, float* dmu, hipStream_t stream) {
  return launch_prior_table_ex(alpha, beta, mu, kind, H, d0, 1, n, stride, d0, d0 + n - 1, scale, tab,
                               dalpha, dbeta, dmu, stream);
}

hipError_t launch_prior_table_ex(const float* alpha, const float* beta, const float* mu, int kind, int H,
                                 int d_first, int step, int n, int stride, int dlo, int dhi, float scale,
                                 float* tab, float* dalpha, float* dbeta, float* dmu, hipStream_t stream) {
  dim3 grid((n + 255) / 256, H);
  const size_t lds = kind == kPriorSandwich ? kSandwichMaxFreq * sizeof(double) : 0;
  hipLaunchKernelGGL(prior_table_kernel, grid, dim3(256), lds, stream, alpha, beta, mu, kind, d_first,
                     step, n, stride, dlo, dhi, scale, tab, dalpha, dbeta, dmu);
  return hipGetLastError();
}

}  // namespace bam
