// Per-head distance table of the Generalized-Gaussian positional prior.
//
// "Résumé Technique : Mécanisme d'Attention Bayésienne (BAM)", "Solution Proposée :
// GGD-BAM": b = -|x / alpha|^beta per head.  The offset convention is x = d - mu with
// d = i - j (query minus key).  The bias depends on the distance only, so one row of
// n values per head replaces the dense T x T matrix; it is rebuilt on every call since
// alpha and beta are trained parameters ("Bayesian Attention Mechanism",
// "Implementation Details").  One pow per (head, distance), evaluated in float64 and
// rounded once to float32.
#include "../../include/bam.h"
#include "bam_device.h"
#include "bam_internal.h"

namespace bam {

// Entry t of head h holds distance d = d_first + step * t.  Distances outside
// [dlo, dhi] are padding: -inf in the bias table (a key never visible), 0 in the
// derivative tables.  ref = 0: alpha-form; ref = 1: the reference parameterisation
// ("Bayesian Attention Mechanism", "Implementation Details"), where alpha / beta / mu
// hold theta_alpha / theta_beta / theta_mu, x = (j - i) - mu = -d - mu,
// mu = e^theta_mu - e^-theta_mu and b = -e^theta_alpha (|x| + eps)^theta_beta.
__global__ void __launch_bounds__(256) prior_table_kernel(const float* __restrict__ alpha,
                                                          const float* __restrict__ beta,
                                                          const float* __restrict__ mu, int ref,
                                                          int d_first, int step, int n, int stride,
                                                          int dlo, int dhi, float scale,
                                                          float* __restrict__ tab,
                                                          float* __restrict__ ta,
                                                          float* __restrict__ tb,
                                                          float* __restrict__ tm) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int h = blockIdx.y;
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
  double b, da = 0.0, db = 0.0, dm = 0.0;
  if (ref) {
    // b = -e^ta g^tb, g = |x| + eps: db/dta = b, db/dtb = b ln g,
    // db/dtm = -b tb sign(x) / g * (e^tm + e^-tm)
    const double em = exp(m), emi = exp(-m);
    const double x = -(double)d - (em - emi);
    const double g = fabs(x) + (double)BAM_REF_EPS;
    b = -exp(a) * pow(g, be);
    da = b;
    db = b * log(g);
    const double sg = x > 0.0 ? 1.0 : (x < 0.0 ? -1.0 : 0.0);
    dm = -b * be * sg / g * (em + emi);
  } else {
    const double x = (double)d - m;
    const double u = __builtin_isinf(a) ? 0.0 : fabs(x) / a;
    if (be == 0.0) {
      b = -1.0;                                   // 0^0 = 1
      if (u != 0.0) db = -log(u);
    } else if (u == 0.0) {
      b = be > 0.0 ? 0.0 : -__builtin_huge_val();  // beta < 0 at u = 0: precondition violated
    } else {
      const double p = pow(u, be);
      b = -p;
      da = be * p / a;
      db = -p * log(u);
      dm = be * p / x;                             // db/dmu, dx/dmu = -1
    }
  }
  tab[idx] = (float)(b * scale);
  if (ta) ta[idx] = (float)da;
  if (tb) tb[idx] = (float)db;
  if (tm) tm[idx] = (float)dm;
}

hipError_t launch_prior_table(const float* alpha, const float* beta, const float* mu, bool ref, int H,
                              int d0, int n, int stride, float scale, float* tab, float* dalpha,
                              float* dbeta, float* dmu, hipStream_t stream) {
  return launch_prior_table_ex(alpha, beta, mu, ref, H, d0, 1, n, stride, d0, d0 + n - 1, scale, tab,
                               dalpha, dbeta, dmu, stream);
}

hipError_t launch_prior_table_ex(const float* alpha, const float* beta, const float* mu, bool ref, int H,
                                 int d_first, int step, int n, int stride, int dlo, int dhi, float scale,
                                 float* tab, float* dalpha, float* dbeta, float* dmu, hipStream_t stream) {
  dim3 grid((n + 255) / 256, H);
  hipLaunchKernelGGL(prior_table_kernel, grid, dim3(256), 0, stream, alpha, beta, mu, ref ? 1 : 0, d_first,
                     step, n, stride, dlo, dhi, scale, tab, dalpha, dbeta, dmu);
  return hipGetLastError();
}

}  // namespace bam
