// The Generalized-Gaussian positional prior at one distance, shared by the distance-table
// kernel and the short-sequence forward kernel (which computes its bias window itself), so
// both produce the same float32 values.
//
// "Résumé Technique : Mécanisme d'Attention Bayésienne (BAM)", "Solution Proposée :
// GGD-BAM": b = -|x / alpha|^beta per head, x = d - mu with d = i - j (query minus key).
// The reference parameterisation ("Bayesian Attention Mechanism", "Implementation
// Details"): alpha / beta / mu hold theta_alpha / theta_beta / theta_mu,
// x = (j - i) - mu = -d - mu, mu = e^theta_mu - e^-theta_mu, b = -e^theta_alpha
// (|x| + eps)^theta_beta.
#pragma once

#include <float.h>
#include <hip/hip_runtime.h>

#include "../../include/bam.h"
#include "bam_internal.h"

namespace bam {

// u^e for u > 0: the exponent y = e log2(u) in float64, split into an integer n and a
// fraction f in [0, 1); 2^f in float32 (one v_exp_f32, about 1 ulp), scaled by 2^n
// exactly.  The result is within about 2 float32 ulps of the float64 pow, which it
// replaces because the bias is rounded to float32 anyway and pow costs several times as
// much.  log2(u) is returned for the derivative tables.  Exponents beyond +-1000 (the
// value is then 0 or inf in float32) go through pow.
__device__ __forceinline__ double pow_pos(double u, double e, double& l2) {
  l2 = log2(u);
  const double y = e * l2;
  if (!(fabs(y) < 1000.0)) return pow(u, e);
  const double n = floor(y);
  return ldexp((double)exp2f((float)(y - n)), (int)n);
}

// Derivatives of b with respect to the head's three parameters (zero where not defined).
struct PriorDerivs {
  double da = 0.0, db = 0.0, dm = 0.0;
};

// b(d) in float64 for kind kPriorAlpha or kPriorRef (a, be, m: the head's alpha, beta, mu
// or theta_alpha, theta_beta, theta_mu); with der, also its derivatives:
//   alpha form: db/dalpha = beta u^beta / alpha, db/dbeta = -u^beta ln u (-ln u at
//     beta = 0, where b = -1), db/dmu = beta u^beta / x;
//   reference form: db/dtheta_alpha = b, db/dtheta_beta = b ln g,
//     db/dtheta_mu = -b theta_beta sign(x) / g (e^theta_mu + e^-theta_mu), g = |x| + eps.
// alpha = +inf gives u = 0 (NoPE for beta > 0); beta < 0 at u = 0 gives -inf.
__device__ __forceinline__ double prior_bias_at(int kind, double a, double be, double m, int d, bool der,
                                                PriorDerivs& D) {
  if (kind == kPriorRef) {
    const double em = exp(m), emi = exp(-m);
    const double x = -(double)d - (em - emi);
    const double g = fabs(x) + (double)BAM_REF_EPS;
    double l2g;
    const double b = -exp(a) * pow_pos(g, be, l2g);
    if (der) {
      D.da = b;
      D.db = b * l2g * 0.6931471805599453;   // b ln g
      const double sg = x > 0.0 ? 1.0 : (x < 0.0 ? -1.0 : 0.0);
      D.dm = -b * be * sg / g * (em + emi);
    }
    return b;
  }
  const double x = (double)d - m;
  const double u = __builtin_isinf(a) ? 0.0 : fabs(x) / a;
  if (be == 0.0) {
    if (u != 0.0) D.db = -log(u);
    return -1.0;                                   // 0^0 = 1
  }
  if (u == 0.0) return be > 0.0 ? 0.0 : -__builtin_huge_val();   // beta < 0 at u = 0: precondition violated
  double l2u;
  const double p = pow_pos(u, be, l2u);
  if (der) {
    D.da = be * p / a;
    D.db = -p * l2u * 0.6931471805599453;  // -p ln u
    D.dm = be * p / x;                     // db/dmu, dx/dmu = -1
  }
  return -p;
}

// b(d) in float32 arithmetic, for kernels that compute their bias window themselves: the
// same cases as prior_bias_at, the power as 2^(beta log2 u) with the hardware log2 and exp2
// (each about 1 ulp), so the value is within a few float32 ulps of prior_bias_at's (the
// exponent's error, |y| 2^-23 for y = beta log2 u, becomes a relative error of about
// 0.7 |y| 2^-23).  No float64 work and a handful of registers.
__device__ __forceinline__ float prior_bias_f32(int kind, float a, float be, float m, int d) {
  if (kind == kPriorRef) {
    const float mu = __expf(m) - __expf(-m);
    const float g = fabsf(-(float)d - mu) + (float)BAM_REF_EPS;
    // -e^theta_alpha g^theta_beta = -2^(theta_alpha log2(e) + theta_beta log2(g))
    return -__builtin_amdgcn_exp2f(fmaf(be, __builtin_amdgcn_logf(g), a * 1.4426950408889634f));
  }
  const float u = __builtin_isinf(a) ? 0.f : fabsf((float)d - m) / a;
  if (be == 0.f) return -1.f;                                    // 0^0 = 1
  if (u == 0.f) return be > 0.f ? 0.f : -__builtin_huge_valf();  // beta < 0 at u = 0: precondition violated
  return -__builtin_amdgcn_exp2f(be * __builtin_amdgcn_logf(u));
}

// b(d) and its three parameter derivatives in float32 (prior_bias_at's cases and formulas),
// the derivatives saturated at +-FLT_MAX as the distance-table kernel stores them (where
// u^beta overflows the bias is -inf and the weight exactly 0, and the backward's product
// 0 * derivative must stay 0).
__device__ __forceinline__ void prior_derivs_f32(int kind, float a, float be, float m, int d, float& b, float& da,
                                                 float& db, float& dm) {
  constexpr float kLn2f = 0.6931471805599453f, kLog2ef = 1.4426950408889634f;
  da = db = dm = 0.f;
  if (kind == kPriorRef) {
    const float em = __expf(m), emi = __expf(-m);
    const float x = -(float)d - (em - emi);
    const float g = fabsf(x) + (float)BAM_REF_EPS;
    const float l2g = __builtin_amdgcn_logf(g);
    b = -__builtin_amdgcn_exp2f(fmaf(be, l2g, a * kLog2ef));
    da = b;
    db = b * l2g * kLn2f;   // b ln g
    const float sg = x > 0.f ? 1.f : (x < 0.f ? -1.f : 0.f);
    dm = -b * be * sg / g * (em + emi);
  } else {
    const float x = (float)d - m;
    const float u = __builtin_isinf(a) ? 0.f : fabsf(x) / a;
    if (be == 0.f) {
      b = -1.f;                                              // 0^0 = 1
      if (u != 0.f) db = -__builtin_amdgcn_logf(u) * kLn2f;  // -ln u
    } else if (u == 0.f) {
      b = be > 0.f ? 0.f : -__builtin_huge_valf();
    } else {
      const float l2u = __builtin_amdgcn_logf(u);
      const float p = __builtin_amdgcn_exp2f(be * l2u);
      b = -p;
      da = be * p / a;
      db = -p * l2u * kLn2f;   // -p ln u
      dm = be * p / x;         // db/dmu, dx/dmu = -1
    }
  }
  da = fminf(FLT_MAX, fmaxf(-FLT_MAX, da));
  db = fminf(FLT_MAX, fmaxf(-FLT_MAX, db));
  dm = fminf(FLT_MAX, fmaxf(-FLT_MAX, dm));
}

}  // namespace bam
