// tau_solve.hpp -- pieces of the alpha-entmax threshold solve used inside the
// routing and dense-entmax kernels.
//
// alpha-entmax (named with its alpha and n_iter arguments in the AdaSplash
// README, "Usage: Triton Entmax"; definition of Peters, Niculae & Martins 2019):
//   p_i = max(u_i - tau, 0)^beta,  beta = 1 / (alpha - 1),  sum_i p_i = 1.
// tau is the root of the decreasing function
//   f(tau)   = sum_i max(u_i - tau, 0)^beta - 1
//   f'(tau)  = -beta         sum_i max(u_i - tau, 0)^(beta - 1)
//   f''(tau) =  beta (beta-1) sum_i max(u_i - tau, 0)^(beta - 2)
// bracketed by [max u - 1, max u - n^-(alpha-1)] (f >= 0 at the left end since
// the largest term is 1; f <= 0 at the right end since every p <= n^-1 there).
// Each step evaluates f, f', f'' at tau, shrinks the bracket by the sign of f,
// takes the Halley step tau - 2 f f' / (2 f'^2 - f f'') and falls back to
// bisection when the step leaves the bracket ("Halley's method + bisection").
//
// KIND selects closed forms of the powers: 2 for alpha = 1.5 (beta = 2),
// 1 for alpha = 2 (beta = 1, Halley reduces to Newton), 0 for any other alpha.
#pragma once

#include "cdna4.hpp"

namespace dash {

template <int KIND>
__device__ __forceinline__ void tau_terms(float u, float tau, float beta, float& f0, float& f1,
                                          float& f2) {
  const float t = u - tau;
  if constexpr (KIND == 2) {
    const float p = fmaxf(t, 0.f);
    f0 = fmaf(p, p, f0);
    f1 += p;
    f2 += (t > 0.f) ? 1.f : 0.f;
  } else if constexpr (KIND == 1) {
    f0 += fmaxf(t, 0.f);
    f1 += (t > 0.f) ? 1.f : 0.f;
  } else {
    if (t > 0.f) {
      const float lg = fast_log2(t);
      f0 += fast_exp2(beta * lg);
      f1 += fast_exp2((beta - 1.f) * lg);
      f2 += fast_exp2((beta - 2.f) * lg);
    }
  }
}

// One safeguarded step from tau with sums (f0, f1, f2) evaluated at tau.
// Updates the bracket [lo, hi]; returns the next tau.
template <int KIND>
__device__ __forceinline__ float tau_step(float tau, float f0, float f1, float f2, float beta,
                                          float& lo, float& hi) {
  const float f = f0 - 1.f;
  if (f == 0.f) {
    lo = hi = tau;
    return tau;
  }
  float fp, fpp;
  if constexpr (KIND == 2) {
    fp = -2.f * f1;
    fpp = 2.f * f2;
  } else if constexpr (KIND == 1) {
    fp = -f1;
    fpp = 0.f;
  } else {
    fp = -beta * f1;
    fpp = beta * (beta - 1.f) * f2;
  }
  if (f > 0.f) {
    lo = tau;
  } else {
    hi = tau;
  }
  const float den = 2.f * fp * fp - f * fpp;
  float nt = (den != 0.f) ? tau - 2.f * f * fp / den : 0.5f * (lo + hi);
  if (!(nt >= lo && nt <= hi)) nt = 0.5f * (lo + hi);  // closed: a step that stays put is kept
  return nt;
}

__device__ __forceinline__ bool tau_converged(float old_tau, float new_tau) {
  return fabsf(new_tau - old_tau) <= 1e-6f * fmaxf(1.f, fabsf(new_tau));
}

// log2 of the prior max(t, 0)^beta for t > 0.
template <int KIND>
__device__ __forceinline__ float log2_prior(float t, float beta) {
  const float lg = fast_log2(t);
  if constexpr (KIND == 2) return 2.f * lg;
  else if constexpr (KIND == 1) return lg;
  else return beta * lg;
}

// The prior max(t, 0)^beta itself.
template <int KIND>
__device__ __forceinline__ float prior_of(float t, float beta) {
  const float p = fmaxf(t, 0.f);
  if constexpr (KIND == 2) return p * p;
  else if constexpr (KIND == 1) return p;
  else return (t > 0.f) ? fast_exp2(beta * fast_log2(t)) : 0.f;
}

// Right end of the bracket: max u - n^-(alpha - 1).
__device__ __forceinline__ float tau_upper(float mx, int n, float alpha) {
  return mx - fast_exp2(-(alpha - 1.f) * fast_log2((float)n));
}

}  // namespace dash
