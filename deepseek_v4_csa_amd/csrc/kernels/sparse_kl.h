// The sparse-loss teacher and KL of one query row, finished by one wave.
//
// Page "[Bug] DSV4 unfused CSA indexer loss uses a compressed-only teacher ...":
//   "Paper reference": t_j = sum_h exp(c_hj)/Z_h, L1-normalised over the compressed set;
//   dsa.py excerpt: the L1 sum is clamped at 1e-10 and the KL takes log(x + 1e-10) on
//   both sides (kept as written, review comment "KL numerical contract");
//   dsa_kernels.py excerpt: the sparse predictor is the softmax of the indexer scores at
//   the top-k ids, -1 slots left out.
// Used by the stand-alone teacher kernel and by the attention kernel that finishes the
// loss in its epilogue, so both take the same arithmetic.
#pragma once
#include "common.h"

namespace csa {

// What a kernel that finishes the sparse loss itself needs besides its own outputs:
// the scores at the selected slots (slot j of row t holds the score of ids[t, j], row
// stride ld), the teacher output (NULL: not written; row stride ldt) and kl_row [T].
struct KlArgs {
  const float *scores;
  int64_t ld;
  float *teacher;
  int64_t ldt;
  float *kl_row;
};

// The predictor's exponential e^(s - mx) in fp64 (s and mx are fp32, so the difference is
// exact) and one KL term t (log(t + eps) - log(p + eps)) = t log1p((t - p) / (p + eps))
// in fp64.  For nearly equal t and p the KL is second order in t - p, so p must carry far
// more than fp32's 24 bits for the KL of such a row to keep 1e-5 relative accuracy; an
// error in the sum of the e_j shifts the KL by the same amount in absolute terms.
constexpr double KL_EPS = 1e-10;
// e^d for d <= 0: d log2(e) = n + f with n = rint(d log2(e)) and |f| <= 1/2, so
// e^d = 2^n e^x with x = f ln 2, |x| <= 0.35, and e^x is its Taylor series to degree 10
// (truncation below 3e-13 relative); arguments below -1100 log 2 give 0.
__device__ __forceinline__ double exp_nonpos_f64(double d) {
  const double y = fmax(d * 1.4426950408889634074, -1100.0);
  const double n = rint(y);
  const double x = (y - n) * 0.69314718055994530942;
  double p = 1.0 / 3628800.0;
  p = fma(p, x, 1.0 / 362880.0);
  p = fma(p, x, 1.0 / 40320.0);
  p = fma(p, x, 1.0 / 5040.0);
  p = fma(p, x, 1.0 / 720.0);
  p = fma(p, x, 1.0 / 120.0);
  p = fma(p, x, 1.0 / 24.0);
  p = fma(p, x, 1.0 / 6.0);
  p = fma(p, x, 0.5);
  p = fma(p, x, 1.0);
  p = fma(p, x, 1.0);
  return ldexp(p, (int)n);
}
__device__ __forceinline__ double pred_exp(float s, float mx) { return exp_nonpos_f64((double)s - (double)mx); }
// log(1 + x), x > -1.  For |x| < 1/2 from log(1 + x) = 2 atanh(u), u = x / (2 + x), |u| < 1/3:
// 2 (u + u^3/3 + ... + u^27/27), truncation below 1e-14 relative (the log-ratios of a KL row
// are small, so this is the common case); otherwise the device library's log1p.
__device__ __forceinline__ double log1p_kl(double x) {
  if (fabs(x) < 0.5) {
    const double u = x / (2.0 + x), u2 = u * u;
    double p = 1.0 / 27;
#pragma unroll
    for (int k = 25; k >= 1; k -= 2) p = fma(p, u2, 1.0 / k);
    return 2.0 * u * p;
  }
  return log1p(x);
}
template <bool SERIES = true>
__device__ __forceinline__ double kl_term(double t, double p) {
  const double x = (t - p) / (p + KL_EPS);
  return t * (SERIES ? log1p_kl(x) : log1p(x));
}

// Reductions over the lanes that hold one row: a whole wave (WaveRed), or NW waves of one
// workgroup (GroupRed: one LDS entry per wave, combined in wave order, so the result is the
// same in every lane and every run).  With GroupRed every wave of the workgroup must reach
// every reduction, whatever row it holds.
struct WaveRed {
  __device__ __forceinline__ float max(float v) const { return wave_max_dpp(v); }
  __device__ __forceinline__ double sum(double v) const { return wave_sum_f64_dpp(v); }
};
template <int NW> struct GroupRed {
  float *fb;    // NW floats of LDS for this row
  double *db;   // NW doubles of LDS for this row
  int w;        // this wave's index among the row's NW waves
  __device__ __forceinline__ float max(float v) const {
    v = wave_max_dpp(v);
    if ((threadIdx.x & 63) == 0) fb[w] = v;
    __syncthreads();
    float r = fb[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) r = fmaxf(r, fb[i]);
    __syncthreads();
    return r;
  }
  __device__ __forceinline__ double sum(double v) const {
    v = wave_sum_f64_dpp(v);
    if ((threadIdx.x & 63) == 0) db[w] = v;
    __syncthreads();
    double r = db[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) r += db[i];
    __syncthreads();
    return r;
  }
};

// The lanes that hold a row hold its support slots, N per lane in any arrangement: ok[v] marks a slot
// of the support (a valid id), c[v] its head-summed mass m_j, sc[v] its indexer score.
// Returns the row's KL (the same value in every lane) and leaves the teacher value of each
// slot in c[v] (0 off the support, the array reused so that long rows keep few registers).
// Every lane of the wave must take part.
//
// The KL of two nearly equal distributions is a second-order quantity, so everything after
// the inputs is fp64: the teacher normaliser, the predictor's exponentials and their sum,
// and the log-ratios (pred_exp, kl_term).
// LEAN = false keeps the N exponentials in registers between the two loops (2N VGPRs) and
// takes the log-ratios from the series; a kernel short of registers passes LEAN = true and
// recomputes the exponentials and calls the library's log1p.
template <int N, class Red = WaveRed, bool LEAN = false>
__device__ __forceinline__ double sparse_kl_wave(const bool (&ok)[N], float (&c)[N], float (&sc)[N],
                                                 const Red &red = Red()) {
  float mx = -__builtin_inff();
  double ms = 0.0;
#pragma unroll
  for (int v = 0; v < N; ++v) {
    mx = fmaxf(mx, ok[v] ? sc[v] : -__builtin_inff());
    ms += ok[v] ? (double)c[v] : 0.0;
  }
  mx = red.max(mx);
  ms = red.sum(ms);
  constexpr bool KEEP_E = !LEAN;
  double es = 0.0, e[KEEP_E ? N : 1];
#pragma unroll
  for (int v = 0; v < N; ++v) {
    const double x = ok[v] ? pred_exp(sc[v], mx) : 0.0;
    if constexpr (KEEP_E) e[v] = x;
    es += x;
  }
  es = red.sum(es);
  const double inv_es = 1.0 / es;
  const double inv_m = 1.0 / fmax(ms, KL_EPS);
  double kl = 0.0;
#pragma unroll
  for (int v = 0; v < N; ++v) {
    double t = 0.0;
    if (ok[v]) {
      t = (double)c[v] * inv_m;
      kl += kl_term<!LEAN>(t, (KEEP_E ? e[v] : pred_exp(sc[v], mx)) * inv_es);
    }
    c[v] = (float)t;   // the teacher value
  }
  return red.sum(kl);
}

}  // namespace csa
