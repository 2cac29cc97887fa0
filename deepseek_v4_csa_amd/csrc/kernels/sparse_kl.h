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

constexpr float KL_EPS = 1e-10f;

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

// log(1 + x) for x > -1: |x| < 1/2 by the series 2 atanh(u), u = x / (2 + x) (|u| < 1/3,
// terms through u^15: truncation below 3e-9 relative; the quotient by the hardware
// reciprocal, 1 ulp); otherwise the hardware log of 1 + x, where 1 + x is exact enough
// (relative error ~1e-7 of the result).
__device__ __forceinline__ float log1p_kl(float x) {
  if (fabsf(x) < 0.5f) {
    const float u = x * __builtin_amdgcn_rcpf(2.f + x);
    const float u2 = u * u;
    float p = 1.f / 15.f;
    p = fmaf(p, u2, 1.f / 13.f);
    p = fmaf(p, u2, 1.f / 11.f);
    p = fmaf(p, u2, 1.f / 9.f);
    p = fmaf(p, u2, 1.f / 7.f);
    p = fmaf(p, u2, 1.f / 5.f);
    p = fmaf(p, u2, 1.f / 3.f);
    p = fmaf(p, u2, 1.f);
    return 2.f * u * p;
  }
  return __log2f(1.f + x) * LN2;
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
// slot in c[v] (0 off the support); sc[v] is overwritten (the predictor's exponentials
// take its place: the arrays are reused so that long rows keep few registers).  Every lane
// of the wave must take part.
//
// The KL of two nearly equal distributions is a second-order quantity, so the normalisers
// and the log-ratios are finished in fp64: an fp32 error in either normaliser would shift
// the KL by about that relative error.  The predictor terms are fp32 (an independent
// relative error d_j of e_j moves the KL only through sum_j (t_j - p_j) d_j).
// log(t + eps) - log(p + eps) is taken as log1p(x), x = (t - p) / (p + eps), with t - p in
// fp64 and the rest in fp32 (the quotient by the hardware reciprocal, 1 ulp), so the KL
// moves by ~1e-7 * sum_j t_j |x_j|.
template <int N, class Red = WaveRed>
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
  double es = 0.0;
#pragma unroll
  for (int v = 0; v < N; ++v) {
    sc[v] = ok[v] ? fast_exp2((sc[v] - mx) * LOG2E) : 0.f;   // e_j from here on
    es += (double)sc[v];
  }
  es = red.sum(es);
  const double inv_es = 1.0 / es;
  const double inv_m = 1.0 / fmax(ms, (double)KL_EPS);
  double kl = 0.0;
#pragma unroll
  for (int v = 0; v < N; ++v) {
    double t = 0.0;
    if (ok[v]) {
      t = (double)c[v] * inv_m;
      const double pj = (double)sc[v] * inv_es;
      const float x = (float)(t - pj) * __builtin_amdgcn_rcpf((float)pj + KL_EPS);
      kl += t * (double)log1p_kl(x);
    }
    c[v] = (float)t;   // the teacher value
  }
  return red.sum(kl);
}

}  // namespace csa
