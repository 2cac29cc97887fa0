// Lightning-Indexer scores on gfx950 MFMA.
//
//   scores[t, j] = sum_h ws[t,h] * max(0, q_idx[t,h,:] . k_idx[cu_k[s]+j, :])   j < n_valid(t)
//                = -inf                                                          otherwise
// (scale folded into the weights as fp32(w * s_idx): csa.py SBHD excerpt of the page
// "[Bug] DSV4 unfused CSA indexer loss uses a compressed-only teacher ..."; mask
// j < i // ratio from the same excerpt; per-segment bottom-right offsets from the page
// "Megatron-LM pull request 8539", item 2.)
//
// Work decomposition: one workgroup = 4 waves = a 64-token x 64-key output tile of one
// segment.  Wave w owns tokens [16w, 16w+16) of the tile and all 64 keys (4 MFMA
// N-tiles).  The key tile (one k_idx row shared by every indexer head) stays in
// registers for the whole head loop; for each head the wave loads its 16 q_idx rows
// and runs Di/32 MFMAs per N-tile, then folds ReLU x weight into a per-(token,key) fp32
// accumulator.  The per-head [token, head, key] product never leaves registers.
// Tiles entirely above the causal limit are only filled with -inf.
#include "common.h"
#include "../launch.h"

namespace csa {

constexpr int IDX_BT = 64;   // tokens per workgroup
constexpr int IDX_BN = 64;   // keys per workgroup
constexpr int IDX_THREADS = 256;

// Operand fragments.  bf16: a lane holds Di/4 consecutive elements of one row
// (Di/32 chunks of 8 bf16); the MFMA K index g*8+e of chunk c maps to the feature
// d = g*(Di/4) + c*8 + e, identically for A and B, so the sum over K covers every d
// once.  fp32: a lane holds Di/4 consecutive floats; chunk c, lane group g -> d =
// g*(Di/4) + c.
template <typename IN, int DI> struct Frag;

template <int DI> struct Frag<uint16_t, DI> {
  static constexpr int NC = DI / 32;
  u32x4 v[NC];
  __device__ __forceinline__ void load(const uint16_t *row, int g, bool ok) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(row + g * (DI / 4));
#pragma unroll
    for (int c = 0; c < NC; ++c) v[c] = ok ? p[c] : u32x4{0, 0, 0, 0};
  }
  __device__ __forceinline__ static f32x4 dot(const Frag &a, const Frag &b) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) acc = mfma16x16x32(a.v[c], b.v[c], acc);
    return acc;
  }
};

template <int DI> struct Frag<float, DI> {
  static constexpr int NC = DI / 4;
  float v[NC];
  __device__ __forceinline__ void load(const float *row, int g, bool ok) {
    const f32x4 *p = reinterpret_cast<const f32x4 *>(row + g * (DI / 4));
#pragma unroll
    for (int c = 0; c < NC / 4; ++c) {
      f32x4 x = ok ? p[c] : f32x4{0.f, 0.f, 0.f, 0.f};
      v[4 * c + 0] = x[0]; v[4 * c + 1] = x[1]; v[4 * c + 2] = x[2]; v[4 * c + 3] = x[3];
    }
  }
  __device__ __forceinline__ static f32x4 dot(const Frag &a, const Frag &b) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) acc = mfma16x16x4f32(a.v[c], b.v[c], acc);
    return acc;
  }
};

template <typename IN, int DI>
__global__ __launch_bounds__(IDX_THREADS) void indexer_score_kernel(
    LayoutDev L, const IN *__restrict__ q_idx, const IN *__restrict__ k_idx,
    const float *__restrict__ weights, int Hi, float idx_scale, float *__restrict__ scores,
    int64_t ld, int max_sk, int nqb) {
  extern __shared__ float ws_lds[];  // [Hi][IDX_BT]
  const int seg = blockIdx.x / nqb;
  const int qb = blockIdx.x - seg * nqb;
  const int q_start = __ldg(L.cu_q + seg);
  const int q_len = __ldg(L.cu_q + seg + 1) - q_start;
  const int t0 = qb * IDX_BT;
  if (t0 >= q_len) return;
  const int k_base = __ldg(L.cu_k + seg);
  const int s_k = __ldg(L.cu_k + seg + 1) - k_base;
  const int off = seg_offset(L, seg, q_len, s_k);
  const int j0 = blockIdx.y * IDX_BN;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int t_last = min(t0 + IDX_BT, q_len) - 1;
  const int nv_last = n_valid_of(t_last, off, L.ratio, s_k);

  // rows of this lane's output: tokens t0 + 16w + 4g + i, keys j0 + 16n + r16
  int nv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) nv[i] = n_valid_of(t0 + 16 * w + 4 * g + i, off, L.ratio, s_k);

  if (j0 >= nv_last) {  // the whole tile is above the causal limit
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 16 * w + 4 * g + i;
      if (t >= q_len) continue;
      float *dst = scores + (int64_t)(q_start + t) * ld;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int j = j0 + 16 * n + r16;
        if (j < max_sk) dst[j] = -__builtin_inff();
      }
    }
    return;
  }

  // fp32(w * s_idx) for the tile's tokens, stored head-major so a lane reads its 4
  // consecutive tokens with one 16-byte LDS load
  for (int e = tid; e < Hi * IDX_BT; e += IDX_THREADS) {
    const int tt = e / Hi, h = e - tt * Hi;
    const int t = t0 + tt;
    ws_lds[h * IDX_BT + tt] = t < q_len ? weights[(int64_t)(q_start + t) * Hi + h] * idx_scale : 0.f;
  }

  // key fragments: 4 N-tiles of 16 keys, kept for the whole head loop
  Frag<IN, DI> kf[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int j = j0 + 16 * n + r16;
    const bool ok = j < s_k;
    kf[n].load(k_idx + (int64_t)(ok ? k_base + j : 0) * DI, g, ok);
  }
  __syncthreads();

  const int tq = t0 + 16 * w + r16;  // A-operand row of this lane
  const bool qok = tq < q_len;
  const IN *qrow = q_idx + ((int64_t)(q_start + (qok ? tq : 0)) * Hi) * DI;

  f32x4 acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  Frag<IN, DI> qa, qn;
  qa.load(qrow, g, qok);
  for (int h = 0; h < Hi; ++h) {
    if (h + 1 < Hi) qn.load(qrow + (int64_t)(h + 1) * DI, g, qok);
    const f32x4 wv = *reinterpret_cast<const f32x4 *>(ws_lds + h * IDX_BT + 16 * w + 4 * g);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const f32x4 d = Frag<IN, DI>::dot(qa, kf[n]);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[n][i] = fmaf(wv[i], fmaxf(d[i], 0.f), acc[n][i]);
    }
    qa = qn;
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 16 * w + 4 * g + i;
    if (t >= q_len) continue;
    float *dst = scores + (int64_t)(q_start + t) * ld;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int j = j0 + 16 * n + r16;
      if (j < max_sk) dst[j] = j < nv[i] ? acc[n][i] : -__builtin_inff();
    }
  }
}

template <typename IN, int DI>
static hipError_t launch_t(const LaunchLayout &LL, const void *q_idx, const void *k_idx,
                           const float *weights, int Hi, float idx_scale, float *scores,
                           int64_t ld, hipStream_t st) {
  const int nqb = (LL.max_seqlen_q + IDX_BT - 1) / IDX_BT;
  const int nkb = (LL.max_seqlen_k + IDX_BN - 1) / IDX_BN;
  dim3 grid((unsigned)(LL.num_seqs * nqb), (unsigned)nkb);
  const size_t lds = (size_t)Hi * IDX_BT * sizeof(float);
  hipLaunchKernelGGL((indexer_score_kernel<IN, DI>), grid, dim3(IDX_THREADS), lds, st, LL.dev,
                     static_cast<const IN *>(q_idx), static_cast<const IN *>(k_idx), weights, Hi,
                     idx_scale, scores, ld, LL.max_seqlen_k, nqb);
  return hipGetLastError();
}

hipError_t launch_indexer_score(const LaunchLayout &LL, const void *q_idx, const void *k_idx,
                                const float *weights, bool bf16, int Hi, int Di, float idx_scale,
                                float *scores, int64_t ld, hipStream_t st) {
  if (bf16) {
    switch (Di) {
      case 32: return launch_t<uint16_t, 32>(LL, q_idx, k_idx, weights, Hi, idx_scale, scores, ld, st);
      case 64: return launch_t<uint16_t, 64>(LL, q_idx, k_idx, weights, Hi, idx_scale, scores, ld, st);
      case 128: return launch_t<uint16_t, 128>(LL, q_idx, k_idx, weights, Hi, idx_scale, scores, ld, st);
    }
  } else {
    switch (Di) {
      case 32: return launch_t<float, 32>(LL, q_idx, k_idx, weights, Hi, idx_scale, scores, ld, st);
      case 64: return launch_t<float, 64>(LL, q_idx, k_idx, weights, Hi, idx_scale, scores, ld, st);
      case 128: return launch_t<float, 128>(LL, q_idx, k_idx, weights, Hi, idx_scale, scores, ld, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace csa

namespace csa {
bool indexer_supported(bool, int Hi, int Di) {
  return Hi >= 1 && Hi <= 128 && (Di == 32 || Di == 64 || Di == 128);
}
}  // namespace csa
