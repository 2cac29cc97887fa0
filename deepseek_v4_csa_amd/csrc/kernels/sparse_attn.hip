// Sliding-window + top-k compressed attention with a per-head sink (gfx950 MFMA).
//
// Per query row t and head h (page "[Bug] DSV4 unfused CSA indexer loss uses a
// compressed-only teacher ...": "Paper reference" Z_h equation; csa.py sparse-attention
// excerpt: window ids then top-k ids, sink as fp32, softmax_scale on q.k):
//   Z_h = exp(sink_h) + sum_{window} exp(w_ht') + sum_{valid ids} exp(c_hj)
//   out = (sum_window e^w kv[t'] + sum_ids e^c ckv[id]) / Z_h
//   lse = log Z_h,  lse_nc = log(exp(sink_h) + sum_window e^w)   (u_h of the proposal
//   comment in that page's discussion thread)
//   cmass[t, j] = sum_h exp(c_hj - lse_h)       (head-summed compressed probabilities)
//
// One workgroup per query row; wave w owns heads [16w, 16w+16).  All waves share the
// gathered KV rows, staged 32 at a time in LDS (one KV head serves every attention
// head, so a row is fetched once per query and reused by all H heads).  Two passes over
// the rows: pass 1 computes the exact per-head max and sum (so lse is final before any
// probability is formed), pass 2 recomputes the logits, forms P = exp(s - lse) once,
// accumulates O^T += V^T P^T on MFMA and sums P over heads into cmass.  With lse known
// up front nothing is rescaled and the teacher's per-head denominators are exact.
//
// MFMA layouts (16x16x32 bf16; 16x16x4 fp32 for fp32 inputs):
//   S^T = K Q^T : A = K rows (row = l%16), B = Q^T (head = l%16); C lane l holds
//                 S^T[row 4g+i][head l%16]  -> every per-head statistic is lane-local
//                 up to a reduction over the 4 lane groups g = l/16.
//   O^T += V^T P^T : A = V^T read from LDS column-wise, B = P^T built from two S^T
//                 tiles: MFMA k index 8g+e <-> chunk row (e<4 ? 4g+e : 16+4g+e-4).
#include "common.h"
#include "../launch.h"

namespace csa {

constexpr int ATT_CHUNK = 32;  // KV rows staged per step

template <typename IN> struct Elt;
template <> struct Elt<uint16_t> { static constexpr int bytes = 2; };
template <> struct Elt<float> { static constexpr int bytes = 4; };

template <typename IN, int D>
struct AttnCfg {
  static constexpr int EB = Elt<IN>::bytes;
  static constexpr int ROW_BYTES = D * EB;
  static constexpr int RS = ROW_BYTES + 16;  // padded LDS row stride (bytes)
  static constexpr int PIECES = ROW_BYTES / 16;  // 16-byte pieces per row
  // bf16: D/32 K-chunks of 8 per lane (lane group g holds features [g*D/4, (g+1)*D/4));
  // fp32: D/4 K-steps of 1 per lane over the same span.
  static constexpr int NKC = (EB == 2) ? D / 32 : D / 4;
  static constexpr int NDT = D / 16;  // output d-tiles
};

// Q^T fragment of one wave (16 heads): lane holds head l%16, features of its group.
template <typename IN, int D> struct QFrag;
template <int D> struct QFrag<uint16_t, D> {
  u32x4 v[D / 32];
  __device__ __forceinline__ void load(const uint16_t *qrow, int g, bool ok) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(qrow + g * (D / 4));
#pragma unroll
    for (int c = 0; c < D / 32; ++c) v[c] = ok ? p[c] : u32x4{0, 0, 0, 0};
  }
};
template <int D> struct QFrag<float, D> {
  float v[D / 4];
  __device__ __forceinline__ void load(const float *qrow, int g, bool ok) {
    const f32x4 *p = reinterpret_cast<const f32x4 *>(qrow + g * (D / 4));
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const f32x4 x = ok ? p[c] : f32x4{0.f, 0.f, 0.f, 0.f};
      v[4 * c] = x[0]; v[4 * c + 1] = x[1]; v[4 * c + 2] = x[2]; v[4 * c + 3] = x[3];
    }
  }
};

// S^T tile (16 rows of the chunk starting at row0) for this wave's 16 heads
template <int D>
__device__ __forceinline__ f32x4 s_tile(const char *lds, int row0, const QFrag<uint16_t, D> &q, int lane) {
  const int g = lane >> 4, r = lane & 15;
  const char *base = lds + (row0 + r) * AttnCfg<uint16_t, D>::RS + g * (D / 4) * 2;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const u32x4 a = *reinterpret_cast<const u32x4 *>(base + 16 * c);
    acc = mfma16x16x32(a, q.v[c], acc);
  }
  return acc;
}
template <int D>
__device__ __forceinline__ f32x4 s_tile(const char *lds, int row0, const QFrag<float, D> &q, int lane) {
  const int g = lane >> 4, r = lane & 15;
  const float *base = reinterpret_cast<const float *>(lds + (row0 + r) * AttnCfg<float, D>::RS) + g * (D / 4);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 4; ++c) acc = mfma16x16x4f32(base[c], q.v[c], acc);
  return acc;
}

// O^T += V^T P^T for one 32-row chunk (p0: rows 4g+i, p1: rows 16+4g+i of this lane)
template <int D>
__device__ __forceinline__ void pv_chunk(const char *lds, f32x4 *o, f32x4 p0, f32x4 p1, int lane,
                                         uint16_t) {
  const int g = lane >> 4, c = lane & 15;
  const u32x4 pb = {pack_bf16x2(p0[0], p0[1]), pack_bf16x2(p0[2], p0[3]),
                    pack_bf16x2(p1[0], p1[1]), pack_bf16x2(p1[2], p1[3])};
  constexpr int RS = AttnCfg<uint16_t, D>::RS;
  const char *r0 = lds + (4 * g) * RS;
  const char *r1 = lds + (16 + 4 * g) * RS;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const int cb = (dt * 16 + c) * 2;
    const uint32_t v0 = *reinterpret_cast<const uint16_t *>(r0 + 0 * RS + cb);
    const uint32_t v1 = *reinterpret_cast<const uint16_t *>(r0 + 1 * RS + cb);
    const uint32_t v2 = *reinterpret_cast<const uint16_t *>(r0 + 2 * RS + cb);
    const uint32_t v3 = *reinterpret_cast<const uint16_t *>(r0 + 3 * RS + cb);
    const uint32_t v4 = *reinterpret_cast<const uint16_t *>(r1 + 0 * RS + cb);
    const uint32_t v5 = *reinterpret_cast<const uint16_t *>(r1 + 1 * RS + cb);
    const uint32_t v6 = *reinterpret_cast<const uint16_t *>(r1 + 2 * RS + cb);
    const uint32_t v7 = *reinterpret_cast<const uint16_t *>(r1 + 3 * RS + cb);
    const u32x4 a = {v0 | (v1 << 16), v2 | (v3 << 16), v4 | (v5 << 16), v6 | (v7 << 16)};
    o[dt] = mfma16x16x32(a, pb, o[dt]);
  }
}
template <int D>
__device__ __forceinline__ void pv_chunk(const char *lds, f32x4 *o, f32x4 p0, f32x4 p1, int lane,
                                         float) {
  const int g = lane >> 4, c = lane & 15;
  constexpr int RS = AttnCfg<float, D>::RS;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v0 = *reinterpret_cast<const float *>(lds + (4 * g + i) * RS + (dt * 16 + c) * 4);
      o[dt] = mfma16x16x4f32(v0, p0[i], o[dt]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v1 = *reinterpret_cast<const float *>(lds + (16 + 4 * g + i) * RS + (dt * 16 + c) * 4);
      o[dt] = mfma16x16x4f32(v1, p1[i], o[dt]);
    }
  }
}

template <typename IN, int D, int HG>
__global__ __launch_bounds__(64 * HG) void sparse_attn_kernel(
    LayoutDev L, const IN *__restrict__ q, const IN *__restrict__ kv, const IN *__restrict__ ckv,
    const float *__restrict__ sink, const int32_t *__restrict__ ids, int k_eff, int window, int H,
    float scale_log2, IN *__restrict__ out, float *__restrict__ lse, float *__restrict__ lse_nc,
    float *__restrict__ cmass) {
  using C = AttnCfg<IN, D>;
  constexpr int NT = 64 * HG;
  __shared__ __attribute__((aligned(16))) char rows[ATT_CHUNK * C::RS];
  __shared__ int row_ok[ATT_CHUNK];
  __shared__ float cm_part[HG][ATT_CHUNK];

  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, hl = lane & 15;
  const int h = 16 * w + hl;
  const bool h_ok = h < H;
  const RowGeo geo = row_geo(L, t);
  const int w_lo = max(geo.q_start, t - window + 1);
  const int nw = window > 0 ? t - w_lo + 1 : 0;
  const int32_t *idrow = ids + (int64_t)t * k_eff;
  const int nwc = (nw + ATT_CHUNK - 1) / ATT_CHUNK;
  const int ncc = (k_eff + ATT_CHUNK - 1) / ATT_CHUNK;

  QFrag<IN, D> qf;
  qf.load(q + ((int64_t)t * H + (h_ok ? h : 0)) * D, g, h_ok);

  // stage chunk `ci` (window chunks first, then compressed) into LDS
  auto stage = [&](int ci) {
    const bool win = ci < nwc;
    const int s0 = (win ? ci : ci - nwc) * ATT_CHUNK;
    for (int p = tid; p < ATT_CHUNK * C::PIECES; p += NT) {
      const int r = p / C::PIECES, pc = p - r * C::PIECES;
      const int slot = s0 + r;
      const IN *src = nullptr;
      if (win) {
        if (slot < nw) src = kv + (int64_t)(w_lo + slot) * D;
      } else if (slot < k_eff) {
        const int id = idrow[slot];
        if (id >= 0) src = ckv + (int64_t)id * D;
      }
      u32x4 val = {0, 0, 0, 0};
      if (src) val = reinterpret_cast<const u32x4 *>(src)[pc];
      *reinterpret_cast<u32x4 *>(rows + r * C::RS + pc * 16) = val;
      if (pc == 0) row_ok[r] = src != nullptr;
    }
  };

  // ---------------------------------------------------------------- pass 1: max / sum
  const float a2 = sink[h_ok ? h : 0] * LOG2E;
  float m = (g == 0 && h_ok) ? a2 : -__builtin_inff();
  float l = (g == 0 && h_ok && a2 > -__builtin_inff()) ? 1.f : 0.f;
  float m_nc = m, l_nc = l;
  const int nch = nwc + ncc;
  for (int ci = 0; ci < nch; ++ci) {
    if (ci == nwc) { m_nc = m; l_nc = l; }
    stage(ci);
    __syncthreads();
    float s[8];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const f32x4 st = s_tile<D>(rows, 16 * tau, qf, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = row_ok[16 * tau + 4 * g + i] && h_ok;
        s[4 * tau + i] = ok ? st[i] * scale_log2 : -__builtin_inff();
      }
    }
    float cm = s[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, s[e]);
    const float mn = fmaxf(m, cm);
    if (mn > -__builtin_inff()) {
      float acc = l * exp2f(m - mn);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += exp2f(s[e] - mn);
      l = acc;
      m = mn;
    }
    __syncthreads();
  }
  if (ncc == 0) { m_nc = m; l_nc = l; }
  // combine the 4 lane groups of each head
  const float M = across_groups_max(m);
  const float Lsum = across_groups_sum(M > -__builtin_inff() ? l * exp2f(m - M) : 0.f);
  const float Mnc = across_groups_max(m_nc);
  const float Lnc = across_groups_sum(Mnc > -__builtin_inff() ? l_nc * exp2f(m_nc - Mnc) : 0.f);
  const float lse2 = Lsum > 0.f ? M + __log2f(Lsum) : -__builtin_inff();
  const float lse2_nc = Lnc > 0.f ? Mnc + __log2f(Lnc) : -__builtin_inff();

  // ---------------------------------------------------------------- pass 2: P, O, cmass
  f32x4 o[C::NDT];
#pragma unroll
  for (int i = 0; i < C::NDT; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool any = lse2 > -__builtin_inff();
  for (int ci = 0; ci < nch; ++ci) {
    stage(ci);
    __syncthreads();
    f32x4 p[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const f32x4 st = s_tile<D>(rows, 16 * tau, qf, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = row_ok[16 * tau + 4 * g + i] && h_ok && any;
        p[tau][i] = ok ? exp2f(st[i] * scale_log2 - lse2) : 0.f;
      }
    }
    pv_chunk<D>(rows, o, p[0], p[1], lane, IN{});
    if (cmass && ci >= nwc) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sh = group16_sum(p[tau][i]);
          if (hl == 0) cm_part[w][16 * tau + 4 * g + i] = sh;
        }
      __syncthreads();
      if (tid < ATT_CHUNK) {
        const int slot = (ci - nwc) * ATT_CHUNK + tid;
        if (slot < k_eff) {
          float sum = 0.f;
#pragma unroll
          for (int ww = 0; ww < HG; ++ww) sum += cm_part[ww][tid];
          cmass[(int64_t)t * k_eff + slot] = sum;
        }
      }
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- outputs
  if (h_ok) {
    IN *orow = out + ((int64_t)t * H + h) * D;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
      const int d0 = dt * 16 + 4 * g;
      if constexpr (C::EB == 2) {
        uint2 pk = {pack_bf16x2(o[dt][0], o[dt][1]), pack_bf16x2(o[dt][2], o[dt][3])};
        *reinterpret_cast<uint2 *>(orow + d0) = pk;
      } else {
        *reinterpret_cast<f32x4 *>(orow + d0) = o[dt];
      }
    }
    if (g == 0) {
      lse[(int64_t)t * H + h] = lse2 * LN2;
      lse_nc[(int64_t)t * H + h] = lse2_nc * LN2;
    }
  }
}

template <typename IN, int D>
static hipError_t launch_d(const LaunchLayout &LL, const void *q, const void *kv, const void *ckv,
                           const float *sink, const int32_t *ids, int k_eff, int window, int H,
                           float scale, void *out, float *lse, float *lse_nc, float *cmass,
                           hipStream_t st) {
  const float sl2 = scale * LOG2E;
  dim3 grid((unsigned)LL.total_q);
  const int hg = (H + 15) / 16;
#define CSA_ATT_CASE(G)                                                                           \
  if (hg <= G) {                                                                                  \
    hipLaunchKernelGGL((sparse_attn_kernel<IN, D, G>), grid, dim3(64 * G), 0, st, LL.dev,         \
                       static_cast<const IN *>(q), static_cast<const IN *>(kv),                   \
                       static_cast<const IN *>(ckv), sink, ids, k_eff, window, H, sl2,            \
                       static_cast<IN *>(out), lse, lse_nc, cmass);                               \
    return hipGetLastError();                                                                     \
  }
  CSA_ATT_CASE(1)
  CSA_ATT_CASE(2)
  CSA_ATT_CASE(4)
  CSA_ATT_CASE(8)
#undef CSA_ATT_CASE
  return hipErrorInvalidValue;
}

bool attn_supported(bool bf16, int H, int D, int k_eff) {
  if (H < 1 || H > 128 || k_eff < 0 || k_eff > 4096) return false;
  if (bf16) return D == 64 || D == 128 || D == 192 || D == 256 || D == 512;
  return D == 64 || D == 128;
}

hipError_t launch_sparse_attn(const LaunchLayout &LL, const void *q, const void *kv,
                              const void *ckv, const float *sink, const int32_t *ids, int k_eff,
                              int window, bool bf16, int H, int D, float scale, void *out,
                              float *lse, float *lse_nc, float *cmass, hipStream_t st) {
  if (LL.total_q == 0) return hipSuccess;
#define CSA_ARGS LL, q, kv, ckv, sink, ids, k_eff, window, H, scale, out, lse, lse_nc, cmass, st
  if (bf16) {
    switch (D) {
      case 64: return launch_d<uint16_t, 64>(CSA_ARGS);
      case 128: return launch_d<uint16_t, 128>(CSA_ARGS);
      case 192: return launch_d<uint16_t, 192>(CSA_ARGS);
      case 256: return launch_d<uint16_t, 256>(CSA_ARGS);
      case 512: return launch_d<uint16_t, 512>(CSA_ARGS);
    }
  } else {
    switch (D) {
      case 64: return launch_d<float, 64>(CSA_ARGS);
      case 128: return launch_d<float, 128>(CSA_ARGS);
    }
  }
#undef CSA_ARGS
  return hipErrorInvalidValue;
}

}  // namespace csa
