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
#include <algorithm>
#include <utility>

#include "common.h"
#include "sparse_kl.h"
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
  constexpr int PPT = (ATT_CHUNK * C::PIECES + NT - 1) / NT;   // 16-byte pieces per thread
  // dynamic LDS: two row buffers, then the query's ids
  extern __shared__ __attribute__((aligned(16))) char att_dyn[];
  int *ids_lds = reinterpret_cast<int *>(att_dyn + 2 * ATT_CHUNK * C::RS);
  __shared__ int row_ok[2][ATT_CHUNK];
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
  for (int i = tid; i < k_eff; i += NT) ids_lds[i] = idrow[i];

  QFrag<IN, D> qf;
  qf.load(q + ((int64_t)t * H + (h_ok ? h : 0)) * D, g, h_ok);

  // chunk `ci` (window chunks first, then compressed) is staged through registers into LDS
  // buffer ci & 1 while chunk ci - 1 is consumed from the other one, so each chunk costs one
  // barrier; the loads are issued after the compute (issuing them before it costs occupancy
  // for no gain on these shapes)
  u32x4 stg[PPT];
  bool stg_ok[PPT];
  auto load_regs = [&](int ci) __attribute__((always_inline)) {
    const bool win = ci < nwc;
    const int s0 = (win ? ci : ci - nwc) * ATT_CHUNK;
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = tid + k * NT;
      const int r = p / C::PIECES, pc = p - r * C::PIECES;
      const int slot = s0 + r;
      const IN *src = nullptr;
      if (p < ATT_CHUNK * C::PIECES) {
        if (win) {
          if (slot < nw) src = kv + (int64_t)(w_lo + slot) * D;
        } else if (slot < k_eff) {
          const int id = ids_lds[slot];
          if (id >= 0) src = ckv + (int64_t)id * D;
        }
      }
      stg[k] = src ? reinterpret_cast<const u32x4 *>(src)[pc] : u32x4{0, 0, 0, 0};
      stg_ok[k] = src != nullptr;
    }
  };
  auto store_regs = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = tid + k * NT;
      if (p < ATT_CHUNK * C::PIECES) {
        const int r = p / C::PIECES, pc = p - r * C::PIECES;
        *reinterpret_cast<u32x4 *>((att_dyn + buf * (ATT_CHUNK * C::RS)) + r * C::RS + pc * 16) = stg[k];
        if (pc == 0) row_ok[buf][r] = stg_ok[k];
      }
    }
  };
  __syncthreads();   // ids in LDS

  // ---------------------------------------------------------------- pass 1: max / sum
  const float a2 = sink[h_ok ? h : 0] * LOG2E;
  float m = (g == 0 && h_ok) ? a2 : -__builtin_inff();
  float l = (g == 0 && h_ok && a2 > -__builtin_inff()) ? 1.f : 0.f;
  float m_nc = m, l_nc = l;
  const int nch = nwc + ncc;
  if (nch > 0) {
    load_regs(0);
    store_regs(0);
  }
  for (int ci = 0; ci < nch; ++ci) {
    if (ci == nwc) { m_nc = m; l_nc = l; }
    __syncthreads();   // chunk ci in row buffer ci & 1; that buffer's previous readers are done
    const char *rows = att_dyn + (ci & 1) * (ATT_CHUNK * C::RS);
    const int *rok = row_ok[ci & 1];
    float s[8];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const f32x4 st = s_tile<D>(rows, 16 * tau, qf, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = rok[16 * tau + 4 * g + i] && h_ok;
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
    if (ci + 1 < nch) {
      load_regs(ci + 1);
      store_regs((ci + 1) & 1);
    }
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
  __syncthreads();   // pass 1 is done with both buffers
  if (nch > 0) {
    load_regs(0);
    store_regs(0);
  }
  for (int ci = 0; ci < nch; ++ci) {
    __syncthreads();   // chunk ci in row buffer ci & 1; that buffer's previous readers are done
    const char *rows = att_dyn + (ci & 1) * (ATT_CHUNK * C::RS);
    const int *rok = row_ok[ci & 1];
    f32x4 p[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const f32x4 st = s_tile<D>(rows, 16 * tau, qf, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = rok[16 * tau + 4 * g + i] && h_ok && any;
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
    if (ci + 1 < nch) {
      load_regs(ci + 1);
      store_regs((ci + 1) & 1);
    }
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

// ============================================================================
// Workgroup variant (bf16; any H up to 16*HG; D = 64, 128, 192, 256 or 512; k_eff <= 4096).
//
// One workgroup per query row, wave w owning NG groups of 16 heads, in two passes.  Pass 1
// runs over every chunk: the per-head sum under a running max shared by a head's lane
// groups (raised lazily, by at least 2^8), and for the window chunks P V straight into O,
// rescaled with the max.  Pass 2 runs over the compressed chunks only, with lse final:
// their probabilities P = exp(s - lse) are formed once, for O and for cmass.  So a window
// row's logits and exponentials are computed once, a compressed row's twice.  The gathered rows are staged 32 at a time into two LDS tiles by
// direct buffer->LDS loads: the waves split the D/16 load instructions of a tile between
// them, and the next tile's loads are issued right after the step's barrier, so they
// stream in while the current tile is consumed.  Rows are stored with the XOR swizzle
// of row_swz<D> (position = piece ^ swz(R)), so both operand reads are conflict-free:
//   S^T = K Q^T     K operand: 16-byte LDS reads, piece 4c+g of row r16 for K-chunk c
//   O^T += V^T P^T  V^T operand: transposing LDS reads of 4 rows x 16 features
// Per-key sums over heads (cmass) are reduced across waves through LDS one step later,
// behind the next barrier.
// ============================================================================
// (at least three waves per SIMD where the registers of a shape allow it)
template <int D, int HG, int NG>
__global__ __launch_bounds__(64 * HG, (D == 192 || D == 512) ? 2 : 3) void sparse_attn_wg_kernel(
    LayoutDev L, const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const uint16_t *__restrict__ ckv, const float *__restrict__ sink,
    const int32_t *__restrict__ ids, int k_eff, int window, int H, int total_q, int total_k,
    float sl2, uint16_t *__restrict__ out, float *__restrict__ lse, float *__restrict__ lse_nc,
    float *__restrict__ cmass) {
  constexpr int NC = D / 32;          // MFMA K-chunks per row
  constexpr int ROWB = D * 2;         // bytes per KV row
  constexpr int PIECES = D / 8;       // 16-byte pieces per row
  constexpr int NI = PIECES / 2;      // load instructions per 32-row tile (64 pieces each)
  constexpr int NIW = (NI + HG - 1) / HG;   // of them issued by one wave
  constexpr int TILE = 32 * ROWB;
  constexpr int NT = 64 * HG;
  constexpr int BDT = D >= 512 ? D / 128 : D / 32;   // d-tiles per batch of V^T reads
  constexpr int HPW = 16 * NG;        // heads per wave
  constexpr float NINF = -__builtin_inff();
  extern __shared__ __attribute__((aligned(16))) char wg_dyn[];   // 2 tiles, then the ids
  int *ids_l = reinterpret_cast<int *>(wg_dyn + 2 * TILE);
  __shared__ float cm_part[2][HG][32];

  const int t = blockIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  // head group gi of the wave: heads HPW*w + 16*gi + (0..15), lane r16 holding one of them
  int hh[NG];
  bool h_ok[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    hh[gi] = HPW * w + 16 * gi + r16;
    h_ok[gi] = hh[gi] < H;
  }
  const RowGeo geo = row_geo(L, t);
  const int w_lo = max(geo.q_start, t - window + 1);
  const int nw = window > 0 ? t - w_lo + 1 : 0;
  const int nwc = (nw + 31) >> 5, ncc_all = (k_eff + 31) >> 5;
  // the row's ids, padded with -1 to whole 32-row chunks: unconditional loads through a
  // buffer resource of exactly k_eff ids, four per thread in flight at once (a load under a
  // per-element branch is waited for before the next is issued).  The last slot holding
  // an id (jlast) bounds the compressed chunks: those after it have no row, contribute
  // nothing, and are skipped (top-k rows with fewer causal keys than k_eff end in -1s).
  __shared__ int jlast;
  if (tid == 0) jlast = -1;
  __syncthreads();
  {
    const __amdgpu_buffer_rsrc_t rid = make_rsrc(ids + (int64_t)t * k_eff, (uint32_t)k_eff * 4);
    int jl = -1;
    for (int i0 = tid; i0 < ncc_all * 32; i0 += 4 * NT) {
      int x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = __builtin_amdgcn_raw_buffer_load_b32(rid, (i0 + u * NT) * 4, 0, 0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = i0 + u * NT;
        const int id = j < k_eff ? x[u] : -1;
        if (j < ncc_all * 32) ids_l[j] = id;
        if (id >= 0) jl = j;   // j grows with u and i0
      }
    }
    if (jl >= 0) atomicMax(&jlast, jl);
  }
  // Q^T operands, MFMA K index <-> feature: piece c of lane group g holds features [(4c+g)*8, +8)
  // (a lane of a head past H loads head 0's row: its logits are masked, the values never used)
  u32x4 qf[NG][NC];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(q + ((int64_t)t * H + (h_ok[gi] ? hh[gi] : 0)) * D) + g;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[gi][c] = p[4 * c];
  }
  // window rows past the query lie past the end of rkv: they read zeros
  const __amdgpu_buffer_rsrc_t rkv = make_rsrc(kv, (uint32_t)(t + 1) * ROWB);
  const __amdgpu_buffer_rsrc_t rck = make_rsrc(ckv, (uint32_t)total_k * ROWB);
  // This wave's loads: instruction i = w + k*HG writes tile bytes [1024 i, 1024 i + 1024),
  // lane l the 16 bytes of piece slot pc of row R (64 i + l = R * PIECES + pc), which hold
  // the row's logical piece pc ^ swz(R).  An id of -1 gives an offset of 2^32 - ROWB +
  // (< ROWB), past the end of rck: zeros.
  // When a load covers whole rows (RPI = 512 / D of them), R = i RPI + l / PIECES and the
  // swizzle splits into a per-lane and a per-load term, so the lane's part is one value
  // re-derived at each use from an opaque copy of the lane index; rows of 384 bytes keep,
  // per load, the lane's row and piece offset packed in one register (R << 16 | offset).
  constexpr bool SPLIT = 512 % D == 0;
  constexpr int NPK = SPLIT ? 1 : NIW;
  uint32_t lpk[NPK];
#pragma unroll
  for (int k = 0; k < NPK; ++k) {
    const int P = 64 * (w + k * HG) + lane, R = P / PIECES;
    lpk[k] = ((uint32_t)R << 16) | (uint32_t)(16 * ((P - R * PIECES) ^ row_swz<D>(R)));
  }
  if constexpr (SPLIT) static_assert(swz_splits<D>(), "row_swz(i RPI + g) = row_swz(g) ^ row_swz(i RPI)");
  // K operand: row r16 (+16), piece (4c + g) ^ swz = 4 (c ^ (swz >> 2)) + (g ^ (swz & 3))
  const int ksw = row_swz<D>(r16);
  const int kbase = r16 * ROWB + 16 * (g ^ (ksw & 3)), kx = ksw >> 2;
  // V^T operand: rows rho (+16), piece (2dt + hb) ^ swz = 2 (dt ^ (swz >> 1)) + (hb ^ (swz & 1))
  const int rho = 4 * g + (r16 >> 2);
  const int vsw = row_swz<D>(rho);
  const int vbase = rho * ROWB + 16 * (((r16 & 3) >> 1) ^ (vsw & 1)) + 8 * (r16 & 1), vx = vsw >> 1;

  // rows of chunk ci (window chunks first, then compressed) into tile `buf`
  auto issue = [&](int ci, char *buf) {
    if constexpr (SPLIT) {
      constexpr int RPI = SPLIT ? 512 / D : 1;
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int gl = ln / PIECES;
      const uint32_t d0 = 16 * ((ln % PIECES) ^ row_swz<D>(gl));   // < ROWB
#pragma unroll
      for (int k = 0; k < NIW; ++k) {
        const int i = w + k * HG;
        if (NI % HG == 0 || i < NI) {
          const uint32_t sx = 16 * row_swz<D>(i * RPI);
          if (ci < nwc) {
            dma16(rkv, buf + i * 1024, (uint32_t)(w_lo + 32 * ci + i * RPI + gl) * ROWB + (d0 ^ sx));
          } else {
            const int id = ids_l[32 * (ci - nwc) + i * RPI + gl];
            dma16(rck, buf + i * 1024, (uint32_t)id * ROWB + (d0 ^ sx));
          }
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < NIW; ++k) {
        const int i = w + k * HG;
        if (NI % HG == 0 || i < NI) {
          const uint32_t R = lpk[k] >> 16, off = lpk[k] & 0xffffu;
          if (ci < nwc) {
            dma16(rkv, buf + i * 1024, (uint32_t)(w_lo + 32 * ci) * ROWB + R * ROWB + off);
          } else {
            const int id = ids_l[32 * (ci - nwc) + R];
            dma16(rck, buf + i * 1024, (uint32_t)id * ROWB + off);
          }
        }
      }
    }
  };
  // valid rows of chunk ci as bits
  auto row_mask = [&](int ci) -> uint32_t {
    if (ci < nwc) {
      const int n = nw - 32 * ci;
      return n >= 32 ? 0xffffffffu : (1u << n) - 1u;
    }
    return (uint32_t)__ballot(ids_l[32 * (ci - nwc) + (lane & 31)] >= 0);
  };
  // S^T for the 32 rows of a tile: this lane's 8 products q.k per head group (rows 4g+i
  // and 16+4g+i, head 16 gi + r16 of the wave), unscaled, -inf where masked.  Each K
  // operand read from LDS feeds the MFMAs of every head group.  The masking is skipped
  // when every row of the tile is valid and every head of the wave exists.
  const bool wave_full = HPW * (w + 1) <= H;
  auto logits = [&](const char *base, uint32_t bm, float (&sv)[NG][8]) {
    int kxs = kx;
    asm volatile("" : "+v"(kxs));
    f32x4 acc0[NG], acc1[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) acc0[gi] = acc1[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const char *kp = base + kbase + 64 * (c ^ kxs);
      const u32x4 k0 = *reinterpret_cast<const u32x4 *>(kp);
      const u32x4 k1 = *reinterpret_cast<const u32x4 *>(kp + 16 * ROWB);
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        acc0[gi] = mfma16x16x32(k0, qf[gi][c], acc0[gi]);
        acc1[gi] = mfma16x16x32(k1, qf[gi][c], acc1[gi]);
      }
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int i = 0; i < 4; ++i) { sv[gi][i] = acc0[gi][i]; sv[gi][4 + i] = acc1[gi][i]; }
    if (!(wave_full && bm == 0xffffffffu)) {   // masked in place
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const uint32_t m0 = h_ok[gi] ? (bm >> (4 * g)) : 0u, m1 = h_ok[gi] ? (bm >> (16 + 4 * g)) : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[gi][i] = ((m0 >> i) & 1) ? sv[gi][i] : NINF;
          sv[gi][4 + i] = ((m1 >> i) & 1) ? sv[gi][4 + i] : NINF;
        }
      }
    }
  };

  __syncthreads();   // ids and jlast in LDS
  const int ncc = (jlast + 32) >> 5, nch = nwc + ncc;
  if (cmass != nullptr)   // the skipped chunks' slots hold no id: mass 0
    for (int j = 32 * ncc + tid; j < k_eff; j += NT) cmass[(int64_t)t * k_eff + j] = 0.f;
  // Steps: pass 1 over every chunk, then pass 2 over the compressed chunks; step n reads
  // tile n & 1 and, right after its barrier (its own loads have landed, so after the
  // barrier every wave's have, and every wave has finished reading tile n - 1), requests
  // the rows of step n + 1 into the other tile, where they stream in while tile n is
  // consumed.  (A third tile, requests two steps ahead, measured slower on these shapes.)
  const int ns = nch + ncc;
  auto chunk_of = [&](int n) { return n < nch ? n : nwc + (n - nch); };
  auto tile = [&](int n) { return wg_dyn + (n & 1) * TILE; };
  auto top = [&](int n) {
    wait_vmcnt<0>();
    __syncthreads();
    if (n + 1 < ns) issue(chunk_of(n + 1), tile(n + 1));
  };
  if (ns > 0) issue(0, tile(0));

  f32x4 o[NG][D / 16];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi)
#pragma unroll
    for (int i = 0; i < D / 16; ++i) o[gi][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // O^T += V^T P^T for the tile at `base`: V^T operands in batches of BDT d-tiles (fewer
  // registers in flight), each feeding the MFMAs of every head group
  auto pv = [&](const char *base, const float (&p)[NG][8]) __attribute__((always_inline)) {
    u32x4 pb[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
      pb[gi] = u32x4{pack2_bf16(p[gi][0], p[gi][1]), pack2_bf16(p[gi][2], p[gi][3]),
                     pack2_bf16(p[gi][4], p[gi][5]), pack2_bf16(p[gi][6], p[gi][7])};
    int vxs = vx;
    asm volatile("" : "+v"(vxs));
#pragma unroll
    for (int hf = 0; hf < D / 16 / BDT; ++hf) {
      uint2 xv[2 * BDT];
      uint32_t va[BDT];
#pragma unroll
      for (int k = 0; k < BDT; ++k) va[k] = lds_addr_of(base + vbase + 32 * ((hf * BDT + k) ^ vxs));
      lds_read_tr16_pairs<16 * ROWB>(xv, va);
#pragma unroll
      for (int k = 0; k < BDT; ++k) {
        const int dt = hf * BDT + k;
        const u32x4 a = {xv[2 * k].x, xv[2 * k].y, xv[2 * k + 1].x, xv[2 * k + 1].y};
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) o[gi][dt] = mfma16x16x32(a, pb[gi], o[gi][dt]);
      }
    }
  };

  // ------------------------------------------------- pass 1: sums, and P V of the window
  // One running max per head, shared by its 4 lane groups and raised only when a logit
  // exceeds it by 2^8 (then the wave agrees on the new per-head max and rescales l and O),
  // so the window's probabilities exp2(sl2 s - m) <= 2^8 go straight into O.
  constexpr float RESCALE = 8.f;
  float m[NG], l[NG], m_nc[NG], l_nc[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const float a2 = h_ok[gi] ? sink[hh[gi]] * LOG2E : NINF;
    m[gi] = a2;
    l[gi] = (g == 0 && a2 > NINF) ? 1.f : 0.f;   // the sink counted once per head
    m_nc[gi] = m[gi];
    l_nc[gi] = l[gi];
  }
  for (int ci = 0; ci < nch; ++ci) {
    const int n = ci;
    top(n);
    if (ci == nwc) {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) { m_nc[gi] = m[gi]; l_nc[gi] = l[gi]; }
    }
    const char *base = tile(n);
    float sv[NG][8];
    logits(base, row_mask(ci), sv);
    float cmx[NG];
    bool up = false;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      cmx[gi] = sv[gi][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) cmx[gi] = fmaxf(cmx[gi], sv[gi][e]);
      up = up || cmx[gi] * sl2 > m[gi] + RESCALE;   // log2 units (sl2 > 0 keeps the order)
    }
    if (__builtin_expect(__ballot(up) != 0, 0)) {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const float cand = across_groups_max(cmx[gi]) * sl2;
        const float mn = cand > m[gi] + RESCALE ? cand : m[gi];
        const float alpha = mn == m[gi] ? 1.f : fast_exp2(m[gi] - mn);
        l[gi] *= alpha;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) o[gi][i] *= alpha;
        m[gi] = mn;
      }
    }
    float p[NG][8];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const float nms = m[gi] == NINF ? 0.f : -m[gi];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[gi][e] = fast_exp2(fmaf(sv[gi][e], sl2, nms));
        l[gi] += p[gi][e];
      }
    }
    if (ci < nwc) pv(base, p);
  }
  // lse, lse_nc; the window part of O normalised, so pass 2 adds normalised terms to it
  float lse2[NG], lse2_nc[NG], nl[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    if (ncc == 0) { m_nc[gi] = m[gi]; l_nc[gi] = l[gi]; }
    const float Ls = across_groups_sum(l[gi]);
    const float Lnc = across_groups_sum(l_nc[gi]);
    lse2[gi] = Ls > 0.f ? m[gi] + __log2f(Ls) : NINF;
    lse2_nc[gi] = Lnc > 0.f ? m_nc[gi] + __log2f(Lnc) : NINF;
    nl[gi] = lse2[gi] > NINF ? -lse2[gi] : NINF;   // exp2(-inf) = 0: no probability at all
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) o[gi][i] *= inv;
  }

  // ------------------------------------------- pass 2: compressed chunks, P, O and cmass
  float *crow = cmass ? cmass + (int64_t)t * k_eff : nullptr;
  // sums over the waves of the compressed chunk staged at the previous step
  auto flush = [&](int cprev, int pbuf) {
    if (crow && cprev >= nwc && tid < 32) {
      const int slot = 32 * (cprev - nwc) + tid;
      if (slot < k_eff) {
        float sum = 0.f;
#pragma unroll
        for (int ww = 0; ww < HG; ++ww) sum += cm_part[pbuf][ww][tid];
        crow[slot] = sum;
      }
    }
  };
  for (int cc = 0; cc < ncc; ++cc) {
    const int ci = nwc + cc, n = nch + cc;
    top(n);
    if (cc > 0) flush(ci - 1, (n - 1) & 1);
    const char *base = tile(n);
    float sv[NG][8];
    logits(base, row_mask(ci), sv);
    float p[NG][8];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int e = 0; e < 8; ++e) p[gi][e] = fast_exp2(fmaf(sv[gi][e], sl2, nl[gi]));
    pv(base, p);
    if (crow) {
      // value e of group g is row 16 (e >> 2) + 4g + (e & 3); lane r16 ends with the head
      // sum of value sum8_index(r16)
      float ps[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ps[e] = p[0][e];
#pragma unroll
        for (int gi = 1; gi < NG; ++gi) ps[e] += p[gi][e];
      }
      const float sh = group16_sum8(ps, r16);
      const int el = sum8_index(r16);
      if ((r16 & 1) == 0) cm_part[n & 1][w][16 * (el >> 2) + 4 * g + (el & 3)] = sh;
    }
  }
  if (ncc > 0) {
    __syncthreads();
    flush(nch - 1, (ns - 1) & 1);
  }

  // ---------------------------------------------------------------- outputs
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    if (h_ok[gi]) {
      uint16_t *orow = out + ((int64_t)t * H + hh[gi]) * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        *reinterpret_cast<uint2 *>(orow + 16 * dt) =
            uint2{pack2_bf16(o[gi][dt][0], o[gi][dt][1]), pack2_bf16(o[gi][dt][2], o[gi][dt][3])};
      if (g == 0) {
        lse[(int64_t)t * H + hh[gi]] = lse2[gi] * LN2;
        lse_nc[(int64_t)t * H + hh[gi]] = lse2_nc[gi] * LN2;
      }
    }
  }
}

// ============================================================================
// Gather-optimised variant (bf16; 16 heads per wave; k_eff <= 32*KC, KC <= 8).
//
// One wave per (query row, group of 16 heads), independent waves (no barriers).
// Row gathers are the cost that matters here: a load instruction whose 64 lanes touch
// 16 different rows (the MFMA register layout) sustains about a third of the rate of
// one whose lanes cover 4 whole rows.  So rows are fetched row-coalesced with direct
// buffer->LDS loads (16 lanes x 16 bytes per 256-byte row, no VGPRs involved) into a
// per-wave double-buffered LDS tile, while the previous tile is consumed:
//   S^T = K Q^T     K operand read from the tile (16-byte LDS reads)
//   O^T += V^T P^T  V^T operand read from the same tile with the transposing LDS read
// The 16-byte pieces of row R are stored XOR-swizzled (position = piece ^ swz(R)) so
// that both read patterns are free of bank conflicts.  An online softmax carries the
// per-head running max (identical in the 4 lane groups of a head, raised only when a
// logit exceeds it by 2^8) and a per-lane partial sum; the compressed logits stay in
// registers so that cmass = sum_h exp(c - lse) is formed once lse is final.
// ============================================================================

template <int D, int KC>
__global__ __launch_bounds__(256) void sparse_attn_dma_kernel(
    LayoutDev L, const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const uint16_t *__restrict__ ckv, const float *__restrict__ sink,
    const int32_t *__restrict__ ids, int k_eff, int window, int H, int total_q, int total_k,
    float sl2, uint16_t *__restrict__ out, float *__restrict__ lse, float *__restrict__ lse_nc,
    float *__restrict__ cmass) {
  constexpr int NC = D / 32;          // MFMA K-chunks per row
  constexpr int ROWB = D * 2;         // bytes per KV row
  constexpr int PIECES = D / 8;       // 16-byte pieces per row
  constexpr int RPI = 64 / PIECES;    // rows per direct-to-LDS load instruction
  constexpr int NI = 32 / RPI;        // load instructions per 32-row step
  constexpr int TILE = 32 * ROWB;     // one 32-row tile
  constexpr int IDS = 32 * KC;        // id slots staged in LDS
  constexpr float NINF = -__builtin_inff();
  constexpr float RESCALE = 8.f;
  static_assert(NI <= 15, "vmcnt");
  __shared__ __attribute__((aligned(16))) char lds_all[4][2 * TILE + IDS * 4];
  // the wave index is uniform: readfirstlane lets every per-query value live in SGPRs
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int hgc = (H + 15) >> 4;            // waves per query (1, 2 or 4)
  const int t = blockIdx.x * (4 / hgc) + w / hgc;
  if (t >= total_q) return;                 // no block-level barrier below
  const int hgrp = w % hgc;
  char *tiles = lds_all[w];
  int *ids_l = reinterpret_cast<int *>(tiles + 2 * TILE);
  const int h = 16 * hgrp + r16;
  const bool h_ok = h < H;
  const bool group_full = 16 * (hgrp + 1) <= H;
  const RowGeo geo = row_geo(L, t);
  const int w_lo = max(geo.q_start, t - window + 1);
  const int nw = window > 0 ? t - w_lo + 1 : 0;
  const int nwc = (nw + 31) >> 5;
  const __amdgpu_buffer_rsrc_t rkv = make_rsrc(kv, (uint32_t)total_q * ROWB);
  const __amdgpu_buffer_rsrc_t rck = make_rsrc(ckv, (uint32_t)total_k * ROWB);
  const int x16 = (lane ^ 16) << 2, x32 = (lane ^ 32) << 2;   // bpermute addresses

  // Masked rows read zeros or keep stale tile contents; the tiles start zeroed so those
  // are always finite (their probabilities are exactly 0).
#pragma unroll
  for (int i = 0; i < 2 * TILE / 1024; ++i) reinterpret_cast<u32x4 *>(tiles)[i * 64 + lane] = u32x4{0, 0, 0, 0};
  // ids in LDS ordered [step][row-in-instruction][instruction]: a lane's ids of one step
  // are contiguous
#pragma unroll
  for (int s0 = 0; s0 < IDS; s0 += 64) {
    const int s = s0 + lane;
    if (s < IDS) {
      const int rs = s & 31;
      ids_l[(s & ~31) + (rs % RPI) * NI + rs / RPI] = s < k_eff ? ids[(int64_t)t * k_eff + s] : -1;
    }
  }
  // MFMA K index <-> feature: piece c of lane group g holds features [(4c+g)*8, +8)
  u32x4 qf[NC];
  {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(q + ((int64_t)t * H + (h_ok ? h : 0)) * D) + g;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = p[4 * c];   // (masked where the head is past H)
  }
  // per-lane LDS offsets (relative to a tile)
  const int gg = lane / PIECES, pp = lane % PIECES;   // load: row-in-instruction, piece position
  int kro[NC];                                         // K operand: row r16, piece 4c+g
#pragma unroll
  for (int c = 0; c < NC; ++c) kro[c] = r16 * ROWB + 16 * ((4 * c + g) ^ row_swz<D>(r16));
  const int rho = 4 * g + (r16 >> 2);                  // V^T operand: rows rho (+16)
  int tro[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    tro[dt] = rho * ROWB + 16 * ((2 * dt + ((r16 & 3) >> 1)) ^ row_swz<D>(rho)) + 8 * (r16 & 1);

  auto dma_window = [&](int c, char *base) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int R = i * RPI + gg, slot = 32 * c + R;
      const uint32_t off = slot < nw ? (uint32_t)(w_lo + slot) * ROWB + 16 * (pp ^ row_swz<D>(R)) : BUF_OOB;
      dma16(rkv, base + i * 1024, off);
    }
  };
  auto dma_comp = [&](int c, char *base) {
    int idr[NI];
    if (c < KC) {
#pragma unroll
      for (int i = 0; i < NI; ++i) idr[i] = ids_l[c * 32 + gg * NI + i];
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) idr[i] = -1;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int R = i * RPI + gg;
      const uint32_t off = idr[i] >= 0 ? (uint32_t)idr[i] * ROWB + 16 * (pp ^ row_swz<D>(R)) : BUF_OOB;
      dma16(rck, base + i * 1024, off);
    }
  };

  const float a2 = h_ok ? sink[h] * LOG2E : NINF;
  float m = a2;                                        // shared by the 4 lane groups of a head
  float l = (g == 0 && a2 > NINF) ? 1.f : 0.f;         // per-lane partial sum
  f32x4 o[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one 32-row step on the tile at `base`; bm = row validity bits; leaves this lane's
  // unscaled masked logits in raw
  auto step = [&](const char *base, uint32_t bm, float(&raw)[8]) {
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const u32x4 k0 = *reinterpret_cast<const u32x4 *>(base + kro[c]);
      const u32x4 k1 = *reinterpret_cast<const u32x4 *>(base + 16 * ROWB + kro[c]);
      acc0 = mfma16x16x32(k0, qf[c], acc0);
      acc1 = mfma16x16x32(k1, qf[c], acc1);
    }
    if (group_full && bm == 0xffffffffu) {
#pragma unroll
      for (int i = 0; i < 4; ++i) { raw[i] = acc0[i]; raw[4 + i] = acc1[i]; }
    } else {
      const uint32_t m0 = h_ok ? (bm >> (4 * g)) : 0u, m1 = h_ok ? (bm >> (16 + 4 * g)) : 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        raw[i] = ((m0 >> i) & 1) ? acc0[i] : NINF;
        raw[4 + i] = ((m1 >> i) & 1) ? acc1[i] : NINF;
      }
    }
    // Common path without cross-lane traffic: each lane tests its logits against the
    // shared reference max; only a logit 2^8 above it makes the wave agree on a new
    // per-head max and rescale.
    float cmx = fmaxf(fmaxf(fmaxf(raw[0], raw[1]), fmaxf(raw[2], raw[3])),
                      fmaxf(fmaxf(raw[4], raw[5]), fmaxf(raw[6], raw[7])));
    if (__builtin_expect(__ballot(cmx * sl2 > m + RESCALE) != 0, 0)) {
      cmx = fmaxf(cmx, bperm(x16, cmx));
      cmx = fmaxf(cmx, bperm(x32, cmx));
      const float cand = cmx * sl2;
      const float mn = cand > m + RESCALE ? cand : m;
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) o[i] *= alpha;
      m = mn;
    }
    const float nms = m == NINF ? 0.f : -m;
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { p[e] = fast_exp2(fmaf(raw[e], sl2, nms)); l += p[e]; }
    const u32x4 pb = {pack2_bf16(p[0], p[1]), pack2_bf16(p[2], p[3]), pack2_bf16(p[4], p[5]),
                      pack2_bf16(p[6], p[7])};
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const uint2 x0 = lds_read_tr16(base + tro[dt]);
      const uint2 x1 = lds_read_tr16(base + 16 * ROWB + tro[dt]);
      const u32x4 a = {x0.x, x0.y, x1.x, x1.y};
      o[dt] = mfma16x16x32(a, pb, o[dt]);
    }
  };
  // row validity of compressed step c: bit R set iff the id of row R is >= 0
  auto comp_mask = [&](int c) -> uint32_t {
    const int R = lane & 31;
    const bool v = ids_l[c * 32 + (R % RPI) * NI + R / RPI] >= 0;
    return (uint32_t)__ballot(v);
  };
  auto win_mask = [&](int c) -> uint32_t {
    const int n = nw - 32 * c;
    return n >= 32 ? 0xffffffffu : (n > 0 ? (1u << n) - 1u : 0u);
  };

  // Pipeline: step n reads tile n&1 while step n+1's rows stream into the other tile.
  // Before a tile is overwritten every earlier LDS read has returned (lgkmcnt 0); before
  // a tile is read its NI loads have landed (vmcnt NI: only the next step's NI loads may
  // still be in flight).  Past the last step the prefetch reads out of range (zeros).
  float raw[8];
  int n = 0;  // global step index
  __builtin_amdgcn_s_waitcnt(0xC07F);   // the zeroing and id stores have executed
  if (nwc > 0) dma_window(0, tiles); else dma_comp(0, tiles);
  for (int c = 0; c < nwc; ++c, ++n) {
    char *cur = tiles + (n & 1) * TILE, *nxt = tiles + ((n + 1) & 1) * TILE;
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    if (c + 1 < nwc) dma_window(c + 1, nxt); else dma_comp(0, nxt);
    wait_vmcnt<NI>();
    step(cur, win_mask(c), raw);
  }
  const float m_nc = m, l_nc = l;

  float sk[KC][8];  // unscaled compressed logits (-inf when masked)
#pragma unroll
  for (int c = 0; c < KC; ++c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sk[c][e] = NINF;
    if (32 * c < k_eff) {
      char *cur = tiles + (n & 1) * TILE, *nxt = tiles + ((n + 1) & 1) * TILE;
      __builtin_amdgcn_s_waitcnt(0xC07F);
      dma_comp(32 * (c + 1) < k_eff ? c + 1 : KC, nxt);
      wait_vmcnt<NI>();
      const uint32_t bm = comp_mask(c);
      if (bm) step(cur, bm, sk[c]);
      ++n;
    }
  }

  // ---- final statistics (the 4 lane groups of a head share m; sums are partial)
  const float Ls = across_groups_sum(l);
  const float Lnc = across_groups_sum(l_nc);
  const float lse2 = Ls > 0.f ? m + __log2f(Ls) : NINF;
  const float lse2_nc = Lnc > 0.f ? m_nc + __log2f(Lnc) : NINF;
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  if (h_ok && g == 0) {
    lse[(int64_t)t * H + h] = lse2 * LN2;
    lse_nc[(int64_t)t * H + h] = lse2_nc * LN2;
  }
  // O through the LDS tile so every lane stores 16 contiguous bytes: rows of the tile
  // are heads (D bf16 each)
  wait_vmcnt<0>();
  __builtin_amdgcn_s_waitcnt(0xC07F);
  {
    char *ob = tiles;  // 16 heads x ROWB bytes (<= one tile)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      uint2 pk = {pack2_bf16(o[dt][0] * inv, o[dt][1] * inv), pack2_bf16(o[dt][2] * inv, o[dt][3] * inv)};
      // dims dt*16 + 4g .. +3 = half (g & 1) of piece 2dt + (g >> 1), swizzled like the tiles
      *reinterpret_cast<uint2 *>(ob + r16 * ROWB + 16 * ((2 * dt + (g >> 1)) ^ row_swz<D>(r16)) + 8 * (g & 1)) = pk;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    const int nh = min(16, H - 16 * hgrp);   // heads of this group that exist
    uint16_t *obase = out + ((int64_t)t * H + 16 * hgrp) * D;
#pragma unroll
    for (int k = 0; k < 16 * ROWB / 1024; ++k) {
      const int byte = k * 1024 + lane * 16;       // LDS: row hr, piece position pos
      const int hr = byte / ROWB, pos = (byte % ROWB) >> 4;
      if (byte < nh * ROWB)
        *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(obase) + hr * ROWB + 16 * (pos ^ row_swz<D>(hr))) =
            *reinterpret_cast<const u32x4 *>(ob + byte);
    }
  }
  if (cmass != nullptr && hgc == 1) {
    const float nl = (lse2 == NINF || !h_ok) ? NINF : -lse2;   // exp2(-inf) = 0 for dead heads
    float *crow = cmass + (int64_t)t * k_eff;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (32 * c >= k_eff) break;
      float sums[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sums[e] = group16_sum(fast_exp2(fmaf(sk[c][e], sl2, nl)));
      // lane r16 = tau of group g writes slots 32c + 16*tau + 4g + (0..3)
      const int slot0 = 32 * c + 16 * r16 + 4 * g;
      if (r16 < 2) {
        const f32x4 v = r16 ? f32x4{sums[4], sums[5], sums[6], sums[7]} : f32x4{sums[0], sums[1], sums[2], sums[3]};
        if (slot0 + 4 <= k_eff) {
          *reinterpret_cast<f32x4 *>(crow + slot0) = v;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (slot0 + i < k_eff) crow[slot0 + i] = v[i];
        }
      }
    }
  }
}

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N-1>{}), inlined
template <class F, int... Cs>
__device__ __forceinline__ void static_for_impl(F &f, std::integer_sequence<int, Cs...>) {
  (f(std::integral_constant<int, Cs>{}), ...);
}
template <int N, class F> __device__ __forceinline__ void static_for(F &f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ============================================================================
// Persistent pipelined variant (bf16; H <= 16; 1 <= k_eff <= 32*KC, KC <= 8; window > 0).
//
// Same per-query arithmetic and swizzled LDS tiles as the kernel above, but each wave
// walks a strided list of query rows (t, t + W, t + 2W, ... for W waves in the grid)
// as one continuous stream of 32-row steps, with two tiles and a prefetch distance of
// two steps: as soon as step n has read its tile (K operand, then the transposing V
// reads), the rows of step n+2 are requested into that same tile, so every load has a
// whole step to land and the request is issued behind the step's PV MFMAs.  Step n+2
// may belong to the next query (its first or second step), whose ids are fetched during
// the current query's first step and written to the other ids buffer at its second.
//
// Every step requests exactly NI loads (out-of-range ones past the end of the stream),
// so "at most NI vector-memory operations outstanding" at the top of a step means the
// tile of this step has landed: loads complete in order, and any other memory operation
// issued in between (output stores, q and id loads) only makes that wait stricter.
//
// Compressed probabilities are kept in fp32 (rescaled with O when the running max is
// raised), so at the end cmass[j] = sum_h p_hj / L_h needs no second exponential.
// ============================================================================
template <int D, int KC, bool KL>
__global__ __launch_bounds__(256, 2) void sparse_attn_pipe_kernel(
    LayoutDev L, const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const uint16_t *__restrict__ ckv, const float *__restrict__ sink,
    const int32_t *__restrict__ ids, int k_eff, int window, int H, int total_q, int total_k,
    float sl2, uint16_t *__restrict__ out, float *__restrict__ lse, float *__restrict__ lse_nc,
    float *__restrict__ cmass, KlArgs kla) {
  constexpr int NC = D / 32;          // MFMA K-chunks per row
  constexpr int ROWB = D * 2;         // bytes per KV row
  constexpr int PIECES = D / 8;       // 16-byte pieces per row
  constexpr int RPI = 64 / PIECES;    // rows per direct-to-LDS load instruction
  constexpr int NI = 32 / RPI;        // load instructions per 32-row step
  constexpr int TILE = 32 * ROWB;     // one 32-row tile
  constexpr int IDS = 32 * KC;        // id slots per query
  constexpr int IPL = (IDS + 63) / 64;  // id slots per lane
  constexpr float NINF = -__builtin_inff();
  constexpr float RESCALE = 8.f;
  constexpr int NSC = (IDS + 63) / 64;  // 4-byte loads of a row's selected scores (KL)
  static_assert(NI <= 15, "vmcnt");
  static_assert(swz_splits<D>(), "row_swz(i RPI + g) = row_swz(g) ^ row_swz(i RPI)");
  // per wave: two tiles, two id buffers and (KL) the selected scores of the current query
  __shared__ __attribute__((aligned(16))) char lds_all[4][2 * TILE + 2 * IDS * 4 + (KL ? 4 * 64 * NSC : 0)];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int nwaves = gridDim.x * 4;
  int t = blockIdx.x * 4 + w;
  if (t >= total_q) return;           // no block-level barrier below
  char *tiles = lds_all[w];
  int *ids_lds = reinterpret_cast<int *>(tiles + 2 * TILE);   // [2][IDS]
  float *sc_lds = reinterpret_cast<float *>(tiles + 2 * TILE + 2 * IDS * 4);   // [64 NSC] (KL)
  const int h = r16;
  const bool h_ok = h < H;
  const bool group_full = H >= 16;
  const int ncc = (k_eff + 31) >> 5;  // compressed steps per query
  const __amdgpu_buffer_rsrc_t rck = make_rsrc(ckv, (uint32_t)total_k * ROWB);
  const int x16 = (lane ^ 16) << 2, x32 = (lane ^ 32) << 2;   // bpermute addresses
  const int gg = lane / PIECES, pp = lane % PIECES;   // load: row-in-instruction, piece position
  // K operand: row r16, piece (4c + g) ^ swz = 4 (c ^ (swz >> 2)) + (g ^ (swz & 3))
  const int ksw = row_swz<D>(r16);
  const int kbase = r16 * ROWB + 16 * (g ^ (ksw & 3)), kx = ksw >> 2;
  // V^T operand: rows rho (+16), piece (2dt + hb) ^ swz = 2 (dt ^ (swz >> 1)) + (hb ^ (swz & 1))
  const int rho = 4 * g + (r16 >> 2);
  const int vsw = row_swz<D>(rho);
  const int vbase = rho * ROWB + 16 * (((r16 & 3) >> 1) ^ (vsw & 1)) + 8 * (r16 & 1), vx = vsw >> 1;

  // Masked rows read zeros or keep stale tile contents (rows of earlier steps, always
  // finite); their probabilities are exactly 0.
#pragma unroll
  for (int i = 0; i < 2 * TILE / 1024; ++i) reinterpret_cast<u32x4 *>(tiles)[i * 64 + lane] = u32x4{0, 0, 0, 0};

  // a query's geometry is found one query ahead, so its loads have landed long before use
  // (kl_empty: the row is left out of the loss; KL only)
  struct Geo { int w_lo, nw, nwc; bool kl_empty; };
  auto geo_of = [&](int tq) {
    const RowGeo rg = row_geo(L, tq);
    Geo o;
    o.w_lo = max(rg.q_start, tq - window + 1);
    o.nw = tq - o.w_lo + 1;
    o.nwc = (o.nw + 31) >> 5;
    o.kl_empty = KL ? loss_row_empty(L, rg, tq) : false;
    return o;
  };
  // The ids of query tq go straight into id buffer b by 4-byte buffer->LDS loads (no
  // registers, so no wait for them beyond the step waits).  LDS order [step]
  // [row-in-instruction][instruction], so a lane's ids of one step are contiguous: position
  // p holds slot (p & ~31) + ((p & 31) % NI) * RPI + (p & 31) / NI.  Lanes whose slot is
  // at or past k_eff are masked off, so those positions keep the -1 written at the start.
  auto dma_ids = [&](int tq, int b) {
    const __amdgpu_buffer_rsrc_t rid = make_rsrc(ids + (int64_t)tq * k_eff, (uint32_t)k_eff * 4);
#pragma unroll
    for (int i = 0; i < IPL; ++i) {
      const int p = 64 * i + lane, pl = p & 31;
      const int sl = (p & ~31) + (pl % NI) * RPI + pl / NI;
      if (p < IDS && sl < k_eff) dma4(rid, ids_lds + b * IDS + 64 * i, (uint32_t)sl * 4);
    }
  };
  // MFMA K index <-> feature: piece c of lane group g holds features [(4c+g)*8, +8)
  // (a lane of a head past H loads head 0's row: its logits are masked, the values unused)
  auto load_q = [&](int tq, u32x4 (&f)[NC]) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(q + ((int64_t)tq * H + (h_ok ? h : 0)) * D) + g;
#pragma unroll
    for (int c = 0; c < NC; ++c) f[c] = p[4 * c];
  };
  // the NI row loads of step s of a query (window steps first, then compressed steps)
  // into `base`; valid = false requests NI out-of-range loads.  Load i, lane l writes the
  // 16 bytes of tile row R = i RPI + gg, piece slot pp, which hold the row's logical piece
  // pp ^ row_swz(R) = (pp ^ row_swz(gg)) ^ row_swz(i RPI): a per-lane byte offset d0 and a
  // constant per load, so a load costs one or two address instructions.
  auto dma_step = [&](bool valid, const Geo &G, int buf, int s, char *base) {
    int d0 = 16 * (pp ^ row_swz<D>(gg)), ggs = gg;
    asm volatile("" : "+v"(d0), "+v"(ggs));
    if (valid && s < G.nwc) {
      // rows past the query (slot >= nw) lie past the end of this resource: zeros
      const __amdgpu_buffer_rsrc_t rw = make_rsrc(kv, (uint32_t)(G.w_lo + G.nw) * ROWB);
      const uint32_t wb = (uint32_t)(G.w_lo + 32 * s + ggs) * ROWB;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        dma16(rw, base + i * 1024, (wb + (uint32_t)(i * RPI * ROWB)) + (uint32_t)(d0 ^ (16 * row_swz<D>(i * RPI))));
    } else {
      int idr[NI];
      if (valid) {
        const int *il = ids_lds + buf * IDS + (s - G.nwc) * 32 + ggs * NI;
#pragma unroll
        for (int i = 0; i < NI; ++i) idr[i] = il[i];
      } else {
#pragma unroll
        for (int i = 0; i < NI; ++i) idr[i] = -1;
      }
      // an id of -1 gives 2^32 - ROWB + (< ROWB): past the end of the resource, zeros
#pragma unroll
      for (int i = 0; i < NI; ++i)
        dma16(rck, base + i * 1024, (uint32_t)idr[i] * ROWB + (uint32_t)(d0 ^ (16 * row_swz<D>(i * RPI))));
    }
  };

  // the sink logit of this lane's head (the same for every query)
  const float a2 = h_ok ? sink[h] * LOG2E : NINF;
  // ---- stream start: the first query's ids and q, then its first two tiles
  u32x4 qf[NC];
  int buf = 0;
#pragma unroll
  for (int i = 0; i < 2 * IPL; ++i)
    if (64 * i + lane < 2 * IDS) ids_lds[64 * i + lane] = -1;
  __builtin_amdgcn_s_waitcnt(0xC07F);   // the -1 fill is in LDS before any id load lands
  dma_ids(t, 0);
  load_q(t, qf);
  wait_vmcnt<0>();                      // the first query's ids are in LDS
  Geo G = geo_of(t);
  int tn = t + nwaves;
  bool has_next = tn < total_q;
  Geo Gn = {0, 0, 0, false};
  if (has_next) Gn = geo_of(tn);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // zeroing and id stores have executed
  dma_step(true, G, 0, 0, tiles);
  {
    const bool own = 1 < G.nwc + ncc;   // always true with a window
    dma_step(own || has_next, own ? G : Gn, own ? 0 : 1, own ? 1 : 0, tiles + TILE);
  }
  int n = 0;  // stream step index: step n reads tile n & 1

  // head sums of a compressed step: lane r16 of group g ends with the one of value
  // e = sum8_index(r16), slot jl of the step (lanes r16 and r16 ^ 1 hold the same slot).
  // KL: each lane keeps it for every other step c = 2i + half, so the 64 lanes share a
  // row's slots evenly
  constexpr int NO = (KC + 1) / 2;
  const int half = r16 & 1;
  const int el = sum8_index(r16);
  const int jl = 16 * (el >> 2) + 4 * g + (el & 3);             // slot within a step
  const int jo = (jl % RPI) * NI + jl / RPI;                    // its place in ids_lds
  int kp_t = -1;          // the query whose teacher and KL are pending (-1: none)
  bool kp_empty = false;  // its row is left out of the loss
  bool kp_ok[NO];         // slot in the support (a valid id)
  float kp_own[NO], kp_sc[NO];   // head-summed mass and selected score of the slot
  auto kl_finish = [&]() __attribute__((always_inline)) {
    float *te = kla.teacher ? kla.teacher + (int64_t)kp_t * kla.ldt : nullptr;
    double kl = 0.0;
    if (kp_empty) {
#pragma unroll
      for (int i = 0; i < NO; ++i) kp_own[i] = 0.f;
    } else {
      kl = sparse_kl_wave<NO, WaveRed, true>(kp_ok, kp_own, kp_sc);   // kp_own now holds the teacher
    }
    if (te) {
#pragma unroll
      for (int i = 0; i < NO; ++i) {
        const int c = 2 * i + half, j = 32 * c + jl;
        if (c < ncc && j < k_eff) te[j] = kp_own[i];
      }
    }
    if (lane == 0) kla.kl_row[kp_t] = (float)kl;
  };

  for (;;) {
    const int nsteps = G.nwc + ncc;

    float m = a2;                                        // shared by the 4 lane groups of a head
    float l = (g == 0 && a2 > NINF) ? 1.f : 0.f;         // per-lane partial sum
    f32x4 o[D / 16];
#pragma unroll
    for (int i = 0; i < D / 16; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float pk[KC][8];  // compressed probabilities exp2(sl2*s - m), kept for cmass
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) pk[c][e] = 0.f;

    // Top of step s: its tile has landed (at most the NI loads of step n+1 outstanding)
    // and every LDS access of step n-1 has returned.  At s = 0 the next query's ids are
    // requested into the other id buffer (issued before the request of step 2, they have
    // landed by the top of step 1; they are first read by a request issued at s >= 1: the
    // next query's first step is a window step).
    auto top = [&](int s) __attribute__((always_inline)) {
      wait_vmcnt<NI>();
      __builtin_amdgcn_s_waitcnt(0xC07F);
      // KL: this query's selected scores into LDS; issued before the request of step 2,
      // they have landed by the top of step 1 (there are always at least two steps)
      if constexpr (KL) {
        if (s == 0) {
          const __amdgpu_buffer_rsrc_t rsc = make_rsrc(kla.scores + (int64_t)t * kla.ld, (uint32_t)k_eff * 4);
#pragma unroll
          for (int i = 0; i < NSC; ++i) dma4(rsc, sc_lds + 64 * i, (uint32_t)(64 * i + lane) * 4);
        }
      }
      // the next query's ids and q rows: issued ahead of this query's row requests, so
      // that waiting for them never waits for a tile still in flight
      if (s == 0 && has_next) dma_ids(tn, buf ^ 1);
    };
    // the rows of stream step n+2 into the tile step n has just finished reading
    auto request = [&](int s) __attribute__((always_inline)) {
      char *dst = tiles + (n & 1) * TILE;
      const int s2 = s + 2;
      if (s2 < nsteps) dma_step(true, G, buf, s2, dst);
      else dma_step(has_next, Gn, buf ^ 1, s2 - nsteps, dst);
    };

    // one 32-row step on the tile at `base`; bm = row validity bits; leaves this lane's
    // compressed step CI keeps its fp32 probabilities in pk[CI] (CI < 0: window step)
    auto step = [&](auto ci, int s, uint32_t bm) __attribute__((always_inline)) {
      constexpr int CI = decltype(ci)::value;
      float raw[8];
      const char *base = tiles + (n & 1) * TILE;
      // the per-lane address terms are re-derived every step (opaque copies), so that
      // the compiler does not keep all the operand addresses live across the loop
      int kxs = kx, vxs = vx;
      asm volatile("" : "+v"(kxs), "+v"(vxs));
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const char *kp = base + kbase + 64 * (c ^ kxs);
        const u32x4 k0 = *reinterpret_cast<const u32x4 *>(kp);
        const u32x4 k1 = *reinterpret_cast<const u32x4 *>(kp + 16 * ROWB);
        acc0 = mfma16x16x32(k0, qf[c], acc0);
        acc1 = mfma16x16x32(k1, qf[c], acc1);
      }
      // (masked in place: the common full-tile path then needs no register copies)
#pragma unroll
      for (int i = 0; i < 4; ++i) { raw[i] = acc0[i]; raw[4 + i] = acc1[i]; }
      if (!(group_full && bm == 0xffffffffu)) {
        const uint32_t m0 = h_ok ? (bm >> (4 * g)) : 0u, m1 = h_ok ? (bm >> (16 + 4 * g)) : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          raw[i] = ((m0 >> i) & 1) ? raw[i] : NINF;
          raw[4 + i] = ((m1 >> i) & 1) ? raw[4 + i] : NINF;
        }
      }
      // Common path without cross-lane traffic: each lane tests its logits against the
      // shared reference max; only a logit 2^8 above it makes the wave agree on a new
      // per-head max and rescale.
      float cmx = fmaxf(fmaxf(fmaxf(raw[0], raw[1]), fmaxf(raw[2], raw[3])),
                        fmaxf(fmaxf(raw[4], raw[5]), fmaxf(raw[6], raw[7])));
      if (__builtin_expect(__ballot(cmx * sl2 > m + RESCALE) != 0, 0)) {
        cmx = fmaxf(cmx, bperm(x16, cmx));
        cmx = fmaxf(cmx, bperm(x32, cmx));
        const float cand = cmx * sl2;
        const float mn = cand > m + RESCALE ? cand : m;
        const float alpha = fast_exp2(m - mn);
        l *= alpha;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) o[i] *= alpha;
#pragma unroll
        for (int c = 0; c < KC; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) pk[c][e] *= alpha;
        m = mn;
      }
      const float nms = m == NINF ? 0.f : -m;
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { p[e] = fast_exp2(fmaf(raw[e], sl2, nms)); l += p[e]; }
      if constexpr (CI >= 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pk[CI][e] = p[e];
      }
      const u32x4 pb = {pack2_bf16(p[0], p[1]), pack2_bf16(p[2], p[3]), pack2_bf16(p[4], p[5]),
                        pack2_bf16(p[6], p[7])};
      // V^T operands in two halves of D/32 d-tiles (fewer registers in flight)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        uint2 xv[D / 16];
        uint32_t va[D / 32];
#pragma unroll
        for (int k = 0; k < D / 32; ++k) va[k] = lds_addr_of(base + vbase + 32 * ((hf * (D / 32) + k) ^ vxs));
        lds_read_tr16_pairs<16 * ROWB>(xv, va);
#pragma unroll
        for (int k = 0; k < D / 32; ++k) {
          const int dt = hf * (D / 32) + k;
          const u32x4 a = {xv[2 * k].x, xv[2 * k].y, xv[2 * k + 1].x, xv[2 * k + 1].y};
          o[dt] = mfma16x16x32(a, pb, o[dt]);
        }
      }
      request(s);   // the tile is free: its LDS reads have all returned
    };

    top(0);
    // the previous query's teacher and KL: their chain of wave reductions runs while the
    // rows of step 1 are in flight, and their stores go out before the request of step 2
    // (a store issued after it would make the wait at the top of step 1 wait for it)
    if constexpr (KL) {
      if (kp_t >= 0) kl_finish();
    }
    step(std::integral_constant<int, -1>{}, 0, G.nw >= 32 ? 0xffffffffu : (1u << G.nw) - 1u);
    ++n;
    for (int s = 1; s < G.nwc; ++s, ++n) {
      top(s);
      const int nwin = G.nw - 32 * s;
      step(std::integral_constant<int, -1>{}, s, nwin >= 32 ? 0xffffffffu : (1u << nwin) - 1u);
    }
    const float m_nc = m, l_nc = l;
    // compressed steps, unrolled so that step c writes pk[c] with constant indices
    auto comp_step = [&](auto ci) __attribute__((always_inline)) {
      constexpr int C = decltype(ci)::value;
      if (C < ncc) {
        const int s = G.nwc + C;
        top(s);
        // row validity of compressed step C: bit R set iff the id of row R is >= 0
        const int R = lane & 31;
        const uint32_t bm = (uint32_t)__ballot(ids_lds[buf * IDS + C * 32 + (R % RPI) * NI + R / RPI] >= 0);
        step(ci, s, bm);
        ++n;
      }
    };
    static_for<KC>(comp_step);
    // the next query's q rows stream in during this query's epilogue
    if (has_next) load_q(tn, qf);

    // ---- final statistics (the 4 lane groups of a head share m; sums are partial)
    const float Ls = across_groups_sum(l);
    const float Lnc = across_groups_sum(l_nc);
    const float lse2 = Ls > 0.f ? m + __log2f(Ls) : NINF;
    const float lse2_nc = Lnc > 0.f ? m_nc + __log2f(Lnc) : NINF;
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    if (h_ok) {
      if (g == 0) {
        lse[(int64_t)t * H + h] = lse2 * LN2;
        lse_nc[(int64_t)t * H + h] = lse2_nc * LN2;
      }
      // O straight from the accumulator: lane (head r16, group g) holds dims 16dt+4g..+3
      uint16_t *orow = out + ((int64_t)t * H + h) * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        *reinterpret_cast<uint2 *>(orow + 16 * dt) =
            uint2{pack2_bf16(o[dt][0] * inv, o[dt][1] * inv), pack2_bf16(o[dt][2] * inv, o[dt][3] * inv)};
    }
    // head sums of the compressed probabilities: value e of a lane of group g is slot
    // 32c + 16 (e >> 2) + 4g + (e & 3); lane r16 ends with the sum of slot 32c + jl.  For
    // the KL each lane keeps the steps c = 2i + half in own[i].
    float own[NO];
#pragma unroll
    for (int i = 0; i < NO; ++i) own[i] = 0.f;
    if (cmass != nullptr || KL) {
      float *crow = cmass ? cmass + (int64_t)t * k_eff : nullptr;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        if (c < ncc) {
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = pk[c][e] * inv;
          const float sum = group16_sum8(pv, r16);
          if constexpr (KL) {
            if (half == (c & 1)) own[c >> 1] = sum;
          }
          const int j = 32 * c + jl;
          if (crow && half == 0 && j < k_eff) crow[j] = sum;
        }
      }
    }
    if constexpr (KL) {
      // what the row's teacher and KL need, taken before its id and score buffers are
      // reused; the arithmetic is finished during the next query's first step
      kp_t = t;
      kp_empty = G.kl_empty;
#pragma unroll
      for (int i = 0; i < NO; ++i) {
        const int c = 2 * i + half, j = 32 * c + jl;
        kp_ok[i] = c < ncc && j < k_eff && ids_lds[buf * IDS + 32 * c + jo] >= 0;
        kp_sc[i] = kp_ok[i] ? sc_lds[j] : 0.f;
        kp_own[i] = own[i];
      }
    }
    if (!has_next) break;
    t = tn;
    G = Gn;
    buf ^= 1;
    tn = t + nwaves;
    has_next = tn < total_q;
    if (has_next) Gn = geo_of(tn);
  }
  if constexpr (KL) kl_finish();   // the last query's
  wait_vmcnt<0>();   // the stream's trailing out-of-range requests
}

// kla != nullptr: the pipelined kernel also finishes the sparse teacher and KL (only
// called so when pipe_kl_supported holds)
template <int D>
static hipError_t launch_dma(const LaunchLayout &LL, const void *q, const void *kv, const void *ckv,
                             const float *sink, const int32_t *ids, int k_eff, int window, int H,
                             float scale, void *out, float *lse, float *lse_nc, float *cmass,
                             hipStream_t st, const KlArgs *kla = nullptr) {
  const int hgc = (H + 15) / 16;
  const int qpw = 4 / hgc;
  const float sl2 = scale * LOG2E;
  if (hgc == 1 && window > 0) {
    // persistent: two workgroups of 4 waves per CU, each wave walking a strided list of rows
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
      ncu = 256;   // the query failed: assume the MI355X's count
    const int64_t need = (LL.total_q + 3) / 4;
    dim3 pgrid((unsigned)std::min<int64_t>(need, 2 * (int64_t)ncu));
#define CSA_PIPE_CASE(K)                                                                             \
    if (k_eff <= 32 * K) {                                                                           \
      if (kla != nullptr)                                                                            \
        hipLaunchKernelGGL((sparse_attn_pipe_kernel<D, K, true>), pgrid, dim3(256), 0, st, LL.dev,   \
                           static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(kv),      \
                           static_cast<const uint16_t *>(ckv), sink, ids, k_eff, window, H,          \
                           LL.total_q, LL.total_k, sl2, static_cast<uint16_t *>(out), lse, lse_nc,   \
                           cmass, *kla);                                                             \
      else                                                                                           \
        hipLaunchKernelGGL((sparse_attn_pipe_kernel<D, K, false>), pgrid, dim3(256), 0, st, LL.dev,  \
                           static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(kv),      \
                           static_cast<const uint16_t *>(ckv), sink, ids, k_eff, window, H,          \
                           LL.total_q, LL.total_k, sl2, static_cast<uint16_t *>(out), lse, lse_nc,   \
                           cmass, KlArgs{});                                                         \
      return hipGetLastError();                                                                      \
    }
    CSA_PIPE_CASE(1)
    CSA_PIPE_CASE(2)
    CSA_PIPE_CASE(4)
    CSA_PIPE_CASE(8)
#undef CSA_PIPE_CASE
    return hipErrorInvalidValue;
  }
  dim3 grid((unsigned)((LL.total_q + qpw - 1) / qpw));
#define CSA_DMA_CASE(K)                                                                              \
  if (k_eff <= 32 * K) {                                                                             \
    hipLaunchKernelGGL((sparse_attn_dma_kernel<D, K>), grid, dim3(256), 0, st, LL.dev,               \
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(kv),          \
                       static_cast<const uint16_t *>(ckv), sink, ids, k_eff, window, H, LL.total_q,  \
                       LL.total_k, sl2, static_cast<uint16_t *>(out), lse, lse_nc, cmass);           \
    return hipGetLastError();                                                                        \
  }
  CSA_DMA_CASE(1)
  CSA_DMA_CASE(2)
  CSA_DMA_CASE(4)
  CSA_DMA_CASE(8)
#undef CSA_DMA_CASE
  return hipErrorInvalidValue;
}

template <typename IN, int D>
static hipError_t launch_d(const LaunchLayout &LL, const void *q, const void *kv, const void *ckv,
                           const float *sink, const int32_t *ids, int k_eff, int window, int H,
                           float scale, void *out, float *lse, float *lse_nc, float *cmass,
                           hipStream_t st) {
  const float sl2 = scale * LOG2E;
  dim3 grid((unsigned)LL.total_q);
  const int hg = (H + 15) / 16;
  const size_t dyn = 2 * (size_t)ATT_CHUNK * AttnCfg<IN, D>::RS + (size_t)k_eff * sizeof(int);
#define CSA_ATT_CASE(G)                                                                           \
  if (hg <= G) {                                                                                  \
    if (dyn > 65536) {                                                                            \
      const hipError_t ea = hipFuncSetAttribute(                                                  \
          reinterpret_cast<const void *>(sparse_attn_kernel<IN, D, G>),                          \
          hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);                                  \
      if (ea != hipSuccess) return ea;                                                            \
    }                                                                                             \
    hipLaunchKernelGGL((sparse_attn_kernel<IN, D, G>), grid, dim3(64 * G), dyn, st, LL.dev,       \
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

// NG head groups of 16 per wave: 2 where the registers allow it (D <= 192), so that every
// K and V operand read from LDS feeds two MFMAs
template <int D>
static hipError_t launch_wg(const LaunchLayout &LL, const void *q, const void *kv, const void *ckv,
                            const float *sink, const int32_t *ids, int k_eff, int window, int H,
                            float scale, void *out, float *lse, float *lse_nc, float *cmass,
                            hipStream_t st) {
  constexpr int NG = D <= 192 ? 2 : 1;
  const float sl2 = scale * LOG2E;
  const int hg = (H + 16 * NG - 1) / (16 * NG);
  const int ncc = (k_eff + 31) / 32;
  const size_t dyn = 2 * (size_t)32 * D * 2 + (size_t)ncc * 32 * sizeof(int);
#define CSA_WG_CASE(G)                                                                                \
  if (hg <= G) {                                                                                      \
    auto kern = sparse_attn_wg_kernel<D, G, NG>;                                                      \
    if (dyn > 65536) {                                                                                \
      const hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),                 \
                                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn); \
      if (ea != hipSuccess) return ea;                                                                \
    }                                                                                                 \
    hipLaunchKernelGGL(kern, dim3((unsigned)LL.total_q), dim3(64 * G), dyn, st, LL.dev,               \
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(kv),           \
                       static_cast<const uint16_t *>(ckv), sink, ids, k_eff, window, H, LL.total_q,   \
                       LL.total_k, sl2, static_cast<uint16_t *>(out), lse, lse_nc, cmass);            \
    return hipGetLastError();                                                                         \
  }
  CSA_WG_CASE(1)
  CSA_WG_CASE(2)
  CSA_WG_CASE(4)
  CSA_WG_CASE(8)
#undef CSA_WG_CASE
  return hipErrorInvalidValue;
}

// shapes of the pipelined kernel (bf16, one wave per query for H <= 16 heads, a window,
// 1 <= k_eff <= 256, KV within the 2 GiB reach of 32-bit buffer offsets)
static bool pipe_shape(const LaunchLayout &LL, bool bf16, int H, int D, int k_eff, int window) {
  return bf16 && H <= 16 && k_eff >= 1 && k_eff <= 256 && window > 0 && (D == 64 || D == 128) &&
         (int64_t)LL.total_q * D * 2 < (1ll << 31) && (int64_t)LL.total_k * D * 2 < (1ll << 31);
}

bool attn_kl_fused_supported(const LaunchLayout &LL, bool bf16, int H, int D, int k_eff, int window) {
  return pipe_shape(LL, bf16, H, D, k_eff, window);
}

hipError_t launch_sparse_attn_kl(const LaunchLayout &LL, const void *q, const void *kv,
                                 const void *ckv, const float *sink, const int32_t *ids, int k_eff,
                                 int window, int H, int D, float scale, void *out, float *lse,
                                 float *lse_nc, float *cmass, const KlArgs &kla, hipStream_t st) {
  if (LL.total_q == 0) return hipSuccess;
  switch (D) {
    case 64: return launch_dma<64>(LL, q, kv, ckv, sink, ids, k_eff, window, H, scale, out, lse, lse_nc, cmass, st, &kla);
    case 128: return launch_dma<128>(LL, q, kv, ckv, sink, ids, k_eff, window, H, scale, out, lse, lse_nc, cmass, st, &kla);
  }
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
  // gather-optimised variant: one wave per 16 heads, cmass from kept logits
  // (buffer offsets are 32-bit: both KV tensors must stay below 2 GiB)
  if (bf16 && H <= 16 && k_eff >= 1 && k_eff <= 256 && (int64_t)LL.total_q * D * 2 < (1ll << 31) &&
      (int64_t)LL.total_k * D * 2 < (1ll << 31)) {
    switch (D) {
      case 64: return launch_dma<64>(CSA_ARGS);
      case 128: return launch_dma<128>(CSA_ARGS);
    }
  }
  // workgroup variant: rows staged by direct buffer->LDS loads (32-bit buffer offsets)
  if (bf16 && (int64_t)LL.total_q * D * 2 < (1ll << 31) && (int64_t)LL.total_k * D * 2 < (1ll << 31)) {
    switch (D) {
      case 64: return launch_wg<64>(CSA_ARGS);
      case 128: return launch_wg<128>(CSA_ARGS);
      case 192: return launch_wg<192>(CSA_ARGS);
      case 256: return launch_wg<256>(CSA_ARGS);
      case 512: return launch_sparse_attn_wide(CSA_ARGS);
    }
  }
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
