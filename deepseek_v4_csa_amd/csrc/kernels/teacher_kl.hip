// Paper-equivalent indexer teacher, KL(teacher || indexer softmax) and the loss.
//
// Page "[Bug] DSV4 unfused CSA indexer loss uses a compressed-only teacher ...":
//   "Paper reference": t_j = sum_h exp(c_hj)/Z_h, L1-normalised over the compressed set,
//   Z_h keeping the sink and window terms;
//   proposal comment (discussion thread): l_h = log(exp(u_h) + sum_{j in C} exp(c_hj)),
//   p_hj = exp(c_hj - l_h); C = top-k intersected with the causally valid entries
//   (sparse loss) or every causally visible entry (dense loss);
//   dsa.py excerpt: L1 clamp 1e-10, KL with log(x + 1e-10) on both sides (kept as
//   written per the review comment "KL numerical contract");
//   dsa_kernels.py excerpt: the sparse predictor is the softmax of the indexer scores
//   gathered at the top-k ids, -1 slots excluded.
//
// Sparse mode: the attention pass already produced cmass[t, j] = sum_h exp(c_hj -
// lse_h) with lse_h = l_h (its compressed set is C), so the teacher is cmass / sum.
// One wave per row.  Dense mode: c_hj is recomputed here for every visible key (MFMA,
// one workgroup per row, keys streamed through LDS in two passes: exact l_h first,
// then the head-summed probabilities).  kl_row is then reduced to the loss by a
// single-workgroup kernel in a fixed order (deterministic, no atomics).
#include "common.h"
#include "sparse_kl.h"
#include "../launch.h"

namespace csa {

// ---------------------------------------------------------------- sparse
// NW waves per row (1, 2 or 4: a row's slots / 64 lanes / NW <= 8, so a lane keeps few
// registers however long the row); slot j = (v*NW + wr)*64 + lane for wave wr of the row,
// so every load is issued up front and coalesced except the score gather (one dependent
// load per slot); the row is finished by sparse_kl_wave, its sums over the row's waves
// combined through LDS when NW > 1 (every wave then reaches every reduction: rows past T
// or left out of the loss run them with an empty support).
template <int SPL, int NW>
__global__ __launch_bounds__(256) void teacher_kl_sparse_kernel(
    LayoutDev L, int T, const float *__restrict__ scores, int64_t ld, int selected,
    const int32_t *__restrict__ ids, int k_eff, const float *__restrict__ cmass, float *__restrict__ teacher,
    int64_t ldt, float *__restrict__ kl_row) {
  constexpr int RPB = 4 / NW;   // rows per workgroup
  __shared__ float fred[RPB][NW];
  __shared__ double dred[RPB][NW];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int rw = w / NW, wr = w % NW;   // the wave's row within the workgroup, its index there
  const int t = blockIdx.x * RPB + rw;
  if (NW == 1 && t >= T) return;        // (a lone wave has no barrier to meet)
  const bool live = t < T;
  const int tt = live ? t : 0;
  const float *sr = scores + (int64_t)tt * ld;
  float *te = (teacher && live) ? teacher + (int64_t)tt * ldt : nullptr;
  // every load that needs only the row index goes out first (ids, cmass and, in place,
  // the selected scores), through buffer resources of exactly k_eff elements: the loads
  // are unconditional (past the end they read zeros) and all in flight at once -- a load
  // under a per-slot branch is waited for at the branch's end, before the next is issued
  const __amdgpu_buffer_rsrc_t rid = make_rsrc(ids + (int64_t)tt * k_eff, (uint32_t)k_eff * 4);
  const __amdgpu_buffer_rsrc_t rcm = make_rsrc(cmass + (int64_t)tt * k_eff, (uint32_t)k_eff * 4);
  const __amdgpu_buffer_rsrc_t rsc = make_rsrc(sr, selected ? (uint32_t)k_eff * 4 : 0u);
  int id[SPL];
  float c[SPL], sc[SPL];
#pragma unroll
  for (int v = 0; v < SPL; ++v) {
    const int j = (v * NW + wr) * 64 + lane;
    id[v] = __builtin_amdgcn_raw_buffer_load_b32(rid, j * 4, 0, 0);
    c[v] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rcm, j * 4, 0, 0));
    sc[v] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsc, j * 4, 0, 0));
  }
#pragma unroll
  for (int v = 0; v < SPL; ++v) {
    const bool in = live && (v * NW + wr) * 64 + lane < k_eff;
    id[v] = in ? id[v] : -1;
    c[v] = in ? c[v] : 0.f;
  }
  const RowGeo geo = row_geo(L, tt);
  const bool empty = !live || loss_row_empty(L, geo, tt);
  if (NW == 1 && empty) {
    if (te)
      for (int j = lane; j < k_eff; j += 64) te[j] = 0.f;
    if (lane == 0) kl_row[t] = 0.f;
    return;
  }
  bool ok[SPL];
#pragma unroll
  for (int v = 0; v < SPL; ++v) ok[v] = !empty && id[v] >= 0;
  if (!selected) {
    // the score of slot j gathered from the full row, unconditionally (a slot off the
    // support reads past the resource: zero, unused)
    const __amdgpu_buffer_rsrc_t rrow = make_rsrc(sr, (uint32_t)geo.n_valid * 4);
#pragma unroll
    for (int v = 0; v < SPL; ++v)
      sc[v] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rrow, ok[v] ? (uint32_t)(id[v] - geo.k_base) * 4 : BUF_OOB, 0, 0));
  }
  double kl;   // c now holds the teacher (0 off the support, and on an empty row)
  if constexpr (NW == 1) kl = sparse_kl_wave(ok, c, sc);
  else kl = sparse_kl_wave(ok, c, sc, GroupRed<NW>{fred[rw], dred[rw], wr});
  if (te) {
#pragma unroll
    for (int v = 0; v < SPL; ++v) {
      const int j = (v * NW + wr) * 64 + lane;
      if (j < k_eff) te[j] = c[v];
    }
  }
  if (live && wr == 0 && lane == 0) kl_row[t] = empty ? 0.f : (float)kl;
}

// ---------------------------------------------------------------- dense
// One workgroup per row, wave w owning two groups of 16 heads (32w..32w+31), so that each
// K operand read from LDS feeds the MFMAs of both.  The row's visible keys are the
// first n rows of its segment's ckv, contiguous: they are staged 32 at a time into two LDS
// tiles by buffer->LDS loads that the waves split between them (D/16 instructions of
// 1 KiB per tile), each 16-byte piece p of tile row R at position p ^ row_swz<D>(R), and
// the next tile is requested right after each step's barrier.  The buffer resource spans
// exactly the n visible rows, so the loads past them read zeros.  Two passes over the
// tiles: the exact l_h, then the head-summed probabilities m_j (summed within a wave on
// DPP, across waves through LDS one step later, behind the next barrier).
template <int D, int HG, int NG>
__global__ __launch_bounds__(64 * HG) void teacher_kl_dense_kernel(
    LayoutDev L, const float *__restrict__ scores, int64_t ld, const uint16_t *__restrict__ q,
    const uint16_t *__restrict__ ckv, const float *__restrict__ lse_nc, int H, float scale_log2,
    float *__restrict__ teacher, int64_t ldt, float *__restrict__ kl_row) {
  constexpr int NC = D / 32;          // MFMA K-chunks per row
  constexpr int ROWB = D * 2;
  constexpr int PIECES = D / 8;
  constexpr int NI = PIECES / 2;      // load instructions per 32-row tile
  constexpr int NIW = (NI + HG - 1) / HG;
  constexpr int TILE = 32 * ROWB;
  constexpr int NT = 64 * HG;
  constexpr int HPW = 16 * NG;        // heads per wave (NG groups of 16)
  constexpr float NINF = -__builtin_inff();
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float *mj = reinterpret_cast<float *>(smem + 2 * TILE);      // [n_valid]
  __shared__ float part[2][HG][32];
  __shared__ float red[2 * 16];

  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, hl = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int hh[NG];
  bool h_ok[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    hh[gi] = HPW * w + 16 * gi + hl;
    h_ok[gi] = hh[gi] < H;
  }
  const bool wave_full = HPW * (w + 1) <= H;
  const RowGeo geo = row_geo(L, t);
  const int n = geo.n_valid;
  if (loss_row_empty(L, geo, t)) {
    if (teacher)
      for (int j = tid; j < ldt; j += NT) teacher[(int64_t)t * ldt + j] = 0.f;
    if (tid == 0) kl_row[t] = 0.f;
    return;
  }
  // Q^T operands, MFMA K index <-> feature: piece c of lane group g holds features [(4c+g)*8, +8)
  u32x4 qf[NG][NC];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(q + ((int64_t)t * H + (h_ok[gi] ? hh[gi] : 0)) * D) + g;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[gi][c] = p[4 * c];   // (masked where the head is past H)
  }
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(ckv + (int64_t)geo.k_base * D, (uint32_t)n * ROWB);
  const int nch = (n + 31) / 32;
  // this wave's loads of chunk ci: instruction i = w + k*HG, lane l -> piece slot 64 i + l
  // (when a load covers whole rows, RPI = 512 / D of them, the row is i RPI + l / PIECES
  // and the swizzle splits into a per-lane and a per-load term)
  auto issue = [&](int ci, char *buf) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int k = 0; k < NIW; ++k) {
      const int i = w + k * HG;
      if (NI % HG == 0 || i < NI) {
        if constexpr (512 % D == 0) {
          static_assert(512 % D != 0 || swz_splits<D>(), "row_swz(i RPI + g) = row_swz(g) ^ row_swz(i RPI)");
          constexpr int RPI = 512 % D == 0 ? 512 / D : 1;
          const int gl = ln / PIECES;
          const uint32_t d0 = 16 * ((ln % PIECES) ^ row_swz<D>(gl)), sx = 16 * row_swz<D>(i * RPI);
          dma16(rk, buf + i * 1024, (uint32_t)(32 * ci + i * RPI + gl) * ROWB + (d0 ^ sx));
        } else {
          const int P = 64 * i + ln;
          const int R = P / PIECES, pc = P - R * PIECES;
          dma16(rk, buf + i * 1024, (uint32_t)(32 * ci + R) * ROWB + 16 * (pc ^ row_swz<D>(R)));
        }
      }
    }
  };
  // K operand: row r16 (+16), piece (4c + g) ^ swz = 4 (c ^ (swz >> 2)) + (g ^ (swz & 3))
  const int ksw = row_swz<D>(hl);
  const int kbase = hl * ROWB + 16 * (g ^ (ksw & 3)), kx = ksw >> 2;
  // this lane's 8 products q.k of chunk ci per head group (rows 4g+i and 16+4g+i, head
  // 16 gi + hl of the wave), unscaled, -inf past n or for a head past H; each K operand
  // read from LDS feeds the MFMAs of every head group
  auto logits = [&](const char *base, int ci, float (&sv)[NG][8]) {
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
    const int j0 = 32 * ci + 4 * g;
    if (wave_full && 32 * ci + 32 <= n) {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
#pragma unroll
        for (int i = 0; i < 4; ++i) { sv[gi][i] = acc0[gi][i]; sv[gi][4 + i] = acc1[gi][i]; }
    } else {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[gi][i] = (j0 + i < n && h_ok[gi]) ? acc0[gi][i] : NINF;
          sv[gi][4 + i] = (j0 + 16 + i < n && h_ok[gi]) ? acc1[gi][i] : NINF;
        }
    }
  };
  const int ns = 2 * nch;   // steps: pass 1 over the chunks, then pass 2
  auto tile = [&](int s) { return smem + (s & 1) * TILE; };
  auto top = [&](int s) {
    wait_vmcnt<0>();
    __syncthreads();   // step s's tile landed for every wave; tile s-1 is no longer read
    if (s + 1 < ns) issue(s + 1 < nch ? s + 1 : s + 1 - nch, tile(s + 1));
  };
  if (ns > 0) issue(0, tile(0));

  // pass 1: l_h = log2(2^{u_h} + sum_j 2^{c_hj})   (base-2 logits; scale_log2 > 0, so the
  // maximum of the unscaled products is the maximum of the logits)
  // (one running max per head, shared by its 4 lane groups and raised only when a logit
  // exceeds it by 2^8, so the common chunk needs no rescaling and no cross-lane traffic)
  constexpr float RESCALE = 8.f;
  float m[NG], l[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const float u2 = h_ok[gi] ? lse_nc[(int64_t)t * H + hh[gi]] * LOG2E : NINF;
    m[gi] = u2;
    l[gi] = (g == 0 && u2 > NINF) ? 1.f : 0.f;   // e^{u_h} counted once per head
  }
  for (int ci = 0; ci < nch; ++ci) {
    top(ci);
    float s[NG][8];
    logits(tile(ci), ci, s);
    float cmx[NG];
    bool up = false;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      cmx[gi] = s[gi][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) cmx[gi] = fmaxf(cmx[gi], s[gi][e]);
      up = up || cmx[gi] * scale_log2 > m[gi] + RESCALE;
    }
    if (__builtin_expect(__ballot(up) != 0, 0)) {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const float cand = across_groups_max(cmx[gi]) * scale_log2;
        const float mn = cand > m[gi] + RESCALE ? cand : m[gi];
        l[gi] *= mn == m[gi] ? 1.f : fast_exp2(m[gi] - mn);
        m[gi] = mn;
      }
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const float nms = m[gi] == NINF ? 0.f : -m[gi];
#pragma unroll
      for (int e = 0; e < 8; ++e) l[gi] += fast_exp2(fmaf(s[gi][e], scale_log2, nms));
    }
  }
  float nl[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const float Ls = across_groups_sum(l[gi]);
    const float ell2 = Ls > 0.f ? m[gi] + __log2f(Ls) : NINF;
    nl[gi] = ell2 > NINF ? -ell2 : NINF;   // exp2(-inf) = 0: no mass at all
  }

  // pass 2: m_j = sum_h 2^{c_hj - l_h}
  auto flush = [&](int cprev) {
    if (tid < 32) {
      const int j = 32 * cprev + tid;
      if (j < n) {
        float sum = 0.f;
#pragma unroll
        for (int ww = 0; ww < HG; ++ww) sum += part[(nch + cprev) & 1][ww][tid];
        mj[j] = sum;
      }
    }
  };
  for (int ci = 0; ci < nch; ++ci) {
    const int st = nch + ci;
    top(st);
    if (ci > 0) flush(ci - 1);
    float s[NG][8];
    logits(tile(st), ci, s);
    // value e of group g is key 16 (e >> 2) + 4g + (e & 3); lane hl ends with the head
    // sum of value sum8_index(hl)
    float ps[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ps[e] = fast_exp2(fmaf(s[0][e], scale_log2, nl[0]));
#pragma unroll
      for (int gi = 1; gi < NG; ++gi) ps[e] += fast_exp2(fmaf(s[gi][e], scale_log2, nl[gi]));
    }
    const float sh = group16_sum8(ps, hl);
    const int el = sum8_index(hl);
    if ((hl & 1) == 0) part[st & 1][w][16 * (el >> 2) + 4 * g + (el & 3)] = sh;
  }
  __syncthreads();
  if (nch > 0) flush(nch - 1);
  __syncthreads();   // m_j complete

  // predictor over j < n, teacher normalisation, KL: all in fp64 from the fp32 scores and
  // masses (pred_exp, kl_term: the same arithmetic as the sparse loss)
  const float *sr = scores + (int64_t)t * ld;
  __shared__ double dred[2 * 16];
  // the row's scores in batches of 8 per thread through a buffer resource of exactly n
  // floats: unconditional loads, all 8 in flight at once (a loop of single guarded loads
  // would wait for each before the next)
  constexpr int UB = 8;
  const __amdgpu_buffer_rsrc_t rsr = make_rsrc(sr, (uint32_t)n * 4);
  auto load_batch = [&](int base, float (&x)[UB]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < UB; ++u)
      x[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsr, (base + u * NT) * 4, 0, 0));
  };
  float mx = NINF;
  double msum = 0.0;
  for (int base = tid; base < n; base += UB * NT) {
    float x[UB];
    load_batch(base, x);
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int j = base + u * NT;
      if (j < n) { mx = fmaxf(mx, x[u]); msum += (double)mj[j]; }
    }
  }
  mx = wave_max(mx);
  msum = wave_sum_f64(msum);
  if (lane == 0) { red[w] = mx; dred[w] = msum; }
  __syncthreads();
  mx = red[0]; msum = dred[0];
  for (int ww = 1; ww < HG; ++ww) { mx = fmaxf(mx, red[ww]); msum += dred[ww]; }
  __syncthreads();
  double es = 0.0;
  for (int base = tid; base < n; base += UB * NT) {
    float x[UB];
    load_batch(base, x);
#pragma unroll
    for (int u = 0; u < UB; ++u)
      if (base + u * NT < n) es += pred_exp(x[u], mx);
  }
  es = wave_sum_f64(es);
  if (lane == 0) dred[16 + w] = es;
  __syncthreads();
  es = 0.0;
  for (int ww = 0; ww < HG; ++ww) es += dred[16 + ww];
  const double inv_es = 1.0 / es;
  const double inv_m = 1.0 / fmax(msum, KL_EPS);
  double kl = 0.0;
  for (int base = tid; base < n; base += UB * NT) {
    float x[UB];
    load_batch(base, x);
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int j = base + u * NT;
      if (j < n) {
        const double tj = (double)mj[j] * inv_m;
        kl += kl_term<true>(tj, pred_exp(x[u], mx) * inv_es);
        if (teacher) teacher[(int64_t)t * ldt + j] = (float)tj;
      }
    }
  }
  if (teacher)
    for (int j = n + tid; j < ldt; j += NT) teacher[(int64_t)t * ldt + j] = 0.f;
  kl = wave_sum_f64(kl);
  __shared__ double kred[16];
  __syncthreads();
  if (lane == 0) kred[w] = kl;
  __syncthreads();
  if (tid == 0) {
    double sacc = 0.0;
    for (int ww = 0; ww < HG; ++ww) sacc += kred[ww];
    kl_row[t] = (float)sacc;
  }
}

// ---------------------------------------------------------------- loss
__global__ __launch_bounds__(1024) void loss_reduce_kernel(const float *__restrict__ kl_row, int T,
                                                           int per_token, float *__restrict__ loss) {
  __shared__ double part[16];
  double s = 0.0;
  // eight loads in flight per thread, then added in index order (a fixed order per T)
  int i = threadIdx.x;
  for (; i + 7 * 1024 < T; i += 8 * 1024) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = kl_row[i + u * 1024];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += (double)v[u];
  }
  for (; i < T; i += 1024) s += (double)kl_row[i];
  s = wave_sum_f64_dpp(s);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x < 64) {
    double v = threadIdx.x < 16 ? part[threadIdx.x] : 0.0;
    v = wave_sum_f64_dpp(v);
    if (threadIdx.x == 0) loss[0] = (float)(per_token ? v : (T > 0 ? v / (double)T : 0.0));
  }
}

bool dense_teacher_supported(bool bf16, int H, int D, int max_seqlen_k) {
  if (!bf16 || H < 1 || H > 128 || max_seqlen_k > 8192) return false;
  if (!(D == 64 || D == 128 || D == 192 || D == 256 || D == 512)) return false;
  // dynamic LDS: two staged key tiles plus the row's head-summed masses (static: < 4 KiB)
  return (size_t)2 * 32 * D * 2 + (size_t)max_seqlen_k * sizeof(float) <= 156 * 1024;
}

template <int D>
static hipError_t launch_dense(const LaunchLayout &LL, const float *scores, int64_t ld, const void *q,
                               const void *ckv, const float *lse_nc, int H, float scale,
                               float *teacher, int64_t ldt, float *kl_row, hipStream_t st) {
  // two head groups of 16 per wave where the registers allow it: every K operand read
  // from LDS then feeds two MFMAs
  constexpr int NG = 2;
  const int hg = (H + 16 * NG - 1) / (16 * NG);
  const size_t lds = (size_t)2 * 32 * D * 2 + (size_t)LL.max_seqlen_k * sizeof(float);
  const float sl2 = scale * LOG2E;
#define CSA_DN_CASE(G)                                                                              \
  if (hg <= G) {                                                                                    \
    if (lds > 65536) {                                                                              \
      const hipError_t ea = hipFuncSetAttribute(                                                    \
          reinterpret_cast<const void *>(teacher_kl_dense_kernel<D, G, NG>),                            \
          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);                                    \
      if (ea != hipSuccess) return ea;                                                              \
    }                                                                                               \
    hipLaunchKernelGGL((teacher_kl_dense_kernel<D, G, NG>), dim3((unsigned)LL.total_q), dim3(64 * G), \
                       lds, st, LL.dev, scores, ld, static_cast<const uint16_t *>(q),               \
                       static_cast<const uint16_t *>(ckv), lse_nc, H, sl2, teacher, ldt, kl_row);   \
    return hipGetLastError();                                                                       \
  }
  CSA_DN_CASE(1)
  CSA_DN_CASE(2)
  CSA_DN_CASE(4)
  CSA_DN_CASE(8)
#undef CSA_DN_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_teacher_kl(const LaunchLayout &LL, bool sparse, const float *scores, int64_t ld,
                             bool selected, const int32_t *ids, int k_eff, const float *cmass, const void *q,
                             const void *ckv, const float *lse_nc, bool bf16, int H, int D,
                             float scale, bool per_token, float *teacher, int64_t ld_teacher,
                             float *kl_row, float *loss, hipStream_t st) {
  hipError_t e = hipSuccess;
  if (LL.total_q > 0) {
    if (sparse) {
      // slots per lane of a one-wave row; rows longer than 8 * 64 slots are shared by
      // 2 or 4 waves (up to 16 slots per lane at 4 waves: k_eff <= 4096)
      const int spl = (k_eff + 63) / 64;
#define CSA_TKS_CASE(V, NW)                                                                          \
      if (spl <= V * NW) {                                                                           \
        const dim3 grid((unsigned)((LL.total_q + 4 / NW - 1) / (4 / NW)));                          \
        hipLaunchKernelGGL((teacher_kl_sparse_kernel<V, NW>), grid, dim3(256), 0, st, LL.dev,        \
                           LL.total_q, scores, ld, selected ? 1 : 0, ids, k_eff, cmass, teacher,     \
                           ld_teacher, kl_row);                                                      \
        e = hipGetLastError();                                                                       \
      } else
      CSA_TKS_CASE(1, 1) CSA_TKS_CASE(2, 1) CSA_TKS_CASE(4, 1) CSA_TKS_CASE(8, 1) CSA_TKS_CASE(8, 2)
      CSA_TKS_CASE(8, 4) CSA_TKS_CASE(16, 4) { return hipErrorInvalidValue; }
#undef CSA_TKS_CASE
    } else {
      (void)bf16;
      switch (D) {
        case 64: e = launch_dense<64>(LL, scores, ld, q, ckv, lse_nc, H, scale, teacher, ld_teacher, kl_row, st); break;
        case 128: e = launch_dense<128>(LL, scores, ld, q, ckv, lse_nc, H, scale, teacher, ld_teacher, kl_row, st); break;
        case 192: e = launch_dense<192>(LL, scores, ld, q, ckv, lse_nc, H, scale, teacher, ld_teacher, kl_row, st); break;
        case 256: e = launch_dense<256>(LL, scores, ld, q, ckv, lse_nc, H, scale, teacher, ld_teacher, kl_row, st); break;
        case 512: e = launch_dense<512>(LL, scores, ld, q, ckv, lse_nc, H, scale, teacher, ld_teacher, kl_row, st); break;
        default: return hipErrorInvalidValue;
      }
    }
    if (e != hipSuccess) return e;
  }
  if (loss == nullptr) return hipSuccess;   // the caller reduces kl_row itself
  return launch_loss_reduce(kl_row, LL.total_q, per_token, loss, st);
}

hipError_t launch_loss_reduce(const float *kl_row, int T, bool per_token, float *loss, hipStream_t st) {
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(1024), 0, st, kl_row, T, per_token ? 1 : 0, loss);
  return hipGetLastError();
}

}  // namespace csa
