// Indexer-loss backward: gradients for the indexer q, weights and k.
//
// The step after the forward path (page "[Bug] DSV4 unfused CSA indexer loss uses a
// compressed-only teacher ...": the proposal comment keeps a custom backward that
// recomputes from saved tensors and returns gradients only for the indexer q, weights
// and k, the teacher being detached; page "Megatron-LM pull request 8539", item 1: the
// sparse path's ids are global).  The kernels:
//
//  1. score gradients, one wave per row: with the forward's predictor p = softmax of the
//     scores over the support and the given teacher t,
//        g_j = c (p_j R - r_j),  r_j = t_j p_j / (p_j + 1e-10),  R = sum_j r_j,
//     written densely into G[t, 0..W) (0 off the support), W = the key tiles that the
//     row's 16-token block reaches -- every column the next two kernels read (the sparse
//     mode writes the zeros, waits for them, then scatters).  Normalisers and g in fp64,
//     like the forward's KL.
//  2. dq / dweights.  Sparse loss: per token, its selected key rows gathered 32 at a time
//     (idx_bwd_dq_sparse_kernel, heads in the place of tokens below).  Dense loss: one
//     workgroup per 16-token block: for every 64-key tile below the block's causal limit
//     and every indexer head h, D^T = K Q_h^T (keys x tokens) is recomputed on MFMA,
//     E = G o [D > 0], and U_h^T += K^T E on MFMA; at the end dq = ws * U and
//     dweights = s_idx * sum_j G max(D, 0).
//  3. dk, one workgroup per (128-key tile of a segment, chunk of 16-token blocks) (wave =
//     2 x 16 keys): for every block of the chunk with a token that sees the tile,
//     D = Q_h K^T, E'' = G * ws o [D > 0], and dK^T += Q_h^T E'' on MFMA, summed over
//     heads and blocks in a fixed order.  With more than one chunk per tile each chunk
//     writes its partial to the caller's workspace and a fourth kernel adds the partials
//     of every key in chunk order (in fp64).
//
// The gradient factors E are fp32; they enter the bf16 MFMAs as a hi/lo pair
// (hi = bf16(E), lo = bf16(E - hi)), so every product carries ~16 significant bits of E
// and the bf16 inputs exactly, with fp32 accumulation.  Transposed operands (K^T, Q_h^T)
// come from LDS through the transposing 64-bit read.  No atomics: every output element
// is written once, in a fixed summation order.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "../launch.h"

namespace csa {

constexpr float BWD_EPS = 1e-10f;   // the KL's epsilon
constexpr int BWD_TOK = 16;         // tokens per block
constexpr int DK_TILE = 128;        // keys per dk workgroup (4 waves x 32)
static_assert(DK_TILE % 64 == 0, "G is zeroed in DK_TILE steps, which must cover the 64-key dq tiles");

// bf16 hi/lo split of four fp32 values, as two 16x16x16 MFMA operands
__device__ __forceinline__ void split_bf16x4(const float (&x)[4], uint2 &hi, uint2 &lo) {
  hi = uint2{pack2_bf16(x[0], x[1]), pack2_bf16(x[2], x[3])};
  const float r0 = x[0] - bf16_lo(hi.x), r1 = x[1] - bf16_hi(hi.x);
  const float r2 = x[2] - bf16_lo(hi.y), r3 = x[3] - bf16_hi(hi.y);
  lo = uint2{pack2_bf16(r0, r1), pack2_bf16(r2, r3)};
}

// the same for eight values, as the K = 32 MFMA operands
__device__ __forceinline__ void split_bf16x8(const float (&x)[8], u32x4 &hi, u32x4 &lo) {
  uint2 h0, l0, h1, l1;
  split_bf16x4({x[0], x[1], x[2], x[3]}, h0, l0);
  split_bf16x4({x[4], x[5], x[6], x[7]}, h1, l1);
  hi = u32x4{h0.x, h0.y, h1.x, h1.y};
  lo = u32x4{l0.x, l0.y, l1.x, l1.y};
}

// ---------------------------------------------------------------- 1. score gradients
// SPL support slots per lane: sparse -> k_eff slots (slot j <-> ids[t, j]); dense ->
// columns j < max_seqlen_k
template <int SPL>
__global__ __launch_bounds__(256) void grad_scores_kernel(
    LayoutDev L, int T, int sparse, const float *__restrict__ scores, int64_t ld, int selected,
    const int32_t *__restrict__ ids, int k_eff, const float *__restrict__ teacher, int64_t ldt,
    float gscale, float *__restrict__ grad, int64_t ldg, int max_sk) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;
  if (t >= T) return;
  const RowGeo geo = row_geo(L, t);
  float *gr = grad + (int64_t)t * ldg;
  const int nslot = sparse ? k_eff : max_sk;
  // columns read later: the key tiles (64 keys in the dq kernel, DK_TILE in the dk
  // kernel) below the causal limit of the row's 16-token block (its last token sees the
  // most keys); every one of them must hold g or 0
  const int last = min(((t - geo.q_start) / BWD_TOK) * BWD_TOK + BWD_TOK, geo.q_len) - 1;
  const int off = seg_offset(L, geo.seg, geo.q_len, geo.s_k);
  const int nvl = n_valid_of(last, off, L.ratio, geo.s_k);
  const int wcols = min(max_sk, (nvl + DK_TILE - 1) / DK_TILE * DK_TILE);
  auto zero_cols = [&]() {   // G[t, 0..wcols) = 0: 16-byte stores where the row allows
    const int wv = (reinterpret_cast<uintptr_t>(gr) & 15) == 0 ? (wcols & ~3) : 0;
    for (int j = 4 * lane; j < wv; j += 256) *reinterpret_cast<f32x4 *>(gr + j) = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = wv + lane; j < wcols; j += 64) gr[j] = 0.f;
  };
  int col[SPL];
  float s[SPL], te[SPL];
  float mx = -__builtin_inff();
#pragma unroll
  for (int v = 0; v < SPL; ++v) {
    const int j = v * 64 + lane;
    bool valid;
    if (sparse) {
      const int id = j < k_eff ? ids[(int64_t)t * k_eff + j] : -1;
      valid = id >= 0;
      col[v] = id - geo.k_base;
    } else {
      valid = j < geo.n_valid;
      col[v] = j;
    }
    if (!valid) col[v] = -1;
    // sparse + selected: the score of slot j sits at column j of the selected-score row
    s[v] = valid ? scores[(int64_t)t * ld + (selected ? j : col[v])] : -__builtin_inff();
    te[v] = valid ? teacher[(int64_t)t * ldt + j] : 0.f;
    mx = fmaxf(mx, s[v]);
  }
  if (loss_row_empty(L, geo, t)) {
    zero_cols();
    return;
  }
  mx = wave_max_dpp(mx);
  float e[SPL];
  double es = 0.0;
#pragma unroll
  for (int v = 0; v < SPL; ++v) {
    e[v] = col[v] >= 0 ? fast_exp2((s[v] - mx) * LOG2E) : 0.f;
    es += (double)e[v];
  }
  es = wave_sum_f64_dpp(es);
  const double inv_es = 1.0 / es;
  double rs = 0.0;
#pragma unroll
  for (int v = 0; v < SPL; ++v) {
    const double pv = (double)e[v] * inv_es;
    rs += (double)te[v] * pv / (pv + (double)BWD_EPS);
  }
  rs = wave_sum_f64_dpp(rs);
  float gval[SPL];
#pragma unroll
  for (int v = 0; v < SPL; ++v) {
    const double pv = (double)e[v] * inv_es;
    const double rv = (double)te[v] * pv / (pv + (double)BWD_EPS);
    gval[v] = (float)((double)gscale * (pv * rs - rv));
  }
  if (sparse) {
    zero_cols();
    wait_vmcnt<0>();   // the zeros have landed before any lane scatters over them
#pragma unroll
    for (int v = 0; v < SPL; ++v)
      if (col[v] >= 0) gr[col[v]] = gval[v];
  } else {
#pragma unroll
    for (int v = 0; v < SPL; ++v) {
      const int j = v * 64 + lane;
      if (j < nslot && j < wcols) gr[j] = col[v] >= 0 ? gval[v] : 0.f;
    }
  }
}

// ---------------------------------------------------------------- shared LDS staging
// Bytes [col0, col0 + PB) of the rows row0 .. row0+15 of a tensor with RB-byte rows ->
// LDS (PB bytes per row), 16-byte chunk q of row r at slot r*(PB/16) + (q ^ r) (rows past
// the end of the buffer read as zeros).  One instruction moves 1 KiB: a part of one row
// (PB >= 1 KiB) or whole rows (PB < 1 KiB).  Waves w, w + nw, ... of the workgroup share it.
template <int RB, int PB>
__device__ __forceinline__ void dma_rows(const uint16_t *base, int row0, int total_rows, int col0, char *dst,
                                         int w, int nw, int lane) {
  constexpr int CPP = PB / 16;
  static_assert(CPP >= BWD_TOK && (PB % 512) == 0, "the XOR swizzle needs 16-chunk rows");
  // uniform, but v_med3 computes it in a VGPR: without readfirstlane the descriptor is
  // taken as divergent and every load below gets a waterfall loop
  const int rows_left = __builtin_amdgcn_readfirstlane(max(min(BWD_TOK, total_rows - row0), 0));
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(base + (int64_t)row0 * (RB / 2), (uint32_t)(rows_left * RB));
  if constexpr (PB >= 1024) {
    constexpr int IPR = PB / 1024;
    for (int m = w; m < BWD_TOK * IPR; m += nw) {
      const int r = m / IPR, q0 = (m - r * IPR) * 64;
      dma16(rq, dst + (size_t)(r * CPP + q0) * 16, (uint32_t)(r * RB + col0 + (((q0 + lane) ^ r) << 4)));
    }
  } else {
    constexpr int RPI = 1024 / PB;
    for (int m = w; m < BWD_TOK / RPI; m += nw) {
      const int r = m * RPI + lane / CPP, c = lane % CPP;
      dma16(rq, dst + (size_t)m * 1024, (uint32_t)(r * RB + col0 + ((c ^ r) << 4)));
    }
  }
}

template <int RB>
__device__ __forceinline__ void dma_q_block(const uint16_t *q_idx, int row0, int total_q, char *dst,
                                            int w, int nw, int lane) {
  dma_rows<RB, RB>(q_idx, row0, total_q, 0, dst, w, nw, lane);
}

// ---------------------------------------------------------------- 2. dq / dweights
// A workgroup takes HW of the HI heads (head group hg of HI / HW; the q slice of those
// heads, HW * DI * 2 bytes of each token row, is what it stages); HPW heads per wave per
// pass; 4 waves; passes = HW / (4 * HPW).  The head groups of a token block are
// independent: each recomputes the block's key tiles for its own heads.
template <int DI, int HI, int HPW, int HW>
__global__ __launch_bounds__(256) void idx_bwd_dq_kernel(
    LayoutDev L, const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ k_idx,
    const float *__restrict__ weights, float idx_scale, const float *__restrict__ grad, int64_t ldg,
    int max_sk, int total_q, int nqb, float *__restrict__ dq, float *__restrict__ dw) {
  constexpr int RB = HI * DI * 2;      // bytes of a token's q row
  constexpr int SB = HW * DI * 2, CPR = SB / 16;   // staged bytes of it
  static_assert(HI % HW == 0, "head groups");
  constexpr int NCD = DI / 32;         // MFMA 16x16x32 K-chunks per dot product
  constexpr int NDT = DI / 16;         // 16-dim output tiles
  constexpr int ROWB = DI * 2;         // bytes per key row
  constexpr int PIECES = DI / 8, RPI = 64 / PIECES, NI = 64 / RPI;   // key-tile DMA shape
  constexpr int KT = 64 * ROWB;        // one 64-key tile
  constexpr int PASSES = HW / (4 * HPW);
  static_assert(HW % (4 * HPW) == 0, "heads per pass");
  __shared__ __attribute__((aligned(16))) u32x4 qs[BWD_TOK * CPR];
  __shared__ __attribute__((aligned(16))) char kt_lds[2][KT];

  const int seg = blockIdx.x % L.num_seqs;
  const int bi = (int)(blockIdx.x / L.num_seqs);
  const int hg0 = (bi % (HI / HW)) * HW;          // first head of the group
  const int qb = nqb - 1 - bi / (HI / HW);        // heaviest blocks first
  const int q_start = __ldg(L.cu_q + seg);
  const int q_len = __ldg(L.cu_q + seg + 1) - q_start;
  const int t0 = qb * BWD_TOK;
  if (t0 >= q_len) return;
  const int k_base = __ldg(L.cu_k + seg);
  const int s_k = __ldg(L.cu_k + seg + 1) - k_base;
  const int off = seg_offset(L, seg, q_len, s_k);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nv_last = n_valid_of(min(t0 + BWD_TOK, q_len) - 1, off, L.ratio, s_k);
  const int nlive = (nv_last + 63) / 64;
  const int t = t0 + r16;              // this lane's token (C / B operand column)
  const bool t_ok = t < q_len;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k_idx + (int64_t)k_base * DI, (uint32_t)(max(s_k, 0) * ROWB));

  dma_rows<RB, SB>(q_idx, q_start + t0, total_q, hg0 * DI * 2, reinterpret_cast<char *>(qs), w, 4, lane);
  // key tile kt -> buffer b: NI instructions of RPI rows, dealt over the 4 waves
  const int kgg = lane / PIECES, kpp = lane % PIECES;
  auto dma_k = [&](int kt, int b) {
    for (int i = w; i < NI; i += 4) {
      const int R = i * RPI + kgg, j = kt * 64 + R;
      const uint32_t o = j < s_k ? (uint32_t)j * ROWB + 16 * (kpp ^ row_swz<DI>(R)) : BUF_OOB;
      dma16(rk, kt_lds[b] + i * 1024, o);
    }
  };
  const char *qrow = reinterpret_cast<const char *>(qs) + r16 * SB;
  auto a_frag = [&](int h, int c) -> u32x4 {   // Q_h^T operand (h within the group): token r16, piece 4c+g
    const int q = h * (DI / 8) + 4 * c + g;
    return *reinterpret_cast<const u32x4 *>(qrow + ((q ^ r16) << 4));
  };

  for (int pass = 0; pass < PASSES; ++pass) {
    f32x4 u[HPW][NDT];
    float dwa[HPW];
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
      dwa[k] = 0.f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) u[k][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // G[t, j0 + 16m + 4g + i]: this lane's E^T entries of tile kt (0 past the row or
    // segment), loaded one tile ahead
    float gcur[4][4], gnext[4][4];
    auto load_g = [&](int kt, float (&dst)[4][4]) __attribute__((always_inline)) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = kt * 64 + 16 * m + 4 * g + i;
          dst[m][i] = (t_ok && j < max_sk) ? grad[(int64_t)(q_start + t) * ldg + j] : 0.f;
        }
    };
    if (nlive > 0) {
      dma_k(0, 0);
      load_g(0, gcur);
    }
    for (int kt = 0; kt < nlive; ++kt) {
      wait_vmcnt<0>();
      __syncthreads();   // tile kt (and, first time, the q block) visible to every wave
      if (kt + 1 < nlive) {
        dma_k(kt + 1, (kt + 1) & 1);
        load_g(kt + 1, gnext);
      }
      const char *kb = kt_lds[kt & 1];
#pragma unroll
      for (int mp = 0; mp < 2; ++mp) {   // 32 keys: sub-tiles m = 2mp, 2mp + 1
        // K row operands (rows 16m + r16) for D^T = K Q_h^T
        u32x4 ka[2][NCD];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int R = 16 * (2 * mp + s) + r16;
#pragma unroll
          for (int c = 0; c < NCD; ++c)
            ka[s][c] = *reinterpret_cast<const u32x4 *>(kb + R * ROWB + 16 * ((4 * c + g) ^ row_swz<DI>(R)));
        }
        // K^T operand of U^T += K^T E over 32 keys: MFMA k index 8g+e <-> key
        // 16m + 4g + e (e < 4, m = 2mp) or 16(m+1) + 4g + e-4 (e >= 4), two transposing
        // reads per dim tile
        u32x4 kt_op[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int piece = 2 * dt + ((r16 & 3) >> 1);
          uint2 h2[2];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const int rr = 16 * (2 * mp + s) + 4 * g + (r16 >> 2);
            h2[s] = lds_read_tr16(kb + rr * ROWB + 16 * (piece ^ row_swz<DI>(rr)) + 8 * (r16 & 1));
          }
          kt_op[dt] = u32x4{h2[0].x, h2[0].y, h2[1].x, h2[1].y};
        }
#pragma unroll
        for (int k = 0; k < HPW; ++k) {
          const int h = pass * 4 * HPW + k * 4 + w;   // within the group
          float e[8];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NCD; ++c) d = mfma16x16x32(ka[s][c], a_frag(h, c), d);
            const float *gv = gcur[2 * mp + s];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              e[4 * s + i] = d[i] > 0.f ? gv[i] : 0.f;
              dwa[k] = fmaf(gv[i], fmaxf(d[i], 0.f), dwa[k]);
            }
          }
          u32x4 ehi, elo;
          split_bf16x8(e, ehi, elo);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            u[k][dt] = mfma16x16x32(kt_op[dt], ehi, u[k][dt]);
            u[k][dt] = mfma16x16x32(kt_op[dt], elo, u[k][dt]);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) gcur[m][i] = gnext[m][i];
      __syncthreads();   // every wave is done with tile kt before it is overwritten
    }
    // outputs: lane (token r16, group g) holds dims 16dt + 4g + i of U_h^T
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
      const int h = hg0 + pass * 4 * HPW + k * 4 + w;
      float s = dwa[k];
      s += __shfl_xor(s, 16, 64);
      s += __shfl_xor(s, 32, 64);
      if (t_ok) {
        const int64_t row = (int64_t)(q_start + t) * HI + h;
        const float ws = weights[row] * idx_scale;
        float *dst = dq + row * DI + 4 * g;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          *reinterpret_cast<f32x4 *>(dst + 16 * dt) = u[k][dt] * ws;
        if (g == 0) dw[row] = s * idx_scale;
      }
    }
  }
}

// ---------------------------------------------------------------- 2'. dq / dweights, sparse loss
// With the sparse loss a token's score gradients are zero off its K_t selected keys, so
// this kernel gathers those key rows (as the attention does) instead of walking every key
// tile below the causal limit (at 2,048 of 16,384 keys, an eighth of the work).  Per token
// the products are the dense kernel's with heads in the place of tokens: D^T = K Q^T over
// a chunk of 32 selected keys (keys x heads), E = G o [D > 0], U^T += K^T E (the MFMA k
// index 8g + e <-> key 4g + e of the first 16-key tile, e < 4, or of the second, e >= 4,
// so that D^T's output layout is E's operand layout); dq = ws * U, dweights = s_idx *
// sum_j G max(D, 0).
// A workgroup of 4 waves takes SP_TOK = 4 / WPT tokens; the WPT waves of a token split
// its heads (32 each at Hi = 64) and share its LDS: the token's ids, two buffers of 32
// gathered key rows (16-byte pieces XOR-swizzled by row_swz) and two of the 32 gathered
// score gradients.  Each step: wait for the chunk's rows, one barrier, then the next
// chunk's gradient gather and row loads (in that order: the gather's value is waited for
// at the step's end without waiting for the rows), the products, the gradients into LDS.
constexpr int SP_CH = 32;   // selected keys per step
template <int DI, int HI>
struct SparseDqShape {
  static constexpr int WPT = HI == 64 ? 2 : 1;          // waves per token
  static constexpr int TOK = 4 / WPT;                   // tokens per workgroup
  static constexpr int HPW = HI / WPT;                  // heads per wave (<= 32)
  static constexpr int NHT = HPW > 16 ? 2 : 1;          // 16-head MFMA tiles per wave
  static constexpr int ROWB = DI * 2;
  static constexpr int RB = SP_CH * ROWB;               // one chunk of rows
  static constexpr int RPI = 1024 / ROWB;               // rows per 1 KiB load
  static constexpr int NLD = SP_CH / RPI;               // loads per chunk
  static_assert(NLD % WPT == 0, "the loads of a chunk split over the token's waves");
};
size_t sparse_dq_token_bytes(int DI, int k_eff) {
  const int nsl = (k_eff + SP_CH - 1) / SP_CH * SP_CH;
  return (size_t)2 * SP_CH * DI * 2 + (size_t)2 * SP_CH * 4 + (size_t)nsl * 4;
}

template <int DI, int HI>
__global__ __launch_bounds__(256) void idx_bwd_dq_sparse_kernel(
    LayoutDev L, const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ k_idx,
    const float *__restrict__ weights, float idx_scale, const int32_t *__restrict__ ids, int k_eff,
    const float *__restrict__ grad, int64_t ldg, int total_q, int total_k, float *__restrict__ dq,
    float *__restrict__ dw) {
  using S = SparseDqShape<DI, HI>;
  constexpr int NCD = DI / 32, NDT = DI / 16, PIECES = DI / 8;
  extern __shared__ __attribute__((aligned(16))) char sp_dyn[];
  __shared__ int nch_wg;
  const int nsl = (k_eff + SP_CH - 1) / SP_CH * SP_CH;
  const int tokb = 2 * S::RB + 2 * SP_CH * 4 + nsl * 4;   // bytes per token (a multiple of 16)
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tk = w / S::WPT, wt = w % S::WPT;             // token of the workgroup, wave within it
  const int t = total_q - 1 - ((int)blockIdx.x * S::TOK + tk);   // the longest rows first
  const bool t_ok = t >= 0;
  char *rows = sp_dyn + tk * tokb;                         // [2][SP_CH][ROWB]
  float *gbuf = reinterpret_cast<float *>(rows + 2 * S::RB);   // [2][SP_CH]
  int *ids_l = reinterpret_cast<int *>(gbuf + 2 * SP_CH);       // [nsl]
  const int tq = t_ok ? t : 0;
  const RowGeo geo = row_geo(L, tq);

  // the token's ids (-1 past k_eff or for a token past the end) and its last valid slot
  if (tid == 0) nch_wg = 0;
  __syncthreads();
  {
    const __amdgpu_buffer_rsrc_t rid = make_rsrc(ids + (int64_t)tq * k_eff, t_ok ? (uint32_t)k_eff * 4 : 0u);
    int jl = -1;
    for (int j = 64 * wt + lane; j < nsl; j += 64 * S::WPT) {
      const int x = __builtin_amdgcn_raw_buffer_load_b32(rid, j * 4, 0, 0);
      const int id = j < k_eff && t_ok ? x : -1;
      ids_l[j] = id;
      jl = id >= 0 ? j : jl;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) jl = max(jl, __shfl_xor(jl, m, 64));
    if (lane == 0 && jl >= 0) atomicMax(&nch_wg, jl / SP_CH + 1);
  }
  // Q^T operands of the wave's head tiles: piece c of lane group g holds features
  // [(4c + g) 8, +8) of head h0 + 16 ht + r16 (a head past the wave's loads head 0's row:
  // its outputs are not written)
  const int h0 = wt * S::HPW;
  u32x4 qf[S::NHT][NCD];
#pragma unroll
  for (int ht = 0; ht < S::NHT; ++ht) {
    const int hl = 16 * ht + r16;
    const int h = hl < S::HPW ? h0 + hl : 0;
    const u32x4 *p = reinterpret_cast<const u32x4 *>(q_idx + ((int64_t)tq * HI + h) * DI) + g;
#pragma unroll
    for (int c = 0; c < NCD; ++c) qf[ht][c] = p[4 * c];
  }
  __syncthreads();   // ids and nch_wg
  const int nch = nch_wg;   // steps of every token of the workgroup (its longest)
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k_idx, (uint32_t)total_k * S::ROWB);   // id -1: past the end
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(grad + (int64_t)tq * ldg, t_ok ? (uint32_t)ldg * 4 : 0u);
  // the score gradient of slot 32 c + (lane & 31) (0 at a -1 slot): one load per lane of
  // the token's first wave
  auto g_load = [&](int c) -> float {
    const int id = ids_l[SP_CH * c + (lane & 31)];
    const uint32_t off = id >= 0 ? (uint32_t)(id - geo.k_base) * 4 : BUF_OOB;
    return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rg, (int)off, 0, 0));
  };
  // rows of chunk c into buffer c & 1: load k (of NLD) moves rows k RPI .. k RPI + RPI - 1,
  // lane l writes piece l % PIECES of row k RPI + l / PIECES at slot piece ^ row_swz(row)
  const int kgg = lane / PIECES, kpp = lane % PIECES;
  auto rows_load = [&](int c) {
    char *dst = rows + (c & 1) * S::RB;
#pragma unroll
    for (int k = wt; k < S::NLD; k += S::WPT) {
      const int R = k * S::RPI + kgg;
      const int id = ids_l[SP_CH * c + R];
      const uint32_t o = id >= 0 ? (uint32_t)id * S::ROWB + 16 * (kpp ^ row_swz<DI>(R)) : BUF_OOB;
      dma16(rk, dst + k * 1024, o);
    }
  };
  if (nch > 0) {
    float gv0 = 0.f;
    if (wt == 0) gv0 = g_load(0);
    asm volatile("" ::: "memory");   // the gather before the row loads (waited for alone)
    rows_load(0);
    if (wt == 0 && lane < 32) gbuf[lane] = gv0;
  }

  f32x4 u[S::NHT][NDT];
  float dwa[S::NHT];
#pragma unroll
  for (int ht = 0; ht < S::NHT; ++ht) {
    dwa[ht] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) u[ht][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // K^T operand rows: lane (g, r16) reads row 4g + r16 / 4 (+ 16), 8 bytes at piece
  // 2 dt + ((r16 & 3) >> 1), half r16 & 1
  const int rr = 4 * g + (r16 >> 2);
  const int trb = rr * S::ROWB + 8 * (r16 & 1), trsw = row_swz<DI>(rr), trh = (r16 & 3) >> 1;
  for (int c = 0; c < nch; ++c) {
    wait_vmcnt<0>();   // the wave's rows of chunk c (the only loads in flight)
    lds_barrier();     // every wave's rows and the gradients of chunk c; chunk c - 1's buffers free
    float gnext = 0.f;
    if (c + 1 < nch) {
      if (wt == 0) gnext = g_load(c + 1);
      asm volatile("" ::: "memory");
      rows_load(c + 1);
    }
    const char *kb = rows + (c & 1) * S::RB;
    const float *gb = gbuf + (c & 1) * SP_CH;
    // D^T = K Q^T for the 32 keys (two 16-key tiles s) and the wave's head tiles
    f32x4 d[2][S::NHT];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int R = 16 * s + r16;
      u32x4 ka[NCD];
#pragma unroll
      for (int cc = 0; cc < NCD; ++cc)
        ka[cc] = *reinterpret_cast<const u32x4 *>(kb + R * S::ROWB + 16 * ((4 * cc + g) ^ row_swz<DI>(R)));
#pragma unroll
      for (int ht = 0; ht < S::NHT; ++ht) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < NCD; ++cc) acc = mfma16x16x32(ka[cc], qf[ht][cc], acc);
        d[s][ht] = acc;
      }
    }
    // G of keys 16 s + 4 g + i
    const f32x4 g0 = *reinterpret_cast<const f32x4 *>(gb + 4 * g);
    const f32x4 g1 = *reinterpret_cast<const f32x4 *>(gb + 16 + 4 * g);
    u32x4 ehi[S::NHT], elo[S::NHT];
#pragma unroll
    for (int ht = 0; ht < S::NHT; ++ht) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[i] = d[0][ht][i] > 0.f ? g0[i] : 0.f;
        e[4 + i] = d[1][ht][i] > 0.f ? g1[i] : 0.f;
        dwa[ht] = fmaf(g0[i], fmaxf(d[0][ht][i], 0.f), dwa[ht]);
        dwa[ht] = fmaf(g1[i], fmaxf(d[1][ht][i], 0.f), dwa[ht]);
      }
      split_bf16x8(e, ehi[ht], elo[ht]);
    }
    // K^T operands of the NDT dim tiles (one batch of transposing reads with its wait; the
    // rows requested ahead stay in flight)
    uint32_t ta[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) ta[dt] = lds_addr_of(kb + trb + 16 * ((2 * dt + trh) ^ trsw));
    uint2 tv[2 * NDT];
    lds_read_tr16_pairs<16 * S::ROWB, NDT>(tv, ta);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const u32x4 kt_op = u32x4{tv[2 * dt].x, tv[2 * dt].y, tv[2 * dt + 1].x, tv[2 * dt + 1].y};
#pragma unroll
      for (int ht = 0; ht < S::NHT; ++ht) {
        u[ht][dt] = mfma16x16x32(kt_op, ehi[ht], u[ht][dt]);
        u[ht][dt] = mfma16x16x32(kt_op, elo[ht], u[ht][dt]);
      }
    }
    if (wt == 0 && lane < 32 && c + 1 < nch) gbuf[((c + 1) & 1) * SP_CH + lane] = gnext;
  }
  wait_vmcnt<0>();   // no load into the LDS outlives the workgroup
  // outputs: lane (head r16 of tile ht, group g) holds dims 16 dt + 4 g + i of U^T
#pragma unroll
  for (int ht = 0; ht < S::NHT; ++ht) {
    float sdw = dwa[ht];
    sdw += __shfl_xor(sdw, 16, 64);
    sdw += __shfl_xor(sdw, 32, 64);
    const int hl = 16 * ht + r16;
    if (t_ok && hl < S::HPW) {
      const int64_t row = (int64_t)t * HI + h0 + hl;
      const float ws = weights[row] * idx_scale;
      float *dst = dq + row * DI + 4 * g;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4 *>(dst + 16 * dt) = u[ht][dt] * ws;
      if (g == 0) dw[row] = sdw * idx_scale;
    }
  }
}

// ---------------------------------------------------------------- 3. dk
// First 16-token block of a segment holding a token that sees key j0: n_valid(t) > j0
// exactly when the token's position i = t + 1 + off reaches (j0 + 1) * ratio.  The number
// of blocks if no token does.
__device__ __forceinline__ int first_block_seeing(int j0, int off, int ratio, int q_len) {
  const long long tmin = (long long)(j0 + 1) * ratio - 1 - off;
  if (tmin >= q_len) return (q_len + BWD_TOK - 1) / BWD_TOK;
  return tmin <= 0 ? 0 : (int)(tmin / BWD_TOK);
}

// grid: num_seqs x nkt x nsplit (segment fastest); a workgroup owns a DK_TILE-key tile
// (wave = two 16-key sub-tiles, so every LDS operand read feeds both) and the blocks
// [s*ch, (s+1)*ch) of split s that see it, and writes its sum to out + s*split_stride
// (split_stride 0 with one split: out is dk itself).  The blocks are taken in pairs, so
// that dK^T += Q_h^T E'' contracts 32 tokens per MFMA (the 16x16x32 form; MFMA k index
// 8g + e <-> token 4g + e of the pair's first block, e < 4, or of its second, e >= 4 --
// exactly the two blocks' D output layouts); a pair is taken in NG steps of HG heads, so
// only 2 x 16 rows x HG heads of q sit in each LDS buffer.  A second block past the
// workgroup's range contributes nothing (its G is 0).
template <int DI, int HI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void idx_bwd_dk_kernel(
    LayoutDev L, const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ k_idx,
    const float *__restrict__ weights, float idx_scale, const float *__restrict__ grad, int64_t ldg,
    int total_q, int nkt, int ch, int64_t split_stride, float *__restrict__ out) {
  constexpr int RB = HI * DI * 2;
  constexpr int HG = HI < 512 / DI ? HI : 512 / DI;   // heads per step
  constexpr int NG = HI / HG, PB = HG * DI * 2;       // steps per block, bytes per staged row
  constexpr int NCD = DI / 32, NDT = DI / 16;
  constexpr int QBLK = BWD_TOK * PB / 16;   // u32x4 of one staged block
  __shared__ __attribute__((aligned(16))) u32x4 qs[2][2 * QBLK];            // [buffer][block of the pair]
  __shared__ __attribute__((aligned(16))) float wsl[2][2][HI * BWD_TOK];   // [buffer][block][h][token]

  const int seg = blockIdx.x % L.num_seqs;
  const int rest = (int)(blockIdx.x / L.num_seqs);
  const int kt = rest % nkt, split = rest / nkt;
  const int k_base = __ldg(L.cu_k + seg);
  const int s_k = __ldg(L.cu_k + seg + 1) - k_base;
  const int j0 = kt * DK_TILE;
  if (j0 >= s_k) return;
  const int q_start = __ldg(L.cu_q + seg);
  const int q_len = __ldg(L.cu_q + seg + 1) - q_start;
  const int off = seg_offset(L, seg, q_len, s_k);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int jj[2];
  bool jok[2];
  u32x4 kb[2][NCD];   // key operand of D = Q_h K^T: key row jj[u], piece 4c+g
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    jj[u] = j0 + 32 * w + 16 * u + r16;
    jok[u] = jj[u] < s_k;
    const u32x4 *p = reinterpret_cast<const u32x4 *>(k_idx + (int64_t)(k_base + min(jj[u], s_k - 1)) * DI) + g;
#pragma unroll
    for (int c = 0; c < NCD; ++c) kb[u][c] = p[4 * c];
  }
  // this workgroup's blocks: those of its chunk from the first block that sees key j0
  const int b_lo = max(first_block_seeing(j0, off, L.ratio, q_len), split * ch);
  const int b_hi = min((q_len + BWD_TOK - 1) / BWD_TOK, (split + 1) * ch);
  f32x4 acc[2][NDT];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto store_out = [&]() __attribute__((always_inline)) {
    // lane (key r16 of sub-tile u, group g) holds dims 16dt + 4g + i of dK^T[:, key]
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (jok[u]) {
        float *dst = out + split * split_stride + (int64_t)(k_base + jj[u]) * DI + 4 * g;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4 *>(dst + 16 * dt) = acc[u][dt];
      }
  };
  if (b_lo >= b_hi) {
    if (split_stride == 0) store_out();   // a single chunk writes dk itself: zeros here
    return;
  }

  // per pair p: fp32(w * s_idx) through registers into wsl[p & 1] (loaded at the pair
  // before's first step, stored after its last), this lane's G[t0 + 4g + i, jj] of both
  // blocks (0 past the range or the segment) likewise one pair ahead; per step: the step's
  // q rows of both blocks by DMA into qs[step & 1], issued one step ahead
  const int npair = (b_hi - b_lo + 1) / 2;
  constexpr int WPT = (HI * BWD_TOK + 255) / 256;
  float wreg[2][WPT];
  auto load_w = [&](int p) __attribute__((always_inline)) {
#pragma unroll
    for (int bs = 0; bs < 2; ++bs) {
      const int b = b_lo + 2 * p + bs;
#pragma unroll
      for (int k = 0; k < WPT; ++k) {
        const int e = tid + 256 * k, tt = e / HI, h = e - tt * HI;
        const int t = b * BWD_TOK + tt;
        wreg[bs][k] = (e < HI * BWD_TOK && b < b_hi && t < q_len) ? weights[(int64_t)(q_start + t) * HI + h] : 0.f;
      }
    }
  };
  auto store_w = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int bs = 0; bs < 2; ++bs)
#pragma unroll
      for (int k = 0; k < WPT; ++k) {
        const int e = tid + 256 * k, tt = e / HI, h = e - tt * HI;
        if (e < HI * BWD_TOK) wsl[buf][bs][h * BWD_TOK + tt] = wreg[bs][k] * idx_scale;
      }
  };
  float gcur[2][2][4], gnext[2][2][4];   // [block][sub-tile][i]
  auto load_g = [&](int p, float (&dst)[2][2][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int bs = 0; bs < 2; ++bs) {
      const int b = b_lo + 2 * p + bs;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = b * BWD_TOK + 4 * g + i;
          dst[bs][u][i] = (b < b_hi && t < q_len && jok[u]) ? grad[(int64_t)(q_start + t) * ldg + jj[u]] : 0.f;
        }
    }
  };
  auto stage_q = [&](int st, int buf) __attribute__((always_inline)) {
    const int p = st / NG, hg = st - (st / NG) * NG;
#pragma unroll
    for (int bs = 0; bs < 2; ++bs)
      dma_rows<RB, PB>(q_idx, q_start + (b_lo + 2 * p + bs) * BWD_TOK, total_q, hg * PB,
                       reinterpret_cast<char *>(qs[buf] + bs * QBLK), w, 4, lane);
  };
  // the same loads one at a time (load k of the wave's NSL), spread over a step's heads: a
  // burst of them holds the issuing wave until the memory pipeline's queue takes them
  constexpr int RPL = PB >= 1024 ? 1 : 1024 / PB;       // rows per load
  constexpr int NSL = 2 * (BWD_TOK / RPL) * (PB >= 1024 ? PB / 1024 : 1) / 4;   // the wave's loads per step
  static_assert(NSL >= 1 && (NSL % HG == 0 || HG % NSL == 0), "loads per head");
  auto stage_q_part = [&](int st, int buf, int k) __attribute__((always_inline)) {
    const int p = st / NG, hg = st - (st / NG) * NG;
    constexpr int PERB = NSL / 2;                         // the wave's loads per block
    const int bs = k / PERB, m = w + 4 * (k - bs * PERB);   // load m of the block (dma_rows' order)
    const int row0 = q_start + (b_lo + 2 * p + bs) * BWD_TOK;
    const int rows_left = __builtin_amdgcn_readfirstlane(max(min(BWD_TOK, total_q - row0), 0));
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q_idx + (int64_t)row0 * (RB / 2), (uint32_t)(rows_left * RB));
    char *dst = reinterpret_cast<char *>(qs[buf] + bs * QBLK);
    constexpr int CPP = PB / 16;
    if constexpr (PB >= 1024) {
      constexpr int IPR = PB / 1024;
      const int r = m / IPR, q0 = (m - r * IPR) * 64;
      dma16(rq, dst + (size_t)(r * CPP + q0) * 16, (uint32_t)(r * RB + hg * PB + (((q0 + lane) ^ r) << 4)));
    } else {
      const int r = m * RPL + lane / CPP, c = lane % CPP;
      dma16(rq, dst + (size_t)m * 1024, (uint32_t)(r * RB + hg * PB + ((c ^ r) << 4)));
    }
  };
  stage_q(0, 0);
  load_w(0);
  load_g(0, gcur);
  store_w(0);
  const int nsteps = npair * NG;
  const int rr = 4 * g + (r16 >> 2);   // row this lane addresses in the transposing read
  // At DI >= 128 a head's 16-byte chunks are a multiple of 16 (DI / 8), so the swizzle (XOR
  // with a row < 16) leaves the head's part of a chunk index alone: an operand's LDS byte
  // offset is a per-lane part, the same for every head and step, plus 16 DI / 8 x the head.
  // Both parts are kept apart so the loop adds one uniform value per head.
  constexpr bool SPLIT = DI >= 128;
  uint32_t offq[NCD], offt[NDT];
#pragma unroll
  for (int c = 0; c < NCD; ++c) offq[c] = (uint32_t)(r16 * PB + (((4 * c + g) ^ r16) << 4));
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
    offt[dt] = (uint32_t)(rr * PB + (((2 * dt + ((r16 >> 1) & 1)) ^ rr) << 4) + 8 * (r16 & 1));
  for (int st = 0; st < nsteps; ++st) {
    const int p = st / NG, hg = st - p * NG;
    const bool more = p + 1 < npair;
    wait_vmcnt<0>();
    __syncthreads();   // step st staged (q rows by DMA; at a pair's first step its weights)
    if (hg == 0 && more) {
      load_w(p + 1);
      load_g(p + 1, gnext);
    }
    const char *qb = reinterpret_cast<const char *>(qs[st & 1]);
#pragma unroll 2
    for (int hh = 0; hh < HG; ++hh) {
      // the next step's q rows, NSL / HG loads per head (or one every HG / NSL heads)
      if (st + 1 < nsteps) {
        if constexpr (NSL >= HG) {
#pragma unroll
          for (int k = hh * (NSL / HG); k < (hh + 1) * (NSL / HG); ++k) stage_q_part(st + 1, (st + 1) & 1, k);
        } else if (hh % (HG / NSL) == 0) {
          stage_q_part(st + 1, (st + 1) & 1, hh / (HG / NSL));
        }
      }
      // D = Q_h K^T per block and sub-tile: A = Q_h rows (token r16, piece 4c+g), B = key
      // operand; lane (key r16, group g) holds D[token 4g + i][key]
      f32x4 d[2][2] = {{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}};
#pragma unroll
      for (int bs = 0; bs < 2; ++bs) {
        const char *qrow = qb + bs * BWD_TOK * PB + r16 * PB;
#pragma unroll
        for (int c = 0; c < NCD; ++c) {
          const int q = hh * (DI / 8) + 4 * c + g;
          const u32x4 qa = SPLIT ? *reinterpret_cast<const u32x4 *>(qb + bs * BWD_TOK * PB + hh * (2 * DI) + offq[c])
                                 : *reinterpret_cast<const u32x4 *>(qrow + ((q ^ r16) << 4));
          d[bs][0] = mfma16x16x32(qa, kb[0][c], d[bs][0]);
          d[bs][1] = mfma16x16x32(qa, kb[1][c], d[bs][1]);
        }
      }
      const int wo = (hg * HG + hh) * BWD_TOK + 4 * g;
      const f32x4 wv0 = *reinterpret_cast<const f32x4 *>(&wsl[p & 1][0][wo]);
      const f32x4 wv1 = *reinterpret_cast<const f32x4 *>(&wsl[p & 1][1][wo]);
      u32x4 ehi[2], elo[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e[i] = d[0][u][i] > 0.f ? gcur[0][u][i] * wv0[i] : 0.f;
          e[4 + i] = d[1][u][i] > 0.f ? gcur[1][u][i] * wv1[i] : 0.f;
        }
        split_bf16x8(e, ehi[u], elo[u]);
      }
      // Q_h^T operand (dims 16dt + r16 x the pair's tokens) by two transposing reads, one
      // per block (rows 16 apart: the same swizzle): lane supplies row 4g + r16/4, dims
      // 16dt + 4(r16%4) .. +3 of head h.  One batch with its own wait: the builtin read
      // would first wait for the next step's q rows in flight
      uint32_t ta[NDT];
      const uint32_t tbase = lds_addr_of(qb) + (uint32_t)(hh * (2 * DI));
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int col = hh * DI + 16 * dt + 4 * (r16 & 3);   // bf16 column in the staged row
        const int q = col >> 3;                               // 16-byte chunk
        ta[dt] = SPLIT ? tbase + offt[dt] : lds_addr_of(qb + rr * PB + ((q ^ rr) << 4) + 8 * ((col >> 2) & 1));
      }
      uint2 tv[2 * NDT];
      lds_read_tr16_pairs<BWD_TOK * PB, NDT>(tv, ta);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const u32x4 qt = u32x4{tv[2 * dt].x, tv[2 * dt].y, tv[2 * dt + 1].x, tv[2 * dt + 1].y};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          acc[u][dt] = mfma16x16x32(qt, ehi[u], acc[u][dt]);
          acc[u][dt] = mfma16x16x32(qt, elo[u], acc[u][dt]);
        }
      }
    }
    if (hg == NG - 1 && more) {
      store_w((p + 1) & 1);   // its last readers (pair p - 1) passed the barriers of pair p
#pragma unroll
      for (int bs = 0; bs < 2; ++bs)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) gcur[bs][u][i] = gnext[bs][u][i];
    }
    __syncthreads();   // every wave is done with qs[st & 1] before it is restaged
  }
  store_out();
}

// dk[key] = sum over the chunks that wrote a partial for the key's tile, in chunk order,
// in fp64 (one thread per element of a key row, so each load instruction reads 1 KiB of
// consecutive partial rows; eight chunks in flight; keys that no token sees get 0).
template <int DI>
__global__ __launch_bounds__(256) void idx_bwd_dk_reduce_kernel(LayoutDev L, int total_k, int ch,
                                                                const float *__restrict__ part,
                                                                int64_t split_stride,
                                                                float *__restrict__ dk) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)total_k * DI) return;
  const int key = (int)(e / DI);
  const int seg = segment_of(L.cu_k, L.num_seqs, key);
  const int k_base = __ldg(L.cu_k + seg);
  const int s_k = __ldg(L.cu_k + seg + 1) - k_base;
  const int q_start = __ldg(L.cu_q + seg);
  const int q_len = __ldg(L.cu_q + seg + 1) - q_start;
  const int off = seg_offset(L, seg, q_len, s_k);
  const int j0 = ((key - k_base) / DK_TILE) * DK_TILE;
  const int b_lo = first_block_seeing(j0, off, L.ratio, q_len);
  const int nqb = (q_len + BWD_TOK - 1) / BWD_TOK;
  double a = 0.0;
  if (b_lo < nqb) {
    const int s_end = (nqb - 1) / ch + 1;
    int s = b_lo / ch;
    const float *p = part + e;
    for (; s + 8 <= s_end; s += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)(s + u) * split_stride];
#pragma unroll
      for (int u = 0; u < 8; ++u) a += (double)v[u];
    }
    for (; s < s_end; ++s) a += (double)p[(int64_t)s * split_stride];
  }
  dk[e] = (float)a;
}

// ---------------------------------------------------------------- launch
// Chunks of token blocks per key tile: enough workgroups to fill the chip (about 1024),
// at least 4 and at most DK_MAX_CHUNK blocks per chunk.  The cap matters for long
// sequences: causality leaves only about half of the key tile x chunk workgroups with
// work, each the same length, and with chunks of hundreds of blocks their count lands
// just above the 512 the chip holds at once (two per CU), so a second round of a few
// runs on an idle chip; short chunks make it a smaller share of the whole.
constexpr int DK_MAX_CHUNK = 64;
void indexer_bwd_dk_split(int num_seqs, int max_seqlen_q, int max_seqlen_k, int *ch, int *ns) {
  const int nqb = (max_seqlen_q + BWD_TOK - 1) / BWD_TOK;
  const int nkt = (max_seqlen_k + DK_TILE - 1) / DK_TILE;
  const long long tiles = (long long)num_seqs * nkt;
  long long want = (1024 + tiles - 1) / tiles;
  want = std::max(1LL, std::min(want, (long long)(nqb + 3) / 4));
  const int c = (int)((nqb + want - 1) / want);
  *ch = std::min(std::max(c, 1), DK_MAX_CHUNK);
  *ns = (nqb + *ch - 1) / *ch;
}

int64_t indexer_bwd_workspace_bytes(int num_seqs, int total_k, int max_seqlen_q, int max_seqlen_k, int Di) {
  int ch, ns;
  indexer_bwd_dk_split(num_seqs, max_seqlen_q, max_seqlen_k, &ch, &ns);
  return ns > 1 ? (int64_t)ns * total_k * Di * (int64_t)sizeof(float) : 0;
}

// dq / dweights: the selected keys' rows gathered per token (sparse loss), else every
// causal key tile per 16-token block
template <int DI, int HI, int HPW, int HW = HI>
static hipError_t launch_bwd_t(const LaunchLayout &LL, bool sparse, const int32_t *ids, int k_eff,
                               const void *q_idx, const void *k_idx,
                               const float *weights, float idx_scale, const float *grad, int64_t ldg,
                               float *dq, float *dw, float *dk, float *ws, hipStream_t st) {
  const int nqb = (LL.max_seqlen_q + BWD_TOK - 1) / BWD_TOK;
  const int nkt = (LL.max_seqlen_k + DK_TILE - 1) / DK_TILE;
  int ch, ns;
  indexer_bwd_dk_split(LL.num_seqs, LL.max_seqlen_q, LL.max_seqlen_k, &ch, &ns);
  if (LL.total_q > 0 && sparse) {
    using S = SparseDqShape<DI, HI>;
    const size_t dyn = (size_t)S::TOK * sparse_dq_token_bytes(DI, k_eff);
    auto kern = idx_bwd_dq_sparse_kernel<DI, HI>;
    const hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (ea != hipSuccess) return ea;
    hipLaunchKernelGGL(kern, dim3((unsigned)((LL.total_q + S::TOK - 1) / S::TOK)), dim3(256), dyn, st, LL.dev,
                       static_cast<const uint16_t *>(q_idx), static_cast<const uint16_t *>(k_idx), weights,
                       idx_scale, ids, k_eff, grad, ldg, LL.total_q, LL.total_k, dq, dw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (LL.total_q > 0) {
    hipLaunchKernelGGL((idx_bwd_dq_kernel<DI, HI, HPW, HW>), dim3((unsigned)(LL.num_seqs * nqb * (HI / HW))),
                       dim3(256), 0, st,
                       LL.dev, static_cast<const uint16_t *>(q_idx), static_cast<const uint16_t *>(k_idx),
                       weights, idx_scale, grad, ldg, LL.max_seqlen_k, LL.total_q, nqb, dq, dw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t stride = ns > 1 ? (int64_t)LL.total_k * DI : 0;
  float *out = ns > 1 ? ws : dk;
  hipLaunchKernelGGL((idx_bwd_dk_kernel<DI, HI>), dim3((unsigned)((int64_t)LL.num_seqs * nkt * ns)), dim3(256),
                     0, st, LL.dev, static_cast<const uint16_t *>(q_idx), static_cast<const uint16_t *>(k_idx),
                     weights, idx_scale, grad, ldg, LL.total_q, nkt, ch, stride, out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ns == 1) return e;
  const int64_t nthr = (int64_t)LL.total_k * DI;
  hipLaunchKernelGGL(idx_bwd_dk_reduce_kernel<DI>, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, st, LL.dev,
                     LL.total_k, ch, ws, stride, dk);
  return hipGetLastError();
}

hipError_t launch_indexer_loss_bwd(const LaunchLayout &LL, bool sparse, const void *q_idx,
                                  const void *k_idx, const float *weights, int Hi, int Di,
                                  float idx_scale, const float *scores, int64_t ld_scores,
                                  bool selected, const int32_t *ids, int k_eff, const float *teacher,
                                  int64_t ld_teacher, float grad_scale, float *grad, int64_t ld_grad,
                                  float *dq, float *dw, float *dk, void *workspace, hipStream_t st) {
  if (LL.total_q > 0) {
    const int nslot = sparse ? k_eff : LL.max_seqlen_k;
    const dim3 grid((unsigned)((LL.total_q + 3) / 4));
#define CSA_GS_CASE(S)                                                                              \
    if (nslot <= 64 * S) {                                                                          \
      hipLaunchKernelGGL(grad_scores_kernel<S>, grid, dim3(256), 0, st, LL.dev, LL.total_q,         \
                         sparse ? 1 : 0, scores, ld_scores, selected ? 1 : 0, ids, k_eff, teacher,  \
                         ld_teacher,                                                                \
                         grad_scale, grad, ld_grad, LL.max_seqlen_k);                               \
    } else
    CSA_GS_CASE(1) CSA_GS_CASE(2) CSA_GS_CASE(4) CSA_GS_CASE(8) CSA_GS_CASE(16) CSA_GS_CASE(32)
    CSA_GS_CASE(64) { return hipErrorInvalidValue; }
#undef CSA_GS_CASE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
#define CSA_BWD_ARGS LL, sparse, ids, k_eff, q_idx, k_idx, weights, idx_scale, grad, ld_grad, dq, dw, dk, \
                     static_cast<float *>(workspace), st
  if (Di == 64) {
    switch (Hi) {
      case 4: return launch_bwd_t<64, 4, 1>(CSA_BWD_ARGS);
      case 8: return launch_bwd_t<64, 8, 2>(CSA_BWD_ARGS);
      case 16: return launch_bwd_t<64, 16, 4>(CSA_BWD_ARGS);
      case 32: return launch_bwd_t<64, 32, 4>(CSA_BWD_ARGS);
      case 64: return launch_bwd_t<64, 64, 4, 32>(CSA_BWD_ARGS);
    }
  } else if (Di == 128) {
    switch (Hi) {
      case 4: return launch_bwd_t<128, 4, 1>(CSA_BWD_ARGS);
      case 8: return launch_bwd_t<128, 8, 2>(CSA_BWD_ARGS);
      case 16: return launch_bwd_t<128, 16, 2>(CSA_BWD_ARGS);
      case 32: return launch_bwd_t<128, 32, 2, 16>(CSA_BWD_ARGS);
      case 64: return launch_bwd_t<128, 64, 2, 16>(CSA_BWD_ARGS);
    }
  }
#undef CSA_BWD_ARGS
  return hipErrorInvalidValue;
}

bool indexer_bwd_supported(bool bf16, int Hi, int Di, int k_eff, bool sparse, int max_seqlen_k) {
  if (!bf16) return false;
  if ((sparse ? k_eff : max_seqlen_k) > 64 * 64) return false;   // score-gradient slots per row
  if (Di == 64) return Hi == 4 || Hi == 8 || Hi == 16 || Hi == 32 || Hi == 64;
  if (Di == 128) return Hi == 4 || Hi == 8 || Hi == 16 || Hi == 32 || Hi == 64;
  return false;
}

// ---------------------------------------------------------------- the no-allocation route
// Device scratch of the backward for callers that cannot allocate: the score-gradient
// matrix G and the dk chunk partials live in this file-scope array instead of caller
// workspaces.  Each GPU the library runs on holds its own copy for the life of the
// process.  Host code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol); it passes the device address that hipGetSymbolAddress returns
// for the current device, looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};
}  // namespace

hipError_t noalloc_scratch_ptr(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// The scratch layout of a call: G [total_q, ld] fp32 with ld = max_seqlen_k rounded up to
// 64 floats, then the dk partials at the next 256-byte boundary.
NoallocPlan noalloc_plan(int num_seqs, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int Di) {
  NoallocPlan p;
  p.ld_grad = ((int64_t)max_seqlen_k + 63) / 64 * 64;
  p.ws_offset = ((int64_t)total_q * p.ld_grad * 4 + 255) / 256 * 256;
  p.bytes = p.ws_offset + indexer_bwd_workspace_bytes(num_seqs, total_k, max_seqlen_q, max_seqlen_k, Di);
  return p;
}

}  // namespace csa
