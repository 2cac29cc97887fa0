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
#include "wave_select.h"
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

// ============================================================================
// LDS-staged variant (bf16; Di = 64 with Hi*Di*2 in {1, 2, 4} KiB, or Di = 128 with
// Hi <= 8).  One workgroup (8 waves) = two 16-token blocks of one segment, paired
// heaviest with lightest (blocks p and nqb-1-p), so that every workgroup has about the
// same number of key tiles below the causal limit; the 64-key tiles of both blocks are
// dealt round-robin to the 8 waves.
//
// q_idx of a block is one contiguous run of 16 rows, read from HBM once: it is copied
// into LDS by buffer-load-to-LDS, each wave instruction moving 1 KiB of one row, so the
// reads are fully coalesced.  In LDS, 16-byte chunk q of token r sits at slot
// r*CPR + (q ^ r): a 1 KiB piece of a row maps onto itself under the XOR (r < 16), so
// lane i of the copy fetches chunk (q0 + i) ^ r and lands at slot q0 + i; when the MFMA
// A operand is read (lane (r, g) wants chunk h*Di/8 + 4c + g of token r) the 16 lanes of
// a group hit 16 different 16-byte bank groups.
//
// Per tile and head: Di/32 MFMAs per 16-key N-tile (the key tile sits in registers, the
// next one is prefetched), then the ReLU x fp32(w * s_idx) epilogue folded into the
// (token, key) accumulator; the MFMAs of head h+1 are issued between the epilogue
// instructions of head h.  Tiles entirely above the causal limit are only filled with
// -inf.
// ============================================================================
constexpr int IXL_TOK = 16;
constexpr int IXL_WAVES = 8;

// Outputs of the fused score + top-k variant (FUSED = true): the score tiles go to an LDS
// row area instead of HBM and each row is then selected there by one wave.
struct TopkOut {
  int32_t *ids;    // [T, k_eff] global ids, ascending, -1 tail
  float *sel;      // [T, k_eff] score of each selected key, -inf at -1 slots
  float *lse;      // [T] log-sum-exp of the row's visible scores (-inf if none), or null
  int k_eff;
  int cap;         // score area capacity in 64-key tiles per 16 rows
};

// max(x, 0) in one integer max on the bit pattern: a float with the sign bit set is a
// negative int32 (-> +0), a non-negative float keeps its bits
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

template <int DI, int HI, bool FUSED, int VPL>
__global__ __launch_bounds__(64 * IXL_WAVES) void indexer_score_lds_kernel(
    LayoutDev L, const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ k_idx,
    const float *__restrict__ weights, float idx_scale, float *__restrict__ scores, int64_t ld,
    int max_sk, int total_q, TopkOut to) {
  constexpr int RB = HI * DI * 2;   // bytes of one token's q_idx row
  constexpr int CPR = RB / 16;      // 16-byte chunks per row
  constexpr int PPR = RB / 1024;    // 1 KiB pieces per row
  constexpr int CH = DI / 8;        // 16-byte chunks per head
  constexpr int NCD = DI / 32;
  constexpr int NTHR = 64 * IXL_WAVES;
  static_assert(RB % 1024 == 0 && (2 * IXL_TOK * PPR) % IXL_WAVES == 0, "row of whole KiB pieces");
  static_assert(CH == 8 || CH == 16, "Di of 64 or 128");
  __shared__ __attribute__((aligned(16))) u32x4 qs[2][IXL_TOK * CPR];
  __shared__ __attribute__((aligned(16))) float ws[2][HI * IXL_TOK];
  // FUSED: score rows of the blocks of the current phase (row stride = live tiles * 64 + 4
  // floats, so the four token groups of a tile store hit different banks), then one
  // 256-word histogram per wave for the selection
  extern __shared__ __attribute__((aligned(16))) float score_lds[];

  const int seg = blockIdx.x % L.num_seqs;
  const int pair = blockIdx.x / L.num_seqs;
  const int q_start = __ldg(L.cu_q + seg);
  const int q_len = __ldg(L.cu_q + seg + 1) - q_start;
  const int nqb = (q_len + IXL_TOK - 1) / IXL_TOK;
  if (2 * pair >= nqb) return;
  const int nblk = (nqb - 1 - pair > pair) ? 2 : 1;
  const int tb0 = (nqb - 1 - pair) * IXL_TOK, tb1 = pair * IXL_TOK;  // first token of block 0 / 1
  const int k_base = __ldg(L.cu_k + seg);
  const int s_k = __ldg(L.cu_k + seg + 1) - k_base;
  const int off = seg_offset(L, seg, q_len, s_k);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntiles = (max_sk + 63) / 64;   // tiles of one output row
  auto nlive_of = [&](int t0) {             // tiles with a key below the causal limit
    return (n_valid_of(min(t0 + IXL_TOK, q_len) - 1, off, L.ratio, s_k) + 63) / 64;
  };
  const int nl0 = nlive_of(tb0), nl1 = nblk > 1 ? nlive_of(tb1) : 0;

  auto store_tile = [&](int t0, int jw, const f32x4 (&acc)[4], bool masked_only) {
    const int nv_first = n_valid_of(t0, off, L.ratio, s_k);
    if (!masked_only && t0 + IXL_TOK <= q_len && jw + 64 <= nv_first && jw + 64 <= max_sk) {
      // every key of the tile is below the causal limit of all 16 tokens
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float *dst = scores + (int64_t)(q_start + t0 + 4 * g + i) * ld + jw + r16;
#pragma unroll
        for (int n = 0; n < 4; ++n) dst[16 * n] = acc[n][i];
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * g + i;
      if (t >= q_len) continue;
      const int nv = n_valid_of(t, off, L.ratio, s_k);
      float *dst = scores + (int64_t)(q_start + t) * ld;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int j = jw + 16 * n + r16;
        if (j < max_sk) dst[j] = (!masked_only && j < nv) ? acc[n][i] : -__builtin_inff();
      }
    }
  };
  const f32x4 zero4[4] = {};
  // tiles above the causal limit: (block, tile) pairs dealt round-robin over the waves
  if constexpr (!FUSED) {
    const int nf0 = ntiles - nl0, nf = nf0 + (nblk > 1 ? ntiles - nl1 : 0);
    for (int v = w; v < nf; v += IXL_WAVES) {
      if (v < nf0) store_tile(tb0, (nl0 + v) * 64, zero4, true);
      else store_tile(tb1, (nl1 + v - nf0) * 64, zero4, true);
    }
  }
  const int nlive = nl0 + nl1;
  if constexpr (FUSED) {
    if (nlive == 0) {   // no row of either block sees a key: -1 ids, -inf scores and lse
      for (int bk = 0; bk < nblk; ++bk) {
        const int t0 = bk ? tb1 : tb0;
        for (int e = tid; e < IXL_TOK * to.k_eff; e += NTHR) {
          const int r = e / to.k_eff, c = e - r * to.k_eff;
          if (t0 + r < q_len) {
            to.ids[(int64_t)(q_start + t0 + r) * to.k_eff + c] = -1;
            to.sel[(int64_t)(q_start + t0 + r) * to.k_eff + c] = -__builtin_inff();
          }
        }
        if (to.lse && tid < IXL_TOK && t0 + tid < q_len) to.lse[q_start + t0 + tid] = -__builtin_inff();
      }
      return;
    }
  }
  if (nlive == 0) return;  // uniform: no barrier is skipped by part of the workgroup

  // q_idx rows of both blocks -> LDS (rows past the end of the buffer read as zeros)
#pragma unroll
  for (int bk = 0; bk < 2; ++bk) {
    if (bk < nblk) {
      const int t0 = bk ? tb1 : tb0;
      const int rows_left = min(IXL_TOK, total_q - (q_start + t0));
      const __amdgpu_buffer_rsrc_t rq =
          make_rsrc(q_idx + (int64_t)(q_start + t0) * (RB / 2), (uint32_t)(rows_left * RB));
#pragma unroll
      for (int k = 0; k < IXL_TOK * PPR / IXL_WAVES + (IXL_TOK * PPR % IXL_WAVES ? 1 : 0); ++k) {
        const int m = k * IXL_WAVES + w;   // wave instruction index: row r, piece p
        if (m < IXL_TOK * PPR) {
          const int r = m / PPR, q0 = (m - r * PPR) * 64;
          dma16(rq, reinterpret_cast<char *>(qs[bk]) + (size_t)(r * CPR + q0) * 16,
                (uint32_t)(r * RB + (((q0 + lane) ^ r) << 4)));
        }
      }
    }
  }
  // live tile u of this workgroup: block 0 tiles first, then block 1
  auto tile_of = [&](int u, int &bk, int &tile) {
    bk = u >= nl0;
    tile = bk ? u - nl0 : u;
  };
  // key tile fragments (MFMA B operand: lane column r16 = key, piece 4c+g); keys past
  // the segment are clamped to its last key (their scores are masked)
  auto load_k = [&](int tile, u32x4 (&kb)[4][NCD]) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int j = min(tile * 64 + 16 * n + r16, s_k - 1);
      const u32x4 *kp = reinterpret_cast<const u32x4 *>(k_idx + (int64_t)(k_base + j) * DI) + g;
#pragma unroll
      for (int c = 0; c < NCD; ++c) kb[n][c] = kp[4 * c];
    }
  };
  u32x4 kb[4][NCD], kbn[4][NCD];
  if (w < nlive) {
    int bk, tile;
    tile_of(w, bk, tile);
    load_k(tile, kbn);
  }
  // fp32(w * s_idx), head-major: one 16-byte LDS read gives a lane its 4 tokens.  The
  // loads are unconditional (a token past the segment reads its last row, then is zeroed),
  // so all of a thread's are in flight at once
  {
    constexpr int NW8 = (2 * HI * IXL_TOK + NTHR - 1) / NTHR;
    float x[NW8];
#pragma unroll
    for (int k = 0; k < NW8; ++k) {
      const int e = tid + k * NTHR;
      const int bk = e >= HI * IXL_TOK, e2 = e - bk * HI * IXL_TOK;
      const int tt = e2 / HI, h = e2 - tt * HI;
      const int t = min((bk ? tb1 : tb0) + tt, q_len - 1);
      x[k] = e < 2 * HI * IXL_TOK ? weights[(int64_t)(q_start + t) * HI + h] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < NW8; ++k) {
      const int e = tid + k * NTHR;
      if (e < 2 * HI * IXL_TOK) {
        const int bk = e >= HI * IXL_TOK, e2 = e - bk * HI * IXL_TOK;
        const int tt = e2 / HI, h = e2 - tt * HI;
        const int t = (bk ? tb1 : tb0) + tt;
        ws[bk][h * IXL_TOK + tt] = (bk < nblk && t < q_len) ? x[k] * idx_scale : 0.f;
      }
    }
  }
  wait_vmcnt<0>();
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);

  // LDS address of A chunk (head h, piece c): chunk index h*CH + 4c + g, swizzled by
  // XOR with r16.  For CH = 16 the XOR only touches the piece bits; for CH = 8 it also
  // flips bit 0 of h when r16 >= 8, which is folded into two per-parity base offsets
  // so that h always ends up in the instruction's immediate offset.
  int abase[2][NCD];
#pragma unroll
  for (int c = 0; c < NCD; ++c) {
    const int x = 4 * c + g;
    if constexpr (CH == 16) {
      abase[0][c] = abase[1][c] = r16 * RB + ((x ^ r16) << 4);
    } else {
      const int hb = r16 >> 3, b0 = r16 * RB + ((x ^ (r16 & 7)) << 4);
      abase[0][c] = b0 + 128 * hb;   // even h: h ^ hb = h + hb
      abase[1][c] = b0 - 128 * hb;   // odd h:  h ^ hb = h - hb
    }
  }

  // FUSED: both blocks' rows in one phase when they fit the score area, else block 0 then
  // block 1 (each phase: its tiles, a barrier, the selection of its rows, a barrier)
  const bool one_phase = !FUSED || nl0 + nl1 <= to.cap;
  const int nphase = one_phase ? 1 : 2;
  const int str0 = nl0 * 64 + 4, str1 = nl1 * 64 + 4;   // row strides of the score area
  auto row_ptr = [&](int bk, int r) -> float * {
    return score_lds + (bk ? (one_phase ? IXL_TOK * str0 : 0) + r * str1 : r * str0);
  };
  for (int ph = 0; ph < nphase; ++ph) {
  const int u_lo = one_phase ? 0 : (ph ? nl0 : 0), u_hi = one_phase ? nlive : (ph ? nlive : nl0);
  if (ph > 0 && u_lo + w < u_hi) {   // phase 2: its first key tile (phase 1 stopped short)
    int bk, tile;
    tile_of(u_lo + w, bk, tile);
    load_k(tile, kbn);
  }
  for (int u = u_lo + w; u < u_hi; u += IXL_WAVES) {
    int bk, tile;
    tile_of(u, bk, tile);
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int c = 0; c < NCD; ++c) kb[n][c] = kbn[n][c];
    if (u + IXL_WAVES < u_hi) {
      int bk2, tile2;
      tile_of(u + IXL_WAVES, bk2, tile2);
      load_k(tile2, kbn);
    }
    __builtin_amdgcn_sched_barrier(0);

    const char *qb = reinterpret_cast<const char *>(qs[bk]);
    const float *wsp = ws[bk] + 4 * g;
    auto a_frag = [&](int h, u32x4 (&qa)[NCD]) {
#pragma unroll
      for (int c = 0; c < NCD; ++c)
        qa[c] = *reinterpret_cast<const u32x4 *>(qb + abase[h & 1][c] + h * CH * 16);
    };
    auto head_mfma = [&](const u32x4 (&qa)[NCD], f32x4 (&d)[4]) {
#pragma unroll
      for (int n = 0; n < 4; ++n) d[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NCD; ++c)
#pragma unroll
        for (int n = 0; n < 4; ++n) d[n] = mfma16x16x32(qa[c], kb[n][c], d[n]);
    };
    f32x4 acc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto epilogue = [&](const f32x4 (&d)[4], const f32x4 &wv) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[n][i] = fmaf(wv[i], relu_bits(d[n][i]), acc[n][i]);
        asm volatile("" : "+v"(acc[n]));  // the epilogue of head h stays in its iteration
      }
    };
    auto interleave = [&]() {
#pragma unroll
      for (int m = 0; m < 4 * NCD; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 32 / (4 * NCD), 0);  // then VALU
      }
    };
    // two register sets alternate between "MFMAs in flight" and "epilogue"
    u32x4 qa0[NCD], qa1[NCD];
    f32x4 d0[4], d1[4];
    a_frag(0, qa0);
    head_mfma(qa0, d0);
    if (HI > 1) a_frag(1, qa1);
#pragma unroll
    for (int h = 0; h < HI; h += 2) {
      const f32x4 w0 = *reinterpret_cast<const f32x4 *>(wsp + h * IXL_TOK);
      if (h + 1 < HI) {
        head_mfma(qa1, d1);
        if (h + 2 < HI) a_frag(h + 2, qa0);
      }
      epilogue(d0, w0);
      if (h + 1 < HI) interleave();
      __builtin_amdgcn_sched_barrier(0);
      if (h + 1 < HI) {
        const f32x4 w1 = *reinterpret_cast<const f32x4 *>(wsp + (h + 1) * IXL_TOK);
        if (h + 2 < HI) {
          head_mfma(qa0, d0);
          if (h + 3 < HI) a_frag(h + 3, qa1);
        }
        epilogue(d1, w1);
        if (h + 2 < HI) interleave();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (FUSED) {
      // lane (token 4g+i, key tile*64 + 16n + r16) -> the block's LDS score row
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float *dst = row_ptr(bk, 4 * g + i) + tile * 64 + r16;
#pragma unroll
        for (int n = 0; n < 4; ++n) dst[16 * n] = acc[n][i];
      }
    } else {
      store_tile(bk ? tb1 : tb0, tile * 64, acc, false);
    }
  }
  if constexpr (FUSED) {
    __syncthreads();   // every score tile of the phase is in LDS
    // rows of the phase, one wave per row: top-k, selected scores, log-sum-exp
    const int b_lo = one_phase ? 0 : ph, b_hi = one_phase ? nblk : ph + 1;
    uint32_t *hist = reinterpret_cast<uint32_t *>(
        score_lds + IXL_TOK * (one_phase ? str0 + (nblk > 1 ? str1 : 0) : max(str0, str1))) + 256 * w;
    for (int rr = w; rr < (b_hi - b_lo) * IXL_TOK; rr += IXL_WAVES) {
      const int bk = b_lo + rr / IXL_TOK, r = rr % IXL_TOK;
      const int t = (bk ? tb1 : tb0) + r;
      if (t >= q_len) continue;
      const int n = n_valid_of(t, off, L.ratio, s_k);
      const float *row = row_ptr(bk, r);
      float val[VPL];
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int j = v * 64 + lane;
        val[v] = j < n ? row[j] : -__builtin_inff();
      }
      const int64_t o = (int64_t)(q_start + t) * to.k_eff;
      if (to.lse) {
        float m = -__builtin_inff();
#pragma unroll
        for (int v = 0; v < VPL; ++v) m = fmaxf(m, val[v]);
        m = wave_max_dpp(m);
        double sum = 0.0;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
          if (v * 64 + lane < n) sum += (double)__expf(val[v] - m);
        sum = wave_sum_f64_dpp(sum);
        if (lane == 0) to.lse[q_start + t] = n > 0 ? m + (float)log(sum) : -__builtin_inff();
      }
      if (n <= to.k_eff) {   // every visible key is selected
        for (int c = lane; c < to.k_eff; c += 64) {
          to.ids[o + c] = c < n ? k_base + c : -1;
          to.sel[o + c] = c < n ? row[c] : -__builtin_inff();
        }
      } else {
        // the row's two outputs through buffer stores sharing one 32-bit offset
        const __amdgpu_buffer_rsrc_t rid = make_rsrc(to.ids + o, (uint32_t)to.k_eff * 4);
        const __amdgpu_buffer_rsrc_t rsel = make_rsrc(to.sel + o, (uint32_t)to.k_eff * 4);
        wave_select<VPL>(val, n, to.k_eff, hist, [&](int pos, int j, int v) {
          __builtin_amdgcn_raw_buffer_store_b32(k_base + j, rid, pos * 4, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val[v]), rsel, pos * 4, 0, 0);
        });
      }
    }
    __syncthreads();   // the score area is free for the next phase
  }
  }
}

template <int DI, int HI>
static hipError_t launch_lds(const LaunchLayout &LL, const void *q_idx, const void *k_idx,
                             const float *weights, float idx_scale, float *scores, int64_t ld,
                             hipStream_t st) {
  const int npair = ((LL.max_seqlen_q + IXL_TOK - 1) / IXL_TOK + 1) / 2;
  const int64_t grid = (int64_t)LL.num_seqs * npair;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((indexer_score_lds_kernel<DI, HI, false, 1>), dim3((unsigned)grid), dim3(64 * IXL_WAVES),
                     0, st, LL.dev, static_cast<const uint16_t *>(q_idx), static_cast<const uint16_t *>(k_idx),
                     weights, idx_scale, scores, ld, LL.max_seqlen_k, LL.total_q, TopkOut{});
  return hipGetLastError();
}

// ---------------------------------------------------------------- fused score + top-k
// Static LDS of the paired-block kernel (q rows of both blocks + fp32(w * s_idx)).
template <int DI, int HI> constexpr int lds_static_bytes() {
  return 2 * IXL_TOK * HI * DI * 2 + 2 * HI * IXL_TOK * 4;
}
constexpr int LDS_PER_CU = 160 * 1024;

// Score area: one phase holds the rows of both blocks when their live tiles fit `cap`
// tiles; a single block always fits (cap >= tiles of a row).  cap = one row's tiles + 1
// covers the usual pairing (a heavy and a light block of one causal segment).
static int fused_cap(int max_sk) { return (max_sk + 63) / 64 + 1; }
static int fused_dyn_bytes(int max_sk) {
  const int cap = fused_cap(max_sk);
  return (IXL_TOK * (cap * 64 + 8) + 256 * IXL_WAVES) * 4;
}

template <int DI, int HI, int VPL>
static hipError_t launch_fused_t(const LaunchLayout &LL, const void *q_idx, const void *k_idx,
                                 const float *weights, float idx_scale, const TopkOut &to, hipStream_t st) {
  const int npair = ((LL.max_seqlen_q + IXL_TOK - 1) / IXL_TOK + 1) / 2;
  const int64_t grid = (int64_t)LL.num_seqs * npair;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int dyn = fused_dyn_bytes(LL.max_seqlen_k);
  auto kern = indexer_score_lds_kernel<DI, HI, true, VPL>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, dyn);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * IXL_WAVES), dyn, st, LL.dev,
                     static_cast<const uint16_t *>(q_idx), static_cast<const uint16_t *>(k_idx), weights,
                     idx_scale, nullptr, (int64_t)0, LL.max_seqlen_k, LL.total_q, to);
  return hipGetLastError();
}

template <int DI, int HI>
static hipError_t launch_fused_v(const LaunchLayout &LL, const void *q_idx, const void *k_idx,
                                 const float *weights, float idx_scale, const TopkOut &to, hipStream_t st) {
  const int vpl = (LL.max_seqlen_k + 63) / 64;
  if (vpl <= 4) return launch_fused_t<DI, HI, 4>(LL, q_idx, k_idx, weights, idx_scale, to, st);
  if (vpl <= 8) return launch_fused_t<DI, HI, 8>(LL, q_idx, k_idx, weights, idx_scale, to, st);
  if (vpl <= 16) return launch_fused_t<DI, HI, 16>(LL, q_idx, k_idx, weights, idx_scale, to, st);
  if (vpl <= 32) return launch_fused_t<DI, HI, 32>(LL, q_idx, k_idx, weights, idx_scale, to, st);
  return hipErrorInvalidValue;
}


// ---------------------------------------------------------------- fused, head-grouped
// Fused score + top-k for q rows too long for the paired-block kernel to stage whole
// (HI * DI * 2 above 2 KiB: thd-varlen-16k's 32 x 64).  One workgroup (8 waves) per
// 16-token block, heaviest blocks first.  The heads are taken HGF at a time: the block's q
// slice of a head group is staged in LDS (chunk q of row r at slot q ^ r, as in the
// paired-block kernel), and every wave runs the group's heads over its key tiles,
// continuing each (token, key) accumulator from the block's LDS score row where the
// previous group left it -- so the heads are summed in the same order, with the same
// fused multiply-adds, as in the score kernels, and the scores are bit-identical.  Then
// one wave per row selects from LDS (wave_select, as in the paired-block kernel).
template <int DI, int HI, int HGF> constexpr int grouped_static_bytes() {
  return IXL_TOK * HGF * DI * 2 + HI * IXL_TOK * 4;
}

template <int DI, int HI, int HGF, int VPL>
__global__ __launch_bounds__(64 * IXL_WAVES) void indexer_topk_grouped_kernel(
    LayoutDev L, const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ k_idx,
    const float *__restrict__ weights, float idx_scale, int max_sk, int total_q, TopkOut to) {
  constexpr int RB = HI * DI * 2;     // bytes of one token's q_idx row
  constexpr int GB = HGF * DI * 2;    // bytes of it in one head group
  constexpr int CPG = GB / 16;        // 16-byte chunks per staged row
  constexpr int PPG = GB / 1024;      // 1 KiB pieces per staged row
  constexpr int CH = DI / 8;          // 16-byte chunks per head
  constexpr int NCD = DI / 32;
  constexpr int NG = HI / HGF;
  constexpr int NTHR = 64 * IXL_WAVES;
  static_assert(HI % HGF == 0 && GB % 1024 == 0 && CPG >= 16, "head groups of whole KiB pieces");
  __shared__ __attribute__((aligned(16))) u32x4 qs[IXL_TOK * CPG];
  __shared__ __attribute__((aligned(16))) float ws[HI * IXL_TOK];   // [h][token]
  extern __shared__ __attribute__((aligned(16))) float score_lds[];  // rows, then histograms

  const int seg = blockIdx.x % L.num_seqs;
  const int rev = (int)(blockIdx.x / L.num_seqs);
  const int q_start = __ldg(L.cu_q + seg);
  const int q_len = __ldg(L.cu_q + seg + 1) - q_start;
  const int nqb = (q_len + IXL_TOK - 1) / IXL_TOK;
  if (rev >= nqb) return;
  const int t0 = (nqb - 1 - rev) * IXL_TOK;
  const int k_base = __ldg(L.cu_k + seg);
  const int s_k = __ldg(L.cu_k + seg + 1) - k_base;
  const int off = seg_offset(L, seg, q_len, s_k);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nlive = (n_valid_of(min(t0 + IXL_TOK, q_len) - 1, off, L.ratio, s_k) + 63) / 64;
  if (nlive == 0) {   // no row of the block sees a key: -1 ids, -inf scores and lse
    for (int e = tid; e < IXL_TOK * to.k_eff; e += NTHR) {
      const int r = e / to.k_eff, c = e - r * to.k_eff;
      if (t0 + r < q_len) {
        to.ids[(int64_t)(q_start + t0 + r) * to.k_eff + c] = -1;
        to.sel[(int64_t)(q_start + t0 + r) * to.k_eff + c] = -__builtin_inff();
      }
    }
    if (to.lse && tid < IXL_TOK && t0 + tid < q_len) to.lse[q_start + t0 + tid] = -__builtin_inff();
    return;
  }
  const int str = nlive * 64 + 4;   // score row stride (the four token groups of a store hit different banks)
  auto row_ptr = [&](int r) { return score_lds + r * str; };

  const int rows_left = min(IXL_TOK, total_q - (q_start + t0));
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(q_idx + (int64_t)(q_start + t0) * (RB / 2), (uint32_t)(rows_left * RB));
  auto stage = [&](int gi) {   // head group gi of the block's 16 rows -> qs
    for (int m = w; m < IXL_TOK * PPG; m += IXL_WAVES) {
      const int r = m / PPG, q0 = (m - r * PPG) * 64;
      dma16(rq, reinterpret_cast<char *>(qs) + (size_t)(r * CPG + q0) * 16,
            (uint32_t)(r * RB + gi * GB + (((q0 + lane) ^ r) << 4)));
    }
  };
  stage(0);
  // fp32(w * s_idx), head-major (unconditional loads: a token past the segment reads its
  // last row, then is zeroed)
  {
    constexpr int NW = (HI * IXL_TOK + NTHR - 1) / NTHR;
    float x[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const int e = tid + k * NTHR;
      const int tt = e / HI, h = e - tt * HI;
      const int t = min(t0 + tt, q_len - 1);
      x[k] = e < HI * IXL_TOK ? weights[(int64_t)(q_start + t) * HI + h] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const int e = tid + k * NTHR;
      if (e < HI * IXL_TOK) {
        const int tt = e / HI, h = e - tt * HI;
        ws[h * IXL_TOK + tt] = t0 + tt < q_len ? x[k] * idx_scale : 0.f;
      }
    }
  }
  // key tile fragments (MFMA B operand: lane column r16 = key, piece 4c+g); keys past the
  // segment are clamped to its last key (their scores are never selected)
  auto load_k = [&](int tile, u32x4 (&kb)[4][NCD]) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int j = min(tile * 64 + 16 * n + r16, s_k - 1);
      const u32x4 *kp = reinterpret_cast<const u32x4 *>(k_idx + (int64_t)(k_base + j) * DI) + g;
#pragma unroll
      for (int c = 0; c < NCD; ++c) kb[n][c] = kp[4 * c];
    }
  };
  const char *qrow = reinterpret_cast<const char *>(qs) + r16 * CPG * 16;
  const float *wsp = ws + 4 * g;
  for (int gi = 0; gi < NG; ++gi) {
    if (gi > 0) {
      __syncthreads();   // every wave is done with the previous group's q rows
      stage(gi);
    }
    wait_vmcnt<0>();
    __syncthreads();     // group gi staged (and, the first time, the weights)
    u32x4 kb[4][NCD], kbn[4][NCD];
    if (w < nlive) load_k(w, kbn);
    for (int u = w; u < nlive; u += IXL_WAVES) {
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int c = 0; c < NCD; ++c) kb[n][c] = kbn[n][c];
      if (u + IXL_WAVES < nlive) load_k(u + IXL_WAVES, kbn);
      // the accumulators continue where the previous head group left them
      f32x4 acc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float *src = row_ptr(4 * g + i) + u * 64 + r16;
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[n][i] = gi > 0 ? src[16 * n] : 0.f;
      }
      __builtin_amdgcn_sched_barrier(0);
      auto a_frag = [&](int hl, u32x4 (&qa)[NCD]) {
#pragma unroll
        for (int c = 0; c < NCD; ++c)
          qa[c] = *reinterpret_cast<const u32x4 *>(qrow + (((hl * CH + 4 * c + g) ^ r16) << 4));
      };
      auto head_mfma = [&](const u32x4 (&qa)[NCD], f32x4 (&d)[4]) {
#pragma unroll
        for (int n = 0; n < 4; ++n) d[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NCD; ++c)
#pragma unroll
          for (int n = 0; n < 4; ++n) d[n] = mfma16x16x32(qa[c], kb[n][c], d[n]);
      };
      auto epilogue = [&](const f32x4 (&d)[4], const f32x4 &wv) {
#pragma unroll
        for (int n = 0; n < 4; ++n) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[n][i] = fmaf(wv[i], relu_bits(d[n][i]), acc[n][i]);
          asm volatile("" : "+v"(acc[n]));   // the epilogue of head h stays in its iteration
        }
      };
      auto interleave = [&]() {
#pragma unroll
        for (int m = 0; m < 4 * NCD; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 32 / (4 * NCD), 0);  // then VALU
        }
      };
      // two register sets alternate between "MFMAs in flight" and "epilogue"
      u32x4 qa0[NCD], qa1[NCD];
      f32x4 d0[4], d1[4];
      a_frag(0, qa0);
      head_mfma(qa0, d0);
      if (HGF > 1) a_frag(1, qa1);
#pragma unroll
      for (int hl = 0; hl < HGF; hl += 2) {
        const f32x4 w0 = *reinterpret_cast<const f32x4 *>(wsp + (gi * HGF + hl) * IXL_TOK);
        if (hl + 1 < HGF) {
          head_mfma(qa1, d1);
          if (hl + 2 < HGF) a_frag(hl + 2, qa0);
        }
        epilogue(d0, w0);
        if (hl + 1 < HGF) interleave();
        __builtin_amdgcn_sched_barrier(0);
        if (hl + 1 < HGF) {
          const f32x4 w1 = *reinterpret_cast<const f32x4 *>(wsp + (gi * HGF + hl + 1) * IXL_TOK);
          if (hl + 2 < HGF) {
            head_mfma(qa0, d0);
            if (hl + 3 < HGF) a_frag(hl + 3, qa1);
          }
          epilogue(d1, w1);
          if (hl + 2 < HGF) interleave();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // lane (token 4g+i, key u*64 + 16n + r16) -> the block's LDS score row
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float *dst = row_ptr(4 * g + i) + u * 64 + r16;
#pragma unroll
        for (int n = 0; n < 4; ++n) dst[16 * n] = acc[n][i];
      }
    }
  }
  __syncthreads();   // every score tile of the block is in LDS
  uint32_t *hist = reinterpret_cast<uint32_t *>(score_lds + IXL_TOK * str) + 256 * w;
  for (int r = w; r < IXL_TOK; r += IXL_WAVES) {
    const int t = t0 + r;
    if (t >= q_len) continue;
    const int n = n_valid_of(t, off, L.ratio, s_k);
    const float *row = row_ptr(r);
    float val[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int j = v * 64 + lane;
      val[v] = j < n ? row[j] : -__builtin_inff();
    }
    const int64_t o = (int64_t)(q_start + t) * to.k_eff;
    if (to.lse) {
      float m = -__builtin_inff();
#pragma unroll
      for (int v = 0; v < VPL; ++v) m = fmaxf(m, val[v]);
      m = wave_max_dpp(m);
      double sum = 0.0;
#pragma unroll
      for (int v = 0; v < VPL; ++v)
        if (v * 64 + lane < n) sum += (double)__expf(val[v] - m);
      sum = wave_sum_f64_dpp(sum);
      if (lane == 0) to.lse[q_start + t] = n > 0 ? m + (float)log(sum) : -__builtin_inff();
    }
    if (n <= to.k_eff) {   // every visible key is selected
      for (int c = lane; c < to.k_eff; c += 64) {
        to.ids[o + c] = c < n ? k_base + c : -1;
        to.sel[o + c] = c < n ? row[c] : -__builtin_inff();
      }
    } else {
      const __amdgpu_buffer_rsrc_t rid = make_rsrc(to.ids + o, (uint32_t)to.k_eff * 4);
      const __amdgpu_buffer_rsrc_t rsel = make_rsrc(to.sel + o, (uint32_t)to.k_eff * 4);
      wave_select<VPL>(val, n, to.k_eff, hist, [&](int pos, int j, int v) {
        __builtin_amdgcn_raw_buffer_store_b32(k_base + j, rid, pos * 4, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val[v]), rsel, pos * 4, 0, 0);
      });
    }
  }
}

static int grouped_dyn_bytes(int max_sk) { return (IXL_TOK * ((max_sk + 63) / 64 * 64 + 4) + 256 * IXL_WAVES) * 4; }

template <int DI, int HI, int HGF, int VPL>
static hipError_t launch_grouped_t(const LaunchLayout &LL, const void *q_idx, const void *k_idx,
                                   const float *weights, float idx_scale, const TopkOut &to, hipStream_t st) {
  const int nqb = (LL.max_seqlen_q + IXL_TOK - 1) / IXL_TOK;
  const int64_t grid = (int64_t)LL.num_seqs * nqb;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int dyn = grouped_dyn_bytes(LL.max_seqlen_k);
  auto kern = indexer_topk_grouped_kernel<DI, HI, HGF, VPL>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, dyn);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * IXL_WAVES), dyn, st, LL.dev,
                     static_cast<const uint16_t *>(q_idx), static_cast<const uint16_t *>(k_idx), weights,
                     idx_scale, LL.max_seqlen_k, LL.total_q, to);
  return hipGetLastError();
}

template <int DI, int HI, int HGF>
static hipError_t launch_grouped_v(const LaunchLayout &LL, const void *q_idx, const void *k_idx,
                                   const float *weights, float idx_scale, const TopkOut &to, hipStream_t st) {
  const int vpl = (LL.max_seqlen_k + 63) / 64;
  if (vpl <= 4) return launch_grouped_t<DI, HI, HGF, 4>(LL, q_idx, k_idx, weights, idx_scale, to, st);
  if (vpl <= 8) return launch_grouped_t<DI, HI, HGF, 8>(LL, q_idx, k_idx, weights, idx_scale, to, st);
  if (vpl <= 16) return launch_grouped_t<DI, HI, HGF, 16>(LL, q_idx, k_idx, weights, idx_scale, to, st);
  if (vpl <= 32) return launch_grouped_t<DI, HI, HGF, 32>(LL, q_idx, k_idx, weights, idx_scale, to, st);
  return hipErrorInvalidValue;
}

// head-group size of the grouped kernel: 2 KiB of each q row per group
template <int DI> constexpr int grouped_hgf() { return 1024 / DI; }

bool indexer_topk_supported(bool bf16, int Hi, int Di, int max_seqlen_k) {
  // rows up to 2048 keys (Di = 64) or 512 keys (Di = 128: longer rows would spill the
  // selection's registers)
  if (!bf16 || max_seqlen_k > (Di == 128 ? 8 : 32) * 64) return false;
  int stat;
  if (Di == 64 && Hi == 8) stat = lds_static_bytes<64, 8>();
  else if (Di == 64 && Hi == 16) stat = lds_static_bytes<64, 16>();
  else if (Di == 128 && Hi == 4) stat = lds_static_bytes<128, 4>();
  else if (Di == 128 && Hi == 8) stat = lds_static_bytes<128, 8>();
  else if (Di == 64 && Hi == 32) return grouped_static_bytes<64, 32, grouped_hgf<64>()>() + grouped_dyn_bytes(max_seqlen_k) <= LDS_PER_CU;
  else if (Di == 64 && Hi == 64) return grouped_static_bytes<64, 64, grouped_hgf<64>()>() + grouped_dyn_bytes(max_seqlen_k) <= LDS_PER_CU;
  else if (Di == 128 && Hi == 16) return grouped_static_bytes<128, 16, grouped_hgf<128>()>() + grouped_dyn_bytes(max_seqlen_k) <= LDS_PER_CU;
  else if (Di == 128 && Hi == 32) return grouped_static_bytes<128, 32, grouped_hgf<128>()>() + grouped_dyn_bytes(max_seqlen_k) <= LDS_PER_CU;
  else return false;
  return stat + fused_dyn_bytes(max_seqlen_k) <= LDS_PER_CU;
}

hipError_t launch_indexer_topk(const LaunchLayout &LL, const void *q_idx, const void *k_idx,
                               const float *weights, int Hi, int Di, float idx_scale, int k_eff,
                               int32_t *ids, float *sel, float *lse, hipStream_t st) {
  if (LL.total_q == 0) return hipSuccess;
  const TopkOut to{ids, sel, lse, k_eff, fused_cap(LL.max_seqlen_k)};
  if (Di == 64 && Hi == 8) return launch_fused_v<64, 8>(LL, q_idx, k_idx, weights, idx_scale, to, st);
  if (Di == 64 && Hi == 16) return launch_fused_v<64, 16>(LL, q_idx, k_idx, weights, idx_scale, to, st);
  if (Di == 128 && Hi == 4) return launch_fused_v<128, 4>(LL, q_idx, k_idx, weights, idx_scale, to, st);
  if (Di == 128 && Hi == 8) return launch_fused_v<128, 8>(LL, q_idx, k_idx, weights, idx_scale, to, st);
  if (Di == 64 && Hi == 32) return launch_grouped_v<64, 32, grouped_hgf<64>()>(LL, q_idx, k_idx, weights, idx_scale, to, st);
  if (Di == 64 && Hi == 64) return launch_grouped_v<64, 64, grouped_hgf<64>()>(LL, q_idx, k_idx, weights, idx_scale, to, st);
  if (Di == 128 && Hi == 16) return launch_grouped_v<128, 16, grouped_hgf<128>()>(LL, q_idx, k_idx, weights, idx_scale, to, st);
  if (Di == 128 && Hi == 32) return launch_grouped_v<128, 32, grouped_hgf<128>()>(LL, q_idx, k_idx, weights, idx_scale, to, st);
  return hipErrorInvalidValue;
}

// ============================================================================
// Head-grouped variant for long q_idx rows (bf16, Hi * Di * 2 above what the paired-block
// kernel stages).  One workgroup (4 waves) = 16 tokens x 256 keys; wave w = the 16 tokens
// x 64 keys (64 w), its key fragments in registers for the whole head loop.  The q rows
// are staged in LDS one head group at a time (HG heads = 512 bytes of each token row,
// 8 KiB per group: two 1 KiB buffer->LDS loads, four rows, per wave), chunk q of token row
// r at slot q ^ r so the 16 lanes of an A-operand read hit 16 bank groups, in a ring of
// four buffers requested three groups ahead (a group's MFMAs take far less time than its
// rows take to arrive from L2); fp32(w * s_idx) of every head is staged once.  Per head:
// Di/32 x 4 MFMAs, then the ReLU x weight accumulate.  Each staged byte of q feeds 256
// keys; four independent workgroups per compute unit (rather than two of 8 waves, which
// fed 512 keys per byte) overlap one another's group barriers and tile prologues.
// ============================================================================
constexpr int HGK_TOK = 16;
constexpr int HGK_KEYS = 256;
constexpr int HGK_WAVES = 4;
constexpr int HGK_NBUF = 4;
// The staged weights [Hi][16 tokens]: token tt of head h sits at h * 16 + (tt ^ wsw(h)).
// The staging writes go across heads (lane = head), which without the XOR would put 4
// lanes on one LDS bank per row of 16 heads; the XOR is a multiple of 4, so the 4 tokens a
// lane reads as one f32x4 stay one aligned group.
__device__ __forceinline__ int wsw(int h) { return 4 * ((h >> 2) & 3); }

template <int DI>
__global__ __launch_bounds__(64 * HGK_WAVES) __attribute__((amdgpu_waves_per_eu(4))) void indexer_score_hg_kernel(
    LayoutDev L, const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ k_idx,
    const float *__restrict__ weights, int Hi, float idx_scale, float *__restrict__ scores, int64_t ld,
    int max_sk, int total_q, int nqb) {
  constexpr int HG = 256 / DI;        // heads per staged group
  constexpr int PB = HG * DI * 2;     // bytes of a token row per group (512)
  constexpr int CPP = PB / 16;        // 16-byte chunks per staged row
  constexpr int NCD = DI / 32;
  constexpr int NTHR = 64 * HGK_WAVES;
  constexpr int NL = HGK_TOK * PB / 1024 / HGK_WAVES;   // 1 KiB loads per wave and group
  static_assert(PB == 512 && CPP == 32 && NL == 2, "two 1 KiB loads per wave and group");
  __shared__ __attribute__((aligned(16))) u32x4 qs[HGK_NBUF][HGK_TOK * CPP];
  extern __shared__ __attribute__((aligned(16))) float wsl[];   // [Hi][HGK_TOK], tokens XOR wsw(h)

  // Workgroup id -> tile, XCD-aware: workgroups are dealt to the 8 XCDs round-robin by id,
  // so id = 8 * slot + xcd; token block b goes to XCD b % 8, and an XCD's consecutive slots
  // walk all key tiles of one of its token blocks before the next.  The 16 q rows of a
  // block (Hi * Di * 2 bytes each) are then fetched from HBM about once and re-read from
  // that XCD's L2 by the block's key tiles, instead of once per key tile.
  const int nkb = (max_sk + HGK_KEYS - 1) / HGK_KEYS;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int lq = slot / nkb, kt = slot - lq * nkb;
  const int b = lq * 8 + xcd;
  if (b >= L.num_seqs * nqb) return;
  const int seg = b / nqb;
  const int qb = b - seg * nqb;
  const int q_start = __ldg(L.cu_q + seg);
  const int q_len = __ldg(L.cu_q + seg + 1) - q_start;
  const int t0 = qb * HGK_TOK;
  if (t0 >= q_len) return;
  const int k_base = __ldg(L.cu_k + seg);
  const int s_k = __ldg(L.cu_k + seg + 1) - k_base;
  const int off = seg_offset(L, seg, q_len, s_k);
  const int j0 = kt * HGK_KEYS;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jw = j0 + 64 * w;
  const int nv_last = n_valid_of(min(t0 + HGK_TOK, q_len) - 1, off, L.ratio, s_k);

  if (j0 >= nv_last) {   // the whole tile is above the causal limit
    for (int e = tid; e < HGK_TOK * HGK_KEYS; e += NTHR) {
      const int tt = e / HGK_KEYS, j = j0 + (e - tt * HGK_KEYS);
      if (t0 + tt < q_len && j < max_sk) scores[(int64_t)(q_start + t0 + tt) * ld + j] = -__builtin_inff();
    }
    return;
  }
  const int64_t RB = (int64_t)Hi * DI * 2;   // bytes of one token's q_idx row
  const int rows_left = min(HGK_TOK, total_q - (q_start + t0));
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(q_idx + (int64_t)(q_start + t0) * Hi * DI, (uint32_t)(rows_left * RB));
  // group grp's rows into buffer grp % NBUF: load k of wave w moves rows 2(2w + k) and
  // 2(2w + k) + 1 (lane >> 5), 1 KiB of the buffer at (2w + k) KiB
  uint32_t soff[NL];
#pragma unroll
  for (int k = 0; k < NL; ++k) {
    const int srow = 2 * (NL * w + k) + (lane >> 5), sc = lane & 31;
    soff[k] = (uint32_t)(srow * RB + ((sc ^ (srow & 15)) << 4));
  }
  auto stage = [&](int grp) {
#pragma unroll
    for (int k = 0; k < NL; ++k)
      dma16(rq, reinterpret_cast<char *>(qs[grp % HGK_NBUF]) + (size_t)(NL * w + k) * 1024,
            soff[k] + (uint32_t)(grp * PB));
  };
  const int ngrp = Hi / HG;
#pragma unroll
  for (int k = 0; k < HGK_NBUF - 1; ++k)
    if (k < ngrp) stage(k);
  // key fragments (B operand: lane column r16 = key, piece 4c+g); keys past the segment
  // are clamped to its last key (their scores are masked)
  u32x4 kb[4][NCD];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int j = min(jw + 16 * n + r16, s_k - 1);
    const u32x4 *kp = reinterpret_cast<const u32x4 *>(k_idx + (int64_t)(k_base + j) * DI) + g;
#pragma unroll
    for (int c = 0; c < NCD; ++c) kb[n][c] = kp[4 * c];
  }
  // the block's weights are one contiguous run of rows_w * Hi floats: unconditional loads
  // through a buffer resource of exactly that run (tokens past the segment read zeros),
  // several per thread in flight at once -- a guarded load per element would be waited
  // for (with every earlier load of the wave) before the next is issued
  {
    const int rows_w = min(HGK_TOK, q_len - t0);
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(weights + (int64_t)(q_start + t0) * Hi, (uint32_t)(rows_w * Hi) * 4);
    for (int e0 = tid; e0 < Hi * HGK_TOK; e0 += 2 * NTHR) {
      float x[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
        x[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rw, (e0 + u * NTHR) * 4, 0, 0));
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = e0 + u * NTHR;
        if (e < Hi * HGK_TOK) {
          const int tt = e / Hi, h = e - tt * Hi;
          wsl[h * HGK_TOK + (tt ^ wsw(h))] = x[u] * idx_scale;
        }
      }
    }
  }
  f32x4 acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int rrow = r16 * PB;
  for (int grp = 0; grp < ngrp; ++grp) {
    // group grp's rows have landed once at most the loads of the groups after it that were
    // requested (NL per wave and group) are outstanding; the barrier publishes every
    // wave's rows (and, first time, the weights) and frees the buffer of group grp - 1
    if (grp + 2 < ngrp) wait_vmcnt<2 * NL>();
    else if (grp + 1 < ngrp) wait_vmcnt<NL>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (grp + HGK_NBUF - 1 < ngrp) stage(grp + HGK_NBUF - 1);
    const char *qb = reinterpret_cast<const char *>(qs[grp % HGK_NBUF]) + rrow;
#pragma unroll
    for (int hl = 0; hl < HG; ++hl) {
      u32x4 qa[NCD];
#pragma unroll
      for (int c = 0; c < NCD; ++c)
        qa[c] = *reinterpret_cast<const u32x4 *>(qb + (((hl * (DI / 8) + 4 * c + g) ^ r16) << 4));
      f32x4 d[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) d[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NCD; ++c)
#pragma unroll
        for (int n = 0; n < 4; ++n) d[n] = mfma16x16x32(qa[c], kb[n][c], d[n]);
      const int hw = grp * HG + hl;
      const f32x4 wv = *reinterpret_cast<const f32x4 *>(wsl + hw * HGK_TOK + ((4 * g) ^ wsw(hw)));
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[n][i] = fmaf(wv[i], relu_bits(d[n][i]), acc[n][i]);
    }
  }
  // lane (token 4g + i, key jw + 16n + r16)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * g + i;
    if (t >= q_len) continue;
    const int nv = n_valid_of(t, off, L.ratio, s_k);
    float *dst = scores + (int64_t)(q_start + t) * ld;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int j = jw + 16 * n + r16;
      if (j < max_sk) dst[j] = j < nv ? acc[n][i] : -__builtin_inff();
    }
  }
}

template <int DI>
static hipError_t launch_hg(const LaunchLayout &LL, const void *q_idx, const void *k_idx,
                            const float *weights, int Hi, float idx_scale, float *scores, int64_t ld,
                            hipStream_t st) {
  const int nqb = (LL.max_seqlen_q + HGK_TOK - 1) / HGK_TOK;
  const int nkb = (LL.max_seqlen_k + HGK_KEYS - 1) / HGK_KEYS;
  const int64_t nblk = ((int64_t)LL.num_seqs * nqb + 7) / 8 * 8;   // token blocks, padded to the 8 XCDs
  if (nblk * nkb > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)(nblk * nkb));
  const size_t lds = (size_t)Hi * HGK_TOK * sizeof(float);
  hipLaunchKernelGGL((indexer_score_hg_kernel<DI>), grid, dim3(64 * HGK_WAVES), lds, st, LL.dev,
                     static_cast<const uint16_t *>(q_idx), static_cast<const uint16_t *>(k_idx), weights, Hi,
                     idx_scale, scores, ld, LL.max_seqlen_k, LL.total_q, nqb);
  return hipGetLastError();
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
    if (Di == 64 && Hi == 8) return launch_lds<64, 8>(LL, q_idx, k_idx, weights, idx_scale, scores, ld, st);
    if (Di == 64 && Hi == 16) return launch_lds<64, 16>(LL, q_idx, k_idx, weights, idx_scale, scores, ld, st);
    if (Di == 64 && Hi == 32) return launch_lds<64, 32>(LL, q_idx, k_idx, weights, idx_scale, scores, ld, st);
    if (Di == 128 && Hi == 4) return launch_lds<128, 4>(LL, q_idx, k_idx, weights, idx_scale, scores, ld, st);
    if (Di == 128 && Hi == 8) return launch_lds<128, 8>(LL, q_idx, k_idx, weights, idx_scale, scores, ld, st);
    // long rows: head groups staged in LDS (16 tokens x 512 bytes per group)
    if (Di == 64 && Hi >= 64 && Hi % 4 == 0)
      return launch_hg<64>(LL, q_idx, k_idx, weights, Hi, idx_scale, scores, ld, st);
    if (Di == 128 && Hi >= 16 && Hi % 2 == 0)
      return launch_hg<128>(LL, q_idx, k_idx, weights, Hi, idx_scale, scores, ld, st);
  }
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
