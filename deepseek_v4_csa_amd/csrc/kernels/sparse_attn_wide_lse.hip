// First pass of the D = 512 attention: the per-head normalisers of each query row.
//
// Page "[Bug] DSV4 unfused CSA indexer loss uses a compressed-only teacher ...": the
// "Paper reference" Z_h equation and the csa.py sparse-attention excerpt (window ids then
// top-k ids, the sink as a fp32 logit, softmax_scale on q.k); the proposal's u_h:
//   lse_h    = log Z_h = log(exp(sink_h) + sum_window exp(w_ht') + sum_valid ids exp(c_hj))
//   lse_nc_h = log(exp(sink_h) + sum_window exp(w_ht'))
// The second kernel (sparse_attn_wide.hip) needs lse before it can form P, the output and
// the head-summed probabilities, so the logits are formed twice; this pass only sums
// exponentials and holds no output accumulators, which leaves room for two waves per SIMD:
// one wave's exponentials, masks and LDS waits run while the other's MFMAs do.
//
// One workgroup of four waves per query row, two workgroups per compute unit (one wave of
// each per SIMD): the two rows' steps are not synchronised, so one workgroup's waits,
// barriers and exponentials run while the other's MFMAs do.  Wave w holds the Q rows of
// heads [32 w, +32) in registers and forms S^T = K Q^T over all 32 keys of every chunk:
// each K operand it reads from LDS feeds two MFMAs (its two 16-head tiles).  The row's KV
// rows are staged a chunk (32 rows, 32 KiB) at a time in two LDS tiles by direct
// buffer->LDS loads, the next chunk requested right after each step's barrier, 16-byte
// pieces XOR-swizzled by row_swz as in the other D = 512 kernel.  Each wave keeps a
// running maximum per head (raised lazily, by 2^8 or more) and the sum of exponentials,
// folding a chunk's logits in while the next chunk's MFMAs run.
#include <hip/hip_runtime.h>

#include "common.h"
#include "../launch.h"

namespace csa {

namespace {
constexpr int LD = 512;                 // head dim
constexpr int LWV = 4;                  // waves per workgroup
constexpr int LNT = 64 * LWV;           // threads
constexpr int LROWB = LD * 2;           // bytes per KV row (1 KiB)
constexpr int LTILE = 32 * LROWB;       // one 32-row chunk (32 KiB)
constexpr int LNTILE = 2;               // tiles in the ring: the next chunk requested one step ahead
constexpr int LNC = LD / 32;            // MFMA K-chunks per row
constexpr int LRPW = 32 / LWV;          // rows each wave stages per chunk
constexpr int LLA = 3;                  // K operand pairs requested ahead of their MFMAs
constexpr int LIDS = 8;                 // ids per thread in the first batch (2,048 slots)
}  // namespace

// the tiles, then the id slots: whole chunks, at least the first batch's LIDS * LNT
size_t wide_lse_lds_bytes(int k_eff) {
  const int ncc = (k_eff + 31) / 32;
  return (size_t)LNTILE * LTILE + (size_t)max(ncc * 32, LIDS * LNT) * sizeof(int);
}

__global__ __launch_bounds__(LNT, 1) void sparse_attn_wide_lse_kernel(
    LayoutDev L, const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const uint16_t *__restrict__ ckv, const float *__restrict__ sink,
    const int32_t *__restrict__ ids, int k_eff, int window, int H, int total_q, int total_k,
    float sl2, float *__restrict__ lse, float *__restrict__ lse_nc) {
  constexpr float NINF = -__builtin_inff();
  constexpr float RESCALE = 8.f;
  extern __shared__ __attribute__((aligned(16))) char lse_dyn[];   // tiles, then ids
  int *ids_l = reinterpret_cast<int *>(lse_dyn + LNTILE * LTILE);
  __shared__ int jlast;

  const int t = total_q - 1 - (int)blockIdx.x;   // the longest rows (last) first
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  int hh[2];
  bool ok[2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    hh[hi] = 32 * w + 16 * hi + r16;
    ok[hi] = hh[hi] < H;
  }
  const RowGeo geo = row_geo(L, t);
  const int w_lo = max(geo.q_start, t - window + 1);
  const int nw = window > 0 ? t - w_lo + 1 : 0;
  const int nwc = (nw + 31) >> 5, ncc_all = (k_eff + 31) >> 5;
  if (tid == 0) jlast = -1;

  // The row's ids (slots past k_eff hold -1) and the Q^T operands: the first LIDS ids of
  // each thread are requested, then Q, and only then are the ids stored (the compiler waits
  // for the older loads only; a buffer load past k_eff returns 0)
  const __amdgpu_buffer_rsrc_t rid = make_rsrc(ids + (int64_t)t * k_eff, (uint32_t)k_eff * 4);
  int x[LIDS];
#pragma unroll
  for (int u = 0; u < LIDS; ++u) x[u] = __builtin_amdgcn_raw_buffer_load_b32(rid, (tid + u * LNT) * 4, 0, 0);
  asm volatile("" ::: "memory");
  // piece c of lane group g holds features [(4c+g)*8, +8) (a head past H loads head 0's
  // row: its statistics are never written)
  u32x4 qf[2][LNC];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(q + ((int64_t)t * H + (ok[hi] ? hh[hi] : 0)) * LD) + g;
#pragma unroll
    for (int c = 0; c < LNC; ++c) qf[hi][c] = p[4 * c];
  }
  asm volatile("" ::: "memory");
  lds_barrier();   // jlast initialised
  {
    // jlast = the last slot holding an id: the wave's maximum, then one LDS atomic per wave
    int jl = -1;
    auto put = [&](int j, int v) __attribute__((always_inline)) {   // no branch: the loads stay above Q's
      const int id = j < k_eff ? v : -1;
      ids_l[j] = id;
      jl = id >= 0 ? j : jl;
    };
#pragma unroll
    for (int u = 0; u < LIDS; ++u) put(tid + u * LNT, x[u]);
    for (int j = tid + LIDS * LNT; j < ncc_all * 32; j += LNT) put(j, __builtin_amdgcn_raw_buffer_load_b32(rid, j * 4, 0, 0));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) jl = max(jl, __shfl_xor(jl, m, 64));
    if (lane == 0 && jl >= 0) atomicMax(&jlast, jl);
  }
  const __amdgpu_buffer_rsrc_t rkv = make_rsrc(kv, (uint32_t)(t + 1) * LROWB);   // rows past t: zeros
  const __amdgpu_buffer_rsrc_t rck = make_rsrc(ckv, (uint32_t)total_k * LROWB);  // id -1: past the end
  const __amdgpu_buffer_rsrc_t rnone = make_rsrc(kv, 0);                         // every load: zeros
  // K operand: row r16 (+16), piece (4c + g) ^ swz = 4 (c ^ (swz >> 2)) + (g ^ (swz & 3));
  // with c = 4 (c >> 2) + j that is byte 256 (c >> 2) + kbj[j] of the row
  const int ksw = row_swz<LD>(r16);
  int kbj[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) kbj[j] = r16 * LROWB + 16 * (g ^ (ksw & 3)) + 64 * (j ^ (ksw >> 2));

  lds_barrier();   // ids and jlast in LDS (the Q loads stay in flight)
  // key masks of the compressed chunks (bit b of chunk c: slot 32 c + b holds an id), lane
  // c of cbits[h] holding chunk 64 h + c
  uint32_t cbits[2] = {0u, 0u};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = 64 * h + lane;
    if (c < ncc_all) {   // eight 16-byte reads, rotated by lane
      uint32_t m = 0;
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int vv = (v + lane) & 7;
        const int4 x = reinterpret_cast<const int4 *>(ids_l + 32 * c)[vv];
        m |= (uint32_t)(x.x >= 0) << (4 * vv) | (uint32_t)(x.y >= 0) << (4 * vv + 1) |
             (uint32_t)(x.z >= 0) << (4 * vv + 2) | (uint32_t)(x.w >= 0) << (4 * vv + 3);
      }
      cbits[h] = m;
    }
  }
  auto row_mask = [&](int ci) -> uint32_t {
    if (ci < nwc) {
      const int n = nw - 32 * ci;
      return n >= 32 ? 0xffffffffu : (1u << n) - 1u;
    }
    const int cc = ci - nwc;
    return (uint32_t)__builtin_amdgcn_readlane(cc < 64 ? cbits[0] : cbits[1], cc & 63);
  };
  const int ncc = (jlast + 32) >> 5, nch = nwc + ncc;
  auto tile = [&](int n) { return lse_dyn + (n & 1) * LTILE; };

  // Loads of chunk n: instruction k of wave w moves row i = w + 4k (1 KiB); lane l writes
  // slot l, which holds the row's piece l ^ row_swz(i).  A chunk past the last loads zeros
  // (so every wave issues exactly LRPW loads per step), spread one per two K-chunks over
  // the step's MFMAs.
  struct ChunkReq {
    __amdgpu_buffer_rsrc_t r;
    char *buf;
    int myrow;   // lane l (< 32) holds the KV or compressed row that is chunk row l
  };
  uint32_t d0 = 16 * lane;
  asm volatile("" : "+v"(d0));
  auto request = [&](int n) -> ChunkReq {
    ChunkReq rq;
    rq.buf = tile(n);
    if (n >= nch) {
      rq.r = rnone;
      rq.myrow = 0;
    } else if (n < nwc) {
      rq.r = rkv;
      rq.myrow = w_lo + 32 * n + (lane & 31);
    } else {
      rq.r = rck;
      rq.myrow = ids_l[32 * (n - nwc) + (lane & 31)];
    }
    return rq;
  };
  auto issue_row = [&](const ChunkReq &rq, int k) __attribute__((always_inline)) {
    const int i = w + LWV * k;
    const uint32_t off = d0 ^ (uint32_t)(16 * row_swz<LD>(i));
    dma16(rq.r, rq.buf + i * LROWB, (uint32_t)__builtin_amdgcn_readlane(rq.myrow, i) * LROWB + off);
  };
  {
    const ChunkReq rq = request(0);
#pragma unroll
    for (int r = 0; r < LRPW; ++r) issue_row(rq, r);
  }

  float m[2], l[2], m_nc[2], l_nc[2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const float a2 = ok[hi] ? sink[hh[hi]] * LOG2E : NINF;
    m[hi] = a2;
    l[hi] = (g == 0 && a2 > NINF) ? 1.f : 0.f;   // the sink counted once per head
    m_nc[hi] = m[hi];
    l_nc[hi] = l[hi];
  }
  // The masked logits of a chunk (sv) are folded one step later, beside the next chunk's
  // MFMAs: the running maximum first (raised only when a logit passes it by RESCALE, in log2
  // units; rarely, a branch), then one value's exponential per K-chunk
  float sv[2][8];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[hi][e] = NINF;
  auto raise_max = [&]() __attribute__((always_inline)) {
    float cmx[2];
    bool up = false;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      cmx[hi] = sv[hi][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) cmx[hi] = fmaxf(cmx[hi], sv[hi][e]);
      up = up || cmx[hi] * sl2 > m[hi] + RESCALE;   // sl2 > 0 keeps the order
    }
    if (__builtin_expect(__ballot(up) != 0, 0)) {
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const float cand = across_groups_max(cmx[hi]) * sl2;
        const float mn = cand > m[hi] + RESCALE ? cand : m[hi];
        l[hi] *= mn == m[hi] ? 1.f : fast_exp2(m[hi] - mn);
        m[hi] = mn;
      }
    }
  };
  float nm[2], fx[16];
  // the sum of value v (head tile v / 8): its FMA, exponential and addition in three MFMA
  // windows of K-chunk v (j = 0, 1, 3), tied there by empty asm statements
  auto add_step = [&](int v, int j) __attribute__((always_inline)) {
    const int hi = v >> 3, e = v & 7;
    if (j == 0) {
      asm volatile("" : "+v"(sv[hi][e]));
      fx[v] = fmaf(sv[hi][e], sl2, nm[hi]);
      asm volatile("" : "+v"(fx[v]));
    } else if (j == 1) {
      asm volatile("" : "+v"(fx[v]));
      fx[v] = fast_exp2(fx[v]);
      asm volatile("" : "+v"(fx[v]));
    } else if (j == 3) {
      asm volatile("" : "+v"(fx[v]));
      l[hi] += fx[v];
      asm volatile("" : "+v"(l[hi]));
    }
  };
  for (int n = 0; n < nch; ++n) {
    // the wave's loads of chunk n are the only ones in flight (the Q loads are older): then
    // the barrier publishes every wave's rows and frees the tile of chunk n - 1, which the
    // request of chunk n + 1 reuses
    wait_vmcnt<0>();
    lds_barrier();
    const ChunkReq rq = request(n + 1);
    raise_max();   // chunk n - 1
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) nm[hi] = m[hi] == NINF ? 0.f : -m[hi];
    // S^T = K Q^T of the chunk's 32 keys and the wave's 32 heads: acc[kt][hi][i] is the
    // logit (unscaled) of key 16 kt + 4 g + i and head 32 w + 16 hi + r16
    const char *tb = tile(n);
    u32x4 kr[LLA][2];
    auto kread = [&](int c, u32x4 (&dst)[2]) __attribute__((always_inline)) {
      const char *kp = tb + kbj[c & 3] + 256 * (c >> 2);
      dst[0] = *reinterpret_cast<const u32x4 *>(kp);
      dst[1] = *reinterpret_cast<const u32x4 *>(kp + 16 * LROWB);
    };
#pragma unroll
    for (int c = 0; c < LLA; ++c) kread(c, kr[c]);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) asm volatile("" : "+v"(nm[hi]), "+v"(l[hi]));
    f32x4 acc[2][2];   // acc[kt][hi]
#pragma unroll
    for (int c = 0; c < LNC; ++c) {
      const u32x4 k0 = kr[c % LLA][0], k1 = kr[c % LLA][1];
      if (c + LLA < LNC) kread(c + LLA, kr[c % LLA]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 &kk = (j & 1) ? k1 : k0;
        if (c == 0) mfma_v_first(acc[j & 1][j >> 1], kk, qf[j >> 1][c]);
        else mfma_v(acc[j & 1][j >> 1], kk, qf[j >> 1][c]);
        add_step(c, j);   // chunk n - 1, value c
      }
      if (c % 2 == 1) issue_row(rq, c / 2);
    }
    mfma_v_fence(acc);
    if (n == nwc && n > 0) {   // every window chunk folded
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) { m_nc[hi] = m[hi]; l_nc[hi] = l[hi]; }
    }
    const uint32_t bm = row_mask(n) >> (4 * g);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sv[hi][e] = ((bm >> (16 * (e >> 2) + (e & 3))) & 1) ? acc[e >> 2][hi][e & 3] : NINF;
  }
  // the last chunk
  raise_max();
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) nm[hi] = m[hi] == NINF ? 0.f : -m[hi];
#pragma unroll
  for (int v = 0; v < 16; ++v)
#pragma unroll
    for (int j = 0; j < 4; ++j) add_step(v, j);
  if (nch == nwc && nch > 0) {
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) { m_nc[hi] = m[hi]; l_nc[hi] = l[hi]; }
  }
  wait_vmcnt<0>();   // no load into the LDS outlives the workgroup

  // the four lane groups of a head share m (raised on their common maximum)
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const float Ls = across_groups_sum(l[hi]), Lnc = across_groups_sum(l_nc[hi]);
    const float lse2 = (m[hi] > NINF && Ls > 0.f) ? m[hi] + __log2f(Ls) : NINF;
    const float lse2_nc = (m_nc[hi] > NINF && Lnc > 0.f) ? m_nc[hi] + __log2f(Lnc) : NINF;
    if (ok[hi] && g == 0) {
      lse[(int64_t)t * H + hh[hi]] = lse2 * LN2;
      lse_nc[(int64_t)t * H + hh[hi]] = lse2_nc * LN2;
    }
  }
}

// two workgroups per compute unit where the LDS holds two rings beside their ids (k_eff up
// to 4,096 with the 160 KiB of gfx950), else one
hipError_t launch_sparse_attn_wide_lse(const LaunchLayout &LL, const void *q, const void *kv, const void *ckv,
                                       const float *sink, const int32_t *ids, int k_eff, int window, int H,
                                       float scale, float *lse, float *lse_nc, hipStream_t st) {
  const size_t dyn = wide_lse_lds_bytes(k_eff);
  const hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void *>(sparse_attn_wide_lse_kernel),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL(sparse_attn_wide_lse_kernel, dim3((unsigned)LL.total_q), dim3(LNT), dyn, st, LL.dev,
                     static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(kv),
                     static_cast<const uint16_t *>(ckv), sink, ids, k_eff, window, H, LL.total_q, LL.total_k,
                     scale * LOG2E, lse, lse_nc);
  return hipGetLastError();
}

}  // namespace csa
