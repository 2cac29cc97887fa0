// Sliding-window + top-k compressed attention with a per-head sink for wide heads:
// D = 512 (a shared 512-wide latent KV row serving up to 128 attention heads), bf16.
//
// Same outputs and arithmetic contract as the other attention kernels (page "[Bug] DSV4
// unfused CSA indexer loss uses a compressed-only teacher ...": "Paper reference" Z_h
// equation; csa.py sparse-attention excerpt: window ids then top-k ids, the sink as a
// fp32 logit, softmax_scale on q.k):
//   Z_h = exp(sink_h) + sum_window exp(w_ht') + sum_valid ids exp(c_hj)
//   out = (sum_window e^w kv[t'] + sum_ids e^c ckv[id]) / Z_h,  lse = log Z_h,
//   lse_nc = log(exp(sink_h) + sum_window e^w),  cmass[t, j] = sum_h exp(c_hj - lse_h).
//
// One workgroup of four waves (one per SIMD, each with the whole 512-entry register file:
// 256 VGPRs and 256 AGPRs) per query row.  The row's KV rows are staged 32 at a time (one
// "chunk", 32 KiB) in a ring of three or four LDS tiles by direct buffer->LDS loads, the
// chunk one or two steps ahead requested right after each step's barrier.  With one KV
// row shared by every head, the cost that matters is LDS reads per MFMA; a wave holding
// the Q rows of 32 heads in registers reads each K operand once for four MFMAs:
//
//  pass 1 (lse and lse_nc): wave w takes heads [32 w, 32 w + 32) over all 32 keys of every
//    chunk (S^T = K Q^T on MFMA), with a running max per head (raised lazily, by 2^8 or
//    more) and a running sum.
//  pass 2 (P, out and cmass, lse final): the same S^T again, P = exp(s - lse) written as
//    bf16 to an LDS buffer holding the chunk's P for all 128 heads, its head sums added
//    into cmass.  One step later (behind the next barrier) wave w accumulates the output
//    columns [128 w, 128 w + 128) of every head in AGPRs: O^T[d, h] += V^T[d, j] P^T[j, h],
//    V^T read with the transposing LDS read (8 KiB per chunk) and P^T with 16-byte reads
//    (8 KiB per chunk).  Those 64 MFMAs do not depend on the chunk's softmax, so the two
//    are interleaved.
//
// LDS per query and 32-key chunk: pass 1 reads 128 KiB of K, pass 2 128 KiB of K plus
// 64 KiB of V and P; the 16-byte pieces of a tile row are XOR-swizzled (row_swz) so the K
// reads, the transposing V reads and the staging writes are free of bank conflicts, and
// P row h keeps its 16-byte key blocks XOR-swizzled by a function of h for the same reason
// (16 lanes reading 16 rows of 64 bytes).
#include <hip/hip_runtime.h>

#include "common.h"
#include "../launch.h"

namespace csa {

namespace {
constexpr int WD = 512;                 // head dim
constexpr int WW = 4;                   // waves per workgroup
constexpr int WNT = 64 * WW;            // threads
constexpr int WROWB = WD * 2;           // bytes per KV row (1 KiB)
constexpr int WTILE = 32 * WROWB;       // one 32-row chunk (32 KiB)
constexpr int WPROW = 64;               // bytes per P row (32 keys, bf16)
constexpr int WPBUF = 128 * WPROW;      // P of one chunk for 128 heads (8 KiB)
constexpr int WNC = WD / 32;            // MFMA K-chunks per row
constexpr int WRPW = 32 / WW;           // rows each wave stages per chunk
#ifndef WIDE_NTILE_MAX
#define WIDE_NTILE_MAX 4
#endif
#ifndef WIDE_LA
#define WIDE_LA 3
#endif
constexpr int LA = WIDE_LA;             // K operand pairs requested ahead of their MFMAs
constexpr int SG_VALU = 0x002, SG_MFMA = 0x008, SG_TRANS = 0x400;
// the compiler's machine scheduler places the instructions of a region in the order of
// these groups (used to interleave independent MFMAs and vector ALU work)
template <int MASK, int N> __device__ __forceinline__ void sched_group() {
  __builtin_amdgcn_sched_group_barrier(MASK, N, 0);
}
// S^T products on the 16x16x32 bf16 MFMA with C and D in VGPRs.  The builtin takes the
// accumulator form the output tiles need (AGPRs, all 256 of them), which pushes 16 output
// registers into VGPRs and copies them through AGPRs around every step; as asm statements
// the S^T tiles stay in VGPRs.  The compiler does not pad hazards it does not see, so:
//  * D is read only after mfma_v_fence: 16 wait states (this shape needs 8 before a vector
//    instruction reads its result and 3 before one overwrites a C operand still being read);
//  * C is the constant 0 or exactly D of the chain's previous MFMA (an exactly overlapping
//    accumulation chain needs no wait states);
//  * A and B are results of LDS and global loads, which the compiler waits for (it tracks the
//    registers an asm statement reads); no vector instruction writes them.
// Being volatile, the statements keep their order among themselves and with every memory
// access, so the LDS reads and row requests issue where the source places them.
__device__ __forceinline__ void mfma_v_first(f32x4 &d, const u32x4 &a, const u32x4 &b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x4 &d, const u32x4 &a, const u32x4 &b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_fence(f32x4 (&d)[2][2]) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(d[0][0]), "+v"(d[0][1]), "+v"(d[1][0]), "+v"(d[1][1]));
}
}  // namespace

// NTILE tiles in the ring: 3 requests the next chunk one step ahead, 4 two steps ahead
// (pass 2 still reads a tile one step after its own, for P.V)
size_t wide_attn_lds_bytes(int ntile, int k_eff) {
  const int ncc = (k_eff + 31) / 32;
  return (size_t)ntile * WTILE + 2 * (size_t)WPBUF + (size_t)ncc * 32 * sizeof(int);
}

template <int NTILE>
__global__ __launch_bounds__(WNT, 1) void sparse_attn_wide_kernel(
    LayoutDev L, const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const uint16_t *__restrict__ ckv, const float *__restrict__ sink,
    const int32_t *__restrict__ ids, int k_eff, int window, int H, int total_q, int total_k,
    float sl2, uint16_t *__restrict__ out, float *__restrict__ lse, float *__restrict__ lse_nc,
    float *__restrict__ cmass) {
  constexpr float NINF = -__builtin_inff();
  constexpr float RESCALE = 8.f;
  extern __shared__ __attribute__((aligned(16))) char wide_dyn[];   // tiles, P buffers, ids
  constexpr int DIST = NTILE - 2;          // request distance in steps
  char *pbufs = wide_dyn + NTILE * WTILE;
  int *ids_l = reinterpret_cast<int *>(pbufs + 2 * WPBUF);
  __shared__ float cm_part[2][WW][33];   // slot 32: spare target of stores not needed
  __shared__ int jlast;

  const int t = total_q - 1 - (int)blockIdx.x;   // the longest rows (last) first: a lighter tail
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  // the wave's heads: tile hi holds heads 32 w + 16 hi + r16
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

  // the row's ids, padded with -1 to whole chunks, through a buffer resource of exactly
  // k_eff ids (unconditional loads, four per thread in flight); jlast = the last slot that
  // holds an id: compressed chunks after it have no row and are skipped
  if (tid == 0) jlast = -1;
  __syncthreads();
  {
    const __amdgpu_buffer_rsrc_t rid = make_rsrc(ids + (int64_t)t * k_eff, (uint32_t)k_eff * 4);
    int jl = -1;
    for (int i0 = tid; i0 < ncc_all * 32; i0 += 4 * WNT) {
      int x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = __builtin_amdgcn_raw_buffer_load_b32(rid, (i0 + u * WNT) * 4, 0, 0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = i0 + u * WNT;
        const int id = j < k_eff ? x[u] : -1;
        if (j < ncc_all * 32) ids_l[j] = id;
        if (id >= 0) jl = j;
      }
    }
    if (jl >= 0) atomicMax(&jlast, jl);
  }
  // Q^T operands of both head tiles; piece c of lane group g holds features
  // [(4c+g)*8, +8) (a head past H loads head 0's row: its logits are masked)
  u32x4 qf[2][WNC];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(q + ((int64_t)t * H + (ok[hi] ? hh[hi] : 0)) * WD) + g;
#pragma unroll
    for (int c = 0; c < WNC; ++c) qf[hi][c] = p[4 * c];
  }
  const __amdgpu_buffer_rsrc_t rkv = make_rsrc(kv, (uint32_t)(t + 1) * WROWB);   // rows past t: zeros
  const __amdgpu_buffer_rsrc_t rck = make_rsrc(ckv, (uint32_t)total_k * WROWB);  // id -1: past the end
  // key masks of the compressed chunks (bit b of chunk c: slot 32 c + b holds an id), lane
  // c of cbits[h] holding chunk 64 h + c; built once from the staged ids below, so a step
  // takes its mask by a lane read instead of an LDS round trip before its first products
  uint32_t cbits[2] = {0u, 0u};
  auto row_mask = [&](int ci) -> uint32_t {
    if (ci < nwc) {
      const int n = nw - 32 * ci;
      return n >= 32 ? 0xffffffffu : (1u << n) - 1u;
    }
    const int cc = ci - nwc;
    return (uint32_t)__builtin_amdgcn_readlane(cc < 64 ? cbits[0] : cbits[1], cc & 63);
  };
  // K operand: row r16 (+16), piece (4c + g) ^ swz = 4 (c ^ (swz >> 2)) + (g ^ (swz & 3));
  // with c = 4 (c >> 2) + j that is byte 256 (c >> 2) + kbj[j] of the row
  const int ksw = row_swz<WD>(r16);
  int kbj[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) kbj[j] = r16 * WROWB + 16 * (g ^ (ksw & 3)) + 64 * (j ^ (ksw >> 2));
  // V^T operand: rows rho (+16), piece (2dt + hb) ^ swz = 2 (dt ^ (swz >> 1)) + (hb ^ (swz & 1))
  const int rho = 4 * g + (r16 >> 2);
  const int vsw = row_swz<WD>(rho);
  const int vbase = rho * WROWB + 16 * (((r16 & 3) >> 1) ^ (vsw & 1)) + 8 * (r16 & 1), vx = vsw >> 1;

  __syncthreads();   // ids and jlast in LDS
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = 64 * h + lane;
    if (c < ncc_all) {   // lane c reads the 32 ids of chunk c (eight 16-byte reads, rotated by lane)
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
  const int ncc = (jlast + 32) >> 5, nch = nwc + ncc;
  float *crow = cmass ? cmass + (int64_t)t * k_eff : nullptr;
  if (crow)   // the skipped chunks' slots hold no id: mass 0
    for (int j = 32 * ncc + tid; j < k_eff; j += WNT) crow[j] = 0.f;
  const int ns = 2 * nch;   // steps: pass 1 over every chunk, then pass 2
  auto chunk_of = [&](int n) { return n < nch ? n : n - nch; };
  auto tile = [&](int n) { return wide_dyn + (n % NTILE) * WTILE; };
  // Loads of the chunk of step n: instruction k of wave w moves row i = w + 4k (1 KiB);
  // lane l writes slot l, which holds the row's piece l ^ row_swz(i).  A step issues the
  // rows it requests one at a time between its QK MFMAs: a burst of eight 1 KiB loads
  // would hold the wave until the memory pipeline's queue takes them.
  struct ChunkReq {
    __amdgpu_buffer_rsrc_t r;
    char *buf;
    int myrow;   // lane l (< 32) holds the KV or compressed row that is chunk row l
  };
  const __amdgpu_buffer_rsrc_t rnone = make_rsrc(kv, 0);   // every load out of range: zeros
  uint32_t d0 = 16 * lane;
  asm volatile("" : "+v"(d0));
  auto request = [&](int n) -> ChunkReq {
    ChunkReq rq;
    rq.buf = tile(n);
    const int ci = chunk_of(n);
    if (n >= ns) {   // nothing left to load: zeros into the free tile
      rq.r = rnone;
      rq.myrow = 0;
    } else if (ci < nwc) {
      rq.r = rkv;
      rq.myrow = w_lo + 32 * ci + (lane & 31);
    } else {
      rq.r = rck;
      rq.myrow = ids_l[32 * (ci - nwc) + (lane & 31)];
    }
    return rq;
  };
  auto issue_row = [&](const ChunkReq &rq, int k) __attribute__((always_inline)) {
    const int i = w + WW * k;
    const uint32_t off = d0 ^ (uint32_t)(16 * row_swz<WD>(i));
    dma16(rq.r, rq.buf + i * WROWB, (uint32_t)__builtin_amdgcn_readlane(rq.myrow, i) * WROWB + off);
  };
  // Every wave issues exactly WRPW row loads per step (before the next step's barrier), so
  // with DIST steps requested ahead
  // "at most WRPW (DIST - 1) vector-memory operations outstanding" means step n's rows
  // have landed (loads complete in order; stores issued in between only make the wait
  // stricter).  After the barrier every wave has finished step n - 1, the last reader
  // (P.V) of the tile of step n - 2 = n + DIST - NTILE, which the new request reuses.
  auto top = [&](int n) -> ChunkReq {
    if (n + DIST - 1 < ns) wait_vmcnt<WRPW * (DIST - 1)>();
    else wait_vmcnt<0>();
    lds_barrier();
    return request(n + DIST);
  };
#pragma unroll
  for (int k = 0; k < DIST; ++k) {
    const ChunkReq rq = request(k);
#pragma unroll
    for (int r = 0; r < WRPW; ++r) issue_row(rq, r);
  }

  // S^T of the chunk of step n for the wave's 32 heads: acc[kt][hi][i] is the logit of
  // key 16 kt + 4 g + i and head 32 w + 16 hi + r16 (unscaled).  at(c, j) runs after MFMA
  // j of K-chunk c, at(-1, 0) before the first (once the first K operands are requested):
  // vector work there runs beside the MFMAs when its inputs and results are tied to that
  // place by empty asm statements, which keep their order with the MFMA statements.  One
  // wave issues in order, so a window between two MFMAs holds best one short instruction
  // or one exponential, none depending on another of the same window.
  auto qk = [&](int n, f32x4 (&acc)[2][2], const ChunkReq &rq, auto &&at) __attribute__((always_inline)) {
    const char *tb = tile(n);
    u32x4 kr[LA][2];
    auto kread = [&](int c, u32x4 (&dst)[2]) __attribute__((always_inline)) {
      const char *kp = tb + kbj[c & 3] + 256 * (c >> 2);   // the rest of the offset is immediate
      dst[0] = *reinterpret_cast<const u32x4 *>(kp);
      dst[1] = *reinterpret_cast<const u32x4 *>(kp + 16 * WROWB);
    };
#pragma unroll
    for (int c = 0; c < LA; ++c) kread(c, kr[c]);
    at(-1, 0);
#pragma unroll
    for (int c = 0; c < WNC; ++c) {
      const u32x4 k0 = kr[c % LA][0], k1 = kr[c % LA][1];
      if (c + LA < WNC) kread(c + LA, kr[c % LA]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {   // acc[kt = j & 1][hi = j >> 1]
        const u32x4 &kk = (j & 1) ? k1 : k0;
        if (c == 0) mfma_v_first(acc[j & 1][j >> 1], kk, qf[j >> 1][c]);
        else mfma_v(acc[j & 1][j >> 1], kk, qf[j >> 1][c]);
        at(c, j);
      }
      if (c % 2 == 1) issue_row(rq, c / 2);
    }
    mfma_v_fence(acc);
  };

  // ------------------------------------------------------------------ pass 1: lse, lse_nc
  float m[2], l[2], m_nc[2], l_nc[2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const float a2 = ok[hi] ? sink[hh[hi]] * LOG2E : NINF;
    m[hi] = a2;
    l[hi] = (g == 0 && a2 > NINF) ? 1.f : 0.f;   // the sink counted once per head
    m_nc[hi] = m[hi];
    l_nc[hi] = l[hi];
  }
  // The logits of a chunk (masked, unscaled) are folded into the running max and sums at
  // the next step, while that step's MFMAs run: the max is raised first (rarely; a branch),
  // then the exponentials are summed beside the MFMAs.
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
      up = up || cmx[hi] * sl2 > m[hi] + RESCALE;   // log2 units (sl2 > 0 keeps the order)
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
  // The sum of value v (head tile v / 8) of the 16: its FMA, exponential and addition in
  // three windows of K-chunk v (j = 0, 1, 3; the sums keep their order)
  float fx[16];
  auto add_sums_step = [&](int v, int j) __attribute__((always_inline)) {
    const int hi = v >> 3, e = v & 7;
    if (j == 0) {
      asm volatile("" : "+v"(sv[hi][e]));
      fx[v] = fmaf(sv[hi][e], sl2, m[hi] == NINF ? 0.f : -m[hi]);
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
  for (int ci = 0; ci < nch; ++ci) {
    const ChunkReq rq = top(ci);
    const uint32_t bm_all = row_mask(ci), bm = bm_all >> (4 * g);   // read before the products
    f32x4 acc[2][2];
    qk(ci, acc, rq, [&](int c, int j) __attribute__((always_inline)) {
      if (c < 0) {   // chunk ci - 1 into the running max, beside the first K reads
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
#pragma unroll
          for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(sv[hi][e]));
        raise_max();
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) asm volatile("" : "+v"(m[hi]), "+v"(l[hi]));
      } else {
        add_sums_step(c, j);
      }
    });
    if (ci == nwc) {   // every window chunk folded
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) { m_nc[hi] = m[hi]; l_nc[hi] = l[hi]; }
    }
    // a head past H keeps finite garbage statistics that are never written
    if (bm_all == 0xffffffffu) {
#pragma unroll
      for (int hi = 0; hi < 2; ++hi)
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[hi][e] = acc[e >> 2][hi][e & 3];
    } else {
#pragma unroll
      for (int hi = 0; hi < 2; ++hi)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          sv[hi][e] = ((bm >> (16 * (e >> 2) + (e & 3))) & 1) ? acc[e >> 2][hi][e & 3] : NINF;
    }
  }
  raise_max();   // the last chunk
#pragma unroll
  for (int v = 0; v < 16; ++v)
#pragma unroll
    for (int j = 0; j < 4; ++j) add_sums_step(v, j);
  if (ncc == 0) {
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) { m_nc[hi] = m[hi]; l_nc[hi] = l[hi]; }
  }
  // lse of the wave's heads (log2 units), -inf for a head with no probability at all
  float nl[2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const float Ls = across_groups_sum(l[hi]), Lnc = across_groups_sum(l_nc[hi]);
    const float lse2 = (m[hi] > NINF && Ls > 0.f) ? m[hi] + __log2f(Ls) : NINF;
    const float lse2_nc = (m_nc[hi] > NINF && Lnc > 0.f) ? m_nc[hi] + __log2f(Lnc) : NINF;
    nl[hi] = (ok[hi] && lse2 > NINF) ? -lse2 : NINF;   // exp2(-inf) = 0
    if (ok[hi] && g == 0) {
      lse[(int64_t)t * H + hh[hi]] = lse2 * LN2;
      lse_nc[(int64_t)t * H + hh[hi]] = lse2_nc * LN2;
    }
  }

  // ------------------------------------------------------- pass 2: P, cmass, then P.V
  f32x4 o[8][8];   // O^T[d = 128 w + 16 dt + 4 g + i][head 16 ht + r16]
#pragma unroll
  for (int ht = 0; ht < 8; ++ht)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[ht][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // P row swizzle of rows 16x + r16 (16-byte key block b at position b ^ psw): with the
  // 16-byte read service order of the LDS every quarter wave hits 16 distinct slots
  const int psw = (2 * ((r16 >> 2) & 1)) ^ (3 * ((r16 >> 3) & 1));
  auto pbuf = [&](int n) { return pbufs + (n & 1) * WPBUF; };
  // P.V operands of the chunk of step n: V^T of the wave's 8 d-tiles by transposing reads
  // (one batch with its wait, at the end of step n: the wait overlaps the step barrier that
  // follows; the tile stays until step n + 2 requests rows) and P^T of the 8 head tiles
  // (read during the last QK MFMAs of step n + 1, behind the barrier that publishes them)
  u32x4 va[8], pb[8];
  auto v_read = [&](int n) __attribute__((always_inline)) {
    const char *base = tile(n);
    int vxs = vx;
    asm volatile("" : "+v"(vxs));
    uint32_t a[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) a[dt] = lds_addr_of(base + vbase + 32 * ((8 * w + dt) ^ vxs));
    uint2 xv[16];
    lds_read_tr16_pairs<16 * WROWB>(xv, a);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) va[dt] = u32x4{xv[2 * dt].x, xv[2 * dt].y, xv[2 * dt + 1].x, xv[2 * dt + 1].y};
  };
  auto pv_read_p = [&](int n) __attribute__((always_inline)) {
    const char *pr = pbuf(n) + r16 * WPROW + 16 * (g ^ psw);
#pragma unroll
    for (int ht = 0; ht < 8; ++ht) pb[ht] = *reinterpret_cast<const u32x4 *>(pr + 16 * ht * WPROW);
  };
  auto pv_mma = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ht = 0; ht < 8; ++ht)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[ht][dt] = mfma16x16x32(va[dt], pb[ht], o[ht][dt]);
  };
  auto flush = [&](int cprev, int nprev) {
    if (crow && cprev >= nwc && tid < 32) {
      const int slot = 32 * (cprev - nwc) + tid;
      if (slot < k_eff) {
        float sum = 0.f;
#pragma unroll
        for (int ww = 0; ww < WW; ++ww) sum += cm_part[nprev & 1][ww][tid];
        crow[slot] = sum;
      }
    }
  };
  // the P buffer the first pass-2 step's P.V reads (there is no chunk before it) holds
  // zeros; its tile holds the last pass-1 chunk's finite rows
  if (nch > 0) {
    for (int i = tid; i < WPBUF / 16; i += WNT) reinterpret_cast<u32x4 *>(pbuf(nch - 1))[i] = u32x4{0, 0, 0, 0};
    v_read(nch - 1);
  }
  for (int ci = 0; ci < nch; ++ci) {
    const int n = nch + ci;
    const ChunkReq rq = top(n);
    if (ci > 0) flush(ci - 1, n - 1);
    // P^T of the chunk before (at the first step: the zeroed P buffer) read during the last
    // QK MFMAs; its V^T operands are in registers since the end of the step before
    const uint32_t bm_all = row_mask(ci), bm = bm_all >> (4 * g);   // read before the products
    f32x4 acc[2][2];
    qk(n, acc, rq, [&](int c, int j) __attribute__((always_inline)) {
      if (c == WNC - 2 && j == 0) pv_read_p(n - 1);
    });
    __builtin_amdgcn_sched_barrier(0);
    // P = exp2(s sl2 - lse) of the chunk, its bf16 copy for P.V and the head sums for
    // cmass, interleaved with the P.V MFMAs of the chunk before (no dependence either way;
    // stores the step does not need go to a spare slot, so the block has no branch)
    float p[2][8];   // [hi][4 kt + i]; a head past H has nl = -inf: P = 0
    if (bm_all != 0xffffffffu) {
#pragma unroll
      for (int hi = 0; hi < 2; ++hi)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (!((bm >> (16 * (e >> 2) + (e & 3))) & 1)) acc[e >> 2][hi][e & 3] = NINF;
    }
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int e = 0; e < 8; ++e) p[hi][e] = fast_exp2(fmaf(acc[e >> 2][hi][e & 3], sl2, nl[hi]));
    // P row 32 w + 16 hi + r16, key block g (MFMA k order: keys 4g..4g+3, 16+4g..16+4g+3)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
      *reinterpret_cast<u32x4 *>(pbuf(n) + (32 * w + 16 * hi + r16) * WPROW + 16 * (g ^ psw)) =
          u32x4{pack2_bf16(p[hi][0], p[hi][1]), pack2_bf16(p[hi][2], p[hi][3]), pack2_bf16(p[hi][4], p[hi][5]),
                pack2_bf16(p[hi][6], p[hi][7])};
    // value e of group g is key 16 (e >> 2) + 4g + (e & 3); lane r16 ends with the head sum
    // of value sum8_index(r16); window chunks and odd lanes store to the spare slot 32
    float ps[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ps[e] = p[0][e] + p[1][e];
    const float sh = group16_sum8(ps, r16);
    const int el = sum8_index(r16);
    const bool cm_on = crow != nullptr && ci >= nwc && (r16 & 1) == 0;
    cm_part[n & 1][w][cm_on ? 16 * (el >> 2) + 4 * g + (el & 3) : 32] = sh;
    pv_mma();
    // one exponential per MFMA (each holds the vector unit for four FMA issue slots), then
    // two other vector instructions per MFMA
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      sched_group<SG_MFMA, 1>();
      sched_group<SG_TRANS, 1>();
      sched_group<SG_VALU, 1>();
    }
#pragma unroll
    for (int k = 16; k < 64; ++k) {
      sched_group<SG_MFMA, 1>();
      sched_group<SG_VALU, 2>();
    }
    __builtin_amdgcn_sched_barrier(0);
    v_read(n);
  }
  wait_vmcnt<0>();   // no load into the LDS outlives the workgroup
  if (nch > 0) {
    __syncthreads();   // the last chunk's P and cmass partials of every wave
    flush(nch - 1, ns - 1);
    pv_read_p(ns - 1);
    pv_mma();
  }

  // ---------------------------------------------------------------- outputs
#pragma unroll
  for (int ht = 0; ht < 8; ++ht) {
    const int h = 16 * ht + r16;
    if (h < H) {
      uint16_t *orow = out + ((int64_t)t * H + h) * WD + 128 * w + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<uint2 *>(orow + 16 * dt) =
            uint2{pack2_bf16(o[ht][dt][0], o[ht][dt][1]), pack2_bf16(o[ht][dt][2], o[ht][dt][3])};
    }
  }
}

template <int NTILE>
static hipError_t launch_wide_t(const LaunchLayout &LL, const void *q, const void *kv, const void *ckv,
                                const float *sink, const int32_t *ids, int k_eff, int window, int H, float scale,
                                void *out, float *lse, float *lse_nc, float *cmass, hipStream_t st) {
  const size_t dyn = wide_attn_lds_bytes(NTILE, k_eff);
  auto kern = sparse_attn_wide_kernel<NTILE>;
  const hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL(kern, dim3((unsigned)LL.total_q), dim3(WNT), dyn, st, LL.dev,
                     static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(kv),
                     static_cast<const uint16_t *>(ckv), sink, ids, k_eff, window, H, LL.total_q, LL.total_k,
                     scale * LOG2E, static_cast<uint16_t *>(out), lse, lse_nc, cmass);
  return hipGetLastError();
}

// four tiles (two chunks requested ahead) where the LDS holds them beside the P buffers,
// the ids and the static arrays, else three
hipError_t launch_sparse_attn_wide(const LaunchLayout &LL, const void *q, const void *kv, const void *ckv,
                                   const float *sink, const int32_t *ids, int k_eff, int window, int H,
                                   float scale, void *out, float *lse, float *lse_nc, float *cmass,
                                   hipStream_t st) {
  constexpr size_t LDS_CU = 160 * 1024, STATIC = 2 * 1024;   // cm_part and jlast
  if (WIDE_NTILE_MAX >= 4 && wide_attn_lds_bytes(4, k_eff) + STATIC <= LDS_CU)
    return launch_wide_t<WIDE_NTILE_MAX>(LL, q, kv, ckv, sink, ids, k_eff, window, H, scale, out, lse, lse_nc,
                                         cmass, st);
  return launch_wide_t<3>(LL, q, kv, ckv, sink, ids, k_eff, window, H, scale, out, lse, lse_nc, cmass, st);
}

}  // namespace csa
