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
// Two kernels per call.  sparse_attn_wide_lse.hip forms every logit once for lse and
// lse_nc; this kernel forms them again for P = exp(s - lse), the output and cmass.
//
// One workgroup of four waves (one per SIMD, each with the whole 512-entry register file:
// 256 VGPRs and 256 AGPRs) per query row.  The row's KV rows are staged 32 at a time (one
// "chunk", 32 KiB) in a ring of three or four LDS tiles by direct buffer->LDS loads, the
// chunk two or three steps ahead requested right after each step's barrier.  With one KV
// row shared by every head, the cost that matters is LDS reads per MFMA; a wave holding
// the Q rows of 32 heads in registers reads each K operand once for four MFMAs.  Per chunk:
// S^T = K Q^T for the wave's heads [32 w, 32 w + 32) over all 32 keys, P = exp(s - lse)
// written as bf16 to an LDS buffer holding the chunk's P for all 128 heads, its head sums
// added into cmass.  One step later (behind the next barrier) wave w accumulates the
// output columns [128 w, 128 w + 128) of every head in AGPRs: O^T[d, h] += V^T[d, j] P^T[j, h],
// V^T read with the transposing LDS read (8 KiB per chunk, at the end of the chunk's own
// step) and P^T with 16-byte reads (8 KiB per chunk).  Those 64 MFMAs do not depend on the
// chunk's softmax, so the two are interleaved.
//
// LDS per query and 32-key chunk: 128 KiB of K reads plus 64 KiB of V and P; the 16-byte
// pieces of a tile row are XOR-swizzled (row_swz) so the K reads, the transposing V reads
// and the staging writes are free of bank conflicts, and P row h keeps its 16-byte key
// blocks XOR-swizzled by a function of h for the same reason (16 lanes reading 16 rows of
// 64 bytes).
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
constexpr int WIDS = 8;                 // ids per thread in the first batch (2,048 slots)
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
// S^T products: the asm-statement MFMAs of common.h (mfma_v_first, mfma_v, mfma_v_fence).
// The builtin would take the accumulator form the output tiles need (AGPRs, all 256 of
// them), which pushes 16 output registers into VGPRs and copies them through AGPRs around
// every step; as asm statements the S^T tiles stay in VGPRs.
}  // namespace

// NTILE tiles in the ring: chunks are requested NTILE - 1 steps ahead (a tile is last read
// at the end of its own step, by the V^T reads)
// (the id slots: whole chunks, at least the first batch's WIDS * WNT)
size_t wide_attn_lds_bytes(int ntile, int k_eff) {
  const int ncc = (k_eff + 31) / 32;
  return (size_t)ntile * WTILE + 2 * (size_t)WPBUF + (size_t)max(ncc * 32, WIDS * WNT) * sizeof(int);
}

template <int NTILE>
__global__ __launch_bounds__(WNT, 1) void sparse_attn_wide_kernel(
    LayoutDev L, const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const uint16_t *__restrict__ ckv, const int32_t *__restrict__ ids, int k_eff, int window, int H,
    int total_q, int total_k, float sl2, const float *__restrict__ lse, uint16_t *__restrict__ out,
    float *__restrict__ cmass) {
  constexpr float NINF = -__builtin_inff();
  extern __shared__ __attribute__((aligned(16))) char wide_dyn[];   // tiles, P buffers, ids
  constexpr int DIST = NTILE - 1;          // request distance in steps
  char *pbufs = wide_dyn + NTILE * WTILE;
  int *ids_l = reinterpret_cast<int *>(pbufs + 2 * WPBUF);
  __shared__ float cm_part[2][WW][33];   // slot 32: spare target of stores not needed
  __shared__ int jlast;
  __shared__ uint32_t cmask[128];   // key masks of the compressed chunks

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

  // Requested in order, so that each wait covers only what it needs: the first kernel's lse
  // of the wave's heads, the first WIDS ids of each thread, the Q^T operands; only then are
  // the ids stored (slots past k_eff hold -1; a buffer load past k_eff returns 0)
  float lsev[2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) lsev[hi] = lse[(int64_t)t * H + (ok[hi] ? hh[hi] : 0)];
  if (tid == 0) jlast = -1;
  const __amdgpu_buffer_rsrc_t rid = make_rsrc(ids + (int64_t)t * k_eff, (uint32_t)k_eff * 4);
  int x[WIDS];
#pragma unroll
  for (int u = 0; u < WIDS; ++u) x[u] = __builtin_amdgcn_raw_buffer_load_b32(rid, (tid + u * WNT) * 4, 0, 0);
  asm volatile("" ::: "memory");
  // Q^T operands of both head tiles; piece c of lane group g holds features
  // [(4c+g)*8, +8) (a head past H loads head 0's row: its logits are masked)
  u32x4 qf[2][WNC];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(q + ((int64_t)t * H + (ok[hi] ? hh[hi] : 0)) * WD) + g;
#pragma unroll
    for (int c = 0; c < WNC; ++c) qf[hi][c] = p[4 * c];
  }
  asm volatile("" ::: "memory");
  lds_barrier();   // jlast initialised
  {
    // jlast = the last slot that holds an id (compressed chunks after it have no row and are
    // skipped): the wave's maximum, then one LDS atomic per wave
    int jl = -1;
    auto put = [&](int j, int v) __attribute__((always_inline)) {   // no branch: the loads stay above Q's
      const int id = j < k_eff ? v : -1;
      ids_l[j] = id;
      jl = id >= 0 ? j : jl;
    };
#pragma unroll
    for (int u = 0; u < WIDS; ++u) put(tid + u * WNT, x[u]);
    for (int j = tid + WIDS * WNT; j < ncc_all * 32; j += WNT) put(j, __builtin_amdgcn_raw_buffer_load_b32(rid, j * 4, 0, 0));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) jl = max(jl, __shfl_xor(jl, m, 64));
    if (lane == 0 && jl >= 0) atomicMax(&jlast, jl);
  }
  // exp2 offsets of the wave's heads (-inf for a head with no probability at all, or past
  // H: P = 0), complete before the steps (whose waits count only the row loads)
  float nl[2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const float l2 = ok[hi] ? lsev[hi] * LOG2E : NINF;
    nl[hi] = l2 > NINF ? -l2 : NINF;
    asm volatile("" : "+v"(nl[hi]));
  }
  const __amdgpu_buffer_rsrc_t rkv = make_rsrc(kv, (uint32_t)(t + 1) * WROWB);   // rows past t: zeros
  const __amdgpu_buffer_rsrc_t rck = make_rsrc(ckv, (uint32_t)total_k * WROWB);  // id -1: past the end
  // key mask of chunk ci (bit b: slot b holds a row): the window chunks' from nw, the
  // compressed chunks' from a table built once from the staged ids below (cmask, at most
  // 128 chunks).  No branch: the table is read at a clamped index every time (cmask_raw,
  // issued by a step before its V^T batch, whose wait covers it) and the choice is a select
  auto cmask_raw = [&](int ci) -> uint32_t { return cmask[(ci - nwc) & 127]; };
  auto row_mask = [&](int ci, uint32_t raw) -> uint32_t {
    const int n = max(min(nw - 32 * ci, 32), 0);
    const uint32_t win = (uint32_t)(((uint64_t)1 << n) - 1);
    const uint32_t cm = (uint32_t)__builtin_amdgcn_readfirstlane(raw);
    return ci < nwc ? win : cm;
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

  lds_barrier();   // ids and jlast in LDS (the Q loads stay in flight)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = 64 * h + lane;
    if (c < ncc_all && w == 0) {   // lane c reads the 32 ids of chunk c (eight 16-byte reads, rotated by lane)
      uint32_t m = 0;
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int vv = (v + lane) & 7;
        const int4 x = reinterpret_cast<const int4 *>(ids_l + 32 * c)[vv];
        m |= (uint32_t)(x.x >= 0) << (4 * vv) | (uint32_t)(x.y >= 0) << (4 * vv + 1) |
             (uint32_t)(x.z >= 0) << (4 * vv + 2) | (uint32_t)(x.w >= 0) << (4 * vv + 3);
      }
      cmask[c] = m;
    }
  }
  const int ncc = (jlast + 32) >> 5, nch = nwc + ncc;
  float *crow = cmass ? cmass + (int64_t)t * k_eff : nullptr;
  if (crow)   // the skipped chunks' slots hold no id: mass 0
    for (int j = 32 * ncc + tid; j < k_eff; j += WNT) crow[j] = 0.f;
  const int ns = nch;   // one step per chunk
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
    if (n >= ns) {   // nothing left to load: zeros into the free tile
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
    const int i = w + WW * k;
    const uint32_t off = d0 ^ (uint32_t)(16 * row_swz<WD>(i));
    dma16(rq.r, rq.buf + i * WROWB, (uint32_t)__builtin_amdgcn_readlane(rq.myrow, i) * WROWB + off);
  };
  // Every wave issues exactly WRPW row loads per step (before the next step's barrier), so
  // with DIST steps requested ahead
  // "at most WRPW (DIST - 1) vector-memory operations outstanding" means step n's rows
  // have landed (loads complete in order; stores issued in between only make the wait
  // stricter).  After the barrier every wave has finished step n - 1, whose tile (read last
  // by the V^T reads at that step's end) the new request reuses: n + DIST - NTILE = n - 1.
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

  // ------------------------------------------------------- P, cmass, then P.V
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
  // (one batch with its wait, at the end of step n: the next step's request reuses the
  // tile) and P^T of the 8 head tiles
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
  // the first step's P.V (there is no chunk before it) multiplies zeros: its P buffer
  // (that of step -1) is cleared, its V^T operands are zero
  for (int i = tid; i < WPBUF / 16; i += WNT) reinterpret_cast<u32x4 *>(pbuf(-1))[i] = u32x4{0, 0, 0, 0};
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) va[dt] = u32x4{0, 0, 0, 0};
  lds_barrier();   // the mask table (written by wave 0)
  uint32_t raw_next = cmask_raw(0);
  for (int ci = 0; ci < nch; ++ci) {
    const int n = ci;
    const ChunkReq rq = top(n);
    if (ci > 0) flush(ci - 1, n - 1);
    // P^T of the chunk before (at the first step: the zeroed P buffer) read during the last
    // QK MFMAs; its V^T operands are in registers since the end of the step before
    const uint32_t bm_all = row_mask(ci, raw_next), bm = bm_all >> (4 * g);
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
    // LDS reads before the V^T batch, whose wait covers them: the next chunk's key mask
    // (past the last: unused) and the cmass partials of the chunk before (published by this
    // step's barrier, overwritten only after the next one)
    raw_next = cmask_raw(ci + 1);
    v_read(n);
  }
  wait_vmcnt<0>();   // no load into the LDS outlives the workgroup
  // every wave's loads have landed and its tile reads are done: the tiles are free below
  __syncthreads();   // (also: the last chunk's P and cmass partials of every wave)
  if (nch > 0) {
    flush(nch - 1, ns - 1);
    pv_read_p(ns - 1);
    pv_mma();
  }

  // ---------------------------------------------------------------- outputs
  // O^T of the wave's d-quarter goes through its own 16 KiB of the freed tiles, 64 heads at
  // a time: bf16 rows [head][128 d] of 256 bytes whose 16-byte pieces are XOR-swizzled by
  // head (the 8-byte writes of 32 lanes then cover all 64 banks once), read back 16 bytes
  // per lane, so that each store writes four whole 256-byte row segments (stores of
  // 16 head rows x 32 bytes each were several times slower)
  char *ob = wide_dyn + w * (64 * 256);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int hq = 0; hq < 4; ++hq) {
      const int ht = 4 * half + hq;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<uint2 *>(ob + (16 * hq + r16) * 256 + 16 * ((2 * dt + (g >> 1)) ^ r16) + 8 * (g & 1)) =
            uint2{pack2_bf16(o[ht][dt][0], o[ht][dt][1]), pack2_bf16(o[ht][dt][2], o[ht][dt][3])};
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {   // rows 4 i + (lane >> 4), logical piece lane & 15
      const int row = 4 * i + (lane >> 4), pc = lane & 15;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(ob + row * 256 + 16 * (pc ^ (row & 15)));
      const int h = 64 * half + row;
      if (h < H) *reinterpret_cast<u32x4 *>(out + ((int64_t)t * H + h) * WD + 128 * w + 8 * pc) = v;
    }
  }
}

template <int NTILE>
static hipError_t launch_wide_t(const LaunchLayout &LL, const void *q, const void *kv, const void *ckv,
                                const int32_t *ids, int k_eff, int window, int H, float scale, const float *lse,
                                void *out, float *cmass, hipStream_t st) {
  const size_t dyn = wide_attn_lds_bytes(NTILE, k_eff);
  auto kern = sparse_attn_wide_kernel<NTILE>;
  const hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL(kern, dim3((unsigned)LL.total_q), dim3(WNT), dyn, st, LL.dev,
                     static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(kv),
                     static_cast<const uint16_t *>(ckv), ids, k_eff, window, H, LL.total_q, LL.total_k,
                     scale * LOG2E, lse, static_cast<uint16_t *>(out), cmass);
  return hipGetLastError();
}

// lse and lse_nc first (their own kernel), then P, out and cmass: four tiles (three chunks
// requested ahead) where the LDS holds them beside the P buffers, the ids and the static
// arrays, else three
hipError_t launch_sparse_attn_wide(const LaunchLayout &LL, const void *q, const void *kv, const void *ckv,
                                   const float *sink, const int32_t *ids, int k_eff, int window, int H,
                                   float scale, void *out, float *lse, float *lse_nc, float *cmass,
                                   hipStream_t st) {
  const hipError_t e = launch_sparse_attn_wide_lse(LL, q, kv, ckv, sink, ids, k_eff, window, H, scale, lse, lse_nc, st);
  if (e != hipSuccess) return e;
  constexpr size_t LDS_CU = 160 * 1024, STATIC = 2 * 1024;   // cm_part and jlast
  if (WIDE_NTILE_MAX >= 4 && wide_attn_lds_bytes(4, k_eff) + STATIC <= LDS_CU)
    return launch_wide_t<WIDE_NTILE_MAX>(LL, q, kv, ckv, ids, k_eff, window, H, scale, lse, out, cmass, st);
  return launch_wide_t<3>(LL, q, kv, ckv, ids, k_eff, window, H, scale, lse, out, cmass, st);
}

}  // namespace csa
