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
// One workgroup (8 waves) per query row; the row's KV rows are staged 32 at a time (one
// "chunk", 32 KiB) in a ring of three or four LDS tiles by direct buffer->LDS loads, the
// chunk one or two steps ahead requested right after each step's barrier.  With one KV row shared by every head
// the cost that matters is LDS reads per MFMA, so the two passes are organised to read
// each operand from LDS as few times as the registers allow:
//
//  pass 1 (lse and lse_nc, no output accumulators needed): waves 2p and 2p+1 share 32
//    heads (their own 16 and their partner's 16) and split every chunk's keys between
//    them (rows 0..15 / 16..31): each K operand read feeds two MFMAs and each wave reads
//    half a chunk.  Each keeps a running max (raised lazily, by 2^8 or more) and sum per
//    head; the two halves are combined through LDS at the end.
//  pass 2 (P, out and cmass, with lse final): wave w forms P = exp(s - lse) of its own 16
//    heads over the whole chunk (S^T = K Q^T on MFMA), writes it as bf16 to an LDS
//    buffer holding the chunk's P for all 128 heads, and adds its head sums into cmass.
//    One step later (behind the next barrier) wave w accumulates the output columns
//    [64 w, 64 w + 64) of every head: O^T[d, h] += V^T[d, j] P^T[j, h], V^T read with the
//    transposing LDS read (4 KiB per chunk) and P^T with 16-byte reads (8 KiB per chunk),
//    instead of every wave reading all 32 KiB of the chunk's V for its own heads.
//
// LDS per query and 32-key chunk: pass 1 reads 128 KiB of K, pass 2 256 KiB of K plus
// 96 KiB of V and P; the 16-byte pieces of a tile row are XOR-swizzled (row_swz) so the K
// reads, the transposing V reads and the staging writes are free of bank conflicts, and
// P row h keeps its 16-byte key blocks XOR-swizzled by a function of h for the same reason
// (16 lanes reading 16 rows of 64 bytes).
#include <hip/hip_runtime.h>

#include "common.h"
#include "../launch.h"

namespace csa {

namespace {
constexpr int WD = 512;                 // head dim
constexpr int WHG = 8;                  // waves per workgroup
constexpr int WNT = 64 * WHG;           // threads
constexpr int WROWB = WD * 2;           // bytes per KV row (1 KiB)
constexpr int WTILE = 32 * WROWB;       // one 32-row chunk (32 KiB)
constexpr int WPROW = 64;               // bytes per P row (32 keys, bf16)
constexpr int WPBUF = 128 * WPROW;      // P of one chunk for 128 heads (8 KiB)
constexpr int WNC = WD / 32;            // MFMA K-chunks per row
#ifndef WIDE_NTILE_MAX
#define WIDE_NTILE_MAX 4
#endif
#ifndef WIDE_LA1
#define WIDE_LA1 4
#endif
#ifndef WIDE_LA2
#define WIDE_LA2 3
#endif
#ifndef WIDE_LAP
#define WIDE_LAP 2
#endif
constexpr int LA1 = WIDE_LA1;   // pass 1: K operands requested ahead (one per K-chunk)
constexpr int LA2 = WIDE_LA2;   // pass 2: K operand pairs requested ahead
constexpr int LAP = WIDE_LAP;   // P.V: P^T operands requested ahead
// Scheduling groups for the compiler's machine scheduler: the instructions of a region are
// placed in the order of these calls (DS reads issued ahead of the MFMAs that consume them)
constexpr int SG_MFMA = 0x008, SG_DS_READ = 0x100;
template <int MASK, int N> __device__ __forceinline__ void sched_group() {
  __builtin_amdgcn_sched_group_barrier(MASK, N, 0);
}
}  // namespace

// NTILE tiles in the ring: 3 requests the next chunk one step ahead, 4 two steps ahead
// (pass 2 still reads a tile one step after its own, for P.V)
size_t wide_attn_lds_bytes(int ntile, int k_eff) {
  const int ncc = (k_eff + 31) / 32;
  return (size_t)ntile * WTILE + 2 * (size_t)WPBUF + (size_t)ncc * 32 * sizeof(int);
}

template <int NTILE>
__global__ __launch_bounds__(WNT, 2) void sparse_attn_wide_kernel(
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
  __shared__ float cm_part[2][WHG][33];   // slot 32: spare target of stores not needed
  __shared__ float4 stat[2][128];   // per key half and head: m, L, m_nc, L_nc (log2 units)
  __shared__ int jlast;

  const int t = blockIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int kh = w & 1;                         // pass 1: key half of every chunk
  // pass 1 head groups: gi = 0 the wave's own heads 16 w + r16, gi = 1 its partner's
  int h1[2];
  bool ok1[2];
  h1[0] = 16 * w + r16;
  h1[1] = 16 * (w ^ 1) + r16;
  ok1[0] = h1[0] < H;
  ok1[1] = h1[1] < H;
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
  // Q^T operands of both head groups; piece c of lane group g holds features
  // [(4c+g)*8, +8) (a head past H loads head 0's row: its logits are masked)
  u32x4 qf[2][WNC];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(q + ((int64_t)t * H + (ok1[gi] ? h1[gi] : 0)) * WD) + g;
#pragma unroll
    for (int c = 0; c < WNC; ++c) qf[gi][c] = p[4 * c];
  }
  const __amdgpu_buffer_rsrc_t rkv = make_rsrc(kv, (uint32_t)(t + 1) * WROWB);   // rows past t: zeros
  const __amdgpu_buffer_rsrc_t rck = make_rsrc(ckv, (uint32_t)total_k * WROWB);  // id -1: past the end
  // loads of chunk ci: instruction i = w + 8k moves row i (1 KiB); lane l writes slot l,
  // which holds the row's piece l ^ row_swz(i)
  auto issue = [&](int ci, char *buf) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const uint32_t d0 = 16 * ln;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = w + WHG * k;
      const uint32_t off = d0 ^ (uint32_t)(16 * row_swz<WD>(i));
      if (ci < nwc) {
        dma16(rkv, buf + i * 1024, (uint32_t)(w_lo + 32 * ci + i) * WROWB + off);
      } else {
        const int id = ids_l[32 * (ci - nwc) + i];
        dma16(rck, buf + i * 1024, (uint32_t)id * WROWB + off);
      }
    }
  };
  auto row_mask = [&](int ci) -> uint32_t {
    if (ci < nwc) {
      const int n = nw - 32 * ci;
      return n >= 32 ? 0xffffffffu : (1u << n) - 1u;
    }
    return (uint32_t)__ballot(ids_l[32 * (ci - nwc) + (lane & 31)] >= 0);
  };
  // K operand: row r16 (+16), piece (4c + g) ^ swz = 4 (c ^ (swz >> 2)) + (g ^ (swz & 3))
  const int ksw = row_swz<WD>(r16);
  const int kbase = r16 * WROWB + 16 * (g ^ (ksw & 3)), kx = ksw >> 2;
  // V^T operand: rows rho (+16), piece (2dt + hb) ^ swz = 2 (dt ^ (swz >> 1)) + (hb ^ (swz & 1))
  const int rho = 4 * g + (r16 >> 2);
  const int vsw = row_swz<WD>(rho);
  const int vbase = rho * WROWB + 16 * (((r16 & 3) >> 1) ^ (vsw & 1)) + 8 * (r16 & 1), vx = vsw >> 1;

  __syncthreads();   // ids and jlast in LDS
  const int ncc = (jlast + 32) >> 5, nch = nwc + ncc;
  float *crow = cmass ? cmass + (int64_t)t * k_eff : nullptr;
  if (crow)   // the skipped chunks' slots hold no id: mass 0
    for (int j = 32 * ncc + tid; j < k_eff; j += WNT) crow[j] = 0.f;
  const int ns = 2 * nch;   // steps: pass 1 over every chunk, then pass 2
  auto chunk_of = [&](int n) { return n < nch ? n : n - nch; };
  auto tile = [&](int n) { return wide_dyn + (n % NTILE) * WTILE; };
  // Every wave issues exactly 4 row loads per step, so with DIST steps requested ahead
  // "at most 4 (DIST - 1) vector-memory operations outstanding" means step n's rows have
  // landed (loads complete in order; stores issued in between only make the wait stricter).
  // After the barrier every wave has finished step n - 1, the last reader (P.V) of the tile
  // of step n - 2 = n + DIST - NTILE, which the new request reuses.
  auto top = [&](int n) {
    if (n + DIST - 1 < ns) wait_vmcnt<4 * (DIST - 1)>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (n + DIST < ns) issue(chunk_of(n + DIST), tile(n + DIST));
  };
#pragma unroll
  for (int k = 0; k < DIST; ++k)
    if (k < ns) issue(chunk_of(k), tile(k));

  // ------------------------------------------------------------------ pass 1: lse, lse_nc
  float m[2], l[2], m_nc[2], l_nc[2];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const float a2 = ok1[gi] ? sink[h1[gi]] * LOG2E : NINF;
    m[gi] = a2;
    l[gi] = (g == 0 && kh == 0 && a2 > NINF) ? 1.f : 0.f;   // the sink counted once per head
    m_nc[gi] = m[gi];
    l_nc[gi] = l[gi];
  }
  for (int ci = 0; ci < nch; ++ci) {
    top(ci);
    if (ci == nwc) {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) { m_nc[gi] = m[gi]; l_nc[gi] = l[gi]; }
    }
    // this wave's 16 keys (rows 16 kh + 4g + i) for both head groups, unscaled
    const char *kb = tile(ci) + kbase + 16 * kh * WROWB;
    int kxs = kx;
    asm volatile("" : "+v"(kxs));
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    u32x4 kr[LA1];   // K operands requested LA1 K-chunks ahead
#pragma unroll
    for (int c = 0; c < LA1; ++c) kr[c] = *reinterpret_cast<const u32x4 *>(kb + 64 * (c ^ kxs));
    sched_group<SG_DS_READ, LA1>();
#pragma unroll
    for (int c = 0; c < WNC; ++c) {
      const u32x4 k0 = kr[c % LA1];
      if (c + LA1 < WNC) {
        kr[c % LA1] = *reinterpret_cast<const u32x4 *>(kb + 64 * ((c + LA1) ^ kxs));
        sched_group<SG_DS_READ, 1>();
      }
      acc[0] = mfma16x16x32(k0, qf[0][c], acc[0]);
      acc[1] = mfma16x16x32(k0, qf[1][c], acc[1]);
      sched_group<SG_MFMA, 2>();
    }
    const uint32_t bm = (row_mask(ci) >> (16 * kh)) >> (4 * g);
    float sv[2][4];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[gi][i] = (ok1[gi] && ((bm >> i) & 1)) ? acc[gi][i] : NINF;
    float cmx[2];
    bool up = false;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      cmx[gi] = fmaxf(fmaxf(sv[gi][0], sv[gi][1]), fmaxf(sv[gi][2], sv[gi][3]));
      up = up || cmx[gi] * sl2 > m[gi] + RESCALE;   // log2 units (sl2 > 0 keeps the order)
    }
    if (__builtin_expect(__ballot(up) != 0, 0)) {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const float cand = across_groups_max(cmx[gi]) * sl2;
        const float mn = cand > m[gi] + RESCALE ? cand : m[gi];
        l[gi] *= mn == m[gi] ? 1.f : fast_exp2(m[gi] - mn);
        m[gi] = mn;
      }
    }
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const float nms = m[gi] == NINF ? 0.f : -m[gi];
#pragma unroll
      for (int i = 0; i < 4; ++i) l[gi] += fast_exp2(fmaf(sv[gi][i], sl2, nms));
    }
  }
  if (ncc == 0) {
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) { m_nc[gi] = m[gi]; l_nc[gi] = l[gi]; }
  }
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const float Ls = across_groups_sum(l[gi]), Lnc = across_groups_sum(l_nc[gi]);
    if (g == 0 && ok1[gi]) stat[kh][h1[gi]] = make_float4(m[gi], Ls, m_nc[gi], Lnc);
  }
  __syncthreads();   // both key halves' sums of every head
  // lse of the wave's own heads (pass 2): the two halves combined
  const bool ok2 = ok1[0];
  float lse2 = NINF, lse2_nc = NINF;
  if (ok2) {
    const float4 a = stat[0][h1[0]], b = stat[1][h1[0]];
    auto comb = [&](float ma, float la, float mb, float lb) {
      const float mm = fmaxf(ma, mb);
      if (mm == NINF) return NINF;
      const float s = (ma == NINF ? 0.f : la * fast_exp2(ma - mm)) + (mb == NINF ? 0.f : lb * fast_exp2(mb - mm));
      return s > 0.f ? mm + __log2f(s) : NINF;
    };
    lse2 = comb(a.x, a.y, b.x, b.y);
    lse2_nc = comb(a.z, a.w, b.z, b.w);
  }
  const float nl = lse2 > NINF ? -lse2 : NINF;   // exp2(-inf) = 0: no probability at all
  if (ok2 && g == 0) {
    lse[(int64_t)t * H + h1[0]] = lse2 * LN2;
    lse_nc[(int64_t)t * H + h1[0]] = lse2_nc * LN2;
  }

  // ------------------------------------------------------- pass 2: P, cmass, then P.V
  f32x4 o[8][4];   // O^T[d = 64 w + 16 dt + 4g + i][head 16 ht + r16]
#pragma unroll
  for (int ht = 0; ht < 8; ++ht)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[ht][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // P row swizzle of rows 16x + r16 (16-byte key block b at position b ^ psw): with the
  // 16-byte read service order of the LDS every quarter wave hits 16 distinct slots
  const int psw = (2 * ((r16 >> 2) & 1)) ^ (3 * ((r16 >> 3) & 1));
  auto pbuf = [&](int n) { return pbufs + (n & 1) * WPBUF; };
  // O^T += V^T P^T for the chunk of step n (its tile and P buffer)
  auto pv = [&](int n) __attribute__((always_inline)) {
    const char *base = tile(n);
    int vxs = vx;
    asm volatile("" : "+v"(vxs));
    uint2 xv[8];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const uint32_t va = lds_addr_of(base + vbase + 32 * ((4 * w + dt) ^ vxs));
      xv[2 * dt] = lds_read_tr16_nowait_off<0>(va);
      xv[2 * dt + 1] = lds_read_tr16_nowait_off<16 * WROWB>(va);
    }
    lds_tr16_wait(xv);
    u32x4 a[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) a[dt] = u32x4{xv[2 * dt].x, xv[2 * dt].y, xv[2 * dt + 1].x, xv[2 * dt + 1].y};
    const char *pb = pbuf(n) + r16 * WPROW + 16 * (g ^ psw);
    u32x4 br[LAP];   // P^T operands requested LAP head tiles ahead
#pragma unroll
    for (int ht = 0; ht < LAP; ++ht) br[ht] = *reinterpret_cast<const u32x4 *>(pb + 16 * ht * WPROW);
    sched_group<SG_DS_READ, LAP>();
#pragma unroll
    for (int ht = 0; ht < 8; ++ht) {
      const u32x4 b = br[ht % LAP];
      if (ht + LAP < 8) {
        br[ht % LAP] = *reinterpret_cast<const u32x4 *>(pb + 16 * (ht + LAP) * WPROW);
        sched_group<SG_DS_READ, 1>();
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[ht][dt] = mfma16x16x32(a[dt], b, o[ht][dt]);
      sched_group<SG_MFMA, 4>();
    }
  };
  auto flush = [&](int cprev, int nprev) {
    if (crow && cprev >= nwc && tid < 32) {
      const int slot = 32 * (cprev - nwc) + tid;
      if (slot < k_eff) {
        float sum = 0.f;
#pragma unroll
        for (int ww = 0; ww < WHG; ++ww) sum += cm_part[nprev & 1][ww][tid];
        crow[slot] = sum;
      }
    }
  };
  // the P buffer the first pass-2 step's P.V reads (there is no chunk before it) holds
  // zeros; its tile holds the last pass-1 chunk's finite rows
  if (nch > 0)
    for (int i = tid; i < WPBUF / 16; i += WNT) reinterpret_cast<u32x4 *>(pbuf(nch - 1))[i] = u32x4{0, 0, 0, 0};
  for (int ci = 0; ci < nch; ++ci) {
    const int n = nch + ci;
    top(n);
    if (ci > 0) flush(ci - 1, n - 1);
    // S^T for the 32 rows of the chunk and the wave's 16 heads
    const char *base = tile(n);
    int kxs = kx;
    asm volatile("" : "+v"(kxs));
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
    // K operands requested LA K-chunks ahead of their MFMAs (a ring of LA pairs), so that
    // LDS latency overlaps the MFMAs instead of being paid before each of them
    u32x4 kr[LA2][2];
    auto kread = [&](int c, u32x4 (&dst)[2]) __attribute__((always_inline)) {
      const char *kp = base + kbase + 64 * (c ^ kxs);
      dst[0] = *reinterpret_cast<const u32x4 *>(kp);
      dst[1] = *reinterpret_cast<const u32x4 *>(kp + 16 * WROWB);
    };
#pragma unroll
    for (int c = 0; c < LA2; ++c) kread(c, kr[c]);
    sched_group<SG_DS_READ, 2 * LA2>();
#pragma unroll
    for (int c = 0; c < WNC; ++c) {
      const u32x4 k0 = kr[c % LA2][0], k1 = kr[c % LA2][1];
      if (c + LA2 < WNC) {
        kread(c + LA2, kr[c % LA2]);
        sched_group<SG_DS_READ, 2>();
      }
      acc0 = mfma16x16x32(k0, qf[0][c], acc0);
      acc1 = mfma16x16x32(k1, qf[0][c], acc1);
      sched_group<SG_MFMA, 2>();
    }
    // Masking, P, its bf16 copy for P.V, the head sums for cmass and the P.V of the chunk
    // before form one branch-free block (stores the step does not need go to a spare
    // slot), so the compiler can overlap the vector work of this chunk with the MFMAs of
    // the previous chunk's P.V.
    const uint32_t bm = row_mask(ci);
    const uint32_t m0 = ok2 ? (bm >> (4 * g)) : 0u, m1 = ok2 ? (bm >> (16 + 4 * g)) : 0u;
    float p[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = ((m0 >> i) & 1) ? acc0[i] : NINF;
      p[4 + i] = ((m1 >> i) & 1) ? acc1[i] : NINF;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(p[e], sl2, nl));
    // P row 16 w + r16, key block g (MFMA k order: keys 4g..4g+3, 16+4g..16+4g+3)
    *reinterpret_cast<u32x4 *>(pbuf(n) + (16 * w + r16) * WPROW + 16 * (g ^ psw)) =
        u32x4{pack2_bf16(p[0], p[1]), pack2_bf16(p[2], p[3]), pack2_bf16(p[4], p[5]), pack2_bf16(p[6], p[7])};
    // value e of group g is row 16 (e >> 2) + 4g + (e & 3); lane r16 ends with the head sum
    // of value sum8_index(r16); window chunks and odd lanes store to the spare slot 32
    const float sh = group16_sum8(p, r16);
    const int el = sum8_index(r16);
    const bool cm_on = crow != nullptr && ci >= nwc && (r16 & 1) == 0;
    cm_part[n & 1][w][cm_on ? 16 * (el >> 2) + 4 * g + (el & 3) : 32] = sh;
    // P.V of the chunk before (at the first step: a zeroed P buffer)
    pv(n - 1);
  }
  if (nch > 0) {
    __syncthreads();   // the last chunk's P and cmass partials of every wave
    flush(nch - 1, ns - 1);
    pv(ns - 1);
  }

  // ---------------------------------------------------------------- outputs
#pragma unroll
  for (int ht = 0; ht < 8; ++ht) {
    const int h = 16 * ht + r16;
    if (h < H) {
      uint16_t *orow = out + ((int64_t)t * H + h) * WD + 64 * w + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
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
  constexpr size_t LDS_CU = 160 * 1024, STATIC = 8 * 1024;
  if (WIDE_NTILE_MAX >= 4 && wide_attn_lds_bytes(4, k_eff) + STATIC <= LDS_CU)
    return launch_wide_t<WIDE_NTILE_MAX>(LL, q, kv, ckv, sink, ids, k_eff, window, H, scale, out, lse, lse_nc,
                                         cmass, st);
  return launch_wide_t<3>(LL, q, kv, ckv, sink, ids, k_eff, window, H, scale, out, lse, lse_nc, cmass, st);
}

}  // namespace csa
