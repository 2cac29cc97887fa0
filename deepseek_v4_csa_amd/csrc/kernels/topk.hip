// Per-row top-k with lowest-index ties, ascending global ids and -1 padding.
//
// K_t = min(k_eff, n_valid(t)) largest scores among the causally visible columns
// (k = min(index_topk, n_compressed): csa.py excerpts of the page "[Bug] DSV4 unfused
// CSA indexer loss uses a compressed-only teacher ..."; picks beyond the causal limit
// are -1 in its sparse-attention excerpt); ids are global, cu_k[s] + j (page
// "Megatron-LM pull request 8539", item 1).
//
// One workgroup (512 threads) per row; the row's visible scores sit in registers as
// order-preserving uint32 keys.  The k-th largest key is found by radix selection on
// (key - row_min_key), starting at the highest set bit of (max - min) so the first
// 8-bit digit already spreads the values over the histogram (the raw top byte of
// same-sign floats of similar magnitude would put them all in one or two bins).
// Ties at the threshold are resolved by index order with a block prefix count, and
// the selected ids are compacted in ascending order.
#include "common.h"
#include "wave_select.h"
#include "../launch.h"

namespace csa {

constexpr int TK_THREADS = 512;   // 256 and 1,024 measured slower on 16k-key rows
constexpr int TK_WAVES = TK_THREADS / 64;

// One workgroup per row (rows above 4096 keys).  Each lane holds vpt = ceil(n / 512) <= VPT
// of the row's n visible keys (the rows of one launch differ in length, and every pass
// below runs over vpt slots, not VPT); wave w owns the contiguous run of keys
// j = 64 vpt w + 64 v + lane (key[v] of the lane), so every load instruction reads 256
// bytes of the row contiguously and index order is wave, then v, then lane.  The radix
// passes stop as soon as the threshold bin is taken whole.  Compaction: each wave counts
// its keys above the threshold and its ties (ballot popcounts), the waves' totals pass
// through LDS once, and each lane places its picks at its wave's offset plus the running
// counts of the wave's earlier v plus its mbcnt rank.
// the float whose order-preserving key is k (the inverse of ordered_key)
__device__ __forceinline__ float float_of_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// SEL: the selected scores are written too (sel, slot-aligned with ids)
template <int VPT, bool SEL>
__global__ __launch_bounds__(TK_THREADS) void topk_kernel(LayoutDev L, const float *__restrict__ scores,
                                                          int64_t ld, int k_eff, int32_t *__restrict__ ids,
                                                          float *__restrict__ sel) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t red[2 * TK_WAVES];
  __shared__ int wtot[2 * TK_WAVES];
  __shared__ uint32_t sel_digit, sel_above, sel_cnt;

  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const RowGeo g = row_geo(L, t);
  const int n = g.n_valid;
  // slots in use (uniform; the loops below stop at vpt).  At VPT = 64 a run-time bound
  // leaves the compiler unable to keep key[] in registers, so those rows take all slots
  const int vpt = VPT >= 64 ? VPT : min(VPT, (n + 64 * TK_WAVES - 1) / (64 * TK_WAVES));
  auto jof = [&](int v) { return 64 * vpt * w + 64 * v + lane; };
  int32_t *out = ids + (int64_t)t * k_eff;
  float *sout = SEL ? sel + (int64_t)t * k_eff : nullptr;
  const float *row = scores + (int64_t)t * ld;
  if (n <= k_eff) {  // every visible key is selected
    for (int j = tid; j < k_eff; j += TK_THREADS) {
      out[j] = j < n ? g.k_base + j : -1;
      if constexpr (SEL) sout[j] = j < n ? row[j] : -__builtin_inff();
    }
    return;
  }

  // the row through a buffer resource of exactly n floats: the loads are unconditional
  // (past n they read zeros), so all VPT of them are in flight at once -- a load under a
  // per-slot branch would be waited for before the next one is issued
  const __amdgpu_buffer_rsrc_t rrow = make_rsrc(row, (uint32_t)n * 4);
  uint32_t key[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v)
    key[v] = v < vpt ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rrow, jof(v) * 4, 0, 0) : 0u;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const bool in = v < vpt && jof(v) < n;
    key[v] = in ? ordered_key(__uint_as_float(key[v])) : 0u;
    kmin = in ? min(kmin, key[v]) : kmin;
    kmax = in ? max(kmax, key[v]) : kmax;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, m, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, m, 64));
  }
  if (lane == 0) { red[w] = kmin; red[TK_WAVES + w] = kmax; }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TK_WAVES; ++i) { kmin = min(kmin, red[i]); kmax = max(kmax, red[TK_WAVES + i]); }
#pragma unroll
  for (int v = 0; v < VPT; ++v) key[v] -= kmin;  // relative keys (garbage where j >= n)

  // radix selection of the k-th largest relative key
  const uint32_t range = kmax - kmin;
  uint32_t thr = 0;       // known high bits of the threshold (relative key)
  int need = k_eff;       // elements still to take among those matching `thr`
  int cur = range ? 32 - __builtin_clz(range) : 0;   // bits above `cur` are all equal
  bool whole = false;     // the last threshold bin was taken whole
  while (cur > 0) {
    const int width = cur < 8 ? cur : 8;
    const int sh = cur - width;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      if (v >= vpt) break;
      const bool in_play = jof(v) < n && (cur >= 32 || (key[v] >> cur) == thr);
      if (in_play) atomicAdd(&hist[(key[v] >> sh) & ((1u << width) - 1u)], 1u);
    }
    __syncthreads();
    if (w == 0) {
      const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2], c3 = hist[4 * lane + 3];
      const uint32_t mine = c0 + c1 + c2 + c3;
      uint32_t suf = mine;  // sum over lanes >= lane
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = (uint32_t)__shfl_down((int)suf, o, 64);
        if (lane + o < 64) suf += y;
      }
      uint32_t above = suf - mine;  // bins held by higher lanes
      if (above < (uint32_t)need && suf >= (uint32_t)need) {
        uint32_t d;
        if (above + c3 >= (uint32_t)need) d = 3;
        else if ((above += c3) + c2 >= (uint32_t)need) d = 2;
        else if ((above += c2) + c1 >= (uint32_t)need) d = 1;
        else { above += c1; d = 0; }
        sel_digit = 4 * lane + d;
        sel_above = above;
        sel_cnt = d == 3 ? c3 : d == 2 ? c2 : d == 1 ? c1 : c0;
      }
    }
    __syncthreads();
    thr = (thr << width) | sel_digit;
    need -= (int)sel_above;
    cur = sh;
    const bool done = (uint32_t)need == sel_cnt;
    __syncthreads();
    if (done) { whole = true; break; }
  }

  // compaction in index order: keys whose prefix (bits >= cur) is above thr -- or equal to
  // it when the bin was taken whole -- and the first `need` ties otherwise
  // (the ballots are taken twice rather than kept: 2 * VPT 64-bit masks would not fit the
  // scalar registers)
  auto ballots = [&](int v, uint64_t &bg, uint64_t &be) __attribute__((always_inline)) {
    const bool valid = jof(v) < n;
    const uint32_t kp = key[v] >> cur;
    bg = __ballot(valid && (kp > thr || (whole && kp == thr)));
    be = __ballot(valid && !whole && kp == thr);
  };
  // the wave's totals, then every wave's offset from the waves before it
  int tg = 0, te = 0;
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    if (v >= vpt) break;
    uint64_t bg, be;
    ballots(v, bg, be);
    tg += __popcll(bg);
    te += __popcll(be);
  }
  if (lane == 0) { wtot[w] = tg; wtot[TK_WAVES + w] = te; }
  __syncthreads();
  int og = 0, oe = 0;
#pragma unroll
  for (int i = 0; i < TK_WAVES; ++i) {
    og += i < w ? wtot[i] : 0;
    oe += i < w ? wtot[TK_WAVES + i] : 0;
  }
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    if (v >= vpt) break;
    uint64_t bg, be;
    ballots(v, bg, be);
    const int gt_before = og + __builtin_amdgcn_mbcnt_hi((uint32_t)(bg >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bg, 0));
    const int eq_before = oe + __builtin_amdgcn_mbcnt_hi((uint32_t)(be >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)be, 0));
    const bool gt = (bg >> lane) & 1, eq = (be >> lane) & 1;
    const bool sel_ = gt || (eq && eq_before < need);
    const int pos = gt_before + min(eq_before, need);
    og += __popcll(bg);
    oe += __popcll(be);
    if (sel_ && pos < k_eff) {
      out[pos] = g.k_base + jof(v);
      if constexpr (SEL) sout[pos] = float_of_key(key[v] + kmin);
    }
  }
}

// One wave per row (rows up to 64*VPL visible keys): the same selection as above with
// wave-level primitives only (wave_select), so there is no workgroup barrier.  The row's
// loads are issued before its geometry is known (every column below max_seqlen_k exists).
template <int VPL, bool SEL>
__global__ __launch_bounds__(256) void topk_wave_kernel(LayoutDev L, int T, const float *__restrict__ scores,
                                                        int64_t ld, int max_sk, int k_eff,
                                                        int32_t *__restrict__ ids, float *__restrict__ sel) {
  __shared__ __attribute__((aligned(16))) uint32_t hist_all[4][256];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;
  if (t >= T) return;
  const float *row = scores + (int64_t)t * ld;
  float val[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int j = v * 64 + lane;
    val[v] = j < max_sk ? row[j] : 0.f;
  }
  const RowGeo g = row_geo(L, t);
  const int n = g.n_valid;
  int32_t *out = ids + (int64_t)t * k_eff;
  float *sout = SEL ? sel + (int64_t)t * k_eff : nullptr;
  if (n <= k_eff) {  // every visible key is selected
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int j = v * 64 + lane;
      if (j < k_eff) {
        out[j] = j < n ? g.k_base + j : -1;
        if constexpr (SEL) sout[j] = j < n ? val[v] : -__builtin_inff();
      }
    }
    return;
  }
  if constexpr (SEL) {
    wave_select<VPL>(val, n, k_eff, hist_all[w], [&](int pos, int j, int v) {
      out[pos] = g.k_base + j;
      sout[pos] = val[v];
    });
  } else {
    wave_select<VPL>(val, n, k_eff, hist_all[w], [&](int pos, int j, int) { out[pos] = g.k_base + j; });
  }
}

bool topk_supported(int max_seqlen_k, int k_eff) { return max_seqlen_k <= 16384 && k_eff >= 0; }

hipError_t launch_topk(const LaunchLayout &LL, const float *scores, int64_t ld, int k_eff,
                       int32_t *ids, float *sel, hipStream_t st) {
  if (LL.total_q == 0 || k_eff == 0) return hipSuccess;
  if (LL.max_seqlen_k <= 64 * 64) {  // one wave per row
    const int vpl = (LL.max_seqlen_k + 63) / 64;
    const dim3 wgrid((unsigned)((LL.total_q + 3) / 4));
#define CSA_TOPKW_CASE(V)                                                                            \
    if (vpl <= V) {                                                                                  \
      if (sel)                                                                                       \
        hipLaunchKernelGGL((topk_wave_kernel<V, true>), wgrid, dim3(256), 0, st, LL.dev, LL.total_q, \
                           scores, ld, LL.max_seqlen_k, k_eff, ids, sel);                            \
      else                                                                                           \
        hipLaunchKernelGGL((topk_wave_kernel<V, false>), wgrid, dim3(256), 0, st, LL.dev, LL.total_q, \
                           scores, ld, LL.max_seqlen_k, k_eff, ids, sel);                            \
      return hipGetLastError();                                                                      \
    }
    CSA_TOPKW_CASE(4)
    CSA_TOPKW_CASE(8)
    CSA_TOPKW_CASE(16)
    CSA_TOPKW_CASE(32)
    CSA_TOPKW_CASE(64)
#undef CSA_TOPKW_CASE
  }
  const int per = (LL.max_seqlen_k + TK_THREADS - 1) / TK_THREADS;
  dim3 grid((unsigned)LL.total_q), block(TK_THREADS);
#define CSA_TOPK_CASE(V)                                                                         \
  if (per <= V) {                                                                                \
    if (sel)                                                                                     \
      hipLaunchKernelGGL((topk_kernel<V, true>), grid, block, 0, st, LL.dev, scores, ld, k_eff, ids, sel); \
    else                                                                                         \
      hipLaunchKernelGGL((topk_kernel<V, false>), grid, block, 0, st, LL.dev, scores, ld, k_eff, ids, sel); \
    return hipGetLastError();                                                                    \
  }
  CSA_TOPK_CASE(1)
  CSA_TOPK_CASE(2)
  CSA_TOPK_CASE(4)
  CSA_TOPK_CASE(8)
  CSA_TOPK_CASE(16)
  CSA_TOPK_CASE(32)
  CSA_TOPK_CASE(64)
#undef CSA_TOPK_CASE
  return hipErrorInvalidValue;
}

}  // namespace csa
