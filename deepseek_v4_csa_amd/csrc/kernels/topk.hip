// Per-row top-k with lowest-index ties, ascending global ids and -1 padding.
//
// K_t = min(k_eff, n_valid(t)) largest scores among the causally visible columns
// (k = min(index_topk, n_compressed): csa.py excerpts of the page "[Bug] DSV4 unfused
// CSA indexer loss uses a compressed-only teacher ..."; picks beyond the causal limit
// are -1 in its sparse-attention excerpt); ids are global, cu_k[s] + j (page
// "Megatron-LM pull request 8539", item 1).
//
// One workgroup (256 threads) per row; the row's visible scores sit in registers as
// order-preserving uint32 keys.  The k-th largest key is found by radix selection on
// (key - row_min_key), starting at the highest set bit of (max - min) so the first
// 8-bit digit already spreads the values over the histogram (the raw top byte of
// same-sign floats of similar magnitude would put them all in one or two bins).
// Ties at the threshold are resolved by index order with a block prefix count, and
// the selected ids are compacted in ascending order.
#include "common.h"
#include "../launch.h"

namespace csa {

constexpr int TK_THREADS = 256;
constexpr int TK_WAVES = TK_THREADS / 64;

__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// exclusive prefix count of `flag` over the block in thread order; returns the rank
// and writes the block total.  Uses two LDS slots per wave and two barriers.
__device__ __forceinline__ int block_rank(bool flag, int *wsum, int &total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  const int in_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
  if (lane == 0) wsum[w] = __popcll(m);
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < TK_WAVES; ++i) {
    const int c = wsum[i];
    before += i < w ? c : 0;
    total += c;
  }
  __syncthreads();
  return before + in_wave;
}

template <int VPT>
__global__ __launch_bounds__(TK_THREADS) void topk_kernel(LayoutDev L, const float *__restrict__ scores,
                                                          int64_t ld, int k_eff, int32_t *__restrict__ ids) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t red[2 * TK_WAVES];
  __shared__ int wsum[TK_WAVES];
  __shared__ uint32_t sel_digit, sel_above;

  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const RowGeo g = row_geo(L, t);
  const int n = g.n_valid;
  int32_t *out = ids + (int64_t)t * k_eff;
  if (n <= k_eff) {  // every visible key is selected
    for (int j = tid; j < k_eff; j += TK_THREADS) out[j] = j < n ? g.k_base + j : -1;
    return;
  }
  const float *row = scores + (int64_t)t * ld;

  uint32_t key[VPT];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int j = v * TK_THREADS + tid;
    key[v] = j < n ? ordered_key(row[j]) : 0u;
    if (j < n) { kmin = min(kmin, key[v]); kmax = max(kmax, key[v]); }
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
  while (cur > 0) {
    const int width = cur < 8 ? cur : 8;
    const int sh = cur - width;
    hist[tid] = 0;  // TK_THREADS == 256 bins
    __syncthreads();
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      const int j = v * TK_THREADS + tid;
      const bool in_play = j < n && (cur >= 32 || (key[v] >> cur) == thr);
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
      }
    }
    __syncthreads();
    thr = (thr << width) | sel_digit;
    need -= (int)sel_above;
    cur = sh;
    __syncthreads();
  }

  // compaction in index order: key > thr, or key == thr among the first `need` ties
  int base = 0, tie_base = 0;
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    if (v * TK_THREADS >= n) break;  // block-uniform
    const int j = v * TK_THREADS + tid;
    const bool valid = j < n;
    const bool gt = valid && key[v] > thr;
    const bool eq = valid && key[v] == thr;
    int eq_total;
    const int eq_rank = block_rank(eq, wsum, eq_total);
    const bool sel = gt || (eq && tie_base + eq_rank < need);
    int sel_total;
    const int pos = block_rank(sel, wsum, sel_total);
    if (sel && base + pos < k_eff) out[base + pos] = g.k_base + j;
    base += sel_total;
    tie_base += eq_total;
  }
}

// One wave per row (rows up to 64*VPL visible keys): the same selection as above with
// wave-level primitives only, so there is no workgroup barrier.  The row's loads are
// issued before its geometry is known (every column below max_seqlen_k exists); row
// min/max and the prefix count over the 256 histogram bins use DPP within 16-lane rows
// plus four readlanes; the selection stops after the first pass whose threshold bin is
// taken whole (count in the bin == keys still needed), which is the usual case once a
// pass has narrowed the bin to a single key.
template <int CTRL> __device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, true);
}
__device__ __forceinline__ uint32_t group16_min_u(uint32_t v) {
  v = min(v, dpp_u<0xB1>(v));
  v = min(v, dpp_u<0x4E>(v));
  v = min(v, dpp_u<0x141>(v));
  return min(v, dpp_u<0x140>(v));
}
__device__ __forceinline__ uint32_t group16_max_u(uint32_t v) {
  v = max(v, dpp_u<0xB1>(v));
  v = max(v, dpp_u<0x4E>(v));
  v = max(v, dpp_u<0x141>(v));
  return max(v, dpp_u<0x140>(v));
}
__device__ __forceinline__ uint32_t rl(uint32_t v, int l) { return (uint32_t)__builtin_amdgcn_readlane((int)v, l); }

template <int VPL>
__global__ __launch_bounds__(256) void topk_wave_kernel(LayoutDev L, int T, const float *__restrict__ scores,
                                                        int64_t ld, int max_sk, int k_eff,
                                                        int32_t *__restrict__ ids) {
  __shared__ __attribute__((aligned(16))) uint32_t hist_all[4][256];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;
  if (t >= T) return;
  uint32_t *hist = hist_all[w];
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
  if (n <= k_eff) {  // every visible key is selected
    for (int j = lane; j < k_eff; j += 64) out[j] = j < n ? g.k_base + j : -1;
    return;
  }
  uint32_t key[VPL];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int j = v * 64 + lane;
    key[v] = j < n ? ordered_key(val[v]) : 0u;
    kmin = j < n ? min(kmin, key[v]) : kmin;
    kmax = j < n ? max(kmax, key[v]) : kmax;
  }
  kmin = group16_min_u(kmin);
  kmax = group16_max_u(kmax);
  // the four row results combine in scalar registers: uniform from here on
  kmin = min(min(rl(kmin, 0), rl(kmin, 16)), min(rl(kmin, 32), rl(kmin, 48)));
  kmax = max(max(rl(kmax, 0), rl(kmax, 16)), max(rl(kmax, 32), rl(kmax, 48)));
#pragma unroll
  for (int v = 0; v < VPL; ++v) key[v] -= kmin;   // relative keys (garbage where j >= n)
  const uint32_t range = kmax - kmin;
  uint32_t thr = 0;
  int need = k_eff;
  int cur = range ? 32 - __builtin_clz(range) : 0;
  bool whole = false;   // the last threshold bin was taken whole
  while (cur > 0) {
    const int width = cur < 8 ? cur : 8;
    const int sh = cur - width;
    reinterpret_cast<u32x4 *>(hist)[lane] = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int j = v * 64 + lane;
      const bool in_play = j < n && (cur >= 32 || (key[v] >> cur) == thr);
      if (in_play) atomicAdd(&hist[(key[v] >> sh) & ((1u << width) - 1u)], 1u);
    }
    const u32x4 cb = reinterpret_cast<const u32x4 *>(hist)[lane];
    const uint32_t mine = cb[0] + cb[1] + cb[2] + cb[3];
    // inclusive prefix over lanes: DPP shifts within each 16-lane row, then row totals
    uint32_t pre = mine;
    pre += dpp_u<0x111>(pre);
    pre += dpp_u<0x112>(pre);
    pre += dpp_u<0x114>(pre);
    pre += dpp_u<0x118>(pre);
    const uint32_t r0 = rl(pre, 15), r1 = rl(pre, 31), r2 = rl(pre, 47), r3 = rl(pre, 63);
    const int rw = lane >> 4;
    pre += (rw >= 1 ? r0 : 0u) + (rw >= 2 ? r1 : 0u) + (rw >= 3 ? r2 : 0u);
    const uint32_t suf = (r0 + r1 + r2 + r3) - pre + mine;  // keys in bins >= 4*lane
    uint32_t above = suf - mine;                            // keys in bins >= 4*lane + 4
    const bool here = above < (uint32_t)need && suf >= (uint32_t)need;
    uint32_t d = 0;
    if (above + cb[3] >= (uint32_t)need) d = 3;
    else if ((above += cb[3]) + cb[2] >= (uint32_t)need) d = 2;
    else if ((above += cb[2]) + cb[1] >= (uint32_t)need) d = 1;
    else { above += cb[1]; d = 0; }
    const uint32_t cnt_d = d == 3 ? cb[3] : d == 2 ? cb[2] : d == 1 ? cb[1] : cb[0];
    const int src = __builtin_amdgcn_readfirstlane(__builtin_ctzll(__ballot(here)));
    const uint32_t digit = rl(4 * lane + d, src);
    const uint32_t ab = rl(above, src);
    const uint32_t cnt = rl(cnt_d, src);
    thr = (thr << width) | digit;
    need -= (int)ab;
    cur = sh;
    if ((uint32_t)need == cnt) { whole = true; break; }
  }
  // compaction in index order: the prefix (bits >= cur) above thr, or equal to thr --
  // all of them when the bin was taken whole, else the first `need` ties (cur == 0)
  int base = 0, tie_base = 0;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    if (v * 64 >= n) break;
    const int j = v * 64 + lane;
    const bool valid = j < n;
    const uint32_t kp = key[v] >> cur;
    const bool gt = valid && (kp > thr || (whole && kp == thr));
    const bool eq = valid && !whole && kp == thr;
    const uint64_t be = __ballot(eq);
    const int eq_rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(be >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)be, 0));
    const bool sel = gt || (eq && tie_base + eq_rank < need);
    const uint64_t bs = __ballot(sel);
    const int pos = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bs >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bs, 0));
    if (sel && pos < k_eff) out[pos] = g.k_base + j;
    base += __popcll(bs);
    tie_base += __popcll(be);
  }
}

bool topk_supported(int max_seqlen_k, int k_eff) { return max_seqlen_k <= 16384 && k_eff >= 0; }

hipError_t launch_topk(const LaunchLayout &LL, const float *scores, int64_t ld, int k_eff,
                       int32_t *ids, hipStream_t st) {
  if (LL.total_q == 0 || k_eff == 0) return hipSuccess;
  if (LL.max_seqlen_k <= 64 * 64) {  // one wave per row
    const int vpl = (LL.max_seqlen_k + 63) / 64;
    const dim3 wgrid((unsigned)((LL.total_q + 3) / 4));
#define CSA_TOPKW_CASE(V)                                                                            \
    if (vpl <= V) {                                                                                  \
      hipLaunchKernelGGL(topk_wave_kernel<V>, wgrid, dim3(256), 0, st, LL.dev, LL.total_q, scores, ld, \
                         LL.max_seqlen_k, k_eff, ids);                                               \
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
    hipLaunchKernelGGL(topk_kernel<V>, grid, block, 0, st, LL.dev, scores, ld, k_eff, ids);     \
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
