// Top-k of one row held by one wave: the selection shared by the stand-alone top-k
// kernel and the fused score + top-k kernel.
//
// K = min(k_eff, n) largest of the row's first n values, ties to the lower index, emitted
// in ascending index order (page "[Bug] DSV4 unfused CSA indexer loss uses a
// compressed-only teacher ...": k = min(index_topk, n_compressed) over the causally visible
// keys; the lowest-index tie rule makes the selection a function of the values alone).
//
// Value j = v*64 + lane sits in val[v] of that lane.  The values become order-preserving
// uint32 keys; the k-th largest is found by radix selection on (key - row min), starting at
// the highest set bit of (max - min), so the first 8-bit digit already spreads the values
// over the 256-bin histogram (the raw top byte of same-sign floats of similar magnitude
// would put them all in one or two bins).  Row min/max and the prefix count over the bins
// use DPP within 16-lane rows plus four readlanes; the selection stops after the first
// pass whose threshold bin is taken whole (count in the bin == keys still needed).  Ties
// at the threshold are taken in index order with ballot / mbcnt ranks.
#pragma once

#include "common.h"

namespace csa {

__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

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

// emit(pos, j, v) is called by the lane holding value j = v*64 + lane for every selected
// value, pos = its rank in index order (0 .. K-1).  The caller handles n <= k_eff (every
// value selected) itself; here n > k_eff >= 1.  hist: 256 words of LDS owned by the wave.
template <int VPL, typename Emit>
__device__ __forceinline__ void wave_select(const float (&val)[VPL], int n, int k_eff, uint32_t *hist,
                                            Emit emit) {
  const int lane = threadIdx.x & 63;
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
  if (whole) {   // the usual case: no tie to rank, every prefix >= thr is selected
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      if (v * 64 >= n) break;
      const int j = v * 64 + lane;
      const bool sel = j < n && (key[v] >> cur) >= thr;
      const uint64_t bs = __ballot(sel);
      const int pos = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bs >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bs, 0));
      if (sel && pos < k_eff) emit(pos, j, v);
      base += __popcll(bs);
    }
    return;
  }
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    if (v * 64 >= n) break;
    const int j = v * 64 + lane;
    const bool valid = j < n;
    const uint32_t kp = key[v] >> cur;
    const bool gt = valid && kp > thr;
    const bool eq = valid && kp == thr;   // ties at the threshold (cur == 0 here)
    const uint64_t be = __ballot(eq);
    const int eq_rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(be >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)be, 0));
    const bool sel = gt || (eq && tie_base + eq_rank < need);
    const uint64_t bs = __ballot(sel);
    const int pos = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bs >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bs, 0));
    if (sel && pos < k_eff) emit(pos, j, v);
    base += __popcll(bs);
    tie_base += __popcll(be);
  }
}

}  // namespace csa
