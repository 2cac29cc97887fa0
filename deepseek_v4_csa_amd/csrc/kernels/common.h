// Device helpers shared by the CSA kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
// round-to-nearest-even (lowers to v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// ---------------------------------------------------------------- MFMA wrappers
// 16x16x32 bf16: lane l supplies A[l%16][(l/16)*8 + e] and B[(l/16)*8 + e][l%16],
// e = 0..7; receives C[(l/16)*4 + i][l%16], i = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// The same 16x16x32 bf16 product as asm statements, C and D in VGPRs: vector work placed
// between them (tied to its place by empty asm statements, which keep their order with
// these) runs beside the MFMAs.  The compiler does not pad hazards it does not see, so:
//  * D is read only after mfma_v_fence: 16 wait states (this shape needs 8 before a vector
//    instruction reads its result and 3 before one overwrites a C operand still being read);
//  * C is the constant 0 or exactly D of the chain's previous MFMA (an exactly overlapping
//    accumulation chain needs no wait states);
//  * A and B are results of LDS and global loads, which the compiler waits for (it tracks the
//    registers an asm statement reads); no vector instruction writes them.
// Being volatile, the statements keep their order among themselves and with every memory
// access, so the LDS reads and row requests issue where the source places them.
// tests/test_mfma_hazards_cpu.py checks the compiled kernels against these rules.
__device__ __forceinline__ void mfma_v_first(f32x4 &d, const u32x4 &a, const u32x4 &b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x4 &d, const u32x4 &a, const u32x4 &b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_fence(f32x4 (&d)[2][2]) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(d[0][0]), "+v"(d[0][1]), "+v"(d[1][0]), "+v"(d[1][1]));
}
// 16x16x16 bf16: lane l supplies A[l%16][(l/16)*4 + e] and B[(l/16)*4 + e][l%16],
// e = 0..3 (4 bf16 in two dwords); same C layout.
typedef short v4i16_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16x16x16(uint2 a, uint2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16_t, a),
                                                   __builtin_bit_cast(v4i16_t, b), c, 0, 0, 0);
}
// 16x16x4 fp32: lane l supplies A[l%16][l/16] and B[l/16][l%16]; same C layout.
__device__ __forceinline__ f32x4 mfma16x16x4f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- wave reductions
template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) { return __shfl_xor(v, m, WAVE); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
  return v;
}
// reductions over the 16 lanes of a lane group (lanes with the same l/16), on DPP:
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], quad_perm [3,2,1,0], row_half_mirror,
// row_mirror.  These controls are permutations within a 16-lane row (every lane has a
// source), so the plain DPP move is used: no old value to set up first.
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  static_assert(CTRL == 0xB1 || CTRL == 0x4E || CTRL == 0x1B || CTRL == 0x141 || CTRL == 0x140,
                "a full in-row permutation");
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float group16_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return v;
}
// Eight sums over the 16 lanes of a lane group at once, as a reduce-scatter: at each of
// four exchanges (row_mirror i <-> 15-i, row_half_mirror i <-> 7-i within eight,
// quad_perm i <-> 3-i, quad_perm i <-> i^1) a lane keeps half of its partial sums and adds
// the partner's copies of them, so the eight totals cost 22 vector instructions instead of
// 32 and land spread over the lanes.  Lane r of the group returns the total of value
// sum8_index(r); lanes r and r ^ 1 return the same one.
__device__ __forceinline__ int sum8_index(int r) { return 4 * ((r >> 3) & 1) + 2 * ((r >> 2) & 1) + ((r >> 1) & 1); }
__device__ __forceinline__ float group16_sum8(const float (&v)[8], int r) {
  const bool u1 = (r & 8) != 0, u2 = (r & 4) != 0, u3 = (r & 2) != 0;
  float w[4], x[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = (u1 ? v[4 + k] : v[k]) + dpp<0x140>(u1 ? v[k] : v[4 + k]);
#pragma unroll
  for (int k = 0; k < 2; ++k) x[k] = (u2 ? w[2 + k] : w[k]) + dpp<0x141>(u2 ? w[k] : w[2 + k]);
  const float y = (u3 ? x[1] : x[0]) + dpp<0x1B>(u3 ? x[0] : x[1]);
  return y + dpp<0xB1>(y);
}
// full-wave reductions on DPP (16-lane rows) plus four readlanes; the result is uniform
template <int CTRL> __device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  static_assert(CTRL == 0xB1 || CTRL == 0x4E || CTRL == 0x141 || CTRL == 0x140, "a full in-row permutation");
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xf, 0xf, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double wave_sum_f64_dpp(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
// 2^x on the hardware unit (no denormal range fix-up: results below 2^-126 flush to 0)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// reductions over the 4 lane groups holding the same l%16
__device__ __forceinline__ float across_groups_max(float v) {
  v = fmaxf(v, shfl_xor(v, 16));
  v = fmaxf(v, shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float across_groups_sum(float v) {
  v += shfl_xor(v, 16);
  v += shfl_xor(v, 32);
  return v;
}

// ---------------------------------------------------------------- row geometry
struct LayoutDev {
  const int32_t *cu_q;
  const int32_t *cu_k;
  const int32_t *off;  // may be null: bottom-right default
  const int32_t *cu_q_real;  // may be null: no padding rows
  int32_t num_seqs;
  int32_t ratio;
};

// segment s with cu_q[s] <= t < cu_q[s+1] (binary search; cu_q is non-decreasing,
// empty segments are skipped because the search finds the last s with cu_q[s] <= t)
// A load through the constant address space: the layout arrays are never written while a
// kernel runs, so at a wave-uniform address this is a scalar load (counted by lgkmcnt),
// and waiting for it does not wait for the wave's vector-memory traffic in flight.
__device__ __forceinline__ int32_t ldc(const int32_t *p) {
  return *(const __attribute__((address_space(4))) int32_t *)(p);
}

__device__ __forceinline__ int segment_of(const int32_t *cu_q, int nseq, int t) {
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (ldc(cu_q + mid) <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct RowGeo {
  int seg, q_start, q_len, k_base, s_k, n_valid;
};

__device__ __forceinline__ int n_valid_of(int local, int off, int ratio, int s_k) {
  int i = local + 1 + off;
  int n = i > 0 ? i / ratio : 0;
  return n < s_k ? n : s_k;
}

__device__ __forceinline__ RowGeo row_geo(const LayoutDev &L, int t) {
  RowGeo g;
  g.seg = segment_of(L.cu_q, L.num_seqs, t);
  g.q_start = ldc(L.cu_q + g.seg);
  g.q_len = ldc(L.cu_q + g.seg + 1) - g.q_start;
  g.k_base = ldc(L.cu_k + g.seg);
  g.s_k = ldc(L.cu_k + g.seg + 1) - g.k_base;
  int off = L.off ? ldc(L.off + g.seg) : g.s_k * L.ratio - g.q_len;
  g.n_valid = n_valid_of(t - g.q_start, off, L.ratio, g.s_k);
  return g;
}

// A row adds nothing to the loss when it sees no compressed key or is a padding row (its
// position in the segment at or past the segment's real length).  Padding rows are still
// scored, selected and attended like any row.
__device__ __forceinline__ bool loss_row_empty(const LayoutDev &L, const RowGeo &g, int t) {
  if (g.n_valid == 0) return true;
  if (!L.cu_q_real) return false;
  const int real = ldc(L.cu_q_real + g.seg + 1) - ldc(L.cu_q_real + g.seg);
  return t - g.q_start >= real;
}

__device__ __forceinline__ int seg_offset(const LayoutDev &L, int s, int q_len, int s_k) {
  return L.off ? ldc(L.off + s) : s_k * L.ratio - q_len;
}

}  // namespace csa

namespace csa {
// ---------------------------------------------------------------- LDS transposing read
// ds_read_b64_tr_b16 (gfx950): within each 16-lane group, lane j supplies the address of
// 4 consecutive bf16 X[j][0..3]; lane i receives X[4k + i/4][i%4], k = 0..3.  When lane j
// points at row R + j/4, columns C + 4*(j%4) of a row-major bf16 tile, lane i receives
// column C + i of rows R..R+3 -- a 4x16 transpose, the K-major operand layout of MFMA.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
__device__ __forceinline__ uint2 lds_read_tr16(const char *lds_ptr) {
  lds_v4i16 *p = (lds_v4i16 *)(const_cast<char *>(lds_ptr));
  v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
  return __builtin_bit_cast(uint2, v);
}
__device__ __forceinline__ uint32_t lds_addr_of(const void *lds_ptr) {
  return (uint32_t)(uintptr_t)(const lds_v4i16 *)(lds_ptr);
}
// A batch of N pairs of transposing reads (read 2k at LDS byte address a[k], read 2k + 1 at
// a[k] + OFF2) and the wait for them, in one asm block: the results are complete when the
// block ends, so the compiler may move or reuse their registers freely.  (For the builtin
// read above the compiler first waits for every buffer->LDS load still in flight, the next
// tiles' prefetch included; the asm form is not taken for such an LDS access.)  The wait is
// lgkmcnt(0): LDS operations issued before the block complete with it.
#define CSA_TRP(k)                                                   \
  "ds_read_b64_tr_b16 %[o" #k "a], %[a" #k "]\n\t"                   \
  "ds_read_b64_tr_b16 %[o" #k "b], %[a" #k "] offset:%[off]\n\t"
#define CSA_TRO(k) [o##k##a] "=&v"(v[2 * k]), [o##k##b] "=&v"(v[2 * k + 1])
#define CSA_TRI(k) [a##k] "v"(a[k])
template <int> constexpr bool tr_pairs_unsupported = false;
template <int OFF2, int N>
__device__ __forceinline__ void lds_read_tr16_pairs(uint2 (&v)[2 * N], const uint32_t (&a)[N]) {
  static_assert(OFF2 >= 0 && OFF2 < 65536, "ds offset field");
  if constexpr (N == 2) {
    asm volatile(CSA_TRP(0) CSA_TRP(1) "s_waitcnt lgkmcnt(0)"
                 : CSA_TRO(0), CSA_TRO(1)
                 : CSA_TRI(0), CSA_TRI(1), [off] "i"(OFF2)
                 : "memory");
  } else if constexpr (N == 4) {
    asm volatile(CSA_TRP(0) CSA_TRP(1) CSA_TRP(2) CSA_TRP(3) "s_waitcnt lgkmcnt(0)"
                 : CSA_TRO(0), CSA_TRO(1), CSA_TRO(2), CSA_TRO(3)
                 : CSA_TRI(0), CSA_TRI(1), CSA_TRI(2), CSA_TRI(3), [off] "i"(OFF2)
                 : "memory");
  } else if constexpr (N == 6) {
    asm volatile(CSA_TRP(0) CSA_TRP(1) CSA_TRP(2) CSA_TRP(3) CSA_TRP(4) CSA_TRP(5) "s_waitcnt lgkmcnt(0)"
                 : CSA_TRO(0), CSA_TRO(1), CSA_TRO(2), CSA_TRO(3), CSA_TRO(4), CSA_TRO(5)
                 : CSA_TRI(0), CSA_TRI(1), CSA_TRI(2), CSA_TRI(3), CSA_TRI(4), CSA_TRI(5), [off] "i"(OFF2)
                 : "memory");
  } else if constexpr (N == 8) {
    asm volatile(CSA_TRP(0) CSA_TRP(1) CSA_TRP(2) CSA_TRP(3) CSA_TRP(4) CSA_TRP(5) CSA_TRP(6) CSA_TRP(7)
                 "s_waitcnt lgkmcnt(0)"
                 : CSA_TRO(0), CSA_TRO(1), CSA_TRO(2), CSA_TRO(3), CSA_TRO(4), CSA_TRO(5), CSA_TRO(6), CSA_TRO(7)
                 : CSA_TRI(0), CSA_TRI(1), CSA_TRI(2), CSA_TRI(3), CSA_TRI(4), CSA_TRI(5), CSA_TRI(6), CSA_TRI(7),
                   [off] "i"(OFF2)
                 : "memory");
  } else {
    static_assert(tr_pairs_unsupported<N>, "pairs per batch: 2, 4, 6 or 8");
  }
}
#undef CSA_TRP
#undef CSA_TRO
#undef CSA_TRI
}  // namespace csa

namespace csa {
// ---------------------------------------------------------------- buffer loads
// A raw buffer resource over [base, base + bytes): loads at byte offsets >= bytes return
// zeros instead of touching memory (the hardware range check of gfx9 raw buffers).
constexpr uint32_t BUF_OOB = 0x7fffffffu;  // an offset past every resource used here
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
// lane shuffle through the LDS crossbar with a precomputed byte address (lane * 4)
__device__ __forceinline__ float bperm(int addr, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(addr, __builtin_bit_cast(int, v)));
}
}  // namespace csa

namespace csa {
// Row tiles of D bf16 (D*2 bytes per row) staged in LDS: 16-byte piece p of tile row R is
// stored at piece position p ^ row_swz<D>(R).  The LDS of gfx950 (measured with the bank
// conflict counter on access patterns of their own): 16-byte reads are served a quarter
// wave per cycle, the quarter being half-wave h = lane >> 5 and parity
// bit2 ^ bit3 ^ bit4 of the lane index (lanes 0-3, 12-15, 20-23, 24-27 together); two of
// its lanes conflict when they hit the same 16-byte slot (address bits 7:4) at different
// addresses.  8-byte transposing reads are served a half wave (32 consecutive lanes) per
// cycle over the 32 8-byte words of a 256-byte line.  The swizzle is linear in the bits of
// R and keeps conflict-free, for every MFMA K-chunk and d-tile: the row-operand reads
// (lane (g, r) reads piece 4c + g of row r), the transposing reads (lane (g, r) reads
// pieces 2dt, 2dt + 1 of row 4g + r / 4) and the row-staging writes (whole rows).  Rows
// of 256*k bytes (D = 128, 256, 512) take 16 values; rows of 128 or 384 bytes (D = 64,
// 192), which start half a line apart, take 8 values (p ^ swz then stays inside the row's
// 8-piece group).  The pattern repeats every 16 rows.
template <int D> __host__ __device__ constexpr int row_swz(int r) {
  static_assert(D == 64 || D == 128 || D == 192 || D == 256 || D == 512, "row size");
  if constexpr (D == 64 || D == 192) return (2 * ((r >> 1) & 3)) ^ (5 * ((r >> 3) & 1));
  else return (2 * (r & 7)) ^ (9 * ((r >> 3) & 1));
}
// A load instruction of 64 lanes x 16 bytes covers RPI = 64 / (D / 8) whole rows when D
// divides 512; then the swizzle of row i RPI + g (g < RPI) splits into a per-lane and a
// per-instruction term.
template <int D> constexpr bool swz_splits() {
  constexpr int RPI = 512 / D;
  for (int i = 0; i * RPI < 32; ++i)
    for (int g = 0; g < RPI; ++g)
      if (row_swz<D>(i * RPI + g) != (row_swz<D>(g) ^ row_swz<D>(i * RPI))) return false;
  return true;
}

// ---------------------------------------------------------------- LDS DMA
// buffer_load_dwordx4 ... lds (gfx950): lane i's 16 bytes from rsrc+voffset land at
// lds_base + 16*i; an out-of-range offset reads zeros.  Completion is tracked by vmcnt,
// which the kernels wait on explicitly before reading the tile.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void *lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds_base, 16, (int)voff, 0, 0, 0);
}
// the 4-byte form: lane l writes lds_base + 4 l
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void *lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds_base, 4, (int)voff, 0, 0, 0);
}
// s_waitcnt with only vmcnt constrained (expcnt 7 and lgkmcnt 15 = no wait); the 6-bit
// count is split over bits 3:0 and 15:14 of the immediate
// Workgroup barrier of the LDS-staged pipelines: the wave's own LDS reads and writes are
// waited for (lgkmcnt 0), then s_barrier.  __syncthreads() would also wait for every direct
// buffer->LDS load still in flight (its workgroup-scope release fence counts them as LDS
// writes), which drains the tiles requested ahead at every step; the kernels instead wait
// for each tile's own loads with wait_vmcnt before this barrier.  The memory clobber keeps
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
}  // namespace csa
