// Device-side types and helpers shared by the TiDAR kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tidar {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
// Reductions over the four lanes l, l^16, l^32, l^48 of a wave (the lanes
// that hold one row of an MFMA 16x16 result), with the gfx950 row-swap
// instructions instead of LDS permutes: the 32-lane halves are exchanged,
// then the 16-lane rows within each half.
__device__ __forceinline__ float row4_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// (value, index) argmax across lanes: the larger value wins and equal
// values keep the lower index, so the result is the same in every lane
// whatever the pairing order.  Within a 16-lane row the partners come from
// DPP (quad swaps, half-row mirror, row mirror); across rows from the
// row-swap instructions.
__device__ __forceinline__ bool argmax_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}
__device__ __forceinline__ void argmax_take(float& v, int& i, float ov, int oi) {
  if (argmax_better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float& v, int& i) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xF, 0xF, false);
  argmax_take(v, i, ov, oi);
}
__device__ __forceinline__ void argmax_row16(float& v, int& i) {
  argmax_dpp<0xB1>(v, i);   // quad_perm [1,0,3,2]
  argmax_dpp<0x4E>(v, i);   // quad_perm [2,3,0,1]
  argmax_dpp<0x141>(v, i);  // half-row mirror
  argmax_dpp<0x140>(v, i);  // row mirror
}
__device__ __forceinline__ void argmax_wave(float& v, int& i) {
  argmax_row16(v, i);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const auto b = __builtin_amdgcn_permlane16_swap((unsigned)i, (unsigned)i, false, false);
  v = __uint_as_float(a[0]);
  i = (int)b[0];
  argmax_take(v, i, __uint_as_float(a[1]), (int)b[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const auto d = __builtin_amdgcn_permlane32_swap((unsigned)i, (unsigned)i, false, false);
  v = __uint_as_float(c[0]);
  i = (int)d[0];
  argmax_take(v, i, __uint_as_float(c[1]), (int)d[1]);
}

// Running-max start value: finite, so a chunk that sees no key keeps
// exp2(m_old - m_new) == 1 and contributes exp2(-inf - m) == 0.
constexpr float kNoMax = -1.0e30f;

// Visibility of step row j (0..R-1) from step row r, for k candidates.
// Candidates are scored strictly left to right; the slot group g (the
// outcome "candidates 0..g survive") sees those candidates and its own k
// slots ("TiDAR : l'hybride de NVIDIA qui rédige par diffusion et parle de
// manière autorégressive", nodesdaily.com, paragraph on masking).  Settled
// positions are visible to every row and never reach this test.
__device__ __forceinline__ bool step_visible(int r, int j, int k) {
  if (r < k) return j <= r;
  const int g = (r - k) / k;
  if (j < k) return j <= g;
  return (j - k) / k == g;
}

// The same zones per query row, for tests of many step rows j against one
// row r: step rows [0, cand_last] and [slot_lo, slot_hi) are visible
// (settled positions, j < 0, always are).
struct StepZone {
  int cand_last, slot_lo, slot_hi;
  __device__ __forceinline__ bool sees(int j) const { return (j <= cand_last) | ((j >= slot_lo) & (j < slot_hi)); }
};
__device__ __forceinline__ StepZone step_zone(int r, int k) {
  if (r < k) return {r, 0, 0};
  const int g = (r - k) / k;
  return {g, k + g * k, k + (g + 1) * k};
}

// The duplicated training sequence [x_0 .. x_{N-1} ; m_0 .. m_{N-1}]: each
// example appears once for next-token supervision and once as a fully
// masked block filled in parallel ("TiDAR : l'hybride de NVIDIA ...",
// nodesdaily.com, paragraph on training).  Clean row r sees positions
// 0..r; masked row N + j of block [lo, hi) (lo = j - j % bs) sees the clean
// prefix 0..lo-1 and its own block N+lo .. N+hi-1, as a draft group sees
// the prefix, its accepted candidates and itself.  In the StepZone form
// over absolute positions.
__device__ __forceinline__ StepZone train_zone(int r, int N, int bs) {
  if (r < N) return {r, 0, 0};
  const int lo = (r - N) / bs * bs;
  return {lo - 1, N + lo, N + min(lo + bs, N)};
}

// Block index remap for a 8-XCD part: the hardware hands consecutive
// workgroup ids round-robin to the XCDs, so ids i, i+8, i+16, ... share an
// XCD (and its L2).  The returned logical id makes runs of consecutive
// logical ids land on one XCD.
__device__ __forceinline__ int xcd_logical_block(int bid, int nblk) {
  const int per = nblk >> 3;
  return (bid < (per << 3)) ? ((bid & 7) * per + (bid >> 3)) : bid;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

}  // namespace tidar
