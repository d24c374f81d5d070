// Argmax of one chunk of an fp32 logit row by a 256-thread workgroup, shared
// by the greedy verification kernels (gfx950).  The largest value wins and
// equal values keep the lower index; -0.0 == +0.0 as IEEE compares them.
#pragma once

#include <climits>

#include "common.h"
#include "launch.h"

namespace tidar {

namespace {

// (value, index) of the chunk [lo, hi) of row `src` (V entries); the result
// is valid in thread 0.  With chunk_elems == SPAN every thread issues its
// loads first (SPAN / 256 values; their latencies overlap; nontemporal: each
// logit is read once), then compares in ascending index order (strict '>'
// keeps the lowest index), so the wave and workgroup reductions see each
// thread's first maximum.
template <int SPAN = kArgmaxChunk>
__device__ __forceinline__ void block_chunk_argmax(const float* src, int lo, int hi, int V, int chunk_elems,
                                                   float& out_v, int& out_i) {
  static_assert(SPAN % 1024 == 0, "whole float4 rounds of 256 threads");
  __shared__ float sv[4];
  __shared__ int si[4];
  float bv = -INFINITY;
  int bi = INT_MAX;
  auto take = [&](float x, int i) {
    if (x > bv) {
      bv = x;
      bi = i;
    }
  };
  if (chunk_elems == SPAN) {
    if ((V & 3) == 0) {
      floatx4 x[SPAN / 1024];
#pragma unroll
      for (int j = 0; j < SPAN / 1024; ++j) {
        const int i = lo + 4 * (int)threadIdx.x + 1024 * j;
        x[j] = i < hi ? __builtin_nontemporal_load((const floatx4*)(src + i))
                      : (floatx4){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
#pragma unroll
      for (int j = 0; j < SPAN / 1024; ++j) {
        const int i = lo + 4 * (int)threadIdx.x + 1024 * j;
        take(x[j].x, i);
        take(x[j].y, i + 1);
        take(x[j].z, i + 2);
        take(x[j].w, i + 3);
      }
    } else {
      float x[SPAN / 256];
#pragma unroll
      for (int j = 0; j < SPAN / 256; ++j) {
        const int i = lo + (int)threadIdx.x + 256 * j;
        x[j] = i < hi ? __builtin_nontemporal_load(src + i) : -INFINITY;
      }
#pragma unroll
      for (int j = 0; j < SPAN / 256; ++j) take(x[j], lo + (int)threadIdx.x + 256 * j);
    }
  } else if ((V & 3) == 0) {
    for (int i = lo + 4 * (int)threadIdx.x; i < hi; i += 4 * 256) {
      const float4 x = *(const float4*)(src + i);
      take(x.x, i);
      take(x.y, i + 1);
      take(x.z, i + 2);
      take(x.w, i + 3);
    }
  } else {
    for (int i = lo + (int)threadIdx.x; i < hi; i += 256) take(src[i], i);
  }
  argmax_wave(bv, bi);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (argmax_better(sv[w], si[w], bv, bi)) {
        bv = sv[w];
        bi = si[w];
      }
  }
  out_v = bv;
  out_i = bi;
}

}  // namespace

}  // namespace tidar
