// Greedy verification and next-draft selection on gfx950.
//
// Candidates are confirmed strictly left to right; the drafts prepared for
// the confirmed outcome become the next candidates ("TiDAR : l'hybride de
// NVIDIA qui rédige par diffusion et parle de manière autorégressive",
// nodesdaily.com, paragraph on drafting for every outcome).
//
// The work is a streaming argmax over fp32 logit rows (HBM-bound):
//   argmax_partial_kernel<false>  (chunk, AR row): 16 B loads, per-thread
//       (value, index) with strict '>' (indices ascend inside a thread, so
//       the lowest index wins ties), a register-only wave reduction, then
//       LDS across waves.
//   verify_select_kernel   one workgroup per sequence, one wave per AR row:
//       each wave reduces its row's chunk results, then the first mismatch
//       is taken by a ballot: accept length, bonus token, draft group.
//   argmax_partial_kernel<true>   the selected group's draft rows 1..k-1.
//   draft_finalize_kernel  one workgroup per sequence, one wave per draft
//       row: the next drafts.
// Ties compare as (value, lower index); -0.0 == +0.0 by IEEE compare.
#include <algorithm>
#include <climits>

#include "common.h"
#include "launch.h"

namespace tidar {

namespace {

template <bool DRAFT>
__global__ __launch_bounds__(256) void argmax_partial_kernel(VerifyArgs a) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int chunk = blockIdx.x;
  const int row = blockIdx.y;
  const float* src;
  float2* dst;
  if (!DRAFT) {
    src = a.ar_logits + (size_t)row * a.V;
    dst = a.part_ar + (size_t)row * a.n_chunks + chunk;
  } else {
    const int b = row / (a.k - 1);
    const int mm = 1 + row % (a.k - 1);
    const int g = min(max(a.group[b], 0), a.k - 1);  // written by verify_select_kernel; clamped regardless
    src = a.draft_logits + (((size_t)b * a.k + g) * a.k + mm) * a.V;
    dst = a.part_draft + (size_t)row * a.n_chunks + chunk;
  }
  const int lo = chunk * a.chunk_elems;
  const int hi = min(a.V, lo + a.chunk_elems);
  float bv = -INFINITY;
  int bi = INT_MAX;
  auto take = [&](float x, int i) {
    if (x > bv) {
      bv = x;
      bi = i;
    }
  };
  if (a.chunk_elems == kArgmaxChunk) {
    // every load of the thread first (their latencies overlap; nontemporal:
    // each logit is read once), then the compares in ascending index order
    // (strict '>' keeps the lowest index)
    if ((a.V & 3) == 0) {
      floatx4 x[kArgmaxChunk / 1024];
#pragma unroll
      for (int j = 0; j < kArgmaxChunk / 1024; ++j) {
        const int i = lo + 4 * (int)threadIdx.x + 1024 * j;
        x[j] = i < hi ? __builtin_nontemporal_load((const floatx4*)(src + i))
                      : (floatx4){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
#pragma unroll
      for (int j = 0; j < kArgmaxChunk / 1024; ++j) {
        const int i = lo + 4 * (int)threadIdx.x + 1024 * j;
        take(x[j].x, i);
        take(x[j].y, i + 1);
        take(x[j].z, i + 2);
        take(x[j].w, i + 3);
      }
    } else {
      float x[kArgmaxChunk / 256];
#pragma unroll
      for (int j = 0; j < kArgmaxChunk / 256; ++j) {
        const int i = lo + (int)threadIdx.x + 256 * j;
        x[j] = i < hi ? __builtin_nontemporal_load(src + i) : -INFINITY;
      }
#pragma unroll
      for (int j = 0; j < kArgmaxChunk / 256; ++j) take(x[j], lo + (int)threadIdx.x + 256 * j);
    }
  } else if ((a.V & 3) == 0) {
    for (int i = lo + 4 * (int)threadIdx.x; i < hi; i += 4 * 256) {
      const float4 x = *(const float4*)(src + i);
      if (x.x > bv) { bv = x.x; bi = i; }
      if (x.y > bv) { bv = x.y; bi = i + 1; }
      if (x.z > bv) { bv = x.z; bi = i + 2; }
      if (x.w > bv) { bv = x.w; bi = i + 3; }
    }
  } else {
    for (int i = lo + (int)threadIdx.x; i < hi; i += 256) {
      const float x = src[i];
      if (x > bv) { bv = x; bi = i; }
    }
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
    *dst = make_float2(bv, __int_as_float(bi));
  }
}

// One wave per row: the wave reduces that row's chunk results (one round
// of loads, one shuffle tree); the rows of a sequence run in parallel and
// meet in LDS.  A workgroup has at most kMaxWaves waves; with more rows a
// wave takes rows w, w + kMaxWaves, ...
constexpr int kMaxRows = 17;   // k + 1 for the largest k
constexpr int kMaxWaves = 16;  // 1024 threads

__device__ __forceinline__ int reduce_row(const float2* part, int n_chunks) {
  const int lane = threadIdx.x & 63;
  float bv = -INFINITY;
  int bi = INT_MAX;
  for (int c = lane; c < n_chunks; c += 64) {
    const float2 p = part[c];
    const int pi = __float_as_int(p.y);
    if (argmax_better(p.x, pi, bv, bi)) {
      bv = p.x;
      bi = pi;
    }
  }
  argmax_wave(bv, bi);
  return bi;
}

// block: min(k+1, kMaxWaves) waves over the k+1 AR rows of sequence blockIdx.x
__global__ __launch_bounds__(64 * kMaxWaves) void verify_select_kernel(VerifyArgs a) {
  __shared__ int t_row[kMaxRows];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  // the candidates, requested before the row reductions so the two round
  // trips overlap
  const int cand = wave == 0 && lane < a.k ? a.cand[(size_t)b * a.k + lane] : 0;
  for (int row = wave; row <= a.k; row += nw) {
    const int t = reduce_row(a.part_ar + ((size_t)b * (a.k + 1) + row) * a.n_chunks, a.n_chunks);
    if (lane == 0) t_row[row] = t;
  }
  __syncthreads();
  const int row = wave;
  if (row == 0) {
    // the accepted length is the first i < k with cand[i] != t_i (k if none)
    const bool miss = lane < a.k && cand != t_row[lane];
    const unsigned long long mm = __ballot(miss || lane == a.k);
    const int acc = __ffsll((long long)mm) - 1;
    if (lane == 0) {
      a.accept_len[b] = acc;
      a.next_cand[(size_t)b * a.k] = t_row[acc];
      a.group[b] = (acc > 0 ? acc : 1) - 1;
    }
  }
}

// block: min(k-1, kMaxWaves) waves over the k-1 draft rows of sequence blockIdx.x
__global__ __launch_bounds__(64 * kMaxWaves) void draft_finalize_kernel(VerifyArgs a) {
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int row = wave; row < a.k - 1; row += nw) {
    const int t = reduce_row(a.part_draft + ((size_t)b * (a.k - 1) + row) * a.n_chunks, a.n_chunks);
    if ((threadIdx.x & 63) == 0) a.next_cand[(size_t)b * a.k + 1 + row] = t;
  }
}

}  // namespace

// The selection and the draft finalisation on their own, for producers of
// the chunk results other than argmax_partial_kernel (the fused LM head).
hipError_t launch_verify_select(const VerifyArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  if (a.k + 1 > kMaxRows) return hipErrorInvalidValue;
  hipLaunchKernelGGL(verify_select_kernel, dim3(a.B), dim3(64 * std::min(a.k + 1, kMaxWaves)), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_draft_finalize(const VerifyArgs& a, hipStream_t s) {
  if (a.B == 0 || a.k == 1) return hipSuccess;
  hipLaunchKernelGGL(draft_finalize_kernel, dim3(a.B), dim3(64 * std::min(a.k - 1, kMaxWaves)), 0, s, a);
  return hipGetLastError();
}

// Each launch is checked before the next: the draft kernels index rows by
// the group the selection writes.
hipError_t launch_verify(const VerifyArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  if (a.k + 1 > kMaxRows) return hipErrorInvalidValue;
  hipLaunchKernelGGL(argmax_partial_kernel<false>, dim3(a.n_chunks, a.B * (a.k + 1)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(verify_select_kernel, dim3(a.B), dim3(64 * std::min(a.k + 1, kMaxWaves)), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.k == 1) return e;
  hipLaunchKernelGGL(argmax_partial_kernel<true>, dim3(a.n_chunks, a.B * (a.k - 1)), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(draft_finalize_kernel, dim3(a.B), dim3(64 * std::min(a.k - 1, kMaxWaves)), 0, s, a);
  return hipGetLastError();
}

}  // namespace tidar
