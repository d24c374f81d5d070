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

#include "argmax_block.h"
#include "check.h"
#include "common.h"
#include "launch.h"

namespace tidar {

namespace {

template <bool DRAFT>
__global__ __launch_bounds__(256) void argmax_partial_kernel(VerifyArgs a) {
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
    // written by verify_select_kernel; clamped so that no read leaves the
    // draft logits (draft_finalize_kernel surfaces an out-of-range group)
    const int g_read = a.group[b];
    if (threadIdx.x == 0 && chunk == 0) (void)TIDAR_CHECK(g_read >= 0 && g_read < a.k, TIDAR_CHECK_GROUP, g_read);
    const int g = min(max(g_read, 0), a.k - 1);
    src = a.draft_logits + (((size_t)b * a.k + g) * a.k + mm) * a.V;
    dst = a.part_draft + (size_t)row * a.n_chunks + chunk;
  }
  const int lo = chunk * a.chunk_elems;
  const int hi = min(a.V, lo + a.chunk_elems);
  float bv;
  int bi;
  block_chunk_argmax(src, lo, hi, a.V, a.chunk_elems, bv, bi);
  if (threadIdx.x == 0) *dst = make_float2(bv, __int_as_float(bi));
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
      (void)TIDAR_CHECK(acc >= 0 && acc <= a.k, TIDAR_CHECK_ACCEPT, acc);
      (void)TIDAR_CHECK(t_row[acc] >= 0 && t_row[acc] < a.V, TIDAR_CHECK_TOKEN, t_row[acc]);
      a.accept_len[b] = acc;
      a.next_cand[(size_t)b * a.k] = t_row[acc];
      a.group[b] = (acc > 0 ? acc : 1) - 1;
    }
  }
}

// block: min(k-1, kMaxWaves) waves over the k-1 draft rows of sequence blockIdx.x
// A group outside 0..k-1 can only mean that the selection did not run for
// this sequence; its drafts are then written as -1, no token id, rather
// than as the clamped group's argmax.
__global__ __launch_bounds__(64 * kMaxWaves) void draft_finalize_kernel(VerifyArgs a) {
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int g = a.group[b];
  const bool valid = g >= 0 && g < a.k;
  if (threadIdx.x == 0) (void)TIDAR_CHECK(valid, TIDAR_CHECK_GROUP, g);
  for (int row = wave; row < a.k - 1; row += nw) {
    const int t = reduce_row(a.part_draft + ((size_t)b * (a.k - 1) + row) * a.n_chunks, a.n_chunks);
    if ((threadIdx.x & 63) == 0) {
      if (valid) (void)TIDAR_CHECK(t >= 0 && t < a.V, TIDAR_CHECK_TOKEN, t);
      a.next_cand[(size_t)b * a.k + 1 + row] = valid ? t : -1;
    }
  }
}

}  // namespace

int verify_launch_shapes(int B, int k, int V, LaunchShape* out) {
  const int n_chunks = (V + kArgmaxChunk - 1) / kArgmaxChunk;
  out[0] = {n_chunks, B * (k + 1), 256};
  out[1] = {B, 1, 64 * std::min(k + 1, kMaxWaves)};
  if (k == 1) return 2;
  out[2] = {n_chunks, B * (k - 1), 256};
  out[3] = {B, 1, 64 * std::min(k - 1, kMaxWaves)};
  return 4;
}

// The selection and the draft finalisation on their own, for producers of
// the chunk results other than argmax_partial_kernel (the fused LM head).
hipError_t launch_verify_select(const VerifyArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  if (a.k + 1 > kMaxRows) return hipErrorInvalidValue;
  LaunchShape sh[kMaxLaunches];
  verify_launch_shapes(a.B, a.k, a.V, sh);
  hipLaunchKernelGGL(verify_select_kernel, dim3(sh[1].gx, sh[1].gy), dim3(sh[1].block), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_draft_finalize(const VerifyArgs& a, hipStream_t s) {
  if (a.B == 0 || a.k == 1) return hipSuccess;
  LaunchShape sh[kMaxLaunches];
  verify_launch_shapes(a.B, a.k, a.V, sh);
  hipLaunchKernelGGL(draft_finalize_kernel, dim3(sh[3].gx, sh[3].gy), dim3(sh[3].block), 0, s, a);
  return hipGetLastError();
}

// Each launch is checked before the next: the draft kernels index rows by
// the group the selection writes.
hipError_t launch_verify(const VerifyArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  if (a.k + 1 > kMaxRows) return hipErrorInvalidValue;
  LaunchShape sh[kMaxLaunches];
  const int n = verify_launch_shapes(a.B, a.k, a.V, sh);
  hipLaunchKernelGGL(argmax_partial_kernel<false>, dim3(sh[0].gx, sh[0].gy), dim3(sh[0].block), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(verify_select_kernel, dim3(sh[1].gx, sh[1].gy), dim3(sh[1].block), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess || n == 2) return e;
  hipLaunchKernelGGL(argmax_partial_kernel<true>, dim3(sh[2].gx, sh[2].gy), dim3(sh[2].block), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(draft_finalize_kernel, dim3(sh[3].gx, sh[3].gy), dim3(sh[3].block), 0, s, a);
  return hipGetLastError();
}

#if TIDAR_CHECKED
TIDAR_CHECK_RECORD_ACCESSOR(check_record_verify)
#endif

}  // namespace tidar
