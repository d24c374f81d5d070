// KV-cache commit / evict on gfx950, in place.
//
// The settled cache is reused and rejected entries are evicted ("TiDAR :
// l'hybride de NVIDIA qui rédige par diffusion et parle de manière
// autorégressive", nodesdaily.com, paragraph on the three zones; "KV Cache"
// section of "TiDAR: Think in Diffusion, Talk in Autoregression",
// mauroscia.it).  One workgroup per sequence appends the a accepted
// candidate rows (step rows 0..a-1) at positions lens..lens+a-1 -- keys into
// their rows, values transposed into their 64-position value page -- then
// advances lens in place.  Rejected candidates and slot rows are evicted by
// never being written.  The work is a few KB per sequence: latency-bound.
//
// Paged caches: position p of sequence b lives in page table[b][p / 64] of
// the pools (keys [n_pages][Hkv][64][D], values [n_pages][Hkv][D][64]), at
// row p % 64.  The caller provides the pages; a page entry outside the pools
// is reported and nothing of that sequence is written.
#include "check.h"
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace tidar {

namespace {

// One workgroup per sequence.  The k candidate rows of keys and values are
// loaded in 16 B pieces before the accept length and settled length are
// known (step rows 0..k-1 always exist), so the kernel waits for memory
// once; then every thread stores its key piece into the cache row and
// scatters its value piece (PER consecutive head-dim elements of one
// position) into PER value-page rows.  The settled length moves after a
// barrier that only orders it behind every thread's read of the old value.
template <typename E, int D, bool PAGED>
__global__ __launch_bounds__(1024) void kv_commit_kernel(CommitArgs a) {
  constexpr int PER = 16 / sizeof(E);  // elements per 16 B piece
  constexpr int PPR = D / PER;         // pieces per row
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  constexpr int kSlots = 2;            // pieces per thread and tensor held at once
  const int b = blockIdx.x;
  const int acc = a.accept_len[b];
  const int L = a.lens[b];
  const int n_piece = a.Hkv * a.k * PPR;  // per tensor: (candidate row, head, piece)
  const size_t row_stride = (size_t)a.Hkv * D;
  const E* ks = (const E*)a.k_step + (size_t)b * a.R * row_stride;
  const E* vs = (const E*)a.v_step + (size_t)b * a.R * row_stride;
  // flags: 2 bad accept length, 1 capacity, 3 a page outside the pools.
  // Paged: the (at most two) pages that positions L .. L+acc-1 fall in.
  int pg0 = 0, pg1 = 0;
  auto check = [&]() {
    int f = (acc < 0 || acc > a.k) ? 2 : ((L < 0 || L + acc > a.S_max) ? 1 : 0);
    if constexpr (PAGED) {
      if (!f && acc > 0) {
        const int32_t* tbl = a.block_table + (size_t)b * a.max_pages;
        pg0 = tbl[L / 64];
        pg1 = tbl[(L + acc - 1) / 64];
        if ((unsigned)pg0 >= (unsigned)a.n_pages || (unsigned)pg1 >= (unsigned)a.n_pages) f = 3;
      }
    }
    return f;
  };

  for (int p0 = threadIdx.x; p0 < n_piece; p0 += kSlots * blockDim.x) {
    u32x4 kp[kSlots], vp[kSlots];
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      const int p = p0 + u * blockDim.x;
      if (p < n_piece) {  // p = (i * Hkv + h) * PPR + c: row i's head h, piece c
        kp[u] = *(const u32x4*)(ks + (size_t)p * PER);
        vp[u] = *(const u32x4*)(vs + (size_t)p * PER);
      }
    }
    if (check()) break;
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      const int p = p0 + u * blockDim.x;
      if (p >= n_piece) continue;
      const int c = p % PPR, ih = p / PPR;
      const int h = ih % a.Hkv, i = ih / a.Hkv;
      if (i >= acc) continue;
      const int pos = L + i;
      E* dk;
      E* dv;
      if constexpr (PAGED) {
        const size_t slot = (size_t)(pos / 64 == L / 64 ? pg0 : pg1) * a.Hkv + h;  // (page, head)
        dk = (E*)a.k_cache + (slot * 64 + pos % 64) * D + c * PER;
        dv = (E*)a.v_cache + slot * D * 64 + pos % 64;
      } else {
        dk = (E*)a.k_cache + (((size_t)b * a.Hkv + h) * a.S_max + pos) * D + c * PER;
        dv = (E*)a.v_cache + ((size_t)b * a.Hkv + h) * a.S_max * D + (size_t)(pos / 64) * D * 64 + pos % 64;
      }
      *(u32x4*)dk = kp[u];
      const E* ve = (const E*)&vp[u];
#pragma unroll
      for (int j = 0; j < PER; ++j) dv[(size_t)(c * PER + j) * 64] = ve[j];
    }
  }
  const int flag = check();
  if (threadIdx.x == 0 && flag)
    (void)TIDAR_CHECK(false,
                      flag == 2 ? TIDAR_CHECK_ACCEPT
                                : (flag == 3 ? TIDAR_CHECK_PAGE : (L < 0 ? TIDAR_CHECK_LENS : TIDAR_CHECK_CAPACITY)),
                      flag == 2 ? acc : L + acc);
  if (threadIdx.x == 0 && a.err_flags) a.err_flags[b] = flag;
  __builtin_amdgcn_s_barrier();  // every thread has read lens[b]
  if (threadIdx.x == 0 && !flag) a.lens[b] = L + acc;
}

template <bool PAGED>
void launch_paged(const CommitArgs& a, hipStream_t s, int threads) {
  if (a.elem_bytes == 2) {
    if (a.D == 128) hipLaunchKernelGGL((kv_commit_kernel<uint16_t, 128, PAGED>), dim3(a.B), dim3(threads), 0, s, a);
    else hipLaunchKernelGGL((kv_commit_kernel<uint16_t, 64, PAGED>), dim3(a.B), dim3(threads), 0, s, a);
  } else {
    if (a.D == 128) hipLaunchKernelGGL((kv_commit_kernel<uint32_t, 128, PAGED>), dim3(a.B), dim3(threads), 0, s, a);
    else hipLaunchKernelGGL((kv_commit_kernel<uint32_t, 64, PAGED>), dim3(a.B), dim3(threads), 0, s, a);
  }
}

void launch_typed(const CommitArgs& a, hipStream_t s, int threads) {
  if (a.block_table) launch_paged<true>(a, s, threads);
  else launch_paged<false>(a, s, threads);
}

}  // namespace

// one workgroup per sequence, one thread per 16 B piece of a candidate row
// (keys and values side by side), at most 1024
int commit_launch_shapes(int B, int Hkv, int D, int k, int elem_bytes, LaunchShape* out) {
  const int pieces = Hkv * k * D * elem_bytes / 16;
  out[0] = {B, 1, std::min(1024, std::max(64, ((pieces + 63) / 64) * 64))};
  return 1;
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  LaunchShape sh[kMaxLaunches];
  commit_launch_shapes(a.B, a.Hkv, a.D, a.k, a.elem_bytes, sh);
  launch_typed(a, s, sh[0].block);  // bf16 elements move as raw 16-bit words
  return hipGetLastError();
}

#if TIDAR_CHECKED
TIDAR_CHECK_RECORD_ACCESSOR(check_record_commit)
#endif

}  // namespace tidar
