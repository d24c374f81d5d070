// Greedy verification, next-draft selection and the KV commit of one TiDAR
// step in two launches (gfx950).
//
// The pass scores the carried candidates strictly left to right; the
// drafts prepared for the confirmed outcome become the next candidates; the
// accepted entries are appended to the settled cache and the rejected ones
// evicted ("TiDAR : l'hybride de NVIDIA qui rédige par diffusion et parle de
// manière autorégressive", nodesdaily.com, paragraphs on the three zones
// and on drafting for every outcome).  Same results as the separate
// verification and commit calls; two launches instead of five:
//
//   ar_key_kernel     (chunk, AR row): the chunk's (max, lower index) folded
//       into one 64-bit key per row by an atomic max; a key orders by value,
//       then by lower index.
//   draft_commit_kernel  (span, draft slot) per sequence: every workgroup
//       reads the k+1 row keys of its sequence and the candidates and takes
//       the accept length itself (72 bytes, the same in all of them),
//       reduces its span (two chunks) of the selected group's draft row
//       into that row's key, and copies its share of the accepted step rows
//       into the cache.  The last of the sequence's workgroups to arrive
//       then writes the accept length, bonus token and next drafts, the new
//       settled length, and clears the sequence's state for the next call.
// Nothing waits on another workgroup.  The keys and arrival counters are
// device-scope atomics, performed at the one coherence point for every XCD;
// a workgroup increments its sequence's counter only after its own key
// update has returned, so the workgroup that sees the count complete reads
// final keys.  No fence is needed for that (a device-scope release and
// acquire per workgroup would write back and invalidate the XCD's L2).
//
// State: [B*(k+1)] AR keys, [B*max(k-1,1)] draft keys and [B] arrival
// counters, one per 128-byte line, zero between calls (each call leaves
// them so; the memory must be zero before its first use).
#include <algorithm>
#include <mutex>

#include "argmax_block.h"
#include "check.h"
#include "common.h"
#include "launch.h"

// State of the allocation-free entry point: one array per GPU, alive until
// the process ends.  Host code never names it except in the address lookup
// below: its host-side symbol is not the device address.
static __device__ __align__(256) unsigned char scratch[tidar::kNoAllocScratchBytes];

namespace tidar {

namespace {

typedef unsigned long long u64;

// Each row key sits in its own 128-byte line: the atomics of one row's
// chunks then never queue behind another row's at the coherence point.
constexpr int kKeyStride = kFusedKeyBytes / 8;
constexpr int kArriveStride = kFusedKeyBytes / 4;

// Orders (value, index) as the greedy rule does: larger value first, then
// lower index; -0.0 is folded onto +0.0 so the two tie.  Never 0 for a
// finite value, so 0 is below every key.
__device__ __forceinline__ u64 argmax_key(float v, int i) {
  unsigned u = __float_as_uint(v + 0.0f);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((u64)u << 32) | (u64)(0xFFFFFFFFu - (unsigned)i);
}
__device__ __forceinline__ int key_index(u64 key) { return (int)(0xFFFFFFFFu - (unsigned)key); }

__device__ __forceinline__ u64 load_key(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_zero(u64* p) {
  __hip_atomic_store(p, (u64)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until every memory operation this wave has issued has completed
// (atomics with a result: the result has returned from the coherence point),
// and keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void wait_memory() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }

__global__ __launch_bounds__(256) void ar_key_kernel(FusedVerifyArgs a) {
  const int chunk = blockIdx.x;
  const int row = blockIdx.y;  // b * (k+1) + i
  const int lo = chunk * kArgmaxChunk;
  const int hi = min(a.V, lo + kArgmaxChunk);
  float bv;
  int bi;
  block_chunk_argmax(a.ar_logits + (size_t)row * a.V, lo, hi, a.V, kArgmaxChunk, bv, bi);
  if (threadIdx.x == 0)
    __hip_atomic_fetch_max(&a.key[(size_t)row * kKeyStride], argmax_key(bv, bi), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Copy of accepted step row i, KV head h, into the cache at position pos:
// keys into their row, values into column pos % 64 of their transposed page.
// PER elements per 16 B piece; threads [0, PPR) move key pieces, [PPR,
// 2*PPR) value pieces.
template <typename E, int D, bool PAGED>
__device__ __forceinline__ void commit_row(const FusedVerifyArgs& a, int b, int i, int h, int pos, int page) {
  constexpr int PER = 16 / sizeof(E);
  constexpr int PPR = D / PER;
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const int t = threadIdx.x;
  if (t >= 2 * PPR) return;
  const bool is_v = t >= PPR;
  const int c = is_v ? t - PPR : t;
  if (!TIDAR_CHECK(i >= 0 && i < a.R, TIDAR_CHECK_ROW, i)) return;
  if (!TIDAR_CHECK(pos >= 0 && pos < (PAGED ? a.max_pages * 64 : a.S_max), TIDAR_CHECK_CAPACITY, pos)) return;
  if (PAGED && !TIDAR_CHECK((unsigned)page < (unsigned)a.n_pages, TIDAR_CHECK_PAGE, page)) return;
  const size_t src = (((size_t)b * a.R + i) * a.Hkv + h) * D + (size_t)c * PER;
  const u32x4 piece = *(const u32x4*)((const E*)(is_v ? a.v_step : a.k_step) + src);
  if (!is_v) {
    E* dk = PAGED ? (E*)a.k_cache + (((size_t)page * a.Hkv + h) * 64 + pos % 64) * D + c * PER
                  : (E*)a.k_cache + (((size_t)b * a.Hkv + h) * a.S_max + pos) * D + c * PER;
    *(u32x4*)dk = piece;
  } else {
    E* dv = PAGED ? (E*)a.v_cache + ((size_t)page * a.Hkv + h) * D * 64 + pos % 64
                  : (E*)a.v_cache + ((size_t)b * a.Hkv + h) * a.S_max * D + (size_t)(pos / 64) * D * 64 + pos % 64;
    const E* ve = (const E*)&piece;
#pragma unroll
    for (int j = 0; j < PER; ++j) dv[(size_t)(c * PER + j) * 64] = ve[j];
  }
}

// Accept length of sequence b from its AR row keys: the first i < k with
// cand[i] != argmax of AR row i, k if none; and the bonus token, the argmax
// of AR row acc.  One wave; every lane gets both.
__device__ __forceinline__ void accept_from_keys(const FusedVerifyArgs& a, int b, int lane, int& acc, int& bonus) {
  const int k = a.k;
  const u64 key = lane <= k ? load_key(&a.key[((size_t)b * (k + 1) + lane) * kKeyStride]) : 0;
  const int cand = lane < k ? a.cand[(size_t)b * k + lane] : 0;
  const int t = key_index(key);
  const bool miss = (lane < k && cand != t) || lane == k;
  acc = __ffsll((long long)__ballot(miss)) - 1;
  bonus = __shfl(t, acc);
}

// The commit's decision for sequence b: flag 1 (capacity or a negative
// length) or 3 (a page outside the pools) leaves it unwritten; pg0, pg1
// are the (at most two) pages positions L .. L+acc-1 fall in.
template <bool PAGED>
__device__ __forceinline__ int commit_flag(const FusedVerifyArgs& a, int b, int L, int acc, int& pg0, int& pg1) {
  int flag = (L < 0 || L + acc > a.S_max) ? 1 : 0;
  pg0 = pg1 = 0;
  if (PAGED && !flag && acc > 0) {
    const int32_t* tbl = a.block_table + (size_t)b * a.max_pages;
    pg0 = tbl[L / 64];
    pg1 = tbl[(L + acc - 1) / 64];
    if ((unsigned)pg0 >= (unsigned)a.n_pages || (unsigned)pg1 >= (unsigned)a.n_pages) flag = 3;
  }
  return flag;
}

// The results of sequence b once every draft key is final: accept length,
// bonus token and next drafts; the commit flag and the new settled length;
// the sequence's keys and counter cleared.  One wave (lane < 64).
// acc, bonus: what this workgroup derived from the AR keys at its start; L,
// flag: the settled length it read and the commit decision it took.
template <bool PAGED, bool COMMIT>
__device__ __forceinline__ void finalize_sequence(const FusedVerifyArgs& a, int b, int lane, int acc, int bonus, int L,
                                                  int flag) {
  const int k = a.k;
  if (lane < k - 1) {
    u64* dk = &a.dkey[((size_t)b * (k - 1) + lane) * kKeyStride];
    const int t = key_index(load_key(dk));
    (void)TIDAR_CHECK(t >= 0 && t < a.V, TIDAR_CHECK_TOKEN, t);
    a.next_cand[(size_t)b * k + 1 + lane] = t;
    store_zero(dk);
  }
  if (lane == 0) {
    (void)TIDAR_CHECK(acc >= 0 && acc <= k, TIDAR_CHECK_ACCEPT, acc);
    (void)TIDAR_CHECK(bonus >= 0 && bonus < a.V, TIDAR_CHECK_TOKEN, bonus);
    if (COMMIT && flag)
      (void)TIDAR_CHECK(false, flag == 3 ? TIDAR_CHECK_PAGE : (L < 0 ? TIDAR_CHECK_LENS : TIDAR_CHECK_CAPACITY), L + acc);
    a.next_cand[(size_t)b * k] = bonus;
    a.accept_len[b] = acc;
    if (COMMIT) {
      if (a.err_flags) a.err_flags[b] = flag;
      if (!flag) a.lens[b] = L + acc;
    }
    __hip_atomic_store(&a.arrive[(size_t)b * kArriveStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // every workgroup of the sequence read the keys before it arrived
  if (lane <= k) store_zero(&a.key[((size_t)b * (k + 1) + lane) * kKeyStride]);
}

template <typename E, int D, bool PAGED, bool COMMIT>
__global__ __launch_bounds__(256) void draft_commit_kernel(FusedVerifyArgs a) {
  __shared__ int s_acc, s_bonus, s_last;
  const int span = blockIdx.x;
  const int b = blockIdx.y / a.n_draft_rows;
  const int m = blockIdx.y % a.n_draft_rows;  // draft slot m + 1
  const int k = a.k;
  if (threadIdx.x < 64) {
    int acc, bonus;
    accept_from_keys(a, b, threadIdx.x, acc, bonus);
    if (threadIdx.x == 0) {
      s_acc = acc;
      s_bonus = bonus;
    }
  }
  __syncthreads();
  const int acc = s_acc;
  const int g = (acc > 0 ? acc : 1) - 1;

  u64 done = 0;  // thread 0: the draft key's old value, once returned
  if (k > 1) {  // this span of draft row (group g, slot m + 1)
    const float* src = a.draft_logits + (((size_t)b * k + g) * k + m + 1) * a.V;
    const int lo = span * kDraftSpan;
    const int hi = min(a.V, lo + kDraftSpan);
    float bv;
    int bi;
    block_chunk_argmax<kDraftSpan>(src, lo, hi, a.V, kDraftSpan, bv, bi);
    if (threadIdx.x == 0)
      done = __hip_atomic_fetch_max(&a.dkey[((size_t)b * (k - 1) + m) * kKeyStride], argmax_key(bv, bi),
                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  int L = 0, flag = 0;
  if (COMMIT) {
    // every workgroup of the sequence takes the same decision; units
    // (accepted row i, KV head h) are dealt over them
    L = a.lens[b];
    int pg0, pg1;
    flag = commit_flag<PAGED>(a, b, L, acc, pg0, pg1);
    if (!flag) {
      const int n_wg = gridDim.x * a.n_draft_rows;
      for (int u = m * gridDim.x + span; u < acc * a.Hkv; u += n_wg) {
        const int i = u / a.Hkv, h = u % a.Hkv, pos = L + i;
        commit_row<E, D, PAGED>(a, b, i, h, pos, pos / 64 == L / 64 ? pg0 : pg1);
      }
    }
  }

  // arrival: after this workgroup's key update has returned (and its reads
  // of lens and the keys are done), one count on the sequence's counter; the
  // workgroup that completes the count finalises the sequence
  __syncthreads();  // every thread's reads of lens are done
  if (threadIdx.x == 0) {
    asm volatile("" ::"v"((unsigned)done), "v"((unsigned)(done >> 32)));  // the update's result is used
    wait_memory();
    const unsigned n =
        __hip_atomic_fetch_add(&a.arrive[(size_t)b * kArriveStride], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = n + 1 == (unsigned)(gridDim.x * a.n_draft_rows);
    (void)TIDAR_CHECK(n < (unsigned)(gridDim.x * a.n_draft_rows), TIDAR_CHECK_STATE, n);
  }
  __syncthreads();
  if (s_last && threadIdx.x < 64) finalize_sequence<PAGED, COMMIT>(a, b, threadIdx.x, acc, s_bonus, L, flag);
}

template <typename E, int D, bool PAGED>
void launch_draft_typed(const FusedVerifyArgs& a, dim3 grid, hipStream_t s) {
  if (a.commit) hipLaunchKernelGGL((draft_commit_kernel<E, D, PAGED, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((draft_commit_kernel<E, D, PAGED, false>), grid, dim3(256), 0, s, a);
}

}  // namespace

FusedVerifyGeometry fused_verify_geometry(int B, int k, int V) {
  FusedVerifyGeometry g;
  const int n_chunks = (V + kArgmaxChunk - 1) / kArgmaxChunk;
  g.ar_grid_x = n_chunks;
  g.ar_grid_y = B * (k + 1);
  g.draft_rows = std::max(k - 1, 1);
  g.draft_grid_x = k > 1 ? (V + kDraftSpan - 1) / kDraftSpan : 1;
  g.draft_grid_y = B * g.draft_rows;
  g.block = 256;
  return g;
}

int fused_launch_shapes(int B, int k, int V, LaunchShape* out) {
  const FusedVerifyGeometry g = fused_verify_geometry(B, k, V);
  out[0] = {g.ar_grid_x, g.ar_grid_y, g.block};
  out[1] = {g.draft_grid_x, g.draft_grid_y, g.block};  // its last workgroup per sequence finalises with one wave
  return 2;
}

namespace {

__global__ __launch_bounds__(256) void zero_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  void* ptr = nullptr;  // device address of `scratch` on this device
  bool zero = false;    // known to be all zero once the work already enqueued on it has run
};
std::mutex g_scratch_mu;
ScratchSlot g_scratch[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchSlot& sl = g_scratch[dev];
  if (!sl.ptr) {  // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    sl.ptr = p;
  }
  if (!sl.zero) {  // first use on this device, or after a failed launch: clear on the caller's stream
    hipLaunchKernelGGL(zero_kernel, dim3(256), dim3(256), 0, s, static_cast<uint4*>(sl.ptr),
                       kNoAllocScratchBytes / 16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    sl.zero = true;
  }
  *out = sl.ptr;
  return hipSuccess;
}

void noalloc_scratch_dirty() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  g_scratch[dev].zero = false;
}

hipError_t launch_fused_verify(const FusedVerifyArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const FusedVerifyGeometry g = fused_verify_geometry(a.B, a.k, a.V);
  if (g.draft_rows != a.n_draft_rows) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ar_key_kernel, dim3(g.ar_grid_x, g.ar_grid_y), dim3(g.block), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(g.draft_grid_x, g.draft_grid_y);
  const bool paged = a.block_table != nullptr;
  if (a.elem_bytes == 2) {
    if (a.D == 128) paged ? launch_draft_typed<uint16_t, 128, true>(a, grid, s)
                          : launch_draft_typed<uint16_t, 128, false>(a, grid, s);
    else paged ? launch_draft_typed<uint16_t, 64, true>(a, grid, s)
               : launch_draft_typed<uint16_t, 64, false>(a, grid, s);
  } else {
    if (a.D == 128) paged ? launch_draft_typed<uint32_t, 128, true>(a, grid, s)
                          : launch_draft_typed<uint32_t, 128, false>(a, grid, s);
    else paged ? launch_draft_typed<uint32_t, 64, true>(a, grid, s)
               : launch_draft_typed<uint32_t, 64, false>(a, grid, s);
  }
  return hipGetLastError();
}

#if TIDAR_CHECKED
TIDAR_CHECK_RECORD_ACCESSOR(check_record_verify_fused)
#endif

}  // namespace tidar
