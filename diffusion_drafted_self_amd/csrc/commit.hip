// KV-cache commit / evict on gfx950, in place.
//
// The settled cache is reused and rejected entries are evicted ("TiDAR :
// l'hybride de NVIDIA qui rédige par diffusion et parle de manière
// autorégressive", nodesdaily.com, paragraph on the three zones; "KV Cache"
// section of "TiDAR: Think in Diffusion, Talk in Autoregression",
// mauroscia.it).  One workgroup per sequence appends the a accepted
// candidate rows (step rows 0..a-1) at positions lens..lens+a-1 -- keys as
// 16 B row copies, values transposed into their 64-position value page -- then
// advances lens in place.  Rejected candidates and slot rows are evicted by
// never being written.  The work is a few KB per sequence: latency-bound.
#include "common.h"
#include "launch.h"

namespace tidar {

namespace {

__global__ __launch_bounds__(256) void kv_commit_kernel(CommitArgs a) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int acc = a.accept_len[b];
  const int L = a.lens[b];
  const int flag = (acc < 0 || acc > a.k) ? 2 : ((L < 0 || L + acc > a.S_max) ? 1 : 0);
  if (tid == 0 && a.err_flags) a.err_flags[b] = flag;
  if (flag) return;

  const int esz = a.elem_bytes;
  const int cpr = a.D * esz / 16;  // 16 B chunks per key row
  const char* ks = (const char*)a.k_step;
  char* kc = (char*)a.k_cache;
  const int nk = a.Hkv * acc * cpr;
  for (int id = tid; id < nk; id += 256) {
    const int h = id / (acc * cpr);
    const int rem = id % (acc * cpr);
    const int i = rem / cpr, c = rem % cpr;
    const size_t src = (((size_t)b * a.R + i) * a.Hkv + h) * a.D * esz + 16 * c;
    const size_t dst = (((size_t)b * a.Hkv + h) * a.S_max + L + i) * a.D * esz + 16 * c;
    *(uint4*)(kc + dst) = *(const uint4*)(ks + src);
  }

  const int nv = a.Hkv * a.D * acc;
  for (int id = tid; id < nv; id += 256) {
    const int h = id / (a.D * acc);
    const int rem = id % (a.D * acc);
    const int d = rem / acc, i = rem % acc;
    const size_t src = (((size_t)b * a.R + i) * a.Hkv + h) * a.D + d;
    const int pos = L + i;
    const size_t dst = ((size_t)b * a.Hkv + h) * a.S_max * a.D + (size_t)(pos / 64) * a.D * 64 + d * 64 + pos % 64;
    if (esz == 2) ((uint16_t*)a.v_cache)[dst] = ((const uint16_t*)a.v_step)[src];
    else ((uint32_t*)a.v_cache)[dst] = ((const uint32_t*)a.v_step)[src];
  }
  __syncthreads();  // every thread has read lens[b] before it moves
  if (tid == 0) a.lens[b] = L + acc;
}

}  // namespace

hipError_t launch_commit(const CommitArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_commit_kernel, dim3(a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tidar
