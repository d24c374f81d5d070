// Issue rate of the matrix cores, for the reasoning about what bounds the
// attention loops (a measurement helper, not part of the decode step).
//
// kMfmaProbeBlocks workgroups, one per CU (each holds most of the CU's LDS,
// so no second one fits beside it), of 4 x wps waves: wps waves on each of
// the four SIMDs.  Every wave runs `iters` rounds of eight independent
// v_mfma_f32_16x16x32_bf16 (eight accumulators), with the A operand either
// in registers or read from LDS before each MFMA (16 B per lane, a 1 KB
// conflict-free block per read, requested four MFMAs ahead, the attention
// loops' operand pattern), and records the shader-clock cycles of its
// rounds.  Cycles per MFMA of one wave, times the waves that share a SIMD,
// give the SIMD's issue interval.
#include "common.h"
#include "probe.h"

namespace tidar {

namespace {

constexpr int kProbeAcc = 8;       // independent accumulators per wave
constexpr int kProbeDepth = 4;     // LDS reads in flight ahead of their MFMA
constexpr int kProbeLdsBytes = 96 * 1024;

template <bool LDS>
__global__ __launch_bounds__(512) void mfma_probe_kernel(int iters, unsigned long long* cycles) {
  __shared__ __attribute__((aligned(16))) char lds[kProbeLdsBytes];
  typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;
  typedef __attribute__((address_space(3))) char lds_byte;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // LDS contents: small bf16 values, so the accumulators stay finite
  for (int i = threadIdx.x; i < kProbeLdsBytes / 16; i += blockDim.x) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)(0.001f * (float)((i + e) & 7));
    *(lds_bf16x8_t*)(lds + 16 * i) = v;
  }
  __syncthreads();
  bf16x8 a0, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a0[e] = (bf16)(0.001f * (float)(lane & 3));
    b[e] = (bf16)(0.002f * (float)((lane >> 2) & 3));
  }
  floatx4 acc[kProbeAcc];
#pragma unroll
  for (int k = 0; k < kProbeAcc; ++k) acc[k] = (floatx4){0.f, 0.f, 0.f, 0.f};
  // each wave reads its own 8 KB: read k of a round is 1 KB at k * 1024
  const lds_byte* base = (const lds_byte*)lds + (wave % 12) * 8192 + lane * 16;
  bf16x8 fr[kProbeDepth + 1];
  if (LDS) {
#pragma unroll
    for (int k = 0; k < kProbeDepth; ++k) fr[k] = *(const lds_bf16x8_t*)(base + k * 1024);
  }
  const unsigned long long t0 = __builtin_readcyclecounter();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kProbeAcc; ++k) {
      if (LDS) {
        const int kn = (k + kProbeDepth) % kProbeAcc;
        fr[(k + kProbeDepth) % (kProbeDepth + 1)] = *(const lds_bf16x8_t*)(base + kn * 1024);
        acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[k % (kProbeDepth + 1)], b, acc[k], 0, 0, 0);
      } else {
        acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, acc[k], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the results are used: a sum no input can produce marks the record
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < kProbeAcc; ++k) sum += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  const unsigned long long t1 = __builtin_readcyclecounter();
  if (lane == 0) {
    unsigned long long c = t1 - t0;
    // (reading LDS here also keeps the register form's LDS allocation, so
    // one workgroup per CU holds in both forms)
    if (sum == -1.0f && *(const volatile float*)(lds + 4 * lane) == 2.0f) c |= 1ull << 63;
    cycles[(size_t)blockIdx.x * (blockDim.x >> 6) + wave] = c;
  }
}

}  // namespace

hipError_t launch_mfma_probe(int waves_per_simd, int lds_reads, int iters, unsigned long long* cycles, hipStream_t s) {
  const dim3 grid(kMfmaProbeBlocks), block(256 * waves_per_simd);
  if (lds_reads) hipLaunchKernelGGL(mfma_probe_kernel<true>, grid, block, 0, s, iters, cycles);
  else hipLaunchKernelGGL(mfma_probe_kernel<false>, grid, block, 0, s, iters, cycles);
  return hipGetLastError();
}

}  // namespace tidar
