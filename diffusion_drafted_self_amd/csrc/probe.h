// The matrix-core issue probe (a measurement helper, not part of the decode
// step): its launcher, for the C ABI.
#pragma once

#include <hip/hip_runtime.h>

namespace tidar {

constexpr int kMfmaProbeBlocks = 256;  // workgroups of the MFMA issue-rate probe, one per CU
hipError_t launch_mfma_probe(int waves_per_simd, int lds_reads, int iters, unsigned long long* cycles, hipStream_t s);

}  // namespace tidar
