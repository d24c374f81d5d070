// Device-side bounds tests of the checked build (libtidar_checked.so,
// compiled with TIDAR_CHECKED=1).
//
// Every index a kernel reads from device memory (a settled length, a
// block-table entry, a draft group) and every key tile, query row, output
// row or chunk index it derives before addressing a buffer is tested
// against the bound the call's arguments give it.  A failed test records
// {code, workgroup, thread, value} in the record of the translation unit
// whose kernel failed it (the first failure on a GPU wins; later ones are
// dropped) and the access is redirected to an in-bounds address or
// skipped, so the kernel still runs to its end: no trap, no fault.
// tidar_check_read() returns and clears the records.
//
// In the release build every test is the constant `true`: the conditions
// are not evaluated and the kernels are instruction-for-instruction those
// of an unchecked source.
#pragma once

#include <hip/hip_runtime.h>

#include "tidar.h"

#ifndef TIDAR_CHECKED
#define TIDAR_CHECKED 0
#endif

namespace tidar {

#if TIDAR_CHECKED
// One record per translation unit and GPU: {code, workgroup, thread, value}.
static __device__ __align__(16) unsigned g_check[4];

static __device__ __noinline__ bool check_fail(unsigned code, int value) {
  if (atomicCAS(&g_check[0], 0u, code) == 0u) {
    g_check[1] = blockIdx.x;
    g_check[2] = threadIdx.x;
    g_check[3] = (unsigned)value;
  }
  return false;
}

// Host: copy this translation unit's record of the current device into
// rec[4] and, if `clear`, zero it.  The caller has synchronised the device.
#define TIDAR_CHECK_RECORD_ACCESSOR(NAME)                                       \
  hipError_t NAME(unsigned* rec, bool clear) {                                \
    void* p = nullptr;                                                          \
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_check));                \
    if (e != hipSuccess) return e;                                              \
    e = hipMemcpy(rec, p, 4 * sizeof(unsigned), hipMemcpyDeviceToHost);         \
    if (e != hipSuccess || !clear) return e;                                    \
    const unsigned zero[4] = {0u, 0u, 0u, 0u};                                  \
    return hipMemcpy(p, zero, sizeof(zero), hipMemcpyHostToDevice);             \
  }

// True when `cond` holds; otherwise records (code, value) and is false.
#define TIDAR_CHECK(cond, code, value) \
  (__builtin_expect(!!(cond), 1) ? true : ::tidar::check_fail((unsigned)(code), (int)(value)))
#else
__device__ __forceinline__ constexpr bool check_pass() { return true; }
#define TIDAR_CHECK(cond, code, value) (::tidar::check_pass())
#endif

}  // namespace tidar
