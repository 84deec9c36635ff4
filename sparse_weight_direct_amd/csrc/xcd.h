// Device helper shared by the gfx950 kernels (HIP sources only).
#pragma once
#include <hip/hip_runtime.h>

namespace sc {

// Workgroups are handed to the 8 XCDs round-robin; renumber them so that consecutive
// logical ids sit on one XCD and share its L2 (nb = grid size, b = blockIdx.x).
__device__ __forceinline__ int xcd_logical(int b, int nb) {
  const int q = nb >> 3, rmd = nb & 7;
  const int xcd = b & 7, k = b >> 3;
  return xcd < rmd ? xcd * (q + 1) + k : rmd * (q + 1) + (xcd - rmd) * q + k;
}

}  // namespace sc
