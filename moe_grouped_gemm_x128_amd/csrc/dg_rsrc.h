// dg_rsrc.h -- the range arithmetic of the GEMM kernel's buffer resources,
// callable on the host too (its boundary cases are pinned by a CPU test).
//
// A raw buffer resource covers [base, base + num) bytes; a load at an offset
// past num reads zeros and touches no memory.  The kernel moves a resource
// along a row (to a K block, or to a scale piece's first row) by adding to
// the 48-bit base and cutting the range by the same amount, so the range
// still ends where the original one did.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// The range after moving the base by `bytes`: what is left of num, or empty
// if !on or bytes reaches num (it never wraps below zero).
__host__ __device__ inline uint32_t range_after(uint32_t num, uint32_t bytes, bool on) {
  return on && bytes < num ? num - bytes : 0u;
}

// The range after moving the base by a K offset `koff` inside a row, for a
// resource whose range is empty or spans whole rows longer than any K offset
// (koff < row length <= num): scalar arithmetic with no comparison against
// num.  Empty stays empty (a dead source reads nothing at every K block),
// and a dead block (!live) reads nothing.
__host__ __device__ inline uint32_t range_at_k(uint32_t num, uint32_t koff, bool live) {
  return live && num != 0u ? num - koff : 0u;
}

// The 48-bit base moved by `bytes`: low word, and high 16 bits with the carry.
__host__ __device__ inline void base_moved(uint32_t lo, uint32_t hi, uint32_t bytes, uint32_t* new_lo,
                                           uint32_t* new_hi) {
  const uint64_t b = (((uint64_t)hi << 32) | lo) + bytes;
  *new_lo = (uint32_t)b;
  *new_hi = (uint32_t)(b >> 32) & 0xffffu;
}

}  // namespace dg
