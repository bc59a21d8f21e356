// Cross-lane reductions on CDNA4 (gfx950) shared by the attention kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace pad {

// Reductions over the lanes l, l^16, l^32, l^48 (the four lane groups that
// hold one row), on the vector ALU: v_permlane16_swap / v_permlane32_swap
// given the same values in both registers leave (rows of 16 lanes) the even
// and the odd rows, resp. the low and the high half, in both halves.  Issued
// as inline assembly with both registers as explicit in-out operands (this
// compiler's lowering of the two-result builtin reads the first result twice),
// after the two wait states a vector-ALU write of an operand needs.
__device__ inline void swap16(float v, float& lo_rows, float& hi_rows) {
  lo_rows = v;
  hi_rows = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(lo_rows), "+v"(hi_rows));
}
__device__ inline void swap32(float v, float& lo_half, float& hi_half) {
  lo_half = v;
  hi_half = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo_half), "+v"(hi_half));
}
__device__ inline float group_max(float v) {
  float a, b;
  swap16(v, a, b);
  swap32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ inline float group_sum(float v) {
  float a, b;
  swap16(v, a, b);
  swap32(a + b, a, b);
  return a + b;
}

}  // namespace pad
