// One-pass attention kernels, f32 caches in the rows layout: one or four waves per workgroup.
#include "pad_attn.hpp"

namespace pad {

hipError_t launch_attn_f32_rows_one_pass(const AttnParams& a, int d, int gh, int waves, dim3 grid,
                                             hipStream_t stream) {
  AttnKernelFn fn = waves == 1 ? select_attn<F32, false, 1, kLayoutRows>(d, gh) : select_attn<F32, false, 4, kLayoutRows>(d, gh);
  return launch_kernel(fn, grid, dim3(waves * kWave), a, stream);
}

}  // namespace pad
