// Phase-1 (split) attention kernels for f32 caches: one wave per workgroup.
#include "pad_attn.hpp"

namespace pad {

hipError_t launch_attn_f32_split(const AttnParams& a, int d, int gh, dim3 grid, hipStream_t stream) {
  AttnKernelFn fn = select_attn<F32, true, 1>(d, gh);
  return launch_kernel(fn, grid, dim3(kWave), a, stream);
}

}  // namespace pad
