// Phase-1 (split) attention kernels for bf16 caches: one wave per workgroup.
#include "pad_attn.hpp"

namespace pad {

hipError_t launch_attn_bf16_split(const AttnParams& a, int d, int gh, dim3 grid, hipStream_t stream) {
  AttnKernelFn fn = select_attn<BF16, true, 1>(d, gh);
  return launch_kernel(fn, grid, dim3(kWave), a, stream);
}

}  // namespace pad
