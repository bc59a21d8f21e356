// Phase-1 (split) attention kernels, f32 caches in the rows layout: PAD_SPLIT_WAVES waves per workgroup.
#include "pad_attn.hpp"

namespace pad {

hipError_t launch_attn_f32_rows_split(const AttnParams& a, int d, int gh, dim3 grid, hipStream_t stream) {
  return launch_kernel(select_attn<F32, true, PAD_SPLIT_WAVES, kLayoutRows>(d, gh), grid, dim3(PAD_SPLIT_WAVES * kWave), a,
                       stream);
}

}  // namespace pad
