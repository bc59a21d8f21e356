// Phase-1 (split) attention kernels, bf16 caches in the rows layout: PAD_SPLIT_WAVES waves per workgroup.
#include "pad_attn.hpp"

namespace pad {

hipError_t launch_attn_bf16_rows_split(const AttnParams& a, int d, int gh, dim3 grid, hipStream_t stream) {
  return launch_kernel(select_attn<BF16, true, PAD_SPLIT_WAVES, kLayoutRows>(d, gh), grid, dim3(PAD_SPLIT_WAVES * kWave), a,
                       stream);
}

}  // namespace pad
