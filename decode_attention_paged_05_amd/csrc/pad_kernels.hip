// Phase 2 (log-sum-exp merge), the workspace fill and the launchers for all
// kernels.  The attention kernels themselves live in pad_attn.hpp and are
// instantiated in the pad_attn_*.hip units.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "pad_attn.hpp"
#include "pad_internal.h"

namespace pad {

hipError_t launch_attn_bf16_rows_split(const AttnParams& a, int d, int gh, dim3 grid, hipStream_t stream);
hipError_t launch_attn_f32_rows_split(const AttnParams& a, int d, int gh, dim3 grid, hipStream_t stream);
hipError_t launch_attn_bf16_tiled_split(const AttnParams& a, int d, int gh, dim3 grid, hipStream_t stream);
hipError_t launch_attn_f32_tiled_split(const AttnParams& a, int d, int gh, dim3 grid, hipStream_t stream);
hipError_t launch_attn_bf16_rows_one_pass(const AttnParams& a, int d, int gh, int waves, dim3 grid,
                                          hipStream_t stream);
hipError_t launch_attn_f32_rows_one_pass(const AttnParams& a, int d, int gh, int waves, dim3 grid,
                                         hipStream_t stream);
hipError_t launch_attn_bf16_tiled_one_pass(const AttnParams& a, int d, int gh, int waves, dim3 grid,
                                           hipStream_t stream);
hipError_t launch_attn_f32_tiled_one_pass(const AttnParams& a, int d, int gh, int waves, dim3 grid,
                                          hipStream_t stream);

namespace {

// ---------------------------------------------------------------------------
// Phase 2: log-sum-exp merge.  Grid (D/64, H, S), 256 threads; the workgroup
// owns 64 dims of one (sequence, head).  Its partitions are taken 256 at a
// time; for each chunk every load is issued in one round before any
// arithmetic (the merge is latency-bound, not bandwidth-bound):
//   thread t     max_logits and exp_sums of partition t of the chunk;
//   lanes        16 lanes x float4 cover the 64 dims, 16 lane groups take
//                partitions g, g+16, ... of the chunk (16 float4 each).
// Then: chunk max -> running max (earlier chunks rescaled), weights
// w_p = exp_sum_p * exp(max_p - max) through LDS, weighted sums, and a final
// LDS reduction over the 16 lane groups divided by the summed weights.
// Slots past the sequence's partition count are read (they exist) but
// discarded by select, so stale or NaN contents never enter the sums.
// ---------------------------------------------------------------------------
struct MergeParams {
  float* out;
  const int32_t* seq_lens;
  const float* max_logits;
  const float* exp_sums;
  const float* tmp_out;
  int num_heads;
  int head_size;
  int max_tokens;  // W * block_size
  int partition;
  int num_partitions;
};

constexpr int kMergeThreads = 256;
constexpr int kMergeChunk = 256;  // partitions per round
constexpr int kMergeGroups = 16;  // lane groups striding over a chunk
constexpr int kMergePerThread = kMergeChunk / kMergeGroups;

__device__ inline float block_reduce_256(float v, bool is_max, float* scratch) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float o = __shfl_xor(v, off);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  const int wave = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[wave] = v;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / kWave; ++w) r = is_max ? fmaxf(r, scratch[w]) : r + scratch[w];
  return r;
}

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeParams p) {
  __shared__ float scratch[kMergeThreads / kWave];
  __shared__ float w_lds[kMergeChunk];
  __shared__ f32x4_t part_acc[kMergeGroups][16];
  const int tid = threadIdx.x;
  const int s = blockIdx.z;
  const int h = blockIdx.y;
  const int D = p.head_size;
  const int d0 = blockIdx.x * 64;
  const int dl = tid & 15;
  const int pg = tid >> 4;
  const int NP = p.num_partitions;
  const size_t row0 = ((size_t)s * p.num_heads + h) * NP;
  const float* ml = p.max_logits + row0;
  const float* es = p.exp_sums + row0;
  const float* tmp = p.tmp_out + row0 * D + d0 + 4 * dl;
  float* orow = p.out + ((size_t)s * p.num_heads + h) * D + d0;

  f32x4_t a = {0.0f, 0.0f, 0.0f, 0.0f};
  float wsum = 0.0f;
  float mrun = -INFINITY;  // running max, log2 units
  int np = -1;             // partitions of this sequence (known after the first round's loads)
  for (int c0 = 0; c0 < NP; c0 += kMergeChunk) {
    // one round of loads: slots that exist, whatever the sequence length
    const int ti = c0 + tid;
    const float my_ml = ti < NP ? ml[ti] : -INFINITY;
    const float my_es = ti < NP ? es[ti] : 0.0f;
    f32x4_t t[kMergePerThread];
#pragma unroll
    for (int k = 0; k < kMergePerThread; ++k) {
      const int i = c0 + pg + kMergeGroups * k;
      t[k] = i < NP ? *reinterpret_cast<const f32x4_t*>(tmp + (size_t)i * D) : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    if (np < 0) {
      const int L = p.seq_lens[s];
      if (L <= 0 || L > p.max_tokens) {
        if (tid < 64) orow[tid] = (L == 0) ? 0.0f : __builtin_nanf("");
        return;
      }
      np = (L + p.partition - 1) / p.partition;
    }
    if (c0 >= np) break;
    const bool valid = ti < np;
    const float m2 = valid ? my_ml * kLog2e : -INFINITY;
    const float cmax = block_reduce_256(m2, true, scratch);
    const float mnew = fmaxf(mrun, cmax);
    const float resc = fast_exp2(mrun - mnew);  // 0 on the first chunk
    a *= resc;
    wsum *= resc;
    mrun = mnew;
    const float w = valid ? my_es * fast_exp2(m2 - mnew) : 0.0f;
    wsum += w;
    w_lds[tid] = w;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMergePerThread; ++k) {
      const int i = c0 + pg + kMergeGroups * k;
      if (i < np) a += w_lds[pg + kMergeGroups * k] * t[k];
    }
    __syncthreads();  // w_lds is rewritten by the next chunk
  }
  wsum = block_reduce_256(wsum, false, scratch);
  part_acc[pg][dl] = a;
  __syncthreads();
  if (tid < 16) {
    f32x4_t r = part_acc[0][tid];
#pragma unroll
    for (int g = 1; g < kMergeGroups; ++g) r += part_acc[g][tid];
    *reinterpret_cast<f32x4_t*>(orow + 4 * tid) = r * (1.0f / wsum);
  }
}

__global__ __launch_bounds__(256) void fill_kernel(float* ml, float* es, float* tmp, size_t n_stats,
                                                   size_t n_tmp) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_stats; i += stride) {
    ml[i] = -INFINITY;
    es[i] = 0.0f;
  }
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_tmp; i += stride) tmp[i] = 0.0f;
}

// Smallest instantiated accumulator width that holds `heads` heads.
int heads_template(int heads) {
  if (heads <= 1) return 1;
  if (heads <= 2) return 2;
  if (heads <= 4) return 4;
  if (heads <= 6) return 6;
  if (heads <= 8) return 8;
  return 16;
}

// Compute units of the current device, cached per device ordinal.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();  // our own failed query: do not leave it behind
    return 256;
  }
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

AttnParams make_params(const Plan& plan, const void* q, const void* k, const void* v, const int32_t* tables,
                       const int32_t* lens) {
  AttnParams a{};
  a.query = static_cast<const char*>(q);
  a.key_cache = static_cast<const char*>(k);
  a.value_cache = static_cast<const char*>(v);
  a.block_tables = tables;
  a.seq_lens = lens;
  a.num_blocks = plan.num_blocks;
  a.num_heads = plan.num_heads;
  a.num_kv_heads = plan.num_kv_heads;
  a.group = plan.group;
  a.head_chunks = plan.head_chunks;
  a.max_blocks = plan.max_blocks;
  a.partition = plan.partition;
  a.num_partitions = plan.num_partitions;
  a.qscale = plan.scale * kLog2e;
  a.max_logits = plan.max_logits;
  a.exp_sums = plan.exp_sums;
  a.tmp_out = plan.tmp_out;
  return a;
}

}  // namespace

hipError_t launch_phase1(const Plan& plan, const void* query, const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, const int32_t* seq_lens, hipStream_t stream) {
  const AttnParams a = make_params(plan, query, key_cache, value_cache, block_tables, seq_lens);
  const dim3 grid(plan.num_partitions, plan.num_kv_heads * plan.head_chunks, plan.num_seqs);
  const int gh = heads_template(plan.heads_per_wg);
  if (plan.layout == kLayoutTiled)
    return plan.dtype == 0 ? launch_attn_f32_tiled_split(a, plan.head_size, gh, grid, stream)
                           : launch_attn_bf16_tiled_split(a, plan.head_size, gh, grid, stream);
  return plan.dtype == 0 ? launch_attn_f32_rows_split(a, plan.head_size, gh, grid, stream)
                         : launch_attn_bf16_rows_split(a, plan.head_size, gh, grid, stream);
}

hipError_t launch_one_pass(const Plan& plan, float* out, const void* query, const void* key_cache,
                           const void* value_cache, const int32_t* block_tables, const int32_t* seq_lens,
                           hipStream_t stream) {
  AttnParams a = make_params(plan, query, key_cache, value_cache, block_tables, seq_lens);
  a.out = out;
  const dim3 grid(1, plan.num_kv_heads * plan.head_chunks, plan.num_seqs);
  const int gh = heads_template(plan.heads_per_wg);
  // one wave per workgroup once the batch alone gives every SIMD a workgroup;
  // otherwise four waves share each workgroup's context
  const int64_t wgs = (int64_t)grid.y * grid.z;
  const int waves = wgs >= 4 * (int64_t)device_cus() ? 1 : 4;
  if (plan.layout == kLayoutTiled)
    return plan.dtype == 0 ? launch_attn_f32_tiled_one_pass(a, plan.head_size, gh, waves, grid, stream)
                           : launch_attn_bf16_tiled_one_pass(a, plan.head_size, gh, waves, grid, stream);
  return plan.dtype == 0 ? launch_attn_f32_rows_one_pass(a, plan.head_size, gh, waves, grid, stream)
                         : launch_attn_bf16_rows_one_pass(a, plan.head_size, gh, waves, grid, stream);
}

hipError_t launch_phase2(const Plan& plan, float* out, const int32_t* seq_lens, hipStream_t stream) {
  MergeParams m{};
  m.out = out;
  m.seq_lens = seq_lens;
  m.max_logits = plan.max_logits;
  m.exp_sums = plan.exp_sums;
  m.tmp_out = plan.tmp_out;
  m.num_heads = plan.num_heads;
  m.head_size = plan.head_size;
  m.max_tokens = plan.max_blocks * kBlockTokens;
  m.partition = plan.partition;
  m.num_partitions = plan.num_partitions;
  const dim3 grid(plan.head_size / 64, plan.num_heads, plan.num_seqs);
  void* args[] = {&m};
  return hipLaunchKernel(reinterpret_cast<const void*>(&merge_kernel), grid, dim3(256), args, 0, stream);
}

hipError_t launch_workspace_fill(float* max_logits, float* exp_sums, float* tmp_out, size_t n_stats, size_t n_tmp,
                                 hipStream_t stream) {
  const size_t n = n_tmp > n_stats ? n_tmp : n_stats;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  void* args[] = {&max_logits, &exp_sums, &tmp_out, &n_stats, &n_tmp};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fill_kernel), dim3((unsigned)blocks), dim3(256), args, 0,
                         stream);
}

}  // namespace pad
