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
// Phase 2: log-sum-exp merge.  Grid (D / kDims, H, S), kThreads threads (one
// wave or four); the workgroup owns kDims dims of one (sequence, head), as
// kDims / 4 dim lanes (4 dims each) x G source groups.  Thread t = kDims/4 g + l
// takes dims 4 l .. 4 l + 3 of entries g, g + G, g + 2 G, ... of the head's
// partition slots.  Every load of a round -- each entry's max and exp-sum and
// its four dims -- is issued before any arithmetic (the merge is
// latency-bound, not bandwidth-bound), and the first round is issued before
// the entry count is known.  Each thread keeps a running max, exp-sum and
// weighted row over its own entries; the source groups are then combined by
// the same log-sum-exp rule, by shuffles within a wave and through LDS across
// waves.  Slots past the head's entry count are read (they exist) but
// discarded by select, so stale or NaN contents never enter the sums.
//
// Entry count of (sequence s, head h): ceil(L_s / P) for one workgroup per
// partition; for the balanced split, the ranges that meet its head group,
// from the launch info phase 1 published (which must match this call's
// lengths, or the row is NaN).
// ---------------------------------------------------------------------------
struct MergeParams {
  float* out;              // rows of sequence s at s * out_stride
  int64_t out_stride;
  const int32_t* seq_lens;
  const float* max_logits;
  const float* exp_sums;
  const float* tmp_out;
  int num_heads;
  int head_size;
  int max_tokens;  // W * block_size
  int partition;
  int num_partitions;
  int balanced;
  const unsigned* info;  // balanced: launch info of phase 1
  int num_seqs;
  int gy_count;
  int head_chunks;
  int group;
};

// Merge workgroup shapes: kThreads threads own kDims dims of one (sequence,
// head); kDims / 4 "dim lanes" (4 dims each) x kThreads / (kDims / 4) source
// groups, kRound sources per round of loads.
template <int kThreads, int kDims, int kRound>
struct MergeShape {
  static constexpr int kDL = kDims / 4;            // dim lanes
  static constexpr int kG = kThreads / kDL;        // source groups
  static constexpr int kPerThread = kRound / kG;   // sources per thread per round
  static constexpr int kChunk = kG * kPerThread;   // sources per round
  static constexpr int kWaves = kThreads / kWave;
  static_assert(kDL >= 1 && kDL <= 16 && (kWave % kDL) == 0, "dim lanes within a wave");
  static_assert(kPerThread >= 1 && kChunk == kRound, "a round is a whole number of sources per thread");
};

// Entries to merge for (sequence s, head h): > 0; 0 for an empty sequence
// (zero row); -1 for a row that must be NaN (a length outside [0, W * 16],
// or launch info that does not match the lengths).
__device__ inline int merge_sources(const MergeParams& p, int s, int h) {
  const int L = p.seq_lens[s];
  if (L == 0) return 0;
  if (L < 0 || L > p.max_tokens) return -1;
  if (!p.balanced) return (L + p.partition - 1) / p.partition;
  const unsigned N = p.info[0];
  const uint64_t B = (uint64_t)p.info[1] | ((uint64_t)p.info[2] << 32);
  const unsigned pre_s = p.info[kInfoPrefix + s];
  const unsigned pre_s1 = p.info[kInfoPrefix + s + 1];
  const unsigned pre_all = p.info[kInfoPrefix + p.num_seqs];
  const unsigned nb = (unsigned)((L + kBlockTokens - 1) / kBlockTokens);
  if (N == 0 || pre_s1 - pre_s != nb || B != (uint64_t)pre_all * (uint64_t)p.gy_count) return -1;
  const int g = h / p.group;
  const int gy = g * p.head_chunks + (h - g * p.group) / kMaxHeadsPerGroup;
  const uint64_t g0 = (uint64_t)p.gy_count * pre_s + (uint64_t)gy * nb;
  const uint64_t n = range_owner(g0 + nb - 1, N, B) - range_owner(g0, N, B) + 1;
  return n > (uint64_t)p.num_partitions ? -1 : (int)n;
}

// Log-sum-exp combine of (max m, exp-sum l, weighted row a) with another
// partial; an empty partial has m = -inf, l = 0, a = 0; NaN propagates.
__device__ inline void lse_combine(float& m, float& l, f32x4_t& a, float m2, float l2, f32x4_t a2) {
  const float M = fmaxf(m, m2);
  const float f1 = m > -INFINITY ? fast_exp2(m - M) : 0.0f;
  const float f2 = m2 > -INFINITY ? fast_exp2(m2 - M) : 0.0f;
  l = l * f1 + l2 * f2;
  a = a * f1 + a2 * f2;
  m = M;
}

template <int kThreads, int kDims, int kRound>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeParams p) {
  using SH = MergeShape<kThreads, kDims, kRound>;
  constexpr int kDL = SH::kDL;
  constexpr int kMergeGroups = SH::kG;
  constexpr int kMergePerThread = SH::kPerThread;
  constexpr int kMergeChunk = SH::kChunk;
  __shared__ float m_sh[SH::kWaves][kDL];
  __shared__ float l_sh[SH::kWaves][kDL];
  __shared__ f32x4_t a_sh[SH::kWaves][kDL];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int s = blockIdx.z;
  const int h = blockIdx.y;
  const int D = p.head_size;
  const int d0 = blockIdx.x * kDims;
  const int dl = tid % kDL;
  const int pg = tid / kDL;
  const int NP = p.num_partitions;
  const size_t row0 = ((size_t)s * p.num_heads + h) * NP;
  const float* ml = p.max_logits + row0;
  const float* es = p.exp_sums + row0;
  const float* tmp = p.tmp_out + row0 * D + d0 + 4 * dl;
  float* orow = p.out + (size_t)s * (size_t)p.out_stride + (size_t)h * D + d0;
  f32x4_t a = {0.0f, 0.0f, 0.0f, 0.0f};
  float lrun = 0.0f;
  float mrun = -INFINITY;  // running max of this thread's sources, log2 units
  int nvalid = -1;         // entries of this (sequence, head): known after the first round's loads are issued
  for (int c0 = 0; c0 < NP; c0 += kMergeChunk) {
    // one round of loads: slots that exist, whatever the entry count (a slot
    // past the table reads slot 0, dropped below by select)
    float m2[kMergePerThread], l[kMergePerThread];
    f32x4_t t[kMergePerThread];
#pragma unroll
    for (int k = 0; k < kMergePerThread; ++k) {
      const int i = c0 + pg + kMergeGroups * k;
      const int ir = i < NP ? i : 0;
      m2[k] = ml[ir] * kLog2e;
      l[k] = es[ir];
      t[k] = *reinterpret_cast<const f32x4_t*>(tmp + (size_t)ir * D);
    }
    if (nvalid < 0) {
      nvalid = merge_sources(p, s, h);
      if (nvalid <= 0) {
        if (tid < kDims) orow[tid] = (nvalid == 0) ? 0.0f : __builtin_nanf("");
        return;
      }
    }
    if (c0 >= nvalid) break;
    float cm = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMergePerThread; ++k)
      if (c0 + pg + kMergeGroups * k < nvalid) cm = fmaxf(cm, m2[k]);
    if (cm > mrun) {
      const float resc = fast_exp2(mrun - cm);  // 0 while nothing was summed
      a *= resc;
      lrun *= resc;
      mrun = cm;
    }
#pragma unroll
    for (int k = 0; k < kMergePerThread; ++k) {
      if (c0 + pg + kMergeGroups * k >= nvalid) continue;
      // an entry without tokens (max -inf, exp-sum 0) weighs nothing; a NaN
      // max (a bad block id in phase 1) poisons the row
      const float w = m2[k] > -INFINITY ? l[k] * fast_exp2(m2[k] - mrun) : (m2[k] != m2[k] ? m2[k] : 0.0f);
      lrun += w;
      a += w * t[k];
    }
  }
  // combine the source groups: within each wave by shuffles over the lanes
  // that hold the same dims, then across the waves through LDS
#pragma unroll
  for (int off = kDL; off < kWave; off <<= 1) {
    const float m2 = __shfl_xor(mrun, off);
    const float l2 = __shfl_xor(lrun, off);
    f32x4_t a2;
#pragma unroll
    for (int e = 0; e < 4; ++e) a2[e] = __shfl_xor(a[e], off);
    lse_combine(mrun, lrun, a, m2, l2, a2);
  }
  if constexpr (SH::kWaves > 1) {
    if (lane < kDL) {
      m_sh[wave][lane] = mrun;
      l_sh[wave][lane] = lrun;
      a_sh[wave][lane] = a;
    }
    __syncthreads();
    if (tid < kDL) {
#pragma unroll
      for (int w = 1; w < SH::kWaves; ++w) lse_combine(mrun, lrun, a, m_sh[w][tid], l_sh[w][tid], a_sh[w][tid]);
    }
  }
  if (tid < kDL) *reinterpret_cast<f32x4_t*>(orow + 4 * tid) = a * (1.0f / lrun);
}

__global__ __launch_bounds__(256) void fill_kernel(float* ml, float* es, float* tmp, size_t n_stats,
                                                   size_t n_tmp, unsigned* info, size_t n_info) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (size_t i = i0; i < n_stats; i += stride) {
    ml[i] = -INFINITY;
    es[i] = 0.0f;
  }
  for (size_t i = i0; i < n_tmp; i += stride) tmp[i] = 0.0f;
  for (size_t i = i0; i < n_info; i += stride) info[i] = 0u;
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


AttnParams make_params(const Plan& plan, const void* q, const void* k, const void* v, const int32_t* tables,
                       const int32_t* lens) {
  AttnParams a{};
  a.query = static_cast<const char*>(q);
  a.key_cache = static_cast<const char*>(k);
  a.value_cache = static_cast<const char*>(v);
  a.block_tables = tables;
  a.seq_lens = lens;
  a.num_blocks = plan.num_blocks;
  a.q_stride = plan.q_stride;
  a.out_stride = plan.out_stride;
  a.num_seqs = plan.num_seqs;
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
  a.info = plan.info;
  a.gy_count = plan.num_kv_heads * plan.head_chunks;
  a.num_cus = device_cus();
  return a;
}


bool use_balanced(const Plan& plan) {
  return PAD_SPLIT_WAVES == 1 && plan.info != nullptr &&
         balanced_split(plan.num_seqs, (int64_t)plan.num_kv_heads * plan.head_chunks, plan.num_partitions,
                        plan.max_blocks, device_cus());
}

}  // namespace

hipError_t launch_phase1(const Plan& plan, const void* query, const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, const int32_t* seq_lens, hipStream_t stream) {
  AttnParams a = make_params(plan, query, key_cache, value_cache, block_tables, seq_lens);
  const bool bal = use_balanced(plan);
  a.balanced = bal ? 1 : 0;
  const dim3 grid = bal ? dim3((unsigned)(balanced_wgs_per_cu(plan.layout, plan.head_size, plan.dtype == 0 ? 4 : 2) *
                                          a.num_cus))
                        : dim3(plan.num_partitions, plan.num_kv_heads * plan.head_chunks, plan.num_seqs);
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

#ifndef PAD_MERGE_SHAPE
#define PAD_MERGE_SHAPE 0  // 0: chosen per launch below
#endif

hipError_t launch_phase2(const Plan& plan, float* out, const int32_t* seq_lens, hipStream_t stream) {
  MergeParams m{};
  m.out = out;
  m.out_stride = plan.out_stride;
  m.seq_lens = seq_lens;
  m.max_logits = plan.max_logits;
  m.exp_sums = plan.exp_sums;
  m.tmp_out = plan.tmp_out;
  m.num_heads = plan.num_heads;
  m.head_size = plan.head_size;
  m.max_tokens = plan.max_blocks * kBlockTokens;
  m.partition = plan.partition;
  m.num_partitions = plan.num_partitions;
  m.balanced = use_balanced(plan) ? 1 : 0;
  m.info = plan.info;
  m.num_seqs = plan.num_seqs;
  m.gy_count = plan.num_kv_heads * plan.head_chunks;
  m.head_chunks = plan.head_chunks;
  m.group = plan.group;
  void* args[] = {&m};
  const int D = plan.head_size;
  auto launch = [&](const void* k, int threads, int dims) {
    return hipLaunchKernel(k, dim3(D / dims, plan.num_heads, plan.num_seqs), dim3(threads), args, 0, stream);
  };
#define PAD_MERGE(T, DIMS, R) launch(reinterpret_cast<const void*>(&merge_kernel<T, DIMS, R>), T, DIMS)
#if PAD_MERGE_SHAPE
  // fixed shape (tuning builds)
  switch (PAD_MERGE_SHAPE) {
    case 1: return PAD_MERGE(64, 64, 16);
    case 2: return PAD_MERGE(64, 32, 64);
    case 3: return PAD_MERGE(256, 16, 256);
    case 4: return PAD_MERGE(256, 32, 256);
    case 5: return PAD_MERGE(256, 64, 256);
    case 6: return PAD_MERGE(64, 64, 64);
    default: return PAD_MERGE(64, 16, 16);
  }
#endif
  // Entries per (sequence, head) the first round of loads should cover: for
  // the balanced split about (ranges + head groups) / head groups when the
  // sequences are alike (the ranges number balanced_wgs_per_cu per compute
  // unit at most); for
  // one workgroup per partition up to the table's partition count.
  const int64_t cus = device_cus();
  const int64_t groups = (int64_t)plan.num_seqs * plan.num_kv_heads * plan.head_chunks;
  const int64_t expect =
      m.balanced ? (pad::balanced_wgs_per_cu(plan.layout, plan.head_size, plan.dtype == 0 ? 4 : 2) * cus + groups +
                    groups - 1) / groups
                 : plan.num_partitions;
  // Measured on 256 compute units: one wave on 64 dims with rounds of 16
  // entries when a head has few (8 x 131072 MHA tokens or a batch of 32
  // sequences under the balanced split); one wave on 32 dims with rounds of 64
  // up to 64 entries; otherwise 256 threads on 32 dims while the grid stays
  // within about eight workgroups per compute unit, else on 64 dims.  (One
  // 100K sequence, 128 entries per head: 32 dims 70.5-71.0 us per step, 16
  // dims 71.4-71.9 us, 64 dims 71.2 us; with three phase-1 workgroups per
  // compute unit and 192 entries, 16 dims had been the fastest.)
  const int64_t rows = (int64_t)plan.num_heads * plan.num_seqs;
  if (expect <= 16) return PAD_MERGE(64, 64, 16);
  if (expect <= 64) return PAD_MERGE(64, 32, 64);
  if (rows * (D / 32) <= 8 * cus) return PAD_MERGE(256, 32, 256);
  return PAD_MERGE(256, 64, 256);
#undef PAD_MERGE
}

hipError_t launch_workspace_fill(float* max_logits, float* exp_sums, float* tmp_out, size_t n_stats, size_t n_tmp,
                                 unsigned* info, size_t n_info, hipStream_t stream) {
  const size_t n = n_tmp > n_stats ? n_tmp : n_stats;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  void* args[] = {&max_logits, &exp_sums, &tmp_out, &n_stats, &n_tmp, &info, &n_info};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fill_kernel), dim3((unsigned)blocks), dim3(256), args, 0,
                         stream);
}

// The workspace of paged_attention_decode_no_alloc: a file-scope device array,
// one per GPU the library runs on, held until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is a stand-in, not
// a device address): static_workspace() looks up each device's address once,
// with that device current, and every launch takes that pointer.
static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

hipError_t static_workspace(void** ptr) {
  static std::atomic<void*> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    cache[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace pad
