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
// Phase 2: log-sum-exp merge.  Grid (D / kDims, H, S), kThreads threads (one
// wave or four); the workgroup owns kDims dims of one (sequence, head), as
// kDims / 4 dim lanes (4 dims each) x G source groups.  Thread t = kDims/4 g + l
// takes dims 4 l .. 4 l + 3 of sources g, g + G, g + 2 G, ... (a source is a
// partition entry or a chunk entry).  Every load of a round -- each source's
// max and exp-sum and its four dims -- is issued before any arithmetic (the
// merge is latency-bound, not bandwidth-bound).  Each thread keeps a running
// max, exp-sum and weighted row over its own sources; the source groups are
// then combined by the same log-sum-exp rule, by shuffles within a wave and
// through LDS across waves.  Slots past the sequence's source count are read
// (they exist) but discarded by select, so stale or NaN contents never enter
// the sums.
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
  // phase-1 pool (pool_chunks == 0: none): partitions >= main_parts arrive as
  // pool_chunks chunk entries each in `scratch`
  const float* scratch;
  int main_parts;
  int pool_parts;
  int pool_chunks;
  int gy_count;
  int head_chunks;
  int group;
  // phase-1 queue (queue == 0: none): queue_info[0] = T live items,
  // queue_info[1 + s] = items before sequence s; the last min(T, queue_tail)
  // items arrive as pool_chunks chunk entries each
  int queue;
  int queue_tail;
  const unsigned* queue_info;
};

// Merge workgroup shapes: kThreads threads own kDims dims of one (sequence,
// head); kDims / 4 "dim lanes" (4 dims each) x kThreads / (kDims / 4) source
// groups.  Sources per round: 256 for 256 threads, 64 for one wave.
template <int kThreads, int kDims>
struct MergeShape {
  static constexpr int kDL = kDims / 4;            // dim lanes
  static constexpr int kG = kThreads / kDL;        // source groups
  static constexpr int kPerThread = (kThreads == 64 ? 64 : 256) / kG;  // sources per thread per round
  static constexpr int kChunk = kG * kPerThread;   // sources per round
  static constexpr int kWaves = kThreads / kWave;
  static_assert(kDL >= 1 && kDL <= 16 && (kWave % kDL) == 0, "dim lanes within a wave");
};

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

template <int kThreads, int kDims>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeParams p) {
  using SH = MergeShape<kThreads, kDims>;
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
  float* orow = p.out + ((size_t)s * p.num_heads + h) * D + d0;
  // Sources: partition entries [0, n_reg), then the chunk entries of the
  // partitions from n_reg on, C per partition, in scratch slots first_slot,
  // first_slot + 1, ...
  const int C = p.pool_chunks;
  // this head's place among the pooled items and inside a chunk entry
  const int g = h / p.group;
  const int within = h - g * p.group;
  const int hc = within / kMaxHeadsPerGroup;
  const int hh = within - hc * kMaxHeadsPerGroup;
  const int gy = g * p.head_chunks + hc;
  int n_reg, n_src, first_slot;
  int nvalid = -1;  // sources of this sequence (pool / plain: known after the first round's loads)
  if (p.queue) {
    // the sequence's live items are pre_s + gy * np + partition; items from
    // cut = T - K on are chunked (slot = (item - cut) * C + chunk)
    const int L = p.seq_lens[s];
    if (L <= 0 || L > p.max_tokens) {
      if (tid < kDims) orow[tid] = (L == 0) ? 0.0f : __builtin_nanf("");
      return;
    }
    const int np = (L + p.partition - 1) / p.partition;
    const unsigned T = p.queue_info[0];
    const unsigned K = T < (unsigned)p.queue_tail ? T : (unsigned)p.queue_tail;
    const long long cut = (long long)(T - K);
    const long long base = (long long)p.queue_info[1 + s] + (long long)gy * np;
    const long long r = cut - base;
    n_reg = r <= 0 ? 0 : (r >= np ? np : (int)r);
    first_slot = (int)((base + n_reg - cut) * C);
    n_src = n_reg + (np - n_reg) * C;
    nvalid = n_src;
  } else if (C > 0) {
    // pool: partitions [main_parts, NP) of every (sequence, head group), item
    // (s * gy_count + gy) * pool_parts + pp, slot item * C + chunk
    n_reg = p.main_parts;
    n_src = p.main_parts + p.pool_parts * C;
    first_slot = (s * p.gy_count + gy) * p.pool_parts * C;
  } else {
    n_reg = NP;
    n_src = NP;
    first_slot = 0;
  }
  const int PF = piece_floats(D);

  f32x4_t a = {0.0f, 0.0f, 0.0f, 0.0f};
  float lrun = 0.0f;
  float mrun = -INFINITY;  // running max of this thread's sources, log2 units
  for (int c0 = 0; c0 < n_src; c0 += kMergeChunk) {
    // one round of loads: sources that exist, whatever the sequence length
    float m2[kMergePerThread], l[kMergePerThread];
    f32x4_t t[kMergePerThread];
#pragma unroll
    for (int k = 0; k < kMergePerThread; ++k) {
      // branch-free: pick the three addresses, load unconditionally (a source
      // past the list reads partition 0's entry, dropped below by select)
      const int i = c0 + pg + kMergeGroups * k;
      const bool reg = i < n_reg || i >= n_src;
      const int ir = i < n_reg ? i : 0;
      const float* q = p.scratch + (size_t)(reg ? 0 : first_slot + (i - n_reg)) * PF;
      const float* pm = reg ? ml + ir : q + hh;
      const float* pl = reg ? es + ir : q + 16 + hh;
      const float* pr = reg ? tmp + (size_t)ir * D : q + kPieceStats + hh * D + d0 + 4 * dl;
      m2[k] = *pm * (reg ? kLog2e : 1.0f);
      l[k] = *pl;
      t[k] = *reinterpret_cast<const f32x4_t*>(pr);
    }
    if (nvalid < 0) {
      const int L = p.seq_lens[s];
      if (L <= 0 || L > p.max_tokens) {
        if (tid < kDims) orow[tid] = (L == 0) ? 0.0f : __builtin_nanf("");
        return;
      }
      const int np = (L + p.partition - 1) / p.partition;
      nvalid = C > 0 ? (np <= n_reg ? np : n_reg + (np - n_reg) * C) : np;
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
      // a chunk without tokens (max -inf, exp-sum 0) weighs nothing; a NaN max
      // (a bad block id in phase 1) poisons the row
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
                                                   size_t n_tmp, unsigned* counters, size_t n_counters) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (size_t i = i0; i < n_stats; i += stride) {
    ml[i] = -INFINITY;
    es[i] = 0.0f;
  }
  for (size_t i = i0; i < n_tmp; i += stride) tmp[i] = 0.0f;
  for (size_t i = i0; i < n_counters; i += stride) counters[i] = 0u;
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
  a.counters = plan.counters;
  a.scratch = plan.scratch;
  a.gy_count = plan.num_kv_heads * plan.head_chunks;
  return a;
}

#ifndef PAD_POOL_CHUNK_BLOCKS
#define PAD_POOL_CHUNK_BLOCKS 4  // blocks per pooled chunk
#endif

// The load-balance rule (phase 1 and phase 2 derive the same plan from the
// same sizes).  With `items` one-wave partition workgroups and C compute units:
//  * C < items <= 4 C, not a multiple of C (one resident round): pool.  The
//    first k * C partition workgroups (k = items / C) are launched; the other
//    partitions of every (sequence, head group) are cut into chunks;
//  * items > 4 C and at most kQueueMaxSeqs sequences: queue.  4 C resident
//    workgroups take live items from the ticket counter; up to
//    kMaxPoolTickets / chunks of the last live items are cut into chunks.
struct PoolPlan {
  int main_parts = 0;  // pool: partitions per (sequence, head group) launched as workgroups
  int pool_parts = 0;
  int chunks = 0;      // chunks per pooled partition (or queue tail item); 0 = neither mode
  int chunk_blocks = 0;
  int tickets = 0;     // pool: chunk tickets
  bool queue = false;
  int queue_wgs = 0;   // queue: resident workgroups
  int queue_tail = 0;  // queue: most tail items cut into chunks
};

PoolPlan plan_pool(const Plan& plan) {
  PoolPlan pp;
  const int np = plan.num_partitions;
  pp.main_parts = np;
  if (PAD_SPLIT_WAVES != 1 || plan.counters == nullptr || plan.scratch == nullptr) return pp;
  const int64_t per_col = (int64_t)plan.num_seqs * plan.num_kv_heads * plan.head_chunks;
  const int64_t items = per_col * np;
  const int64_t cus = device_cus();
  const int pblocks = plan.partition / kBlockTokens;
  const int cb = PAD_POOL_CHUNK_BLOCKS;
  const int chunks = (pblocks + cb - 1) / cb;
  if (chunks > kMaxPoolChunks) return pp;
  if (items > 4 * cus) {
    if (plan.num_seqs > kQueueMaxSeqs) return pp;
    pp.queue = true;
    pp.queue_wgs = (int)(4 * cus);
    pp.chunks = chunks;
    pp.chunk_blocks = cb;
    pp.queue_tail = kMaxPoolTickets / chunks;
    return pp;
  }
  if (items <= cus || items % cus == 0) return pp;
  const int64_t main_parts = (items / cus) * cus / per_col;
  const int64_t pool_parts = np - main_parts;
  const int64_t tickets = per_col * pool_parts * chunks;
  if (main_parts < 1 || pool_parts < 1 || tickets > kMaxPoolTickets) return pp;
  pp.main_parts = (int)main_parts;
  pp.pool_parts = (int)pool_parts;
  pp.chunks = chunks;
  pp.chunk_blocks = cb;
  pp.tickets = (int)tickets;
  return pp;
}

}  // namespace

hipError_t launch_phase1(const Plan& plan, const void* query, const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, const int32_t* seq_lens, hipStream_t stream) {
  AttnParams a = make_params(plan, query, key_cache, value_cache, block_tables, seq_lens);
  const PoolPlan pp = plan_pool(plan);
  a.main_parts = pp.main_parts;
  a.pool_parts = pp.pool_parts;
  a.pool_chunks = pp.chunks;
  a.pool_chunk_blocks = pp.chunk_blocks;
  a.pool_tickets = pp.tickets;
  a.queue = pp.queue ? 1 : 0;
  a.queue_tail = pp.queue_tail;
  const dim3 grid = pp.queue ? dim3((unsigned)pp.queue_wgs)
                             : dim3(pp.main_parts, plan.num_kv_heads * plan.head_chunks, plan.num_seqs);
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
  m.seq_lens = seq_lens;
  m.max_logits = plan.max_logits;
  m.exp_sums = plan.exp_sums;
  m.tmp_out = plan.tmp_out;
  m.num_heads = plan.num_heads;
  m.head_size = plan.head_size;
  m.max_tokens = plan.max_blocks * kBlockTokens;
  m.partition = plan.partition;
  m.num_partitions = plan.num_partitions;
  const PoolPlan pp = plan_pool(plan);
  m.scratch = plan.scratch;
  m.main_parts = pp.main_parts;
  m.pool_parts = pp.pool_parts;
  m.pool_chunks = pp.chunks;
  m.gy_count = plan.num_kv_heads * plan.head_chunks;
  m.head_chunks = plan.head_chunks;
  m.group = plan.group;
  m.queue = pp.queue ? 1 : 0;
  m.queue_tail = pp.queue_tail;
  m.queue_info = plan.counters + kQueueInfoOffset;
  const dim3 grid(plan.head_size / 64, plan.num_heads, plan.num_seqs);
  void* args[] = {&m};
#if PAD_MERGE_SHAPE
  // fixed shape (tuning builds): 1 <64,64>, 2 <256,16>, 3 <256,32>, 4 <256,64>, 5 <64,16>, 6 <64,32>
  {
    const void* k = PAD_MERGE_SHAPE == 1 ? reinterpret_cast<const void*>(&merge_kernel<64, 64>)
                  : PAD_MERGE_SHAPE == 2 ? reinterpret_cast<const void*>(&merge_kernel<256, 16>)
                  : PAD_MERGE_SHAPE == 3 ? reinterpret_cast<const void*>(&merge_kernel<256, 32>)
                  : PAD_MERGE_SHAPE == 4 ? reinterpret_cast<const void*>(&merge_kernel<256, 64>)
                  : PAD_MERGE_SHAPE == 5 ? reinterpret_cast<const void*>(&merge_kernel<64, 16>)
                                         : reinterpret_cast<const void*>(&merge_kernel<64, 32>);
    const int dims = (PAD_MERGE_SHAPE == 2 || PAD_MERGE_SHAPE == 5) ? 16 : (PAD_MERGE_SHAPE == 3 || PAD_MERGE_SHAPE == 6) ? 32 : 64;
    const int threads = (PAD_MERGE_SHAPE == 1 || PAD_MERGE_SHAPE >= 5) ? 64 : 256;
    return hipLaunchKernel(k, dim3(plan.head_size / dims, plan.num_heads, plan.num_seqs), dim3(threads), args, 0,
                           stream);
  }
#endif
  // Measured on 256 compute units (phase 2 alone): one wave on 32 dims for
  // tables of at most 64 partitions (a batch of 32 sequences up to 32K tokens:
  // 22 us against 27 us with 64 dims); otherwise 256 threads on 16 dims while
  // the grid stays within about three workgroups per compute unit (one 100K
  // sequence), on 32 dims up to about eight (8 x 131072 tokens, MHA: 17.5 us
  // against 19 us with 64 dims), else on 64 dims.
  const int64_t rows = (int64_t)plan.num_heads * plan.num_seqs;
  const int64_t cus = device_cus();
  if (plan.num_partitions <= 64)
    return hipLaunchKernel(reinterpret_cast<const void*>(&merge_kernel<64, 32>),
                           dim3(plan.head_size / 32, plan.num_heads, plan.num_seqs), dim3(64), args, 0, stream);
  if (rows * (plan.head_size / 16) <= 3 * cus)
    return hipLaunchKernel(reinterpret_cast<const void*>(&merge_kernel<256, 16>),
                           dim3(plan.head_size / 16, plan.num_heads, plan.num_seqs), dim3(256), args, 0, stream);
  if (rows * (plan.head_size / 32) <= 8 * cus)
    return hipLaunchKernel(reinterpret_cast<const void*>(&merge_kernel<256, 32>),
                           dim3(plan.head_size / 32, plan.num_heads, plan.num_seqs), dim3(256), args, 0, stream);
  return hipLaunchKernel(reinterpret_cast<const void*>(&merge_kernel<256, 64>), grid, dim3(256), args, 0, stream);
}

hipError_t launch_workspace_fill(float* max_logits, float* exp_sums, float* tmp_out, size_t n_stats, size_t n_tmp,
                                 unsigned* counters, size_t n_counters, hipStream_t stream) {
  const size_t n = n_tmp > n_stats ? n_tmp : n_stats;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  void* args[] = {&max_logits, &exp_sums, &tmp_out, &n_stats, &n_tmp, &counters, &n_counters};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fill_kernel), dim3((unsigned)blocks), dim3(256), args, 0,
                         stream);
}

}  // namespace pad
