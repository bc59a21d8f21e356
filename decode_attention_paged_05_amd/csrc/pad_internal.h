// Internal interface between the C-ABI host layer (pad_api.cpp) and the
// kernel launchers (pad_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pad {

// Tokens per KV block handled by the kernels.
constexpr int kBlockTokens = 16;
// Query heads one workgroup serves: the N width of the 16x16 matrix-core tile.
constexpr int kMaxHeadsPerGroup = 16;

// Phase-1 load balance: the balanced split.  When a launch's fixed-size
// partitions would give more workgroups than compute units (and it has at
// most kBalancedMaxSeqs sequences), phase 1 does not cut each context into
// partition_size-token partitions.  It lays the live (KV block, head group)
// units of all sequences end to end -- sequence by sequence, head group by
// head group, block by block -- and cuts that line into N equal ranges, one
// per resident one-wave workgroup.  Workgroup j walks units
// [floor(j B / N), floor((j + 1) B / N)) of the B live units; where its range
// crosses from one (sequence, head group) into the next, it writes one entry
// per (sequence, head group) it touched.  An entry is what a partition entry
// is (max logit, exp-sum, normalised partial output per query head), for a
// contiguous stretch of blocks rather than a fixed partition; the entries of
// a (sequence, head group) occupy its partition slots 0, 1, ... in order.  N
// is capped so that no (sequence, head group) gets more entries than it has
// partition slots.  Workgroup 0 publishes N, B and the per-sequence block
// prefix in the workspace's launch-info area, which phase 2 reads to find how
// many entries each (sequence, head) has.  Nothing in the workspace is read
// by phase 1, so no state carries from call to call.
constexpr int kBalancedMaxSeqs = 1024;
// Resident one-wave workgroups per compute unit that the balanced split
// launches, by cache layout, head size and element size.  Tiled, head size
// 256, bf16: two
// measured faster than three on every split workload (100K tokens 71.4-71.6
// against 72.1-72.3 us per step; 32 mixed sequences 344 against 349 us; 8 x
// 131072 MHA 3 748 against 3 779 us): phase 1 is as fast, and the merge has a
// third fewer entries; one was 13 % slower.  Tiled, smaller heads (a block of
// 8 KB or less, the same arithmetic and bookkeeping per block): four (64 / 8
// heads of 64: 100K tokens 40.9 against 51.7 us, 16 x 32K 174 against 208 us;
// heads of 128 unchanged; six slower).  Rows (P.V on the vector ALUs, four
// times the vector work per block): three, 72.5-72.7 against 74.3-74.8 us
// with two on the 100K step.  Tiled, head size 256, fp32 (a 32 KB block
// fills 128 registers: one block in flight per wave): three, 131-134 against
// 174-177 us with two on the 100K step; four 134 us.
#ifndef PAD_BALANCED_WGS_PER_CU_TILED
#define PAD_BALANCED_WGS_PER_CU_TILED 2
#endif
#ifndef PAD_BALANCED_WGS_PER_CU_TILED_SMALL
#define PAD_BALANCED_WGS_PER_CU_TILED_SMALL 4
#endif
#ifndef PAD_BALANCED_WGS_PER_CU_ROWS
#define PAD_BALANCED_WGS_PER_CU_ROWS 3
#endif
#ifndef PAD_BALANCED_WGS_PER_CU_TILED_F32
#define PAD_BALANCED_WGS_PER_CU_TILED_F32 3
#endif
constexpr int kBalancedWgsPerCuMax = 4;  // the most of them (partition sizes leave slots for it)
constexpr int balanced_wgs_per_cu(int kv_layout, int head_size, int elem_bytes) {
  return kv_layout != 1 ? PAD_BALANCED_WGS_PER_CU_ROWS  // 1: PAD_KV_TILED
         : head_size < 256 ? PAD_BALANCED_WGS_PER_CU_TILED_SMALL
         : elem_bytes == 4 ? PAD_BALANCED_WGS_PER_CU_TILED_F32
                           : PAD_BALANCED_WGS_PER_CU_TILED;
}
// Fewest blocks a balanced range holds (a range costs a query load, a table
// load and an entry write besides its blocks).
constexpr int kMinRangeBlocks = 8;
// launch-info words: [0] N, [1] B low 32 bits, [2] B high 32 bits,
// [3] zero, [4 + s] live blocks before sequence s (per head group), s <= S
constexpr int kInfoPrefix = 4;
constexpr int kInfoWords = kInfoPrefix + kBalancedMaxSeqs + 1;

// Whether phase 1 runs the balanced split: one workgroup per partition would
// give more workgroups than compute units, the batch has at most
// kBalancedMaxSeqs sequences, every head group has at least two partition
// slots, and the live blocks per head group fit 31 bits.  Phase 1, phase 2 and
// the host-side plan derive it from the same sizes and compute-unit count.
inline bool balanced_split(int64_t num_seqs, int64_t head_groups, int64_t num_partitions, int64_t max_blocks,
                           int64_t cus) {
  return num_seqs * head_groups * num_partitions > cus && num_seqs <= kBalancedMaxSeqs && num_partitions >= 2 &&
         num_seqs * max_blocks < ((int64_t)1 << 31);
}

// Which range holds unit x (the largest j with floor(j B / N) <= x).
__host__ __device__ inline uint64_t range_owner(uint64_t x, uint64_t N, uint64_t B) {
  return ((x + 1) * N - 1) / B;
}

// N for B units of which one head group holds at most nb_max: at most
// `wgs` ranges, at least kMinRangeBlocks units per range, and at most
// `slots` ranges touching any one head group (a head group of nb units meets
// at most 1 + ceil(nb N / B) ranges, so N nb_max <= (slots - 1) B suffices);
// above `cus`, a whole multiple of `cus`.  0 when there is nothing to do.
__host__ __device__ inline unsigned balanced_ranges(uint64_t B, uint64_t nb_max, unsigned wgs, unsigned slots,
                                                    unsigned cus) {
  if (B == 0 || nb_max == 0 || slots < 2 || wgs == 0) return 0;
  uint64_t n = wgs;
  const uint64_t a = slots - 1;
  const uint64_t lim = (uint64_t)wgs * nb_max;  // n nb_max <= a B for every n <= wgs once a B >= lim
  if (B < (lim + a - 1) / a) {
    const uint64_t cap = a * B / nb_max;  // a B < lim: no overflow
    if (cap < n) n = cap;
  }
  const uint64_t by_size = (B + kMinRangeBlocks - 1) / kMinRangeBlocks;
  if (by_size < n) n = by_size;
  if (cus > 0 && n > cus) n = n / cus * cus;
  return n < 1 ? 1u : (unsigned)n;
}

// Everything the launchers need, validated and derived on the host.
struct Plan {
  int dtype;          // PAD_DTYPE_*
  int layout;         // PAD_KV_* (0 rows, 1 tiled)
  int num_seqs;       // S
  int num_heads;      // H
  int num_kv_heads;   // Hkv
  int group;          // G = H / Hkv query heads per KV head
  int head_chunks;    // ceil(G / 16): workgroups per KV head
  int heads_per_wg;   // min(G, 16)
  int head_size;      // D
  int64_t num_blocks; // NB
  int max_blocks;     // W
  int partition;      // P tokens (0 = one-pass)
  int num_partitions; // NP = ceil(W * 16 / P) (0 for one-pass)
  float scale;        // softmax scale
  int64_t q_stride;   // elements between sequences' query rows
  int64_t out_stride; // floats between sequences' output rows
  // workspace arrays (split only)
  float* max_logits;  // [S, H, NP]
  float* exp_sums;    // [S, H, NP]
  float* tmp_out;     // [S, H, NP, D]
  unsigned* info;     // [kInfoWords]: the balanced split's launch info
};

// Compute units of the current device (cached per device; 256 if the query fails).
int device_cus();

hipError_t launch_phase1(const Plan& plan, const void* query, const void* key_cache,
                         const void* value_cache, const int32_t* block_tables,
                         const int32_t* seq_lens, hipStream_t stream);

hipError_t launch_phase2(const Plan& plan, float* out, const int32_t* seq_lens,
                         hipStream_t stream);

hipError_t launch_one_pass(const Plan& plan, float* out, const void* query,
                           const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           hipStream_t stream);

// Bytes of the library's static device workspace (the allocation-free entry
// point's), and its address on the current device, looked up once per device.
constexpr size_t kStaticWorkspaceBytes = (size_t)64 << 20;
hipError_t static_workspace(void** ptr);

hipError_t launch_workspace_fill(float* max_logits, float* exp_sums, float* tmp_out,
                                 size_t n_stats, size_t n_tmp, unsigned* info,
                                 size_t n_info, hipStream_t stream);

}  // namespace pad
