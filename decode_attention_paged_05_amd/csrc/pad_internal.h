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

// Phase-1 load balance.  Two modes share the chunk machinery:
//  * pool (a launch that fills the GPU once to four times over, but not by a
//    whole multiple of the compute units): workgroups are launched for the
//    first partitions only; the remaining partitions are cut into chunks that
//    workgroups take when they finish their own partition;
//  * queue (a launch of more than four workgroups per compute unit, at most
//    kQueueMaxSeqs sequences): a resident grid of 4 workgroups per compute
//    unit takes the live (sequence, head group, partition) items from a
//    ticket counter, the last ones cut into chunks.
// Phase 2 merges chunk entries with partition entries.  The workspace holds
// the ticket counter, the queue's live-item prefix (for phase 2) and one
// scratch slot per chunk.
constexpr int kMaxPoolChunks = 32;    // chunks per pooled partition
constexpr int kMaxPoolTickets = 512;  // chunks per launch
constexpr int kQueueMaxSeqs = 1024;
// counter area: the ticket counter alone in its first 256 bytes, then the
// queue's live-item count T and the live items before each sequence
constexpr int kQueueInfoOffset = 64;  // in uint32 (256 bytes)
constexpr int kPoolCounters = kQueueInfoOffset + 1 + kQueueMaxSeqs;
// One chunk entry in the scratch area (floats): per head h < 16 of the
// group its max logit (log2 units; -inf when the chunk holds no token, NaN
// after a block id outside the pool) at [h], its exp-sum relative to that max
// at [16 + h], and its normalised partial output row at [kPieceStats + h * D].
constexpr int kPieceStats = 64;
__host__ __device__ constexpr int piece_floats(int d) { return kPieceStats + kMaxHeadsPerGroup * d; }

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
  // workspace arrays (split only)
  float* max_logits;  // [S, H, NP]
  float* exp_sums;    // [S, H, NP]
  float* tmp_out;     // [S, H, NP, D]
  unsigned* counters; // [kPoolCounters]: [0] ticket counter (zero between calls); queue info
  float* scratch;     // [kMaxPoolTickets][piece_floats(D)]: chunk entries
};

hipError_t launch_phase1(const Plan& plan, const void* query, const void* key_cache,
                         const void* value_cache, const int32_t* block_tables,
                         const int32_t* seq_lens, hipStream_t stream);

hipError_t launch_phase2(const Plan& plan, float* out, const int32_t* seq_lens,
                         hipStream_t stream);

hipError_t launch_one_pass(const Plan& plan, float* out, const void* query,
                           const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           hipStream_t stream);

hipError_t launch_workspace_fill(float* max_logits, float* exp_sums, float* tmp_out,
                                 size_t n_stats, size_t n_tmp, unsigned* counters,
                                 size_t n_counters, hipStream_t stream);

}  // namespace pad
