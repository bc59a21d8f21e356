// Internal interface between the C-ABI host layer (pad_api.cpp) and the
// prefix-attention launchers (pad_prefill.hip).  Not installed; not part of
// the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pad_internal.h"

namespace pad {

// Prefix (chunked prefill) attention and the chunk write (pad_prefill.hip).
constexpr int kKvRows = 0;   // PAD_KV_ROWS
constexpr int kKvTiled = 1;  // PAD_KV_TILED

struct PrefillArgs {
  float* out;                  // [T, H, D]
  const char* query;           // bf16 [T, H, D]
  const char* key_cache;       // bf16, tiled layout
  const char* value_cache;
  const int32_t* block_tables; // [S, W]
  const int32_t* query_start;  // [S + 1]
  const int32_t* context_lens; // [S]
  float qscale;                // softmax scale (the launcher folds in log2(e) and takes |.|)
  int negate_q;                // the scale was negative: the kernel flips the query's sign
  int num_tokens;              // T
  int num_heads;               // H
  int num_kv_heads;            // Hkv
  int group;                   // H / Hkv
  int head_groups;             // workgroups per KV head along the heads (set by the launcher)
  int max_blocks;              // W
  int64_t num_blocks;          // NB
};

struct WriteKvArgs {
  char* key_cache;             // [NB, Hkv, ...] in the cache layout
  char* value_cache;
  const char* key;             // [T, Hkv, D]
  const char* value;
  const int32_t* block_tables;
  const int32_t* query_start;
  const int32_t* context_lens;
  int num_tokens;
  int num_kv_heads;
  int head_size;
  int max_blocks;
  int64_t num_blocks;
};

// Query heads and chunk tokens one prefill workgroup serves, and whether a
// launch runs the solo layout (256 rows per workgroup; always below head size
// 256) or the paired one (128 rows).
int prefill_heads_per_wg(int group);
bool prefill_solo(int head_size, int group, int num_kv_heads, int max_query_len);
int prefill_tokens_per_wg(int group, bool solo);

hipError_t launch_prefill(const PrefillArgs& args, int num_seqs, int max_query_len, int head_size,
                          hipStream_t stream);

// Split launch of the prefix attention (solo layout): the resident
// workgroups of its walk kernel on the current device (N), the workspace it
// needs, and the launch (plan, walks, merge).
int prefill_split_ranges(int head_size, int group);
size_t prefill_split_workspace_bytes(int num_seqs, int num_kv_heads, int group, int head_size, int max_query_len,
                                     int max_blocks, int ranges);
// whether the split launch serves these lengths (host arrays) better: a
// batch of more than one sequence with chunk tokens, or walks it would cut
bool prefill_split_pays(const int32_t* context_lens, const int32_t* query_lens, int num_seqs, int num_kv_heads,
                        int group, int ranges);
// workgroups of the walk kernel (a bound on its units x head chunks)
int64_t prefill_split_grid(int num_seqs, int num_kv_heads, int group, int max_query_len, int max_blocks, int ranges);
hipError_t launch_prefill_split(const PrefillArgs& args, int num_seqs, int max_query_len, int head_size,
                                int ranges, void* workspace, hipStream_t stream);

hipError_t launch_write_kv(const WriteKvArgs& args, int num_seqs, int max_query_len, int elem_bytes, int layout,
                           hipStream_t stream);

}  // namespace pad
