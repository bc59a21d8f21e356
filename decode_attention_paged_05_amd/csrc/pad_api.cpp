// Host side of the C ABI: argument validation (before any HIP call), the
// workspace layout, the one-pass/split choice and the launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <algorithm>
#include <vector>

#include "paged_attention_decode.h"
#include "paged_attention_prefill.h"
#include "pad_internal.h"
#include "pad_prefill_internal.h"

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Layout {
  size_t ml, es, tmp, info, total;
  int64_t np;
  size_t n_stats, n_tmp;
};

// Workspace layout for a split call; returns false on invalid sizes.
bool workspace_layout(int32_t S, int32_t H, int32_t D, int32_t W, int32_t bs, int32_t P, Layout* out) {
  if (S < 0 || H <= 0 || D <= 0 || W <= 0 || bs <= 0 || P < 0) return false;
  if (P == 0) {
    *out = Layout{0, 0, 0, 0, 0, 0, 0, 0};
    return true;
  }
  if (P % bs) return false;
  const int64_t tokens = (int64_t)W * bs;
  const int64_t np = (tokens + P - 1) / P;
  const size_t n_stats = (size_t)S * (size_t)H * (size_t)np;
  const size_t n_tmp = n_stats * (size_t)D;
  Layout l;
  l.np = np;
  l.n_stats = n_stats;
  l.n_tmp = n_tmp;
  l.ml = 0;
  l.es = round_up(n_stats * sizeof(float), kAlign);
  l.tmp = l.es + round_up(n_stats * sizeof(float), kAlign);
  // the balanced split's launch info
  l.info = l.tmp + round_up(n_tmp * sizeof(float), kAlign);
  l.total = l.info + round_up(pad::kInfoWords * sizeof(unsigned), kAlign);
  *out = l;
  return true;
}

// Validation shared by the attention entry points.
int32_t validate(const void* query, const void* key_cache, const void* value_cache, const int32_t* block_tables,
                 const int32_t* seq_lens, float scale, int32_t num_kv_heads, int32_t block_size,
                 int32_t partition_size, const pad_dims_t* dims) {
  if (!dims) return PAD_ERR_NULL;
  if (dims->dtype != PAD_DTYPE_F32 && dims->dtype != PAD_DTYPE_BF16) return PAD_ERR_DTYPE;
  if (dims->kv_layout != PAD_KV_ROWS && dims->kv_layout != PAD_KV_TILED) return PAD_ERR_DTYPE;
  if (dims->num_seqs < 0 || dims->num_heads <= 0 || num_kv_heads <= 0 || dims->num_blocks <= 0 ||
      dims->max_blocks_per_seq <= 0 || dims->head_size <= 0)
    return PAD_ERR_SHAPE;
  if (dims->num_heads % num_kv_heads != 0) return PAD_ERR_SHAPE;
  if (!std::isfinite(scale)) return PAD_ERR_SHAPE;
  if (dims->head_size != 64 && dims->head_size != 128 && dims->head_size != 256) return PAD_ERR_UNSUPPORTED;
  if (block_size != pad::kBlockTokens) return PAD_ERR_UNSUPPORTED;
  // grid limits: y = KV heads x head chunks, z = sequences
  const int group = dims->num_heads / num_kv_heads;
  const int chunks = (group + pad::kMaxHeadsPerGroup - 1) / pad::kMaxHeadsPerGroup;
  if ((int64_t)num_kv_heads * chunks > 65535 || dims->num_seqs > 65535) return PAD_ERR_UNSUPPORTED;
  // token counts must fit int32 inside the kernels
  if ((int64_t)dims->max_blocks_per_seq * block_size > INT32_MAX / 2) return PAD_ERR_UNSUPPORTED;
  if (partition_size < 0 || partition_size % block_size) return PAD_ERR_PARTITION;
  // row strides: 0 = contiguous; otherwise at least one sequence's rows, and
  // rows that stay 16-byte aligned
  const int64_t row = (int64_t)dims->num_heads * dims->head_size;
  if ((dims->query_seq_stride != 0 && dims->query_seq_stride < row) ||
      (dims->out_seq_stride != 0 && dims->out_seq_stride < row))
    return PAD_ERR_SHAPE;
  const int64_t elem = dims->dtype == PAD_DTYPE_BF16 ? 2 : 4;
  if ((dims->query_seq_stride * elem) % 16 || (dims->out_seq_stride * 4) % 16) return PAD_ERR_ALIGN;
  if (dims->num_seqs == 0) return PAD_OK;
  if (!query || !key_cache || !value_cache || !block_tables || !seq_lens) return PAD_ERR_NULL;
  if (!aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) || (reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return PAD_ERR_ALIGN;
  return PAD_OK;
}

pad::Plan make_plan(float scale, int32_t num_kv_heads, int32_t partition_size, const pad_dims_t* dims) {
  pad::Plan p{};
  p.dtype = dims->dtype;
  p.layout = dims->kv_layout;
  p.num_seqs = dims->num_seqs;
  p.num_heads = dims->num_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = dims->num_heads / num_kv_heads;
  p.head_chunks = (p.group + pad::kMaxHeadsPerGroup - 1) / pad::kMaxHeadsPerGroup;
  p.heads_per_wg = p.group < pad::kMaxHeadsPerGroup ? p.group : pad::kMaxHeadsPerGroup;
  p.head_size = dims->head_size;
  p.num_blocks = dims->num_blocks;
  p.max_blocks = dims->max_blocks_per_seq;
  p.partition = partition_size;
  p.scale = scale;
  const int64_t row = (int64_t)dims->num_heads * dims->head_size;
  p.q_stride = dims->query_seq_stride ? dims->query_seq_stride : row;
  p.out_stride = dims->out_seq_stride ? dims->out_seq_stride : row;
  return p;
}

// Attach the workspace arrays; false if it is missing or too small.
bool attach_workspace(pad::Plan* p, void* workspace, size_t workspace_bytes) {
  Layout l;
  if (!workspace_layout(p->num_seqs, p->num_heads, p->head_size, p->max_blocks, pad::kBlockTokens, p->partition, &l))
    return false;
  if (!workspace || workspace_bytes < l.total || !aligned16(workspace)) return false;
  char* base = static_cast<char*>(workspace);
  p->num_partitions = (int)l.np;
  p->max_logits = reinterpret_cast<float*>(base + l.ml);
  p->exp_sums = reinterpret_cast<float*>(base + l.es);
  p->tmp_out = reinterpret_cast<float*>(base + l.tmp);
  p->info = reinterpret_cast<unsigned*>(base + l.info);
  return true;
}

int32_t status_of(hipError_t e) { return e == hipSuccess ? PAD_OK : (int32_t)e; }

// Validation shared by the prefill entry points (sizes first, then pointers).
int32_t validate_prefill(const pad_prefill_dims_t* d, int32_t num_kv_heads, int32_t block_size, bool attention) {
  if (!d) return PAD_ERR_NULL;
  if (d->dtype != PAD_DTYPE_F32 && d->dtype != PAD_DTYPE_BF16) return PAD_ERR_DTYPE;
  if (d->kv_layout != PAD_KV_ROWS && d->kv_layout != PAD_KV_TILED) return PAD_ERR_DTYPE;
  if (d->num_seqs < 0 || d->num_tokens < 0 || d->max_query_len < 0 || d->num_heads <= 0 || num_kv_heads <= 0 ||
      d->num_blocks <= 0 || d->max_blocks_per_seq <= 0 || d->head_size <= 0)
    return PAD_ERR_SHAPE;
  if (attention && d->num_heads % num_kv_heads != 0) return PAD_ERR_SHAPE;
  if (d->head_size != 64 && d->head_size != 128 && d->head_size != 256) return PAD_ERR_UNSUPPORTED;
  if (block_size != pad::kBlockTokens) return PAD_ERR_UNSUPPORTED;
  // the attention kernels are bf16, tiled layout
  if (attention && (d->dtype != PAD_DTYPE_BF16 || d->kv_layout != PAD_KV_TILED)) return PAD_ERR_UNSUPPORTED;
  // offsets inside the kernels are 32-bit: query / out bytes, positions
  const int64_t heads = attention ? d->num_heads : num_kv_heads;
  if ((int64_t)d->num_tokens * heads * d->head_size * 4 > INT32_MAX) return PAD_ERR_UNSUPPORTED;
  if ((int64_t)d->max_blocks_per_seq * block_size > INT32_MAX / 2) return PAD_ERR_UNSUPPORTED;
  if (d->num_seqs > 65535) return PAD_ERR_UNSUPPORTED;
  if (attention) {
    const int group = d->num_heads / num_kv_heads;
    const int64_t y = (int64_t)num_kv_heads * (group / pad::prefill_heads_per_wg(group));
    if (y > 65535) return PAD_ERR_UNSUPPORTED;
  }
  return PAD_OK;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

extern "C" {

size_t paged_attention_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_size,
                                             int32_t max_blocks_per_seq, int32_t block_size, int32_t partition_size) {
  Layout l;
  if (!workspace_layout(num_seqs, num_heads, head_size, max_blocks_per_seq, block_size, partition_size, &l))
    return (size_t)-1;
  return l.total;
}

int32_t paged_attention_decode_workspace_layout(int32_t num_seqs, int32_t num_heads, int32_t head_size,
                                                int32_t max_blocks_per_seq, int32_t block_size,
                                                int32_t partition_size, size_t* max_logits_offset,
                                                size_t* exp_sums_offset, size_t* tmp_output_offset) {
  Layout l;
  if (!workspace_layout(num_seqs, num_heads, head_size, max_blocks_per_seq, block_size, partition_size, &l))
    return partition_size < 0 || (block_size > 0 && partition_size % block_size) ? PAD_ERR_PARTITION : PAD_ERR_SHAPE;
  if (max_logits_offset) *max_logits_offset = l.ml;
  if (exp_sums_offset) *exp_sums_offset = l.es;
  if (tmp_output_offset) *tmp_output_offset = l.tmp;
  return PAD_OK;
}

int32_t paged_attention_decode_workspace_init(void* workspace, size_t workspace_bytes, int32_t num_seqs,
                                              int32_t num_heads, int32_t head_size, int32_t max_blocks_per_seq,
                                              int32_t block_size, int32_t partition_size, void* stream) {
  Layout l;
  if (partition_size < 0 || (block_size > 0 && partition_size % block_size)) return PAD_ERR_PARTITION;
  if (!workspace_layout(num_seqs, num_heads, head_size, max_blocks_per_seq, block_size, partition_size, &l))
    return PAD_ERR_SHAPE;
  if (l.total == 0) return PAD_OK;
  if (!workspace) return PAD_ERR_WORKSPACE;
  if (workspace_bytes < l.total) return PAD_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PAD_ERR_ALIGN;
  char* base = static_cast<char*>(workspace);
  return status_of(pad::launch_workspace_fill(reinterpret_cast<float*>(base + l.ml),
                                              reinterpret_cast<float*>(base + l.es),
                                              reinterpret_cast<float*>(base + l.tmp), l.n_stats, l.n_tmp,
                                              reinterpret_cast<unsigned*>(base + l.info), pad::kInfoWords,
                                              static_cast<hipStream_t>(stream)));
}

int32_t paged_attention_decode_phase1(const void* query, const void* key_cache, const void* value_cache,
                                      const int32_t* block_tables, const int32_t* seq_lens, float scale,
                                      int32_t num_kv_heads, int32_t block_size, int32_t partition_size,
                                      void* workspace, size_t workspace_bytes, const pad_dims_t* dims,
                                      void* stream) {
  int32_t st = validate(query, key_cache, value_cache, block_tables, seq_lens, scale, num_kv_heads, block_size,
                        partition_size, dims);
  if (st != PAD_OK) return st;
  if (partition_size == 0) return PAD_ERR_PARTITION;
  if (dims->num_seqs == 0) return PAD_OK;
  pad::Plan plan = make_plan(scale, num_kv_heads, partition_size, dims);
  if (!attach_workspace(&plan, workspace, workspace_bytes)) return PAD_ERR_WORKSPACE;
  return status_of(pad::launch_phase1(plan, query, key_cache, value_cache, block_tables, seq_lens,
                                      static_cast<hipStream_t>(stream)));
}

int32_t paged_attention_decode_phase2(float* out, const int32_t* seq_lens, int32_t num_kv_heads,
                                      int32_t block_size, int32_t partition_size, const void* workspace,
                                      size_t workspace_bytes, const pad_dims_t* dims, void* stream) {
  if (!dims) return PAD_ERR_NULL;
  if (dims->dtype != PAD_DTYPE_F32 && dims->dtype != PAD_DTYPE_BF16) return PAD_ERR_DTYPE;
  if (dims->num_seqs < 0 || dims->num_heads <= 0 || dims->max_blocks_per_seq <= 0 || num_kv_heads <= 0 ||
      dims->num_heads % num_kv_heads != 0)
    return PAD_ERR_SHAPE;
  if (dims->head_size != 64 && dims->head_size != 128 && dims->head_size != 256) return PAD_ERR_UNSUPPORTED;
  if (block_size != pad::kBlockTokens) return PAD_ERR_UNSUPPORTED;
  if (dims->num_seqs > 65535 || dims->num_heads > 65535) return PAD_ERR_UNSUPPORTED;
  if ((int64_t)dims->max_blocks_per_seq * block_size > INT32_MAX / 2) return PAD_ERR_UNSUPPORTED;
  if (partition_size <= 0 || partition_size % block_size) return PAD_ERR_PARTITION;
  if (dims->out_seq_stride != 0 && dims->out_seq_stride < (int64_t)dims->num_heads * dims->head_size)
    return PAD_ERR_SHAPE;
  if ((dims->out_seq_stride * 4) % 16) return PAD_ERR_ALIGN;
  if (dims->num_seqs == 0) return PAD_OK;
  if (!out || !seq_lens) return PAD_ERR_NULL;
  if (!aligned16(out) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u)) return PAD_ERR_ALIGN;
  // the same plan phase 1 made (it decides which partitions became chunk entries)
  pad::Plan plan = make_plan(1.0f, num_kv_heads, partition_size, dims);
  if (!attach_workspace(&plan, const_cast<void*>(workspace), workspace_bytes)) return PAD_ERR_WORKSPACE;
  return status_of(pad::launch_phase2(plan, out, seq_lens, static_cast<hipStream_t>(stream)));
}

int32_t paged_attention_decode(float* out, const void* query, const void* key_cache, const void* value_cache,
                               const int32_t* block_tables, const int32_t* seq_lens, float scale,
                               int32_t num_kv_heads, int32_t block_size, int32_t partition_size, void* workspace,
                               size_t workspace_bytes, const pad_dims_t* dims, void* stream) {
  int32_t st = validate(query, key_cache, value_cache, block_tables, seq_lens, scale, num_kv_heads, block_size,
                        partition_size, dims);
  if (st != PAD_OK) return st;
  if (dims->num_seqs == 0) return PAD_OK;
  if (!out) return PAD_ERR_NULL;
  if (!aligned16(out)) return PAD_ERR_ALIGN;
  pad::Plan plan = make_plan(scale, num_kv_heads, partition_size, dims);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (partition_size == 0)
    return status_of(pad::launch_one_pass(plan, out, query, key_cache, value_cache, block_tables, seq_lens, s));
  if (!attach_workspace(&plan, workspace, workspace_bytes)) return PAD_ERR_WORKSPACE;
  hipError_t e = pad::launch_phase1(plan, query, key_cache, value_cache, block_tables, seq_lens, s);
  if (e != hipSuccess) return status_of(e);
  return status_of(pad::launch_phase2(plan, out, seq_lens, s));
}

int32_t paged_attention_decode_no_alloc(float* out, const void* query, const void* key_cache,
                                        const void* value_cache, const int32_t* block_tables,
                                        const int32_t* seq_lens, float scale, int32_t num_kv_heads,
                                        int32_t block_size, int32_t partition_size, const pad_dims_t* dims,
                                        void* stream) {
  int32_t st = validate(query, key_cache, value_cache, block_tables, seq_lens, scale, num_kv_heads, block_size,
                        partition_size, dims);
  if (st != PAD_OK) return st;
  if (dims->num_seqs == 0) return PAD_OK;
  if (!out) return PAD_ERR_NULL;
  if (!aligned16(out)) return PAD_ERR_ALIGN;
  pad::Plan plan = make_plan(scale, num_kv_heads, partition_size, dims);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (partition_size == 0)
    return status_of(pad::launch_one_pass(plan, out, query, key_cache, value_cache, block_tables, seq_lens, s));
  Layout l;
  if (!workspace_layout(dims->num_seqs, dims->num_heads, dims->head_size, dims->max_blocks_per_seq, block_size,
                        partition_size, &l))
    return PAD_ERR_SHAPE;
  if (l.total > pad::kStaticWorkspaceBytes) return PAD_ERR_TOO_LARGE;
  void* ws = nullptr;
  hipError_t e = pad::static_workspace(&ws);
  if (e != hipSuccess) return status_of(e);
  if (!attach_workspace(&plan, ws, pad::kStaticWorkspaceBytes)) return PAD_ERR_WORKSPACE;
  e = pad::launch_phase1(plan, query, key_cache, value_cache, block_tables, seq_lens, s);
  if (e != hipSuccess) return status_of(e);
  return status_of(pad::launch_phase2(plan, out, seq_lens, s));
}

int32_t paged_attention_prefill(float* out, const void* query, const void* key_cache, const void* value_cache,
                                const int32_t* block_tables, const int32_t* query_start,
                                const int32_t* context_lens, float scale, int32_t num_kv_heads,
                                int32_t block_size, const pad_prefill_dims_t* dims, void* stream) {
  int32_t st = validate_prefill(dims, num_kv_heads, block_size, true);
  if (st != PAD_OK) return st;
  if (!std::isfinite(scale)) return PAD_ERR_SHAPE;
  if (dims->num_seqs == 0 || dims->num_tokens == 0 || dims->max_query_len == 0) return PAD_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !query_start || !context_lens)
    return PAD_ERR_NULL;
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) ||
      !aligned4(block_tables) || !aligned4(query_start) || !aligned4(context_lens))
    return PAD_ERR_ALIGN;
  pad::PrefillArgs a{};
  a.out = out;
  a.query = static_cast<const char*>(query);
  a.key_cache = static_cast<const char*>(key_cache);
  a.value_cache = static_cast<const char*>(value_cache);
  a.block_tables = block_tables;
  a.query_start = query_start;
  a.context_lens = context_lens;
  a.qscale = scale;
  a.num_tokens = dims->num_tokens;
  a.num_heads = dims->num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = dims->num_heads / num_kv_heads;
  a.max_blocks = dims->max_blocks_per_seq;
  a.num_blocks = dims->num_blocks;
  return status_of(pad::launch_prefill(a, dims->num_seqs, dims->max_query_len, dims->head_size,
                                       static_cast<hipStream_t>(stream)));
}

int32_t paged_attention_prefill_split_ranges(int32_t head_size, int32_t num_heads, int32_t num_kv_heads) {
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return PAD_ERR_SHAPE;
  if (head_size != 64 && head_size != 128 && head_size != 256) return PAD_ERR_UNSUPPORTED;
  return pad::prefill_split_ranges(head_size, num_heads / num_kv_heads);
}

size_t paged_attention_prefill_split_workspace_size(const pad_prefill_dims_t* dims, int32_t num_kv_heads,
                                                    int32_t num_ranges) {
  if (!dims || num_ranges <= 0 || num_kv_heads <= 0 || dims->num_seqs < 0 || dims->max_query_len < 0 ||
      dims->max_blocks_per_seq <= 0 || dims->num_heads <= 0 || dims->num_heads % num_kv_heads != 0 ||
      (dims->head_size != 64 && dims->head_size != 128 && dims->head_size != 256))
    return (size_t)-1;
  return pad::prefill_split_workspace_bytes(dims->num_seqs, num_kv_heads, dims->num_heads / num_kv_heads,
                                            dims->head_size, dims->max_query_len, dims->max_blocks_per_seq,
                                            num_ranges);
}

int32_t paged_attention_prefill_choose_split(const int32_t* context_lens, const int32_t* query_lens,
                                             int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                             int32_t head_size, int32_t num_ranges) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || num_ranges <= 0)
    return PAD_ERR_SHAPE;
  if (head_size != 64 && head_size != 128 && head_size != 256) return PAD_ERR_UNSUPPORTED;
  if (num_seqs == 0) return 0;
  if (!context_lens || !query_lens) return PAD_ERR_NULL;
  for (int s = 0; s < num_seqs; ++s)
    if (context_lens[s] < 0 || query_lens[s] < 0) return PAD_ERR_SHAPE;
  return pad::prefill_split_pays(context_lens, query_lens, num_seqs, num_kv_heads, num_heads / num_kv_heads,
                                 num_ranges) ? 1 : 0;
}

int32_t paged_attention_prefill_split(float* out, const void* query, const void* key_cache, const void* value_cache,
                                      const int32_t* block_tables, const int32_t* query_start,
                                      const int32_t* context_lens, float scale, int32_t num_kv_heads,
                                      int32_t block_size, const pad_prefill_dims_t* dims, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  int32_t st = validate_prefill(dims, num_kv_heads, block_size, true);
  if (st != PAD_OK) return st;
  if (!std::isfinite(scale)) return PAD_ERR_SHAPE;
  if (dims->num_seqs == 0 || dims->num_tokens == 0 || dims->max_query_len == 0) return PAD_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !query_start || !context_lens)
    return PAD_ERR_NULL;
  if (!workspace) return PAD_ERR_WORKSPACE;
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) ||
      !aligned16(workspace) || !aligned4(block_tables) || !aligned4(query_start) || !aligned4(context_lens))
    return PAD_ERR_ALIGN;
  const int group = dims->num_heads / num_kv_heads;
  const int ranges = pad::prefill_split_ranges(dims->head_size, group);
  // the walk kernel's grid is 32-bit
  const int hg = group / pad::prefill_heads_per_wg(group);
  if (pad::prefill_split_grid(dims->num_seqs, num_kv_heads, group, dims->max_query_len, dims->max_blocks_per_seq,
                              ranges) > INT32_MAX)
    return PAD_ERR_UNSUPPORTED;
  // the plan's 64-bit step count: S x KV heads x head groups x tiles x steps per tile
  const int tpw = pad::prefill_tokens_per_wg(group, true);
  const unsigned __int128 tiles = ((unsigned)dims->max_query_len + tpw - 1) / tpw;
  const unsigned __int128 steps = ((unsigned __int128)dims->max_blocks_per_seq * block_size + 31) / 32;
  if ((unsigned __int128)dims->num_seqs * num_kv_heads * hg * tiles * steps >> 62) return PAD_ERR_UNSUPPORTED;
  if ((size_t)workspace_bytes < pad::prefill_split_workspace_bytes(dims->num_seqs, num_kv_heads, group,
                                                                   dims->head_size, dims->max_query_len,
                                                                   dims->max_blocks_per_seq, ranges))
    return PAD_ERR_WORKSPACE;
  pad::PrefillArgs a{};
  a.out = out;
  a.query = static_cast<const char*>(query);
  a.key_cache = static_cast<const char*>(key_cache);
  a.value_cache = static_cast<const char*>(value_cache);
  a.block_tables = block_tables;
  a.query_start = query_start;
  a.context_lens = context_lens;
  a.qscale = scale;
  a.num_tokens = dims->num_tokens;
  a.num_heads = dims->num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.max_blocks = dims->max_blocks_per_seq;
  a.num_blocks = dims->num_blocks;
  return status_of(pad::launch_prefill_split(a, dims->num_seqs, dims->max_query_len, dims->head_size, ranges,
                                             workspace, static_cast<hipStream_t>(stream)));
}

int32_t paged_attention_prefill_write_kv(void* key_cache, void* value_cache, const void* key, const void* value,
                                         const int32_t* block_tables, const int32_t* query_start,
                                         const int32_t* context_lens, int32_t num_kv_heads,
                                         int32_t block_size, const pad_prefill_dims_t* dims, void* stream) {
  int32_t st = validate_prefill(dims, num_kv_heads, block_size, false);
  if (st != PAD_OK) return st;
  if (dims->num_seqs == 0 || dims->num_tokens == 0 || dims->max_query_len == 0) return PAD_OK;
  if (!key_cache || !value_cache || !key || !value || !block_tables || !query_start || !context_lens)
    return PAD_ERR_NULL;
  if (!aligned16(key_cache) || !aligned16(value_cache) || !aligned16(key) || !aligned16(value) ||
      !aligned4(block_tables) || !aligned4(query_start) || !aligned4(context_lens))
    return PAD_ERR_ALIGN;
  pad::WriteKvArgs a{};
  a.key_cache = static_cast<char*>(key_cache);
  a.value_cache = static_cast<char*>(value_cache);
  a.key = static_cast<const char*>(key);
  a.value = static_cast<const char*>(value);
  a.block_tables = block_tables;
  a.query_start = query_start;
  a.context_lens = context_lens;
  a.num_tokens = dims->num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.head_size = dims->head_size;
  a.max_blocks = dims->max_blocks_per_seq;
  a.num_blocks = dims->num_blocks;
  const int eb = dims->dtype == PAD_DTYPE_BF16 ? 2 : 4;
  return status_of(pad::launch_write_kv(a, dims->num_seqs, dims->max_query_len, eb, dims->kv_layout,
                                        static_cast<hipStream_t>(stream)));
}

namespace {

// Constants of the batch rule below, fitted on MI355X (256 compute units; 24
// query / 4 KV heads, head 256, bf16; batches of 64 and 256 sequences of
// 1024 or 4096 tokens with one sequence 1-16 times as long):
constexpr double kBatchBytesPerSec = 6.5e12;  // one-pass over a batch of equal lengths
constexpr double kWalkBytesPerSec1 = 21e9;    // one one-wave workgroup walking its context alone
constexpr double kWalkBytesPerSec4 = 55e9;    // one four-wave workgroup walking alone
constexpr double kSplitFixedSec = 30e-6;      // what the split costs beyond one-pass on equal lengths:
constexpr double kSplitShare = 0.06;          // a fixed part and a share of the step

// The largest partition size in {2048, ..., 128} whose slots let the
// balanced split launch its full width on the longest sequence, whatever the
// layout and head size (up to kBalancedWgsPerCuMax workgroups per compute
// unit): N nb_max <= (NP - 1) B with N = 4 num_cus ranges, nb_max = max_ctx /
// 16 and B = total / 16 x the workgroups per sequence.  128 when none does.
// (Smaller sizes cost workspace: S x H x NP entries.)
int32_t partition_for_lengths(int64_t max_ctx, int64_t total, int64_t wgs_per_seq, int32_t num_cus) {
  static const int32_t kSizes[] = {2048, 1024, 512, 256, 128};
  for (int32_t p : kSizes) {
    const int64_t np = (max_ctx + p - 1) / p;
    if (np >= 2 && (np - 1) * total * wgs_per_seq >= (int64_t)pad::kBalancedWgsPerCuMax * num_cus * max_ctx)
      return p;
  }
  return 128;
}

}  // namespace

int32_t paged_attention_decode_choose_partition(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                                int32_t max_context_len, int32_t block_size, int32_t num_cus) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads || max_context_len < 0 ||
      num_cus <= 0)
    return PAD_ERR_SHAPE;
  if (block_size != pad::kBlockTokens) return PAD_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_context_len == 0) return 0;
  const int64_t group = num_heads / num_kv_heads;
  const int64_t chunks = (group + pad::kMaxHeadsPerGroup - 1) / pad::kMaxHeadsPerGroup;
  const int64_t wg_one_pass = (int64_t)num_seqs * num_kv_heads * chunks;
  // Fitted by timing sweeps on 256 compute units (24 q / 4 KV heads, head
  // 256, bf16): the one-pass form wins once the batch alone gives every
  // compute unit a workgroup (it also saves the workspace round trip), and
  // for contexts of one partition or less.  Otherwise phase 1 runs the
  // balanced split, and the partition size only sets how many slots a head
  // has: the largest size that leaves the split its full width was the
  // fastest or within 1 % of it (batch 1-16, context 2048-100K).
  if (wg_one_pass >= num_cus || max_context_len <= 512) return 0;
  return partition_for_lengths(max_context_len, (int64_t)num_seqs * max_context_len, num_kv_heads * chunks, num_cus);
}

int32_t paged_attention_decode_choose_partition_for_batch(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                                          int32_t head_size, int32_t dtype,
                                                          int32_t max_context_len, int64_t total_context_len,
                                                          int32_t block_size, int32_t num_cus) {
  const int32_t base = paged_attention_decode_choose_partition(num_seqs, num_heads, num_kv_heads, max_context_len,
                                                               block_size, num_cus);
  if (base < 0) return base;
  if (head_size != 64 && head_size != 128 && head_size != 256) return PAD_ERR_UNSUPPORTED;
  if (dtype != PAD_DTYPE_F32 && dtype != PAD_DTYPE_BF16) return PAD_ERR_DTYPE;
  if (total_context_len < max_context_len || total_context_len > (int64_t)num_seqs * max_context_len)
    return PAD_ERR_SHAPE;
  if (num_seqs == 0 || max_context_len == 0) return 0;
  const int64_t group = num_heads / num_kv_heads;
  const int64_t chunks = (group + pad::kMaxHeadsPerGroup - 1) / pad::kMaxHeadsPerGroup;
  const int64_t wgs_per_seq = (int64_t)num_kv_heads * chunks;
  if (num_seqs > pad::kBalancedMaxSeqs) return base;  // no balanced split: the fixed rule
  if (base > 0) return partition_for_lengths(max_context_len, total_context_len, wgs_per_seq, num_cus);
  if (max_context_len <= 512) return 0;
  // One-pass: the step lasts at least until the workgroup of the longest
  // sequence has walked the tokens it has beyond the others, mostly alone at
  // the end.  The split shares those tokens among all workgroups for a fixed
  // cost; it is chosen when the one-pass tail is larger.
  const double bytes_per_token = 2.0 * head_size * (dtype == PAD_DTYPE_BF16 ? 2 : 4);
  const int64_t wgs = (int64_t)num_seqs * wgs_per_seq;
  const double walk = wgs >= 4 * (int64_t)num_cus ? kWalkBytesPerSec1 : kWalkBytesPerSec4;
  const double mean = (double)total_context_len / num_seqs;
  const double tail = (max_context_len - mean) * bytes_per_token / walk;
  const double step = (double)total_context_len * num_kv_heads * bytes_per_token / kBatchBytesPerSec;
  if (tail <= kSplitFixedSec + kSplitShare * step) return 0;
  return partition_for_lengths(max_context_len, total_context_len, wgs_per_seq, num_cus);
}

int32_t paged_attention_decode_entry_ranges(const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                                            int32_t num_kv_heads, int32_t head_size, int32_t dtype,
                                            int32_t max_blocks_per_seq, int32_t block_size, int32_t partition_size,
                                            int32_t kv_layout, int32_t num_cus, int32_t* entry_count,
                                            int32_t* entry_begin, int32_t* entry_end) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads || max_blocks_per_seq <= 0 ||
      num_cus <= 0)
    return PAD_ERR_SHAPE;
  if (kv_layout != PAD_KV_ROWS && kv_layout != PAD_KV_TILED) return PAD_ERR_UNSUPPORTED;
  if (dtype != PAD_DTYPE_F32 && dtype != PAD_DTYPE_BF16) return PAD_ERR_DTYPE;
  if (head_size != 64 && head_size != 128 && head_size != 256) return PAD_ERR_UNSUPPORTED;
  if (block_size != pad::kBlockTokens) return PAD_ERR_UNSUPPORTED;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX / 2) return PAD_ERR_UNSUPPORTED;
  if (partition_size <= 0 || partition_size % block_size) return PAD_ERR_PARTITION;
  if (num_seqs == 0) return 0;
  if (!seq_lens || !entry_count || !entry_begin || !entry_end) return PAD_ERR_NULL;
  const int64_t S = num_seqs, H = num_heads;
  const int group = num_heads / num_kv_heads;
  const int chunks = (group + pad::kMaxHeadsPerGroup - 1) / pad::kMaxHeadsPerGroup;
  const int64_t gyc = (int64_t)num_kv_heads * chunks;
  const int64_t maxtok = (int64_t)max_blocks_per_seq * block_size;
  const int64_t np = (maxtok + partition_size - 1) / partition_size;
  const bool bal = pad::balanced_split(S, gyc, np, max_blocks_per_seq, num_cus);
  // live blocks per sequence and their prefix, as phase 1 derives them
  std::vector<uint64_t> pre(S + 1, 0);
  uint64_t nb_max = 0;
  for (int64_t s = 0; s < S; ++s) {
    const int64_t L = seq_lens[s];
    const uint64_t nb = (L > 0 && L <= maxtok) ? (uint64_t)((L + block_size - 1) / block_size) : 0;
    nb_max = nb > nb_max ? nb : nb_max;
    pre[s + 1] = pre[s] + nb;
  }
  const uint64_t B = pre[S] * (uint64_t)gyc;
  const uint64_t N = bal ? pad::balanced_ranges(B, nb_max,
                                                (unsigned)(pad::balanced_wgs_per_cu(kv_layout, head_size,
                                                                                    dtype == PAD_DTYPE_F32 ? 4 : 2) *
                                                           num_cus),
                                                (unsigned)np, (unsigned)num_cus)
                         : 0;
  for (int64_t s = 0; s < S; ++s) {
    const int64_t L = seq_lens[s];
    for (int64_t h = 0; h < H; ++h) {
      int32_t* cnt = entry_count + s * H + h;
      int32_t* lo = entry_begin + (s * H + h) * np;
      int32_t* hi = entry_end + (s * H + h) * np;
      if (L == 0 || L < 0 || L > maxtok) {
        *cnt = L == 0 ? 0 : -1;
        continue;
      }
      if (!bal) {
        const int64_t n = (L + partition_size - 1) / partition_size;
        *cnt = (int32_t)n;
        for (int64_t e = 0; e < n; ++e) {
          lo[e] = (int32_t)(e * partition_size);
          hi[e] = (int32_t)std::min<int64_t>((e + 1) * partition_size, L);
        }
        continue;
      }
      const int64_t g = h / group;
      const int64_t gy = g * chunks + (h - g * group) / pad::kMaxHeadsPerGroup;
      const uint64_t nb = pre[s + 1] - pre[s];
      const uint64_t g0 = (uint64_t)gyc * pre[s] + (uint64_t)gy * nb;
      const uint64_t j0 = pad::range_owner(g0, N, B), j1 = pad::range_owner(g0 + nb - 1, N, B);
      *cnt = (int32_t)(j1 - j0 + 1);
      for (uint64_t j = j0; j <= j1; ++j) {
        const uint64_t a = std::max<uint64_t>(j * B / N, g0) - g0;
        const uint64_t b = std::min<uint64_t>((j + 1) * B / N, g0 + nb) - g0;
        lo[j - j0] = (int32_t)(a * block_size);
        hi[j - j0] = (int32_t)std::min<int64_t>((int64_t)b * block_size, L);
      }
    }
  }
  return bal ? 1 : 0;
}

#ifndef PAD_SOURCE_HASH
#define PAD_SOURCE_HASH "unknown"
#endif

const char* paged_attention_decode_build_id(void) { return PAD_SOURCE_HASH; }

const char* paged_attention_decode_strerror(int32_t status) {
  switch (status) {
    case PAD_OK: return "success";
    case PAD_ERR_NULL: return "a required pointer is NULL";
    case PAD_ERR_DTYPE: return "dtype must be PAD_DTYPE_F32 or PAD_DTYPE_BF16 and kv_layout PAD_KV_ROWS or PAD_KV_TILED";
    case PAD_ERR_SHAPE: return "invalid sizes: need num_seqs >= 0, num_heads, num_kv_heads, num_blocks, max_blocks_per_seq >= 1, num_heads % num_kv_heads == 0, finite scale";
    case PAD_ERR_UNSUPPORTED: return "unsupported shape: head_size must be 64, 128 or 256 and block_size 16 (the prefill attention also needs bf16 and the tiled layout), or a size limit is exceeded";
    case PAD_ERR_PARTITION: return "partition_size must be >= 0 and a multiple of block_size (> 0 for phase calls)";
    case PAD_ERR_WORKSPACE: return "workspace is NULL, misaligned or smaller than paged_attention_decode_workspace_size()";
    case PAD_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case PAD_ERR_TOO_LARGE: return "the split call needs more workspace than the library's 64 MiB static workspace holds (paged_attention_decode_no_alloc); pass a workspace to paged_attention_decode instead";
    default: break;
  }
  if (status > 0) return hipGetErrorString(static_cast<hipError_t>(status));
  return "unknown status";
}

}  // extern "C"
