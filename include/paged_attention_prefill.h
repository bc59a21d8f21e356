/*
 * paged_attention_prefill.h - C ABI of the MI355X (gfx950) paged prefix
 * (chunked prefill) attention, the step on the other side of decode.
 *
 * Operation (first page, prefill note; second page, the prefix-attention
 * allocator-reuse message and the rewrite that gathers the whole context's
 * K/V before attending): a sequence s already holds context_lens[s] tokens in
 * the paged KV cache and receives a chunk of n_s = query_start[s+1] -
 * query_start[s] new tokens.
 * Chunk token i sits at absolute position p = context_lens[s] + i and takes
 * softmax attention over the sequence's positions 0 .. p:
 *
 *     x_j      = scale * <query[t,h,:], K_s[g(h), j, :]>        j = 0 .. p
 *     out[t,h] = sum_j exp(x_j - max x) V_s[g(h), j, :] / sum_j exp(x_j - max x)
 *
 * with t = query_start[s] + i, g(h) = h / (num_heads / num_kv_heads), and
 * K_s[g, j, :] = key_cache[block_tables[s, j / block_size], g, j % block_size, :]
 * (likewise V).  The pages compute it as a K-tiled online softmax, the
 * context's tiles first and then the chunk's own tiles under the causal
 * mask.  Here the chunk's keys and values are first stored in the cache at
 * their positions (paged_attention_prefill_write_kv), after which the
 * attention reads every key through the block table in one walk with the same
 * running max and sum.
 *
 * Conventions are those of paged_attention_decode.h (device pointers of the
 * current HIP device, contiguous, 16-byte aligned; row-major; every buffer
 * belongs to the caller; calls only enqueue work on `stream`; 0 = success, a
 * negative status is an argument error found on the host before any HIP call,
 * a positive status the hipError_t of a failed launch).  Layouts:
 *   out          float32 [num_tokens, num_heads, head_size]
 *   query        dtype   [num_tokens, num_heads, head_size]: the chunk rows of
 *                        all sequences, sequence after sequence
 *   key, value   dtype   [num_tokens, num_kv_heads, head_size]: the chunk's own
 *                        keys and values (write_kv only)
 *   key_cache,   dtype   as in paged_attention_decode.h, PAD_KV_ROWS or PAD_KV_TILED
 *   value_cache
 *   block_tables int32   [num_seqs, max_blocks_per_seq]
 *   query_start  int32   [num_seqs + 1]: query_start[0] = 0, non-decreasing,
 *                        query_start[num_seqs] = num_tokens
 *   context_lens int32   [num_seqs]
 *
 * Device-side contract (not checkable without a synchronisation): the
 * query_start bounds above; n_s <= max_query_len; 0 <= context_lens[s] and
 * context_lens[s] + n_s <= max_blocks_per_seq * block_size; block_tables[s, j]
 * lies in [0, num_blocks) for j < ceil((context_lens[s] + n_s) / block_size).
 * A violation never faults: the attention writes NaN rows for that sequence
 * (only rows inside [0, num_tokens), and for n_s > max_query_len only the
 * first rows the launch grid covers, at least max_query_len of them), and the
 * chunk write skips a sequence with n_s > max_query_len entirely and tokens
 * whose slot would fall outside the table or the pool.
 */
#ifndef PAGED_ATTENTION_PREFILL_H
#define PAGED_ATTENTION_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#include "paged_attention_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Problem sizes of a prefill call.
 *   dtype              PAD_DTYPE_BF16 for the attention; PAD_DTYPE_F32 or
 *                      PAD_DTYPE_BF16 for the chunk write
 *   num_seqs           S >= 0 (0 makes every call a no-op)
 *   num_tokens         T >= 0, the packed chunk rows of all sequences
 *   num_heads          H >= 1, a multiple of num_kv_heads
 *   head_size          D in {64, 128, 256}
 *   max_query_len      >= every n_s (sizes the launch grid), >= 0
 *   num_blocks         physical blocks in the KV pool, >= 1
 *   max_blocks_per_seq W >= 1, the block-table row width
 *   kv_layout          PAD_KV_TILED for the attention; PAD_KV_ROWS or
 *                      PAD_KV_TILED for the chunk write
 */
typedef struct pad_prefill_dims {
  int32_t dtype;
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t num_heads;
  int32_t head_size;
  int32_t max_query_len;
  int64_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t kv_layout;
} pad_prefill_dims_t;

/*
 * Prefix attention of every chunk token over its sequence's cached positions
 * up to and including its own (the chunk's keys and values must already be
 * in the cache), written to `out` (float32).
 *   scale          multiplies every query-key dot product; finite
 *   num_kv_heads   KV heads in the pool (>= 1, divides num_heads)
 *   block_size     tokens per block; must be 16
 * Supported: bf16 query and cache in the PAD_KV_TILED layout (else
 * PAD_ERR_UNSUPPORTED).  Sequences with n_s == 0 produce no rows.
 * Accumulation is fp32.  The attention weights enter the P.V product as one
 * fp16 value each (relative rounding at most 2^-11; V is exact in fp16 down
 * to 2^-14 in magnitude, and below that within 2^-14 absolute); a
 * walk whose keys hold a V value beyond fp16's range (|v| > 65504, or
 * infinite, or NaN) is computed again with each weight as a bf16 hi + lo pair
 * (about 2^-16 relative).  The products are exact and accumulate in
 * fp32; the fp16 weights' rounding bounds the error by 2^-11 max |v| where
 * every rounding points one way.  Measured maximum error against an fp64
 * reference (bf16 normal inputs): 4.0e-4 over walks of at most 328 keys,
 * 1.4e-4 on a ragged 4-sequence batch, under 1e-5 on one 8192-token chunk
 * over 32768.
 */
int32_t paged_attention_prefill(float* out, const void* query, const void* key_cache, const void* value_cache,
                                const int32_t* block_tables, const int32_t* query_start,
                                const int32_t* context_lens, float scale, int32_t num_kv_heads,
                                int32_t block_size, const pad_prefill_dims_t* dims, void* stream);

/*
 * Split launch of the same prefix attention, for batches whose walks differ
 * in length.  It applies the first page's two-pass message (partitions of the
 * keys accumulated in parallel, then combined by log-sum-exp rescaling) and
 * its even-share note (about the same work for every workgroup) to the
 * prefill walks.  A walk is the key range of one workgroup's rows: one
 * sequence, one KV head's query heads (or a chunk of them), one tile of chunk
 * tokens, in 32-key steps up to the tile's last position.  Every walk longer
 * than C steps -- C = the launch's total steps over 4 N (N =
 * paged_attention_prefill_split_ranges()), at least 16 and at least the
 * longest walk over 32 -- is cut into ceil(steps / C) pieces of equal
 * length, which are served first (longest sequence first); the whole walks
 * follow.  No walk is cut when the longest is at most half of the total
 * steps over N (see paged_attention_prefill_choose_split).  Pieces leave
 * unnormalised rows in the workspace and a merge combines them.  Same
 * operation, arguments and contract as paged_attention_prefill, except:
 *   workspace        device memory of at least workspace_bytes bytes, 16-byte
 *                    aligned; contents on entry do not matter (every byte read
 *                    is written first by the same call); two calls in flight
 *                    must not share it
 *   workspace_bytes  >= paged_attention_prefill_split_workspace_size(dims,
 *                    num_kv_heads, N), else PAD_ERR_WORKSPACE
 * A sequence with n_s > max_query_len is out of contract here for any
 * excess: its first max_query_len rows (inside the output) are NaN.  Results
 * agree with paged_attention_prefill's to fp32 rounding (a cut walk's partial
 * sums are added in another order), not bit for bit; walks that are not cut
 * give the same bits.  PAD_ERR_UNSUPPORTED also for launches whose unit list
 * would pass 2^31 workgroups.  Enqueues three kernels on `stream`.
 */
int32_t paged_attention_prefill_split(float* out, const void* query, const void* key_cache, const void* value_cache,
                                      const int32_t* block_tables, const int32_t* query_start,
                                      const int32_t* context_lens, float scale, int32_t num_kv_heads,
                                      int32_t block_size, const pad_prefill_dims_t* dims, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * N for paged_attention_prefill_split on the current HIP device: its compute
 * units times the split walk kernel's resident workgroups per unit at this
 * head size.  PAD_ERR_SHAPE or PAD_ERR_UNSUPPORTED (negative) for sizes the
 * prefill attention rejects.
 */
int32_t paged_attention_prefill_split_ranges(int32_t head_size, int32_t num_heads, int32_t num_kv_heads);

/*
 * Which launch serves these lengths better: 1 for paged_attention_prefill_split
 * when more than one sequence has chunk tokens (its longest-first unit list
 * measured 0 to 40 % faster on ragged batches, and 3 % slower on one of the
 * twelve batches timed), or when some walk is longer than half of a resident
 * workgroup's fair share of the launch's steps (the split cuts it); 0 for
 * paged_attention_prefill otherwise (one sequence whose walks are all short:
 * the one-walk-per-workgroup launch measured 1 to 3 % faster there).
 * context_lens and query_lens are HOST arrays of num_seqs entries (>= 0);
 * num_ranges is N of this device (paged_attention_prefill_split_ranges).
 * Negative status for bad sizes.  Host-only; no HIP call.
 */
int32_t paged_attention_prefill_choose_split(const int32_t* context_lens, const int32_t* query_lens,
                                             int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                             int32_t head_size, int32_t num_ranges);

/*
 * Workspace bytes of paged_attention_prefill_split for these sizes (num_seqs,
 * num_heads, head_size, max_query_len and max_blocks_per_seq of dims) and
 * N = num_ranges: the unit list (at most W = num_seqs x num_kv_heads x
 * ceil(max_query_len / tokens per walk) walks, and fewer than
 * min(8 N / head chunks, k W) pieces, k = the pieces a walk of the block
 * table's width can be cut into: 0 below 512 positions, at most 32), and
 * partial slots of 256 rows x (head_size + 2) floats, one per piece and head
 * chunk.  (size_t)-1 for sizes out of range.  Host-only; no HIP call.
 */
size_t paged_attention_prefill_split_workspace_size(const pad_prefill_dims_t* dims, int32_t num_kv_heads,
                                                    int32_t num_ranges);

/*
 * Store the chunk's keys and values in the cache: row query_start[s] + i of
 * `key` / `value` goes to position context_lens[s] + i of sequence s, that
 * is to block block_tables[s, p / block_size], slot p % block_size, in the
 * cache layout dims->kv_layout.  Nothing else in the cache changes.
 *   num_kv_heads   KV heads (>= 1); block_size must be 16
 * dims->num_heads is not used (any value >= 1).
 */
int32_t paged_attention_prefill_write_kv(void* key_cache, void* value_cache, const void* key, const void* value,
                                         const int32_t* block_tables, const int32_t* query_start,
                                         const int32_t* context_lens, int32_t num_kv_heads,
                                         int32_t block_size, const pad_prefill_dims_t* dims, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTENTION_PREFILL_H */
