/*
 * paged_attention_decode.h - C ABI of the MI355X (gfx950) paged decode-attention library.
 *
 * Operation (second page, "V2 implementation" message; first page, two-pass
 * message): for every sequence s and query head h, one new query row attends
 * over the sequence's cached keys and values, which live in a pool of
 * fixed-size blocks addressed through a per-sequence block table:
 *
 *     x_t      = scale * <query[s,h,:], K_s[g(h), t, :]>      for t < seq_lens[s]
 *     out[s,h] = sum_t exp(x_t - max x) V_s[g(h), t, :] / sum_t exp(x_t - max x)
 *
 * with g(h) = h / (num_heads / num_kv_heads) (query heads grouped contiguously
 * per KV head) and K_s[g, t, :] = key_cache[block_tables[s, t / block_size], g,
 * t % block_size, :] (likewise V).
 *
 * The split form computes this in two passes.  Phase 1 runs one workgroup per
 * (sequence, KV head, partition of partition_size tokens) and stores, for each
 * query head of the group, the partition's max logit, its exp-sum and its
 * normalised partial output.  Phase 2 merges the partitions by log-sum-exp:
 * weight_p = exp_sum_p * exp(max_p - max over p), out = sum_p weight_p *
 * partial_p / sum_p weight_p.  partition_size == 0 selects the one-pass path,
 * which walks the whole context in one workgroup per (sequence, KV head) with
 * an online softmax and needs no workspace.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers named as device pointers must be device memory of the current HIP
 * device (e.g. torch CUDA tensors), 16-byte aligned, contiguous except for the
 * sequence strides of query and out (pad_dims_t).  Layouts (row-major,
 * innermost last):
 *   out          float32 [num_seqs, num_heads, head_size] (sequence stride out_seq_stride)
 *   query        dtype   [num_seqs, num_heads, head_size] (sequence stride query_seq_stride)
 *   key_cache    dtype   PAD_KV_ROWS:  [num_blocks, num_kv_heads, block_size, head_size]
 *                        PAD_KV_TILED: [num_blocks, num_kv_heads, head_size/x, block_size, x]
 *                                      with x = 16 bytes of elements (8 bf16, 4 fp32)
 *   value_cache  dtype   PAD_KV_ROWS:  [num_blocks, num_kv_heads, block_size, head_size]
 *                        PAD_KV_TILED: [num_blocks, num_kv_heads, head_size, block_size]
 *   block_tables int32   [num_seqs, max_blocks_per_seq]
 *   seq_lens     int32   [num_seqs]
 * The second page's hardware-test message lists both layouts: the 4-D
 * token-row layout for K and V of its split kernel, and the 5-D x-split K
 * with the dims-by-tokens V of its one-pass kernel.  In both, each (block, KV
 * head) tile is block_size * head_size contiguous elements.  PAD_KV_TILED is
 * the faster one here: every K and V load feeds a matrix-core instruction
 * directly, so P.V runs on the matrix cores as well as Q.K^T.
 *
 * Ownership: every buffer belongs to the caller.  The library allocates no
 * memory and keeps no per-call state outside the workspace (it caches each
 * device's compute-unit count); calls only enqueue kernels on `stream`
 * (a hipStream_t; NULL = the null stream) and return without synchronising.
 * Buffers must stay valid until that work completes.  One workspace must not
 * be used by two calls whose work may overlap.
 *
 * Errors: 0 = success.  A negative status is an argument error found on the
 * host before any HIP call: nothing is enqueued and no buffer is touched.  A
 * positive status is the hipError_t of a failed launch.  No function throws.
 *
 * Device-side contract (not checkable without a synchronisation): 0 <=
 * seq_lens[s] <= max_blocks_per_seq * block_size, and block_tables[s, j] lies in
 * [0, num_blocks) for j < ceil(seq_lens[s] / block_size); other table entries
 * are never read.  A violation does not fault: a length outside the range or a
 * block id outside the pool makes that sequence's output rows NaN.
 */
#ifndef PAGED_ATTENTION_DECODE_H
#define PAGED_ATTENTION_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types of query, key_cache and value_cache */
#define PAD_DTYPE_F32 0
#define PAD_DTYPE_BF16 1

/* KV cache layouts (see "Conventions") */
#define PAD_KV_ROWS 0
#define PAD_KV_TILED 1

/* status codes */
#define PAD_OK 0
#define PAD_ERR_NULL (-1)        /* a required pointer is NULL */
#define PAD_ERR_DTYPE (-2)       /* dtype is neither PAD_DTYPE_F32 nor PAD_DTYPE_BF16, or kv_layout unknown */
#define PAD_ERR_SHAPE (-3)       /* a size is out of range or sizes disagree (e.g. num_heads % num_kv_heads != 0) */
#define PAD_ERR_UNSUPPORTED (-4) /* head_size not 64/128/256, or block_size not 16 */
#define PAD_ERR_PARTITION (-5)   /* partition_size negative or not a multiple of block_size */
#define PAD_ERR_WORKSPACE (-6)   /* split call with a NULL or too small workspace */
#define PAD_ERR_ALIGN (-7)       /* a device pointer is not 16-byte aligned */
#define PAD_ERR_TOO_LARGE (-8)   /* paged_attention_decode_no_alloc: workspace beyond its 64 MiB */

/*
 * Problem sizes shared by the entry points.
 *   dtype              PAD_DTYPE_F32 | PAD_DTYPE_BF16 (query, key_cache, value_cache)
 *   num_seqs           S >= 0 (0 makes every call a no-op)
 *   num_heads          H >= 1, a multiple of num_kv_heads
 *   head_size          D in {64, 128, 256}
 *   num_blocks         physical blocks in the KV pool, >= 1
 *   max_blocks_per_seq W >= 1, the block-table row width
 *   kv_layout          PAD_KV_ROWS | PAD_KV_TILED (key_cache and value_cache)
 *   query_seq_stride   elements from sequence s's query rows to sequence s+1's;
 *                      0 = num_heads * head_size (contiguous).  Within a sequence
 *                      the [num_heads, head_size] rows are contiguous.  Lets
 *                      query be a view of a wider buffer, e.g. the query part
 *                      of a fused QKV projection [S, (H + 2 Hkv) * D].  Must be
 *                      0 or >= num_heads * head_size, and a multiple of 16 bytes.
 *   out_seq_stride     likewise for out (float32 elements), e.g. a slice of a
 *                      wider activation buffer; 0 = contiguous.
 */
typedef struct pad_dims {
  int32_t dtype;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t head_size;
  int64_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t kv_layout;
  int64_t query_seq_stride;
  int64_t out_seq_stride;
} pad_dims_t;

/*
 * Decode attention for one new token per sequence (both phases, or the
 * one-pass path), written to `out` (float32).
 *   scale          multiplies every query-key dot product (usually 1/sqrt(D)); finite
 *   num_kv_heads   KV heads in the pool (>= 1, divides num_heads)
 *   block_size     tokens per block; must be 16
 *   partition_size 0 = one-pass; else tokens per partition, a multiple of block_size
 *   workspace      device buffer of >= paged_attention_decode_workspace_size(...)
 *                  bytes, used only when partition_size > 0 (may be NULL otherwise).
 *                  Its contents need no initialisation: phase 1 writes every
 *                  entry and record phase 2 reads, and reads nothing from it.
 *                  (paged_attention_decode_workspace_init sets the defined
 *                  starting values the pages' workspace message gives.)
 * Sequences with seq_lens[s] == 0 get all-zero output rows.
 */
int32_t paged_attention_decode(float* out, const void* query, const void* key_cache,
                               const void* value_cache, const int32_t* block_tables,
                               const int32_t* seq_lens, float scale, int32_t num_kv_heads,
                               int32_t block_size, int32_t partition_size, void* workspace,
                               size_t workspace_bytes, const pad_dims_t* dims, void* stream);

/*
 * paged_attention_decode without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * split path's workspace is the library's own static device array of 64 MiB
 * (kept by every GPU the library runs on until the process ends; its address
 * is looked up once per device).  Arguments, results and errors are those of
 * paged_attention_decode, plus PAD_ERR_TOO_LARGE (nothing enqueued) when
 * paged_attention_decode_workspace_size(...) of this call exceeds 64 MiB
 * (e.g. 24 heads x 256 dims: S x NP up to about 2 700 partition slots).  Every
 * call on one GPU shares that array: calls whose work may overlap on one GPU
 * (two streams, two threads) race and must not be made.  Nothing in the array
 * has to start at zero: phase 1 writes every value phase 2 reads.
 */
int32_t paged_attention_decode_no_alloc(float* out, const void* query, const void* key_cache,
                                        const void* value_cache, const int32_t* block_tables,
                                        const int32_t* seq_lens, float scale, int32_t num_kv_heads,
                                        int32_t block_size, int32_t partition_size, const pad_dims_t* dims,
                                        void* stream);

/*
 * Phase 1 alone (partition_size > 0): per (sequence, KV head, partition)
 * workgroup, the partition's max logit, exp-sum and normalised partial output
 * for each query head of the group, written into `workspace`.  Arguments as in
 * paged_attention_decode.  Partitions at or beyond ceil(seq_lens[s] /
 * partition_size) are left untouched.
 *
 * Load balance (the balanced split).  When one workgroup per partition
 * would give more workgroups than the GPU has compute units, and there are at
 * most 1024 sequences and at least two partition slots per head, phase 1
 * does not use fixed partition_size-token partitions.  It lays the live
 * (KV block, head group) pairs of all sequences end to end -- sequence by
 * sequence, head group by head group, block by block; a sequence with length
 * 0 or outside [0, max_blocks_per_seq * block_size] has none -- and cuts
 * them into N equal contiguous ranges, one per workgroup of a grid that is
 * resident all at once (2 per compute unit for the tiled layout at head
 * size 256 in bf16, 3 there in fp32, 4 below head size 256, 3 for the rows
 * layout; N capped so that no head gets
 * more entries than it has partition slots, and so that a range holds at
 * least 8 blocks).  Each entry then covers a contiguous run of whole blocks
 * (the last one cut at seq_lens[s]) instead of partition e's tokens
 * [e * partition_size, (e + 1) * partition_size); a head's entries still
 * fill its slots 0, 1, ... in token order, and never more than
 * ceil(max_blocks_per_seq * block_size / partition_size) of them.
 * paged_attention_decode_entry_ranges reports, from a host copy of
 * seq_lens, which slots hold which tokens in either case.  Phase 1 reads
 * nothing from the workspace; it writes the entries and, for the balanced
 * split, a small launch record (N, the number of live pairs and the
 * per-sequence block prefix) that phase 2 reads to find each head's entries.
 */
int32_t paged_attention_decode_phase1(const void* query, const void* key_cache,
                                      const void* value_cache, const int32_t* block_tables,
                                      const int32_t* seq_lens, float scale, int32_t num_kv_heads,
                                      int32_t block_size, int32_t partition_size, void* workspace,
                                      size_t workspace_bytes, const pad_dims_t* dims, void* stream);

/*
 * Phase 2 alone: log-sum-exp merge of each (sequence, head)'s phase-1
 * entries in `workspace` into `out`: the first ceil(seq_lens[s] /
 * partition_size) slots, or under the balanced split the slots its launch
 * record names.  Reads only entries phase 1 wrote for the same seq_lens.
 * num_kv_heads, block_size, partition_size and dims must be those of the
 * phase-1 call, on the same device: they determine where phase 1 put each
 * result.  A balanced-split launch record that does not match this call's
 * seq_lens (phase 1 not run, or run with other lengths or sizes) makes the
 * affected rows NaN.
 */
int32_t paged_attention_decode_phase2(float* out, const int32_t* seq_lens, int32_t num_kv_heads,
                                      int32_t block_size, int32_t partition_size,
                                      const void* workspace, size_t workspace_bytes,
                                      const pad_dims_t* dims, void* stream);

/*
 * Bytes of workspace a split call needs: three float32 arrays, each starting on
 * a 256-byte boundary,
 *   max_logits [S, H, NP] | exp_sums [S, H, NP] | tmp_output [S, H, NP, D]
 * with NP = ceil(max_blocks_per_seq * block_size / partition_size), the most
 * partitions any sequence can have (the pages' tmp_output, exp_sums and
 * max_logits, second page, workspace-initialisation message), followed by the
 * balanced split's launch record: 4352 bytes (1029 uint32 words).
 * Returns 0 when partition_size == 0 and (size_t)-1 for invalid arguments.
 */
size_t paged_attention_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_size,
                                             int32_t max_blocks_per_seq, int32_t block_size,
                                             int32_t partition_size);

/* Byte offsets of the three workspace arrays (same arguments); each may be NULL. */
int32_t paged_attention_decode_workspace_layout(int32_t num_seqs, int32_t num_heads,
                                                int32_t head_size, int32_t max_blocks_per_seq,
                                                int32_t block_size, int32_t partition_size,
                                                size_t* max_logits_offset, size_t* exp_sums_offset,
                                                size_t* tmp_output_offset);

/*
 * Enqueue the workspace's defined starting contents on `stream`: max_logits =
 * -inf, exp_sums = 0, tmp_output = 0 (second page, workspace-initialisation
 * message) and the launch record = 0.  Done with a fill kernel, so the call
 * may be captured in a HIP graph.  Not needed for correct results: phase 1
 * reads nothing from the workspace.
 */
int32_t paged_attention_decode_workspace_init(void* workspace, size_t workspace_bytes,
                                              int32_t num_seqs, int32_t num_heads,
                                              int32_t head_size, int32_t max_blocks_per_seq,
                                              int32_t block_size, int32_t partition_size,
                                              void* stream);

/*
 * One-pass versus split choice for a batch of equal lengths, sized for a GPU
 * with `num_cus` compute units (256 on MI355X).  Returns 0 (one-pass) when
 * the batch's (sequence, KV head) workgroups already give every compute unit
 * one, or the context is at most 512 tokens.  Otherwise phase 1 runs the
 * balanced split, where the partition size only bounds the slots of a head:
 * this returns the largest size in {2048, 1024, 512, 256, 128} whose slots
 * let the split launch its full width (up to four workgroups per compute
 * unit, depending on the layout and head size),
 * (ceil(max_context_len / P) - 1) x num_seqs x workgroups per sequence >=
 * 4 x num_cus (else 128).  The first page's two-pass message weighs
 * partition count against workgroups per compute unit for a 16-unit GPU;
 * this rule redoes that for num_cus units, fitted by timing sweeps over
 * batch 1-256 and context 512-100K.  Negative status on invalid arguments.
 */
int32_t paged_attention_decode_choose_partition(int32_t num_seqs, int32_t num_heads,
                                                int32_t num_kv_heads, int32_t max_context_len,
                                                int32_t block_size, int32_t num_cus);

/*
 * The same choice for a batch whose lengths may differ, told also the head
 * size, the element type (PAD_DTYPE_*) and the batch's total context
 * (the sum of its sequence lengths, known to the caller on the host).  Where
 * paged_attention_decode_choose_partition picks one-pass because the batch
 * fills the compute units, one workgroup walks each (sequence, KV head)
 * alone, and the tokens the longest sequence has beyond the mean set the
 * step's end.  When that tail is longer than the split costs beyond
 * one-pass (about 30 us plus 6 % of the step on MI355X; measured on batches
 * of 64 and 256 with one sequence 1-16 times the others' length), this
 * returns a split partition size instead.  For any split it returns the
 * largest size in {2048, ..., 128} whose slots let the balanced split
 * launch its full width on the longest sequence:
 * (ceil(max_context_len / P) - 1) x total_context_len x workgroups per
 * sequence >= 4 x num_cus x max_context_len.  Batches above 1024 sequences get the fixed rule.  With
 * total_context_len = num_seqs * max_context_len (equal lengths) one-pass
 * choices are the fixed rule's.  Negative status on invalid arguments,
 * among them a total below the maximum or above num_seqs times it.
 */
int32_t paged_attention_decode_choose_partition_for_batch(int32_t num_seqs, int32_t num_heads,
                                                          int32_t num_kv_heads, int32_t head_size,
                                                          int32_t dtype, int32_t max_context_len,
                                                          int64_t total_context_len, int32_t block_size,
                                                          int32_t num_cus);

/*
 * Where phase 1 puts each (sequence, head)'s results, computed on the host
 * from a host copy of seq_lens, for heads of head_size, elements of dtype
 * (PAD_DTYPE_*) and a cache in kv_layout (PAD_KV_*: the balanced split
 * launches two workgroups per compute unit for the tiled layout at head size
 * 256 in bf16, three there in fp32, four below head size 256, and three for
 * the rows layout) on a device with num_cus compute units (the same rule
 * phase 1 applies on the device).  Arrays (row-major, host
 * memory, caller-owned):
 *   seq_lens     int32 [num_seqs]
 *   entry_count  int32 [num_seqs, num_heads]: entries of (s, h); 0 for
 *                seq_lens[s] == 0, -1 for a length outside the table (those
 *                rows are written without entries: zeros, NaN)
 *   entry_begin, entry_end  int32 [num_seqs, num_heads, NP]: token range
 *                [begin, end) of slot e < entry_count (other slots untouched)
 * with NP = ceil(max_blocks_per_seq * block_size / partition_size).  Returns
 * 1 when phase 1 runs the balanced split, 0 for one workgroup per partition
 * (slot e = tokens [e * partition_size, min((e + 1) * partition_size, L))),
 * or a negative status for invalid arguments.
 */
int32_t paged_attention_decode_entry_ranges(const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                                            int32_t num_kv_heads, int32_t head_size, int32_t dtype,
                                            int32_t max_blocks_per_seq, int32_t block_size,
                                            int32_t partition_size, int32_t kv_layout, int32_t num_cus,
                                            int32_t* entry_count, int32_t* entry_begin,
                                            int32_t* entry_end);

/*
 * The library's build id: the first 16 hex digits of a SHA-256 over the
 * names and contents of the source files (csrc/ and include/) it was built
 * from, fixed at build time (never NULL).  Lets a caller or a test check that
 * the loaded binary was built from the sources at hand.
 */
const char* paged_attention_decode_build_id(void);

/* Static text for a status code (never NULL). */
const char* paged_attention_decode_strerror(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTENTION_DECODE_H */
