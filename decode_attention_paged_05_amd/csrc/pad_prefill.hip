// Prefix (chunked prefill) attention over the paged KV cache, and the chunk
// write that stores the chunk's keys and values in the cache, on CDNA4
// (gfx950).
//
// Operation (first page, prefill note; second page, prefix-attention
// messages): a sequence holds ctx tokens in the paged cache and receives a
// chunk of n new tokens; chunk token i sits at absolute position ctx + i and
// takes softmax attention over the sequence's positions 0 .. ctx + i.  The
// chunk's own keys and values are stored in the cache first (write_kv_kernel),
// so the attention reads every key through the block table and the causal rule
// is a comparison of absolute positions.  The pages' form walks the context
// tiles and then the chunk tiles with an online softmax; this kernel walks the
// same keys as one range, in 32-key steps, with the same running max / sum.
//
// Work decomposition.  A workgroup of 8 waves serves one (sequence, KV head,
// HC query heads of its group, a run of chunk tokens) in one of two layouts.
// Solo (every head size): 8 row groups of 32 query rows (32 consecutive chunk
// tokens of one head, as two 16-row column tiles), 256 / HC tokens; each wave
// holds its rows over all of D and forms both logit tiles of a step itself.
// Paired (head size 256, chosen per launch when the solo layout's larger
// workgroups would leave the compute units a long tail): four row groups,
// 128 / HC tokens, each owned by a pair of waves; the rest of this note
// describes the paired one, of which solo is the exchange-free case.  The
// workgroup walks the keys its
// last row can see in 32-key steps (two 16-token blocks).  Each wave of a
// pair forms the logits of half of the step's keys, over all of D, and
// leaves them in LDS for its partner; both then run the softmax over the whole
// step, and each accumulates the output for one half of D.  The logits are
// formed one step ahead, so the step barrier that every workgroup needs
// anyway also orders the exchange.  Each step's two K and two V tiles are
// copied from the pool into LDS by direct-to-LDS buffer loads (one wave of
// each pair a tile, 16 bytes per lane per load) into a ring of three step
// buffers, two steps ahead (issued after the wave's next-step logits, away
// from the waits the compiler places on its own loads); one barrier per
// step.  Each wave:
//   * forms its 16 x 32 tile of S^T = K Q^T for step st + 1 on
//     v_mfma_f32_16x16x32_bf16: A = K (rows = keys; lane l reads one key and 8
//     consecutive dims, one 16-byte LDS read of the tiled K layout), B = Q^T
//     (columns = query rows, in registers), contracting over D.  The keys are
//     dealt to tile rows so that lane group g ends up holding, over the two
//     tiles, the 8 consecutive keys 8 (g & 1) .. of block g >> 1;
//   * masks keys beyond each row's position (logit -inf by select) and updates
//     each row's running max (in-lane over 8 keys, then two lane swaps),
//     exp2-domain with a lazy reference: the accumulator is rescaled only when
//     a row's max grows by more than 2^8.  The scale enters through the exp2
//     argument (one FMA per logit); the launcher makes it positive;
//   * accumulates O^T += V^T P^T for its half of D on the same MFMA: A = V^T
//     (rows = dims; lane l reads dim l%16 and the same 8 keys, one 16-byte
//     LDS read of the tiled V layout, stored swizzled so that a lane group's
//     reads hit distinct banks), B = P^T (exactly the lane layout the logits
//     came out in).  p is split into bf16 hi + lo (two MFMAs), ~2^-16
//     relative precision.  Lane l holds output dims of row l%16, so the
//     softmax state and the rescale stay in the lane.
// Both layouts multiply P.V in fp16 instead (one MFMA, v_mfma_f32_16x16x32_f16):
// p rounded to fp16, V converted to fp16 in LDS once per step by the waves
// that copied it; a V value beyond fp16's range sends the walk to the bf16
// form above (walk_rows has the details).
// V elements at positions the walk does not hold are zeroed before the MFMA,
// so NaN padding never reaches a row.  Masking runs only on the steps that
// need it (the diagonal, the end of the walk), in separate code.  Workgroups
// are ordered so that those sharing K/V tiles share an XCD's L2
// (remap_workgroup).
//
// Two launches run this walk (walk_rows): prefill_kernel, one workgroup per
// walk; and the split launch (split_plan_kernel, split_walk_kernel,
// split_merge_kernel), which cuts walks much longer than the launch's
// average into pieces that run first and are combined by their log-sum-exp.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <algorithm>
#include <atomic>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "pad_lane_ops.h"
#include "pad_prefill_internal.h"

namespace pad {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) unsigned short u16x2_t;

constexpr int kWave = 64;
constexpr int kWaves = 8;          // waves per workgroup: 4 row groups x 2 halves of D
constexpr int kRowGroups = 4;      // 32-row groups per workgroup
constexpr int kRowsPerWave = 32;   // two 16-row column tiles
constexpr int kRsrcWord3 = 0x00020000;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.0f;  // headroom of the lazy softmax reference
constexpr float kNoKeysMax = -1e30f;  // reference max of a row that has seen no key
// fp16 P.V with a bf16 fallback (1), or the bf16 hi + lo pair only (0)
#ifndef PAD_PREFILL_F16_PV
#define PAD_PREFILL_F16_PV 1
#endif
// fp16 weights are formed against the reference less this (log2 units): with
// the lazy reference's 2^8 of headroom they lie in [0, 2^15]
constexpr float kF16Shift = 7.0f;

// s_waitcnt immediate: at most n vector-memory loads outstanding and every
// LDS access done (export counter left at its maximum)
constexpr int kWaitVmLds(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4); }

// N (1 to 4) copies of 16 bytes per lane from a buffer into LDS, 1 KB apart:
// copy j takes the bytes at voffset + 1024 j of the buffer and leaves lane i's
// at lds + 1024 j + 16 i.  One M0 (the LDS address) serves the whole run, as
// the instruction offset moves the LDS address along with the buffer one; M0
// is restored afterwards.  The copies are issued so that the compiler does not
// track them: it would otherwise wait for every copy in flight before each LDS
// read.  The caller waits on the vector-memory counter itself (one count per
// copy).  The LDS destination is passed as a pointer so that the compiler
// knows the statement writes there.
typedef __attribute__((address_space(3))) char lds_char;
template <int N>
__device__ inline void lds_copy16_run(lds_char* lds, int voffset, u32x4_t rsrc) {
  static_assert(N >= 1 && N <= 4, "1 to 4 copies per run");
  uint32_t saved;
  if constexpr (N == 1)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved) : "s"(lds), "v"(voffset), "s"(rsrc) : "memory");
  else if constexpr (N == 2)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen offset:1024 lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved) : "s"(lds), "v"(voffset), "s"(rsrc) : "memory");
  else if constexpr (N == 3)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen offset:2048 lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved) : "s"(lds), "v"(voffset), "s"(rsrc) : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen offset:2048 lds\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen offset:3072 lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved) : "s"(lds), "v"(voffset), "s"(rsrc) : "memory");
}

// s_barrier without the memory fences of __syncthreads (those would wait for
// the copies in flight); the "memory" clobber keeps the compiler from moving
// LDS accesses across it.  Callers wait for their own copies and LDS reads first.
__device__ inline void workgroup_barrier() { asm volatile("s_barrier" ::: "memory"); }

// max over the four lane groups of a row, as group_max, with v_max_f32 as
// written: the compiler's fmaxf first quiets signalling NaNs of operands it
// cannot prove quiet (two more instructions per swap), and these come out of
// the matrix cores and the lane swaps
__device__ inline float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ inline float group_max_raw(float v) {
  float a, b;
  swap16(v, a, b);
  swap32(vmax(a, b), a, b);
  return vmax(a, b);
}

__device__ inline void* uniform_ptr(const void* ptr) {
  const uint64_t a = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
}

__device__ inline f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}
__device__ inline f32x4_t mfma_f16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}

// Workgroup order.  The dispatcher deals linear workgroup ids to the 8 XCDs
// in turn, and each XCD has its own L2; workgroups of one (sequence, KV head)
// read the same K/V tiles.  The grid is (token tiles, KV heads x head_groups,
// sequences); this returns the (x, y, z) a workgroup serves.
//  * One sequence whose KV heads divide 8 (or are a multiple of 8): each XCD
//    serves the token tiles of one KV head (of one residue class of them, when
//    there are fewer than 8 heads; of every 8th head, when there are more), so
//    the L2 of an XCD holds one K/V stream at a time.
//  * Otherwise (a batch, whose sequences may differ in length and must stay
//    spread over all XCDs): the head_groups workgroups that share a (sequence,
//    KV head, token tile) get linear ids 8 apart -- same XCD, back to back.
// Token tiles keep their order within an XCD (x ascending = longest first).
__device__ inline void remap_workgroup(int HG, int* bx, int* by, int* bz) {
  const int NX = gridDim.x, NY = gridDim.y, NZ = gridDim.z;
  const int NG = NY / HG;  // KV heads
  const int L = blockIdx.x + NX * (blockIdx.y + NY * blockIdx.z);
  const int c = L & 7, k = L >> 3;  // XCD, and place in its dispatch order
  if (NZ == 1 && 8 % NG == 0 && NX % (8 / NG) == 0) {
    const int R = 8 / NG;  // XCDs per KV head
    const int j = k / HG;
    *bx = j * R + c % R;
    *by = (c / R) * HG + k % HG;
    *bz = 0;
    return;
  }
  if (NZ == 1 && NG % 8 == 0) {
    const int j = k / HG;
    *bx = j % NX;
    *by = ((j / NX) * 8 + c) * HG + k % HG;
    *bz = 0;
    return;
  }
  const int N = NX * NY * NZ;
  const int M = N / (8 * HG) * (8 * HG);
  int U, hp;  // unit = (KV head, token tile, sequence), KV head fastest; head group within it
  if (L < M) {
    U = (k / HG) * 8 + c;
    hp = k % HG;
  } else {
    U = M / HG + (L - M) / HG;
    hp = (L - M) % HG;
  }
  *by = (U % NG) * HG + hp;
  *bx = (U / NG) % NX;
  *bz = U / NG / NX;
}

// Sequence order of a batch.  The dispatcher starts workgroups in linear-id
// order, and a batch ends with its last long walk: a heavy sequence whose
// workgroups come last leaves most compute units idle at the end.  For up to
// kOrderMaxSeqs sequences every workgroup ranks the sequences by their
// longest walk (context + chunk tokens, ties by index), heaviest first, and
// serves the sequence of rank z; larger batches keep the given order.  Returns
// the sequence of rank z.  Uses `key` and `seq` (kOrderMaxSeqs entries each)
// and two workgroup barriers; every thread of the workgroup must call it.
constexpr int kOrderMaxSeqs = 64;
__device__ inline int sequence_of_rank(const PrefillArgs& a, int nseq, int z, int64_t* key, int* seq) {
  const int t = threadIdx.x;
  if (t < nseq) key[t] = (int64_t)a.context_lens[t] + (a.query_start[t + 1] - a.query_start[t]);
  __syncthreads();
  if (t < nseq) {
    const int64_t k = key[t];
    int rank = 0;
    for (int j = 0; j < nseq; ++j) rank += (key[j] > k) || (key[j] == k && j < t);
    seq[rank] = t;  // a strict total order: every rank gets one sequence
  }
  __syncthreads();
  return seq[z];
}

// LDS of a walk: the ring of K/V step buffers, the logits a paired wave
// leaves for its partner ([step parity][row group][block][column tile][lane]),
// and the fp16 range flag of the F16 pass.
template <int D, bool SOLO>
struct WalkLds {
  static constexpr int kTileStride = kBlockTokens * D * 2 + 64;
  static constexpr int kBufs = 3;
  __attribute__((aligned(16))) char kv[kBufs * 4 * kTileStride];
  f32x4_t xs[SOLO ? 1 : 2][SOLO ? 1 : kRowGroups][2][2][kWave];
  int f16_bad;
};

// Where a walk leaves its rows: the output itself (normalised), or, for a
// piece of a walk split between workgroups, a partial slot (unnormalised rows
// and each row's running max and sum, combined by merge_kernel).  Slot layout
// for the solo layout: rows [wave][column tile][16-dim tile][lane] as float4
// (lane = 16 lane-group + row), stats [wave][column tile][row][max, sum].
struct WalkOut {
  float* part;   // null: final rows into the output
  float* stats;
};

// Walks steps [st_lo, min(st_hi, its walk's steps)) of one workgroup's rows --
// sequence s (chunk rows q_lo .., n tokens over ctx cached), head group `by`
// (KV head by / head_groups), token tile qt -- and leaves the rows in `dst`.
// `poison` writes NaN rows instead (a sequence out of contract).  All threads
// of the workgroup call it with the same arguments; st_lo must lie below the
// walk's step count.
template <int D, int HC, bool SOLO>
__device__ __forceinline__ void walk_rows(const PrefillArgs& a, int s, int by, int qt, int q_lo, int n, int ctx,
                                          int st_lo, int st_hi, bool poison, WalkOut dst, WalkLds<D, SOLO>& L) {
  // Solo layout: a wave holds its 32 output rows over all of D and owns them
  // alone (8 row groups, 256 rows per workgroup); it forms both logit tiles of
  // a step itself, and nothing is exchanged.  Paired layout (D = 256 only):
  // two waves share 32 rows, one half of D each (4 row groups, 128 rows).
  static_assert(SOLO || D == 256, "the paired layout serves head size 256");
  constexpr bool kSolo = SOLO;
  constexpr bool kF16 = PAD_PREFILL_F16_PV;
  constexpr int RG = kSolo ? 2 * kRowGroups : kRowGroups;  // 32-row groups per workgroup
  constexpr int TW = RG / HC;            // 32-token groups per workgroup
  constexpr int KS = D / 32;             // QK steps (32 dims each)
  constexpr int DT = kSolo ? D / 16 : D / 32;  // 16-dim output tiles of this wave's part of D
  constexpr int kTileBytes = kBlockTokens * D * 2;
  // tiles sit 64 bytes apart in the LDS bank space, so that the K reads of the
  // two blocks' keys in one lane group hit distinct banks
  constexpr int kTileStride = kTileBytes + 64;
  constexpr int kStepBytes = 4 * kTileStride;  // K and V of two blocks
  constexpr int CH = kTileBytes / 1024;  // 1 KB copies per tile (one per load instruction)
  // step buffers: in iteration st the arithmetic reads V of step st and K of
  // step st + 1, and the copies of step st + 2 are in flight
  constexpr int kBufs = 3;
  // The copies of step st + 2 are issued after this wave's logits of step
  // st + 1, not at the top of the step.  The compiler guards each vector load
  // it issues itself (the reload of a spilled register, for one) with a wait
  // for the whole vector-memory counter, which counts these copies too;
  // issued at the top, they could be waited for inside the step they were
  // issued in.  Issued late, the prefix attention measured 8 % faster at
  // D = 256 (where a spilled register was then reloaded in every step), 7 %
  // at D = 128 and, once the block ids came by scalar loads, 6 % at D = 64.
  static_assert(WalkLds<D, SOLO>::kTileStride == kTileStride && WalkLds<D, SOLO>::kBufs == kBufs, "LDS shape");
  char* const kv_lds = L.kv;
  auto& xs_lds = L.xs;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int rg = kSolo ? wave : wave >> 1;   // row group
  const int dh = kSolo ? 0 : wave & 1;       // half of D this wave accumulates
  const int lg = lane >> 4;              // lane group
  const int g = by / a.head_groups;
  const int h = g * a.group + (by % a.head_groups) * HC + rg % HC;
  const int wg_tok0 = qt * (kRowsPerWave * TW);
  const int tok0 = wg_tok0 + (rg / HC) * kRowsPerWave;

  // rows of this wave: column tile ct, lane -> chunk token tok0 + 16 ct + lane%16
  int rpos[2];
  bool row_ok[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int tok = tok0 + 16 * ct + (lane & 15);
    row_ok[ct] = tok < n;
    rpos[ct] = ctx + tok;
  }
  auto store_rows = [&](const f32x4_t (*o)[DT], const float* inv) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int row = q_lo + tok0 + 16 * ct + (lane & 15);
      if (!row_ok[ct] || row < 0 || row >= a.num_tokens) continue;
      float* dst = a.out + ((size_t)row * a.num_heads + h) * D + 16 * DT * dh + 4 * lg;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4_t v = o[ct][dt] * inv[ct];
        *reinterpret_cast<f32x4_t*>(dst + 16 * dt) = v;
      }
    }
  };
  if (poison) {
    // out-of-contract sizes: NaN rows, within the output's bounds
    f32x4_t o[2][DT];
    const float nan[2] = {NAN, NAN};
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[ct][dt] = f32x4_t{1.0f, 1.0f, 1.0f, 1.0f};
    store_rows(o, nan);
    return;
  }

  // Q^T operand, held in registers for the whole walk: column tile ct, step
  // ks -> the row's dims 32 ks + 8 lg .. + 8
  u32x4_t qop[2][KS];
  {
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(a.query), (short)0, (int)((size_t)a.num_tokens * a.num_heads * D * 2), kRsrcWord3);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int row = q_lo + tok0 + 16 * ct + (lane & 15);
      const int off = ((row * a.num_heads + h) * D + 8 * lg) * 2;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 64 * ks, 0, 0);
        if (a.negate_q) v ^= u32x4_t{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
        qop[ct][ks] = row_ok[ct] ? v : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }

  // keys the workgroup walks: up to its last row's position; each wave masks
  // to its own rows
  const int kend = ctx + min(wg_tok0 + kRowsPerWave * TW, n);
  const int nblk = (kend + kBlockTokens - 1) / kBlockTokens;
  const int nsteps = (nblk + 1) / 2;
  // the steps this call walks
  const int lo = st_lo;
  const int hi = min(st_hi, nsteps);
  // keys below a wave's first row position are visible to all its rows
  const int diag_from = ctx + tok0;
  // V is zeroed from here on: the tail slots of the sequence's last block, and
  // a step's second block when the walk has an odd number of blocks (its LDS
  // tile is not written)
  const int v_end = min(ctx + n, nblk * kBlockTokens);
  const int32_t* table_row = a.block_tables + (size_t)s * a.max_blocks;
  const size_t head_off = (size_t)g * kTileBytes;
  const size_t block_stride = (size_t)a.num_kv_heads * kTileBytes;
  bool bad = false;
  f32x4_t o[2][DT];
  // The reference max starts at a finite floor, not -inf: a piece of a split
  // walk that starts past key 0 can hold rows that see none of its keys, and
  // their weights exp2(-inf - ref) must come out 0, not NaN.  The first keys
  // a row sees always lift the reference (the rescale factor exp2(floor - max)
  // is then 0, as from -inf), so whole walks give the same bits either way.
  float m_ref[2];
  float l_run[2];

  // Tile kb of a step's S^T (16 of its 32 keys x the wave's 32 rows, over all
  // of D): the A operand comes straight from the step's K tiles in LDS
  const int kb = dh;  // the tile of every step that this wave forms (paired waves)
  // tile kb's row r (lane r % 16) is key 8 ((r >> 2) & 1) + 4 kb + (r & 3) of
  // the step's block r >> 3, so that the rows a lane holds in the two tiles are
  // 8 consecutive keys of one block: its P.V operand is one 16-byte V read
  const int k_lane = ((lane & 15) >> 3) * kTileStride + 256 * lg +
                     16 * (8 * (((lane & 15) >> 2) & 1) + 4 * kb + (lane & 3));
  auto qk_block = [&](const char* kv, f32x4_t* r) {
    r[0] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    r[1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(kv + k_lane + 1024 * ks);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const u32x4_t qb = qop[ct][ks];
        r[ct] = mfma_bf16(kf, qb, r[ct]);
      }
    }
  };
  // V elements stored in LDS with the two 16-byte halves of every other group
  // of 8 dims swapped (16-byte chunk c of the tile lands at c ^ ((c >> 4) & 1)),
  // so that the V operand reads of a half-wave hit distinct banks
  const int k_src = 16 * lane;
  const int v_src = 16 * (lane ^ ((lane >> 4) & 1));
  constexpr int kLead = kBufs - 1;  // iteration st issues the copies of step st + kLead

  // One pass over steps [lo, hi).  F16: P.V runs on
  // v_mfma_f32_16x16x32_f16 with one fp16 term for p, and V is converted to
  // fp16 in LDS once per step, instead of two bf16 products per tile (p split
  // into hi + lo).  V is exact in fp16 where |v| <= 65504; p is computed
  // against a reference kF16Shift below the running one, so the weights lie in
  // [0, 2^15] and a weight below 2^-14 of the largest is all that lands in
  // fp16's subnormal range.  A V value beyond 65504 (or an infinity) sets a
  // flag; the pass then returns false, and the walk starts over in the bf16
  // form.  (The flag is read once, after the last step's barrier: an exit
  // from the step loop on it made the compiler hold about 90 more registers
  // and spill at D = 256.)
  auto run = [&](auto f16_tag) -> bool {
    constexpr bool F16 = decltype(f16_tag)::value;
    // Copies.  bf16 form: the first wave of pair t copies tile t of each step
    // into LDS (K of the step's first block, K of its second, V of the first,
    // V of the second); the second wave of each pair copies nothing.
    // (Measured: copies issued by four waves, one per SIMD pair, beat the same
    // copies spread over all eight by 2.5 %; by one or two waves, they were
    // slower.)  F16 form (both layouts): copying wave w (w < 4) takes half
    // w & 1 of block w >> 1's K tile and of its V tile, so that each of the
    // four converts the V it copied, on its own SIMD; at D = 256 every wave
    // copies a quarter (below).
    const int my_tile = kSolo ? wave & 3 : wave >> 1;  // bf16 form: 0, 1: K of the two blocks; 2, 3: V
    // F16 form at D = 256: all eight waves copy, a quarter of one block's K
    // and V tiles each, and convert their own quarter of V, so that the two
    // waves of a SIMD share the conversion: 2 % faster than four copying
    // waves there (and 9 % slower at D = 128, whose quarters are single 1 KB
    // copies; D = 64's tiles do not split in quarters of whole copies).
    constexpr bool k8 = F16 && D == 256;
    constexpr int kParts = k8 ? 4 : 2;          // F16 form: parts of a tile, one per copying wave
    constexpr int kPartBytes = kTileBytes / kParts;
    constexpr int kPartCopies = CH / kParts;    // 1 KB copies of one part
    // this wave's copies per step: the two parts (K and V), or one tile
    constexpr int CPS = F16 ? 2 * kPartCopies : CH;
    const bool copier = k8 ? true : (kSolo || F16) ? wave < 4 : dh == 0;
    const int my_b = k8 ? wave >> 2 : F16 ? (wave >> 1) & 1 : my_tile & 1;
    const int my_part = k8 ? wave & 3 : wave & 1;  // F16 form
    const char* pool = (my_tile < 2) ? a.key_cache : a.value_cache;
    // The block table is read-only for the launch: each wave fetches the id of
    // the block it copies next by a scalar load, one issue ahead.  (Loaded 64
    // at a time into a vector register instead, the id load left the loop with
    // a wait for the whole vector-memory counter at its back edge, which
    // drained the step's own copies: 3 to 5 % slower.)
    const int32_t __attribute__((address_space(4)))* table_c =
        (const int32_t __attribute__((address_space(4)))*)table_row;
    auto fetch_id = [&](int step) {
      const int blk = 2 * step + my_b;
      return blk < nblk ? table_c[blk] : 0;
    };
    int next_id = fetch_id(lo);
    const int src_off = my_tile < 2 ? k_src : v_src;
    auto rsrc = [&](const char* base_pool, int phys, uint32_t bytes) {
      const uint64_t base = reinterpret_cast<uint64_t>(base_pool + (size_t)phys * block_stride + head_off);
      return u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base),
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)) & 0xffffu,
                     (uint32_t)__builtin_amdgcn_readfirstlane(bytes), (uint32_t)kRsrcWord3};
    };
    auto issue = [&](int step, char* buf) {
      const int blk = 2 * step + my_b;
      int phys = next_id;
      next_id = fetch_id(step + 1);
      const bool live = blk < nblk;
      const bool ok = phys >= 0 && (int64_t)phys < a.num_blocks;
      bad |= live && !ok;
      const uint32_t bytes = (live && ok) ? kTileBytes : 0u;
      if (!ok) phys = 0;
      if (!copier) return;
      if constexpr (F16) {
        const int h_off = my_part * kPartBytes;
        lds_copy16_run<kPartCopies>((lds_char*)(buf + my_b * kTileStride + h_off), k_src + h_off,
                                    rsrc(a.key_cache, phys, bytes));
        lds_copy16_run<kPartCopies>((lds_char*)(buf + (2 + my_b) * kTileStride + h_off), v_src + h_off,
                                    rsrc(a.value_cache, phys, bytes));
      } else {
        const u32x4_t rs = rsrc(pool, phys, bytes);
        lds_char* lds = (lds_char*)(buf + my_tile * kTileStride);
        static_assert(CH <= 8, "at most two runs of copies per tile");
        if constexpr (CH <= 4) {
          lds_copy16_run<CH>(lds, src_off, rs);
        } else {
          lds_copy16_run<4>(lds, src_off, rs);
          lds_copy16_run<CH - 4>(lds + 4096, src_off + 4096, rs);
        }
      }
    };
    // F16 form: a copying wave's conversion of the V it copied for `step`, in
    // place.  Lane l holds 16-byte chunks 64 j + l of its half of the tile:
    // 8 consecutive tokens of one dim, the first at 8 ((l & 1) ^ ((l >> 4) & 1))
    // in the block (the swizzle above).  The masked form (a pass's last step)
    // first zeroes the positions from v_end on, on the walk's last step (the
    // tail slots of the last block, and an odd walk's second block, which was
    // not copied).  Returns whether a value lies beyond fp16's range.
    // The range check runs on the bf16 bits, two at a time: a magnitude of
    // 0x4780 (65536) or more is beyond fp16's largest value (the bf16 below it
    // is 65280), and infinities and NaNs lie above it too.  (As float maxima
    // it cost two more instructions a pair, which the compiler added to quiet
    // signalling NaNs; this form and the lane-group max without them measured
    // 2.5 % faster at D = 256.)
    auto convert_v = [&](int step, char* buf, auto masked) {
      char* vt = buf + (2 + my_b) * kTileStride + my_part * kPartBytes + 16 * lane;
      const int pos0 = (2 * step + my_b) * kBlockTokens + 8 * ((lane & 1) ^ ((lane >> 4) & 1));
      const bool tail = decltype(masked)::value && step == nsteps - 1;
      u16x2_t mx = {0, 0};
#pragma unroll
      for (int j = 0; j < kPartCopies; ++j) {
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(vt + 1024 * j);
        u32x4_t r;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t u = w[k];
          if (tail)
            u &= (pos0 + 2 * k < v_end ? 0xffffu : 0u) | (pos0 + 2 * k + 1 < v_end ? 0xffff0000u : 0u);
          mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2_t, u & 0x7fff7fffu));
          const float v0 = __builtin_bit_cast(float, u << 16);
          const float v1 = __builtin_bit_cast(float, u & 0xffff0000u);
          r[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{v0, v1}), f16x2_t));
        }
        *reinterpret_cast<u32x4_t*>(vt + 1024 * j) = r;
      }
      return mx[0] >= 0x4780u || mx[1] >= 0x4780u;
    };

#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[ct][dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m_ref[0] = m_ref[1] = kNoKeysMax;
    l_run[0] = l_run[1] = 0.0f;
    bad = false;
    if constexpr (F16) {
      // the range flag starts clear before any wave can set it
      if (threadIdx.x == 0) L.f16_bad = 0;
      __syncthreads();
    }
    for (int k = lo; k < lo + kLead && k < hi; ++k) {
      issue(k, kv_lds + (k % kBufs) * kStepBytes);
    }
    // F16: V of step lo (the last step's is converted in its own iteration)
    if (F16 && copier && lo + 1 < hi) {
      __builtin_amdgcn_s_waitcnt(kWaitVmLds(CPS));
      if (convert_v(lo, kv_lds + (lo % kBufs) * kStepBytes, std::false_type{})) L.f16_bad = 1;
    }
    // step 0's logits (paired waves: formed ahead, for the exchange)
    if constexpr (!kSolo) {
      if (hi - lo > 1)
        __builtin_amdgcn_s_waitcnt(kWaitVmLds(CPS));
      else
        __builtin_amdgcn_s_waitcnt(kWaitVmLds(0));
      workgroup_barrier();
      f32x4_t first[2];
      qk_block(kv_lds + (lo % kBufs) * kStepBytes, first);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) xs_lds[lo & 1][rg][kb][ct][lane] = first[ct];
    }

    // Iteration st: wait for the copies of step st + 1 (this wave's; the
    // barrier makes every wave's visible, publishes every wave's logits of step
    // st, and retires all reads of the buffer the next copies reuse); then the
    // softmax of step st, this wave's logits of step st + 1, the copies of step
    // st + 2 and the P.V of step st.
    //
    // Only the last step can hold V positions the walk does not hold (every
    // earlier step ends at least one block before the end of the keys), so it
    // alone runs the masked P.V, as separate code after the loop.  With the
    // choice made per step inside the loop, the two P.V forms met at a join
    // where the compiler kept the accumulators in two register sets and copied
    // all of them on every step (32 64-bit moves); that also held 44 more
    // registers at D = 256 and made the allocator spill a query operand.  Taken
    // out of the loop: 7 % faster at D = 256, 5-7 % at D = 128.
    auto iter = [&](int st, auto last) {
      // paired waves need K of step st + 1 now; solo waves only step st
      if (kSolo && st + 1 < hi)
        __builtin_amdgcn_s_waitcnt(kWaitVmLds(CPS));
      else
        __builtin_amdgcn_s_waitcnt(kWaitVmLds(0));
      workgroup_barrier();
      const int b0 = 2 * st;  // first block of this step
      const char* kv = kv_lds + (st % kBufs) * kStepBytes;
      // F16: the pass's last step converts its own V here (the masked form),
      // published by a barrier before its P.V: kept out of the loop, the
      // masking code made the compiler spill at D = 256
      if constexpr (F16 && decltype(last)::value)
        if (copier && convert_v(st, kv_lds + (st % kBufs) * kStepBytes, std::true_type{})) L.f16_bad = 1;

      // ---- logits S^T of the step: two blocks x two column tiles, one block
      // formed by each wave of the pair
      f32x4_t sc[2][2];
      if constexpr (kSolo) {
        // solo waves: kb = 0, so k_lane is tile 0's offset; tile 1's is 64 bytes on
        qk_block(kv, sc[0]);
        qk_block(kv + 64, sc[1]);
      } else {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) sc[b][ct] = xs_lds[st & 1][rg][b][ct][lane];
      }

      // ---- mask, running max, weights.  Only steps that reach the wave's first
      // row position (the diagonal) or the end of the keys need the mask.
      const bool diag = (b0 + 2) * kBlockTokens > diag_from;
      float x[2][2][4];
      float bm[2];
      // separate code for the masked steps, so the common step carries no selects
      auto logits = [&](auto masked) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          bm[ct] = -INFINITY;
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float v = sc[b][ct][i];
              if constexpr (decltype(masked)::value) {
                const int jpos = (b0 + (lg >> 1)) * kBlockTokens + 8 * (lg & 1) + 4 * b + i;
                x[b][ct][i] = (jpos <= rpos[ct] && jpos < kend) ? v : -INFINITY;
              } else {
                x[b][ct][i] = v;
              }
              bm[ct] = fmaxf(bm[ct], x[b][ct][i]);
            }
          bm[ct] = group_max_raw(bm[ct]);
          // the scale is positive: the max of the scaled logits is the scaled max
          bm[ct] = bm[ct] > -INFINITY ? bm[ct] * a.qscale : -INFINITY;
        }
      };
      if (diag)
        logits(std::true_type{});
      else
        logits(std::false_type{});
      // Lazy rescale: a uniform branch, taken when some row's max grows past
      // its reference by more than 2^8.  (Up to D = 64 it once ran every
      // step, branch-free, with a factor of 1 where the reference stays: 15 %
      // faster than the branch with the bf16 hi + lo weights, whose register
      // copies around the branch cost more; with fp16 weights the branch
      // measured 13 % faster there, 754 -> 854 TFLOP/s.)
      if (__builtin_expect(__ballot(bm[0] > m_ref[0] + kLazyLog2 || bm[1] > m_ref[1] + kLazyLog2) != 0, 0)) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const float m_new = bm[ct] > m_ref[ct] + kLazyLog2 ? bm[ct] : m_ref[ct];
          const float alpha = __builtin_amdgcn_exp2f(m_ref[ct] - m_new);  // 0 on a row's first keys
          l_run[ct] *= alpha;
          m_ref[ct] = m_new;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[ct][dt] *= alpha;
        }
      }
      // The weights.  bf16 form: p = hi + lo, hi keeping the top 16 bits of p
      // (truncation, so p - hi is exact), lo the top 16 bits of the remainder;
      // packed by byte permutes.  F16 form: p rounded to fp16 (nearest even),
      // against the reference less kF16Shift.
      u32x4_t p_hi[2], p_lo[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const float m_sub = F16 ? m_ref[ct] - kF16Shift : m_ref[ct];
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int b = k >> 1, i = 2 * (k & 1);
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[b][ct][i], a.qscale, -m_sub));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[b][ct][i + 1], a.qscale, -m_sub));
          l_run[ct] += p0 + p1;
          if constexpr (F16) {
            hi[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{p0, p1}), f16x2_t));
          } else {
            const uint32_t u0 = __builtin_bit_cast(uint32_t, p0), u1 = __builtin_bit_cast(uint32_t, p1);
            const float r0 = p0 - __builtin_bit_cast(float, u0 & 0xffff0000u);
            const float r1 = p1 - __builtin_bit_cast(float, u1 & 0xffff0000u);
            hi[k] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
            lo[k] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, r1), __builtin_bit_cast(uint32_t, r0),
                                          0x07060302u);
          }
        }
        p_hi[ct] = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
        if constexpr (!F16) p_lo[ct] = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
      }

      // ---- this wave's logits of the next step, for the pair (issued after
      // the softmax, so that the matrix cores work through them while P.V's
      // operands are read)
      if (!kSolo && st + 1 < hi) {
        f32x4_t next[2];
        qk_block(kv_lds + ((st + 1) % kBufs) * kStepBytes, next);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) xs_lds[(st + 1) & 1][rg][kb][ct][lane] = next[ct];
      }

      // ---- the copies of step st + 2 (here, after the logits of step st + 1)
      if (st + kLead < hi) {
        issue(st + kLead, kv_lds + ((st + kLead) % kBufs) * kStepBytes);
      }

      // ---- O^T += V^T P^T.  V elements at positions the walk does not hold are
      // zeroed: p is 0 there, but 0 * NaN would poison the row (the F16 form
      // zeroed them in its conversion).
      auto pv = [&](auto masked) {
        uint32_t vm[4];
        if constexpr (decltype(masked)::value) {
          const int pos = (b0 + (lg >> 1)) * kBlockTokens + 8 * (lg & 1);
#pragma unroll
          for (int w = 0; w < 4; ++w)
            vm[w] = (pos + 2 * w < v_end ? 0xffffu : 0u) | (pos + 2 * w + 1 < v_end ? 0xffff0000u : 0u);
        }
        // dim d = 16 dt + lane%16, tokens 8 (lg & 1) .. + 8 of block lg >> 1:
        // 16-byte chunk 2 d + (lg & 1) of that block's tile, stored swizzled
        const char* vt = kv + (2 + (lg >> 1)) * kTileStride + 512 * DT * dh + (lane & 15) * 32 +
                         16 * ((lg & 1) ^ ((lane >> 3) & 1));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          u32x4_t va = *reinterpret_cast<const u32x4_t*>(vt + 512 * dt);
          if constexpr (decltype(masked)::value)
            va = u32x4_t{va[0] & vm[0], va[1] & vm[1], va[2] & vm[2], va[3] & vm[3]};
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            if constexpr (F16) {
              o[ct][dt] = mfma_f16(va, p_hi[ct], o[ct][dt]);
            } else {
              o[ct][dt] = mfma_bf16(va, p_hi[ct], o[ct][dt]);
              o[ct][dt] = mfma_bf16(va, p_lo[ct], o[ct][dt]);
            }
          }
        }
      };
      // In the bf16 form at D = 256 solo waves issue their P.V products at
      // raised priority, so that a wave keeps the matrix core for its whole
      // run of 2 DT products instead of interleaving with the other waves'
      // logits: measured 3 % faster there.  The pairs (which trade logits
      // through LDS) and the smaller head sizes (shorter runs) lose 1 to 2 %
      // with it, and so does the F16 form, whose run is half as long (0.6 %).
      constexpr bool kPvPriority = kSolo && D == 256 && !F16;
      if constexpr (F16 && decltype(last)::value) {
        __builtin_amdgcn_s_waitcnt(kWaitVmLds(0));
        workgroup_barrier();
      }
      if constexpr (kPvPriority) __builtin_amdgcn_s_setprio(1);
      if constexpr (F16)
        pv(std::false_type{});
      else
        pv(last);
      if constexpr (kPvPriority) __builtin_amdgcn_s_setprio(0);

      if constexpr (F16) {
        // the conversion of step st + 1's V, once this wave's copies of it are
        // in (those of step st + 2 may still be in flight).  The compiler
        // barrier keeps its LDS reads out of the P.V above, where they held
        // enough registers to spill at D = 256.  (Placed before the P.V
        // instead, so that the other wave of the SIMD would multiply
        // meanwhile, the kernel measured 3 % slower.)
        asm volatile("" ::: "memory");
        if (copier && st + 2 < hi) {
          __builtin_amdgcn_s_waitcnt(kWaitVmLds(CPS));
          if (convert_v(st + 1, kv_lds + ((st + 1) % kBufs) * kStepBytes, std::false_type{})) L.f16_bad = 1;
        }
      }

    };
    for (int st = lo; st + 1 < hi; ++st) iter(st, std::false_type{});
    if (hi > lo) iter(hi - 1, std::true_type{});
    // F16: every conversion came before the last step's P.V barrier, so
    // every wave reads the same flag here
    return F16 ? __builtin_amdgcn_readfirstlane(L.f16_bad) == 0 : true;
  };
  bool done = false;
  if constexpr (kF16) done = run(std::true_type{});
  if (!done) {
    if constexpr (kF16) {
      // the F16 pass stopped: every wave's copies landed and every LDS read
      // retired before the ring is reused
      __builtin_amdgcn_s_waitcnt(kWaitVmLds(0));
      workgroup_barrier();
    }
    run(std::false_type{});
  }
  // every wave's block-id checks count for the whole workgroup's tiles (and
  // the barrier retires every LDS read before a next walk's copies)
  bad = __syncthreads_or(bad);
  float l[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) l[ct] = group_sum(l_run[ct]);
  if (dst.part) {
    // a piece of a split walk: unnormalised rows, and each row's reference
    // max (log2 units of the scaled logits; that of the weights, so the F16
    // pass's less kF16Shift) and sum; NaN sums mark a bad block id
    float* po = dst.part + (size_t)wave * (2 * DT * kWave * 4);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f32x4_t*>(po + ((ct * DT + dt) * kWave + lane) * 4) = o[ct][dt];
    if (lg == 0 && dh == 0) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        float* ps = dst.stats + ((rg * 2 + ct) * 16 + lane) * 2;
        ps[0] = done ? m_ref[ct] - kF16Shift : m_ref[ct];
        ps[1] = bad ? NAN : l[ct];
      }
    }
    return;
  }
  float inv[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) inv[ct] = bad ? NAN : 1.0f / l[ct];
  store_rows(o, inv);
}

// One workgroup per (token tile, head group, sequence), longest walks first.
template <int D, int HC, bool SOLO>
__global__ __launch_bounds__(kWaves * kWave) void prefill_kernel(PrefillArgs a) {
  constexpr int TPW = kRowsPerWave * (SOLO ? 2 * kRowGroups : kRowGroups) / HC;  // chunk tokens per workgroup
  int bx, by, bz;
  remap_workgroup(a.head_groups, &bx, &by, &bz);
  __shared__ int64_t order_key[kOrderMaxSeqs];
  __shared__ int order_seq[kOrderMaxSeqs];
  const int s = (gridDim.z > 1 && gridDim.z <= kOrderMaxSeqs)
                    ? __builtin_amdgcn_readfirstlane(sequence_of_rank(a, gridDim.z, bz, order_key, order_seq))
                    : bz;
  const int qt = gridDim.x - 1 - bx;  // longest walks first
  const int q_lo = a.query_start[s];
  const int q_hi = a.query_start[s + 1];
  const int n = q_hi - q_lo;
  const int ctx = a.context_lens[s];
  // out of contract: bad offsets or sizes, or a chunk longer than the grid
  // covers (n_s > max_query_len), whose rows past the grid no workgroup writes
  const bool bad_seq = ctx < 0 || n < 0 || q_lo < 0 || q_hi > a.num_tokens ||
                       (int64_t)ctx + n > (int64_t)a.max_blocks * kBlockTokens ||
                       (int64_t)n > (int64_t)gridDim.x * TPW;
  // the whole workgroup leaves together (it shares barriers)
  if (qt * TPW >= max(n, 0)) return;
  __shared__ WalkLds<D, SOLO> lds;
  walk_rows<D, HC, SOLO>(a, s, by, qt, q_lo, n, ctx, 0, INT_MAX, bad_seq, WalkOut{nullptr, nullptr}, lds);
}

// ---------------------------------------------------------------------------
// Split launch.  In a batch whose walks differ in length, the longest walks
// decide when the launch ends while most compute units sit idle.  The split
// launch cuts every walk longer than C steps into k = ceil(steps / C) pieces
// of equal length -- C is the launch's total steps over kSplitRounds rounds of
// its resident workgroups -- and serves the pieces before the whole walks:
// the dispatcher, which starts workgroups in order as compute units free up,
// then evens the units out.  A unit (a piece or a whole walk of one KV head,
// for its HG head chunks) is listed by split_plan_kernel in this order:
//   1. the pieces: by piece index j, then sequence (longest walk first), then
//      tile (longest first), then KV head.  Pieces with one index start at
//      nearly the same key, so the workgroups that run together read the same
//      K/V tiles through L2;
//   2. the whole walks: by sequence, tile (longest first), KV head.
// Each piece leaves its unnormalised rows in a partial slot, and
// split_merge_kernel combines the pieces of a cut walk by their log-sum-exp.
// ---------------------------------------------------------------------------
#ifndef PAD_PREFILL_SPLIT_ROUNDS
#define PAD_PREFILL_SPLIT_ROUNDS 4
#endif
constexpr int kSplitRounds = PAD_PREFILL_SPLIT_ROUNDS;  // rounds of resident workgroups the pieces fill
// Walks are cut only when the longest is above 1 / kSplitShare of a resident
// workgroup's fair share (total steps / N): below that the dispatcher's
// longest-first order already evens the compute units out.
#ifndef PAD_PREFILL_SPLIT_SHARE
#define PAD_PREFILL_SPLIT_SHARE 2
#endif
constexpr int kSplitShare = PAD_PREFILL_SPLIT_SHARE;
constexpr int kSplitMaxPieces = 32;  // pieces of one walk, at most
constexpr int kSplitMinSteps = 16;   // C, at least
constexpr int kSplitRows = 2 * kRowGroups * kRowsPerWave;  // rows of a solo workgroup
constexpr int kSplitStatFloats = 2 * kSplitRows;
constexpr int kSplitPlanThreads = 1024;

// Header words the plan writes (int32 at the workspace's start): units
// listed, pieces among them (listed first), cut walks, C, the most pieces of
// one walk, sequences with cut walks.  The walk and merge kernels read the
// first and third; tests read them all.
enum { kHdrUnits = 0, kHdrPieces, kHdrCutWalks, kHdrStep, kHdrMaxPieces, kHdrCutSeqs, kHdrWords = 16 };

struct PrefillSplit {
  int32_t* hdr;        // [kHdrWords]
  int4* units;         // {sequence, tile, KV head, j << 16 | k}
  int32_t* order;      // [S]: sequence of each rank (longest walk first), past the plan's LDS
  int32_t* cut_idx;    // [S]: rank of the sequence among those with cut walks, or -1
  int32_t* cut_seq;    // [cut_seq_cap]: sequence of each such rank, past the plan's LDS
  int32_t* pair_off;   // [kSplitMaxPieces x cut_seq_cap]: first unit of (piece index, cut sequence)
  float* part;         // partial slots of 256 rows x D floats
  float* stats;        // partial slots of 256 rows x (max, sum)
  int num_seqs;
  int max_query_len;
  int ranges;          // N, resident workgroups of the walk kernel
  int tokens_per_wg;   // TPW, a multiple of 32
  int cut_seq_cap;
};

// 32-key steps of token tile t (its last row sees keys 0 .. ctx + min((t + 1) TPW, n) - 1).
__host__ __device__ inline int64_t tile_steps(int64_t t, int64_t ctx, int64_t n, int64_t tpw) {
  const int64_t e = (t + 1) * tpw;
  return (ctx + (e < n ? e : n) + 31) / 32;
}

// Steps of all of a sequence's walks (one head group): the tiles before the
// last are full, and tile t of them takes ceil(ctx / 32) + (t + 1) TPW / 32.
__host__ __device__ inline int64_t seq_walk_steps(int64_t ctx, int64_t n, int64_t tpw) {
  if (n <= 0) return 0;
  const int64_t T = (n + tpw - 1) / tpw;
  return (T - 1) * ((ctx + 31) / 32) + (tpw / 32) * ((T - 1) * T / 2) + tile_steps(T - 1, ctx, n, tpw);
}

// Tiles (of T) whose walks take more than thr steps: the longest ones, since
// the steps grow with the tile.
__device__ inline int tiles_above(int64_t thr, int64_t ctx, int64_t n, int64_t tpw, int T) {
  int lo = 0, hi = T;  // the first tile above thr
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (tile_steps(mid, ctx, n, tpw) > thr) hi = mid; else lo = mid + 1;
  }
  return T - lo;
}

// Whether sequence s is inside the contract (its walks are served).
__device__ inline bool split_seq_ok(const PrefillArgs& a, const PrefillSplit& p, int s, int* q_lo, int* n,
                                    int* ctx) {
  *q_lo = a.query_start[s];
  const int q_hi = a.query_start[s + 1];
  *n = q_hi - *q_lo;
  *ctx = a.context_lens[s];
  return *ctx >= 0 && *n >= 0 && *q_lo >= 0 && q_hi <= a.num_tokens && *n <= p.max_query_len &&
         (int64_t)*ctx + *n <= (int64_t)a.max_blocks * kBlockTokens;
}

// Exclusive scan of one value per thread over the workgroup (kSplitPlanThreads
// threads); returns the thread's offset and leaves the total in *total.
__device__ inline int plan_scan(int v, int* wave_sum, int* total) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) wave_sum[w] = x;
  __syncthreads();
  int before = 0, all = 0;
  for (int k = 0; k < kSplitPlanThreads / kWave; ++k) {
    if (k < w) before += wave_sum[k];
    all += wave_sum[k];
  }
  __syncthreads();  // wave_sum is reused by the next scan
  *total = all;
  return before + x - v;
}

// One workgroup: the unit list.  Up to kSplitPlanThreads sequences, their
// sizes, order and cut list live in LDS.
__global__ __launch_bounds__(kSplitPlanThreads) void split_plan_kernel(PrefillArgs a, PrefillSplit p) {
  __shared__ int wave_sum[kSplitPlanThreads / kWave];
  __shared__ unsigned long long total_steps;
  __shared__ int max_steps;
  __shared__ int64_t rank_key[kSplitPlanThreads];
  __shared__ int c_ctx[kSplitPlanThreads], c_n[kSplitPlanThreads];
  __shared__ int c_order[kSplitPlanThreads], c_cut[kSplitPlanThreads];
  const int tid = threadIdx.x;
  const int S = p.num_seqs, Hkv = a.num_kv_heads, HG = a.head_groups;
  const int64_t tpw = p.tokens_per_wg;
  const bool cached = S <= kSplitPlanThreads;
  int* const order = cached ? c_order : p.order;
  int* const cut_seq = cached ? c_cut : p.cut_seq;
  // context and chunk length of sequence s; chunk 0 for one out of contract
  auto seq = [&](int s, int* ctx, int* n) {
    if (cached) {
      *ctx = c_ctx[s];
      *n = c_n[s];
    } else {
      int q_lo;
      if (!split_seq_ok(a, p, s, &q_lo, n, ctx)) *n = 0;
    }
  };
  if (tid == 0) {
    total_steps = 0;
    max_steps = 0;
  }
  if (cached && tid < S) {
    int q_lo, n, ctx;
    const bool ok = split_seq_ok(a, p, tid, &q_lo, &n, &ctx);
    c_ctx[tid] = ctx;
    c_n[tid] = ok ? n : 0;
  }
  __syncthreads();
  // (1) total steps (all head groups) and the longest walk
  for (int s = tid; s < S; s += kSplitPlanThreads) {
    int n, ctx;
    seq(s, &ctx, &n);
    if (n == 0) continue;
    atomicAdd(&total_steps, (unsigned long long)seq_walk_steps(ctx, n, tpw) * (unsigned long long)(Hkv * HG));
    atomicMax(&max_steps, (int)tile_steps((n + tpw - 1) / tpw - 1, ctx, n, tpw));
  }
  __syncthreads();
  const int64_t B = (int64_t)total_steps;
  const int64_t rounds = (int64_t)kSplitRounds * p.ranges;
  int64_t C = (B + rounds - 1) / rounds;
  C = max(C, (int64_t)(max_steps + kSplitMaxPieces - 1) / kSplitMaxPieces);
  C = max(C, (int64_t)kSplitMinSteps);
  if ((int64_t)max_steps * kSplitShare * p.ranges <= B) C = max(C, (int64_t)max_steps);  // no walk is cut
  const int kmax = max_steps > C ? (int)((max_steps + C - 1) / C) : 1;
  // (2) serving order: longest walk (context + chunk) first; sequences out of
  // contract or without tokens last.  Past kSplitPlanThreads sequences, the
  // given order.
  if (cached) {
    if (tid < S) rank_key[tid] = c_n[tid] > 0 ? (int64_t)c_ctx[tid] + c_n[tid] : -1;
    __syncthreads();
    if (tid < S) {
      const int64_t k = rank_key[tid];
      int r = 0;
      for (int j = 0; j < S; ++j) r += (rank_key[j] > k) || (rank_key[j] == k && j < tid);
      order[r] = tid;
    }
  } else {
    for (int s = tid; s < S; s += kSplitPlanThreads) order[s] = s;
  }
  __syncthreads();  // order is read back below
  // (3) the sequences with cut walks, in serving order
  int n_cut = 0;
  for (int base = 0; base < S; base += kSplitPlanThreads) {
    const int r = base + tid;
    int cut = 0, s = -1;
    if (r < S) {
      s = order[r];
      int n, ctx;
      seq(s, &ctx, &n);
      cut = n > 0 && tile_steps((n + tpw - 1) / tpw - 1, ctx, n, tpw) > C;
    }
    int tot;
    const int o = n_cut + plan_scan(cut, wave_sum, &tot);
    if (r < S) {
      p.cut_idx[s] = cut ? o : -1;
      if (cut) cut_seq[o] = s;
    }
    n_cut += tot;
  }
  __syncthreads();  // cut_seq is read back below
  // (4) the pieces: pair (j, c) = (piece index, cut sequence c) holds, for
  // every KV head, the tiles whose walks have a piece j (the longest ones)
  const int pairs = kmax * n_cut;
  int n_pieces = 0, n_first = 0;
  for (int base = 0; base < pairs; base += kSplitPlanThreads) {
    const int q = base + tid;
    int cnt = 0, s = 0, j = 0, c = 0, ctx = 0, n = 0, T = 0;
    if (q < pairs) {
      j = q / n_cut;
      c = q - j * n_cut;
      s = cut_seq[c];
      seq(s, &ctx, &n);
      T = (int)((n + tpw - 1) / tpw);
      cnt = Hkv * tiles_above((j > 0 ? j : 1) * C, ctx, n, tpw, T);
    }
    int tot, tot_first;
    const int o = n_pieces + plan_scan(cnt, wave_sum, &tot);
    plan_scan(j == 0 ? cnt : 0, wave_sum, &tot_first);
    if (q < pairs) {
      p.pair_off[j * p.cut_seq_cap + c] = o;
      for (int i = 0; i < cnt; ++i) {
        const int t = T - 1 - i / Hkv;
        const int k = (int)((tile_steps(t, ctx, n, tpw) + C - 1) / C);
        p.units[o + i] = make_int4(s, t, i % Hkv, (j << 16) | k);
      }
    }
    n_pieces += tot;
    n_first += tot_first;
  }
  // (5) the whole walks, after the pieces
  int placed = 0;
  for (int base = 0; base < S; base += kSplitPlanThreads) {
    const int r = base + tid;
    int cnt = 0, s = 0, T = 0, above = 0;
    if (r < S) {
      s = order[r];
      int n, ctx;
      seq(s, &ctx, &n);
      if (n > 0) {
        T = (int)((n + tpw - 1) / tpw);
        above = tiles_above(C, ctx, n, tpw, T);
        cnt = Hkv * (T - above);
      }
    }
    int tot;
    const int o = n_pieces + placed + plan_scan(cnt, wave_sum, &tot);
    for (int i = 0; i < cnt; ++i) p.units[o + i] = make_int4(s, T - above - 1 - i / Hkv, i % Hkv, 1);
    placed += tot;
  }
  if (tid == 0) {
    p.hdr[kHdrUnits] = n_pieces + placed;
    p.hdr[kHdrPieces] = n_pieces;
    p.hdr[kHdrCutWalks] = n_first;
    p.hdr[kHdrStep] = (int)min(C, (int64_t)INT_MAX);
    p.hdr[kHdrMaxPieces] = kmax;
    p.hdr[kHdrCutSeqs] = n_cut;
  }
}

// Unit and head chunk of this workgroup.  The HG workgroups of a unit (its
// head chunks, which read the same K/V tiles) get linear ids 8 apart: the
// dispatcher deals linear ids to the 8 XCDs in turn, so they share one L2.
// The grid is a whole number of units.
__device__ inline void split_unit_of(int HG, int* unit, int* hp) {
  const int L = blockIdx.x, N = gridDim.x;
  const int M = N / (8 * HG) * (8 * HG);
  const int c = L & 7, k = L >> 3;
  if (L < M) {
    *unit = (k / HG) * 8 + c;
    *hp = k % HG;
  } else {
    *unit = M / HG + (L - M) / HG;
    *hp = (L - M) % HG;
  }
}

template <int D, int HC>
__global__ __launch_bounds__(kWaves * kWave) void split_walk_kernel(PrefillArgs a, PrefillSplit p) {
  __shared__ WalkLds<D, true> lds;
  int U, hp;
  split_unit_of(a.head_groups, &U, &hp);
  if (U >= p.hdr[kHdrUnits]) return;
  const int4 u = p.units[U];
  const int s = u.x, t = u.y, g = u.z, j = u.w >> 16, k = u.w & 0xffff;
  const int q_lo = a.query_start[s];
  const int n = a.query_start[s + 1] - q_lo;
  const int ctx = a.context_lens[s];
  const int64_t st = tile_steps(t, ctx, n, p.tokens_per_wg);
  const int lo = (int)(j * st / k), hi = (int)((j + 1) * st / k);
  WalkOut dst{nullptr, nullptr};
  if (k > 1) {
    const size_t slot = (size_t)U * a.head_groups + hp;
    dst.part = p.part + slot * ((size_t)kSplitRows * D);
    dst.stats = p.stats + slot * kSplitStatFloats;
  }
  walk_rows<D, HC, true>(a, s, g * a.head_groups + hp, t, q_lo, n, ctx, lo, hi, false, dst, lds);
}

// Merge grid: (8 HG, kMergeWalkRows + kMergeSeqRows).  Workgroup (8 hp + rg,
// y < kMergeWalkRows) combines, for head chunk hp and row group rg (32 rows
// over all of D), the pieces of cut walks y, y + kMergeWalkRows, ... (walk w
// = the unit of its first piece); the HG x 8 workgroups of one walk are
// adjacent in the dispatch order.  Rows y >= kMergeWalkRows write the NaN rows
// of sequences out of contract (their first min(n, max_query_len) chunk rows
// inside the output).
constexpr int kMergeWalkRows = 128;
constexpr int kMergeSeqRows = 16;

template <int D, int HC>
__device__ inline void merge_walk(const PrefillArgs& a, const PrefillSplit& p, int x, int hp, int rg) {
  constexpr int DT = D / 16;
  constexpr int TPW = kSplitRows / HC;
  const int tid = threadIdx.x;
  const int4 u = p.units[x];  // piece 0 of the walk
  const int s = u.x, t = u.y, g = u.z, k = u.w & 0xffff;
  const int q_lo = a.query_start[s];
  const int n = a.query_start[s + 1] - q_lo;
  const int T = (n + TPW - 1) / TPW;
  const int c = p.cut_idx[s];
  const int within = (T - 1 - t) * a.num_kv_heads + g;  // the walk's place in each of its pairs
  const int i = tid >> 3, ct = i >> 4, l16 = i & 15, qg = tid & 7;
  const size_t stat_off = ((size_t)(rg * 2 + ct) * 16 + l16) * 2;
  auto slot_of = [&](int j) {
    return (size_t)(p.pair_off[j * p.cut_seq_cap + c] + within) * a.head_groups + hp;
  };
  // Pieces four at a time, every load of a group in flight together, with a
  // running max: the sums are rescaled when a group raises it.  A group's
  // places past the last piece repeat the last piece with weight 0.
  float M = -INFINITY, l = 0.0f;
  f32x4_t acc[D / 32];
#pragma unroll
  for (int q = 0; q < D / 32; ++q) acc[q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  for (int j0 = 0; j0 < k; j0 += 4) {
    size_t sl[4];
    float mj[4], lj[4];
    f32x4_t oj[4][D / 32];
#pragma unroll
    for (int e = 0; e < 4; ++e) sl[e] = slot_of(min(j0 + e, k - 1));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float* st = p.stats + sl[e] * kSplitStatFloats + stat_off;
      mj[e] = st[0];
      lj[e] = st[1];
      const float* po = p.part + sl[e] * ((size_t)kSplitRows * D) + (size_t)rg * (2 * DT * kWave * 4);
#pragma unroll
      for (int q = 0; q < D / 32; ++q) {
        const int d4 = qg + 8 * q;  // 4-dim quad: dims 4 d4 .. = 16 (d4 >> 2) + 4 (d4 & 3) + e
        const int lane = (d4 & 3) * 16 + l16;
        oj[e][q] = *reinterpret_cast<const f32x4_t*>(po + (((size_t)ct * DT + (d4 >> 2)) * kWave + lane) * 4);
      }
    }
    float m4 = mj[0];
#pragma unroll
    for (int e = 1; e < 4; ++e) m4 = fmaxf(m4, mj[e]);
    if (m4 > M) {
      const float r = __builtin_amdgcn_exp2f(M - m4);  // 0 for the first group
      l *= r;
#pragma unroll
      for (int q = 0; q < D / 32; ++q) acc[q] *= r;
      M = m4;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // a piece without keys for this row (max kNoKeysMax) weighs exp2(-1e30 -
      // M) = 0 beside one with keys; a NaN sum propagates
      const float w = j0 + e < k ? __builtin_amdgcn_exp2f(mj[e] - M) : 0.0f;
      l += w * lj[e];
#pragma unroll
      for (int q = 0; q < D / 32; ++q) acc[q] += w * oj[e][q];
    }
  }
  const int tok = t * TPW + (rg / HC) * kRowsPerWave + 16 * ct + l16;
  const int64_t row = (int64_t)q_lo + tok;
  if (tok >= n || row >= a.num_tokens) return;
  const int h = g * a.group + hp * HC + rg % HC;
  float* dst = a.out + ((size_t)row * a.num_heads + h) * D;
  const float inv = 1.0f / l;
#pragma unroll
  for (int q = 0; q < D / 32; ++q) *reinterpret_cast<f32x4_t*>(dst + 4 * (qg + 8 * q)) = acc[q] * inv;
}

template <int D, int HC>
__global__ __launch_bounds__(256) void split_merge_kernel(PrefillArgs a, PrefillSplit p) {
  const int hp = blockIdx.x / (2 * kRowGroups), rg = blockIdx.x % (2 * kRowGroups);
  if ((int)blockIdx.y < kMergeWalkRows) {
    const int walks = p.hdr[kHdrCutWalks];
    for (int x = blockIdx.y; x < walks; x += kMergeWalkRows) merge_walk<D, HC>(a, p, x, hp, rg);
    return;
  }
  const int64_t per_row = (int64_t)a.num_heads * (D / 4);
  for (int s = blockIdx.y - kMergeWalkRows; s < p.num_seqs; s += gridDim.y - kMergeWalkRows) {
    int q_lo, n, ctx;
    if (split_seq_ok(a, p, s, &q_lo, &n, &ctx)) continue;
    const int64_t rows = n < 0 ? 0 : (n < p.max_query_len ? n : p.max_query_len);
    for (int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x; f < rows * per_row; f += 256 * (int64_t)gridDim.x) {
      const int64_t row = (int64_t)q_lo + f / per_row;
      if (row < 0 || row >= a.num_tokens) continue;
      *reinterpret_cast<f32x4_t*>(a.out + row * a.num_heads * D + (f % per_row) * 4) = f32x4_t{NAN, NAN, NAN, NAN};
    }
  }
}


// Chunk write: key/value rows [T, Hkv, D] of the chunk tokens go to the cache
// slots of their positions.  One thread per 16 bytes of one (token, KV head)
// row.
template <int EB, int LAYOUT>
__global__ __launch_bounds__(256) void write_kv_kernel(WriteKvArgs a) {
  constexpr int X = 16 / EB;  // elements per 16 bytes
  const int s = blockIdx.y;
  const int q_lo = a.query_start[s];
  const int n = a.query_start[s + 1] - q_lo;
  const int ctx = a.context_lens[s];
  const int chunks = a.head_size / X;
  const int per_token = a.num_kv_heads * chunks;
  const int flat = blockIdx.x * 256 + threadIdx.x;
  const int i = flat / per_token;
  // a chunk longer than the grid covers (n_s > max_query_len) is out of
  // contract: none of its tokens is written
  const int64_t covered = (int64_t)gridDim.x * 256 / per_token;
  if (i >= n || ctx < 0 || q_lo < 0 || (int64_t)n > covered) return;
  const int rem = flat - i * per_token;
  const int g = rem / chunks;
  const int c = rem - g * chunks;
  const int t = q_lo + i;
  const int64_t pos = (int64_t)ctx + i;
  if (t >= a.num_tokens || pos >= (int64_t)a.max_blocks * kBlockTokens) return;
  const int blk = a.block_tables[(size_t)s * a.max_blocks + (int)(pos / kBlockTokens)];
  if (blk < 0 || (int64_t)blk >= a.num_blocks) return;
  const int slot = (int)(pos % kBlockTokens);
  const size_t src = ((size_t)t * a.num_kv_heads + g) * a.head_size + (size_t)c * X;  // elements
  const size_t tile = ((size_t)blk * a.num_kv_heads + g) * (size_t)kBlockTokens * a.head_size;
  const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(a.key + src * EB);
  const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(a.value + src * EB);
  if (LAYOUT == kKvRows) {
    const size_t dst = tile + (size_t)slot * a.head_size + (size_t)c * X;
    *reinterpret_cast<u32x4_t*>(a.key_cache + dst * EB) = kv;
    *reinterpret_cast<u32x4_t*>(a.value_cache + dst * EB) = vv;
  } else {
    // K [D/X][16][X]: the 16 bytes stay together; V [D][16]: one element per dim
    const size_t kdst = tile + ((size_t)c * kBlockTokens + slot) * X;
    *reinterpret_cast<u32x4_t*>(a.key_cache + kdst * EB) = kv;
    const size_t vdst = tile + (size_t)c * X * kBlockTokens + slot;
    if (EB == 2) {
#pragma unroll
      for (int e = 0; e < X; ++e) {
        const uint32_t w = vv[e / 2];
        reinterpret_cast<uint16_t*>(a.value_cache)[vdst + (size_t)e * kBlockTokens] =
            (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
      }
    } else {
#pragma unroll
      for (int e = 0; e < X; ++e) reinterpret_cast<uint32_t*>(a.value_cache)[vdst + (size_t)e * kBlockTokens] = vv[e];
    }
  }
}

// Launch and return this launch's own status (not a stale error another call
// left on the thread).
template <class Args>
hipError_t launch_args(const void* fn, dim3 grid, dim3 block, const Args& a, hipStream_t stream) {
  void* args[] = {const_cast<Args*>(&a)};
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

template <int D, bool SOLO>
hipError_t launch_prefill_d(const PrefillArgs& a, int hc, dim3 grid, hipStream_t stream) {
  const void* fn = hc == 1   ? reinterpret_cast<const void*>(&prefill_kernel<D, 1, SOLO>)
                   : hc == 2 ? reinterpret_cast<const void*>(&prefill_kernel<D, 2, SOLO>)
                             : reinterpret_cast<const void*>(&prefill_kernel<D, 4, SOLO>);
  return launch_args(fn, grid, dim3(kWaves * kWave), a, stream);
}

// Chunk tokens per workgroup: 32-row groups (8 solo, 4 paired) x 32 tokens / HC.
int tokens_per_wg(int hc, bool solo) { return kRowsPerWave * (solo ? 2 * kRowGroups : kRowGroups) / hc; }

// Whether head size 256 runs the solo layout.  Solo serves 256 rows per
// workgroup and measured 1.42 times the paired layout's rate (8192 new tokens
// over 32768, 24 query / 4 KV heads: 1090 against 770 TFLOP/s, both with fp16
// P.V), but its workgroups are twice as large, so fewer of them share the
// longest chunk.  Rule: solo unless rounding the longest chunk's workgroups
// up to whole rounds of the compute units costs more than the rate gains.
// On a 4-sequence batch whose longest chunk gives 288 solo workgroups (two
// rounds of 256) against 576 paired ones (three), solo measured 691 to 699
// against 649 TFLOP/s; paired stays where its whole grid fits one round.
bool solo_at_256(int max_query_len, int hc, int y, int cus) {
  const int64_t np = (int64_t)((max_query_len + tokens_per_wg(hc, false) - 1) / tokens_per_wg(hc, false)) * y;
  const int64_t ns = (int64_t)((max_query_len + tokens_per_wg(hc, true) - 1) / tokens_per_wg(hc, true)) * y;
  const int64_t rp = (np + cus - 1) / cus, rs = (ns + cus - 1) / cus;
  return rs * 2 * 100 <= rp * 142;
}

}  // namespace

int prefill_heads_per_wg(int group) {
  // the largest of 4, 2, 1 that divides the group: the workgroup's waves are
  // (head, 32-token group) pairs of one KV head
  return group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
}

bool prefill_solo(int head_size, int group, int num_kv_heads, int max_query_len) {
  if (head_size <= 128) return true;
  const int hc = prefill_heads_per_wg(group);
  return solo_at_256(max_query_len, hc, num_kv_heads * (group / hc), device_cus());
}

int prefill_tokens_per_wg(int group, bool solo) { return tokens_per_wg(prefill_heads_per_wg(group), solo); }

namespace {

// The kernels' view of the arguments: head groups per KV head, and the scale.
// The kernels apply the scale in the exp2 argument and take maxima over the
// raw logits, which needs a positive scale: a negative one moves onto the
// query's sign, and 0 becomes the smallest normal float (for logits below
// 2^100 in magnitude every weight is then exp2 of less than 2^-26, which
// rounds to 1, as with 0).
PrefillArgs kernel_args(const PrefillArgs& args) {
  PrefillArgs a = args;
  a.head_groups = a.group / prefill_heads_per_wg(a.group);
  const float qs = args.qscale * kLog2e;
  a.negate_q = qs < 0.0f ? 1 : 0;
  a.qscale = qs < 0.0f ? -qs : (qs > 0.0f ? qs : 1.17549435e-38f);
  return a;
}

const void* split_walk_fn(int head_size, int hc) {
#define PAD_SPLIT_FN(DD)                                                                  \
  (hc == 1   ? reinterpret_cast<const void*>(&split_walk_kernel<DD, 1>)                  \
   : hc == 2 ? reinterpret_cast<const void*>(&split_walk_kernel<DD, 2>)                  \
             : reinterpret_cast<const void*>(&split_walk_kernel<DD, 4>))
  return head_size == 64 ? PAD_SPLIT_FN(64) : head_size == 128 ? PAD_SPLIT_FN(128) : PAD_SPLIT_FN(256);
#undef PAD_SPLIT_FN
}

const void* split_merge_fn(int head_size, int hc) {
#define PAD_MERGE_FN(DD)                                                                  \
  (hc == 1   ? reinterpret_cast<const void*>(&split_merge_kernel<DD, 1>)                 \
   : hc == 2 ? reinterpret_cast<const void*>(&split_merge_kernel<DD, 2>)                 \
             : reinterpret_cast<const void*>(&split_merge_kernel<DD, 4>))
  return head_size == 64 ? PAD_MERGE_FN(64) : head_size == 128 ? PAD_MERGE_FN(128) : PAD_MERGE_FN(256);
#undef PAD_MERGE_FN
}

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of a split launch.  Bounds (rounds = kSplitRounds x N, C >= the
// total steps / rounds; walks W = S x Hkv x ceil(max_query_len / TPW) at
// most): a cut walk has more than C steps, so fewer than rounds / HG walks
// are cut, in fewer than rounds / (Hkv HG) sequences; a cut walk's k =
// ceil(steps / C) pieces number under 2 steps / C, and, as C >= 16, at most
// ceil(Lmax / 16) (Lmax = the longest walk the block table allows; none is
// cut below 17 steps) and kSplitMaxPieces: fewer than min(2 rounds / HG,
// kmax W) pieces.
struct SplitLayout {
  int64_t units_cap, cut_seq_cap, slots_cap;
  size_t units, order, cut_idx, cut_seq, pair_off, stats, part, bytes;
};
SplitLayout split_layout(int num_seqs, int num_kv_heads, int group, int head_size, int max_query_len, int max_blocks,
                         int ranges) {
  const int64_t hg = group / prefill_heads_per_wg(group);
  const int64_t tpw = tokens_per_wg(prefill_heads_per_wg(group), true);
  const int64_t rounds = (int64_t)kSplitRounds * ranges;
  SplitLayout l;
  const int64_t walks = (int64_t)num_seqs * num_kv_heads * ((max_query_len + tpw - 1) / tpw);
  const int64_t longest = ((int64_t)max_blocks * kBlockTokens + 31) / 32;
  const int64_t kmax = longest > kSplitMinSteps
                           ? std::min<int64_t>(kSplitMaxPieces, (longest + kSplitMinSteps - 1) / kSplitMinSteps)
                           : 0;
  const int64_t pieces = std::min<int64_t>(2 * rounds / hg + 2, kmax * walks);
  l.units_cap = walks + pieces;
  l.cut_seq_cap = std::min<int64_t>(num_seqs, rounds / (hg * num_kv_heads) + 1);
  l.slots_cap = pieces * hg;
  l.units = 256;  // the header
  l.order = l.units + align256((size_t)l.units_cap * 16);
  l.cut_idx = l.order + align256((size_t)num_seqs * 4);
  l.cut_seq = l.cut_idx + align256((size_t)num_seqs * 4);
  l.pair_off = l.cut_seq + align256((size_t)l.cut_seq_cap * 4);
  l.stats = l.pair_off + align256((size_t)kSplitMaxPieces * l.cut_seq_cap * 4);
  l.part = l.stats + align256((size_t)l.slots_cap * kSplitStatFloats * 4);
  l.bytes = l.part + (size_t)l.slots_cap * kSplitRows * head_size * 4;
  return l;
}

}  // namespace

int prefill_split_ranges(int head_size, int group) {
  // resident walk workgroups per CU, per device, head size and head chunk
  // (queried once: the occupancy query costs microseconds of host time)
  static std::atomic<int> cache[64][3][3];
  const int hc = prefill_heads_per_wg(group);
  const int di = head_size == 64 ? 0 : head_size == 128 ? 1 : 2, ci = hc == 1 ? 0 : hc == 2 ? 1 : 2;
  int dev = 0;
  const bool cacheable = hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64;
  if (!cacheable) (void)hipGetLastError();
  int per_cu = cacheable ? cache[dev][di][ci].load(std::memory_order_relaxed) : 0;
  if (per_cu <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, split_walk_fn(head_size, hc), kWaves * kWave, 0) !=
            hipSuccess ||
        per_cu < 1) {
      (void)hipGetLastError();  // our own failed query: do not leave it behind
      per_cu = 1;
    } else if (cacheable) {
      cache[dev][di][ci].store(per_cu, std::memory_order_relaxed);
    }
  }
  return per_cu * device_cus();
}

size_t prefill_split_workspace_bytes(int num_seqs, int num_kv_heads, int group, int head_size, int max_query_len,
                                     int max_blocks, int ranges) {
  return split_layout(num_seqs, num_kv_heads, group, head_size, max_query_len, max_blocks, ranges).bytes;
}

bool prefill_split_pays(const int32_t* context_lens, const int32_t* query_lens, int num_seqs, int num_kv_heads,
                        int group, int ranges) {
  const int64_t hg = group / prefill_heads_per_wg(group);
  const int64_t tpw = tokens_per_wg(prefill_heads_per_wg(group), true);
  int64_t total = 0, longest = 0;
  int busy = 0;  // sequences with chunk tokens
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t ctx = context_lens[s], n = query_lens[s];
    if (n <= 0) continue;
    ++busy;
    total += seq_walk_steps(ctx, n, tpw);
    longest = std::max(longest, tile_steps((n + tpw - 1) / tpw - 1, ctx, n, tpw));
  }
  // a batch: the split's longest-first unit list beat the plain launch's
  // order; one sequence: only when the plan would cut a walk (its rule)
  return busy > 1 || longest * kSplitShare * ranges > total * num_kv_heads * hg;
}

int64_t prefill_split_grid(int num_seqs, int num_kv_heads, int group, int max_query_len, int max_blocks,
                           int ranges) {
  const SplitLayout l = split_layout(num_seqs, num_kv_heads, group, 256, max_query_len, max_blocks, ranges);
  return l.units_cap * (group / prefill_heads_per_wg(group));
}

hipError_t launch_prefill_split(const PrefillArgs& args, int num_seqs, int max_query_len, int head_size,
                                int ranges, void* workspace, hipStream_t stream) {
  if (num_seqs == 0) return hipSuccess;
  const PrefillArgs a = kernel_args(args);
  const int hc = prefill_heads_per_wg(a.group);
  const SplitLayout l = split_layout(num_seqs, a.num_kv_heads, a.group, head_size, max_query_len, a.max_blocks,
                                     ranges);
  char* base = static_cast<char*>(workspace);
  PrefillSplit p{};
  p.hdr = reinterpret_cast<int32_t*>(base);
  p.units = reinterpret_cast<int4*>(base + l.units);
  p.order = reinterpret_cast<int32_t*>(base + l.order);
  p.cut_idx = reinterpret_cast<int32_t*>(base + l.cut_idx);
  p.cut_seq = reinterpret_cast<int32_t*>(base + l.cut_seq);
  p.pair_off = reinterpret_cast<int32_t*>(base + l.pair_off);
  p.stats = reinterpret_cast<float*>(base + l.stats);
  p.part = reinterpret_cast<float*>(base + l.part);
  p.num_seqs = num_seqs;
  p.max_query_len = max_query_len;
  p.ranges = ranges;
  p.tokens_per_wg = tokens_per_wg(hc, true);
  p.cut_seq_cap = (int)l.cut_seq_cap;
  void* kargs[] = {const_cast<PrefillArgs*>(&a), &p};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&split_plan_kernel), dim3(1),
                                 dim3(kSplitPlanThreads), kargs, 0, stream);
  if (e != hipSuccess) return e;
  e = hipLaunchKernel(split_walk_fn(head_size, hc), dim3((unsigned)(l.units_cap * a.head_groups)),
                      dim3(kWaves * kWave), kargs, 0, stream);
  if (e != hipSuccess) return e;
  const unsigned seq_rows = (unsigned)std::min(num_seqs, kMergeSeqRows);
  return hipLaunchKernel(split_merge_fn(head_size, hc),
                         dim3((unsigned)(2 * kRowGroups * a.head_groups), kMergeWalkRows + seq_rows), dim3(256),
                         kargs, 0, stream);
}

hipError_t launch_prefill(const PrefillArgs& args, int num_seqs, int max_query_len, int head_size,
                          hipStream_t stream) {
  const PrefillArgs a = kernel_args(args);
  const int hc = prefill_heads_per_wg(a.group);
  const bool solo = prefill_solo(head_size, a.group, a.num_kv_heads, max_query_len);
  const int tpw = prefill_tokens_per_wg(a.group, solo);
  const int tiles = (max_query_len + tpw - 1) / tpw;
  if (num_seqs == 0 || tiles == 0) return hipSuccess;
  const dim3 grid(tiles, a.num_kv_heads * a.head_groups, num_seqs);
  switch (head_size) {
    case 64: return launch_prefill_d<64, true>(a, hc, grid, stream);
    case 128: return launch_prefill_d<128, true>(a, hc, grid, stream);
    default:
      return solo ? launch_prefill_d<256, true>(a, hc, grid, stream) : launch_prefill_d<256, false>(a, hc, grid, stream);
  }
}

hipError_t launch_write_kv(const WriteKvArgs& a, int num_seqs, int max_query_len, int elem_bytes, int layout,
                           hipStream_t stream) {
  const int per_token = a.num_kv_heads * (a.head_size * elem_bytes / 16);
  const int64_t threads = (int64_t)max_query_len * per_token;
  if (num_seqs == 0 || threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256), num_seqs);
  const void* fn = elem_bytes == 2 ? (layout == kKvRows ? reinterpret_cast<const void*>(&write_kv_kernel<2, kKvRows>)
                                                         : reinterpret_cast<const void*>(&write_kv_kernel<2, kKvTiled>))
                                   : (layout == kKvRows ? reinterpret_cast<const void*>(&write_kv_kernel<4, kKvRows>)
                                                        : reinterpret_cast<const void*>(&write_kv_kernel<4, kKvTiled>));
  return launch_args(fn, grid, dim3(256), a, stream);
}

}  // namespace pad
