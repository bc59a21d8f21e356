// Attention kernel template for paged single-token decode on CDNA4 (gfx950).
// Included by the pad_attn_*.hip translation units, each of which
// instantiates one (element type, split/one-pass, layout) family.
//
// Split form (second page, "V2 implementation" message; first page, two-pass
// message):
//   phase 1  one workgroup per (sequence, KV head [, head chunk], partition):
//            Q.K^T over the partition's tokens, the partition max and
//            exp-sum, and the normalised partial P.V (this kernel, kSplit);
//   phase 2  the log-sum-exp merge (merge_kernel in pad_kernels.hip).
// One-pass form: one workgroup per (sequence, KV head [, head chunk]) walks
// the whole context with an online softmax and writes the output directly
// (this kernel, !kSplit).
//
// Work decomposition inside a workgroup.  Its NW waves share the workgroup's
// token range; wave w takes blocks w, w+NW, w+2NW, ...  Each wave keeps its
// own running max m, exp-sum l and P.V accumulator for the group's query
// heads, so the main loop has no barrier; waves are merged at the end (a
// log2(NW)-step tree through LDS, fixed order, so results are bitwise
// repeatable).
//
// Two cache layouts (second page, hardware-test message, lists both):
//   rows   K and V [blocks, kv_heads, block_size, D]: every token's row is
//          contiguous.
//   tiled  K [blocks, kv_heads, D/x, block_size, x] with x = 16 bytes of
//          elements, V [blocks, kv_heads, D, block_size].
// Per 16-token block a wave:
//   * loads the block's K and V tile (8 KB each for bf16 D=256) with buffer
//     loads bounded to the tile (a block id outside the pool reads nothing);
//   * forms the 16 tokens x 16 heads logit tile on the matrix cores: A = K
//     (rows = tokens), B = Q^T (columns = the group's heads), contracting over
//     D.  Lane l supplies token l%16 and one 16-byte run of dims, exactly one
//     16-byte load: in the tiled layout the runs of one MFMA step are a
//     contiguous 1 KB, in the rows layout 16 rows x 64 B;
//   * updates the running max per head (a 4-lane shuffle reduction) and turns
//     the logits into exp2 weights p, still in the tile layout: lane l holds
//     tokens 4*(l/16)+i of head l%16;
//   * accumulates P.V:
//       tiled: on the matrix cores.  That p layout is the A operand of a
//       16x16x16 bf16 MFMA (rows = heads, k = tokens), and a V load of 8 bytes
//       (4 consecutive tokens of one dim) is its B operand, so nothing moves
//       through LDS.  p is split into bf16 hi + lo parts (two MFMAs), which
//       keeps ~2^-17 relative precision; fp32 caches use the fp32 MFMA on p
//       directly.
//       rows: on the vector ALUs in fp32: p goes through a 1 KB per-wave LDS
//       tile, lane l owns a 16-byte run of dims of one token per V load.
//     Tail tokens of the last block are masked by select: logits to -inf,
//     and (tiled) their V elements to zero before the MFMA, so NaN padding
//     never reaches the output.
// Loads run up to R-1 blocks ahead of the arithmetic through a register ring.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "pad_internal.h"
#include "pad_lane_ops.h"

namespace pad {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;
// Buffer resource word 3 for CDNA: raw 32-bit data format, bounds checked
// against num_records in bytes.
constexpr int kRsrcWord3 = 0x00020000;

struct F32 {
  static constexpr int kBytes = 4;
};
struct BF16 {
  static constexpr int kBytes = 2;
};

// Geometry of one (block, KV head) tile: 16 token rows of D elements.
template <class DT, int D>
struct Geom {
  static constexpr int kRowBytes = D * DT::kBytes;
  static constexpr int kTileBytes = kBlockTokens * kRowBytes;
  // K: one load step covers 16 rows x 64 bytes (4 lane groups x 16 B).
  static constexpr int kSteps = kRowBytes / 64;
  // V: lanes per token row (16 B each), rows per wave load, loads per tile.
  static constexpr int kLanesPerRow = kRowBytes / 16;
  static constexpr int kRowsPerLoad = kWave / kLanesPerRow;
  static constexpr int kVLoads = kBlockTokens / kRowsPerLoad;
  static constexpr int kElemsPerLane = 16 / DT::kBytes;
  static_assert(kVLoads == kSteps, "K and V load counts agree");
  static_assert(kRowsPerLoad >= 1, "row fits in a wave");
};

struct AttnParams {
  const char* query;
  const char* key_cache;
  const char* value_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* out;         // one-pass output [S, H, D], rows of sequence s at s * out_stride
  int64_t q_stride;   // elements between consecutive sequences' query rows (>= H * D)
  int64_t out_stride; // floats between consecutive sequences' output rows (>= H * D)
  float* max_logits;  // split workspace
  float* exp_sums;
  float* tmp_out;
  int64_t num_blocks;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int group;
  int head_chunks;
  int max_blocks;
  int partition;       // tokens per partition (split)
  int num_partitions;  // NP (split)
  float qscale;        // scale * log2(e)
  // balanced split (balanced == 0: one workgroup per partition)
  unsigned* info;      // launch info (N, B, block prefix) published by workgroup 0
  int gy_count;        // head groups per sequence (num_kv_heads * head_chunks)
  int balanced;
  int num_cus;         // compute units of the device
};

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A pointer every lane agrees on, moved to scalar registers.
__device__ inline void* uniform_ptr(const char* ptr) {
  const uint64_t a = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
}

__device__ inline float readlane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// One 16x16 logit tile step: C += A(K rows) * B(Q^T columns) over one
// 16-byte run per lane.
__device__ inline f32x4_t qk_step(BF16, u32x4_t k, u32x4_t q, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k), __builtin_bit_cast(bf16x8_t, q),
                                                 c, 0, 0, 0);
}
// (The whole vector is reinterpreted before indexing: a bit_cast of one
// element of an ext-vector lvalue reads element 0 with this compiler.)
__device__ inline f32x4_t qk_step(F32, u32x4_t k, u32x4_t q, f32x4_t c) {
  const f32x4_t kf = __builtin_bit_cast(f32x4_t, k);
  const f32x4_t qf = __builtin_bit_cast(f32x4_t, q);
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[j], qf[j], c, 0, 0, 0);
  return c;
}

// 16 bytes of V -> fp32 elements (the low half of each word is the lower address).
__device__ inline void widen(BF16, u32x4_t w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}
__device__ inline void widen(F32, u32x4_t w, float* f) {
  const f32x4_t v = __builtin_bit_cast(f32x4_t, w);
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = v[i];
}

// Cache layouts of the K and V pools.
constexpr int kLayoutRows = 0;
// Log2 headroom of the lazy softmax reference (weights stay <= 2^8).
constexpr float kLazyLog2 = 8.0f;

// Build-time tuning knobs (defaults are the tuned values).
#ifndef PAD_RING_MAX
// most blocks a wave keeps in flight; 0: by layout and head size.  Tiled
// layout: 2 at head size 256 (3 measured slower on the 100K step) and 4
// below, where a block is 8 KB or less (at 100K tokens, 64 / 8 heads of 64:
// 57.1 against 48.1 us per step; 32 / 8 heads of 128: 74.6 against 73.4 us;
// 8 was slower than 4 at both).  Rows layout: 2 (4 spills registers at head
// size 128).
#define PAD_RING_MAX 0
#endif
#ifndef PAD_SPLIT_WAVES
#define PAD_SPLIT_WAVES 1  // waves per phase-1 workgroup
#endif
#ifndef PAD_KV_LOAD_POLICY
// cache-policy bits of the K/V buffer loads: non-temporal (each byte is read
// once; measured ~11 % faster than the default policy on the 100K workload)
#define PAD_KV_LOAD_POLICY 2
#endif
constexpr int kLayoutTiled = 1;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;

// Where lane `lane` finds its pieces of one tile, per layout.
template <class DT, int D, int LAYOUT>
struct TileMap {
  using G_ = Geom<DT, D>;
  static constexpr bool kMfmaPV = LAYOUT == kLayoutTiled;
  // K: kSteps 16-byte loads per lane; step s covers dims [32 s, 32 s + 32)
  // (bf16) of all 16 tokens
  __device__ static int k_off(int lane) {
    return LAYOUT == kLayoutTiled ? 16 * lane : (lane & 15) * G_::kRowBytes + 16 * (lane >> 4);
  }
  static constexpr int kKStepBytes = LAYOUT == kLayoutTiled ? 1024 : 64;
  // V: rows layout, kSteps 16-byte loads (1 KB contiguous per wave load);
  // tiled layout, one load per 16-dim slice: 4 tokens of one dim per lane
  // (8 bytes bf16, 16 bytes fp32)
  static constexpr int kVLoads = LAYOUT == kLayoutTiled ? D / 16 : G_::kSteps;
  static constexpr int kVBytes = (LAYOUT == kLayoutTiled && DT::kBytes == 2) ? 8 : 16;
  using VReg = typename std::conditional<kVBytes == 8, u32x2_t, u32x4_t>::type;
  __device__ static int v_off(int lane) {
    if (LAYOUT != kLayoutTiled) return 16 * lane;
    // dim-major tile [D][16 tokens]: dim (lane%16), tokens 4*(lane/16) ...
    return (lane & 15) * kBlockTokens * DT::kBytes + 4 * DT::kBytes * (lane >> 4);
  }
  static constexpr int kVLoadStride = LAYOUT == kLayoutTiled ? 16 * kBlockTokens * DT::kBytes : 1024;
  static constexpr int kStageVgprs = G_::kSteps * 4 + kVLoads * kVBytes / 4;
  // accumulator registers per lane
  template <int GH>
  static constexpr int acc_vgprs() { return kMfmaPV ? (D / 16) * 4 : GH * G_::kElemsPerLane; }
  // blocks in flight per wave: as many (up to 3) as fit next to the Q operand
  // and the accumulator in ~400 of the 512 registers one wave per SIMD owns
  template <int GH>
  static constexpr int ring() {
    constexpr int cap = PAD_RING_MAX ? PAD_RING_MAX : (LAYOUT == kLayoutTiled && D < 256 ? 4 : 2);
    constexpr int fixed = G_::kSteps * 4 + acc_vgprs<GH>() + 48;
    constexpr int r = (400 - fixed) / kStageVgprs;
    return r < 1 ? 1 : (r > cap ? cap : r);
  }
};

template <int N>
__device__ inline u32x4_t buffer_load(__amdgpu_buffer_rsrc_t r, int off, u32x4_t*) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, PAD_KV_LOAD_POLICY);
}
template <int N>
__device__ inline u32x2_t buffer_load(__amdgpu_buffer_rsrc_t r, int off, u32x2_t*) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, PAD_KV_LOAD_POLICY);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ inline uint32_t bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// P.V step of the tiled layout for one 16-dim slice: C[head][dim] += sum over
// the block's 16 tokens of p[head][token] * V[token][dim].
__device__ inline f32x4_t pv_step(BF16, s16x4_t p_hi, s16x4_t p_lo, const float*, u32x2_t v, f32x4_t c) {
  const s16x4_t vb = __builtin_bit_cast(s16x4_t, v);
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p_hi, vb, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p_lo, vb, c, 0, 0, 0);
}
__device__ inline f32x4_t pv_step(F32, s16x4_t, s16x4_t, const float* p, u32x4_t v, f32x4_t c) {
  const f32x4_t vf = __builtin_bit_cast(f32x4_t, v);
#pragma unroll
  for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(p[i], vf[i], c, 0, 0, 0);
  return c;
}

// Zero the V elements of tokens >= rows (lane holds tokens 4*(lane/16)+e).
__device__ inline u32x2_t mask_tail(u32x2_t v, int t0, int rows) {
  const uint32_t m0 = (t0 < rows ? 0xffffu : 0u) | (t0 + 1 < rows ? 0xffff0000u : 0u);
  const uint32_t m1 = (t0 + 2 < rows ? 0xffffu : 0u) | (t0 + 3 < rows ? 0xffff0000u : 0u);
  return u32x2_t{v[0] & m0, v[1] & m1};
}
__device__ inline u32x4_t mask_tail(u32x4_t v, int t0, int rows) {
  return u32x4_t{t0 < rows ? v[0] : 0u, t0 + 1 < rows ? v[1] : 0u, t0 + 2 < rows ? v[2] : 0u,
                 t0 + 3 < rows ? v[3] : 0u};
}

// One wave's walk over a range of blocks for one (sequence, KV head, head
// chunk): its running max, exp-sum and P.V accumulator, plus the flag of a
// block id outside the pool.
template <class DT, int D, int GH, int NW, int LAYOUT>
struct Walker {
  using G_ = Geom<DT, D>;
  using TM = TileMap<DT, D, LAYOUT>;
  using VReg = typename TM::VReg;
  static constexpr bool kMfmaPV = TM::kMfmaPV;
  static constexpr int R = TM::template ring<GH>();
  static constexpr int kSteps = G_::kSteps;
  static constexpr int kVLoads = TM::kVLoads;
  static constexpr int LPR = G_::kLanesPerRow;
  static constexpr int RPL = G_::kRowsPerLoad;
  static constexpr int EPL = G_::kElemsPerLane;
  static constexpr int kSlices = D / 16;                               // tiled: 16-dim output slices
  static constexpr int kRowsHeld = kMfmaPV ? kMaxHeadsPerGroup : GH;   // head rows an accumulator covers
  static constexpr int kPTile = kMfmaPV ? 0 : kBlockTokens * kMaxHeadsPerGroup;  // floats per wave

  struct Stage {
    u32x4_t k[kSteps];
    VReg v[kVLoads];
  };

  int lane;
  int rbase;  // first of the lane's 4 tokens in the logit tile
  u32x4_t qop[kSteps];
  // Online softmax with a lazy reference: p = exp2(x - m_run) where m_run is
  // raised (and the accumulators rescaled) only when a block's max exceeds it
  // by more than kLazyLog2, so p <= 2^kLazyLog2 and rescaling is rare.  The
  // result does not depend on the reference; m_true keeps the exact max.
  float m_run;   // reference max (log2 units) of head column lane%16
  float m_true;  // running max of that head's logits (log2 units)
  float l_run;   // this lane's share of that head's exp-sum, relative to m_run
  // P.V accumulator.  rows: acc[h][e] = head h, dim EPL*(lane%LPR)+e, summed
  // over this lane's tokens.  tiled: accm[j][i] = head rbase+i, dim 16 j + lane%16.
  float acc[kMfmaPV ? 1 : GH][EPL];
  f32x4_t accm[kMfmaPV ? kSlices : 1];
  bool bad;

  __device__ explicit Walker(int lane_) : lane(lane_), rbase(4 * (lane_ >> 4)) {}

  // Q^T operand: lane l supplies head column l%16 and the 16-byte run of dims
  // that the same lane's K load holds.
  __device__ void load_q(const AttnParams& p, int s, int h0, int gc) {
    const int qh = lane & 15;
    const char* qrow = p.query + ((size_t)s * (size_t)p.q_stride + (size_t)(h0 + qh) * D) * DT::kBytes + 16 * (lane >> 4);
#pragma unroll
    for (int st = 0; st < kSteps; ++st)
      qop[st] = (qh < gc) ? *reinterpret_cast<const u32x4_t*>(qrow + 64 * st) : u32x4_t{0, 0, 0, 0};
  }

  __device__ void reset() {
    m_run = -INFINITY;
    m_true = -INFINITY;
    l_run = 0.0f;
#pragma unroll
    for (int h = 0; h < (kMfmaPV ? 1 : GH); ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
#pragma unroll
    for (int j = 0; j < (kMfmaPV ? kSlices : 1); ++j) accm[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    bad = false;
  }

  // Multiply the accumulator rows of head h by the factor lane h holds.
  __device__ void scale_heads(float f) {
    if constexpr (kMfmaPV) {
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = __shfl(f, rbase + i);
#pragma unroll
      for (int j = 0; j < kSlices; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) accm[j][i] *= a[i];
    } else {
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        const float a = readlane_f(f, h);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= a;
      }
    }
  }

  // Blocks [blk_begin, blk_end) of sequence s (L tokens), KV head g; wave
  // `wave` of NW takes blocks blk_begin + wave, + NW, ...
  __device__ void walk(const AttnParams& p, int s, int g, int L, int blk_begin, int blk_end, int wave,
                       float* ptile) {
    const int32_t* table_row = p.block_tables + (size_t)s * p.max_blocks;
    const size_t head_off = (size_t)g * G_::kTileBytes;
    const size_t block_stride = (size_t)p.num_kv_heads * G_::kTileBytes;
    const int koff = TM::k_off(lane);
    const int voff = TM::v_off(lane);

    for (int seg = blk_begin; seg < blk_end; seg += kWave * NW) {
      const int seg_end = min(seg + kWave * NW, blk_end);
      const int first = seg + wave;
      const int n = first < seg_end ? (seg_end - first + NW - 1) / NW : 0;
      const int my_id = lane < n ? table_row[first + NW * lane] : -1;

      // Enqueue the loads of the wave's idx-th block (zero-length, no traffic,
      // past the wave's last block).
      auto issue = [&](Stage& st, int idx) {
        const bool live = idx < n;
        int phys = live ? __builtin_amdgcn_readlane(my_id, idx) : 0;
        const int blk = first + NW * idx;
        int rows = live ? min(kBlockTokens, L - blk * kBlockTokens) : 0;
        const bool ok = phys >= 0 && (int64_t)phys < p.num_blocks;
        bad |= live && !ok;
        if (!ok) {
          phys = 0;
          rows = 0;
        }
        const size_t base = (size_t)phys * block_stride + head_off;
        // rows layout: the bound drops the tail rows; tiled layout interleaves
        // tokens, so the whole tile is read and the tail is masked by select
        const int bytes = __builtin_amdgcn_readfirstlane(
            LAYOUT == kLayoutTiled ? (rows > 0 ? G_::kTileBytes : 0) : rows * G_::kRowBytes);
        __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(p.key_cache + base), (short)0, bytes, kRsrcWord3);
        __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(p.value_cache + base), (short)0, bytes, kRsrcWord3);
#pragma unroll
        for (int j = 0; j < kSteps; ++j)
          st.k[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff + TM::kKStepBytes * j, 0, PAD_KV_LOAD_POLICY);
#pragma unroll
        for (int j = 0; j < kVLoads; ++j)
          st.v[j] = buffer_load<0>(rv, voff + TM::kVLoadStride * j, static_cast<VReg*>(nullptr));
      };

      auto compute = [&](const Stage& st, int blk) {
        // logits: lane l holds tokens rbase+i of the block for head column l%16
        f32x4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < kSteps; ++j) c = qk_step(DT{}, st.k[j], qop[j], c);
        const int rows = min(kBlockTokens, L - blk * kBlockTokens);
        float x[4];
        float bm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = (rbase + i < rows) ? c[i] * p.qscale : -INFINITY;
          bm = fmaxf(bm, x[i]);
        }
        // lanes l, l^16, l^32, l^48 share a head column
        bm = group_max(bm);
        m_true = fmaxf(m_true, bm);
        if (__ballot(bm > m_run + kLazyLog2) != 0) {
          // raise the reference of every head to its running max
          const float m_new = fmaxf(m_run, bm);
          const float alpha = fast_exp2(m_run - m_new);  // 0 on the first block
          l_run *= alpha;
          m_run = m_new;
          scale_heads(alpha);
        }
        float pw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pw[i] = fast_exp2(x[i] - m_run);
          l_run += pw[i];
        }
        if constexpr (kMfmaPV) {
          s16x4_t p_hi = {0, 0, 0, 0}, p_lo = {0, 0, 0, 0};
          if constexpr (DT::kBytes == 2) {
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              hi[i] = bf16_rne(pw[i]);
              lo[i] = bf16_rne(pw[i] - __builtin_bit_cast(float, hi[i] << 16));
            }
            p_hi = __builtin_bit_cast(s16x4_t, u32x2_t{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)});
            p_lo = __builtin_bit_cast(s16x4_t, u32x2_t{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)});
          }
          // V of tail tokens (padding, possibly NaN) is zeroed: 0 * NaN would poison the sum
#pragma unroll
          for (int j = 0; j < kVLoads; ++j)
            accm[j] = pv_step(DT{}, p_hi, p_lo, pw, mask_tail(st.v[j], rbase, rows), accm[j]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) ptile[(rbase + i) * kMaxHeadsPerGroup + (lane & 15)] = pw[i];
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int j = 0; j < kSteps; ++j) {
            const int r = RPL * j + lane / LPR;
            float pr[GH];
#pragma unroll
            for (int h = 0; h < GH; ++h) pr[h] = ptile[r * kMaxHeadsPerGroup + h];
            float vf[EPL];
            widen(DT{}, st.v[j], vf);
#pragma unroll
            for (int h = 0; h < GH; ++h)
#pragma unroll
              for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pr[h], vf[e], acc[h][e]);
          }
          __builtin_amdgcn_wave_barrier();
        }
      };

      Stage ring[R];
#pragma unroll
      for (int r = 0; r < R; ++r) issue(ring[r], r);
      for (int i = 0; i < n; i += R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int idx = i + r;
          if (idx < n) compute(ring[r], first + NW * idx);
          issue(ring[r], idx + R);
        }
      }
    }
  }

  // Wave totals: fold the token groups of acc (rows) and the 4 lanes of l.
  __device__ void fold() {
    if constexpr (!kMfmaPV) {
#pragma unroll
      for (int off = LPR; off < kWave; off <<= 1)
#pragma unroll
        for (int h = 0; h < GH; ++h)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
    }
    l_run = group_sum(l_run);
  }

  // Normalised rows of heads [0, gc): store(h, d, value) with value scaled by
  // the factor lane h holds.
  template <class Store>
  __device__ void write_rows(int gc, float inv_of_lane, Store store) const {
    if constexpr (kMfmaPV) {
      // lane l: heads rbase+i, dims 16 j + lane%16
      float inv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) inv[i] = __shfl(inv_of_lane, rbase + i);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = rbase + i;
        if (h < gc) {
#pragma unroll
          for (int j = 0; j < kSlices; ++j) store(h, 16 * j + (lane & 15), accm[j][i] * inv[i]);
        }
      }
    } else {
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        if (h >= gc) continue;
        const float inv = readlane_f(inv_of_lane, h);
        if (lane < LPR) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) store(h, EPL * lane + e, acc[h][e] * inv);
        }
      }
    }
  }
};



// One unit of phase-1 work for a workgroup: blocks [b0, b1) of sequence s,
// KV head g, query heads [h0, h0 + gc); its entry goes to partition slot
// `part` (split) or to the output (one-pass).
struct WorkItem {
  int s, g, h0, gc, L, part, b0, b1;
  bool len_ok;
};

__device__ inline WorkItem make_item(const AttnParams& p, int s, int gy, int part) {
  WorkItem it;
  it.s = s;
  it.g = gy / p.head_chunks;
  const int chunk = gy - it.g * p.head_chunks;
  it.h0 = it.g * p.group + chunk * kMaxHeadsPerGroup;
  it.gc = min(kMaxHeadsPerGroup, p.group - chunk * kMaxHeadsPerGroup);
  it.L = p.seq_lens[s];
  it.len_ok = it.L >= 0 && it.L <= p.max_blocks * kBlockTokens;
  it.part = part;
  it.b0 = 0;
  it.b1 = 0;
  return it;
}

// The result of one wave's walk (after fold), written where the item says:
// split, the entry (max logit in natural-log units, exp-sum relative to it,
// normalised row per query head) in partition slot it.part; one-pass, the
// output rows.  A block id outside the pool (w.bad) makes the rows and the
// max NaN.
template <class W_, int D, bool kSplit>
__device__ inline void write_result(const AttnParams& p, const W_& w, const WorkItem& it) {
  constexpr bool kMfmaPV = W_::kMfmaPV;
  constexpr int EPL = W_::EPL;
  constexpr int LPR = W_::LPR;
  const int lane = w.lane;
  const int H = p.num_heads;
  const float nan = __builtin_nanf("");
  const float inv = w.bad ? nan : 1.0f / w.l_run;
  const size_t hstride = kSplit ? (size_t)p.num_partitions * D : (size_t)D;
  float* base = p.out + (size_t)it.s * (size_t)p.out_stride + (size_t)it.h0 * D;
  if constexpr (kSplit) base = p.tmp_out + ((size_t)it.s * H + it.h0) * hstride + (size_t)it.part * D;
  if constexpr (kMfmaPV) {
    w.write_rows(it.gc, inv, [&](int h, int d, float v) { base[h * hstride + d] = v; });
  } else {
    // four consecutive dims per store
#pragma unroll
    for (int h = 0; h < W_::kRowsHeld; ++h) {
      if (h >= it.gc) continue;
      const float ih = readlane_f(inv, h);
      if (lane < LPR) {
        float* dst = base + h * hstride + EPL * lane;
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
          *reinterpret_cast<f32x4_t*>(dst + e) =
              f32x4_t{w.acc[h][e] * ih, w.acc[h][e + 1] * ih, w.acc[h][e + 2] * ih, w.acc[h][e + 3] * ih};
      }
    }
  }
  if constexpr (kSplit) {
    // lane h holds head h's max and exp-sum
    if (lane < it.gc) {
      const size_t row = ((size_t)it.s * H + it.h0 + lane) * p.num_partitions + it.part;
      p.max_logits[row] = w.bad ? nan : w.m_true * kLn2;
      p.exp_sums[row] = w.l_run * fast_exp2(w.m_run - w.m_true);
    }
  }
}

// ---- phase-1 balanced split ----
// The launch's live units are the (block, head group) pairs of every
// sequence with a valid, non-empty length, laid end to end: sequence s
// occupies [gy_count * pre[s], gy_count * pre[s + 1]), head group gy of it
// [gy_count * pre[s] + gy * nb_s, + nb_s), nb_s = ceil(L_s / 16), pre[s] the
// live blocks of the sequences before s.  B = gy_count * pre[S] units are cut
// into N ranges: workgroup j takes [floor(j B / N), floor((j + 1) B / N)).
// The entry of the part of range j that lies in (sequence s, head group gy)
// goes to partition slot j - owner(first unit of that head group), where
// owner(x) = floor(((x + 1) N - 1) / B) is the range that holds unit x.
struct Balance {
  unsigned* pre;  // LDS [S + 1]
  int* len;       // LDS [S]
  uint64_t B;
  unsigned N;
};

// The live-block prefix (one wave; every workgroup computes the same), B and
// N.  Workgroup 0 publishes them for phase 2.
template <int kUnused = 0>
__device__ inline Balance balance_plan(const AttnParams& p, int lane) {
  __shared__ unsigned pre[kBalancedMaxSeqs + 1];
  __shared__ int len[kBalancedMaxSeqs];
  constexpr int kRounds = kBalancedMaxSeqs / kWave;
  const int S = p.num_seqs;
  const int maxtok = p.max_blocks * kBlockTokens;
  int L[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int s = r * kWave + lane;
    L[r] = s < S ? p.seq_lens[s] : 0;
  }
  unsigned run = 0, nb_max = 0;
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    if (r * kWave >= S) break;
    const int s = r * kWave + lane;
    const bool ok = s < S && L[r] > 0 && L[r] <= maxtok;
    const unsigned nb = ok ? (unsigned)((L[r] + kBlockTokens - 1) / kBlockTokens) : 0u;
    nb_max = max(nb_max, nb);
    unsigned x = nb;  // inclusive scan over the wave
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const unsigned y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (s < S) {
      pre[s] = run + x - nb;
      len[s] = L[r];
    }
    run += __shfl(x, kWave - 1);
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) nb_max = max(nb_max, (unsigned)__shfl_xor(nb_max, off));
  if (lane == 0) pre[S] = run;
  __builtin_amdgcn_wave_barrier();
  Balance b;
  b.pre = pre;
  b.len = len;
  b.B = (uint64_t)__builtin_amdgcn_readfirstlane(run) * (uint64_t)p.gy_count;
  b.N = __builtin_amdgcn_readfirstlane(
      balanced_ranges(b.B, __builtin_amdgcn_readfirstlane(nb_max), gridDim.x, p.num_partitions, p.num_cus));
  if (blockIdx.x == 0) {
    if (lane == 0) {
      p.info[0] = b.N;
      p.info[1] = (unsigned)b.B;
      p.info[2] = (unsigned)(b.B >> 32);
      p.info[3] = 0u;
    }
    for (int s = lane; s <= S; s += kWave) p.info[kInfoPrefix + s] = pre[s];
  }
  return b;
}

// Workgroup j of the balanced split: its range, one entry per head group it
// meets.
template <class W_, int D>
__device__ inline void run_balanced(const AttnParams& p, W_& w, float* ptile) {
  const Balance bal = balance_plan(p, w.lane);
  const unsigned j = blockIdx.x;
  if (j >= bal.N) return;
  const uint64_t B = bal.B, N = bal.N;
  const uint64_t gyc = (uint64_t)p.gy_count;
  uint64_t a = (uint64_t)j * B / N;
  const uint64_t end = ((uint64_t)j + 1) * B / N;
  while (a < end) {
    // the sequence: the last s with gy_count * pre[s] <= a (it has live blocks)
    int lo = 0, hi = p.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (gyc * __builtin_amdgcn_readfirstlane(bal.pre[mid]) <= a) lo = mid;
      else hi = mid - 1;
    }
    const int s = lo;
    const uint64_t s0 = gyc * __builtin_amdgcn_readfirstlane(bal.pre[s]);
    const int nb = (int)(__builtin_amdgcn_readfirstlane(bal.pre[s + 1]) - __builtin_amdgcn_readfirstlane(bal.pre[s]));
    if (nb <= 0) break;  // cannot happen (the unit lies in sequence s); keeps every access in bounds regardless
    const int gy = (int)((a - s0) / (uint64_t)nb);
    const uint64_t g0 = s0 + (uint64_t)gy * (uint64_t)nb;  // first unit of (s, gy)
    const uint64_t stop = min(end, g0 + (uint64_t)nb);
    WorkItem it;
    it.s = s;
    it.g = gy / p.head_chunks;
    const int hc = gy - it.g * p.head_chunks;
    it.h0 = it.g * p.group + hc * kMaxHeadsPerGroup;
    it.gc = min(kMaxHeadsPerGroup, p.group - hc * kMaxHeadsPerGroup);
    it.L = __builtin_amdgcn_readfirstlane(bal.len[s]);
    it.len_ok = true;
    it.part = (int)(j - range_owner(g0, N, B));
    it.b0 = (int)(a - g0);
    it.b1 = (int)(stop - g0);
    // the slot is below num_partitions by the choice of N; checked so that no store can leave the table
    if (gy >= p.gy_count || it.part >= p.num_partitions) break;
    w.reset();
    w.load_q(p, it.s, it.h0, it.gc);
    w.walk(p, it.s, it.g, it.L, it.b0, it.b1, 0, ptile);
    w.fold();
    write_result<W_, D, true>(p, w, it);
    a = stop;
  }
}

template <class DT, int D, int GH, int NW, bool kSplit, int LAYOUT>
__global__ __launch_bounds__((NW * kWave)) void attn_kernel(AttnParams p) {
  using W_ = Walker<DT, D, GH, NW, LAYOUT>;
  constexpr bool kMfmaPV = W_::kMfmaPV;
  constexpr int kRowsHeld = W_::kRowsHeld;
  constexpr int kPTile = W_::kPTile;
  constexpr int kSlices = W_::kSlices;
  constexpr int EPL = W_::EPL;
  constexpr int LPR = W_::LPR;
  constexpr int kTreeFloats = (NW / 2) * kRowsHeld * D;  // tree-merge buffer
  constexpr int kLdsFloats1 = (NW * kPTile > kTreeFloats) ? NW * kPTile : kTreeFloats;
  constexpr int kLdsFloats = kLdsFloats1 > 0 ? kLdsFloats1 : 1;
  static_assert((NW & (NW - 1)) == 0, "NW is a power of two");

  __shared__ float lds[kLdsFloats];  // rows layout: p tiles in the loop; then the tree-merge buffer
  __shared__ float m_lds[NW][kMaxHeadsPerGroup];
  __shared__ float t_lds[NW][kMaxHeadsPerGroup];
  __shared__ float l_lds[NW > 1 ? NW / 2 : 1][kMaxHeadsPerGroup];

  const int lane = threadIdx.x & (kWave - 1);
  // wave index is uniform across the wave; say so, so that everything derived
  // from it (block ids, buffer resources) stays in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  float* ptile = lds + wave * kPTile;
  W_ w(lane);
  const int rbase = w.rbase;

  if constexpr (kSplit && NW == 1) {
    if (p.balanced) {
      run_balanced<W_, D>(p, w, ptile);
      return;
    }
  }

  // the workgroup's own item: its partition (split) or the whole context
  WorkItem it = make_item(p, blockIdx.z, blockIdx.y, kSplit ? blockIdx.x : 0);
  bool live;
  if constexpr (kSplit) {
    // partitions past the sequence end write nothing; an invalid length is
    // reported by phase 2
    const int tok_begin = it.part * p.partition;
    live = it.len_ok && tok_begin < it.L;
    it.b0 = tok_begin / kBlockTokens;
    it.b1 = live ? (min(tok_begin + p.partition, it.L) + kBlockTokens - 1) / kBlockTokens : it.b0;
  } else {
    if (!it.len_ok || it.L == 0) {
      const float fill = it.len_ok ? 0.0f : __builtin_nanf("");
      for (int i = threadIdx.x; i < it.gc * D; i += NW * kWave)
        p.out[(size_t)it.s * (size_t)p.out_stride + (size_t)(it.h0 + i / D) * D + (i % D)] = fill;
      return;
    }
    live = true;
    it.b1 = (it.L + kBlockTokens - 1) / kBlockTokens;
  }

  w.reset();
  if (it.b0 < it.b1) {
    w.load_q(p, it.s, it.h0, it.gc);
    w.walk(p, it.s, it.g, it.L, it.b0, it.b1, wave, ptile);
  }
  w.fold();

  // (head, dim) -> accumulator element held by this lane, for the merge and
  // the epilogue.  rows: lanes < LPR hold dims EPL*lane..+EPL-1 of heads 0..GH-1.
  // tiled: every lane holds heads rbase..rbase+3 at dims 16 j + lane%16.
  if constexpr (NW > 1) {
    // common max per head, each wave rescales itself, then a fixed-order tree sum
    w.bad = __syncthreads_or(w.bad);
    if (lane < kMaxHeadsPerGroup) {
      m_lds[wave][lane] = w.m_run;
      t_lds[wave][lane] = w.m_true;
    }
    __syncthreads();
    float mx = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      mx = fmaxf(mx, m_lds[ww][lane & 15]);
      w.m_true = fmaxf(w.m_true, t_lds[ww][lane & 15]);
    }
    const float sc = fast_exp2(w.m_run - mx);
    w.l_run *= sc;
    w.scale_heads(sc);
    w.m_run = mx;
#pragma unroll
    for (int half = NW / 2; half >= 1; half /= 2) {
      __syncthreads();
      if (wave >= half && wave < 2 * half) {
        float* dst = lds + (wave - half) * kRowsHeld * D;
        if constexpr (kMfmaPV) {
#pragma unroll
          for (int j = 0; j < kSlices; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(rbase + i) * D + 16 * j + (lane & 15)] = w.accm[j][i];
        } else if (lane < LPR) {
#pragma unroll
          for (int h = 0; h < kRowsHeld; ++h)
#pragma unroll
            for (int e = 0; e < EPL; ++e) dst[h * D + EPL * lane + e] = w.acc[h][e];
        }
        if (lane < kMaxHeadsPerGroup) l_lds[wave - half][lane] = w.l_run;
      }
      __syncthreads();
      if (wave < half) {
        const float* src = lds + wave * kRowsHeld * D;
        if constexpr (kMfmaPV) {
#pragma unroll
          for (int j = 0; j < kSlices; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) w.accm[j][i] += src[(rbase + i) * D + 16 * j + (lane & 15)];
        } else if (lane < LPR) {
#pragma unroll
          for (int h = 0; h < kRowsHeld; ++h)
#pragma unroll
            for (int e = 0; e < EPL; ++e) w.acc[h][e] += src[h * D + EPL * lane + e];
        }
        w.l_run += l_lds[wave][lane & 15];
      }
    }
    if (wave != 0) return;
  }

  // ---- epilogue (wave 0) ----
  if (live) write_result<W_, D, kSplit>(p, w, it);
}

using AttnKernelFn = void (*)(AttnParams);

// Launch and return this launch's own status (not a stale error another call
// left on the thread).
inline hipError_t launch_kernel(AttnKernelFn fn, dim3 grid, dim3 block, const AttnParams& a, hipStream_t stream) {
  void* args[] = {const_cast<AttnParams*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), grid, block, args, 0, stream);
}

// Kernel for (D, GH) within one (element type, form, waves, layout) family.
// The tiled layout's accumulator always spans 16 head rows, so it has a single
// kernel per D.
template <class DT, bool kSplit, int NW, int LAYOUT>
AttnKernelFn select_attn(int d, int gh) {
  if constexpr (LAYOUT == kLayoutTiled) {
    switch (d) {
      case 64: return attn_kernel<DT, 64, 16, NW, kSplit, LAYOUT>;
      case 128: return attn_kernel<DT, 128, 16, NW, kSplit, LAYOUT>;
      default: return attn_kernel<DT, 256, 16, NW, kSplit, LAYOUT>;
    }
  } else {
#define PAD_GH_CASES(DV)                                           \
  switch (gh) {                                                    \
    case 1: return attn_kernel<DT, DV, 1, NW, kSplit, LAYOUT>;     \
    case 2: return attn_kernel<DT, DV, 2, NW, kSplit, LAYOUT>;     \
    case 4: return attn_kernel<DT, DV, 4, NW, kSplit, LAYOUT>;     \
    case 6: return attn_kernel<DT, DV, 6, NW, kSplit, LAYOUT>;     \
    case 8: return attn_kernel<DT, DV, 8, NW, kSplit, LAYOUT>;     \
    default: return attn_kernel<DT, DV, 16, NW, kSplit, LAYOUT>;   \
  }
    switch (d) {
      case 64: PAD_GH_CASES(64)
      case 128: PAD_GH_CASES(128)
      default: PAD_GH_CASES(256)
    }
#undef PAD_GH_CASES
  }
}

}  // namespace pad
