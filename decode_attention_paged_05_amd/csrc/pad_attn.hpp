// Attention kernel template for paged single-token decode on CDNA4 (gfx950).
// Included by the pad_attn_*.hip translation units, each of which
// instantiates one (element type, split/one-pass) family.
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
// Per 16-token block a wave:
//   * loads the K tile (16 rows x D) and the V tile with 16-byte buffer loads
//     whose bounds (num_records) are the block's valid rows: tail slots of the
//     last block read as zero and never reach the arithmetic, and a block id
//     outside the pool reads nothing at all;
//   * forms the 16 tokens x 16 heads logit tile on the matrix cores: A = K
//     (rows = tokens), B = Q^T (columns = the group's heads), contracting over
//     head_size.  The K tile's 16-byte pieces are already in the operand
//     layout (lane l holds token l%16 and a 16-byte run of dims; the same run
//     of Q supplies the B operand), so K goes from the load into the MFMA;
//   * updates the running max per head (a 4-lane shuffle reduction), turns
//     the logits into exp2 weights and publishes them through a 1 KB per-wave
//     LDS tile;
//   * accumulates P.V in fp32 on the vector ALUs: lane l owns a 16-byte run
//     of dims of one token per load, so each V load is one contiguous 1 KB
//     wave access.  Probabilities stay fp32 (bf16 probabilities would cost up
//     to 2^-9 relative per weight).
// Loads run R-1 blocks ahead of the arithmetic through a register ring.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pad_internal.h"

namespace pad {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
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
  // registers of one in-flight block (K and V)
  static constexpr int kStageVgprs = 2 * kSteps * 4;
  // blocks in flight per wave: as many (up to 3) as fit next to the Q operand
  // and a GH-head accumulator in ~400 of the 512 registers one wave per SIMD owns
  template <int GH>
  static constexpr int ring() {
    constexpr int fixed = kSteps * 4 + GH * kElemsPerLane + 48;
    constexpr int r = (400 - fixed) / kStageVgprs;
    return r < 1 ? 1 : (r > 3 ? 3 : r);
  }
  static_assert(kVLoads == kSteps, "K and V load counts agree");
  static_assert(kRowsPerLoad >= 1, "row fits in a wave");
};

struct AttnParams {
  const char* query;
  const char* key_cache;
  const char* value_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* out;         // one-pass output [S, H, D]
  float* max_logits;  // split workspace
  float* exp_sums;
  float* tmp_out;
  int64_t num_blocks;
  int num_heads;
  int num_kv_heads;
  int group;
  int head_chunks;
  int max_blocks;
  int partition;       // tokens per partition (split)
  int num_partitions;  // NP (split)
  float qscale;        // scale * log2(e)
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

template <class DT, int D, int GH, int NW, bool kSplit>
__global__ __launch_bounds__((NW * kWave)) void attn_kernel(AttnParams p) {
  using G_ = Geom<DT, D>;
  constexpr int R = G_::template ring<GH>();
  constexpr int kSteps = G_::kSteps;
  constexpr int LPR = G_::kLanesPerRow;
  constexpr int RPL = G_::kRowsPerLoad;
  constexpr int EPL = G_::kElemsPerLane;
  constexpr int kPTile = kBlockTokens * kMaxHeadsPerGroup;  // floats per wave
  constexpr int kTreeFloats = (NW / 2) * GH * D;             // tree-merge buffer
  constexpr int kLdsFloats = (NW * kPTile > kTreeFloats) ? NW * kPTile : kTreeFloats;
  static_assert((NW & (NW - 1)) == 0, "NW is a power of two");

  __shared__ float lds[kLdsFloats];  // p tiles in the loop, then the tree-merge buffer
  __shared__ float m_lds[NW][kMaxHeadsPerGroup];
  __shared__ float l_lds[NW > 1 ? NW / 2 : 1][kMaxHeadsPerGroup];

  const int lane = threadIdx.x & (kWave - 1);
  // wave index is uniform across the wave; say so, so that everything derived
  // from it (block ids, buffer resources) stays in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int part = blockIdx.x;
  const int s = blockIdx.z;
  const int g = blockIdx.y / p.head_chunks;
  const int chunk = blockIdx.y - g * p.head_chunks;
  const int h0 = g * p.group + chunk * kMaxHeadsPerGroup;
  const int gc = min(kMaxHeadsPerGroup, p.group - chunk * kMaxHeadsPerGroup);
  const int H = p.num_heads;
  const int L = p.seq_lens[s];
  const bool len_ok = L >= 0 && L <= p.max_blocks * kBlockTokens;

  int tok_begin = 0, tok_end = L;
  if constexpr (kSplit) {
    tok_begin = part * p.partition;
    // partitions past the sequence end write nothing; an invalid length is
    // reported by phase 2
    if (!len_ok || tok_begin >= L) return;
    tok_end = min(tok_begin + p.partition, L);
  } else {
    if (!len_ok || L == 0) {
      const float fill = len_ok ? 0.0f : __builtin_nanf("");
      for (int i = threadIdx.x; i < gc * D; i += NW * kWave) p.out[((size_t)s * H + h0 + i / D) * D + (i % D)] = fill;
      return;
    }
  }
  const int blk_begin = tok_begin / kBlockTokens;
  const int blk_end = (tok_end + kBlockTokens - 1) / kBlockTokens;

  // Q^T operand: lane l supplies head column l%16 and 16-byte run l/16 of
  // each 64-byte step (the run the K rows use).
  u32x4_t qop[kSteps];
  {
    const int qh = lane & 15;
    const char* qrow = p.query + ((size_t)s * H + h0 + qh) * G_::kRowBytes + 16 * (lane >> 4);
#pragma unroll
    for (int st = 0; st < kSteps; ++st)
      qop[st] = (qh < gc) ? *reinterpret_cast<const u32x4_t*>(qrow + 64 * st) : u32x4_t{0, 0, 0, 0};
  }

  float m_run = -INFINITY;  // running max (log2 units) of head column lane%16
  float l_run = 0.0f;       // this lane's share of that head's exp-sum
  float acc[GH][EPL];       // P.V partial: heads x this lane's dims
#pragma unroll
  for (int h = 0; h < GH; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
  bool bad = false;

  float* ptile = lds + wave * kPTile;
  const int32_t* table_row = p.block_tables + (size_t)s * p.max_blocks;
  const size_t head_off = (size_t)g * G_::kTileBytes;
  const size_t block_stride = (size_t)p.num_kv_heads * G_::kTileBytes;
  const int koff = (lane & 15) * G_::kRowBytes + 16 * (lane >> 4);
  const int voff = 16 * lane;

  struct Stage {
    u32x4_t k[kSteps];
    u32x4_t v[kSteps];
  };

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
      const int bytes = __builtin_amdgcn_readfirstlane(rows * G_::kRowBytes);
      __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(p.key_cache + base), (short)0, bytes, kRsrcWord3);
      __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(p.value_cache + base), (short)0, bytes, kRsrcWord3);
#pragma unroll
      for (int j = 0; j < kSteps; ++j) st.k[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff + 64 * j, 0, 0);
#pragma unroll
      for (int j = 0; j < kSteps; ++j) st.v[j] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff + 1024 * j, 0, 0);
    };

    auto compute = [&](const Stage& st, int blk) {
      // logits: lane l holds tokens 4*(l/16)+i of the block for head column l%16
      f32x4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < kSteps; ++j) c = qk_step(DT{}, st.k[j], qop[j], c);
      const int rbase = 4 * (lane >> 4);
      const int t0 = blk * kBlockTokens + rbase;
      float x[4];
      float bm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = (t0 + i < L) ? c[i] * p.qscale : -INFINITY;
        bm = fmaxf(bm, x[i]);
      }
      // lanes l, l^16, l^32, l^48 share a head column
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float m_new = fmaxf(m_run, bm);
      const float alpha = fast_exp2(m_run - m_new);
      float psum = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pw = fast_exp2(x[i] - m_new);
        psum += pw;
        ptile[(rbase + i) * kMaxHeadsPerGroup + (lane & 15)] = pw;
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int h = 0; h < GH; ++h) {
          const float a = readlane_f(alpha, h);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] *= a;
        }
      }
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

  // ---- wave totals: fold the token groups of acc and the 4 lanes of l ----
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1)
#pragma unroll
    for (int h = 0; h < GH; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  if constexpr (NW > 1) {
    // common max per head, each wave rescales itself, then a fixed-order tree sum
    bad = __syncthreads_or(bad);
    if (lane < kMaxHeadsPerGroup) m_lds[wave][lane] = m_run;
    __syncthreads();
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, m_lds[w][lane & 15]);
    const float sc = fast_exp2(m_run - mx);
    l_run *= sc;
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      const float a = readlane_f(sc, h);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= a;
    }
    m_run = mx;
#pragma unroll
    for (int half = NW / 2; half >= 1; half /= 2) {
      __syncthreads();
      if (wave >= half && wave < 2 * half) {
        float* dst = lds + (wave - half) * GH * D;
        if (lane < LPR)
#pragma unroll
          for (int h = 0; h < GH; ++h)
#pragma unroll
            for (int e = 0; e < EPL; ++e) dst[h * D + EPL * lane + e] = acc[h][e];
        if (lane < kMaxHeadsPerGroup) l_lds[wave - half][lane] = l_run;
      }
      __syncthreads();
      if (wave < half) {
        const float* src = lds + wave * GH * D;
        if (lane < LPR)
#pragma unroll
          for (int h = 0; h < GH; ++h)
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] += src[h * D + EPL * lane + e];
        l_run += l_lds[wave][lane & 15];
      }
    }
    if (wave != 0) return;
  }

  // ---- epilogue (wave 0): lanes < LPR hold EPL dims of every head ----
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    if (h >= gc) continue;
    const float mh = readlane_f(m_run, h);
    const float lh = readlane_f(l_run, h);
    const float inv = bad ? __builtin_nanf("") : 1.0f / lh;
    if constexpr (kSplit) {
      const size_t row = ((size_t)s * H + h0 + h) * p.num_partitions + part;
      if (lane < LPR) {
        float* dst = p.tmp_out + row * D + EPL * lane;
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
          *reinterpret_cast<f32x4_t*>(dst + e) =
              f32x4_t{acc[h][e] * inv, acc[h][e + 1] * inv, acc[h][e + 2] * inv, acc[h][e + 3] * inv};
      }
      if (lane == 0) {
        p.max_logits[row] = bad ? __builtin_nanf("") : mh * kLn2;
        p.exp_sums[row] = lh;
      }
    } else {
      if (lane < LPR) {
        float* dst = p.out + ((size_t)s * H + h0 + h) * D + EPL * lane;
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
          *reinterpret_cast<f32x4_t*>(dst + e) =
              f32x4_t{acc[h][e] * inv, acc[h][e + 1] * inv, acc[h][e + 2] * inv, acc[h][e + 3] * inv};
      }
    }
  }
}

using AttnKernelFn = void (*)(AttnParams);

// Launch and return this launch's own status (not a stale error another call
// left on the thread).
inline hipError_t launch_kernel(AttnKernelFn fn, dim3 grid, dim3 block, const AttnParams& a, hipStream_t stream) {
  void* args[] = {const_cast<AttnParams*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), grid, block, args, 0, stream);
}

// Kernel for (D, GH, NW) within one (element type, form) family.
template <class DT, bool kSplit, int NW>
AttnKernelFn select_attn(int d, int gh) {
#define PAD_GH_CASES(DV)                                   \
  switch (gh) {                                            \
    case 1: return attn_kernel<DT, DV, 1, NW, kSplit>;     \
    case 2: return attn_kernel<DT, DV, 2, NW, kSplit>;     \
    case 4: return attn_kernel<DT, DV, 4, NW, kSplit>;     \
    case 6: return attn_kernel<DT, DV, 6, NW, kSplit>;     \
    case 8: return attn_kernel<DT, DV, 8, NW, kSplit>;     \
    default: return attn_kernel<DT, DV, 16, NW, kSplit>;   \
  }
  switch (d) {
    case 64: PAD_GH_CASES(64)
    case 128: PAD_GH_CASES(128)
    default: PAD_GH_CASES(256)
  }
#undef PAD_GH_CASES
}

}  // namespace pad
