// Device helpers shared by the decode-attention kernels (per query head, and grouped
// query heads): vector types, the float16 staging of the step-t codebook slices in
// LDS, the two-part RoPE phase table, and the token-balanced work list (a sequence's
// coded tiles, then its bf16 tiles, cut into equal contiguous ranges).
#pragma once
#include "lvq_internal.h"

namespace lvq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescale = 8.0f;   // lazy-max slack, log2 units
constexpr float kNoMax = -1e30f;   // running maximum before the first valid score (finite,
                                   // so an invalid score of -inf still gives weight 0)
constexpr int kTile = 16;          // positions per tile (RoPE table granularity)
constexpr int kPtBatch = 128;      // page ids staged in LDS per wave at a time

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Page ids read outside their pool ([0, n_index_pages) for coded pages, [0, n_bf16_pages)
// for bf16 pages) are skipped: those tokens are left out.  When the caller passes a
// counter, every such lookup also adds one to it (a lookup is one lane reading one table
// entry, so an entry read by several heads or waves counts once for each).
__device__ __forceinline__ void note_rejected(unsigned* counter, bool bad) {
  if (counter && bad) atomicAdd(counter, 1u);
}

// 16-byte LDS read at a byte address.  The attention kernel declares no static LDS, so
// its dynamic LDS starts at address 0 and the code-table offsets are LDS addresses.
typedef const f16x8 __attribute__((address_space(3)))* lds_f16x8_ptr;
__device__ __forceinline__ f16x8 lds_read16(uint32_t addr) { return *(lds_f16x8_ptr)(size_t)addr; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
// sum over the 4 lanes of a quad (lanes 4i..4i+3), by DPP quad permutes
__device__ __forceinline__ float quad_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));   // [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));   // [2,3,0,1]
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// phase (cos, sin) of position p for pair j from the two-part table (float32 product)
__device__ __forceinline__ float2 phase(const float* __restrict__ rope, int tiles, int D, int p, int j) {
  const float* e0 = rope + (size_t)(p / kTile) * D + 2 * j;
  const float* e1 = rope + (size_t)(tiles + p % kTile) * D + 2 * j;
  const float c0 = e0[0], s0 = e0[1], c1 = e1[0], s1 = e1[1];
  return make_float2(c0 * c1 - s0 * s1, s0 * c1 + c0 * s1);
}

// Stage the step-tau [256][c] slices of all groups of book (beta, kv, h) into LDS as
// float16, laid out [code][chunk][8]: chunk k of code x holds channels 8k..8k+7 of
// code x's share.  A gather's LDS bank then depends on the chunk, not on the code.
// The K and V slices are staged together: load() puts every 16-byte piece of a thread
// in flight (one memory latency, not one per load, overlapping the work-list scan);
// store() converts and writes them.
template <int D, int C, int NTH>   // NTH: threads of the workgroup
struct SliceStage {
  static constexpr int NG = D / C;
  static constexpr int NCH = D / 8;
  static constexpr int PER = (kCodes * D / 8 + NTH - 1) / NTH;   // 16-byte pieces per thread and slice
  u16x8 v[2][PER];
  __device__ __forceinline__ void load(const AttnArgs& a, int beta, int h, int tau);
  __device__ __forceinline__ void store(_Float16* dst) const;
};
template <int D, int C, int NTH>
__device__ __forceinline__ void SliceStage<D, C, NTH>::load(const AttnArgs& a, int beta, int h, int tau) {
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const uint16_t* src = a.codebooks + ((((size_t)beta * 2 + kv) * a.H + h) * NG) * ((size_t)a.Tc * kCodes * C);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = (threadIdx.x + i * NTH) * 8;
      if (e < kCodes * D) {
        const int x = e / D, k = (e % D) / 8;                // destination code and chunk
        const int g = (8 * k) / C, j = (8 * k) % C;
        v[kv][i] = *(const u16x8*)(src + (((size_t)g * a.Tc + tau) * kCodes + x) * C + j);
      }
    }
  }
}
template <int D, int C, int NTH>
__device__ __forceinline__ void SliceStage<D, C, NTH>::store(_Float16* dst) const {
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = (threadIdx.x + i * NTH) * 8;
      if (e < kCodes * D) {
        const int x = e / D, k = (e % D) / 8;
        f16x8 o;
#pragma unroll
        for (int q = 0; q < 8; ++q) o[q] = (_Float16)bf2f(v[kv][i][q]);
        *(f16x8*)(dst + (size_t)kv * kCodes * D + ((size_t)x * NCH + k) * 8) = o;
      }
    }
  }
}

// ------------------------------------------------------------------ decode attention
// Work units of sequence b in a query head's work list: one per coded tile (two pages
// each), then kBfCost per bf16 virtual tile (the sink tile and the tiles over [r0, L)),
// which read float32 keys and values from HBM and cost that much more than a coded tile.
constexpr int kBfCost = 4;
struct SeqTiles {
  int coded;   // coded tiles (= their units)
  int total;   // units
};
// from sequence b's seq_len and q_end entries
__device__ __forceinline__ SeqTiles seq_tiles_of(const AttnArgs& a, int len, int q_end) {
  const int L = max(min(len, a.max_seq_len), 0);
  const int qe = max(min(q_end & ~7, L), 0);
  const int ns = min(a.n_sink, L);
  const int r0 = max(qe, a.n_sink);
  const int vt_lo = r0 / kTile;
  const int vt_hi = L > r0 ? (L - 1) / kTile + 1 : vt_lo;
  const int coded = a.n_index_pages > 0 ? ((qe >> 3) + 1) >> 1 : 0;
  return {coded, coded + kBfCost * ((ns > 0 ? 1 : 0) + (vt_hi - vt_lo))};
}
__device__ __forceinline__ SeqTiles seq_tiles(const AttnArgs& a, int b) {
  return seq_tiles_of(a, a.seq_len[b], a.q_end[b]);
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off);
    v += lane >= off ? u : 0;
  }
  return v;
}

// Token-balanced work split.  Every query head has the same work list: the units of
// sequences 0..B-1 in order, total units in all.  The W waves of a head take equal
// contiguous ranges [wg*total/W, (wg+1)*total/W) of it, crossing sequence boundaries;
// a wave writes one partial record per sequence its range meets (empty if it takes no
// tile there), at record wg + b of the head (distinct, since ranges and sequences are
// both in order).
__device__ __forceinline__ int range_lo(int wg, int total, int W) { return (int)((long)wg * total / W); }

}  // namespace
}  // namespace lvq
