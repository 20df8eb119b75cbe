// Multi-row attention over the LoopVQ cache, gfx950: many query rows per KV head.
//
// What it computes (LoopVQ summary, onedev.kr/papers/1681, sections "전제와 한계" and
// "무엇과 다른가"; the same attention as the decode kernel): at loop step t, query i of
// sequence b and query head hq (RoPE position pos[b] + i) attends over the paged cache
// [0, prefix_len[b]) -- coded tokens rebuilt from the step-(t % Tc) codebook slices,
// bf16 sink and recent tokens, keys rotated after dequantisation -- and, when the call
// carries them, over the chunk's own new keys 0 .. i (positions prefix_len[b] + i',
// causal).  Two uses: a prefill chunk attending to an existing coded prefix (the
// summary notes prefill runs slightly slower than bf16), and GQA decode, where the
// query heads of one KV head are the rows.
//
// Design (MI355X): a workgroup of 8 waves owns 16 query rows (a row block) of one KV
// head; the (KV head, row block) work list -- every sequence's 16-key tiles in order --
// is cut into equal ranges, one per wave (token-balanced, as in the decode kernel), so
// mixed sequence lengths keep every wave busy.  Each key is rebuilt and rotated once per
// tile in float32 and shared by all 16 rows through the matrix cores:
//  * lane (key j, quarter k) holds key j's channel pairs [16k, 16k+16) with their
//    partners + d/2, rebuilt by four 16-byte LDS gathers and rotated in registers (the
//    rotation of a pair stays inside the lane); those 32 values are its B operands of
//    the score MFMAs, whose A operands are the rotated query rows in the same order;
//  * the 16 x 16 scores land one row quarter per lane group; the online softmax keeps
//    (max, sum) per row, with the same lazy maximum as the decode kernel;
//  * probabilities go through a 1 KB LDS tile to the A-operand layout of the value
//    MFMAs; lane (column c, key quarter) gathers chunk c (channels 8c .. 8c+7) of four
//    keys, so output channel 8c + b of value block b sits in that lane.
// Precision.  Coded tiles run on float16 MFMAs with float32 accumulation: the rotated
// query and key values are split into float16 hi + lo parts and a score is the sum of
// hi*hi, hi*lo and lo*hi (12 v_mfma_f32_16x16x32_f16 per tile); the probabilities are
// split the same way against the float16 codewords, which are exact (16
// v_mfma_f32_16x16x16_f16).  Products of float16 values are exact in float32, so a score
// misses only the lo*lo terms and the rounding of the lo parts, about 2^-20 of each
// product: float32-level results at a sixteenth of the float32 matrix-core time.  The
// few bf16 tiles (sink, recent window, new keys) keep v_mfma_f32_16x16x4f32.
#include "lvq_internal.h"

namespace lvq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int kRW = 8;          // waves per workgroup
constexpr int kRows = 16;       // query rows per workgroup
constexpr int kKeys = 16;       // keys per tile (the RoPE table's tile)
constexpr float kRescaleR = 8.0f;
constexpr int kD = 128;         // head dim compiled

constexpr int kPtR = 256;       // page ids staged in LDS per wave at a time
constexpr int kErow = 4 * 36;   // tile-phase row: 4 quarters of 16 pairs, padded to 36 floats

constexpr size_t rows_lds_bytes() {
  // K and V slices (float16) + per wave: a 16 x 16 probability tile, a tile-phase row,
  // a batch of page ids
  return (size_t)2 * kCodes * kD * 2 + (size_t)kRW * (kKeys * kRows + kErow + kPtR) * 4;
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Page ids read outside their pool ([0, n_index_pages) for coded pages, [0, n_bf16_pages)
// for bf16 pages) are skipped: those tokens are left out.  When the caller passes a
// counter, every such lookup also adds one to it (a lookup is one lane reading one table
// entry, so an entry read by several heads or waves counts once for each).
__device__ __forceinline__ void note_rejected(unsigned* counter, bool bad) {
  if (counter && bad) atomicAdd(counter, 1u);
}

// x = hi + lo + e with hi, lo float16 (hi the nearest float16 to x, lo the nearest to the
// exact float32 remainder x - hi), so |e| <= 2^-11 |x - hi| <= 2^-22 |x| where no lo is
// subnormal.  Products of float16 operands are exact in the MFMA's float32 accumulation:
// a product of two split operands taken as hi*hi + hi*lo + lo*hi misses only lo*lo and the
// e terms, about 2^-20 of |x y|.
struct Split16 {
  _Float16 hi, lo;
};
__device__ __forceinline__ Split16 split16(float x) {
  const _Float16 hi = (_Float16)x;
  return {hi, (_Float16)(x - (float)hi)};
}
// The same split of two values at once, as packed float16 words (one v_cvt_pk_f16_f32 for
// each word; the remainders are exact in float32 and taken by v_fma_mix from the hi word).
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
  f32x2 r;
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r[0]) : "v"(hi), "v"(a));
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r[1]) : "v"(hi), "v"(b));
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, f16x2));
}

// Chunk k of code x sits at slot k ^ (x mod 16) of the key slice (XOR swizzle): the 16
// lanes that gather the same key chunk of random codes then spread over the LDS banks.
// The value slice keeps slot = k; its gathers already read distinct chunks per lane.
// The two slices are loaded by every thread's 2 x 8 sixteen-byte pieces at once, all in
// flight together (one after another, each load's round trip would add up: about 30 us
// for a workgroup), then converted and stored.
template <int C>
struct RowSlices {
  static constexpr int NG = kD / C;
  static constexpr int NCH = kD / 8;
  static constexpr int PER = kCodes * kD / 8 / (kRW * 64);   // pieces per thread and slice
  static_assert(PER * kRW * 64 * 8 == kCodes * kD, "whole pieces per thread");
  u16x8 v[2][PER];
  __device__ __forceinline__ void load(const RowsArgs& a, int beta, int h, int tau) {
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const uint16_t* src = a.codebooks + ((((size_t)beta * 2 + kv) * a.H + h) * NG) * ((size_t)a.Tc * kCodes * C);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = (threadIdx.x + i * kRW * 64) * 8;
        const int x = e / kD, k = (e % kD) / 8;
        const int g = (8 * k) / C, j = (8 * k) % C;
        v[kv][i] = *(const u16x8*)(src + (((size_t)g * a.Tc + tau) * kCodes + x) * C + j);
      }
    }
  }
  __device__ __forceinline__ void store(_Float16* kdst, _Float16* vdst) const {
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = (threadIdx.x + i * kRW * 64) * 8;
        const int x = e / kD, k = (e % kD) / 8;
        f16x8 o;
#pragma unroll
        for (int q = 0; q < 8; ++q) o[q] = (_Float16)bf2f(v[kv][i][q]);
        const int slot = kv == 0 ? (k ^ (x & (NCH - 1))) : k;
        *(f16x8*)((kv == 0 ? kdst : vdst) + ((size_t)x * NCH + slot) * 8) = o;
      }
    }
  }
};

// max over the 16 lanes of a lane group (xor offsets stay inside the group)
__device__ __forceinline__ float group16_max(float v) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
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

// Token-balanced work split, as in the decode kernel.  The work list of one (KV head,
// row block) is the units of sequences 0..B-1 in order: one per coded tile (two pages),
// then kBfCostR per virtual tile (the bf16 sink and recent tiles, then the new-key tiles
// the block's rows can see).  A virtual tile reads its keys and values from HBM through
// dependent loads and runs float32 matrix instructions, so it costs about four coded
// tiles on the float16 path; counted as one, a sequence's five sink and recent tiles fall
// to one wave, which then finishes last (GQA decode at 32K: 61.3 against 55.3 us at 16
// heads per KV head; the 512-token prefill is the same either way).  The W waves of a
// list take equal contiguous ranges [wg*total/W, (wg+1)*total/W) and write one partial
// record per (row, sequence their range meets), at record wg + b of the list.
constexpr int kBfCostR = 4;
struct RowSeq {
  int coded;   // coded tiles (= their units)
  int n_vt;    // virtual tiles
  int total;   // units
};
// from sequence b's prefix_len and q_end entries
__device__ __forceinline__ RowSeq row_seq_of(const RowsArgs& a, int prefix_len, int q_end, int n_new) {
  const int L = min(max(prefix_len, 0), a.max_prefix);
  const int qe = max(min(q_end & ~7, L), 0);
  const int ns = min(a.n_sink, L);
  const int r0 = max(qe, a.n_sink);
  const int vt_lo = r0 / kKeys;
  const int vt_hi = L > r0 ? (L - 1) / kKeys + 1 : vt_lo;
  const int coded = a.n_index_pages > 0 ? ((qe >> 3) + 1) >> 1 : 0;
  const int n_vt = (ns > 0 ? 1 : 0) + (vt_hi - vt_lo) + n_new;
  return {coded, n_vt, coded + kBfCostR * n_vt};
}
__device__ __forceinline__ RowSeq row_seq(const RowsArgs& a, int b, int n_new) {
  return row_seq_of(a, a.prefix_len[b], a.q_end[b], n_new);
}
__device__ __forceinline__ int range_lo(int wg, int total, int W) { return (int)((long)wg * total / W); }

template <int C>
__global__ __launch_bounds__(kRW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void rows_kernel(RowsArgs a, int wph) {
  constexpr int D = kD, HALF = D / 2, NG = D / C, NCH = D / 8;
  extern __shared__ __align__(16) unsigned char smem[];
  _Float16* kl = (_Float16*)smem;
  _Float16* vl = kl + (size_t)kCodes * D;
  float* ptile_all = (float*)(vl + (size_t)kCodes * D);
  float* erow_all = ptile_all + kRW * kKeys * kRows;
  int* ptl_all = (int*)(erow_all + kRW * kErow);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_lists = a.H * a.n_rb;
  const int list = blockIdx.x % n_lists, kw = blockIdx.x / n_lists;
  const int h = list / a.n_rb, rb = list % a.n_rb;
  const int g = a.Hq / a.H;
  const int R = a.NQ * g;
  const int beta = a.t / a.Tc, tau = a.t % a.Tc, nblk = a.T / a.Tc;
  const int W = wph * kRW;          // waves on this list
  const int wg = kw * kRW + wave;   // this wave among them
  // new-key tiles: up to the largest query index among this block's rows
  const int i_max = min(a.NQ - 1, (rb * kRows + kRows - 1) / g);
  const int n_new = a.k_new ? i_max / kKeys + 1 : 0;

  // The lengths of the first 64 sequences are loaded before the slices (vector loads
  // return in order: loaded after them, the scan below would wait for every slice piece).
  const int b_first = min(lane, a.B - 1);
  const int pl_first = a.prefix_len[b_first], qe_first = a.q_end[b_first];
  __builtin_amdgcn_sched_barrier(0);   // keep the two length loads ahead of the slice loads
  RowSlices<C> slices;
  slices.load(a, beta, h, tau);

  // the list's length and (one wave per row block) the sequences' first units
  int* tstart = a.tile_start + (size_t)rb * (a.B + 1);
  int total = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int bb = b0 + lane;
    const int n = bb < a.B ? (b0 == 0 ? row_seq_of(a, pl_first, qe_first, n_new) : row_seq(a, bb, n_new)).total : 0;
    if (h == 0 && wg == 0) {
      const int incl = total + wave_incl_scan(n);
      if (bb < a.B) tstart[bb] = incl - n;
    }
    total += wave_sum_i(n);
  }
  if (h == 0 && wg == 0 && lane == 0) tstart[a.B] = total;
  total = __builtin_amdgcn_readfirstlane(total);
  const int w_lo = __builtin_amdgcn_readfirstlane(range_lo(wg, total, W));
  const int w_hi = __builtin_amdgcn_readfirstlane(range_lo(wg + 1, total, W));

  slices.store(kl, vl);
  __syncthreads();
  if (w_lo == w_hi) return;

  // the sequence holding unit w_lo, and its first unit
  int b = 0, tb = 0;
  {
    int base = 0;
    for (int b0 = 0; b0 < a.B; b0 += 64) {
      const int bb = b0 + lane;
      const int n = bb < a.B ? (b0 == 0 ? row_seq_of(a, pl_first, qe_first, n_new) : row_seq(a, bb, n_new)).total : 0;
      const int incl = base + wave_incl_scan(n);
      const uint64_t hit = __ballot(bb < a.B && incl - n <= w_lo && w_lo < incl);
      if (hit) {
        const int src = __ffsll((unsigned long long)hit) - 1;
        b = b0 + src;
        tb = __shfl(incl - n, src);
        break;
      }
      base = __shfl(incl, 63);
    }
  }
  b = __builtin_amdgcn_readfirstlane(b);
  tb = __builtin_amdgcn_readfirstlane(tb);

  int pos_t = w_lo;
  while (pos_t < w_hi && b < a.B) {
    const RowSeq seq = row_seq(a, b, n_new);
    const int u_lo = pos_t - tb, u_hi = min(w_hi - tb, seq.total);
    if (u_lo < u_hi) {
      const int L = min(max(a.prefix_len[b], 0), a.max_prefix);
      const int qe = max(min(a.q_end[b] & ~7, L), 0);
      const int P_lo = 2 * u_lo;
      const int P_hi = min(2 * min(u_hi, seq.coded), qe >> 3);
      const int ns = min(a.n_sink, L);
      const int r0 = max(qe, a.n_sink);
      const int vt_lo = r0 / kKeys;
      const int vt_hi = L > r0 ? (L - 1) / kKeys + 1 : vt_lo;
      // virtual tiles whose first unit lies in the range
      const int vt_first = (max(u_lo, seq.coded) - seq.coded + kBfCostR - 1) / kBfCostR;
      const int vt_end = u_hi > seq.coded ? (u_hi - seq.coded + kBfCostR - 1) / kBfCostR : 0;

      // the lane's layout values from an opaque copy of the lane id, so nothing derived from
      // them for this sequence is held in registers across the sequence loop
      int lane_s = lane;
      asm volatile("" : "+v"(lane_s));
      const int j = lane_s & 15, kq = lane_s >> 4;   // key in tile / quarter (B side); row / quarter (A side)
      // A operands: rotated query rows, pairs [16 kq, 16 kq + 16) then their partners
      float qf[32];
      int row_q[4];                                  // query index of the 4 rows this lane holds in D layout
      {
        const int r_abs = rb * kRows + j;
        const bool row_ok = r_abs < R;
        const int qi = row_ok ? r_abs / g : 0, hq = h * g + (row_ok ? r_abs % g : 0);
        const int pq = min(max(a.pos[b] + qi, 0), a.rope_tiles * kKeys - 1);
        const uint16_t* qv = a.q + (((size_t)b * a.NQ + qi) * a.Hq + hq) * D;
        const float* e0 = a.rope + (size_t)(pq / kKeys) * D;
        const float* e1 = a.rope + (size_t)(a.rope_tiles + pq % kKeys) * D;
        // the lane's 16 query pairs and partners and their phases in 16-byte loads
        // (qi and hq stay in range for a padding row; its values are replaced by zeros)
        const u16x8 xq[2] = {((const u16x8*)(qv + 16 * kq))[0], ((const u16x8*)(qv + 16 * kq))[1]};
        const u16x8 yq[2] = {((const u16x8*)(qv + HALF + 16 * kq))[0], ((const u16x8*)(qv + HALF + 16 * kq))[1]};
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          const f32x4 p0 = ((const f32x4*)(e0 + 32 * kq))[s2], p1 = ((const f32x4*)(e1 + 32 * kq))[s2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int s = 2 * s2 + u;
            const float c0 = p0[2 * u], s0 = p0[2 * u + 1], c1 = p1[2 * u], s1 = p1[2 * u + 1];
            const float c = c0 * c1 - s0 * s1, sn = s0 * c1 + c0 * s1;
            const float x = row_ok ? bf2f(xq[s >> 3][s & 7]) : 0.f, y = row_ok ? bf2f(yq[s >> 3][s & 7]) : 0.f;
            qf[s] = (x * c - y * sn) * a.scale_log2e;
            qf[16 + s] = (y * c + x * sn) * a.scale_log2e;
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ra = rb * kRows + 4 * kq + r;
          row_q[r] = ra < R ? ra / g : -1;
        }
      }
      // the in-tile offset phase of key j for this lane's pairs
      float e1c[16], e1s[16];
      {
        const float* e1 = a.rope + (size_t)(a.rope_tiles + j) * D;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          e1c[s] = e1[2 * (16 * kq + s)];
          e1s[s] = e1[2 * (16 * kq + s) + 1];
        }
      }
      float m[4], lp[4];
      f32x4 O[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) { m[r] = -__builtin_inff(); lp[r] = 0.f; }
#pragma unroll
      for (int c8 = 0; c8 < 8; ++c8) O[c8] = f32x4{0.f, 0.f, 0.f, 0.f};
      float* ptile = ptile_all + wave * kKeys * kRows;

      const size_t row_stride = (size_t)kPage * NG;
      const size_t page_bytes = (size_t)nblk * a.H * 2 * row_stride;
      const uint8_t* head_rows = a.index_pages + (((size_t)beta * a.H + h) * 2) * row_stride;
      const int32_t* pt = a.page_table + (size_t)b * a.max_pages;
      const int32_t* bt = a.bf16_table + (size_t)b * a.bf16_row;

      auto gather = [&](const _Float16* slice, uint32_t code, int ch) -> f16x8 {
        return *(const f16x8*)(slice + ((size_t)code * NCH + ch) * 8);
      };
      auto gather_k = [&](uint32_t code, int ch) -> f16x8 {
        return *(const f16x8*)(kl + ((size_t)code * NCH + (ch ^ (code & (NCH - 1)))) * 8);
      };
      // One tile: keys at positions pbase + 0..15 (pbase a multiple of 16).
      //  kf: this lane's 32 raw key values (pairs of quarter kq, then partners), float32;
      //  vraw[s2][0..7]: chunk j of the value of key 4 s2 + kq;
      //  kok: the key of this lane is valid for every row; causal_base >= 0: new-key tile
      //  whose key i' = causal_base + j is visible to rows with query index >= i'.
      // rotate this lane's key values by position pbase + j (pbase a multiple of 16): the
      // tile phase E(pbase) times the lane's offset phase E(j)
      auto rotate_aligned = [&](int pbase, float (&kf)[32]) {
        const int a_tile = min(pbase / kKeys, a.rope_tiles - 1);
        const f32x4* e0 = (const f32x4*)(a.rope + (size_t)a_tile * D + 2 * 16 * kq);
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          const f32x4 e = e0[s2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int s = 2 * s2 + u;
            const float c0 = e[2 * u], s0 = e[2 * u + 1];
            const float c = c0 * e1c[s] - s0 * e1s[s], sn = s0 * e1c[s] + c0 * e1s[s];
            const float lo = kf[s], hi = kf[16 + s];
            kf[s] = lo * c - hi * sn;
            kf[16 + s] = lo * sn + hi * c;
          }
        }
      };
      // Masks, online softmax and the transpose of the probabilities into the A layout of
      // the value MFMAs: returns pa[s2] = P[row j][key 4 s2 + kq].
      //  kok: the key of lane column j exists; causal_base >= 0: new-key tile whose key
      //  i' = causal_base + j is visible to rows with query index >= i'.
      auto softmax_step = [&](const f32x4& S, bool kok, int causal_base, float (&pa)[4]) {
        float sv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          bool ok = kok && row_q[r] >= 0;
          if (causal_base >= 0) ok = ok && causal_base + j <= row_q[r];
          sv[r] = ok ? S[r] : -__builtin_inff();
        }
        if (__any(sv[0] > m[0] + kRescaleR || sv[1] > m[1] + kRescaleR || sv[2] > m[2] + kRescaleR ||
                  sv[3] > m[3] + kRescaleR)) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float mn = fmaxf(m[r], group16_max(sv[r]));
            const float f = mn == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(m[r] - mn);
            lp[r] *= f;
#pragma unroll
            for (int c8 = 0; c8 < 8; ++c8) O[c8][r] *= f;
            m[r] = mn;
          }
        }
        f32x4 P;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          P[r] = sv[r] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(sv[r] - m[r]);
          lp[r] += P[r];
        }
        *(f32x4*)(ptile + j * kRows + 4 * kq) = P;          // [key][row]
        asm volatile("" ::: "memory");
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) pa[s2] = ptile[(4 * s2 + kq) * kRows + j];
        asm volatile("" ::: "memory");
      };
      // A tile of 16 rotated keys (kf: this lane's 32 values, pairs of quarter kq then the
      // partners) and values (vraw[s2]: chunk j of key 4 s2 + kq) against the 16 rows.
      auto tile = [&](const float (&kf)[32], const float (&vraw)[4][8], bool kok, int causal_base) {
        f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 32; ++s) S = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[s], kf[s], S, 0, 0, 0);
        float pa[4];
        softmax_step(S, kok, causal_base, pa);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
          for (int c8 = 0; c8 < 8; ++c8)
            O[c8] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[s2], vraw[s2][c8], O[c8], 0, 0, 0);
      };

      // ---- virtual tiles: bf16 sink, recent window, new keys
      for (int vt = vt_first; vt < vt_end; ++vt) {
        const bool sink_tile = ns > 0 && vt == 0;
        const int after_sink = vt - (ns > 0 ? 1 : 0);
        const bool new_tile = after_sink >= vt_hi - vt_lo;
        float kf[32], vraw[4][8];
        bool kok = false;
        int pbase = 0, causal = -1;
        // this lane's key row (channels of quarter kq and their partners) as float32
        auto load_krow = [&](const uint16_t* krow, float (&kf)[32]) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int ch0 = (u >> 1) * HALF + 16 * kq + 8 * (u & 1);
            u16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
            if (krow) x = *(const u16x8*)(krow + ch0);
#pragma unroll
            for (int i = 0; i < 8; ++i) kf[(u & 1) * 8 + (u >> 1) * 16 + i] = bf2f(x[i]);
          }
        };
        if (new_tile) {
          const int nt = after_sink - (vt_hi - vt_lo);
          causal = nt * kKeys;
          const int ik = causal + j;
          kok = ik < a.NQ;
          load_krow(kok ? a.k_new + (((size_t)b * a.NQ + ik) * a.H + h) * D : nullptr, kf);
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) {
            const int iv = causal + 4 * s2 + kq;
            u16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
            if (iv < a.NQ) x = *(const u16x8*)(a.v_new + (((size_t)b * a.NQ + iv) * a.H + h) * D + 8 * j);
#pragma unroll
            for (int c8 = 0; c8 < 8; ++c8) vraw[s2][c8] = bf2f(x[c8]);
          }
          // new key i' sits at position L + i' (not tile aligned): its own phase E0 * E1
          const int pc = min(L + ik, a.rope_tiles * kKeys - 1);
          const float* e0 = a.rope + (size_t)(pc / kKeys) * D;
          const float* e1 = a.rope + (size_t)(a.rope_tiles + pc % kKeys) * D;
#pragma unroll
          for (int s = 0; s < 16; ++s) {
            const int pr = 16 * kq + s;
            const float c0 = e0[2 * pr], s0 = e0[2 * pr + 1], c1 = e1[2 * pr], s1 = e1[2 * pr + 1];
            const float c = c0 * c1 - s0 * s1, sn = s0 * c1 + c0 * s1;
            const float lo = kf[s], hi = kf[16 + s];
            kf[s] = lo * c - hi * sn;
            kf[16 + s] = lo * sn + hi * c;
          }
        } else {
          const int a_tile = sink_tile ? 0 : vt_lo + after_sink;
          const int lo = sink_tile ? 0 : r0, hi = sink_tile ? ns : L;
          pbase = kKeys * a_tile;
          auto row_of = [&](int p) -> const uint16_t* {
            if (p < lo || p >= hi) return nullptr;
            const int slot = sink_tile ? 0 : 1 + (p >> 3) - (qe >> 3);
            const int pg = slot < a.bf16_row ? bt[slot] : -1;
            note_rejected(a.rejected, pg < 0 || pg >= a.n_bf16_pages);
            if (pg < 0 || pg >= a.n_bf16_pages) return nullptr;
            return a.bf16_pages + (((((size_t)pg * a.T + a.t) * a.H + h) * 2) * kPage + (p & 7)) * D;
          };
          const uint16_t* krow = row_of(pbase + j);
          kok = krow != nullptr;
          load_krow(krow, kf);
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) {
            const uint16_t* vr = row_of(pbase + 4 * s2 + kq);
            u16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
            if (vr) x = *(const u16x8*)(vr + (size_t)kPage * D + 8 * j);
#pragma unroll
            for (int c8 = 0; c8 < 8; ++c8) vraw[s2][c8] = bf2f(x[c8]);
          }
          rotate_aligned(pbase, kf);
        }
        tile(kf, vraw, kok, causal);
      }

      // ---- coded tiles: pages [P_lo, P_hi), two pages per tile; the index words and the
      // tile phase of the next tile are loaded while the current one computes
      {
        float* erow = erow_all + wave * kErow;
        int* ptl = ptl_all + wave * kPtR;
        int pt_base = -kPtR;
        auto stage_pt = [&](int P) {
          pt_base = P;
          int v[kPtR / 64];
#pragma unroll
          for (int k = 0; k < kPtR / 64; ++k) v[k] = pt[min(P + k * 64 + lane, a.max_pages - 1)];
#pragma unroll
          for (int k = 0; k < kPtR / 64; ++k) {
            const int q = P + k * 64 + lane;
            const bool in_pool = v[k] >= 0 && v[k] < a.n_index_pages;
            note_rejected(a.rejected, q < P_hi && !in_pool);
            ptl[k * 64 + lane] = (q < P_hi && in_pool) ? v[k] : -1;
          }
          asm volatile("" ::: "memory");
        };
        // index-word byte offsets and code shifts of this lane (key chunks 2kq, 2kq+1 share
        // word wl, their partners word wh; value chunk j sits in word wv)
        const int gl = (16 * kq) / C, gh = (HALF + 16 * kq) / C, gv = (8 * j) / C;
        const int wl = gl & ~3, wh = gh & ~3, wv = gv & ~3;
        uint32_t shk[4];
        {
          const int chs[4] = {2 * kq, 2 * kq + 1, NCH / 2 + 2 * kq, NCH / 2 + 2 * kq + 1};
#pragma unroll
          for (int u = 0; u < 4; ++u) shk[u] = 8 * (((8 * chs[u]) / C) & 3);
        }
        const uint32_t shv = 8 * (gv & 3);
        struct CIn {
          uint32_t kwl, kwh, vw[4];
          float2 e0;
          int physk;
        };
        auto fetch = [&](int P0) -> CIn {
          CIn in;
          if (P0 + 2 > pt_base + kPtR) stage_pt(P0);
          const int ph0 = P0 < P_hi ? ptl[P0 - pt_base] : -1;
          const int ph1 = P0 + 1 < P_hi ? ptl[P0 + 1 - pt_base] : -1;
          in.physk = (j >> 3) ? ph1 : ph0;
          const uint8_t* kb = head_rows + (size_t)max(in.physk, 0) * page_bytes + (j & 7) * NG;
          in.kwl = *(const uint32_t*)(kb + wl);
          in.kwh = *(const uint32_t*)(kb + wh);
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) {
            const int kv = 4 * s2 + kq;
            const int ph = (kv >> 3) ? ph1 : ph0;
            const uint8_t* vb = head_rows + (size_t)max(ph, 0) * page_bytes + row_stride + (kv & 7) * NG;
            in.vw[s2] = *(const uint32_t*)(vb + wv);
          }
          const int a_tile = min((8 * P0) / kKeys, a.rope_tiles - 1);
          in.e0 = *(const float2*)(a.rope + (size_t)a_tile * D + 2 * lane);
          return in;
        };
        // A operands of the coded tiles' score MFMAs (v_mfma_f32_16x16x32_f16): the rotated
        // query rows split into float16 hi + lo.  Block m holds, for lane (row j, quarter kq),
        // k = 8 kq .. 8 kq + 7 <-> pairs 16 kq + 8 (m & 1) + i (m < 2) or their partners
        // (m >= 2); the keys use the same order.
        f16x8 qh[4], ql[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const Split16 v = split16(qf[(mb >> 1) * 16 + 8 * (mb & 1) + i]);
            qh[mb][i] = v.hi;
            ql[mb][i] = v.lo;
          }
        auto coded_tile = [&](int P0, const CIn& in) {
          const int pbase = 8 * P0;
          *(float2*)(erow + 36 * (lane >> 4) + 2 * (lane & 15)) = in.e0;     // pair `lane`
          asm volatile("" ::: "memory");
          const bool kok = in.physk >= 0 && pbase + j >= a.n_sink;
          f16x8 xk[4];
          {
            const int chs[4] = {2 * kq, 2 * kq + 1, NCH / 2 + 2 * kq, NCH / 2 + 2 * kq + 1};
#pragma unroll
            for (int u = 0; u < 4; ++u)
              xk[u] = gather_k(__builtin_amdgcn_ubfe(u < 2 ? in.kwl : in.kwh, shk[u], 8), chs[u]);
          }
          // the lane's 32 rotated key values (float32; the float16 key values enter the
          // rotation through v_fma_mix), split pairwise into float16 hi + lo words
          uint32_t khw[4][4], klw[4][4];   // [block][word]: elements 2 w, 2 w + 1 of the block
#pragma unroll
          for (int s2 = 0; s2 < 8; ++s2) {
            const f32x4 e = *(const f32x4*)(erow + 36 * kq + 4 * s2);
            float rx[2], ry[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int s = 2 * s2 + u;
              const float c0 = e[2 * u], s0 = e[2 * u + 1];
              const float c = c0 * e1c[s] - s0 * e1s[s], sn = s0 * e1c[s] + c0 * e1s[s];
              const float lo = (float)xk[s >> 3][s & 7], hi = (float)xk[2 + (s >> 3)][s & 7];
              rx[u] = fmaf(lo, c, fmaf(hi, -sn, 0.f));
              ry[u] = fmaf(lo, sn, fmaf(hi, c, 0.f));
            }
            split_pair(rx[0], rx[1], khw[s2 >> 2][s2 & 3], klw[s2 >> 2][s2 & 3]);
            split_pair(ry[0], ry[1], khw[2 + (s2 >> 2)][s2 & 3], klw[2 + (s2 >> 2)][s2 & 3]);
          }
          f16x8 kh[4], kl[4];
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) {
            kh[mb] = __builtin_bit_cast(f16x8, u32x4{khw[mb][0], khw[mb][1], khw[mb][2], khw[mb][3]});
            kl[mb] = __builtin_bit_cast(f16x8, u32x4{klw[mb][0], klw[mb][1], klw[mb][2], klw[mb][3]});
          }
          // scores: hi*hi on one accumulator, the two cross terms on another
          f32x4 S = {0.f, 0.f, 0.f, 0.f}, Sx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) {
            S = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[mb], kh[mb], S, 0, 0, 0);
            Sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[mb], kl[mb], Sx, 0, 0, 0);
            Sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql[mb], kh[mb], Sx, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) S[r] += Sx[r];
          float pa[4];
          softmax_step(S, kok, -1, pa);
          // values (v_mfma_f32_16x16x16_f16): k = 4 kq + i <-> key 4 i + kq, so lane (row j,
          // kq) holds P[j][4 i + kq] = pa[i] (split into hi + lo) and lane (column j, kq) the
          // channel 8 j + c8 of the value chunks it gathered; the float16 codewords are exact.
          // Invalid keys have P = 0 and finite codewords, so their values need no mask.
          f16x8 xv[4];
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) xv[s2] = gather(vl, __builtin_amdgcn_ubfe(in.vw[s2], shv, 8), j);
          f16x4 ph, pl;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const Split16 v = split16(pa[i]);
            ph[i] = v.hi;
            pl[i] = v.lo;
          }
#pragma unroll
          for (int c8 = 0; c8 < 8; ++c8) {
            const f16x4 vb = {xv[0][c8], xv[1][c8], xv[2][c8], xv[3][c8]};
            O[c8] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, vb, O[c8], 0, 0, 0);
            O[c8] = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, vb, O[c8], 0, 0, 0);
          }
        };
        // three tiles per iteration in three register sets, each tile's inputs loaded two
        // tiles ahead (a tile's float16 products take less time than an index load from
        // HBM takes to return; fetches past the range read page 0 and are not used)
        if (P_lo < P_hi) {
          CIn in0 = fetch(P_lo);
          CIn in1 = fetch(P_lo + 2);
          for (int P0 = P_lo;; P0 += 6) {
            const CIn in2 = fetch(P0 + 4);
            coded_tile(P0, in0);
            if (P0 + 2 >= P_hi) break;
            in0 = fetch(P0 + 6);
            coded_tile(P0 + 2, in1);
            if (P0 + 4 >= P_hi) break;
            in1 = fetch(P0 + 8);
            coded_tile(P0 + 4, in2);
            if (P0 + 6 >= P_hi) break;
          }
        }
      }

      // ---- partial records of the 4 rows this lane holds
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float l = group16_sum(lp[r]);
        const int ra = rb * kRows + 4 * kq + r;
        if (ra < R) {
          float* rec = a.part + ((((size_t)list * a.n_rec + wg + b) * kRows) + 4 * kq + r) * (D + 2);
          if (j == 0) { rec[0] = m[r]; rec[1] = l; }
          f32x4 o0 = {O[0][r], O[1][r], O[2][r], O[3][r]};
          f32x4 o1 = {O[4][r], O[5][r], O[6][r], O[7][r]};
          *(f32x4*)(rec + 2 + 8 * j) = o0;
          *(f32x4*)(rec + 2 + 8 * j + 4) = o1;
        }
      }
    }   // u_lo < u_hi
    pos_t = __builtin_amdgcn_readfirstlane(tb + u_hi);
    tb = __builtin_amdgcn_readfirstlane(tb + seq.total);
    b = __builtin_amdgcn_readfirstlane(b + 1);
  }   // sequences
}

template <int C>
hipError_t launch_rows_t(const RowsArgs& a, hipStream_t s) {
  constexpr size_t lds = rows_lds_bytes();
  static std::atomic<uint64_t> attr_set{0};
  hipError_t ea = once_per_device(attr_set, [&] {
    return hipFuncSetAttribute((const void*)rows_kernel<C>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds);
  });
  if (ea != hipSuccess) return ea;
  const int wph = a.n_waves / kRW;   // workgroups per (KV head, row block)
  if (wph < 1 || a.n_waves % kRW || a.n_rec != a.n_waves + a.B || !a.tile_start) return hipErrorInvalidValue;
  const long grid = (long)wph * a.n_rb * a.H;
  hipLaunchKernelGGL((rows_kernel<C>), dim3((unsigned)grid), dim3(kRW * 64), lds, s, a, wph);
  return hipGetLastError();
}

}  // namespace

bool rows_supported(int d, int c) { return d == kD && (c == 8 || c == 16 || c == 32); }
int rows_waves_per_group() { return kRW; }

hipError_t launch_rows(const RowsArgs& a, hipStream_t s) {
  const int c = a.G / a.Tc;
  if (c == 8) return launch_rows_t<8>(a, s);
  if (c == 16) return launch_rows_t<16>(a, s);
  return launch_rows_t<32>(a, s);
}

}  // namespace lvq
