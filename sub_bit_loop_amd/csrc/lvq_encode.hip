// Joint loop-axis nearest-codeword encoder for gfx950.
//
// What it computes (LoopVQ summary, onedev.kr/papers/1681, sections "무엇과
// 다른가" and "전제와 한계"): for every (loop block beta, token n, head h,
// channel group g) the G-vector x[tau*c + i] = X[beta*Tc + tau][n][h][g*c + i]
// is replaced by the index of its nearest codeword (squared L2, lowest index
// on ties) among the 256 codewords of book (beta, K/V, h, g).  The summary
// notes that the distances are obtained with a matrix product; here that
// product runs on the MFMA units.
//
// Design (MI355X):
//  * One wave owns one codebook for a whole token range.  The 256 codewords,
//    pre-scaled by -2 (exact in bf16), sit in VGPRs as the A operand of
//    v_mfma_f32_32x32x16_bf16 (8 blocks of 32 codes, G/16 K-halves each); a
//    32-token tile of joint vectors is the B operand (columns = vectors), loaded
//    straight from the cache in the layout the MFMA wants (8 or 4 contiguous
//    channels of one loop step per lane).  The accumulator input is |C_k|^2, so each
//    block returns D'_k = |C_k|^2 - 2 x.C_k = |x - C_k|^2 - |x|^2 for 32 codes x 32
//    vectors, float32.
//  * Argmin: each lane holds 128 candidates of one vector (8 blocks x 16 rows).
//    Each becomes a key, D' with its six low mantissa bits replaced by the
//    candidate's position; keys are folded a pair at a time (v_min3, v_med3) into
//    the smallest and second smallest key (2.25 VALU per candidate), then the two
//    lanes of the vector (lane ^ 32) merge through v_permlane32_swap.
//  * Exactness: a vector is recomputed in float64 by direct differences over
//    all 256 codewords (the definition itself) when its second smallest key is
//    within the float32 error bound of the smallest.  So the chosen index is the
//    float64 nearest codeword with lowest-index ties: float32 decides only where
//    no other candidate can be within rounding of the winner.
//  * Input tiles (32 tokens) are loaded two tiles ahead of their use; the |C_k|^2
//    of the next block of MFMAs is read from LDS while the current block folds.
//  * A workgroup holds the waves of up to 4 consecutive groups of one
//    (block, head); the workgroups that read the other halves of the same
//    128-byte cache rows run on the same XCD at the same time, and the waves of a
//    workgroup meet at a barrier every two tiles, so a row line stays in L2 until
//    its readers have taken it (the input is read from memory about 1.1-1.3 times).
#include "lvq_internal.h"

#include <atomic>
#include <cstdint>
#include <type_traits>

namespace lvq {
namespace {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// v_min_f32 / v_max_f32 / v_min3_f32 / v_med3_f32 on argmin keys.  The keys are finite floats built by bit
// operations; written through fminf the compiler would first quiet each one (an
// extra v_max per candidate) because it cannot prove the operand is not a
// signalling NaN.
__device__ __forceinline__ float key_min(float a, float b) {
  float r;
  asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float key_max(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float key_min3(float a, float b, float c) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float key_med3(float a, float b, float c) {
  float r;
  asm("v_med3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Exchange with lane ^ 32 (v_permlane32_swap), a VALU instruction with no LDS round
// trip.  Each lane gets its own value and its partner's as (lo, hi), where lo is the
// value of the pair's lower lane on both lanes, so an operation of (lo, hi) gives
// bit-identical results in the two lanes.
__device__ __forceinline__ void pair32(float v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Loads the lane's 8 joint-vector elements e = e0 .. e0 + 7 (a multiple of 8) of one
// vector whose step-tau channel slices start at row(tau) (element tau * C + i is
// row(tau)[i]): one 16-byte load when 8 divides C, two 8-byte loads when C = 4.
template <int C, typename RowFn>
__device__ __forceinline__ u16x8 load8(RowFn row, int e0) {
  if constexpr (C % 8 == 0) {
    return *(const u16x8*)(row(e0 / C) + e0 % C);
  } else {
    const u16x4 lo = *(const u16x4*)(row(e0 / C));
    const u16x4 hi = *(const u16x4*)(row(e0 / C + 1));
    u16x8 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) { v[q] = lo[q]; v[q + 4] = hi[q]; }
    return v;
  }
}

__device__ __forceinline__ f32x16 mfma32(const u16x8& a, const u16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

// Float64 direct-difference nearest codeword of vector column cv of the current tile,
// computed from registers.  The wave holds the codebook as MFMA operand A: lane
// (kk, col) holds elements 16 hh + 8 kk .. + 7 of codeword 32 b + col, times -2 (exact);
// the tile is operand B: lane (kk, col) holds the same elements of vector col.  Each lane
// sums its elements for codes 32 b + col, the lane pair (kk = 0, 1) adds its parts (the
// same sum in both lanes), and the 32 columns compare.  Ties resolve to the lowest code.
template <int NH, int NB>
__device__ __forceinline__ int exact_in_registers(const u16x8 (&A)[NB][NH], const u16x8 (&B)[NH], int cv,
                                                  int lane) {
  const int kk = lane >> 5, col = lane & 31;
  const int src = (kk << 5) | cv;
  double x[NH][8];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const uint32_t w = (uint32_t)__shfl((int)((uint32_t)B[hh][e] | ((uint32_t)B[hh][e + 1] << 16)), src);
      x[hh][e] = (double)bf2f((uint16_t)(w & 0xffffu));
      x[hh][e + 1] = (double)bf2f((uint16_t)(w >> 16));
    }
  double best = __builtin_inf();
  int bidx = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    double part = 0.0;
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        // opaque copy: keeps the conversions here instead of hoisted out of the token loop
        uint32_t w = (uint32_t)A[b][hh][e] | ((uint32_t)A[b][hh][e + 1] << 16);
        asm volatile("" : "+v"(w));
        const double d0 = fma(0.5, (double)bf2f((uint16_t)(w & 0xffffu)), x[hh][e]);   // x - C, A = -2 C
        const double d1 = fma(0.5, (double)bf2f((uint16_t)(w >> 16)), x[hh][e + 1]);
        part = fma(d0, d0, part);
        part = fma(d1, d1, part);
      }
    part += __shfl_xor(part, 32);
    if (part < best) { best = part; bidx = 32 * b + col; }   // b ascending: lowest code kept
  }
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) {
    const double ob = __shfl_xor(best, off);
    const int oi = __shfl_xor(bidx, off);
    if (ob < best || (ob == best && oi < bidx)) { best = ob; bidx = oi; }
  }
  return bidx;
}

// Waves per workgroup: one per channel group, up to 4.
template <int D, int C>
constexpr int waves_per_group_block() { return D / C < 4 ? D / C : 4; }

// Work items are (token range, channel-group block, head, loop block, K/V).  The
// items of one (token range, head, loop block, K/V) that read the same 128-byte rows
// differ only in the group block and are numbered 8 apart, so with a grid that is a
// multiple of 8 x (group blocks) they run on the same XCD (round-robin dispatch) at
// the same time and each row is fetched from HBM once.
constexpr int kXcds = 8;
constexpr int kTileTokens = 32;   // vectors per MFMA tile (the 32 columns)

// Per-layer pools and books of a pages -> pages launch (the decode-time re-encode of
// several layers at once); the other modes take none.
struct NoLayers {};
template <int MODE>
using LayersArg = typename std::conditional<MODE == 2, ReencodeLayers, NoLayers>::type;

// MODE: 0 dense source and destination, 1 dense source into coded pages,
// 2 bf16 pages into coded pages (items of all layers in one grid, the layer
// outermost).  Occupancy: 3 waves per SIMD at G = 32 (the codebook takes 64
// VGPRs), 4 at G = 16.  The grid is persistent: each workgroup loads a codebook
// once per item and streams the item's whole token range.
template <int G, int C, int D, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(G == 32 ? 3 : 4, 8)))
void encode_kernel(EncodeArgs a0, int n_items, LayersArg<MODE> layers) {
  constexpr bool kDenseSrc = MODE != 2;
  constexpr bool kDenseDst = MODE == 0;
  constexpr int NG = D / C;
  constexpr int WPG = waves_per_group_block<D, C>();   // waves (groups) per workgroup
  constexpr int NGB = NG / WPG;
  constexpr int TC = G / C;
  constexpr int NH = G / 16;             // 16-element K halves: MFMAs per block of 32 codes
  constexpr int NB = kCodes / 32;        // blocks of 32 codes (the MFMA rows)
  constexpr int kRing = 2;               // tiles in flight
  __shared__ __attribute__((aligned(16))) float s_bias[WPG][kCodes];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int H = a0.H, N = a0.N;
  const int nblk = a0.T / TC;
  const int tpi = a0.tokens_per_block;
  const int nparts = (N + tpi - 1) / tpi;
  // Items of one "combo" (token range, block of HB heads, loop block, K/V, layer) run on
  // one XCD: its HB x NGB workgroups read every 128-byte row of their tokens and write
  // every dense index row of them (HB heads x ng groups), so rows meet in that XCD's L2.
  const int HB = a0.head_block;
  const int nhb = H / HB;
  const int ncombo_layer = nparts * nhb * nblk * (a0.kv_sel >= 0 ? 1 : 2);
  int n_layers = 1;
  if constexpr (MODE == 2) n_layers = layers.n;
  const int ncombo = ncombo_layer * n_layers;
  const int per_combo = HB * NGB;
  // MFMA 32x32x16 lane roles: operand A row / operand B column / result column col,
  // K elements 8 kk .. 8 kk + 7 of each 16-element half; result rows 8 jj + 4 kk + r
  const int kk = lane >> 5, col = lane & 31;

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int xcd = item % kXcds;
    const int j = item / kXcds;
    const int inner = j % per_combo;
    int rest = (j / per_combo) * kXcds + xcd;   // the combo
    if (rest >= ncombo) continue;   // padding to whole XCD rounds (uniform per workgroup)
    const int gb = inner % NGB;
    const int hh0 = inner / NGB;
    EncodeArgs a = a0;
    if constexpr (MODE == 2) {     // the item's layer: its pools and books
      const ReencodeLayer& L = layers.layer[rest / ncombo_layer];
      rest %= ncombo_layer;
      a.src = L.bf16_pages;
      a.codebooks = L.codebooks;
      a.out = L.index_pages;
      a.n_src_pages = L.n_bf16_pages;
      a.n_dst_pages = L.n_index_pages;
    }
    const int part = rest % nparts; rest /= nparts;
    const int h = (rest % nhb) * HB + hh0; rest /= nhb;
    const int beta = rest % nblk;   rest /= nblk;
    const int kv = (a.kv_sel >= 0) ? a.kv_sel : rest;
    const int g = gb * WPG + wave;
    const int nb0 = part * tpi;
    const int nb1 = min(N, nb0 + tpi);

    // ---- the codebook as MFMA A operand, scaled by -2 (exact); |C_k|^2 in float64, rounded once
    const uint16_t* cb = a.codebooks + ((((size_t)beta * 2 + kv) * H + h) * NG + g) * ((size_t)TC * kCodes * C);
    u16x8 A[NB][NH];
    float cmax2 = 0.f;
  #pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int code = 32 * b + col;
      double s = 0.0;
  #pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const u16x8 v = load8<C>([&](int tau) { return cb + ((size_t)tau * kCodes + code) * C; }, 16 * hh + 8 * kk);
        u16x8 w;
  #pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = bf2f(v[e]);
          s = fma((double)f, (double)f, s);
          w[e] = (uint16_t)(__float_as_uint(-2.f * f) >> 16);
        }
        A[b][hh] = w;
      }
      s += __shfl_xor(s, 32);
      const float sf = (float)s;
      cmax2 = fmaxf(cmax2, sf);
      if (kk == 0) s_bias[wave][code] = sf;
    }
  #pragma unroll
    for (int off = 1; off < 32; off <<= 1) cmax2 = fmaxf(cmax2, __shfl_xor(cmax2, off));
    const float* bias = &s_bias[wave][4 * kk];   // + 32 b + 8 jj: codes 32 b + 8 jj + 4 kk + r
    // Dense rows of (loop step tau, token n) start at src_base + tau * N * H * d + n * H * d.
    const size_t src_stride = (size_t)H * a.d;
    const size_t step_stride = (size_t)N * H * a.d;
    const size_t dst_stride = (size_t)H * NG;
    const uint16_t* src_base = a.src + ((size_t)beta * TC * N * H + h) * a.d + g * C;
    uint8_t* dst_lane = a.out + ((size_t)beta * N * H + h) * NG + g + (size_t)(nb0 + col) * dst_stride;

    // Load the lane's elements of tile n0's vector col (and its destination page id).
    // Every load is unconditional, a slot past the range reading a row of this block and
    // a missing bf16 page reading the codebook, so the compiler can count the loads in
    // flight; ok says whether the slot is a real token.
    auto fetch = [&](int n0, u16x8 (&v)[NH], bool& ok, int& pg) {
      const int n = n0 + col;
      ok = n < nb1;
      if constexpr (kDenseSrc) {
        const uint16_t* rowp = src_base + (size_t)(ok ? n : nb0) * src_stride;
  #pragma unroll
        for (int hh = 0; hh < NH; ++hh)
          v[hh] = load8<C>([&](int tau) { return rowp + (size_t)tau * step_stride; }, 16 * hh + 8 * kk);
      } else {
        const int P = a.src_pages[(ok ? n : nb0) >> 3];
        const bool have = P >= 0 && P < a.n_src_pages;
        ok = ok && have;
        const uint16_t* pb = a.src + ((((size_t)(have ? P : 0) * a.T + beta * TC) * H + h) * 2 + kv) * kPage * a.d +
                             (size_t)((ok ? n : nb0) & 7) * a.d + g * C;
        const size_t pstep = (size_t)H * 2 * kPage * a.d;
  #pragma unroll
        for (int hh = 0; hh < NH; ++hh)
          v[hh] = have ? load8<C>([&](int tau) { return pb + (size_t)tau * pstep; }, 16 * hh + 8 * kk)
                       : *(const u16x8*)cb;
      }
      if constexpr (kDenseDst) {
        pg = 0;
      } else {
        pg = a.dst_pages[(ok ? n : nb0) >> 3];
      }
    };

    // One 32-token tile: distances, argmin, certification, index write or deferral.
    auto tile = [&](int n0, bool ok, const u16x8 (&B)[NH], int pg) {
      // keep the |C_k|^2 reads from LDS inside the tile (hoisted, they would take 128 VGPRs)
      asm volatile("" ::: "memory");
      const int n = n0 + col;
      // |x|^2 of the vector, only for the error bound
      float xx = 0.f;
  #pragma unroll
      for (int hh = 0; hh < NH; ++hh)
  #pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 two = __builtin_bit_cast(bf16x2, (uint32_t)B[hh][e] | ((uint32_t)B[hh][e + 1] << 16));
          xx = __builtin_amdgcn_fdot2_f32_bf16(two, two, xx, false);
        }
      {
        float lo, hi;
        pair32(xx, lo, hi);
        xx = lo + hi;
      }

      // The lane's 128 candidates (codes 32 b + 8 jj + 4 kk + r) become keys in two halves
      // of four blocks: D'_k with its six low mantissa bits replaced by
      // 63 - (16 (b mod 4) + 4 jj + r) (an inline constant, so one v_and_or_b32 per key).
      // A smaller key is a smaller D' at key precision.  Four chains (half, pair parity)
      // fold their keys a pair (x, y) at a time: the smallest key b1 becomes
      // min3(b1, x, y), and med3(b1, x, y) -- the second smallest of {b1, x, y} -- is a
      // candidate for the second smallest overall, which is the minimum of these
      // candidates (taken two at a time); 2.25 VALU per key.
      float c1[4], c2[4], pend[4];
  #pragma unroll
      for (int ch = 0; ch < 4; ++ch) c1[ch] = c2[ch] = pend[ch] = __builtin_inff();
      auto key = [](float v, int idx) {
        return __uint_as_float((__float_as_uint(v) & ~63u) | (63u - (uint32_t)idx));
      };
      // pairs [p0, p1) of block b (b, p0, p1 compile-time)
      auto fold = [&](const f32x16& acc, int b, int p0, int p1) {
  #pragma unroll
        for (int pi = p0; pi < p1; ++pi) {
          const int ch = 2 * (b >> 2) + (pi & 1);
          const float x = key(acc[2 * pi], 16 * (b & 3) + 2 * pi);
          const float y = key(acc[2 * pi + 1], 16 * (b & 3) + 2 * pi + 1);
          const float p = key_med3(c1[ch], x, y);
          c1[ch] = key_min3(c1[ch], x, y);
          if (pi & 2) c2[ch] = key_min3(c2[ch], pend[ch], p);
          else pend[ch] = p;
        }
      };
      // Blocks of 32 codes, software-pipelined: each block's accumulators start as
      // |C_k|^2, read from LDS before the first half of the previous block's fold; its
      // MFMAs issue between the two halves, so neither the LDS read nor the MFMAs sit
      // on the critical path (the scheduling barriers keep that order).
      auto bias_of = [&](int b) {
        f32x16 c;
  #pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 q = *(const f32x4*)(bias + 32 * b + 8 * jj);
  #pragma unroll
          for (int r = 0; r < 4; ++r) c[4 * jj + r] = q[r];
        }
        return c;
      };
      auto mfmas = [&](int b, f32x16 c) {
  #pragma unroll
        for (int hh = 0; hh < NH; ++hh) c = mfma32(A[b][hh], B[hh], c);
        return c;
      };
      f32x16 acc[2];
      acc[0] = mfmas(0, bias_of(0));
  #pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int cur = b & 1;
        if (b + 1 < NB) acc[cur ^ 1] = bias_of(b + 1);
        __builtin_amdgcn_sched_barrier(0);
        fold(acc[cur], b, 0, 4);
        __builtin_amdgcn_sched_barrier(0);
        if (b + 1 < NB) acc[cur ^ 1] = mfmas(b + 1, acc[cur ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
        fold(acc[cur], b, 4, 8);
      }
      // the halves' smallest and second smallest, then the lane's (keys of the two halves
      // share index bits: the half of the winner is kept aside; equal keys make b2 == b1)
      float m1[2], m2[2];
  #pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        m1[hf] = key_min(c1[2 * hf], c1[2 * hf + 1]);
        m2[hf] = key_min3(key_max(c1[2 * hf], c1[2 * hf + 1]), c2[2 * hf], c2[2 * hf + 1]);
      }
      const int half = m1[1] < m1[0] ? 1 : 0;
      float b1 = key_min(m1[0], m1[1]);
      float b2 = key_min3(key_max(m1[0], m1[1]), m2[0], m2[1]);
      // Merge the two lanes of the vector (lane ^ 32): smallest and second smallest key
      // overall, the same in both lanes.  The lane whose own smallest key survives holds
      // the winning code; equal keys in the two lanes make b2 == b1, which sends the
      // vector to the float64 pass.
      const float own = b1;
      {
        float lo1, hi1, lo2, hi2;
        pair32(b1, lo1, hi1);
        pair32(b2, lo2, hi2);
        b1 = key_min(lo1, hi1);
        b2 = key_min3(key_max(lo1, hi1), lo2, hi2);
      }
      const bool owner = own == b1;
      // Float32 error bound for the two distances and the six truncated key bits.  A
      // distance is |C_k|^2, rounded once, plus G exact products summed in float32: at
      // most G + 2 roundings of sums whose magnitudes stay below |C_k|^2 + 2 |x| |C_k|
      // <= S = max|C|^2 + 2 |x| max|C|, so each is within (G + 2) u S (u = 2^-24); the
      // tolerance takes 1.2 times that for two distances.  Products or sums below the
      // float32 normal range may be flushed to zero, an absolute error under 2^-126
      // per term: kTolAbs covers G + 2 of them per distance, so vectors of tiny
      // magnitude always go to the float64 pass (as do those whose S overflows, where
      // the tolerance is infinite).  The approximate square root only enters the bound.
      constexpr float kTolU = 2.4f * (G + 2);
      constexpr float kTolAbs = 2.f * (G + 2) * 1.17549435e-38f;
      const float S = cmax2 + 2.f * __builtin_amdgcn_sqrtf(xx * cmax2);
      const float tol = kTolU * 5.9604645e-8f * S + (3.0517578e-5f * fabsf(b1) + kTolAbs);
      const bool need_exact = ok && !(b2 - b1 > tol);
      uint8_t* o = nullptr;   // this lane's destination byte (vector col)
      if constexpr (kDenseDst) {
        o = dst_lane + (size_t)(n0 - nb0) * dst_stride;
      } else if (pg >= 0 && pg < a.n_dst_pages) {
        o = a.out + (((((size_t)pg * nblk + beta) * H + h) * 2 + kv) * kPage + (n & 7)) * NG + g;
      }
      if (ok && owner && !need_exact && o) {
        const uint32_t p = 63u - (__float_as_uint(b1) & 63u);
        *o = (uint8_t)(32 * (4 * half + (int)(p >> 4)) + 8 * (int)((p >> 2) & 3u) + 4 * kk + (int)(p & 3u));
      }
      // Vectors whose float32 decision is not certain: float64 from registers, one at a time.
      uint64_t todo = __ballot(need_exact && kk == 0);   // bits = vector columns
      while (todo) {
        const int cv = (int)__builtin_ctzll(todo);
        todo &= todo - 1;
        const int ex = exact_in_registers<NH, NB>(A, B, cv, lane);
        if (lane == cv && o) *o = (uint8_t)ex;
      }
    };

    // Buffer j is refilled right after its tile is consumed and used again kRing - 1
    // tiles later, so each load overlaps that much work.  The workgroup's waves meet at a
    // barrier once per kRing tiles: every 128-byte line of a token's row is read by the
    // four waves of this workgroup and by those of the workgroup of the neighbouring
    // groups, and waves left to drift apart over a long token range find the line evicted
    // from L2 between its readers (2.5 times the input read from memory at G = 32, 1.3
    // with the barrier).
    u16x8 Bq[kRing][NH];
    bool okq[kRing];
    int pgq[kRing];
#pragma unroll
    for (int jt = 0; jt < kRing; ++jt) fetch(nb0 + kTileTokens * jt, Bq[jt], okq[jt], pgq[jt]);
    for (int n0 = nb0; n0 < nb1; n0 += kTileTokens * kRing) {
#pragma unroll
      for (int jt = 0; jt < kRing; ++jt) {
        if (n0 + kTileTokens * jt < nb1) tile(n0 + kTileTokens * jt, okq[jt], Bq[jt], pgq[jt]);
        if (jt == kRing - 1) __syncthreads();   // n0, nb1: the same in every wave of the workgroup
        fetch(n0 + kTileTokens * (jt + kRing), Bq[jt], okq[jt], pgq[jt]);
      }
    }
  }
}

// Workgroups the device holds at once: the CU count times the workgroups per CU that
// the kernel's VGPR count allows (512 per SIMD lane, at most 8 waves per SIMD; a
// workgroup of W waves puts W / 4 waves on each SIMD), or the runtime's occupancy figure
// if that is higher.  Cached per device in the caller's cache (one per kernel instance).
template <typename K>
int resident_workgroups(K kernel, int threads, std::atomic<int> (&cache)[64]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  hipFuncAttributes fa{};
  if (hipFuncGetAttributes(&fa, (const void*)kernel) == hipSuccess && fa.numRegs > 0) {
    const int vgprs = (fa.numRegs + 7) / 8 * 8;
    int waves_per_simd = 512 / vgprs;
    if (waves_per_simd > 8) waves_per_simd = 8;
    const int wg_waves = (threads + 63) / 64;
    const int by_regs = 4 * waves_per_simd / wg_waves;
    if (by_regs > per_cu) per_cu = by_regs;
  }
  const int v = per_cu * cus;
  if (v > 0 && dev < 64) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

template <int G, int C, int D, int MODE>
hipError_t launch_mode(const EncodeArgs& args, const LayersArg<MODE>& layers, int n_layers, hipStream_t s) {
  constexpr int NG = D / C;
  constexpr int WPG = waves_per_group_block<D, C>();
  constexpr int NGB = NG / WPG;
  if (args.N <= 0) return hipSuccess;
  auto kernel = encode_kernel<G, C, D, MODE>;
  static std::atomic<int> slot_cache[64];   // this kernel instance's, per device
  int slots = resident_workgroups(kernel, WPG * 64, slot_cache);
  if (slots <= 0) slots = 256;
  const int round = kXcds * NGB;
  slots = slots / round * round;
  if (slots < round) slots = round;
  // split every (layer, head, block, K/V) codebook set into enough token ranges to fill
  // the slots (each range loads its codebook once, so no more ranges than that)
  const long sets = (long)args.H * (args.T / args.Tc) * (args.kv_sel < 0 ? 2 : 1);
  long parts = slots / (sets * NGB * n_layers);
  if (parts < 1) parts = 1;
  long tpi = (args.N + parts - 1) / parts;
  tpi = (tpi + kTileTokens - 1) / kTileTokens * kTileTokens;
  parts = (args.N + tpi - 1) / tpi;
  // heads whose dense index rows share 128-byte lines go to one XCD together
  int hb = args.H < 8 ? args.H : 8;
  while (args.H % hb) --hb;
  const long ncombo = parts * (sets / hb) * n_layers;
  const long items = (ncombo + kXcds - 1) / kXcds * kXcds * hb * NGB;
  if (items > INT32_MAX) return hipErrorInvalidValue;
  const long grid = items < slots ? items : slots;
  EncodeArgs a = args;
  a.tokens_per_block = (int)tpi;
  a.head_block = hb;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(WPG * 64), 0, s, a, (int)items, layers);
  return hipGetLastError();
}

template <int G, int C, int D>
hipError_t launch_one(const EncodeArgs& a, const ReencodeLayers* layers, hipStream_t s) {
  if (a.src_mode == kSrcPages) {
    // pages -> pages: the given layers, or the single layer the arguments name
    ReencodeLayers one{};
    if (!layers) {
      one.n = 1;
      one.layer[0] = {a.src, a.codebooks, a.out, a.n_src_pages, a.n_dst_pages};
      layers = &one;
    }
    if (layers->n < 1 || layers->n > kMaxReencodeLayers) return hipErrorInvalidValue;
    return launch_mode<G, C, D, 2>(a, *layers, layers->n, s);
  }
  if (a.dst_mode == kDstPages) return launch_mode<G, C, D, 1>(a, NoLayers{}, 1, s);
  return launch_mode<G, C, D, 0>(a, NoLayers{}, 1, s);
}

template <int G, int C>
hipError_t by_d(const EncodeArgs& a, const ReencodeLayers* layers, hipStream_t s) {
  if (a.d == 64) return launch_one<G, C, 64>(a, layers, s);
  return launch_one<G, C, 128>(a, layers, s);
}

}  // namespace

bool encode_supported(int G, int c, int d) {
  if (d != 64 && d != 128) return false;
  if (G == 32) return c == 8 || c == 16 || c == 32;
  if (G == 16) return c == 4 || c == 8 || c == 16;
  return false;
}

hipError_t launch_encode(const EncodeArgs& a, hipStream_t s, const ReencodeLayers* layers) {
  const int c = a.G / a.Tc;
  if (a.G == 32) {
    if (c == 8) return by_d<32, 8>(a, layers, s);
    if (c == 16) return by_d<32, 16>(a, layers, s);
    return by_d<32, 32>(a, layers, s);
  }
  if (c == 4) return by_d<16, 4>(a, layers, s);
  if (c == 8) return by_d<16, 8>(a, layers, s);
  return by_d<16, 16>(a, layers, s);
}

}  // namespace lvq
