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
//    pre-scaled by -2 (exact in bf16), sit in VGPRs as the A operand of 16
//    MFMAs (rows = codes); a 16-token tile of joint vectors is the B operand
//    (columns = vectors), loaded straight from the cache in the layout the
//    MFMA wants (8 or 4 contiguous channels of one loop step per lane).  The
//    accumulator input is |C_k|^2, so each MFMA returns D'_k = |C_k|^2 - 2 x.C_k
//    = |x - C_k|^2 - |x|^2 for 16 codes x 16 vectors, float32.
//  * Argmin: each lane holds 64 candidates of one vector (16 MFMAs x 4 rows).
//    Each becomes a key, D' with its six low mantissa bits replaced by the
//    candidate's position; keys are folded three at a time (v_min3, v_med3)
//    into the lane's smallest and second smallest key, then the four lanes of
//    the vector merge.
//  * Exactness: a vector is recomputed in float64 by direct differences over
//    all 256 codewords (the definition itself) when its second smallest key is
//    within the float32 error bound of the smallest.  So the chosen index is the
//    float64 nearest codeword with lowest-index ties: float32 decides only where
//    no other candidate can be within rounding of the winner.
//  * Input tiles (16 tokens) are loaded two tiles ahead of their use; the |C_k|^2
//    of the next group of MFMAs is read from LDS while the current group folds.
//  * A workgroup holds the waves of up to 4 consecutive groups of one
//    (block, head); the workgroups that read the other halves of the same
//    128-byte cache rows run on the same XCD at the same time, so the K/V
//    bytes are fetched from HBM once.
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

// Exchange with lane ^ 16 (v_permlane16_swap) or lane ^ 32 (v_permlane32_swap), VALU
// instructions with no LDS round trip.  Each lane gets its own value and its partner's
// as (lo, hi), where lo is the value of the pair's lower lane on both lanes, so an
// operation of (lo, hi) gives bit-identical results in the two lanes.
__device__ __forceinline__ void pair16(float v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

template <int EPL>
using raw_t = typename std::conditional<EPL == 8, u16x8, u16x4>::type;

template <int EPL>
__device__ __forceinline__ f32x4 mfma_bf16(raw_t<EPL> a, raw_t<EPL> b, f32x4 c) {
  if constexpr (EPL == 8) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  }
}

// Row of channels of (loop step t, token n, head h) in the source, or null if the token is absent.
__device__ __forceinline__ const uint16_t* src_row(const EncodeArgs& a, int t, int n, int h, int kv) {
  if (a.src_mode == kSrcDense) {
    return a.src + ((size_t)((size_t)t * a.N + n) * a.H + h) * a.d;
  }
  const int P = a.src_pages[n >> 3];
  if (P < 0 || P >= a.n_src_pages) return nullptr;
  return a.src + (((((size_t)P * a.T + t) * a.H + h) * 2 + kv) * kPage + (n & 7)) * a.d;
}

__device__ __forceinline__ uint8_t* dst_byte(const EncodeArgs& a, int beta, int n, int h, int g,
                                             int kv, int ng) {
  const int nblk = a.T / a.Tc;
  if (a.dst_mode == kDstDense) {
    return a.out + ((size_t)((size_t)beta * a.N + n) * a.H + h) * ng + g;
  }
  const int P = a.dst_pages[n >> 3];
  if (P < 0 || P >= a.n_dst_pages) return nullptr;
  return a.out + (((((size_t)P * nblk + beta) * a.H + h) * 2 + kv) * kPage + (n & 7)) * ng + g;
}

// Float64 direct-difference nearest codeword of vector column cv of the current tile,
// computed from registers: the wave holds the codebook as MFMA operand (A[m] = -2 C,
// exact) and the tile as operand B (lane (q4, col) holds elements e0..e0+EPL-1 of
// vector col).  Lane (q4, col) sums its EPL elements for codes 16m + col, the four
// lanes of a column add their parts (the same sum in every lane), and the 16 columns
// compare.  Ties resolve to the lowest code.
template <int EPL, typename R>
__device__ __forceinline__ int exact_in_registers(const R (&A)[16], const R& B, int cv, int lane) {
  const int q4 = lane >> 4, col = lane & 15;
  const int src = (q4 << 4) | cv;
  double x[EPL];
#pragma unroll
  for (int e = 0; e < EPL; e += 2) {
    const uint32_t w = (uint32_t)__shfl((int)((uint32_t)B[e] | ((uint32_t)B[e + 1] << 16)), src);
    x[e] = (double)bf2f((uint16_t)(w & 0xffffu));
    x[e + 1] = (double)bf2f((uint16_t)(w >> 16));
  }
  double best = __builtin_inf();
  int bidx = 0;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    double part = 0.0;
#pragma unroll
    for (int e = 0; e < EPL; e += 2) {
      // opaque copy: keeps the conversions here instead of hoisted out of the token loop
      uint32_t w = (uint32_t)A[m][e] | ((uint32_t)A[m][e + 1] << 16);
      asm volatile("" : "+v"(w));
      const double d0 = fma(0.5, (double)bf2f((uint16_t)(w & 0xffffu)), x[e]);   // x - C, A = -2 C
      const double d1 = fma(0.5, (double)bf2f((uint16_t)(w >> 16)), x[e + 1]);
      part = fma(d0, d0, part);
      part = fma(d1, d1, part);
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    if (part < best) { best = part; bidx = 16 * m + col; }   // m ascending: lowest code kept
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
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
// items of one (token range, head, loop block, K/V) that read the same 128-byte
// rows differ only in the group block and are numbered 8 apart, so with a grid that
// is a multiple of 8 x (group blocks) they run on the same XCD (round-robin
// dispatch) at the same time and each row is fetched from HBM once.
constexpr int kXcds = 8;

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
  constexpr int EPL = (G == 32) ? 8 : 4; // elements per lane per MFMA operand
  constexpr int TC = G / C;
  constexpr int kPart = 4;               // MFMAs issued before their results are folded
  constexpr int kRing = 3;               // tiles in flight
  using R = raw_t<EPL>;
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
  const int q4 = lane >> 4, col = lane & 15;
  const int e0 = EPL * q4;
  const int tau0 = e0 / C, i0 = e0 % C;

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int xcd = item % kXcds;
    const int j = item / kXcds;
    const int inner = j % per_combo;
    int rest = (j / per_combo) * kXcds + xcd;   // the combo
    if (rest >= ncombo) continue;   // padding to whole XCD rounds (uniform per workgroup)
    const int gb = inner % NGB;
    const int hh = inner / NGB;
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
    const int h = (rest % nhb) * HB + hh; rest /= nhb;
    const int beta = rest % nblk;   rest /= nblk;
    const int kv = (a.kv_sel >= 0) ? a.kv_sel : rest;
    const int g = gb * WPG + wave;
    const int nb0 = part * tpi;
    const int nb1 = min(N, nb0 + tpi);

    // ---- the codebook as MFMA A operand, scaled by -2 (exact); |C_k|^2 in float64, rounded once
    const uint16_t* cb = a.codebooks + ((((size_t)beta * 2 + kv) * H + h) * NG + g) * ((size_t)TC * kCodes * C);
    R A[16];
    float cmax2 = 0.f;
  #pragma unroll
    for (int m = 0; m < 16; ++m) {
      const R v = *(const R*)(cb + ((size_t)tau0 * kCodes + 16 * m + col) * C + i0);
      R w;
      double s = 0.0;
  #pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float f = bf2f(v[e]);
        s = fma((double)f, (double)f, s);
        w[e] = (uint16_t)(__float_as_uint(-2.f * f) >> 16);
      }
      A[m] = w;
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      const float sf = (float)s;
      cmax2 = fmaxf(cmax2, sf);
      if (q4 == 0) s_bias[wave][16 * m + col] = sf;
    }
  #pragma unroll
    for (int off = 1; off < 16; off <<= 1) cmax2 = fmaxf(cmax2, __shfl_xor(cmax2, off));
    const float* bias = &s_bias[wave][4 * q4];
    // Dense rows of the lane's (loop step, channel slice) start at src_base + n * H * d;
    // the lane's source and destination pointers advance by one tile (16 tokens) per step.
    const size_t src_stride = (size_t)H * a.d;
    const size_t dst_stride = (size_t)H * NG;
    const uint16_t* src_base = a.src + ((size_t)(beta * TC + tau0) * N * H + h) * a.d + g * C + i0;
    const uint16_t* src_any = src_base + (size_t)nb0 * src_stride;   // a readable row of this block
    const uint16_t* src_lane = src_base + (size_t)(nb0 + col) * src_stride;
    uint8_t* dst_lane = a.out + ((size_t)beta * N * H + h) * NG + g + (size_t)(nb0 + col) * dst_stride;

    // Load the lane's channel slice of tile n0 (and its destination page id).  Every load
    // is unconditional, a slot past the range reading a row of this block and a missing
    // bf16 page reading the codebook, so the compiler can count the loads in flight; ok
    // says whether the slot is a real token.
    auto fetch = [&](int n0, R& v, bool& ok, int& pg) {
      const int n = n0 + col;
      ok = n < nb1;
      const uint16_t* ptr;
      if constexpr (kDenseSrc) {
        ptr = ok ? src_lane + (size_t)(n0 - nb0) * src_stride : src_any;
      } else {
        const uint16_t* r = src_row(a, beta * TC + tau0, ok ? n : nb0, h, kv);
        ok = ok && r != nullptr;
        ptr = r ? r + g * C + i0 : cb;
      }
      v = *(const R*)ptr;
      if constexpr (kDenseDst) {
        pg = 0;
      } else {
        pg = a.dst_pages[(ok ? n : nb0) >> 3];
      }
    };

    // One 16-token tile: distances, argmin, certification, index write or deferral.
    auto tile = [&](int n0, bool ok, const R& B, int pg) {
      // keep the |C_k|^2 reads from LDS inside the tile (hoisted, they would take 64 VGPRs)
      asm volatile("" ::: "memory");
      const int n = n0 + col;
      // |x|^2 of the vector, only for the error bound
      float xx = 0.f;
  #pragma unroll
      for (int e = 0; e < EPL; e += 2) {
        const bf16x2 two = __builtin_bit_cast(bf16x2, (uint32_t)B[e] | ((uint32_t)B[e + 1] << 16));
        xx = __builtin_amdgcn_fdot2_f32_bf16(two, two, xx, false);
      }
      {
        float lo, hi;
        pair16(xx, lo, hi);
        xx = lo + hi;
        pair32(xx, lo, hi);
        xx = lo + hi;
      }

      // The lane's 64 candidates (codes 16m + 4 q4 + r) become keys: D'_k with its six
      // low mantissa bits replaced by 63 - (4m + r).  A smaller key is a smaller D' at
      // key precision, and every key of the lane is distinct.  Two chains (rows 0-1 and
      // rows 2-3 of each MFMA) fold their keys a pair (x, y) at a time: the smallest key
      // b1 becomes min3(b1, x, y), and med3(b1, x, y) -- the second smallest of
      // {b1, x, y} -- is a candidate for the second smallest overall, which is the
      // minimum of these candidates (taken two at a time); 2.25 VALU per key.
      float c1[2] = {__builtin_inff(), __builtin_inff()};
      float c2[2] = {__builtin_inff(), __builtin_inff()};
      float pend[2] = {__builtin_inff(), __builtin_inff()};
      auto key = [](float v, int idx) {
        return __uint_as_float((__float_as_uint(v) & ~63u) | (63u - (uint32_t)idx));
      };
      auto fold = [&](const f32x4& acc, int m) {   // m: compile-time MFMA number
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          const float x = key(acc[2 * ch], 4 * m + 2 * ch);
          const float y = key(acc[2 * ch + 1], 4 * m + 2 * ch + 1);
          const float p = key_med3(c1[ch], x, y);
          c1[ch] = key_min3(c1[ch], x, y);
          if (m & 1) c2[ch] = key_min3(c2[ch], pend[ch], p);
          else pend[ch] = p;
        }
      };
      // MFMA groups of kPart codes-blocks, software-pipelined: group p + 1 is issued
      // before group p is folded.  Each group's accumulators start as |C_k|^2, read from
      // LDS one group ahead.
      constexpr int NP = 16 / kPart;
      f32x4 acc[2][kPart];
#pragma unroll
      for (int mm = 0; mm < kPart; ++mm) acc[0][mm] = *(const f32x4*)(bias + 16 * mm);
#pragma unroll
      for (int mm = 0; mm < kPart; ++mm) acc[0][mm] = mfma_bf16<EPL>(A[mm], B, acc[0][mm]);
#pragma unroll
      for (int part = 0; part < NP; ++part) {
        const int cur = part & 1;
        if (part + 1 < NP) {
#pragma unroll
          for (int mm = 0; mm < kPart; ++mm)
            acc[cur ^ 1][mm] = *(const f32x4*)(bias + 16 * (kPart * (part + 1) + mm));
#pragma unroll
          for (int mm = 0; mm < kPart; ++mm)
            acc[cur ^ 1][mm] = mfma_bf16<EPL>(A[kPart * (part + 1) + mm], B, acc[cur ^ 1][mm]);
        }
#pragma unroll
        for (int mm = 0; mm < kPart; ++mm) fold(acc[cur][mm], kPart * part + mm);
      }
      float b1 = key_min(c1[0], c1[1]);
      float b2 = key_min3(key_max(c1[0], c1[1]), c2[0], c2[1]);
      // Merge the four lanes of the vector (lane ^ 16, then lane ^ 32): smallest and second
      // smallest key overall, the same in all four lanes.  The lane whose own smallest key
      // survives holds the winning code.
      const float own = b1;
      {
        float lo1, hi1, lo2, hi2;
        pair16(b1, lo1, hi1);
        pair16(b2, lo2, hi2);
        b1 = key_min(lo1, hi1);
        b2 = key_min3(key_max(lo1, hi1), lo2, hi2);
        pair32(b1, lo1, hi1);
        pair32(b2, lo2, hi2);
        b1 = key_min(lo1, hi1);
        b2 = key_min3(key_max(lo1, hi1), lo2, hi2);
      }
      const bool owner = own == b1;
      // Float32 error bound for two expanded distances (33 or 17 rounded terms, each
      // sum bounded by S = (|x| + max|C|)^2, plus the rounded |C|^2) and the six
      // truncated key bits; the approximate square root only enters the bound.
      const float S = xx + cmax2 + 2.f * __builtin_amdgcn_sqrtf(xx * cmax2);
      const float tol = 80.f * 5.9604645e-8f * S + 3.0517578e-5f * fabsf(b1);
      const bool need_exact = ok && !(b2 - b1 > tol);
      uint8_t* o = nullptr;   // this lane's destination byte (vector col)
      if constexpr (kDenseDst) {
        o = dst_lane + (size_t)(n0 - nb0) * dst_stride;
      } else if (pg >= 0 && pg < a.n_dst_pages) {
        o = a.out + (((((size_t)pg * nblk + beta) * H + h) * 2 + kv) * kPage + (n & 7)) * NG + g;
      }
      if (ok && owner && !need_exact && o) {
        const uint32_t p = 63u - (__float_as_uint(b1) & 63u);
        *o = (uint8_t)(16 * (int)(p >> 2) + 4 * q4 + (int)(p & 3u));
      }
      // Vectors whose float32 decision is not certain: float64 from registers, one at a time.
      uint64_t todo = __ballot(need_exact && q4 == 0);   // bits = vector columns
      while (todo) {
        const int cv = (int)__builtin_ctzll(todo);
        todo &= todo - 1;
        const int ex = exact_in_registers<EPL>(A, B, cv, lane);
        if (lane == cv && o) *o = (uint8_t)ex;
      }
    };

    // Buffer j is refilled right after its tile is consumed and used again kRing - 1
    // tiles later, so each load overlaps that much work.
    R Bq[kRing];
    bool okq[kRing];
    int pgq[kRing];
#pragma unroll
    for (int j = 0; j < kRing; ++j) fetch(nb0 + 16 * j, Bq[j], okq[j], pgq[j]);
    for (int n0 = nb0; n0 < nb1; n0 += 16 * kRing) {
#pragma unroll
      for (int j = 0; j < kRing; ++j) {
        if (n0 + 16 * j < nb1) tile(n0 + 16 * j, okq[j], Bq[j], pgq[j]);
        fetch(n0 + 16 * (j + kRing), Bq[j], okq[j], pgq[j]);
      }
    }
  }
}

// Workgroups per CU the kernel reaches and the device's CU count, cached per device.
template <typename K>
int resident_workgroups(K kernel, int threads) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
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
  int slots = resident_workgroups(kernel, WPG * 64);
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
  tpi = (tpi + 15) / 16 * 16;
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
