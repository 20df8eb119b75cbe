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
//    It folds them in four chains of 16 with v_min3 on keys whose low four
//    mantissa bits carry the chain position (ordering ties toward the lowest
//    code for negative D'), then merges the chain winners and the four lanes
//    of the vector, tracking the runner-up among chain winners.
//  * Exactness: a vector is recomputed in float64 by direct differences over
//    all 256 codewords (the definition itself) when the minimum is not safely
//    negative or when its runner-up is within the float32 error bound of the
//    winner.  That keeps the chosen index equal to the float64 nearest
//    codeword except for candidates inside the float32 error band.
//  * A workgroup holds the waves of up to 8 consecutive groups of one
//    (block, head): together they read whole 128-byte rows of the cache, so
//    the K/V bytes are fetched from HBM once.
#include "lvq_internal.h"

namespace lvq {
namespace {

constexpr int kMaxTokensPerBlock = 512;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

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

// Float64 direct-difference nearest codeword of one vector, whole wave cooperating.
// Lane l scores codes l, l+64, l+128, l+192; ties resolve to the lowest code.
template <int G, int C>
__device__ __forceinline__ int exact_nearest(const EncodeArgs& a, const uint16_t* cb, int beta, int n,
                                          int h, int g, int kv, int lane) {
  constexpr int TC = G / C;
  double best = __builtin_inf();
  int bidx = 0x7fffffff;
#pragma unroll 1
  for (int j = 0; j < 4; ++j) {
    const int k = lane + 64 * j;
    double dsum = 0.0;
#pragma unroll 1
    for (int tau = 0; tau < TC; ++tau) {
      const uint16_t* row = src_row(a, beta * TC + tau, n, h, kv);
      const uint16_t* cw = cb + ((size_t)tau * kCodes + k) * C;
#pragma unroll 4
      for (int i = 0; i < C; ++i) {
        const double xv = row ? (double)bf2f(row[g * C + i]) : 0.0;
        const double df = xv - (double)bf2f(cw[i]);
        dsum = fma(df, df, dsum);
      }
    }
    if (dsum < best) { best = dsum; bidx = k; }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const double ob = __shfl_xor(best, off);
    const int oi = __shfl_xor(bidx, off);
    if (ob < best || (ob == best && oi < bidx)) { best = ob; bidx = oi; }
  }
  return bidx;
}

template <int G, int C, int D>
__global__ __launch_bounds__(512) void encode_kernel(EncodeArgs a) {
  constexpr int NG = D / C;
  constexpr int WPG = NG < 8 ? NG : 8;   // waves (groups) per workgroup
  constexpr int NGB = NG / WPG;
  constexpr int EPL = (G == 32) ? 8 : 4; // elements per lane per MFMA operand
  constexpr int TC = G / C;
  using R = raw_t<EPL>;
  __shared__ __attribute__((aligned(16))) float s_bias[WPG][kCodes];
  __shared__ int s_flag[WPG][kMaxTokensPerBlock];   // vectors left for the float64 pass
  __shared__ int s_nflag[WPG];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int H = a.H, N = a.N;
  const int nblk = a.T / TC;
  const int nchunk = (N + a.tokens_per_block - 1) / a.tokens_per_block;
  int bid = blockIdx.x;
  const int chunk = bid % nchunk; bid /= nchunk;
  const int gb = bid % NGB;       bid /= NGB;
  const int h = bid % H;          bid /= H;
  const int beta = bid % nblk;    bid /= nblk;
  const int kv = (a.kv_sel >= 0) ? a.kv_sel : bid;
  const int g = gb * WPG + wave;

  const int q4 = lane >> 4, col = lane & 15;
  const int e0 = EPL * q4;
  const int tau0 = e0 / C, i0 = e0 % C;

  // ---- the codebook as MFMA A operand, scaled by -2; |C_k|^2 for the bias
  const uint16_t* cb = a.codebooks + ((((size_t)beta * 2 + kv) * H + h) * NG + g) * ((size_t)TC * kCodes * C);
  R A[16];
  float cmax2 = 0.f;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const R v = *(const R*)(cb + ((size_t)tau0 * kCodes + 16 * m + col) * C + i0);
    R w;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float f = bf2f(v[e]);
      s = fmaf(f, f, s);
      w[e] = (uint16_t)(__float_as_uint(-2.f * f) >> 16);
    }
    A[m] = w;
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    cmax2 = fmaxf(cmax2, s);
    if (q4 == 0) s_bias[wave][16 * m + col] = s;
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) cmax2 = fmaxf(cmax2, __shfl_xor(cmax2, off));
  if (lane == 0) s_nflag[wave] = 0;
  __syncthreads();
  const float* bias = &s_bias[wave][4 * q4];

  const int nb0 = chunk * a.tokens_per_block;
  const int nb1 = min(N, nb0 + a.tokens_per_block);
  for (int n0 = nb0; n0 < nb1; n0 += 16) {
    const int n = n0 + col;
    const bool in_range = n < nb1;
    const uint16_t* row = in_range ? src_row(a, beta * TC + tau0, n, h, kv) : nullptr;
    R B;
#pragma unroll
    for (int e = 0; e < EPL; ++e) B[e] = 0;
    if (row) B = *(const R*)(row + g * C + i0);
    float xx = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) { const float f = bf2f(B[e]); xx = fmaf(f, f, xx); }
    xx += __shfl_xor(xx, 16);
    xx += __shfl_xor(xx, 32);

    // Argmin over the 256 expanded distances D'_k of this lane's vector.  Four
    // chains (one per accumulator row) of 16 candidates each are folded with
    // float min on keys whose low four mantissa bits hold the code block m;
    // the fill makes a tie at key precision go to the lowest code: 15 - m for
    // negative D' (a larger pattern is more negative), m for positive D'.  The
    // MFMAs are issued in two halves of 8 to bound the live accumulators.
    auto fold = [&](const bool positive, float& bv, float& sv, int& code) {
      float best[4] = {__builtin_inff(), __builtin_inff(), __builtin_inff(), __builtin_inff()};
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f32x4 acc[8];
#pragma unroll
        for (int mm = 0; mm < 8; ++mm) {
          const int m = 8 * half + mm;
          acc[mm] = mfma_bf16<EPL>(A[m], B, *(const f32x4*)(bias + 16 * m));
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int mm = 0; mm < 8; ++mm) {
            const int m = 8 * half + mm;
            const uint32_t fill = positive ? (uint32_t)m : (uint32_t)(15 - m);
            const uint32_t u = (__float_as_uint(acc[mm][r]) & 0xFFFFFFF0u) | fill;
            best[r] = fminf(best[r], __uint_as_float(u));
          }
        }
      }
      bv = best[0];
      sv = __builtin_inff();
      int rr = 0;
#pragma unroll
      for (int r = 1; r < 4; ++r) {
        if (best[r] < bv) { sv = bv; bv = best[r]; rr = r; }
        else sv = fminf(sv, best[r]);
      }
      const uint32_t low = __float_as_uint(bv) & 15u;
      const int m = positive ? (int)low : 15 - (int)low;
      code = 16 * m + 4 * q4 + rr;
#pragma unroll
      for (int off = 16; off <= 32; off <<= 1) {
        const float ob = __shfl_xor(bv, off);
        const float os = __shfl_xor(sv, off);
        const int oc = __shfl_xor(code, off);
        if (ob < bv || (ob == bv && oc < code)) { sv = fminf(bv, os); bv = ob; code = oc; }
        else sv = fminf(sv, fminf(ob, os));
      }
    };
    float bv, sv;
    int code;
    fold(false, bv, sv, code);
    if (__any(row != nullptr && !(bv < 0.f))) {
      float bv2, sv2;
      int code2;
      fold(true, bv2, sv2, code2);
      if (!(bv < 0.f)) { bv = bv2; sv = sv2; code = code2; }
    }
    // float32 error bound of two expanded distances plus the key truncation
    const float S = xx + cmax2 + 2.f * sqrtf(xx * cmax2);
    const float tol = 80.f * 5.9604645e-8f * S + 4.0f * 1.9073486e-6f * fabsf(bv);
    const bool need_exact = row && !(sv - bv > tol);
    const uint64_t todo = __ballot(need_exact && q4 == 0);
    if (todo) {
      const int base = s_nflag[wave];
      if (need_exact && q4 == 0) s_flag[wave][base + __popcll(todo & ((1ull << lane) - 1))] = n;
      if (lane == 0) s_nflag[wave] = base + __popcll(todo);
    }
    if (row && q4 == 0 && !need_exact) {
      uint8_t* o = dst_byte(a, beta, n, h, g, kv, NG);
      if (o) *o = (uint8_t)code;
    }
  }
  // float64 pass over the vectors whose float32 decision was not certain
  const int nflag = s_nflag[wave];
#pragma unroll 1
  for (int f = 0; f < nflag; ++f) {
    const int n = s_flag[wave][f];
    const int ex = exact_nearest<G, C>(a, cb, beta, n, h, g, kv, lane);
    if (lane == 0) {
      uint8_t* o = dst_byte(a, beta, n, h, g, kv, NG);
      if (o) *o = (uint8_t)ex;
    }
  }
}

template <int G, int C, int D>
hipError_t launch_one(const EncodeArgs& a, hipStream_t s) {
  constexpr int NG = D / C;
  constexpr int WPG = NG < 8 ? NG : 8;
  const int nblk = a.T / a.Tc;
  const int nchunk = (a.N + a.tokens_per_block - 1) / a.tokens_per_block;
  const long grid = (long)nchunk * (NG / WPG) * a.H * nblk * (a.kv_sel < 0 ? 2 : 1);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((encode_kernel<G, C, D>), dim3((unsigned)grid), dim3(WPG * 64), 0, s, a);
  return hipGetLastError();
}

template <int G, int C>
hipError_t by_d(const EncodeArgs& a, hipStream_t s) {
  if (a.d == 64) return launch_one<G, C, 64>(a, s);
  return launch_one<G, C, 128>(a, s);
}

}  // namespace

bool encode_supported(int G, int c, int d) {
  if (d != 64 && d != 128) return false;
  if (G == 32) return c == 8 || c == 16 || c == 32;
  if (G == 16) return c == 4 || c == 8 || c == 16;
  return false;
}

hipError_t launch_encode(const EncodeArgs& a, hipStream_t s) {
  const int c = a.G / a.Tc;
  if (a.G == 32) {
    if (c == 8) return by_d<32, 8>(a, s);
    if (c == 16) return by_d<32, 16>(a, s);
    return by_d<32, 32>(a, s);
  }
  if (c == 4) return by_d<16, 4>(a, s);
  if (c == 8) return by_d<16, 8>(a, s);
  return by_d<16, 16>(a, s);
}

}  // namespace lvq
