// LoopVQ codebook builder for gfx950: k-means++ seeding and Lloyd iterations.
//
// What it computes (LoopVQ summary, onedev.kr/papers/1681, section "어떻게 쓰나": the
// codebooks are learned by k-means on calibration keys and values): for every book
// (loop block beta, head h, group g) of one of K / V, the 256 codewords of the joint
// vectors x_s[tau*c + i] = X[beta*Tc + tau][s][h][g*c + i] of S sample tokens.
//  * Seeding: draw 0 picks sample floor(u_0 S); draw k >= 1 picks the first s whose
//    running sum D^2_0 + ... + D^2_s (sample order, float64) exceeds u_k times the total,
//    D^2 being the squared distance to the nearest chosen center; the last s with
//    D^2 > 0 if rounding leaves none; floor(u_k S) if every D^2 is 0.
//  * Lloyd iteration: assign every sample to the nearest center rounded to bf16 (the
//    stored codebook precision; the assignment is the encoder itself, exact with
//    lowest-index ties), then move each center to the float64 mean of its members,
//    summed in sample order; an empty cluster keeps its center.
//  * The final centers are rounded to bf16 through float32 (round to nearest even).
// Float64 sums are formed with separate multiply and add roundings in a fixed order,
// so every step is reproducible to the bit.
//
// Design (MI355X): one workgroup per book for the seeding (D^2 and its running sums
// in LDS, the running sum by one lane, the search by the whole workgroup) and for
// the update (one lane per cluster); the assignment is the MFMA encoder over all
// books at once.
#include "lvq_internal.h"

#include <cstdint>

namespace lvq {
namespace {

constexpr int kKmThreads = 256;

__device__ __forceinline__ double bf2d(uint16_t b) {
  return (double)__uint_as_float((uint32_t)b << 16);
}

// Joint vector of sample s for book (beta, h, g), as float64.
template <int G, int C>
__device__ __forceinline__ void load_joint(const KmeansArgs& a, int beta, int h, int g, int s,
                                           double (&x)[G]) {
  constexpr int TC = G / C;
#pragma unroll
  for (int tau = 0; tau < TC; ++tau) {
    const uint16_t* row = a.samples + (((size_t)(beta * TC + tau) * a.S + s) * a.H + h) * a.d + g * C;
#pragma unroll
    for (int i = 0; i < C; ++i) x[tau * C + i] = bf2d(row[i]);
  }
}

// sum_e (x[e] - c[e])^2, squares added in order e = 0, 1, ...
template <int G>
__device__ __forceinline__ double sq_dist(const double (&x)[G], const double* c) {
  double d = 0.0;
#pragma unroll
  for (int e = 0; e < G; ++e) {
    const double df = __dsub_rn(x[e], c[e]);
    d = __dadd_rn(d, __dmul_rn(df, df));
  }
  return d;
}

// floor(u * S) clamped into [0, S): a draw outside [0, 1) (or NaN) still names a sample
__device__ __forceinline__ int draw_index(double u, int S) {
  const double v = u * (double)S;
  if (!(v >= 0.0)) return 0;
  return v >= (double)(S - 1) ? S - 1 : (int)v;
}

__device__ __forceinline__ void book_coords(const KmeansArgs& a, int book, int ng, int& beta, int& h,
                                            int& g) {
  g = book % ng;
  h = (book / ng) % a.H;
  beta = book / (ng * a.H);
}

// ------------------------------------------------------------------ seeding
template <int G, int C>
__global__ __launch_bounds__(kKmThreads) void seed_kernel(KmeansArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* D2 = (double*)smem;          // [S]
  double* cum = D2 + a.S;              // [S] running sums
  __shared__ double cen[G];
  __shared__ double s_target;
  __shared__ int s_mode, s_pick, s_red[kKmThreads / 64];
  const int ng = a.d / C;
  const int book = blockIdx.x;
  int beta, h, g;
  book_coords(a, book, ng, beta, h, g);
  const double* u = a.draws + (size_t)book * kCodes;
  double* centers = a.centers + (size_t)book * kCodes * G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S;

  auto take = [&](int k, int pick) {
    // center k = sample `pick`: lane e < G copies element e = tau*c + i
    if (tid < G) {
      const int tau = tid / C, i = tid % C;
      const double v = bf2d(a.samples[(((size_t)(beta * (G / C) + tau) * S + pick) * a.H + h) * a.d + g * C + i]);
      cen[tid] = v;
      centers[(size_t)k * G + tid] = v;
    }
    __syncthreads();
  };
  take(0, draw_index(u[0], S));
  for (int s = tid; s < S; s += kKmThreads) {
    double x[G];
    load_joint<G, C>(a, beta, h, g, s, x);
    D2[s] = sq_dist<G>(x, cen);
  }
  for (int k = 1; k < kCodes; ++k) {
    __syncthreads();
    if (tid == 0) {
      double acc = 0.0;
      for (int s = 0; s < S; ++s) {
        acc = __dadd_rn(acc, D2[s]);
        cum[s] = acc;
      }
      if (acc > 0.0) {
        s_target = __dmul_rn(u[k], acc);
        s_mode = 1;
      } else {
        s_pick = draw_index(u[k], S);
        s_mode = 0;
      }
    }
    __syncthreads();
    if (s_mode == 1) {
      // first s with cum[s] > target; failing that, the last s with D2[s] > 0
      const double target = s_target;
      int first = INT32_MAX, last = -1;
      for (int s = tid; s < S; s += kKmThreads) {
        if (cum[s] > target && s < first) first = s;
        if (D2[s] > 0.0) last = s;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        first = min(first, __shfl_xor(first, off));
        last = max(last, __shfl_xor(last, off));
      }
      if (lane == 0) s_red[wave] = first;
      __syncthreads();
      if (tid == 0) {
        int f = INT32_MAX;
        for (int w = 0; w < kKmThreads / 64; ++w) f = min(f, s_red[w]);
        s_pick = f;
      }
      __syncthreads();
      if (s_pick == INT32_MAX) {
        if (lane == 0) s_red[wave] = last;
        __syncthreads();
        if (tid == 0) {
          int l = -1;
          for (int w = 0; w < kKmThreads / 64; ++w) l = max(l, s_red[w]);
          s_pick = l;
        }
      }
      __syncthreads();
    }
    take(k, s_pick);
    for (int s = tid; s < S; s += kKmThreads) {
      double x[G];
      load_joint<G, C>(a, beta, h, g, s, x);
      const double dn = sq_dist<G>(x, cen);
      if (dn < D2[s]) D2[s] = dn;
    }
  }
}

// ------------------------------------------------------------------ bf16 rounding
// centers [book][256][G] (float64) -> codebooks [nblk][2][H][ng][Tc][256][c], half kv_sel
__global__ void round_kernel(KmeansArgs a, int G, int C) {
  const int ng = a.d / C, TC = G / C;
  const size_t n = (size_t)a.n_books * kCodes * G;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int e = (int)(i % G);
    const int k = (int)((i / G) % kCodes);
    const int book = (int)(i / ((size_t)G * kCodes));
    const int gg = book % ng, h = (book / ng) % a.H, beta = book / (ng * a.H);
    const int tau = e / C, ci = e % C;
    const uint32_t bits = __float_as_uint((float)a.centers[i]);
    const uint16_t bf = (uint16_t)((bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16);
    a.codebooks[((((((size_t)beta * 2 + a.kv_sel) * a.H + h) * ng + gg) * TC + tau) * kCodes + k) * C + ci] = bf;
  }
}

// ------------------------------------------------------------------ update
template <int G, int C>
__global__ __launch_bounds__(kKmThreads) void update_kernel(KmeansArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint8_t* asg = smem;                 // [S] cluster of each sample
  const int ng = a.d / C;
  const int book = blockIdx.x;
  int beta, h, g;
  book_coords(a, book, ng, beta, h, g);
  const int S = a.S;
  for (int s = threadIdx.x; s < S; s += kKmThreads)
    asg[s] = a.assign[(((size_t)beta * S + s) * a.H + h) * ng + g];
  __syncthreads();
  const int k = threadIdx.x;           // one cluster per lane
  double acc[G];
#pragma unroll
  for (int e = 0; e < G; ++e) acc[e] = 0.0;
  int cnt = 0;
  for (int s = 0; s < S; ++s) {
    if (asg[s] == k) {
      double x[G];
      load_joint<G, C>(a, beta, h, g, s, x);
#pragma unroll
      for (int e = 0; e < G; ++e) acc[e] = __dadd_rn(acc[e], x[e]);
      ++cnt;
    }
  }
  if (cnt > 0) {
    double* c = a.centers + ((size_t)book * kCodes + k) * G;
    const double n = (double)cnt;
#pragma unroll
    for (int e = 0; e < G; ++e) c[e] = __ddiv_rn(acc[e], n);
  }
}

template <int G, int C>
hipError_t build_t(const KmeansArgs& a, hipStream_t s) {
  const size_t seed_lds = (size_t)2 * a.S * sizeof(double);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)seed_kernel<G, C>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)(2 * kMaxKmeansSamples * sizeof(double)));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((seed_kernel<G, C>), dim3(a.n_books), dim3(kKmThreads), seed_lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rgrid = (int)((a.n_books * (size_t)kCodes * G + 255) / 256);
  for (int it = 0; it < a.n_iter; ++it) {
    hipLaunchKernelGGL(round_kernel, dim3(rgrid), dim3(256), 0, s, a, G, C);
    EncodeArgs ea{};
    ea.src = a.samples;
    ea.codebooks = a.codebooks;
    ea.out = a.assign;
    ea.src_mode = kSrcDense;
    ea.dst_mode = kDstDense;
    ea.kv_sel = a.kv_sel;
    ea.T = a.T;
    ea.Tc = a.Tc;
    ea.G = G;
    ea.N = a.S;
    ea.H = a.H;
    ea.d = a.d;
    ea.tokens_per_block = 512;
    e = launch_encode(ea, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((update_kernel<G, C>), dim3(a.n_books), dim3(kKmThreads), (size_t)a.S, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(round_kernel, dim3(rgrid), dim3(256), 0, s, a, G, C);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_build_codebooks(const KmeansArgs& a, hipStream_t s) {
  const int c = a.G / a.Tc;
  if (a.G == 32) {
    if (c == 8) return build_t<32, 8>(a, s);
    if (c == 16) return build_t<32, 16>(a, s);
    return build_t<32, 32>(a, s);
  }
  if (c == 4) return build_t<16, 4>(a, s);
  if (c == 8) return build_t<16, 8>(a, s);
  return build_t<16, 16>(a, s);
}

}  // namespace lvq
