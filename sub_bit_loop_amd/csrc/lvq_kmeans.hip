// LoopVQ codebook builder for gfx950: k-means++ seeding and Lloyd iterations.
//
// What it computes (LoopVQ summary, onedev.kr/papers/1681, section "무엇과 다른가":
// the codebooks are initialised by Fisher-weighted k-means; section "전제와 한계",
// experiments paragraph: a k-means calibration on calibration sequences, timed per model): for every book (loop block beta,
// head h, group g) of one of K / V, the 256 codewords of the joint vectors
// x_s[tau*c + i] = X[beta*Tc + tau][s][h][g*c + i] of S sample tokens, each with a
// weight w_s >= 0 (all 1 when no weights are given; the weights stand in for the
// Fisher information, which needs model gradients).
//  * Seeding: draw k picks the first s whose running sum of terms (sample order,
//    float64) exceeds u_k times the total; the last s with a positive term if
//    rounding leaves none; floor(u_k S) if the total is not positive.  The terms are
//    w_s for draw 0 (so sample floor(u_0 S) without weights) and w_s D^2_s for k >= 1,
//    D^2 being the squared distance to the nearest chosen center.
//  * Lloyd iteration: assign every sample to the nearest center rounded to bf16 (the
//    stored codebook precision; the assignment is the encoder itself, exact with
//    lowest-index ties), then move each center to sum(w_s x_s) / sum(w_s) over its
//    members, both sums in sample order; a cluster with zero total weight (no
//    members, in particular) keeps its center.
//  * The final centers are rounded to bf16 through float32 (round to nearest even).
// Float64 sums are formed with separate multiply and add roundings in a fixed order,
// so every step is reproducible to the bit; with all weights 1 the products are
// exact and the result is plain k-means.
//
// Design (MI355X): one workgroup per book.  Workgroups are dealt to the 8 XCDs
// round-robin; blocks are mapped to books so that each XCD gets a run of neighbouring
// channel groups, which share the 128-byte lines of the sample rows in its L2.
//  * Seeding (512 threads): each thread owns up to 8 samples whose joint vectors
//    (packed bf16, S <= 4096), D^2 and weights stay in its registers for all 256
//    draws, so the samples are read from HBM once.  LDS holds the terms, which one
//    lane sums in order: a chain of dependent float64 adds, with the next 16 terms
//    loaded into registers while the current 16 are added, keeping only the sum at
//    the end of each batch of 16.  Terms are >= 0, so the sums never decrease and
//    the crossing lies in the first batch whose end sum crosses; the workgroup
//    finds that batch, one lane redoes its 16 sums, and the workgroup refreshes D^2
//    against the new center.  Above 4096 samples the joint vectors are re-read
//    from memory on every draw.
//  * The update sorts the samples by cluster once (a counting sort; one wave places
//    64 samples at a time in sample order, so each cluster's list stays ascending),
//    stages 512 samples' joint vectors in LDS at a time, and lets lane k walk the
//    members of cluster k: the lanes run their own lists side by side instead of
//    the wave stepping through every sample.
//  * The assignment is the MFMA encoder over all books at once.
#include "lvq_internal.h"

#include <cstdint>

namespace lvq {
namespace {

constexpr int kKmThreads = 256;
constexpr int kKmXcds = 8;
constexpr int kChain = 16;     // running-sum batch; D^2 arrays are padded with zeros to 2 batches
constexpr int kStage = 512;    // samples staged in LDS per update pass

__device__ __forceinline__ double bf2d(uint16_t b) {
  return (double)__uint_as_float((uint32_t)b << 16);
}

// workgroup -> book: XCD x (= block mod 8) gets books [x n/8, (x+1) n/8) when 8 divides n
__device__ __forceinline__ int book_of_block(int b, int n) {
  if (n % kKmXcds) return b;
  return (b % kKmXcds) * (n / kKmXcds) + b / kKmXcds;
}

struct Book {
  int beta, h, g, ng;
  const uint16_t* base;   // samples + ((beta*Tc*S)*H + h)*d + g*c: element (tau, s, i) at
                          // base[(tau*S + s)*H*d + i]
  size_t wstride;         // weights / assignments: element s at [(beta*S + s)*H*ng + h*ng + g]
  size_t wbase;
};

template <int G, int C>
__device__ __forceinline__ Book book_at(const KmeansArgs& a, int book) {
  Book bk;
  bk.ng = a.d / C;
  bk.g = book % bk.ng;
  bk.h = (book / bk.ng) % a.H;
  bk.beta = book / (bk.ng * a.H);
  bk.base = a.samples + ((size_t)bk.beta * (G / C) * a.S * a.H + bk.h) * a.d + bk.g * C;
  bk.wstride = (size_t)a.H * bk.ng;
  bk.wbase = (size_t)bk.beta * a.S * bk.wstride + (size_t)bk.h * bk.ng + bk.g;
  return bk;
}

// floor(u * S) clamped into [0, S): a draw outside [0, 1) (or NaN) still names a sample
__device__ __forceinline__ int draw_index(double u, int S) {
  const double v = u * (double)S;
  if (!(v >= 0.0)) return 0;
  return v >= (double)(S - 1) ? S - 1 : (int)v;
}

// ------------------------------------------------------------------ seeding
constexpr int kSeedThreads = 512;
constexpr int kSeedWaves = kSeedThreads / 64;
constexpr int kSeedRegPer = 8;     // samples per thread kept in registers (S <= 4096)
constexpr int kSeedMaxPer = kMaxKmeansSamplesLds / kSeedThreads;

// C bf16 values at p (8-byte aligned, 16-byte when 8 divides C) -> C/2 packed words
template <int C>
__device__ __forceinline__ void load_piece(const uint16_t* p, uint32_t* w) {
  if constexpr (C % 8 == 0) {
#pragma unroll
    for (int q = 0; q < C / 8; ++q) {
      const uint4 v = ((const uint4*)p)[q];
      w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < C / 4; ++q) {
      const uint2 v = ((const uint2*)p)[q];
      w[2 * q] = v.x; w[2 * q + 1] = v.y;
    }
  }
}

// element e of a joint vector held as packed bf16 words, as float64
__device__ __forceinline__ double packed_elem(const uint32_t* w, int e) {
  const uint32_t v = w[e >> 1];
  return (double)__uint_as_float((e & 1) ? (v & 0xFFFF0000u) : (v << 16));
}

template <int G, int C>
__device__ __forceinline__ void load_packed(const KmeansArgs& a, const Book& bk, int s, uint32_t (&w)[G / 2]) {
  const size_t tstride = (size_t)a.S * a.H * a.d;
  const uint16_t* row = bk.base + (size_t)s * a.H * a.d;
#pragma unroll
  for (int tau = 0; tau < G / C; ++tau) load_piece<C>(row + tau * tstride, w + tau * (C / 2));
}

// Thread t owns samples j * 512 + t, j < NPER: their D^2 (and weights) live in
// registers, and with REG their joint vectors too (read from HBM once instead of
// once per draw).  LDS holds only the terms / running sums the chain walks.
template <int G, int C, int NPER, bool REG>
__global__ __launch_bounds__(kSeedThreads) void seed_kernel(KmeansArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int S = a.S;
  const int Sp = (S + 2 * kChain - 1) / (2 * kChain) * (2 * kChain);
  double* run = (double*)smem;   // [Sp] terms w_s D^2_s; pad = 0
  double* ckpt = run + Sp;       // [Sp / 16] running sum at the end of each batch of 16 terms
  __shared__ double cen[G];
  __shared__ double s_total;
  __shared__ int s_first[kSeedWaves], s_last[kSeedWaves], s_pick;
  const int book = book_of_block(blockIdx.x, a.n_books);
  const Book bk = book_at<G, C>(a, book);
  const double* u = a.draws + (size_t)book * kCodes;
  double* centers = a.centers + (size_t)book * kCodes * G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  uint32_t xr[REG ? NPER : 1][G / 2];
  double d2[NPER], w[REG ? NPER : 1];   // without REG the weights are re-read when needed
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const int s = j * kSeedThreads + tid;
    d2[j] = 1.0;          // draw 0 takes every distance as 1: it picks by weight alone
    if constexpr (REG) {
      w[j] = 1.0;
      if (s < S) {
        if (a.weights) w[j] = a.weights[bk.wbase + (size_t)s * bk.wstride];
        load_packed<G, C>(a, bk, s, xr[j]);
      }
    }
  }
  auto term = [&](int j) {
    if (!a.weights) return d2[j];
    const double wj = REG ? w[REG ? j : 0] : a.weights[bk.wbase + (size_t)(j * kSeedThreads + tid) * bk.wstride];
    return __dmul_rn(wj, d2[j]);
  };
  auto publish = [&]() {
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      const int s = j * kSeedThreads + tid;
      if (s < Sp) run[s] = s < S ? term(j) : 0.0;
    }
  };
  publish();
  for (int k = 0; k < kCodes; ++k) {
    __syncthreads();
    if (tid == 0) {
      // running sum in sample order over two register batches: one batch is loaded
      // while the other is added (the empty asm statements keep the loads ahead).
      // Only each batch's last sum is stored: for terms >= 0 the sums never
      // decrease, so the crossing lies in the first batch whose last sum crosses.
      double acc = 0.0;
      double ba[kChain], bb[kChain];
#pragma unroll
      for (int j = 0; j < kChain; ++j) ba[j] = run[j];
      for (int s0 = 0; s0 < Sp; s0 += 2 * kChain) {
        const int nb = s0 + kChain;
#pragma unroll
        for (int j = 0; j < kChain; ++j) bb[j] = run[nb + j];
        asm volatile("" ::: "memory");
#pragma unroll
        for (int j = 0; j < kChain; ++j) acc = __dadd_rn(acc, ba[j]);
        ckpt[s0 / kChain] = acc;
        const int na = s0 + 2 * kChain < Sp ? s0 + 2 * kChain : 0;   // last pass: an unused reload
#pragma unroll
        for (int j = 0; j < kChain; ++j) ba[j] = run[na + j];
        asm volatile("" ::: "memory");
#pragma unroll
        for (int j = 0; j < kChain; ++j) acc = __dadd_rn(acc, bb[j]);
        ckpt[nb / kChain] = acc;
      }
      s_total = acc;
    }
    __syncthreads();
    const double total = s_total;
    int pick;
    if (total > 0.0) {
      // first batch whose last sum exceeds the target; the last s with a positive term
      const double target = __dmul_rn(u[k], total);
      int fb = INT32_MAX, last = -1;
      for (int b = tid; b < Sp / kChain; b += kSeedThreads)
        if (ckpt[b] > target) {
          fb = b;
          break;
        }
#pragma unroll
      for (int j = NPER - 1; j >= 0; --j) {
        const int s = j * kSeedThreads + tid;
        if (s < S && last < 0 && term(j) > 0.0) last = s;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        fb = min(fb, __shfl_xor(fb, off));
        last = max(last, __shfl_xor(last, off));
      }
      if (lane == 0) {
        s_first[wave] = fb;
        s_last[wave] = last;
      }
      __syncthreads();
      if (tid == 0) {
        int f = INT32_MAX, l = -1;
#pragma unroll
        for (int v = 0; v < kSeedWaves; ++v) {
          f = min(f, s_first[v]);
          l = max(l, s_last[v]);
        }
        int p;
        if (f != INT32_MAX) {
          // redo that batch's sums from the previous batch's last one: same values as the chain
          double acc = f > 0 ? ckpt[f - 1] : 0.0;
          p = f * kChain + kChain - 1;
          for (int j = 0; j < kChain; ++j) {
            acc = __dadd_rn(acc, run[f * kChain + j]);
            if (acc > target) {
              p = f * kChain + j;
              break;
            }
          }
        } else {
          // a positive total has a positive term, so l >= 0; the clamp only guards the index
          p = l >= 0 ? l : 0;
        }
        s_pick = p < S ? p : S - 1;
      }
      __syncthreads();
      pick = s_pick;
    } else {
      pick = draw_index(u[k], S);
    }
    // center k = sample `pick`: lane e < G copies element e = tau*c + i
    if (tid < G) {
      const int tau = tid / C, i = tid % C;
      const double v = bf2d(bk.base[((size_t)tau * S + pick) * a.H * a.d + i]);
      cen[tid] = v;
      centers[(size_t)k * G + tid] = v;
    }
    __syncthreads();
    if (k + 1 == kCodes) break;
    // D^2 against the new center, squares added in element order
    if constexpr (REG) {
      // opaque to the compiler: keeps the float64 conversions inside the loop over draws
      // (hoisted, they would need NPER * G float64 registers)
#pragma unroll
      for (int j = 0; j < NPER; ++j)
#pragma unroll
        for (int i = 0; i < G / 2; ++i) asm volatile("" : "+v"(xr[j][i]));
      double dn[NPER];
#pragma unroll
      for (int j = 0; j < NPER; ++j) dn[j] = 0.0;
#pragma unroll
      for (int e = 0; e < G; ++e) {
        const double c = cen[e];
#pragma unroll
        for (int j = 0; j < NPER; ++j) {
          const double df = __dsub_rn(packed_elem(xr[j], e), c);
          dn[j] = __dadd_rn(dn[j], __dmul_rn(df, df));
        }
      }
#pragma unroll
      for (int j = 0; j < NPER; ++j)
        if (k == 0 || dn[j] < d2[j]) d2[j] = dn[j];
    } else {
#pragma unroll
      for (int j = 0; j < NPER; ++j) {
        const int s = j * kSeedThreads + tid;
        if (s < S) {
          uint32_t xw[G / 2];
          load_packed<G, C>(a, bk, s, xw);
          double dn = 0.0;
#pragma unroll
          for (int e = 0; e < G; ++e) {
            const double df = __dsub_rn(packed_elem(xw, e), cen[e]);
            dn = __dadd_rn(dn, __dmul_rn(df, df));
          }
          if (k == 0 || dn < d2[j]) d2[j] = dn;
        }
        asm volatile("" ::: "memory");   // one sample's loads in flight at a time (no spills)
      }
    }
    publish();
  }
}

// ------------------------------------------------------------------ seeding, large S
// Above kMaxKmeansSamplesLds samples a book's D^2 live in the workspace (one float64 per
// sample) instead of registers and LDS.  Each draw streams the terms w_s D^2_s through
// a two-chunk LDS ring: waves 1..7 load and form chunk i + 1 while lane 0 of wave 0
// adds chunk i in sample order (the same chain of float64 adds as the kernel above,
// only batch-end sums kept), then the workgroup finds the crossing batch, lane 0 redoes
// its sums from the workspace, and every thread refreshes the D^2 of its samples
// against the new center, re-reading their joint vectors.
constexpr int kWalkChunk = 2048;   // terms per LDS chunk (a multiple of 2 kChain)

constexpr size_t seed_ws_lds_bytes(int S) {
  return ((size_t)2 * kWalkChunk + (size_t)((S + 2 * kChain - 1) / (2 * kChain) * (2 * kChain)) / kChain) *
         sizeof(double);
}

template <int G, int C>
__global__ __launch_bounds__(kSeedThreads) void seed_kernel_ws(KmeansArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int S = a.S;
  const int Sp = (S + 2 * kChain - 1) / (2 * kChain) * (2 * kChain);
  double* ring = (double*)smem;                 // [2][kWalkChunk] terms of the walk
  double* ckpt = ring + 2 * kWalkChunk;         // [Sp / kChain] running sum at each batch end
  __shared__ double cen[G];
  __shared__ double s_total;
  __shared__ int s_first[kSeedWaves], s_pick;
  const int book = book_of_block(blockIdx.x, a.n_books);
  const Book bk = book_at<G, C>(a, book);
  const double* u = a.draws + (size_t)book * kCodes;
  double* centers = a.centers + (size_t)book * kCodes * G;
  double* d2 = a.d2 + (size_t)book * Sp;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunk = (Sp + kWalkChunk - 1) / kWalkChunk;

  auto term_of = [&](int s) -> double {
    if (s >= S) return 0.0;
    const double dd = d2[s];
    return a.weights ? __dmul_rn(a.weights[bk.wbase + (size_t)s * bk.wstride], dd) : dd;
  };
  // chunk i into ring slot i & 1, by threads first .. kSeedThreads - 1
  auto load_chunk = [&](int i, int first) {
    double* dst = ring + (i & 1) * kWalkChunk;
    const int c0 = i * kWalkChunk, n = min(kWalkChunk, Sp - c0);
    for (int j = tid - first; j < n; j += kSeedThreads - first) dst[j] = term_of(c0 + j);
  };

  for (int s = tid; s < Sp; s += kSeedThreads) d2[s] = 1.0;   // draw 0 takes every distance as 1
  __syncthreads();
  for (int k = 0; k < kCodes; ++k) {
    load_chunk(0, 0);
    __syncthreads();
    double acc = 0.0;
    for (int i = 0; i < nchunk; ++i) {
      if (wave == 0) {
        if (lane == 0) {
          // running sum in sample order, two register batches alternating as above
          const double* run = ring + (i & 1) * kWalkChunk;
          const int n = min(kWalkChunk, Sp - i * kWalkChunk);
          double ba[kChain], bb[kChain];
#pragma unroll
          for (int j = 0; j < kChain; ++j) ba[j] = run[j];
          for (int s0 = 0; s0 < n; s0 += 2 * kChain) {
            const int nb = s0 + kChain;
#pragma unroll
            for (int j = 0; j < kChain; ++j) bb[j] = run[nb + j];
            asm volatile("" ::: "memory");
#pragma unroll
            for (int j = 0; j < kChain; ++j) acc = __dadd_rn(acc, ba[j]);
            ckpt[(i * kWalkChunk + s0) / kChain] = acc;
            const int na = s0 + 2 * kChain < n ? s0 + 2 * kChain : 0;
#pragma unroll
            for (int j = 0; j < kChain; ++j) ba[j] = run[na + j];
            asm volatile("" ::: "memory");
#pragma unroll
            for (int j = 0; j < kChain; ++j) acc = __dadd_rn(acc, bb[j]);
            ckpt[(i * kWalkChunk + nb) / kChain] = acc;
          }
        }
      } else if (i + 1 < nchunk) {
        load_chunk(i + 1, 64);
      }
      __syncthreads();
    }
    if (tid == 0) s_total = acc;
    __syncthreads();
    const double total = s_total;
    int pick;
    if (total > 0.0) {
      const double target = __dmul_rn(u[k], total);
      int fb = INT32_MAX;
      for (int b = tid; b < Sp / kChain; b += kSeedThreads)
        if (ckpt[b] > target) {
          fb = b;
          break;
        }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) fb = min(fb, __shfl_xor(fb, off));
      if (lane == 0) s_first[wave] = fb;
      __syncthreads();
      if (tid == 0) {
        int f = INT32_MAX;
#pragma unroll
        for (int v = 0; v < kSeedWaves; ++v) f = min(f, s_first[v]);
        int p;
        if (f != INT32_MAX) {
          // redo that batch's sums from the previous batch's last one: same values as the chain
          double acc2 = f > 0 ? ckpt[f - 1] : 0.0;
          p = f * kChain + kChain - 1;
          for (int j = 0; j < kChain; ++j) {
            acc2 = __dadd_rn(acc2, term_of(f * kChain + j));
            if (acc2 > target) {
              p = f * kChain + j;
              break;
            }
          }
        } else {
          // rounding left no crossing: the last sample with a positive term (one exists,
          // since the total is positive)
          p = 0;
          for (int s = S - 1; s >= 0; --s)
            if (term_of(s) > 0.0) {
              p = s;
              break;
            }
        }
        s_pick = p < S ? p : S - 1;
      }
      __syncthreads();
      pick = s_pick;
    } else {
      pick = draw_index(u[k], S);
    }
    if (tid < G) {
      const int tau = tid / C, i = tid % C;
      const double v = bf2d(bk.base[((size_t)tau * S + pick) * a.H * a.d + i]);
      cen[tid] = v;
      centers[(size_t)k * G + tid] = v;
    }
    __syncthreads();
    if (k + 1 == kCodes) break;
    // D^2 against the new center, squares added in element order
    for (int s = tid; s < S; s += kSeedThreads) {
      uint32_t xw[G / 2];
      load_packed<G, C>(a, bk, s, xw);
      double dn = 0.0;
#pragma unroll
      for (int e = 0; e < G; ++e) {
        const double df = __dsub_rn(packed_elem(xw, e), cen[e]);
        dn = __dadd_rn(dn, __dmul_rn(df, df));
      }
      if (k == 0 || dn < d2[s]) d2[s] = dn;
    }
    __syncthreads();
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
constexpr size_t update_lds_bytes(int G, int S) {
  // staged joint vectors, staged weights, member lists, assignments
  return (size_t)kStage * G * 2 + (size_t)kStage * 8 + ((size_t)S * 2 + 15) / 16 * 16 + (size_t)S;
}

template <int G, int C>
__global__ __launch_bounds__(kKmThreads) void update_kernel(KmeansArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int TC = G / C;
  const int S = a.S;
  uint16_t* xs = (uint16_t*)smem;                                // [kStage][G]
  double* wst = (double*)(xs + kStage * G);                      // [kStage]
  uint16_t* list = (uint16_t*)(wst + kStage);                    // [S] members by cluster
  uint8_t* asg = (uint8_t*)list + ((size_t)S * 2 + 15) / 16 * 16;  // [S]
  __shared__ int cnt[kCodes], cursor[kCodes];
  const int book = book_of_block(blockIdx.x, a.n_books);
  const Book bk = book_at<G, C>(a, book);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  static_assert(kKmThreads == kCodes, "one lane per cluster");

  cnt[tid] = 0;
  __syncthreads();
  for (int s = tid; s < S; s += kKmThreads) {
    const uint8_t c = a.assign[bk.wbase + (size_t)s * bk.wstride];
    asg[s] = c;
    atomicAdd(&cnt[c], 1);
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive prefix of the counts: lane l holds clusters 4l .. 4l+3
    const int c0 = cnt[4 * lane], c1 = cnt[4 * lane + 1], c2 = cnt[4 * lane + 2], c3 = cnt[4 * lane + 3];
    const int loc = c0 + c1 + c2 + c3;
    int incl = loc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    const int base = incl - loc;
    cursor[4 * lane] = base;
    cursor[4 * lane + 1] = base + c0;
    cursor[4 * lane + 2] = base + c0 + c1;
    cursor[4 * lane + 3] = base + c0 + c1 + c2;
  }
  __syncthreads();
  const int begin = cursor[tid], end = begin + cnt[tid];
  __syncthreads();
  if (wave == 0) {
    // stable placement, 64 samples at a time in sample order: a lane's slot is its
    // cluster's cursor plus the number of lower lanes with the same cluster
    const uint64_t below = (1ull << lane) - 1ull;
    for (int s0 = 0; s0 < S; s0 += 64) {
      const int s = s0 + lane;
      const bool valid = s < S;
      const int c = valid ? asg[s] : 0;
      uint64_t same = __ballot(valid);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const bool bit = (c >> b) & 1;
        const uint64_t ones = __ballot(valid && bit);
        same &= bit ? ones : ~ones;
      }
      if (valid) {
        const int rank = __popcll(same & below);
        const int pos = cursor[c] + rank;
        list[pos] = (uint16_t)s;
        if (rank == (int)__popcll(same) - 1) cursor[c] = pos + 1;
      }
    }
  }
  __syncthreads();

  double acc[G];
#pragma unroll
  for (int e = 0; e < G; ++e) acc[e] = 0.0;
  double wsum = 0.0;
  int p = begin;
  const size_t tstride = (size_t)S * a.H * a.d;
  for (int c0 = 0; c0 < S; c0 += kStage) {
    const int n = min(kStage, S - c0);
    // stage the joint vectors of samples c0 .. c0+n-1, in pieces of 4 elements
    for (int u = tid; u < n * TC * (C / 4); u += kKmThreads) {
      const int piece = u % (C / 4), tau = (u / (C / 4)) % TC, j = u / (TC * (C / 4));
      const uint2 v = *(const uint2*)(bk.base + tau * tstride + (size_t)(c0 + j) * a.H * a.d + piece * 4);
      *(uint2*)(xs + j * G + tau * C + piece * 4) = v;
    }
    if (a.weights)
      for (int j = tid; j < n; j += kKmThreads) wst[j] = a.weights[bk.wbase + (size_t)(c0 + j) * bk.wstride];
    __syncthreads();
    for (; p < end; ++p) {
      const int s = list[p];
      if (s >= c0 + n) break;
      const uint16_t* xr = xs + (s - c0) * G;
      if (a.weights) {
        const double w = wst[s - c0];
#pragma unroll
        for (int e = 0; e < G; ++e) acc[e] = __dadd_rn(acc[e], __dmul_rn(w, bf2d(xr[e])));
        wsum = __dadd_rn(wsum, w);
      } else {
#pragma unroll
        for (int e = 0; e < G; ++e) acc[e] = __dadd_rn(acc[e], bf2d(xr[e]));
        wsum = __dadd_rn(wsum, 1.0);
      }
    }
    __syncthreads();
  }
  if (wsum != 0.0) {
    double* c = a.centers + ((size_t)book * kCodes + tid) * G;
#pragma unroll
    for (int e = 0; e < G; ++e) c[e] = __ddiv_rn(acc[e], wsum);
  }
}

template <int G, int C>
hipError_t build_t(const KmeansArgs& a, hipStream_t s) {
  const int Sp = (a.S + 2 * kChain - 1) / (2 * kChain) * (2 * kChain);
  const size_t seed_lds = a.S <= kMaxKmeansSamplesLds ? (size_t)(Sp + Sp / kChain) * sizeof(double) : 0;
  const size_t upd_lds = update_lds_bytes(G, a.S);
  static std::atomic<uint64_t> attr_set{0};
  hipError_t ea = once_per_device(attr_set, [&] {
    hipError_t e = hipFuncSetAttribute((const void*)seed_kernel<G, C, kSeedMaxPer, false>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)((kMaxKmeansSamplesLds + kMaxKmeansSamplesLds / kChain) * sizeof(double)));
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)seed_kernel_ws<G, C>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)seed_ws_lds_bytes(kMaxKmeansSamples));
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute((const void*)update_kernel<G, C>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)update_lds_bytes(G, kMaxKmeansSamples));
  });
  if (ea != hipSuccess) return ea;
  if (a.S <= kSeedRegPer * kSeedThreads)
    hipLaunchKernelGGL((seed_kernel<G, C, kSeedRegPer, true>), dim3(a.n_books), dim3(kSeedThreads), seed_lds, s, a);
  else if (a.S <= kMaxKmeansSamplesLds)
    hipLaunchKernelGGL((seed_kernel<G, C, kSeedMaxPer, false>), dim3(a.n_books), dim3(kSeedThreads), seed_lds, s,
                       a);
  else if (a.d2)
    hipLaunchKernelGGL((seed_kernel_ws<G, C>), dim3(a.n_books), dim3(kSeedThreads), seed_ws_lds_bytes(a.S), s, a);
  else
    return hipErrorInvalidValue;
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
    hipLaunchKernelGGL((update_kernel<G, C>), dim3(a.n_books), dim3(kKmThreads), upd_lds, s, a);
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
