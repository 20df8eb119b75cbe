// LoopVQ paged cache manager for gfx950: page bookkeeping of the decode loop on the device.
//
// What it keeps (LoopVQ summary, onedev.kr/papers/1681, section "전제와 한계"): the
// cache lives in 8-token pages; the sink tokens and the recent window stay bf16; once a
// token's forward pass is done and the recent window holds n_recent + 8 tokens, its
// oldest page is quantised across all layers and loop steps and leaves the window.
// With q_end the first bf16 token after the coded run, the state keeps, for every
// sequence b and at every step boundary,
//     q_end[b] = 8 * floor((seq_len[b] - n_recent) / 8)   (0 when negative),
// logical pages [0, q_end/8) in coded pages (page_table), logical page 0 also in a bf16
// page (bf16_table entry 0, the sink), and logical pages q_end/8 .. in bf16 pages
// (bf16_table entries 1 ..).  Page ids are shared by every layer: a layer's pools are
// indexed by the same ids.
//
// Design (MI355X): the bookkeeping kernels are one wave each.  Lanes take 64 sequences
// at a time; an allocation takes ids from the top of a free-page stack in lane order
// (ballot + popcount ranks), so ids are handed out deterministically, lowest first,
// sequences in index order, with no atomics.  Each kernel reads the stack counts once
// and writes them back at its end; kernels on one stream run in order, so no other
// synchronisation is needed.  Token copies (prefill bf16 parts, the decode append) are
// 16-byte vector copies, one thread per 8 channels.
#include "lvq_internal.h"

#include <cstdint>

namespace lvq {
namespace {

constexpr int kErrIndexPool = 1, kErrBf16Pool = 2, kErrMaxPages = 4, kErrBf16Row = 8;

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (1ull << lane) - 1ull; }

// Pops one id per lane with `need`, in lane order, from stack[0 .. count): lane of rank r
// gets stack[count - 1 - r].  Wave-uniform call; `count` is the caller's register copy.
__device__ __forceinline__ int pop_ranked(bool need, const int32_t* stack, int& count, int lane,
                                          int& err, int errbit) {
  const uint64_t m = __ballot(need);
  const int rank = __popcll(m & lanes_below(lane));
  int id = -1;
  if (need) {
    if (rank < count) id = stack[count - 1 - rank];
    else err |= errbit;
  }
  const int want = __popcll(m);
  count -= want < count ? want : count;
  return id;
}

// Pushes one id per lane with `give`, in lane order.
__device__ __forceinline__ void push_ranked(bool give, int id, int32_t* stack, int& count, int cap,
                                            int lane) {
  const uint64_t m = __ballot(give);
  const int rank = __popcll(m & lanes_below(lane));
  if (give && count + rank < cap) stack[count + rank] = id;
  count += __popcll(m);
  if (count > cap) count = cap;
}

__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v |= __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ int q_end_rule(int L, int n_recent) {
  const int r = L - n_recent;
  return r > 0 ? (r / kPage) * kPage : 0;
}

__global__ void cache_init_kernel(CacheArgs c) {
  const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x, st = (size_t)gridDim.x * blockDim.x;
  for (size_t i = i0; i < (size_t)c.n_index_pages; i += st) c.index_free[i] = c.n_index_pages - 1 - (int)i;
  for (size_t i = i0; i < (size_t)c.n_bf16_pages; i += st) c.bf16_free[i] = c.n_bf16_pages - 1 - (int)i;
  for (size_t i = i0; i < (size_t)c.B * c.max_pages; i += st) c.page_table[i] = -1;
  for (size_t i = i0; i < (size_t)c.B * c.bf16_row; i += st) c.bf16_table[i] = -1;
  for (size_t i = i0; i < (size_t)c.B; i += st) {
    c.seq_len[i] = 0;
    c.q_end[i] = 0;
    c.re_src[i] = -1;
    c.re_dst[i] = -1;
  }
  if (i0 == 0) {
    c.counters[0] = c.n_index_pages;
    c.counters[1] = c.n_bf16_pages;
    c.counters[2] = 0;
    c.counters[3] = 0;
  }
}

// Prefill: sequences with seq_len == 0 and lengths[b] > 0 get their pages.  One wave,
// sequences in order, the pages of one sequence spread over the lanes.
__global__ void cache_prefill_kernel(CacheArgs c, const int32_t* lengths) {
  const int lane = threadIdx.x;
  int ni = c.counters[0], nb = c.counters[1], err = 0;
  for (int b = 0; b < c.B; ++b) {
    const int L = lengths[b];
    if (c.seq_len[b] != 0 || L <= 0) continue;
    const int qe = q_end_rule(L, c.n_recent);
    const int nq = qe / kPage, npg = (L + kPage - 1) / kPage, nrec = npg - nq;
    const int nbf = nrec + (nq > 0 ? 1 : 0);
    if (npg > c.max_pages) { err |= kErrMaxPages; continue; }
    if (1 + nrec > c.bf16_row) { err |= kErrBf16Row; continue; }
    if (nq > ni) { err |= kErrIndexPool; continue; }
    if (nbf > nb) { err |= kErrBf16Pool; continue; }
    int32_t* pt = c.page_table + (size_t)b * c.max_pages;
    int32_t* bt = c.bf16_table + (size_t)b * c.bf16_row;
    for (int j = lane; j < nq; j += 64) pt[j] = c.index_free[ni - 1 - j];
    // bf16 ids in order: logical page 0 first (the sink copy; also the first recent page
    // when nothing is coded), then the recent pages
    for (int j = lane; j < nbf; j += 64) {
      const int id = c.bf16_free[nb - 1 - j];
      if (nq > 0) {
        if (j == 0) bt[0] = id;
        else bt[j] = id;                       // recent page nq + j - 1 -> entry j
      } else {
        bt[1 + j] = id;                        // recent page j -> entry 1 + j
        if (j == 0) bt[0] = id;
      }
    }
    ni -= nq;
    nb -= nbf;
    if (lane == 0) {
      c.seq_len[b] = L;
      c.q_end[b] = qe;
    }
  }
  err = wave_or(err);
  if (lane == 0) {
    c.counters[0] = ni;
    c.counters[1] = nb;
    c.counters[2] |= err;
  }
}

// A new token for every live sequence: a bf16 page when it starts a page, seq_len += 1.
__global__ void cache_begin_kernel(CacheArgs c) {
  const int lane = threadIdx.x;
  int nb = c.counters[1], err = 0;
  for (int b0 = 0; b0 < c.B; b0 += 64) {
    const int b = b0 + lane;
    const bool live = b < c.B && c.seq_len[b] > 0;
    const int L = live ? c.seq_len[b] : 0;
    const int qe = live ? c.q_end[b] : 0;
    const int ri = 1 + L / kPage - qe / kPage;           // bf16_table entry of the new token's page
    bool need = live && L % kPage == 0;
    if (need && L / kPage >= c.max_pages) { err |= kErrMaxPages; need = false; }
    if (need && ri >= c.bf16_row) { err |= kErrBf16Row; need = false; }
    const int id = pop_ranked(need, c.bf16_free, nb, lane, err, kErrBf16Pool);
    if (need) c.bf16_table[(size_t)b * c.bf16_row + ri] = id;
    if (live) c.seq_len[b] = L + 1;
  }
  err = wave_or(err);
  if (lane == 0) {
    c.counters[1] = nb;
    c.counters[2] |= err;
  }
}

// After the token's forward pass: sequences whose window reached n_recent + 8 get a
// coded page for their oldest recent page (re_src -> re_dst); the others get -1.
__global__ void cache_end_kernel(CacheArgs c) {
  const int lane = threadIdx.x;
  int ni = c.counters[0], err = 0;
  for (int b0 = 0; b0 < c.B; b0 += 64) {
    const int b = b0 + lane;
    const bool live = b < c.B && c.seq_len[b] > 0;
    const int L = live ? c.seq_len[b] : 0;
    const int qe = live ? c.q_end[b] : 0;
    const bool need = live && L - qe >= c.n_recent + kPage;
    const int id = pop_ranked(need, c.index_free, ni, lane, err, kErrIndexPool);
    if (b < c.B) {
      const bool go = need && id >= 0;
      c.re_src[b] = go ? c.bf16_table[(size_t)b * c.bf16_row + 1] : -1;
      c.re_dst[b] = go ? id : -1;
    }
  }
  err = wave_or(err);
  if (lane == 0) {
    c.counters[0] = ni;
    c.counters[2] |= err;
  }
}

// Applies the re-encodes: the coded page joins the page table, the bf16 page leaves the
// window (and returns to the pool unless it is logical page 0, the sink copy).
__global__ void cache_commit_kernel(CacheArgs c) {
  const int lane = threadIdx.x;
  int nb = c.counters[1];
  for (int b0 = 0; b0 < c.B; b0 += 64) {
    const int b = b0 + lane;
    const bool go = b < c.B && c.re_dst[b] >= 0;
    const int qe = go ? c.q_end[b] : 0;
    const int src = go ? c.re_src[b] : -1;
    const bool give = go && qe > 0 && src >= 0;
    push_ranked(give, src, c.bf16_free, nb, c.n_bf16_pages, lane);
    if (go) {
      c.page_table[(size_t)b * c.max_pages + qe / kPage] = c.re_dst[b];
      int32_t* bt = c.bf16_table + (size_t)b * c.bf16_row;
      for (int j = 1; j + 1 < c.bf16_row; ++j) bt[j] = bt[j + 1];
      bt[c.bf16_row - 1] = -1;
      c.q_end[b] = qe + kPage;
    }
    if (b < c.B) {
      c.re_src[b] = -1;
      c.re_dst[b] = -1;
    }
  }
  if (lane == 0) c.counters[1] = nb;
}

// Returns every page of the sequences with mask[b] != 0 and empties them.
__global__ void cache_release_kernel(CacheArgs c, const int32_t* mask) {
  const int lane = threadIdx.x;
  int ni = c.counters[0], nb = c.counters[1];
  for (int b = 0; b < c.B; ++b) {
    if (!mask[b] || c.seq_len[b] <= 0) continue;
    const int L = c.seq_len[b], qe = c.q_end[b];
    int32_t* pt = c.page_table + (size_t)b * c.max_pages;
    int32_t* bt = c.bf16_table + (size_t)b * c.bf16_row;
    const int nq = min(qe / kPage, c.max_pages);
    for (int j0 = 0; j0 < nq; j0 += 64) {
      const int j = j0 + lane;
      const int id = j < nq ? pt[j] : -1;
      push_ranked(id >= 0, id, c.index_free, ni, c.n_index_pages, lane);
    }
    // bf16: entry 0, then recent entries that are not the same page as entry 0
    for (int j0 = 0; j0 < c.bf16_row; j0 += 64) {
      const int j = j0 + lane;
      int id = j < c.bf16_row ? bt[j] : -1;
      if (j >= 1 && id == bt[0]) id = -1;
      push_ranked(id >= 0, id, c.bf16_free, nb, c.n_bf16_pages, lane);
    }
    for (int j = lane; j < c.max_pages; j += 64) pt[j] = -1;
    for (int j = lane; j < c.bf16_row; j += 64) bt[j] = -1;
    if (lane == 0) {
      c.seq_len[b] = 0;
      c.q_end[b] = 0;
      c.re_src[b] = -1;
      c.re_dst[b] = -1;
    }
    (void)L;
  }
  if (lane == 0) {
    c.counters[0] = ni;
    c.counters[1] = nb;
  }
}

__device__ __forceinline__ uint4* bf16_slot(const CacheArgs& c, uint16_t* pool, int page, int t, int T, int H,
                                            int h, int kv, int slot, int d) {
  return (uint4*)(pool + (((((size_t)page * T + t) * H + h) * 2 + kv) * kPage + slot) * d);
}

// Tokens first .. first+n-1 of sequence b (k, v: [T][n][H][d]) into the bf16 pages that
// hold them: logical page 0 (entry 0) and the recent window (entries 1 ..).
__global__ void cache_store_kernel(CacheArgs c, TokenCopy tc, int b, int first, int n) {
  const int d8 = tc.d / 8;
  const size_t per_tok = (size_t)tc.T * tc.H * 2 * d8;
  const size_t total = per_tok * n;
  const int L = c.seq_len[b], qe = c.q_end[b];
  const int32_t* bt = c.bf16_table + (size_t)b * c.bf16_row;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (size_t)gridDim.x * blockDim.x) {
    const int ch = (int)(u % d8);
    const int kv = (int)((u / d8) % 2);
    const int h = (int)((u / (d8 * 2)) % tc.H);
    const int t = (int)((u / ((size_t)d8 * 2 * tc.H)) % tc.T);
    const int i = (int)(u / per_tok);
    const int p = first + i;
    if (p >= L) continue;
    const uint16_t* src = (kv ? tc.v : tc.k) + (((size_t)t * n + i) * tc.H + h) * tc.d;
    const uint4 val = ((const uint4*)src)[ch];
    int page0 = -1, pager = -1;
    if (p < kPage) page0 = bt[0];
    if (p >= qe) {
      const int ri = 1 + p / kPage - qe / kPage;
      if (ri < c.bf16_row) pager = bt[ri];
    }
    if (pager == page0) page0 = -1;
    if (page0 >= 0 && page0 < c.n_bf16_pages)
      bf16_slot(c, tc.pool, page0, t, tc.T, tc.H, h, kv, p % kPage, tc.d)[ch] = val;
    if (pager >= 0 && pager < c.n_bf16_pages)
      bf16_slot(c, tc.pool, pager, t, tc.T, tc.H, h, kv, p % kPage, tc.d)[ch] = val;
  }
}

// The newest token (position seq_len - 1) of every live sequence, loop steps
// t0 .. t0+n_steps-1 (k, v: [n_steps][B][H][d]).
__global__ void cache_append_kernel(CacheArgs c, TokenCopy tc, int t0, int n_steps) {
  const int d8 = tc.d / 8;
  const size_t per_seq = (size_t)n_steps * tc.H * 2 * d8;
  const size_t total = per_seq * c.B;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (size_t)gridDim.x * blockDim.x) {
    const int ch = (int)(u % d8);
    const int kv = (int)((u / d8) % 2);
    const int h = (int)((u / (d8 * 2)) % tc.H);
    const int s = (int)((u / ((size_t)d8 * 2 * tc.H)) % n_steps);
    const int b = (int)(u / per_seq);
    const int L = c.seq_len[b];
    if (L <= 0) continue;
    const int p = L - 1, qe = c.q_end[b];
    const int ri = 1 + p / kPage - qe / kPage;
    if (ri < 1 || ri >= c.bf16_row) continue;
    const int page = c.bf16_table[(size_t)b * c.bf16_row + ri];
    if (page < 0 || page >= c.n_bf16_pages) continue;
    const uint16_t* src = (kv ? tc.v : tc.k) + (((size_t)s * c.B + b) * tc.H + h) * tc.d;
    bf16_slot(c, tc.pool, page, t0 + s, tc.T, tc.H, h, kv, p % kPage, tc.d)[ch] = ((const uint4*)src)[ch];
  }
}

int copy_grid(size_t units) {
  const size_t g = (units + 255) / 256;
  return (int)(g < 4096 ? (g > 0 ? g : 1) : 4096);
}

}  // namespace

hipError_t launch_cache_init(const CacheArgs& c, hipStream_t s) {
  size_t n = (size_t)c.B * c.max_pages;
  if ((size_t)c.n_index_pages > n) n = c.n_index_pages;
  if ((size_t)c.n_bf16_pages > n) n = c.n_bf16_pages;
  if ((size_t)c.B * c.bf16_row > n) n = (size_t)c.B * c.bf16_row;
  hipLaunchKernelGGL(cache_init_kernel, dim3(copy_grid(n)), dim3(256), 0, s, c);
  return hipGetLastError();
}

hipError_t launch_cache_prefill(const CacheArgs& c, const int32_t* lengths, hipStream_t s) {
  hipLaunchKernelGGL(cache_prefill_kernel, dim3(1), dim3(64), 0, s, c, lengths);
  return hipGetLastError();
}

hipError_t launch_cache_step(const CacheArgs& c, int which, hipStream_t s) {
  if (which == 0) hipLaunchKernelGGL(cache_begin_kernel, dim3(1), dim3(64), 0, s, c);
  else if (which == 1) hipLaunchKernelGGL(cache_end_kernel, dim3(1), dim3(64), 0, s, c);
  else hipLaunchKernelGGL(cache_commit_kernel, dim3(1), dim3(64), 0, s, c);
  return hipGetLastError();
}

hipError_t launch_cache_release(const CacheArgs& c, const int32_t* mask, hipStream_t s) {
  hipLaunchKernelGGL(cache_release_kernel, dim3(1), dim3(64), 0, s, c, mask);
  return hipGetLastError();
}

hipError_t launch_cache_store(const CacheArgs& c, const TokenCopy& tc, int b, int first, int n, hipStream_t s) {
  const size_t units = (size_t)n * tc.T * tc.H * 2 * (tc.d / 8);
  hipLaunchKernelGGL(cache_store_kernel, dim3(copy_grid(units)), dim3(256), 0, s, c, tc, b, first, n);
  return hipGetLastError();
}

hipError_t launch_cache_append(const CacheArgs& c, const TokenCopy& tc, int t0, int n_steps, hipStream_t s) {
  const size_t units = (size_t)c.B * n_steps * tc.H * 2 * (tc.d / 8);
  hipLaunchKernelGGL(cache_append_kernel, dim3(copy_grid(units)), dim3(256), 0, s, c, tc, t0, n_steps);
  return hipGetLastError();
}

}  // namespace lvq
