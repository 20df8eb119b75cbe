// Paged decode attention over the LoopVQ cache, gfx950.
//
// What it computes (LoopVQ summary, onedev.kr/papers/1681, section "전제와
// 한계"; rit.work article, section "Когда LoopVQ меняет план развёртывания"):
// at loop step t, query q of sequence b attends over all L_b cached tokens.
// Coded tokens are rebuilt from their index rows of loop block t/Tc: group g of
// the key (value) is the step-(t % Tc) c-channel share of the chosen K (V)
// codeword, and only that slice of the codebooks is read.  Sink and recent
// tokens are bf16.  Keys are stored before RoPE and rotated here (summary,
// section "무엇과 다른가").  The coded range is split Flash-Decoding style;
// partial (max, sum, unnormalised output) triples are merged by log-sum-exp and
// combined with the bf16 part.
//
// Design (MI355X; MHA decode is bound by per-token VALU and LDS work, not HBM):
//  * Workgroup = 8 waves (2 per SIMD) on one (sequence, query head); each wave
//    owns one chunk of coded pages.  The step-t K and V slices of the head
//    (2 x 256 codes x d channels, 128 KB at d = 128) are staged once per
//    workgroup in LDS as float16, which holds the bf16 codewords exactly.
//  * A tile is 16 positions (2 pages); four lanes share a token: lane quarter
//    qt owns channel pairs [qt*d/8, (qt+1)*d/8) of the score and output channels
//    [qt*d/4, (qt+1)*d/4) of the value sum.  Keys and values are gathered from
//    LDS (16-byte reads), the value sum is accumulated in registers.
//  * RoPE after dequantisation without per-token trigonometry: position
//    16a + o has phase E(16a) * E(o); the lane folds E(o) and the query once per
//    chunk into coefficients F, G, so per channel pair j the score gets
//    (c0 F_j + s0 G_j) k_j + (c0 G_j - s0 F_j) k_{j+d/2} with (c0, s0) = E(16a)
//    read from a per-tile LDS row: six float32 operations, the key read by
//    v_fma_mix straight from float16.
//  * Index rows (only the bytes a lane needs) and tile phases of the next batch
//    of 4 tiles are loaded while the current batch computes.
//  * Scores are kept in log2 units (scale * log2 e folded into the query); a
//    running maximum is kept lazily (rescale only when a score passes it by
//    more than 8 in log2 units).
//  * The bf16 sink + recent tokens of every (b, query head) run as extra
//    workgroups placed first in the grid; their partial is the last split.
#include "lvq_internal.h"

namespace lvq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescale = 8.0f;   // lazy-max slack, log2 units
constexpr int kNW = 8;             // waves per workgroup
constexpr int kTile = 16;          // positions per tile (RoPE table granularity)
constexpr int kPtBatch = 128;      // page ids staged in LDS per wave at a time
constexpr int kBfTok = 32;         // bf16 tokens per batch

// LDS bytes per wave of the bf16 part: K and V rows of a batch, weights, query, row addresses
template <int D>
constexpr size_t kBf16Scratch = 2 * kBfTok * (2 * D + 16) + kBfTok * 4 + D * 4 + kBfTok * 8;

template <int D>
constexpr size_t lds_bytes() {
  const size_t coded = (size_t)2 * kCodes * D * 2 + (size_t)kNW * (D * 4 + 2 * D * 4 + kPtBatch * 4);
  const size_t bf = (size_t)kNW * kBf16Scratch<D>;
  return coded > bf ? coded : bf;
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
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

// Stage the step-tau [256][c] slices of all groups of book (beta, kv, h) into LDS as float16.
template <int D, int C>
__device__ __forceinline__ void stage_slice(const AttnArgs& a, int beta, int kv, int h, int tau,
                                            _Float16* dst) {
  constexpr int NG = D / C;
  const uint16_t* src = a.codebooks + ((((size_t)beta * 2 + kv) * a.H + h) * NG) * ((size_t)a.Tc * kCodes * C);
  for (int e = threadIdx.x * 8; e < kCodes * D; e += kNW * 64 * 8) {
    const int g = e / (kCodes * C), rem = e % (kCodes * C);
    const u16x8 v = *(const u16x8*)(src + ((size_t)g * a.Tc + tau) * kCodes * C + rem);
    f16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (_Float16)bf2f(v[i]);
    *(f16x8*)(dst + e) = o;
  }
}

// ------------------------------------------------------------------ bf16 part
// One wave per (b, hq): the sink tokens [0, n_sink) and the recent tokens
// [max(q_end, n_sink), L), 32 at a time.  The K and V rows of a batch are
// copied into LDS with all loads in flight at once; lane i < 32 scores token i
// (RoPE on the key from the two-part phase table), then each lane accumulates
// one channel pair of the output over the batch.
template <int D>
__device__ void bf16_part(const AttnArgs& a, const float* __restrict__ rope, int item, int lane,
                          unsigned char* scratch) {
  constexpr int HALF = D / 2;
  constexpr int ROWB = 2 * D + 16;        // padded LDS row (bytes): spreads lanes over banks
  const int b = item / a.Hq, hq = item % a.Hq;
  if (b >= a.B) return;
  const int h = hq / (a.Hq / a.H);
  const int L = min(a.seq_len[b], a.max_seq_len);
  const int qe = min(a.q_end[b] & ~7, L);
  const int ns = min(a.n_sink, L);
  const int r0 = max(qe, a.n_sink);
  const int n_tok = ns + max(0, L - r0);
  unsigned char* krow = scratch;                         // [kBfTok][ROWB]
  unsigned char* vrow = scratch + kBfTok * ROWB;         // [kBfTok][ROWB]
  float* wl = (float*)(scratch + 2 * kBfTok * ROWB);     // [kBfTok] weights
  float* qp = wl + kBfTok;                               // [D] rotated query (pairs)
  const uint16_t** src = (const uint16_t**)(qp + D);     // [kBfTok] K row address per token

  // rotated query, pairs (j, j + d/2) interleaved, log2 units
  if (lane < HALF) {
    const int pq = min(max(a.pos[b], 0), a.rope_tiles * kTile - 1);
    const uint16_t* qv = a.q + ((size_t)b * a.Hq + hq) * D;
    const float2 cs = phase(rope, a.rope_tiles, D, pq, lane);
    const float x = bf2f(qv[lane]), y = bf2f(qv[lane + HALF]);
    qp[2 * lane] = (x * cs.x - y * cs.y) * a.scale_log2e;
    qp[2 * lane + 1] = (y * cs.x + x * cs.y) * a.scale_log2e;
  }
  float m = -__builtin_inff(), l = 0.f, oa = 0.f, ob = 0.f;   // oa, ob: channels j, j + d/2 (j = lane)
  for (int i0 = 0; i0 < n_tok; i0 += kBfTok) {
    // token of this lane, its position and its K row in the page pool
    const int i = i0 + lane;
    const bool ok = lane < kBfTok && i < n_tok;
    const int p = ok ? (i < ns ? i : r0 + (i - ns)) : 0;
    const uint16_t* kr = nullptr;
    if (ok) {
      const int slot = (p < ns) ? 0 : 1 + (p >> 3) - (qe >> 3);
      const int pg = slot < a.bf16_row ? a.bf16_table[(size_t)b * a.bf16_row + slot] : -1;
      if (pg >= 0 && pg < a.n_bf16_pages)
        kr = a.bf16_pages + (((((size_t)pg * a.T + a.t) * a.H + h) * 2 + 0) * kPage + (p & 7)) * D;
    }
    if (lane < kBfTok) src[lane] = kr;
    // copy the batch's K and V rows into LDS: 16 bytes per lane per step, all loads issued first
    constexpr int CPR = 2 * D / 16;                    // 16-byte chunks per row
    constexpr int NCH = kBfTok * CPR / 64;             // chunks per lane per half
    u32x4 kbuf[NCH], vbuf[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int cidx = k * 64 + lane, row = cidx / CPR, part = cidx % CPR;
      const uint16_t* rp = src[row];
      kbuf[k] = rp ? *(const u32x4*)(rp + part * 8) : u32x4{0, 0, 0, 0};
      vbuf[k] = rp ? *(const u32x4*)(rp + (size_t)kPage * D + part * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int cidx = k * 64 + lane, row = cidx / CPR, part = cidx % CPR;
      *(u32x4*)(krow + row * ROWB + part * 16) = kbuf[k];
      *(u32x4*)(vrow + row * ROWB + part * 16) = vbuf[k];
    }
    // score of this lane's token
    float s = -__builtin_inff();
    if (kr) {
      const uint16_t* kk = (const uint16_t*)(krow + lane * ROWB);
      float acc0 = 0.f, acc1 = 0.f;
#pragma unroll 8
      for (int j = 0; j < HALF; ++j) {
        const float2 cs = phase(rope, a.rope_tiles, D, p, j);
        const float x = bf2f(kk[j]), y = bf2f(kk[j + HALF]);
        acc0 = fmaf(qp[2 * j], x * cs.x - y * cs.y, acc0);
        acc1 = fmaf(qp[2 * j + 1], y * cs.x + x * cs.y, acc1);
      }
      s = acc0 + acc1;
      if (a.scores) a.scores[((size_t)b * a.Hq + hq) * a.max_seq_len + p] = s * kLn2;
    }
    // online softmax over the batch
    const float mb = wave_max(s);
    const float mn = fmaxf(m, mb);
    if (mn > -__builtin_inff()) {
      const float f = __builtin_amdgcn_exp2f(m - mn);
      const float w = kr ? __builtin_amdgcn_exp2f(s - mn) : 0.f;
      if (lane < kBfTok) wl[lane] = w;
      l = l * f + wave_sum(w);
      oa *= f;
      ob *= f;
      m = mn;
      // output channels j and j + d/2 (j = lane) over the batch's tokens
      if (lane < HALF) {
        const int nb = min(kBfTok, n_tok - i0);
        for (int r = 0; r < nb; ++r) {
          const float w_r = wl[r];
          const uint16_t* vv = (const uint16_t*)(vrow + r * ROWB);
          oa = fmaf(w_r, bf2f(vv[lane]), oa);
          ob = fmaf(w_r, bf2f(vv[lane + HALF]), ob);
        }
      }
    }
  }
  float* rec = a.part + (((size_t)b * a.Hq + hq) * (a.n_chunks + 1) + a.n_chunks) * (D + 2);
  if (lane == 0) { rec[0] = m; rec[1] = l; }
  if (lane < HALF) {
    rec[2 + lane] = oa;
    rec[2 + lane + HALF] = ob;
  }
}

// ------------------------------------------------------------------ coded part
template <int D, int C, bool SCORES>
__global__ __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_kernel(AttnArgs a, const float* __restrict__ rope, int n_bf16_wg, int n_cg) {
  constexpr int NG = D / C;       // groups per head
  constexpr int HALF = D / 2;
  constexpr int QP = HALF / 4;    // channel pairs per lane (score)
  constexpr int QV = D / 4;       // output channels per lane (value sum)
  constexpr int NT = 4;           // tiles per prefetch batch
  static_assert(NG >= 4 && QP % 8 == 0 && QV % 8 == 0, "shape outside the compiled set");
  extern __shared__ __align__(16) unsigned char smem[];
  _Float16* kl = (_Float16*)smem;                          // [NG][256][C]
  _Float16* vl = kl + (size_t)kCodes * D;                  // [NG][256][C]
  float* qs = (float*)(vl + (size_t)kCodes * D);           // [kNW][D]
  float* e0buf = qs + kNW * D;                             // [kNW][2][D]
  int* ptbuf = (int*)(e0buf + kNW * 2 * D);                // [kNW][kPtBatch]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  if ((int)blockIdx.x < n_bf16_wg) {
    bf16_part<D>(a, rope, blockIdx.x * kNW + wave, lane, smem + (size_t)wave * kBf16Scratch<D>);
    return;
  }
  int bid = blockIdx.x - n_bf16_wg;
  const int cg = bid % n_cg; bid /= n_cg;
  const int hq = bid % a.Hq; bid /= a.Hq;
  const int b = bid;
  const int h = hq / (a.Hq / a.H);
  const int beta = a.t / a.Tc, tau = a.t % a.Tc;
  const int nblk = a.T / a.Tc;
  const int chunk = cg * kNW + wave;
  const int qe = min(a.q_end[b] & ~7, min(a.seq_len[b], a.max_seq_len));
  const int P_lo = chunk * a.chunk_pages;
  const int P_hi = min(qe >> 3, P_lo + a.chunk_pages);
  const bool active = chunk < a.n_chunks;

  stage_slice<D, C>(a, beta, 0, h, tau, kl);
  stage_slice<D, C>(a, beta, 1, h, tau, vl);
  // rotated query of this (b, hq), log2 units, pairs interleaved
  float* qw = qs + wave * D;
  if (lane < HALF) {
    const int pq = min(max(a.pos[b], 0), a.rope_tiles * kTile - 1);
    const uint16_t* qv = a.q + ((size_t)b * a.Hq + hq) * D;
    const float2 cs = phase(rope, a.rope_tiles, D, pq, lane);
    const float x = bf2f(qv[lane]), y = bf2f(qv[lane + HALF]);
    qw[2 * lane] = (x * cs.x - y * cs.y) * a.scale_log2e;
    qw[2 * lane + 1] = (y * cs.x + x * cs.y) * a.scale_log2e;
  }
  __syncthreads();
  if (!active) return;

  const int qt = lane & 3, t = lane >> 2;       // lane quarter, token in tile
  float m = -__builtin_inff(), l = 0.f;
  float o[QV];
#pragma unroll
  for (int i = 0; i < QV; ++i) o[i] = 0.f;

  if (P_lo < P_hi && a.n_index_pages > 0) {
    // F, G: the query turned back by the token's in-tile offset t, for this lane's pairs
    float F[QP], Gc[QP];
    {
      const float* e1 = rope + (size_t)(a.rope_tiles + t) * D;
#pragma unroll
      for (int jj = 0; jj < QP; ++jj) {
        const int j = qt * QP + jj;
        const float A = qw[2 * j], Bq = qw[2 * j + 1];
        const float c1 = e1[2 * j], s1 = e1[2 * j + 1];
        F[jj] = A * c1 + Bq * s1;
        Gc[jj] = Bq * c1 - A * s1;
      }
    }
    // byte offsets (4-aligned) of the index-row words holding this lane's codes
    const int glo = (qt * QP) / C, ghi = (qt * QP + HALF) / C, gv = (qt * QV) / C;
    const int wlo = glo & ~3, whi = ghi & ~3, wv = gv & ~3;
    const int r = t & 7;
    const size_t row_stride = (size_t)kPage * NG;
    float* e0s = e0buf + wave * 2 * D;
    int* ptl = ptbuf + wave * kPtBatch;
    const int* pt = a.page_table + (size_t)b * a.max_pages;
    int pt_base = -kPtBatch;
    // stage the page ids of pages [P, P + kPtBatch) into LDS (all loads in flight, one wait)
    auto stage_pt = [&](int P) {
      pt_base = P;
      int v[kPtBatch / 64];
#pragma unroll
      for (int k = 0; k < kPtBatch / 64; ++k) v[k] = pt[min(P + k * 64 + lane, a.max_pages - 1)];
#pragma unroll
      for (int k = 0; k < kPtBatch / 64; ++k) {
        const int q = P + k * 64 + lane;
        ptl[k * 64 + lane] = (q < P_hi && v[k] >= 0 && v[k] < a.n_index_pages) ? v[k] : -1;
      }
    };
    // everything a lane loads for the tile starting at page P0
    struct TileIn {
      int phys;
      uint32_t kwl, kwh, vw;
      float2 e0;
    };
    auto fetch = [&](int P0) -> TileIn {
      TileIn in;
      if (P0 + 1 >= pt_base + kPtBatch) stage_pt(P0);
      in.phys = P0 < P_hi ? ptl[P0 - pt_base + (t >> 3)] : -1;
      const uint8_t* base = a.index_pages + ((((size_t)max(in.phys, 0) * nblk + beta) * a.H + h) * 2) * row_stride + r * NG;
      in.kwl = *(const uint32_t*)(base + wlo);
      in.kwh = *(const uint32_t*)(base + whi);
      in.vw = *(const uint32_t*)(base + row_stride + wv);
      const int tile_idx = min((8 * P0) / kTile, a.rope_tiles - 1);
      in.e0 = *(const float2*)(rope + (size_t)tile_idx * D + 2 * (lane % HALF));
      return in;
    };
    auto tile = [&](int P0, const TileIn& in, int buf) {
      float* er = e0s + buf * D;
      if (lane < HALF) *(float2*)(er + 2 * lane) = in.e0;
      const int p = 8 * P0 + t;
      const bool valid = in.phys >= 0 && p >= a.n_sink;
      // keys: low channels [qt*QP, qt*QP + QP) and the partners + d/2
      f16x8 xl[QP / 8], xh[QP / 8];
#pragma unroll
      for (int v = 0; v < QP / 8; ++v) {
        const int cl = qt * QP + 8 * v, ch = cl + HALF;
        const int gl = cl / C, gh = ch / C;
        const int codl = (in.kwl >> (8 * (gl - wlo))) & 0xff;
        const int codh = (in.kwh >> (8 * (gh - whi))) & 0xff;
        xl[v] = *(const f16x8*)(kl + ((size_t)gl * kCodes + codl) * C + cl % C);
        xh[v] = *(const f16x8*)(kl + ((size_t)gh * kCodes + codh) * C + ch % C);
      }
      float s0acc = 0.f, s1acc = 0.f;
#pragma unroll
      for (int v = 0; v < QP / 8; ++v) {
#pragma unroll
        for (int i4 = 0; i4 < 2; ++i4) {
          const f32x4 e_a = *(const f32x4*)(er + 2 * (qt * QP + 8 * v + 4 * i4));
          const f32x4 e_b = *(const f32x4*)(er + 2 * (qt * QP + 8 * v + 4 * i4) + 4);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int i = 4 * i4 + k, jj = 8 * v + i;
            const float c0 = k < 2 ? e_a[2 * k] : e_b[2 * (k - 2)];
            const float sn = k < 2 ? e_a[2 * k + 1] : e_b[2 * (k - 2) + 1];
            const float u = c0 * F[jj] + sn * Gc[jj];
            const float w_ = c0 * Gc[jj] - sn * F[jj];
            if (i & 1) { s1acc = fmaf(u, (float)xl[v][i], s1acc); s1acc = fmaf(w_, (float)xh[v][i], s1acc); }
            else       { s0acc = fmaf(u, (float)xl[v][i], s0acc); s0acc = fmaf(w_, (float)xh[v][i], s0acc); }
          }
        }
      }
      float s = s0acc + s1acc;
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s = valid ? s : -__builtin_inff();
      if (SCORES && valid && qt == 0) a.scores[((size_t)b * a.Hq + hq) * a.max_seq_len + p] = s * kLn2;
      if (__any(s > m + kRescale)) {
        const float mn = fmaxf(m, wave_max(s));
        const float f = __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
        for (int i = 0; i < QV; ++i) o[i] *= f;
        l *= f;
        m = mn;
      }
      const float w = valid ? __builtin_amdgcn_exp2f(s - m) : 0.f;
      l += (qt == 0) ? w : 0.f;
      // values: output channels [qt*QV, qt*QV + QV)
#pragma unroll
      for (int v = 0; v < QV / 8; ++v) {
        const int cv = qt * QV + 8 * v;
        const int g = cv / C;
        const int cod = (in.vw >> (8 * (g - wv))) & 0xff;
        const f16x8 x = *(const f16x8*)(vl + ((size_t)g * kCodes + cod) * C + cv % C);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[8 * v + i] = fmaf(w, (float)x[i], o[8 * v + i]);
      }
    };
    // Software pipeline in batches of NT tiles: each iteration loads the inputs of
    // the next batch, computes the current batch, then moves next to current, so no
    // load is in flight across the loop back-edge.
    TileIn cur[NT], nxt[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) cur[i] = fetch(P_lo + 2 * i);
    for (int P0 = P_lo; P0 < P_hi; P0 += 2 * NT) {
#pragma unroll
      for (int i = 0; i < NT; ++i) nxt[i] = fetch(P0 + 2 * NT + 2 * i);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        if (P0 + 2 * i < P_hi) tile(P0 + 2 * i, cur[i], i & 1);
      }
#pragma unroll
      for (int i = 0; i < NT; ++i) cur[i] = nxt[i];
    }
  }
  // fold the 16 token lanes of each quarter and write the partial (m, l, o)
#pragma unroll
  for (int off = 4; off < 64; off <<= 1) {
#pragma unroll
    for (int i = 0; i < QV; ++i) o[i] += __shfl_xor(o[i], off);
  }
  l = wave_sum(l);
  float* rec = a.part + (((size_t)b * a.Hq + hq) * (a.n_chunks + 1) + chunk) * (D + 2);
  if (lane == 0) { rec[0] = m; rec[1] = l; }
  if (t == 0) {
#pragma unroll
    for (int i = 0; i < QV; ++i) rec[2 + qt * QV + i] = o[i];
  }
}

// ------------------------------------------------------------------ merge
// One workgroup per (b, hq): m = max m_i, l = sum l_i 2^(m_i - m),
// out = sum o_i 2^(m_i - m) / l, lse = (m + log2 l) ln 2.
constexpr int kMergeMax = 1024;
__global__ __launch_bounds__(128) void merge_kernel(AttnArgs a) {
  __shared__ float sw[kMergeMax];
  __shared__ float red[2];
  const int item = blockIdx.x;           // b * Hq + hq
  const int S = a.n_chunks + 1;
  const float* rec = a.part + (size_t)item * S * (a.d + 2);
  const int tid = threadIdx.x;
  float mloc = -__builtin_inff();
  for (int i = tid; i < S; i += blockDim.x) {
    const float mi = rec[(size_t)i * (a.d + 2)];
    sw[i] = mi;
    mloc = fmaxf(mloc, mi);
  }
  mloc = wave_max(mloc);
  if ((tid & 63) == 0) red[tid >> 6] = mloc;
  __syncthreads();
  const float M = fmaxf(red[0], red[1]);
  __syncthreads();
  float lloc = 0.f;
  for (int i = tid; i < S; i += blockDim.x) {
    const float li = rec[(size_t)i * (a.d + 2) + 1];
    const float f = (M > -__builtin_inff() && li > 0.f) ? exp2f(sw[i] - M) : 0.f;
    sw[i] = f;
    lloc += li * f;
  }
  lloc = wave_sum(lloc);
  if ((tid & 63) == 0) red[tid >> 6] = lloc;
  __syncthreads();
  const float Ls = red[0] + red[1];
  for (int ch = tid; ch < a.d; ch += blockDim.x) {
    float acc = 0.f;
#pragma unroll 8
    for (int i = 0; i < S; ++i) {
      const float f = sw[i];
      if (f > 0.f) acc += rec[(size_t)i * (a.d + 2) + 2 + ch] * f;
    }
    a.out[(size_t)item * a.d + ch] = Ls > 0.f ? acc / Ls : 0.f;
  }
  if (a.lse && tid == 0) a.lse[item] = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : -__builtin_inff();
}

// ------------------------------------------------------------------ RoPE tables
// rows [0, ntile): phase at 16 a; rows [ntile, ntile + 16): phase at offset o; then theta (double)
__global__ void rope_kernel(int ntile, int d, double base, float* tab) {
  const int half = d / 2;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int j = i % half;
  const double theta = pow(base, -2.0 * j / d);
  if (i < (ntile + kTile) * half) {
    const int row = i / half;
    const double p = row < ntile ? (double)kTile * row : (double)(row - ntile);
    const double ang = p * theta;
    tab[2 * (size_t)i] = (float)cos(ang);
    tab[2 * (size_t)i + 1] = (float)sin(ang);
  }
  if (i < half) ((double*)(tab + (size_t)(ntile + kTile) * d))[i] = theta;
}

template <int D, int C, bool SCORES>
hipError_t launch_attn_t(const AttnArgs& a, hipStream_t s) {
  constexpr size_t lds = lds_bytes<D>();
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_kernel<D, C, SCORES>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int n_items = a.B * a.Hq;
  const int n_bf16_wg = (n_items + kNW - 1) / kNW;
  const int n_cg = (a.n_chunks + kNW - 1) / kNW;
  const long grid = (long)n_bf16_wg + (long)n_cg * n_items;
  hipLaunchKernelGGL((attn_kernel<D, C, SCORES>), dim3((unsigned)grid), dim3(kNW * 64), lds, s, a,
                     a.rope, n_bf16_wg, n_cg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(n_items), dim3(128), 0, s, a);
  return hipGetLastError();
}

template <int D, int C>
hipError_t launch_attn_s(const AttnArgs& a, hipStream_t s) {
  return a.scores ? launch_attn_t<D, C, true>(a, s) : launch_attn_t<D, C, false>(a, s);
}

}  // namespace

int rope_tile() { return kTile; }

bool attn_supported(int d, int c) {
  if (d == 128) return c == 8 || c == 16 || c == 32;
  if (d == 64) return c == 8 || c == 16;
  return false;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  const int c = a.G / a.Tc;
  if (a.d == 128) {
    if (c == 8) return launch_attn_s<128, 8>(a, s);
    if (c == 16) return launch_attn_s<128, 16>(a, s);
    return launch_attn_s<128, 32>(a, s);
  }
  if (c == 8) return launch_attn_s<64, 8>(a, s);
  return launch_attn_s<64, 16>(a, s);
}

hipError_t launch_rope_tables(int ntile, int d, double base, float* tab, hipStream_t s) {
  const int n = (ntile + kTile) * (d / 2);
  hipLaunchKernelGGL(rope_kernel, dim3((n + 255) / 256), dim3(256), 0, s, ntile, d, base, tab);
  return hipGetLastError();
}

}  // namespace lvq
