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
//  * Workgroup = 12 waves (3 per SIMD) on one query head; 256/Hq workgroups per
//    head, one resident per CU.  The step-t K and V slices of the head
//    (2 x 256 codes x d channels, 128 KB at d = 128) are staged once per
//    workgroup in LDS as float16, which holds the bf16 codewords exactly.
//  * Token-balanced split: a head's work list is the batch's 16-token tiles in
//    sequence order (each sequence's coded tiles, then its bf16 tiles counted as
//    kBfCost units); each wave takes an equal contiguous range of it, crossing
//    sequence boundaries, and writes one partial (max, sum, output) record per
//    sequence its range meets.  Mixed lengths and single long sequences keep every
//    wave busy for the same time.
//  * A tile is 16 positions (2 pages); four lanes share a token: lane quarter
//    qt owns channel pairs [qt*d/8, (qt+1)*d/8) of the score and output channels
//    [qt*d/4, (qt+1)*d/4) of the value sum.  Keys and values are gathered from
//    LDS (16-byte reads), the value sum is accumulated in registers.
//  * RoPE after dequantisation without per-token trigonometry: position
//    16a + o has phase E(16a) * E(o); the lane folds E(o) and the query once per
//    sequence into coefficients F, G, so per channel pair j the score gets
//    (c0 F_j + s0 G_j) k_j + (c0 G_j - s0 F_j) k_{j+d/2} with (c0, s0) = E(16a)
//    read from a per-tile LDS row: six float32 operations, the key read by
//    v_fma_mix straight from float16.
//  * Index words (only the bytes a lane needs) and the tile phases of the next
//    tile are loaded while the current tile computes, into the other of two
//    register sets (the loop body holds two tiles, so nothing is copied).
//  * Scores are kept in log2 units (scale * log2 e folded into the query); a
//    running maximum is kept lazily (rescale only when a score passes it by
//    more than 8 in log2 units).
//  * The bf16 sink and recent tiles are read from the bf16 pages in float32 with
//    the same lane layout and factorisation.
//  * LDS layout [code][16-byte chunk] and a per-lane chunk order keep the lanes
//    of an LDS access phase on distinct banks.
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
constexpr int kNW = 12;            // waves per workgroup
constexpr int kWavesPerSimd = 3;   // occupancy the register budget is sized for
constexpr int kTile = 16;          // positions per tile (RoPE table granularity)
constexpr int kPtBatch = 128;      // page ids staged in LDS per wave at a time

// Tile-phase buffer (floats): the d/2 pairs in 4 quarter blocks of d/8 pairs, each
// block followed by 16 bytes of padding so the four quarters read distinct LDS banks.
template <int D>
constexpr int phase_buf_floats() { return 4 * (2 * (D / 8) + 4); }

template <int D>
constexpr size_t lds_bytes() {
  return (size_t)2 * kCodes * D * 2 + (size_t)kNW * (2 * phase_buf_floats<D>() * 4 + kPtBatch * 4);
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

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
template <int D, int C>
struct SliceStage {
  static constexpr int NG = D / C;
  static constexpr int NCH = D / 8;
  static constexpr int NTH = kNW * 64;
  static constexpr int PER = (kCodes * D / 8 + NTH - 1) / NTH;   // 16-byte pieces per thread and slice
  u16x8 v[2][PER];
  __device__ __forceinline__ void load(const AttnArgs& a, int beta, int h, int tau);
  __device__ __forceinline__ void store(_Float16* dst) const;
};
template <int D, int C>
__device__ __forceinline__ void SliceStage<D, C>::load(const AttnArgs& a, int beta, int h, int tau) {
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
template <int D, int C>
__device__ __forceinline__ void SliceStage<D, C>::store(_Float16* dst) const {
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

template <int D, int C, bool SCORES, bool WIDE>
__global__ __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd, kWavesPerSimd)))
void attn_kernel(AttnArgs a, const float* __restrict__ rope, int wph) {
  constexpr int NG = D / C;       // groups per head
  constexpr int HALF = D / 2;
  constexpr int QP = HALF / 4;    // channel pairs per lane (score)
  constexpr int QV = D / 4;       // output channels per lane (value sum)
  constexpr int NCH = D / 8;      // 16-byte chunks per codeword row in LDS
  constexpr int KPC = QP / 8;     // key chunks per lane in each half
  constexpr int NV = QV / 8;      // value chunks per lane
  static_assert(NG >= 4 && QP % 8 == 0 && QV % 8 == 0, "shape outside the compiled set");
  extern __shared__ __align__(16) unsigned char smem[];
  _Float16* kl = (_Float16*)smem;                          // [256][D/8][8]
  _Float16* vl = kl + (size_t)kCodes * D;                  // [256][D/8][8]
  constexpr int ER = phase_buf_floats<D>();
  static_assert(2 * ER >= D, "the phase buffers also hold the rotated query");
  float* e0buf = (float*)(vl + (size_t)kCodes * D);        // [kNW][2][ER]
  int* ptbuf = (int*)(e0buf + kNW * 2 * ER);               // [kNW][kPtBatch]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // block = kw * Hq + hq: with Hq a multiple of 8 a head's workgroups share one XCD (and its
  // L2 copy of the head's codebook slices)
  const int hq = blockIdx.x % a.Hq, kw = blockIdx.x / a.Hq;
  const int h = hq / (a.Hq / a.H);
  const int beta = a.t / a.Tc, tau = a.t % a.Tc;
  const int nblk = a.T / a.Tc;
  const int W = wph * kNW;          // waves on this query head
  const int wg = kw * kNW + wave;   // this wave among them

  // The first 64 sequences' lengths are loaded before the slices: vector loads return
  // in order, so loaded after them the scan below would wait for every slice load.
  // (unconditional loads at a clamped index: a load under a lane mask is waited for at
  // the end of its branch; a.B >= 1 for every launch)
  const int b_first = min(lane, a.B - 1);
  const int len_first = a.seq_len[b_first];
  const int qe_first = a.q_end[b_first];
  SliceStage<D, C> slices;
  slices.load(a, beta, h, tau);
  // the work list's length, and (one wave of the launch) the sequences' first units;
  // the first 64 sequences' counts and inclusive sums stay in registers
  int total = 0, n_first = 0, incl_first = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int b = b0 + lane;
    const int n = b < a.B ? (b0 == 0 ? seq_tiles_of(a, len_first, qe_first) : seq_tiles(a, b)).total : 0;
    const int incl = total + wave_incl_scan(n);
    if (b0 == 0) { n_first = n; incl_first = incl; }
    if (hq == 0 && wg == 0 && b < a.B) a.tile_start[b] = incl - n;
    total += wave_sum_i(n);
  }
  if (hq == 0 && wg == 0 && lane == 0) a.tile_start[a.B] = total;
  total = __builtin_amdgcn_readfirstlane(total);   // wave-uniform: keep it in a scalar register
  const int w_lo = __builtin_amdgcn_readfirstlane(range_lo(wg, total, W));
  const int w_hi = __builtin_amdgcn_readfirstlane(range_lo(wg + 1, total, W));

  // the sequence holding unit w_lo, and its first unit
  int b = 0, tb = 0;
  if (w_lo < w_hi) {
    int base = 0;
    for (int b0 = 0; b0 < a.B; b0 += 64) {
      const int bb = b0 + lane;
      const int n = b0 == 0 ? n_first : (bb < a.B ? seq_tiles(a, bb).total : 0);
      const int incl = b0 == 0 ? incl_first : base + wave_incl_scan(n);
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

  slices.store(kl);
  __syncthreads();
  if (w_lo == w_hi) return;

  const int qt = lane & 3, t = lane >> 2;       // lane quarter, token in tile
  // Chunk order per lane, so the lanes of one LDS access phase hit distinct banks:
  // register block v of the keys holds the lane's chunk kperm(v) (pairs swap with the
  // token's parity), value block v holds chunk (v + vrot) mod NV.
  const int kswap = (KPC == 2) ? (t & 1) : 0;
  const int vrot = (NV == 4) ? ((t + 2 * (qt >> 1)) & 3) : (t & (NV - 1));
  // byte offsets (4-aligned) of the index-row words holding this lane's codes
  const int glo = (qt * QP) / C, ghi = (qt * QP + HALF) / C, gv = (qt * QV) / C;
  const int wlo = glo & ~3, whi = ghi & ~3, wv = gv & ~3;
  const int r = t & 7;
  const size_t row_stride = (size_t)kPage * NG;
  const size_t page_bytes = (size_t)nblk * a.H * 2 * row_stride;
  // the rows of (beta, h) in page 0 (wave-uniform), and the lane's three index words
  // as byte offsets from a page's start
  const uint8_t* head_rows = a.index_pages + (((size_t)beta * a.H + h) * 2) * row_stride;
  uint32_t o_kl = r * NG + wlo, o_kh = r * NG + whi, o_v = (uint32_t)row_stride + r * NG + wv;
  // opaque copies: three independent 32-bit offsets from the uniform base (otherwise the
  // compiler derives one load's address from another's with 64-bit arithmetic)
  asm volatile("" : "+v"(o_kl), "+v"(o_kh), "+v"(o_v));
  // Per-lane gather constants: bit offset of the code in its index word, and the LDS
  // byte offset of the chunk (code x of chunk k sits at byte (x * NCH + k) * 16).
  constexpr int kRowShift = (NCH == 16) ? 8 : 7;   // log2(NCH * 16)
  // A partner chunk (channels + d/2) sits HALF / 8 chunks further on (an immediate
  // offset of the LDS read) and its code is KSH bits further along in its index word
  // than the low chunk's code in its own word (the same for every lane).
  constexpr uint32_t kHighOff = (HALF / 8) * 16;
  // HALF / C groups separate the two codes; with a multiple of 4 they sit at the same
  // byte of their words, with 2 (the low code in byte 0 or 1) two bytes further on.
  static_assert((HALF / C) % 4 == 0 || HALF / C == 2, "shape outside the compiled set");
  constexpr uint32_t kHighShift = ((HALF / C) % 4 == 0) ? 0 : 8 * (HALF / C);
  // With 256-byte code rows (d = 128) the gather address is one byte permute: byte 0 is
  // the chunk offset, byte 1 the code taken from its index word, byte 2 the slice base
  // (0 for keys, 1 for values at 64 KB).  Otherwise a bit-field extract and a shift.
  constexpr bool kPermAddr = kRowShift == 8;
  auto code_sel = [](uint32_t sh) -> uint32_t {
    return kPermAddr ? (0x0c020000u | ((4u + sh / 8) << 8)) : sh;
  };
  uint32_t sell[KPC], selh[KPC], offl[KPC], selv[NV], offv[NV];
#pragma unroll
  for (int v = 0; v < KPC; ++v) {
    const int cl = qt * QP + 8 * (v ^ kswap);
    const uint32_t sh = 8 * (cl / C - wlo);
    sell[v] = code_sel(sh);
    selh[v] = code_sel(sh + kHighShift);
    offl[v] = (uint32_t)(cl / 8) * 16;
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int cv = qt * QV + 8 * ((v + vrot) & (NV - 1));
    selv[v] = code_sel(8 * (cv / C - wv));
    offv[v] = (uint32_t)(kCodes * D * 2) + (uint32_t)(cv / 8) * 16;   // value slices follow the keys
  }
  auto gather = [&](uint32_t word, uint32_t sel, uint32_t off) -> uint32_t {
    if constexpr (kPermAddr) return __builtin_amdgcn_perm(word, off, sel);
    else return (__builtin_amdgcn_ubfe(word, sel, 8) << kRowShift) + off;
  };
  float* e0s = e0buf + wave * 2 * ER;
  int* ptl = ptbuf + wave * kPtBatch;

  // ---- the sequences the range meets, one partial record each
  int pos_t = w_lo;
  while (pos_t < w_hi && b < a.B) {
    const SeqTiles st = seq_tiles(a, b);
    const int u_lo = pos_t - tb, u_hi = min(w_hi - tb, st.total);
    if (u_lo < u_hi) {
      // the lane's layout values again, from an opaque copy of the lane id, so nothing
      // derived from them for this sequence is held in registers across the loop
      int lane_s = lane;
      asm volatile("" : "+v"(lane_s));
      const int qt = lane_s & 3, t = lane_s >> 2;
      const int kswap = (KPC == 2) ? (t & 1) : 0;
      const int vrot = (NV == 4) ? ((t + 2 * (qt >> 1)) & 3) : (t & (NV - 1));
      const int L = max(min(a.seq_len[b], a.max_seq_len), 0);
      const int qe = max(min(a.q_end[b] & ~7, L), 0);
      const int ns = min(a.n_sink, L);
      const int r0 = max(qe, a.n_sink);
      const int vt_lo = r0 / kTile;
      // F, G: the rotated query (log2 units) turned back by the token's in-tile offset t,
      // for this lane's pairs
      float F[QP], Gc[QP];
      {
        // lane j < d/2 rotates pair j of the query into the wave's phase buffer (free
        // between tiles; the wave's LDS accesses complete in order)
        float* qw = e0s;
        if (lane < HALF) {
          const int pq = min(max(a.pos[b], 0), a.rope_tiles * kTile - 1);
          const uint16_t* qv = a.q + ((size_t)b * a.Hq + hq) * D;
          const float2 cs = phase(rope, a.rope_tiles, D, pq, lane);
          const float x = bf2f(qv[lane]), y = bf2f(qv[lane + HALF]);
          qw[2 * lane] = (x * cs.x - y * cs.y) * a.scale_log2e;
          qw[2 * lane + 1] = (y * cs.x + x * cs.y) * a.scale_log2e;
        }
        // pairs j = qt*QP + 8*(v ^ kswap) + i of register block v, read at constant offsets
        // from one base per block (no per-pair offsets held across the sequence loop)
        // (32-bit element offsets from the uniform table base)
#pragma unroll
        for (int v = 0; v < KPC; ++v) {
          const int jb = qt * QP + 8 * (v ^ kswap);
          const float* qwv = qw + 2 * jb;
          const uint32_t e1v = (uint32_t)((a.rope_tiles + t) * D + 2 * jb);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int jj = 8 * v + i;
            const float A = qwv[2 * i], Bq = qwv[2 * i + 1];
            const float c1 = rope[e1v + 2 * i], s1 = rope[e1v + 2 * i + 1];
            F[jj] = A * c1 + Bq * s1;
            Gc[jj] = Bq * c1 - A * s1;
          }
        }
      }
      float m = kNoMax, l = 0.f;
      float m_hi = kNoMax + kRescale;   // rescale threshold
      float o[QV];
#pragma unroll
      for (int i = 0; i < QV; ++i) o[i] = 0.f;
      const int P_lo = 2 * u_lo;
      const int P_hi = min(2 * min(u_hi, st.coded), qe >> 3);
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
        if constexpr (WIDE) {
          const uint8_t* base = head_rows + (size_t)(uint32_t)max(in.phys, 0) * page_bytes;
          in.kwl = *(const uint32_t*)(base + o_kl);
          in.kwh = *(const uint32_t*)(base + o_kh);
          in.vw = *(const uint32_t*)(base + o_v);
        } else {
          // the pool spans under 4 GiB and 2^24 pages: 32-bit offsets from a uniform base
          const uint32_t po = __umul24((uint32_t)max(in.phys, 0), (uint32_t)page_bytes);
          in.kwl = *(const uint32_t*)(head_rows + (po + o_kl));
          in.kwh = *(const uint32_t*)(head_rows + (po + o_kh));
          in.vw = *(const uint32_t*)(head_rows + (po + o_v));
        }
        const int tile_idx = min((8 * P0) / kTile, a.rope_tiles - 1);
        in.e0 = *(const float2*)((const char*)rope + (uint32_t)(4 * (tile_idx * D + 2 * (lane % HALF))));
        return in;
      };
      auto tile = [&](int P0, const TileIn& in, int buf) {
        float* er = e0s + buf * ER;
        if (lane < HALF) *(float2*)(er + (lane / QP) * (2 * QP + 4) + 2 * (lane % QP)) = in.e0;
        const int p = 8 * P0 + t;
        const bool valid = in.phys >= 0 && p >= a.n_sink;
        // keys: low channels [qt*QP, qt*QP + QP) and the partners + d/2
        f16x8 xl[QP / 8], xh[QP / 8];
  #pragma unroll
        for (int v = 0; v < KPC; ++v) {
          xl[v] = lds_read16(gather(in.kwl, sell[v], offl[v]));
          xh[v] = lds_read16(gather(in.kwh, selh[v], offl[v]) + kHighOff);
        }
        float s0acc = 0.f, s1acc = 0.f;
  #pragma unroll
        for (int v = 0; v < QP / 8; ++v) {
  #pragma unroll
          for (int i4 = 0; i4 < 2; ++i4) {
            const float* ep = er + qt * (2 * QP + 4) + 2 * (8 * (v ^ kswap) + 4 * i4);
            const f32x4 e_a = *(const f32x4*)ep;
            const f32x4 e_b = *(const f32x4*)(ep + 4);
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
        const float s = valid ? quad_sum(s0acc + s1acc) : -__builtin_inff();
        if (SCORES && valid && qt == 0) a.scores[((size_t)b * a.Hq + hq) * a.max_seq_len + p] = s * kLn2;
        if (__any(s > m_hi)) {
          const float mn = fmaxf(m, wave_max(s));
          const float f = __builtin_amdgcn_exp2f(m - mn);
  #pragma unroll
          for (int i = 0; i < QV; ++i) o[i] *= f;
          l *= f;
          m = mn;
          m_hi = mn + kRescale;
        }
        const float w = __builtin_amdgcn_exp2f(s - m);   // 0 for an invalid token (s = -inf)
        l += w;   // every lane of a token adds the same weight; folded over tokens only
        // values: output channels [qt*QV, qt*QV + QV)
  #pragma unroll
        for (int v = 0; v < NV; ++v) {
          const f16x8 x = lds_read16(gather(in.vw, selv[v], offv[v]));
  #pragma unroll
          for (int i = 0; i < 8; ++i) o[8 * v + i] = fmaf(w, (float)x[i], o[8 * v + i]);
        }
      };
      // Software pipeline, two tiles per iteration: each tile's inputs are loaded while
      // the tile before it is computed, into the other of two register sets, so the
      // sets alternate without copies.
      if (P_lo < P_hi) {
        TileIn in0 = fetch(P_lo);
        for (int P0 = P_lo;; P0 += 4) {
          const TileIn in1 = fetch(P0 + 2);
          tile(P0, in0, 0);
          if (P0 + 2 >= P_hi) break;
          in0 = fetch(P0 + 4);
          tile(P0 + 2, in1, 1);
          if (P0 + 4 >= P_hi) break;
        }
      }
      // bf16 sink and recent tokens (virtual tiles after the coded ones; a wave takes
      // those whose first unit lies in its range), with the same lane layout and RoPE
      // factorisation; keys and values are read from the bf16 pages and used in float32
      // (a bf16 value need not fit float16).
      const int vt_first = (max(u_lo, st.coded) - st.coded + kBfCost - 1) / kBfCost;
      const int vt_end = u_hi > st.coded ? (u_hi - st.coded + kBfCost - 1) / kBfCost : 0;
      for (int vt = vt_first; vt < vt_end; ++vt) {
        const bool sink_tile = ns > 0 && vt == 0;
        const int a_tile = sink_tile ? 0 : vt_lo + vt - (ns > 0 ? 1 : 0);
        const int lo = sink_tile ? 0 : r0, hi = sink_tile ? ns : L;
        const int p = kTile * a_tile + t;
        const uint16_t* krow = nullptr;
        if (p >= lo && p < hi) {
          const int slot = sink_tile ? 0 : 1 + (p >> 3) - (qe >> 3);
          const int pg = slot < a.bf16_row ? a.bf16_table[(size_t)b * a.bf16_row + slot] : -1;
          if (pg >= 0 && pg < a.n_bf16_pages)
            krow = a.bf16_pages + (((((size_t)pg * a.T + a.t) * a.H + h) * 2) * kPage + (p & 7)) * D;
        }
        const bool valid = krow != nullptr;
        float* er = e0s;
        if (lane < HALF) {
          const int tile_idx = min(a_tile, a.rope_tiles - 1);
          *(float2*)(er + (lane / QP) * (2 * QP + 4) + 2 * (lane % QP)) =
              *(const float2*)(rope + (size_t)tile_idx * D + 2 * lane);
        }
        float s0acc = 0.f, s1acc = 0.f;
        if (valid) {
  #pragma unroll
          for (int v = 0; v < KPC; ++v) {
            const int cl = qt * QP + 8 * (v ^ kswap), ch = cl + HALF;
            const u16x8 xlr = *(const u16x8*)(krow + cl);
            const u16x8 xhr = *(const u16x8*)(krow + ch);
  #pragma unroll
            for (int i4 = 0; i4 < 2; ++i4) {
              const float* ep = er + qt * (2 * QP + 4) + 2 * (8 * (v ^ kswap) + 4 * i4);
              const f32x4 e_a = *(const f32x4*)ep;
              const f32x4 e_b = *(const f32x4*)(ep + 4);
  #pragma unroll
              for (int k = 0; k < 4; ++k) {
                const int i = 4 * i4 + k, jj = 8 * v + i;
                const float c0 = k < 2 ? e_a[2 * k] : e_b[2 * (k - 2)];
                const float sn = k < 2 ? e_a[2 * k + 1] : e_b[2 * (k - 2) + 1];
                const float u = c0 * F[jj] + sn * Gc[jj];
                const float w_ = c0 * Gc[jj] - sn * F[jj];
                s0acc = fmaf(u, bf2f(xlr[i]), s0acc);
                s1acc = fmaf(w_, bf2f(xhr[i]), s1acc);
              }
            }
          }
        }
        const float s = valid ? quad_sum(s0acc + s1acc) : -__builtin_inff();
        if (SCORES && valid && qt == 0) a.scores[((size_t)b * a.Hq + hq) * a.max_seq_len + p] = s * kLn2;
        if (__any(s > m_hi)) {
          const float mn = fmaxf(m, wave_max(s));
          const float f = __builtin_amdgcn_exp2f(m - mn);
  #pragma unroll
          for (int i = 0; i < QV; ++i) o[i] *= f;
          l *= f;
          m = mn;
          m_hi = mn + kRescale;
        }
        const float w = __builtin_amdgcn_exp2f(s - m);   // 0 for an invalid token (s = -inf)
        l += w;   // every lane of a token adds the same weight; folded over tokens only
        if (valid) {
          const uint16_t* vrow = krow + (size_t)kPage * D;
  #pragma unroll
          for (int v = 0; v < NV; ++v) {
            const u16x8 x = *(const u16x8*)(vrow + qt * QV + 8 * ((v + vrot) & (NV - 1)));
  #pragma unroll
            for (int i = 0; i < 8; ++i) o[8 * v + i] = fmaf(w, bf2f(x[i]), o[8 * v + i]);
          }
        }
      }
      // value block v holds chunk (v + vrot) mod NV: put chunk c back in block c
      {
        float ot[QV];
#pragma unroll
        for (int c = 0; c < NV; ++c) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            float val = o[8 * c + i];
#pragma unroll
            for (int k = 1; k < NV; ++k) val = (vrot == k) ? o[8 * ((c - k) & (NV - 1)) + i] : val;
            ot[8 * c + i] = val;
          }
        }
#pragma unroll
        for (int i = 0; i < QV; ++i) o[i] = ot[i];
      }
      // fold the 16 token lanes of each quarter and write the partial (m, l, o)
#pragma unroll
      for (int off = 4; off < 64; off <<= 1) {
#pragma unroll
        for (int i = 0; i < QV; ++i) o[i] += __shfl_xor(o[i], off);
      }
#pragma unroll
      for (int off = 4; off < 64; off <<= 1) l += __shfl_xor(l, off);
      float* rec = a.part + ((size_t)hq * a.n_rec + wg + b) * (D + 2);
      if (lane == 0) { rec[0] = m; rec[1] = l; }
      if (t == 0) {
#pragma unroll
        for (int i = 0; i < QV; ++i) rec[2 + qt * QV + i] = o[i];
      }
    }
    pos_t = __builtin_amdgcn_readfirstlane(tb + u_hi);
    tb = __builtin_amdgcn_readfirstlane(tb + st.total);
    b = __builtin_amdgcn_readfirstlane(b + 1);
  }
}

// ------------------------------------------------------------------ grouped-query decode
// kGroupHeads (4) query heads per KV head share each key's dequantisation and tile
// rotation.  A quad of four waves covers the 16 positions of a tile: member m of the quad
// takes in-tile offsets 4m..4m+3, one per 16-lane row r (offset o = 4m + r), so a lane's
// offset never changes and its query coefficients F, G (4 heads x 4 channel pairs) are set
// once per sequence.  Lane s of a row owns channel pairs 4s..4s+3 of the score (channels
// 4s.. and d/2 + 4s..) and output channels 8s..8s+7 of the value sum, for all four heads.
// Per token the lane rotates its four key pairs by the tile phase E(16a) once (four mixed
// float16/float32 operations per pair) and forms the four partial scores (two FMAs per
// pair and head); a transposing reduction over the row (eleven DPP and select operations
// for the four heads) leaves the score of head s/4 in the lanes 4(s/4)..4(s/4)+3, which
// keep that head's running maximum and sum, and three DPP row rotations give every lane
// the four weights for the value sum.  About 7 lane operations per (token, head) against
// 10.4 for the per-head kernel.  The work list of a KV head is the same as a query
// head's; its ranges go to quads, and each wave of a quad writes its own partial record
// (four rows, one per head) per sequence its range meets.
constexpr int kGW = 16;     // waves per workgroup: four quads, four waves per SIMD
constexpr int kGPh = 128;   // floats per phase row: 64 pairs of (cos, sin)

template <int D>
constexpr size_t group_lds_bytes() {
  return (size_t)2 * kCodes * D * 2 + (size_t)kGW * (2 * kGPh * 4 + kPtBatch * 4);
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef const f16x4 __attribute__((address_space(3)))* lds_f16x4_ptr;
__device__ __forceinline__ f16x4 lds_read8(uint32_t addr) { return *(lds_f16x4_ptr)(size_t)addr; }

// DPP lane moves within 16-lane rows (every lane of the wave active)
constexpr int kDppRowRor4 = 0x124, kDppRowRor8 = 0x128, kDppRowRor12 = 0x12C;
constexpr int kDppHalfMirror = 0x141, kDppQuad1032 = 0xB1, kDppQuad2301 = 0x4E;
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum of the four per-lane partial scores p[0..3] over a 16-lane row.  Lanes s and s ^ 8
// trade a pair of heads (s < 8 keeps heads 0, 1), then s and s ^ 7 a single head (bit 2
// of s picks the odd one), then the quad adds its four lanes: every lane of quad s / 4
// ends with the whole row sum of head s / 4.
__device__ __forceinline__ float row_scores4(const float p[4], bool hi, bool b2) {
  const float a0 = (hi ? p[2] : p[0]) + dpp_f<kDppRowRor8>(hi ? p[0] : p[2]);
  const float a1 = (hi ? p[3] : p[1]) + dpp_f<kDppRowRor8>(hi ? p[1] : p[3]);
  float v = (b2 ? a1 : a0) + dpp_f<kDppHalfMirror>(b2 ? a0 : a1);
  v += dpp_f<kDppQuad1032>(v);
  v += dpp_f<kDppQuad2301>(v);
  return v;
}

template <int D, int C, bool WIDE>
__global__ __launch_bounds__(kGW * 64) void attn_group_kernel(AttnArgs a, const float* __restrict__ rope, int wpl) {
  constexpr int NG = D / C;       // groups per head
  constexpr int HALF = D / 2;
  constexpr int NCH = D / 8;      // 16-byte chunks per codeword row in LDS
  static_assert(D == 128 && HALF == 64 && NCH * 16 == 256, "the grouped kernel is compiled for d = 128");
  static_assert(kGroupHeads == 4 && kGroupQuad == 4, "four heads per KV head, four waves per range");
  extern __shared__ __align__(16) unsigned char smem[];
  _Float16* kl = (_Float16*)smem;                                   // K, V slices [256][D/8][8]
  float* phbuf = (float*)(smem + (size_t)2 * kCodes * D * 2);       // [kGW][2][kGPh]
  int* ptbuf = (int*)(phbuf + kGW * 2 * kGPh);                      // [kGW][kPtBatch]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // block = kw * H + h: the workgroups of a KV head share its codebook slices
  const int h = blockIdx.x % a.H, kw = blockIdx.x / a.H;
  const int beta = a.t / a.Tc, tau = a.t % a.Tc;
  const int nblk = a.T / a.Tc;
  const int W4 = wpl * (kGW / kGroupQuad);                // ranges (quads) on this KV head
  const int quad = kw * (kGW / kGroupQuad) + (wave >> 2);
  const int member = wave & 3;

  const int b_first = min(lane, a.B - 1);
  const int len_first = a.seq_len[b_first];
  const int qe_first = a.q_end[b_first];
  SliceStage<D, C> slices;
  slices.load(a, beta, h, tau);
  int total = 0, n_first = 0, incl_first = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int b = b0 + lane;
    const int n = b < a.B ? (b0 == 0 ? seq_tiles_of(a, len_first, qe_first) : seq_tiles(a, b)).total : 0;
    const int incl = total + wave_incl_scan(n);
    if (b0 == 0) { n_first = n; incl_first = incl; }
    if (h == 0 && quad == 0 && member == 0 && b < a.B) a.tile_start[b] = incl - n;
    total += wave_sum_i(n);
  }
  if (h == 0 && quad == 0 && member == 0 && lane == 0) a.tile_start[a.B] = total;
  total = __builtin_amdgcn_readfirstlane(total);
  const int w_lo = __builtin_amdgcn_readfirstlane(range_lo(quad, total, W4));
  const int w_hi = __builtin_amdgcn_readfirstlane(range_lo(quad + 1, total, W4));
  int b = 0, tb = 0;
  if (w_lo < w_hi) {
    int base = 0;
    for (int b0 = 0; b0 < a.B; b0 += 64) {
      const int bb = b0 + lane;
      const int n = b0 == 0 ? n_first : (bb < a.B ? seq_tiles(a, bb).total : 0);
      const int incl = b0 == 0 ? incl_first : base + wave_incl_scan(n);
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

  slices.store(kl);
  __syncthreads();
  if (w_lo == w_hi) return;

  const int s = lane & 15, r = lane >> 4;
  const int toff = 4 * member + r;          // in-tile offset of this lane's tokens
  const bool hi = (s & 8) != 0, b2 = (s & 4) != 0;
  const int hsel = s >> 2;                  // the head whose score, maximum and sum the lane keeps
  // heads whose weights the three row rotations bring (row_ror n moves lane i's value
  // to lane i + n of the row): the output sums of head src[k] sit in o[k]
  int src[4];
  src[0] = hsel;
  src[1] = __builtin_amdgcn_mov_dpp(hsel, kDppRowRor4, 0xF, 0xF, true);
  src[2] = __builtin_amdgcn_mov_dpp(hsel, kDppRowRor8, 0xF, 0xF, true);
  src[3] = __builtin_amdgcn_mov_dpp(hsel, kDppRowRor12, 0xF, 0xF, true);
  // the groups of the lane's codes: low key channels 4s.., high key channels d/2 + 4s..,
  // value channels 8s..
  const int g_lo = (4 * s) / C, g_hi = (HALF + 4 * s) / C, g_v = (8 * s) / C;
  const int r8 = toff & 7;
  const size_t row_stride = (size_t)kPage * NG;
  const size_t page_bytes = (size_t)nblk * a.H * 2 * row_stride;
  const uint8_t* head_rows = a.index_pages + (((size_t)beta * a.H + h) * 2) * row_stride;
  uint32_t o_kl = r8 * NG + (g_lo & ~3), o_kh = r8 * NG + (g_hi & ~3),
           o_v = (uint32_t)row_stride + r8 * NG + (g_v & ~3);
  asm volatile("" : "+v"(o_kl), "+v"(o_kh), "+v"(o_v));
  // gather address by one byte permute: byte 0 the offset in the code row, byte 1 the code
  // from its index word, byte 2 the slice (0 keys, 1 values at 64 KB)
  auto code_sel = [](int g) -> uint32_t { return 0x0c020000u | ((4u + (uint32_t)(g & 3)) << 8); };
  const uint32_t sel_lo = code_sel(g_lo), sel_hi = code_sel(g_hi), sel_v = code_sel(g_v);
  const uint32_t off_lo = (uint32_t)(s >> 1) * 16 + (uint32_t)(s & 1) * 8;   // chunk s/2, half s%2
  const uint32_t off_v = (uint32_t)(kCodes * D * 2) + (uint32_t)s * 16;      // chunk s of the values
  constexpr uint32_t kHighOff = (HALF / 8) * 16;
  float* ph = phbuf + wave * 2 * kGPh;
  int* ptl = ptbuf + wave * kPtBatch;

  int pos_t = w_lo;
  while (pos_t < w_hi && b < a.B) {
    const SeqTiles st = seq_tiles(a, b);
    const int u_lo = pos_t - tb, u_hi = min(w_hi - tb, st.total);
    if (u_lo < u_hi) {
      const int L = max(min(a.seq_len[b], a.max_seq_len), 0);
      const int qe = max(min(a.q_end[b] & ~7, L), 0);
      const int ns = min(a.n_sink, L);
      const int r0 = max(qe, a.n_sink);
      const int vt_lo = r0 / kTile;
      // F, G: each head's query, rotated to its position (log2 units), turned back by the
      // lane's in-tile offset, for the lane's four pairs
      float F[4][4], Gc[4][4];
      {
        const f32x4 e1a = *(const f32x4*)(rope + (size_t)(a.rope_tiles + toff) * D + 8 * s);
        const f32x4 e1b = *(const f32x4*)(rope + (size_t)(a.rope_tiles + toff) * D + 8 * s + 4);
        const int pq = min(max(a.pos[b], 0), a.rope_tiles * kTile - 1);
        const float2 cs = phase(rope, a.rope_tiles, D, pq, lane);   // pair `lane` (64 pairs)
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
          const uint16_t* qv = a.q + ((size_t)b * a.Hq + h * 4 + hh) * D;
          const float x = bf2f(qv[lane]), y = bf2f(qv[lane + HALF]);
          ph[2 * lane] = (x * cs.x - y * cs.y) * a.scale_log2e;
          ph[2 * lane + 1] = (y * cs.x + x * cs.y) * a.scale_log2e;
          const f32x4 qa = *(const f32x4*)(ph + 8 * s);
          const f32x4 qb = *(const f32x4*)(ph + 8 * s + 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float A = i < 2 ? qa[2 * i] : qb[2 * i - 4], Bq = i < 2 ? qa[2 * i + 1] : qb[2 * i - 3];
            const float c1 = i < 2 ? e1a[2 * i] : e1b[2 * i - 4], s1 = i < 2 ? e1a[2 * i + 1] : e1b[2 * i - 3];
            F[hh][i] = A * c1 + Bq * s1;
            Gc[hh][i] = Bq * c1 - A * s1;
          }
        }
      }
      float m = kNoMax, l = 0.f;
      float m_hi = kNoMax + kRescale;
      float o[4][8];
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int c = 0; c < 8; ++c) o[k][c] = 0.f;
      // one token per row: the lane's rotated key pairs (x, y) give its four partial
      // scores; the row sum, the head's lazy maximum and the weights of the four heads
      auto weights = [&](const float x[4], const float y[4], bool valid, float wr[4]) {
        float ps[4];
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
          float acc = F[hh][0] * x[0];
          acc = fmaf(Gc[hh][0], y[0], acc);
#pragma unroll
          for (int i = 1; i < 4; ++i) {
            acc = fmaf(F[hh][i], x[i], acc);
            acc = fmaf(Gc[hh][i], y[i], acc);
          }
          ps[hh] = acc;
        }
        // (the row sum runs in every lane: the DPP moves read the other lanes of the row)
        const float rs = row_scores4(ps, hi, b2);
        const float sc = valid ? rs : -__builtin_inff();
        if (__any(sc > m_hi)) {
          // the head's maximum over the wave's four rows (every lane of a quad holds the
          // same score)
          float mx = fmaxf(sc, __shfl_xor(sc, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          const float mn = fmaxf(m, mx);
          const float f = __builtin_amdgcn_exp2f(m - mn);
          l *= f;
          m = mn;
          m_hi = mn + kRescale;
          const float fr[4] = {f, dpp_f<kDppRowRor4>(f), dpp_f<kDppRowRor8>(f), dpp_f<kDppRowRor12>(f)};
#pragma unroll
          for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int c = 0; c < 8; ++c) o[k][c] *= fr[k];
        }
        const float w = __builtin_amdgcn_exp2f(sc - m);   // 0 for an invalid token
        l += w;
        wr[0] = w;
        wr[1] = dpp_f<kDppRowRor4>(w);
        wr[2] = dpp_f<kDppRowRor8>(w);
        wr[3] = dpp_f<kDppRowRor12>(w);
      };
      const int P_lo = 2 * u_lo;
      const int P_hi = min(2 * min(u_hi, st.coded), qe >> 3);
      const int* pt = a.page_table + (size_t)b * a.max_pages;
      int pt_base = -kPtBatch;
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
      struct TileIn {
        int phys;
        uint32_t kwl, kwh, vw;
        float2 e0;
      };
      auto fetch = [&](int P0) -> TileIn {
        TileIn in;
        if (P0 + 1 >= pt_base + kPtBatch) stage_pt(P0);
        in.phys = P0 < P_hi ? ptl[P0 - pt_base + (toff >> 3)] : -1;
        if constexpr (WIDE) {
          const uint8_t* base = head_rows + (size_t)(uint32_t)max(in.phys, 0) * page_bytes;
          in.kwl = *(const uint32_t*)(base + o_kl);
          in.kwh = *(const uint32_t*)(base + o_kh);
          in.vw = *(const uint32_t*)(base + o_v);
        } else {
          const uint32_t po = __umul24((uint32_t)max(in.phys, 0), (uint32_t)page_bytes);
          in.kwl = *(const uint32_t*)(head_rows + (po + o_kl));
          in.kwh = *(const uint32_t*)(head_rows + (po + o_kh));
          in.vw = *(const uint32_t*)(head_rows + (po + o_v));
        }
        const int tile_idx = min((8 * P0) / kTile, a.rope_tiles - 1);
        in.e0 = *(const float2*)((const char*)rope + (uint32_t)(4 * (tile_idx * D + 2 * lane)));
        return in;
      };
      auto tile = [&](int P0, const TileIn& in, int buf) {
        float* er = ph + buf * kGPh;
        *(float2*)(er + 2 * lane) = in.e0;
        const int p = 8 * P0 + toff;
        const bool valid = in.phys >= 0 && p >= a.n_sink;
        const f16x4 klo = lds_read8(__builtin_amdgcn_perm(in.kwl, off_lo, sel_lo));
        const f16x4 khi = lds_read8(__builtin_amdgcn_perm(in.kwh, off_lo, sel_hi) + kHighOff);
        const f32x4 ea = *(const f32x4*)(er + 8 * s);
        const f32x4 eb = *(const f32x4*)(er + 8 * s + 4);
        float x[4], y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float c0 = i < 2 ? ea[2 * i] : eb[2 * i - 4], s0 = i < 2 ? ea[2 * i + 1] : eb[2 * i - 3];
          x[i] = fmaf(c0, (float)klo[i], -(s0 * (float)khi[i]));
          y[i] = fmaf(s0, (float)klo[i], c0 * (float)khi[i]);
        }
        float wr[4];
        weights(x, y, valid, wr);
        const f16x8 v = lds_read16(__builtin_amdgcn_perm(in.vw, off_v, sel_v));
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int c = 0; c < 8; ++c) o[k][c] = fmaf(wr[k], (float)v[c], o[k][c]);
      };
      if (P_lo < P_hi) {
        TileIn in0 = fetch(P_lo);
        for (int P0 = P_lo;; P0 += 4) {
          const TileIn in1 = fetch(P0 + 2);
          tile(P0, in0, 0);
          if (P0 + 2 >= P_hi) break;
          in0 = fetch(P0 + 4);
          tile(P0 + 2, in1, 1);
          if (P0 + 4 >= P_hi) break;
        }
      }
      // bf16 sink and recent tiles, in float32
      const int vt_first = (max(u_lo, st.coded) - st.coded + kBfCost - 1) / kBfCost;
      const int vt_end = u_hi > st.coded ? (u_hi - st.coded + kBfCost - 1) / kBfCost : 0;
      for (int vt = vt_first; vt < vt_end; ++vt) {
        const bool sink_tile = ns > 0 && vt == 0;
        const int a_tile = sink_tile ? 0 : vt_lo + vt - (ns > 0 ? 1 : 0);
        const int lo = sink_tile ? 0 : r0, hi_p = sink_tile ? ns : L;
        const int p = kTile * a_tile + toff;
        const uint16_t* krow = nullptr;
        if (p >= lo && p < hi_p) {
          const int slot = sink_tile ? 0 : 1 + (p >> 3) - (qe >> 3);
          const int pg = slot < a.bf16_row ? a.bf16_table[(size_t)b * a.bf16_row + slot] : -1;
          if (pg >= 0 && pg < a.n_bf16_pages)
            krow = a.bf16_pages + (((((size_t)pg * a.T + a.t) * a.H + h) * 2) * kPage + (p & 7)) * D;
        }
        const bool valid = krow != nullptr;
        float* er = ph;
        {
          const int tile_idx = min(a_tile, a.rope_tiles - 1);
          *(float2*)(er + 2 * lane) = *(const float2*)(rope + (size_t)tile_idx * D + 2 * lane);
        }
        u16x4 klo = {0, 0, 0, 0}, khi = {0, 0, 0, 0};
        if (valid) {
          klo = *(const u16x4*)(krow + 4 * s);
          khi = *(const u16x4*)(krow + HALF + 4 * s);
        }
        const f32x4 ea = *(const f32x4*)(er + 8 * s);
        const f32x4 eb = *(const f32x4*)(er + 8 * s + 4);
        float x[4], y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float c0 = i < 2 ? ea[2 * i] : eb[2 * i - 4], s0 = i < 2 ? ea[2 * i + 1] : eb[2 * i - 3];
          const float kx = bf2f(klo[i]), ky = bf2f(khi[i]);
          x[i] = c0 * kx - s0 * ky;
          y[i] = s0 * kx + c0 * ky;
        }
        float wr[4];
        weights(x, y, valid, wr);
        if (valid) {
          const u16x8 v = *(const u16x8*)(krow + (size_t)kPage * D + 8 * s);
#pragma unroll
          for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int c = 0; c < 8; ++c) o[k][c] = fmaf(wr[k], bf2f(v[c]), o[k][c]);
        }
      }
      // head hh's sums are o[k] with src[k] == hh; then the sums over the four rows
      float oh[4][8];
#pragma unroll
      for (int hh = 0; hh < 4; ++hh)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float val = o[0][c];
#pragma unroll
          for (int k = 1; k < 4; ++k) val = src[k] == hh ? o[k][c] : val;
          oh[hh][c] = src[0] == hh ? o[0][c] : val;
        }
#pragma unroll
      for (int hh = 0; hh < 4; ++hh)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          oh[hh][c] += __shfl_xor(oh[hh][c], 16);
          oh[hh][c] += __shfl_xor(oh[hh][c], 32);
        }
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      float* rec = a.part + ((size_t)h * a.n_rec + (size_t)(quad + b) * kGroupQuad + member) * (4 * (D + 2));
      if (r == 0) {
#pragma unroll
        for (int hh = 0; hh < 4; ++hh)
#pragma unroll
          for (int c = 0; c < 8; c += 2)
            *(float2*)(rec + hh * (D + 2) + 2 + 8 * s + c) = make_float2(oh[hh][c], oh[hh][c + 1]);
        if ((s & 3) == 0) *(float2*)(rec + hsel * (D + 2)) = make_float2(m, l);
      }
    }
    pos_t = __builtin_amdgcn_readfirstlane(tb + u_hi);
    tb = __builtin_amdgcn_readfirstlane(tb + st.total);
    b = __builtin_amdgcn_readfirstlane(b + 1);
  }
}

// ------------------------------------------------------------------ merge
// One workgroup per (b, hq).  The split partials (m_i, l_i, o_i) are in log2 units:
// m = max m_i, l = sum l_i 2^(m_i - m), out = sum o_i 2^(m_i - m) / l,
// lse = (m + log2 l) ln 2.  The (m_i, l_i) pairs are read in one round into LDS and the
// weights computed there; then each (channel, record group) thread sums its records.
// The records of an item are those of the waves whose token-balanced ranges meet
// sequence b's units in the item's work list: record wg + b of the list for wg in a
// window found from the unit counts, each checked (a wave with an empty intersection
// wrote nothing there).  Decode (merge_rows = 0): item b * Hq + hq, list hq, one row per
// record.  Multi-row (merge_rows = 1): item (b * NQ + i) * Hq + hq, list = (KV head,
// block of 16 rows), records hold 16 rows.  Grouped decode (merge_rows = 2): item
// b * Hq + hq, list = KV head, records hold the Hq / H heads of the KV head, and the
// ranges belong to quads of waves: quad Q's four waves write records 4 (Q + b) + m.
constexpr int kMergeMax = 4096;   // candidate records per (b, hq) at most (the host checks)
constexpr int kMergeThreads = 512;
// THREADS threads per item, each record group's first PRE records loaded with the (m, l)
// pairs: 512 / 8 where an item has few records, 1024 / 32 where one sequence spans many
// waves (up to 256 records in the first round of loads at d = 128, so an item of a single
// sequence over a whole launch of 16 query heads is merged in one round).
template <int THREADS, int PRE>
__global__ __launch_bounds__(THREADS) void merge_kernel(AttnArgs a, int cap) {
  extern __shared__ __align__(16) unsigned char merge_smem[];
  float2* sml = (float2*)merge_smem;            // [cap]
  float* s_w = (float*)(sml + cap);             // [cap]
  __shared__ float s_ml[2];
  __shared__ float s_part[THREADS];             // per (record group, channel) sums
  const int item = blockIdx.x;           // b * Hq + hq
  const int D2 = a.d + 2;
  const int tid = threadIdx.x;
  int b, list, row = 0, rec_rows = 1, rg = 1;   // rg: records per range
  const int* ts = a.tile_start;
  if (a.merge_rows == 2) {
    b = item / a.Hq;
    const int hq = item % a.Hq, g = a.Hq / a.H;
    list = hq / g;
    row = hq % g;
    rec_rows = g;
    rg = kGroupQuad;
  } else if (a.merge_rows) {
    const int hq = item % a.Hq, bi = item / a.Hq;
    b = bi / a.NQ;
    const int g = a.Hq / a.H;
    const int r_abs = (bi % a.NQ) * g + hq % g;
    list = (hq / g) * a.n_rb + r_abs / 16;
    row = r_abs % 16;
    rec_rows = 16;
    ts += (size_t)(r_abs / 16) * (a.B + 1);
  } else {
    b = item / a.Hq;
    list = item % a.Hq;
  }
  const int tb = ts[b], tb1 = ts[b + 1], total = ts[a.B];
  const int W = a.n_waves / rg;   // ranges in the list
  int lo = 0, hi = -1;
  if (tb < tb1) {   // then total > 0
    lo = max(0, (int)(((long)(tb + 1) * W + total - 1) / total) - 2);
    hi = min(W - 1, (int)(((long)tb1 * W + total - 1) / total));
  }
  const int S = min((hi - lo + 1) * rg, cap);   // (hi - lo + 1) * rg <= (W + 1) * rg = cap
  const size_t rstride = (size_t)rec_rows * D2;   // between consecutive records of a list
  const float* rec = a.part + (((size_t)list * a.n_rec + (size_t)(lo + b) * rg) * rec_rows + row) * D2;
  for (int i = tid; i < S; i += blockDim.x) {
    const int wg = lo + i / rg;
    const bool meets = max(range_lo(wg, total, W), tb) < min(range_lo(wg + 1, total, W), tb1);
    sml[i] = meets ? *(const float2*)(rec + (size_t)i * rstride) : make_float2(-__builtin_inff(), 0.f);
  }
  // Thread (group, channel): record group g takes records g, g + NGR, ...  Its first PRE
  // records' values are loaded now, so their latency overlaps that of the (m, l) pairs.
  // Every slot below S exists in the list; a record with weight 0 (possibly never
  // written, so holding anything) is discarded by a select, never multiplied.
  const int NGR = THREADS / a.d;
  const int ch = tid % a.d, g = tid / a.d;
  float pre[PRE];
#pragma unroll
  for (int u = 0; u < PRE; ++u) {
    const int i = g + u * NGR;
    pre[u] = (g < NGR && i < S) ? rec[(size_t)i * rstride + 2 + ch] : 0.f;
  }
  __syncthreads();
  if (tid < 64) {
    float mloc = -__builtin_inff();
    for (int i = tid; i < S; i += 64) mloc = sml[i].y > 0.f ? fmaxf(mloc, sml[i].x) : mloc;
    const float M = wave_max(mloc);
    float lloc = 0.f;
    for (int i = tid; i < S; i += 64) {
      const float w = sml[i].y > 0.f ? __builtin_amdgcn_exp2f(sml[i].x - M) : 0.f;
      s_w[i] = w;
      lloc = fmaf(sml[i].y, w, lloc);
    }
    const float Ls = wave_sum(lloc);
    if (tid == 0) { s_ml[0] = M; s_ml[1] = Ls; }
  }
  __syncthreads();
  const float M = s_ml[0], Ls = s_ml[1];
  // Record group g sums its records with 8 loads in flight (the first PRE preloaded);
  // the groups are then added in order.  Beyond the first PRE, records with weight 0 are
  // not read.
  float acc = 0.f;
  if (g < NGR) {
    float p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) p[u] = 0.f;
#pragma unroll
    for (int u = 0; u < PRE; ++u) {
      const int i = g + u * NGR;
      const float w = i < S ? s_w[i] : 0.f;
      p[u % 8] = w != 0.f ? fmaf(pre[u], w, p[u % 8]) : p[u % 8];
    }
    int i = g + PRE * NGR;
    for (; i + 7 * NGR < S; i += 8 * NGR) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = s_w[i + u * NGR];
        const float o = w != 0.f ? rec[(size_t)(i + u * NGR) * rstride + 2 + ch] : 0.f;
        p[u] = fmaf(o, w, p[u]);
      }
    }
    for (; i < S; i += NGR)
      if (s_w[i] != 0.f) p[0] = fmaf(rec[(size_t)i * rstride + 2 + ch], s_w[i], p[0]);
    acc = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  }
  s_part[tid] = acc;
  __syncthreads();
  if (tid < a.d) {
    float sum = 0.f;
    for (int k = 0; k < NGR; ++k) sum += s_part[k * a.d + tid];
    a.out[(size_t)item * a.d + tid] = Ls > 0.f ? sum / Ls : 0.f;
  }
  if (a.lse && tid == 0) a.lse[item] = Ls > 0.f ? (M + __log2f(Ls)) * kLn2 : -__builtin_inff();
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

template <int D, int C, bool SCORES, bool WIDE>
hipError_t launch_attn_t(const AttnArgs& a, hipStream_t s) {
  constexpr size_t lds = lds_bytes<D>();
  static std::atomic<uint64_t> attr_set{0};
  hipError_t ea = once_per_device(attr_set, [&] {
    return hipFuncSetAttribute((const void*)attn_kernel<D, C, SCORES, WIDE>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  });
  if (ea != hipSuccess) return ea;
  const int n_items = a.B * a.Hq;
  const int wph = a.n_waves / kNW;   // workgroups per query head
  if (wph < 1 || a.n_waves % kNW || a.n_waves + 1 > kMergeMax || a.n_rec != a.n_waves + a.B || !a.tile_start)
    return hipErrorInvalidValue;
  const long grid = (long)wph * a.Hq;
  hipLaunchKernelGGL((attn_kernel<D, C, SCORES, WIDE>), dim3((unsigned)grid), dim3(kNW * 64), lds, s, a,
                     a.rope, wph);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // records per item: the waves over one sequence's share of the list, plus one
  const bool many = a.n_waves / (a.B > 0 ? a.B : 1) + 1 > 8 * (kMergeThreads / D);
  if (many)
    hipLaunchKernelGGL((merge_kernel<2 * kMergeThreads, 32>), dim3(n_items), dim3(2 * kMergeThreads),
                       (size_t)(a.n_waves + 1) * 12, s, a, a.n_waves + 1);
  else
    hipLaunchKernelGGL((merge_kernel<kMergeThreads, 8>), dim3(n_items), dim3(kMergeThreads),
                       (size_t)(a.n_waves + 1) * 12, s, a, a.n_waves + 1);
  return hipGetLastError();
}

template <int D, int C>
hipError_t launch_attn_s(const AttnArgs& a, hipStream_t s) {
  // 32-bit index-pool offsets when every page starts below 4 GiB and ids fit 24 bits
  const uint64_t page_bytes = (uint64_t)(a.T / a.Tc) * a.H * 2 * kPage * (D / C);
  const bool wide = (uint64_t)a.n_index_pages * page_bytes > 0xFFFFFFFFull || a.n_index_pages > (1 << 24) ||
                    page_bytes >= (1u << 24);
  if (a.scores) return wide ? launch_attn_t<D, C, true, true>(a, s) : launch_attn_t<D, C, true, false>(a, s);
  return wide ? launch_attn_t<D, C, false, true>(a, s) : launch_attn_t<D, C, false, false>(a, s);
}

}  // namespace

int rope_tile() { return kTile; }

int attn_waves_per_group() { return kNW; }

int merge_max_records() { return kMergeMax; }

bool attn_supported(int d, int c) {
  if (d == 128) return c == 8 || c == 16 || c == 32;
  if (d == 64) return c == 8 || c == 16;
  return false;
}

hipError_t launch_merge(const AttnArgs& a, hipStream_t s) {
  if (a.n_waves + 1 > kMergeMax || !a.tile_start || a.d > kMergeThreads || kMergeThreads % a.d) return hipErrorInvalidValue;
  const int items = a.B * (a.merge_rows ? a.NQ : 1) * a.Hq;
  hipLaunchKernelGGL((merge_kernel<kMergeThreads, 8>), dim3(items), dim3(kMergeThreads),
                     (size_t)(a.n_waves + 1) * 12, s, a, a.n_waves + 1);
  return hipGetLastError();
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

namespace {

template <int D, int C, bool WIDE>
hipError_t launch_attn_group_t(const AttnArgs& a, hipStream_t s) {
  constexpr size_t lds = group_lds_bytes<D>();
  static std::atomic<uint64_t> attr_set{0};
  hipError_t ea = once_per_device(attr_set, [&] {
    return hipFuncSetAttribute((const void*)attn_group_kernel<D, C, WIDE>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  });
  if (ea != hipSuccess) return ea;
  const int wpl = a.n_waves / kGW;   // workgroups per KV head
  const int ranges = a.n_waves / kGroupQuad;
  if (wpl < 1 || a.n_waves % kGW || (ranges + 1) * kGroupQuad > kMergeMax ||
      a.n_rec != a.n_waves + kGroupQuad * a.B || !a.tile_start || a.Hq != kGroupHeads * a.H || a.d != D)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_group_kernel<D, C, WIDE>), dim3((unsigned)(wpl * a.H)), dim3(kGW * 64), lds, s, a,
                     a.rope, wpl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  AttnArgs m = a;
  m.merge_rows = 2;
  const int cap = (ranges + 1) * kGroupQuad;
  const bool many = (ranges / (a.B > 0 ? a.B : 1) + 2) * kGroupQuad > 8 * (kMergeThreads / D);
  if (many)
    hipLaunchKernelGGL((merge_kernel<2 * kMergeThreads, 32>), dim3(a.B * a.Hq), dim3(2 * kMergeThreads),
                       (size_t)cap * 12, s, m, cap);
  else
    hipLaunchKernelGGL((merge_kernel<kMergeThreads, 8>), dim3(a.B * a.Hq), dim3(kMergeThreads),
                       (size_t)cap * 12, s, m, cap);
  return hipGetLastError();
}

}  // namespace

bool attn_group_supported(int d, int c) { return d == 128 && (c == 8 || c == 16 || c == 32); }

int attn_group_waves_per_group() { return kGW; }

hipError_t launch_attn_group(const AttnArgs& a, hipStream_t s) {
  const int c = a.G / a.Tc;
  if (a.d != 128 || !attn_group_supported(a.d, c)) return hipErrorInvalidValue;
  const uint64_t page_bytes = (uint64_t)(a.T / a.Tc) * a.H * 2 * kPage * (128 / c);
  const bool wide = (uint64_t)a.n_index_pages * page_bytes > 0xFFFFFFFFull || a.n_index_pages > (1 << 24) ||
                    page_bytes >= (1u << 24);
  if (c == 8) return wide ? launch_attn_group_t<128, 8, true>(a, s) : launch_attn_group_t<128, 8, false>(a, s);
  if (c == 16) return wide ? launch_attn_group_t<128, 16, true>(a, s) : launch_attn_group_t<128, 16, false>(a, s);
  return wide ? launch_attn_group_t<128, 32, true>(a, s) : launch_attn_group_t<128, 32, false>(a, s);
}

hipError_t launch_rope_tables(int ntile, int d, double base, float* tab, hipStream_t s) {
  const int n = (ntile + kTile) * (d / 2);
  hipLaunchKernelGGL(rope_kernel, dim3((n + 255) / 256), dim3(256), 0, s, ntile, d, base, tab);
  return hipGetLastError();
}

}  // namespace lvq
