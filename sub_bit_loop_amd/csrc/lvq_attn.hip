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
#include "lvq_attn_common.h"

namespace lvq {
namespace {

constexpr int kNW = 12;            // waves per workgroup
constexpr int kWavesPerSimd = 3;   // occupancy the register budget is sized for

// Tile-phase buffer (floats): the d/2 pairs in 4 quarter blocks of d/8 pairs, each
// block followed by 16 bytes of padding so the four quarters read distinct LDS banks.
template <int D>
constexpr int phase_buf_floats() { return 4 * (2 * (D / 8) + 4); }

template <int D>
constexpr size_t lds_bytes() {
  return (size_t)2 * kCodes * D * 2 + (size_t)kNW * (2 * phase_buf_floats<D>() * 4 + kPtBatch * 4);
}


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
  SliceStage<D, C, kNW * 64> slices;
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
          const bool in_pool = v[k] >= 0 && v[k] < a.n_index_pages;
          note_rejected(a.rejected, q < P_hi && !in_pool);
          ptl[k * 64 + lane] = (q < P_hi && in_pool) ? v[k] : -1;
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
          note_rejected(a.rejected, !(pg >= 0 && pg < a.n_bf16_pages));
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
  const int wph = a.n_waves / kNW;   // workgroups per query head
  if (wph < 1 || a.n_waves % kNW || a.n_waves + 1 > kMergeMax || a.n_rec != a.n_waves + a.B || !a.tile_start)
    return hipErrorInvalidValue;
  const long grid = (long)wph * a.Hq;
  hipLaunchKernelGGL((attn_kernel<D, C, SCORES, WIDE>), dim3((unsigned)grid), dim3(kNW * 64), lds, s, a,
                     a.rope, wph);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // records per item: the waves over one sequence's share of the list, plus one
  return launch_merge_records(a, a.n_waves + 1, a.n_waves / (a.B > 0 ? a.B : 1) + 1, s);
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

hipError_t launch_merge_records(const AttnArgs& m, int cap, int per_item, hipStream_t s) {
  if (cap > kMergeMax || !m.tile_start || m.d > kMergeThreads || kMergeThreads % m.d) return hipErrorInvalidValue;
  const int n_items = m.B * m.Hq;
  if (per_item > 8 * (kMergeThreads / m.d))
    hipLaunchKernelGGL((merge_kernel<2 * kMergeThreads, 32>), dim3(n_items), dim3(2 * kMergeThreads),
                       (size_t)cap * 12, s, m, cap);
  else
    hipLaunchKernelGGL((merge_kernel<kMergeThreads, 8>), dim3(n_items), dim3(kMergeThreads),
                       (size_t)cap * 12, s, m, cap);
  return hipGetLastError();
}

hipError_t launch_merge(const AttnArgs& a, hipStream_t s) {
  if (a.n_waves + 1 > kMergeMax || !a.tile_start || a.d > kMergeThreads || kMergeThreads % a.d) return hipErrorInvalidValue;
  const int items = a.B * (a.merge_rows ? a.NQ : 1) * a.Hq;
  // records an item meets: its sequence's share of the list's waves, plus two
  const int per_item = a.n_waves / (a.B > 0 ? a.B : 1) + 2;
  if (per_item > 8 * (kMergeThreads / a.d))
    hipLaunchKernelGGL((merge_kernel<2 * kMergeThreads, 32>), dim3(items), dim3(2 * kMergeThreads),
                       (size_t)(a.n_waves + 1) * 12, s, a, a.n_waves + 1);
  else
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

hipError_t launch_rope_tables(int ntile, int d, double base, float* tab, hipStream_t s) {
  const int n = (ntile + kTile) * (d / 2);
  hipLaunchKernelGGL(rope_kernel, dim3((n + 255) / 256), dim3(256), 0, s, ntile, d, base, tab);
  return hipGetLastError();
}

}  // namespace lvq
