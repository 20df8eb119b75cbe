// Grouped-query decode attention over the LoopVQ cache, gfx950 (the same attention as
// the per-head kernel in lvq_attn.hip: LoopVQ summary, onedev.kr/papers/1681, sections
// "전제와 한계" and "무엇과 다른가"; rit.work article, section "Когда LoopVQ меняет
// план развёртывания").
//
// QH query heads per KV head (2 or 4) share each key's dequantisation and tile
// rotation.  A quad of four waves covers the 16 positions of a tile: member m of the quad
// takes in-tile offsets 4m..4m+3, one per 16-lane row r (offset o = 4m + r), so a lane's
// offset never changes and its query coefficients F, G (QH heads x 4 channel pairs) are
// set once per sequence.  Lane s of a row owns channel pairs 4s..4s+3 of the score
// (channels 4s.. and d/2 + 4s..) and output channels 8s..8s+7 of the value sum, for all
// QH heads.  Per token the lane rotates its four key pairs by the tile phase E(16a) once
// (four mixed float16/float32 operations per pair) and forms the QH partial scores (two
// FMAs per pair and head); a transposing reduction over the row (lanes trading halves of
// their heads) leaves the score of head s / (16 / QH) in the 16 / QH lanes that keep that
// head's running maximum and sum, and QH - 1 DPP row rotations give every lane the QH
// weights for the value sum.  At QH = 4, about 7.2 wave instructions per (token, head)
// on the coded path against 9.6 for the per-head kernel.  The work list of a KV head is the same as a
// query head's; its ranges go to quads, and each wave of a quad writes its own partial
// record (QH rows, one per head) per sequence its range meets.  Four waves per SIMD
// (16-wave workgroups).  From 8 query heads per KV head the multi-row kernel, whose float16
// matrix-core products serve the heads as rows, is the faster one.
#include "lvq_attn_common.h"

namespace lvq {
namespace {
// waves per workgroup: four quads (four waves per SIMD)
constexpr int kGroupWaves = 16;
constexpr int kGPh = 128;   // floats per phase row: 64 pairs of (cos, sin)

template <int D, int NW>
constexpr size_t group_lds_bytes() {
  return (size_t)2 * kCodes * D * 2 + (size_t)NW * (2 * kGPh * 4 + kPtBatch * 4);
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef const f16x4 __attribute__((address_space(3)))* lds_f16x4_ptr;
__device__ __forceinline__ f16x4 lds_read8(uint32_t addr) { return *(lds_f16x4_ptr)(size_t)addr; }

// DPP lane moves within 16-lane rows (every lane of the wave active): row rotations by
// 4, 8 and 12 lanes, the half-row mirror and quad permutes
constexpr int kDppRowRor0 = 0x120;
constexpr int kDppRowRor8 = kDppRowRor0 + 8;
constexpr int kDppHalfMirror = 0x141, kDppQuad1032 = 0xB1, kDppQuad2301 = 0x4E;
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum of the QH per-lane partial scores p[] over a 16-lane row, by lanes trading halves
// of their heads: s and s ^ 8 (row rotation by 8) first, then (QH = 4) s and the
// half-row mirror of s (bit 2 differs), and the rest of the row by the half-row mirror
// or quad permutes.  Every lane ends with the whole row sum of head s / (16 / QH).
template <int QH>
__device__ __forceinline__ float row_scores(const float (&p)[QH], int s) {
  const bool hi = (s & 8) != 0, b2 = (s & 4) != 0;
  if constexpr (QH == 2) {
    float v = (hi ? p[1] : p[0]) + dpp_f<kDppRowRor8>(hi ? p[0] : p[1]);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppQuad2301>(v);
    v += dpp_f<kDppQuad1032>(v);
    return v;
  } else {
    static_assert(QH == 4, "2 or 4 query heads per KV head");
    const float a0 = (hi ? p[2] : p[0]) + dpp_f<kDppRowRor8>(hi ? p[0] : p[2]);
    const float a1 = (hi ? p[3] : p[1]) + dpp_f<kDppRowRor8>(hi ? p[1] : p[3]);
    float v = (b2 ? a1 : a0) + dpp_f<kDppHalfMirror>(b2 ? a0 : a1);
    v += dpp_f<kDppQuad1032>(v);
    v += dpp_f<kDppQuad2301>(v);
    return v;
  }
}

// out[k] = v of the lane 16 k / QH places back in the row (row rotation), k < QH: the
// value each head's lanes hold, spread to every lane
template <int QH>
__device__ __forceinline__ void row_spread(float v, float (&out)[QH]) {
  out[0] = v;
  if constexpr (QH == 2) {
    out[1] = dpp_f<kDppRowRor0 + 8>(v);
  } else {
    out[1] = dpp_f<kDppRowRor0 + 4>(v);
    out[2] = dpp_f<kDppRowRor0 + 8>(v);
    out[3] = dpp_f<kDppRowRor0 + 12>(v);
  }
}

template <int D, int C, int QH, bool WIDE>
__global__ __launch_bounds__(kGroupWaves * 64) void attn_group_kernel(AttnArgs a, const float* __restrict__ rope,
                                                                      int wpl) {
  constexpr int kGW = kGroupWaves;
  constexpr int LPH = 16 / QH;    // lanes of a row per head after the row sum
  constexpr int NG = D / C;       // groups per head
  constexpr int HALF = D / 2;
  constexpr int NCH = D / 8;      // 16-byte chunks per codeword row in LDS
  static_assert(D == 128 && HALF == 64 && NCH * 16 == 256, "the grouped kernel is compiled for d = 128");
  static_assert(kGroupQuad == 4 && (QH == 2 || QH == 4), "2 or 4 heads per KV head, four waves per range");
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
  __builtin_amdgcn_sched_barrier(0);   // keep the two length loads ahead of the slice loads
  SliceStage<D, C, kGW * 64> slices;
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
  const int hsel = s / LPH;                 // the head whose score, maximum and sum the lane keeps
  // heads whose weights the row rotations bring: the output sums of head src[k] sit in
  // o[k] (taken with the same moves, so nothing depends on the rotation's direction)
  int src[QH];
  {
    float sf[QH];
    row_spread<QH>(__int_as_float(hsel), sf);
#pragma unroll
    for (int k = 0; k < QH; ++k) src[k] = __float_as_int(sf[k]);
  }
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
      float F[QH][4], Gc[QH][4];
      {
        const f32x4 e1a = *(const f32x4*)(rope + (size_t)(a.rope_tiles + toff) * D + 8 * s);
        const f32x4 e1b = *(const f32x4*)(rope + (size_t)(a.rope_tiles + toff) * D + 8 * s + 4);
        const int pq = min(max(a.pos[b], 0), a.rope_tiles * kTile - 1);
        const float2 cs = phase(rope, a.rope_tiles, D, pq, lane);   // pair `lane` (64 pairs)
#pragma unroll
        for (int hh = 0; hh < QH; ++hh) {
          const uint16_t* qv = a.q + ((size_t)b * a.Hq + h * QH + hh) * D;
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
      float o[QH][8];
#pragma unroll
      for (int k = 0; k < QH; ++k)
#pragma unroll
        for (int c = 0; c < 8; ++c) o[k][c] = 0.f;
      // one token per row: the lane's rotated key pairs (x, y) give its four partial
      // scores; the row sum, the head's lazy maximum and the weights of the four heads
      auto weights = [&](const float x[4], const float y[4], bool valid, float (&wr)[QH]) {
        float ps[QH];
#pragma unroll
        for (int hh = 0; hh < QH; ++hh) {
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
        const float rs = row_scores<QH>(ps, s);
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
          float fr[QH];
          row_spread<QH>(f, fr);
#pragma unroll
          for (int k = 0; k < QH; ++k)
#pragma unroll
            for (int c = 0; c < 8; ++c) o[k][c] *= fr[k];
        }
        const float w = __builtin_amdgcn_exp2f(sc - m);   // 0 for an invalid token
        l += w;
        row_spread<QH>(w, wr);
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
          const bool in_pool = v[k] >= 0 && v[k] < a.n_index_pages;
          note_rejected(a.rejected, q < P_hi && !in_pool);
          ptl[k * 64 + lane] = (q < P_hi && in_pool) ? v[k] : -1;
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
        float wr[QH];
        weights(x, y, valid, wr);
        const f16x8 v = lds_read16(__builtin_amdgcn_perm(in.vw, off_v, sel_v));
#pragma unroll
        for (int k = 0; k < QH; ++k)
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
          note_rejected(a.rejected, !(pg >= 0 && pg < a.n_bf16_pages));
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
        float wr[QH];
        weights(x, y, valid, wr);
        if (valid) {
          const u16x8 v = *(const u16x8*)(krow + (size_t)kPage * D + 8 * s);
#pragma unroll
          for (int k = 0; k < QH; ++k)
#pragma unroll
            for (int c = 0; c < 8; ++c) o[k][c] = fmaf(wr[k], bf2f(v[c]), o[k][c]);
        }
      }
      // head hh's sums are o[k] with src[k] == hh; then the sums over the four rows
      float oh[QH][8];
#pragma unroll
      for (int hh = 0; hh < QH; ++hh)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float val = o[0][c];
#pragma unroll
          for (int k = 1; k < QH; ++k) val = src[k] == hh ? o[k][c] : val;
          oh[hh][c] = val;
        }
#pragma unroll
      for (int hh = 0; hh < QH; ++hh)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          oh[hh][c] += __shfl_xor(oh[hh][c], 16);
          oh[hh][c] += __shfl_xor(oh[hh][c], 32);
        }
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      float* rec = a.part + ((size_t)h * a.n_rec + (size_t)(quad + b) * kGroupQuad + member) * (QH * (D + 2));
      if (r == 0) {
#pragma unroll
        for (int hh = 0; hh < QH; ++hh)
#pragma unroll
          for (int c = 0; c < 8; c += 2)
            *(float2*)(rec + hh * (D + 2) + 2 + 8 * s + c) = make_float2(oh[hh][c], oh[hh][c + 1]);
        if (s % LPH == 0) *(float2*)(rec + hsel * (D + 2)) = make_float2(m, l);
      }
    }
    pos_t = __builtin_amdgcn_readfirstlane(tb + u_hi);
    tb = __builtin_amdgcn_readfirstlane(tb + st.total);
    b = __builtin_amdgcn_readfirstlane(b + 1);
  }
}

template <int D, int C, int QH, bool WIDE>
hipError_t launch_attn_group_t(const AttnArgs& a, hipStream_t s) {
  constexpr int kGW = kGroupWaves;
  constexpr size_t lds = group_lds_bytes<D, kGW>();
  static std::atomic<uint64_t> attr_set{0};
  hipError_t ea = once_per_device(attr_set, [&] {
    return hipFuncSetAttribute((const void*)attn_group_kernel<D, C, QH, WIDE>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  });
  if (ea != hipSuccess) return ea;
  const int wpl = a.n_waves / kGW;   // workgroups per KV head
  const int ranges = a.n_waves / kGroupQuad;
  if (wpl < 1 || a.n_waves % kGW || (ranges + 1) * kGroupQuad > merge_max_records() ||
      a.n_rec != a.n_waves + kGroupQuad * a.B || !a.tile_start || a.Hq != QH * a.H || a.d != D)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_group_kernel<D, C, QH, WIDE>), dim3((unsigned)(wpl * a.H)), dim3(kGW * 64), lds, s, a,
                     a.rope, wpl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  AttnArgs m = a;
  m.merge_rows = 2;
  // records per item: the quads over one sequence's share of the list, plus two, four each
  return launch_merge_records(m, (ranges + 1) * kGroupQuad, (ranges / (a.B > 0 ? a.B : 1) + 2) * kGroupQuad, s);
}

template <int QH>
hipError_t launch_group_heads(const AttnArgs& a, int c, bool wide, hipStream_t s) {
  if (c == 8) return wide ? launch_attn_group_t<128, 8, QH, true>(a, s) : launch_attn_group_t<128, 8, QH, false>(a, s);
  if (c == 16) return wide ? launch_attn_group_t<128, 16, QH, true>(a, s) : launch_attn_group_t<128, 16, QH, false>(a, s);
  return wide ? launch_attn_group_t<128, 32, QH, true>(a, s) : launch_attn_group_t<128, 32, QH, false>(a, s);
}

}  // namespace

bool attn_group_supported(int d, int c, int heads) {
  return d == 128 && (c == 8 || c == 16 || c == 32) && (heads == 2 || heads == 4);
}

int attn_group_waves_per_group() { return kGroupWaves; }

hipError_t launch_attn_group(const AttnArgs& a, hipStream_t s) {
  const int c = a.G / a.Tc;
  const int heads = a.H > 0 ? a.Hq / a.H : 0;
  if (a.H <= 0 || a.Hq % a.H || !attn_group_supported(a.d, c, heads)) return hipErrorInvalidValue;
  const uint64_t page_bytes = (uint64_t)(a.T / a.Tc) * a.H * 2 * kPage * (128 / c);
  const bool wide = (uint64_t)a.n_index_pages * page_bytes > 0xFFFFFFFFull || a.n_index_pages > (1 << 24) ||
                    page_bytes >= (1u << 24);
  if (heads == 2) return launch_group_heads<2>(a, c, wide, s);
  return launch_group_heads<4>(a, c, wide, s);
}

}  // namespace lvq
