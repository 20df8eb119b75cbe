// C ABI of the LoopVQ hot path: argument validation, split planning and
// dispatch to the HIP kernels.  Nothing here allocates device memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <string>

#include "lvq_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return LVQ_OK;
}

}  // namespace

namespace lvq {
int set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}
}  // namespace lvq

namespace {

int device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(LVQ_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Shape rules shared by the encoder and the decoder (Tc | T, Tc | G, c | d).
int check_code_shape(int T, int Tc, int G, int d) {
  if (T <= 0 || Tc <= 0 || G <= 0 || d <= 0)
    return fail(LVQ_EINVAL, "T=%d Tc=%d G=%d d=%d must be positive", T, Tc, G, d);
  if (T % Tc || G % Tc) return fail(LVQ_EINVAL, "Tc=%d must divide T=%d and G=%d", Tc, T, G);
  if (d % (G / Tc)) return fail(LVQ_EINVAL, "c=G/Tc=%d must divide d=%d", G / Tc, d);
  if (d % 2) return fail(LVQ_EINVAL, "d=%d must be even", d);
  return LVQ_OK;
}

struct SplitPlan {
  int n_waves;   // waves per query head (whole workgroups)
  int n_rec;     // partial records per query head: n_waves + B
};

constexpr int kComputeUnits = 256;   // MI355X: one resident decode workgroup per CU

// Token-balanced split: every query head's work list (the 16-token tiles of all the
// batch's sequences, coded and bf16) is cut into n_waves equal ranges, one per wave.
// Automatic sizing gives each head an equal share of the compute units (one workgroup
// each), but not more waves than about 4 tiles each of the largest possible work list.
// n_splits > 0 asks for that many waves per head (rounded up to whole workgroups).
SplitPlan plan_splits(const lvq_attn_shape& s) {
  const int w = lvq::attn_waves_per_group();
  const int max_wph = (lvq::merge_max_records() - 1) / w;
  int wph;
  if (s.n_splits > 0) {
    wph = (s.n_splits + w - 1) / w;
  } else {
    wph = kComputeUnits / s.Hq;
    const long tiles_bound = (long)s.B * ((s.max_seq_len + 15) / 16 + 3);
    const long by_work = (tiles_bound + 4L * w - 1) / (4L * w);
    if (wph > by_work) wph = (int)by_work;
  }
  if (wph < 1) wph = 1;
  if (wph > max_wph) wph = max_wph;
  SplitPlan p;
  p.n_waves = wph * w;
  p.n_rec = p.n_waves + s.B;
  return p;
}

int check_attn(const void* q, const void* page_table, const void* index_pages,
               const void* bf16_pages, const void* bf16_table, const void* codebooks, int t,
               const void* pos, const void* seq_len, const void* q_end, const void* rope_tab,
               const lvq_attn_shape* shp, const void* out) {
  if (!shp) return fail(LVQ_EINVAL, "shape is null");
  const lvq_attn_shape& s = *shp;
  if (!q || !page_table || !index_pages || !bf16_pages || !bf16_table || !codebooks || !pos ||
      !seq_len || !q_end || !rope_tab || !out)
    return fail(LVQ_EINVAL, "null pointer argument");
  if (s.B <= 0 || s.H <= 0 || s.Hq <= 0) return fail(LVQ_EINVAL, "B, H, Hq must be positive");
  if (s.Hq % s.H) return fail(LVQ_EINVAL, "Hq=%d must be a multiple of H=%d", s.Hq, s.H);
  int st = check_code_shape(s.T, s.Tc, s.G, s.d);
  if (st) return st;
  if (t < 0 || t >= s.T) return fail(LVQ_EINVAL, "t=%d outside [0, T=%d)", t, s.T);
  if (s.n_sink < 0 || s.n_sink > lvq::kPage) return fail(LVQ_EINVAL, "n_sink=%d outside [0, 8]", s.n_sink);
  if (s.max_seq_len <= 0) return fail(LVQ_EINVAL, "max_seq_len must be positive");
  if ((long)s.max_pages * lvq::kPage < s.max_seq_len)
    return fail(LVQ_EINVAL, "max_pages=%d too small for max_seq_len=%d", s.max_pages, s.max_seq_len);
  if (s.bf16_row < 1) return fail(LVQ_EINVAL, "bf16_row must be >= 1");
  // an all-bf16 cache still passes a coded pool of at least one page: a zero-page pool
  // would make every coded token's page id out of range, and those tokens are skipped
  if (s.n_index_pages <= 0 || s.n_bf16_pages <= 0) return fail(LVQ_EINVAL, "pool sizes must be positive");
  if (s.rope_max_len <= s.max_seq_len)
    return fail(LVQ_EINVAL, "rope_max_len=%d must exceed max_seq_len=%d", s.rope_max_len, s.max_seq_len);
  if (!(s.scale >= 0.f) || isinf(s.scale)) return fail(LVQ_EINVAL, "scale must be finite and >= 0");
  if (!lvq::attn_supported(s.d, s.G / s.Tc))
    return fail(LVQ_EUNSUPPORTED, "decode shape d=%d c=%d not compiled (d=128: c in {8,16,32}; d=64: c in {8,16})",
                s.d, s.G / s.Tc);
  return LVQ_OK;
}

// ------------------------------------------------------------------ multi-row attention
struct RowsPlan {
  int n_rb;      // row blocks of 16 per KV head
  int n_waves;   // waves per (KV head, row block) work list
  int n_rec;     // records per list and row: n_waves + B
};

// Token-balanced split of the multi-row kernel: each (KV head, row block) work list
// (every sequence's 16-key tiles) is cut into n_waves equal ranges.  Automatic sizing
// gives each list an equal share of the compute units (one workgroup of 8 waves each),
// but not more waves than about 4 tiles each of the largest possible list.
RowsPlan plan_rows(const lvq_rows_shape& s) {
  RowsPlan p;
  const int g = s.Hq / s.H;
  p.n_rb = (s.NQ * g + 15) / 16;
  const int w = lvq::rows_waves_per_group();
  const int lists = s.H * p.n_rb;
  const int max_wph = (lvq::merge_max_records() - 1) / w;
  int wph;
  if (s.n_splits > 0) {
    wph = (s.n_splits + w - 1) / w;
  } else {
    wph = kComputeUnits / lists;
    const long tiles_bound = (long)s.B * ((s.max_prefix + 15) / 16 + 3 + (s.NQ + 15) / 16);
    const long by_work = (tiles_bound + 4L * w - 1) / (4L * w);
    if (wph > by_work) wph = (int)by_work;
  }
  if (wph < 1) wph = 1;
  if (wph > max_wph) wph = max_wph;
  p.n_waves = wph * w;
  p.n_rec = p.n_waves + s.B;
  return p;
}

int check_rows(const void* q, const void* k_new, const void* v_new, const void* page_table,
               const void* index_pages, const void* bf16_pages, const void* bf16_table,
               const void* codebooks, int t, const void* pos, const void* prefix_len,
               const void* q_end, const void* rope_tab, const lvq_rows_shape* shp, const void* out) {
  if (!shp) return fail(LVQ_EINVAL, "shape is null");
  const lvq_rows_shape& s = *shp;
  if (!q || !page_table || !index_pages || !bf16_pages || !bf16_table || !codebooks || !pos ||
      !prefix_len || !q_end || !rope_tab || !out)
    return fail(LVQ_EINVAL, "null pointer argument");
  if (!k_new != !v_new) return fail(LVQ_EINVAL, "k_new and v_new must both be given or both be null");
  if (s.B <= 0 || s.NQ <= 0 || s.H <= 0 || s.Hq <= 0) return fail(LVQ_EINVAL, "B, NQ, H, Hq must be positive");
  if (s.Hq % s.H) return fail(LVQ_EINVAL, "Hq=%d must be a multiple of H=%d", s.Hq, s.H);
  int st = check_code_shape(s.T, s.Tc, s.G, s.d);
  if (st) return st;
  if (t < 0 || t >= s.T) return fail(LVQ_EINVAL, "t=%d outside [0, T=%d)", t, s.T);
  if (s.n_sink < 0 || s.n_sink > lvq::kPage) return fail(LVQ_EINVAL, "n_sink=%d outside [0, 8]", s.n_sink);
  if (s.max_prefix < 0) return fail(LVQ_EINVAL, "max_prefix must be >= 0");
  if ((long)s.max_pages * lvq::kPage < s.max_prefix)
    return fail(LVQ_EINVAL, "max_pages=%d too small for max_prefix=%d", s.max_pages, s.max_prefix);
  if (s.bf16_row < 1) return fail(LVQ_EINVAL, "bf16_row must be >= 1");
  // an all-bf16 cache still passes a coded pool of at least one page: a zero-page pool
  // would make every coded token's page id out of range, and those tokens are skipped
  if (s.n_index_pages <= 0 || s.n_bf16_pages <= 0) return fail(LVQ_EINVAL, "pool sizes must be positive");
  if ((long)s.rope_max_len < (long)s.max_prefix + s.NQ)
    return fail(LVQ_EINVAL, "rope_max_len=%d below max_prefix + NQ = %ld", s.rope_max_len, (long)s.max_prefix + s.NQ);
  if (!(s.scale >= 0.f) || isinf(s.scale)) return fail(LVQ_EINVAL, "scale must be finite and >= 0");
  if (!lvq::rows_supported(s.d, s.G / s.Tc))
    return fail(LVQ_EUNSUPPORTED, "multi-row shape d=%d c=%d not compiled (d=128, c in {8,16,32})", s.d, s.G / s.Tc);
  return LVQ_OK;
}

size_t rows_workspace(const lvq_rows_shape& s) {
  const RowsPlan p = plan_rows(s);
  // records [H * n_rb][n_rec][16 rows][d + 2], then the row blocks' first units [n_rb][B + 1]
  return (size_t)s.H * p.n_rb * p.n_rec * 16 * (s.d + 2) * sizeof(float) +
         (size_t)p.n_rb * (s.B + 1) * sizeof(int);
}

// Decode with 8 or more query heads per KV head runs on the multi-row kernel (one key
// rebuild for all the heads, scores and values on the matrix cores); at 2 and 4 the
// grouped kernel below is the faster.
constexpr int kRowsMinGroup = 8;

bool decode_on_rows(const lvq_attn_shape& s) {
  return s.Hq / s.H >= kRowsMinGroup && lvq::rows_supported(s.d, s.G / s.Tc);
}

// Decode with 2 or 4 query heads per KV head (d = 128) runs on the grouped kernel: the
// heads share each key's dequantisation and rotation.  lvq_decode_scores keeps the
// per-head kernel (it writes per-head scores).
int group_heads(const lvq_attn_shape& s) { return s.H > 0 && s.Hq % s.H == 0 ? s.Hq / s.H : 0; }

bool decode_on_group(const lvq_attn_shape& s) {
  return !decode_on_rows(s) && group_heads(s) > 1 && lvq::attn_group_supported(s.d, s.G / s.Tc, group_heads(s));
}

// Token-balanced split of a KV head's work list over quads of waves: automatic sizing
// gives each KV head an equal share of the compute units (one workgroup each), but not
// more quads than about 4 tiles each of the largest possible work list.  n_splits > 0
// asks for that many waves per KV head (rounded up to whole workgroups).
SplitPlan plan_group_splits(const lvq_attn_shape& s) {
  const int w = lvq::attn_group_waves_per_group();
  const int quads_per_wg = w / lvq::kGroupQuad;
  const int max_wpl = (lvq::merge_max_records() / lvq::kGroupQuad - 1) / quads_per_wg;
  int wpl;
  if (s.n_splits > 0) {
    wpl = (s.n_splits + w - 1) / w;
  } else {
    wpl = kComputeUnits / s.H;
    const long tiles_bound = (long)s.B * ((s.max_seq_len + 15) / 16 + 3);
    const long by_work = (tiles_bound + 4L * quads_per_wg - 1) / (4L * quads_per_wg);
    if (wpl > by_work) wpl = (int)by_work;
  }
  if (wpl < 1) wpl = 1;
  if (wpl > max_wpl) wpl = max_wpl;
  SplitPlan p;
  p.n_waves = wpl * w;
  p.n_rec = p.n_waves + lvq::kGroupQuad * s.B;
  return p;
}

size_t group_workspace(const lvq_attn_shape& s) {
  const SplitPlan p = plan_group_splits(s);
  // records [H][n_rec][Hq / H rows][d + 2], then the sequences' first tiles [B + 1]
  return (size_t)s.H * p.n_rec * group_heads(s) * (s.d + 2) * sizeof(float) + (size_t)(s.B + 1) * sizeof(int);
}

lvq_rows_shape rows_shape_of(const lvq_attn_shape& s) {
  lvq_rows_shape r{};
  r.B = s.B; r.NQ = 1; r.H = s.H; r.Hq = s.Hq; r.d = s.d; r.T = s.T; r.Tc = s.Tc; r.G = s.G;
  r.n_sink = s.n_sink; r.max_pages = s.max_pages; r.bf16_row = s.bf16_row;
  r.n_index_pages = s.n_index_pages; r.n_bf16_pages = s.n_bf16_pages;
  r.max_prefix = s.max_seq_len; r.rope_max_len = s.rope_max_len; r.n_splits = s.n_splits; r.scale = s.scale;
  r.rejected = s.rejected;
  return r;
}

size_t workspace_bytes(const lvq_attn_shape& s) {
  const SplitPlan p = plan_splits(s);
  // partial records [Hq][n_rec][d + 2], then the sequences' first tiles [B + 1]
  const size_t dec = (size_t)s.Hq * p.n_rec * (s.d + 2) * sizeof(float) + (size_t)(s.B + 1) * sizeof(int);
  if (decode_on_group(s)) {
    const size_t grp = group_workspace(s);
    return grp > dec ? grp : dec;
  }
  if (!decode_on_rows(s)) return dec;
  const size_t rows = rows_workspace(rows_shape_of(s));
  return rows > dec ? rows : dec;
}

int run_attn(const uint16_t* q, const int32_t* page_table, const uint8_t* index_pages,
             const uint16_t* bf16_pages, const int32_t* bf16_table, const uint16_t* codebooks,
             int t, const int32_t* pos, const int32_t* seq_len, const int32_t* q_end,
             const float* rope_tab, const lvq_attn_shape* shp, float* out, float* lse,
             float* scores, void* ws, size_t ws_bytes, void* stream) {
  int st = check_attn(q, page_table, index_pages, bf16_pages, bf16_table, codebooks, t, pos,
                      seq_len, q_end, rope_tab, shp, out);
  if (st) return st;
  const lvq_attn_shape& s = *shp;
  const size_t need = workspace_bytes(s);
  if (!ws || ws_bytes < need)
    return fail(LVQ_ENOSPC, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
  if (!scores && decode_on_rows(s)) {
    // the same attention with the query heads of a KV head as the rows (NQ = 1, no chunk)
    const lvq_rows_shape rs = rows_shape_of(s);
    return lvq_rows_attn(q, nullptr, nullptr, page_table, index_pages, bf16_pages, bf16_table, codebooks, t,
                         pos, seq_len, q_end, rope_tab, &rs, out, lse, ws, ws_bytes, stream);
  }
  const bool group = !scores && decode_on_group(s);
  const SplitPlan p = group ? plan_group_splits(s) : plan_splits(s);
  lvq::AttnArgs a{};
  a.q = q;
  a.page_table = page_table;
  a.index_pages = index_pages;
  a.bf16_pages = bf16_pages;
  a.bf16_table = bf16_table;
  a.codebooks = codebooks;
  a.pos = pos;
  a.seq_len = seq_len;
  a.q_end = q_end;
  a.rope = rope_tab;
  a.part = (float*)ws;
  a.out = out;
  a.lse = lse;
  a.scores = scores;
  a.rejected = s.rejected;
  a.t = t;
  a.B = s.B;
  a.H = s.H;
  a.Hq = s.Hq;
  a.d = s.d;
  a.T = s.T;
  a.Tc = s.Tc;
  a.G = s.G;
  a.n_sink = s.n_sink;
  a.max_pages = s.max_pages;
  a.bf16_row = s.bf16_row;
  a.n_index_pages = s.n_index_pages;
  a.n_bf16_pages = s.n_bf16_pages;
  a.max_seq_len = s.max_seq_len;
  a.rope_tiles = (s.rope_max_len + lvq::rope_tile() - 1) / lvq::rope_tile();
  a.n_waves = p.n_waves;
  a.n_rec = p.n_rec;
  const size_t rec_floats = group ? (size_t)s.H * p.n_rec * group_heads(s) * (s.d + 2)
                                  : (size_t)s.Hq * p.n_rec * (s.d + 2);
  a.tile_start = (int*)((char*)ws + rec_floats * sizeof(float));
  const float scale = s.scale > 0.f ? s.scale : 1.0f / sqrtf((float)s.d);
  a.scale_log2e = scale * 1.4426950408889634f;
  if (group) return device_status(lvq::launch_attn_group(a, (hipStream_t)stream), "lvq_decode_attn launch");
  return device_status(lvq::launch_attn(a, (hipStream_t)stream), "lvq_decode_attn launch");
}

int check_encode_common(const void* kv, const void* codebooks, int T, int Tc, int G, int N,
                        int H, int d) {
  if (!kv || !codebooks) return fail(LVQ_EINVAL, "null pointer argument");
  int st = check_code_shape(T, Tc, G, d);
  if (st) return st;
  if (N < 0 || H <= 0) return fail(LVQ_EINVAL, "N=%d must be >= 0 and H=%d > 0", N, H);
  if (!lvq::encode_supported(G, G / Tc, d))
    return fail(LVQ_EUNSUPPORTED, "encode shape G=%d c=%d d=%d not compiled", G, G / Tc, d);
  return LVQ_OK;
}

int cache_args(const lvq_cache* c, lvq::CacheArgs& a) {
  if (!c) return fail(LVQ_EINVAL, "null pointer argument");
  if (c->B <= 0 || c->max_pages <= 0 || c->n_index_pages <= 0 || c->n_bf16_pages <= 0)
    return fail(LVQ_EINVAL, "B, max_pages and pool sizes must be positive");
  if (c->n_sink < 0 || c->n_sink > lvq::kPage) return fail(LVQ_EINVAL, "n_sink=%d outside [0, 8]", c->n_sink);
  if (c->n_recent < 0) return fail(LVQ_EINVAL, "n_recent=%d must be >= 0", c->n_recent);
  const int need_row = 1 + (c->n_recent + 2 * lvq::kPage - 1) / lvq::kPage;
  if (c->bf16_row < need_row)
    return fail(LVQ_EINVAL, "bf16_row=%d below %d for n_recent=%d", c->bf16_row, need_row, c->n_recent);
  if (!c->page_table || !c->bf16_table || !c->seq_len || !c->q_end || !c->index_free || !c->bf16_free ||
      !c->counters || !c->re_src || !c->re_dst)
    return fail(LVQ_EINVAL, "null pointer in lvq_cache");
  a.B = c->B;
  a.max_pages = c->max_pages;
  a.bf16_row = c->bf16_row;
  a.n_sink = c->n_sink;
  a.n_recent = c->n_recent;
  a.n_index_pages = c->n_index_pages;
  a.n_bf16_pages = c->n_bf16_pages;
  a.page_table = c->page_table;
  a.bf16_table = c->bf16_table;
  a.seq_len = c->seq_len;
  a.q_end = c->q_end;
  a.index_free = c->index_free;
  a.bf16_free = c->bf16_free;
  a.counters = c->counters;
  a.re_src = c->re_src;
  a.re_dst = c->re_dst;
  return LVQ_OK;
}

int token_copy(const uint16_t* k, const uint16_t* v, int T, int H, int d, uint16_t* pool,
               lvq::TokenCopy& tc) {
  if (!k || !v || !pool) return fail(LVQ_EINVAL, "null pointer argument");
  if (T <= 0 || H <= 0 || d <= 0 || d % 8)
    return fail(LVQ_EINVAL, "T=%d H=%d d=%d: positive, d a multiple of 8", T, H, d);
  tc.k = k;
  tc.v = v;
  tc.pool = pool;
  tc.T = T;
  tc.H = H;
  tc.d = d;
  return LVQ_OK;
}

}  // namespace

extern "C" {

int lvq_version(void) { return LVQ_ABI_VERSION; }

const char* lvq_last_error(void) { return g_err.c_str(); }

int lvq_encode(const uint16_t* kv, const uint16_t* codebooks, int kv_sel, int T, int Tc, int G,
               int N, int H, int d, uint8_t* idx, void* stream) {
  int st = check_encode_common(kv, codebooks, T, Tc, G, N, H, d);
  if (st) return st;
  if (!idx) return fail(LVQ_EINVAL, "null pointer argument");
  if (kv_sel != 0 && kv_sel != 1) return fail(LVQ_EINVAL, "kv_sel=%d must be 0 or 1", kv_sel);
  if (N == 0) return ok();
  lvq::EncodeArgs a{};
  a.src = kv;
  a.codebooks = codebooks;
  a.out = idx;
  a.src_mode = lvq::kSrcDense;
  a.dst_mode = lvq::kDstDense;
  a.kv_sel = kv_sel;
  a.T = T; a.Tc = Tc; a.G = G; a.N = N; a.H = H; a.d = d;
  a.tokens_per_block = 512;
  return device_status(lvq::launch_encode(a, (hipStream_t)stream), "lvq_encode launch");
}

int lvq_encode_pages(const uint16_t* kv, const uint16_t* codebooks, int kv_sel, int T, int Tc,
                     int G, int N, int H, int d, const int32_t* chunk_page, int n_index_pages,
                     uint8_t* index_pages, void* stream) {
  int st = check_encode_common(kv, codebooks, T, Tc, G, N, H, d);
  if (st) return st;
  if (!index_pages || (N > 0 && !chunk_page)) return fail(LVQ_EINVAL, "null pointer argument");
  if (kv_sel != 0 && kv_sel != 1) return fail(LVQ_EINVAL, "kv_sel=%d must be 0 or 1", kv_sel);
  if (N % lvq::kPage) return fail(LVQ_EINVAL, "N=%d must be a multiple of 8", N);
  if (n_index_pages < 0) return fail(LVQ_EINVAL, "n_index_pages must be >= 0");
  if (N == 0) return ok();
  lvq::EncodeArgs a{};
  a.src = kv;
  a.codebooks = codebooks;
  a.out = index_pages;
  a.dst_pages = chunk_page;
  a.src_mode = lvq::kSrcDense;
  a.dst_mode = lvq::kDstPages;
  a.kv_sel = kv_sel;
  a.T = T; a.Tc = Tc; a.G = G; a.N = N; a.H = H; a.d = d;
  a.n_dst_pages = n_index_pages;
  a.tokens_per_block = 512;
  return device_status(lvq::launch_encode(a, (hipStream_t)stream), "lvq_encode_pages launch");
}

int lvq_reencode_pages(const uint16_t* bf16_pages, const int32_t* src_pages,
                       const int32_t* dst_pages, int n, const uint16_t* codebooks, int T, int Tc,
                       int G, int H, int d, int n_bf16_pages, int n_index_pages,
                       uint8_t* index_pages, void* stream) {
  if (n < 0) return fail(LVQ_EINVAL, "n=%d must be >= 0", n);
  int st = check_encode_common(bf16_pages, codebooks, T, Tc, G, lvq::kPage * n, H, d);
  if (st) return st;
  if (!index_pages || (n > 0 && (!src_pages || !dst_pages))) return fail(LVQ_EINVAL, "null pointer argument");
  if (n_bf16_pages < 0 || n_index_pages < 0) return fail(LVQ_EINVAL, "pool sizes must be >= 0");
  if (n == 0) return ok();
  lvq::EncodeArgs a{};
  a.src = bf16_pages;
  a.src_pages = src_pages;
  a.codebooks = codebooks;
  a.out = index_pages;
  a.dst_pages = dst_pages;
  a.src_mode = lvq::kSrcPages;
  a.dst_mode = lvq::kDstPages;
  a.kv_sel = -1;
  a.T = T; a.Tc = Tc; a.G = G; a.N = lvq::kPage * n; a.H = H; a.d = d;
  a.n_src_pages = n_bf16_pages;
  a.n_dst_pages = n_index_pages;
  a.tokens_per_block = 512;
  return device_status(lvq::launch_encode(a, (hipStream_t)stream), "lvq_reencode_pages launch");
}

int lvq_reencode_pages_layers(const lvq_reencode_layer* layers, int n_layers,
                              const int32_t* src_pages, const int32_t* dst_pages, int n, int T,
                              int Tc, int G, int H, int d, void* stream) {
  if (n < 0 || n_layers < 0) return fail(LVQ_EINVAL, "n=%d and n_layers=%d must be >= 0", n, n_layers);
  if (n_layers > 0 && !layers) return fail(LVQ_EINVAL, "null layer array");
  for (int l = 0; l < n_layers; ++l) {
    const lvq_reencode_layer& L = layers[l];
    int st = check_encode_common(L.bf16_pages, L.codebooks, T, Tc, G, lvq::kPage * n, H, d);
    if (st) return st;
    if (!L.index_pages) return fail(LVQ_EINVAL, "layer %d: null index_pages", l);
    if (L.n_bf16_pages < 0 || L.n_index_pages < 0)
      return fail(LVQ_EINVAL, "layer %d: pool sizes must be >= 0", l);
  }
  if (n > 0 && n_layers > 0 && (!src_pages || !dst_pages)) return fail(LVQ_EINVAL, "null pointer argument");
  if (n == 0 || n_layers == 0) return ok();
  lvq::EncodeArgs a{};
  a.src_pages = src_pages;
  a.dst_pages = dst_pages;
  a.src_mode = lvq::kSrcPages;
  a.dst_mode = lvq::kDstPages;
  a.kv_sel = -1;
  a.T = T; a.Tc = Tc; a.G = G; a.N = lvq::kPage * n; a.H = H; a.d = d;
  a.tokens_per_block = 512;
  // The layer table travels as a kernel argument, so larger models take several launches.
  for (int l0 = 0; l0 < n_layers; l0 += lvq::kMaxReencodeLayers) {
    lvq::ReencodeLayers tab{};
    tab.n = std::min(lvq::kMaxReencodeLayers, n_layers - l0);
    for (int i = 0; i < tab.n; ++i) {
      const lvq_reencode_layer& L = layers[l0 + i];
      tab.layer[i] = {L.bf16_pages, L.codebooks, L.index_pages, L.n_bf16_pages, L.n_index_pages};
    }
    a.src = tab.layer[0].bf16_pages;
    a.codebooks = tab.layer[0].codebooks;
    a.out = tab.layer[0].index_pages;
    int st = device_status(lvq::launch_encode(a, (hipStream_t)stream, &tab),
                           "lvq_reencode_pages_layers launch");
    if (st) return st;
  }
  return ok();
}

size_t lvq_build_codebooks_workspace_bytes(int T, int Tc, int G, int S, int H, int d) {
  if (T <= 0 || Tc <= 0 || G <= 0 || S <= 0 || H <= 0 || d <= 0) return 0;
  if (T % Tc || G % Tc || d % (G / Tc)) return 0;
  const size_t nblk = (size_t)(T / Tc), ng = (size_t)(d / (G / Tc));
  const size_t centers = nblk * H * ng * lvq::kCodes * (size_t)G * sizeof(double);
  const size_t assign = nblk * (size_t)S * H * ng;
  // centers (256-byte aligned), assignments, and above the LDS seeding limit one float64
  // D^2 per (book, sample) after the assignments (256-byte aligned)
  const size_t head = (centers + 255) / 256 * 256;
  if (S <= lvq::kMaxKmeansSamplesLds) return head + assign;
  return head + (assign + 255) / 256 * 256 + nblk * H * ng * (size_t)((S + 31) / 32 * 32) * sizeof(double);
}

int lvq_build_codebooks(const uint16_t* samples, const double* draws, const double* weights,
                        int kv_sel, int T, int Tc, int G, int S, int H, int d, int n_iter,
                        uint16_t* codebooks, void* ws, size_t ws_bytes, void* stream) {
  int st = check_encode_common(samples, codebooks, T, Tc, G, S, H, d);
  if (st) return st;
  if (!draws) return fail(LVQ_EINVAL, "null pointer argument");
  if (kv_sel != 0 && kv_sel != 1) return fail(LVQ_EINVAL, "kv_sel=%d must be 0 or 1", kv_sel);
  if (S < 1) return fail(LVQ_EINVAL, "S=%d samples: at least one is needed", S);
  if (S > lvq::kMaxKmeansSamples)
    return fail(LVQ_EUNSUPPORTED, "S=%d samples per book above the supported %d", S, lvq::kMaxKmeansSamples);
  if (n_iter < 0 || n_iter > 1000) return fail(LVQ_EINVAL, "n_iter=%d outside [0, 1000]", n_iter);
  const size_t need = lvq_build_codebooks_workspace_bytes(T, Tc, G, S, H, d);
  if (!ws || ws_bytes < need)
    return fail(LVQ_ENOSPC, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
  lvq::KmeansArgs a{};
  a.samples = samples;
  a.draws = draws;
  a.weights = weights;
  a.codebooks = codebooks;
  a.kv_sel = kv_sel;
  a.T = T; a.Tc = Tc; a.G = G; a.S = S; a.H = H; a.d = d;
  a.n_iter = n_iter;
  a.n_books = (T / Tc) * H * (d / (G / Tc));
  const size_t centers = (size_t)a.n_books * lvq::kCodes * G * sizeof(double);
  a.centers = (double*)ws;
  a.assign = (uint8_t*)ws + (centers + 255) / 256 * 256;
  const size_t assign = (size_t)(T / Tc) * S * H * (d / (G / Tc));
  a.d2 = S > lvq::kMaxKmeansSamplesLds ? (double*)(a.assign + (assign + 255) / 256 * 256) : nullptr;
  return device_status(lvq::launch_build_codebooks(a, (hipStream_t)stream), "lvq_build_codebooks launch");
}

size_t lvq_rope_table_bytes(int max_len, int d) {
  if (max_len <= 0 || d <= 0 || d % 2) return 0;
  const size_t tile = (size_t)lvq::rope_tile();
  const size_t ntile = ((size_t)max_len + tile - 1) / tile;
  return (ntile + tile) * (size_t)(d / 2) * 2 * sizeof(float) + (size_t)(d / 2) * sizeof(double);
}

int lvq_rope_tables(int max_len, int d, double base, float* rope_tab, size_t rope_bytes,
                    void* stream) {
  if (!rope_tab) return fail(LVQ_EINVAL, "null pointer argument");
  if (max_len <= 0 || d <= 0 || d % 2) return fail(LVQ_EINVAL, "max_len=%d d=%d invalid", max_len, d);
  if (!(base > 1.0) || isinf(base)) return fail(LVQ_EINVAL, "base must be finite and > 1");
  const size_t need = lvq_rope_table_bytes(max_len, d);
  if (rope_bytes < need) return fail(LVQ_ENOSPC, "rope table needs %zu bytes, %zu given", need, rope_bytes);
  const int tile = lvq::rope_tile();
  return device_status(lvq::launch_rope_tables((max_len + tile - 1) / tile, d, base, rope_tab, (hipStream_t)stream),
                       "lvq_rope_tables launch");
}

int lvq_cache_min_bf16_row(int n_recent) {
  if (n_recent < 0) return 0;
  return 1 + (n_recent + 2 * lvq::kPage - 1) / lvq::kPage;
}

int lvq_cache_init(const lvq_cache* c, void* stream) {
  lvq::CacheArgs a;
  int st = cache_args(c, a);
  if (st) return st;
  return device_status(lvq::launch_cache_init(a, (hipStream_t)stream), "lvq_cache_init launch");
}

int lvq_cache_prefill(const lvq_cache* c, const int32_t* lengths, void* stream) {
  lvq::CacheArgs a;
  int st = cache_args(c, a);
  if (st) return st;
  if (!lengths) return fail(LVQ_EINVAL, "null pointer argument");
  return device_status(lvq::launch_cache_prefill(a, lengths, (hipStream_t)stream), "lvq_cache_prefill launch");
}

int lvq_cache_store_tokens(const lvq_cache* c, int b, int first, int n, const uint16_t* k,
                           const uint16_t* v, int T, int H, int d, uint16_t* bf16_pages,
                           void* stream) {
  lvq::CacheArgs a;
  int st = cache_args(c, a);
  if (st) return st;
  if (b < 0 || b >= c->B) return fail(LVQ_EINVAL, "sequence %d outside [0, %d)", b, c->B);
  if (first < 0 || n < 0) return fail(LVQ_EINVAL, "first=%d n=%d must be >= 0", first, n);
  if (n == 0) return ok();
  lvq::TokenCopy tc;
  st = token_copy(k, v, T, H, d, bf16_pages, tc);
  if (st) return st;
  return device_status(lvq::launch_cache_store(a, tc, b, first, n, (hipStream_t)stream),
                       "lvq_cache_store_tokens launch");
}

int lvq_cache_begin_token(const lvq_cache* c, void* stream) {
  lvq::CacheArgs a;
  int st = cache_args(c, a);
  if (st) return st;
  return device_status(lvq::launch_cache_step(a, 0, (hipStream_t)stream), "lvq_cache_begin_token launch");
}

int lvq_cache_append(const lvq_cache* c, int t0, int n_steps, const uint16_t* k,
                     const uint16_t* v, int T, int H, int d, uint16_t* bf16_pages, void* stream) {
  lvq::CacheArgs a;
  int st = cache_args(c, a);
  if (st) return st;
  if (n_steps < 1 || t0 < 0 || t0 + n_steps > T)
    return fail(LVQ_EINVAL, "steps [%d, %d) outside [0, T=%d)", t0, t0 + n_steps, T);
  lvq::TokenCopy tc;
  st = token_copy(k, v, T, H, d, bf16_pages, tc);
  if (st) return st;
  return device_status(lvq::launch_cache_append(a, tc, t0, n_steps, (hipStream_t)stream),
                       "lvq_cache_append launch");
}

int lvq_cache_end_token(const lvq_cache* c, void* stream) {
  lvq::CacheArgs a;
  int st = cache_args(c, a);
  if (st) return st;
  return device_status(lvq::launch_cache_step(a, 1, (hipStream_t)stream), "lvq_cache_end_token launch");
}

int lvq_cache_commit(const lvq_cache* c, void* stream) {
  lvq::CacheArgs a;
  int st = cache_args(c, a);
  if (st) return st;
  return device_status(lvq::launch_cache_step(a, 2, (hipStream_t)stream), "lvq_cache_commit launch");
}

int lvq_cache_release(const lvq_cache* c, const int32_t* mask, void* stream) {
  lvq::CacheArgs a;
  int st = cache_args(c, a);
  if (st) return st;
  if (!mask) return fail(LVQ_EINVAL, "null pointer argument");
  return device_status(lvq::launch_cache_release(a, mask, (hipStream_t)stream), "lvq_cache_release launch");
}

size_t lvq_rows_attn_workspace_bytes(const lvq_rows_shape* shp) {
  if (!shp || shp->B <= 0 || shp->NQ <= 0 || shp->H <= 0 || shp->Hq <= 0 || shp->d <= 0 || shp->Hq % shp->H ||
      shp->max_prefix < 0)
    return 0;
  return rows_workspace(*shp);
}

int lvq_rows_attn(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                  const int32_t* page_table, const uint8_t* index_pages, const uint16_t* bf16_pages,
                  const int32_t* bf16_table, const uint16_t* codebooks, int t, const int32_t* pos,
                  const int32_t* prefix_len, const int32_t* q_end, const float* rope_tab,
                  const lvq_rows_shape* shp, float* out, float* lse, void* ws, size_t ws_bytes,
                  void* stream) {
  int st = check_rows(q, k_new, v_new, page_table, index_pages, bf16_pages, bf16_table, codebooks, t, pos,
                      prefix_len, q_end, rope_tab, shp, out);
  if (st) return st;
  const lvq_rows_shape& s = *shp;
  const size_t need = rows_workspace(s);
  if (!ws || ws_bytes < need)
    return fail(LVQ_ENOSPC, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
  const RowsPlan p = plan_rows(s);
  lvq::RowsArgs a{};
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.page_table = page_table;
  a.index_pages = index_pages;
  a.bf16_pages = bf16_pages;
  a.bf16_table = bf16_table;
  a.codebooks = codebooks;
  a.pos = pos;
  a.prefix_len = prefix_len;
  a.q_end = q_end;
  a.rope = rope_tab;
  a.part = (float*)ws;
  a.rejected = s.rejected;
  a.t = t;
  a.B = s.B;
  a.NQ = s.NQ;
  a.H = s.H;
  a.Hq = s.Hq;
  a.d = s.d;
  a.T = s.T;
  a.Tc = s.Tc;
  a.G = s.G;
  a.n_sink = s.n_sink;
  a.max_pages = s.max_pages;
  a.bf16_row = s.bf16_row;
  a.n_index_pages = s.n_index_pages;
  a.n_bf16_pages = s.n_bf16_pages;
  a.max_prefix = s.max_prefix;
  a.rope_tiles = (s.rope_max_len + lvq::rope_tile() - 1) / lvq::rope_tile();
  a.n_rb = p.n_rb;
  a.n_waves = p.n_waves;
  a.n_rec = p.n_rec;
  a.tile_start = (int*)((char*)ws + (size_t)s.H * p.n_rb * p.n_rec * 16 * (s.d + 2) * sizeof(float));
  const float scale = s.scale > 0.f ? s.scale : 1.0f / sqrtf((float)s.d);
  a.scale_log2e = scale * 1.4426950408889634f;
  hipError_t e = lvq::launch_rows(a, (hipStream_t)stream);
  if (e != hipSuccess) return device_status(e, "lvq_rows_attn launch");
  lvq::AttnArgs m{};
  m.part = a.part;
  m.out = out;
  m.lse = lse;
  m.B = s.B;
  m.NQ = s.NQ;
  m.H = s.H;
  m.Hq = s.Hq;
  m.d = s.d;
  m.n_rb = p.n_rb;
  m.n_waves = p.n_waves;
  m.n_rec = p.n_rec;
  m.tile_start = a.tile_start;
  m.merge_rows = 1;
  return device_status(lvq::launch_merge(m, (hipStream_t)stream), "lvq_rows_attn merge launch");
}

size_t lvq_decode_attn_workspace_bytes(const lvq_attn_shape* shp) {
  if (!shp || shp->B <= 0 || shp->H <= 0 || shp->Hq <= 0 || shp->Hq % shp->H || shp->d <= 0 ||
      shp->max_seq_len <= 0 || shp->Tc <= 0 || shp->G <= 0)
    return 0;
  return workspace_bytes(*shp);
}

int lvq_decode_attn(const uint16_t* q, const int32_t* page_table, const uint8_t* index_pages,
                    const uint16_t* bf16_pages, const int32_t* bf16_table,
                    const uint16_t* codebooks, int t, const int32_t* pos, const int32_t* seq_len,
                    const int32_t* q_end, const float* rope_tab, const lvq_attn_shape* shp,
                    float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return run_attn(q, page_table, index_pages, bf16_pages, bf16_table, codebooks, t, pos, seq_len,
                  q_end, rope_tab, shp, out, lse, nullptr, ws, ws_bytes, stream);
}

int lvq_decode_scores(const uint16_t* q, const int32_t* page_table, const uint8_t* index_pages,
                      const uint16_t* bf16_pages, const int32_t* bf16_table,
                      const uint16_t* codebooks, int t, const int32_t* pos,
                      const int32_t* seq_len, const int32_t* q_end, const float* rope_tab,
                      const lvq_attn_shape* shp, float* out, float* lse, float* scores,
                      void* ws, size_t ws_bytes, void* stream) {
  if (!scores) return fail(LVQ_EINVAL, "null pointer argument");
  return run_attn(q, page_table, index_pages, bf16_pages, bf16_table, codebooks, t, pos, seq_len,
                  q_end, rope_tab, shp, out, lse, scores, ws, ws_bytes, stream);
}

}  // extern "C"
