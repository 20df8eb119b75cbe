// Host-side check of the C ABI layer (lvq_abi.cpp) with no GPU, built with AddressSanitizer
// and UndefinedBehaviorSanitizer (tests/test_abi_sanitized.py builds and runs it).
//
// The kernel launchers are replaced by stubs.  For every launch the ABI makes, a stub
// checks that each buffer the kernels would write lies inside the caller's workspace, at
// the place the workspace-size query accounted for, and that the split plan obeys the
// kernels' launch rules (waves in whole workgroups, records per list, merge capacity).
// The driver draws seeded random shapes for decode attention (every route: per head,
// grouped, multi-row), multi-row attention and the codebook builder, calls each entry
// point with exactly the reported workspace size (the launch must pass the checks) and
// with one byte less (it must be refused with LVQ_ENOSPC), plus a set of invalid shapes
// that must be refused without a launch.  Device pointers are host addresses that are
// never dereferenced: the ABI only checks them for null.
//
// Output: one line per drawn shape and reported size on stdout (so the test can compare
// the sizes with the real library's), then a summary; the exit status is the number of
// failed checks (capped at 100), 0 when all pass.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "lvq_internal.h"

namespace {

const char* g_ws = nullptr;
size_t g_ws_bytes = 0;
long g_launches = 0;
long g_failures = 0;

void failure(int line, const char* fmt, ...) {
  std::fprintf(stderr, "abi_host_check.cpp:%d: ", line);
  va_list ap;
  va_start(ap, fmt);
  std::vfprintf(stderr, fmt, ap);
  va_end(ap);
  std::fputc('\n', stderr);
  ++g_failures;
}
#define CHECK(cond, ...)                          \
  do {                                            \
    if (!(cond)) failure(__LINE__, __VA_ARGS__);  \
  } while (0)

// [p, p + bytes) inside the current workspace
bool inside(const void* p, size_t bytes) {
  const char* c = static_cast<const char*>(p);
  return g_ws && c >= g_ws && bytes <= g_ws_bytes && (size_t)(c - g_ws) <= g_ws_bytes - bytes;
}

}  // namespace

namespace lvq {

// The launch rules of the kernel sources (the same values; the test compares the
// workspace sizes this build reports with the real library's for every shape drawn).
bool encode_supported(int G, int c, int d) {
  if (d != 64 && d != 128) return false;
  if (G == 32) return c == 8 || c == 16 || c == 32;
  if (G == 16) return c == 4 || c == 8 || c == 16;
  return false;
}
bool attn_supported(int d, int c) {
  if (d == 128) return c == 8 || c == 16 || c == 32;
  if (d == 64) return c == 8 || c == 16;
  return false;
}
bool rows_supported(int d, int c) { return d == 128 && (c == 8 || c == 16 || c == 32); }
bool attn_group_supported(int d, int c, int heads) {
  return d == 128 && (c == 8 || c == 16 || c == 32) && (heads == 2 || heads == 4);
}
int attn_waves_per_group() { return 12; }
int attn_group_waves_per_group() { return 16; }
int rows_waves_per_group() { return 8; }
int merge_max_records() { return 4096; }
int rope_tile() { return 16; }

hipError_t launch_attn(const AttnArgs& a, hipStream_t) {
  ++g_launches;
  CHECK(a.n_waves > 0 && a.n_waves % 12 == 0, "per-head: n_waves %d not whole workgroups of 12", a.n_waves);
  CHECK(a.n_rec == a.n_waves + a.B, "per-head: n_rec %d != n_waves %d + B %d", a.n_rec, a.n_waves, a.B);
  CHECK(a.n_waves + 1 <= merge_max_records(), "per-head: %d waves beyond the merge's capacity", a.n_waves);
  const size_t rec = (size_t)a.Hq * a.n_rec * (a.d + 2) * sizeof(float);
  CHECK((const char*)a.part == g_ws, "per-head: records do not start the workspace");
  CHECK(inside(a.part, rec), "per-head: records [%d][%d][%d] outside the workspace", a.Hq, a.n_rec, a.d + 2);
  CHECK((const char*)a.tile_start == (const char*)a.part + rec, "per-head: tile_start does not follow the records");
  CHECK(inside(a.tile_start, (size_t)(a.B + 1) * sizeof(int)), "per-head: tile_start[%d] outside the workspace",
        a.B + 1);
  CHECK(a.rope_tiles * 16 >= a.max_seq_len, "per-head: rope table shorter than max_seq_len");
  return hipSuccess;
}

hipError_t launch_attn_group(const AttnArgs& a, hipStream_t) {
  ++g_launches;
  const int g = a.H > 0 ? a.Hq / a.H : 0;
  const int w = attn_group_waves_per_group();
  CHECK(a.H > 0 && a.Hq % a.H == 0 && (g == 2 || g == 4), "grouped: Hq %d over H %d", a.Hq, a.H);
  CHECK(a.n_waves > 0 && a.n_waves % w == 0, "grouped: n_waves %d not whole workgroups of %d", a.n_waves, w);
  CHECK(a.n_rec == a.n_waves + kGroupQuad * a.B, "grouped: n_rec %d != n_waves %d + 4 B", a.n_rec, a.n_waves);
  CHECK((a.n_waves / kGroupQuad + 1) * kGroupQuad <= merge_max_records(), "grouped: merge capacity");
  const size_t rec = (size_t)a.H * a.n_rec * g * (a.d + 2) * sizeof(float);
  CHECK((const char*)a.part == g_ws, "grouped: records do not start the workspace");
  CHECK(inside(a.part, rec), "grouped: records [%d][%d][%d][%d] outside the workspace", a.H, a.n_rec, g, a.d + 2);
  CHECK((const char*)a.tile_start == (const char*)a.part + rec, "grouped: tile_start does not follow the records");
  CHECK(inside(a.tile_start, (size_t)(a.B + 1) * sizeof(int)), "grouped: tile_start outside the workspace");
  CHECK(a.scores == nullptr, "grouped: a scores probe on the grouped route");
  return hipSuccess;
}

hipError_t launch_rows(const RowsArgs& a, hipStream_t) {
  ++g_launches;
  const int g = a.Hq / a.H;
  CHECK(a.n_waves > 0 && a.n_waves % 8 == 0, "rows: n_waves %d not whole workgroups of 8", a.n_waves);
  CHECK(a.n_rec == a.n_waves + a.B, "rows: n_rec %d != n_waves %d + B %d", a.n_rec, a.n_waves, a.B);
  CHECK(a.n_waves + 1 <= merge_max_records(), "rows: merge capacity");
  CHECK(a.n_rb * 16 >= a.NQ * g, "rows: %d row blocks for %d rows", a.n_rb, a.NQ * g);
  const size_t rec = (size_t)a.H * a.n_rb * a.n_rec * 16 * (a.d + 2) * sizeof(float);
  CHECK((const char*)a.part == g_ws, "rows: records do not start the workspace");
  CHECK(inside(a.part, rec), "rows: records outside the workspace");
  CHECK((const char*)a.tile_start == (const char*)a.part + rec, "rows: tile_start does not follow the records");
  CHECK(inside(a.tile_start, (size_t)a.n_rb * (a.B + 1) * sizeof(int)), "rows: tile_start outside the workspace");
  return hipSuccess;
}

hipError_t launch_merge(const AttnArgs& m, hipStream_t) {
  ++g_launches;
  CHECK(m.merge_rows == 1, "merge of multi-row records expected");
  CHECK(m.n_waves + 1 <= merge_max_records(), "merge capacity");
  CHECK(inside(m.tile_start, (size_t)m.n_rb * (m.B + 1) * sizeof(int)), "merge: tile_start outside the workspace");
  return hipSuccess;
}

hipError_t launch_build_codebooks(const KmeansArgs& a, hipStream_t) {
  ++g_launches;
  const int c = a.G / a.Tc, ng = a.d / c, nblk = a.T / a.Tc;
  CHECK(a.n_books == nblk * a.H * ng, "builder: %d books for %d x %d x %d", a.n_books, nblk, a.H, ng);
  CHECK((const char*)a.centers == g_ws, "builder: centers do not start the workspace");
  CHECK(inside(a.centers, (size_t)a.n_books * kCodes * a.G * sizeof(double)), "builder: centers outside");
  CHECK(inside(a.assign, (size_t)nblk * a.S * a.H * ng), "builder: assignments outside");
  CHECK((const char*)a.assign >= (const char*)(a.centers + (size_t)a.n_books * kCodes * a.G),
        "builder: assignments overlap the centers");
  if (a.S > kMaxKmeansSamplesLds) {
    const size_t s32 = ((size_t)a.S + 31) / 32 * 32;
    CHECK(a.d2 != nullptr && inside(a.d2, (size_t)a.n_books * s32 * sizeof(double)), "builder: D^2 outside");
    CHECK((const char*)a.d2 >= (const char*)a.assign + (size_t)nblk * a.S * a.H * ng,
          "builder: D^2 overlaps the assignments");
  } else {
    CHECK(a.d2 == nullptr, "builder: D^2 workspace below the LDS limit");
  }
  CHECK(a.S >= 256 && a.S <= kMaxKmeansSamples, "builder: S = %d", a.S);
  return hipSuccess;
}

// launches with no workspace: recorded only
hipError_t launch_encode(const EncodeArgs&, hipStream_t, const ReencodeLayers*) { ++g_launches; return hipSuccess; }
hipError_t launch_cache_init(const CacheArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_cache_prefill(const CacheArgs&, const int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_cache_step(const CacheArgs&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_cache_release(const CacheArgs&, const int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_cache_store(const CacheArgs&, const TokenCopy&, int, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_cache_append(const CacheArgs&, const TokenCopy&, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_rope_tables(int, int, double, float*, hipStream_t) { return hipSuccess; }

}  // namespace lvq

// The one runtime function the ABI layer calls (only to format a failed launch).
const char* hipGetErrorString(hipError_t) { return "host check: no device"; }

namespace {

unsigned char g_fake[64];   // stands for every device pointer: non-null, never read
const void* dev() { return g_fake; }

// A workspace of `bytes`: host memory up to 64 MiB (so the sanitizer sees it), above that
// an address range nothing maps (the ABI never dereferences it; the stubs check ranges).
struct Workspace {
  std::vector<char> mem;
  char* base;
  explicit Workspace(size_t bytes) {
    if (bytes <= ((size_t)64 << 20)) {
      mem.resize(bytes);
      base = mem.data();
    } else {
      base = reinterpret_cast<char*>((uintptr_t)1 << 44);
    }
  }
};

struct Rng {
  std::mt19937_64 m;
  explicit Rng(uint64_t seed) : m(seed) {}
  int in(int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(m); }   // [lo, hi]
  template <typename T, size_t N>
  T pick(const T (&v)[N]) { return v[in(0, (int)N - 1)]; }
};

struct Code { int T, Tc, G; };
const Code kCodesSet[] = {{4, 4, 32}, {4, 2, 32}, {4, 2, 16}, {4, 4, 16}, {8, 4, 32}, {1, 1, 32}, {4, 1, 16},
                          {2, 2, 32}, {4, 1, 32}};

int call_attn(const lvq_attn_shape& s, void* ws, size_t bytes, bool scores) {
  g_ws = static_cast<const char*>(ws);
  g_ws_bytes = bytes;
  const auto* p16 = static_cast<const uint16_t*>(dev());
  const auto* p32 = static_cast<const int32_t*>(dev());
  float* out = const_cast<float*>(static_cast<const float*>(dev()));
  if (scores)
    return lvq_decode_scores(p16, p32, static_cast<const uint8_t*>(dev()), p16, p32, p16, s.T - 1, p32, p32, p32,
                             static_cast<const float*>(dev()), &s, out, out, out, ws, bytes, nullptr);
  return lvq_decode_attn(p16, p32, static_cast<const uint8_t*>(dev()), p16, p32, p16, s.T - 1, p32, p32, p32,
                         static_cast<const float*>(dev()), &s, out, out, ws, bytes, nullptr);
}

void decode_shapes(Rng& r, int n, long& ok_calls) {
  const int heads[] = {1, 2, 4, 8, 16};
  const int groups[] = {1, 1, 2, 3, 4, 8, 16};
  for (int i = 0; i < n; ++i) {
    lvq_attn_shape s{};
    const Code cd = r.pick(kCodesSet);
    s.B = r.in(1, 80);
    s.H = r.pick(heads);
    s.Hq = s.H * r.pick(groups);
    s.d = r.in(0, 3) ? 128 : 64;
    s.T = cd.T;
    s.Tc = cd.Tc;
    s.G = cd.G;
    s.n_sink = r.in(0, 8);
    s.max_seq_len = r.in(0, 3) ? r.in(1, 70000) : r.in(1, 400);
    s.max_pages = (s.max_seq_len + 7) / 8 + r.in(0, 3);
    s.bf16_row = r.in(3, 12);
    s.n_index_pages = r.in(1, 1 << 20);
    s.n_bf16_pages = r.in(1, 4096);
    s.rope_max_len = s.max_seq_len + 1 + r.in(0, 50);
    s.n_splits = r.in(0, 2) ? 0 : r.in(1, 5000);
    s.scale = 0.f;
    const size_t need = lvq_decode_attn_workspace_bytes(&s);
    std::printf("attn %d %d %d %d %d %d %d %d %d %d %d %d %d %d %d %zu\n", s.B, s.H, s.Hq, s.d, s.T, s.Tc, s.G,
                s.n_sink, s.max_pages, s.bf16_row, s.n_index_pages, s.n_bf16_pages, s.max_seq_len,
                s.rope_max_len, s.n_splits, need);
    CHECK(need > 0, "workspace query refused a valid shape");
    if (need == 0) continue;
    Workspace ws(need);
    for (int sc = 0; sc < 2; ++sc) {
      const int st = call_attn(s, ws.base, need, sc == 1);
      CHECK(st == LVQ_OK || st == LVQ_EUNSUPPORTED, "decode %s returned %d: %s", sc ? "scores" : "attn", st,
            lvq_last_error());
      if (st == LVQ_OK) {
        ++ok_calls;
        const int st2 = call_attn(s, ws.base, need - 1, sc == 1);
        CHECK(st2 == LVQ_ENOSPC, "one byte short of the workspace returned %d", st2);
      }
    }
  }
}

void rows_shapes(Rng& r, int n, long& ok_calls) {
  const int heads[] = {1, 2, 4, 8, 16};
  const int groups[] = {1, 2, 4, 8, 16};
  for (int i = 0; i < n; ++i) {
    lvq_rows_shape s{};
    const Code cd = r.pick(kCodesSet);
    s.B = r.in(1, 16);
    s.NQ = r.in(0, 1) ? 1 : r.in(1, 600);
    s.H = r.pick(heads);
    s.Hq = s.H * r.pick(groups);
    s.d = 128;
    s.T = cd.T;
    s.Tc = cd.Tc;
    s.G = cd.G;
    s.n_sink = r.in(0, 8);
    s.max_prefix = r.in(0, 40000);
    s.max_pages = (s.max_prefix + 7) / 8 + 1;
    s.bf16_row = r.in(3, 12);
    s.n_index_pages = r.in(1, 1 << 20);
    s.n_bf16_pages = r.in(1, 4096);
    s.rope_max_len = s.max_prefix + s.NQ + 1;
    s.n_splits = r.in(0, 2) ? 0 : r.in(1, 4000);
    const size_t need = lvq_rows_attn_workspace_bytes(&s);
    std::printf("rows %d %d %d %d %d %d %d %d %d %d %d %d %d %d %d %zu\n", s.B, s.NQ, s.H, s.Hq, s.d, s.T, s.Tc,
                s.G, s.n_sink, s.max_pages, s.bf16_row, s.n_index_pages, s.n_bf16_pages, s.max_prefix,
                s.n_splits, need);
    CHECK(need > 0, "rows workspace query refused a valid shape");
    if (need == 0) continue;
    Workspace ws(need);
    const auto* p16 = static_cast<const uint16_t*>(dev());
    const auto* p32 = static_cast<const int32_t*>(dev());
    float* out = const_cast<float*>(static_cast<const float*>(dev()));
    for (int short_by = 0; short_by < 2; ++short_by) {
      g_ws = ws.base;
      g_ws_bytes = need - short_by;
      const int st = lvq_rows_attn(p16, nullptr, nullptr, p32, static_cast<const uint8_t*>(dev()), p16, p32, p16,
                                   s.T - 1, p32, p32, p32, static_cast<const float*>(dev()), &s, out, out, ws.base,
                                   need - short_by, nullptr);
      if (short_by == 0) {
        CHECK(st == LVQ_OK || st == LVQ_EUNSUPPORTED, "rows returned %d: %s", st, lvq_last_error());
        if (st != LVQ_OK) break;
        ++ok_calls;
      } else {
        CHECK(st == LVQ_ENOSPC, "rows one byte short returned %d", st);
      }
    }
  }
}

void builder_shapes(Rng& r, int n, long& ok_calls) {
  const int heads[] = {1, 2, 4, 16};
  for (int i = 0; i < n; ++i) {
    const Code cd = r.pick(kCodesSet);
    const int H = r.pick(heads), d = r.in(0, 3) ? 128 : 64;
    const int S = r.in(0, 2) ? r.in(256, 8192) : r.in(8193, 32768);
    const size_t need = lvq_build_codebooks_workspace_bytes(cd.T, cd.Tc, cd.G, S, H, d);
    std::printf("build %d %d %d %d %d %d %zu\n", cd.T, cd.Tc, cd.G, S, H, d, need);
    if (need == 0) continue;   // shape outside the compiled set
    Workspace ws(need);
    const auto* p16 = static_cast<const uint16_t*>(dev());
    uint16_t* books = const_cast<uint16_t*>(p16);
    for (int short_by = 0; short_by < 2; ++short_by) {
      g_ws = ws.base;
      g_ws_bytes = need - short_by;
      const int st = lvq_build_codebooks(p16, static_cast<const double*>(dev()), nullptr, r.in(0, 1), cd.T, cd.Tc,
                                         cd.G, S, H, d, 10, books, ws.base, need - short_by, nullptr);
      if (short_by == 0) {
        CHECK(st == LVQ_OK, "builder returned %d: %s", st, lvq_last_error());
        if (st != LVQ_OK) break;
        ++ok_calls;
      } else {
        CHECK(st == LVQ_ENOSPC, "builder one byte short returned %d", st);
      }
    }
  }
}

// shapes every entry point must refuse before any launch
void invalid_shapes() {
  const long before = g_launches;
  lvq_attn_shape base{};
  base.B = 2; base.H = 2; base.Hq = 4; base.d = 128; base.T = 4; base.Tc = 4; base.G = 32; base.n_sink = 4;
  base.max_pages = 64; base.bf16_row = 12; base.n_index_pages = 100; base.n_bf16_pages = 20;
  base.max_seq_len = 512; base.rope_max_len = 513;
  std::vector<char> ws(1 << 22);
  auto refused = [&](lvq_attn_shape s, const char* what) {
    const int st = call_attn(s, ws.data(), ws.size(), false);
    CHECK(st != LVQ_OK, "accepted %s", what);
    (void)lvq_decode_attn_workspace_bytes(&s);   // must not trap (division by H etc.)
  };
  lvq_attn_shape s = base; s.H = 0; refused(s, "H = 0");
  s = base; s.Hq = 3; refused(s, "Hq not a multiple of H");
  s = base; s.H = -2; refused(s, "H < 0");
  s = base; s.B = 0; refused(s, "B = 0");
  s = base; s.n_index_pages = 0; refused(s, "n_index_pages = 0");
  s = base; s.rope_max_len = 100; refused(s, "a rope table shorter than max_seq_len");
  s = base; s.Tc = 3; refused(s, "T not a multiple of Tc");
  s = base; s.n_sink = 9; refused(s, "n_sink > 8");
  s = base; s.d = 96; refused(s, "d = 96");
  CHECK(g_launches == before, "an invalid shape reached a launch");
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
  const int n = argc > 2 ? std::atoi(argv[2]) : 400;
  Rng r(seed);
  long ok_attn = 0, ok_rows = 0, ok_build = 0;
  decode_shapes(r, n, ok_attn);
  rows_shapes(r, n / 2, ok_rows);
  builder_shapes(r, n / 4, ok_build);
  invalid_shapes();
  std::printf("summary: %ld launches checked (decode calls %ld, rows %ld, builder %ld), failures %ld\n",
              g_launches, ok_attn, ok_rows, ok_build, g_failures);
  return g_failures > 100 ? 100 : (int)g_failures;
}
