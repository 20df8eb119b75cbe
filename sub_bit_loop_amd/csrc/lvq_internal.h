// Internal launch interface between the C ABI (lvq_abi.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "lvq.h"

namespace lvq {

// Runs set() (a kernel attribute such as its dynamic-LDS limit, which applies to the
// current device) the first time it is needed on each device.  Flags are per device
// and atomic; two first calls racing on one device both run set(), which is
// idempotent.  Devices beyond 64 run set() on every call.
template <typename F>
inline hipError_t once_per_device(std::atomic<uint64_t>& done, F&& set) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = set();
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

constexpr int kPage = 8;
constexpr int kCodes = 256;

// Sets the calling thread's error text (printf format) and returns code.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Size of the fixed device scratch array behind lvq_decode_attn_noalloc.
constexpr size_t kNoAllocScratchBytes = LVQ_NOALLOC_SCRATCH_BYTES;

// ---------------------------------------------------------------- encoder
enum EncodeSrc { kSrcDense = 0, kSrcPages = 1 };
enum EncodeDst { kDstDense = 0, kDstPages = 1 };

struct EncodeArgs {
  const uint16_t* src;        // dense kv [T][N][H][d] or bf16 pages [P'][T][H][2][8][d]
  const int32_t* src_pages;   // [N/8] bf16 page ids (kSrcPages)
  const uint16_t* codebooks;  // [nblk][2][H][ng][Tc][256][c]
  uint8_t* out;               // dense idx [nblk][N][H][ng] or index pages
  const int32_t* dst_pages;   // [N/8] coded page ids (kDstPages)
  int src_mode, dst_mode;
  int kv_sel;                 // 0 / 1, or -1: both halves (pages source)
  int T, Tc, G, N, H, d;
  int n_src_pages, n_dst_pages;
  int tokens_per_block;       // multiple of 16
  int head_block;             // heads whose items share an XCD (a divisor of H, at most 8)
};
// The pools and books of one layer in a multi-layer re-encode (pages -> pages).
struct ReencodeLayer {
  const uint16_t* bf16_pages;
  const uint16_t* codebooks;
  uint8_t* index_pages;
  int n_bf16_pages, n_index_pages;
};
constexpr int kMaxReencodeLayers = 48;   // layers per launch (passed by value as kernel arguments)
struct ReencodeLayers {
  int n;
  ReencodeLayer layer[kMaxReencodeLayers];
};
bool encode_supported(int G, int c, int d);
// layers: for a pages -> pages launch, the layers to encode (null: the one a names)
hipError_t launch_encode(const EncodeArgs& a, hipStream_t s, const ReencodeLayers* layers = nullptr);

// ---------------------------------------------------------------- codebook builder
constexpr int kMaxKmeansSamples = 32768;     // samples per book (the update's member lists fit LDS)
constexpr int kMaxKmeansSamplesLds = 8192;   // up to here the seeding keeps D^2 and running sums in LDS
struct KmeansArgs {
  const uint16_t* samples;    // bf16 [T][S][H][d]
  const double* draws;        // [n_books][256] uniform in [0, 1), book = (beta * H + h) * ng + g
  const double* weights;      // [nblk][S][H][ng] per joint vector, or null (all 1)
  uint16_t* codebooks;        // bf16 [nblk][2][H][ng][Tc][256][c]; half kv_sel is written
  double* centers;            // workspace [n_books][256][G]
  uint8_t* assign;            // workspace [nblk][S][H][ng]
  double* d2;                 // workspace [n_books][S rounded up to 32] (S > kMaxKmeansSamplesLds), else null
  int kv_sel, T, Tc, G, S, H, d, n_iter, n_books;
};
hipError_t launch_build_codebooks(const KmeansArgs& a, hipStream_t s);

// ---------------------------------------------------------------- multi-row attention
// Query rows (query token i of a chunk, query head hq) of one KV head share each key's
// dequantisation and rotation; scores and the value sum run on fp32 MFMA.
struct RowsArgs {
  const uint16_t* q;          // [B][NQ][Hq][d]
  const uint16_t* k_new;      // [B][NQ][H][d] or null: the chunk's own keys at step t
  const uint16_t* v_new;      // [B][NQ][H][d] or null
  const int32_t* page_table;
  const uint8_t* index_pages;
  const uint16_t* bf16_pages;
  const int32_t* bf16_table;
  const uint16_t* codebooks;
  const int32_t* pos;         // [B] position of query 0
  const int32_t* prefix_len;  // [B] paged tokens, visible to every query
  const int32_t* q_end;       // [B]
  const float* rope;
  float* part;                // [H * n_rb][n_rec][16 rows][d + 2]
  unsigned* rejected;         // optional counter of page-id lookups outside their pool, or null
  int t, B, NQ, H, Hq, d, T, Tc, G;
  int n_sink, max_pages, bf16_row, n_index_pages, n_bf16_pages, max_prefix, rope_tiles;
  int n_rb;                   // row blocks of 16 per KV head
  int n_waves;                // waves per (KV head, row block) list
  int n_rec;                  // records per list and row: n_waves + B
  int* tile_start;            // [n_rb][B + 1] first unit of each sequence in a row block's list
  float scale_log2e;
};
bool rows_supported(int d, int c);
int rows_waves_per_group();
hipError_t launch_rows(const RowsArgs& a, hipStream_t s);

// ---------------------------------------------------------------- paged cache manager
struct CacheArgs {
  int B, max_pages, bf16_row, n_sink, n_recent, n_index_pages, n_bf16_pages;
  int32_t* page_table;        // [B][max_pages]
  int32_t* bf16_table;        // [B][bf16_row]
  int32_t* seq_len;           // [B]
  int32_t* q_end;             // [B]
  int32_t* index_free;        // [n_index_pages] stack of free coded page ids
  int32_t* bf16_free;         // [n_bf16_pages] stack of free bf16 page ids
  int32_t* counters;          // [4] free coded, free bf16, error bits, 0
  int32_t* re_src;            // [B]
  int32_t* re_dst;            // [B]
};
struct TokenCopy {
  const uint16_t* k;          // bf16 keys of the tokens to copy
  const uint16_t* v;          // bf16 values
  uint16_t* pool;             // bf16 pages [n_bf16_pages][T][H][2][8][d] of one layer
  int T, H, d;
};
hipError_t launch_cache_init(const CacheArgs& c, hipStream_t s);
hipError_t launch_cache_prefill(const CacheArgs& c, const int32_t* lengths, hipStream_t s);
hipError_t launch_cache_step(const CacheArgs& c, int which, hipStream_t s);   // 0 begin, 1 end, 2 commit
hipError_t launch_cache_release(const CacheArgs& c, const int32_t* mask, hipStream_t s);
hipError_t launch_cache_store(const CacheArgs& c, const TokenCopy& tc, int b, int first, int n, hipStream_t s);
hipError_t launch_cache_append(const CacheArgs& c, const TokenCopy& tc, int t0, int n_steps, hipStream_t s);

// ---------------------------------------------------------------- RoPE tables
hipError_t launch_rope_tables(int ntile, int d, double base, float* tab, hipStream_t s);

// ---------------------------------------------------------------- decode attention
struct AttnArgs {
  const uint16_t* q;
  const int32_t* page_table;
  const uint8_t* index_pages;
  const uint16_t* bf16_pages;
  const int32_t* bf16_table;
  const uint16_t* codebooks;
  const int32_t* pos;
  const int32_t* seq_len;
  const int32_t* q_end;
  const float* rope;          // tile rows [ntile][d/2][2], offset rows [16][d/2][2], theta [d/2] (double)
  float* part;                // partial records [lists][n_rec][rows][d + 2]
  float* out;                 // [B][Hq][d]
  float* lse;                 // [B][Hq] or null
  float* scores;              // [B][Hq][max_seq_len] or null (probe)
  unsigned* rejected;         // optional counter of page-id lookups outside their pool, or null
  int t, B, H, Hq, d, T, Tc, G;
  int n_sink, max_pages, bf16_row, n_index_pages, n_bf16_pages, max_seq_len, rope_tiles;
  int n_waves;                // waves per work list (token-balanced ranges)
  int n_rec;                  // records per work list: n_waves + B
  int* tile_start;            // [lists' row blocks][B + 1] first unit of each sequence
  int merge_rows;             // merge input: 0 decode records, 1 multi-row records (16 rows),
                              // 2 grouped decode records (Hq / H rows, kGroupQuad per range)
  int NQ, n_rb;               // multi-row merge: queries per sequence, row blocks per KV head
  float scale_log2e;          // softmax scale * log2(e)
};
hipError_t launch_merge(const AttnArgs& a, hipStream_t s);   // merge of multi-row records into a.out / a.lse
// Merge of decode records (merge_rows 0 or 2) into m.out / m.lse: cap candidate records
// per (b, hq), about per_item of them written (it picks the merge's width).
hipError_t launch_merge_records(const AttnArgs& m, int cap, int per_item, hipStream_t s);
bool attn_supported(int d, int c);
int rope_tile();   // positions per row of the first RoPE table part
int attn_waves_per_group();   // waves per decode-attention workgroup
int merge_max_records();      // candidate partial records per (b, query head) the merge accepts
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);

// Grouped-query decode: the 2 or 4 query heads of a KV head share each key's
// dequantisation and rotation; a range of a KV head's work list belongs to a quad of
// kGroupQuad waves, each of which writes a record of Hq / H rows per sequence (n_rec =
// n_waves + kGroupQuad * B per list).
constexpr int kGroupQuad = 4;
bool attn_group_supported(int d, int c, int heads);
int attn_group_waves_per_group();   // waves per grouped-decode workgroup
hipError_t launch_attn_group(const AttnArgs& a, hipStream_t s);

}  // namespace lvq
