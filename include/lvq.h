/*
 * lvq.h -- C ABI of the LoopVQ hot path for AMD Instinct MI355X (gfx950).
 *
 * LoopVQ codes the KV cache of a looped transformer along the loop axis: the T
 * loop steps are split into contiguous blocks of Tc steps, and one 8-bit code
 * (K = 256 codewords) covers c = G / Tc channels of every step of a block, so
 * the cache keeps 8 / G bits per element whatever Tc is.  Each loop step reads
 * back only its own c-channel share of the chosen codeword.  Keys are coded
 * before RoPE; attention applies RoPE to the reconstructed keys.  Sources:
 * the LoopVQ summary (onedev.kr/papers/1681), sections "무엇과 다른가" (the
 * joint code, the shared index, pre-RoPE keys) and "전제와 한계" (8-token
 * pages, bf16 sink and recent tokens, one index row per loop block, encoding by
 * a codebook-distance matrix product once all Tc steps exist, re-encoding the
 * oldest recent page every 8 decode tokens, a decode kernel that reads only the
 * loop-step-t codebook slice and merges Flash-Decoding splits with a
 * log-sum-exp); the rit.work LoopVQ article, section "Когда LoopVQ меняет план
 * развёртывания" (keys and values both rebuilt from the codebooks, merged with
 * the uncompressed part of the cache).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every array argument is DEVICE memory owned by the caller.  The library
 *    never allocates, frees or keeps a pointer; scratch space comes only from
 *    the caller's workspace argument.
 *  - bf16 arrays are passed as uint16_t bit patterns.  All layouts are dense,
 *    row-major, with the listed dimension order (last dimension contiguous).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    with no host synchronisation; outputs are valid once the stream has
 *    reached that point.  Entry points are thread-safe; the only state is the
 *    calling thread's last error string.
 *  - The return value is a status code.  Every argument check happens on the
 *    host before anything is enqueued, so on LVQ_EINVAL, LVQ_EUNSUPPORTED or
 *    LVQ_ENOSPC nothing ran.  LVQ_EDEVICE reports a failed launch; a call made of
 *    several launches may have run the earlier ones, and its outputs are then
 *    unspecified.
 *    LVQ_EINVAL: a null pointer, a size <= 0 where one is required, Tc not
 *    dividing T or G, c = G/Tc not dividing d, t >= T, Hq not a multiple of H,
 *    n_sink > 8, a table too small for the requested lengths.
 *    LVQ_EUNSUPPORTED: a valid shape outside the compiled set (see each call).
 *    LVQ_ENOSPC: the workspace is smaller than the size query returns.
 *    LVQ_EDEVICE: a HIP launch error.
 *  - Device-side indices (page ids, page-table entries) are range-checked in
 *    the kernels: an out-of-range id is skipped (its tokens are treated as
 *    absent / its rows are not written) instead of being dereferenced.  The
 *    attention calls count such lookups in a caller's device counter when the
 *    shape names one (lvq_attn_shape.rejected, lvq_rows_shape.rejected).
 *  - Codebook values must lie in the float16 range (|x| < 65504): the decode
 *    kernel stages the step-t slice in LDS as float16, which holds every such
 *    bfloat16 value exactly up to float16 subnormals.
 *  - Code indices are unsigned bytes; any value 0..255 is a valid code.
 */
#ifndef LVQ_H
#define LVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LVQ_ABI_VERSION 1
#define LVQ_PAGE 8      /* tokens per cache page */
#define LVQ_NCODES 256  /* codewords per codebook (8-bit codes) */

enum lvq_status {
  LVQ_OK = 0,
  LVQ_EINVAL = 1,
  LVQ_EUNSUPPORTED = 2,
  LVQ_ENOSPC = 3,
  LVQ_EDEVICE = 4
};

/* ABI version (LVQ_ABI_VERSION of the built library). */
int lvq_version(void);

/* Text describing the calling thread's last non-zero status ("" if none). */
const char* lvq_last_error(void);

/*
 * Codebook layout (all encode and decode calls):
 *   codebooks: bf16 [nblk][2][H][ng][Tc][256][c], nblk = T/Tc, c = G/Tc,
 *   ng = d/c.  Index [beta][kv][h][g][tau][k][i] is element tau*c + i of
 *   codeword k of the book of loop block beta, K (kv = 0) or V (kv = 1),
 *   KV head h and channel group g (channels g*c .. g*c+c-1).  The step-tau
 *   share of every codeword of a book is one contiguous [256][c] slice.
 *
 * Joint vector of (block beta, token n, head h, group g), G elements:
 *   x[tau*c + i] = X[beta*Tc + tau][n][h][g*c + i],  tau < Tc, i < c.
 * Its code is the lowest index k minimising the squared L2 distance
 * sum_e (x[e] - codeword_k[e])^2 (the summary, section "전제와 한계", computes
 * these distances with a matrix product; the kernel uses the expansion
 * |x|^2 - 2 x.C + |C|^2 on bf16 MFMA with float32 accumulation and recomputes
 * in float64, by direct differences, every vector whose top two candidates
 * are too close for float32 to separate them; vectors whose products fall below
 * the float32 normal range or whose norms overflow it always take that path, so
 * the codes are the float64 ones at every finite bf16 input).
 *
 * Supported encoder shapes: G in {16, 32}; c = G/Tc in {8, 16, 32} for
 * G = 32 and {4, 8, 16} for G = 16; d in {64, 128}.
 */

/*
 * lvq_encode -- code one of K or V for N tokens (prefill).
 *   kv:        bf16 [T][N][H][d], the keys (pre-RoPE) or values of all T steps.
 *   codebooks: see above.  kv_sel = 0 uses the K books, 1 the V books.
 *   idx:       out, uint8 [nblk][N][H][ng].
 * Encoding needs all Tc steps of a block (the summary, section "전제와 한계").
 */
int lvq_encode(const uint16_t* kv, const uint16_t* codebooks, int kv_sel, int T, int Tc,
               int G, int N, int H, int d, uint8_t* idx, void* stream);

/*
 * lvq_encode_pages -- as lvq_encode, but writes the rows into the paged cache.
 *   chunk_page:  int32 [N/8], physical coded page of tokens 8j .. 8j+7.  N must
 *                be a multiple of 8.  Ids outside [0, n_index_pages) are skipped.
 *   index_pages: in/out, uint8 [n_index_pages][nblk][H][2][8][ng].  Token n is
 *                written to page chunk_page[n/8], half kv_sel, slot n%8: one
 *                index row per loop block (the summary, section "전제와 한계").
 *                Only the rows of the selected half are written.
 */
int lvq_encode_pages(const uint16_t* kv, const uint16_t* codebooks, int kv_sel, int T, int Tc,
                     int G, int N, int H, int d, const int32_t* chunk_page, int n_index_pages,
                     uint8_t* index_pages, void* stream);

/*
 * lvq_reencode_pages -- decode-time re-encode: code whole bf16 pages (every
 * loop step, head, K and V) into coded pages, all in one launch.  This is the
 * step that turns the oldest recent page of a sequence into index rows every
 * 8 generated tokens (the summary, section "전제와 한계").
 *   bf16_pages:  bf16 [n_bf16_pages][T][H][2][8][d] (pre-RoPE keys, values).
 *   src_pages:   int32 [n], bf16 pages to encode.
 *   dst_pages:   int32 [n], coded pages to write (all 8 slots, K and V halves).
 *   index_pages: in/out, uint8 [n_index_pages][nblk][H][2][8][ng].
 * Ids out of range are skipped.  n = 0 is a no-op.
 */
int lvq_reencode_pages(const uint16_t* bf16_pages, const int32_t* src_pages,
                       const int32_t* dst_pages, int n, const uint16_t* codebooks, int T, int Tc,
                       int G, int H, int d, int n_bf16_pages, int n_index_pages,
                       uint8_t* index_pages, void* stream);

/*
 * lvq_reencode_pages_layers -- lvq_reencode_pages for several layers at once: the
 * same page ids (a page id names the same page in every layer's pools) re-encoded
 * in every listed layer, each with its own pools and codebooks, in one launch per
 * 48 layers instead of one per layer.  Every 8 generated tokens a sequence's oldest
 * recent page is coded in all layers (the summary, section "전제와 한계"), so this
 * is the per-token re-encode of a whole model.
 *   layers:      host array [n_layers], read during the call only; per layer its
 *                bf16 pool ([n_bf16_pages][T][H][2][8][d]), codebooks
 *                ([nblk][2][H][ng][Tc][256][c]) and coded pool
 *                ([n_index_pages][nblk][H][2][8][ng], in/out), device pointers.
 *   src_pages, dst_pages: int32 [n] device arrays as in lvq_reencode_pages.
 * T, Tc, G, H, d are shared by all layers.  Results are bit-identical to one
 * lvq_reencode_pages call per layer.  Ids out of range are skipped; n = 0 or
 * n_layers = 0 is a no-op.  Any invalid layer fails the call before any launch.
 */
typedef struct lvq_reencode_layer {
  const uint16_t* bf16_pages;
  const uint16_t* codebooks;
  uint8_t* index_pages;
  int32_t n_bf16_pages;
  int32_t n_index_pages;
} lvq_reencode_layer;

int lvq_reencode_pages_layers(const lvq_reencode_layer* layers, int n_layers,
                              const int32_t* src_pages, const int32_t* dst_pages, int n, int T,
                              int Tc, int G, int H, int d, void* stream);

/*
 * lvq_build_codebooks -- learn the 256-word codebooks of one of K / V from sample
 * tokens on the device: k-means on calibration keys and values (the summary,
 * section "전제와 한계", experiments paragraph: k-means calibration on 16
 * calibration sequences of 2,048 tokens), Fisher-weighted when weights are given
 * (section "무엇과 다른가": the codebooks start from Fisher-weighted k-means; the
 * Fisher information needs model gradients, so the weights are an input).  Every book (loop block,
 * head, group) is built at once.
 *   samples:   bf16 [T][S][H][d], S sample tokens (pre-RoPE keys or values), the
 *              encoder's input layout.  1 <= S <= 32768 (the summary's calibration set
 *              is 16 sequences of 2,048 tokens: 32,768 sample tokens).
 *   draws:     float64 [nblk][H][ng][256], uniform numbers in [0, 1) that drive the
 *              k-means++ seeding of each book.  Draw k picks the first sample s whose
 *              running sum of terms (sample order, float64) exceeds u_k times the
 *              total: the terms are w_s for draw 0 (so sample floor(u0 S) without
 *              weights) and w_s D^2_s for k >= 1, D^2 the squared distance to the
 *              nearest chosen center; the last s with a positive term if rounding
 *              leaves none; sample floor(u_k S) if the total is not positive.
 *   weights:   float64 [nblk][S][H][ng], one finite weight >= 0 per joint vector (the
 *              assignment layout), or NULL for all 1.  Negative or non-finite
 *              weights give unspecified books (the kernels stay in bounds).
 *   n_iter:    Lloyd iterations, 0 .. 1000.  Each assigns every sample to its nearest
 *              center rounded to bf16 (exact, lowest index on ties) and moves each
 *              center to sum(w_s x_s) / sum(w_s) over its members, both float64 sums
 *              in sample order (a cluster of zero total weight keeps its center).
 *   codebooks: out, bf16 [nblk][2][H][ng][Tc][256][c]; only half kv_sel is written,
 *              the final centers rounded to bf16 through float32.
 *   ws:        device workspace of lvq_build_codebooks_workspace_bytes() bytes.
 * Same shapes as lvq_encode (status 2 outside them, or for S > 32768).  The result
 * is bit-reproducible: every float64 step has a fixed order.
 */
size_t lvq_build_codebooks_workspace_bytes(int T, int Tc, int G, int S, int H, int d);
int lvq_build_codebooks(const uint16_t* samples, const double* draws, const double* weights,
                        int kv_sel, int T, int Tc, int G, int S, int H, int d, int n_iter,
                        uint16_t* codebooks, void* ws, size_t ws_bytes, void* stream);

/*
 * RoPE phase tables.  Keys are coded before RoPE and attention rotates the
 * reconstructed keys (the summary, section "무엇과 다른가"), so the decode kernel
 * needs the phase of every cached position.  Rotate-half convention: channel j
 * pairs with j + d/2 and turns by the angle p * theta_j, theta_j = base^(-2j/d).  Phases are formed
 * in float64 (angle and cos/sin); the table holds, in order:
 *   float32 rows 0 .. ntile-1:       (cos, sin)(16 a * theta_j), j < d/2   (a = p / 16)
 *   float32 rows ntile .. ntile+15:  (cos, sin)(o * theta_j),    j < d/2   (o = p % 16)
 *   float64 theta_j, j < d/2
 * with ntile = ceil(max_len / 16) and float32 row layout [d/2][2].  A position
 * p < max_len is the float32 product of one row of each of the first two parts
 * (error ~1e-7).  The table must be built with the d of the decode call.
 */
size_t lvq_rope_table_bytes(int max_len, int d);
int lvq_rope_tables(int max_len, int d, double base, float* rope_tab, size_t rope_bytes,
                    void* stream);

/* Shape of one decode-attention call. */
typedef struct lvq_attn_shape {
  int32_t B;              /* sequences */
  int32_t H;              /* KV heads */
  int32_t Hq;             /* query heads, a multiple of H; query head hq reads KV head hq/(Hq/H) */
  int32_t d;              /* head dim (64 or 128) */
  int32_t T, Tc, G;       /* loop steps, steps per joint block, joint length */
  int32_t n_sink;         /* bf16 sink tokens (<= 8), read from the bf16 copy of page 0 */
  int32_t max_pages;      /* row length of page_table */
  int32_t bf16_row;       /* row length of bf16_table */
  int32_t n_index_pages;  /* rows of index_pages (range check of page ids), >= 1 even when
                             every token is bf16; a coded token whose page id is outside
                             [0, n_index_pages) is left out of the attention */
  int32_t n_bf16_pages;   /* rows of bf16_pages, >= 1 */
  int32_t max_seq_len;    /* upper bound of seq_len[b]; sizes the automatic split */
  int32_t rope_max_len;   /* max_len the rope table was built for; every pos and seq_len must be < it */
  int32_t n_splits;       /* waves per query head (per KV head on the grouped route, per
                             work list of lvq_rows_attn on the multi-row route);
                             0 = automatic (see lvq_decode_attn) */
  float scale;            /* softmax scale; 0 = 1/sqrt(d) */
  uint32_t* rejected;     /* NULL, or a device uint32 the kernels add one to for every page-id
                             lookup outside its pool (page_table entries outside
                             [0, n_index_pages) within a sequence's coded range, bf16_table
                             entries outside [0, n_bf16_pages) for its sink and recent
                             tokens); those tokens are left out whether or not it is given.
                             An entry read by several heads or waves counts once for each.
                             The caller clears it; calls that share it add up. */
} lvq_attn_shape;

/* Workspace bytes of lvq_decode_attn / lvq_decode_scores for this shape: the
 * partial (max, sum, output) records of the Flash-Decoding split that the
 * log-sum-exp merge combines (the summary, section "전제와 한계").  Returns 0 for a
 * null or malformed shape (B, H, Hq, d, Tc, G or max_seq_len not positive, Hq not a
 * multiple of H). */
size_t lvq_decode_attn_workspace_bytes(const lvq_attn_shape* shp);

/*
 * lvq_decode_attn -- decode attention at loop step t over the paged cache (the
 * summary, section "전제와 한계": the kernel reads only the loop-step-t codebook
 * slice, splits the coded tokens Flash-Decoding style and merges the parts by
 * log-sum-exp; section "무엇과 다른가": RoPE on the reconstructed keys; the rit.work
 * article, section "Когда LoopVQ меняет план развёртывания": keys and values are
 * rebuilt from the codebooks and merged with the uncompressed bf16 tokens).
 *   q:           bf16 [B][Hq][d], pre-RoPE query of loop step t.
 *   page_table:  int32 [B][max_pages], logical page -> coded page id.  Entries of
 *                logical pages 0 .. q_end[b]/8 - 1 are read.
 *   index_pages: uint8 [n_index_pages][nblk][H][2][8][ng] (layout of lvq_encode_pages).
 *   bf16_pages:  bf16 [n_bf16_pages][T][H][2][8][d], pre-RoPE keys and values.
 *   bf16_table:  int32 [B][bf16_row]: entry 0 = bf16 copy of logical page 0 (the
 *                sink tokens), entries 1.. = the pages of logical pages q_end/8,
 *                q_end/8 + 1, ... (the recent window).
 *   codebooks:   see above.
 *   t:           loop step, 0 <= t < T; block t/Tc, step slice t%Tc are read.
 *   pos:         int32 [B], RoPE position of the query.
 *   seq_len:     int32 [B], cached tokens L_b (positions 0 .. L_b-1).  L_b = 0 (an
 *                empty slot of the batch) gives out = 0 and lse = -inf for its heads.
 *   q_end:       int32 [B], multiple of 8: tokens [n_sink, q_end) are coded,
 *                [0, n_sink) and [q_end, L_b) are bf16 (sink wins where both apply).
 *   rope_tab:    table built by lvq_rope_tables for this d and base.
 *   out:         float32 [B][Hq][d], softmax(q'.k'/scale) v over all L_b tokens.
 *   lse:         float32 [B][Hq] or NULL: natural log-sum-exp of the scaled scores.
 *   ws:          workspace of at least lvq_decode_attn_workspace_bytes(shp) bytes.
 * Each call overwrites the workspace; concurrent calls need distinct workspaces.
 * Work split: per query head, the 16-token tiles of all sequences (coded tiles, then
 * the bf16 sink and recent tiles, sequence by sequence) form one list that is cut
 * into equal contiguous ranges, one per wave, whatever the mix of lengths; partial
 * results are merged per (b, hq) by log-sum-exp.  n_splits > 0 sets the number of
 * waves per query head (rounded up to whole workgroups of 12); 0 gives each head an
 * equal share of the 256 compute units.
 * Supported: d = 128 with c in {8, 16, 32}; d = 64 with c in {8, 16}.  With 2 or 4
 * query heads per KV head at d = 128 the call runs on the grouped kernel, which
 * dequantises and rotates each key once for the KV head's query heads; the list is then
 * per KV head, its ranges go to quads of 4 waves, and n_splits counts waves per KV head
 * (whole workgroups of 16).  With 8 or more query heads per KV head at d = 128 it runs on
 * the multi-row kernel (see lvq_rows_attn), which shares each key's reconstruction among
 * those heads as the rows of its matrix-core products.  The workspace size accounts for
 * every route.
 */
int lvq_decode_attn(const uint16_t* q, const int32_t* page_table, const uint8_t* index_pages,
                    const uint16_t* bf16_pages, const int32_t* bf16_table,
                    const uint16_t* codebooks, int t, const int32_t* pos, const int32_t* seq_len,
                    const int32_t* q_end, const float* rope_tab, const lvq_attn_shape* shp,
                    float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * lvq_decode_attn_noalloc -- lvq_decode_attn for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, kernels and results as lvq_decode_attn, without the
 * workspace: the partial records live in a fixed device array of the library,
 * LVQ_NOALLOC_SCRATCH_BYTES per device, that each device keeps from its first use
 * until the process ends.  The call allocates nothing and calls no allocating routine.
 * A shape whose lvq_decode_attn_workspace_bytes() exceeds that size returns
 * LVQ_ENOSPC before anything is enqueued.  Every call on one device shares that
 * device's array, so calls whose work overlaps on one device (concurrent streams, or
 * host threads on one device without ordering) race on it and give undefined
 * results; calls ordered on one stream are safe.  The array keeps the last call's
 * contents, which no call reads before writing them.
 */
#define LVQ_NOALLOC_SCRATCH_BYTES (32u << 20)
int lvq_decode_attn_noalloc(const uint16_t* q, const int32_t* page_table,
                            const uint8_t* index_pages, const uint16_t* bf16_pages,
                            const int32_t* bf16_table, const uint16_t* codebooks, int t,
                            const int32_t* pos, const int32_t* seq_len, const int32_t* q_end,
                            const float* rope_tab, const lvq_attn_shape* shp, float* out,
                            float* lse, void* stream);

/*
 * lvq_decode_scores -- test probe: same inputs as lvq_decode_attn (same passages),
 * always on the per-head kernel (the grouped and multi-row routes of lvq_decode_attn
 * do not apply), which also writes the scaled scores q'.k' * scale
 * (natural units) of every cached token to scores, from which the attention mass
 * of a span of positions (the long-context retrieval check of the summary, section
 * "전제와 한계", RULER needle tasks) follows as sum exp(s_p - lse): float32 [B][Hq][max_seq_len]
 * (entries at p >= seq_len[b] are left untouched).  out and lse are produced too.
 */
int lvq_decode_scores(const uint16_t* q, const int32_t* page_table, const uint8_t* index_pages,
                      const uint16_t* bf16_pages, const int32_t* bf16_table,
                      const uint16_t* codebooks, int t, const int32_t* pos,
                      const int32_t* seq_len, const int32_t* q_end, const float* rope_tab,
                      const lvq_attn_shape* shp, float* out, float* lse, float* scores,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * Multi-row attention: many query rows per KV head in one call, each key rebuilt
 * and rotated once and shared by the rows.  Two uses (the summary, sections "전제와
 * 한계" -- the same decode attention, and a prefill that the summary notes runs
 * slightly slower than bf16 -- and "무엇과 다른가" -- RoPE after reconstruction):
 *  - prefill chunk over an existing coded prefix: NQ new tokens per sequence, each
 *    attending to the paged prefix and causally to the chunk's own keys;
 *  - GQA decode (NQ = 1, no new keys): the Hq/H query heads of a KV head are the rows.
 * Query i of sequence b, head hq, at RoPE position pos[b] + i, attends over the paged
 * tokens [0, prefix_len[b]) exactly as lvq_decode_attn does with seq_len = prefix_len
 * (coded [n_sink, q_end), bf16 sink and recent), plus, when k_new is given, the new
 * keys 0 .. i at positions prefix_len[b] + i'.
 *   q:            bf16 [B][NQ][Hq][d], pre-RoPE.
 *   k_new, v_new: bf16 [B][NQ][H][d] pre-RoPE keys and values of the chunk at loop
 *                 step t, or both NULL.
 *   page_table, index_pages, bf16_pages, bf16_table, codebooks, t, q_end, rope_tab:
 *                 as lvq_decode_attn.
 *   prefix_len:   int32 [B], paged tokens visible to every query.  A row that sees no
 *                 key at all (prefix_len 0 and no new keys) gets out = 0, lse = -inf.
 *   out:          float32 [B][NQ][Hq][d]; lse: float32 [B][NQ][Hq] or NULL.
 *   ws:           lvq_rows_attn_workspace_bytes(shp) bytes.
 * Scores and the value sum run on the matrix cores at float32 precision: on coded tiles
 * the float32 operands are split into float16 hi + lo parts and three (scores) or two
 * (values) float16 products are summed in float32, each missing about 2^-20 of its
 * value; bf16 tiles use float32 matrix instructions.  The split needs the rotated
 * query values times scale * log2(e) and the rotated key values inside the float16
 * range (|x| < 65504), next to the codebook range every decode kernel needs.
 * Supported: d = 128, c in {8, 16, 32}.
 */
typedef struct lvq_rows_shape {
  int32_t B, NQ, H, Hq, d, T, Tc, G;
  int32_t n_sink, max_pages, bf16_row, n_index_pages, n_bf16_pages;
  int32_t max_prefix;     /* upper bound of prefix_len[b] */
  int32_t rope_max_len;   /* >= max_prefix + NQ; every pos[b] + NQ - 1 must be below it */
  int32_t n_splits;       /* waves per work list (a KV head's block of 16 rows), rounded up
                             to whole workgroups of 8; 0 = automatic */
  float scale;            /* softmax scale; 0 = 1/sqrt(d) */
  uint32_t* rejected;     /* NULL, or a device uint32 counting page-id lookups outside their
                             pool, as in lvq_attn_shape */
} lvq_rows_shape;

size_t lvq_rows_attn_workspace_bytes(const lvq_rows_shape* shp);
int lvq_rows_attn(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                  const int32_t* page_table, const uint8_t* index_pages, const uint16_t* bf16_pages,
                  const int32_t* bf16_table, const uint16_t* codebooks, int t, const int32_t* pos,
                  const int32_t* prefix_len, const int32_t* q_end, const float* rope_tab,
                  const lvq_rows_shape* shp, float* out, float* lse, void* ws, size_t ws_bytes,
                  void* stream);

/*
 * Paged cache manager -- the page bookkeeping of the decode loop, on the device,
 * with no host synchronisation.  It keeps the rules of the summary, section
 * "전제와 한계": the cache is paged in 8 tokens; the sink tokens and the recent
 * window stay bf16; once a token's forward pass (all loop steps and layers) is
 * done and the window holds n_recent + 8 tokens, its oldest page is quantised
 * across every layer and loop step and leaves the window.  Between calls, for every
 * live sequence b:
 *   q_end[b] = 8 * floor((seq_len[b] - n_recent) / 8), or 0 when that is negative;
 *   page_table[b][0 .. q_end/8) = its coded pages;
 *   bf16_table[b][0] = the bf16 page of logical page 0 (the sink copy), and
 *   bf16_table[b][1 ..] = the bf16 pages of logical pages q_end/8, q_end/8 + 1, ...
 * which are exactly the arrays lvq_decode_attn reads.  A page id names the same
 * page in every layer's pools (index_pages and bf16_pages of each layer), so one
 * state serves the whole model.
 *
 * Every array is int32 device memory owned by the caller:
 *   page_table [B][max_pages], bf16_table [B][bf16_row], seq_len [B], q_end [B];
 *   index_free [n_index_pages], bf16_free [n_bf16_pages]: stacks of free page ids;
 *   counters [4]: free coded pages, free bf16 pages, error bits, 0;
 *   re_src [B], re_dst [B]: the pending re-encode of each sequence (bf16 page ->
 *   coded page) between lvq_cache_end_token and lvq_cache_commit, else -1.
 * Page ids are handed out lowest first, sequences in index order, so the state is
 * a deterministic function of the calls.  Error bits (counters[2], sticky, read by
 * the caller when convenient): 1 coded pool empty, 2 bf16 pool empty, 4 a sequence
 * longer than max_pages pages, 8 a window longer than bf16_row allows.  The
 * allocation that fails is skipped (its entry stays -1, which attention and
 * encoding skip as out of range); the contents are then unspecified, but every
 * kernel stays within the arrays above.
 *
 * One decode token, in order: lvq_cache_begin_token; for each loop step t and
 * layer: lvq_cache_append (that layer's K/V at step t), then lvq_decode_attn;
 * lvq_cache_end_token; lvq_reencode_pages_layers over every layer's pools with
 * re_src, re_dst, B (or lvq_reencode_pages per layer); lvq_cache_commit.  All calls
 * on one stream.
 */
typedef struct lvq_cache {
  int32_t B;              /* sequence slots */
  int32_t max_pages;      /* page_table row length: at most 8 * max_pages tokens */
  int32_t bf16_row;       /* bf16_table row length, >= lvq_cache_min_bf16_row(n_recent) */
  int32_t n_sink;         /* bf16 sink tokens, 0 .. 8 (kept in logical page 0) */
  int32_t n_recent;       /* recent bf16 tokens kept, >= 0 */
  int32_t n_index_pages;  /* coded pages per layer pool */
  int32_t n_bf16_pages;   /* bf16 pages per layer pool */
  int32_t* page_table;
  int32_t* bf16_table;
  int32_t* seq_len;
  int32_t* q_end;
  int32_t* index_free;
  int32_t* bf16_free;
  int32_t* counters;
  int32_t* re_src;
  int32_t* re_dst;
} lvq_cache;

/* Smallest bf16_row for n_recent: entry 0 plus ceil((n_recent + 8) / 8) pages. */
int lvq_cache_min_bf16_row(int n_recent);

/* Empty cache: every page free, tables -1, lengths 0, no error. */
int lvq_cache_init(const lvq_cache* c, void* stream);

/*
 * Prefill bookkeeping: each slot b with seq_len[b] == 0 and lengths[b] > 0 (int32
 * [B], device) gets L = lengths[b] tokens: q_end by the rule above, coded pages for
 * logical pages [0, q_end/8), bf16 pages for logical page 0 and [q_end/8, ceil(L/8)).
 * The caller then fills them per layer: lvq_encode_pages of tokens [0, q_end) with
 * chunk_page = page_table + b * max_pages, and lvq_cache_store_tokens.
 */
int lvq_cache_prefill(const lvq_cache* c, const int32_t* lengths, void* stream);

/*
 * Copies tokens first .. first+n-1 of sequence b into one layer's bf16 pages, the
 * tokens that live there (logical page 0 and positions >= q_end[b]); tokens at or
 * beyond seq_len[b] are ignored.  k, v: bf16 [T][n][H][d] (pre-RoPE); bf16_pages:
 * [n_bf16_pages][T][H][2][8][d].  d must be a multiple of 8.
 */
int lvq_cache_store_tokens(const lvq_cache* c, int b, int first, int n, const uint16_t* k,
                           const uint16_t* v, int T, int H, int d, uint16_t* bf16_pages,
                           void* stream);

/* A new token for every live sequence (seq_len > 0): a bf16 page when the token
 * starts a page, then seq_len += 1. */
int lvq_cache_begin_token(const lvq_cache* c, void* stream);

/*
 * Writes the new token (position seq_len[b] - 1) of every live sequence into one
 * layer's bf16 pages, loop steps t0 .. t0+n_steps-1.  k, v: bf16 [n_steps][B][H][d];
 * T is the pages' loop-step count (t0 + n_steps <= T).
 */
int lvq_cache_append(const lvq_cache* c, int t0, int n_steps, const uint16_t* k,
                     const uint16_t* v, int T, int H, int d, uint16_t* bf16_pages, void* stream);

/* After the token's forward pass: re_src/re_dst name the pages to re-encode (a coded
 * page is taken for every sequence whose window reached n_recent + 8), -1 elsewhere. */
int lvq_cache_end_token(const lvq_cache* c, void* stream);

/* After the re-encode of every layer: the coded pages join the page tables, q_end
 * advances by 8, and the re-encoded bf16 pages leave the windows (back to the pool,
 * except logical page 0, which stays as the sink copy). */
int lvq_cache_commit(const lvq_cache* c, void* stream);

/* Frees every page of the slots with mask[b] != 0 (int32 [B], device) and empties
 * them (seq_len 0), ready for lvq_cache_prefill. */
int lvq_cache_release(const lvq_cache* c, const int32_t* mask, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LVQ_H */
