/*
 * libcsa — Compressed Sparse Attention (CSA) and Heavily Compressed Attention
 * (HCA) for AMD MI355X (gfx950), as a C ABI.
 *
 * The method (pages about DeepSeek-V4):
 *   [xmsumi]    xmsumi.com DeepSeek-V4 article, § CSA (压缩稀疏注意力): the KV
 *               entries of every m tokens merge by weighted compression into
 *               one compressed entry; a lightning indexer picks the top-k
 *               entries per query token; multi-query attention runs over the
 *               selected entries plus a sliding-window branch.
 *               § HCA (重度压缩注意力): compression ratio m' >> m, no selection,
 *               dense attention over every compressed entry.
 *               § 关键技术细节: RoPE only on the last 64 dims of queries and
 *               entries with reverse compensation on the output; KV cache with
 *               bf16 RoPE dims and FP8 for the rest; the indexer in FP4.
 *   [hortopato] hortopato.cc wiki "DeepSeek-V4 — MoE nyelvmodellek milliós
 *               kontextussal", CSA list: m = 4, k = 1024, window 128;
 *               § Heavily Compressed Attention (HCA): m' = 128.
 *   [zcldvi]    zcldvi.com V4 article: both attentions add a window branch.
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers owned by the caller; the library never
 *     allocates, frees or synchronises.  Work is enqueued on `stream` (a
 *     hipStream_t; NULL is the null stream).  Inputs and outputs must not
 *     alias.  Outputs are fully overwritten.
 *   - Return value: CSA_OK, or a negative error code; the reason is available
 *     from csa_last_error() on the calling thread.  Errors are detected on the
 *     host before anything is enqueued.  Device-side faults surface at the
 *     caller's next synchronisation.
 *   - Shapes are validated on the host; values inside device arrays (seq,
 *     pos, idx) are trusted except where a call documents a check.
 *   - Determinism.  Every call is run-to-run deterministic: no floating-point
 *     atomics, fixed reduction orders; the backward calls sum shared
 *     gradients in 64-bit fixed point (order-independent integer sums).
 *   - Batch invariance.  csa_compress* and csa_topk give each row (entry)
 *     the same bits whatever the other rows of the call and T.  So does
 *     csa_index_scores* under its exactness precondition (every score exact
 *     in fp32; the kernel chosen for a shape then cannot change a bit).  The
 *     attention calls never read another row's inputs, but each row's key
 *     list is cut into S split-KV ranges, range s = positions
 *     [n*s/S, n*(s+1)/S) of the row's n keys, with
 *       S = min(ceil(256 / T), ceil(bound / 64), 64),
 *       bound = k + window (csa_sparse_mqa) or max_vis + window (hca_dense_mqa),
 *     and the partial results are merged in split order.  With 64 heads the
 *     heads of a split are shared by two workgroups (another summation order)
 *     when T * S <= 128 and the splits hold at most 384 keys; otherwise, when
 *     S' = ceil(S / 2) splits would hold at most 128 keys each and
 *     T * S' <= 128, the row takes S' splits, shared the same way.  A row's
 *     out and lse are bit-identical across calls that give the same splits
 *     and the same sharing (at k = 1024, window = 128: T <= 7 takes 18 shared
 *     splits, 8 <= T <= 14 takes 9 shared splits, T = 15 takes 18 splits of
 *     one workgroup); otherwise the fp16 partials and P round differently
 *     and the results agree to about 3e-4 relative RMS (each meets the 2e-3
 *     relative-RMS bar against the fp64 reference).
 *
 * Storage formats
 *   - Compressed KV entry (and window-ring entry), d = d_nope + 64:
 *     nope[d_nope] FP8 E4M3FN codes, value = code * scale; rope[64] bf16;
 *     scale fp32.  Structure-of-arrays, see csa_kv_t.
 *   - Indexer vectors: MXFP4 (OCP MX): d_i E2M1 values packed two per byte
 *     (element 2i in the low nibble) and one E8M0 scale (2^(b-127)) per 32
 *     consecutive elements.
 *
 * Positions: a query row has absolute position t = pos[row].  Compressed entry
 * j at ratio m covers tokens j*m .. j*m+m-1 and is visible to t iff
 * (j+1)*m - 1 <= t, i.e. j < (t+1)/m (complete blocks only; the incomplete
 * tail lives in the window ring).  Entries are roped at p_j = (j+1)*m - 1.
 */
#ifndef LIBCSA_CSA_H
#define LIBCSA_CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_VERSION 109

enum {
    CSA_OK = 0,
    CSA_EINVAL = -1,       /* null pointer, bad shape, bad alignment */
    CSA_EUNSUPPORTED = -2, /* valid but not implemented (d, heads, k, ...) */
    CSA_EHIP = -3,         /* the HIP runtime refused a launch */
    CSA_EWORKSPACE = -4    /* workspace missing or too small */
};

/* A hipStream_t, passed through untouched. */
typedef void* csa_stream_t;

/*
 * Mixed-precision entries for n_seq sequences, `cap` slots each.  Sequence s,
 * slot i lives at row s*cap + i of every array:
 *   nope  [rows][d - 64]  FP8 E4M3FN codes
 *   rope  [rows][64]      bf16 bit patterns
 *   scale [rows]          fp32
 * Compressed entry j lives at slot j % cap (cap >= entries kept).  A window
 * ring holds raw tokens (m = 1 entries): token p at slot p % cap.
 * Alignment: nope and rope rows must start on 16-byte boundaries
 * ((d-64) % 16 == 0 and 16-byte aligned base pointers).
 *
 * Paged layout (the pages' compressed-entry cache of a two-level KV cache
 * whose entries can be shared by sequences with a common prefix: [xmsumi]
 * § 百万Token 长上下文真实表现): with `pages` non-NULL, slot i of sequence s
 * lives at row pages[s * (cap / page) + i / page] * page + i % page.  page is
 * a power of two dividing cap; the table holds physical page numbers, and
 * sequences may share pages (a common prefix stored once; a page written by
 * csa_compress must not be shared with a sequence that reads it in the same
 * call).  pages == NULL (page ignored) is the contiguous layout above.
 */
typedef struct csa_kv {
    uint8_t* nope;
    uint16_t* rope;
    float* scale;
    int64_t cap;
    const int32_t* pages; /* NULL: contiguous rows */
    int32_t page;         /* slots per page when paged */
} csa_kv_t;

/*
 * MXFP4 indexer keys, one per compressed entry, n_seq*cap rows:
 *   data  [rows][d_i / 2]  packed E2M1
 *   scale [rows][d_i / 32] E8M0
 * Key of entry j of sequence s is row s*cap + j.  16-byte aligned data.
 * Paged layout (as csa_kv_t): with `pages` non-NULL the key of entry j of
 * sequence s lives at row pages[s * (cap / page) + j / page] * page + j % page;
 * page a power of two dividing cap; sequences may share pages.  A compressed
 * cache and its keys can use one page table, so an entry and its key share a
 * page number (what csa_pages_store / csa_pages_load move).
 */
typedef struct csa_index_keys {
    uint8_t* data;
    uint8_t* scale;
    int64_t cap;
    const int32_t* pages; /* NULL: contiguous rows */
    int32_t page;         /* slots per page when paged */
} csa_index_keys_t;

/*
 * csa_compress — token compression ([xmsumi] § CSA: the KV entries of every m
 * tokens merge into one compressed entry by weighted compression; [hortopato]
 * CSA list: m = 4; § HCA: m' = 128).
 *
 * For each complete block b of m tokens, b = 0 .. n_tok/m - 1:
 *   w = softmax(logits[b*m .. b*m+m-1])        (one scalar logit per token)
 *   c = sum_i w_i * kv[b*m + i]                 (fp64, tokens in order)
 *   c[d-64:] rotated by RoPE at p = (J+1)*m - 1, J = tok0/m + b
 *   scale = amax(|c[:d-64]|)/448 (1 if 0); nope = E4M3(c[:d-64]/scale), RNE,
 *   saturating; rope = bf16(c[d-64:]), RNE; both roundings are taken from
 *   the fp64 values (no intermediate fp32 rounding)
 * and stores entry J at slot J % out.cap of sequence `seq`.  With m = 1 it
 * writes raw tokens into a window ring (slot p % cap).
 *
 *   kv      [n_tok][d] bf16, tokens tok0 .. tok0+n_tok-1 of sequence seq
 *   logits  [n_tok] fp32
 *   tok0    multiple of m;  n_tok multiple of m, >= 0 (0 is a no-op);
 *           n_tok/m <= out.cap (one call never writes a slot twice)
 *   m       1 .. 1024;  d in {128, 512}
 *   rope_base  RoPE base (10000 in the pages' setting)
 * RoPE convention: pairs (2i, 2i+1) of the last 64 dims, theta_i =
 * rope_base^(-2i/64), angle = pos * theta_i evaluated in fp64.
 */
int csa_compress(const uint16_t* kv, const float* logits, int64_t tok0, int64_t n_tok, int32_t m, int32_t d,
                 float rope_base, int32_t seq, csa_kv_t out, csa_stream_t stream);

/*
 * csa_compress_channel — csa_compress with one logit per token and channel
 * (the pages call the merge a weighted compression without fixing the
 * weights' shape: [xmsumi] § CSA).  Channel e of block b merges its m tokens
 * with weights softmax_i(logits[bm+i][e]); RoPE, storage and slot rules as
 * csa_compress.  With logits equal across channels it equals csa_compress.
 *   logits [n_tok][d] fp32 (16-byte aligned)
 */
int csa_compress_channel(const uint16_t* kv, const float* logits, int64_t tok0, int64_t n_tok, int32_t m, int32_t d,
                         float rope_base, int32_t seq, csa_kv_t out, csa_stream_t stream);

/*
 * csa_compress_index_keys — the indexer's key for each compressed entry from
 * raw key tokens: the same weighted merge of every m tokens as csa_compress
 * ([xmsumi] § CSA; how the indexer's keys are formed is not on the pages,
 * this is the reading taken), no RoPE (the indexer has none), then MXFP4
 * ([xmsumi] § 关键技术细节: the indexer runs in FP4): per 32 elements the E8M0
 * scale 2^(floor(log2 amax) - 2) (byte 127 for an all-zero block, clamped to
 * 0..254) and E2M1 codes of value / scale, nearest with ties to the even
 * mantissa bit, saturating at 6, zero stored as +0.  Merge in fp64.
 *   k      [n_tok][d_i] bf16 raw key tokens tok0 .. tok0+n_tok-1 of sequence seq
 *   logits [n_tok] fp32 (one per token, as csa_compress)
 *   out    entry J = tok0/m + b at slot J % out.cap of sequence seq (through
 *          out.pages when paged)
 * d_i in {64, 128}; 1 <= m <= 1024; tok0 and n_tok multiples of m.
 */
int csa_compress_index_keys(const uint16_t* k, const float* logits, int64_t tok0, int64_t n_tok, int32_t m,
                            int32_t d_i, int32_t seq, csa_index_keys_t out, csa_stream_t stream);

/*
 * csa_index_scores — lightning-indexer scores ([xmsumi] § CSA: a lightweight
 * indexer ranks compressed entries per query token; § 关键技术细节: FP4
 * arithmetic inside the indexer; [zcldvi]: FP4 relevance of each query token
 * to each compressed block).
 *
 *   score[t][j] = sum_h w[t][h] * max(0, <q[t][h], key_j>)   over MXFP4 values
 *   score[t][j] = -inf for j >= (pos[t]+1)/m
 *
 *   q        [T][h_i][d_i/2] packed E2M1;  q_scale [T][h_i][d_i/32] E8M0
 *   w        [T][h_i] fp32 head weights
 *   seq      [T] int32 sequence of each row;  pos [T] int64 position
 *   keys     index keys (key of entry j of seq s at row s*cap + j)
 *   n_cols   columns written per row (<= keys.cap, < 2^31)
 *   scores   [T][n_cols] fp32
 *   topk_ws  optional (NULL, 0 to skip): the workspace of the csa_topk call
 *            that will read these scores.  When given, the indexer also
 *            writes the selection's row summary into it (for shapes whose
 *            selection uses one: the largest score of every 32-column
 *            group), and that csa_topk call passes CSA_TOPK_PREPARED so the
 *            selection skips its own pass over the scores.  Results are the
 *            same bit for bit either way.
 * h_i in {4, 8}; d_i in {64, 128}.  With power-of-two head weights and block
 * scales whose exponents span a few binades, every score is exact in fp32
 * (each E2M1 product is a multiple of 1/4 below 36 in magnitude).
 */
int csa_index_scores(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq,
                     const int64_t* pos, int64_t T, int32_t h_i, int32_t d_i, csa_index_keys_t keys, int32_t m,
                     int64_t n_cols, float* scores, void* topk_ws, size_t topk_ws_bytes, csa_stream_t stream);

/*
 * csa_index_scores_grouped — csa_index_scores for query rows that come in
 * groups of one sequence, as in multi-token decode (the pages keep
 * multi-token prediction from V3: [xmsumi] § 四大架构创新; its draft tokens
 * are extra query rows of the same sequence at the next positions).
 *
 * Rows g*group .. g*group+group-1 are expected to belong to one sequence; each
 * group then streams its keys once for all its rows (group x h_i rows of the
 * MXFP4 matrix product instead of h_i).  A row of a group whose sequence
 * differs from the group's first row is handled in a separate pass, so the
 * scores (and the row summary) equal those of csa_index_scores bit for bit
 * for any seq / pos.
 *   group  1, 2 or 4 (1 is csa_index_scores);  T % group == 0
 * Every other argument, layout and workspace rule as csa_index_scores.
 */
int csa_index_scores_grouped(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq,
                             const int64_t* pos, int64_t T, int32_t h_i, int32_t d_i, csa_index_keys_t keys,
                             int32_t m, int64_t n_cols, int32_t group, float* scores, void* topk_ws,
                             size_t topk_ws_bytes, csa_stream_t stream);

/*
 * csa_index_topk — the indexer and the top-k selection fused, without
 * writing the score rows ([xmsumi] § CSA: the indexer ranks the compressed
 * entries per query token and only the top-k are kept; [hortopato] CSA list:
 * k = 1024).  idx receives what csa_index_scores followed by csa_topk would
 * give (same arguments, same order rule and padding), bit for bit under the
 * indexer's exactness precondition.
 *
 * How: the indexer scores a sample of each row (all of its first
 * max(2048, 2k) columns, then one 32-column group in 16) and a per-row
 * threshold is set where the sample predicts about 2k columns above it; a
 * second indexer pass emits only the columns whose score reaches the
 * threshold, and the exact top-k is taken among them.  The count is verified:
 * a row with fewer than k such columns, or more than its candidate space, is
 * scored again on its own and selected over the whole row (correct, slower).
 *   idx        [T][k] int32 (written)
 *   1 <= k <= 2048;  n_cols >= 1;  h_i in {4, 8};  d_i in {64, 128}
 * Workspace: csa_index_topk_workspace(T, n_cols, k, h_i) bytes, 256-byte
 * aligned, contents need no initialisation; calls sharing it must not run
 * concurrently.  It holds the sample keys, the candidates (a few times k per
 * row) and 16 scratch rows of n_cols floats for re-scored rows.
 */
size_t csa_index_topk_workspace(int64_t T, int64_t n_cols, int32_t k, int32_t h_i);
int csa_index_topk(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq, const int64_t* pos,
                   int64_t T, int32_t h_i, int32_t d_i, csa_index_keys_t keys, int32_t m, int64_t n_cols, int32_t k,
                   int32_t* idx, void* ws, size_t ws_bytes, csa_stream_t stream);

/*
 * csa_index_bwd — gradient of the lightning-indexer scores (training side:
 * the pages warm the indexer up and train its QK path in FP4, [xmsumi]
 * § 预训练：32T Token 炼就基座 and [hortopato]'s training section; no page
 * gives the gradient, so this is the exact derivative of csa_index_scores).
 * Given G = dL/dscore at the selected columns j = idx[t][a] (entries with
 * j < 0 or j >= (pos[t]+1)/m are ignored), with dot_h = <q[t][h], key_j> and
 * the ReLU's derivative taken as 0 at 0:
 *   dq[t][h]  = sum_a G[t][a] w[t][h] [dot_h > 0] key_j
 *   dw[t][h]  = sum_a G[t][a] max(0, dot_h)
 *   dkeys[row of key_j] += sum_t sum_a G[t][a] sum_h w[t][h] [dot_h > 0] q[t][h]
 * with respect to the dequantised MXFP4 values (quantisation passes the
 * gradient straight through).
 *   idx, g     [T][n_sel] int32 / fp32 (e.g. csa_topk's indices and the loss's
 *              gradient at them; any n_sel >= 1)
 *   dq         [T][h_i][d_i] fp32, dw [T][h_i] fp32: written
 *   dkeys      [key_rows][d_i] fp32, indexed like the keys (seq * keys.cap + j):
 *              ACCUMULATED into; every referenced row must be < key_rows
 * The key gradients are summed in 64-bit fixed point (each term rounded to a
 * multiple of 2^-40; |partial sums| < 2^23), so dkeys does not depend on the
 * order the rows' terms arrive in: repeated calls give the same bits.  dq and
 * dw are summed in a fixed order per row.  The dot products are exact under
 * csa_index_scores' precondition, so the ReLU decisions match its scores.
 * Workspace: csa_index_bwd_workspace(key_rows, d_i) bytes, 8-byte aligned
 * (cleared by the call).  h_i in {4, 8}; d_i in {64, 128}.
 */
size_t csa_index_bwd_workspace(int64_t key_rows, int32_t d_i);
int csa_index_bwd(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq, const int64_t* pos,
                  int64_t T, int32_t h_i, int32_t d_i, csa_index_keys_t keys, int32_t m, const int32_t* idx,
                  const float* g, int32_t n_sel, float* dq, float* dw, float* dkeys, int64_t key_rows, void* ws,
                  size_t ws_bytes, csa_stream_t stream);

/*
 * csa_topk — top-k selection ([xmsumi] § CSA: the top-k compressed entries
 * per query token; [hortopato] CSA list: k = 1024).
 *
 * For each row t, among columns j < min(n_cols, (pos[t]+1)/m), the
 * min(k, visible) largest scores under the total order (score descending,
 * index ascending; -0.0 equals +0.0), written in ascending index order,
 * padded with -1.
 *   scores [T][n_cols] fp32 (NaN not supported);  idx [T][k] int32
 *   1 <= k <= 2048;  n_cols < 2^31
 * Workspace: csa_topk_workspace(T, n_cols, k) bytes (may be 0), 256-byte
 * aligned; its contents need no initialisation, and one buffer serves any
 * sequence of calls (any shapes) on one stream.  Calls that share a
 * workspace must not run concurrently.
 * flags: 0, or CSA_TOPK_PREPARED when the preceding csa_index_scores call
 * for these scores was given this workspace (it wrote the row summary).
 */
#define CSA_TOPK_PREPARED 1u
size_t csa_topk_workspace(int64_t T, int64_t n_cols, int32_t k);
int csa_topk(const float* scores, int64_t T, int64_t n_cols, const int64_t* pos, int32_t m, int32_t k, int32_t* idx,
             void* ws, size_t ws_bytes, uint32_t flags, csa_stream_t stream);

/*
 * csa_topk_noalloc — csa_topk for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same selection, arguments and results as csa_topk with flags 0;
 * instead of a caller workspace it uses a 12 MiB scratch array of the library
 * (one per GPU, held until the process ends).  It allocates nothing.
 *   Limit: shapes whose csa_topk_workspace(T, n_cols, k) exceeds 12 MiB
 *   (few rows of very many columns, e.g. T x n_cols beyond ~32 M for T < 128)
 *   are refused with CSA_EUNSUPPORTED; other shapes need no scratch.
 * Every call on one GPU shares that array: calls that overlap on one GPU
 * (concurrent streams, threads) race and must be serialised by the caller.
 */
int csa_topk_noalloc(const float* scores, int64_t T, int64_t n_cols, const int64_t* pos, int32_t m, int32_t k,
                     int32_t* idx, csa_stream_t stream);

/*
 * csa_sparse_mqa — CSA attention: multi-query attention (one shared KV head;
 * every entry is both key and value) over the selected compressed entries
 * plus the sliding-window branch, merged in one softmax (what a log-sum-exp
 * merge of the two branches gives) ([xmsumi] § CSA; [hortopato] CSA list:
 * window 128; RoPE and reverse compensation per [xmsumi] § 关键技术细节).
 *
 * Row t, head h: key set U = { comp entry idx[t][a] : 0 <= idx < (t+1)/m }
 * (entries outside that range are ignored) plus window tokens
 * max(0, t-window+1) .. t (ring slot p % win.cap); duplicates kept.
 *   q~ = q[t][h] with RoPE at t on its last 64 dims
 *   s_u = sm_scale * <q~, e_u>;  lse = log sum exp s_u;  o = sum exp(s_u-lse) e_u
 *   o[d-64:] rotated by RoPE at -t;  empty U gives o = 0, lse = -inf
 *
 *   q   [T][H][d] bf16 (before RoPE);  seq [T] int32;  pos [T] int64
 *   idx [T][k] int32;  comp / win: compressed cache / window ring
 *   out [T][H][d] fp32;  lse [T][H] fp32
 * H in {16, 32, 64}; d in {128, 512}; 1 <= k <= 2048; 0 <= window <= 1024.
 * The window ring must hold every token max(0, t-window+1) .. t of every row
 * at slot p % win.cap (win.cap >= window).
 * Range: the kernels stage the entries' bf16 RoPE dims as fp16, so every
 * entry read must have |rope value| <= 65504 (larger values are clamped or
 * overflow; entries written by csa_compress from data of that magnitude
 * qualify).  With the environment variable CSA_DEBUG_CHECKS=1 this call and
 * hca_dense_mqa first scan the entries they will read and return CSA_EINVAL
 * on a violation (the scan synchronises the stream; not for graph capture).
 * Workspace: csa_mqa_workspace(T, H, d, k + window) bytes (split-KV partials).
 */
size_t csa_mqa_workspace(int64_t T, int32_t H, int32_t d, int64_t max_keys);
int csa_sparse_mqa(const uint16_t* q, const int32_t* seq, const int64_t* pos, int64_t T, int32_t H, int32_t d,
                   const int32_t* idx, int32_t k, int32_t m, csa_kv_t comp, csa_kv_t win, int32_t window,
                   float sm_scale, float rope_base, float* out, float* lse, void* ws, size_t ws_bytes,
                   csa_stream_t stream);

/*
 * hca_dense_mqa — HCA attention ([xmsumi] § HCA: no selection, dense attention
 * over every compressed entry; [hortopato] § HCA: m' = 128; [zcldvi]: window
 * branch in both attentions).  Same as csa_sparse_mqa with the key set
 * { every comp entry j < (t+1)/m } plus the window.
 *   max_vis  an upper bound on (pos[t]+1)/m over the rows, >= 1; with T it
 *            sets the split-KV partition (see the batch-invariance rule at the
 *            top: results are bit-identical for equal partitions and agree
 *            to rounding level otherwise); the workspace is
 *            csa_mqa_workspace(T, H, d, max_vis + window).
 */
int hca_dense_mqa(const uint16_t* q, const int32_t* seq, const int64_t* pos, int64_t T, int32_t H, int32_t d,
                  int32_t m, int64_t max_vis, csa_kv_t comp, csa_kv_t win, int32_t window, float sm_scale,
                  float rope_base, float* out, float* lse, void* ws, size_t ws_bytes, csa_stream_t stream);

/*
 * csa_mqa_bwd — gradient of the attention step (training side: the pages
 * train with the sparse attention in place, [xmsumi] § 预训练, after an
 * indexer warm-up; no page gives the gradient, so this is the exact
 * derivative of csa_sparse_mqa / hca_dense_mqa).  With q~ = q[t][h] roped at
 * pos[t], g = dout[t][h], g~ = g roped at pos[t] on its last 64 dims, and the
 * forward's out and lse:
 *   p_u = exp(sm_scale <q~, e_u> - lse);  ds_u = p_u (<g~, e_u> - <g, out>)
 *   dq[t][h] = sm_scale * sum_u ds_u e_u, rotated back by RoPE at -pos[t]
 *   dcomp / dwin row of entry u += sm_scale ds_u q~ + p_u g~
 * over the same key set U as the forward (idx non-null: the selected entries
 * as csa_sparse_mqa; idx null: every visible entry as hca_dense_mqa, k ignored),
 * gradients taken with respect to the dequantised entries (FP8 * scale, BF16).
 *
 *   q [T][H][d] bf16, out [T][H][d] fp32, lse [T][H] fp32: the forward's
 *   inputs and outputs; dout [T][H][d] fp32;  dq [T][H][d] fp32 (written)
 *   dcomp [comp_rows][d], dwin [win_rows][d] fp32: indexed by the same cache
 *            row as the entries (seq * cap + slot, or through the page
 *            table); ACCUMULATED into (the caller clears them); every row
 *            an entry of the key sets lives at must be < comp_rows / win_rows.
 *            dwin may be null (win_rows ignored) when window == 0.
 * H in {16, 32, 64}; d = 512 only; 16-byte aligned q, out, dout, dq.
 * Determinism: entries shared by rows and heads are summed in 64-bit fixed
 * point (each term rounded to a multiple of 2^-40; |partial sums| < 2^23), so
 * dcomp and dwin do not depend on the order the terms arrive in: repeated
 * calls give the same bits.  dq is summed in a fixed order per row.
 * The output gradient is scaled by a power of two per (row, 16 heads) inside;
 * entries with |e|_2 above ~3e4 may overflow the fp16 products.
 * Workspace: csa_mqa_bwd_workspace(comp_rows, win_rows, d) bytes (win_rows 0
 * when window == 0), 8-byte aligned, cleared by the call.
 */
size_t csa_mqa_bwd_workspace(int64_t comp_rows, int64_t win_rows, int32_t d);
int csa_mqa_bwd(const uint16_t* q, const int32_t* seq, const int64_t* pos, int64_t T, int32_t H, int32_t d,
                const int32_t* idx, int32_t k, int32_t m, csa_kv_t comp, csa_kv_t win, int32_t window, float sm_scale,
                float rope_base, const float* out, const float* lse, const float* dout, float* dq, float* dcomp,
                int64_t comp_rows, float* dwin, int64_t win_rows, void* ws, size_t ws_bytes, csa_stream_t stream);

/*
 * csa_pages_store / csa_pages_load — move physical pages of a compressed cache
 * and of its index keys between the GPU and a host buffer, for reuse of a
 * shared prefix beyond the GPU's memory (the pages keep the compressed
 * entries of a two-level KV cache and store them on disk for shared-prefix
 * reuse: [xmsumi] § 百万Token 长上下文真实表现).
 *
 * Physical page p is rows p*page .. p*page+page-1 of every array (page =
 * kv.page, a power of two; keys.page must be the same, so an entry and its
 * index key share a page number; the page tables are not read).  The host
 * layout holds the n_pages pages in the order given, each as its arrays one
 * after the other: nope [page][d-64], rope [page][64] bf16, scale [page] fp32,
 * then (d_i > 0) key data [page][d_i/2] and key scales [page][d_i/32];
 * csa_pages_bytes(page, d, d_i) bytes per page.  d_i = 0 moves entries only.
 *   pages      HOST array of n_pages physical page numbers, each >= 0 and
 *              within the arrays (the library cannot see their extent: that
 *              bound is the caller's); all are checked to be >= 0 before
 *              any copy is enqueued
 *   host       host buffer (pinned memory lets the copies run asynchronously)
 * The copies are enqueued on `stream`; the caller synchronises before it
 * reads (store) or reuses (load) the host buffer.  A load followed by a
 * store of the same pages gives back the same bytes.
 */
size_t csa_pages_bytes(int32_t page, int32_t d, int32_t d_i);
int csa_pages_store(csa_kv_t kv, csa_index_keys_t keys, int32_t d, int32_t d_i, const int32_t* pages,
                    int32_t n_pages, void* host, size_t host_bytes, csa_stream_t stream);
int csa_pages_load(csa_kv_t kv, csa_index_keys_t keys, int32_t d, int32_t d_i, const int32_t* pages,
                   int32_t n_pages, const void* host, size_t host_bytes, csa_stream_t stream);

/*
 * csa_mfma_probe — a measurement helper, not a step of the path: `blocks`
 * workgroups of 256 threads issue MFMAs back to back with no memory traffic
 * (each wave iters x 4 of them in four independent chains; iters a multiple
 * of 4) and write one
 * float per thread to sink (blocks x 256 floats, meaningless values).  A
 * timed launch gives the rate the matrix cores sustain on this GPU for the
 * shapes the path uses:
 *   kind 0: fp16 16x16x32 (the attention);  kind 1: MXFP4 32x32x64 (the indexer)
 * csa_mfma_probe_flops returns the flop count of such a launch (-1 for a bad
 * argument).
 */
int64_t csa_mfma_probe_flops(int32_t kind, int32_t blocks, int64_t iters);
int csa_mfma_probe(int32_t kind, int32_t blocks, int64_t iters, float* sink, int64_t sink_len, csa_stream_t stream);

/* Text of the last error on the calling thread ("" if none). */
const char* csa_last_error(void);

/* CSA_VERSION of the built library. */
int csa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBCSA_CSA_H */
