/*
 * clsa.h - C ABI of libclsa, shared-routing sparse decode attention for
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes (CLSA explainer, ai-papers.net, "CLSAとは？
 * ルーティング共有で128Kコンテキスト推論を17倍高速化するスパースアテンション",
 * section "CLSAの仕組み"): for every query token a single routing step picks
 * the top-k positions of the KV cache once, and every cross-decoder layer
 * reuses that one index list to run softmax attention over only those rows.
 * Section "計算コストの削減効果" of the same page gives the reason: routing is
 * paid once per token (cost ~ N) instead of once per layer (~ L*N).
 * The threshold variant follows the Louver summary (gist.science,
 * "技術サマリー：スパースアテンションを範囲検索問題として捉える",
 * section "1. 半空間範囲検索への帰着"): return every key whose inner product
 * with the query is at least tau, with no false negatives.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers, 16-byte aligned, dense
 *    row-major with the layouts given below.  Pointer arrays (one entry per
 *    layer) are HOST arrays of device pointers.
 *  - The caller owns every buffer.  The library allocates no device memory
 *    and keeps no state between calls; scratch space comes from the caller's
 *    workspace `ws` of at least the size returned by the matching
 *    *_workspace_size function (same shape arguments).  A size of 0 means
 *    either that the call needs no workspace (ws may then be NULL) or that
 *    the call would reject the shapes.  The one exception is
 *    clsa_route_static, whose scratch is a fixed device array of the
 *    library (see there).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it and returns without synchronizing.  Calls that share
 *    one workspace must be ordered (same stream, or synchronized).
 *  - Arguments are validated on the host before anything is enqueued; a call
 *    that returns an error has written nothing.  Conditions that can only
 *    be seen on the device are reported through the outputs (see `counts`).
 *  - q, q_idx, K, V and K_idx share the call's dtype; `out` has that dtype.
 *    All arithmetic accumulates in fp32.  NaN/Inf inputs are undefined.
 */
#ifndef CLSA_H
#define CLSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CLSA_VERSION 1
/* Maximum number of layers one clsa_sparse_attn call accepts. */
#define CLSA_MAX_LAYERS 64

/* Element type of keys, queries and K/V.  A caller may pass any int: the
 * calls reject values other than these two with CLSA_ERR_UNSUPPORTED_DTYPE.
 * C++ gives the enum int as its underlying type so that such a value is
 * well defined there too (in C every int already is). */
#ifdef __cplusplus
typedef enum clsa_dtype : int {
#else
typedef enum clsa_dtype {
#endif
  CLSA_F32 = 0,  /* IEEE binary32 */
  CLSA_BF16 = 1  /* bfloat16, stored as uint16 bit patterns */
} clsa_dtype;

typedef enum clsa_status {
  CLSA_OK = 0,
  CLSA_ERR_INVALID = -1,           /* null pointer, bad shape or size */
  CLSA_ERR_WORKSPACE = -2,         /* ws too small (or NULL with a nonzero need) */
  CLSA_ERR_UNSUPPORTED_DTYPE = -3, /* dtype not CLSA_F32 / CLSA_BF16 */
  CLSA_ERR_HIP = -4,               /* a kernel launch failed */
  CLSA_ERR_SCRATCH_LIMIT = -5      /* clsa_route_static: the shapes need more
                                      than CLSA_STATIC_SCRATCH_BYTES */
} clsa_status;

/* Library version (CLSA_VERSION of the build). */
int clsa_version(void);

/* Static description of a status code. Never NULL. */
const char* clsa_status_string(int status);

/*
 * clsa_route - top-k routing, computed once and shared by all layers.
 * (CLSA explainer, section "CLSAの仕組み": top-k indices of the important KV
 * pairs for each query token; k = 2048 is the pages' operating point.)
 *
 * Rows: R = B*M query rows; row (b, m) uses routing key set b.
 *   q_idx  [B][M][d]      routing queries.
 *   K_idx  [B][n_cap][d]  routing keys (one index head), n_cap slots per
 *                         sequence; only the first n_ctx[b] are visible.
 *   n_ctx  [B] int32, DEVICE, or NULL (then every sequence has n_cap keys).
 *          Values are clamped to [0, n_cap].
 *   q_pos0 -1 for decode (row (b, m) sees n_ctx[b] keys).  q_pos0 >= 0 marks
 *          a prefill chunk: row m is the token at position q_pos0 + m and
 *          sees keys 0 .. q_pos0 + m (causal, diagonal included), capped at
 *          n_ctx[b].
 *   k      routed tokens per row, k >= 1.
 *   idx    [B][M][cap] int32 out: the selected key positions of the row, in
 *          ascending order, then -1 up to cap.  cap >= k.
 *   counts [B][M] int32 out: min(k, visible keys).
 * Score: s_j = sum_i q_idx[i] * K_idx[j][i], fp32 accumulation of exact
 * products (bf16 x bf16 is exact in fp32).  Selection: the counts largest
 * scores; equal scores are taken in increasing j.  -0.0 equals +0.0.
 * d must be 32, 64 or 128.
 * Blocks of query rows (bf16, M >= 64, k <= 2048, n_cap <= 512K, e.g. a
 * prefill chunk) score on the matrix cores: the score matrix is filtered
 * against a per-row sampled threshold inside the MFMA epilogue and never
 * written out; the workspace then holds up to 8 bytes per (row, key) for
 * the filtered candidates.  Scores within a row are computed one way for
 * every key, so the selection and tie rule are the same on both paths; the
 * scores themselves may differ from the one-query path in the last bits
 * (fp32 summation order).
 * Other bf16 rows with k <= 2048 and n_cap <= 512K (decode: one query per
 * sequence) first score up to 4096 evenly spaced keys for a per-row lower
 * bound of the k-th score, then stream every visible key once and keep only
 * those at or above it; the workspace holds about 72 KB per row whatever
 * n_cap is (up to 512K).  A row whose bound keeps fewer than k keys, more
 * than 6144, or more than one chunk's share of the candidate entries,
 * is redone exactly (much slower, results unchanged).  Other rows (fp32, or
 * k > 2048) keep every key's score in the workspace (12 bytes per key).
 * Errors: CLSA_ERR_INVALID (null pointer, B/M/k < 1, d unsupported,
 * n_cap outside [1, 2^31 - 1], B*M > 65535, cap < k),
 * CLSA_ERR_UNSUPPORTED_DTYPE, CLSA_ERR_WORKSPACE, CLSA_ERR_HIP.
 */
size_t clsa_route_workspace_size(int B, int M, int d, int64_t n_cap, int k, int cap,
                                 clsa_dtype dt);
int clsa_route(const void* q_idx, const void* K_idx, int B, int M, int d, int64_t n_cap,
               const int32_t* n_ctx, int64_t q_pos0, int k, clsa_dtype dt, int32_t* idx,
               int32_t* counts, int cap, void* ws, size_t ws_bytes, void* stream);

/*
 * clsa_route_static - clsa_route for callers that cannot allocate.
 * For callers that may not call hipMalloc or any allocating routine
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation, kernels and results as clsa_route,
 * with the workspace taken from a fixed array of CLSA_STATIC_SCRATCH_BYTES
 * in device memory that the library holds on every GPU it runs on, until
 * the process ends.  The caller still passes the inputs and outputs.
 *
 * Arguments are those of clsa_route without ws / ws_bytes.  The call runs
 * on the calling thread's current device, which must be the device of
 * `stream`.  It allocates nothing (the array's address is looked up once per
 * device, on the first call there).
 * Shapes whose clsa_route_workspace_size exceeds CLSA_STATIC_SCRATCH_BYTES
 * are rejected with CLSA_ERR_SCRATCH_LIMIT before anything is enqueued:
 * with bf16 keys and k <= 2048, at least 109 decode rows (M = 1) fit at any
 * context length up to 512K (113 at 128K).
 * Every call on one GPU uses that GPU's one array, which keeps the previous
 * call's contents (the kernels clear what they need zeroed): calls that
 * overlap on one GPU (different streams, or different host threads without
 * ordering) race and give undefined results.  Order them on one stream.
 * Errors: as clsa_route, plus CLSA_ERR_SCRATCH_LIMIT, and CLSA_ERR_HIP when
 * the current device cannot be queried.
 */
#define CLSA_STATIC_SCRATCH_BYTES (8u << 20)
int clsa_route_static(const void* q_idx, const void* K_idx, int B, int M, int d, int64_t n_cap,
                      const int32_t* n_ctx, int64_t q_pos0, int k, clsa_dtype dt, int32_t* idx,
                      int32_t* counts, int cap, void* stream);

/*
 * clsa_route_threshold - half-space selection with no false negatives.
 * (Louver summary, section "1. 半空間範囲検索への帰着": every key with
 * <q, k> >= tau is returned.)
 *
 * Same arguments as clsa_route, with
 *   tau    [B][M] float, DEVICE: the row's threshold.
 * Writes every visible j with s_j >= tau (fp32 score, fp32 compare) in
 * ascending order.  counts[b][m] is the TRUE size of the set; if it exceeds
 * cap only the first cap indices are written, and the caller re-runs with a
 * larger cap (nothing is dropped silently).  Unused slots hold -1.
 * Errors: as clsa_route (cap >= 1 instead of cap >= k).
 */
size_t clsa_route_threshold_workspace_size(int B, int M, int d, int64_t n_cap, int cap,
                                           clsa_dtype dt);
int clsa_route_threshold(const void* q_idx, const void* K_idx, int B, int M, int d,
                         int64_t n_cap, const int32_t* n_ctx, int64_t q_pos0, const float* tau,
                         clsa_dtype dt, int32_t* idx, int32_t* counts, int cap, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * clsa_sparse_attn - softmax attention of every layer over the shared lists.
 * (CLSA explainer, section "CLSAの仕組み": each cross-decoder layer reuses
 * the one index list; the KV cache is the YOCO shared cache, so passing the
 * same K/V pointer for every layer is the single-cache case.)
 *
 *   q[l]   [B][M][Hq][D]     query of layer l.
 *   K[l], V[l] [B][n_cap][Hkv][D]  key/value cache of layer l, token-major.
 *   idx    [B][M][cap] int32, counts [B][M] int32: as written by clsa_route
 *          or clsa_route_threshold.  Row (b, m) attends over its first
 *          min(counts, cap) entries (none if counts < 0); entries outside
 *          [0, n_cap) are padding and skipped; a position listed twice
 *          counts twice in the softmax.
 *   scale  logit scale; 0 means 1/sqrt(D).
 *   out[l] [B][M][Hq][D] out, dtype of V.
 *   lse    [L][B][M][Hq] float out (natural log-sum-exp of the scaled
 *          logits), or NULL.
 * Query head h reads KV head h / (Hq/Hkv) (grouped-query attention).
 * An empty list gives out = 0 and lse = -inf.
 * Constraints: 1 <= L <= CLSA_MAX_LAYERS, B*M <= 65535, cap >= 1,
 * Hq % Hkv == 0, Hq/Hkv <= 16, Hkv <= 64, Hq <= 64, 8 <= D <= 256 and
 * D % 8 == 0, Hq*D <= 8192, scale finite and >= 0.
 * Errors: CLSA_ERR_INVALID, CLSA_ERR_UNSUPPORTED_DTYPE, CLSA_ERR_WORKSPACE,
 * CLSA_ERR_HIP.
 */
size_t clsa_sparse_attn_workspace_size(int L, int B, int M, int Hq, int Hkv, int D, int cap,
                                       clsa_dtype dt);
int clsa_sparse_attn(int L, int B, int M, int Hq, int Hkv, int D, const void* const* q,
                     const void* const* K, const void* const* V, int64_t n_cap,
                     const int32_t* idx, const int32_t* counts, int cap, float scale,
                     clsa_dtype dt, void* const* out, float* lse, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * Louver index - threshold selection that checks only the keys of clusters
 * whose bounding ball reaches the query's half-space.
 * (Louver summary, gist.science, section "2. Louver インデックス": the key
 * space is cut into S contiguous subspaces; in each, a balanced PCA tree
 * groups the keys into clusters of at most r keys, each wrapped in a
 * bounding ball; a query prunes the clusters whose ball misses the
 * half-space and checks the others' keys exactly; keys added while decoding
 * wait in a buffer and are clustered into the index when it fills.
 * Section "クエリアルゴリズム": Query 1 (mode 1) prunes every subspace with
 * its own threshold; Query 2 (mode 2) is the threshold algorithm: clusters
 * scanned in descending bound until the bounds of the next depth sum below
 * tau.  Both have no false negatives.)
 *
 * The index of B sequences covers key positions [0, n_max) of K_idx
 * [B][n_cap][d] (bf16, d = 32, 64 or 128) in segments: segment k is one
 * tree over positions [seg_bounds[k], seg_bounds[k+1]) of every sequence,
 * with seg_bounds[0] = 0, strictly increasing, at most 16 segments, at most
 * 8192 clusters per segment.  S is 1, 2 or 4 (d / S a multiple of 8);
 * 8 <= r <= 256; n_max <= 2^24.
 *
 *   index   caller-owned device buffer of clsa_louver_index_bytes(...).
 *   clsa_louver_build builds segment nseg - 1 of an index whose segments
 *           0 .. nseg - 2 were built by earlier calls (so clustering the
 *           buffer of appended keys is one more call; nothing is rebuilt).
 *           seg_bounds is a HOST array of nseg + 1 entries, last <= n_cap;
 *           every sequence must hold valid keys up to it.  ws: device
 *           workspace of clsa_louver_build_workspace_size(...).
 *   clsa_louver_query selects, for each sequence b (one query row each:
 *           q_idx [B][d], tau [B] float DEVICE, n_ctx [B] int32 DEVICE or
 *           NULL), every visible position j (j < n_ctx[b]) with
 *           q_idx[b] . K_idx[b][j] >= tau[b] -- fp32 sums of exact products,
 *           compared in fp32 as in clsa_route_threshold, so the results are
 *           the same.  Positions past seg_bounds[nseg] are checked exactly
 *           (the buffer).  Outputs as clsa_route_threshold (M = 1): idx
 *           [B][cap] ascending then -1, counts [B] the true set size.
 *           checked [B] (device, may be NULL) receives the number of keys
 *           whose exact score the query computed.  The index must have been
 *           built with the same B, d, S, r, n_max and segments.
 * Errors: CLSA_ERR_INVALID (null pointer, shapes, segments, mode not 1/2,
 * index_bytes too small), CLSA_ERR_UNSUPPORTED_DTYPE (not CLSA_BF16),
 * CLSA_ERR_WORKSPACE, CLSA_ERR_HIP.
 */
size_t clsa_louver_index_bytes(int B, int d, int64_t n_max, int S, int r);
size_t clsa_louver_build_workspace_size(int B, int d, int64_t n_max, int S, int r);
int clsa_louver_build(const void* K_idx, int B, int d, int64_t n_cap, clsa_dtype dt, int S, int r,
                      int64_t n_max, int nseg, const int64_t* seg_bounds, void* index,
                      size_t index_bytes, void* ws, size_t ws_bytes, void* stream);
size_t clsa_louver_query_workspace_size(int B, int d, int64_t n_cap, int S, int r, int64_t n_max,
                                        int nseg, const int64_t* seg_bounds);
int clsa_louver_query(const void* q_idx, const void* K_idx, int B, int d, int64_t n_cap,
                      const int32_t* n_ctx, const float* tau, clsa_dtype dt, int S, int r,
                      int64_t n_max, int nseg, const int64_t* seg_bounds, const void* index,
                      int mode, int32_t* idx, int32_t* counts, int cap, uint32_t* checked,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * clsa_route_aggregated - top-k routing of cross-layer aggregated scores.
 * (CLAA abstract, fugumt.com, "CLAA: Cross-Layer Attention Aggregation for
 * Accelerating LLM Prefill": token importance taken from single layers is
 * unstable; aggregating it across layers ranks tokens stably.)
 * H index heads (one per layer): q_idx and K_idx are HOST arrays of H device
 * pointers, each laid out as in clsa_route; the score of key j for row
 * (b, m) is sum_h q_idx[h][b][m] . K_idx[h][b][j] (fp32 sums of exact
 * products), and the row's list is the top-k of that sum with clsa_route's
 * rules and outputs.  1 <= H <= 64; the workspace is that of the exhaustive
 * path (12 bytes per key and row).
 * Errors: as clsa_route.
 */
size_t clsa_route_aggregated_workspace_size(int H, int B, int M, int d, int64_t n_cap, int k,
                                            int cap, clsa_dtype dt);
int clsa_route_aggregated(int H, const void* const* q_idx, const void* const* K_idx, int B, int M,
                          int d, int64_t n_cap, const int32_t* n_ctx, int64_t q_pos0, int k,
                          clsa_dtype dt, int32_t* idx, int32_t* counts, int cap, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * Centroid table router - decode routing through a table built at prefill.
 * (CSAttention summary, news.neo-ai.one: the queries of a long context
 * cluster, so centroids predict which keys matter; prefill builds a
 * fixed-size query-centroid lookup table per request and decoding consults
 * it instead of scanning the whole context.)
 *
 * clsa_csa_build: for each sequence b, Lloyd's k-means over its M prefill
 *   routing queries q_prefill [B][M][d] (bf16): centroid c starts at query
 *   floor(c M / C); `rounds` rounds of nearest-centroid assignment (squared
 *   Euclidean distance in fp32, ties to the lower centroid) and mean update
 *   (an empty cluster keeps its centroid).  centroids [B][C][d] (bf16,
 *   device, out) are the results rounded to bf16; table [B][C][T] (int32,
 *   device, out) row c lists the T keys of K_idx [B][n_cap][d] that centroid
 *   c scores highest, ascending (clsa_route's rules, over n_ctx[b] keys).
 *   M >= C, 1 <= C <= 1024 with C * d <= 16384, 1 <= T <= 2048,
 *   n_cap <= 512K, B * C <= 65535, rounds <= 100.
 * clsa_csa_route: for each sequence b (q_idx [B][d]): the P (1 <= P <= 16)
 *   centroids with the highest q . centroid (ties to the lower centroid);
 *   the candidates are the keys of their table rows plus every position in
 *   [n_table, n_ctx[b]) (keys appended since the table was built), keeping
 *   positions below n_ctx[b]; the list is the top-k of the candidates'
 *   exact scores (fp32 sums of exact products; ties to the lower position),
 *   ascending, -1 padded to cap; counts[b] = min(k, candidates).  The table
 *   is read as built by clsa_csa_build with the same B, d, C, T.
 *   P * T + (n_cap - n_table) <= 8192 (rebuild the table as the buffer of
 *   appended keys grows).
 * Both calls: bf16 only (CLSA_ERR_UNSUPPORTED_DTYPE otherwise); device
 * workspace of the matching *_workspace_size; errors CLSA_ERR_INVALID,
 * CLSA_ERR_WORKSPACE, CLSA_ERR_HIP.
 */
size_t clsa_csa_build_workspace_size(int B, int M, int d, int64_t n_cap, int C, int T);
int clsa_csa_build(const void* q_prefill, const void* K_idx, int B, int M, int d, int64_t n_cap,
                   const int32_t* n_ctx, int C, int rounds, int T, clsa_dtype dt, void* centroids,
                   int32_t* table, void* ws, size_t ws_bytes, void* stream);
size_t clsa_csa_route_workspace_size(int B, int d, int64_t n_cap, int C, int T, int P);
int clsa_csa_route(const void* q_idx, const void* K_idx, int B, int d, int64_t n_cap,
                   const int32_t* n_ctx, const void* centroids, const int32_t* table, int C, int T,
                   int64_t n_table, int P, int k, clsa_dtype dt, int32_t* idx, int32_t* counts,
                   int cap, void* ws, size_t ws_bytes, void* stream);

/*
 * clsa_kv_append - write one new token's rows into preallocated caches.
 * (CLSA explainer, section "CLSAの仕組み": the self-decoder writes the KV
 * cache that every cross-decoder layer then reads.)  This is that per-step
 * cache write, not part of routing or attention; it appends the routing key
 * row and every layer's K and V rows of each sequence in one launch.
 *
 *   pos     [B] int32, DEVICE: slot written in sequence b; sequences whose
 *           pos is outside [0, n_cap) are left untouched.
 *   src_idx [B][d] -> dst_idx [B][n_cap][d]   (both NULL: no routing key)
 *   src_k[l], src_v[l] [B][Hkv][D] -> K[l], V[l] [B][n_cap][Hkv][D],
 *           l < L (L = 0: routing key only).  Pointer arrays are HOST arrays.
 * Constraints: rows are 16-byte multiples (d*esize and Hkv*D*esize % 16 == 0).
 * Errors: CLSA_ERR_INVALID, CLSA_ERR_UNSUPPORTED_DTYPE, CLSA_ERR_HIP.
 */
int clsa_kv_append(int L, int B, int Hkv, int D, int d, int64_t n_cap, const int32_t* pos,
                   const void* src_idx, void* dst_idx, const void* const* src_k, void* const* K,
                   const void* const* src_v, void* const* V, clsa_dtype dt, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CLSA_H */
