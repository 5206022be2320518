/*
 * lrkv.h -- decode attention read directly from a low-rank-compressed KV cache,
 * for AMD Instinct MI355X (gfx950). Plain C ABI of liblrkv.so.
 *
 * What the library computes (sources are the pages' titles and sections):
 *
 *  - Palu: KV-Cache Compression with Low-Rank Projection (digest), Method details.
 *    Keys and values are cached as per-token latents h = x A (rank r per unit,
 *    a unit being a G-LRD group of s heads or, with s = 1, one KV head). At
 *    decode the keys are rebuilt on chip as K = H^k B^k, RoPE is applied at each
 *    token's position, and the query attends; the value reconstruction B^v is
 *    folded into W^o offline, so the output stays in latent space: o = p H^v.
 *    Without RoPE, B^k is absorbed into the query (q' = q (B^k)^T) and the
 *    scores are H^k q'. The Hadamard fold (A R)(R^T B) lets the latents be
 *    stored as int4 (per-token groups of 32, see the Supplementary details of
 *    the Palu digest, and section 5 of the Shard post for the symmetric [-7, 7]
 *    range).
 *  - PuzzleKV: page-based low-rank decomposition for KV-cache compression,
 *    section 3.3. Dense sink / local-window pages plus per-page factors
 *    X_hat = L R (Eq. 2), obtained from the P x P Gram matrix; attention runs
 *    over dense and factored pages and merges them by online softmax; a page is
 *    factored once it is full and has left the window.
 *
 * Conventions for every entry point:
 *  - Ownership: the caller owns every buffer (device memory, e.g. PyTorch
 *    tensors). The library allocates nothing; scratch memory is the caller's
 *    `workspace`, sized by lrkv_decode_workspace_bytes (lrkv_decode_attn_noalloc
 *    uses a static device array instead).
 *  - Pointers marked "device" must be device memory of the current HIP device.
 *  - Asynchrony: calls only enqueue kernels on `stream` (a hipStream_t; NULL is
 *    the default stream) and never synchronise. Results are ready when the
 *    stream reaches them.
 *  - Errors: arguments are validated on the host before anything is enqueued;
 *    a failing call returns a negative lrkv_status and leaves device memory
 *    untouched. A failed kernel launch returns LRKV_ERR_HIP. No C++ exception
 *    crosses the ABI.
 *  - Thread safety: calls are re-entrant; the library keeps no global state
 *    beyond its loaded code objects, except the static scratch array of
 *    lrkv_decode_attn_noalloc and its per-device address.
 *  - Lengths: `lens` (device, int32 [batch]) holds each sequence's current
 *    number of cached tokens; `host_max_len` is the caller's host-side bound on
 *    max(lens) (used for capacity checks and grid sizing; it must not be
 *    smaller than the true maximum).
 */
#ifndef LRKV_H
#define LRKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LRKV_OK = 0,
    LRKV_ERR_INVALID_ARG = -1,   /* null pointer, bad size or shape                  */
    LRKV_ERR_UNSUPPORTED = -2,   /* valid but not compiled: rank / head_dim / groups */
    LRKV_ERR_CAPACITY = -3,      /* the append would overflow the cache              */
    LRKV_ERR_WORKSPACE = -4,     /* workspace missing or too small                   */
    LRKV_ERR_HIP = -5,           /* a HIP call failed                                */
    LRKV_ERR_SCRATCH = -6        /* more than lrkv_decode_attn_noalloc's static
                                    scratch (LRKV_NOALLOC_SCRATCH_BYTES) needed      */
} lrkv_status;

typedef enum {
    LRKV_FMT_FP16 = 0,           /* latents stored as fp16                            */
    LRKV_FMT_INT4_G32 = 1        /* symmetric int4 codes, one fp16 scale per 32 dims  */
} lrkv_fmt;

typedef enum {
    LRKV_MODE_ROPE_RECON = 0,    /* rebuild K = H^k B^k per tile, RoPE, attend        */
    LRKV_MODE_ABSORBED = 1,      /* no RoPE: scores = H^k q', q' given by the caller  */
    LRKV_MODE_HYBRID_PAGED = 2   /* dense + factored pages (PuzzleKV)                 */
} lrkv_mode;

/* Tokens per cache block of the value layout and per attention tile. */
#define LRKV_BLOCK 32

/*
 * Latent cache (Palu modes). Query head j (of Hq = units * s * g_q) reads KV
 * head k = j / g_q, which is column block (k % s) of unit k / s.
 *
 * Layouts (all device memory, caller-owned, `capacity` a multiple of 32):
 *   fp16:  hk  [batch][units][capacity][rank]               half, token-major
 *          hv  [batch][units][capacity/32][rank][32]        half, each 32-token
 *                                                          block stored dim-major
 *   int4:  hk  [batch][units][capacity][rank/2]             uint8; dims 2i and 2i+1
 *                                                          in the low / high nibble
 *          sk  [batch][units][capacity][rank/32]            half scales
 *          hv  [batch][units][capacity/32][rank][16]        uint8; within a block,
 *                                                          tokens 2i and 2i+1 of one
 *                                                          dim in the low / high nibble
 *          sv  [batch][units][capacity/32][rank/32][32]     half scales, token-minor
 *   Codes are 4-bit two's complement in [-7, 7]; value = code * scale.
 */
typedef struct lrkv_latent_cache {
    int32_t batch;        /* B                                                  */
    int32_t units;        /* U: G-LRD groups, or KV heads when kv_per_unit = 1  */
    int32_t kv_per_unit;  /* s: KV heads rebuilt from one unit's latents        */
    int32_t q_per_kv;     /* g_q: query heads per KV head (GQA)                 */
    int32_t head_dim;     /* d_h                                                */
    int32_t rank;         /* r: latent width per unit                           */
    int32_t capacity;     /* tokens per sequence (multiple of 32)               */
    int32_t fmt;          /* lrkv_fmt                                           */
    float rope_theta;     /* RoPE base; 0 disables RoPE                         */
    void *hk, *hv;        /* key / value latents (layouts above)                */
    void *sk, *sv;        /* int4 scales; NULL for fp16                         */
    int32_t *lens;        /* device int32 [batch]                               */
} lrkv_latent_cache;

/*
 * Hybrid paged cache (PuzzleKV). Page p of a sequence holds tokens
 * [p*P, (p+1)*P). page_table[b][h][p] >= 0: the page is factored and its
 * factors sit at that slot of lk/rk/lv/rv; < 0: the page is dense and sits in
 * dense slot (-1 - entry); LRKV_PAGE_EMPTY: not written yet. Dense slots: sink
 * page p < sink_pages uses slot p; any other dense page uses slot
 * sink_pages + (p - sink_pages) % window_pages.
 *
 *   dense_k     [batch][kv_heads][sink_pages+window_pages][P][head_dim]  half
 *   dense_v     [batch][kv_heads][sink_pages+window_pages][head_dim][P]  half
 *   lk          [batch][kv_heads][max_pages][P][rank_k]                  half  L_K
 *   rk          [batch][kv_heads][max_pages][rank_k][head_dim]           half  R_K
 *   lv          [batch][kv_heads][max_pages][rank_v][P]                  half  L_V^T
 *   rv          [batch][kv_heads][max_pages][head_dim][rank_v]           half  R_V^T
 *   page_table  [batch][kv_heads][max_pages]                             int32
 *
 * factor_fmt LRKV_FMT_INT4_G32 (PuzzleKV, Abstract and the contributions list
 * of section 1: per-factor INT4 quantisation; ranks up to 16): lk/rk/lv hold
 * the factors' codes in the element order above and rv in rank quads, R_V^T as [rank_v/4][head_dim][4], two codes per
 * byte (element 2i in the low nibble); lk_s/rk_s/lv_s/rv_s hold one fp16
 * scale per 32 consecutive elements of one page's factor, [batch][kv_heads]
 * [max_pages][elements / 32], with the latent codec of lrkv_append_latent
 * (symmetric codes in [-7, 7], s16 = fp16(amax / 7)). lrkv_factor_page
 * quantises L first and forms R = L_hat^T X from the dequantised L_hat. The
 * code arrays must be 16-byte aligned (INVALID_ARG otherwise).
 *
 * A factored page holds X_hat = L R (PuzzleKV Eq. 2: L = the page's top left
 * singular vectors, R = Sigma W^T). Key-side arrays are stored as L and R, the
 * value side transposed (dimension-major), as are the dense values: each decode
 * product then reads a contiguous run of its contraction index. Supported:
 * head_dim 128, P 32, q_per_kv <= 16, ranks multiples of 4 up to 32,
 * max_pages <= 65536 (LRKV_ERR_UNSUPPORTED otherwise).
 */
#define LRKV_PAGE_EMPTY ((int32_t)0x80000000)

typedef struct lrkv_paged_cache {
    int32_t batch, kv_heads, q_per_kv, head_dim;
    int32_t page_size;    /* P                                                  */
    int32_t sink_pages, window_pages;
    int32_t rank_k, rank_v;
    int32_t max_pages;    /* pages per sequence (capacity = max_pages * P)      */
    void *dense_k, *dense_v;
    void *lk, *rk, *lv, *rv;
    int32_t *page_table;  /* device                                             */
    int32_t *lens;        /* device int32 [batch]                               */
    int32_t factor_fmt;   /* lrkv_fmt of lk/rk/lv/rv (dense pages stay fp16)    */
    void *lk_s, *rk_s, *lv_s, *rv_s;   /* int4 factor scales; NULL for fp16     */
} lrkv_paged_cache;

/* Human-readable name of a status code (static string). */
const char *lrkv_status_string(int32_t status);

/* ABI version (major * 100 + minor). */
int32_t lrkv_version(void);

/*
 * Bytes of workspace lrkv_decode_attn needs for this cache, length bound and
 * split count (n_split <= 0 picks the library's default). Returns 0 when the
 * arguments are invalid. `cache` points to an lrkv_latent_cache for the Palu
 * modes and to an lrkv_paged_cache for LRKV_MODE_HYBRID_PAGED.
 */
size_t lrkv_decode_workspace_bytes(int32_t mode, const void *cache, int32_t host_max_len,
                                   int32_t n_split);

/*
 * Append n_new tokens to every sequence: token i of sequence b is written at
 * position lens[b] + i, then lens[b] += n_new.
 *
 * Defined by: Palu digest, Method details (the cache holds the latents h = x A
 * instead of the keys and values; the Hadamard fold (A R)(R^T B) and, in the
 * Supplementary details, per-token quantisation groups) and the Shard post,
 * section 5, step 4 (symmetric int4 codes in [-7, 7]); for the hybrid cache,
 * PuzzleKV section 3.3, step 5 (a new key/value pair goes to the newest dense
 * page).
 *
 * Palu modes (cache = lrkv_latent_cache*): new_k, new_v are device float32
 * [batch][units][n_new][rank] latents h = x A (in the Hadamard-mixed basis for
 * int4 caches). fp16 caches store round-to-nearest-even fp16. int4 caches
 * quantise each token's 32-element groups: s = fp16_rne(fp32(amax) / 7)
 * (+inf saturates to 65504), code = clamp(round_half_even(x / s), -7, 7) with
 * the quotient formed in fp64; s == 0 gives zero codes.
 *
 * Hybrid mode (cache = lrkv_paged_cache*): new_k, new_v are device fp16
 * [batch][kv_heads][n_new][head_dim]. A token is written to its page's dense
 * slot unless the page is already factored (then it is skipped: prefill
 * factors those pages from the caller's buffer first). Before a token reuses a
 * window slot, the page that owned it must have been factored
 * (lrkv_factor_page); the first token of a page records the dense slot in the
 * page table.
 *
 * Errors: INVALID_ARG (null pointers, n_new < 1, bad shapes), UNSUPPORTED
 * (rank not a multiple of 32 for int4, unsupported sizes), CAPACITY
 * (host_max_len + n_new exceeds the capacity). The capacity check uses the
 * caller's host_max_len; should it be stale (below a device length), the
 * kernels still write nothing at or past the capacity (or past max_pages in
 * the hybrid cache): such tokens are dropped, although lens still advances.
 */
int32_t lrkv_append_latent(int32_t mode, const void *cache, const void *new_k, const void *new_v,
                           int32_t n_new, int32_t host_max_len, void *stream);

/*
 * Single-query decode attention for every sequence and query head.
 *
 * Defined by: Palu digest, Method details (K = H^k B^k rebuilt on chip, RoPE
 * applied to the rebuilt keys before the query attends, B^v fused into W^o so
 * that the output is o = p H^v; without RoPE, key fusion q' = q (B^k)^T and
 * scores H^k q') and Background (multi-head attention); PuzzleKV section 3.2,
 * Eq. 1 (softmax attention) and section 3.3, step 4 (attention over dense and
 * factored pages, factored pages scored as (q R^T) L^T, partial results merged
 * by online softmax).
 *
 * LRKV_MODE_ROPE_RECON: q device float32 [batch][Hq][head_dim], un-rotated;
 *   bk device fp16 [units][rank][kv_per_unit*head_dim] (B^k, or the
 *   Hadamard-mixed R^T B^k for int4 caches); q_pos device int32 [batch] query
 *   positions (NULL: lens[b] - 1). Keys of token t are rotated at position t,
 *   the query at q_pos. out: device float32 [batch][Hq][rank], o = p H^v.
 * LRKV_MODE_ABSORBED: q device float32 [batch][Hq][rank] absorbed queries
 *   q' = q (B^k)^T; bk and q_pos must be NULL; rope_theta is ignored.
 *   out: float32 [batch][Hq][rank].
 * LRKV_MODE_HYBRID_PAGED: q device float32 [batch][Hq][head_dim]; bk, q_pos
 *   NULL; out float32 [batch][Hq][head_dim].
 *
 * sm_scale: softmax scale (<= 0 selects 1/sqrt(head_dim)). n_split: number of
 * sequence chunks attended in parallel and merged by online softmax (<= 0:
 * library default); the result does not depend on it beyond rounding.
 * Every lens[b] must be >= 1.
 *
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE (ws_bytes smaller than
 * lrkv_decode_workspace_bytes for the same arguments).
 */
int32_t lrkv_decode_attn(int32_t mode, const void *cache, const float *q, const void *bk,
                         const int32_t *q_pos, float sm_scale, float *out, void *workspace,
                         size_t ws_bytes, int32_t host_max_len, int32_t n_split, void *stream);

/*
 * One decode step: lrkv_append_latent(mode, cache, new_k, new_v, n_new,
 * host_max_len) followed by lrkv_decode_attn(mode, cache, q, bk, q_pos,
 * sm_scale, out, workspace, ws_bytes, host_max_len + n_new, n_split), with the
 * same results, bit for bit, and the same cache contents and lens afterwards.
 * host_max_len bounds the lengths before the append; the workspace is sized as
 * lrkv_decode_workspace_bytes(mode, cache, host_max_len + n_new, n_split);
 * q_pos NULL is each sequence's newest token after the append.
 *
 * Defined by: the two calls it combines (Palu digest, Method details: new
 * tokens enter the cache as latents, then the query attends over all of them).
 *
 * With the RoPE mode and a decode-size append (fp16: at most 1024 new 8-element
 * rows, batch * units * n_new * rank / 8; int4: at most 1024 key groups plus
 * value token-pair groups, batch * units * (n_new + n_new / 2 + 2) * rank / 32)
 * the append runs inside the query preparation's launch and lens advances in
 * the merge's: three launches instead of four (six with int4). Other modes and
 * sizes enqueue the append and the decode in turn.
 *
 * Errors: those of the two calls; every check of both is made before anything
 * is enqueued, so a rejected call leaves the cache, lens and out unchanged.
 */
int32_t lrkv_decode_step(int32_t mode, const void *cache, const void *new_k, const void *new_v,
                         int32_t n_new, const float *q, const void *bk, const int32_t *q_pos,
                         float sm_scale, float *out, void *workspace, size_t ws_bytes,
                         int32_t host_max_len, int32_t n_split, void *stream);

/*
 * lrkv_decode_attn for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * same validation, kernels and result as lrkv_decode_attn with the same
 * arguments, but the workspace is a static device array of
 * LRKV_NOALLOC_SCRATCH_BYTES inside the library instead of a caller buffer.
 * The caller still passes the cache, q, bk, q_pos and out; the call performs no
 * allocation of any kind.
 *
 * Each device the library runs on holds its own copy of the array until the
 * process ends; its address is looked up once per device, on the first call
 * made with that device current. The array keeps the last call's contents
 * (nothing in it needs clearing between calls). All calls on one device share
 * it, so two calls whose executions overlap on that device (different streams,
 * or host threads without ordering) race and give undefined results: order
 * them on one stream.
 *
 * Errors: as lrkv_decode_attn, except that a call whose workspace
 * (lrkv_decode_workspace_bytes for the same arguments) exceeds
 * LRKV_NOALLOC_SCRATCH_BYTES returns LRKV_ERR_SCRATCH before anything is
 * enqueued; LRKV_ERR_HIP if the array's address cannot be obtained.
 */
#define LRKV_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int32_t lrkv_decode_attn_noalloc(int32_t mode, const void *cache, const float *q, const void *bk,
                                 const int32_t *q_pos, float sm_scale, float *out,
                                 int32_t host_max_len, int32_t n_split, void *stream);

/*
 * The three steps lrkv_decode_attn enqueues, callable one by one with the same
 * cache, workspace, host_max_len and n_split (lrkv_decode_attn is exactly
 * prepare + partials + merge). Splitting them lets a caller time each step, or
 * exchange the per-chunk partial states before merging (e.g. when the
 * sequence is sharded over several devices).
 *
 * lrkv_decode_prepare: query preparation. RoPE mode: combines q (un-rotated,
 *   float32 [batch][Hq][head_dim]) with bk, and builds the RoPE angle tables for
 *   q_pos (NULL: lens[b] - 1), in the workspace; other modes: nothing to do
 *   (returns LRKV_OK after validation).
 * lrkv_decode_partials: streams the cache chunk by chunk and writes each
 *   chunk's softmax state (running max, running sum, unnormalised output) to
 *   the workspace. RoPE mode reads what prepare wrote (q may be NULL); the
 *   absorbed and hybrid modes read q and sm_scale.
 * lrkv_merge_partials: merges the chunk states by online softmax into out.
 *
 * Errors as for lrkv_decode_attn.
 */
int32_t lrkv_decode_prepare(int32_t mode, const void *cache, const float *q, const void *bk,
                            const int32_t *q_pos, float sm_scale, void *workspace, size_t ws_bytes,
                            int32_t host_max_len, int32_t n_split, void *stream);
int32_t lrkv_decode_partials(int32_t mode, const void *cache, const float *q, float sm_scale,
                             void *workspace, size_t ws_bytes, int32_t host_max_len,
                             int32_t n_split, void *stream);
int32_t lrkv_merge_partials(int32_t mode, const void *cache, float *out, void *workspace,
                            size_t ws_bytes, int32_t host_max_len, int32_t n_split, void *stream);

/*
 * Defined by: PuzzleKV section 3.3, Eq. 2 (a page X ~ L R with L = U_r, the
 * top-r left singular vectors, and R = Sigma_r W_r^T) and the Gram route of the
 * same section (the top-r eigenvectors of the P x P matrix X X^T are U_r, so
 * R = U_r^T X), with step 5 (a page is factored once it is full and has left
 * the local window); the truncation is the Eckart-Young optimum of section 3.2.
 *
 * Factor pages of a hybrid cache: for each (b, kv_head, page) triple in
 * `pages` (device int32 [n_pages][3]) and for K and V separately, form the
 * Gram matrix G = X X^T of the P x head_dim page X, take its top-r eigenvectors
 * Q_r (cyclic Jacobi in fp32, at most max_sweeps sweeps, <= 0: 15), store
 * L = Q_r and R = Q_r^T X as fp16 in factor slot `page`, and set the page-table
 * entry to `page`.
 *
 * src_k / src_v NULL: X is read from the page's dense slot (decode path; a
 * triple whose entry is not dense is skipped). Otherwise X is read from the
 * caller's device fp16 [batch][kv_heads][src_len][head_dim] buffers (prefill
 * path; the page must satisfy (page+1)*P <= src_len). Triples out of range are
 * skipped.
 *
 * Errors: INVALID_ARG (null cache/pages, n_pages < 0, bad shapes),
 * UNSUPPORTED (page_size != 32 or ranks outside 1..32).
 */
int32_t lrkv_factor_page(const lrkv_paged_cache *cache, const int32_t *pages, int32_t n_pages,
                         const void *src_k, const void *src_v, int32_t src_len,
                         int32_t max_sweeps, void *stream);

/*
 * Host-side planner for the hybrid cache (no device access, no launch): list
 * the (b, kv_head, page) triples that become factored when n_new tokens are
 * appended to sequences whose current lengths are host_lens[0..batch) (host
 * memory): pages p with sink_pages <= p < ceil((len + n_new) / P) -
 * window_pages that were not already factored at length len (PuzzleKV section
 * 3.3, step 5: a page is factored once it is full and has left the window).
 * Writes at most max_out triples to out (host int32 [max_out][3], ordered by b,
 * kv_head, page) and returns how many there are in total (which may exceed
 * max_out), or a negative lrkv_status on invalid arguments.
 *
 * Decode (n_new = 1): factor the returned pages (src NULL) before appending.
 * Prefill (every len = 0): factor them from the caller's dense buffer, then
 * append all tokens; the append skips tokens of factored pages.
 */
int32_t lrkv_paged_plan(const lrkv_paged_cache *cache, const int32_t *host_lens, int32_t n_new,
                        int32_t *out, int32_t max_out);

/*
 * Chunked-prefill attention on the reconstruct-with-RoPE path (Palu digest,
 * Method details: K = H^k B^k rebuilt on chip, RoPE at each side's position,
 * latent-space output o = p H^v). The m_tokens new tokens of each sequence
 * must already be appended (lrkv_append_latent): token m of sequence b sits at
 * position p0[b] + m, and its queries attend causally to tokens 0 .. p0[b] + m
 * (positions are clamped to 0 .. lens[b] - 1). Arithmetic: the rotated
 * queries and the rebuilt, rotated keys are each rounded once to fp16 for the
 * score products, p once to fp16 for the value product; accumulation in fp32.
 *
 *   cache    lrkv_latent_cache with fp16 latents, rank 256, head_dim 128 (any
 *            kv_per_unit and q_per_kv; LRKV_ERR_UNSUPPORTED otherwise)
 *   q        device float32 [batch][m_tokens][Hq][head_dim], un-rotated queries
 *   bk       device fp16 [units][rank][kv_per_unit * head_dim] (B^k)
 *   p0       device int32 [batch], the chunk's first position per sequence
 *   host_max_len  the host's bound on p0[b] + m_tokens (1 .. capacity): sizes
 *            the angle table and the key range
 *   sm_scale softmax scale (<= 0 selects 1/sqrt(head_dim))
 *   out      device float32 [batch][m_tokens][Hq][rank], 16-byte aligned
 *   workspace device, at least lrkv_prefill_workspace_bytes(cache, m_tokens,
 *            host_max_len) bytes (rotated queries and fp64-reduced angle tables),
 *            else LRKV_ERR_WORKSPACE
 *
 * Enqueued on `stream`; nothing is allocated. INVALID_ARG for null or unaligned
 * pointers and out-of-range sizes. lrkv_prefill_workspace_bytes returns 0 for
 * invalid or unsupported arguments.
 */
size_t lrkv_prefill_workspace_bytes(const lrkv_latent_cache *cache, int32_t m_tokens, int32_t host_max_len);
int32_t lrkv_prefill_attn(const lrkv_latent_cache *cache, const float *q, const void *bk, const int32_t *p0,
                          int32_t m_tokens, int32_t host_max_len, float sm_scale, float *out, void *workspace,
                          size_t ws_bytes, void *stream);

/*
 * The projections on either side of the decode path (Palu digest, Method
 * details: a token is cached as its latents h = x A, and the value
 * up-projection B^v is fused offline into W^o, so the layer output is
 * y = sum_j o_j (B^v_j W^o_j) with o_j the latent-space output of head j).
 * Both compute C[M][N] = X[M][K] W^T[N][K]^T with fp32 X and C and fp16
 * weights W^T stored with K contiguous (row-major [N][K]); all pointers are
 * device memory, 16-byte aligned; K must be a multiple of 32 and N of 16
 * (LRKV_ERR_UNSUPPORTED otherwise). The partial sums of the K split go to the
 * caller's `workspace` (device, at least lrkv_project_workspace_bytes(M, N, K)
 * bytes, else LRKV_ERR_WORKSPACE); their final sum is in a fixed order, so a
 * call is deterministic. Enqueued on `stream`; nothing is allocated.
 *
 * lrkv_latent_project: x [n_tok][d_model] (one token per row), a_t
 *   [units * rank][d_model] = (A_u)^T of each unit stacked, h [n_tok][units][rank]
 *   (for one new token per sequence this is lrkv_append_latent's new_k / new_v
 *   layout). M = n_tok, K = d_model, N = units * rank.
 * lrkv_output_project: o [batch][q_heads][rank] (lrkv_decode_attn's output in
 *   the Palu modes), w_t [d_model][q_heads * rank] with column j * rank + i =
 *   row i of head j's fused B^v_j W^o_j, y [batch][d_model].
 *   M = batch, K = q_heads * rank, N = d_model.
 * lrkv_project_workspace_bytes: 0 for invalid sizes.
 */
size_t lrkv_project_workspace_bytes(int32_t m, int32_t n, int32_t k);
int32_t lrkv_latent_project(const float *x, int32_t n_tok, int32_t d_model, const void *a_t, int32_t units,
                            int32_t rank, float *h, void *workspace, size_t ws_bytes, void *stream);
int32_t lrkv_output_project(const float *o, int32_t batch, int32_t q_heads, int32_t rank, const void *w_t,
                            int32_t d_model, float *y, void *workspace, size_t ws_bytes, void *stream);

/*
 * Measurement aid, not part of the decode path: reads `bytes` (a multiple of
 * 16) of device memory `buf` once with a streaming kernel of `blocks`
 * workgroups (1..65535) and writes one word per workgroup to device `out`
 * (uint32 [blocks]). Its duration is the practical HBM read rate the decode
 * kernels are compared against, beside the nominal peak. LRKV_ERR_INVALID_ARG
 * on a NULL or unaligned buffer, a size not a multiple of 16 or a bad block
 * count.
 */
int32_t lrkv_probe_stream_read(const void *buf, size_t bytes, uint32_t *out, int32_t blocks,
                               void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LRKV_H */
