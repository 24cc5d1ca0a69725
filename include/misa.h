/*
 * misa.h -- C ABI of the MISA (Mixture of Indexer Sparse Attention) indexer
 * for AMD Instinct MI355X (gfx950).
 *
 * The indexer picks, for every query token, the top-k prefix tokens that
 * DSA-style sparse attention will attend to.  MISA replaces the dense
 * all-head DSA indexer with four stages (gist.science technical summary of
 * "MISA: Mixture of Indexer Sparse Attention for Long-Context LLM Inference",
 * "Metodologia: MISA" items 1-2; agents-report summary, method overview):
 *
 *   misa_pool_keys          block mean-pooling of the shared indexer keys
 *   misa_route_heads        block-summary router: top-h indexer heads per query
 *   misa_sparse_head_logits token scoring with the routed heads only
 *   misa_topk               per-query top-k token selection
 *
 * plus the whole pipeline (misa_indexer, optionally the hierarchical
 * MISA-dagger variant of "Variante Hierárquica (MISA†)") and the dense DSA
 * indexer that MISA replaces (dsa_dense_logits; the baseline path named in
 * the GitHub issue "Clarification on the Figure 3 baseline ...").
 *
 * Token score (the DSA indexer score, DeepSeek-V3.2 lightning indexer):
 *     I[t, s] = sum_{j in heads(t)} w[t, j] * ReLU(q[t, j] . k[s] * sigma[s])
 * for every prefix key s <= t, and -inf for s > t.  sigma[s] is the per-token
 * scale of an fp8 key cache and 1 for bf16 keys.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory   All tensor pointers are DEVICE pointers owned by the caller.  The
 *          library never allocates, frees or synchronises; scratch space comes
 *          from a caller-provided workspace (misa_indexer_noalloc: from a fixed
 *          device buffer of the library).  Every tensor is densely
 *          packed in the layout given (row-major, last index fastest) and
 *          16-byte aligned.
 * Streams  `stream` is a hipStream_t passed as void* (NULL = the default
 *          stream).  Every call only enqueues work on it and returns.
 * Errors   Arguments are checked on the host before anything is enqueued; a
 *          bad argument returns a negative misa_status and enqueues nothing.
 *          A failed kernel launch returns MISA_ERR_HIP.  No C++ exception
 *          crosses this interface.  The only global state is the per-device
 *          address of misa_indexer_noalloc's fixed scratch (looked up once
 *          under a lock), so calls from several host threads are safe, except
 *          that misa_indexer_noalloc calls sharing one GPU must not overlap.
 * Numerics Preconditions that are documented, not checked: inputs are finite;
 *          fp8 scales are > 0.  Accumulation is fp32.
 * Shapes   A call covers n_seq independent sequences.  Sequence b has n_keys
 *          keys (positions 0..n_keys-1) and q_per_seq queries; query i of a
 *          sequence sits at absolute position t = q_pos0 + i and sees the keys
 *          0..t (causal).  Prefill chunk: n_seq = 1, q_pos0 = n_keys - M.
 *          Decode batch: q_per_seq = 1, q_pos0 = n_keys - 1.
 * Blocks   Block m covers key positions [m*B, (m+1)*B).  For query t the
 *          prefix holds floor((t+1)/B) complete blocks and, when (t+1) % B != 0,
 *          one partial block [floor((t+1)/B)*B, t] (its "tail").
 */
#ifndef MISA_H
#define MISA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MISA_OK = 0,
  MISA_ERR_INVALID_ARG = -1,   /* null pointer, bad size, bad alignment */
  MISA_ERR_UNSUPPORTED = -2,   /* a valid request outside what is implemented */
  MISA_ERR_WORKSPACE = -3,     /* workspace missing or too small */
  MISA_ERR_HIP = -4,           /* a HIP runtime call or kernel launch failed */
  MISA_ERR_SCRATCH = -5        /* misa_indexer_noalloc: more scratch needed than
                                  MISA_NOALLOC_SCRATCH_BYTES */
} misa_status;

typedef enum {
  MISA_K_BF16 = 0,             /* k: uint16 bf16 bits [n_seq][n_keys][128] */
  MISA_K_FP8_E4M3 = 1          /* k: uint8 OCP e4m3fn codes [n_seq][n_keys][128],
                                  k_scale: float [n_seq][n_keys], > 0 */
} misa_kdtype;

typedef struct {
  int32_t n_seq;      /* independent sequences, >= 1 */
  int32_t q_per_seq;  /* M: queries per sequence, >= 0 (0 = nothing to do) */
  int64_t n_keys;     /* N: keys per sequence, 1..2^26 (larger: MISA_ERR_UNSUPPORTED) */
  int64_t q_pos0;     /* position of query 0; 0 <= q_pos0 and q_pos0 + M <= N */
  int32_t n_heads;    /* H: indexer heads (H_I on the pages), 1..64 */
  int32_t head_dim;   /* d: must be 128 */
  int32_t block;      /* B: pooling block size, >= 1 */
} misa_shape;

#define MISA_HEAD_DIM 128
#define MISA_MAX_HEADS 64
#define MISA_MAX_TOPK 8192

/* Human-readable name of a status code (static string, never NULL). */
const char* misa_status_str(misa_status s);

/*
 * Block mean-pooling of the shared indexer keys (gist.science summary,
 * "Metodologia: MISA" item 1: mean-pooled indexer keys per block;
 * agents-report: one summary key per block of the prefix).
 *   pooled[b][m][:] = mean(key[b][m*B .. m*B+B-1][:])   for m < floor(N/B)
 *   tail[b][i][:]   = mean(key[b][floor((t+1)/B)*B .. t][:]),  t = q_pos0+i,
 *                     or all zeros when (t+1) % B == 0 (no partial block).
 * key = bf16 value, or e4m3 value * k_scale.  fp32 sums in key order.
 * k: see misa_kdtype.  k_scale: NULL for bf16, required for fp8.
 * pooled: float [n_seq][floor(N/B)][128] (not touched when floor(N/B) = 0).
 * tail:   float [n_seq][M][128].
 */
misa_status misa_pool_keys(const misa_shape* shape, const void* k, misa_kdtype kdtype,
                           const float* k_scale, float* pooled, float* tail, void* stream);

/*
 * Head router (gist.science summary, "Metodologia: MISA" item 1: per-head
 * affinities against the pooled keys, aggregated into a per-head importance,
 * top-h heads kept; agents-report: MISA aggregates along the blocks to pick
 * heads).  For query t of sequence b and head j:
 *   S[j] = sum_{m < floor((t+1)/B)} ReLU(q[t,j] . pooled[m]) + ReLU(q[t,j] . tail[t])
 *          (the tail term only when the partial block is non-empty)
 *   r[j] = w[t,j] * S[j]
 *   heads[b][i][:] = the h heads with the largest r (equal r -> lower head id),
 *                    stored in ascending head order.
 * q: uint16 bf16 bits [n_seq][M][H][128].  w: float [n_seq][M][H].
 * pooled, tail: as written by misa_pool_keys.  1 <= h <= H.
 * heads: int32 [n_seq][M][h].  scores: float [n_seq][M][H] receives r, or NULL.
 */
misa_status misa_route_heads(const misa_shape* shape, const uint16_t* q, const float* w,
                             const float* pooled, const float* tail, int32_t h,
                             int32_t* heads, float* scores, void* stream);

/*
 * Token scoring with the routed heads only (gist.science summary,
 * "Metodologia: MISA" item 2: only the h active heads score the whole prefix
 * token by token).
 *   logits[b][i][s] = sum_{j in heads[b][i]} w[t,j] * ReLU(q[t,j] . k[s] * sigma[s])
 *                     for s <= t,   -inf for t < s < N.   Columns N..roundup4(N)-1
 *                     may also be set to -inf; columns roundup4(N)..ld-1 are untouched.
 * heads: int32 [n_seq][M][h], ascending, distinct, each in [0, H).  1 <= h <= H.
 * logits: float [n_seq][M][ld]; ld >= N, ld % 4 == 0 and ld <= 2^27 (larger:
 *         MISA_ERR_UNSUPPORTED; row offsets of a 4-row group stay 32-bit).
 */
misa_status misa_sparse_head_logits(const misa_shape* shape, const uint16_t* q, const float* w,
                                    const void* k, misa_kdtype kdtype, const float* k_scale,
                                    const int32_t* heads, int32_t h, float* logits, int64_t ld,
                                    void* stream);

/*
 * The dense DSA indexer: the token score with all H heads (the baseline MISA
 * replaces; the abstract of arXiv 2605.07363 and the GitHub issue's dense
 * all-head path).
 * cand == NULL:  logits[b][i][s] over every key, exactly as
 *                misa_sparse_head_logits with heads = 0..H-1 (and bitwise equal
 *                to it); ld >= N, ld % 4 == 0, ld <= 2^27.
 * cand != NULL:  re-rank mode of MISA-dagger ("Variante Hierárquica (MISA†)":
 *                the original all-head indexer re-scores only the candidates).
 *                cand: int32 [n_seq][M][n_cand] token ids (any order; -1 = no
 *                candidate); logits[b][i][c] = score of token cand[b][i][c]
 *                (-inf where cand < 0); ld >= n_cand, ld % 4 == 0.  Every
 *                candidate id must be in [0, t].  Each value is bitwise equal
 *                to the cand == NULL value of the same (query, token).
 */
misa_status dsa_dense_logits(const misa_shape* shape, const uint16_t* q, const float* w,
                             const void* k, misa_kdtype kdtype, const float* k_scale,
                             const int32_t* cand, int32_t n_cand, float* logits, int64_t ld,
                             void* stream);

/*
 * Per-query top-k token selection (the selection step after scoring; the
 * issue's pipeline runs it as a separate top-k over the returned logits).
 * Order: value descending; equal values (with -0.0 == +0.0) -> lower token id.
 * cand == NULL:  row i of sequence b considers columns s in [0, min(n_cols, t+1));
 *                the token id is the column.
 * cand != NULL:  row considers columns c in [0, n_cols) with cand[b][i][c] >= 0;
 *                the token id is cand[b][i][c] (ids distinct within a row).
 * sorted != 0: idx lists the selection in that order.  sorted == 0: the same set in an
 *                unspecified order (enough for a candidate list), cheaper.
 * idx:  int32 [n_seq][M][k]; rows with fewer than k candidates are padded with -1 (the
 *       padding always comes last).
 * vals: float [n_seq][M][k] (the selected values, -inf padding), or NULL.
 * 1 <= k <= MISA_MAX_TOPK.  logits: float [n_seq][M][ld], ld % 4 == 0, ld >= n_cols.
 * ws / ws_bytes: workspace of at least misa_topk_workspace_bytes() bytes
 *                (may be NULL when that is 0).
 */
misa_status misa_topk(const misa_shape* shape, const float* logits, int64_t ld,
                      const int32_t* cand, int32_t n_cols, int32_t k, int32_t sorted,
                      int32_t* idx, float* vals, void* ws, size_t ws_bytes, void* stream);

size_t misa_topk_workspace_bytes(const misa_shape* shape, int32_t n_cols, int32_t k);

/*
 * Routed-head scoring and top-k token selection in one call, without
 * materialising the logits where that can be avoided (the fused scoring ->
 * top-k the GitHub issue asks for as a "fused MISA kernel").  The result is
 * exactly misa_topk(misa_sparse_head_logits(...), topk, sorted): same ids,
 * same values, same order (sorted != 0) or the same set (sorted == 0).
 * When h <= 8, topk <= 8192 and every query's prefix has at least
 * max(16384, 4 topk) keys, the scores of
 * a key sample (every kstride-th key, kstride >= 32) give each row a
 * threshold; the routed scoring keeps only the scores at or above it, as
 * candidates, and the exact top-k is taken over them.  A row whose
 * candidates fall short of topk (or overflow their buffers) is re-scored into
 * full logits in the workspace and selected from them, so the result does
 * not depend on the sample.  Otherwise the logits are materialised in the
 * workspace and misa_topk runs on them.
 * heads: int32 [n_seq][M][h], as misa_sparse_head_logits.  idx / vals: as
 * misa_topk.  1 <= topk <= MISA_MAX_TOPK.
 * ws / ws_bytes: at least misa_sparse_head_topk_workspace_bytes() bytes.
 */
misa_status misa_sparse_head_topk(const misa_shape* shape, const uint16_t* q, const float* w,
                                  const void* k, misa_kdtype kdtype, const float* k_scale,
                                  const int32_t* heads, int32_t h, int32_t topk, int32_t sorted,
                                  int32_t* idx, float* vals, void* ws, size_t ws_bytes, void* stream);

/* Workspace of misa_sparse_head_topk for keys of type kdtype (fp8 keys add a
 * bf16 copy of the keys, widened exactly once per call for the scoring's
 * direct global -> LDS staging); 0 for an invalid shape. */
size_t misa_sparse_head_topk_workspace_bytes(const misa_shape* shape, misa_kdtype kdtype, int32_t h,
                                             int32_t topk);

/*
 * fp8 path.  The pages' indexer runs on fp8 inputs, and the GitHub issue on
 * the vLLM kernel ("Clarification on the Figure 3 baseline and plans for an
 * optimized vLLM MISA kernel", second question) asks for an fp8 MISA kernel
 * that avoids widening fp8 to bf16.  These calls score with fp8 queries and
 * fp8 keys on the fp8 matrix cores; the result is the routed score of the
 * dequantised inputs (within the scoring tolerance: the fp8 MFMA accumulates
 * at slightly less than fp32 precision).
 *
 * misa_quantize_q: per (query, head) row of 128 values,
 *   q_scale = fp32(amax / 448), amax = max |q| over the row (1 for a zero row),
 *   q8      = e4m3fn round-to-nearest-even of fp32(q / q_scale),
 * both divisions correctly rounded (448 is the largest finite e4m3fn value).
 * q: bf16 [n_seq][M][H][128] (16-byte aligned); q8: uint8 [n_seq][M][H][128]
 * (16-byte aligned); q_scale: float [n_seq][M][H].
 */
misa_status misa_quantize_q(const misa_shape* shape, const uint16_t* q, uint8_t* q8, float* q_scale,
                            void* stream);

/*
 * misa_sparse_head_logits on fp8 queries (misa_quantize_q's q8 and q_scale):
 *   I[t,s] = sigma[s] * sum_{j in heads(t)} w[t,j] * q_scale[t,j] * ReLU(q8[t,j] . k8[s])
 * for s <= t, -inf after (the q and key codes taken as e4m3fn values).
 * kdtype must be MISA_K_FP8_E4M3 (MISA_ERR_UNSUPPORTED otherwise), and
 * 1 <= h <= 8 (MISA_ERR_UNSUPPORTED above 8).  Other arguments as
 * misa_sparse_head_logits; columns N .. roundup4(N)-1 may be set to -inf.
 */
misa_status misa_sparse_head_logits_q8(const misa_shape* shape, const uint8_t* q8, const float* q_scale,
                                       const float* w, const void* k, misa_kdtype kdtype, const float* k_scale,
                                       const int32_t* heads, int32_t h, float* logits, int64_t ld,
                                       void* stream);

/*
 * dsa_dense_logits on fp8 queries, every key (the fp8-query dense DSA
 * indexer, the production-style comparator of the GitHub issue's Figure 3
 * discussion, whose dense path scores fp8 queries and keys):
 *   D[t,s] = sigma[s] * sum_{j < H} w[t,j] * q_scale[t,j] * ReLU(q8[t,j] . k8[s])
 * for s <= t, -inf after.  kdtype must be MISA_K_FP8_E4M3
 * (MISA_ERR_UNSUPPORTED otherwise).  logits: float [n_seq][M][ld], ld >= N,
 * ld % 4 == 0, 16-byte aligned; columns N .. roundup4(N)-1 may be set to -inf.
 */
misa_status dsa_dense_logits_q8(const misa_shape* shape, const uint8_t* q8, const float* q_scale, const float* w,
                                const void* k, misa_kdtype kdtype, const float* k_scale, float* logits, int64_t ld,
                                void* stream);

/*
 * misa_sparse_head_topk on fp8 queries: exactly
 * misa_topk(misa_sparse_head_logits_q8(...), topk) (ids, values and order;
 * the set when sorted == 0), through the same fused path (logits only for
 * the rows the candidates cannot settle).  The second question of the GitHub
 * issue asks for an fp8 MISA kernel with the top-k overhead cut; this is it.
 * kdtype must be MISA_K_FP8_E4M3 and 1 <= h <= 8 (MISA_ERR_UNSUPPORTED
 * otherwise).  The workspace is misa_sparse_head_topk_workspace_bytes(shape,
 * MISA_K_FP8_E4M3, h, topk) bytes (16-byte aligned; the fp8 keys feed the
 * fp8 matrix cores as they are, so part of it stays unused).  Other arguments
 * as misa_sparse_head_topk.
 */
misa_status misa_sparse_head_topk_q8(const misa_shape* shape, const uint8_t* q8, const float* q_scale,
                                     const float* w, const void* k, misa_kdtype kdtype, const float* k_scale,
                                     const int32_t* heads, int32_t h, int32_t topk, int32_t sorted, int32_t* idx,
                                     float* vals, void* ws, size_t ws_bytes, void* stream);

/*
 * The whole indexer on the caller's stream: pool -> route -> routed scoring ->
 * top-k (k_prime == 0, MISA), or pool -> route -> routed scoring -> top-k' ->
 * all-head re-rank of the k' candidates -> top-k (k_prime >= topk, MISA-dagger;
 * "Variante Hierárquica (MISA†)" of the gist.science summary).
 * idx: int32 [n_seq][M][topk], vals: float [n_seq][M][topk] or NULL.
 * 1 <= h <= H; 1 <= topk <= MISA_MAX_TOPK; k_prime == 0 or topk <= k_prime <= MISA_MAX_TOPK.
 * ws / ws_bytes: the workspace (16-byte aligned) holds the pooled keys,
 * tails, routed heads, sampled scores, candidate regions and the logits rows
 * of rows the candidates cannot settle.  misa_indexer_workspace_bytes() bytes
 * is the fast plan (every such row re-scored in one pass); any size down to
 * misa_indexer_workspace_min_bytes() also works, with the same result: the
 * plan is taken from ws_bytes, the re-scoring then runs through a smaller
 * logits slab, a batch of query tiles at a time (two more launches per
 * batch), and candidate regions may be sized closer to the expected
 * candidates.  Below the minimum: MISA_ERR_WORKSPACE, nothing enqueued.
 */
misa_status misa_indexer(const misa_shape* shape, const uint16_t* q, const float* w, const void* k,
                         misa_kdtype kdtype, const float* k_scale, int32_t h, int32_t topk,
                         int32_t k_prime, int32_t* idx, float* vals, void* ws, size_t ws_bytes,
                         void* stream);

/* Workspace of misa_indexer's fast plan for keys of type kdtype; 0 for an
 * invalid shape. */
size_t misa_indexer_workspace_bytes(const misa_shape* shape, misa_kdtype kdtype, int32_t h, int32_t topk,
                                    int32_t k_prime);

/* The least workspace misa_indexer takes (its lean plan: a logits slab no
 * larger than the sampled scores, which it shares memory with, and tighter
 * candidate regions); 0 for an invalid shape.  E.g. about 0.94 GiB for
 * 8192 queries over 131072 fp8 keys, h = 8, topk = 2048, against 6 GiB for
 * the fast plan. */
size_t misa_indexer_workspace_min_bytes(const misa_shape* shape, misa_kdtype kdtype, int32_t h, int32_t topk,
                                        int32_t k_prime);

/*
 * misa_indexer for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments and the same result as misa_indexer, but no workspace
 * argument.  Its scratch is a fixed device buffer of the library,
 * MISA_NOALLOC_SCRATCH_BYTES (256 MiB) per GPU, held until the process ends,
 * planned as a workspace of that size (see misa_indexer); a request whose
 * misa_indexer_workspace_min_bytes() exceeds it returns MISA_ERR_SCRATCH and
 * enqueues nothing (256 MiB holds, e.g., a decode batch of 64 sequences x
 * 131072 keys, or a prefill chunk of 512 queries over 65536 keys).  The call allocates, frees and synchronises nothing.  All
 * calls on one GPU share that GPU's buffer, which keeps the last call's
 * contents: calls that may overlap on one GPU (several streams, several host
 * threads) race, so the caller must order them (one stream, or events).
 * The first call on a device looks up the buffer's device address; later calls
 * reuse it.
 */
#define MISA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
misa_status misa_indexer_noalloc(const misa_shape* shape, const uint16_t* q, const float* w, const void* k,
                                 misa_kdtype kdtype, const float* k_scale, int32_t h, int32_t topk,
                                 int32_t k_prime, int32_t* idx, float* vals, void* stream);

/*
 * misa_indexer with fp8 queries for the routed scoring: pool -> route (bf16
 * q) -> misa_quantize_q into the workspace -> misa_sparse_head_topk_q8 (the
 * k' candidates when k_prime > 0, then the MISA-dagger re-rank with bf16 q
 * and all heads, as misa_indexer).  The result is exactly that sequence of
 * calls.  kdtype must be MISA_K_FP8_E4M3 and 1 <= h <= 8
 * (MISA_ERR_UNSUPPORTED otherwise); other arguments as misa_indexer; ws: at
 * least misa_indexer_q8_workspace_bytes() bytes.
 */
misa_status misa_indexer_q8(const misa_shape* shape, const uint16_t* q, const float* w, const void* k,
                            misa_kdtype kdtype, const float* k_scale, int32_t h, int32_t topk, int32_t k_prime,
                            int32_t* idx, float* vals, void* ws, size_t ws_bytes, void* stream);

size_t misa_indexer_q8_workspace_bytes(const misa_shape* shape, int32_t h, int32_t topk, int32_t k_prime);

/*
 * Paged key cache -> the contiguous keys every call here reads.  Serving
 * engines keep the indexer keys in pages of page_keys keys named by a
 * per-sequence block table (the GitHub issue's per-layer boundary includes
 * this cache handling).  Key s of sequence b is row s % page_keys of page
 * block_table[b * max_pages + s / page_keys]; the call writes keys
 * [0, n_keys) of every sequence to k_out [n_seq][n_keys][128] (16-byte
 * aligned) and, for fp8, their scales to scale_out [n_seq][n_keys].
 * k_pages: [n_pages][page_keys][128] bf16 or e4m3 codes (16-byte aligned),
 * scale_pages: [n_pages][page_keys] (fp8 only).  max_pages >=
 * ceil(n_keys / page_keys).  Page ids outside [0, n_pages) are a
 * precondition violation: those keys are written as zeros (scale 1), never
 * read.  HBM-bound: 2 x the keys' bytes.
 */
misa_status misa_gather_keys_paged(const misa_shape* shape, const void* k_pages, misa_kdtype kdtype,
                                   const float* scale_pages, const int32_t* block_table, int64_t max_pages,
                                   int64_t n_pages, int32_t page_keys, void* k_out, float* scale_out, void* stream);

/*
 * Pooled-key cache (chunked prefill and decode).  The GitHub issue measures
 * the indexer at a per-layer boundary that includes cache handling, under
 * chunked prefill of 8192 tokens up to a 128K prompt ("Clarification on the
 * Figure 3 baseline ...", the measured configuration).  Block means of keys
 * already pooled do not change as the sequence grows, so a caller-owned
 * cache keeps them across calls and each call pools only the blocks that
 * have become complete since (decode then reads K once per step instead of
 * twice).
 *
 * The cache of a shape's n_seq sequences, caller-owned device memory:
 *   pooled:       float    [n_seq][cap_blocks][128]     block means
 *   pooled_split: uint16_t [n_seq][2][cap_blocks][128]  their bf16 hi rows, then
 *                 lo rows (pooled - hi), which the router stages directly
 * both 16-byte aligned, cap_blocks >= n_keys / block.  n_cached: the number of
 * leading complete blocks whose rows already hold the means of these keys
 * (0 for an empty cache; after a call with n_keys keys the cache holds
 * n_keys / block blocks).  0 <= n_cached <= n_keys / block, else
 * MISA_ERR_INVALID_ARG.  The keys of the cached blocks are not read again,
 * so they must be the keys the cache was built from.
 */

/* misa_pool_keys into the cache: pools complete blocks [n_cached, N/B) and
 * the tails of the shape's queries (tail: float [n_seq][M][128], may be NULL
 * when M == 0). */
misa_status misa_pool_keys_cached(const misa_shape* shape, const void* k, misa_kdtype kdtype,
                                  const float* k_scale, int64_t n_cached, float* pooled,
                                  uint16_t* pooled_split, int64_t cap_blocks, float* tail, void* stream);

/* misa_indexer with the pooled keys in the cache (brought up to date first).
 * The result is exactly misa_indexer's on the same arguments.  ws: at least
 * misa_indexer_cached_workspace_bytes() bytes.  With M == 0 it only updates
 * the cache (q, w and idx may then be NULL). */
misa_status misa_indexer_cached(const misa_shape* shape, const uint16_t* q, const float* w, const void* k,
                                misa_kdtype kdtype, const float* k_scale, int32_t h, int32_t topk,
                                int32_t k_prime, int64_t n_cached, float* pooled, uint16_t* pooled_split,
                                int64_t cap_blocks, int32_t* idx, float* vals, void* ws, size_t ws_bytes,
                                void* stream);

size_t misa_indexer_cached_workspace_bytes(const misa_shape* shape, misa_kdtype kdtype, int32_t h,
                                           int32_t topk, int32_t k_prime);

/* misa_indexer_cached (k_prime = 0) on keys read in place from a paged cache
 * (the serving engine's KV pages; the GitHub issue's measured configuration
 * counts the cache handling inside the indexer): the pooling of the new
 * blocks and tails, and the routed scoring, read key t of sequence b from
 * page block_table[b * max_pages + t / page_keys], row t % page_keys, of the
 * pools k_pages (key rows of the kdtype, [n_pages][page_keys][128]) and, for
 * fp8 keys, scale_pages (float [n_pages][page_keys]).  No copy of the keys is
 * made (fp8 pages are widened on their way into LDS, never into the
 * workspace): the selection runs as misa_indexer_cached's does, its
 * sampled pass looking up each sampled key's page, its 64-key tiles one page
 * each, and the result equals misa_indexer_cached's on the keys
 * misa_gather_keys_paged would gather, bit for bit.
 * page_keys >= 64 and a multiple of 64 (a 64-key scoring tile then lies in
 * one page), n_pages >= 1, max_pages >= ceil(N / page_keys), else
 * MISA_ERR_INVALID_ARG; table entries are a precondition (in [0, n_pages);
 * out-of-range ones are clamped, never faulting); 1 <= h <= 8 (else
 * MISA_ERR_UNSUPPORTED).  Cache arguments as misa_indexer_cached; ws: at
 * least misa_indexer_paged_workspace_bytes() bytes.  With M == 0 it only
 * updates the cache (q, w and idx may then be NULL). */
misa_status misa_indexer_paged(const misa_shape* shape, const uint16_t* q, const float* w, const void* k_pages,
                               misa_kdtype kdtype, const float* scale_pages, const int32_t* block_table,
                               int64_t max_pages, int64_t n_pages, int32_t page_keys, int32_t h, int32_t topk,
                               int64_t n_cached, float* pooled, uint16_t* pooled_split, int64_t cap_blocks,
                               int32_t* idx, float* vals, void* ws, size_t ws_bytes, void* stream);

size_t misa_indexer_paged_workspace_bytes(const misa_shape* shape, misa_kdtype kdtype, int32_t h, int32_t topk);

/* Chunked prefill driver: the indexer over the shape's M queries (positions
 * q_pos0 .. q_pos0+M-1 of each sequence) in chunks of `chunk` queries, the way
 * a serving engine prefills a long prompt: chunk c sees the keys through its
 * own last query, and the pooled-key cache (kept in the workspace) grows from
 * chunk to chunk.  Sequences are processed one after another.  idx / vals as
 * misa_indexer over the whole shape, and equal to it: each query's top-k
 * depends only on its own prefix.  ws: at least misa_prefill_workspace_bytes()
 * bytes (the cache of one sequence plus the largest chunk's indexer
 * workspace).  chunk >= 1, else MISA_ERR_INVALID_ARG. */
misa_status misa_prefill_chunked(const misa_shape* shape, const uint16_t* q, const float* w, const void* k,
                                 misa_kdtype kdtype, const float* k_scale, int32_t h, int32_t topk,
                                 int32_t k_prime, int32_t chunk, int32_t* idx, float* vals, void* ws,
                                 size_t ws_bytes, void* stream);

size_t misa_prefill_workspace_bytes(const misa_shape* shape, misa_kdtype kdtype, int32_t h, int32_t topk,
                                    int32_t k_prime, int32_t chunk);

/*
 * Profiling.  The stages of misa_indexer (and of the calls that run parts of
 * it: misa_sparse_head_topk[_q8], misa_indexer_cached, misa_indexer_q8,
 * misa_indexer_noalloc, misa_prefill_chunked) whose kernels a caller can time
 * on their own with HIP events.  The fused-selection stages apply when that
 * path is taken (misa_sparse_head_topk above).
 */
typedef enum {
  MISA_STAGE_NONE = 0,
  MISA_STAGE_POOL = 1,               /* block pooling (inside the indexer calls) */
  MISA_STAGE_ROUTE = 2,              /* head routing (inside the indexer calls) */
  MISA_STAGE_SCORE_SAMPLE = 3,       /* scores of the key sample */
  MISA_STAGE_SAMPLE_THRESHOLD = 4,   /* per-row thresholds from the sample */
  MISA_STAGE_SCORE_CANDIDATES = 5,   /* routed scoring that keeps the candidates */
  MISA_STAGE_REGION_SELECT = 6,      /* exact top-k of the candidates */
  MISA_STAGE_RESCORE = 7,            /* re-scoring and top-k of the rows the candidates could not settle */
  MISA_STAGE_RERANK = 8,             /* MISA-dagger: all-head re-rank of the k' candidates */
  MISA_STAGE_FINAL_TOPK = 9,         /* MISA-dagger: top-k of the re-ranked candidates */
  MISA_STAGE_SCORE_LOGITS = 10,      /* routed scoring into whole logits rows (few queries, short prefixes, paged keys) */
  MISA_STAGE_LOGITS_TOPK = 11        /* top-k of those logits */
} misa_stage;

/*
 * Until the next misa_profile_stage call on the same host thread, every call
 * made on that thread records start_event on its stream just before it
 * enqueues the kernels of `stage`, and stop_event just after (hipEvent_t
 * passed as void*, created by the caller; the setting is per host thread).
 * A call that does not run the stage records nothing.  MISA_STAGE_NONE (events
 * may be NULL) turns it off.  An unknown stage or a null event:
 * MISA_ERR_INVALID_ARG.
 */
misa_status misa_profile_stage(int32_t stage, void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* MISA_H */
