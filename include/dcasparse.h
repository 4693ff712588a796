/*
 * dcasparse.h — C ABI of the MI355X (gfx950) library for long-context prefill
 * attention with Dual Chunk Attention (DCA), YaRN logit scaling and
 * vertical-slash sparsity chosen per prefill chunk, and the generation-step
 * (decode) attention over a rotated key cache.
 *
 * What is computed (sources: "Qwen2.5-1M Technical Report" as summarised on
 * the xllm-io paper-review page, section 4 "Inference & deployment":
 * Dual Chunk Attention (Figure 2), the YaRN attention-scaling equation, and
 * the sparse attention of Figure 4; chunk size from the agentlenshq release
 * blog, section "Sparse Attention"):
 *
 *   For query head h (KV head g = h / (h_q / h_kv)), query row i at absolute
 *   position p_i and key j of the prefix, with S = dca_chunk, W = dca_local,
 *   r = position mod S and m = position div S:
 *     key position      pi_k = r_j
 *     query position    pi_q = r_i                    if m_j == m_i   (intra-chunk)
 *                             = min(S + r_i, S+W-1)    if m_j == m_i-1 (successive chunk)
 *                             = S + W - 1              if m_j <= m_i-2 (inter-chunk)
 *     logit l_ij = (0.1 ln s + 1)^2 / sqrt(d) * < RoPE(q_i, pi_q), RoPE(k_j, pi_k) >
 *   RoPE pairs component c with c + d/2 and turns it by position * base^(-2c/d).
 *   out_i = sum_{j in A(i)} softmax_j(l_ij) v_j, lse_i = ln sum_{j in A(i)} e^{l_ij}.
 *   Dense: A(i) = { j <= p_i }.  Sparse (block cover, 64-row granule): for the
 *   query block whose first row sits at i0 (a multiple of 64), every selected
 *   slash offset delta (delta = 0 is always included) covers keys
 *   [i0-delta, i0-delta+63]; the selected vertical columns are added; row i
 *   attends the covered keys j <= p_i.
 *
 * Conventions shared by every entry point:
 *   - Tensors are row-major, contiguous, device memory, raw bfloat16 bits:
 *       q, out : [n_q][h_q][head_dim]      k, v : [n_k][h_kv][head_dim]
 *     q and k are BEFORE any rotary embedding: the library applies every
 *     rotation itself.
 *   - positions is a DEVICE int32 array of n_q entries that must be the
 *     contiguous run p0, p0+1, ..., n_k-1 with p0 = n_k - n_q (a chunk of a
 *     chunked prefill whose KV prefix ends with the chunk), p0 a multiple of
 *     64.  The host checks p0 from n_k and n_q before anything is enqueued.
 *     The entries are checked on the device by the call's first kernel: if
 *     any differs from p0 + i, the call writes none of its outputs (out,
 *     lse_out, v_idx, s_off, cover_pairs, attended_pairs keep their contents)
 *     and stores DCA_EINVAL in *cfg->status when status is given (DCA_OK
 *     otherwise).  The workspace holds the check's result, so its contents
 *     after such a call are unspecified.
 *   - Every buffer belongs to the caller.  No entry point allocates device
 *     memory: scratch comes from cfg->workspace, sized by dca_workspace_size
 *     (dca_decode_workspace_size for dca_decode).
 *   - Work is enqueued on cfg->stream and the call returns without waiting.
 *     Outputs are bitwise deterministic for identical inputs.
 *   - Calls sharing one workspace must not overlap in time (same stream, or
 *     the caller orders them).
 *   - Errors: validation happens before any launch; on error nothing is
 *     enqueued and no output is written.  No exception crosses the ABI.
 */
#ifndef DCASPARSE_H
#define DCASPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define DCA_API __attribute__((visibility("default")))
#else
#define DCA_API
#endif

#define DCA_OK            0
#define DCA_EINVAL       (-1)  /* null pointer, inconsistent sizes, bad positions */
#define DCA_EUNSUPPORTED (-2)  /* head_dim != 128, dca_chunk % 64, p0 % 64, W > S, ... */
#define DCA_EWORKSPACE   (-3)  /* workspace missing or smaller than dca_workspace_size */
#define DCA_EHIP         (-4)  /* a HIP launch or runtime call failed */
#define DCA_ESCRATCH     (-5)  /* dca_sparse_prefill_noalloc: the call needs more than its static scratch */

typedef uint16_t dca_bf16;     /* raw bfloat16 bits */

/* Number of optional timing events dca_sparse_prefill records (see stage_events). */
#define DCA_STAGE_COUNT 4      /* 0: key and query rotations, 1: sparse plan, 2: attention, 3: LSE merge */

typedef struct dca_cfg {
  int32_t n_q;            /* query rows in this call (>= 1) */
  int32_t n_k;            /* keys in the prefix; positions[i] must equal n_k - n_q + i */
  int32_t h_q, h_kv;      /* query / KV heads; h_q % h_kv == 0 (GQA: consecutive grouping) */
  int32_t head_dim;       /* must be 128 */
  int32_t dca_chunk;      /* S: multiple of 64, >= 64 */
  int32_t dca_local;      /* W: 0 < W <= S */
  double  rope_base;      /* RoPE base, > 1 (e.g. 1e6, 1e7) */
  double  yarn_s;         /* s: logit factor (0.1 ln s + 1)^2 when s > 1, else 1 */
  int32_t vs_last_q;      /* index builder: scoring rows = the last min(vs_last_q, n_q) rows; 1..64 */
  int32_t vs_k_vertical;  /* k_v: vertical columns per query head (>= 0) */
  int32_t vs_k_slash;     /* k_s: slash offsets per query head (>= 0) */
  /* Sparse pattern for dca_sparse_prefill (device int32).  Both NULL: dense
   * causal DCA attention.  Otherwise v_idx is [h_q][vs_k_vertical] absolute
   * key ids and s_off is [h_q][vs_k_slash] offsets, each row ascending, with
   * -1 entries as padding (vs_index_build's output format).  Entries out of
   * range are ignored; a row that is not ascending gives an unspecified cover
   * but never an out-of-bounds access. */
  const int32_t *v_idx;
  const int32_t *s_off;
  float   *lse_out;       /* optional device [h_q][n_q] natural-log LSE of each row; NULL: not written */
  int64_t *cover_pairs;   /* optional device int64: dca_sparse_prefill writes sum over heads and query
                             blocks of rows(block) * |cover(block)|, the (row, key) pairs of the computed
                             blocks; 4 * head_dim * cover_pairs is the computed-block FLOP count.  NULL: not written */
  float   precise_norm;   /* keys whose L2 norm exceeds this get split-bf16 (hi+lo) logits;
                             0: default 2*sqrt(head_dim); < 0: never */
  int32_t split_k;        /* key-range splits per query block (0..256), merged by LSE: 0 = library's
                             choice (about one split per 16K keys, at most 64) */
  void   *workspace;      /* device scratch, >= dca_workspace_size bytes, 256-byte aligned */
  size_t  workspace_bytes;
  void   *stream;         /* hipStream_t; NULL = the null stream */
  /* Optional: array of 2*DCA_STAGE_COUNT hipEvent_t (start, stop per stage)
   * that dca_sparse_prefill records on cfg->stream around each stage; NULL =
   * no timing.  Stages that do not run still get both events recorded. */
  void  **stage_events;
  /* Sparse semantics of dca_sparse_prefill.  0: the block cover above (64-row
   * granule).  1: exact diagonals: row i attends key j <= p_i when p_i - j is a
   * selected offset (or 0) or j a selected vertical column.  Both compute the
   * same covered tiles (cover_pairs is the block cover in both); the exact
   * reading masks each row to its own diagonals. */
  int32_t slash_exact;
  /* Optional device int32 [h_q][2]: per-head budgets (k_v, k_s) for
   * vs_index_build, each clamped to [0, vs_k_vertical] / [0, vs_k_slash]; a
   * head's rows hold its own k best, padded with -1.  NULL: every head takes
   * vs_k_vertical and vs_k_slash. */
  const int32_t *vs_k_per_head;
  /* Optional device int64: dca_sparse_prefill writes the sum over heads and
   * rows of |A(i)|, the (row, key) pairs each row attends (causal, and in the
   * sparse readings only its covered or exact keys); 4 * head_dim *
   * attended_pairs is F_attended.  For exact diagonals it costs one pass over
   * the selected offsets per vertical column.  NULL: not written. */
  int64_t *attended_pairs;
  /* Optional device int32: calls that take positions store DCA_OK there, or
   * DCA_EINVAL when the device check of positions fails.  NULL: not written. */
  int32_t *status;
} dca_cfg;

/* Bytes of workspace both entry points need for this configuration (the
 * largest of the two).  Pure host computation.  Returns DCA_OK and writes
 * *bytes, or a validation error. */
DCA_API int dca_workspace_size(const dca_cfg *cfg, size_t *bytes);

/* Vertical-slash index of one prefill chunk (paper-review page, section 4,
 * Figure 4: key tokens chosen per chunk, with continuous relative positions
 * restored while choosing).  Scores the last n_s = min(vs_last_q, n_q) rows
 * against every key j <= p_i in float64, with query position r_i for keys of
 * its own DCA chunk and S + r_i for keys of any earlier chunk (key position
 * r_j), the same YaRN-scaled logits, and a row softmax.  vertical[j] = sum of
 * the rows' probabilities in column j; slash[delta] = sum over rows of the
 * probability at key p_i - delta.  Offset 0 is always selected.  The k best
 * of each list by (score desc, index asc) are written ascending:
 *   v_idx [h_q][vs_k_vertical] key ids, s_off [h_q][vs_k_slash] offsets,
 * padded with -1 when there are fewer candidates (n_k keys, p_last+1 offsets).
 * Inputs q (only its last n_s rows are read) and k as in the conventions. */
DCA_API int vs_index_build(const dca_bf16 *q, const dca_bf16 *k, const int32_t *positions,
                   const dca_cfg *cfg, int32_t *v_idx, int32_t *s_off);

/* DCA prefill attention of one chunk over its KV prefix, dense or
 * block-sparse (see the definition at the top).  Writes out [n_q][h_q][128]
 * bf16 (round to nearest even from fp32) and, when cfg->lse_out is set, the
 * natural-log LSE of every row.  bf16 inputs, fp32 accumulation. */
DCA_API int dca_sparse_prefill(const dca_bf16 *q, const dca_bf16 *k, const dca_bf16 *v,
                       const int32_t *positions, const dca_cfg *cfg, dca_bf16 *out);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * dca_sparse_prefill with the scratch taken from a static device array of
 * DCA_STATIC_SCRATCH_BYTES per GPU that the library owns (each GPU the
 * library runs on keeps its copy until the process ends) instead of
 * cfg->workspace, which is ignored.  Same arguments, definition and outputs
 * (bitwise equal to dca_sparse_prefill's).  Calls that need more scratch
 * than the array holds (dca_workspace_size > DCA_STATIC_SCRATCH_BYTES) return
 * DCA_ESCRATCH before anything is enqueued.  The call allocates nothing.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind: calls that overlap in time on one GPU (different streams, threads
 * or processes sharing the library) race, so the caller orders them. */
#define DCA_STATIC_SCRATCH_BYTES (256u << 20)
DCA_API int dca_sparse_prefill_noalloc(const dca_bf16 *q, const dca_bf16 *k, const dca_bf16 *v,
                                       const int32_t *positions, const dca_cfg *cfg, dca_bf16 *out);

/* ---- Generation step (decode) ------------------------------------------
 * After a prefill, each generated token attends the whole key cache with the
 * same DCA positions, densely (the pages apply the sparse attention to the
 * prefill only).  A key's rotation depends only on r_j = j mod S, not on the
 * query, so keys are rotated once, when they enter the cache, into the three
 * arrays below (caller-owned device memory of the given capacity):
 *   k_hi    [capacity][h_kv][head_dim]  RoPE(k_j, r_j) rounded to bf16
 *   k_lo    [capacity][h_kv][head_dim]  bf16 residual of that rounding
 *   k_flags [h_kv][(capacity + 31) / 32] bit j set: key j's L2 norm exceeds
 *           cfg->precise_norm (its logits then use hi + lo). */
typedef struct dca_key_cache {
  dca_bf16 *k_hi;
  dca_bf16 *k_lo;
  uint32_t *k_flags;
  int32_t   capacity;     /* keys the arrays hold; capacity * h_kv * head_dim * 2 < 2^32 */
} dca_key_cache;

/* Rotates keys j0 .. j0+n-1 into the cache (k points at key j0, layout
 * [n][h_kv][head_dim] raw bf16 before rotation) and rewrites their flag bits
 * (other bits are kept).  Reads cfg->h_kv, head_dim, dca_chunk, rope_base,
 * precise_norm and stream; needs no workspace.  Requires 0 <= j0,
 * 1 <= n, j0 + n <= capacity.  Asynchronous on cfg->stream. */
DCA_API int dca_key_cache_append(const dca_bf16 *k, int32_t j0, int32_t n, const dca_cfg *cfg,
                                 const dca_key_cache *cache);

/* dca_sparse_prefill with the keys taken from a rotated key cache instead of
 * raw k: keys 0 .. n_k-1 must have been appended (the chunk's own keys
 * included), so a chunked prefill rotates every key once rather than its
 * whole prefix per chunk.  Same definition, outputs and workspace
 * (dca_workspace_size) as dca_sparse_prefill; with the same keys the outputs
 * are bitwise equal. */
DCA_API int dca_sparse_prefill_cached(const dca_bf16 *q, const dca_key_cache *cache, const dca_bf16 *v,
                                      const int32_t *positions, const dca_cfg *cfg, dca_bf16 *out);

/* Workspace bytes of dca_decode for this configuration (cfg->n_q new tokens,
 * cfg->n_k cached keys).  Pure host computation. */
DCA_API int dca_decode_workspace_size(const dca_cfg *cfg, size_t *bytes);

/* Attention of the n_q = cfg->n_q newest tokens, at positions
 * n_k - n_q .. n_k - 1, over cache keys 0 .. n_k - 1 (all appended): dense
 * DCA, A(i) = { j <= p_i } in the definition at the top.  q [n_q][h_q][128]
 * raw bf16 before rotation; v [capacity][h_kv][128] (rows < n_k are read).
 * Writes out [n_q][h_q][128] bf16 and, when cfg->lse_out is set, the
 * natural-log LSE [h_q][n_q].  1 <= n_q <= 64 and n_q <= n_k <= capacity;
 * cfg->v_idx and cfg->s_off must be NULL; cfg->split_k (0..4096) sets the
 * number of key parts (0: the library's choice, ~2048 workgroups); positions
 * are implied.  bf16 inputs, fp32 accumulation; deterministic.
 * cfg->stage_events, when set, are recorded as for dca_sparse_prefill:
 * 0 query rotations, 1 (empty), 2 attention over the cache, 3 LSE merge. */
DCA_API int dca_decode(const dca_bf16 *q, const dca_key_cache *cache, const dca_bf16 *v, const dca_cfg *cfg,
                       dca_bf16 *out);

/* ---- Paged key / value cache for generation ------------------------------
 * The same rotated keys, their values and flags, kept in a pool of
 * fixed-size pages shared by many sequences; a sequence owns a page table.
 * Pools (caller-owned device memory), each page laid out head-major so that
 * the keys of one KV head in a page are consecutive rows:
 *   k_hi, k_lo, v [n_pages][h_kv][page_keys][head_dim]
 *   k_flags       [n_pages][h_kv][page_keys / 32]  bit j % 32 of word
 *                 (page, g, (j % page_keys) / 32): key j of KV head g is high-norm
 * page_table (device int32 [n_table]): logical page p (keys p * page_keys ..
 * (p+1) * page_keys - 1 of the sequence) lives in pool page page_table[p].
 * Entries outside [0, n_pages) are never written through and are clamped
 * when read (that key range then holds unspecified data, never an
 * out-of-bounds access). */
typedef struct dca_paged_kv {
  dca_bf16 *k_hi;
  dca_bf16 *k_lo;
  dca_bf16 *v;
  uint32_t *k_flags;
  int32_t   n_pages;      /* >= 1; n_pages * page_keys * h_kv * head_dim * 2 < 2^32 */
  int32_t   page_keys;    /* multiple of 32 */
  const int32_t *page_table;
  int32_t   n_table;      /* entries of page_table */
} dca_paged_kv;

/* Rotates keys j0 .. j0+n-1 of the sequence into their pages (k, v point at
 * key j0, layout [n][h_kv][head_dim] raw bf16), copies their values and
 * rewrites their flag bits.  Requires j0 >= 0, n >= 1 and
 * j0 + n <= n_table * page_keys.  Reads the same cfg fields as
 * dca_key_cache_append; no workspace. */
DCA_API int dca_paged_append(const dca_bf16 *k, const dca_bf16 *v, int32_t j0, int32_t n, const dca_cfg *cfg,
                             const dca_paged_kv *cache);

/* dca_decode over a paged cache: keys and values 0 .. cfg->n_k - 1 of the
 * sequence through its page table (cfg->n_k <= n_table * page_keys).  Same
 * workspace (dca_decode_workspace_size), outputs and events; with the same
 * keys and values the outputs equal dca_decode's bit for bit. */
DCA_API int dca_decode_paged(const dca_bf16 *q, const dca_paged_kv *cache, const dca_cfg *cfg, dca_bf16 *out);

/* Workspace bytes of dca_sparse_prefill_paged for this configuration:
 * dca_workspace_size's plus room for the sequence's values gathered from
 * the pool.  Pure host computation. */
DCA_API int dca_paged_prefill_workspace_size(const dca_cfg *cfg, size_t *bytes);

/* dca_sparse_prefill with keys and values 0 .. n_k-1 of a sequence taken
 * from a paged pool through its page table (dca_paged_append put them
 * there, the chunk's own keys included; n_k <= n_table * page_keys).  Same
 * definition and outputs as dca_sparse_prefill_cached: with the same keys
 * and values the outputs are bitwise equal.  The call first copies the
 * sequence's rotated keys, values and flag words from their pages into the
 * workspace (dca_paged_prefill_workspace_size); page entries outside
 * [0, n_pages) are clamped (that key range then holds unspecified data,
 * never an out-of-bounds access). */
DCA_API int dca_sparse_prefill_paged(const dca_bf16 *q, const dca_paged_kv *cache, const int32_t *positions,
                                     const dca_cfg *cfg, dca_bf16 *out);

/* ---- Whole-sequence prefill ----------------------------------------------
 * The pages' chunked prefill runs a long prompt chunk by chunk: chunk c holds
 * query rows [b_c, b_{c+1}) and attends the prefix [0, b_{c+1}).  Dynamic
 * chunked pipeline parallelism (paper-review page, section 4, "Pipeline
 * parallelism", Figure 9) sizes the chunks by the attention kernel's cost so
 * that every chunk takes about the same time.  The pages give no cost
 * formula; the model below prices a chunk of rows [a, b) at
 *   per_call + per_row * (b - a) + per_index_key * b
 *     + per_pair * sum over its 64-row blocks [i0, i0 + r) of r * cover(i0 + r)
 * where cover(E) = E for a dense block (its causal extent) and, with
 * cap = cover_cap > 0, E (1 - exp(-cap / E)) for a sparse one: the expected
 * union of cap keys' worth of 64-key footprints scattered over the extent
 * (E while cap >> E, tending to cap when E >> cap). */
typedef struct dca_chunk_cost {
  double  per_call;       /* fixed cost of one chunk (launches, LSE merge) */
  double  per_row;        /* per query row of the chunk (query rotations, key append, output) */
  double  per_index_key;  /* per key of the chunk's prefix (the index build scores the whole prefix) */
  double  per_pair;       /* per computed (query row, key) pair, all query heads together */
  int64_t cover_cap;      /* keys of a sparse block's budget, 64 k_s + k_v; <= 0: dense (no bound) */
} dca_chunk_cost;

/* Cost coefficients, in microseconds, fitted to this library's measured
 * chunk times on MI355X, scaled to the heads of cfg (n_q, n_k are ignored):
 * per (row, key, head) of attention, per (row, head), per (prefix key, head)
 * of index build, per chunk; cover_cap = 64 * vs_k_slash + vs_k_vertical for
 * a sparse prefill (sparse = 1), no cap and no index cost for a dense one. */
DCA_API int dca_chunk_cost_default(const dca_cfg *cfg, int32_t sparse, dca_chunk_cost *cost);

/* Equal-time chunk schedule: splits tokens [0, n_tokens) into exactly
 * min(n_chunks, ceil(n_tokens / 64)) chunks, each starting on a multiple of
 * 64 and at most max_rows rows long (max_rows >= 64), minimising the largest
 * chunk cost under *cost (exact optimum of that min-max problem, found by a
 * bisection over greedy packings).  Writes bounds[0 .. *n_out] (host int32,
 * room for n_chunks + 1 entries): 0 = bounds[0] < ... < bounds[*n_out] =
 * n_tokens; and, when max_cost is not NULL, the largest chunk cost.  Pure
 * host computation.  DCA_EINVAL when n_chunks chunks of max_rows rows cannot
 * hold n_tokens, or on negative coefficients. */
DCA_API int dca_chunk_schedule(int32_t n_tokens, int32_t n_chunks, int32_t max_rows, const dca_chunk_cost *cost,
                               int32_t *bounds, int32_t *n_out, double *max_cost);

/* How dca_prefill_sequence runs a prompt. */
typedef struct dca_sequence_plan {
  const int32_t *bounds;  /* host int32 [n_chunks + 1]: 0 = bounds[0] < ... < bounds[n_chunks] = cfg->n_k,
                             bounds[c] % 64 == 0 for c < n_chunks (e.g. from dca_chunk_schedule) */
  int32_t  n_chunks;      /* >= 1 */
  int32_t  sparse;        /* 1: every chunk builds its vertical-slash index (vs_index_build) and runs the
                             block-sparse prefill with it; a chunk whose prefix has at most vs_k_slash keys
                             (with no per-head budgets) selects every offset, so its cover is the dense causal
                             set and it runs dense.  0: every chunk dense */
  void    *index_stream;  /* hipStream_t: index builds run on it, one chunk ahead of the attention on
                             cfg->stream, so the index of chunk c+1 overlaps the attention of chunk c.  NULL:
                             everything runs on cfg->stream in order */
  void   **chunk_events;  /* optional 2 * n_chunks hipEvent_t recorded on cfg->stream around chunk c's key
                             append and prefill (start 2c, stop 2c+1); NULL: none */
  void   **index_events;  /* optional 2 * n_chunks hipEvent_t recorded around chunk c's index build, on the
                             stream it runs on (recorded empty for dense chunks); NULL: none */
  int64_t *cover_pairs;   /* optional device int64 [n_chunks]: each chunk's cover_pairs (see dca_cfg) */
} dca_sequence_plan;

/* Workspace bytes of dca_prefill_sequence for cfg (the whole prompt: n_q =
 * n_k = its length) and plan: one chunk's workspace and index buffers, twice
 * when plan->index_stream is set.  Pure host computation. */
DCA_API int dca_prefill_sequence_workspace_size(const dca_cfg *cfg, const dca_sequence_plan *plan, size_t *bytes);

/* Chunked prefill of a whole prompt of n = cfg->n_k tokens (cfg->n_q must
 * equal n; positions are implied: 0 .. n-1).  For each chunk c in order:
 * appends its keys to the rotated key cache (dca_key_cache_append), builds
 * its index when sparse (vs_index_build on raw q and k), and runs its
 * attention from the cache (dca_sparse_prefill_cached), writing rows
 * [b_c, b_{c+1}) of out [n][h_q][128] and, when cfg->lse_out is set, columns
 * [b_c, b_{c+1}) of lse_out [h_q][n].  Every key is rotated once.  The outputs
 * are bitwise those of the per-chunk calls.  cfg->v_idx, s_off, cover_pairs,
 * attended_pairs and stage_events must be NULL (plan->cover_pairs takes the
 * role of cover_pairs); cfg->status is not written; cache->capacity >= n.  Work is ordered on cfg->stream: when it
 * reaches the end of the call there, every chunk is done.  Events are created
 * and released inside the call. */
DCA_API int dca_prefill_sequence(const dca_bf16 *q, const dca_bf16 *k, const dca_bf16 *v,
                                 const dca_sequence_plan *plan, const dca_cfg *cfg, const dca_key_cache *cache,
                                 dca_bf16 *out);

/* Workspace bytes of dca_prefill_sequence_paged (as
 * dca_prefill_sequence_workspace_size, with the paged prefill's chunk
 * workspace).  Pure host computation. */
DCA_API int dca_prefill_sequence_paged_workspace_size(const dca_cfg *cfg, const dca_sequence_plan *plan,
                                                      size_t *bytes);

/* dca_prefill_sequence over a paged pool: each chunk's keys and values are
 * appended into their pages (dca_paged_append) and its attention reads them
 * back through the page table (dca_sparse_prefill_paged), so the pool a
 * generation step reads (dca_decode_paged) is filled by the prefill itself.
 * Requires n <= n_table * page_keys.  Same rules, schedule and streams as
 * dca_prefill_sequence; the outputs are bitwise those of the contiguous
 * driver. */
DCA_API int dca_prefill_sequence_paged(const dca_bf16 *q, const dca_bf16 *k, const dca_bf16 *v,
                                       const dca_sequence_plan *plan, const dca_cfg *cfg, const dca_paged_kv *cache,
                                       dca_bf16 *out);

/* Static message for an error code; never NULL. */
DCA_API const char *dca_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* DCASPARSE_H */
