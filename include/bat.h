/*
 * bat.h -- C ABI of the MI355X (gfx950) prefix-reuse ("bipartite") attention
 * library, libbat.so.
 *
 * The method is the one the Bat page ("Bat: Efficient Generative Recommender
 * Serving with Bipartite Attention") describes (sections "This paper's idea",
 * "Why it works"): a recommendation prompt holds a user's history and a set
 * of items, neither carrying positions, so the two groups can trade places,
 * and whichever one comes first has its key/value cache computed once and
 * served again; user-prefix and item-prefix caches are kept in separate pools
 * (section "Why it works", the disaggregated cache pool).  This library is
 * the data-parallel hot path of that method on one GPU: building the paged
 * prefix cache, and prefill attention of the fresh (suffix) tokens over the
 * cached prefix plus their own group.  Around it: prefix rows (how the next
 * layer's cache is built), candidate-isolated suffixes, grouped key/value
 * heads, and a host-side choice of each query's prefix mode (bat_sched_*).
 *
 * Attention semantics (identical in both prefix modes): scaled dot-product
 * softmax, no positional encoding, no causal mask.  For request r and head h
 * with prefix tokens P and suffix tokens U, a suffix row i sees every token
 * of P and U:
 *     S_ij = softmax_scale * <q_i, k_j>
 *     lse_i = ln sum_j exp(S_ij),   out_i = sum_j exp(S_ij - lse_i) v_j.
 * A prefix row sees P only (bat_attn_prefix_rows); in an item pool, a
 * cached item's own tokens can instead see only their item
 * (bat_attn_item_local).  These build the prefix for the next layer.
 *
 * Conventions for every entry point
 *   - Ownership: the caller owns every buffer.  The library allocates no
 *     device or host memory and keeps no state between calls; scratch space
 *     is the caller's workspace.
 *   - Pointers named "device" must be device (HBM) pointers; host scalars are
 *     passed by value.  `stream` is a hipStream_t (NULL = the null stream);
 *     all work is enqueued asynchronously on it.
 *   - Layouts are row-major.  "Packed" activations are token-major
 *     [tokens, H, D] with a cumulative-length array cu_* of B+1 int32
 *     (cu[0] = 0, cu[r+1] - cu[r] = tokens of request r).
 *   - Errors: a bat_status is returned; nothing is thrown across the ABI.
 *     Host-detectable argument errors return before anything is enqueued.
 *     With the environment variable BAT_VALIDATE=1 the library also checks
 *     on the device, synchronises the stream and returns
 *     BAT_ERR_BLOCK_TABLE when any of these fails:
 *       - every block id read lies in [0, num_blocks) of its pool;
 *       - a suffix length is in [0, max_suffix_len] and cu_suffix_lens[r+1]
 *         <= total_suffix (bat_attn_prefix_rows: the prefix lengths against
 *         max_prefix_len);
 *       - a prefix length is in [0, max_prefix_len] and fits its block-table
 *         row: prefix_lens[r] <= bt_stride * block_size of its pool;
 *       - bat_kv_build: cu_lens is non-decreasing up to total_tokens and each
 *         request's tokens fit its block-table row.
 *     Without it, the same violations are never dereferenced (a prefix
 *     longer than max_prefix_len is cut to it, an out-of-range block id
 *     reads as zero keys/values or is not written) but the result is
 *     unspecified.
 *   - Thread safety: calls are independent; concurrent calls must not share
 *     a workspace.  Validated calls on different streams or threads report
 *     only their own violations.
 *   - Environment variables, read on every call (tests use them to reach
 *     every kernel form; none changes what is computed, only how):
 *       BAT_VALIDATE=1       the device checks above
 *       BAT_WAVES=4|8        bf16 rows per work item: 4 or 8 waves of 32 rows
 *                            (default: 8 when suffixes average > 128 rows,
 *                            else 4; also 4 at D=64 when a bfloat16 pool's
 *                            blocks hold fewer than 64 tokens, and for fp8
 *                            pools at D=128).  Workspace sizes cover either
 *                            shape.
 *       BAT_GATHER=flat      per-key gathers of small pool blocks by global
 *                            loads (the form a pool of blocks smaller than
 *                            a key tile takes at 2 GiB or more) instead of
 *                            buffer loads
 *       BAT_SPLIT_CHUNK=n    split every prefix into chunks of n keys
 *                            (rounded up to the key tile) merged by
 *                            log-sum-exp; a value above every prefix never
 *                            splits (default: split only when the batch has
 *                            too few work items to fill the GPU)
 */
#ifndef BAT_H_
#define BAT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bat_status {
  BAT_OK = 0,
  BAT_ERR_INVALID_ARG = 1, /* null pointer, negative or inconsistent size */
  BAT_ERR_UNSUPPORTED = 2, /* no kernel for this (dtype, head_dim) */
  BAT_ERR_BLOCK_TABLE = 3, /* device validation: bad block id or length */
  BAT_ERR_WORKSPACE = 4,   /* workspace NULL or too small */
  BAT_ERR_HIP = 5          /* a HIP runtime call or launch failed */
} bat_status;

typedef enum bat_dtype {
  BAT_F32 = 0,  /* float32 in/out; scores and running sums in float64 (per-item rows of
                   at most 8 keys: float32) */
  BAT_BF16 = 1  /* bfloat16 in/out, float32 accumulation */
} bat_dtype;

/* Which pool a request's prefix comes from (one byte per request). */
typedef enum bat_prefix_mode {
  BAT_PREFIX_USER = 0, /* the user's history, paged in the user pool */
  BAT_PREFIX_ITEM = 1  /* cached items, one item per item-pool block */
} bat_prefix_mode;

/*
 * A paged key/value pool (the disaggregated cache pool of the Bat page,
 * section "Why it works": user-prefix and item-prefix caches are separate
 * pools).  k and v are device buffers laid out [num_blocks, H, block_size, D]
 * in the dtype of the call.  Token t of a prefix lives in block
 * block_table[t / block_size], slot t % block_size.  block_size is a power
 * of two in [1, 256].  An item pool holds one item per block, so an item id
 * is its block id and block_size is the item's token count (4 here).
 */
typedef struct bat_kv_pool {
  void *k;
  void *v;
  int32_t num_blocks;
  int32_t block_size;
} bat_kv_pool;

/*
 * bat_kv_build -- write prefix keys and values into a paged pool.
 *
 * Builds the reusable prefix cache that later prefills read (Bat page,
 * sections "Problem" and "Why this problem is worth solving": the prefix's
 * key/value cache is computed once and reused).  A bit-exact copy: token t
 * of request r, head h goes to pool->k/v[block_table[r*bt_stride + t/bs],
 * h, t % bs, :].
 *
 *   k, v          device, packed [total_tokens, H, D], dtype dt
 *   cu_lens       device int32 [B+1]; cu_lens[B] must equal total_tokens
 *   block_table   device int32 [B, bt_stride]; only the first
 *                 ceil(len_r / bs) entries of row r are read
 *   B, H, D       requests (or items), heads, head dim (D in {32, 64, 128})
 *   total_tokens  host copy of cu_lens[B] (sizes the launch); 0 is a no-op
 *   pool          host pointer to the destination pool description
 * Slots that no token maps to are left untouched.  Ids outside
 * [0, num_blocks) are skipped (and reported under BAT_VALIDATE=1).
 */
bat_status bat_kv_build(const void *k, const void *v, const int32_t *cu_lens,
                        const int32_t *block_table, int32_t bt_stride,
                        int32_t B, int32_t H, int32_t D, int32_t total_tokens,
                        bat_dtype dt, const bat_kv_pool *pool, void *stream);

/*
 * bat_attn_workspace_size -- bytes of device workspace bat_attn_prefill needs
 * for these host-side bounds (work list, per-request metadata, and the
 * partial results of prefixes split across workgroups).  Returns 0 for
 * invalid arguments.
 */
size_t bat_attn_workspace_size(int32_t B, int32_t H, int32_t D, bat_dtype dt,
                               int32_t total_suffix, int32_t max_suffix_len,
                               int32_t max_prefix_len);

/*
 * bat_attn_prefill_workspace_size -- an upper bound of
 * bat_attn_workspace_size over both dtypes and every max_suffix_len up to
 * total_suffix: enough workspace for any bat_attn_prefill call with these
 * B, H, D, total_suffix and max_prefix_len.  bat_attn_workspace_size gives
 * the exact (smaller) figure when the dtype and the suffix bound are known.
 * Returns 0 for invalid arguments, or when the bound would need work lists
 * of 2^30 items or more.
 */
size_t bat_attn_prefill_workspace_size(int32_t B, int32_t H, int32_t D,
                                       int32_t total_suffix,
                                       int32_t max_prefix_len);

/*
 * bat_attn_prefill -- prefill attention of the suffix rows over the cached
 * prefix and their own group (the Bipartite Attention of the Bat page,
 * section "This paper's idea": either the user history or a set of cached
 * items is the prefix; the suffix is computed fresh).
 *
 *   q, k, v         device, packed fresh suffix [total_suffix, H, D], dtype dt
 *   cu_suffix_lens  device int32 [B+1]
 *   prefix_lens     device int32 [B]; prefix tokens of each request (0 ok).
 *                   An item-mode prefix has block_size tokens per listed item.
 *   prefix_mode     device uint8 [B], bat_prefix_mode per request
 *   block_table     device int32 [B, bt_stride]: user-mode rows list user-pool
 *                   blocks, item-mode rows list item ids (item-pool blocks),
 *                   in the order the request sees them
 *   user_pool, item_pool  host pointers; either may be NULL if no request
 *                   uses it
 *   softmax_scale   multiplies q.k (pass 1/sqrt(D) for standard attention)
 *   total_suffix    host copy of cu_suffix_lens[B]
 *   max_suffix_len, max_prefix_len  host upper bounds over requests; every
 *                   request must lie within them (checked under
 *                   BAT_VALIDATE=1).  When B * max_suffix_len ==
 *                   total_suffix (all suffixes equally long) and no prefix
 *                   is split, the kernels place the work themselves and no
 *                   planner launch precedes them.
 *   out             device [total_suffix, H, D], dtype dt
 *   lse             device float32 [H, total_suffix] (natural log), or NULL
 *   workspace       device, >= bat_attn_workspace_size(...) bytes (or
 *                   bat_attn_prefill_workspace_size(...))
 * Supported: BAT_BF16 with D in {64, 128}; BAT_F32 with D in {32, 64, 128}.
 * Requests with no suffix tokens write nothing.  The result does not depend
 * on the physical placement of blocks, nor on where the work runs: the
 * reduction order of a row depends only on logical lengths.
 */
bat_status bat_attn_prefill(const void *q, const void *k, const void *v,
                            const int32_t *cu_suffix_lens,
                            const int32_t *prefix_lens,
                            const uint8_t *prefix_mode,
                            const int32_t *block_table, int32_t bt_stride,
                            const bat_kv_pool *user_pool,
                            const bat_kv_pool *item_pool, int32_t B, int32_t H,
                            int32_t D, bat_dtype dt, float softmax_scale,
                            int32_t total_suffix, int32_t max_suffix_len,
                            int32_t max_prefix_len, void *out, float *lse,
                            void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * bat_attn_prefill_noalloc -- bat_attn_prefill with no workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).
 *
 * Arguments, semantics, dtypes and head dims as bat_attn_prefill; the work
 * list and any split-prefix partials live in a device array inside the
 * library (bat_attn_noalloc_scratch_bytes() bytes, 32 MiB; one copy per
 * GPU, held until the process ends; its address is looked up on the first
 * call on each device).  The call allocates nothing.  When bat_attn_prefill
 * would split the prefixes and the partials do not fit, the rows are
 * computed unsplit (the same rows up to rounding); a batch whose unsplit
 * work list does not fit returns BAT_ERR_WORKSPACE.  Every call on one GPU
 * uses that GPU's one array: calls that overlap on one GPU (other streams,
 * other threads) race and must not be issued.
 */
bat_status bat_attn_prefill_noalloc(const void *q, const void *k,
                                    const void *v,
                                    const int32_t *cu_suffix_lens,
                                    const int32_t *prefix_lens,
                                    const uint8_t *prefix_mode,
                                    const int32_t *block_table,
                                    int32_t bt_stride,
                                    const bat_kv_pool *user_pool,
                                    const bat_kv_pool *item_pool, int32_t B,
                                    int32_t H, int32_t D, bat_dtype dt,
                                    float softmax_scale, int32_t total_suffix,
                                    int32_t max_suffix_len,
                                    int32_t max_prefix_len, void *out,
                                    float *lse, void *stream);

/* Bytes of the device array bat_attn_prefill_noalloc works in. */
size_t bat_attn_noalloc_scratch_bytes(void);

/*
 * An fp8 key/value pool: half the bytes of a bfloat16 pool, so twice the
 * cached prefixes fit in the same memory (the Bat page, "What it costs
 * (trade-offs and scope)", counts cache memory against item caches; the
 * pages prescribe no cache format).  Each (block, head) of the keys, and of
 * the values, holds OCP FP8 E4M3 codes and one scale 2^e, e the smallest
 * integer with amax <= 448 * 2^e (amax: that block's largest magnitude,
 * e = 0 for an all-zero block); a value x is the code nearest to x / 2^e
 * (ties to the even code, sign kept) and reads back as code value * 2^e,
 * which bfloat16 holds exactly.
 *   k, v               device uint8 [num_blocks, H, block_size, D], codes
 *   k_scale, v_scale   device float32 [num_blocks, H], the scales 2^e
 * Layout and addressing otherwise as bat_kv_pool.
 */
typedef struct bat_kv_pool_fp8 {
  void *k;
  void *v;
  float *k_scale;
  float *v_scale;
  int32_t num_blocks;
  int32_t block_size;
} bat_kv_pool_fp8;

/*
 * bat_kv_build_fp8 -- write prefix keys and values into an fp8 pool:
 * bat_kv_build's scatter, each (request, block of its tokens, head) turned
 * into codes with the block's own scale (a partial last block takes its
 * amax over the tokens it holds).  Arguments as bat_kv_build; k and v are
 * bfloat16 or float32 (dt) and D in {32, 64, 128}.  Each block must be named
 * by one table entry only (two requests sharing a block would each write
 * its scale).  Non-finite inputs give unspecified codes.
 */
bat_status bat_kv_build_fp8(const void *k, const void *v, const int32_t *cu_lens,
                            const int32_t *block_table, int32_t bt_stride,
                            int32_t B, int32_t H, int32_t D,
                            int32_t total_tokens, bat_dtype dt,
                            const bat_kv_pool_fp8 *pool, void *stream);

/* Bytes of device workspace bat_attn_prefill_fp8 needs (0: invalid). */
size_t bat_attn_fp8_workspace_size(int32_t B, int32_t H, int32_t D,
                                   int32_t total_suffix,
                                   int32_t max_suffix_len,
                                   int32_t max_prefix_len);

/*
 * bat_attn_prefill_fp8 -- bat_attn_prefill over fp8 pools: the same rows,
 * with each prefix key and value read back from its codes (code value *
 * scale, exact in bfloat16) on the way into the attention tiles.  The suffix
 * q, k, v and out are bfloat16 (D in {64, 128}); other arguments as
 * bat_attn_prefill, with workspace >= bat_attn_fp8_workspace_size(...).
 */
bat_status bat_attn_prefill_fp8(const void *q, const void *k, const void *v,
                                const int32_t *cu_suffix_lens,
                                const int32_t *prefix_lens,
                                const uint8_t *prefix_mode,
                                const int32_t *block_table, int32_t bt_stride,
                                const bat_kv_pool_fp8 *user_pool,
                                const bat_kv_pool_fp8 *item_pool, int32_t B,
                                int32_t H, int32_t D, float softmax_scale,
                                int32_t total_suffix, int32_t max_suffix_len,
                                int32_t max_prefix_len, void *out, float *lse,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * bat_attn_prefix_rows -- attention of the prefix rows over their prefix.
 *
 * The prefix rows of the bipartite mask: a prefix token sees every token of
 * its own request's prefix and nothing of the suffix (the UG-Separation
 * page's abstract: the tokens kept purely user-side are the ones whose
 * key/value cache can be reused; with no positions or causal mask on the Bat
 * page, the prefix attends bidirectionally within itself).  This is how the
 * cached keys/values of the next layer are produced from this layer's
 * prefix.  For an item prefix it is the prefix-wide form (every listed item
 * sees all of them); see bat_attn_item_local for items that see only
 * themselves.
 *
 *   q, k, v         device, packed prefix [total_prefix, H, D], dtype dt
 *   cu_prefix_lens  device int32 [B+1]: request r owns rows
 *                   cu_prefix_lens[r] .. cu_prefix_lens[r+1]
 *   softmax_scale   multiplies q.k
 *   total_prefix    host copy of cu_prefix_lens[B]; 0 is a no-op
 *   max_prefix_len  host upper bound over requests (> 0 unless total is 0)
 *   out             device [total_prefix, H, D], dtype dt
 *   lse             device float32 [H, total_prefix] (natural log), or NULL
 *   workspace       device, >= bat_attn_workspace_size(B, H, D, dt,
 *                   total_prefix, max_prefix_len, 0) bytes
 * Same kernels, dtypes and head dims as bat_attn_prefill.
 */
bat_status bat_attn_prefix_rows(const void *q, const void *k, const void *v,
                                const int32_t *cu_prefix_lens, int32_t B,
                                int32_t H, int32_t D, bat_dtype dt,
                                float softmax_scale, int32_t total_prefix,
                                int32_t max_prefix_len, void *out, float *lse,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * bat_attn_item_local -- attention of each cached item's tokens within that
 * item only (the per-item, block-diagonal variant of the prefix rows).
 *
 * The Bat page's item-as-prefix mode reuses popular items' key/value blocks
 * from a shared pool in whatever combination a request lists them
 * (sections "This paper's idea" and "Why it works"); an item's cached
 * keys/values beyond the first layer can only be shared that way when its
 * tokens attended to nothing but their own item.  Item i owns rows
 * i*T .. i*T+T-1 of the packed inputs; each such row sees exactly those T
 * keys: S_ab = softmax_scale * <q_a, k_b>, lse_a = ln sum_b exp(S_ab),
 * out_a = sum_b exp(S_ab - lse_a) v_b.
 *
 *   q, k, v          device, packed [n_items * T, H, D], dtype dt
 *   n_items          items; n_items * T rows and n_items * H (item, head)
 *                    pairs must stay below 2^31 (else BAT_ERR_INVALID_ARG)
 *   tokens_per_item  T, one of 1, 2, 4, 8 (else BAT_ERR_UNSUPPORTED)
 *   out              device [n_items * T, H, D], dtype dt
 *   lse              device float32 [H, n_items * T] (natural log), or NULL
 * Dtypes and head dims as bat_attn_prefill.  Needs no workspace.
 */
bat_status bat_attn_item_local(const void *q, const void *k, const void *v,
                               int32_t n_items, int32_t tokens_per_item,
                               int32_t H, int32_t D, bat_dtype dt,
                               float softmax_scale, void *out, float *lse,
                               void *stream);

/*
 * bat_attn_gqa_workspace_size -- bytes of device workspace
 * bat_attn_prefill_gqa needs.  Returns 0 for invalid arguments (including
 * H not a multiple of H_kv).
 */
size_t bat_attn_gqa_workspace_size(int32_t B, int32_t H, int32_t H_kv,
                                   int32_t D, bat_dtype dt,
                                   int32_t total_suffix,
                                   int32_t max_suffix_len,
                                   int32_t max_prefix_len);

/*
 * bat_attn_prefill_gqa -- bat_attn_prefill with grouped key/value heads.
 *
 * H query heads share H_kv key/value heads (H a multiple of H_kv): query
 * head h attends with key/value head h / (H / H_kv); everything else is
 * bat_attn_prefill's definition (the pages fix no head layout; this is the
 * grouped form of the same attention, with a cache H / H_kv times smaller).
 *
 *   q, out          device [total_suffix, H, D]; lse [H, total_suffix]
 *   k, v            device, packed fresh suffix [total_suffix, H_kv, D]
 *   user_pool, item_pool  pools of H_kv heads: [num_blocks, H_kv, bs, D]
 *                   (bat_kv_build with H = H_kv builds them)
 *   H, H_kv         query and key/value heads; H % H_kv == 0, else
 *                   BAT_ERR_INVALID_ARG
 *   workspace       >= bat_attn_gqa_workspace_size(B, H, H_kv, ...) bytes
 * Other arguments, dtypes and head dims as bat_attn_prefill.  The work of
 * the query heads that share a key/value head is placed on one XCD so that
 * their key/value tiles are read from HBM once.
 */
bat_status bat_attn_prefill_gqa(const void *q, const void *k, const void *v,
                                const int32_t *cu_suffix_lens,
                                const int32_t *prefix_lens,
                                const uint8_t *prefix_mode,
                                const int32_t *block_table, int32_t bt_stride,
                                const bat_kv_pool *user_pool,
                                const bat_kv_pool *item_pool, int32_t B,
                                int32_t H, int32_t H_kv, int32_t D,
                                bat_dtype dt, float softmax_scale,
                                int32_t total_suffix, int32_t max_suffix_len,
                                int32_t max_prefix_len, void *out, float *lse,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * bat_attn_isolated_workspace_size -- bytes of device workspace
 * bat_attn_prefill_isolated needs (the work list plus one fp32 prefix
 * partial per suffix row and head).  Returns 0 for invalid arguments.
 */
size_t bat_attn_isolated_workspace_size(int32_t B, int32_t H, int32_t D,
                                        bat_dtype dt, int32_t total_suffix,
                                        int32_t max_suffix_len,
                                        int32_t max_prefix_len);

/*
 * bat_attn_prefill_isolated -- suffix rows over the cached prefix and their
 * own candidate only (candidate-isolated suffix).
 *
 * The suffix of a recommendation request is a list of candidate items
 * scored together (Bat page, "This paper's idea": the item tokens are the
 * candidates; order-agnostic, so no positions).  Where candidates must be
 * scored independently of one another, each candidate's T tokens see the
 * request's prefix and themselves, not the other candidates: for a row i of
 * candidate c of request r,
 *     visible keys = P(r) + the T tokens of c,
 *     lse_i = ln sum_visible exp(S_ij), out_i = sum_visible exp(S_ij - lse_i) v_j.
 * Candidate c of request r is suffix rows cu_suffix_lens[r] + c*T ..
 * + c*T + T-1; every request's suffix length must be a multiple of T (the
 * result is unspecified otherwise).  Computed as the prefix part of every
 * row (the attention kernels over the prefix only, fp32 partials in the
 * workspace) merged exactly with each candidate's own part; for T = 1 in
 * bf16 the attention kernel folds the row's own key into its prefix result
 * and writes the row in the same launch.
 *
 *   Arguments as bat_attn_prefill, plus
 *   tokens_per_candidate  T, one of 1, 2, 4, 8 (else BAT_ERR_UNSUPPORTED);
 *                   total_suffix must be a multiple of T
 *   workspace       device, >= bat_attn_isolated_workspace_size(...) bytes
 */
bat_status bat_attn_prefill_isolated(const void *q, const void *k, const void *v,
                                     const int32_t *cu_suffix_lens,
                                     const int32_t *prefix_lens,
                                     const uint8_t *prefix_mode,
                                     const int32_t *block_table,
                                     int32_t bt_stride,
                                     const bat_kv_pool *user_pool,
                                     const bat_kv_pool *item_pool, int32_t B,
                                     int32_t H, int32_t D, bat_dtype dt,
                                     float softmax_scale,
                                     int32_t tokens_per_candidate,
                                     int32_t total_suffix,
                                     int32_t max_suffix_len,
                                     int32_t max_prefix_len, void *out,
                                     float *lse, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * bat_lse_merge -- combine n_parts attention partials over disjoint key sets
 * into one result (the log-sum-exp merge; it is how a prefix split across
 * workgroups, or across devices, is recombined, and it is exact: merging the
 * prefix partial with the suffix partial gives the same rows as attending to
 * both at once).
 *
 *   o_parts    device float32 [n_parts, rows, H, D], each part normalised
 *              over its own keys
 *   lse_parts  device float32 [n_parts, H, rows], natural log; -inf marks an
 *              empty part (contributes nothing)
 *   out        device [rows, H, D] in dtype dt
 *   lse        device float32 [H, rows] or NULL
 * lse = ln sum_p exp(lse_p); out = sum_p exp(lse_p - lse) o_p.
 */
bat_status bat_lse_merge(const float *o_parts, const float *lse_parts,
                         int32_t n_parts, int32_t rows, int32_t H, int32_t D,
                         bat_dtype dt, void *out, float *lse, void *stream);

/*
 * Prefix-mode choice (host side).
 *
 * The Bat page (sections "The idea" and "Why it works") has a hotness-aware
 * scheduler pick, per query and under memory limits, the user history or the
 * query's items as the cached prefix, favouring caches that are hot and
 * resident; user-prefix and item-prefix caches live in separate pools.  The
 * page gives no policy in detail.  These calls implement one plain reading,
 * query by query in arrival order:
 *   score  the prefix tokens that are hot: resident, or asked for by an
 *          earlier query and able to stay resident.  User mode: n_u if the
 *          user is resident, or was asked for before and its blocks fit the
 *          user pool, else 0; item mode: T per item of the query that is
 *          resident, or was asked for before while the item pool has slots.
 *          Item mode only on a strictly larger score (BAT_POLICY_HOTNESS);
 *          BAT_POLICY_USER_PREFIX always picks the user (the conventional
 *          baseline).  requests_x counts the earlier queries naming x.
 *   cache  only the chosen prefix: the user pool evicts least recently used
 *          users until ceil(n_u / user_block) blocks fit (a user larger
 *          than the pool is never kept); each missing item takes the lowest
 *          unused slot, else replaces the resident item, not of this query,
 *          with the fewest requests, then least recent use, then lowest id,
 *          if that item had strictly fewer requests than the newcomer.
 *   count  the user and every item of the query gain one request.
 *   work   user mode: prefix tokens computed = 0 on a hit else n_u, suffix
 *          tokens = m*T, query-key pairs = (0 or n_u^2) + m*T*(n_u + m*T);
 *          item mode: prefix = T*(m - hits), suffix = n_u,
 *          pairs = (m - hits)*T^2 + n_u*(n_u + m*T).
 * All state lives in a caller-owned host buffer (no allocation, no hidden
 * state); one buffer serves one stream of queries, calls on the same buffer
 * must not overlap.
 */
typedef enum bat_sched_policy {
  BAT_POLICY_USER_PREFIX = 0, /* always the user history (baseline) */
  BAT_POLICY_HOTNESS = 1      /* the scoring above */
} bat_sched_policy;

typedef struct bat_sched_config {
  int32_t policy;               /* bat_sched_policy */
  int32_t item_tokens;          /* T > 0, tokens per item */
  int32_t user_block;           /* > 0, tokens per user-pool block */
  int32_t item_capacity;        /* >= 0, item-pool slots */
  int64_t user_capacity_blocks; /* >= 0, user-pool blocks */
  int32_t num_users;            /* >= 0, user ids are 0 .. num_users-1 */
  int32_t num_items;            /* >= 0, item ids are 0 .. num_items-1 */
} bat_sched_config;

/* Bytes of host state for cfg; 0 if cfg is NULL or invalid. */
size_t bat_sched_state_size(const bat_sched_config *cfg);

/*
 * bat_sched_init -- empty pools, zero request counts.
 *   user_len  host int32 [num_users], history tokens per user (>= 0)
 *   state     host buffer, 8-byte aligned, >= bat_sched_state_size(cfg)
 *             bytes, owned by the caller (BAT_ERR_WORKSPACE if smaller)
 */
bat_status bat_sched_init(const bat_sched_config *cfg, const int32_t *user_len,
                          void *state, size_t state_bytes);

/*
 * bat_sched_step -- serve R queries of m items each, in order; the state
 * carries over between calls (the query clock continues).
 *   user      host int32 [R], ids < num_users
 *   items     host int32 [R, m], ids < num_items, distinct within a query
 *   outputs   host arrays, each may be NULL:
 *             mode [R] uint8 (bat_prefix_mode), user_hit [R] uint8,
 *             item_hits [R] int32 (the query's resident items when it
 *             arrived, whatever the mode), prefix_tokens / suffix_tokens /
 *             pairs [R] int64 (the work above), item_slot [R, m] int32
 *             (item mode: the slot each item is read from or was stored
 *             in; -1 for an item not kept and for every user-mode query).
 * Any out-of-range id or repeated item returns BAT_ERR_INVALID_ARG before
 * any query is served.
 */
bat_status bat_sched_step(void *state, int32_t R, int32_t m, const int32_t *user,
                          const int32_t *items, uint8_t *mode, uint8_t *user_hit,
                          int32_t *item_hits, int64_t *prefix_tokens,
                          int64_t *suffix_tokens, int64_t *pairs,
                          int32_t *item_slot);

/*
 * bat_sched_pools -- the pools' contents: resident users, most recently
 * used first (host int32 [num_users] or NULL), their number, and the item
 * in each item-pool slot (host int32 [item_capacity] or NULL; -1 unused).
 */
bat_status bat_sched_pools(const void *state, int32_t *resident_users,
                           int32_t *n_resident_users, int32_t *slot_item);

/* Human-readable name of a status code (static storage, never NULL). */
const char *bat_status_string(bat_status s);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
int32_t bat_version(void);

/*
 * The name of the last HIP runtime error a library call saw in the calling
 * thread ("hipSuccess" if none): the cause behind a BAT_ERR_HIP.  Static
 * storage, never NULL.
 */
const char *bat_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BAT_H_ */
