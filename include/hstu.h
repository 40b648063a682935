/*
 * hstu.h - C ABI of the HSTU attention library for AMD Instinct MI355X (gfx950).
 *
 * The library computes HSTU pointwise SiLU attention over jagged user
 * sequences and its two serving variants. The operation, per user sequence b
 * and head h (local indices, keys j allowed by the mask of the variant):
 *
 *   s_ij = alpha * <q_i, k_j> + P[min(p_i - p_j, n_pos - 1)]
 *                             + T[min(floor(log2(|ts_i - ts_j| + 1)), n_time - 1)]
 *   o_i  = sum_j SiLU(s_ij) / N_b * v_j          (masked pairs contribute 0)
 *   y_i  = (LayerNorm_{H*d}(o_i) * ln_w + ln_b) (elementwise *) u_i
 *
 * Sources. SiLU weighting in place of softmax, relative attention bias and
 * elementwise gating before the output projection: "Generative recommenders
 * at scale", section "Inside NVIDIA's GPU-native stack for HSTU and Semantic
 * IDs", and "How Generative Recommenders Are Redefining RecSys at Scale",
 * Takeaways. Timestamp-ordered user histories: the latter page's
 * description. Reuse of a cached prefix with a paged GPU table and append:
 * "Deploying an HSTU Generative Recommender with NVIDIA Dynamo-Triton",
 * section "Technical Stack and Performance Gains", and page
 * "recomendador-generativo-hstu-dynamo-triton", section "Como o recomendador
 * generativo HSTU reutiliza o histórico". M-FALCON candidate scoring by a
 * changed mask and bias: "HSTU Generative Recommenders: Deploy on GPU Cloud",
 * section "M-FALCON: Microbatched Attention for Scoring Multiple Candidates
 * at Once". The pages print no formula; N_b, the bucket functions and the
 * norm are the plain readings stated with each entry point.
 *
 * Conventions shared by every entry point
 *   - Tokens are packed back to back ("jagged"): Q, K, V are [T, H, d] row
 *     major (d fastest), U and Y are [T, H*d]. seq_offsets[b] is the first row
 *     of user b, seq_offsets[0] = 0, seq_offsets[B] = T, non-decreasing.
 *   - dtype HSTU_BF16: Q, K, V, U, Y and the K/V pages hold bf16; arithmetic
 *     is bf16 products with fp32 accumulation (the SiLU weights are rounded
 *     to bf16 before the second product). HSTU_F32: everything fp32.
 *   - All pointers except `params` and the hstu_kv_cache_t struct itself are
 *     device pointers. Bias tables, LayerNorm weights, offsets, lengths and
 *     the page table are device memory too.
 *   - Every call is asynchronous on `stream`, performs no host
 *     synchronisation and allocates nothing: the caller owns all buffers,
 *     including the workspace (hstu_attn_fwd_cached_noalloc alone uses a
 *     scratch array the library holds instead). Calls with different workspaces may run
 *     concurrently; calls sharing a workspace must be ordered on one stream.
 *     No call records a memset, so a caller may capture a sequence of calls
 *     (for example hstu_kv_append then hstu_attn_fwd_cached) into a HIP graph
 *     and replay it; the buffers named at capture time are the ones used.
 *   - Errors: argument checks run on the host before anything is launched and
 *     return a status; nothing is launched then. HSTU_ERR_LAUNCH reports a
 *     failed kernel launch. Device-side content (offsets, lengths, page
 *     indices, timestamps) is trusted: page indices outside [0, num_pages)
 *     read as zero keys and are never written, but inconsistent offsets or
 *     lengths are undefined behaviour.
 *   - Debug mode: with HSTU_DEBUG=1 in the environment (read at every call),
 *     hstu_attn_fwd, hstu_attn_fwd_cached, hstu_mfalcon_fwd,
 *     hstu_mfalcon_fwd_cached and hstu_attn_bwd first check that content on
 *     the device and write the result, an int32 of hstu_debug_bits_t, at byte
 *     HSTU_WS_DEBUG_FLAG_OFFSET of the workspace (0: valid). When it is not 0
 *     no attention work runs (Y, or the gradients, then hold unspecified but
 *     finite-sized garbage, and no memory outside the given buffers is read
 *     or written). The call stays asynchronous: read the word after the
 *     stream has finished. hstu_layer_fwd checks through its attention call.
 *   - Timestamps are int64 seconds. Within one user any two timestamps must
 *     differ by less than 2^62.
 */
#ifndef HSTU_H_
#define HSTU_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HSTU_OK = 0,
  HSTU_ERR_INVALID_ARG = 1,  /* NULL pointer, negative size, bad alignment  */
  HSTU_ERR_UNSUPPORTED = 2,  /* dtype / head_dim / table size not supported */
  HSTU_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required  */
  HSTU_ERR_LAUNCH = 4        /* a kernel launch failed                      */
} hstu_status_t;

typedef enum { HSTU_F32 = 0, HSTU_BF16 = 1 } hstu_dtype_t;

/* Debug mode (HSTU_DEBUG=1): where the content-check result sits in the
 * workspace, and its bits. */
#define HSTU_WS_DEBUG_FLAG_OFFSET 128
typedef enum {
  HSTU_DEBUG_BAD_OFFSETS = 1,     /* offsets[0] != 0, decreasing, or offsets[B] != total rows */
  HSTU_DEBUG_BAD_LENGTH = 2,      /* a user's rows above max_len (max_new, max_cand)           */
  HSTU_DEBUG_BAD_CANDIDATES = 4,  /* num_candidates[b] outside [0, L_b]                        */
  HSTU_DEBUG_BAD_CACHE_LEN = 8,   /* cache (history) length < 0 or keys above max_total       */
  HSTU_DEBUG_BAD_PAGE = 16        /* a needed page missing from the table or not in the pool  */
} hstu_debug_bits_t;

/* Which entry point a workspace is sized for. */
typedef enum {
  HSTU_FN_FULL = 0,
  HSTU_FN_CACHED = 1,
  HSTU_FN_MFALCON = 2,
  HSTU_FN_MFALCON_CACHED = 3,
  HSTU_FN_FULL_BWD = 4
} hstu_fn_t;

/*
 * Layer parameters shared by every attention entry point.
 *   num_heads     H >= 1
 *   head_dim      d in {32, 64, 128}; H*d <= 2048
 *   dtype         hstu_dtype_t
 *   alpha         scale of <q, k>; 1.0 in the plain reading
 *   norm_n        0: N_b is per user (full: L_b; cached: C_b + M_b;
 *                 M-FALCON: n_b + 1). > 0: that fixed N for every user.
 *   pos_tab       NULL (no position bias) or fp32 [H][pos_head_stride] with
 *                 n_pos valid entries per head; pos_head_stride = 0 shares one
 *                 table across heads. 1 <= n_pos <= 2048.
 *   time_tab      NULL (no time bias) or fp32 likewise; n_time >= 1 (entries
 *                 beyond index 63 are unreachable for int64 seconds).
 *   ln_w, ln_b    NULL for 1 / 0, else fp32 [H*d] affine terms of the norm.
 *   ln_eps        LayerNorm epsilon (1e-5 in the plain reading), > 0.
 *   timing_events optional hipEvent_t handles (cast to void*), each NULL to
 *                 skip, recorded on the stream: [0] before the tile scheduler,
 *                 [1] before the fused attention kernel, [2] after it, [3]
 *                 after the LayerNorm/gating epilogue. For timing the kernels
 *                 of one call separately; the library never waits on them.
 *   flags         0, or HSTU_FLAG_FP32_NORM_INPUT. How the attention kernel
 *                 hands its output to the norm on the bf16 full and M-FALCON
 *                 paths: by default the attention store is norm-ready (per
 *                 token and head, the mean and the sum of squared deviations
 *                 of the head's d values, computed from the fp32
 *                 accumulators, plus the deviations rounded to bf16), and the
 *                 norm kernel only merges the heads' statistics and applies
 *                 the affine terms and U. With the flag the attention output
 *                 makes an fp32 round trip instead (twice the bytes); the two
 *                 agree within bf16 rounding of the deviations. fp32 layers,
 *                 the split paged paths and the backward always use fp32.
 *                 HSTU_FLAG_SAVED_FORWARD (read by hstu_attn_bwd only): see
 *                 hstu_attn_bwd. Other bits: HSTU_ERR_INVALID_ARG.
 */
typedef struct {
  int32_t num_heads;
  int32_t head_dim;
  int32_t dtype;
  float alpha;
  int32_t norm_n;
  const float* pos_tab;
  int32_t n_pos;
  int32_t pos_head_stride;
  const float* time_tab;
  int32_t n_time;
  int32_t time_head_stride;
  const float* ln_w;
  const float* ln_b;
  float ln_eps;
  void* timing_events[4];
  int32_t flags;
} hstu_params_t;

/* hstu_params_t.flags bits */
#define HSTU_FLAG_FP32_NORM_INPUT 1
#define HSTU_FLAG_SAVED_FORWARD 2

/*
 * Paged KV cache ("paged GPU table", page "recomendador-generativo-hstu-
 * dynamo-triton", section "Como o recomendador generativo HSTU reutiliza o
 * histórico"). Logical token position p of user b lives in page
 * page_table[b * max_pages_per_seq + p / page_size] at slot p % page_size.
 *   k_pages, v_pages  [num_pages, H, page_size, d] in the layer dtype
 *   ts_pages          int64 [num_pages, page_size]
 *   page_table        int32 [batch, max_pages_per_seq]; -1 = no page
 *   num_pages, max_pages_per_seq  >= 1
 *   page_size         must be 64
 * The caller owns the pages and the table and decides which pages a user
 * holds; the library never allocates, frees or evicts pages.
 */
typedef struct {
  void* k_pages;
  void* v_pages;
  int64_t* ts_pages;
  const int32_t* page_table;
  int32_t num_pages;
  int32_t page_size;
  int32_t max_pages_per_seq;
} hstu_kv_cache_t;

/* Human-readable name of a status code (static string). */
const char* hstu_status_string(hstu_status_t status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t hstu_version(void);

/*
 * Workspace bytes needed by one call of entry point `fn`.
 *   batch           number of users B
 *   total_q_tokens  query rows T (full, M-FALCON) or new rows (cached)
 *   max_len         longest user: L (full), history + candidates (M-FALCON),
 *                   cache_len + new tokens (cached)
 * Returns 0 when the arguments are invalid. The value depends only on these
 * arguments and never decreases when one of them grows, so a workspace sized
 * once for the largest call serves every smaller one.
 */
size_t hstu_workspace_size(int32_t fn, const hstu_params_t* params, int32_t batch,
                           int64_t total_q_tokens, int32_t max_len);

/*
 * Full causal path: every token attends to itself and the earlier tokens of
 * its own user; N_b = L_b (unless params->norm_n > 0).
 *   seq_offsets  int32 [batch + 1]
 *   max_len      >= every L_b (only used to size the launch)
 *   total_tokens T = seq_offsets[batch]
 *   q, k, v      [T, H, d]; u, y: [T, H*d]; ts: int64 [T]
 *   ws, ws_bytes workspace of at least hstu_workspace_size(HSTU_FN_FULL, ...)
 * y must not alias any input. All tensors 16-byte aligned.
 */
hstu_status_t hstu_attn_fwd(const hstu_params_t* params, int32_t batch, const int32_t* seq_offsets,
                            int32_t max_len, int64_t total_tokens, const void* q, const void* k,
                            const void* v, const void* u, const int64_t* ts, void* y, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * Gradients written by hstu_attn_bwd. dq, dk, dv: [T, H, d]; du: [T, H*d];
 * all bf16. d_pos_tab and d_time_tab are fp32 with the layout of
 * params->pos_tab / time_tab ([n] when the head stride is 0, else [H][stride];
 * entries past n_pos / n_time in a row are left untouched); each may be NULL
 * to skip that gradient and must be NULL when its table is. d_ln_w, d_ln_b:
 * fp32 [H*d], NULL to skip, NULL when the matching affine term is. Every
 * requested gradient is overwritten, not accumulated.
 */
typedef struct {
  void* dq;
  void* dk;
  void* dv;
  void* du;
  float* d_pos_tab;
  float* d_time_tab;
  float* d_ln_w;
  float* d_ln_b;
} hstu_grads_t;

/*
 * Backward of hstu_attn_fwd (training). Given the forward's inputs and dy,
 * the gradient of the loss with respect to y, writes the gradients of q, k,
 * v, u, the bias tables and the norm's affine terms. The pages print no
 * backward; it is the chain rule of the forward (pointwise SiLU attention
 * with relative bias, "Generative recommenders at scale", section "Inside
 * NVIDIA's GPU-native stack for HSTU and Semantic IDs"; norm and gating, "How
 * Generative Recommenders Are Redefining RecSys at Scale", Takeaways), for
 * the training workload of "HSTU Generative Recommenders: Deploy on GPU
 * Cloud", section "Scaling Training and Serving Across Multiple GPUs".
 * The attention output is recomputed inside the call (nothing is saved
 * between forward and backward).
 *   arguments as hstu_attn_fwd, plus dy [T, H*d] and grads (see above)
 *   ws, ws_bytes  workspace of at least hstu_workspace_size(HSTU_FN_FULL_BWD, ...)
 * For head_dim 128 the workspace also holds the bf16 gradient of the scores
 * of every causal 64 x 64 (key, query) block, written by the dK/dV pass and
 * read by the dQ pass (about H * sum_b L_b^2 bytes, sized from batch,
 * total_tokens and max_len). There max_len must bound every L_b: a longer
 * user leaves the gradients unspecified (debug mode reports it) while no
 * memory outside the given buffers is read or written.
 * bf16 only (HSTU_ERR_UNSUPPORTED for fp32) and n_pos <= 512. Outputs must
 * not alias inputs. All tensors 16-byte aligned. Results do not depend on
 * scheduling: every sum runs in a fixed order. params->timing_events, if
 * set, are recorded [0] before the recomputed forward, [1] before the norm
 * backward, [2] before the attention backward, [3] at the end.
 * Saved forward (params->flags & HSTU_FLAG_SAVED_FORWARD): ws must be the
 * workspace that an hstu_attn_fwd call with the same params (bar this bit),
 * batch, seq_offsets, max_len, total_tokens and q, k, v, u, ts used last,
 * unchanged since (a workspace sized for the backward also serves the
 * forward). That call left its norm-ready attention store there (per token
 * and head the mean and sum of squared deviations, and the bf16 deviations);
 * the backward then does not recompute the attention forward and takes the
 * norm backward's input from it. With HSTU_FLAG_FP32_NORM_INPUT also set:
 * HSTU_ERR_INVALID_ARG. Anything else in ws leaves the gradients
 * unspecified (no memory outside the given buffers is touched).
 */
hstu_status_t hstu_attn_bwd(const hstu_params_t* params, int32_t batch, const int32_t* seq_offsets,
                            int32_t max_len, int64_t total_tokens, const void* q, const void* k,
                            const void* v, const void* u, const int64_t* ts, const void* dy,
                            const hstu_grads_t* grads, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Paged KV append: new token m of user b (packed row new_offsets[b] + m)
 * is written at logical position cache_lens[b] + m of that user's pages:
 * its K and V rows for every head, and its timestamp.
 *   new_offsets  int32 [batch + 1] over the packed new tokens
 *   cache_lens   int32 [batch], length of each user's cache before this call
 *   k_new, v_new [T_new, H, d]; ts_new int64 [T_new]
 * The table must already hold pages for positions up to cache_lens[b] +
 * M_b - 1; positions whose page index is outside [0, num_pages) are skipped.
 * cache_lens is not updated (the caller advances it).
 */
hstu_status_t hstu_kv_append(const hstu_kv_cache_t* cache, const hstu_params_t* params, int32_t batch,
                             const int32_t* new_offsets, const int32_t* cache_lens, int64_t total_new,
                             const void* k_new, const void* v_new, const int64_t* ts_new,
                             hipStream_t stream);

/*
 * KV-cache delta path: the M_b new tokens of user b, already appended with
 * hstu_kv_append, attend causally to the C_b = cache_lens[b] cached tokens
 * and to themselves. Query m sits at position C_b + m and sees keys
 * 0 .. C_b + m, all read from the pages; N_b = C_b + M_b. The result equals
 * rows C_b .. C_b + M_b - 1 of the full path over the user's C_b + M_b
 * tokens.
 *   new_offsets  int32 [batch + 1] over the packed new tokens
 *   max_new      >= every M_b;  max_total >= every C_b + M_b
 *   q_new        [T_new, H, d]; u_new, y_new [T_new, H*d]; ts_new int64 [T_new]
 */
hstu_status_t hstu_attn_fwd_cached(const hstu_params_t* params, int32_t batch, const int32_t* new_offsets,
                                   const int32_t* cache_lens, int32_t max_new, int32_t max_total,
                                   int64_t total_new, const void* q_new, const void* u_new,
                                   const int64_t* ts_new, const hstu_kv_cache_t* cache, void* y_new,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the KV-cache
 * delta path of hstu_attn_fwd_cached, same arguments and same result, without
 * the workspace argument. Its scratch is a device array inside the library
 * of HSTU_NOALLOC_SCRATCH_BYTES per GPU, held from the first call on that GPU
 * until the process ends; the call itself allocates nothing. A call whose
 * workspace size (hstu_workspace_size(HSTU_FN_CACHED, ...)) exceeds it
 * returns HSTU_ERR_WORKSPACE before touching the GPU. The KV-delta serving
 * shape (8 users x 128 new tokens, 8,192 cached, 4 heads x 128) needs 32.1
 * MiB. Nothing in the scratch has to start at zero: every call writes what
 * it reads. In debug mode the check result goes to the scratch too, where
 * the caller cannot read it: debug with hstu_attn_fwd_cached. All calls on one GPU share its array, which keeps the last
 * call's contents: calls that overlap on one GPU (different streams without
 * ordering, or different host threads) race; order them on one stream.
 */
#define HSTU_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
hstu_status_t hstu_attn_fwd_cached_noalloc(const hstu_params_t* params, int32_t batch,
                                           const int32_t* new_offsets, const int32_t* cache_lens,
                                           int32_t max_new, int32_t max_total, int64_t total_new,
                                           const void* q_new, const void* u_new, const int64_t* ts_new,
                                           const hstu_kv_cache_t* cache, void* y_new, hipStream_t stream);

/*
 * M-FALCON candidate path. User b spans rows [history (n_b) | candidates
 * (m_b = num_candidates[b])]. History rows are causal over the history.
 * Every candidate sits at position n_b, attends to all n_b history keys
 * (relative position n_b - j) and to itself (relative position 0, time
 * difference 0), and to no other candidate. N_b = n_b + 1 for all rows of
 * the user. Each candidate row therefore equals the last row of the full
 * path on [history | that candidate].
 *   num_candidates  int32 [batch], 0 <= m_b <= L_b
 *   other arguments as in hstu_attn_fwd (max_len >= n_b + m_b)
 */
hstu_status_t hstu_mfalcon_fwd(const hstu_params_t* params, int32_t batch, const int32_t* seq_offsets,
                               const int32_t* num_candidates, int32_t max_len, int64_t total_tokens,
                               const void* q, const void* k, const void* v, const void* u,
                               const int64_t* ts, void* y, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/*
 * M-FALCON over a paged history: the candidates of user b (packed rows
 * cand_offsets[b] .. cand_offsets[b+1]) are scored against the user's
 * n_b = hist_lens[b] history tokens already in the paged cache ("HSTU
 * Generative Recommenders: Deploy on GPU Cloud", section "M-FALCON:
 * Microbatched Attention for Scoring Multiple Candidates at Once", with the
 * history kept in the paged GPU table of page "recomendador-generativo-hstu-
 * dynamo-triton", section "Como o recomendador generativo HSTU reutiliza o
 * histórico"). Every candidate sits at position n_b, attends to history keys
 * 0 .. n_b - 1 (read from the pages, relative position n_b - j) and to
 * itself (relative position 0, time difference 0), and to no other
 * candidate; N_b = n_b + 1. Each output row therefore equals the candidate's
 * row of hstu_mfalcon_fwd on [history | candidates].
 *   cand_offsets      int32 [batch + 1] over the packed candidate rows
 *   hist_lens         int32 [batch], history tokens in the cache (may be 0)
 *   max_cand          >= every candidate count; max_hist >= every n_b
 *   q, k, v           [T_cand, H, d] candidates' own query, key, value rows
 *   u, y              [T_cand, H*d]; ts int64 [T_cand] candidate timestamps
 *   ws                hstu_workspace_size(HSTU_FN_MFALCON_CACHED, params,
 *                     batch, T_cand, max_hist) bytes
 * Nothing is appended to the cache: candidates are scored, not stored.
 */
hstu_status_t hstu_mfalcon_fwd_cached(const hstu_params_t* params, int32_t batch, const int32_t* cand_offsets,
                                      const int32_t* hist_lens, int32_t max_cand, int32_t max_hist,
                                      int64_t total_cand, const void* q, const void* k, const void* v,
                                      const void* u, const int64_t* ts, const hstu_kv_cache_t* cache, void* y,
                                      void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Page manager of the paged KV cache (host side). It decides which pages of a
 * pool of num_pages hold which user's history and evicts the least recently
 * used users when the pool or the user slots run out: the lookup / allocate /
 * append / evict operations of the paged GPU table on page
 * "recomendador-generativo-hstu-dynamo-triton", section "Como o recomendador
 * generativo HSTU reutiliza o histórico". It moves page ids only: the K, V and
 * timestamp bytes stay in the device pools that hstu_kv_append writes. One
 * manager serves every layer of a model (each layer has its own pools indexed
 * by the same page ids). All functions are host-only, thread-safe, and never
 * touch the GPU. Users are 64-bit ids; pages hold 64 tokens.
 *
 * A serving step for a batch of users:
 *   1. hstu_pm_reserve(batch ids, new token counts) -> each user's cached
 *      length before this step and its page-table row ([batch,
 *      max_pages_per_seq] int32, -1 = none), with pages added for the new
 *      tokens; copy both to the device. A user evicted earlier (or never seen)
 *      comes back with cached length 0: the caller sends its whole history.
 *   2. per layer: hstu_kv_append, then hstu_attn_fwd_cached.
 *   3. hstu_pm_commit(batch ids, new token counts) advances the lengths.
 * A reserve replaces the user's earlier reservation if that was never
 * committed (or committed for fewer tokens): the row then holds exactly
 * ceil((cached length + new tokens) / 64) pages, reusing the pages reserved
 * before and returning the rest to the pool. Reserved pages are never lost:
 * they stay with the user until its next reserve or its eviction.
 * Every lookup, and every user of a reserve in batch order, counts as a use;
 * eviction takes the least recently used user outside the request. Users of
 * the batch are never evicted by their own reserve. A reserve that
 * cannot fit even after evicting every other user returns
 * HSTU_ERR_WORKSPACE and changes nothing; a user whose history would exceed
 * max_pages_per_seq pages gives HSTU_ERR_UNSUPPORTED; duplicate ids in one
 * call give HSTU_ERR_INVALID_ARG.
 */
typedef struct hstu_page_manager hstu_page_manager_t;

/* NULL when an argument is < 1 or memory runs out. */
hstu_page_manager_t* hstu_pm_create(int32_t num_pages, int32_t max_pages_per_seq, int32_t max_users);
void hstu_pm_destroy(hstu_page_manager_t* pm);
/* cache_lens: [batch] out; page_table: [batch, max_pages_per_seq] out; evicted: users evicted (may be NULL) */
hstu_status_t hstu_pm_reserve(hstu_page_manager_t* pm, int32_t batch, const int64_t* user_ids,
                              const int32_t* n_new, int32_t* cache_lens, int32_t* page_table, int32_t* evicted);
hstu_status_t hstu_pm_commit(hstu_page_manager_t* pm, int32_t batch, const int64_t* user_ids,
                             const int32_t* n_new);
/* cached length of a user (marks it recently used), or -1 when not resident */
int32_t hstu_pm_lookup(hstu_page_manager_t* pm, int64_t user_id);
/* drop a resident user and free its pages; HSTU_ERR_INVALID_ARG if absent */
hstu_status_t hstu_pm_evict(hstu_page_manager_t* pm, int64_t user_id);
/* free pages, resident users, evictions so far (each may be NULL) */
hstu_status_t hstu_pm_stats(hstu_page_manager_t* pm, int32_t* free_pages, int32_t* users, int64_t* evictions);

/*
 * Full HSTU layer ("How Generative Recommenders Are Redefining RecSys at
 * Scale", Takeaways: elementwise gating before the output projection;
 * "Generative recommenders at scale", section "Inside NVIDIA's GPU-native
 * stack for HSTU and Semantic IDs"). With E = embed_dim and HD = H*d:
 *
 *   [U | V | Q | K] = SiLU(X W1)        X [T, E], W1 [E, 4*HD], split in
 *                                       this column order, each [T, HD]
 *   A = hstu_attn_fwd(Q, K, V, U, ts)   the full causal path above
 *   out = A W2                          W2 [HD, E], out [T, E]
 *
 * f1 and f2 have no bias term. weights->products picks where the two
 * products run: HSTU_PRODUCTS_HIPBLASLT (0, f1 with its SiLU epilogue, one
 * product per U/V/Q/K column block, each writing a packed [T, HD] buffer in
 * the workspace) or HSTU_PRODUCTS_OWN (1, hstu_matmul_bf16: f1 as one
 * product with SiLU and the U/V/Q/K split fused in its epilogue; needs
 * 4*H*d and E multiples of 256 and E and H*d multiples of 64, else
 * HSTU_ERR_UNSUPPORTED) or HSTU_PRODUCTS_AUTO (2: f1 on hstu_matmul_bf16
 * when those limits hold, else on hipBLASLt; f2 on hipBLASLt. On the
 * 16-user E = 1,024 layer the own kernel is the faster f1, whose SiLU and
 * split it fuses, and hipBLASLt the faster f2). The attention runs on this
 * library's kernels. Only HSTU_BF16 is supported (HSTU_ERR_UNSUPPORTED for
 * HSTU_F32): bf16 operands, fp32 accumulation, bf16 U, V, Q, K, A and out.
 *   weights->w1, weights->w2  row-major device matrices in bf16
 *   x    [T, E] bf16; ts int64 [T]; out [T, E] bf16 (must not alias x)
 *   ws   at least hstu_layer_workspace_size(...) bytes
 * params->timing_events, if set, are recorded [0] before f1, [1] before the
 * attention, [2] before f2, [3] after f2. The first call on a device
 * creates a hipBLASLt handle for it, kept until the process ends (the only
 * host state the library holds); later calls reuse it and the chosen GEMM
 * algorithms. Callable from several host threads.
 */
typedef enum { HSTU_PRODUCTS_HIPBLASLT = 0, HSTU_PRODUCTS_OWN = 1, HSTU_PRODUCTS_AUTO = 2 } hstu_products_t;

typedef struct {
  int32_t embed_dim;  /* E >= 1, multiple of 8 */
  const void* w1;     /* [E, 4 * H * d] */
  const void* w2;     /* [H * d, E] */
  int32_t products;   /* hstu_products_t */
} hstu_layer_weights_t;

/* Epilogues of hstu_matmul_bf16. */
typedef enum { HSTU_EPI_NONE = 0, HSTU_EPI_SILU_SPLIT = 1 } hstu_epilogue_t;

/*
 * The layer's dense product on the library's own MFMA kernel: C = A B with
 * A [M, K] and B [K, N] row-major bf16, fp32 accumulation, bf16 output.
 * Epilogues (the layer's f1 and f2: a pointwise projection with SiLU that
 * produces U, V, Q, K, and the output projection, "How Generative
 * Recommenders Are Redefining RecSys at Scale", Takeaways):
 *   HSTU_EPI_NONE        C is [M, N].
 *   HSTU_EPI_SILU_SPLIT  SiLU of every entry, then columns are split into
 *                        N / split_width blocks written one after another,
 *                        block i = columns [i*w, (i+1)*w) as [M, w]
 *                        (w = split_width; U, V, Q, K for w = H*d, N = 4w).
 * N must be a multiple of 256 and K of 64 (else HSTU_ERR_UNSUPPORTED);
 * split_width a multiple of 32 dividing N. M >= 0 (M = 0 does nothing).
 * Pointers 16-byte aligned; C must not alias A or B. No workspace; runs on
 * `stream`, allocates nothing.
 */
hstu_status_t hstu_matmul_bf16(int64_t M, int32_t N, int32_t K, const void* a, const void* b, void* c,
                               int32_t epilogue, int32_t split_width, hipStream_t stream);

/* Workspace bytes of hstu_layer_fwd; 0 for invalid arguments. Monotone in
 * every argument like hstu_workspace_size. */
size_t hstu_layer_workspace_size(const hstu_params_t* params, int32_t embed_dim, int32_t batch,
                                 int64_t total_tokens, int32_t max_len);

hstu_status_t hstu_layer_fwd(const hstu_params_t* params, const hstu_layer_weights_t* weights,
                             int32_t batch, const int32_t* seq_offsets, int32_t max_len,
                             int64_t total_tokens, const void* x, const int64_t* ts, void* out,
                             void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_H_ */
