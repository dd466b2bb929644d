/*
 * csa.h -- C ABI of libcsa.so: the Compressed Sparse Attention (CSA) hot path
 * of DeepSeek-V4 hybrid attention, its Heavily Compressed Attention (HCA)
 * variant and the DeepSeek-V3.2 token-level sparse attention (DSA), as
 * hand-written HIP kernels for MI355X (gfx950).
 *
 * The operations follow the Hugging Face Transformers model pages
 * "DeepSeek-V4" (sections "Hybrid attention (§2.3)", "Attention mask layout",
 * "Cache layers", DeepseekV4Config) and "DeepSeek-V3.2" (section "DeepSeek
 * Sparse Attention (DSA)", DeepseekV32Config).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library never allocates or frees device memory.  Its state is a
 *    thread-local error string and, for csa_sparse_attn_noalloc only, a static
 *    device array per GPU (see there).  Scratch space otherwise comes in
 *    through a caller-owned workspace argument.
 *  - Tensors are dense, row-major, innermost dimension contiguous, and 16-byte
 *    aligned.  Element type: `dtype` (CSA_F32 = fp32, CSA_BF16 = bfloat16)
 *    unless an argument says fp32 or int32 explicitly.
 *  - Positions: query row i of sequence b sits at absolute position
 *    t = q_pos[b] + i (q_pos is a device int32 array [B]).  Pool entry w
 *    covers the source block starting at token w*m of the sequence.
 *  - Readiness (page "DeepSeek-V4", "Attention mask layout"): the query at t
 *    may use pool entry w only when w < R(t) = min(T, floor((t+1)/m)).
 *  - RoPE (page "DeepSeek-V4", "Hybrid attention", partial RoPE): the trailing
 *    rope_dim channels of a row form interleaved pairs (2i, 2i+1) relative to
 *    channel D-rope_dim; pair i at position p is rotated by the angle
 *    p * theta^(-2i/rope_dim), i.e. (a, b) -> (a cos - b sin, a sin + b cos).
 *    Kernels read cos/sin from a table built by csa_rope_table.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work and return; they never synchronize.  Device faults surface at
 *    the caller's next synchronization.  (The debug build of the library,
 *    libcsa_debug.so, is the exception: before each attention launch it
 *    checks the index rows on the device, synchronizes the stream and returns
 *    CSA_ERR_INVALID for an entry outside [-1, T); it is not for graph
 *    capture.)
 *  - Every call returns a csa_status_t.  On a non-OK status nothing was
 *    enqueued and csa_last_error() describes the problem.  Calls never abort
 *    or throw.
 *  - Values read from device memory (q_pos, win_pos0, idx) cannot be checked
 *    on the host; the kernels treat them defensively: idx entries outside
 *    [0, T) count as empty slots, window rows outside [0, L_win) are absent,
 *    and a query row whose position lies outside the RoPE table is written as
 *    NaN.  No input value makes a kernel access memory out of bounds.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CSA_OK = 0,
    CSA_ERR_INVALID = 1,     /* bad pointer, size, alignment or combination */
    CSA_ERR_UNSUPPORTED = 2, /* valid, but no kernel is compiled for it */
    CSA_ERR_LAUNCH = 3       /* the HIP runtime rejected a launch */
} csa_status_t;

typedef enum { CSA_F32 = 0, CSA_BF16 = 1 } csa_dtype_t;

/* Text of the last non-OK status returned on the calling thread ("" if none). */
const char *csa_last_error(void);

/* Library version string. */
const char *csa_version(void);

/*
 * csa_rope_table -- cos/sin table for partial RoPE.
 * Page "DeepSeek-V4", "Hybrid attention" (partial RoPE on the trailing
 * qk_rope_head_dim channels) and DeepseekV4Config (rope_theta,
 * compress_rope_theta).
 *   cs       [n_pos][rope_dim/2][2] fp32, out: cs[p][i] = {cos a, sin a} with
 *            a = p * theta^(-2i/rope_dim), the angle formed and evaluated in
 *            fp64 and rounded once to fp32.
 *   n_pos >= 1, rope_dim even and >= 2, theta > 0.
 */
csa_status_t csa_rope_table(float *cs, int32_t n_pos, int32_t rope_dim, double theta,
                            void *stream);

/*
 * csa_rope_table_yarn -- the same table with YaRN-scaled frequencies.  Page
 * "DeepSeek-V4", DeepseekV4Config (compress_rope_theta is used together with
 * rope scaling for YaRN; rope_parameters carry the scaling for a longer
 * max_position_embeddings).  The pages name the method only; the frequencies
 * follow the published YaRN "NTK-by-parts" rule in its per-pair-index form:
 * with f_i = theta^(-2i/rope_dim) and i(r) = rope_dim ln(L / (2 pi r)) /
 * (2 ln theta) (L = original_max_pos), low = max(floor(i(beta_fast)), 0),
 * high = min(ceil(i(beta_slow)), rope_dim - 1) (+0.001 if equal),
 * ramp_i = clamp((i - low) / (high - low), 0, 1) and pair i turns at
 *   f'_i = (f_i / factor) ramp_i + f_i (1 - ramp_i),
 * i.e. fast pairs keep their frequency and slow pairs are stretched by the
 * factor.  The table stays a pure rotation (|cs[p][i]| = 1); YaRN's logit
 * temperature, a scalar, is the caller's to fold into the attention scale.
 * With factor = 1 the table equals csa_rope_table's.
 *   factor >= 1, original_max_pos >= 1, beta_fast > beta_slow > 0, theta > 1.
 */
csa_status_t csa_rope_table_yarn(float *cs, int32_t n_pos, int32_t rope_dim, double theta,
                                 double factor, int32_t original_max_pos, double beta_fast,
                                 double beta_slow, void *stream);

/*
 * csa_compress -- the compressor: pools a token stream into one entry per m
 * tokens.  Page "DeepSeek-V4", "Hybrid attention" (CSA pool at rate m with
 * overlapping windows; HCA pool at rate m' with non-overlapping windows) and
 * "Cache layers" (compressor buffer/pool/count, overlap state, the parallel
 * indexer compressor at index_head_dim).
 *   x         [B][S][D] dtype   token rows (K=V rows, or indexer key rows)
 *   gate      [B][S][D] dtype   per-channel gate logits, or NULL (all zero)
 *   slot_bias [(1+overlap)*m][D] fp32  per-slot logit bias, or NULL
 *   pool      [B][T][D] dtype   out, T = floor(S/m) complete windows
 *   overlap   1: entry w pools tokens [(w-1)m, (w+1)m) clipped at 0 (CSA);
 *             0: tokens [wm, (w+1)m) (HCA; with m=1 a plain copy)
 *   For every channel c the weights are softmax over the window of
 *   gate[j][c] + slot_bias[j-(w-overlap)m][c]; entry = sum_j weight_j x[j][c];
 *   then the trailing rope_dim channels are rotated to position pos0 + w*m
 *   (cs, n_pos: the RoPE table; unused when rope_dim == 0) and the entry is
 *   stored in dtype (round to nearest even for bf16).
 *   Requires D % 8 == 0, D <= 1024, m >= 1, rope_dim even, rope_dim <= D,
 *   pos0 >= 0 and pos0 + (T-1)*m < n_pos when rope_dim > 0.
 *   With m = 1, overlap = 0 and gate = NULL this rotates every token at its
 *   own position: the sliding-window K=V rows, and the DSA token keys.
 */
csa_status_t csa_compress(const void *x, const void *gate, const float *slot_bias,
                          void *pool, int32_t B, int32_t S, int32_t D, int32_t m,
                          int32_t overlap, int32_t rope_dim, const float *cs,
                          int32_t n_pos, int32_t pos0, int32_t dtype, void *stream);

/*
 * csa_compress_many -- several csa_compress passes in as few launches as
 * possible (a prefill step's window rows, K=V pool and index keys: one
 * launch).  Each pass has exactly csa_compress's arguments, meaning and
 * requirements and produces exactly its result; the passes must not write
 * memory another pass reads.  Passes the batched kernel takes (m = 1 copies
 * without gate or bias, and windows of (1+overlap)m = 4 or 8 tokens) share a
 * launch, up to four per launch; the others run as csa_compress runs them.
 * Every pass is checked before anything is enqueued.  n_passes <= 16.
 */
typedef struct {
    const void *x, *gate;
    const float *slot_bias;
    void *pool;
    int32_t B, S, D, m, overlap, rope_dim;
    const float *cs;
    int32_t n_pos, pos0;
} csa_compress_pass_t;

csa_status_t csa_compress_many(const csa_compress_pass_t *passes, int32_t n_passes,
                               int32_t dtype, void *stream);

/*
 * csa_cache_append -- the decode-time cache update: appends n tokens per
 * sequence to the compressor state, the pool and the sliding window.  Page
 * "DeepSeek-V4", "Cache layers" (a sliding window of K=V rows plus the
 * compressor's buffer / pool / count, with overlap state for CSA; the indexer
 * keys run the same compressor at index_head_dim).
 *   x, gate   [B][n][D] dtype   the new token rows (gate NULL: all zero)
 *   slot_bias [(1+overlap)*m][D] fp32, or NULL
 *   ring_x    [B][L][D] dtype   in/out, L = (1+overlap)*m: raw x of the last L
 *                               tokens, position p at row p mod L
 *   ring_g    [B][L][D] dtype   in/out, the same for gate; NULL iff gate NULL
 *   pool      [B][T_cap][D] dtype  in/out: entry w is written when token
 *                               (w+1)m-1 arrives, pooled exactly as
 *                               csa_compress pools it (pos0 = 0: positions
 *                               count from the first token); entries at or
 *                               past T_cap are not written
 *   win       [B][W][D] dtype   in/out, or NULL (W = 0): the last W tokens,
 *                               rotated at their positions, position p at row
 *                               p mod W -- the ring csa_sparse_attn reads when
 *                               its win_pos0 is NULL
 *   count     [B] int32         tokens appended before this call, per
 *                               sequence (read only: the caller adds n after
 *                               the call, e.g. with a device add)
 *   Rows at positions past the RoPE table (n_pos) are written as NaN when
 *   rope_dim > 0.  Two kernels in stream order (the entries read the ring
 *   before the new tokens overwrite it); calls on one cache must not overlap.
 *   Requires D % 8 == 0, D <= 1024, m >= 1, (1+overlap)*m <= 256, n >= 0.
 */
csa_status_t csa_cache_append(const void *x, const void *gate, const float *slot_bias,
                              void *ring_x, void *ring_g, void *pool, void *win,
                              const int32_t *count, int32_t B, int32_t n, int32_t D,
                              int32_t m, int32_t overlap, int32_t T_cap, int32_t W,
                              int32_t rope_dim, const float *cs, int32_t n_pos,
                              int32_t dtype, void *stream);

/*
 * csa_cache_append_many -- several csa_cache_append updates in as few launches
 * as possible (a decode step's K=V cache and index-key cache: one launch).
 * Each pass has exactly csa_cache_append's arguments, meaning and requirements
 * and leaves its cache exactly as csa_cache_append leaves it; the passes must
 * update different caches (no buffer written by one pass is read or written
 * by another).  Passes of one token per sequence (n = 1) share launches, up to
 * four caches per launch; others run as csa_cache_append runs them.  Every
 * pass is checked before anything is enqueued.  n_passes <= 16.
 */
typedef struct {
    const void *x, *gate;
    const float *slot_bias;
    void *ring_x, *ring_g, *pool, *win;
    const int32_t *count;
    int32_t B, n, D, m, overlap, T_cap, W, rope_dim;
    const float *cs;
    int32_t n_pos;
} csa_cache_pass_t;

csa_status_t csa_cache_append_many(const csa_cache_pass_t *passes, int32_t n_passes,
                                   int32_t dtype, void *stream);

/*
 * csa_index_scores -- Lightning-Indexer index scores.  Page "DeepSeek-V4",
 * "Hybrid attention" (indexer scoring queries against the pool, eqs. 13-17)
 * and DeepseekV4Config (index_n_heads = n_h^I of eq. 14, index_head_dim);
 * page "DeepSeek-V3.2", "DeepSeek Sparse Attention" (a low-head-count score
 * between each query and earlier keys, a dot product against one shared key
 * head, per-head weights).
 *   q_idx   [B][S][n_heads][head_dim] dtype  indexer queries
 *   w_idx   [B][S][n_heads] fp32             per-head weights
 *   k_pool  [B][T][head_dim] dtype           compressed indexer keys
 *   scores  [B][S][T] fp32, out: for w < R(t),
 *             scores = sum_j w_idx[j] * max(0, <q_idx[j], k_pool[w]>)
 *           with -0 written as +0; entries w >= R(t) are left untouched.
 *   m: compression rate behind the readiness rule (m = 1 for DSA tokens).
 *   Products are formed in fp32 (bf16 inputs go through bf16 matrix cores
 *   with fp32 accumulation).
 */
csa_status_t csa_index_scores(const void *q_idx, const float *w_idx, const void *k_pool,
                              float *scores, const int32_t *q_pos, int32_t B, int32_t S,
                              int32_t T, int32_t n_heads, int32_t head_dim, int32_t m,
                              int32_t dtype, void *stream);

/*
 * csa_topk -- per-query top-k over the ready entries.  Page "DeepSeek-V4",
 * DeepseekV4Config (index_topk, eq. 17) and "Attention mask layout" (the -1
 * sentinel fills slots that cannot be filled yet).
 *   scores  [B][S][T] fp32 (only w < R(t) is read)
 *   idx     [B][S][k] int32, out: the min(k, R(t)) ready entries with the
 *           largest scores (equal scores: the lower index wins; -0 equals +0),
 *           written in ascending index order, then -1 in the remaining slots.
 *   The result is unique and deterministic.  Scores must not be NaN.
 */
csa_status_t csa_topk(const float *scores, int32_t *idx, const int32_t *q_pos, int32_t B,
                      int32_t S, int32_t T, int32_t k, int32_t m, void *stream);

/*
 * csa_index_topk -- csa_index_scores followed by csa_topk as one call, the
 * scores kept on chip.  Page "DeepSeek-V3.2", "DeepSeek Sparse Attention"
 * (the indexer scores each query against the earlier keys and only the top-k
 * tokens go on to attention; the indexer is cheap next to the attention) and
 * page "DeepSeek-V4", "Hybrid attention" (the Lightning Indexer picks the
 * index_topk compressed entries per query).
 *   Arguments as csa_index_scores and csa_topk; idx [B][S][k] int32, out,
 *   exactly as csa_topk(csa_index_scores(...)) writes it (the same scores, so
 *   the same selection); no scores are written.
 *   bf16 with 64 x 128 indexer heads, S >= 16, T <= 2048 and m >= 2 (CSA
 *   prefill) runs one kernel: each workgroup scores 4 query rows into LDS and selects
 *   from there (workspace unused).  Every other shape computes the scores into
 *   the caller's workspace (csa_index_topk_workspace_size bytes) and selects
 *   from it; a missing or small workspace is CSA_ERR_INVALID.
 */
csa_status_t csa_index_topk(const void *q_idx, const float *w_idx, const void *k_pool,
                            int32_t *idx, const int32_t *q_pos, int32_t B, int32_t S, int32_t T,
                            int32_t n_heads, int32_t head_dim, int32_t k, int32_t m,
                            void *workspace, size_t ws_bytes, int32_t dtype, void *stream);

/* Bytes of workspace csa_index_topk needs for this shape (0: fused on chip). */
size_t csa_index_topk_workspace_size(int32_t B, int32_t S, int32_t T, int32_t n_heads,
                                     int32_t head_dim, int32_t k, int32_t m, int32_t dtype);

/*
 * csa_sparse_attn -- core attention of a CSA (or DSA) layer.  Page
 * "DeepSeek-V4", "Hybrid attention": multi-query attention with one shared
 * K=V head, partial RoPE on q, the output's rope slice rotated at position
 * -t (eq. 26), a learnable per-head sink (eq. 27), and the sliding-window K=V
 * branch concatenated with the selected compressed entries; "Attention mask
 * layout" (the query's k indexer slots, -1 = empty).  Page "DeepSeek-V3.2",
 * "DeepSeek Sparse Attention": attention over the selected tokens only.
 *   q        [B][S][H][D] dtype   queries, NOT yet rotated
 *   kv_win   [B][L_win][D] dtype  sliding-window K=V rows, already rotated;
 *            row r of sequence b is position win_pos0[b] + r; NULL iff
 *            window == 0 or L_win == 0
 *   win_pos0 [B] int32
 *   pool     [B][T][D] dtype      compressed K=V entries, already rotated
 *   idx      [B][S][k] int32      selected entries, -1 = empty slot
 *   sink     [H] fp32             sink logits z_h, or NULL for no sink
 *   out      [B][S][H][dv] dtype  out
 *   For each (row, head): keys = window rows at positions (t-window, t] plus
 *   pool rows idx[..] != -1; q~ = q rotated at +t; l_j = scale * <q~, key_j>;
 *   p_j = exp(l_j) / (exp(z_h) + sum exp(l)); o = sum_j p_j key_j[:dv]; when
 *   dv == D the trailing rope_dim channels of o are rotated at -t.  dv may be
 *   D or D - rope_dim (DSA: the latent part is the value).  A row with no
 *   visible key and no sink is written as zeros.
 *   cs, n_pos: the RoPE table (t must be < n_pos; unused when rope_dim == 0).
 *   workspace/ws_bytes: optional scratch (see csa_sparse_attn_workspace_size);
 *   with less than that size the call still runs, without splitting a row's
 *   keys over several workgroups.
 */
csa_status_t csa_sparse_attn(const void *q, const void *kv_win, const int32_t *win_pos0,
                             int32_t L_win, const void *pool, int32_t T, const int32_t *idx,
                             int32_t k, const float *sink, void *out, const int32_t *q_pos,
                             int32_t B, int32_t S, int32_t H, int32_t D, int32_t dv,
                             int32_t rope_dim, const float *cs, int32_t n_pos,
                             int32_t window, float scale, void *workspace, size_t ws_bytes,
                             int32_t dtype, void *stream);

/*
 * csa_sparse_attn_noalloc -- csa_sparse_attn without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * result and kernels as csa_sparse_attn given a workspace of
 * csa_sparse_attn_workspace_size bytes; the split partials go to a 24 MiB
 * device array of the library instead (one per GPU, held until the process
 * ends; its address is looked up on the first call on each device).  The call
 * allocates nothing.  A shape whose split needs more than 24 MiB returns
 * CSA_ERR_UNSUPPORTED.  Every call on one GPU shares that array: calls that
 * overlap in time on one GPU (other streams, other host threads) race and
 * must be serialized by the caller.  The array needs no clearing (every
 * partial a call reads was written earlier in the same call).
 */
csa_status_t csa_sparse_attn_noalloc(const void *q, const void *kv_win,
                                     const int32_t *win_pos0, int32_t L_win, const void *pool,
                                     int32_t T, const int32_t *idx, int32_t k,
                                     const float *sink, void *out, const int32_t *q_pos,
                                     int32_t B, int32_t S, int32_t H, int32_t D, int32_t dv,
                                     int32_t rope_dim, const float *cs, int32_t n_pos,
                                     int32_t window, float scale, int32_t dtype, void *stream);

/* Bytes of workspace csa_sparse_attn uses for this shape on the current
 * device (0 = it never splits this shape). */
size_t csa_sparse_attn_workspace_size(int32_t B, int32_t S, int32_t H, int32_t D,
                                      int32_t dv, int32_t rope_dim, int32_t k,
                                      int32_t window, int32_t dtype);

/*
 * hca_attn -- core attention of an HCA layer.  Page "DeepSeek-V4", "Hybrid
 * attention" (heavily compressed pool at rate m', no indexer: every entry
 * contributes) and "Attention mask layout" (entry w visible once
 * w < (t+1)//m').  Same as csa_sparse_attn with the pool rows fixed to all
 * ready entries w < R(t) = min(T, floor((t+1)/m)) instead of an index list.
 * With T = 0 (or pool = NULL) it is plain sliding-window attention.
 */
csa_status_t hca_attn(const void *q, const void *kv_win, const int32_t *win_pos0,
                      int32_t L_win, const void *pool, int32_t T, int32_t m,
                      const float *sink, void *out, const int32_t *q_pos, int32_t B,
                      int32_t S, int32_t H, int32_t D, int32_t dv, int32_t rope_dim,
                      const float *cs, int32_t n_pos, int32_t window, float scale,
                      void *workspace, size_t ws_bytes, int32_t dtype, void *stream);

/* Bytes of workspace hca_attn uses for this shape on the current device. */
size_t hca_attn_workspace_size(int32_t B, int32_t S, int32_t H, int32_t D, int32_t dv,
                               int32_t rope_dim, int32_t T, int32_t window, int32_t dtype);

/*
 * csa_grouped_out_proj -- grouped low-rank output projection of the attention
 * output.  Page "DeepSeek-V4", "Hybrid attention (§2.3)" (the heads are split
 * into o_groups groups; each group goes through its own projection to
 * o_lora_rank values (o_a_proj), the concatenated groups through one more
 * linear map to hidden_size (o_b_proj)) and DeepseekV4Config (o_groups = 8,
 * o_lora_rank = 1024, hidden_size = 4096, attention_bias = False).
 *   o     [M][groups * group_in] dtype   attention output rows (the [S][H][dv]
 *                                        output of csa_sparse_attn / hca_attn
 *                                        with group_in = H dv / groups: group g
 *                                        holds heads g H/groups .. (g+1) H/groups - 1)
 *   w_a   [groups][rank][group_in] dtype  per-group projection (rows = outputs)
 *   w_b   [hidden][groups * rank] dtype   the second projection
 *   mid   [M][groups * rank] dtype, out:  mid[m][g rank + j] =
 *             sum_c o[m][g group_in + c] * w_a[g][j][c]   (stored in dtype)
 *   out   [M][hidden] dtype, out:         out[m][n] = sum_i mid[m][i] * w_b[n][i]
 *   Products accumulate in fp32; bf16 results are rounded to nearest even.
 *   The stored mid (bf16 for bf16) is what the second product reads.
 *   group_in, rank, hidden must be multiples of 8; tensors 16-byte aligned.
 *   Two kernels in stream order.
 */
csa_status_t csa_grouped_out_proj(const void *o, const void *w_a, const void *w_b, void *mid,
                                  void *out, int32_t M, int32_t groups, int32_t group_in,
                                  int32_t rank, int32_t hidden, int32_t dtype, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H */
