/*
 * hsa.h - C ABI of libhsa: one global iteration of Heterogeneous Step
 * Allocation (HSA) for flow-matching DiT video sampling, on AMD Instinct
 * MI355X (gfx950).
 *
 * Source of the method: "Not All Tokens Need 40 Steps: Heterogeneous Step
 * Allocation in Diffusion Transformers for Efficient Video Generation"
 * (gist.science technical summary of arXiv 2605.06892).  Section numbers in
 * the comments below refer to that summary.
 *
 * Conventions shared by every call:
 *  - Pointers are DEVICE pointers unless marked (host).  The caller owns every
 *    buffer; the library allocates nothing and keeps no global state, except
 *    for the fixed device array of hsa_attn_active_noalloc (at the end).
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).  Calls
 *    enqueue work on it and return before the work completes.
 *  - Arguments are validated on the host before anything is enqueued.  An
 *    invalid call enqueues nothing and returns a negative hsa_status.  A HIP
 *    launch error is returned as HSA_ERR_HIP; faults inside kernels surface at
 *    the caller's next synchronisation.
 *  - Device pointers must be 16-byte aligned.  Matrices are row-major and
 *    dense.  Activations are token-major: row r of an [rows][D] matrix is one
 *    token.  Linear weights are out-major, W[out][in], so y = a W^T.
 *  - HSA_BF16 tensors hold bfloat16; HSA_F32 tensors hold float32.  Latents,
 *    velocities, scores and the residual stream are always float32.
 *    Accumulation is float32 in both modes.
 */
#ifndef HSA_H_
#define HSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSA_MAX_GROUPS 8

typedef enum {
  HSA_OK = 0,
  HSA_ERR_ARG = -1,       /* null pointer, negative size, bad flag          */
  HSA_ERR_SHAPE = -2,     /* sizes inconsistent or outside supported range  */
  HSA_ERR_DTYPE = -3,     /* unsupported dtype for this call                */
  HSA_ERR_ALIGN = -4,     /* a device pointer is not 16-byte aligned        */
  HSA_ERR_WORKSPACE = -5, /* workspace missing or smaller than required     */
  HSA_ERR_HIP = -6,       /* a HIP runtime call failed                      */
  HSA_ERR_SCHEDULE = -7,  /* budgets do not divide T, counts do not sum to N */
  HSA_ERR_TOO_LARGE = -8  /* needs more than HSA_NOALLOC_SCRATCH_BYTES       */
} hsa_status;

/* HSA_DTYPE_MAX_ENUM only widens the type: a caller may pass any int32 value
 * and an unsupported one returns HSA_ERR_DTYPE (it is never a valid dtype). */
typedef enum { HSA_F32 = 0, HSA_BF16 = 1, HSA_DTYPE_MAX_ENUM = 0x7fffffff } hsa_dtype;

/* Optional block features, OR-ed into hsa_dims.features (0: none, the plain
 * block below).  The pages run HSA on Wan-family DiTs (section 4) but define
 * none of their layers; each feature follows the published general
 * definition it is named after:
 *  HSA_FEAT_QK_NORM  q and k rows, after the projection, are divided by
 *                    sqrt(mean(x^2) + 1e-6) over the whole width D and
 *                    multiplied by the block's q_gain / k_gain [D].
 *  HSA_FEAT_ROPE3D   rotary position embedding of q and k (after the
 *                    RMSNorm), per head: coordinate pair (2j, 2j+1) turns by
 *                    pos * 10000^(-j'/p).  A head's P = Dh/2 pairs form a
 *                    frame section of P - 2*floor(P/3) pairs, then a row and
 *                    a column section of floor(P/3) pairs each; p is the
 *                    section's pair count, j' the pair's index in it, pos
 *                    token n's frame, row or column in the latent grid, n =
 *                    (f * grid_h + y) * grid_w + x.  The K cache holds
 *                    rotated keys.
 *  HSA_FEAT_ADALN    timestep modulation.  t = 1000 * sigma_i; sinusoid
 *                    s = [cos(t w_k), sin(t w_k)], w_k = 10000^(-k/128),
 *                    k < 128; e = t_w2 silu(t_w1 s + t_b1) + t_b2 [D];
 *                    e0 = t_w3 silu(e) + t_b3 [6][D].  Block l uses
 *                    mod_l + e0 = (shift, scale, gate) of the attention
 *                    branch, then of the MLP branch: the branch reads
 *                    LN(h) (1 + scale) + shift and its output is multiplied
 *                    by gate before the residual add.  Cross-attention is
 *                    neither modulated nor gated.  The final LayerNorm uses
 *                    (shift, scale) = head_mod + e.
 *  HSA_FEAT_CFG      classifier-free guidance with batch 2 (needs
 *                    n_text > 0): the model runs on the active rows once
 *                    with (k_text, v_text, k_cache, v_cache) and once with
 *                    the unconditional set (k_text_u, v_text_u, k_cache_u,
 *                    v_cache_u); the velocity is v_u + cfg_scale (v_c - v_u). */
#define HSA_FEAT_QK_NORM 1
#define HSA_FEAT_ROPE3D 2
#define HSA_FEAT_ADALN 4
#define HSA_FEAT_CFG 8

/* Model shape.  N tokens, C latent channels, width D = H * Dh, MLP width F,
 * L blocks, n_text text tokens for cross-attention (0: no cross-attention),
 * `features` a subset of HSA_FEAT_*, (grid_f, grid_h, grid_w) the latent
 * token grid with grid_f * grid_h * grid_w == N (read with HSA_FEAT_ROPE3D
 * only).  bf16 operands are streamed through 32-bit buffer descriptors:
 * every bf16 matrix a kernel reads whole (N x D, N x F, weights) must stay
 * below 4 GiB, i.e. N * max(D, F) * 2 < 2^32; larger shapes return
 * HSA_ERR_SHAPE. */
typedef struct {
  int32_t N, C, D, H, Dh, F, L, n_text;
  hsa_dtype dtype;
  int32_t features;
  int32_t grid_f, grid_h, grid_w;
} hsa_dims;

/* Step schedule (section 2.1).  K groups; budget[k] = s_k steps out of T,
 * budget[0] == T (the baseline group G_1), T % budget[k] == 0; count[k] =
 * |G_k|, sum == N.  m = phase window (section 2.4): iterations i < m and
 * i >= T - m run every token. */
typedef struct {
  int32_t T, K, m;
  int32_t budget[HSA_MAX_GROUPS];
  int32_t count[HSA_MAX_GROUPS];
} hsa_schedule;

/* One transformer block (dtype of hsa_dims):
 *   w_qkv [3D][D]  rows 0..D-1 -> q, D..2D-1 -> k, 2D..3D-1 -> v
 *   w_o [D][D], w_1 [F][D], w_2 [D][F]
 *   k_cache, v_cache [N][D]: the per-layer K/V cache of section 2.2, row n =
 *     token n, head h in columns h*Dh .. h*Dh+Dh-1.
 *   Cross-attention (n_text > 0): w_qx, w_ox [D][D]; k_text, v_text
 *     [n_text][D] (projected once per run by the caller).  NULL otherwise.
 *   Feature parameters, float32, NULL when their feature is off:
 *     q_gain, k_gain [D] (HSA_FEAT_QK_NORM); mod [6][D] (HSA_FEAT_ADALN);
 *     k_text_u, v_text_u [n_text][D] and k_cache_u, v_cache_u [N][D] of the
 *     unconditional branch (HSA_FEAT_CFG, dtype of hsa_dims). */
typedef struct {
  const void *w_qkv, *w_o, *w_1, *w_2;
  const void *w_qx, *w_ox;
  void *k_cache, *v_cache;
  const void *k_text, *v_text;
  const float *q_gain, *k_gain, *mod;
  const void *k_text_u, *v_text_u;
  void *k_cache_u, *v_cache_u;
} hsa_block;

/* Model: embed w_in [D][C] (latent -> width), unembed w_out [C][D]; blocks
 * is a HOST array of L hsa_block.  HSA_FEAT_ADALN: timestep MLP t_w1
 * [D][256], t_b1 [D], t_w2 [D][D], t_b2 [D], t_w3 [6D][D], t_b3 [6D] and
 * head_mod [2][D], all float32 (NULL otherwise).  HSA_FEAT_CFG: cfg_scale
 * is the guidance scale. */
typedef struct {
  hsa_dims dims;
  const void *w_in, *w_out;
  const hsa_block *blocks;
  const float *t_w1, *t_b1, *t_w2, *t_b2, *t_w3, *t_b3, *head_mod;
  float cfg_scale;
} hsa_model;

/* Sampler state, all float32 except group/active_idx/pos:
 *   x [N][C] latents, v_hat [N][C] cached velocity (section 2.3), score [N]
 *   L1 relative change (section 2.1), group [N] (0 = G_1), active_idx [N]
 *   (first |A_i| entries valid, ascending), pos [N] (j if active_idx[j] == n,
 *   else -1), workspace of at least hsa_workspace_size() bytes. */
typedef struct {
  float *x, *v_hat, *score;
  uint8_t *group;
  int32_t *active_idx, *pos;
  void *workspace;
  size_t workspace_bytes;
} hsa_state;

/* Status code as text (static string, never NULL). */
const char *hsa_status_str(int32_t status);

/* Library ABI version (increments when a signature or struct changes); a
 * library built from this header returns HSA_ABI_VERSION. */
#define HSA_ABI_VERSION 4
int32_t hsa_abi_version(void);

/* Workspace needed by hsa_step / hsa_block_forward for these dims (host out). */
hsa_status hsa_workspace_size(const hsa_dims *dims, size_t *bytes);

/* Workspace needed by hsa_attn_active for n_active queries (host out). */
hsa_status hsa_attn_workspace_size(int32_t n_active, int32_t n_kv, int32_t H, int32_t Dh,
                                   size_t *bytes);

/* Workspace needed by hsa_select (host out). */
hsa_status hsa_select_workspace_size(int32_t N, int32_t K, size_t *bytes);

/* |A_i| in closed form (host): sum_k count[k] [iter mod (T/budget[k]) == 0],
 * or N inside the phase window.  Section 2.1 (activity rule), 2.4. */
hsa_status hsa_n_active(const hsa_schedule *sched, int32_t iter, int32_t *n_active);

/* Active set A_i (section 2.1 activity rule, section 2.2 item 1): writes the
 * ascending indices of tokens n with iter mod (T/budget[group[n]]) == 0 (or
 * all tokens inside the phase window) into active_idx[0..|A_i|), pos[N] as
 * the inverse map (-1 for skipped tokens) and |A_i| into *n_active_dev
 * (device int32).  Bit-exact; group values must be < sched->K, and group k
 * must hold exactly sched->count[k] tokens (select's output always does).
 * Otherwise *n_active_dev differs from hsa_n_active(): active_idx is still
 * written up to hsa_n_active() entries (padded with token 0) and tokens past
 * them are marked skipped, so every later access stays in bounds, but the
 * iteration's results are meaningless. */
hsa_status hsa_active_set(const uint8_t *group, int32_t N, const hsa_schedule *sched,
                          int32_t iter, int32_t *active_idx, int32_t *pos,
                          int32_t *n_active_dev, void *stream);

/* Dynamic token selection (section 2.1): ranks tokens by (score descending,
 * index ascending; NaN as +inf, -0 as +0) and writes group_out[n] = k for
 * ranks in [count[0]+..+count[k-1], count[0]+..+count[k]).  count is a HOST
 * array of K entries summing to N.  Bit-exact given identical scores. */
hsa_status hsa_select(const float *score, int32_t N, const int32_t *count, int32_t K,
                      uint8_t *group_out, void *ws, size_t ws_bytes, void *stream);

/* The same selection for a batch of B independent score vectors (one per
 * video), each ranked and split by the same count[] (host, K entries summing
 * to N): score [B][N] float32 -> group_out [B][N], row b of the output from
 * row b of the input only.  Bit-exact per row, as hsa_select.  B, N > 0 and
 * B * N <= 2^38 (HSA_ERR_SHAPE otherwise); HSA_ERR_SCHEDULE when the counts
 * are negative or do not sum to N. */
hsa_status hsa_select_batch(const float *score, int32_t B, int32_t N, const int32_t *count,
                            int32_t K, uint8_t *group_out, void *stream);

/* Cached Euler update (section 2.3) with the L1 score (section 2.1): for
 * each token n with pos[n] >= 0, if update_score: score[n] =
 * sum_c|v_new[pos[n]] - v_hat[n]| / (sum_c|v_hat[n]| + eps); then v_hat[n] =
 * v_new[pos[n]].  Then for every n: x[n] += dsigma * v_hat[n].
 * x, v_hat [N][C]; v_new [|A|][C]; pos [N]; score [N].  In place. */
hsa_status hsa_euler(float *x, float *v_hat, float *score, const float *v_new,
                     const int32_t *pos, int32_t N, int32_t C, float dsigma, float eps,
                     int32_t update_score, void *stream);

/* Active-query attention (section 2.2 items 3-4): for each of n_active query
 * rows and each head h, o = softmax(q_h K_h^T * scale) V_h over all n_kv rows
 * of k and v, no mask.  q, o [n_active][H*Dh]; k, v [n_kv][H*Dh].  Dh is 64
 * or 128; bf16 needs n_kv * H * Dh * 2 < 2^32 (HSA_ERR_SHAPE otherwise).
 * ws: at least hsa_attn_workspace_size() bytes (may be NULL when that size
 * is 0). */
hsa_status hsa_attn_active(const void *q, const void *k, const void *v, void *o,
                           int32_t n_active, int32_t n_kv, int32_t H, int32_t Dh, float scale,
                           hsa_dtype dtype, void *ws, size_t ws_bytes, void *stream);

/* Row LayerNorm (no affine, eps 1e-6): out[r] = (h[r]-mean)/sqrt(var+eps),
 * h [rows][D] float32 -> out [rows][D] in dtype.  With shift and scale
 * ([D] float32, both or neither; the HSA_FEAT_ADALN modulation) out[r] =
 * LN(h[r]) * (1 + scale) + shift. */
hsa_status hsa_layernorm(const float *h, void *out, int32_t rows, int32_t D, const float *shift,
                         const float *scale, hsa_dtype dtype, void *stream);

/* Gather + embed (section 2.2 item 1, the active rows enter the model):
 * h[j] = x[active_idx[j]] w_in^T, x [N][C] float32, w_in [D][C] dtype,
 * h [n_active][D] float32. */
hsa_status hsa_embed(const float *x, const int32_t *active_idx, const void *w_in, float *h,
                     int32_t n_active, int32_t C, int32_t D, hsa_dtype dtype, void *stream);

/* Final LayerNorm + unembed: v_new[j] = LN(h[j]) w_out^T, h [n_active][D]
 * float32, w_out [C][D] dtype, v_new [n_active][C] float32.  shift, scale
 * as for hsa_layernorm (NULL: unmodulated). */
hsa_status hsa_unembed(const float *h, const void *w_out, float *v_new, int32_t n_active,
                       int32_t D, int32_t C, const float *shift, const float *scale,
                       hsa_dtype dtype, void *stream);

/* Linear map on rows: out = act(a w^T), a [M][K], w [Nout][K], out [M][Nout],
 * all in dtype; act 0 = identity, 1 = GELU (tanh form).  bf16: K % 64 == 0,
 * Nout % 4 == 0, M * K * 2 and Nout * K * 2 below 2^32 (HSA_ERR_SHAPE
 * otherwise; the same holds for hsa_linear_residual and hsa_qkv_scatter). */
hsa_status hsa_linear(const void *a, const void *w, void *out, int32_t M, int32_t Nout,
                      int32_t K, int32_t act, hsa_dtype dtype, void *stream);

/* Linear map added to the float32 residual stream: h += a w^T, a [M][K]
 * dtype, w [Nout][K] dtype, h [M][Nout] float32.  With gate ([Nout]
 * float32, the HSA_FEAT_ADALN gate; NULL: none) h[m][n] += gate[n] (a w^T)[m][n]. */
hsa_status hsa_linear_residual(const void *a, const void *w, float *h, int32_t M, int32_t Nout,
                               int32_t K, const float *gate, hsa_dtype dtype, void *stream);

/* KV-cache synchronisation steps 1-2 (section 2.2): [q | k | v] = a_j w_qkv^T
 * for the n_active active rows; q goes to q_out [n_active][D]; k and v rows
 * overwrite k_cache[active_idx[j]] and v_cache[active_idx[j]] ([N][D]).
 * Rows of the cache not in active_idx are not touched.  gather 0: a_j is row
 * j of a [n_active][D]; gather 1: a_j = a[active_idx[j]] of a [N][D] (the
 * active rows read straight from a per-token hidden state; bf16 needs
 * N * D * 2 < 2^32). */
hsa_status hsa_qkv_scatter(const void *a, const int32_t *active_idx, int32_t gather,
                           const void *w_qkv, void *q_out, void *k_cache, void *v_cache,
                           int32_t n_active, int32_t N, int32_t D, hsa_dtype dtype, void *stream);

/* qk-RMSNorm and 3D rotary embedding (HSA_FEAT_QK_NORM / HSA_FEAT_ROPE3D,
 * whichever dims->features holds; neither: nothing to do) in place on q
 * [n_active][D] (row j is token active_idx[j]) and on rows active_idx[j] of
 * k_cache [N][D], dtype of dims.  q_gain, k_gain [D] float32, needed with
 * HSA_FEAT_QK_NORM. */
hsa_status hsa_qk_norm_rope(void *q, void *k_cache, const int32_t *active_idx, int32_t n_active,
                            const hsa_dims *dims, const float *q_gain, const float *k_gain,
                            void *stream);

/* Timestep embedding of HSA_FEAT_ADALN for sigma (float32, t = 1000 sigma):
 * e [D] and e0 [6][D], float32 device outputs (e0 also serves as scratch
 * during the call).  Model weights as in hsa_model. */
hsa_status hsa_time_embed(const hsa_model *model, float sigma, float *e, float *e0, void *stream);

/* Classifier-free guidance combine (HSA_FEAT_CFG): v = v + g (v_cond - v)
 * elementwise over rows x C float32 values, v holding the unconditional
 * velocity on entry. */
hsa_status hsa_guidance(const float *v_cond, float *v, int32_t rows, int32_t C, float g,
                        void *stream);

/* One transformer block on the active rows (section 2.2): LN, QKV with cache
 * scatter, active-query attention over all N cached rows, out-projection,
 * optional cross-attention, GELU MLP, residual adds, with the features of
 * model->dims.  h [n_active][D] float32 in place; caches of block `layer`
 * updated.  e0 [6][D]: the timestep projection from hsa_time_embed (needed
 * with HSA_FEAT_ADALN, else ignored).  branch 0 uses the conditional text
 * set and caches, 1 the unconditional ones (HSA_FEAT_CFG only).  ws as for
 * hsa_step. */
hsa_status hsa_block_forward(const hsa_model *model, int32_t layer, float *h,
                             const int32_t *active_idx, int32_t n_active, const float *e0,
                             int32_t branch, void *ws, size_t ws_bytes, void *stream);

/* One global HSA iteration `iter` (0-based) from sigma_i to sigma_next:
 *  1. if regroup: group = hsa_select(score, count)   (section 2.1)
 *  2. A_i = hsa_active_set(group, iter)               (sections 2.1, 2.4)
 *  3. h = embed(x[A_i]); L blocks (section 2.2); v_new = unembed(h); with
 *     HSA_FEAT_ADALN the timestep embedding of sigma_i first; with
 *     HSA_FEAT_CFG once per branch, then combined by hsa_guidance
 *  4. if v_field != NULL: v_new[j] = v_field[A_i[j]]  ([N][C] float32; a
 *     synthetic velocity replaces the model's in the Euler/score path)
 *  5. hsa_euler with dsigma = sigma_next - sigma_i, eps = 1e-6, score
 *     updated when iter >= 1                         (section 2.3)
 * |A_i| comes from the closed form on the host: no device synchronisation. */
hsa_status hsa_step(const hsa_model *model, const hsa_schedule *sched, hsa_state *state,
                    int32_t iter, float sigma_i, float sigma_next, int32_t regroup,
                    const float *v_field, void *stream);

/* Allocation-free active-query attention, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Computes exactly what hsa_attn_active
 * computes, with the same kernels, arguments and results, but takes no
 * workspace: the KV-split partials (hsa_attn_workspace_size() bytes) live in
 * a fixed device array of HSA_NOALLOC_SCRATCH_BYTES that each GPU holds from
 * the library's load until the process ends.  A call that would need more
 * returns HSA_ERR_TOO_LARGE and enqueues nothing (use hsa_attn_active with a
 * workspace then).  The call never allocates or frees memory; its first call
 * on a device looks up that device's array address (the stream's device
 * must be current).  All calls on one GPU share its array: calls that
 * overlap on one GPU (other streams, other threads) race, so serialise
 * them. */
#define HSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
hsa_status hsa_attn_active_noalloc(const void *q, const void *k, const void *v, void *o,
                                   int32_t n_active, int32_t n_kv, int32_t H, int32_t Dh,
                                   float scale, hsa_dtype dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* HSA_H_ */
