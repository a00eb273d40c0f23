/*
 * eagle.h -- C-ABI of the MI355X (gfx950) EAGLE draft-and-verify library.
 *
 * One draft-and-verify round of EAGLE speculative decoding:
 *
 *   eagle_tree_init           root of every request's draft tree
 *   eagle_draft_step  x gamma one pass of the draft head over the rows of a step
 *   eagle_tree_expand_rerank  x gamma grow the tree from that step's top-k; the
 *                             last call also reranks and builds the verify tree
 *   eagle_tree_attend         (optional) tree-masked attention over the verify tree
 *   eagle_tree_verify         accept the longest root path matching the target
 *   (or eagle_tree_verify_sample: lossless multi-round speculative sampling)
 *   eagle_target_verify_logits (optional) the target's own pass over the tree
 *                             (its logits feed the verify calls)
 *   eagle_kv_commit           (optional) append the accepted path's K/V to a cache
 *
 * The method is the one described on the pages
 *   "transformer_math / tm_eagle_deep" (aicassindra.com), sections "The
 *     recurrence, written out", "What is actually in the head", "EAGLE-2: expand
 *     and rerank" and "Tree attention in one verification pass";
 *   "Speculative Decoding Deep Dive III: EAGLE, DFlash" (zackli.ai), sections
 *     "EAGLE-1", "EAGLE-2" and "EAGLE-3";
 *   "EAGLE / DFlash / DSpark" explainer (kaushalya.io), "How speculative
 *     decoding works" steps 3-4;
 *   "EAGLE: Drafting in Feature Space" (stable-lab.github.io), sections "The
 *     Mechanism" and "Drafting a Tree, Not a Chain".
 *
 * Conventions (all entry points):
 *   - Every pointer named "device" is a device (HBM) address owned by the
 *     caller.  The library never allocates or frees device memory and keeps no
 *     pointer after a call returns.  Scratch space comes from the caller's
 *     workspace (eagle_workspace_bytes) and tree state (eagle_tree_state_bytes).
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls only
 *     enqueue work on it and return; nothing synchronises inside the library.
 *   - Matrices are row-major [out][in] (the input dimension contiguous), in the
 *     head's dtype (bf16 or fp32).  Activations between kernels are stored in
 *     that dtype; accumulation, softmax and confidences are fp32.
 *   - Every argument is validated on the host before anything is launched; on
 *     any error nothing is enqueued.  A failed launch returns EAGLE_EHIP.
 *   - Calls that share a workspace or tree state must be ordered on one stream.
 */
#ifndef EAGLE_H
#define EAGLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  EAGLE_OK = 0,
  EAGLE_EINVAL = -1,       /* null pointer, bad size or step out of range   */
  EAGLE_EUNSUPPORTED = -2, /* shape outside what the kernels implement      */
  EAGLE_ECAPACITY = -3,    /* workspace / state / tree larger than allowed  */
  EAGLE_EHIP = -4          /* a HIP launch or runtime call failed           */
} eagle_status;

enum { EAGLE_BF16 = 0, EAGLE_F32 = 1 };
enum { EAGLE_ACT_SWIGLU = 0, EAGLE_ACT_GELU = 1 };
enum { EAGLE_NORM_RMS = 0, EAGLE_NORM_LAYER = 1 };
enum { EAGLE_MODE_1 = 1, EAGLE_MODE_3 = 3 };
enum { EAGLE_TREE_CHAIN = 0, EAGLE_TREE_STATIC = 1, EAGLE_TREE_DYNAMIC = 2 };

#define EAGLE_MAX_SLOTS 64      /* expanded nodes per request (64-bit masks)   */
#define EAGLE_MAX_POSITIONS 64  /* verify-tree positions per request (root+m)  */
#define EAGLE_MAX_TOPK 16
#define EAGLE_MAX_INV_TEMP 65536.0f  /* largest inverse temperature s of the draft */
#define EAGLE_VERIFY_DRAWS 17   /* uniforms per verify position: 16 child tests + 1 residual draw */

/*
 * The draft head ("What is actually in the head": an fc of shape [2d, d], one
 * decoder layer of width d, and the target's shared embedding and LM head).
 *
 *   EAGLE-1 (mode 1):  h = x W_fc^T with x = [f ; emb(t)]           w_fc [d][2d]
 *   EAGLE-3 (mode 3):  g = [l ; m ; h] W_fuse^T, x = g + emb(t)     w_fuse [d][3d]
 *                      at verified positions; a + emb(t) afterwards (no fc)
 *   layer (pre-norm):  h1 = h + Attn(N1(h)) W_o^T,  out = h1 + MLP(N2(h1))
 *                      w_q [Hq*hd][d], w_k, w_v [Hkv*hd][d], w_o [d][Hq*hd]
 *                      SwiGLU: w_gate, w_up [ffn][d], w_down [d][ffn]
 *                      GELU:   w_up [ffn][d], w_down [d][ffn] (w_gate unused)
 *                      N1, N2: RMSNorm (gain) or LayerNorm (gain, bias), eps
 *                      RoPE rotate-half, inv_freq = theta^(-2i/hd); theta 0 = off
 *   LM head:           logits = W_LM out, lm_head [V][d]; emb [V][d]
 * Constraints: d % 64 == 0, ffn % 32 == 0, head_dim in {64, 128},
 * n_q_heads % n_kv_heads == 0, V >= 16.
 */
typedef struct eagle_head {
  int32_t d, vocab, n_q_heads, n_kv_heads, head_dim, ffn;
  int32_t act;    /* EAGLE_ACT_*  */
  int32_t norm;   /* EAGLE_NORM_* */
  int32_t dtype;  /* EAGLE_BF16 or EAGLE_F32: weights, caches, activations */
  int32_t mode;   /* EAGLE_MODE_1 or EAGLE_MODE_3 */
  float eps, rope_theta;
  const void *w_fc, *w_fuse;                 /* device; the one of the mode  */
  const void *w_q, *w_k, *w_v, *w_o;         /* device */
  const void *w_gate, *w_up, *w_down;        /* device */
  const void *norm1_g, *norm1_b, *norm2_g, *norm2_b;  /* device [d]; b: LN only */
  const void *emb, *lm_head;                 /* device [V][d] */
} eagle_head;

/*
 * Key/value caches of the draft layer ("The recurrence, written out": the
 * layer runs over a cache).  Requests are packed without padding (explainer,
 * "Serving batch": variable-length blocks may be packed).
 *   k_ctx, v_ctx  [total_n][Hkv][hd]  context K/V (rotated); read by the
 *                                     attention, written by the ingest
 *   k_slot,v_slot [B][64][Hkv][hd]    K/V of every expanded tree node (slot)
 *   feat_slot     [B][64][d]          layer output of every expanded node
 * Steady state ("Speculative Decoding Deep Dive III", EAGLE-3 example: each
 * round feeds the fused features of the tokens the target has just verified;
 * EAGLE-1 "Inference": the drafter reads the target's features of the
 * verified prefix; the draft cache of older positions is kept).  With n_new
 * set, request b already holds the K/V of its first n[b] - n_new[b]
 * positions in k_ctx/v_ctx, and step 0 ingests only its last n_new[b] >= 1
 * positions (EAGLE-3: the accepted path and the target's token; EAGLE-1: the
 * positions verified since the last round, whose rows are
 * fc([f_{j-1} ; emb(t_j)]) from the target's features; the EAGLE-1 root row
 * stays at position n[b]).  With n_new NULL an EAGLE-3 round ingests every
 * one of the n[b] positions (a first round) and an EAGLE-1 round none.
 * The caller keeps 1 <= n_new[b] <= n[b] and cu_new the prefix sum of n_new;
 * rows that break this are skipped on the device, never written outside
 * k_ctx/v_ctx.
 */
typedef struct eagle_kv {
  int32_t B;
  int32_t max_n;       /* host copy of max_b n[b]  (sizes launch grids)  */
  int64_t total_n;     /* host copy of sum_b n[b]                         */
  const int32_t *n;    /* device [B]   */
  const int32_t *cu_n; /* device [B+1] */
  void *k_ctx, *v_ctx, *k_slot, *v_slot, *feat_slot; /* device */
  int64_t total_new;      /* host copy of sum_b n_new[b] (0 when n_new NULL) */
  const int32_t *n_new;   /* device [B] or NULL                             */
  const int32_t *cu_new;  /* device [B+1] or NULL; required with n_new      */
} eagle_kv;

/*
 * Draft tree of every request.
 *   CHAIN    gamma steps of top-1
 *   STATIC   fixed template (EAGLE-1, "Drafting a Tree, Not a Chain"):
 *            template_parent[i] is the parent of template node i+1 (node 0 is
 *            the root, parents precede children, siblings in rank order); a
 *            node's token is the rank-th best of its parent's top-k
 *   DYNAMIC  EAGLE-2 ("EAGLE-2: expand and rerank"): value = product of the
 *            confidences on the root path; at every step the top_k nodes of
 *            the newest depth by value are expanded to their top_k children;
 *            after gamma steps the top_m nodes by value are kept
 * Ordering: top-k by (logit desc, id asc); frontier and rerank by (value
 * desc, depth asc, creation index asc); creation index = (step, frontier rank
 * of the parent, child rank).  value(child) = fp32(value(parent) * conf).
 * Position id of a node = root position + depth (root at n_b for EAGLE-1, at
 * n_b - 1, the last verified position, for EAGLE-3).
 * `state` (device, eagle_tree_state_bytes) holds the node pool, the rows of
 * the next step, this step's top-k and the verify tree; its layout is given by
 * eagle_tree_layout.
 */
typedef struct eagle_tree {
  int32_t kind;          /* EAGLE_TREE_* */
  int32_t B, gamma, top_k, top_m;
  int32_t n_template;            /* STATIC: number of non-root nodes      */
  const int32_t *template_parent;/* STATIC: HOST array [n_template]       */
  float inv_temp;                /* s in conf = softmax(s * logits):
                                    0 < s <= EAGLE_MAX_INV_TEMP           */
  void *state;                   /* device */
  size_t state_bytes;
  /* Sampled drafting ("Speculative Decoding Deep Dive III", EAGLE-1
   * "Inference": the drafter samples t ~ p-hat).  sample = 1: the top_k
   * children of a row are drawn without replacement from
   * softmax(inv_temp * logits) by Gumbel-top-k: the top_k of
   * inv_temp * logit + G, G = -log(-log(u)) in fp32 with
   * u = ((bits >> 9) + 0.5) 2^-23 and bits from Philox4x32-10 (Salmon et al.,
   * SC'11) with key (low, high word of sample_seed) and counter
   * (id / 4, b * 1024 + node, 0, 0), word id % 4; confidences stay the
   * softmax probabilities.  sample = 0: top_k by logit. */
  uint64_t sample_seed;
  int32_t sample;
} eagle_tree;

/* Byte offsets of the arrays inside eagle_tree.state (all per request b).
 *   pool_* [B][pool_cap]: tok, parent (pool index, -1 root), depth, slot
 *     (-1 if never expanded) int32; conf, value fp32
 *   pool_count [B], slot_count [B], root_pos [B] int32; slot_mask [B][64] u64
 *   rows of each draft step, double-buffered by step parity: the rows of
 *   step s are entries (s % 2) * B*max_rows + b * W_s + i of
 *     row_node, row_tok, row_pos int32, row_slot (b*64 + slot), row_pidx int32,
 *     row_mask u64, each [2][B*max_rows]
 *     (row_pidx = index of the input feature: b for the root row of an
 *      EAGLE-1 round, the packed row of the last verified position for
 *      EAGLE-3, else b*64 + parent slot)
 *   topk_id [B*max_rows][top_k] int32, topk_conf [..][top_k] fp32,
 *   lse [B*max_rows] fp32 (log-partition of s * logits)
 *   verify tree [B][64]: f_node, f_tok, f_parent (position), f_depth, f_pos
 *     int32, f_mask u64 (ancestor-or-self over positions); f_count [B]
 *   choice [B][64] int32: target's greedy token per verify position
 *   choice_part [B][64][16] (float max, int32 index): argmax of each of the
 *     16 vocabulary slices of a verify position's target logits
 *   status [B] int32: 0 while request b's tree state is consistent; set to
 *     EAGLE_TREE_STATE_BAD by an expansion that finds its pool or slots
 *     already full (calls out of order); eagle_tree_init clears it, and a
 *     verify of a flagged request reports accept_len[b] = -1
 */
#define EAGLE_TREE_STATE_BAD 1
typedef struct eagle_tree_layout {
  int32_t pool_cap, max_rows, positions;
  size_t pool_tok, pool_parent, pool_depth, pool_slot, pool_conf, pool_value;
  size_t pool_count, slot_count, root_pos, slot_mask;
  size_t row_node, row_tok, row_pos, row_slot, row_pidx, row_mask;
  size_t topk_id, topk_conf, lse;
  size_t f_node, f_tok, f_parent, f_depth, f_pos, f_mask, f_count;
  size_t choice, choice_part;
  size_t status;
  size_t total;
} eagle_tree_layout;

/* Fill *out for this tree.  Returns EAGLE_OK or EAGLE_EINVAL/EUNSUPPORTED. */
int eagle_tree_layout_of(const eagle_tree *tree, eagle_tree_layout *out);
/* Bytes needed for tree->state (0 on invalid arguments). */
size_t eagle_tree_state_bytes(const eagle_tree *tree);
/* Rows per request processed by draft step `step` (0 on invalid arguments). */
int eagle_step_rows(const eagle_tree *tree, int step);
/* Workspace bytes eagle_draft_step / eagle_tree_attend need (0 on error). */
size_t eagle_workspace_bytes(const eagle_head *head, const eagle_kv *kv,
                             const eagle_tree *tree);

/*
 * Start the round: node 0 of every request is the anchor token root_tokens[b]
 * (device [B]) with value 1; the rows of step 0 are the B roots.
 */
int eagle_tree_init(const eagle_head *head, const eagle_kv *kv,
                    const eagle_tree *tree, const int32_t *root_tokens,
                    void *stream);

/*
 * One draft step ("The recurrence, written out"): for every row of the step
 * (node u of request b at depth `step`):
 *   EAGLE-1: x = [f ; emb(tok(u))] with f = f_root[b] for the root, else the
 *            layer output stored in the parent's slot; h = x W_fc^T.  In the
 *            steady state step 0 first ingests the new positions j:
 *            h_j = [lmh_j ; emb(ctx_tokens[j])] W_fc^T, K/V of N1(h_j) to
 *            their rows of k_ctx/v_ctx.
 *   EAGLE-3: step 0 ingests every new verified position j of every request
 *            (all n[b] of them, or the last n_new[b] in the steady state):
 *            g_j = lmh_j W_fuse^T, x_j = g_j + emb(ctx_tokens[j]); K/V of each
 *            are written to k_ctx/v_ctx at the position's own row of the
 *            request's segment; the root row is each request's last position.
 *            Later steps: h = a_parent + emb(tok(u)).
 *   then the decoder layer at position root_pos + depth; attention sees the
 *   request's context plus the ancestor-or-self slots (row_mask); K/V and the
 *   output go to the row's slot; logits = W_LM out; top_k ids, their
 *   confidences softmax(inv_temp * logits)[id] and the log-partition go to
 *   the tree state.
 * f_root:     device [B][d]           (EAGLE-1, step 0; else unused)
 * lmh:        device [T][3d]          (EAGLE-3, step 0; l, m, h concatenated;
 *             T = total_new in the steady state, else total_n; packed by
 *             cu_new, else cu_n); EAGLE-1 steady state: [total_new][d], the
 *             target's feature of the position before each new one
 * ctx_tokens: device [T] int32        (step 0 of an ingest; EAGLE-3: token
 *             after each ingested position, the anchor token last; EAGLE-1:
 *             the token at each new position)
 * logits_out: optional device [M][V] fp32 (M = B * eagle_step_rows)
 * feat_out:   optional device [M][d] in the head dtype (layer outputs)
 * ws:         device workspace of at least eagle_workspace_bytes
 */
int eagle_draft_step(const eagle_head *head, const eagle_kv *kv,
                     const eagle_tree *tree, int step, const void *f_root,
                     const void *lmh, const int32_t *ctx_tokens,
                     float *logits_out, void *feat_out, void *ws,
                     size_t ws_bytes, void *stream);

/*
 * eagle_draft_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same step and arguments, with the workspace taken from a device array
 * the library holds, EAGLE_NOALLOC_SCRATCH_BYTES on every GPU it runs on,
 * until the process ends, instead of a caller buffer.  Nothing in the call
 * allocates.  Returns EAGLE_ECAPACITY when eagle_workspace_bytes(head, kv,
 * tree) exceeds the array (it covers the 8B-shaped static tree and the small
 * shapes, not the large-batch trees), EAGLE_EHIP if the array's address
 * cannot be obtained.  Every call on one GPU shares that GPU's array and
 * leaves its contents behind: calls that overlap on one GPU race, whatever
 * their streams, so order them on one stream.
 */
#define EAGLE_NOALLOC_SCRATCH_BYTES (32u << 20)
int eagle_draft_step_noalloc(const eagle_head *head, const eagle_kv *kv,
                             const eagle_tree *tree, int step, const void *f_root,
                             const void *lmh, const int32_t *ctx_tokens,
                             float *logits_out, void *feat_out, void *stream);

/*
 * Grow the tree from draft step `step`'s top-k ("EAGLE-2: expand and
 * rerank"; chain and static trees follow their shape).  Writes the rows of
 * step+1.  When step == gamma-1 it also reranks (dynamic: keep top_m by
 * value; chain/static: keep every node) and writes the verify tree: the kept
 * nodes in creation order, root at position 0, parent positions, depth,
 * position ids and ancestor-or-self masks ("Tree attention in one
 * verification pass").
 */
int eagle_tree_expand_rerank(const eagle_tree *tree, int step, void *stream);

/*
 * Tree-masked attention over the verify tree, standing in for one target
 * layer's verification pass ("Tree attention in one verification pass"): row
 * u of request b has x = emb(f_tok[u]); q, k, v = N1(x) W^T with RoPE at
 * f_pos[u]; it attends to the whole context plus the tree positions in
 * f_mask[u].  out: device [B*positions][Hq*hd] in the head dtype.
 */
int eagle_tree_attend(const eagle_head *head, const eagle_kv *kv,
                      const eagle_tree *tree, void *out, void *ws,
                      size_t ws_bytes, void *stream);

/*
 * Greedy verification (explainer steps 3-4): the target's choice at verify
 * position u is argmax_v target_logits[b][u][v] (lowest id on ties); starting
 * at the root, move to the child whose token equals the choice while one
 * exists.
 * target_logits: device [B][positions][vocab], dtype EAGLE_BF16 or EAGLE_F32
 *   (positions >= the verify tree's position count, vocab >= 1)
 * accept_len:  device [B]          accepted draft tokens (0..gamma)
 * accept_path: device [B][gamma+1] verify positions, root first, -1 padded
 * out_tokens:  device [B][gamma+1] accepted tokens then the target's token at
 *              the deepest accepted node, -1 padded
 */
int eagle_tree_verify(const eagle_tree *tree, const void *target_logits,
                      int positions, int vocab, int dtype, int32_t *accept_len,
                      int32_t *accept_path, int32_t *out_tokens, void *stream);

/*
 * Lossless verification by multi-round speculative sampling over the verify
 * tree ("Speculative Decoding Deep Dive III", EAGLE-1 "Inference": one
 * target pass checks the tree and keeps the target's distribution;
 * "transformer_math / tm_eagle_deep", "Why draft confidence is a usable
 * acceptance proxy": keep a drafted token with probability
 * min(1, p_target / p_draft)).  Top-k drafting proposes each child with
 * certainty (p_draft = 1), so at verify position u, with the target
 * distribution p = softmax(inv_temp * target_logits[b][u]), the children of
 * u are tried in verify-tree order and child i (token x) is accepted iff
 *   draws[b][u][i] < p(x) / (1 - sum of p over the children rejected before it);
 * the walk moves to the first accepted child.  Where no child is accepted
 * (or u has none, or is at depth gamma) one token is drawn from p with the
 * rejected tokens removed and renormalised: the smallest token id whose
 * cumulative mass exceeds draws[b][u][16] times the residual mass.
 * Arithmetic: scaled logits and exponentials exp(v - max v) in fp32; sums of
 * 8 (bf16) or 4 (fp32) consecutive ids in fp32, every sum above that in
 * fp64, all in a fixed order (bit-reproducible).
 * draws:   device [B][positions][EAGLE_VERIFY_DRAWS] fp32 uniforms in [0, 1)
 *          (the caller's random numbers; the library draws none)
 * inv_temp: > 0 and finite.  vocab <= 524288 (bf16) or 262144 (fp32), else
 * EAGLE_EUNSUPPORTED.  Other arguments and outputs as eagle_tree_verify;
 * one workgroup per request reads only the rows the walk visits.
 */
int eagle_tree_verify_sample(const eagle_tree *tree, const void *target_logits,
                             int positions, int vocab, int dtype, float inv_temp,
                             const float *draws, int32_t *accept_len,
                             int32_t *accept_path, int32_t *out_tokens,
                             void *stream);

/*
 * Lossless verification of a sampled draft (tree->sample = 1): multi-round
 * speculative sampling with the draft's proposal probabilities
 * ("Speculative Decoding Deep Dive III", EAGLE-1 "Inference": the drafter
 * samples its tokens and one target pass checks the tree, keeping the
 * target's distribution; "transformer_math / tm_eagle_deep", "Why draft
 * confidence is a usable acceptance proxy": keep a drafted token with
 * probability min(1, p_target / p_draft)).
 * At verify position u, with p = softmax(inv_temp * target_logits[b][u]) and
 * the draft q = softmax(tree->inv_temp * z), z = u's row of draft_logits, the
 * children drafting drew at u (every one of them, in draw order, also those
 * the verify tree dropped) are tested in turn: the j-th, token x, is kept iff
 *   draws[b][u][j] < r_j(x) / q_j(x),
 * q_j = q over the tokens not drawn before x, renormalised; r_1 = p and, after
 * a rejection, r_{j+1} = max(r_j - q_j, 0) renormalised.  A kept child in the
 * verify tree continues the walk; a kept child the tree dropped ends it with
 * its token.  With none kept (or no drawn child) one token is drawn from the
 * last residual: the smallest id whose cumulative mass exceeds
 * draws[b][u][16] times the residual mass.
 * draft_logits: device fp32, the logits_out of draft steps 0 .. gamma-1 one
 *   after another: step s's block holds B * eagle_step_rows(tree, s) rows of
 *   vocab entries in that step's row order (rows b * W_s + i).
 * Arithmetic: fp32 scaled logits and expf per id; sums of 4 consecutive ids in
 * fp32, every sum above that and every test in fp64, in a fixed order
 * (bit-reproducible).  One workgroup per request; each rejection costs one
 * pass over the two rows of the visited position.
 * Returns EAGLE_EINVAL when tree->sample != 1 (top-k drafts propose each child
 * with certainty: eagle_tree_verify_sample), EAGLE_EUNSUPPORTED for
 * vocab > 524288.  Other arguments and outputs as eagle_tree_verify_sample;
 * accept_len[b] = -1 (path[b][0] = -1) when request b's tree state is
 * inconsistent (flagged, or a drawn node without its draft row).
 */
int eagle_tree_verify_sample_drafted(const eagle_tree *tree, const void *target_logits,
                                     int positions, int vocab, int dtype, float inv_temp,
                                     const float *draft_logits, const float *draws,
                                     int32_t *accept_len, int32_t *accept_path,
                                     int32_t *out_tokens, void *stream);

/*
 * The target model for its verification pass: n_layers decoder layers of the
 * draft head's layer shape (d, heads, head_dim, ffn, act, norm, eps,
 * rope_theta and dtype are the head's), each with its own context cache, a
 * final RMSNorm, and the embedding and LM head the draft head shares.
 * Every pointer is a device pointer except `layers` (a HOST array).
 */
typedef struct eagle_layer {
  const void *w_q, *w_k, *w_v, *w_o;          /* [out][in], as in eagle_head */
  const void *w_gate, *w_up, *w_down;
  const void *norm1_g, *norm1_b, *norm2_g, *norm2_b;  /* [d]; b: LayerNorm */
  const void *k_ctx, *v_ctx;   /* [total_n][Hkv][hd] this layer's context cache
                                  (rotated), packed like eagle_kv's */
} eagle_layer;

typedef struct eagle_target {
  int32_t n_layers;
  const eagle_layer *layers;   /* HOST array [n_layers] */
  const void *final_norm_g;    /* [d] RMSNorm gain before the LM head */
} eagle_target;

/*
 * The target's verification pass over the verify tree ("transformer_math /
 * tm_eagle_deep", "Tree attention in one verification pass": the flattened
 * tree goes through the target once; each position attends to the context
 * and to its ancestors-or-self, at position id root position + depth).
 * Row m = b * positions + u is verify position u of request b: x = emb(f_tok),
 * then every layer (as eagle_draft_step's decoder layer, with the layer's
 * context cache and the tree masks f_mask), then RMSNorm(final_norm_g) and the
 * LM head.
 * head:   dims, dtype, emb and lm_head (its draft weights are not read)
 * kv:     B, n, cu_n, max_n, total_n of the target's context: request b's
 *         cache holds positions [0, n[b]), which must end where the tree's
 *         root position starts (EAGLE-1 roots sit at n[b]); k_ctx / v_ctx are
 *         not read (each layer brings its own); slots as for eagle_draft_step
 * logits_out: device fp32 [B * positions][vocab] (positions from
 *         eagle_tree_layout_of), for eagle_tree_verify(_sample) with EAGLE_F32
 * k_tree, v_tree: optional device [n_layers][B][64][Hkv][hd]: every layer's
 *         keys / values of the verify positions (for eagle_kv_commit); both
 *         NULL: kept in the workspace only
 * hidden_out: optional device [n_layers + 1][B * positions][d] in the head
 *         dtype: the residual stream entering every layer (entry 0 =
 *         emb(f_tok)) and leaving the last one, as stored between kernels;
 *         NULL: kept in the workspace only
 * ws:     device workspace of eagle_target_workspace_bytes
 */
int eagle_target_verify_logits(const eagle_head *head, const eagle_target *target,
                               const eagle_kv *kv, const eagle_tree *tree,
                               float *logits_out, void *k_tree, void *v_tree,
                               void *hidden_out, void *ws, size_t ws_bytes, void *stream);
/* Workspace bytes eagle_target_verify_logits needs (0 on invalid arguments). */
size_t eagle_target_workspace_bytes(const eagle_head *head, const eagle_target *target,
                                    const eagle_kv *kv, const eagle_tree *tree);

/*
 * Commit of the accepted path to a key/value cache ("EAGLE / DFlash / DSpark"
 * explainer, "How speculative decoding works", step 4: the accepted prefix
 * joins the sequence before the next round): for request b and
 * i = 0 .. accept_len[b], row accept_path[b][i] of request b in k_tree /
 * v_tree ([B][64][kv_heads][head_dim], one layer's tree keys and values, e.g.
 * from eagle_target_verify_logits) is copied to row dst_row[b] + i of k_dst /
 * v_dst ([dst_rows][kv_heads][head_dim]): the root first, then the accepted
 * nodes in path order; the rest of the tree is dropped.  accept_len /
 * accept_path as written by eagle_tree_verify(_sample).  The caller leaves
 * room for accept_len[b] + 1 rows after dst_row[b]; rows outside
 * [0, dst_rows) are skipped.  Rows must be whole 16-byte multiples and every
 * buffer 16-byte aligned (EAGLE_EINVAL otherwise).
 */
int eagle_kv_commit(const eagle_tree *tree, int kv_heads, int head_dim, int dtype,
                    const int32_t *accept_len, const int32_t *accept_path,
                    const void *k_tree, const void *v_tree, const int32_t *dst_row,
                    int64_t dst_rows, void *k_dst, void *v_dst, void *stream);

/*
 * Kernel timing for benchmarks (off by default).  While enabled, every launch
 * of a kernel family is bracketed by HIP events recorded on the launch stream,
 * and the algorithmic bytes and flops of that launch (each weight, cache and
 * logit byte counted once) are added up.  eagle_profile_read waits for the
 * recorded events and returns, since the last reset, the launch count, the
 * summed kernel time in milliseconds, the summed bytes / flops and the summed
 * per-launch roofline time max(bytes / 8 TB/s, flops / peak) in milliseconds
 * (peak: 2.5 PFLOP/s dense bf16 MFMA, 157.3 TFLOP/s fp32; MI355X datasheet).  Up to
 * 16384 launches per family are timed; later ones are counted but not timed
 * (timed_launches tells how many were).  Not thread-safe across concurrent
 * callers.
 */
enum {
  EAGLE_PROF_LMHEAD = 0,  /* LM head + fused softmax/top-k partials      */
  EAGLE_PROF_GEMM = 1,    /* weight-streaming GEMMs of the draft layer    */
  EAGLE_PROF_ATTN = 2,    /* tree-masked attention (split-KV partials)    */
  EAGLE_PROF_VERIFY = 3,  /* target-logit argmax of the verifier          */
  EAGLE_PROF_OTHER = 4,   /* epilogues, merges, tree bookkeeping          */
  EAGLE_PROF_FAMILIES = 5
};
/* family_mask: bit (1 << EAGLE_PROF_x) enables family x; 0 disables all. */
int eagle_profile_enable(int family_mask);
int eagle_profile_reset(void);
int eagle_profile_read(int family, int64_t *launches, int64_t *timed_launches,
                       double *total_ms, double *bytes, double *flops,
                       double *roofline_ms);

/* Text for a status code. */
const char *eagle_strerror(int status);
/* Library version string. */
const char *eagle_version(void);

#ifdef __cplusplus
}
#endif
#endif /* EAGLE_H */
