/*
 * eagle3.h -- C ABI of the MI355X (gfx950) EAGLE-3 draft-and-verify library.
 *
 * The method: "EAGLE-3 精读" (edgeai1 speculative-decoding knowledge base)
 *   §1 为什么推翻 feature regression -- low/mid/high target features are
 *      concatenated to 3d and projected to d (g); a one-layer draft decoder
 *      combines g, its own state and the token embedding; the target model
 *      and its LM head are frozen.
 *   §2 Training-Time Test -- ~5 self-fed rollout steps trained in one graph
 *      under a special attention mask; inference uses EAGLE-2's
 *      confidence-value dynamic tree and strict target verification.
 *   §5 正确性、复现与风险 -- the standard verifier keeps the greedy sequence
 *      or the sampling distribution if the residual correction is kept.
 * EAGLE-4 blog (10100.com), 几条技术路线正在收敛 -- tree confidence is the
 *   product of draft probabilities.  "EAGLE-3" quote page (scholarfeed) --
 *   every added tree depth is one more sequential drafter round.
 *
 * Conventions (all entry points)
 *  - Every pointer argument that names a tensor is DEVICE memory owned by
 *    the caller, row-major and contiguous, unless stated otherwise.  Struct
 *    arguments (eagle3_dims, eagle3_weights, eagle3_kv) are HOST memory read
 *    during the call only.  The library never allocates and keeps no state
 *    between calls: scratch memory comes from a caller workspace sized by
 *    the *_size queries, tree state lives in a caller buffer.
 *  - Each call validates its arguments on the host, then only enqueues
 *    kernels on `stream` (a hipStream_t; NULL = the default stream).  No
 *    call synchronises or copies to the host.  Enqueued work never uses
 *    hipMemset*, so every call may be captured into a HIP graph.
 *  - Types: activations, weights and KV are float32 (EAGLE3_F32) or
 *    bfloat16 (EAGLE3_BF16, raw 16-bit patterns) as `dims->dtype` says;
 *    residual stream, logits, log-probs, scores and CE are float32;
 *    verification uniforms are float64; ids and indices are int32; tree
 *    masks are uint64 bitsets.  Matrices are [out, in] row-major.
 *  - Errors: every call returns 0 (EAGLE3_OK) or a negative code.  Argument
 *    errors are detected before anything is launched; eagle3_last_error()
 *    gives a thread-local message for the most recent failure.
 *  - Calls that share a workspace or tree-state buffer must be ordered on
 *    one stream; concurrent calls on one buffer race.
 *  - Workspaces of eagle3_fuse / eagle3_draft_step / eagle3_topk / the TTT
 *    forward need no initialisation (the top-k arrival counters are cleared
 *    by each call itself).  The verify workspace must be zero-filled once
 *    after allocation: its last sixth holds arrival counters that every
 *    call leaves at zero.
 */
#ifndef EAGLE3_H
#define EAGLE3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ------------------------------------------------------ */
#define EAGLE3_OK 0
#define EAGLE3_EINVAL (-1)       /* NULL pointer, bad size, dtype mismatch          */
#define EAGLE3_ECAPACITY (-2)    /* (D-1)k > 64 tree slots, m+1 > 64, k > 16, ...   */
#define EAGLE3_EUNSUPPORTED (-3) /* a shape the kernels do not handle (see each call)*/
#define EAGLE3_EWORKSPACE (-4)   /* workspace smaller than the size query returned  */
#define EAGLE3_EHIP (-5)         /* a HIP launch failed                             */
#define EAGLE3_ENUMERIC (-6)     /* NaN in target logits (written per request)      */

/* ---- enums ------------------------------------------------------------- */
#define EAGLE3_F32 0
#define EAGLE3_BF16 1

#define EAGLE3_COMMIT 0 /* draft_step: append committed rows (causal)        */
#define EAGLE3_TREE 1   /* draft_step: one row per frontier node (tree mask) */

#define EAGLE3_TOPK_ALL 0  /* top-k of every row                           */
#define EAGLE3_TOPK_LAST 1 /* top-k of the last row of each request only   */

#define EAGLE3_INIT 0  /* tree_expand: root's top-k -> depth-1 nodes  */
#define EAGLE3_STEP 1  /* tree_expand: one expansion round            */
#define EAGLE3_FINAL 2 /* tree_expand: top-m rerank -> verify tree    */

#define EAGLE3_GREEDY 0
#define EAGLE3_SAMPLE 1

#define EAGLE3_MAX_TREE_SLOTS 64 /* drafted tree rows per request per cycle */
#define EAGLE3_MAX_TOPK 16
#define EAGLE3_MAX_ROWS 64 /* query rows per request per draft_step */

typedef void *eagle3_stream_t; /* hipStream_t */

/* Drafter dimensions.  head_dim must be 64 or 128; n_q_heads a multiple of
 * n_kv_heads (q-head h reads KV head floor(h*n_kv_heads/n_q_heads)); d at
 * most 8192 and vocab at most 262144 (EAGLE3_EUNSUPPORTED otherwise).  With
 * dtype BF16 every GEMM K (3d, 2d, n_q_heads*head_dim, ffn) must be a
 * multiple of 32 and d a multiple of 16; ffn a multiple of 8.  rms_eps is
 * the RMSNorm epsilon; rope_theta the rotary base (rotate-half form). */
typedef struct eagle3_dims {
  int32_t d, n_q_heads, n_kv_heads, head_dim, ffn, vocab, dtype;
  float rms_eps, rope_theta;
} eagle3_dims;

#define EAGLE3_LAYOUT_ROWMAJOR 0 /* matrices [out, in] row-major                       */
#define EAGLE3_LAYOUT_PACKED 1   /* fc/qkv/o/gate_up/down/lm in MFMA fragment order     */

/* Drafter weights (device, dtype of dims, [out, in] row-major unless
 * layout == EAGLE3_LAYOUT_PACKED, see eagle3_pack_weights):
 *  fc      [d, 3d]           fusion projection (rows: output features; the
 *                            3d inputs are [f_low | f_mid | f_high])
 *  emb     [vocab, d]        frozen target token embedding
 *  qkv     [(Hq+2Hkv)hd, 2d] rows: Hq*hd query, Hkv*hd key, Hkv*hd value;
 *                            the 2d inputs are [rms(emb[t]) | rms(s)]
 *  o       [d, Hq*hd]
 *  gate_up [2*ffn, d]        rows 0..ffn-1 gate, ffn..2ffn-1 up
 *  down    [d, ffn]
 *  lm      [vocab, d]        frozen target LM head
 *  norm_*  [d] float32       RMSNorm gains (embedding, state, FFN, output)
 * The EAGLE-3.1 variants that EAGLE-4 keeps (EAGLE-4 blog, the paragraph on
 * what EAGLE-4 keeps of EAGLE-3.1), each off when its gains are NULL:
 *  norm_fc         FC norm: g = rms(fc . [f_low|f_mid|f_high]) * norm_fc
 *  norm_post_attn, norm_post_ffn  post-norm (both or neither): h1 =
 *                  rms(s + o.a) * norm_post_attn; the FFN reads h1 itself
 *                  (norm_ffn unused); h2 = rms(h1 + down.(...)) *
 *                  norm_post_ffn, which children receive as their state. */
typedef struct eagle3_weights {
  const void *fc, *emb, *qkv, *o, *gate_up, *down, *lm;
  const float *norm_e, *norm_s, *norm_ffn, *norm_out;
  int32_t layout; /* EAGLE3_LAYOUT_ROWMAJOR or EAGLE3_LAYOUT_PACKED */
  const float *norm_fc, *norm_post_attn, *norm_post_ffn;
} eagle3_weights;

/* Draft KV cache of a batch of requests (device, dtype of dims).
 *  k, v        committed keys/values (after RoPE).  Contiguous when
 *              block_table == NULL: [B][cap][Hkv][hd], row p = position p.
 *              Paged otherwise: a pool [n_blocks][block_size][Hkv][hd];
 *              logical row p of request b lives in block
 *              block_table[b*max_blocks + p/block_size], offset p%block_size.
 *  ctx_len     [B] int32: committed rows of each request before this call.
 *  tk, tv      tree slots [B][64][Hkv][hd] (one slot per drafted tree row). */
typedef struct eagle3_kv {
  void *k, *v;
  int32_t cap;
  const int32_t *block_table;
  int32_t max_blocks, block_size;
  const int32_t *ctx_len;
  void *tk, *tv;
} eagle3_kv;

/* Bytes of the packed copy of fc, qkv, o, gate_up, down and lm (bf16 only). */
int eagle3_packed_weights_size(const eagle3_dims *dims, size_t *bytes);

/* Copy the six GEMM matrices of `src` (row-major, bf16) into `dst` (device,
 * dst_bytes >= eagle3_packed_weights_size) in MFMA fragment order, and fill
 * `packed` (host) with pointers into dst plus src's emb and norm gains,
 * layout = EAGLE3_LAYOUT_PACKED.  Fragment order of a matrix W [N][K]: for
 * each 16-row tile t, each 32-wide k chunk c and lane l < 64, the 16 bytes
 * W[row(t, l%16)][32c + 8(l/16) .. +8], where row() is the identity except
 * for qkv (rows i and i+hd/2 of one head share a tile at m and m+8) and
 * gate_up (gate row j and up row F+j share a tile at m and m+8).  A weight
 * streaming wave then reads each MFMA A operand as one contiguous 1 KB
 * block.  Enqueued on `stream`; src must stay valid until it completes. */
int eagle3_pack_weights(const eagle3_dims *dims, const eagle3_weights *src, void *dst, size_t dst_bytes,
                        eagle3_weights *packed, eagle3_stream_t stream);

/* Message for a return code (static string). */
const char *eagle3_strerror(int code);
/* Detail of the most recent failure on the calling thread ("" if none). */
const char *eagle3_last_error(void);
/* Library version string. */
const char *eagle3_version(void);

/* Workspace bytes needed by eagle3_fuse / eagle3_draft_step / eagle3_topk for
 * batch B with at most max_rows query rows per request (fuse: n <= B*max_rows
 * feature rows).  Contiguous KV prefixes up to max_ctx rows (paged: the
 * largest logical length) are covered.  No initialisation is needed. */
int eagle3_workspace_size(const eagle3_dims *dims, int B, int max_rows, int max_ctx,
                          size_t *bytes);

/* Bytes of tree state for B requests, top-k k and depth D. */
int eagle3_tree_state_size(int B, int k, int D, size_t *bytes);

/* Workspace bytes needed by eagle3_ttt_forward for B sequences of S tokens
 * and R rollout steps. */
int eagle3_ttt_workspace_size(const eagle3_dims *dims, int B, int S, int R, size_t *bytes);

/* Step 1 -- multi-layer feature fusion ("EAGLE-3 精读" §1):
 *   g[i] = [f_low(i) ; f_mid(i) ; f_high(i)] . fc^T       (no bias, no norm)
 * feats [n][3][d] (dtype), g [n][d] (dtype; bf16 rounds once, RNE).
 * fp32 accumulation.  n >= 1, processed in 64-row chunks by the
 * weight-streaming kernel.  ws: a workspace of eagle3_workspace_size
 * bytes. */
int eagle3_fuse(const eagle3_dims *dims, const eagle3_weights *w, const void *feats, int n,
                void *g, void *ws, size_t ws_bytes, eagle3_stream_t stream);

/* Step 2+3 -- one drafter round ("EAGLE-3 精读" §1; the quote page: one
 * sequential drafter round per tree depth), then the LM head and per-row
 * top-k with log-probabilities.
 *
 * Per query row (b, r) with state s, token t, position p:
 *   x = [rms(emb[t])*norm_e ; rms(s)*norm_s]; q,k,v = qkv.x; RoPE(q,k,p)
 *   a = softmax(q k^T / sqrt(hd)) v over the visible keys (GQA)
 *   h1 = s + o.a ; h2 = h1 + down.(silu(gate.u) * up.u), u = rms(h1)*norm_ffn
 *   logits = lm.(rms(h2)*norm_out)
 * bf16 workloads round x, q/k/v (after RoPE), a, u, silu(gate)*up and
 * rms(h2) to bf16; s, h1, h2 stay float32.
 *
 * mode COMMIT: rows r = 0..rows-1 of request b are new committed rows; row r
 *   writes its k/v at cache row ctx_len[b]+r and sees cache rows
 *   0..ctx_len[b]+r.  state = [B][rows][d] (dtype; normally g).  The last
 *   row's h2 is written to h_tree[b][0] (the root state).  parent_slot, anc
 *   unused (may be NULL).
 * mode TREE: row r of request b is a drafted tree node; state = NULL and s =
 *   h_tree[b][parent_slot[b][r]] (0 = root, 1+j = tree slot j).  It writes
 *   its k/v to tree slot slot_base+r, sees cache rows 0..ctx_len[b]-1 and
 *   every tree slot j with bit j of anc[b][r] set (its ancestors and itself),
 *   and writes h2 to h_tree[b][1+slot_base+r].  slot_base+rows <= 64.
 * tokens, pos [B][rows] int32.  h_tree [B][65][d] float32.
 * k in 1..16; topk_rows ALL -> topk_id/topk_lp [B][rows][k], LAST ->
 *   [B][1][k].  Order: logit desc, token id asc; lp = logit - logsumexp in
 *   float32.
 * logits_out: optional (NULL) float32 [B][rows or 1][vocab] copy of the
 *   logits of the rows whose top-k is taken.  With k = 1, bf16 weights,
 *   logits_out = NULL and at most 64 such rows, the logits are never stored:
 *   the LM head keeps per-block {max, sum of exp, lowest argmax} and merges
 *   them; ids are identical and lp agrees to float32 summation order.
 * Requires rows <= 64, head_dim in {64,128}; paged KV requires bf16. */
int eagle3_draft_step(const eagle3_dims *dims, const eagle3_weights *w, const eagle3_kv *kv,
                      int mode, int B, int rows, const void *state, const int32_t *parent_slot,
                      const int32_t *tokens, const int32_t *pos, const uint64_t *anc,
                      int slot_base, int k, int topk_rows, float *h_tree, int32_t *topk_id,
                      float *topk_lp, float *logits_out, void *ws, size_t ws_bytes,
                      eagle3_stream_t stream);

/* Step 3, efficient variant -- the two-stage draft LM head of EAGLE-4 (EAGLE-4
 * blog, 10100.com: the paragraph "EAGLE Efficient LM Head" and the section
 * 关于 Efficient LM Head).  Stage 1: a low-rank head scores every token,
 * s = a . (b . y) with y = rms(h2)*norm_out (b . y rounded to bf16 like every
 * GEMM input), and the `candidates` best float32 scores (score desc, id asc)
 * become the candidates.  Stage 2: the full LM head computes the exact logits
 * of the candidates only.  The top-k are the k best candidates by (exact
 * logit desc, id asc); lp = logit - logsumexp over the candidates (the draft
 * distribution restricted to the candidate set).
 *  a           [vocab, rank] bf16, b [rank, d] bf16, row-major or packed
 *              (eagle3_pack_matrix) as `layout` says
 *  rank        a multiple of 64, at most d
 *  candidates  k <= candidates <= 256 and <= vocab/16 */
typedef struct eagle3_lowrank_head {
  const void *a, *b;
  int32_t rank, candidates, layout;
} eagle3_lowrank_head;

/* eagle3_draft_step with the LM head replaced by the efficient head `head`
 * (same arguments and outputs otherwise; the full LM head `w->lm` is only
 * read for the candidates' rows).  logits_out, if not NULL, receives the
 * stage-1 scores [B][rows or 1][vocab]; cand_out / cand_logits_out, if not
 * NULL, the candidate ids (by score) [..][candidates] and their exact
 * logits.  Requires bf16, at most 64 LM-head rows (EAGLE3_EUNSUPPORTED
 * otherwise). */
int eagle3_draft_step_lowrank(const eagle3_dims *dims, const eagle3_weights *w, const eagle3_kv *kv,
                              int mode, int B, int rows, const void *state, const int32_t *parent_slot,
                              const int32_t *tokens, const int32_t *pos, const uint64_t *anc,
                              int slot_base, int k, int topk_rows, float *h_tree, int32_t *topk_id,
                              float *topk_lp, float *logits_out, const eagle3_lowrank_head *head,
                              int32_t *cand_out, float *cand_logits_out, void *ws, size_t ws_bytes,
                              eagle3_stream_t stream);

/* Copy one bf16 matrix src [n][k] (row-major, device) into dst (device,
 * dst_bytes >= n*k*2) in the MFMA fragment order of eagle3_pack_weights
 * (plain row order).  n a multiple of 16, k of 32.  Enqueued on `stream`. */
int eagle3_pack_matrix(const void *src, int n, int k, void *dst, size_t dst_bytes, eagle3_stream_t stream);

/* Step 3b -- EAGLE-2 confidence-value dynamic tree and rerank ("EAGLE-3 精读"
 * §2; EAGLE-4 blog, 几条技术路线正在收敛: confidence = product of draft
 * probabilities, kept here as a float32 sum of log-probs).
 *
 * INIT: topk_id/topk_lp [B][1][k] are the root's top-k; they become the
 *   depth-1 nodes (score = lp) and the frontier.  root_tok/root_pos [B] are
 *   stored.  Emits the frontier rows for the next TREE draft step.
 * STEP: topk_id/topk_lp [B][k][k] are the top-k of the k frontier rows (row
 *   rho = frontier rank rho).  Every child gets score = score(parent) + lp
 *   (one float32 add) and flat index rho*k+i; all k*k join the pool; the new
 *   frontier is the first k by (score desc, flat asc).  Unless the new depth
 *   equals D, emits the frontier rows.
 *   Frontier rows (INIT/STEP) -> next_tok, next_parent_slot (h_tree index of
 *   the parent), next_pos (root_pos + depth), next_anc (parent's bitset plus
 *   the node's own tree slot (depth-1)*k + rank), each [B][k].
 * FINAL: keeps the first m pool nodes by (score desc, depth asc, flat asc) --
 *   a set closed under ancestors -- and writes the verify tree in canonical
 *   order (root 0, then by depth, parent's index, child rank): v_tok,
 *   v_parent (-1 for the root), v_depth, v_pos [B][m+1] int32 and v_anc
 *   [B][m+1] (bit i set iff verify node i is an ancestor-or-self).
 * Limits: k <= 16, (D-1)*k <= 64, m+1 <= 64, m <= k + (D-1)k^2. */
int eagle3_tree_expand(int phase, int B, int k, int D, int m, const int32_t *root_tok,
                       const int32_t *root_pos, void *tree_state, const int32_t *topk_id,
                       const float *topk_lp, int32_t *next_tok, int32_t *next_parent_slot,
                       int32_t *next_pos, uint64_t *next_anc, int32_t *v_tok, int32_t *v_parent,
                       int32_t *v_depth, int32_t *v_pos, uint64_t *v_anc,
                       eagle3_stream_t stream);

/* Step 4 -- strict target verification ("EAGLE-3 精读" §5), one kernel that
 * walks each request's tree.
 * v_tok, v_parent [B][m+1] (canonical order as emitted by FINAL);
 * target_logits [B][m+1][V] float32 (row i = target logits after node i).
 * GREEDY: at each node t* = argmax (lowest id on ties); follow the child
 *   whose token is t* (the first in sibling order if several are), else
 *   stop: bonus = t*.
 * SAMPLE (temperature T > 0): float64 weights w(y) = exp((L-max)/T) and
 *   remaining mass Rm; child c (sibling order) is accepted iff u_try[c]*Rm <
 *   w(tok c), otherwise its token leaves the support (Rm -= w).  With no
 *   child accepted the bonus is the smallest token y outside the rejected set
 *   whose cumulative weight in id order exceeds u_res[node]*Rm (if rounding
 *   leaves none: the last y with w > 0).  u_try, u_res [B][m+1] float64.
 * Outputs: accept_len [B], accepted [B][Dmax] (verify-node indices, -1
 * padded), bonus [B], status [B] (0, or EAGLE3_ENUMERIC when a visited row
 * holds a NaN; -inf logits mean probability 0; every row needs one finite
 * logit).  A walk that reaches Dmax accepted nodes ends there as at a leaf.
 * ws: at least eagle3_verify_workspace_size bytes, zero-filled once after
 *   allocation.  Partials fill it from the start; 32-bit arrival counters
 *   (one per verify row, then one per request, 64 bytes apart) live from
 *   byte (ws_bytes / 6 * 5) rounded down to a multiple of 256, a place that
 *   depends on ws_bytes only.  Every call leaves the counters it used at
 *   zero, so calls of any (B, m, V) that fit may share one buffer as long as
 *   they pass the same ws_bytes and are ordered on one stream; passing
 *   another ws_bytes for the same buffer needs a new zero fill. */
int eagle3_verify(int B, int m, int V, int Dmax, const int32_t *v_tok, const int32_t *v_parent,
                  const float *target_logits, int mode, float temperature, const double *u_try,
                  const double *u_res, int32_t *accept_len, int32_t *accepted, int32_t *bonus,
                  int32_t *status, void *ws, size_t ws_bytes, eagle3_stream_t stream);

/* Scratch bytes eagle3_verify needs for B requests, m kept nodes, vocab V. */
int eagle3_verify_workspace_size(int B, int m, int V, size_t *bytes);

/* eagle3_verify without a caller workspace, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, semantics and outputs as
 * eagle3_verify, minus ws/ws_bytes.  The scratch is a static device array
 * of 8 MiB per GPU, held from the first call on that GPU until the process
 * ends; the first call on a device looks up its address and enqueues one
 * kernel that zero-fills it.  Nothing is allocated.  Shapes whose
 * eagle3_verify_workspace_size exceeds 8 MiB return EAGLE3_ECAPACITY (the
 * 8B batch-64 chain needs 0.3 MiB; B * (m+1) * ceil(V/4096) up to ~290k
 * fits).  Every call on one GPU shares the array, which keeps the last
 * call's contents: calls that overlap on one GPU (different streams, or
 * threads) race; order them on one stream. */
int eagle3_verify_noalloc(int B, int m, int V, int Dmax, const int32_t *v_tok, const int32_t *v_parent,
                          const float *target_logits, int mode, float temperature, const double *u_try,
                          const double *u_res, int32_t *accept_len, int32_t *accepted, int32_t *bonus,
                          int32_t *status, eagle3_stream_t stream);

/* Step 5 -- training-time-test forward ("EAGLE-3 精读" §2 and §5).
 * feats [B][S][3][d] (dtype), tokens [B][S].  Rows (j,i), j = 1..R: step 1
 * feeds (g_i, x_i) at position i; step j >= 2 feeds h2(j-1,i) and the
 * argmax token of (j-1,i) (or forced_tokens[b][j-2][i] when forced_tokens
 * != NULL, [B][R-1][S]) at position i+j-1.  Query (j,i) sees step-1 keys
 * i' <= i and its own chain keys (j',i), 2 <= j' <= j.
 * Outputs: pred [B][R][S] (argmax of logits(j,i)), ce [B][R][S] = logsumexp
 * - logit[x_{i+j}] where i+j <= S-1 (0 elsewhere), loss[0] = mean of the
 * valid ce.  Logits are never materialised.  Requires dtype BF16, head_dim
 * 128 or 64, d and ffn multiples of 64, d <= 8192, S a multiple of 64
 * (EAGLE3_EUNSUPPORTED otherwise); token ids must lie in [0, vocab).
 * Precision: bf16 operands, fp32 accumulation; the attention probabilities
 * enter P.V in bf16; log-sum-exp merged in fp64.  The
 * EAGLE-3.1 norm variants (norm_fc, post-norm) are not supported here
 * (EAGLE3_EUNSUPPORTED).
 * ws: eagle3_ttt_workspace_size bytes, no initialisation needed.  All
 * outputs are written with fixed reduction orders (bit-reproducible). */
int eagle3_ttt_forward(const eagle3_dims *dims, const eagle3_weights *w, const void *feats,
                       const int32_t *tokens, int B, int S, int R, const int32_t *forced_tokens,
                       int32_t *pred, float *ce, float *loss, void *ws, size_t ws_bytes,
                       eagle3_stream_t stream);

/* Gradients of the training-time-test loss, fp32 device arrays in the
 * logical row-major layout of eagle3_weights (independent of w->layout):
 * fc [d][3d], qkv [(Hq+2Hkv)hd][2d], o [d][Hq hd], gate_up [2F][d] (gate
 * rows then up rows), down [d][F]; the RMSNorm gains [d]. */
typedef struct {
  float *fc, *qkv, *o, *gate_up, *down;
  float *norm_e, *norm_s, *norm_ffn, *norm_out;
} eagle3_grads;

/* Workspace bytes needed by eagle3_ttt_train (it keeps every step's
 * activations: about 3.8 GB per step plus 4.3 GB for one step's logit
 * gradient at the 8B drafter's shape with B*S = 16384; 43.3 GB for 5 steps). */
int eagle3_ttt_train_workspace_size(const eagle3_dims *dims, int B, int S, int R, size_t *bytes);

/* Training-time-test forward and backward ("EAGLE-3 精读" §1: the target
 * and its LM head are frozen and the light decoder is trained; §2: the
 * rollout's CE at every step under the training-time-test mask).  The
 * forward and its outputs are those of eagle3_ttt_forward; `grads` receives
 * the gradients of loss[0] (the mean CE over the valid rows) with respect to
 * the drafter's trained parameters: the fusion FC, the layer's qkv, o,
 * gate_up and down, and its gains norm_e, norm_s, norm_ffn, norm_out
 * (every array overwritten).  The embedding and the LM head get none, nor
 * do the fed tokens (an argmax or forced choice); gradients reach earlier
 * steps through the fed state h2 and through the keys and values later
 * queries attend to.  bf16 roundings of the forward pass gradients straight
 * through.  Precision: bf16 GEMM operands (every gradient tensor that feeds a
 * GEMM is rounded to bf16), fp32 accumulation; the weight gradients sum all
 * R*B*S rows in one fp32 accumulation, deterministic (fixed orders, no
 * atomics).  Requirements: those of eagle3_ttt_forward plus Hq/Hkv in
 * {1, 2, 4, 8} and vocab a multiple of 16 (EAGLE3_EUNSUPPORTED otherwise).
 * Optimizer steps, clipping and data are the caller's.  ws:
 * eagle3_ttt_train_workspace_size bytes, no initialisation needed. */
int eagle3_ttt_train(const eagle3_dims *dims, const eagle3_weights *w, const void *feats,
                     const int32_t *tokens, int B, int S, int R, const int32_t *forced_tokens,
                     int32_t *pred, float *ce, float *loss, const eagle3_grads *grads, void *ws,
                     size_t ws_bytes, eagle3_stream_t stream);

/* ---- EAGLE-4 Harness: cost-aware tree control ----------------------------
 * (EAGLE-4 blog, the EAGLE-Harness paragraph: a warm-up measures draft and
 * verify times over batch sizes, context lengths and token counts into a
 * lookup table; every round asks, in three places, whether the expected
 * extra accepted tokens per extra unit of time exceed a threshold: one more
 * draft layer, how many tokens to verify, and the branch cap per node, 8 at
 * light load and 4 at heavy load.  The section on converging trends: the
 * confidence is the product of draft probabilities, compensated by a
 * threshold that rises with depth.)
 *
 * The rules are host code; their inputs are a few scores per request
 * (eagle3_tree_confidence copies them out of the tree state, or the top-k
 * log-probs of the root) and the warm-up table.  All arithmetic in double,
 * sums in index order; confidence c = exp(log-confidence).  Every pointer
 * of these calls is HOST memory except where stated. */
#define EAGLE3_COST_DRAFT 0  /* one drafter round: tok rows per request (eagle3_draft_step) */
#define EAGLE3_COST_VERIFY 1 /* one verification step: tok verify rows per request */

/* Warm-up table: batch[n_batch], ctx[n_ctx], tok[n_tok] ascending measured
 * values; draft_ms / verify_ms [n_batch][n_ctx][n_tok] milliseconds. */
typedef struct eagle3_cost_table {
  int32_t n_batch, n_ctx, n_tok;
  const int32_t *batch, *ctx, *tok;
  const float *draft_ms, *verify_ms;
} eagle3_cost_table;

/* Time of `kind` at (B, ctx, n tokens per request): B and ctx take the
 * smallest measured value >= them (the largest if none is); n is
 * interpolated linearly between measured token counts, clamped to the
 * measured range. */
int eagle3_harness_cost(const eagle3_cost_table *t, int kind, int B, int ctx, float n, double *ms);

/* One more draft layer?  frontier_logconf [B][k]: the log-confidences of
 * each request's frontier (eagle3_tree_confidence).  go = 1 iff
 *   sum_b sum_j c_bj / T_draft(B, ctx, k) > tau0 * (1 + alpha * depth)
 * (or the round's time is not positive); depth = the frontier's depth. */
int eagle3_harness_continue(const eagle3_cost_table *t, int B, int ctx, int k, int depth,
                            const float *frontier_logconf, double tau0, double alpha, int *go);

/* How many drafted tokens to verify: logconf_sorted [B][m_max], each
 * request's pool log-confidences in rerank order (descending).  Rank i is
 * kept while sum_b c_b,i / (T_verify(B, ctx, i+2) - T_verify(B, ctx, i+1))
 * > tau (a rank whose extra time is not positive is kept); m = the number
 * of leading ranks kept, 0..m_max. */
int eagle3_harness_verify_count(const eagle3_cost_table *t, int B, int ctx, int m_max, const float *logconf_sorted,
                                double tau, int *m);

/* Branch cap: root_lp [B][8], the root's top-8 log-probs (draft step with
 * k = 8).  k = 8 iff sum_b sum_{i=4..7} exp(root_lp[b][i]) /
 * (T_draft(B, ctx, 8) - T_draft(B, ctx, 4)) > tau (or the extra time is
 * not positive), else 4. */
int eagle3_harness_branch_cap(const eagle3_cost_table *t, int B, int ctx, const float *root_lp, double tau, int *k);

/* The harness's inputs from the tree state (DEVICE pointers, enqueued on
 * `stream`): frontier_logconf [B][k], the current frontier's scores in
 * frontier-rank order; pool_logconf [B][m_max], the pool's scores in
 * rerank order (descending), -inf past the pool.  Either may be NULL. */
int eagle3_tree_confidence(int B, int k, int D, int m_max, const void *tree_state, float *frontier_logconf,
                           float *pool_logconf, eagle3_stream_t stream);

/* ---- the target's verification forward ---------------------------------
 * ("EAGLE-3 精读" §2 and §5: drafting ends in strict verification by the
 * target's standard verifier, which needs the target's logits at every
 * kept node; §1: the target exposes low/mid/high hidden states, the next
 * fusion's input; the "EAGLE-3" quote page (scholarfeed): verification is
 * the larger part of the computation.)
 *
 * The target: n_layers pre-norm decoder layers with the drafter's layer
 * shape (eagle3_dims: d, heads, head_dim, ffn, vocab, dtype, rms_eps,
 * rope_theta) and a d-wide attention input, then a final RMSNorm and the LM
 * head.  Per layer, on the float32 residual stream h:
 *   x = rms(h)*norm_attn; q,k,v = qkv.x; RoPE(q,k,pos); a = attention
 *   h1 = h + o.a;  h = h1 + down.(silu(gate.u) * up.u), u = rms(h1)*norm_ffn
 * The stream starts at the token embedding; logits = lm.(rms(h)*norm_out).
 * bf16 targets round x, q/k/v, a, u, silu(gate)*up, rms(h)*norm_out and the
 * features to bf16 like the drafter.
 *
 * One target layer (device matrices, dtype of dims, [out, in] row-major or
 * packed by eagle3_pack_target_layer as eagle3_target.layout says):
 *  qkv     [(Hq+2Hkv)hd, d]    o [d, Hq*hd]
 *  gate_up [2*ffn, d]          down [d, ffn]
 *  norm_attn, norm_ffn [d] float32 */
typedef struct eagle3_target_layer {
  const void *qkv, *o, *gate_up, *down;
  const float *norm_attn, *norm_ffn;
} eagle3_target_layer;

/* The target model.  layers: HOST array [n_layers].  emb, lm [vocab, d]
 * (lm packed by eagle3_pack_matrix when layout is PACKED); norm_out [d]
 * float32.  feat_layers: the low, mid and high feature layers, each in
 * 1..n_layers, counted from 1 (feature j = the state h after layer
 * feat_layers[j]); they may repeat. */
typedef struct eagle3_target {
  int32_t n_layers;
  const eagle3_target_layer *layers;
  const void *emb, *lm;
  const float *norm_out;
  int32_t layout;
  int32_t feat_layers[3];
} eagle3_target;

/* Bytes of one layer's packed copy (bf16 only). */
int eagle3_target_layer_packed_size(const eagle3_dims *dims, size_t *bytes);
/* Copy one layer's four matrices (row-major bf16) into dst in MFMA fragment
 * order (qkv: RoPE pairs share a tile; gate_up: gate/up rows share a tile;
 * as eagle3_pack_weights) and fill `packed` (host) with pointers into dst
 * plus src's gains.  Enqueued on `stream`; src must stay valid until then. */
int eagle3_pack_target_layer(const eagle3_dims *dims, const eagle3_target_layer *src, void *dst,
                             size_t dst_bytes, eagle3_target_layer *packed, eagle3_stream_t stream);

/* Workspace bytes of eagle3_target_forward for B requests of `rows` verify
 * rows whose layers hold at most max_cap committed rows (contiguous cap, or
 * max_blocks*block_size when paged).  No initialisation is needed. */
int eagle3_target_workspace_size(const eagle3_dims *dims, int B, int rows, int max_cap, size_t *bytes);

/* The verification forward: target layers layer_begin..layer_end-1 on
 * B x rows verify rows.  Row i of request b is verify node i (0 = the root,
 * the last committed token, whose k/v are not yet cached): token
 * tokens[b][i], position pos[b][i]; in every layer it writes its k/v to tree
 * slot i of kv[l] (tk/tv [B][64][Hkv][hd]) and attends over committed rows
 * 0..ctx_len[b]-1 of kv[l] plus every tree slot j with bit j of anc[b][i]
 * set (the verify tree's ancestor-or-self bitsets, v_anc of
 * eagle3_tree_expand FINAL; a chain is the tree whose row i has bits 0..i).
 * Bits at or above `rows` must be clear.
 *  kv          HOST array [n_layers] of per-layer caches (eagle3_kv; paged
 *              needs bf16).  Only tree slots 0..rows-1 are written.
 *  hidden      [B][rows][d] float32: the residual stream.  layer_begin == 0
 *              starts it at emb[tokens] (ids clamped to [0, vocab)); else
 *              it must hold the state after layer_begin layers (a previous
 *              call's output).  On return: the state after layer_end layers.
 *  feats       [B][rows][3][d] dtype, or NULL: feature j of a row is written
 *              when feat_layers[j] lies in (layer_begin, layer_end].
 *  logits      [B][rows][vocab] float32, or NULL: written when layer_end ==
 *              n_layers; row i = target logits after node i (the
 *              target_logits of eagle3_verify).
 * 0 <= layer_begin <= layer_end <= n_layers; rows <= 64; ws of
 * eagle3_target_workspace_size bytes.  EAGLE3_EUNSUPPORTED: a shape the
 * drafter step rejects (head_dim, d > 8192, ...). */
int eagle3_target_forward(const eagle3_dims *dims, const eagle3_target *target, const eagle3_kv *kv, int B,
                          int rows, const int32_t *tokens, const int32_t *pos, const uint64_t *anc,
                          int layer_begin, int layer_end, float *hidden, void *feats, float *logits, void *ws,
                          size_t ws_bytes, eagle3_stream_t stream);

/* After verification: commit the root and the accepted nodes.  For request
 * b, n = accept_len[b] + 1 (clamped to 1..min(Dmax+1, rows)) verify rows --
 * row 0, then accepted[b][0..n-2] (eagle3_verify's outputs) -- move from
 * tree slots to committed rows ctx_len[b] .. ctx_len[b]+n-1 of every layer
 * (kv: HOST array [n_layers]; ctx_len is read from kv[0], and every layer
 * must share those lengths).  feats / feats_next (optional, dtype):
 * feats_next[b][j] ([B][Dmax+1][3][d]) = feats[b][row j] ([B][rows][3][d])
 * for j < n, the fusion input of the next cycle.  ctx_len_out [B]
 * (optional, may alias kv[0].ctx_len) = ctx_len + n; status [B] (optional)
 * = 0.  A request whose rows do not fit the smallest layer capacity gets
 * status EAGLE3_ECAPACITY and is left unchanged (ctx_len_out = ctx_len).
 * Paged caches need the blocks of the new rows in the block table (a
 * negative entry skips the row). */
int eagle3_kv_commit(const eagle3_dims *dims, int n_layers, const eagle3_kv *kv, int B, int rows,
                     const int32_t *accept_len, const int32_t *accepted, int Dmax, const void *feats,
                     void *feats_next, int32_t *ctx_len_out, int32_t *status, eagle3_stream_t stream);

/* The top-k/log-prob reduction of eagle3_draft_step on caller logits:
 * logits [rows][V] float32 -> ids [rows][k], lp [rows][k], lse [rows] (lse
 * may be NULL).  Same order and tie rule.  k in 1..16, V <= 262144 (also
 * the vocabulary limit of eagle3_draft_step). */
int eagle3_topk(const float *logits, int rows, int V, int k, int32_t *ids, float *lp, float *lse,
                void *ws, size_t ws_bytes, eagle3_stream_t stream);

/* ---- kernel timing (diagnostics) ---------------------------------------
 * Kernel classes of the draft/verify path.  When timing is enabled for a
 * class, every launch of that class records a HIP event pair on the stream
 * it is launched on; eagle3_timing_read synchronises on the last event and
 * returns the summed elapsed time and the number of launches recorded since
 * the class was enabled.  Event creation happens in eagle3_timing_enable
 * (host memory/handles only); recording adds two hipEventRecord calls per
 * launch.  Not thread safe; meant for benchmarks and profiling. */
#define EAGLE3_KC_FUSE 0
#define EAGLE3_KC_ROWOPS 1  /* prologue, RMSNorm and other row kernels (TTT: also the CE merge) */
#define EAGLE3_KC_QKV 2     /* QKV GEMM with RoPE / KV scatter        */
#define EAGLE3_KC_ATTN 3    /* attention partials + merge            */
#define EAGLE3_KC_O 4
#define EAGLE3_KC_GATEUP 5
#define EAGLE3_KC_DOWN 6
#define EAGLE3_KC_LMHEAD 7
#define EAGLE3_KC_TOPK 8
#define EAGLE3_KC_TREE 9
#define EAGLE3_KC_VERIFY 10
#define EAGLE3_KC_TTT_GEMM 11 /* TTT fusion, QKV, O, gate/up, down GEMMs  */
#define EAGLE3_KC_TTT_ATTN 12 /* TTT rollout-mask attention              */
#define EAGLE3_KC_TTT_CE 13   /* TTT LM-head GEMM with the CE epilogue    */
#define EAGLE3_KC_LR_SCORES 14 /* efficient head: the low-rank scores kernel (the rest of
                                  stage 1 stays in EAGLE3_KC_LMHEAD, stage 2 in _TOPK) */
#define EAGLE3_KC_TARGET 15     /* eagle3_target_forward, whole call          */
#define EAGLE3_KC_TGT_GATEUP 16 /* its gate/up GEMMs (principal kernel)       */
#define EAGLE3_KC_TGT_LMHEAD 17 /* its LM-head GEMM (principal kernel)        */
#define EAGLE3_KC_TTT_BWD_GEMM 18 /* TTT backward: data-gradient GEMMs (dy, dz, du, da, dx) */
#define EAGLE3_KC_TTT_BWD_ATTN 19 /* TTT backward: attention                              */
#define EAGLE3_KC_TTT_WGRAD 20    /* TTT backward: weight-gradient GEMMs                  */
#define EAGLE3_KC_TTT_BWD_ROWS 21 /* TTT backward: norm backward, transposes, reductions  */
#define EAGLE3_KC_COUNT 22

/* max_launches > 0 enables class `kc` with room for that many launches
 * (counters reset); 0 disables it and frees its events. */
int eagle3_timing_enable(int kc, int max_launches);
/* Total milliseconds and launch count recorded for class `kc`. */
int eagle3_timing_read(int kc, double *total_ms, int *launches);
/* mode 0 (default): an event pair around each launch scope of the class.
 * mode 1: only the class's principal kernel is timed, each launch recording
 * its own start and end (hipExtLaunchKernel events, the dispatch timestamps
 * a profiler reads): the LM-head GEMM for EAGLE3_KC_LMHEAD, the scores
 * kernel for EAGLE3_KC_LR_SCORES, the CE GEMM for EAGLE3_KC_TTT_CE, the
 * target's gate/up and LM-head GEMMs for EAGLE3_KC_TGT_GATEUP and
 * EAGLE3_KC_TGT_LMHEAD, the TTT backward's dy GEMM (dlogits . W_lm) for
 * EAGLE3_KC_TTT_BWD_GEMM and its weight-gradient GEMMs for
 * EAGLE3_KC_TTT_WGRAD; other classes then record nothing. */
int eagle3_timing_mode(int kc, int mode);

#ifdef __cplusplus
}
#endif
#endif /* EAGLE3_H */
