/*
 * nsa.h -- C ABI of the MI355X (gfx950) Native Sparse Attention forward.
 *
 * The operation (sources cited by page and section):
 *   [P1] "Zhang Xiaojun Business Interviews #94" transcript (bidclub.ai),
 *        s4 "Inside Native Sparse Attention", s5 "Hardware Makes Sparsity
 *        Work", s6 "Why Sparse Attention Wins", s7 "Kimi Simplifies The
 *        Sparse Route";
 *   [P5] LateTalk #103 notes (zjai.club), close reading s12-s13.
 *
 * For every query token and head the output is a gated sum of three
 * attention branches over the causal past ([P1] s4):
 *   - compressed: softmax attention over one mean summary per complete KV
 *     block (summaries of blocks that end after the query are masked);
 *   - selected:   one softmax over all tokens (up to the query) of the
 *     top_k blocks chosen for the token's KV group -- the group's heads add
 *     up their compressed-branch probabilities so that they all pick the
 *     same blocks;
 *   - window:     softmax over the last `window` positions.
 * MoBA ([P1] s7, [P5] s13) is the special case of one head per KV group,
 * block means as block keys, the current block always chosen, and the
 * selected branch alone.  Decoding ([P1] s6) is q_len = 1 with a long cache.
 *
 * Conventions shared by every call
 *   Positions: the q_len queries sit at absolute positions
 *     kv_len - q_len .. kv_len - 1 of their sequence (prefill: q_len == kv_len).
 *   Heads: H = n_kv_groups * heads_per_group; head h uses KV group
 *     h / heads_per_group.
 *   Layouts (row-major, last dimension contiguous, every base pointer
 *   16-byte aligned, all device memory unless stated):
 *     q      [B, q_len, H, d_qk]          k     [B, kv_len, G, d_qk]
 *     v      [B, kv_len, G, d_v]          gates [B, q_len, H, 3] (cmp, slc, win)
 *     k_cmp  [B, nb, G, d_qk]             v_cmp [B, nb, G, d_v]   nb = kv_len / block
 *            (when nb == 0 there is nothing to hold and k_cmp / v_cmp may be NULL)
 *     idx    int32 [B, q_len, G, top_k]   ascending block ids, padded with -1
 *     out    [B, q_len, H, d_v]
 *   Element type: dtype (NSA_BF16 or NSA_F32) for q, k, v, gates, k_cmp,
 *     v_cmp and out (out is fp32 when NSA_F_OUT_F32 is set).  Arithmetic is
 *     fp32 (bf16 inputs feed bf16 matrix cores with fp32 accumulation).
 *   Ownership: the caller allocates and owns every buffer, including the
 *     workspace (size from nsa_workspace_bytes).  The library allocates and
 *     frees nothing, keeps no pointer after a call returns, and never
 *     synchronises: work is queued on `stream` (a hipStream_t; NULL = the
 *     default stream) and results are ready when that stream reaches them.
 *   Errors: arguments are validated before anything is queued; on any error
 *     nothing is launched and no output is written.  NSA_ERR_HIP reports a
 *     failed launch (hipGetLastError), in which case outputs are undefined.
 *   Thread safety: calls hold no global state (apart from the fixed scratch
 *     of nsa_forward_noalloc) and may come from several threads; calls
 *     sharing a workspace must be ordered on one stream.
 */
#ifndef NSA_H
#define NSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NSA_OK = 0,
  NSA_ERR_INVALID_ARG = 1,  /* NULL/misaligned pointer, inconsistent sizes or flags */
  NSA_ERR_UNSUPPORTED = 2,  /* valid but outside what the kernels handle (limits below) */
  NSA_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than nsa_workspace_bytes */
  NSA_ERR_HIP = 4           /* a kernel launch failed */
} nsa_status;

enum { NSA_BF16 = 0, NSA_F32 = 1 };

enum {
  NSA_F_FORCE_FIRST = 1u,    /* block 0 is always chosen (attention-sink rationale, [P1] s4) */
  NSA_F_FORCE_CURRENT = 2u,  /* the query's own block is always chosen ([P5] s13) */
  NSA_F_CMP = 4u,            /* compressed branch enters the output */
  NSA_F_SLC = 8u,            /* selected branch enters the output */
  NSA_F_WIN = 16u,           /* window branch enters the output */
  NSA_F_GATE_LOGITS = 32u,   /* gates hold logits; the kernel applies a sigmoid */
  NSA_F_OUT_F32 = 64u        /* out is fp32 whatever dtype is */
};

/*
 * Problem description.  Limits (NSA_ERR_UNSUPPORTED outside them):
 *   1 <= heads_per_group <= 16; 1 <= d_qk, d_v <= 256; 1 <= block <= 4096;
 *   top_k <= 64 and top_k * block <= 16384; window <= 16384;
 *   nb = kv_len / block <= 16384.
 * Invalid (NSA_ERR_INVALID_ARG): batch, q_len, n_kv_groups < 1;
 *   kv_len < q_len; top_k smaller than the number of forced blocks;
 *   window < 0; scale < 0; dtype unknown; flags outside NSA_F_*.
 */
typedef struct {
  int32_t batch, q_len, kv_len;
  int32_t n_kv_groups, heads_per_group;
  int32_t d_qk, d_v;
  int32_t block, top_k, window;
  uint32_t flags;          /* NSA_F_* */
  int32_t dtype;           /* NSA_BF16 or NSA_F32 */
  float scale;             /* softmax scale; 0 means 1/sqrt(d_qk) */
  const void* k_cmp;       /* nsa_forward: precomputed block summaries (e.g. a  */
  const void* v_cmp;       /* decode cache) or NULL to compute them in workspace */
  void* workspace;         /* device scratch owned by the caller */
  size_t workspace_bytes;
  void* stream;            /* hipStream_t */
  /* Optional timing hook (NULL = none): n_phase_events hipEvent_t handles
   * owned by the caller.  nsa_forward records phase_events[0] on `stream`
   * before its first kernel and phase_events[i + 1] after its i-th kernel
   * (as far as events are given); nsa_forward_phases names the kernels.
   * nsa_backward does the same per kernel group (nsa_backward_phases). */
  void* const* phase_events;
  int32_t n_phase_events;
  /* Selection block size in tokens (0 means `block`): a multiple of
   * `block`.  Selection works on blocks of sel_block tokens, each the run
   * of sel_block / block whole compression blocks it covers; its importance
   * is the sum of theirs ([P1] s4 notes the two sizes may differ and leaves
   * the mechanism open; this is the reading taken).  idx values count
   * selection blocks. */
  int32_t sel_block;
} nsa_params;

/*
 * Block compression ([P1] s4, s7): k_cmp[b, j, g, :] is the mean of the
 * `block` keys of block j (j < nb), v_cmp likewise.  The sum is taken in
 * fp64 in token order, divided by `block` and rounded once (to nearest,
 * ties to even) to dtype, so results are reproducible bit for bit.
 * Reads k, v; writes k_cmp, v_cmp.  Uses no workspace.
 */
nsa_status nsa_compress(const void* k, const void* v, void* k_cmp, void* v_cmp,
                        const nsa_params* params);

/*
 * Learned block compression ([P1] s4: each block is compressed into one
 * learned representation; [P1] s7: NSA forms it with an MLP where MoBA takes
 * the mean).  For every complete block j and group g, with X the block's
 * `block` keys flattened in token order (vec(X)[i * d + c] = k[b, j*block + i,
 * g, c]):  k_cmp[b, j, g, :] = W2 relu(W1 vec(X) + b1) + b2, and v_cmp
 * likewise with the value weights.  One MLP for keys and one for values,
 * shared by every block and group; flattening in order gives each position
 * in the block its own weights.  Weights and biases are dtype, row-major,
 * output features first:
 *   w1 [d_hidden, block * d]   b1 [d_hidden] or NULL
 *   w2 [d, d_hidden]           b2 [d] or NULL      (d = d_qk for keys, d_v for values)
 * Arithmetic: fp32 accumulation on bf16 matrix cores; the hidden layer is
 * rounded to bf16 after the ReLU, the summaries once to dtype.  The result
 * can be handed to nsa_forward through params->k_cmp / v_cmp.
 * Limits (NSA_ERR_UNSUPPORTED otherwise): dtype NSA_BF16; d_qk, d_v and
 * d_hidden in {64, 128, 192, 256}; block a multiple of 4.  No workspace.
 */
typedef struct {
  int32_t d_hidden;
  const void* k_w1;
  const void* k_b1;
  const void* k_w2;
  const void* k_b2;
  const void* v_w1;
  const void* v_b1;
  const void* v_w2;
  const void* v_b2;
} nsa_mlp_weights;

nsa_status nsa_compress_mlp(const void* k, const void* v, const nsa_mlp_weights* weights, void* k_cmp,
                            void* v_cmp, const nsa_params* params);

/*
 * Gate projection ([P1] s4: each branch's weight is learned from the token's
 * input representation through a projection):
 *   gates[b, t, h, branch] = sigmoid(x[b, t, :] . w[3 h + branch, :] + bias[3 h + branch])
 * x [B, q_len, d_model], w [3 H, d_model], bias [3 H] or NULL, gates
 * [B, q_len, H, 3], all dtype.  With NSA_F_GATE_LOGITS in params->flags the
 * sigmoid is left out (the attention then applies it).  fp32 accumulation on
 * bf16 matrix cores, one rounding to dtype.
 * Limits (NSA_ERR_UNSUPPORTED otherwise): dtype NSA_BF16, d_model a positive
 * multiple of 32.  No workspace.
 */
nsa_status nsa_gate_proj(const void* x, int32_t d_model, const void* w, const void* bias, void* gates,
                         const nsa_params* params);

/*
 * Block selection ([P1] s4 compressed branch + group-summed importance;
 * [P1] s7 and [P5] s13 for MoBA).  For query token t at position p and
 * group g: each head's softmax over the summaries of the complete blocks
 * j with (j + 1) * block <= p + 1, added up over the group's heads, is the
 * importance of summary j; a selection block (sel_block tokens, = block by
 * default) has the summed importance of the summaries it covers and is a
 * candidate once complete.  Forced blocks (flags: selection block 0, the
 * query's own selection block) come first; the remaining top_k slots take
 * the candidates with the highest importance (ties to the lower block id).
 * idx[b, t, g, :] lists the chosen selection blocks ascending, padded with
 * -1.  score_or_null (fp32, same shape) receives each listed block's
 * importance, +inf for forced blocks and -inf for padding.
 * Reads q and k_cmp (params->k_cmp is ignored here); may use the workspace.
 */
nsa_status nsa_select_topk(const void* q, const void* k_cmp, int32_t* idx,
                           float* score_or_null, const nsa_params* params);

/*
 * Selected branch alone ([P1] s4, s5): for each token and head, one softmax
 * over every position s <= p of the selection blocks listed in idx
 * (sel_block tokens each; entries < 0 are skipped; entries must be distinct
 * and begin at or before p), written to
 * out (no gate).  lse_or_null (fp32 [B, q_len, H]) receives the natural-log
 * sum of the exponentiated scaled logits (-inf for an empty set, whose
 * output is 0).  May use the workspace.
 */
nsa_status nsa_sparse_attn(const void* q, const void* k, const void* v, const int32_t* idx,
                           void* out, float* lse_or_null, const nsa_params* params);

/*
 * The whole forward ([P1] s4): summaries (taken from params->k_cmp/v_cmp
 * when both are given, else computed into the workspace), selection, the
 * branches enabled by flags, and out = sum over enabled branches of
 * gate * branch output.  gates may be NULL only when exactly one branch is
 * enabled (its weight is then 1).  Needs the workspace.
 */
nsa_status nsa_forward(const void* q, const void* k, const void* v, const void* gates,
                       const nsa_params* params, void* out);

/* Bytes of the fixed device scratch that nsa_forward_noalloc works in. */
#define NSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * nsa_forward without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same operation, arguments, limits and results as
 * nsa_forward, except that params->workspace and workspace_bytes are ignored:
 * the scratch is one fixed array of NSA_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends (its device
 * address is looked up once per device, on the first call there).  The call
 * allocates and frees nothing.
 *   Limit: a call whose workspace (nsa_workspace_bytes) exceeds
 *   NSA_NOALLOC_SCRATCH_BYTES returns NSA_ERR_WORKSPACE before anything is
 *   queued.  Decoding steps over a caller-held summary cache
 *   (params->k_cmp / v_cmp) fit, e.g. 64 sequences x 64k tokens; a 64k prefill
 *   does not.
 *   Sharing: every call on one GPU uses that GPU's one array, which keeps
 *   whatever the last call left (no result depends on its prior contents).
 *   Calls that may overlap in time on one GPU (other streams, other threads)
 *   race on it and must be ordered by the caller.
 *   NSA_ERR_HIP also when the scratch's device address cannot be obtained.
 */
nsa_status nsa_forward_noalloc(const void* q, const void* k, const void* v, const void* gates,
                               const nsa_params* params, void* out);

/*
 * Training forward: nsa_forward (summaries mean-pooled in the workspace)
 * that also hands back what its backward needs, so nsa_backward need not
 * recompute it ([P1] s6: NSA trains end to end, so every forward in
 * training is followed by a backward over the same selection).
 *   out    as nsa_forward.
 *   idx    int32 [B, q_len, G, top_k]: the selection (as nsa_select_topk).
 *   saved  nsa_train_saved_bytes(params) bytes, owned by the caller, to be
 *          passed to nsa_backward with the same q, k, v, gates and idx:
 *          fp32 [3][B, q_len, H] per branch (compressed, selected, window)
 *          the natural log-sum-exp of the scaled logits over the branch's
 *          key set (-inf when the set is empty or the branch off), then at
 *          the next 256-byte boundary bf16 [3][B, q_len, H, d_v] the
 *          branch's normalised output O_b (zeros when empty or off).
 * params->k_cmp / v_cmp must be NULL.  Limits (NSA_ERR_UNSUPPORTED
 * otherwise): those of nsa_backward, and q_len > 8 (shorter calls take the
 * decoding path, which keeps no statistics).  Needs the workspace of
 * nsa_forward.
 */
nsa_status nsa_forward_train(const void* q, const void* k, const void* v, const void* gates,
                             const nsa_params* params, void* out, int32_t* idx, void* saved);

/* Bytes of nsa_forward_train's saved statistics (0 if the params are invalid
 * or outside its limits). */
size_t nsa_train_saved_bytes(const nsa_params* params);

/*
 * Backward of nsa_forward ([P1] s4 the gated three-branch sum; [P1] s6: NSA
 * trains end to end, the top-k choice passes no gradient, and the compressed
 * branch's output carries a training signal to every block).  Given the
 * upstream gradient dout [B, q_len, H, d_v] (dtype) and the selection idx
 * the forward used (nsa_select_topk's output for the same inputs; any
 * selection of distinct blocks that begin at or before each query is
 * accepted), writes the fp32 gradients
 *   dq      [B, q_len, H, d_qk]
 *   dk      [B, kv_len, G, d_qk]   dv [B, kv_len, G, d_v]
 *           (the compressed branch's summary gradient reaches every token of
 *           its block divided by `block`: the mean's derivative; the rounding
 *           of the stored summaries is passed through unchanged)
 *   dgates  [B, q_len, H, 3] or NULL: the gradient with respect to the
 *           gates as given (logits when NSA_F_GATE_LOGITS is set); 0 for a
 *           branch that is off.  Must be NULL when gates is NULL.
 * Per branch b with key set S, P = softmax(scale q.k), O_b = sum P v and
 * gate g_b: dg_b = <dout, O_b>, dS = g_b P (<dout, v> - dg_b),
 * dq += scale sum dS k, dk += scale dS q, dv += g_b P dout.
 * The summaries are recomputed (params->k_cmp / v_cmp are ignored).
 * saved_or_null: nsa_forward_train's statistics for these inputs and idx;
 * the per-branch log-sum-exp and <dout, O_b> are then read from it (the
 * latter from the bf16 O_b) instead of being recomputed from q, k and v.
 * NULL: all of it is recomputed.
 * Results are deterministic (no floating-point atomics).
 * Limits (NSA_ERR_UNSUPPORTED otherwise): dtype NSA_BF16, heads_per_group
 * 16, block 64 with sel_block 0 or 64, d_qk in {64, 128, 192}, d_v in
 * {64, 128}, top_k <= 32; with saved statistics also q_len > 8.  Needs
 * nsa_backward_workspace_bytes of workspace.
 */
nsa_status nsa_backward(const void* q, const void* k, const void* v, const void* gates,
                        const int32_t* idx, const void* dout, const void* saved_or_null, float* dq,
                        float* dk, float* dv, float* dgates, const nsa_params* params);

/* Workspace bytes nsa_backward needs for these params (0 if they are invalid
 * or outside its limits). */
size_t nsa_backward_workspace_bytes(const nsa_params* params);

/* Number of kernel groups nsa_backward times through params->phase_events
 * (0 if the params are invalid or outside its limits); names[i]
 * (i < max_names) receives a static name of group i.  nsa_backward records
 * phase_events[0] before its first kernel and phase_events[i + 1] after
 * group i, as far as events are given.  With saved statistics the group
 * "bwd_kv_selected_stats" launches nothing. */
int32_t nsa_backward_phases(const nsa_params* params, const char** names, int32_t max_names);

/* Number of kernels nsa_forward launches for these params (0 if they are
 * invalid); names[i] (i < max_names) receives a static name of kernel i. */
int32_t nsa_forward_phases(const nsa_params* params, const char** names, int32_t max_names);

/* Workspace bytes that any call above needs for these params (0 if none). */
size_t nsa_workspace_bytes(const nsa_params* params);

/* Static description of a status code; any int is accepted, values that
 * are not an nsa_status give "unknown status". */
const char* nsa_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* NSA_H */
