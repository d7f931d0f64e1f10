/*
 * spec_verify.h -- C ABI of libspecverify.so: the single-forward speculative
 * verification step of a block-diffusion language model on AMD Instinct
 * MI355X (gfx950).
 *
 * The step (one transformer attention layer's worth of it plus the
 * verification epilogue) as described on the page "SimSD: Simple Speculative
 * Decoding in Diffusion Language Models":
 *   - 关键设计 1: after the cached prompt come B data slots D_1..D_B (draft
 *     tokens) and B mask slots D~_1..D~_B; D~_k is the slot whose output
 *     verifies slot k.  Response rows are numbered r = 0..2B-1: r < B is
 *     D_{r+1}, r >= B is D~_{r-B+1}.
 *   - 关键设计 2: step labels tau(k) in 1..B (a permutation; the prompt has
 *     label 0) and the temporal-causal mask A_ij.
 *   - 关键设计 3: RoPE in which D~_k reuses the position of D_k; the prompt
 *     uses positions 0..P-1 and slot k uses P + k (0-based k).
 *   - 关键设计 4: acceptance alpha_r = min(1, p_theta/p_phi) in draft order,
 *     the longest accepted prefix, and a resample at the first rejection from
 *     the residual (P_target - P_draft)^+ (page "S2D2: Fast Decoding for
 *     Diffusion LLMs via Training-Free Self-Speculation", 方法步骤 (5)).
 * Around it: the same epilogue at a sampling temperature T; shared-noise and
 * greedy verification, the multi-copy attention and draft-tree verification
 * of "SPOT: Enhancing Speculative Decoding for Diffusion Language Models via
 * Commit-Order Prediction"; S2D2's verify-routing estimate; a paged prompt
 * cache with per-sequence lengths, the commit step and the cache append
 * (each call below cites its passage).
 *
 * Conventions shared by every call:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller,
 *     contiguous, row-major and 16-byte aligned.  The library allocates no
 *     memory, keeps no state between calls, never synchronises the device
 *     and is reentrant; scratch memory comes in through `workspace`.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *     the null stream).  A call returns once the work is enqueued.
 *   - Arguments are checked on the host before anything is enqueued; on any
 *     non-zero status nothing is enqueued and no output is touched.
 *     SV_E_LAUNCH reports a launch the runtime refused.
 *   - tau being a permutation of 1..block is a precondition (not checked on
 *     the device by the compute calls; spec_verify_check_tau validates it).
 *   - dtype SV_BF16: bfloat16 tensors, bf16 MFMA with fp32 accumulation.
 *     dtype SV_F32: float32 tensors and float32 arithmetic throughout.
 *   - Shape limits: 1 <= block <= 64, n_qh % n_kvh == 0, head_dim in
 *     {64, 128}, prefix_len >= 0, batch >= 1; the calls that stream a
 *     vocabulary (accept, accept_coupled, route, tree): 1 <= gamma <= block,
 *     1 <= vocab <= 2^21, batch * rows <= 2^26 and batch * rows * vocab <=
 *     2^40 (rows = block, or n_nodes for the tree); the workspace-size calls
 *     return 0 outside these limits.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_VERIFY_ABI_VERSION 5

/* Size of the static device scratch buffer of spec_verify_accept_noalloc. */
#define SPEC_VERIFY_SCRATCH_BYTES (4 << 20)

enum {
    SV_OK = 0,
    SV_E_NULL = -1,        /* a required pointer is NULL                  */
    SV_E_SHAPE = -2,       /* a size is out of range or inconsistent      */
    SV_E_UNSUPPORTED = -3, /* dtype / head_dim not provided by the library */
    SV_E_ALIGN = -4,       /* a tensor pointer is not 16-byte aligned     */
    SV_E_WORKSPACE = -5,   /* workspace missing or smaller than required  */
    SV_E_LAUNCH = -6,      /* the HIP runtime refused a kernel launch     */
    SV_E_INVALID_TAU = -7, /* validation only: tau not a permutation      */
    SV_E_SCRATCH = -8      /* sizes beyond the static scratch buffer      */
};

enum { SV_F32 = 0, SV_BF16 = 1 };

/* verify-routing estimators of spec_verify_route */
enum { SV_ROUTE_MARGIN = 0, SV_ROUTE_ENTROPY = 1 };

/* Returns SPEC_VERIFY_ABI_VERSION of the built library. */
int spec_verify_abi_version(void);

/* Static, never-NULL description of a status code. */
const char *spec_verify_status_string(int status);

/*
 * Copy-aligned RoPE (SimSD 关键设计 3) of the 2B response rows.
 *   q_in  [batch][2*block][n_qh][head_dim], k_in [batch][2*block][n_kvh][head_dim]
 *   q_out, k_out: same shapes; may equal q_in / k_in (in place).
 * Row r is rotated at position prefix_len + (r mod block), rotate-half pairs
 * (i, i + head_dim/2) turning by pos * theta^(-2i/head_dim); angles are
 * formed in float64.  theta > 0.
 */
int spec_verify_rope(const void *q_in, const void *k_in, void *q_out, void *k_out, int dtype,
                     int batch, int block, int n_qh, int n_kvh, int head_dim, int prefix_len,
                     double theta, void *stream);

/* Bytes of workspace spec_verify_attn needs for these sizes and dtype. */
size_t spec_verify_attn_workspace_size(int dtype, int batch, int block, int prefix_len, int n_qh,
                                       int n_kvh, int head_dim);

/*
 * Masked GQA attention of the 2B response rows over [prompt KV | D | D~]
 * (SimSD 关键设计 1-3).
 *   q      [batch][2*block][n_qh][head_dim]
 *   k_new, v_new [batch][2*block][n_kvh][head_dim]   (response keys/values)
 *   k_cache, v_cache [batch][n_kvh][prefix_len][head_dim] (prompt KV, keys
 *          already rotated at positions 0..prefix_len-1; may be NULL when
 *          prefix_len == 0).  Head-major, so that one (sequence, kv head)
 *          reads one contiguous stream; a caller that keeps its cache
 *          position-major ([prefix_len][n_kvh][head_dim]) must transpose it
 *          first, a copy of the whole cache (268 MB for 32 sequences of 2048
 *          rows, 8 kv heads, head_dim 128) that this call's time does not
 *          include -- or keep it in pages (spec_verify_attn_paged), which
 *          the append keeps up to date in place.
 *   tau    [batch][block] int32, step labels 1..block
 *   out    [batch][2*block][n_qh][head_dim] in dtype
 * rope_theta > 0: q and k_new are raw and are rotated on the fly with the
 * copy-aligned positions (as spec_verify_rope would); rope_theta <= 0: q and
 * k_new are taken as already rotated.  softmax_scale <= 0 means
 * 1/sqrt(head_dim).  Query head h reads kv head h / (n_qh / n_kvh).
 * Response row i sees key j iff j is a prompt key, or j is a response key
 * and the four-case mask admits it.
 */
int spec_verify_attn(const void *q, const void *k_new, const void *v_new, const void *k_cache,
                     const void *v_cache, const int32_t *tau, void *out, int dtype, int batch,
                     int block, int prefix_len, int n_qh, int n_kvh, int head_dim,
                     double rope_theta, float softmax_scale, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Bytes of workspace spec_verify_attn_copies needs for these sizes. */
size_t spec_verify_attn_copies_workspace_size(int dtype, int batch, int block, int n_copies, int prefix_len,
                                              int n_qh, int n_kvh, int head_dim);

/*
 * Multi-copy verification attention (page "SPOT: Enhancing Speculative
 * Decoding for Diffusion Language Models via Commit-Order Prediction",
 * 核心方法 第三步 and 方法步骤详情: the target runs one batched forward over the
 * root state and the draft states, (1+D)L positions, each state a copy of
 * the block; 前置知识 "块扩散语言模型": attention is bidirectional inside a
 * block and causal across blocks).
 *   q      [batch][n_copies*block][n_qh][head_dim], copy-major (row r belongs
 *          to copy r / block)
 *   k_new, v_new [batch][n_copies*block][n_kvh][head_dim]
 *   k_cache, v_cache [batch][n_kvh][prefix_len][head_dim] (prompt keys already
 *          rotated; may be NULL when prefix_len == 0)
 *   out    [batch][n_copies*block][n_qh][head_dim]
 * Row r of copy c sees every prompt key and the block keys of copy c only.
 * Rows and keys of every copy sit at positions prefix_len + (r mod block)
 * (all copies are the same block); rope_theta > 0 rotates q and k_new on the
 * fly as spec_verify_attn does, <= 0 takes them as rotated.  dtype SV_BF16
 * only (SV_E_UNSUPPORTED otherwise); 1 <= n_copies, n_copies * block <= 1024;
 * other limits and conventions as spec_verify_attn.
 */
int spec_verify_attn_copies(const void *q, const void *k_new, const void *v_new, const void *k_cache,
                            const void *v_cache, void *out, int dtype, int batch, int block, int n_copies,
                            int prefix_len, int n_qh, int n_kvh, int head_dim, double rope_theta,
                            float softmax_scale, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace spec_verify_attn_paged needs for these sizes. */
size_t spec_verify_attn_paged_workspace_size(int dtype, int batch, int block, int n_copies, int max_prefix,
                                             int n_qh, int n_kvh, int head_dim);

/*
 * Verification attention over a paged prompt cache with per-sequence prompt
 * lengths: spec_verify_attn (n_copies == 0, paired layout, tau required) or
 * spec_verify_attn_copies (n_copies >= 1, tau ignored) with the prompt K/V
 * read through a page table.  The pages say the prompt's K/V are cached
 * ("SimSD: Simple Speculative Decoding in Diffusion Language Models",
 * 损失函数 / 训练策略) and that finished blocks join that prefix (the
 * block-diffusion prior, "SPOT", 前置知识); the paging is a storage layout.
 *   k_pages, v_pages  with block_table: [n_pages][n_kvh][page_size][head_dim]
 *          bf16 (page_size a multiple of 64); prompt row j of sequence b is
 *          row j % page_size of page block_table[b * max_pages + j /
 *          page_size].  Without a table (block_table NULL): contiguous
 *          [batch][n_kvh][page_size][head_dim], page_size >= max_prefix the
 *          row stride (0 means max_prefix); max_pages, n_pages ignored.
 *   block_table [batch][max_pages] int32 page ids; ids outside [0, n_pages)
 *          are clamped into range (wrong rows, never an access outside the
 *          pages); max_pages * page_size >= max_prefix.
 *   prefix_lens [batch] int32 per-sequence prompt lengths, clamped to
 *          [0, max_prefix]; NULL: every sequence has max_prefix.  Each
 *          sequence's response rows sit at positions prefix_lens[b] + ...
 *   Other arguments, layouts and limits as spec_verify_attn /
 *   spec_verify_attn_copies (q, k_new, v_new, out row-major as there).
 * dtype SV_BF16 only.  SV_E_SHAPE for inconsistent page sizes.
 */
int spec_verify_attn_paged(const void *q, const void *k_new, const void *v_new, const void *k_pages,
                           const void *v_pages, const int32_t *block_table, const int32_t *prefix_lens,
                           const int32_t *tau, void *out, int dtype, int batch, int block, int n_copies,
                           int max_prefix, int page_size, int max_pages, int n_pages, int n_qh, int n_kvh,
                           int head_dim, double rope_theta, float softmax_scale, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Bytes of workspace spec_verify_tree needs for these sizes. */
size_t spec_verify_tree_workspace_size(int batch, int n_nodes, int64_t vocab);

/*
 * Verification of a draft tree ("SPOT: Enhancing Speculative Decoding for
 * Diffusion Language Models via Commit-Order Prediction", 核心方法, second
 * step: a tree of draft states, each child its parent plus one commit
 * (position, token); 方法步骤详情, 验证: one forward gives the target's own next
 * commit at the root and at every draft state, edges equal to it are
 * accepted, otherwise the target's own commit is made).  Per sequence,
 * nodes 0..n_nodes-1, node 0 the root state (its copy the root copy of
 * spec_verify_attn_copies):
 *   parent [batch][n_nodes]: node n's parent (node 0's is ignored);
 *   node_pos, node_tok [batch][n_nodes]: node n is its parent plus the
 *     commit of node_tok at position node_pos;
 *   target_pos [batch][n_nodes]: the position the target's own policy
 *     commits next at state n (the policy belongs to the model);
 *   target_logits, gumbel [batch][n_nodes][vocab] float32: the target's
 *     logits at that position in node n's copy, and the noise-table row of
 *     that position's absolute index (gumbel may be NULL when temperature
 *     == 0).
 * The target's own token at node n is argmax_v fmaf(l_v, 1/T, g_v) in
 * float32 (T == 0: argmax_v l_v), the smallest v among equal scores.  From
 * the root the walk moves to the child (smallest index if several) whose
 * commit equals the target's own commit at the current node.
 * Outputs: path_len [batch] = accepted edges L; path [batch][n_nodes] = the
 * nodes of the walk (root first), -1 after; commit_pos, commit_tok [batch] =
 * the target's own commit at the last node; target_tok [batch][n_nodes]
 * (optional) = the target's own token at every node.
 * 1 <= n_nodes <= 64, 1 <= vocab <= 2^21, temperature >= 0 finite.  A walk
 * has at most n_nodes - 1 edges, so a malformed parent array gives a wrong
 * path but the call still ends.
 */
int spec_verify_tree(const float *target_logits, const float *gumbel, const int32_t *parent, const int32_t *node_pos,
                     const int32_t *node_tok, const int32_t *target_pos, int batch, int n_nodes, int64_t vocab,
                     float temperature, int32_t *path_len, int32_t *path, int32_t *commit_pos, int32_t *commit_tok,
                     int32_t *target_tok, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace spec_verify_tree_states needs for these sizes (0 when
 * the sizes are out of range). */
size_t spec_verify_tree_states_workspace_size(int batch, int n_nodes, int block, int64_t vocab);

/*
 * Verification of a tree of block states, the target's own transition
 * computed from its logits ("SPOT: Enhancing Speculative Decoding for
 * Diffusion Language Models via Commit-Order Prediction": 前置知识
 * "块扩散语言模型", a decoding step commits the masked position of highest
 * confidence; 前置知识 "动态阈值解码", confidence c_s = max_v p_theta,s(v), every
 * masked position above a threshold committed, else the single highest;
 * 核心方法 third step and 方法步骤详情 验证, one forward over the root and all
 * draft copies gives the target's own next transition at every state, Phi_0
 * at T = 0 and Phi_G for the fixed noise table at T > 0, edges whose child
 * equals it are accepted, otherwise the target's own result is committed).
 * Per sequence, nodes 0..n_nodes-1, node 0 the root (the copies of
 * spec_verify_attn_copies):
 *   target_logits [batch][n_nodes][block][vocab] float32: the target's
 *     logits at every slot of every node's copy; rows of decided slots are
 *     never read.  -inf entries have probability 0.
 *   gumbel [batch][block][vocab] float32: the noise-table rows of the
 *     block's absolute positions, shared by every copy (NULL allowed when
 *     temperature == 0).
 *   parent [batch][n_nodes]: node n's parent, in [0, n) (node 0's is
 *     ignored; a node whose parent lies outside that range is never
 *     entered).
 *   state [batch][n_nodes][block]: each node's block, a token >= 0 at every
 *     decided slot, -1 where masked.
 *   threshold: the dynamic-threshold rule; any value >= 1 gives the
 *     one-commit decoder (no confidence exceeds 1).
 * At every node: c_s = 1 / sum_v exp(l_v - max l) per masked slot (the
 * untempered distribution at every temperature; normaliser in float64), the
 * commit set is every masked slot with c_s > threshold (compared in
 * float64), else the masked slot of highest c_s (the smallest slot among
 * equal values), and the token at a committed slot is argmax_v fmaf(l_v,
 * 1/T, g_v) in float32 (T == 0: argmax_v l_v), the smallest v among equal
 * scores.  From the root the walk moves to the child (smallest index if
 * several) whose state equals the current state with the current commit
 * applied; it stops at a node without masked slots or where no child
 * matches.
 * Outputs: path_len [batch] = accepted edges; path [batch][n_nodes] = the
 * nodes of the walk, root first, -1 after; next_state [batch][block] = the
 * last node's state with its commit applied (the block after this step);
 * commit [batch][n_nodes][block] (optional) = each node's commit, token or
 * -1; confidence [batch][n_nodes][block] float32 (optional) = c_s at masked
 * slots, -1 at decided ones.
 * 1 <= n_nodes <= 64, 1 <= block <= 64, 1 <= vocab <= 2^21, batch * n_nodes *
 * block <= 2^26 rows and rows * vocab <= 2^40, temperature >= 0 finite,
 * threshold not NaN; logits and gumbel 16-byte aligned.  Status: SV_E_SHAPE
 * for sizes out of range, a negative, NaN or infinite temperature (or one
 * whose 1/T overflows float32) or a NaN threshold; SV_E_NULL for a missing
 * input or output (gumbel is required when temperature > 0; commit and
 * confidence may be NULL); SV_E_ALIGN; SV_E_WORKSPACE when the workspace is
 * missing or smaller than spec_verify_tree_states_workspace_size (24 bytes
 * per (node, slot, vocabulary part), written before it is read within the
 * call's two launches).  A parent array that is not a tree gives a wrong path
 * but the call still ends (a walk has at most n_nodes - 1 edges).
 */
int spec_verify_tree_states(const float *target_logits, const float *gumbel, const int32_t *parent,
                            const int32_t *state, int batch, int n_nodes, int block, int64_t vocab, float temperature,
                            float threshold, int32_t *path_len, int32_t *path, int32_t *next_state, int32_t *commit,
                            float *confidence, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Validation of the step labels ("SimSD: Simple Speculative Decoding in
 * Diffusion Language Models", 关键设计 2: tau assigns each slot of the block
 * its draft step, a permutation of 1..block).  The other calls take this as
 * a precondition and do not check it on the device (an invalid tau gives
 * wrong results but no access outside the buffers).
 *   tau [batch][block] int32; bad [batch] int32 out: 0 when row b is a
 *   permutation of 1..block, else 1.  1 <= block <= 64.  The caller reads
 *   bad after the stream reaches this point (SV_E_INVALID_TAU names the
 *   condition for its own error handling).
 */
int spec_verify_check_tau(const int32_t *tau, int batch, int block, int32_t *bad, void *stream);

/*
 * Commit step after a verification round ("SimSD", 关键设计 4: the accepted
 * prefix is kept, the first rejected position is resampled in place; a block
 * with fewer undecoded positions than the draft length is finished by
 * ordinary target denoising).
 *   out_tokens   [batch][block] int32: spec_verify_accept's (or
 *                spec_verify_accept_coupled's) output, the committed token of
 *                each slot or -1.
 *   block_tokens [batch][block] int32, in/out: the block, -1 where masked;
 *                each committed token is written into its slot.
 *   remaining [batch]: masked slots left (R); state [batch]: 2 = the block is
 *   finished, 1 = 0 < R < gamma (finish by target denoising), 0 = keep
 *   speculating; n_append [batch]: block when finished, else 0 (the rows
 *   spec_verify_kv_append should add).
 * 1 <= gamma <= block <= 64.  Device pointers, caller-owned.
 */
int spec_verify_commit(const int32_t *out_tokens, int32_t *block_tokens, int batch, int block, int gamma,
                       int32_t *remaining, int32_t *state, int32_t *n_append, void *stream);

/*
 * Append rows to each sequence's prompt cache (the finished block joins the
 * cached prefix: "SPOT", 前置知识; "SimSD", 损失函数 / 训练策略).  Sequence b
 * appends rows 0 .. n_append[b]-1 of k_rows / v_rows [batch][src_stride]
 * [n_kvh][head_dim] bf16 at positions prefix_lens[b] + i, then
 * prefix_lens[b] += n_append[b].  With rope_theta > 0 each key is rotated at
 * its position first (the cache holds rotated keys; rotate-half pairs, as
 * spec_verify_rope), stored as bf16 rounded to nearest even.  Cache layout,
 * block_table and page_size as spec_verify_attn_paged (capacity max_pages *
 * page_size, or the row stride page_size without a table).
 *   status [batch] (optional): 0 appended (or nothing to append), 1 the rows
 *   would pass the capacity (nothing written, length unchanged), 2 n_append[b]
 *   outside [0, src_stride] (nothing written), 3 a block-table entry of a
 *   page the rows would land in lies outside [0, n_pages) (nothing written,
 *   length unchanged).
 * n_append and prefix_lens live on the device (n_append as spec_verify_commit
 * leaves it).  Pages shared by several sequences are the caller's to copy
 * before an append.  dtype SV_BF16, head_dim 64 or 128.
 */
int spec_verify_kv_append(const void *k_rows, const void *v_rows, int src_stride, const int32_t *n_append,
                          void *k_pages, void *v_pages, const int32_t *block_table, int32_t *prefix_lens,
                          int32_t *status, int dtype, int batch, int page_size, int max_pages, int n_pages,
                          int n_kvh, int head_dim, double rope_theta, void *stream);

/* Bytes of workspace spec_verify_accept needs for these sizes. */
size_t spec_verify_accept_workspace_size(int batch, int block, int gamma, int64_t vocab);

/*
 * Verification epilogue (SimSD 关键设计 4; S2D2 方法步骤 (5)).
 *   target_logits [batch][block][vocab] float32: target logits of each
 *                 slot's D~ row (slot order)
 *   draft_probs   [batch][block][vocab] float32: the draft distribution
 *                 p_phi of each slot
 *   draft_tokens  [batch][block] int32 in [0, vocab)
 *   tau           [batch][block] int32 step labels 1..block
 *   uniforms      [batch][gamma+1] float32 in [0,1): uniforms[r-1] tests
 *                 draft step r, uniforms[gamma] drives the resample
 * Draft step r = 1..gamma verifies the slot o_r with tau(o_r) = r:
 * p_theta = softmax(target_logits[o_r]) (normaliser accumulated in float64),
 * alpha_r = min(1, p_theta(x)/p_phi(x)) for x = draft_tokens[o_r] (alpha = 1
 * when p_phi(x) = 0); step r is accepted iff uniforms[r-1] < alpha_r.
 * Outputs:
 *   accept_len [batch]: L = number of leading accepted steps (0..gamma)
 *   out_tokens [batch][block]: the draft token for slots with tau <= L; for
 *     the slot with tau = L+1 (only when L < gamma) the resampled token: the
 *     smallest v whose running sum of r(v) = max(0, p_theta(v) - p_phi(v))
 *     in ascending token order exceeds uniforms[gamma] * sum_v r(v) (p_theta
 *     itself when that sum is zero); -1 for every other slot
 *   alpha [batch][gamma] float32 (may be NULL): alpha_r of every step, in
 *     draft order
 * Target logits may be -inf (masked or filtered vocabulary entries: they
 * get probability 0); each verified slot's row needs at least one finite
 * logit and no NaN or +inf -- a row without a finite logit has no target
 * distribution: its alpha is NaN, its step is rejected and the resampled
 * token is unspecified.
 */
int spec_verify_accept(const float *target_logits, const float *draft_probs,
                       const int32_t *draft_tokens, const int32_t *tau, const float *uniforms,
                       int batch, int block, int gamma, int64_t vocab, int32_t *accept_len,
                       int32_t *out_tokens, float *alpha, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * spec_verify_accept without a workspace, for callers that cannot allocate
 * device memory: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid allocation.  Arguments, outputs and results are
 * those of spec_verify_accept with the workspace dropped.  Its scratch is a
 * static device buffer of SPEC_VERIFY_SCRATCH_BYTES (4 MiB) inside the
 * library, one per GPU, held from the first call on that GPU until the
 * process ends; the call itself allocates nothing.  Sizes whose
 * spec_verify_accept_workspace_size exceeds SPEC_VERIFY_SCRATCH_BYTES
 * return SV_E_SCRATCH before anything is enqueued (32 sequences of 32 slots
 * over a 151936-token vocabulary need ~90 KB; 64 x 64 slots ~210 KB).
 * Every call on one GPU shares that GPU's buffer: two calls whose work
 * overlaps on one GPU (different streams without ordering, or different
 * threads) race and give wrong results; calls on one stream, or ordered by
 * events, are safe.  SV_E_LAUNCH if the buffer's device address cannot be
 * obtained.
 */
int spec_verify_accept_noalloc(const float *target_logits, const float *draft_probs,
                               const int32_t *draft_tokens, const int32_t *tau, const float *uniforms,
                               int batch, int block, int gamma, int64_t vocab, int32_t *accept_len,
                               int32_t *out_tokens, float *alpha, void *stream);

/*
 * The same verification epilogue when target and draft sample at temperature
 * T > 0 (speculative sampling with the min(1, q/p) acceptance: "S2D2",
 * 前置知识; the classic rejection-sampling verifier that "SPOT" (核心创新,
 * 新颖性) sets beside shared-noise verification at any temperature).  The
 * target distribution of a slot is p_theta = softmax(target_logits[k] * 1/T):
 * 1/T is rounded to float32 once and every product l * (1/T) is rounded to
 * float32 before use.  draft_probs is the drafter's distribution, already at
 * its own temperature.  Arguments, outputs, workspace
 * (spec_verify_accept_workspace_size) and errors as spec_verify_accept; a
 * temperature that is not finite and positive, or whose reciprocal overflows
 * float32, gives SV_E_SHAPE.  T = 1 gives exactly spec_verify_accept's
 * results.  (T = 0, greedy verification, is spec_verify_accept_coupled.)
 */
int spec_verify_accept_temperature(const float *target_logits, const float *draft_probs,
                                   const int32_t *draft_tokens, const int32_t *tau, const float *uniforms,
                                   int batch, int block, int gamma, int64_t vocab, float temperature,
                                   int32_t *accept_len, int32_t *out_tokens, float *alpha, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* Bytes of workspace spec_verify_accept_coupled needs for these sizes. */
size_t spec_verify_accept_coupled_workspace_size(int batch, int block, int gamma, int64_t vocab);

/*
 * Shared-noise (temperature > 0) or greedy (temperature == 0) verification
 * (page "SPOT: Enhancing Speculative Decoding for Diffusion Language Models
 * via Commit-Order Prediction", 前置知识 "Gumbel-Max 技巧与随机耦合" and
 * 核心创新 / 方法步骤详情: a Gumbel noise table indexed by absolute output
 * position is shared by draft and target; given the noise the target's
 * transition is deterministic, a step is accepted when the draft's state
 * equals the target's, otherwise the target's own result is committed).
 *   target_logits [batch][block][vocab] float32: target logits of each slot
 *   gumbel        [batch][block][vocab] float32: each slot's row of the
 *                 shared noise table (standard Gumbel noise at the slot's
 *                 absolute output position -- the noise the drafter sampled
 *                 with); not read, and may be NULL, when temperature == 0
 *   draft_tokens, tau [batch][block] int32 (tau: step labels 1..block)
 *   temperature   >= 0 and finite
 * The target's choice at a verified slot (tau <= gamma) is
 * argmax_v fmaf(l[v], 1/T, g[v]), computed in float32 with 1/T rounded to
 * float32 (T > 0), or argmax_v l[v] (T == 0); equal scores go to the smallest
 * v.  Draft step r = 1..gamma (the slot with tau = r) is accepted iff its
 * draft token equals that choice; L = number of leading accepted steps.
 * Outputs:
 *   accept_len [batch]: L (0..gamma)
 *   out_tokens [batch][block]: the draft token where tau <= L, the target's
 *     choice where tau == L+1 (only when L < gamma), -1 elsewhere
 *   target_tokens [batch][block] (may be NULL): the target's choice where
 *     tau <= gamma, -1 elsewhere
 * Logits and noise are finite (a precondition).  Limits as for
 * spec_verify_accept; SV_E_SHAPE for a negative or non-finite temperature,
 * SV_E_NULL for a NULL gumbel at temperature > 0.
 */
int spec_verify_accept_coupled(const float *target_logits, const float *gumbel,
                               const int32_t *draft_tokens, const int32_t *tau, int batch, int block,
                               int gamma, int64_t vocab, float temperature, int32_t *accept_len,
                               int32_t *out_tokens, int32_t *target_tokens, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Bytes of workspace spec_verify_route needs for these sizes. */
size_t spec_verify_route_workspace_size(int batch, int block, int gamma, int64_t vocab);

/*
 * Verify-routing estimator (page "S2D2: Fast Decoding for Diffusion LLMs via
 * Training-Free Self-Speculation", 方法步骤详情 (4): the expected accepted
 * prefix length K = sum_k prod_{i<=k} alpha_i decides whether verifying is
 * worth a forward; alpha_i is estimated from the draft distribution by its
 * margin or its entropy).
 *   draft_probs [batch][block][vocab] float32: the draft distribution of each
 *               slot (entries >= 0)
 *   tau         [batch][block] int32 step labels 1..block
 *   estimator   SV_ROUTE_MARGIN: alpha = 1 if p_(1) - p_(2) >= param (the two
 *               largest entries, difference exact in float64), else 0;
 *               SV_ROUTE_ENTROPY: alpha = exp(-param * H / ln vocab) with
 *               H = -sum_v p_v ln p_v (0 when vocab == 1; entries below the
 *               smallest normal float count as 0)
 *   param       the margin threshold or beta; finite
 * Steps are taken in draft order r = 1..gamma (the slot with tau = r):
 *   khat [batch] float32: sum_{k=1}^{gamma} prod_{r=1}^{k} alpha_r
 *   alpha_hat [batch][gamma] float32 (may be NULL): alpha_r in draft order
 * Limits as for spec_verify_accept; SV_E_UNSUPPORTED for an unknown
 * estimator, SV_E_SHAPE for a non-finite param.
 */
int spec_verify_route(const float *draft_probs, const int32_t *tau, int batch, int block, int gamma,
                      int64_t vocab, int estimator, double param, float *khat, float *alpha_hat,
                      void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
