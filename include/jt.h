/*
 * jt.h -- C ABI of libjt: one draft-and-verify step over a candidate token tree
 * on an AMD Instinct MI355X (gfx950).
 *
 * The step (JetSpec causal parallel tree drafting):
 *   1. jt_build_tree_mask  parent indices -> per-node 256-bit ancestor rows + depths
 *   2. jt_tree_attention   all B tree nodes attend, in one pass, to the prefix KV and
 *                          to the tree KV under the tree-causal mask
 *   3. jt_topw_per_depth   top-W token ids and log-probs of each draft logit row
 *   4. jt_verify_greedy    longest root path whose tokens equal the target argmax at
 *                          their parent, plus the bonus token
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The library never
 *     allocates, frees or keeps any of them after the call returns.
 *   - Scratch memory is passed in as `workspace` after a *_workspace_size() query; a
 *     NULL workspace is allowed only when the query returns 0.  Its contents need no
 *     initialisation and are meaningless after the call.  Calls that overlap in time
 *     need distinct workspaces.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are asynchronous and
 *     stream-ordered; outputs are valid once the stream reaches them.  No call
 *     synchronises the host.  The library holds no state: concurrent calls on
 *     different streams with disjoint outputs and workspaces are safe.
 *   - Shape, dtype, NULL-pointer, alignment and workspace problems are detected on the
 *     host and returned synchronously before anything is launched.  A failed launch
 *     returns JT_ERR_LAUNCH.  No C++ exception crosses this boundary.
 *   - Data-dependent faults are only visible on the device.  Entry points that take an
 *     `err` array (int32 [S], may be NULL) OVERWRITE err[s] with the OR of the JT_DEV_*
 *     flags found for sequence s (0 when clean).  Outputs of a flagged sequence are
 *     unspecified but every memory access stays in bounds.
 *   - Tensors are dense row-major (C order) unless a stride argument says otherwise.
 *   - bf16 = bfloat16 (1 sign, 8 exponent, 7 mantissa bits); JT_F32 = IEEE binary32.
 */
#ifndef JT_H
#define JT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define JT_ABI_VERSION 2

typedef enum {
    JT_OK = 0,
    JT_ERR_NULL = 1,      /* a required pointer is NULL */
    JT_ERR_SHAPE = 2,     /* a size is out of the supported range (see each call) */
    JT_ERR_DTYPE = 3,     /* unsupported element type for this call */
    JT_ERR_WORKSPACE = 4, /* workspace smaller than the *_workspace_size() answer */
    JT_ERR_LAUNCH = 5,    /* the HIP runtime rejected a kernel launch */
    JT_ERR_ALIGN = 6,     /* a pointer or stride breaks the stated alignment */
    JT_ERR_SCRATCH = 7    /* the shape needs more scratch than the static buffer of
                             jt_draft_verify_step_noalloc holds */
} jt_status;

typedef enum { JT_F32 = 0, JT_BF16 = 1 } jt_dtype;

/* device-side per-sequence flags written to err[s] */
enum {
    JT_DEV_BAD_PARENT = 1,  /* parent[s,0] != -1 or parent[s,i] not in [0, i) */
    JT_DEV_DEPTH_GT_N = 2,  /* some node is deeper than N (commit: accept_len not in [0, N]) */
    JT_DEV_BAD_BLOCK = 4,   /* a block-table entry needed by the prefix is outside the pool */
    JT_DEV_NAN = 8,         /* a target logit row holds a NaN */
    JT_DEV_BAD_PREFIX = 16  /* prefix_len[s] outside [0, max_prefix] (it is clamped; commit:
                               the path would not fit the cache) */
};

#define JT_MAX_NODES 256 /* B limit: one 256-bit ancestor row per node */
#define JT_MAX_W 16

int jt_abi_version(void);
const char *jt_status_string(int status);

/*
 * Step 1 -- tree-causal mask from parent indices.
 * Defines M[v,u] = 0 iff u is an ancestor of v or v itself, -inf otherwise (JetSpec
 * review on startedourmission.github.io, "How it works", mask equation); the verifier
 * consumes parent indices, depths and this mask without a dense per-request matrix
 * (paperlayer.ai JetSpec summary, appendix E "Verification").
 *
 *   parent  int32 [S,B]     parent[s,0] = -1 (node 0 is the root, the last committed
 *                           token); 0 <= parent[s,i] < i for i >= 1.
 *   anc     uint64 [S,B,4]  out: bit u of row (s,v) -- word u>>6, bit u&63 -- is set
 *                           iff u is an ancestor of v or u == v.  Bits >= B are 0.
 *   depth   int32 [S,B]     out: parent steps from v to the root (root 0).
 *   err     int32 [S]       out (optional): JT_DEV_BAD_PARENT; such a sequence gets
 *                           anc = 0 and depth = -1.
 * Supported: S >= 0, 1 <= B <= 256.  One workgroup per sequence.
 */
jt_status jt_build_tree_mask(const int32_t *parent, int32_t S, int32_t B, uint64_t *anc,
                             int32_t *depth, int32_t *err, void *stream);

/*
 * Step 2 -- tree-causal GQA attention, all nodes in one pass.
 * For sequence s, node v and query head h (KV head g = h / (Hq/Hkv)):
 *   out[s,v,h] = softmax_j(scale * <q[s,v,h], k_j>) . v_j over j = every prefix key of s
 *                and every tree node u with bit u set in anc[s,v];
 * i.e. a node sees the prefix, its ancestors and itself, never siblings or descendants
 * (startedourmission.github.io review, mask equation; paperlayer.ai JetSpec summary,
 * section 2 "Architecture" and appendix E "Verification").  Tree keys come after the
 * prefix.  q and k are post-RoPE: position prefix_len[s] + depth[s,v] is the caller's.
 *
 *   q                 [S,B,Hq,d]      dtype
 *   k_tree, v_tree    [S,B,Hkv,d]     dtype
 *   k_prefix,v_prefix block_table == NULL: contiguous [S,max_prefix,Hkv,d];
 *                     otherwise a pool [num_blocks,block_size,Hkv,d] in which logical
 *                     key j of sequence s is slot j % block_size of block
 *                     block_table[s*max_blocks_per_seq + j/block_size].
 *   block_table       int32 [S,max_blocks_per_seq] or NULL; entries past the prefix
 *                     are never read.
 *   prefix_len        int32 [S] device; keys j >= prefix_len[s] are never read.
 *   anc               uint64 [S,B,4] as written by jt_build_tree_mask.
 *   scale             <= 0 selects 1/sqrt(d).
 *   out               [S,B,Hq,d] dtype.
 *   lse               float [S,B,Hq] (optional): natural-log sum of exp of the scaled
 *                     visible scores.
 *   err               int32 [S] (optional): JT_DEV_BAD_PREFIX, JT_DEV_BAD_BLOCK (the
 *                     flagged sequence's output is unspecified; nothing outside the
 *                     pool is read).
 * Supported: d in {64,128}; Hq % Hkv == 0 and 1 <= Hq/Hkv <= 8; 1 <= B <= 256;
 * block_size a power of two; dtype JT_BF16 or JT_F32; q/k/v/out 16-byte aligned.
 * bf16 runs on MFMA (fp32 accumulate, bf16 out); fp32 runs on the vector ALU.
 */
/* block_size: the paged pool's block size, or 0 for a contiguous prefix.  The workspace
 * holds split-KV partial rows (and, for several sequences with more than 128 query rows
 * per KV head, where every workgroup takes an equal share of all sequences' key tiles,
 * each unit's first and last share); its contents need no initialisation.  Calls that
 * overlap on one workspace race. */
size_t jt_tree_attention_workspace_size(int32_t S, int32_t B, int32_t Hq, int32_t Hkv,
                                        int32_t d, int32_t max_prefix, int32_t block_size,
                                        jt_dtype dtype);
jt_status jt_tree_attention(const void *q, const void *k_tree, const void *v_tree,
                            const void *k_prefix, const void *v_prefix,
                            const int32_t *block_table, int32_t max_blocks_per_seq,
                            int32_t block_size, int32_t num_blocks,
                            const int32_t *prefix_len, int32_t max_prefix, const uint64_t *anc,
                            int32_t S, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                            jt_dtype dtype, float scale, void *out, float *lse, int32_t *err,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Step 3 -- per-depth top-W with log-probabilities.
 * The proposer extracts the top-k tokens and their log-probabilities at each future
 * position (paperlayer.ai JetSpec summary, appendix E "Drafting"), W candidates per
 * depth (paper.rainbus.top summary, method steps).  Row r of the draft logits gives the
 * candidates of depth r+1 (per sequence: rows s*N .. s*N+N-1).
 *
 *   logits    [rows, row_stride] dtype; the first V entries of a row are the vocabulary.
 *   ids       int32 [rows,W] out: token ids, logit descending, id ascending on ties
 *             (-0 == +0; NaN ranks below -inf).
 *   logprob   float [rows,W] out: logit - row_lse.
 *   row_lse   float [rows] (optional) out: log sum_t exp(logit_t) over the whole row
 *             (NaN if the row holds a NaN, -inf if every entry is -inf).
 *   row_entropy float [rows] (optional) out: the entropy -sum_t p_t log p_t of the row's
 *             softmax, computed in the same pass (the per-depth entropy that
 *             entropy-guided and hybrid tree scoring rank by: paperlayer.ai JetSpec
 *             summary, appendices C and E); NaN for a row holding a NaN, 0 for a row of
 *             -inf.  Leaving it NULL skips the extra sums.
 * Supported: rows >= 0, 1 <= W <= min(16, V), V < 2^31, row_stride >= V.
 */
size_t jt_topw_workspace_size(int32_t rows, int32_t V, int32_t W, jt_dtype dtype);
jt_status jt_topw_per_depth(const void *logits, int64_t row_stride, int32_t rows, int32_t V,
                            int32_t W, jt_dtype dtype, int32_t *ids, float *logprob,
                            float *row_lse, float *row_entropy, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * Step 4 -- greedy tree verification.
 * The verifier accepts the longest prefix whose draft tokens pass the acceptance test
 * and commits it plus one bonus token (paperlayer.ai JetSpec summary, section 2;
 * JetSpec++ summary, section 3).  At temperature 0 the test min(1, p/q)
 * (startedourmission.github.io review, inference) with a point-mass draft
 * (paperlayer.ai JetSpec++ summary, appendix F.3) is "token == target argmax at the
 * parent":
 *   am[s,v]       = argmax_t target_logits[s,v,t], lowest id on ties, NaN skipped;
 *   v accepted    iff tokens[s,u] == am[s,parent[s,u]] for every non-root u on the
 *                 root path of v (the root is always accepted);
 *   v*            = the deepest accepted node, lowest index on ties.
 *
 *   target_logits [S*B, row_stride] dtype (row s*B+v belongs to node v of sequence s).
 *   parent, tokens int32 [S,B]; tokens[s,0] is never checked.
 *   anc, depth    as written by jt_build_tree_mask for the same parent array.
 *   accept_len    int32 [S] out: depth(v*) = number of accepted draft tokens.
 *   accept_path   int32 [S,N+1] out: root .. v*, then -1.
 *   bonus         int32 [S] out: am[s,v*].
 *   argmax_out    int32 [S,B] (optional) out: am.
 *   err           int32 [S] (optional): JT_DEV_BAD_PARENT, JT_DEV_DEPTH_GT_N,
 *                 JT_DEV_NAN.  A bad-parent or too-deep sequence gets accept_len 0,
 *                 path [0,-1,...] and bonus am[s,0].
 * Supported: 1 <= B <= 256, 0 <= N <= 255, V < 2^31, row_stride >= V.
 */
size_t jt_verify_workspace_size(int32_t S, int32_t B, int32_t V, jt_dtype dtype);
jt_status jt_verify_greedy(const void *target_logits, int64_t row_stride, int32_t V,
                           jt_dtype dtype, const int32_t *parent, const int32_t *tokens,
                           const uint64_t *anc, const int32_t *depth, int32_t S, int32_t B,
                           int32_t N, int32_t *accept_len, int32_t *accept_path,
                           int32_t *bonus, int32_t *argmax_out, int32_t *err,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * The whole step in one call -- steps 3, 1, 2 and 4 with the arguments and outputs
 * documented above, in two kernel launches instead of seven: the bandwidth-bound logit
 * scans (top-W partials, target arg-max partials), the mask and the attention's main pass
 * share the first launch; the split-KV merge, the top-W merge and the verification walk
 * share the second.  In fp32 the attention (vector ALU, no split-KV) joins the second
 * launch instead, after the mask.  When a KV group holds more than 128 query rows (G*B > 128)
 * in several sequences, the attention runs 256-row workgroups whose LDS leaves no room
 * beside them, and the scans and the mask take a launch of their own before it (three
 * launches); those sequences take the attention's balanced schedule, which spreads all
 * sequences' key tiles evenly over the workgroups whatever their prefix lengths (each
 * workgroup finds its own share from the prefix lengths).  A single such sequence keeps
 * two launches: its attention runs 128-row workgroups in the first, beside the scans, in
 * fewer and longer key chunks than jt_tree_attention uses.  In the two-launch form the
 * attention builds the ancestor rows it needs from `parent` itself, so it does not wait
 * for the mask.  The integer outputs (ids, anc, depth, the accepted path, bonus, arg-max)
 * and the attention outputs equal bit for bit what the four separate calls produce,
 * except that single sequence's attention outputs, whose other key split makes them agree
 * to bf16 rounding; logprob, row_lse and row_entropy agree to float rounding, because the
 * step may cut a logit row into pieces differently from jt_topw_per_depth (the sums then
 * add in another order).  `err` (int32 [S], optional) receives the OR of the flags the mask,
 * attention and verification calls would report.
 *
 *   draft_logits   [S*N, draft_row_stride]   target_logits [S*B, target_row_stride]
 *   (both dtype, V used columns, 16-byte aligned, row strides a multiple of 16 bytes)
 *   W, N           as for jt_topw_per_depth (rows = S*N) and jt_verify_greedy
 *   row_entropy    optional, as for jt_topw_per_depth
 *   attention args as for jt_tree_attention (anc is produced here)
 * Supported: dtype JT_BF16 or JT_F32; d in {64, 128}; the ranges of the four calls.
 * Anything else returns JT_ERR_DTYPE / JT_ERR_ALIGN / JT_ERR_SHAPE: use the four calls
 * instead.
 */
size_t jt_step_workspace_size(int32_t S, int32_t B, int32_t N, int32_t W, int32_t V, int32_t Hq,
                              int32_t Hkv, int32_t d, int32_t max_prefix, int32_t block_size,
                              jt_dtype dtype);
jt_status jt_draft_verify_step(const void *draft_logits, int64_t draft_row_stride,
                               const void *target_logits, int64_t target_row_stride, int32_t V,
                               int32_t W, const int32_t *parent, const int32_t *tokens,
                               int32_t S, int32_t B, int32_t N, const void *q,
                               const void *k_tree, const void *v_tree, const void *k_prefix,
                               const void *v_prefix, const int32_t *block_table,
                               int32_t max_blocks_per_seq, int32_t block_size,
                               int32_t num_blocks, const int32_t *prefix_len, int32_t max_prefix,
                               int32_t Hq, int32_t Hkv, int32_t d, float scale, jt_dtype dtype,
                               int32_t *ids, float *logprob, float *row_lse,
                               float *row_entropy, uint64_t *anc,
                               int32_t *depth, void *out, float *lse, int32_t *accept_len,
                               int32_t *accept_path, int32_t *bonus, int32_t *argmax_out,
                               int32_t *err, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * jt_draft_verify_step without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Arguments, outputs and results are those of jt_draft_verify_step (bit for
 * bit the same); the scratch that call takes as `workspace` is instead a static device
 * array of JT_STATIC_SCRATCH_BYTES (48 MiB) inside the library, one per GPU the call runs
 * on, held until the process ends.  The call allocates nothing (the first call on a
 * device only looks up that device's address of the array).  Every call on one GPU uses
 * the same array, which keeps the last call's contents (the step needs none of them):
 * calls that overlap in time on one GPU race and must be serialised by the caller.
 * Returns JT_ERR_SCRATCH when jt_step_workspace_size() for the shape exceeds
 * JT_STATIC_SCRATCH_BYTES (use jt_draft_verify_step with a workspace then).
 */
#define JT_STATIC_SCRATCH_BYTES (48u << 20)
jt_status jt_draft_verify_step_noalloc(const void *draft_logits, int64_t draft_row_stride,
                                       const void *target_logits, int64_t target_row_stride,
                                       int32_t V, int32_t W, const int32_t *parent,
                                       const int32_t *tokens, int32_t S, int32_t B, int32_t N,
                                       const void *q, const void *k_tree, const void *v_tree,
                                       const void *k_prefix, const void *v_prefix,
                                       const int32_t *block_table, int32_t max_blocks_per_seq,
                                       int32_t block_size, int32_t num_blocks,
                                       const int32_t *prefix_len, int32_t max_prefix, int32_t Hq,
                                       int32_t Hkv, int32_t d, float scale, jt_dtype dtype,
                                       int32_t *ids, float *logprob, float *row_lse,
                                       float *row_entropy, uint64_t *anc, int32_t *depth,
                                       void *out, float *lse, int32_t *accept_len,
                                       int32_t *accept_path, int32_t *bonus, int32_t *argmax_out,
                                       int32_t *err, void *stream);

/*
 * Stochastic tree verification at temperature T > 0.  With a fixed draft every proposal
 * is a point mass at the draft token, accepted with the target probability, and after a
 * rejection the next token comes from the residual, so every committed token is the
 * target's own draw (JetSpec review, inference, acceptance equation; JetSpec++ summary,
 * appendices F.1 and F.3).  Sibling tokens being distinct, this is done as one draw per
 * node, x[s,v] ~ softmax(target_logits[s,v,:] / T): the first token t, in id order, whose
 * cumulative weight exceeds uniform[s,v] times the row's total weight.  Then the walk of
 * jt_verify_greedy with x in place of the arg-max: v is accepted iff every edge of its
 * root path carries the draw of its parent, v* is the deepest accepted node (lowest index
 * on ties), accept_len = depth(v*), bonus = x[s,v*].  NaN entries weigh 0 and flag the
 * sequence (JT_DEV_NAN); a row of -inf draws token 0.
 *
 *   target_logits [S*B, row_stride] dtype    uniform float [S,B], values in [0, 1)
 *   parent, tokens, anc, depth, N, outputs and err as for jt_verify_greedy
 *   sample_out    int32 [S,B] (optional) out: the draw at every node
 * A draw whose uniform lies within about 1e-5 of its token's interval end (as a fraction of
 * the row's weight) may go to the neighbouring token under a different summation order.
 * Supported: temperature > 0 and finite, with log2(e) / temperature finite in fp32 (so
 * temperature >= about 4.2e-39; smaller values return JT_ERR_SHAPE); otherwise as
 * jt_verify_greedy.
 */
size_t jt_verify_sampled_workspace_size(int32_t S, int32_t B, int32_t V, jt_dtype dtype);
jt_status jt_verify_sampled(const void *target_logits, int64_t row_stride, int32_t V,
                            jt_dtype dtype, float temperature, const float *uniform,
                            const int32_t *parent, const int32_t *tokens, const uint64_t *anc,
                            const int32_t *depth, int32_t S, int32_t B, int32_t N,
                            int32_t *accept_len, int32_t *accept_path, int32_t *bonus,
                            int32_t *sample_out, int32_t *err, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * Best-first construction of the draft tree from the per-depth candidate lists that
 * jt_topw_per_depth produces (paperlayer.ai JetSpec summary, appendix B "Tree-Drafting
 * Algorithm Details", section 2 and appendix E "Drafting"; JetSpec review, inference,
 * path-score equation; paper.rainbus.top summary, method steps).  Per sequence: node 0
 * is the root (depth 0, score 0, token root_token[s]); the queued node that pops first --
 * larger score, then lower node index, a NaN score last -- leaves the queue; a node at
 * depth N is not expanded; otherwise it gains children of rank r = 0..W-1 in order while
 * the tree holds fewer than B nodes.  Child r of a node at depth d carries token
 * ids[s*N + d][r] and the score
 *     score(parent) + (w_lp * logprob[s*N + d][r] - w_ent * entropy[s*N + d]),
 * each product, the difference and the sum rounded to float in turn (no fused
 * multiply-add).  w_lp = 1, w_ent = 0 scores by the path's cumulative draft
 * log-probability; w_lp = 0, w_ent = 1 by per-depth entropy alone; w_lp = 1, w_ent =
 * alpha is the hybrid.  When the queue empties before B nodes exist, slots n..B-1 are
 * padding: parent 0, token -1, score -inf (a node that can never be accepted).
 *
 *   ids, logprob  [S*N, W] int32 / float32 (row s*N + d: the candidates of depth d+1)
 *   entropy       [S*N] float32, or NULL (taken as 0)
 *   root_token    [S] int32, or NULL (root token -1)
 *   parent, tokens [S, B] int32 out: parent[s,0] = -1 and 0 <= parent[s,i] < i, the
 *                 layout the mask, attention and verification calls take
 *   score         [S, B] float32 out, or NULL      n_nodes [S] int32 out, or NULL
 * Supported: 1 <= W <= 16, 1 <= B <= 256, 0 <= N <= 255.  No workspace; one wave per
 * sequence.
 */
jt_status jt_build_tree_best_first(const int32_t *ids, const float *logprob,
                                   const float *entropy, float w_lp, float w_ent,
                                   const int32_t *root_token, int32_t S, int32_t N, int32_t W,
                                   int32_t B, int32_t *parent, int32_t *tokens, float *score,
                                   int32_t *n_nodes, void *stream);

/*
 * Accepted-path commit: the K/V of the accepted root path join the prefix cache.  The
 * verifier commits the longest accepted root path (paperlayer.ai JetSpec summary,
 * section 2; JetSpec++ summary, section 3), whose K/V this pass computed in k_tree /
 * v_tree.  Node 0 is the root (the last committed token), so for sequence s with
 * L = accept_len[s] and P = prefix_len[s], node accept_path[s][i] is written to prefix
 * position P + i for i = 0..L, every KV head, and new_prefix_len[s] = P + L + 1.  A node
 * at depth i has rotary position P + i, which is its slot; nothing is re-rotated.
 *
 *   accept_len [S], accept_path [S, N+1]   as jt_verify_greedy writes them
 *   k_tree, v_tree   [S, B, Hkv, d] dtype
 *   k_cache, v_cache contiguous [S, max_prefix, Hkv, d] when block_table is NULL; else
 *                    paged [num_blocks, block_size, Hkv, d], position j of sequence s in
 *                    block block_table[s * max_blocks_per_seq + j / block_size]
 *   prefix_len [S] in, new_prefix_len [S] out (may be the same array: the update is then
 *                    in place)
 *   err [S] (optional) out: JT_DEV_DEPTH_GT_N when accept_len is outside [0, N] and
 *                    JT_DEV_BAD_PREFIX when P < 0 or P + L + 1 exceeds the capacity
 *                    (max_prefix, or max_blocks_per_seq * block_size) -- nothing is
 *                    written then; JT_DEV_BAD_PARENT for a path entry outside [0, B) and
 *                    JT_DEV_BAD_BLOCK for a block id outside [0, num_blocks) -- that row
 *                    is skipped.  A flagged sequence keeps new_prefix_len = P.
 * Supported: d in {64, 128}; dtype JT_BF16 or JT_F32; 0 <= N <= 255; 1 <= B <= 256;
 * the four K/V pointers 16-byte aligned.  No workspace; one workgroup per sequence.
 */
jt_status jt_commit_accepted_kv(const int32_t *accept_len, const int32_t *accept_path, int32_t N,
                                const void *k_tree, const void *v_tree, int32_t S, int32_t B,
                                int32_t Hkv, int32_t d, jt_dtype dtype, void *k_cache,
                                void *v_cache, const int32_t *block_table,
                                int32_t max_blocks_per_seq, int32_t block_size,
                                int32_t num_blocks, const int32_t *prefix_len,
                                int32_t max_prefix, int32_t *new_prefix_len, int32_t *err,
                                void *stream);

/*
 * Measurement helper, not a step of the method: the bf16 matrix-core rate the device
 * sustains, reported beside the nominal dense peak.  Launches `blocks` workgroups of 4
 * waves; every wave issues iters * 8 independent v_mfma_f32_32x32x16_bf16 (32x32x16
 * products, 32,768 flops each), so the work is blocks * 4 * iters * 8 * 32768 flops; time
 * it with events on `stream`.  4 workgroups per compute unit (1024 on MI355X) put 4 waves
 * on every SIMD.
 *   out   float [blocks * 256] device, overwritten with the accumulators' sums.
 * Supported: iters >= 1, blocks >= 1.
 */
jt_status jt_probe_mfma_rate(int32_t iters, int32_t blocks, float *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* JT_H */
