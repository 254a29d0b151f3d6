// extern "C" entry points of libjt: argument checks on the host, then stream-ordered
// launches.  Nothing here allocates, synchronises or keeps state.
#include <math.h>

#include "jt_internal.h"

using namespace jt;

static_assert(kStaticScratchBytes == JT_STATIC_SCRATCH_BYTES, "static scratch size");

namespace {

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int x)
{
    int r = 0;
    while ((1 << r) < x)
        ++r;
    return r;
}

} // namespace

extern "C" {

int jt_abi_version(void) { return JT_ABI_VERSION; }

const char *jt_status_string(int status)
{
    switch (status) {
    case JT_OK: return "ok";
    case JT_ERR_NULL: return "a required pointer is NULL";
    case JT_ERR_SHAPE: return "a size is outside the supported range";
    case JT_ERR_DTYPE: return "unsupported element type";
    case JT_ERR_WORKSPACE: return "workspace too small";
    case JT_ERR_LAUNCH: return "kernel launch failed";
    case JT_ERR_ALIGN: return "pointer or stride misaligned";
    case JT_ERR_SCRATCH:
        return "the shape needs more scratch than the library's static buffer holds "
               "(use the call that takes a workspace)";
    default: return "unknown status";
    }
}

jt_status jt_build_tree_mask(const int32_t *parent, int32_t S, int32_t B, uint64_t *anc,
                             int32_t *depth, int32_t *err, void *stream)
{
    if (S < 0 || B < 1 || B > JT_MAX_NODES)
        return JT_ERR_SHAPE;
    if (S == 0)
        return JT_OK;
    if (!parent || !anc || !depth)
        return JT_ERR_NULL;
    return launch_build_mask(parent, S, B, anc, depth, err, as_stream(stream));
}

static jt_status attn_shape(int32_t S, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                            int32_t max_prefix, jt_dtype dtype)
{
    if (dtype != JT_BF16 && dtype != JT_F32)
        return JT_ERR_DTYPE;
    if (S < 0 || B < 1 || B > JT_MAX_NODES || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 ||
        Hq / Hkv > 8 || (d != 64 && d != 128) || max_prefix < 0)
        return JT_ERR_SHAPE;
    if ((int64_t)S * B * Hq > INT32_MAX / 2 || (int64_t)S * Hkv > 65535)
        return JT_ERR_SHAPE;
    return JT_OK;
}

size_t jt_tree_attention_workspace_size(int32_t S, int32_t B, int32_t Hq, int32_t Hkv,
                                        int32_t d, int32_t max_prefix, int32_t block_size,
                                        jt_dtype dtype)
{
    if (attn_shape(S, B, Hq, Hkv, d, max_prefix, dtype) != JT_OK || S == 0)
        return 0;
    return attention_workspace(S, B, Hq, Hkv, d, max_prefix, block_size > 0 ? block_size : 0,
                               dtype);
}

jt_status jt_tree_attention(const void *q, const void *k_tree, const void *v_tree,
                            const void *k_prefix, const void *v_prefix,
                            const int32_t *block_table, int32_t max_blocks_per_seq,
                            int32_t block_size, int32_t num_blocks,
                            const int32_t *prefix_len, int32_t max_prefix, const uint64_t *anc,
                            int32_t S, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                            jt_dtype dtype, float scale, void *out, float *lse, int32_t *err,
                            void *workspace, size_t workspace_bytes, void *stream)
{
    jt_status st = attn_shape(S, B, Hq, Hkv, d, max_prefix, dtype);
    if (st != JT_OK)
        return st;
    if (S == 0)
        return JT_OK;
    if (!q || !k_tree || !v_tree || !prefix_len || !anc || !out)
        return JT_ERR_NULL;
    if (max_prefix > 0 && (!k_prefix || !v_prefix))
        return JT_ERR_NULL;
    if (block_table) {
        if (!is_pow2(block_size) || max_blocks_per_seq < 0 || num_blocks < 0 ||
            (int64_t)max_blocks_per_seq * block_size < max_prefix)
            return JT_ERR_SHAPE;
    }
    if (!aligned16(q) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(out) ||
        (k_prefix && !aligned16(k_prefix)) || (v_prefix && !aligned16(v_prefix)))
        return JT_ERR_ALIGN;
    const size_t need =
        attention_workspace(S, B, Hq, Hkv, d, max_prefix, block_table ? block_size : 0, dtype);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return JT_ERR_WORKSPACE;
    if (need > 0 && !aligned16(workspace))
        return JT_ERR_ALIGN;
    AttnArgs a;
    a.q = q;
    a.k_tree = k_tree;
    a.v_tree = v_tree;
    a.k_prefix = k_prefix;
    a.v_prefix = v_prefix;
    a.block_table = block_table;
    a.max_blocks = max_blocks_per_seq;
    a.block_size = block_table ? block_size : 1;
    a.block_shift = block_table ? log2i(block_size) : 0;
    a.num_blocks = num_blocks;
    a.prefix_len = prefix_len;
    a.max_prefix = max_prefix;
    a.anc = anc;
    a.parent = nullptr;
    a.S = S;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.d = d;
    a.G = Hq / Hkv;
    a.dtype = dtype;
    a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
    a.out = out;
    a.lse = lse;
    a.err = err;
    return launch_attention(a, workspace, as_stream(stream));
}

static jt_status topw_shape(int32_t rows, int32_t V, int32_t W, jt_dtype dtype)
{
    if (dtype != JT_BF16 && dtype != JT_F32)
        return JT_ERR_DTYPE;
    if (rows < 0 || V < 1 || W < 1 || W > JT_MAX_W || W > V)
        return JT_ERR_SHAPE;
    return JT_OK;
}

size_t jt_topw_workspace_size(int32_t rows, int32_t V, int32_t W, jt_dtype dtype)
{
    if (topw_shape(rows, V, W, dtype) != JT_OK || rows == 0)
        return 0;
    return topw_workspace(rows, V, W, dtype);
}

jt_status jt_topw_per_depth(const void *logits, int64_t row_stride, int32_t rows, int32_t V,
                            int32_t W, jt_dtype dtype, int32_t *ids, float *logprob,
                            float *row_lse, float *row_entropy, void *workspace,
                            size_t workspace_bytes, void *stream)
{
    jt_status st = topw_shape(rows, V, W, dtype);
    if (st != JT_OK)
        return st;
    if (row_stride < V)
        return JT_ERR_SHAPE;
    if (rows == 0)
        return JT_OK;
    if (!logits || !ids || !logprob)
        return JT_ERR_NULL;
    const size_t need = topw_workspace(rows, V, W, dtype);
    if (!workspace || workspace_bytes < need)
        return JT_ERR_WORKSPACE;
    if (!aligned16(workspace))
        return JT_ERR_ALIGN;
    return launch_topw(logits, row_stride, rows, V, W, dtype, ids, logprob, row_lse, row_entropy,
                       workspace, as_stream(stream));
}

static jt_status verify_shape(int32_t S, int32_t B, int32_t V, int32_t N, jt_dtype dtype)
{
    if (dtype != JT_BF16 && dtype != JT_F32)
        return JT_ERR_DTYPE;
    if (S < 0 || B < 1 || B > JT_MAX_NODES || V < 1 || N < 0 || N > 255)
        return JT_ERR_SHAPE;
    return JT_OK;
}

size_t jt_verify_workspace_size(int32_t S, int32_t B, int32_t V, jt_dtype dtype)
{
    if (verify_shape(S, B, V, 0, dtype) != JT_OK || S == 0)
        return 0;
    return verify_workspace(S, B, V, dtype);
}

jt_status jt_verify_greedy(const void *target_logits, int64_t row_stride, int32_t V,
                           jt_dtype dtype, const int32_t *parent, const int32_t *tokens,
                           const uint64_t *anc, const int32_t *depth, int32_t S, int32_t B,
                           int32_t N, int32_t *accept_len, int32_t *accept_path,
                           int32_t *bonus, int32_t *argmax_out, int32_t *err,
                           void *workspace, size_t workspace_bytes, void *stream)
{
    jt_status st = verify_shape(S, B, V, N, dtype);
    if (st != JT_OK)
        return st;
    if (row_stride < V)
        return JT_ERR_SHAPE;
    if (S == 0)
        return JT_OK;
    if (!target_logits || !parent || !tokens || !anc || !depth || !accept_len ||
        !accept_path || !bonus)
        return JT_ERR_NULL;
    const size_t need = verify_workspace(S, B, V, dtype);
    if (!workspace || workspace_bytes < need)
        return JT_ERR_WORKSPACE;
    if (!aligned16(workspace))
        return JT_ERR_ALIGN;
    return launch_verify(target_logits, row_stride, V, dtype, parent, tokens, anc, depth, S, B, N,
                         accept_len, accept_path, bonus, argmax_out, err, workspace,
                         as_stream(stream));
}

size_t jt_verify_sampled_workspace_size(int32_t S, int32_t B, int32_t V, jt_dtype dtype)
{
    if (verify_shape(S, B, V, 0, dtype) != JT_OK || S == 0)
        return 0;
    return sample_workspace(S, B, V);
}

jt_status jt_verify_sampled(const void *target_logits, int64_t row_stride, int32_t V,
                            jt_dtype dtype, float temperature, const float *uniform,
                            const int32_t *parent, const int32_t *tokens, const uint64_t *anc,
                            const int32_t *depth, int32_t S, int32_t B, int32_t N,
                            int32_t *accept_len, int32_t *accept_path, int32_t *bonus,
                            int32_t *sample_out, int32_t *err, void *workspace,
                            size_t workspace_bytes, void *stream)
{
    jt_status st = verify_shape(S, B, V, N, dtype);
    if (st != JT_OK)
        return st;
    // the draw weighs logits by 2^((x - max) * log2(e) / T): a temperature so small that
    // log2(e) / T overflows fp32 (below about 4.2e-39) would turn the weight at the row
    // maximum into 0 * inf = NaN, so it is refused like T <= 0
    if (row_stride < V || !(temperature > 0.f) || !(temperature < INFINITY) ||
        !(1.4426950408889634f / temperature < INFINITY))
        return JT_ERR_SHAPE;
    if (S == 0)
        return JT_OK;
    if (!target_logits || !uniform || !parent || !tokens || !anc || !depth || !accept_len ||
        !accept_path || !bonus)
        return JT_ERR_NULL;
    const size_t need = sample_workspace(S, B, V);
    if (!workspace || workspace_bytes < need)
        return JT_ERR_WORKSPACE;
    if (!aligned16(workspace))
        return JT_ERR_ALIGN;
    return launch_verify_sampled(target_logits, row_stride, V, dtype, temperature, uniform,
                                 parent, tokens, anc, depth, S, B, N, accept_len, accept_path,
                                 bonus, sample_out, err, workspace, as_stream(stream));
}

size_t jt_step_workspace_size(int32_t S, int32_t B, int32_t N, int32_t W, int32_t V, int32_t Hq,
                              int32_t Hkv, int32_t d, int32_t max_prefix, int32_t block_size,
                              jt_dtype dtype)
{
    if (attn_shape(S, B, Hq, Hkv, d, max_prefix, dtype) != JT_OK ||
        topw_shape(S * N, V, W, dtype) != JT_OK || verify_shape(S, B, V, N, dtype) != JT_OK ||
        S == 0)
        return 0;
    return step_workspace(S, B, N, W, V, Hq, Hkv, d, max_prefix, block_size > 0 ? block_size : 0,
                          dtype);
}

} // extern "C"

static jt_status step_setup(const void *draft_logits, int64_t draft_row_stride,
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
                               int32_t *err, StepLaunch &in, size_t &need)
{
    if (dtype != JT_BF16 && dtype != JT_F32)
        return JT_ERR_DTYPE;
    jt_status st = attn_shape(S, B, Hq, Hkv, d, max_prefix, dtype);
    if (st == JT_OK)
        st = verify_shape(S, B, V, N, dtype);
    if (st == JT_OK && (int64_t)S * N > INT32_MAX)
        st = JT_ERR_SHAPE;
    if (st == JT_OK)
        st = topw_shape(S * N, V, W, dtype);
    if (st != JT_OK)
        return st;
    if (draft_row_stride < V || target_row_stride < V)
        return JT_ERR_SHAPE;
    if (S == 0) {
        in.attn.S = 0;
        need = 0;
        return JT_OK;
    }
    if (!target_logits || !parent || !tokens || !q || !k_tree || !v_tree || !prefix_len ||
        !anc || !depth || !out || !accept_len || !accept_path || !bonus)
        return JT_ERR_NULL;
    if (N > 0 && (!draft_logits || !ids || !logprob))
        return JT_ERR_NULL;
    if (max_prefix > 0 && (!k_prefix || !v_prefix))
        return JT_ERR_NULL;
    if (block_table) {
        if (!is_pow2(block_size) || max_blocks_per_seq < 0 || num_blocks < 0 ||
            (int64_t)max_blocks_per_seq * block_size < max_prefix)
            return JT_ERR_SHAPE;
    }
    if (!aligned16(q) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(out) ||
        (k_prefix && !aligned16(k_prefix)) || (v_prefix && !aligned16(v_prefix)))
        return JT_ERR_ALIGN;
    const int per16 = dtype == JT_BF16 ? 8 : 4;  // elements per 16 bytes
    if (!aligned16(target_logits) || target_row_stride % per16 != 0 ||
        (N > 0 && (!aligned16(draft_logits) || draft_row_stride % per16 != 0)))
        return JT_ERR_ALIGN;
    need = step_workspace(S, B, N, W, V, Hq, Hkv, d, max_prefix, block_table ? block_size : 0,
                          dtype);
    AttnArgs &a = in.attn;
    a.q = q;
    a.k_tree = k_tree;
    a.v_tree = v_tree;
    a.k_prefix = k_prefix;
    a.v_prefix = v_prefix;
    a.block_table = block_table;
    a.max_blocks = max_blocks_per_seq;
    a.block_size = block_table ? block_size : 1;
    a.block_shift = block_table ? log2i(block_size) : 0;
    a.num_blocks = num_blocks;
    a.prefix_len = prefix_len;
    a.max_prefix = max_prefix;
    a.anc = nullptr;
    a.parent = parent;
    a.S = S;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.d = d;
    a.G = Hq / Hkv;
    a.dtype = dtype;
    a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
    a.out = out;
    a.lse = lse;
    a.err = nullptr;
    in.draft = draft_logits;
    in.target = target_logits;
    in.draft_stride = draft_row_stride;
    in.target_stride = target_row_stride;
    in.V = V;
    in.W = W;
    in.N = N;
    in.ids = ids;
    in.logprob = logprob;
    in.row_lse = row_lse;
    in.row_entropy = row_entropy;
    in.parent = parent;
    in.tokens = tokens;
    in.anc = anc;
    in.depth = depth;
    in.accept_len = accept_len;
    in.accept_path = accept_path;
    in.bonus = bonus;
    in.argmax_out = argmax_out;
    in.err = err;
    return JT_OK;
}

extern "C" {

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
                               void *stream)
{
    StepLaunch in;
    size_t need = 0;
    const jt_status st = step_setup(draft_logits, draft_row_stride, target_logits,
                                    target_row_stride, V, W, parent, tokens, S, B, N, q, k_tree,
                                    v_tree, k_prefix, v_prefix, block_table, max_blocks_per_seq,
                                    block_size, num_blocks, prefix_len, max_prefix, Hq, Hkv, d,
                                    scale, dtype, ids, logprob, row_lse, row_entropy, anc, depth,
                                    out, lse, accept_len, accept_path, bonus, argmax_out, err, in,
                                    need);
    if (st != JT_OK || S == 0)
        return st;
    if (!workspace || workspace_bytes < need)
        return JT_ERR_WORKSPACE;
    if (!aligned16(workspace))
        return JT_ERR_ALIGN;
    return launch_step(in, workspace, as_stream(stream));
}

jt_status jt_draft_verify_step_noalloc(const void *draft_logits, int64_t draft_row_stride,
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
                               int32_t *err,
                                       void *stream)
{
    StepLaunch in;
    size_t need = 0;
    const jt_status st = step_setup(draft_logits, draft_row_stride, target_logits,
                                    target_row_stride, V, W, parent, tokens, S, B, N, q, k_tree,
                                    v_tree, k_prefix, v_prefix, block_table, max_blocks_per_seq,
                                    block_size, num_blocks, prefix_len, max_prefix, Hq, Hkv, d,
                                    scale, dtype, ids, logprob, row_lse, row_entropy, anc, depth,
                                    out, lse, accept_len, accept_path, bonus, argmax_out, err, in,
                                    need);
    if (st != JT_OK || S == 0)
        return st;
    if (need > kStaticScratchBytes)
        return JT_ERR_SCRATCH;
    return launch_step_static(in, as_stream(stream));
}

jt_status jt_build_tree_best_first(const int32_t *ids, const float *logprob,
                                   const float *entropy, float w_lp, float w_ent,
                                   const int32_t *root_token, int32_t S, int32_t N, int32_t W,
                                   int32_t B, int32_t *parent, int32_t *tokens, float *score,
                                   int32_t *n_nodes, void *stream)
{
    if (S < 0 || N < 0 || N > 255 || W < 1 || W > JT_MAX_W || B < 1 || B > JT_MAX_NODES)
        return JT_ERR_SHAPE;
    if (S == 0)
        return JT_OK;
    if (!parent || !tokens || (N > 0 && (!ids || !logprob)))
        return JT_ERR_NULL;
    return launch_build_tree(ids, logprob, entropy, w_lp, w_ent, root_token, S, N, W, B, parent,
                             tokens, score, n_nodes, as_stream(stream));
}

jt_status jt_commit_accepted_kv(const int32_t *accept_len, const int32_t *accept_path, int32_t N,
                                const void *k_tree, const void *v_tree, int32_t S, int32_t B,
                                int32_t Hkv, int32_t d, jt_dtype dtype, void *k_cache,
                                void *v_cache, const int32_t *block_table,
                                int32_t max_blocks_per_seq, int32_t block_size,
                                int32_t num_blocks, const int32_t *prefix_len,
                                int32_t max_prefix, int32_t *new_prefix_len, int32_t *err,
                                void *stream)
{
    if (dtype != JT_BF16 && dtype != JT_F32)
        return JT_ERR_DTYPE;
    if (S < 0 || N < 0 || N > 255 || B < 1 || B > JT_MAX_NODES || Hkv < 1 ||
        (d != 64 && d != 128))
        return JT_ERR_SHAPE;
    if (block_table ? (max_blocks_per_seq < 1 || block_size < 1 || num_blocks < 1)
                    : max_prefix < 0)
        return JT_ERR_SHAPE;
    if (S == 0)
        return JT_OK;
    if (!accept_len || !accept_path || !k_tree || !v_tree || !k_cache || !v_cache ||
        !prefix_len || !new_prefix_len)
        return JT_ERR_NULL;
    if (!aligned16(k_tree) || !aligned16(v_tree) || !aligned16(k_cache) || !aligned16(v_cache))
        return JT_ERR_ALIGN;
    return launch_commit_kv(accept_len, accept_path, N, k_tree, v_tree, S, B, Hkv, d,
                            dtype == JT_BF16 ? 2 : 4, k_cache, v_cache, block_table,
                            max_blocks_per_seq, block_size, num_blocks, prefix_len, max_prefix,
                            new_prefix_len, err, as_stream(stream));
}

jt_status jt_probe_mfma_rate(int32_t iters, int32_t blocks, float *out, void *stream)
{
    if (iters < 1 || blocks < 1)
        return JT_ERR_SHAPE;
    if (!out)
        return JT_ERR_NULL;
    return launch_mfma_rate(iters, blocks, out, as_stream(stream));
}

} // extern "C"
