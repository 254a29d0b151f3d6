/*
 * jt_oracle.c -- CPU oracle for one draft-and-verify step over a token tree.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header, table or constant with the HIP library.
 *
 * Plain, slow, single-threaded C11.  Every floating-point input is widened to
 * double (bf16 -> float is exact, float -> double is exact) and every result is
 * computed and returned in double.  Masks are dense, sorts are full sorts, and
 * softmax is the two-pass max-subtracted textbook form.  No blocking, fusion or
 * reordering beyond what the definitions state.
 *
 * Sources (the JetSpec pages):
 *  - tree-causal mask: M[v,u] = 0 iff u is an ancestor of v or v itself,
 *    -inf otherwise ("How it works", mask equation, startedourmission.github.io
 *    review of JetSpec); nodes see the prefix, their ancestors and themselves,
 *    never siblings or descendants (paperlayer.ai JetSpec summary, section 2
 *    "Architecture").
 *  - verification uses parent indices, depths and the tree mask in one pass
 *    (paperlayer.ai JetSpec summary, appendix E "Verification").
 *  - per-position top-k tokens and log-probabilities (same page, appendix E
 *    "Drafting"); top-W per depth (paper.rainbus.top summary, method steps).
 *  - best-first tree construction by cumulative path score from the per-depth
 *    candidate lists (paperlayer.ai JetSpec summary, appendix B; review,
 *    inference, path-score equation; paper.rainbus.top summary, method steps).
 *  - acceptance of the longest valid prefix plus a bonus token (paperlayer.ai
 *    JetSpec summary section 2; JetSpec++ summary section 3); at temperature 0
 *    the min(1, p/q) rule of the review's inference section reduces to
 *    "draft token equals the target argmax" (point-mass proposal, JetSpec++
 *    summary appendix F.3).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - node 0 is the tree root and is counted in B; parent[0] = -1 and
 *    0 <= parent[i] < i for i >= 1, anything else is a bad parent array;
 *  - softmax scale 1/sqrt(d) when the caller passes scale <= 0;
 *  - query head h reads KV head h / (Hq/Hkv) (contiguous GQA groups);
 *  - top-W order is value descending, token id ascending; -0 equals +0;
 *    NaN ranks below -inf;
 *  - argmax ties go to the lowest token id; NaN entries are skipped and flagged;
 *  - among accepted nodes the deepest wins, ties to the lowest node index;
 *  - tree construction pops ties in node-index order, accumulates scores in
 *    float (they decide integers), and pads unfilled slots (parent 0, token -1).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* device-style per-sequence flags (same meaning as the library's, values
 * restated here on purpose: the oracle includes no library header) */
#define ORA_BAD_PARENT 1
#define ORA_DEPTH_GT_N 2
#define ORA_BAD_BLOCK 4
#define ORA_NAN 8
#define ORA_BAD_PREFIX 16

/* element types: 0 = IEEE float32, 1 = bfloat16 stored as raw 16-bit words */
static double elem(const void *base, int64_t i, int dtype)
{
    if (dtype == 0)
        return (double)((const float *)base)[i];
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

int jto_version(void) { return 1; }

/* ---------------------------------------------------------------- mask -- */

/* Checks the parent-array layout of one sequence.  Returns 1 when valid. */
static int parents_valid(const int32_t *par, int B)
{
    if (B < 1 || par[0] != -1)
        return 0;
    for (int i = 1; i < B; i++)
        if (par[i] < 0 || par[i] >= i)
            return 0;
    return 1;
}

/*
 * Dense tree-causal visibility and depths.
 *   vis[s][v][u] = 1 iff u in Anc(v) or u == v (walk parents up to the root),
 *   depth[s][v]  = number of parent steps from v to the root.
 * A sequence with a bad parent array gets ORA_BAD_PARENT in err[s], an
 * all-zero vis block and depth -1 everywhere.
 */
int jto_build_mask(const int32_t *parent, int S, int B, uint8_t *vis,
                   int32_t *depth, int32_t *err)
{
    if (S < 0 || B < 1)
        return 2;
    for (int s = 0; s < S; s++) {
        const int32_t *par = parent + (int64_t)s * B;
        uint8_t *V = vis + (int64_t)s * B * B;
        int32_t *dep = depth + (int64_t)s * B;
        memset(V, 0, (size_t)B * B);
        if (!parents_valid(par, B)) {
            err[s] = ORA_BAD_PARENT;
            for (int v = 0; v < B; v++)
                dep[v] = -1;
            continue;
        }
        err[s] = 0;
        for (int v = 0; v < B; v++) {
            int steps = 0;
            for (int u = v; u != -1; u = par[u]) {
                V[(int64_t)v * B + u] = 1;
                steps++;
            }
            dep[v] = steps - 1;
        }
    }
    return 0;
}

/* ----------------------------------------------------------- attention -- */

/*
 * Tree-causal GQA attention of all B tree nodes of each sequence against that
 * sequence's prefix KV and the tree's own KV.
 *
 * For sequence s, node v, query head h (KV head g = h / (Hq/Hkv)):
 *   score_j = scale * <q[s,v,h], k_prefix[s,j,g]>            j < prefix_len[s]
 *   score_u = scale * <q[s,v,h], k_tree[s,u,g]> + M[v,u]     u < B
 *   out     = sum_j softmax(score)_j * value_j,  lse = log sum_j exp(score_j)
 * with M from jto_build_mask (0 visible, -inf hidden, exp(-inf) = 0 exactly).
 *
 * Prefix layout: block_table == NULL -> contiguous [S, max_prefix, Hkv, d];
 * otherwise a pool [num_blocks, block_size, Hkv, d] where logical key j of
 * sequence s lives in block block_table[s*max_blocks + j/block_size], slot
 * j % block_size.  Keys of a block id outside [0, num_blocks) are skipped and
 * flagged ORA_BAD_BLOCK; prefix_len outside [0, max_prefix] is flagged
 * ORA_BAD_PREFIX and clamped.
 *
 * Rows: n_sel == 0 -> every (s, v, h) in that order, out is [S,B,Hq,d];
 * otherwise the n_sel (s, v, h) triples in sel[], out is [n_sel, d].
 * Returns 0, or 2 on a shape error.
 */
int jto_tree_attention(const void *q, const void *k_tree, const void *v_tree,
                       const void *k_prefix, const void *v_prefix,
                       const int32_t *block_table, int max_blocks, int block_size,
                       int num_blocks, const int32_t *prefix_len, int max_prefix,
                       const int32_t *parent, int S, int B, int Hq, int Hkv, int d,
                       int dtype, double scale, int n_sel, const int32_t *sel,
                       double *out, double *lse, int32_t *err)
{
    if (S < 1 || B < 1 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv != 0 || max_prefix < 0)
        return 2;
    if (block_table && (block_size < 1 || max_blocks < 0))
        return 2;
    const int G = Hq / Hkv;
    if (scale <= 0.0)
        scale = 1.0 / sqrt((double)d);

    uint8_t *vis = (uint8_t *)malloc((size_t)S * B * B);
    int32_t *dep = (int32_t *)malloc(sizeof(int32_t) * (size_t)S * B);
    int32_t *merr = (int32_t *)malloc(sizeof(int32_t) * (size_t)S);
    double *sc = (double *)malloc(sizeof(double) * ((size_t)max_prefix + B));
    int32_t *kpos = (int32_t *)malloc(sizeof(int32_t) * ((size_t)max_prefix + 1));
    if (!vis || !dep || !merr || !sc || !kpos) {
        free(vis); free(dep); free(merr); free(sc); free(kpos);
        return 3;
    }
    jto_build_mask(parent, S, B, vis, dep, merr);
    for (int s = 0; s < S; s++) {
        int32_t e = merr[s];
        int P = prefix_len[s];
        if (P < 0 || P > max_prefix)
            e |= ORA_BAD_PREFIX;
        if (block_table) {
            int P2 = P < 0 ? 0 : (P > max_prefix ? max_prefix : P);
            for (int j = 0; j < P2; j += block_size) {
                int lb = j / block_size;
                int blk = lb < max_blocks ? block_table[(int64_t)s * max_blocks + lb] : -1;
                if (blk < 0 || blk >= num_blocks)
                    e |= ORA_BAD_BLOCK;
            }
        }
        err[s] = e;
    }

    int64_t nrows = n_sel > 0 ? n_sel : (int64_t)S * B * Hq;
    for (int64_t r = 0; r < nrows; r++) {
        int s, v, h;
        if (n_sel > 0) {
            s = sel[3 * r]; v = sel[3 * r + 1]; h = sel[3 * r + 2];
        } else {
            s = (int)(r / ((int64_t)B * Hq));
            v = (int)((r / Hq) % B);
            h = (int)(r % Hq);
        }
        int g = h / G;
        int P = prefix_len[s];
        if (P < 0) P = 0;
        if (P > max_prefix) P = max_prefix;
        const int64_t qoff = (((int64_t)s * B + v) * Hq + h) * d;

        /* physical row index of each logical prefix key, -1 when skipped */
        for (int j = 0; j < P; j++) {
            if (!block_table) {
                kpos[j] = j;
            } else {
                int lb = j / block_size;
                int blk = lb < max_blocks ? block_table[(int64_t)s * max_blocks + lb] : -1;
                kpos[j] = (blk < 0 || blk >= num_blocks) ? -1 : blk * block_size + j % block_size;
            }
        }
        /* pass 0: scores */
        int nk = P + B;
        for (int j = 0; j < P; j++) {
            if (kpos[j] < 0) { sc[j] = -INFINITY; continue; }
            int64_t koff = block_table ? ((int64_t)kpos[j] * Hkv + g) * d
                                       : (((int64_t)s * max_prefix + j) * Hkv + g) * d;
            double acc = 0.0;
            for (int c = 0; c < d; c++)
                acc += elem(q, qoff + c, dtype) * elem(k_prefix, koff + c, dtype);
            sc[j] = scale * acc;
        }
        const uint8_t *mrow = vis + ((int64_t)s * B + v) * B;
        for (int u = 0; u < B; u++) {
            int64_t koff = (((int64_t)s * B + u) * Hkv + g) * d;
            double acc = 0.0;
            for (int c = 0; c < d; c++)
                acc += elem(q, qoff + c, dtype) * elem(k_tree, koff + c, dtype);
            sc[P + u] = mrow[u] ? scale * acc : -INFINITY;
        }
        /* pass 1: max; pass 2: exp and normaliser */
        double m = -INFINITY;
        for (int j = 0; j < nk; j++)
            if (sc[j] > m) m = sc[j];
        double Z = 0.0;
        for (int j = 0; j < nk; j++) {
            sc[j] = (sc[j] == -INFINITY) ? 0.0 : exp(sc[j] - m);
            Z += sc[j];
        }
        /* pass 3: weighted sum of values */
        double *o = out + r * d;
        for (int c = 0; c < d; c++)
            o[c] = 0.0;
        for (int j = 0; j < P; j++) {
            if (sc[j] == 0.0) continue;
            int64_t voff = block_table ? ((int64_t)kpos[j] * Hkv + g) * d
                                       : (((int64_t)s * max_prefix + j) * Hkv + g) * d;
            for (int c = 0; c < d; c++)
                o[c] += sc[j] * elem(v_prefix, voff + c, dtype);
        }
        for (int u = 0; u < B; u++) {
            if (sc[P + u] == 0.0) continue;
            int64_t voff = (((int64_t)s * B + u) * Hkv + g) * d;
            for (int c = 0; c < d; c++)
                o[c] += sc[P + u] * elem(v_tree, voff + c, dtype);
        }
        if (Z > 0.0) {
            for (int c = 0; c < d; c++)
                o[c] /= Z;
            lse[r] = m + log(Z);
        } else {
            lse[r] = -INFINITY;
        }
    }
    free(vis); free(dep); free(merr); free(sc); free(kpos);
    return 0;
}

/* ---------------------------------------------------------------- top-W -- */

typedef struct { double x; int32_t i; } ora_item;

/* total order: non-NaN before NaN; larger value first; lower id first */
static int item_cmp(const void *pa, const void *pb)
{
    const ora_item *a = (const ora_item *)pa, *b = (const ora_item *)pb;
    int an = isnan(a->x), bn = isnan(b->x);
    if (an != bn)
        return an ? 1 : -1;
    if (!an) {
        if (a->x > b->x) return -1;
        if (a->x < b->x) return 1;
    }
    return (a->i > b->i) - (a->i < b->i);
}

/*
 * Entropy of the row's softmax distribution, H = -sum_t p_t log p_t with
 * log p_t = x_t - lse (the per-depth entropy that entropy-guided and hybrid
 * scoring rank by: paperlayer.ai JetSpec summary, appendices C and E).  Terms
 * with p_t = 0 contribute 0 (the limit).  NaN if the row holds a NaN; 0 for a
 * row whose every entry is -inf (lse = -inf: no distribution, read as a point).
 */
static double row_entropy(const ora_item *it, int V, double L)
{
    if (isnan(L))
        return NAN;
    if (L == -INFINITY)
        return 0.0;
    double H = 0.0;
    for (int t = 0; t < V; t++) {
        const double lp = it[t].x - L;
        const double p = exp(lp);
        if (p > 0.0)
            H -= p * lp;
    }
    return H;
}

/*
 * Per row: the W largest logits in (value desc, id asc) order, by a full sort
 * of the row; lse = m + log(sum exp(x - m)) over the whole row (m = row max);
 * logprob = x - lse; entropy (optional) as row_entropy.  Row r starts at
 * logits + r*row_stride elements.  A row whose finite maximum is -inf has
 * lse = -inf.
 */
int jto_topw(const void *logits, int64_t row_stride, int rows, int V, int W,
             int dtype, int32_t *ids, double *logprob, double *lse, double *entropy)
{
    if (rows < 0 || V < 1 || W < 1 || W > V || row_stride < V)
        return 2;
    ora_item *it = (ora_item *)malloc(sizeof(ora_item) * (size_t)V);
    if (!it)
        return 3;
    for (int r = 0; r < rows; r++) {
        const int64_t base = (int64_t)r * row_stride;
        double m = -INFINITY;
        int has_nan = 0;
        for (int t = 0; t < V; t++) {
            it[t].x = elem(logits, base + t, dtype);
            it[t].i = t;
            if (isnan(it[t].x)) has_nan = 1;
            else if (it[t].x > m) m = it[t].x;
        }
        double L;
        if (has_nan) {
            L = NAN;
        } else if (m == -INFINITY) {
            L = -INFINITY;
        } else {
            double Z = 0.0;
            for (int t = 0; t < V; t++)
                Z += exp(it[t].x - m);
            L = m + log(Z);
        }
        if (lse)
            lse[r] = L;
        if (entropy)
            entropy[r] = row_entropy(it, V, L);
        qsort(it, (size_t)V, sizeof(ora_item), item_cmp);
        for (int w = 0; w < W; w++) {
            ids[(int64_t)r * W + w] = it[w].i;
            logprob[(int64_t)r * W + w] = it[w].x - L;
        }
    }
    free(it);
    return 0;
}

/* --------------------------------------------------------------- verify -- */

/* first index of the row maximum by a linear scan; NaN entries are skipped */
static int32_t row_argmax(const void *logits, int64_t base, int V, int dtype, int *saw_nan)
{
    int32_t best_i = -1;
    double best = 0.0;
    for (int t = 0; t < V; t++) {
        double x = elem(logits, base + t, dtype);
        if (isnan(x)) { *saw_nan = 1; continue; }
        if (best_i < 0 || x > best) { best = x; best_i = t; }
    }
    return best_i < 0 ? 0 : best_i;
}

/*
 * The verification walk shared by the greedy and sampled rules, given the
 * target's token am[v] at every node (its argmax, or its draw):
 *   v accepted iff every node u != root on the root path of v has
 *              tokens[u] == am[parent[u]];
 *   v*        = deepest accepted node, lowest index on ties (root is always
 *              accepted);
 *   accept_len = depth(v*), path[0..N] = root..v* padded with -1, bonus =
 *   am[v*].  Returns the flags ORA_BAD_PARENT / ORA_DEPTH_GT_N; such a
 *   sequence gets accept_len 0, path [0, -1, ...] and bonus am[0].
 */
static int tree_walk(const int32_t *par, const int32_t *tok, const int32_t *am, int B, int N,
                     int32_t *accept_len, int32_t *path, int32_t *bonus)
{
    for (int k = 0; k <= N; k++)
        path[k] = -1;
    path[0] = 0;
    *accept_len = 0;
    *bonus = am[0];
    if (!parents_valid(par, B))
        return ORA_BAD_PARENT;
    for (int v = 0; v < B; v++) {
        int dv = 0;
        for (int u = v; par[u] != -1; u = par[u])
            dv++;
        if (dv > N)
            return ORA_DEPTH_GT_N;
    }
    int best_v = 0, best_d = 0;
    for (int v = 0; v < B; v++) {
        int ok = 1, dv = 0;
        for (int u = v; par[u] != -1; u = par[u]) {
            if (tok[u] != am[par[u]])
                ok = 0;
            dv++;
        }
        if (ok && dv > best_d) {
            best_d = dv;
            best_v = v;
        }
    }
    *accept_len = best_d;
    for (int u = best_v; u != -1; u = par[u]) {
        int du = 0;
        for (int w = u; par[w] != -1; w = par[w])
            du++;
        path[du] = u;
    }
    *bonus = am[best_v];
    return 0;
}

/*
 * Greedy tree verification: am[s,v] = argmax_t target_logits[s,v,t] (lowest id
 * on ties), then tree_walk.  Row (s, v) of the logits starts at
 * (s*B + v)*row_stride elements.  err[s]: ORA_BAD_PARENT, ORA_DEPTH_GT_N (some
 * node deeper than N), ORA_NAN.
 */
int jto_verify_greedy(const void *target_logits, int64_t row_stride, int V, int dtype,
                      const int32_t *parent, const int32_t *tokens, int S, int B, int N,
                      int32_t *accept_len, int32_t *accept_path, int32_t *bonus,
                      int32_t *argmax, int32_t *err)
{
    if (S < 0 || B < 1 || V < 1 || N < 0 || row_stride < V)
        return 2;
    for (int s = 0; s < S; s++) {
        int32_t *am = argmax + (int64_t)s * B;
        int saw_nan = 0;
        for (int v = 0; v < B; v++)
            am[v] = row_argmax(target_logits, ((int64_t)s * B + v) * row_stride, V, dtype, &saw_nan);
        const int flags = tree_walk(parent + (int64_t)s * B, tokens + (int64_t)s * B, am, B, N,
                                    &accept_len[s], accept_path + (int64_t)s * (N + 1), &bonus[s]);
        err[s] = flags | (saw_nan ? ORA_NAN : 0);
    }
    return 0;
}

/*
 * One draw from softmax(x / T) by the inverse of its cumulative distribution
 * in token-id order: the first t whose cumulative weight exceeds r * Z, with
 * weights e_t = exp((x_t - m) / T) (m = row maximum, Z = their sum).  NaN
 * entries weigh 0 and set *saw_nan (the greedy rule skips them too).  A row
 * with no finite maximum gives token 0, like the argmax of such a row.
 * *margin = the distance of r * Z from the nearer end of the drawn token's
 * interval, divided by Z (how far the draw is from going to a neighbour).
 */
static int32_t row_sample(const void *logits, int64_t base, int V, int dtype, double T, double r,
                          int *saw_nan, double *margin)
{
    double m = -INFINITY;
    for (int t = 0; t < V; t++) {
        double x = elem(logits, base + t, dtype);
        if (isnan(x)) { *saw_nan = 1; continue; }
        if (x > m) m = x;
    }
    if (m == -INFINITY) {
        *margin = INFINITY;
        return 0;
    }
    double Z = 0.0;
    for (int t = 0; t < V; t++) {
        double x = elem(logits, base + t, dtype);
        if (!isnan(x))
            Z += exp((x - m) / T);
    }
    const double target = r * Z;
    double cum = 0.0;
    int32_t last = 0;
    for (int t = 0; t < V; t++) {
        double x = elem(logits, base + t, dtype);
        if (isnan(x))
            continue;
        const double e = exp((x - m) / T);
        if (e > 0.0)
            last = t;
        const double prev = cum;
        cum += e;
        if (cum > target) {
            *margin = fmin(target - prev, cum - target) / Z;
            return t;
        }
    }
    *margin = 0.0;
    return last;
}

/*
 * Stochastic tree verification at temperature T > 0.  The target's own draw
 * decides every position: with a fixed draft every proposal is a point mass at
 * the draft token, accepted with the target probability, and after a
 * rejection the next token comes from the residual (JetSpec review, inference,
 * acceptance equation; JetSpec++ summary, appendices F.1 and F.3).  Sibling
 * tokens are distinct, so trying the children of a node one by one that way
 * is the same in distribution as drawing one token x ~ softmax(logits / T) at
 * the node and descending to the child carrying x, or stopping with bonus x.
 * This function does the latter: am[s,v] = row_sample(row (s,v), uniform[s,v])
 * for every node, then tree_walk.  margin (optional) [S,B] receives each
 * draw's margin.  err[s]: as for jto_verify_greedy.
 */
int jto_verify_sampled(const void *target_logits, int64_t row_stride, int V, int dtype,
                       double T, const double *uniform, const int32_t *parent,
                       const int32_t *tokens, int S, int B, int N, int32_t *accept_len,
                       int32_t *accept_path, int32_t *bonus, int32_t *sample, double *margin,
                       int32_t *err)
{
    if (S < 0 || B < 1 || V < 1 || N < 0 || row_stride < V || !(T > 0.0))
        return 2;
    for (int s = 0; s < S; s++) {
        int32_t *am = sample + (int64_t)s * B;
        int saw_nan = 0;
        for (int v = 0; v < B; v++) {
            double mg;
            am[v] = row_sample(target_logits, ((int64_t)s * B + v) * row_stride, V, dtype, T,
                               uniform[(int64_t)s * B + v], &saw_nan, &mg);
            if (margin)
                margin[(int64_t)s * B + v] = mg;
        }
        const int flags = tree_walk(parent + (int64_t)s * B, tokens + (int64_t)s * B, am, B, N,
                                    &accept_len[s], accept_path + (int64_t)s * (N + 1), &bonus[s]);
        err[s] = flags | (saw_nan ? ORA_NAN : 0);
    }
    return 0;
}

/* ------------------------------------------------------- tree construction -- */

/*
 * Does node (a, ia) leave the queue before node (b, ib)?  Larger score first,
 * then the lower node index; a NaN score ranks below every other score (the
 * top-W reading).  -0 equals +0.
 */
static int pops_before(float a, int ia, float b, int ib)
{
    int an = isnan(a), bn = isnan(b);
    if (an != bn)
        return bn;
    if (!an && a != b)
        return a > b;
    return ia < ib;
}

/*
 * Best-first construction of the draft tree from the per-depth candidate lists
 * (paperlayer.ai JetSpec summary, appendix B "Tree-Drafting Algorithm Details"
 * and appendix E "Drafting"; review of JetSpec, "inference", the path-score
 * equation; paper.rainbus.top summary, method steps).  The root (node 0, depth
 * 0, score 0) starts in the queue.  Repeatedly the queued node that pops first
 * (pops_before) leaves the queue; a node at depth N is not expanded; otherwise
 * it gains up to W children, rank r = 0..W-1 in order, while the tree holds
 * fewer than B nodes.  Child r of a node at depth d carries token ids[d][r] of
 * its sequence (row d gives the candidates for depth d+1, shared by every node
 * at depth d) and the score
 *     score(parent) + (w_lp * logprob[d][r] - w_ent * entropy[d]),
 * each product, the difference and the sum rounded to float in that order (the
 * scores decide integers, so they are accumulated in the precision the device
 * path uses).  w_lp = 1, w_ent = 0 is the cumulative log-probability of the
 * path; w_lp = 0, w_ent = 1 scores by per-depth entropy alone; w_lp = 1,
 * w_ent = alpha is the hybrid (appendix C of the same summary names all three;
 * the combination is a reading).  entropy may be NULL (taken as 0).
 * Construction ends when B nodes exist or the queue is empty; then slots
 * n..B-1 are padding: parent 0, token -1, score -inf.
 *
 *   ids, logprob  [S*N, W]     entropy [S*N] or NULL   root_token [S] or NULL (-1)
 *   parent, tokens [S, B]      score [S, B] or NULL     n_nodes [S] or NULL
 */
int jto_build_tree(const int32_t *ids, const float *logprob, const float *entropy,
                   float w_lp, float w_ent, const int32_t *root_token, int S, int N,
                   int W, int B, int32_t *parent, int32_t *tokens, float *score,
                   int32_t *n_nodes)
{
    if (S < 0 || N < 0 || W < 1 || B < 1)
        return 2;
    float *sc = (float *)malloc(sizeof(float) * (size_t)B);
    int *dep = (int *)malloc(sizeof(int) * (size_t)B);
    int *queued = (int *)malloc(sizeof(int) * (size_t)B);
    if (!sc || !dep || !queued) {
        free(sc); free(dep); free(queued);
        return 3;
    }
    for (int s = 0; s < S; s++) {
        int32_t *par = parent + (int64_t)s * B, *tok = tokens + (int64_t)s * B;
        par[0] = -1;
        tok[0] = root_token ? root_token[s] : -1;
        sc[0] = 0.0f;
        dep[0] = 0;
        queued[0] = 1;
        int n = 1;
        while (n < B) {
            int v = -1;
            for (int i = 0; i < n; i++)
                if (queued[i] && (v < 0 || pops_before(sc[i], i, sc[v], v)))
                    v = i;
            if (v < 0)
                break;
            queued[v] = 0;
            if (dep[v] >= N)
                continue;
            const int64_t row = (int64_t)s * N + dep[v];
            const float h = entropy ? entropy[row] : 0.0f;
            const float eterm = w_ent * h;
            for (int r = 0; r < W && n < B; r++) {
                const float lterm = w_lp * logprob[row * W + r];
                const float inc = lterm - eterm;
                par[n] = v;
                tok[n] = ids[row * W + r];
                dep[n] = dep[v] + 1;
                sc[n] = sc[v] + inc;
                queued[n] = 1;
                n++;
            }
        }
        if (n_nodes)
            n_nodes[s] = n;
        for (int i = n; i < B; i++) {
            par[i] = 0;
            tok[i] = -1;
            sc[i] = -INFINITY;
        }
        if (score)
            for (int i = 0; i < B; i++)
                score[(int64_t)s * B + i] = sc[i];
    }
    free(sc); free(dep); free(queued);
    return 0;
}

/* ------------------------------------------------------ accepted-path commit -- */

/*
 * After verification the accepted root path becomes part of the prefix: the
 * verifier commits the longest accepted prefix (paperlayer.ai JetSpec summary,
 * section 2; JetSpec++ summary, section 3), whose keys and values this pass
 * already computed in the tree buffers.  Node 0 is the root (the last
 * committed token, computed in this pass), so path nodes path[0..L] (L =
 * accept_len[s], path[0] = 0) are written to prefix positions P .. P + L of
 * sequence s, P = prefix_len[s]; node path[i] has depth i, so its rotary
 * position P + i is its slot and nothing is re-rotated.  new_prefix_len[s] =
 * P + L + 1.  Plain byte copies of each (position, KV head) row of d elements.
 *
 * Cache layout: contiguous [S, max_prefix, Hkv, d] when block_table is NULL,
 * else paged [num_blocks, block_size, Hkv, d] with position j of sequence s in
 * block block_table[s*max_blocks + j/block_size], row j % block_size.
 * Flags per sequence (err, optional): accept_len outside [0, N] -> DEPTH_GT_N
 * (2), nothing written; P < 0 or P + L + 1 beyond the capacity (max_prefix, or
 * max_blocks * block_size) -> BAD_PREFIX (16), nothing written; a path entry
 * outside [0, B) -> BAD_PARENT (1), that row skipped; a block id outside
 * [0, num_blocks) -> BAD_BLOCK (4), that row skipped.  A flagged sequence
 * keeps new_prefix_len = P.
 */
int jto_commit_kv(const int32_t *accept_len, const int32_t *accept_path, int N,
                  const void *k_tree, const void *v_tree, int S, int B, int Hkv, int d,
                  int elem_bytes, void *k_cache, void *v_cache,
                  const int32_t *block_table, int max_blocks, int block_size,
                  int num_blocks, const int32_t *prefix_len, int max_prefix,
                  int32_t *new_prefix_len, int32_t *err)
{
    if (S < 0 || B < 1 || N < 0 || Hkv < 1 || d < 1 || (elem_bytes != 2 && elem_bytes != 4))
        return 2;
    const size_t row = (size_t)d * (size_t)elem_bytes;
    for (int s = 0; s < S; s++) {
        int flag = 0;
        const int L = accept_len[s];
        const int P = prefix_len[s];
        const long cap = block_table ? (long)max_blocks * block_size : (long)max_prefix;
        int committed = 0;
        if (L < 0 || L > N) {
            flag |= 2;
        } else if (P < 0 || (long)P + L + 1 > cap) {
            flag |= 16;
        } else {
            committed = 1;
            for (int i = 0; i <= L; i++) {
                const int v = accept_path[(int64_t)s * (N + 1) + i];
                if (v < 0 || v >= B) {
                    flag |= 1;
                    continue;
                }
                const long j = (long)P + i;
                int64_t slot;  /* (position or pool row) whose Hkv rows are written */
                if (block_table) {
                    const int blk = block_table[(int64_t)s * max_blocks + j / block_size];
                    if (blk < 0 || blk >= num_blocks) {
                        flag |= 4;
                        continue;
                    }
                    slot = (int64_t)blk * block_size + j % block_size;
                } else {
                    slot = (int64_t)s * max_prefix + j;
                }
                for (int g = 0; g < Hkv; g++) {
                    const int64_t src = (((int64_t)s * B + v) * Hkv + g) * (int64_t)row;
                    const int64_t dst = (slot * Hkv + g) * (int64_t)row;
                    memcpy((char *)k_cache + dst, (const char *)k_tree + src, row);
                    memcpy((char *)v_cache + dst, (const char *)v_tree + src, row);
                }
            }
        }
        if (new_prefix_len)
            new_prefix_len[s] = (committed && !flag) ? P + L + 1 : P;
        if (err)
            err[s] = flag;
    }
    return 0;
}
