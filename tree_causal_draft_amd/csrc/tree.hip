// Best-first construction of the draft tree from the per-depth candidate lists.
//
// The tree grows by repeatedly popping the queued node with the highest path score and
// giving it up to W children, until the node budget is spent; nodes at the maximum depth
// are not expanded (paperlayer.ai JetSpec summary, appendix B "Tree-Drafting Algorithm
// Details" and section 2; the JetSpec review's inference section, path-score equation;
// paper.rainbus.top summary, method steps).  The candidates of depth d+1 are one list
// shared by every node at depth d (paperlayer.ai JetSpec summary, appendix E
// "Drafting"), so a child's score is its parent's plus a per-(depth, rank) increment.
//
// One wave per sequence.  The queue is never materialised as a heap: lane L keeps the
// score, depth and queued bit of nodes L, L+64, L+128, L+192 in registers, and a pop is
// one wave-wide maximum of 32-bit order codes (DPP) over each lane's best slot (found, with
// its score and depth, beside the reduction), then one ballot for the lane holding it (a
// tie between lanes takes three more, by slot, for the lowest node index).  An expansion creates at most 16 children, so
// each lane owns at most one of them and computes its score itself from the increment
// table in LDS: a pop moves no data between lanes beyond the popped node's score and
// depth.  Parent and token stay in registers until the end.  Pops are inherently
// sequential (a child may outrank every queued node), so the kernel is bound by the
// latency of one pop, about a hundred dependent instructions (0.3 us measured).  Nodes at
// the depth limit are never queued: their pops would expand nothing.
#include "jt_internal.h"

namespace jt {

constexpr int kTreeSlots = JT_MAX_NODES / kWave;     // nodes per lane
constexpr int kTreeMaxDepth = 255;                   // N limit
constexpr int kTreeTable = kTreeMaxDepth * JT_MAX_W; // (depth, rank) entries in LDS

struct TreeArgs {
    const int32_t *ids;
    const float *logprob;
    const float *entropy;
    float w_lp, w_ent;
    const int32_t *root_token;
    int S, N, W, B;
    int32_t *parent, *tokens;
    float *score;
    int32_t *n_nodes;
};

// The increment of child rank r at depth d + 1: each product, then the difference, is
// rounded to float on its own (no fused multiply-add), the order the scores are defined in.
__device__ __forceinline__ float tree_increment(float w_lp, float lp, float w_ent, float h)
{
#pragma clang fp contract(off)
    const float lterm = w_lp * lp;
    const float eterm = w_ent * h;
    return lterm - eterm;
}
__device__ __forceinline__ float tree_add(float a, float b)
{
#pragma clang fp contract(off)
    return a + b;
}

// Pop order as a 32-bit code: larger score first, NaN below every other score, 0 for a
// slot that is not queued.  Equal codes pop by node index.
__device__ __forceinline__ uint32_t tree_key(bool queued, float sc)
{
    return queued ? order_code(sc) + 1u : 0u;
}

__global__ void __launch_bounds__(64) tree_build_kernel(TreeArgs a)
{
    __shared__ float inc[kTreeTable];
    __shared__ int32_t cid[kTreeTable];
    const int s = blockIdx.x, lane = threadIdx.x;
    const int N = a.N, W = a.W, B = a.B;
    const int64_t tb = (int64_t)s * N * W;
    for (int i = lane; i < N * W; i += kWave) {
        const int d = i / W;
        const float h = a.entropy ? a.entropy[(int64_t)s * N + d] : 0.f;
        inc[i] = tree_increment(a.w_lp, a.logprob[tb + i], a.w_ent, h);
        cid[i] = a.ids[tb + i];
    }
    __syncthreads();

    // lane state: node lane + 64k in slot k -- score, depth, pop key (0: not queued),
    // parent and token (stored once at the end)
    float sc[kTreeSlots];
    int dp[kTreeSlots], pa[kTreeSlots], tk[kTreeSlots];
    uint32_t key[kTreeSlots];
#pragma unroll
    for (int k = 0; k < kTreeSlots; ++k) {
        sc[k] = -INFINITY;
        dp[k] = 0;
        pa[k] = 0;
        tk[k] = -1;
        key[k] = 0u;
    }
    if (lane == 0) {
        sc[0] = 0.f;
        pa[0] = -1;
        tk[0] = a.root_token ? a.root_token[s] : -1;
        key[0] = tree_key(true, 0.f);
    }
    int n = 1;
    while (n < B) {
        // the lane's best queued slot (lowest slot on equal keys) with its score and depth,
        // found while the wave maximum runs
        uint32_t best = key[0];
        int bslot = 0;
        float bsc = sc[0];
        int bdp = dp[0];
#pragma unroll
        for (int k = 1; k < kTreeSlots; ++k) {
            const bool gt = key[k] > best;
            best = gt ? key[k] : best;
            bslot = gt ? k : bslot;
            bsc = gt ? sc[k] : bsc;
            bdp = gt ? dp[k] : bdp;
        }
        const uint32_t M = wave_max_u32(best);
        if (M == 0u)
            break;  // queue empty
        // the lowest node index holding M: one ballot when a single lane holds it; on a tie
        // between lanes, the lowest slot first (lower slot, lower index), then the lowest lane
        static_assert(kTreeSlots == 4, "four slots per lane");
        const uint64_t hit = __ballot(best == M);
        int ln;
        if (__popcll(hit) == 1) {
            ln = (int)__builtin_ctzll(hit);
        } else {
            const uint64_t b0 = __ballot(best == M && bslot == 0),
                           b1 = __ballot(best == M && bslot == 1),
                           b2 = __ballot(best == M && bslot == 2);
            ln = (int)__builtin_ctzll(b0 ? b0 : b1 ? b1 : b2 ? b2 : hit);
        }
        const int kk = __builtin_amdgcn_readlane(bslot, ln);
        const int v = ln + kWave * kk;
        const float sv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bsc), ln));
        const int dv = __builtin_amdgcn_readlane(bdp, ln);
        if (lane == ln) {
#pragma unroll
            for (int k = 0; k < kTreeSlots; ++k)
                if (k == kk)
                    key[k] = 0u;
        }
        if (dv >= N)
            continue;  // at the depth limit: popped, not expanded (only the root when N = 0)
        // children n .. n+cnt-1; cnt <= 16, so a lane receives at most one of them
        const int cnt = min(W, B - n);
        const int r = (lane - n) & (kWave - 1);
        if (r < cnt) {
            const int e = dv * W + r;
            const float cs = tree_add(sv, inc[e]);
            const int ct = cid[e];
            const int k = (n + r) >> 6;
            // a child at the depth limit is never expanded, so its pop would change nothing:
            // it is not queued at all, and the pops that remain are the same, in order
            const uint32_t ck = tree_key(dv + 1 < N, cs);
#pragma unroll
            for (int q = 0; q < kTreeSlots; ++q) {
                const bool at = q == k;  // selects, not a branch per slot
                sc[q] = at ? cs : sc[q];
                dp[q] = at ? dv + 1 : dp[q];
                key[q] = at ? ck : key[q];
                pa[q] = at ? v : pa[q];
                tk[q] = at ? ct : tk[q];
            }
        }
        n += cnt;
    }
    if (lane == 0 && a.n_nodes)
        a.n_nodes[s] = n;
    int32_t *par = a.parent + (int64_t)s * B;
    int32_t *tok = a.tokens + (int64_t)s * B;
#pragma unroll
    for (int k = 0; k < kTreeSlots; ++k) {
        const int idx = lane + kWave * k;
        if (idx >= B)
            continue;
        // slots at or past n keep their initial padding: parent 0, token -1, score -inf
        par[idx] = pa[k];
        tok[idx] = tk[k];
        if (a.score)
            a.score[(int64_t)s * B + idx] = sc[k];
    }
}

jt_status launch_build_tree(const int32_t *ids, const float *logprob, const float *entropy,
                            float w_lp, float w_ent, const int32_t *root_token, int S, int N,
                            int W, int B, int32_t *parent, int32_t *tokens, float *score,
                            int32_t *n_nodes, hipStream_t st)
{
    if (S == 0)
        return JT_OK;
    TreeArgs a{ids, logprob, entropy, w_lp, w_ent, root_token, S, N, W, B,
               parent, tokens, score, n_nodes};
    hipLaunchKernelGGL(tree_build_kernel, dim3(S), dim3(kWave), 0, st, a);
    return launch_status(hipGetLastError());
}

} // namespace jt
