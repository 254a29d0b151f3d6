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
// one wave-wide maximum of 32-bit order codes (DPP) followed by at most four ballots that
// find the lowest node index holding it.  The owners of the new children compute their
// scores themselves from the increment table in LDS, so a pop moves no data between
// lanes beyond the popped node's score and depth.  Pops are inherently sequential (a
// child may outrank every queued node), so the kernel is bound by the latency of one
// pop, about a hundred dependent instructions.
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
    int32_t *par = a.parent + (int64_t)s * B;
    int32_t *tok = a.tokens + (int64_t)s * B;
    if (lane == 0) {
        par[0] = -1;
        tok[0] = a.root_token ? a.root_token[s] : -1;
    }
    __syncthreads();

    float sc[kTreeSlots];
    int dp[kTreeSlots];
    bool q[kTreeSlots];
#pragma unroll
    for (int k = 0; k < kTreeSlots; ++k) {
        sc[k] = -INFINITY;
        dp[k] = 0;
        q[k] = false;
    }
    if (lane == 0) {
        sc[0] = 0.f;
        q[0] = true;
    }
    int n = 1;
    while (n < B) {
        uint32_t key[kTreeSlots], mine = 0u;
#pragma unroll
        for (int k = 0; k < kTreeSlots; ++k) {
            key[k] = tree_key(q[k], sc[k]);
            mine = max(mine, key[k]);
        }
        const uint32_t M = wave_max_u32(mine);
        if (M == 0u)
            break;  // queue empty
        // the lowest node index holding M: slot k first (lower k, lower index), then lane
        int kk = kTreeSlots - 1;
        uint64_t hit = 0ull;
#pragma unroll
        for (int k = 0; k < kTreeSlots; ++k) {
            const uint64_t b = __ballot(key[k] == M);
            if (hit == 0ull && b != 0ull) {
                hit = b;
                kk = k;
            }
        }
        const int ln = (int)__builtin_ctzll(hit);
        const int v = ln + kWave * kk;
        float s_sel = sc[0];
        int d_sel = dp[0];
#pragma unroll
        for (int k = 1; k < kTreeSlots; ++k)
            if (k == kk) {
                s_sel = sc[k];
                d_sel = dp[k];
            }
        const float sv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s_sel), ln));
        const int dv = __builtin_amdgcn_readlane(d_sel, ln);
#pragma unroll
        for (int k = 0; k < kTreeSlots; ++k)
            if (k == kk && lane == ln)
                q[k] = false;
        if (dv >= N)
            continue;  // at the depth limit: popped, not expanded
        const int cnt = min(W, B - n);
        const int row = dv * W;
#pragma unroll
        for (int k = 0; k < kTreeSlots; ++k) {
            const int idx = lane + kWave * k;
            const int r = idx - n;
            if (r >= 0 && r < cnt) {
                sc[k] = tree_add(sv, inc[row + r]);
                dp[k] = dv + 1;
                q[k] = true;
                par[idx] = v;
                tok[idx] = cid[row + r];
            }
        }
        n += cnt;
    }
    if (lane == 0 && a.n_nodes)
        a.n_nodes[s] = n;
#pragma unroll
    for (int k = 0; k < kTreeSlots; ++k) {
        const int idx = lane + kWave * k;
        if (idx >= B)
            continue;
        if (idx >= n) {
            par[idx] = 0;
            tok[idx] = -1;
        }
        if (a.score)
            a.score[(int64_t)s * B + idx] = idx < n ? sc[k] : -INFINITY;
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
