// Step 1: parent array -> 256-bit ancestor rows and depths, one workgroup per sequence.
//
// The tree-causal mask keeps M[v,u] = 0 exactly for the ancestors of v and v itself
// (JetSpec review, startedourmission.github.io, "How it works", mask equation), and the
// verifier needs depths next to it (paperlayer.ai JetSpec summary, appendix E).
//
// Pointer doubling in LDS: node v keeps a jump pointer j(v), the set R(v) of nodes on the
// path from v up to j(v) (exclusive) as a 256-bit row, and the number of edges covered.
// Each round merges the row of the jump target and doubles the jump:
//   R(v) |= R(j(v)), dist(v) += dist(j(v)), j(v) = j(j(v)).
// After ceil(log2 B) <= 8 rounds every jump has reached past the root, so R(v) is the
// ancestor row of v (itself included) and dist(v) its depth.
#include "jt_internal.h"

namespace jt {

// Rows and depths of sequence s by one workgroup of at least B threads (thread v = node v);
// `row`, `jmp`, `dist` are JT_MAX_NODES entries of LDS.
__device__ __forceinline__ void mask_block(const int32_t *__restrict__ parent, int B, uint64_t *__restrict__ anc,
                           int32_t *__restrict__ depth, int32_t *__restrict__ err, int s,
                           uint64_t (*row)[4], int32_t *jmp, int32_t *dist)
{
    const int v = threadIdx.x;
    const int32_t *par = parent + (int64_t)s * B;

    int p = -1;
    int bad = 0;
    if (v < B) {
        p = par[v];
        bad = (v == 0) ? (p != -1) : (p < 0 || p >= v);
    }
    bad = __syncthreads_or(bad);
    uint64_t *arow = anc + ((int64_t)s * B + v) * 4;
    if (bad) {
        if (v < B) {
            arow[0] = arow[1] = arow[2] = arow[3] = 0ull;
            depth[(int64_t)s * B + v] = -1;
        }
        if (v == 0 && err)
            err[s] = JT_DEV_BAD_PARENT;
        return;
    }
    if (v < B) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
            row[v][w] = (w == (v >> 6)) ? (1ull << (v & 63)) : 0ull;
        jmp[v] = p;
        dist[v] = (p >= 0) ? 1 : 0;
    }
    __syncthreads();
    // ceil(log2(B)) rounds suffice: after k rounds a jump covers 2^k edges.
    int rounds = 0;
    while ((1 << rounds) < B)
        ++rounds;
    for (int r = 0; r < rounds; ++r) {
        uint64_t r0 = 0, r1 = 0, r2 = 0, r3 = 0;
        int nj = -1, nd = 0;
        const bool act = v < B && jmp[v] >= 0;
        if (act) {
            const int j = jmp[v];
            r0 = row[v][0] | row[j][0];
            r1 = row[v][1] | row[j][1];
            r2 = row[v][2] | row[j][2];
            r3 = row[v][3] | row[j][3];
            nd = dist[v] + dist[j];
            nj = jmp[j];
        }
        __syncthreads();
        if (act) {
            row[v][0] = r0;
            row[v][1] = r1;
            row[v][2] = r2;
            row[v][3] = r3;
            dist[v] = nd;
            jmp[v] = nj;
        }
        __syncthreads();
    }
    if (v < B) {
        arow[0] = row[v][0];
        arow[1] = row[v][1];
        arow[2] = row[v][2];
        arow[3] = row[v][3];
        depth[(int64_t)s * B + v] = dist[v];
    }
    if (v == 0 && err)
        err[s] = 0;
}

__global__ void __launch_bounds__(256) build_mask_kernel(const int32_t *__restrict__ parent, int B,
                                                         uint64_t *__restrict__ anc,
                                                         int32_t *__restrict__ depth,
                                                         int32_t *__restrict__ err)
{
    __shared__ uint64_t row[JT_MAX_NODES][4];
    __shared__ int32_t jmp[JT_MAX_NODES];
    __shared__ int32_t dist[JT_MAX_NODES];
    mask_block(parent, B, anc, depth, err, blockIdx.x, row, jmp, dist);
}

jt_status launch_build_mask(const int32_t *parent, int S, int B, uint64_t *anc, int32_t *depth,
                            int32_t *err, hipStream_t st)
{
    if (S == 0)
        return JT_OK;
    hipLaunchKernelGGL(build_mask_kernel, dim3(S), dim3(256), 0, st, parent, B, anc, depth, err);
    return launch_status(hipGetLastError());
}

} // namespace jt
