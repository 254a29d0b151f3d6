// Accepted-path commit: the keys and values of the accepted root path join the prefix.
//
// The verifier commits the longest accepted root path (paperlayer.ai JetSpec summary,
// section 2; JetSpec++ summary, section 3), whose K/V this pass already computed in the
// tree buffers.  Node 0 is the root, the last committed token, so path nodes path[0..L]
// become prefix positions P..P+L and the prefix grows to P+L+1.  A node at depth i has
// rotary position P + i, which is exactly its slot: nothing is re-rotated.
//
// One workgroup per sequence.  It reads the sequence's length and path first and writes
// the new length last, so the length may be updated in place, and it ORs its flags in
// LDS.  The copy is a gather of (position, KV head) rows of d elements in 16-byte pieces
// (d = 64 or 128: every row is a whole number of pieces): at most (N+1) * Hkv * d * e * 2
// bytes per sequence, bound by the latency of one dependent round trip (path entry, then
// block id, then the copy).
#include "jt_internal.h"

namespace jt {

struct CommitArgs {
    const int32_t *accept_len, *accept_path;
    int N;
    const uint8_t *k_tree, *v_tree;
    int S, B, Hkv, row_bytes;  // row_bytes = d * element size, a multiple of 16
    uint8_t *k_cache, *v_cache;
    const int32_t *block_table;
    int max_blocks, block_size, num_blocks;
    const int32_t *prefix_len;
    int max_prefix;
    int32_t *new_prefix_len, *err;
};

__global__ void __launch_bounds__(256) commit_kv_kernel(CommitArgs a)
{
    __shared__ int sflag;
    const int s = blockIdx.x, tid = threadIdx.x;
    if (tid == 0)
        sflag = 0;
    const int L = a.accept_len[s];
    const int P = a.prefix_len[s];
    const long cap = a.block_table ? (long)a.max_blocks * a.block_size : (long)a.max_prefix;
    int flag = 0;
    if (L < 0 || L > a.N)
        flag = JT_DEV_DEPTH_GT_N;
    else if (P < 0 || (long)P + L + 1 > cap)
        flag = JT_DEV_BAD_PREFIX;
    __syncthreads();
    if (flag == 0) {
        const int qn = a.row_bytes >> 4;  // 16-byte pieces per row
        const int total = (L + 1) * a.Hkv * qn;
        const int32_t *path = a.accept_path + (int64_t)s * (a.N + 1);
        int f = 0;
        for (int u = tid; u < total; u += blockDim.x) {
            const int q = u % qn, t = u / qn;
            const int g = t % a.Hkv, i = t / a.Hkv;
            const int v = path[i];
            if (v < 0 || v >= a.B) {
                f |= JT_DEV_BAD_PARENT;
                continue;
            }
            const long j = (long)P + i;
            int64_t slot;
            if (a.block_table) {
                const int blk = a.block_table[(int64_t)s * a.max_blocks + j / a.block_size];
                if (blk < 0 || blk >= a.num_blocks) {
                    f |= JT_DEV_BAD_BLOCK;
                    continue;
                }
                slot = (int64_t)blk * a.block_size + j % a.block_size;
            } else {
                slot = (int64_t)s * a.max_prefix + j;
            }
            const int64_t src = (((int64_t)s * a.B + v) * a.Hkv + g) * a.row_bytes + q * 16;
            const int64_t dst = (slot * a.Hkv + g) * a.row_bytes + q * 16;
            const uint4 kk = *reinterpret_cast<const uint4 *>(a.k_tree + src);
            const uint4 vv = *reinterpret_cast<const uint4 *>(a.v_tree + src);
            *reinterpret_cast<uint4 *>(a.k_cache + dst) = kk;
            *reinterpret_cast<uint4 *>(a.v_cache + dst) = vv;
        }
        if (f)
            atomicOr(&sflag, f);
    }
    __syncthreads();
    if (tid == 0) {
        flag |= sflag;
        if (a.err)
            a.err[s] = flag;
        a.new_prefix_len[s] = flag == 0 ? P + L + 1 : P;
    }
}

jt_status launch_commit_kv(const int32_t *accept_len, const int32_t *accept_path, int N,
                           const void *k_tree, const void *v_tree, int S, int B, int Hkv, int d,
                           int elem_bytes, void *k_cache, void *v_cache,
                           const int32_t *block_table, int max_blocks, int block_size,
                           int num_blocks, const int32_t *prefix_len, int max_prefix,
                           int32_t *new_prefix_len, int32_t *err, hipStream_t st)
{
    if (S == 0)
        return JT_OK;
    CommitArgs a;
    a.accept_len = accept_len;
    a.accept_path = accept_path;
    a.N = N;
    a.k_tree = static_cast<const uint8_t *>(k_tree);
    a.v_tree = static_cast<const uint8_t *>(v_tree);
    a.S = S;
    a.B = B;
    a.Hkv = Hkv;
    a.row_bytes = d * elem_bytes;
    a.k_cache = static_cast<uint8_t *>(k_cache);
    a.v_cache = static_cast<uint8_t *>(v_cache);
    a.block_table = block_table;
    a.max_blocks = max_blocks;
    a.block_size = block_size;
    a.num_blocks = num_blocks;
    a.prefix_len = prefix_len;
    a.max_prefix = max_prefix;
    a.new_prefix_len = new_prefix_len;
    a.err = err;
    hipLaunchKernelGGL(commit_kv_kernel, dim3(S), dim3(256), 0, st, a);
    return launch_status(hipGetLastError());
}

} // namespace jt
