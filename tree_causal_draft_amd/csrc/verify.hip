// Step 4: greedy tree verification -- target argmax per node, then the accepted path.
//
// The verifier commits the longest root path whose draft tokens pass acceptance plus a
// bonus token (paperlayer.ai JetSpec summary, section 2; JetSpec++ summary, section 3).
// At temperature 0 the test min(1, p/q) of the review's inference section, with a
// point-mass draft (JetSpec++ summary, appendix F.3), is token == argmax at the parent.
//
// Phase 1 (HBM-bound, the bulk of the bytes): arg-max of every target row.  A row is cut
// into runs of 8192-logit sub-chunks, one workgroup per run, so a handful of rows still
// fills the chip while 2048 rows stream whole.  Threads walk their logits in increasing
// id order with a strict '>' so each keeps the first maximum; the workgroup then takes
// the largest 64-bit key (order code << 32 | ~id): largest value, lowest id.
// Phase 2 (one workgroup per sequence, thread v = node v; every global read is issued
// in one batch, the partial keys fold into LDS with 64-bit atomic max):
//   ok bits     ok[v] = tokens[v] == am[parent[v]] (root ok), one ballot per 64 nodes;
//   accepted(v) (anc[v] & ~ok) == 0 -- every node on the root path is ok;
//   v*          block max of (depth << 16 | 65535 - v) over accepted nodes;
//   path        node u with bit u set in anc[v*] writes path[depth[u]] = u.
#include "jt_internal.h"

namespace jt {

constexpr int kArgThreads = 256;
constexpr int kArgSub = 8192;
constexpr int kArgMaxChunks = 64;

template <typename T> struct AVec;
template <> struct AVec<uint16_t> { static constexpr int kElems = 8; };
template <> struct AVec<float> { static constexpr int kElems = 4; };

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// Partial arg-max of (row, chunk) `vb` by a workgroup of NT threads; `wkey` / `wnan` hold
// NT / 64 entries of LDS.  Two passes keep the per-logit work small: the scan keeps only
// each thread's maximum (NaN skipped; a packed 16-bit maximum of the magnitudes detects
// NaN) and the sub-chunk where it first reached it; after a block-wide maximum M, the
// threads holding M re-read that sub-chunk (an L2 hit; the last one is still in
// registers) for their first index of M, and a block-wide minimum gives the lowest.  With no value above -inf the chunk's first
// element stands (a row of -inf keeps its first id).
// kPrefetch: the next sub-chunk's loads are issued while one is reduced (for a role that
// runs at few waves per SIMD; with many waves resident the copies already overlap).
template <typename T, bool kAligned, int NT, bool kPrefetch = true>
__device__ __forceinline__ void argmax_partial_block(const T *__restrict__ logits, int64_t row_stride, int V,
                                     int nsub, int sub_per_wg, int nchunk,
                                     uint64_t *__restrict__ ws_keys, uint32_t *__restrict__ ws_nan,
                                     int vb, uint64_t *wkey, uint32_t *wnan)
{
    constexpr int E = AVec<T>::kElems;
    constexpr int L = kArgSub / (E * NT);  // loads of 16 bytes per thread per sub-chunk
    constexpr int NW = NT / 64;
    static_assert(L * E * NT == kArgSub, "sub-chunk split");
    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int row_idx = vb / nchunk;
    const int chunk = vb % nchunk;
    const T *row = logits + (int64_t)row_idx * row_stride;
    const int sc0 = chunk * sub_per_wg;
    const int sc1 = min(nsub, sc0 + sub_per_wg);

    // raw words of a thread's share of one sub-chunk (entries at or past V are not read)
    auto load_sub = [&](int sc, uint4 (&u)[L]) {
        const int64_t base = (int64_t)sc * kArgSub;
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const int64_t e0 = base + (int64_t)(tid + NT * i) * E;
            if (kAligned && e0 + E <= V) {
                u[i] = *reinterpret_cast<const uint4 *>(row + e0);
            } else {
                uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    const int64_t e = e0 + k;
                    if (e < V) {
                        if constexpr (sizeof(T) == 2)
                            w[k >> 1] |= (uint32_t)row[e] << (16 * (k & 1));
                        else
                            w[k] = __float_as_uint(row[e]);
                    }
                }
                u[i] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    };
    auto unpack = [](const uint4 &u, float (&x)[E]) {
        if constexpr (sizeof(T) == 2) {
            x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
            x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z); x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
        } else {
            x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
            x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
        }
    };

    float best = -INFINITY;  // thread maximum, NaN skipped
    int sc_best = -1;        // sub-chunk where it was first reached (-1: nothing above -inf)
    u16x2_t mag = {0, 0};    // bf16: maximum of the magnitude bits (NaN iff > 0x7f80)
    uint32_t magf = 0u;      // fp32: the same on 32-bit words (NaN iff > 0x7f800000)
    uint4 u[L];  // after the scan: the words of the last sub-chunk
    uint4 un[L];  // the next sub-chunk's words, loaded while this one is reduced
    if (kPrefetch && sc0 < sc1)
        load_sub(sc0, un);
    for (int sc = sc0; sc < sc1; ++sc) {
        const int64_t base = (int64_t)sc * kArgSub;
        if constexpr (kPrefetch) {
#pragma unroll
            for (int i = 0; i < L; ++i)
                u[i] = un[i];
            if (sc + 1 < sc1)
                load_sub(sc + 1, un);
        } else {
            load_sub(sc, u);
        }
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const int64_t e0 = base + (int64_t)(tid + NT * i) * E;
            float x[E];
            unpack(u[i], x);
            if (e0 + E <= V) {
#pragma unroll
                for (int k = 0; k < E; ++k)
                    m = fmaxf(m, x[k]);
                if constexpr (sizeof(T) == 2) {
                    mag = __builtin_elementwise_max(mag, __builtin_bit_cast(u16x2_t, u[i].x & 0x7fff7fffu));
                    mag = __builtin_elementwise_max(mag, __builtin_bit_cast(u16x2_t, u[i].y & 0x7fff7fffu));
                    mag = __builtin_elementwise_max(mag, __builtin_bit_cast(u16x2_t, u[i].z & 0x7fff7fffu));
                    mag = __builtin_elementwise_max(mag, __builtin_bit_cast(u16x2_t, u[i].w & 0x7fff7fffu));
                } else {
                    magf = max(magf, max(max(u[i].x & 0x7fffffffu, u[i].y & 0x7fffffffu),
                                         max(u[i].z & 0x7fffffffu, u[i].w & 0x7fffffffu)));
                }
            } else {
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    if (e0 + k < V) {
                        m = fmaxf(m, x[k]);
                        const uint32_t b = __float_as_uint(x[k]) & 0x7fffffffu;
                        if (b > 0x7f800000u)
                            magf = 0xffffffffu;  // NaN (either dtype)
                    }
                }
            }
        }
        if (m > best) {
            best = m;
            sc_best = sc;
        }
    }
    bool nan = magf > 0x7f800000u;
    if constexpr (sizeof(T) == 2)
        nan |= mag[0] > 0x7f80 || mag[1] > 0x7f80;

    // block maximum M and NaN flag
    const float wm = wave_max_f32(best);
    const uint32_t wn = __ballot(nan) != 0ull;
    if (lane == 0) {
        reinterpret_cast<float *>(wkey)[wid] = wm;
        wnan[wid] = wn;
    }
    __syncthreads();
    float M = reinterpret_cast<const float *>(wkey)[0];
    uint32_t bn = wnan[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        M = fmaxf(M, reinterpret_cast<const float *>(wkey)[w]);
        bn |= wnan[w];
    }
    // first index of M among the threads that reached it
    int first = INT_MAX;
    if (sc_best >= 0 && best == M) {
        if (sc_best != sc1 - 1)  // else its words are still in registers
            load_sub(sc_best, u);
        const int64_t base = (int64_t)sc_best * kArgSub;
#pragma unroll
        for (int i = L - 1; i >= 0; --i) {
            const int64_t e0 = base + (int64_t)(tid + NT * i) * E;
            float x[E];
            unpack(u[i], x);
#pragma unroll
            for (int k = E - 1; k >= 0; --k)
                if (e0 + k < V && x[k] == M)
                    first = (int)(e0 + k);
        }
    }
    // (a shuffle butterfly: a DPP maximum of complements measured 0.5 us slower per step)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        first = min(first, __shfl_xor(first, o, kWave));
    __syncthreads();  // every thread has read M from the slice
    if (lane == 0)
        reinterpret_cast<int *>(wkey)[wid] = first;
    __syncthreads();
    if (tid == 0) {
        int f = reinterpret_cast<const int *>(wkey)[0];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            f = min(f, reinterpret_cast<const int *>(wkey)[w]);
        const int64_t f0 = (int64_t)sc0 * kArgSub;
        uint64_t key;
        if (f != INT_MAX)
            key = rank_key(M, (uint32_t)f);
        else
            key = f0 < V ? rank_key(-INFINITY, (uint32_t)f0) : 0ull;
        ws_keys[vb] = key;
        ws_nan[vb] = bn;
    }
}

template <typename T, bool kAligned>
__global__ void __launch_bounds__(kArgThreads)
argmax_partial_kernel(const T *__restrict__ logits, int64_t row_stride, int V, int nsub,
                      int sub_per_wg, int nchunk, uint64_t *__restrict__ ws_keys,
                      uint32_t *__restrict__ ws_nan)
{
    __shared__ uint64_t wkey[kArgThreads / 64];
    __shared__ uint32_t wnan[kArgThreads / 64];
    argmax_partial_block<T, kAligned, kArgThreads>(logits, row_stride, V, nsub, sub_per_wg, nchunk,
                                                   ws_keys, ws_nan, blockIdx.x, wkey, wnan);
}

// Phase 2 for sequence s by a workgroup of 256 threads.  err[s] receives the verification
// flags OR-ed with extra0[s] and extra1[s] (flags of other steps; either may be NULL).
__device__ __forceinline__ void verify_walk_block(int s, int B, int N, int nchunk, const uint64_t *__restrict__ ws_keys,
                                  const uint32_t *__restrict__ ws_nan, const int32_t *__restrict__ parent,
                                  const int32_t *__restrict__ tokens, const uint64_t *__restrict__ anc,
                                  const int32_t *__restrict__ depth, int32_t *__restrict__ accept_len,
                                  int32_t *__restrict__ accept_path, int32_t *__restrict__ bonus,
                                  int32_t *__restrict__ argmax_out, int32_t *__restrict__ err,
                                  const int32_t *__restrict__ extra0, const int32_t *__restrict__ extra1)
{
    __shared__ unsigned long long amk[JT_MAX_NODES];
    __shared__ uint32_t amn[JT_MAX_NODES];
    __shared__ uint64_t ancl[JT_MAX_NODES][4];
    __shared__ uint64_t okw[4];
    __shared__ uint32_t wbest[4];
    __shared__ int fl[4];
    const int v = threadIdx.x;
    const int lane = v & 63, wid = v >> 6;
    const int64_t nb = (int64_t)s * B + v;
    int extra = 0;
    if (v == 0) {
        if (extra0)
            extra |= extra0[s];
        if (extra1)
            extra |= extra1[s];
    }

    if (v < B) {
        amk[v] = 0ull;
        amn[v] = 0u;
    }
    __syncthreads();

    // One memory round trip: the node's own parent, depth, token and ancestor row, and a
    // share of the B * nchunk partial argmax keys (item i = node i / nchunk, chunk
    // i % nchunk), all issued before any is used.
    int p = -1, dv = 0, tok = 0;
    uint64_t a0 = 0ull, a1 = 0ull, a2 = 0ull, a3 = 0ull;
    if (v < B) {
        p = parent[nb];
        dv = depth[nb];
        tok = tokens[nb];
        const uint64_t *ar = anc + nb * 4;
        a0 = ar[0];
        a1 = ar[1];
        a2 = ar[2];
        a3 = ar[3];
    }
    const int items = B * nchunk;
    const uint64_t *kbase = ws_keys + (int64_t)s * items;
    const uint32_t *nbase = ws_nan + (int64_t)s * items;
    constexpr int kItemBatch = 8;
    for (int i0 = 0; i0 < items; i0 += 256 * kItemBatch) {
        uint64_t kc[kItemBatch];
        uint32_t nc[kItemBatch];
#pragma unroll
        for (int q = 0; q < kItemBatch; ++q) {
            const int i = i0 + v + 256 * q;
            kc[q] = i < items ? kbase[i] : 0ull;
            nc[q] = i < items ? nbase[i] : 0u;
        }
#pragma unroll
        for (int q = 0; q < kItemBatch; ++q) {
            const int i = i0 + v + 256 * q;
            if (i < items) {
                const int u = i / nchunk;
                atomicMax(&amk[u], (unsigned long long)kc[q]);
                if (nc[q])
                    atomicOr(&amn[u], nc[q]);
            }
        }
    }
    int flags = 0;
    if (v < B) {
        ancl[v][0] = a0;
        ancl[v][1] = a1;
        ancl[v][2] = a2;
        ancl[v][3] = a3;
        if (v == 0 ? (p != -1) : (p < 0 || p >= v))
            flags |= JT_DEV_BAD_PARENT;
        if (dv > N || dv < 0)
            flags |= JT_DEV_DEPTH_GT_N;
    }
    __syncthreads();
    int am_v = 0;
    if (v < B) {
        const uint64_t k = amk[v];
        am_v = (k == 0ull) ? 0 : (int32_t)key_id(k);
        if (amn[v])
            flags |= JT_DEV_NAN;
    }
    // OR of the flags over the block
    int f = (int)wave_or_u32((uint32_t)flags);
    if (lane == 0)
        fl[wid] = f;
    __syncthreads();
    f = fl[0] | fl[1] | fl[2] | fl[3];
    if (argmax_out && v < B)
        argmax_out[nb] = am_v;
    auto am_of = [&](int u) {
        const uint64_t k = amk[u];
        return (k == 0ull) ? 0 : (int32_t)key_id(k);
    };
    int32_t *path = accept_path + (int64_t)s * (N + 1);
    if (f & (JT_DEV_BAD_PARENT | JT_DEV_DEPTH_GT_N)) {
        if (f & JT_DEV_BAD_PARENT)
            f &= ~JT_DEV_DEPTH_GT_N;  // depths are meaningless without a valid tree
        for (int k = v; k <= N; k += blockDim.x)
            path[k] = (k == 0) ? 0 : -1;
        if (v == 0) {
            accept_len[s] = 0;
            bonus[s] = am_v;
            if (err)
                err[s] = f | extra;
        }
        return;
    }
    const bool ok = (v < B) && (v == 0 || tok == am_of(p));
    const uint64_t word = __ballot(ok);
    if (lane == 0)
        okw[wid] = word;
    __syncthreads();
    uint32_t key = 0u;
    if (v < B) {
        const bool accepted = ((ancl[v][0] & ~okw[0]) | (ancl[v][1] & ~okw[1]) |
                               (ancl[v][2] & ~okw[2]) | (ancl[v][3] & ~okw[3])) == 0ull;
        if (accepted)
            key = ((uint32_t)dv << 16) | (uint32_t)(65535 - v);
    }
    key = wave_max_u32(key);
    if (lane == 0)
        wbest[wid] = key;
    __syncthreads();
    const uint32_t kb = max(max(wbest[0], wbest[1]), max(wbest[2], wbest[3]));
    const int vstar = 65535 - (int)(kb & 0xffffu);
    const int len = (int)(kb >> 16);
    // path: every ancestor u of v* (itself included) sits at index depth[u]
    for (int k = len + 1 + v; k <= N; k += blockDim.x)
        path[k] = -1;
    if (v < B && ((ancl[vstar][v >> 6] >> (v & 63)) & 1ull))
        path[dv] = v;
    if (v == 0) {
        accept_len[s] = len;
        bonus[s] = am_of(vstar);
        if (err)
            err[s] = f | extra;
    }
}

__global__ void __launch_bounds__(256)
verify_walk_kernel(int B, int N, int nchunk, const uint64_t *__restrict__ ws_keys,
                   const uint32_t *__restrict__ ws_nan, const int32_t *__restrict__ parent,
                   const int32_t *__restrict__ tokens, const uint64_t *__restrict__ anc,
                   const int32_t *__restrict__ depth, int32_t *__restrict__ accept_len,
                   int32_t *__restrict__ accept_path, int32_t *__restrict__ bonus,
                   int32_t *__restrict__ argmax_out, int32_t *__restrict__ err)
{
    verify_walk_block(blockIdx.x, B, N, nchunk, ws_keys, ws_nan, parent, tokens, anc, depth,
                      accept_len, accept_path, bonus, argmax_out, err, nullptr, nullptr);
}

struct ArgPlan {
    int nsub, sub_per_wg, nchunk;
};

static ArgPlan arg_plan(int rows, int V)
{
    ArgPlan p;
    p.nsub = (V + kArgSub - 1) / kArgSub;
    int want = (rows > 0) ? (2048 + rows - 1) / rows : 1;
    int spw = (p.nsub + want - 1) / want;
    if (spw < 1)
        spw = 1;
    while ((p.nsub + spw - 1) / spw > kArgMaxChunks)
        ++spw;
    p.sub_per_wg = spw;
    p.nchunk = (p.nsub + spw - 1) / spw;
    return p;
}

size_t verify_workspace(int S, int B, int V, int /*dtype*/)
{
    const ArgPlan p = arg_plan(S * B, V);
    const size_t parts = (size_t)S * B * p.nchunk;
    return parts * (sizeof(uint64_t) + sizeof(uint32_t)) + 256;
}

jt_status launch_verify(const void *logits, int64_t row_stride, int V, int dtype,
                        const int32_t *parent, const int32_t *tokens, const uint64_t *anc,
                        const int32_t *depth, int S, int B, int N, int32_t *accept_len,
                        int32_t *accept_path, int32_t *bonus, int32_t *argmax_out,
                        int32_t *err, void *ws, hipStream_t st)
{
    if (S == 0)
        return JT_OK;
    const int rows = S * B;
    const ArgPlan p = arg_plan(rows, V);
    const size_t parts = (size_t)rows * p.nchunk;
    uint64_t *wk = reinterpret_cast<uint64_t *>(ws);
    uint32_t *wn = reinterpret_cast<uint32_t *>(wk + parts);
    const dim3 grid((unsigned)parts), block(kArgThreads);
    const uintptr_t addr = reinterpret_cast<uintptr_t>(logits);
    if (dtype == JT_BF16) {
        if ((addr % 16 == 0) && (row_stride % 8 == 0))
            hipLaunchKernelGGL((argmax_partial_kernel<uint16_t, true>), grid, block, 0, st,
                               (const uint16_t *)logits, row_stride, V, p.nsub, p.sub_per_wg,
                               p.nchunk, wk, wn);
        else
            hipLaunchKernelGGL((argmax_partial_kernel<uint16_t, false>), grid, block, 0, st,
                               (const uint16_t *)logits, row_stride, V, p.nsub, p.sub_per_wg,
                               p.nchunk, wk, wn);
    } else {
        if ((addr % 16 == 0) && (row_stride % 4 == 0))
            hipLaunchKernelGGL((argmax_partial_kernel<float, true>), grid, block, 0, st,
                               (const float *)logits, row_stride, V, p.nsub, p.sub_per_wg,
                               p.nchunk, wk, wn);
        else
            hipLaunchKernelGGL((argmax_partial_kernel<float, false>), grid, block, 0, st,
                               (const float *)logits, row_stride, V, p.nsub, p.sub_per_wg,
                               p.nchunk, wk, wn);
    }
    jt_status e = launch_status(hipGetLastError());
    if (e != JT_OK)
        return e;
    hipLaunchKernelGGL(verify_walk_kernel, dim3(S), dim3(256), 0, st, B, N, p.nchunk, wk, wn,
                       parent, tokens, anc, depth, accept_len, accept_path, bonus, argmax_out,
                       err);
    return launch_status(hipGetLastError());
}

jt_status launch_verify_walk(const int32_t *parent, const int32_t *tokens, const uint64_t *anc,
                             const int32_t *depth, int S, int B, int N, int nchunk,
                             const uint64_t *keys, const uint32_t *nan, int32_t *accept_len,
                             int32_t *accept_path, int32_t *bonus, int32_t *argmax_out,
                             int32_t *err, hipStream_t st)
{
    hipLaunchKernelGGL(verify_walk_kernel, dim3(S), dim3(256), 0, st, B, N, nchunk, keys, nan,
                       parent, tokens, anc, depth, accept_len, accept_path, bonus, argmax_out,
                       err);
    return launch_status(hipGetLastError());
}

} // namespace jt
