// Step 3: per-depth top-W token ids and log-probabilities over vocabulary-wide rows.
//
// The proposer keeps the top-k tokens and their log-probabilities at every future
// position (paperlayer.ai JetSpec summary, appendix E "Drafting"); W per depth
// (paper.rainbus.top summary, method steps).
//
// Bytes, not flops, bound this step: every logit is read once.  Layout of the work:
//   * a row is cut into sub-chunks of 8192 logits; one workgroup (4 waves) owns a run of
//     consecutive sub-chunks of one row, so even 16 rows fill the 256 CUs;
//   * a sub-chunk is pulled into registers with 16-byte loads (32 logits per thread) and
//     reduced there: thread max, then sum of exp(x - max) (exact per-thread rescale);
//   * a threshold tau (the W-th largest thread maximum inside one wave, found by a 32-step
//     ballot bisection on order codes) bounds the chunk's W-th largest logit from below,
//     so only threads whose maximum reaches tau scan for candidates;
//   * candidates land in LDS as 64-bit keys (order code << 32 | ~id): value descending,
//     id ascending in one integer compare, so bf16 ties resolve exactly like a full
//     sort; the running top-W is kept in LDS across the sub-chunks of a workgroup;
//   * a merge kernel (one wave per row) combines the partial top-W lists and the
//     (max, sum-exp) pairs into ids, log-probs and the row log-sum-exp.
#include "jt_internal.h"

namespace jt {

constexpr int kTopwThreads = 256;
constexpr int kSub = 8192;          // logits per sub-chunk (32 per thread)
constexpr int kCap = 1024;          // candidate slots in LDS
constexpr int kMaxMergeChunks = 64; // partial lists per row seen by the merge kernel
constexpr float kLog2e = 1.4426950408889634f;

template <typename T> struct Vec;
template <> struct Vec<uint16_t> { static constexpr int kElems = 8; static constexpr int kLoads = 4; };
template <> struct Vec<float> { static constexpr int kElems = 4; static constexpr int kLoads = 8; };

// Loads the thread's 32 logits of one sub-chunk.  Element k of load i sits at index
// base + (tid + 256*i)*E + k.  Out-of-row entries become -inf with valid = false.
template <typename T, bool kAligned>
__device__ __forceinline__ void load_sub(const T *__restrict__ row, int64_t base, int V, int tid,
                                         float (&x)[32], uint32_t &valid)
{
    constexpr int E = Vec<T>::kElems;
    constexpr int L = Vec<T>::kLoads;
    valid = 0;
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int64_t e0 = base + (int64_t)(tid + kTopwThreads * i) * E;
        if (kAligned && e0 + E <= V) {
            const uint4 u = *reinterpret_cast<const uint4 *>(row + e0);
            if constexpr (sizeof(T) == 2) {
                x[i * 8 + 0] = bf16_lo(u.x); x[i * 8 + 1] = bf16_hi(u.x);
                x[i * 8 + 2] = bf16_lo(u.y); x[i * 8 + 3] = bf16_hi(u.y);
                x[i * 8 + 4] = bf16_lo(u.z); x[i * 8 + 5] = bf16_hi(u.z);
                x[i * 8 + 6] = bf16_lo(u.w); x[i * 8 + 7] = bf16_hi(u.w);
            } else {
                x[i * 4 + 0] = __uint_as_float(u.x); x[i * 4 + 1] = __uint_as_float(u.y);
                x[i * 4 + 2] = __uint_as_float(u.z); x[i * 4 + 3] = __uint_as_float(u.w);
            }
            valid |= ((1u << E) - 1u) << (i * E);
        } else {
#pragma unroll
            for (int k = 0; k < E; ++k) {
                const int64_t e = e0 + k;
                if (e < V) {
                    if constexpr (sizeof(T) == 2)
                        x[i * E + k] = bf16_to_f32(row[e]);
                    else
                        x[i * E + k] = row[e];
                    valid |= 1u << (i * E + k);
                } else {
                    x[i * E + k] = -INFINITY;
                }
            }
        }
    }
}

template <typename T>
__device__ __forceinline__ uint32_t elem_id(int64_t base, int tid, int j)
{
    constexpr int E = Vec<T>::kElems;
    return (uint32_t)(base + (int64_t)(tid + kTopwThreads * (j / E)) * E + (j % E));
}

// Largest code t such that at least W lanes of the wave hold a code >= t.
__device__ __forceinline__ uint32_t wave_wth_code(uint32_t code, int W)
{
    uint32_t prefix = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = prefix | (1u << bit);
        const int cnt = __popcll(__ballot(code >= cand));
        if (cnt >= W)
            prefix = cand;
    }
    return prefix;
}

// Selects the W largest keys among keys[0..n) (distinct keys; 0 = empty) into out[0..W)
// sorted descending, padding with 0.  Block-wide; ends with a barrier.
__device__ void select_topw(const uint64_t *keys, int n, int W, uint64_t *out)
{
    for (int i = threadIdx.x; i < W; i += blockDim.x)
        out[i] = 0ull;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const uint64_t k = keys[i];
        if (k == 0ull)
            continue;
        int rank = 0;
        for (int j = 0; j < n; ++j)
            rank += keys[j] > k;
        if (rank < W)
            out[rank] = k;
    }
    __syncthreads();
}

template <typename T, bool kAligned>
__global__ void __launch_bounds__(kTopwThreads)
topw_partial_kernel(const T *__restrict__ logits, int64_t row_stride, int V, int W, int nsub,
                    int sub_per_wg, int nchunk, uint64_t *__restrict__ ws_keys,
                    float2 *__restrict__ ws_ms)
{
    __shared__ uint64_t cand[kCap + JT_MAX_W];
    __shared__ uint64_t best[JT_MAX_W];
    __shared__ int ncand;
    __shared__ uint32_t wave_tau[4];
    __shared__ float wave_m[4], wave_s[4];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int row_idx = blockIdx.x / nchunk;
    const int chunk = blockIdx.x % nchunk;
    const T *row = logits + (int64_t)row_idx * row_stride;
    const int sc0 = chunk * sub_per_wg;
    const int sc1 = min(nsub, sc0 + sub_per_wg);

    if (tid < JT_MAX_W)
        best[tid] = 0ull;
    float run_m = -INFINITY, run_s = 0.f;   // this thread's running (max, sum exp(x-max))

    for (int sc = sc0; sc < sc1; ++sc) {
        const int64_t base = (int64_t)sc * kSub;
        float x[32];
        uint32_t valid;
        load_sub<T, kAligned>(row, base, V, tid, x, valid);

        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < 32; ++j)
            m = fmaxf(m, x[j]);
        // sum exp(x - m) over this sub-chunk, then fold into the running pair
        float s = 0.f;
        if (m != -INFINITY) {
            const float mb = m * kLog2e;
#pragma unroll
            for (int j = 0; j < 32; ++j)
                s += __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], kLog2e, -mb));
        } else {
            // every entry is -inf, padding or NaN: only a NaN must still poison the sum
#pragma unroll
            for (int j = 0; j < 32; ++j)
                if (x[j] != x[j])
                    s = x[j];
        }
        if (m > run_m) {
            const float prev = (run_m == -INFINITY)
                                   ? ((run_s != run_s) ? run_s : 0.f)
                                   : run_s * __builtin_amdgcn_exp2f((run_m - m) * kLog2e);
            run_s = prev + s;
            run_m = m;
        } else if (m == -INFINITY) {
            run_s += s;  // adds 0, or propagates a NaN
        } else {
            run_s += s * __builtin_amdgcn_exp2f((m - run_m) * kLog2e);
        }

        // ---- candidate threshold
        // a thread's code counts only if it holds a real (non-NaN) element equal to m
        bool real = m != -INFINITY;
        if (!real) {
#pragma unroll
            for (int j = 0; j < 32; ++j)
                real |= ((valid >> j) & 1u) && x[j] == -INFINITY;
        }
        const uint32_t my_code = real ? order_code(m) : 0u;
        const uint32_t tau_w = wave_wth_code(my_code, W);
        if (lane == 0)
            wave_tau[wid] = tau_w;
        if (tid == 0)
            ncand = 0;
        __syncthreads();
        uint32_t tau = max(max(wave_tau[0], wave_tau[1]), max(wave_tau[2], wave_tau[3]));
        const uint64_t wth = best[W - 1];
        if (wth != 0ull)
            tau = max(tau, (uint32_t)(wth >> 32));
        // tau == 0 means "fewer than W thread maxima": every valid element is a candidate
        if (tau == 0u || my_code >= tau) {
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                if (!((valid >> j) & 1u))
                    continue;
                const uint32_t c = order_code(x[j]);
                if (c >= tau) {
                    const int slot = atomicAdd(&ncand, 1);
                    if (slot < kCap)
                        cand[slot] = ((uint64_t)c << 32) | (uint64_t)(~elem_id<T>(base, tid, j));
                }
            }
        }
        __syncthreads();
        const int n = ncand;
        if (n <= kCap) {
            // merge the previous top-W into the candidate list, then re-select
            if (tid < W)
                cand[n + tid] = best[tid];
            __syncthreads();
            select_topw(cand, n + W, W, best);
        } else {
            // rare overflow (huge ties): W rounds of exact arg-max over the registers
            uint64_t prev = ~0ull;
            for (int r = 0; r < W; ++r) {
                uint64_t mine = 0ull;
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    if (!((valid >> j) & 1u))
                        continue;
                    const uint64_t k = rank_key(x[j], elem_id<T>(base, tid, j));
                    if (k < prev && k > mine)
                        mine = k;
                }
                mine = wave_max_u64(mine);
                if (lane == 0)
                    cand[wid] = mine;
                __syncthreads();
                const uint64_t g = max(max(cand[0], cand[1]), max(cand[2], cand[3]));
                __syncthreads();
                if (tid == 0)
                    cand[4 + r] = g;
                prev = g;
            }
            __syncthreads();
            if (tid < W)
                cand[4 + W + tid] = best[tid];
            __syncthreads();
            select_topw(cand + 4, 2 * W, W, best);
        }
    }

    // ---- (max, sum) over the workgroup
    float m = wave_max_f32(run_m);
    float s = (run_m == -INFINITY) ? ((run_s != run_s) ? run_s : 0.f)
                                   : run_s * __builtin_amdgcn_exp2f((run_m - m) * kLog2e);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        s += __shfl_xor(s, o, kWave);
    if (lane == 0) {
        wave_m[wid] = m;
        wave_s[wid] = s;
    }
    __syncthreads();
    if (tid == 0) {
        float M = fmaxf(fmaxf(wave_m[0], wave_m[1]), fmaxf(wave_m[2], wave_m[3]));
        float Ssum = 0.f;
        for (int w = 0; w < 4; ++w) {
            if (wave_m[w] == -INFINITY)
                Ssum += (wave_s[w] != wave_s[w]) ? wave_s[w] : 0.f;
            else
                Ssum += wave_s[w] * __builtin_amdgcn_exp2f((wave_m[w] - M) * kLog2e);
        }
        ws_ms[blockIdx.x] = make_float2(M, Ssum);
    }
    if (tid < W)
        ws_keys[(int64_t)blockIdx.x * W + tid] = best[tid];
}

// One wave per row: merge the partial lists and (max, sum) pairs.
__global__ void __launch_bounds__(64)
topw_merge_kernel(int rows, int W, int nchunk, const uint64_t *__restrict__ ws_keys,
                  const float2 *__restrict__ ws_ms, int32_t *__restrict__ ids,
                  float *__restrict__ logprob, float *__restrict__ row_lse)
{
    __shared__ uint64_t keys[kMaxMergeChunks * JT_MAX_W];
    __shared__ uint64_t top[JT_MAX_W];
    const int r = blockIdx.x;
    const int lane = threadIdx.x;
    const int n = nchunk * W;
    for (int i = lane; i < n; i += 64)
        keys[i] = ws_keys[(int64_t)r * n + i];
    // LSE over the row
    float m = -INFINITY;
    for (int c = lane; c < nchunk; c += 64)
        m = fmaxf(m, ws_ms[(int64_t)r * nchunk + c].x);
    m = wave_max_f32(m);
    float s = 0.f;
    for (int c = lane; c < nchunk; c += 64) {
        const float2 p = ws_ms[(int64_t)r * nchunk + c];
        if (p.x == -INFINITY)
            s += (p.y != p.y) ? p.y : 0.f;
        else
            s += p.y * __builtin_amdgcn_exp2f((p.x - m) * kLog2e);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        s += __shfl_xor(s, o, kWave);
    float lse;
    if (s != s)
        lse = s;
    else if (m == -INFINITY)
        lse = -INFINITY;
    else
        lse = m + logf(s);
    __syncthreads();
    select_topw(keys, n, W, top);
    if (lane < W) {
        const uint64_t k = top[lane];
        ids[(int64_t)r * W + lane] = (int32_t)key_id(k);
        logprob[(int64_t)r * W + lane] = key_value(k) - lse;
    }
    if (lane == 0 && row_lse)
        row_lse[r] = lse;
}

struct TopwPlan {
    int nsub, sub_per_wg, nchunk;
};

static TopwPlan topw_plan(int rows, int V)
{
    TopwPlan p;
    p.nsub = (V + kSub - 1) / kSub;
    // aim for ~2048 workgroups in flight, at most kMaxMergeChunks partial lists per row
    int want = (rows > 0) ? (2048 + rows - 1) / rows : 1;
    int spw = (p.nsub + want - 1) / want;
    if (spw < 1)
        spw = 1;
    while ((p.nsub + spw - 1) / spw > kMaxMergeChunks)
        ++spw;
    p.sub_per_wg = spw;
    p.nchunk = (p.nsub + spw - 1) / spw;
    return p;
}

size_t topw_workspace(int rows, int V, int W, int /*dtype*/)
{
    const TopwPlan p = topw_plan(rows, V);
    const size_t parts = (size_t)rows * p.nchunk;
    return parts * (size_t)W * sizeof(uint64_t) + parts * sizeof(float2) + 256;
}

jt_status launch_topw(const void *logits, int64_t row_stride, int rows, int V, int W, int dtype,
                      int32_t *ids, float *logprob, float *row_lse, void *ws, hipStream_t st)
{
    if (rows == 0)
        return JT_OK;
    const TopwPlan p = topw_plan(rows, V);
    const size_t parts = (size_t)rows * p.nchunk;
    uint64_t *wk = reinterpret_cast<uint64_t *>(ws);
    uintptr_t mp = reinterpret_cast<uintptr_t>(wk + parts * W);
    mp = (mp + 15) & ~(uintptr_t)15;
    float2 *wm = reinterpret_cast<float2 *>(mp);
    const dim3 grid((unsigned)parts), block(kTopwThreads);
    const uintptr_t addr = reinterpret_cast<uintptr_t>(logits);
    if (dtype == JT_BF16) {
        const bool al = (addr % 16 == 0) && (row_stride % 8 == 0);
        if (al)
            hipLaunchKernelGGL((topw_partial_kernel<uint16_t, true>), grid, block, 0, st,
                               (const uint16_t *)logits, row_stride, V, W, p.nsub, p.sub_per_wg,
                               p.nchunk, wk, wm);
        else
            hipLaunchKernelGGL((topw_partial_kernel<uint16_t, false>), grid, block, 0, st,
                               (const uint16_t *)logits, row_stride, V, W, p.nsub, p.sub_per_wg,
                               p.nchunk, wk, wm);
    } else {
        const bool al = (addr % 16 == 0) && (row_stride % 4 == 0);
        if (al)
            hipLaunchKernelGGL((topw_partial_kernel<float, true>), grid, block, 0, st,
                               (const float *)logits, row_stride, V, W, p.nsub, p.sub_per_wg,
                               p.nchunk, wk, wm);
        else
            hipLaunchKernelGGL((topw_partial_kernel<float, false>), grid, block, 0, st,
                               (const float *)logits, row_stride, V, W, p.nsub, p.sub_per_wg,
                               p.nchunk, wk, wm);
    }
    jt_status e = launch_status(hipGetLastError());
    if (e != JT_OK)
        return e;
    hipLaunchKernelGGL(topw_merge_kernel, dim3(rows), dim3(64), 0, st, rows, W, p.nchunk, wk, wm,
                       ids, logprob, row_lse);
    return launch_status(hipGetLastError());
}

} // namespace jt
