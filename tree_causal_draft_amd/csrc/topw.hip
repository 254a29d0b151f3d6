// Step 3: per-depth top-W token ids and log-probabilities over vocabulary-wide rows.
//
// The proposer keeps the top-k tokens and their log-probabilities at every future
// position (paperlayer.ai JetSpec summary, appendix E "Drafting"); W per depth
// (paper.rainbus.top summary, method steps).
//
// Bytes, not flops, bound this step: every logit is read once.  Layout of the work:
//   * a row is cut into pieces of 2048 logits; each wave of a workgroup owns one piece
//     (or a run of them for very long rows) and works alone, with no workgroup barrier,
//     so the many small pieces spread the row over the whole chip;
//   * a piece is pulled into registers with 16-byte loads (32 logits per lane) and
//     reduced there: lane max, then sum of exp(x - max) (exact per-lane rescale);
//   * a threshold tau (the W-th largest lane maximum, found by a 32-step ballot
//     bisection on order codes) bounds the piece's W-th largest logit from below, so
//     only logits >= tau become candidates;
//   * candidates land in the wave's LDS slice as 64-bit keys (order code << 32 | ~id):
//     value descending, id ascending in one integer compare, so bf16 ties resolve
//     exactly like a full sort; W rounds of a DPP wave max extract the W largest;
//   * a merge kernel (one wave per row) combines the per-wave top-W lists and the
//     (max, sum-exp) pairs into ids, log-probs and the row log-sum-exp.
#include "jt_internal.h"

namespace jt {

constexpr int kTopwThreads = 256;   // 4 independent waves per workgroup
constexpr int kPiece = 2048;        // logits per wave piece (32 per lane)
constexpr int kWaveCap = 512;       // candidate slots per wave in LDS
constexpr int kMaxLists = 128;      // partial lists per row seen by the merge kernel
constexpr float kLog2e = 1.4426950408889634f;

template <typename T> struct Vec;
template <> struct Vec<uint16_t> { static constexpr int kElems = 8; static constexpr int kLoads = 4; };
template <> struct Vec<float> { static constexpr int kElems = 4; static constexpr int kLoads = 8; };

// Loads a lane's 32 logits of one piece.  Element k of load i sits at index
// base + (lane + 64*i)*E + k.  Out-of-row entries become -inf with valid = false.
template <typename T, bool kAligned>
__device__ __forceinline__ void load_piece(const T *__restrict__ row, int64_t base, int V, int lane,
                                           float (&x)[32], uint32_t &valid)
{
    constexpr int E = Vec<T>::kElems;
    constexpr int L = Vec<T>::kLoads;
    valid = 0;
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int64_t e0 = base + (int64_t)(lane + kWave * i) * E;
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
__device__ __forceinline__ uint32_t elem_id(int64_t base, int lane, int j)
{
    constexpr int E = Vec<T>::kElems;
    return (uint32_t)(base + (int64_t)(lane + kWave * (j / E)) * E + (j % E));
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

// Orders the LDS accesses of one wave: writes by some lanes before reads by others.
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave selects the W largest of keys[0..n) (distinct keys; 0 = empty) into out[0..W),
// descending, padding with 0: W rounds, each taking the largest key below the previous
// winner (lane-local scan, then a DPP wave max).  Keys are distinct because ids are, so
// the order is exactly (value desc, id asc).
__device__ void wave_select_topw(const uint64_t *keys, int n, int W, uint64_t *out)
{
    const int lane = threadIdx.x & 63;
    uint64_t prev = ~0ull;
    for (int r = 0; r < W; ++r) {
        uint64_t mine = 0ull;
        for (int i = lane; i < n; i += 64) {
            const uint64_t k = keys[i];
            mine = (k < prev && k > mine) ? k : mine;
        }
        mine = wave_max_u64_dpp(mine);
        if (lane == 0)
            out[r] = mine;
        prev = mine;
    }
    wave_sync();
}

// Each wave owns `ppw` consecutive pieces of 2048 logits of one row and works alone (no
// workgroup barrier): lane max and sum of exp(x - max); a threshold tau = the W-th
// largest lane maximum of the piece, a lower bound on the piece's W-th largest logit;
// the logits >= tau (and above the running W-th best) compacted into the wave's LDS
// slice by ballot + mbcnt; W rounds of a wave max over those and the running top-W.
// Output per wave: its W best keys and its (max, sum-exp) pair.
template <typename T, bool kAligned>
__global__ void __launch_bounds__(kTopwThreads)
topw_partial_kernel(const T *__restrict__ logits, int64_t row_stride, int rows, int V, int W,
                    int npiece, int ppw, int nlist, uint64_t *__restrict__ ws_keys,
                    float2 *__restrict__ ws_ms)
{
    __shared__ uint64_t cand_all[4][kWaveCap + JT_MAX_W];
    __shared__ uint64_t best_all[4][JT_MAX_W];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int gl = blockIdx.x * 4 + wid;  // list index = (row, list within the row)
    if (gl >= rows * nlist)
        return;
    const int row_idx = gl / nlist, li = gl % nlist;
    const T *row = logits + (int64_t)row_idx * row_stride;
    uint64_t *cand = cand_all[wid];
    uint64_t *best = best_all[wid];
    if (lane < JT_MAX_W)
        best[lane] = 0ull;
    wave_sync();
    float run_m = -INFINITY, run_s = 0.f;  // lane's running (max, sum exp(x - max))
    const int p0 = li * ppw, p1 = min(npiece, p0 + ppw);
    for (int pc = p0; pc < p1; ++pc) {
        const int64_t base = (int64_t)pc * kPiece;
        float x[32];
        uint32_t valid;
        load_piece<T, kAligned>(row, base, V, lane, x, valid);
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < 32; ++j)
            m = fmaxf(m, x[j]);
        float sx = 0.f;
        if (m != -INFINITY) {
            const float mb = m * kLog2e;
#pragma unroll
            for (int j = 0; j < 32; ++j)
                sx += __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], kLog2e, -mb));
        } else {
            // every entry is -inf, padding or NaN: only a NaN must still poison the sum
#pragma unroll
            for (int j = 0; j < 32; ++j)
                if (x[j] != x[j])
                    sx = x[j];
        }
        if (m > run_m) {
            const float prev = (run_m == -INFINITY)
                                   ? ((run_s != run_s) ? run_s : 0.f)
                                   : run_s * __builtin_amdgcn_exp2f((run_m - m) * kLog2e);
            run_s = prev + sx;
            run_m = m;
        } else if (m == -INFINITY) {
            run_s += sx;  // adds 0, or propagates a NaN
        } else {
            run_s += sx * __builtin_amdgcn_exp2f((m - run_m) * kLog2e);
        }

        // ---- threshold: a lane's code counts only if it holds a real (non-NaN) element
        // equal to its maximum
        bool real = m != -INFINITY;
        if (!real) {
#pragma unroll
            for (int j = 0; j < 32; ++j)
                real |= ((valid >> j) & 1u) && x[j] == -INFINITY;
        }
        uint32_t tau = wave_wth_code(real ? order_code(m) : 0u, W);
        const uint64_t wth = best[W - 1];
        if (wth != 0ull)
            tau = max(tau, (uint32_t)(wth >> 32));
        // tau == 0: fewer than W lane maxima, every valid element is a candidate
        int n = 0;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const uint32_t c = order_code(x[j]);
            const bool pred = ((valid >> j) & 1u) && c >= tau;
            const uint64_t b = __ballot(pred);
            if (b) {
                const int slot = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
                if (pred && slot < kWaveCap)
                    cand[slot] = ((uint64_t)c << 32) | (uint64_t)(~elem_id<T>(base, lane, j));
                n += __popcll(b);
            }
        }
        wave_sync();
        if (n <= kWaveCap) {
            if (lane < W)
                cand[n + lane] = best[lane];
            wave_sync();
            wave_select_topw(cand, n + W, W, best);
        } else {
            // rare overflow (huge ties): W rounds of exact arg-max over the registers
            uint64_t prev = ~0ull;
            for (int r = 0; r < W; ++r) {
                uint64_t mine = 0ull;
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    if (!((valid >> j) & 1u))
                        continue;
                    const uint64_t k = rank_key(x[j], elem_id<T>(base, lane, j));
                    if (k < prev && k > mine)
                        mine = k;
                }
                mine = wave_max_u64_dpp(mine);
                if (lane == 0)
                    cand[r] = mine;
                prev = mine;
            }
            if (lane < W)
                cand[W + lane] = best[lane];
            wave_sync();
            wave_select_topw(cand, 2 * W, W, best);
        }
    }

    // ---- (max, sum) over the wave
    const float m = wave_max_f32(run_m);
    float sw = (run_m == -INFINITY) ? ((run_s != run_s) ? run_s : 0.f)
                                    : run_s * __builtin_amdgcn_exp2f((run_m - m) * kLog2e);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        sw += __shfl_xor(sw, o, kWave);
    if (lane == 0)
        ws_ms[gl] = make_float2(m, sw);
    if (lane < W)
        ws_keys[(int64_t)gl * W + lane] = best[lane];
}

// One wave per row: merge the partial lists and (max, sum) pairs.
__global__ void __launch_bounds__(64)
topw_merge_kernel(int rows, int W, int nchunk, const uint64_t *__restrict__ ws_keys,
                  const float2 *__restrict__ ws_ms, int32_t *__restrict__ ids,
                  float *__restrict__ logprob, float *__restrict__ row_lse)
{
    __shared__ uint64_t keys[kMaxLists * JT_MAX_W];
    __shared__ uint64_t top[JT_MAX_W];
    const int r = blockIdx.x;
    const int lane = threadIdx.x;
    const int n = nchunk * W;
    // Every load is issued before any result is used (one memory round trip for lists of
    // up to 64 * kKeyBatch keys): the (max, sum) pairs, then the keys.
    constexpr int kMsPerLane = kMaxLists / kWave;
    constexpr int kKeyBatch = 16;
    const float2 *msr = ws_ms + (int64_t)r * nchunk;
    const uint64_t *src = ws_keys + (int64_t)r * n;
    float2 ms[kMsPerLane];
#pragma unroll
    for (int j = 0; j < kMsPerLane; ++j) {
        const int c = lane + kWave * j;
        ms[j] = c < nchunk ? msr[c] : make_float2(-INFINITY, 0.f);
    }
    for (int i0 = 0; i0 < n; i0 += kWave * kKeyBatch) {
        uint64_t kr[kKeyBatch];
#pragma unroll
        for (int q = 0; q < kKeyBatch; ++q) {
            const int i = i0 + lane + kWave * q;
            kr[q] = i < n ? src[i] : 0ull;
        }
#pragma unroll
        for (int q = 0; q < kKeyBatch; ++q) {
            const int i = i0 + lane + kWave * q;
            if (i < n)
                keys[i] = kr[q];
        }
    }
    // LSE over the row
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMsPerLane; ++j)
        m = fmaxf(m, ms[j].x);
    m = wave_max_f32(m);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kMsPerLane; ++j) {
        const float2 p = ms[j];
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
    wave_select_topw(keys, n, W, top);
    __syncthreads();
    if (lane < W) {
        const uint64_t k = top[lane];
        ids[(int64_t)r * W + lane] = (int32_t)key_id(k);
        logprob[(int64_t)r * W + lane] = key_value(k) - lse;
    }
    if (lane == 0 && row_lse)
        row_lse[r] = lse;
}

struct TopwPlan {
    int npiece, ppw, nlist;
};

static TopwPlan topw_plan(int rows, int V)
{
    TopwPlan p;
    p.npiece = (V + kPiece - 1) / kPiece;
    p.ppw = (p.npiece + kMaxLists - 1) / kMaxLists;  // pieces per wave
    p.nlist = (p.npiece + p.ppw - 1) / p.ppw;        // partial lists per row
    return p;
}

size_t topw_workspace(int rows, int V, int W, int /*dtype*/)
{
    const TopwPlan p = topw_plan(rows, V);
    const size_t parts = (size_t)rows * p.nlist;
    return parts * (size_t)W * sizeof(uint64_t) + parts * sizeof(float2) + 256;
}

jt_status launch_topw(const void *logits, int64_t row_stride, int rows, int V, int W, int dtype,
                      int32_t *ids, float *logprob, float *row_lse, void *ws, hipStream_t st)
{
    if (rows == 0)
        return JT_OK;
    const TopwPlan p = topw_plan(rows, V);
    const size_t parts = (size_t)rows * p.nlist;
    uint64_t *wk = reinterpret_cast<uint64_t *>(ws);
    uintptr_t mp = reinterpret_cast<uintptr_t>(wk + parts * W);
    mp = (mp + 15) & ~(uintptr_t)15;
    float2 *wm = reinterpret_cast<float2 *>(mp);
    const dim3 grid((unsigned)((parts + 3) / 4)), block(kTopwThreads);
    const uintptr_t addr = reinterpret_cast<uintptr_t>(logits);
    if (dtype == JT_BF16) {
        const bool al = (addr % 16 == 0) && (row_stride % 8 == 0);
        if (al)
            hipLaunchKernelGGL((topw_partial_kernel<uint16_t, true>), grid, block, 0, st,
                               (const uint16_t *)logits, row_stride, rows, V, W, p.npiece, p.ppw,
                               p.nlist, wk, wm);
        else
            hipLaunchKernelGGL((topw_partial_kernel<uint16_t, false>), grid, block, 0, st,
                               (const uint16_t *)logits, row_stride, rows, V, W, p.npiece, p.ppw,
                               p.nlist, wk, wm);
    } else {
        const bool al = (addr % 16 == 0) && (row_stride % 4 == 0);
        if (al)
            hipLaunchKernelGGL((topw_partial_kernel<float, true>), grid, block, 0, st,
                               (const float *)logits, row_stride, rows, V, W, p.npiece, p.ppw,
                               p.nlist, wk, wm);
        else
            hipLaunchKernelGGL((topw_partial_kernel<float, false>), grid, block, 0, st,
                               (const float *)logits, row_stride, rows, V, W, p.npiece, p.ppw,
                               p.nlist, wk, wm);
    }
    jt_status e = launch_status(hipGetLastError());
    if (e != JT_OK)
        return e;
    hipLaunchKernelGGL(topw_merge_kernel, dim3(rows), dim3(64), 0, st, rows, W, p.nlist, wk, wm,
                       ids, logprob, row_lse);
    return launch_status(hipGetLastError());
}

} // namespace jt
