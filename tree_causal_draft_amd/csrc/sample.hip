// Stochastic tree verification: one target draw per node, then the verification walk.
//
// With a fixed draft each proposal is a point mass at the draft token, accepted with the
// target probability, and a rejected position takes a draw from the residual, so every
// committed token is the target's own draw at any temperature (JetSpec review, inference,
// acceptance equation; JetSpec++ summary, appendices F.1 and F.3).  Sibling tokens are
// distinct, so at a node this is the same in distribution as one draw x ~ softmax(logits /
// T): descend to the child carrying x, or stop with bonus x.  The draw is the inverse of
// the cumulative distribution in token-id order at the caller's uniform r: the first t
// whose cumulative weight exceeds r * Z.
//
// Three launches:
//   sample_partial_kernel  streams every row once (HBM-bound, like the arg-max scan): per
//                          8192-logit sub-chunk, its maximum m and weight sum
//                          S = sum exp((x - m) / T); NaN entries weigh 0 and are flagged;
//   sample_select_kernel   one workgroup per row: Z from the sub-chunk sums, the sub-chunk
//                          whose cumulative weight passes r * Z, then a rescan of that one
//                          sub-chunk (an L2 / Infinity Cache hit) with block scans for the
//                          exact token; the draw goes out as a one-entry arg-max key;
//   verify_walk_kernel     the greedy walk, reading the draws as its arg-max.
#include "jt_internal.h"

namespace jt {

constexpr int kSmpThreads = 256;

struct SmpPlan {
    int nsub, sub_per_wg, nrun;  // sub-chunks per row, per workgroup, workgroups per row
};

static SmpPlan smp_plan(int rows, int V)
{
    SmpPlan p;
    p.nsub = (V + kArgSub - 1) / kArgSub;
    const int want = rows > 0 ? (2048 + rows - 1) / rows : 1;  // workgroups per row
    int spw = (p.nsub + want - 1) / want;
    if (spw < 1)
        spw = 1;
    p.sub_per_wg = spw;
    p.nrun = (p.nsub + spw - 1) / spw;
    return p;
}

// Words of a thread's share of sub-chunk sc: element k of load i is element
// (tid + NT*i)*E + k of the sub-chunk (entries at or past V are left 0 and masked later).
template <typename T, int NT, int L>
__device__ __forceinline__ void smp_load(const T *row, int64_t base, int V, int tid, bool aligned,
                                         uint4 (&u)[L])
{
    constexpr int E = AVec<T>::kElems;
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int64_t e0 = base + (int64_t)(tid + NT * i) * E;
        if (aligned && e0 + E <= V) {
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
}

template <typename T>
__device__ __forceinline__ void smp_unpack(const uint4 &u, float (&x)[AVec<T>::kElems])
{
    if constexpr (sizeof(T) == 2) {
        x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
        x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z); x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
    } else {
        x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
        x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
    }
}

// weight of one logit against reference m: exp((x - m) / T) as exp2((x - m) * c), c =
// log2(e) / T; a NaN, -inf or padding entry weighs 0
__device__ __forceinline__ float smp_weight(float x, float m, float c, bool in_range)
{
    const float e = __builtin_amdgcn_exp2f((x - m) * c);
    return (in_range && x == x && x != -INFINITY) ? e : 0.f;
}

__device__ __forceinline__ float block_sum_f32(float v, float *red)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o, kWave);
    __syncthreads();
    if (lane == 0)
        red[wid] = v;
    __syncthreads();
    float t = 0.f;
    for (int w = 0; w < nw; ++w)
        t += red[w];
    return t;
}
__device__ __forceinline__ float block_max_f32(float v, float *red)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    v = wave_max_f32(v);
    __syncthreads();
    if (lane == 0)
        red[wid] = v;
    __syncthreads();
    float t = -INFINITY;
    for (int w = 0; w < nw; ++w)
        t = fmaxf(t, red[w]);
    return t;
}
// exclusive prefix sum over the block in thread order; *total gets the block sum
__device__ __forceinline__ float block_excl_scan_f32(float v, float *red, float *total)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    float inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(inc, o, kWave);
        if (lane >= o)
            inc += y;
    }
    __syncthreads();
    if (lane == 63)
        red[wid] = inc;
    __syncthreads();
    float before = 0.f, all = 0.f;
    for (int w = 0; w < nw; ++w) {
        if (w < wid)
            before += red[w];
        all += red[w];
    }
    *total = all;
    return before + inc - v;
}

// Per (row, run of sub-chunks): each sub-chunk's (max, weight sum), and the run's NaN bit.
template <typename T>
__global__ void __launch_bounds__(kSmpThreads)
sample_partial_kernel(const T *__restrict__ logits, int64_t row_stride, int V, float c,
                      SmpPlan p, float2 *__restrict__ ws_ms, uint32_t *__restrict__ ws_nan,
                      bool aligned)
{
    constexpr int E = AVec<T>::kElems;
    constexpr int NT = kSmpThreads;
    constexpr int L = kArgSub / (E * NT);
    __shared__ float red[NT / 64];
    const int tid = threadIdx.x;
    const int row_idx = blockIdx.x / p.nrun, run = blockIdx.x % p.nrun;
    const T *row = logits + (int64_t)row_idx * row_stride;
    const int sc0 = run * p.sub_per_wg, sc1 = min(p.nsub, sc0 + p.sub_per_wg);
    bool nan = false;
    uint4 u[L];
    if (sc0 < sc1)
        smp_load<T, NT, L>(row, (int64_t)sc0 * kArgSub, V, tid, aligned, u);
    for (int sc = sc0; sc < sc1; ++sc) {
        const int64_t base = (int64_t)sc * kArgSub;
        float x[L][E];
#pragma unroll
        for (int i = 0; i < L; ++i)
            smp_unpack<T>(u[i], x[i]);
        if (sc + 1 < sc1)  // the next sub-chunk's loads overlap this one's reductions
            smp_load<T, NT, L>(row, base + kArgSub, V, tid, aligned, u);
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const int64_t e0 = base + (int64_t)(tid + NT * i) * E;
#pragma unroll
            for (int k = 0; k < E; ++k) {
                if (e0 + k < V) {
                    nan |= x[i][k] != x[i][k];
                    m = fmaxf(m, x[i][k]);
                }
            }
        }
        const float M = block_max_f32(m, red);
        float s = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                const int64_t e0 = base + (int64_t)(tid + NT * i) * E;
#pragma unroll
                for (int k = 0; k < E; ++k)
                    s += smp_weight(x[i][k], M, c, e0 + k < V);
            }
        }
        const float S = block_sum_f32(s, red);
        if (tid == 0)
            ws_ms[(int64_t)row_idx * p.nsub + sc] = make_float2(M, S);
    }
    const bool any = __syncthreads_or(nan);
    if (tid == 0)
        ws_nan[blockIdx.x] = any ? 1u : 0u;
}

// One workgroup per row: the draw.  Writes a one-entry arg-max key (any nonzero order
// code, id = the draw) and NaN bit per row for the walk, and the draw to sample_out.
template <typename T>
__global__ void __launch_bounds__(kSmpThreads)
sample_select_kernel(const T *__restrict__ logits, int64_t row_stride, int V, float c,
                     SmpPlan p, const float *__restrict__ uniform,
                     const float2 *__restrict__ ws_ms, const uint32_t *__restrict__ ws_nan,
                     uint64_t *__restrict__ keys, uint32_t *__restrict__ nan_out,
                     int32_t *__restrict__ sample_out, bool aligned)
{
    constexpr int E = AVec<T>::kElems;
    constexpr int NT = kSmpThreads;
    constexpr int L = kArgSub / (E * NT);
    __shared__ float red[NT / 64];
    __shared__ int pick;
    const int tid = threadIdx.x;
    const int r = blockIdx.x;
    const float2 *ms = ws_ms + (int64_t)r * p.nsub;
    const T *row = logits + (int64_t)r * row_stride;

    // row maximum and NaN bit
    float m = -INFINITY;
    for (int i = tid; i < p.nsub; i += NT)
        m = fmaxf(m, ms[i].x);
    const float M = block_max_f32(m, red);
    uint32_t nb = 0u;
    for (int i = tid; i < p.nrun; i += NT)
        nb |= ws_nan[(int64_t)r * p.nrun + i];
    const bool nan = __syncthreads_or(nb != 0u);
    int draw = 0;  // a row with no finite maximum draws token 0, like its arg-max
    if (M != -INFINITY) {
        // sub-chunk weights against M, Z, and the sub-chunk where the cumulative weight
        // passes r * Z (blocks of NT sub-chunks, scanned in order)
        float Z = 0.f;
        for (int i0 = 0; i0 < p.nsub; i0 += NT) {
            const int i = i0 + tid;
            const float2 q = i < p.nsub ? ms[i] : make_float2(-INFINITY, 0.f);
            const float w = q.x == -INFINITY ? 0.f : q.y * __builtin_amdgcn_exp2f((q.x - M) * c);
            Z += block_sum_f32(w, red);
        }
        const float target = uniform[r] * Z;
        float carry = 0.f;
        int sc = -1;
        for (int i0 = 0; i0 < p.nsub && sc < 0; i0 += NT) {
            const int i = i0 + tid;
            const float2 q = i < p.nsub ? ms[i] : make_float2(-INFINITY, 0.f);
            const float w = q.x == -INFINITY ? 0.f : q.y * __builtin_amdgcn_exp2f((q.x - M) * c);
            float tot;
            const float before = carry + block_excl_scan_f32(w, red, &tot);
            __syncthreads();
            if (tid == 0)
                pick = INT_MAX;
            __syncthreads();
            if (i < p.nsub && w > 0.f && before + w > target && before <= target)
                atomicMin(&pick, i);
            __syncthreads();
            if (pick != INT_MAX)
                sc = pick;
            carry += tot;
            __syncthreads();
        }
        // rounding can leave r * Z past the last sub-chunk: take the last with weight
        __shared__ int last_sc;
        if (sc < 0) {
            if (tid == 0) {
                last_sc = 0;
                for (int i = p.nsub - 1; i >= 0; --i)
                    if (ms[i].x != -INFINITY && ms[i].y > 0.f) {
                        last_sc = i;
                        break;
                    }
            }
            __syncthreads();
            sc = last_sc;
        }
        // cumulative weight before sub-chunk sc, in the same order as above
        float before_sc = 0.f;
        for (int i0 = 0; i0 < sc; i0 += NT) {
            const int i = i0 + tid;
            const float2 q = i < sc ? ms[i] : make_float2(-INFINITY, 0.f);
            const float w = q.x == -INFINITY ? 0.f : q.y * __builtin_amdgcn_exp2f((q.x - M) * c);
            before_sc += block_sum_f32(w, red);
        }
        // rescan sub-chunk sc in token order: load i covers elements [2048 i, 2048 i + 2048)
        // of the sub-chunk, thread tid the E of them at 2048 i + E tid
        uint4 u[L];
        const int64_t base = (int64_t)sc * kArgSub;
        smp_load<T, NT, L>(row, base, V, tid, aligned, u);
        __syncthreads();
        if (tid == 0)
            pick = INT_MAX;
        int first_pos = INT_MAX, last_pos = -1;  // weighted elements of this thread
        float run = before_sc;
#pragma unroll
        for (int i = 0; i < L; ++i) {
            float x[E];
            smp_unpack<T>(u[i], x);
            const int64_t e0 = base + (int64_t)(tid + NT * i) * E;
            float w[E], s = 0.f;
#pragma unroll
            for (int k = 0; k < E; ++k) {
                w[k] = smp_weight(x[k], M, c, e0 + k < V);
                s += w[k];
                if (w[k] > 0.f) {
                    first_pos = min(first_pos, (int)(e0 + k));
                    last_pos = max(last_pos, (int)(e0 + k));
                }
            }
            float tot;
            float cum = run + block_excl_scan_f32(s, red, &tot);
#pragma unroll
            for (int k = 0; k < E; ++k) {
                const float nxt = cum + w[k];
                if (w[k] > 0.f && cum <= target && nxt > target)
                    atomicMin(&pick, (int)(e0 + k));
                cum = nxt;
            }
            run += tot;
        }
        // no crossing inside (rounding near an end of the sub-chunk): its first or last
        // weighted element, whichever end the target lies past
        __shared__ int lo_pos, hi_pos;
        if (tid == 0) {
            lo_pos = INT_MAX;
            hi_pos = -1;
        }
        __syncthreads();
        if (first_pos != INT_MAX)
            atomicMin(&lo_pos, first_pos);
        if (last_pos >= 0)
            atomicMax(&hi_pos, last_pos);
        __syncthreads();
        if (pick != INT_MAX)
            draw = pick;
        else
            draw = target < before_sc ? lo_pos : hi_pos;
        if (draw < 0 || draw == INT_MAX)
            draw = 0;
    }
    if (tid == 0) {
        keys[r] = rank_key(0.f, (uint32_t)draw);
        nan_out[r] = nan ? 1u : 0u;
        if (sample_out)
            sample_out[r] = draw;
    }
}

size_t sample_workspace(int S, int B, int V)
{
    const int rows = S * B;
    const SmpPlan p = smp_plan(rows, V);
    return (size_t)rows * p.nsub * sizeof(float2) + (size_t)rows * p.nrun * sizeof(uint32_t) +
           (size_t)rows * (sizeof(uint64_t) + sizeof(uint32_t)) + 1024;
}

jt_status launch_verify_sampled(const void *logits, int64_t row_stride, int V, int dtype,
                                float temperature, const float *uniform, const int32_t *parent,
                                const int32_t *tokens, const uint64_t *anc, const int32_t *depth,
                                int S, int B, int N, int32_t *accept_len, int32_t *accept_path,
                                int32_t *bonus, int32_t *sample_out, int32_t *err, void *ws,
                                hipStream_t st)
{
    if (S == 0)
        return JT_OK;
    const int rows = S * B;
    const SmpPlan p = smp_plan(rows, V);
    uint8_t *w = static_cast<uint8_t *>(ws);
    auto take = [&](size_t bytes) {
        uint8_t *q = w;
        w += (bytes + 255) & ~(size_t)255;
        return q;
    };
    float2 *ms = reinterpret_cast<float2 *>(take((size_t)rows * p.nsub * sizeof(float2)));
    uint32_t *nanr = reinterpret_cast<uint32_t *>(take((size_t)rows * p.nrun * sizeof(uint32_t)));
    uint64_t *keys = reinterpret_cast<uint64_t *>(take((size_t)rows * sizeof(uint64_t)));
    uint32_t *nanw = reinterpret_cast<uint32_t *>(take((size_t)rows * sizeof(uint32_t)));
    const float c = 1.4426950408889634f / temperature;
    const uintptr_t addr = reinterpret_cast<uintptr_t>(logits);
    const dim3 g1((unsigned)(rows * p.nrun)), g2((unsigned)rows), blk(kSmpThreads);
    if (dtype == JT_BF16) {
        const bool al = addr % 16 == 0 && row_stride % 8 == 0;
        hipLaunchKernelGGL(sample_partial_kernel<uint16_t>, g1, blk, 0, st,
                           (const uint16_t *)logits, row_stride, V, c, p, ms, nanr, al);
        hipLaunchKernelGGL(sample_select_kernel<uint16_t>, g2, blk, 0, st,
                           (const uint16_t *)logits, row_stride, V, c, p, uniform, ms, nanr,
                           keys, nanw, sample_out, al);
    } else {
        const bool al = addr % 16 == 0 && row_stride % 4 == 0;
        hipLaunchKernelGGL(sample_partial_kernel<float>, g1, blk, 0, st, (const float *)logits,
                           row_stride, V, c, p, ms, nanr, al);
        hipLaunchKernelGGL(sample_select_kernel<float>, g2, blk, 0, st, (const float *)logits,
                           row_stride, V, c, p, uniform, ms, nanr, keys, nanw, sample_out, al);
    }
    jt_status e = launch_status(hipGetLastError());
    if (e != JT_OK)
        return e;
    return launch_verify_walk(parent, tokens, anc, depth, S, B, N, 1, keys, nanw, accept_len,
                              accept_path, bonus, nullptr, err, st);
}

} // namespace jt
