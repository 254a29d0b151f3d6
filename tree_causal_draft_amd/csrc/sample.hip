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
//   sample_partial_kernel  streams every row once (HBM-bound, like the arg-max scan): each
//                          wave owns 2048-logit pieces of a row and writes every piece's
//                          maximum m and weight sum S = sum exp((x - m) / T) with wave
//                          reductions only; NaN entries weigh 0 and are flagged;
//   sample_select_kernel   one workgroup per row: Z and the piece whose cumulative weight
//                          passes r * Z from one block scan over the piece sums, then a
//                          rescan of that one piece (an L2 / Infinity Cache hit) with one
//                          block scan in token order for the exact token; the draw goes
//                          out as a one-entry arg-max key;
//   verify_walk_kernel     the greedy walk, reading the draws as its arg-max.
#include "jt_internal.h"

namespace jt {

constexpr int kSmpThreads = 256;
constexpr int kSmpPiece = 2048;       // logits per wave piece (32 per lane)
constexpr int kSmpMaxWaves = 16384;   // partial waves to aim for at most

struct SmpPlan {
    int npiece;  // pieces per row
    int ppw;     // pieces per wave
    int nwave;   // waves per row
};

static SmpPlan smp_plan(int rows, int V)
{
    SmpPlan p;
    p.npiece = (V + kSmpPiece - 1) / kSmpPiece;
    const long total = (long)rows * p.npiece;
    p.ppw = (int)max(1L, (total + kSmpMaxWaves - 1) / kSmpMaxWaves);
    p.nwave = (p.npiece + p.ppw - 1) / p.ppw;
    return p;
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

// 16 bytes of a row starting at element e0 (entries at or past V read as 0 bits)
template <typename T>
__device__ __forceinline__ uint4 smp_load16(const T *row, int64_t e0, int V, bool aligned)
{
    constexpr int E = AVec<T>::kElems;
    if (aligned && e0 + E <= V)
        return *reinterpret_cast<const uint4 *>(row + e0);
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
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// weight of one logit against reference m: exp((x - m) / T) as exp2((x - m) * c), c =
// log2(e) / T; a NaN, -inf or padding entry weighs 0
__device__ __forceinline__ float smp_weight(float x, float m, float c, bool in_range)
{
    const float e = __builtin_amdgcn_exp2f((x - m) * c);
    return (in_range && x == x && x != -INFINITY) ? e : 0.f;
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

// Each wave owns ppw consecutive 2048-logit pieces of one row (lane l holds elements
// (l + 64 i) * E .. + E - 1 of a piece) and writes each piece's (max, weight sum) and NaN
// bit; no workgroup barrier.  The next piece's loads are issued before the current one is
// reduced.
template <typename T>
__global__ void __launch_bounds__(kSmpThreads)
sample_partial_kernel(const T *__restrict__ logits, int64_t row_stride, int V, float c,
                      SmpPlan p, int rows, float2 *__restrict__ ws_ms,
                      uint32_t *__restrict__ ws_nan, bool aligned)
{
    constexpr int E = AVec<T>::kElems;
    constexpr int L = kSmpPiece / (kWave * E);  // 16-byte loads per lane per piece
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * (kSmpThreads / kWave) + (threadIdx.x >> 6);
    if (gw >= rows * p.nwave)
        return;
    const int r = gw / p.nwave, wv = gw % p.nwave;
    const T *row = logits + (int64_t)r * row_stride;
    const int pc0 = wv * p.ppw, pc1 = min(p.npiece, pc0 + p.ppw);
    uint4 nxt[L];
    auto load = [&](int pc, uint4 (&u)[L]) {
#pragma unroll
        for (int i = 0; i < L; ++i)
            u[i] = smp_load16<T>(row, (int64_t)pc * kSmpPiece + (int64_t)(lane + kWave * i) * E, V,
                                 aligned);
    };
    if (pc0 < pc1)
        load(pc0, nxt);
    for (int pc = pc0; pc < pc1; ++pc) {
        float x[L][E];
#pragma unroll
        for (int i = 0; i < L; ++i)
            smp_unpack<T>(nxt[i], x[i]);
        if (pc + 1 < pc1)
            load(pc + 1, nxt);
        const int64_t base = (int64_t)pc * kSmpPiece;
        float m = -INFINITY;
        bool nan = false;
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const int64_t e0 = base + (int64_t)(lane + kWave * i) * E;
#pragma unroll
            for (int k = 0; k < E; ++k)
                if (e0 + k < V) {
                    nan |= x[i][k] != x[i][k];
                    m = fmaxf(m, x[i][k]);
                }
        }
        const float M = wave_max_f32(m);
        float s = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                const int64_t e0 = base + (int64_t)(lane + kWave * i) * E;
#pragma unroll
                for (int k = 0; k < E; ++k)
                    s += smp_weight(x[i][k], M, c, e0 + k < V);
            }
        }
        const float S = wave_sum_f32(s);
        const bool any_nan = __ballot(nan) != 0ull;
        if (lane == 0) {
            ws_ms[(int64_t)r * p.npiece + pc] = make_float2(M, S);
            ws_nan[(int64_t)r * p.npiece + pc] = any_nan ? 1u : 0u;
        }
    }
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
    constexpr int PER = kSmpPiece / NT;  // logits of the rescanned piece per thread (8)
    static_assert(PER % E == 0, "whole 16-byte loads per thread");
    __shared__ float red[NT / 64];
    __shared__ int pick, lo_pos, hi_pos;
    __shared__ float pick_before;
    const int tid = threadIdx.x;
    const int r = blockIdx.x;
    const float2 *ms = ws_ms + (int64_t)r * p.npiece;
    const T *row = logits + (int64_t)r * row_stride;

    // row maximum and NaN bit
    float m = -INFINITY;
    uint32_t nb = 0u;
    for (int i = tid; i < p.npiece; i += NT) {
        m = fmaxf(m, ms[i].x);
        nb |= ws_nan[(int64_t)r * p.npiece + i];
    }
    const float M = block_max_f32(m, red);
    const bool nan = __syncthreads_or(nb != 0u);
    int draw = 0;  // a row with no finite maximum draws token 0, like its arg-max
    if (M != -INFINITY) {
        auto piece_w = [&](int i) {
            const float2 q = ms[i];
            return q.x == -INFINITY ? 0.f : q.y * __builtin_amdgcn_exp2f((q.x - M) * c);
        };
        // Z, then the piece where the cumulative weight passes r * Z: one block scan per
        // NT pieces (one in all for rows up to 524,288 logits)
        float Z = 0.f;
        for (int i0 = 0; i0 < p.npiece; i0 += NT) {
            const int i = i0 + tid;
            float tot;
            block_excl_scan_f32(i < p.npiece ? piece_w(i) : 0.f, red, &tot);
            Z += tot;
        }
        const float target = uniform[r] * Z;
        if (tid == 0) {
            pick = INT_MAX;
            pick_before = 0.f;
        }
        float carry = 0.f;
        int pc = -1;
        float before_pc = 0.f;
        for (int i0 = 0; i0 < p.npiece && pc < 0; i0 += NT) {
            const int i = i0 + tid;
            const float w = i < p.npiece ? piece_w(i) : 0.f;
            float tot;
            const float before = carry + block_excl_scan_f32(w, red, &tot);
            if (w > 0.f && before <= target && before + w > target)
                atomicMin(&pick, i);
            __syncthreads();
            if (pick != INT_MAX && i == pick)
                pick_before = before;
            __syncthreads();
            if (pick != INT_MAX) {
                pc = pick;
                before_pc = pick_before;
            }
            carry += tot;
        }
        if (pc < 0) {
            // rounding left r * Z past the last piece: the last piece with weight, entered
            // at its end (its last weighted logit is drawn below)
            if (tid == 0) {
                int last = 0;
                for (int i = p.npiece - 1; i >= 0; --i)
                    if (piece_w(i) > 0.f) {
                        last = i;
                        break;
                    }
                pick = last;
            }
            __syncthreads();
            pc = pick;
            before_pc = -INFINITY;  // the crossing search below then fails, past the end
        }
        // rescan piece pc in token order: thread tid holds logits PER*tid .. PER*tid+PER-1
        const int64_t base = (int64_t)pc * kSmpPiece + (int64_t)tid * PER;
        float x[PER];
#pragma unroll
        for (int q = 0; q < PER / E; ++q) {
            const uint4 u = smp_load16<T>(row, base + q * E, V, aligned);
            float xe[E];
            smp_unpack<T>(u, xe);
#pragma unroll
            for (int k = 0; k < E; ++k)
                x[q * E + k] = xe[k];
        }
        float w[PER], s = 0.f;
        int first_pos = INT_MAX, last_pos = -1;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            w[k] = smp_weight(x[k], M, c, base + k < V);
            s += w[k];
            if (w[k] > 0.f) {
                first_pos = min(first_pos, (int)(base + k));
                last_pos = max(last_pos, (int)(base + k));
            }
        }
        float tot;
        float cum = before_pc + block_excl_scan_f32(s, red, &tot);
        if (tid == 0) {
            pick = INT_MAX;
            lo_pos = INT_MAX;
            hi_pos = -1;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const float nx = cum + w[k];
            if (w[k] > 0.f && cum <= target && nx > target)
                atomicMin(&pick, (int)(base + k));
            cum = nx;
        }
        if (first_pos != INT_MAX)
            atomicMin(&lo_pos, first_pos);
        if (last_pos >= 0)
            atomicMax(&hi_pos, last_pos);
        __syncthreads();
        // no crossing inside (rounding near an end of the piece): its first or last
        // weighted logit, whichever end the target lies past (-inf start: past the end)
        if (pick != INT_MAX)
            draw = pick;
        else
            draw = (before_pc != -INFINITY && target < before_pc) ? lo_pos : hi_pos;
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
    return (size_t)rows * p.npiece * (sizeof(float2) + sizeof(uint32_t)) +
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
    float2 *ms = reinterpret_cast<float2 *>(take((size_t)rows * p.npiece * sizeof(float2)));
    uint32_t *nanr = reinterpret_cast<uint32_t *>(take((size_t)rows * p.npiece * sizeof(uint32_t)));
    uint64_t *keys = reinterpret_cast<uint64_t *>(take((size_t)rows * sizeof(uint64_t)));
    uint32_t *nanw = reinterpret_cast<uint32_t *>(take((size_t)rows * sizeof(uint32_t)));
    const float c = 1.4426950408889634f / temperature;
    const uintptr_t addr = reinterpret_cast<uintptr_t>(logits);
    const long waves = (long)rows * p.nwave;
    const dim3 g1((unsigned)((waves + 3) / 4)), g2((unsigned)rows), blk(kSmpThreads);
    if (dtype == JT_BF16) {
        const bool al = addr % 16 == 0 && row_stride % 8 == 0;
        hipLaunchKernelGGL(sample_partial_kernel<uint16_t>, g1, blk, 0, st,
                           (const uint16_t *)logits, row_stride, V, c, p, rows, ms, nanr, al);
        hipLaunchKernelGGL(sample_select_kernel<uint16_t>, g2, blk, 0, st,
                           (const uint16_t *)logits, row_stride, V, c, p, uniform, ms, nanr,
                           keys, nanw, sample_out, al);
    } else {
        const bool al = addr % 16 == 0 && row_stride % 4 == 0;
        hipLaunchKernelGGL(sample_partial_kernel<float>, g1, blk, 0, st, (const float *)logits,
                           row_stride, V, c, p, rows, ms, nanr, al);
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
