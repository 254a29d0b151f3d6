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
//                          passes r * Z from a wave prefix sum over the piece sums, then a
//                          rescan of that one piece (an L2 / Infinity Cache hit) in token
//                          order for the exact token; the draw goes out as a one-entry
//                          arg-max key;
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

// Each wave owns ppw consecutive 2048-logit pieces of one row (lane l holds elements
// (l + 64 i) * E .. + E - 1 of a piece) and writes each piece's (max, weight sum) and NaN
// bit; no workgroup barrier.  The next piece's loads are issued before the current one is
// reduced.
//
// A whole, aligned piece first takes an unmasked pass: the maximum with the 3-operand
// NaN-propagating maximum and four unmasked partial sums.  A NaN logit makes its own weight,
// and so the sum, NaN whatever the maximum came out as; a -inf logit weighs exp2(-inf) = 0
// already; so a finite sum with a finite maximum is the masked pass's result up to the order
// of the additions, and anything else (a NaN, +inf, a piece of -inf only, the row's ragged
// last piece) is redone by the masked pass.
template <typename T>
__global__ void __launch_bounds__(kSmpThreads)
sample_partial_kernel(const T *__restrict__ logits, int64_t row_stride, int V, float c,
                      SmpPlan p, int rows, float2 *__restrict__ ws_ms,
                      uint32_t *__restrict__ ws_nan, bool aligned)
{
    constexpr int E = AVec<T>::kElems;
    constexpr int L = kSmpPiece / (kWave * E);  // 16-byte loads per lane per piece
    constexpr int NX = L * E;                   // logits per lane per piece
    const int lane = threadIdx.x & 63;
    // wave-uniform, so that the piece loop and its branches stay scalar
    const int gw = __builtin_amdgcn_readfirstlane(blockIdx.x * (kSmpThreads / kWave) +
                                                  (threadIdx.x >> 6));
    if (gw >= rows * p.nwave)
        return;
    const int r = gw / p.nwave, wv = gw % p.nwave;
    const T *row = logits + (int64_t)r * row_stride;
    const int pc0 = wv * p.ppw, pc1 = min(p.npiece, pc0 + p.ppw);
    // pieces [0, nfull) lie wholly inside the row (and are 16-byte aligned when it is)
    const int nfull = aligned ? V / kSmpPiece : 0;
    uint4 nxt[L];
    auto load = [&](int pc, uint4 (&u)[L]) {
        const int64_t e0 = (int64_t)pc * kSmpPiece + (int64_t)lane * E;
        if (pc < nfull) {
#pragma unroll
            for (int i = 0; i < L; ++i)
                u[i] = *reinterpret_cast<const uint4 *>(row + e0 + kWave * E * i);
        } else {
#pragma unroll
            for (int i = 0; i < L; ++i)
                u[i] = smp_load16<T>(row, e0 + kWave * E * i, V, aligned);
        }
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
        float M = -INFINITY, S = __builtin_nanf("");
        if (pc < nfull) {
            float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
            for (int j = 0; j < NX; j += 2) {
                m0 = __builtin_elementwise_maximum(m0, x[j / E][j % E]);
                m1 = __builtin_elementwise_maximum(m1, x[j / E][j % E + 1]);
            }
            M = wave_max_f32(__builtin_elementwise_maximum(m0, m1));
            float s4[4];
#pragma unroll
            for (int j = 0; j < NX; ++j) {
                const float w = __builtin_amdgcn_exp2f((x[j / E][j % E] - M) * c);
                s4[j & 3] = j < 4 ? w : s4[j & 3] + w;
            }
            S = wave_sum_f32((s4[0] + s4[1]) + (s4[2] + s4[3]));
        }
        bool any_nan = false;
        if (!(M > -INFINITY && M < INFINITY && S == S)) {
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
            M = wave_max_f32(m);
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
            S = wave_sum_f32(s);
            any_nan = __ballot(nan) != 0ull;
        }
        if (lane == 0) {
            ws_ms[(int64_t)r * p.npiece + pc] = make_float2(M, S);
            ws_nan[(int64_t)r * p.npiece + pc] = any_nan ? 1u : 0u;
        }
    }
}

// One workgroup per row: the draw.  Writes a one-entry arg-max key (any nonzero order
// code, id = the draw) and NaN bit per row for the walk, and the draw to sample_out.
//
// Every wave finds the piece by itself from the piece sums (wave reductions and a DPP
// prefix sum, no LDS): the same instructions on the same data, so the same piece in each.
// The four waves then share the rescan of that piece in token order, with one exchange of
// wave totals and one of per-wave results through LDS.
template <typename T>
__global__ void __launch_bounds__(kSmpThreads)
sample_select_kernel(const T *__restrict__ logits, int64_t row_stride, int V, float c,
                     SmpPlan p, const float *__restrict__ uniform,
                     const float2 *__restrict__ ws_ms, const uint32_t *__restrict__ ws_nan,
                     uint64_t *__restrict__ keys, uint32_t *__restrict__ nan_out,
                     int32_t *__restrict__ sample_out, bool aligned)
{
    constexpr int E = AVec<T>::kElems;
    constexpr int NWV = kSmpThreads / kWave;
    constexpr int PER = kSmpPiece / kSmpThreads;  // logits of the rescanned piece per thread (8)
    constexpr int KP = 4;                         // piece sums per lane per chunk
    constexpr int CH = kWave * KP;                // pieces per chunk
    static_assert(PER % E == 0, "whole 16-byte loads per thread");
    __shared__ float wtot[NWV];
    __shared__ int wpick[NWV], wlo[NWV], whi[NWV];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int r = blockIdx.x;
    const float2 *ms = ws_ms + (int64_t)r * p.npiece;
    const uint32_t *nr = ws_nan + (int64_t)r * p.npiece;
    const T *row = logits + (int64_t)r * row_stride;
    const float u = uniform[r];

    // row maximum and NaN bit
    float m = -INFINITY;
    uint32_t nb = 0u;
    for (int i = lane; i < p.npiece; i += kWave) {
        m = fmaxf(m, ms[i].x);
        nb |= nr[i];
    }
    const float M = wave_max_f32(m);
    const bool nan = __ballot(nb != 0u) != 0ull;
    int draw = 0;  // a row with no finite maximum draws token 0, like its arg-max
    if (M != -INFINITY) {
        auto piece_w = [&](int i) {
            if (i >= p.npiece)
                return 0.f;
            const float2 q = ms[i];
            return q.x == -INFINITY ? 0.f : q.y * __builtin_amdgcn_exp2f((q.x - M) * c);
        };
        // Z over chunks of CH pieces, lane l holding pieces KP l .. KP l + KP - 1 of each
        float Z = 0.f;
        for (int i0 = 0; i0 < p.npiece; i0 += CH) {
            float s = 0.f;
#pragma unroll
            for (int k = 0; k < KP; ++k)
                s += piece_w(i0 + lane * KP + k);
            Z += wave_sum_f32(s);
        }
        const float target = u * Z;
        // the piece whose cumulative interval [before, before + w) holds the target
        int pc = -1;
        float before_pc = 0.f, carry = 0.f;
        for (int i0 = 0; i0 < p.npiece && pc < 0; i0 += CH) {
            float w[KP], s = 0.f;
#pragma unroll
            for (int k = 0; k < KP; ++k) {
                w[k] = piece_w(i0 + lane * KP + k);
                s += w[k];
            }
            const float incl = wave_incl_scan_f32(s);
            float b = carry + (incl - s);
            int hit = -1;
            float hb = 0.f;
#pragma unroll
            for (int k = 0; k < KP; ++k) {
                if (hit < 0 && w[k] > 0.f && b <= target && b + w[k] > target) {
                    hit = i0 + lane * KP + k;
                    hb = b;
                }
                b += w[k];
            }
            const uint64_t any = __ballot(hit >= 0);
            if (any) {
                const int at = __builtin_ctzll(any);
                pc = __builtin_amdgcn_readlane(hit, at);
                before_pc = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hb), at));
            }
            carry += __builtin_bit_cast(float,
                                        __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 63));
        }
        if (pc < 0) {
            // rounding left r * Z past the last piece: the last piece with weight, entered
            // at its end (its last weighted logit is drawn below)
            int last = -1;
            for (int i = lane; i < p.npiece; i += kWave)
                if (piece_w(i) > 0.f)
                    last = i;
            const uint64_t any = __ballot(last >= 0);
            pc = any ? __builtin_amdgcn_readlane(last, 63 - __builtin_clzll(any)) : 0;
            before_pc = -INFINITY;  // the crossing search below then fails, past the end
        }
        // rescan piece pc in token order: thread t holds logits PER t .. PER t + PER - 1
        const int64_t base = (int64_t)pc * kSmpPiece + (int64_t)threadIdx.x * PER;
        float x[PER];
#pragma unroll
        for (int q = 0; q < PER / E; ++q) {
            const uint4 v = smp_load16<T>(row, base + q * E, V, aligned);
            float xe[E];
            smp_unpack<T>(v, xe);
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
        const float incl = wave_incl_scan_f32(s);
        if (lane == 63)
            wtot[wid] = incl;
        __syncthreads();
        float off = 0.f;
        for (int q = 0; q < wid; ++q)
            off += wtot[q];
        float cum = before_pc + (off + (incl - s));
        int hit = INT_MAX;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const float nx = cum + w[k];
            if (hit == INT_MAX && w[k] > 0.f && cum <= target && nx > target)
                hit = (int)(base + k);
            cum = nx;
        }
        const uint64_t bh = __ballot(hit != INT_MAX), bl = __ballot(first_pos != INT_MAX),
                       bu = __ballot(last_pos >= 0);
        if (lane == 0) {
            wpick[wid] = bh ? __builtin_amdgcn_readlane(hit, __builtin_ctzll(bh)) : INT_MAX;
            wlo[wid] = bl ? __builtin_amdgcn_readlane(first_pos, __builtin_ctzll(bl)) : INT_MAX;
            whi[wid] = bu ? __builtin_amdgcn_readlane(last_pos, 63 - __builtin_clzll(bu)) : -1;
        }
        __syncthreads();
        int pick = INT_MAX, lo_pos = INT_MAX, hi_pos = -1;
#pragma unroll
        for (int q = 0; q < NWV; ++q) {
            pick = min(pick, wpick[q]);
            lo_pos = min(lo_pos, wlo[q]);
            hi_pos = max(hi_pos, whi[q]);
        }
        // no crossing inside (rounding near an end of the piece): its first or last
        // weighted logit, whichever end the target lies past (-inf start: past the end)
        if (pick != INT_MAX)
            draw = pick;
        else
            draw = (before_pc != -INFINITY && target < before_pc) ? lo_pos : hi_pos;
        if (draw < 0 || draw == INT_MAX)
            draw = 0;
    }
    if (threadIdx.x == 0) {
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
