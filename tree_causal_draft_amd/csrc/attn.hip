// Step 2: tree-causal GQA attention -- every tree node in one pass.
//
// Node v of sequence s sees every prefix key of s, its ancestors and itself, never a
// sibling or a descendant (JetSpec review, startedourmission.github.io, "How it works",
// mask equation; paperlayer.ai JetSpec summary, section 2 "Architecture").  The verifier
// runs all nodes in one forward with this mask and no dense per-request matrix
// (paperlayer.ai JetSpec summary, appendix E "Verification"); the mask arrives here as
// the 256-bit ancestor rows of the mask step.
//
// Keys live in one virtual sequence per (s, KV head g): prefix keys 0..P-1 followed by
// tree keys P..P+B-1.  Ancestors of v have indices <= v, so a workgroup whose deepest row
// belongs to node v_hi never needs keys past P + v_hi (causal trim of the tree part).
//
// bf16 -> attn_mfma_kernel.  The G query heads of a KV group times the B nodes form the
// rows of one dense problem (row r = node r / G, head r % G), so every K/V tile staged
// in LDS is shared by all G*B rows.  Per 64-key tile and 16-row block a wave runs
//   S^T = K . Q^T    v_mfma_f32_16x16x32_bf16, K from LDS (row-major), Q in registers
//   online softmax   exp2 domain, per-lane running max / partial sum
//   O^T += V^T . P^T  V^T from LDS (written transposed), P^T straight from the S^T
//                     accumulators (the key permutation is applied to V^T's reads)
// Long prefixes with few rows are split over workgroups (split-KV); each split writes a
// normalised fp32 partial and its log2-sum-exp, and attn_combine_kernel merges them.
//
// fp32 -> attn_simple_kernel: one workgroup per (s, v, g) on the vector ALU.
#include "jt_internal.h"

namespace jt {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2eA = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- shared helpers --

// Element offset of K/V row of virtual key j (j < P: prefix, else tree node j - P) for
// sequence s and KV head g; -1 when the key is absent (past the range, or a bad block).
__device__ __forceinline__ int64_t kv_offset(const AttnArgs &a, int s, int g, int P, int j)
{
    if (j < P) {
        if (!a.block_table)
            return (((int64_t)s * a.max_prefix + j) * a.Hkv + g) * a.d;
        const int lb = j >> a.block_shift;
        const int blk = a.block_table[(int64_t)s * a.max_blocks + lb];
        if (blk < 0 || blk >= a.num_blocks)
            return -1;
        const int slot = j & (a.block_size - 1);
        return (((int64_t)blk * a.block_size + slot) * a.Hkv + g) * a.d;
    }
    const int u = j - P;
    if (u >= a.B)
        return -1;
    return (((int64_t)s * a.B + u) * a.Hkv + g) * a.d;
}

__device__ __forceinline__ int clamp_prefix(const AttnArgs &a, int s)
{
    int P = a.prefix_len[s];
    return P < 0 ? 0 : (P > a.max_prefix ? a.max_prefix : P);
}

// err[s] for one sequence: prefix length range and the blocks the prefix needs.
__device__ void attn_validate(const AttnArgs &a, int s)
{
    __shared__ int flag;
    if (threadIdx.x == 0)
        flag = 0;
    __syncthreads();
    const int Praw = a.prefix_len[s];
    int f = (Praw < 0 || Praw > a.max_prefix) ? JT_DEV_BAD_PREFIX : 0;
    if (a.block_table) {
        const int P = clamp_prefix(a, s);
        const int nb = (P + a.block_size - 1) >> a.block_shift;
        for (int b = threadIdx.x; b < nb; b += blockDim.x) {
            const int blk = b < a.max_blocks ? a.block_table[(int64_t)s * a.max_blocks + b] : -1;
            if (blk < 0 || blk >= a.num_blocks)
                f |= JT_DEV_BAD_BLOCK;
        }
    }
    if (f)
        atomicOr(&flag, f);
    __syncthreads();
    if (threadIdx.x == 0)
        a.err[s] = flag;
}

// ------------------------------------------------------------------ VALU kernel --

template <typename T>
__device__ __forceinline__ float ld(const T *p, int64_t i)
{
    if constexpr (sizeof(T) == 2)
        return bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[i]);
    else
        return p[i];
}
template <typename T> __device__ __forceinline__ void st(T *p, int64_t i, float v)
{
    if constexpr (sizeof(T) == 2)
        reinterpret_cast<uint16_t *>(p)[i] = f32_to_bf16(v);
    else
        p[i] = v;
}

// grid (B, S*Hkv); 256 threads; one node v and its G heads per workgroup.
template <typename T>
__global__ void __launch_bounds__(256) attn_simple_kernel(AttnArgs a)
{
    __shared__ float qs[8][128];
    __shared__ float ps[8][64];
    __shared__ float alpha_s[8];
    __shared__ float m_s[8], l_s[8];
    const int v = blockIdx.x;
    const int s = blockIdx.y / a.Hkv, g = blockIdx.y % a.Hkv;
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int D = a.d, G = a.G;
    const T *q = reinterpret_cast<const T *>(a.q);
    const T *kp = reinterpret_cast<const T *>(a.k_prefix);
    const T *vp = reinterpret_cast<const T *>(a.v_prefix);
    const T *kt = reinterpret_cast<const T *>(a.k_tree);
    const T *vt = reinterpret_cast<const T *>(a.v_tree);

    if (a.err && v == 0 && g == 0)
        attn_validate(a, s);
    const int P = clamp_prefix(a, s);
    const float c = a.scale * kLog2eA;
    for (int i = t; i < G * D; i += 256) {
        const int hh = i / D, e = i % D;
        qs[hh][e] = ld(q, (((int64_t)s * a.B + v) * a.Hq + g * G + hh) * D + e) * c;
    }
    if (t < G) {
        m_s[t] = -INFINITY;
        l_s[t] = 0.f;
    }
    const uint64_t *ar = a.anc + ((int64_t)s * a.B + v) * 4;
    const uint64_t w0 = ar[0], w1 = ar[1], w2 = ar[2], w3 = ar[3];
    __syncthreads();

    // PV ownership: column e = t % D, heads t / D + k * (256 / D)
    const int e = t % D;
    const int hstep = 256 / D;
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        acc[k] = 0.f;

    const int kend = P + v + 1;
    for (int k0 = 0; k0 < kend; k0 += 64) {
        // scores: key k0 + lane, heads wid, wid + 4
        const int j = k0 + lane;
        int64_t off = -1;
        if (j < kend) {
            off = kv_offset(a, s, g, P, j);
            if (j >= P) {
                const int u = j - P;
                const uint64_t wsel = u < 64 ? w0 : u < 128 ? w1 : u < 192 ? w2 : w3;
                if (!((wsel >> (u & 63)) & 1ull))
                    off = -1;
            }
        }
        const T *kb = j < P ? kp : kt;
        for (int hh = wid; hh < G; hh += 4) {
            float sc = -INFINITY;
            if (off >= 0) {
                float dot = 0.f;
                for (int x = 0; x < D; ++x)
                    dot = __builtin_fmaf(qs[hh][x], ld(kb, off + x), dot);
                sc = dot;
            }
            const float mx = wave_max_f32(sc);
            const float m_old = m_s[hh];
            const float m_new = fmaxf(m_old, mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float p = __builtin_amdgcn_exp2f(sc - m_use);
            float sum = p;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1)
                sum += __shfl_xor(sum, o, kWave);
            ps[hh][lane] = p;
            if (lane == 0) {
                const float al = __builtin_amdgcn_exp2f(m_old - m_use);
                alpha_s[hh] = al;
                l_s[hh] = l_s[hh] * al + sum;
                m_s[hh] = m_new;
            }
        }
        __syncthreads();
        // PV for this tile
        const int nk = min(64, kend - k0);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int hh = t / D + k * hstep;
            if (hh < G)
                acc[k] *= alpha_s[hh];
        }
        for (int jj = 0; jj < nk; ++jj) {
            const int jv = k0 + jj;
            const int64_t o2 = kv_offset(a, s, g, P, jv);
            if (o2 < 0)
                continue;
            if (jv >= P) {
                const int u = jv - P;
                const uint64_t wsel = u < 64 ? w0 : u < 128 ? w1 : u < 192 ? w2 : w3;
                if (!((wsel >> (u & 63)) & 1ull))
                    continue;
            }
            const float vv = ld(jv < P ? vp : vt, o2 + e);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int hh = t / D + k * hstep;
                if (hh < G)
                    acc[k] = __builtin_fmaf(ps[hh][jj], vv, acc[k]);
            }
        }
        __syncthreads();
    }
    T *out = reinterpret_cast<T *>(a.out);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int hh = t / D + k * hstep;
        if (hh >= G)
            continue;
        const int64_t row = ((int64_t)s * a.B + v) * a.Hq + g * G + hh;
        st(out, row * D + e, acc[k] / l_s[hh]);
        if (a.lse && e == 0)
            a.lse[row] = (m_s[hh] + __log2f(l_s[hh])) * kLn2;
    }
}

// ------------------------------------------------------------------ MFMA kernel --

struct MfmaPlan {
    int nqb;        // 16-row blocks per wave (1 or 2)
    int bm;         // rows per workgroup = 4 waves * 16 * nqb
    int n_qtiles;   // row tiles per (s, g)
    int n_splits;   // key splits
    int chunk;      // keys per split (multiple of 64)
};

static MfmaPlan mfma_plan(int S, int B, int Hq, int Hkv, int max_prefix)
{
    MfmaPlan p;
    const int G = Hq / Hkv;
    const int rows = G * B;
    p.nqb = rows >= 128 ? 2 : 1;
    p.bm = 64 * p.nqb;
    p.n_qtiles = (rows + p.bm - 1) / p.bm;
    const long base = (long)S * Hkv * p.n_qtiles;
    const int total = max_prefix + B;
    int want = base >= 512 ? 1 : (int)((512 + base - 1) / base);
    int maxs = (total + 63) / 64;
    if (want > maxs)
        want = maxs;
    if (want < 1)
        want = 1;
    int chunk = (total + want - 1) / want;
    chunk = (chunk + 63) / 64 * 64;
    p.chunk = chunk;
    p.n_splits = (total + chunk - 1) / chunk;
    return p;
}

template <int D, int NQB>
__global__ void __launch_bounds__(256, 2)
attn_mfma_kernel(AttnArgs a, int n_qtiles, int chunk, int n_splits, float *__restrict__ ws_o,
                 float *__restrict__ ws_lse)
{
    constexpr int BN = 64;
    constexpr int KP = D + 8;    // K row pitch (elements): 16-byte rows shift 4 banks
    constexpr int VP = BN + 4;   // V^T row pitch (elements)
    constexpr int SEGS = D / 8;  // 16-byte segments per key row
    constexpr int KPP = 256 / SEGS;
    constexpr int PASSES = BN / KPP;
    constexpr int KK = D / 32;   // MFMA k-steps over the head dim
    constexpr int DB = D / 16;   // 16-wide output blocks over the head dim
    __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KP];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int qt = blockIdx.x % n_qtiles;
    const int split = blockIdx.x / n_qtiles;
    const int s = blockIdx.y / a.Hkv, g = blockIdx.y % a.Hkv;
    const int G = a.G, B = a.B;
    const int rows = G * B;
    const int r0 = qt * (64 * NQB);

    if (a.err && qt == 0 && split == 0 && g == 0)
        attn_validate(a, s);
    const int P = clamp_prefix(a, s);
    const int v_hi = min(B - 1, (r0 + 64 * NQB - 1) / G);
    const int kend_all = P + v_hi + 1;
    const int kbeg = split * chunk;
    const int kend = min(kend_all, kbeg + chunk);

    const uint16_t *qp = reinterpret_cast<const uint16_t *>(a.q);
    const uint16_t *kpre = reinterpret_cast<const uint16_t *>(a.k_prefix);
    const uint16_t *vpre = reinterpret_cast<const uint16_t *>(a.v_prefix);
    const uint16_t *ktr = reinterpret_cast<const uint16_t *>(a.k_tree);
    const uint16_t *vtr = reinterpret_cast<const uint16_t *>(a.v_tree);

    // ---- rows owned by this lane (one query column of each 16-row block)
    const int grp = lane >> 4;   // lane group: k-slots 8*grp.., C rows 4*grp..
    const int col = lane & 15;
    int row_g[NQB];
    bool row_ok[NQB];
    bf16x8_t qf[NQB][KK];
    uint64_t anc_w[NQB][4];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int r = r0 + wid * 16 * NQB + qb * 16 + col;
        row_ok[qb] = r < rows;
        const int v = row_ok[qb] ? r / G : 0;
        const int h = g * G + (row_ok[qb] ? r % G : 0);
        row_g[qb] = (s * B + v) * a.Hq + h;
        const uint16_t *qrow = qp + (int64_t)row_g[qb] * D;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (row_ok[qb])
                u = *reinterpret_cast<const uint4 *>(qrow + kk * 32 + grp * 8);
            qf[qb][kk] = __builtin_bit_cast(bf16x8_t, u);
        }
        const uint64_t *ar = a.anc + ((int64_t)s * B + v) * 4;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            anc_w[qb][w] = row_ok[qb] ? ar[w] : 0ull;
    }

    float m_i[NQB], l_i[NQB];
    f32x4_t o_acc[NQB][DB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        m_i[qb] = -INFINITY;
        l_i[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
            o_acc[qb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const float c = a.scale * kLog2eA;

    const int seg = tid % SEGS;
    const int kl0 = tid / SEGS;
    // K/V rows of one tile: registers first, so the next tile's loads overlap this
    // tile's MFMA work.
    uint4 kr[PASSES], vr[PASSES];
    auto fetch = [&](int kt0) {
#pragma unroll
        for (int i = 0; i < PASSES; ++i) {
            const int j = kt0 + kl0 + i * KPP;
            kr[i] = make_uint4(0, 0, 0, 0);
            vr[i] = make_uint4(0, 0, 0, 0);
            if (j < kend) {
                const int64_t off = kv_offset(a, s, g, P, j);
                if (off >= 0) {
                    const uint16_t *kb = j < P ? kpre : ktr;
                    const uint16_t *vb = j < P ? vpre : vtr;
                    kr[i] = *reinterpret_cast<const uint4 *>(kb + off + seg * 8);
                    vr[i] = *reinterpret_cast<const uint4 *>(vb + off + seg * 8);
                }
            }
        }
    };
    if (kbeg < kend)
        fetch(kbeg);
    for (int k0 = kbeg; k0 < kend; k0 += BN) {
        __syncthreads();  // previous tile fully consumed
#pragma unroll
        for (int i = 0; i < PASSES; ++i) {
            const int kl = kl0 + i * KPP;
            *reinterpret_cast<uint4 *>(&Ks[kl * KP + seg * 8]) = kr[i];
            const uint32_t w[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Vt[(seg * 8 + 2 * e) * VP + kl] = (uint16_t)(w[e] & 0xffffu);
                Vt[(seg * 8 + 2 * e + 1) * VP + kl] = (uint16_t)(w[e] >> 16);
            }
        }
        __syncthreads();
        if (k0 + BN < kend)
            fetch(k0 + BN);

        // ---- S^T = K . Q^T  (4 key blocks of 16)
        f32x4_t sacc[4][NQB];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
                sacc[kb][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const uint4 ku = *reinterpret_cast<const uint4 *>(&Ks[(kb * 16 + col) * KP + kk * 32 + grp * 8]);
                const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, ku);
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb)
                    sacc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][kk], sacc[kb][qb], 0, 0, 0);
            }
        }

        // ---- mask (tiles that reach the tree part or the end of the range)
        const bool need_mask = (k0 + BN > P) || (k0 + BN > kend);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            if (need_mask) {
                // branch-free: visible = inside the range and (prefix key or ancestor bit)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int key = k0 + kb * 16 + grp * 4 + jj;
                        const uint32_t uu = (uint32_t)min(max(key - P, 0), 255);
                        const uint64_t lo = (uu & 64u) ? anc_w[qb][1] : anc_w[qb][0];
                        const uint64_t hi = (uu & 64u) ? anc_w[qb][3] : anc_w[qb][2];
                        const uint64_t wsel = (uu & 128u) ? hi : lo;
                        const uint32_t tb = (uint32_t)(wsel >> (uu & 63u)) & 1u;
                        const uint32_t vis = (uint32_t)(key < kend) & ((uint32_t)(key < P) | tb);
                        sacc[kb][qb][jj] = vis ? sacc[kb][qb][jj] : -INFINITY;
                    }
                }
            }
            // ---- online softmax (exp2 domain), one query column per lane
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    mx = fmaxf(mx, sacc[kb][qb][jj]);
            mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
            mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
            const float m_new = fmaxf(m_i[qb], mx * c);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_i[qb] - m_use);
            m_i[qb] = m_new;
            float psum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][qb][jj], c, -m_use));
                    sacc[kb][qb][jj] = p;
                    psum += p;
                }
            l_i[qb] = l_i[qb] * alpha + psum;
#pragma unroll
            for (int db = 0; db < DB; ++db)
                o_acc[qb][db] *= alpha;
        }

        // ---- P^T fragments: k-slot 8*grp+i <-> key 32*ks + 16*(i/4) + 4*grp + i%4
        bf16x8_t pf[NQB][2];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8_t t8;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    t8[i] = (__bf16)sacc[2 * ks][qb][i];
                    t8[4 + i] = (__bf16)sacc[2 * ks + 1][qb][i];
                }
                pf[qb][ks] = t8;
            }

        // ---- O^T += V^T . P^T
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const uint16_t *vrow = &Vt[(db * 16 + col) * VP];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const uint2 lo = *reinterpret_cast<const uint2 *>(vrow + ks * 32 + grp * 4);
                const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + ks * 32 + 16 + grp * 4);
                const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb)
                    o_acc[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qb][ks], o_acc[qb][db], 0, 0, 0);
            }
        }
    }

    // ---- epilogue
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        float l = l_i[qb];
        l += __shfl_xor(l, 16, kWave);
        l += __shfl_xor(l, 32, kWave);
        if (!row_ok[qb])
            continue;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const float lse2 = l > 0.f ? m_i[qb] + __log2f(l) : -INFINITY;
        if (n_splits == 1) {
            uint16_t *out = reinterpret_cast<uint16_t *>(a.out) + (int64_t)row_g[qb] * D;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const f32x4_t o = o_acc[qb][db] * inv;
                uint2 pk;
                pk.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
                pk.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
                *reinterpret_cast<uint2 *>(out + db * 16 + grp * 4) = pk;
            }
            if (a.lse && grp == 0)
                a.lse[row_g[qb]] = lse2 * kLn2;
        } else {
            const int64_t nrow = (int64_t)a.S * B * a.Hq;
            float *wo = ws_o + ((int64_t)split * nrow + row_g[qb]) * D;
            if (kbeg < kend) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    *reinterpret_cast<f32x4_t *>(wo + db * 16 + grp * 4) = o_acc[qb][db] * inv;
            }
            if (grp == 0)
                ws_lse[(int64_t)split * nrow + row_g[qb]] = kbeg < kend ? lse2 : -INFINITY;
        }
    }
}

// rows x (D/4) threads: merge the split partials of each row.
template <int D>
__global__ void __launch_bounds__(256)
attn_combine_kernel(int64_t nrow, int n_splits, const float *__restrict__ ws_o,
                    const float *__restrict__ ws_lse, uint16_t *__restrict__ out,
                    float *__restrict__ lse_out)
{
    constexpr int TPR = D / 4;
    const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
    const int q4 = threadIdx.x % TPR;
    if (row >= nrow)
        return;
    float M = -INFINITY;
    for (int i = 0; i < n_splits; ++i)
        M = fmaxf(M, ws_lse[(int64_t)i * nrow + row]);
    float wsum = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < n_splits; ++i) {
        const float li = ws_lse[(int64_t)i * nrow + row];
        if (li == -INFINITY)
            continue;
        const float w = __builtin_amdgcn_exp2f(li - M);
        wsum += w;
        acc += w * *reinterpret_cast<const f32x4_t *>(ws_o + ((int64_t)i * nrow + row) * D + q4 * 4);
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    acc *= inv;
    uint2 pk;
    pk.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
    pk.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
    *reinterpret_cast<uint2 *>(out + row * D + q4 * 4) = pk;
    if (lse_out && q4 == 0)
        lse_out[row] = wsum > 0.f ? (M + __log2f(wsum)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------ host side --

size_t attention_workspace(int S, int B, int Hq, int Hkv, int d, int max_prefix, int dtype)
{
    if (dtype != JT_BF16)
        return 0;
    const MfmaPlan p = mfma_plan(S, B, Hq, Hkv, max_prefix);
    if (p.n_splits <= 1)
        return 0;
    const size_t nrow = (size_t)S * B * Hq;
    return (size_t)p.n_splits * nrow * ((size_t)d + 1) * sizeof(float) + 256;
}

template <int D>
static jt_status launch_mfma(const AttnArgs &a, void *ws, hipStream_t st)
{
    const MfmaPlan p = mfma_plan(a.S, a.B, a.Hq, a.Hkv, a.max_prefix);
    const int64_t nrow = (int64_t)a.S * a.B * a.Hq;
    float *wo = reinterpret_cast<float *>(ws);
    float *wl = wo ? wo + (size_t)p.n_splits * nrow * D : nullptr;
    const dim3 grid((unsigned)(p.n_qtiles * p.n_splits), (unsigned)(a.S * a.Hkv));
    if (p.nqb == 2)
        hipLaunchKernelGGL((attn_mfma_kernel<D, 2>), grid, dim3(256), 0, st, a, p.n_qtiles, p.chunk,
                           p.n_splits, wo, wl);
    else
        hipLaunchKernelGGL((attn_mfma_kernel<D, 1>), grid, dim3(256), 0, st, a, p.n_qtiles, p.chunk,
                           p.n_splits, wo, wl);
    jt_status e = launch_status(hipGetLastError());
    if (e != JT_OK || p.n_splits == 1)
        return e;
    constexpr int rows_per_wg = 256 / (D / 4);
    hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((unsigned)((nrow + rows_per_wg - 1) / rows_per_wg)),
                       dim3(256), 0, st, nrow, p.n_splits, wo, wl,
                       reinterpret_cast<uint16_t *>(a.out), a.lse);
    return launch_status(hipGetLastError());
}

jt_status launch_attention(const AttnArgs &a, void *ws, hipStream_t st)
{
    if (a.S == 0)
        return JT_OK;
    if (a.dtype == JT_BF16)
        return a.d == 128 ? launch_mfma<128>(a, ws, st) : launch_mfma<64>(a, ws, st);
    hipLaunchKernelGGL((attn_simple_kernel<float>), dim3(a.B, a.S * a.Hkv), dim3(256), 0, st, a);
    return launch_status(hipGetLastError());
}

} // namespace jt
