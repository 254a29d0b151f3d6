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
// tree keys P..P+B-1.  Ancestors of v have indices <= v, so rows whose deepest node is
// v_hi never need keys past P + v_hi (causal trim of the tree part).
//
// bf16 -> attn_bf16_kernel (MFMA).  The G query heads of a KV group times the B nodes
// form the rows of one dense problem (row r = node r / G, head r % G), so one K/V tile
// in LDS serves every row of the workgroup.  A wave owns 64 rows (two 32-row blocks)
// and runs, per 64-key tile,
//   S^T = K . Q^T     v_mfma_f32_32x32x16_bf16; K rows from LDS (one 16-byte read per
//                     lane), Q^T fragments held in registers for the whole kernel;
//   online softmax    exp2 domain; a lane holds one row and 32 of the tile's keys, the
//                     other 32 sit in lane ^ 32;
//   O^T += V^T . P^T  P^T is the S^T accumulator converted to bf16 in place (the key
//                     order of the accumulator layout is applied to the V reads), V^T
//                     fragments come from row-major V in LDS through ds_read_b64_tr_b16.
// K/V tiles are copied HBM -> LDS by global_load_lds_dwordx4 (no register staging)
// into rows whose 16-byte segments are XOR-swizzled, which keeps both the K reads (16
// rows x 16 bytes) and the transposing V reads (4 rows x 32 bytes) free of bank
// conflicts.  A workgroup (4 waves) is NWR row blocks of 64 x NWK key columns:
//   NWR = 4: 256 rows share one double-buffered tile stream;
//   NWR = 1, 2: the waves of a column walk their own tiles and merge in LDS at the end.
// Work that still leaves the chip idle is split over keys (split-KV): each chunk writes
// an unnormalised fp32 partial (O, running max, running sum) and attn_combine_kernel
// merges them.
//
// fp32 -> attn_simple_kernel: one workgroup per (s, v, g) on the vector ALU.
#include <type_traits>

#include "jt_internal.h"

namespace jt {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr float kLog2eA = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f;  // lazy softmax rescale threshold (log2 units)

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

constexpr int kBtCap = 1024;  // block-table entries of one chunk staged in LDS

// Work decomposition shared by the host launcher and the kernels.
struct AttnPlan {
    int nwr;       // 32-row waves per key column (2, 4 or 8); key columns = 8 / nwr
    int rt;        // rows per workgroup = 32 * nwr
    int n_rtiles;  // row tiles per (s, g)
    int units;     // S * Hkv * n_rtiles
    int ch;        // keys per chunk (multiple of 64 * key columns)
    int n_chunks;  // chunks per unit (1 = no split-KV)
    int remap;     // 1: place consecutive work items on one XCD
    int fused;     // split-KV partials merged in-kernel by the unit's last workgroup
};

// Split-KV workspace: per-unit arrival counters, then (m, l) per partial row, then the
// partial rows themselves (normalised, bf16).
struct AttnWs {
    int *cnt;
    float2 *ml;
    uint16_t *o;
};
constexpr size_t kCntBytes = 256;  // granularity of the counter block

static AttnPlan attn_plan(int S, int B, int Hq, int Hkv, int max_prefix, int block_size)
{
    AttnPlan p;
    const int rows = (Hq / Hkv) * B;
    p.nwr = rows <= 64 ? 2 : (rows <= 128 ? 4 : 8);
    p.rt = 32 * p.nwr;
    p.n_rtiles = (rows + p.rt - 1) / p.rt;
    p.units = S * Hkv * p.n_rtiles;
    const int kcol = 8 / p.nwr;
    const int gran = 64 * kcol;
    const int keys = max_prefix + B;
    const int maxc = (keys + gran - 1) / gran;
    int want = (256 + p.units - 1) / p.units;
    if (want > maxc)
        want = maxc;
    if (want < 1)
        want = 1;
    int ch = (keys + want - 1) / want;
    ch = (ch + gran - 1) / gran * gran;
    // a paged chunk's block-table entries must fit the LDS staging area
    if (block_size > 0) {
        const long cap = (long)(kBtCap - 1) * block_size / gran * gran;
        if (ch > cap)
            ch = (int)(cap > gran ? cap : gran);
    }
    p.ch = ch;
    p.n_chunks = (keys + ch - 1) / ch;
    const long grid = (long)p.units * p.n_chunks;
    p.remap = (grid % 8 == 0) ? 1 : 0;
    // A last-arriving-workgroup merge needs device-scope fences, which write back the whole
    // L2 and cost more than a second launch here: the merge is always a separate pass.
    p.fused = 0;
    return p;
}

static size_t attn_ws_bytes(const AttnPlan &p, int d)
{
    if (p.n_chunks <= 1)
        return 0;
    const size_t slots = (size_t)p.units * p.n_chunks * p.rt;
    const size_t cnt = ((size_t)p.units * sizeof(int) + kCntBytes - 1) / kCntBytes * kCntBytes;
    return cnt + slots * sizeof(float2) + slots * (size_t)d * 2;
}

static AttnWs attn_ws_split(const AttnPlan &p, void *ws)
{
    AttnWs w{nullptr, nullptr, nullptr};
    if (p.n_chunks <= 1 || !ws)
        return w;
    const size_t slots = (size_t)p.units * p.n_chunks * p.rt;
    const size_t cnt = ((size_t)p.units * sizeof(int) + kCntBytes - 1) / kCntBytes * kCntBytes;
    uint8_t *b = reinterpret_cast<uint8_t *>(ws);
    w.cnt = reinterpret_cast<int *>(b);
    w.ml = reinterpret_cast<float2 *>(b + cnt);
    w.o = reinterpret_cast<uint16_t *>(b + cnt + slots * sizeof(float2));
    return w;
}

// 16-byte segment swizzle of an LDS K/V row with SEGS segments.  Eight consecutive rows
// get distinct values in the low three bits (a 16-byte read of one segment from rows
// r..r+7 touches eight different 16-byte bank groups), and the four rows of a
// transposing V read (rows 4a..4a+3, segment pair {2c, 2c+1}) map to eight distinct
// segments; bit 3 separates rows r and r+8.
template <int SEGS> __device__ __forceinline__ int seg_swz(int row)
{
    const int lo = ((row & 3) << 1) | ((row >> 2) & 1);
    if constexpr (SEGS >= 16)
        return lo | (((row >> 3) & 1) << 3);
    else
        return lo;
}

__device__ __forceinline__ void lds_dma16(const void *gsrc, void *ldst)
{
    __builtin_amdgcn_global_load_lds((glb_void_t *)gsrc, (lds_void_t *)ldst, 16, 0, 0);
}
// vmcnt(0) through the builtin (not inline asm), so the compiler's own wait tracking
// knows that every earlier load, DMA included, has completed.
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

typedef int i32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t lds_off(const void *p)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}

// Four 16-byte LDS reads (ds_read_b128) at four row addresses plus one immediate
// offset, then a wait for them -- the K fragments of QK^T.  Inline asm for the same
// reason as the transposing reads below.
template <int OFF>
__device__ __forceinline__ void k_read4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                        uint4 &k0, uint4 &k1, uint4 &k2, uint4 &k3)
{
    asm volatile("ds_read_b128 %0, %4 offset:%8\n\t"
                 "ds_read_b128 %1, %5 offset:%8\n\t"
                 "ds_read_b128 %2, %6 offset:%8\n\t"
                 "ds_read_b128 %3, %7 offset:%8\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(k0), "=&v"(k1), "=&v"(k2), "=&v"(k3)
                 : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "i"(OFF));
}

// Eight transposing LDS reads (ds_read_b64_tr_b16) from two row addresses at four row
// offsets, then a wait for them.  Written as inline asm because the builtin's memory
// operand carries no LDS alias information, which makes the compiler wait for every
// pending HBM->LDS copy (including the next tile's) before the read.
template <int O0, int O1, int O2, int O3>
__device__ __forceinline__ void tr16_x8(uint32_t aa, uint32_t ab, i32x2_t (&r)[8])
{
    asm volatile("ds_read_b64_tr_b16 %0, %8 offset:%10\n\t"
                 "ds_read_b64_tr_b16 %1, %9 offset:%10\n\t"
                 "ds_read_b64_tr_b16 %2, %8 offset:%11\n\t"
                 "ds_read_b64_tr_b16 %3, %9 offset:%11\n\t"
                 "ds_read_b64_tr_b16 %4, %8 offset:%12\n\t"
                 "ds_read_b64_tr_b16 %5, %9 offset:%12\n\t"
                 "ds_read_b64_tr_b16 %6, %8 offset:%13\n\t"
                 "ds_read_b64_tr_b16 %7, %9 offset:%13\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
                   "=&v"(r[6]), "=&v"(r[7])
                 : "v"(aa), "v"(ab), "i"(O0), "i"(O1), "i"(O2), "i"(O3));
}

// Merge of one unit's split-KV partials for output items it .. (row, 8 columns), step
// `stride`.  Partial c of a row holds m_c (log2 domain), l_c and O_c / l_c in bf16; the
// merged row is sum_c 2^(m_c - M) l_c (O_c/l_c) / sum_c 2^(m_c - M) l_c, M = max_c m_c.
template <int D>
__device__ void attn_merge_unit(const AttnArgs &a, const AttnPlan &pl, const AttnWs &w,
                                int unit, int it, int stride)
{
    constexpr int SPR = D / 8;  // 8-column segments per row
    const int rt = unit % pl.n_rtiles;
    const int sg = unit / pl.n_rtiles;
    const int s = sg / a.Hkv, g = sg % a.Hkv;
    const int G = a.G, B = a.B;
    const int P = clamp_prefix(a, s);
    const int v_hi = min(B - 1, (rt * pl.rt + pl.rt - 1) / G);
    const int nact = (P + v_hi + 1 + pl.ch - 1) / pl.ch;
    for (; it < pl.rt * SPR; it += stride) {
        const int rl = it / SPR, sgm = it % SPR;
        const int r = rt * pl.rt + rl;
        if (r >= G * B)
            continue;
        const int64_t base = (int64_t)unit * pl.n_chunks * pl.rt + rl;
        float M = -INFINITY;
        for (int k = 0; k < nact; ++k)
            M = fmaxf(M, w.ml[base + (int64_t)k * pl.rt].x);
        const float Mu = M == -INFINITY ? 0.f : M;
        float l = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < nact; ++k) {
            const int64_t slot = base + (int64_t)k * pl.rt;
            const float2 ml = w.ml[slot];
            const float wk = __builtin_amdgcn_exp2f(ml.x - Mu) * ml.y;
            l += wk;
            const uint4 u = *reinterpret_cast<const uint4 *>(w.o + slot * D + sgm * 8);
            acc[0] += wk * bf16_lo(u.x);
            acc[1] += wk * bf16_hi(u.x);
            acc[2] += wk * bf16_lo(u.y);
            acc[3] += wk * bf16_hi(u.y);
            acc[4] += wk * bf16_lo(u.z);
            acc[5] += wk * bf16_hi(u.z);
            acc[6] += wk * bf16_lo(u.w);
            acc[7] += wk * bf16_hi(u.w);
        }
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int v = r / G, h = g * G + r % G;
        const int64_t row_g = ((int64_t)s * B + v) * a.Hq + h;
        uint4 pk;
        pk.x = (uint32_t)f32_to_bf16(acc[0] * inv) | ((uint32_t)f32_to_bf16(acc[1] * inv) << 16);
        pk.y = (uint32_t)f32_to_bf16(acc[2] * inv) | ((uint32_t)f32_to_bf16(acc[3] * inv) << 16);
        pk.z = (uint32_t)f32_to_bf16(acc[4] * inv) | ((uint32_t)f32_to_bf16(acc[5] * inv) << 16);
        pk.w = (uint32_t)f32_to_bf16(acc[6] * inv) | ((uint32_t)f32_to_bf16(acc[7] * inv) << 16);
        *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(a.out) + row_g * D + sgm * 8) = pk;
        if (a.lse && sgm == 0)
            a.lse[row_g] = l > 0.f ? (M + __log2f(l)) * kLn2 : -INFINITY;
    }
}

// s_waitcnt vmcnt(N), N < 64 (expcnt and lgkmcnt left unconstrained)
template <int N> __device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that does not drain the DMA pipeline: __syncthreads() carries a
// workgroup fence, which the compiler implements with s_waitcnt vmcnt(0) and would wait
// for the copies of later tiles too.  Each wave has already waited for its share of
// the current tile (vmcnt) before this point; LDS reads are drained (lgkmcnt(0)) so a
// buffer may be refilled after the barrier.  The asm memory clobber keeps the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void barrier_keep_dma()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}


template <int D, int NWR>
__global__ void __launch_bounds__(512, 1)
attn_bf16_kernel(AttnArgs a, AttnPlan pl, AttnWs ws)
{
    constexpr int NWK = 8 / NWR;                 // key columns
    constexpr int NST = NWK == 1 ? 4 : (NWK == 2 ? 2 : 1);  // tile buffers per column
    constexpr int SEGS = D / 8;                  // 16-byte segments per K/V row
    constexpr int ROWB = D * 2;                  // bytes per K/V row
    constexpr int TILE = 64;                     // keys per tile
    constexpr int TILEB = TILE * ROWB;           // bytes of one K (or V) tile
    constexpr int RPI = 1024 / ROWB;             // rows per DMA instruction (64 lanes x 16 B)
    constexpr int NINS = TILE / RPI;             // DMA instructions per K (or V) tile
    constexpr int NIW = NINS / NWR;              // of which one wave issues
    constexpr int NOPS = 2 * NIW;                // DMA instructions per tile per wave
    constexpr int KS = D / 16;                   // MFMA k-steps over the head dim
    constexpr int DB = D / 32;                   // 32-wide output blocks over the head dim
    constexpr int NREG = DB * 16 + 2;            // merge record per lane: O, m, l
    constexpr int BUFB = NWK * 2 * TILEB;        // one stage: K and V tile of every column
    constexpr int RECB = NREG * 64 * 4;          // bytes of one merge record
    constexpr int CAP0 = BUFB / RECB;            // merge records per stage buffer
    static_assert(NIW >= 1 && NINS % NWR == 0, "DMA split");
    static_assert((NWK - 1) * NWR <= CAP0 * NST, "LDS too small for the merge");
    static_assert(NOPS * (NST - 2 > 0 ? NST - 2 : 0) < 64, "vmcnt range");
    // One array per stage: distinct objects let the compiler see that a DMA into one
    // stage does not alias the reads of another, so it does not wait for it.
    __shared__ __attribute__((aligned(16))) uint8_t L0[BUFB];
    __shared__ __attribute__((aligned(16))) uint8_t L1[NST > 1 ? BUFB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t L2[NST > 2 ? BUFB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t L3[NST > 3 ? BUFB : 16];
    __shared__ int bt_lds[kBtCap];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wr = wid % NWR, wc = wid / NWR;
    const int col = lane & 31, hh = lane >> 5;

    // ---- work item
    int item = blockIdx.x;
    if (pl.remap) {
        const int per = gridDim.x >> 3;
        item = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    }
    const int rt = item % pl.n_rtiles;
    const int chunk = (item / pl.n_rtiles) % pl.n_chunks;
    const int sg = item / (pl.n_rtiles * pl.n_chunks);
    const int s = sg / a.Hkv, g = sg % a.Hkv;
    const int unit = sg * pl.n_rtiles + rt;
    const int G = a.G, B = a.B, R = G * B;
    const int r0 = rt * pl.rt;

    if (a.err && rt == 0 && chunk == 0 && g == 0)
        attn_validate(a, s);
    const int P = clamp_prefix(a, s);
    const int v_hi = min(B - 1, (r0 + pl.rt - 1) / G);
    const int kend_u = P + v_hi + 1;
    const int kbeg = chunk * pl.ch;
    const int kend = min(kend_u, kbeg + pl.ch);
    if (kbeg >= kend)
        return;  // nothing to do: the combine pass skips this chunk
    const int ntiles = (kend - kbeg + TILE - 1) / TILE;
    const int nsteps = (ntiles + NWK - 1) / NWK;

    const uintptr_t kpre_a = reinterpret_cast<uintptr_t>(a.k_prefix);
    const uintptr_t vpre_a = reinterpret_cast<uintptr_t>(a.v_prefix);
    const uintptr_t ktr_a = reinterpret_cast<uintptr_t>(a.k_tree);
    const uintptr_t vtr_a = reinterpret_cast<uintptr_t>(a.v_tree);
    const int Hkv = a.Hkv;
    const int64_t pre_s = (int64_t)s * a.max_prefix;  // contiguous prefix: first row of s
    const bool paged = a.block_table != nullptr;
    const int bshift = a.block_shift, bsize = a.block_size, nblocks = a.num_blocks;

    // ---- paged prefix: the chunk's block-table entries, staged once in LDS
    const int pend = min(kend, P);                   // prefix keys of this chunk end here
    const int bt0 = kbeg >> bshift;                  // first block of the chunk
    if (paged) {
        const int nb = kbeg < pend ? ((pend - 1) >> bshift) - bt0 + 1 : 0;
        const int32_t *btab = a.block_table + (int64_t)s * a.max_blocks;
        for (int i = tid; i < nb; i += 512)
            bt_lds[i] = (bt0 + i < a.max_blocks) ? btab[bt0 + i] : -1;
        __syncthreads();
    }

    // ---- rows of this wave: one 32-row block, lane holds row `col`; its Q^T fragments
    // and its ancestor row stay in registers
    const int wrow0 = r0 + wr * 32;
    const bool wave_has_rows = wrow0 < R;
    const int rr = wrow0 + col;
    const bool row_ok = rr < R;
    const int vrow = row_ok ? rr / G : 0;
    const int row_g = (s * B + vrow) * a.Hq + g * G + (row_ok ? rr % G : 0);
    bf16x8_t qf[KS];
    {
        const uint16_t *qrow = reinterpret_cast<const uint16_t *>(a.q) + (int64_t)row_g * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (row_ok)
                u = *reinterpret_cast<const uint4 *>(qrow + ks * 16 + hh * 8);
            qf[ks] = __builtin_bit_cast(bf16x8_t, u);
        }
    }
    uint64_t anc0, anc1, anc2, anc3;
    {
        const uint64_t *ar = a.anc + ((int64_t)s * B + vrow) * 4;
        anc0 = ar[0];
        anc1 = ar[1];
        anc2 = ar[2];
        anc3 = ar[3];
    }

    // ---- DMA of one tile (keys kt..kt+63) into `base` (K) and base + TILEB (V).  The
    // NWR waves of a column share the NINS row groups; a lane copies one 16-byte segment.
    // Keys past the range are clamped to the range's last key and absent keys (a bad
    // block) read the sequence's first tree row: a finite value whose score the mask
    // removes, or whose sequence is flagged.  Exactly NOPS loads per wave.
    auto issue_tile = [=](int kt, uint8_t *base) {
        const int rrow = lane / SEGS, pslot = lane % SEGS;
#pragma unroll
        for (int ii = 0; ii < NIW; ++ii) {
            const int i = ii * NWR + wr;
            const int row = i * RPI + rrow;
            const int key = min(kt + row, kend - 1);
            int64_t off;  // element offset of the key's K/V row, -1 if absent
            bool pre = key < P;
            if (pre) {
                if (paged) {
                    const int blk = bt_lds[(key >> bshift) - bt0];
                    off = (blk >= 0 && blk < nblocks)
                              ? (((int64_t)blk * bsize + (key & (bsize - 1))) * Hkv + g) * D
                              : -1;
                } else {
                    off = ((pre_s + key) * Hkv + g) * D;
                }
            } else {
                off = (((int64_t)s * B + (key - P)) * Hkv + g) * D;
            }
            if (off < 0) {
                pre = false;
                off = ((int64_t)s * B * Hkv + g) * D;
            }
            const int seg = pslot ^ seg_swz<SEGS>(row);
            const uintptr_t boff = (uintptr_t)(off * 2 + seg * 16);
            lds_dma16(reinterpret_cast<const void *>((pre ? kpre_a : ktr_a) + boff), base + i * 1024);
            lds_dma16(reinterpret_cast<const void *>((pre ? vpre_a : vtr_a) + boff),
                      base + TILEB + i * 1024);
        }
    };

    float m_i = -INFINITY, l_i = 0.f;
    f32x16_t o_acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j)
            o_acc[db][j] = 0.f;
    const float c = a.scale * kLog2eA;
    const int b2 = (lane >> 4) & 1, j16 = lane & 15;

    // ---- visibility window of a tile: bit i <=> key kt + i is visible to this lane's row
    auto vis_window = [=](int kt) -> uint64_t {
        const int nin = kend - kt;
        const uint64_t inr = nin >= 64 ? ~0ull : (nin <= 0 ? 0ull : ((1ull << nin) - 1ull));
        const int u0 = kt - P;  // tree index of the tile's first key (wave-uniform)
        if (u0 + 64 <= 0)
            return inr;
        const int ua = u0 < 0 ? 0 : u0;
        const int wa = __builtin_amdgcn_readfirstlane(ua >> 6), sh = ua & 63;
        if (wa >= 4)
            return 0ull;
        // uniform branches (no indexed register array, which would live in scratch)
        uint64_t w0, w1;
        if (wa == 0) {
            w0 = anc0;
            w1 = anc1;
        } else if (wa == 1) {
            w0 = anc1;
            w1 = anc2;
        } else if (wa == 2) {
            w0 = anc2;
            w1 = anc3;
        } else {
            w0 = anc3;
            w1 = 0ull;
        }
        const uint64_t t = sh ? ((w0 >> sh) | (w1 << (64 - sh))) : w0;
        const uint64_t win = u0 < 0 ? ((t << (-u0)) | ((1ull << (-u0)) - 1ull)) : t;
        return win & inr;
    };

    // ---- one 64-key tile of this wave, in two parts: (1) QK^T, mask and online softmax,
    // leaving the tile's P^T fragments in pf; (2) PV from pf.
    auto qk_softmax = [&](const uint8_t *kb, uint64_t vis, bf16x8_t (&pf)[2][2]) {
        // S^T = K . Q^T for 2 key blocks of 32.  K row kbk*32 + col, segment 2*ks + hh;
        // the 32-row step keeps the swizzle, so it is an immediate offset.
        f32x16_t sacc[2];
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                sacc[kbk][j] = 0.f;
        const uint32_t kbase = lds_off(kb) + col * ROWB;
        const int zs = seg_swz<SEGS>(col);
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk) {
#pragma unroll
            for (int k4 = 0; k4 < KS; k4 += 4) {
                uint4 kf[4];
                const uint32_t a0 = kbase + (((2 * (k4 + 0) + hh) ^ zs) * 16);
                const uint32_t a1 = kbase + (((2 * (k4 + 1) + hh) ^ zs) * 16);
                const uint32_t a2 = kbase + (((2 * (k4 + 2) + hh) ^ zs) * 16);
                const uint32_t a3 = kbase + (((2 * (k4 + 3) + hh) ^ zs) * 16);
                if (kbk == 0)
                    k_read4<0>(a0, a1, a2, a3, kf[0], kf[1], kf[2], kf[3]);
                else
                    k_read4<32 * ROWB>(a0, a1, a2, a3, kf[0], kf[1], kf[2], kf[3]);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    sacc[kbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8_t, kf[q]), qf[k4 + q], sacc[kbk], 0, 0, 0);
            }
        }
        if (vis != ~0ull) {
#pragma unroll
            for (int kbk = 0; kbk < 2; ++kbk) {
                const uint32_t half = (uint32_t)(vis >> (kbk * 32 + 4 * hh));
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint32_t bit = (half >> (8 * (j >> 2) + (j & 3))) & 1u;
                    sacc[kbk][j] = bit ? sacc[kbk][j] : -INFINITY;
                }
            }
        }
        // Online softmax with a lazily moved reference: the row's reference m_i only moves
        // when the tile maximum exceeds it by more than kRescale (log2 units), so the
        // rescale of O (64 multiplies) is rare.  Probabilities are then at most 2^kRescale,
        // which fp32 and bf16 hold exactly in range; numerator and denominator share m_i.
        float mx = -INFINITY;
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                mx = fmaxf(mx, sacc[kbk][j]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * c;
        const bool move = mx > m_i + kRescale;
        if (__ballot(move)) {
            const float m_new = move ? mx : m_i;
            const float alpha = m_i == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_i - m_new);
            m_i = m_new;
            l_i *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
                o_acc[db] *= alpha;
        }
        const float m_use = m_i == -INFINITY ? 0.f : m_i;
        float psum = 0.f;
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2) {
                // P^T fragment m2 of key block kbk: accumulator entries 8*m2 .. 8*m2+7,
                // i.e. keys 16*m2 + 8*(i/4) + 4*hh + i%4
                bf16x8_t t8;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float p = __builtin_amdgcn_exp2f(
                        __builtin_fmaf(sacc[kbk][8 * m2 + i], c, -m_use));
                    psum += p;
                    t8[i] = (__bf16)p;
                }
                pf[kbk][m2] = t8;
            }
        l_i += psum;
    };
    auto pv = [&](const uint8_t *vb, const bf16x8_t (&pf)[2][2]) {
        // O^T += V^T . P^T; V^T fragments by transposing reads of row-major V.  The key
        // rows of fragment (kbk, m2) are kbk*32 + 16*m2 + 4*hh + j16/4 (+8 for the upper
        // half); the 16- and 32-row steps leave the swizzle unchanged, so they are
        // immediate offsets.
        const int rowa = 4 * hh + (j16 >> 2), rowb = rowa + 8;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int cc = db * 32 + 16 * b2 + 4 * (j16 & 3);
            const int half = (cc & 4) * 2;
            const uint32_t aa = lds_off(vb + rowa * ROWB + (((cc >> 3) ^ seg_swz<SEGS>(rowa)) * 16) + half);
            const uint32_t ab = lds_off(vb + rowb * ROWB + (((cc >> 3) ^ seg_swz<SEGS>(rowb)) * 16) + half);
            i32x2_t r[8];
            tr16_x8<0, 16 * ROWB, 32 * ROWB, 48 * ROWB>(aa, ab, r);
#pragma unroll
            for (int f = 0; f < 4; ++f) {  // f = 2*kbk + m2
                const bf16x8_t vf = __builtin_bit_cast(
                    bf16x8_t, __builtin_shufflevector(r[2 * f], r[2 * f + 1], 0, 1, 2, 3));
                o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[f >> 1][f & 1], o_acc[db], 0, 0, 0);
            }
        }
    };
    auto compute_tile = [&](const uint8_t *kb, const uint8_t *vb, uint64_t vis) {
        bf16x8_t pf[2][2];
        qk_softmax(kb, vis, pf);
        pv(vb, pf);
    };

    auto stage = [&](auto kst) -> uint8_t * {
        constexpr int k = decltype(kst)::value;
        uint8_t *b = k == 0 ? L0 : (k == 1 ? L1 : (k == 2 ? L2 : L3));
        return b + wc * 2 * TILEB;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;

    if constexpr (NWK == 1) {
        // ---- one key column, 8 waves, 4 stages, ping-pong.  Waves 0-3 (group A) and
        // 4-7 (group B) share the SIMDs pairwise; B runs half a tile behind A, so on a SIMD
        // one wave's softmax (VALU) runs under the other's MFMAs.  Barrier j is where A
        // starts tile j and where B has finished the softmax of tile j - 1 (its PV of
        // j - 1 follows); after it, every wave issues its share of the DMA of tile j + 2
        // into the stage of tile j - 2, which both groups have finished.  Before barrier j
        // each wave waits for its own share of tile j's DMA; only DMAs are in flight, so
        // that wait is vmcnt(NOPS) while the DMA of tile j + 1 may still run.
        const int grp = wid >> 2;
        bf16x8_t pf[2][2];
        if (0 < ntiles)
            issue_tile(kbeg, stage(I0{}));
        if (1 < ntiles)
            issue_tile(kbeg + TILE, stage(I1{}));
        auto wait_own = [&](bool newer_in_flight) {
            if (newer_in_flight)
                wait_vm<NOPS>();
            else
                wait_vm<0>();
        };
        if (grp == 1)
            wait_own(1 < ntiles);
        auto body = [&](int j, auto kst) {
            constexpr int k = decltype(kst)::value;
            const int kt = kbeg + j * TILE;
            if (grp == 0)
                wait_own(j + 1 < ntiles);
            barrier_keep_dma();
            if (j + 2 < ntiles)
                issue_tile(kt + 2 * TILE, stage(std::integral_constant<int, (k + 2) % 4>{}));
            if (grp == 0) {
                if (wave_has_rows) {
                    qk_softmax(stage(kst), vis_window(kt), pf);
                    pv(stage(kst) + TILEB, pf);
                }
            } else {
                if (wave_has_rows) {
                    if (j > 0)
                        pv(stage(std::integral_constant<int, (k + 3) % 4>{}) + TILEB, pf);
                    qk_softmax(stage(kst), vis_window(kt), pf);
                }
                wait_own(j + 2 < ntiles);
            }
        };
        for (int j = 0; j < ntiles; j += 4) {
            body(j, I0{});
            if (j + 1 < ntiles)
                body(j + 1, I1{});
            if (j + 2 < ntiles)
                body(j + 2, I2{});
            if (j + 3 < ntiles)
                body(j + 3, I3{});
        }
        if (grp == 1 && wave_has_rows) {  // B's PV of the last tile
            switch ((ntiles - 1) & 3) {
            case 0: pv(stage(I0{}) + TILEB, pf); break;
            case 1: pv(stage(I1{}) + TILEB, pf); break;
            case 2: pv(stage(I2{}) + TILEB, pf); break;
            default: pv(stage(I3{}) + TILEB, pf); break;
            }
        }
    } else {
        // ---- several key columns (few rows): column wc takes tiles wc, wc + NWK, ...;
        // two stages (NWK = 2: the next step's DMA runs under this step's work) or one.
        auto tile_of = [&](int step) { return step * NWK + wc; };
        auto body = [&](int step, auto kst) {
            constexpr int k = decltype(kst)::value;
            uint8_t *cur = stage(kst);
            const int tile = tile_of(step);
            const int kt = kbeg + tile * TILE;
            if constexpr (NST == 1) {
                if (tile < ntiles)
                    issue_tile(kt, cur);
            }
            wait_vm<0>();
            barrier_keep_dma();
            if constexpr (NST > 1) {
                const int tn = tile_of(step + 1);
                if (tn < ntiles)
                    issue_tile(kbeg + tn * TILE, stage(std::integral_constant<int, (k + 1) % NST>{}));
            }
            if (tile < ntiles && wave_has_rows)
                compute_tile(cur, cur + TILEB, vis_window(kt));
            if constexpr (NST == 1)
                barrier_keep_dma();
        };
        if constexpr (NST > 1) {
            if (tile_of(0) < ntiles)
                issue_tile(kbeg + tile_of(0) * TILE, stage(I0{}));
        }
        for (int step = 0; step < nsteps; step += NST) {
            body(step, I0{});
            if constexpr (NST > 1)
                if (step + 1 < nsteps)
                    body(step + 1, std::integral_constant<int, 1 % NST>{});
        }
    }

    // ---- merge the key columns of a row block in LDS (NWK > 1): columns 1.. publish
    // (O, m, l), column 0 folds them in.
    if constexpr (NWK > 1) {
        wait_dma();
        // merge record k lives in buffer set 0 while it fits, then in set 1
        auto rec = [&](int k) -> float * {
            return reinterpret_cast<float *>(k < CAP0 ? L0 + k * RECB : L1 + (k - CAP0) * RECB);
        };
        __syncthreads();
        if (wc > 0) {
            float *mine = rec((wc - 1) * NWR + wr);
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    mine[(db * 16 + j) * 64 + lane] = o_acc[db][j];
            mine[(DB * 16) * 64 + lane] = m_i;
            mine[(DB * 16 + 1) * 64 + lane] = l_i;
        }
        __syncthreads();
        if (wc == 0) {
            float M = m_i;
            for (int k = 1; k < NWK; ++k)
                M = fmaxf(M, rec((k - 1) * NWR + wr)[(DB * 16) * 64 + lane]);
            const float Mu = M == -INFINITY ? 0.f : M;
            const float w0 = __builtin_amdgcn_exp2f(m_i - Mu);
            float l = l_i * w0;
#pragma unroll
            for (int db = 0; db < DB; ++db)
                o_acc[db] *= w0;
            for (int k = 1; k < NWK; ++k) {
                const float *oth = rec((k - 1) * NWR + wr);
                const float wk = __builtin_amdgcn_exp2f(oth[(DB * 16) * 64 + lane] - Mu);
                l += wk * oth[(DB * 16 + 1) * 64 + lane];
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        o_acc[db][j] += wk * oth[(db * 16 + j) * 64 + lane];
            }
            m_i = M;
            l_i = l;
        }
    }
    // ---- epilogue: final output (one chunk), or a normalised bf16 partial plus (m, l)
    const float l = l_i + __shfl_xor(l_i, 32, kWave);
    if (wc == 0 && wave_has_rows && row_ok) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint16_t *dst;
        if (pl.n_chunks == 1) {
            dst = reinterpret_cast<uint16_t *>(a.out) + (int64_t)row_g * D;
            if (a.lse && hh == 0)
                a.lse[row_g] = l > 0.f ? (m_i + __log2f(l)) * kLn2 : -INFINITY;
        } else {
            const int rl = wr * 32 + col;  // row within the unit's tile
            const int64_t slot = ((int64_t)unit * pl.n_chunks + chunk) * pl.rt + rl;
            dst = ws.o + slot * D;
            if (hh == 0)
                ws.ml[slot] = make_float2(m_i, l);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int d0 = db * 32 + 8 * q + 4 * hh;
                uint2 pk;
                pk.x = (uint32_t)f32_to_bf16(o_acc[db][4 * q] * inv) |
                       ((uint32_t)f32_to_bf16(o_acc[db][4 * q + 1] * inv) << 16);
                pk.y = (uint32_t)f32_to_bf16(o_acc[db][4 * q + 2] * inv) |
                       ((uint32_t)f32_to_bf16(o_acc[db][4 * q + 3] * inv) << 16);
                *reinterpret_cast<uint2 *>(dst + d0) = pk;
            }
    }
    // ---- fused merge: the unit's last-arriving workgroup merges its partials.  Release:
    // every thread's partial stores are made visible at device scope before the arrival
    // is counted; acquire: the last workgroup fences before reading the others'.  The
    // counter goes back to zero, ready for the next call on the same workspace.
    if (pl.fused) {
        __shared__ int s_last;
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const int nact = (kend_u + pl.ch - 1) / pl.ch;
            const int old = atomicAdd(ws.cnt + unit, 1);
            s_last = old == nact - 1;
        }
        __syncthreads();
        if (s_last) {
            __threadfence();
            attn_merge_unit<D>(a, pl, ws, unit, tid, 512);
            if (tid == 0)
                ws.cnt[unit] = 0;
        }
    }
}

// Separate merge pass for large units: one thread per (unit, row, 8 output columns).
template <int D>
__global__ void __launch_bounds__(256)
attn_combine_kernel(AttnArgs a, AttnPlan pl, AttnWs ws)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per_unit = (int64_t)pl.rt * (D / 8);
    const int unit = (int)(t / per_unit);
    if (unit >= pl.units)
        return;
    attn_merge_unit<D>(a, pl, ws, unit, (int)(t % per_unit), (int)per_unit);
}

// ------------------------------------------------------------------ host side --

size_t attention_workspace(int S, int B, int Hq, int Hkv, int d, int max_prefix, int block_size,
                           int dtype)
{
    if (dtype != JT_BF16)
        return 0;
    return attn_ws_bytes(attn_plan(S, B, Hq, Hkv, max_prefix, block_size), d);
}

template <int D, int NWR>
static void launch_main(const AttnArgs &a, const AttnPlan &p, const AttnWs &w, hipStream_t st)
{
    const unsigned grid = (unsigned)((long)p.units * p.n_chunks);
    hipLaunchKernelGGL((attn_bf16_kernel<D, NWR>), dim3(grid), dim3(512), 0, st, a, p, w);
}

template <int D>
static jt_status launch_mfma(const AttnArgs &a, void *ws, hipStream_t st)
{
    const AttnPlan p = attn_plan(a.S, a.B, a.Hq, a.Hkv, a.max_prefix, a.block_table ? a.block_size : 0);
    const AttnWs w = attn_ws_split(p, ws);
    if (p.nwr == 2)
        launch_main<D, 2>(a, p, w, st);
    else if (p.nwr == 4)
        launch_main<D, 4>(a, p, w, st);
    else
        launch_main<D, 8>(a, p, w, st);
    jt_status e = launch_status(hipGetLastError());
    if (e != JT_OK || p.n_chunks == 1 || p.fused)
        return e;
    const long threads = (long)p.units * p.rt * (D / 8);
    hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       st, a, p, w);
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
