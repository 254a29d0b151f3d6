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
// in LDS serves every row of the workgroup.  A wave owns 32 rows and runs, per 64-key
// tile,
//   S^T = K . Q^T     v_mfma_f32_32x32x16_bf16; K rows from LDS (one 16-byte read per
//                     lane), Q^T fragments held in registers for the whole kernel;
//   online softmax    exp2 domain, lazily moved reference maximum; a lane holds one row
//                     and 32 of the tile's keys, the other 32 sit in lane ^ 32;
//   O^T += V^T . P^T  P^T is the S^T accumulator converted to bf16 in place (the key
//                     order of the accumulator layout is applied to the V reads), V^T
//                     fragments come from row-major V in LDS through ds_read_b64_tr_b16.
// K/V tiles are copied HBM -> LDS by global_load_lds_dwordx4 (no register staging)
// into rows whose 16-byte segments are XOR-swizzled, which keeps both the K reads and
// the transposing V reads free of bank conflicts.  A workgroup is 2, 4 or 8 waves (64,
// 128 or 256 rows) sharing one tile stream: 8 waves run two half-tile-apart groups over
// 4 stages (ping-pong: one wave's softmax under the other's MFMAs), fewer waves double
// buffer.  All LDS reads of tiles are inline asm and only tile copies are in flight in
// the loop, so each wait is an exact vmcnt.  Keys are split over workgroups
// (split-KV) until the chip is covered; each chunk writes a normalised bf16 partial with
// its (max, sum) and attn_combine_kernel merges them.
//
// fp32 -> attn_f32_kernel: 16 query rows per workgroup on the vector ALU, K/V tiles in LDS.
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

// Workgroup barrier for LDS only, which does not drain the loads in flight:
// __syncthreads() carries a workgroup fence, which the compiler implements with
// s_waitcnt vmcnt(0) and would wait for the copies or prefetches of later tiles too.  A
// wave waits for the global data it uses itself (vmcnt, or the compiler's own wait on the
// registers); LDS accesses are drained (lgkmcnt(0)) so that LDS written before the barrier
// is seen, and may be rewritten, after it.  The asm memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void barrier_keep_dma()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

// grid (ceil(B / NV), S * Hkv), 256 threads: one workgroup per block of NV = 16 / G nodes
// (at least one) of one (sequence s, KV head g), i.e. kF32Rows = 16 query rows, node-major
// (row r: node v0 + r / G, head g * G + r % G; rows past B or past NV * G stay idle).  Per
// 64-key tile the K and V rows go to LDS with coalesced 16-byte loads.  Lane k of every
// wave holds key k and scores it against the wave's four rows (wave w: rows w, w + 4, ...),
// so the online softmax of a row is a wave reduction over the tile's keys; then thread
// (column e, row group) accumulates P . V for its rows.  The scores are in the exp2 domain
// (q is scaled by scale * log2 e when staged).
constexpr int kF32Rows = 16;
// anc: the ancestor rows to read; validate: run the argument checks (they write a.err).
// kPrefetch: issue the next tile's loads before the current tile is computed (measured:
// the fused step's fp32 phase 2 gains, the standalone pass loses on the short runs it is
// for -- tiny 11.2 us without, 12.9 us with; with a 300-key prefix 27.1 against 30.3 us --
// and gains only on long ones, 136 against 130 us over 1,040 keys, so each takes its form).
template <int D, bool kPrefetch>
__device__ __forceinline__ void attn_f32_block(const AttnArgs &a, const uint64_t *anc, bool validate,
                                               int bx, int by)
{
    constexpr int KP = D + 4;    // K row pitch in floats (staggers the lanes' 16-byte reads)
    constexpr int RG = 256 / D;  // row groups of the P . V ownership
    constexpr int NO = kF32Rows / RG;
    __shared__ __attribute__((aligned(16))) float qs[kF32Rows][D];
    __shared__ __attribute__((aligned(16))) float ks[64][KP];
    __shared__ __attribute__((aligned(16))) float vs[64][D];
    __shared__ float ps[kF32Rows][64];
    __shared__ float alpha_s[kF32Rows], m_s[kF32Rows], l_s[kF32Rows];
    __shared__ uint64_t anc_s[kF32Rows][4];
    __shared__ int kval[64];
    const int G = a.G, B = a.B;
    const int NV = max(1, kF32Rows / G);
    const int R = NV * G;
    const int v0 = bx * NV;
    const int s = by / a.Hkv, g = by % a.Hkv;
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const float *qg = reinterpret_cast<const float *>(a.q);
    const float *kp = reinterpret_cast<const float *>(a.k_prefix);
    const float *vp = reinterpret_cast<const float *>(a.v_prefix);
    const float *ktr = reinterpret_cast<const float *>(a.k_tree);
    const float *vtr = reinterpret_cast<const float *>(a.v_tree);

    if (validate && a.err && bx == 0 && g == 0)
        attn_validate(a, s);
    const int P = clamp_prefix(a, s);
    const float c = a.scale * kLog2eA;
    for (int i = t; i < kF32Rows * D; i += 256) {
        const int r = i / D, e = i % D;
        const int v = v0 + r / G;
        qs[r][e] = (r < R && v < B)
                       ? qg[(((int64_t)s * B + v) * a.Hq + g * G + r % G) * D + e] * c
                       : 0.f;
    }
    if (t < NV * 4) {
        const int v = v0 + t / 4;
        anc_s[t / 4][t % 4] = v < B ? anc[((int64_t)s * B + v) * 4 + t % 4] : 0ull;
    }
    const int v_hi = min(B - 1, v0 + NV - 1);
    const int kend = P + v_hi + 1;  // ancestors of v have indices <= v
    float m_r[4], l_r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m_r[i] = -INFINITY;
        l_r[i] = 0.f;
    }
    const int e = t % D, rg = t / D;
    float acc[NO];
#pragma unroll
    for (int j = 0; j < NO; ++j)
        acc[j] = 0.f;

    // A tile's K and V go through registers into LDS.  With kPrefetch the next tile's
    // loads are issued before the current tile is computed, so one HBM round trip overlaps
    // the compute (the pass is latency-bound: a few workgroups, each a short run of tiles).
    constexpr int NL = 64 * (D / 4) / 256;  // float4 loads of K (and of V) per thread
    static_assert(NL * 256 == 64 * (D / 4), "tile split");
    float4 kx[NL], vx[NL];
    bool kok[NL];
    auto load_tile = [&](int kt) {
#pragma unroll
        for (int q = 0; q < NL; ++q) {
            const int i = t + 256 * q;
            const int kk = i / (D / 4), c4 = i % (D / 4);
            const int j = kt + kk;
            const int64_t off = j < kend ? kv_offset(a, s, g, P, j) : -1;
            kx[q] = make_float4(0.f, 0.f, 0.f, 0.f);
            vx[q] = kx[q];
            kok[q] = off >= 0;
            if (off >= 0) {
                kx[q] = *reinterpret_cast<const float4 *>((j < P ? kp : ktr) + off + 4 * c4);
                vx[q] = *reinterpret_cast<const float4 *>((j < P ? vp : vtr) + off + 4 * c4);
            }
        }
    };
    if (kPrefetch && kend > 0)
        load_tile(0);
    for (int kt = 0; kt < kend; kt += 64) {
        // LDS-only barriers inside the loop, so that a prefetch stays in flight
        barrier_keep_dma();  // the previous tile's reads are done (first: q rows staged)
        if (!kPrefetch)
            load_tile(kt);
#pragma unroll
        for (int q = 0; q < NL; ++q) {
            const int i = t + 256 * q;
            const int kk = i / (D / 4), c4 = i % (D / 4);
            *reinterpret_cast<float4 *>(&ks[kk][4 * c4]) = kx[q];
            *reinterpret_cast<float4 *>(&vs[kk][4 * c4]) = vx[q];
            if (c4 == 0)
                kval[kk] = kok[q];
        }
        barrier_keep_dma();
        if (kPrefetch && kt + 64 < kend)
            load_tile(kt + 64);
        // scores of key kt + lane for rows wid + 4i
        const int j = kt + lane;
        float sc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int x = 0; x < D; x += 4) {
            const float4 kx = *reinterpret_cast<const float4 *>(&ks[lane][x]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 qx = *reinterpret_cast<const float4 *>(&qs[wid + 4 * i][x]);
                sc[i] = __builtin_fmaf(qx.x, kx.x, sc[i]);
                sc[i] = __builtin_fmaf(qx.y, kx.y, sc[i]);
                sc[i] = __builtin_fmaf(qx.z, kx.z, sc[i]);
                sc[i] = __builtin_fmaf(qx.w, kx.w, sc[i]);
            }
        }
        const bool key_ok = kval[lane] != 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wid + 4 * i;
            bool vis = key_ok;
            if (j >= P) {
                const int u = j - P;
                vis = vis && ((anc_s[r / G][u >> 6] >> (u & 63)) & 1ull);
            }
            vis = vis && r < R && v0 + r / G < B;
            const float sv = vis ? sc[i] : -INFINITY;
            const float m_new = fmaxf(m_r[i], wave_max_f32(sv));
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float p = __builtin_amdgcn_exp2f(sv - m_use);
            const float al = __builtin_amdgcn_exp2f(m_r[i] - m_use);
            l_r[i] = l_r[i] * al + wave_sum_f32(p);
            m_r[i] = m_new;
            ps[r][lane] = p;
            if (lane == 0)
                alpha_s[r] = al;
        }
        barrier_keep_dma();
        const int nk = min(64, kend - kt);
#pragma unroll
        for (int jo = 0; jo < NO; ++jo)
            acc[jo] *= alpha_s[rg + RG * jo];
        for (int k2 = 0; k2 < nk; ++k2) {
            const float vv = vs[k2][e];
#pragma unroll
            for (int jo = 0; jo < NO; ++jo)
                acc[jo] = __builtin_fmaf(ps[rg + RG * jo][k2], vv, acc[jo]);
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m_s[wid + 4 * i] = m_r[i];
            l_s[wid + 4 * i] = l_r[i];
        }
    }
    __syncthreads();
    float *out = reinterpret_cast<float *>(a.out);
#pragma unroll
    for (int jo = 0; jo < NO; ++jo) {
        const int r = rg + RG * jo;
        const int v = v0 + r / G;
        if (r >= R || v >= B)
            continue;
        const int64_t row = ((int64_t)s * B + v) * a.Hq + g * G + r % G;
        const float l = l_s[r];
        out[row * D + e] = l > 0.f ? acc[jo] / l : 0.f;
        if (a.lse && e == 0)
            a.lse[row] = l > 0.f ? (m_s[r] + __log2f(l)) * kLn2 : -INFINITY;
    }
}

// node blocks of the fp32 pass per (sequence, KV head)
__host__ __device__ inline int attn_f32_blocks(int B, int G)
{
    const int nv = kF32Rows / G > 1 ? kF32Rows / G : 1;
    return (B + nv - 1) / nv;
}

template <int D> __global__ void __launch_bounds__(256) attn_f32_kernel(AttnArgs a)
{
    attn_f32_block<D, false>(a, a.anc, true, blockIdx.x, blockIdx.y);
}

// ------------------------------------------------------------------ MFMA kernel --

constexpr int kBtCap = 1024;  // block-table entries of one chunk staged in LDS

// Work decomposition shared by the host launcher and the kernels.
struct AttnPlan {
    int nwr;       // waves per workgroup, one 32-row block each (4 or 8)
    int rt;        // rows per workgroup = 32 * nwr
    int n_rtiles;  // row tiles per (s, g)
    int units;     // S * Hkv * n_rtiles
    int ch;        // keys per chunk (multiple of 64)
    int n_chunks;  // chunks per unit (1 = no split-KV); 0 with the balanced schedule
    int remap;     // 1: place consecutive work items on one XCD
    int bal;       // 1: balanced schedule (equal shares of all units' key tiles)
    int nwg;       // workgroups of the balanced schedule
};

// Split-KV workspace: (m, l) per partial row, then the partial rows themselves
// (normalised, bf16).  A merge inside the main kernel by the last-arriving workgroup
// would need device-scope fences, which write back a whole L2 and cost more than the
// separate merge pass.
struct AttnWs {
    float2 *ml;
    uint16_t *o;
    int2 *ufl;  // balanced schedule: per unit, the first and last share that holds its tiles
};

// Sequences the balanced schedule handles (each attention workgroup keeps their tile
// offsets in LDS while it finds its share).
constexpr int kBalMaxS = 4096;

// Key tiles of row tile rt of a sequence with prefix length P: the keys its rows can see.
__host__ __device__ inline int attn_unit_tiles(int P, int rt, int rtrows, int B, int G)
{
    const int v_hi = min(B - 1, (rt * rtrows + rtrows - 1) / G);
    return (P + v_hi + 1 + 63) / 64;
}

// allow_bal: several sequences with 8-wave workgroups take the balanced schedule, whose
// key ranges follow the prefix lengths on the device.  (The fused step's 4-wave phase-1
// attention keeps chunks; both entry points plan alike, so their outputs stay bit-equal.)
// w4_target > 0: 4-wave workgroups whatever the row count (several 128-row tiles per KV
// head), in chunks sized for about w4_target workgroups: the plan for one sequence with
// many rows (the fused step's attention then shares its launch and its CUs with the logit
// scans, two workgroups per CU).
static AttnPlan attn_plan(int S, int B, int Hq, int Hkv, int max_prefix, int block_size,
                          bool allow_bal = false, int w4_target = 0)
{
    AttnPlan p;
    p.bal = 0;
    p.nwg = 0;
    const int rows = (Hq / Hkv) * B;
    // At least 4 waves: a 2-wave workgroup leaves the compiler a 512-register budget (its
    // LDS allows one wave per SIMD), and it then keeps the O accumulators in AGPRs and
    // copies all 64 to VGPRs and back around every tile (measured 15.9 us against 15.0 us
    // with 4 waves, two of them idle, on the 16-node, 1024-key shape).
    p.nwr = rows <= 128 || w4_target > 0 ? 4 : 8;
    if (w4_target > 0)
        allow_bal = false;
    p.rt = 32 * p.nwr;
    p.n_rtiles = (rows + p.rt - 1) / p.rt;
    p.units = S * Hkv * p.n_rtiles;
    if (allow_bal && p.nwr == 8 && S > 1 && S <= kBalMaxS) {
        // Prefix lengths differ per sequence and are known on the device only: chunks sized
        // for max_prefix leave the long sequences' workgroups running alone.  The balanced
        // schedule gives each workgroup an equal share of all units' tiles instead.
        long tmax = 0;  // tiles if every prefix held max_prefix keys
        for (int rt = 0; rt < p.n_rtiles; ++rt)
            tmax += attn_unit_tiles(max_prefix, rt, p.rt, B, Hq / Hkv);
        tmax *= (long)S * Hkv;
        if (tmax < (1L << 30)) {
            long nwg = p.nwr == 8 ? 256 : 512;
            if (block_size > 0) {
                // a share's block-table entries must fit the LDS staging area
                const long cap = max(1L, (long)(kBtCap - 2) * block_size / 64);
                nwg = max(nwg, (tmax + cap - 1) / cap);
            }
            nwg = min(nwg, tmax);
            p.bal = 1;
            p.nwg = (int)max(1L, nwg);
            p.ch = 0;
            p.n_chunks = 0;
            // The two row tiles of one (sequence, KV head) need about as many key tiles,
            // so neighbouring shares read the same keys at the same time; with the remap
            // they run on one XCD and the second read hits its L2.
            p.remap = (p.nwg % 8 == 0) ? 1 : 0;
            return p;
        }
    }
    const int gran = 64;
    const int keys = max_prefix + B;
    const int maxc = (keys + gran - 1) / gran;
    // Workgroups to aim for.  8-wave workgroups hold 128 KB of LDS, one per CU: one per
    // CU.  Smaller ones (few rows, a latency-bound pass) take at least two tiles each:
    // fewer, longer chunks cost less in the split-KV merge than they add to the pass
    // (measured on the 16-node, 1024-key shape: 17 one-tile chunks per unit 17.5 us,
    // 9 two-tile chunks 15.8 us), and they leave CUs to the logit scans of the fused step.
    // Longer ones cost more than they save: with 6 three-tile chunks the low_budget step
    // took 15.0 us and with 5 four-tile chunks 16.1 us, against 13.7 us with 9.
    const int target = w4_target > 0 ? w4_target : (p.nwr == 8 ? 256 : 128);
    int want = (target + p.units - 1) / p.units;
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
    return p;
}

// The plan of the attention entry points.  One sequence with more than 128 rows per KV
// head takes 4-wave workgroups over 128-row tiles, in chunks for about `w4` workgroups,
// instead of the 8-wave pass.  Measured on high_budget (one box, two runs each, the
// attention call alone): over inputs beyond the Infinity Cache 24.83 us with 8 waves and
// 24.15 us with w4 = 256; over inputs it holds, 23.90 and 23.10 us (and with w4 = 128,
// 384 and 512: 34.3, 26.2 and 24.6 us against 24.1 us at 256).  The fused step runs
// the same form in phase 1, beside its logit scans (one launch instead of two), with
// w4 = 192: 47.2 us per step with the 8-wave pass, 39.7 us so (40.6 us at 256, 43.3 us
// at 384).
static AttnPlan attn_plan_call(int S, int B, int Hq, int Hkv, int max_prefix, int block_size,
                               int w4 = 256)
{
    AttnPlan p = attn_plan(S, B, Hq, Hkv, max_prefix, block_size, true);
    if (p.nwr == 8 && !p.bal)
        p = attn_plan(S, B, Hq, Hkv, max_prefix, block_size, false, w4);
    return p;
}

// Rows a split-KV merge covers per unit: a row tile, or all G * B rows when they fill less
// than one (the merge's threads cover only rows that exist).
__host__ __device__ inline int attn_merge_rows(const AttnPlan &p, int G, int B)
{
    return p.rt < G * B ? p.rt : G * B;
}

static size_t attn_align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Partial slots: (unit, chunk) in the chunked schedule; in the balanced one, unit u's
// piece from workgroup w sits in slot u + w (unique: along the tiles, each step to the
// next piece moves to the next unit, the next workgroup, or both).
static size_t attn_ws_slots(const AttnPlan &p)
{
    if (p.bal)
        return ((size_t)p.units + p.nwg) * p.rt;
    return p.n_chunks <= 1 ? 0 : (size_t)p.units * p.n_chunks * p.rt;
}

static size_t attn_ws_bytes(const AttnPlan &p, int S, int d)
{
    const size_t slots = attn_ws_slots(p);
    size_t head = 0;
    if (p.bal)
        head = attn_align256((size_t)p.units * sizeof(int2));
    (void)S;
    return head + slots * sizeof(float2) + slots * (size_t)d * 2;
}

static AttnWs attn_ws_split(const AttnPlan &p, int S, void *ws)
{
    AttnWs w{nullptr, nullptr, nullptr};
    const size_t slots = attn_ws_slots(p);
    if (slots == 0 || !ws)
        return w;
    (void)S;
    uint8_t *b = reinterpret_cast<uint8_t *>(ws);
    if (p.bal) {
        w.ufl = reinterpret_cast<int2 *>(b);
        b += attn_align256((size_t)p.units * sizeof(int2));
    }
    w.ml = reinterpret_cast<float2 *>(b);
    w.o = reinterpret_cast<uint16_t *>(b + slots * sizeof(float2));
    return w;
}

// 16-byte segment swizzle of an LDS K/V row with SEGS segments.  With 16 segments (d =
// 128) every 256-byte row starts at the same bank of the 64 four-byte banks, so only the
// segment order separates rows.  Any 16 consecutive rows get 16 distinct values (a
// 16-byte K read of one segment from 16 rows is free of conflicts), and in each group of
// four rows 4a..4a+3 bit 1 is fixed while bits 2-3 take all four values: the lanes of a
// transposing V read, rows 4a..4a+3 (and 4a+4..4a+7) by segments {4b..4b+3}, then touch
// 16 distinct segments, all 64 banks.  (The order it replaced, bits 1-2 from row & 3,
// gave those reads two-way conflicts: measured with SQ_LDS_BANK_CONFLICT.)  With 8
// segments (d = 64), eight consecutive rows get distinct values.
template <int SEGS> __device__ __forceinline__ int seg_swz(int row)
{
    if constexpr (SEGS >= 16)
        return ((row & 3) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
    else
        return ((row & 3) << 1) | ((row >> 2) & 1);
}

__device__ __forceinline__ void lds_dma16(const void *gsrc, void *ldst)
{
    __builtin_amdgcn_global_load_lds((glb_void_t *)gsrc, (lds_void_t *)ldst, 16, 0, 0);
}
// vmcnt(0) through the builtin (not inline asm), so the compiler's own wait tracking
// knows that every earlier load, DMA included, has completed.
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

typedef int i32x2_t __attribute__((ext_vector_type(2)));

// Returns v unchanged but opaque to the compiler, so values derived from it are computed
// where they are used instead of being hoisted out of the tile loop (once per unrolled
// pipeline stage) and held in registers.
template <typename T> __device__ __forceinline__ T opaque(T v)
{
    asm volatile("" : "+v"(v));
    return v;
}

__device__ __forceinline__ uint32_t lds_off(const void *p)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}

// Four 16-byte LDS reads (ds_read_b128) -- K fragments of QK^T: two row addresses at two
// immediate offsets, (a0, O0), (a1, O0), (a0, O1), (a1, O1), i.e. two k-steps of two
// 32-key blocks -- issued without a wait: they are in flight until an lgkm_wait4 on them,
// so the reads of the next k-group overlap the current MFMAs.  Inline asm for the same
// reason as the transposing reads below.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <int O0, int O1>
__device__ __forceinline__ void k_issue2x2(uint32_t a0, uint32_t a1, u32x4_t &k0, u32x4_t &k1,
                                           u32x4_t &k2, u32x4_t &k3)
{
    asm volatile("ds_read_b128 %0, %4 offset:%6\n\t"
                 "ds_read_b128 %1, %5 offset:%6\n\t"
                 "ds_read_b128 %2, %4 offset:%7\n\t"
                 "ds_read_b128 %3, %5 offset:%7"
                 : "=&v"(k0), "=&v"(k1), "=&v"(k2), "=&v"(k3)
                 : "v"(a0), "v"(a1), "i"(O0), "i"(O1));
}
// Waits until at most N LDS operations are outstanding.  LDS reads complete in order, so
// with N = the number of reads issued after these fragments they have arrived; naming
// them as in/out operands keeps their uses after the wait.
template <int N>
__device__ __forceinline__ void lgkm_wait4(u32x4_t &k0, u32x4_t &k1, u32x4_t &k2, u32x4_t &k3)
{
    asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(k0), "+v"(k1), "+v"(k2), "+v"(k3) : "i"(N));
}

// Eight transposing LDS reads (ds_read_b64_tr_b16) for two output blocks (row addresses
// aa0/ab0 and aa1/ab1) at two row offsets -- block 0 at O0, O1, then block 1 at O0, O1 --
// issued without a wait (see k_issue2x2; lgkm_wait8 is the matching wait).  Inline asm
// because the builtin's memory operand carries no LDS alias information, which makes the
// compiler wait for every pending HBM->LDS copy (including the next tile's) before the
// read.
template <int O0, int O1>
__device__ __forceinline__ void tr16_issue2x2(uint32_t aa0, uint32_t ab0, uint32_t aa1,
                                              uint32_t ab1, i32x2_t (&r)[8])
{
    asm volatile("ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
                 "ds_read_b64_tr_b16 %1, %9 offset:%12\n\t"
                 "ds_read_b64_tr_b16 %2, %8 offset:%13\n\t"
                 "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
                 "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
                 "ds_read_b64_tr_b16 %5, %11 offset:%12\n\t"
                 "ds_read_b64_tr_b16 %6, %10 offset:%13\n\t"
                 "ds_read_b64_tr_b16 %7, %11 offset:%13"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
                   "=&v"(r[6]), "=&v"(r[7])
                 : "v"(aa0), "v"(ab0), "v"(aa1), "v"(ab1), "i"(O0), "i"(O1));
}
template <int N> __device__ __forceinline__ void lgkm_wait8(i32x2_t (&r)[8])
{
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]),
                   "+v"(r[6]), "+v"(r[7])
                 : "i"(N));
}

// Merge of one unit's split-KV partials for output items it .. (row, 8 columns), step
// `stride`.  Partial c of a row holds m_c (log2 domain), l_c and O_c / l_c in bf16; the
// merged row is sum_c 2^(m_c - M) l_c (O_c/l_c) / sum_c 2^(m_c - M) l_c, M = max_c m_c.
// NB chunks are loaded per round trip (the host picks NB >= the chunk count when it can).
// kBal: the balanced schedule (pl.bal), whose pass recorded each unit's first and last
// share; a separate instantiation, so that the chunked merges keep their own code.
template <int D, int NB, bool kBal = false>
__device__ __forceinline__ void attn_merge_unit(const AttnArgs &a, const AttnPlan &pl, const AttnWs &w,
                                int unit, int it, int stride)
{
    constexpr int SPR = D / 8;  // 8-column segments per row
    const int rt = unit % pl.n_rtiles;
    const int sg = unit / pl.n_rtiles;
    const int s = sg / a.Hkv, g = sg % a.Hkv;
    const int G = a.G, B = a.B;
    // pieces: nk slots from `first`, one slot apart per piece, of which nact hold keys
    int nk = pl.n_chunks, nact = 0;
    int64_t first = (int64_t)unit * pl.n_chunks;
    if constexpr (kBal) {
        // shares wf .. wl held the unit's tiles; share x wrote its piece to slot unit + x
        const int2 fl = w.ufl[unit];
        if (fl.x == fl.y)
            return;  // one workgroup held the whole unit and wrote its output
        nk = nact = fl.y - fl.x + 1;
        first = (int64_t)unit + fl.x;
    } else {
        const int P = clamp_prefix(a, s);
        const int v_hi = min(B - 1, (rt * pl.rt + pl.rt - 1) / G);
        nact = (P + v_hi + 1 + pl.ch - 1) / pl.ch;
    }
    for (; it < pl.rt * SPR; it += stride) {
        const int rl = it / SPR, sgm = it % SPR;
        const int r = rt * pl.rt + rl;
        if (r >= G * B)
            continue;
        // Chunks are read NB at a time with every load of a batch issued before any is used,
        // and folded with an online max (one pass).  The reads do not wait for the prefix
        // length (inactive chunks' slots lie inside the workspace); a chunk k >= nact is
        // dropped by selection, never multiplied in, since its bytes are stale.
        const int64_t base = first * pl.rt + rl;
        float M = -INFINITY, l = 0.f;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < nk; k0 += NB) {
            float2 ml[NB];
            uint4 u[NB];
#pragma unroll
            for (int q = 0; q < NB; ++q) {
                const int k = min(k0 + q, nk - 1);
                const int64_t slot = base + (int64_t)k * pl.rt;
                ml[q] = w.ml[slot];
                u[q] = *reinterpret_cast<const uint4 *>(w.o + slot * D + sgm * 8);
            }
#pragma unroll
            for (int q = 0; q < NB; ++q) {
                const bool use = k0 + q < nact && k0 + q < nk;
                const float mk = use ? ml[q].x : -INFINITY;
                if (mk == -INFINITY)
                    continue;  // inactive chunk, or no visible key in it
                const float Mn = fmaxf(M, mk);
                const float sc = __builtin_amdgcn_exp2f(M - Mn);  // 0 while M = -inf
                const float wk = __builtin_amdgcn_exp2f(mk - Mn) * ml[q].y;
                l = l * sc + wk;
                acc[0] = acc[0] * sc + wk * bf16_lo(u[q].x);
                acc[1] = acc[1] * sc + wk * bf16_hi(u[q].x);
                acc[2] = acc[2] * sc + wk * bf16_lo(u[q].y);
                acc[3] = acc[3] * sc + wk * bf16_hi(u[q].y);
                acc[4] = acc[4] * sc + wk * bf16_lo(u[q].z);
                acc[5] = acc[5] * sc + wk * bf16_hi(u[q].z);
                acc[6] = acc[6] * sc + wk * bf16_lo(u[q].w);
                acc[7] = acc[7] * sc + wk * bf16_hi(u[q].w);
                M = Mn;
            }
        }
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int v = r / G, h = g * G + r % G;
        const int64_t row_g = ((int64_t)s * B + v) * a.Hq + h;
        uint4 pk;
        pk.x = f32x2_to_bf16x2(acc[0] * inv, acc[1] * inv);
        pk.y = f32x2_to_bf16x2(acc[2] * inv, acc[3] * inv);
        pk.z = f32x2_to_bf16x2(acc[4] * inv, acc[5] * inv);
        pk.w = f32x2_to_bf16x2(acc[6] * inv, acc[7] * inv);
        *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(a.out) + row_g * D + sgm * 8) = pk;
        if (a.lse && sgm == 0)
            a.lse[row_g] = l > 0.f ? (M + __log2f(l)) * kLn2 : -INFINITY;
    }
}

// max(v, v of lane i ^ 32) through v_permlane32_swap (gfx950), which exchanges the upper
// half of one register with the lower half of another: applied to two copies of v, the
// pair holds both halves' values in every lane.  Inline asm on two distinct registers:
// the builtin, given one value for both operands, has its two results folded into one.
// The s_nop covers the wait states after the copies are written.
__device__ __forceinline__ float half_swap_max(float v)
{
    float a = v, b = v;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return fmaxf(a, b);
}
// v + v of lane i ^ 32, the same way (the pair holds v and the other half's value)
__device__ __forceinline__ float half_swap_add(float v)
{
    float a = v, b = v;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return a + b;
}

// s_waitcnt vmcnt(N), N < 64 (expcnt and lgkmcnt left unconstrained)
template <int N> __device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The same wait as inline asm with a memory clobber: no load may move across it, so the
// loads it counts stay issued before it.
template <int N> __device__ __forceinline__ void wait_vm_asm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}



// LDS accesses of the in-kernel ancestor rows, as inline asm for the same reason as the
// tile reads: a compiler-visible LDS access would make it wait for the in-flight copies.
__device__ __forceinline__ void lds_read_row(uint32_t addr, uint64_t (&r)[4])
{
    asm volatile("ds_read_b64 %0, %4\n\t"
                 "ds_read_b64 %1, %4 offset:8\n\t"
                 "ds_read_b64 %2, %4 offset:16\n\t"
                 "ds_read_b64 %3, %4 offset:24\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
                 : "v"(addr)
                 : "memory");
}
__device__ __forceinline__ void lds_write_row(uint32_t addr, const uint64_t (&r)[4])
{
    asm volatile("ds_write_b64 %0, %1\n\t"
                 "ds_write_b64 %0, %2 offset:8\n\t"
                 "ds_write_b64 %0, %3 offset:16\n\t"
                 "ds_write_b64 %0, %4 offset:24"
                 :
                 : "v"(addr), "v"(r[0]), "v"(r[1]), "v"(r[2]), "v"(r[3])
                 : "memory");
}
__device__ __forceinline__ int lds_read_i32(uint32_t addr)
{
    int v;
    asm volatile("ds_read_b32 %0, %1\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v)
                 : "v"(addr)
                 : "memory");
    return v;
}
__device__ __forceinline__ void lds_write_i32(uint32_t addr, int v)
{
    asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// Ancestor rows of one sequence's tree in LDS (the mask step's rows, computed in place):
// thread v holds node v (needs blockDim >= B) and `p` = parent[v].  Pointer doubling:
// row v starts as {v} with jump parent[v]; every round ORs in the row of the jump target
// and doubles the jump, so ceil(log2 B) rounds reach the root.  A parent outside
// [0, v) is treated as the root's -1 here (that sequence is flagged by the mask
// and verification steps; its attention output is unspecified).  Layout at byte
// offset `base`: 256 rows of 32 bytes, then 256 jump pointers.
__device__ __forceinline__ void tree_rows_lds(int p, int B, uint32_t base)
{
    const int v = threadIdx.x;
    const bool mine = v < B;
    int j = (mine && v > 0 && p >= 0 && p < v) ? p : -1;
    uint64_t r[4] = {0ull, 0ull, 0ull, 0ull};
    if (mine)
        r[v >> 6] = 1ull << (v & 63);
    const uint32_t row_at = base + (uint32_t)v * 32u, jmp_at = base + 256u * 32u + (uint32_t)v * 4u;
    if (mine) {
        lds_write_row(row_at, r);
        lds_write_i32(jmp_at, j);
    }
    int rounds = 0;
    while ((1 << rounds) < B)
        ++rounds;
    for (int k = 0; k < rounds; ++k) {
        barrier_keep_dma();
        uint64_t o[4] = {0ull, 0ull, 0ull, 0ull};
        int nj = -1;
        const bool act = mine && j >= 0;
        if (act) {
            lds_read_row(base + (uint32_t)j * 32u, o);
            nj = lds_read_i32(base + 256u * 32u + (uint32_t)j * 4u);
        }
        barrier_keep_dma();
        if (act) {
            r[0] |= o[0];
            r[1] |= o[1];
            r[2] |= o[2];
            r[3] |= o[3];
            j = nj;
            lds_write_row(row_at, r);
            lds_write_i32(jmp_at, j);
        }
    }
    barrier_keep_dma();
}

template <int D, int NWR> struct AttnLds {
    static constexpr int NST = NWR == 8 ? 4 : 2;  // tile stages: 4 for the ping-pong, else 2
    static constexpr int BUFB = 2 * 64 * D * 2;   // one stage: a K and a V tile of 64 keys
    static constexpr int BT_OFF = NST * BUFB;
    static constexpr int ANC_OFF = BT_OFF + kBtCap * 4;
    static constexpr int BYTES = ANC_OFF + NWR * 32 * 5 * 8;
};

// The bf16 MFMA pass over one work item: the rows of row tile `rt` of (sequence s, KV
// head g) against keys kbeg .. min(klim, the rows' last visible key) - 1.  `slot_tile`:
// the item's partial slot (normalised bf16 rows plus (m, l)), unless `final`, when the
// item covers the unit's keys alone and writes the output (and LSE) itself.  `validate`:
// this item checks the sequence's prefix and blocks.  `speculate`: copy the first tiles
// of a contiguous prefix before the prefix length is known.  `lds`: AttnLds<D, NWR>::BYTES
// of LDS, 16-byte aligned.  kTreeRows: build the ancestor rows from the parent array here
// (needs 64 * NWR >= B) instead of reading the mask step's rows.
template <int D, int NWR, bool kTreeRows>
__device__ __forceinline__ void attn_item(const AttnArgs &a, const AttnPlan &pl, const AttnWs &ws,
                                          int s, int g, int rt, int kbeg, int klim,
                                          int64_t slot_tile, bool final, bool validate,
                                          bool speculate, uint8_t *lds)
{
    constexpr int NST = AttnLds<D, NWR>::NST;
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
    constexpr int BUFB = 2 * TILEB;              // one stage: a K and a V tile
    static_assert(NIW >= 1 && NINS % NWR == 0, "DMA split");
    static_assert(NOPS < 64, "vmcnt range");
    // The NST stage buffers.  Every LDS read of a tile is inline asm, so the compiler
    // sees no LDS load to order against the in-flight copies and adds no waits of its
    // own; a stage can therefore be chosen at run time (one loop body, small code).
    static_assert(BUFB == AttnLds<D, NWR>::BUFB, "stage size");
    uint8_t *const L0 = lds;
    int *const bt_lds = reinterpret_cast<int *>(lds + AttnLds<D, NWR>::BT_OFF);
    uint64_t(*const anc_lds)[32][5] =  // rows' ancestor bits (+pad)
        reinterpret_cast<uint64_t(*)[32][5]>(lds + AttnLds<D, NWR>::ANC_OFF);

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wr = wid;  // the wave's share of the tile copies
    const int col = lane & 31, hh = lane >> 5;

    const int G = a.G, B = a.B, R = G * B;
    const int r0 = rt * pl.rt;
    // Paired 4-wave mode: at most 64 rows (two waves' worth) and chunks of at most two
    // tiles.  Waves 2 and 3 then take the rows of waves 0 and 1 over the chunk's second
    // tile while waves 0 and 1 take the first, and the two halves are merged in LDS: no
    // wave idles and the chunk costs one tile's time instead of two.
    const bool paired = NWR == 4 && R - r0 <= 64 && !pl.bal && pl.ch > 0 && pl.ch <= 2 * 64;
    const int wblk = paired ? (wid & 1) : wid;  // the wave's 32-row block
    const int v_hi = min(B - 1, (r0 + pl.rt - 1) / G);

    const uintptr_t kpre_a = reinterpret_cast<uintptr_t>(a.k_prefix);
    const uintptr_t vpre_a = reinterpret_cast<uintptr_t>(a.v_prefix);
    const uintptr_t ktr_a = reinterpret_cast<uintptr_t>(a.k_tree);
    const uintptr_t vtr_a = reinterpret_cast<uintptr_t>(a.v_tree);
    const int Hkv = a.Hkv;
    const int64_t pre_s = (int64_t)s * a.max_prefix;  // contiguous prefix: first row of s
    const bool paged = a.block_table != nullptr;
    const int bshift = a.block_shift, bsize = a.block_size, nblocks = a.num_blocks;
    auto stage = [&](int k) -> uint8_t * { return L0 + k * BUFB; };

    // ---- DMA of one tile (keys kt..kt+63) into `base` (K) and base + TILEB (V).  The
    // NWR waves share the NINS row groups; a lane copies one 16-byte segment.
    // `off_of(key)` gives the key's K/V row (element offset) and whether it lies in the
    // prefix buffers.  Exactly NOPS loads per wave.
    auto dma_tile = [=](int kt, uint8_t *base, auto off_of) {
        const int rrow = lane / SEGS, pslot = lane % SEGS;
#pragma unroll
        for (int ii = 0; ii < NIW; ++ii) {
            const int i = ii * NWR + wr;
            const int row = i * RPI + rrow;
            bool pre;
            const int64_t off = off_of(kt + row, pre);
            const int seg = pslot ^ seg_swz<SEGS>(row);
            const uintptr_t boff = (uintptr_t)(off * 2 + seg * 16);
            lds_dma16(reinterpret_cast<const void *>((pre ? kpre_a : ktr_a) + boff), base + i * 1024);
            lds_dma16(reinterpret_cast<const void *>((pre ? vpre_a : vtr_a) + boff),
                      base + TILEB + i * 1024);
        }
    };

    // ---- copy of a tile that lies inside a contiguous prefix: every lane's row sits at a
    // fixed byte offset from the tile's first row, so the per-lane part is computed once
    // and each copy adds it to a wave-uniform tile base (no per-tile 64-bit address math).
    const uint32_t pre_rowb = (uint32_t)(Hkv * D * 2);  // bytes from one prefix key to the next
    const bool fast_ok = !paged && (uint64_t)Hkv * D * 2 * TILE < (1ull << 31);
    uint32_t lane_seg[NIW];
    {
        const int rrow = lane / SEGS, pslot = lane % SEGS;
#pragma unroll
        for (int ii = 0; ii < NIW; ++ii) {
            const int row = (ii * NWR + wr) * RPI + rrow;
            lane_seg[ii] = (uint32_t)rrow * pre_rowb + (uint32_t)((pslot ^ seg_swz<SEGS>(row)) * 16);
        }
    }
    auto dma_prefix = [=](int kt, uint8_t *base) {
        const uint64_t toff = (uint64_t)(((pre_s + kt) * Hkv + g) * D) * 2;
#pragma unroll
        for (int ii = 0; ii < NIW; ++ii) {
            const int i = ii * NWR + wr;
            const uint64_t ioff = toff + (uint64_t)(i * RPI) * pre_rowb;
            lds_dma16(reinterpret_cast<const uint8_t *>(kpre_a + ioff) + lane_seg[ii], base + i * 1024);
            lds_dma16(reinterpret_cast<const uint8_t *>(vpre_a + ioff) + lane_seg[ii],
                      base + TILEB + i * 1024);
        }
    };

    // node tid's parent (clamped to a real node, so that every wave issues the load),
    // loaded before any tile copy.  The load is inline asm: the compiler does not track
    // it, and the wait before the tree rows counts the copies and query loads issued after
    // it, so the pointer doubling overlaps their flight instead of waiting for all of them
    // (the compiler's own wait there would be vmcnt(0): the masked loads in between defeat
    // its counting).
    int par_v = -1;
    if constexpr (kTreeRows) {
        const int32_t *pp = a.parent + (int64_t)s * B + min(tid, B - 1);
        asm volatile("global_load_dword %0, %1, off" : "=v"(par_v) : "v"(pp) : "memory");
    }

    // ---- speculative copies.  The prefix length is a device value: rather than wait
    // for it before the first copies, the first tiles of a contiguous prefix are fetched
    // as prefix keys right away (valid addresses for any key below max_prefix) and kept
    // if, once the length is known, every key of the tile is an in-range prefix key --
    // the same copy the exact path would have made.
    constexpr int NPRO = 2;  // tiles fetched before the loop (every stage of a double buffer)
    bool spec[NPRO];
#pragma unroll
    for (int k = 0; k < NPRO; ++k) {
        const int kt = kbeg + k * TILE;
        spec[k] = speculate && !paged && kt + TILE <= a.max_prefix;
        if (spec[k]) {
            if (fast_ok) {
                dma_prefix(kt, stage(k));
            } else {
                auto off_spec = [=](int key, bool &pre) -> int64_t {
                    pre = true;
                    return ((pre_s + key) * Hkv + g) * D;
                };
                dma_tile(kt, stage(k), off_spec);
            }
        }
    }

    // ---- rows of this wave: one 32-row block, lane holds row `col`; its Q^T fragments
    // stay in registers.  Loaded, like the speculative copies, before the prefix length.
    const int wrow0 = r0 + wblk * 32;
    const bool wave_has_rows = wrow0 < R;
    const int rr = wrow0 + col;
    const bool row_ok = rr < R;
    const int vrow = row_ok ? rr / G : 0;
    const int row_g = (s * B + vrow) * a.Hq + g * G + (row_ok ? rr % G : 0);
    bf16x8_t qf[KS];
    {
        // every lane loads (a row past the end reads a real row and is zeroed): exactly KS
        // loads per wave, which the wait below counts
        const uint16_t *qrow = reinterpret_cast<const uint16_t *>(a.q) + (int64_t)row_g * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 u = *reinterpret_cast<const uint4 *>(qrow + ks * 16 + hh * 8);
            if (!row_ok)
                u = make_uint4(0, 0, 0, 0);
            qf[ks] = __builtin_bit_cast(bf16x8_t, u);
        }
    }
    // the wave's 32 ancestor rows, later parked in LDS (lane hh holds words 2hh, 2hh+1)
    uint64_t anc_a, anc_b;
    if constexpr (kTreeRows) {
        // built in a stage the speculative copies leave free (the loop's first copy into
        // it is issued after the first barrier, when every wave has read it), or, when
        // they fill every stage, in the block-table and row areas, which are written only
        // after a barrier that follows the last read here
        static_assert(AttnLds<D, NWR>::BYTES - AttnLds<D, NWR>::BT_OFF >= JT_MAX_NODES * 36,
                      "room for the tree rows");
        const uint32_t tr_base = NPRO < NST ? lds_off(stage(NPRO))
                                            : lds_off(lds + AttnLds<D, NWR>::BT_OFF);
        // the parent has landed once at most the later copies (NOPS per speculative tile)
        // and the KS query loads are outstanding
        static_assert(NPRO == 2, "one wait per count of speculative tiles");
        if (spec[0] && spec[1])
            wait_vm_asm<2 * NOPS + KS>();
        else if (spec[0] || spec[1])
            wait_vm_asm<NOPS + KS>();
        else
            wait_vm_asm<KS>();
        tree_rows_lds(par_v, B, tr_base);
        uint64_t rw[4];
        lds_read_row(tr_base + (uint32_t)vrow * 32u, rw);
        anc_a = hh ? rw[2] : rw[0];
        anc_b = hh ? rw[3] : rw[1];
        if constexpr (NPRO == NST)
            barrier_keep_dma();
    } else {
        const uint64_t *anc_src = a.anc + ((int64_t)s * B + vrow) * 4 + 2 * hh;
        anc_a = anc_src[0];
        anc_b = anc_src[1];
    }

    if (a.err && validate)
        attn_validate(a, s);
    const int P = clamp_prefix(a, s);
    const int kend_u = P + v_hi + 1;
    const int kend = min(kend_u, klim);
    if (kbeg >= kend) {
        wait_vm<0>();  // speculative copies land before the workgroup's LDS is released
        return;        // nothing to do: the combine pass skips this chunk
    }
    const int ntiles = (kend - kbeg + TILE - 1) / TILE;
    anc_lds[wid][col][2 * hh] = anc_a;
    anc_lds[wid][col][2 * hh + 1] = anc_b;

    // ---- paged prefix: the chunk's block-table entries, staged once in LDS
    const int pend = min(kend, P);                   // prefix keys of this chunk end here
    const int bt0 = kbeg >> bshift;                  // first block of the chunk
    if (paged) {
        const int nb = kbeg < pend ? ((pend - 1) >> bshift) - bt0 + 1 : 0;
        const int32_t *btab = a.block_table + (int64_t)s * a.max_blocks;
        for (int i = tid; i < nb; i += 64 * NWR)
            bt_lds[i] = (bt0 + i < a.max_blocks) ? btab[bt0 + i] : -1;
        __syncthreads();
    }

    // Exact copy: keys past the range are clamped to the range's last key and absent
    // keys (a bad block) read the sequence's first tree row -- a finite value whose score
    // the mask removes, or whose sequence is flagged.
    auto off_exact = [=](int key_raw, bool &pre) -> int64_t {
        const int key = min(key_raw, kend - 1);
        int64_t off;
        pre = key < P;
        if (pre) {
            if (paged) {
                // inline-asm read: a compiler-visible LDS access here would make it wait for
                // every copy in flight (vmcnt(0)) before each tile's copy is issued
                const int blk = lds_read_i32(lds_off(&bt_lds[(key >> bshift) - bt0]));
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
        return off;
    };
    const int fast_end = min(P, kend);  // tiles ending here or before are plain prefix tiles
    auto issue_tile = [=](int kt, uint8_t *base) {
        if (fast_ok && kt + TILE <= fast_end)
            dma_prefix(kt, base);
        else
            dma_tile(kt, base, off_exact);
    };

    // ---- settle the speculation: keep a copy only if every key is an in-range prefix
    // key; otherwise let it land and fetch the tile exactly.
    bool have_pro[NPRO];
    {
        bool stale = false;
#pragma unroll
        for (int k = 0; k < NPRO; ++k) {
            const int kt = kbeg + k * TILE;
            have_pro[k] = spec[k] && kt + TILE <= min(P, kend);
            stale |= spec[k] && !have_pro[k];
        }
        if (stale)
            wait_vm<0>();
    }

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
        // words wa and wa+1 of this lane's row from LDS (inline asm read: the compiler
        // then has no LDS access to order against the in-flight tile copies)
        uint64_t w0, w1;
        {
            const uint32_t ad = lds_off(&anc_lds[wid][col][wa]);
            asm volatile("ds_read_b64 %0, %2\n\t"
                         "ds_read_b64 %1, %2 offset:8\n\t"
                         "s_waitcnt lgkmcnt(0)"
                         : "=&v"(w0), "=&v"(w1)
                         : "v"(ad));
        }
        if (wa == 3)
            w1 = 0ull;
        const uint64_t t = sh ? ((w0 >> sh) | (w1 << (64 - sh))) : w0;
        const uint64_t win = u0 < 0 ? ((t << (-u0)) | ((1ull << (-u0)) - 1ull)) : t;
        return win & inr;
    };

    // ---- one 64-key tile of this wave, in two parts: (1) QK^T, mask and online softmax,
    // leaving the tile's P^T fragments in pf; (2) PV from pf.
    auto qk = [&](const uint8_t *kb, f32x16_t (&sacc)[2]) {
        // S^T = K . Q^T for 2 key blocks of 32.  K row kbk*32 + col, segment 2*ks + hh;
        // the 32-row step keeps the swizzle, so it is an immediate offset.
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                sacc[kbk][j] = 0.f;
        // segment (2*ks + hh) ^ z = 2*(ks ^ (z >> 1)) + (hh ^ (z & 1)): one XOR per k-step
        const int zs = seg_swz<SEGS>(col);
        const uint32_t kbase =
            lds_off(kb) + opaque((uint32_t)(col * ROWB + (hh ^ (zs & 1)) * 16));
        const int zk = opaque(zs >> 1);
        // k-groups of 4 MFMAs: k-steps k2, k2 + 1 of both key blocks, so that the two
        // accumulator chains alternate; the reads of group n+1 are in flight during group
        // n's MFMAs
        constexpr int NKG = KS / 2;
        u32x4_t kf[2][4];
        auto kissue = [&](int n, u32x4_t (&dst)[4]) {
            const uint32_t a0 = kbase + (uint32_t)(((2 * n) ^ zk) * 32);
            const uint32_t a1 = kbase + (uint32_t)(((2 * n + 1) ^ zk) * 32);
            k_issue2x2<0, 32 * ROWB>(a0, a1, dst[0], dst[1], dst[2], dst[3]);
        };
        kissue(0, kf[0]);
#pragma unroll
        for (int n = 0; n < NKG; ++n) {
            u32x4_t (&cur)[4] = kf[n & 1];
            if (n + 1 < NKG) {
                kissue(n + 1, kf[(n + 1) & 1]);
                lgkm_wait4<4>(cur[0], cur[1], cur[2], cur[3]);
            } else {
                lgkm_wait4<0>(cur[0], cur[1], cur[2], cur[3]);
            }
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int kbk = 0; kbk < 2; ++kbk)
                    sacc[kbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8_t, cur[2 * kbk + q]), qf[2 * n + q], sacc[kbk],
                        0, 0, 0);
        }
    };
    auto softmax = [&](f32x16_t (&sacc)[2], uint64_t vis, bf16x8_t (&pf)[2][2]) {
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
        // the row maximum as a tree (short dependency chains), then across the two
        // half-waves that hold the row's two key halves
        // (each chain starts from -inf, which the compiler folds into three-input maxima of
        // the raw accumulators without canonicalising them first)
        float t8m[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const f32x16_t &a4 = sacc[q >> 2];
            const int j0 = 4 * (q & 3);
            float t = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                t = fmaxf(t, a4[j0 + i]);
            t8m[q] = t;
        }
        float mx = fmaxf(fmaxf(fmaxf(t8m[0], t8m[1]), fmaxf(t8m[2], t8m[3])),
                         fmaxf(fmaxf(t8m[4], t8m[5]), fmaxf(t8m[6], t8m[7])));
        mx = half_swap_max(mx) * c;
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
        float ps[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums: short add chains
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
                    ps[i & 3] += p;
                    t8[i] = (__bf16)p;
                }
                pf[kbk][m2] = t8;
            }
        l_i += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    };
    auto qk_softmax = [&](const uint8_t *kb, uint64_t vis, bf16x8_t (&pf)[2][2]) {
        f32x16_t sacc[2];
        qk(kb, sacc);
        softmax(sacc, vis, pf);
    };
    auto pv = [&](const uint8_t *vb, const bf16x8_t (&pf)[2][2]) {
        // O^T += V^T . P^T; V^T fragments by transposing reads of row-major V.  The key
        // rows of fragment (kbk, m2) are kbk*32 + 16*m2 + 4*hh + j16/4 (+8 for the upper
        // half); the 16- and 32-row steps leave the swizzle unchanged, so they are
        // immediate offsets.
        // segment (4*db + x) ^ z, x = 2*b2 + (j16 & 3)/2 < 4, splits into (x ^ (z & 3)) and
        // 4*(db ^ (z >> 2)): two bases per lane, one XOR per output block
        const int rowa = 4 * hh + (j16 >> 2), rowb = rowa + 8;
        const int xs = 2 * b2 + ((j16 & 3) >> 1), half = (j16 & 1) * 8;
        const int za = seg_swz<SEGS>(rowa), zb = seg_swz<SEGS>(rowb);
        const uint32_t vbase = lds_off(vb);
        const uint32_t basea = vbase + opaque((uint32_t)(rowa * ROWB + (xs ^ (za & 3)) * 16 + half));
        const uint32_t baseb = vbase + opaque((uint32_t)(rowb * ROWB + (xs ^ (zb & 3)) * 16 + half));
        const int zda = opaque(za >> 2), zdb = opaque(zb >> 2);
        // groups of 4 MFMAs: fragments f0, f0 + 1 (f = 2*kbk + m2) of output blocks db0 and
        // db0 + 1, so that two accumulator chains alternate; the reads of group n+1 are in
        // flight during group n's MFMAs
        i32x2_t vr[2][8];
        auto vissue = [&](int n, i32x2_t (&dst)[8]) {
            const int db0 = (n >> 1) * 2;
            const uint32_t aa0 = basea + (uint32_t)((db0 ^ zda) * 64);
            const uint32_t ab0 = baseb + (uint32_t)((db0 ^ zdb) * 64);
            const uint32_t aa1 = basea + (uint32_t)(((db0 + 1) ^ zda) * 64);
            const uint32_t ab1 = baseb + (uint32_t)(((db0 + 1) ^ zdb) * 64);
            if ((n & 1) == 0)
                tr16_issue2x2<0, 16 * ROWB>(aa0, ab0, aa1, ab1, dst);
            else
                tr16_issue2x2<32 * ROWB, 48 * ROWB>(aa0, ab0, aa1, ab1, dst);
        };
        constexpr int NVG = DB;  // (DB / 2 block pairs) x (2 fragment pairs)
        static_assert(DB % 2 == 0, "output blocks in pairs");
        vissue(0, vr[0]);
#pragma unroll
        for (int n = 0; n < NVG; ++n) {
            i32x2_t (&r)[8] = vr[n & 1];
            if (n + 1 < NVG) {
                vissue(n + 1, vr[(n + 1) & 1]);
                lgkm_wait8<8>(r);
            } else {
                lgkm_wait8<0>(r);
            }
            const int db0 = (n >> 1) * 2, f0 = (n & 1) * 2;
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int f = f0 + q;
                    const bf16x8_t vf = __builtin_bit_cast(
                        bf16x8_t, __builtin_shufflevector(r[4 * e + 2 * q], r[4 * e + 2 * q + 1], 0, 1, 2, 3));
                    o_acc[db0 + e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        vf, pf[f >> 1][f & 1], o_acc[db0 + e], 0, 0, 0);
                }
        }
    };
    auto compute_tile = [&](const uint8_t *kb, const uint8_t *vb, uint64_t vis) {
        bf16x8_t pf[2][2];
        qk_softmax(kb, vis, pf);
        pv(vb, pf);
    };

    if constexpr (NWR == 8) {
        // ---- 8 waves, 4 stages, two-phase ping-pong.  Waves 0-3 (group A) and 4-7 (group
        // B) share the SIMDs pairwise (wave w and w + 4 on SIMD w).  A tile j takes two
        // phases, each closed by a workgroup barrier, and in each phase one wave of every
        // SIMD issues MFMAs while the other runs a softmax on the vector ALU:
        //   phase a   A: PV of tile j-1, QK of tile j       B: softmax of tile j-1
        //   phase b   A: softmax of tile j                  B: PV of tile j-1, QK of tile j
        // (32 MFMAs against one softmax per phase).  At the barrier that opens tile j every
        // wave issues its share of the DMA of tile j + 2 into the stage of tile j - 2, whose
        // K and V both groups have finished (its last reader, B's PV, ran in phase b of
        // tile j - 1).  Before that barrier each wave waits for its own share of tile j;
        // only DMAs are in flight, so the wait is vmcnt(NOPS) while tile j + 1 may still
        // run.  A rescale of O by the softmax of tile j follows the PV of tile j - 1 and
        // precedes that of tile j, in both groups.
        const int grp = wid >> 2;
        bf16x8_t pf[2][2];
        f32x16_t sacc[2];
        if (0 < ntiles && !have_pro[0])
            issue_tile(kbeg, stage(0));
        if (1 < ntiles && !have_pro[NPRO - 1])
            issue_tile(kbeg + TILE, stage(1));
        auto mfma_phase = [&](int j) {
            if (j > 0)
                pv(stage((j - 1) & 3) + TILEB, pf);
            if (j < ntiles)
                qk(stage(j & 3), sacc);
        };
        for (int j = 0; j <= ntiles; ++j) {
            const int kt = kbeg + j * TILE;
            if (j < ntiles) {
                if (j + 1 < ntiles)
                    wait_vm<NOPS>();
                else
                    wait_vm<0>();
            }
            barrier_keep_dma();  // phase a of tile j
            if (j + 2 < ntiles)
                issue_tile(kt + 2 * TILE, stage((j + 2) & 3));
            if (wave_has_rows) {
                if (grp == 0)
                    mfma_phase(j);
                else if (j > 0)
                    softmax(sacc, vis_window(kt - TILE), pf);
            }
            barrier_keep_dma();  // phase b of tile j
            if (wave_has_rows) {
                if (grp == 0) {
                    if (j < ntiles)
                        softmax(sacc, vis_window(kt), pf);
                } else {
                    mfma_phase(j);
                }
            }
        }
    } else {
        // ---- 4 waves (few rows), double buffering: tiles 0 and 1 are fetched before the
        // loop (into the two stages); after barrier j (j >= 1), tile j + 1 goes to the
        // stage tile j - 1 used, which every wave has finished.  Before barrier 0 a wave
        // waits for its share of tile 0 only (tile 1's copies, issued after it, may still
        // run); later only tile j can be in flight.
        if (0 < ntiles && !have_pro[0])
            issue_tile(kbeg, stage(0));
        if (1 < ntiles && !have_pro[1])
            issue_tile(kbeg + TILE, stage(1));
        if (paired) {
            // ntiles <= 2: tile j goes to the waves 2j and 2j + 1
            wait_vm<0>();
            barrier_keep_dma();
            const int j = wid >> 1;
            if (wave_has_rows && j < ntiles)
                compute_tile(stage(j), stage(j) + TILEB, vis_window(kbeg + j * TILE));
            // merge: waves 2 and 3 leave (m, l, O) in LDS, beyond the epilogue staging of
            // waves 0 and 1, register by register (64 lanes x 4 bytes per store)
            // (16 bytes per lane per access: O as DB * 4 float4, then (m, l) as a float2)
            constexpr int NQ = DB * 4 + 1;
            constexpr int MOFF = (2 * 32 * (D * 2 + 16) + 255) / 256 * 256;
            static_assert(MOFF + 2 * NQ * 1024 <= NST * BUFB, "merge area fits the stages");
            float4 *mg = reinterpret_cast<float4 *>(L0 + MOFF) + (wid & 1) * NQ * 64 + lane;
            __syncthreads();  // every wave has read its tile
            if (wid >= 2 && wave_has_rows) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        mg[(db * 4 + q4) * 64] =
                            make_float4(o_acc[db][4 * q4], o_acc[db][4 * q4 + 1],
                                        o_acc[db][4 * q4 + 2], o_acc[db][4 * q4 + 3]);
                mg[DB * 4 * 64] = make_float4(m_i, l_i, 0.f, 0.f);
            }
            __syncthreads();
            if (wid < 2 && wave_has_rows) {
                const float4 ml1 = mg[DB * 4 * 64];
                const float m1 = ml1.x, l1 = ml1.y;
                const float M = fmaxf(m_i, m1);
                if (M != -INFINITY) {  // both -inf: nothing visible, keep (-inf, 0, 0)
                    const float s0 = m_i == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_i - M);
                    const float s1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
                    l_i = l_i * s0 + l1 * s1;
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            const float4 o1 = mg[(db * 4 + q4) * 64];
                            o_acc[db][4 * q4] = o_acc[db][4 * q4] * s0 + o1.x * s1;
                            o_acc[db][4 * q4 + 1] = o_acc[db][4 * q4 + 1] * s0 + o1.y * s1;
                            o_acc[db][4 * q4 + 2] = o_acc[db][4 * q4 + 2] * s0 + o1.z * s1;
                            o_acc[db][4 * q4 + 3] = o_acc[db][4 * q4 + 3] * s0 + o1.w * s1;
                        }
                    m_i = M;
                }
            }
        } else {
            for (int j = 0; j < ntiles; ++j) {
                const int k = j & 1;
                const int kt = kbeg + j * TILE;
                if (j == 0 && 1 < ntiles)
                    wait_vm<NOPS>();
                else
                    wait_vm<0>();
                barrier_keep_dma();
                if (j >= 1 && j + 1 < ntiles)
                    issue_tile(kt + TILE, stage(k ^ 1));
                if (wave_has_rows)
                    compute_tile(stage(k), stage(k) + TILEB, vis_window(kt));
            }
        }
    }

    // ---- epilogue: final output (one chunk), or a normalised bf16 partial plus (m, l)
    const float l = half_swap_add(l_i);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t slot0 = slot_tile * pl.rt + wblk * 32;
    // The accumulator spreads one row over the registers of 16 lanes.  A row-major copy of
    // the wave's 32 rows in LDS (row pitch D*2 + 16 bytes, which staggers the banks) lets
    // every lane store 16 contiguous bytes of a row instead of 8-byte pieces of 32 rows.
    constexpr int OPITCH = D * 2 + 16;
    static_assert(NWR * 32 * OPITCH <= NST * BUFB, "epilogue staging fits the tile stages");
    wait_dma();       // no tile copy may still be landing in the stages
    __syncthreads();  // every wave has finished reading the tiles
    // stored only now: vmcnt counts stores too, so a store before wait_dma() would make it
    // wait for the store's completion (measured: about 2 us per workgroup)
    const bool writer = wave_has_rows && !(paired && wid >= 2);  // merged into waves 0, 1
    if (writer && row_ok && hh == 0) {
        if (final) {
            if (a.lse)
                a.lse[row_g] = l > 0.f ? (m_i + __log2f(l)) * kLn2 : -INFINITY;
        } else {
            ws.ml[slot0 + col] = make_float2(m_i, l);
        }
    }
    if (writer) {
        uint8_t *ob = L0 + wid * 32 * OPITCH;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int d0 = db * 32 + 8 * q + 4 * hh;
                uint2 pk;
                pk.x = f32x2_to_bf16x2(o_acc[db][4 * q] * inv, o_acc[db][4 * q + 1] * inv);
                pk.y = f32x2_to_bf16x2(o_acc[db][4 * q + 2] * inv, o_acc[db][4 * q + 3] * inv);
                *reinterpret_cast<uint2 *>(ob + col * OPITCH + d0 * 2) = pk;
            }
        // the rows written by other lanes of this wave are read back below
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        constexpr int RPS = 64 / SEGS;  // rows per store instruction
#pragma unroll
        for (int it = 0; it < 32 / RPS; ++it) {
            const int row = it * RPS + lane / SEGS, sgm = lane % SEGS;
            const int rr2 = wrow0 + row;
            const uint4 val = *reinterpret_cast<const uint4 *>(ob + row * OPITCH + sgm * 16);
            if (rr2 < R) {
                uint16_t *dst;
                if (final) {
                    const int v2 = rr2 / G, h2 = g * G + rr2 % G;
                    dst = reinterpret_cast<uint16_t *>(a.out) + (((int64_t)s * B + v2) * a.Hq + h2) * D;
                } else {
                    dst = ws.o + (slot0 + row) * D;
                }
                *reinterpret_cast<uint4 *>(dst + sgm * 8) = val;
            }
        }
    }
}

// Chunked schedule: work item `blk` of `nblk` is (unit, chunk), chunks of pl.ch keys; with
// pl.remap the chunks of one unit run on one XCD and share its L2.
template <int D, int NWR, bool kTreeRows>
__device__ __forceinline__ void attn_main(const AttnArgs &a, const AttnPlan &pl, const AttnWs &ws,
                                          int blk, int nblk, uint8_t *lds)
{
    int item = blk;
    if (pl.remap) {
        const int per = nblk >> 3;
        item = (blk & 7) * per + (blk >> 3);
    }
    const int rt = item % pl.n_rtiles;
    const int chunk = (item / pl.n_rtiles) % pl.n_chunks;
    const int sg = item / (pl.n_rtiles * pl.n_chunks);
    const int g = sg % a.Hkv;
    const int kbeg = chunk * pl.ch;
    attn_item<D, NWR, kTreeRows>(a, pl, ws, sg / a.Hkv, g, rt, kbeg, kbeg + pl.ch,
                                 ((int64_t)sg * pl.n_rtiles + rt) * pl.n_chunks + chunk,
                                 pl.n_chunks == 1, rt == 0 && chunk == 0 && g == 0, true, lds);
}

// Balanced schedule, found by every workgroup at its start from the device-side prefix
// lengths (no launch of its own): per sequence its tile offset (each thread sums a run of
// sequences; the runs' offsets come from a scan of the NT sums); the thread whose run
// holds this workgroup's first tile then finds the unit and tile there (KV head and row
// tile within the sequence).  `tab`
// (2 S + 3 + NT / 64 integers) lies in LDS that no copy has touched yet; the closing
// barrier orders every read of it before the tile copies reuse that memory.  Returns the
// total tile count T; u0 = -1 for an empty share (with fewer tiles than workgroups only the
// first T take a share, of one tile each, so that the merge finds a piece from every
// workgroup it spans).
template <int NT>
__device__ __forceinline__ int64_t attn_bal_start(const AttnArgs &a, const AttnPlan &pl,
                                                  const AttnWs &ws, int w, int32_t *tab,
                                                  int &u0, int &off0)
{
    constexpr int NWV = NT / kWave;
    const int S = a.S, tid = threadIdx.x;
    int32_t *pre = tab + S + 1;
    int32_t *part = pre + S;
    int32_t *found = part + NWV;
    const int per = (S + NT - 1) / NT;
    const int s0 = min(S, tid * per), s1 = min(S, s0 + per);
    int sum = 0;
    for (int s = s0; s < s1; ++s) {
        const int P = clamp_prefix(a, s);
        pre[s] = P;
        int r = 0;
        for (int rt = 0; rt < pl.n_rtiles; ++rt)
            r += attn_unit_tiles(P, rt, pl.rt, a.B, a.G);
        tab[s] = a.Hkv * r;
        sum += a.Hkv * r;
    }
    // exclusive scan of the run sums: inclusive within each wave, then the wave totals
    const int lane = tid & 63, wid = tid >> 6;
    int inc = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(inc, o, kWave);
        if (lane >= o)
            inc += v;
    }
    if (lane == 63)
        part[wid] = inc;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int k = 0; k < NWV; ++k) {
        base += k < wid ? part[k] : 0;
        total += part[k];
    }
    const int64_t T = total;
    const int64_t nw = min((int64_t)pl.nwg, T);
    // the first tile of this workgroup's share (-1: an empty share)
    const int64_t a0 = w < nw ? (int64_t)w * T / nw : -1;
    int c = base + inc - sum;
    for (int s = s0; s < s1; ++s) {
        const int v = tab[s];  // every sequence has tiles: v >= Hkv
        tab[s] = c;
        if (a0 >= c && a0 < c + v) {
            int rel = (int)(a0 - c);
            const int ts = v / a.Hkv;  // tiles of one KV head
            const int g = rel / ts;
            rel -= g * ts;
            int rt = 0;
            for (; rt < pl.n_rtiles - 1; ++rt) {
                const int t = attn_unit_tiles(pre[s], rt, pl.rt, a.B, a.G);
                if (rel < t)
                    break;
                rel -= t;
            }
            found[0] = (s * a.Hkv + g) * pl.n_rtiles + rt;
            found[1] = rel;
        }
        c += v;
    }
    if (tid == 0)
        tab[S] = total;
    __syncthreads();
    u0 = a0 >= 0 ? found[0] : -1;
    off0 = a0 >= 0 ? found[1] : 0;
    __syncthreads();
    return T;
}

// Balanced schedule: the units' key tiles, in unit order, form one sequence of T tiles;
// workgroup w < n = min(nwg, T) takes tiles floor(w T / n) .. floor((w + 1) T / n) - 1, one
// piece per unit it meets, starting from the unit and tile attn_bal_start found.
template <int D, int NWR>
__device__ __forceinline__ void attn_main_bal(const AttnArgs &a, const AttnPlan &pl, const AttnWs &ws,
                                              int w, uint8_t *lds)
{
    static_assert((2 * kBalMaxS + 3 + NWR) * 4 <= AttnLds<D, NWR>::NST * AttnLds<D, NWR>::BUFB,
                  "the schedule's offsets must fit the tile stages");
    int u, off;
    const int64_t T = attn_bal_start<64 * NWR>(a, pl, ws, w, reinterpret_cast<int32_t *>(lds), u, off);
    if (u < 0)
        return;  // an empty share
    const int64_t nw = min((int64_t)pl.nwg, T);  // every share nonempty
    int64_t left = (int64_t)(w + 1) * T / nw - (int64_t)w * T / nw;
    const int per_seq = a.Hkv * pl.n_rtiles;
    int s = u / per_seq;
    int P = clamp_prefix(a, s);
    bool first = true;
    while (left > 0) {
        const int rt = u % pl.n_rtiles, g = (u / pl.n_rtiles) % a.Hkv;
        const int tu = attn_unit_tiles(P, rt, pl.rt, a.B, a.G);
        const int n = (int)min((int64_t)(tu - off), left);
        if (!first)
            __syncthreads();  // the previous piece's epilogue has read back its LDS staging
        first = false;
        attn_item<D, NWR, false>(a, pl, ws, s, g, rt, off * 64, (off + n) * 64, (int64_t)u + w,
                                 off == 0 && n == tu, off == 0 && g == 0 && rt == 0, false, lds);
        if (threadIdx.x == 0) {
            // the merge finds the unit's pieces from its first and last share
            if (off == 0)
                ws.ufl[u].x = w;
            if (off + n == tu)
                ws.ufl[u].y = w;
        }
        left -= n;
        off = 0;
        ++u;
        if (left > 0 && u / per_seq != s) {
            s = u / per_seq;
            P = clamp_prefix(a, s);
        }
    }
}

template <int D, int NWR>
__global__ void __launch_bounds__(64 * NWR, 8 / NWR)  // 2 waves per SIMD: no AGPR round trips
attn_bf16_kernel(AttnArgs a, AttnPlan pl, AttnWs ws)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[AttnLds<D, NWR>::BYTES];
    // Only 8-wave plans take the balanced schedule, and the entry points plan 8-wave
    // workgroups for nothing else (attn_plan_call turns an unbalanced 8-wave plan into
    // 128-row 4-wave tiles): with 8 waves the entry points never reach the chunked pass below.
    if constexpr (NWR == 8) {
        if (pl.bal) {
            // logical share w: XCD (blockIdx & 7) runs shares [x nwg/8, (x + 1) nwg/8)
            const int b = blockIdx.x;
            attn_main_bal<D, NWR>(a, pl, ws, pl.remap ? (b & 7) * (pl.nwg >> 3) + (b >> 3) : b,
                                  lds);
            return;
        }
    }
    attn_main<D, NWR, false>(a, pl, ws, blockIdx.x, gridDim.x, lds);
}

// Separate merge pass for large units: one thread per (unit, row, 8 output columns).
template <int D, int NB, bool kBal = false>
__global__ void __launch_bounds__(256)
attn_combine_kernel(AttnArgs a, AttnPlan pl, AttnWs ws)
{
    // With the chunked schedule's XCD placement, a unit's pieces were written on one XCD
    // (in order: XCD x holds the x-th eighth of the units) and are still in its L2;
    // workgroup b runs on XCD b mod 8, so the same placement of the merge reads them
    // there.  (The balanced schedule's units differ in length, so that an eighth of them
    // need not sit on one XCD.)
    const int nb = (int)gridDim.x, b0 = (int)blockIdx.x;
    const int b = pl.remap && !pl.bal && nb % 8 == 0 ? (b0 & 7) * (nb >> 3) + (b0 >> 3) : b0;
    const int64_t t = (int64_t)b * 256 + threadIdx.x;
    const int64_t per_unit = (int64_t)attn_merge_rows(pl, a.G, a.B) * (D / 8);
    const int unit = (int)(t / per_unit);
    if (unit >= pl.units)
        return;
    attn_merge_unit<D, NB, kBal>(a, pl, ws, unit, (int)(t % per_unit), (int)per_unit);
}

// ------------------------------------------------------------------ host side --

size_t attention_workspace(int S, int B, int Hq, int Hkv, int d, int max_prefix, int block_size,
                           int dtype)
{
    if (dtype != JT_BF16)
        return 0;
    return attn_ws_bytes(attn_plan_call(S, B, Hq, Hkv, max_prefix, block_size), S, d);
}

template <int D, int NWR>
static void launch_main(const AttnArgs &a, const AttnPlan &p, const AttnWs &w, hipStream_t st)
{
    const unsigned grid = p.bal ? (unsigned)p.nwg : (unsigned)((long)p.units * p.n_chunks);
    hipLaunchKernelGGL((attn_bf16_kernel<D, NWR>), dim3(grid), dim3(64 * NWR), 0, st, a, p, w);
}

template <int D>
static jt_status launch_mfma(const AttnArgs &a, void *ws, hipStream_t st)
{
    const AttnPlan p = attn_plan_call(a.S, a.B, a.Hq, a.Hkv, a.max_prefix,
                                      a.block_table ? a.block_size : 0);
    const AttnWs w = attn_ws_split(p, a.S, ws);
    if (p.nwr == 4)
        launch_main<D, 4>(a, p, w, st);
    else
        launch_main<D, 8>(a, p, w, st);
    jt_status e = launch_status(hipGetLastError());
    if (e != JT_OK || (!p.bal && p.n_chunks == 1))
        return e;
    const long threads = (long)p.units * attn_merge_rows(p, a.G, a.B) * (D / 8);
    const dim3 cgrid((unsigned)((threads + 255) / 256)), cblock(256);
    // 4, 9, 12 or 16 chunks per round trip only where that makes it a single trip; wider
    // batches cost more in registers (occupancy) and padded loads than the trips they save
    // (a batch of 12 for 9 chunks: 15.0 us per low_budget step against 14.75 with 9)
    if (p.bal)
        hipLaunchKernelGGL((attn_combine_kernel<D, 8, true>), cgrid, cblock, 0, st, a, p, w);
    else if (!p.bal && p.n_chunks <= 4)  // one sequence of many rows (128-row workgroups)
        hipLaunchKernelGGL((attn_combine_kernel<D, 4>), cgrid, cblock, 0, st, a, p, w);
    else if (!p.bal && p.n_chunks == 9)
        hipLaunchKernelGGL((attn_combine_kernel<D, 9>), cgrid, cblock, 0, st, a, p, w);
    else if (!p.bal && p.n_chunks > 9 && p.n_chunks <= 12)
        hipLaunchKernelGGL((attn_combine_kernel<D, 12>), cgrid, cblock, 0, st, a, p, w);
    else if (!p.bal && p.n_chunks > 12 && p.n_chunks <= 16)
        hipLaunchKernelGGL((attn_combine_kernel<D, 16>), cgrid, cblock, 0, st, a, p, w);
    else
        hipLaunchKernelGGL((attn_combine_kernel<D, 8>), cgrid, cblock, 0, st, a, p, w);
    return launch_status(hipGetLastError());
}

jt_status launch_attention(const AttnArgs &a, void *ws, hipStream_t st)
{
    if (a.S == 0)
        return JT_OK;
    if (a.dtype == JT_BF16)
        return a.d == 128 ? launch_mfma<128>(a, ws, st) : launch_mfma<64>(a, ws, st);
    const dim3 grid((unsigned)attn_f32_blocks(a.B, a.G), (unsigned)(a.S * a.Hkv));
    if (a.d == 128)
        hipLaunchKernelGGL((attn_f32_kernel<128>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((attn_f32_kernel<64>), grid, dim3(256), 0, st, a);
    return launch_status(hipGetLastError());
}

} // namespace jt
