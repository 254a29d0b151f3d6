// The whole draft-and-verify step in two launches (jt_draft_verify_step); three for
// several sequences of more than 128 rows per KV head, whose attention needs 8-wave
// workgroups (see step_scan_kernel).  An fp32 step takes two launches with the attention
// in the second (see step_scan_f32_kernel).
//
// Each launch runs several steps side by side, one role per range of workgroup ids:
//   phase 1  attention   the split-KV MFMA pass; its workgroups build the tree's ancestor
//                        rows in LDS from the parent array while their first tile copies
//                        are in flight, so they do not wait for the mask step
//            top-W       the per-wave partial lists of the draft logit rows
//            arg-max     the partial arg-max of the target logit rows
//            mask        ancestor rows and depths to global memory
//   phase 2  verify      the per-sequence walk (reads phase 1's rows, depths, arg-max keys)
//            top-W       the per-row merge of the partial lists
//            combine     the split-KV merge
// The roles run the device code of the separate entry points, so every output equals
// what the four calls produce one after the other.  The verification walk is the only
// writer of err[s]: it ORs the mask and attention flags (kept in the workspace) into its
// own.  Splitting the step into two dependent launches, rather than seven, removes five
// kernel boundaries from its critical path and lets the bandwidth-bound logit scans run
// beside the attention without relying on the stream scheduler.
#include "jt_internal.h"

namespace jt {

struct StepArgs {
    AttnArgs attn;
    AttnWs aws;
    const void *draft;
    int64_t draft_stride;
    const void *target;
    int64_t target_stride;
    int V, W, S, B, N;
    int32_t *ids;
    float *logprob, *row_lse, *row_entropy;
    uint64_t *tkeys;
    float2 *tms;
    float *tt;  // the lists' entropy sums, or null when no entropy is asked for
    uint64_t *gkeys;
    uint32_t *gnan;
    const int32_t *parent, *tokens;
    uint64_t *anc;
    int32_t *depth;
    int32_t *accept_len, *accept_path, *bonus, *argmax_out, *err;
    int32_t *err_mask, *err_attn;  // per-sequence flags of the mask and attention roles
};

struct StepPlan {
    AttnPlan ap;     // nwr >= 4: the phase-1 workgroup is 64 * ap.nwr threads
    TopwPlan tp;
    ArgPlan gp;
    int f32;             // fp32 step: attention on the vector ALU, in phase 2
    int nA, nT, nG, nM;  // phase-1 workgroups per role (fp32: nA counts phase 2's)
    int nV;              // fp32: the attention's prefix checks, one workgroup per sequence
    int nC, nR, nW;      // phase-2 workgroups per role
};

constexpr int kStepRowsPerBlock = 4;  // phase 2: top-W rows merged per workgroup (one per wave)
// phase-1 attention workgroups of a many-row sequence (high_budget step: 39.4 us at 192
// and 160, 40.4 at 128, 40.8 at 224, 40.6 at 256, 43.3 at 384)
constexpr int kStepAttnW4 = 192;
constexpr int kPhase1Slots = 2 * 256;  // phase-1 workgroups resident at once: 2 per CU, 256 CUs

template <int D, int NWR> struct StepLds {
    static constexpr int TOPW = NWR * (kWaveCap + 2 * JT_MAX_W) * 8;
    static constexpr int MASK = JT_MAX_NODES * (32 + 4 + 4);
    static constexpr int ARG = 2 * NWR * 8;
    static constexpr int A = AttnLds<D, NWR>::BYTES;
    static constexpr int BYTES = A > TOPW ? (A > MASK ? A : MASK) : (TOPW > MASK ? TOPW : MASK);
    static_assert(ARG <= BYTES, "arg-max slice");
};

// The scan and mask roles, for workgroups of NW waves; `b` counts from the first scan
// workgroup.
// kArgPrefetch: the arg-max role loads its next sub-chunk early, worth it in the scan
// launch (three waves per SIMD) and not in the attention-sharing phase 1.
// T: the logits' element type (uint16_t words of bf16, or float).
// kEnt: the top-W role may compute the row entropies (when asked for at run time).
template <int NW, bool kArgPrefetch, typename T = uint16_t, bool kEnt = true>
__device__ __forceinline__ void step_scan_roles(const StepArgs &sa, const StepPlan &sp, int b,
                                                uint8_t *pool)
{
    if (b < sp.nT) {
        const int wid = threadIdx.x >> 6;
        uint64_t *cand = reinterpret_cast<uint64_t *>(pool) + wid * (kWaveCap + 2 * JT_MAX_W);
        topw_partial_wave<T, true, kEnt>(
            static_cast<const T *>(sa.draft), sa.draft_stride, sa.S * sa.N, sa.V, sa.W,
            sp.tp.npiece, sp.tp.ppw, sp.tp.nlist, sa.tkeys, sa.tms, sa.tt, b * NW + wid, cand,
            cand + kWaveCap + JT_MAX_W);
        return;
    }
    b -= sp.nT;
    if (b < sp.nG) {
        argmax_partial_block<T, true, 64 * NW, kArgPrefetch>(
            static_cast<const T *>(sa.target), sa.target_stride, sa.V, sp.gp.nsub,
            sp.gp.sub_per_wg, sp.gp.nchunk, sa.gkeys, sa.gnan, b,
            reinterpret_cast<uint64_t *>(pool), reinterpret_cast<uint32_t *>(pool + NW * 8));
        return;
    }
    b -= sp.nG;
    mask_block(sa.parent, sa.B, sa.anc, sa.depth, sa.err_mask, b,
               reinterpret_cast<uint64_t(*)[4]>(pool),
               reinterpret_cast<int32_t *>(pool + JT_MAX_NODES * 32),
               reinterpret_cast<int32_t *>(pool + JT_MAX_NODES * 36));
}

template <int D, int NWR>
__device__ __forceinline__ void step_phase1_body(const StepArgs &sa, const StepPlan &sp)
{
    __shared__ __attribute__((aligned(16))) uint8_t pool[StepLds<D, NWR>::BYTES];
    // Workgroups are dispatched in id order: the top-W role first, then the attention,
    // then the arg-max and mask roles.  The top-W and attention roles end last, so they
    // start first (low_budget step: 14.37 us with the attention first, 14.07 us so;
    // 14.37 us with every scan role before the attention).
    const int b = blockIdx.x;
    if (b < sp.nT)
        step_scan_roles<NWR, false>(sa, sp, b, pool);
    else if (b < sp.nT + sp.nA)
        attn_main<D, NWR, true>(sa.attn, sp.ap, sa.aws, b - sp.nT, sp.nA, pool);
    else
        step_scan_roles<NWR, false>(sa, sp, b - sp.nA, pool);
}

// 4 waves: two workgroups per CU (register budget 256 per lane, LDS 2 x 74 KB)
template <int D>
__global__ void __launch_bounds__(256, 2) step_phase1_w4(StepArgs sa, StepPlan sp)
{
    step_phase1_body<D, 4>(sa, sp);
}

// Plans whose attention needs 8-wave workgroups (128 KB of LDS each, one per CU: the
// balanced schedule of several sequences) would leave the scans one workgroup slot per CU
// if they shared its launch.  There the scans and the mask run first in a launch of their
// own (small LDS, many workgroups per CU), then the attention pass (reading the mask's
// rows), then phase 2.
constexpr int kScanLds = 4 * (kWaveCap + 2 * JT_MAX_W) * 8 > JT_MAX_NODES * 40
                             ? 4 * (kWaveCap + 2 * JT_MAX_W) * 8
                             : JT_MAX_NODES * 40;
// Without entropies (kEnt = false) the kernel holds 125 VGPRs, four waves per SIMD.
template <bool kEnt>
__global__ void __launch_bounds__(256) step_scan_kernel(StepArgs sa, StepPlan sp)
{
    __shared__ __attribute__((aligned(16))) uint8_t pool[kScanLds];
    step_scan_roles<4, true, uint16_t, kEnt>(sa, sp, blockIdx.x, pool);
}

// fp32 steps (the tiny configuration is fp32 end to end) have no split-KV pass, so the
// attention moves to phase 2, after the mask: phase 1 (this kernel) runs the fp32 logit
// scans, the mask and, per sequence, the attention's prefix-length and block checks
// (which the verification walk of phase 2 ORs into err).
__global__ void __launch_bounds__(256) step_scan_f32_kernel(StepArgs sa, StepPlan sp)
{
    __shared__ __attribute__((aligned(16))) uint8_t pool[kScanLds];
    const int b = blockIdx.x - (sp.nT + sp.nG + sp.nM);
    if (b < 0)
        step_scan_roles<4, true, float>(sa, sp, blockIdx.x, pool);
    else
        attn_validate(sa.attn, b);
}

// fp32 phase 2: the verification walk, the top-W merge and the fp32 attention pass (over
// the mask's rows; its checks ran in phase 1).
template <int D>
__global__ void __launch_bounds__(256) step_phase2_f32(StepArgs sa, StepPlan sp)
{
    __shared__ __attribute__((aligned(16))) uint64_t mkeys[kStepRowsPerBlock][kMergeLds];
    int b = blockIdx.x;
    if (b < sp.nW) {
        verify_walk_block(b, sa.B, sa.N, sp.gp.nchunk, sa.gkeys, sa.gnan, sa.parent, sa.tokens,
                          sa.anc, sa.depth, sa.accept_len, sa.accept_path, sa.bonus,
                          sa.argmax_out, sa.err, sa.err_mask, sa.err_attn);
        return;
    }
    b -= sp.nW;
    if (b < sp.nR) {
        const int wid = threadIdx.x >> 6;
        const int r = b * kStepRowsPerBlock + wid;
        if (r < sa.S * sa.N)
            topw_merge_row(r, sa.W, sp.tp.nlist, sa.tkeys, sa.tms, sa.tt, sa.ids, sa.logprob,
                           sa.row_lse, sa.row_entropy, mkeys[wid]);
        return;
    }
    b -= sp.nR;
    // the mask role's rows; the argument checks ran in phase 1
    const int nvb = attn_f32_blocks(sa.attn.B, sa.attn.G);
    attn_f32_block<D, true>(sa.attn, sa.anc, false, b % nvb, b / nvb);
}

template <int D, int NB, bool kBal = false>
__global__ void __launch_bounds__(256) step_phase2(StepArgs sa, StepPlan sp)
{
    __shared__ __attribute__((aligned(16))) uint64_t mkeys[kStepRowsPerBlock][kMergeLds];
    // the per-row and per-sequence roles first: they are the longer ones
    int b = blockIdx.x;
    if (b < sp.nW) {
        verify_walk_block(b, sa.B, sa.N, sp.gp.nchunk, sa.gkeys, sa.gnan, sa.parent, sa.tokens,
                          sa.anc, sa.depth, sa.accept_len, sa.accept_path, sa.bonus,
                          sa.argmax_out, sa.err, sa.err_mask, sa.err_attn);
        return;
    }
    b -= sp.nW;
    if (b < sp.nR) {
        const int wid = threadIdx.x >> 6;
        const int r = b * kStepRowsPerBlock + wid;
        if (r < sa.S * sa.N)
            topw_merge_row(r, sa.W, sp.tp.nlist, sa.tkeys, sa.tms, sa.tt, sa.ids, sa.logprob,
                           sa.row_lse, sa.row_entropy, mkeys[wid]);
        return;
    }
    b -= sp.nR;
    // With the chunked schedule's XCD placement a unit's pieces were written on one XCD
    // and are still in its L2: the x-th eighth of the units on XCD (x + o) mod 8, o = the
    // attention role's first workgroup (0 in a launch of its own).  Merge workgroup i runs
    // on XCD (i + nW + nR) mod 8 and takes the units of that XCD, so it reads them there.
    if (sp.ap.remap && !sp.ap.bal && sp.nC % 8 == 0) {
        const int o = sp.ap.nwr == 8 ? 0 : sp.nT;
        b = ((((int)blockIdx.x) - o) & 7) * (sp.nC >> 3) + (b >> 3);
    }
    const int64_t t = (int64_t)b * 256 + threadIdx.x;
    const int64_t per_unit = (int64_t)attn_merge_rows(sp.ap, sa.attn.G, sa.attn.B) * (D / 8);
    const int unit = (int)(t / per_unit);
    if (unit < sp.ap.units)
        attn_merge_unit<D, NB, kBal>(sa.attn, sp.ap, sa.aws, unit, (int)(t % per_unit), (int)per_unit);
}

// ------------------------------------------------------------------ host side --

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Work decomposition of the fused step.  For few rows the phase-1 grid should fit the
// chip in one round (two 4-wave workgroups per CU); see the scan plan below.
static StepPlan step_plan(int S, int B, int N, int V, int Hq, int Hkv, int d, int max_prefix,
                          int block_size, int dtype)
{
    StepPlan sp;
    const int rows_d = S * N, rows_t = S * B;
    sp.nV = 0;
    sp.f32 = dtype == JT_F32;
    if (sp.f32) {
        // no split-KV: an empty attention plan (no workspace), the scans as the separate
        // calls plan them, the fp32 attention pass in phase 2
        sp.ap = AttnPlan{};
        sp.ap.n_chunks = 1;
        sp.tp = topw_plan(rows_d, V);
        sp.gp = arg_plan(rows_t, V);
        sp.nA = attn_f32_blocks(B, Hq / Hkv) * S * Hkv;
        sp.nT = (rows_d * sp.tp.nlist + 3) / 4;
        sp.nG = rows_t * sp.gp.nchunk;
        sp.nM = S;
        sp.nV = S;
        sp.nC = 0;
        sp.nR = (rows_d + kStepRowsPerBlock - 1) / kStepRowsPerBlock;
        sp.nW = S;
        return sp;
    }
    // One sequence with more than 128 rows per KV head: 4-wave attention workgroups over
    // 128-row tiles in phase 1, beside the scans, rather than the 8-wave pass in a launch
    // between the scans and phase 2.  (Keeping the 8-wave pass and giving the scans 8-wave
    // workgroups on the CUs it leaves free measured 50.7-53.6 us per high_budget step,
    // against 47.2 us in three launches: one scan workgroup per CU hides too little
    // latency.)  The chunks aim at fewer workgroups than the standalone call's, leaving
    // slots to the scans, so the two split keys differently.
    sp.ap = attn_plan_call(S, B, Hq, Hkv, max_prefix, block_size, kStepAttnW4);
    const bool split = sp.ap.nwr == 8;  // scans in a launch of their own
    const int nw = split ? 4 : sp.ap.nwr;  // waves per scan workgroup
    if (split) {
        sp.tp = topw_plan(rows_d, V);
        sp.gp = arg_plan(rows_t, V);
    } else {
        // Phase 1 should run in one round of two 4-wave workgroups per CU.  Top-W pieces
        // per wave cost most (the top-W role is the longest scan: 9.1 us with one piece per
        // wave against 10.4 us with two, for 16 rows of 151,936), so take the fewest pieces
        // per wave, then the fewest arg-max sub-chunks per workgroup, that fit; if nothing
        // fits, two pieces per wave and about four sub-chunks per workgroup.
        const int npiece = (V + kPiece - 1) / kPiece;
        const int nsub = (V + kArgSub - 1) / kArgSub;
        const int ppw0 = (npiece + kMaxLists - 1) / kMaxLists;
        const int nA = sp.ap.units * sp.ap.n_chunks;
        int ppw = -1, spw = -1;
        for (int pw = ppw0; pw <= ppw0 + 1 && ppw < 0; ++pw)
            for (int sw = 1; sw <= 8 && ppw < 0; ++sw) {
                const int nch = (nsub + sw - 1) / sw;
                if (nch > kArgMaxChunks)
                    continue;
                const long nT = ((long)rows_d * ((npiece + pw - 1) / pw) + nw - 1) / nw;
                if (nA + nT + (long)rows_t * nch + S <= kPhase1Slots) {
                    ppw = pw;
                    spw = sw;
                }
            }
        if (ppw < 0) {
            ppw = max(2, ppw0);
            int want = max(rows_t > 0 ? (256 + rows_t - 1) / rows_t : 1, (nsub + 3) / 4);
            spw = max(1, (nsub + want - 1) / want);
            while ((nsub + spw - 1) / spw > kArgMaxChunks)
                ++spw;
        }
        sp.tp.npiece = npiece;
        sp.tp.ppw = ppw;
        sp.tp.nlist = (npiece + ppw - 1) / ppw;
        sp.gp.nsub = nsub;
        sp.gp.sub_per_wg = spw;
        sp.gp.nchunk = (nsub + spw - 1) / spw;
    }
    sp.nA = sp.ap.bal ? sp.ap.nwg : sp.ap.units * sp.ap.n_chunks;
    sp.nT = (rows_d * sp.tp.nlist + nw - 1) / nw;
    sp.nG = rows_t * sp.gp.nchunk;
    sp.nM = S;
    sp.nC = sp.ap.bal || sp.ap.n_chunks > 1
                ? (int)(((long)sp.ap.units * attn_merge_rows(sp.ap, Hq / Hkv, B) * (d / 8) + 255) / 256)
                : 0;
    sp.nR = (rows_d + kStepRowsPerBlock - 1) / kStepRowsPerBlock;
    sp.nW = S;
    return sp;
}

struct StepWs {
    size_t attn, tkeys, tms, tt, gkeys, gnan, flags, total;
};

static StepWs step_ws_layout(const StepPlan &sp, int S, int N, int B, int W, int d)
{
    StepWs L;
    size_t off = 0;
    L.attn = off;
    off += align256(attn_ws_bytes(sp.ap, S, d));
    const size_t tparts = (size_t)S * N * sp.tp.nlist;
    L.tkeys = off;
    off += align256(tparts * W * sizeof(uint64_t));
    L.tms = off;
    off += align256(tparts * sizeof(float2));
    L.tt = off;
    off += align256(tparts * sizeof(float));
    const size_t gparts = (size_t)S * B * sp.gp.nchunk;
    L.gkeys = off;
    off += align256(gparts * sizeof(uint64_t));
    L.gnan = off;
    off += align256(gparts * sizeof(uint32_t));
    L.flags = off;
    off += align256((size_t)2 * S * sizeof(int32_t));
    L.total = off;
    return L;
}

size_t step_workspace(int S, int B, int N, int W, int V, int Hq, int Hkv, int d, int max_prefix,
                      int block_size, int dtype)
{
    const StepPlan sp = step_plan(S, B, N, V, Hq, Hkv, d, max_prefix, block_size, dtype);
    return step_ws_layout(sp, S, N, B, W, d).total;
}

template <int D>
static void launch_step_d(const StepArgs &sa, const StepPlan &sp, hipStream_t st)
{
    if (sp.f32) {
        hipLaunchKernelGGL(step_scan_f32_kernel, dim3((unsigned)(sp.nT + sp.nG + sp.nM + sp.nV)),
                           dim3(256), 0, st, sa, sp);
        hipLaunchKernelGGL((step_phase2_f32<D>), dim3((unsigned)(sp.nW + sp.nR + sp.nA)),
                           dim3(256), 0, st, sa, sp);
        return;
    }
    if (sp.ap.nwr == 8) {
        const unsigned gs = (unsigned)(sp.nT + sp.nG + sp.nM);
        if (sa.tt)
            hipLaunchKernelGGL(step_scan_kernel<true>, dim3(gs), dim3(256), 0, st, sa, sp);
        else
            hipLaunchKernelGGL(step_scan_kernel<false>, dim3(gs), dim3(256), 0, st, sa, sp);
        AttnArgs a = sa.attn;
        a.anc = sa.anc;  // the mask role's rows
        a.parent = nullptr;
        hipLaunchKernelGGL((attn_bf16_kernel<D, 8>), dim3((unsigned)sp.nA), dim3(512), 0, st, a,
                           sp.ap, sa.aws);
    } else {
        const unsigned g1 = (unsigned)(sp.nA + sp.nT + sp.nG + sp.nM);
        hipLaunchKernelGGL((step_phase1_w4<D>), dim3(g1), dim3(256), 0, st, sa, sp);
    }
    const unsigned g2 = (unsigned)(sp.nC + sp.nR + sp.nW);
    if (sp.ap.bal)
        hipLaunchKernelGGL((step_phase2<D, 8, true>), dim3(g2), dim3(256), 0, st, sa, sp);
    else if (sp.ap.n_chunks <= 4)  // one sequence of many rows
        hipLaunchKernelGGL((step_phase2<D, 4>), dim3(g2), dim3(256), 0, st, sa, sp);
    else if (sp.ap.n_chunks == 9)  // 1024-key prefixes in two-tile chunks
        hipLaunchKernelGGL((step_phase2<D, 9>), dim3(g2), dim3(256), 0, st, sa, sp);
    else if (sp.ap.n_chunks > 9 && sp.ap.n_chunks <= 12)
        hipLaunchKernelGGL((step_phase2<D, 12>), dim3(g2), dim3(256), 0, st, sa, sp);
    else if (sp.ap.n_chunks > 12 && sp.ap.n_chunks <= 16)
        hipLaunchKernelGGL((step_phase2<D, 16>), dim3(g2), dim3(256), 0, st, sa, sp);
    else
        hipLaunchKernelGGL((step_phase2<D, 8>), dim3(g2), dim3(256), 0, st, sa, sp);
}

jt_status launch_step(const StepLaunch &in, void *ws, hipStream_t st)
{
    if (in.attn.S == 0)
        return JT_OK;
    const AttnArgs &aa = in.attn;
    const StepPlan sp = step_plan(aa.S, aa.B, in.N, in.V, aa.Hq, aa.Hkv, aa.d, aa.max_prefix,
                                  aa.block_table ? aa.block_size : 0, aa.dtype);
    const StepWs L = step_ws_layout(sp, aa.S, in.N, aa.B, in.W, aa.d);
    uint8_t *w = static_cast<uint8_t *>(ws);
    StepArgs sa;
    sa.attn = aa;
    sa.attn.anc = nullptr;
    sa.attn.parent = in.parent;
    sa.err_mask = reinterpret_cast<int32_t *>(w + L.flags);
    sa.err_attn = sa.err_mask + aa.S;
    sa.attn.err = sa.err_attn;
    sa.aws = attn_ws_split(sp.ap, aa.S, w + L.attn);
    sa.draft = in.draft;
    sa.draft_stride = in.draft_stride;
    sa.target = in.target;
    sa.target_stride = in.target_stride;
    sa.V = in.V;
    sa.W = in.W;
    sa.S = aa.S;
    sa.B = aa.B;
    sa.N = in.N;
    sa.ids = in.ids;
    sa.logprob = in.logprob;
    sa.row_lse = in.row_lse;
    sa.row_entropy = in.row_entropy;
    sa.tt = in.row_entropy ? reinterpret_cast<float *>(w + L.tt) : nullptr;
    sa.tkeys = reinterpret_cast<uint64_t *>(w + L.tkeys);
    sa.tms = reinterpret_cast<float2 *>(w + L.tms);
    sa.gkeys = reinterpret_cast<uint64_t *>(w + L.gkeys);
    sa.gnan = reinterpret_cast<uint32_t *>(w + L.gnan);
    sa.parent = in.parent;
    sa.tokens = in.tokens;
    sa.anc = in.anc;
    sa.depth = in.depth;
    sa.accept_len = in.accept_len;
    sa.accept_path = in.accept_path;
    sa.bonus = in.bonus;
    sa.argmax_out = in.argmax_out;
    sa.err = in.err;
    if (aa.d == 128)
        launch_step_d<128>(sa, sp, st);
    else
        launch_step_d<64>(sa, sp, st);
    return launch_status(hipGetLastError());
}

} // namespace jt
