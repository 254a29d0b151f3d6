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
//   * a piece is pulled into registers with 16-byte loads (32 logits per lane; the next
//     piece's loads are issued before the current one is processed) and reduced there:
//     lane max, then sum of exp(x - max) (exact per-lane rescale);
//   * only logits at or above a threshold (a lower bound on the piece's W-th largest)
//     become 64-bit keys (order code << 32 | ~id): value descending, id ascending in one
//     integer compare, so bf16 ties resolve exactly like a full sort; the new list is
//     picked among them and the wave's running list by rank counts;
//   * a merge kernel (one wave per row) combines the per-wave top-W lists and the
//     (max, sum-exp) pairs into ids, log-probs and the row log-sum-exp, selecting by
//     rank counts;
//   * on request the same pass gives the row's softmax entropy (the per-depth entropy of
//     entropy-guided and hybrid tree scoring, paperlayer.ai JetSpec summary, appendices C
//     and E): with S = sum exp(x - m) and T = sum exp(x - m) (x - m) over a set of logits,
//     H = log S - T / S, and both sums move to a new reference m' exactly as
//     S' = c S, T' = c (T + (m - m') S) with c = exp(m - m').
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

// The raw words of a lane's 32 logits of one piece: element k of load i sits at index
// base + (lane + 64*i)*E + k.  Entries at or past V are never read (their bits stay 0);
// unpack_piece marks them invalid.  Split from the unpacking so that the loads of the next
// piece can be in flight while the current one is processed.
template <typename T> struct RawPiece {
    uint4 u[Vec<T>::kLoads];
};

template <typename T, bool kAligned>
__device__ __forceinline__ void load_piece_raw(const T *__restrict__ row, int64_t base, int V,
                                               int lane, RawPiece<T> &r)
{
    constexpr int E = Vec<T>::kElems;
    constexpr int L = Vec<T>::kLoads;
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int64_t e0 = base + (int64_t)(lane + kWave * i) * E;
        if (kAligned && e0 + E <= V) {
            r.u[i] = *reinterpret_cast<const uint4 *>(row + e0);
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
            r.u[i] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

// Logit values of a raw piece; entries at or past V become -inf with valid = false.
template <typename T>
__device__ __forceinline__ void unpack_piece(const RawPiece<T> &r, int64_t base, int V, int lane,
                                             float (&x)[32], uint32_t &valid)
{
    constexpr int E = Vec<T>::kElems;
    constexpr int L = Vec<T>::kLoads;
    valid = 0;
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int64_t e0 = base + (int64_t)(lane + kWave * i) * E;
        const uint4 u = r.u[i];
        if constexpr (sizeof(T) == 2) {
            x[i * 8 + 0] = bf16_lo(u.x); x[i * 8 + 1] = bf16_hi(u.x);
            x[i * 8 + 2] = bf16_lo(u.y); x[i * 8 + 3] = bf16_hi(u.y);
            x[i * 8 + 4] = bf16_lo(u.z); x[i * 8 + 5] = bf16_hi(u.z);
            x[i * 8 + 6] = bf16_lo(u.w); x[i * 8 + 7] = bf16_hi(u.w);
        } else {
            x[i * 4 + 0] = __uint_as_float(u.x); x[i * 4 + 1] = __uint_as_float(u.y);
            x[i * 4 + 2] = __uint_as_float(u.z); x[i * 4 + 3] = __uint_as_float(u.w);
        }
        if (e0 + E <= V) {
            valid |= ((1u << E) - 1u) << (i * E);
        } else {
#pragma unroll
            for (int k = 0; k < E; ++k) {
                if (e0 + k < V)
                    valid |= 1u << (i * E + k);
                else
                    x[i * E + k] = -INFINITY;
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

// Wave-wide maximum / OR of a 32-bit value through DPP row operations and the row
// broadcasts; every lane receives the result.
template <int CTRL, int ROW_MASK> __device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp_u32<0xB1, 0xF>(v));   // quad_perm [1,0,3,2]
    v = max(v, dpp_u32<0x4E, 0xF>(v));   // quad_perm [2,3,0,1]
    v = max(v, dpp_u32<0x141, 0xF>(v));  // row_half_mirror
    v = max(v, dpp_u32<0x140, 0xF>(v));  // row_mirror
    v = max(v, dpp_u32<0x142, 0xA>(v));  // row_bcast:15
    v = max(v, dpp_u32<0x143, 0xC>(v));  // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v)
{
    v |= dpp_u32<0xB1, 0xF>(v);
    v |= dpp_u32<0x4E, 0xF>(v);
    v |= dpp_u32<0x141, 0xF>(v);
    v |= dpp_u32<0x140, 0xF>(v);
    v |= dpp_u32<0x142, 0xA>(v);
    v |= dpp_u32<0x143, 0xC>(v);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// The W-th largest of the lanes' codes, counting equal codes as often as they occur (W
// rounds of a wave max, each removing one occurrence); 0 if fewer than W codes are nonzero.
__device__ __forceinline__ uint32_t wave_wth_code(uint32_t code, int W)
{
    const int lane = threadIdx.x & 63;
    uint32_t t = 0u;
    for (int r = 0; r < W; ++r) {
        t = wave_max_u32(code);
        if (t == 0u)
            return 0u;
        const uint64_t at = __ballot(code == t);
        if (lane == __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(at)))
            code = 0u;
    }
    return t;
}

// For each of a lane's K keys, the number of entries of keys[0..n) greater than it.  n is a
// multiple of 8 (the caller pads with zero keys) and keys is 16-byte aligned.  Every lane
// reads the same entries, so each read is an LDS broadcast.  (Issuing the next reads
// before comparing the current ones measured slower: more registers and copies.)
template <int K>
__device__ __forceinline__ void count_greater(const uint64_t *keys, int n, const uint64_t (&mine)[K],
                                              int (&cnt)[K])
{
#pragma unroll
    for (int k = 0; k < K; ++k)
        cnt[k] = 0;
#pragma unroll 4
    for (int i = 0; i < n; i += 2) {
        const ulonglong2 p = *reinterpret_cast<const ulonglong2 *>(keys + i);
#pragma unroll
        for (int k = 0; k < K; ++k)
            cnt[k] += (p.x > mine[k] ? 1 : 0) + (p.y > mine[k] ? 1 : 0);
    }
}

// Each wave owns `ppw` consecutive pieces of 2048 logits of one row and works alone (no
// workgroup barrier).  Per piece:
//   * the lane's (max, sum of exp(x - max)), merged into a running pair;
//   * a threshold tau: the larger of the W-th largest lane maximum and the W-th entry of
//     the wave's running list (a lower bound on the W-th largest key of the piece and the
//     list together), so only logits >= tau can enter the list;
//   * the candidates, one ballot per slot j (one float compare per logit; slots no lane
//     needs are skipped), compacted into the wave's LDS slice as 64-bit keys (order code
//     << 32 | ~id: value descending, id ascending in one integer compare, so bf16 ties
//     resolve like a full sort) at offsets from mbcnt;
//   * the running list (lane r holds entry r) is appended and the new list picked by
//     rank: with at most 64 keys each key's place is the number of keys above it, counted
//     over LDS broadcast reads, else W rounds of a wave maximum over the LDS slice.
// Output per wave: its W best keys, descending, 0-padded, its (max, sum) pair and, when
// ws_t is not null, the entropy sum T of its logits (relative to the same max).
// `cand` holds kWaveCap + JT_MAX_W keys and `best` JT_MAX_W keys of this wave's LDS.
// kEnt = false compiles the entropy sums out (fewer registers: with them the fused scan
// launch holds 131 VGPRs and three waves per SIMD, without them 125 and four); with
// kEnt = true they run when ws_t is not null.
template <typename T, bool kAligned, bool kEnt = true>
__device__ __forceinline__ void topw_partial_wave(const T *__restrict__ logits, int64_t row_stride,
                                                  int rows, int V, int W, int npiece, int ppw,
                                                  int nlist, uint64_t *__restrict__ ws_keys,
                                                  float2 *__restrict__ ws_ms,
                                                  float *__restrict__ ws_t, int gl,
                                                  uint64_t *cand, uint64_t *best)
{
    constexpr int E = Vec<T>::kElems;
    const bool want_t = kEnt && ws_t != nullptr;
    const int lane = threadIdx.x & 63;
    if (gl >= rows * nlist)
        return;
    const int row_idx = gl / nlist, li = gl % nlist;
    const T *row = logits + (int64_t)row_idx * row_stride;
    float run_m = -INFINITY, run_s = 0.f;  // lane's running (max, sum exp(x - max))
    float run_t = 0.f;                     // and sum exp(x - max) (x - max), on request
    uint64_t run = 0ull;                   // lane r < W: entry r of the running top-W list
    const int p0 = li * ppw, p1 = min(npiece, p0 + ppw);
    RawPiece<T> next;
    if (p0 < p1)
        load_piece_raw<T, kAligned>(row, (int64_t)p0 * kPiece, V, lane, next);
    for (int pc = p0; pc < p1; ++pc) {
        const int64_t base = (int64_t)pc * kPiece;
        const RawPiece<T> cur = next;
        if (pc + 1 < p1)  // the next piece's loads overlap this piece's work
            load_piece_raw<T, kAligned>(row, base + kPiece, V, lane, next);
        float x[32];
        uint32_t valid;
        unpack_piece<T>(cur, base, V, lane, x, valid);
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < 32; ++j)
            m = fmaxf(m, x[j]);
        float sx = 0.f, tx = 0.f;
        if (m != -INFINITY) {
            const float mb = m * kLog2e;
            float part[4] = {0.f, 0.f, 0.f, 0.f};
            if (want_t) {
                float tp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], kLog2e, -mb));
                    part[j & 3] += e;
                    tp[j & 3] += e > 0.f ? e * (x[j] - m) : 0.f;  // p = 0 adds 0
                }
                tx = (tp[0] + tp[1]) + (tp[2] + tp[3]);
            } else {
#pragma unroll
                for (int j = 0; j < 32; ++j)
                    part[j & 3] += __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], kLog2e, -mb));
            }
            sx = (part[0] + part[1]) + (part[2] + part[3]);
        } else {
            // every entry is -inf, padding or NaN: only a NaN must still poison the sum
#pragma unroll
            for (int j = 0; j < 32; ++j)
                if (x[j] != x[j])
                    sx = x[j];
        }
        if (m > run_m) {
            if (run_m == -INFINITY) {
                run_s = ((run_s != run_s) ? run_s : 0.f) + sx;
                run_t = tx;
            } else {
                const float c = __builtin_amdgcn_exp2f((run_m - m) * kLog2e);
                if (want_t)
                    run_t = c * (run_t + (run_m - m) * run_s) + tx;
                run_s = run_s * c + sx;
            }
            run_m = m;
        } else if (m == -INFINITY) {
            run_s += sx;  // adds 0, or propagates a NaN
        } else {
            const float c = __builtin_amdgcn_exp2f((m - run_m) * kLog2e);
            if (want_t)
                run_t += c * (tx + (m - run_m) * sx);
            run_s += sx * c;
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
        const uint32_t run_w =
            (uint32_t)((uint64_t)__builtin_amdgcn_readlane((int)(run >> 32), W - 1));
        tau = max(tau, run_w);
        auto key_of = [&](int j) -> uint64_t {
            const uint32_t id = (uint32_t)(base + (int64_t)lane * E) + (uint32_t)(kWave * E * (j / E) + j % E);
            return ((uint64_t)order_code(x[j]) << 32) | (uint64_t)(~id);
        };
        // candidates: the valid elements at or above the threshold (x >= tf <=> code(x) >=
        // tau for non-NaN x), or every valid element when tau == 0 (fewer than W real lane
        // maxima).  Each slot j is tested with one ballot; slots no lane needs are skipped.
        const bool all = tau == 0u;
        const float tf = all ? 0.f : order_decode(tau);
        auto is_cand = [&](int j) -> bool {
            const bool in = (valid >> j) & 1u;
            return all ? in : (in && x[j] >= tf);
        };
        int n = 0;
        auto take = [&](int j, bool pred) {
            const uint64_t b = __ballot(pred);
            if (b != 0ull) {
                const int slot = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
                if (pred && slot < kWaveCap)
                    cand[slot] = key_of(j);
                n += __popcll(b);
            }
        };
        if (!all && __ballot(valid != 0xffffffffu) == 0ull) {
            // no padding in the piece (every piece but a row's last): one compare per slot
#pragma unroll
            for (int j = 0; j < 32; ++j)
                take(j, x[j] >= tf);
        } else {
#pragma unroll
            for (int j = 0; j < 32; ++j)
                take(j, is_cand(j));
        }
        if (n > kWaveCap) {
            // rare overflow (huge ties): W rounds of exact arg-max over the registers
            uint64_t prev = ~0ull;
            for (int r = 0; r < W; ++r) {
                uint64_t mine = 0ull;
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    if (!is_cand(j))
                        continue;
                    const uint64_t k = key_of(j);
                    if (k < prev && k > mine)
                        mine = k;
                }
                mine = wave_max_u64_dpp(mine);
                if (lane == 0)
                    cand[r] = mine;
                prev = mine;
            }
            n = W;
        }
        if (lane < W)
            cand[n + lane] = run;
        const int tot = n + W;
        const int tot8 = (tot + 7) & ~7;
        if (tot <= kWave && lane < tot8 - tot)
            cand[tot + lane] = 0ull;  // zero keys up to a multiple of 8 for the counting reads
        wave_sync();
        if (tot <= kWave) {
            // rank by count: a key's place in the new list is the number of keys above it
            // (nonzero keys are unique: distinct ids), for all keys at once instead of W
            // dependent wave-wide maxima
            uint64_t mine[1] = {lane < tot ? cand[lane] : 0ull};
            int cnt[1];
            count_greater<1>(cand, tot8, mine, cnt);
            const int nz = __popcll(__ballot(mine[0] != 0ull));
            if (mine[0] != 0ull && cnt[0] < W)
                best[cnt[0]] = mine[0];
            wave_sync();
            run = lane < min(W, nz) ? best[lane] : 0ull;
        } else {
            wave_select_topw(cand, tot, W, best);
            run = lane < W ? best[lane] : 0ull;
        }
        wave_sync();  // the slice is rewritten by the next piece
    }

    // ---- (max, sum) and T over the wave
    const float m = wave_max_f32(run_m);
    float sw, tw = 0.f;
    if (run_m == -INFINITY) {
        sw = (run_s != run_s) ? run_s : 0.f;
    } else {
        const float c = __builtin_amdgcn_exp2f((run_m - m) * kLog2e);
        sw = run_s * c;
        if (want_t)
            tw = c * (run_t + (run_m - m) * run_s);
    }
    sw = wave_sum_f32(sw);
    if (want_t)
        tw = wave_sum_f32(tw);
    if (lane == 0) {
        ws_ms[gl] = make_float2(m, sw);
        if (want_t)
            ws_t[gl] = tw;
    }
    if (lane < W)
        ws_keys[(int64_t)gl * W + lane] = run;
}

template <typename T, bool kAligned, bool kEnt>
__global__ void __launch_bounds__(kTopwThreads)
topw_partial_kernel(const T *__restrict__ logits, int64_t row_stride, int rows, int V, int W,
                    int npiece, int ppw, int nlist, uint64_t *__restrict__ ws_keys,
                    float2 *__restrict__ ws_ms, float *__restrict__ ws_t)
{
    // per wave: kWaveCap + JT_MAX_W candidate keys, then JT_MAX_W list keys
    constexpr int kSlice = kWaveCap + 2 * JT_MAX_W;
    __shared__ __attribute__((aligned(16))) uint64_t pool[4 * kSlice];
    const int wid = threadIdx.x >> 6;
    uint64_t *cand = pool + wid * kSlice;
    topw_partial_wave<T, kAligned, kEnt>(logits, row_stride, rows, V, W, npiece, ppw, nlist,
                                         ws_keys, ws_ms, ws_t, blockIdx.x * 4 + wid, cand,
                                         cand + kWaveCap + JT_MAX_W);
}

constexpr int kMergeCand = JT_MAX_W * JT_MAX_W;  // candidate keys a row merge can keep
constexpr int kMergeLds = kMergeCand + 8;          // LDS keys per merging wave (8 of padding)


// One wave per row: merge the partial lists and (max, sum) pairs of row r.  Every list is
// sorted descending and nonzero keys are unique, so the W-th largest list head bounds the
// row's W-th largest key from below: only keys at or above it compete, at most W from
// each of the W lists whose head reaches it (all keys compete when there are at most W
// lists).  Selection is by rank: a key's place in the output is the number of competing
// keys above it, counted over LDS broadcast reads, first for the list heads (the head
// ranked W - 1 is the bound), then for the competitors.  `keys`: kMergeLds entries of
// this wave's LDS, 16-byte aligned.
//
// With at most 8 keys per lane and W <= 4, W rounds of a DPP wave max straight over the
// registers are cheaper than the two counting passes, and are used instead.
__device__ __forceinline__ void topw_merge_row(int r, int W, int nchunk, const uint64_t *__restrict__ ws_keys,
                               const float2 *__restrict__ ws_ms, const float *__restrict__ ws_t,
                               int32_t *__restrict__ ids, float *__restrict__ logprob,
                               float *__restrict__ row_lse, float *__restrict__ row_entropy,
                               uint64_t *keys)
{
    const int lane = threadIdx.x & 63;
    const int n = nchunk * W;
    // Every load is issued before any result is used (one memory round trip): the (max,
    // sum) pairs, the list heads and all keys.
    constexpr int kMsPerLane = kMaxLists / kWave;
    constexpr int kKeysPerLane = kMaxLists * JT_MAX_W / kWave;
    const float2 *msr = ws_ms + (int64_t)r * nchunk;
    const uint64_t *src = ws_keys + (int64_t)r * n;
    float2 ms[kMsPerLane];
    float ts[kMsPerLane];
    uint64_t hd[kMsPerLane];
#pragma unroll
    for (int j = 0; j < kMsPerLane; ++j) {
        const int c = lane + kWave * j;
        ms[j] = c < nchunk ? msr[c] : make_float2(-INFINITY, 0.f);
        ts[j] = (row_entropy && c < nchunk) ? ws_t[(int64_t)r * nchunk + c] : 0.f;
        hd[j] = c < nchunk ? src[(int64_t)c * W] : 0ull;
    }
    const int nq = (n + kWave - 1) / kWave;  // key slots in use (wave-uniform)
    uint64_t kr[kKeysPerLane];
#pragma unroll
    for (int q = 0; q < kKeysPerLane; ++q) {
        kr[q] = 0ull;
        if (q < nq) {
            const int i = lane + kWave * q;
            if (i < n)
                kr[q] = src[i];
        }
    }
    // LSE over the row
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMsPerLane; ++j)
        m = fmaxf(m, ms[j].x);
    m = wave_max_f32(m);
    float s = 0.f, t = 0.f;
#pragma unroll
    for (int j = 0; j < kMsPerLane; ++j) {
        const float2 p = ms[j];
        if (p.x == -INFINITY) {
            s += (p.y != p.y) ? p.y : 0.f;
        } else {
            const float c = __builtin_amdgcn_exp2f((p.x - m) * kLog2e);
            s += p.y * c;
            t += c * (ts[j] + (p.x - m) * p.y);
        }
    }
    s = wave_sum_f32(s);
    float lse;
    if (s != s)
        lse = s;
    else if (m == -INFINITY)
        lse = -INFINITY;
    else
        lse = m + logf(s);
    if (row_entropy) {
        t = wave_sum_f32(t);
        // H = log S - T / S; a NaN row gives NaN, a row of -inf (no distribution) 0
        const float h = (s != s) ? s : (m == -INFINITY ? 0.f : logf(s) - t / s);
        if (lane == 0)
            row_entropy[r] = h;
    }

    if (nq <= 8 && W <= 4) {
        // W rounds, each taking the largest key below the previous winner
        uint64_t prev = ~0ull, mine_top = 0ull;
        for (int k = 0; k < W; ++k) {
            uint64_t mine = 0ull;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (q < nq)
                    mine = (kr[q] < prev && kr[q] > mine) ? kr[q] : mine;
            const uint64_t K = wave_max_u64_dpp(mine);
            if (lane == k)
                mine_top = K;
            prev = K;
        }
        if (lane < W) {
            ids[(int64_t)r * W + lane] = (int32_t)key_id(mine_top);
            logprob[(int64_t)r * W + lane] = key_value(mine_top) - lse;
        }
        if (lane == 0 && row_lse)
            row_lse[r] = lse;
        return;
    }
    // bound: the head ranked W - 1 (0 when there are at most W lists)
    uint64_t tau = 0ull;
    if (nchunk > W) {
#pragma unroll
        for (int j = 0; j < kMsPerLane; ++j)
            if (lane + kWave * j < nchunk)
                keys[lane + kWave * j] = hd[j];
        if (lane < 8)
            keys[nchunk + lane] = 0ull;  // pad to a multiple of 8
        wave_sync();
        int cnt[kMsPerLane];
        count_greater<kMsPerLane>(keys, (nchunk + 7) & ~7, hd, cnt);
        uint64_t t = 0ull;
#pragma unroll
        for (int j = 0; j < kMsPerLane; ++j)
            if (hd[j] != 0ull && cnt[j] == W - 1)
                t = hd[j];
        const uint64_t own = __ballot(t != 0ull);
        if (own) {
            const int src_lane = (int)__builtin_ctzll(own);
            tau = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(t >> 32), src_lane) << 32) |
                  (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)t, src_lane);
        }
        wave_sync();  // the heads are overwritten by the competitors
    }
    // competitors: nonzero keys >= tau, compacted slot by slot (slots no lane needs skipped)
    uint32_t mk = 0u;
#pragma unroll
    for (int q = 0; q < kKeysPerLane; ++q)
        if (q < nq)
            mk |= (kr[q] != 0ull && kr[q] >= tau ? 1u : 0u) << q;
    const uint32_t jm = wave_or_u32(mk);
    int nc = 0;
#pragma unroll
    for (int q = 0; q < kKeysPerLane; ++q) {
        if (jm & (1u << q)) {
            const bool pred = (mk >> q) & 1u;
            const uint64_t b = __ballot(pred);
            const int slot = nc + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
            if (pred && slot < kMergeCand)
                keys[slot] = kr[q];
            nc += __popcll(b);
        }
    }
    if (nc > kMergeCand)
        nc = kMergeCand;  // not reached: at most W * W keys reach the bound
    if (lane < 8)
        keys[nc + lane] = 0ull;  // pad to a multiple of 8
    wave_sync();
    const int ne = (nc + 7) & ~7;
    auto emit = [&](uint64_t k, int rank) {
        if (k != 0ull && rank < W) {
            ids[(int64_t)r * W + rank] = (int32_t)key_id(k);
            logprob[(int64_t)r * W + rank] = key_value(k) - lse;
        }
    };
    if (nc <= kWave) {
        const uint64_t mine[1] = {lane < nc ? keys[lane] : 0ull};
        int cnt[1];
        count_greater<1>(keys, ne, mine, cnt);
        emit(mine[0], cnt[0]);
    } else {
        constexpr int K = kMergeCand / kWave;
        uint64_t mine[K];
#pragma unroll
        for (int q = 0; q < K; ++q)
            mine[q] = lane + kWave * q < nc ? keys[lane + kWave * q] : 0ull;
        int cnt[K];
        count_greater<K>(keys, ne, mine, cnt);
#pragma unroll
        for (int q = 0; q < K; ++q)
            emit(mine[q], cnt[q]);
    }
    if (lane == 0 && row_lse)
        row_lse[r] = lse;
}

__global__ void __launch_bounds__(64)
topw_merge_kernel(int rows, int W, int nchunk, const uint64_t *__restrict__ ws_keys,
                  const float2 *__restrict__ ws_ms, const float *__restrict__ ws_t,
                  int32_t *__restrict__ ids, float *__restrict__ logprob,
                  float *__restrict__ row_lse, float *__restrict__ row_entropy)
{
    __shared__ __attribute__((aligned(16))) uint64_t keys[kMergeLds];
    topw_merge_row(blockIdx.x, W, nchunk, ws_keys, ws_ms, ws_t, ids, logprob, row_lse,
                   row_entropy, keys);
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
    return parts * (size_t)W * sizeof(uint64_t) + parts * sizeof(float2) +
           parts * sizeof(float) + 512;
}

jt_status launch_topw(const void *logits, int64_t row_stride, int rows, int V, int W, int dtype,
                      int32_t *ids, float *logprob, float *row_lse, float *row_entropy, void *ws,
                      hipStream_t st)
{
    if (rows == 0)
        return JT_OK;
    const TopwPlan p = topw_plan(rows, V);
    const size_t parts = (size_t)rows * p.nlist;
    uint64_t *wk = reinterpret_cast<uint64_t *>(ws);
    uintptr_t mp = reinterpret_cast<uintptr_t>(wk + parts * W);
    mp = (mp + 15) & ~(uintptr_t)15;
    float2 *wm = reinterpret_cast<float2 *>(mp);
    uintptr_t tp = reinterpret_cast<uintptr_t>(wm + parts);
    tp = (tp + 15) & ~(uintptr_t)15;
    float *wt = row_entropy ? reinterpret_cast<float *>(tp) : nullptr;
    const dim3 grid((unsigned)((parts + 3) / 4)), block(kTopwThreads);
    const uintptr_t addr = reinterpret_cast<uintptr_t>(logits);
    const bool ent = wt != nullptr;
    auto go = [&](auto kern, const auto *x) {
        hipLaunchKernelGGL(kern, grid, block, 0, st, x, row_stride, rows, V, W, p.npiece, p.ppw,
                           p.nlist, wk, wm, wt);
    };
    if (dtype == JT_BF16) {
        const uint16_t *x = (const uint16_t *)logits;
        const bool al = (addr % 16 == 0) && (row_stride % 8 == 0);
        if (al)
            ent ? go(topw_partial_kernel<uint16_t, true, true>, x)
                : go(topw_partial_kernel<uint16_t, true, false>, x);
        else
            ent ? go(topw_partial_kernel<uint16_t, false, true>, x)
                : go(topw_partial_kernel<uint16_t, false, false>, x);
    } else {
        const float *x = (const float *)logits;
        const bool al = (addr % 16 == 0) && (row_stride % 4 == 0);
        if (al)
            ent ? go(topw_partial_kernel<float, true, true>, x)
                : go(topw_partial_kernel<float, true, false>, x);
        else
            ent ? go(topw_partial_kernel<float, false, true>, x)
                : go(topw_partial_kernel<float, false, false>, x);
    }
    jt_status e = launch_status(hipGetLastError());
    if (e != JT_OK)
        return e;
    hipLaunchKernelGGL(topw_merge_kernel, dim3(rows), dim3(64), 0, st, rows, W, p.nlist, wk, wm,
                       wt, ids, logprob, row_lse, row_entropy);
    return launch_status(hipGetLastError());
}

} // namespace jt
