// Internal helpers shared by the libjt kernels (gfx950, wave64).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/jt.h"

namespace jt {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16, round to nearest even (NaN stays NaN): the hardware conversion
// (v_cvt_pk_bf16_f32).  A bit-twiddling version compiled to a branch per value around the
// NaN test, about 20 instructions each -- 3 us per workgroup in the attention epilogue.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// two floats -> packed bf16 pair (lo in bits 0..15), one conversion instruction
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Monotone map of a float to uint32 for "value descending" comparisons.
// -0 and +0 map to the same code; NaN maps to 0, below -inf (0x007fffff).
__device__ __forceinline__ uint32_t order_code(float x)
{
    uint32_t u = __float_as_uint(x);
    if (x != x)
        return 0u;
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_decode(uint32_t c)
{
    if (c == 0u)
        return __uint_as_float(0x7fc00000u);
    return __uint_as_float((c & 0x80000000u) ? (c & 0x7fffffffu) : ~c);
}
// 64-bit ranking key: larger key = larger value, then lower id.  Key 0 = "no element".
__device__ __forceinline__ uint64_t rank_key(float x, uint32_t id)
{
    return ((uint64_t)order_code(x) << 32) | (uint64_t)(~id);
}
__device__ __forceinline__ uint32_t key_id(uint64_t k) { return ~(uint32_t)k; }
__device__ __forceinline__ float key_value(uint64_t k) { return order_decode((uint32_t)(k >> 32)); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m)
{
    uint32_t lo = __shfl_xor((uint32_t)v, m, kWave);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, kWave);
    return ((uint64_t)hi << 32) | lo;
}
// Wave-wide maximum of a 64-bit key through DPP moves (no LDS round trips): pairs,
// quads, half rows, rows, then the row broadcasts; lane 63 ends with the maximum, which
// is returned to every lane.
// One 64-bit compare and two selects: a short-circuit form of the compare compiles to
// exec-mask branches, several times slower.
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v, uint32_t ohi, uint32_t olo)
{
    const uint64_t o = ((uint64_t)ohi << 32) | olo;
    return o > v ? o : v;
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_u64_stage(uint64_t v)
{
    const int hi = (int)(v >> 32), lo = (int)(uint32_t)v;
    const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xF, false);
    const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xF, false);
    return dpp_max_step(v, ohi, olo);
}
__device__ __forceinline__ uint64_t wave_max_u64_dpp(uint64_t v)
{
    v = dpp_max_u64_stage<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_max_u64_stage<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = dpp_max_u64_stage<0x141, 0xF>(v);  // row_half_mirror
    v = dpp_max_u64_stage<0x140, 0xF>(v);  // row_mirror
    v = dpp_max_u64_stage<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_max_u64_stage<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), 63);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) { return wave_max_u64_dpp(v); }

// Float wave reductions through the same DPP pattern (no LDS round trips, which a
// shuffle butterfly pays at every step).  Lanes of rows a broadcast stage leaves out keep
// `old`: the value itself for the maximum, 0 for the sum, so every element is counted
// once.  The sum's order is fixed: pairs, quads, half rows, rows, then rows 0+1 and 2+3,
// then both halves.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float v, float old)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                 __builtin_bit_cast(int, v), CTRL,
                                                                 ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_max_f32(float v)
{
    v = fmaxf(v, dpp_f32<0xB1, 0xF>(v, v));
    v = fmaxf(v, dpp_f32<0x4E, 0xF>(v, v));
    v = fmaxf(v, dpp_f32<0x141, 0xF>(v, v));
    v = fmaxf(v, dpp_f32<0x140, 0xF>(v, v));
    v = fmaxf(v, dpp_f32<0x142, 0xA>(v, v));
    v = fmaxf(v, dpp_f32<0x143, 0xC>(v, v));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_sum_f32(float v)
{
    v += dpp_f32<0xB1, 0xF>(v, 0.f);
    v += dpp_f32<0x4E, 0xF>(v, 0.f);
    v += dpp_f32<0x141, 0xF>(v, 0.f);
    v += dpp_f32<0x140, 0xF>(v, 0.f);
    v += dpp_f32<0x142, 0xA>(v, 0.f);
    v += dpp_f32<0x143, 0xC>(v, 0.f);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Inclusive prefix sum over the wave in lane order, through DPP moves that read 0 where
// they have no source lane: each lane first adds its three predecessors in its 16-lane row
// (a 4-lane window), then the window 4 lanes back (lanes 4-15 of each row) and the sum 8
// lanes back (lanes 8-15), which completes every row; then lane 15's total goes into rows
// 1 and 3 and lane 31's into rows 2 and 3.
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ float dpp_f32_or0(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, ROW_MASK, BANK_MASK,
                                                                 true));
}
__device__ __forceinline__ float wave_incl_scan_f32(float v)
{
    float s = v + dpp_f32_or0<0x111, 0xF, 0xF>(v);  // row_shr:1
    s += dpp_f32_or0<0x112, 0xF, 0xF>(v);           // row_shr:2
    s += dpp_f32_or0<0x113, 0xF, 0xF>(v);           // row_shr:3
    s += dpp_f32_or0<0x114, 0xF, 0xE>(s);           // row_shr:4
    s += dpp_f32_or0<0x118, 0xF, 0xC>(s);           // row_shr:8
    s += dpp_f32_or0<0x142, 0xA, 0xF>(s);           // row_bcast:15
    s += dpp_f32_or0<0x143, 0xC, 0xF>(s);           // row_bcast:31
    return s;
}

inline jt_status launch_status(hipError_t e) { return e == hipSuccess ? JT_OK : JT_ERR_LAUNCH; }

// ---- launchers (each .hip file implements its own) ----
jt_status launch_build_mask(const int32_t *parent, int S, int B, uint64_t *anc, int32_t *depth,
                            int32_t *err, hipStream_t st);

size_t topw_workspace(int rows, int V, int W, int dtype);
jt_status launch_topw(const void *logits, int64_t row_stride, int rows, int V, int W, int dtype,
                      int32_t *ids, float *logprob, float *row_lse, float *row_entropy, void *ws,
                      hipStream_t st);

size_t verify_workspace(int S, int B, int V, int dtype);
jt_status launch_verify(const void *logits, int64_t row_stride, int V, int dtype,
                        const int32_t *parent, const int32_t *tokens, const uint64_t *anc,
                        const int32_t *depth, int S, int B, int N, int32_t *accept_len,
                        int32_t *accept_path, int32_t *bonus, int32_t *argmax_out,
                        int32_t *err, void *ws, hipStream_t st);

struct AttnArgs {
    const void *q, *k_tree, *v_tree, *k_prefix, *v_prefix;
    const int32_t *block_table;
    int max_blocks, block_size, block_shift, num_blocks;
    const int32_t *prefix_len;
    int max_prefix;
    const uint64_t *anc;
    const int32_t *parent;  // used instead of anc by the fused step (rows built in place)
    int S, B, Hq, Hkv, d, G;
    int dtype;
    float scale;
    void *out;
    float *lse;
    int32_t *err;
};
size_t attention_workspace(int S, int B, int Hq, int Hkv, int d, int max_prefix, int block_size,
                           int dtype);
jt_status launch_attention(const AttnArgs &a, void *ws, hipStream_t st);

// the fused step: attention arguments (anc and err unused) plus those of the other steps
struct StepLaunch {
    AttnArgs attn;
    const void *draft, *target;
    int64_t draft_stride, target_stride;
    int V, W, N;
    int32_t *ids;
    float *logprob, *row_lse, *row_entropy;
    const int32_t *parent, *tokens;
    uint64_t *anc;
    int32_t *depth;
    int32_t *accept_len, *accept_path, *bonus, *argmax_out, *err;
};
// the walk of verify.hip over per-row arg-max keys (nchunk keys per row)
jt_status launch_verify_walk(const int32_t *parent, const int32_t *tokens, const uint64_t *anc,
                             const int32_t *depth, int S, int B, int N, int nchunk,
                             const uint64_t *keys, const uint32_t *nan, int32_t *accept_len,
                             int32_t *accept_path, int32_t *bonus, int32_t *argmax_out,
                             int32_t *err, hipStream_t st);

size_t sample_workspace(int S, int B, int V);
jt_status launch_verify_sampled(const void *logits, int64_t row_stride, int V, int dtype,
                                float temperature, const float *uniform, const int32_t *parent,
                                const int32_t *tokens, const uint64_t *anc, const int32_t *depth,
                                int S, int B, int N, int32_t *accept_len, int32_t *accept_path,
                                int32_t *bonus, int32_t *sample_out, int32_t *err, void *ws,
                                hipStream_t st);

jt_status launch_build_tree(const int32_t *ids, const float *logprob, const float *entropy,
                            float w_lp, float w_ent, const int32_t *root_token, int S, int N,
                            int W, int B, int32_t *parent, int32_t *tokens, float *score,
                            int32_t *n_nodes, hipStream_t st);

jt_status launch_commit_kv(const int32_t *accept_len, const int32_t *accept_path, int N,
                           const void *k_tree, const void *v_tree, int S, int B, int Hkv, int d,
                           int elem_bytes, void *k_cache, void *v_cache,
                           const int32_t *block_table, int max_blocks, int block_size,
                           int num_blocks, const int32_t *prefix_len, int max_prefix,
                           int32_t *new_prefix_len, int32_t *err, hipStream_t st);

size_t step_workspace(int S, int B, int N, int W, int V, int Hq, int Hkv, int d, int max_prefix,
                      int block_size, int dtype);
jt_status launch_step(const StepLaunch &in, void *ws, hipStream_t st);

// jt_draft_verify_step_noalloc: the step's scratch lives in a static device array of
// this size (each GPU the call runs on holds one until the process ends)
constexpr size_t kStaticScratchBytes = (size_t)48 << 20;
jt_status launch_step_static(const StepLaunch &in, hipStream_t st);

jt_status launch_mfma_rate(int iters, int blocks, float *out, hipStream_t st);

} // namespace jt
