// router.hip -- softmax + top-k router, one wavefront per token.
//
// "vLLM modular_kernel.py notes", section 3 (fused_topk, scoring "softmax"):
// p = softmax(logits) over all E experts, the k largest are kept, and with
// renormalisation their weights are divided by their sum.
//
// gfx950 design: a 64-lane wavefront owns one token. Lane l holds experts
// l, l+64, l+128, l+192 in registers (E <= 256). Each of the k selection
// rounds is a lane-local argmax followed by two wave-wide reductions over DPP
// lane moves (the largest logit, then the lowest id among the lanes holding
// it); no LDS, no atomics. Selection compares the fp32 logits themselves (softmax
// is strictly increasing), so the chosen ids do not depend on exp rounding;
// equal logits go to the lower expert index. With renormalisation the full
// softmax denominator cancels, so only the k chosen exponentials are summed.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int kTokensPerBlock = 4;

__device__ __forceinline__ bool better(float v, int e, float bv, int be) {
    return v > bv || (v == bv && e < be);
}

// Wave-wide maximum (MAX) or minimum of a uint32, in every lane: row shifts by 1,
// 2, 4 and 8 leave each 16-lane row's result in its lane 15, two row broadcasts
// carry it to lane 63, which is read out. DPP moves between lanes run on the
// vector ALU, without the LDS crossbar that a shuffle takes.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x) {
    constexpr uint32_t id = MAX ? 0u : 0xffffffffu;
    auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
    x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x111, 0xf, 0xf, false));  // row_shr:1
    x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x112, 0xf, 0xf, false));  // row_shr:2
    x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x114, 0xf, 0xf, false));  // row_shr:4
    x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x118, 0xf, 0xf, false));  // row_shr:8
    x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x142, 0xa, 0xf, false));  // row_bcast:15
    x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return __builtin_amdgcn_readlane(x, 63);
}

// uint32 with the order of the float (not NaN); -0 and +0 give the same key
__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t b = __float_as_uint(v);
    if ((b & 0x7fffffffu) == 0) b = 0;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Wave-wide (largest, second largest) of the lanes' (m1 >= m2) pairs, counting
// equal values separately, in every lane: the same DPP steps as above, each
// merging two disjoint sets of lanes (identity: -inf, -inf).
__device__ __forceinline__ void wave_top2(float& m1, float& m2) {
    constexpr int ninf = static_cast<int>(0xff800000u);
    auto step = [&](auto ctrl, auto row_mask) {
        constexpr int C = decltype(ctrl)::value, RM = decltype(row_mask)::value;
        const float o1 = __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(m1), C, RM, 0xf, false));
        const float o2 = __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(m2), C, RM, 0xf, false));
        const float hi = fmaxf(m1, o1), lo = fminf(m1, o1);
        m2 = fmaxf(lo, fmaxf(m2, o2));
        m1 = hi;
    };
    step(std::integral_constant<int, 0x111>{}, std::integral_constant<int, 0xf>{});  // row_shr:1
    step(std::integral_constant<int, 0x112>{}, std::integral_constant<int, 0xf>{});  // row_shr:2
    step(std::integral_constant<int, 0x114>{}, std::integral_constant<int, 0xf>{});  // row_shr:4
    step(std::integral_constant<int, 0x118>{}, std::integral_constant<int, 0xf>{});  // row_shr:8
    step(std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xa>{});  // row_bcast:15
    step(std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xc>{});  // row_bcast:31
    m1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m1), 63));
    m2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m2), 63));
}

// The wave's best (value, id) under `better`: the largest value, the lowest id
// among equal values. Every lane passes its own best candidate (id 0x7fffffff
// and -inf when it has none) and receives the winner.
__device__ __forceinline__ void wave_best(float bv, int be, float& v, int& e) {
    const uint32_t key = order_key(bv);
    const uint32_t kmax = wave_reduce_u32<true>(key);
    e = static_cast<int>(wave_reduce_u32<false>(key == kmax ? static_cast<uint32_t>(be) : 0xffffffffu));
    v = key_value(kmax);
}

// A NaN logit is read as -inf: it ranks below every number and its softmax
// term is 0, so every chosen id stays in [0, E) (without this a row of NaNs
// would beat nothing and leave the search's start value as the id).
__device__ __forceinline__ float load_logit(const float* row, int e) {
    const float v = row[e];
    return v != v ? -INFINITY : v;
}

template <int EPL>
__global__ __launch_bounds__(kTokensPerBlock * MOE_WAVE) void topk_softmax_kernel(
    const float* __restrict__ logits, int64_t M, int E, int k, int renormalize,
    int32_t* __restrict__ ids, float* __restrict__ weights) {
    const int lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokensPerBlock + (threadIdx.x >> 6);
    if (t >= M) return;
    const float* row = logits + t * E;

    float v[EPL];
    uint32_t alive = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? load_logit(row, e) : -INFINITY;
        if (e < E) alive |= 1u << i;
    }

    int my_id = 0;
    float my_logit = 0.0f;
    float top = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if ((alive >> i) & 1u) {
                const int e = lane + 64 * i;
                if (better(v[i], e, bv, be)) { bv = v[i]; be = e; }
            }
        wave_best(bv, be, bv, be);
        if ((be & 63) == lane) alive &= ~(1u << (be >> 6));
        if (j == 0) top = bv;
        if (lane == j) { my_id = be; my_logit = bv; }
    }

    const float ex = lane < k ? expf(my_logit - top) : 0.0f;
    float denom;
    if (renormalize) {
        denom = wave_sum(ex);
    } else {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane + 64 * i < E) s += expf(v[i] - top);
        denom = wave_sum(s);
    }
    if (lane < k) {
        ids[t * k + lane] = my_id;
        weights[t * k + lane] = ex / denom;
    }
}

// ------------------------------------------------------------ grouped router --
// "vLLM modular_kernel.py notes", section 3 (fused_topk, scoring softmax or
// sigmoid) and the grouped routing arguments of apply_monolithic
// (num_expert_group, topk_group, e_score_correction_bias,
// routed_scaling_factor). Keys: the logits (both scores increase with them),
// or with a correction bias the fp32 sum sigmoid + bias, the sigmoid evaluated
// in double and rounded to fp32 so that the kept experts do not depend on an
// exp approximation. A group of E / G consecutive experts scores its largest
// key, or with a bias the sum of its two largest; the topk_group best groups
// (lower index on ties) are kept, then the k largest keys among their experts.
// Weights are the unbiased scores, renormalised over the k chosen if asked,
// times routed_scaling_factor.
//
// Same wave layout as above; the score of group g ends in lane g (G <= 64),
// found by a wave-wide merge of (largest, second largest) pairs.
__device__ __forceinline__ float sigmoid_f32(float s) {
    return static_cast<float>(1.0 / (1.0 + exp(-static_cast<double>(s))));
}

template <int EPL>
__global__ __launch_bounds__(kTokensPerBlock * MOE_WAVE) void topk_grouped_kernel(
    const float* __restrict__ logits, int64_t M, int E, int k, int sigmoid, int renormalize, int G,
    int TG, const float* __restrict__ bias, float scale, int32_t* __restrict__ ids,
    float* __restrict__ weights) {
    const int lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokensPerBlock + (threadIdx.x >> 6);
    if (t >= M) return;
    const float* row = logits + t * E;
    const int gs = E / G;

    float v[EPL], key[EPL];
    uint32_t alive = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? load_logit(row, e) : -INFINITY;
        key[i] = v[i];
        if (e < E) {
            alive |= 1u << i;
            if (bias) key[i] = sigmoid_f32(v[i]) + bias[e];
        }
    }

    if (TG < G) {
        float gscore = -INFINITY;  // lane g: score of group g
        for (int g = 0; g < G; ++g) {
            float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (((alive >> i) & 1u) && (lane + 64 * i) / gs == g) {
                    if (key[i] > m1) { m2 = m1; m1 = key[i]; }
                    else if (key[i] > m2) m2 = key[i];
                }
            wave_top2(m1, m2);
            if (lane == g) gscore = bias ? m1 + m2 : m1;
        }
        uint64_t kept = 0;
        for (int r = 0; r < TG; ++r) {
            float bv = lane < G && !((kept >> lane) & 1ull) ? gscore : -INFINITY;
            int bg = lane < G && !((kept >> lane) & 1ull) ? lane : 0x7fffffff;
            wave_best(bv, bg, bv, bg);
            kept |= 1ull << bg;
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;  // e < E: its group index is below G <= 64
            if (e < E && !((kept >> (e / gs)) & 1ull)) alive &= ~(1u << i);
        }
    }

    int my_id = 0;
    float my_logit = 0.0f, top = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if ((alive >> i) & 1u) {
                const int e = lane + 64 * i;
                if (better(key[i], e, bv, be)) { bv = key[i]; be = e; }
            }
        wave_best(bv, be, bv, be);
        if ((be & 63) == lane) alive &= ~(1u << (be >> 6));
        // the chosen expert's logit, from the lane that holds it
        float lg = -INFINITY;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane + 64 * i == be) lg = v[i];
        lg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lg), be & 63));  // be is wave-uniform
        if (j == 0) top = lg;
        if (lane == j) { my_id = be; my_logit = lg; }
    }

    float u = 0.0f;
    if (sigmoid) {
        u = lane < k ? sigmoid_f32(my_logit) : 0.0f;
        if (renormalize) u /= wave_sum(u);
    } else if (renormalize) {
        // the chosen have the largest logits among the kept groups: top is their maximum
        u = lane < k ? expf(my_logit - top) : 0.0f;
        u /= wave_sum(u);
    } else {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < EPL; ++i) mx = fmaxf(mx, v[i]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane + 64 * i < E) sum += expf(v[i] - mx);
        u = lane < k ? expf(my_logit - mx) : 0.0f;
        u /= wave_sum(sum);
    }
    if (lane < k) {
        ids[t * k + lane] = my_id;
        weights[t * k + lane] = u * scale;
    }
}

}  // namespace

hipError_t launch_topk_grouped(const float* logits, int64_t M, int E, int k, int sigmoid,
                               int renormalize, int G, int TG, const float* bias, float scale,
                               int32_t* ids, float* weights, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(ceil_div(M, kTokensPerBlock)));
    const dim3 block(kTokensPerBlock * MOE_WAVE);
    if (E <= 64)
        hipLaunchKernelGGL(topk_grouped_kernel<1>, grid, block, 0, stream, logits, M, E, k, sigmoid,
                           renormalize, G, TG, bias, scale, ids, weights);
    else if (E <= 128)
        hipLaunchKernelGGL(topk_grouped_kernel<2>, grid, block, 0, stream, logits, M, E, k, sigmoid,
                           renormalize, G, TG, bias, scale, ids, weights);
    else
        hipLaunchKernelGGL(topk_grouped_kernel<4>, grid, block, 0, stream, logits, M, E, k, sigmoid,
                           renormalize, G, TG, bias, scale, ids, weights);
    return hipGetLastError();
}

hipError_t launch_topk_softmax(const float* logits, int64_t M, int E, int k, int renormalize,
                               int32_t* ids, float* weights, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(ceil_div(M, kTokensPerBlock)));
    const dim3 block(kTokensPerBlock * MOE_WAVE);
    if (E <= 64)
        hipLaunchKernelGGL(topk_softmax_kernel<1>, grid, block, 0, stream, logits, M, E, k,
                           renormalize, ids, weights);
    else if (E <= 128)
        hipLaunchKernelGGL(topk_softmax_kernel<2>, grid, block, 0, stream, logits, M, E, k,
                           renormalize, ids, weights);
    else
        hipLaunchKernelGGL(topk_softmax_kernel<4>, grid, block, 0, stream, logits, M, E, k,
                           renormalize, ids, weights);
    return hipGetLastError();
}
