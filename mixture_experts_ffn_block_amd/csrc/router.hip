// router.hip -- softmax + top-k router, one wavefront per token.
//
// "vLLM modular_kernel.py notes", section 3 (fused_topk, scoring "softmax"):
// p = softmax(logits) over all E experts, the k largest are kept, and with
// renormalisation their weights are divided by their sum.
//
// gfx950 design: a 64-lane wavefront owns one token. Lane l holds experts
// l, l+64, l+128, l+192 in registers (E <= 256). Each of the k selection
// rounds is a lane-local argmax followed by a 6-step butterfly over the wave;
// no LDS, no atomics. Selection compares the fp32 logits themselves (softmax
// is strictly increasing), so the chosen ids do not depend on exp rounding;
// equal logits go to the lower expert index. With renormalisation the full
// softmax denominator cancels, so only the k chosen exponentials are summed.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kTokensPerBlock = 4;

__device__ __forceinline__ bool better(float v, int e, float bv, int be) {
    return v > bv || (v == bv && e < be);
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
        v[i] = e < E ? row[e] : -INFINITY;
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
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o, 64);
            const int oe = __shfl_xor(be, o, 64);
            if (better(ov, oe, bv, be)) { bv = ov; be = oe; }
        }
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

}  // namespace

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
