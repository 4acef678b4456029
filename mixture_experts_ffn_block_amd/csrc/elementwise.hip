// elementwise.hip -- SiLU-and-mul (+ fp8 group quant), activation quant,
// and the top-k weighted unpermute-reduce.
//
// * SiLU-and-mul: "fused_moe.py analysis", apply_moe_activation /
//   _silu_and_mul_kernel; "DeepGEMM FusedMoE on Blackwell", 2.6.4 (SwiGLU and
//   the dynamic per-128 quantisation in one pass): z = SiLU(gate) * up over
//   the first and second halves of each GEMM1 row.
// * Dynamic quantisation: "DeepGEMM FusedMoE on Blackwell", 2.5
//   (per_token_group_quant_fp8, fp32 scale per 128 columns of a row).
// * Reduce: "DeepGEMM FusedMoE on Blackwell", 2.6.5 (ep_gather: per token,
//   the k expert rows are fetched through inv_perm and summed with their
//   weights in fp32, then cast to bf16); "vLLM modular_kernel.py notes" 7.3.3
//   (multiply by topk_weights, then sum over the top-k dimension).
//
// * Weight packing: "DeepGEMM FusedMoE on Blackwell", 2.8 (c) (weights are
//   rewritten once after loading into the layout the kernel reads).
//
// All are HBM-bound; every thread moves 16-byte vectors.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

// ---------------------------------------------------------------- bf16 act --
// One thread per 8 output elements of a row, the rows strided over the grid's
// y dimension (at most 65535 of them). Rows >= num_tokens_post_padded are not
// touched; padding rows (sentinel item) are written as zeros.
__global__ __launch_bounds__(256) void silu_mul_bf16_kernel(
    const bf16_t* __restrict__ h, bf16_t* __restrict__ z, const int32_t* __restrict__ sorted,
    const float* __restrict__ weights, int R, int I, const int32_t* __restrict__ npp_ptr,
    int on_input) {
    const int i0 = (blockIdx.x * 256 + threadIdx.x) * 8;
    if (i0 >= I) return;
    const int64_t npp = *npp_ptr;
    for (int64_t pos = blockIdx.y; pos < npp; pos += gridDim.y) {
        const int r = sorted[pos];
        u32x4_t out{0, 0, 0, 0};
        if (r < R) {
            const float alpha = on_input ? weights[r] : 1.0f;
            const u32x4_t g = *reinterpret_cast<const u32x4_t*>(h + pos * 2 * I + i0);
            const u32x4_t u = *reinterpret_cast<const u32x4_t*>(h + pos * 2 * I + I + i0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float g0 = __uint_as_float(g[j] << 16), g1 = __uint_as_float(g[j] & 0xffff0000u);
                const float u0 = __uint_as_float(u[j] << 16), u1 = __uint_as_float(u[j] & 0xffff0000u);
                out[j] = pack_bf16x2(alpha * silu_f32(g0) * u0, alpha * silu_f32(g1) * u1);
            }
        }
        *reinterpret_cast<u32x4_t*>(z + pos * I + i0) = out;
    }
}

// ------------------------------------------------------ fp8 group quantiser --
// Quantises 8 fp32 values per lane; the 16 lanes of a quarter-wave form one
// 128-value group. Returns 8 e4m3 codes packed into 2 words and writes the
// group scale from the group's first lane. EXACT: code = RNE(v / s) with the
// correctly rounded quotient (the activation quantiser, whose codes match the
// reference bit for bit); otherwise v times the rounded 1 / s (one division per
// group instead of per value; groups with s below the smallest normal float keep
// the quotient), the form the GEMM1 epilogue uses for z, so that the separate
// pass and the fused epilogue agree bit for bit.
template <bool EXACT>
__device__ __forceinline__ u32x2_t quant_group8(const float (&v)[8], float* scale_out, bool writer) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    const float s = amax / 448.0f;
    if (writer) *scale_out = s;
    float q[8];
    if (EXACT || !(s >= 0x1p-126f)) {  // also groups so small that 1 / s would overflow
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = amax == 0.0f ? 0.0f : fminf(fmaxf(v[j] / s, -448.0f), 448.0f);
    } else {
        const float inv = 1.0f / s;
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = fminf(fmaxf(v[j] * inv, -448.0f), 448.0f);
    }
    return u32x2_t{cvt_e4m3x4(q[0], q[1], q[2], q[3]), cvt_e4m3x4(q[4], q[5], q[6], q[7])};
}

// SiLU-and-mul, then per-row per-128 fp8 quantisation of the fp32 result.
// One wavefront per (row, 4 groups), rows strided over the grid's y dimension.
// The scales are stored group-major,
// zs[g * cap + pos], so that the GEMM reads a block's 128 row scales of one
// group as one contiguous run.
__global__ __launch_bounds__(256) void silu_mul_fp8_kernel(
    const bf16_t* __restrict__ h, uint8_t* __restrict__ zq, float* __restrict__ zs,
    const int32_t* __restrict__ sorted, const float* __restrict__ weights, int R, int I,
    int64_t cap, const int32_t* __restrict__ npp_ptr, int on_input) {
    const int lane = threadIdx.x & 63;
    const int i0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 512 + lane * 8;
    if (i0 >= I) return;  // I is a multiple of 128: whole groups leave together
    const int64_t npp = *npp_ptr;
    for (int64_t pos = blockIdx.y; pos < npp; pos += gridDim.y) {
        const int r = sorted[pos];
        float v[8];
        if (r < R) {
            const float alpha = on_input ? weights[r] : 1.0f;
            const u32x4_t g = *reinterpret_cast<const u32x4_t*>(h + pos * 2 * I + i0);
            const u32x4_t u = *reinterpret_cast<const u32x4_t*>(h + pos * 2 * I + I + i0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[2 * j] = alpha * silu_f32(__uint_as_float(g[j] << 16)) * __uint_as_float(u[j] << 16);
                v[2 * j + 1] = alpha * silu_f32(__uint_as_float(g[j] & 0xffff0000u)) *
                               __uint_as_float(u[j] & 0xffff0000u);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = 0.0f;
        }
        const u32x2_t q = quant_group8<false>(v, zs + (i0 / 128) * cap + pos, (lane & 15) == 0);
        *reinterpret_cast<u32x2_t*>(zq + pos * I + i0) = q;
    }
}

// Per-row, per-128-column quantisation of a bf16 matrix [rows, cols]; rows strided
// over the grid's y dimension.
__global__ __launch_bounds__(256) void quant_fp8_kernel(const bf16_t* __restrict__ x,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ scale, int cols,
                                                        int64_t rows) {
    const int lane = threadIdx.x & 63;
    const int c0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 512 + lane * 8;
    if (c0 >= cols) return;  // cols is a multiple of 128: whole groups leave together
    for (int64_t row = blockIdx.y; row < rows; row += gridDim.y) {
        const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(x + row * cols + c0);
        float v[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(xv[j] << 16);
            v[2 * j + 1] = __uint_as_float(xv[j] & 0xffff0000u);
        }
        const u32x2_t qq = quant_group8<true>(v, scale + row * (cols / 128) + c0 / 128, (lane & 15) == 0);
        *reinterpret_cast<u32x2_t*>(q + row * cols + c0) = qq;
    }
}

// MXFP8 activations ("DeepGEMM FusedMoE on Blackwell", MXFP8 1x32): each 32
// columns of a row share one E8M0 scale, the smallest power of two s with
// amax <= 448 s; codes E4M3(v / s). Four lanes hold a block (8 values each).
__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const bf16_t* __restrict__ x,
                                                          uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ scale, int cols,
                                                          int64_t rows) {
    const int lane = threadIdx.x & 63;
    const int c0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 512 + lane * 8;
    if (c0 >= cols) return;  // cols is a multiple of 128: whole blocks only
    for (int64_t row = blockIdx.y; row < rows; row += gridDim.y) {
        const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(x + row * cols + c0);
        float v[8], m = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(xv[j] << 16);
            v[2 * j + 1] = __uint_as_float(xv[j] & 0xffff0000u);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        const uint32_t code = mx_scale_code(m, 448.0f);
        const float inv = ldexpf(1.0f, 127 - static_cast<int>(code));
        float c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = fminf(fmaxf(v[j] * inv, -448.0f), 448.0f);
        *reinterpret_cast<u32x2_t*>(q + row * cols + c0) =
            u32x2_t{cvt_e4m3x4(c[0], c[1], c[2], c[3]), cvt_e4m3x4(c[4], c[5], c[6], c[7])};
        if ((lane & 3) == 0) scale[row * (cols / 32) + c0 / 32] = static_cast<uint8_t>(code);
    }
}

// MX weight scales into the kernels' order: natural [E, N, K/32] bytes ->
// [E, K/128, N] words, byte b of word (e, j, n) holding block 4 j + b of row n.
__global__ __launch_bounds__(256) void pack_mx_scales_kernel(const uint32_t* __restrict__ s,
                                                             uint32_t* __restrict__ out, int64_t words,
                                                             int N, int KW) {
    for (int64_t d = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; d < words;
         d += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t n = d % N, j = (d / N) % KW, e = d / (static_cast<int64_t>(N) * KW);
        out[d] = s[(e * N + n) * KW + j];
    }
}

// Activation scales of GEMM1 in its row order: out[g * cap + pos] is the
// scale of the token of sorted position pos (0 for padding positions), from
// the per-token scales scale[token, g]. Positions >= npp are not written.
// One thread per position; consecutive threads write consecutive floats.
__global__ __launch_bounds__(256) void permute_scales_kernel(const float* __restrict__ scale,
                                                             int groups, int topk, int R,
                                                             const int32_t* __restrict__ sorted,
                                                             const int32_t* __restrict__ npp_ptr,
                                                             int64_t cap, float* __restrict__ out) {
    const int64_t pos = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (pos >= *npp_ptr) return;
    const int r = sorted[pos];
    const float* src = r < R ? scale + static_cast<int64_t>(r / topk) * groups : nullptr;
    for (int g = 0; g < groups; ++g) out[g * cap + pos] = src ? src[g] : 0.0f;
}

// ------------------------------------------------------------------ reduce --
// y[t, n] = bf16( sum_j alpha_j * o[inv_perm[t, j], n] ), fp32, slot order.
template <int KMAX>
__global__ __launch_bounds__(256) void reduce_kernel(const bf16_t* __restrict__ o,
                                                     const int32_t* __restrict__ inv_perm,
                                                     const float* __restrict__ weights, int k,
                                                     int H, int use_weights,
                                                     bf16_t* __restrict__ y, int64_t M) {
    const int n0 = (blockIdx.x * 256 + threadIdx.x) * 8;
    if (n0 >= H) return;
    for (int64_t t = blockIdx.y; t < M; t += gridDim.y) {
        // all the token's positions and weights, then all its output rows, are loaded
        // before the first use: two memory latencies per token instead of two per slot
        int pos[KMAX];
        float a[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            pos[j] = j < k ? inv_perm[t * k + j] : -1;
            a[j] = (j < k && use_weights) ? weights[t * k + j] : 1.0f;
        }
        u32x4_t v[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            v[j] = pos[j] >= 0 ? *reinterpret_cast<const u32x4_t*>(o + static_cast<int64_t>(pos[j]) * H + n0)
                               : u32x4_t{0, 0, 0, 0};
        // fp32 sum in slot order; slots of experts held elsewhere (-1) are skipped
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (pos[j] < 0) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] += a[j] * __uint_as_float(v[j][i] << 16);
                acc[2 * i + 1] += a[j] * __uint_as_float(v[j][i] & 0xffff0000u);
            }
        }
        u32x4_t out;
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
        *reinterpret_cast<u32x4_t*>(y + t * H + n0) = out;
    }
}

// ------------------------------------------------------------- weight pack --
// One thread per 16-byte piece of the tiled tensor (coalesced writes): piece q of
// tile (e, tile, kf) holds row 16 tile + q / 4, columns 32 kf + 8 (q % 4) .. + 7 of
// expert e.
__global__ __launch_bounds__(256) void pack_tiled_kernel(const uint4* __restrict__ w,
                                                          uint4* __restrict__ wp, int64_t pieces,
                                                          int N, int K) {
    const int64_t kfs = K / 32, tiles = N / 16;
    for (int64_t d = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; d < pieces;
         d += static_cast<int64_t>(gridDim.x) * 256) {
        const int q = static_cast<int>(d & 63);
        const int64_t f = d >> 6;
        const int64_t kf = f % kfs, tile = (f / kfs) % tiles, e = f / (kfs * tiles);
        const int64_t n = tile * 16 + (q >> 2), k = kf * 32 + 8 * (q & 3);
        wp[d] = w[((e * N + n) * K + k) / 8];
    }
}

}  // namespace

hipError_t launch_pack_tiled(const bf16_t* w, bf16_t* wp, int64_t E, int N, int K, hipStream_t stream) {
    const int64_t pieces = E * N * K / 8;
    const int64_t blocks = ceil_div(pieces, 256);
    const dim3 grid(static_cast<unsigned>(blocks < 65536 ? blocks : 65536));
    hipLaunchKernelGGL(pack_tiled_kernel, grid, dim3(256), 0, stream,
                       reinterpret_cast<const uint4*>(w), reinterpret_cast<uint4*>(wp), pieces, N, K);
    return hipGetLastError();
}

// rows go along the grid's y dimension, at most kMaxGridY of them; the kernels
// stride over the rest
constexpr int64_t kMaxGridY = 65535;
unsigned grid_rows(int64_t rows) { return static_cast<unsigned>(rows < kMaxGridY ? (rows > 0 ? rows : 1) : kMaxGridY); }

hipError_t launch_silu_mul_bf16(const bf16_t* h, bf16_t* z, const int32_t* sorted,
                                const float* weights, int R, int I, int64_t cap,
                                const int32_t* npp, int on_input, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(ceil_div(I / 8, 256)), grid_rows(cap));
    hipLaunchKernelGGL(silu_mul_bf16_kernel, grid, dim3(256), 0, stream, h, z, sorted, weights, R,
                       I, npp, on_input);
    return hipGetLastError();
}

hipError_t launch_silu_mul_fp8(const bf16_t* h, uint8_t* zq, float* zs, const int32_t* sorted,
                               const float* weights, int R, int I, int64_t cap,
                               const int32_t* npp, int on_input, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(ceil_div(I, 2048)), grid_rows(cap));
    hipLaunchKernelGGL(silu_mul_fp8_kernel, grid, dim3(256), 0, stream, h, zq, zs, sorted,
                       weights, R, I, cap, npp, on_input);
    return hipGetLastError();
}

hipError_t launch_permute_scales(const float* scale, int groups, int topk, int R,
                                 const int32_t* sorted, const int32_t* npp, int64_t cap,
                                 float* out, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(ceil_div(cap, 256)));
    hipLaunchKernelGGL(permute_scales_kernel, grid, dim3(256), 0, stream, scale, groups, topk, R,
                       sorted, npp, cap, out);
    return hipGetLastError();
}

hipError_t launch_quant_fp8(const bf16_t* x, int64_t rows, int cols, uint8_t* q, float* scale,
                            hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(ceil_div(cols, 2048)), grid_rows(rows));
    hipLaunchKernelGGL(quant_fp8_kernel, grid, dim3(256), 0, stream, x, q, scale, cols, rows);
    return hipGetLastError();
}

hipError_t launch_quant_mxfp8(const bf16_t* x, int64_t rows, int cols, uint8_t* q, uint8_t* scale,
                              hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(ceil_div(cols, 2048)), grid_rows(rows));
    hipLaunchKernelGGL(quant_mxfp8_kernel, grid, dim3(256), 0, stream, x, q, scale, cols, rows);
    return hipGetLastError();
}

hipError_t launch_pack_mx_scales(const uint8_t* s, uint32_t* out, int64_t E, int N, int K, hipStream_t stream) {
    const int64_t words = E * N * (K / 128);
    const int64_t blocks = ceil_div(words, 256);
    const dim3 grid(static_cast<unsigned>(blocks < 65536 ? blocks : 65536));
    hipLaunchKernelGGL(pack_mx_scales_kernel, grid, dim3(256), 0, stream, reinterpret_cast<const uint32_t*>(s),
                       out, words, N, K / 128);
    return hipGetLastError();
}

hipError_t launch_reduce(const bf16_t* o, const int32_t* inv_perm, const float* weights, int64_t M,
                         int k, int H, int use_weights, bf16_t* y, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(ceil_div(H / 8, 256)), grid_rows(M));
    // slots per token rounded up to a power of two (k <= 32)
    auto go = [&](auto kmax) {
        hipLaunchKernelGGL(reduce_kernel<decltype(kmax)::value>, grid, dim3(256), 0, stream, o, inv_perm,
                           weights, k, H, use_weights, y, M);
    };
    if (k <= 1) go(std::integral_constant<int, 1>{});
    else if (k <= 2) go(std::integral_constant<int, 2>{});
    else if (k <= 4) go(std::integral_constant<int, 4>{});
    else if (k <= 8) go(std::integral_constant<int, 8>{});
    else if (k <= 16) go(std::integral_constant<int, 16>{});
    else go(std::integral_constant<int, 32>{});
    return hipGetLastError();
}
