// gemm_stream.hip -- weight-streaming grouped GEMM for small expert blocks.
//
// Same operation as gemm.hip ("fused_moe.py analysis", 1.3 and
// "fused_moe_kernel": BLOCK_M routed rows of one expert times a column tile,
// A rows gathered through sorted_token_ids, fp32 accumulation, cast at the
// end), specialised for BLOCK_M = 16, where decode-sized batches leave most
// experts with only a few tokens and the time goes into reading each touched
// expert's weights once from HBM.
//
// gfx950 design: no LDS. A wavefront owns 16 token rows x 64 weight rows (four
// v_mfma_f32_16x16x32_bf16 column tiles). Per 128-wide K chunk (256 bytes of
// a row) every lane loads four 16-byte pieces of one weight row per column
// tile, and of one token row, straight into the MFMA operand registers: load
// s gives lane group k = lane / 16 the piece at 64*s + 16*k, so each load
// instruction reads 64 contiguous bytes of each of its 16 rows. Both
// operands assign the same K index to the same (lane, register) slot, so the
// MFMA's sum over K is exact regardless of the order the slots take. The next chunk is loaded
// while the current one is multiplied. The token rows (tiny) are re-read by
// every wave from L2; the weights stream from HBM once per expert block.
// GEMM1 with SiLU-and-mul in the epilogue: a wave owns the 16 gate rows and the
// 16 matching up rows of 16 output columns (512-byte chunks), so a lane holds
// gate and up of the same 4 outputs and writes z directly; h never reaches HBM.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kWavesPerWG = 4;

// TILES 16-row weight tiles per wave; per K chunk every row contributes S pieces of
// 64 contiguous bytes (32 S bf16). ACT (GEMM1 with SiLU-and-mul, TILES = 2): tile 0
// holds the 16 gate rows and tile 1 the 16 up rows of the wave's 16 output columns.
template <bool GATHER, bool ACT, int TILES, int S>
__global__ __launch_bounds__(kWavesPerWG * 64) void stream_gemm_bf16_kernel(GemmArgs p) {
    static_assert(!ACT || (GATHER && TILES == 2), "SiLU epilogue: GEMM1, one gate and one up tile");
    constexpr int kColsPerWave = ACT ? 16 : 16 * TILES;  // output columns
    constexpr int kColsPerWG = kWavesPerWG * kColsPerWave;
    const int n_wg = (p.N + kColsPerWG - 1) / kColsPerWG;
    const int mb = blockIdx.x / n_wg, nb = blockIdx.x % n_wg;
    const int npp = *p.npp;
    const int64_t m0 = static_cast<int64_t>(mb) * 16;
    if (m0 >= npp) return;
    const int e = p.expert_ids[mb];
    if (e < 0) return;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row16 = lane & 15, kq = lane >> 4;
    const int nw0 = nb * kColsPerWG + wave * kColsPerWave;
    if (nw0 >= p.N) return;

    int64_t src_row = m0 + row16;
    int r_item = 0;
    if constexpr (GATHER) {
        r_item = p.sorted[m0 + row16];
        src_row = r_item < p.R ? r_item / p.topk : 0;  // padding rows read token 0
    }
    const uint8_t* a_ptr = reinterpret_cast<const uint8_t*>(p.A) + src_row * p.lda_bytes + kq * 16;
    const uint8_t* w_base = reinterpret_cast<const uint8_t*>(p.W) + static_cast<int64_t>(e) * p.w_expert_bytes;
    const uint8_t* w_ptr[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
        // ACT: gate row n (t = 0) or up row N + n (t = 1) of output column n
        const int n = ACT ? t * p.N + min(nw0 + row16, p.N - 1) : min(nw0 + 16 * t + row16, p.N - 1);
        w_ptr[t] = w_base + static_cast<int64_t>(n) * p.ldw_bytes + kq * 16;
    }

    f32x4_t acc[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) acc[t] = f32x4_t{};

    const int KC = p.K / (32 * S);
    u32x4_t a_cur[S], w_cur[TILES][S], a_nxt[S], w_nxt[TILES][S];
    auto load = [&](int kc, u32x4_t (&a)[S], u32x4_t (&w)[TILES][S]) {
        const int64_t off = static_cast<int64_t>(kc) * 64 * S;
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
            for (int s = 0; s < S; ++s)
                w[t][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(w_ptr[t] + off + 64 * s));
#pragma unroll
        for (int s = 0; s < S; ++s) a[s] = *reinterpret_cast<const u32x4_t*>(a_ptr + off + 64 * s);
    };
    load(0, a_cur, w_cur);
    for (int kc = 0; kc < KC; ++kc) {
        if (kc + 1 < KC) load(kc + 1, a_nxt, w_nxt);
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int t = 0; t < TILES; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, w_cur[t][s]), __builtin_bit_cast(bf16x8_t, a_cur[s]),
                    acc[t], 0, 0, 0);
        if (kc + 1 < KC) {
#pragma unroll
            for (int s = 0; s < S; ++s) a_cur[s] = a_nxt[s];
#pragma unroll
            for (int t = 0; t < TILES; ++t)
#pragma unroll
                for (int s = 0; s < S; ++s) w_cur[t][s] = w_nxt[t][s];
        }
    }

    // 16x16 accumulator: lane holds token row (lane & 15) and 4 consecutive
    // weight rows 4*(lane >> 4) + 0..3 of each column tile
    uint8_t* c_row = reinterpret_cast<uint8_t*>(p.C) + (m0 + row16) * p.ldc_bytes;
    if constexpr (ACT) {
        // gate and up rounded to bf16 (the values GEMM1 would store), then
        // z = alpha * SiLU(g) * u in fp32 (alpha: the item's weight in on-input
        // mode, else 1; padding rows 0)
        const int n = nw0 + 4 * kq;
        if (n < p.N) {
            const bool real = r_item < p.R;
            const float alpha = (real && p.act_on_input) ? p.act_weights[r_item] : 1.0f;
            float zv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float g = bf16_to_f32(f32_to_bf16(acc[0][i]));
                const float u = bf16_to_f32(f32_to_bf16(acc[1][i]));
                zv[i] = real ? alpha * silu_f32(g) * u : 0.0f;
            }
            *reinterpret_cast<u32x2_t*>(c_row + n * 2) = u32x2_t{pack_bf16x2(zv[0], zv[1]), pack_bf16x2(zv[2], zv[3])};
        }
    } else {
#pragma unroll
        for (int t = 0; t < TILES; ++t) {
            const int n = nw0 + 16 * t + 4 * kq;
            if (n < p.N) {
                u32x2_t v{pack_bf16x2(acc[t][0], acc[t][1]), pack_bf16x2(acc[t][2], acc[t][3])};
                *reinterpret_cast<u32x2_t*>(c_row + n * 2) = v;
            }
        }
    }
}

template <bool GATHER, bool ACT, int TILES, int S>
hipError_t launch_stream_as(const GemmArgs& a, hipStream_t stream) {
    constexpr int kColsPerWG = kWavesPerWG * (ACT ? 16 : 16 * TILES);
    const int n_wg = (a.N + kColsPerWG - 1) / kColsPerWG;
    const dim3 grid(static_cast<unsigned>(a.m_blocks * n_wg));
    hipLaunchKernelGGL((stream_gemm_bf16_kernel<GATHER, ACT, TILES, S>), grid, dim3(kWavesPerWG * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

// K is a multiple of 128 (checked on the host): 4 pieces of 64 bytes per row always
// divide it; the SiLU variant takes 512-byte chunks where K allows
hipError_t launch_stream_gemm(const GemmArgs& a, hipStream_t stream) {
    if (a.act) {
        if (!a.sorted) return hipErrorInvalidValue;
        return (a.K / 32) % 8 == 0 ? launch_stream_as<true, true, 2, 8>(a, stream)
                                   : launch_stream_as<true, true, 2, 4>(a, stream);
    }
    return a.sorted ? launch_stream_as<true, false, 4, 4>(a, stream) : launch_stream_as<false, false, 4, 4>(a, stream);
}
