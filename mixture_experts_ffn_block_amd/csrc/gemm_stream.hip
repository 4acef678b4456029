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
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kWavesPerWG = 4;
constexpr int kTilesPerWave = 4;                 // 16-column MFMA tiles per wave
constexpr int kColsPerWave = 16 * kTilesPerWave;  // 64
constexpr int kColsPerWG = kWavesPerWG * kColsPerWave;

template <bool GATHER>
__global__ __launch_bounds__(kWavesPerWG * 64) void stream_gemm_bf16_kernel(GemmArgs p) {
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
    if constexpr (GATHER) {
        const int r = p.sorted[m0 + row16];
        src_row = r < p.R ? r / p.topk : 0;  // padding rows read token 0
    }
    const uint8_t* a_ptr = reinterpret_cast<const uint8_t*>(p.A) + src_row * p.lda_bytes + kq * 16;
    const uint8_t* w_base = reinterpret_cast<const uint8_t*>(p.W) + static_cast<int64_t>(e) * p.w_expert_bytes;
    const uint8_t* w_ptr[kTilesPerWave];
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
        const int n = min(nw0 + 16 * t + row16, p.N - 1);
        w_ptr[t] = w_base + static_cast<int64_t>(n) * p.ldw_bytes + kq * 16;
    }

    f32x4_t acc[kTilesPerWave];
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) acc[t] = f32x4_t{};

    const int KC = p.K / 128;  // 128 bf16 = 256 bytes per row per chunk
    u32x4_t a_cur[4], w_cur[kTilesPerWave][4], a_nxt[4], w_nxt[kTilesPerWave][4];
    auto load = [&](int kc, u32x4_t (&a)[4], u32x4_t (&w)[kTilesPerWave][4]) {
        const int64_t off = static_cast<int64_t>(kc) * 256;
#pragma unroll
        for (int s = 0; s < 4; ++s) a[s] = *reinterpret_cast<const u32x4_t*>(a_ptr + off + 64 * s);
#pragma unroll
        for (int t = 0; t < kTilesPerWave; ++t)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                w[t][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(w_ptr[t] + off + 64 * s));
    };
    load(0, a_cur, w_cur);
    for (int kc = 0; kc < KC; ++kc) {
        if (kc + 1 < KC) load(kc + 1, a_nxt, w_nxt);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int t = 0; t < kTilesPerWave; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, w_cur[t][s]), __builtin_bit_cast(bf16x8_t, a_cur[s]),
                    acc[t], 0, 0, 0);
        if (kc + 1 < KC) {
#pragma unroll
            for (int s = 0; s < 4; ++s) a_cur[s] = a_nxt[s];
#pragma unroll
            for (int t = 0; t < kTilesPerWave; ++t)
#pragma unroll
                for (int s = 0; s < 4; ++s) w_cur[t][s] = w_nxt[t][s];
        }
    }

    // 16x16 accumulator: lane holds token row (lane & 15) and 4 consecutive
    // weight rows 4*(lane >> 4) + 0..3 of each column tile
    uint8_t* c_row = reinterpret_cast<uint8_t*>(p.C) + (m0 + row16) * p.ldc_bytes;
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
        const int n = nw0 + 16 * t + 4 * kq;
        if (n < p.N) {
            u32x2_t v{pack_bf16x2(acc[t][0], acc[t][1]), pack_bf16x2(acc[t][2], acc[t][3])};
            *reinterpret_cast<u32x2_t*>(c_row + n * 2) = v;
        }
    }
}

}  // namespace

hipError_t launch_stream_gemm(const GemmArgs& a, hipStream_t stream) {
    const int n_wg = (a.N + kColsPerWG - 1) / kColsPerWG;
    const dim3 grid(static_cast<unsigned>(a.m_blocks * n_wg));
    if (a.sorted)
        hipLaunchKernelGGL(stream_gemm_bf16_kernel<true>, grid, dim3(kWavesPerWG * 64), 0, stream, a);
    else
        hipLaunchKernelGGL(stream_gemm_bf16_kernel<false>, grid, dim3(kWavesPerWG * 64), 0, stream, a);
    return hipGetLastError();
}
