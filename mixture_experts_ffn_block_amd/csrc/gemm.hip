// gemm.hip -- grouped expert GEMMs on MFMA (bf16 and fp8 block-scaled).
//
// "fused_moe.py analysis", 1.3 and "fused_moe_kernel": one program computes
// BLOCK_M routed rows of a single expert times BLOCK_N output columns,
// C[r, n] = sum_k A[t(r), k] * B[e(r), n, k], with the A rows gathered through
// sorted_token_ids (token = item / topk), an fp32 accumulator, and a cast to
// the output type at the end. Block-wise fp8 ("FP8 W8A8"): every K block's
// partial dot product is multiplied by the activation scale and the weight
// block scale. "DeepGEMM FusedMoE on Blackwell", 2.6.3 / 2.6.5: both GEMMs
// run over the contiguous expert-sorted layout.
//
// gfx950 design
//   * Operands are K-contiguous ("NT"): activation rows [*, K] and expert
//     weight rows w[e] [N, K]. Every tile row is 128 bytes of K (64 bf16 or
//     128 e4m3), staged in LDS with a 16-byte-chunk XOR swizzle
//     (chunk ^ (row & 7)) so the MFMA fragment reads of 8 consecutive rows
//     hit distinct banks.
//   * The MFMA A operand is the weight tile and the B operand the token tile,
//     so the 32x32 accumulator holds 4 consecutive output columns per lane and
//     register quad: the epilogue writes 8-byte runs of a row.
//   * bf16: v_mfma_f32_32x32x16_bf16 (K = 16 per instruction, 4 per tile).
//     fp8:  v_mfma_scale_f32_32x32x64_f8f6f4 with unit E8M0 scales (K = 64,
//     2 per tile); each 128-wide K tile is one scale group, accumulated into
//     a temporary and added to the fp32 accumulator times
//     (token scale * weight block scale). The token scale is constant per
//     lane (one output row per lane), the weight scale per workgroup tile.
//   * Loads are prefetched into registers one K tile ahead while the current
//     tile is multiplied; LDS is double buffered (one barrier per K tile).
//   * The 1-D grid is remapped so consecutive tiles run on the same XCD
//     (workgroups are dealt round-robin over the 8 XCDs), and tiles are
//     ordered in groups of GM row blocks per column tile so that an expert's
//     weight tile is reused from that XCD's L2 by the row blocks that need it.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kRowBytes = 128;  // one tile row = 128 bytes of K
constexpr int kChunks = kRowBytes / 16;

__device__ __forceinline__ int swz(int row, int chunk) {  // 16-byte chunk index in LDS
    return row * kChunks + (chunk ^ (row & 7));
}

template <int BM, int BN, int WM, int WN, bool FP8>
struct Tile {
    static constexpr int kThreads = WM * WN * 64;
    static constexpr int WTM = BM / WM;  // token rows per wave
    static constexpr int WTN = BN / WN;  // weight rows per wave
    static constexpr int TM = WTM / 32;
    static constexpr int TN = WTN / 32;
    static constexpr int kAChunks = BM * kChunks / kThreads;  // token chunks per thread
    static constexpr int kBChunks = BN * kChunks / kThreads;  // weight chunks per thread
    static constexpr int kElemsPerRow = FP8 ? 128 : 64;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 MFMA tiles");
    static_assert(BM * kChunks % kThreads == 0 && BN * kChunks % kThreads == 0, "load split");
};

template <int BM, int BN, int WM, int WN, bool FP8>
__global__ __launch_bounds__(WM * WN * 64) void grouped_gemm_kernel(GemmArgs p) {
    using T = Tile<BM, BN, WM, WN, FP8>;
    constexpr int NT = T::kThreads;
    __shared__ __attribute__((aligned(16))) u32x4_t sA[2][BM * kChunks];
    __shared__ __attribute__((aligned(16))) u32x4_t sB[2][BN * kChunks];

    // ---- tile scheduling: XCD-aware remap, then grouped ordering ----------
    const int n_tiles = (p.N + BN - 1) / BN;
    const int total = p.m_blocks * n_tiles;
    // hardware id h runs on XCD h % 8; XCD x receives the contiguous logical
    // range starting at x*q + min(x, rem) (a bijection onto [0, total))
    const int h = blockIdx.x, xcd = h & 7;
    const int q = total >> 3, rem = total & 7;
    const int tile = xcd * q + min(xcd, rem) + (h >> 3);
    const int group_rows = p.group_m;
    const int per_group = group_rows * n_tiles;
    const int g = tile / per_group;
    const int first_mb = g * group_rows;
    const int rows_in_group = min(group_rows, p.m_blocks - first_mb);
    const int mb = first_mb + (tile % per_group) % rows_in_group;
    const int nb = (tile % per_group) / rows_in_group;

    const int npp = *p.npp;
    const int64_t m0 = static_cast<int64_t>(mb) * BM;
    if (m0 >= npp) return;
    const int e = p.expert_ids[mb];
    if (e < 0) return;
    const int n0 = nb * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // ---- per-thread global source pointers --------------------------------
    const uint8_t* a_src[T::kAChunks];
    int a_lds[T::kAChunks];
#pragma unroll
    for (int i = 0; i < T::kAChunks; ++i) {
        const int c = tid + i * NT, row = c / kChunks, ch = c % kChunks;
        int64_t src_row = m0 + row;
        if (p.sorted) {
            const int r = p.sorted[m0 + row];
            src_row = r < p.R ? r / p.topk : 0;  // padding rows read token 0
        }
        a_src[i] = reinterpret_cast<const uint8_t*>(p.A) + src_row * p.lda_bytes + ch * 16;
        a_lds[i] = swz(row, ch);
    }
    const uint8_t* w_base = reinterpret_cast<const uint8_t*>(p.W) + static_cast<int64_t>(e) * p.w_expert_bytes;
    const uint8_t* b_src[T::kBChunks];
    int b_lds[T::kBChunks];
#pragma unroll
    for (int i = 0; i < T::kBChunks; ++i) {
        const int c = tid + i * NT, row = c / kChunks, ch = c % kChunks;
        const int n = min(n0 + row, p.N - 1);  // rows past N load a valid row, never stored
        b_src[i] = w_base + static_cast<int64_t>(n) * p.ldw_bytes + ch * 16;
        b_lds[i] = swz(row, ch);
    }

    // fp8: per-lane token scale rows and the workgroup's weight scale row
    const float* xs_row[T::TM];
    const float* ws_row = nullptr;
    if constexpr (FP8) {
#pragma unroll
        for (int tm = 0; tm < T::TM; ++tm) {
            const int row = wm * T::WTM + tm * 32 + (lane & 31);
            int64_t src_row = m0 + row;
            if (p.sorted) {
                const int r = p.sorted[m0 + row];
                src_row = r < p.R ? r / p.topk : 0;
            }
            xs_row[tm] = p.a_scale + src_row * p.scale_groups;
        }
        ws_row = p.w_scale + static_cast<int64_t>(e) * p.w_scale_expert +
                 static_cast<int64_t>(n0 / 128) * p.scale_groups;
    }

    const int KT = p.K / T::kElemsPerRow;
    u32x4_t ra[T::kAChunks], rb[T::kBChunks];
    auto load = [&](int kt) {
        const int64_t off = static_cast<int64_t>(kt) * kRowBytes;
#pragma unroll
        for (int i = 0; i < T::kAChunks; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(a_src[i] + off);
#pragma unroll
        for (int i = 0; i < T::kBChunks; ++i) rb[i] = *reinterpret_cast<const u32x4_t*>(b_src[i] + off);
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < T::kAChunks; ++i) sA[buf][a_lds[i]] = ra[i];
#pragma unroll
        for (int i = 0; i < T::kBChunks; ++i) sB[buf][b_lds[i]] = rb[i];
    };

    f32x16_t acc[T::TN][T::TM];
#pragma unroll
    for (int i = 0; i < T::TN; ++i)
#pragma unroll
        for (int j = 0; j < T::TM; ++j) acc[i][j] = f32x16_t{};

    const int frag_row = lane & 31, khalf = lane >> 5;

    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) load(kt + 1);
        if constexpr (!FP8) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                bf16x8_t fb[T::TN], fa[T::TM];
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn)
                    fb[tn] = __builtin_bit_cast(
                        bf16x8_t, sB[buf][swz(wn * T::WTN + tn * 32 + frag_row, 2 * ks + khalf)]);
#pragma unroll
                for (int tm = 0; tm < T::TM; ++tm)
                    fa[tm] = __builtin_bit_cast(
                        bf16x8_t, sA[buf][swz(wm * T::WTM + tm * 32 + frag_row, 2 * ks + khalf)]);
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
                    for (int tm = 0; tm < T::TM; ++tm)
                        acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[tn], fa[tm],
                                                                              acc[tn][tm], 0, 0, 0);
            }
        } else {
            float sx[T::TM];
#pragma unroll
            for (int tm = 0; tm < T::TM; ++tm) sx[tm] = xs_row[tm][kt];
            const float sw = ws_row[kt];
            f32x16_t part[T::TN][T::TM];
#pragma unroll
            for (int i = 0; i < T::TN; ++i)
#pragma unroll
                for (int j = 0; j < T::TM; ++j) part[i][j] = f32x16_t{};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                i32x8_t fb[T::TN], fa[T::TM];
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn) {
                    const int row = wn * T::WTN + tn * 32 + frag_row;
                    const u32x4_t lo = sB[buf][swz(row, 4 * ks + 2 * khalf)];
                    const u32x4_t hi = sB[buf][swz(row, 4 * ks + 2 * khalf + 1)];
                    fb[tn] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                }
#pragma unroll
                for (int tm = 0; tm < T::TM; ++tm) {
                    const int row = wm * T::WTM + tm * 32 + frag_row;
                    const u32x4_t lo = sA[buf][swz(row, 4 * ks + 2 * khalf)];
                    const u32x4_t hi = sA[buf][swz(row, 4 * ks + 2 * khalf + 1)];
                    fa[tm] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                }
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
                    for (int tm = 0; tm < T::TM; ++tm)
                        // formats 0/0 = e4m3 x e4m3; E8M0 scale 127 = 1.0
                        part[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fb[tn], fa[tm], part[tn][tm], 0, 0, 0, 127, 0, 127);
            }
#pragma unroll
            for (int tm = 0; tm < T::TM; ++tm) {
                const float s = sx[tm] * sw;
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[tn][tm][r] += part[tn][tm][r] * s;
            }
        }
        if (kt + 1 < KT) store(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: bf16, 4 consecutive columns per lane and register quad --
    uint8_t* c_base = reinterpret_cast<uint8_t*>(p.C);
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) {
        const int64_t row = m0 + wm * T::WTM + tm * 32 + (lane & 31);
#pragma unroll
        for (int tn = 0; tn < T::TN; ++tn) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * T::WTN + tn * 32 + 8 * q + 4 * khalf;
                if (n < p.N) {
                    const f32x16_t& a = acc[tn][tm];
                    u32x2_t v{pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3])};
                    *reinterpret_cast<u32x2_t*>(c_base + row * p.ldc_bytes + n * 2) = v;
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, bool FP8>
hipError_t launch_tile(const GemmArgs& a, hipStream_t stream) {
    const int n_tiles = (a.N + BN - 1) / BN;
    const dim3 grid(static_cast<unsigned>(a.m_blocks * n_tiles));
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, BN, WM, WN, FP8>), grid, dim3(WM * WN * 64), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

int gemm_supported_block_m(int bm) { return bm == 32 || bm == 64 || bm == 128; }

hipError_t launch_grouped_gemm(const GemmArgs& a, int block_m, bool fp8, hipStream_t stream) {
    if (!fp8) {
        switch (block_m) {
            case 32: return launch_tile<32, 128, 1, 4, false>(a, stream);
            case 64: return launch_tile<64, 128, 2, 2, false>(a, stream);
            case 128: return launch_tile<128, 128, 2, 2, false>(a, stream);
        }
    } else {
        switch (block_m) {
            case 32: return launch_tile<32, 128, 1, 4, true>(a, stream);
            case 64: return launch_tile<64, 128, 2, 2, true>(a, stream);
            case 128: return launch_tile<128, 128, 2, 2, true>(a, stream);
        }
    }
    return hipErrorInvalidValue;
}
