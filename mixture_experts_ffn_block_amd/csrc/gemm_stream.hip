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
// MFMA's sum over K is exact regardless of the order the slots take. Chunks
// pass through a ring of D register buffers: D - 1 chunks are in flight while
// one is multiplied, and the ring is unrolled so every buffer index is a
// compile-time constant and the wait before each chunk counts exactly the
// loads issued after it. The token rows (tiny) are re-read by every wave from
// L2; the weights stream from HBM once per expert block.
// Tiled weights (16-row x 32-column tiles, row-major inside, ordered by row
// block then column block) are read 1 KB per instruction: the 64 lanes take
// the 64 pieces of one tile, and a 16-row tile is one contiguous run along K.
// The lanes receive the same values as from row-major weights, so both orders
// give identical bits, and HBM streams whole contiguous runs instead of 64
// bytes from each of 16 rows (about 6-7 TB/s against 5 TB/s on gfx950).
// Each 64-row group of weight rows starts its K sweep at a different offset
// (rotated in units of 256 K elements): waves that start together then read
// different 512-byte phases of their rows instead of all hitting the same
// phase of the same 4 KB-strided rows at once, which spreads the reads over
// the HBM channels. The rotation depends only on the expert block and on the
// output column, so GEMM1 with and without the SiLU epilogue add the K pieces
// of every output in the same order and agree bit for bit.
// GEMM1 with SiLU-and-mul in the epilogue: a wave owns the 16 gate rows and the
// 16 matching up rows of 16 output columns, so a lane holds gate and up of the
// same 4 outputs and writes z directly; h never reaches HBM.
#include "common.h"
#include "kernels.h"
#include "layout.h"

namespace {

// waves per workgroup: 8 on packed weights (2 % faster there), 4 on row-major ones
template <bool PACKED>
constexpr int kWavesPerWG = PACKED ? 8 : 4;

// Routing layout of row block mb (16 rows), rebuilt in LDS from the routed ids by
// the NT threads of a workgroup: the layout the align kernel writes ("fused_moe.py
// analysis", moe_align_block_size; "DeepGEMM FusedMoE on Blackwell", 2.6.2), with
// expert segments padded to 16 rows in expert order and items ascending inside a
// segment. Returns the block's expert (-1 past the padded total), sets npp and
// leaves the block's items in rows[0..15] (R for padding). The workgroup of column
// tile 0 (writer) stores the block's part of the layout for the later stages, and
// the one of block 0 also npp and inv_perm -1 for items no local expert takes.
// The ids are read once (R <= kSelfAlignMaxR); the rest is an LDS histogram, a
// one-wave DPP scan that also finds the block's expert, and a ballot rank over
// that expert's items: five workgroup barriers ahead of the weight stream.
template <int NT>
__device__ int self_layout(const GemmArgs& p, int mb, bool writer, int32_t* rows, int& npp) {
    static_assert(NT % MOE_WAVE == 0 && kSelfAlignMaxR % NT == 0, "whole waves, whole passes");
    constexpr int kPasses = kSelfAlignMaxR / NT;
    __shared__ int32_t count[kMaxE];
    __shared__ int32_t wave_hits[NT / MOE_WAVE];
    __shared__ int32_t blk[3];  // the block's expert, its first rank in that expert, npp
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = p.R, E = p.route_E;
    const int m0 = mb * 16;

    int el[kPasses];  // local expert of item tid + i * NT (-1: none)
#pragma unroll
    for (int i = 0; i < kPasses; ++i) {
        const int r = tid + i * NT;
        el[i] = r < R ? local_expert(p.route_ids[r], p.route_emap, p.route_E_global) : -1;
        if (static_cast<unsigned>(el[i]) >= static_cast<unsigned>(E)) el[i] = -1;
    }
    for (int i = tid; i < kMaxE; i += NT) count[i] = 0;
    if (tid < 16) rows[tid] = R;
    if (tid == 0) blk[0] = -1;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPasses; ++i)
        if (el[i] >= 0) atomicAdd(&count[el[i]], 1);
    __syncthreads();
    if (wave == 0) {
        // padded sizes -> segment starts; the lane holding the segment of row m0
        // (a non-empty one) records the block's expert
        int v[4], size[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ex = 4 * lane + i;
            size[i] = ex < E ? (count[ex] + 15) / 16 * 16 : 0;
            v[i] = size[i];
        }
        const int total = scan_padded(v);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (v[i] <= m0 && m0 < v[i] + size[i]) {
                blk[0] = 4 * lane + i;
                blk[1] = m0 - v[i];
            }
        if (lane == 0) blk[2] = total;
    }
    __syncthreads();
    const int e = blk[0];
    npp = blk[2];
    if (e >= 0) {
        // the block holds ranks j0 .. j0 + 15 of expert e's items (in item order)
        const int j0 = blk[1];
        int base = 0;  // items of expert e in earlier passes (the same in every thread)
#pragma unroll
        for (int i = 0; i < kPasses; ++i) {
            if (i * NT >= R || base >= j0 + 16) break;
            const bool hit = el[i] == e;
            const uint64_t m = ballot64(hit);
            if (lane == 0) wave_hits[wave] = __popcll(m);
            __syncthreads();
            int before = base;
            for (int w = 0; w < NT / MOE_WAVE; ++w) {
                const int c = wave_hits[w];
                if (w < wave) before += c;
                base += c;
            }
            const int j = before + __popcll(m & ((1ull << lane) - 1ull)) - j0;
            if (hit && j >= 0 && j < 16) rows[j] = tid + i * NT;
            __syncthreads();  // rows complete; wave_hits free for the next pass
        }
    }
    if (writer) {
        if (tid < 16) {
            const int r = rows[tid];
            p.out_sorted[m0 + tid] = r;
            if (r < R) p.out_inv_perm[r] = m0 + tid;
        }
        if (tid == 0) p.out_expert_ids[mb] = e;
        if (mb == 0) {
            if (tid == 0) *p.out_npp = npp;
#pragma unroll
            for (int i = 0; i < kPasses; ++i)
                if (tid + i * NT < R && el[i] < 0) p.out_inv_perm[tid + i * NT] = -1;
        }
    }
    return e;
}

// TILES 16-row weight tiles per wave; per K chunk every row contributes S pieces of
// 64 contiguous bytes (32 S bf16), and D chunks share the register ring (the host
// picks D dividing K / (32 S)). ACT (GEMM1 with SiLU-and-mul, TILES = 2): tile 0
// holds the 16 gate rows and tile 1 the 16 up rows of the wave's 16 output columns.
// SELF (with ACT): the workgroup rebuilds its block's routing layout (self_layout)
// instead of reading it.
template <bool GATHER, bool ACT, int TILES, int S, int D, bool PACKED, bool SELF>
__global__ __launch_bounds__(kWavesPerWG<PACKED> * 64) void stream_gemm_bf16_kernel(GemmArgs p) {
    static_assert(!ACT || (GATHER && TILES == 2), "SiLU epilogue: GEMM1, one gate and one up tile");
    static_assert(!SELF || ACT, "self-aligned: GEMM1 with the SiLU epilogue");
    constexpr int kColsPerWave = ACT ? 16 : 16 * TILES;  // output columns
    constexpr int kColsPerWG = kWavesPerWG<PACKED> * kColsPerWave;
    const int n_wg = (p.N + kColsPerWG - 1) / kColsPerWG;
    const int mb = blockIdx.x / n_wg, nb = blockIdx.x % n_wg;
    const int64_t m0 = static_cast<int64_t>(mb) * 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row16 = lane & 15, kq = lane >> 4;

    int e, npp, r_item = 0;
    if constexpr (SELF) {
        __shared__ int32_t rows[16];
        e = self_layout<kWavesPerWG<PACKED> * 64>(p, mb, nb == 0, rows, npp);
        if (m0 >= npp || e < 0) return;
        r_item = rows[row16];
    } else {
        npp = *p.npp;
        if (m0 >= npp) return;
        e = p.expert_ids[mb];
        if (e < 0) return;
        if constexpr (GATHER) r_item = p.sorted[m0 + row16];
    }

    const int nw0 = nb * kColsPerWG + wave * kColsPerWave;
    if (nw0 >= p.N) return;

    int64_t src_row = m0 + row16;
    if constexpr (GATHER) src_row = r_item < p.R ? r_item / p.topk : 0;  // padding rows read token 0
    const uint8_t* a_ptr = reinterpret_cast<const uint8_t*>(p.A) + src_row * p.lda_bytes + kq * 16;
    const uint8_t* w_base = reinterpret_cast<const uint8_t*>(p.W) + static_cast<int64_t>(e) * p.w_expert_bytes;
    // PS: bytes between consecutive 32-wide K pieces of one lane's weight row
    constexpr int PS = PACKED ? 1024 : 64;
    const uint8_t* w_ptr[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
        if constexpr (PACKED) {
            // 16-row tiles (N is a multiple of 64 here): tile of gate row n0 or up row N + n0;
            // the lane's row and 16-byte piece inside each 1 KB tile
            const int tile = ACT ? t * (p.N / 16) + nw0 / 16 : min(nw0 / 16 + t, p.N / 16 - 1);
            w_ptr[t] = w_base + static_cast<int64_t>(tile) * 16 * p.ldw_bytes + row16 * 64 + kq * 16;
        } else {
            // ACT: gate row n (t = 0) or up row N + n (t = 1) of output column n
            const int n = ACT ? t * p.N + min(nw0 + row16, p.N - 1) : min(nw0 + 16 * t + row16, p.N - 1);
            w_ptr[t] = w_base + static_cast<int64_t>(n) * p.ldw_bytes + kq * 16;
        }
    }

    f32x4_t acc[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) acc[t] = f32x4_t{};

    // K rotation: units of 8 pieces (256 K) where K allows, else 4 (S divides it).
    // The 64-row group of the wave's rows: GEMM1 rows fold gate onto up (row mod N/2
    // without the epilogue, the output column with it), so both forms rotate alike.
    const int KC = p.K / (32 * S);
    const int unit = (p.K / 32) % 8 == 0 ? 8 : 4;
    const int n_units = p.K / (32 * unit);
    const int grp = (ACT ? nw0 : nw0 % (p.N / 2)) >> 6;
    const int shift = GATHER ? ((mb + grp) % n_units) * (unit / S) : 0;  // GEMM2: no gain measured

    u32x4_t a_buf[D][S], w_buf[D][TILES][S];
    auto load = [&](int kc, u32x4_t (&a)[S], u32x4_t (&w)[TILES][S]) {
        int kr = kc + shift;
        if (kr >= KC) kr -= KC;
        const int64_t off = static_cast<int64_t>(kr) * 64 * S, woff = static_cast<int64_t>(kr) * PS * S;
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
            for (int s = 0; s < S; ++s)
                w[t][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(w_ptr[t] + woff + PS * s));
#pragma unroll
        for (int s = 0; s < S; ++s) a[s] = *reinterpret_cast<const u32x4_t*>(a_ptr + off + 64 * s);
    };
    auto multiply = [&](const u32x4_t (&a)[S], const u32x4_t (&w)[TILES][S]) {
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int t = 0; t < TILES; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, w[t][s]), __builtin_bit_cast(bf16x8_t, a[s]), acc[t], 0, 0, 0);
    };
    // KC is a multiple of D (host): the last group of D chunks is peeled so that no
    // load is conditional and the compiler's wait counts stay exact
#pragma unroll
    for (int d = 0; d < D - 1; ++d) load(d, a_buf[d], w_buf[d]);
    int kc0 = 0;
    for (; kc0 < KC - D; kc0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            // program order kept: a chunk's loads all go out before the wait for
            // the oldest chunk, never after it
            load(kc0 + d + D - 1, a_buf[(d + D - 1) % D], w_buf[(d + D - 1) % D]);
            __builtin_amdgcn_sched_barrier(0);
            multiply(a_buf[d], w_buf[d]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    load(kc0 + D - 1, a_buf[D - 1], w_buf[D - 1]);
#pragma unroll
    for (int d = 0; d < D; ++d) multiply(a_buf[d], w_buf[d]);

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

template <bool GATHER, bool ACT, int TILES, int S, int D, bool PACKED, bool SELF>
hipError_t launch_stream_as(const GemmArgs& a, hipStream_t stream) {
    constexpr int kColsPerWG = kWavesPerWG<PACKED> * (ACT ? 16 : 16 * TILES);
    const int n_wg = (a.N + kColsPerWG - 1) / kColsPerWG;
    const dim3 grid(static_cast<unsigned>(a.m_blocks * n_wg));
    hipLaunchKernelGGL((stream_gemm_bf16_kernel<GATHER, ACT, TILES, S, D, PACKED, SELF>), grid,
                       dim3(kWavesPerWG<PACKED> * 64), 0, stream, a);
    return hipGetLastError();
}

// ring depth: 4 chunks for the SiLU form, 2 for the 64-row form (deeper rings
// measured no faster there), or the largest smaller depth dividing the chunks
template <bool GATHER, bool ACT, int TILES, int S, bool PACKED, bool SELF = false>
hipError_t launch_stream_ring(const GemmArgs& a, hipStream_t stream) {
    const int kc = a.K / (32 * S);
    if constexpr (ACT) {  // (the 4-deep ring is instantiated for the SiLU form only)
        if (kc % 4 == 0) return launch_stream_as<GATHER, ACT, TILES, S, 4, PACKED, SELF>(a, stream);
    }
    if (kc % 2 == 0) return launch_stream_as<GATHER, ACT, TILES, S, 2, PACKED, SELF>(a, stream);
    return launch_stream_as<GATHER, ACT, TILES, S, 1, PACKED, SELF>(a, stream);
}

template <bool PACKED>
hipError_t launch_stream_layout(const GemmArgs& a, hipStream_t stream) {
    if (a.act) {
        if (a.route_ids) {
            if (a.R > kSelfAlignMaxR || a.route_E > kMaxE || !a.out_sorted || !a.out_expert_ids ||
                !a.out_npp || !a.out_inv_perm)
                return hipErrorInvalidValue;
            return launch_stream_ring<true, true, 2, 4, PACKED, true>(a, stream);
        }
        if (!a.sorted) return hipErrorInvalidValue;
        return launch_stream_ring<true, true, 2, 4, PACKED>(a, stream);
    }
    return a.sorted ? launch_stream_ring<true, false, 4, 4, PACKED>(a, stream)
                    : launch_stream_ring<false, false, 4, 4, PACKED>(a, stream);
}

}  // namespace

// K is a multiple of 128 and N of 64 (checked on the host). Chunks of S = 4 pieces
// of 32 K per row: two 16-row tiles in a ring of up to 4 chunks (SiLU form) or four
// tiles in a ring of 2, so that two waves fit on a SIMD.
hipError_t launch_stream_gemm(const GemmArgs& a, hipStream_t stream) {
    return a.w_packed ? launch_stream_layout<true>(a, stream) : launch_stream_layout<false>(a, stream);
}
