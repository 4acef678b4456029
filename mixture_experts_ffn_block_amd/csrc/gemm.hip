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
//   * The 1-D grid is remapped so consecutive tiles run on the same XCD
//     (workgroups are dealt round-robin over the 8 XCDs), and tiles are
//     ordered in groups of GM row blocks per column tile so that an expert's
//     weight tile is reused from that XCD's L2 by the row blocks that need it.
//
// The kernels in this file, by block_m:
//   * 32 / 64: expert_gemm_kernel, loads prefetched into registers one K tile
//     ahead, LDS double buffered (one barrier per K tile).
//   * 128 / 256, bf16: expert_gemm_dma_kernel, a ring of 4-5 LDS stages filled by
//     direct-to-LDS copies, 8 waves; row groups of padding alone are not
//     multiplied; GEMM1 may carry SiLU-and-mul in its epilogue, GEMM2 splits a
//     last, partly filled round of tiles along K.
//   * 128, fp8 / MXFP8 / W4A8: expert_gemm_fp8_kernel, persistent, one continuous
//     stream of K stages across a workgroup's tiles, scaled MFMA.
// (block_m 16, the weight-streaming decode GEMM, is in gemm_stream.hip.)
#include <atomic>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int kRowBytes = 128;  // one tile row = 128 bytes of K
constexpr int kChunks = kRowBytes / 16;

// 16-byte chunk index in LDS. The XOR key changes every second row, so the 16
// lanes that one ds_read_b128 serves together (rows r..r+15, one logical
// chunk) land in 16 distinct 16-byte bank groups of a 256-byte bank row.
__device__ __forceinline__ int swz(int row, int chunk) {
    return row * kChunks + (chunk ^ ((row >> 1) & 7));
}

// Tile geometry: 4 wavefronts side by side along N. Every wave multiplies all
// BM token rows by its own WN = BN/4 weight rows, so the token fragments it
// reads from LDS are reused across TN weight tiles and vice versa.
template <int BM, int BN, bool FP8>
struct Tile {
    static constexpr int kThreads = 256;
    static constexpr int WN = BN / 4;    // weight rows per wave
    static constexpr int TM = BM / 32;   // 32-row MFMA tiles along M
    static constexpr int TN = WN / 32;   // 32-row MFMA tiles along N
    static constexpr int kAChunks = BM * kChunks / kThreads;  // 16-byte token chunks per thread
    static constexpr int kBChunks = BN * kChunks / kThreads;  // 16-byte weight chunks per thread
    static constexpr int kElemsPerRow = FP8 ? 128 : 64;       // K per 128-byte tile row
    static constexpr int kLdsBytes = 2 * (BM + BN) * kRowBytes;
    static_assert(BM % 32 == 0 && WN % 32 == 0, "whole 32x32 MFMA tiles");
    static_assert(BM * kChunks % kThreads == 0 && BN * kChunks % kThreads == 0, "load split");
    static_assert(kLdsBytes <= 160 * 1024, "fits gfx950 LDS");
};

// ---- epilogue through LDS, shared by the copy-ring kernels -----------------
// A wave's accumulators cover TM*32 token rows x TN*32 weight columns, a lane
// holding 4 consecutive columns of one row per register quad (the swapped
// MFMA orientation). Stored straight to C, every store instruction would
// write 16 bytes into each of 32 rows; staged through the wave's own LDS
// area first, every store instruction writes whole 128-byte lines (8 lanes x
// 16 bytes per row). `stage` holds TMP*32 rows of TN*64 + 16 bytes (the pad
// spreads consecutive rows over the banks; TMP row tiles per pass, the
// passes reusing the area in the wave's program order). col0 and N are
// multiples of 64, so each 64-column chunk is wholly inside or outside C.
template <int TM, int TN, int TMP>
__device__ __forceinline__ void store_block(const f32x16_t (&acc)[TN][TM], uint8_t* stage,
                                            uint8_t* c, int64_t row0, int col0, int64_t ldc_bytes,
                                            int N, int lane) {
    // TMP row tiles of 32 per pass: `stage` holds TMP*32 rows of TN*64 + 16 bytes
    constexpr int PITCH = TN * 64 + 16, CH = TN * 4, RPP = 64 / CH;
    static_assert(TM % TMP == 0, "whole passes");
    const int r32 = lane & 31, half = lane >> 5;
    const int ch = lane % CH;
    const int col = col0 + ch * 8;
#pragma unroll
    for (int t0 = 0; t0 < TM; t0 += TMP) {
#pragma unroll
        for (int tm = t0; tm < t0 + TMP; ++tm)
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x16_t& a = acc[tn][tm];
                    const int cc = tn * 32 + 8 * q + 4 * half;
                    *reinterpret_cast<u32x2_t*>(stage + ((tm - t0) * 32 + r32) * PITCH + cc * 2) =
                        u32x2_t{pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3])};
                }
#pragma unroll
        for (int pass = 0; pass < TMP * 32 / RPP; ++pass) {
            const int row = pass * RPP + lane / CH;
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + row * PITCH + ch * 16);
            // streaming stores: C is not read again by this kernel
            if (col < N)
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(c + (row0 + t0 * 32 + row) * ldc_bytes + col * 2));
        }
    }
}

// ---- tile scheduling, shared by the LDS-tiled kernels ---------------------
// The grid is sized for the worst-case number of expert blocks; only the
// first npp / BM blocks hold rows, so the logical tiles are those of the real
// blocks and the rest of the grid exits at once (otherwise the empty tiles,
// which come last in the logical order, would leave whole XCDs idle).
// Hardware id h runs on XCD h % 8; XCD x receives the contiguous logical range
// starting at x*q + min(x, rem), a bijection onto [0, total), so tiles that
// share token rows or weight rows meet in one L2.
// Logical order: the blocks are cut into groups, each a maximal run of blocks
// of one expert inside an aligned window of group_m blocks, and a group's tiles
// are walked down one column of tiles before the next column. A group never
// mixes two experts, so its tiles of one column share a single weight tile.
// Group [gs, ge) owns exactly the logical tiles [gs, ge) x n_tiles, so a
// workgroup finds its group from at most 2 * group_m expert ids.
struct TilePos {
    int mb, nb;
};
// Called by whole wavefronts (wave-uniform arguments): the window's expert ids
// arrive in one vector load, one per lane (group_m <= 64), and a ballot marks the
// blocks of the tile's expert; the group is the run of marked blocks around b0.
__device__ __forceinline__ void tile_in_group(const GemmArgs& p, int tile, int n_tiles, int m_real,
                                              TilePos& t) {
    const int b0 = tile / n_tiles;
    const int w0 = b0 / p.group_m * p.group_m, w1 = min(w0 + p.group_m, m_real);
    const int lane = threadIdx.x & 63, i0 = b0 - w0;
    const int eid = w0 + lane < w1 ? p.expert_ids[w0 + lane] : -2;  // real blocks hold ids >= 0
    const uint64_t same = ballot64(eid == __shfl(eid, i0, 64));     // bit i0 is set
    const uint64_t up = ~same >> i0, below = ~same & ((1ull << i0) - 1ull);
    const int ge = up != 0 ? b0 + __builtin_ctzll(up) : w0 + 64;
    const int gs = below != 0 ? w0 + 64 - __builtin_clzll(below) : w0;
    const int local = tile - gs * n_tiles, rows = ge - gs;
    t.mb = gs + local % rows;
    t.nb = local / rows;
}
template <int BM, int BN>
__device__ __forceinline__ bool tile_of(const GemmArgs& p, TilePos& t) {
    const int n_tiles = (p.N + BN - 1) / BN;
    const int m_real = min(p.m_blocks, (*p.npp + BM - 1) / BM);
    const int total = m_real * n_tiles;
    const int hw = blockIdx.x;
    if (hw >= total) return false;
    const int xcd = hw & 7, q8 = total >> 3, rem = total & 7;
    tile_in_group(p, xcd * q8 + min(xcd, rem) + (hw >> 3), n_tiles, m_real, t);
    return true;
}

// Split-K of the last round (for the DMA-tiled GEMM without a gather). With
// W = n_cu workgroups running at once and T real tiles, T = F W + tail: the F W
// tiles of the full rounds run whole, and when the tail would fill at most half
// a round, each tail tile is cut into S = 2 or 4 K ranges that fill one round
// (S divides the K stages; tail S <= part_slots). Workgroup h < F W takes tile h
// in the XCD-contiguous order of the F W tiles. The S ranges of a tail tile are
// given workgroup ids congruent mod 8 (unit u = h - F W serves tail tile
// j = u % 8 + 8 ((u / 8) / S), K range (u / 8) % S), which the dispatcher
// places on one XCD when it deals workgroups round-robin, so their partials
// tend to meet in one L2; the partials are published with an agent-scope
// release, so the result does not depend on that placement. The grid has
// W + 32 extra workgroups for this (8 ceil(tail / 8) S <= W + 7 S).
struct SplitPos {
    int tile, S, chunk, slot, tail_tile;  // slot: partial tile index; -1 for a whole tile
};
template <int BM, int COLS>
__device__ __forceinline__ bool split_tile_of(const GemmArgs& p, int KT, TilePos& t, SplitPos& sp) {
    const int n_tiles = (p.N + COLS - 1) / COLS;
    const int m_real = min(p.m_blocks, (*p.npp + BM - 1) / BM);
    const int total = m_real * n_tiles;
    const int hw = blockIdx.x;
    const int W = p.n_cu, F = total / W, tail = total - F * W;
    int S = 1;
    if (p.part != nullptr && tail > 0 && 2 * tail <= W) {
        S = 4 * tail <= W ? 4 : 2;
        while (S > 1 && (KT % S != 0 || tail * S > p.part_slots)) S >>= 1;
    }
    const int main_tiles = S == 1 ? total : F * W;
    sp.S = 1;
    sp.chunk = 0;
    sp.slot = -1;
    sp.tail_tile = -1;
    if (hw < main_tiles) {
        const int xcd = hw & 7, q8 = main_tiles >> 3, rem = main_tiles & 7;
        sp.tile = xcd * q8 + min(xcd, rem) + (hw >> 3);
    } else if (S > 1) {
        const int u = hw - main_tiles, q = u >> 3;
        const int j = (u & 7) + 8 * (q / S);
        if (j >= tail) return false;
        sp.S = S;
        sp.chunk = q % S;
        sp.tail_tile = j;
        sp.slot = j * S + sp.chunk;
        sp.tile = main_tiles + j;
    } else {
        return false;
    }
    tile_in_group(p, sp.tile, n_tiles, m_real, t);
    return true;
}

// Both operands are staged through LDS: 8 consecutive lanes load one row's
// 128-byte K slice, so every global load instruction reads whole cache lines.
// The next K tile is loaded into registers while the current one is
// multiplied, then written to the other LDS buffer (one barrier per K tile).
template <int BM, int BN, bool FP8, bool GATHER>
__global__ __launch_bounds__(256) void expert_gemm_kernel(GemmArgs p) {
    using T = Tile<BM, BN, FP8>;
    __shared__ __attribute__((aligned(16))) u32x4_t sA[2][BM * kChunks];
    __shared__ __attribute__((aligned(16))) u32x4_t sB[2][BN * kChunks];

    TilePos tp;
    if (!tile_of<BM, BN>(p, tp)) return;
    const int mb = tp.mb, nb = tp.nb;
    const int64_t m0 = static_cast<int64_t>(mb) * BM;
    const int e = p.expert_ids[mb];
    if (e < 0) return;
    const int n0 = nb * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r32 = lane & 31, half = lane >> 5;
    const int ld_row = tid >> 3, ld_ch = tid & 7;  // this thread's row (+32 i) and chunk

    auto src_row_of = [&](int row) -> int64_t {
        if constexpr (GATHER) {
            const int r = p.sorted[m0 + row];
            return r < p.R ? r / p.topk : 0;  // padding rows read token 0
        } else {
            return m0 + row;
        }
    };

    const uint8_t* a_src[T::kAChunks];
#pragma unroll
    for (int i = 0; i < T::kAChunks; ++i)
        a_src[i] = reinterpret_cast<const uint8_t*>(p.A) + src_row_of(ld_row + 32 * i) * p.lda_bytes + ld_ch * 16;
    const uint8_t* w_base = reinterpret_cast<const uint8_t*>(p.W) + static_cast<int64_t>(e) * p.w_expert_bytes + ld_ch * 16;
    int32_t b_off[T::kBChunks];  // per-expert byte offsets fit in 32 bits (checked on the host)
#pragma unroll
    for (int i = 0; i < T::kBChunks; ++i)
        b_off[i] = min(n0 + ld_row + 32 * i, p.N - 1) * static_cast<int32_t>(p.ldw_bytes);  // rows past N: never stored

    // fp8: per-lane token scale rows and the wave's weight scale row
    const float* xs_row[T::TM];
    const float* ws_row = nullptr;
    if constexpr (FP8) {
#pragma unroll
        for (int tm = 0; tm < T::TM; ++tm) xs_row[tm] = p.a_scale + m0 + tm * 32 + r32;  // group-major
        // a wave's WN (<= 128, dividing 128) weight rows lie in one 128-row scale
        // block; waves wholly past N (tail tile) read the last block, unused
        static_assert(128 % T::WN == 0, "wave columns within one scale block");
        ws_row = p.w_scale + static_cast<int64_t>(e) * p.w_scale_expert +
                 static_cast<int64_t>(min((n0 + wave * T::WN) / 128, p.N / 128 - 1)) * p.scale_groups;
    }

    const int KT = p.K / T::kElemsPerRow;
    u32x4_t ra[T::kAChunks], rb[T::kBChunks];
    auto load = [&](int kt) {
        const int64_t off = static_cast<int64_t>(kt) * kRowBytes;
#pragma unroll
        for (int i = 0; i < T::kAChunks; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(a_src[i] + off);
#pragma unroll
        for (int i = 0; i < T::kBChunks; ++i) rb[i] = *reinterpret_cast<const u32x4_t*>(w_base + b_off[i] + off);
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < T::kAChunks; ++i) sA[buf][swz(ld_row + 32 * i, ld_ch)] = ra[i];
#pragma unroll
        for (int i = 0; i < T::kBChunks; ++i) sB[buf][swz(ld_row + 32 * i, ld_ch)] = rb[i];
    };

    f32x16_t acc[T::TN][T::TM];
#pragma unroll
    for (int i = 0; i < T::TN; ++i)
#pragma unroll
        for (int j = 0; j < T::TM; ++j) acc[i][j] = f32x16_t{};

    const int wrow = wave * T::WN;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) load(kt + 1);
        if constexpr (!FP8) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                bf16x8_t fa[T::TM], fb[T::TN];
#pragma unroll
                for (int tm = 0; tm < T::TM; ++tm)
                    fa[tm] = __builtin_bit_cast(bf16x8_t, sA[buf][swz(tm * 32 + r32, 2 * ks + half)]);
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn)
                    fb[tn] = __builtin_bit_cast(bf16x8_t, sB[buf][swz(wrow + tn * 32 + r32, 2 * ks + half)]);
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
                    for (int tm = 0; tm < T::TM; ++tm)
                        acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[tn], fa[tm], acc[tn][tm], 0, 0, 0);
            }
        } else {
            float sx[T::TM];
#pragma unroll
            for (int tm = 0; tm < T::TM; ++tm) sx[tm] = xs_row[tm][kt * p.a_scale_ld];
            const float sw = ws_row[kt];
            f32x16_t part[T::TN][T::TM];
#pragma unroll
            for (int i = 0; i < T::TN; ++i)
#pragma unroll
                for (int j = 0; j < T::TM; ++j) part[i][j] = f32x16_t{};
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                i32x8_t fa[T::TM], fb[T::TN];
#pragma unroll
                for (int tm = 0; tm < T::TM; ++tm) {
                    const int row = tm * 32 + r32;
                    const u32x4_t lo = sA[buf][swz(row, 4 * s + 2 * half)];
                    const u32x4_t hi = sA[buf][swz(row, 4 * s + 2 * half + 1)];
                    fa[tm] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                }
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn) {
                    const int row = wrow + tn * 32 + r32;
                    const u32x4_t lo = sB[buf][swz(row, 4 * s + 2 * half)];
                    const u32x4_t hi = sB[buf][swz(row, 4 * s + 2 * half + 1)];
                    fb[tn] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
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
                const float sc = sx[tm] * sw;
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[tn][tm][r] += part[tn][tm][r] * sc;
            }
        }
        if (kt + 1 < KT) store(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: bf16, 4 consecutive columns per lane and register quad --
    uint8_t* c_base = reinterpret_cast<uint8_t*>(p.C);
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) {
        const int64_t row = m0 + tm * 32 + r32;
#pragma unroll
        for (int tn = 0; tn < T::TN; ++tn) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wrow + tn * 32 + 8 * q + 4 * half;
                if (n < p.N) {
                    const f32x16_t& a = acc[tn][tm];
                    u32x2_t v{pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3])};
                    *reinterpret_cast<u32x2_t*>(c_base + row * p.ldc_bytes + n * 2) = v;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bf16, BLOCK_M = 128: DMA-pipelined variant.
//
// Tiles are 128 token rows x 512 weight rows x 32 K (64-byte tile rows). Global
// memory is copied straight into LDS with global_load_lds_dwordx4 (each
// instruction fills 1 KB: 16 rows x 64 bytes, lane l writing bytes 16l..16l+15),
// so no VGPRs or ds_write instructions are spent on staging and four LDS
// stages (160 KB) keep three K tiles in flight per CU. The copies are issued
// from inline assembly and waited for with explicit vmcnt counts, because the
// compiler's own wait insertion cannot tell which stage a copy targets and
// would drain all of them before every LDS read. M0 (the LDS destination) is
// saved and restored around each copy.
//
// LDS row layout: 4 chunks of 16 bytes, chunk c of row r stored at
// r*4 + (c ^ ((r >> 2) & 3)); the 16 lanes one ds_read_b128 serves together
// (16 consecutive rows, one logical chunk) then hit 16 distinct 16-byte bank
// groups of a 256-byte bank row.
namespace dma {

// Copies of 1 KB each into consecutive 1 KB LDS blocks starting at `lds`. M0
// holds the LDS base; the instruction offset is added to both the LDS and the
// global address, so copy i passes its global address minus i KB. One M0 write
// serves up to four copies (the offset field reaches 4095); groups of 1, 2 or 4.
template <int N>
__device__ __forceinline__ void copy_group(const uint8_t* const (&g)[N], uint32_t lds) {
    static_assert(N == 1 || N == 2 || N == 4, "groups of 1, 2 or 4 copies");
    uint32_t saved;
    if constexpr (N == 1)
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %2, off\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(lds), "v"(g[0])
            : "memory");
    else if constexpr (N == 4)
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %2, off\n\t"
            "global_load_lds_dwordx4 %3, off offset:1024\n\t"
            "global_load_lds_dwordx4 %4, off offset:2048\n\t"
            "global_load_lds_dwordx4 %5, off offset:3072\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(lds), "v"(g[0]), "v"(g[1] - 1024), "v"(g[2] - 2048), "v"(g[3] - 3072)
            : "memory");
    else
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %2, off\n\t"
            "global_load_lds_dwordx4 %3, off offset:1024\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(lds), "v"(g[0]), "v"(g[1] - 1024)
            : "memory");
}

// scheduling pattern: R LDS reads spread over Mf MFMAs, one read then its
// share of the MFMAs
template <int I, int R, int Mf>
__device__ __forceinline__ void interleave_step() {
    constexpr int n = (I + 1) * Mf / R - I * Mf / R;
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x008, n, 0);  // MFMA
    if constexpr (I + 1 < R) interleave_step<I + 1, R, Mf>();
}

// wait until the copies of all but the newest `newer` K tiles of this wave have
// landed (L copies per tile), then barrier
template <int L>
__device__ __forceinline__ void wait_barrier(int newer) {
    if (newer >= 3)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(3 * L) : "memory");
    else if (newer == 2)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * L) : "memory");
    else if (newer == 1)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(L) : "memory");
    else
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

// Geometry: BM x BN tile, WM x WN waves (NW in total), each wave TM x TN MFMA
// tiles of 32 x 32; STAGES LDS stages of (BM + BN) rows of ROWB bytes (ROWB/2
// bf16 of K, so ROWB/32 MFMA K steps per stage).
//
// LDS rows hold ROWB/16 chunks of 16 bytes; chunk c of row r sits at
// r*CH + (c ^ key(r)). The key changes so that the 16 lanes one ds_read_b128
// serves together (16 consecutive rows, one logical chunk) land in 16 distinct
// 16-byte bank groups of a 256-byte bank row: (r >> 2) & 3 for 64-byte rows,
// (r >> 1) & 7 for 128-byte rows.
template <int BM_, int BN_, int WM_, int STAGES_, int ROWB_, int NW_ = 4>
struct Cfg {
    static constexpr int NW = NW_;  // waves per workgroup
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = NW_ / WM_, STAGES = STAGES_;
    static constexpr int ROWB = ROWB_, CH = ROWB / 16, KS = ROWB / 2, NKS = ROWB / 32;
    static constexpr int ROWS_PER_COPY = 1024 / ROWB;
    static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB, STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int A_INSTR = A_BYTES / 1024 / NW;  // 1 KB copies per wave
    static constexpr int B_INSTR = B_BYTES / 1024 / NW;
    static constexpr int L = A_INSTR + B_INSTR;
    static constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    static_assert(ROWB == 64 || ROWB == 128, "64- or 128-byte rows");
    static_assert(NKS % 2 == 0, "fragment sets alternate; the last K step uses set 1");
    static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "fits gfx950 LDS");
    static_assert(STAGES >= 3 && STAGES - 3 <= 3, "pipeline depth");
    __device__ static __forceinline__ int swz(int row, int chunk) {
        const int key = ROWB == 64 ? ((row >> 2) & 3) : ((row >> 1) & 7);
        return row * CH + (chunk ^ key);
    }
};

}  // namespace dma

template <class C, bool GATHER, bool ACT>
__global__ __launch_bounds__(C::NW * 64) void expert_gemm_dma_kernel(GemmArgs p) {
    static_assert(!ACT || GATHER, "the SiLU epilogue belongs to GEMM1");
    using namespace dma;
    constexpr int BM = C::BM, BN = C::BN, STAGES = C::STAGES, TM = C::TM, TN = C::TN;
    constexpr int A_INSTR = C::A_INSTR, B_INSTR = C::B_INSTR, NKS = C::NKS;
    extern __shared__ __attribute__((aligned(1024))) u32x4_t smem[];
    const uint32_t lds_base = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) u32x4_t*)smem));

    // ACT: a tile covers BN / 2 output columns (z), its BN weight rows being the gate
    // and up rows of those columns (see below)
    constexpr int TILE_COLS = ACT ? BN / 2 : BN;
    constexpr bool SPLIT = !GATHER;  // the split-K tail applies to the second GEMM
    TilePos tp;
    SplitPos sp{0, 1, 0, -1, -1};
    if constexpr (SPLIT) {
        if (!split_tile_of<BM, TILE_COLS>(p, p.K / C::KS, tp, sp)) return;
    } else {
        if (!tile_of<BM, TILE_COLS>(p, tp)) return;
    }
    const int mb = tp.mb, nb = tp.nb;
    const int64_t m0 = static_cast<int64_t>(mb) * BM;
    const int e = p.expert_ids[mb];
    if (e < 0) return;
    const int n0 = nb * TILE_COLS;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r32 = lane & 31, half = lane >> 5;
    const int wm = wave / C::WN, wn = wave % C::WN;

    // copy sources: a wave's copy i covers ROWS_PER_COPY rows; lane l takes row
    // +l/CH and the logical chunk stored in LDS slot l%CH
    const int cp_row = lane / C::CH, cp_slot = lane % C::CH;
    const uint8_t* a_src[A_INSTR];
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) {
        const int row = (wave * A_INSTR + i) * C::ROWS_PER_COPY + cp_row;
        int64_t src = m0 + row;
        if constexpr (GATHER) {
            const int r = p.sorted[m0 + row];
            src = r < p.R ? r / p.topk : 0;  // padding rows read token 0
        }
        const int chunk = C::swz(row, cp_slot) - row * C::CH;  // XOR is its own inverse
        a_src[i] = reinterpret_cast<const uint8_t*>(p.A) + src * p.lda_bytes + chunk * 16;
    }
    const uint8_t* w_base = reinterpret_cast<const uint8_t*>(p.W) + static_cast<int64_t>(e) * p.w_expert_bytes;
    // Tiled weights (16-row x 32-column tiles, row-major inside, ordered by row block
    // then column block): a copy's 16 rows x 64 bytes of one stage are one contiguous
    // 1 KB tile (64-byte rows only), and the next stage's tile follows it directly.
    const int w_stage_bytes = p.w_packed ? 1024 : C::ROWB;
    int32_t b_off[B_INSTR];
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i) {
        const int row = (wave * B_INSTR + i) * C::ROWS_PER_COPY + cp_row;
        const int chunk = C::swz(row, cp_slot) - row * C::CH;
        // ACT: tile row r is a gate row (r / 32 even) or up row (odd) of output column
        // n0 + 32 * (r / 64) + r % 32; gate rows are w13 rows [0, N), up rows [N, 2N)
        const int wrow = ACT ? ((row >> 5) & 1) * p.N + min(n0 + (row >> 6) * 32 + (row & 31), p.N - 1)
                             : min(n0 + row, p.N - 1);
        if (p.w_packed) {
            // the copy's 16 rows are 16 consecutive weight rows from a multiple of 16 (N is
            // a multiple of 128); past the last row a whole tile is clamped
            const int wrow0 = ACT ? ((row >> 5) & 1) * p.N + min(n0 + (row >> 6) * 32 + (row & 16), p.N - 16)
                                  : min(n0 + (row & ~15), p.N - 16);
            b_off[i] = (wrow0 / 16) * (p.K / 32) * 1024 + (row & 15) * 64 + chunk * 16;
        } else {
            b_off[i] = wrow * static_cast<int32_t>(p.ldw_bytes) + chunk * 16;
        }
    }
    // LDS destinations are wave-uniform: keep them in scalar registers
    const uint32_t a_dst = __builtin_amdgcn_readfirstlane(lds_base + wave * A_INSTR * 1024);
    const uint32_t b_dst = __builtin_amdgcn_readfirstlane(lds_base + C::A_BYTES + wave * B_INSTR * 1024);

    // a split tile covers K stages [chunk KT / S, (chunk + 1) KT / S)
    const int KT = p.K / C::KS / sp.S;
    if (sp.S > 1) {
        const int64_t k_off = static_cast<int64_t>(sp.chunk) * KT * C::ROWB;
#pragma unroll
        for (int i = 0; i < A_INSTR; ++i) a_src[i] += k_off;
        w_base += static_cast<int64_t>(sp.chunk) * KT * w_stage_bytes;
    }
    // copy group j of K tile kt: groups of 4 (or 2) consecutive 1 KB copies
    constexpr int AG = A_INSTR >= 4 ? 4 : A_INSTR, BG = B_INSTR >= 4 ? 4 : B_INSTR;
    static_assert(A_INSTR % AG == 0 && B_INSTR % BG == 0, "whole copy groups");
    constexpr int NGROUPS = A_INSTR / AG + B_INSTR / BG;
    auto copy = [&](int kt, int j) {
        const uint32_t st = static_cast<uint32_t>(kt % STAGES) * C::STAGE_BYTES;
        const int64_t off = static_cast<int64_t>(kt) * C::ROWB;
        if (j < A_INSTR / AG) {
            const uint8_t* g[AG];
#pragma unroll
            for (int i = 0; i < AG; ++i) g[i] = a_src[j * AG + i] + off;
            copy_group<AG>(g, a_dst + st + j * AG * 1024);
        } else {
            const int jb = j - A_INSTR / AG;
            const int64_t woff = static_cast<int64_t>(kt) * w_stage_bytes;
            const uint8_t* g[BG];
#pragma unroll
            for (int i = 0; i < BG; ++i) g[i] = w_base + b_off[jb * BG + i] + woff;
            copy_group<BG>(g, b_dst + st + jb * BG * 1024);
        }
    };
    auto issue = [&](int kt) {
#pragma unroll
        for (int j = 0; j < NGROUPS; ++j) copy(kt, j);
    };

    f32x16_t acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = f32x16_t{};

    const int arow = wm * (BM / C::WM), brow = wn * (BN / C::WN);
    // A block holds an expert's items, then padding rows (sorted id >= R). The
    // wave's 32-row groups past the last one with a real row are not multiplied:
    // their accumulators stay 0 (the SiLU epilogue writes 0 to padding rows
    // anyway), and their LDS reads and MFMAs are left out. The copies and the
    // barriers are the same for every wave.
    // ACT: the tile's sorted ids and on-input weights, loaded here so that their
    // latency passes under the K loop instead of opening the epilogue
    int rid[ACT ? TM : 1];
    float ralpha[ACT ? TM : 1];
    if constexpr (ACT) {
#pragma unroll
        for (int i = 0; i < TM; ++i) rid[i] = p.sorted[m0 + arow + i * 32 + r32];
#pragma unroll
        for (int i = 0; i < TM; ++i) ralpha[i] = (rid[i] < p.R && p.act_on_input) ? p.act_weights[rid[i]] : 1.0f;
    }
    int live = TM;
    if (p.live_ids != nullptr) {
        live = 0;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = ACT ? rid[ACT ? i : 0] : p.live_ids[m0 + arow + i * 32 + r32];
            if (ballot64(r < p.R) != 0) live = i + 1;
        }
    }
    struct Frag {
        bf16x8_t a[TM], b[TN];
    };
    auto stage_ptr = [&](int kt) { return smem + (kt % STAGES) * (C::STAGE_BYTES / 16); };
    auto read_a = [&](int kt, int ks, Frag& f, int i) {
        f.a[i] = __builtin_bit_cast(bf16x8_t, stage_ptr(kt)[C::swz(arow + i * 32 + r32, 2 * ks + half)]);
    };
    auto read_b = [&](int kt, int ks, Frag& f, int i) {
        f.b[i] = __builtin_bit_cast(bf16x8_t,
                                    (stage_ptr(kt) + C::A_BYTES / 16)[C::swz(brow + i * 32 + r32, 2 * ks + half)]);
    };

    // The K loop for LV live 32-row groups (LV = 0: the wave only copies).
    auto k_loop = [&](auto lv) {
        constexpr int LV = decltype(lv)::value;
        auto read = [&](int kt, int ks, Frag& f) {
            if constexpr (LV > 0) {
#pragma unroll
                for (int i = 0; i < TN; ++i) read_b(kt, ks, f, i);
#pragma unroll
                for (int i = 0; i < LV; ++i) read_a(kt, ks, f, i);
            }
        };
        auto mma = [&](const Frag& f) {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int tm = 0; tm < LV; ++tm)
                    acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[tn], f.a[tm], acc[tn][tm], 0, 0, 0);
        };
        // spread the LV + TN fragment reads of the next K step over this step's
        // LV * TN MFMAs
        auto interleave = [&]() {
            if constexpr (LV > 0) dma::interleave_step<0, LV + TN, LV * TN>();
        };

        // MFMAs of fragment set f, one weight row (tn) at a time. Between the rows
        // go the LDS reads of the next K tile's first fragment set (into g) and the
        // copies of tile `ck`: no long run of VMEM or LDS issues holds back the
        // MFMAs queued behind it (a wave issues in order), and every MFMA only
        // depends on LDS reads issued long before it.
        auto mma_and_prefetch = [&](const Frag& f, int next_kt, Frag& g, int ck) {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
                for (int tm = 0; tm < LV; ++tm)
                    acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[tn], f.a[tm], acc[tn][tm], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (LV > 0) {
                    read_b(next_kt, 0, g, tn);
#pragma unroll
                    for (int i = tn * LV / TN; i < (tn + 1) * LV / TN; ++i) read_a(next_kt, 0, g, i);
                }
                if (ck >= 0) {
#pragma unroll
                    for (int j = tn * NGROUPS / TN; j < (tn + 1) * NGROUPS / TN; ++j) copy(ck, j);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // Pipeline per K tile kt (NKS K steps, fragment sets alternating 0, 1):
        //   for each K step but the last: read the next step's set while the MFMAs
        //   of this step run;
        //   last step: wait for tile kt+1, barrier, then its MFMAs interleaved with
        //   the reads of tile kt+1's first set and the copies of tile kt+S-1 into
        //   the stage of tile kt-1.
        // S-2 tiles are in flight while tile kt is multiplied.
        Frag fs[2];
        for (int kt = 0; kt < STAGES - 1 && kt < KT; ++kt) issue(kt);
        wait_barrier<C::L>(min(STAGES - 2, KT - 1));
        read(0, 0, fs[0]);
        auto steps_but_last = [&](int kt) {
#pragma unroll
            for (int ks = 0; ks + 1 < NKS; ++ks) {
                read(kt, ks + 1, fs[(ks + 1) & 1]);
                mma(fs[ks & 1]);
                interleave();
            }
        };
        // (the last K tile is peeled off, so the reads of the next tile's first
        // set are unconditional and the LDS counter waits stay exact)
        for (int kt = 0; kt + 1 < KT; ++kt) {
            steps_but_last(kt);
            // tile kt+1 landed (tiles kt+2 .. kt+S-2 may still be in flight);
            // every wave has finished reading the stage of tile kt-1
            wait_barrier<C::L>(min(STAGES - 3, KT - 2 - kt));
            mma_and_prefetch(fs[1], kt + 1, fs[0], kt + STAGES - 1 < KT ? kt + STAGES - 1 : -1);
        }
        steps_but_last(KT - 1);
        mma(fs[1]);
    };
    static_assert(TM <= 4, "live row group counts 0 .. 4");
    if (live >= TM) {
        k_loop(std::integral_constant<int, TM>{});
    } else if (live == 0) {
        k_loop(std::integral_constant<int, 0>{});
    } else if constexpr (TM > 1) {
        if (live == 1) {
            k_loop(std::integral_constant<int, 1>{});
        } else if constexpr (TM > 2) {
            if (live == 2) k_loop(std::integral_constant<int, 2>{});
            else if constexpr (TM > 3) k_loop(std::integral_constant<int, 3>{});
        }
    }

    // no copies are in flight; once every wave is past its last fragment
    // read, the ring holds the epilogue staging
    __syncthreads();
    constexpr int TMP = TM >= 2 ? 2 : 1;  // 32-row tiles per staging pass
    static_assert(C::NW * TMP * 32 * (TN * 64 + 16) <= STAGES * C::STAGE_BYTES, "staging fits the ring");
    if constexpr (SPLIT) {
        if (sp.slot >= 0) {
            // Every K range writes its fp32 partial tile (in accumulator register
            // order: index ((wave, tn, tm, r), lane)), then counts itself in; the
            // last to arrive sums the S partials in range order (deterministic)
            // and stores the tile. Ordering: every wave waits until its own partial
            // stores are complete (acknowledged by L2; the workgroup barrier alone
            // does not wait for them on this target), then the barrier, then thread
            // 0's counter update, an agent-scope release (L2 written back, so the
            // partials are visible to every CU, on any XCD) and acquire (the last
            // arrival then sees every other range's partials). One release and one
            // acquire per workgroup, not per wave.
            // The ranges of a tile are still placed on one XCD, but only so that
            // their partials meet in one L2; correctness does not depend on it.
            constexpr int TILE_F = C::NW * TN * TM * 16 * 64;
            static_assert(TILE_F == BM * BN, "one partial per output");
            float* part = p.part + static_cast<int64_t>(sp.slot) * TILE_F;
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        part[(((wave * TN + tn) * TM + tm) * 16 + r) * 64 + lane] = acc[tn][tm][r];
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            int* cnt = p.part_cnt + sp.tail_tile;
            int* flag = reinterpret_cast<int*>(smem);
            if (tid == 0) *flag = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            const int arrived = *flag;
            if (arrived != sp.S - 1) return;
            const float* first = p.part + static_cast<int64_t>(sp.slot - sp.chunk) * TILE_F;
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int64_t idx = (((wave * TN + tn) * TM + tm) * 16 + r) * 64 + lane;
                        float v = first[idx];
                        for (int c = 1; c < sp.S; ++c) v += first[static_cast<int64_t>(c) * TILE_F + idx];
                        acc[tn][tm][r] = v;
                    }
            __syncthreads();  // the flag's LDS word is reused by the staging below
        }
    }
    if constexpr (ACT) {
        // SiLU-and-mul: column tiles 2j (gate) and 2j + 1 (up) of a wave hold the same
        // outputs; both are rounded to bf16 (the values GEMM1 would store), then
        // z = alpha * SiLU(g) * u in fp32 (alpha = the routed item's weight in on-input
        // mode, else 1; padding rows 0), written in place into column tile j
        static_assert(TN % 2 == 0 && (BN / C::WN) % 64 == 0, "gate/up column tile pairs");
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const bool real = rid[tm] < p.R;
            const float alpha = ralpha[tm];
#pragma unroll
            for (int j = 0; j < TN / 2; ++j)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float g = bf16_to_f32(f32_to_bf16(acc[2 * j][tm][i]));
                    const float u = bf16_to_f32(f32_to_bf16(acc[2 * j + 1][tm][i]));
                    acc[j][tm][i] = real ? alpha * silu_f32(g) * u : 0.0f;
                }
        }
        static_assert(C::NW * TMP * 32 * (TN / 2 * 64 + 16) <= STAGES * C::STAGE_BYTES, "staging fits the ring");
        store_block<TM, TN / 2, TMP>(reinterpret_cast<const f32x16_t(&)[TN / 2][TM]>(acc),
                                     reinterpret_cast<uint8_t*>(smem) + wave * (TMP * 32 * (TN / 2 * 64 + 16)),
                                     reinterpret_cast<uint8_t*>(p.C), m0 + arow, n0 + brow / 2, p.ldc_bytes,
                                     p.N, lane);
    } else {
        store_block<TM, TN, TMP>(acc, reinterpret_cast<uint8_t*>(smem) + wave * (TMP * 32 * (TN * 64 + 16)),
                                 reinterpret_cast<uint8_t*>(p.C), m0 + arow, n0 + brow, p.ldc_bytes, p.N, lane);
    }
}

// ---------------------------------------------------------------------------
// fp8 W8A8 (e4m3 weights with one scale per 128x128 block, activations with
// one scale per row and 128 columns; "fused_moe.py analysis", "FP8 W8A8",
// block-wise; "DeepGEMM FusedMoE on Blackwell", 1.1 step 4 and 2.5). One K
// stage is 128 e4m3 of every row, i.e. one scale group: two
// v_mfma_scale_f32_32x32x64_f8f6f4 steps (unit block scales) sum it into a
// partial tile, which is then added to the fp32 accumulator times
// token scale x weight-block scale.
//
// Same direct-to-LDS copy ring as the bf16 kernel, with two waves per SIMD
// (eight per workgroup): the per-stage scaling is vector-ALU work that one
// wave does while the other wave of its SIMD keeps the matrix core busy.
// With 64 x 64 outputs per wave every accumulator stays in an
// architectural register, so the scaling needs no accumulator-register moves.
//
// The kernel is persistent: one workgroup per CU walks its share of the
// tiles as one continuous stream of K stages, so the copies of the next
// tile's first stages are in flight while the current tile finishes and
// writes its outputs (no pipeline fill or store drain between tiles).
// Workgroup h runs on XCD h % 8 and takes every (grid/8)-th tile of that
// XCD's contiguous range of the logical tile order.
//
// Per stage the ring slot holds the A and B rows plus the scales: wave 0
// copies the stage's 128 row scales (the activation scales are stored
// group-major by sorted position, 512 contiguous bytes), wave 1 copies the
// tile's weight-block scales of that K block (one 4-byte copy). For a
// gathered A, wave 0 also copies the next tile's 128 sorted ids into one of
// three id slots when the current tile's first stage goes out, so switching
// tiles (and the SiLU epilogue) reads the row indices from LDS. The loop
// issues no other vector memory instruction, so the explicit vmcnt counts
// hold (an id copy only makes one wait stricter).
//
// With ACT the tile is GEMM1 with SiLU-and-mul fused into the epilogue
// ("DeepGEMM FusedMoE on Blackwell", 2.6.4, done here in the GEMM's
// epilogue instead of a separate pass): its 256 weight rows are 128 gate
// rows and the matching 128 up rows, interleaved in 32-row groups so that
// every wave holds the gate and the up value of the same outputs (tile
// rows 64w..64w+31 gate, 64w+32..64w+63 up, of output columns 32w..32w+31).
// The epilogue rounds both to bf16 (the value GEMM1 would store), forms
// z = alpha * SiLU(g) * u in fp32, and quantises each row's 128 outputs to
// e4m3 with scale amax / 448, exactly as the separate activation pass does,
// then writes z and its scales; h never reaches HBM.
namespace f8 {

// FP4W: E2M1 weights, two per byte (W4A8): a stage's weight rows are 64 bytes
template <int BM_, int BN_, int WM_, int WN_, int STAGES_, bool FP4W_ = false>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NW = WM_ * WN_, STAGES = STAGES_;
    static constexpr bool FP4W = FP4W_;
    static constexpr int ROWB = 128, CH = 8, ROWS_PER_COPY = 8;
    static constexpr int BROWB = FP4W ? 64 : 128, BCH = BROWB / 16, B_ROWS_PER_COPY = 1024 / BROWB;
    static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * BROWB;
    static constexpr int SCALE_OFF = A_BYTES + B_BYTES;   // 1 KB of row scales, then weight scales
    static constexpr int WSCALE_OFF = SCALE_OFF + 1024;
    static constexpr int EPI_BYTES = 32 * ((BN / WN / 32) * 64 + 16);  // one 32-row pass of a wave's epilogue
    // a stage also stages a tile's output, so it holds at least the epilogue's bytes
    static constexpr int STAGE_BYTES = (SCALE_OFF + 2048 > NW * EPI_BYTES ? SCALE_OFF + 2048
                                        : (NW * EPI_BYTES + 1023) / 1024 * 1024);
    static constexpr int IDS_OFF = STAGES * STAGE_BYTES;  // three 1 KB slots of sorted ids
    static constexpr int LDS_BYTES = IDS_OFF + 3072;
    static constexpr int A_INSTR = A_BYTES / 1024 / NW, B_INSTR = B_BYTES / 1024 / NW;
    static constexpr int L = A_INSTR + B_INSTR;  // copies per wave per stage (waves 0 and 1: L + 1)
    static constexpr int WBLOCKS = BN / 128;     // weight-scale rows per tile
    static constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    static constexpr bool FP8_OUT = true;                  // SiLU epilogue output: e4m3 z
    static_assert(A_INSTR * NW * 1024 == A_BYTES && B_INSTR * NW * 1024 == B_BYTES, "whole copies");
    static_assert((A_INSTR == 2 || A_INSTR == 4) && (B_INSTR == 2 || B_INSTR % 4 == 0), "copy groups");
    static_assert(BM == 128, "one 1 KB copy carries the 128 row scales and the 128 sorted ids");
    static_assert(BN % 128 == 0 && 128 % (BN / WN) == 0 && WBLOCKS <= 64,
                  "a wave's weight rows lie in one 128-row scale block");
    static_assert(STAGES >= 3 && LDS_BYTES <= 160 * 1024, "fits gfx950 LDS");
    static_assert(STAGE_BYTES % 1024 == 0, "stages keep the 1 KB swizzle alignment");
    static_assert(3 * (L + 2) <= 63, "vmcnt range");
    static_assert(NW * EPI_BYTES <= STAGE_BYTES, "epilogue staging fits one ring slot");
    static_assert(BN == 256 && WN == 4 && TN == 2, "SiLU epilogue: a wave's two column tiles are gate and up");
    static_assert(BM * (128 + 16) + 4 * BM * 4 <= STAGE_BYTES, "SiLU epilogue staging fits one ring slot");
    // 128-byte rows, 16-byte chunks XOR-swizzled by (row / 2) % 8
    __device__ static __forceinline__ int swz(int row, int chunk) { return row * CH + (chunk ^ ((row >> 1) & 7)); }
    // weight rows: as above, or 64-byte rows swizzled by (row / 4) % 4
    __device__ static __forceinline__ int bswz(int row, int chunk) {
        return FP4W ? row * BCH + (chunk ^ ((row >> 2) & 3)) : swz(row, chunk);
    }
};

// one 1 KB copy (16 bytes per lane) to LDS address `lds`
__device__ __forceinline__ void copy1(const void* g, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(g)
        : "memory");
}

// one 256-byte copy (4 bytes per lane) to LDS address `lds`
__device__ __forceinline__ void copy1_dword(const void* g, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(g)
        : "memory");
}

}  // namespace f8

// MX (MXFP8, "DeepGEMM FusedMoE on Blackwell", MXFP8 1x32): activations and weights
// carry one E8M0 scale per 32 K values, which the scaled MFMA applies per lane (a
// lane's 32 K bytes of an operand are exactly one such block), so the stage sums go
// straight into the accumulators. The scales arrive packed four to a word
// (blocks 4 kt .. 4 kt + 3 of a row), MN-major: the activations' [K/128, cap] by
// sorted position, the weights' [E, K/128, N]; a stage copies 128 and 256 words.
// The SiLU epilogue quantises z per 32 columns (one wave's slice of a 128-column
// block) to E4M3 with an E8M0 scale byte.
// FMT 0: fp8 with fp32 128x128 weight-block and per-128 activation scales; 1: MXFP8;
// 2: W4A8 (E2M1 weights with E8M0 scales per 32, applied by the instruction, times
// fp8 activations whose fp32 per-128 scale is folded per stage as in FMT 0).
template <class C, bool GATHER, bool ACT, int FMT>
__global__ __launch_bounds__(C::NW * 64) void expert_gemm_fp8_kernel(GemmArgs p) {
    static_assert(!ACT || GATHER, "the SiLU epilogue belongs to GEMM1");
    static_assert(C::FP4W == (FMT == 2), "E2M1 weight tiles for W4A8 only");
    constexpr bool MX = FMT == 1;       // E8M0 scales on both operands
    constexpr bool WMX = FMT != 0;      // E8M0 scales on the weights
    constexpr int BM = C::BM, BN = C::BN, STAGES = C::STAGES, TM = C::TM, TN = C::TN;
    constexpr int A_INSTR = C::A_INSTR, B_INSTR = C::B_INSTR, L = C::L;
    extern __shared__ __attribute__((aligned(1024))) u32x4_t smem[];
    uint8_t* const lds8 = reinterpret_cast<uint8_t*>(smem);
    const uint32_t lds_base = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) u32x4_t*)smem));

    // ---- this workgroup's tiles --------------------------------------------
    constexpr int TILE_COLS = ACT ? BN / 2 : BN;  // output columns per tile
    const int n_tiles = (p.N + TILE_COLS - 1) / TILE_COLS;
    const int m_real = min(p.m_blocks, (*p.npp + BM - 1) / BM);
    const int total = m_real * n_tiles;
    const int per_xcd = gridDim.x >> 3, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int q8 = total >> 3, rem = total & 7;
    const int x0 = xcd * q8 + min(xcd, rem), xn = q8 + (xcd < rem ? 1 : 0);
    const int my_n = slot < xn ? (xn - slot + per_xcd - 1) / per_xcd : 0;
    if (my_n == 0) return;
    const int KT = p.K / 128;
    const int G = my_n * KT;  // stages of this workgroup
    // logical order: that of tile_of (expert-aligned groups, column by column)
    auto tile_pos = [&](int i, int& mb, int& nb) {
        TilePos tp;
        tile_in_group(p, x0 + slot + i * per_xcd, n_tiles, m_real, tp);
        mb = tp.mb;
        nb = tp.nb;
    };
    using cint = __attribute__((address_space(4))) const int32_t;  // scalar loads
    const cint* eids = (const cint*)(p.expert_ids);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int r32 = lane & 31, half = lane >> 5;
    const int cp_row = lane / C::CH, cp_slot = lane % C::CH;

    // ---- issue side: sources of the tile whose stages are being copied ------
    const uint8_t* a_src[A_INSTR];
    const uint8_t* w_tile = nullptr;
    int32_t b_off[B_INSTR];
    const float* sc_src = nullptr;  // wave 0: row scales; wave 1: weight-block scales
    auto ids_slot = [&](int i) { return reinterpret_cast<const int32_t*>(lds8 + C::IDS_OFF + (i % 3) * 1024); };
    auto setup_issue = [&](int i) {
        int mb, nb;
        tile_pos(i, mb, nb);
        const int e = eids[mb];
        const int64_t m0 = static_cast<int64_t>(mb) * BM;
        const int n0 = nb * TILE_COLS;
#pragma unroll
        for (int c = 0; c < A_INSTR; ++c) {
            const int row = (wave * A_INSTR + c) * C::ROWS_PER_COPY + cp_row;
            const int chunk = C::swz(row, cp_slot) - row * C::CH;
            int64_t src_row = m0 + row;
            if constexpr (GATHER) {
                const int r = i == 0 ? p.sorted[m0 + row] : ids_slot(i)[row];
                src_row = r < p.R ? r / p.topk : 0;  // padding rows read token 0
            }
            a_src[c] = reinterpret_cast<const uint8_t*>(p.A) + src_row * p.lda_bytes + chunk * 16;
        }
        w_tile = reinterpret_cast<const uint8_t*>(p.W) + static_cast<int64_t>(e) * p.w_expert_bytes;
#pragma unroll
        for (int c = 0; c < B_INSTR; ++c) {
            const int row = (wave * B_INSTR + c) * C::B_ROWS_PER_COPY + lane / C::BCH;
            const int chunk = C::bswz(row, lane % C::BCH) - row * C::BCH;
            // ACT: tile row r is gate (r / 32 even) or up row of output column
            // n0 + 32 * (r / 64) + r % 32
            const int wrow = ACT ? ((row >> 5) & 1) * p.N + n0 + (row >> 6) * 32 + (row & 31)
                                 : min(n0 + row, p.N - 1);
            b_off[c] = wrow * static_cast<int32_t>(p.ldw_bytes) + chunk * 16;
        }
        if (wave == 0) {
            sc_src = p.a_scale + m0 + (lane & 31) * 4;
        } else if constexpr (WMX) {
            // 256 weight-row scale words of K block 0: lane l takes 4 of them. ACT:
            // lanes 0-31 the gate rows n0.., lanes 32-63 the up rows N + n0..; else
            // rows n0 + 4 l (clamped: rows past N are never stored)
            const int nw = ACT ? 2 * p.N : p.N;
            const int r0 = ACT ? (lane >> 5) * p.N + n0 + (lane & 31) * 4 : min(n0 + lane * 4, nw - 4);
            sc_src = p.w_scale + static_cast<int64_t>(e) * p.w_scale_expert + r0;
        } else {
            // lane b < WBLOCKS: weight-block row n0/128 + b (rows past N repeat the
            // last); ACT: lane 0 the gate block, lane 1 the up block
            const int b = ACT ? (lane & 1) * (p.N / 128) + n0 / 128
                              : min(n0 / 128 + min(lane, C::WBLOCKS - 1), p.N / 128 - 1);
            sc_src = p.w_scale + static_cast<int64_t>(e) * p.w_scale_expert +
                     static_cast<int64_t>(b) * p.scale_groups;
        }
    };
    // copies of stage gs (tile gs / KT, K block gs % KT), in two parts
    const uint32_t a_dst = __builtin_amdgcn_readfirstlane(lds_base + wave * A_INSTR * 1024);
    const uint32_t b_dst = __builtin_amdgcn_readfirstlane(lds_base + C::A_BYTES + wave * B_INSTR * 1024);
    constexpr int BG = B_INSTR >= 4 ? 4 : B_INSTR;
    auto issue_a = [&](int gs) {
        const int i = gs / KT, kt = gs - i * KT;
        if (kt == 0) {
            if (gs > 0) setup_issue(i);
            // the next tile's sorted ids, for its setup (read after this stage has landed)
            if (GATHER && wave == 0 && i + 1 < my_n) {
                int mb1, nb1;
                tile_pos(i + 1, mb1, nb1);
                f8::copy1(p.sorted + static_cast<int64_t>(mb1) * BM + (lane & 31) * 4,
                          lds_base + C::IDS_OFF + ((i + 1) % 3) * 1024);
            }
        }
        const uint32_t st = static_cast<uint32_t>(gs % STAGES) * C::STAGE_BYTES;
        const int64_t off = static_cast<int64_t>(kt) * C::ROWB;
        const uint8_t* g[A_INSTR];
#pragma unroll
        for (int c = 0; c < A_INSTR; ++c) g[c] = a_src[c] + off;
        dma::copy_group<A_INSTR>(g, a_dst + st);
    };
    auto issue_rest = [&](int gs) {
        const int kt = gs % KT;
        const uint32_t st = static_cast<uint32_t>(gs % STAGES) * C::STAGE_BYTES;
        const int64_t off = static_cast<int64_t>(kt) * C::BROWB;
#pragma unroll
        for (int j = 0; j < B_INSTR / BG; ++j) {
            const uint8_t* g[BG];
#pragma unroll
            for (int c = 0; c < BG; ++c) g[c] = w_tile + b_off[j * BG + c] + off;
            dma::copy_group<BG>(g, b_dst + st + j * BG * 1024);
        }
        if (wave == 0)
            f8::copy1(sc_src + static_cast<int64_t>(kt) * p.a_scale_ld, lds_base + st + C::SCALE_OFF);
        else if (wave == 1 && WMX)
            f8::copy1(sc_src + static_cast<int64_t>(kt) * (ACT ? 2 * p.N : p.N), lds_base + st + C::WSCALE_OFF);
        else if (wave == 1)
            f8::copy1_dword(sc_src + kt, lds_base + st + C::WSCALE_OFF);
    };
    auto wait_barrier = [&](int newer) {
        if (wave <= 1)
            dma::wait_barrier<L + 1>(newer);
        else
            dma::wait_barrier<L>(newer);
    };

    // ---- compute side -------------------------------------------------------
    f32x16_t acc[TN][TM], part[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = f32x16_t{};
    const int arow = wm * (BM / C::WM), brow = wn * (BN / C::WN);
    struct Frag {
        i32x8_t a[TM], b[TN];
    };
    auto stage_ptr = [&](int g) { return smem + (g % STAGES) * (C::STAGE_BYTES / 16); };
    // lane (r32, half) holds K chunks 4ks + half and 4ks + 2 + half (16 bytes each):
    // the matrix core reads a lane's first four registers as K [16 half, +16) of the
    // 64-wide step and the last four as K [32 + 16 half, +16), and scales K [0, 32)
    // and [32, 64) with the scale bytes of lanes of half 0 and half 1; so this order
    // makes each hardware scale block one 32-wide block of K in memory
    auto frag = [&](const u32x4_t* base, int row, int ks) {
        const u32x4_t lo = base[C::swz(row, 4 * ks + half)];
        const u32x4_t hi = base[C::swz(row, 4 * ks + 2 + half)];
        return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    // E2M1 weights: the instruction reads 4 registers, and unlike the e4m3 operand a
    // lane holds 32 consecutive K values there, K [32 half, +32) of the 64-wide step
    // (a probe pairing one-hot rows of both operands): chunk 2 ks + half, whole
    auto frag_w4 = [&](const u32x4_t* base, int row, int ks) {
        const u32x4_t c = base[C::bswz(row, 2 * ks + half)];
        return i32x8_t{(int)c[0], (int)c[1], (int)c[2], (int)c[3], 0, 0, 0, 0};
    };
    auto read = [&](int g, int ks, Frag& f) {
        const u32x4_t* st = stage_ptr(g);
#pragma unroll
        for (int i = 0; i < TN; ++i)
            f.b[i] = C::FP4W ? frag_w4(st + C::A_BYTES / 16, brow + i * 32 + r32, ks)
                             : frag(st + C::A_BYTES / 16, brow + i * 32 + r32, ks);
#pragma unroll
        for (int i = 0; i < TM; ++i) f.a[i] = frag(st, arow + i * 32 + r32, ks);
    };
    // formats 0/0 = e4m3 x e4m3; E8M0 block scale 127 = 1.0
    auto mma = [&](const Frag& f, bool first) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
                part[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    f.b[tn], f.a[tm], first ? f32x16_t{} : part[tn][tm], 0, 0, 0, 127, 0, 127);
    };
    // W4A8: format 4 (E2M1) weights with their E8M0 scale per lane, e4m3 activations
    // at unit scale (their fp32 scale is folded after the stage)
    auto mma_w4 = [&](const Frag& f, int g, int ks, bool first) {
        const uint32_t* sw = reinterpret_cast<const uint32_t*>(stage_ptr(g) + C::WSCALE_OFF / 16);
        const int shift = 8 * (2 * ks + half);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int r = brow + tn * 32 + r32;
            const int wi = ACT ? ((r >> 5) & 1) * 128 + (r >> 6) * 32 + (r & 31) : r;
            const int bsc = static_cast<int>((sw[wi] >> shift) & 0xffu);
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
                part[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    f.b[tn], f.a[tm], first ? f32x16_t{} : part[tn][tm], 4, 0, 0, bsc, 0, 127);
        }
    };
    // MX: each lane's E8M0 bytes (K block 4 kt + 2 ks + half) of its activation row
    // and its weight row; the MFMA scales the products, the sums accumulate directly.
    // ACT weight tile row r is gate row (r / 64) * 32 + r % 32 (r / 32 even) or that
    // up row, whose words sit at [0, 128) and [128, 256) of the stage's scales.
    auto mma_mx = [&](const Frag& f, int g, int ks) {
        const uint32_t* sa = reinterpret_cast<const uint32_t*>(stage_ptr(g) + C::SCALE_OFF / 16);
        const uint32_t* sw = reinterpret_cast<const uint32_t*>(stage_ptr(g) + C::WSCALE_OFF / 16);
        const int shift = 8 * (2 * ks + half);
        int asc[TM];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) asc[tm] = static_cast<int>((sa[arow + tm * 32 + r32] >> shift) & 0xffu);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int r = brow + tn * 32 + r32;
            const int wi = ACT ? ((r >> 5) & 1) * 128 + (r >> 6) * 32 + (r & 31) : r;
            const int bsc = static_cast<int>((sw[wi] >> shift) & 0xffu);
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
                acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    f.b[tn], f.a[tm], acc[tn][tm], 0, 0, 0, bsc, 0, asc[tm]);
        }
    };
    // scale of tile row arow + tm*32 + r32 times the wave's weight-block scale, from
    // stage g's slot (ACT: column tile tn = 0 holds gate rows, tn = 1 up rows, each
    // its own block), and the fold of a stage's sums into the accumulators
    auto stage_scales = [&](int g, float (&sc)[TN][TM]) {
        const float* sx = reinterpret_cast<const float*>(stage_ptr(g) + C::SCALE_OFF / 16);
        const float* swb = reinterpret_cast<const float*>(stage_ptr(g) + C::WSCALE_OFF / 16);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const float x = sx[arow + tm * 32 + r32];
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) sc[tn][tm] = FMT == 2 ? x : x * swb[ACT ? tn : brow / 128];
        }
    };
    auto apply = [&](const float (&sc)[TN][TM]) {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[tn][tm][r] += part[tn][tm][r] * sc[tn][tm];
    };

    // SiLU-and-mul epilogue of one tile (ACT): `ws` is a free ring slot, `ids`
    // the tile's 128 sorted ids, m0 its first row, nb its 128-column block of z.
    // Lane (r32, half) holds, for row arow + tm*32 + r32, the gate (tn = 0) and
    // up (tn = 1) sums of columns 32*wn + 8q + 4*half + j.
    auto act_epilogue = [&](const f32x16_t (&a)[TN][TM], uint8_t* ws, const int32_t* ids, int64_t m0,
                            int nb) {
        constexpr int ZP = 128 + 16;                       // staged z row pitch (bytes)
        float* amax_part = reinterpret_cast<float*>(ws + BM * ZP);  // [4][BM]
        float v[TM][16];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const int rl = arow + tm * 32 + r32;
            const int r = ids[rl];
            const bool real = r < p.R;
            const float alpha = (real && p.act_on_input) ? p.act_weights[r] : 1.0f;
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float gt = bf16_to_f32(f32_to_bf16(a[0][tm][i]));
                const float up = bf16_to_f32(f32_to_bf16(a[1][tm][i]));
                v[tm][i] = real ? alpha * silu_f32(gt) * up : 0.0f;
                m = fmaxf(m, fabsf(v[tm][i]));
            }
            m = fmaxf(m, __shfl_xor(m, 32, 64));  // the other half of the row's 32 columns
            if (half == 0) amax_part[wn * BM + rl] = m;
        }
        // barriers that wait only for LDS traffic: the copies in flight stay in flight
        auto lds_barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
        if constexpr (MX) {
            // the row's 32 columns of this wave are one MX block: E8M0 scale byte wn of
            // the row's word in z_scale [I/128, cap], codes E4M3(v / scale)
            uint8_t* zsc = reinterpret_cast<uint8_t*>(p.z_scale);
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
                const int rl = arow + tm * 32 + r32;
                float m = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[tm][i]));
                m = fmaxf(m, __shfl_xor(m, 32, 64));
                const uint32_t code = mx_scale_code(m, 448.0f);
                const float inv = ldexpf(1.0f, 127 - static_cast<int>(code));
                if (half == 0) zsc[(static_cast<int64_t>(nb) * p.z_scale_ld + m0 + rl) * 4 + wn] = static_cast<uint8_t>(code);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float c4[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) c4[j] = fminf(fmaxf(v[tm][4 * q + j] * inv, -448.0f), 448.0f);
                    *reinterpret_cast<uint32_t*>(ws + rl * ZP + wn * 32 + 8 * q + 4 * half) =
                        cvt_e4m3x4(c4[0], c4[1], c4[2], c4[3]);
                }
            }
            lds_barrier();
            uint8_t* zc = reinterpret_cast<uint8_t*>(p.C);
#pragma unroll
            for (int pass = 0; pass < BM / (8 * C::NW); ++pass) {
                const int rl = (pass * C::NW + wave) * 8 + lane / 8;
                const u32x4_t z16 = *reinterpret_cast<const u32x4_t*>(ws + rl * ZP + (lane % 8) * 16);
                __builtin_nontemporal_store(
                    z16, reinterpret_cast<u32x4_t*>(zc + (m0 + rl) * p.ldc_bytes + nb * 128 + (lane % 8) * 16));
            }
        } else if constexpr (C::FP8_OUT) {
            lds_barrier();
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
                const int rl = arow + tm * 32 + r32;
                const float m = fmaxf(fmaxf(amax_part[rl], amax_part[BM + rl]),
                                      fmaxf(amax_part[2 * BM + rl], amax_part[3 * BM + rl]));
                const float s = m / 448.0f;
                if (wn == 0 && half == 0) p.z_scale[nb * p.z_scale_ld + m0 + rl] = s;
                // codes: v times the rounded 1 / s, or the quotient where s is below the
                // smallest normal float (as the separate activation pass does)
                float c16[16];
                if (!(s >= 0x1p-126f)) {
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        c16[j] = m == 0.0f ? 0.0f : fminf(fmaxf(v[tm][j] / s, -448.0f), 448.0f);
                } else {
                    const float inv = 1.0f / s;
#pragma unroll
                    for (int j = 0; j < 16; ++j) c16[j] = fminf(fmaxf(v[tm][j] * inv, -448.0f), 448.0f);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<uint32_t*>(ws + rl * ZP + wn * 32 + 8 * q + 4 * half) =
                        cvt_e4m3x4(c16[4 * q], c16[4 * q + 1], c16[4 * q + 2], c16[4 * q + 3]);
            }
            lds_barrier();
            // 128 rows x 128 bytes: 8 lanes per row, 8 rows per wave per pass
            uint8_t* zc = reinterpret_cast<uint8_t*>(p.C);
#pragma unroll
            for (int pass = 0; pass < BM / (8 * C::NW); ++pass) {
                const int rl = (pass * C::NW + wave) * 8 + lane / 8;
                const u32x4_t z16 = *reinterpret_cast<const u32x4_t*>(ws + rl * ZP + (lane % 8) * 16);
                __builtin_nontemporal_store(
                    z16, reinterpret_cast<u32x4_t*>(zc + (m0 + rl) * p.ldc_bytes + nb * 128 + (lane % 8) * 16));
            }
        }
    };

    // Per stage g: wait until stage g has landed and every wave is done with
    // stage g-1, send the copies of stage g+S-1 into g-1's slot, then the
    // MFMAs and the scaling of stage g. After a tile's last stage its
    // outputs go out through that stage's slot, which the copies reuse only
    // after the next barrier.
    setup_issue(0);
    if (ACT && wave == 0) {  // tile 0's sorted ids, for its epilogue
        int mb0, nb0;
        tile_pos(0, mb0, nb0);
        f8::copy1(p.sorted + static_cast<int64_t>(mb0) * BM + (lane & 31) * 4, lds_base + C::IDS_OFF);
    }
    for (int gs = 0; gs < STAGES - 1 && gs < G; ++gs) {
        issue_a(gs);
        issue_rest(gs);
    }
    Frag f0, f1;
    int c_tile = 0, kt = 0;
    // The waves of the upper half share each SIMD with one of the lower half. They
    // fold a stage's sums into the accumulators at the start of the next stage
    // (their scales read in its own stage, before its slot is refilled), so that
    // one wave's multiply-adds run while the other's MFMAs do instead of both
    // waves folding at once after their MFMAs. Each output still adds its stages in
    // order, so the bits do not change; a tile's last stage is folded before its
    // epilogue.
    const bool late = wave >= C::NW / 2;
    float held[TN][TM];
    bool pending = false;
    for (int g = 0; g < G; ++g) {
        wait_barrier(min(STAGES - 2, G - 1 - g));
        const int gs = g + STAGES - 1;
        const bool more = gs < G;
        read(g, 0, f0);
        if (more) issue_a(gs);
        read(g, 1, f1);
        if constexpr (!MX) {
            if (late && pending) apply(held);
        }
        if constexpr (MX) {
            mma_mx(f0, g, 0);
            if (more) issue_rest(gs);
            mma_mx(f1, g, 1);
        } else if constexpr (FMT == 2) {
            mma_w4(f0, g, 0, true);
            if (more) issue_rest(gs);
            mma_w4(f1, g, 1, false);
        } else {
            mma(f0, true);
            if (more) issue_rest(gs);
            mma(f1, false);
        }
        if constexpr (!MX) {
            float sc[TN][TM];
            stage_scales(g, sc);
            if (late) {
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                    for (int tm = 0; tm < TM; ++tm) held[tn][tm] = sc[tn][tm];
                pending = true;
            } else {
                apply(sc);
            }
        }
        if (++kt == KT) {
            if constexpr (!MX) {
                if (late) apply(held);
                pending = false;
            }
            kt = 0;
            int mb, nb;
            tile_pos(c_tile, mb, nb);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // slot g is free
            uint8_t* free_slot = lds8 + (g % STAGES) * C::STAGE_BYTES;
            if constexpr (ACT)
                act_epilogue(acc, free_slot, ids_slot(c_tile), static_cast<int64_t>(mb) * BM, nb);
            else
                store_block<TM, TN, 1>(acc, free_slot + wave * C::EPI_BYTES, reinterpret_cast<uint8_t*>(p.C),
                                       static_cast<int64_t>(mb) * BM + arow, nb * BN + brow, p.ldc_bytes,
                                       p.N, lane);
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int j = 0; j < TM; ++j) acc[i][j] = f32x16_t{};
            ++c_tile;
        }
    }
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// one workgroup per CU (multiple of 8 so that every XCD gets the same count); the
// count is cached per device (relaxed atomics: concurrent first calls store the
// same value)
int persistent_grid() {
    static std::atomic<int> cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int c = cus[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) n = 256;
        c = n / 8 * 8;
        cus[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

template <class C, bool GATHER, bool ACT, int FMT>
hipError_t launch_fp8_as(const GemmArgs& a, hipStream_t stream) {
    const size_t lds = C::LDS_BYTES;
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(expert_gemm_fp8_kernel<C, GATHER, ACT, FMT>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (err != hipSuccess) return err;
    const dim3 grid(static_cast<unsigned>(persistent_grid()));
    hipLaunchKernelGGL((expert_gemm_fp8_kernel<C, GATHER, ACT, FMT>), grid, dim3(C::NW * 64), lds, stream, a);
    return hipGetLastError();
}

template <class C, int FMT>
hipError_t launch_fp8_fmt(const GemmArgs& a, hipStream_t stream) {
    if (a.act) return a.sorted ? launch_fp8_as<C, true, true, FMT>(a, stream) : hipErrorInvalidValue;
    return a.sorted ? launch_fp8_as<C, true, false, FMT>(a, stream) : launch_fp8_as<C, false, false, FMT>(a, stream);
}

template <class C, bool GATHER, bool ACT>
hipError_t launch_dma_as(const GemmArgs& a, hipStream_t stream) {
    const int cols = ACT ? C::BN / 2 : C::BN;
    const int n_tiles = (a.N + cols - 1) / cols;
    // the split-K tail adds one round of workgroups (at most n_cu + 32 of them)
    const int extra = (!GATHER && a.part != nullptr) ? a.n_cu + 32 : 0;
    const dim3 grid(static_cast<unsigned>(a.m_blocks * n_tiles + extra));
    const size_t lds = C::STAGES * C::STAGE_BYTES;
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(expert_gemm_dma_kernel<C, GATHER, ACT>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((expert_gemm_dma_kernel<C, GATHER, ACT>), grid, dim3(C::NW * 64), lds, stream, a);
    return hipGetLastError();
}

template <class C>
hipError_t launch_dma(const GemmArgs& a, hipStream_t stream) {
    if (a.w_packed && C::ROWB != 64) return hipErrorInvalidValue;  // one 16 x 32 tile per copy
    if (a.act) return a.sorted ? launch_dma_as<C, true, true>(a, stream) : hipErrorInvalidValue;
    return a.sorted ? launch_dma_as<C, true, false>(a, stream) : launch_dma_as<C, false, false>(a, stream);
}

// 128 tokens x 512 weight rows, 64-byte rows, 1 x 8 waves of 128 x 64 (two per SIMD)
using Dma128 = dma::Cfg<128, 512, 1, 4, 64, 8>;
// 256 tokens x 256 weight rows, 64-byte rows, 2 x 4 waves of 128 x 64 (two per SIMD:
// one wave's MFMAs cover the other's waits)
using Dma256 = dma::Cfg<256, 256, 2, 5, 64, 8>;
// fp8: 128 tokens x 256 weight rows, 2 x 4 waves of 64 x 64, 3 stages
using Fp8x128 = f8::Cfg<128, 256, 2, 4, 3>;
// W4A8: the same tile over 64-byte E2M1 weight rows
using W4x128 = f8::Cfg<128, 256, 2, 4, 3, true>;

// GemmArgs::mx: 0 fp8 blocks, 1 MXFP8, 2 W4A8
hipError_t launch_fp8(const GemmArgs& a, hipStream_t stream) {
    if (a.mx == 2) return launch_fp8_fmt<W4x128, 2>(a, stream);
    return a.mx ? launch_fp8_fmt<Fp8x128, 1>(a, stream) : launch_fp8_fmt<Fp8x128, 0>(a, stream);
}

template <int BM, int BN, bool FP8>
hipError_t launch_tile(const GemmArgs& a, hipStream_t stream) {
    const int n_tiles = (a.N + BN - 1) / BN;
    const dim3 grid(static_cast<unsigned>(a.m_blocks * n_tiles));
    if (a.sorted)
        hipLaunchKernelGGL((expert_gemm_kernel<BM, BN, FP8, true>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((expert_gemm_kernel<BM, BN, FP8, false>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

int concurrent_tiles() { return persistent_grid(); }

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_i32_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

int gemm_supported_block_m(int bm) { return bm == 32 || bm == 64 || bm == 128 || bm == 256; }

bool gemm_act_supported(int block_m, bool fp8, int K) {
    if (!fp8) return block_m == 16 || block_m == 128 || block_m == 256;
    return block_m == 128 && K >= 128 * (Fp8x128::STAGES - 1);
}

hipError_t launch_grouped_gemm(const GemmArgs& a, int block_m, bool fp8, hipStream_t stream) {
    if (a.act && !gemm_act_supported(block_m, fp8, a.K)) return hipErrorInvalidValue;
    if (!fp8) {
        switch (block_m) {
            case 32: return launch_tile<32, 256, false>(a, stream);
            case 64: return launch_tile<64, 512, false>(a, stream);
            case 128: return launch_dma<Dma128>(a, stream);
            case 256: return launch_dma<Dma256>(a, stream);
        }
    } else {
        switch (block_m) {
            case 32: return launch_tile<32, 256, true>(a, stream);
            case 64: return launch_tile<64, 256, true>(a, stream);
            // the streaming kernel needs K / 128 >= STAGES - 1 (one tile's stages fill the
            // ring start); a single 128-wide K block takes the register-staged kernel
            case 128:
                if (a.K >= 128 * (Fp8x128::STAGES - 1)) return launch_fp8(a, stream);
                return a.act ? hipErrorInvalidValue : launch_tile<128, 256, true>(a, stream);
        }
    }
    return hipErrorInvalidValue;
}
