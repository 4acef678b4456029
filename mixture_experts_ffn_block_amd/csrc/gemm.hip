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

// Both operands are staged through LDS: 8 consecutive lanes load one row's
// 128-byte K slice, so every global load instruction reads whole cache lines.
// The next K tile is loaded into registers while the current one is
// multiplied, then written to the other LDS buffer (one barrier per K tile).
template <int BM, int BN, bool FP8, bool GATHER>
__global__ __launch_bounds__(256) void expert_gemm_kernel(GemmArgs p) {
    using T = Tile<BM, BN, FP8>;
    __shared__ __attribute__((aligned(16))) u32x4_t sA[2][BM * kChunks];
    __shared__ __attribute__((aligned(16))) u32x4_t sB[2][BN * kChunks];

    // ---- tile scheduling: XCD-aware remap, then grouped ordering ----------
    const int n_tiles = (p.N + BN - 1) / BN;
    const int total = p.m_blocks * n_tiles;
    // hardware id h runs on XCD h % 8; XCD x receives the contiguous logical
    // range starting at x*q + min(x, rem) (a bijection onto [0, total))
    const int hw = blockIdx.x, xcd = hw & 7;
    const int q8 = total >> 3, rem = total & 7;
    const int tile = xcd * q8 + min(xcd, rem) + (hw >> 3);
    const int per_group = p.group_m * n_tiles;
    const int first_mb = (tile / per_group) * p.group_m;
    const int rows_in_group = min(p.group_m, p.m_blocks - first_mb);
    const int mb = first_mb + (tile % per_group) % rows_in_group;
    const int nb = (tile % per_group) / rows_in_group;

    const int npp = *p.npp;
    const int64_t m0 = static_cast<int64_t>(mb) * BM;
    if (m0 >= npp) return;
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
        for (int tm = 0; tm < T::TM; ++tm) xs_row[tm] = p.a_scale + src_row_of(tm * 32 + r32) * p.scale_groups;
        // a wave's WN (<= 128, dividing 128) weight rows lie in one 128-row scale block
        static_assert(128 % T::WN == 0, "wave columns within one scale block");
        ws_row = p.w_scale + static_cast<int64_t>(e) * p.w_scale_expert +
                 static_cast<int64_t>((n0 + wave * T::WN) / 128) * p.scale_groups;
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
            for (int tm = 0; tm < T::TM; ++tm) sx[tm] = xs_row[tm][kt];
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

constexpr int ROWB = 64, CH = 4;  // tile rows are 32 bf16 = 64 bytes of K

__device__ __forceinline__ int swz64(int row, int chunk) { return row * CH + (chunk ^ ((row >> 2) & 3)); }

// Copies of 1 KB each into consecutive 1 KB LDS blocks starting at `lds`. M0
// holds the LDS base; the instruction offset is added to both the LDS and the
// global address, so copy i passes its global address minus i KB. One M0 write
// serves up to four copies (the offset field reaches 4095).
template <int N>
__device__ __forceinline__ void copy_group(const uint8_t* const (&g)[N], uint32_t lds) {
    static_assert(N == 2 || N == 4, "groups of 2 or 4 copies");
    uint32_t saved;
    if constexpr (N == 4)
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

// Geometry: BM x BN tile, WM x WN waves (4 in total), each wave 128 x 128
// (4 x 4 MFMA tiles), STAGES LDS stages of (BM + BN) x 64 bytes.
template <int BM_, int BN_, int WM_, int STAGES_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = 4 / WM_, STAGES = STAGES_;
    static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB, STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int A_INSTR = A_BYTES / 1024 / 4;  // 1 KB copies per wave
    static constexpr int B_INSTR = B_BYTES / 1024 / 4;
    static constexpr int L = A_INSTR + B_INSTR;
    static constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    static_assert(TM == 4 && TN == 4, "128 x 128 per wave");
    static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "fits gfx950 LDS");
    static_assert(STAGES - 3 <= 3, "wait_barrier covers up to 3 newer tiles");
};

}  // namespace dma

template <class C, bool GATHER>
__global__ __launch_bounds__(256) void expert_gemm_dma_kernel(GemmArgs p) {
    using namespace dma;
    constexpr int BM = C::BM, BN = C::BN, STAGES = C::STAGES, TM = C::TM, TN = C::TN;
    constexpr int A_INSTR = C::A_INSTR, B_INSTR = C::B_INSTR;
    extern __shared__ __attribute__((aligned(1024))) u32x4_t smem[];
    const uint32_t lds_base = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) u32x4_t*)smem));

    const int n_tiles = (p.N + BN - 1) / BN;
    const int total = p.m_blocks * n_tiles;
    const int hw = blockIdx.x, xcd = hw & 7;
    const int q8 = total >> 3, rem = total & 7;
    const int tile = xcd * q8 + min(xcd, rem) + (hw >> 3);
    const int per_group = p.group_m * n_tiles;
    const int first_mb = (tile / per_group) * p.group_m;
    const int rows_in_group = min(p.group_m, p.m_blocks - first_mb);
    const int mb = first_mb + (tile % per_group) % rows_in_group;
    const int nb = (tile % per_group) / rows_in_group;

    const int npp = *p.npp;
    const int64_t m0 = static_cast<int64_t>(mb) * BM;
    if (m0 >= npp) return;
    const int e = p.expert_ids[mb];
    if (e < 0) return;
    const int n0 = nb * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r32 = lane & 31, half = lane >> 5;
    const int wm = wave / C::WN, wn = wave % C::WN;

    // copy sources: a wave's copy i covers 16 rows; lane l takes row +l/4 and the
    // logical chunk stored in LDS slot l%4
    const int cp_row = lane >> 2, cp_slot = lane & 3;
    const uint8_t* a_src[A_INSTR];
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) {
        const int row = (wave * A_INSTR + i) * 16 + cp_row;
        int64_t src = m0 + row;
        if constexpr (GATHER) {
            const int r = p.sorted[m0 + row];
            src = r < p.R ? r / p.topk : 0;  // padding rows read token 0
        }
        const int chunk = cp_slot ^ ((row >> 2) & 3);
        a_src[i] = reinterpret_cast<const uint8_t*>(p.A) + src * p.lda_bytes + chunk * 16;
    }
    const uint8_t* w_base = reinterpret_cast<const uint8_t*>(p.W) + static_cast<int64_t>(e) * p.w_expert_bytes;
    int32_t b_off[B_INSTR];
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i) {
        const int row = (wave * B_INSTR + i) * 16 + cp_row;
        const int chunk = cp_slot ^ ((row >> 2) & 3);
        b_off[i] = min(n0 + row, p.N - 1) * static_cast<int32_t>(p.ldw_bytes) + chunk * 16;
    }
    // LDS destinations are wave-uniform: keep them in scalar registers
    const uint32_t a_dst = __builtin_amdgcn_readfirstlane(lds_base + wave * A_INSTR * 1024);
    const uint32_t b_dst = __builtin_amdgcn_readfirstlane(lds_base + C::A_BYTES + wave * B_INSTR * 1024);

    const int KT = p.K / 32;
    // copy group j of K tile kt: groups of 4 (or 2) consecutive 1 KB copies
    constexpr int AG = A_INSTR >= 4 ? 4 : A_INSTR, BG = 4;
    static_assert(A_INSTR % AG == 0 && B_INSTR % BG == 0, "whole copy groups");
    constexpr int NGROUPS = A_INSTR / AG + B_INSTR / BG;
    auto copy = [&](int kt, int j) {
        const uint32_t st = static_cast<uint32_t>(kt % STAGES) * C::STAGE_BYTES;
        const int64_t off = static_cast<int64_t>(kt) * ROWB;
        if (j < A_INSTR / AG) {
            const uint8_t* g[AG];
#pragma unroll
            for (int i = 0; i < AG; ++i) g[i] = a_src[j * AG + i] + off;
            copy_group<AG>(g, a_dst + st + j * AG * 1024);
        } else {
            const int jb = j - A_INSTR / AG;
            const uint8_t* g[BG];
#pragma unroll
            for (int i = 0; i < BG; ++i) g[i] = w_base + b_off[jb * BG + i] + off;
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
    struct Frag {
        bf16x8_t a[TM], b[TN];
    };
    auto read = [&](int kt, int ks, Frag& f) {
        const u32x4_t* sa = smem + (kt % STAGES) * (C::STAGE_BYTES / 16);
        const u32x4_t* sb = sa + C::A_BYTES / 16;
#pragma unroll
        for (int i = 0; i < TN; ++i) {
            f.b[i] = __builtin_bit_cast(bf16x8_t, sb[swz64(brow + i * 32 + r32, 2 * ks + half)]);
            f.a[i] = __builtin_bit_cast(bf16x8_t, sa[swz64(arow + i * 32 + r32, 2 * ks + half)]);
        }
    };
    auto mma = [&](const Frag& f) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
                acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[tn], f.a[tm], acc[tn][tm], 0, 0, 0);
    };
    // one LDS fragment read per two MFMAs, so LDS traffic is spread over the MFMA time
    auto interleave = [&]() {
#pragma unroll
        for (int i = 0; i < TM + TN; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
        }
    };

    // Pipeline per K tile kt (two K steps, F0 and F1):
    //   read F1(kt) | MFMA F0(kt) | wait tile kt+1, barrier, copy tile kt+S-1 into
    //   the stage of tile kt-1 | read F0(kt+1) | MFMA F1(kt)
    // LDS reads always overlap MFMAs of the other fragment set, and S-2 tiles are
    // in flight while tile kt is multiplied.
    // MFMAs of fragment set f, one weight row (tn) at a time. Between the rows
    // go the LDS reads of the next K tile's first fragment set (into g) and the
    // copies of tile `ck`: no long run of VMEM or LDS issues holds back the
    // MFMAs queued behind it (a wave issues in order), and every MFMA only
    // depends on LDS reads issued long before it.
    auto mma_and_prefetch = [&](const Frag& f, int next_kt, Frag& g, int ck) {
        const u32x4_t* sa = smem + (next_kt % STAGES) * (C::STAGE_BYTES / 16);
        const u32x4_t* sb = sa + C::A_BYTES / 16;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
                acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[tn], f.a[tm], acc[tn][tm], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (next_kt >= 0) {
                g.b[tn] = __builtin_bit_cast(bf16x8_t, sb[swz64(brow + tn * 32 + r32, half)]);
                g.a[tn] = __builtin_bit_cast(bf16x8_t, sa[swz64(arow + tn * 32 + r32, half)]);
            }
            if (ck >= 0) {
#pragma unroll
                for (int j = tn * NGROUPS / TN; j < (tn + 1) * NGROUPS / TN; ++j) copy(ck, j);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Pipeline per K tile kt (two K steps, fragment sets F0 and F1):
    //   read F1(kt) interleaved with MFMA F0(kt) | wait tile kt+1, barrier |
    //   MFMA F1(kt) interleaved with reads of F0(kt+1) and the copies of tile
    //   kt+S-1 into the stage of tile kt-1
    // S-2 tiles are in flight while tile kt is multiplied.
    Frag f0, f1;
    for (int kt = 0; kt < STAGES - 1 && kt < KT; ++kt) issue(kt);
    wait_barrier<C::L>(min(STAGES - 2, KT - 1));
    read(0, 0, f0);
    for (int kt = 0; kt < KT; ++kt) {
        read(kt, 1, f1);
        mma(f0);
        interleave();
        int next = -1, ck = -1;
        if (kt + 1 < KT) {
            // tile kt+1 landed (tiles kt+2 .. kt+S-2 may still be in flight);
            // every wave has finished reading the stage of tile kt-1
            wait_barrier<C::L>(min(STAGES - 3, KT - 2 - kt));
            next = kt + 1;
            if (kt + STAGES - 1 < KT) ck = kt + STAGES - 1;
        }
        mma_and_prefetch(f1, next, f0, ck);
    }

    uint8_t* c_base = reinterpret_cast<uint8_t*>(p.C);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int64_t row = m0 + arow + tm * 32 + r32;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + brow + tn * 32 + 8 * q + 4 * half;
                if (n < p.N) {
                    const f32x16_t& a = acc[tn][tm];
                    u32x2_t v{pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3])};
                    *reinterpret_cast<u32x2_t*>(c_base + row * p.ldc_bytes + n * 2) = v;
                }
            }
        }
    }
}

template <class C>
hipError_t launch_dma(const GemmArgs& a, hipStream_t stream) {
    const int n_tiles = (a.N + C::BN - 1) / C::BN;
    const dim3 grid(static_cast<unsigned>(a.m_blocks * n_tiles));
    const size_t lds = C::STAGES * C::STAGE_BYTES;
    const void* fn = a.sorted ? reinterpret_cast<const void*>(expert_gemm_dma_kernel<C, true>)
                              : reinterpret_cast<const void*>(expert_gemm_dma_kernel<C, false>);
    hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(lds));
    if (err != hipSuccess) return err;
    if (a.sorted)
        hipLaunchKernelGGL((expert_gemm_dma_kernel<C, true>), grid, dim3(256), lds, stream, a);
    else
        hipLaunchKernelGGL((expert_gemm_dma_kernel<C, false>), grid, dim3(256), lds, stream, a);
    return hipGetLastError();
}

using Dma128 = dma::Cfg<128, 512, 1, 4>;  // 128 tokens x 512 weight rows, 1 x 4 waves
using Dma256 = dma::Cfg<256, 256, 2, 5>;  // 256 tokens x 256 weight rows, 2 x 2 waves

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

int gemm_supported_block_m(int bm) { return bm == 32 || bm == 64 || bm == 128 || bm == 256; }

hipError_t launch_grouped_gemm(const GemmArgs& a, int block_m, bool fp8, hipStream_t stream) {
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
            case 128: return launch_tile<128, 256, true>(a, stream);
        }
    }
    return hipErrorInvalidValue;
}
