// kernels.h -- launch entry points of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;

// Arguments of one grouped expert GEMM: C[pos, n] = sum_k A[row(pos), k] * W[e(pos), n, k]
// over the expert-sorted rows pos < num_tokens_post_padded.
struct GemmArgs {
    const void* A;             // activation rows (bf16 or e4m3)
    int64_t lda_bytes;         // row stride of A
    const int32_t* sorted;     // non-null: row(pos) = sorted[pos] / topk (gather); null: row = pos
    const int32_t* live_ids;   // sorted ids read only to find row groups that hold padding alone
                               // (not multiplied); null: every row is multiplied
    int topk;
    int R;                     // M * topk; sorted entries >= R are padding
    const void* W;             // [E, N, K] weights
    int64_t w_expert_bytes;    // bytes per expert of W
    int64_t ldw_bytes;         // row stride of W
    const int32_t* expert_ids; // [m_blocks]
    const int32_t* npp;        // [1] num_tokens_post_padded (device)
    void* C;                   // [m_blocks * BM, N] bf16
    int64_t ldc_bytes;
    int N, K;
    int m_blocks;              // row blocks in the grid (capacity / block_m)
    int group_m;               // row blocks per scheduling group
    // fp8 only
    const float* a_scale;      // [K/128, a_scale_ld] group-major, by sorted position
    int64_t a_scale_ld;        // floats per group row of a_scale (the capacity)
    const float* w_scale;      // [E, N/128, K/128]
    int64_t w_scale_expert;    // floats per expert of w_scale
    int scale_groups;          // K / 128
    // SiLU-and-mul epilogue (GEMM1 only): W holds gate rows [0, N) and up rows
    // [N, 2N); C is z [rows, N] (e4m3 with z_scale, or bf16) with
    // z = alpha * SiLU(bf16(gate)) * bf16(up), padding rows 0
    int act;
    const float* act_weights;  // topk_weights [R] (alpha when act_on_input)
    int act_on_input;
    float* z_scale;            // fp8: [N/128, z_scale_ld] group-major
    int64_t z_scale_ld;
    // split-K of a last, partly filled round of tiles (non-gathered GEMM on the DMA
    // tiles): part holds part_slots fp32 partial tiles, part_cnt one arrival counter
    // per split tile (zeroed by a fill kernel before every launch); null: off
    float* part;
    int* part_cnt;
    int part_slots;
    int n_cu;                  // workgroups of this kernel that run at once (one per CU)
    // MX (E8M0 scale per 32 K values, packed four to a word): a_scale [K/128, a_scale_ld],
    // w_scale [E, K/128, N_w] words (w_scale_expert words per expert), z_scale likewise
    int mx;
    // W tiled: 16-row x 32-column tiles of 1 KB, row-major inside, ordered by row
    // block then column block (bf16; block_m 16, 128 and 256)
    int w_packed;
    // Self-aligned GEMM1 (block_m 16, SiLU epilogue): route_ids non-null. Each
    // workgroup rebuilds its row block's expert and rows from the routed ids
    // (R of them, E local experts, ids mapped through route_emap when non-null,
    // as the align kernel does), instead of reading sorted / expert_ids / npp,
    // and the workgroups of the first column tile write that layout to
    // out_sorted, out_expert_ids, out_npp and out_inv_perm for the later stages
    const int32_t* route_ids;
    const int32_t* route_emap;
    int route_E_global;
    int route_E;
    int32_t* out_sorted;
    int32_t* out_expert_ids;
    int32_t* out_npp;
    int32_t* out_inv_perm;
};

constexpr int kSelfAlignMaxR = 1024;  // routed items up to which GEMM1 may align itself

constexpr int kSplitSlots = 256;  // partial tiles of the split-K workspace

hipError_t launch_topk_softmax(const float* logits, int64_t M, int E, int k, int renormalize,
                               int32_t* ids, float* weights, hipStream_t stream);
// top-1 ids of the batched form: row e * max_M + i goes to expert e if i < counts[e]
hipError_t launch_batched_ids(const int32_t* counts, int E, int64_t max_M, int32_t* ids, hipStream_t stream);
// emap: null, or E_global entries mapping global expert ids to [0, E) or -1 (not local)
hipError_t launch_topk_grouped(const float* logits, int64_t M, int E, int k, int sigmoid,
                               int renormalize, int G, int TG, const float* bias, float scale,
                               int32_t* ids, float* weights, hipStream_t stream);
hipError_t launch_align(const int32_t* ids, int64_t R, int E, int B, int64_t cap,
                        const int32_t* emap, int E_global, int32_t* sorted, int32_t* expert_ids,
                        int32_t* npp, int32_t* inv_perm, hipStream_t stream);
int gemm_supported_block_m(int bm);
hipError_t launch_grouped_gemm(const GemmArgs& a, int block_m, bool fp8, hipStream_t stream);
bool gemm_act_supported(int block_m, bool fp8, int K);  // a fused SiLU-and-mul GEMM1 exists
hipError_t launch_stream_gemm(const GemmArgs& a, hipStream_t stream);
hipError_t launch_silu_mul_bf16(const bf16_t* h, bf16_t* z, const int32_t* sorted,
                                const float* weights, int R, int I, int64_t cap,
                                const int32_t* npp, int on_input, hipStream_t stream);
hipError_t launch_silu_mul_fp8(const bf16_t* h, uint8_t* zq, float* zs, const int32_t* sorted,
                               const float* weights, int R, int I, int64_t cap,
                               const int32_t* npp, int on_input, hipStream_t stream);  // zs [I/128, cap]
hipError_t launch_quant_fp8(const bf16_t* x, int64_t rows, int cols, uint8_t* q, float* scale,
                            hipStream_t stream);
hipError_t launch_permute_scales(const float* scale, int groups, int topk, int R,
                                 const int32_t* sorted, const int32_t* npp, int64_t cap,
                                 float* out, hipStream_t stream);
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t stream);
int concurrent_tiles();  // workgroups of the LDS-tiled GEMMs that run at once
hipError_t launch_quant_mxfp8(const bf16_t* x, int64_t rows, int cols, uint8_t* q, uint8_t* scale,
                              hipStream_t stream);  // scale [rows, cols / 32] E8M0
hipError_t launch_pack_mx_scales(const uint8_t* s, uint32_t* out, int64_t E, int N, int K, hipStream_t stream);
hipError_t launch_pack_tiled(const bf16_t* w, bf16_t* wp, int64_t E, int N, int K, hipStream_t stream);
hipError_t launch_reduce(const bf16_t* o, const int32_t* inv_perm, const float* weights, int64_t M,
                         int k, int H, int use_weights, bf16_t* y, hipStream_t stream);
