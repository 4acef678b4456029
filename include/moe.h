/*
 * moe.h -- C ABI of the gfx950 (MI355X) fused MoE expert forward.
 *
 * The layer computes, for every token t with hidden state x_t,
 *     y_t = sum over the token's top-k experts e of
 *           alpha_{t,e} * W2_e ( SiLU(G_e x_t) * (U_e x_t) )
 * where G_e and U_e are rows [0, I) and [I, 2I) of w13[e]
 * ("fused_moe.py analysis" (FlagDoc), sections 1.1-1.4;
 *  "DeepGEMM FusedMoE on Blackwell (vLLM)", section 1.1, steps 2-8).
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless marked "host".
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call is
 *     stream-ordered, never synchronises the host, and reads no device data
 *     on the host.
 *   - The library allocates nothing and keeps no state beyond a per-device
 *     cache of the compute-unit count: scratch space comes from the caller's
 *     workspace. Calls are thread-safe.
 *   - Arguments are validated on the host before any launch; a failing check
 *     returns its status and launches nothing.
 *   - Tensors are dense, row-major and contiguous. bf16 is stored as its
 *     16-bit pattern, e4m3 as OCP float8_e4m3fn bytes.
 */
#ifndef MOE_GFX950_H
#define MOE_GFX950_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden visibility; these declarations are its
 * exported interface. */
#pragma GCC visibility push(default)

typedef enum {
    MOE_OK = 0,
    MOE_E_INVALID = 1,     /* null pointer, negative size, topk outside [1, min(E, 32)]
                              (E: num_global_experts when it is set) */
    MOE_E_UNSUPPORTED = 2, /* E > 256, H or I not a multiple of 128, unknown block_m,
                              dtype or weight layout, fp8 with block_m 16 or 256, MXFP8
                              other than block_m 128 with H, I >= 256, the
                              tiled layout other than bf16 with block_m 16, 128 or 256,
                              more than 2^31 routed rows, one expert's w13 of 2 GiB
                              or more, or GEMM grids (row blocks x 128-column tiles)
                              of 2^31 workgroups or more */
    MOE_E_WORKSPACE = 3,   /* workspace_bytes < moe_workspace_bytes(p) */
    MOE_E_HIP = 4          /* a kernel launch failed (hipGetLastError) */
} moe_status_t;

typedef enum {
    MOE_W_BF16 = 0,              /* bf16 weights, bf16 activations, fp32 accumulate */
    MOE_W_FP8_E4M3_BLOCK128 = 1, /* e4m3 weights with one fp32 scale per 128x128 block;
                                    activations quantised per token per 128 columns */
    MOE_W_MXFP8 = 2,             /* MXFP8 ("DeepGEMM FusedMoE on Blackwell", MXFP8 1x32):
                                    e4m3 weights and activations, one E8M0 scale (2^(c-127))
                                    per 32 K values, the smallest power of two s with
                                    amax <= 448 s; z is requantised the same way. Weight
                                    scales as packed words from moe_pack_mx_scales;
                                    block_m 128 with H, I >= 256 */
    MOE_W_W4A8_MXFP4 = 3         /* W4A8 ("DeepGEMM FusedMoE on Blackwell", W4A8 MXFP4):
                                    E2M1 weights, two per byte (element 2i in the low
                                    nibble: w13 [E, 2I, H/2], w2 [E, H, I/2] uint8), one
                                    E8M0 scale per 32 K values (packed words as for MXFP8),
                                    times e4m3 activations with one fp32 scale per 128
                                    columns, as MOE_W_FP8_E4M3_BLOCK128 quantises x and z;
                                    block_m 128 with H, I >= 256 */
} moe_wdtype_t;

/*
 * Element order of w13 and w2 in memory. Weights are prepared once after
 * loading into the order the kernel reads best ("DeepGEMM FusedMoE on
 * Blackwell", 2.8 (c): expert weights and scales are post-processed into the
 * kernel's packed layout; "vLLM modular_kernel.py notes", 10.1: expert
 * weights may arrive in a 6-D packed layout).
 *   MOE_LAYOUT_ROWS:  w [E, N, K] row-major (K contiguous).
 *   MOE_LAYOUT_TILED: the same E*N*K values in 16-row x 32-column tiles of
 *     1 KB, row-major inside a tile, tiles ordered by row block then column
 *     block:  tiled[e][n/16][k/32][n%16][k%32] = w[e][n][k],
 *     i.e. w.view(E, N/16, 16, K/32, 32).permute(0, 1, 3, 2, 4).
 *     Every 1 KB tile is what one load instruction of the kernels reads (16
 *     rows x 32 columns), and a 16-row block is one contiguous run along K,
 *     where row-major weights give 64 bytes from each of 16 rows 2*K bytes
 *     apart. bf16 weights with block_m 16, 128 or 256. Written by
 *     moe_pack_weights; results are bit-identical to MOE_LAYOUT_ROWS.
 */
typedef enum {
    MOE_SCORING_SOFTMAX = 0,
    MOE_SCORING_SIGMOID = 1
} moe_scoring_t;

typedef enum {
    MOE_LAYOUT_ROWS = 0,
    MOE_LAYOUT_TILED = 1
} moe_wlayout_t;

/* Sizes and options of one fused_experts call. */
typedef struct {
    int64_t M;         /* tokens */
    int32_t H;         /* hidden size (K of GEMM1, N of GEMM2) */
    int32_t I;         /* intermediate size per expert (w13 has 2I rows) */
    int32_t E;         /* experts */
    int32_t topk;      /* experts per token */
    int32_t block_m;   /* rows per expert block: 16 or 256 (bf16 only), 32, 64 or 128 */
    int32_t wdtype;    /* moe_wdtype_t */
    int32_t apply_router_weight_on_input; /* 0: weight the expert outputs in the final sum;
                                             1: weight the SiLU-and-mul output instead */
    int32_t weight_layout; /* moe_wlayout_t of w13 and w2 (0: row-major) */
    int32_t num_global_experts; /* expert-parallel shard: the range of topk_ids,
                                   E being the experts held here (fused_experts_ep);
                                   0 otherwise. topk <= num_global_experts */
    int32_t chunk_tokens; /* > 0: fused_experts(_ep) runs the layer on chunks of this
                             many tokens, one after another on the stream, and the
                             workspace is sized for one chunk ("fused_moe.py
                             analysis", section 6: 16K-token chunks bound the
                             intermediate buffers); 0: one pass over all M tokens */
} moe_problem_t;

/*
 * Router: softmax over the E logits of each token, then the top-k experts
 * ("vLLM modular_kernel.py notes", section 3, fused_topk with
 *  scoring_func="softmax"; "fused_moe.py analysis", section 1.1).
 *
 *   logits        [M, E] fp32
 *   topk_ids      [M, topk] int32 out: slot j holds the j-th largest logit; equal
 *                 logits go to the lower expert index
 *   topk_weights  [M, topk] fp32 out: softmax probability of the chosen expert;
 *                 when `renormalize` != 0, divided by the sum over the k chosen
 * Limits: 1 <= E <= 256, 1 <= topk <= min(E, 32). M == 0 launches nothing.
 */
moe_status_t moe_topk(const float *logits, int64_t M, int32_t E, int32_t topk,
                      int32_t renormalize, int32_t *topk_ids, float *topk_weights,
                      void *stream);

/*
 * Grouped / sigmoid router ("vLLM modular_kernel.py notes", section 3:
 * fused_topk with scoring_func "softmax" or "sigmoid"; the grouped routing
 * arguments of apply_monolithic: num_expert_group, topk_group,
 * e_score_correction_bias, routed_scaling_factor). Per token:
 *   score u_e   softmax over the E logits, or sigmoid(s_e)
 *   key         the logit s_e; with a correction bias (sigmoid only),
 *               fp32( sigmoid(s_e) evaluated in double ) + bias[e] in fp32
 *   groups      num_expert_group groups of E / G consecutive experts; a group
 *               scores its largest key, or with a bias the sum of its two
 *               largest keys; the topk_group best groups are kept (lower group
 *               index on ties)
 *   selection   the topk largest keys among the kept groups' experts, slots in
 *               descending key order (lower expert index on ties)
 *   weights     u of the chosen (the bias never enters a weight), divided by
 *               their sum when `renormalize`, times routed_scaling_factor
 *   logits [M, E] fp32; e_score_correction_bias [E] fp32 or NULL;
 *   topk_ids [M, topk] int32 out; topk_weights [M, topk] fp32 out.
 * num_expert_group = topk_group (e.g. 1, 1) is plain top-k over all experts.
 * MOE_E_INVALID: G or topk_group outside [1, E] with E % G == 0 and
 * topk_group <= G, topk above topk_group * E / G or 32, a bias with softmax
 * scoring or with groups of one expert; MOE_E_UNSUPPORTED: E > 256 or G > 64.
 */
moe_status_t moe_topk_grouped(const float *logits, int64_t M, int32_t E, int32_t topk,
                              int32_t scoring, int32_t renormalize, int32_t num_expert_group,
                              int32_t topk_group, const float *e_score_correction_bias,
                              float routed_scaling_factor, int32_t *topk_ids, float *topk_weights,
                              void *stream);

/*
 * Host-only, pure: the number of rows the expert-sorted layout may need,
 * roundup(R + min(R, E) * (block_m - 1), block_m) with R = M * topk
 * ("DeepGEMM FusedMoE on Blackwell", section 2.6.1, the bound used when the
 * per-expert counts are not known on the host). Returns -1 on bad arguments.
 */
int64_t moe_align_capacity(int64_t M, int32_t topk, int32_t E, int32_t block_m);

/*
 * Align / permute ("fused_moe.py analysis", "moe_align_block_size";
 * "DeepGEMM FusedMoE on Blackwell", section 2.6.2). Routed item r = t*topk + j.
 *
 *   topk_ids               [M, topk] int32, values in [0, E); other values are
 *                          skipped (not placed, inv_perm = -1)
 *   sorted_token_ids       [cap] int32 out: items grouped by expert (ascending),
 *                          ascending r inside a group, each group padded to a
 *                          multiple of block_m with the sentinel R; the tail
 *                          [num_tokens_post_padded, cap) also holds R
 *   expert_ids             [cap / block_m] int32 out: expert of each block, -1
 *                          for blocks past the padded total
 *   num_tokens_post_padded [1] int32 out: sum over experts of roundup(n_e, block_m)
 *   inv_perm               [M, topk] int32 out: the row of sorted_token_ids that
 *                          holds item r
 * cap = moe_align_capacity(M, topk, E, block_m). The layout is deterministic.
 * With M == 0 only num_tokens_post_padded is written (0); the other pointers
 * may then be NULL.
 */
moe_status_t moe_align_block_size(const int32_t *topk_ids, int64_t M, int32_t topk, int32_t E,
                                  int32_t block_m, int32_t *sorted_token_ids,
                                  int32_t *expert_ids, int32_t *num_tokens_post_padded,
                                  int32_t *inv_perm, void *stream);

/*
 * Align on one rank of an expert-parallel shard: topk_ids hold global ids in
 * [0, num_global_experts); expert_map as for fused_experts_ep. Items of
 * experts not held here get no row and inv_perm -1; the segments are those of
 * the E local experts in local order. Sizes and outputs as for
 * moe_align_block_size (cap = moe_align_capacity(M, topk, E, block_m)).
 */
moe_status_t moe_align_block_size_ep(const int32_t *topk_ids, int64_t M, int32_t topk,
                                     int32_t num_global_experts, const int32_t *expert_map,
                                     int32_t E, int32_t block_m, int32_t *sorted_token_ids,
                                     int32_t *expert_ids, int32_t *num_tokens_post_padded,
                                     int32_t *inv_perm, void *stream);

/*
 * Dynamic fp8 quantisation of activations, per row and per 128 columns
 * ("DeepGEMM FusedMoE on Blackwell", section 2.5 / 1.1 step 4;
 *  "fused_moe.py analysis", "FP8 W8A8").
 *
 *   x      [rows, cols] bf16, cols a multiple of 128
 *   q      [rows, cols] e4m3 out: RNE(clamp(x / scale, -448, 448))
 *   scale  [rows, cols / 128] fp32 out: amax of the group / 448 (0 for an
 *          all-zero group, whose codes are then 0)
 */
moe_status_t moe_quant_fp8_groups(const void *x, int64_t rows, int32_t cols, void *q,
                                  float *scale, void *stream);

/*
 * MXFP8 activations ("DeepGEMM FusedMoE on Blackwell", MXFP8 1x32, dynamic
 * activations): per row, each 32 columns share one E8M0 scale code c (the
 * smallest power of two s = 2^(c-127) with amax <= 448 s; 0 for an all-zero
 * block) and the codes are e4m3(v / s), round to nearest even.
 *   x [rows, cols] bf16; q [rows, cols] e4m3 out; scale [rows, cols / 32] uint8 out
 * cols must be a multiple of 128.
 */
moe_status_t moe_quant_mx_groups(const void *x, int64_t rows, int32_t cols, void *q, void *scale,
                                 void *stream);

/*
 * MXFP8 weight scales into the order the kernels read ("DeepGEMM FusedMoE on
 * Blackwell", 2.8 (c): scales are post-processed after loading into the
 * kernel's packed, MN-major layout, four E8M0 exponents to a 32-bit word):
 *   which = 1: scale [E, 2I, H/32] uint8 -> scale_packed [E, H/128, 2I] uint32
 *   which = 2: scale [E, H, I/32]  uint8 -> scale_packed [E, I/128, H]  uint32
 * byte b of word (e, j, n) holds the scale of K block 4 j + b of row n.
 * Requires p->wdtype MOE_W_MXFP8 or MOE_W_W4A8_MXFP4; buffers 4-byte aligned and distinct.
 */
moe_status_t moe_pack_mx_scales(const moe_problem_t *p, int32_t which, const void *scale,
                                void *scale_packed, void *stream);

/* Host-only, pure: bytes of device workspace fused_experts needs for `p`
 * (0 when M == 0). */
size_t moe_workspace_bytes(const moe_problem_t *p);

/*
 * The fused expert forward: align, GEMM1 (gathered token rows x w13[e]),
 * SiLU-and-mul, GEMM2 (x w2[e]), then the top-k weighted sum in fp32, cast
 * to bf16 ("fused_moe.py analysis", sections 1.2-1.3 and "fused_moe_kernel";
 * "DeepGEMM FusedMoE on Blackwell", sections 2.6.1-2.6.5).
 *
 *   x             [M, H] bf16
 *   w13           [E, 2I, H] bf16 or e4m3 (per p->wdtype); rows [0, I) gate,
 *                 [I, 2I) up
 *   w13_scale     [E, 2I/128, H/128] fp32 for fp8 (NULL is MOE_E_INVALID), ignored for bf16;
 *                 for MXFP8 the packed words [E, H/128, 2I] uint32 of moe_pack_mx_scales
 *                 (w2_scale: [E, I/128, H]), passed through the same pointer
 *   w2            [E, H, I] bf16 or e4m3
 *   w2_scale      [E, H/128, I/128] fp32 for fp8 (NULL is MOE_E_INVALID), ignored for bf16
 *                 (w13 and w2 in the element order p->weight_layout names)
 *   topk_ids      [M, topk] int32, topk_weights [M, topk] fp32 (as from moe_topk)
 *   y             [M, H] bf16 out; may be the same buffer as x (in place)
 *   workspace     device scratch of at least moe_workspace_bytes(p) bytes,
 *                 256-byte aligned; its contents on entry do not matter
 * M == 0 returns MOE_OK and launches nothing. For bf16 weights with block_m 16 and
 * at most 1024 routed items (M * topk), GEMM1 builds the aligned layout itself, so
 * no separate align kernel runs; the layout is moe_align_block_size's either way.
 */
moe_status_t fused_experts(const moe_problem_t *p, const void *x, const void *w13,
                           const float *w13_scale, const void *w2, const float *w2_scale,
                           const int32_t *topk_ids, const float *topk_weights, void *y,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * fused_experts for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * arguments as fused_experts without the workspace; the layer's scratch lives
 * in a static device array of the library, 64 MiB on every GPU the library runs
 * on, held until the process ends. Nothing is allocated or freed by the call.
 *   Returns MOE_E_WORKSPACE when the problem needs more than 64 MiB of scratch:
 *   moe_workspace_bytes(p) without its second-GEMM split-K part, i.e. with
 *   cap = moe_align_capacity(M', topk, E, block_m) and M' = min(M, chunk_tokens
 *   if set), about cap * (max(2 I, H) * 2 + I * 2) + 4 (cap + M' topk) bytes for
 *   bf16 (decode-sized problems and token chunks fit; set chunk_tokens for
 *   larger M). MOE_E_INVALID for num_global_experts != 0 (no expert map here).
 *   The second GEMM sums every tile's K range in one pass (the split-K tail of
 *   fused_experts needs 64 MiB of partials on its own), so with bf16 weights and
 *   block_m 128 / 256 the bits can differ from fused_experts' in the last place;
 *   elsewhere they are the same.
 *   Every call on one GPU uses that GPU's one array: calls that overlap on a GPU
 *   (on different streams, or from different threads without ordering) race and
 *   give undefined results. Everything the layer reads from the array it first
 *   writes in the same call, so its contents between calls do not matter.
 */
moe_status_t fused_experts_static(const moe_problem_t *p, const void *x, const void *w13,
                                  const float *w13_scale, const void *w2, const float *w2_scale,
                                  const int32_t *topk_ids, const float *topk_weights, void *y,
                                  void *stream);

/*
 * The same layer on one rank of an expert-parallel shard ("vLLM
 * modular_kernel.py notes", the expert_map argument of fused_experts: a table
 * from global expert ids to this rank's experts, -1 for experts held by other
 * ranks; "DeepGEMM FusedMoE on Blackwell", 2.6.2 and 2.6.5: ep_scatter and
 * ep_gather skip the items and slots of remote experts).
 *   p->num_global_experts  G > 0, the range of topk_ids; p->E the experts held
 *                 here, whose weights w13 [E, 2I, H] and w2 [E, H, I] are passed
 *   expert_map    [G] int32: the local index in [0, E) of global expert g, or -1
 *                 (entries outside [0, E), and ids outside [0, G), count as not
 *                 held here)
 *   y[t, :] = bf16( sum over the token's slots j whose expert is held here of
 *                   alpha_{t,j} * expert output ): this rank's part of the
 *             layer, which a combine across ranks adds up (not done here).
 * Everything else as for fused_experts; moe_workspace_bytes(p) sizes the
 * workspace. p->num_global_experts must be 0 for fused_experts.
 */
moe_status_t fused_experts_ep(const moe_problem_t *p, const int32_t *expert_map, const void *x,
                              const void *w13, const float *w13_scale, const void *w2,
                              const float *w2_scale, const int32_t *topk_ids,
                              const float *topk_weights, void *y, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * Batched-experts form ("vLLM modular_kernel.py notes", 6.x and 7.1: after a
 * low-latency dispatch the activations of a rank arrive as one batch of up to
 * max_M rows per local expert, [E, max_M, H], with per-expert token counts;
 * "DeepGEMM FusedMoE on Blackwell", 2.5: the masked grouped GEMM computes only
 * the first count rows of each batch, and the combine applies the router
 * weights):
 *   out[e, i, :] = bf16( W2_e ( SiLU(G_e a[e, i]) * (U_e a[e, i]) ) )
 *                  for i < expert_num_tokens[e], unweighted; 0 for the other rows.
 *   p             M = max_M (rows per batch), E = experts (batches), topk = 1,
 *                 apply_router_weight_on_input = 0, num_global_experts = 0;
 *                 H, I, block_m, wdtype and weight_layout as for fused_experts
 *   a             [E, max_M, H] bf16; rows past a count are not read
 *   expert_num_tokens [E] int32 (device); values above max_M act as max_M,
 *                 negative ones as 0
 *   w13, w13_scale, w2, w2_scale as for fused_experts
 *   out           [E, max_M, H] bf16 out (must not overlap a)
 *   workspace     at least moe_batched_workspace_bytes(p) bytes, 256-aligned
 * The rows run through the same kernels as fused_experts with top-1 routing
 * (row e * max_M + i routed to expert e when it is counted, else nowhere).
 * M == 0 returns MOE_OK and launches nothing.
 */
size_t moe_batched_workspace_bytes(const moe_problem_t *p);  /* host, pure; 0 if invalid */
moe_status_t moe_batched_experts(const moe_problem_t *p, const void *a,
                                 const int32_t *expert_num_tokens, const void *w13,
                                 const float *w13_scale, const void *w2, const float *w2_scale,
                                 void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The stages of fused_experts, for callers that build their own pipeline or
 * time the stages one by one. fused_experts launches exactly these kernels:
 * for fp8, moe_quant_fp8_groups(x) and moe_permute_scales after the align;
 * GEMM1 then activation as moe_expert_gemm_act where available, else
 * moe_expert_gemm(1) and moe_silu_and_mul; moe_expert_gemm(2); the reduce.
 * `p` has the same meaning as for fused_experts; cap is
 * moe_align_capacity(M, topk, E, block_m); the layout arrays are those of
 * moe_align_block_size. Rows at or past num_tokens_post_padded are skipped.
 * Weights are in the element order p->weight_layout names.
 */

/*
 * Grouped expert GEMM over the expert-sorted layout ("fused_moe.py
 * analysis", 1.3 and "fused_moe_kernel"; "DeepGEMM FusedMoE on Blackwell",
 * 2.6.3 and 2.6.5): every block b of block_m rows uses expert expert_ids[b].
 *   which = 1: c[pos, 0:2I] = a[sorted_token_ids[pos] / topk, :] . w13[e]^T,
 *              a = x [M, H] (bf16 or e4m3); padding rows (sorted id >= M*topk)
 *              are never consumed, and their values in c are unspecified
 *   which = 2: c[pos, 0:H] = a[pos, :] . w2[e]^T, a = z [cap, I] (bf16 or
 *              e4m3); sorted_token_ids may be NULL (every row is then computed);
 *              given, it marks the padding rows, whose values in c are again
 *              unspecified (groups of padding rows alone may be left out)
 *   c [cap, N] bf16 out (fp32 accumulation, one rounding at the end).
 *   fp8: a_scale is [K/128, cap] fp32, group-major and indexed by sorted
 *   position (a_scale[g * cap + pos] belongs to row pos of the layout; built
 *   by moe_permute_scales for which = 1 and by moe_silu_and_mul for which = 2);
 *   w_scale is [E, N/128, K/128]. Every 128-wide K block's partial sum is
 *   multiplied by a_scale[block * cap + pos] * w_scale[e, n/128, block].
 *   workspace (device, may be NULL): at least moe_expert_gemm_workspace_bytes(p)
 *   bytes, else MOE_E_WORKSPACE. With it, which = 2 on bf16 weights (block_m
 *   128 / 256) cuts the tiles of a last, at most half-full round of tiles into
 *   2 or 4 K ranges, summed in fp32 in a fixed order: the result is
 *   deterministic, and is what fused_experts computes (it always passes one);
 *   without it the K sum runs in one pass, and the bits can differ in the last
 *   place. Calls that share a workspace must not overlap.
 */
size_t moe_expert_gemm_workspace_bytes(const moe_problem_t *p);  /* host, pure; 0 if none is used */
moe_status_t moe_expert_gemm(const moe_problem_t *p, int32_t which, const void *a,
                             const float *a_scale, const void *w, const float *w_scale,
                             const int32_t *sorted_token_ids, const int32_t *expert_ids,
                             const int32_t *num_tokens_post_padded, void *c, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * SiLU-and-mul ("DeepGEMM FusedMoE on Blackwell", 2.6.4; "fused_moe.py
 * analysis", apply_moe_activation): z[pos, i] = SiLU(h[pos, i]) * h[pos, I+i]
 * in fp32 (times topk_weights[item] when apply_router_weight_on_input),
 * padding rows set to 0.
 *   h [cap, 2I] bf16; z [cap, I] bf16 out, or for fp8 z [cap, I] e4m3 plus
 *   z_scale [I/128, cap] fp32 out (per-row, per-128 dynamic quantisation;
 *   the scale of row pos and group g at z_scale[g * cap + pos]).
 */
moe_status_t moe_silu_and_mul(const moe_problem_t *p, const void *h,
                              const int32_t *sorted_token_ids, const float *topk_weights,
                              const int32_t *num_tokens_post_padded, void *z, float *z_scale,
                              void *stream);

/*
 * GEMM1 with SiLU-and-mul fused into its epilogue: the result of
 * moe_expert_gemm(which = 1) followed by moe_silu_and_mul, bit for bit,
 * without writing h. Available where moe_expert_gemm_act_supported(p) is 1
 * (host-only, pure): bf16 weights with block_m 16, 128 or 256, or fp8 weights
 * with block_m 128 and H >= 256; otherwise MOE_E_UNSUPPORTED. fused_experts
 * uses it where it is available.
 *   bf16: x [M, H] bf16, z [cap, I] bf16 out; x_scale, w13_scale and z_scale
 *   are unused (may be NULL).
 *   fp8: x [M, H] e4m3, x_scale [H/128, cap] (from moe_permute_scales), w13
 *   and w13_scale as for fused_experts, z [cap, I] e4m3 out, z_scale
 *   [I/128, cap] fp32 out (as moe_silu_and_mul writes them).
 *   topk_weights [M, topk]: alpha when apply_router_weight_on_input.
 */
int32_t moe_expert_gemm_act_supported(const moe_problem_t *p);
moe_status_t moe_expert_gemm_act(const moe_problem_t *p, const void *x, const float *x_scale,
                                 const void *w13, const float *w13_scale,
                                 const int32_t *sorted_token_ids, const int32_t *expert_ids,
                                 const int32_t *num_tokens_post_padded, const float *topk_weights,
                                 void *z, float *z_scale, void *stream);

/*
 * The fp8 GEMM1 activation scales in the expert-sorted row order
 * ("DeepGEMM FusedMoE on Blackwell", 2.5 and 2.6.2: the per-token group
 * scales travel with the permuted rows, stored column-major for the GEMM):
 *   scale  [M, H/128] fp32, as from moe_quant_fp8_groups(x); for MXFP8 the
 *          [M, H/32] E8M0 bytes of moe_quant_mx_groups, read as [M, H/128]
 *          32-bit words (moved as bit patterns)
 *   out    [H/128, cap] fp32 out: out[g * cap + pos] = scale[sorted_token_ids[pos] / topk, g]
 *          for pos < num_tokens_post_padded, 0 at padding positions; later
 *          positions are not written
 */
moe_status_t moe_permute_scales(const moe_problem_t *p, const float *scale,
                                const int32_t *sorted_token_ids,
                                const int32_t *num_tokens_post_padded, float *out, void *stream);

/*
 * Weighted unpermute-reduce ("DeepGEMM FusedMoE on Blackwell", 2.6.5,
 * ep_gather; "vLLM modular_kernel.py notes", 7.3.3):
 *   y[t, :] = bf16( sum_j a_j * o[inv_perm[t, j], :] ), fp32, slots in order,
 *   a_j = topk_weights[t, j] (1 when apply_router_weight_on_input);
 *   slots with inv_perm < 0 are skipped. o [cap, H] bf16, y [M, H] bf16 out.
 */
moe_status_t moe_unpermute_reduce(const moe_problem_t *p, const void *o, const int32_t *inv_perm,
                                  const float *topk_weights, void *y, void *stream);

/*
 * Weight preparation: rewrite one weight tensor from MOE_LAYOUT_ROWS into
 * MOE_LAYOUT_TILED (a permutation: the bits of every element are kept).
 *   which = 1: w = w13 [E, 2I, H];  which = 2: w = w2 [E, H, I]   (bf16)
 *   w_packed: the same number of bytes, out; must not overlap w.
 * p->wdtype must be MOE_W_BF16; p->M, block_m and weight_layout are not used
 * (beyond the problem's validity). Run once, before fused_experts is called
 * with weight_layout = MOE_LAYOUT_TILED.
 */
moe_status_t moe_pack_weights(const moe_problem_t *p, int32_t which, const void *w,
                              void *w_packed, void *stream);

/* Host-only: a static, human-readable name of a status code. */
const char *moe_status_string(moe_status_t s);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* MOE_GFX950_H */
