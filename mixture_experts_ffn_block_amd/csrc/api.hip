// api.hip -- the C ABI: validation, workspace carving and the launch sequence.
//
// fused_experts follows the pages' expert pipeline ("fused_moe.py analysis",
// fused_experts_impl: quantise the input, align, GEMM1, activation, quantise,
// GEMM2, sum over top-k; "DeepGEMM FusedMoE on Blackwell", 2.6: align M,
// permute, grouped GEMM1, SwiGLU + quant, grouped GEMM2, gather-reduce).
// Everything is enqueued on the caller's stream with no host synchronisation:
// the padded row count stays on the device and every grid is sized from the
// host-side capacity bound, with surplus blocks exiting at once. The
// workspace is one caller-owned block carved into the intermediate buffers;
// the GEMM1 output and the GEMM2 output share storage because their
// lifetimes do not overlap ("fused_moe.py analysis", intermediate caches).
#include <atomic>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

constexpr int64_t kAlign = 256;

// 8-bit activations: fp8 with 128x128 block scales, MXFP8 (E8M0 scales per 32 on both
// operands), or W4A8 (E2M1 weights with E8M0 scales per 32, fp8 activations per 128)
bool q8(const moe_problem_t& p) {
    return p.wdtype == MOE_W_FP8_E4M3_BLOCK128 || p.wdtype == MOE_W_MXFP8 || p.wdtype == MOE_W_W4A8_MXFP4;
}
bool is_mx(const moe_problem_t& p) { return p.wdtype == MOE_W_MXFP8; }
bool is_w4(const moe_problem_t& p) { return p.wdtype == MOE_W_W4A8_MXFP4; }
bool mx_weights(const moe_problem_t& p) { return is_mx(p) || is_w4(p); }  // E8M0 weight scales
int gemm_fmt(const moe_problem_t& p) { return is_mx(p) ? 1 : is_w4(p) ? 2 : 0; }
constexpr int kMaxE = 256;
constexpr int kMaxTopk = 32;
constexpr int kGroupM = 32;  // blocks per tile-scheduling window (groups never span two experts)
static_assert(kGroupM <= 64, "a window's expert ids fit one wavefront");

int64_t up(int64_t b) { return (b + kAlign - 1) / kAlign * kAlign; }

bool block_m_ok(int bm) { return bm == 16 || gemm_supported_block_m(bm); }

// Row geometry of an expert-sorted layout: cap rows, R routed items (entries of
// sorted_token_ids >= R are padding), item r belonging to token r / topk. The
// routed form takes the align capacity; the batched form has E batches of M
// rows, each row its own item (top-1).
struct Rows {
    int64_t cap, R;
    int topk;
};

Rows routed_rows(const moe_problem_t& p) {
    return {moe_align_capacity(p.M, p.topk, p.E, p.block_m), p.M * p.topk, p.topk};
}

Rows batched_rows(const moe_problem_t& p) {
    const int64_t n = static_cast<int64_t>(p.E) * p.M;
    return {n, n, 1};
}

// the problem one chunk of at most chunk_tokens tokens runs as
moe_problem_t chunk_problem(const moe_problem_t& p, int64_t tokens) {
    moe_problem_t q = p;
    q.M = tokens;
    return q;
}

int64_t chunk_of(const moe_problem_t& p) {
    return p.chunk_tokens > 0 && p.chunk_tokens < p.M ? p.chunk_tokens : p.M;
}

struct Layout {
    int64_t cap, R;
    int64_t sorted, expert_ids, npp, inv_perm, xq, xs, xst, ho, z, zs, split, total;
};

// split-K workspace of the second GEMM (bf16 weights, block_m 128 / 256, the DMA
// tiles of 64 Ki outputs): kSplitSlots fp32 partial tiles, then one counter per slot
constexpr int64_t kTileOutputs = 128 * 512;
int64_t split_bytes(const moe_problem_t& p) {
    if (p.wdtype != MOE_W_BF16 || (p.block_m != 128 && p.block_m != 256)) return 0;
    return kSplitSlots * kTileOutputs * 4 + kSplitSlots * 4;
}

// with_split = false: no room for the second GEMM's split-K tail (the layer then
// sums every tile's K range in one pass)
Layout layout(const moe_problem_t& p, const Rows& rows, bool with_split = true) {
    Layout L{};
    L.R = rows.R;
    L.cap = rows.cap;
    const bool fp8 = q8(p);  // MX scale bytes take the same room as the fp32 scales
    int64_t off = 0;
    auto take = [&](int64_t bytes) { const int64_t o = off; off += up(bytes); return o; };
    L.sorted = take(L.cap * 4);
    L.expert_ids = take(L.cap / p.block_m * 4);
    L.npp = take(4);
    L.inv_perm = take(L.R * 4);  // (unused by the batched form)
    L.xq = fp8 ? take(p.M * p.H) : -1;
    L.xs = fp8 ? take(p.M * (p.H / 128) * 4) : -1;
    L.xst = fp8 ? take(L.cap * (p.H / 128) * 4) : -1;  // GEMM1 scales by sorted position
    const int64_t h_bytes = L.cap * 2 * p.I * 2, o_bytes = L.cap * p.H * 2;
    L.ho = take(h_bytes > o_bytes ? h_bytes : o_bytes);
    L.z = take(L.cap * p.I * (fp8 ? 1 : 2));
    L.zs = fp8 ? take(L.cap * (p.I / 128) * 4) : -1;   // [I/128, cap]
    L.split = (with_split && split_bytes(p)) ? take(split_bytes(p)) : -1;
    L.total = off;
    return L;
}

constexpr int kMaxGlobalE = 1 << 16;  // routing range of an expert map

moe_status_t check_problem(const moe_problem_t* p) {
    if (!p) return MOE_E_INVALID;
    if (p->M < 0 || p->H <= 0 || p->I <= 0 || p->E <= 0 || p->topk <= 0) return MOE_E_INVALID;
    if (p->num_global_experts < 0 || p->chunk_tokens < 0) return MOE_E_INVALID;
    if (p->num_global_experts > kMaxGlobalE) return MOE_E_UNSUPPORTED;
    // top-k picks distinct experts of the routing range: the global experts under
    // an expert map, else the E experts held here
    const int e_route = p->num_global_experts > 0 ? p->num_global_experts : p->E;
    if (p->topk > e_route || p->topk > kMaxTopk) return MOE_E_INVALID;
    if (p->E > kMaxE || p->H % 128 || p->I % 128) return MOE_E_UNSUPPORTED;
    if (!block_m_ok(p->block_m)) return MOE_E_UNSUPPORTED;
    if (p->wdtype != MOE_W_BF16 && p->wdtype != MOE_W_FP8_E4M3_BLOCK128 && p->wdtype != MOE_W_MXFP8 &&
        p->wdtype != MOE_W_W4A8_MXFP4)
        return MOE_E_UNSUPPORTED;
    if (p->wdtype == MOE_W_FP8_E4M3_BLOCK128 && (p->block_m == 16 || p->block_m == 256))
        return MOE_E_UNSUPPORTED;
    // MXFP8 runs on the persistent 128-row kernel, which takes K >= 256 in both GEMMs
    if (mx_weights(*p) && (p->block_m != 128 || p->H < 256 || p->I < 256)) return MOE_E_UNSUPPORTED;
    if (p->weight_layout != MOE_LAYOUT_ROWS && p->weight_layout != MOE_LAYOUT_TILED)
        return MOE_E_UNSUPPORTED;
    if (p->weight_layout == MOE_LAYOUT_TILED &&
        (p->wdtype != MOE_W_BF16 || (p->block_m != 16 && p->block_m != 128 && p->block_m != 256)))
        return MOE_E_UNSUPPORTED;
    // one expert's weight matrix is addressed with 32-bit byte offsets
    const int64_t esz = q8(*p) ? 1 : 2;  // (E2M1 weights: half of it)
    if (int64_t(2) * p->I * p->H * esz >= (int64_t(1) << 31)) return MOE_E_UNSUPPORTED;
    // positions and routed items are int32 on the device
    if (p->M * p->topk >= (int64_t(1) << 31)) return MOE_E_UNSUPPORTED;
    const int64_t cap = moe_align_capacity(p->M, p->topk, p->E, p->block_m);
    if (cap >= (int64_t(1) << 31)) return MOE_E_UNSUPPORTED;
    // the GEMM grids (row blocks x column tiles of at least 128 columns, plus one round
    // of split-K workgroups) are int32 on the device and in the launch
    const int64_t n_max = 2 * static_cast<int64_t>(p->I) > p->H ? 2 * static_cast<int64_t>(p->I) : p->H;
    if ((cap / p->block_m) * (n_max / 128 + 1) + 1024 >= (int64_t(1) << 31)) return MOE_E_UNSUPPORTED;
    return MOE_OK;
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_E_HIP; }


// ---- the stages of fused_experts, shared with their exported entry points --

// which == 1: C[pos, :2I] = A[token(pos)] w13[e]^T, A rows gathered through sorted
// which == 2: C[pos, :H]  = A[pos] w2[e]^T
hipError_t gemm_stage(const moe_problem_t& p, const Rows& rows, int which, const void* a,
                      const float* a_scale, const void* w, const float* w_scale,
                      const int32_t* sorted, const int32_t* expert_ids, const int32_t* npp,
                      void* c, void* split_ws, hipStream_t s) {
    const bool fp8 = q8(p);
    const int esz = fp8 ? 1 : 2;  // bytes per weight / activation element
    const int64_t cap = rows.cap;
    const int N = which == 1 ? 2 * p.I : p.H;
    const int K = which == 1 ? p.H : p.I;
    GemmArgs g{};
    g.A = a;
    g.lda_bytes = static_cast<int64_t>(K) * esz;
    g.sorted = which == 1 ? sorted : nullptr;
    g.live_ids = sorted;
    g.topk = rows.topk;
    g.R = static_cast<int>(rows.R);
    g.W = w;
    g.w_expert_bytes = static_cast<int64_t>(N) * K * esz / (is_w4(p) ? 2 : 1);  // E2M1: two per byte
    g.ldw_bytes = static_cast<int64_t>(K) * esz / (is_w4(p) ? 2 : 1);
    g.expert_ids = expert_ids;
    g.npp = npp;
    g.C = c;
    g.ldc_bytes = static_cast<int64_t>(N) * 2;
    g.N = N;
    g.K = K;
    g.m_blocks = static_cast<int>(cap / p.block_m);
    g.group_m = kGroupM;
    g.w_packed = p.weight_layout == MOE_LAYOUT_TILED ? 1 : 0;
    if (fp8) {
        g.a_scale = a_scale;
        g.a_scale_ld = cap;
        g.w_scale = w_scale;
        // fp32 blocks [N/128, K/128] per expert, or MX words [K/128, N]
        g.w_scale_expert = static_cast<int64_t>(mx_weights(p) ? N : N / 128) * (K / 128);
        g.scale_groups = K / 128;
        g.mx = gemm_fmt(p);
    }
    if (which == 2 && split_ws != nullptr && split_bytes(p) > 0) {
        g.part = static_cast<float*>(split_ws);
        g.part_cnt = reinterpret_cast<int*>(static_cast<uint8_t*>(split_ws) + kSplitSlots * kTileOutputs * 4);
        g.part_slots = kSplitSlots;
        g.n_cu = concurrent_tiles();
        // the counters start at zero (a kernel, not a memset: callers may capture this)
        const hipError_t err = launch_zero_i32(g.part_cnt, kSplitSlots, s);
        if (err != hipSuccess) return err;
    }
    return p.block_m == 16 ? launch_stream_gemm(g, s) : launch_grouped_gemm(g, p.block_m, fp8, s);
}

// GEMM1 with SiLU-and-mul in its epilogue: z[pos] = act(x[token(pos)] w13[e]^T)
bool act_fused(const moe_problem_t& p) {
    return gemm_act_supported(p.block_m, q8(p), p.H);
}

// Where GEMM1 builds the routing layout itself instead of reading it: the routed
// ids (with the expert map, if any) and the layout buffers it fills.
struct SelfAlign {
    const int32_t* ids;
    const int32_t* emap;
    int E_global;
    int32_t* sorted;
    int32_t* expert_ids;
    int32_t* npp;
    int32_t* inv_perm;
};

hipError_t gemm_act_stage(const moe_problem_t& p, const Rows& rows, const void* a,
                          const float* a_scale, const void* w13, const float* w13_scale,
                          const int32_t* sorted, const int32_t* expert_ids, const int32_t* npp,
                          const float* weights, void* z, float* z_scale, hipStream_t s,
                          const SelfAlign* self = nullptr) {
    const bool fp8 = q8(p);
    const int esz = fp8 ? 1 : 2;
    const int64_t cap = rows.cap;
    GemmArgs g{};
    g.A = a;
    g.lda_bytes = static_cast<int64_t>(p.H) * esz;
    g.sorted = sorted;
    g.live_ids = sorted;
    g.topk = rows.topk;
    g.R = static_cast<int>(rows.R);
    g.W = w13;
    g.w_expert_bytes = static_cast<int64_t>(2) * p.I * p.H * esz / (is_w4(p) ? 2 : 1);
    g.ldw_bytes = static_cast<int64_t>(p.H) * esz / (is_w4(p) ? 2 : 1);
    g.expert_ids = expert_ids;
    g.npp = npp;
    g.C = z;
    g.ldc_bytes = static_cast<int64_t>(p.I) * esz;
    g.N = p.I;  // output columns; gate rows [0, I), up rows [I, 2I)
    g.K = p.H;
    g.m_blocks = static_cast<int>(cap / p.block_m);
    g.group_m = kGroupM;
    g.w_packed = p.weight_layout == MOE_LAYOUT_TILED ? 1 : 0;
    g.act = 1;
    g.act_weights = weights;
    g.act_on_input = p.apply_router_weight_on_input ? 1 : 0;
    if (self) {
        g.route_ids = self->ids;
        g.route_emap = self->emap;
        g.route_E_global = self->E_global;
        g.route_E = p.E;
        g.out_sorted = self->sorted;
        g.out_expert_ids = self->expert_ids;
        g.out_npp = self->npp;
        g.out_inv_perm = self->inv_perm;
    }
    if (fp8) {
        g.a_scale = a_scale;
        g.a_scale_ld = cap;
        g.w_scale = w13_scale;
        g.w_scale_expert = static_cast<int64_t>(mx_weights(p) ? 2 * p.I : 2 * p.I / 128) * (p.H / 128);
        g.scale_groups = p.H / 128;
        g.z_scale = z_scale;
        g.z_scale_ld = cap;
        g.mx = gemm_fmt(p);
    }
    return p.block_m == 16 ? launch_stream_gemm(g, s) : launch_grouped_gemm(g, p.block_m, fp8, s);
}

hipError_t act_stage(const moe_problem_t& p, const Rows& rows, const void* h, const int32_t* sorted,
                     const float* weights, const int32_t* npp, void* z, float* z_scale,
                     hipStream_t s) {
    const int64_t cap = rows.cap;
    const int R = static_cast<int>(rows.R);
    const int on_input = p.apply_router_weight_on_input ? 1 : 0;
    if (p.wdtype == MOE_W_FP8_E4M3_BLOCK128)
        return launch_silu_mul_fp8(static_cast<const bf16_t*>(h), static_cast<uint8_t*>(z),
                                   z_scale, sorted, weights, R, p.I, cap, npp, on_input, s);
    return launch_silu_mul_bf16(static_cast<const bf16_t*>(h), static_cast<bf16_t*>(z), sorted,
                                weights, R, p.I, cap, npp, on_input, s);
}

hipError_t permute_stage(const moe_problem_t& p, const Rows& rows, const float* scale,
                         const int32_t* sorted, const int32_t* npp, float* out, hipStream_t s) {
    const int64_t cap = rows.cap;
    return launch_permute_scales(scale, p.H / 128, rows.topk, static_cast<int>(rows.R), sorted,
                                 npp, cap, out, s);
}

// weights are applied unless the router weight went onto the SiLU-and-mul input
// or the caller's combine applies them (unweighted, the batched form)
hipError_t reduce_stage(const moe_problem_t& p, const void* o, const int32_t* inv_perm,
                        const float* weights, void* y, hipStream_t s, bool unweighted = false) {
    return launch_reduce(static_cast<const bf16_t*>(o), inv_perm, weights, p.M, p.topk, p.H,
                         (p.apply_router_weight_on_input || unweighted) ? 0 : 1,
                         static_cast<bf16_t*>(y), s);
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_E_INVALID: return "invalid argument";
        case MOE_E_UNSUPPORTED: return "unsupported problem";
        case MOE_E_WORKSPACE: return "workspace too small";
        case MOE_E_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

int64_t moe_align_capacity(int64_t M, int32_t topk, int32_t E, int32_t block_m) {
    if (M < 0 || topk <= 0 || E <= 0 || block_m <= 0) return -1;
    const int64_t R = M * topk;
    const int64_t bound = R + (R < E ? R : E) * static_cast<int64_t>(block_m - 1);
    return (bound + block_m - 1) / block_m * block_m;
}

moe_status_t moe_topk(const float* logits, int64_t M, int32_t E, int32_t topk, int32_t renormalize,
                      int32_t* topk_ids, float* topk_weights, void* stream) {
    if (M < 0 || E <= 0 || topk <= 0 || topk > E || topk > kMaxTopk) return MOE_E_INVALID;
    if (E > kMaxE) return MOE_E_UNSUPPORTED;
    if (M == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_weights) return MOE_E_INVALID;
    return hip_status(launch_topk_softmax(logits, M, E, topk, renormalize, topk_ids, topk_weights,
                                          static_cast<hipStream_t>(stream)));
}

moe_status_t moe_topk_grouped(const float* logits, int64_t M, int32_t E, int32_t topk, int32_t scoring,
                              int32_t renormalize, int32_t num_expert_group, int32_t topk_group,
                              const float* e_score_correction_bias, float routed_scaling_factor,
                              int32_t* topk_ids, float* topk_weights, void* stream) {
    if (M < 0 || E <= 0 || topk <= 0 || topk > kMaxTopk) return MOE_E_INVALID;
    if (scoring != MOE_SCORING_SOFTMAX && scoring != MOE_SCORING_SIGMOID) return MOE_E_INVALID;
    const int G = num_expert_group, TG = topk_group;
    if (G < 1 || TG < 1 || TG > G || E % G) return MOE_E_INVALID;
    if (topk > TG * (E / G)) return MOE_E_INVALID;  // not enough experts in the kept groups
    if (e_score_correction_bias && (scoring != MOE_SCORING_SIGMOID || E / G < 2)) return MOE_E_INVALID;
    if (E > kMaxE || G > 64) return MOE_E_UNSUPPORTED;
    if (M == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_weights) return MOE_E_INVALID;
    return hip_status(launch_topk_grouped(logits, M, E, topk, scoring == MOE_SCORING_SIGMOID ? 1 : 0,
                                          renormalize, G, TG, e_score_correction_bias,
                                          routed_scaling_factor, topk_ids, topk_weights,
                                          static_cast<hipStream_t>(stream)));
}

moe_status_t moe_align_block_size(const int32_t* topk_ids, int64_t M, int32_t topk, int32_t E,
                                  int32_t block_m, int32_t* sorted_token_ids, int32_t* expert_ids,
                                  int32_t* num_tokens_post_padded, int32_t* inv_perm,
                                  void* stream) {
    if (M < 0 || E <= 0 || topk <= 0 || topk > E || topk > kMaxTopk || block_m <= 0)
        return MOE_E_INVALID;
    if (E > kMaxE || !block_m_ok(block_m)) return MOE_E_UNSUPPORTED;
    const int64_t cap = moe_align_capacity(M, topk, E, block_m);
    if (M * topk >= (int64_t(1) << 31) || cap >= (int64_t(1) << 31)) return MOE_E_UNSUPPORTED;
    // with M == 0 only num_tokens_post_padded is written (0); the rest may be null
    if (!num_tokens_post_padded) return MOE_E_INVALID;
    if (M > 0 && (!topk_ids || !sorted_token_ids || !expert_ids || !inv_perm)) return MOE_E_INVALID;
    return hip_status(launch_align(topk_ids, M * topk, E, block_m, cap, nullptr, 0, sorted_token_ids,
                                   expert_ids, num_tokens_post_padded, inv_perm,
                                   static_cast<hipStream_t>(stream)));
}

moe_status_t moe_align_block_size_ep(const int32_t* topk_ids, int64_t M, int32_t topk,
                                     int32_t num_global_experts, const int32_t* expert_map,
                                     int32_t E, int32_t block_m, int32_t* sorted_token_ids,
                                     int32_t* expert_ids, int32_t* num_tokens_post_padded,
                                     int32_t* inv_perm, void* stream) {
    if (M < 0 || E <= 0 || topk <= 0 || block_m <= 0 || num_global_experts <= 0) return MOE_E_INVALID;
    if (topk > num_global_experts || topk > kMaxTopk) return MOE_E_INVALID;
    if (E > kMaxE || num_global_experts > kMaxGlobalE || !block_m_ok(block_m)) return MOE_E_UNSUPPORTED;
    const int64_t cap = moe_align_capacity(M, topk, E, block_m);
    if (M * topk >= (int64_t(1) << 31) || cap >= (int64_t(1) << 31)) return MOE_E_UNSUPPORTED;
    if (!num_tokens_post_padded || !expert_map) return MOE_E_INVALID;
    if (M > 0 && (!topk_ids || !sorted_token_ids || !expert_ids || !inv_perm)) return MOE_E_INVALID;
    return hip_status(launch_align(topk_ids, M * topk, E, block_m, cap, expert_map, num_global_experts,
                                   sorted_token_ids, expert_ids, num_tokens_post_padded, inv_perm,
                                   static_cast<hipStream_t>(stream)));
}

moe_status_t moe_quant_fp8_groups(const void* x, int64_t rows, int32_t cols, void* q, float* scale,
                                  void* stream) {
    if (rows < 0 || cols <= 0) return MOE_E_INVALID;
    if (cols % 128) return MOE_E_UNSUPPORTED;
    if (rows == 0) return MOE_OK;
    if (!x || !q || !scale) return MOE_E_INVALID;
    return hip_status(launch_quant_fp8(static_cast<const bf16_t*>(x), rows, cols,
                                       static_cast<uint8_t*>(q), scale,
                                       static_cast<hipStream_t>(stream)));
}

moe_status_t moe_quant_mx_groups(const void* x, int64_t rows, int32_t cols, void* q, void* scale,
                                 void* stream) {
    if (rows < 0 || cols <= 0) return MOE_E_INVALID;
    if (cols % 128) return MOE_E_UNSUPPORTED;
    if (rows == 0) return MOE_OK;
    if (!x || !q || !scale) return MOE_E_INVALID;
    return hip_status(launch_quant_mxfp8(static_cast<const bf16_t*>(x), rows, cols, static_cast<uint8_t*>(q),
                                         static_cast<uint8_t*>(scale), static_cast<hipStream_t>(stream)));
}

size_t moe_workspace_bytes(const moe_problem_t* p) {
    if (check_problem(p) != MOE_OK || p->M == 0) return 0;
    const moe_problem_t q = chunk_problem(*p, chunk_of(*p));
    return static_cast<size_t>(layout(q, routed_rows(q)).total);
}

}  // extern "C"

namespace {

// fused_experts and fused_experts_ep: emap is null (ids are local) or holds
// p->num_global_experts entries. unweighted (the batched form): every slot enters
// the sum with weight 1 and topk_weights is not read.
moe_status_t run_fused(const moe_problem_t* p, const int32_t* emap, const void* x, const void* w13,
                       const float* w13_scale, const void* w2, const float* w2_scale,
                       const int32_t* topk_ids, const float* topk_weights, void* y,
                       void* workspace, size_t workspace_bytes, void* stream,
                       bool unweighted = false, bool with_split = true) {
    if (p->M == 0) return MOE_OK;
    const bool fp8 = q8(*p);
    if (!x || !w13 || !w2 || !topk_ids || !y || (!topk_weights && !unweighted)) return MOE_E_INVALID;
    if (fp8 && (!w13_scale || !w2_scale)) return MOE_E_INVALID;
    const Rows rows = routed_rows(*p);
    const Layout L = layout(*p, rows, with_split);
    if (!workspace || workspace_bytes < static_cast<size_t>(L.total)) return MOE_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return MOE_E_INVALID;

    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
    int32_t* expert_ids = reinterpret_cast<int32_t*>(ws + L.expert_ids);
    int32_t* npp = reinterpret_cast<int32_t*>(ws + L.npp);
    int32_t* inv_perm = reinterpret_cast<int32_t*>(ws + L.inv_perm);
    void* ho = ws + L.ho;
    void* z = ws + L.z;
    const int M = static_cast<int>(p->M), H = p->H;

    hipError_t err = hipSuccess;
    const void* a1 = x;
    const float* a1_scale = nullptr;
    if (fp8) {
        err = is_mx(*p) ? launch_quant_mxfp8(static_cast<const bf16_t*>(x), M, H, ws + L.xq, ws + L.xs, s)
                        : launch_quant_fp8(static_cast<const bf16_t*>(x), M, H, ws + L.xq,
                                           reinterpret_cast<float*>(ws + L.xs), s);
        if (err != hipSuccess) return MOE_E_HIP;
        a1 = ws + L.xq;
        a1_scale = reinterpret_cast<const float*>(ws + L.xst);
    }
    // decode-sized bf16 problems: GEMM1 builds the layout itself (one launch fewer)
    const bool self_align = p->block_m == 16 && !fp8 && act_fused(*p) && rows.R <= kSelfAlignMaxR;
    const SelfAlign self{topk_ids, emap, p->num_global_experts, sorted, expert_ids, npp, inv_perm};
    if (!self_align) {
        err = launch_align(topk_ids, M * p->topk, p->E, p->block_m, L.cap, emap, p->num_global_experts,
                           sorted, expert_ids, npp, inv_perm, s);
        if (err != hipSuccess) return MOE_E_HIP;
    }
    if (fp8) {
        err = permute_stage(*p, rows, reinterpret_cast<const float*>(ws + L.xs), sorted, npp,
                            reinterpret_cast<float*>(ws + L.xst), s);
        if (err != hipSuccess) return MOE_E_HIP;
    }
    float* zs = fp8 ? reinterpret_cast<float*>(ws + L.zs) : nullptr;
    if (act_fused(*p)) {
        err = gemm_act_stage(*p, rows, a1, a1_scale, w13, w13_scale, sorted, expert_ids, npp,
                             topk_weights, z, zs, s, self_align ? &self : nullptr);
        if (err != hipSuccess) return MOE_E_HIP;
    } else {
        err = gemm_stage(*p, rows, 1, a1, a1_scale, w13, w13_scale, sorted, expert_ids, npp, ho, nullptr, s);
        if (err != hipSuccess) return MOE_E_HIP;
        err = act_stage(*p, rows, ho, sorted, topk_weights, npp, z, zs, s);
        if (err != hipSuccess) return MOE_E_HIP;
    }
    err = gemm_stage(*p, rows, 2, z, zs, w2, w2_scale, sorted, expert_ids, npp, ho,
                     L.split >= 0 ? ws + L.split : nullptr, s);
    if (err != hipSuccess) return MOE_E_HIP;
    return hip_status(reduce_stage(*p, ho, inv_perm, topk_weights, y, s, unweighted));
}

// The batched form as a routed top-1 problem: batch row e * max_M + i is item r
// of its own token, routed to expert e if i < expert_num_tokens[e], else to no
// expert (skipped by align, so its output row reduces to 0).
moe_problem_t batched_as_routed(const moe_problem_t& p) {
    moe_problem_t q = p;
    q.M = static_cast<int64_t>(p.E) * p.M;
    q.topk = 1;
    return q;
}

int64_t batched_ids_bytes(const moe_problem_t& p) { return up(static_cast<int64_t>(p.E) * p.M * 4); }

moe_status_t check_batched(const moe_problem_t* p) {
    if (!p) return MOE_E_INVALID;
    if (p->topk != 1 || p->apply_router_weight_on_input || p->num_global_experts != 0)
        return MOE_E_INVALID;  // one expert per row, unweighted, local experts
    const moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    const moe_problem_t q = batched_as_routed(*p);
    return check_problem(&q);
}

// the layer over chunks of tokens, one after another on the stream, each reusing
// the whole workspace (a chunk's kernels are enqueued after the previous chunk's)
moe_status_t run_chunked(const moe_problem_t* p, const int32_t* emap, const void* x, const void* w13,
                         const float* w13_scale, const void* w2, const float* w2_scale,
                         const int32_t* topk_ids, const float* topk_weights, void* y,
                         void* workspace, size_t workspace_bytes, void* stream,
                         bool with_split = true) {
    const int64_t chunk = chunk_of(*p);
    if (chunk == p->M)
        return run_fused(p, emap, x, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, y,
                         workspace, workspace_bytes, stream, false, with_split);
    if (!x || !topk_ids || !topk_weights || !y) return MOE_E_INVALID;
    const int64_t row = static_cast<int64_t>(p->H) * 2;  // bytes of one x / y row
    for (int64_t t0 = 0; t0 < p->M; t0 += chunk) {
        const moe_problem_t q = chunk_problem(*p, p->M - t0 < chunk ? p->M - t0 : chunk);
        const moe_status_t st = run_fused(
            &q, emap, static_cast<const uint8_t*>(x) + t0 * row, w13, w13_scale, w2, w2_scale,
            topk_ids + t0 * p->topk, topk_weights + t0 * p->topk, static_cast<uint8_t*>(y) + t0 * row,
            workspace, workspace_bytes, stream, false, with_split);
        if (st != MOE_OK) return st;
    }
    return MOE_OK;
}

// ---- scratch for callers that cannot allocate ------------------------------
// A file-scope device array: every GPU the library runs on holds its own copy
// until the process ends. In host code the array's name is only a host-side
// stand-in, so its device address is looked up once per device (with that
// device current, on the entry point's first call there) and kept; kernels and
// copies use that address, never the name.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<uint8_t*> scratch_addr[kMaxDevices];

// this device's copy of `scratch` (null if the lookup fails); concurrent first calls
// look up and store the same address
uint8_t* static_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    uint8_t* ptr = scratch_addr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        void* a = nullptr;
        if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || a == nullptr) return nullptr;
        ptr = static_cast<uint8_t*>(a);
        scratch_addr[dev].store(ptr, std::memory_order_release);
    }
    return ptr;
}

}  // namespace

extern "C" {

moe_status_t fused_experts_static(const moe_problem_t* p, const void* x, const void* w13,
                                  const float* w13_scale, const void* w2, const float* w2_scale,
                                  const int32_t* topk_ids, const float* topk_weights, void* y,
                                  void* stream) {
    const moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (p->num_global_experts != 0) return MOE_E_INVALID;
    if (p->M == 0) return MOE_OK;
    if (!x || !w13 || !w2 || !topk_ids || !topk_weights || !y) return MOE_E_INVALID;
    if (q8(*p) && (!w13_scale || !w2_scale)) return MOE_E_INVALID;
    const moe_problem_t q = chunk_problem(*p, chunk_of(*p));
    const int64_t need = layout(q, routed_rows(q), false).total;
    if (need > static_cast<int64_t>(kStaticScratchBytes)) return MOE_E_WORKSPACE;
    uint8_t* ws = static_scratch();
    if (ws == nullptr) return MOE_E_HIP;
    return run_chunked(p, nullptr, x, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, y, ws,
                       kStaticScratchBytes, stream, false);
}

moe_status_t fused_experts(const moe_problem_t* p, const void* x, const void* w13,
                           const float* w13_scale, const void* w2, const float* w2_scale,
                           const int32_t* topk_ids, const float* topk_weights, void* y,
                           void* workspace, size_t workspace_bytes, void* stream) {
    const moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (p->num_global_experts != 0) return MOE_E_INVALID;  // global ids need the expert map
    return run_chunked(p, nullptr, x, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, y,
                       workspace, workspace_bytes, stream);
}

moe_status_t fused_experts_ep(const moe_problem_t* p, const int32_t* expert_map, const void* x,
                              const void* w13, const float* w13_scale, const void* w2,
                              const float* w2_scale, const int32_t* topk_ids,
                              const float* topk_weights, void* y, void* workspace,
                              size_t workspace_bytes, void* stream) {
    const moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (p->num_global_experts <= 0 || !expert_map) return MOE_E_INVALID;
    return run_chunked(p, expert_map, x, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, y,
                       workspace, workspace_bytes, stream);
}

size_t moe_batched_workspace_bytes(const moe_problem_t* p) {
    if (check_batched(p) != MOE_OK || p->M == 0) return 0;
    const moe_problem_t q = batched_as_routed(*p);
    return static_cast<size_t>(batched_ids_bytes(*p) + layout(q, routed_rows(q)).total);
}

moe_status_t moe_batched_experts(const moe_problem_t* p, const void* a, const int32_t* expert_num_tokens,
                                 const void* w13, const float* w13_scale, const void* w2,
                                 const float* w2_scale, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    const moe_status_t st = check_batched(p);
    if (st != MOE_OK) return st;
    if (p->M == 0) return MOE_OK;
    if (!a || !expert_num_tokens || !out) return MOE_E_INVALID;
    if (!workspace || workspace_bytes < moe_batched_workspace_bytes(p)) return MOE_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return MOE_E_INVALID;
    const moe_problem_t q = batched_as_routed(*p);
    int32_t* ids = static_cast<int32_t*>(workspace);
    const hipError_t err = launch_batched_ids(expert_num_tokens, p->E, p->M, ids,
                                              static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return MOE_E_HIP;
    const int64_t off = batched_ids_bytes(*p);
    return run_fused(&q, nullptr, a, w13, w13_scale, w2, w2_scale, ids, nullptr, out,
                     static_cast<uint8_t*>(workspace) + off, workspace_bytes - off, stream, true);
}

size_t moe_expert_gemm_workspace_bytes(const moe_problem_t* p) {
    if (check_problem(p) != MOE_OK) return 0;
    return static_cast<size_t>(split_bytes(*p));
}

moe_status_t moe_expert_gemm(const moe_problem_t* p, int32_t which, const void* a,
                             const float* a_scale, const void* w, const float* w_scale,
                             const int32_t* sorted_token_ids, const int32_t* expert_ids,
                             const int32_t* num_tokens_post_padded, void* c, void* workspace,
                             size_t workspace_bytes, void* stream) {
    const moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (which != 1 && which != 2) return MOE_E_INVALID;
    if (p->M == 0) return MOE_OK;
    const bool fp8 = q8(*p);
    if (!a || !w || !expert_ids || !num_tokens_post_padded || !c) return MOE_E_INVALID;
    if (which == 1 && !sorted_token_ids) return MOE_E_INVALID;
    if (fp8 && (!a_scale || !w_scale)) return MOE_E_INVALID;
    if (workspace != nullptr && workspace_bytes < static_cast<size_t>(split_bytes(*p))) return MOE_E_WORKSPACE;
    return hip_status(gemm_stage(*p, routed_rows(*p), which, a, a_scale, w, w_scale, sorted_token_ids, expert_ids,
                                 num_tokens_post_padded, c, workspace, static_cast<hipStream_t>(stream)));
}

int32_t moe_expert_gemm_act_supported(const moe_problem_t* p) {
    return check_problem(p) == MOE_OK && act_fused(*p) ? 1 : 0;
}

moe_status_t moe_expert_gemm_act(const moe_problem_t* p, const void* x, const float* x_scale,
                                 const void* w13, const float* w13_scale,
                                 const int32_t* sorted_token_ids, const int32_t* expert_ids,
                                 const int32_t* num_tokens_post_padded, const float* topk_weights,
                                 void* z, float* z_scale, void* stream) {
    const moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!act_fused(*p)) return MOE_E_UNSUPPORTED;
    if (p->M == 0) return MOE_OK;
    const bool fp8 = q8(*p);
    if (!x || !w13 || !sorted_token_ids || !expert_ids || !num_tokens_post_padded || !topk_weights || !z)
        return MOE_E_INVALID;
    if (fp8 && (!x_scale || !w13_scale || !z_scale)) return MOE_E_INVALID;
    return hip_status(gemm_act_stage(*p, routed_rows(*p), x, x_scale, w13, w13_scale, sorted_token_ids, expert_ids,
                                     num_tokens_post_padded, topk_weights, z, z_scale,
                                     static_cast<hipStream_t>(stream)));
}

moe_status_t moe_silu_and_mul(const moe_problem_t* p, const void* h,
                              const int32_t* sorted_token_ids, const float* topk_weights,
                              const int32_t* num_tokens_post_padded, void* z, float* z_scale,
                              void* stream) {
    const moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (p->M == 0) return MOE_OK;
    if (!h || !sorted_token_ids || !topk_weights || !num_tokens_post_padded || !z)
        return MOE_E_INVALID;
    if (is_mx(*p)) return MOE_E_UNSUPPORTED;  // MXFP8 quantises z in GEMM1's epilogue only
    if (p->wdtype == MOE_W_FP8_E4M3_BLOCK128 && !z_scale) return MOE_E_INVALID;
    return hip_status(act_stage(*p, routed_rows(*p), h, sorted_token_ids, topk_weights, num_tokens_post_padded, z,
                                z_scale, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_permute_scales(const moe_problem_t* p, const float* scale,
                                const int32_t* sorted_token_ids,
                                const int32_t* num_tokens_post_padded, float* out, void* stream) {
    const moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (p->M == 0) return MOE_OK;
    if (!scale || !sorted_token_ids || !num_tokens_post_padded || !out) return MOE_E_INVALID;
    return hip_status(permute_stage(*p, routed_rows(*p), scale, sorted_token_ids, num_tokens_post_padded, out,
                                    static_cast<hipStream_t>(stream)));
}

moe_status_t moe_pack_weights(const moe_problem_t* p, int32_t which, const void* w, void* w_packed,
                              void* stream) {
    const moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (which != 1 && which != 2) return MOE_E_INVALID;
    if (p->wdtype != MOE_W_BF16) return MOE_E_UNSUPPORTED;
    if (!w || !w_packed) return MOE_E_INVALID;
    const int N = which == 1 ? 2 * p->I : p->H, K = which == 1 ? p->H : p->I;
    const int64_t bytes = static_cast<int64_t>(p->E) * N * K * 2;
    const uintptr_t a = reinterpret_cast<uintptr_t>(w), b = reinterpret_cast<uintptr_t>(w_packed);
    if (a < b + bytes && b < a + bytes) return MOE_E_INVALID;  // overlapping buffers
    if (a % 16 || b % 16) return MOE_E_INVALID;
    return hip_status(launch_pack_tiled(static_cast<const bf16_t*>(w), static_cast<bf16_t*>(w_packed),
                                         p->E, N, K, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_pack_mx_scales(const moe_problem_t* p, int32_t which, const void* scale,
                                void* scale_packed, void* stream) {
    const moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (which != 1 && which != 2) return MOE_E_INVALID;
    if (!mx_weights(*p)) return MOE_E_UNSUPPORTED;
    if (!scale || !scale_packed || scale == scale_packed) return MOE_E_INVALID;
    if (reinterpret_cast<uintptr_t>(scale) % 4 || reinterpret_cast<uintptr_t>(scale_packed) % 4)
        return MOE_E_INVALID;
    const int N = which == 1 ? 2 * p->I : p->H, K = which == 1 ? p->H : p->I;
    return hip_status(launch_pack_mx_scales(static_cast<const uint8_t*>(scale), static_cast<uint32_t*>(scale_packed),
                                            p->E, N, K, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_unpermute_reduce(const moe_problem_t* p, const void* o, const int32_t* inv_perm,
                                  const float* topk_weights, void* y, void* stream) {
    const moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (p->M == 0) return MOE_OK;
    if (!o || !inv_perm || !topk_weights || !y) return MOE_E_INVALID;
    return hip_status(reduce_stage(*p, o, inv_perm, topk_weights, y,
                                   static_cast<hipStream_t>(stream)));
}

}  // extern "C"
