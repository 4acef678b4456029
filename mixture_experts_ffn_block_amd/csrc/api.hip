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
#include "../../include/moe.h"
#include "kernels.h"

namespace {

constexpr int64_t kAlign = 256;
constexpr int kMaxE = 256;
constexpr int kMaxTopk = 32;
constexpr int kGroupM = 8;

int64_t up(int64_t b) { return (b + kAlign - 1) / kAlign * kAlign; }

bool block_m_ok(int bm) { return bm == 16 || gemm_supported_block_m(bm); }

struct Layout {
    int64_t cap, R;
    int64_t sorted, expert_ids, npp, inv_perm, xq, xs, ho, z, zs, total;
};

Layout layout(const moe_problem_t& p) {
    Layout L{};
    L.R = p.M * p.topk;
    L.cap = moe_align_capacity(p.M, p.topk, p.E, p.block_m);
    const bool fp8 = p.wdtype == MOE_W_FP8_E4M3_BLOCK128;
    int64_t off = 0;
    auto take = [&](int64_t bytes) { const int64_t o = off; off += up(bytes); return o; };
    L.sorted = take(L.cap * 4);
    L.expert_ids = take(L.cap / p.block_m * 4);
    L.npp = take(4);
    L.inv_perm = take(L.R * 4);
    L.xq = fp8 ? take(p.M * p.H) : -1;
    L.xs = fp8 ? take(p.M * (p.H / 128) * 4) : -1;
    const int64_t h_bytes = L.cap * 2 * p.I * 2, o_bytes = L.cap * p.H * 2;
    L.ho = take(h_bytes > o_bytes ? h_bytes : o_bytes);
    L.z = take(L.cap * p.I * (fp8 ? 1 : 2));
    L.zs = fp8 ? take(L.cap * (p.I / 128) * 4) : -1;
    L.total = off;
    return L;
}

moe_status_t check_problem(const moe_problem_t* p) {
    if (!p) return MOE_E_INVALID;
    if (p->M < 0 || p->H <= 0 || p->I <= 0 || p->E <= 0 || p->topk <= 0) return MOE_E_INVALID;
    if (p->topk > p->E || p->topk > kMaxTopk) return MOE_E_INVALID;
    if (p->E > kMaxE || p->H % 128 || p->I % 128) return MOE_E_UNSUPPORTED;
    if (!block_m_ok(p->block_m)) return MOE_E_UNSUPPORTED;
    if (p->wdtype != MOE_W_BF16 && p->wdtype != MOE_W_FP8_E4M3_BLOCK128) return MOE_E_UNSUPPORTED;
    if (p->wdtype == MOE_W_FP8_E4M3_BLOCK128 && p->block_m == 16) return MOE_E_UNSUPPORTED;
    // positions and routed items are int32 on the device
    if (p->M * p->topk >= (int64_t(1) << 31)) return MOE_E_UNSUPPORTED;
    if (moe_align_capacity(p->M, p->topk, p->E, p->block_m) >= (int64_t(1) << 31)) return MOE_E_UNSUPPORTED;
    return MOE_OK;
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_E_HIP; }

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
    return hip_status(launch_align(topk_ids, M * topk, E, block_m, cap, sorted_token_ids,
                                   expert_ids, num_tokens_post_padded, inv_perm,
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

size_t moe_workspace_bytes(const moe_problem_t* p) {
    if (check_problem(p) != MOE_OK || p->M == 0) return 0;
    return static_cast<size_t>(layout(*p).total);
}

moe_status_t fused_experts(const moe_problem_t* p, const void* x, const void* w13,
                           const float* w13_scale, const void* w2, const float* w2_scale,
                           const int32_t* topk_ids, const float* topk_weights, void* y,
                           void* workspace, size_t workspace_bytes, void* stream) {
    const moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (p->M == 0) return MOE_OK;
    const bool fp8 = p->wdtype == MOE_W_FP8_E4M3_BLOCK128;
    if (!x || !w13 || !w2 || !topk_ids || !topk_weights || !y) return MOE_E_INVALID;
    if (fp8 && (!w13_scale || !w2_scale)) return MOE_E_INVALID;
    const Layout L = layout(*p);
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
    const int M = static_cast<int>(p->M), H = p->H, I = p->I, k = p->topk, B = p->block_m;
    const int R = static_cast<int>(L.R);
    const int m_blocks = static_cast<int>(L.cap / B);

    hipError_t err = hipSuccess;
    const void* a1 = x;
    if (fp8) {
        err = launch_quant_fp8(static_cast<const bf16_t*>(x), M, H, ws + L.xq,
                               reinterpret_cast<float*>(ws + L.xs), s);
        if (err != hipSuccess) return MOE_E_HIP;
        a1 = ws + L.xq;
    }
    err = launch_align(topk_ids, R, p->E, B, L.cap, sorted, expert_ids, npp, inv_perm, s);
    if (err != hipSuccess) return MOE_E_HIP;

    const int esz = fp8 ? 1 : 2;  // bytes per weight / activation element
    GemmArgs g1{};
    g1.A = a1;
    g1.lda_bytes = static_cast<int64_t>(H) * esz;
    g1.sorted = sorted;
    g1.topk = k;
    g1.R = R;
    g1.W = w13;
    g1.w_expert_bytes = static_cast<int64_t>(2 * I) * H * esz;
    g1.ldw_bytes = static_cast<int64_t>(H) * esz;
    g1.expert_ids = expert_ids;
    g1.npp = npp;
    g1.C = ho;
    g1.ldc_bytes = static_cast<int64_t>(2 * I) * 2;
    g1.N = 2 * I;
    g1.K = H;
    g1.m_blocks = m_blocks;
    g1.group_m = kGroupM;
    if (fp8) {
        g1.a_scale = reinterpret_cast<const float*>(ws + L.xs);
        g1.w_scale = w13_scale;
        g1.w_scale_expert = static_cast<int64_t>(2 * I / 128) * (H / 128);
        g1.scale_groups = H / 128;
    }
    err = B == 16 ? launch_stream_gemm(g1, s) : launch_grouped_gemm(g1, B, fp8, s);
    if (err != hipSuccess) return MOE_E_HIP;

    const int on_input = p->apply_router_weight_on_input ? 1 : 0;
    if (fp8)
        err = launch_silu_mul_fp8(static_cast<const bf16_t*>(ho), static_cast<uint8_t*>(z),
                                  reinterpret_cast<float*>(ws + L.zs), sorted, topk_weights, R, I,
                                  L.cap, npp, on_input, s);
    else
        err = launch_silu_mul_bf16(static_cast<const bf16_t*>(ho), static_cast<bf16_t*>(z), sorted,
                                   topk_weights, R, I, L.cap, npp, on_input, s);
    if (err != hipSuccess) return MOE_E_HIP;

    GemmArgs g2 = g1;
    g2.A = z;
    g2.lda_bytes = static_cast<int64_t>(I) * esz;
    g2.sorted = nullptr;
    g2.W = w2;
    g2.w_expert_bytes = static_cast<int64_t>(H) * I * esz;
    g2.ldw_bytes = static_cast<int64_t>(I) * esz;
    g2.C = ho;
    g2.ldc_bytes = static_cast<int64_t>(H) * 2;
    g2.N = H;
    g2.K = I;
    if (fp8) {
        g2.a_scale = reinterpret_cast<const float*>(ws + L.zs);
        g2.w_scale = w2_scale;
        g2.w_scale_expert = static_cast<int64_t>(H / 128) * (I / 128);
        g2.scale_groups = I / 128;
    }
    err = B == 16 ? launch_stream_gemm(g2, s) : launch_grouped_gemm(g2, B, fp8, s);
    if (err != hipSuccess) return MOE_E_HIP;

    err = launch_reduce(static_cast<const bf16_t*>(ho), inv_perm, topk_weights, M, k, H,
                        on_input ? 0 : 1, static_cast<bf16_t*>(y), s);
    return hip_status(err);
}

}  // extern "C"
