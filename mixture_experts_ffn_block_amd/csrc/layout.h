// layout.h -- pieces of the expert-sorted routing layout shared by the align
// kernels and the self-aligning decode GEMM.
//
// "fused_moe.py analysis", "moe_align_block_size": every expert's routed items
// form a segment padded to a multiple of BLOCK_M rows, segments in expert order;
// "DeepGEMM FusedMoE on Blackwell", 2.6.2: a prefix sum over the padded counts
// gives each segment's first row. Both users compute the layout from these
// helpers, so they agree bit for bit.
#pragma once

#include "common.h"

namespace {

constexpr int kMaxE = 256;  // experts of one routing (local experts of a rank)

// this rank's expert of global id `id`: the id itself without a map; ids outside
// the routing range and map entries outside [0, E) count as not local (-1)
__device__ __forceinline__ int local_expert(int id, const int32_t* __restrict__ emap, int E_global) {
    if (emap == nullptr) return id;
    return static_cast<unsigned>(id) < static_cast<unsigned>(E_global) ? emap[id] : -1;
}

// Inclusive sum over the 64 lanes of a wavefront: prefix sums inside each row of
// 16 lanes by DPP row shifts of 1, 2, 4 and 8, then row broadcasts of lanes 15 and
// 31 carry each row's total into the rows above (the cross-lane scan AMD published
// for GCN). Lanes whose source is outside the row read 0.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
    return x;
}

// By one wavefront: v[i] is the padded size of expert 4 lane + i; on return it is
// that expert's segment start (the exclusive prefix sum over experts), and the
// padded total is returned to every lane.
__device__ __forceinline__ int scan_padded(int (&v)[4]) {
    static_assert(kMaxE == 4 * MOE_WAVE, "four experts per lane");
    const int sum = v[0] + v[1] + v[2] + v[3];
    const int incl = wave_inclusive_sum(sum);
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int size = v[i];
        v[i] = run;
        run += size;
    }
    return __builtin_amdgcn_readlane(incl, 63);
}

// In place, by one wavefront: seg_start[1 .. kMaxE] holds the padded size of each
// expert and becomes the inclusive prefix sum (seg_start[0] stays 0).
__device__ __forceinline__ void scan_segments(int32_t* seg_start, int lane) {
    int v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = seg_start[4 * lane + i + 1];
    const int last = v[3];
    scan_padded(v);
#pragma unroll
    for (int i = 0; i < 3; ++i) seg_start[4 * lane + i + 1] = v[i + 1];
    seg_start[4 * lane + 4] = v[3] + last;
}

// Expert whose segment holds row `pos` (pos below the padded total): the last e
// with seg_start[e] <= pos. Empty experts share their start with the next one, so
// the last such e is the one with rows.
__device__ __forceinline__ int segment_of(const int32_t* seg_start, int E, int64_t pos) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seg_start[mid] <= pos) lo = mid; else hi = mid - 1;
    }
    return lo;
}

}  // namespace
