// align.hip -- expert-sorted, block-padded layout of the routed items.
//
// "fused_moe.py analysis", "moe_align_block_size": the (token, slot) pairs are
// flattened, grouped by expert and each expert's count is padded to a
// multiple of BLOCK_M, giving sorted_token_ids, expert_ids (one per block)
// and num_tokens_post_padded. "DeepGEMM FusedMoE on Blackwell", 2.6.2: a
// prefix sum of the padded counts gives each expert's start row, and
// inv_perm maps each (token, slot) back to its row.
//
// gfx950 design: one 1024-thread workgroup (16 wavefronts). Each wavefront
// owns a contiguous chunk of items.
//   1. per-wave expert histogram in LDS (counts do not depend on order);
//   2. per-expert totals, padded counts, an LDS scan over experts, and each
//      wave's starting offset inside every expert segment;
//   3. stable scatter: a wave takes 64 items at a time; lanes holding the same
//      expert find each other with 8 ballots over the bits of the expert id
//      (E <= 256), so an item's rank among equal experts is a popcount. No
//      atomics decide positions, so the layout is deterministic: items ascend
//      inside a segment.
// Padding rows and the tail get the sentinel R; blocks past the padded total
// get expert -1.
//
// Expert-parallel shard ("vLLM modular_kernel.py notes", expert_map: global
// expert id -> this rank's expert, -1 for experts on other ranks; "DeepGEMM
// FusedMoE on Blackwell", 2.6.2 ep_scatter skips items of remote experts): with
// a map, each id is looked up first; items whose expert is not local are
// neither counted nor placed and get inv_perm -1, so the GEMMs never see them
// and the reduce skips their slots.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / MOE_WAVE;
constexpr int kMaxE = 256;

// this rank's expert of global id `id`: the id itself without a map; ids outside
// the routing range and map entries outside [0, E) count as not local (-1)
__device__ __forceinline__ int local_expert(int id, const int32_t* __restrict__ emap, int E_global) {
    if (emap == nullptr) return id;
    return static_cast<unsigned>(id) < static_cast<unsigned>(E_global) ? emap[id] : -1;
}

__global__ __launch_bounds__(kThreads) void align_kernel(
    const int32_t* __restrict__ ids, int64_t R, int E, int B, int64_t cap,
    const int32_t* __restrict__ emap, int E_global,
    int32_t* __restrict__ sorted, int32_t* __restrict__ expert_ids, int32_t* __restrict__ npp_out,
    int32_t* __restrict__ inv_perm) {
    __shared__ int32_t wave_off[kWaves][kMaxE];  // counts, then running offsets
    __shared__ int32_t seg_start[kMaxE + 1];     // padded segment starts
    __shared__ int32_t count[kMaxE];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int i = tid; i < kWaves * kMaxE; i += kThreads) (&wave_off[0][0])[i] = 0;
    __syncthreads();

    const int64_t chunk = ceil_div(ceil_div(R, kWaves), 64) * 64;
    const int64_t c0 = wave * chunk;
    const int64_t c1 = c0 + chunk < R ? c0 + chunk : R;

    // 1. histogram
    for (int64_t r = c0 + lane; r < c1; r += 64) {
        const int e = local_expert(ids[r], emap, E_global);
        if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&wave_off[wave][e], 1);
    }
    __syncthreads();

    // 2. totals, padded sizes, scan over experts (Hillis-Steele in LDS)
    int n = 0, padded = 0;
    if (tid < E) {
        for (int w = 0; w < kWaves; ++w) n += wave_off[w][tid];
        padded = static_cast<int>(ceil_div(n, B) * B);
        count[tid] = n;
    }
    if (tid < kMaxE) seg_start[tid + 1] = tid < E ? padded : 0;
    if (tid == 0) seg_start[0] = 0;
    __syncthreads();
    for (int d = 1; d < kMaxE; d <<= 1) {
        int add = 0;
        if (tid < kMaxE && tid + 1 - d >= 1) add = seg_start[tid + 1 - d];
        __syncthreads();
        if (tid < kMaxE) seg_start[tid + 1] += add;
        __syncthreads();
    }
    // seg_start[e] is now the inclusive sum over experts < e of padded sizes
    if (tid < E) {
        int run = seg_start[tid];
        for (int w = 0; w < kWaves; ++w) {
            const int c = wave_off[w][tid];
            wave_off[w][tid] = run;
            run += c;
        }
    }
    const int total = seg_start[E];
    if (tid == 0) *npp_out = total;
    __syncthreads();

    // expert of every block, and the sentinel in padding rows and the tail
    const int64_t nblocks = cap / B;
    for (int64_t b = tid; b < nblocks; b += kThreads) {
        int e = -1;
        if (b * B < total) {
            int lo = 0, hi = E - 1;  // last e with seg_start[e] <= b*B
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (seg_start[mid] <= b * B) lo = mid; else hi = mid - 1;
            }
            e = lo;
        }
        expert_ids[b] = e;
        const int64_t s = e < 0 ? b * B : seg_start[e] + count[e];
        for (int64_t pos = b * B > s ? b * B : s; pos < (b + 1) * B; ++pos)
            sorted[pos] = static_cast<int32_t>(R);
    }

    // 3. stable scatter
    for (int64_t base = c0; base < c1; base += 64) {
        const int64_t r = base + lane;
        const int e = r < c1 ? local_expert(ids[r], emap, E_global) : -1;
        const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
        uint64_t peers = ballot64(valid);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool set = (e >> bit) & 1;
            const uint64_t m = ballot64(set);
            peers &= set ? m : ~m;
        }
        if (valid) {
            const int rank = __popcll(peers & ((1ull << lane) - 1ull));
            const int pos = wave_off[wave][e] + rank;
            sorted[pos] = static_cast<int32_t>(r);
            inv_perm[r] = pos;
            if (lane == 63 - __clzll(peers)) wave_off[wave][e] += __popcll(peers);
        } else if (r < c1) {
            inv_perm[r] = -1;
        }
    }
}

// batched form ("vLLM modular_kernel.py notes", BatchedExperts: E batches of
// max_M rows with per-expert counts): one top-1 id per row, -1 past the count
__global__ __launch_bounds__(256) void batched_ids_kernel(const int32_t* __restrict__ counts, int E,
                                                          int64_t max_M, int32_t* __restrict__ ids) {
    const int64_t n = E * max_M;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; r < n;
         r += static_cast<int64_t>(gridDim.x) * 256) {
        const int e = static_cast<int>(r / max_M);
        ids[r] = r - e * max_M < counts[e] ? e : -1;
    }
}

}  // namespace

hipError_t launch_batched_ids(const int32_t* counts, int E, int64_t max_M, int32_t* ids, hipStream_t stream) {
    const int64_t blocks = ceil_div(E * max_M, 256);
    const dim3 grid(static_cast<unsigned>(blocks < 4096 ? blocks : 4096));
    hipLaunchKernelGGL(batched_ids_kernel, grid, dim3(256), 0, stream, counts, E, max_M, ids);
    return hipGetLastError();
}

hipError_t launch_align(const int32_t* ids, int64_t R, int E, int B, int64_t cap,
                        const int32_t* emap, int E_global, int32_t* sorted, int32_t* expert_ids,
                        int32_t* npp, int32_t* inv_perm, hipStream_t stream) {
    hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kThreads), 0, stream, ids, R, E, B, cap, emap,
                       E_global, sorted, expert_ids, npp, inv_perm);
    return hipGetLastError();
}
