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
//   2. per-expert totals, padded counts, a one-wavefront scan over experts, and each
//      wave's starting offset inside every expert segment;
//   3. stable scatter: a wave takes 64 items at a time; lanes holding the same
//      expert find each other with 8 ballots over the bits of the expert id
//      (E <= 256), so an item's rank among equal experts is a popcount. No
//      atomics decide positions, so the layout is deterministic: items ascend
//      inside a segment.
// Padding rows and the tail get the sentinel R; blocks past the padded total
// get expert -1.
//
// Large inputs (R >= 8192) run the same steps on many CUs, in three kernels, so
// that no single CU makes all the scattered stores: (1) each workgroup counts
// the experts of its chunk of 1024 items into a [G, E] table, kept in the
// inv_perm buffer until (3) overwrites it; (2) each workgroup sums the table
// (totals, and the items of earlier chunks per expert), scans the padded totals
// and places its chunk as in step 3 above, and a share of the blocks get their
// expert and sentinels; (3) inv_perm is the inverse of the placement. The
// layout is the same as the one-workgroup kernel's, bit for bit.
//
// Expert-parallel shard ("vLLM modular_kernel.py notes", expert_map: global
// expert id -> this rank's expert, -1 for experts on other ranks; "DeepGEMM
// FusedMoE on Blackwell", 2.6.2 ep_scatter skips items of remote experts): with
// a map, each id is looked up first; items whose expert is not local are
// neither counted nor placed and get inv_perm -1, so the GEMMs never see them
// and the reduce skips their slots.
#include "common.h"
#include "kernels.h"
#include "layout.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / MOE_WAVE;
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

    // 2. totals, padded sizes, scan over experts
    int n = 0, padded = 0;
    if (tid < E) {
        for (int w = 0; w < kWaves; ++w) n += wave_off[w][tid];
        padded = static_cast<int>(ceil_div(n, B) * B);
        count[tid] = n;
    }
    if (tid < kMaxE) seg_start[tid + 1] = tid < E ? padded : 0;
    if (tid == 0) seg_start[0] = 0;
    __syncthreads();
    // one wavefront scans the padded sizes: lane l sums experts 4l .. 4l+3, a
    // DPP scan over the lanes gives each lane its exclusive prefix
    if (wave == 0) scan_segments(seg_start, lane);
    __syncthreads();
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
        if (b * B < total) e = segment_of(seg_start, E, b * B);
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

// ---- multi-workgroup form -------------------------------------------------
constexpr int kMultiThreads = 256;
constexpr int kMultiWaves = kMultiThreads / MOE_WAVE;
constexpr int kChunk = 1024;  // items per workgroup (kMultiThreads * 4)
constexpr int64_t kMultiMinItems = 8192;

// (1) expert counts of chunk g into table[g][0:E]
__global__ __launch_bounds__(kMultiThreads) void align_count_kernel(
    const int32_t* __restrict__ ids, int64_t R, int E, const int32_t* __restrict__ emap, int E_global,
    int32_t* __restrict__ table) {
    __shared__ int32_t cnt[kMaxE];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kMultiThreads) cnt[e] = 0;
    __syncthreads();
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kChunk;
    const int64_t r1 = r0 + kChunk < R ? r0 + kChunk : R;
    for (int64_t r = r0 + tid; r < r1; r += kMultiThreads) {
        const int e = local_expert(ids[r], emap, E_global);
        if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kMultiThreads) table[static_cast<int64_t>(blockIdx.x) * E + e] = cnt[e];
}

// (2) segment starts from the table, this chunk's stable placement, and the expert
// and sentinels of blocks g, g + G, ...
__global__ __launch_bounds__(kMultiThreads) void align_place_kernel(
    const int32_t* __restrict__ ids, int64_t R, int E, int B, int64_t cap,
    const int32_t* __restrict__ emap, int E_global, const int32_t* __restrict__ table, int G,
    int32_t* __restrict__ sorted, int32_t* __restrict__ expert_ids, int32_t* __restrict__ npp_out) {
    __shared__ int32_t wave_off[kMultiWaves][kMaxE];
    __shared__ int32_t seg_start[kMaxE + 1];
    __shared__ int32_t count[kMaxE];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = blockIdx.x;

    // totals over all chunks and the items of chunks before g, per expert
    int n = 0, before = 0;
    if (tid < E) {
        // 32 loads in flight at a time
        for (int j0 = 0; j0 < G; j0 += 32) {
            int c[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) c[u] = j0 + u < G ? table[static_cast<int64_t>(j0 + u) * E + tid] : 0;
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                n += c[u];
                before += j0 + u < g ? c[u] : 0;
            }
        }
        count[tid] = n;
    }
    if (tid < kMaxE) seg_start[tid + 1] = tid < E ? static_cast<int>(ceil_div(n, B) * B) : 0;
    if (tid == 0) seg_start[0] = 0;
    for (int i = tid; i < kMultiWaves * kMaxE; i += kMultiThreads) (&wave_off[0][0])[i] = 0;
    __syncthreads();
    // (read after the barrier that follows the counts below)
    if (wave == 0) scan_segments(seg_start, lane);

    // per-wave counts of this chunk (wave w owns items [r0 + 256 w, r0 + 256 (w + 1)))
    const int64_t r0 = static_cast<int64_t>(g) * kChunk + wave * (kChunk / kMultiWaves);
    const int64_t end = r0 + kChunk / kMultiWaves;
    const int64_t r1 = end < R ? end : R;
    // the wave's 256 items, four per lane, loaded once for the counts and the placement
    constexpr int PER_LANE = kChunk / kMultiWaves / 64;
    int el[PER_LANE];
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) el[i] = r0 + i * 64 + lane < r1 ? ids[r0 + i * 64 + lane] : -1;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) el[i] = r0 + i * 64 + lane < r1 ? local_expert(el[i], emap, E_global) : -1;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i)
        if (static_cast<unsigned>(el[i]) < static_cast<unsigned>(E)) atomicAdd(&wave_off[wave][el[i]], 1);
    __syncthreads();
    if (tid < E) {
        int run = seg_start[tid] + before;
        for (int w = 0; w < kMultiWaves; ++w) {
            const int c = wave_off[w][tid];
            wave_off[w][tid] = run;
            run += c;
        }
    }
    const int total = seg_start[E];
    if (g == 0 && tid == 0) *npp_out = total;
    __syncthreads();

    // positions g * 256 + tid, stride 256 G: padding rows and the tail get the
    // sentinel, and each block start gives its block's expert
    for (int64_t pos = static_cast<int64_t>(g) * kMultiThreads + tid; pos < cap;
         pos += static_cast<int64_t>(G) * kMultiThreads) {
        int e = -1;
        if (pos < total) e = segment_of(seg_start, E, pos);
        if (pos % B == 0) expert_ids[pos / B] = e;
        if (e < 0 || pos >= seg_start[e] + count[e]) sorted[pos] = static_cast<int32_t>(R);
    }

    // stable placement (as in the one-workgroup kernel)
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const int64_t r = r0 + i * 64 + lane;
        const int e = el[i];
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
            sorted[wave_off[wave][e] + rank] = static_cast<int32_t>(r);
            if (lane == 63 - __clzll(peers)) wave_off[wave][e] += __popcll(peers);
        }
    }
}

// (3) inv_perm[sorted[pos]] = pos for real rows; -1 for items of experts held elsewhere
__global__ __launch_bounds__(256) void align_inverse_kernel(
    const int32_t* __restrict__ ids, int64_t R, int E, int64_t cap, const int32_t* __restrict__ emap,
    int E_global, const int32_t* __restrict__ sorted, int32_t* __restrict__ inv_perm) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < cap; i += stride) {
        const int r = sorted[i];
        if (r < R) inv_perm[r] = static_cast<int32_t>(i);
        if (i < R) {
            const int e = local_expert(ids[i], emap, E_global);
            if (static_cast<unsigned>(e) >= static_cast<unsigned>(E)) inv_perm[i] = -1;
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
    const int64_t G = ceil_div(R, kChunk);
    if (R < kMultiMinItems || G * E > R || G > (1 << 20)) {
        hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kThreads), 0, stream, ids, R, E, B, cap, emap,
                           E_global, sorted, expert_ids, npp, inv_perm);
        return hipGetLastError();
    }
    // the [G, E] count table lives in inv_perm (R entries) until the inverse pass
    hipLaunchKernelGGL(align_count_kernel, dim3(static_cast<unsigned>(G)), dim3(kMultiThreads), 0, stream,
                       ids, R, E, emap, E_global, inv_perm);
    hipLaunchKernelGGL(align_place_kernel, dim3(static_cast<unsigned>(G)), dim3(kMultiThreads), 0, stream,
                       ids, R, E, B, cap, emap, E_global, inv_perm, static_cast<int>(G), sorted, expert_ids, npp);
    const int64_t blocks = ceil_div(cap, 256);
    hipLaunchKernelGGL(align_inverse_kernel, dim3(static_cast<unsigned>(blocks < 2048 ? blocks : 2048)), dim3(256),
                       0, stream, ids, R, E, cap, emap, E_global, sorted, inv_perm);
    return hipGetLastError();
}
