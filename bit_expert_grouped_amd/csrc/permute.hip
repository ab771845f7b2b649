// Permute kernels for gfx950: per-expert histogram, exclusive scan, slot
// scatter, and the device-side tile map that the grouped products walk.
//
// Pages: routing is closed on the GPU with no per-layer host synchronisation
// (aimanavo.com page, section "Lily does not treat prefill and decode as the
// same job"; dzen.guru page, section "Where does the speed-up come from?").  The
// grouped products are therefore launched with a grid sized from T alone and
// read the tile map written here.
//
// Step-by-step call: one workgroup of 1024 threads does everything in LDS
// (histogram with LDS atomics, block scans, scatter with LDS cursors).  Layer
// call: scatter_kernel after the top-k kernel's histogram.  Rows of one expert
// come out in an unspecified order (atomic order); counts and offsets are
// exact.  Expert indices outside [0, E) are skipped.
#include "common.h"
#include "kernels.h"

namespace bitmoe {

namespace {

constexpr int kThreads = 1024;

// Inclusive scan over the block; `tmp` holds kThreads/64 ints.  `total`
// (optional) receives the sum over the block.
__device__ int block_inclusive_scan(int v, int* tmp, int* total = nullptr) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    if (lane == kWave - 1) tmp[wave] = v;
    __syncthreads();
    if (wave == 0) {
        int s = lane < kThreads / kWave ? tmp[lane] : 0;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            int o = __shfl_up(s, off);
            if (lane >= off) s += o;
        }
        if (lane < kThreads / kWave) tmp[lane] = s;
    }
    __syncthreads();
    int r = v + (wave > 0 ? tmp[wave - 1] : 0);
    if (total) *total = tmp[kThreads / kWave - 1];
    __syncthreads();
    return r;
}

// Tiles of a group of n rows: n / tr full tiles of tr (kTileRows or 64) rows
// and one tile of the remainder, so at most 31 rows of a group are MFMA padding.  Thread g (< E, or
// == E for the shared expert) writes the tiles of group g.  The map lists the
// tiles longest first (full tiles, then remainders of 96, 64 and 32 rows or
// fewer), so the grouped products start the long work first and end on short
// tiles.  Tiles beyond `cap` (the workspace capacity) are dropped, so
// inconsistent caller offsets cannot write outside the tile array.
//
// The positions are exclusive scans of each height class's tile counts over
// the groups, one class per wave, all classes at once: lane l of wave q sums
// groups 5 l .. 5 l + 4 of class q, and one wave-wide scan of those sums gives
// every group's start within the class.
constexpr int kTileGroups = kMaxE + 1;                      // routed experts + the shared one
constexpr int kGroupsPerLane = (kTileGroups + kWave - 1) / kWave;  // 5
constexpr int kMaxClasses = kTileRows / 32;                 // 4

__device__ void write_tiles(int g_rows, int row_base, Tile* tiles, int32_t* n_tiles, int cap, int tr) {
    __shared__ int cnt[kMaxClasses][kGroupsPerLane * kWave];
    __shared__ int start[kMaxClasses][kGroupsPerLane * kWave];
    __shared__ int total[kMaxClasses];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int nq = tr / 32;  // class q holds tiles of 32 (nq - q) rows
    const int n = tid < kTileGroups ? max(g_rows, 0) : 0;
    const int full = n / tr, rem = n % tr;
    const int mt_rem = (rem + 31) / 32;  // 0 .. nq
    auto count = [&](int q) { return (q == 0 ? full : 0) + (mt_rem == nq - q ? 1 : 0); };
    for (int i = tid; i < kGroupsPerLane * kWave; i += blockDim.x)
        for (int q = 0; q < nq; q++) cnt[q][i] = 0;
    __syncthreads();
    if (tid < kTileGroups)
        for (int q = 0; q < nq; q++) cnt[q][tid] = count(q);
    __syncthreads();
    if (wave < nq) {
        const int q = wave;
        int v[kGroupsPerLane], sum = 0;
#pragma unroll
        for (int i = 0; i < kGroupsPerLane; i++) {
            v[i] = cnt[q][lane * kGroupsPerLane + i];
            sum += v[i];
        }
        int incl = sum;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int o = __shfl_up(incl, off);
            if (lane >= off) incl += o;
        }
        int run = incl - sum;
#pragma unroll
        for (int i = 0; i < kGroupsPerLane; i++) {
            start[q][lane * kGroupsPerLane + i] = run;
            run += v[i];
        }
        if (lane == kWave - 1) total[q] = incl;
    }
    __syncthreads();
    int first_of_class = 0;
    for (int q = 0; q < nq; q++) {
        const int c = count(q);
        int pos = first_of_class + (tid < kTileGroups ? start[q][tid] : 0);
        for (int j = 0; j < c && pos < cap; j++, pos++) {
            const bool is_rem = j == c - 1 && mt_rem == nq - q;
            Tile t;
            t.group = tid;
            t.row0 = row_base + (is_rem ? full : j) * tr;
            t.rows = is_rem ? rem : tr;
            t.pad = 0;
            tiles[pos] = t;
        }
        first_of_class += total[q];
    }
    if (tid == 0) *n_tiles = min(first_of_class, cap);
    __syncthreads();  // the LDS arrays may be reused by a following call
}

__global__ __launch_bounds__(kThreads) void permute_kernel(const int32_t* __restrict__ topk_idx, int T,
                                                           int k, int E, int shared,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_slot,
                                                           Tile* __restrict__ tiles,
                                                           int32_t* __restrict__ n_tiles, int cap) {
    __shared__ int hist[kMaxE];
    __shared__ int cursor[kMaxE];
    __shared__ int tmp[kThreads / kWave];
    const int tid = threadIdx.x;
    const int n = T * k;
    if (tid < kMaxE) hist[tid] = 0;
    __syncthreads();
    for (int s = tid; s < n; s += kThreads) {
        const int e = topk_idx[s];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    const int c = tid < E ? hist[tid] : 0;
    const int incl = block_inclusive_scan(c, tmp);
    const int excl = incl - c;
    if (tid < E) {
        cursor[tid] = excl;
        offsets[tid] = excl;
        if (counts) counts[tid] = c;
    }
    if (tid == E - 1) offsets[E] = incl;
    const int g_rows = tid < E ? c : ((tid == E && shared) ? T : 0);
    const int row_base = tid < E ? excl : n;
    write_tiles(g_rows, row_base, tiles, n_tiles, cap, kTileRows);
    __syncthreads();
    for (int s = tid; s < n; s += kThreads) {
        const int e = topk_idx[s];
        if (e >= 0 && e < E) sorted_slot[atomicAdd(&cursor[e], 1)] = s;
    }
}

__global__ __launch_bounds__(kThreads) void tiles_kernel(const int32_t* __restrict__ offsets, int T, int k,
                                                         int E, int shared, Tile* __restrict__ tiles,
                                                         int32_t* __restrict__ n_tiles, int cap) {
    const int tid = threadIdx.x;
    int g_rows = 0, row_base = T * k;
    if (tid < E) {
        row_base = offsets[tid];
        g_rows = offsets[tid + 1] - row_base;
    } else if (tid == E && shared) {
        g_rows = T;
    }
    write_tiles(g_rows, row_base, tiles, n_tiles, cap, kTileRows);
}

// The layer's permute after topk_kernel has counted the histogram: every
// workgroup scans the counts itself (E <= 256 values), workgroup 0 also writes
// the offsets and the tile map, and each workgroup places its 1024 slots: ranks
// within the workgroup from LDS atomics, one global atomic per (workgroup,
// expert) on a per-expert cursor (zeroed before the top-k) to reserve the run,
// so the scatter spreads over ceil(T k / 1024) workgroups with little
// contention on the cursors.
__global__ __launch_bounds__(kThreads) void scatter_kernel(const int32_t* __restrict__ topk_idx,
                                                           const int32_t* __restrict__ hist, int T, int k,
                                                           int E, int shared, int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ cursor,
                                                           int32_t* __restrict__ sorted_slot,
                                                           Tile* __restrict__ tiles, int32_t* __restrict__ n_tiles,
                                                           int cap, int tr, Tile* __restrict__ tiles2,
                                                           int32_t* __restrict__ n_tiles2, int cap2) {
    __shared__ int off[kMaxE];
    __shared__ int local[kMaxE];  // this workgroup's slots per expert, then their global base
    __shared__ int tmp[kThreads / kWave];
    const int tid = threadIdx.x;
    const int n = T * k;
    // this thread's slot goes out first: its load overlaps the counts' loads
    // and the scan below
    const int s = blockIdx.x * kThreads + tid;
    const int e = topk_idx[min(s, n - 1)];
    if (tid < kMaxE) local[tid] = 0;
    const int c =
        tid < E ? __hip_atomic_load(hist + tid * kCounterStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
    const int incl = block_inclusive_scan(c, tmp);
    const int excl = incl - c;
    if (tid < E) off[tid] = excl;
    if (blockIdx.x == 0) {
        if (tid < E) {
            offsets[tid] = excl;
            if (counts) counts[tid] = c;
        }
        if (tid == E - 1) offsets[E] = incl;
        const int g_rows = tid < E ? c : ((tid == E && shared) ? T : 0);
        const int row_base = tid < E ? excl : n;
        write_tiles(g_rows, row_base, tiles, n_tiles, cap, tr);
    }
    // the second map from workgroup 1 (0 if alone), beside workgroup 0's
    if (tiles2 && blockIdx.x == (gridDim.x > 1 ? 1u : 0u)) {
        const int g_rows = tid < E ? c : ((tid == E && shared) ? T : 0);
        const int row_base = tid < E ? excl : n;
        write_tiles(g_rows, row_base, tiles2, n_tiles2, cap2, 64);
    }
    __syncthreads();
    // rank each slot among this workgroup's slots of its expert (LDS atomics),
    // then reserve the workgroup's run of each expert with one global atomic
    const bool valid = s < n && e >= 0 && e < E;
    const int rank = valid ? atomicAdd(&local[e], 1) : 0;
    __syncthreads();
    // a lone workgroup holds every slot: its runs start at the offsets, with
    // no global cursor to reserve them from
    if (tid < E && local[tid] > 0)
        local[tid] = off[tid] + (gridDim.x == 1 ? 0 : atomicAdd(cursor + tid * kCounterStride, local[tid]));
    __syncthreads();
    if (valid) sorted_slot[local[e] + rank] = s;
}

}  // namespace

hipError_t launch_permute(const int32_t* topk_idx, int T, int k, int E, bool shared, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_slot, Tile* tiles, int32_t* n_tiles,
                          hipStream_t stream) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kThreads), 0, stream, topk_idx, T, k, E, shared ? 1 : 0,
                       counts, offsets, sorted_slot, tiles, n_tiles, (int)max_tiles(T, k, E, shared));
    return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* topk_idx, const int32_t* hist, int T, int k, int E, bool shared,
                          int32_t* counts, int32_t* offsets, int32_t* cursor, int32_t* sorted_slot, Tile* tiles,
                          int32_t* n_tiles, int tile_rows, Tile* tiles64, int32_t* n_tiles64,
                          hipStream_t stream) {
    if (tile_rows != kTileRows && tile_rows != 64) return hipErrorInvalidValue;
    const int n = T * k;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(scatter_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, stream, topk_idx,
                       hist, T, k, E, shared ? 1 : 0, counts, offsets, cursor, sorted_slot, tiles, n_tiles,
                       (int)max_tiles(T, k, E, shared, tile_rows), tile_rows, tiles64, n_tiles64,
                       (int)max_tiles(T, k, E, shared, 64));
    return hipGetLastError();
}

hipError_t launch_tiles(const int32_t* offsets, int T, int k, int E, bool shared, Tile* tiles,
                        int32_t* n_tiles, hipStream_t stream) {
    hipLaunchKernelGGL(tiles_kernel, dim3(1), dim3(kThreads), 0, stream, offsets, T, k, E, shared ? 1 : 0,
                       tiles, n_tiles, (int)max_tiles(T, k, E, shared));
    return hipGetLastError();
}

}  // namespace bitmoe
