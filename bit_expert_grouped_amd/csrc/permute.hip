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

// Inclusive scan over the block; `tmp` holds kThreads/64 ints.
__device__ int block_inclusive_scan(int v, int* tmp) {
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
    __syncthreads();
    return r;
}

// Rows per tile for a group of n rows: split into ceil(n / kTileRows) near-equal
// chunks rounded up to the 32-row MFMA tile.
__device__ void chunking(int n, int* rows_per_tile, int* ntiles) {
    if (n <= 0) {
        *rows_per_tile = kTileRows;
        *ntiles = 0;
        return;
    }
    int nch = (n + kTileRows - 1) / kTileRows;
    int cs = (n + nch - 1) / nch;
    cs = (cs + 31) / 32 * 32;
    *rows_per_tile = cs;
    *ntiles = (n + cs - 1) / cs;
}

// Thread g (< E, or == E for the shared expert) writes the tiles of group g.
// Tiles beyond `cap` (the workspace capacity) are dropped, so inconsistent
// caller offsets cannot write outside the tile array.
__device__ void write_tiles(int g_rows, int row_base, int* tmp, Tile* tiles, int32_t* n_tiles, int cap) {
    int cs, nt;
    chunking(g_rows, &cs, &nt);
    const int incl = block_inclusive_scan(nt, tmp);
    const int first = incl - nt;
    for (int c = 0; c < nt && first + c < cap; c++) {
        Tile t;
        t.group = threadIdx.x;
        t.row0 = row_base + c * cs;
        t.rows = min(cs, g_rows - c * cs);
        t.pad = 0;
        tiles[first + c] = t;
    }
    if (threadIdx.x == kThreads - 1) *n_tiles = min(incl, cap);
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
    write_tiles(g_rows, row_base, tmp, tiles, n_tiles, cap);
    __syncthreads();
    for (int s = tid; s < n; s += kThreads) {
        const int e = topk_idx[s];
        if (e >= 0 && e < E) sorted_slot[atomicAdd(&cursor[e], 1)] = s;
    }
}

__global__ __launch_bounds__(kThreads) void tiles_kernel(const int32_t* __restrict__ offsets, int T, int k,
                                                         int E, int shared, Tile* __restrict__ tiles,
                                                         int32_t* __restrict__ n_tiles, int cap) {
    __shared__ int tmp[kThreads / kWave];
    const int tid = threadIdx.x;
    int g_rows = 0, row_base = T * k;
    if (tid < E) {
        row_base = offsets[tid];
        g_rows = offsets[tid + 1] - row_base;
    } else if (tid == E && shared) {
        g_rows = T;
    }
    write_tiles(g_rows, row_base, tmp, tiles, n_tiles, cap);
}

// The layer's permute after topk_kernel has counted the histogram: every
// workgroup scans the counts itself (E <= 256 values), workgroup 0 also writes
// the offsets and the tile map, and each thread places one slot through a
// global per-expert cursor (zeroed before the top-k), so the scatter spreads
// over ceil(T k / 1024) workgroups instead of one.
__global__ __launch_bounds__(kThreads) void scatter_kernel(const int32_t* __restrict__ topk_idx,
                                                           const int32_t* __restrict__ hist, int T, int k,
                                                           int E, int shared, int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ cursor,
                                                           int32_t* __restrict__ sorted_slot,
                                                           Tile* __restrict__ tiles, int32_t* __restrict__ n_tiles,
                                                           int cap) {
    __shared__ int off[kMaxE];
    __shared__ int tmp[kThreads / kWave];
    const int tid = threadIdx.x;
    const int n = T * k;
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
        write_tiles(g_rows, row_base, tmp, tiles, n_tiles, cap);
    }
    __syncthreads();
    const int s = blockIdx.x * kThreads + tid;
    if (s < n) {
        const int e = topk_idx[s];
        if (e >= 0 && e < E) sorted_slot[off[e] + atomicAdd(cursor + e * kCounterStride, 1)] = s;
    }
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
                          int32_t* n_tiles, hipStream_t stream) {
    const int n = T * k;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(scatter_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, stream, topk_idx,
                       hist, T, k, E, shared ? 1 : 0, counts, offsets, cursor, sorted_slot, tiles, n_tiles,
                       (int)max_tiles(T, k, E, shared));
    return hipGetLastError();
}

hipError_t launch_tiles(const int32_t* offsets, int T, int k, int E, bool shared, Tile* tiles,
                        int32_t* n_tiles, hipStream_t stream) {
    hipLaunchKernelGGL(tiles_kernel, dim3(1), dim3(kThreads), 0, stream, offsets, T, k, E, shared ? 1 : 0,
                       tiles, n_tiles, (int)max_tiles(T, k, E, shared));
    return hipGetLastError();
}

}  // namespace bitmoe
