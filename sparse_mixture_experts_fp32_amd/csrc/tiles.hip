// The m-tile list of the grouped GEMM over experts (the expert SwiGLU FFN of
// "Kimi K3: Open Frontier Intelligence", section "Operational Execution Flow":
// each expert applied to the rows routed to it, rows grouped by expert).
//
// Work unit of the expert GEMM: one m-tile (up to BM consecutive rows of one
// expert) x one n-tile of output columns. An expert with M rows gets
// ceil(M / BM) m-tiles of equal size (within one row). The list is built on the
// device from expert_offsets and every grid is sized from an upper bound on its
// length, so no token count ever goes back to the host (same page, section
// "Systems Optimization, Load Balancing, and Post-Training Alignment": waiting
// on dynamic per-expert counts stalls the device); surplus workgroups exit.
#include "device_common.h"
#include "launch.h"

namespace moe {

// One workgroup of 1024 threads; E <= 1024.
// tiles[i] = {expert, first row, rows, 0} for i < tile_start[E];
// tile_start[e] = index of expert e's first m-tile (tile_start[E] = number of m-tiles).
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                           int64_t n_rows, int bm, int max_tiles,
                                                           int4* __restrict__ tiles,
                                                           int32_t* __restrict__ tile_start) {
    __shared__ int32_t part[1024];
    const int tid = threadIdx.x;
    int lo = 0, cnt = 0, nt = 0;
    if (tid < E) {
        const int64_t a = min(max(static_cast<int64_t>(offsets[tid]), int64_t(0)), n_rows);
        const int64_t b = min(max(static_cast<int64_t>(offsets[tid + 1]), a), n_rows);
        lo = static_cast<int>(a);
        cnt = static_cast<int>(b - a);
        nt = (cnt + bm - 1) / bm;
    }
    part[tid] = nt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int32_t v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    const int start = part[tid] - nt;
    if (tid < E) tile_start[tid] = min(start, max_tiles);
    if (tid == 1023) tile_start[E] = min(part[1023], max_tiles);
    if (nt > 0) {
        // equal tiles (within one row): the workgroups that stream the same
        // expert's weights for different m-tiles then do the same work, stay in
        // step and share those weights through L2 (tiles rounded to 16 rows
        // drifted apart and re-read them from HBM)
        const int per = (cnt + nt - 1) / nt;
        for (int i = 0; i < nt; ++i) {
            const int r0 = i * per;
            const int rows = max(0, min(per, cnt - r0));
            if (start + i < max_tiles) tiles[start + i] = make_int4(tid, lo + r0, rows, 0);
        }
    }
}

static int max_tiles_for(int64_t n_rows, int E, int bm) {
    int64_t t = (n_rows + bm - 1) / bm + E;
    if (t > n_rows) t = n_rows;
    if (t < 1) t = 1;
    return static_cast<int>(t);
}

// m-tiles of up to 192 rows: 12 blocks of 16 rows, what one LDS-ring workgroup multiplies
int ffn_tile_rows() { return 192; }

// Capacity of a tile list: enough for m-tiles of 128 rows, shorter than any pass uses
// (bf16 192 rows, MX 144), so one workspace serves every pass.
constexpr int kMinTileRows = 128;
int ffn_max_tiles(int64_t n_rows, int E) { return max_tiles_for(n_rows, E, kMinTileRows); }

hipError_t launch_build_tiles_rows(const int32_t* expert_offsets, int64_t n_rows, int E, int bm, int4* tiles,
                                   int32_t* tile_start, hipStream_t stream) {
    if (bm < kMinTileRows || bm % 16 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, stream, expert_offsets, E, n_rows, bm,
                       ffn_max_tiles(n_rows, E), tiles, tile_start);
    return hipGetLastError();
}

hipError_t launch_build_tiles(const int32_t* expert_offsets, int64_t n_rows, int E, int4* tiles,
                              int32_t* tile_start, hipStream_t stream) {
    return launch_build_tiles_rows(expert_offsets, n_rows, E, ffn_tile_rows(), tiles, tile_start, stream);
}

}  // namespace moe
