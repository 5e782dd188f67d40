// Grouped GEMM over experts on bf16 MFMA (float32 accumulation): the expert
// SwiGLU FFN of "Kimi K3: Open Frontier Intelligence", section "Operational
// Execution Flow" (SwiGLU-form experts applied to the rows routed to them).
//
//   gate/up pass: H[r, n] = silu(sum_i A[r, i] Wg[e, n, i]) * (sum_i A[r, i] Wu[e, n, i])
//   down pass:    Y[r, n] = sum_i H[r, i] Wd[e, n, i]
// for every row r of expert e (rows grouped by expert, contiguous). H is
// rounded once to bf16 (the down pass's MFMA operand); Y stays float32.
//
// Work unit: one m-tile (up to BM consecutive rows of one expert) x one n-tile
// of output columns. An expert with M rows gets ceil(M / BM) m-tiles of nearly
// equal size. The m-tile list is built on the device from expert_offsets and
// the grid is sized from an upper bound, so no token count ever goes back to
// the host; surplus workgroups find no work and exit.
//
// Inside a workgroup (8 wavefronts): the A rows of the current K step (128
// deep) are staged in LDS, double-buffered, and shared by all waves; each wave
// streams its own weight rows straight from HBM into registers, one K step
// ahead of the matrix cores (each weight byte is used by exactly one wave, so
// staging it in LDS would buy nothing). Weights are stored [N, K] (K
// contiguous), so one lane's 8 consecutive k values are a single 16-byte load
// that is directly an MFMA operand. The K loop is unrolled by two so the two
// register sets of weights swap roles without copies, and rows past the tile
// end are clamped to its last row, so every load is unconditional: the wait
// before each step's MFMAs then covers only that step's weights, never the
// loads already issued for the next step.
//
// Scheduling for the 8 XCDs (each with its own L2): workgroup ids are dealt to
// the XCDs round-robin, so XCD x runs ids x, x + 8, x + 16, ... in order. The
// m-tile list is cut into 8 contiguous chunks, one per XCD, and inside a chunk
// the work is ordered expert by expert, n-tile by n-tile, with the expert's
// m-tiles innermost. The m-tiles that share one weight n-tile therefore run
// side by side on one XCD and fetch those weights from HBM once (the others
// hit in L2), and all n-tiles of an expert follow each other, so its A rows
// stay in that L2 as well.
#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kGemmWaves = 8;
constexpr int kGemmThreads = kGemmWaves * 64;
constexpr int kKStep = 128;
constexpr int kAStride = kKStep + 8;  // bf16 per LDS row: 272 B keeps 16-B reads conflict-free
constexpr int kXcds = 8;
constexpr int kMaxRowBlocks = 8;      // m-tile of up to 128 rows

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
        // nearly equal tiles, each a multiple of 16 rows except the last
        const int per = ((cnt + nt - 1) / nt + 15) / 16 * 16;
        for (int i = 0; i < nt; ++i) {
            const int r0 = i * per;
            const int rows = max(0, min(per, cnt - r0));
            if (start + i < max_tiles) tiles[start + i] = make_int4(tid, lo + r0, rows, 0);
        }
    }
}

// Register-array helpers of the K loop (force-inlined so the arrays stay in registers).
template <int kP>
__device__ __forceinline__ void load_rows(u32x4 (&dst)[kP], const uint16_t* src, const int64_t (&off)[kP], int k0) {
#pragma unroll
    for (int p = 0; p < kP; ++p) dst[p] = *reinterpret_cast<const u32x4*>(src + off[p] + k0);
}

template <int kP>
__device__ __forceinline__ void store_rows(uint16_t* dst, const u32x4 (&src)[kP]) {
#pragma unroll
    for (int p = 0; p < kP; ++p) *reinterpret_cast<u32x4*>(dst + p * 32 * kAStride) = src[p];
}

__device__ __forceinline__ void load_weights(bf16x8 (&dst)[2][4], const uint16_t* w0, const uint16_t* w1, int k0) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        dst[0][s] = *reinterpret_cast<const bf16x8*>(w0 + k0 + 32 * s);
        dst[1][s] = *reinterpret_cast<const bf16x8*>(w1 + k0 + 32 * s);
    }
}

// acc[b][m] += (A rows 16m .. 16m+15 of one K step, from LDS) x (weight block b).
template <int kMB>
__device__ __forceinline__ void mfma_step(f32x4 (&acc)[2][kMB], const uint16_t* frag, const bf16x8 (&bw)[2][4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int m = 0; m < kMB; ++m) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(frag + m * 16 * kAStride + 32 * s);
            acc[0][m] = mfma_16x16x32(a, bw[0][s], acc[0][m]);
            acc[1][m] = mfma_16x16x32(a, bw[1][s], acc[1][m]);
        }
    }
}

// One (m-tile, n-tile) work item with kMB row blocks of 16 (M <= 16 * kMB rows).
// Every load and LDS store in the K loop is unconditional: rows past M re-read
// row M - 1 and the prefetch index is clamped to the last K step (a repeated
// step is loaded but never used), so the compiler's wait before each MFMA
// group covers only the weights that group consumes.
template <bool kGated, int kMB>
__device__ __forceinline__ void ffn_tile(uint16_t* sA, const uint16_t* __restrict__ A, int64_t row0, int M,
                                         const uint16_t* wb0, const uint16_t* wb1, bool wave_on, int N, int K,
                                         int n_wave, void* __restrict__ Cout) {
    constexpr int kAPasses = (kMB * 16 + 31) / 32;  // 16 threads x 16 B per row, 32 rows per pass
    constexpr int kBufElems = 16 * kMaxRowBlocks * kAStride;
    const int tid = threadIdx.x, lane = tid & 63;
    const int frag_row = lane & 15, frag_k = 8 * (lane >> 4);

    const int a_row = tid >> 4, a_col = 8 * (tid & 15);
    const bool a_on = a_row < 16 * kMB;  // kMB == 1: only the first 16 rows are staged
    const uint16_t* a_src = A + row0 * K + a_col;
    int64_t a_off[kAPasses];
#pragma unroll
    for (int p = 0; p < kAPasses; ++p) a_off[p] = static_cast<int64_t>(min(p * 32 + a_row, M - 1)) * K;
    uint16_t* a_dst0 = sA + a_row * kAStride + a_col;
    uint16_t* a_dst1 = a_dst0 + kBufElems;
    const uint16_t* a_frag0 = sA + frag_row * kAStride + frag_k;
    const uint16_t* a_frag1 = a_frag0 + kBufElems;

    f32x4 acc[2][kMB];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int m = 0; m < kMB; ++m) acc[b][m] = f32x4{0.f, 0.f, 0.f, 0.f};

    // K loop over pairs of steps: register sets b0 / b1 and LDS buffers 0 / 1
    // alternate between "being consumed" and "being filled", without copies.
    const int nk = K / kKStep;
    u32x4 a_reg[kAPasses];
    bf16x8 b0[2][4], b1[2][4];
    load_rows(a_reg, a_src, a_off, 0);
    load_weights(b0, wb0, wb1, 0);
    if (a_on) store_rows(a_dst0, a_reg);
    __syncthreads();
    for (int s0 = 0; s0 < nk; s0 += 2) {
        const int k1 = min(s0 + 1, nk - 1) * kKStep;
        load_rows(a_reg, a_src, a_off, k1);
        load_weights(b1, wb0, wb1, k1);
        if (wave_on) mfma_step(acc, a_frag0, b0);
        if (a_on) store_rows(a_dst1, a_reg);
        __syncthreads();
        const int k2 = min(s0 + 2, nk - 1) * kKStep;
        load_rows(a_reg, a_src, a_off, k2);
        load_weights(b0, wb0, wb1, k2);
        if (wave_on && s0 + 1 < nk) mfma_step(acc, a_frag1, b1);
        if (a_on) store_rows(a_dst0, a_reg);
        __syncthreads();
    }

    if (!wave_on) return;
    const int col = n_wave + frag_row;
#pragma unroll
    for (int m = 0; m < kMB; ++m) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = m * 16 + 4 * (lane >> 4) + q;
            if (r >= M) continue;
            if (kGated) {  // H row: bf16, the operand of the down pass
                uint16_t* crow = static_cast<uint16_t*>(Cout) + (row0 + r) * N;
                const float g = acc[0][m][q], u = acc[1][m][q];
                crow[col] = f32_to_bf16_bits(g / (1.0f + __expf(-g)) * u);
            } else {       // Y row: float32
                float* crow = static_cast<float*>(Cout) + (row0 + r) * N;
                crow[col] = acc[0][m][q];
                crow[col + 16] = acc[1][m][q];
            }
        }
    }
}

template <bool kGated>
__global__ __launch_bounds__(kGemmThreads) void grouped_ffn_kernel(
    const uint16_t* __restrict__ A, const int4* __restrict__ tiles, const int32_t* __restrict__ tile_start,
    int E, int n_tiles, const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1, int N, int K,
    void* __restrict__ Cout) {
    constexpr int kColsW = kGated ? 16 : 32;  // output columns per wave
    constexpr int kColsWG = kColsW * kGemmWaves;
    __shared__ __attribute__((aligned(16))) uint16_t sA[2 * 16 * kMaxRowBlocks * kAStride];

    // ---- work item: (m-tile, n-tile) from the XCD-ordered schedule
    const int n_mt = tile_start[E];
    const int xcd = blockIdx.x % kXcds;
    const int j = blockIdx.x / kXcds;
    const int lo = static_cast<int>(static_cast<int64_t>(xcd) * n_mt / kXcds);
    const int hi = static_cast<int>(static_cast<int64_t>(xcd + 1) * n_mt / kXcds);
    const int slot = j / n_tiles;
    if (lo + slot >= hi) return;  // uniform for the whole workgroup, before any barrier
    const int e = tiles[lo + slot].x;
    const int g0 = max(lo, tile_start[e]);
    const int g1 = min(hi, tile_start[e + 1]);
    const int gs = g1 - g0;
    const int rr = j - (g0 - lo) * n_tiles;
    const int nt = rr / gs;
    const int4 tile = tiles[g0 + rr % gs];
    const int M = tile.z;
    if (M <= 0) return;
    const int64_t row0 = tile.y;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_wave = nt * kColsWG + wave * kColsW;
    const bool wave_on = n_wave < N;  // uniform per wave
    const int frag_row = lane & 15, frag_k = 8 * (lane >> 4);

    // weight rows of this lane for the two B blocks (an idle wave reads valid rows it never uses)
    const int n_safe = wave_on ? n_wave : 0;
    const int64_t wexp = static_cast<int64_t>(e) * N * K;
    const uint16_t* wb0 = W0 + wexp + static_cast<int64_t>(n_safe + frag_row) * K + frag_k;
    const uint16_t* wb1 = kGated ? W1 + wexp + static_cast<int64_t>(n_safe + frag_row) * K + frag_k
                                 : W0 + wexp + static_cast<int64_t>(n_safe + 16 + frag_row) * K + frag_k;

    // one straight-line K loop per row-block count, chosen once per tile
    if (M <= 32)
        ffn_tile<kGated, 2>(sA, A, row0, M, wb0, wb1, wave_on, N, K, n_wave, Cout);
    else if (M <= 64)
        ffn_tile<kGated, 4>(sA, A, row0, M, wb0, wb1, wave_on, N, K, n_wave, Cout);
    else
        ffn_tile<kGated, kMaxRowBlocks>(sA, A, row0, M, wb0, wb1, wave_on, N, K, n_wave, Cout);
}

// ---------------------------------------------------------------- launchers

int ffn_tile_rows() { return 16 * kMaxRowBlocks; }

int ffn_max_tiles(int64_t n_rows, int E) {
    const int64_t bm = ffn_tile_rows();
    int64_t t = (n_rows + bm - 1) / bm + E;
    if (t > n_rows) t = n_rows;
    if (t < 1) t = 1;
    return static_cast<int>(t);
}

static int xcd_slots(int max_tiles) { return (max_tiles + kXcds - 1) / kXcds; }

hipError_t launch_build_tiles(const int32_t* expert_offsets, int64_t n_rows, int E, int4* tiles,
                              int32_t* tile_start, hipStream_t stream) {
    hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, stream, expert_offsets, E, n_rows,
                       ffn_tile_rows(), ffn_max_tiles(n_rows, E), tiles, tile_start);
    return hipGetLastError();
}

hipError_t launch_gate_up(const uint16_t* x_perm, const int4* tiles, const int32_t* tile_start, int64_t n_rows,
                          int d, int E, int h, const uint16_t* w_gate, const uint16_t* w_up, uint16_t* h_act,
                          hipStream_t stream) {
    const int n_tiles = (h + 16 * kGemmWaves - 1) / (16 * kGemmWaves);
    const int64_t grid = static_cast<int64_t>(kXcds) * xcd_slots(ffn_max_tiles(n_rows, E)) * n_tiles;
    hipLaunchKernelGGL(grouped_ffn_kernel<true>, dim3(static_cast<unsigned>(grid)), dim3(kGemmThreads),
                       0, stream, x_perm, tiles, tile_start, E, n_tiles, w_gate, w_up, h, d, h_act);
    return hipGetLastError();
}

hipError_t launch_down(const uint16_t* h_act, const int4* tiles, const int32_t* tile_start, int64_t n_rows, int d,
                       int E, int h, const uint16_t* w_down, float* y_rows, hipStream_t stream) {
    const int n_tiles = (d + 32 * kGemmWaves - 1) / (32 * kGemmWaves);
    const int64_t grid = static_cast<int64_t>(kXcds) * xcd_slots(ffn_max_tiles(n_rows, E)) * n_tiles;
    hipLaunchKernelGGL(grouped_ffn_kernel<false>, dim3(static_cast<unsigned>(grid)), dim3(kGemmThreads),
                       0, stream, h_act, tiles, tile_start, E, n_tiles, w_down, nullptr, d, h, y_rows);
    return hipGetLastError();
}

}  // namespace moe
