// Grouped GEMM over experts on bf16 MFMA (float32 accumulation): the expert
// SwiGLU FFN of "Kimi K3: Open Frontier Intelligence", section "Operational
// Execution Flow" (SwiGLU-form experts applied to the rows routed to them).
//
//   gate/up pass: H[r, n] = silu(sum_i A[r, i] Wg[e, n, i]) * (sum_i A[r, i] Wu[e, n, i])
//   down pass:    Y[r, n] = sum_i H[r, i] Wd[e, n, i]
// H is rounded once to bf16 (the down pass's MFMA operand); Y stays float32.
// for every row r of expert e (rows grouped by expert, contiguous).
//
// Work unit: one m-tile (up to BM consecutive rows of one expert) x one
// n-tile of output columns. The list of m-tiles is built on the device from
// expert_offsets, and the grid is sized from an upper bound, so no token count
// ever goes back to the host; surplus workgroups find an empty tile and exit.
//
// Inside a workgroup (8 wavefronts): the A rows of the current K step (128
// deep) are staged in LDS, double-buffered, and shared by all waves; each wave
// streams its own weight rows straight from HBM into registers (each weight
// byte is used by exactly one wave, so staging it in LDS would buy nothing),
// one K step ahead of the matrix cores. Weights are stored [N, K] (K
// contiguous), so one lane's 8 consecutive k values are a single 16-byte load
// that is directly an MFMA operand.
//
// Workgroup ids are dealt round-robin to the 8 XCDs; the id -> tile map gives
// all n-tiles of one m-tile to the same XCD, back to back, so that m-tile's A
// rows are fetched into that XCD's L2 once and reused by every n-tile.
#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kGemmWaves = 8;
constexpr int kGemmThreads = kGemmWaves * 64;
constexpr int kKStep = 128;
constexpr int kAStride = kKStep + 8;  // bf16 per LDS row: 272 B keeps 16-B reads conflict-free

// tiles[i] = {expert, first row, rows, 0}; entries past the real count have rows = 0.
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                           int64_t n_rows, int bm, int max_tiles,
                                                           int4* __restrict__ tiles) {
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
    for (int i = 0; i < nt; ++i)
        if (start + i < max_tiles) tiles[start + i] = make_int4(tid, lo + i * bm, min(bm, cnt - i * bm), 0);
    for (int i = part[1023] + tid; i < max_tiles; i += 1024) tiles[i] = make_int4(0, 0, 0, 0);
}

template <bool kGated, int kMSub>
__global__ __launch_bounds__(kGemmThreads) void grouped_ffn_kernel(
    const uint16_t* __restrict__ A, int64_t n_rows, const int4* __restrict__ tiles, int n_tiles,
    const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1, int N, int K,
    void* __restrict__ Cout) {
    constexpr int kBM = 16 * kMSub;
    constexpr int kColsW = kGated ? 16 : 32;  // output columns per wave
    constexpr int kColsWG = kColsW * kGemmWaves;
    constexpr int kAPasses = kBM / 32;        // 16 threads x 16 B per row, 32 rows per pass
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBM * kAStride];

    const int bid = blockIdx.x;
    const int xcd = bid & 7, j = bid >> 3;
    const int mt = 8 * (j / n_tiles) + xcd;
    const int nt = j % n_tiles;
    const int4 tile = tiles[mt];
    const int M = tile.z;
    if (M <= 0) return;  // uniform for the whole workgroup, before any barrier
    const int e = tile.x;
    const int64_t row0 = tile.y;
    const int nsub = (M + 15) >> 4;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_wave = nt * kColsWG + wave * kColsW;
    const bool wave_on = n_wave < N;
    const int frag_row = lane & 15, frag_k = 8 * (lane >> 4);

    // weight rows of this lane for the two B blocks
    const int64_t wexp = static_cast<int64_t>(e) * N * K;
    const uint16_t* wb[2];
    if (kGated) {
        wb[0] = W0 + wexp + static_cast<int64_t>(n_wave + frag_row) * K + frag_k;
        wb[1] = W1 + wexp + static_cast<int64_t>(n_wave + frag_row) * K + frag_k;
    } else {
        wb[0] = W0 + wexp + static_cast<int64_t>(n_wave + frag_row) * K + frag_k;
        wb[1] = W0 + wexp + static_cast<int64_t>(n_wave + 16 + frag_row) * K + frag_k;
    }

    // A staging: thread owns row (pass * 32 + tid / 16), 8 bf16 at column 8 * (tid % 16)
    const int a_row = tid >> 4, a_col = 8 * (tid & 15);
    uint4 a_reg[kAPasses];
    auto load_A = [&](int k0) {
#pragma unroll
        for (int p = 0; p < kAPasses; ++p) {
            const int r = p * 32 + a_row;
            a_reg[p] = (r < M) ? *reinterpret_cast<const uint4*>(A + (row0 + r) * K + k0 + a_col)
                               : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_A = [&](int buf) {
#pragma unroll
        for (int p = 0; p < kAPasses; ++p)
            *reinterpret_cast<uint4*>(&sA[buf][(p * 32 + a_row) * kAStride + a_col]) = a_reg[p];
    };
    bf16x8 bcur[2][4], bnext[2][4];
    auto load_B = [&](int k0, bf16x8 (&dst)[2][4]) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int s = 0; s < 4; ++s) dst[b][s] = *reinterpret_cast<const bf16x8*>(wb[b] + k0 + 32 * s);
    };

    f32x4 acc[2][kMSub];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int m = 0; m < kMSub; ++m) acc[b][m] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / kKStep;
    load_A(0);
    if (wave_on) load_B(0, bcur);
    store_A(0);
    __syncthreads();
    for (int step = 0; step < nk; ++step) {
        const int cur = step & 1;
        const bool more = step + 1 < nk;
        if (more) {
            load_A((step + 1) * kKStep);
            if (wave_on) load_B((step + 1) * kKStep, bnext);
        }
        if (wave_on) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int m = 0; m < kMSub; ++m) {
                    if (m < nsub) {
                        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                            &sA[cur][(m * 16 + frag_row) * kAStride + 32 * s + frag_k]);
                        acc[0][m] = mfma_16x16x32(a, bcur[0][s], acc[0][m]);
                        acc[1][m] = mfma_16x16x32(a, bcur[1][s], acc[1][m]);
                    }
                }
            }
        }
        if (more) store_A(cur ^ 1);
        __syncthreads();
        if (more && wave_on) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int s = 0; s < 4; ++s) bcur[b][s] = bnext[b][s];
        }
    }

    if (!wave_on) return;
    const int col = n_wave + frag_row;
#pragma unroll
    for (int m = 0; m < kMSub; ++m) {
        if (m >= nsub) continue;
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

// ---------------------------------------------------------------- launchers

constexpr int kFfnMSub = 8;  // m-tile of 128 rows

int ffn_tile_rows() { return 16 * kFfnMSub; }

int ffn_max_tiles(int64_t n_rows, int E) {
    const int64_t bm = ffn_tile_rows();
    int64_t t = (n_rows + bm - 1) / bm + E;
    if (t > n_rows) t = n_rows;
    if (t < 1) t = 1;
    return static_cast<int>((t + 7) / 8 * 8);  // multiple of 8 for the XCD map
}

hipError_t launch_build_tiles(const int32_t* expert_offsets, int64_t n_rows, int E, int4* tiles,
                              hipStream_t stream) {
    hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, stream, expert_offsets, E, n_rows,
                       ffn_tile_rows(), ffn_max_tiles(n_rows, E), tiles);
    return hipGetLastError();
}

hipError_t launch_gate_up(const uint16_t* x_perm, const int4* tiles, int64_t n_rows, int d, int E, int h,
                          const uint16_t* w_gate, const uint16_t* w_up, uint16_t* h_act, hipStream_t stream) {
    const int max_tiles = ffn_max_tiles(n_rows, E);
    const int n_tiles = (h + 16 * kGemmWaves - 1) / (16 * kGemmWaves);
    hipLaunchKernelGGL((grouped_ffn_kernel<true, kFfnMSub>), dim3(max_tiles * n_tiles), dim3(kGemmThreads), 0,
                       stream, x_perm, n_rows, tiles, n_tiles, w_gate, w_up, h, d, h_act);
    return hipGetLastError();
}

hipError_t launch_down(const uint16_t* h_act, const int4* tiles, int64_t n_rows, int d, int E, int h,
                       const uint16_t* w_down, float* y_rows, hipStream_t stream) {
    const int max_tiles = ffn_max_tiles(n_rows, E);
    const int n_tiles = (d + 32 * kGemmWaves - 1) / (32 * kGemmWaves);
    hipLaunchKernelGGL((grouped_ffn_kernel<false, kFfnMSub>), dim3(max_tiles * n_tiles), dim3(kGemmThreads), 0,
                       stream, h_act, n_rows, tiles, n_tiles, w_down, nullptr, d, h, y_rows);
    return hipGetLastError();
}

}  // namespace moe
