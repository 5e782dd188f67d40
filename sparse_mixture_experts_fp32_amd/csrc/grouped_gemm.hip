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
// Inside a workgroup: the A rows of the current K step are staged in LDS,
// double-buffered, and shared by all waves; each wave streams its own weight
// rows straight from HBM into registers, one K step ahead of the matrix cores
// (each weight byte is used by exactly one wave, so staging it in LDS would buy
// nothing). Weights are stored [N, K] (K contiguous), so one lane's 8
// consecutive k values are a single 16-byte load that is directly an MFMA
// operand. The K loop is unrolled by two so the two register sets of weights
// swap roles without copies, rows past the tile end are clamped to its last row
// and the prefetch index is clamped to the last K step, so every load is
// unconditional and the wait before each step's MFMAs covers only that step's
// weights, never the loads already issued for the next step. The number of
// 16-row blocks is a compile-time constant per K loop (one loop per block
// count, chosen once per tile), so the MFMA sequence is straight-line code.
//
// Scheduling for the 8 XCDs (each with its own L2): workgroup ids are dealt to
// the XCDs round-robin, so XCD x runs ids x, x + 8, x + 16, ... in order. The
// m-tile list is cut into 8 contiguous chunks, one per XCD, and inside a chunk
// the work is ordered expert by expert, n-tile by n-tile, with the expert's
// m-tiles innermost. The m-tiles that share one weight n-tile therefore run
// side by side on one XCD and fetch those weights from HBM once (the others
// hit in L2), and all n-tiles of an expert follow each other, so its A rows
// stay in that L2 as well.
//
// This kernel serves row-major expert weights and the dense passes of the
// latent layer; packed weights run on the LDS-ring kernel (ffn_ring.hip). Both
// walk the m-tile list that build_tiles_kernel below writes.
#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kXcds = 8;
constexpr int kFragAhead = 4;  // A fragments read ahead of the MFMAs that consume them

// Tile configuration of one grouped-GEMM kernel. The workgroup's waves form a
// kWM x kWN grid: wave (wm, wn) owns the 16-row blocks b with b % kWM == wm and
// kNB blocks of 16 weight rows (gate/up: half gate, half up columns).
template <int kWM_, int kWN_, int kNB_, int kKS_, int kMaxMB_, bool kDeep_, int kPad_ = 8>
struct GemmCfg {
    static constexpr int kWM = kWM_;          // wave rows (split the m-tile's row blocks)
    static constexpr int kWN = kWN_;          // wave columns (split the n-tile)
    static constexpr int kNB = kNB_;          // 16-row weight blocks per wave
    static constexpr int kWaves = kWM * kWN;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int kKS = kKS_;          // K step staged per barrier (multiple of 32)
    static constexpr int kSub = kKS / 32;     // MFMA K sub-steps per K step
    static constexpr int kAStride = kKS + kPad_;  // bf16 per LDS row (padded against bank conflicts)
    static constexpr int kMaxMB = kMaxMB_;    // 16-row blocks per m-tile (multiple of kWM)
    static constexpr int kBM = 16 * kMaxMB;   // rows per m-tile
    static constexpr int kBufElems = kBM * kAStride;
    static constexpr int kWRows = 16 * kNB;   // weight rows per wave
    static constexpr bool kDeep = kDeep_;     // weights 3 K steps ahead, A rows 2 (else 1 and 1)
    static constexpr int kStepMB = kWM < 2 ? 2 : kWM;  // granularity of the per-tile block count
    static_assert(kMaxMB % kWM == 0, "row blocks split evenly over wave rows");
    static_assert(kNB % 2 == 0, "gate/up waves hold matching gate and up blocks");
};

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

// Register-array helpers of the K loop (force-inlined so the arrays stay in registers).
template <int kP>
__device__ __forceinline__ void load_rows(u32x4 (&dst)[kP], const uint16_t* src, const int64_t (&off)[kP], int k0) {
#pragma unroll
    for (int p = 0; p < kP; ++p) dst[p] = *reinterpret_cast<const u32x4*>(src + off[p] + k0);
}

template <int kP, int kStep>
__device__ __forceinline__ void store_rows(uint16_t* dst, const u32x4 (&src)[kP]) {
#pragma unroll
    for (int p = 0; p < kP; ++p) *reinterpret_cast<u32x4*>(dst + p * kStep) = src[p];
}

// dst[b][s]: 16 weight rows of block b, K sub-step s of one K step
template <int kNB, int kSub>
__device__ __forceinline__ void load_weights(bf16x8 (&dst)[kNB][kSub], const uint16_t* const (&w)[kNB], int k0) {
#pragma unroll
    for (int s = 0; s < kSub; ++s)
#pragma unroll
        for (int b = 0; b < kNB; ++b) dst[b][s] = *reinterpret_cast<const bf16x8*>(w[b] + k0 + 32 * s);
}

// acc[b][i] += (A rows of block kWM * i + wm, one K step, from LDS) x (weight block b).
// The A fragments of the step (kSub x kMBW of them) are read from LDS through a
// rolling window kFragAhead deep, so each read has that many MFMA groups to land.
template <int kMBW, int kWM, int kNB, int kSub, int kAStride>
__device__ __forceinline__ void mfma_step(f32x4 (&acc)[kNB][kMBW], const uint16_t* frag,
                                          const bf16x8 (&bw)[kNB][kSub]) {
    constexpr int kF = kSub * kMBW;  // fragments in one K step, f = s * kMBW + i
    constexpr int kAhead = kF < kFragAhead ? kF : kFragAhead;
    bf16x8 a[kAhead + 1];
#pragma unroll
    for (int f = 0; f < kAhead; ++f)
        a[f] = *reinterpret_cast<const bf16x8*>(frag + (f % kMBW) * kWM * 16 * kAStride + 32 * (f / kMBW));
#pragma unroll
    for (int f = 0; f < kF; ++f) {
        const int g = f + kAhead;
        if (g < kF)
            a[g % (kAhead + 1)] =
                *reinterpret_cast<const bf16x8*>(frag + (g % kMBW) * kWM * 16 * kAStride + 32 * (g / kMBW));
        const int i = f % kMBW, s = f / kMBW;
#pragma unroll
        for (int b = 0; b < kNB; ++b) acc[b][i] = mfma_16x16x32(a[f % (kAhead + 1)], bw[b][s], acc[b][i]);
    }
    // Keep that order through instruction scheduling (which would otherwise sink
    // each read next to its use): kAhead LDS reads, then {kNB MFMAs, 1 LDS read}.
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int f = 0; f < kF; ++f) {
        __builtin_amdgcn_sched_group_barrier(0x008, kNB, 0);
        if (f + kAhead < kF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
}

// One (m-tile, n-tile) work item with kMB row blocks of 16 (M <= 16 * kMB rows).
// Every load and LDS store in the K loop is unconditional: rows past M re-read
// row M - 1 and prefetch indices are clamped to the last K step (a repeated
// step is loaded but never used).
template <class C, bool kGated, bool kBf16, int kMB>
__device__ __forceinline__ void ffn_tile(uint16_t* sA, const uint16_t* __restrict__ A,
                                         const int32_t* __restrict__ A_rows, int64_t A_nrows, int64_t row0, int M,
                                         const uint16_t* const (&wb)[C::kNB], bool wave_on, int N, int K, int wm,
                                         int n_wave, void* __restrict__ Cout) {
    constexpr int kNB = C::kNB, kSub = C::kSub, kKS = C::kKS;
    constexpr int kMBW = kMB / C::kWM;   // row blocks of this wave
    constexpr int kChunks = kKS / 8;     // 16-byte chunks per staged row
    constexpr int kRowsPerPass = C::kThreads / kChunks;
    constexpr int kAPasses = (16 * kMB + kRowsPerPass - 1) / kRowsPerPass;
    static_assert(kMB % C::kWM == 0, "row blocks split evenly over wave rows");
    static_assert(kAPasses * kRowsPerPass <= C::kBM, "staged rows must fit the LDS tile");
    const int tid = threadIdx.x, lane = tid & 63;
    const int frag_row = lane & 15, frag_k = 8 * (lane >> 4);

    const int a_row = tid / kChunks, a_col = 8 * (tid % kChunks);
    // row r of the tile is A[row0 + r], or A[A_rows[row0 + r]] when the rows are
    // gathered on the fly (the dispatch fused into this pass)
    const uint16_t* a_src = A + a_col;
    int64_t a_off[kAPasses];
#pragma unroll
    for (int p = 0; p < kAPasses; ++p) {
        const int64_t r = row0 + min(p * kRowsPerPass + a_row, M - 1);
        const int64_t src = A_rows ? min(max(static_cast<int64_t>(A_rows[r]), int64_t(0)), A_nrows - 1) : r;
        a_off[p] = src * K;
    }
    uint16_t* a_dst[2] = {sA + a_row * C::kAStride + a_col, sA + a_row * C::kAStride + a_col + C::kBufElems};
    const uint16_t* a_frag[2] = {sA + (wm * 16 + frag_row) * C::kAStride + frag_k,
                                 sA + (wm * 16 + frag_row) * C::kAStride + frag_k + C::kBufElems};
    constexpr int kPassStride = kRowsPerPass * C::kAStride;

    f32x4 acc[kNB][kMBW];
#pragma unroll
    for (int b = 0; b < kNB; ++b)
#pragma unroll
        for (int i = 0; i < kMBW; ++i) acc[b][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / kKS;
    if constexpr (!C::kDeep) {
        // Weights and A rows one K step ahead: register sets b0 / b1 and LDS
        // buffers 0 / 1 alternate between "being consumed" and "being filled".
        u32x4 a_reg[kAPasses];
        bf16x8 b0[kNB][kSub], b1[kNB][kSub];
        load_rows(a_reg, a_src, a_off, 0);
        load_weights(b0, wb, 0);
        store_rows<kAPasses, kPassStride>(a_dst[0], a_reg);
        __syncthreads();
        for (int s0 = 0; s0 < nk; s0 += 2) {
            const int k1 = min(s0 + 1, nk - 1) * kKS;
            load_rows(a_reg, a_src, a_off, k1);
            load_weights(b1, wb, k1);
            if (wave_on) mfma_step<kMBW, C::kWM, kNB, kSub, C::kAStride>(acc, a_frag[0], b0);
            store_rows<kAPasses, kPassStride>(a_dst[1], a_reg);
            __syncthreads();
            const int k2 = min(s0 + 2, nk - 1) * kKS;
            load_rows(a_reg, a_src, a_off, k2);
            load_weights(b0, wb, k2);
            if (wave_on && s0 + 1 < nk) mfma_step<kMBW, C::kWM, kNB, kSub, C::kAStride>(acc, a_frag[1], b1);
            store_rows<kAPasses, kPassStride>(a_dst[0], a_reg);
            __syncthreads();
        }
    } else {
        // Weights three K steps ahead (a ring of four register sets), A rows two
        // steps ahead (two register sets) and written to LDS one step ahead (two
        // buffers). Step i: load A rows i+2, then weights i+3, multiply step i,
        // store A rows i+1, barrier. Vector-memory counters retire in issue
        // order, so the A rows are issued first: waiting for A rows i+1 at the
        // end of step i then does not wait for weights i+2. Four steps per loop
        // trip, so every ring index is a compile-time constant.
        u32x4 ar[2][kAPasses];
        bf16x8 bw[4][kNB][kSub];
        load_rows(ar[0], a_src, a_off, 0);
        load_rows(ar[1], a_src, a_off, min(1, nk - 1) * kKS);
        load_weights(bw[0], wb, 0);
        load_weights(bw[1], wb, min(1, nk - 1) * kKS);
        load_weights(bw[2], wb, min(2, nk - 1) * kKS);
        store_rows<kAPasses, kPassStride>(a_dst[0], ar[0]);
        __syncthreads();
#define MOE_DEEP_STEP(U)                                                                                  \
    {                                                                                                     \
        const int step = s0 + (U);                                                                        \
        load_rows(ar[(U) % 2], a_src, a_off, min(step + 2, nk - 1) * kKS);                                \
        load_weights(bw[((U) + 3) % 4], wb, min(step + 3, nk - 1) * kKS);                                 \
        if (wave_on && step < nk)                                                                         \
            mfma_step<kMBW, C::kWM, kNB, kSub, C::kAStride>(acc, a_frag[(U) % 2], bw[(U) % 4]);            \
        store_rows<kAPasses, kPassStride>(a_dst[((U) + 1) % 2], ar[((U) + 1) % 2]);                       \
        __syncthreads();                                                                                  \
    }
        for (int s0 = 0; s0 < nk; s0 += 4) {
            MOE_DEEP_STEP(0)
            MOE_DEEP_STEP(1)
            MOE_DEEP_STEP(2)
            MOE_DEEP_STEP(3)
        }
#undef MOE_DEEP_STEP
    }

    if (!wave_on) return;
#pragma unroll
    for (int i = 0; i < kMBW; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = (i * C::kWM + wm) * 16 + 4 * (lane >> 4) + q;
            if (r >= M) continue;
            if (kGated) {  // H row: bf16, the operand of the down pass; first half gate blocks, second up
                uint16_t* crow = static_cast<uint16_t*>(Cout) + (row0 + r) * N + n_wave + frag_row;
#pragma unroll
                for (int c = 0; c < kNB / 2; ++c) {
                    const float g = acc[c][i][q], u = acc[kNB / 2 + c][i][q];
                    crow[16 * c] = f32_to_bf16_bits(g / (1.0f + __expf(-g)) * u);
                }
            } else if (kBf16) {  // plain product rounded to bf16 (an operand of a later pass)
                uint16_t* crow = static_cast<uint16_t*>(Cout) + (row0 + r) * N + n_wave + frag_row;
#pragma unroll
                for (int b = 0; b < kNB; ++b) crow[16 * b] = f32_to_bf16_bits(acc[b][i][q]);
            } else {             // Y row: float32, read back only by a later pass over many other bytes
                float* crow = static_cast<float*>(Cout) + (row0 + r) * N + n_wave + frag_row;
#pragma unroll
                for (int b = 0; b < kNB; ++b) __builtin_nontemporal_store(acc[b][i][q], crow + 16 * b);
            }
        }
    }
}

// One workgroup per CU is the design point (LDS tile and register budget), so the
// register allocator is told that occupancy is fixed and may spend registers on
// keeping loads in flight rather than on reaching a higher wave count.
template <class C, bool kGated, bool kBf16>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(1, C::kWaves / 4)))
void grouped_ffn_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ A_rows, int64_t A_nrows,
    const int4* __restrict__ tiles, const int32_t* __restrict__ tile_start, int E, int n_tiles,
    const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1, int N, int K, void* __restrict__ Cout) {
    constexpr int kColsW = kGated ? C::kWRows / 2 : C::kWRows;  // output columns per wave
    constexpr int kColsWG = kColsW * C::kWN;
    __shared__ __attribute__((aligned(16))) uint16_t sA[2 * C::kBufElems];

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
    const int wm = wave % C::kWM, wn = wave / C::kWM;
    const int n_wave = nt * kColsWG + wn * kColsW;
    const bool wave_on = n_wave < N;  // uniform per wave
    const int frag_row = lane & 15, frag_k = 8 * (lane >> 4);

    // weight rows of this lane for the four B blocks (an idle wave reads valid rows it never uses)
    const int n_safe = wave_on ? n_wave : 0;
    const int64_t wexp = static_cast<int64_t>(e) * N * K;
    const int64_t lane_off = static_cast<int64_t>(n_safe + frag_row) * K + frag_k;
    const uint16_t* w0 = W0 + wexp + lane_off;
    const uint16_t* w1 = kGated ? W1 + wexp + lane_off : w0;
    const int64_t blk = 16 * static_cast<int64_t>(K);
    // gate/up: blocks 0 .. kNB/2-1 are gate rows, the rest the same rows of up
    const uint16_t* wb[C::kNB];
#pragma unroll
    for (int b = 0; b < C::kNB; ++b)
        wb[b] = kGated ? (b < C::kNB / 2 ? w0 + b * blk : w1 + (b - C::kNB / 2) * blk) : w0 + b * blk;

    // one straight-line K loop per row-block count, chosen once per tile
    constexpr int kStepMB = C::kStepMB;
    const int mb = min(C::kMaxMB, ((M + 16 * kStepMB - 1) / (16 * kStepMB)) * kStepMB);
#define MOE_TILE(NB)                                                                                   \
    if (mb == (NB)) {                                                                                  \
        ffn_tile<C, kGated, kBf16, ((NB) < C::kMaxMB ? (NB) : C::kMaxMB)>(sA, A, A_rows, A_nrows, row0, M,          \
                                                                          wb, wave_on, N, K, wm, n_wave, Cout); \
        return;                                                                                        \
    }
    MOE_TILE(kStepMB)
    MOE_TILE(2 * kStepMB)
    MOE_TILE(3 * kStepMB)
    MOE_TILE(4 * kStepMB)
    MOE_TILE(5 * kStepMB)
    MOE_TILE(6 * kStepMB)
    MOE_TILE(7 * kStepMB)
    MOE_TILE(8 * kStepMB)
#undef MOE_TILE
}

// ---------------------------------------------------------------- launchers

static int max_tiles_for(int64_t n_rows, int E, int bm) {
    int64_t t = (n_rows + bm - 1) / bm + E;
    if (t > n_rows) t = n_rows;
    if (t < 1) t = 1;
    return static_cast<int>(t);
}

template <class C, bool kGated, bool kBf16 = false>
hipError_t launch_ffn(const uint16_t* A, const int32_t* A_rows, int64_t A_nrows, const int4* tiles,
                      const int32_t* tile_start, int64_t n_rows, int E, const uint16_t* W0, const uint16_t* W1, int N,
                      int K, void* Cout, hipStream_t stream) {
    static_assert(C::kMaxMB <= 8 * C::kStepMB && C::kMaxMB % C::kStepMB == 0,
                  "the block-count dispatch covers up to 8 steps");
    const int cols_wg = (kGated ? C::kWRows / 2 : C::kWRows) * C::kWN;
    const int n_tiles = (N + cols_wg - 1) / cols_wg;
    // sized for any tile list (tiles of at least kMinTileRows rows); surplus workgroups exit
    const int slots = (ffn_max_tiles(n_rows, E) + kXcds - 1) / kXcds;
    const int64_t grid = static_cast<int64_t>(kXcds) * slots * n_tiles;
    hipLaunchKernelGGL((grouped_ffn_kernel<C, kGated, kBf16>), dim3(static_cast<unsigned>(grid)), dim3(C::kThreads), 0, stream, A, A_rows, A_nrows, tiles, tile_start, E, n_tiles, W0, W1, N, K, Cout);
    return hipGetLastError();
}

// 8 waves x 32 weight rows, K step 64, m-tiles of up to 192 rows, LDS rows padded
// by 32 B (chosen by measurement on the prefill, decode, many-expert and skewed
// loads: padding by 16 B showed bank conflicts on gfx950, 2-D wave grids and
// 4-wave workgroups were slower). The gate/up pass (K = d) keeps weights three
// steps ahead; the down pass (K = h, a quarter as deep) measured best one ahead.
using GateUpCfg = GemmCfg<1, 8, 2, 64, 12, true, 16>;
using DownCfg = GemmCfg<1, 8, 2, 64, 12, false, 16>;
// plain products with a deep K (the latent projections: K = d or l)
using DenseCfg = GemmCfg<1, 8, 2, 64, 12, true, 16>;
static_assert(GateUpCfg::kBM == DownCfg::kBM && DenseCfg::kBM == DownCfg::kBM, "all passes share one m-tile size");

int ffn_tile_rows() { return GateUpCfg::kBM; }

// Capacity of a tile list: enough for the shortest m-tiles any pass uses (the MX
// passes' 128 rows), so one workspace serves every pass.
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

hipError_t launch_gate_up(const uint16_t* a, const int32_t* a_rows, int64_t a_nrows, const int4* tiles,
                          const int32_t* tile_start, int64_t n_rows, int d, int E, int h, const uint16_t* w_gate,
                          const uint16_t* w_up, uint16_t* h_act, hipStream_t stream, bool packed) {
    if (packed)
        return launch_gate_up_ring(a, a_rows, a_nrows, tiles, tile_start, n_rows, d, E, h, w_gate, w_up, h_act, stream);
    return launch_ffn<GateUpCfg, true>(a, a_rows, a_nrows, tiles, tile_start, n_rows, E, w_gate, w_up, h, d, h_act,
                                       stream);
}

hipError_t launch_down(const uint16_t* h_act, const int4* tiles, const int32_t* tile_start, int64_t n_rows, int d,
                       int E, int h, const uint16_t* w_down, float* y_rows, hipStream_t stream, bool packed) {
    if (packed) return launch_down_ring(h_act, tiles, tile_start, n_rows, d, E, h, w_down, y_rows, stream);
    return launch_ffn<DownCfg, false>(h_act, nullptr, n_rows, tiles, tile_start, n_rows, E, w_down, nullptr, d, h,
                                      y_rows, stream);
}

hipError_t launch_dense(const uint16_t* a, const int32_t* a_rows, int64_t a_nrows, const int4* tiles,
                        const int32_t* tile_start, int64_t n_rows, int E, const uint16_t* w, int N, int K, void* c,
                        bool bf16_out, hipStream_t stream) {
    if (bf16_out)
        return launch_ffn<DenseCfg, false, true>(a, a_rows, a_nrows, tiles, tile_start, n_rows, E, w, nullptr, N, K,
                                                 c, stream);
    return launch_ffn<DenseCfg, false, false>(a, a_rows, a_nrows, tiles, tile_start, n_rows, E, w, nullptr, N, K, c,
                                              stream);
}

}  // namespace moe
