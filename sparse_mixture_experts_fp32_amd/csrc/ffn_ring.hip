// Grouped GEMM over experts on bf16 MFMA with float32 accumulation, an LDS ring
// fed by direct-to-LDS loads: the expert SwiGLU FFN of "Kimi K3: Open Frontier
// Intelligence", section "Operational Execution Flow" (SwiGLU-form experts
// applied to the rows routed to them). Expert weights are in the packed layout
// below (moe_pack_weights converts a row-major [N, K] matrix once).
//
//   gate/up pass: H[r, n] = silu(sum_i A[r, i] Wg[e, n, i]) * (sum_i A[r, i] Wu[e, n, i])
//   down pass:    Y[r, n] = sum_i H[r, i] Wd[e, n, i]
// for every row r of expert e. H is rounded once to bf16 (the down pass's MFMA
// operand); Y stays float32. Each output is a sum over K in steps of 32, one
// 16x16x32 MFMA per step and output block, in ascending K.
//
// Work unit: one m-tile of up to 192 rows of one expert (tiles.hip) x one
// n-tile of 512 weight rows. Scheduling for the 8 XCDs (each with its own L2):
// workgroup ids are dealt to the XCDs round-robin, so XCD x runs ids x, x + 8,
// ... in order. The m-tile list is cut into 8 contiguous chunks, one per XCD,
// and inside a chunk the work is ordered expert by expert, n-tile by n-tile,
// with the expert's m-tiles innermost: the m-tiles that share one weight n-tile
// run side by side on one XCD and fetch those weights from HBM once, and all
// n-tiles of an expert follow each other, so its A rows stay in that L2.
//
// Where the operands wait:
//
//  * Every operand byte goes from HBM/L2 straight into LDS with
//    global_load_lds_dwordx4 (64 lanes x 16 B = 1 KiB per instruction, no
//    registers involved). A ring of three stages, each one K step of 32 (the A
//    rows of the m-tile and the weight rows of all waves), keeps two stages in
//    flight while the third is multiplied. The register file then only holds the
//    accumulators, so a wave can own 64 weight rows (4 blocks of 16) instead of
//    32: each A fragment read from LDS feeds 4 MFMAs instead of 2, and a
//    workgroup covers 512 weight rows, halving how often the A tile is re-read
//    per weight byte.
//  * Both operands sit in LDS in MFMA fragment order: 1 KiB per 16 rows x 32 K,
//    lane l's 16 bytes (row l % 16, K 8 (l / 16) .. + 7) at byte 16 l. The DMA
//    writes exactly that order (lane l of a load writes byte 16 l), the
//    fragment reads are 16-byte lane-linear reads (no bank conflicts), and with
//    packed weights each weight load is one contiguous kilobyte of HBM.
//  * One barrier per K step: wait for this wave's loads of step i (vmcnt),
//    barrier (now every wave's step-i A rows are in LDS, and every wave is done
//    with step i - 1), issue the A rows of step i + 2 into the slot step i - 1
//    used, multiply step i. A wave's weight region of a slot is its own, so it
//    issues its weight loads of step i + 3 as soon as it has finished reading
//    step i, without waiting for the other waves. The waits are exact counts
//    of the loads issued after the ones step i needs (vector-memory counters
//    retire in issue order) and are written out: the compiler does not track
//    LDS writes of these loads precisely and would otherwise drain every load
//    at every barrier.
//
// Packed weight layout (moe_pack_weights): matrix [N, K] as tiles of 16 rows x
// 32 columns, 512 elements each, in (row block, column block) order; inside a
// tile element (r, c) sits at ((r + 16 (c / 8)) * 8 + c % 8).
#include "device_common.h"
#include "launch.h"
#include "lds_dma.h"

namespace moe {

constexpr int kXcdsR = 8;
constexpr int kRWaves = 8;                           // waves per workgroup
constexpr int kRThreads = 64 * kRWaves;
constexpr int kRNB = 4;                              // 16-row weight blocks per wave
constexpr int kRKS = 32;                             // K per stage
constexpr int kRStages = 3;
constexpr int kRMaxMB = 12;                          // 16-row A blocks per m-tile (192 rows)
constexpr int kRAStage = kRMaxMB * 1024;             // bytes of A rows per stage
constexpr int kRWStage = kRWaves * kRNB * 1024;      // bytes of weight rows per stage
constexpr int kRStage = kRAStage + kRWStage;         // 44 KiB
constexpr int kRFragAhead = 4;                       // A fragments read ahead of their MFMAs

// Wait until at most n (wave-uniform, 0..12) of this wave's vector-memory
// operations are in flight and its LDS operations are done, then barrier.
__device__ __forceinline__ void ring_wait_barrier(int n) {
    switch (n) {
        case 0: wait_barrier<0>(); break;
        case 1: wait_barrier<1>(); break;
        case 2: wait_barrier<2>(); break;
        case 3: wait_barrier<3>(); break;
        case 4: wait_barrier<4>(); break;
        case 5: wait_barrier<5>(); break;
        case 6: wait_barrier<6>(); break;
        case 7: wait_barrier<7>(); break;
        case 8: wait_barrier<8>(); break;
        case 9: wait_barrier<9>(); break;
        case 10: wait_barrier<10>(); break;
        case 11: wait_barrier<11>(); break;
        default: wait_barrier<12>(); break;
    }
}

// Keep each step's matrix instructions inside the step: an empty volatile asm
// that reads and rewrites every accumulator (it emits no instruction).
template <int kMB>
__device__ __forceinline__ void ring_pin(f32x4 (&acc)[kRNB][kMB]) {
#pragma unroll
    for (int j = 0; j < kRNB; ++j)
#pragma unroll
        for (int i = 0; i < kMB; ++i) asm volatile("" : "+v"(acc[j][i]));
}

// acc[j][i] += A block i (from LDS) x weight block j (from LDS), one K step.
template <int kMB>
__device__ __forceinline__ void ring_mfma(f32x4 (&acc)[kRNB][kMB], const uint8_t* a_lds, const uint8_t* w_lds) {
    constexpr int kAhead = kMB < kRFragAhead ? kMB : kRFragAhead;
    bf16x8 b[kRNB];
#pragma unroll
    for (int j = 0; j < kRNB; ++j) b[j] = *reinterpret_cast<const bf16x8*>(w_lds + 1024 * j);
    bf16x8 a[kAhead + 1];
#pragma unroll
    for (int f = 0; f < kAhead; ++f) a[f] = *reinterpret_cast<const bf16x8*>(a_lds + 1024 * f);
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
        const int g = i + kAhead;
        if (g < kMB) a[g % (kAhead + 1)] = *reinterpret_cast<const bf16x8*>(a_lds + 1024 * g);
#pragma unroll
        for (int j = 0; j < kRNB; ++j) acc[j][i] = mfma_16x16x32(a[i % (kAhead + 1)], b[j], acc[j][i]);
    }
    // keep the reads ahead of their MFMAs: (4 + kAhead) LDS reads, then {4 MFMAs, 1 LDS read}
    __builtin_amdgcn_sched_group_barrier(0x100, kRNB + kAhead, 0);
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, kRNB, 0);
        if (i + kAhead < kMB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
}

// One (m-tile, n-tile) work item with kMB blocks of 16 rows (M <= 16 kMB).
template <bool kGated, bool kBf16, int kMB>
__device__ __forceinline__ void ring_tile(uint8_t* ring, const uint16_t* __restrict__ A,
                                          const int32_t* __restrict__ A_rows, int64_t A_nrows, int64_t row0, int M,
                                          const uint16_t* const (&wblk)[kRNB], bool wave_on, int N, int K,
                                          int n_out, void* __restrict__ Cout) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches below
    const int frag_row = lane & 15, frag_k = 8 * (lane >> 4);
    const uint32_t ring_lds = lds_addr(ring);

    // A blocks this wave loads: wave and wave + 8 (when below kMB); lane l reads
    // row 16 blk + l % 16 (clamped to the tile, gathered through A_rows), K 8 (l / 16) ...
    const int nA = (wave < kMB ? 1 : 0) + (wave + kRWaves < kMB ? 1 : 0);
    const uint16_t* a_src[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int blk = min(wave + kRWaves * p, kMB - 1);
        const int64_t r = row0 + min(16 * blk + frag_row, M - 1);
        const int64_t src = A_rows ? min(max(static_cast<int64_t>(A_rows[r]), int64_t(0)), A_nrows - 1) : r;
        a_src[p] = A + src * K + frag_k;
    }
    // weight loads: the stage's 1 KiB of block j is contiguous (lane l at 16 l)
    const uint32_t w_lane = 16u * lane;
    constexpr uint32_t kWStep = 1024u;  // bytes per K step

    auto issue_a = [&](int s) {  // A rows of K step s into ring slot s % 3
        const uint32_t slot = ring_lds + static_cast<uint32_t>((s % kRStages) * kRStage);
#pragma unroll
        for (int p = 0; p < 2; ++p)
            if (p < nA) dma_vaddr(slot + 1024u * (wave + kRWaves * p), a_src[p] + kRKS * s);
    };
    auto issue_w = [&](int s) {  // this wave's weight rows of K step s
        const uint32_t wslot = ring_lds + static_cast<uint32_t>((s % kRStages) * kRStage) + kRAStage +
                               1024u * kRNB * wave;
        const uint32_t voff = w_lane + kWStep * s;
#pragma unroll
        for (int j = 0; j < kRNB; ++j) dma_saddr(wslot + 1024u * j, wblk[j], voff);
    };

    f32x4 acc[kRNB][kMB];
#pragma unroll
    for (int j = 0; j < kRNB; ++j)
#pragma unroll
        for (int i = 0; i < kMB; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / kRKS;
    // One K loop per wave role (the branch stays outside the loop, so the
    // accumulators never pass through a merge point inside it).
    if (!wave_on) {  // loads A rows for the others (nA per step), multiplies nothing
        issue_a(0);
        if (nk > 1) issue_a(1);
        for (int s = 0; s < nk; ++s) {
            wait_loads_barrier(s + 1 < nk ? nA : 0);
            if (s + 2 < nk) issue_a(s + 2);
        }
        return;
    }
    // Issue order W(0) A(0) W(1) A(1) W(2), then per step s: A(s + 2) after the
    // barrier, W(s + 3) after the multiply; so the loads issued after A(s) are
    // W(s + 1), A(s + 1) and W(s + 2), and waiting until only those are in flight
    // completes step s (W(s) went out before A(s)).
    issue_w(0);
    issue_a(0);
    if (nk > 1) {
        issue_w(1);
        issue_a(1);
    }
    if (nk > 2) issue_w(2);
    const uint8_t* a_lds = ring + 16 * lane;
    const uint8_t* w_lds = ring + kRAStage + 1024 * kRNB * wave + 16 * lane;
    for (int s = 0; s < nk; ++s) {
        ring_wait_barrier((s + 1 < nk ? kRNB + nA : 0) + (s + 2 < nk ? kRNB : 0));
        if (s + 2 < nk) issue_a(s + 2);
        const int off = (s % kRStages) * kRStage;
        ring_mfma<kMB>(acc, a_lds + off, w_lds + off);
        ring_pin(acc);
        if (s + 3 < nk) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave is done reading slot s % 3
            issue_w(s + 3);
        }
    }
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = 16 * i + 4 * (lane >> 4) + q;
            if (r >= M) continue;
            if (kGated) {  // H row: bf16; blocks 0, 1 gate, blocks 2, 3 the same rows of up
                uint16_t* crow = static_cast<uint16_t*>(Cout) + (row0 + r) * N + n_out + frag_row;
#pragma unroll
                for (int c = 0; c < kRNB / 2; ++c) {
                    const float g = acc[c][i][q], u = acc[kRNB / 2 + c][i][q];
                    crow[16 * c] = f32_to_bf16_bits(g / (1.0f + __expf(-g)) * u);
                }
            } else if (kBf16) {  // plain product rounded to bf16 (an operand of a later pass)
                uint16_t* crow = static_cast<uint16_t*>(Cout) + (row0 + r) * N + n_out + frag_row;
#pragma unroll
                for (int j = 0; j < kRNB; ++j) crow[16 * j] = f32_to_bf16_bits(acc[j][i][q]);
            } else {  // Y row: float32, written once and read back only by the combine: non-temporal
                float* crow = static_cast<float*>(Cout) + (row0 + r) * N + n_out + frag_row;
#pragma unroll
                for (int j = 0; j < kRNB; ++j) __builtin_nontemporal_store(acc[j][i][q], crow + 16 * j);
            }
        }
    }
}

// One workgroup per CU (132 KiB of LDS), so the register allocator may give each
// of the two waves per SIMD half the register file.
template <bool kGated, bool kBf16>
__global__ __launch_bounds__(kRThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
void ffn_ring_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ A_rows, int64_t A_nrows,
                     const int4* __restrict__ tiles, const int32_t* __restrict__ tile_start, int E, int n_tiles,
                     const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1, int N, int K,
                     void* __restrict__ Cout) {
    constexpr int kColsW = kGated ? 16 * kRNB / 2 : 16 * kRNB;  // output columns per wave
    constexpr int kColsWG = kColsW * kRWaves;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kRStages * kRStage];

    // ---- work item: (m-tile, n-tile) from the XCD-ordered schedule
    const int n_mt = tile_start[E];
    const int xcd = blockIdx.x % kXcdsR;
    const int j = blockIdx.x / kXcdsR;
    const int lo = static_cast<int>(static_cast<int64_t>(xcd) * n_mt / kXcdsR);
    const int hi = static_cast<int>(static_cast<int64_t>(xcd + 1) * n_mt / kXcdsR);
    const int slot = j / n_tiles;
    if (lo + slot >= hi) return;  // uniform for the workgroup, before any barrier
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

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_out = nt * kColsWG + wave * kColsW;
    const bool wave_on = n_out < N;  // uniform per wave; N is a multiple of kColsW

    // first weight row of each of this wave's blocks (gate/up: 2 gate blocks, then the same rows of up)
    const uint16_t* wblk[kRNB];
    const int64_t wexp = static_cast<int64_t>(e) * N * K;
#pragma unroll
    for (int b = 0; b < kRNB; ++b) {
        const int row = wave_on ? (kGated ? n_out + 16 * (b % (kRNB / 2)) : n_out + 16 * b) : 0;
        const uint16_t* base = (kGated && b >= kRNB / 2) ? W1 : W0;
        // the tiles of rows row .. row + 15 start at (row / 16) * (K / 32) tiles of 512 elements
        const int64_t off = static_cast<int64_t>(row / 16) * (K / kRKS) * 512;
        wblk[b] = static_cast<const uint16_t*>(uniform_ptr(base + wexp + off));
    }

    const int mb = min(kRMaxMB, (M + 15) / 16);
#define MOE_RING_TILE(NB)                                                                                  \
    if (mb == (NB)) {                                                                                      \
        ring_tile<kGated, kBf16, (NB)>(ring, A, A_rows, A_nrows, row0, M, wblk, wave_on, N, K, n_out, Cout);        \
        return;                                                                                            \
    }
    MOE_RING_TILE(1)
    MOE_RING_TILE(2)
    MOE_RING_TILE(3)
    MOE_RING_TILE(4)
    MOE_RING_TILE(5)
    MOE_RING_TILE(6)
    MOE_RING_TILE(7)
    MOE_RING_TILE(8)
    MOE_RING_TILE(9)
    MOE_RING_TILE(10)
    MOE_RING_TILE(11)
    MOE_RING_TILE(12)
#undef MOE_RING_TILE
}

template <bool kGated, bool kBf16 = false>
static hipError_t launch_ring(const uint16_t* A, const int32_t* A_rows, int64_t A_nrows, const int4* tiles,
                       const int32_t* tile_start, int64_t n_rows, int E, const uint16_t* W0, const uint16_t* W1, int N,
                       int K, void* Cout, hipStream_t stream) {
    static_assert(16 * kRMaxMB == 192, "m-tiles of the shared tile list hold up to 192 rows");
    const int cols_wg = (kGated ? 16 * kRNB / 2 : 16 * kRNB) * kRWaves;
    const int n_tiles = (N + cols_wg - 1) / cols_wg;
    const int slots = (ffn_max_tiles(n_rows, E) + kXcdsR - 1) / kXcdsR;
    const int64_t grid = static_cast<int64_t>(kXcdsR) * slots * n_tiles;
    hipLaunchKernelGGL((ffn_ring_kernel<kGated, kBf16>), dim3(static_cast<unsigned>(grid)), dim3(kRThreads), 0,
                       stream, A, A_rows, A_nrows, tiles, tile_start, E, n_tiles, W0, W1, N, K, Cout);
    return hipGetLastError();
}

hipError_t launch_gate_up(const uint16_t* a, const int32_t* a_rows, int64_t a_nrows, const int4* tiles,
                          const int32_t* tile_start, int64_t n_rows, int d, int E, int h, const uint16_t* w_gate,
                          const uint16_t* w_up, uint16_t* h_act, hipStream_t stream) {
    return launch_ring<true>(a, a_rows, a_nrows, tiles, tile_start, n_rows, E, w_gate, w_up, h, d, h_act, stream);
}

hipError_t launch_down(const uint16_t* h_act, const int4* tiles, const int32_t* tile_start, int64_t n_rows, int d,
                       int E, int h, const uint16_t* w_down, float* y_rows, hipStream_t stream) {
    return launch_ring<false>(h_act, nullptr, n_rows, tiles, tile_start, n_rows, E, w_down, nullptr, d, h, y_rows,
                              stream);
}

hipError_t launch_dense(const uint16_t* a, const int32_t* a_rows, int64_t a_nrows, const int4* tiles,
                        const int32_t* tile_start, int64_t n_rows, int E, const uint16_t* w, int N, int K, void* c,
                        bool bf16_out, hipStream_t stream) {
    if (bf16_out)
        return launch_ring<false, true>(a, a_rows, a_nrows, tiles, tile_start, n_rows, E, w, nullptr, N, K, c, stream);
    return launch_ring<false, false>(a, a_rows, a_nrows, tiles, tile_start, n_rows, E, w, nullptr, N, K, c, stream);
}

// Row-major [rows, K] bf16 -> packed tiles (see the layout above). One thread per
// 8 elements (16 bytes).
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t* __restrict__ w, int64_t rows, int K,
                                                           uint16_t* __restrict__ out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;  // 8-element chunk
    const int64_t per_row = K / 8;
    if (i >= rows * per_row) return;
    const int64_t n = i / per_row;
    const int k = static_cast<int>(i % per_row) * 8;
    const int64_t dst = ((n / 16) * (K / kRKS) + k / kRKS) * 512 + ((n % 16) + 16 * ((k % kRKS) / 8)) * 8;
    *reinterpret_cast<u32x4*>(out + dst) = *reinterpret_cast<const u32x4*>(w + n * K + k);
}

hipError_t launch_pack_weights(const uint16_t* w, int64_t rows, int K, uint16_t* out, hipStream_t stream) {
    const int64_t n = rows * (K / 8);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_weights_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, w,
                       rows, K, out);
    return hipGetLastError();
}

}  // namespace moe
