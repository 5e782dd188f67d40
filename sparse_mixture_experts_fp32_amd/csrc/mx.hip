// MX-format expert FFN: MXFP4 (E2M1) expert weights and MXFP8 (E4M3) activations
// ("Kimi K3: Open Frontier Intelligence", section "Systems Optimization, Load
// Balancing, and Post-Training Alignment": the serving variant of the MoE
// weights and activations). The formats are the OCP Microscaling ones: blocks of
// 32 elements along K share an E8M0 scale 2^s, s = floor(log2 amax) - emax
// (emax 2 for E2M1, 8 for E4M3); each element is v / 2^s rounded to the nearest
// element value, ties to the even code, clamped to the largest one.
//
// The grouped GEMM runs on gfx950's block-scaled matrix instruction
// v_mfma_scale_f32_16x16x128_f8f6f4 (A = E4M3 rows, B = E2M1 weights). Its
// operand layout, as measured on the device:
//   B (4-bit): lane c + 16 g holds K = 32 g .. 32 g + 31 of column c, 16 bytes,
//              element 2 i in the low nibble of byte i;
//   A (8-bit): lane r + 16 g holds K = 16 g .. 16 g + 15 (bytes 0..15) and
//              K = 64 + 16 g .. 64 + 16 g + 15 (bytes 16..31) of row r;
//   scales:    the scale byte of lane r + 16 g applies to block g, K = 32 g ..
//              32 g + 31, of row (or column) r; a byte select picks one of the
//              four bytes of the lane's scale register;
//   D:         as the other 16x16 instructions, lane c + 16 q holds rows 4 q .. 4 q + 3
//              of column c.
// Products of the element values are exact; the instruction accumulates them
// in float32.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "lds_dma.h"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kMxBlock = 32;
constexpr int kMxKStep = 128;  // K of one MFMA
constexpr int kXcdsMx = 8;  // workgroup ids are dealt to the 8 XCDs round-robin

// ------------------------------------------------------------ conversion

// floor(log2(a)) of a positive finite float (subnormals included).
__device__ __forceinline__ int floor_log2(float a) {
    const uint32_t b = __float_as_uint(a);
    const int ef = static_cast<int>((b >> 23) & 0xffu);
    if (ef > 0) return ef - 127;
    return -149 + (31 - __clz(static_cast<int>(b & 0x7fffffu)));
}

// Shared exponent of a block with largest magnitude amax (-127 for an all-zero block).
__device__ __forceinline__ int mx_block_exp(float amax, int emax) {
    if (!(amax > 0.f)) return -127;
    return min(max(floor_log2(amax) - emax, -127), 127);
}

// Magnitude code of y = |v| / 2^s in E2M1 (3 bits), round to nearest even, saturating.
__device__ __forceinline__ uint32_t e2m1_mag(float y) {
    if (y >= 6.f) return 7u;
    if (y < 1.f) return static_cast<uint32_t>(rintf(y * 2.f));             // 0, 0.5, 1 -> codes 0, 1, 2
    const int e = floor_log2(y);                                           // 0, 1 or 2
    const float m = rintf((ldexpf(y, -e) - 1.f) * 2.f);                    // 0, 1 or 2 (2 carries)
    return static_cast<uint32_t>(((e + 1) << 1) + static_cast<int>(m));
}

// Magnitude code of y in E4M3 (7 bits), round to nearest even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_mag(float y) {
    if (y >= 448.f) return 0x7eu;
    if (y < 0.015625f) return static_cast<uint32_t>(rintf(y * 512.f));     // subnormals, 8 -> 2^-6
    const int e = floor_log2(y);                                           // -6 .. 8
    const float m = rintf((ldexpf(y, -e) - 1.f) * 8.f);                    // 0 .. 8 (8 carries)
    return static_cast<uint32_t>(((e + 7) << 3) + static_cast<int>(m));
}

template <class In>
__device__ __forceinline__ float load_elem(const In* p);
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p) { return bf16_bits_to_f32(*p); }
template <>
__device__ __forceinline__ float load_elem<float>(const float* p) { return *p; }

// Weight layouts in matrix-core order (rows counted across all matrices, N % 16 == 0):
//  codes: each 16-row x 128-K tile (one K step of a 16-row MFMA block) is one
//  contiguous kilobyte, tiles in (row block, K step) order; inside it row r's 64
//  bytes, inside those block kb % 4's 16 bytes (element 2 i in the low nibble of
//  byte i), so one wavefront's operand load for a block and K step reads one
//  kilobyte;
//  scales: each 16-row x 512-K group is 256 contiguous bytes, groups in (row
//  block, four K steps) order; inside it row r's 16 bytes, holding the scales of
//  the row's 16 blocks transposed 4 x 4 (byte 4 g + j = block 4 j + g), so one
//  32-bit word gives lane group g the scales of four consecutive K steps.
__device__ __host__ __forceinline__ int64_t wcode_offset(int64_t n, int kb, int K) {
    return ((n / 16) * (K / kMxKStep) + kb / 4) * 1024 + (n % 16) * 64 + (kb % 4) * 16;
}
__device__ __host__ __forceinline__ int64_t wscale_offset(int64_t n, int kb, int K) {
    return ((n / 16) * (K / (4 * kMxKStep)) + kb / 16) * 256 + (n % 16) * 16 + (kb % 4) * 4 + (kb / 4) % 4;
}

// One thread per block of 32 along K. kFp4: E2M1 codes packed two per byte, codes
// and scales in matrix-core order (weights); else E4M3 codes, one per byte, codes
// and scales in row order (activations).
template <bool kFp4, class In>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const In* __restrict__ in, int64_t rows, int K,
                                                          uint8_t* __restrict__ q, uint8_t* __restrict__ scales) {
    const int nb = K / kMxBlock;
    const int64_t blk = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (blk >= rows * nb) return;
    const int64_t row = blk / nb;
    const int kb = static_cast<int>(blk % nb);
    const In* src = in + row * K + static_cast<int64_t>(kb) * kMxBlock;
    float v[kMxBlock];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < kMxBlock; ++i) {
        v[i] = load_elem<In>(src + i);
        amax = fmaxf(amax, fabsf(v[i]));
    }
    const int s = mx_block_exp(amax, kFp4 ? 2 : 8);
    if (kFp4) {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < kMxBlock; ++i) {
            const uint32_t c = e2m1_mag(ldexpf(fabsf(v[i]), -s)) | (signbit(v[i]) ? 8u : 0u);
            w[i / 8] |= c << (4 * (i % 8));
        }
        *reinterpret_cast<uint4*>(q + wcode_offset(row, kb, K)) = make_uint4(w[0], w[1], w[2], w[3]);
        scales[wscale_offset(row, kb, K)] = static_cast<uint8_t>(s + 127);
    } else {
        uint32_t w[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < kMxBlock; ++i) {
            const uint32_t c = e4m3_mag(ldexpf(fabsf(v[i]), -s)) | (signbit(v[i]) ? 0x80u : 0u);
            w[i / 4] |= c << (8 * (i % 4));
        }
        uint4* dst = reinterpret_cast<uint4*>(q + row * K + kb * kMxBlock);
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
        scales[row * nb + kb] = static_cast<uint8_t>(s + 127);
    }
}

// --------------------------------------------------------- grouped GEMM
//
// Work unit and schedule as in the bf16 grouped GEMM (m-tiles of one expert
// from the device-built tile list, here of up to 128 rows, n-tiles of the
// weight rows, m-tiles of one expert innermost within each XCD's contiguous
// share). Workgroup: 8 wavefronts; each owns four 16-row blocks of weight rows
// (gate and up rows of the same 32 outputs for the gate/up pass, 64 output rows
// for the down pass) and every row of the m-tile, so each 32-byte A fragment
// read from LDS feeds four matrix instructions. Per K step of 128: the A rows (128
// bytes each) and their four scale bytes are staged in LDS, double-buffered;
// each lane loads its 16 bytes of E2M1 weights per block straight into
// registers (one kilobyte per wavefront, contiguous) three steps ahead, and one
// scale word per block every four steps.

constexpr int kMxWaves = 8;
constexpr int kMxThreads = kMxWaves * 64;
constexpr int kMxNB = 4;
constexpr int kMxKS = 128;
constexpr int kMxMaxMB = 8;
constexpr int kMxBM = 16 * kMxMaxMB;
constexpr int kMxARow = kMxKS + 32;  // LDS bytes per staged row: 32 B of padding keeps the 16-byte
                                     // fragment reads of 16 rows conflict-free (16 B measured 39 %
                                     // of LDS-active cycles in bank conflicts)
constexpr int kMxRowsPerPass = kMxThreads / (kMxKS / 16);
static_assert(kMxBM % kMxRowsPerPass == 0, "whole staging passes");

template <int kSel>
__device__ __forceinline__ f32x4 mfma_e4m3_e2m1(const v8i& a, const v8i& b, const f32x4& c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, kSel, sb);
}

template <bool kGated, int kMB>
__device__ __forceinline__ void mx_tile(uint8_t* sA, uint32_t* sS, const uint8_t* __restrict__ A,
                                        const uint8_t* __restrict__ As, const int32_t* __restrict__ A_rows,
                                        int64_t A_nrows, int64_t row0, int M, const uint8_t* const (&wq)[kMxNB],
                                        const uint8_t* const (&wsc)[kMxNB], uint32_t lane_q, uint32_t lane_s,
                                        bool wave_on, int N, int K, int n_wave,
                                        float* __restrict__ C) {
    constexpr int kPasses = (16 * kMB + kMxRowsPerPass - 1) / kMxRowsPerPass;
    const int tid = threadIdx.x, lane = tid & 63;
    const int fr = lane & 15, fg = lane >> 4;
    const int nb = K / kMxBlock;

    // staging: thread -> (row, 16-byte chunk); the first 16 * kMB threads also move a scale word
    const int a_row = tid / (kMxKS / 16), a_chunk = tid % (kMxKS / 16);
    int64_t a_off[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int64_t r = row0 + min(p * kMxRowsPerPass + a_row, M - 1);
        const int64_t src = A_rows ? min(max(static_cast<int64_t>(A_rows[r]), int64_t(0)), A_nrows - 1) : r;
        a_off[p] = src * K + a_chunk * 16;
    }
    const bool s_on = tid < 16 * kMB;
    int64_t s_off;
    {
        const int64_t r = row0 + min(tid, M - 1);
        const int64_t src = A_rows ? min(max(static_cast<int64_t>(A_rows[r]), int64_t(0)), A_nrows - 1) : r;
        s_off = src * nb;
    }
    constexpr int kBufA = kMxBM * kMxARow, kBufS = kMxBM;

    f32x4 acc[kMxNB][kMB];
#pragma unroll
    for (int b = 0; b < kMxNB; ++b)
#pragma unroll
        for (int i = 0; i < kMB; ++i) acc[b][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / kMxKS;  // a multiple of 4
    u32x4 ar[2][kPasses];      // A rows, two K steps ahead
    uint32_t sr[2] = {0u, 0u}; // their scale words
    auto load_a = [&](u32x4 (&dst)[kPasses], uint32_t& sdst, int s) {
#pragma unroll
        for (int p = 0; p < kPasses; ++p) dst[p] = *reinterpret_cast<const u32x4*>(A + a_off[p] + s * kMxKS);
        if (s_on) sdst = *reinterpret_cast<const uint32_t*>(As + s_off + s * 4);
    };
    auto store_a = [&](int buf, const u32x4 (&src)[kPasses], uint32_t ssrc) {
#pragma unroll
        for (int p = 0; p < kPasses; ++p)
            *reinterpret_cast<u32x4*>(sA + buf * kBufA + (p * kMxRowsPerPass + a_row) * kMxARow + a_chunk * 16) =
                src[p];
        if (s_on) sS[buf * kBufS + tid] = ssrc;
    };
    u32x4 bq[4][kMxNB];        // weights, a ring of four K steps (three ahead)
    uint32_t bs[2][kMxNB];     // weight scale words, two sets of four K steps
    auto load_b = [&](u32x4 (&dst)[kMxNB], int s) {
#pragma unroll
        for (int b = 0; b < kMxNB; ++b) dst[b] = *reinterpret_cast<const u32x4*>(wq[b] + (lane_q + s * 1024u));
    };
    auto load_bs = [&](uint32_t (&dst)[kMxNB], int q4) {
#pragma unroll
        for (int b = 0; b < kMxNB; ++b) dst[b] = *reinterpret_cast<const uint32_t*>(wsc[b] + (lane_s + q4 * 256u));
    };
    // multiply one K step from LDS buffer `buf` with weights w and scale byte sel of words ws
    auto step = [&](int buf, const u32x4 (&w)[kMxNB], const uint32_t (&ws)[kMxNB], auto sel) {
        constexpr int kSel = decltype(sel)::value;
        v8i bop[kMxNB];
#pragma unroll
        for (int b = 0; b < kMxNB; ++b) bop[b] = v8i{static_cast<int>(w[b].x), static_cast<int>(w[b].y),
                                                    static_cast<int>(w[b].z), static_cast<int>(w[b].w), 0, 0, 0, 0};
        const uint8_t* arow = sA + buf * kBufA + fr * kMxARow + 16 * fg;
        const uint32_t* srow = sS + buf * kBufS + fr;
#pragma unroll
        for (int i = 0; i < kMB; ++i) {
            const u32x4 lo = *reinterpret_cast<const u32x4*>(arow + i * 16 * kMxARow);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(arow + i * 16 * kMxARow + 64);
            const v8i aop = v8i{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z),
                                static_cast<int>(lo.w), static_cast<int>(hi.x), static_cast<int>(hi.y),
                                static_cast<int>(hi.z), static_cast<int>(hi.w)};
            const int sa = static_cast<int>(srow[i * 16] >> (8 * fg));
#pragma unroll
            for (int b = 0; b < kMxNB; ++b)
                acc[b][i] = mfma_e4m3_e2m1<kSel>(aop, bop[b], acc[b][i], sa, static_cast<int>(ws[b]));
        }
    };

    load_a(ar[0], sr[0], 0);
    load_a(ar[1], sr[1], min(1, nk - 1));
    load_b(bq[0], 0);
    load_b(bq[1], min(1, nk - 1));
    load_b(bq[2], min(2, nk - 1));
    load_bs(bs[0], 0);
    store_a(0, ar[0], sr[0]);
    __syncthreads();
    // Eight steps per trip (every register index a compile-time constant): steps
    // 0-3 use scale word set 0 (word s0 / 4), steps 4-7 set 1 (word s0 / 4 + 1),
    // each set loaded four steps before it is used. Step U: load A rows of step
    // s + 2, then weights of step s + 3 (vector-memory counters retire in issue
    // order, so waiting for the A rows of s + 1 never waits for later weights),
    // multiply step s (scale byte U % 4), store the A rows of s + 1 in the other
    // LDS buffer, barrier.
#define MOE_MX_STEP(U, SET)                                                                           \
    {                                                                                                 \
        const int s = s0 + (U);                                                                       \
        load_a(ar[(U) % 2], sr[(U) % 2], min(s + 2, nk - 1));                                         \
        load_b(bq[((U) + 3) % 4], min(s + 3, nk - 1));                                                \
        if (wave_on) step((U) % 2, bq[(U) % 4], bs[SET], std::integral_constant<int, (U) % 4>{});     \
        store_a(((U) + 1) % 2, ar[((U) + 1) % 2], sr[((U) + 1) % 2]);                                 \
        __syncthreads();                                                                              \
    }
    for (int s0 = 0; s0 < nk; s0 += 8) {
        load_bs(bs[1], min(s0 / 4 + 1, nk / 4 - 1));
        MOE_MX_STEP(0, 0) MOE_MX_STEP(1, 0) MOE_MX_STEP(2, 0) MOE_MX_STEP(3, 0)
        if (s0 + 4 < nk) {  // uniform
            load_bs(bs[0], min(s0 / 4 + 2, nk / 4 - 1));
            MOE_MX_STEP(4, 1) MOE_MX_STEP(5, 1) MOE_MX_STEP(6, 1) MOE_MX_STEP(7, 1)
        }
    }
#undef MOE_MX_STEP

    if (!wave_on) return;
    // Every value first, then the stores back to back: a store reads its data and
    // address registers after issue, so interleaving each store with the next
    // value's arithmetic would make the compiler wait for every store to finish.
    if (kGated) {  // H row (float32): gate blocks 0 .. kMxNB / 2 - 1, then the same rows of up
#pragma unroll
        for (int c = 0; c < kMxNB / 2; ++c)
#pragma unroll
            for (int i = 0; i < kMB; ++i)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const float g = acc[c][i][qq], u = acc[kMxNB / 2 + c][i][qq];
                    acc[c][i][qq] = g / (1.0f + __expf(-g)) * u;
                }
    }
    float* cbase = C + row0 * N + n_wave + fr;
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int r = i * 16 + 4 * fg + qq;
            if (r >= M) continue;
            float* crow = cbase + static_cast<int64_t>(r) * N;
            if (kGated) {
#pragma unroll
                for (int c = 0; c < kMxNB / 2; ++c) crow[16 * c] = acc[c][i][qq];
            } else {
#pragma unroll
                for (int b = 0; b < kMxNB; ++b) __builtin_nontemporal_store(acc[b][i][qq], crow + 16 * b);  // Y rows
            }
        }
    }
}

template <bool kGated>
__global__ __launch_bounds__(kMxThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
void mx_grouped_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
                       const int32_t* __restrict__ A_rows, int64_t A_nrows, const int4* __restrict__ tiles,
                       const int32_t* __restrict__ tile_start, int E, int n_tiles, const uint8_t* __restrict__ W0q,
                       const uint8_t* __restrict__ W0s, const uint8_t* __restrict__ W1q,
                       const uint8_t* __restrict__ W1s, int N, int K, float* __restrict__ C) {
    constexpr int kColsW = kGated ? 16 * kMxNB / 2 : 16 * kMxNB;
    constexpr int kColsWG = kColsW * kMxWaves;
    __shared__ __attribute__((aligned(16))) uint8_t sA[2 * kMxBM * kMxARow];
    __shared__ uint32_t sS[2 * kMxBM];

    const int n_mt = tile_start[E];
    const int xcd = blockIdx.x % kXcdsMx;
    const int j = blockIdx.x / kXcdsMx;
    const int lo = static_cast<int>(static_cast<int64_t>(xcd) * n_mt / kXcdsMx);
    const int hi = static_cast<int>(static_cast<int64_t>(xcd + 1) * n_mt / kXcdsMx);
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

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_wave = nt * kColsWG + wave * kColsW;
    const bool wave_on = n_wave < N;
    const int n_safe = wave_on ? n_wave : 0;
    const int fr = lane & 15, fg = lane >> 4;
    const int64_t wrows = static_cast<int64_t>(e) * N;  // first weight row of expert e
    // each block's tile row (16 weight rows) starts at a wave-uniform address; a lane's operand
    // sits at a fixed offset inside every 1 KiB tile (and every 256-byte scale group)
    const uint8_t* wq[kMxNB];
    const uint8_t* wsc[kMxNB];
#pragma unroll
    for (int b = 0; b < kMxNB; ++b) {
        const bool up = kGated && b >= kMxNB / 2;  // gate/up: blocks 0 .. kMxNB / 2 - 1 gate, then up
        const uint8_t* q = up ? W1q : W0q;
        const uint8_t* s = up ? W1s : W0s;
        const int64_t n0 = wrows + n_safe + 16 * (kGated ? b % (kMxNB / 2) : b);  // a multiple of 16
        wq[b] = static_cast<const uint8_t*>(uniform_ptr(q + wcode_offset(n0, 0, K)));
        wsc[b] = static_cast<const uint8_t*>(uniform_ptr(s + wscale_offset(n0, 0, K)));
    }
    const uint32_t lane_q = 64u * fr + 16u * fg;  // K step s: + s * 1024
    const uint32_t lane_s = 16u * fr + 4u * fg;   // four K steps q4: + q4 * 256
    const int mb = min(kMxMaxMB, (M + 31) / 32 * 2);  // 2, 4, 6 or 8 blocks
#define MOE_MX_TILE(NB)                                                                                   \
    if (mb == (NB)) {                                                                                     \
        mx_tile<kGated, (NB)>(sA, sS, A, As, A_rows, A_nrows, row0, M, wq, wsc, lane_q, lane_s, wave_on, N, K, n_wave, \
                              C);                                                                         \
        return;                                                                                           \
    }
    MOE_MX_TILE(2)
    MOE_MX_TILE(4)
    MOE_MX_TILE(6)
    MOE_MX_TILE(8)
#undef MOE_MX_TILE
}

// ---------------------------------------------------------------- launchers

int mx_tile_rows() { return kMxBM; }

hipError_t launch_mx_quantize(const void* in, bool in_f32, int64_t rows, int K, bool fp4, uint8_t* q,
                              uint8_t* scales, hipStream_t stream) {
    const int64_t n = rows * (K / kMxBlock);
    if (n == 0) return hipSuccess;
    dim3 grid(static_cast<unsigned>((n + 255) / 256));
    if (fp4) {
        if (in_f32) return hipErrorInvalidValue;
        hipLaunchKernelGGL((mx_quantize_kernel<true, uint16_t>), grid, dim3(256), 0, stream,
                           static_cast<const uint16_t*>(in), rows, K, q, scales);
    } else if (in_f32) {
        hipLaunchKernelGGL((mx_quantize_kernel<false, float>), grid, dim3(256), 0, stream,
                           static_cast<const float*>(in), rows, K, q, scales);
    } else {
        hipLaunchKernelGGL((mx_quantize_kernel<false, uint16_t>), grid, dim3(256), 0, stream,
                           static_cast<const uint16_t*>(in), rows, K, q, scales);
    }
    return hipGetLastError();
}

hipError_t launch_mx_ffn_pass(bool gated, const uint8_t* a, const uint8_t* a_scales, const int32_t* a_rows,
                              int64_t a_nrows, const int4* tiles, const int32_t* tile_start, int64_t n_rows, int E,
                              const uint8_t* w0q, const uint8_t* w0s, const uint8_t* w1q, const uint8_t* w1s, int N,
                              int K, float* c, hipStream_t stream) {
    const int cols_wg = (gated ? 16 * kMxNB / 2 : 16 * kMxNB) * kMxWaves;
    const int n_tiles = (N + cols_wg - 1) / cols_wg;
    const int slots = (ffn_max_tiles(n_rows, E) + kXcdsMx - 1) / kXcdsMx;
    const int64_t grid = static_cast<int64_t>(kXcdsMx) * slots * n_tiles;
    if (gated)
        hipLaunchKernelGGL((mx_grouped_kernel<true>), dim3(static_cast<unsigned>(grid)), dim3(kMxThreads), 0, stream,
                           a, a_scales, a_rows, a_nrows, tiles, tile_start, E, n_tiles, w0q, w0s, w1q, w1s, N, K, c);
    else
        hipLaunchKernelGGL((mx_grouped_kernel<false>), dim3(static_cast<unsigned>(grid)), dim3(kMxThreads), 0,
                           stream, a, a_scales, a_rows, a_nrows, tiles, tile_start, E, n_tiles, w0q, w0s, w0q, w0s, N,
                           K, c);
    return hipGetLastError();
}

}  // namespace moe
