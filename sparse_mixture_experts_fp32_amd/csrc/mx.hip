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

// Codes of four elements v[0..3] in E4M3 scaled by 2^-s, packed into one word (element i in byte i):
// y = |v| / 2^s (exact: a power-of-two scaling), capped at the largest value 448, rounded to the
// nearest value with ties to the even code by the matrix cores' float32 -> E4M3 conversion (for every
// float32 y in [0, 448] it equals the rounding the OCP MX conversion defines), and the sign of v on
// top, also where y rounds to zero.
__device__ __forceinline__ uint32_t e4m3_codes4(const float* v, int s) {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = fminf(ldexpf(fabsf(v[i]), -s), 448.f);
    int packed = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    packed = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], packed, true);
    uint32_t sign = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) sign |= signbit(v[i]) ? (0x80u << (8 * i)) : 0u;
    return static_cast<uint32_t>(packed) | sign;
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
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = e4m3_codes4(v + 4 * i, s);
        uint4* dst = reinterpret_cast<uint4*>(q + row * K + kb * kMxBlock);
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
        scales[row * nb + kb] = static_cast<uint8_t>(s + 127);
    }
}

// --------------------------------------------------------- grouped GEMM
//
// Work unit and schedule as in the bf16 ring kernel (m-tiles of one expert from
// the device-built tile list, here of up to 144 rows; n-tiles of the weight
// rows; the m-tiles that share an expert's n-tile side by side on one XCD).
// Workgroup: 8 wavefronts; each owns four 16-row blocks of weight rows (gate
// and up rows of the same 32 outputs for the gate/up pass, 64 output rows for
// the down pass) and every row of the m-tile, so each 32-byte A fragment read
// from LDS feeds four matrix instructions.
//
// Operands reach LDS through direct-to-LDS loads into a ring of three stages,
// one K step of 128 each:
//   * A rows (E4M3): per 16-row block two loads of 1 KiB, the first holding
//     bytes 0..63 of each row's K step, the second bytes 64..127, lane l at
//     byte 16 l as the fragment reads want them (row l % 16, bytes 16 (l / 16)
//     of each half); the row's scale word (its four block scales for the step)
//     at word r;
//   * weights (E2M1): one contiguous kilobyte per block and step, permuted on
//     the way so that lane l's 16 bytes land at byte 16 l;
//   * weight scales: one 256-byte group per block and four steps, in a region
//     of each wave's own, loaded with the step that first needs it.
// A wave's weight region of a slot is its own, so its weight loads for step
// s + 3 go out as soon as it has finished reading step s, before the next
// barrier; the shared A rows for step s + 2 go out after the barrier that
// starts step s. The waits are exact counts of the loads issued after the
// ones a step needs (vector-memory counters retire in issue order), so a step
// never waits for later stages.
constexpr int kMxWaves = 8;
constexpr int kMxThreads = kMxWaves * 64;
constexpr int kMxNB = 4;                                 // 16-row weight blocks per wave
constexpr int kMxStages = 3;
constexpr int kMxMaxMB = 9;                              // 16-row A blocks per m-tile (144 rows)
constexpr int kMxAStage = kMxMaxMB * 2048;               // A rows of one step
constexpr int kMxWStage = kMxWaves * kMxNB * 1024;       // weight rows of one step
constexpr int kMxSStage = 16 * kMxMaxMB * 4;             // A scale words of one step
constexpr int kMxStage = kMxAStage + kMxWStage + kMxSStage;
constexpr int kMxWSOff = kMxStages * kMxStage;           // weight scale groups, 1 KiB per wave
constexpr int kMxLds = kMxWSOff + kMxWaves * 1024;
static_assert(kMxLds <= 160 * 1024, "the ring fits one CU's LDS");
constexpr int kMxAInstMax = (2 * kMxMaxMB + kMxWaves - 1) / kMxWaves;  // A loads per wave and step, at most
constexpr int kMxSInst = (16 * kMxMaxMB + 63) / 64;      // scale-word loads per step (the last one partial)

template <int kSel>
__device__ __forceinline__ f32x4 mfma_e4m3_e2m1(const v8i& a, const v8i& b, const f32x4& c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, kSel, sb);
}

// Wait until at most n (wave-uniform, 0..15) of this wave's vector-memory
// operations are in flight and its LDS operations are done, then barrier.
__device__ __forceinline__ void mx_wait_barrier(int n) {
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
        case 12: wait_barrier<12>(); break;
        case 13: wait_barrier<13>(); break;
        case 14: wait_barrier<14>(); break;
        default: wait_barrier<15>(); break;
    }
}

// Keep each step's matrix instructions inside the step: an empty volatile asm
// that reads and rewrites every accumulator (it emits no instruction).
template <int kMB>
__device__ __forceinline__ void pin_acc(f32x4 (&acc)[kMxNB][kMB]) {
#pragma unroll
    for (int j = 0; j < kMxNB; ++j)
#pragma unroll
        for (int i = 0; i < kMB; ++i) asm volatile("" : "+v"(acc[j][i]));
}

// One K step from one ring slot: acc[j][i] += A block i x weight block j, scale
// byte kSel of the weight scale words (a word covers four steps). Fragment i + 1
// is read while fragment i multiplies; the fences keep that order.
template <int kMB, int kSel>
__device__ __forceinline__ void mx_step(f32x4 (&acc)[kMxNB][kMB], const uint8_t* a_lds, const uint32_t* s_lds,
                                        const uint8_t* w_lds, uint32_t (&ws)[kMxNB], const uint32_t* ws_lds,
                                        int fg) {
    if (kSel == 0) {
#pragma unroll
        for (int j = 0; j < kMxNB; ++j) ws[j] = ws_lds[64 * j];
    }
    v8i b[kMxNB];
#pragma unroll
    for (int j = 0; j < kMxNB; ++j) {
        const u32x4 t = *reinterpret_cast<const u32x4*>(w_lds + 1024 * j);
        b[j] = v8i{static_cast<int>(t.x), static_cast<int>(t.y), static_cast<int>(t.z), static_cast<int>(t.w), 0, 0,
                   0, 0};
    }
    u32x4 lo[2], hi[2];
    uint32_t sw[2];
    lo[0] = *reinterpret_cast<const u32x4*>(a_lds);
    hi[0] = *reinterpret_cast<const u32x4*>(a_lds + 1024);
    sw[0] = s_lds[0];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
        if (i + 1 < kMB) {
            lo[(i + 1) % 2] = *reinterpret_cast<const u32x4*>(a_lds + 2048 * (i + 1));
            hi[(i + 1) % 2] = *reinterpret_cast<const u32x4*>(a_lds + 2048 * (i + 1) + 1024);
            sw[(i + 1) % 2] = s_lds[16 * (i + 1)];
        }
        __builtin_amdgcn_sched_barrier(0);
        const u32x4 l = lo[i % 2], h = hi[i % 2];
        const v8i a = v8i{static_cast<int>(l.x), static_cast<int>(l.y), static_cast<int>(l.z), static_cast<int>(l.w),
                          static_cast<int>(h.x), static_cast<int>(h.y), static_cast<int>(h.z), static_cast<int>(h.w)};
        const int sa = static_cast<int>(sw[i % 2] >> (8 * fg));
#pragma unroll
        for (int j = 0; j < kMxNB; ++j)
            acc[j][i] = mfma_e4m3_e2m1<kSel>(a, b[j], acc[j][i], sa, static_cast<int>(ws[j]));
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <bool kGated, int kMB>
__device__ __forceinline__ void mx_tile(uint8_t* lds, const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
                                        const int32_t* __restrict__ A_rows, int64_t A_nrows, int64_t row0, int M,
                                        const uint8_t* const (&wq)[kMxNB], const uint8_t* const (&wsc)[kMxNB], int N,
                                        int K, int n_out, float* __restrict__ C) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int fr = lane & 15, fg = lane >> 4;
    const uint32_t base = lds_addr(lds);
    const int nb = K / kMxBlock;
    const int nk = K / kMxKStep;  // a multiple of 4

    // A loads q = wave, wave + 8, wave + 16 (while q < 2 kMB): block q / 2, half q % 2;
    // lane l reads row 16 (q / 2) + l % 16 (clamped to the tile, gathered through
    // A_rows), bytes 64 (q % 2) + 16 (l / 16) of the step. Offsets are 32-bit (A
    // holds fewer than 2^32 bytes; the launcher checks).
    constexpr int kAInst = 2 * kMB;
    int nA = 0;
    uint32_t a_off[kMxAInstMax];
#pragma unroll
    for (int p = 0; p < kMxAInstMax; ++p) {
        const int q = min(wave + kMxWaves * p, kAInst - 1);
        nA += wave + kMxWaves * p < kAInst ? 1 : 0;
        const int64_t r = row0 + min(16 * (q / 2) + fr, M - 1);
        const int64_t src = A_rows ? min(max(static_cast<int64_t>(A_rows[r]), int64_t(0)), A_nrows - 1) : r;
        a_off[p] = static_cast<uint32_t>(src * K + 64 * (q % 2) + 16 * fg);
    }
    // scale-word loads p = 0 .. kMxSInst - 1 by waves 7, 6, ...: lane l moves the word of
    // row 64 p + l (the last load only for the rows that exist in a full tile)
    const int ps = kMxWaves - 1 - wave;
    const bool s_on = ps < kMxSInst;
    const bool s_part = ps == kMxSInst - 1 && (16 * kMxMaxMB) % 64 != 0;
    uint32_t s_off;
    {
        const int64_t r = row0 + min(64 * min(ps, kMxSInst - 1) + lane, M - 1);
        const int64_t src = A_rows ? min(max(static_cast<int64_t>(A_rows[r]), int64_t(0)), A_nrows - 1) : r;
        s_off = static_cast<uint32_t>(src * nb);
    }
    // weight scale groups: lane l moves bytes 16 (l % 16) of block l / 16's group
    const int lb = lane >> 4;
    const uint8_t* ws_src = (lb == 0 ? wsc[0] : lb == 1 ? wsc[1] : lb == 2 ? wsc[2] : wsc[3]) + 16 * (lane & 15);
    const uint32_t lane_q = 64u * fr + 16u * fg;  // weights: lane l reads its fragment's 16 bytes
    const int nAS = nA + (s_on ? 1 : 0);

    auto issue_a = [&](int s) {  // A rows and their scale words of step s (after the barrier)
        const uint32_t slot = base + static_cast<uint32_t>((s % kMxStages) * kMxStage);
        if (s_on) {
            const uint32_t dst = slot + kMxAStage + kMxWStage + 256u * ps;
            if (!s_part)
                dma_saddr_dword(dst, As, s_off + 4u * s);
            else if (lane < 16 * kMxMaxMB - 64 * (kMxSInst - 1))
                dma_saddr_dword(dst, As, s_off + 4u * s);
        }
#pragma unroll
        for (int p = 0; p < kMxAInstMax; ++p)
            if (p < nA) dma_saddr(slot + 1024u * (wave + kMxWaves * p), A, a_off[p] + 128u * s);
    };
    auto issue_w = [&](int s) {  // this wave's weights (and scale group) of step s
        const uint32_t slot = base + static_cast<uint32_t>((s % kMxStages) * kMxStage);
        if (s % 4 == 0) dma_vaddr(base + kMxWSOff + 1024u * wave, ws_src + 256 * (s / 4));
        const uint32_t wslot = slot + kMxAStage + 4096u * wave;
#pragma unroll
        for (int j = 0; j < kMxNB; ++j) dma_saddr(wslot + 1024u * j, wq[j], lane_q + 1024u * s);
    };
    // loads issued after the A rows of step s: W(s + 1), A(s + 1), W(s + 2)
    auto after_a = [&](int s) {
        int n = 0;
        if (s + 1 < nk) n += kMxNB + ((s + 1) % 4 == 0 ? 1 : 0) + nAS;
        if (s + 2 < nk) n += kMxNB + ((s + 2) % 4 == 0 ? 1 : 0);
        return n;
    };

    f32x4 acc[kMxNB][kMB];
#pragma unroll
    for (int j = 0; j < kMxNB; ++j)
#pragma unroll
        for (int i = 0; i < kMB; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    issue_w(0);
    issue_a(0);
    if (nk > 1) {
        issue_w(1);
        issue_a(1);
    }
    if (nk > 2) issue_w(2);
    const uint8_t* a_lds = lds + 16 * lane;
    const uint32_t* s_lds = reinterpret_cast<const uint32_t*>(lds + kMxAStage + kMxWStage) + fr;
    const uint8_t* w_lds = lds + kMxAStage + 4096 * wave + 16 * lane;
    const uint32_t* ws_lds = reinterpret_cast<const uint32_t*>(lds + kMxWSOff + 1024 * wave + 16 * fr + 4 * fg);
    uint32_t ws[kMxNB];
    // Step U of a group of four: wait for step s's loads, barrier (every wave is
    // done with step s - 1), issue the A rows of s + 2 into the slot s - 1 used,
    // multiply, then issue this wave's weights of s + 3 into the slot it just read.
#define MOE_MX_STEP(U)                                                                                 \
    {                                                                                                  \
        const int s = s0 + (U);                                                                        \
        mx_wait_barrier(after_a(s));                                                                   \
        if (s + 2 < nk) issue_a(s + 2);                                                                \
        const int off = (s % kMxStages) * kMxStage;                                                    \
        mx_step<kMB, (U)>(acc, a_lds + off, s_lds + off / 4, w_lds + off, ws, ws_lds, fg);             \
        pin_acc(acc);                                                                                  \
        if (s + 3 < nk) {                                                                              \
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");                                         \
            issue_w(s + 3);                                                                            \
        }                                                                                              \
    }
    for (int s0 = 0; s0 < nk; s0 += 4) {
        MOE_MX_STEP(0) MOE_MX_STEP(1) MOE_MX_STEP(2) MOE_MX_STEP(3)
    }
#undef MOE_MX_STEP

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
    float* cbase = C + row0 * N + n_out + fr;
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

// One workgroup per CU (157 KiB of LDS), so the register allocator may give each
// of the two waves per SIMD half the register file.
template <bool kGated>
__global__ __launch_bounds__(kMxThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
void mx_ring_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const int32_t* __restrict__ A_rows,
                    int64_t A_nrows, const int4* __restrict__ tiles, const int32_t* __restrict__ tile_start, int E,
                    int n_tiles, const uint8_t* __restrict__ W0q, const uint8_t* __restrict__ W0s,
                    const uint8_t* __restrict__ W1q, const uint8_t* __restrict__ W1s, int N, int K,
                    float* __restrict__ C) {
    constexpr int kColsW = kGated ? 16 * kMxNB / 2 : 16 * kMxNB;  // output columns per wave
    constexpr int kColsWG = kColsW * kMxWaves;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kMxLds];

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

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_out = nt * kColsWG + wave * kColsW;  // N is a multiple of kColsWG: every wave has columns
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
        const int64_t n0 = wrows + n_out + 16 * (kGated ? b % (kMxNB / 2) : b);  // a multiple of 16
        wq[b] = static_cast<const uint8_t*>(uniform_ptr(q + wcode_offset(n0, 0, K)));
        wsc[b] = static_cast<const uint8_t*>(uniform_ptr(s + wscale_offset(n0, 0, K)));
    }
    const int mb = min(kMxMaxMB, (M + 15) / 16);
#define MOE_MX_TILE(NB)                                                                                  \
    if (mb == (NB)) {                                                                                    \
        mx_tile<kGated, (NB)>(lds, A, As, A_rows, A_nrows, row0, M, wq, wsc, N, K, n_out, C);           \
        return;                                                                                          \
    }
    MOE_MX_TILE(1)
    MOE_MX_TILE(2)
    MOE_MX_TILE(3)
    MOE_MX_TILE(4)
    MOE_MX_TILE(5)
    MOE_MX_TILE(6)
    MOE_MX_TILE(7)
    MOE_MX_TILE(8)
    MOE_MX_TILE(9)
#undef MOE_MX_TILE
}

// ---------------------------------------------------------------- launchers

int mx_tile_rows() { return 16 * kMxMaxMB; }

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
    // whole n-tiles, whole groups of four K steps, 32-bit A offsets
    if (N % cols_wg != 0 || K % (4 * kMxKStep) != 0 || a_nrows * K >= (int64_t(1) << 32)) return hipErrorInvalidValue;
    const int n_tiles = N / cols_wg;
    const int slots = (ffn_max_tiles(n_rows, E) + kXcdsMx - 1) / kXcdsMx;
    const int64_t grid = static_cast<int64_t>(kXcdsMx) * slots * n_tiles;
    if (gated)
        hipLaunchKernelGGL((mx_ring_kernel<true>), dim3(static_cast<unsigned>(grid)), dim3(kMxThreads), 0, stream, a,
                           a_scales, a_rows, a_nrows, tiles, tile_start, E, n_tiles, w0q, w0s, w1q, w1s, N, K, c);
    else
        hipLaunchKernelGGL((mx_ring_kernel<false>), dim3(static_cast<unsigned>(grid)), dim3(kMxThreads), 0, stream, a,
                           a_scales, a_rows, a_nrows, tiles, tile_start, E, n_tiles, w0q, w0s, w0q, w0s, N, K, c);
    return hipGetLastError();
}

}  // namespace moe
