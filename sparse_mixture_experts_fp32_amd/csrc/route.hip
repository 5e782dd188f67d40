// Routing: gate logits (a dense contraction on the matrix cores) and the
// per-token softmax / top-k / renormalisation (one wavefront per token).
//
// Gate, softmax and top-k: "Kimi K3: The Open Model That Just Cornered the AI
// Frontier", section "Mixture-of-Experts with Dynamic Load Balancing".
#include "device_common.h"
#include "launch.h"
#include "lds_dma.h"
#include "select.h"

#include <algorithm>

namespace moe {

// ---------------------------------------------------------------- gate GEMM
//
// logits[t, e] = sum_i x[t, i] * w[e, i] (+ bias[e]), x bf16, w float32.
//
// Every float32 weight is split exactly into three bfloat16 terms,
// w = hi + mid + lo (8 + 8 + 8 significant bits; each term is the RNE rounding
// of what the previous ones left, and that residue is exact), once per call by
// router_split_kernel. Each product x * part is exact in float32 because both
// factors carry at most 8 significant bits, and the three products accumulate
// in the MFMA's float32 accumulator: a float32 accumulation of exact products
// on the bf16 matrix cores. Per 32-deep K step and output block the order is
// lo, mid, hi.
//
// The parts are written in MFMA fragment order (16 experts x 32 K per
// kilobyte, lane l's 16 bytes = expert l % 16, K 8 (l / 16) .. + 7), the expert
// count padded to a multiple of 16 with zero rows, so that one direct-to-LDS
// load brings one operand.
//
// router_gemm_kernel<kBM, kWM, kSt>: kBM tokens x 128 experts per 512-thread
// workgroup, the 8 waves as kWM token rows x (8 / kWM) expert columns, each
// wave owning 8 x 16 tokens and 128 / (8 / kWM) experts, so every fragment read
// from LDS feeds between 6 and 12 MFMAs. x rows and weight parts go straight
// into an LDS ring of kSt stages (one K step of 32 each; the weight loads of a
// step are issued before its x rows). Two shapes:
//  * 256 tokens, waves 2 x 4, three stages (two in flight while one is
//    multiplied): batches of up to a few thousand tokens;
//  * 512 tokens, waves 4 x 2, two stages: once the token x expert tiles alone
//    fill the CUs, the taller tile carries half the weight bytes per MFMA, which
//    matters more there than a second stage in flight.
// Each step reads the 3 x (experts / 16) weight fragments and the first x
// fragment, then reads x fragment i + 1 while fragment i multiplies
// (scheduling fences keep that order). The traffic of such a GEMM is x once per
// expert block plus the weights once per token block, so the tile is tall in
// tokens (the three parts weigh three x rows). K is split into S ranges when
// the token x expert tiles alone would leave CUs idle (a decode-sized batch has
// one token block): each range writes a float32 partial sum and
// router_reduce_kernel adds the S partials in range order (and the bias), so
// the result does not depend on scheduling. The workgroups of one (token block,
// K range) are dealt to one XCD back to back, so its x rows come from HBM once.

constexpr int kRtBN = 128, kRtKS = 32;
constexpr int kRtBStage = 3 * (kRtBN / 16) * 1024;    // 24 KiB of weight parts per stage
constexpr int kRtNB = kRtBStage / 1024 / 8;           // weight-part loads per wave per stage (3)

static __host__ __device__ int router_epad(int E) { return (E + 15) / 16 * 16; }

// w [E, d] float32 -> parts [3][Epad x d] bf16 in fragment order, w = parts[0] + parts[1] + parts[2]
// exactly; rows E .. Epad - 1 are zero. One thread per 16 bytes of each part, in destination order
// (a wavefront writes one contiguous kilobyte; its lane l reads 8 consecutive K of expert l % 16).
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ w, int E, int epad, int d,
                                                           uint16_t* __restrict__ parts) {
    const int64_t chunks = static_cast<int64_t>(epad) * (d / 8);
    const int64_t pn = static_cast<int64_t>(epad) * d;  // elements per part
    const int ktiles = d / 32;
    for (int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < chunks;
         c += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t tile = c / 64;
        const int l = static_cast<int>(c % 64);
        const int e = static_cast<int>(tile / ktiles) * 16 + l % 16;
        const int k = static_cast<int>(tile % ktiles) * 32 + 8 * (l / 16);
        float v[8];
        if (e < E) {
            const float4 lo = *reinterpret_cast<const float4*>(w + static_cast<int64_t>(e) * d + k);
            const float4 hi = *reinterpret_cast<const float4*>(w + static_cast<int64_t>(e) * d + k + 4);
            v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w; v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = 0.f;
        }
        uint16_t h[8], m[8], lo16[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            h[i] = f32_to_bf16_bits(v[i]);
            const float r1 = v[i] - bf16_bits_to_f32(h[i]);
            m[i] = f32_to_bf16_bits(r1);
            lo16[i] = f32_to_bf16_bits(r1 - bf16_bits_to_f32(m[i]));
        }
        u32x4 vh, vm, vl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            vh[i] = h[2 * i] | (static_cast<uint32_t>(h[2 * i + 1]) << 16);
            vm[i] = m[2 * i] | (static_cast<uint32_t>(m[2 * i + 1]) << 16);
            vl[i] = lo16[2 * i] | (static_cast<uint32_t>(lo16[2 * i + 1]) << 16);
        }
        *reinterpret_cast<u32x4*>(parts + 8 * c) = vh;
        *reinterpret_cast<u32x4*>(parts + pn + 8 * c) = vm;
        *reinterpret_cast<u32x4*>(parts + 2 * pn + 8 * c) = vl;
    }
}

// Wait until at most n (wave-uniform, 0..5) of this wave's vector-memory operations are in flight
// and its LDS operations are done, then barrier.
__device__ __forceinline__ void router_wait_barrier(int n) {
    switch (n) {
        case 0: wait_barrier<0>(); break;
        case 1: wait_barrier<1>(); break;
        case 2: wait_barrier<2>(); break;
        case 3: wait_barrier<3>(); break;
        case 4: wait_barrier<4>(); break;
        default: wait_barrier<5>(); break;
    }
}

// Keep each step's matrix instructions inside the step: an empty volatile asm that reads and
// rewrites every accumulator (it emits no instruction).
template <int kMI, int kNJ>
__device__ __forceinline__ void router_pin(f32x4 (&acc)[kMI][kNJ]) {
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
        for (int j = 0; j < kNJ; ++j) asm volatile("" : "+v"(acc[i][j]));
}

// out: logits [T, E] (+ bias) when n_split == 1, else partial sums [n_split][T][E].
template <int kBM, int kWM, int kSt>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 2)))
void router_gemm_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ parts,
                        const float* __restrict__ bias, float* __restrict__ out, int64_t T, int d, int E,
                        int n_mblocks, int n_nblocks, int n_split) {
    constexpr int kWN = 8 / kWM;
    constexpr int kMI = kBM / kWM / 16, kNJ = kRtBN / kWN / 16;  // 16 x 16 blocks per wave
    constexpr int kAStage = (kBM / 16) * 1024;                   // x rows per stage
    constexpr int kStage = kAStage + kRtBStage;
    constexpr int kNA = kBM / 16 / 8;                            // x-row loads per wave per stage
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kSt * kStage];
    // (token block m, K range r) pairs go to XCD (block id % 8) in turn, each with its expert blocks in a row
    const int xcd = blockIdx.x % 8, j = blockIdx.x / 8;
    const int pair = 8 * (j / n_nblocks) + xcd, nblk = j % n_nblocks;
    if (pair >= n_mblocks * n_split) return;  // uniform, before any barrier
    const int mblk = pair / n_split, range = pair % n_split;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % kWM, wn = wave / kWM;
    const int frag_row = lane & 15, frag_k = 8 * (lane >> 4);
    const int64_t m0 = static_cast<int64_t>(mblk) * kBM;
    const int n0 = nblk * kRtBN;
    const int eblocks = router_epad(E) / 16;
    const int64_t pn = static_cast<int64_t>(eblocks) * 16 * d;
    const uint32_t ring_lds = lds_addr(ring);
    const int nk_all = d / kRtKS;
    const int s_lo = static_cast<int>(static_cast<int64_t>(range) * nk_all / n_split);
    const int s_hi = static_cast<int>(static_cast<int64_t>(range + 1) * nk_all / n_split);
    const int nk = s_hi - s_lo;  // >= 1: n_split <= nk_all

    // this wave's loads per stage: x row blocks wave + 8 p (lane: row, K 8 (l / 16)); weight blocks
    // wave + 8 q of the 24 (part idx / 8, expert block idx % 8)
    const uint16_t* a_src[kNA];
#pragma unroll
    for (int p = 0; p < kNA; ++p) {
        const int64_t row = min(m0 + 16 * (wave + 8 * p) + frag_row, T - 1);
        a_src[p] = x + row * d + frag_k + kRtKS * s_lo;
    }
    const uint16_t* b_src[kRtNB];
#pragma unroll
    for (int q = 0; q < kRtNB; ++q) {
        const int idx = wave + 8 * q;
        const int eb = min(n0 / 16 + idx % 8, eblocks - 1);  // clamped: such columns are never stored
        b_src[q] = static_cast<const uint16_t*>(
            uniform_ptr(parts + (idx / 8) * pn + (static_cast<int64_t>(eb) * (d / 32) + s_lo) * 512));
    }
    auto issue = [&](int s) {  // local step s of this K range into ring slot s % kSt
        const uint32_t slot = ring_lds + static_cast<uint32_t>((s % kSt) * kStage);
#pragma unroll
        for (int q = 0; q < kRtNB; ++q)
            dma_saddr(slot + kAStage + 1024u * (wave + 8 * q), b_src[q], 16u * lane + 1024u * s);
#pragma unroll
        for (int p = 0; p < kNA; ++p) dma_vaddr(slot + 1024u * (wave + 8 * p), a_src[p] + kRtKS * s);
    };

    f32x4 acc[kMI][kNJ];
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
        for (int jn = 0; jn < kNJ; ++jn) acc[i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int s = 0; s < kSt - 1; ++s)
        if (s < nk) issue(s);
    const uint8_t* a_lds = ring + 1024 * (kMI * wm) + 16 * lane;
    const uint8_t* b_lds = ring + kAStage + 1024 * (kNJ * wn) + 16 * lane;
    for (int s = 0; s < nk; ++s) {
        // step s has landed once only the later steps' loads (at most kSt - 2 of them) are in flight
        router_wait_barrier((kNA + kRtNB) * min(kSt - 2, nk - 1 - s));
        if (s + kSt - 1 < nk) issue(s + kSt - 1);
        const int off = (s % kSt) * kStage;
        bf16x8 b[3][kNJ];
#pragma unroll
        for (int q = 0; q < 3; ++q)
#pragma unroll
            for (int jn = 0; jn < kNJ; ++jn)
                b[q][jn] = *reinterpret_cast<const bf16x8*>(b_lds + off + 1024 * (8 * q + jn));
        bf16x8 a[2];
        a[0] = *reinterpret_cast<const bf16x8*>(a_lds + off);
#pragma unroll
        for (int i = 0; i < kMI; ++i) {
            if (i + 1 < kMI) a[(i + 1) & 1] = *reinterpret_cast<const bf16x8*>(a_lds + off + 1024 * (i + 1));
#pragma unroll
            for (int jn = 0; jn < kNJ; ++jn) {
                acc[i][jn] = mfma_16x16x32(a[i & 1], b[2][jn], acc[i][jn]);  // smallest part first
                acc[i][jn] = mfma_16x16x32(a[i & 1], b[1][jn], acc[i][jn]);
                acc[i][jn] = mfma_16x16x32(a[i & 1], b[0][jn], acc[i][jn]);
            }
        }
        // the weight fragments and x fragment 0 first, then x fragment i + 1 after the first MFMA of i
        __builtin_amdgcn_sched_group_barrier(0x100, 3 * kNJ + 1, 0);
#pragma unroll
        for (int i = 0; i < kMI; ++i) {
            if (i + 1 < kMI) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 3 * kNJ - 1, 0);
            } else {
                __builtin_amdgcn_sched_group_barrier(0x008, 3 * kNJ, 0);
            }
        }
        router_pin(acc);
    }

    float* dst = n_split == 1 ? out : out + static_cast<int64_t>(range) * T * E;
#pragma unroll
    for (int jn = 0; jn < kNJ; ++jn) {
        const int col = n0 + (kRtBN / kWN) * wn + 16 * jn + frag_row;
        if (col >= E) continue;
        const float bcol = (n_split == 1 && bias) ? bias[col] : 0.f;
#pragma unroll
        for (int i = 0; i < kMI; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t row = m0 + (kBM / kWM) * wm + 16 * i + 4 * (lane >> 4) + q;
                if (row < T) dst[row * E + col] = acc[i][jn][q] + bcol;
            }
    }
}

// logits[t, e] = sum over r = 0 .. n_split - 1 of partial[r][t][e] (in that order) + bias[e]; the
// loads of 8 partials are issued before their adds
__global__ __launch_bounds__(256) void router_reduce_kernel(const float* __restrict__ partial, int n_split,
                                                            const float* __restrict__ bias, int64_t n, int E,
                                                            float* __restrict__ logits) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        float v = partial[i];
        for (int r0 = 1; r0 < n_split; r0 += 8) {
            float p[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) p[u] = r0 + u < n_split ? partial[static_cast<int64_t>(r0 + u) * n + i] : 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (r0 + u < n_split) v += p[u];
        }
        logits[i] = v + (bias ? bias[i % E] : 0.f);
    }
}

// ------------------------------------------------------------ softmax + top-k
//
// One wavefront per token; lane l holds experts l, l + 64, ... Each logit
// becomes a 64-bit key whose upper half orders the float value (-0.0 folded
// onto +0.0, NaN below everything) and whose lower half is ~expert id, so the
// largest key is the largest logit with ties going to the lower id. select_top
// (select.h) leaves the j-th largest key in lane j: a threshold from the lane
// maxima prunes the candidates, which are then ranked in LDS.
//
// Renormalised weights: p_j / sum_{i<k} p_i with p = softmax over all E equals
// exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0): the softmax denominator cancels,
// so only the k selected logits are exponentiated.

template <int NPER>
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ logits,
                                                           int64_t T, int E, int k,
                                                           int32_t* __restrict__ topk_idx,
                                                           float* __restrict__ topk_w) {
    __shared__ uint64_t sel[4][kSelectLds];
    const int lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* row = logits + t * E;

    float v[NPER];
    load_row_strided<NPER>(row, E, 0.f, v);
    // lane j < k: the j-th largest key
    const uint64_t best = select_top<NPER>(v, E, k, sel[threadIdx.x >> 6]);
    const int my_id = static_cast<int>(0xffffffffu - static_cast<uint32_t>(best));
    const float my_val = key_value(static_cast<uint32_t>(best >> 32));
    const float top = __shfl(my_val, 0, kWave);
    const float ex = (lane < k) ? expf(my_val - top) : 0.f;
    const float sum = wave_sum_f32(ex);
    if (lane < k) {
        topk_idx[t * k + lane] = my_id;
        topk_w[t * k + lane] = ex / sum;
    }
}

// ------------------------------------------------------------------ launchers

// Tile height and K ranges. 512-token tiles once the 256-token tiles fill the CUs without a K
// split and the taller tiles take no more rounds of the 256 CUs (counted in 256-token tile
// work). Otherwise 256-token tiles with K split into S ranges: enough (token block, expert block,
// K range) workgroups to give most CUs one, at most 32 ranges (their partial sums are read back
// once more), never a range shorter than one K step.
struct RouterPlan {
    int bm, split;
};
static RouterPlan router_plan(int64_t T, int d, int E) {
    const int64_t nb = (E + kRtBN - 1) / kRtBN;
    const int64_t t256 = ((T + 255) / 256) * nb, t512 = ((T + 511) / 512) * nb;
    if (t256 >= 192) {
        if ((t512 + 255) / 256 * 2 <= (t256 + 255) / 256) return {512, 1};
        return {256, 1};
    }
    const int64_t s = (256 + t256 - 1) / t256;
    return {256, static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(s, 32), d / kRtKS)))};
}

size_t router_ws_bytes(int64_t T, int d, int E) {
    const size_t parts = sizeof(uint16_t) * 3 * static_cast<size_t>(router_epad(E)) * d;
    const int S = router_plan(T, d, E).split;
    const size_t partial = S > 1 ? sizeof(float) * static_cast<size_t>(S) * static_cast<size_t>(T) * E : 0;
    return (parts + 255) / 256 * 256 + partial;
}

hipError_t launch_router_gemm(const uint16_t* x, const float* w, const float* bias, float* logits, int64_t T, int d,
                              int E, void* ws, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    uint16_t* parts = static_cast<uint16_t*>(ws);
    float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                              (sizeof(uint16_t) * 3 * static_cast<size_t>(router_epad(E)) * d + 255) /
                                                  256 * 256);
    const int64_t chunks = static_cast<int64_t>(router_epad(E)) * (d / 8);
    const int64_t blocks = std::min<int64_t>((chunks + 255) / 256, 4096);
    hipLaunchKernelGGL(router_split_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, w, E,
                       router_epad(E), d, parts);
    const RouterPlan plan = router_plan(T, d, E);
    const int S = plan.split;
    const int n_mblocks = static_cast<int>((T + plan.bm - 1) / plan.bm);
    const int n_nblocks = (E + kRtBN - 1) / kRtBN;
    const int64_t pairs = static_cast<int64_t>(n_mblocks) * S;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(8) * ((pairs + 7) / 8) * n_nblocks));
    float* dst = S == 1 ? logits : partial;
    if (plan.bm == 512)
        hipLaunchKernelGGL((router_gemm_kernel<512, 4, 2>), grid, dim3(512), 0, stream, x, parts, bias, dst, T, d, E,
                           n_mblocks, n_nblocks, S);
    else
        hipLaunchKernelGGL((router_gemm_kernel<256, 2, 3>), grid, dim3(512), 0, stream, x, parts, bias, dst, T, d, E,
                           n_mblocks, n_nblocks, S);
    if (S > 1) {
        const int64_t n = T * E;
        const int64_t rb = std::min<int64_t>((n + 255) / 256, 8192);
        hipLaunchKernelGGL(router_reduce_kernel, dim3(static_cast<unsigned>(rb)), dim3(256), 0, stream, partial, S,
                           bias, n, E, logits);
    }
    return hipGetLastError();
}

hipError_t launch_topk_softmax(const float* logits, int64_t T, int E, int k, int32_t* topk_idx,
                               float* topk_w, hipStream_t stream) {
    dim3 grid(static_cast<unsigned>((T + 3) / 4));
    const int nper = (E + 63) / 64;
#define MOE_TOPK_CASE(N)                                                                        \
    case N:                                                                                     \
        hipLaunchKernelGGL(topk_softmax_kernel<N>, grid, dim3(256), 0, stream, logits, T, E, k, \
                           topk_idx, topk_w);                                                   \
        break;
    switch (nper) {
        MOE_TOPK_CASE(1) MOE_TOPK_CASE(2) MOE_TOPK_CASE(3) MOE_TOPK_CASE(4)
        MOE_TOPK_CASE(5) MOE_TOPK_CASE(6) MOE_TOPK_CASE(7) MOE_TOPK_CASE(8)
        MOE_TOPK_CASE(9) MOE_TOPK_CASE(10) MOE_TOPK_CASE(11) MOE_TOPK_CASE(12)
        MOE_TOPK_CASE(13) MOE_TOPK_CASE(14) MOE_TOPK_CASE(15) MOE_TOPK_CASE(16)
        default:
            return hipErrorInvalidValue;
    }
#undef MOE_TOPK_CASE
    return hipGetLastError();
}

}  // namespace moe
