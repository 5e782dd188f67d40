// Routing: gate logits (a dense contraction on the matrix cores) and the
// per-token softmax / top-k / renormalisation (one wavefront per token).
//
// Gate, softmax and top-k: "Kimi K3: The Open Model That Just Cornered the AI
// Frontier", section "Mixture-of-Experts with Dynamic Load Balancing".
#include "device_common.h"
#include "launch.h"
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
// on the bf16 matrix cores.
//
// Tile: 64 tokens x 64 experts per 256-thread workgroup, K step 64, the token
// rows and the three weight parts staged in LDS (double-buffered); wave
// (wm, wn) owns a 32 x 32 quarter as 2 x 2 blocks of 16 x 16.

constexpr int kRBM = 64, kRBN = 64, kRBK = 64;
constexpr int kRStride = kRBK + 16;  // bf16 per LDS row (32 B of padding: conflict-free 16-B reads)

// w [E, d] float32 -> parts [3][E][d] bf16 with w = parts[0] + parts[1] + parts[2] exactly.
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ w, int64_t n,
                                                           uint16_t* __restrict__ parts) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const float v = w[i];
        const uint16_t h = f32_to_bf16_bits(v);
        const float r1 = v - bf16_bits_to_f32(h);
        const uint16_t m = f32_to_bf16_bits(r1);
        const float r2 = r1 - bf16_bits_to_f32(m);
        parts[i] = h;
        parts[n + i] = m;
        parts[2 * n + i] = f32_to_bf16_bits(r2);
    }
}

__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ parts,
                                                          const float* __restrict__ bias,
                                                          float* __restrict__ logits, int64_t T, int d, int E) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][kRBM * kRStride];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][3][kRBN * kRStride];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * kRBN;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kRBM;
    const int64_t pn = static_cast<int64_t>(E) * d;  // elements per weight part

    // global -> register staging: 512 16-byte chunks per 64 x 64 tile, two per
    // thread (rows tid / 8 and tid / 8 + 32, chunk tid % 8); rows past the
    // matrix end re-read its last row (results never stored)
    const int ld_row = tid >> 3, ld_col = 8 * (tid & 7);
    int64_t a_off[2], b_off[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        a_off[p] = min(m0 + ld_row + 32 * p, T - 1) * d + ld_col;
        b_off[p] = static_cast<int64_t>(min(n0 + ld_row + 32 * p, E - 1)) * d + ld_col;
    }
    u32x4 a_reg[2], b_reg[3][2];
    auto load_tile = [&](int k0) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            a_reg[p] = *reinterpret_cast<const u32x4*>(x + a_off[p] + k0);
#pragma unroll
            for (int q = 0; q < 3; ++q) b_reg[q][p] = *reinterpret_cast<const u32x4*>(parts + q * pn + b_off[p] + k0);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int off = (ld_row + 32 * p) * kRStride + ld_col;
            *reinterpret_cast<u32x4*>(&sA[buf][off]) = a_reg[p];
#pragma unroll
            for (int q = 0; q < 3; ++q) *reinterpret_cast<u32x4*>(&sB[buf][q][off]) = b_reg[q][p];
        }
    };

    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int frag_row = lane & 15, frag_k = 8 * (lane >> 4);
    const int nk = d / kRBK;
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int step = 0; step < nk; ++step) {
        const int cur = step & 1;
        if (step + 1 < nk) load_tile((step + 1) * kRBK);
#pragma unroll
        for (int s = 0; s < kRBK / 32; ++s) {
            bf16x8 a[2], b[3][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const bf16x8*>(&sA[cur][(wm * 32 + i * 16 + frag_row) * kRStride + s * 32 + frag_k]);
#pragma unroll
            for (int q = 0; q < 3; ++q)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    b[q][j] = *reinterpret_cast<const bf16x8*>(
                        &sB[cur][q][(wn * 32 + j * 16 + frag_row) * kRStride + s * 32 + frag_k]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    acc[i][j] = mfma_16x16x32(a[i], b[2][j], acc[i][j]);  // smallest part first
                    acc[i][j] = mfma_16x16x32(a[i], b[1][j], acc[i][j]);
                    acc[i][j] = mfma_16x16x32(a[i], b[0][j], acc[i][j]);
                }
        }
        if (step + 1 < nk) store_tile(cur ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn * 32 + j * 16 + (lane & 15);
        if (col >= E) continue;
        const float bcol = bias ? bias[col] : 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t row = m0 + wm * 32 + i * 16 + 4 * (lane >> 4) + q;
                if (row < T) logits[row * E + col] = acc[i][j][q] + bcol;
            }
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

    uint64_t key[NPER];
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
        const int e = lane + 64 * i;
        key[i] = (e < E) ? ((static_cast<uint64_t>(order_key(row[e])) << 32) | (0xffffffffu - static_cast<uint32_t>(e)))
                         : 0ull;
    }
    // lane j < k: the j-th largest key
    const uint64_t best = select_top<NPER>(key, k, sel[threadIdx.x >> 6]);
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

size_t router_parts_bytes(int d, int E) { return sizeof(uint16_t) * 3 * static_cast<size_t>(E) * d; }

hipError_t launch_router_gemm(const uint16_t* x, const float* w, const float* bias, float* logits, int64_t T, int d,
                              int E, uint16_t* parts, hipStream_t stream) {
    const int64_t n = static_cast<int64_t>(E) * d;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(router_split_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, w, n, parts);
    dim3 grid((E + kRBN - 1) / kRBN, static_cast<unsigned>((T + kRBM - 1) / kRBM));
    hipLaunchKernelGGL(router_gemm_kernel, grid, dim3(256), 0, stream, x, parts, bias, logits, T, d, E);
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
