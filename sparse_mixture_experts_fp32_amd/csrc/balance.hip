// Load-balancing statistics of the router.
//
// Auxiliary loss ("Kimi K3: The Open Model That Just Cornered the AI Frontier",
// section "Mixture-of-Experts with Dynamic Load Balancing"): each expert's
// softmax probability averaged over the batch, and the sum over experts of its
// squared distance from 1/E.
//
// Quantile Balancing ("Kimi K3: Open Frontier Intelligence", section "Systems
// Optimization, Load Balancing, and Post-Training Alignment"): top-(k+1)
// routing on biased scores gives every token a cutoff alpha (its (k+1)-th
// biased score); the margins s - alpha of every (token, expert) pair are
// counted in a per-expert histogram; the (1 - k/E)-quantile of each row,
// read off the histogram, gives the expert's next bias -Q.
//
// Every integer here (ids, bins, counts) is decided in float32 on float32
// data; counts are merged with integer adds, whose order cannot change the
// sum, and the float sums run in a fixed order, so every result is
// deterministic.
#include <algorithm>

#include "device_common.h"
#include "launch.h"
#include "select.h"

namespace moe {

// ------------------------------------------------------------ QB selection
//
// One wavefront per token, as in the plain top-k: 64-bit keys (ordered float
// bits of s + b, then ~id), the k + 1 largest selected by select_top. Lanes
// 0..k-1 end with the chosen ids in slot order and lane k with the cutoff. The weights
// use the unbiased logits of the chosen experts: exp(s_j - M) / sum_i exp(s_i - M),
// M their maximum (the softmax denominator over all E cancels).

template <int NPER>
__global__ __launch_bounds__(256) void qb_select_kernel(const float* __restrict__ logits,
                                                        const float* __restrict__ bias, int64_t T, int E, int k,
                                                        int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                                        float* __restrict__ alpha) {
    __shared__ uint64_t sel[4][kSelectLds];
    const int lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wavefront
    const float* row = logits + t * E;

    float v[NPER], b[NPER];
    load_row_strided<NPER>(row, E, 0.f, v);
    load_row_strided<NPER>(bias, E, 0.f, b);
    float sc[NPER];
#pragma unroll
    for (int i = 0; i < NPER; ++i) sc[i] = v[i] + b[i];
    // lane j <= k: the j-th largest biased key (lane k: the cutoff)
    const uint64_t best = select_top<NPER>(sc, E, k + 1, sel[threadIdx.x >> 6]);
    const int my_id = static_cast<int>(0xffffffffu - static_cast<uint32_t>(best));
    const float my_score = key_value(static_cast<uint32_t>(best >> 32));
    const bool chosen = lane < k;
    // my_id < E always: k + 1 <= E valid keys exist and padding keys are 0
    const float s = chosen ? row[my_id] : -INFINITY;
    const float top = wave_max_f32(s);
    const float ex = chosen ? expf(s - top) : 0.f;
    const float sum = wave_sum_f32(ex);
    if (chosen) {
        topk_idx[t * k + lane] = my_id;
        topk_w[t * k + lane] = ex / sum;
    }
    if (lane == k) alpha[t] = my_score;
}

// ------------------------------------------------------------ QB histogram
//
// Block = a slab of SE consecutive experts x a contiguous token range. Thread
// (row, col) reads logits[t, slab * SE + col] for tokens t = row, row + R, ...
// (R = threads / SE): every token contributes a 4 * SE-byte contiguous segment.
// Counts go to a private LDS histogram [SE][n_bins] with LDS integer adds, then
// its non-zero bins are added to the global histogram with integer atomics
// (the global histogram is cleared first, by a fill kernel).

constexpr int kHistThreads = 512;
constexpr int kHistUnroll = 8;
constexpr int kHistLdsBytes = 128 * 1024;
constexpr int kHistMaxBins = 4096;
static_assert(kHistMaxBins * 8 * sizeof(int32_t) <= kHistLdsBytes, "8 experts of the widest histogram fit in LDS");

__device__ __forceinline__ int qb_bin(float s, float a, float lo, float width, int n_bins) {
    const float m = s - a;            // margin, rounded once
    const float u = (m - lo) / width; // correctly rounded float32 division
    if (!(u >= 0.f)) return 0;        // below the range, or NaN
    if (u >= static_cast<float>(n_bins)) return n_bins - 1;
    return min(static_cast<int>(u), n_bins - 1);
}

template <int SE>
__global__ __launch_bounds__(kHistThreads) void qb_hist_kernel(const float* __restrict__ logits,
                                                               const float* __restrict__ alpha, int64_t T, int E,
                                                               float lo, float width, int n_bins, int nslab,
                                                               int64_t tok_per_block, int32_t* __restrict__ hist) {
    __shared__ int32_t sh[kHistLdsBytes / sizeof(int32_t)];  // [SE][n_bins], SE * n_bins <= its size
    constexpr int R = kHistThreads / SE;
    const int slab = blockIdx.x % nslab;
    const int64_t split = blockIdx.x / nslab;
    for (int i = threadIdx.x; i < SE * n_bins; i += kHistThreads) sh[i] = 0;
    __syncthreads();

    const int col = threadIdx.x % SE, row = threadIdx.x / SE;
    const int e = slab * SE + col;
    const bool on = e < E;
    const int64_t t0 = split * tok_per_block;
    const int64_t t1 = min(t0 + tok_per_block, T);
    int32_t* my = sh + col * n_bins;
    for (int64_t tb = t0 + row; tb < t1; tb += static_cast<int64_t>(R) * kHistUnroll) {
        float v[kHistUnroll], a[kHistUnroll];
#pragma unroll
        for (int u = 0; u < kHistUnroll; ++u) {  // all loads first
            const int64_t t = tb + static_cast<int64_t>(u) * R;
            const bool ok = on && t < t1;
            v[u] = ok ? logits[t * E + e] : 0.f;
            a[u] = ok ? alpha[t] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kHistUnroll; ++u) {
            const int64_t t = tb + static_cast<int64_t>(u) * R;
            if (on && t < t1) atomicAdd(my + qb_bin(v[u], a[u], lo, width, n_bins), 1);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < SE * n_bins; i += kHistThreads) {
        const int c = sh[i];
        const int ee = slab * SE + i / n_bins;
        if (c != 0 && ee < E) atomicAdd(hist + static_cast<int64_t>(ee) * n_bins + (i % n_bins), c);
    }
}

// --------------------------------------------------------------- QB update
//
// One wavefront per expert. Lane l sums bins [l*c, (l+1)*c) of the row
// (c = ceil(n_bins / 64)); a wavefront scan of those sums finds the lane where
// the cumulative count first reaches p*m, p = 1 - k/E (compared exactly, as
// C * E >= m * (E - k) in 64-bit integers); that lane walks its bins to the
// crossing bin b and evaluates Q = lo + width * (b + (p*m - C_{b-1}) / H_b) in
// float64 rounding after every operation (no fused multiply-add), then
// stores -Q. A row with no counts keeps its bias.

__global__ __launch_bounds__(256) void qb_update_kernel(const int32_t* __restrict__ hist, int E, int k, int n_bins,
                                                        float lo, float width, const float* bias_in,
                                                        float* bias_out) {
#pragma clang fp contract(off)  // Q rounds after each operation, as written
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    const int32_t* row = hist + static_cast<int64_t>(e) * n_bins;
    const int c = (n_bins + 63) / 64;
    const int b0 = min(lane * c, n_bins), b1 = min(b0 + c, n_bins);
    int64_t s = 0;
    for (int b = b0; b < b1; ++b) s += row[b];
    int64_t incl = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t v = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += v;
    }
    const int64_t m = __shfl(incl, 63, kWave);
    if (m <= 0) {
        if (lane == 0) bias_out[e] = bias_in[e];
        return;
    }
    const int64_t need = m * (E - k);
    const uint64_t hit = __ballot(incl * E >= need);  // lane 63 always hits
    const int L = __ffsll(static_cast<unsigned long long>(hit)) - 1;
    if (lane != L) return;
    int64_t cum = incl - s;
    for (int b = b0; b < b1; ++b) {
        const int64_t hb = row[b];
        if ((cum + hb) * E >= need) {
            const double frac = static_cast<double>(need - cum * E) / static_cast<double>(E * hb);
            const double q = static_cast<double>(lo) + static_cast<double>(width) * (static_cast<double>(b) + frac);
            bias_out[e] = static_cast<float>(-q);
            return;
        }
        cum += hb;
    }
}

// ---------------------------------------------------------------- aux loss
//
// Pass 1: block g owns tokens [64 g, 64 g + 64); wave w takes tokens w, w + 4,
// ... of them in order, computes each token's softmax (wavefront max and sum)
// and adds the probabilities to per-lane float32 column sums; the 4 waves are
// added in wave order, giving partial[g][e].
// Pass 2: block b owns columns [64 b, 64 b + 64); wave w sums a contiguous run
// of the partial rows in float64, in order; the 16 runs are added in order;
// mean[e] = total / T.
// Pass 3: one block: sum_e (mean_e - 1/E)^2 in float64 by a fixed tree.

constexpr int kAuxTokens = 64;

template <int NPER>
__global__ __launch_bounds__(256) void aux_partial_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                          float* __restrict__ partial) {
    __shared__ float red[4][NPER * 64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    float acc[NPER];
#pragma unroll
    for (int i = 0; i < NPER; ++i) acc[i] = 0.f;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kAuxTokens;
    for (int r = w; r < kAuxTokens; r += 4) {
        const int64_t t = t0 + r;
        if (t >= T) break;  // whole wavefront
        const float* row = logits + t * E;
        float v[NPER];
        load_row_strided<NPER>(row, E, -INFINITY, v);
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < NPER; ++i) mx = fmaxf(mx, v[i]);
        mx = wave_max_f32(mx);
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < NPER; ++i) {
            const int e = lane + 64 * i;
            v[i] = e < E ? expf(v[i] - mx) : 0.f;
            s += v[i];
        }
        s = wave_sum_f32(s);
        const float inv = 1.0f / s;  // one division per token, then a fused multiply-add per expert
#pragma unroll
        for (int i = 0; i < NPER; ++i) acc[i] = fmaf(v[i], inv, acc[i]);
    }
#pragma unroll
    for (int i = 0; i < NPER; ++i) red[w][i * 64 + lane] = acc[i];
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256)
        partial[blockIdx.x * static_cast<int64_t>(E) + e] = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
}

__global__ __launch_bounds__(1024) void aux_colsum_kernel(const float* __restrict__ partial, int64_t G, int E,
                                                          int64_t T, double* __restrict__ mean64,
                                                          float* __restrict__ prob_mean) {
    __shared__ double red[16][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + lane;
    const int64_t per = (G + 15) / 16;
    const int64_t g0 = min(w * per, G), g1 = min(g0 + per, G);
    double s = 0.0;
    if (e < E)
        for (int64_t g = g0; g < g1; ++g) s += static_cast<double>(partial[g * E + e]);
    red[w][lane] = s;
    __syncthreads();
    if (w == 0 && e < E) {
        double tot = 0.0;
#pragma unroll
        for (int v = 0; v < 16; ++v) tot += red[v][lane];
        const double m = tot / static_cast<double>(T);
        mean64[e] = m;
        prob_mean[e] = static_cast<float>(m);
    }
}

__global__ __launch_bounds__(1024) void aux_loss_kernel(const double* __restrict__ mean64, int E,
                                                        float* __restrict__ aux_loss) {
#pragma clang fp contract(off)
    __shared__ double red[1024];
    const int tid = threadIdx.x;
    double v = 0.0;
    if (tid < E) {
        const double dlt = mean64[tid] - 1.0 / static_cast<double>(E);
        v = dlt * dlt;
    }
    red[tid] = v;
    __syncthreads();
    for (int off = 512; off > 0; off >>= 1) {
        if (tid < off) red[tid] += red[tid + off];
        __syncthreads();
    }
    if (tid == 0) aux_loss[0] = static_cast<float>(red[0]);
}

// ---------------------------------------------------------------- launchers

#define MOE_NPER_SWITCH(nper, CASE)                                   \
    switch (nper) {                                                   \
        CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8) \
        CASE(9) CASE(10) CASE(11) CASE(12) CASE(13) CASE(14) CASE(15) CASE(16) \
        default: return hipErrorInvalidValue;                          \
    }

hipError_t launch_qb_select(const float* logits, const float* bias, int64_t T, int E, int k, int32_t* topk_idx,
                            float* topk_w, float* alpha, hipStream_t stream) {
    dim3 grid(static_cast<unsigned>((T + 3) / 4));
#define MOE_QB_CASE(N)                                                                                        \
    case N:                                                                                                   \
        hipLaunchKernelGGL(qb_select_kernel<N>, grid, dim3(256), 0, stream, logits, bias, T, E, k, topk_idx, \
                           topk_w, alpha);                                                                    \
        break;
    MOE_NPER_SWITCH((E + 63) / 64, MOE_QB_CASE)
#undef MOE_QB_CASE
    return hipGetLastError();
}

int qb_max_bins() { return kHistMaxBins; }

hipError_t launch_qb_histogram(const float* logits, const float* alpha, int64_t T, int E, float lo, float width,
                               int n_bins, int32_t* hist, hipStream_t stream) {
    hipError_t err = launch_zero_i32(hist, E * n_bins, stream);
    if (err != hipSuccess || T == 0) return err;
    // experts per block: as many as the LDS histogram holds (n_bins <= kHistMaxBins)
    constexpr int kLdsInts = kHistLdsBytes / sizeof(int32_t);
    const int se = n_bins * 32 <= kLdsInts ? 32 : (n_bins * 16 <= kLdsInts ? 16 : 8);
    const int nslab = (E + se - 1) / se;
    // one block per compute unit (its LDS histogram fills most of the CU's LDS), at least 64 tokens each:
    // every block ends by adding its non-zero bins to the global histogram with atomics, so fewer,
    // larger token ranges flush fewer bins
    const int64_t want = std::max<int64_t>(1, 256 / nslab);
    const int64_t splits = std::max<int64_t>(1, std::min<int64_t>(want, (T + 63) / 64));
    const int64_t per = (T + splits - 1) / splits;
    const int64_t nblk = static_cast<int64_t>(nslab) * ((T + per - 1) / per);
#define MOE_HIST(SE)                                                                                              \
    hipLaunchKernelGGL(qb_hist_kernel<SE>, dim3(static_cast<unsigned>(nblk)), dim3(kHistThreads), 0, stream,    \
                       logits, alpha, T, E, lo, width, n_bins, nslab, per, hist)
    if (se == 32) {
        MOE_HIST(32);
    } else if (se == 16) {
        MOE_HIST(16);
    } else {
        MOE_HIST(8);
    }
#undef MOE_HIST
    return hipGetLastError();
}

hipError_t launch_qb_update(const int32_t* hist, int E, int k, int n_bins, float lo, float width,
                            const float* bias_in, float* bias_out, hipStream_t stream) {
    hipLaunchKernelGGL(qb_update_kernel, dim3((E + 3) / 4), dim3(256), 0, stream, hist, E, k, n_bins, lo, width,
                       bias_in, bias_out);
    return hipGetLastError();
}

size_t aux_ws_bytes(int64_t T, int E) {
    const int64_t G = (T + kAuxTokens - 1) / kAuxTokens;
    const size_t part = (sizeof(float) * static_cast<size_t>(G) * E + 255) / 256 * 256;
    return part + sizeof(double) * static_cast<size_t>(E);
}

hipError_t launch_aux_loss(const float* logits, int64_t T, int E, float* prob_mean, float* aux_loss, void* ws,
                           hipStream_t stream) {
    const int64_t G = (T + kAuxTokens - 1) / kAuxTokens;
    float* partial = static_cast<float*>(ws);
    const size_t part = (sizeof(float) * static_cast<size_t>(G) * E + 255) / 256 * 256;
    double* mean64 = reinterpret_cast<double*>(static_cast<char*>(ws) + part);
#define MOE_AUX_CASE(N)                                                                                     \
    case N:                                                                                                 \
        hipLaunchKernelGGL(aux_partial_kernel<N>, dim3(static_cast<unsigned>(G)), dim3(256), 0, stream, logits, \
                           T, E, partial);                                                                  \
        break;
    MOE_NPER_SWITCH((E + 63) / 64, MOE_AUX_CASE)
#undef MOE_AUX_CASE
    hipLaunchKernelGGL(aux_colsum_kernel, dim3((E + 63) / 64), dim3(1024), 0, stream, partial, G, E, T, mean64,
                       prob_mean);
    hipLaunchKernelGGL(aux_loss_kernel, dim3(1), dim3(1024), 0, stream, mean64, E, aux_loss);
    return hipGetLastError();
}

#undef MOE_NPER_SWITCH

}  // namespace moe
