// The pieces of the Stable LatentMoE layer that are not grouped GEMMs
// ("Kimi K3: Open Frontier Intelligence", section "Operational Execution
// Flow"): the routed sum u followed by an explicit RMSNorm, the row maps that
// let the grouped GEMM run the dense projections and the shared experts, and
// the final sum of the up-projected routed branch and the shared experts.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace moe {

// ----------------------------------------------------- combine + RMSNorm
//
// One wavefront per token. Lane l owns the float4 chunks c = l, l + 64, ... of
// the latent row (NC of them, kept in registers): it forms
// u = sum_{j<k} w[t, j] * Y[row_of[t, j]] in slot order (as moe_combine does),
// then the wavefront sums u^2 (each lane over its chunks in order, then a
// butterfly), and writes bf16(u * (1 / sqrt(mean u^2 + eps)) * g). u itself is
// written as well when u_out is given.

template <int NC>
__global__ __launch_bounds__(256) void combine_rmsnorm_kernel(const float* __restrict__ Y, int l,
                                                              const int32_t* __restrict__ row_of,
                                                              const float* __restrict__ w, int64_t T, int k,
                                                              int64_t n_rows, const float* __restrict__ gain,
                                                              float eps, float* __restrict__ u_out,
                                                              uint16_t* __restrict__ r_out) {
    const int lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wavefront
    int my_row = -1;
    float my_w = 0.f;
    if (lane < k) {
        my_row = row_of[t * k + lane];
        my_w = w[t * k + lane];
        if (my_row < 0 || my_row >= n_rows) my_row = -1;
    }
    const int nchunk = l / 4;
    float4 u[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) u[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        const int r = __shfl(my_row, j, 64);
        const float wj = __shfl(my_w, j, 64);
        if (r < 0) continue;  // uniform
        const float4* yrow = reinterpret_cast<const float4*>(Y + static_cast<int64_t>(r) * l);
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = lane + 64 * i;
            if (c < nchunk) {
                const float4 v = yrow[c];
                u[i].x = fmaf(wj, v.x, u[i].x);
                u[i].y = fmaf(wj, v.y, u[i].y);
                u[i].z = fmaf(wj, v.z, u[i].z);
                u[i].w = fmaf(wj, v.w, u[i].w);
            }
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        ss = fmaf(u[i].x, u[i].x, ss);
        ss = fmaf(u[i].y, u[i].y, ss);
        ss = fmaf(u[i].z, u[i].z, ss);
        ss = fmaf(u[i].w, u[i].w, ss);
    }
    ss = wave_sum_f32(ss);
    const float rs = 1.0f / sqrtf(ss / static_cast<float>(l) + eps);
    const float4* g4 = reinterpret_cast<const float4*>(gain);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = lane + 64 * i;
        if (c >= nchunk) continue;
        const float4 g = g4[c];
        if (u_out != nullptr) reinterpret_cast<float4*>(u_out + t * l)[c] = u[i];
        const uint32_t lo = f32_to_bf16_bits(u[i].x * rs * g.x) | (uint32_t(f32_to_bf16_bits(u[i].y * rs * g.y)) << 16);
        const uint32_t hi = f32_to_bf16_bits(u[i].z * rs * g.z) | (uint32_t(f32_to_bf16_bits(u[i].w * rs * g.w)) << 16);
        reinterpret_cast<uint2*>(r_out + t * l)[c] = make_uint2(lo, hi);
    }
}

// ------------------------------------------------------------- row maps
//
// The dense projections are grouped GEMMs with one "expert" holding all T rows;
// the S shared experts are grouped GEMMs whose expert s holds rows
// s*T .. s*T + T - 1, all read from x through the row map rows[r] = r mod T.

__global__ void latent_maps_kernel(int64_t T, int S, int32_t* __restrict__ dense_off,
                                   int32_t* __restrict__ shared_off, int32_t* __restrict__ shared_rows) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < 2) dense_off[i] = static_cast<int32_t>(i * T);
    if (i <= S) shared_off[i] = static_cast<int32_t>(i * T);
    if (i < S * T) shared_rows[i] = static_cast<int32_t>(i % T);
}

// ------------------------------------------------------------ final sum
//
// out[t] += sum_s Ys[s*T + t], s in order (out already holds the up-projected
// routed branch), float4 per thread.

__global__ __launch_bounds__(256) void add_shared_kernel(float* __restrict__ out, const float* __restrict__ ys,
                                                         int64_t T, int d, int S) {
    const int64_t n4 = T * d / 4;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 acc = reinterpret_cast<float4*>(out)[i];
        for (int s = 0; s < S; ++s) {
            const float4 v = reinterpret_cast<const float4*>(ys)[s * n4 + i];
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        reinterpret_cast<float4*>(out)[i] = acc;
    }
}

// ---------------------------------------------------------------- launchers

int combine_rmsnorm_max_width() { return 64 * 4 * 32; }

hipError_t launch_combine_rmsnorm(const float* y_rows, const int32_t* row_of, const float* topk_w, int64_t T, int l,
                                  int k, int64_t n_rows, const float* gain, float eps, float* u_out,
                                  uint16_t* r_out, hipStream_t stream) {
    const int nc = (l / 4 + 63) / 64;
    dim3 grid(static_cast<unsigned>((T + 3) / 4));
#define MOE_CR(N)                                                                                               \
    hipLaunchKernelGGL(combine_rmsnorm_kernel<N>, grid, dim3(256), 0, stream, y_rows, l, row_of, topk_w, T, k, \
                       n_rows, gain, eps, u_out, r_out)
    if (nc <= 2) {
        MOE_CR(2);
    } else if (nc <= 4) {
        MOE_CR(4);
    } else if (nc <= 8) {
        MOE_CR(8);
    } else if (nc <= 14) {
        MOE_CR(14);
    } else if (nc <= 16) {
        MOE_CR(16);
    } else if (nc <= 24) {
        MOE_CR(24);
    } else if (nc <= 32) {
        MOE_CR(32);
    } else {
        return hipErrorInvalidValue;
    }
#undef MOE_CR
    return hipGetLastError();
}

hipError_t launch_latent_maps(int64_t T, int S, int32_t* dense_off, int32_t* shared_off, int32_t* shared_rows,
                              hipStream_t stream) {
    const int64_t n = std::max<int64_t>(S * T, S + 1);
    hipLaunchKernelGGL(latent_maps_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, T, S,
                       dense_off, shared_off, shared_rows);
    return hipGetLastError();
}

hipError_t launch_add_shared(float* out, const float* ys, int64_t T, int d, int S, hipStream_t stream) {
    const int64_t n4 = T * d / 4;
    const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 8192);
    hipLaunchKernelGGL(add_shared_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, out, ys, T, d, S);
    return hipGetLastError();
}

}  // namespace moe
