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
// One workgroup of four wavefronts per token. Thread i owns the float4 chunks
// c = i, i + 256, ... of the latent row (NCT of them): it forms
// u = sum_{j<k} w[t, j] * Y[row_of[t, j]] in slot order (as moe_combine does, so
// u is bitwise moe_combine's row), issuing the loads of kSl slots before their
// multiply-adds (Y rows are read once, so non-temporally). The sum of u^2 runs
// over each thread's chunks in order, a wavefront butterfly, then the four
// wavefront sums in order (the same value in every thread); the kernel writes
// bf16(u * (1 / sqrt(mean u^2 + eps)) * g), and u itself when u_out is given.

template <int NCT, int kSl>
__global__ __launch_bounds__(256) void combine_rmsnorm_kernel(const float* __restrict__ Y, int l,
                                                              const int32_t* __restrict__ row_of,
                                                              const float* __restrict__ w, int64_t T, int k,
                                                              int64_t n_rows, const float* __restrict__ gain,
                                                              float eps, float* __restrict__ u_out,
                                                              uint16_t* __restrict__ r_out) {
    __shared__ float wave_ss[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t = blockIdx.x;
    if (t >= T) return;  // whole workgroup
    int my_row = -1;
    float my_w = 0.f;
    if (lane < k) {
        my_row = row_of[t * k + lane];
        my_w = w[t * k + lane];
        if (my_row < 0 || my_row >= n_rows) my_row = -1;
    }
    const int nchunk = l / 4;
    f32x4 u[NCT];
#pragma unroll
    for (int i = 0; i < NCT; ++i) u[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < k; j0 += kSl) {
        f32x4 v[kSl][NCT];
        float wj[kSl];
#pragma unroll
        for (int s = 0; s < kSl; ++s) {  // all loads of this group first
            const int j = j0 + s;
            const int r = __shfl(my_row, j & 63, kWave);
            wj[s] = __shfl(my_w, j & 63, kWave);
            const bool on = j < k && r >= 0;
            const f32x4* yrow = reinterpret_cast<const f32x4*>(Y + static_cast<int64_t>(on ? r : 0) * l);
#pragma unroll
            for (int i = 0; i < NCT; ++i) {
                const int c = tid + 256 * i;
                v[s][i] = (on && c < nchunk) ? __builtin_nontemporal_load(yrow + c) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
            if (!on) wj[s] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < kSl; ++s) {  // then the sums, in slot order
            if (j0 + s >= k) break;      // uniform
            const int r = __shfl(my_row, (j0 + s) & 63, kWave);
            if (r < 0) continue;         // uniform: a skipped slot adds nothing
#pragma unroll
            for (int i = 0; i < NCT; ++i) {
                u[i].x = fmaf(wj[s], v[s][i].x, u[i].x);
                u[i].y = fmaf(wj[s], v[s][i].y, u[i].y);
                u[i].z = fmaf(wj[s], v[s][i].z, u[i].z);
                u[i].w = fmaf(wj[s], v[s][i].w, u[i].w);
            }
        }
    }
    float ss = 0.f;  // chunks past the row end hold zeros
#pragma unroll
    for (int i = 0; i < NCT; ++i) {
        ss = fmaf(u[i].x, u[i].x, ss);
        ss = fmaf(u[i].y, u[i].y, ss);
        ss = fmaf(u[i].z, u[i].z, ss);
        ss = fmaf(u[i].w, u[i].w, ss);
    }
    ss = wave_sum_f32(ss);
    if (lane == 0) wave_ss[wave] = ss;
    __syncthreads();
    const float total = ((wave_ss[0] + wave_ss[1]) + wave_ss[2]) + wave_ss[3];
    const float rs = 1.0f / sqrtf(total / static_cast<float>(l) + eps);
    const f32x4* g4 = reinterpret_cast<const f32x4*>(gain);
#pragma unroll
    for (int i = 0; i < NCT; ++i) {
        const int c = tid + 256 * i;
        if (c >= nchunk) continue;
        const f32x4 g = g4[c];
        if (u_out != nullptr) reinterpret_cast<f32x4*>(u_out + t * l)[c] = u[i];
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
    if (T <= 0) return hipSuccess;
    const int nct = (l / 4 + 255) / 256;  // float4 chunks per thread
    dim3 grid(static_cast<unsigned>(T));
#define MOE_CR(N, S)                                                                                               \
    hipLaunchKernelGGL((combine_rmsnorm_kernel<N, S>), grid, dim3(256), 0, stream, y_rows, l, row_of, topk_w, T, k, \
                       n_rows, gain, eps, u_out, r_out)
    if (nct <= 1) {
        MOE_CR(1, 8);
    } else if (nct <= 2) {
        MOE_CR(2, 4);
    } else if (nct <= 4) {
        MOE_CR(4, 4);
    } else if (nct <= 8) {
        MOE_CR(8, 2);
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
