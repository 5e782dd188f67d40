// Weighted combine: out[t] = sum_{j<k} w[t, j] * Y[row_of[t, j]] ("Kimi K3: Open
// Frontier Intelligence", section "Operational Execution Flow": a token's routed
// output is the probability-weighted sum of its experts' outputs).
//
// A gather, not a scatter: one wavefront owns one token's output row and reads
// its k expert rows, so no two wavefronts write the same address and there are
// no atomics; the float32 sum runs in slot order j = 0..k-1, which makes the
// result bitwise repeatable.
#include "device_common.h"
#include "launch.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Y, int d,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ w, int64_t T, int k,
                                                      int64_t n_rows, float* __restrict__ out) {
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
    const int nchunk = d / 4;  // float4 chunks per row
    // the chunk loop is uniform across the wavefront so that every lane takes
    // part in the slot broadcasts; lanes past the row end only skip the memory ops
    for (int c0 = 0; c0 < nchunk; c0 += 64) {
        const int c = c0 + lane;
        const bool on = c < nchunk;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = 0; j < k; ++j) {
            const int r = __shfl(my_row, j, 64);
            const float wj = __shfl(my_w, j, 64);
            if (r < 0 || !on) continue;
            const float4 v = *reinterpret_cast<const float4*>(Y + static_cast<int64_t>(r) * d + 4 * c);
            acc.x = fmaf(wj, v.x, acc.x);
            acc.y = fmaf(wj, v.y, acc.y);
            acc.z = fmaf(wj, v.z, acc.z);
            acc.w = fmaf(wj, v.w, acc.w);
        }
        if (on) *reinterpret_cast<float4*>(out + t * d + 4 * c) = acc;
    }
}

hipError_t launch_combine(const float* y_rows, const int32_t* row_of, const float* topk_w, int64_t T,
                          int d, int k, int64_t n_rows, float* out, hipStream_t stream) {
    hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>((T + 3) / 4)), dim3(256), 0, stream, y_rows,
                       d, row_of, topk_w, T, k, n_rows, out);
    return hipGetLastError();
}

}  // namespace moe
