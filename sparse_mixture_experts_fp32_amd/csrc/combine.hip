// Weighted combine: out[t] = sum_{j<k} w[t, j] * Y[row_of[t, j]] ("Kimi K3: Open
// Frontier Intelligence", section "Operational Execution Flow": a token's routed
// output is the probability-weighted sum of its experts' outputs).
//
// A gather, not a scatter: one wavefront owns one token's output row and reads
// its k expert rows, so no two wavefronts write the same address and there are
// no atomics; the float32 sum runs in slot order j = 0..k-1, which makes the
// result bitwise repeatable.
//
// Bandwidth: a lane owns float4 chunks c and c + 64 of the row at a time and
// issues the loads of up to kSlots slots for both before the first multiply-add,
// so a wavefront keeps 2 * kSlots * 1 KiB in flight instead of one load per
// lane; the sum order per element is unchanged.
#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kSlots = 8;   // slots whose loads are issued together
constexpr int kChunks = 2;  // float4 chunks per lane per pass

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
    for (int c0 = 0; c0 < nchunk; c0 += 64 * kChunks) {
        float4 acc[kChunks];
#pragma unroll
        for (int u = 0; u < kChunks; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j0 = 0; j0 < k; j0 += kSlots) {
            float4 v[kSlots][kChunks];
            float wj[kSlots];
#pragma unroll
            for (int s = 0; s < kSlots; ++s) {  // all loads of this group first
                const int j = j0 + s;
                const int r = __shfl(my_row, j & 63, 64);
                wj[s] = __shfl(my_w, j & 63, 64);
                const bool row_on = j < k && r >= 0;
#pragma unroll
                for (int u = 0; u < kChunks; ++u) {
                    const int c = c0 + 64 * u + lane;
                    v[s][u] = (row_on && c < nchunk)
                                  ? *reinterpret_cast<const float4*>(Y + static_cast<int64_t>(r) * d + 4 * c)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
                }
                if (!row_on) wj[s] = 0.f;
            }
#pragma unroll
            for (int s = 0; s < kSlots; ++s) {  // then the sums, in slot order
                if (j0 + s >= k) break;         // uniform
                const int r = __shfl(my_row, (j0 + s) & 63, 64);
                if (r < 0) continue;            // uniform: a skipped slot adds nothing
#pragma unroll
                for (int u = 0; u < kChunks; ++u) {
                    acc[u].x = fmaf(wj[s], v[s][u].x, acc[u].x);
                    acc[u].y = fmaf(wj[s], v[s][u].y, acc[u].y);
                    acc[u].z = fmaf(wj[s], v[s][u].z, acc[u].z);
                    acc[u].w = fmaf(wj[s], v[s][u].w, acc[u].w);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kChunks; ++u) {
            const int c = c0 + 64 * u + lane;
            if (c < nchunk) *reinterpret_cast<float4*>(out + t * d + 4 * c) = acc[u];
        }
    }
}

hipError_t launch_combine(const float* y_rows, const int32_t* row_of, const float* topk_w, int64_t T,
                          int d, int k, int64_t n_rows, float* out, hipStream_t stream) {
    hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>((T + 3) / 4)), dim3(256), 0, stream, y_rows,
                       d, row_of, topk_w, T, k, n_rows, out);
    return hipGetLastError();
}

}  // namespace moe
