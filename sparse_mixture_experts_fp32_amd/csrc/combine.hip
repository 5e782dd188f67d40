// Weighted combine: out[t] = sum_{j<k} w[t, j] * Y[row_of[t, j]] ("Kimi K3: Open
// Frontier Intelligence", section "Operational Execution Flow": a token's routed
// output is the probability-weighted sum of its experts' outputs).
//
// A gather, not a scatter: one wavefront owns one 256-column block of one token's
// output row and reads that block of its k expert rows, so no two wavefronts write
// the same address and there are no atomics; the float32 sum runs in slot order
// j = 0..k-1, which makes the result bitwise repeatable.
//
// Bandwidth: each lane owns one float4 of the block; the loads of up to kSlots
// slots (8, or 16 for more than 8 slots) are issued before the first
// multiply-add (kSlots KiB in flight per wavefront). Y rows and out are touched once, so both go through non-temporal
// loads and stores that do not displace other data from the caches. Small work
// items (T * d / 256 of them) keep every CU busy to the end of the launch.
// Measured on MI355X (d = 7168): 5.8-6.0 TB/s at T = 8192, k = 4 and 5.7-6.0 TB/s
// at T = 16384, k = 16, where 8 slots at a time gave 5.5 TB/s (16 slots at k = 4:
// 5% slower); one wavefront per whole row gave 4.9 TB/s.
#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kBlockCols = 256; // float columns per work item (one float4 per lane)

// kSlots: slots whose loads are issued together (16 VGPR-heavy slots halve the occupancy, so they pay
// only when a token has more than 8 slots to fetch)
template <int kSlots>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Y, int d,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ w, int64_t T, int k,
                                                      int64_t n_rows, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int nblk = (d + kBlockCols - 1) / kBlockCols;
    const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int64_t t = item / nblk;
    if (t >= T) return;  // whole wavefront
    const int c = static_cast<int>(item - t * nblk) * (kBlockCols / 4) + lane;  // float4 index in the row
    const bool col_on = c < d / 4;
    int my_row = -1;
    float my_w = 0.f;
    if (lane < k) {
        my_row = row_of[t * k + lane];
        my_w = w[t * k + lane];
        if (my_row < 0 || my_row >= n_rows) my_row = -1;
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // the slot loop is uniform across the wavefront so that every lane takes part
    // in the slot broadcasts; lanes past the row end only skip the memory ops
    for (int j0 = 0; j0 < k; j0 += kSlots) {
        f32x4 v[kSlots];
        float wj[kSlots];
#pragma unroll
        for (int s = 0; s < kSlots; ++s) {  // all loads of this group first
            const int j = j0 + s;
            const int r = __shfl(my_row, j & 63, kWave);
            wj[s] = __shfl(my_w, j & 63, kWave);
            const bool row_on = j < k && r >= 0;
            v[s] = (row_on && col_on)
                       ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Y + static_cast<int64_t>(r) * d) + c)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
            if (!row_on) wj[s] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < kSlots; ++s) {  // then the sums, in slot order
            if (j0 + s >= k) break;         // uniform
            const int r = __shfl(my_row, (j0 + s) & 63, kWave);
            if (r < 0) continue;            // uniform: a skipped slot adds nothing
            acc.x = fmaf(wj[s], v[s].x, acc.x);
            acc.y = fmaf(wj[s], v[s].y, acc.y);
            acc.z = fmaf(wj[s], v[s].z, acc.z);
            acc.w = fmaf(wj[s], v[s].w, acc.w);
        }
    }
    if (col_on) __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(out + t * d) + c);
}

hipError_t launch_combine(const float* y_rows, const int32_t* row_of, const float* topk_w, int64_t T,
                          int d, int k, int64_t n_rows, float* out, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    const int64_t items = T * ((d + kBlockCols - 1) / kBlockCols);
    if ((items + 3) / 4 > INT32_MAX) return hipErrorInvalidValue;  // beyond one launch's grid
    const dim3 grid(static_cast<unsigned>((items + 3) / 4));
    if (k > 8)
        hipLaunchKernelGGL(combine_kernel<16>, grid, dim3(256), 0, stream, y_rows, d, row_of, topk_w, T, k, n_rows, out);
    else
        hipLaunchKernelGGL(combine_kernel<8>, grid, dim3(256), 0, stream, y_rows, d, row_of, topk_w, T, k, n_rows, out);
    return hipGetLastError();
}

}  // namespace moe
