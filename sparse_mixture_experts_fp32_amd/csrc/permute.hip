// Grouping the (token, slot) assignments by expert: per-chunk histograms, one
// prefix scan, then a stable rank within each chunk, and the row gather.
//
// The assignments a = t * k + j are cut into chunks of `chunk` consecutive
// indices. Rows of expert e are ordered by a, so the first row of chunk c
// inside expert e is
//     offsets[e] + sum_{c' < c} count[e, c'],
// i.e. an exclusive scan of count laid out expert-major, chunk-minor. Inside a
// chunk, one wavefront walks the assignments in order, 64 at a time, and ranks
// equal experts within the 64 lanes with ballots (no atomics on the order), so
// the permutation is exact and deterministic. Per-expert token counts never
// leave the device ("Kimi K3: Open Frontier Intelligence", section "Systems
// Optimization, Load Balancing, and Post-Training Alignment": waiting on dynamic
// counts on the host stalls the device).
#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kMaxExperts = 1024;

// count[e * nchunks + c] = number of assignments of chunk c that chose expert e.
__global__ __launch_bounds__(256) void expert_count_kernel(const int32_t* __restrict__ topk_idx,
                                                           int64_t n_assign, int E, int chunk,
                                                           int nchunks, int32_t* __restrict__ count) {
    __shared__ int32_t hist[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
    const int c = blockIdx.x;
    const int64_t lo = static_cast<int64_t>(c) * chunk;
    const int64_t hi = min(lo + chunk, n_assign);
    for (int64_t a = lo + threadIdx.x; a < hi; a += blockDim.x) {
        const int e = topk_idx[a];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);  // integer counts: order-independent
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) count[static_cast<int64_t>(e) * nchunks + c] = hist[e];
}

// In-place exclusive scan of count[0 .. E*nchunks) by one 1024-thread workgroup;
// also writes expert_offsets[e] = scanned value of (e, chunk 0) and the total.
__global__ __launch_bounds__(1024) void expert_scan_kernel(int32_t* __restrict__ count, int E, int nchunks,
                                                           int32_t* __restrict__ expert_offsets) {
    __shared__ int32_t part[1024];
    const int64_t n = static_cast<int64_t>(E) * nchunks;
    const int tid = threadIdx.x;
    const int64_t per = (n + 1023) / 1024;
    const int64_t lo = min(n, tid * per), hi = min(n, lo + per);
    int32_t s = 0;
    for (int64_t i = lo; i < hi; ++i) s += count[i];
    part[tid] = s;
    __syncthreads();
    // Hillis-Steele inclusive scan over the 1024 partial sums
    for (int off = 1; off < 1024; off <<= 1) {
        const int32_t v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int32_t run = part[tid] - s;  // exclusive prefix of this thread's segment
    for (int64_t i = lo; i < hi; ++i) {
        const int32_t v = count[i];
        count[i] = run;
        if (i % nchunks == 0) expert_offsets[i / nchunks] = run;
        run += v;
    }
    if (tid == 1023) expert_offsets[E] = part[1023];
}

// One wavefront per chunk: stable ranks, row_of and row_src.
__global__ __launch_bounds__(64) void expert_rank_kernel(const int32_t* __restrict__ topk_idx,
                                                         int64_t n_assign, int k, int E, int chunk,
                                                         int nchunks, const int32_t* __restrict__ base,
                                                         int32_t* __restrict__ row_of,
                                                         int32_t* __restrict__ row_src) {
    __shared__ int32_t next[kMaxExperts];
    const int lane = threadIdx.x;
    const int c = blockIdx.x;
    for (int e = lane; e < E; e += 64) next[e] = base[static_cast<int64_t>(e) * nchunks + c];
    __syncthreads();
    const int64_t lo = static_cast<int64_t>(c) * chunk;
    const int64_t hi = min(lo + chunk, n_assign);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int64_t a0 = lo; a0 < hi; a0 += 64) {
        const int64_t a = a0 + lane;
        int e = (a < hi) ? topk_idx[a] : -1;
        const bool valid = (e >= 0 && e < E);
        if (!valid) e = -1;
        int pos = -1;
        uint64_t pending = __ballot(valid);
        while (pending) {
            const int leader = __ffsll(static_cast<unsigned long long>(pending)) - 1;
            const int el = __shfl(e, leader, 64);
            const uint64_t same = __ballot(e == el);
            const int b = next[el];
            if (e == el) pos = b + __popcll(same & below);
            __syncthreads();  // every lane has read next[el] before the leader moves it
            if (lane == leader) next[el] = b + __popcll(same);
            __syncthreads();
            pending &= ~same;
        }
        if (a < hi) {
            row_of[a] = pos;
            if (pos >= 0) row_src[pos] = static_cast<int32_t>(a / k);
        }
    }
}

// x_perm[r] = x[row_src[r]]: one wavefront copies one row, 16 bytes per lane.
// Rows past expert_offsets[E] (only when some ids were out of range) are left alone.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ x, int64_t T, int d,
                                                          const int32_t* __restrict__ row_src,
                                                          const int32_t* __restrict__ n_valid,
                                                          int64_t n_rows, uint16_t* __restrict__ x_perm) {
    const int lane = threadIdx.x & 63;
    const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (r >= n_rows || r >= *n_valid) return;
    const int src = row_src[r];
    if (src < 0 || src >= T) return;
    const uint4* s = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(src) * d);
    uint4* o = reinterpret_cast<uint4*>(x_perm + r * d);
    for (int c = lane; c < d / 8; c += 64) o[c] = s[c];
}

__global__ void zero_i32_kernel(int32_t* __restrict__ p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// ---------------------------------------------------------------- launchers

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t stream) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

int permute_chunk(int64_t n_assign) {
    int64_t c = (n_assign + 255) / 256;  // at most 256 chunks
    c = (c + 63) / 64 * 64;
    return static_cast<int>(c < 256 ? 256 : c);
}

int permute_nchunks(int64_t n_assign) {
    const int c = permute_chunk(n_assign);
    return static_cast<int>((n_assign + c - 1) / c);
}

hipError_t launch_permute(const uint16_t* x, const int32_t* topk_idx, int64_t T, int d, int E, int k,
                          int32_t* expert_offsets, int32_t* row_of, int32_t* row_src, uint16_t* x_perm,
                          int32_t* count_ws, hipStream_t stream) {
    const int64_t n = T * k;
    const int chunk = permute_chunk(n);
    const int nchunks = permute_nchunks(n);
    hipLaunchKernelGGL(expert_count_kernel, dim3(nchunks), dim3(256), 0, stream, topk_idx, n, E, chunk,
                       nchunks, count_ws);
    hipLaunchKernelGGL(expert_scan_kernel, dim3(1), dim3(1024), 0, stream, count_ws, E, nchunks,
                       expert_offsets);
    hipLaunchKernelGGL(expert_rank_kernel, dim3(nchunks), dim3(64), 0, stream, topk_idx, n, k, E, chunk,
                       nchunks, count_ws, row_of, row_src);
    if (x_perm != nullptr)
        hipLaunchKernelGGL(gather_rows_kernel, dim3(static_cast<unsigned>((n + 3) / 4)), dim3(256), 0, stream,
                           x, T, d, row_src, expert_offsets + E, n, x_perm);
    return hipGetLastError();
}

}  // namespace moe
