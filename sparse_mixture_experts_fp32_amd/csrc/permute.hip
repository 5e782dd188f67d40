// Grouping the (token, slot) assignments by expert: per-chunk histograms, one
// prefix scan, then a stable rank within each chunk, and the row gather.
//
// The assignments a = t * k + j are cut into at most kMaxChunks chunks of
// consecutive indices. Rows of expert e are ordered by a, so the first row of
// chunk c inside expert e is
//     offsets[e] + sum_{c' < c} count[e, c'],
// an exclusive scan of count laid out expert-major, chunk-minor. A chunk is
// handled by one workgroup of kRankWaves wavefronts, each owning a contiguous
// slice of the chunk and walking it 64 assignments at a time in order.
//
// Equal experts among the 64 lanes are found without atomics and without a
// loop over distinct experts: one ballot per bit of the expert id gives every
// lane the mask of lanes holding the same id (AND of the ballots where its bit
// is set and of the complements where it is clear). The lane's rank among
// them is a popcount of the lower lanes in that mask, and only the lowest such
// lane updates the expert's counter, so the result is exact and deterministic.
// Per-expert token counts never leave the device ("Kimi K3: Open Frontier
// Intelligence", section "Systems Optimization, Load Balancing, and
// Post-Training Alignment": waiting on dynamic counts on the host stalls the
// device).
#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxChunks = 32;
constexpr int kRankWaves = 16;

// Mask of the lanes whose key equals this lane's key (keys below 2^nbits).
__device__ __forceinline__ uint64_t same_key_lanes(uint32_t key, int nbits, uint64_t active) {
    uint64_t same = active;
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1u;
        const uint64_t m = __ballot(bit);
        same &= bit ? m : ~m;
    }
    return same;
}

// Assignment slice [lo, hi) of wave w inside chunk c (slices are multiples of 64).
__device__ __forceinline__ void wave_slice(int64_t n_assign, int chunk, int c, int w, int64_t& lo, int64_t& hi) {
    const int64_t c0 = static_cast<int64_t>(c) * chunk;
    const int64_t c1 = min(c0 + chunk, n_assign);
    const int64_t per = ((c1 - c0 + kRankWaves * 64 - 1) / (kRankWaves * 64)) * 64;
    lo = min(c0 + w * per, c1);
    hi = min(lo + per, c1);
}

// ids of assignments a0 + 64 u + lane (u < kIdBatch), -1 at and past hi (a0 < hi).
// All kIdBatch loads read a clamped index and are in flight together: one
// memory round trip per batch instead of one per 64 assignments.
constexpr int kIdBatch = 8;
__device__ __forceinline__ void load_ids(const int32_t* __restrict__ topk_idx, int64_t a0, int64_t hi,
                                         int (&e)[kIdBatch]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) e[u] = topk_idx[min(a0 + 64 * u + lane, hi - 1)];
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u)
        if (a0 + 64 * u + lane >= hi) e[u] = -1;
}

// Adds the expert histogram of this wave's slice to hist[0 .. E) (hist private to the wave).
__device__ void wave_histogram(const int32_t* __restrict__ topk_idx, int64_t lo, int64_t hi, int E, int nbits,
                               int32_t* hist) {
    const int lane = threadIdx.x & 63;
    const uint64_t below = (1ull << lane) - 1ull;
    for (int64_t a00 = lo; a00 < hi; a00 += 64 * kIdBatch) {
        int ev[kIdBatch];
        load_ids(topk_idx, a00, hi, ev);
#pragma unroll
        for (int u = 0; u < kIdBatch; ++u) {
            if (a00 + 64 * u >= hi) break;  // uniform
            const int e = ev[u];            // -1 past hi
            const bool valid = e >= 0 && e < E;
            const uint32_t key = valid ? static_cast<uint32_t>(e) : (1u << nbits) - 1u;
            const uint64_t same = same_key_lanes(key, nbits, __ballot(valid));
            if (valid && (same & below) == 0) hist[e] += __popcll(same);
        }
    }
}

// count[e * nchunks + c] = assignments of chunk c that chose expert e.
__global__ __launch_bounds__(kRankWaves * 64) void expert_count_kernel(const int32_t* __restrict__ topk_idx,
                                                                       int64_t n_assign, int E, int nbits, int chunk,
                                                                       int nchunks, int32_t* __restrict__ count) {
    __shared__ int32_t hist[kRankWaves][kMaxExperts];
    const int w = threadIdx.x >> 6, c = blockIdx.x;
    for (int i = threadIdx.x; i < kRankWaves * kMaxExperts; i += blockDim.x) (&hist[0][0])[i] = 0;
    __syncthreads();
    int64_t lo, hi;
    wave_slice(n_assign, chunk, c, w, lo, hi);
    wave_histogram(topk_idx, lo, hi, E, nbits, hist[w]);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int32_t s = 0;
#pragma unroll
        for (int v = 0; v < kRankWaves; ++v) s += hist[v][e];
        count[static_cast<int64_t>(e) * nchunks + c] = s;
    }
}

// One 1024-thread workgroup. Rewrites count[e, c] as the first row of (e, c);
// expert_offsets[e] = first row of e, expert_offsets[E] = all rows. The E x nchunks
// counts (<= 1024 x 32) are read and written coalesced through LDS (rows padded to
// nchunks + 1 words, so thread e's walk along its row is free of bank conflicts);
// the scan over experts is a wavefront scan (shuffles) plus a scan of the 16
// wavefront totals.
__global__ __launch_bounds__(1024) void expert_scan_kernel(int32_t* __restrict__ count, int E, int nchunks,
                                                           int32_t* __restrict__ expert_offsets) {
    __shared__ int32_t cs[kMaxExperts * (kMaxChunks + 1)];
    __shared__ int32_t wsum[1024 / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int stride = nchunks + 1;
    // half-wavefront h of wave w moves row e = 2 * (16 * it + w) + h, lane & 31 = its chunk
    const int half_row = 2 * wave + (lane >> 5), col = lane & 31;
    for (int e0 = 0; e0 < E; e0 += 32 * kIdBatch) {  // kIdBatch loads in flight per thread
        int32_t v[kIdBatch];
#pragma unroll
        for (int u = 0; u < kIdBatch; ++u) {
            const int e = min(e0 + 32 * u + half_row, E - 1);
            v[u] = count[e * nchunks + min(col, nchunks - 1)];
        }
#pragma unroll
        for (int u = 0; u < kIdBatch; ++u) {
            const int e = e0 + 32 * u + half_row;
            if (e < E && col < nchunks) cs[e * stride + col] = v[u];
        }
    }
    __syncthreads();
    int32_t total = 0;
    if (tid < E)
        for (int c = 0; c < nchunks; ++c) total += cs[tid * stride + c];
    // inclusive scan of the totals within the wavefront
    int32_t incl = total;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int32_t before = 0;  // totals of the lower wavefronts
    for (int v = 0; v < wave; ++v) before += wsum[v];
    int32_t run = before + incl - total;  // exclusive prefix of expert tid
    if (tid < E) {
        expert_offsets[tid] = run;
        for (int c = 0; c < nchunks; ++c) {
            const int32_t cnt = cs[tid * stride + c];
            cs[tid * stride + c] = run;
            run += cnt;
        }
    }
    if (tid == 1023) {
        int32_t all = 0;
        for (int v = 0; v < 1024 / 64; ++v) all += wsum[v];
        expert_offsets[E] = all;
    }
    __syncthreads();
    for (int e = half_row; e < E; e += 32)
        if (col < nchunks) count[e * nchunks + col] = cs[e * stride + col];
}

// One workgroup per chunk: stable ranks, row_of and row_src.
__global__ __launch_bounds__(kRankWaves * 64) void expert_rank_kernel(
    const int32_t* __restrict__ topk_idx, int64_t n_assign, int k, int E, int nbits, int chunk, int nchunks,
    const int32_t* __restrict__ base, int32_t* __restrict__ row_of, int32_t* __restrict__ row_src) {
    __shared__ int32_t next[kRankWaves][kMaxExperts];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, c = blockIdx.x;
    for (int i = threadIdx.x; i < kRankWaves * kMaxExperts; i += blockDim.x) (&next[0][0])[i] = 0;
    __syncthreads();
    int64_t lo, hi;
    wave_slice(n_assign, chunk, c, w, lo, hi);
    wave_histogram(topk_idx, lo, hi, E, nbits, next[w]);
    __syncthreads();
    // first row of (expert e, wave v) = chunk base + assignments of e in waves < v
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int32_t run = base[static_cast<int64_t>(e) * nchunks + c];
#pragma unroll
        for (int v = 0; v < kRankWaves; ++v) {
            const int32_t n = next[v][e];
            next[v][e] = run;
            run += n;
        }
    }
    __syncthreads();
    int32_t* nx = next[w];
    const uint64_t below = (1ull << lane) - 1ull;
    for (int64_t a00 = lo; a00 < hi; a00 += 64 * kIdBatch) {
        int ev[kIdBatch];
        load_ids(topk_idx, a00, hi, ev);
#pragma unroll
        for (int u = 0; u < kIdBatch; ++u) {
            const int64_t a0 = a00 + 64 * u;
            if (a0 >= hi) break;  // uniform
            const int64_t a = a0 + lane;
            const bool in = a < hi;
            const int e = ev[u];  // -1 past hi
            const bool valid = e >= 0 && e < E;
            const uint32_t key = valid ? static_cast<uint32_t>(e) : (1u << nbits) - 1u;
            const uint64_t same = same_key_lanes(key, nbits, __ballot(valid));
            int pos = -1;
            if (valid) pos = nx[e] + static_cast<int>(__popcll(same & below));
            // every lane has read nx[e] (one LDS instruction, in program order) before the
            // lowest lane of each expert moves that expert's counter
            if (valid && (same & below) == 0) nx[e] += static_cast<int>(__popcll(same));
            if (in) {
                row_of[a] = pos;
                if (pos >= 0) row_src[pos] = static_cast<int32_t>(static_cast<uint32_t>(a) / static_cast<uint32_t>(k));
            }
        }
    }
}

// x_perm[r] = x[row_src[r]]: one wavefront copies one 512-element (1 KiB) block of
// one row, 16 bytes per lane, so there are many small work items and each lane
// makes a single load and store. x_perm is written once and read by a later
// pass over many other bytes, so it is stored non-temporally. Rows past
// expert_offsets[E] (only when some ids were out of range) are left alone.
constexpr int kGatherCols = 512;  // bf16 elements per work item
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ x, int64_t T, int d,
                                                          const int32_t* __restrict__ row_src,
                                                          const int32_t* __restrict__ n_valid,
                                                          int64_t n_rows, uint16_t* __restrict__ x_perm) {
    const int lane = threadIdx.x & 63;
    const int nblk = (d + kGatherCols - 1) / kGatherCols;
    const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int64_t r = item / nblk;
    if (r >= n_rows || r >= *n_valid) return;
    const int src = row_src[r];
    if (src < 0 || src >= T) return;
    const int c = static_cast<int>(item - r * nblk) * (kGatherCols / 8) + lane;  // 16-byte chunk of the row
    if (c >= d / 8) return;
    const u32x4 v = reinterpret_cast<const u32x4*>(x + static_cast<int64_t>(src) * d)[c];
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(x_perm + r * d) + c);
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

// Chunk length: a multiple of kRankWaves * 64, at least that, so that there are
// at most kMaxChunks chunks.
int permute_chunk(int64_t n_assign) {
    const int64_t unit = kRankWaves * 64;
    const int64_t per = (n_assign + kMaxChunks - 1) / kMaxChunks;
    const int64_t c = (per + unit - 1) / unit * unit;
    return static_cast<int>(c < unit ? unit : c);
}

int permute_nchunks(int64_t n_assign) {
    const int c = permute_chunk(n_assign);
    return static_cast<int>((n_assign + c - 1) / c);
}

static int id_bits(int E) {  // bits of the ids 0 .. E (E itself marks "no expert")
    int b = 1;
    while ((1 << b) <= E) ++b;
    return b;
}

hipError_t launch_permute(const uint16_t* x, const int32_t* topk_idx, int64_t T, int d, int E, int k,
                          int32_t* expert_offsets, int32_t* row_of, int32_t* row_src, uint16_t* x_perm,
                          int32_t* count_ws, hipStream_t stream) {
    const int64_t n = T * k;
    const int chunk = permute_chunk(n);
    const int nchunks = permute_nchunks(n);
    const int nbits = id_bits(E);
    hipLaunchKernelGGL(expert_count_kernel, dim3(nchunks), dim3(kRankWaves * 64), 0, stream, topk_idx, n, E, nbits,
                       chunk, nchunks, count_ws);
    hipLaunchKernelGGL(expert_scan_kernel, dim3(1), dim3(1024), 0, stream, count_ws, E, nchunks, expert_offsets);
    hipLaunchKernelGGL(expert_rank_kernel, dim3(nchunks), dim3(kRankWaves * 64), 0, stream, topk_idx, n, k, E, nbits,
                       chunk, nchunks, count_ws, row_of, row_src);
    if (x_perm != nullptr) {
        const int64_t items = n * ((d + kGatherCols - 1) / kGatherCols);
        if ((items + 3) / 4 > INT32_MAX) return hipErrorInvalidValue;  // beyond one launch's grid
        hipLaunchKernelGGL(gather_rows_kernel, dim3(static_cast<unsigned>((items + 3) / 4)), dim3(256), 0, stream,
                           x, T, d, row_src, expert_offsets + E, n, x_perm);
    }
    return hipGetLastError();
}

}  // namespace moe
