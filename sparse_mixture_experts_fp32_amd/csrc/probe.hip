// Ceiling probes of the MI355X (gfx950): how fast this chip reads, copies and
// streams HBM into LDS, and how fast its matrix cores run back-to-back bf16
// products. The layer's kernels are measured against these beside the published
// peaks. Each probe produces a result the caller can check exactly (a checksum,
// a copy, a known sum), so none can be fast by skipping work.
#include "moe_probe.h"

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "lds_dma.h"

namespace moe {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocksPerCu = 8;
constexpr int kDmaStage = 32768;  // 8 waves x 4 loads of 1 KiB

__device__ __forceinline__ uint32_t word_sum(const u32x4& v) { return v.x + v.y + v.z + v.w; }

// One atomic per workgroup (one per wave would serialise thousands of atomics on
// one address and dominate the time of a small probe).
__device__ __forceinline__ void add_to_sink(uint32_t acc, uint32_t* sink) {
    __shared__ uint32_t part[16];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kWave);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < static_cast<int>(blockDim.x) / kWave; ++w) t += part[w];
        atomicAdd(sink, t);
    }
}

// One pass over the buffer: workgroup b reads 32 KiB tile b (256 threads x eight 16-byte
// loads, all issued before any is summed; the last tile may be partial) and writes
// out[b] = the sum of its words modulo 2^32. No loop and no atomic, so a buffer of tens
// of MB is read as fast as one launch can read it.
constexpr int kTileChunks = 8 * 256;  // 16-byte chunks per tile
__global__ __launch_bounds__(256) void probe_read_tiles_kernel(const u32x4* __restrict__ p, int64_t n,
                                                               uint32_t* __restrict__ out) {
    __shared__ uint32_t part[4];
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kTileChunks + threadIdx.x;
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = p[min(base + 256 * j, n - 1)];
    uint32_t acc = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (base + 256 * j < n) acc += word_sum(v[j]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kWave);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
}

// Each wave reads contiguous 4 KiB runs (four 1 KiB loads in flight, lane l at 16 l of
// each), striding over the runs by the number of waves; the last partial run by lanes.
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4* __restrict__ p, int64_t n,
                                                                   uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = static_cast<int64_t>(gridDim.x) * (kProbeThreads / kWave);
    const int64_t w = static_cast<int64_t>(blockIdx.x) * (kProbeThreads / kWave) + (threadIdx.x >> 6);
    const int64_t runs = n / 256;  // 256 chunks of 16 bytes per run
    uint32_t acc = 0;
    for (int64_t r = w; r < runs; r += waves) {
        const u32x4* q = p + r * 256 + lane;
        const u32x4 a = q[0], b = q[64], c = q[128], d = q[192];
        acc += word_sum(a) + word_sum(b) + word_sum(c) + word_sum(d);
    }
    for (int64_t i = runs * 256 + w * kWave + lane; i < n; i += waves * kWave) acc += word_sum(p[i]);
    add_to_sink(acc, sink);
}

// The same walk as the read probe, storing each run to dst.
__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst, int64_t n) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = static_cast<int64_t>(gridDim.x) * (kProbeThreads / kWave);
    const int64_t w = static_cast<int64_t>(blockIdx.x) * (kProbeThreads / kWave) + (threadIdx.x >> 6);
    const int64_t runs = n / 256;
    for (int64_t r = w; r < runs; r += waves) {
        const int64_t i = r * 256 + lane;
        const u32x4 a = src[i], b = src[i + 64], c = src[i + 128], d = src[i + 192];
        dst[i] = a;
        dst[i + 64] = b;
        dst[i + 128] = c;
        dst[i + 192] = d;
    }
    for (int64_t i = runs * 256 + w * kWave + lane; i < n; i += waves * kWave) dst[i] = src[i];
}

// One 8-wave workgroup per CU streams 32 KiB chunks blockIdx.x, + gridDim.x, ... of the
// buffer through a three-stage LDS ring with direct-to-LDS loads (two chunks in
// flight while the third is read back), the load pattern of the expert GEMM.
__global__ __launch_bounds__(512) void probe_dma_kernel(const uint8_t* __restrict__ buf, int64_t n_chunks,
                                                        uint32_t* __restrict__ sink) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[3 * kDmaStage];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t mine = (n_chunks - blockIdx.x + gridDim.x - 1) / gridDim.x;  // chunks of this workgroup
    if (mine <= 0) return;  // uniform, before any barrier
    const uint32_t ring_lds = lds_addr(ring);
    auto issue = [&](int64_t c) {
        const uint8_t* src = buf + (blockIdx.x + gridDim.x * c) * kDmaStage + 4096 * wave;
        const void* base = uniform_ptr(src);
        const uint32_t slot = ring_lds + static_cast<uint32_t>((c % 3) * kDmaStage + 4096 * wave);
#pragma unroll
        for (int q = 0; q < 4; ++q) dma_saddr(slot + 1024u * q, base, 16u * lane + 1024u * q);
    };
    issue(0);
    if (mine > 1) issue(1);
    uint32_t acc = 0;
    for (int64_t c = 0; c < mine; ++c) {
        if (c + 1 < mine)
            wait_barrier<4>();  // this wave's loads of chunk c landed; chunk c + 1's may fly
        else
            wait_barrier<0>();
        if (c + 2 < mine) issue(c + 2);  // into the slot chunk c - 1 used (read back before the barrier)
        const u32x4* st = reinterpret_cast<const u32x4*>(ring + (c % 3) * kDmaStage);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc += word_sum(st[threadIdx.x + 512 * q]);
    }
    add_to_sink(acc, sink);
}

// Each wave: iters rounds of 16 independent 16x16x32 bf16 products of all-ones operands.
__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(int iters, float* __restrict__ sink) {
    const float one = iters > 0 ? 1.0f : 0.0f;  // a value the compiler cannot fold
    bf16x8 a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = static_cast<__bf16>(one);
    f32x4 acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = mfma_16x16x32(a, a, acc[j]);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[j][0];
    const int w = blockIdx.x * (kProbeThreads / kWave) + (threadIdx.x >> 6);
    if ((threadIdx.x & 63) == 0) sink[w] = s;
}

static int probe_grid() {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    return cus;
}

}  // namespace moe

using namespace moe;

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

extern "C" int moe_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (buf == nullptr || sink == nullptr || !aligned16(buf) || bytes % 16 != 0 || bytes == 0) return -1;
    hipLaunchKernelGGL(probe_read_kernel, dim3(probe_grid() * kProbeBlocksPerCu), dim3(kProbeThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf),
                       static_cast<int64_t>(bytes / 16), sink);
    return static_cast<int>(hipGetLastError());
}

extern "C" int moe_probe_read_tiles(const void* buf, size_t bytes, uint32_t* out, void* stream) {
    if (buf == nullptr || out == nullptr || !aligned16(buf) || bytes % 16 != 0 || bytes == 0) return -1;
    const int64_t n = static_cast<int64_t>(bytes / 16);
    const int64_t tiles = (n + kTileChunks - 1) / kTileChunks;
    if (tiles > 0x7fffffff) return -1;
    hipLaunchKernelGGL(probe_read_tiles_kernel, dim3(static_cast<unsigned>(tiles)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), n, out);
    return static_cast<int>(hipGetLastError());
}

extern "C" int moe_probe_dma_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (buf == nullptr || sink == nullptr || !aligned16(buf) || bytes % kDmaStage != 0 || bytes == 0) return -1;
    hipLaunchKernelGGL(probe_dma_kernel, dim3(probe_grid()), dim3(512), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint8_t*>(buf), static_cast<int64_t>(bytes / kDmaStage), sink);
    return static_cast<int>(hipGetLastError());
}

extern "C" int moe_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (src == nullptr || dst == nullptr || !aligned16(src) || !aligned16(dst) || bytes % 16 != 0 || bytes == 0)
        return -1;
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    if (s < d + bytes && d < s + bytes) return -1;
    hipLaunchKernelGGL(probe_copy_kernel, dim3(probe_grid() * kProbeBlocksPerCu), dim3(kProbeThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), static_cast<u32x4*>(dst),
                       static_cast<int64_t>(bytes / 16));
    return static_cast<int>(hipGetLastError());
}

extern "C" int moe_probe_mfma(int32_t waves, int32_t iters, float* sink, void* stream) {
    if (sink == nullptr || waves <= 0 || waves % 4 != 0 || iters < 1 || iters > 32768) return -1;
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(waves / 4), dim3(kProbeThreads), 0, static_cast<hipStream_t>(stream),
                       iters, sink);
    return static_cast<int>(hipGetLastError());
}
