// Wavefront top-K of up to 64 * NPER 64-bit keys (one wavefront per token).
//
// Each lane holds NPER keys (0 = absent); a key's upper 32 bits order the value,
// its lower 32 bits are ~id, so keys are distinct and the largest key is the
// largest value with ties to the lower id. select_top leaves, in lane j < K, the
// j-th largest key.
//
// Instead of K rounds of "local maximum over NPER keys, wavefront maximum,
// clear the winner" (K * NPER work per lane), a threshold prunes first:
//   1. tau = the K-th largest of the 64 lanes' largest value halves, found bit
//      by bit with ballots. At least K keys have a value half >= tau (those
//      lane maxima), so every one of the K largest keys has value half >= tau.
//   2. The keys with value half >= tau (the candidates) are compacted into a
//      64-entry LDS array of the wavefront with ballot prefix counts.
//   3. Each candidate counts the candidates above it (its rank) by reading the
//      array back (one broadcast read per candidate); the candidate of rank j
//      is written to entry j of a second array and lane j reads it.
// More than 64 candidates (massive ties) fall back to the round-based selection.
#pragma once

#include "device_common.h"

namespace moe {

// v[i] = row[lane + 64 i] for i < NPER, or `fill` past the row's end (n entries).
// Every load reads a clamped index inside the row, so none sits behind a branch and
// all NPER are in flight together; a load under `if (e < n)` would be followed by its
// own wait, one memory round trip per element.
template <int NPER>
__device__ __forceinline__ void load_row_strided(const float* __restrict__ row, int n, float fill, float (&v)[NPER]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NPER; ++i) v[i] = row[min(lane + 64 * i, n - 1)];
#pragma unroll
    for (int i = 0; i < NPER; ++i)
        if (lane + 64 * i >= n) v[i] = fill;
}

constexpr int kSelectLds = 128;  // uint64 entries of LDS per wavefront (two arrays of 64)

template <int NPER>
__device__ __forceinline__ uint64_t select_top(uint64_t (&key)[NPER], int K, uint64_t* lds) {
    const int lane = threadIdx.x & 63;
    const uint64_t below = (1ull << lane) - 1ull;
    // 1. tau over the lanes' largest value halves
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < NPER; ++i) m = max(m, static_cast<uint32_t>(key[i] >> 32));
    uint32_t tau = 0u;
    for (int b = 31; b >= 0; --b) {
        const uint32_t cand = tau | (1u << b);
        if (__popcll(__ballot(m >= cand)) >= K) tau = cand;
    }
    // 2. candidates and their count
    int total = 0;
    uint64_t ball[NPER];
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
        ball[i] = __ballot(key[i] != 0ull && static_cast<uint32_t>(key[i] >> 32) >= tau);
        total += __popcll(ball[i]);
    }
    uint64_t mine = 0ull;
    if (total <= 64) {
        int base = 0;
#pragma unroll
        for (int i = 0; i < NPER; ++i) {
            if ((ball[i] >> lane) & 1ull) lds[base + __popcll(ball[i] & below)] = key[i];
            base += __popcll(ball[i]);
        }
        __builtin_amdgcn_wave_barrier();
        // 3. ranks, then the candidates in rank order
        const uint64_t my = lane < total ? lds[lane] : 0ull;
        int rank = 0;
        for (int c = 0; c < total; ++c) rank += lds[c] > my ? 1 : 0;
        __builtin_amdgcn_wave_barrier();
        if (lane < total && rank < K) lds[64 + rank] = my;
        __builtin_amdgcn_wave_barrier();
        mine = lane < K ? lds[64 + lane] : 0ull;
    } else {
        for (int j = 0; j < K; ++j) {
            uint64_t best = key[0];
#pragma unroll
            for (int i = 1; i < NPER; ++i) best = key[i] > best ? key[i] : best;
            best = wave_max_u64(best);
#pragma unroll
            for (int i = 0; i < NPER; ++i)
                if (key[i] == best) key[i] = 0ull;
            if (lane == j) mine = best;
        }
    }
    return mine;
}

}  // namespace moe
