// Wavefront top-K of up to 64 * NPER scores (one wavefront per token).
//
// Element i of lane l is expert e = l + 64 i (valid when e < E). Its 64-bit key
// is (order_key(score) << 32) | ~e, so keys are distinct and the largest key is
// the largest score with ties to the lower id (-0 ties +0, NaN below every
// number). select_top leaves, in lane j < K, the j-th largest key.
//
// Instead of K rounds of "local maximum over NPER keys, wavefront maximum,
// clear the winner" (K * NPER work per lane), a threshold prunes first:
//   1. tau = the K-th largest of the 64 lanes' largest value keys, found bit
//      by bit with ballots down to its upper 16 bits (so rounded down). At
//      least K keys have a value key >= tau (those lane maxima), so every one
//      of the K largest keys has value key >= tau.
//   2. The elements with value key >= tau (the candidates) are compacted into
//      a 64-entry LDS array of the wavefront: the ballot of each element index
//      is the write mask, and each writing lane's slot is the count of writing
//      lanes below it (mbcnt).
//   3. Each candidate counts the candidates above it (its rank) by reading the
//      array back (one broadcast read per candidate); the candidate of rank j
//      is written to entry j of a second array and lane j reads it.
// Step 2 compares the scores as floats: order_key is monotone and maps the
// non-NaN floats (-0 and +0 to one key) one to one onto the keys it produces, so
// for a threshold f = key_value(tau) that is a number, order_key(s) >= tau
// exactly when s >= f (denormals are kept, -0 == +0, NaN fails both; tau =
// 0x7fffffff gives f = -0, and both sides then admit exactly s >= 0). Only the
// candidates get their 64-bit keys. A zero tau (NaN or padding among the lane
// maxima), a threshold that is not a number (a k-th lane maximum of -inf) and
// more than 64 candidates (massive ties) take the round-based selection on full
// keys.
#pragma once

#include "device_common.h"

namespace moe {

// v[i] = row[lane + 64 i] for i < NPER, or `fill` past the row's end (n entries,
// n > 64 (NPER - 1), so only the last element can be past it). The first NPER - 1
// loads share one address with immediate offsets and the last reads a clamped
// index, so none sits behind a branch and all NPER are in flight together; a load
// under `if (e < n)` would be followed by its own wait, one memory round trip per
// element.
template <int NPER>
__device__ __forceinline__ void load_row_strided(const float* __restrict__ row, int n, float fill, float (&v)[NPER]) {
    const int lane = threadIdx.x & 63;
    const float* p = row + lane;
#pragma unroll
    for (int i = 0; i < NPER - 1; ++i) v[i] = p[64 * i];
    const int last = lane + 64 * (NPER - 1);
    v[NPER - 1] = row[min(last, n - 1)];
    if (last >= n) v[NPER - 1] = fill;
}

constexpr int kSelectLds = 128;  // uint64 entries of LDS per wavefront (two arrays of 64)
// The bisection for tau stops above this many low key bits: tau is then at most
// the k-th largest lane maximum and within 2^-7 of it in relative terms, still a
// valid threshold (at least K value keys reach it), which admits a few more
// candidates in exchange for half the serial ballot steps.
constexpr int kSelectLowBits = 16;

// v[i]: score of element i; E: valid elements (64 (NPER - 1) < E <= 64 NPER); K <= E.
template <int NPER>
__device__ __forceinline__ uint64_t select_top(const float (&v)[NPER], int E, int K, uint64_t* lds) {
    const int lane = threadIdx.x & 63;
    const bool last_on = lane + 64 * (NPER - 1) < E;  // only the last element can be padding
    auto key_of = [](float x, uint32_t id) {
        return (static_cast<uint64_t>(order_key(x)) << 32) | (0xffffffffu - id);
    };
    // 1. tau over the lanes' largest value keys (padding and NaN count as 0)
    float mf = last_on ? v[NPER - 1] : __uint_as_float(0x7fc00000u);
#pragma unroll
    for (int i = 0; i < NPER - 1; ++i) mf = fmaxf(mf, v[i]);  // a NaN operand loses
    uint32_t m = order_key(mf);
    asm volatile("" : "+v"(m));  // materialise m once (else its NaN select is re-evaluated in every step below)
    uint32_t tau = 0u;
    for (int b = 31; b >= kSelectLowBits; --b) {
        const uint32_t cand = tau | (1u << b);
        if (__popcll(__ballot(m >= cand)) >= K) tau = cand;
    }
    // 2. candidates, compacted as (score bits, id) in (element, lane) order while they are counted
    int total = 65;
    const float f = key_value(tau);
    if (tau != 0u && f == f) {
        total = 0;
#pragma unroll
        for (int i = 0; i < NPER; ++i) {
            const bool c = v[i] >= f && (i < NPER - 1 || last_on);
            const uint64_t bal = __ballot(c);
            if (c && total + __popcll(bal) <= 64) {
                const uint32_t below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0u));
                lds[total + static_cast<int>(below)] =
                    (static_cast<uint64_t>(__float_as_uint(v[i])) << 32) | static_cast<uint32_t>(lane + 64 * i);
            }
            total += __popcll(bal);
        }
    }
    uint64_t mine = 0ull;
    if (total <= 64) {
        __builtin_amdgcn_wave_barrier();
        // 3. each candidate's key into its own slot, then ranks, then the candidates in rank order
        uint64_t my = 0ull;
        if (lane < total) {
            const uint64_t p = lds[lane];
            my = key_of(__uint_as_float(static_cast<uint32_t>(p >> 32)), static_cast<uint32_t>(p));
        }
        __builtin_amdgcn_wave_barrier();
        if (lane < total) lds[lane] = my;
        __builtin_amdgcn_wave_barrier();
        int rank = 0;
        for (int c = 0; c < total; ++c) rank += lds[c] > my ? 1 : 0;
        __builtin_amdgcn_wave_barrier();
        if (lane < total && rank < K) lds[64 + rank] = my;
        __builtin_amdgcn_wave_barrier();
        mine = lane < K ? lds[64 + lane] : 0ull;
    } else {
        uint64_t key[NPER];
#pragma unroll
        for (int i = 0; i < NPER; ++i)
            key[i] = (i < NPER - 1 || last_on) ? key_of(v[i], static_cast<uint32_t>(lane + 64 * i)) : 0ull;
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
