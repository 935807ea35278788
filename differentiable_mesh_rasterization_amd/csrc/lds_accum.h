// Per-workgroup LDS accumulation of float triples keyed by a 32-bit id
// (a vertex or a point), for gradients that many lanes of a workgroup add
// to the same few ids: an open-addressing table of 64-bit fixed-point sums,
// flushed with one float atomic per (id, coordinate).
#pragma once

#include "dmr_internal.h"

namespace dmr {

constexpr int kHashBits = 10;
constexpr int kHashSize = 1 << kHashBits;
constexpr int kProbe = 32;

// LDS sums are kept in 64-bit fixed point with kFixBits fractional bits: an
// integer LDS atomic add is about 20x faster than a float one on gfx950 and
// serialises conflicting lanes without retry loops. A contribution is
// rounded to a multiple of 2^-kFixBits (3.7e-9); only contributions below
// kFixLimit in magnitude take this path (larger ones go straight to global
// float atomics), so a tile's sum for one vertex coordinate -- at most
// 256 pixels x 64 slots contributions -- stays below 2^34 < 2^(63-kFixBits).
constexpr int kFixBits = 28;
constexpr float kFixLimit = 0x1.0p20f;

// (double)v * 2^kFixBits is exact; adding 1.5 * 2^52 rounds it to the
// nearest integer (ties to even), which then sits in the low mantissa bits
// of the sum as a two's complement offset from those of 1.5 * 2^52 (valid
// for magnitudes below 2^51, here below 2^48).
__device__ __forceinline__ unsigned long long to_fixed(float v) {
    const double kRound = 6755399441055744.0;   // 1.5 * 2^52
    const double d = (double)v * (double)(1ull << kFixBits) + kRound;
    return (unsigned long long)(__double_as_longlong(d) - __double_as_longlong(kRound));
}
__device__ __forceinline__ float from_fixed(unsigned long long x) {
    return (float)((double)(long long)x * (1.0 / (double)(1ull << kFixBits)));
}

// Adds one id's three partials into the tile's LDS hash table (2^HB
// entries), or into grad_verts directly when the table has no room for it
// or a value is too large for the fixed-point sums.
template <int HB = kHashBits>
__device__ __forceinline__ void vertex_add(int32_t* hkey, unsigned long long (*hval)[3],
                                           float* __restrict__ grad_verts, int64_t vi, float gx, float gy, float gz,
                                           bool use_hash) {
    const float lim = kFixLimit;
    if (use_hash && fabsf(gx) < lim && fabsf(gy) < lim && fabsf(gz) < lim) {
        const int32_t vid = (int32_t)vi;
        uint32_t h = ((uint32_t)vid * 2654435761u) >> (32 - HB);
#pragma unroll 1
        for (int p = 0; p < kProbe; ++p) {
            const int32_t cur = atomicCAS(&hkey[h], -1, vid);
            if (cur == -1 || cur == vid) {
                atomicAdd(&hval[h][0], to_fixed(gx));
                atomicAdd(&hval[h][1], to_fixed(gy));
                atomicAdd(&hval[h][2], to_fixed(gz));
                return;
            }
            h = (h + 1) & ((1u << HB) - 1u);
        }
    }
    atomicAdd(&grad_verts[3 * vi + 0], gx);
    atomicAdd(&grad_verts[3 * vi + 1], gy);
    atomicAdd(&grad_verts[3 * vi + 2], gz);
}


// The three vertices of one face at once: the first probe of all three is
// issued before any result is waited for, further probes (rare) follow in a
// loop, then the nine fixed-point adds (or global float atomics for a
// vertex the table cannot take).
template <int HB = kHashBits>
__device__ __forceinline__ void vertex_add3(int32_t* hkey, unsigned long long (*hval)[3],
                                            float* __restrict__ grad_verts, const int64_t (&vi)[3],
                                            const float (&g)[9], bool use_hash) {
    const float lim = kFixLimit;
    bool elig[3];
    uint32_t h[3];
    int32_t cur[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        elig[k] = use_hash && fabsf(g[3 * k]) < lim && fabsf(g[3 * k + 1]) < lim && fabsf(g[3 * k + 2]) < lim;
        h[k] = ((uint32_t)(int32_t)vi[k] * 2654435761u) >> (32 - HB);
        cur[k] = elig[k] ? atomicCAS(&hkey[h[k]], -1, (int32_t)vi[k]) : 0;
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int32_t vid = (int32_t)vi[k];
        int slot = -1;
        if (elig[k]) {
            if (cur[k] == -1 || cur[k] == vid) {
                slot = (int)h[k];
            } else {
                uint32_t hp = h[k];
#pragma unroll 1
                for (int p = 1; p < kProbe; ++p) {
                    hp = (hp + 1) & ((1u << HB) - 1u);
                    const int32_t c = atomicCAS(&hkey[hp], -1, vid);
                    if (c == -1 || c == vid) {
                        slot = (int)hp;
                        break;
                    }
                }
            }
        }
        if (slot >= 0) {
            atomicAdd(&hval[slot][0], to_fixed(g[3 * k]));
            atomicAdd(&hval[slot][1], to_fixed(g[3 * k + 1]));
            atomicAdd(&hval[slot][2], to_fixed(g[3 * k + 2]));
        } else {
            atomicAdd(&grad_verts[3 * vi[k] + 0], g[3 * k]);
            atomicAdd(&grad_verts[3 * vi[k] + 1], g[3 * k + 1]);
            atomicAdd(&grad_verts[3 * vi[k] + 2], g[3 * k + 2]);
        }
    }
}

// Flushes a workgroup's table into grad (3 floats per id) with float atomics.
template <int HB = kHashBits>
__device__ __forceinline__ void flush_table(const int32_t* hkey, const unsigned long long (*hval)[3],
                                            float* __restrict__ grad, int nthreads) {
    for (int e = threadIdx.x; e < (1 << HB); e += nthreads) {
        const int32_t vid = hkey[e];
        if (vid >= 0) {
            atomicAdd(&grad[3 * (int64_t)vid + 0], from_fixed(hval[e][0]));
            atomicAdd(&grad[3 * (int64_t)vid + 1], from_fixed(hval[e][1]));
            atomicAdd(&grad[3 * (int64_t)vid + 2], from_fixed(hval[e][2]));
        }
    }
}

template <int HB = kHashBits>
__device__ __forceinline__ void clear_table(int32_t* hkey, unsigned long long (*hval)[3], int nthreads) {
    for (int e = threadIdx.x; e < (1 << HB); e += nthreads) {
        hkey[e] = -1;
        hval[e][0] = 0;
        hval[e][1] = 0;
        hval[e][2] = 0;
    }
}

}  // namespace dmr
