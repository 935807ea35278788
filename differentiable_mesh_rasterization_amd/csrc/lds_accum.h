// Per-workgroup LDS accumulation of float triples keyed by an id (a vertex or
// a point), for gradients that many lanes of a workgroup add to the same few
// ids: an open-addressing table of 64-bit fixed-point sums, flushed with one
// float atomic per (id, coordinate).
//
// Each entry's fixed-point scale is relative, not absolute: it is set when
// the entry is inserted, to the power of two just above the largest partial
// of the slot that inserts it (for a face's slot, the largest of its nine
// partials, shared by its three vertices), and stored in the key word next
// to the id, so the accuracy of the sums does not depend on the scale of the
// upstream gradients. A vertex's own partial in a slot can be far smaller
// than the slot's others (with perspective correction, a vertex whose
// barycentric is near 0); a scale taken from it alone would push the
// vertex's later, ordinary contributions out of the entry's range.
#pragma once

#include "dmr_internal.h"

namespace dmr {

constexpr int kHashBits = 10;
constexpr int kHashSize = 1 << kHashBits;
constexpr int kProbe = 32;

// Key word of an entry: the id in the low kIdBits bits, the entry's exponent
// code (below) in the high 8 bits; all ones marks an empty entry. Ids up to
// kTableMaxId can use the table (larger ones would collide with the empty
// mark or overflow the id field); callers with larger ids pass use_hash =
// false and add every contribution with global float atomics.
constexpr int kIdBits = 24;
constexpr uint32_t kIdMask = (1u << kIdBits) - 1u;
constexpr uint32_t kEmptyKey = 0xffffffffu;
constexpr int64_t kTableMaxId = (int64_t)kIdMask - 1;

// Fixed point relative to an entry exponent e (every partial of the slot
// that inserted the entry is below 2^e in magnitude): a contribution is
// rounded to a multiple of 2^(e - kFixFrac) and taken into the entry only if
// its coordinates are below 2^(e + kFixAhead); larger ones go straight to
// global float atomics. A tile adds at most 2^14 contributions to one entry
// (256 pixels x 64 slots), so a sum stays below 2^(14 + kFixAhead +
// kFixFrac) = 2^62 units. The quantum is 2^-30 relative to the inserting
// slot's largest partial, far below binary32 resolution.
constexpr int kFixFrac = 30;
constexpr int kFixAhead = 18;
static_assert(14 + kFixFrac + kFixAhead <= 62, "64-bit fixed-point headroom");

// Exponent code of a magnitude m (finite, > 0): the biased binary32 exponent
// of m, at least 1, so that m < 2^(code - 126). 0 marks "no contribution"
// (m == 0), 255 "not finite".
__device__ __forceinline__ uint32_t mag_code(float m) {
    const uint32_t eb = __float_as_uint(m) >> 23;   // m >= 0: the sign bit is clear
    return m == 0.0f ? 0u : (eb == 0u ? 1u : eb);
}

// 2^k as a binary64 for |k| well inside the normal range.
__device__ __forceinline__ double pow2d(int k) {
    return __longlong_as_double((long long)(1023 + k) << 52);
}

// v / 2^(e - kFixFrac) rounded to the nearest integer, as a two's complement
// 64-bit pattern. For an entry with code c, e = c - 126. The product is
// exact in binary64 (a power-of-two scale); adding 1.5 * 2^52 rounds it to
// the nearest integer (ties to even), which then sits in the low mantissa
// bits of the sum as an offset from those of 1.5 * 2^52 (valid for
// magnitudes below 2^51; here below 2^(kFixAhead + kFixFrac) = 2^48).
__device__ __forceinline__ unsigned long long to_fixed(float v, uint32_t code) {
    const double kRound = 6755399441055744.0;   // 1.5 * 2^52
    const double d = (double)v * pow2d(kFixFrac + 126 - (int)code) + kRound;
    return (unsigned long long)(__double_as_longlong(d) - __double_as_longlong(kRound));
}
__device__ __forceinline__ float from_fixed(unsigned long long x, uint32_t code) {
    return (float)((double)(long long)x * pow2d((int)code - 126 - kFixFrac));
}

// Finds or inserts the entry of `id`, a new entry with exponent code `code`
// (1..254); returns its slot and the entry's code, or -1 when the probe
// sequence finds no room. `first` is the result of the first probe's
// compare-and-swap at slot h0 (issued by the caller).
template <int HB>
__device__ __forceinline__ int table_find(uint32_t* hkey, uint32_t id, uint32_t code, uint32_t h0, uint32_t first,
                                          uint32_t& entry_code) {
    uint32_t cur = first;
    uint32_t h = h0;
#pragma unroll 1
    for (int p = 0;; ) {
        if (cur == kEmptyKey) {
            entry_code = code;
            return (int)h;
        }
        if ((cur & kIdMask) == id) {
            entry_code = cur >> kIdBits;
            return (int)h;
        }
        if (++p >= kProbe) return -1;
        h = (h + 1) & ((1u << HB) - 1u);
        cur = atomicCAS(&hkey[h], kEmptyKey, id | (code << kIdBits));
    }
}

// First probe slot of `id` in a table of 2^hb entries: a multiplicative hash
// of id >> run_bits with the low run_bits of the id kept, so that a run of
// 2^run_bits consecutive ids takes consecutive slots (run_bits = 0: a plain
// multiplicative hash of the id). Consecutive slots are flushed by
// consecutive lanes, so runs of ids that are neighbours in grad reach memory
// in the same atomic instruction; the price is longer probe sequences when
// the table is well filled, so callers keep run_bits = 0 unless the ids of
// one workgroup come in runs.
__device__ __forceinline__ uint32_t hash_slot0(uint32_t id, int hb, int run_bits) {
    return ((((id >> run_bits) * 2654435761u) >> (32 - hb + run_bits)) << run_bits) | (id & ((1u << run_bits) - 1u));
}

__device__ __forceinline__ void global_add3(float* __restrict__ grad, int64_t vi, float gx, float gy, float gz) {
    atomicAdd(&grad[3 * vi + 0], gx);
    atomicAdd(&grad[3 * vi + 1], gy);
    atomicAdd(&grad[3 * vi + 2], gz);
}

// Adds one id's three partials into the tile's LDS hash table (2^HB
// entries), or into grad directly when the table cannot take them (no room,
// a coordinate not finite, or too large for the entry's scale). A
// contribution of three zeros adds nothing.
template <int HB = kHashBits>
__device__ __forceinline__ void vertex_add(uint32_t* hkey, unsigned long long (*hval)[3],
                                           float* __restrict__ grad, int64_t vi, float gx, float gy, float gz,
                                           bool use_hash, int run_bits = 0) {
    const float m = fmaxf(fabsf(gx), fmaxf(fabsf(gy), fabsf(gz)));   // fmaxf drops a NaN operand
    const uint32_t code = mag_code(m);
    const bool nan = (gx != gx) || (gy != gy) || (gz != gz);
    if (code == 0u && !nan) return;   // three zeros: nothing to add
    if (use_hash && m <= 3.402823466e38f && !nan) {
        const uint32_t id = (uint32_t)vi;
        const uint32_t h = hash_slot0(id, HB, run_bits);
        const uint32_t first = atomicCAS(&hkey[h], kEmptyKey, id | (code << kIdBits));
        uint32_t ec = 0;
        const int slot = table_find<HB>(hkey, id, code, h, first, ec);
        if (slot >= 0 && code <= ec + kFixAhead) {
            atomicAdd(&hval[slot][0], to_fixed(gx, ec));
            atomicAdd(&hval[slot][1], to_fixed(gy, ec));
            atomicAdd(&hval[slot][2], to_fixed(gz, ec));
            return;
        }
    }
    global_add3(grad, vi, gx, gy, gz);
}

// The three vertices of one face at once: the first probe of all three is
// issued before any result is waited for, further probes (rare) follow in a
// loop, then the nine fixed-point adds (or global float atomics for a
// vertex the table cannot take). New entries take the slot's scale: the
// largest exponent code among the three vertices that go to the table.
template <int HB = kHashBits>
__device__ __forceinline__ void vertex_add3(uint32_t* hkey, unsigned long long (*hval)[3],
                                            float* __restrict__ grad_verts, const int64_t (&vi)[3],
                                            const float (&g)[9], bool use_hash, int run_bits) {
    uint32_t code[3], h[3], cur[3];
    bool elig[3], zero[3];
    uint32_t slot_code = 0;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const float gx = g[3 * k], gy = g[3 * k + 1], gz = g[3 * k + 2];
        const float m = fmaxf(fabsf(gx), fmaxf(fabsf(gy), fabsf(gz)));   // fmaxf drops a NaN operand
        const bool nan = (gx != gx) || (gy != gy) || (gz != gz);
        code[k] = mag_code(m);
        zero[k] = code[k] == 0u && !nan;   // three zeros: nothing to add
        elig[k] = use_hash && !zero[k] && m <= 3.402823466e38f && !nan;
        slot_code = elig[k] ? max(slot_code, code[k]) : slot_code;
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const uint32_t id = (uint32_t)vi[k];
        h[k] = hash_slot0(id, HB, run_bits);
        cur[k] = elig[k] ? atomicCAS(&hkey[h[k]], kEmptyKey, id | (slot_code << kIdBits)) : 0u;
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        if (zero[k]) continue;
        int slot = -1;
        uint32_t ec = 0;
        if (elig[k]) slot = table_find<HB>(hkey, (uint32_t)vi[k], slot_code, h[k], cur[k], ec);
        if (slot >= 0 && code[k] <= ec + kFixAhead) {
            atomicAdd(&hval[slot][0], to_fixed(g[3 * k], ec));
            atomicAdd(&hval[slot][1], to_fixed(g[3 * k + 1], ec));
            atomicAdd(&hval[slot][2], to_fixed(g[3 * k + 2], ec));
        } else {
            global_add3(grad_verts, vi[k], g[3 * k], g[3 * k + 1], g[3 * k + 2]);
        }
    }
}

// Flushes a workgroup's table into grad (3 floats per id) with float atomics.
// Consecutive lanes take consecutive floats of the table (entry j / 3,
// coordinate j % 3), so that the three coordinates of an id, and the ids of
// neighbouring entries when they are neighbours in grad, reach memory in the
// same wave-wide atomic instruction: fewer cache lines per instruction than
// one entry per lane with a separate instruction per coordinate.
template <int HB = kHashBits>
__device__ __forceinline__ void flush_table(const uint32_t* hkey, const unsigned long long (*hval)[3],
                                            float* __restrict__ grad, int nthreads) {
    static_assert(HB <= 14, "division by multiplication");
    for (int j = threadIdx.x; j < 3 * (1 << HB); j += nthreads) {
        const int e = (int)(((uint32_t)j * 0xAAABu) >> 17);   // j / 3, exact for j < 3 * 2^14
        const int c = j - 3 * e;
        const uint32_t key = hkey[e];
        if (key != kEmptyKey) {
            const int64_t vid = (int64_t)(key & kIdMask);
            atomicAdd(&grad[3 * vid + c], from_fixed(hval[e][c], key >> kIdBits));
        }
    }
}

template <int HB = kHashBits>
__device__ __forceinline__ void clear_table(uint32_t* hkey, unsigned long long (*hval)[3], int nthreads) {
    for (int e = threadIdx.x; e < (1 << HB); e += nthreads) {
        hkey[e] = kEmptyKey;
        hval[e][0] = 0;
        hval[e][1] = 0;
        hval[e][2] = 0;
    }
}

}  // namespace dmr
