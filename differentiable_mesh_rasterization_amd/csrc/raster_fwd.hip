// Forward pass of the K-nearest-face rasterizer on gfx950.
//
// Coarse stage (gptget.net summary of "Accelerating 3D Deep Learning with
// PyTorch3D", "Methodology": a first stage selects the faces that can affect
// each pixel): every face is set up once and counted into the 16x16-pixel
// bins its conservative pixel box overlaps; an exclusive prefix sum turns
// the counts into per-bin list offsets, and a fill pass writes the face ids.
// Fine stage (nubint.ai review, "Proposed method": each pixel keeps its K
// nearest faces): one 256-thread workgroup per bin stages the bin's face
// records in LDS, every thread evaluates its pixel against them and keeps a
// sorted register top-K of (z, face) keys, then writes the K slots.
#include <algorithm>

#include "dmr_internal.h"

namespace dmr {

// ---------------------------------------------------------------------------
// zero fill (used instead of a memset so that the launch sequence holds
// kernels only)
// ---------------------------------------------------------------------------
__global__ void zero_i32x2(int32_t* p, int64_t n, int32_t* p2, int64_t n2) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t k = i; k < n; k += stride) p[k] = 0;
    for (int64_t k = i; k < n2; k += stride) p2[k] = 0;
}

// ---------------------------------------------------------------------------
// K1: per-face setup, culling and bin counting
// ---------------------------------------------------------------------------
// Bin counts are privatised in LDS for the faces of the block's "home" mesh
// (the mesh of its first face; packed faces of one mesh are contiguous, so
// that is nearly every face): LDS atomics per (face, bin), then one global
// atomic per non-empty (block, bin). Faces of other meshes, and images with
// more than kHistBins bins, count with global atomics directly.
constexpr int kHistBins = 4096;

__device__ __forceinline__ int64_t mesh_of(const int64_t* __restrict__ off, int64_t N, int64_t f) {
    int64_t lo = 0, hi = N - 1;
    while (lo < hi) {
        int64_t mid = (lo + hi) >> 1;
        if (off[mid + 1] > f) hi = mid; else lo = mid + 1;
    }
    return lo;
}

template <int TPB>
__global__ __launch_bounds__(TPB) void face_setup_count(
    const float* __restrict__ verts, int64_t V, const int64_t* __restrict__ faces, int64_t F,
    const int64_t* __restrict__ off, int64_t N, int32_t H, int32_t W, float blur, uint32_t settings,
    int32_t nbx, int32_t nby, FaceRec* __restrict__ recs, FaceBin* __restrict__ fbin,
    int32_t* __restrict__ rep_count, int32_t replicas, int64_t bins, int32_t* __restrict__ block_live,
    WsHeader* __restrict__ hdr) {
    __shared__ int32_t hist[kHistBins];
    int32_t* __restrict__ bin_count = rep_count + (int64_t)(blockIdx.x % (uint32_t)replicas) * bins;
    __shared__ int64_t home_s, home_lo, home_hi;
    __shared__ int32_t live_s;
    const int per_img = nbx * nby;
    const bool use_lds = per_img <= kHistBins;
    const int64_t f = (int64_t)blockIdx.x * TPB + threadIdx.x;
    // home mesh: the one holding the block's first face, found by all
    // threads at once (one round of loads instead of a binary search)
    const int64_t first = (int64_t)blockIdx.x * TPB;
    if (threadIdx.x == 0) {
        home_s = -1;
        live_s = 0;
    }
    __syncthreads();
    for (int64_t q = threadIdx.x; q < N; q += TPB)
        if (off[q] <= first && first < off[q + 1]) home_s = q;
    __syncthreads();
    if (threadIdx.x == 0) {
        int64_t h = home_s;
        if (h < 0) h = mesh_of(off, N, first);   // offsets not covering the face
        home_s = h;
        home_lo = off[h];
        home_hi = off[h + 1];
    }
    if (use_lds)
        for (int q = threadIdx.x; q < per_img; q += TPB) hist[q] = 0;
    __syncthreads();
    const int64_t home = home_s;
    bool live = false;
    FaceRec r{};
    if (f < F) {
        int32_t box_lo = 0x7fff7fff, box_hi = 0;   // empty box: lo > hi
        // the faces of a block nearly always belong to the mesh of its first
        const bool in_home = home_lo <= f && f < home_hi;
        const int64_t n = in_home ? home : mesh_of(off, N, f);
        bool ok = in_home || ((off[n] <= f) && (f < off[n + 1]));
        int64_t vi0 = faces[3 * f + 0], vi1 = faces[3 * f + 1], vi2 = faces[3 * f + 2];
        bool idx_ok = vi0 >= 0 && vi0 < V && vi1 >= 0 && vi1 < V && vi2 >= 0 && vi2 < V;
        if (!idx_ok) atomicOr(&hdr->flags, DMR_FLAG_BAD_VERTEX_INDEX);
        const bool ids32 = idx_ok && V <= (int64_t)INT32_MAX;
        r.v0 = ids32 ? (int32_t)vi0 : -1;
        r.v1 = ids32 ? (int32_t)vi1 : -1;
        r.v2 = ids32 ? (int32_t)vi2 : -1;
        float x0 = 0, y0 = 0, z0 = 0, x1 = 0, y1 = 0, z1 = 0, x2 = 0, y2 = 0, z2 = 0;
        if (idx_ok) {
            x0 = verts[3 * vi0]; y0 = verts[3 * vi0 + 1]; z0 = verts[3 * vi0 + 2];
            x1 = verts[3 * vi1]; y1 = verts[3 * vi1 + 1]; z1 = verts[3 * vi1 + 2];
            x2 = verts[3 * vi2]; y2 = verts[3 * vi2 + 1]; z2 = verts[3 * vi2 + 2];
        }
        float A = (x1 - x0) * (y2 - y0) - (y1 - y0) * (x2 - x0);
        // All depths <= 0 means z <= 0 at every pixel: the interpolation
        // weights are >= 0, so each product and each sum stays <= 0. With
        // perspective correction every depth must be > 0. Back faces (A > 0:
        // the normal's depth component is positive) are dropped on request.
        bool zpos = (z0 > 0.0f) || (z1 > 0.0f) || (z2 > 0.0f);
        if (settings & DMR_RASTER_PERSPECTIVE_CORRECT) zpos = (z0 > 0.0f) && (z1 > 0.0f) && (z2 > 0.0f);
        r.x0 = x0; r.y0 = y0; r.x1 = x1; r.y1 = y1; r.x2 = x2; r.y2 = y2;
        r.z0 = z0; r.z1 = z1; r.z2 = z2;
        r.invA = 1.0f / A;
        {
            float ux = x1 - x0, uy = y1 - y0;
            r.il0 = 1.0f / (ux * ux + uy * uy);
            ux = x2 - x1; uy = y2 - y1;
            r.il1 = 1.0f / (ux * ux + uy * uy);
            ux = x0 - x2; uy = y0 - y2;
            r.il2 = 1.0f / (ux * ux + uy * uy);
        }
        float xmin = fminf(x0, fminf(x1, x2)), xmax = fmaxf(x0, fmaxf(x1, x2));
        float ymin = fminf(y0, fminf(y1, y2)), ymax = fmaxf(y0, fmaxf(y1, y2));
        const bool back = (settings & DMR_RASTER_CULL_BACKFACES) && A > 0.0f;
        if (ok && idx_ok && A != 0.0f && zpos && !back) {
            // Conservative pixel box: the face's box grown by the blur radius
            // and by a margin far above the rounding of the inclusion tests.
            float rb = sqrtf(blur);
            float mag = fmaxf(1.0f, fmaxf(fmaxf(fabsf(xmin), fabsf(xmax)), fmaxf(fabsf(ymin), fabsf(ymax))));
            float m = 1e-5f * mag + 1e-5f * rb;
            float xl = xmin - rb - m, xh = xmax + rb + m;
            float yl = ymin - rb - m, yh = ymax + rb + m;
            float jl = ceilf(((xl + 1.0f) * (float)W - 1.0f) * 0.5f);
            float jh = floorf(((xh + 1.0f) * (float)W - 1.0f) * 0.5f);
            float il = ceilf(((yl + 1.0f) * (float)H - 1.0f) * 0.5f);
            float ih = floorf(((yh + 1.0f) * (float)H - 1.0f) * 0.5f);
            jl = fmaxf(jl, 0.0f);
            il = fmaxf(il, 0.0f);
            jh = fminf(jh, (float)(W - 1));
            ih = fminf(ih, (float)(H - 1));
            if (jl <= jh && il <= ih) {
                int j0 = (int)jl, j1 = (int)jh, i0 = (int)il, i1 = (int)ih;
                box_lo = j0 | (i0 << 16);
                box_hi = j1 | (i1 << 16);
                live = true;
                const bool local = use_lds && n == home;
                int32_t* cnt = bin_count + n * per_img;
                for (int by = i0 / kBin; by <= i1 / kBin; ++by)
                    for (int bx = j0 / kBin; bx <= j1 / kBin; ++bx) {
                        if (local) atomicAdd(&hist[by * nbx + bx], 1);
                        else atomicAdd(&cnt[by * nbx + bx], 1);
                    }
            }
        }
        FaceBin fb;
        fb.box_lo = box_lo;
        fb.box_hi = box_hi;
        fb.mesh = (int32_t)n;
        fb.zmin_bits = __float_as_uint(fminf(z0, fminf(z1, z2)));
        fbin[f] = fb;
    }
    {
        // Records are stored a lane quad at a time: after the transpose lane
        // p of the quad writes piece p of the quad's four records, so that a
        // store instruction writes whole 64-byte records (16 per wave)
        // instead of a 16-byte piece of 64 records (16.8 against 21.5 us on
        // 16 meshes of 450,560 faces).
        int w[16];
        const int* rw = reinterpret_cast<const int*>(&r);
#pragma unroll
        for (int i = 0; i < 16; ++i) w[i] = rw[i];
        quad_transpose(w);
        const int p = threadIdx.x & 3;
        const int64_t fq = f - p;   // the quad's first face
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (fq + k < F)
                reinterpret_cast<int4*>(recs + fq + k)[p] = make_int4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]);
    }
    // live-face count: one LDS atomic per wave, one plain store per block
    // (the scan kernel adds the per-block counts)
    unsigned long long m = __ballot(live);
    if ((threadIdx.x & 63) == 0 && m) atomicAdd(&live_s, (int32_t)__popcll(m));
    __syncthreads();
    if (threadIdx.x == 0) block_live[blockIdx.x] = live_s;
    if (use_lds) {
        int32_t* cnt = bin_count + home * per_img;
        for (int q = threadIdx.x; q < per_img; q += TPB) {
            const int32_t c = hist[q];
            if (c) atomicAdd(&cnt[q], c);
        }
    }
}

// ---------------------------------------------------------------------------
// K2: exclusive prefix sum of the bin counts (one workgroup), header stats,
// the fill cursors, the order in which the sort visits the bins, and the
// work items of the fine pass. Both orders put the heaviest work first (counting
// sort on floor(log2(weight)) buckets), so that long workgroups start early
// and do not form the kernel's tail. A bin with at least kSplitMin faces
// (when K allows) gives four quarter items of a quarter of its weight.
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 1024;
constexpr int kOrderBuckets = 33;

__device__ __forceinline__ int order_bucket(int32_t c) {
    // descending: bucket 0 holds the largest weights, bucket 32 the empty bins
    return c <= 0 ? 32 : __clz(c);
}

// Exclusive prefix sum over a kScanThreads workgroup (wave scans, then the
// wave totals scanned by the first wave).
__device__ __forceinline__ int64_t block_exclusive_sum64(int64_t v, int64_t* wsum, int64_t& total) {
    constexpr int kWaves = kScanThreads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int64_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int64_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (wave == 0) {
        int64_t y = lane < kWaves ? wsum[lane] : 0;
        const int64_t y0 = y;
#pragma unroll
        for (int d = 1; d < kWaves; d <<= 1) {
            const int64_t z = __shfl_up(y, d, 64);
            if (lane >= d) y += z;
        }
        if (lane < kWaves) wsum[lane] = y - y0;
        if (lane == kWaves - 1) wsum[kWaves] = y;
    }
    __syncthreads();
    const int64_t r = wsum[wave] + x - v;
    total = wsum[kWaves];
    __syncthreads();
    return r;
}

// Sums of two values over a kScanThreads workgroup (wave sums, one LDS
// atomic per wave and value, one barrier).
__device__ __forceinline__ void block_sum64x2(int64_t& a, int64_t& b, unsigned long long* acc) {
    for (int d = 32; d >= 1; d >>= 1) {
        a += __shfl_xor(a, d, 64);
        b += __shfl_xor(b, d, 64);
    }
    if ((threadIdx.x & 63) == 0) {
        atomicAdd(&acc[0], (unsigned long long)a);
        atomicAdd(&acc[1], (unsigned long long)b);
    }
    __syncthreads();
    a = (int64_t)acc[0];
    b = (int64_t)acc[1];
}

// Lanes below this one among the lanes of mask m.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Adds one per active lane to the LDS counter arr[key] and returns each
// active lane's place (the counter's value before its unit). The lanes that
// share the key of the first active lane add with one atomic (the weight
// buckets of neighbouring bins are mostly the same, and a wave's atomics on
// one LDS address serialise); the others add one each.
__device__ __forceinline__ int32_t lds_take(int32_t* arr, int32_t key, bool active) {
    const uint64_t act = __ballot(active);
    if (act == 0) return 0;
    const int lane = threadIdx.x & 63;
    const int leader = __builtin_ctzll(act);
    const int32_t k = __builtin_amdgcn_readlane(key, leader);
    const bool same = active && key == k;
    const uint64_t m = __ballot(same);
    int32_t base = 0, own = 0;
    if (lane == leader) base = atomicAdd(&arr[k], (int32_t)__popcll(m));
    if (active && !same) own = atomicAdd(&arr[key], 1);
    base = __builtin_amdgcn_readlane(base, leader);
    return same ? base + lanes_below(m) : own;
}

// Loads v[g..g+3] (entries at or past `end` read as 0): one 16-byte load
// when the four are whole and aligned.
__device__ __forceinline__ void load4(const int32_t* __restrict__ v, int64_t g, int64_t end, bool vec, int32_t (&c)[4]) {
    if (vec && g + 4 <= end) {
        const int4 x = *reinterpret_cast<const int4*>(v + g);
        c[0] = x.x; c[1] = x.y; c[2] = x.z; c[3] = x.w;
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) c[k] = g + k < end ? v[g + k] : 0;
    }
}
__device__ __forceinline__ void store4(int32_t* __restrict__ v, int64_t g, int64_t end, bool vec, const int32_t (&c)[4]) {
    if (vec && g + 4 <= end) {
        *reinterpret_cast<int4*>(v + g) = make_int4(c[0], c[1], c[2], c[3]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (g + k < end) v[g + k] = c[k];
    }
}

__global__ __launch_bounds__(kScanThreads) void bin_scan(int32_t* __restrict__ count,
                                                         int64_t* __restrict__ offset,
                                                         int32_t* __restrict__ rep, int32_t replicas,
                                                         int32_t* __restrict__ perm, uint32_t* __restrict__ items,
                                                         int64_t bins, int32_t allow_split, int32_t sort_min,
                                                         const int32_t* __restrict__ block_live,
                                                         int64_t nblocks, int64_t capacity, size_t base_bytes,
                                                         WsHeader* __restrict__ hdr) {
    __shared__ int64_t wsum[kScanThreads / 64 + 1];
    __shared__ unsigned long long acc[2];
    __shared__ int32_t bucket_n[kOrderBuckets];
    __shared__ int32_t bucket_at[kOrderBuckets];
    __shared__ int32_t item_n[kOrderBuckets];
    __shared__ int32_t item_at[kOrderBuckets];
    const int t = threadIdx.x;
    if (t < kOrderBuckets) {
        bucket_n[t] = 0;
        item_n[t] = 0;
    }
    if (t < 2) acc[t] = 0;
    // Thread t owns the bins [b0, b1), in groups of four (16-byte accesses
    // where bins is a multiple of four, so that every copy's groups are
    // aligned).
    const int64_t per = (((bins + kScanThreads - 1) / kScanThreads) + 3) & ~(int64_t)3;
    const int64_t b0 = min(bins, (int64_t)t * per);
    const int64_t b1 = min(bins, b0 + per);
    const bool vec = (bins & 3) == 0;
    // the live-face counts of the setup blocks, loaded ahead
    int64_t lv = 0;
    for (int64_t q = t; q < nblocks; q += kScanThreads) lv += block_live[q];
    __syncthreads();   // the bucket counters are zero
    // Each bin's count is the sum of its copies; their running sums become
    // the copies' fill cursors (copy r's faces follow those of copies < r).
    // The bins and items are counted into their weight buckets.
    int64_t s = 0;
    for (int64_t g = b0; g < b1; g += 4) {
        int32_t cr[kCountReplicas][4];
#pragma unroll
        for (int r = 0; r < kCountReplicas; ++r) {
            if (r < replicas) load4(rep + (int64_t)r * bins, g, b1, vec, cr[r]);
        }
        int32_t c[4] = {0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < kCountReplicas; ++r) {
            if (r < replicas) {
                int32_t cur[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    cur[k] = c[k];
                    c[k] += cr[r][k];
                }
                store4(rep + (int64_t)r * bins, g, b1, vec, cur);
            }
        }
        store4(count, g, b1, vec, c);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const bool valid = g + k < b1;
            s += c[k];
            const bool split = valid && allow_split && c[k] >= kSplitMin;
            lds_take(bucket_n, order_bucket(c[k]), valid);
            lds_take(item_n, order_bucket(c[k]), valid && !split);
            if (split) atomicAdd(&item_n[order_bucket(c[k] / 4)], 4);
        }
    }
    int64_t total = 0;
    int64_t run = block_exclusive_sum64(s, wsum, total);   // synchronises: the bucket counts are complete
    if (t < 64) {
        // bucket starts: exclusive sums over the kOrderBuckets buckets (first wave)
        int x = t < kOrderBuckets ? bucket_n[t] : 0;
        int y = t < kOrderBuckets ? item_n[t] : 0;
        const int x0 = x, y0 = y;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int xs = __shfl_up(x, d, 64);
            const int ys = __shfl_up(y, d, 64);
            if (t >= d) {
                x += xs;
                y += ys;
            }
        }
        if (t < kOrderBuckets) {
            bucket_at[t] = x - x0;
            item_at[t] = y - y0;
        }
        if (t == kOrderBuckets - 1) hdr->fine_items = y;
        // every bin with more than sort_min faces lies in a bucket up to
        // that of sort_min + 1: the sort visits the order's prefix of those
        // buckets
        if (t == order_bucket(sort_min + 1)) hdr->sort_bins = x;
    }
    __syncthreads();
    // list offsets, the sort order and the fine pass's items
    int64_t over = 0;
    for (int64_t g = b0; g < b1; g += 4) {
        int32_t c[4];
        load4(count, g, b1, vec, c);   // this thread's own stores above
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t b = g + k;
            const bool valid = b < b1;
            if (valid) {
                offset[b] = run;
                if (run + c[k] > capacity) ++over;
                run += c[k];
            }
            const bool split = valid && allow_split && c[k] >= kSplitMin;
            const int32_t pos = lds_take(bucket_at, order_bucket(c[k]), valid);
            const int32_t at = lds_take(item_at, order_bucket(c[k]), valid && !split);
            const uint32_t code = (uint32_t)b << 3;
            if (valid) perm[pos] = (int32_t)b;
            if (valid && !split) items[at] = code | (uint32_t)kItemWhole;
            if (split) {
                const int a4 = atomicAdd(&item_at[order_bucket(c[k] / 4)], 4);
                for (int q = 0; q < 4; ++q) items[a4 + q] = code | (uint32_t)q;
            }
        }
    }
    int64_t o = over, live = lv;
    block_sum64x2(o, live, acc);
    if (t == 0) {
        hdr->live_faces = live;
        offset[bins] = total;
        hdr->bin_entries = total;
        hdr->bin_capacity = capacity;
        hdr->bins = bins;
        hdr->overflow_bins = o;
        hdr->required_bytes = (int64_t)base_bytes + total * (int64_t)sizeof(int32_t);
    }
}

// ---------------------------------------------------------------------------
// K3: bin fill
// ---------------------------------------------------------------------------
// Same privatisation as K1: the block counts its home-mesh entries per bin
// in LDS, reserves each bin's range with one global atomic (a thread's
// atomics for its bins are all issued before any result is waited for),
// then places its faces inside the reserved ranges with LDS atomics on the
// same counters, which now hold the ranges' starts. The order of
// faces inside a bin list does not affect any result.
template <int TPB>
__global__ __launch_bounds__(TPB) void bin_fill(const FaceBin* __restrict__ fbin, int64_t F,
                                                          const int32_t* __restrict__ count,
                                                          const int64_t* __restrict__ offset,
                                                          int32_t* __restrict__ rep, int32_t replicas, int64_t bins,
                                                          int32_t* __restrict__ entries, int64_t capacity,
                                                          int32_t nbx, int32_t nby) {
    // this workgroup's copy of the cursors (the copy its setup workgroup
    // counted into)
    int32_t* __restrict__ cursor = rep + (int64_t)(blockIdx.x % (uint32_t)replicas) * bins;
    __shared__ int32_t hist[kHistBins];   // counts, then cursors
    __shared__ int64_t home_s;
    const int per_img = nbx * nby;
    const bool use_lds = per_img <= kHistBins;
    const int64_t f = (int64_t)blockIdx.x * TPB + threadIdx.x;
    if (threadIdx.x == 0) home_s = fbin[(int64_t)blockIdx.x * TPB].mesh;
    if (use_lds)
        for (int q = threadIdx.x; q < per_img; q += TPB) hist[q] = 0;
    __syncthreads();
    const int64_t home = home_s;
    bool live = false;
    int j0 = 0, i0 = 0, j1 = -1, i1 = -1;
    int64_t n = 0;
    if (f < F) {
        const FaceBin fb = fbin[f];
        j0 = fb.box_lo & 0xffff; i0 = fb.box_lo >> 16; j1 = fb.box_hi & 0xffff; i1 = fb.box_hi >> 16;
        live = j0 <= j1 && i0 <= i1;
        n = fb.mesh;
    }
    const bool local = live && use_lds && n == home;
    if (local)
        for (int by = i0 / kBin; by <= i1 / kBin; ++by)
            for (int bx = j0 / kBin; bx <= j1 / kBin; ++bx) atomicAdd(&hist[by * nbx + bx], 1);
    if (use_lds) {
        __syncthreads();
        const int64_t hb = home * per_img;
        constexpr int kPerT = kHistBins / TPB;
        int32_t c[kPerT], r[kPerT];
#pragma unroll
        for (int k = 0; k < kPerT; ++k) {
            const int q = threadIdx.x + k * TPB;
            c[k] = q < per_img ? hist[q] : 0;
        }
#pragma unroll
        for (int k = 0; k < kPerT; ++k) {
            const int q = threadIdx.x + k * TPB;
            r[k] = c[k] ? atomicAdd(&cursor[hb + q], c[k]) : 0;
        }
#pragma unroll
        for (int k = 0; k < kPerT; ++k) {
            const int q = threadIdx.x + k * TPB;
            if (q < per_img) hist[q] = r[k];   // the block's start in the bin's range
        }
        __syncthreads();
    }
    if (!live) return;
    const int64_t binbase = n * per_img;
    for (int by = i0 / kBin; by <= i1 / kBin; ++by)
        for (int bx = j0 / kBin; bx <= j1 / kBin; ++bx) {
            const int q = by * nbx + bx;
            const int64_t gb = binbase + q;
            const int64_t o = offset[gb];
            int32_t pos;
            if (local) pos = atomicAdd(&hist[q], 1);
            else pos = atomicAdd(&cursor[gb], 1);
            if (o + count[gb] <= capacity) entries[o + pos] = (int32_t)f;
        }
}

// ---------------------------------------------------------------------------
// K3b: order each bin's list by the faces' smallest vertex depth
// ---------------------------------------------------------------------------
// A bucket sort in LDS (256 buckets over the bin's zmin range, O(n)) puts
// near faces first. The order is approximate inside a bucket, so the exact
// guarantee the fine pass relies on is stored beside it: for every round of
// 256 list positions, the smallest zmin over that round and all later ones.
// A pixel whose last key lies below a round's bound can skip the rest of the
// list. Lists longer than kSortMax are left as they are (their bound is -inf).
constexpr int kSortThreads = 256;
constexpr int kSortBuckets = 1024;

__device__ __forceinline__ uint32_t float_order_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_bits_float(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

constexpr int kSortPer = kSortMax / kSortThreads;   // list entries per thread

// Exclusive prefix sum over a 256-thread workgroup (wave scans, then the
// four wave totals).
__device__ __forceinline__ int block256_exclusive_sum(int v, int* wsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < kSortThreads / 64; ++w) before += (w < wave) ? wsum[w] : 0;
    __syncthreads();
    return before + x - v;
}

// Sorts one list of at most PER * kSortThreads entries over NB buckets (the
// list held in registers: entry q = t + kSortThreads * i).
template <int PER, int NB>
__device__ __forceinline__ void sort_list(const FaceBin* __restrict__ fbin, int32_t* __restrict__ entries, int64_t o,
                                          int32_t cnt, float* __restrict__ lb, int32_t* hist, uint32_t* bmin,
                                          int* wsum, uint32_t* wmin, uint32_t& lo_s, uint32_t& hi_s,
                                          uint32_t* rmin) {
    constexpr int BPT = NB / kSortThreads;   // buckets per thread
    static_assert(NB % kSortThreads == 0 && NB <= kSortBuckets, "whole buckets per sort thread");
    const int t = threadIdx.x;
    if (t == 0) {
        lo_s = 0xffffffffu;
        hi_s = 0u;
    }
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        hist[t * BPT + i] = 0;
        bmin[t * BPT + i] = 0xffffffffu;
    }
    if (t < kRoundsPerBin) rmin[t] = 0xffffffffu;
    int32_t id[PER];
    uint32_t zb[PER];   // order bits of zmin
    uint32_t mylo = 0xffffffffu, myhi = 0u;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int q = t + kSortThreads * i;
        id[i] = q < cnt ? entries[o + q] : 0;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int q = t + kSortThreads * i;
        zb[i] = 0;
        if (q < cnt) {
            zb[i] = float_order_bits(__uint_as_float(fbin[id[i]].zmin_bits));
            mylo = min(mylo, zb[i]);
            myhi = max(myhi, zb[i]);
        }
    }
    __syncthreads();
    atomicMin(&lo_s, mylo);
    atomicMax(&hi_s, myhi);
    __syncthreads();
    const float lo = order_bits_float(lo_s), hi = order_bits_float(hi_s);
    const float scale = (hi > lo) ? (float)NB / (hi - lo) : 0.0f;
    int bk[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        int k = (int)((order_bits_float(zb[i]) - lo) * scale);
        k = k < 0 ? 0 : (k >= NB ? NB - 1 : k);
        bk[i] = k;
        if (t + kSortThreads * i < cnt) {
            atomicAdd(&hist[k], 1);
            atomicMin(&bmin[k], zb[i]);
        }
    }
    __syncthreads();
    // Bucket starts (each thread owns BPT consecutive buckets), and the
    // rounds' depth bounds: round r's bound is the smallest zmin of the
    // bucket holding list position 256 r and of every later bucket, a lower
    // bound on the zmin of every face from round r on (the sorted list
    // holds no earlier bucket past that position). The buckets' minima come
    // from atomics spread over all buckets; per-round atomics on at most 16
    // counters had serialised the whole wave on one address.
    {
        int c[BPT];
        uint32_t sm[BPT];   // suffix minima over this thread's buckets
        int local = 0;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            c[i] = hist[t * BPT + i];
            local += c[i];
            sm[i] = bmin[t * BPT + i];
        }
#pragma unroll
        for (int i = BPT - 2; i >= 0; --i) sm[i] = min(sm[i], sm[i + 1]);
        // smallest bucket minimum of the threads after this one (a reverse
        // scan: within the wave, then over the four waves)
        const int lane = t & 63, wave = t >> 6;
        uint32_t x = sm[0];
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t y = __shfl_down(x, d, 64);
            if (lane + d < 64) x = min(x, y);
        }
        if (lane == 0) wmin[wave] = x;
        uint32_t after = __shfl_down(x, 1, 64);   // suffix from the next lane
        if (lane == 63) after = 0xffffffffu;
        int run = block256_exclusive_sum(local, wsum);   // synchronises: wmin is complete
#pragma unroll
        for (int w = 0; w < kSortThreads / 64; ++w)
            if (w > wave) after = min(after, wmin[w]);
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            // the rounds starting inside this bucket (a long bucket can hold
            // several round starts)
            for (int r = (run + kFineThreads - 1) / kFineThreads;
                 c[i] > 0 && r * kFineThreads < run + c[i] && r < kRoundsPerBin; ++r)
                rmin[r] = min(sm[i], after);
            hist[t * BPT + i] = run;
            run += c[i];
        }
    }
    __syncthreads();
    // Every entry has been read: scatter the ids to their sorted places in
    // the list.
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (t + kSortThreads * i < cnt) {
            const int pos = atomicAdd(&hist[bk[i]], 1);
            entries[o + pos] = id[i];
        }
    }
    __syncthreads();
    // round r's bound (a round past the list has none: +inf)
    if (t < kRoundsPerBin) lb[t] = (rmin[t] == 0xffffffffu) ? __builtin_inff() : order_bits_float(rmin[t]);
}

__global__ __launch_bounds__(kSortThreads) void bin_sort(const FaceBin* __restrict__ fbin,
                                                         const int32_t* __restrict__ count,
                                                         const int64_t* __restrict__ offset,
                                                         const int32_t* __restrict__ perm,
                                                         int32_t* __restrict__ entries, int64_t capacity,
                                                         int32_t sort_min, const WsHeader* __restrict__ hdr,
                                                         float* __restrict__ round_lb) {
    __shared__ int32_t hist[kSortBuckets];
    __shared__ uint32_t bmin[kSortBuckets];
    __shared__ int wsum[kSortThreads / 64];
    __shared__ uint32_t wmin[kSortThreads / 64];
    __shared__ uint32_t lo_s, hi_s;
    __shared__ uint32_t rmin[kRoundsPerBin];
    // the bins past the order's prefix of sortable ones end at once
    if ((int32_t)blockIdx.x >= hdr->sort_bins) return;
    const int64_t b = perm[blockIdx.x];
    const int32_t cnt = count[b];
    const int64_t o = offset[b];
    float* lb = round_lb + b * kRoundsPerBin;
    if (!list_sorted(o, cnt, capacity, sort_min)) return;   // the fine passes read no bound of it
    // short lists (the common case) take a variant with fewer registers and
    // buckets
    if (cnt <= 2 * kSortThreads)
        sort_list<2, kSortThreads>(fbin, entries, o, cnt, lb, hist, bmin, wsum, wmin, lo_s, hi_s, rmin);
    else if (cnt <= 4 * kSortThreads)
        sort_list<4, kSortBuckets>(fbin, entries, o, cnt, lb, hist, bmin, wsum, wmin, lo_s, hi_s, rmin);
    else
        sort_list<kSortPer, kSortBuckets>(fbin, entries, o, cnt, lb, hist, bmin, wsum, wmin, lo_s, hi_s, rmin);
}

// ---------------------------------------------------------------------------
// K4: fine rasterization with a register top-K
// ---------------------------------------------------------------------------
// Keys of the top-K lists. A list is ordered by (depth, face), i.e. by the
// 64-bit pattern (depth bits << 32) | face of a depth > 0. Read as a binary64
// number such a pattern is finite, non-negative and not a NaN, and numeric
// order is pattern order, so one v_min_f64 or v_max_f64 moves a key; +inf
// marks an empty slot. The two instructions are written out because the
// compiler's fmin and fmax first quiet both operands (one more instruction
// per operand at every step of the chain below).
constexpr uint64_t kEmptyKeyBits = 0x7ff0000000000000ull;

__device__ __forceinline__ double empty_key() { return __longlong_as_double((long long)kEmptyKeyBits); }
__device__ __forceinline__ double make_key(float z, int32_t face) {
    return __hiloint2double((int)__float_as_uint(z), face);
}
__device__ __forceinline__ uint64_t key_bits(double k) { return (uint64_t)__double_as_longlong(k); }
__device__ __forceinline__ double key_min(double a, double b) {
    double r;
    asm("v_min_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Push k through the ascending list key[0..KMAX-1]: each slot keeps the
// smaller of its key and the carried one and carries the larger on, so the
// list ends as the KMAX smallest of its keys and k.
template <int KMAX>
__device__ __forceinline__ void topk_push(double (&key)[KMAX], double k) {
#pragma unroll
    for (int q = 0; q < KMAX; ++q) {
        double hi;
        asm("v_max_f64 %0, %1, %2" : "=v"(hi) : "v"(key[q]), "v"(k));
        asm("v_min_f64 %0, %0, %1" : "+v"(key[q]) : "v"(k));
        k = hi;
    }
}

// Squared distance from the pixel to the segment a->b, given dxa = ax - px,
// dya = ay - py and the segment vector (ux, uy). The conventions write the
// clamp parameter with q = p - a = -(dxa, dya); negation is exact in
// binary32, so t and the residual below equal theirs up to sign, and the
// squared length is bit-identical.
__device__ __forceinline__ float edge_dist2(float dxa, float dya, float ux, float uy, float il) {
    float t = -((dxa * ux + dya * uy) * il);
    t = t < 0.0f ? 0.0f : t;
    t = t > 1.0f ? 1.0f : t;
    const float rx = dxa + t * ux;
    const float ry = dya + t * uy;
    return rx * rx + ry * ry;
}

// Key of one (pixel, face) pair, or +inf when the pair is not a candidate
// or its key is not below `bound`, with the binary32 operations of the
// conventions in their fixed order. There are no branches: the lanes of a
// wave evaluate unrelated pairs, and most pairs lie outside their triangle
// and need the three edge distances anyway.
template <bool PERSP>
__device__ __forceinline__ double pair_key(const FaceRec& r, int32_t face, float px, float py, float blur,
                                           double bound) {
    const float dx0 = r.x0 - px, dy0 = r.y0 - py;
    const float dx1 = r.x1 - px, dy1 = r.y1 - py;
    const float dx2 = r.x2 - px, dy2 = r.y2 - py;
    const float w0 = dx1 * dy2 - dy1 * dx2;
    const float w1 = dx2 * dy0 - dy2 * dx0;
    const float w2 = dx0 * dy1 - dy0 * dx1;
    const float b0 = w0 * r.invA, b1 = w1 * r.invA, b2 = w2 * r.invA;
    const FaceBox bb = face_box(r);
    const bool in_box = (px >= bb.xmin) && (px <= bb.xmax) && (py >= bb.ymin) && (py <= bb.ymax);
    const bool inside = in_box && (b0 > 0.0f) && (b1 > 0.0f) && (b2 > 0.0f);
    float c0 = b0 < 0.0f ? 0.0f : b0;
    float c1 = b1 < 0.0f ? 0.0f : b1;
    float c2 = b2 < 0.0f ? 0.0f : b2;
    c0 = c0 > 1.0f ? 1.0f : c0;
    c1 = c1 > 1.0f ? 1.0f : c1;
    c2 = c2 > 1.0f ? 1.0f : c2;
    float z;
    if (PERSP) {
        float n0, n1, n2;
        persp_weights(c0, c1, c2, r.z0, r.z1, r.z2, n0, n1, n2);
        const float invD = 1.0f / ((n0 + n1) + n2);
        z = ((n0 * invD) * r.z0 + (n1 * invD) * r.z1) + (n2 * invD) * r.z2;
    } else {
        const float S = (c0 + c1) + c2;
        const float invS = 1.0f / S;
        z = ((c0 * invS) * r.z0 + (c1 * invS) * r.z1) + (c2 * invS) * r.z2;
    }
    // Outside the triangle, d < blur fails for every blur <= 0 (d is a sum
    // of squares, >= 0 or NaN), so the distances are only needed with a
    // positive blur (a test on a kernel argument: uniform, no divergence).
    bool near = false;
    if (blur > 0.0f) {
        const float d0 = edge_dist2(dx0, dy0, r.x1 - r.x0, r.y1 - r.y0, r.il0);
        const float d1 = edge_dist2(dx1, dy1, r.x2 - r.x1, r.y2 - r.y1, r.il1);
        const float d2 = edge_dist2(dx2, dy2, r.x0 - r.x2, r.y0 - r.y2, r.il2);
        float d = d0;
        d = d1 < d ? d1 : d;
        d = d2 < d ? d2 : d;
        near = d < blur;
    }
    const bool cand = (inside || near) && (z > 0.0f);
    const double kk = make_key(z, face);
    return (cand && kk < bound) ? kk : empty_key();
}

// Outputs of a kept (pixel, face) pair: the returned barycentrics and the
// signed squared distance (negative inside), with the operations of
// eval_pair in the same order; the distance is edge_dist2's, which equals
// eval_pair's bit for bit.
template <bool PERSP>
__device__ __forceinline__ void slot_outputs(const FaceRec& r, float px, float py, bool unclipped, float& o0,
                                             float& o1, float& o2, float& sd) {
    const float dx0 = r.x0 - px, dy0 = r.y0 - py;
    const float dx1 = r.x1 - px, dy1 = r.y1 - py;
    const float dx2 = r.x2 - px, dy2 = r.y2 - py;
    const float w0 = dx1 * dy2 - dy1 * dx2;
    const float w1 = dx2 * dy0 - dy2 * dx0;
    const float w2 = dx0 * dy1 - dy0 * dx1;
    const float b0 = w0 * r.invA, b1 = w1 * r.invA, b2 = w2 * r.invA;
    const FaceBox bb = face_box(r);
    const bool in_box = (px >= bb.xmin) && (px <= bb.xmax) && (py >= bb.ymin) && (py <= bb.ymax);
    const bool inside = in_box && (b0 > 0.0f) && (b1 > 0.0f) && (b2 > 0.0f);
    float c0 = b0 < 0.0f ? 0.0f : b0;
    float c1 = b1 < 0.0f ? 0.0f : b1;
    float c2 = b2 < 0.0f ? 0.0f : b2;
    c0 = c0 > 1.0f ? 1.0f : c0;
    c1 = c1 > 1.0f ? 1.0f : c1;
    c2 = c2 > 1.0f ? 1.0f : c2;
    if (PERSP) {
        float n0, n1, n2;
        if (unclipped) persp_weights(b0, b1, b2, r.z0, r.z1, r.z2, n0, n1, n2);
        else persp_weights(c0, c1, c2, r.z0, r.z1, r.z2, n0, n1, n2);
        const float inv = 1.0f / ((n0 + n1) + n2);
        o0 = n0 * inv;
        o1 = n1 * inv;
        o2 = n2 * inv;
    } else if (unclipped) {
        o0 = b0;
        o1 = b1;
        o2 = b2;
    } else {
        const float invS = 1.0f / ((c0 + c1) + c2);
        o0 = c0 * invS;
        o1 = c1 * invS;
        o2 = c2 * invS;
    }
    const float d0 = edge_dist2(dx0, dy0, r.x1 - r.x0, r.y1 - r.y0, r.il0);
    const float d1 = edge_dist2(dx1, dy1, r.x2 - r.x1, r.y2 - r.y1, r.il1);
    const float d2 = edge_dist2(dx2, dy2, r.x0 - r.x2, r.y0 - r.y2, r.il2);
    float d = d0;
    d = d1 < d ? d1 : d;
    d = d2 < d ? d2 : d;
    sd = inside ? -d : d;
}

// Smallest of the keys held by the four lanes of an aligned lane quad.
__device__ __forceinline__ double quad_min(double x) {
    x = key_min(x, __shfl_xor(x, 1));
    return key_min(x, __shfl_xor(x, 2));
}

// Merge the sorted lists of the lane `mask` apart into this lane's: both
// lanes end with the K smallest keys of the two (disjoint) lists.
template <int KMAX>
__device__ __forceinline__ void merge_with_lane(double (&key)[KMAX], int mask) {
    double other[KMAX];
#pragma unroll
    for (int q = 0; q < KMAX; ++q) other[q] = __shfl_xor(key[q], mask);
#pragma unroll
    for (int q = 0; q < KMAX; ++q)
        if (other[q] < key[KMAX - 1]) topk_push<KMAX>(key, other[q]);
}

// Exclusive prefix sum over a 256-thread workgroup, and the total.
__device__ __forceinline__ int block256_exclusive_sum_total(int v, int* wsum, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kFineThreads / 64; ++w) {
        const int c = wsum[w];
        before += (w < wave) ? c : 0;
        all += c;
    }
    __syncthreads();
    total = all;
    return before + x - v;
}

// Padding of `rows` rows of an output array whose slots are all empty: the
// run of run_words 32-bit words of row r starts at word first + r *
// row_words and takes `pattern` (all ones for an index of -1, the bits of
// -1.0f for a value). Sixteen threads share a row, with 16-byte stores when
// the array and its rows are 16-byte aligned.
__device__ __forceinline__ void pad_rows(uint32_t* __restrict__ base, int64_t first, int64_t row_words, int rows,
                                         int run_words, uint32_t pattern) {
    const int r = threadIdx.x >> 4, c0 = threadIdx.x & 15;
    if (r >= rows) return;
    uint32_t* row = base + first + (int64_t)r * row_words;
    const bool aligned = (reinterpret_cast<uintptr_t>(base) & 15) == 0 && (row_words & 3) == 0;
    int c = c0;
    if (aligned) {
        const int chunks = run_words >> 2;
        const uint4 v = make_uint4(pattern, pattern, pattern, pattern);
        uint4* row4 = reinterpret_cast<uint4*>(row);
        for (; c < chunks; c += 16) row4[c] = v;
        c = (chunks << 2) + c0;
    }
    for (; c < run_words; c += 16) row[c] = pattern;
}

// A face record staged piece-major in LDS.
__device__ __forceinline__ FaceRec staged_rec(const int4* s, uint32_t u) {
    FaceRec r;
    int4* d = reinterpret_cast<int4*>(&r);
#pragma unroll
    for (int p = 0; p < 4; ++p) d[p] = s[p * kFineThreads + u];
    return r;
}

// Pixel centre and current pruning bound of one owner of the fine pass.
struct OwnerRec {
    float px, py;
    double bound;
};

// Fine pass: one workgroup per work item, in the heaviest-first order of
// bin_scan (the grid has room for four items per bin; the workgroups past
// the item count return at once).
//
// Each thread is an owner: a whole-bin item gives each thread one pixel of
// the 16x16 bin (each wave owning an 8x8 quarter, whose pixels' face sets
// overlap more than those of four full bin rows would). A quarter item
// gives each of its 64 pixels four owners (an aligned lane quad, the pixels
// of a wave forming a 4x4 block); owner s of the quad takes the faces of
// list positions 64s..64s+63 of every round and keeps its own top-K, the
// quad shares the smallest of the four K-th keys as its pruning bound (the
// K-th of any owner bounds the K-th of their union from above), and the
// four lists are merged at the end.
//
// Each round stages up to 256 of the bin's faces in LDS (one per thread),
// piece-major (the 16-byte piece p of every record together), so that the
// lanes of a wave reading the records of unrelated faces spread over the
// LDS banks. Every wave then describes the pixel boxes of its 64 faces with ballots:
// colmask[c] has bit u set when face slot u's box covers bin column c, and
// rowmask[r] likewise for bin row r. An owner's candidate faces in the
// round are colmask[its column] & rowmask[its row].
//
// The candidate pairs are evaluated pair-parallel: their number differs
// from pixel to pixel, so one lane per pixel would leave most lanes of a
// wave idle. Per window of at most kPairWin pairs, the owners write their
// pairs' codes (face slot, owner) to positions given by a workgroup prefix
// sum; all 256 threads evaluate the window's pairs, moving the keys that
// pass to the front of their owner's positions; and each owner pushes
// those keys into its register top-K. A pair is tested against its owner's
// bound from the window's start, which is at least the owner's current
// one, so a key that passes may still fall off the list: the push drops
// it. With a depth-sorted list an owner stops at the first round whose
// depth lower bound exceeds its bound, and the workgroup stops the item
// when all its owners have.
// The K output slots of each row of the item's region are then written
// slot-linearly (lane q writes slot q of the row's contiguous run) after the
// keys are exchanged through LDS, so that stores are contiguous across lanes.
constexpr int kPairWin = 1536;
// For K <= 2 the pair buffers hold half as many entries (those passes
// evaluate their pairs in per-owner loops; the buffers serve the output
// stage's lists).
constexpr int kPairWinSmallK = 768;
constexpr int kLaneMinPairs = 24;    // a dense round: at least kLaneMinOwners owners
constexpr int kLaneMinOwners = 240;  // with at least kLaneMinPairs candidate pairs each

template <int KMAX, bool PERSP>
__global__ __launch_bounds__(kFineThreads) __attribute__((amdgpu_waves_per_eu(KMAX <= 10 ? 4 : 1, 8))) void fine_raster(
    const FaceRec* __restrict__ recs, const FaceBin* __restrict__ fbin, int64_t F, const int64_t* __restrict__ off,
    const int32_t* __restrict__ count, const int64_t* __restrict__ offset, const uint32_t* __restrict__ items,
    WsHeader* __restrict__ hdr, const int32_t* __restrict__ entries, const float* __restrict__ round_lb,
    int64_t capacity, int32_t sort_min, int32_t H, int32_t W, int32_t K, float blur, uint32_t settings, int32_t nbx,
    int32_t nby, int64_t* __restrict__ pix_to_face, float* __restrict__ zbuf, float* __restrict__ bary,
    float* __restrict__ dists) {
    // staged face records, their face indices and the owners' records; the
    // output phase reuses the whole block for its key exchange
    __shared__ __align__(16) unsigned char stage[kFineThreads * (sizeof(FaceRec) + 4 + sizeof(OwnerRec))];
    int4* srec4 = reinterpret_cast<int4*>(stage);   // piece p of record u at [p * kFineThreads + u]
    int32_t* sface = reinterpret_cast<int32_t*>(stage + kFineThreads * sizeof(FaceRec));
    OwnerRec* orec = reinterpret_cast<OwnerRec*>(stage + kFineThreads * (sizeof(FaceRec) + 4));
    // the round's masks
    __shared__ __align__(16) unsigned char aux[2 * kBin * (kFineThreads / 64) * 8];
    constexpr int kWin = KMAX <= 2 ? kPairWinSmallK : kPairWin;
    __shared__ uint16_t pcode[kWin];
    __shared__ double pres[kWin];
    __shared__ int32_t ofill[kFineThreads];
    __shared__ float pcx[kBin], pcy[kBin];   // pixel centres of the bin's columns and rows
    __shared__ int wsum[kFineThreads / 64];
    __shared__ int32_t nfill;
    uint64_t(*colmask)[kFineThreads / 64] = reinterpret_cast<uint64_t(*)[kFineThreads / 64]>(aux);
    uint64_t(*rowmask)[kFineThreads / 64] =
        reinterpret_cast<uint64_t(*)[kFineThreads / 64]>(aux + kBin * (kFineThreads / 64) * 8);
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int32_t n_items = hdr->fine_items;
    const int64_t per_img = (int64_t)nbx * nby;

    {
        if ((int64_t)blockIdx.x >= (int64_t)n_items) return;
        const uint32_t code = items[blockIdx.x];
        const int64_t b = (int64_t)(code >> 3);
        const int part = (int)(code & 7u);
        const bool quarter = part != kItemWhole;
        const int64_t n = b / per_img;
        const int rem = (int)(b - n * per_img);
        const int by = rem / nbx, bx = rem - (rem / nbx) * nbx;

        // region of the item inside the bin, and this thread's pixel
        const int reg_r = quarter ? (part >> 1) * (kBin / 2) : 0;
        const int reg_c = quarter ? (part & 1) * (kBin / 2) : 0;
        const int reg_w = quarter ? kBin / 2 : kBin;
        const int sub = quarter ? (lane & 3) : 0;
        int il, jl;
        if (quarter) {
            const int p = lane >> 2;   // 0..15: 4x4 block of the wave
            il = reg_r + (wave >> 1) * 4 + (p >> 2);
            jl = reg_c + (wave & 1) * 4 + (p & 3);
        } else {
            il = (wave >> 1) * (kBin / 2) + (lane >> 3);
            jl = (wave & 1) * (kBin / 2) + (lane & 7);
        }
        const int i = by * kBin + il;
        const int j = bx * kBin + jl;
        const bool valid = (i < H) && (j < W);
        const float px = pixel_centre(j, W);
        const float py = pixel_centre(i, H);
        if (t < kBin) pcx[t] = pixel_centre(bx * kBin + t, W);
        else if (t < 2 * kBin) pcy[t - kBin] = pixel_centre(by * kBin + t - kBin, H);

        double key[KMAX];
#pragma unroll
        for (int q = 0; q < KMAX; ++q) key[q] = empty_key();

        const int32_t cnt = count[b];
        const int64_t o = offset[b];
        const bool list_mode = (o + cnt <= capacity);
        const bool sorted = list_sorted(o, cnt, capacity, sort_min);
        const float* lb = round_lb + b * kRoundsPerBin;
        int64_t f0 = off[n], f1 = off[n + 1];
        f0 = f0 < 0 ? 0 : f0;
        f1 = f1 > F ? F : f1;
        const int64_t total = list_mode ? (int64_t)cnt : (f1 > f0 ? f1 - f0 : 0);
        bool done = !valid;

        // A bin with no face (a whole item: split bins have many) has every
        // slot empty: its region is padded row by row, with no keys, lists
        // or slot arithmetic. Such items come last in the queue and form
        // the pass's tail.
        if (total == 0) {
            const int rows = min(kBin, H - by * kBin), cols = min(kBin, W - bx * kBin);
            const int64_t px0 = ((int64_t)n * H + by * kBin) * W + bx * kBin;   // the region's first pixel
            const int64_t wk = (int64_t)W * K;
            const uint32_t none = __float_as_uint(-1.0f);
            pad_rows(reinterpret_cast<uint32_t*>(pix_to_face), 2 * px0 * K, 2 * wk, rows, 2 * cols * K, 0xffffffffu);
            pad_rows(reinterpret_cast<uint32_t*>(zbuf), px0 * K, wk, rows, cols * K, none);
            pad_rows(reinterpret_cast<uint32_t*>(bary), 3 * px0 * K, 3 * wk, rows, 3 * cols * K, none);
            pad_rows(reinterpret_cast<uint32_t*>(dists), px0 * K, wk, rows, cols * K, none);
            return;
        }

        // The next round's list entry is loaded once this round's records
        // are staged, and its box at the round's end, so that a round waits
        // on its record loads only (the first round loads all three).
        int64_t nfid = -1;
        FaceBin nfb;
        nfb.box_lo = 0x7fff7fff;
        nfb.box_hi = 0;
        nfb.mesh = 0;
        nfb.zmin_bits = 0;
        if (t < total) {
            nfid = list_mode ? (int64_t)entries[o + t] : f0 + t;
            nfb = fbin[nfid];
        }
        for (int64_t base = 0; base < total; base += kFineThreads) {
            // pruning bound: this owner's last key, or the quad's smallest
            double bound = quarter ? quad_min(key[KMAX - 1]) : key[KMAX - 1];
            // Every face from this round on has zmin >= lb[round]; an owner
            // whose bound is below that (with the rounding margin of the
            // depth interpolation) is finished.
            if (sorted && !done) {
                const float zl = lb[base / kFineThreads] * (1.0f - 0x1.0p-19f) - 1e-30f;
                if (zl > __uint_as_float((uint32_t)(key_bits(bound) >> 32))) done = true;
            }
            if (__syncthreads_count(!done) == 0) break;
            bool live = false;
            int c0 = 0, c1 = -1, r0 = 0, r1 = -1;
            const int64_t fid = nfid;
            if (fid >= 0) {
                // the face's pixel box, clipped to the item's region (empty
                // for a face that is never a candidate); only faces that
                // reach the region have their full record staged
                const FaceBin fb = nfb;
                c0 = max((fb.box_lo & 0xffff) - bx * kBin, reg_c);
                c1 = min((fb.box_hi & 0xffff) - bx * kBin, reg_c + reg_w - 1);
                r0 = max((fb.box_lo >> 16) - by * kBin, reg_r);
                r1 = min((fb.box_hi >> 16) - by * kBin, reg_r + reg_w - 1);
                live = (c0 <= c1) && (r0 <= r1);
                if (live) {
                    const int4* src = reinterpret_cast<const int4*>(recs + fid);
#pragma unroll
                    for (int p = 0; p < 4; ++p) srec4[p * kFineThreads + t] = src[p];
                    sface[t] = (int32_t)fid;
                }
            }
            const int64_t qn = base + kFineThreads + t;
            nfid = -1;
            if (qn < total) nfid = list_mode ? (int64_t)entries[o + qn] : f0 + qn;
            // the face's columns and rows as bit sets; ballot c of them is
            // the wave's mask for bin column (row) c (every lane writes the
            // same value)
            const uint32_t colbits = live ? (((2u << c1) - 1u) & ~((1u << c0) - 1u)) : 0u;
            const uint32_t rowbits = live ? (((2u << r1) - 1u) & ~((1u << r0) - 1u)) : 0u;
#pragma unroll
            for (int c = 0; c < kBin; ++c) {
                colmask[c][wave] = __ballot((colbits >> c) & 1u);
                rowmask[c][wave] = __ballot((rowbits >> c) & 1u);
            }
            __syncthreads();
            // this owner's candidate faces of the round, one word per wave
            // of staged faces (a quarter owner reads only its own word)
            uint64_t m0 = 0, m1 = 0, m2 = 0, m3 = 0;
            if (!done) {
                if (quarter) {
                    m0 = colmask[jl][sub] & rowmask[il][sub];
                } else {
                    m0 = colmask[jl][0] & rowmask[il][0];
                    m1 = colmask[jl][1] & rowmask[il][1];
                    m2 = colmask[jl][2] & rowmask[il][2];
                    m3 = colmask[jl][3] & rowmask[il][3];
                }
            }
            int ubase = quarter ? 64 * sub : 0;
            int left = (int)(__popcll(m0) + __popcll(m1) + __popcll(m2) + __popcll(m3));
            orec[t] = OwnerRec{px, py, bound};
            // Windows: every owner with pairs left takes up to cap of them,
            // cap = kPairWin / (owners with pairs left), so that all of them
            // progress in every window and the window holds at most kPairWin
            // pairs. One prefix sum per window gives the positions (low 16
            // bits) and counts the owners left for the next window (high
            // bits).
            // A dense round of a long list (nearly every owner with many
            // pairs) is evaluated by per-owner loops instead: the lanes of a
            // wave then have similar trip counts, and each pair is tested
            // against its owner's current bound, which prunes more where a
            // push costs two instructions per list slot.
            // For K <= 2 every round takes the per-owner loops: a pair's push
            // is one or two instructions, and the windows' codes, prefix sums
            // and LDS indirection cost more per pair than the lanes that a
            // loop's uneven trip counts leave idle (1M-triangle soup, K = 1:
            // 102.8 -> 95.1 us; at K = 8 the windows stay faster).
            if (KMAX <= 2 || (KMAX >= 16 && __syncthreads_count(left >= kLaneMinPairs) >= kLaneMinOwners)) {
                const uint64_t mw[4] = {m0, m1, m2, m3};
#pragma unroll 1
                for (int w = 0; w < 4; ++w) {
#pragma unroll 1
                    for (uint64_t x = mw[w]; x; x &= x - 1) {
                        const uint32_t u = (uint32_t)(ubase + 64 * w + __builtin_ctzll(x));
                        const double kk =
                            pair_key<PERSP>(staged_rec(srec4, u), sface[u], px, py, blur, key[KMAX - 1]);
                        if (kk < key[KMAX - 1]) topk_push<KMAX>(key, kk);
                    }
                }
                left = 0;
            }
            int active = __syncthreads_count(left > 0);
            while (active > 0) {
                const int cap = kWin / active;
                const int take = left < cap ? left : cap;
                left -= take;
                int packed_total;
                const int start =
                    block256_exclusive_sum_total(take | ((left > 0) ? 0x10000 : 0), wsum, packed_total) & 0xffff;
                const int wtotal = packed_total & 0xffff;
                active = packed_total >> 16;
                ofill[t] = start;
                for (int x = 0; x < take; ++x) {
                    while (m0 == 0) {
                        m0 = m1;
                        m1 = m2;
                        m2 = m3;
                        m3 = 0;
                        ubase += 64;
                    }
                    const int u = ubase + __builtin_ctzll(m0);
                    m0 &= m0 - 1;
                    pcode[start + x] = (uint16_t)(u | (t << 8));
                }
                __syncthreads();
                // the keys that pass go to the front of their owner's range
                for (int e = t; e < wtotal; e += kFineThreads) {
                    const uint32_t pc = pcode[e];
                    const OwnerRec ow = orec[pc >> 8];
                    const double kk =
                        pair_key<PERSP>(staged_rec(srec4, pc & 255u), sface[pc & 255u], ow.px, ow.py, blur, ow.bound);
                    if (key_bits(kk) != kEmptyKeyBits) pres[atomicAdd(&ofill[pc >> 8], 1)] = kk;
                }
                __syncthreads();
                const int passed = ofill[t] - start;
                for (int x = 0; x < passed; ++x) topk_push<KMAX>(key, pres[start + x]);
                bound = quarter ? quad_min(key[KMAX - 1]) : key[KMAX - 1];
                orec[t].bound = bound;
            }
            if (nfid >= 0) nfb = fbin[nfid];
            __syncthreads();
        }
        __syncthreads();
        if (quarter) {
            merge_with_lane<KMAX>(key, 1);
            merge_with_lane<KMAX>(key, 2);
        }

        // ---- output: exchange keys through LDS (reusing the staging
        // block); write each region row's reg_w*K slots with consecutive
        // lanes on consecutive slots (indices, depths and the padding of
        // empty slots), collecting the filled slots in a list (reusing the
        // pair buffers); then evaluate the listed slots densely for their
        // barycentrics and distances.
        uint64_t* kbuf = reinterpret_cast<uint64_t*>(stage);
        constexpr int kBufKeys = (int)sizeof(stage) / (int)sizeof(uint64_t);
        uint16_t* olist = reinterpret_cast<uint16_t*>(pres);
        constexpr int kOutList = (int)sizeof(pres) / (int)sizeof(uint16_t);
        const int row_slots = reg_w * K;
        const int rows_per_pass = max(1, min(reg_w, min(kBufKeys, kOutList) / row_slots));
        const bool writer = !quarter || sub == 0;
        const int64_t row0 = ((int64_t)n * H + by * kBin + reg_r) * W + bx * kBin + reg_c;
        // slot e of a pass -> (row, slot within the row, column): divisions
        // by multiplication (exact while e * divisor < 2^32)
        const uint32_t m_row = 0xffffffffu / (uint32_t)row_slots + 1u;
        const uint32_t m_k = K > 1 ? 0xffffffffu / (uint32_t)K + 1u : 0u;
        for (int ra = 0; ra < reg_w; ra += rows_per_pass) {
            const int rb = min(reg_w, ra + rows_per_pass);
            const int rr_me = il - reg_r;
            if (writer && rr_me >= ra && rr_me < rb) {
                uint64_t* dst = kbuf + ((rr_me - ra) * reg_w + (jl - reg_c)) * K;
#pragma unroll
                for (int q = 0; q < KMAX; ++q)
                    if (q < K) dst[q] = key_bits(key[q]);
            }
            if (t == 0) nfill = 0;
            __syncthreads();
            const int npass = (rb - ra) * row_slots;
            for (int e0 = 0; e0 < npass; e0 += kFineThreads) {
                const int e = e0 + t;
                bool filled = false;
                if (e < npass) {
                    const int rr = (int)__umulhi((uint32_t)e, m_row);
                    const int within = e - rr * row_slots;
                    const int jj = K > 1 ? (int)__umulhi((uint32_t)within, m_k) : within;
                    if (by * kBin + reg_r + ra + rr < H && bx * kBin + reg_c + jj < W) {
                        const int64_t so = (row0 + (int64_t)(ra + rr) * W) * K + within;
                        const uint64_t kk = kbuf[e];
                        if (kk == kEmptyKeyBits) {
                            pix_to_face[so] = -1;
                            zbuf[so] = -1.0f;
                            bary[3 * so + 0] = -1.0f;
                            bary[3 * so + 1] = -1.0f;
                            bary[3 * so + 2] = -1.0f;
                            dists[so] = -1.0f;
                        } else {
                            pix_to_face[so] = (int32_t)(kk & 0xffffffffull);
                            zbuf[so] = __uint_as_float((uint32_t)(kk >> 32));
                            filled = true;
                        }
                    }
                }
                const uint64_t bal = __ballot(filled);
                int at = 0;
                if (lane == 0 && bal) at = atomicAdd(&nfill, (int)__popcll(bal));
                at = __shfl(at, 0, 64);
                if (filled)
                    olist[at + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] =
                        (uint16_t)e;
            }
            __syncthreads();
            // (each thread's next slot's record is loaded while the current
            // one is evaluated: in a dense bin most slots are filled, and a
            // chain of dependent record gathers made the output stage of the
            // longest items as long as two of their rounds)
            const int nf = nfill;
            FaceRec rnext;
            if (t < nf) rnext = recs[(int32_t)(kbuf[olist[t]] & 0xffffffffull)];
            for (int x = t; x < nf; x += kFineThreads) {
                const int e = olist[x];
                const FaceRec rcur = rnext;
                if (x + kFineThreads < nf) rnext = recs[(int32_t)(kbuf[olist[x + kFineThreads]] & 0xffffffffull)];
                const int rr = (int)__umulhi((uint32_t)e, m_row);
                const int within = e - rr * row_slots;
                const int jj = K > 1 ? (int)__umulhi((uint32_t)within, m_k) : within;
                const int64_t so = (row0 + (int64_t)(ra + rr) * W) * K + within;
                float o0, o1, o2, sd;
                slot_outputs<PERSP>(rcur, pcx[reg_c + jj], pcy[reg_r + ra + rr],
                                    (settings & DMR_RASTER_UNCLIPPED_BARY) != 0, o0, o1, o2, sd);
                bary[3 * so + 0] = o0;
                bary[3 * so + 1] = o1;
                bary[3 * so + 2] = o2;
                dists[so] = sd;
            }
            __syncthreads();
        }
    }
}

template <int KMAX>
static void launch_fine(const FwdArgs& a, dim3 grid, const FaceRec* recs, const FaceBin* fbin, const int32_t* count,
                        const int64_t* offset, const uint32_t* items, WsHeader* hdr, const int32_t* entries,
                        const float* round_lb) {
    if (a.settings & DMR_RASTER_PERSPECTIVE_CORRECT)
        fine_raster<KMAX, true><<<grid, kFineThreads, 0, a.stream>>>(
            recs, fbin, a.F, a.off, count, offset, items, hdr, entries, round_lb, a.capacity, sort_min_entries(a.K),
            a.H, a.W, a.K, a.blur, a.settings, (int32_t)a.L.nbx, (int32_t)a.L.nby, a.pix_to_face, a.zbuf, a.bary,
            a.dists);
    else
        fine_raster<KMAX, false><<<grid, kFineThreads, 0, a.stream>>>(
            recs, fbin, a.F, a.off, count, offset, items, hdr, entries, round_lb, a.capacity, sort_min_entries(a.K),
            a.H, a.W, a.K, a.blur, a.settings, (int32_t)a.L.nbx, (int32_t)a.L.nby, a.pix_to_face, a.zbuf, a.bary,
            a.dists);
}

hipError_t launch_binning(const FwdArgs& a, bool sort) {
    char* ws = a.ws;
    WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
    FaceRec* recs = reinterpret_cast<FaceRec*>(ws + a.L.off_records);
    FaceBin* fbin = reinterpret_cast<FaceBin*>(ws + a.L.off_fbin);
    int32_t* count = reinterpret_cast<int32_t*>(ws + a.L.off_count);
    int64_t* offset = reinterpret_cast<int64_t*>(ws + a.L.off_offset);
    int32_t* rep = reinterpret_cast<int32_t*>(ws + a.L.off_rep);
    int32_t* perm = reinterpret_cast<int32_t*>(ws + a.L.off_perm);
    int32_t* block_live = reinterpret_cast<int32_t*>(ws + a.L.off_live);
    float* round_lb = reinterpret_cast<float*>(ws + a.L.off_roundlb);
    int32_t* entries = reinterpret_cast<int32_t*>(ws + a.L.off_entries);

    // header + bin counts to zero (header words are int32-sized multiples)
    {
        timing_begin(kKZeroFwd, a.stream);
        const int64_t nrep = (int64_t)count_replicas(a.L.bins) * a.L.bins;
        zero_i32x2<<<(unsigned)std::min<int64_t>(1024, (nrep + 255) / 256 + 1), 256, 0, a.stream>>>(
            reinterpret_cast<int32_t*>(hdr), (int64_t)(sizeof(WsHeader) / 4), rep, nrep);
        timing_end(kKZeroFwd, a.stream);
    }
    // Faces that share no vertices (V >= 2F: a triangle soup, whose faces
    // come in no spatial order) are set up and filled 512 to a workgroup:
    // one LDS histogram then serves twice the faces, and the about 256 bins
    // that each workgroup of a soup's faces touches cost half the global
    // count atomics per face (1M-triangle soup: setup 46 -> 38 us, fill 42.6
    // -> 33.7 us). The faces of a mesh come in spatial order and share few
    // bins per workgroup; there larger workgroups were slower (16 meshes:
    // setup 21.4 -> 26.4 us, fill 12.1 -> 14.8 us).
    const bool wide = !a.points && a.V >= 2 * a.F;
    const int tpb = wide ? kSetupThreadsWide : kSetupThreads;
    const int64_t setup_blocks = (a.F + tpb - 1) / tpb;
    if (a.F > 0 && a.points) {
        hipError_t err = launch_point_setup(a, reinterpret_cast<PointRec*>(recs), fbin, rep, block_live, hdr);
        if (err != hipSuccess) return err;
    } else if (a.F > 0) {
        timing_begin(kKFaceSetup, a.stream);
        if (wide)
            face_setup_count<kSetupThreadsWide><<<(unsigned)setup_blocks, kSetupThreadsWide, 0, a.stream>>>(
                a.verts, a.V, a.faces, a.F, a.off, a.N, a.H, a.W, a.blur, a.settings, (int32_t)a.L.nbx,
                (int32_t)a.L.nby, recs, fbin, rep, count_replicas(a.L.bins), a.L.bins, block_live, hdr);
        else
            face_setup_count<kSetupThreads><<<(unsigned)setup_blocks, kSetupThreads, 0, a.stream>>>(
                a.verts, a.V, a.faces, a.F, a.off, a.N, a.H, a.W, a.blur, a.settings, (int32_t)a.L.nbx,
                (int32_t)a.L.nby, recs, fbin, rep, count_replicas(a.L.bins), a.L.bins, block_live, hdr);
        timing_end(kKFaceSetup, a.stream);
    }
    timing_begin(kKBinScan, a.stream);
    uint32_t* items = reinterpret_cast<uint32_t*>(ws + a.L.off_items);
    // heavy bins are split into quarter items for the mesh fine pass only
    const int split = (a.K <= kSplitMaxK && !a.points) ? 1 : 0;
    bin_scan<<<1, kScanThreads, 0, a.stream>>>(count, offset, rep, count_replicas(a.L.bins), perm, items, a.L.bins,
                                                 split, sort_min_entries(a.K), block_live,
                                                 a.F > 0 ? setup_blocks : 0, a.capacity, a.L.min_bytes, hdr);
    timing_end(kKBinScan, a.stream);
    if (a.F > 0) {
        timing_begin(kKBinFill, a.stream);
        // the same workgroup size as the setup (a workgroup fills the copy
        // of the counts its setup workgroup counted into)
        if (wide)
            bin_fill<kSetupThreadsWide><<<(unsigned)setup_blocks, kSetupThreadsWide, 0, a.stream>>>(
                fbin, a.F, count, offset, rep, count_replicas(a.L.bins), a.L.bins, entries, a.capacity,
                (int32_t)a.L.nbx, (int32_t)a.L.nby);
        else
            bin_fill<kSetupThreads><<<(unsigned)setup_blocks, kSetupThreads, 0, a.stream>>>(
                fbin, a.F, count, offset, rep, count_replicas(a.L.bins), a.L.bins, entries, a.capacity,
                (int32_t)a.L.nbx, (int32_t)a.L.nby);
        timing_end(kKBinFill, a.stream);
    }
    if (a.F > 0 && sort) {
        timing_begin(kKBinSort, a.stream);
        bin_sort<<<(unsigned)a.L.bins, kSortThreads, 0, a.stream>>>(fbin, count, offset, perm, entries, a.capacity,
                                                                     sort_min_entries(a.K), hdr, round_lb);
        timing_end(kKBinSort, a.stream);
    }
    return hipGetLastError();
}

hipError_t launch_forward(const FwdArgs& a) {
    hipError_t err = launch_binning(a, true);
    if (err != hipSuccess) return err;
    char* ws = a.ws;
    WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
    FaceRec* recs = reinterpret_cast<FaceRec*>(ws + a.L.off_records);
    FaceBin* fbin = reinterpret_cast<FaceBin*>(ws + a.L.off_fbin);
    int32_t* count = reinterpret_cast<int32_t*>(ws + a.L.off_count);
    int64_t* offset = reinterpret_cast<int64_t*>(ws + a.L.off_offset);
    uint32_t* items = reinterpret_cast<uint32_t*>(ws + a.L.off_items);
    float* round_lb = reinterpret_cast<float*>(ws + a.L.off_roundlb);
    int32_t* entries = reinterpret_cast<int32_t*>(ws + a.L.off_entries);
    // room for every item: four per bin when bins may be split (a loop over
    // items on a smaller grid would save the empty workgroups' few
    // microseconds, but its live state spills scalar registers: measured
    // slower)
    dim3 grid((unsigned)(a.L.bins * (a.K <= kSplitMaxK ? 4 : 1)));
    timing_begin(kKFineRaster, a.stream);
#define DMR_FINE(KM) launch_fine<KM>(a, grid, recs, fbin, count, offset, items, hdr, entries, round_lb)
    if (a.K <= 1) DMR_FINE(1);
    else if (a.K <= 2) DMR_FINE(2);
    else if (a.K <= 4) DMR_FINE(4);
    else if (a.K <= 8) DMR_FINE(8);
    else if (a.K <= 10) DMR_FINE(10);
    else if (a.K <= 16) DMR_FINE(16);
    else if (a.K <= 32) DMR_FINE(32);
    else if (a.K <= 50) DMR_FINE(50);
    else DMR_FINE(64);
#undef DMR_FINE
    timing_end(kKFineRaster, a.stream);
    return hipGetLastError();
}

}  // namespace dmr
