// Point-cloud rasterization on gfx950: for every pixel, the K nearest points
// of its own cloud within a radius, and the backward pass to the point
// positions. The pages list point clouds among the data the renderer takes,
// beside meshes (rocketrecap summary, "2:02 Data Structures and I/O"), with
// the same two-stage, per-pixel K-nearest selection over heterogeneous
// batches (gptget.net summary, "Methodology"). The reading is stated in
// include/dmr.h: a point with z > 0 is a candidate for a pixel when its
// squared 2D distance to the pixel centre, (px - x)^2 + (py - y)^2 in
// binary32, is below radius^2 (strict); the K smallest (z, index) are kept.
//
// The coarse stage is the mesh rasterizer's: a setup pass writes each
// point's 16-byte record and pixel box (FaceBin) and counts it into the
// 16x16 bins the box overlaps; the scan, fill and depth sort are shared.
// The fine pass gives each bin one 256-thread workgroup, one pixel per
// thread, stages the bin's points in LDS round by round and keeps a sorted
// register top-K, stopping once the round's depth bound passes every
// pixel's K-th key.
#include <algorithm>

#include "dmr_internal.h"
#include "lds_accum.h"

namespace dmr {

constexpr int kPointThreads = 256;

__device__ __forceinline__ int64_t cloud_of(const int64_t* __restrict__ off, int64_t N, int64_t p) {
    // last n with off[n] <= p, clamped to [0, N - 1]
    int64_t lo = 0, hi = N - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (off[mid] <= p) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// setup: per point record, pixel box and bin counts (LDS histogram for the
// block's home cloud, global atomics otherwise)
// ---------------------------------------------------------------------------
constexpr int kPointHistBins = 4096;

__global__ __launch_bounds__(kSetupThreads) void point_setup_count(
    const float* __restrict__ pts, int64_t P, const int64_t* __restrict__ off, int64_t N, int32_t H, int32_t W,
    float radius, int32_t nbx, int32_t nby, PointRec* __restrict__ recs, FaceBin* __restrict__ fbin,
    int32_t* __restrict__ rep_count, int32_t replicas, int64_t bins, int32_t* __restrict__ block_live) {
    int32_t* __restrict__ bin_count = rep_count + (int64_t)(blockIdx.x % (uint32_t)replicas) * bins;
    __shared__ int32_t hist[kPointHistBins];
    __shared__ int64_t home_s, home_lo, home_hi;
    __shared__ int32_t live_s;
    const int per_img = nbx * nby;
    const bool use_lds = per_img <= kPointHistBins;
    const int64_t first = (int64_t)blockIdx.x * kSetupThreads;
    if (threadIdx.x == 0) {
        const int64_t h = cloud_of(off, N, first);
        home_s = h;
        home_lo = off[h];
        home_hi = off[h + 1];
        live_s = 0;
    }
    if (use_lds)
        for (int q = threadIdx.x; q < per_img; q += kSetupThreads) hist[q] = 0;
    __syncthreads();
    const int64_t home = home_s;
    const int64_t p = first + threadIdx.x;
    bool live = false;
    if (p < P) {
        const bool in_home = home_lo <= p && p < home_hi;
        const int64_t n = in_home ? home : cloud_of(off, N, p);
        const bool ok = in_home || (off[n] <= p && p < off[n + 1]);
        PointRec r;
        r.x = pts[3 * p];
        r.y = pts[3 * p + 1];
        r.z = pts[3 * p + 2];
        r.idx = -1;
        FaceBin fb;
        fb.box_lo = 0x7fff7fff;  // empty box: lo > hi
        fb.box_hi = 0;
        fb.mesh = (int32_t)n;
        fb.zmin_bits = __float_as_uint(r.z);
        if (ok && r.z > 0.0f) {
            // conservative pixel box: the point's square of half-side radius,
            // grown by a margin far above the rounding of the distance test
            const float mag = fmaxf(1.0f, fmaxf(fabsf(r.x), fabsf(r.y)));
            const float m = 1e-5f * mag + 1e-5f * radius;
            const float xl = r.x - radius - m, xh = r.x + radius + m;
            const float yl = r.y - radius - m, yh = r.y + radius + m;
            float jl = ceilf(((xl + 1.0f) * (float)W - 1.0f) * 0.5f);
            float jh = floorf(((xh + 1.0f) * (float)W - 1.0f) * 0.5f);
            float il = ceilf(((yl + 1.0f) * (float)H - 1.0f) * 0.5f);
            float ih = floorf(((yh + 1.0f) * (float)H - 1.0f) * 0.5f);
            jl = fmaxf(jl, 0.0f);
            il = fmaxf(il, 0.0f);
            jh = fminf(jh, (float)(W - 1));
            ih = fminf(ih, (float)(H - 1));
            if (jl <= jh && il <= ih) {
                const int j0 = (int)jl, j1 = (int)jh, i0 = (int)il, i1 = (int)ih;
                r.idx = (int32_t)p;
                fb.box_lo = j0 | (i0 << 16);
                fb.box_hi = j1 | (i1 << 16);
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
        recs[p] = r;
        fbin[p] = fb;
    }
    const unsigned long long m = __ballot(live);
    if ((threadIdx.x & 63) == 0 && m) atomicAdd(&live_s, (int32_t)__popcll(m));
    __syncthreads();
    if (threadIdx.x == 0) block_live[blockIdx.x] = live_s;
    if (use_lds) {
        int32_t* cnt = bin_count + home * per_img;
        for (int q = threadIdx.x; q < per_img; q += kSetupThreads) {
            const int32_t c = hist[q];
            if (c) atomicAdd(&cnt[q], c);
        }
    }
}

hipError_t launch_point_setup(const FwdArgs& a, PointRec* recs, FaceBin* fbin, int32_t* count, int32_t* block_live,
                              WsHeader* hdr) {
    (void)hdr;
    timing_begin(kKPointSetup, a.stream);
    point_setup_count<<<(unsigned)((a.F + kSetupThreads - 1) / kSetupThreads), kSetupThreads, 0, a.stream>>>(
        a.points, a.F, a.off, a.N, a.H, a.W, a.radius, (int32_t)a.L.nbx, (int32_t)a.L.nby, recs, fbin, count,
        count_replicas(a.L.bins), a.L.bins, block_live);
    timing_end(kKPointSetup, a.stream);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fine pass
// ---------------------------------------------------------------------------

// Keys: (z bits << 32) | point index with z > 0. Read as binary64 such a
// pattern is finite, non-negative and not a NaN, and numeric order is
// pattern order, so one v_min_f64 / v_max_f64 moves a key one slot (+inf
// marks an empty slot); written out because the compiler's fmin/fmax first
// quiet their operands.
constexpr uint64_t kPointEmptyBits = 0x7ff0000000000000ull;

template <int KMAX>
__device__ __forceinline__ void point_topk_push(double (&key)[KMAX], double k) {
#pragma unroll
    for (int q = 0; q < KMAX; ++q) {
        double hi;
        asm("v_max_f64 %0, %1, %2" : "=v"(hi) : "v"(key[q]), "v"(k));
        asm("v_min_f64 %0, %0, %1" : "+v"(key[q]) : "v"(k));
        k = hi;
    }
}

// Squared distance of the pixel centre to the point, in the fixed order.
__device__ __forceinline__ float point_d2(float px, float py, float x, float y) {
    const float dx = px - x, dy = py - y;
    return dx * dx + dy * dy;
}

template <int KMAX>
__global__ __launch_bounds__(kPointThreads) void point_raster(
    const PointRec* __restrict__ recs, const FaceBin* __restrict__ fbin, int64_t P, const int64_t* __restrict__ off,
    const int32_t* __restrict__ count, const int64_t* __restrict__ offset, const uint32_t* __restrict__ items,
    const WsHeader* __restrict__ hdr, const int32_t* __restrict__ entries, const float* __restrict__ round_lb,
    int64_t capacity, int32_t sort_min, int32_t H, int32_t W, int32_t K, float r2, int32_t nbx, int32_t nby,
    int64_t* __restrict__ out_idx, float* __restrict__ zbuf, float* __restrict__ dists) {
    __shared__ PointRec spt[kPointThreads];
    __shared__ uint64_t colmask[kBin][kPointThreads / 64];
    __shared__ uint64_t rowmask[kBin][kPointThreads / 64];
    constexpr int kBufKeys = 2560;   // one pass for K <= 10
    __shared__ uint64_t kbuf[kBufKeys];
    __shared__ float pcx[kBin], pcy[kBin];   // pixel centres of the bin's columns and rows
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    if ((int64_t)blockIdx.x >= (int64_t)hdr->fine_items) return;
    const int64_t b = (int64_t)(items[blockIdx.x] >> 3);
    const int64_t per_img = (int64_t)nbx * nby;
    const int64_t n = b / per_img;
    const int rem = (int)(b - n * per_img);
    const int by = rem / nbx, bx = rem - (rem / nbx) * nbx;
    // each wave owns an 8x8 quarter of the bin
    const int il = (wave >> 1) * (kBin / 2) + (lane >> 3);
    const int jl = (wave & 1) * (kBin / 2) + (lane & 7);
    const int i = by * kBin + il, j = bx * kBin + jl;
    const bool valid = i < H && j < W;
    const float px = pixel_centre(j, W), py = pixel_centre(i, H);
    if (t < kBin) pcx[t] = pixel_centre(bx * kBin + t, W);
    else if (t < 2 * kBin) pcy[t - kBin] = pixel_centre(by * kBin + t - kBin, H);

    double key[KMAX];
#pragma unroll
    for (int q = 0; q < KMAX; ++q) key[q] = __longlong_as_double((long long)kPointEmptyBits);

    const int32_t cnt = count[b];
    const int64_t o = offset[b];
    const bool list_mode = o + cnt <= capacity;
    const bool sorted = list_sorted(o, cnt, capacity, sort_min);
    const float* lb = round_lb + b * kRoundsPerBin;
    int64_t f0 = off[n], f1 = off[n + 1];
    f0 = f0 < 0 ? 0 : f0;
    f1 = f1 > P ? P : f1;
    const int64_t total = list_mode ? (int64_t)cnt : (f1 > f0 ? f1 - f0 : 0);
    bool done = !valid;

    for (int64_t base = 0; base < total; base += kPointThreads) {
        // every point from this round on has z >= lb[round]
        if (sorted && !done) {
            const uint64_t last = (uint64_t)__double_as_longlong(key[KMAX - 1]);
            if (lb[base / kPointThreads] > __uint_as_float((uint32_t)(last >> 32))) done = true;
        }
        if (__syncthreads_count(!done) == 0) break;
        const int64_t q = base + t;
        bool live = false;
        int c0 = 0, c1 = -1, r0 = 0, r1 = -1;
        if (q < total) {
            const int64_t pid = list_mode ? (int64_t)entries[o + q] : f0 + q;
            const FaceBin fb = fbin[pid];
            c0 = max((fb.box_lo & 0xffff) - bx * kBin, 0);
            c1 = min((fb.box_hi & 0xffff) - bx * kBin, kBin - 1);
            r0 = max((fb.box_lo >> 16) - by * kBin, 0);
            r1 = min((fb.box_hi >> 16) - by * kBin, kBin - 1);
            live = c0 <= c1 && r0 <= r1;
            if (live) spt[t] = recs[pid];
        }
        // the point's columns and rows as bit sets; ballot c of them is the
        // wave's mask for bin column (row) c (every lane writes the same value)
        const uint32_t colbits = live ? (((2u << c1) - 1u) & ~((1u << c0) - 1u)) : 0u;
        const uint32_t rowbits = live ? (((2u << r1) - 1u) & ~((1u << r0) - 1u)) : 0u;
#pragma unroll
        for (int c = 0; c < kBin; ++c) {
            colmask[c][wave] = __ballot((colbits >> c) & 1u);
            rowmask[c][wave] = __ballot((rowbits >> c) & 1u);
        }
        __syncthreads();
        if (!done) {
#pragma unroll 1
            for (int w = 0; w < kPointThreads / 64; ++w) {
                uint64_t m = colmask[jl][w] & rowmask[il][w];
                while (m) {
                    const int u = w * 64 + __builtin_ctzll(m);
                    m &= m - 1;
                    const PointRec r = spt[u];
                    if (point_d2(px, py, r.x, r.y) < r2) {
                        const double kk = __hiloint2double((int)__float_as_uint(r.z), r.idx);
                        if (kk < key[KMAX - 1]) point_topk_push<KMAX>(key, kk);
                    }
                }
            }
        }
        __syncthreads();
    }

    // output: keys through LDS, bin rows written slot-linearly (consecutive
    // lanes on consecutive slots of a row's contiguous 16*K run)
    const int row_slots = kBin * K;
    const int rows_per_pass = max(1, min(kBin, kBufKeys / row_slots));
    const int64_t row0 = ((int64_t)n * H + by * kBin) * W + bx * kBin;
    // slot e -> (row, slot within the row, column): divisions by
    // multiplication (exact while e * divisor < 2^32)
    const uint32_t m_row = 0xffffffffu / (uint32_t)row_slots + 1u;
    const uint32_t m_k = K > 1 ? 0xffffffffu / (uint32_t)K + 1u : 0u;
    for (int ra = 0; ra < kBin; ra += rows_per_pass) {
        const int rb = min(kBin, ra + rows_per_pass);
        __syncthreads();
        if (il >= ra && il < rb) {
            uint64_t* dst = kbuf + ((il - ra) * kBin + jl) * K;
#pragma unroll
            for (int q = 0; q < KMAX; ++q)
                if (q < K) dst[q] = (uint64_t)__double_as_longlong(key[q]);
        }
        __syncthreads();
        const int npass = (rb - ra) * row_slots;
        for (int e = t; e < npass; e += kPointThreads) {
            const int rr = (int)__umulhi((uint32_t)e, m_row);
            const int within = e - rr * row_slots;
            const int jj = K > 1 ? (int)__umulhi((uint32_t)within, m_k) : within;
            const int gi = by * kBin + ra + rr, gj = bx * kBin + jj;
            if (gi >= H || gj >= W) continue;
            const int64_t so = (row0 + (int64_t)(ra + rr) * W) * K + within;
            const uint64_t kk = kbuf[e];
            if (kk == kPointEmptyBits) {
                out_idx[so] = -1;
                zbuf[so] = -1.0f;
                dists[so] = -1.0f;
            } else {
                const int32_t pid = (int32_t)(kk & 0xffffffffull);
                const PointRec r = recs[pid];
                out_idx[so] = pid;
                zbuf[so] = __uint_as_float((uint32_t)(kk >> 32));
                dists[so] = point_d2(pcx[jj], pcy[ra + rr], r.x, r.y);
            }
        }
    }
}

hipError_t launch_points_forward(const FwdArgs& a) {
    hipError_t err = launch_binning(a, true);
    if (err != hipSuccess) return err;
    char* ws = a.ws;
    const WsHeader* hdr = reinterpret_cast<const WsHeader*>(ws);
    const PointRec* recs = reinterpret_cast<const PointRec*>(ws + a.L.off_records);
    const FaceBin* fbin = reinterpret_cast<const FaceBin*>(ws + a.L.off_fbin);
    const int32_t* count = reinterpret_cast<const int32_t*>(ws + a.L.off_count);
    const int64_t* offset = reinterpret_cast<const int64_t*>(ws + a.L.off_offset);
    const uint32_t* items = reinterpret_cast<const uint32_t*>(ws + a.L.off_items);
    const float* round_lb = reinterpret_cast<const float*>(ws + a.L.off_roundlb);
    const int32_t* entries = reinterpret_cast<const int32_t*>(ws + a.L.off_entries);
    const float r2 = a.radius * a.radius;
    const dim3 grid((unsigned)a.L.bins);
    timing_begin(kKPointRaster, a.stream);
#define DMR_POINTS(KM)                                                                                               \
    point_raster<KM><<<grid, kPointThreads, 0, a.stream>>>(recs, fbin, a.F, a.off, count, offset, items, hdr,       \
                                                           entries, round_lb, a.capacity,                           \
                                                           sort_min_entries(a.K), a.H, a.W, a.K, r2,                \
                                                           (int32_t)a.L.nbx, (int32_t)a.L.nby, a.pix_to_face,       \
                                                           a.zbuf, a.dists)
    if (a.K <= 1) DMR_POINTS(1);
    else if (a.K <= 2) DMR_POINTS(2);
    else if (a.K <= 4) DMR_POINTS(4);
    else if (a.K <= 8) DMR_POINTS(8);
    else if (a.K <= 10) DMR_POINTS(10);
    else if (a.K <= 16) DMR_POINTS(16);
    else if (a.K <= 32) DMR_POINTS(32);
    else DMR_POINTS(64);
#undef DMR_POINTS
    timing_end(kKPointRaster, a.stream);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// backward: one workgroup per 16x16 tile; zbuf = z_q and dists = d2 give
// dL/dz_q += g_z and dL/d(x_q, y_q) += -2 (px - x_q, py - y_q) g_d. A point
// reaches the few pixels within its radius, nearly all in one tile: the
// tile's terms are summed per point in LDS (lds_accum.h), then added to
// grad_points with one float atomic per (tile, point, coordinate).
// The tile's slots are read slot-linearly in chunks of kPointList
// (coalesced, the next chunk issued before the current one is evaluated);
// the filled ones (about one in ten) are compacted into an LDS list, and
// each thread evaluates the list's slots two at a time.
// ---------------------------------------------------------------------------
// The table size of the mesh backward (1024 entries); a 512-entry table,
// with more resident workgroups, measured 14% slower.
constexpr int kPointHashBits = kHashBits;
constexpr int kPointList = 1536;
static_assert(kPointList % kPointThreads == 0, "whole loads per thread");

__global__ void point_zero(float* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t k = i; k < n; k += stride) p[k] = 0.0f;
}

__global__ __launch_bounds__(kPointThreads) void point_backward(const float* __restrict__ pts, int64_t P,
                                                                int32_t H, int32_t W, int32_t K, int32_t nbx,
                                                                int32_t nby, const int64_t* __restrict__ idx,
                                                                const float* __restrict__ gz,
                                                                const float* __restrict__ gd,
                                                                float* __restrict__ grad, int32_t use_hash) {
    __shared__ uint32_t hkey[1 << kPointHashBits];
    __shared__ unsigned long long hval[1 << kPointHashBits][3];
    __shared__ int32_t lpt[kPointList];
    __shared__ uint16_t lslot[kPointList];   // slot index within the tile
    __shared__ int32_t nlist;
    constexpr int kPer = kPointList / kPointThreads;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int64_t per_img = (int64_t)nbx * nby;
    const int64_t b = blockIdx.x;
    const int64_t n = b / per_img;
    const int rem = (int)(b - n * per_img);
    const int by = rem / nbx, bx = rem - (rem / nbx) * nbx;
    const int rows = min(kBin, H - by * kBin), cols = min(kBin, W - bx * kBin);
    const int64_t tile0 = (((int64_t)n * H + by * kBin) * W + bx * kBin) * K;
    // tile slot s -> (row, slot within the row, column): divisions by
    // multiplication (exact while s * divisor < 2^32)
    const int row_slots = kBin * K;
    const uint32_t m_row = 0xffffffffu / (uint32_t)row_slots + 1u;
    const uint32_t m_k = K > 1 ? 0xffffffffu / (uint32_t)K + 1u : 0u;
    const int tile_slots = kBin * row_slots;
    auto load_chunk = [&](int cbase, int64_t (&fv)[kPer]) {
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int sidx = cbase + q * kPointThreads + t;
            fv[q] = -1;
            if (sidx < tile_slots) {
                const int r = (int)__umulhi((uint32_t)sidx, m_row);
                const int within = sidx - r * row_slots;
                const int col = K > 1 ? (int)__umulhi((uint32_t)within, m_k) : within;
                if (r < rows && col < cols) fv[q] = idx[tile0 + (int64_t)r * W * K + within];
            }
        }
    };
    clear_table<kPointHashBits>(hkey, hval, kPointThreads);
    int64_t fv[kPer];
    load_chunk(0, fv);
    for (int cbase = 0; cbase < tile_slots; cbase += kPointList) {
        if (t == 0) nlist = 0;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const bool filled = fv[q] >= 0 && fv[q] < P;
            const uint64_t bal = __ballot(filled);
            int at = 0;
            if (lane == 0 && bal) at = atomicAdd(&nlist, (int)__popcll(bal));
            at = __shfl(at, 0, 64);
            if (filled) {
                const int e = at + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                lpt[e] = (int32_t)fv[q];
                lslot[e] = (uint16_t)(cbase + q * kPointThreads + t);
            }
        }
        __syncthreads();
        if (cbase + kPointList < tile_slots) load_chunk(cbase + kPointList, fv);
        const int m = nlist;
        for (int e0 = 0; e0 < m; e0 += 2 * kPointThreads) {
            int32_t pq[2];
            float px[2], py[2], g_z[2], g_d[2], x[2], y[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int e = e0 + t + u * kPointThreads;
                pq[u] = -1;
                px[u] = py[u] = g_z[u] = g_d[u] = x[u] = y[u] = 0.0f;
                if (e < m) {
                    pq[u] = lpt[e];
                    const int sidx = lslot[e];
                    const int r = (int)__umulhi((uint32_t)sidx, m_row);
                    const int within = sidx - r * row_slots;
                    const int col = K > 1 ? (int)__umulhi((uint32_t)within, m_k) : within;
                    const int64_t so = tile0 + (int64_t)r * W * K + within;
                    px[u] = pixel_centre(bx * kBin + col, W);
                    py[u] = pixel_centre(by * kBin + r, H);
                    g_z[u] = gz ? gz[so] : 0.0f;
                    g_d[u] = gd ? gd[so] : 0.0f;
                    x[u] = pts[3 * (int64_t)pq[u]];
                    y[u] = pts[3 * (int64_t)pq[u] + 1];
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (pq[u] < 0) continue;
                const float gx = -2.0f * (px[u] - x[u]) * g_d[u];
                const float gy = -2.0f * (py[u] - y[u]) * g_d[u];
                vertex_add<kPointHashBits>(hkey, hval, grad, pq[u], gx, gy, g_z[u], use_hash != 0);
            }
        }
        __syncthreads();
    }
    flush_table<kPointHashBits>(hkey, hval, grad, kPointThreads);
}

hipError_t launch_points_backward(const PointBwdArgs& a) {
    timing_begin(kKPointBwd, a.stream);
    const int64_t n3 = 3 * a.P;
    if (n3 > 0)
        point_zero<<<(unsigned)std::min<int64_t>(2048, (n3 + 255) / 256), 256, 0, a.stream>>>(a.grad_points, n3);
    const int32_t nbx = (a.W + kBin - 1) / kBin, nby = (a.H + kBin - 1) / kBin;
    const int64_t bins = a.N * (int64_t)nbx * nby;
    if (bins > 0 && a.P > 0 && (a.gz || a.gd))
        point_backward<<<(unsigned)bins, kPointThreads, 0, a.stream>>>(a.points, a.P, a.H, a.W, a.K, nbx, nby,
                                                                        a.idx, a.gz, a.gd, a.grad_points,
                                                                        a.P - 1 <= kTableMaxId ? 1 : 0);
    timing_end(kKPointBwd, a.stream);
    return hipGetLastError();
}

}  // namespace dmr
