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
__global__ void zero_i32(int32_t* p, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = 0;
}

// ---------------------------------------------------------------------------
// K1: per-face setup, culling and bin counting
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void face_setup_count(
    const float* __restrict__ verts, int64_t V, const int64_t* __restrict__ faces, int64_t F,
    const int64_t* __restrict__ off, int64_t N, int32_t H, int32_t W, float blur,
    int32_t nbx, int32_t nby, FaceRec* __restrict__ recs, int32_t* __restrict__ bin_count,
    WsHeader* __restrict__ hdr) {
    int64_t f = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    bool live = false;
    if (f < F) {
        FaceRec r;
        r.face = -1;
        r.box_lo = 0x7fff7fff;  // empty box: lo > hi
        r.box_hi = 0;
        // mesh of face f: the n with off[n] <= f < off[n+1]
        int64_t lo = 0, hi = N - 1;
        while (lo < hi) {
            int64_t mid = (lo + hi) >> 1;
            if (off[mid + 1] > f) hi = mid; else lo = mid + 1;
        }
        int64_t n = lo;
        bool ok = (off[n] <= f) && (f < off[n + 1]);
        int64_t vi0 = faces[3 * f + 0], vi1 = faces[3 * f + 1], vi2 = faces[3 * f + 2];
        bool idx_ok = vi0 >= 0 && vi0 < V && vi1 >= 0 && vi1 < V && vi2 >= 0 && vi2 < V;
        if (!idx_ok) atomicOr(&hdr->flags, DMR_FLAG_BAD_VERTEX_INDEX);
        float x0 = 0, y0 = 0, z0 = 0, x1 = 0, y1 = 0, z1 = 0, x2 = 0, y2 = 0, z2 = 0;
        if (idx_ok) {
            x0 = verts[3 * vi0]; y0 = verts[3 * vi0 + 1]; z0 = verts[3 * vi0 + 2];
            x1 = verts[3 * vi1]; y1 = verts[3 * vi1 + 1]; z1 = verts[3 * vi1 + 2];
            x2 = verts[3 * vi2]; y2 = verts[3 * vi2 + 1]; z2 = verts[3 * vi2 + 2];
        }
        float A = (x1 - x0) * (y2 - y0) - (y1 - y0) * (x2 - x0);
        // All depths <= 0 means z <= 0 at every pixel: the interpolation
        // weights are >= 0, so each product and each sum stays <= 0.
        bool zpos = (z0 > 0.0f) || (z1 > 0.0f) || (z2 > 0.0f);
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
        r.xmin = xmin; r.xmax = xmax; r.ymin = ymin; r.ymax = ymax;
        if (ok && idx_ok && A != 0.0f && zpos) {
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
                r.face = (int32_t)f;
                r.box_lo = j0 | (i0 << 16);
                r.box_hi = j1 | (i1 << 16);
                live = true;
                int32_t* cnt = bin_count + (int64_t)n * nbx * nby;
                for (int by = i0 / kBin; by <= i1 / kBin; ++by)
                    for (int bx = j0 / kBin; bx <= j1 / kBin; ++bx) atomicAdd(&cnt[by * nbx + bx], 1);
            }
        }
        recs[f] = r;
    }
    // one atomic per wave for the live-face count
    unsigned long long m = __ballot(live);
    if ((threadIdx.x & 63) == 0 && m) atomicAdd((unsigned long long*)&hdr->live_faces, (unsigned long long)__popcll(m));
}

// ---------------------------------------------------------------------------
// K2: exclusive prefix sum of the bin counts (one workgroup), header stats,
// cursor reset
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void bin_scan(const int32_t* __restrict__ count,
                                                         int64_t* __restrict__ offset,
                                                         int32_t* __restrict__ cursor, int64_t bins,
                                                         int64_t capacity, size_t base_bytes,
                                                         WsHeader* __restrict__ hdr) {
    __shared__ int64_t part[kScanThreads];
    __shared__ int64_t ovf[kScanThreads];
    const int t = threadIdx.x;
    const int64_t per = (bins + kScanThreads - 1) / kScanThreads;
    const int64_t b0 = t * per;
    const int64_t b1 = min(bins, b0 + per);
    int64_t s = 0;
    for (int64_t b = b0; b < b1; ++b) s += count[b];
    part[t] = s;
    __syncthreads();
    // Hillis-Steele inclusive scan over the per-thread sums
    for (int d = 1; d < kScanThreads; d <<= 1) {
        int64_t v = (t >= d) ? part[t - d] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    int64_t run = part[t] - s;  // exclusive prefix of this thread's chunk
    int64_t over = 0;
    for (int64_t b = b0; b < b1; ++b) {
        offset[b] = run;
        int32_t c = count[b];
        if (run + c > capacity) ++over;
        run += c;
        cursor[b] = 0;
    }
    ovf[t] = over;
    __syncthreads();
    if (t == 0) {
        int64_t total = part[kScanThreads - 1];
        int64_t o = 0;
        for (int q = 0; q < kScanThreads; ++q) o += ovf[q];
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
__global__ __launch_bounds__(256) void bin_fill(const FaceRec* __restrict__ recs, int64_t F,
                                                const int64_t* __restrict__ off, int64_t N,
                                                const int32_t* __restrict__ count,
                                                const int64_t* __restrict__ offset,
                                                int32_t* __restrict__ cursor, int32_t* __restrict__ entries,
                                                int64_t capacity, int32_t nbx, int32_t nby) {
    int64_t f = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (f >= F) return;
    const int32_t box_lo = recs[f].box_lo;
    const int32_t box_hi = recs[f].box_hi;
    if (recs[f].face < 0) return;
    int64_t lo = 0, hi = N - 1;
    while (lo < hi) {
        int64_t mid = (lo + hi) >> 1;
        if (off[mid + 1] > f) hi = mid; else lo = mid + 1;
    }
    const int64_t binbase = lo * nbx * nby;
    int j0 = box_lo & 0xffff, i0 = box_lo >> 16, j1 = box_hi & 0xffff, i1 = box_hi >> 16;
    for (int by = i0 / kBin; by <= i1 / kBin; ++by)
        for (int bx = j0 / kBin; bx <= j1 / kBin; ++bx) {
            int64_t b = binbase + by * nbx + bx;
            int64_t o = offset[b];
            if (o + count[b] <= capacity) {
                int32_t pos = atomicAdd(&cursor[b], 1);
                entries[o + pos] = (int32_t)f;
            }
        }
}

// ---------------------------------------------------------------------------
// K4: fine rasterization with a register top-K
// ---------------------------------------------------------------------------
template <int KMAX>
__device__ __forceinline__ void topk_insert(uint64_t (&key)[KMAX], uint64_t k) {
#pragma unroll
    for (int q = 0; q < KMAX; ++q) {
        uint64_t a = key[q];
        bool lt = k < a;
        key[q] = lt ? k : a;
        k = lt ? a : k;
    }
}

// Writes one output slot: padding for the empty key, else the face's
// re-evaluated values (the same operations give the same bits as the key's z).
__device__ __noinline__ void write_slot(const FaceRec* __restrict__ recs, uint64_t kk, float px, float py,
                                        float blur, int64_t so, int64_t* __restrict__ pix_to_face,
                                        float* __restrict__ zbuf, float* __restrict__ bary,
                                        float* __restrict__ dists) {
    if (kk == ~0ull) {
        pix_to_face[so] = -1;
        zbuf[so] = -1.0f;
        bary[3 * so + 0] = -1.0f;
        bary[3 * so + 1] = -1.0f;
        bary[3 * so + 2] = -1.0f;
        dists[so] = -1.0f;
        return;
    }
    const int32_t face = (int32_t)(kk & 0xffffffffull);
    PairState s;
    eval_pair(recs[face], px, py, blur, true, s);
    pix_to_face[so] = face;
    zbuf[so] = s.z;
    bary[3 * so + 0] = s.bh0;
    bary[3 * so + 1] = s.bh1;
    bary[3 * so + 2] = s.bh2;
    dists[so] = s.inside ? -s.d2 : s.d2;
}

template <int KMAX>
__global__ __launch_bounds__(kFineThreads) void fine_raster(
    const FaceRec* __restrict__ recs, int64_t F, const int64_t* __restrict__ off,
    const int32_t* __restrict__ count, const int64_t* __restrict__ offset,
    const int32_t* __restrict__ entries, int64_t capacity, int32_t H, int32_t W, int32_t K, float blur,
    int32_t nbx, int32_t nby, int64_t* __restrict__ pix_to_face, float* __restrict__ zbuf,
    float* __restrict__ bary, float* __restrict__ dists) {
    __shared__ FaceRec srec[kFineThreads];
    const int64_t b = blockIdx.x;
    const int64_t per_img = (int64_t)nbx * nby;
    const int64_t n = b / per_img;
    const int rem = (int)(b - n * per_img);
    const int by = rem / nbx, bx = rem - (rem / nbx) * nbx;
    const int t = threadIdx.x;
    const int i = by * kBin + t / kBin;
    const int j = bx * kBin + (t % kBin);
    const bool valid = (i < H) && (j < W);
    const float px = pixel_centre(j, W);
    const float py = pixel_centre(i, H);

    uint64_t key[KMAX];
#pragma unroll
    for (int q = 0; q < KMAX; ++q) key[q] = ~0ull;

    const int32_t cnt = count[b];
    const int64_t o = offset[b];
    const bool list_mode = (o + cnt <= capacity);
    int64_t f0 = off[n], f1 = off[n + 1];
    f0 = f0 < 0 ? 0 : f0;
    f1 = f1 > F ? F : f1;
    const int64_t total = list_mode ? (int64_t)cnt : (f1 > f0 ? f1 - f0 : 0);

    for (int64_t base = 0; base < total; base += kFineThreads) {
        int64_t q = base + t;
        if (q < total) {
            int64_t fid = list_mode ? (int64_t)entries[o + q] : f0 + q;
            srec[t] = recs[fid];
        }
        __syncthreads();
        const int m = (int)min((int64_t)kFineThreads, total - base);
        if (valid) {
            for (int u = 0; u < m; ++u) {
                const int32_t face = srec[u].face;
                const int32_t lo = srec[u].box_lo, hi = srec[u].box_hi;
                if (face < 0) continue;
                if (j < (lo & 0xffff) || j > (hi & 0xffff) || i < (lo >> 16) || i > (hi >> 16)) continue;
                PairState s;
                eval_pair(srec[u], px, py, blur, false, s);
                if (!s.cand) continue;
                uint64_t kk = ((uint64_t)__float_as_uint(s.z) << 32) | (uint32_t)face;
                if (kk < key[KMAX - 1]) topk_insert<KMAX>(key, kk);
            }
        }
        __syncthreads();
    }
    if (!valid) return;
    const int64_t pix = ((int64_t)n * H + i) * W + j;
    const int64_t sbase = pix * K;
#pragma unroll
    for (int q = 0; q < KMAX; ++q) {
        if (q < K) write_slot(recs, key[q], px, py, blur, sbase + q, pix_to_face, zbuf, bary, dists);
    }
}
template <int KMAX>
static void launch_fine(const FwdArgs& a, dim3 grid, const FaceRec* recs, const int32_t* count,
                        const int64_t* offset, const int32_t* entries) {
    fine_raster<KMAX><<<grid, kFineThreads, 0, a.stream>>>(
        recs, a.F, a.off, count, offset, entries, a.capacity, a.H, a.W, a.K, a.blur, (int32_t)a.L.nbx,
        (int32_t)a.L.nby, a.pix_to_face, a.zbuf, a.bary, a.dists);
}

hipError_t launch_forward(const FwdArgs& a) {
    char* ws = a.ws;
    WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
    FaceRec* recs = reinterpret_cast<FaceRec*>(ws + a.L.off_records);
    int32_t* count = reinterpret_cast<int32_t*>(ws + a.L.off_count);
    int64_t* offset = reinterpret_cast<int64_t*>(ws + a.L.off_offset);
    int32_t* cursor = reinterpret_cast<int32_t*>(ws + a.L.off_cursor);
    int32_t* entries = reinterpret_cast<int32_t*>(ws + a.L.off_entries);

    // header + bin counts to zero (header words are int32-sized multiples)
    {
        timing_begin(kKZeroFwd, a.stream);
        zero_i32<<<64, 256, 0, a.stream>>>(reinterpret_cast<int32_t*>(hdr), (int64_t)(sizeof(WsHeader) / 4));
        zero_i32<<<(unsigned)std::min<int64_t>(1024, (a.L.bins + 255) / 256 + 1), 256, 0, a.stream>>>(count, a.L.bins);
        timing_end(kKZeroFwd, a.stream);
    }
    if (a.F > 0) {
        timing_begin(kKFaceSetup, a.stream);
        face_setup_count<<<(unsigned)((a.F + 255) / 256), 256, 0, a.stream>>>(
            a.verts, a.V, a.faces, a.F, a.off, a.N, a.H, a.W, a.blur, (int32_t)a.L.nbx, (int32_t)a.L.nby, recs,
            count, hdr);
        timing_end(kKFaceSetup, a.stream);
    }
    timing_begin(kKBinScan, a.stream);
    bin_scan<<<1, kScanThreads, 0, a.stream>>>(count, offset, cursor, a.L.bins, a.capacity, a.L.min_bytes, hdr);
    timing_end(kKBinScan, a.stream);
    if (a.F > 0) {
        timing_begin(kKBinFill, a.stream);
        bin_fill<<<(unsigned)((a.F + 255) / 256), 256, 0, a.stream>>>(recs, a.F, a.off, a.N, count, offset, cursor,
                                                                      entries, a.capacity, (int32_t)a.L.nbx,
                                                                      (int32_t)a.L.nby);
        timing_end(kKBinFill, a.stream);
    }
    dim3 grid((unsigned)a.L.bins);
    timing_begin(kKFineRaster, a.stream);
    if (a.K <= 1) launch_fine<1>(a, grid, recs, count, offset, entries);
    else if (a.K <= 2) launch_fine<2>(a, grid, recs, count, offset, entries);
    else if (a.K <= 4) launch_fine<4>(a, grid, recs, count, offset, entries);
    else if (a.K <= 8) launch_fine<8>(a, grid, recs, count, offset, entries);
    else if (a.K <= 10) launch_fine<10>(a, grid, recs, count, offset, entries);
    else if (a.K <= 16) launch_fine<16>(a, grid, recs, count, offset, entries);
    else if (a.K <= 32) launch_fine<32>(a, grid, recs, count, offset, entries);
    else if (a.K <= 50) launch_fine<50>(a, grid, recs, count, offset, entries);
    else launch_fine<64>(a, grid, recs, count, offset, entries);
    timing_end(kKFineRaster, a.stream);
    return hipGetLastError();
}

}  // namespace dmr
