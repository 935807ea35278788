// Backward pass of the K-nearest-face rasterizer on gfx950: gradients flow
// from the per-pixel outputs back to vertex positions (rocketrecap summary of
// the PyTorch3D walkthrough, "3:52 Differentiable Renderer").
//
// One workgroup per 16x16 tile. The tile's filled slots (padding is a suffix
// of each pixel's list) are compacted into an LDS list, so that every lane
// works on a real (pixel, face) pair. Each pair re-runs the forward
// evaluation and applies the chain rule of zbuf = sum bh_k z_k,
// bh = clip(b)/S (with perspective correction bh = n/D, n_k = c_k z_{k+1}
// z_{k+2}), b = w/A and dists = +-|q - t u|^2 (t held at its minimiser or
// clamp); the returned barycentrics are bh, or the unclipped b (perspective-
// weighted the same way) on request. The nine partials are summed per vertex in an LDS
// hash table, then flushed into grad_verts with one float32 global atomic
// per (tile, vertex, coordinate).
//
// The LDS sums are 64-bit fixed point (see vertex_add): on gfx950 a float
// atomic add in LDS sustains about a third of a lane per clock per CU, an
// integer one more than seven.
#include <algorithm>

#include "dmr_internal.h"
#include "lds_accum.h"

namespace dmr {

// Zero fill of grad_verts; also resets the tile queue counter when given.
__global__ void zero_f32(float* p, int64_t n, int32_t* counter) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (counter && i == 0) *counter = 0;
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = 0.0f;
}

__device__ __forceinline__ void load_face(const float* __restrict__ verts, const int64_t* __restrict__ faces,
                                          int64_t f, int64_t V, FaceRec& r, int64_t (&vi)[3], bool& ok) {
    vi[0] = faces[3 * f + 0];
    vi[1] = faces[3 * f + 1];
    vi[2] = faces[3 * f + 2];
    ok = vi[0] >= 0 && vi[0] < V && vi[1] >= 0 && vi[1] < V && vi[2] >= 0 && vi[2] < V;
    if (!ok) return;
    r.x0 = verts[3 * vi[0]]; r.y0 = verts[3 * vi[0] + 1]; r.z0 = verts[3 * vi[0] + 2];
    r.x1 = verts[3 * vi[1]]; r.y1 = verts[3 * vi[1] + 1]; r.z1 = verts[3 * vi[1] + 2];
    r.x2 = verts[3 * vi[2]]; r.y2 = verts[3 * vi[2] + 1]; r.z2 = verts[3 * vi[2] + 2];
    float A = (r.x1 - r.x0) * (r.y2 - r.y0) - (r.y1 - r.y0) * (r.x2 - r.x0);
    ok = (A != 0.0f);
    r.invA = 1.0f / A;
    float ux = r.x1 - r.x0, uy = r.y1 - r.y0;
    r.il0 = 1.0f / (ux * ux + uy * uy);
    ux = r.x2 - r.x1; uy = r.y2 - r.y1;
    r.il1 = 1.0f / (ux * ux + uy * uy);
    ux = r.x0 - r.x2; uy = r.y0 - r.y2;
    r.il2 = 1.0f / (ux * ux + uy * uy);
    r.xmin = fminf(r.x0, fminf(r.x1, r.x2));
    r.xmax = fmaxf(r.x0, fmaxf(r.x1, r.x2));
    r.ymin = fminf(r.y0, fminf(r.y1, r.y2));
    r.ymax = fmaxf(r.y0, fmaxf(r.y1, r.y2));
}

// Backward of the perspective weighting o = n / D, n_k = a_k z_{k+1} z_{k+2}
// (a: the weighted barycentrics, inv_d = 1 / D): adds dL/da to ga and the
// depth partials to gzv, from the gradient go of o.
__device__ __forceinline__ void persp_backward(float go0, float go1, float go2, float o0, float o1, float o2,
                                               float inv_d, float a0, float a1, float a2, const FaceRec& r,
                                               float& ga0, float& ga1, float& ga2, float& gzv0, float& gzv1,
                                               float& gzv2) {
    const float dot = (go0 * o0 + go1 * o1) + go2 * o2;
    const float gn0 = (go0 - dot) * inv_d, gn1 = (go1 - dot) * inv_d, gn2 = (go2 - dot) * inv_d;
    ga0 += gn0 * (r.z1 * r.z2);
    ga1 += gn1 * (r.z2 * r.z0);
    ga2 += gn2 * (r.z0 * r.z1);
    gzv1 += gn0 * (a0 * r.z2);
    gzv2 += gn0 * (a0 * r.z1);
    gzv2 += gn1 * (a1 * r.z0);
    gzv0 += gn1 * (a1 * r.z2);
    gzv0 += gn2 * (a2 * r.z1);
    gzv1 += gn2 * (a2 * r.z0);
}

// Per-slot chain rule. Returns the nine partials (x, y, z of the three
// vertices) of L = gz*zbuf + gb.bary + gd*dists for one filled slot; `gout`
// is the gradient of the returned barycentrics.
__device__ __forceinline__ void slot_partials(const FaceRec& r, const PairState& s, float px, float py, float gz,
                                              float gout0, float gout1, float gout2, float gd, uint32_t settings,
                                              float (&g)[9]) {
    const bool persp = (settings & DMR_RASTER_PERSPECTIVE_CORRECT) != 0;
    const bool unclipped = (settings & DMR_RASTER_UNCLIPPED_BARY) != 0;
    // depth
    float gzv0 = gz * s.bh0, gzv1 = gz * s.bh1, gzv2 = gz * s.bh2;
    float gbh0 = (unclipped ? 0.0f : gout0) + gz * r.z0;
    float gbh1 = (unclipped ? 0.0f : gout1) + gz * r.z1;
    float gbh2 = (unclipped ? 0.0f : gout2) + gz * r.z2;
    // normalisation (or perspective weighting) and clip
    float gc0 = 0.0f, gc1 = 0.0f, gc2 = 0.0f;
    if (persp) {
        persp_backward(gbh0, gbh1, gbh2, s.bh0, s.bh1, s.bh2, s.invS, s.c0, s.c1, s.c2, r, gc0, gc1, gc2, gzv0, gzv1,
                       gzv2);
    } else {
        const float dot = (gbh0 * s.bh0 + gbh1 * s.bh1) + gbh2 * s.bh2;
        gc0 = (gbh0 - dot) * s.invS;
        gc1 = (gbh1 - dot) * s.invS;
        gc2 = (gbh2 - dot) * s.invS;
    }
    float gb0 = (s.b0 > 0.0f && s.b0 < 1.0f) ? gc0 : 0.0f;
    float gb1 = (s.b1 > 0.0f && s.b1 < 1.0f) ? gc1 : 0.0f;
    float gb2 = (s.b2 > 0.0f && s.b2 < 1.0f) ? gc2 : 0.0f;
    // unclipped barycentrics returned: their gradient reaches b directly
    if (unclipped && persp) {
        persp_backward(gout0, gout1, gout2, s.o0, s.o1, s.o2, s.invDr, s.b0, s.b1, s.b2, r, gb0, gb1, gb2, gzv0, gzv1,
                       gzv2);
    } else if (unclipped) {
        gb0 += gout0;
        gb1 += gout1;
        gb2 += gout2;
    }
    // b = w / A
    const float gw0 = gb0 * r.invA, gw1 = gb1 * r.invA, gw2 = gb2 * r.invA;
    const float gA = -((gb0 * s.b0 + gb1 * s.b1) + gb2 * s.b2) * r.invA;
    const float dx0 = r.x0 - px, dy0 = r.y0 - py;
    const float dx1 = r.x1 - px, dy1 = r.y1 - py;
    const float dx2 = r.x2 - px, dy2 = r.y2 - py;
    float gx0 = 0.0f, gy0 = 0.0f, gx1 = 0.0f, gy1 = 0.0f, gx2 = 0.0f, gy2 = 0.0f;
    // w0 = dx1*dy2 - dy1*dx2
    gx1 += gw0 * dy2; gy2 += gw0 * dx1; gy1 -= gw0 * dx2; gx2 -= gw0 * dy1;
    // w1 = dx2*dy0 - dy2*dx0
    gx2 += gw1 * dy0; gy0 += gw1 * dx2; gy2 -= gw1 * dx0; gx0 -= gw1 * dy2;
    // w2 = dx0*dy1 - dy0*dx1
    gx0 += gw2 * dy1; gy1 += gw2 * dx0; gy0 -= gw2 * dx1; gx1 -= gw2 * dy0;
    // A = (x1-x0)(y2-y0) - (y1-y0)(x2-x0)
    gx0 += gA * (r.y1 - r.y2); gx1 += gA * (r.y2 - r.y0); gx2 += gA * (r.y0 - r.y1);
    gy0 += gA * (r.x2 - r.x1); gy1 += gA * (r.x0 - r.x2); gy2 += gA * (r.x1 - r.x0);
    // dists = +-d2 on the nearest edge (a, b)
    const float gd2 = s.inside ? -gd : gd;
    const float ga = gd2 * -2.0f * (1.0f - s.t);
    const float gbv = gd2 * -2.0f * s.t;
    const int ea = s.argmin, eb = (s.argmin + 1) % 3;
    const float gax = ga * s.rx, gay = ga * s.ry, gbx = gbv * s.rx, gby = gbv * s.ry;
    gx0 += (ea == 0 ? gax : 0.0f) + (eb == 0 ? gbx : 0.0f);
    gy0 += (ea == 0 ? gay : 0.0f) + (eb == 0 ? gby : 0.0f);
    gx1 += (ea == 1 ? gax : 0.0f) + (eb == 1 ? gbx : 0.0f);
    gy1 += (ea == 1 ? gay : 0.0f) + (eb == 1 ? gby : 0.0f);
    gx2 += (ea == 2 ? gax : 0.0f) + (eb == 2 ? gbx : 0.0f);
    gy2 += (ea == 2 ? gay : 0.0f) + (eb == 2 ? gby : 0.0f);
    g[0] = gx0; g[1] = gy0; g[2] = gzv0;
    g[3] = gx1; g[4] = gy1; g[5] = gzv1;
    g[6] = gx2; g[7] = gy2; g[8] = gzv2;
}

constexpr int kBwdThreads = kBin * kBin;
constexpr int kListCap = 1024;   // compacted slots per chunk

__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) wave_tot[wave] = x;
    __syncthreads();
    int base = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kBwdThreads / 64; ++w) {
        const int tw = wave_tot[w];
        base += (w < wave) ? tw : 0;
        total += tw;
    }
    __syncthreads();
    return base + x - v;
}

// Tiles come from the grid (one workgroup per tile) or, with the forward's
// workspace, from a queue in the forward's heaviest-first bin order: each
// workgroup takes tiles until it meets a bin without faces (those come last
// and have no filled slot) or the end of the order. SETTINGS holds the
// DMR_RASTER_* bits that change the per-slot evaluation (perspective
// correction, unclipped barycentrics), fixed at compile time so that each
// variant carries only its own arithmetic.
template <uint32_t SETTINGS>
__global__ __launch_bounds__(kBwdThreads) void backward_slots(
    const FaceRec* __restrict__ recs, const int32_t* __restrict__ bin_order, const int32_t* __restrict__ bin_count,
    int32_t* __restrict__ queue, int64_t bins, const float* __restrict__ verts,
    const int64_t* __restrict__ faces, int64_t V, int64_t F, int32_t H, int32_t W, int32_t K, int32_t nbx,
    int32_t nby, const int64_t* __restrict__ pix_to_face, const float* __restrict__ gzb,
    const float* __restrict__ gba, const float* __restrict__ gds, float* __restrict__ grad_verts,
    int32_t use_hash_arg) {
    __shared__ int32_t hkey[kHashSize];
    __shared__ unsigned long long hval[kHashSize][3];
    __shared__ int32_t lface[kListCap];
    __shared__ uint16_t lslot[kListCap];   // tile pixel << 8 | slot
    __shared__ int wave_tot[kBwdThreads / 64];
    __shared__ int64_t tile_s;
    const bool use_hash = use_hash_arg != 0;
    const int64_t per_img = (int64_t)nbx * nby;
    for (int64_t next = blockIdx.x;; next += gridDim.x) {
    if (queue) {
        if (threadIdx.x == 0) {
            const int32_t q = atomicAdd(queue, 1);
            int64_t tb = -1;
            if ((int64_t)q < bins) {
                tb = bin_order[q];
                if (bin_count[tb] == 0) tb = -1;
            }
            tile_s = tb;
        }
        __syncthreads();
    } else if (threadIdx.x == 0) {
        tile_s = next < bins ? next : -1;
    }
    __syncthreads();
    const int64_t b = __builtin_amdgcn_readfirstlane((int32_t)tile_s);
    __syncthreads();   // tile_s is rewritten by the next iteration
    if (b < 0) break;
    const int64_t n = b / per_img;
    const int rem = (int)(b - n * per_img);
    const int by = rem / nbx, bx = rem - (rem / nbx) * nbx;
    const int t = threadIdx.x;
    const int i = by * kBin + t / kBin;
    const int j = bx * kBin + (t % kBin);
    const bool valid = (i < H) && (j < W);
    for (int e = t; e < kHashSize; e += kBwdThreads) {
        hkey[e] = -1;
        hval[e][0] = 0;
        hval[e][1] = 0;
        hval[e][2] = 0;
    }
    const int64_t pbase = valid ? ((((int64_t)n * H + i) * W + j) * K) : 0;
    int c = 0;
    if (valid)
        for (int k = 0; k < K; ++k) c += pix_to_face[pbase + k] >= 0 ? 1 : 0;
    int total = 0;
    const int off = block_exclusive_scan(c, wave_tot, total);
    for (int chunk = 0; chunk < total; chunk += kListCap) {
        for (int k = 0; k < c; ++k) {
            const int e = off + k - chunk;
            if (e >= 0 && e < kListCap) {
                lface[e] = (int32_t)pix_to_face[pbase + k];
                lslot[e] = (uint16_t)((t << 8) | k);
            }
        }
        __syncthreads();
        const int m = min(kListCap, total - chunk);
        for (int e = t; e < m; e += kBwdThreads) {
            const int64_t f = lface[e];
            if (f < 0 || f >= F) continue;
            const int pl = lslot[e] >> 8, slot = lslot[e] & 0xff;
            const int gi = by * kBin + pl / kBin, gj = bx * kBin + pl % kBin;
            FaceRec r;
            int64_t vi[3];
            bool ok;
            if (recs) {
                r = recs[f];
                vi[0] = faces[3 * f + 0];
                vi[1] = faces[3 * f + 1];
                vi[2] = faces[3 * f + 2];
                ok = r.face >= 0 || (vi[0] >= 0 && vi[0] < V && vi[1] >= 0 && vi[1] < V && vi[2] >= 0 && vi[2] < V);
            } else {
                load_face(verts, faces, f, V, r, vi, ok);
            }
            if (!ok) continue;
            const float px = pixel_centre(gj, W), py = pixel_centre(gi, H);
            const int64_t so = (((int64_t)n * H + gi) * W + gj) * K + slot;
            PairState s;
            eval_pair(r, px, py, __builtin_inff(), true, SETTINGS, s);
            const float gz = gzb ? gzb[so] : 0.0f;
            const float gd = gds ? gds[so] : 0.0f;
            const float gb0 = gba ? gba[3 * so + 0] : 0.0f;
            const float gb1 = gba ? gba[3 * so + 1] : 0.0f;
            const float gb2 = gba ? gba[3 * so + 2] : 0.0f;
            float g[9];
            slot_partials(r, s, px, py, gz, gb0, gb1, gb2, gd, SETTINGS, g);
            vertex_add(hkey, hval, grad_verts, vi[0], g[0], g[1], g[2], use_hash);
            vertex_add(hkey, hval, grad_verts, vi[1], g[3], g[4], g[5], use_hash);
            vertex_add(hkey, hval, grad_verts, vi[2], g[6], g[7], g[8], use_hash);
        }
        __syncthreads();
    }
    for (int e = t; e < kHashSize; e += kBwdThreads) {
        const int32_t vid = hkey[e];
        if (vid >= 0) {
            atomicAdd(&grad_verts[3 * (int64_t)vid + 0], from_fixed(hval[e][0]));
            atomicAdd(&grad_verts[3 * (int64_t)vid + 1], from_fixed(hval[e][1]));
            atomicAdd(&grad_verts[3 * (int64_t)vid + 2], from_fixed(hval[e][2]));
        }
    }
    __syncthreads();   // the table is cleared for the next tile
    }
}

template <uint32_t SETTINGS>
static void launch_backward_slots(const BwdArgs& a, bool reuse, const FaceRec* recs, const int32_t* order,
                                  const int32_t* count, int32_t* queue) {
    int64_t grid = a.L.bins;
    if (reuse) {
        // as many workgroups as stay resident; each takes tiles from the queue
        static int resident_per_cu = 0;
        int dev = 0, cus = 0;
        if (resident_per_cu == 0 &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&resident_per_cu, backward_slots<SETTINGS>, kBwdThreads,
                                                         0) != hipSuccess)
            resident_per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        const int64_t resident = (int64_t)std::max(1, cus) * std::max(1, resident_per_cu);
        grid = std::min<int64_t>(grid, resident);
    }
    backward_slots<SETTINGS><<<(unsigned)grid, kBwdThreads, 0, a.stream>>>(
        recs, order, count, queue, a.L.bins, a.verts, a.faces, a.V, a.F, a.H, a.W, a.K, (int32_t)a.L.nbx,
        (int32_t)a.L.nby, a.pix_to_face, a.gz, a.gb, a.gd, a.grad_verts, a.V <= (int64_t)INT32_MAX ? 1 : 0);
}

hipError_t launch_backward(const BwdArgs& a) {
    const int64_t n3 = 3 * a.V;
    const int64_t npix = a.N * (int64_t)a.H * a.W;
    const bool work = npix > 0 && a.F > 0;
    // With the forward's workspace, its per-face records (vertex positions,
    // 1/A, inverse edge lengths) replace the per-slot gathers and divisions,
    // and its bin order and counts drive a tile queue that skips empty bins.
    const bool reuse = a.reuse_forward && work;
    WsHeader* hdr = reuse ? reinterpret_cast<WsHeader*>(a.ws) : nullptr;
    int32_t* queue = reuse ? &hdr->bwd_next : nullptr;
    if (n3 > 0) {
        timing_begin(kKZeroGrad, a.stream);
        zero_f32<<<(unsigned)std::min<int64_t>(2048, (n3 + 255) / 256), 256, 0, a.stream>>>(a.grad_verts, n3, queue);
        timing_end(kKZeroGrad, a.stream);
    }
    if (!work) return hipGetLastError();
    const FaceRec* recs = reuse ? reinterpret_cast<const FaceRec*>(a.ws + a.L.off_records) : nullptr;
    const int32_t* order = reuse ? reinterpret_cast<const int32_t*>(a.ws + a.L.off_perm) : nullptr;
    const int32_t* count = reuse ? reinterpret_cast<const int32_t*>(a.ws + a.L.off_count) : nullptr;
    constexpr uint32_t kP = DMR_RASTER_PERSPECTIVE_CORRECT, kU = DMR_RASTER_UNCLIPPED_BARY;
    timing_begin(kKBackward, a.stream);
    switch (a.settings & (kP | kU)) {
        case 0: launch_backward_slots<0>(a, reuse, recs, order, count, queue); break;
        case kP: launch_backward_slots<kP>(a, reuse, recs, order, count, queue); break;
        case kU: launch_backward_slots<kU>(a, reuse, recs, order, count, queue); break;
        default: launch_backward_slots<kP | kU>(a, reuse, recs, order, count, queue); break;
    }
    timing_end(kKBackward, a.stream);
    return hipGetLastError();
}

}  // namespace dmr
