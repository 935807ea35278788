// Backward pass of the K-nearest-face rasterizer on gfx950: gradients flow
// from the per-pixel outputs back to vertex positions (rocketrecap summary of
// the PyTorch3D walkthrough, "3:52 Differentiable Renderer").
//
// One thread per pixel walks its filled slots (padding is a suffix), re-runs
// the forward evaluation of that (pixel, face) pair, applies the chain rule
// of zbuf = sum bh_k z_k, bh = clip(b)/S, b = w/A and dists = +-|q - t u|^2
// (t held at its minimiser or clamp), and sums the nine partials per vertex,
// first in LDS per 16x16 tile, then into grad_verts with float32 atomics.
#include <algorithm>

#include "dmr_internal.h"

namespace dmr {

__global__ void zero_f32(float* p, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
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

// Per-slot chain rule. Returns the nine partials (x, y, z of the three
// vertices) of L = gz*zbuf + gb.bary + gd*dists for one filled slot.
__device__ __forceinline__ void slot_partials(const FaceRec& r, const PairState& s, float px, float py, float gz,
                                              float gbh0, float gbh1, float gbh2, float gd, float (&g)[9]) {
    // depth
    const float gzv0 = gz * s.bh0, gzv1 = gz * s.bh1, gzv2 = gz * s.bh2;
    gbh0 = gbh0 + gz * r.z0;
    gbh1 = gbh1 + gz * r.z1;
    gbh2 = gbh2 + gz * r.z2;
    // renormalisation and clip
    const float dot = (gbh0 * s.bh0 + gbh1 * s.bh1) + gbh2 * s.bh2;
    const float gb0 = (s.b0 > 0.0f && s.b0 < 1.0f) ? (gbh0 - dot) * s.invS : 0.0f;
    const float gb1 = (s.b1 > 0.0f && s.b1 < 1.0f) ? (gbh1 - dot) * s.invS : 0.0f;
    const float gb2 = (s.b2 > 0.0f && s.b2 < 1.0f) ? (gbh2 - dot) * s.invS : 0.0f;
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

// One workgroup per 16x16 pixel tile, one thread per pixel. Partials are
// first summed per vertex in an LDS hash table (open addressing, LDS float
// atomics), so that neighbouring pixels covered by the same faces do not
// hammer the same global addresses; the table is then flushed with one
// global float atomic per (tile, vertex, coordinate). A vertex that finds no
// free entry within the probe limit goes straight to global atomics.
constexpr int kBwdThreads = kBin * kBin;
constexpr int kHashSize = 2048;
constexpr int kProbe = 16;

__global__ __launch_bounds__(kBwdThreads) void backward_tiles(
    const float* __restrict__ verts, int64_t V, const int64_t* __restrict__ faces, int64_t F, int32_t H,
    int32_t W, int32_t K, int32_t nbx, int32_t nby, const int64_t* __restrict__ pix_to_face,
    const float* __restrict__ gzb, const float* __restrict__ gba, const float* __restrict__ gds,
    float* __restrict__ grad_verts, int32_t use_hash) {
    __shared__ int32_t hkey[kHashSize];
    __shared__ float hval[kHashSize][3];
    const int64_t b = blockIdx.x;
    const int64_t per_img = (int64_t)nbx * nby;
    const int64_t n = b / per_img;
    const int rem = (int)(b - n * per_img);
    const int by = rem / nbx, bx = rem - (rem / nbx) * nbx;
    const int t = threadIdx.x;
    const int i = by * kBin + t / kBin;
    const int j = bx * kBin + (t % kBin);
    const bool valid = (i < H) && (j < W);
    for (int e = t; e < kHashSize; e += kBwdThreads) {
        hkey[e] = -1;
        hval[e][0] = 0.0f;
        hval[e][1] = 0.0f;
        hval[e][2] = 0.0f;
    }
    __syncthreads();
    if (valid) {
        const float px = pixel_centre(j, W);
        const float py = pixel_centre(i, H);
        const int64_t pix = ((int64_t)n * H + i) * W + j;
        for (int k = 0; k < K; ++k) {
            const int64_t so = pix * K + k;
            const int64_t f = pix_to_face[so];
            if (f < 0) break;
            if (f >= F) continue;
            FaceRec r;
            int64_t vi[3];
            bool ok;
            load_face(verts, faces, f, V, r, vi, ok);
            if (!ok) continue;
            PairState s;
            eval_pair(r, px, py, __builtin_inff(), true, s);
            const float gz = gzb ? gzb[so] : 0.0f;
            const float gd = gds ? gds[so] : 0.0f;
            const float gb0 = gba ? gba[3 * so + 0] : 0.0f;
            const float gb1 = gba ? gba[3 * so + 1] : 0.0f;
            const float gb2 = gba ? gba[3 * so + 2] : 0.0f;
            float g[9];
            slot_partials(r, s, px, py, gz, gb0, gb1, gb2, gd, g);
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                bool placed = false;
                if (use_hash) {
                    const int32_t vid = (int32_t)vi[c];
                    uint32_t h = ((uint32_t)vid * 2654435761u) >> (32 - 11);
                    for (int p = 0; p < kProbe; ++p) {
                        int32_t cur = hkey[h];
                        if (cur == -1) cur = atomicCAS(&hkey[h], -1, vid);
                        if (cur == -1 || cur == vid) {
                            atomicAdd(&hval[h][0], g[3 * c + 0]);
                            atomicAdd(&hval[h][1], g[3 * c + 1]);
                            atomicAdd(&hval[h][2], g[3 * c + 2]);
                            placed = true;
                            break;
                        }
                        h = (h + 1) & (kHashSize - 1);
                    }
                }
                if (!placed) {
                    atomicAdd(&grad_verts[3 * vi[c] + 0], g[3 * c + 0]);
                    atomicAdd(&grad_verts[3 * vi[c] + 1], g[3 * c + 1]);
                    atomicAdd(&grad_verts[3 * vi[c] + 2], g[3 * c + 2]);
                }
            }
        }
    }
    __syncthreads();
    for (int e = t; e < kHashSize; e += kBwdThreads) {
        const int32_t vid = hkey[e];
        if (vid >= 0) {
            atomicAdd(&grad_verts[3 * (int64_t)vid + 0], hval[e][0]);
            atomicAdd(&grad_verts[3 * (int64_t)vid + 1], hval[e][1]);
            atomicAdd(&grad_verts[3 * (int64_t)vid + 2], hval[e][2]);
        }
    }
}

hipError_t launch_backward(const BwdArgs& a) {
    const int64_t n3 = 3 * a.V;
    if (n3 > 0) {
        timing_begin(kKZeroGrad, a.stream);
        zero_f32<<<(unsigned)std::min<int64_t>(2048, (n3 + 255) / 256), 256, 0, a.stream>>>(a.grad_verts, n3);
        timing_end(kKZeroGrad, a.stream);
    }
    const int64_t npix = a.N * (int64_t)a.H * a.W;
    if (npix > 0 && a.F > 0) {
        const int32_t nbx = (a.W + kBin - 1) / kBin, nby = (a.H + kBin - 1) / kBin;
        const int64_t tiles = a.N * nbx * nby;
        timing_begin(kKBackward, a.stream);
        backward_tiles<<<(unsigned)tiles, kBwdThreads, 0, a.stream>>>(
            a.verts, a.V, a.faces, a.F, a.H, a.W, a.K, nbx, nby, a.pix_to_face, a.gz, a.gb, a.gd, a.grad_verts,
            a.V <= (int64_t)INT32_MAX ? 1 : 0);
        timing_end(kKBackward, a.stream);
    }
    return hipGetLastError();
}

}  // namespace dmr
