// Upstream projection on gfx950: world-space vertices of a packed batch of
// meshes to the screen space the rasterizer takes, and its backward pass to
// the vertices and the cameras. The pages differentiate from image pixels
// back to the 3D parameters (rocketrecap summary, "3:52 Differentiable
// Renderer"); the camera model is the library's reading stated in
// include/dmr.h: h = M_n (X, 1), (x, y, z) = (h0 / h3, h1 / h3, h2).
//
// One thread per vertex; 12 bytes in and 12 out per vertex, so the kernels
// are bound by HBM. A workgroup's vertices nearly always belong to one mesh
// (vertices are packed per mesh): its camera is read once into LDS;
// vertices of other meshes (at mesh boundaries) read theirs directly. The
// camera gradient is a separate pass over mesh-aligned slices.
#include <algorithm>

#include "dmr_internal.h"

namespace dmr {

constexpr int kProjThreads = 256;

__device__ __forceinline__ int64_t mesh_of_vertex(const int64_t* __restrict__ off, int64_t N, int64_t v) {
    // last n with off[n] <= v, clamped to [0, N - 1]
    int64_t lo = 0, hi = N - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (off[mid] <= v) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// The block's home mesh (that of its first vertex) and its vertex range.
__device__ __forceinline__ void home_mesh(const int64_t* __restrict__ off, int64_t N, int64_t first, int64_t& home,
                                          int64_t& lo, int64_t& hi) {
    __shared__ int64_t s_home, s_lo, s_hi;
    if (threadIdx.x == 0) {
        const int64_t h = mesh_of_vertex(off, N, first);
        s_home = h;
        s_lo = off[h];
        s_hi = off[h + 1];
    }
    __syncthreads();
    home = s_home;
    lo = s_lo;
    hi = s_hi;
}

struct Homog {
    float h0, h1, h2, h3;
};

// h = M (X, 1), each row a left-to-right sum of four products.
__device__ __forceinline__ Homog apply_camera(const float* m, float x, float y, float z) {
    Homog h;
    h.h0 = ((m[0] * x + m[1] * y) + m[2] * z) + m[3];
    h.h1 = ((m[4] * x + m[5] * y) + m[6] * z) + m[7];
    h.h2 = ((m[8] * x + m[9] * y) + m[10] * z) + m[11];
    h.h3 = ((m[12] * x + m[13] * y) + m[14] * z) + m[15];
    return h;
}

__global__ __launch_bounds__(kProjThreads) void project_forward(const float* __restrict__ verts, int64_t V,
                                                                const int64_t* __restrict__ off, int64_t N,
                                                                const float* __restrict__ cameras,
                                                                float* __restrict__ out) {
    __shared__ float cam[16];
    const int64_t first = (int64_t)blockIdx.x * kProjThreads;
    int64_t home, lo, hi;
    home_mesh(off, N, first, home, lo, hi);
    if (threadIdx.x < 16) cam[threadIdx.x] = cameras[home * 16 + threadIdx.x];
    __syncthreads();
    const int64_t v = first + threadIdx.x;
    if (v >= V) return;
    const float x = verts[3 * v], y = verts[3 * v + 1], z = verts[3 * v + 2];
    const bool in_home = lo <= v && v < hi;
    const float* m = in_home ? cam : cameras + mesh_of_vertex(off, N, v) * 16;
    const Homog h = apply_camera(m, x, y, z);
    out[3 * v + 0] = h.h0 / h.h3;
    out[3 * v + 1] = h.h1 / h.h3;
    out[3 * v + 2] = h.h2;
}

// dL/dh from the gradient g of (x, y, z): (g0 / h3, g1 / h3, g2,
// -(g0 x + g1 y) / h3) with x = h0 / h3, y = h1 / h3.
__device__ __forceinline__ void project_grad_h(const Homog& h, float g0, float g1, float g2, float (&gh)[4]) {
    const float px = h.h0 / h.h3, py = h.h1 / h.h3;
    gh[0] = g0 / h.h3;
    gh[1] = g1 / h.h3;
    gh[2] = g2;
    gh[3] = -(g0 * px + g1 * py) / h.h3;
}

__global__ __launch_bounds__(kProjThreads) void project_backward(
    const float* __restrict__ verts, int64_t V, const int64_t* __restrict__ off, int64_t N,
    const float* __restrict__ cameras, const float* __restrict__ grad_out, float* __restrict__ grad_verts) {
    __shared__ float cam[16];
    const int64_t first = (int64_t)blockIdx.x * kProjThreads;
    int64_t home, lo, hi;
    home_mesh(off, N, first, home, lo, hi);
    if (threadIdx.x < 16) cam[threadIdx.x] = cameras[home * 16 + threadIdx.x];
    __syncthreads();
    const int64_t v = first + threadIdx.x;
    if (v >= V) return;
    const float x = verts[3 * v], y = verts[3 * v + 1], z = verts[3 * v + 2];
    const bool in_home = lo <= v && v < hi;
    const float* m = in_home ? cam : cameras + mesh_of_vertex(off, N, v) * 16;
    const Homog h = apply_camera(m, x, y, z);
    float gh[4];
    project_grad_h(h, grad_out[3 * v], grad_out[3 * v + 1], grad_out[3 * v + 2], gh);
    // dL/dX_c = sum_r M_rc gh_r
    grad_verts[3 * v + 0] = ((m[0] * gh[0] + m[4] * gh[1]) + m[8] * gh[2]) + m[12] * gh[3];
    grad_verts[3 * v + 1] = ((m[1] * gh[0] + m[5] * gh[1]) + m[9] * gh[2]) + m[13] * gh[3];
    grad_verts[3 * v + 2] = ((m[2] * gh[0] + m[6] * gh[1]) + m[10] * gh[2]) + m[14] * gh[3];
}

// Camera gradient dL/dM_n = sum over the mesh's vertices of gh (X, 1)^T.
// Workgroup (n, s) sums slice s of kCamSlices equal slices of mesh n in
// registers, then across the workgroup, and adds the 16 sums with float
// atomics: kCamSlices atomics per entry. (Float atomics on one address
// serialise; one per 256-vertex workgroup over a large mesh cost more than
// the whole pass.)
constexpr int kCamSlices = 16;

__global__ __launch_bounds__(kProjThreads) void project_camera_grad(
    const float* __restrict__ verts, const int64_t* __restrict__ off, const float* __restrict__ cameras,
    const float* __restrict__ grad_out, float* __restrict__ grad_cameras) {
    __shared__ float cam[16];
    __shared__ float part[kProjThreads / 64][16];
    const int64_t n = blockIdx.x / kCamSlices;
    const int s = (int)(blockIdx.x % kCamSlices);
    const int64_t lo = off[n], hi = off[n + 1];
    const int64_t len = hi > lo ? hi - lo : 0;
    const int64_t per = (len + kCamSlices - 1) / kCamSlices;
    const int64_t a = lo + s * per;
    const int64_t b = a + per < hi ? a + per : hi;
    if (a >= b) return;   // uniform over the workgroup
    if (threadIdx.x < 16) cam[threadIdx.x] = cameras[n * 16 + threadIdx.x];
    __syncthreads();
    float gm[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) gm[e] = 0.0f;
    for (int64_t v = a + threadIdx.x; v < b; v += kProjThreads) {
        const float x = verts[3 * v], y = verts[3 * v + 1], z = verts[3 * v + 2];
        const Homog h = apply_camera(cam, x, y, z);
        float gh[4];
        project_grad_h(h, grad_out[3 * v], grad_out[3 * v + 1], grad_out[3 * v + 2], gh);
        const float xh[4] = {x, y, z, 1.0f};
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) gm[4 * r + c] += gh[r] * xh[c];
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        float t = gm[e];
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) t += __shfl_xor(t, d, 64);
        if (lane == 0) part[wave][e] = t;
    }
    __syncthreads();
    if (threadIdx.x < 16) {
        float t = 0.0f;
#pragma unroll
        for (int w = 0; w < kProjThreads / 64; ++w) t += part[w][threadIdx.x];
        atomicAdd(&grad_cameras[n * 16 + threadIdx.x], t);
    }
}

__global__ void zero_cameras(float* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t k = i; k < n; k += stride) p[k] = 0.0f;
}

static unsigned proj_grid(int64_t V) { return (unsigned)((V + kProjThreads - 1) / kProjThreads); }

hipError_t launch_project_forward(const ProjectArgs& a) {
    if (a.V == 0) return hipSuccess;
    timing_begin(kKProjectFwd, a.stream);
    project_forward<<<proj_grid(a.V), kProjThreads, 0, a.stream>>>(a.verts, a.V, a.off, a.N, a.cameras, a.out);
    timing_end(kKProjectFwd, a.stream);
    return hipGetLastError();
}

hipError_t launch_project_backward(const ProjectArgs& a) {
    timing_begin(kKProjectBwd, a.stream);
    if (a.V > 0)
        project_backward<<<proj_grid(a.V), kProjThreads, 0, a.stream>>>(a.verts, a.V, a.off, a.N, a.cameras,
                                                                        a.grad_out, a.grad_verts);
    if (a.grad_cameras && a.N > 0) {
        zero_cameras<<<(unsigned)std::min<int64_t>(64, (16 * a.N + 255) / 256), 256, 0, a.stream>>>(a.grad_cameras,
                                                                                                  16 * a.N);
        if (a.V > 0)
            project_camera_grad<<<(unsigned)(a.N * kCamSlices), kProjThreads, 0, a.stream>>>(
                a.verts, a.off, a.cameras, a.grad_out, a.grad_cameras);
    }
    timing_end(kKProjectBwd, a.stream);
    return hipGetLastError();
}

}  // namespace dmr
