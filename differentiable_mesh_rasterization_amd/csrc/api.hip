// C ABI of libdmr (include/dmr.h): host-side validation, workspace layout,
// launch sequencing and optional per-kernel event timing.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "dmr_internal.h"

namespace dmr {

// ---------------------------------------------------------------------------
// per-kernel event timing
// ---------------------------------------------------------------------------
namespace {

struct Pending {
    hipEvent_t start, stop;
};

struct Timing {
    std::vector<Pending> pending[kKernelCount];
    std::vector<hipEvent_t> pool;
    double total_ms[kKernelCount] = {};
    int64_t launches[kKernelCount] = {};
    hipEvent_t open_start[kKernelCount] = {};
};

// The bookkeeping below is shared by every host thread that launches
// kernels: it is only touched under g_timing_mu. The mask (bit id set:
// kernel id is timed) is read without the lock on every launch.
Timing g_timing;
std::mutex g_timing_mu;
std::atomic<uint32_t> g_timing_mask{0};

const char* const kKernelNames[kKernelCount] = {
    "zero_fwd", "face_setup_count", "bin_scan", "bin_fill", "bin_sort", "fine_raster", "zero_grad", "backward_slots",
    "blend_fwd", "blend_bwd", "project_fwd", "project_bwd", "point_setup", "point_raster", "point_bwd",
};

hipEvent_t take_event() {
    if (!g_timing.pool.empty()) {
        hipEvent_t e = g_timing.pool.back();
        g_timing.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

hipError_t drain(int id) {
    for (auto& p : g_timing.pending[id]) {
        hipError_t err = hipEventSynchronize(p.stop);
        if (err != hipSuccess) return err;
        float ms = 0.0f;
        err = hipEventElapsedTime(&ms, p.start, p.stop);
        if (err != hipSuccess) return err;
        g_timing.total_ms[id] += ms;
        g_timing.launches[id] += 1;
        g_timing.pool.push_back(p.start);
        g_timing.pool.push_back(p.stop);
    }
    g_timing.pending[id].clear();
    return hipSuccess;
}

}  // namespace

void timing_begin(KernelId id, hipStream_t s) {
    if (!(g_timing_mask.load(std::memory_order_relaxed) >> id & 1u)) return;
    std::lock_guard<std::mutex> lk(g_timing_mu);
    hipEvent_t e = take_event();
    if (e && hipEventRecord(e, s) == hipSuccess) g_timing.open_start[id] = e;
}

void timing_end(KernelId id, hipStream_t s) {
    if (!(g_timing_mask.load(std::memory_order_relaxed) >> id & 1u)) return;
    std::lock_guard<std::mutex> lk(g_timing_mu);
    if (!g_timing.open_start[id]) return;
    hipEvent_t e = take_event();
    if (e && hipEventRecord(e, s) == hipSuccess) g_timing.pending[id].push_back({g_timing.open_start[id], e});
    g_timing.open_start[id] = nullptr;
}

}  // namespace dmr

using namespace dmr;

namespace {

bool mul_overflows(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return true;
    if (a != 0 && b > INT64_MAX / a) return true;
    *out = a * b;
    return false;
}

// Shared validation of the geometry arguments. Returns DMR_SUCCESS or the
// status to report.
dmr_status check_geometry(const float* verts, int64_t V, const int64_t* faces, int64_t F,
                          const int64_t* off, int64_t N, int32_t H, int32_t W, int32_t K,
                          int64_t* slots_out) {
    if (V < 0 || F < 0 || N < 0) return DMR_ERROR_INVALID_VALUE;
    if (H < 1 || W < 1 || K < 1) return DMR_ERROR_INVALID_VALUE;
    if (H > DMR_MAX_IMAGE_SIDE || W > DMR_MAX_IMAGE_SIDE || K > DMR_MAX_K) return DMR_ERROR_UNSUPPORTED;
    if (F > (int64_t)INT32_MAX - 1) return DMR_ERROR_UNSUPPORTED;  // face ids are 32-bit inside
    if (V > INT64_MAX / 3) return DMR_ERROR_UNSUPPORTED;
    int64_t pix, slots, slots3;
    if (mul_overflows(N, (int64_t)H * W, &pix)) return DMR_ERROR_UNSUPPORTED;
    if (mul_overflows(pix, K, &slots)) return DMR_ERROR_UNSUPPORTED;
    if (mul_overflows(slots, 3, &slots3)) return DMR_ERROR_UNSUPPORTED;
    if (F > 0 && faces == nullptr) return DMR_ERROR_INVALID_VALUE;
    if (V > 0 && verts == nullptr) return DMR_ERROR_INVALID_VALUE;
    if (N > 0 && off == nullptr) return DMR_ERROR_INVALID_VALUE;
    *slots_out = slots;
    return DMR_SUCCESS;
}

}  // namespace

// The kernels read the workspace's per-face records and bin tables with
// 16-byte vector accesses at 256-byte aligned offsets from its start.
static bool ws_aligned(const void* workspace) {
    return (reinterpret_cast<uintptr_t>(workspace) & 15) == 0;
}

extern "C" {

const char* dmr_status_string(dmr_status s) {
    switch (s) {
        case DMR_SUCCESS: return "success";
        case DMR_ERROR_INVALID_VALUE: return "invalid argument";
        case DMR_ERROR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case DMR_ERROR_HIP: return "HIP runtime error";
        case DMR_ERROR_UNSUPPORTED: return "unsupported size or parameter";
    }
    return "unknown status";
}

size_t dmr_workspace_min_size(int64_t N, int64_t F, int32_t H, int32_t W) {
    if (N < 0 || F < 0 || H < 1 || W < 1 || H > DMR_MAX_IMAGE_SIDE || W > DMR_MAX_IMAGE_SIDE) return 0;
    return fwd_layout(N, F, H, W).min_bytes;
}

size_t dmr_workspace_size_hint(int64_t N, int64_t F, int32_t H, int32_t W, int32_t K, float blur_radius) {
    (void)K;
    size_t base = dmr_workspace_min_size(N, F, H, W);
    if (base == 0 || !(blur_radius >= 0.0f) || !isfinite(blur_radius)) return 0;
    FwdLayout L = fwd_layout(N, F, H, W);
    // Face boxes grow by the blur radius (in pixels: sqrt(blur) * side / 2);
    // allow each face the bins of a box one blur diameter wider than a bin.
    double rpx = sqrt((double)blur_radius) * 0.5 * (double)(H > W ? H : W);
    double per_face = (1.0 + (2.0 * rpx + 2.0) / kBin) * (1.0 + (2.0 * rpx + 2.0) / kBin);
    double entries = 2.0 * per_face * (double)F + 4.0 * (double)L.bins + 1024.0;
    if (entries > (double)INT32_MAX) entries = (double)INT32_MAX;
    return align_up(base + (size_t)entries * sizeof(int32_t), 256);
}

dmr_status rasterize_meshes_fwd(const float* verts, int64_t V, const int64_t* faces, int64_t F,
                                const int64_t* mesh_face_offsets, int64_t N, int32_t H, int32_t W, int32_t K,
                                float blur_radius, int64_t* pix_to_face, float* zbuf, float* bary,
                                float* dists, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return rasterize_meshes_fwd_ex(verts, V, faces, F, mesh_face_offsets, N, H, W, K, blur_radius, pix_to_face, zbuf,
                                   bary, dists, workspace, workspace_bytes, 0u, stream);
}

dmr_status rasterize_meshes_fwd_ex(const float* verts, int64_t V, const int64_t* faces, int64_t F,
                                   const int64_t* mesh_face_offsets, int64_t N, int32_t H, int32_t W, int32_t K,
                                   float blur_radius, int64_t* pix_to_face, float* zbuf, float* bary,
                                   float* dists, void* workspace, size_t workspace_bytes, uint32_t flags,
                                   hipStream_t stream) {
    int64_t slots = 0;
    dmr_status st = check_geometry(verts, V, faces, F, mesh_face_offsets, N, H, W, K, &slots);
    if (st != DMR_SUCCESS) return st;
    if (!isfinite(blur_radius) || blur_radius < 0.0f) return DMR_ERROR_INVALID_VALUE;
    if ((flags & ~(uint32_t)DMR_RASTER_SETTINGS) != 0) return DMR_ERROR_INVALID_VALUE;
    if (slots == 0) return DMR_SUCCESS;
    if (!pix_to_face || !zbuf || !bary || !dists) return DMR_ERROR_INVALID_VALUE;
    FwdLayout L = fwd_layout(N, F, H, W);
    // work items of the fine pass are bin << 3 | part in 32 bits, four per bin at most
    if (L.bins >= ((int64_t)1 << 28)) return DMR_ERROR_UNSUPPORTED;
    if (workspace == nullptr || workspace_bytes < L.min_bytes) return DMR_ERROR_WORKSPACE_TOO_SMALL;
    if (!ws_aligned(workspace)) return DMR_ERROR_INVALID_VALUE;
    int64_t cap = (int64_t)((workspace_bytes - L.min_bytes) / sizeof(int32_t));
    if (cap > (int64_t)INT32_MAX) cap = INT32_MAX;

    FwdArgs a;
    a.verts = verts; a.V = V; a.faces = faces; a.F = F; a.off = mesh_face_offsets; a.N = N;
    a.H = H; a.W = W; a.K = K; a.blur = blur_radius; a.settings = flags;
    a.points = nullptr; a.radius = 0.0f;
    a.pix_to_face = pix_to_face; a.zbuf = zbuf; a.bary = bary; a.dists = dists;
    a.ws = static_cast<char*>(workspace); a.ws_bytes = workspace_bytes;
    a.L = L; a.capacity = cap; a.stream = stream;
    return launch_forward(a) == hipSuccess ? DMR_SUCCESS : DMR_ERROR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// allocation-free forward: its workspace is a file-scope device array
// ---------------------------------------------------------------------------
// Every device the library runs on holds its own copy of `scratch` until the
// process ends. Host code never passes the array's name to a kernel or a
// copy (on the host it only stands for the symbol): the device address is
// looked up once per device with hipGetSymbolAddress and used from then on.
static __device__ __align__(256) unsigned char scratch[DMR_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// This device's `scratch`: the device of `stream` (the current device for
// the null stream), looked up on first use with that device current.
dmr_status scratch_for(hipStream_t stream, void** out) {
    int dev = 0;
    if (stream == nullptr) {
        if (hipGetDevice(&dev) != hipSuccess) return DMR_ERROR_HIP;
    } else if (hipStreamGetDevice(stream, &dev) != hipSuccess) {
        return DMR_ERROR_HIP;
    }
    if (dev < 0 || dev >= kMaxScratchDevices) return DMR_ERROR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return DMR_ERROR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return DMR_ERROR_HIP;
        void* p = nullptr;
        const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return DMR_ERROR_HIP;
        if (err != hipSuccess || p == nullptr) return DMR_ERROR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DMR_SUCCESS;
}

}  // namespace

extern "C" {

dmr_status rasterize_meshes_fwd_noalloc(const float* verts, int64_t V, const int64_t* faces, int64_t F,
                                        const int64_t* mesh_face_offsets, int64_t N, int32_t H, int32_t W,
                                        int32_t K, float blur_radius, int64_t* pix_to_face, float* zbuf, float* bary,
                                        float* dists, hipStream_t stream) {
    int64_t slots = 0;
    dmr_status st = check_geometry(verts, V, faces, F, mesh_face_offsets, N, H, W, K, &slots);
    if (st != DMR_SUCCESS) return st;
    if (!isfinite(blur_radius) || blur_radius < 0.0f) return DMR_ERROR_INVALID_VALUE;
    if (slots == 0) return DMR_SUCCESS;
    if (!pix_to_face || !zbuf || !bary || !dists) return DMR_ERROR_INVALID_VALUE;
    // face records and bin tables must fit; bin lists that do not fit take
    // the exact full-face-range path, as with any small workspace
    if (fwd_layout(N, F, H, W).min_bytes > (size_t)DMR_NOALLOC_SCRATCH_BYTES) return DMR_ERROR_UNSUPPORTED;
    void* ws = nullptr;
    st = scratch_for(stream, &ws);
    if (st != DMR_SUCCESS) return st;
    return rasterize_meshes_fwd_ex(verts, V, faces, F, mesh_face_offsets, N, H, W, K, blur_radius, pix_to_face,
                                   zbuf, bary, dists, ws, (size_t)DMR_NOALLOC_SCRATCH_BYTES, 0u, stream);
}

dmr_status rasterize_meshes_bwd(const float* verts, int64_t V, const int64_t* faces, int64_t F,
                                const int64_t* mesh_face_offsets, int64_t N, int32_t H, int32_t W, int32_t K,
                                float blur_radius, const int64_t* pix_to_face, const float* grad_zbuf,
                                const float* grad_bary, const float* grad_dists, float* grad_verts, void* workspace,
                                size_t workspace_bytes, uint32_t flags, hipStream_t stream) {
    int64_t slots = 0;
    dmr_status st = check_geometry(verts, V, faces, F, mesh_face_offsets, N, H, W, K, &slots);
    if (st != DMR_SUCCESS) return st;
    if (!isfinite(blur_radius) || blur_radius < 0.0f) return DMR_ERROR_INVALID_VALUE;
    if ((flags & ~(uint32_t)(DMR_BWD_REUSE_FORWARD_WORKSPACE | DMR_RASTER_SETTINGS)) != 0)
        return DMR_ERROR_INVALID_VALUE;
    if (V > 0 && grad_verts == nullptr) return DMR_ERROR_INVALID_VALUE;
    if (slots > 0 && pix_to_face == nullptr) return DMR_ERROR_INVALID_VALUE;
    if (V == 0) return DMR_SUCCESS;
    FwdLayout L = fwd_layout(N, F, H, W);
    if (L.bins >= ((int64_t)1 << 28)) return DMR_ERROR_UNSUPPORTED;  // as in the forward pass
    const bool reuse = (flags & DMR_BWD_REUSE_FORWARD_WORKSPACE) != 0;
    if (reuse && slots > 0 && (workspace == nullptr || workspace_bytes < L.min_bytes))
        return DMR_ERROR_WORKSPACE_TOO_SMALL;
    if (reuse && slots > 0 && !ws_aligned(workspace)) return DMR_ERROR_INVALID_VALUE;
    int64_t cap = (reuse && slots > 0) ? (int64_t)((workspace_bytes - L.min_bytes) / sizeof(int32_t)) : 0;
    if (cap > (int64_t)INT32_MAX) cap = INT32_MAX;
    BwdArgs a;
    a.verts = verts; a.V = V; a.faces = faces; a.F = F; a.off = mesh_face_offsets; a.N = N;
    a.H = H; a.W = W; a.K = K; a.blur = blur_radius; a.settings = flags & DMR_RASTER_SETTINGS;
    a.pix_to_face = pix_to_face;
    a.gz = grad_zbuf; a.gb = grad_bary; a.gd = grad_dists; a.grad_verts = grad_verts;
    a.ws = static_cast<char*>(workspace); a.ws_bytes = workspace_bytes; a.L = L; a.capacity = cap;
    a.reuse_forward = reuse;
    a.stream = stream;
    return launch_backward(a) == hipSuccess ? DMR_SUCCESS : DMR_ERROR_HIP;
}

namespace {

dmr_status check_blend(const int64_t* pix_to_face, const float* zbuf, const float* dists, int64_t P, int32_t K,
                       const float* colors, int64_t F, const dmr_blend_params* params) {
    if (P < 0 || F < 0 || K < 1 || params == nullptr) return DMR_ERROR_INVALID_VALUE;
    if (K > DMR_MAX_K) return DMR_ERROR_UNSUPPORTED;
    // face indices are staged as int32; one 64-pixel workgroup per grid entry
    if (F > INT32_MAX || P > (int64_t)INT32_MAX * 64) return DMR_ERROR_UNSUPPORTED;
    int64_t slots = 0;
    if (mul_overflows(P, K, &slots) || slots > INT64_MAX / 3) return DMR_ERROR_UNSUPPORTED;
    const dmr_blend_params& p = *params;
    if (!(p.sigma > 0.0f) || !isfinite(p.sigma) || !(p.gamma > 0.0f) || !isfinite(p.gamma)) return DMR_ERROR_INVALID_VALUE;
    if (!isfinite(p.znear) || !isfinite(p.zfar) || !(p.zfar > p.znear) || !isfinite(p.eps)) return DMR_ERROR_INVALID_VALUE;
    for (int c = 0; c < 3; ++c)
        if (!isfinite(p.background[c])) return DMR_ERROR_INVALID_VALUE;
    if (P > 0 && (!pix_to_face || !zbuf || !dists)) return DMR_ERROR_INVALID_VALUE;
    if (F > 0 && !colors) return DMR_ERROR_INVALID_VALUE;
    return DMR_SUCCESS;
}

}  // namespace

dmr_status dmr_blend_fwd(const int64_t* pix_to_face, const float* zbuf, const float* dists, int64_t P, int32_t K,
                         const float* face_colors, int64_t F, const dmr_blend_params* params, float* rgba,
                         hipStream_t stream) {
    dmr_status st = check_blend(pix_to_face, zbuf, dists, P, K, face_colors, F, params);
    if (st != DMR_SUCCESS) return st;
    if (P == 0) return DMR_SUCCESS;
    if (!rgba || reinterpret_cast<uintptr_t>(rgba) % 16 != 0) return DMR_ERROR_INVALID_VALUE;
    BlendArgs a{};
    a.pix_to_face = pix_to_face; a.zbuf = zbuf; a.dists = dists; a.P = P; a.K = K;
    a.colors = face_colors; a.F = F; a.prm = *params; a.rgba = rgba; a.stream = stream;
    return launch_blend_forward(a) == hipSuccess ? DMR_SUCCESS : DMR_ERROR_HIP;
}

dmr_status dmr_blend_bwd(const int64_t* pix_to_face, const float* zbuf, const float* dists, int64_t P, int32_t K,
                         const float* face_colors, int64_t F, const dmr_blend_params* params,
                         const float* grad_rgba, float* grad_zbuf, float* grad_dists, hipStream_t stream) {
    dmr_status st = check_blend(pix_to_face, zbuf, dists, P, K, face_colors, F, params);
    if (st != DMR_SUCCESS) return st;
    if (P == 0) return DMR_SUCCESS;
    if (!grad_rgba || !grad_zbuf || !grad_dists || reinterpret_cast<uintptr_t>(grad_rgba) % 16 != 0)
        return DMR_ERROR_INVALID_VALUE;
    BlendArgs a{};
    a.pix_to_face = pix_to_face; a.zbuf = zbuf; a.dists = dists; a.P = P; a.K = K;
    a.colors = face_colors; a.F = F; a.prm = *params; a.grad_rgba = grad_rgba; a.grad_zbuf = grad_zbuf;
    a.grad_dists = grad_dists; a.stream = stream;
    return launch_blend_backward(a) == hipSuccess ? DMR_SUCCESS : DMR_ERROR_HIP;
}

namespace {

dmr_status check_project(const float* verts, int64_t V, const int64_t* off, int64_t N, const float* cameras) {
    if (V < 0 || N < 0) return DMR_ERROR_INVALID_VALUE;
    if (V > INT64_MAX / 3 || N > INT64_MAX / 16) return DMR_ERROR_UNSUPPORTED;
    // one 256-vertex workgroup per grid entry
    if (V > (int64_t)UINT32_MAX * 256) return DMR_ERROR_UNSUPPORTED;
    // the camera gradient takes 16 workgroups per mesh
    if (N > (int64_t)(UINT32_MAX / 16)) return DMR_ERROR_UNSUPPORTED;
    if (V > 0 && (N == 0 || !verts || !off || !cameras)) return DMR_ERROR_INVALID_VALUE;
    return DMR_SUCCESS;
}

}  // namespace

dmr_status dmr_project_fwd(const float* verts_world, int64_t V, const int64_t* mesh_vert_offsets, int64_t N,
                           const float* cameras, float* verts_ndc, hipStream_t stream) {
    dmr_status st = check_project(verts_world, V, mesh_vert_offsets, N, cameras);
    if (st != DMR_SUCCESS) return st;
    if (V == 0) return DMR_SUCCESS;
    if (!verts_ndc) return DMR_ERROR_INVALID_VALUE;
    ProjectArgs a{};
    a.verts = verts_world; a.V = V; a.off = mesh_vert_offsets; a.N = N; a.cameras = cameras; a.out = verts_ndc;
    a.stream = stream;
    return launch_project_forward(a) == hipSuccess ? DMR_SUCCESS : DMR_ERROR_HIP;
}

dmr_status dmr_project_bwd(const float* verts_world, int64_t V, const int64_t* mesh_vert_offsets, int64_t N,
                           const float* cameras, const float* grad_verts_ndc, float* grad_verts_world,
                           float* grad_cameras, hipStream_t stream) {
    dmr_status st = check_project(verts_world, V, mesh_vert_offsets, N, cameras);
    if (st != DMR_SUCCESS) return st;
    if (V > 0 && (!grad_verts_ndc || !grad_verts_world)) return DMR_ERROR_INVALID_VALUE;
    if (V == 0 && (N == 0 || grad_cameras == nullptr)) return DMR_SUCCESS;
    ProjectArgs a{};
    a.verts = verts_world; a.V = V; a.off = mesh_vert_offsets; a.N = N; a.cameras = cameras;
    a.grad_out = grad_verts_ndc; a.grad_verts = grad_verts_world; a.grad_cameras = grad_cameras;
    a.stream = stream;
    return launch_project_backward(a) == hipSuccess ? DMR_SUCCESS : DMR_ERROR_HIP;
}

size_t dmr_points_workspace_min_size(int64_t N, int64_t P, int32_t H, int32_t W) {
    if (N < 0 || P < 0 || H < 1 || W < 1 || H > DMR_MAX_IMAGE_SIDE || W > DMR_MAX_IMAGE_SIDE) return 0;
    return fwd_layout(N, P, H, W, sizeof(PointRec)).min_bytes;
}

size_t dmr_points_workspace_size_hint(int64_t N, int64_t P, int32_t H, int32_t W, int32_t K, float radius) {
    (void)K;
    size_t base = dmr_points_workspace_min_size(N, P, H, W);
    if (base == 0 || !(radius >= 0.0f) || !isfinite(radius)) return 0;
    FwdLayout L = fwd_layout(N, P, H, W, sizeof(PointRec));
    // a point's box is 2 radius wide: the bins of a box one bin wider than that
    double rpx = (double)radius * 0.5 * (double)(H > W ? H : W);
    double per_point = (1.0 + (2.0 * rpx + 2.0) / kBin) * (1.0 + (2.0 * rpx + 2.0) / kBin);
    double entries = 2.0 * per_point * (double)P + 4.0 * (double)L.bins + 1024.0;
    if (entries > (double)INT32_MAX) entries = (double)INT32_MAX;
    return align_up(base + (size_t)entries * sizeof(int32_t), 256);
}

namespace {

dmr_status check_points(const float* points, int64_t P, const int64_t* off, int64_t N, int32_t H, int32_t W,
                        int32_t K, int64_t* slots_out) {
    if (P < 0 || N < 0 || H < 1 || W < 1 || K < 1) return DMR_ERROR_INVALID_VALUE;
    if (H > DMR_MAX_IMAGE_SIDE || W > DMR_MAX_IMAGE_SIDE || K > DMR_MAX_K) return DMR_ERROR_UNSUPPORTED;
    if (P > (int64_t)INT32_MAX - 1) return DMR_ERROR_UNSUPPORTED;   // point ids are 32-bit inside
    int64_t pix, slots;
    if (mul_overflows(N, (int64_t)H * W, &pix) || mul_overflows(pix, K, &slots)) return DMR_ERROR_UNSUPPORTED;
    if (slots > (int64_t)UINT32_MAX * 256) return DMR_ERROR_UNSUPPORTED;
    if (P > 0 && points == nullptr) return DMR_ERROR_INVALID_VALUE;
    if (N > 0 && off == nullptr) return DMR_ERROR_INVALID_VALUE;
    *slots_out = slots;
    return DMR_SUCCESS;
}

}  // namespace

dmr_status rasterize_points_fwd(const float* points, int64_t P, const int64_t* cloud_offsets, int64_t N, int32_t H,
                                int32_t W, int32_t K, float radius, int64_t* idx, float* zbuf, float* dists,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int64_t slots = 0;
    dmr_status st = check_points(points, P, cloud_offsets, N, H, W, K, &slots);
    if (st != DMR_SUCCESS) return st;
    if (!isfinite(radius) || radius < 0.0f) return DMR_ERROR_INVALID_VALUE;
    if (slots == 0) return DMR_SUCCESS;
    if (!idx || !zbuf || !dists) return DMR_ERROR_INVALID_VALUE;
    FwdLayout L = fwd_layout(N, P, H, W, sizeof(PointRec));
    if (L.bins >= ((int64_t)1 << 28)) return DMR_ERROR_UNSUPPORTED;
    if (workspace == nullptr || workspace_bytes < L.min_bytes) return DMR_ERROR_WORKSPACE_TOO_SMALL;
    if (!ws_aligned(workspace)) return DMR_ERROR_INVALID_VALUE;
    int64_t cap = (int64_t)((workspace_bytes - L.min_bytes) / sizeof(int32_t));
    if (cap > (int64_t)INT32_MAX) cap = INT32_MAX;
    FwdArgs a{};
    a.verts = nullptr; a.V = 0; a.faces = nullptr; a.F = P; a.off = cloud_offsets; a.N = N;
    a.H = H; a.W = W; a.K = K; a.blur = 0.0f; a.settings = 0u;
    a.points = points; a.radius = radius;
    a.pix_to_face = idx; a.zbuf = zbuf; a.bary = nullptr; a.dists = dists;
    a.ws = static_cast<char*>(workspace); a.ws_bytes = workspace_bytes;
    a.L = L; a.capacity = cap; a.stream = stream;
    return launch_points_forward(a) == hipSuccess ? DMR_SUCCESS : DMR_ERROR_HIP;
}

dmr_status rasterize_points_bwd(const float* points, int64_t P, const int64_t* cloud_offsets, int64_t N, int32_t H,
                                int32_t W, int32_t K, const int64_t* idx, const float* grad_zbuf,
                                const float* grad_dists, float* grad_points, hipStream_t stream) {
    int64_t slots = 0;
    dmr_status st = check_points(points, P, cloud_offsets, N, H, W, K, &slots);
    if (st != DMR_SUCCESS) return st;
    if (P > 0 && grad_points == nullptr) return DMR_ERROR_INVALID_VALUE;
    if (slots > 0 && idx == nullptr) return DMR_ERROR_INVALID_VALUE;
    if (P == 0) return DMR_SUCCESS;
    if (fwd_layout(N, P, H, W, sizeof(PointRec)).bins >= ((int64_t)1 << 28)) return DMR_ERROR_UNSUPPORTED;
    PointBwdArgs a{};
    a.points = points; a.P = P; a.N = N; a.H = H; a.W = W; a.K = K;
    a.idx = idx; a.gz = grad_zbuf; a.gd = grad_dists; a.grad_points = grad_points; a.stream = stream;
    return launch_points_backward(a) == hipSuccess ? DMR_SUCCESS : DMR_ERROR_HIP;
}

dmr_status dmr_workspace_stats(const void* workspace, dmr_stats* out, hipStream_t stream) {
    if (workspace == nullptr || out == nullptr) return DMR_ERROR_INVALID_VALUE;
    WsHeader h;
    if (hipMemcpyAsync(&h, workspace, sizeof(h), hipMemcpyDeviceToHost, stream) != hipSuccess)
        return DMR_ERROR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return DMR_ERROR_HIP;
    out->required_bytes = h.required_bytes;
    out->bin_entries = h.bin_entries;
    out->bin_capacity = h.bin_capacity;
    out->bins = h.bins;
    out->overflow_bins = h.overflow_bins;
    out->live_faces = h.live_faces;
    out->flags = h.flags;
    out->reserved = 0;
    return DMR_SUCCESS;
}

int32_t dmr_kernel_count(void) { return kKernelCount; }

const char* dmr_kernel_name(int32_t id) {
    if (id < 0 || id >= kKernelCount) return "";
    return kKernelNames[id];
}

dmr_status dmr_set_kernel_timing(int32_t enable) {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    g_timing_mask.store(enable != 0 ? (1u << kKernelCount) - 1u : 0u);
    return DMR_SUCCESS;
}

dmr_status dmr_set_kernel_timing_mask(uint32_t mask) {
    if (mask >> kKernelCount) return DMR_ERROR_INVALID_VALUE;
    std::lock_guard<std::mutex> lk(g_timing_mu);
    g_timing_mask.store(mask);
    return DMR_SUCCESS;
}

dmr_status dmr_kernel_timing(int32_t id, double* total_ms, int64_t* launches) {
    if (id < 0 || id >= kKernelCount || !total_ms || !launches) return DMR_ERROR_INVALID_VALUE;
    std::lock_guard<std::mutex> lk(g_timing_mu);
    if (drain(id) != hipSuccess) return DMR_ERROR_HIP;
    *total_ms = g_timing.total_ms[id];
    *launches = g_timing.launches[id];
    return DMR_SUCCESS;
}

dmr_status dmr_reset_kernel_timing(void) {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    for (int id = 0; id < kKernelCount; ++id) {
        if (drain(id) != hipSuccess) return DMR_ERROR_HIP;
        g_timing.total_ms[id] = 0.0;
        g_timing.launches[id] = 0;
    }
    return DMR_SUCCESS;
}

}  // extern "C"
