// Internal definitions shared by the HIP translation units of libdmr.
//
// Everything here is gfx950 device code or host-side layout arithmetic for
// the K-nearest-face rasterizer declared in include/dmr.h. The per-pair
// evaluation is written so that every binary32 operation happens in the
// order the library's conventions fix (see dmr.h); the translation units are
// compiled with -ffp-contract=off so that no multiply-add is fused, and
// binary32 division and square root are correctly rounded (hipcc's default).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dmr.h"

namespace dmr {

// Side of a coarse bin in pixels; the fine pass gives each bin one
// 256-thread workgroup, one pixel per thread.
constexpr int kBin = 16;
constexpr int kBinPixels = kBin * kBin;
constexpr int kFineThreads = kBinPixels;
// Faces per setup/fill workgroup (kSetupThreadsWide for triangle soups; the
// workspace holds a live count per workgroup of the smaller size).
constexpr int kSetupThreads = 256;
constexpr int kSetupThreadsWide = 512;
// Bin lists of more than one round and up to kSortMax faces are ordered by
// depth lower bound; each such list has kSortMax / kFineThreads per-round
// depth bounds. A list of one round (at most kSortMin entries) is left as
// it is: the fine passes evaluate a round's faces all together, so their
// order changes nothing, and no earlier round could end the list. With
// K = 1 a list of two rounds is left as it is too: sorting it costs more
// than the second round it may let a pixel skip (on a 1M-triangle soup at
// 1024x1024: forward 23 us faster without).
constexpr int kSortMax = 4096;
constexpr int kSortMin = kFineThreads;
constexpr int kRoundsPerBin = kSortMax / kFineThreads;
__host__ __device__ __forceinline__ int32_t sort_min_entries(int32_t K) {
    return K <= 1 ? 2 * kSortMin : kSortMin;
}
// The setup passes count faces into kCountReplicas copies of the bin counts
// (workgroup w into copy w % kCountReplicas), so that a bin's global atomics
// from many workgroups spread over several addresses; the scan adds the
// copies, and the fill places each copy's faces after those of the copies
// before it (the same workgroup-to-copy rule in the setup and fill).
constexpr int kCountReplicas = 8;
// Copies used for a given number of bins: with many bins each one sees few
// workgroups and the scan's cost of adding copies dominates.
__host__ __device__ __forceinline__ int32_t count_replicas(int64_t bins) {
    return bins <= 8192 ? kCountReplicas : 1;
}

// Whether a bin list (offset o, cnt entries) is in the workspace and
// depth-sorted with round bounds (sort_min: sort_min_entries(K)).
__host__ __device__ __forceinline__ bool list_sorted(int64_t o, int32_t cnt, int64_t capacity, int32_t sort_min) {
    return o + cnt <= capacity && cnt > sort_min && cnt <= kSortMax;
}
// The fine pass takes its work from a queue of items, heaviest first. A bin
// with at least kSplitMin faces becomes four items, one per 8x8 quarter,
// each worked by four lanes per pixel (for K <= kSplitMaxK); any other bin
// is one item worked by one lane per pixel.
// (2048 measured best with the pair-parallel fine pass on 16 spheres of
// 1,280 to 81,920 faces at 256x256: 149 us against 172 at 1024 and 160 with
// no split.)
constexpr int kSplitMin = 2048;
constexpr int kSplitMaxK = 16;
constexpr int kItemWhole = 4;   // item code: bin << 3 | quarter (0..3) or kItemWhole

// Per-face record written by the setup pass and read by the fine and
// backward passes (64 bytes, four 16-byte vectors): the vertex positions,
// 1/A, the inverse squared edge lengths, and the vertex indices (-1 when an
// index is out of range, or when the vertex count does not fit in int32;
// the backward pass then reads the face array). Which faces can be
// candidates, and their pixel boxes, are in FaceBin.
struct alignas(16) FaceRec {
    float x0, y0, x1, y1;
    float x2, y2, z0, z1;
    float z2, invA, il0, il1;      // invA = 1/A; il_e = 1/|edge e|^2, edges (0,1) (1,2) (2,0)
    float il2;
    int32_t v0, v1, v2;
};
static_assert(sizeof(FaceRec) == 64, "FaceRec layout");

// Closed xy bounding box of the three vertices (exact: min and max round
// nothing).
struct FaceBox {
    float xmin, xmax, ymin, ymax;
};
__device__ __forceinline__ FaceBox face_box(const FaceRec& r) {
    FaceBox b;
    b.xmin = fminf(r.x0, fminf(r.x1, r.x2));
    b.xmax = fmaxf(r.x0, fmaxf(r.x1, r.x2));
    b.ymin = fminf(r.y0, fminf(r.y1, r.y2));
    b.ymax = fmaxf(r.y0, fmaxf(r.y1, r.y2));
    return b;
}

// What the binning passes need of a face (16 bytes): its pixel box (first
// column | first row << 16, last column | last row << 16; empty, lo > hi,
// for a face that is never a candidate: degenerate, all depths <= 0, no
// pixel centre near it, bad vertex index), its mesh, and the bits of its
// smallest vertex depth.
struct alignas(16) FaceBin {
    int32_t box_lo, box_hi;
    int32_t mesh;
    uint32_t zmin_bits;
};
static_assert(sizeof(FaceBin) == 16, "FaceBin layout");

// Per-point record of the point rasterizer (16 bytes): position, depth and
// global index (-1: never a candidate: z <= 0 or no pixel centre near it).
struct alignas(16) PointRec {
    float x, y, z;
    int32_t idx;
};
static_assert(sizeof(PointRec) == 16, "PointRec layout");

// Workspace header (first 256 bytes of the forward workspace).
struct WsHeader {
    int64_t required_bytes;
    int64_t bin_entries;
    int64_t bin_capacity;
    int64_t bins;
    int64_t overflow_bins;
    int64_t live_faces;
    uint32_t flags;
    uint32_t reserved;
    int32_t fine_items;    // work items of the fine pass (written by the scan)
    int32_t sort_bins;     // bins of the sort order that may hold a sorted list (a prefix of it)
    int64_t pad[24];
};
static_assert(sizeof(WsHeader) == 256, "WsHeader layout");

// Forward workspace layout; every section starts on a 256-byte boundary.
struct FwdLayout {
    int64_t bins, nbx, nby;
    int64_t setup_blocks;
    size_t off_records, off_fbin, off_count, off_offset, off_rep, off_perm, off_items, off_live, off_roundlb,
        off_entries;
    size_t min_bytes;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// F items (faces, or points) of rec_bytes each: FaceRec for meshes,
// PointRec for point clouds.
inline FwdLayout fwd_layout(int64_t N, int64_t F, int32_t H, int32_t W, size_t rec_bytes = sizeof(FaceRec)) {
    FwdLayout L;
    L.nbx = (W + kBin - 1) / kBin;
    L.nby = (H + kBin - 1) / kBin;
    L.bins = N * L.nbx * L.nby;
    size_t o = sizeof(WsHeader);
    L.off_records = o;
    o = align_up(o + (size_t)F * rec_bytes, 256);
    L.off_fbin = o;
    o = align_up(o + (size_t)F * sizeof(FaceBin), 256);
    L.off_count = o;
    o = align_up(o + (size_t)L.bins * sizeof(int32_t), 256);
    L.off_offset = o;
    o = align_up(o + (size_t)(L.bins + 1) * sizeof(int64_t), 256);
    L.off_rep = o;   // kCountReplicas x bins: per-copy counts, then per-copy fill cursors
    o = align_up(o + (size_t)kCountReplicas * L.bins * sizeof(int32_t), 256);
    L.off_perm = o;
    o = align_up(o + (size_t)L.bins * sizeof(int32_t), 256);
    L.off_items = o;
    o = align_up(o + (size_t)L.bins * 4 * sizeof(int32_t), 256);
    L.setup_blocks = (F + kSetupThreads - 1) / kSetupThreads;
    L.off_live = o;
    o = align_up(o + (size_t)L.setup_blocks * sizeof(int32_t), 256);
    L.off_roundlb = o;
    o = align_up(o + (size_t)L.bins * kRoundsPerBin * sizeof(float), 256);
    L.off_entries = o;
    L.min_bytes = o;
    return L;
}

// 16-byte pieces of 64-byte records moved within an aligned lane quad: a
// DPP permutation of the quad's four lanes, and the 4x4 transpose of pieces
// and lanes. Before the transpose w[4k + c] is dword c of piece k of this
// lane's record; after it, dword c of piece p (this lane's position in the
// quad) of quad lane k's record, and the other way round (the transpose is
// its own inverse). Two rounds: where lane bit b and piece bit b differ, a
// lane takes the element of piece k ^ 2^b held by lane p ^ 2^b. All lanes of
// the quad must take part.
template <int CTRL>
__device__ __forceinline__ int quad_perm(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ void quad_transpose(int (&w)[16]) {
    const int p = threadIdx.x & 3;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int bit = 1 << b;
        int t[16];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const bool take = ((p ^ k) & bit) != 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int o = w[4 * (k ^ bit) + c];
                const int x = b == 0 ? quad_perm<0xb1>(o) : quad_perm<0x4e>(o);
                t[4 * k + c] = take ? x : w[4 * k + c];
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) w[i] = t[i];
    }
}

// Pixel centre coordinate for index j of an image side of size W.
__device__ __forceinline__ float pixel_centre(int j, int W) {
    return (float)(2 * j + 1) / (float)W - 1.0f;
}

// Full evaluation of one (pixel, face) pair, mirroring the conventions
// operation by operation. `want_dist` forces the distance even when the
// pixel is inside (needed for the dists output); `settings` holds the
// DMR_RASTER_* bits of include/dmr.h.
struct PairState {
    float b0, b1, b2;      // raw barycentrics
    bool inside;
    float d2;              // squared distance to the nearest edge (if computed)
    int argmin;            // nearest edge (first minimum)
    float t, rx, ry;       // its clamp parameter and residual
    float c0, c1, c2;      // clipped barycentrics
    float invS;            // 1 / (c0 + c1 + c2), or with perspective 1 / (n0 + n1 + n2)
    float bh0, bh1, bh2;   // normalised (and perspective-weighted) clipped barycentrics
    float z;               // depth at the pixel
    bool cand;             // included and z > 0
    float o0, o1, o2;      // the returned barycentrics
    float invDr;           // unclipped with perspective: 1 / (nr0 + nr1 + nr2)
};

// Perspective weights of barycentrics a at vertex depths z: n_k = (a_k
// z_{k+1}) z_{k+2}, i.e. a_k / z_k scaled by z0 z1 z2.
__device__ __forceinline__ void persp_weights(float a0, float a1, float a2, float z0, float z1, float z2, float& n0,
                                              float& n1, float& n2) {
    n0 = (a0 * z1) * z2;
    n1 = (a1 * z2) * z0;
    n2 = (a2 * z0) * z1;
}

__device__ __forceinline__ void edge_distance(float px, float py, float ax, float ay, float bx, float by,
                                              float il, float& d, float& t, float& rx, float& ry) {
    float ux = bx - ax;
    float uy = by - ay;
    float qx = px - ax;
    float qy = py - ay;
    t = (qx * ux + qy * uy) * il;
    t = t < 0.0f ? 0.0f : t;
    t = t > 1.0f ? 1.0f : t;
    rx = qx - t * ux;
    ry = qy - t * uy;
    d = rx * rx + ry * ry;
}

__device__ __forceinline__ void eval_pair(const FaceRec& r, float px, float py, float blur, bool want_dist,
                                          uint32_t settings, PairState& s) {
    float dx0 = r.x0 - px, dy0 = r.y0 - py;
    float dx1 = r.x1 - px, dy1 = r.y1 - py;
    float dx2 = r.x2 - px, dy2 = r.y2 - py;
    float w0 = dx1 * dy2 - dy1 * dx2;
    float w1 = dx2 * dy0 - dy2 * dx0;
    float w2 = dx0 * dy1 - dy0 * dx1;
    s.b0 = w0 * r.invA;
    s.b1 = w1 * r.invA;
    s.b2 = w2 * r.invA;
    const FaceBox bb = face_box(r);
    bool in_box = (px >= bb.xmin) && (px <= bb.xmax) && (py >= bb.ymin) && (py <= bb.ymax);
    s.inside = in_box && (s.b0 > 0.0f) && (s.b1 > 0.0f) && (s.b2 > 0.0f);
    s.d2 = 0.0f;
    s.argmin = 0;
    s.t = s.rx = s.ry = 0.0f;
    bool included = s.inside;
    // With blur_radius == 0 the distance test d2 < 0 can never pass, so the
    // distance is only needed for the dists output.
    if (want_dist || (!s.inside && blur > 0.0f)) {
        float d0, t0, rx0, ry0, d1, t1, rx1, ry1, d2e, t2, rx2, ry2;
        edge_distance(px, py, r.x0, r.y0, r.x1, r.y1, r.il0, d0, t0, rx0, ry0);
        edge_distance(px, py, r.x1, r.y1, r.x2, r.y2, r.il1, d1, t1, rx1, ry1);
        edge_distance(px, py, r.x2, r.y2, r.x0, r.y0, r.il2, d2e, t2, rx2, ry2);
        s.d2 = d0; s.argmin = 0; s.t = t0; s.rx = rx0; s.ry = ry0;
        if (d1 < s.d2) { s.d2 = d1; s.argmin = 1; s.t = t1; s.rx = rx1; s.ry = ry1; }
        if (d2e < s.d2) { s.d2 = d2e; s.argmin = 2; s.t = t2; s.rx = rx2; s.ry = ry2; }
        included = s.inside || (s.d2 < blur);
    }
    s.cand = false;
    if (!included) return;
    float c0 = s.b0 < 0.0f ? 0.0f : s.b0;
    float c1 = s.b1 < 0.0f ? 0.0f : s.b1;
    float c2 = s.b2 < 0.0f ? 0.0f : s.b2;
    c0 = c0 > 1.0f ? 1.0f : c0;
    c1 = c1 > 1.0f ? 1.0f : c1;
    c2 = c2 > 1.0f ? 1.0f : c2;
    s.c0 = c0; s.c1 = c1; s.c2 = c2;
    const bool persp = (settings & DMR_RASTER_PERSPECTIVE_CORRECT) != 0;
    if (persp) {
        float n0, n1, n2;
        persp_weights(c0, c1, c2, r.z0, r.z1, r.z2, n0, n1, n2);
        s.invS = 1.0f / ((n0 + n1) + n2);
        s.bh0 = n0 * s.invS;
        s.bh1 = n1 * s.invS;
        s.bh2 = n2 * s.invS;
    } else {
        float S = (c0 + c1) + c2;
        s.invS = 1.0f / S;
        s.bh0 = c0 * s.invS;
        s.bh1 = c1 * s.invS;
        s.bh2 = c2 * s.invS;
    }
    s.z = (s.bh0 * r.z0 + s.bh1 * r.z1) + s.bh2 * r.z2;
    s.cand = s.z > 0.0f;
    s.o0 = s.bh0; s.o1 = s.bh1; s.o2 = s.bh2;
    s.invDr = 0.0f;
    if (settings & DMR_RASTER_UNCLIPPED_BARY) {
        if (persp) {
            float n0, n1, n2;
            persp_weights(s.b0, s.b1, s.b2, r.z0, r.z1, r.z2, n0, n1, n2);
            s.invDr = 1.0f / ((n0 + n1) + n2);
            s.o0 = n0 * s.invDr;
            s.o1 = n1 * s.invDr;
            s.o2 = n2 * s.invDr;
        } else {
            s.o0 = s.b0; s.o1 = s.b1; s.o2 = s.b2;
        }
    }
}

// ---------------------------------------------------------------------------
// host-side launch helpers implemented in the .hip files
// ---------------------------------------------------------------------------
enum KernelId : int32_t {
    kKZeroFwd = 0,
    kKFaceSetup,
    kKBinScan,
    kKBinFill,
    kKBinSort,
    kKFineRaster,
    kKZeroGrad,
    kKBackward,
    kKBlendFwd,
    kKBlendBwd,
    kKProjectFwd,
    kKProjectBwd,
    kKPointSetup,
    kKPointRaster,
    kKPointBwd,
    kKernelCount
};

struct FwdArgs {
    const float* verts; int64_t V;
    const int64_t* faces; int64_t F;
    const int64_t* off; int64_t N;
    int32_t H, W, K;
    float blur;
    uint32_t settings;     // DMR_RASTER_* bits
    const float* points;   // point clouds instead of meshes (F points, off = cloud offsets)
    float radius;          // point radius (NDC)
    int64_t* pix_to_face; float* zbuf; float* bary; float* dists;
    char* ws; size_t ws_bytes;
    FwdLayout L;
    int64_t capacity;
    hipStream_t stream;
};

struct BwdArgs {
    const float* verts; int64_t V;
    const int64_t* faces; int64_t F;
    const int64_t* off; int64_t N;
    int32_t H, W, K;
    float blur;
    uint32_t settings;     // DMR_RASTER_* bits
    const int64_t* pix_to_face;
    const float* gz; const float* gb; const float* gd;
    float* grad_verts;
    char* ws; size_t ws_bytes;
    FwdLayout L;
    int64_t capacity;
    bool reuse_forward;
    hipStream_t stream;
};

struct BlendArgs {
    const int64_t* pix_to_face; const float* zbuf; const float* dists;
    int64_t P; int32_t K;
    const float* colors; int64_t F;
    dmr_blend_params prm;
    float* rgba;
    const float* grad_rgba; float* grad_zbuf; float* grad_dists;
    hipStream_t stream;
};

struct ProjectArgs {
    const float* verts; int64_t V;
    const int64_t* off; int64_t N;
    const float* cameras;
    float* out;                                   // forward
    const float* grad_out; float* grad_verts; float* grad_cameras;   // backward
    hipStream_t stream;
};

// Launch wrappers with optional event timing; return hipSuccess or the error.
hipError_t launch_binning(const FwdArgs& a, bool sort);
hipError_t launch_forward(const FwdArgs& a);
hipError_t launch_backward(const BwdArgs& a);
hipError_t launch_blend_forward(const BlendArgs& a);
hipError_t launch_blend_backward(const BlendArgs& a);
struct PointBwdArgs {
    const float* points; int64_t P;
    int64_t N; int32_t H, W, K;
    const int64_t* idx; const float* gz; const float* gd;
    float* grad_points;
    hipStream_t stream;
};

hipError_t launch_project_forward(const ProjectArgs& a);
// Point clouds: the setup pass (binning uses the mesh kernels after it),
// the fine pass and the backward pass.
hipError_t launch_point_setup(const FwdArgs& a, PointRec* recs, FaceBin* fbin, int32_t* count, int32_t* block_live,
                              WsHeader* hdr);
hipError_t launch_points_forward(const FwdArgs& a);
hipError_t launch_points_backward(const PointBwdArgs& a);
hipError_t launch_project_backward(const ProjectArgs& a);

// Timing hooks (api.hip).
void timing_begin(KernelId id, hipStream_t s);
void timing_end(KernelId id, hipStream_t s);

}  // namespace dmr
