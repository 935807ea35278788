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
// The LDS sums are 64-bit fixed point (see to_fixed): on gfx950 a float
// atomic add in LDS sustains about a third of a lane per clock per CU, an
// integer one more than seven.
#include <algorithm>

#include "dmr_internal.h"
#include "lds_accum.h"

namespace dmr {

// Zero fill of grad_verts.
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
    r.v0 = r.v1 = r.v2 = -1;
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
constexpr int kListCap = 1536;   // tile slots read (and at most compacted) per chunk

// Records of the four slots of a lane quad, loaded cooperatively: in load k
// lane p of the quad fetches the 16-byte piece p of slot k's record, so each
// load instruction reads whole 64-byte records (one cache request per
// record instead of four), and a 4x4 transpose within the quad (two rounds
// of quad permutations) leaves every lane with its own slot's record. All
// lanes of the wave must take part; `f` is this lane's face, or any valid
// face index when the lane has no slot.
__device__ __forceinline__ FaceRec quad_load_record(const FaceRec* __restrict__ recs, int32_t f) {
    const int p = threadIdx.x & 3;
    // faces of the quad's four slots
    int32_t fq[4];
    fq[0] = quad_perm<0x00>(f);
    fq[1] = quad_perm<0x55>(f);
    fq[2] = quad_perm<0xaa>(f);
    fq[3] = quad_perm<0xff>(f);
    // w[4k + c] = dword c of piece p of slot k's record
    int w[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int4 v = reinterpret_cast<const int4*>(recs + fq[k])[p];
        w[4 * k + 0] = v.x;
        w[4 * k + 1] = v.y;
        w[4 * k + 2] = v.z;
        w[4 * k + 3] = v.w;
    }
    // afterwards w[4k + c] = dword c of piece k of this lane's slot's record
    quad_transpose(w);
    static_assert(sizeof(FaceRec) == 64, "record of four pieces");
    FaceRec r;
    r.x0 = __int_as_float(w[0]);
    r.y0 = __int_as_float(w[1]);
    r.x1 = __int_as_float(w[2]);
    r.y1 = __int_as_float(w[3]);
    r.x2 = __int_as_float(w[4]);
    r.y2 = __int_as_float(w[5]);
    r.z0 = __int_as_float(w[6]);
    r.z1 = __int_as_float(w[7]);
    r.z2 = __int_as_float(w[8]);
    r.invA = __int_as_float(w[9]);
    r.il0 = __int_as_float(w[10]);
    r.il1 = __int_as_float(w[11]);
    r.il2 = __int_as_float(w[12]);
    r.v0 = w[13];
    r.v1 = w[14];
    r.v2 = w[15];
    return r;
}

// One filled slot's inputs, loaded ahead of its evaluation.
struct SlotIn {
    FaceRec r;
    int64_t vi[3];
    bool ok;
    float px, py;
    float gz, gd, gb0, gb1, gb2;
};

// The rest of a slot's inputs once its record is in `in.r` (with the
// forward's records; `in.ok` says whether the slot has a valid face).
__device__ __forceinline__ void load_slot_rest(const FaceRec* __restrict__ recs, const float* __restrict__ verts,
                                               const int64_t* __restrict__ faces, int64_t V, int64_t f, int64_t so,
                                               float px, float py, const float* __restrict__ gzb,
                                               const float* __restrict__ gba, const float* __restrict__ gds,
                                               SlotIn& in) {
    if (!in.ok) return;
    if (recs) {
        // the record carries the vertex indices unless one is out of range
        // or they do not fit in int32
        if (in.r.v0 >= 0) {
            in.vi[0] = in.r.v0;
            in.vi[1] = in.r.v1;
            in.vi[2] = in.r.v2;
        } else {
            in.vi[0] = faces[3 * f + 0];
            in.vi[1] = faces[3 * f + 1];
            in.vi[2] = faces[3 * f + 2];
            in.ok = in.vi[0] >= 0 && in.vi[0] < V && in.vi[1] >= 0 && in.vi[1] < V && in.vi[2] >= 0 && in.vi[2] < V;
        }
    } else {
        load_face(verts, faces, f, V, in.r, in.vi, in.ok);
    }
    in.px = px;
    in.py = py;
    in.gz = gzb ? gzb[so] : 0.0f;
    in.gd = gds ? gds[so] : 0.0f;
    in.gb0 = gba ? gba[3 * so + 0] : 0.0f;
    in.gb1 = gba ? gba[3 * so + 1] : 0.0f;
    in.gb2 = gba ? gba[3 * so + 2] : 0.0f;
}

template <uint32_t SETTINGS>
__device__ __forceinline__ void apply_slot(const SlotIn& in, uint32_t* hkey, unsigned long long (*hval)[3],
                                           float* __restrict__ grad_verts, bool use_hash, int run_bits) {
    if (!in.ok) return;
    PairState st;
    eval_pair(in.r, in.px, in.py, __builtin_inff(), true, SETTINGS, st);
    float g[9];
    slot_partials(in.r, st, in.px, in.py, in.gz, in.gb0, in.gb1, in.gb2, in.gd, SETTINGS, g);
    vertex_add3(hkey, hval, grad_verts, in.vi, g, use_hash, run_bits);
}

// One workgroup per tile: workgroup w takes bin w or, with the forward's
// workspace, the w-th bin of its heaviest-first order (so that the longest
// tiles start first and the dispatcher fills in behind them); a bin without
// faces has no filled slot and ends at once. SETTINGS holds the
// DMR_RASTER_* bits that change the per-slot evaluation (perspective
// correction, unclipped barycentrics), fixed at compile time so that each
// variant carries only its own arithmetic.
//
// A tile's slots are read slot-linearly in chunks of kListCap (coalesced,
// all loads of a chunk in flight together, and the next chunk's issued
// before this one is evaluated); the filled ones are compacted into an LDS
// list (their order is free: the LDS sums are exact), and each thread
// evaluates the list's slots two at a time, the second slot's loads
// issued with the first's. The face records are loaded a lane quad at a
// time (quad_load_record).
template <uint32_t SETTINGS>
__global__ __launch_bounds__(kBwdThreads) void backward_slots(
    const FaceRec* __restrict__ recs, const int32_t* __restrict__ bin_order, const int32_t* __restrict__ bin_count,
    const float* __restrict__ verts, const int64_t* __restrict__ faces, int64_t V, int64_t F,
    int32_t H, int32_t W, int32_t K, int32_t nbx, int32_t nby, const int64_t* __restrict__ pix_to_face,
    const float* __restrict__ gzb, const float* __restrict__ gba, const float* __restrict__ gds,
    float* __restrict__ grad_verts, int32_t use_hash_arg, int32_t soup_run_bits) {
    __shared__ uint32_t hkey[kHashSize];
    __shared__ unsigned long long hval[kHashSize][3];
    __shared__ int32_t lface[kListCap];
    __shared__ uint16_t lslot[kListCap];   // slot index within the tile
    __shared__ int32_t nlist;
    const bool use_hash = use_hash_arg != 0;
    const int64_t per_img = (int64_t)nbx * nby;
    const int t = threadIdx.x;
    const int lane = t & 63;
    // tile slot s -> (row, slot within the row, column): divisions by
    // multiplication (exact while s * divisor < 2^32)
    const int row_slots = kBin * K;
    const uint32_t m_row = 0xffffffffu / (uint32_t)row_slots + 1u;
    const uint32_t m_k = K > 1 ? 0xffffffffu / (uint32_t)K + 1u : 0u;
    const int tile_slots = kBin * row_slots;
    int64_t b = blockIdx.x;
    int run_bits = 0;
    if (bin_order) {
        b = bin_order[b];
        const int32_t c = bin_count[b];
        if (c == 0) return;   // no face, no filled slot
        // runs of ids only where the tile's vertices (at most three per
        // face of its bin list) fit the table and each face has few slots
        // (at most two on average), so that the flush's atomics outnumber
        // the table's adds
        if (3 * (int64_t)c <= kHashSize && (int64_t)K * kBinPixels <= 2 * (int64_t)c) run_bits = soup_run_bits;
    }
    const int64_t n = b / per_img;
    const int rem = (int)(b - n * per_img);
    const int by = rem / nbx, bx = rem - (rem / nbx) * nbx;
    const int rows = min(kBin, H - by * kBin), cols = min(kBin, W - bx * kBin);
    const int64_t tile0 = (((int64_t)n * H + by * kBin) * W + bx * kBin) * K;
    constexpr int kPer = kListCap / kBwdThreads;
    // the chunk's face ids (-1 outside the image or past the tile)
    auto load_chunk = [&](int cbase, int64_t (&fv)[kPer]) {
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int sidx = cbase + q * kBwdThreads + t;
            fv[q] = -1;
            if (sidx < tile_slots) {
                const int r = (int)__umulhi((uint32_t)sidx, m_row);
                const int within = sidx - r * row_slots;
                const int col = K > 1 ? (int)__umulhi((uint32_t)within, m_k) : within;
                if (r < rows && col < cols) fv[q] = pix_to_face[tile0 + (int64_t)r * W * K + within];
            }
        }
    };
    clear_table(hkey, hval, kBwdThreads);
    int64_t fv[kPer];
    load_chunk(0, fv);
    for (int cbase = 0; cbase < tile_slots; cbase += kListCap) {
        if (t == 0) nlist = 0;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const bool filled = fv[q] >= 0;
            const uint64_t bal = __ballot(filled);
            int at = 0;
            if (lane == 0 && bal) at = atomicAdd(&nlist, (int)__popcll(bal));
            at = __shfl(at, 0, 64);
            if (filled) {
                const int e = at + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                lface[e] = (int32_t)fv[q];
                lslot[e] = (uint16_t)(cbase + q * kBwdThreads + t);
            }
        }
        __syncthreads();
        // the next chunk is read while this one is evaluated
        if (cbase + kListCap < tile_slots) load_chunk(cbase + kListCap, fv);
        const int m = nlist;
        // (a trip count uniform over the workgroup: every lane takes part
        // in the cooperative record loads; a lane without a slot loads
        // the list's last face, so that no one address is shared by the
        // idle lanes of every workgroup)
        const int32_t f_last = m > 0 ? lface[m - 1] : 0;
        const int32_t f_idle = (f_last >= 0 && (int64_t)f_last < F) ? f_last : 0;
        for (int e0 = 0; e0 < m; e0 += 2 * kBwdThreads) {
            SlotIn in[2];
            // the second slot only where this pass of the list has one
            // (uniform: a tile of fewer filled slots than threads takes one
            // slot per thread, without the second's cooperative loads)
            const int nu = (e0 + kBwdThreads < m) ? 2 : 1;
            in[1].ok = false;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (u >= nu) break;
                const int x = e0 + t + u * kBwdThreads;
                const int64_t f = x < m ? (int64_t)lface[x] : -1;
                in[u].ok = f >= 0 && f < F;
                if (recs) in[u].r = quad_load_record(recs, in[u].ok ? (int32_t)f : f_idle);
                if (x < m) {
                    const int sidx = lslot[x];
                    const int r = (int)__umulhi((uint32_t)sidx, m_row);
                    const int within = sidx - r * row_slots;
                    const int col = K > 1 ? (int)__umulhi((uint32_t)within, m_k) : within;
                    const int gi = by * kBin + r, gj = bx * kBin + col;
                    load_slot_rest(recs, verts, faces, V, f, tile0 + (int64_t)r * W * K + within,
                                   pixel_centre(gj, W), pixel_centre(gi, H), gzb, gba, gds, in[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) apply_slot<SETTINGS>(in[u], hkey, hval, grad_verts, use_hash, run_bits);
        }
        __syncthreads();
    }
    flush_table(hkey, hval, grad_verts, kBwdThreads);
}

// Table slots for runs of 2^kSoupRunBits consecutive vertex ids when the
// vertices mostly belong to one face each (V >= 2F, as in triangle soups,
// where V = 3F): a tile's ids then come in runs (the three vertices of a
// face are numbered together), and consecutive slots flush as contiguous
// floats. Only tiles whose vertices fit the table and whose faces have few
// slots each use it (runs lengthen the probe sequences of every add when
// the table is well filled); meshes that share vertices keep the plain
// hash.
constexpr int kSoupRunBits = 3;

template <uint32_t SETTINGS>
static void launch_backward_slots(const BwdArgs& a, const FaceRec* recs, const int32_t* order,
                                  const int32_t* count) {
    backward_slots<SETTINGS><<<(unsigned)a.L.bins, kBwdThreads, 0, a.stream>>>(
        recs, order, count, a.verts, a.faces, a.V, a.F, a.H, a.W, a.K, (int32_t)a.L.nbx, (int32_t)a.L.nby,
        a.pix_to_face, a.gz, a.gb, a.gd, a.grad_verts, a.V - 1 <= kTableMaxId ? 1 : 0,
        a.V >= 2 * a.F ? kSoupRunBits : 0);
}

hipError_t launch_backward(const BwdArgs& a) {
    const int64_t n3 = 3 * a.V;
    const int64_t npix = a.N * (int64_t)a.H * a.W;
    const bool work = npix > 0 && a.F > 0;
    // With the forward's workspace, its per-face records (vertex positions,
    // 1/A, inverse edge lengths) replace the per-slot gathers and divisions,
    // and its heaviest-first bin order and counts order the tiles.
    const bool reuse = a.reuse_forward && work;
    if (n3 > 0) {
        timing_begin(kKZeroGrad, a.stream);
        zero_f32<<<(unsigned)std::min<int64_t>(2048, (n3 + 255) / 256), 256, 0, a.stream>>>(a.grad_verts, n3);
        timing_end(kKZeroGrad, a.stream);
    }
    if (!work) return hipGetLastError();
    const FaceRec* recs = reuse ? reinterpret_cast<const FaceRec*>(a.ws + a.L.off_records) : nullptr;
    const int32_t* order = reuse ? reinterpret_cast<const int32_t*>(a.ws + a.L.off_perm) : nullptr;
    const int32_t* count = reuse ? reinterpret_cast<const int32_t*>(a.ws + a.L.off_count) : nullptr;
    constexpr uint32_t kP = DMR_RASTER_PERSPECTIVE_CORRECT, kU = DMR_RASTER_UNCLIPPED_BARY;
    timing_begin(kKBackward, a.stream);
    switch (a.settings & (kP | kU)) {
        case 0: launch_backward_slots<0>(a, recs, order, count); break;
        case kP: launch_backward_slots<kP>(a, recs, order, count); break;
        case kU: launch_backward_slots<kU>(a, recs, order, count); break;
        default: launch_backward_slots<kP | kU>(a, recs, order, count); break;
    }
    timing_end(kKBackward, a.stream);
    return hipGetLastError();
}

}  // namespace dmr
