// Second stage on gfx950: each pixel's kept faces fused into RGBA (soft
// silhouette and depth-weighted colour), and its backward pass to zbuf and
// dists. The formula is the reading stated in include/dmr.h (the pages say
// only that the second stage merges the influence of the faces a pixel
// keeps: gptget.net summary, "Methodology").
//
// Per-slot coverage uses the two
// complementary logistic forms so that 1 - p keeps its precision when p is
// close to 1, and the colour weight exponent is formed from the depth
// difference to the nearest slot, which binary32 holds much more accurately
// than a difference of normalised inverse depths.
#include <algorithm>

#include "dmr_internal.h"

namespace dmr {

// One wavefront per 64 pixels. The pixels' slots are staged in LDS chunk by
// chunk (kChunk slots per pixel at a time) with loads in slot order, so the
// wave reads contiguous memory; each lane then works on its own pixel from
// LDS. Gradients go out the same way: through LDS, stored in slot order.
constexpr int kBlendThreads = 64;
constexpr int kChunk = 16;
// Row stride of a pixel's staged slots: odd, so that the 64 lanes reading
// slot s of their own pixels hit distinct LDS banks.
constexpr int kStride = kChunk + 1;

struct BlendPixel {
    float one_minus_alpha;   // prod (1 - p_k)
    float zmin;              // nearest filled depth
    float den;               // sum w_k + w_bg
    float num[3];            // sum w_k c_k + w_bg background
    bool any;
};

struct BlendStage {
    int32_t face[kBlendThreads * kStride];   // -1: empty slot (or index outside [0, F))
    float z[kBlendThreads * kStride];
    float d[kBlendThreads * kStride];
};

__device__ __forceinline__ float logistic(float x) { return 1.0f / (1.0f + expf(x)); }

// Stage slots [k0, k0 + n) of the block's pixels [pix0, pix0 + np): slot
// k0 + s of pixel pix0 + p goes to entry p * kStride + s.
__device__ __forceinline__ void stage_chunk(const int64_t* __restrict__ p2f, const float* __restrict__ zbuf,
                                            const float* __restrict__ dists, int64_t F, int32_t K, int64_t pix0,
                                            int np, int k0, int n, BlendStage& st) {
    const int total = np * n;
    for (int e = threadIdx.x; e < total; e += kBlendThreads) {
        const int p = e / n, sidx = e - (e / n) * n;
        const int64_t g = (pix0 + p) * K + k0 + sidx;
        const int64_t f = p2f[g];
        const int l = p * kStride + sidx;
        st.face[l] = (f >= 0 && f < F) ? (int32_t)f : -1;
        st.z[l] = zbuf[g];
        st.d[l] = dists[g];
    }
}

// Accumulates one staged chunk of this lane's pixel into bp. The colour
// sums are kept relative to the nearest depth seen so far (rescaled when a
// nearer slot appears).
__device__ __forceinline__ void accumulate_chunk(const BlendStage& st, int lane, int n,
                                                 const float* __restrict__ colors, const dmr_blend_params& prm,
                                                 float inv_range_gamma, BlendPixel& bp) {
    for (int sidx = 0; sidx < n; ++sidx) {
        const int e = lane * kStride + sidx;
        const int32_t f = st.face[e];
        if (f < 0) continue;
        const float z = st.z[e], d = st.d[e];
        bp.any = true;
        bp.one_minus_alpha *= logistic(-d / prm.sigma);
        if (z < bp.zmin) {
            const float r = bp.zmin == __builtin_inff() ? 0.0f : expf((z - bp.zmin) * inv_range_gamma);
            bp.den *= r;
            bp.num[0] *= r;
            bp.num[1] *= r;
            bp.num[2] *= r;
            bp.zmin = z;
        }
        // zeta_k - zeta_max = (zmin - z_k) / (zfar - znear)
        const float w = logistic(d / prm.sigma) * expf((bp.zmin - z) * inv_range_gamma);
        bp.den += w;
        bp.num[0] += w * colors[3 * f + 0];
        bp.num[1] += w * colors[3 * f + 1];
        bp.num[2] += w * colors[3 * f + 2];
    }
}

// Adds the background weight w_bg = exp((eps - zeta_max) / gamma), with
// zeta_max = (zfar - zmin) / (zfar - znear).
__device__ __forceinline__ void finish_pixel(const dmr_blend_params& prm, BlendPixel& bp) {
    const float zeta_max = (prm.zfar - bp.zmin) / (prm.zfar - prm.znear);
    const float wbg = bp.any ? expf((prm.eps - zeta_max) / prm.gamma) : 0.0f;
    bp.den += wbg;
    bp.num[0] += wbg * prm.background[0];
    bp.num[1] += wbg * prm.background[1];
    bp.num[2] += wbg * prm.background[2];
}

__device__ __forceinline__ void blend_block_pixels(const int64_t* __restrict__ p2f, const float* __restrict__ zbuf,
                                                   const float* __restrict__ dists, const float* __restrict__ colors,
                                                   int64_t F, int32_t K, int64_t pix0, int np,
                                                   const dmr_blend_params& prm, float inv_range_gamma,
                                                   BlendStage& st, BlendPixel& bp) {
    const int lane = threadIdx.x;
    bp.one_minus_alpha = 1.0f;
    bp.zmin = __builtin_inff();
    bp.den = 0.0f;
    bp.num[0] = bp.num[1] = bp.num[2] = 0.0f;
    bp.any = false;
    for (int k0 = 0; k0 < K; k0 += kChunk) {
        const int n = min(kChunk, K - k0);
        __syncthreads();
        stage_chunk(p2f, zbuf, dists, F, K, pix0, np, k0, n, st);
        __syncthreads();
        if (lane < np) accumulate_chunk(st, lane, n, colors, prm, inv_range_gamma, bp);
    }
    finish_pixel(prm, bp);
}

__global__ __launch_bounds__(kBlendThreads) void blend_forward(const int64_t* __restrict__ p2f,
                                                               const float* __restrict__ zbuf,
                                                               const float* __restrict__ dists, int64_t P,
                                                               int32_t K, const float* __restrict__ colors, int64_t F,
                                                               dmr_blend_params prm, float inv_range_gamma,
                                                               float4* __restrict__ rgba) {
    __shared__ BlendStage st;
    const int64_t pix0 = (int64_t)blockIdx.x * kBlendThreads;
    const int np = (int)min<int64_t>(kBlendThreads, P - pix0);
    BlendPixel bp;
    blend_block_pixels(p2f, zbuf, dists, colors, F, K, pix0, np, prm, inv_range_gamma, st, bp);
    if ((int)threadIdx.x >= np) return;
    float4 out;
    if (bp.any) {
        out.x = bp.num[0] / bp.den;
        out.y = bp.num[1] / bp.den;
        out.z = bp.num[2] / bp.den;
        out.w = 1.0f - bp.one_minus_alpha;
    } else {
        out.x = prm.background[0];
        out.y = prm.background[1];
        out.z = prm.background[2];
        out.w = 0.0f;
    }
    rgba[pix0 + threadIdx.x] = out;
}

__global__ __launch_bounds__(kBlendThreads) void blend_backward(
    const int64_t* __restrict__ p2f, const float* __restrict__ zbuf, const float* __restrict__ dists, int64_t P,
    int32_t K, const float* __restrict__ colors, int64_t F, dmr_blend_params prm, float inv_range_gamma,
    const float4* __restrict__ grad_rgba, float* __restrict__ grad_zbuf, float* __restrict__ grad_dists) {
    __shared__ BlendStage st;
    const int lane = threadIdx.x;
    const int64_t pix0 = (int64_t)blockIdx.x * kBlendThreads;
    const int np = (int)min<int64_t>(kBlendThreads, P - pix0);
    BlendPixel bp;
    blend_block_pixels(p2f, zbuf, dists, colors, F, K, pix0, np, prm, inv_range_gamma, st, bp);
    float4 g = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (lane < np) g = grad_rgba[pix0 + lane];
    const float inv_den = 1.0f / bp.den;
    const float r0 = bp.num[0] * inv_den, r1 = bp.num[1] * inv_den, r2 = bp.num[2] * inv_den;
    const float inv_sigma = 1.0f / prm.sigma;
    for (int k0 = 0; k0 < K; k0 += kChunk) {
        const int n = min(kChunk, K - k0);
        // with one chunk the staged slots are still in LDS
        if (K > kChunk) {
            __syncthreads();
            stage_chunk(p2f, zbuf, dists, F, K, pix0, np, k0, n, st);
            __syncthreads();
        }
        // per-slot gradients into the staging arrays (z <- grad_zbuf, d <- grad_dists)
        if (lane < np) {
            for (int sidx = 0; sidx < n; ++sidx) {
                const int e = lane * kStride + sidx;
                const int32_t f = st.face[e];
                float gz = 0.0f, gd = 0.0f;
                if (f >= 0) {
                    const float z = st.z[e], d = st.d[e];
                    const float p = logistic(d * inv_sigma);
                    const float q = logistic(-d * inv_sigma);
                    const float w = p * expf((bp.zmin - z) * inv_range_gamma);
                    // d rgb / d w_k = (c_k - rgb) / den, contracted with the rgb gradient
                    const float gw = ((g.x * (colors[3 * f + 0] - r0) + g.y * (colors[3 * f + 1] - r1)) +
                                      g.z * (colors[3 * f + 2] - r2)) * inv_den;
                    gz = gw * (-w * inv_range_gamma);
                    gd = gw * (-w * q * inv_sigma) + g.w * (-bp.one_minus_alpha * p * inv_sigma);
                }
                st.z[e] = gz;
                st.d[e] = gd;
            }
        }
        __syncthreads();
        const int total = np * n;
        for (int e = lane; e < total; e += kBlendThreads) {
            const int p = e / n, sidx = e - (e / n) * n;
            const int64_t gidx = (pix0 + p) * K + k0 + sidx;
            grad_zbuf[gidx] = st.z[p * kStride + sidx];
            grad_dists[gidx] = st.d[p * kStride + sidx];
        }
    }
}

static unsigned blend_grid(int64_t P) { return (unsigned)((P + kBlendThreads - 1) / kBlendThreads); }

hipError_t launch_blend_forward(const BlendArgs& a) {
    const float inv_range_gamma = 1.0f / ((a.prm.zfar - a.prm.znear) * a.prm.gamma);
    timing_begin(kKBlendFwd, a.stream);
    blend_forward<<<blend_grid(a.P), kBlendThreads, 0, a.stream>>>(a.pix_to_face, a.zbuf, a.dists, a.P, a.K,
                                                                   a.colors, a.F, a.prm, inv_range_gamma,
                                                                   reinterpret_cast<float4*>(a.rgba));
    timing_end(kKBlendFwd, a.stream);
    return hipGetLastError();
}

hipError_t launch_blend_backward(const BlendArgs& a) {
    const float inv_range_gamma = 1.0f / ((a.prm.zfar - a.prm.znear) * a.prm.gamma);
    timing_begin(kKBlendBwd, a.stream);
    blend_backward<<<blend_grid(a.P), kBlendThreads, 0, a.stream>>>(
        a.pix_to_face, a.zbuf, a.dists, a.P, a.K, a.colors, a.F, a.prm, inv_range_gamma,
        reinterpret_cast<const float4*>(a.grad_rgba), a.grad_zbuf, a.grad_dists);
    timing_end(kKBlendBwd, a.stream);
    return hipGetLastError();
}

}  // namespace dmr
