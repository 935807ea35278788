// Second stage on gfx950: each pixel's kept faces fused into RGBA (soft
// silhouette and depth-weighted colour), and its backward pass to zbuf and
// dists. The formula is the reading stated in include/dmr.h (the pages say
// only that the second stage merges the influence of the faces a pixel
// keeps: gptget.net summary, "Methodology").
//
// Per-slot coverage takes p and 1 - p from one exponential of -|d|/sigma,
// so that both keep their relative precision when either is close to 0. The
// colour weights are summed in the log domain with a running maximum (the
// largest term is exp(0) = 1): log w_k = log p_k + (zmin - z_k) c with
// log p_k = -softplus(d_k / sigma), so that a pixel whose weights all
// underflow binary32 (a sharp sigma far from every face) still gets their
// ratio, not 0/0. Depths enter as differences to the pixel's first filled
// slot, which binary32 holds much more accurately than a difference of
// normalised inverse depths; the common shift cancels in the ratio.
#include <algorithm>

#include "dmr_internal.h"

namespace dmr {

// One wavefront per 64 pixels. The pixels' slots are staged in LDS chunk by
// chunk (up to kChunk slots per pixel at a time): every lane first issues
// all of its loads for the chunk, in slot order across the wave, and only
// then writes them to LDS, so that a wave has its whole chunk in flight at
// once. Each lane then works on its own pixel from LDS; the face colours are
// gathered there. Gradients go out the same way, through LDS and in slot
// order, with streaming (non-temporal) stores since nothing reads them back.
constexpr int kBlendThreads = 64;
constexpr int kChunk = 16;

// LDS view of one staged chunk: three arrays of kBlendThreads rows; slot s
// of the block's pixel p sits at p * stride + s. The stride is odd, so that
// 64 lanes reading slot s of their own pixels hit distinct banks.
struct BlendStage {
    int32_t* face;   // -1: empty slot (or index outside [0, F))
    float* z;
    float* d;
    int stride;
};

__device__ __forceinline__ BlendStage stage_view(float* smem, int stride) {
    BlendStage st;
    st.face = reinterpret_cast<int32_t*>(smem);
    st.z = smem + kBlendThreads * stride;
    st.d = smem + 2 * kBlendThreads * stride;
    st.stride = stride;
    return st;
}

static int stage_stride(int32_t K) { return std::min<int32_t>(K, kChunk) | 1; }
static size_t stage_bytes(int32_t K) { return (size_t)3 * kBlendThreads * stage_stride(K) * sizeof(float); }

struct BlendPixel {
    float one_minus_alpha;   // prod (1 - p_k)
    float zmin;              // nearest filled depth
    float zref;              // depth of the first filled slot (exponent origin)
    float m;                 // running maximum of the log weights
    float den;               // sum exp(e_k - m) (+ background)
    float num[3];            // sum exp(e_k - m) c_k (+ background)
    bool any;
};

// p = 1 / (1 + exp(d / sigma)) and q = 1 - p: with t = exp(-|d| / sigma),
// the one that is at least 1/2 is a = 1 / (1 + t) and the other t a; so
// log p = log a, or -|d| / sigma + log a. log a lies in [-log 2, 0], where
// the hardware logarithm's absolute error is a few units of 2^-24.
__device__ __forceinline__ void coverage(float d, float inv_sigma, float& p, float& q, float& logp) {
    const float x = d * inv_sigma;
    const float t = expf(-fabsf(x));
    const float a = 1.0f / (1.0f + t);
    const float b = t * a;
    const float la = __logf(a);
    p = d <= 0.0f ? a : b;
    q = d <= 0.0f ? b : a;
    logp = d <= 0.0f ? la : la - x;
}

// Stage slots [k0, k0 + n) of the block's pixels [pix0, pix0 + np). Element
// e = p * n + s (slot k0 + s of pixel pix0 + p) is handled by lane
// e % kBlendThreads, so a lane holds at most n <= kChunk elements. div_n is
// ceil(2^16 / n), so that (e * div_n) >> 16 == e / n for every e < 64 * n.
__device__ __forceinline__ void stage_chunk(const int64_t* __restrict__ p2f, const float* __restrict__ zbuf,
                                            const float* __restrict__ dists, int64_t F, int32_t K, int64_t pix0,
                                            int np, int k0, int n, uint32_t div_n, const BlendStage& st) {
    const int total = np * n;
    int32_t fr[kChunk];
    float zr[kChunk], dr[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        const int e = threadIdx.x + i * kBlendThreads;
        fr[i] = -1;
        if (e < total) {
            const int p = (int)(((uint32_t)e * div_n) >> 16), sidx = e - p * n;
            const int64_t gi = (pix0 + p) * K + k0 + sidx;
            const int64_t f = p2f[gi];
            fr[i] = (f >= 0 && f < F) ? (int32_t)f : -1;
            zr[i] = zbuf[gi];
            dr[i] = dists[gi];
        }
    }
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        const int e = threadIdx.x + i * kBlendThreads;
        if (e < total) {
            const int p = (int)(((uint32_t)e * div_n) >> 16), sidx = e - p * n;
            const int l = p * st.stride + sidx;
            st.face[l] = fr[i];
            st.z[l] = zr[i];
            st.d[l] = dr[i];
        }
    }
}

// Accumulates one staged chunk of this lane's pixel into bp: the colour sums
// are kept relative to the largest log weight seen so far (rescaled when a
// larger one appears).
__device__ __forceinline__ void accumulate_chunk(const BlendStage& st, const float* __restrict__ colors, int lane,
                                                 int n, float inv_sigma, float inv_range_gamma, BlendPixel& bp) {
    for (int sidx = 0; sidx < n; ++sidx) {
        const int e = lane * st.stride + sidx;
        const int32_t f = st.face[e];
        if (f < 0) continue;
        const float z = st.z[e], d = st.d[e];
        const float cr = colors[3 * (int64_t)f + 0], cg = colors[3 * (int64_t)f + 1], cb = colors[3 * (int64_t)f + 2];
        float p, q, logp;
        coverage(d, inv_sigma, p, q, logp);
        if (!bp.any) bp.zref = z;
        bp.any = true;
        bp.one_minus_alpha *= q;
        bp.zmin = fminf(bp.zmin, z);
        // (zeta_k - zeta_max) / gamma = (zmin - z_k) c, shifted by (zmin - zref) c
        const float lw = logp + (bp.zref - z) * inv_range_gamma;
        if (lw > bp.m) {
            const float r = bp.m == -__builtin_inff() ? 0.0f : expf(bp.m - lw);
            bp.den *= r;
            bp.num[0] *= r;
            bp.num[1] *= r;
            bp.num[2] *= r;
            bp.m = lw;
        }
        const float w = expf(lw - bp.m);
        bp.den += w;
        bp.num[0] += w * cr;
        bp.num[1] += w * cg;
        bp.num[2] += w * cb;
    }
}

// Adds the background weight w_bg = exp((eps - zeta_max) / gamma), with
// zeta_max = (zfar - zmin) / (zfar - znear), in the slots' shifted log scale.
__device__ __forceinline__ void finish_pixel(const dmr_blend_params& prm, float inv_range_gamma, BlendPixel& bp) {
    if (!bp.any) return;
    const float zeta_max = (prm.zfar - bp.zmin) / (prm.zfar - prm.znear);
    const float e = (prm.eps - zeta_max) / prm.gamma - (bp.zmin - bp.zref) * inv_range_gamma;
    if (e > bp.m) {
        const float r = expf(bp.m - e);
        bp.den *= r;
        bp.num[0] *= r;
        bp.num[1] *= r;
        bp.num[2] *= r;
        bp.m = e;
    }
    const float wbg = expf(e - bp.m);
    bp.den += wbg;
    bp.num[0] += wbg * prm.background[0];
    bp.num[1] += wbg * prm.background[1];
    bp.num[2] += wbg * prm.background[2];
}

__device__ __forceinline__ void blend_block_pixels(const int64_t* __restrict__ p2f, const float* __restrict__ zbuf,
                                                   const float* __restrict__ dists, const float* __restrict__ colors,
                                                   int64_t F, int32_t K, int64_t pix0, int np,
                                                   const dmr_blend_params& prm, float inv_sigma, float inv_range_gamma,
                                                   const BlendStage& st, BlendPixel& bp) {
    const int lane = threadIdx.x;
    bp.one_minus_alpha = 1.0f;
    bp.zmin = __builtin_inff();
    bp.zref = 0.0f;
    bp.m = -__builtin_inff();
    bp.den = 0.0f;
    bp.num[0] = bp.num[1] = bp.num[2] = 0.0f;
    bp.any = false;
    for (int k0 = 0; k0 < K; k0 += kChunk) {
        const int n = min(kChunk, K - k0);
        const uint32_t div_n = (65536u + (uint32_t)n - 1u) / (uint32_t)n;
        __syncthreads();
        stage_chunk(p2f, zbuf, dists, F, K, pix0, np, k0, n, div_n, st);
        __syncthreads();
        if (lane < np) accumulate_chunk(st, colors, lane, n, inv_sigma, inv_range_gamma, bp);
    }
    finish_pixel(prm, inv_range_gamma, bp);
}

__global__ __launch_bounds__(kBlendThreads) void blend_forward(const int64_t* __restrict__ p2f,
                                                               const float* __restrict__ zbuf,
                                                               const float* __restrict__ dists, int64_t P,
                                                               int32_t K, const float* __restrict__ colors, int64_t F,
                                                               dmr_blend_params prm, float inv_range_gamma,
                                                               int stride, float4* __restrict__ rgba) {
    extern __shared__ float smem[];
    const BlendStage st = stage_view(smem, stride);
    const int64_t pix0 = (int64_t)blockIdx.x * kBlendThreads;
    const int np = (int)min<int64_t>(kBlendThreads, P - pix0);
    const float inv_sigma = 1.0f / prm.sigma;
    BlendPixel bp;
    blend_block_pixels(p2f, zbuf, dists, colors, F, K, pix0, np, prm, inv_sigma, inv_range_gamma, st, bp);
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
    float* o = reinterpret_cast<float*>(rgba + pix0 + threadIdx.x);
    __builtin_nontemporal_store(out.x, o + 0);
    __builtin_nontemporal_store(out.y, o + 1);
    __builtin_nontemporal_store(out.z, o + 2);
    __builtin_nontemporal_store(out.w, o + 3);
}

__global__ __launch_bounds__(kBlendThreads) void blend_backward(
    const int64_t* __restrict__ p2f, const float* __restrict__ zbuf, const float* __restrict__ dists, int64_t P,
    int32_t K, const float* __restrict__ colors, int64_t F, dmr_blend_params prm, float inv_range_gamma, int stride,
    const float4* __restrict__ grad_rgba, float* __restrict__ grad_zbuf, float* __restrict__ grad_dists) {
    extern __shared__ float smem[];
    const BlendStage st = stage_view(smem, stride);
    const int lane = threadIdx.x;
    const int64_t pix0 = (int64_t)blockIdx.x * kBlendThreads;
    const int np = (int)min<int64_t>(kBlendThreads, P - pix0);
    float4 g = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (lane < np) g = grad_rgba[pix0 + lane];
    const float inv_sigma = 1.0f / prm.sigma;
    BlendPixel bp;
    blend_block_pixels(p2f, zbuf, dists, colors, F, K, pix0, np, prm, inv_sigma, inv_range_gamma, st, bp);
    const float inv_den = 1.0f / bp.den;
    const float r0 = bp.num[0] * inv_den, r1 = bp.num[1] * inv_den, r2 = bp.num[2] * inv_den;
    for (int k0 = 0; k0 < K; k0 += kChunk) {
        const int n = min(kChunk, K - k0);
        const uint32_t div_n = (65536u + (uint32_t)n - 1u) / (uint32_t)n;
        // with one chunk the staged slots are still in LDS
        if (K > kChunk) {
            __syncthreads();
            stage_chunk(p2f, zbuf, dists, F, K, pix0, np, k0, n, div_n, st);
            __syncthreads();
        }
        // per-slot gradients into the staging arrays (z <- grad_zbuf, d <- grad_dists)
        if (lane < np) {
            for (int sidx = 0; sidx < n; ++sidx) {
                const int e = lane * st.stride + sidx;
                const int32_t f = st.face[e];
                float gz = 0.0f, gd = 0.0f;
                if (f >= 0) {
                    const float z = st.z[e], d = st.d[e];
                    const float cr = colors[3 * (int64_t)f + 0], cg = colors[3 * (int64_t)f + 1],
                                cb = colors[3 * (int64_t)f + 2];
                    float p, q, logp;
                    coverage(d, inv_sigma, p, q, logp);
                    // normalised weight w_k / den
                    const float wn = expf((logp + (bp.zref - z) * inv_range_gamma) - bp.m) * inv_den;
                    // d rgb / d log w_k = (c_k - rgb) w_k / den, contracted with the rgb
                    // gradient; d log w_k / dz_k = -c, d log w_k / dd_k = -q_k / sigma
                    const float gl = ((g.x * (cr - r0) + g.y * (cg - r1)) + g.z * (cb - r2)) * wn;
                    gz = gl * -inv_range_gamma;
                    gd = gl * (-q * inv_sigma) + g.w * (-bp.one_minus_alpha * p * inv_sigma);
                }
                st.z[e] = gz;
                st.d[e] = gd;
            }
        }
        __syncthreads();
        const int total = np * n;
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            const int e = lane + i * kBlendThreads;
            if (e < total) {
                const int p = (int)(((uint32_t)e * div_n) >> 16), sidx = e - p * n;
                const int64_t gi = (pix0 + p) * K + k0 + sidx;
                __builtin_nontemporal_store(st.z[p * st.stride + sidx], grad_zbuf + gi);
                __builtin_nontemporal_store(st.d[p * st.stride + sidx], grad_dists + gi);
            }
        }
    }
}

static unsigned blend_grid(int64_t P) { return (unsigned)((P + kBlendThreads - 1) / kBlendThreads); }

hipError_t launch_blend_forward(const BlendArgs& a) {
    const float inv_range_gamma = 1.0f / ((a.prm.zfar - a.prm.znear) * a.prm.gamma);
    timing_begin(kKBlendFwd, a.stream);
    blend_forward<<<blend_grid(a.P), kBlendThreads, stage_bytes(a.K), a.stream>>>(
        a.pix_to_face, a.zbuf, a.dists, a.P, a.K, a.colors, a.F, a.prm, inv_range_gamma, stage_stride(a.K),
        reinterpret_cast<float4*>(a.rgba));
    timing_end(kKBlendFwd, a.stream);
    return hipGetLastError();
}

hipError_t launch_blend_backward(const BlendArgs& a) {
    const float inv_range_gamma = 1.0f / ((a.prm.zfar - a.prm.znear) * a.prm.gamma);
    timing_begin(kKBlendBwd, a.stream);
    blend_backward<<<blend_grid(a.P), kBlendThreads, stage_bytes(a.K), a.stream>>>(
        a.pix_to_face, a.zbuf, a.dists, a.P, a.K, a.colors, a.F, a.prm, inv_range_gamma, stage_stride(a.K),
        reinterpret_cast<const float4*>(a.grad_rgba), a.grad_zbuf, a.grad_dists);
    timing_end(kKBlendBwd, a.stream);
    return hipGetLastError();
}

}  // namespace dmr
