/*
 * Body of the CPU oracle. raster_oracle.c includes this file twice: once with
 * R = float (the canonical binary32 evaluation every decision is taken in) and
 * once with R = double (used for finite-difference checks of the backward
 * pass and to report fp32-versus-binary64 drift).
 *
 * TEST INFRASTRUCTURE ONLY: this is the slow, plain definition the GPU path is
 * checked against. Nothing on the product path may link or call it.
 *
 * Every operation below is one IEEE-754 operation of type R, evaluated in the
 * parenthesisation written, with no contraction into fused multiply-adds
 * (built with -ffp-contract=off, no fast-math) and correctly rounded division.
 *
 * What it computes follows "Accelerating 3D Deep Learning with PyTorch3D":
 *   - each pixel keeps the K nearest faces of its own mesh (nubint.ai review,
 *     "Proposed method" and "Main findings": per-pixel K nearest faces);
 *   - batches hold meshes of different sizes, packed with per-mesh face
 *     ranges (gptget.net summary, "Methodology"; rocketrecap summary,
 *     "1:00 Heterogeneous Batching");
 *   - the pass is differentiable from pixels back to vertex positions
 *     (rocketrecap summary, "3:52 Differentiable Renderer"), with the
 *     per-pixel intermediates exposed so that shading can be composed on top
 *     (nubint.ai review, "Proposed method").
 * The pages leave the arithmetic conventions open; the ones used here are:
 *   pixel centre     px = fl(fl((2j+1)/W) - 1), py = fl(fl((2i+1)/H) - 1), no axis flip;
 *   barycentrics     edge functions of (vertex - pixel) differences, times 1/A;
 *   inside           strictly inside: all three barycentrics > 0 (and the centre
 *                    in the face's closed bounding box, implied in exact arithmetic);
 *   distance         squared distance to the nearest of the three closed edges;
 *   inclusion        inside, or squared distance strictly below blur_radius;
 *   depth            z from barycentrics clipped to [0,1] and renormalised,
 *                    faces with z <= 0 at the pixel are skipped;
 *   degenerate       faces with A == 0 (exactly, in type R) are skipped;
 *   order            K smallest (z, global face index), ascending;
 *   padding          -1 in pix_to_face, zbuf, every bary component and dists;
 *   signed distance  dists = -d2 when inside, +d2 otherwise.
 *
 * Settings (bit mask `settings`; rocketrecap summary, "32:56 Technical Bug
 * Fix", names a perspective_correct setting of the rasterizer, with no
 * definition; the readings here are the library's):
 *   0x2 perspective-correct: a face is a candidate only if all three vertex
 *       depths are > 0; the clipped barycentrics c are weighted by the inverse
 *       vertex depths, n_k = c_k z_{k+1} z_{k+2}, bh = n / (n0 + n1 + n2)
 *       (this normalisation replaces the division by c0 + c1 + c2), and
 *       z = sum bh_k z_k, i.e. 1 / z is interpolated linearly in screen space;
 *   0x4 back-face culling: a face whose doubled area A is > 0 is skipped (A is
 *       the z component of (v1 - v0) x (v2 - v0), so its normal points away
 *       from the viewer, toward larger depth);
 *   0x8 unclipped barycentrics: the returned bary are the barycentrics before
 *       clipping (with 0x2, perspective-corrected the same way from the
 *       unclipped values); depth, inclusion and order are unchanged.
 * Settings 0 gives the conventions listed above.
 */
#ifndef ORACLE_SETTINGS_DEFINED
#define ORACLE_SETTINGS_DEFINED
#define ORACLE_PERSPECTIVE 0x2u
#define ORACLE_CULL_BACK 0x4u
#define ORACLE_UNCLIPPED 0x8u
#endif

#ifndef R
#error "define R (float or double) and SFX(name) before including"
#endif

typedef struct {
    int64_t face;
    int64_t vi[3];
    R x[3], y[3], z[3];
    R A, invA;
    R dx[3], dy[3];
    R w[3], b[3];
    int inside;
    R d[3], t[3], rx[3], ry[3];
    int argmin;
    R d2;
    R c[3], S, invS, bh[3];
    R n[3], D, invD;     /* perspective weights of c */
    R out[3];            /* returned barycentrics */
    R nr[3], Dr, invDr;  /* perspective weights of the unclipped b */
    R zp;   /* interpolated depth at the pixel */
    R dist; /* signed squared distance */
} SFX(slot_t);

typedef struct {
    R z;
    int64_t face;
} SFX(cand_t);

/* Pixel centre in normalised device coordinates: column j -> x, row i -> y. */
static R SFX(pixel_centre)(int64_t j, int64_t W) {
    return (R)(2 * j + 1) / (R)W - (R)1;
}

/*
 * Evaluates one (pixel, face) pair. Returns 1 when the face is a candidate
 * for the pixel (included and z > 0); the full intermediate state is left in
 * *s for the backward pass. Faces with an out-of-range vertex index are never
 * candidates.
 */
static int SFX(eval_face)(const R* verts, int64_t V, const int64_t* faces, int64_t f,
                          R px, R py, R blur, uint32_t settings, SFX(slot_t)* s) {
    s->face = f;
    for (int k = 0; k < 3; ++k) {
        int64_t vi = faces[3 * f + k];
        if (vi < 0 || vi >= V) return 0;
        s->vi[k] = vi;
        s->x[k] = verts[3 * vi + 0];
        s->y[k] = verts[3 * vi + 1];
        s->z[k] = verts[3 * vi + 2];
    }
    /* Twice the signed area; zero means a degenerate face, which is skipped. */
    s->A = (s->x[1] - s->x[0]) * (s->y[2] - s->y[0]) - (s->y[1] - s->y[0]) * (s->x[2] - s->x[0]);
    if (s->A == (R)0) return 0;
    if ((settings & ORACLE_CULL_BACK) && s->A > (R)0) return 0;
    if ((settings & ORACLE_PERSPECTIVE) && !(s->z[0] > (R)0 && s->z[1] > (R)0 && s->z[2] > (R)0)) return 0;
    s->invA = (R)1 / s->A;

    for (int k = 0; k < 3; ++k) {
        s->dx[k] = s->x[k] - px;
        s->dy[k] = s->y[k] - py;
    }
    /* Edge function k is the doubled signed area of (pixel, v[k+1], v[k+2]). */
    s->w[0] = s->dx[1] * s->dy[2] - s->dy[1] * s->dx[2];
    s->w[1] = s->dx[2] * s->dy[0] - s->dy[2] * s->dx[0];
    s->w[2] = s->dx[0] * s->dy[1] - s->dy[0] * s->dx[1];
    for (int k = 0; k < 3; ++k) s->b[k] = s->w[k] * s->invA;
    /* A point strictly inside the triangle lies in its closed bounding box;
     * requiring it too changes nothing in exact arithmetic and keeps rounding
     * noise of near-degenerate faces from reaching beyond that box. */
    {
        R xmin = s->x[0], xmax = s->x[0], ymin = s->y[0], ymax = s->y[0];
        for (int k = 1; k < 3; ++k) {
            if (s->x[k] < xmin) xmin = s->x[k];
            if (s->x[k] > xmax) xmax = s->x[k];
            if (s->y[k] < ymin) ymin = s->y[k];
            if (s->y[k] > ymax) ymax = s->y[k];
        }
        int in_box = (px >= xmin) && (px <= xmax) && (py >= ymin) && (py <= ymax);
        s->inside = in_box && (s->b[0] > (R)0) && (s->b[1] > (R)0) && (s->b[2] > (R)0);
    }

    /* Squared distance to each closed edge (v[e], v[e+1]); keep the first minimum. */
    for (int e = 0; e < 3; ++e) {
        int a = e, bb = (e + 1) % 3;
        R ux = s->x[bb] - s->x[a];
        R uy = s->y[bb] - s->y[a];
        R il = (R)1 / (ux * ux + uy * uy);
        R qx = px - s->x[a];
        R qy = py - s->y[a];
        R t = (qx * ux + qy * uy) * il;
        if (t < (R)0) t = (R)0;
        if (t > (R)1) t = (R)1;
        s->t[e] = t;
        s->rx[e] = qx - t * ux;
        s->ry[e] = qy - t * uy;
        s->d[e] = s->rx[e] * s->rx[e] + s->ry[e] * s->ry[e];
    }
    s->argmin = 0;
    s->d2 = s->d[0];
    for (int e = 1; e < 3; ++e) {
        if (s->d[e] < s->d2) {
            s->d2 = s->d[e];
            s->argmin = e;
        }
    }
    if (!(s->inside || s->d2 < blur)) return 0;

    /* Clip to [0,1], renormalise, interpolate depth. */
    for (int k = 0; k < 3; ++k) {
        R c = s->b[k];
        if (c < (R)0) c = (R)0;
        if (c > (R)1) c = (R)1;
        s->c[k] = c;
    }
    if (settings & ORACLE_PERSPECTIVE) {
        /* weight of vertex k: c_k / z_k, scaled by z0 z1 z2 */
        for (int k = 0; k < 3; ++k) s->n[k] = (s->c[k] * s->z[(k + 1) % 3]) * s->z[(k + 2) % 3];
        s->D = (s->n[0] + s->n[1]) + s->n[2];
        s->invD = (R)1 / s->D;
        for (int k = 0; k < 3; ++k) s->bh[k] = s->n[k] * s->invD;
    } else {
        s->S = (s->c[0] + s->c[1]) + s->c[2];
        s->invS = (R)1 / s->S;
        for (int k = 0; k < 3; ++k) s->bh[k] = s->c[k] * s->invS;
    }
    s->zp = (s->bh[0] * s->z[0] + s->bh[1] * s->z[1]) + s->bh[2] * s->z[2];
    if (!(s->zp > (R)0)) return 0;
    s->dist = s->inside ? -s->d2 : s->d2;
    for (int k = 0; k < 3; ++k) s->out[k] = s->bh[k];
    if ((settings & ORACLE_UNCLIPPED) && (settings & ORACLE_PERSPECTIVE)) {
        for (int k = 0; k < 3; ++k) s->nr[k] = (s->b[k] * s->z[(k + 1) % 3]) * s->z[(k + 2) % 3];
        s->Dr = (s->nr[0] + s->nr[1]) + s->nr[2];
        s->invDr = (R)1 / s->Dr;
        for (int k = 0; k < 3; ++k) s->out[k] = s->nr[k] * s->invDr;
    } else if (settings & ORACLE_UNCLIPPED) {
        for (int k = 0; k < 3; ++k) s->out[k] = s->b[k];
    }
    return 1;
}

static int SFX(cand_cmp)(const void* pa, const void* pb) {
    const SFX(cand_t)* a = (const SFX(cand_t)*)pa;
    const SFX(cand_t)* b = (const SFX(cand_t)*)pb;
    if (a->z < b->z) return -1;
    if (a->z > b->z) return 1;
    if (a->face < b->face) return -1;
    if (a->face > b->face) return 1;
    return 0;
}

/* Discrete state of a slot, packed for the finite-difference guard:
 * bit 0 inside; bits 1-6 clip state of b0..b2 (2 bits each: 0 below, 1 open,
 * 2 above); bits 7-9 nearest boundary feature of the triangle: vertex k (k)
 * when the nearest edge's t is clamped to an endpoint, else edge e (3 + e). */
static int32_t SFX(slot_code)(const SFX(slot_t)* s) {
    int32_t code = s->inside ? 1 : 0;
    for (int k = 0; k < 3; ++k) {
        int cs = s->b[k] <= (R)0 ? 0 : (s->b[k] >= (R)1 ? 2 : 1);
        code |= cs << (1 + 2 * k);
    }
    int e = s->argmin;
    R t = s->t[e];
    int feature = t <= (R)0 ? e : (t >= (R)1 ? (e + 1) % 3 : 3 + e);
    code |= feature << 7;
    return code;
}

/*
 * Vertex positions are of type R: the binary32 entry points take the
 * library's float32 inputs as they are; the binary64 ones take doubles (the
 * float32 inputs widened exactly, or perturbed copies for finite differences).
 *
 * Forward pass over a list of pixels (flat ids n*H*W + i*W + j; all pixels
 * when pixels == NULL). Outputs are [npix, K] (bary [npix, K, 3]); state (may
 * be NULL) receives slot_code() per filled slot and -1 on padding.
 * For every pixel: visit every face of that pixel's mesh, collect the
 * candidates, sort them by (z, face) and keep the first K.
 */
int SFX(oracle_raster)(const R* verts, int64_t V, const int64_t* faces, int64_t F,
                       const int64_t* offsets, int64_t N, int64_t H, int64_t W, int64_t K, R blur,
                       uint32_t settings, const int64_t* pixels, int64_t npix,
                       int64_t* pix_to_face, R* zbuf, R* bary, R* dists, int32_t* state) {
    if (V < 0 || F < 0 || N < 0 || H < 1 || W < 1 || K < 1) return 1;
    int64_t total = N * H * W;
    if (pixels == NULL) npix = total;
    int err = 0;

#pragma omp parallel
    {
        int64_t cap = 256;
        SFX(cand_t)* cand = (SFX(cand_t)*)malloc(sizeof(SFX(cand_t)) * (size_t)cap);
        SFX(slot_t) s;
#pragma omp for schedule(dynamic, 16)
        for (int64_t q = 0; q < npix; ++q) {
            int64_t pid = pixels ? pixels[q] : q;
            if (pid < 0 || pid >= total) {
#pragma omp atomic write
                err = 2;
                continue;
            }
            int64_t n = pid / (H * W);
            int64_t i = (pid / W) % H;
            int64_t j = pid % W;
            R px = SFX(pixel_centre)(j, W);
            R py = SFX(pixel_centre)(i, H);
            int64_t f0 = offsets[n], f1 = offsets[n + 1];
            if (f0 < 0) f0 = 0;
            if (f1 > F) f1 = F;
            int64_t nc = 0;
            for (int64_t f = f0; f < f1; ++f) {
                if (!SFX(eval_face)(verts, V, faces, f, px, py, blur, settings, &s)) continue;
                if (nc == cap) {
                    cap *= 2;
                    cand = (SFX(cand_t)*)realloc(cand, sizeof(SFX(cand_t)) * (size_t)cap);
                }
                cand[nc].z = s.zp;
                cand[nc].face = f;
                ++nc;
            }
            qsort(cand, (size_t)nc, sizeof(SFX(cand_t)), SFX(cand_cmp));
            for (int64_t k = 0; k < K; ++k) {
                int64_t o = q * K + k;
                if (k < nc) {
                    SFX(eval_face)(verts, V, faces, cand[k].face, px, py, blur, settings, &s);
                    pix_to_face[o] = cand[k].face;
                    zbuf[o] = s.zp;
                    for (int c = 0; c < 3; ++c) bary[3 * o + c] = s.out[c];
                    dists[o] = s.dist;
                    if (state) state[o] = SFX(slot_code)(&s);
                } else {
                    pix_to_face[o] = -1;
                    zbuf[o] = (R)-1;
                    for (int c = 0; c < 3; ++c) bary[3 * o + c] = (R)-1;
                    dists[o] = (R)-1;
                    if (state) state[o] = -1;
                }
            }
        }
        free(cand);
    }
    return err;
}

/*
 * Backward pass over the same pixel list: for every filled slot (pixel,
 * face = pix_to_face), recompute the forward state and apply the chain rule
 * of L = sum over slots of gz*zbuf + gb.bary + gd*dists. Per-slot partials
 * are formed in type R and summed into grad_verts (binary64, [V,3], caller
 * zeroes it) in slot order. Gradient arrays are [npix, K] ([npix, K, 3] for
 * bary); NULL means zero. Padded slots (pix_to_face < 0) are ignored.
 */
int SFX(oracle_backward)(const R* verts, int64_t V, const int64_t* faces, int64_t F,
                         const int64_t* offsets, int64_t N, int64_t H, int64_t W, int64_t K, R blur,
                         uint32_t settings, const int64_t* pixels, int64_t npix, const int64_t* pix_to_face,
                         const float* grad_zbuf, const float* grad_bary, const float* grad_dists,
                         double* grad_verts) {
    if (V < 0 || F < 0 || N < 0 || H < 1 || W < 1 || K < 1) return 1;
    (void)offsets;
    int64_t total = N * H * W;
    if (pixels == NULL) npix = total;
    int err = 0;
    SFX(slot_t) s;
    for (int64_t q = 0; q < npix; ++q) {
        int64_t pid = pixels ? pixels[q] : q;
        if (pid < 0 || pid >= total) {
            err = 2;
            continue;
        }
        int64_t i = (pid / W) % H;
        int64_t j = pid % W;
        R px = SFX(pixel_centre)(j, W);
        R py = SFX(pixel_centre)(i, H);
        for (int64_t k = 0; k < K; ++k) {
            int64_t o = q * K + k;
            int64_t f = pix_to_face[o];
            if (f < 0) continue;
            if (f >= F || !SFX(eval_face)(verts, V, faces, f, px, py, blur, settings, &s)) {
                err = 3; /* pix_to_face does not come from a forward pass on these inputs */
                continue;
            }
            R gz = grad_zbuf ? (R)grad_zbuf[o] : (R)0;
            R gd = grad_dists ? (R)grad_dists[o] : (R)0;
            R gbh[3], gout[3];
            for (int c = 0; c < 3; ++c) gout[c] = grad_bary ? (R)grad_bary[3 * o + c] : (R)0;
            /* the returned barycentrics are bh unless they are the unclipped ones */
            for (int c = 0; c < 3; ++c) gbh[c] = (settings & ORACLE_UNCLIPPED) ? (R)0 : gout[c];

            R gx[3] = {0, 0, 0}, gy[3] = {0, 0, 0}, gzv[3];
            /* depth: zp = sum bh[k] z[k] */
            for (int c = 0; c < 3; ++c) {
                gzv[c] = gz * s.bh[c];
                gbh[c] = gbh[c] + gz * s.z[c];
            }
            R dot = (gbh[0] * s.bh[0] + gbh[1] * s.bh[1]) + gbh[2] * s.bh[2];
            R gb[3];
            for (int c = 0; c < 3; ++c) {
                R gc;
                if (settings & ORACLE_PERSPECTIVE) {
                    /* bh = n / D, n_c = c_c z_{c+1} z_{c+2} */
                    R gn = (gbh[c] - dot) * s.invD;
                    int c1 = (c + 1) % 3, c2 = (c + 2) % 3;
                    gc = gn * (s.z[c1] * s.z[c2]);
                    gzv[c1] += gn * (s.c[c] * s.z[c2]);
                    gzv[c2] += gn * (s.c[c] * s.z[c1]);
                } else {
                    /* renormalisation bh = c / S */
                    gc = (gbh[c] - dot) * s.invS;
                }
                /* clip to [0,1]: passes the gradient only strictly inside the interval */
                gb[c] = (s.b[c] > (R)0 && s.b[c] < (R)1) ? gc : (R)0;
            }
            if ((settings & ORACLE_UNCLIPPED) && (settings & ORACLE_PERSPECTIVE)) {
                /* out = nr / Dr, nr_c = b_c z_{c+1} z_{c+2} */
                R dotr = (gout[0] * s.out[0] + gout[1] * s.out[1]) + gout[2] * s.out[2];
                for (int c = 0; c < 3; ++c) {
                    R gn = (gout[c] - dotr) * s.invDr;
                    int c1 = (c + 1) % 3, c2 = (c + 2) % 3;
                    gb[c] += gn * (s.z[c1] * s.z[c2]);
                    gzv[c1] += gn * (s.b[c] * s.z[c2]);
                    gzv[c2] += gn * (s.b[c] * s.z[c1]);
                }
            } else if (settings & ORACLE_UNCLIPPED) {
                for (int c = 0; c < 3; ++c) gb[c] += gout[c];
            }
            /* b = w / A */
            R gw[3];
            for (int c = 0; c < 3; ++c) gw[c] = gb[c] * s.invA;
            R gA = -((gb[0] * s.b[0] + gb[1] * s.b[1]) + gb[2] * s.b[2]) * s.invA;
            /* w0 = dx1*dy2 - dy1*dx2, with dx = x - px, dy = y - py */
            gx[1] += gw[0] * s.dy[2];
            gy[2] += gw[0] * s.dx[1];
            gy[1] -= gw[0] * s.dx[2];
            gx[2] -= gw[0] * s.dy[1];
            /* w1 = dx2*dy0 - dy2*dx0 */
            gx[2] += gw[1] * s.dy[0];
            gy[0] += gw[1] * s.dx[2];
            gy[2] -= gw[1] * s.dx[0];
            gx[0] -= gw[1] * s.dy[2];
            /* w2 = dx0*dy1 - dy0*dx1 */
            gx[0] += gw[2] * s.dy[1];
            gy[1] += gw[2] * s.dx[0];
            gy[0] -= gw[2] * s.dx[1];
            gx[1] -= gw[2] * s.dy[0];
            /* A = (x1-x0)(y2-y0) - (y1-y0)(x2-x0) */
            gx[0] += gA * (s.y[1] - s.y[2]);
            gx[1] += gA * (s.y[2] - s.y[0]);
            gx[2] += gA * (s.y[0] - s.y[1]);
            gy[0] += gA * (s.x[2] - s.x[1]);
            gy[1] += gA * (s.x[0] - s.x[2]);
            gy[2] += gA * (s.x[1] - s.x[0]);
            /* dists = +-d2, d2 = |q - t u|^2 on the nearest edge (a, b), t held fixed
             * (it is either the stationary point or clamped) */
            R gd2 = s.inside ? -gd : gd;
            {
                int e = s.argmin, a = e, bb = (e + 1) % 3;
                R t = s.t[e];
                R ga = gd2 * (R)-2 * ((R)1 - t);
                R gbv = gd2 * (R)-2 * t;
                gx[a] += ga * s.rx[e];
                gy[a] += ga * s.ry[e];
                gx[bb] += gbv * s.rx[e];
                gy[bb] += gbv * s.ry[e];
            }
            for (int c = 0; c < 3; ++c) {
                int64_t vi = s.vi[c];
                grad_verts[3 * vi + 0] += (double)gx[c];
                grad_verts[3 * vi + 1] += (double)gy[c];
                grad_verts[3 * vi + 2] += (double)gzv[c];
            }
        }
    }
    return err;
}
