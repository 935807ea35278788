/*
 * CPU oracle for K-nearest-face mesh rasterization and its backward pass.
 *
 * TEST INFRASTRUCTURE ONLY. This library is the plain, slow definition that
 * the GPU path is checked against; only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it. It shares no code, header or
 * constant with the GPU path.
 *
 * The method and its conventions are described in raster_oracle_impl.h.
 * Exported symbols (suffix _f32: canonical binary32; _f64: binary64):
 *   oracle_raster_f32/_f64, oracle_backward_f32/_f64, oracle_num_threads.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fno-fast-math -fPIC -shared
 */
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#if defined(__FLT_EVAL_METHOD__) && __FLT_EVAL_METHOD__ != 0
#error "the oracle needs every float operation rounded to float (FLT_EVAL_METHOD == 0)"
#endif
#if defined(__FAST_MATH__)
#error "the oracle must not be built with fast-math"
#endif
/* Contraction is disabled by -ffp-contract=off on the build line. */

#define R float
#define SFX(name) name##_f32
#include "raster_oracle_impl.h"
#undef R
#undef SFX

#define R double
#define SFX(name) name##_f64
#include "raster_oracle_impl.h"
#undef R
#undef SFX

/* Number of OpenMP threads a parallel region of the oracle uses. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
