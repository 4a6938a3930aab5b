/*
 * oracle_edt.h -- CPU reference for the exact Euclidean distance transform.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or constant with the GPU library and never calls it.
 *
 * Conventions (both routines):
 *   mask      uint8, C order, shape[0] x ... x shape[ndim-1]; 0 = background.
 *   sampling  ndim grid spacings (NULL = all 1.0); sampling[k] scales axis k.
 *   sqdist    out, N doubles: squared distance to the nearest background.
 *   feature   out, N*ndim int32 (may be NULL): coordinates of that background
 *             element, element-major (feature[p*ndim + k] is axis k of p).
 *   An image without any background uses a virtual background element at
 *   (-1, 0, ..., 0) (the convention SciPy follows; see the test fixtures).
 * Return 0 on success, -1 on bad arguments, -2 on allocation failure.
 */
#ifndef ORACLE_EDT_H
#define ORACLE_EDT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int oracle_edt_separable(const uint8_t* mask, int ndim, const int64_t* shape,
                         const double* sampling, double* sqdist, int32_t* feature);

int oracle_edt_brute(const uint8_t* mask, int ndim, const int64_t* shape,
                     const double* sampling, double* sqdist, int32_t* feature);

#ifdef __cplusplus
}
#endif

#endif
