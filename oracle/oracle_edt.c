/*
 * oracle_edt.c -- CPU reference for the exact Euclidean distance transform.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU library.  Plain, serial,
 * float64 code written for a reader to check against the sources by eye.
 *
 * What is computed.  "GPU-Based Parallel Euclidean Distance Transform
 * Algorithm" (Mathematics 14(4), §1 Introduction) defines the transform: each
 * pixel is a point with integer coordinates, and each foreground pixel gets
 * the Euclidean distance to its nearest background pixel; equivalently each
 * pixel lies in the Voronoi cell of that background pixel.  Here the squared
 * distance (with per-axis grid spacing s_k) and the coordinates of that
 * nearest background element are returned, for any rank.
 *
 * oracle_edt_brute      -- the definition itself: every element against every
 *                          background element (as the per-cell raster Voronoi
 *                          method of the Chinese-language GPU Voronoi page,
 *                          §2.2 Step 4, and TorchMorph's brute-force transform).
 * oracle_edt_separable  -- the independent-scanning scheme (§2.1 of the
 *                          PR-EDT paper): a per-line pass along axis 0 (§3.2,
 *                          upper/lower candidates from forward and backward
 *                          propagation), then one lower-envelope pass per
 *                          remaining axis (TorchMorph, the separable
 *                          lower-envelope paragraph; PR-EDT §3.3 dominance
 *                          test of Figures 4-5 and the insertion sweep of
 *                          Algorithm 1; §3.4 query of the 1-D Voronoi diagram).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - mask value 0 is background, anything else foreground;
 *  - ties between equidistant background elements: each 1-D step keeps the
 *    smaller coordinate; a middle parabola whose bisector intersections
 *    coincide (x == y in the dominance test) is removed;
 *  - an image with no background uses a virtual background element at
 *    (-1, 0, ..., 0), the convention SciPy follows.
 */
#include "oracle_edt.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int64_t element_count(int ndim, const int64_t* shape) {
    int64_t n = 1;
    for (int k = 0; k < ndim; ++k) n *= shape[k];
    return n;
}

static int check_args(const uint8_t* mask, int ndim, const int64_t* shape,
                      const double* sampling, const double* sqdist) {
    if (!mask || !shape || !sqdist || ndim < 1 || ndim > 8) return -1;
    for (int k = 0; k < ndim; ++k) {
        if (shape[k] < 1) return -1;
        if (sampling && !(sampling[k] > 0.0)) return -1;
    }
    return 0;
}

/* Coordinates of flat index p (C order). */
static void unravel(int64_t p, int ndim, const int64_t* shape, int64_t* coord) {
    for (int k = ndim - 1; k >= 0; --k) {
        coord[k] = p % shape[k];
        p /= shape[k];
    }
}

/* No background anywhere: the virtual background element (-1, 0, ..., 0). */
static void virtual_background(int ndim, const int64_t* shape, const double* s2,
                               double* sqdist, int32_t* feature) {
    int64_t n = element_count(ndim, shape);
    int64_t coord[8];
    for (int64_t p = 0; p < n; ++p) {
        unravel(p, ndim, shape, coord);
        double d = s2[0] * (double)(coord[0] + 1) * (double)(coord[0] + 1);
        for (int k = 1; k < ndim; ++k) d += s2[k] * (double)coord[k] * (double)coord[k];
        sqdist[p] = d;
        if (feature) {
            feature[p * ndim + 0] = -1;
            for (int k = 1; k < ndim; ++k) feature[p * ndim + k] = 0;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Brute force: the definition.                                              */
/* ------------------------------------------------------------------------ */

int oracle_edt_brute(const uint8_t* mask, int ndim, const int64_t* shape,
                     const double* sampling, double* sqdist, int32_t* feature) {
    if (check_args(mask, ndim, shape, sampling, sqdist)) return -1;
    double s2[8];
    for (int k = 0; k < ndim; ++k) s2[k] = sampling ? sampling[k] * sampling[k] : 1.0;
    int64_t n = element_count(ndim, shape);

    int64_t nbg = 0;
    for (int64_t p = 0; p < n; ++p) nbg += (mask[p] == 0);
    if (nbg == 0) {
        virtual_background(ndim, shape, s2, sqdist, feature);
        return 0;
    }
    int64_t* bg = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nbg * ndim));
    if (!bg) return -2;
    int64_t j = 0;
    for (int64_t p = 0; p < n; ++p)
        if (mask[p] == 0) unravel(p, ndim, shape, bg + (j++) * ndim);

    int64_t coord[8];
    for (int64_t p = 0; p < n; ++p) {
        unravel(p, ndim, shape, coord);
        double best = INFINITY;
        int64_t who = -1;
        for (int64_t b = 0; b < nbg; ++b) {
            double d = 0.0;
            for (int k = 0; k < ndim; ++k) {
                double t = (double)(coord[k] - bg[b * ndim + k]);
                d += s2[k] * t * t;
            }
            if (d < best) { best = d; who = b; }   /* first minimiser wins */
        }
        sqdist[p] = best;
        if (feature)
            for (int k = 0; k < ndim; ++k) feature[p * ndim + k] = (int32_t)bg[who * ndim + k];
    }
    free(bg);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Separable scheme.                                                         */
/* ------------------------------------------------------------------------ */

/*
 * Lower envelope of the parabolas  y_j(q) = s2*(q - j)^2 + f[j]  for the
 * candidates j (0 <= j < n) with finite f[j]; for every q in [0, n) returns
 * the minimising candidate owner[q] (-1 if there is none) and the minimum.
 *
 * With Y_j = f[j] + s2*j^2, parabolas a < b meet at q = (Y_b - Y_a) / (2*s2*(b-a)):
 * the bisector of the two background elements crosses the line there (PR-EDT
 * §3.3, Figure 4).  For consecutive members a < b < c, b keeps a non-empty
 * interval iff x(a,b) < x(b,c) (Figure 5); multiplying out the positive
 * denominators gives the division-free test below.
 */
static int dominated(const double* Y, int a, int b, int c) {
    return (Y[b] - Y[a]) * (double)(c - b) >= (Y[c] - Y[b]) * (double)(b - a);
}

static void envelope_1d(int n, double s2, const double* f, double* Y, int* stack,
                        int* owner, double* out) {
    int k = 0;
    /* Build: insert candidates by increasing coordinate; after each insertion
       remove the earlier members it dominates (PR-EDT Algorithm 1). */
    for (int j = 0; j < n; ++j) {
        if (!isfinite(f[j])) continue;
        Y[j] = f[j] + s2 * (double)j * (double)j;
        while (k >= 2 && dominated(Y, stack[k - 2], stack[k - 1], j)) --k;
        stack[k++] = j;
    }
    if (k == 0) {
        for (int q = 0; q < n; ++q) { owner[q] = -1; out[q] = INFINITY; }
        return;
    }
    /* Query: walk the 1-D Voronoi diagram of the line (PR-EDT §3.4); move to
       the next member only where it is strictly nearer. */
    int m = 0;
    for (int q = 0; q < n; ++q) {
        while (m + 1 < k &&
               2.0 * s2 * (double)q * (double)(stack[m + 1] - stack[m]) >
                   Y[stack[m + 1]] - Y[stack[m]])
            ++m;
        int j = stack[m];
        owner[q] = j;
        out[q] = s2 * (double)(q - j) * (double)(q - j) + f[j];
    }
}

int oracle_edt_separable(const uint8_t* mask, int ndim, const int64_t* shape,
                         const double* sampling, double* sqdist, int32_t* feature) {
    if (check_args(mask, ndim, shape, sampling, sqdist)) return -1;
    double s2[8];
    for (int k = 0; k < ndim; ++k) s2[k] = sampling ? sampling[k] * sampling[k] : 1.0;
    const int64_t n = element_count(ndim, shape);
    int64_t stride[8];
    stride[ndim - 1] = 1;
    for (int k = ndim - 2; k >= 0; --k) stride[k] = stride[k + 1] * shape[k + 1];

    int64_t maxlen = 0;
    for (int k = 0; k < ndim; ++k) if (shape[k] > maxlen) maxlen = shape[k];

    /* The nearest background element found so far, per element, as its
       coordinates along the axes processed so far. */
    int32_t* feat = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n * ndim));
    double* fl = (double*)malloc(sizeof(double) * (size_t)maxlen);
    double* Y = (double*)malloc(sizeof(double) * (size_t)maxlen);
    double* outl = (double*)malloc(sizeof(double) * (size_t)maxlen);
    int* stack = (int*)malloc(sizeof(int) * (size_t)maxlen);
    int* owner = (int*)malloc(sizeof(int) * (size_t)maxlen);
    int32_t* featl = (int32_t*)malloc(sizeof(int32_t) * (size_t)(maxlen * ndim));
    if (!feat || !fl || !Y || !outl || !stack || !owner || !featl) {
        free(feat); free(fl); free(Y); free(outl); free(stack); free(owner); free(featl);
        return -2;
    }

    int any_background = 0;
    int64_t coord[8];

    /* Axis 0: nearest background on each line along axis 0.  A forward sweep
       gives the nearest at or before i (the "upper candidate"), a backward
       sweep the nearest at or after i (the "lower candidate"), PR-EDT §3.2;
       the nearer one is kept, the earlier on a tie.  Keeping only the nearer
       candidate is exact because the offset along the other axes is the same
       for both. */
    {
        const int64_t n0 = shape[0], st = stride[0];
        for (int64_t base = 0; base < st; ++base) {
            int64_t last = -1;
            for (int64_t i = 0; i < n0; ++i) {   /* forward: record "up" in owner[] */
                if (mask[base + i * st] == 0) last = i;
                owner[i] = (int)last;
            }
            int64_t next = -1;
            for (int64_t i = n0 - 1; i >= 0; --i) {   /* backward: choose */
                int64_t p = base + i * st;
                if (mask[p] == 0) { next = i; any_background = 1; }
                int64_t up = owner[i], g = -1;
                if (up >= 0 && (next < 0 || i - up <= next - i)) g = up;
                else if (next >= 0) g = next;
                if (g >= 0) {
                    sqdist[p] = s2[0] * (double)(i - g) * (double)(i - g);
                    unravel(p, ndim, shape, coord);
                    feat[p * ndim + 0] = (int32_t)g;
                    for (int k = 1; k < ndim; ++k) feat[p * ndim + k] = (int32_t)coord[k];
                } else {
                    sqdist[p] = INFINITY;
                }
            }
        }
    }

    if (!any_background) {
        virtual_background(ndim, shape, s2, sqdist, feature);
        free(feat); free(fl); free(Y); free(outl); free(stack); free(owner); free(featl);
        return 0;
    }

    /* Axes 1..ndim-1: lower envelope of parabolas along every line
       (TorchMorph's separable lower-envelope formulation). */
    for (int ax = 1; ax < ndim; ++ax) {
        const int64_t nk = shape[ax], st = stride[ax];
        const int64_t block = nk * st;
        for (int64_t outer = 0; outer < n / block; ++outer) {
            for (int64_t inner = 0; inner < st; ++inner) {
                const int64_t base = outer * block + inner;
                for (int64_t j = 0; j < nk; ++j) {
                    int64_t p = base + j * st;
                    fl[j] = sqdist[p];
                    memcpy(featl + j * ndim, feat + p * ndim, sizeof(int32_t) * (size_t)ndim);
                }
                envelope_1d((int)nk, s2[ax], fl, Y, stack, owner, outl);
                for (int64_t q = 0; q < nk; ++q) {
                    int64_t p = base + q * st;
                    sqdist[p] = outl[q];
                    if (owner[q] >= 0) {
                        memcpy(feat + p * ndim, featl + (int64_t)owner[q] * ndim,
                               sizeof(int32_t) * (size_t)ndim);
                        feat[p * ndim + ax] = owner[q];
                    }
                }
            }
        }
    }

    if (feature) memcpy(feature, feat, sizeof(int32_t) * (size_t)(n * ndim));
    free(feat); free(fl); free(Y); free(outl); free(stack); free(owner); free(featl);
    return 0;
}
