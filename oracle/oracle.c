/*
 * Oracle for sparse direct convolution -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct CPU reference.  It shares no code, header or table with
 * the GPU library; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * may load it.  Nothing on the product path calls it.
 *
 * Sources (cited by page title and section; formulas are restated, not copied):
 *  [T] Tuteja et al., "Theoretical and Empirical Analysis of Sparse Convolution":
 *      Sec. 3 Eq. (1) (multi-channel convolution with the sum clipped to the image),
 *      Eq. (2) (output size), Eq. (3) (sparse form: sum over the non-zeros whose
 *      padding-shifted input position is inside the image).
 *  [E] "Escoin: Efficient Sparse Convolutional Neural Network Inference on GPUs":
 *      the 7-variable CONV loop nest (its Eq. 1 / Algorithm 1), the CSR format
 *      (value / colidx / rowptr over the M x CRS filter matrix), the layout function
 *      f(c,y,x) with f(c,y+r,x+s) = f(c,y,x) + f(0,r,s) and CHW form
 *      f(c,r,s) = (c*H + r)*W + s ("weight stretching"), and the sequential direct
 *      sparse convolution (its Algorithm 2: image n, output channel m, non-zero j,
 *      then the 2-D output plane).
 *  [T] Sec. 5.3 and Fig. 4 (the packed weight word): one u32 per non-zero holding the fp16
 *      weight in bits 31-16, the input channel in bits 15-8, the kernel column offset px in
 *      bits 7-4 and the kernel row offset py in bits 3-0; the weight is widened to fp32
 *      before use and all accumulation stays in fp32 (here: double).
 *
 * Readings taken where the pages are silent (each also listed in the design notes):
 *  - stride enters as iy = e*stride - pad + r, ix = f*stride - pad + s (cross-correlation,
 *    no kernel flip); Eq. (1) is written for stride 1.
 *  - the stretched offset uses the UNPADDED input dims: off = c*H*W + r*W + s.
 *  - which positions are non-zeros: with a mask, exactly the mask bits (explicit zero values
 *    kept); without a mask, every w != 0.0f (so -0.0 is dropped and NaN kept).
 *  - accumulation in double precision; the caller rounds the result once to fp32.
 *  - MAG[n,m,e,f] = sum of |w * x| over the same terms, the scale of the error bound.
 *  - fp32 -> fp16 of the packed word: IEEE 754 binary16, round to nearest with ties to
 *    even (the pages name no rounding); magnitudes at or above 65520 become infinity, NaN
 *    stays NaN.  px is the filter column s, py the filter row r.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* [T] Eq. (2): number of output positions along one axis; <= 0 means the layer is empty. */
int64_t oracle_out_size(int64_t in, int64_t pad, int64_t k, int64_t stride) {
    if (stride <= 0) return 0;
    int64_t span = in + 2 * pad - k;
    if (span < 0) return 0;
    return span / stride + 1;
}

/* Whether filter position p (row-major m,c,r,s) is a stored non-zero. */
static int kept_at(const float* w, const uint8_t* mask, int64_t p) {
    if (mask) return mask[p] != 0;
    return w[p] != 0.0f; /* NaN != 0 is true: NaN is kept; -0.0 == 0.0: dropped */
}

/* Number of stored non-zeros of an M x CRS dense filter matrix. */
int64_t oracle_count_kept(const float* w, const uint8_t* mask, int64_t total) {
    int64_t n = 0;
    for (int64_t p = 0; p < total; p++) n += kept_at(w, mask, p);
    return n;
}

/* [E] CSR of the M x CRS filter matrix: rows m ascending, columns ascending in a row.
 * rowptr has M+1 entries, colidx and value have nnz entries. */
void oracle_csr_from_dense(int32_t M, int32_t CRS, const float* w, const uint8_t* mask,
                           int32_t* rowptr, int32_t* colidx, float* value) {
    int32_t j = 0;
    rowptr[0] = 0;
    for (int32_t m = 0; m < M; m++) {
        for (int32_t col = 0; col < CRS; col++) {
            int64_t p = (int64_t)m * CRS + col;
            if (kept_at(w, mask, p)) {
                colidx[j] = col;
                value[j] = w[p];
                j++;
            }
        }
        rowptr[m + 1] = j;
    }
}

/* [E] weight stretching: column index c*R*S + r*S + s becomes the CHW input offset
 * f(c,r,s) = (c*H + r)*W + s of the unpadded input. */
void oracle_stretch(int32_t C, int32_t R, int32_t S, int32_t H, int32_t W, int64_t nnz,
                    const int32_t* colidx, uint32_t* off) {
    (void)C;
    for (int64_t j = 0; j < nnz; j++) {
        int32_t col = colidx[j];
        int32_t c = col / (R * S);
        int32_t r = (col / S) % R;
        int32_t s = col % S;
        off[j] = (uint32_t)(((int64_t)c * H + r) * W + s);
    }
}

/*
 * Definitional form: the 7-variable loop nest n, m, e, f, c, r, s of [E] Eq. 1 with the
 * clipping of [T] Eq. (1) and a skip of every filter position that is not a non-zero.
 * x: N*C*H*W, w: M*C*R*S (row-major), mask: M*C*R*S or NULL.  y, mag: N*M*E*F doubles.
 */
void oracle_conv_def(int32_t N, int32_t C, int32_t H, int32_t W, int32_t M, int32_t R,
                     int32_t S, int32_t stride, int32_t pad, const float* x, const float* w,
                     const uint8_t* mask, double* y, double* mag) {
    int64_t E = oracle_out_size(H, pad, R, stride);
    int64_t F = oracle_out_size(W, pad, S, stride);
    if (E <= 0 || F <= 0) return;
    for (int64_t n = 0; n < N; n++)
        for (int64_t m = 0; m < M; m++)
            for (int64_t e = 0; e < E; e++)
                for (int64_t f = 0; f < F; f++) {
                    double acc = 0.0, am = 0.0;
                    for (int64_t c = 0; c < C; c++)
                        for (int64_t r = 0; r < R; r++)
                            for (int64_t s = 0; s < S; s++) {
                                int64_t p = ((m * C + c) * R + r) * S + s;
                                if (!kept_at(w, mask, p)) continue;
                                int64_t iy = e * stride - pad + r;
                                int64_t ix = f * stride - pad + s;
                                if (iy < 0 || iy >= H || ix < 0 || ix >= W) continue;
                                double prod = (double)w[p] * (double)x[((n * C + c) * H + iy) * W + ix];
                                acc += prod;
                                am += fabs(prod);
                            }
                    int64_t o = ((n * M + m) * E + e) * F + f;
                    y[o] = acc;
                    mag[o] = am;
                }
}

/*
 * List form, in the order of [E] Algorithm 2, for one (n, m) plane: walk the CSR row's
 * non-zeros j (column -> c, r, s; value v) and add v * x over the output plane, keeping
 * only the terms [T] Eq. (3) keeps (input position inside the image).  The plane is
 * accumulated in doubles in this fixed order.
 */
static void conv_plane_csr(int64_t n, int64_t m, int32_t C, int32_t H, int32_t W, int32_t R,
                           int32_t S, int32_t stride, int32_t pad, int64_t E, int64_t F,
                           const float* x, const int32_t* rowptr, const int32_t* colidx,
                           const float* value, double* yp, double* ap) {
    for (int64_t i = 0; i < E * F; i++) { yp[i] = 0.0; ap[i] = 0.0; }
    for (int64_t j = rowptr[m]; j < rowptr[m + 1]; j++) {
        int64_t col = colidx[j];
        int64_t c = col / ((int64_t)R * S);
        int64_t r = (col / S) % R;
        int64_t s = col % S;
        double v = (double)value[j];
        const float* xp = x + (n * C + c) * (int64_t)H * W;
        for (int64_t e = 0; e < E; e++) {
            int64_t iy = e * stride - pad + r;
            if (iy < 0 || iy >= H) continue;
            for (int64_t f = 0; f < F; f++) {
                int64_t ix = f * stride - pad + s;
                if (ix < 0 || ix >= W) continue;
                double prod = v * (double)xp[iy * W + ix];
                yp[e * F + f] += prod;
                ap[e * F + f] += fabs(prod);
            }
        }
    }
}

/* List form over every (n, m) plane; planes are independent and spread over threads. */
void oracle_conv_csr(int32_t N, int32_t C, int32_t H, int32_t W, int32_t M, int32_t R,
                     int32_t S, int32_t stride, int32_t pad, const float* x,
                     const int32_t* rowptr, const int32_t* colidx, const float* value,
                     double* y, double* mag, int32_t nthreads) {
    int64_t E = oracle_out_size(H, pad, R, stride);
    int64_t F = oracle_out_size(W, pad, S, stride);
    if (E <= 0 || F <= 0) return;
    int64_t planes = (int64_t)N * M;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#else
    (void)nthreads;
#endif
    for (int64_t nm = 0; nm < planes; nm++)
        conv_plane_csr(nm / M, nm % M, C, H, W, R, S, stride, pad, E, F, x, rowptr, colidx,
                       value, y + nm * E * F, mag + nm * E * F);
}

/* The list form restricted to selected planes (ids n*M + m in planes_sel); y and mag hold
 * one E*F plane per selected id.  Used to check sampled outputs of full-size layers. */
void oracle_conv_csr_planes(int32_t N, int32_t C, int32_t H, int32_t W, int32_t M, int32_t R,
                            int32_t S, int32_t stride, int32_t pad, const float* x,
                            const int32_t* rowptr, const int32_t* colidx, const float* value,
                            int64_t nsel, const int64_t* planes_sel, double* y, double* mag,
                            int32_t nthreads) {
    int64_t E = oracle_out_size(H, pad, R, stride);
    int64_t F = oracle_out_size(W, pad, S, stride);
    if (E <= 0 || F <= 0) return;
    (void)N;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#else
    (void)nthreads;
#endif
    for (int64_t q = 0; q < nsel; q++)
        conv_plane_csr(planes_sel[q] / M, planes_sel[q] % M, C, H, W, R, S, stride, pad, E, F,
                       x, rowptr, colidx, value, y + q * E * F, mag + q * E * F);
}

/*
 * IEEE 754 binary16 bits of the fp32 value v, rounded to nearest, ties to even.  Written
 * from the format's definition: a finite half is (-1)^sign * n * 2^(e-10) with an 11-bit
 * significand n in [1024, 2048) for normal exponents e in [-14, 15], and n * 2^-24 with
 * n < 1024 below 2^-14 (subnormals).  The magnitude is divided by its quantum (exact, both
 * are powers of two times fp32 values in a double), rounded with rint (ties to even in the
 * default rounding mode) and re-assembled; a carry into the next binade is handled by the
 * re-assembly, and a result past 65504 is infinity.
 */
uint16_t oracle_fp16_bits(float v) {
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7E00u);
    double a = fabs((double)v);
    if (isinf(v) || a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
    if (a < ldexp(1.0, -14)) {                 /* subnormal quantum 2^-24 */
        double n = rint(a / ldexp(1.0, -24)); /* 0 .. 1024 (1024 is the smallest normal) */
        return (uint16_t)(sign | (uint16_t)n);
    }
    int k;
    (void)frexp(a, &k);                        /* a = f * 2^k, f in [0.5, 1): exponent e = k-1 */
    int e = k - 1;
    double n = rint(a / ldexp(1.0, e - 10));   /* 1024 .. 2048 */
    if (n == 2048.0) { n = 1024.0; e += 1; }
    if (e > 15) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(n - 1024.0));
}

/* Value of the binary16 bits h, as a double (exact). */
double oracle_fp16_value(uint16_t h) {
    double sgn = (h & 0x8000u) ? -1.0 : 1.0;
    int ex = (h >> 10) & 31;
    int mant = h & 1023;
    if (ex == 31) return mant ? NAN : sgn * INFINITY;
    if (ex == 0) return sgn * ldexp((double)mant, -24);
    return sgn * ldexp((double)(1024 + mant), ex - 25);
}

/* [T] Sec. 5.3 / Fig. 4: the packed word of one non-zero. ic < 256, px, py < 16. */
uint32_t oracle_pack_word(float v, int32_t ic, int32_t px, int32_t py) {
    return ((uint32_t)oracle_fp16_bits(v) << 16) | ((uint32_t)ic << 8) | ((uint32_t)px << 4) |
           (uint32_t)py;
}

/* Fields of a packed word: the fp16 weight widened to double, ic, px, py. */
void oracle_unpack_word(uint32_t wd, double* v, int32_t* ic, int32_t* px, int32_t* py) {
    *v = oracle_fp16_value((uint16_t)(wd >> 16));
    *ic = (int32_t)((wd >> 8) & 255u);
    *px = (int32_t)((wd >> 4) & 15u);
    *py = (int32_t)(wd & 15u);
}

/* Packed words of every CSR non-zero, in CSR order: column c*R*S + r*S + s gives ic = c,
 * px = s (kernel column), py = r (kernel row). */
void oracle_words_from_csr(int32_t R, int32_t S, int64_t nnz, const int32_t* colidx,
                           const float* value, uint32_t* words) {
    for (int64_t j = 0; j < nnz; j++) {
        int32_t col = colidx[j];
        int32_t c = col / (R * S);
        int32_t r = (col / S) % R;
        int32_t s = col % S;
        words[j] = oracle_pack_word(value[j], c, s, r);
    }
}

/* The CSR non-zeros a list of packed words describes: column c*R*S + r*S + s from
 * (ic, py, px) and the fp16 weight widened to fp32 (exact). */
void oracle_csr_from_words(int32_t R, int32_t S, int64_t nnz, const uint32_t* words,
                           int32_t* colidx, float* value) {
    for (int64_t j = 0; j < nnz; j++) {
        double v;
        int32_t ic, px, py;
        oracle_unpack_word(words[j], &v, &ic, &px, &py);
        colidx[j] = (ic * R + py) * S + px;
        value[j] = (float)v;
    }
}

int32_t oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
