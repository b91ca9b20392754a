/*
 * eqref.c -- plain fp64 CPU oracle for the equivariant linear layers.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library calls this file; only the
 * tests, the smoke check and the benchmark's CPU-baseline leg load it.  It
 * shares no code, header or table with the GPU path.
 *
 * Every routine computes a plain definition, with plain loops, in fp64:
 *
 *  - C_N layer.  "Flash EQ-Linear" (gist.science summary), Core Insight: the
 *    layer is a circular convolution along the group axis composed with a
 *    channel mixing, and its weight matrix is group-circulant, i.e. built by
 *    cyclically shifting and replicating a small set of learnable parameters.
 *    Problem Statement: the usual implementation replicates those parameters
 *    into a dense matrix and multiplies.  Written out:
 *        W_dense[o*N+g][i*N+h] = w[o][i][(g-h) mod N]
 *        y[t][o*N+g] = sum_{i,h} W_dense[o*N+g][i*N+h] * x[t][i*N+h]
 *    (eqref_cn_expand + eqref_apply_dense), and the same sum taken directly
 *    as a convolution (eqref_cn_direct).
 *
 *  - Weight spectrum.  Algorithmic Approach: the group axis is taken to the
 *    Fourier domain with the DFT; for real data only the non-redundant half
 *    of the bins is kept.  eqref_cn_weight_dft evaluates
 *        What[k] = sum_m w[m] * exp(-2*pi*i*m*k/N),  k = 0 .. floor(N/2)
 *    and packs it into N real planes: plane 0 = Re What[0]; planes 2k-1, 2k =
 *    Re, Im What[k] for 1 <= k < N/2; plane N-1 = Re What[N/2] when N is even.
 *
 *  - Gradients of the C_N layer.  "Flash EQ-Linear", Implementation: the
 *    kernels cover the backward pass as well as the forward pass (Experimental
 *    Results, Operator Level: backward speedups).  The pages give no formula;
 *    these are the derivatives of the layer's definition above.  For an
 *    upstream gradient dy = dL/dy,
 *        dx[t][i][h] = sum_{o,g} w[o][i][(g-h) mod N] * dy[t][o][g]
 *                    = (W_dense^T dy[t])[i*N+h]
 *    (eqref_cn_backward_data, and the dense route eqref_apply_dense_t), and
 *        dw[o][i][m] = sum_{t,g} dy[t][o][g] * x[t][i][(g-m) mod N]
 *    (eqref_cn_backward_weight).
 *
 *  - Fused neighbours of the layer in an MLP.  "Quick ViTs" (papernotes), key
 *    design 2: the MLP keeps its expansion, GELU and contraction, and GELU is
 *    applied where the group acts by permuting coordinates (the regular
 *    representation), which for C_N is y[t][o][g] itself: the group acts by a
 *    cyclic shift along g.  A per-channel bias constant along g and a pointwise
 *    GELU both commute with that shift.  eqref_bias_act applies, in place,
 *        y[t][o][g] <- act(y[t][o][g] + b[o]),  GELU(v) = v * Phi(v)
 *    with Phi the standard normal distribution function, written as
 *    erfc(-v/sqrt 2) / 2 (equal to (1 + erf(v/sqrt 2)) / 2, but without the
 *    cancellation of 1 + erf for negative v, so the tail keeps its digits).
 *
 *  - D8 Fourier-domain layer.  "Quick ViTs" (papernotes), key design 2
 *    (Fourier-domain equivariant computation): a width-C map is four square
 *    blocks of size C/8 (irreps A1, A2, B1, B2) and one square block of size
 *    C/4 that is applied to both coordinates of the 2-D irrep E.  With the
 *    feature layout [A1 | A2 | B1 | B2 | E coord 0 | E coord 1] the layer is a
 *    block-diagonal matrix (eqref_d8_expand) times x.
 *
 *  - D8 round trip around GELU.  "Quick ViTs", key design 2: GELU does not
 *    commute with a general representation, so the features go back to the
 *    regular representation (where the group only permutes the 8 values of a
 *    channel), GELU is applied there, and they return to the Fourier domain;
 *    the page fuses the round trip and GELU into one kernel.  The transform is
 *    the group's orthonormal Fourier matrix (eqref_d8_fourier_matrix, built
 *    from the irreps' generator matrices), one regular channel j of m = C/8
 *    gathering A1..B2 at j and E copies 2j, 2j+1 (eqref_d8_to_regular,
 *    eqref_d8_to_fourier, eqref_d8_bias_act).  A bias that keeps the block
 *    equivariant is constant over the group elements: one value per channel j.
 *
 *  - Dihedral groups beyond D8.  "Flash EQ-Linear" (Dutch summary, closing
 *    paragraph) names other shapes and motions as the extension of the 90-degree
 *    case; the reflection groups of the regular n-gon are the direct one.
 *    D_n = <r, s | r^n = s^2 = 1, s r s = r^-1> has order 2n and real irreps
 *    A1 (r, s) -> (1, 1), A2 (1, -1), for even n also B1 (-1, 1), B2 (-1, -1),
 *    and E_k (k = 1 .. n/2 - 1 for even n, .. (n-1)/2 for odd n): r -> rotation
 *    by 2 pi k / n, s -> diag(1, -1).  The layer keeps the D8 layout: per token,
 *    the 1-D irreps' slabs of m = C/2n channels, then for each E_k its
 *    coordinate-0 and coordinate-1 slabs of 2m copies; a square block per 1-D
 *    irrep and one 2m x 2m block per E_k, shared by its two coordinates
 *    (eqref_dn_expand).  The Fourier matrix, transforms and round trip follow
 *    the D8 ones with rows sqrt(d / 2n) times the irreps' entries
 *    (eqref_dn_fourier_matrix, eqref_dn_to_regular, eqref_dn_to_fourier,
 *    eqref_dn_bias_act).  For n = 4 every one of them is the D8 routine.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int eqref_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* W_dense[(o*N+g)*(N*C_in) + i*N+h] = w[(o*C_in+i)*N + (g-h) mod N]. */
void eqref_cn_expand(int N, int C_in, int C_out, const double* w, double* W) {
    const int64_t cols = (int64_t)N * C_in;
    for (int o = 0; o < C_out; ++o)
        for (int g = 0; g < N; ++g)
            for (int i = 0; i < C_in; ++i)
                for (int h = 0; h < N; ++h) {
                    int m = ((g - h) % N + N) % N;
                    W[((int64_t)o * N + g) * cols + (int64_t)i * N + h] =
                        w[((int64_t)o * C_in + i) * N + m];
                }
}

/* y[t][r] = sum_c W[r][c] * x[t][c] for every token (rows x cols matrix). */
void eqref_apply_dense(int64_t T, int64_t rows, int64_t cols, const double* W,
                       const double* x, double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double* xt = x + t * cols;
        double* yt = y + t * rows;
        for (int64_t r = 0; r < rows; ++r) {
            const double* Wr = W + r * cols;
            double acc = 0.0;
            for (int64_t c = 0; c < cols; ++c) acc += Wr[c] * xt[c];
            yt[r] = acc;
        }
    }
}

/* dx[t][c] = sum_r W[r][c] * dy[t][r]: the transposed matrix applied to every token. */
void eqref_apply_dense_t(int64_t T, int64_t rows, int64_t cols, const double* W,
                         const double* dy, double* dx) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double* dyt = dy + t * rows;
        double* dxt = dx + t * cols;
        for (int64_t c = 0; c < cols; ++c) {
            double acc = 0.0;
            for (int64_t r = 0; r < rows; ++r) acc += W[r * cols + c] * dyt[r];
            dxt[c] = acc;
        }
    }
}

/* Replicate-and-multiply: the dense definition of the C_N layer.
 * Returns 0 on success, -1 if the dense matrix cannot be allocated. */
int eqref_cn_dense(int N, int C_in, int C_out, int64_t T, const double* x,
                   const double* w, double* y) {
    const int64_t rows = (int64_t)N * C_out, cols = (int64_t)N * C_in;
    double* W = (double*)malloc(sizeof(double) * rows * cols);
    if (!W) return -1;
    eqref_cn_expand(N, C_in, C_out, w, W);
    eqref_apply_dense(T, rows, cols, W, x, y);
    free(W);
    return 0;
}

/* The same layer as a direct circular convolution along the group axis:
 * y[t][o][g] = sum_i sum_m w[o][i][m] * x[t][i][(g-m) mod N]. */
void eqref_cn_direct(int N, int C_in, int C_out, int64_t T, const double* x,
                     const double* w, double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int o = 0; o < C_out; ++o)
            for (int g = 0; g < N; ++g) {
                double acc = 0.0;
                for (int i = 0; i < C_in; ++i)
                    for (int m = 0; m < N; ++m) {
                        int h = ((g - m) % N + N) % N;
                        acc += w[((int64_t)o * C_in + i) * N + m] *
                               x[(t * C_in + i) * N + h];
                    }
                y[(t * C_out + o) * N + g] = acc;
            }
}

/* Input gradient, directly: dx[t][i][h] = sum_{o,g} w[o][i][(g-h) mod N] dy[t][o][g]. */
void eqref_cn_backward_data(int N, int C_in, int C_out, int64_t T, const double* dy,
                            const double* w, double* dx) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int i = 0; i < C_in; ++i)
            for (int h = 0; h < N; ++h) {
                double acc = 0.0;
                for (int o = 0; o < C_out; ++o)
                    for (int g = 0; g < N; ++g) {
                        int m = ((g - h) % N + N) % N;
                        acc += w[((int64_t)o * C_in + i) * N + m] *
                               dy[(t * C_out + o) * N + g];
                    }
                dx[(t * C_in + i) * N + h] = acc;
            }
}

/* Weight gradient: dw[o][i][m] = sum_{t,g} dy[t][o][g] x[t][i][(g-m) mod N]. */
void eqref_cn_backward_weight(int N, int C_in, int C_out, int64_t T, const double* x,
                              const double* dy, double* dw) {
#pragma omp parallel for schedule(static)
    for (int o = 0; o < C_out; ++o)
        for (int i = 0; i < C_in; ++i)
            for (int m = 0; m < N; ++m) {
                double acc = 0.0;
                for (int64_t t = 0; t < T; ++t)
                    for (int g = 0; g < N; ++g) {
                        int h = ((g - m) % N + N) % N;
                        acc += dy[(t * C_out + o) * N + g] * x[(t * C_in + i) * N + h];
                    }
                dw[((int64_t)o * C_in + i) * N + m] = acc;
            }
}

/* In place: y[t][o][g] = act(y[t][o][g] + bias[o]); bias may be NULL, act 0 =
 * identity, 1 = GELU (erf form, GELU(v) = v Phi(v), Phi(v) = erfc(-v/sqrt 2)/2). */
void eqref_bias_act(int64_t T, int C_out, int N, const double* bias, int act, double* y) {
    const double rsqrt2 = 1.0 / sqrt(2.0);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int o = 0; o < C_out; ++o)
            for (int g = 0; g < N; ++g) {
                double v = y[(t * C_out + o) * N + g];
                if (bias) v += bias[o];
                if (act == 1) v = 0.5 * v * erfc(-v * rsqrt2);
                y[(t * C_out + o) * N + g] = v;
            }
}

/* Real DFT of w along its last axis, packed into N planes [N][C_out][C_in]. */
void eqref_cn_weight_dft(int N, int C_out, int C_in, const double* w, double* planes) {
    const double two_pi = 2.0 * acos(-1.0);
    const int64_t plane = (int64_t)C_out * C_in;
    for (int64_t oi = 0; oi < plane; ++oi) {
        const double* wm = w + oi * N;
        for (int k = 0; k <= N / 2; ++k) {
            double re = 0.0, im = 0.0;
            for (int m = 0; m < N; ++m) {
                double ang = two_pi * (double)((m * k) % N) / (double)N;
                re += wm[m] * cos(ang);
                im -= wm[m] * sin(ang);
            }
            if (k == 0) {
                planes[oi] = re;
            } else if (2 * k == N) {
                planes[(int64_t)(N - 1) * plane + oi] = re;
            } else {
                planes[(int64_t)(2 * k - 1) * plane + oi] = re;
                planes[(int64_t)(2 * k) * plane + oi] = im;
            }
        }
    }
}

/* D8 block-diagonal matrix [C_out][C_in] from the packed blocks
 * wb = [W_A1 | W_A2 | W_B1 | W_B2 | W_E], each row-major [out][in];
 * 1-D blocks are (C_out/8 x C_in/8), W_E is (C_out/4 x C_in/4). */
void eqref_d8_expand(int C_in, int C_out, const double* wb, double* W) {
    const int mi = C_in / 8, mo = C_out / 8;
    memset(W, 0, sizeof(double) * (size_t)C_in * (size_t)C_out);
    const double* blk = wb;
    for (int b = 0; b < 4; ++b) { /* A1, A2, B1, B2 */
        for (int r = 0; r < mo; ++r)
            for (int c = 0; c < mi; ++c)
                W[(int64_t)(b * mo + r) * C_in + b * mi + c] = blk[(int64_t)r * mi + c];
        blk += (int64_t)mo * mi;
    }
    for (int e = 0; e < 2; ++e) /* W_E on E coordinate 0, then coordinate 1 */
        for (int r = 0; r < 2 * mo; ++r)
            for (int c = 0; c < 2 * mi; ++c)
                W[(int64_t)(4 * mo + 2 * e * mo + r) * C_in + 4 * mi + 2 * e * mi + c] =
                    blk[(int64_t)r * (2 * mi) + c];
}

/* The D8 group Fourier transform on one regular-representation channel.
 * D8 = <r, s | r^4 = s^2 = 1, s r s = r^-1>; element q = a + 4b (0 <= a < 4,
 * b in {0, 1}) is r^a s^b.  Its real irreps, with the generators the layer's
 * feature action uses: A1 (r, s) -> (1, 1), A2 (1, -1), B1 (-1, 1), B2 (-1, -1),
 * and E: r -> [[0, -1], [1, 0]], s -> diag(1, -1), so E(r^a s^b) = E(r)^a E(s)^b.
 * F[p][q] (8 x 8, row-major): rows 0..3 are the 1-D irreps' values at element q
 * times sqrt(1/8); row 4 + 2k + c is entry (k, c) of E(q) times sqrt(2/8).  By
 * Schur orthogonality the rows are orthonormal: F^-1 = F^T.  The coefficients of
 * a function f on the group are F f; under a left translation of f the 2 x 2
 * matrix of E coefficients is multiplied by E(g) on the left, so each of its
 * columns c is one copy of E (coordinates k = 0, 1). */
void eqref_d8_fourier_matrix(double* F) {
    const double Er[2][2] = {{0.0, -1.0}, {1.0, 0.0}}, Es[2][2] = {{1.0, 0.0}, {0.0, -1.0}};
    const double chi_r[4] = {1.0, 1.0, -1.0, -1.0}, chi_s[4] = {1.0, -1.0, 1.0, -1.0};
    const double n1 = sqrt(1.0 / 8.0), n2 = sqrt(2.0 / 8.0);
    for (int q = 0; q < 8; ++q) {
        const int a = q % 4, b = q / 4;
        double M[2][2] = {{1.0, 0.0}, {0.0, 1.0}};
        for (int i = 0; i < a; ++i) { /* M <- E(r) M */
            double T2[2][2];
            for (int k = 0; k < 2; ++k)
                for (int c = 0; c < 2; ++c) T2[k][c] = Er[k][0] * M[0][c] + Er[k][1] * M[1][c];
            memcpy(M, T2, sizeof M);
        }
        if (b) { /* M <- M E(s) */
            double T2[2][2];
            for (int k = 0; k < 2; ++k)
                for (int c = 0; c < 2; ++c) T2[k][c] = M[k][0] * Es[0][c] + M[k][1] * Es[1][c];
            memcpy(M, T2, sizeof M);
        }
        for (int p = 0; p < 4; ++p) {
            double v = 1.0;
            for (int i = 0; i < a; ++i) v *= chi_r[p];
            if (b) v *= chi_s[p];
            F[p * 8 + q] = n1 * v;
        }
        for (int k = 0; k < 2; ++k)
            for (int c = 0; c < 2; ++c) F[(4 + 2 * k + c) * 8 + q] = n2 * M[k][c];
    }
}

/* Fourier features of regular channel j (of m) in one token row of width 8m,
 * laid out [A1 | A2 | B1 | B2 | E coord 0 | E coord 1]: A1..B2 at j, the E
 * copies of channel j are 2j + c (column c of its E coefficient matrix), each
 * with coordinates k = 0, 1 in the two E slabs.  Index p as in F. */
static int64_t d8_slot(int m, int j, int p) {
    if (p < 4) return (int64_t)p * m + j;
    const int k = (p - 4) / 2, c = (p - 4) % 2;
    return 4 * (int64_t)m + 2 * (int64_t)m * k + 2 * j + c;
}

/* Fourier layout [T][8m] -> regular layout [T][m][8]: f = F^T v per channel. */
void eqref_d8_to_regular(int64_t T, int m, const double* v, double* f) {
    double F[64];
    eqref_d8_fourier_matrix(F);
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < m; ++j)
            for (int q = 0; q < 8; ++q) {
                double acc = 0.0;
                for (int p = 0; p < 8; ++p) acc += F[p * 8 + q] * v[t * 8 * m + d8_slot(m, j, p)];
                f[(t * m + j) * 8 + q] = acc;
            }
}

/* Regular layout [T][m][8] -> Fourier layout [T][8m]: v = F f per channel. */
void eqref_d8_to_fourier(int64_t T, int m, const double* f, double* v) {
    double F[64];
    eqref_d8_fourier_matrix(F);
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < m; ++j)
            for (int p = 0; p < 8; ++p) {
                double acc = 0.0;
                for (int q = 0; q < 8; ++q) acc += F[p * 8 + q] * f[(t * m + j) * 8 + q];
                v[t * 8 * m + d8_slot(m, j, p)] = acc;
            }
}

/* In place on D8 Fourier features y[T][8m]: the pointwise neighbours of the
 * layer applied where the group only permutes coordinates ("Quick ViTs", key
 * design 2: back to the regular representation, GELU, forward again).  Per
 * token and regular channel j: f = F^T v_j; f <- act(f + bias[j]) (bias may be
 * NULL: a constant over the group elements, act as eqref_bias_act); v_j = F f. */
void eqref_d8_bias_act(int64_t T, int m, const double* bias, int act, double* y) {
    double F[64];
    eqref_d8_fourier_matrix(F);
    const double rsqrt2 = 1.0 / sqrt(2.0);
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < m; ++j) {
            double v[8], f[8];
            for (int p = 0; p < 8; ++p) v[p] = y[t * 8 * m + d8_slot(m, j, p)];
            for (int q = 0; q < 8; ++q) {
                double acc = 0.0;
                for (int p = 0; p < 8; ++p) acc += F[p * 8 + q] * v[p];
                if (bias) acc += bias[j];
                if (act == 1) acc = 0.5 * acc * erfc(-acc * rsqrt2);
                f[q] = acc;
            }
            for (int p = 0; p < 8; ++p) {
                double acc = 0.0;
                for (int q = 0; q < 8; ++q) acc += F[p * 8 + q] * f[q];
                y[t * 8 * m + d8_slot(m, j, p)] = acc;
            }
        }
}

/* ---- dihedral groups D_n (order 2n) ---- */

/* Number of 1-D irreps (2 or 4) and of 2-D irreps of D_n. */
static int dn_one_dim(int n) { return n % 2 == 0 ? 4 : 2; }
static int dn_two_dim(int n) { return n % 2 == 0 ? n / 2 - 1 : (n - 1) / 2; }

/* Block-diagonal matrix [C_out][C_in] of the D_n layer from the packed blocks
 * wb = [W of each 1-D irrep (C_out/2n x C_in/2n) | W of each E_k (C_out/n x C_in/n)]. */
void eqref_dn_expand(int n, int C_in, int C_out, const double* wb, double* W) {
    const int mi = C_in / (2 * n), mo = C_out / (2 * n), n1 = dn_one_dim(n), n2 = dn_two_dim(n);
    memset(W, 0, sizeof(double) * (size_t)C_in * (size_t)C_out);
    const double* blk = wb;
    for (int b = 0; b < n1; ++b) {
        for (int r = 0; r < mo; ++r)
            for (int c = 0; c < mi; ++c)
                W[(int64_t)(b * mo + r) * C_in + b * mi + c] = blk[(int64_t)r * mi + c];
        blk += (int64_t)mo * mi;
    }
    for (int k = 0; k < n2; ++k) {
        for (int e = 0; e < 2; ++e) /* coordinate e of E_{k+1} */
            for (int r = 0; r < 2 * mo; ++r)
                for (int c = 0; c < 2 * mi; ++c)
                    W[(int64_t)(n1 * mo + 4 * k * mo + 2 * e * mo + r) * C_in + n1 * mi + 4 * k * mi + 2 * e * mi + c] =
                        blk[(int64_t)r * (2 * mi) + c];
        blk += (int64_t)(2 * mo) * (2 * mi);
    }
}

int eqref_dn_dense(int n, int C_in, int C_out, int64_t T, const double* x, const double* wb, double* y) {
    double* W = (double*)malloc(sizeof(double) * (size_t)C_in * (size_t)C_out);
    if (!W) return -1;
    eqref_dn_expand(n, C_in, C_out, wb, W);
    eqref_apply_dense(T, C_out, C_in, W, x, y);
    free(W);
    return 0;
}

/* Orthonormal Fourier matrix F[p][q] of D_n, 2n x 2n, element q = a + n b being
 * r^a s^b.  Rows: the 1-D irreps' values times sqrt(1/2n); then for each E_k
 * (k = 1, 2, ...) entry (kk, c) of E_k(q) times sqrt(2/2n), row index
 * n1 + 4(k-1) + 2 kk + c. */
void eqref_dn_fourier_matrix(int n, double* F) {
    const int n1 = dn_one_dim(n), n2 = dn_two_dim(n), G = 2 * n;
    const double chi_r[4] = {1.0, 1.0, -1.0, -1.0}, chi_s[4] = {1.0, -1.0, 1.0, -1.0};
    const double two_pi = 2.0 * acos(-1.0);
    for (int q = 0; q < G; ++q) {
        const int a = q % n, b = q / n;
        for (int p = 0; p < n1; ++p) {
            double v = 1.0;
            for (int i = 0; i < a; ++i) v *= chi_r[p];
            if (b) v *= chi_s[p];
            F[p * G + q] = sqrt(1.0 / G) * v;
        }
        for (int k = 1; k <= n2; ++k) {
            /* E_k(r)^a E_k(s)^b, E_k(r) = rotation by 2 pi k / n */
            const double c1 = cos(two_pi * k / n), s1 = sin(two_pi * k / n);
            double M[2][2] = {{1.0, 0.0}, {0.0, 1.0}};
            for (int i = 0; i < a; ++i) {
                double T2[2][2];
                for (int kk = 0; kk < 2; ++kk) {
                    T2[0][kk] = c1 * M[0][kk] - s1 * M[1][kk];
                    T2[1][kk] = s1 * M[0][kk] + c1 * M[1][kk];
                }
                memcpy(M, T2, sizeof M);
            }
            if (b) { /* right factor diag(1, -1): negate column 1 */
                M[0][1] = -M[0][1];
                M[1][1] = -M[1][1];
            }
            for (int kk = 0; kk < 2; ++kk)
                for (int c = 0; c < 2; ++c) F[(n1 + 4 * (k - 1) + 2 * kk + c) * G + q] = sqrt(2.0 / G) * M[kk][c];
        }
    }
}

/* Fourier-layout column of coefficient p of regular channel j (of m), D_n layout. */
static int64_t dn_slot(int n, int m, int j, int p) {
    const int n1 = dn_one_dim(n);
    if (p < n1) return (int64_t)p * m + j;
    const int e = p - n1, k = e / 4, kk = (e % 4) / 2, c = e % 2;
    return (int64_t)n1 * m + 4 * (int64_t)m * k + 2 * (int64_t)m * kk + 2 * j + c;
}

/* Fourier layout [T][2n m] -> regular layout [T][m][2n]: f = F^T v per channel. */
void eqref_dn_to_regular(int n, int64_t T, int m, const double* v, double* f) {
    const int G = 2 * n;
    double* F = (double*)malloc(sizeof(double) * G * G);
    if (!F) return;
    eqref_dn_fourier_matrix(n, F);
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < m; ++j)
            for (int q = 0; q < G; ++q) {
                double acc = 0.0;
                for (int p = 0; p < G; ++p) acc += F[p * G + q] * v[t * G * m + dn_slot(n, m, j, p)];
                f[(t * m + j) * G + q] = acc;
            }
    free(F);
}

/* Regular layout [T][m][2n] -> Fourier layout [T][2n m]: v = F f per channel. */
void eqref_dn_to_fourier(int n, int64_t T, int m, const double* f, double* v) {
    const int G = 2 * n;
    double* F = (double*)malloc(sizeof(double) * G * G);
    if (!F) return;
    eqref_dn_fourier_matrix(n, F);
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < m; ++j)
            for (int p = 0; p < G; ++p) {
                double acc = 0.0;
                for (int q = 0; q < G; ++q) acc += F[p * G + q] * f[(t * m + j) * G + q];
                v[t * G * m + dn_slot(n, m, j, p)] = acc;
            }
    free(F);
}

/* In place on D_n Fourier features y[T][2n m]: per token and regular channel j,
 * f = F^T v_j, f <- act(f + bias[j]), v_j = F f (as eqref_d8_bias_act). */
void eqref_dn_bias_act(int n, int64_t T, int m, const double* bias, int act, double* y) {
    const int G = 2 * n;
    double* F = (double*)malloc(sizeof(double) * G * G);
    double* v = (double*)malloc(sizeof(double) * G);
    double* f = (double*)malloc(sizeof(double) * G);
    if (!F || !v || !f) {
        free(F);
        free(v);
        free(f);
        return;
    }
    eqref_dn_fourier_matrix(n, F);
    const double rsqrt2 = 1.0 / sqrt(2.0);
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < m; ++j) {
            for (int p = 0; p < G; ++p) v[p] = y[t * G * m + dn_slot(n, m, j, p)];
            for (int q = 0; q < G; ++q) {
                double acc = 0.0;
                for (int p = 0; p < G; ++p) acc += F[p * G + q] * v[p];
                if (bias) acc += bias[j];
                if (act == 1) acc = 0.5 * acc * erfc(-acc * rsqrt2);
                f[q] = acc;
            }
            for (int p = 0; p < G; ++p) {
                double acc = 0.0;
                for (int q = 0; q < G; ++q) acc += F[p * G + q] * f[q];
                y[t * G * m + dn_slot(n, m, j, p)] = acc;
            }
        }
    free(F);
    free(v);
    free(f);
}

int eqref_d8_dense(int C_in, int C_out, int64_t T, const double* x, const double* wb,
                   double* y) {
    double* W = (double*)malloc(sizeof(double) * (size_t)C_in * (size_t)C_out);
    if (!W) return -1;
    eqref_d8_expand(C_in, C_out, wb, W);
    eqref_apply_dense(T, C_out, C_in, W, x, y);
    free(W);
    return 0;
}
