// dn_group.h -- the dihedral groups' Fourier transforms, shared by the passes
// (d8_round_trip.hip) and the fused regular-feature layer (dn_regular.hip).
//
// D_n is the symmetry group of the regular n-gon, order G = 2n; element
// q = a + n b is r^a s^b (r the turn by 2 pi / n, s the mirror).  Its real
// irreps: 1-D ones A1, A2 (and B1, B2 for even n) and 2-D ones E_k turning by
// 2 pi k / n ("Quick ViTs", key design 2, works out n = 4).  A regular channel
// holds G values; its Fourier features are the 1-D irreps' coefficients and,
// per E_k, the 2 x 2 coefficient matrix M[kk][c] (rows kk the coordinates,
// columns c the copies).  The transform is the orthonormal Fourier matrix F:
// rows sqrt(1/G) chi(q) for the 1-D irreps and sqrt(2/G) E_k(q)[kk][c] for the
// 2-D ones, so regular and Fourier features have the same scale.
#pragma once

#include "eq_device.h"

namespace eql {

constexpr float kC8 = 0.35355339059327376f;  // 1/sqrt(8)

// f = F^T v: the 8 regular values of one channel from its Fourier features
// v = (a1, a2, b1, b2, M00, M01, M10, M11).
__device__ __forceinline__ void to_regular8(const float (&v)[8], float (&f)[8]) {
    const float s1 = (v[0] + v[1]) * kC8, s2 = (v[0] - v[1]) * kC8;  // a1 +- a2
    const float d1 = (v[2] + v[3]) * kC8, d2 = (v[2] - v[3]) * kC8;  // b1 +- b2
    const float p = 0.5f * (v[4] + v[7]), pm = 0.5f * (v[4] - v[7]);  // M00 +- M11
    const float n = 0.5f * (v[6] - v[5]), np = 0.5f * (v[5] + v[6]);  // M10 -+ M01
    const float u0 = s1 + d1, u1 = s1 - d1, u4 = s2 + d2, u5 = s2 - d2;
    f[0] = u0 + p;
    f[2] = u0 - p;
    f[1] = u1 + n;
    f[3] = u1 - n;
    f[4] = u4 + pm;
    f[6] = u4 - pm;
    f[5] = u5 + np;
    f[7] = u5 - np;
}

// v = F f: the Fourier features of one channel from its 8 regular values.
__device__ __forceinline__ void to_fourier8(const float (&f)[8], float (&v)[8]) {
    const float e0 = f[0] + f[2], o0 = f[0] - f[2], e1 = f[1] + f[3], o1 = f[1] - f[3];
    const float e4 = f[4] + f[6], o4 = f[4] - f[6], e5 = f[5] + f[7], o5 = f[5] - f[7];
    const float g0 = e0 + e1, g1 = e0 - e1, g4 = e4 + e5, g5 = e4 - e5;
    v[0] = (g0 + g4) * kC8;   // A1
    v[1] = (g0 - g4) * kC8;   // A2
    v[2] = (g1 + g5) * kC8;   // B1
    v[3] = (g1 - g5) * kC8;   // B2
    v[4] = 0.5f * (o0 + o4);  // M00
    v[5] = 0.5f * (o5 - o1);  // M01
    v[6] = 0.5f * (o1 + o5);  // M10
    v[7] = 0.5f * (o0 - o4);  // M11
}

// --- other dihedral orders ------------------------------------------------------------
// The Fourier matrix of D_n as a compile-time table (exact twiddles): each
// channel's transforms become unrolled multiply-adds with the zero entries gone.
// Feature order p: the N1 1-D irreps, then for each E_k the entries
// (kk, c) = (0,0), (0,1), (1,0), (1,1).
constexpr double csqrt(double x) {
    double r = x > 1.0 ? x : 1.0;
    for (int i = 0; i < 60; ++i) r = 0.5 * (r + x / r);
    return r;
}

template <int n>
struct DnGroup {
    static constexpr int G = 2 * n;
    static constexpr int N1 = n % 2 == 0 ? 4 : 2;
    static constexpr int N2 = n % 2 == 0 ? n / 2 - 1 : (n - 1) / 2;
    // F[p][q], element q = a + n b = r^a s^b
    static constexpr double entry(int p, int q) {
        const int a = q % n, b = q / n;
        if (p < N1) {
            const double cr = (p >= 2) ? -1.0 : 1.0, cs = (p % 2) ? -1.0 : 1.0;
            double v = 1.0;
            for (int i = 0; i < a; ++i) v *= cr;
            if (b) v *= cs;
            return v / csqrt((double)G);
        }
        const int e = p - N1, k = e / 4 + 1, kk = (e % 4) / 2, c = e % 2;
        const double co = turn_trig((long)k * a, n, false), si = turn_trig((long)k * a, n, true);
        // E_k(r^a) = rotation by 2 pi k a / n; E_k(s) = diag(1, -1) negates column 1
        const double m = c == 0 ? (kk == 0 ? co : si) : (kk == 0 ? -si : co) * (b ? -1.0 : 1.0);
        return m * csqrt(2.0 / (double)G);
    }
    static constexpr int64_t slot(int m, int j, int p) {  // Fourier column of (channel j, coefficient p)
        if (p < N1) return (int64_t)p * m + j;
        const int e = p - N1, k = e / 4, kk = (e % 4) / 2, c = e % 2;
        return (int64_t)N1 * m + 4 * (int64_t)m * k + 2 * (int64_t)m * kk + 2 * j + c;
    }
};

}  // namespace eql
