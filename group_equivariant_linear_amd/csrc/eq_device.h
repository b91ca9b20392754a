// eq_device.h -- device helpers shared by the gfx950 kernels of libeqlinear.
//
// Compile-time twiddles, bf16 conversion, MFMA fragment types and the
// XCD-aware workgroup remap.  Everything here is written for CDNA4 (gfx950):
// 64-lane wavefronts, 16x16 MFMA tiles, 8 XCDs with one L2 each.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace eql {

// Cache-policy bits of the stores that write a layer's output: y is written
// once and not read again by the kernel that writes it, so it carries the
// non-temporal hint (nt, bit 1 of the gfx950 cache policy).
#ifndef EQL_Y_STORE_AUX
#define EQL_Y_STORE_AUX 2
#endif
constexpr int kYStoreAux = EQL_Y_STORE_AUX;


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Compile-time trigonometry for the twiddle factors exp(-2 pi i j / n).
// The angle 2*pi*j/n is reduced to q*(pi/2) + phi with |phi| <= pi/4 and
// phi computed from the exact rational (8*j mod 8n)/n; the Taylor series of
// sin and cos are summed in double.  Multiples of a quarter turn are exact.

constexpr double kPi = 3.141592653589793238462643383279502884;

constexpr double taylor_sin(double x) {
    double x2 = x * x, term = x, sum = x;
    for (int n = 1; n <= 12; ++n) {
        term *= -x2 / ((2.0 * n) * (2.0 * n + 1.0));
        sum += term;
    }
    return sum;
}

constexpr double taylor_cos(double x) {
    double x2 = x * x, term = 1.0, sum = 1.0;
    for (int n = 1; n <= 12; ++n) {
        term *= -x2 / ((2.0 * n - 1.0) * (2.0 * n));
        sum += term;
    }
    return sum;
}

// Returns cos (want_sin == false) or sin of 2*pi*j/n.
constexpr double turn_trig(long j, long n, bool want_sin) {
    long jm = ((j % n) + n) % n;
    long num = 8 * jm;       // angle = (pi/4) * num / n
    long oct = num / n;      // 0..7
    long q = (oct + 1) / 2;  // nearest quarter turn, 0..4
    double phi = (kPi / 4.0) * (double)(num - 2 * q * n) / (double)n;
    double s = taylor_sin(phi), c = taylor_cos(phi);
    switch (q % 4) {
        case 0: return want_sin ? s : c;
        case 1: return want_sin ? c : -s;
        case 2: return want_sin ? -s : -c;
        default: return want_sin ? -c : s;
    }
}

// Known values, to within 2 units in the last place of a double.
static_assert(turn_trig(1, 8, false) - 0.70710678118654752440 < 2.3e-16 &&
                  turn_trig(1, 8, false) - 0.70710678118654752440 > -2.3e-16,
              "cos(pi/4)");
static_assert(turn_trig(1, 12, true) - 0.5 < 1.2e-16 && turn_trig(1, 12, true) - 0.5 > -1.2e-16,
              "sin(pi/6)");
static_assert(turn_trig(1, 6, true) - 0.86602540378443864676 < 2.3e-16 &&
                  turn_trig(1, 6, true) - 0.86602540378443864676 > -2.3e-16,
              "sin(pi/3)");
static_assert(turn_trig(1, 4, false) == 0.0 && turn_trig(1, 4, true) == 1.0, "quarter turn");
static_assert(turn_trig(3, 4, true) == -1.0 && turn_trig(2, 4, false) == -1.0, "half turns");

// Twiddle table of one group order, in fp32 (rounded once from double).
// cs[j] = scale*cos(2 pi j/N), sn[j] = scale*sin(2 pi j/N).
template <int N>
struct TwTable {
    float cs[N];
    float sn[N];
};

template <int N>
constexpr TwTable<N> make_tw(double scale) {
    TwTable<N> t{};
    for (int j = 0; j < N; ++j) {
        t.cs[j] = (float)(scale * turn_trig(j, N, false));
        t.sn[j] = (float)(scale * turn_trig(j, N, true));
    }
    return t;
}

template <int N>
struct Tw {
    static constexpr TwTable<N> fwd = make_tw<N>(1.0);        // forward DFT
    static constexpr TwTable<N> inv = make_tw<N>(2.0 / N);    // inverse, doubled bins
    static constexpr float inv_dc = (float)(1.0 / N);         // inverse, DC/Nyquist
};

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// acc + c*v with a compile-time coefficient: 0 drops the term, +-1 is an add.
template <typename C>
__device__ __forceinline__ float cmac(float acc, C, float v) {
    constexpr float c = C::value;
    if constexpr (c == 0.0f) return acc;
    else if constexpr (c == 1.0f) return acc + v;
    else if constexpr (c == -1.0f) return acc - v;
    else return __builtin_fmaf(c, v, acc);
}

template <typename T, T V>
struct fconst { static constexpr T value = V; };

// ---------------------------------------------------------------------------
// Real DFT along the group axis ("Flash EQ-Linear", Algorithmic Approach).
// Kept bins k = 0..floor(N/2), packed into N real planes:
//   P[0] = Re X[0]; P[2k-1] = Re X[k], P[2k] = Im X[k] (1 <= k < N/2);
//   P[N-1] = Re X[N/2] (even N),  X[k] = sum_h x[h] exp(-2 pi i h k / N).
// Symmetric form: with s_h = x_h + x_{N-h} and d_h = x_h - x_{N-h},
//   Re X[k] = x_0 + sum_h s_h cos(2 pi hk/N) (+ (-1)^k x_{N/2}),
//   Im X[k] = -sum_h d_h sin(2 pi hk/N).
// For N = 4 every coefficient is 0 or +-1: adds and subtracts only
// ("Flash EQ-Linear", Specialization for p4 Rotation Group).
template <int N>
__device__ __forceinline__ void rdft_forward(const float (&x)[N], float (&P)[N]) {
    constexpr int H = (N - 1) / 2;  // symmetric pairs == complex bins
    float s[H + 1], d[H + 1];
    static_for<1, H + 1>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        s[h] = x[h] + x[N - h];
        d[h] = x[h] - x[N - h];
    });
    float dc = x[0];
    static_for<1, H + 1>([&](auto hc) { dc += s[decltype(hc)::value]; });
    if constexpr (N % 2 == 0) dc += x[N / 2];
    P[0] = dc;
    static_for<1, H + 1>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        float re = x[0];
        static_for<1, H + 1>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            re = cmac(re, fconst<float, Tw<N>::fwd.cs[(h * k) % N]>{}, s[h]);
        });
        if constexpr (N % 2 == 0) {
            if constexpr (k % 2 == 0) re += x[N / 2];
            else re -= x[N / 2];
        }
        float im = -Tw<N>::fwd.sn[k % N] * d[1];
        static_for<2, H + 1>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            im = cmac(im, fconst<float, -Tw<N>::fwd.sn[(h * k) % N]>{}, d[h]);
        });
        P[2 * k - 1] = re;
        P[2 * k] = im;
    });
    if constexpr (N % 2 == 0 && N > 1) {
        float ny = x[0];
        static_for<1, H + 1>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            if constexpr (h % 2 == 0) ny += s[h];
            else ny -= s[h];
        });
        if constexpr ((N / 2) % 2 == 0) ny += x[N / 2];
        else ny -= x[N / 2];
        P[N - 1] = ny;
    }
}

// Inverse real DFT from the N packed planes, 1/N included:
//   y[g] = (1/N) (P0 + (-1)^g Pnyq) + (2/N) sum_k (Re_k cos(2 pi gk/N) - Im_k sin(2 pi gk/N)).
// Symmetric form: y[g] = E_g - O_g and y[N-g] = E_g + O_g.
template <int N>
__device__ __forceinline__ void rdft_inverse(const float (&P)[N], float (&y)[N]) {
    constexpr int H = (N - 1) / 2;
    constexpr float idc = Tw<N>::inv_dc;
    static_for<0, N / 2 + 1>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        float e = P[0] * idc;
        if constexpr (N % 2 == 0 && N > 1) {
            if constexpr (g % 2 == 0) e = __builtin_fmaf(idc, P[N - 1], e);
            else e = __builtin_fmaf(-idc, P[N - 1], e);
        }
        static_for<1, H + 1>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            e = cmac(e, fconst<float, Tw<N>::inv.cs[(g * k) % N]>{}, P[2 * k - 1]);
        });
        if constexpr (g == 0 || 2 * g == N) {
            y[g] = e;
        } else {
            float o = 0.0f;
            static_for<1, H + 1>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                o = cmac(o, fconst<float, Tw<N>::inv.sn[(g * k) % N]>{}, P[2 * k]);
            });
            y[g] = e - o;
            y[N - g] = e + o;
        }
    });
}

// Minimal-operation forms for the orders the workloads use most (same
// results as the generic forms up to fp32 rounding order).
//   N = 8: 20 adds/FMAs forward, 25 inverse (radix-2 split of the symmetric
//          form; c = cos(pi/4)).
//   N = 4: 6 adds forward, 7 inverse -- every coefficient is 0, +-1 or a power
//          of two ("Flash EQ-Linear", Specialization for p4 Rotation Group).
template <>
__device__ __forceinline__ void rdft_forward<8>(const float (&x)[8], float (&P)[8]) {
    constexpr float c = Tw<8>::fwd.cs[1];
    const float a0 = x[0] + x[4], a1 = x[0] - x[4];
    const float s1 = x[1] + x[7], d1 = x[1] - x[7];
    const float s2 = x[2] + x[6], d2 = x[2] - x[6];
    const float s3 = x[3] + x[5], d3 = x[3] - x[5];
    const float b0 = a0 + s2, c0 = s1 + s3, c1 = s1 - s3, e = d1 + d3;
    P[0] = b0 + c0;                          // Re X0
    P[7] = b0 - c0;                          // Re X4 (Nyquist)
    P[1] = __builtin_fmaf(c, c1, a1);        // Re X1
    P[5] = __builtin_fmaf(-c, c1, a1);       // Re X3
    P[2] = __builtin_fmaf(-c, e, -d2);       // Im X1
    P[6] = __builtin_fmaf(-c, e, d2);        // Im X3
    P[3] = a0 - s2;                          // Re X2
    P[4] = d3 - d1;                          // Im X2
}

template <>
__device__ __forceinline__ void rdft_inverse<8>(const float (&P)[8], float (&y)[8]) {
    constexpr float c = Tw<8>::fwd.cs[1];
    const float R1 = P[1], I1 = P[2], R2 = P[3], I2 = P[4], R3 = P[5], I3 = P[6];
    const float t = P[0] * 0.125f;
    const float u0 = __builtin_fmaf(P[7], 0.125f, t), u1 = __builtin_fmaf(P[7], -0.125f, t);
    const float p = R1 - R3, m = R1 + R3, n = I1 + I3, k2 = I1 - I3;
    y[0] = __builtin_fmaf(m + R2, 0.25f, u0);
    y[4] = __builtin_fmaf(R2 - m, 0.25f, u0);
    y[2] = __builtin_fmaf(R2 + k2, -0.25f, u0);
    y[6] = __builtin_fmaf(k2 - R2, 0.25f, u0);
    const float pm = p - n, pp = p + n;
    y[1] = __builtin_fmaf(__builtin_fmaf(c, pm, -I2), 0.25f, u1);
    y[7] = __builtin_fmaf(__builtin_fmaf(c, pp, I2), 0.25f, u1);
    y[3] = __builtin_fmaf(__builtin_fmaf(-c, pp, I2), 0.25f, u1);
    y[5] = __builtin_fmaf(__builtin_fmaf(-c, pm, -I2), 0.25f, u1);
}

template <>
__device__ __forceinline__ void rdft_forward<4>(const float (&x)[4], float (&P)[4]) {
    const float a0 = x[0] + x[2];
    const float s1 = x[1] + x[3];
    P[0] = a0 + s1;       // Re X0
    P[3] = a0 - s1;       // Re X2 (Nyquist)
    P[1] = x[0] - x[2];   // Re X1
    P[2] = x[3] - x[1];   // Im X1
}

template <>
__device__ __forceinline__ void rdft_inverse<4>(const float (&P)[4], float (&y)[4]) {
    const float t = P[0] * 0.25f;
    const float u0 = __builtin_fmaf(P[3], 0.25f, t), u1 = __builtin_fmaf(P[3], -0.25f, t);
    y[0] = __builtin_fmaf(P[1], 0.5f, u0);
    y[2] = __builtin_fmaf(P[1], -0.5f, u0);
    y[1] = __builtin_fmaf(P[2], -0.5f, u1);
    y[3] = __builtin_fmaf(P[2], 0.5f, u1);
}

// ---------------------------------------------------------------------------
// bf16 helpers.

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even fp32 -> bf16, two values packed in one dword
// (a single v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// fp16 (IEEE binary16) helpers.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even fp32 -> fp16 (overflow to infinity), two values packed
// in one dword.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// The two 16-bit storage types behind one interface: an 8-element MFMA
// fragment, packing two fp32 values (RNE) and reading either half of a dword.
template <typename IO>
struct Half;
template <>
struct Half<__bf16> {
    using x8 = bf16x8;
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
    static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
    static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
};
template <>
struct Half<_Float16> {
    using x8 = f16x8;
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) { return pack_f16x2(lo, hi); }
    static __device__ __forceinline__ float lo(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    }
    static __device__ __forceinline__ float hi(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
};

// fp16 spectra held in 16 bits (the VALU-transform kernels, the
// weight-gradient planes) are those of x/N (so that a bin never exceeds the largest |x|:
// fp16 keeps its range wherever x and y do); the accumulators then hold the
// spectrum of y/N, and the inverse transform first multiplies by N.  (Exact
// for N a power of two; one fp32 rounding otherwise.)  bf16 and fp32 have the
// range of fp32 and keep the unscaled spectra.
template <typename IO, int N>
constexpr float spec_scale = std::is_same_v<IO, _Float16> ? (float)(1.0 / N) : 1.0f;
template <typename IO, int N>
constexpr float spec_unscale = std::is_same_v<IO, _Float16> ? (float)N : 1.0f;

// ---------------------------------------------------------------------------
// Workgroup ids are handed to the 8 XCDs round-robin.  Remap them so that a
// run of consecutive logical tiles executes on one XCD and shares its L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t id, uint32_t total) {
    constexpr uint32_t kXcd = 8;
    uint32_t xcd = id % kXcd, local = id / kXcd;
    uint32_t q = total / kXcd, r = total % kXcd;
    // XCDs below r take q + 1 tiles, the others q (branch-free form)
    uint32_t base = xcd * q + (xcd < r ? xcd : r);
    return base + local;
}

}  // namespace eql
