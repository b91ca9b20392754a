// d8_round_trip.hip -- the D8 layer's regular-representation passes ("Quick
// ViTs", key design 2).  GELU does not commute with a general representation,
// so the MLP takes the layer's Fourier features back to the regular
// representation -- where the group only permutes the 8 values of a channel --
// applies GELU there and returns to the Fourier domain; the page fuses that
// round trip into one kernel.  This file does the same in one pass over y, and
// also runs either half alone (regular inputs into the Fourier layout, Fourier
// outputs back to the regular layout).
//
// Layouts: Fourier [T][8m] = [A1 | A2 | B1 | B2 | E coord 0 | E coord 1] with
// widths (m, m, m, m, 2m, 2m); regular [T][m][8], element q = a + 4b of the
// group being r^a s^b (r the quarter turn, s the mirror).  Regular channel j
// owns A1..B2 at j and the E copies 2j, 2j+1 (the two columns c of its E
// coefficient matrix M, coordinates k = 0, 1 its rows).  The transform is the
// group's orthonormal Fourier matrix: rows sqrt(1/8) chi(q) for the 1-D irreps
// and (1/2) E(q)[k][c] for E, E(r) = [[0,-1],[1,0]], E(s) = diag(1,-1); its
// entries are 0, +-1/2 and +-1/sqrt 8, so both directions are butterflies.
//
// One thread owns G consecutive regular channels of one token (G = 4 when m is
// a multiple of 4: 8- and 16-byte vector accesses for bf16, 16- and 32-byte
// for fp32; else, and for regular-layout outputs, G = 1), reads their
// features, transforms and writes them in one pass.  The identity passes run at about 1.5x the time of a device copy of
// the same bytes; the GELU round trip adds about 25 VALU operations per value
// (cn_fused.h: gelu_erf), which at one pass per element do not hide under the
// memory time.  (Tiles staged in LDS, with or without a register prefetch of
// the next tile, measured no faster.)
#include "cn_fused.h"
#include "dn_group.h"

namespace eql {

namespace {

// K consecutive elements <-> fp32, with vector accesses (K*sizeof(IO) is a
// multiple of 4 here except K = 1, 2 bf16, which take element accesses).
template <typename IO, int K>
__device__ __forceinline__ void load_k(const IO* p, float (&o)[K]) {
    if constexpr (sizeof(IO) == 4 && K % 4 == 0) {
#pragma unroll
        for (int i = 0; i < K / 4; ++i) {
            const u32x4 w = reinterpret_cast<const u32x4*>(p)[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[4 * i + e] = __uint_as_float(w[e]);
        }
    } else if constexpr (sizeof(IO) == 2 && K % 8 == 0) {
#pragma unroll
        for (int i = 0; i < K / 8; ++i) {
            const u32x4 w = reinterpret_cast<const u32x4*>(p)[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[8 * i + 2 * e] = Half<IO>::lo(w[e]);
                o[8 * i + 2 * e + 1] = Half<IO>::hi(w[e]);
            }
        }
    } else if constexpr (sizeof(IO) == 2 && K == 4) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(p);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            o[2 * e] = Half<IO>::lo(w[e]);
            o[2 * e + 1] = Half<IO>::hi(w[e]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < K; ++e) o[e] = (float)p[e];
    }
}

template <typename IO, int K>
__device__ __forceinline__ void store_k(IO* p, const float (&v)[K]) {
    if constexpr (sizeof(IO) == 4 && K % 4 == 0) {
#pragma unroll
        for (int i = 0; i < K / 4; ++i)
            reinterpret_cast<u32x4*>(p)[i] = u32x4{__float_as_uint(v[4 * i]), __float_as_uint(v[4 * i + 1]),
                                                   __float_as_uint(v[4 * i + 2]), __float_as_uint(v[4 * i + 3])};
    } else if constexpr (sizeof(IO) == 2 && K % 8 == 0) {
#pragma unroll
        for (int i = 0; i < K / 8; ++i)
            reinterpret_cast<u32x4*>(p)[i] =
                u32x4{Half<IO>::pack2(v[8 * i], v[8 * i + 1]), Half<IO>::pack2(v[8 * i + 2], v[8 * i + 3]),
                      Half<IO>::pack2(v[8 * i + 4], v[8 * i + 5]), Half<IO>::pack2(v[8 * i + 6], v[8 * i + 7])};
    } else if constexpr (sizeof(IO) == 2 && K == 4) {
        *reinterpret_cast<u32x2*>(p) = u32x2{Half<IO>::pack2(v[0], v[1]), Half<IO>::pack2(v[2], v[3])};
    } else {
#pragma unroll
        for (int e = 0; e < K; ++e) {
            if constexpr (sizeof(IO) == 4) p[e] = v[e];
            else reinterpret_cast<uint16_t*>(p)[e] = (uint16_t)(Half<IO>::pack2(v[e], 0.f) & 0xffffu);
        }
    }
}

enum D8Pass { kRoundTrip = 0, kToFourier = 1, kToRegular = 2 };

// MODE kRoundTrip: Fourier in, act(F^T v + b) back through F, Fourier out
// (in == out allowed: a thread reads every element it writes before writing).
// kToFourier: regular in, Fourier out.  kToRegular: Fourier in, regular out.
template <typename IO, int G, int MODE>
__global__ __launch_bounds__(256) void d8_pass_kernel(const IO* in, IO* out, const IO* bias, int act, int m,
                                                      uint32_t groups, uint32_t total) {
    const uint32_t idx = blockIdx.x * 256u + threadIdx.x;  // total < 2^31 (host-checked)
    if (idx >= total) return;
    const uint32_t t = idx / groups;
    const int j0 = (int)(idx - t * groups) * G;
    const int64_t row = (int64_t)t * 8 * (int64_t)m;  // first element of this token (either layout)

    float v[G][8];  // Fourier features of the G channels
    float f[G][8];  // their regular values
    if constexpr (MODE == kToFourier) {
        float r[8 * G];
        load_k<IO, 8 * G>(in + row + 8 * (int64_t)j0, r);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int q = 0; q < 8; ++q) f[g][q] = r[8 * g + q];
    } else {
        float a[4][G], e[2][2 * G];
#pragma unroll
        for (int p = 0; p < 4; ++p) load_k<IO, G>(in + row + (int64_t)p * m + j0, a[p]);
#pragma unroll
        for (int k = 0; k < 2; ++k) load_k<IO, 2 * G>(in + row + 4 * (int64_t)m + 2 * (int64_t)m * k + 2 * j0, e[k]);
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int p = 0; p < 4; ++p) v[g][p] = a[p][g];
            v[g][4] = e[0][2 * g];
            v[g][5] = e[0][2 * g + 1];
            v[g][6] = e[1][2 * g];
            v[g][7] = e[1][2 * g + 1];
            to_regular8(v[g], f[g]);
        }
    }

    if constexpr (MODE == kRoundTrip) {
        float b[G];
#pragma unroll
        for (int g = 0; g < G; ++g) b[g] = bias != nullptr ? (float)bias[j0 + g] : 0.0f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (act == 1) {
#pragma unroll
                for (int q = 0; q < 8; ++q) f[g][q] = gelu_erf(f[g][q] + b[g]);
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) f[g][q] += b[g];
            }
        }
    }

    if constexpr (MODE == kToRegular) {
        float r[8 * G];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int q = 0; q < 8; ++q) r[8 * g + q] = f[g][q];
        store_k<IO, 8 * G>(out + row + 8 * (int64_t)j0, r);
    } else {
        float a[4][G], e[2][2 * G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            to_fourier8(f[g], v[g]);
#pragma unroll
            for (int p = 0; p < 4; ++p) a[p][g] = v[g][p];
            e[0][2 * g] = v[g][4];
            e[0][2 * g + 1] = v[g][5];
            e[1][2 * g] = v[g][6];
            e[1][2 * g + 1] = v[g][7];
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) store_k<IO, G>(out + row + (int64_t)p * m + j0, a[p]);
#pragma unroll
        for (int k = 0; k < 2; ++k) store_k<IO, 2 * G>(out + row + 4 * (int64_t)m + 2 * (int64_t)m * k + 2 * j0, e[k]);
    }
}

template <typename IO, int MODE>
hipError_t launch_pass(const void* in, void* out, const void* bias, int act, int m, int64_t T, hipStream_t stream) {
    // regular-layout output: one channel per thread, so a wave's stores are
    // consecutive 8-value records (with four, they would stride 4 records)
    const int G = (MODE != kToRegular && m % 4 == 0) ? 4 : 1;
    const int64_t groups = m / G, total = T * groups;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;  // 32-bit thread indices
    const uint32_t blocks = (uint32_t)((total + 255) / 256);
    if (G == 4)
        hipLaunchKernelGGL((d8_pass_kernel<IO, 4, MODE>), dim3(blocks), dim3(256), 0, stream, (const IO*)in,
                           (IO*)out, (const IO*)bias, act, m, (uint32_t)groups, (uint32_t)total);
    else
        hipLaunchKernelGGL((d8_pass_kernel<IO, 1, MODE>), dim3(blocks), dim3(256), 0, stream, (const IO*)in,
                           (IO*)out, (const IO*)bias, act, m, (uint32_t)groups, (uint32_t)total);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_pass_dt(int io, const void* in, void* out, const void* bias, int act, int m, int64_t T,
                          hipStream_t stream) {
    if (io == kIoF16) return launch_pass<_Float16, MODE>(in, out, bias, act, m, T, stream);
    if (io == kIoBF16) return launch_pass<__bf16, MODE>(in, out, bias, act, m, T, stream);
    return launch_pass<float, MODE>(in, out, bias, act, m, T, stream);
}

// --- other dihedral orders ------------------------------------------------------------
// D_n of the regular n-gon (order G = 2n): 1-D irreps A1, A2 (and B1, B2 for even
// n), 2-D irreps E_k turning by 2 pi k / n, the layer's layout generalised (1-D
// slabs of m channels, then per E_k a coordinate-0 and a coordinate-1 slab of 2m
// copies; regular channel j owns column j of each 1-D slab and copies 2j, 2j+1).
// The Fourier matrix is a compile-time table (exact twiddles), so each channel's
// transforms are unrolled multiply-adds with the zero entries gone; one thread
// per channel.
template <typename IO, int n, int MODE>
__global__ __launch_bounds__(256) void dn_pass_kernel(const IO* in, IO* out, const IO* bias, int act, int m,
                                                      uint32_t total) {
    using D = DnGroup<n>;
    constexpr int G = D::G;
    const uint32_t idx = blockIdx.x * 256u + threadIdx.x;  // total < 2^31 (host-checked)
    if (idx >= total) return;
    const uint32_t t = idx / (uint32_t)m;
    const int j = (int)(idx - t * (uint32_t)m);
    const int64_t row = (int64_t)t * G * m;
    float v[G], f[G];
    if constexpr (MODE == kToFourier) {
#pragma unroll
        for (int q = 0; q < G; ++q) f[q] = (float)in[row + (int64_t)G * j + q];
    } else {
#pragma unroll
        for (int p = 0; p < G; ++p) v[p] = (float)in[row + D::slot(m, j, p)];
        static_for<0, G>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            float acc = 0.0f;
            static_for<0, G>([&](auto pc) {
                constexpr int p = decltype(pc)::value;
                constexpr float c = (float)D::entry(p, q);
                if constexpr (c != 0.0f) acc = fmaf(c, v[p], acc);
            });
            f[q] = acc;
        });
    }
    if constexpr (MODE == kRoundTrip) {
        const float b = bias != nullptr ? (float)bias[j] : 0.0f;
        if (act == 1) {
#pragma unroll
            for (int q = 0; q < G; ++q) f[q] = gelu_erf(f[q] + b);
        } else {
#pragma unroll
            for (int q = 0; q < G; ++q) f[q] += b;
        }
    }
    if constexpr (MODE == kToRegular) {
#pragma unroll
        for (int q = 0; q < G; ++q) out[row + (int64_t)G * j + q] = (IO)f[q];
    } else {
        static_for<0, G>([&](auto pc) {
            constexpr int p = decltype(pc)::value;
            float acc = 0.0f;
            static_for<0, G>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                constexpr float c = (float)D::entry(p, q);
                if constexpr (c != 0.0f) acc = fmaf(c, f[q], acc);
            });
            out[row + D::slot(m, j, p)] = (IO)acc;
        });
    }
}

template <typename IO, int MODE>
hipError_t launch_dn_pass(int n, const void* in, void* out, const void* bias, int act, int m, int64_t T,
                          hipStream_t stream) {
    const int64_t total = T * m;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    const uint32_t blocks = (uint32_t)((total + 255) / 256);
    switch (n) {
#define EQL_DN(k)                                                                                       \
    case k:                                                                                             \
        hipLaunchKernelGGL((dn_pass_kernel<IO, k, MODE>), dim3(blocks), dim3(256), 0, stream, (const IO*)in, \
                           (IO*)out, (const IO*)bias, act, m, (uint32_t)total);                         \
        return hipGetLastError();
        EQL_DN(2) EQL_DN(3) EQL_DN(5) EQL_DN(6) EQL_DN(7) EQL_DN(8) EQL_DN(9) EQL_DN(10) EQL_DN(11) EQL_DN(12)
#undef EQL_DN
        default: return hipErrorInvalidValue;
    }
}

// n == 4 (D8) takes the butterfly kernel above; other orders the table kernel
template <int MODE>
hipError_t launch_dihedral_pass(int n, int io, const void* in, void* out, const void* bias, int act, int m,
                                int64_t T, hipStream_t stream) {
    if (n == 4) return launch_pass_dt<MODE>(io, in, out, bias, act, m, T, stream);
    if (io == kIoF16) return launch_dn_pass<_Float16, MODE>(n, in, out, bias, act, m, T, stream);
    if (io == kIoBF16) return launch_dn_pass<__bf16, MODE>(n, in, out, bias, act, m, T, stream);
    return launch_dn_pass<float, MODE>(n, in, out, bias, act, m, T, stream);
}

}  // namespace

hipError_t launch_dn_round_trip(int n, int io, const void* y_in, void* y_out, const void* bias, int act,
                                int m, int64_t T, hipStream_t stream) {
    return launch_dihedral_pass<kRoundTrip>(n, io, y_in, y_out, bias, act, m, T, stream);
}

hipError_t launch_dn_to_fourier(int n, int io, const void* x_reg, void* x_four, int m, int64_t T,
                                hipStream_t stream) {
    return launch_dihedral_pass<kToFourier>(n, io, x_reg, x_four, nullptr, 0, m, T, stream);
}

hipError_t launch_dn_to_regular(int n, int io, const void* y_four, void* y_reg, int m, int64_t T,
                                hipStream_t stream) {
    return launch_dihedral_pass<kToRegular>(n, io, y_four, y_reg, nullptr, 0, m, T, stream);
}

hipError_t launch_d8_round_trip(int io, const void* y_in, void* y_out, const void* bias, int act, int m,
                                int64_t T, hipStream_t stream) {
    return launch_pass_dt<kRoundTrip>(io, y_in, y_out, bias, act, m, T, stream);
}

hipError_t launch_d8_to_fourier(int io, const void* x_reg, void* x_four, int m, int64_t T,
                                hipStream_t stream) {
    return launch_pass_dt<kToFourier>(io, x_reg, x_four, nullptr, 0, m, T, stream);
}

hipError_t launch_d8_to_regular(int io, const void* y_four, void* y_reg, int m, int64_t T,
                                hipStream_t stream) {
    return launch_pass_dt<kToRegular>(io, y_four, y_reg, nullptr, 0, m, T, stream);
}

}  // namespace eql
