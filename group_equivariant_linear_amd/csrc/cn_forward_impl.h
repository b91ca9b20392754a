// cn_forward_impl.h -- fused C_N equivariant linear forward for gfx950.
//
// One kernel does the whole layer ("Flash EQ-Linear", Algorithmic Approach and
// Implementation: DFT along the group axis, per-frequency channel products over
// the non-redundant half of the spectrum, inverse DFT, no intermediate global
// writes):
//
//   for each (token tile, output-channel tile) workgroup:
//     for each chunk of KC input channels:
//       load x[t0:t0+TT][i0:i0+KC][0:N] from HBM (16-byte vector loads, the
//         next chunk is in flight while the current one is multiplied),
//       real DFT of every (token, channel) record in VGPRs -> N planes,
//       planes -> LDS (bf16 RNE for bf16 plans), w_hat chunk -> LDS,
//       per plane: MFMA 16x16 products, fp32 accumulators for all N planes:
//         DC, Nyquist:   Y += X * W^T                         (real)
//         bin k:         Yr += Xr Wr^T - Xi Wi^T, Yi += Xr Wi^T + Xi Wr^T
//                        (the complex product as a real 2x2 block product)
//     inverse real DFT of the N accumulator planes in each lane, y written once.
//
// The accumulator of output (t, o) for every plane lives in the same lane, so
// the inverse transform needs no data exchange.
#pragma once

#include "eq_device.h"
#include "eq_launch.h"

namespace eql {

template <typename IO>
struct IoTraits;
template <>
struct IoTraits<float> {
    static constexpr int KC = 16;  // channels per chunk: 4 MFMA 16x16x4 steps
    static constexpr int R = 4;    // channels per load group (16 B of fp32 planes)
};
template <>
struct IoTraits<__bf16> {
    static constexpr int KC = 32;  // one MFMA 16x16x32 step
    static constexpr int R = 8;    // 16 B of bf16 planes
};

template <int N_, typename IO_, int WT_, int WC_, int TPW_, int CPW_>
struct CnCfg {
    static constexpr int N = N_;
    using IO = IO_;
    static constexpr int WT = WT_, WC = WC_, TPW = TPW_, CPW = CPW_;
    static constexpr int kThreads = 64 * WT * WC;
    static constexpr int TT = WT * TPW * 16;  // tokens per tile
    static constexpr int CT = WC * CPW * 16;  // output channels per tile
    static constexpr int KC = IoTraits<IO>::KC;
    static constexpr int R = IoTraits<IO>::R;
    static constexpr int S = (int)sizeof(IO);
    static constexpr int PITCH = KC + 16 / S;  // LDS row pitch (elements): 80 bytes
    static constexpr int A_ELEMS = N * TT * PITCH;
    static constexpr int B_ELEMS = N * CT * PITCH;
    static constexpr int XGROUPS = TT * (KC / R);  // (token, R-channel group) per chunk
    static constexpr int XG = (XGROUPS + kThreads - 1) / kThreads;
    static constexpr int WVECS = N * CT * (KC / R);  // 16-byte w_hat vectors per chunk
    static constexpr int WV = (WVECS + kThreads - 1) / kThreads;
    static constexpr int XW = 4 * N;  // dwords of one load group (R*N elements = 16N bytes)
};

// --- element access inside a dword array -----------------------------------

template <typename IO>
__device__ __forceinline__ float get_elem(const uint32_t* w, int e);
template <>
__device__ __forceinline__ float get_elem<float>(const uint32_t* w, int e) {
    return __uint_as_float(w[e]);
}
template <>
__device__ __forceinline__ float get_elem<__bf16>(const uint32_t* w, int e) {
    uint32_t d = w[e >> 1];
    return (e & 1) ? __uint_as_float(d & 0xffff0000u) : __uint_as_float(d << 16);
}

template <typename IO>
__device__ __forceinline__ uint32_t load_bits(const IO* p);
template <>
__device__ __forceinline__ uint32_t load_bits<float>(const float* p) {
    return __float_as_uint(*p);
}
template <>
__device__ __forceinline__ uint32_t load_bits<__bf16>(const __bf16* p) {
    return (uint32_t)*reinterpret_cast<const uint16_t*>(p);
}

template <typename IO>
__device__ __forceinline__ void set_elem(uint32_t* w, int e, uint32_t bits);
template <>
__device__ __forceinline__ void set_elem<float>(uint32_t* w, int e, uint32_t bits) {
    w[e] = bits;
}
template <>
__device__ __forceinline__ void set_elem<__bf16>(uint32_t* w, int e, uint32_t bits) {
    if (e & 1) w[e >> 1] = (w[e >> 1] & 0x0000ffffu) | (bits << 16);
    else w[e >> 1] = (w[e >> 1] & 0xffff0000u) | bits;
}

// --- global -> registers ----------------------------------------------------

// x records of one load group: R consecutive channels of one token, N elements each.
template <class C>
__device__ __forceinline__ void load_x_chunk(const typename C::IO* __restrict__ x, int64_t T,
                                             int C_in, int64_t t0, int i0, bool vec_ok,
                                             uint32_t (&xr)[C::XG][C::XW]) {
    using IO = typename C::IO;
#pragma unroll
    for (int g = 0; g < C::XG; ++g) {
        const int gi = (int)threadIdx.x + g * C::kThreads;
        if (C::XGROUPS % C::kThreads != 0 && gi >= C::XGROUPS) continue;
        const int ts = gi / (C::KC / C::R), q = gi % (C::KC / C::R);
        const int64_t t = t0 + ts;
        const int c0 = i0 + q * C::R;
        const IO* src = x + (t * C_in + c0) * C::N;
        if (vec_ok && t < T && c0 + C::R <= C_in) {
            const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
#pragma unroll
            for (int j = 0; j < C::N; ++j) {
                u32x4 v = __builtin_nontemporal_load(s4 + j);
                xr[g][4 * j + 0] = v.x;
                xr[g][4 * j + 1] = v.y;
                xr[g][4 * j + 2] = v.z;
                xr[g][4 * j + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < C::XW; ++j) xr[g][j] = 0u;
            if (t < T) {
#pragma unroll
                for (int e = 0; e < C::R * C::N; ++e) {
                    if (c0 + e / C::N < C_in) set_elem<IO>(xr[g], e, load_bits<IO>(src + e));
                }
            }
        }
    }
}

// One chunk of w_hat: planes [N][CT rows][KC channels] as 16-byte vectors.
template <class C>
__device__ __forceinline__ void load_w_chunk(const typename C::IO* __restrict__ w_hat, int C_in,
                                             int C_out, int o0, int i0, bool wvec_ok,
                                             uint32_t (&wr)[C::WV][4]) {
    using IO = typename C::IO;
    constexpr int PARTS = C::KC / C::R;
#pragma unroll
    for (int v = 0; v < C::WV; ++v) {
        const int vi = (int)threadIdx.x + v * C::kThreads;
        if (C::WVECS % C::kThreads != 0 && vi >= C::WVECS) continue;
        const int p = vi / (C::CT * PARTS);
        const int row = (vi / PARTS) % C::CT;
        const int part = vi % PARTS;
        const int o = o0 + row, ch = i0 + part * C::R;
        const IO* src = w_hat + ((int64_t)p * C_out + o) * C_in + ch;
        if (wvec_ok && o < C_out && ch + C::R <= C_in) {
            uint4 u = *reinterpret_cast<const uint4*>(src);
            wr[v][0] = u.x;
            wr[v][1] = u.y;
            wr[v][2] = u.z;
            wr[v][3] = u.w;
        } else {
            wr[v][0] = wr[v][1] = wr[v][2] = wr[v][3] = 0u;
            if (o < C_out) {
#pragma unroll
                for (int e = 0; e < C::R; ++e)
                    if (ch + e < C_in) set_elem<IO>(wr[v], e, load_bits<IO>(src + e));
            }
        }
    }
}

// --- registers -> LDS ---------------------------------------------------------

template <class C>
__device__ __forceinline__ void store_x_planes(const uint32_t (&xr)[C::XG][C::XW],
                                               typename C::IO* sA) {
    using IO = typename C::IO;
    constexpr int N = C::N;
#pragma unroll
    for (int g = 0; g < C::XG; ++g) {
        const int gi = (int)threadIdx.x + g * C::kThreads;
        if (C::XGROUPS % C::kThreads != 0 && gi >= C::XGROUPS) continue;
        const int ts = gi / (C::KC / C::R), q = gi % (C::KC / C::R);
        uint32_t pk[N][4];
        if constexpr (std::is_same<IO, float>::value) {
#pragma unroll
            for (int r = 0; r < C::R; ++r) {
                float xv[N], P[N];
#pragma unroll
                for (int h = 0; h < N; ++h) xv[h] = get_elem<IO>(xr[g], r * N + h);
                rdft_forward<N>(xv, P);
#pragma unroll
                for (int p = 0; p < N; ++p) pk[p][r] = __float_as_uint(P[p]);
            }
        } else {
#pragma unroll
            for (int r = 0; r < C::R; r += 2) {
                float xa[N], xb[N], Pa[N], Pb[N];
#pragma unroll
                for (int h = 0; h < N; ++h) {
                    xa[h] = get_elem<IO>(xr[g], r * N + h);
                    xb[h] = get_elem<IO>(xr[g], (r + 1) * N + h);
                }
                rdft_forward<N>(xa, Pa);
                rdft_forward<N>(xb, Pb);
#pragma unroll
                for (int p = 0; p < N; ++p) pk[p][r / 2] = pack_bf16x2(Pa[p], Pb[p]);
            }
        }
#pragma unroll
        for (int p = 0; p < N; ++p) {
            uint4 v = {pk[p][0], pk[p][1], pk[p][2], pk[p][3]};
            *reinterpret_cast<uint4*>(sA + (p * C::TT + ts) * C::PITCH + q * C::R) = v;
        }
    }
}

template <class C>
__device__ __forceinline__ void store_w_planes(const uint32_t (&wr)[C::WV][4],
                                               typename C::IO* sB) {
    constexpr int PARTS = C::KC / C::R;
#pragma unroll
    for (int v = 0; v < C::WV; ++v) {
        const int vi = (int)threadIdx.x + v * C::kThreads;
        if (C::WVECS % C::kThreads != 0 && vi >= C::WVECS) continue;
        const int p = vi / (C::CT * PARTS);
        const int row = (vi / PARTS) % C::CT;
        const int part = vi % PARTS;
        uint4 u = {wr[v][0], wr[v][1], wr[v][2], wr[v][3]};
        *reinterpret_cast<uint4*>(sB + (p * C::CT + row) * C::PITCH + part * C::R) = u;
    }
}

// --- MFMA ---------------------------------------------------------------------

// A fragment: 16 rows x KC, this lane's row = lane%16 and 16 bytes of k.
template <typename IO>
struct Frag;
template <>
struct Frag<__bf16> {
    using T = bf16x8;
};
template <>
struct Frag<float> {
    using T = f32x4;
};

__device__ __forceinline__ void mma(f32x4& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const f32x4& a, const f32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 neg(const bf16x8& v) {
    uint4 u = __builtin_bit_cast(uint4, v);
    u.x ^= 0x80008000u;
    u.y ^= 0x80008000u;
    u.z ^= 0x80008000u;
    u.w ^= 0x80008000u;
    return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ f32x4 neg(const f32x4& v) { return -v; }

template <class C>
__device__ __forceinline__ void chunk_products(const typename C::IO* sA,
                                               const typename C::IO* sB,
                                               f32x4 (&acc)[C::N][C::TPW][C::CPW]) {
    using IO = typename C::IO;
    using F = typename Frag<IO>::T;
    constexpr int N = C::N;
    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
    const int wt = wave / C::WC, wc = wave % C::WC;
    const int kofs = (lane >> 4) * (C::KC / 4);
    const IO* a_base = sA + (wt * C::TPW * 16 + (lane & 15)) * C::PITCH + kofs;
    const IO* b_base = sB + (wc * C::CPW * 16 + (lane & 15)) * C::PITCH + kofs;
    auto ldA = [&](int p, int a) {
        return *reinterpret_cast<const F*>(a_base + (p * C::TT + a * 16) * C::PITCH);
    };
    auto ldB = [&](int p, int b) {
        return *reinterpret_cast<const F*>(b_base + (p * C::CT + b * 16) * C::PITCH);
    };
    // DC bin: real product
    {
        F A[C::TPW], B[C::CPW];
#pragma unroll
        for (int a = 0; a < C::TPW; ++a) A[a] = ldA(0, a);
#pragma unroll
        for (int b = 0; b < C::CPW; ++b) B[b] = ldB(0, b);
#pragma unroll
        for (int a = 0; a < C::TPW; ++a)
#pragma unroll
            for (int b = 0; b < C::CPW; ++b) mma(acc[0][a][b], A[a], B[b]);
    }
    // complex bins: real 2x2 block product
#pragma unroll
    for (int k = 1; k <= (N - 1) / 2; ++k) {
        const int pr = 2 * k - 1, pi = 2 * k;
        F Ar[C::TPW], Ai[C::TPW], Br[C::CPW], Bi[C::CPW], nBi[C::CPW];
#pragma unroll
        for (int a = 0; a < C::TPW; ++a) {
            Ar[a] = ldA(pr, a);
            Ai[a] = ldA(pi, a);
        }
#pragma unroll
        for (int b = 0; b < C::CPW; ++b) {
            Br[b] = ldB(pr, b);
            Bi[b] = ldB(pi, b);
            nBi[b] = neg(Bi[b]);
        }
#pragma unroll
        for (int a = 0; a < C::TPW; ++a)
#pragma unroll
            for (int b = 0; b < C::CPW; ++b) {
                mma(acc[pr][a][b], Ar[a], Br[b]);
                mma(acc[pr][a][b], Ai[a], nBi[b]);
                mma(acc[pi][a][b], Ar[a], Bi[b]);
                mma(acc[pi][a][b], Ai[a], Br[b]);
            }
    }
    // Nyquist bin (even N): real product
    if constexpr (N % 2 == 0 && N > 1) {
        F A[C::TPW], B[C::CPW];
#pragma unroll
        for (int a = 0; a < C::TPW; ++a) A[a] = ldA(N - 1, a);
#pragma unroll
        for (int b = 0; b < C::CPW; ++b) B[b] = ldB(N - 1, b);
#pragma unroll
        for (int a = 0; a < C::TPW; ++a)
#pragma unroll
            for (int b = 0; b < C::CPW; ++b) mma(acc[N - 1][a][b], A[a], B[b]);
    }
}

// --- epilogue: inverse DFT and the single write of y ------------------------------

template <class C>
__device__ __forceinline__ void store_y(const f32x4 (&acc)[C::N][C::TPW][C::CPW],
                                        typename C::IO* __restrict__ y, int64_t T, int C_out,
                                        int64_t t0, int o0) {
    using IO = typename C::IO;
    constexpr int N = C::N;
    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
    const int wt = wave / C::WC, wc = wave % C::WC;
#pragma unroll
    for (int a = 0; a < C::TPW; ++a)
#pragma unroll
        for (int b = 0; b < C::CPW; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t t = t0 + wt * C::TPW * 16 + a * 16 + (lane >> 4) * 4 + r;
                const int o = o0 + wc * C::CPW * 16 + b * 16 + (lane & 15);
                float P[N], yv[N];
#pragma unroll
                for (int p = 0; p < N; ++p) P[p] = acc[p][a][b][r];
                rdft_inverse<N>(P, yv);
                if (t >= T || o >= C_out) continue;
                IO* dst = y + (t * C_out + o) * N;
                if constexpr (std::is_same<IO, float>::value) {
                    if constexpr (N % 4 == 0) {
#pragma unroll
                        for (int j = 0; j < N / 4; ++j) {
                            f32x4 v = {yv[4 * j], yv[4 * j + 1], yv[4 * j + 2], yv[4 * j + 3]};
                            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst) + j);
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < N; ++j) dst[j] = yv[j];
                    }
                } else {
                    if constexpr (N % 8 == 0) {
#pragma unroll
                        for (int j = 0; j < N / 8; ++j) {
                            u32x4 v = {pack_bf16x2(yv[8 * j], yv[8 * j + 1]),
                                       pack_bf16x2(yv[8 * j + 2], yv[8 * j + 3]),
                                       pack_bf16x2(yv[8 * j + 4], yv[8 * j + 5]),
                                       pack_bf16x2(yv[8 * j + 6], yv[8 * j + 7])};
                            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst) + j);
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < N; ++j) dst[j] = (__bf16)yv[j];
                    }
                }
            }
}

template <class C>
__global__ __launch_bounds__(C::kThreads) void cn_forward_kernel(
    const typename C::IO* __restrict__ x, const typename C::IO* __restrict__ w_hat,
    typename C::IO* __restrict__ y, int64_t T, int C_in, int C_out, int n_c_tiles,
    uint32_t total_tiles, int vec_ok, int wvec_ok) {
    using IO = typename C::IO;
    __shared__ __attribute__((aligned(16))) IO smem[C::A_ELEMS + C::B_ELEMS];
    IO* sA = smem;
    IO* sB = smem + C::A_ELEMS;

    const uint32_t tile = xcd_remap(blockIdx.x, total_tiles);
    const int64_t t0 = (int64_t)(tile / n_c_tiles) * C::TT;
    const int o0 = (int)(tile % n_c_tiles) * C::CT;

    f32x4 acc[C::N][C::TPW][C::CPW];
#pragma unroll
    for (int p = 0; p < C::N; ++p)
#pragma unroll
        for (int a = 0; a < C::TPW; ++a)
#pragma unroll
            for (int b = 0; b < C::CPW; ++b) acc[p][a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint32_t xr[C::XG][C::XW];
    uint32_t wr[C::WV][4];
    const int nchunks = (C_in + C::KC - 1) / C::KC;
    load_x_chunk<C>(x, T, C_in, t0, 0, vec_ok != 0, xr);
    load_w_chunk<C>(w_hat, C_in, C_out, o0, 0, wvec_ok != 0, wr);
    for (int c = 0; c < nchunks; ++c) {
        store_x_planes<C>(xr, sA);
        store_w_planes<C>(wr, sB);
        __syncthreads();
        if (c + 1 < nchunks) {
            load_x_chunk<C>(x, T, C_in, t0, (c + 1) * C::KC, vec_ok != 0, xr);
            load_w_chunk<C>(w_hat, C_in, C_out, o0, (c + 1) * C::KC, wvec_ok != 0, wr);
        }
        chunk_products<C>(sA, sB, acc);
        __syncthreads();
    }
    store_y<C>(acc, y, T, C_out, t0, o0);
}

// --- host-side launch ---------------------------------------------------------------

template <class C>
hipError_t launch_cfg(const void* x, const void* w_hat, void* y, int64_t T, int C_in,
                             int C_out, hipStream_t stream) {
    using IO = typename C::IO;
    const int64_t n_t = (T + C::TT - 1) / C::TT;
    const int n_c = (C_out + C::CT - 1) / C::CT;
    const int64_t total = n_t * n_c;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    const int S = (int)sizeof(IO);
    const int vec_ok = ((int64_t)C_in * C::N * S) % 16 == 0;
    const int wvec_ok = ((int64_t)C_in * S) % 16 == 0;
    hipLaunchKernelGGL((cn_forward_kernel<C>), dim3((uint32_t)total), dim3(C::kThreads), 0, stream,
                       (const IO*)x, (const IO*)w_hat, (IO*)y, T, C_in, C_out, n_c,
                       (uint32_t)total, vec_ok, wvec_ok);
    return hipGetLastError();
}

// Tile choice: prefer the 64x64 tile; fall back to smaller tiles while the
// grid would leave CUs idle (256 CUs, two resident workgroups each).
template <int N, typename IO>
hipError_t launch_n(const void* x, const void* w_hat, void* y, int64_t T, int C_in,
                           int C_out, hipStream_t stream, int tile_override) {
    using Big = std::conditional_t<(N <= 8), CnCfg<N, IO, 2, 2, 2, 2>, CnCfg<N, IO, 2, 2, 2, 1>>;
    using Mid = CnCfg<N, IO, 2, 2, 1, 1>;
    using Tiny = CnCfg<N, IO, 1, 1, 1, 1>;
    auto tiles = [&](int TT, int CT) { return ((T + TT - 1) / TT) * (int64_t)((C_out + CT - 1) / CT); };
    int choice = tile_override;
    if (choice < 0) {
        if (C_out > Mid::CT && tiles(Big::TT, Big::CT) >= 512) choice = 0;
        else if (tiles(Mid::TT, Mid::CT) >= 512) choice = 1;
        else choice = 2;
    }
    switch (choice) {
        case 0: return launch_cfg<Big>(x, w_hat, y, T, C_in, C_out, stream);
        case 1: return launch_cfg<Mid>(x, w_hat, y, T, C_in, C_out, stream);
        default: return launch_cfg<Tiny>(x, w_hat, y, T, C_in, C_out, stream);
    }
}

}  // namespace eql
