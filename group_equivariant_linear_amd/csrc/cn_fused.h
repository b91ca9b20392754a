// cn_fused.h -- fused C_N equivariant linear forward for gfx950.
//
// One kernel does the whole layer ("Flash EQ-Linear", Algorithmic Approach and
// Implementation: DFT along the group axis, per-frequency channel products over
// the non-redundant half of the spectrum, inverse DFT; fused, with the Fourier
// fragments kept in registers and no intermediate global writes).
//
// Work split: a workgroup owns WAVES x 16 tokens and CT = 16*CB output channels;
// each wave owns 16 of those tokens and all CT channels.  Per chunk of KC input
// channels (32 for bf16, 16 for fp32 -- 64 bytes of weight row either way):
//
//   x   : every lane loads the N-element records of KC/4 consecutive channels of
//         one token straight from HBM into VGPRs (16N contiguous bytes), in the
//         MFMA A-operand layout (row = token lane%16, k = channels of lane/16);
//         the real DFT runs on those registers and yields the A fragments of all
//         N frequency planes -- x never passes through LDS;
//   w_hat: the chunk [N planes][CT rows][KC] streams from L2 into one of two LDS
//         buffers with direct global->LDS loads (no staging registers), in an
//         XOR-swizzled order that makes the B-fragment reads bank-conflict free;
//   MFMA: per plane, 16x16 products into fp32 accumulators for all N planes:
//           DC, Nyquist:  Y += X W^T
//           bin k:        Yr += Xr Wr^T - Xi Wi^T,  Yi += Xr Wi^T + Xi Wr^T
//         (the complex product as a real 2x2 block product).
//
// After the last chunk every lane holds, for each of its (token, channel)
// outputs, the accumulators of all N planes: the inverse real DFT is lane-local
// and y is written exactly once.
#pragma once

#include "eq_device.h"
#include "eq_launch.h"

namespace eql {

// GELU in its erf form, v * Phi(v), Phi(v) = erfc(-v / sqrt 2) / 2 (Phi: standard
// normal distribution function).  erfc(z) for z >= 0 is the Chebyshev-fitted form
// of Numerical Recipes (Press et al., 2nd ed., section 6.2, "erfcc"):
// erfc(z) = t exp(-z^2 + P(t)), t = 1 / (1 + z/2), P of degree 9, with a fractional
// error below 1.2e-7 for every z >= 0, so both tails of GELU keep their relative
// accuracy; erfc(-z) = 2 - erfc(z).  Branch-free: one reciprocal and one exp2 on
// the transcendental unit and a dozen FMAs, about half the cost of erff.  The
// constants are folded at compile time: z/2 = |v| / (2 sqrt 2); P is scaled by
// log2(e) (exp -> exp2) with the halving of erfc/2 as -1 in its constant term;
// -z^2 log2(e) = -|v| (|v| log2(e) / 2), the product exact inside the fma.
struct GeluCoef {
    static constexpr double kLog2e = 1.44269504088896340736;
    static constexpr double c[10] = {0.17087277, -0.82215223, 1.48851587, -1.13520398, 0.27886807,
                                     -0.18628806, 0.09678418, 0.37409196, 1.00002368, -1.26551223};
    static constexpr float scaled(int i) { return (float)(c[i] * kLog2e - (i == 9 ? 1.0 : 0.0)); }
};

__device__ __forceinline__ float gelu_erf(float v) {
    const float a = fabsf(v);
    const float t = __builtin_amdgcn_rcpf(fmaf(a, 0.35355339059327376f, 1.0f));
    float p = GeluCoef::scaled(0);
    p = fmaf(p, t, GeluCoef::scaled(1));
    p = fmaf(p, t, GeluCoef::scaled(2));
    p = fmaf(p, t, GeluCoef::scaled(3));
    p = fmaf(p, t, GeluCoef::scaled(4));
    p = fmaf(p, t, GeluCoef::scaled(5));
    p = fmaf(p, t, GeluCoef::scaled(6));
    p = fmaf(p, t, GeluCoef::scaled(7));
    p = fmaf(p, t, GeluCoef::scaled(8));
    p = fmaf(p, t, GeluCoef::scaled(9));
    // h = erfc(|v| / sqrt 2) / 2 = Phi(-|v|)
    const float h = t * __builtin_amdgcn_exp2f(fmaf(-a, a * (float)(0.5 * GeluCoef::kLog2e), p));
    return v * (v < 0.0f ? h : 1.0f - h);
}

constexpr uint32_t kOOB = 0x80000000u;  // offset past every resource (extents < 2^31)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    // word 3 = 0x00020000: raw (untyped) buffer, 32-bit data format, as on all gfx9 parts
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Fused neighbours of the layer ("Quick ViTs", key design 2: an MLP keeps its
// GELU, applied where the group permutes coordinates -- for C_N the output y
// itself, whose group axis a rotation shifts cyclically; a per-channel bias is
// constant along that axis).  The epilogue runs them when epi_on(epi): the NV
// values of one output channel become act(v + b).  Off, nothing is touched (an
// added zero would turn -0 into +0).
__device__ __forceinline__ bool epi_on(const Epi& epi) { return epi.bias != nullptr || epi.act != 0; }

template <int NV>
__device__ __forceinline__ void epi_apply(float* v, float b, int act) {
    if (act == 1) {
#pragma unroll
        for (int k = 0; k < NV; ++k) v[k] = gelu_erf(v[k] + b);
    } else {
#pragma unroll
        for (int k = 0; k < NV; ++k) v[k] += b;
    }
}

// Bias element o of the layer as raw bits, through a buffer resource over the
// bias alone: o past C_out, and a NULL bias (an empty resource), read 0 without
// a branch or a memory access.  The register is not touched until the epilogue,
// so the load's latency hides under the main loop (vector loads complete in
// issue order, so the main loop's own waits cover it).  A load issued in the
// store phase would instead wait behind the stores in flight: one counter
// tracks both.
template <typename IO>
__device__ __forceinline__ uint32_t bias_fetch(const Epi& epi, int C_out, int o) {
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(epi.bias, epi.bias ? (uint32_t)C_out * (uint32_t)sizeof(IO) : 0u);
    const uint32_t off = o < C_out ? (uint32_t)o * (uint32_t)sizeof(IO) : kOOB;
    if constexpr (sizeof(IO) == 4) return __builtin_amdgcn_raw_buffer_load_b32(rb, off, 0, 0);
    else return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, off, 0, 0);
}
template <typename IO>
__device__ __forceinline__ float bias_value(uint32_t bits) {
    if constexpr (sizeof(IO) == 4) return __uint_as_float(bits);
    else return Half<IO>::lo(bits);
}

// Workgroups per CU that an LDS allocation of b bytes allows (512-byte granules).
constexpr int lds_groups(int b) { return 163840 / ((b + 511) / 512 * 512); }

// The bias of a workgroup's CT output channels [o0, o0 + CT) (thread t holds
// channels t, t + NT, ...), published to LDS and read back per channel in the
// epilogue.  OWN: a slice of its own after the kernel's LDS bytes, fetched and
// published just before the main loop, so the load's latency overlaps the first
// stage's and no register carries it through the loop; taken only when the extra
// bytes keep as many workgroups per CU.  Otherwise the bytes from FREE_OFF, which
// the epilogue does not use but the main loop does: fetched and published after
// the epilogue's first barrier, read after a second (those kernels run two or
// more workgroups per CU, which hide the load).  FITS is false when neither
// exists (the epilogue's staging fills the CU's LDS); such kernels keep each
// lane's bias values in registers instead.
template <typename IO, int CT, int NT, int LDS, int FREE_OFF>
struct BiasTile {
    static constexpr int NR = (CT + NT - 1) / NT;
    static constexpr int BYTES = (CT * 4 + 15) / 16 * 16;
    static constexpr bool OWN = LDS + BYTES <= 163840 && lds_groups(LDS + BYTES) == lds_groups(LDS);
    static constexpr bool FITS = OWN || FREE_OFF + BYTES <= LDS;
    static constexpr int OFF = OWN ? LDS : FREE_OFF;
    static constexpr int SMEM = OWN ? LDS + BYTES : LDS;  // the kernel's LDS allocation
    uint32_t r[NR];
    __device__ __forceinline__ void fetch(const Epi& epi, int o0, int C_out) {
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const int c = (int)threadIdx.x + k * NT;
            r[k] = bias_fetch<IO>(epi, C_out, c < CT ? o0 + c : C_out);
        }
    }
    // call before a barrier that precedes every read of the slice
    __device__ __forceinline__ void publish(float* lds) const {
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const int c = (int)threadIdx.x + k * NT;
            if (c < CT) lds[c] = bias_value<IO>(r[k]);
        }
    }
};

template <typename IO>
struct IoTraits;
template <>
struct IoTraits<float> {
    static constexpr int KC = 16;  // channels per chunk: 4 MFMA 16x16x4 steps
    static constexpr int R = 4;    // channels per lane per chunk
};
template <>
struct IoTraits<__bf16> {
    static constexpr int KC = 32;  // one MFMA 16x16x32 step
    static constexpr int R = 8;
};
template <>
struct IoTraits<_Float16> {
    static constexpr int KC = 32;  // one MFMA 16x16x32 step
    static constexpr int R = 8;
};

template <int N_, typename IO_, int WAVES_, int CB_>
struct FusedCfg {
    static constexpr int N = N_;
    using IO = IO_;
    static constexpr int WAVES = WAVES_, CB = CB_;
    static constexpr int kThreads = 64 * WAVES;
    static constexpr int TT = 16 * WAVES;  // tokens per workgroup
    static constexpr int CT = 16 * CB;     // output channels per workgroup
    static constexpr int KC = IoTraits<IO>::KC;
    static constexpr int R = IoTraits<IO>::R;
    static constexpr int S = (int)sizeof(IO);
    static constexpr int XW = 4 * N;                // dwords of one lane's x records (16N bytes)
    static constexpr int SLOTS = N * CT * 4;        // 16-byte slots of one w_hat chunk
    static constexpr int BUF_BYTES = SLOTS * 16;    // one LDS buffer
    static constexpr int DMA_ITERS = (SLOTS + kThreads - 1) / kThreads;
};

// 16-byte slot of (row o, part q) inside one plane of a w_hat chunk.
__device__ __forceinline__ int wslot(int o, int q) { return o * 4 + (q ^ ((o >> 1) & 3)); }

template <typename IO>
__device__ __forceinline__ float elem_f32(const uint32_t* w, int e) {
    if constexpr (sizeof(IO) == 4) return __uint_as_float(w[e]);
    else return (e & 1) ? Half<IO>::hi(w[e >> 1]) : Half<IO>::lo(w[e >> 1]);
}

template <typename IO>
__device__ __forceinline__ void set_bits(uint32_t* w, int e, uint32_t b) {
    if constexpr (sizeof(IO) == 4) {
        w[e] = b;
    } else {
        if (e & 1) w[e >> 1] = (w[e >> 1] & 0x0000ffffu) | (b << 16);
        else w[e >> 1] = (w[e >> 1] & 0xffff0000u) | b;
    }
}

template <typename IO>
__device__ __forceinline__ uint32_t raw_bits(const IO* p) {
    if constexpr (sizeof(IO) == 4) return *reinterpret_cast<const uint32_t*>(p);
    else return (uint32_t)*reinterpret_cast<const uint16_t*>(p);
}

// One lane's x records for a chunk: R channels (c0 .. c0+R-1) of token t.
template <class C>
__device__ __forceinline__ void load_x(const typename C::IO* __restrict__ x, int64_t T, int C_in,
                                       int64_t t, int c0, bool vec_ok, uint32_t (&xr)[C::XW]) {
    using IO = typename C::IO;
    const IO* src = x + (t * C_in + c0) * C::N;
    if (vec_ok && t < T && c0 + C::R <= C_in) {
        const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
#pragma unroll
        for (int j = 0; j < C::N; ++j) {
            const u32x4 v = __builtin_nontemporal_load(s4 + j);
            xr[4 * j + 0] = v.x;
            xr[4 * j + 1] = v.y;
            xr[4 * j + 2] = v.z;
            xr[4 * j + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < C::XW; ++j) xr[j] = 0u;
        if (t < T) {
#pragma unroll
            for (int e = 0; e < C::R * C::N; ++e)
                if (c0 + e / C::N < C_in) set_bits<IO>(xr, e, raw_bits<IO>(src + e));
        }
    }
}

template <typename IO>
struct AFrag;
template <>
struct AFrag<__bf16> {
    using T = bf16x8;
};
template <>
struct AFrag<_Float16> {
    using T = f16x8;
};
template <>
struct AFrag<float> {
    using T = f32x4;
};

// Real DFT of the lane's R records -> A fragments of the N planes.
template <class C>
__device__ __forceinline__ void x_to_planes(const uint32_t (&xr)[C::XW],
                                            typename AFrag<typename C::IO>::T (&A)[C::N]) {
    using IO = typename C::IO;
    constexpr int N = C::N;
    if constexpr (sizeof(IO) == 4) {
#pragma unroll
        for (int r = 0; r < C::R; ++r) {
            float xv[N], P[N];
#pragma unroll
            for (int h = 0; h < N; ++h) xv[h] = elem_f32<IO>(xr, r * N + h);
            rdft_forward<N>(xv, P);
#pragma unroll
            for (int p = 0; p < N; ++p) A[p][r] = P[p];
        }
    } else {
        uint32_t pk[N][4];
#pragma unroll
        for (int r = 0; r < C::R; r += 2) {
            float xa[N], xb[N], Pa[N], Pb[N];
#pragma unroll
            for (int h = 0; h < N; ++h) {
                xa[h] = elem_f32<IO>(xr, r * N + h);
                xb[h] = elem_f32<IO>(xr, (r + 1) * N + h);
            }
            rdft_forward<N>(xa, Pa);
            rdft_forward<N>(xb, Pb);
#pragma unroll
            for (int p = 0; p < N; ++p)
                pk[p][r / 2] = Half<IO>::pack2(Pa[p] * spec_scale<IO, N>, Pb[p] * spec_scale<IO, N>);
        }
#pragma unroll
        for (int p = 0; p < N; ++p) {
            const u32x4 v = {pk[p][0], pk[p][1], pk[p][2], pk[p][3]};
            A[p] = __builtin_bit_cast(typename AFrag<IO>::T, v);
        }
    }
}

// Issue the direct global->LDS loads of one w_hat chunk (all threads of the
// workgroup together).  Slots whose row is past C_out or whose channels are past
// C_in read w_hat[0] instead: finite values that only meet zero activations
// (K tail) or feed outputs that are never stored (rows past C_out).
template <class C>
__device__ __forceinline__ void dma_w_chunk(const typename C::IO* __restrict__ w_hat, int C_in,
                                            int C_out, int o0, int i0, char* lds_buf) {
    using IO = typename C::IO;
    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
#pragma unroll
    for (int it = 0; it < C::DMA_ITERS; ++it) {
        const int base = (it * C::WAVES + wave) * 64;  // first slot of this wave instruction
        if (C::SLOTS % C::kThreads != 0 && base >= C::SLOTS) continue;
        const int s = base + lane;
        const int p = s / (C::CT * 4);
        const int sp = s % (C::CT * 4);
        const int o = sp >> 2;
        const int q = (sp & 3) ^ ((o >> 1) & 3);
        const int orow = o0 + o, ch = i0 + q * C::R;
        const IO* src = w_hat;
        if (s < C::SLOTS && orow < C_out && ch < C_in) src = w_hat + ((int64_t)p * C_out + orow) * C_in + ch;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds_buf + base * 16), 16, 0, 0);
    }
}

// Register-staged fallback for w_hat rows that are not 16-byte aligned
// (C_in * sizeof(IO) not a multiple of 16): plain loads with zero fill.
template <class C>
__device__ __forceinline__ void copy_w_chunk(const typename C::IO* __restrict__ w_hat, int C_in,
                                             int C_out, int o0, int i0, char* lds_buf) {
    using IO = typename C::IO;
    for (int s = (int)threadIdx.x; s < C::SLOTS; s += C::kThreads) {
        const int p = s / (C::CT * 4);
        const int sp = s % (C::CT * 4);
        const int o = sp >> 2;
        const int q = (sp & 3) ^ ((o >> 1) & 3);
        const int orow = o0 + o, ch = i0 + q * C::R;
        uint32_t w4[4] = {0u, 0u, 0u, 0u};
        if (orow < C_out) {
            const IO* src = w_hat + ((int64_t)p * C_out + orow) * C_in + ch;
#pragma unroll
            for (int e = 0; e < C::R; ++e)
                if (ch + e < C_in) set_bits<IO>(w4, e, raw_bits<IO>(src + e));
        }
        *reinterpret_cast<u32x4*>(lds_buf + s * 16) = u32x4{w4[0], w4[1], w4[2], w4[3]};
    }
}

__device__ __forceinline__ void mma(f32x4& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const f16x8& a, const f16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const f32x4& a, const f32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 neg(const bf16x8& v) {
    u32x4 u = __builtin_bit_cast(u32x4, v);
    u ^= 0x80008000u;
    return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ f16x8 neg(const f16x8& v) {
    u32x4 u = __builtin_bit_cast(u32x4, v);
    u ^= 0x80008000u;
    return __builtin_bit_cast(f16x8, u);
}
__device__ __forceinline__ f32x4 neg(const f32x4& v) { return -v; }

template <class C>
__device__ __forceinline__ void chunk_products(const typename AFrag<typename C::IO>::T (&A)[C::N],
                                               const char* lds_buf,
                                               f32x4 (&acc)[C::N][C::CB]) {
    using F = typename AFrag<typename C::IO>::T;
    constexpr int N = C::N;
    const int lane = (int)threadIdx.x & 63;
    const int q = lane >> 4;
    // byte offset of this lane's B fragment for cout block b, plane p:
    //   p * CT * 64 + wslot(b*16 + lane%16, q) * 16; the swizzle term only
    //   depends on (lane%16), so one base offset per lane covers every block.
    const int o_l = lane & 15;
    const int lane_off = (o_l * 4 + (q ^ ((o_l >> 1) & 3))) * 16;
    auto ldB = [&](int p, int b) {
        return *reinterpret_cast<const F*>(lds_buf + p * C::CT * 64 + b * 16 * 64 + lane_off);
    };
#pragma unroll
    for (int b = 0; b < C::CB; ++b) mma(acc[0][b], A[0], ldB(0, b));
#pragma unroll
    for (int k = 1; k <= (N - 1) / 2; ++k) {
        const int pr = 2 * k - 1, pi = 2 * k;
        const F nAi = neg(A[pi]);
#pragma unroll
        for (int b = 0; b < C::CB; ++b) {
            const F Br = ldB(pr, b), Bi = ldB(pi, b);
            mma(acc[pr][b], A[pr], Br);
            mma(acc[pr][b], nAi, Bi);
            mma(acc[pi][b], A[pr], Bi);
            mma(acc[pi][b], A[pi], Br);
        }
    }
    if constexpr (N % 2 == 0 && N > 1) {
#pragma unroll
        for (int b = 0; b < C::CB; ++b) mma(acc[N - 1][b], A[N - 1], ldB(N - 1, b));
    }
}

template <class C>
__device__ __forceinline__ void store_y(const f32x4 (&acc)[C::N][C::CB], typename C::IO* __restrict__ y,
                                        int64_t T, int C_out, int64_t tw0, int o0, const Epi& epi,
                                        const float* lbias) {
    using IO = typename C::IO;
    constexpr int N = C::N;
    const int lane = (int)threadIdx.x & 63;
#pragma unroll
    for (int b = 0; b < C::CB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t t = tw0 + (lane >> 4) * 4 + r;
            const int o = o0 + b * 16 + (lane & 15);
            float P[N], yv[N];
#pragma unroll
            for (int p = 0; p < N; ++p) P[p] = acc[p][b][r] * spec_unscale<IO, N>;
            rdft_inverse<N>(P, yv);
            if (epi_on(epi)) epi_apply<N>(yv, epi.bias != nullptr ? lbias[o - o0] : 0.0f, epi.act);
            if (t >= T || o >= C_out) continue;
            IO* dst = y + (t * C_out + o) * N;
            if constexpr (sizeof(IO) == 4) {
                if constexpr (N % 4 == 0) {
#pragma unroll
                    for (int j = 0; j < N / 4; ++j)
                        __builtin_nontemporal_store(f32x4{yv[4 * j], yv[4 * j + 1], yv[4 * j + 2], yv[4 * j + 3]},
                                                    reinterpret_cast<f32x4*>(dst) + j);
                } else {
#pragma unroll
                    for (int j = 0; j < N; ++j) dst[j] = yv[j];
                }
            } else {
                if constexpr (N % 8 == 0) {
#pragma unroll
                    for (int j = 0; j < N / 8; ++j) {
                        const u32x4 v = {Half<IO>::pack2(yv[8 * j], yv[8 * j + 1]), Half<IO>::pack2(yv[8 * j + 2], yv[8 * j + 3]),
                                         Half<IO>::pack2(yv[8 * j + 4], yv[8 * j + 5]), Half<IO>::pack2(yv[8 * j + 6], yv[8 * j + 7])};
                        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst) + j);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < N; ++j) dst[j] = (IO)yv[j];
                }
            }
        }
}

template <class C>
__global__ __launch_bounds__(C::kThreads) void cn_fused_kernel(
    const typename C::IO* __restrict__ x, const typename C::IO* __restrict__ w_hat,
    typename C::IO* __restrict__ y, int64_t T, int C_in, int C_out, int n_c_tiles,
    uint32_t total_tiles, int vec_ok, int w_dma_ok, Epi epi) {
    using IO = typename C::IO;
    using F = typename AFrag<IO>::T;
    using BiasT = BiasTile<IO, C::CT, C::kThreads, 2 * C::BUF_BYTES, 0>;
    static_assert(BiasT::FITS, "the chunk buffers are free in the epilogue");
    __shared__ __attribute__((aligned(16))) char smem[BiasT::SMEM];
    float* lbias = reinterpret_cast<float*>(smem + BiasT::OFF);

    const uint32_t tile = xcd_remap(blockIdx.x, total_tiles);
    const int64_t t0 = (int64_t)(tile / n_c_tiles) * C::TT;
    const int o0 = (int)(tile % n_c_tiles) * C::CT;
    BiasT bias;
    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
    const int64_t tw0 = t0 + wave * 16;          // this wave's first token
    const int64_t t_lane = tw0 + (lane & 15);    // token of this lane's A row
    const int q = lane >> 4;

    f32x4 acc[C::N][C::CB];
#pragma unroll
    for (int p = 0; p < C::N; ++p)
#pragma unroll
        for (int b = 0; b < C::CB; ++b) acc[p][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nch = (C_in + C::KC - 1) / C::KC;
    uint32_t xr[C::XW];
    if (w_dma_ok) dma_w_chunk<C>(w_hat, C_in, C_out, o0, 0, smem);
    else copy_w_chunk<C>(w_hat, C_in, C_out, o0, 0, smem);
    load_x<C>(x, T, C_in, t_lane, q * C::R, vec_ok != 0, xr);
    // the bias slice is its own: fetch and publish it now, after the first
    // stage's loads (the wait for the bias load then overlaps the wait for that
    // stage, which the loop does first); the loop's barriers order it before
    // the epilogue's reads, and no register carries it through the loop
    if (BiasT::OWN && epi.bias != nullptr) {
        bias.fetch(epi, o0, C_out);
        bias.publish(lbias);
    }
    for (int c = 0; c < nch; ++c) {
        char* cur = smem + (c & 1) * C::BUF_BYTES;
        char* nxt = smem + ((c + 1) & 1) * C::BUF_BYTES;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (c + 1 < nch) {
            if (w_dma_ok) dma_w_chunk<C>(w_hat, C_in, C_out, o0, (c + 1) * C::KC, nxt);
            else copy_w_chunk<C>(w_hat, C_in, C_out, o0, (c + 1) * C::KC, nxt);
        }
        F A[C::N];
        x_to_planes<C>(xr, A);
        if (c + 1 < nch) load_x<C>(x, T, C_in, t_lane, (c + 1) * C::KC + q * C::R, vec_ok != 0, xr);
        chunk_products<C>(A, cur, acc);
    }
    if (!BiasT::OWN && epi.bias != nullptr) {
        __syncthreads();  // every wave is done with the chunk buffers
        bias.fetch(epi, o0, C_out);
        bias.publish(lbias);
        __syncthreads();
    }
    store_y<C>(acc, y, T, C_out, tw0, o0, epi, lbias);
}

// --- fast path: buffer-resource traffic, coalesced through LDS -----------------
//
// Used when C_in is a multiple of R (every x record group and every w_hat row
// chunk is a whole, 16-byte aligned vector).  All global traffic goes through
// buffer resources: one SGPR base per tensor and a 32-bit VGPR offset per lane,
// with the chunk advance in the SGPR offset.  Offsets past the resource's extent
// read as zero and drop writes, which covers the token tail, rows past C_out and
// the input-channel tail without branches; every lane issues the same loads.
//
// x reaches the MFMA A layout in two moves: a coalesced load (each wave
// instruction reads whole 16-byte pieces of consecutive token rows) and an
// exchange through a per-wave LDS region, read back as each lane's records.
// y leaves the same way: the tile is staged in LDS by (token, channel) record and
// written as contiguous 16-byte pieces.  Both LDS layouts are conflict-free: row
// pitches that are multiples of 8 pieces rotate each row by its index, other
// pitches are made odd.


template <int N_, typename IO_, int WAVES_, int CB_>
struct FastCfg : FusedCfg<N_, IO_, WAVES_, CB_> {
    using Base = FusedCfg<N_, IO_, WAVES_, CB_>;
    static constexpr int kThreads = 64 * WAVES_;
    static constexpr int DMA_ITERS = (Base::SLOTS + kThreads - 1) / kThreads;
    // w_hat tile buffer, padded so every wave issues exactly DMA_ITERS loads
    static constexpr int BUF_BYTES = DMA_ITERS * kThreads * 16;
    // x exchange: 16 token rows x XP pieces (one chunk of one wave)
    static constexpr int XP = 4 * N_;  // KC * N * sizeof / 16
    static constexpr bool XROT = (XP % 8) == 0;
    static constexpr int XPITCH = XROT ? XP : (XP | 1);
    static constexpr int XEX_BYTES = 16 * XPITCH * 16;
    static constexpr int W_REGION = 2 * BUF_BYTES;
    static constexpr int X_REGION = WAVES_ * XEX_BYTES;
    // y staging: 16 token rows x YP pieces per wave, after the main loop
    static constexpr int YROW = Base::CT * N_ * Base::S;  // bytes of one token row of the tile
    static constexpr int YP = YROW / 16;
    static constexpr bool YROT = (YP % 8) == 0;
    static constexpr int YPITCH = YROT ? YP : (YP | 1);
    static constexpr int YST_BYTES = 16 * YPITCH * 16;
    static constexpr int MAIN_BYTES = W_REGION + X_REGION;
    static constexpr int LDS_BYTES =
        MAIN_BYTES > WAVES_ * YST_BYTES ? MAIN_BYTES : WAVES_ * YST_BYTES;
    static_assert(YROW % 16 == 0, "tile rows are whole pieces");
};

// LDS piece index of piece k of row r in a region with pitch P and X pieces per row.
template <bool ROT, int X, int P>
__device__ __forceinline__ int xpiece(int r, int k) {
    if constexpr (ROT) return r * P + ((k + r) % X);
    else return r * P + k;
}

// slot s of a w_hat chunk -> plane p, row o, channel part q (inverse of wslot)
template <class C>
__device__ __forceinline__ void slot_coords(int s, int& p, int& o, int& q) {
    p = s / (C::CT * 4);
    const int sp = s % (C::CT * 4);
    o = sp >> 2;
    q = (sp & 3) ^ ((o >> 1) & 3);
}

template <class C>
__device__ __forceinline__ void fast_dma_w(__amdgpu_buffer_rsrc_t rw, const uint32_t (&woff)[C::DMA_ITERS],
                                           uint32_t chunk_off, bool tail, int k0, int C_in,
                                           char* lds_buf) {
    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
#pragma unroll
    for (int it = 0; it < C::DMA_ITERS; ++it) {
        const int base = (it * C::WAVES + wave) * 64;  // slots past SLOTS land in the padding
        uint32_t off = woff[it];
        if (tail) {
            int p, o, q;
            slot_coords<C>(base + lane, p, o, q);
            if (k0 + q * C::R >= C_in) off = kOOB;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rw, (__attribute__((address_space(3))) void*)(lds_buf + base * 16), 16, off, chunk_off, 0, 0);
    }
}

template <class C>
__device__ __forceinline__ void fast_products(const typename AFrag<typename C::IO>::T (&A)[C::N],
                                              const char* lds_buf, f32x4 (&acc)[C::N][C::CB]) {
    using F = typename AFrag<typename C::IO>::T;
    constexpr int N = C::N;
    const int lane = (int)threadIdx.x & 63;
    const int q = lane >> 4, o_l = lane & 15;
    const int lane_off = (o_l * 4 + (q ^ ((o_l >> 1) & 3))) * 16;
    auto ldB = [&](int p, int b) {
        return *reinterpret_cast<const F*>(lds_buf + p * C::CT * 64 + b * 1024 + lane_off);
    };
#pragma unroll
    for (int b = 0; b < C::CB; ++b) mma(acc[0][b], A[0], ldB(0, b));
#pragma unroll
    for (int k = 1; k <= (N - 1) / 2; ++k) {
        const int pr = 2 * k - 1, pi = 2 * k;
        const F nAi = neg(A[pi]);
#pragma unroll
        for (int b = 0; b < C::CB; ++b) {
            const F Br = ldB(pr, b), Bi = ldB(pi, b);
            // the two products into one accumulator are a product apart
            mma(acc[pr][b], A[pr], Br);
            mma(acc[pi][b], A[pr], Bi);
            mma(acc[pr][b], nAi, Bi);
            mma(acc[pi][b], A[pi], Br);
        }
    }
    if constexpr (N % 2 == 0 && N > 1) {
#pragma unroll
        for (int b = 0; b < C::CB; ++b) mma(acc[N - 1][b], A[N - 1], ldB(N - 1, b));
    }
}

template <class C>
__global__ __launch_bounds__(C::kThreads) void cn_fast_kernel(
    const typename C::IO* __restrict__ x, const typename C::IO* __restrict__ w_hat,
    typename C::IO* __restrict__ y, int64_t T, int C_in, int C_out, int n_c_tiles,
    uint32_t total_tiles, uint32_t w_bytes, int y_coalesced, Epi epi) {
    using IO = typename C::IO;
    using F = typename AFrag<IO>::T;
    constexpr int N = C::N, S = C::S, XP = C::XP;
    using BiasT = BiasTile<IO, C::CT, C::kThreads, C::LDS_BYTES, C::WAVES * C::YST_BYTES>;
    constexpr bool kLdsBias = BiasT::FITS;
    __shared__ __attribute__((aligned(16))) char smem[BiasT::SMEM];
    float* lbias = reinterpret_cast<float*>(smem + BiasT::OFF);

    const uint32_t tile = xcd_remap(blockIdx.x, total_tiles);
    const int64_t t0 = (int64_t)(tile / n_c_tiles) * C::TT;
    const int o0 = (int)(tile % n_c_tiles) * C::CT;
    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
    const int q = lane >> 4;
    // the epilogue's lane holds output channels o0 + 16 b + lane % 16
    BiasT bias;
    uint32_t breg[kLdsBias ? 1 : C::CB];
    if constexpr (!kLdsBias) {
#pragma unroll
        for (int b = 0; b < C::CB; ++b) {
            breg[b] = 0u;
            if (epi.bias != nullptr) breg[b] = bias_fetch<IO>(epi, C_out, o0 + b * 16 + (lane & 15));
        }
    }
    auto bias_of = [&](int b) -> float {
        if constexpr (kLdsBias) return epi.bias != nullptr ? lbias[b * 16 + (lane & 15)] : 0.0f;
        else return bias_value<IO>(breg[b]);
    };

    const uint32_t row_x = (uint32_t)C_in * (N * S), row_y = (uint32_t)C_out * (N * S);
    const int64_t rem = T - t0;
    const uint32_t rows = (uint32_t)(rem < C::TT ? rem : C::TT);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + t0 * C_in * N, rows * row_x);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(y + t0 * C_out * N, rows * row_y);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_hat, w_bytes);

    char* wbuf = smem;                                         // two w_hat tile buffers
    char* xex = smem + C::W_REGION + wave * C::XEX_BYTES;      // this wave's x exchange region

    // loop-invariant offsets of the coalesced x loads: instruction j, lane l
    // fetches piece k of row r of this wave's 16 rows (pc = 64 j + l = r XP + k)
    uint32_t xoff[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const int pc = 64 * j + lane, r = pc / XP, k = pc % XP;
        xoff[j] = (uint32_t)(wave * 16 + r) * row_x + (uint32_t)k * 16u;
    }
    uint32_t woff[C::DMA_ITERS];
#pragma unroll
    for (int it = 0; it < C::DMA_ITERS; ++it) {
        int p, o, qq;
        slot_coords<C>((it * C::WAVES + wave) * 64 + lane, p, o, qq);
        woff[it] = (o0 + o < C_out && p < N)
                       ? (uint32_t)((((int64_t)p * C_out + o0 + o) * C_in + qq * C::R) * S)
                       : kOOB;
    }

    f32x4 acc[N][C::CB];
#pragma unroll
    for (int p = 0; p < N; ++p)
#pragma unroll
        for (int b = 0; b < C::CB; ++b) acc[p][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nch = (C_in + C::KC - 1) / C::KC;
    const uint32_t chunk_x = (uint32_t)C::KC * (N * S);
    auto load_x = [&](int c, uint32_t(&xr)[C::XW]) {
        const bool tail = c * C::KC + C::KC > C_in;
        const uint32_t valid = tail ? (uint32_t)(C_in - c * C::KC) * (N * S) : 0xffffffffu;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int k = (64 * j + lane) % XP;
            const uint32_t off = (c < nch && (uint32_t)k * 16u < valid) ? xoff[j] : kOOB;
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rx, off, (uint32_t)c * chunk_x, 0);
            xr[4 * j + 0] = v.x;
            xr[4 * j + 1] = v.y;
            xr[4 * j + 2] = v.z;
            xr[4 * j + 3] = v.w;
        }
    };
    auto dma = [&](int c, char* buf) {
        if (c < nch)
            fast_dma_w<C>(rw, woff, (uint32_t)(c * C::KC * S), c * C::KC + C::KC > C_in, c * C::KC, C_in, buf);
    };
    // coalesced pieces -> LDS -> this lane's records (A layout: row = lane%16,
    // pieces q*N .. q*N+N-1 of that row)
    auto exchange = [&](const uint32_t(&xr)[C::XW], uint32_t(&xa)[C::XW]) {
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int pc = 64 * j + lane, r = pc / XP, k = pc % XP;
            *reinterpret_cast<u32x4*>(xex + xpiece<C::XROT, XP, C::XPITCH>(r, k) * 16) =
                u32x4{xr[4 * j], xr[4 * j + 1], xr[4 * j + 2], xr[4 * j + 3]};
        }
        const int r = lane & 15;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(xex + xpiece<C::XROT, XP, C::XPITCH>(r, q * N + j) * 16);
            xa[4 * j + 0] = v.x;
            xa[4 * j + 1] = v.y;
            xa[4 * j + 2] = v.z;
            xa[4 * j + 3] = v.w;
        }
    };

    // Per chunk c: wait for w_hat chunk c (LDS) and x chunk c (VGPRs); start the
    // w_hat DMA of chunk c+1; move x through the exchange; transform; start the
    // x loads of chunk c+1 into the registers just freed; multiply while those
    // loads are in flight.
    uint32_t xr[C::XW];
    dma(0, wbuf);
    load_x(0, xr);
    if (kLdsBias && BiasT::OWN && epi.bias != nullptr) {  // as in the generic kernel
        bias.fetch(epi, o0, C_out);
        bias.publish(lbias);
    }
    for (int c = 0; c < nch; ++c) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        dma(c + 1, wbuf + ((c + 1) & 1) * C::BUF_BYTES);
        uint32_t xa[C::XW];
        exchange(xr, xa);
        F A[N];
        x_to_planes<C>(xa, A);
        // unconditional: past the last chunk the offsets are out of range (zeros,
        // no memory access), and the registers keep a single definition
        load_x(c + 1, xr);
        fast_products<C>(A, wbuf + (c & 1) * C::BUF_BYTES, acc);
    }

    // Epilogue: inverse DFT of each (token, channel) record, then y written once.
    if (y_coalesced) {
        __syncthreads();  // the staging area overlaps the tile and exchange buffers
        if (kLdsBias && !BiasT::OWN && epi.bias != nullptr) {
            bias.fetch(epi, o0, C_out);
            bias.publish(lbias);
            __syncthreads();
        }
        char* yst = smem + wave * C::YST_BYTES;
#pragma unroll
        for (int b = 0; b < C::CB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tl = (lane >> 4) * 4 + r, ol = b * 16 + (lane & 15);
                float P[N], yv[N];
#pragma unroll
                for (int p = 0; p < N; ++p) P[p] = acc[p][b][r] * spec_unscale<IO, N>;
                rdft_inverse<N>(P, yv);
                if (epi_on(epi)) epi_apply<N>(yv, bias_of(b), epi.act);
                // record bytes [ol*N*S, ol*N*S + N*S) of row tl, piece-rotated like x
                const int byte0 = ol * N * S;
                if constexpr ((N * S) % 16 == 0) {
#pragma unroll
                    for (int j = 0; j < N * S / 16; ++j) {
                        u32x4 v;
                        if constexpr (sizeof(IO) == 4) {
                            v = u32x4{__float_as_uint(yv[4 * j]), __float_as_uint(yv[4 * j + 1]),
                                      __float_as_uint(yv[4 * j + 2]), __float_as_uint(yv[4 * j + 3])};
                        } else {
                            v = u32x4{Half<IO>::pack2(yv[8 * j], yv[8 * j + 1]), Half<IO>::pack2(yv[8 * j + 2], yv[8 * j + 3]),
                                      Half<IO>::pack2(yv[8 * j + 4], yv[8 * j + 5]), Half<IO>::pack2(yv[8 * j + 6], yv[8 * j + 7])};
                        }
                        *reinterpret_cast<u32x4*>(yst + xpiece<C::YROT, C::YP, C::YPITCH>(tl, byte0 / 16 + j) * 16) = v;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < N; ++e) {
                        const int by = byte0 + e * S;
                        char* dst = yst + xpiece<C::YROT, C::YP, C::YPITCH>(tl, by / 16) * 16 + (by % 16);
                        if constexpr (sizeof(IO) == 4) *reinterpret_cast<float*>(dst) = yv[e];
                        else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(Half<IO>::pack2(yv[e], 0.f) & 0xffffu);
                    }
                }
            }
        // wave-local: its own rows, written and read by the same wave
        const uint32_t cols = (uint32_t)(C_out - o0) * (N * S);  // valid bytes of a tile row
        for (int pc = lane; pc < 16 * C::YP; pc += 64) {
            const int r = pc / C::YP, k = pc % C::YP;
            const u32x4 v = *reinterpret_cast<const u32x4*>(yst + xpiece<C::YROT, C::YP, C::YPITCH>(r, k) * 16);
            const uint32_t off = ((uint32_t)k * 16u < cols)
                                     ? (uint32_t)(wave * 16 + r) * row_y + (uint32_t)o0 * (N * S) + (uint32_t)k * 16u
                                     : kOOB;
            __builtin_amdgcn_raw_buffer_store_b128(v, ry, off, 0, kYStoreAux);
        }
    } else {
        if (kLdsBias && !BiasT::OWN && epi.bias != nullptr) {
            __syncthreads();
            bias.fetch(epi, o0, C_out);
            bias.publish(lbias);
            __syncthreads();
        }
#pragma unroll
        for (int b = 0; b < C::CB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t tl = (uint32_t)(wave * 16 + (lane >> 4) * 4 + r);
                const int o = o0 + b * 16 + (lane & 15);
                const uint32_t off = o < C_out ? tl * row_y + (uint32_t)o * (N * S) : kOOB;
                float P[N], yv[N];
#pragma unroll
                for (int p = 0; p < N; ++p) P[p] = acc[p][b][r] * spec_unscale<IO, N>;
                rdft_inverse<N>(P, yv);
                if (epi_on(epi)) epi_apply<N>(yv, bias_of(b), epi.act);
#pragma unroll
                for (int e = 0; e < N; ++e) {
                    if constexpr (sizeof(IO) == 4)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv[e]), ry, off + 4u * e, 0, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(Half<IO>::pack2(yv[e], 0.f) & 0xffffu), ry,
                                                             off + 2u * e, 0, 0);
                }
            }
    }
}

// --- host side ----------------------------------------------------------------------

template <class C>
hipError_t launch_fused_cfg(const void* x, const void* w_hat, void* y, int64_t T, int C_in,
                            int C_out, hipStream_t stream, Epi epi) {
    using IO = typename C::IO;
    const int64_t n_t = (T + C::TT - 1) / C::TT;
    const int n_c = (C_out + C::CT - 1) / C::CT;
    const int64_t total = n_t * n_c;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    const int S = (int)sizeof(IO);
    const int vec_ok = ((int64_t)C_in * C::N * S) % 16 == 0;
    const int w_dma_ok = ((int64_t)C_in * S) % 16 == 0;
    hipLaunchKernelGGL((cn_fused_kernel<C>), dim3((uint32_t)total), dim3(C::kThreads), 0, stream,
                       (const IO*)x, (const IO*)w_hat, (IO*)y, T, C_in, C_out, n_c, (uint32_t)total,
                       vec_ok, w_dma_ok, epi);
    return hipGetLastError();
}

template <class C>
hipError_t launch_fast_cfg(const void* x, const void* w_hat, void* y, int64_t T, int C_in,
                           int C_out, hipStream_t stream, Epi epi) {
    using IO = typename C::IO;
    const int64_t n_t = (T + C::TT - 1) / C::TT;
    const int n_c = (C_out + C::CT - 1) / C::CT;
    const int64_t total = n_t * n_c;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    const int64_t w_bytes = (int64_t)C::N * C_out * C_in * (int64_t)sizeof(IO);
    // staged, coalesced y stores need whole 16-byte pieces in every row of y
    const int y_coalesced = ((int64_t)C_out * C::N * (int64_t)sizeof(IO)) % 16 == 0;
    hipLaunchKernelGGL((cn_fast_kernel<C>), dim3((uint32_t)total), dim3(C::kThreads), 0, stream,
                       (const IO*)x, (const IO*)w_hat, (IO*)y, T, C_in, C_out, n_c, (uint32_t)total,
                       (uint32_t)w_bytes, y_coalesced, epi);
    return hipGetLastError();
}

// The fast path needs whole 16-byte record groups and 32-bit buffer offsets.
template <int N, typename IO>
bool fast_ok(int C_in, int C_out, int TT) {
    constexpr int R = IoTraits<IO>::R;
    const int64_t S = (int64_t)sizeof(IO);
    const int64_t lim = (int64_t)1 << 30;
    return C_in % R == 0 && (int64_t)N * C_out * C_in * S < lim &&
           (int64_t)TT * C_in * N * S < lim && (int64_t)TT * C_out * N * S < lim;
}

// Tile configurations: (waves per token group, 16-channel output blocks per
// wave, input-channel split), largest output tile first.  Accumulators per
// lane = 4 * N * CB.
template <int N, typename IO>
struct FusedMenu {
    static constexpr int kCount = 7;
    static constexpr int waves[kCount] = {4, 4, 4, 4, 4, 1, 1};
    static constexpr int cb[kCount] = {6, 5, 4, 3, 2, 2, 1};
};

template <int N, typename IO, int I>
hipError_t launch_menu_entry(const void* x, const void* w_hat, void* y, int64_t T, int C_in,
                             int C_out, hipStream_t stream, Epi epi) {
    constexpr int W = FusedMenu<N, IO>::waves[I];
    constexpr int CBr = FusedMenu<N, IO>::cb[I];
    // keep the accumulators within 192 registers per lane and the LDS tiles
    // (two w_hat buffers of N*CB KiB plus the x exchange) within 160 KiB
    // (two w_hat buffers of N*CB KiB plus the x exchange, and afterwards the
    // y staging of 16 rows x 16*CB*N*sizeof bytes per wave) within 160 KiB
    constexpr int cap_acc = 48 / N > 0 ? 48 / N : 1;
    constexpr int cap_lds = 64 / N > 0 ? 64 / N : 1;
    constexpr int cap_y = 163840 / (W * 256 * N * (int)sizeof(IO)) > 0 ? 163840 / (W * 256 * N * (int)sizeof(IO)) : 1;
    constexpr int cap = cap_acc < cap_lds ? (cap_acc < cap_y ? cap_acc : cap_y) : (cap_lds < cap_y ? cap_lds : cap_y);
    constexpr int CB = CBr < cap ? CBr : cap;
    using Cfg = FastCfg<N, IO, W, CB>;
    if (fast_ok<N, IO>(C_in, C_out, Cfg::TT))
        return launch_fast_cfg<Cfg>(x, w_hat, y, T, C_in, C_out, stream, epi);
    // generic path (ragged channel groups): two shapes only
    if constexpr (W == 4) return launch_fused_cfg<FusedCfg<N, IO, 4, (N <= 8 ? 2 : 1)>>(x, w_hat, y, T, C_in, C_out, stream, epi);
    else return launch_fused_cfg<FusedCfg<N, IO, 1, 1>>(x, w_hat, y, T, C_in, C_out, stream, epi);
}

}  // namespace eql
