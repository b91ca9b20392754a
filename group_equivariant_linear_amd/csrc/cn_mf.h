// cn_mf.h -- 16-bit (bf16 or fp16) C_N forward with the group transform on
// the matrix cores.
//
// Same dataflow as the fused kernel ("Flash EQ-Linear", Algorithmic Approach
// and Implementation: DFT along the group axis, per-frequency channel products
// over the non-redundant half of the spectrum, inverse DFT, one pass, no
// intermediate global writes), but the forward DFT of x is itself an MFMA
// product instead of VALU arithmetic.  Per token and channel the real DFT is a
// fixed N x N matrix F applied to the channel's N group elements, so for four
// channels at a time it is one block-diagonal 16 x 32 matrix:
//
//   rows  (g, i)  -> channel g of the four, plane 4m + i      (g, i < 4)
//   cols  (g', h) -> channel g', group element h               (h < 8)
//   entry         =  F[4m + i][h] if g == g' and both in range, else 0
//
// With x as the B operand (each lane's 8 k-values = one channel record of one
// token) the product gives, per lane, 4 planes of one channel of one token in
// fp32.  Eight such products (channels 8g + j, j = 0..7) leave in every lane
// the 8 channels 8g .. 8g+7 of each plane: exactly the B operand of the channel
// products, which are computed transposed,
//
//   Yhat^T[o][t] (+)= What[o][c] Xhat^T[c][t]   (per plane; complex bins as
//                                                the real 2x2 block product)
//
// with the w_hat tile (same LDS layout as the fused kernel) as the A operand.
// Each lane then holds, for one token and four output channels, the
// accumulators of all N planes.  The inverse DFT is the mirror image: the N
// planes of one channel, rounded to bf16, are a lane's 8 k-values, and a
// block-diagonal inverse matrix (rows = 4 group elements of each of the four
// channels) returns y in fp32, which leaves through an LDS staging area as
// contiguous 16-byte pieces.
//
// Supported: bf16 and fp16, 2 <= N <= 8 (one channel record per 8 k-values),
// C_in a multiple of 8.  The transform coefficients enter the matrix cores in
// the I/O type: exact for 0, +-1, +-1/2^j and the quarter turns; other
// twiddles carry a rounding of at most 2^-9 (bf16) or 2^-12 (fp16) relative,
// and the Fourier-domain outputs one more rounding to that type before the
// inverse -- both of the order of the rounding of Xhat and of y that the fused
// kernel already makes.  The forward coefficients carry 1/N and the inverse
// ones N, so the 16-bit spectra are those of x/N and y/N: a bin is at most the
// largest |x| (|y|), and fp16 stays within its range whenever x and y do.
#pragma once

#include "cn_fused.h"
#include "dft_coef.h"

// y leaves the kernel once and is not read again by it: the store phase
// writes whole 128-byte lines (8 lanes per tile row) with the non-temporal
// hint (kYStoreAux).  Measured on MI355X, cache-cold: c3 96.3 ->
// 91.6 us, C7 x 1120 70.7-72.3 -> 68.3-69.0 us; either change alone moved
// neither by more than run-to-run noise.
#ifndef EQL_MF_STORE_LPR
#define EQL_MF_STORE_LPR 8  // lanes per y row in the store phase (4 or 8)
#endif

namespace eql {

// Inverse real-DFT coefficient of group element g from plane p, 1/N included
// (as in rdft_inverse: DC and Nyquist weigh 1/N, the other bins 2/N).
template <int N>
constexpr double inv_coef(int g, int p) {
    if (p == 0) return 1.0 / N;
    if (N % 2 == 0 && p == N - 1) return ((g % 2) ? -1.0 : 1.0) / N;
    const int k = (p + 1) / 2;
    return (p % 2) ? 2.0 / N * turn_trig((long)g * k, N, false) : -2.0 / N * turn_trig((long)g * k, N, true);
}

template <int N_, int WAVES_, int CB_, typename IO_ = __bf16>
struct MfCfg : FastCfg<N_, IO_, WAVES_, CB_> {
    using Base = FastCfg<N_, IO_, WAVES_, CB_>;
    using F8 = typename Half<IO_>::x8;  // 16-bit MFMA fragment (bf16 or fp16)
    static constexpr int N = N_, CB = CB_, CT = 16 * CB_;
    static constexpr int MQ = (N_ + 3) / 4;  // transform products per four channels
    static constexpr int XP = 4 * N_;        // 16-byte pieces of a token row of one chunk
    // records sit inside one piece for N = 2, 4, 8: those rows may be rotated;
    // other orders read records across pieces and need contiguous rows
    static constexpr bool XALIGN = (16 % (2 * N_)) == 0;
    static constexpr bool XROT = XALIGN && (XP % 8) == 0;
    static constexpr int XPITCH = XROT ? XP : (XP | 1);
    // x reaches its exchange rows by direct global->LDS loads: slot s of the
    // region is written by lane s%64 of load s/64, so the region holds whole loads
    static constexpr int XDMA = (16 * XPITCH + 63) / 64;
    static constexpr int XEX_BYTES = XDMA * 1024;
    static constexpr int W_REGION = 2 * Base::BUF_BYTES;
    static constexpr int X_REGION = WAVES_ * XEX_BYTES;
    static constexpr int YP = CT * N_ * 2 / 16;  // pieces of one token row of the y tile
    static constexpr bool YROT = (YP % 8) == 0;
    static constexpr int YPITCH = YROT ? YP : (YP | 1);
    static constexpr int YST_BYTES = 16 * YPITCH * 16;
    static constexpr int MAIN_BYTES = W_REGION + X_REGION;
    static constexpr int LDS_BYTES = MAIN_BYTES > WAVES_ * YST_BYTES ? MAIN_BYTES : WAVES_ * YST_BYTES;
    static_assert(N_ >= 2 && N_ <= 8, "one channel record per 8 k-values");
};

// The MQ block-diagonal transform fragments (A operand) of this lane:
// row (gr, ir) of fragment m, k-values (kg, e): coef(4m + ir, e) / N if kg == gr
// (the inverse: N coef).
// INV selects the inverse transform (rows = group elements, k = planes).
template <class C, bool INV>
__device__ __forceinline__ void make_frags(typename C::F8 (&Fa)[C::MQ]) {
    constexpr int N = C::N;
    const int lane = (int)threadIdx.x & 63;
    const int r = lane & 15, kg = lane >> 4;
    const int gr = r >> 2, ir = r & 3;
    const bool diag = kg == gr;
    static_for<0, C::MQ>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        float v[8];
#pragma unroll
        for (int h = 0; h < 8; ++h) v[h] = 0.0f;
        static_for<0, 4>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            constexpr int p = 4 * m + i;
            if constexpr (p < N) {
                static_for<0, N>([&](auto hc) {
                    constexpr int h = decltype(hc)::value;
                    constexpr float c = (float)(INV ? N * inv_coef<N>(p, h) : fwd_coef<N>(p, h) / N);
                    v[h] = (ir == i) ? c : v[h];
                });
            }
        });
        u32x4 u;
#pragma unroll
        for (int q = 0; q < 4; ++q) u[q] = diag ? Half<typename C::IO>::pack2(v[2 * q], v[2 * q + 1]) : 0u;
        Fa[m] = __builtin_bit_cast(typename C::F8, u);
    });
}

// Record of channel 8*kg + J of token row t (this lane's k-values of transform
// product J): elements 0..N-1 of the record, zeros after.
template <class C, int J>
__device__ __forceinline__ typename C::F8 read_record(const char* xex, int t, int kg) {
    constexpr int N = C::N;
    u32x4 e = {0u, 0u, 0u, 0u};
    if constexpr (N == 8) {
        e = *reinterpret_cast<const u32x4*>(xex + xpiece<C::XROT, C::XP, C::XPITCH>(t, 8 * kg + J) * 16);
    } else if constexpr (C::XALIGN) {
        // N = 2 or 4: a 4- or 8-byte record inside piece (2N c) / 16
        constexpr int per = 16 / (2 * N);                 // records per piece
        const int c = 8 * kg + J;
        const char* p = xex + xpiece<C::XROT, C::XP, C::XPITCH>(t, c / per) * 16 + (c % per) * (2 * N);
        if constexpr (N == 4) {
            const u32x2 v = *reinterpret_cast<const u32x2*>(p);
            e[0] = v[0];
            e[1] = v[1];
        } else {
            e[0] = *reinterpret_cast<const uint32_t*>(p);
        }
    } else {
        // contiguous rows: the record starts SH bytes into a dword
        constexpr int B0 = 2 * N * J;
        constexpr int SH = B0 % 4;
        constexpr int ND = (SH + 2 * N + 3) / 4;
        const uint32_t* d = reinterpret_cast<const uint32_t*>(xex + t * C::XPITCH * 16 + 16 * N * kg + (B0 - SH));
        uint32_t w[ND];
#pragma unroll
        for (int q = 0; q < ND; ++q) w[q] = d[q];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (2 * q + 1 < N) {
                e[q] = SH == 0 ? w[q] : __builtin_amdgcn_alignbit(w[q + 1], w[q], 16);
            } else if (2 * q < N) {
                e[q] = SH == 0 ? (w[q] & 0xffffu) : (w[q] >> 16);
            }
        }
    }
    return __builtin_bit_cast(typename C::F8, e);
}

__device__ __forceinline__ void mma_ab(f32x4& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_ab(f32x4& acc, const f16x8& a, const f16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}

template <class C>
__global__ __launch_bounds__(C::kThreads) void cn_mf_kernel(
    const typename C::IO* __restrict__ x, const typename C::IO* __restrict__ w_hat, typename C::IO* __restrict__ y,
    int64_t T, int C_in, int C_out, int n_c_tiles, uint32_t total_tiles, uint32_t w_bytes,
    int y_coalesced, Epi epi) {
    constexpr int N = C::N, XP = C::XP, MQ = C::MQ, CB = C::CB;
    constexpr int S = 2;
    using IO = typename C::IO;
    using F8 = typename C::F8;
    using BiasT = BiasTile<IO, C::CT, C::kThreads, C::LDS_BYTES, C::WAVES * C::YST_BYTES>;
    static_assert(BiasT::FITS, "room in LDS for the bias of the tile");
    __shared__ __attribute__((aligned(16))) char smem[BiasT::SMEM];
    float* lbias = reinterpret_cast<float*>(smem + BiasT::OFF);

    const uint32_t tile = xcd_remap(blockIdx.x, total_tiles);
    const int64_t t0 = (int64_t)(tile / n_c_tiles) * C::TT;
    const int o0 = (int)(tile % n_c_tiles) * C::CT;
    BiasT bias;
    // the wave index is uniform: held in a scalar register, LDS destinations of
    // the direct loads (M0) are then scalar arithmetic
    const int lane = (int)threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int kg = lane >> 4, tl = lane & 15;

    const uint32_t row_x = (uint32_t)C_in * (N * S), row_y = (uint32_t)C_out * (N * S);
    const int64_t rem = T - t0;
    const uint32_t rows = (uint32_t)(rem < C::TT ? rem : C::TT);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + t0 * C_in * N, rows * row_x);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(y + t0 * C_out * N, rows * row_y);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_hat, w_bytes);

    char* wbuf = smem;
    char* xex = smem + C::W_REGION + wave * C::XEX_BYTES;

    // x loads: load j, lane l fills slot s = 64 j + l of this wave's region,
    // i.e. row r = s / XPITCH at position s % XPITCH.  Rotated rows hold piece
    // (position - r) mod XP there; padded rows hold piece = position, and the
    // pad slots (and slots past the 16 rows) read nothing.
    uint32_t xoff[C::XDMA];
#pragma unroll
    for (int j = 0; j < C::XDMA; ++j) {
        const int sl = 64 * j + lane, r = sl / C::XPITCH, pos = sl % C::XPITCH;
        const int k = C::XROT ? (pos + XP - r % XP) % XP : pos;
        xoff[j] = (r < 16 && k < XP) ? (uint32_t)(wave * 16 + r) * row_x + (uint32_t)k * 16u : kOOB;
    }
    // DMA slot (it*WAVES + wave)*64 + lane: a plane holds 64*CB slots, so the
    // plane and the 16-row block of a wave instruction are wave-uniform
    uint32_t woff[C::DMA_ITERS];
#pragma unroll
    for (int it = 0; it < C::DMA_ITERS; ++it) {
        const int wi = it * C::WAVES + wave;
        const int p = wi / CB, blk = wi % CB;
        const int o = blk * 16 + (lane >> 2);
        const int qq = (lane & 3) ^ ((o >> 1) & 3);
        woff[it] = (o0 + o < C_out && p < N)
                       ? (((uint32_t)p * (uint32_t)C_out + (uint32_t)(o0 + o)) * (uint32_t)C_in + (uint32_t)(qq * C::R)) * S
                       : kOOB;
    }

    // Ragged shapes leave some w_hat tile slots unloaded (rows past C_out,
    // channels past C_in).  Clear both buffers once, so those slots hold finite
    // values: the transforms multiply every k-value, zero coefficients included.
    if ((C_in % C::KC) != 0 || (C_out % 16) != 0) {
        for (int i = (int)threadIdx.x; i < C::W_REGION / 16; i += C::kThreads)
            reinterpret_cast<u32x4*>(wbuf)[i] = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
    }

    F8 Fa[MQ];
    make_frags<C, false>(Fa);

    f32x4 acc[N][CB];

    const int nch = (C_in + C::KC - 1) / C::KC;
    const uint32_t chunk_x = (uint32_t)C::KC * (N * S);
    // Only a last, partial chunk needs per-lane masking of channels past C_in;
    // full chunks issue their loads with the precomputed offsets alone.
    auto dma_x = [&](int c) {
        if (c >= nch) return;
        if (c * C::KC + C::KC > C_in) {
            const uint32_t valid = (uint32_t)(C_in - c * C::KC) * (N * S);  // bytes of this chunk's rows
#pragma unroll
            for (int j = 0; j < C::XDMA; ++j) {
                const int sl = 64 * j + lane, pos = sl % C::XPITCH;
                const int k = C::XROT ? (pos + XP - (sl / C::XPITCH) % XP) % XP : pos;
                const uint32_t off = (uint32_t)k * 16u < valid ? xoff[j] : kOOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (__attribute__((address_space(3))) void*)(xex + j * 1024), 16, off, (uint32_t)c * chunk_x, 0, 0);
            }
        } else {
            // (the offsets pass through locals: an array element given straight
            // to the builtin makes the host compilation drop the kernel's stub)
#pragma unroll
            for (int j = 0; j < C::XDMA; ++j) {
                const uint32_t off = xoff[j];
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (__attribute__((address_space(3))) void*)(xex + j * 1024), 16, off, (uint32_t)c * chunk_x, 0, 0);
            }
        }
    };
    auto dma = [&](int c, char* buf) {
        if (c >= nch) return;
        if (c * C::KC + C::KC > C_in) {
            fast_dma_w<C>(rw, woff, (uint32_t)(c * C::KC * S), true, c * C::KC, C_in, buf);
        } else {
#pragma unroll
            for (int it = 0; it < C::DMA_ITERS; ++it) {
                const uint32_t off = woff[it];
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rw, (__attribute__((address_space(3))) void*)(buf + (it * C::WAVES + wave) * 1024), 16, off,
                    (uint32_t)(c * C::KC * S), 0, 0);
            }
        }
    };
    const int o_l = lane & 15;
    const int lane_off = (o_l * 4 + (kg ^ ((o_l >> 1) & 3))) * 16;
    auto ldW = [&](const char* buf, int p, int b) {
        return *reinterpret_cast<const F8*>(buf + p * C::CT * 64 + b * 1024 + lane_off);
    };

    // Frequency bins in product order: 0 (DC), 1..H (complex), Nyquist (even N).
    constexpr int H = (N - 1) / 2;
    constexpr int NB = 1 + H + (N % 2 == 0 ? 1 : 0);
    // w_hat fragments of bin s (re part; im part for complex bins), one bin ahead
    auto load_bin = [&](auto sc, const char* buf, F8(&Wr)[CB], F8(&Wi)[CB]) {
        constexpr int sb = decltype(sc)::value;
#pragma unroll
        for (int b = 0; b < CB; ++b) {
            if constexpr (sb == 0) {
                Wr[b] = ldW(buf, 0, b);
            } else if constexpr (sb <= H) {
                Wr[b] = ldW(buf, 2 * sb - 1, b);
                Wi[b] = ldW(buf, 2 * sb, b);
            } else {
                Wr[b] = ldW(buf, N - 1, b);
            }
        }
    };

    // Per chunk c: wait for w_hat chunk c and x chunk c (both in LDS); start
    // the w_hat loads of chunk c+1; read this wave's records and transform them
    // on the matrix cores; start the x loads of chunk c+1; channel products,
    // each bin's w_hat fragments read while the previous bin multiplies.
#pragma unroll
    for (int p = 0; p < N; ++p)
#pragma unroll
        for (int b = 0; b < CB; ++b) acc[p][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    dma(0, wbuf);
    dma_x(0);
    // the bias slice is its own: fetch and publish it now, after the first
    // stage's loads (the wait for the bias load then overlaps the wait for that
    // stage, which the loop does first); the loop's barriers order it before
    // the epilogue's reads, and no register carries it through the loop
    if (BiasT::OWN && epi.bias != nullptr) {
        bias.fetch(epi, o0, C_out);
        bias.publish(lbias);
    }
    for (int c = 0; c < nch; ++c) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        dma(c + 1, wbuf + ((c + 1) & 1) * C::BUF_BYTES);
        const char* buf = wbuf + (c & 1) * C::BUF_BYTES;

        // records of channels 8kg + j (j = 0..7) of token tl
        F8 rec[8];
        static_for<0, 8>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            rec[j] = read_record<C, j>(xex, tl, kg);
        });
        __builtin_amdgcn_sched_barrier(0);
        if (c * C::KC + C::KC > C_in) {  // channel tail: records past C_in are zero
            const int left = C_in - c * C::KC;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (8 * kg + j >= left) rec[j] = F8{};
        }
        // transform: Xh[p] = planes p of channels 8kg .. 8kg+7, token tl
        F8 Xh[N];
        {
            uint32_t pk[N][4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                f32x4 d0[MQ], d1[MQ];
#pragma unroll
                for (int m = 0; m < MQ; ++m) {
                    d0[m] = f32x4{0.f, 0.f, 0.f, 0.f};
                    d1[m] = f32x4{0.f, 0.f, 0.f, 0.f};
                    mma_ab(d0[m], Fa[m], rec[2 * jj]);
                    mma_ab(d1[m], Fa[m], rec[2 * jj + 1]);
                }
#pragma unroll
                for (int p = 0; p < N; ++p) pk[p][jj] = Half<IO>::pack2(d0[p / 4][p % 4], d1[p / 4][p % 4]);
            }
#pragma unroll
            for (int p = 0; p < N; ++p) {
                const u32x4 v = {pk[p][0], pk[p][1], pk[p][2], pk[p][3]};
                Xh[p] = __builtin_bit_cast(F8, v);
            }
        }
        // the records are consumed: the exchange rows may be refilled
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        dma_x(c + 1);
        F8 Wr[2][CB], Wi[2][CB];
        load_bin(std::integral_constant<int, 0>{}, buf, Wr[0], Wi[0]);
        __builtin_amdgcn_sched_barrier(0);

        static_for<0, NB>([&](auto sc) {
            constexpr int sb = decltype(sc)::value;
            constexpr int cur = sb & 1, nxt = cur ^ 1;
            if constexpr (sb + 1 < NB) load_bin(std::integral_constant<int, sb + 1>{}, buf, Wr[nxt], Wi[nxt]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (sb == 0) {
#pragma unroll
                for (int b = 0; b < CB; ++b) mma_ab(acc[0][b], Wr[cur][b], Xh[0]);
            } else if constexpr (sb <= H) {
                constexpr int pr = 2 * sb - 1, pi = 2 * sb;
                const F8 nXi = neg(Xh[pi]);
#pragma unroll
                for (int b = 0; b < CB; ++b) mma_ab(acc[pr][b], Wr[cur][b], Xh[pr]);
#pragma unroll
                for (int b = 0; b < CB; ++b) mma_ab(acc[pi][b], Wi[cur][b], Xh[pr]);
#pragma unroll
                for (int b = 0; b < CB; ++b) mma_ab(acc[pr][b], Wi[cur][b], nXi);
#pragma unroll
                for (int b = 0; b < CB; ++b) mma_ab(acc[pi][b], Wr[cur][b], Xh[pi]);
            } else {
#pragma unroll
                for (int b = 0; b < CB; ++b) mma_ab(acc[N - 1][b], Wr[cur][b], Xh[N - 1]);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    }

    // Epilogue.  Lane (tl, kg) holds token tl and output channels 16b + 4kg + i.
    if (y_coalesced) {
        __syncthreads();  // the staging area overlaps the tile and exchange buffers
        if (!BiasT::OWN && epi.bias != nullptr) {
            bias.fetch(epi, o0, C_out);
            bias.publish(lbias);
            __syncthreads();
        }
        char* yst = smem + wave * C::YST_BYTES;
        F8 Ga[MQ];
        make_frags<C, true>(Ga);
#pragma unroll
        for (int b = 0; b < CB; ++b) {
            // records of channels 16b+4kg .. +3 of token tl: 4N bf16 = 2N dwords.
            // Channel 16b+4kg+i: its N planes (rounded to bf16) are this lane's
            // k-values of inverse product i; product (i, m) returns its group
            // elements 4m .. 4m+3.
            float flat[4 * N];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u32x4 bu;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float lo = 2 * q < N ? acc[2 * q < N ? 2 * q : 0][b][i] : 0.f;
                    const float hi = 2 * q + 1 < N ? acc[2 * q + 1 < N ? 2 * q + 1 : 0][b][i] : 0.f;
                    bu[q] = Half<IO>::pack2(lo, hi);
                }
                const F8 Bv = __builtin_bit_cast(F8, bu);
#pragma unroll
                for (int m = 0; m < MQ; ++m) {
                    f32x4 d = {0.f, 0.f, 0.f, 0.f};
                    mma_ab(d, Ga[m], Bv);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (4 * m + r < N) flat[i * N + 4 * m + r] = d[r];
                }
            }
            if (epi_on(epi)) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    epi_apply<N>(flat + i * N, epi.bias != nullptr ? lbias[16 * b + 4 * kg + i] : 0.0f, epi.act);
            }
            uint32_t pk[2 * N];
#pragma unroll
            for (int q = 0; q < 2 * N; ++q) pk[q] = Half<IO>::pack2(flat[2 * q], flat[2 * q + 1]);
            // 8N bytes at byte (16b + 4kg) * 2N of row tl: N dword pairs, each
            // inside one 16-byte piece
            const int byte0 = (16 * b + 4 * kg) * 2 * N;
#pragma unroll
            for (int q = 0; q < N; ++q) {
                const int by = byte0 + 8 * q;
                *reinterpret_cast<u32x2*>(yst + xpiece<C::YROT, C::YP, C::YPITCH>(tl, by / 16) * 16 + (by % 16)) =
                    u32x2{pk[2 * q], pk[2 * q + 1]};
            }
        }
        // LPR lanes per tile row: lane (r = lane / LPR, u = lane % LPR) stores
        // pieces u, u + LPR, ... of rows r, r + 64/LPR, ...: every instruction
        // writes 64/LPR rows x 16 LPR contiguous bytes, with no per-piece index
        // arithmetic beyond the rotation's single wrap.
        constexpr int LPR = EQL_MF_STORE_LPR, RPI = 64 / LPR, RG = 16 / RPI;
        constexpr int NIT = (C::YP + LPR - 1) / LPR;
        const uint32_t cols = (uint32_t)(C_out - o0) * (N * S);  // valid bytes of a tile row
        const bool full = cols >= (uint32_t)(C::YP * 16);
        const int r_in = lane / LPR, u = lane % LPR;
        constexpr int G = 6;  // LDS reads issued ahead of their stores
        auto store_rows = [&](auto fullc) {
            constexpr bool FULL = decltype(fullc)::value;
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                const int r = rg * RPI + r_in;
                const uint32_t gbase =
                    (uint32_t)(wave * 16 + r) * row_y + (uint32_t)o0 * (N * S) + (uint32_t)u * 16u;
                const char* lrow = yst + r * C::YPITCH * 16;
                const int rot0 = C::YROT ? (u + r) % C::YP : u;  // rotated position of piece u
#pragma unroll
                for (int i0 = 0; i0 < NIT; i0 += G) {
                    u32x4 v[G];
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const int it = i0 + g;
                        if (it < NIT) {
                            int pos = rot0 + LPR * it;
                            if constexpr (C::YROT) pos = pos >= C::YP ? pos - C::YP : pos;
                            v[g] = *reinterpret_cast<const u32x4*>(lrow + pos * 16);
                        }
                    }
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const int it = i0 + g;
                        if (it < NIT) {
                            const uint32_t k = (uint32_t)(u + LPR * it);
                            // pieces past the row (YP not a multiple of LPR) and
                            // columns past C_out are dropped by an out-of-range offset
                            const bool ok = (C::YP % LPR == 0 || it < NIT - 1 || k < (uint32_t)C::YP) &&
                                            (FULL || k * 16u < cols);
                            __builtin_amdgcn_raw_buffer_store_b128(v[g], ry, ok ? gbase + 16u * LPR * it : kOOB, 0,
                                                                   kYStoreAux);
                        }
                    }
                }
            }
        };
        if (full) store_rows(std::true_type{});
        else store_rows(std::false_type{});
    } else {
        if (!BiasT::OWN && epi.bias != nullptr) {
            __syncthreads();
            bias.fetch(epi, o0, C_out);
            bias.publish(lbias);
            __syncthreads();
        }
        const uint32_t trow = (uint32_t)(wave * 16 + tl);
#pragma unroll
        for (int b = 0; b < CB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int o = o0 + 16 * b + 4 * kg + i;
                const uint32_t off = o < C_out ? trow * row_y + (uint32_t)o * (N * S) : kOOB;
                float P[N], yv[N];
#pragma unroll
                for (int p = 0; p < N; ++p) P[p] = acc[p][b][i] * (float)N;  // the spectrum of y/N
                rdft_inverse<N>(P, yv);
                if (epi_on(epi)) epi_apply<N>(yv, epi.bias != nullptr ? lbias[o - o0] : 0.0f, epi.act);
#pragma unroll
                for (int e = 0; e < N; ++e)
                    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(Half<IO>::pack2(yv[e], 0.f) & 0xffffu), ry,
                                                         off + 2u * e, 0, 0);
            }
    }
}

// --- host side ----------------------------------------------------------------------

template <class C>
hipError_t launch_mf_cfg(const void* x, const void* w_hat, void* y, int64_t T, int C_in, int C_out,
                         hipStream_t stream, Epi epi) {
    const int64_t n_t = (T + C::TT - 1) / C::TT;
    const int n_c = (C_out + C::CT - 1) / C::CT;
    const int64_t total = n_t * n_c;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    const int64_t w_bytes = (int64_t)C::N * C_out * C_in * 2;
    const int y_coalesced = ((int64_t)C_out * C::N * 2) % 16 == 0;
    hipLaunchKernelGGL((cn_mf_kernel<C>), dim3((uint32_t)total), dim3(C::kThreads), 0, stream,
                       (const typename C::IO*)x, (const typename C::IO*)w_hat, (typename C::IO*)y, T, C_in, C_out, n_c,
                       (uint32_t)total, (uint32_t)w_bytes, y_coalesced, epi);
    return hipGetLastError();
}

template <int N, typename IO>
constexpr bool mf_supported = (std::is_same_v<IO, __bf16> || std::is_same_v<IO, _Float16>) && N >= 2 && N <= 8;

// Largest output-block count <= CB whose LDS fits the CU and whose
// accumulators stay within 192 registers per lane.
template <int N, int W, int CB>
constexpr int mf_cap() {
    if constexpr (CB <= 1) return 1;
    else if constexpr (MfCfg<N, W, CB>::LDS_BYTES <= 163840 && 4 * N * CB <= 192) return CB;
    else return mf_cap<N, W, CB - 1>();
}  // (the LDS layout is the same for both 16-bit types)

// Menu entry I (same shapes as FusedMenu) on the matrix-core transform kernel;
// shapes it cannot take (ragged C_in, huge rows) go to the fused kernel.
template <int N, typename IO, int I>
hipError_t launch_mf_entry(const void* x, const void* w_hat, void* y, int64_t T, int C_in, int C_out,
                           hipStream_t stream, Epi epi) {
    constexpr int W = FusedMenu<N, IO>::waves[I];
    constexpr int CB = mf_cap<N, W, FusedMenu<N, IO>::cb[I]>();
    using Cfg = MfCfg<N, W, CB, IO>;
    if (fast_ok<N, IO>(C_in, C_out, Cfg::TT))
        return launch_mf_cfg<Cfg>(x, w_hat, y, T, C_in, C_out, stream, epi);
    return launch_menu_entry<N, IO, I>(x, w_hat, y, T, C_in, C_out, stream, epi);
}

}  // namespace eql
