// cn_split.h -- fp32 C_N forward with the input channels split over waves.
//
// Same computation as the fused kernels ("Flash EQ-Linear", Algorithmic Approach
// and Implementation: real DFT along the group axis, per-frequency channel
// products over the kept bins, inverse DFT, all in one launch), arranged for
// layers too small to give every SIMD a wave when one wave owns a 16-token x
// 16-channel tile (few tokens, few output channels; fp32 products on the matrix
// cores run at 1/16 of the bf16 rate, so they dominate such layers).
//
// A workgroup owns 16 tokens and CT = 16*OB output channels.  Its OB*KS waves
// each take one 16-channel output block and one of KS slices of every step of
// input channels: a wave loads (through a shared, coalesced LDS tile) and
// transforms only its slice of the x records, and multiplies it with its block's
// weights.  The KS partial spectra of a block are then summed through LDS in a
// fixed order (each wave finishes 4/KS of the accumulator rows of its block),
// inverse-transformed, staged in LDS and written as contiguous 16-byte pieces.
//
// Grids of a few workgroups (XD) are pure latency: there every lane loads its
// own records (R channels of one token, R N contiguous floats) straight into
// registers, with no LDS tile and no barrier before the transform, and writes
// its N outputs of a token from registers as 16-byte pieces when N % 4 == 0.
// (Measured on MI355X, cache-cold: the C4 layer of 64 tokens x 8 channels
// 2.74 -> 2.27 us; the C8 layer of 4096 tokens x 32 channels, 256 workgroups,
// 5.72 -> 5.95 us, where the per-lane loads touch eight times the cache lines
// of the coalesced tile: it keeps the tile.)
//
// Complex bins use three real products instead of four (Gauss's method):
//   t1 = Xr Wr^T, t2 = Xi Wi^T, t3 = (Xr + Xi)(Wr + Wi)^T,
//   Re = t1 - t2, Im = t3 - t1 - t2.
#pragma once

#include "cn_fused.h"

namespace eql {

#ifndef EQL_SPLIT_GAUSS
#define EQL_SPLIT_GAUSS 1
#endif

template <int N_, int OB_, int KS_, int R_, bool XD_ = false>
struct SplitCfg {
    static constexpr int N = N_, OB = OB_, KS = KS_, R = R_;
    static constexpr bool XD = XD_;  // records straight into registers (few workgroups)
    static constexpr int H = (N - 1) / 2;  // complex bins
    static constexpr bool GAUSS = EQL_SPLIT_GAUSS != 0 && H > 0;
    static constexpr int kWaves = OB * KS, kThreads = 64 * kWaves;
    static constexpr int TT = 16, CT = 16 * OB;
    static constexpr int KW = 4 * R;          // channels of one wave per step (R per lane)
    static constexpr int KSTEP = KS * KW;     // channels per step
    static constexpr int XP = KSTEP * N / 4;  // 16-byte pieces of one token row of a step
    static constexpr bool XROT = XP % 8 == 0;
    static constexpr int XPITCH = XROT ? XP : (XP | 1);
    static constexpr int XBUF = 16 * XPITCH * 16;
    static constexpr int XL = (16 * XP + kThreads - 1) / kThreads;  // x loads per thread per step
    // XD: a lane's records of one step, R N contiguous floats, 16-byte aligned
    // for R = 4 (8-byte for R = 2), loaded 16 or 8 bytes at a time
    static constexpr int RF = R * N;
    static constexpr int XW = R == 4 ? 4 : 2;
    static constexpr int XLD = RF / XW;
    static constexpr int ROWS = 4 / KS;                // accumulator rows each wave finishes
    static constexpr int RED = N * 64 * 16;            // one wave's partial spectra: N f32x4 per lane
    static constexpr bool YDIRECT = XD_ && N % 4 == 0;  // y stored from registers
    static constexpr int YROW = CT * N * 4;
    static constexpr int YP = YROW / 16;
    static constexpr bool YROT = YP % 8 == 0;
    static constexpr int YPITCH = YROT ? YP : (YP | 1);
    static constexpr int YST = YDIRECT ? 0 : 16 * YPITCH * 16;
    static constexpr int XTILES = XD_ ? 0 : 2 * XBUF;
    // the y staging overlaps the x tiles (both at offset 0); the partials follow
    static constexpr int PART_OFF = XTILES > YST ? XTILES : YST;
    // the tile's bias (fp32) has a slice of its own when that keeps as many
    // workgroups per CU; otherwise each lane fetches its one value in the epilogue
    static constexpr int BIAS_OFF = PART_OFF + kWaves * RED;
    static constexpr int BIAS_BYTES = (CT * 4 + 15) / 16 * 16;
    static constexpr bool BIAS_OWN = lds_groups(BIAS_OFF + BIAS_BYTES) == lds_groups(BIAS_OFF);
    static constexpr int LDS = BIAS_OFF + (BIAS_OWN ? BIAS_BYTES : 0);
    static_assert(LDS <= 163840, "the CU's LDS");
    static_assert(4 % KS == 0, "KS divides the 4 accumulator rows");
    static_assert(R == 2 || R == 4, "two or four channels per lane");
    static_assert(YROW % 16 == 0, "tile rows are whole pieces");
};

// LDS barrier without the wait on outstanding global loads that __syncthreads
// implies (those loads are the next step's prefetch).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <class C>
__global__ __launch_bounds__(C::kThreads) void cn_split_kernel(
    const float* __restrict__ x, const float* __restrict__ w_hat, float* __restrict__ y, int64_t T,
    int C_in, int C_out, int n_c_tiles, uint32_t total_tiles, uint32_t w_bytes, int y_coalesced,
    Epi epi) {
    constexpr int N = C::N, R = C::R, H = C::H, XP = C::XP;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];

    const uint32_t tile = xcd_remap(blockIdx.x, total_tiles);
    const int64_t t0 = (int64_t)(tile / n_c_tiles) * C::TT;
    const int o0 = (int)(tile % n_c_tiles) * C::CT;
    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ob = wave % C::OB, kh = wave / C::OB;
    const int q = lane >> 4, l16 = lane & 15;

    const uint32_t row_x = (uint32_t)C_in * (N * 4), row_y = (uint32_t)C_out * (N * 4);
    const int64_t rem = T - t0;
    const uint32_t rows = (uint32_t)(rem < C::TT ? rem : C::TT);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + t0 * C_in * N, rows * row_x);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(y + t0 * C_out * N, rows * row_y);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_hat, w_bytes);

    const int steps = (C_in + C::KSTEP - 1) / C::KSTEP;
    const uint32_t step_x = (uint32_t)C::KSTEP * (N * 4);

    // x tile of a step: piece pc = tid + j*kThreads is piece k of token row r
    uint32_t xoff[C::XL];
#pragma unroll
    for (int j = 0; j < C::XL; ++j) {
        const int pc = tid + j * C::kThreads, r = pc / XP, k = pc % XP;
        xoff[j] = pc < 16 * XP ? (uint32_t)r * row_x + (uint32_t)k * 16u : kOOB;
    }
    auto load_x = [&](int s, u32x4 (&xr)[C::XL]) {
        const int left = C_in - s * C::KSTEP;  // channels of this step that exist
        const uint32_t valid = left > 0 ? (uint32_t)left * (N * 4) : 0u;
#pragma unroll
        for (int j = 0; j < C::XL; ++j) {
            const int k = (tid + j * C::kThreads) % XP;
            const uint32_t off = (uint32_t)k * 16u < valid ? xoff[j] : kOOB;
            xr[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, (uint32_t)s * step_x, 0);
        }
    };
    // XD: this lane's records of step s are token row l16, channels
    // s KSTEP + ch_lane .. + R-1.  C_in is a multiple of four, so the R channels
    // of a lane are all inside C_in or all past it; rows past T lie past the
    // resource.  Either way the loads return zeros.
    const int ch_lane = kh * C::KW + q * R;
    constexpr int XR = C::XD ? C::RF : 1;
    auto load_xd = [&](int s, float (&xv)[XR]) {
        if constexpr (C::XD) {
            const uint32_t off = s * C::KSTEP + ch_lane < C_in ? (uint32_t)l16 * row_x + (uint32_t)ch_lane * (N * 4)
                                                                : kOOB;
            const uint32_t soff = (uint32_t)s * step_x;
#pragma unroll
            for (int j = 0; j < C::XLD; ++j) {
                if constexpr (C::XW == 4) {
                    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16u * j, soff, 0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) xv[4 * j + e] = __uint_as_float(v[e]);
                } else {
                    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rx, off + 8u * j, soff, 0);
                    xv[2 * j] = __uint_as_float(v[0]);
                    xv[2 * j + 1] = __uint_as_float(v[1]);
                }
            }
        }
    };

    // B fragments (weights): lane (column l16, k-group q) holds channels
    // ch .. ch+R-1 of output row orow in every plane
    const int orow = o0 + ob * 16 + l16;
    const uint32_t plane_w = (uint32_t)C_out * (uint32_t)C_in * 4u;
    const uint32_t wbase = (uint32_t)orow * (uint32_t)C_in * 4u + (uint32_t)ch_lane * 4u;
    auto load_w = [&](int s, float (&B)[N][R]) {
        const bool ok = orow < C_out && s * C::KSTEP + ch_lane < C_in;
        const uint32_t soff = (uint32_t)(s * C::KSTEP) * 4u;
#pragma unroll
        for (int p = 0; p < N; ++p) {
            const uint32_t off = ok ? wbase + (uint32_t)p * plane_w : kOOB;
            if constexpr (R == 4) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rw, off, soff, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) B[p][r] = __uint_as_float(v[r]);
            } else {
                const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rw, off, soff, 0);
                B[p][0] = __uint_as_float(v[0]);
                B[p][1] = __uint_as_float(v[1]);
            }
        }
    };

    f32x4 acc[N];
    f32x4 gs[H > 0 ? H : 1];  // Gauss: (Xr + Xi)(Wr + Wi) per complex bin
#pragma unroll
    for (int p = 0; p < N; ++p) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < (H > 0 ? H : 1); ++k) gs[k] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 xr[C::XD ? 1 : C::XL];
    float X0[XR], X1[XR];
    float B0[N][R], B1[N][R];
    if constexpr (C::XD) load_xd(0, X0);
    else load_x(0, xr);
    __builtin_amdgcn_sched_barrier(0);  // x first: it is needed first
    load_w(0, B0);
    // The tile's bias to its LDS slice, fetched after the first step's loads (the
    // wait for it overlaps theirs); the loop's barriers order it before the
    // epilogue's reads, and no register carries it through the loop.
    float* lbias = reinterpret_cast<float*>(smem + C::BIAS_OFF);
    if (C::BIAS_OWN && epi.bias != nullptr && tid < C::CT)
        lbias[tid] = bias_value<float>(bias_fetch<float>(epi, C_out, o0 + tid));

    // One step with weights B; the next step's weights load into Bnext.  VALU
    // work placed between fp32 MFMAs stretches each of them by about half, so
    // everything the products read (transforms, Gauss sums) is computed first
    // and the products issue as one uninterrupted run.
    auto step = [&](int s, const float (&B)[N][R], float (&Bnext)[N][R], const float (&X)[XR], float (&Xn)[XR]) {
        // this lane's records: token row l16, channels ch_lane .. ch_lane+R-1
        float rec[R * N];
        if constexpr (C::XD) {
            if (s + 1 < steps) {
                load_xd(s + 1, Xn);
                load_w(s + 1, Bnext);
            }
#pragma unroll
            for (int j = 0; j < R * N; ++j) rec[j] = X[j];
        } else {
        char* xbuf = smem + (s & 1) * C::XBUF;
#pragma unroll
        for (int j = 0; j < C::XL; ++j) {
            const int pc = tid + j * C::kThreads;
            if (16 * XP % C::kThreads != 0 && pc >= 16 * XP) continue;
            *reinterpret_cast<u32x4*>(xbuf + xpiece<C::XROT, XP, C::XPITCH>(pc / XP, pc % XP) * 16) = xr[j];
        }
        // next step's loads (past the last step: offsets out of range, no access)
        load_x(s + 1, xr);
        if (s + 1 < steps) load_w(s + 1, Bnext);
        lds_barrier();

        const int byte0 = ch_lane * N * 4;
        if constexpr ((R * N) % 4 == 0) {
#pragma unroll
            for (int j = 0; j < R * N / 4; ++j) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(
                    xbuf + xpiece<C::XROT, XP, C::XPITCH>(l16, byte0 / 16 + j) * 16);
#pragma unroll
                for (int e = 0; e < 4; ++e) rec[4 * j + e] = __uint_as_float(v[e]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < R * N / 2; ++j) {
                const int b = byte0 + 8 * j;
                const u32x2 v = *reinterpret_cast<const u32x2*>(
                    xbuf + xpiece<C::XROT, XP, C::XPITCH>(l16, b / 16) * 16 + (b % 16));
                rec[2 * j] = __uint_as_float(v[0]);
                rec[2 * j + 1] = __uint_as_float(v[1]);
            }
        }
        }
        float A[N][R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float xv[N], P[N];
#pragma unroll
            for (int h = 0; h < N; ++h) xv[h] = rec[r * N + h];
            rdft_forward<N>(xv, P);
#pragma unroll
            for (int p = 0; p < N; ++p) A[p][r] = P[p];
        }
        constexpr int HG = H > 0 ? H : 1;
        float SA[HG][R], SB[HG][R];  // Gauss: Xr + Xi and Wr + Wi per complex bin (else -Xi in SA)
        if constexpr (C::GAUSS) {
#pragma unroll
            for (int k = 1; k <= H; ++k)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    SA[k - 1][r] = A[2 * k - 1][r] + A[2 * k][r];
                    SB[k - 1][r] = B[2 * k - 1][r] + B[2 * k][r];
                }
        } else {
#pragma unroll
            for (int k = 1; k <= H; ++k)
#pragma unroll
                for (int r = 0; r < R; ++r) SA[k - 1][r] = -A[2 * k][r];
        }
        __builtin_amdgcn_sched_barrier(0);

        // products: consecutive MFMAs go to different accumulators
#pragma unroll
        for (int r = 0; r < R; ++r) {
            acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(A[0][r], B[0][r], acc[0], 0, 0, 0);
            if constexpr (N % 2 == 0 && N > 1)
                acc[N - 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(A[N - 1][r], B[N - 1][r], acc[N - 1], 0, 0, 0);
#pragma unroll
            for (int k = 1; k <= H; ++k) {
                const int pr = 2 * k - 1, pi = 2 * k;
                if constexpr (C::GAUSS) {
                    acc[pr] = __builtin_amdgcn_mfma_f32_16x16x4f32(A[pr][r], B[pr][r], acc[pr], 0, 0, 0);
                    acc[pi] = __builtin_amdgcn_mfma_f32_16x16x4f32(A[pi][r], B[pi][r], acc[pi], 0, 0, 0);
                    gs[k - 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(SA[k - 1][r], SB[k - 1][r], gs[k - 1], 0, 0, 0);
                } else {
                    // Yr += Xr Wr - Xi Wi, Yi += Xr Wi + Xi Wr (SA holds -Xi)
                    acc[pr] = __builtin_amdgcn_mfma_f32_16x16x4f32(A[pr][r], B[pr][r], acc[pr], 0, 0, 0);
                    acc[pi] = __builtin_amdgcn_mfma_f32_16x16x4f32(A[pr][r], B[pi][r], acc[pi], 0, 0, 0);
                    acc[pr] = __builtin_amdgcn_mfma_f32_16x16x4f32(SA[k - 1][r], B[pi][r], acc[pr], 0, 0, 0);
                    acc[pi] = __builtin_amdgcn_mfma_f32_16x16x4f32(A[pi][r], B[pr][r], acc[pi], 0, 0, 0);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // C_in >= 1: at least one step, no branch ahead of the first loads; the two
    // weight buffers alternate without register copies
    for (int s = 0;;) {
        step(s, B0, B1, X0, X1);
        if (++s >= steps) break;
        step(s, B1, B0, X1, X0);
        if (++s >= steps) break;
    }
    if constexpr (C::GAUSS) {
#pragma unroll
        for (int k = 1; k <= H; ++k) {
            const f32x4 t1 = acc[2 * k - 1], t2 = acc[2 * k];
            acc[2 * k - 1] = t1 - t2;
            acc[2 * k] = gs[k - 1] - t1 - t2;
        }
    }

    // Sum the KS partial spectra of each block through LDS: every wave leaves
    // its accumulators there ([plane][lane], 16 bytes each), and row i is
    // finished by the wave with kh == i / ROWS, adding the KS partials in order
    // (no per-lane selects).  The partials have a region of their own, so they
    // are written as soon as the products are done; the barrier after them also
    // ends every wave's use of the x tiles, which the y staging then overwrites.
    {
        f32x4* mine = reinterpret_cast<f32x4*>(smem + C::PART_OFF + wave * C::RED);
#pragma unroll
        for (int p = 0; p < N; ++p) mine[p * 64 + lane] = acc[p];
    }
    __syncthreads();
    // this lane's bias: from the slice, or fetched now (its latency overlaps the sums)
    float bias_v = 0.0f;
    if (epi.bias != nullptr) {
        if constexpr (C::BIAS_OWN) bias_v = lbias[orow - o0];
        else bias_v = bias_value<float>(bias_fetch<float>(epi, C_out, orow));
    }
    const float* red =
        reinterpret_cast<const float*>(smem + C::PART_OFF) + ob * (C::RED / 4) + lane * 4 + kh * C::ROWS;
    float P[C::ROWS][N];
#pragma unroll
    for (int p = 0; p < N; ++p) {
        float v[C::ROWS];
#pragma unroll
        for (int src = 0; src < C::KS; ++src) {
            const float* pp = red + src * C::OB * (C::RED / 4) + p * 256;
            float u[C::ROWS];
            if constexpr (C::ROWS == 2) {
                const f32x2 t = *reinterpret_cast<const f32x2*>(pp);
                u[0] = t[0];
                u[1] = t[1];
            } else {
#pragma unroll
                for (int ii = 0; ii < C::ROWS; ++ii) u[ii] = pp[ii];
            }
#pragma unroll
            for (int ii = 0; ii < C::ROWS; ++ii) v[ii] = src == 0 ? u[ii] : v[ii] + u[ii];
        }
#pragma unroll
        for (int ii = 0; ii < C::ROWS; ++ii) P[ii][p] = v[ii];
    }

    // Epilogue: inverse DFT of each finished (token, channel) record, y written once.
    if constexpr (C::YDIRECT) {
        // N contiguous floats per lane, stored as 16-byte pieces
#pragma unroll
        for (int ii = 0; ii < C::ROWS; ++ii) {
            const uint32_t tl = (uint32_t)(q * 4 + kh * C::ROWS + ii);
            const uint32_t off = orow < C_out ? tl * row_y + (uint32_t)orow * (N * 4) : kOOB;
            float yv[N];
            rdft_inverse<N>(P[ii], yv);
            if (epi_on(epi)) epi_apply<N>(yv, bias_v, epi.act);
#pragma unroll
            for (int j = 0; j < N / 4; ++j)
                __builtin_amdgcn_raw_buffer_store_b128(
                    u32x4{__float_as_uint(yv[4 * j]), __float_as_uint(yv[4 * j + 1]), __float_as_uint(yv[4 * j + 2]),
                          __float_as_uint(yv[4 * j + 3])},
                    ry, off + 16u * j, 0, kYStoreAux);
        }
    } else if (y_coalesced) {
        char* yst = smem;
#pragma unroll
        for (int ii = 0; ii < C::ROWS; ++ii) {
            const int tl = q * 4 + kh * C::ROWS + ii, ol = ob * 16 + l16;
            float yv[N];
            rdft_inverse<N>(P[ii], yv);
            if (epi_on(epi)) epi_apply<N>(yv, bias_v, epi.act);
            const int byte0 = ol * N * 4;
            if constexpr (N % 4 == 0) {
#pragma unroll
                for (int j = 0; j < N / 4; ++j)
                    *reinterpret_cast<u32x4*>(yst + xpiece<C::YROT, C::YP, C::YPITCH>(tl, byte0 / 16 + j) * 16) =
                        u32x4{__float_as_uint(yv[4 * j]), __float_as_uint(yv[4 * j + 1]),
                              __float_as_uint(yv[4 * j + 2]), __float_as_uint(yv[4 * j + 3])};
            } else {
#pragma unroll
                for (int e = 0; e < N; ++e) {
                    const int b = byte0 + 4 * e;
                    *reinterpret_cast<float*>(yst + xpiece<C::YROT, C::YP, C::YPITCH>(tl, b / 16) * 16 + (b % 16)) =
                        yv[e];
                }
            }
        }
        __syncthreads();
        const int left = C_out - o0;
        const uint32_t cols = (uint32_t)(left < C::CT ? left : C::CT) * (N * 4);  // valid bytes of a tile row
        for (int pc = tid; pc < 16 * C::YP; pc += C::kThreads) {
            const int r = pc / C::YP, k = pc % C::YP;
            const u32x4 v = *reinterpret_cast<const u32x4*>(yst + xpiece<C::YROT, C::YP, C::YPITCH>(r, k) * 16);
            const uint32_t off = (uint32_t)k * 16u < cols
                                     ? (uint32_t)r * row_y + (uint32_t)o0 * (N * 4) + (uint32_t)k * 16u
                                     : kOOB;
            __builtin_amdgcn_raw_buffer_store_b128(v, ry, off, 0, kYStoreAux);
        }
    } else {
#pragma unroll
        for (int ii = 0; ii < C::ROWS; ++ii) {
            const uint32_t tl = (uint32_t)(q * 4 + kh * C::ROWS + ii);
            const uint32_t off = orow < C_out ? tl * row_y + (uint32_t)orow * (N * 4) : kOOB;
            float yv[N];
            rdft_inverse<N>(P[ii], yv);
            if (epi_on(epi)) epi_apply<N>(yv, bias_v, epi.act);
#pragma unroll
            for (int e = 0; e < N; ++e)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv[e]), ry, off + 4u * e, 0, 0);
        }
    }
}

// Whole 16-byte pieces of x rows and 32-bit buffer offsets.
template <int N>
bool split_ok(int C_in, int C_out) {
    const int64_t lim = (int64_t)1 << 30;
    return C_in % 4 == 0 && (int64_t)N * C_out * C_in * 4 < lim && (int64_t)16 * C_in * N * 4 < lim &&
           (int64_t)16 * C_out * N * 4 < lim;
}

template <class C>
hipError_t launch_split_cfg(const void* x, const void* w_hat, void* y, int64_t T, int C_in, int C_out,
                            hipStream_t stream, Epi epi) {
    const int64_t n_t = (T + C::TT - 1) / C::TT;
    const int n_c = (C_out + C::CT - 1) / C::CT;
    const int64_t total = n_t * n_c;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    const int64_t w_bytes = (int64_t)C::N * C_out * C_in * 4;
    const int y_coalesced = ((int64_t)C_out * C::N * 4) % 16 == 0;
    hipLaunchKernelGGL((cn_split_kernel<C>), dim3((uint32_t)total), dim3(C::kThreads), 0, stream,
                       (const float*)x, (const float*)w_hat, (float*)y, T, C_in, C_out, n_c, (uint32_t)total,
                       (uint32_t)w_bytes, y_coalesced, epi);
    return hipGetLastError();
}

// Grids below this many workgroups take the register-loaded form (XD).
constexpr int64_t kSplitDirectBelow = 128;

// KS input-channel slices: 2 (four channels per lane up to N = 8, else two) or
// 4 (two per lane); one output block per workgroup when C_out fits in 16
// channels, else two.
template <int N, int KS>
hipError_t launch_split(const void* x, const void* w_hat, void* y, int64_t T, int C_in, int C_out,
                        hipStream_t stream, Epi epi) {
    constexpr int R = (KS == 2 && N <= 8) ? 4 : 2;
    const int OB = C_out <= 16 ? 1 : 2;
    const int64_t total = (T + 15) / 16 * ((C_out + 16 * OB - 1) / (16 * OB));
    if (total < kSplitDirectBelow) {
        if (OB == 1) return launch_split_cfg<SplitCfg<N, 1, KS, R, true>>(x, w_hat, y, T, C_in, C_out, stream, epi);
        return launch_split_cfg<SplitCfg<N, 2, KS, R, true>>(x, w_hat, y, T, C_in, C_out, stream, epi);
    }
    if (OB == 1) return launch_split_cfg<SplitCfg<N, 1, KS, R>>(x, w_hat, y, T, C_in, C_out, stream, epi);
    return launch_split_cfg<SplitCfg<N, 2, KS, R>>(x, w_hat, y, T, C_in, C_out, stream, epi);
}

}  // namespace eql
