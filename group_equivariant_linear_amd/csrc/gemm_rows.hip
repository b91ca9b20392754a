// gemm_rows.hip -- row-wise products y[t][ycol+n] = sum_k W[n][k] x[t][xcol+k] on
// gfx950 MFMA, for a small table of independent jobs in one launch.
//
// Used by
//  - the D8 Fourier-domain layer ("Quick ViTs", key design 2): jobs A1, A2,
//    B1, B2 (C/8 x C/8 blocks) and W_E applied to E coordinate 0 and to E
//    coordinate 1 (C/4 x C/4), all in one launch;
//  - the expanded-dense comparator ("Flash EQ-Linear", Problem Statement):
//    one job, the full replicated matrix.
//
// Tile: NT output channels x TT tokens per workgroup (4 waves, 2 x 2).  The
// MFMA A operand is a W row block, B a token block, so every lane ends up with
// four consecutive output channels of one token and stores them as one vector.
#include "eq_device.h"
#include "eq_launch.h"

namespace eql {

template <typename IO>
struct GemmTraits;
template <>
struct GemmTraits<float> {
    static constexpr int KC = 16;
    static constexpr int R = 4;
};
template <>
struct GemmTraits<__bf16> {
    static constexpr int KC = 32;
    static constexpr int R = 8;
};
template <>
struct GemmTraits<_Float16> {
    static constexpr int KC = 32;
    static constexpr int R = 8;
};

template <typename IO_, int NPW_, int TPW_>
struct GemmCfg {
    using IO = IO_;
    static constexpr int NPW = NPW_, TPW = TPW_;
    static constexpr int WN = 2, WT = 2;
    static constexpr int kThreads = 64 * WN * WT;
    static constexpr int NT = WN * NPW * 16;
    static constexpr int TT = WT * TPW * 16;
    static constexpr int KC = GemmTraits<IO>::KC;
    static constexpr int R = GemmTraits<IO>::R;
    static constexpr int S = (int)sizeof(IO);
    static constexpr int PITCH = KC + 16 / S;
    static constexpr int PARTS = KC / R;  // 16-byte vectors per row chunk (4)
    static constexpr int WVEC = NT * PARTS;
    static constexpr int XVEC = TT * PARTS;
    static constexpr int WV = (WVEC + kThreads - 1) / kThreads;
    static constexpr int XV = (XVEC + kThreads - 1) / kThreads;
};

template <typename IO>
__device__ __forceinline__ void set_half(uint32_t* w, int e, uint32_t bits);
template <>
__device__ __forceinline__ void set_half<float>(uint32_t* w, int e, uint32_t bits) {
    w[e] = bits;
}
template <>
__device__ __forceinline__ void set_half<__bf16>(uint32_t* w, int e, uint32_t bits) {
    if (e & 1) w[e >> 1] = (w[e >> 1] & 0x0000ffffu) | (bits << 16);
    else w[e >> 1] = (w[e >> 1] & 0xffff0000u) | bits;
}
template <>
__device__ __forceinline__ void set_half<_Float16>(uint32_t* w, int e, uint32_t bits) {
    set_half<__bf16>(w, e, bits);  // the same 16-bit placement
}

template <typename IO>
__device__ __forceinline__ uint32_t bits_of(const IO* p) {
    if constexpr (sizeof(IO) == 4) return *reinterpret_cast<const uint32_t*>(p);
    else return (uint32_t)*reinterpret_cast<const uint16_t*>(p);
}

// Load R consecutive elements of a row (16 bytes) with bounds and alignment checks.
template <typename IO, int R>
__device__ __forceinline__ uint4 load_row_vec(const IO* src, bool row_ok, int avail, bool vec_ok) {
    if (row_ok && vec_ok && avail >= R) return *reinterpret_cast<const uint4*>(src);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (row_ok) {
#pragma unroll
        for (int e = 0; e < R; ++e)
            if (e < avail) set_half<IO>(w, e, bits_of<IO>(src + e));
    }
    return uint4{w[0], w[1], w[2], w[3]};
}

__device__ __forceinline__ void mma16(f32x4& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& acc, const f16x8& a, const f16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& acc, const f32x4& a, const f32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
}

template <class C>
__global__ __launch_bounds__(C::kThreads) void gemm_rows_kernel(
    GemmJobs jobs, const typename C::IO* __restrict__ x, const typename C::IO* __restrict__ w,
    typename C::IO* __restrict__ y, int64_t T, int ldx, int ldy, uint32_t total_tiles) {
    using IO = typename C::IO;
    using F = std::conditional_t<std::is_same<IO, float>::value, f32x4,
                                 std::conditional_t<std::is_same<IO, _Float16>::value, f16x8, bf16x8>>;
    __shared__ __attribute__((aligned(16))) IO sW[C::NT * C::PITCH];
    __shared__ __attribute__((aligned(16))) IO sX[C::TT * C::PITCH];

    const uint32_t tile = xcd_remap(blockIdx.x, total_tiles);
    const int64_t t0 = (int64_t)(tile / jobs.tiles_per_row) * C::TT;
    const int jt = (int)(tile % jobs.tiles_per_row);
    int ji = 0;
#pragma unroll
    for (int j = 1; j < kMaxGemmJobs; ++j)
        if (j < jobs.njobs && jt >= jobs.j[j].tile_begin) ji = j;
    const GemmJob job = jobs.j[ji];
    const int n0 = (jt - job.tile_begin) * C::NT;
    const IO* wj = w + job.w_off;
    const int K = job.K, Nn = job.Nn;
    const bool xvec_ok = job.x_vec_ok != 0, wvec_ok = job.w_vec_ok != 0;

    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
    const int wn = wave / C::WT, wt = wave % C::WT;
    const int kofs = (lane >> 4) * (C::KC / 4);

    f32x4 acc[C::NPW][C::TPW];
#pragma unroll
    for (int a = 0; a < C::NPW; ++a)
#pragma unroll
        for (int b = 0; b < C::TPW; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 wr[C::WV], xr[C::XV];
    auto load = [&](int k0) {
#pragma unroll
        for (int v = 0; v < C::WV; ++v) {
            const int vi = (int)threadIdx.x + v * C::kThreads;
            if (C::WVEC % C::kThreads != 0 && vi >= C::WVEC) continue;
            const int row = vi / C::PARTS, part = vi % C::PARTS;
            const int n = n0 + row, k = k0 + part * C::R;
            wr[v] = load_row_vec<IO, C::R>(wj + (int64_t)n * job.ldw + k, n < Nn, K - k, wvec_ok);
        }
#pragma unroll
        for (int v = 0; v < C::XV; ++v) {
            const int vi = (int)threadIdx.x + v * C::kThreads;
            if (C::XVEC % C::kThreads != 0 && vi >= C::XVEC) continue;
            const int row = vi / C::PARTS, part = vi % C::PARTS;
            const int64_t t = t0 + row;
            const int k = k0 + part * C::R;
            xr[v] = load_row_vec<IO, C::R>(x + t * ldx + job.x_col + k, t < T, K - k, xvec_ok);
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int v = 0; v < C::WV; ++v) {
            const int vi = (int)threadIdx.x + v * C::kThreads;
            if (C::WVEC % C::kThreads != 0 && vi >= C::WVEC) continue;
            *reinterpret_cast<uint4*>(sW + (vi / C::PARTS) * C::PITCH + (vi % C::PARTS) * C::R) = wr[v];
        }
#pragma unroll
        for (int v = 0; v < C::XV; ++v) {
            const int vi = (int)threadIdx.x + v * C::kThreads;
            if (C::XVEC % C::kThreads != 0 && vi >= C::XVEC) continue;
            *reinterpret_cast<uint4*>(sX + (vi / C::PARTS) * C::PITCH + (vi % C::PARTS) * C::R) = xr[v];
        }
    };

    const int nchunks = (K + C::KC - 1) / C::KC;
    load(0);
    for (int c = 0; c < nchunks; ++c) {
        stage();
        __syncthreads();
        if (c + 1 < nchunks) load((c + 1) * C::KC);
        F A[C::NPW], B[C::TPW];
#pragma unroll
        for (int a = 0; a < C::NPW; ++a)
            A[a] = *reinterpret_cast<const F*>(sW + (wn * C::NPW * 16 + a * 16 + (lane & 15)) * C::PITCH + kofs);
#pragma unroll
        for (int b = 0; b < C::TPW; ++b)
            B[b] = *reinterpret_cast<const F*>(sX + (wt * C::TPW * 16 + b * 16 + (lane & 15)) * C::PITCH + kofs);
#pragma unroll
        for (int a = 0; a < C::NPW; ++a)
#pragma unroll
            for (int b = 0; b < C::TPW; ++b) mma16(acc[a][b], A[a], B[b]);
        __syncthreads();
    }

    // lane holds outputs n = nb*16 + (lane/16)*4 + r, r = 0..3, for token tb*16 + lane%16
    const bool yvec_ok = job.y_vec_ok != 0;
#pragma unroll
    for (int a = 0; a < C::NPW; ++a)
#pragma unroll
        for (int b = 0; b < C::TPW; ++b) {
            const int n = n0 + wn * C::NPW * 16 + a * 16 + (lane >> 4) * 4;
            const int64_t t = t0 + wt * C::TPW * 16 + b * 16 + (lane & 15);
            if (t >= T || n >= Nn) continue;
            IO* dst = y + t * ldy + job.y_col + n;
            const f32x4 v = acc[a][b];
            if (yvec_ok && n + 4 <= Nn) {
                if constexpr (std::is_same<IO, float>::value) {
                    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
                } else {
                    u32x2 u = {Half<IO>::pack2(v[0], v[1]), Half<IO>::pack2(v[2], v[3])};
                    __builtin_nontemporal_store(u, reinterpret_cast<u32x2*>(dst));
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < Nn) dst[r] = (IO)v[r];
            }
        }
}

template <class C>
static hipError_t launch_gemm_cfg(GemmJobs jobs, const void* x, const void* w, void* y, int64_t T,
                                  int ldx, int ldy, hipStream_t stream) {
    using IO = typename C::IO;
    const int S = (int)sizeof(IO);
    int tiles = 0;
    for (int j = 0; j < jobs.njobs; ++j) {
        GemmJob& jb = jobs.j[j];
        jb.tile_begin = tiles;
        tiles += (jb.Nn + C::NT - 1) / C::NT;
        jb.x_vec_ok = ((int64_t)ldx * S % 16 == 0) && ((int64_t)jb.x_col * S % 16 == 0);
        jb.w_vec_ok = ((int64_t)jb.ldw * S % 16 == 0) && ((int64_t)jb.w_off * S % 16 == 0);
        jb.y_vec_ok = ((int64_t)ldy * S % (4 * S) == 0) && ((int64_t)jb.y_col * S % (4 * S) == 0);
    }
    for (int j = jobs.njobs; j < kMaxGemmJobs; ++j) jobs.j[j] = jobs.j[0];
    jobs.tiles_per_row = tiles;
    const int64_t n_t = (T + C::TT - 1) / C::TT;
    const int64_t total = n_t * tiles;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gemm_rows_kernel<C>), dim3((uint32_t)total), dim3(C::kThreads), 0, stream,
                       jobs, (const IO*)x, (const IO*)w, (IO*)y, T, ldx, ldy, (uint32_t)total);
    return hipGetLastError();
}

template <typename IO>
static hipError_t launch_gemm_dt(GemmJobs jobs, const void* x, const void* w, void* y, int64_t T,
                                 int ldx, int ldy, hipStream_t stream) {
    bool all160 = true;
    int64_t work_tiles64 = 0;
    for (int j = 0; j < jobs.njobs; ++j) {
        all160 = all160 && (jobs.j[j].Nn % 160 == 0);
        work_tiles64 += (jobs.j[j].Nn + 127) / 128;
    }
    work_tiles64 *= (T + 127) / 128;
    if (all160) {
        if ((T + 127) / 128 * 8 >= 512) return launch_gemm_cfg<GemmCfg<IO, 5, 4>>(jobs, x, w, y, T, ldx, ldy, stream);
        return launch_gemm_cfg<GemmCfg<IO, 5, 2>>(jobs, x, w, y, T, ldx, ldy, stream);
    }
    if (work_tiles64 >= 512) return launch_gemm_cfg<GemmCfg<IO, 4, 4>>(jobs, x, w, y, T, ldx, ldy, stream);
    return launch_gemm_cfg<GemmCfg<IO, 2, 2>>(jobs, x, w, y, T, ldx, ldy, stream);
}

hipError_t launch_gemm_rows(int io, GemmJobs jobs, const void* x, const void* w, void* y,
                            int64_t T, int ldx, int ldy, hipStream_t stream) {
    if (io == kIoBF16) return launch_gemm_dt<__bf16>(jobs, x, w, y, T, ldx, ldy, stream);
    if (io == kIoF16) return launch_gemm_dt<_Float16>(jobs, x, w, y, T, ldx, ldy, stream);
    return launch_gemm_dt<float>(jobs, x, w, y, T, ldx, ldy, stream);
}

}  // namespace eql
