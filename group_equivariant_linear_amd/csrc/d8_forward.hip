// d8_forward.hip -- bf16 D8 Fourier-domain layer on gfx950 MFMA.
//
// The layer is a block-diagonal product in the irrep basis ("Quick ViTs", key
// design 2): y_rho = W_rho x_rho for the four 1-D irreps and W_E applied to
// each of the two coordinates of the 2-D irrep.  Each of the six products is
// a job y[t][y_col + n] = sum_k W[n][k] x[t][x_col + k]; one launch covers
// all of them.
//
// Workgroup: a grid of waves over TT tokens x CT output channels of one job.
// Per chunk of 64 input channels both operands reach LDS by direct
// global->LDS loads into an ST-stage ring (ST-1 chunks in flight, one barrier
// per chunk): the W rows and the x rows of the tile, both in the XOR-swizzled
// 16-byte-part order that makes the fragment reads conflict-free.
// Every thread issues the same number of loads for every chunk slot (slots
// past the last chunk load nothing), so one fixed vmcnt waits for exactly the
// oldest chunk.  The MFMA A operand is a
// W row block, B the wave's token block, so every lane ends with four
// consecutive output channels of one token; y leaves through an LDS staging
// area as contiguous 16-byte pieces.
//
// Requirements (checked by the launcher, which otherwise uses gemm_rows):
// bf16, job columns, widths and W rows in whole 16-byte pieces.
#include "eq_device.h"
#include "eq_launch.h"

namespace eql {

namespace {

constexpr uint32_t kD8OOB = 0x80000000u;  // offset past every resource (extents < 2^31)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t d8_rsrc(const void* base, uint32_t bytes) {
    // word 3 = 0x00020000: raw (untyped) buffer, 32-bit data format
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16-byte part q (0..7) of row o of a 128-byte row chunk sits at part
// q ^ ((o >> 1) & 7): a fragment read (16 lanes, rows o..o+15, one part) then
// touches 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int o, int q) { return o * 8 + (q ^ ((o >> 1) & 7)); }

// Workgroup tile: WT x WN waves; wave (wt, wn) owns TPW 16-token blocks and
// NPW 16-channel blocks, so each W fragment it reads from LDS feeds TPW
// products and each x fragment NPW.
template <int WT_, int WN_, int TPW_, int NPW_, int ST_>
struct D8Cfg {
    static constexpr int WT = WT_, WN = WN_, TPW = TPW_, NPW = NPW_;
    static constexpr int ST = ST_;  // pipeline stages (LDS buffers per operand)
    static constexpr int WAVES = WT * WN;
    static constexpr int kThreads = 64 * WAVES;
    static constexpr int TT = 16 * TPW * WT;  // tokens per workgroup
    static constexpr int CT = 16 * NPW * WN;  // output channels per workgroup
    static constexpr int KC = 64;             // input channels per chunk: two 16x16x32 steps
    static constexpr int W_SLOTS = CT * 8;    // 16-byte parts of a W chunk
    static constexpr int W_LOADS = (W_SLOTS + kThreads - 1) / kThreads;
    static constexpr int W_BUF = W_LOADS * kThreads * 16;
    static constexpr int X_SLOTS = TT * 8;
    static constexpr int X_LOADS = (X_SLOTS + kThreads - 1) / kThreads;
    static constexpr int X_BUF = X_LOADS * kThreads * 16;
    static constexpr int MAIN = ST * (W_BUF + X_BUF);
    static constexpr int LOADS = W_LOADS + X_LOADS;  // per thread and chunk
    static_assert((ST - 2) * LOADS <= 63, "vmcnt range");
    // y staging per wave: 16 TPW token rows of 16 NPW channels
    static constexpr int YP = 16 * NPW * 2 / 16;  // 16-byte pieces of one staged row
    static constexpr bool YROT = (YP % 8) == 0;
    static constexpr int YPITCH = YROT ? YP : (YP | 1);
    static constexpr int YST = 16 * TPW * YPITCH * 16;
    static constexpr int LDS = MAIN > WAVES * YST ? MAIN : WAVES * YST;
};

// s_waitcnt immediate that waits for vmcnt <= n and leaves lgkmcnt and
// expcnt unconstrained (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8]
// | vmcnt[5:4] at [15:14]).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

template <bool ROT, int X, int P>
__device__ __forceinline__ int ypiece(int r, int k) {
    if constexpr (ROT) return r * P + ((k + r) % X);
    else return r * P + k;
}

__device__ __forceinline__ f32x4 d8_mma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 d8_mma(const f16x8& a, const f16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// One tile: tokens t0 .. t0+TT-1, output channels n0 .. n0+CT-1 of job.  IO is
// __bf16 or _Float16 (the matrix-core product of the same shape for either).
template <class C, typename IO>
__device__ __forceinline__ void d8_tile(const GemmJob& job, int n0, int64_t t0, const IO* __restrict__ x,
                                        const IO* __restrict__ w, IO* __restrict__ y, int64_t T, int ldx,
                                        int ldy, uint32_t w_bytes, char* smem) {
    using F8 = typename Half<IO>::x8;
    constexpr int TPW = C::TPW, NPW = C::NPW;
    const int K = job.K, Nn = job.Nn;

    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wt = wave / C::WN, wn = wave % C::WN;
    const int kg = lane >> 4, tl = lane & 15;
    const uint32_t row_x = (uint32_t)ldx * 2u, row_y = (uint32_t)ldy * 2u;
    const int64_t rem = T - t0;
    const uint32_t rows = (uint32_t)(rem < C::TT ? rem : C::TT);
    const __amdgpu_buffer_rsrc_t rx = d8_rsrc(x + t0 * ldx, rows * row_x);
    const __amdgpu_buffer_rsrc_t ry = d8_rsrc(y + t0 * ldy, rows * row_y);
    const __amdgpu_buffer_rsrc_t rw = d8_rsrc(w, w_bytes);

    char* wbuf = smem;
    char* xbuf = smem + C::ST * C::W_BUF;

    // Slot s of a chunk tile (W: CT rows, x: TT rows, 128 bytes each) is row
    // s/8, stored part s%8, holding part (s%8) ^ ((row >> 1) & 7).  W rows past
    // Nn and slots past the tile read nothing (never used).
    uint32_t woff[C::W_LOADS], xoff[C::X_LOADS];
#pragma unroll
    for (int it = 0; it < C::W_LOADS; ++it) {
        const int sl = it * C::kThreads + tid, o = sl >> 3;
        const int q = (sl & 7) ^ ((o >> 1) & 7);
        woff[it] = (sl < C::W_SLOTS && n0 + o < Nn)
                       ? (uint32_t)(((int64_t)job.w_off + (int64_t)(n0 + o) * job.ldw + q * 8) * 2)
                       : kD8OOB;
    }
#pragma unroll
    for (int it = 0; it < C::X_LOADS; ++it) {
        const int sl = it * C::kThreads + tid, r = sl >> 3;
        const int q = (sl & 7) ^ ((r >> 1) & 7);
        xoff[it] = sl < C::X_SLOTS ? (uint32_t)r * row_x + (uint32_t)(job.x_col + q * 8) * 2u : kD8OOB;
    }

    const int nch = (K + C::KC - 1) / C::KC;
    // loads of chunk c into stage c % ST (past the last chunk: out-of-range
    // offsets, no memory access, same instruction count)
    auto dma = [&](int c) {
        const bool past = c >= nch;
        const bool tail = c * C::KC + C::KC > K;
        char* wb = wbuf + (c % C::ST) * C::W_BUF;
        char* xb = xbuf + (c % C::ST) * C::X_BUF;
#pragma unroll
        for (int it = 0; it < C::W_LOADS; ++it) {
            uint32_t off = past ? kD8OOB : woff[it];
            if (tail && !past) {
                const int sl = it * C::kThreads + tid, o = sl >> 3;
                if (c * C::KC + ((sl & 7) ^ ((o >> 1) & 7)) * 8 >= K) off = kD8OOB;
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rw, (__attribute__((address_space(3))) void*)(wb + (it * C::kThreads + wave * 64) * 16), 16, off,
                (uint32_t)(c * C::KC * 2), 0, 0);
        }
#pragma unroll
        for (int it = 0; it < C::X_LOADS; ++it) {
            uint32_t off = past ? kD8OOB : xoff[it];
            if (tail && !past) {
                const int sl = it * C::kThreads + tid, r = sl >> 3;
                if (c * C::KC + ((sl & 7) ^ ((r >> 1) & 7)) * 8 >= K) off = kD8OOB;
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (__attribute__((address_space(3))) void*)(xb + (it * C::kThreads + wave * 64) * 16), 16, off,
                (uint32_t)(c * C::KC * 2), 0, 0);
        }
    };

    f32x4 acc[NPW][TPW];
#pragma unroll
    for (int a = 0; a < NPW; ++a)
#pragma unroll
        for (int b = 0; b < TPW; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int c = 0; c < C::ST - 1; ++c) dma(c);
    for (int c = 0; c < nch; ++c) {
        // chunk c has landed once at most the ST-2 younger chunks are in flight;
        // after the barrier every wave's part of it has.  (A plain s_barrier:
        // __syncthreads would also wait for the younger chunks.)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((C::ST - 2) * C::LOADS));
        __builtin_amdgcn_s_barrier();
        dma(c + C::ST - 1);  // into the stage every wave finished with last step
        const char* wb = wbuf + (c % C::ST) * C::W_BUF + wn * NPW * 2048;
        const char* xb = xbuf + (c % C::ST) * C::X_BUF + wt * TPW * 2048;
        // two k-steps of 32 channels: parts 4 ks + kg of this lane's rows
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (c * C::KC + 32 * ks >= K) break;  // a last chunk's empty half (uniform per job)
            const int l_off = swz(tl, 4 * ks + kg) * 16;
            F8 A[NPW], B[TPW];
#pragma unroll
            for (int a = 0; a < NPW; ++a) A[a] = *reinterpret_cast<const F8*>(wb + a * 2048 + l_off);
#pragma unroll
            for (int b = 0; b < TPW; ++b) B[b] = *reinterpret_cast<const F8*>(xb + b * 2048 + l_off);
            if (c * C::KC + C::KC > K && c * C::KC + 32 * ks + kg * 8 >= K) {
                // input-channel tail: k-values past K are zero on both sides (the
                // parts there were never loaded)
#pragma unroll
                for (int a = 0; a < NPW; ++a) A[a] = F8{};
#pragma unroll
                for (int b = 0; b < TPW; ++b) B[b] = F8{};
            }
#pragma unroll
            for (int a = 0; a < NPW; ++a)
#pragma unroll
                for (int b = 0; b < TPW; ++b)
                    acc[a][b] = d8_mma(A[a], B[b], acc[a][b]);
        }
    }

    // Epilogue: lane (tl, kg) holds channels 16(wn NPW + a) + 4kg + i of token
    // 16(wt TPW + b) + tl; each wave stages its 16 TPW rows x 16 NPW channels.
    __syncthreads();  // the staging area overlaps the operand buffers
    char* yst = smem + wave * C::YST;
#pragma unroll
    for (int a = 0; a < NPW; ++a)
#pragma unroll
        for (int b = 0; b < TPW; ++b) {
            const int by = (16 * a + 4 * kg) * 2;  // 8 bytes, inside one 16-byte piece
            *reinterpret_cast<u32x2*>(yst + ypiece<C::YROT, C::YP, C::YPITCH>(16 * b + tl, by / 16) * 16 + (by % 16)) =
                u32x2{Half<IO>::pack2(acc[a][b][0], acc[a][b][1]), Half<IO>::pack2(acc[a][b][2], acc[a][b][3])};
        }
    const int nw0 = n0 + wn * NPW * 16;   // first channel of this wave
    const int lim = (Nn - nw0) * 2;       // valid bytes of a staged row
    const uint32_t col = (uint32_t)(job.y_col + nw0) * 2u;
    const int tw0 = wt * TPW * 16;        // first token row of this wave
#pragma unroll
    for (int it = 0; it < (16 * TPW * C::YP + 63) / 64; ++it) {
        const int pc = it * 64 + lane;
        if ((16 * TPW * C::YP) % 64 != 0 && pc >= 16 * TPW * C::YP) break;
        const int r = pc / C::YP, k = pc % C::YP;
        const u32x4 v = *reinterpret_cast<const u32x4*>(yst + ypiece<C::YROT, C::YP, C::YPITCH>(r, k) * 16);
        const uint32_t off = k * 16 < lim ? (uint32_t)(tw0 + r) * row_y + col + (uint32_t)k * 16u : kD8OOB;
        __builtin_amdgcn_raw_buffer_store_b128(v, ry, off, 0, kYStoreAux);
    }
}

// Workgroups take one tile each.  Jobs flagged narrow (the ones with twice the
// input channels: W_E on an E coordinate) use the CN shape, the others CW, so
// that every workgroup has the same number of products.
template <class CW, class CN, typename IO>
__global__ __launch_bounds__(CW::kThreads) void d8_kernel(GemmJobs jobs, const IO* __restrict__ x,
                                                          const IO* __restrict__ w, IO* __restrict__ y,
                                                          int64_t T, int ldx, int ldy, uint32_t total_tiles,
                                                          uint32_t w_bytes) {
    static_assert(CW::TT == CN::TT && CW::kThreads == CN::kThreads, "one workgroup shape");
    __shared__ __attribute__((aligned(16))) char smem[CW::LDS > CN::LDS ? CW::LDS : CN::LDS];

    const uint32_t tile = xcd_remap(blockIdx.x, total_tiles);
    const int64_t t0 = (int64_t)(tile / jobs.tiles_per_row) * CW::TT;
    const int jt = (int)(tile % jobs.tiles_per_row);
    int ji = 0;
#pragma unroll
    for (int j = 1; j < kMaxGemmJobs; ++j)
        if (j < jobs.njobs && jt >= jobs.j[j].tile_begin) ji = j;
    const GemmJob job = jobs.j[ji];
    if (job.narrow)
        d8_tile<CN, IO>(job, (jt - job.tile_begin) * CN::CT, t0, x, w, y, T, ldx, ldy, w_bytes, smem);
    else
        d8_tile<CW, IO>(job, (jt - job.tile_begin) * CW::CT, t0, x, w, y, T, ldx, ldy, w_bytes, smem);
}

template <class CW, class CN, typename IO>
hipError_t launch_d8_cfg(GemmJobs jobs, const void* x, const void* w, void* y, int64_t T, int ldx, int ldy,
                         int64_t w_elems, hipStream_t stream) {
    int kmin = jobs.j[0].K;
    for (int j = 1; j < jobs.njobs; ++j) kmin = jobs.j[j].K < kmin ? jobs.j[j].K : kmin;
    int tiles = 0;
    for (int j = 0; j < jobs.njobs; ++j) {
        jobs.j[j].narrow = (kmin > 0 && jobs.j[j].K >= 2 * kmin) ? 1 : 0;
        jobs.j[j].tile_begin = tiles;
        tiles += (jobs.j[j].Nn + (jobs.j[j].narrow ? CN::CT : CW::CT) - 1) / (jobs.j[j].narrow ? CN::CT : CW::CT);
    }
    for (int j = jobs.njobs; j < kMaxGemmJobs; ++j) jobs.j[j] = jobs.j[0];
    jobs.tiles_per_row = tiles;
    const int64_t total = (T + CW::TT - 1) / CW::TT * tiles;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((d8_kernel<CW, CN, IO>), dim3((uint32_t)total), dim3(CW::kThreads), 0, stream, jobs,
                       (const IO*)x, (const IO*)w, (IO*)y, T, ldx, ldy, (uint32_t)total,
                       (uint32_t)(w_elems * 2));
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_d8_shape(GemmJobs jobs, const void* x, const void* w, void* y, int64_t T, int ldx, int ldy,
                           int64_t w_elems, int cb, hipStream_t stream) {
    // 128 tokens x 160 channels (2x2 waves), or x 80 channels (4x1 waves) for
    // the jobs with twice the input channels; the smaller shapes use one tile
    // for every job
    using Wide = D8Cfg<2, 2, 4, 5, 2>;
    using Narrow = D8Cfg<4, 1, 2, 5, 2>;
    using Small = D8Cfg<4, 1, 1, 2, 2>;
    switch (cb) {
        case 5:
            return launch_d8_cfg<D8Cfg<2, 1, 4, 5, 2>, D8Cfg<2, 1, 4, 5, 2>, IO>(jobs, x, w, y, T, ldx, ldy, w_elems,
                                                                                stream);
        case 6:  // 96-channel blocks (D6 at width 1152): 64 tokens x 96 channels, 2x2 waves
            return launch_d8_cfg<D8Cfg<2, 2, 2, 3, 2>, D8Cfg<2, 2, 2, 3, 2>, IO>(jobs, x, w, y, T, ldx, ldy,
                                                                                w_elems, stream);
        case 2: return launch_d8_cfg<Small, Small, IO>(jobs, x, w, y, T, ldx, ldy, w_elems, stream);
        default: return launch_d8_cfg<Wide, Narrow, IO>(jobs, x, w, y, T, ldx, ldy, w_elems, stream);
    }
}

}  // namespace

// The D8 jobs on the kernel above (bf16 or fp16) when every job column, width
// and W row is a whole number of 16-byte pieces and all offsets fit 32 bits;
// otherwise hipErrorNotSupported (the caller then uses gemm_rows).
hipError_t launch_d8_fast(int io, GemmJobs jobs, const void* x, const void* w, void* y, int64_t T, int ldx, int ldy,
                          int64_t w_elems, int cb, hipStream_t stream) {
    const int64_t lim = (int64_t)1 << 30;
    if (ldx % 8 || ldy % 8 || w_elems * 2 >= lim || (int64_t)128 * ldx * 2 >= lim || (int64_t)128 * ldy * 2 >= lim)
        return hipErrorNotSupported;
    for (int j = 0; j < jobs.njobs; ++j) {
        const GemmJob& g = jobs.j[j];
        if (g.x_col % 8 || g.y_col % 8 || g.K % 8 || g.Nn % 8 || g.ldw % 8 || g.w_off % 8) return hipErrorNotSupported;
    }
    if (io == kIoF16) return launch_d8_shape<_Float16>(jobs, x, w, y, T, ldx, ldy, w_elems, cb, stream);
    if (io == kIoBF16) return launch_d8_shape<__bf16>(jobs, x, w, y, T, ldx, ldy, w_elems, cb, stream);
    return hipErrorNotSupported;
}

}  // namespace eql
