// dn_regular.hip -- the dihedral layer between regular-representation features
// in one launch ("Quick ViTs", key design 2: the MLP of an equivariant ViT
// keeps its features in the regular representation, where the group only
// permutes each channel's G values and GELU can act pointwise; the linear map
// itself is block-diagonal in the group-Fourier basis).
//
//   y_reg = act( to_regular( W_blocks . to_fourier(x_reg) ) + b )
//
// x_reg [T][m_in][G] and y_reg [T][m_out][G] hold G = 2n values per regular
// channel (dn_group.h: element order, Fourier matrix F).  One workgroup owns
// TT tokens x JT output regular channels and walks the input channels in
// chunks of 32:
//   prologue  every thread loads four consecutive regular input channels of
//             one token (global -> registers, the next chunk's loads in flight
//             during this chunk's products), applies F in fp32 and writes the
//             Fourier features, rounded once to the I/O type, into an LDS tile
//             with one slab per 1-D irrep (32 values per token) and one per
//             E_k coordinate (64 copies per token);
//   products  on the matrix cores, fp32 accumulation: each 1-D irrep's block
//             times its slab, and each E_k block times both coordinate slabs.
//             The W blocks reach LDS by direct global->LDS loads (two stages);
//             the rows of each E_k block are split by parity (copies 2j and
//             2j+1 of output channel j), so that a lane ends up holding every
//             Fourier feature -- N1 1-D values and four per E_k -- of the same
//             four output channels of one token;
//   epilogue  per output channel: F^T back to the G regular values (fp32), the
//             bias (one value per regular channel, the same for all G values:
//             it commutes with the group) and GELU, one rounding to the I/O
//             type, staged in LDS and stored as contiguous 16-byte pieces.
// No Fourier-domain tensor goes to memory; the layer reads x once and writes y
// once.
#include "cn_fused.h"
#include "dn_group.h"

namespace eql {

namespace {

template <int n_, typename IO_, int WT_, int WN_, int TPW_, int CB_>
struct DnrCfg {
    using IO = IO_;
    using D = DnGroup<n_>;
    using F8 = typename Half<IO_>::x8;
    static constexpr int n = n_, G = D::G, N1 = D::N1, N2 = D::N2;
    static constexpr int WT = WT_, WN = WN_, TPW = TPW_, CB = CB_;
    static constexpr int WAVES = WT * WN, kThreads = 64 * WAVES;
    static constexpr int TT = 16 * TPW * WT;  // tokens per workgroup
    static constexpr int JT = 16 * CB * WN;   // output regular channels per workgroup
    static constexpr int KJ = 32;             // input regular channels per chunk
    // Fourier tile of one chunk: the 1-D slabs [TT][32] (64-byte rows), then
    // for each E_k its coordinate-0 and coordinate-1 slabs [TT][64] (128-byte
    // rows); TT * 64 * G bytes in all
    static constexpr int F1 = TT * 64, FE = TT * 128;
    static constexpr int F_BYTES = N1 * F1 + 2 * N2 * FE;
    // W chunk: the 1-D blocks [JT][32], then for each E_k the rows of copy
    // parity 0 and 1 [JT][64]
    static constexpr int W1 = JT * 64, WE = JT * 128;
    static constexpr int W_BYTES = N1 * W1 + 2 * N2 * WE;
    static constexpr int W_SLOTS = W_BYTES / 16;
    static constexpr int W_LOADS = (W_SLOTS + kThreads - 1) / kThreads;
    static constexpr int W_BUF = W_LOADS * kThreads * 16;
    // x: groups of four regular channels of one token, G/2 16-byte loads each
    static constexpr int XG = TT * (KJ / 4);
    static_assert(XG % kThreads == 0, "whole groups per thread");
    static constexpr int RX = XG / kThreads;
    static constexpr int XL = G / 2;
    // y staging per wave: 16 TPW token rows of 16 CB channels x G values
    static constexpr int YP = 2 * CB * G;  // 16-byte pieces of one staged row
    static constexpr int YPITCH = YP + 1;  // odd: the rows start in different bank groups
    static constexpr int YST = 16 * TPW * YPITCH * 16;
    static constexpr int MAIN = F_BYTES + 2 * W_BUF;
    static constexpr int LDS = MAIN > WAVES * YST ? MAIN : WAVES * YST;
    static_assert(LDS <= 163840, "LDS of one CU");
};

// 16-byte part p of row r of a 64-byte row (4 parts) or 128-byte row (8
// parts), stored XOR-swizzled so that 16 lanes reading one part of 16
// consecutive rows touch 16 distinct 16-byte bank groups.
__device__ __forceinline__ int sw64(int r, int p) { return r * 64 + 16 * (p ^ ((r >> 2) & 3)); }
__device__ __forceinline__ int sw128(int r, int p) { return r * 128 + 16 * (p ^ ((r >> 1) & 7)); }

__device__ __forceinline__ f32x4 dn_mma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 dn_mma(const f16x8& a, const f16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// v = F f for one channel (G values in, G Fourier features out)
template <int n>
__device__ __forceinline__ void dn_fourier(const float* f, float* v) {
    using D = DnGroup<n>;
    if constexpr (n == 4) {
        float a[8], b[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) a[q] = f[q];
        to_fourier8(a, b);
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = b[q];
    } else {
        static_for<0, D::G>([&](auto pc) {
            constexpr int p = decltype(pc)::value;
            float acc = 0.0f;
            static_for<0, D::G>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                constexpr float c = (float)D::entry(p, q);
                if constexpr (c != 0.0f) acc = __builtin_fmaf(c, f[q], acc);
            });
            v[p] = acc;
        });
    }
}

// f = F^T v for one channel
template <int n>
__device__ __forceinline__ void dn_regular(const float* v, float* f) {
    using D = DnGroup<n>;
    if constexpr (n == 4) {
        float a[8], b[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) a[q] = v[q];
        to_regular8(a, b);
#pragma unroll
        for (int q = 0; q < 8; ++q) f[q] = b[q];
    } else {
        static_for<0, D::G>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            float acc = 0.0f;
            static_for<0, D::G>([&](auto pc) {
                constexpr int p = decltype(pc)::value;
                constexpr float c = (float)D::entry(p, q);
                if constexpr (c != 0.0f) acc = __builtin_fmaf(c, v[p], acc);
            });
            f[q] = acc;
        });
    }
}

template <class C>
__global__ __launch_bounds__(C::kThreads) void dn_regular_kernel(
    const typename C::IO* __restrict__ x, const typename C::IO* __restrict__ w, const typename C::IO* __restrict__ bias,
    int act, typename C::IO* __restrict__ y, int64_t T, int m_in, int m_out, int n_j_tiles, uint32_t total_tiles,
    uint32_t w_bytes) {
    using IO = typename C::IO;
    using F8 = typename C::F8;
    constexpr int G = C::G, N1 = C::N1, N2 = C::N2, CB = C::CB, TPW = C::TPW;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];
    char* ftile = smem;
    char* wbuf = smem + C::F_BYTES;

    // the output-channel tiles of one token tile are consecutive ids: the
    // remap puts them on one XCD, where they share the token tile's x in L2
    const uint32_t tile = xcd_remap(blockIdx.x, total_tiles);
    const int64_t t0 = (int64_t)(tile / n_j_tiles) * C::TT;
    const int j0 = (int)(tile % n_j_tiles) * C::JT;
    const int tid = (int)threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wt = wave / C::WN, wn = wave % C::WN;
    const int kg = lane >> 4, tl = lane & 15;

    const uint32_t row_x = (uint32_t)m_in * (uint32_t)(G * 2), row_y = (uint32_t)m_out * (uint32_t)(G * 2);
    const int64_t rem = T - t0;
    const uint32_t rows = (uint32_t)(rem < C::TT ? rem : C::TT);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + t0 * m_in * G, rows * row_x);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(y + t0 * m_out * G, rows * row_y);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, w_bytes);

    const int nch = (m_in + C::KJ - 1) / C::KJ;
    const bool k_tail = (m_in % C::KJ) != 0;

    // --- W slots: slot s of a stage holds the 16-byte part that its position
    // in the swizzled layout asks for.  Per load: the chunk-0 byte offset, the
    // advance per chunk (64 bytes for a 1-D row, 128 for an E row) and the
    // number of chunk columns before the part (for the input-channel tail).
    uint32_t woff[C::W_LOADS], wadv[C::W_LOADS];
    int wcol[C::W_LOADS], wlim[C::W_LOADS];
    {
        const int64_t blk = (int64_t)m_out * m_in;
#pragma unroll
        for (int it = 0; it < C::W_LOADS; ++it) {
            const int s = it * C::kThreads + tid;
            int r = 0, p = 0, lim = 0;
            int64_t el = -1;
            uint32_t adv = 64;
            if (s < N1 * (C::W1 / 16)) {
                const int rho = s / (C::W1 / 16), rs = s % (C::W1 / 16);
                r = rs >> 2;
                p = (rs & 3) ^ ((r >> 2) & 3);
                if (j0 + r < m_out) el = rho * blk + (int64_t)(j0 + r) * m_in + 8 * p;
                lim = m_in;
            } else if (s < C::W_SLOTS) {
                const int se = s - N1 * (C::W1 / 16);
                const int kc = se / (C::WE / 16), rs = se % (C::WE / 16);  // kc = 2k + parity
                const int k = kc >> 1, par = kc & 1;
                r = rs >> 3;
                p = (rs & 7) ^ ((r >> 1) & 7);
                if (j0 + r < m_out)
                    el = N1 * blk + (int64_t)k * 4 * blk + (int64_t)(2 * (j0 + r) + par) * (2 * m_in) + 8 * p;
                lim = 2 * m_in;
                adv = 128;
            }
            woff[it] = el >= 0 ? (uint32_t)(el * 2) : kOOB;
            wadv[it] = adv;
            wcol[it] = 8 * p;
            wlim[it] = lim;
        }
    }
    // A partial last chunk leaves W parts past the input channels unloaded;
    // their x side is zero, so they only need to be finite: clear the stages.
    if (k_tail) {
        for (int i = tid; i < 2 * C::W_BUF / 16; i += C::kThreads)
            reinterpret_cast<u32x4*>(wbuf)[i] = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
    }
    auto dma_w = [&](int c) {
        if (c >= nch) return;
        char* wb = wbuf + (c & 1) * C::W_BUF;
        const bool tail = c == nch - 1 && k_tail;
#pragma unroll
        for (int it = 0; it < C::W_LOADS; ++it) {
            uint32_t off = woff[it];
            if (off != kOOB) {
                const int cc = c * (int)(wadv[it] >> 1);  // chunk's first column in this row
                off = (tail && cc + wcol[it] >= wlim[it]) ? kOOB : off + (uint32_t)c * wadv[it];
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rw, (__attribute__((address_space(3))) void*)(wb + (it * C::kThreads + wave * 64) * 16), 16, off, 0,
                0, 0);
        }
    };

    // --- x: group i of this thread is token xt[i], channels 4 xg[i] .. +3 of the chunk
    u32x4 xr[C::RX][C::XL];
    auto load_x = [&](int c) {
        if (c >= nch) return;
#pragma unroll
        for (int i = 0; i < C::RX; ++i) {
            const int idx = i * C::kThreads + tid, t = idx >> 3, g = idx & 7;
            const int ch = c * C::KJ + 4 * g;
            const uint32_t base = ch < m_in ? (uint32_t)t * row_x + (uint32_t)ch * (uint32_t)(G * 2) : kOOB;
#pragma unroll
            for (int q = 0; q < C::XL; ++q)
                xr[i][q] = __builtin_amdgcn_raw_buffer_load_b128(rx, base == kOOB ? kOOB : base + 16u * q, 0, 0);
        }
    };
    // F applied to this thread's groups, written to the Fourier tile
    auto transform = [&]() {
#pragma unroll
        for (int i = 0; i < C::RX; ++i) {
            const int idx = i * C::kThreads + tid, t = idx >> 3, g = idx & 7;
            float v[4][G];
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                float f[G];
#pragma unroll
                for (int e = 0; e < G; ++e) {
                    const int el = ch * G + e;  // element of the group's 4G values
                    const uint32_t wd = xr[i][el / 8][(el % 8) / 2];
                    f[e] = (el % 2) ? Half<IO>::hi(wd) : Half<IO>::lo(wd);
                }
                dn_fourier<C::n>(f, v[ch]);
            }
            // 1-D slab rho: channels 4g .. 4g+3 are bytes 8g .. 8g+7 of row t
#pragma unroll
            for (int rho = 0; rho < N1; ++rho)
                *reinterpret_cast<u32x2*>(ftile + rho * C::F1 + sw64(t, g >> 1) + 8 * (g & 1)) =
                    u32x2{Half<IO>::pack2(v[0][rho], v[1][rho]), Half<IO>::pack2(v[2][rho], v[3][rho])};
            // E_k coordinate kk: copies 8g .. 8g+7 (channel-major, copy c minor) are part g
#pragma unroll
            for (int k = 0; k < N2; ++k)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int p0 = N1 + 4 * k + 2 * kk;
                    *reinterpret_cast<u32x4*>(ftile + N1 * C::F1 + (2 * k + kk) * C::FE + sw128(t, g)) =
                        u32x4{Half<IO>::pack2(v[0][p0], v[0][p0 + 1]), Half<IO>::pack2(v[1][p0], v[1][p0 + 1]),
                              Half<IO>::pack2(v[2][p0], v[2][p0 + 1]), Half<IO>::pack2(v[3][p0], v[3][p0 + 1])};
                }
        }
    };

    // bias of this lane's output channels, before any store is issued
    float bv[CB][4];
#pragma unroll
    for (int b = 0; b < CB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = j0 + 16 * (wn * CB + b) + 4 * kg + i;
            bv[b][i] = (bias != nullptr && j < m_out) ? (float)bias[j] : 0.0f;
        }

    // accumulators: feature p of output block b, token block tb (p < N1: 1-D
    // irrep p; N1 + 4k + 2kk + c: E_k coordinate kk, copy parity c)
    f32x4 acc[G][CB][TPW];
#pragma unroll
    for (int p = 0; p < G; ++p)
#pragma unroll
        for (int b = 0; b < CB; ++b)
#pragma unroll
            for (int tb = 0; tb < TPW; ++tb) acc[p][b][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

    dma_w(0);
    load_x(0);
    for (int c = 0; c < nch; ++c) {
        // this thread's loads of chunk c have landed; after the barrier, every
        // thread's have, and every wave is done with chunk c-1's tiles
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        dma_w(c + 1);
        transform();
        load_x(c + 1);  // the registers of chunk c are consumed
        __syncthreads();  // the Fourier tile is complete
        const char* wb = wbuf + (c & 1) * C::W_BUF;
        // 1-D irreps: one 32-deep product per (block, token block)
#pragma unroll
        for (int rho = 0; rho < N1; ++rho) {
            F8 A[CB], B[TPW];
#pragma unroll
            for (int b = 0; b < CB; ++b)
                A[b] = *reinterpret_cast<const F8*>(wb + rho * C::W1 + sw64(16 * (wn * CB + b) + tl, kg));
#pragma unroll
            for (int tb = 0; tb < TPW; ++tb)
                B[tb] = *reinterpret_cast<const F8*>(ftile + rho * C::F1 + sw64(16 * (wt * TPW + tb) + tl, kg));
#pragma unroll
            for (int b = 0; b < CB; ++b)
#pragma unroll
                for (int tb = 0; tb < TPW; ++tb) acc[rho][b][tb] = dn_mma(A[b], B[tb], acc[rho][b][tb]);
        }
        // E_k: 64 copies deep, the parity-c rows times coordinate slab kk
#pragma unroll
        for (int k = 0; k < N2; ++k)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                F8 A[2][CB], B[2][TPW];
#pragma unroll
                for (int par = 0; par < 2; ++par)
#pragma unroll
                    for (int b = 0; b < CB; ++b)
                        A[par][b] = *reinterpret_cast<const F8*>(wb + N1 * C::W1 + (2 * k + par) * C::WE +
                                                                 sw128(16 * (wn * CB + b) + tl, 4 * e + kg));
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int tb = 0; tb < TPW; ++tb)
                        B[kk][tb] = *reinterpret_cast<const F8*>(ftile + N1 * C::F1 + (2 * k + kk) * C::FE +
                                                                 sw128(16 * (wt * TPW + tb) + tl, 4 * e + kg));
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int par = 0; par < 2; ++par)
#pragma unroll
                        for (int b = 0; b < CB; ++b)
#pragma unroll
                            for (int tb = 0; tb < TPW; ++tb) {
                                f32x4& a = acc[N1 + 4 * k + 2 * kk + par][b][tb];
                                a = dn_mma(A[par][b], B[kk][tb], a);
                            }
            }
    }

    // --- epilogue: lane (tl, kg) holds, for output channels 16(wn CB + b) + 4kg
    // + i of token 16(wt TPW + tb) + tl, all G Fourier features
    __syncthreads();  // the staging area overlaps the tiles
    char* yst = smem + wave * C::YST;
#pragma unroll
    for (int b = 0; b < CB; ++b)
#pragma unroll
        for (int tb = 0; tb < TPW; ++tb) {
            uint32_t pk[4][G / 2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v[G], f[G];
#pragma unroll
                for (int p = 0; p < G; ++p) v[p] = acc[p][b][tb][i];
                dn_regular<C::n>(v, f);
                if (act == 1) {
#pragma unroll
                    for (int q = 0; q < G; ++q) f[q] = gelu_erf(f[q] + bv[b][i]);
                } else {
#pragma unroll
                    for (int q = 0; q < G; ++q) f[q] += bv[b][i];
                }
#pragma unroll
                for (int q = 0; q < G / 2; ++q) pk[i][q] = Half<IO>::pack2(f[2 * q], f[2 * q + 1]);
            }
            // channels 16b + 4kg .. +3 of staged row 16 tb + tl: 8G contiguous bytes
            char* row = yst + (16 * tb + tl) * C::YPITCH * 16 + (16 * b + 4 * kg) * G * 2;
#pragma unroll
            for (int q = 0; q < G; ++q)  // G/2 dwords per channel: 2G dwords, G pairs
                *reinterpret_cast<u32x2*>(row + 8 * q) = u32x2{pk[(2 * q) / (G / 2)][(2 * q) % (G / 2)],
                                                               pk[(2 * q + 1) / (G / 2)][(2 * q + 1) % (G / 2)]};
        }
    // the wave stores its own staged rows: LDS operations of one wave are
    // performed in order, so no barrier is needed; the asm keeps the compiler
    // from moving the reads above the writes
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int jw = j0 + 16 * wn * CB;  // first output channel of this wave
    const int valid = jw < m_out ? (m_out - jw) * G * 2 : 0;  // valid bytes of a staged row
    const int tw = 16 * wt * TPW;  // first token row of this wave
    constexpr int PIECES = 16 * TPW * C::YP;
#pragma unroll
    for (int it = 0; it < (PIECES + 63) / 64; ++it) {
        const int pc = it * 64 + lane;
        if (PIECES % 64 != 0 && pc >= PIECES) break;
        const int r = pc / C::YP, k = pc % C::YP;
        const u32x4 v = *reinterpret_cast<const u32x4*>(yst + (r * C::YPITCH + k) * 16);
        const uint32_t off = (k * 16 < valid && (uint32_t)(tw + r) < rows)
                                 ? (uint32_t)(tw + r) * row_y + (uint32_t)jw * (uint32_t)(G * 2) + (uint32_t)k * 16u
                                 : kOOB;
        __builtin_amdgcn_raw_buffer_store_b128(v, ry, off, 0, kYStoreAux);
    }
}

template <class C>
hipError_t launch_dnr_cfg(const void* x, const void* w, const void* bias, int act, void* y, int64_t T, int m_in,
                          int m_out, int64_t w_elems, hipStream_t stream) {
    const int64_t n_t = (T + C::TT - 1) / C::TT;
    const int n_j = (m_out + C::JT - 1) / C::JT;
    const int64_t total = n_t * n_j;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    using IO = typename C::IO;
    hipLaunchKernelGGL((dn_regular_kernel<C>), dim3((uint32_t)total), dim3(C::kThreads), 0, stream, (const IO*)x,
                       (const IO*)w, (const IO*)bias, act, (IO*)y, T, m_in, m_out, n_j, (uint32_t)total,
                       (uint32_t)(w_elems * 2));
    return hipGetLastError();
}

#ifndef EQL_DNR_TILE
#define EQL_DNR_TILE 0
#endif

template <int n, typename IO>
hipError_t launch_dnr_n(const void* x, const void* w, const void* bias, int act, void* y, int64_t T, int m_in,
                        int m_out, int64_t w_elems, hipStream_t stream) {
    // 4 waves over 32 tokens x 32 output channels (2 x 2 waves of 16 x 16)
    // Wider tiles (64 x 32, 128 x 32, 32 x 64 and 64 x 64 per workgroup)
    // measured slower on both the D8 and the D6 layer, so every n uses this
    // one: the larger tiles leave one wave per SIMD or one workgroup per CU.
    using C = DnrCfg<n, IO, 2, 2, 1, 1>;
    return launch_dnr_cfg<C>(x, w, bias, act, y, T, m_in, m_out, w_elems, stream);
}

template <typename IO>
hipError_t launch_dnr_io(int n, const void* x, const void* w, const void* bias, int act, void* y, int64_t T,
                         int m_in, int m_out, int64_t w_elems, hipStream_t stream) {
    switch (n) {
#define EQL_DNR(k) \
    case k: return launch_dnr_n<k, IO>(x, w, bias, act, y, T, m_in, m_out, w_elems, stream);
        EQL_DNR(2) EQL_DNR(3) EQL_DNR(4) EQL_DNR(5) EQL_DNR(6) EQL_DNR(7) EQL_DNR(8) EQL_DNR(9) EQL_DNR(10)
        EQL_DNR(11) EQL_DNR(12)
#undef EQL_DNR
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_dn_regular(int n, int io, const void* x_reg, const void* wb, const void* bias, int act,
                             void* y_reg, int64_t T, int m_in, int m_out, int64_t w_elems, hipStream_t stream) {
    // whole 16-byte W parts and 32-bit offsets
    if (m_in % 8 || m_out % 8 || w_elems * 2 >= ((int64_t)1 << 31)) return hipErrorNotSupported;
    if ((int64_t)32 * m_in * 2 * n * 2 >= ((int64_t)1 << 31) || (int64_t)32 * m_out * 2 * n * 2 >= ((int64_t)1 << 31))
        return hipErrorNotSupported;
    if (io == kIoF16) return launch_dnr_io<_Float16>(n, x_reg, wb, bias, act, y_reg, T, m_in, m_out, w_elems, stream);
    if (io == kIoBF16) return launch_dnr_io<__bf16>(n, x_reg, wb, bias, act, y_reg, T, m_in, m_out, w_elems, stream);
    return hipErrorNotSupported;
}

}  // namespace eql
