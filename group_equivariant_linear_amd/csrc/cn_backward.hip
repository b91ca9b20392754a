// cn_backward.hip -- gradients of the C_N layer on gfx950.
//
// "Flash EQ-Linear", Implementation: the method's kernels cover the backward
// pass as well as the forward (Experimental Results, Operator Level: backward
// speedups, a little below the forward's because of the extra arithmetic and
// memory traffic of the gradients).  The pages give no formulas; these are the
// derivatives of the layer y[t][o][g] = sum_{i,m} w[o][i][m] x[t][i][(g-m) mod N].
//
// Input gradient.  dx[t][i][h] = sum_{o,g} w[o][i][(g-h) mod N] dy[t][o][g] is
// the same kind of layer with C_in and C_out exchanged and the weight
// w'[i][o][m] = w[o][i][(-m) mod N], whose spectrum is conj(What[k])^T.  The
// library forms that adjoint spectrum once per weight (w_hat_adjoint_kernel)
// and runs the forward kernels on dy with it.
//
// Weight gradient.  dw[o][i][m] = sum_{t,g} dy[t][o][g] x[t][i][(g-m) mod N] is
// a cross-correlation along the group axis, i.e. in the frequency domain
//     C_k[o][i] = sum_t DY[t][o][k] conj(X[t][i][k]),   dw = inverse real DFT of C,
// a contraction over tokens for every kept bin (complex bins: Re C = a c + b d,
// Im C = b c - a d with DY = a + ib, X = c + id).  Three launches:
//   1. bw_planes_kernel: real DFT of every record of x and of dy, written as
//      planes in chunk-major order [plane][chunk][channel][KC tokens] (64
//      bytes per channel and chunk; tokens padded to Tp), through an LDS
//      transpose.  A product stage, one chunk of some rows of one plane, then
//      reads a few contiguous runs of C x 64 bytes, not one 64-byte piece per
//      row from rows Tp S bytes apart (each piece a DRAM page of its own);
//   2. bw_bin_kernel (whole tiles, one bin per workgroup) or bw_gemm_kernel
//      (64 x 64 tiles, all bins): per tile and range of tokens, the products on
//      the matrix cores with the operand planes streamed through an LDS ring by
//      direct global->LDS loads; fp32 partial spectra per range;
//   3. bw_reduce_kernel: partials summed in a fixed order, inverse real DFT
//      per (o, i), dw written in fp32 [C_out][C_in][N].
// Layers of at most 32 channels each way run 1 and 2 as one launch
// (bw_small_kernel: transforms into LDS, no planes in HBM), then 3; so do the
// other 16-bit layers of even order up to 8 (bw_xf_kernel: 64 x 64 tiles, the
// transforms on the matrix cores inside the product kernel).
// Every step is deterministic (no atomics).
#include <mutex>

#include "dft_coef.h"
#include "eq_device.h"
#include "eq_launch.h"

namespace eql {

// Scratch memory of the weight gradient for callers that cannot allocate
// (launch_cn_backward_weight_noalloc): one array per GPU, held by the loaded
// code object until the process ends.  Host code never passes the array's name
// to a kernel: it takes the device address from hipGetSymbolAddress, once per
// device, and passes that.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr uint32_t kBwOOB = 0x80000000u;  // offset past every resource (extents < 2^31)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t bw_rsrc(const void* base, uint32_t bytes) {
    // word 3 = 0x00020000: raw (untyped) buffer, 32-bit data format
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Stride of one plane of the partial spectra [split][plane][o][i]: C_out C_in
// rounded up to a multiple of four, so that the reduction reads 16-byte groups.
__host__ __device__ constexpr int64_t bw_pstride(int C_in, int C_out) {
    return ((int64_t)C_out * C_in + 3) / 4 * 4;
}

// s_waitcnt immediate: vmcnt <= n, lgkmcnt and expcnt unconstrained.
constexpr int bw_vmcnt(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

template <typename IO>
__device__ __forceinline__ float to_f32(IO v) {
    return (float)v;
}

// plane p of the packed real spectrum holds an imaginary part
__host__ __device__ constexpr bool imag_plane(int N, int p) {
    return p > 0 && p % 2 == 0 && !(N % 2 == 0 && p == N - 1);
}

// --- adjoint spectrum ---------------------------------------------------------------
// out[p][i][o] = s_p in[p][o][i], s_p = -1 on imaginary planes: the w_hat of
// the layer with exchanged channels and reversed group axis.
template <typename IO>
__global__ __launch_bounds__(256) void w_hat_adjoint_kernel(const IO* __restrict__ in, IO* __restrict__ out,
                                                            int N, int C_in, int C_out) {
    __shared__ float tile[32][33];
    const int p = (int)blockIdx.z;
    const int o0 = (int)blockIdx.y * 32, i0 = (int)blockIdx.x * 32;
    const int tx = (int)threadIdx.x & 31, ty = (int)threadIdx.x >> 5;
    const int64_t plane = (int64_t)C_out * C_in;
    const IO* src = in + p * plane;
    for (int r = ty; r < 32; r += 8) {
        const int o = o0 + r, i = i0 + tx;
        if (o < C_out && i < C_in) tile[r][tx] = to_f32(src[(int64_t)o * C_in + i]);
    }
    __syncthreads();
    const float s = imag_plane(N, p) ? -1.0f : 1.0f;
    IO* dst = out + p * plane;
    for (int r = ty; r < 32; r += 8) {
        const int i = i0 + r, o = o0 + tx;
        if (i < C_in && o < C_out) dst[(int64_t)i * C_out + o] = (IO)(s * tile[tx][r]);
    }
}

// --- 1. planes ------------------------------------------------------------------------
// Block: 64 tokens (one per lane) x TC = 4R channels (R per wave, R = 16/S, so a
// lane's R records are 16N contiguous bytes).  When every token row (C N S
// bytes) is a whole number of 16-byte pieces, the block first copies its 64
// token segments of TC records (4N pieces each) into LDS with consecutive
// lanes on consecutive pieces (coalesced), at a row pitch of an odd number of
// pieces so that the lanes' reads of their own token's records do not collide;
// otherwise each lane loads its elements one by one.  The lane transforms its
// records in fp32 and writes each plane value to LDS rows [plane][channel]
// [token] (the raw tile's space, after a barrier), where the 64 lanes fill one
// contiguous row; the block then writes each (plane, channel) row segment of
// 64 tokens as 16-byte pieces.  Tokens T .. Tp-1 lie past the input's buffer
// range and come out as zeros.  x and dy go through the same launch
// (blockIdx.z).  Channels past C belong to the next token's row (or to
// nothing) and are transformed but never written.  (Measured on MI355X: blocks
// of 128 or 256 tokens, for longer store segments, were no faster.)
template <int N, typename IO>
struct PlanesCfg {
    static constexpr int S = (int)sizeof(IO);
    static constexpr int R = 16 / S;           // channels per lane
    static constexpr int TT = 64, TC = 4 * R;  // tokens and channels per block
    static constexpr int ROW = TT * S;         // bytes of one (plane, channel) row segment
    static constexpr int PLANES = N * TC * ROW;
    static constexpr int PPT = 4 * N;              // 16-byte pieces of a token's TC records
    static constexpr int RAW_PITCH = (PPT + 1) * 16;
    static constexpr int RAW = TT * RAW_PITCH;
    static constexpr int LDS = PLANES > RAW ? PLANES : RAW;
    static constexpr int PIECES = PLANES / 16;
    static constexpr int KC = 64 / S;              // tokens of a plane chunk: 64 bytes
    static_assert(TC * N * S == PPT * 16, "a token's TC records are 4N pieces");
    static_assert(TT % KC == 0, "a block covers whole chunks");
};

template <typename IO>
__device__ __forceinline__ float plane_elem(const uint32_t* w, int v) {
    if constexpr (sizeof(IO) == 4) return __uint_as_float(w[v]);
    else return (v & 1) ? Half<IO>::hi(w[v >> 1]) : Half<IO>::lo(w[v >> 1]);
}

template <int N, typename IO>
__global__ __launch_bounds__(256) void bw_planes_kernel(const IO* __restrict__ x, IO* __restrict__ xp, int C_in,
                                                        const IO* __restrict__ dy, IO* __restrict__ dyp, int C_out,
                                                        int64_t T, int64_t Tp) {
    using P = PlanesCfg<N, IO>;
    constexpr int S = P::S, R = P::R;
    __shared__ __attribute__((aligned(16))) char stage[P::LDS];
    const bool is_dy = blockIdx.z != 0;
    const IO* src = is_dy ? dy : x;
    IO* planes = is_dy ? dyp : xp;
    const int C = is_dy ? C_out : C_in;
    const int c0 = (int)blockIdx.y * P::TC;
    if (c0 >= C) return;  // uniform over the block: the grid spans the wider operand
    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * P::TT, t = t0 + lane;
    const int cw = c0 + wave * R;
    const uint32_t row_bytes = (uint32_t)C * N * S;
    const __amdgpu_buffer_rsrc_t rs = bw_rsrc(src, (uint32_t)(T * row_bytes));
    const uint32_t off = t < T ? (uint32_t)t * row_bytes + (uint32_t)cw * N * S : kBwOOB;

    uint32_t w[4 * N];  // R records: 16N bytes
    if ((row_bytes & 15u) == 0) {
        u32x4 v[N];
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int k = j * 256 + (int)threadIdx.x, tok = k / P::PPT, pc = k % P::PPT;
            const uint32_t o = t0 + tok < T ? (uint32_t)(t0 + tok) * row_bytes + (uint32_t)(c0 * N * S + pc * 16)
                                            : kBwOOB;
            v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int k = j * 256 + (int)threadIdx.x, tok = k / P::PPT, pc = k % P::PPT;
            *reinterpret_cast<u32x4*>(stage + tok * P::RAW_PITCH + pc * 16) = v[j];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const u32x4 e = *reinterpret_cast<const u32x4*>(stage + lane * P::RAW_PITCH + (wave * N + j) * 16);
            w[4 * j] = e[0]; w[4 * j + 1] = e[1]; w[4 * j + 2] = e[2]; w[4 * j + 3] = e[3];
        }
        __syncthreads();  // the planes reuse the raw tile's space
    } else {
#pragma unroll
        for (int v = 0; v < R * N; ++v) {
            uint32_t e;
            if constexpr (S == 4) e = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 4u * v, 0);
            else e = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, off, 2u * v, 0);
            if constexpr (S == 4) w[v] = e;
            else if (v & 1) w[v >> 1] |= e << 16;
            else w[v >> 1] = e;
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float xv[N], Pv[N];
#pragma unroll
        for (int h = 0; h < N; ++h) xv[h] = plane_elem<IO>(w, r * N + h);
        rdft_forward<N>(xv, Pv);
#pragma unroll
        for (int p = 0; p < N; ++p)
            *reinterpret_cast<IO*>(stage + (p * P::TC + wave * R + r) * P::ROW + lane * S) =
                (IO)(Pv[p] * spec_scale<IO, N>);
    }
    __syncthreads();
    constexpr int RP = P::ROW / 16;  // pieces per row
#pragma unroll
    for (int k0 = 0; k0 < P::PIECES; k0 += 256) {
        const int k = k0 + (int)threadIdx.x;
        if (P::PIECES % 256 != 0 && k >= P::PIECES) break;
        const int row = k / RP, piece = k % RP;
        const int p = row / P::TC, cl = row % P::TC;
        if (c0 + cl >= C) continue;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * P::ROW + piece * 16);
        // chunk-major: [plane][chunk of KC tokens][channel][KC tokens]
        const int64_t tk = t0 + piece * (16 / S), chunk = tk / P::KC;
        char* dst = reinterpret_cast<char*>(planes) +
                    (((int64_t)p * (Tp / P::KC) + chunk) * C + c0 + cl) * 64 + (tk % P::KC) * S;
        *reinterpret_cast<u32x4*>(dst) = v;
    }
}

// --- 2. per-bin products over tokens --------------------------------------------------
template <int N_, typename IO_, int WG_>
struct BwCfg {
    static constexpr int N = N_;
    using IO = IO_;
    static constexpr int S = (int)sizeof(IO);
    static constexpr int KC = 64 / S;          // tokens of one chunk: 64 bytes of a plane row
    static constexpr int WG = WG_;             // waves per side: WG x WG waves of 32 x 32 outputs
    static constexpr int TM = 32 * WG, TN = 32 * WG;  // output rows (o) and columns (i) per workgroup
    static constexpr int kThreads = 64 * WG * WG;
    static constexpr int H = (N - 1) / 2;      // complex bins
    static constexpr bool NYQ = N % 2 == 0 && N > 1;
    static constexpr int NB = 1 + H + (NYQ ? 1 : 0);  // bins
    static constexpr int PBYTES = TM * 64;     // one plane of one operand: TM rows x 64 bytes
    static constexpr int PL = PBYTES / 16 / kThreads;  // direct loads per thread and plane
    static constexpr int STAGE = 4 * PBYTES;   // two planes of each operand
    static constexpr int ST = 5;               // ring stages (four in flight)
    static constexpr int LDS = ST * STAGE;
    static constexpr int LOADS = 4 * PL;       // direct loads per thread and stage
    static_assert(PBYTES % (16 * kThreads) == 0, "whole loads per plane");
};

__device__ __forceinline__ void bw_mma(f32x4& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void bw_mma(f32x4& acc, const f16x8& a, const f16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void bw_mma(f32x4& acc, const f32x4& a, const f32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 bw_neg(const bf16x8& v) {
    u32x4 u = __builtin_bit_cast(u32x4, v);
    u ^= 0x80008000u;
    return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ f16x8 bw_neg(const f16x8& v) {
    u32x4 u = __builtin_bit_cast(u32x4, v);
    u ^= 0x80008000u;
    return __builtin_bit_cast(f16x8, u);
}
__device__ __forceinline__ f32x4 bw_neg(const f32x4& v) { return -v; }

template <typename IO>
struct BwFrag;
template <>
struct BwFrag<__bf16> {
    using T = bf16x8;  // 8 tokens of one row: k-values of one 16x16x32 product
};
template <>
struct BwFrag<_Float16> {
    using T = f16x8;
};
template <>
struct BwFrag<float> {
    using T = f32x4;   // 4 tokens of one row: one value for each of four 16x16x4 products
};

// Workgroup: (o, i) tile (blockIdx % tiles) and token range (blockIdx / tiles).
// Stage q = chunk * NB + bin holds, for KC tokens, the bin's planes (one for
// DC and Nyquist, real and imaginary part otherwise) of the tile's 64 dy rows
// (A) and 64 x rows (B), each row 64 bytes = 4 parts in LDS order.  The MFMA A
// operand is a 16-row block of dy planes (rows o, k = tokens), B a block of x
// planes (k = tokens, columns i): lane l ends with o = 4(l/16)+r, i = l%16.
template <class C>
__global__ __launch_bounds__(C::kThreads) void bw_gemm_kernel(const typename C::IO* __restrict__ dyp,
                                                              const typename C::IO* __restrict__ xp,
                                                              float* __restrict__ part, int C_out, int C_in,
                                                              int64_t Tp, int n_i, int tiles, int chunks_per_split,
                                                              int nchunks) {
    using IO = typename C::IO;
    using F = typename BwFrag<IO>::T;
    constexpr int N = C::N, H = C::H, NB = C::NB, ST = C::ST, S = C::S;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];

    // the tiles of one token range are consecutive logical blocks, kept on one
    // XCD: they read the same plane rows, which its L2 then serves once
    const uint32_t lb = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = (int)(lb % (uint32_t)tiles), split = (int)(lb / (uint32_t)tiles);
    const int o0 = (tile / n_i) * C::TM, i0 = (tile % n_i) * C::TN;
    const int c_begin = split * chunks_per_split;
    const int c_end = c_begin + chunks_per_split < nchunks ? c_begin + chunks_per_split : nchunks;
    const int nq = (c_end - c_begin) * NB;

    const int tid = (int)threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WG, wn = wave % C::WG;

    const uint32_t row_bytes = (uint32_t)(Tp * S);
    const uint32_t pa = (uint32_t)C_out * row_bytes, pb = (uint32_t)C_in * row_bytes;  // plane strides
    const __amdgpu_buffer_rsrc_t ra = bw_rsrc(dyp, (uint32_t)N * pa);
    const __amdgpu_buffer_rsrc_t rb = bw_rsrc(xp, (uint32_t)N * pb);

    // load l of this thread fills slot l*kThreads + tid: row slot/4, 16-byte part slot%4
    uint32_t offa[C::PL], offb[C::PL];
#pragma unroll
    for (int l = 0; l < C::PL; ++l) {
        const int slot = l * C::kThreads + tid, r = slot >> 2, u = slot & 3;
        offa[l] = o0 + r < C_out ? (uint32_t)(o0 + r) * 64u + (uint32_t)u * 16u : kBwOOB;
        offb[l] = i0 + r < C_in ? (uint32_t)(i0 + r) * 64u + (uint32_t)u * 16u : kBwOOB;
    }

    // planes of bin b: first (real part, or the only plane), second (imaginary)
    auto plane0 = [&](int b) { return b == 0 ? 0 : (b <= H ? 2 * b - 1 : N - 1); };
    auto dma = [&](int q) {
        char* st = smem + (q % ST) * C::STAGE;
        const bool live = q < nq;
        const int cq = live ? c_begin + q / NB : 0, b = live ? q % NB : 0;
        const int p0 = plane0(b);
        const bool cplx = b >= 1 && b <= H;
        // chunk cq of every plane row: C x 64 bytes per chunk (chunk-major planes)
        const uint32_t soffa = (uint32_t)cq * (uint32_t)C_out * 64u, soffb = (uint32_t)cq * (uint32_t)C_in * 64u;
        // every thread issues LOADS loads for every stage, so vmcnt counts stages
#pragma unroll
        for (int l = 0; l < C::PL; ++l) {
            const uint32_t a0 = live && offa[l] != kBwOOB ? offa[l] + (uint32_t)p0 * pa : kBwOOB;
            const uint32_t b0 = live && offb[l] != kBwOOB ? offb[l] + (uint32_t)p0 * pb : kBwOOB;
            const uint32_t a1 = live && cplx && offa[l] != kBwOOB ? a0 + pa : kBwOOB;
            const uint32_t b1 = live && cplx && offb[l] != kBwOOB ? b0 + pb : kBwOOB;
            char* d = st + (l * C::kThreads + wave * 64) * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(d), 16, a0,
                                                     soffa, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(d + C::PBYTES), 16,
                                                     a1, soffa, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (__attribute__((address_space(3))) void*)(d + 2 * C::PBYTES), 16, b0, soffb, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (__attribute__((address_space(3))) void*)(d + 3 * C::PBYTES), 16, b1, soffb, 0, 0);
        }
    };

    f32x4 acc[2][2][N];
#pragma unroll
    for (int ob = 0; ob < 2; ++ob)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int p = 0; p < N; ++p) acc[ob][ib][p] = f32x4{0.f, 0.f, 0.f, 0.f};

    // fragment of 16-row block blk of a plane region: row blk*16 + lane%16, part lane/16
    const int frag_off = (lane & 15) * 64 + (lane >> 4) * 16;
    auto frag = [&](const char* region, int blk) {
        return *reinterpret_cast<const F*>(region + blk * 1024 + frag_off);
    };

#pragma unroll
    for (int q = 0; q < ST - 1; ++q) dma(q);
    for (int q = 0; q < nq; ++q) {
        // this thread's loads of stage q are done once at most ST-2 stages remain
        __builtin_amdgcn_s_waitcnt(bw_vmcnt((ST - 2) * C::LOADS));
        asm volatile("s_barrier" ::: "memory");
        dma(q + ST - 1);
        const char* st = smem + (q % ST) * C::STAGE;
        const int b = q % NB;
        F A0[2], B0[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            A0[k] = frag(st, 2 * wm + k);
            B0[k] = frag(st + 2 * C::PBYTES, 2 * wn + k);
        }
        if (b >= 1 && b <= H) {
            F A1[2], B1[2], nA0[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                A1[k] = frag(st + C::PBYTES, 2 * wm + k);
                B1[k] = frag(st + 3 * C::PBYTES, 2 * wn + k);
                nA0[k] = bw_neg(A0[k]);
            }
            // bins are uniform across the workgroup; plane pair chosen at run time
            static_for<1, H + 1>([&](auto kc) {
                constexpr int kb = decltype(kc)::value;
                if (b == kb) {
                    constexpr int pr = 2 * kb - 1, pi = 2 * kb;
#pragma unroll
                    for (int ob = 0; ob < 2; ++ob)
#pragma unroll
                        for (int ib = 0; ib < 2; ++ib) {
                            bw_mma(acc[ob][ib][pr], A0[ob], B0[ib]);   // a c
                            bw_mma(acc[ob][ib][pi], A1[ob], B0[ib]);   // b c
                            bw_mma(acc[ob][ib][pr], A1[ob], B1[ib]);   // + b d
                            bw_mma(acc[ob][ib][pi], nA0[ob], B1[ib]);  // - a d
                        }
                }
            });
        } else {
            const int p = b == 0 ? 0 : N - 1;
            if (p == 0) {
#pragma unroll
                for (int ob = 0; ob < 2; ++ob)
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) bw_mma(acc[ob][ib][0], A0[ob], B0[ib]);
            } else if constexpr (C::NYQ) {
#pragma unroll
                for (int ob = 0; ob < 2; ++ob)
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) bw_mma(acc[ob][ib][N - 1], A0[ob], B0[ib]);
            }
        }
    }

    // partial spectra of this token range: part[split][p][o][i]
    const int64_t plane = bw_pstride(C_in, C_out);  // partial planes padded to whole 16-byte groups
    float* dst = part + (int64_t)split * N * plane;
#pragma unroll
    for (int ob = 0; ob < 2; ++ob)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            const int i = i0 + 32 * wn + 16 * ib + (lane & 15);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int o = o0 + 32 * wm + 16 * ob + 4 * (lane >> 4) + rr;
                if (o < C_out && i < C_in) {
#pragma unroll
                    for (int p = 0; p < N; ++p) dst[p * plane + (int64_t)o * C_in + i] = acc[ob][ib][p][rr];
                }
            }
        }
}

// --- 2'. per-bin products over whole tiles ---------------------------------------------
// Workgroup: one bin, one (o, i) tile of WM x WN waves (32 x 64 outputs per wave,
// up to 16 waves), one range of tokens.  The tile spans as much of C_out x C_in
// as the waves cover (all of it for 160 x 160), so each operand plane is read
// once per tile column or row instead of once per 64-wide tile, and a bin's
// workgroup reads only the bin's planes.  Stage q holds chunk q of the range:
// the bin's planes (real and imaginary part, or the one real plane) of the
// tile's TM dy rows (A) and TN x rows (B), each row 64 bytes, rows in LDS order
// [A re][A im][B re][B im]; L direct 16-byte loads per thread fill a stage
// (slots past the stage's rows, and planes a real bin lacks, read as zeros).
// Three stages in flight round a ring; the stage size is a run-time value.
template <int N_, typename IO_>
struct BinCfg {
    static constexpr int N = N_;
    using IO = IO_;
    static constexpr int S = (int)sizeof(IO);
    static constexpr int H = (N - 1) / 2;
    static constexpr int ST = 3;                // ring stages
    static constexpr int kMaxStage = 53248;     // bytes: ST stages fit the CU's LDS
};
// Two instances: up to 16 waves (128 VGPRs a lane, so at most 4 direct loads
// per thread and stage stay in registers) and up to 8 waves (256 VGPRs, up to
// 8 loads: narrower tiles such as 96 x 96 need 5).
template <int MAXT>
constexpr int bin_max_loads() { return MAXT > 512 ? 4 : 8; }

template <class C, int MAXT>
__global__ __launch_bounds__(MAXT) void bw_bin_kernel(const char* __restrict__ ws, uint32_t xp_bytes,
                                                      uint32_t span, float* __restrict__ part, int C_out,
                                                      int C_in, int64_t Tp, int WM, int WN, int n_o, int n_i,
                                                      int nb, int L, int stage_bytes, int splits_c, int cps_c,
                                                      int cps_r, int nchunks, int64_t pstride) {
    using IO = typename C::IO;
    using F = typename BwFrag<IO>::T;
    constexpr int N = C::N, H = C::H, ST = C::ST, S = C::S;
    __shared__ __attribute__((aligned(16))) char smem[ST * C::kMaxStage];

    // workgroups of the complex bins first (splits_c token ranges of cps_c chunks
    // each), then those of the real bins (DC, Nyquist: half the bytes and a
    // quarter of the products per chunk, so ranges of cps_r ~ 2 cps_c chunks)
    const uint32_t lb = xcd_remap(blockIdx.x, gridDim.x);
    const uint32_t tiles = (uint32_t)(n_i * n_o), ncw = (uint32_t)H * tiles * (uint32_t)splits_c;
    const bool cw = lb < ncw;
    const uint32_t t = cw ? lb : lb - ncw;
    const int ti = (int)(t % (uint32_t)n_i);
    const int to = (int)((t / (uint32_t)n_i) % (uint32_t)n_o);
    const uint32_t rest = t / tiles;
    const uint32_t nr = (uint32_t)(nb - H);  // real bins: 1 or 2
    constexpr uint32_t HC = H > 0 ? H : 1;  // (no complex workgroups when H = 0)
    const int bin = cw ? 1 + (int)(rest % HC) : ((rest % nr) == 0 ? 0 : H + 1);
    const int split = cw ? (int)(rest / HC) : (int)(rest / nr);
    const int chunks_per_split = cw ? cps_c : cps_r;
    const int TM = 32 * WM, TN = 64 * WN;
    const int o0 = to * TM, i0 = ti * TN;
    const bool cplx = bin >= 1 && bin <= H;
    const int p0 = bin == 0 ? 0 : (bin <= H ? 2 * bin - 1 : N - 1);
    const int c_begin = split * chunks_per_split;
    const int c_end = c_begin + chunks_per_split < nchunks ? c_begin + chunks_per_split : nchunks;
    const int nq = c_end - c_begin;

    const int threads = 64 * WM * WN;
    const int tid = (int)threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // one resource over both plane sets: x planes at 0, dy planes at xp_bytes
    const __amdgpu_buffer_rsrc_t rw = bw_rsrc(ws, span);
    const uint32_t row_bytes = (uint32_t)(Tp * S);
    const int slots = 8 * (TM + TN);
    uint32_t off[8];  // the first bin_max_loads<MAXT>() are used
#pragma unroll
    for (int l = 0; l < bin_max_loads<MAXT>(); ++l) {
        const int slot = l * threads + tid, u = slot & 3, rid = slot >> 2;
        uint32_t o = kBwOOB;
        if (l < L && slot < slots) {
            if (rid < 2 * TM) {
                const int pa = rid / TM, r = o0 + rid % TM;
                if (r < C_out && (pa == 0 || cplx))
                    o = xp_bytes + (uint32_t)(p0 + pa) * (uint32_t)C_out * row_bytes + (uint32_t)r * 64u + 16u * u;
            } else {
                const int rb = rid - 2 * TM, pb = rb / TN, r = i0 + rb % TN;
                if (r < C_in && (pb == 0 || cplx))
                    o = (uint32_t)(p0 + pb) * (uint32_t)C_in * row_bytes + (uint32_t)r * 64u + 16u * u;
            }
        }
        off[l] = o;
    }

    // chunk c of a plane starts C x 64 bytes after chunk c - 1 (chunk-major
    // planes); a wave's 64 slots of one load lie all in A or all in B (8 TM is
    // a multiple of 64), so the chunk offset is uniform per load instruction
    auto dma = [&](int q) {
        char* st = smem + (q % ST) * stage_bytes;
        const bool live = q < nq;
        const uint32_t cq = live ? (uint32_t)(c_begin + q) : 0u;
#pragma unroll
        for (int l = 0; l < bin_max_loads<MAXT>(); ++l) {
            if (l < L) {
                const bool in_a = l * threads + wave * 64 < 8 * TM;
                const uint32_t soff = cq * (uint32_t)(in_a ? C_out : C_in) * 64u;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rw, (__attribute__((address_space(3))) void*)(st + (l * threads + wave * 64) * 16), 16,
                    live ? off[l] : kBwOOB, soff, 0, 0);
            }
        }
    };
    // this thread's loads of stage q are done once at most (ST - 2) L remain
    auto wait_stage = [&]() {
        switch (L) {
            case 1: __builtin_amdgcn_s_waitcnt(bw_vmcnt((ST - 2) * 1)); break;
            case 2: __builtin_amdgcn_s_waitcnt(bw_vmcnt((ST - 2) * 2)); break;
            case 3: __builtin_amdgcn_s_waitcnt(bw_vmcnt((ST - 2) * 3)); break;
            case 4: __builtin_amdgcn_s_waitcnt(bw_vmcnt((ST - 2) * 4)); break;
            case 5: __builtin_amdgcn_s_waitcnt(bw_vmcnt((ST - 2) * 5)); break;
            case 6: __builtin_amdgcn_s_waitcnt(bw_vmcnt((ST - 2) * 6)); break;
            case 7: __builtin_amdgcn_s_waitcnt(bw_vmcnt((ST - 2) * 7)); break;
            default: __builtin_amdgcn_s_waitcnt(bw_vmcnt((ST - 2) * 8)); break;
        }
    };

    f32x4 acc[2][4][2];
#pragma unroll
    for (int ob = 0; ob < 2; ++ob)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) acc[ob][ib][0] = acc[ob][ib][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int frag_off = (lane & 15) * 64 + (lane >> 4) * 16;
    auto frag = [&](const char* region, int row) {
        return *reinterpret_cast<const F*>(region + row * 64 + frag_off);
    };

#pragma unroll
    for (int q = 0; q < ST - 1; ++q) dma(q);
    for (int q = 0; q < nq; ++q) {
        wait_stage();
        asm volatile("s_barrier" ::: "memory");
        dma(q + ST - 1);
        const char* st = smem + (q % ST) * stage_bytes;
        const char* sb = st + 2 * TM * 64;
        F A0[2], B0[4];
#pragma unroll
        for (int ob = 0; ob < 2; ++ob) A0[ob] = frag(st, wm * 32 + ob * 16);
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) B0[ib] = frag(sb, wn * 64 + ib * 16);
        if (cplx) {
            F A1[2];
#pragma unroll
            for (int ob = 0; ob < 2; ++ob) A1[ob] = frag(st, TM + wm * 32 + ob * 16);
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                const F B1 = frag(sb, TN + wn * 64 + ib * 16), nB1 = bw_neg(B1);
#pragma unroll
                for (int ob = 0; ob < 2; ++ob) {
                    bw_mma(acc[ob][ib][0], A0[ob], B0[ib]);   // a c
                    bw_mma(acc[ob][ib][1], A1[ob], B0[ib]);   // b c
                    bw_mma(acc[ob][ib][0], A1[ob], B1);       // + b d
                    bw_mma(acc[ob][ib][1], A0[ob], nB1);      // - a d
                }
            }
        } else {
#pragma unroll
            for (int ob = 0; ob < 2; ++ob)
#pragma unroll
                for (int ib = 0; ib < 4; ++ib) bw_mma(acc[ob][ib][0], A0[ob], B0[ib]);
        }
    }

    // this bin's partial planes of this token range: part[split][p][o][i]
    float* dst = part + (int64_t)split * N * pstride;
#pragma unroll
    for (int ob = 0; ob < 2; ++ob)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            const int i = i0 + wn * 64 + ib * 16 + (lane & 15);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int o = o0 + wm * 32 + ob * 16 + 4 * (lane >> 4) + rr;
                if (o < C_out && i < C_in) {
                    dst[(int64_t)p0 * pstride + (int64_t)o * C_in + i] = acc[ob][ib][0][rr];
                    if (cplx) dst[(int64_t)(p0 + 1) * pstride + (int64_t)o * C_in + i] = acc[ob][ib][1][rr];
                }
            }
        }
}

// --- small layers: transforms and products in one launch ---------------------------------
// For C_in, C_out <= 32 the plane round trip through HBM and the launches around
// it dominate, so a workgroup (4 waves) does both steps for its token chunks
// [c_begin, c_end) of 16 tokens.  Per chunk, 256 threads load the (token,
// channel) records of x and dy (zeros past T and past the channel counts, padded
// to 32), transform them in fp32 and leave the N planes in LDS ([plane][token]
// [channel], a pitch of 48 floats so that the two token rows of a 16-lane half
// sit in different banks); the next chunk's records load while wave w runs the
// products of the bins it owns, accumulating the 32 x 32 (o, i) tile of each of
// its planes.  Bins go to waves greedily by cost (a complex bin is four real
// products, a real bin one), so no plane is shared between waves and nothing is
// summed across them.  The planes stay in fp32 for both I/O types.  The partial
// spectrum of the range goes to part[split][p][o][i] for the reduction.
template <int N>
constexpr int bw_small_wave(int bin) {
    int load[4] = {0, 0, 0, 0};
    int owner = 0;
    for (int pass = 0; pass < 2; ++pass)  // complex bins first, then the real ones
        for (int k = 0; k <= N / 2; ++k) {
            const bool cplx = k > 0 && 2 * k != N;
            if ((pass == 0) != cplx) continue;
            int w = 0;
            for (int j = 1; j < 4; ++j)
                if (load[j] < load[w]) w = j;
            load[w] += cplx ? 4 : 1;
            if (k == bin) owner = w;
        }
    return owner;
}

template <int N, typename IO>
struct BwSmallCfg {
    static constexpr int TT = 16, CH = 32, PITCH = 48;
    static constexpr int PLANE = TT * PITCH;            // floats of one plane in LDS
    static constexpr int RECS = 2 * TT * CH / 256;      // records per thread per chunk (x and dy)
};

template <int N, typename IO>
__global__ __launch_bounds__(256) void bw_small_kernel(const IO* __restrict__ x, const IO* __restrict__ dy,
                                                       float* __restrict__ part, int64_t T, int C_in, int C_out,
                                                       int chunks_per_split, int nchunks) {
    using C = BwSmallCfg<N, IO>;
    __shared__ __attribute__((aligned(16))) float xs[N * C::PLANE];
    __shared__ __attribute__((aligned(16))) float ds[N * C::PLANE];
    const int tid = (int)threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int split = (int)blockIdx.x;
    const int c_begin = split * chunks_per_split;
    const int c_end = c_begin + chunks_per_split < nchunks ? c_begin + chunks_per_split : nchunks;

    // a record is whole 16-byte pieces when N * sizeof(IO) is a multiple of 16
    // (records then start 16-byte aligned: the base pointers are)
    constexpr int RB = N * (int)sizeof(IO);
    constexpr int VP = RB % 16 == 0 ? RB / 16 : 0;
    float rec[C::RECS][N];
    auto load = [&](int c) {
#pragma unroll
        for (int j = 0; j < C::RECS; ++j) {
            const int r = tid + 256 * j, rr = r % (C::TT * C::CH);
            const bool is_dy = r >= C::TT * C::CH;
            const int t = rr / C::CH, ch = rr % C::CH;
            const int64_t tok = (int64_t)c * C::TT + t;
            const int Cn = is_dy ? C_out : C_in;
            const IO* src = (is_dy ? dy : x) + (tok * Cn + ch) * N;
            const bool ok = tok < T && ch < Cn;
            if constexpr (VP > 0) {
                uint32_t w[4 * VP];
#pragma unroll
                for (int v = 0; v < VP; ++v) {
                    const u32x4 q = ok ? reinterpret_cast<const u32x4*>(src)[v] : u32x4{0u, 0u, 0u, 0u};
                    w[4 * v] = q[0];
                    w[4 * v + 1] = q[1];
                    w[4 * v + 2] = q[2];
                    w[4 * v + 3] = q[3];
                }
#pragma unroll
                for (int h = 0; h < N; ++h) {
                    if constexpr (sizeof(IO) == 4) rec[j][h] = __uint_as_float(w[h]);
                    else rec[j][h] = (h & 1) ? Half<IO>::hi(w[h >> 1]) : Half<IO>::lo(w[h >> 1]);
                }
            } else {
#pragma unroll
                for (int h = 0; h < N; ++h) rec[j][h] = ok ? (float)src[h] : 0.0f;
            }
        }
    };

    // accumulators of this wave's planes: bin k -> planes (2k-1, 2k) or one real plane
    f32x4 acc[N][2][2];
#pragma unroll
    for (int p = 0; p < N; ++p)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) acc[p][a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (c_begin < c_end) load(c_begin);
    for (int c = c_begin; c < c_end; ++c) {
#pragma unroll
        for (int j = 0; j < C::RECS; ++j) {
            const int r = tid + 256 * j, rr = r % (C::TT * C::CH);
            float* dstp = (r >= C::TT * C::CH ? ds : xs) + (rr / C::CH) * C::PITCH + rr % C::CH;
            float P[N];
            rdft_forward<N>(rec[j], P);
#pragma unroll
            for (int p = 0; p < N; ++p) dstp[p * C::PLANE] = P[p];
        }
        __syncthreads();
        if (c + 1 < c_end) load(c + 1);  // in flight during the products
        const int row = lane >> 4, col = lane & 15;
        static_for<0, N / 2 + 1>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            constexpr bool cplx = k > 0 && 2 * k != N;
            constexpr int pr = k == 0 ? 0 : (cplx ? 2 * k - 1 : N - 1);
            constexpr int pi = cplx ? 2 * k : pr;
            if (wave != bw_small_wave<N>(k)) return;
#pragma unroll
            for (int ks = 0; ks < C::TT / 4; ++ks) {
                const int off = (4 * ks + row) * C::PITCH + col;
                float a[2], b[2], cc[2], d[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    a[h] = ds[pr * C::PLANE + off + 16 * h];
                    cc[h] = xs[pr * C::PLANE + off + 16 * h];
                    if constexpr (cplx) {
                        b[h] = ds[pi * C::PLANE + off + 16 * h];
                        d[h] = xs[pi * C::PLANE + off + 16 * h];
                    }
                }
#pragma unroll
                for (int to = 0; to < 2; ++to)
#pragma unroll
                    for (int ti = 0; ti < 2; ++ti) {
                        // Re C += a c + b d, Im C += b c - a d (DY = a + ib, X = c + id)
                        acc[pr][to][ti] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[to], cc[ti], acc[pr][to][ti], 0, 0, 0);
                        if constexpr (cplx) {
                            acc[pr][to][ti] = __builtin_amdgcn_mfma_f32_16x16x4f32(b[to], d[ti], acc[pr][to][ti], 0, 0, 0);
                            acc[pi][to][ti] = __builtin_amdgcn_mfma_f32_16x16x4f32(b[to], cc[ti], acc[pi][to][ti], 0, 0, 0);
                            acc[pi][to][ti] = __builtin_amdgcn_mfma_f32_16x16x4f32(-a[to], d[ti], acc[pi][to][ti], 0, 0, 0);
                        }
                    }
            }
        });
        __syncthreads();  // the next chunk's planes overwrite these
    }

    const int64_t plane = bw_pstride(C_in, C_out);  // partial planes padded to whole 16-byte groups
    float* dst = part + (int64_t)split * N * plane;
    static_for<0, N / 2 + 1>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        constexpr bool cplx = k > 0 && 2 * k != N;
        constexpr int pr = k == 0 ? 0 : (cplx ? 2 * k - 1 : N - 1);
        if (wave != bw_small_wave<N>(k)) return;
#pragma unroll
        for (int h = 0; h < (cplx ? 2 : 1); ++h) {
            const int p = pr + h;
#pragma unroll
            for (int to = 0; to < 2; ++to)
#pragma unroll
                for (int ti = 0; ti < 2; ++ti) {
                    const int i = 16 * ti + (lane & 15);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int o = 16 * to + 4 * (lane >> 4) + rr;
                        if (o < C_out && i < C_in) dst[p * plane + (int64_t)o * C_in + i] = acc[p][to][ti][rr];
                    }
                }
        }
    });
}

// --- 2b. transforms and products in one launch (16-bit, N = 2, 4, 6, 8) ------------
// Workgroup: one 64 x 64 (o, i) tile, every kept bin, one range of 32-token
// chunks; eight waves, wave (wm, wn) owning outputs o in 32 wm + [0, 32) and
// i in 16 wn + [0, 16).  Per chunk, the tile's 64 dy rows and 64 x rows are
// transformed on the matrix cores straight from their records, and every plane
// of both operands goes to LDS; the products then read them from there.  No
// plane reaches HBM: x and dy are read once per tile row or column of the
// output (the planes path writes both plane sets out and reads them back).
//
// Transform: a record fragment is 16 tokens x 4 channels of one operand, one
// record per lane (token l%16, channel l/16; its N elements as the lane's
// k-values, zeros after).  As the A operand against the coefficient fragment
//   B[(g', h)][(g, i)] = coef(plane 4m + i, element h) if g == g' else 0
// it returns, per lane, 4 consecutive tokens (rows 4(l/16) .. +3) of one
// channel g = (l%16)/4 and one plane 4m + i, i = l%4: 8 bytes of that plane's
// row in LDS.  The coefficients are those of the planes path (the spectrum of
// x and dy; of x/N and dy/N for fp16) rounded to the I/O type, and the
// operands of the products are the transform's fp32 outputs rounded once.
//
// LDS: per chunk N planes x {dy, x} x 64 rows x 64 bytes (32 tokens), for two
// chunks (one multiplied while the next is written); the 16-byte parts of a
// row of plane p sit at part ^ (p & 3).  A lane reads each record (2N bytes, N
// even: dword-aligned) with one 16-byte load, two chunks ahead, into
// registers; window bytes past the record are masked off, and those past the
// operand's end read as zeros.
//
// Measured on MI355X, cache-cold, against the planes path (planes, per-bin
// products, reduction): N = 8, 12608 tokens, 96 -> 96 38 -> 32 us, 96 -> 384
// 74 -> 66 us, 384 -> 96 70 -> 67 us; but C7 160 -> 160 (32768 tokens, odd N:
// records on 2-byte boundaries) 101 -> 106 us.  Odd orders keep the planes
// path.  The per-lane record loads read rows 2 N C bytes apart, and each x and
// dy row is read once per 64-wide tile of the other axis.  (A row-dependent
// swizzle that halved the fragment reads' bank conflicts, 15 -> 12 % of
// cycles, made the kernel 20 % slower: the reads lost their immediate offsets.)
template <int N_, typename IO_>
struct BwXfCfg {
    static constexpr int N = N_;
    using IO = IO_;
    using F8 = typename Half<IO_>::x8;
    static constexpr int KC = 32;               // tokens per chunk: the K of one product
    static constexpr int TM = 64, TN = 64;      // output rows (o) and columns (i) per workgroup
    static constexpr int kWaves = 8, kThreads = 64 * kWaves;
    static constexpr int H = (N_ - 1) / 2;
    static constexpr bool NYQ = N_ % 2 == 0;
    static constexpr int MQ = (N_ + 3) / 4;     // transform products per record fragment
    static constexpr int NF = 64 / kWaves;      // record fragments per wave and chunk
    static constexpr int REGION = 64 * 64;      // one plane of one operand: 64 rows x 64 bytes
    static constexpr int BUF = N_ * 2 * REGION;
    static constexpr int LDS = 2 * BUF;
    static_assert(N_ >= 2 && N_ <= 8 && N_ % 2 == 0, "one dword-aligned record per 8 k-values");
    static_assert(LDS <= 163840, "two chunks of planes fit the CU's LDS");
};

template <class C>
__global__ __launch_bounds__(C::kThreads) void bw_xf_kernel(const typename C::IO* __restrict__ x,
                                                            const typename C::IO* __restrict__ dy,
                                                            float* __restrict__ part, int64_t T, int C_out, int C_in,
                                                            int n_i, int tiles, int chunks_per_split, int nchunks) {
    using IO = typename C::IO;
    using F8 = typename C::F8;
    constexpr int N = C::N, H = C::H, MQ = C::MQ, NF = C::NF;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];

    // the tiles of one token range are consecutive logical blocks, kept on one
    // XCD: they read the same x and dy rows, which its L2 then serves once
    const uint32_t lb = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = (int)(lb % (uint32_t)tiles), split = (int)(lb / (uint32_t)tiles);
    const int o0 = (tile / n_i) * C::TM, i0 = (tile % n_i) * C::TN;
    const int c_begin = split * chunks_per_split;
    const int c_end = c_begin + chunks_per_split < nchunks ? c_begin + chunks_per_split : nchunks;
    const int nq = c_end - c_begin;

    const int tid = (int)threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;

    // Record fragments: wave w transforms fragments F = w NF + f: operand
    // F / 32 (0: dy rows o, waves 0-3; 1: x rows i, waves 4-7), channel group
    // (F % 32) / 2 of four rows, token half F % 2.
    const int rs = wave >= 4 ? 1 : 0;
    const int Crs = rs ? C_in : C_out, r0 = rs ? i0 : o0;
    constexpr uint32_t rec_b = 2u * N;  // bytes of one record
    const uint32_t row_b = (uint32_t)Crs * rec_b;
    const uint32_t rbytes = (uint32_t)(T * Crs) * rec_b;  // the operand's extent
    const __amdgpu_buffer_rsrc_t rr = rs ? bw_rsrc(x, rbytes) : bw_rsrc(dy, rbytes);
    uint32_t roff[NF];  // this lane's record at chunk 0 (or out of range)
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const int F = wave * NF + f, g16 = (F & 31) >> 1, th = F & 1;
        const int row = r0 + 4 * g16 + (lane >> 4), tok = 16 * th + (lane & 15);
        roff[f] = row < Crs ? (uint32_t)tok * row_b + (uint32_t)row * rec_b : kBwOOB;
    }
    // a fragment whose four channels all lie past the operand's rows is skipped
    // (uniform across the wave): its rows are never read
    auto frag_live = [&](int f) { return r0 + 4 * (((wave * NF + f) & 31) >> 1) < Crs; };
    const uint32_t chunk_b = (uint32_t)C::KC * row_b;  // chunk advance (scalar)
    auto load = [&](int q, u32x4 (&W)[NF]) {
        const bool live = q < nq;
        // (uniform: a scalar offset; stated, or the compiler loops over lanes)
        const uint32_t soff = __builtin_amdgcn_readfirstlane(live ? (uint32_t)(c_begin + q) * chunk_b : 0u);
#pragma unroll
        for (int f = 0; f < NF; ++f)
            W[f] = __builtin_amdgcn_raw_buffer_load_b128(rr, live && frag_live(f) ? roff[f] : kBwOOB, soff, 0);
    };
    // coefficient fragments (B operand): lane (k-group g' = l/16, column
    // j = l%16 = (g, i)) holds coef(4m + i, h), h = 0..7, if g == g'
    F8 Fb[MQ];
    {
        const int gp = lane >> 4, j = lane & 15, g = j >> 2, i = j & 3;
        static_for<0, MQ>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            float v[8];
#pragma unroll
            for (int h = 0; h < 8; ++h) v[h] = 0.0f;
            static_for<0, 4>([&](auto ic) {
                constexpr int ii = decltype(ic)::value;
                constexpr int p = 4 * m + ii;
                if constexpr (p < N) {
                    static_for<0, N>([&](auto hc) {
                        constexpr int h = decltype(hc)::value;
                        constexpr float c = (float)(fwd_coef<N>(p, h) * (double)spec_scale<IO, N>);
                        v[h] = i == ii ? c : v[h];
                    });
                }
            });
            u32x4 u;
#pragma unroll
            for (int q = 0; q < 4; ++q) u[q] = g == gp ? Half<IO>::pack2(v[2 * q], v[2 * q + 1]) : 0u;
            Fb[m] = __builtin_bit_cast(F8, u);
        });
    }

    // LDS address of part u of row r of plane p of operand o_ (0: dy, 1: x)
    auto plane_at = [&](char* buf, int p, int o_, int r, int u) {
        return buf + (p * 2 + o_) * C::REGION + r * 64 + ((u ^ (p & 3)) << 4);
    };

    // transform the chunk held in W into buf
    auto transform = [&](const u32x4 (&W)[NF], char* buf) {
        const int j = lane & 15, g = j >> 2, ii = j & 3, kq = lane >> 4;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            if (!frag_live(f)) continue;
            const int F = wave * NF + f, g16 = (F & 31) >> 1, th = F & 1;
            // the record's N elements, zeros after
            u32x4 e = W[f];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (2 * q >= N) e[q] = 0u;
            const F8 a = __builtin_bit_cast(F8, e);
            const int r = 4 * g16 + g;
            // tokens 16 th + 4 kq .. + 3: part 2 th + kq / 2, half kq % 2
            const int u = 2 * th + (kq >> 1);
            static_for<0, MQ>([&](auto mc) {
                constexpr int m = decltype(mc)::value;
                f32x4 d = {0.f, 0.f, 0.f, 0.f};
                bw_mma(d, a, Fb[m]);
                const int p = 4 * m + ii;
                if (p < N)
                    *reinterpret_cast<u32x2*>(plane_at(buf, p, rs, r, u) + ((kq & 1) << 3)) =
                        u32x2{Half<IO>::pack2(d[0], d[1]), Half<IO>::pack2(d[2], d[3])};
            });
        }
    };

    f32x4 acc[2][N];
#pragma unroll
    for (int ob = 0; ob < 2; ++ob)
#pragma unroll
        for (int p = 0; p < N; ++p) acc[ob][p] = f32x4{0.f, 0.f, 0.f, 0.f};

    // fragment of 16-row block blk of plane p of operand o_: row 16 blk + l%16,
    // tokens 8 (l/16) .. + 7
    auto frag = [&](char* buf, int p, int o_, int blk) {
        return *reinterpret_cast<const F8*>(plane_at(buf, p, o_, 16 * blk + (lane & 15), lane >> 4));
    };
    auto products = [&](char* buf) {
        static_for<0, H + 1 + (C::NYQ ? 1 : 0)>([&](auto bc) {
            constexpr int b = decltype(bc)::value;
            constexpr bool cplx = b >= 1 && b <= H;
            constexpr int pr = b == 0 ? 0 : (cplx ? 2 * b - 1 : N - 1), pi = pr + 1;
            F8 A0[2];
            const F8 B0 = frag(buf, pr, 1, wn);
#pragma unroll
            for (int ob = 0; ob < 2; ++ob) A0[ob] = frag(buf, pr, 0, 2 * wm + ob);
            if constexpr (cplx) {
                F8 A1[2];
                const F8 B1 = frag(buf, pi, 1, wn);
#pragma unroll
                for (int ob = 0; ob < 2; ++ob) A1[ob] = frag(buf, pi, 0, 2 * wm + ob);
#pragma unroll
                for (int ob = 0; ob < 2; ++ob) {
                    bw_mma(acc[ob][pr], A0[ob], B0);          // a c
                    bw_mma(acc[ob][pi], A1[ob], B0);          // b c
                    bw_mma(acc[ob][pr], A1[ob], B1);          // + b d
                    bw_mma(acc[ob][pi], bw_neg(A0[ob]), B1);  // - a d
                }
            } else {
#pragma unroll
                for (int ob = 0; ob < 2; ++ob) bw_mma(acc[ob][pr], A0[ob], B0);
            }
        });
    };

    // Two chunks in flight: the records of chunk q + 2 load while chunk q's
    // planes are multiplied.  One barrier per chunk: after it chunk q's planes
    // are in, and every wave is done with chunk q - 1's, whose buffer chunk
    // q + 1 then takes.
    u32x4 W0[NF], W1[NF];
    load(0, W0);
    load(1, W1);
    for (int q = 0; q < nq;) {
        {
            char* buf = smem + (q & 1) * C::BUF;
            transform(W0, buf);
            load(q + 2, W0);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            products(buf);
        }
        if (++q >= nq) break;
        {
            char* buf = smem + (q & 1) * C::BUF;
            transform(W1, buf);
            load(q + 2, W1);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            products(buf);
        }
        ++q;
    }

    // partial spectra of this token range: part[split][p][o][i]
    const int64_t plane = bw_pstride(C_in, C_out);  // partial planes padded to whole 16-byte groups
    float* dst = part + (int64_t)split * N * plane;
    const int i = i0 + 16 * wn + (lane & 15);
#pragma unroll
    for (int ob = 0; ob < 2; ++ob)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int o = o0 + 32 * wm + 16 * ob + 4 * (lane >> 4) + r;
            if (o < C_out && i < C_in) {
#pragma unroll
                for (int p = 0; p < N; ++p) dst[p * plane + (int64_t)o * C_in + i] = acc[ob][p][r];
            }
        }
}

// --- 3. reduction and inverse transform ------------------------------------------------
// Block: 32 G consecutive (o, i) elements (G = 4 per lane, 16-byte loads, for
// planes of at least 128 such blocks; else G = 1.  Measured on MI355X: 96 x 96
// reduces in 6.2 us at G = 1 against 6.8 at G = 4 (72 blocks), 160 x 160 in
// 10.5 us at G = 4 against 15.6 at G = 2 and 11.2 at G = 1) x N planes x R lanes
// (R = 1024 / 32N, at most 8).  Lane r of (p, group) sums the r-th contiguous
// sub-range of the splits in order, sixteen loads in flight; the R sub-sums
// are added in lane order.  The order is fixed, so the result is
// deterministic.  Then one thread per element runs the inverse real DFT of its
// packed spectrum and writes dw[o][i][0 .. N-1].
template <int N, int G>
struct BwReduceCfg {
    static constexpr int R0 = 1024 / (32 * N);
    static constexpr int R = R0 > 8 ? 8 : R0;
    static constexpr int kThreads = 32 * N * R;
    static constexpr int EL = 32 * G;  // elements per block
    using V = std::conditional_t<G == 4, f32x4, float>;
    static_assert(G == 1 || G == 4, "one element or a 16-byte group per lane");
    static_assert(kThreads >= EL, "a thread per element for the inverse transform");
};

template <int N, int G>
__global__ __launch_bounds__((BwReduceCfg<N, G>::kThreads)) void bw_reduce_kernel(const float* __restrict__ part,
                                                                                float* __restrict__ dw, int splits_c,
                                                                                int splits_r, int64_t plane,
                                                                                int64_t pstride, float post) {
    using RC = BwReduceCfg<N, G>;
    using V = typename RC::V;
    constexpr int R = RC::R;
    __shared__ V red[R][32][N];
    const int g = (int)threadIdx.x & 31, p = ((int)threadIdx.x >> 5) % N, r = (int)threadIdx.x / (32 * N);
    const int64_t e0 = (int64_t)blockIdx.x * RC::EL + G * g;
    // the DC and Nyquist planes may have their own number of token ranges
    const int splits = (p == 0 || (N % 2 == 0 && p == N - 1)) ? splits_r : splits_c;
    const int len = (splits + R - 1) / R;
    const int s0 = r * len, s1 = s0 + len < splits ? s0 + len : splits;
    V v = {};
    if (e0 < pstride) {  // pstride is a multiple of 4: a group lies inside the padded plane
        const V* src = reinterpret_cast<const V*>(part + (int64_t)p * pstride + e0);
        const int64_t step = (int64_t)N * pstride / G;
        int s = s0;
        for (; s + 16 <= s1; s += 16) {
            V t[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) t[j] = src[(int64_t)(s + j) * step];
#pragma unroll
            for (int j = 0; j < 16; ++j) v += t[j];
        }
        for (; s < s1; ++s) v += src[(int64_t)s * step];
    }
    red[r][g][p] = v;
    __syncthreads();
    const int q = (int)threadIdx.x;  // element of the block
    const int64_t e = (int64_t)blockIdx.x * RC::EL + q;
    if (q < RC::EL && e < plane) {
        auto comp = [&](const V& w) {
            if constexpr (G > 1) return w[q % G];
            else return w;
        };
        float P[N], y[N];
#pragma unroll
        for (int k = 0; k < N; ++k) {
            float sum = comp(red[0][q / G][k]);
#pragma unroll
            for (int rr = 1; rr < R; ++rr) sum += comp(red[rr][q / G][k]);
            P[k] = sum * post;
        }
        rdft_inverse<N>(P, y);
#pragma unroll
        for (int m = 0; m < N; ++m) dw[e * N + m] = y[m];
    }
}

template <int N>
// post: the scale of the summed spectra (N^2 for fp16 planes, which hold the
// spectra of x/N and dy/N; 1 otherwise)
void launch_bw_reduce(const float* part, float* dw, int splits, int splits_r, int64_t plane, int64_t pstride,
                      hipStream_t stream, float post = 1.0f) {
    if (plane >= 128 * BwReduceCfg<N, 4>::EL) {
        using RC = BwReduceCfg<N, 4>;
        hipLaunchKernelGGL((bw_reduce_kernel<N, 4>), dim3((uint32_t)((plane + RC::EL - 1) / RC::EL)),
                           dim3(RC::kThreads), 0, stream, part, dw, splits, splits_r, plane, pstride, post);
    } else {
        using RC = BwReduceCfg<N, 1>;
        hipLaunchKernelGGL((bw_reduce_kernel<N, 1>), dim3((uint32_t)((plane + RC::EL - 1) / RC::EL)),
                           dim3(RC::kThreads), 0, stream, part, dw, splits, splits_r, plane, pstride, post);
    }
}

// --- host side ---------------------------------------------------------------------------

struct BwShape {
    int64_t Tp;
    int n_o, n_i, tiles, nchunks, splits, chunks_per_split;
    bool fused;  // small layers: transforms and products in one launch, no planes
    bool xf;     // 16-bit, N = 2, 4, 6, 8: transforms inside the product kernel (bw_xf_kernel)
    bool bin;    // products per bin over whole tiles (bw_bin_kernel)
    int WM, WN, nb, L, stage_bytes;
    int splits_r, chunks_per_split_r;  // token ranges of the real bins (the others: splits)
    size_t xp_bytes, dyp_bytes, part_bytes, total;
};

// Tile of the bin-major product kernel: WM x WN waves of 32 x 64 outputs (at most
// 16 waves, one stage of at most kMaxStage bytes), the tile counts that stream
// the fewest plane rows per token (n_i C_out + n_o C_in).  False if none fits.
bool bw_bin_tile(int C_in, int C_out, BwShape& s) {
    const int WMt = (C_out + 31) / 32, WNt = (C_in + 63) / 64;
    int64_t best = -1;
    for (int no = 1; no <= WMt; ++no)
        for (int ni = 1; ni <= WNt; ++ni) {
            const int WM = (WMt + no - 1) / no, WN = (WNt + ni - 1) / ni;
            if (WM * WN > 16) continue;
            const int threads = 64 * WM * WN, slots = 8 * (32 * WM + 64 * WN);
            const int L = (slots + threads - 1) / threads;
            const int max_loads = WM * WN <= 8 ? bin_max_loads<512>() : bin_max_loads<1024>();
            if (L > max_loads || L * threads * 16 > BinCfg<1, float>::kMaxStage) continue;
            const int n_o = (C_out + 32 * WM - 1) / (32 * WM), n_i = (C_in + 64 * WN - 1) / (64 * WN);
            const int64_t cost = (int64_t)n_i * C_out + (int64_t)n_o * C_in;
            if (best < 0 || cost < best) {
                best = cost;
                s.WM = WM; s.WN = WN; s.n_o = n_o; s.n_i = n_i; s.L = L; s.stage_bytes = L * threads * 16;
            }
        }
    return best >= 0;
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }


BwShape bw_shape(int N, int io, int64_t T, int C_in, int C_out) {
    BwShape s{};
    if (C_in <= 32 && C_out <= 32) {
        // one fused launch: token chunks of 16 over at most 256 workgroups, two
        // chunks or more each where the tokens allow (the second chunk's loads
        // then overlap the first one's products; c2: 13.0 us at 128 ranges, 15.0
        // at 256 or 64)
        s.fused = true;
        s.Tp = (T + 15) / 16 * 16;
        s.tiles = 1;
        s.nchunks = (int)(s.Tp / 16);
        int sp = s.nchunks / 2;
        sp = sp < 1 ? 1 : (sp > 256 ? 256 : sp);
        s.chunks_per_split = (s.nchunks + sp - 1) / sp;
        s.splits = (s.nchunks + s.chunks_per_split - 1) / s.chunks_per_split;
        s.part_bytes = round256((size_t)s.splits * N * bw_pstride(C_in, C_out) * 4);
        s.total = s.part_bytes;
        return s;
    }
    const int S = io == kIoF32 ? 4 : 2, KC = 64 / S;
    if (io != kIoF32 && N >= 2 && N <= 8 && N % 2 == 0) {
        // one launch of 64 x 64 tiles over 32-token chunks, then the reduction;
        // token ranges give about one workgroup per CU (two chunks or more each)
        const int64_t Tp = (T + 31) / 32 * 32;
        if ((int64_t)N * C_in * Tp * S < ((int64_t)1 << 31) && (int64_t)N * C_out * Tp * S < ((int64_t)1 << 31)) {
            s.xf = true;
            s.Tp = Tp;
            s.nchunks = (int)(Tp / 32);
            s.n_o = (C_out + 63) / 64;
            s.n_i = (C_in + 63) / 64;
            s.tiles = s.n_o * s.n_i;
            const int64_t cap = s.nchunks / 2 > 0 ? s.nchunks / 2 : 1;
            int64_t sp = 256 / s.tiles;
            sp = sp < 1 ? 1 : (sp > cap ? cap : sp);
            s.chunks_per_split = (int)((s.nchunks + sp - 1) / sp);
            s.splits = (s.nchunks + s.chunks_per_split - 1) / s.chunks_per_split;
            s.part_bytes = round256((size_t)s.splits * N * bw_pstride(C_in, C_out) * 4);
            s.total = s.part_bytes;
            return s;
        }
    }
    const int tm = 64;  // bw_gemm_kernel tiles: 2 x 2 waves of 32 x 32
    const int H = (N - 1) / 2;
    s.nb = 1 + H + ((N % 2 == 0 && N > 1) ? 1 : 0);
    s.Tp = (T + 63) / 64 * 64;
    s.nchunks = (int)(s.Tp / KC);
    // the per-bin kernel reaches both plane sets through one resource: under
    // 2 GiB together (otherwise the 64 x 64 kernel, whose limit is per set)
    const size_t both = round256((size_t)N * C_in * s.Tp * S) + round256((size_t)N * C_out * s.Tp * S);
    s.bin = both < ((size_t)1 << 31) && bw_bin_tile(C_in, C_out, s);
    if (s.bin) {
        // one workgroup per CU (the ring takes most of its LDS): bins x tiles x
        // token ranges of at least two chunks, about 256 in all
        // a real bin's workgroup costs about half a complex one (half the bytes;
        // its bytes, not its quarter of the products, set the pace), so it takes
        // ranges twice as long: H S + nr S / 2 workgroups per tile in all (on
        // MI355X three and four times as long were slower: c4 104 and 114 us
        // against 95)
        s.tiles = s.n_o * s.n_i;
        const int nr = s.nb - H;
        const int64_t cap = s.nchunks / 2 > 0 ? s.nchunks / 2 : 1;
        int64_t sp = (int64_t)(512 / (s.tiles * (2 * H + nr)));
        sp = sp < 1 ? 1 : (sp > cap ? cap : sp);
        s.chunks_per_split = (int)((s.nchunks + sp - 1) / sp);
        s.splits = (s.nchunks + s.chunks_per_split - 1) / s.chunks_per_split;
        s.chunks_per_split_r = H > 0 ? 2 * s.chunks_per_split : s.chunks_per_split;
        s.splits_r = (s.nchunks + s.chunks_per_split_r - 1) / s.chunks_per_split_r;
        s.xp_bytes = round256((size_t)N * C_in * s.Tp * S);
        s.dyp_bytes = round256((size_t)N * C_out * s.Tp * S);
        const int smax = s.splits > s.splits_r ? s.splits : s.splits_r;
        s.part_bytes = round256((size_t)smax * N * bw_pstride(C_in, C_out) * 4);
        s.total = s.xp_bytes + s.dyp_bytes + s.part_bytes;
        return s;
    }
    s.n_o = (C_out + tm - 1) / tm;
    s.n_i = (C_in + tm - 1) / tm;
    s.tiles = s.n_o * s.n_i;
    // token ranges: enough to give every CU two workgroups (ranges of four
    // chunks or more).  The product loop waits on its ring once per stage, and a second
    // workgroup on the CU fills those waits: on MI355X 512 workgroups ran c4
    // (C7, 160 -> 160, T = 32768) in 132 us against 174 at 256 and 149 at 1024
    // (more ranges, more partial spectra to write and sum); a deeper ring at one
    // workgroup per CU instead was slower still (252 us at nine stages).
    const int64_t want = (512 + s.tiles - 1) / s.tiles;
    const int64_t cap = s.nchunks / 4;
    int64_t sp = want < cap ? want : cap;
    sp = sp < 1 ? 1 : (sp > s.nchunks ? s.nchunks : sp);
    s.chunks_per_split = (int)((s.nchunks + sp - 1) / sp);
    s.splits = (s.nchunks + s.chunks_per_split - 1) / s.chunks_per_split;
    s.xp_bytes = round256((size_t)N * C_in * s.Tp * S);
    s.dyp_bytes = round256((size_t)N * C_out * s.Tp * S);
    s.part_bytes = round256((size_t)s.splits * N * bw_pstride(C_in, C_out) * 4);
    s.total = s.xp_bytes + s.dyp_bytes + s.part_bytes;
    return s;
}

template <int N, typename IO>
hipError_t run_backward_weight(const void* x, const void* dy, float* dw, int64_t T, int C_in, int C_out,
                               char* ws, const BwShape& s, hipStream_t stream) {
    using Cfg = BwCfg<N, IO, 2>;
    const int64_t plane = (int64_t)C_out * C_in, pstride = bw_pstride(C_in, C_out);
    if (s.fused) {
        float* part = reinterpret_cast<float*>(ws);
        hipLaunchKernelGGL((bw_small_kernel<N, IO>), dim3((uint32_t)s.splits), dim3(256), 0, stream, (const IO*)x,
                           (const IO*)dy, part, T, C_in, C_out, s.chunks_per_split, s.nchunks);
        launch_bw_reduce<N>(part, dw, s.splits, s.splits, plane, pstride, stream);
        return hipGetLastError();
    }
    if constexpr (!std::is_same_v<IO, float> && N >= 2 && N <= 8 && N % 2 == 0) {
        if (s.xf) {
            using XC = BwXfCfg<N, IO>;
            float* part = reinterpret_cast<float*>(ws);
            hipLaunchKernelGGL((bw_xf_kernel<XC>), dim3((uint32_t)(s.tiles * s.splits)), dim3(XC::kThreads), 0, stream,
                               (const IO*)x, (const IO*)dy, part, T, C_out, C_in, s.n_i, s.tiles, s.chunks_per_split,
                               s.nchunks);
            launch_bw_reduce<N>(part, dw, s.splits, s.splits, plane, pstride, stream,
                                spec_unscale<IO, N> * spec_unscale<IO, N>);
            return hipGetLastError();
        }
    }
    IO* xp = reinterpret_cast<IO*>(ws);
    IO* dyp = reinterpret_cast<IO*>(ws + s.xp_bytes);
    float* part = reinterpret_cast<float*>(ws + s.xp_bytes + s.dyp_bytes);
    using PC = PlanesCfg<N, IO>;  // Tp is a multiple of 64 = PC::TT
    const int cmax = C_in > C_out ? C_in : C_out;
    const dim3 gp((uint32_t)(s.Tp / PC::TT), (uint32_t)((cmax + PC::TC - 1) / PC::TC), 2);
    hipLaunchKernelGGL((bw_planes_kernel<N, IO>), gp, dim3(256), 0, stream, (const IO*)x, xp, C_in, (const IO*)dy,
                       dyp, C_out, T, s.Tp);
    if (s.bin) {
        using BC = BinCfg<N, IO>;
        constexpr int H = (N - 1) / 2;
        const int64_t bwgs = (int64_t)s.tiles * (H * s.splits + (s.nb - H) * s.splits_r);
        auto kern = s.WM * s.WN <= 8 ? bw_bin_kernel<BC, 512> : bw_bin_kernel<BC, 1024>;
        hipLaunchKernelGGL(kern, dim3((uint32_t)bwgs), dim3(64 * s.WM * s.WN), 0, stream, (const char*)ws,
                           (uint32_t)s.xp_bytes, (uint32_t)(s.xp_bytes + s.dyp_bytes), part, C_out, C_in, s.Tp, s.WM,
                           s.WN, s.n_o, s.n_i, s.nb, s.L, s.stage_bytes, s.splits, s.chunks_per_split,
                           s.chunks_per_split_r, s.nchunks, pstride);
        launch_bw_reduce<N>(part, dw, s.splits, s.splits_r, plane, pstride, stream,
                            spec_unscale<IO, N> * spec_unscale<IO, N>);
        return hipGetLastError();
    }
    const int64_t wgs = (int64_t)s.tiles * s.splits;
    hipLaunchKernelGGL((bw_gemm_kernel<Cfg>), dim3((uint32_t)wgs), dim3(Cfg::kThreads), 0, stream,
                       (const IO*)dyp, (const IO*)xp, part, C_out, C_in, s.Tp, s.n_i, s.tiles,
                       s.chunks_per_split, s.nchunks);
    launch_bw_reduce<N>(part, dw, s.splits, s.splits, plane, pstride, stream,
                        spec_unscale<IO, N> * spec_unscale<IO, N>);
    return hipGetLastError();
}

template <typename IO>
hipError_t dispatch_backward_weight(int N, const void* x, const void* dy, float* dw, int64_t T, int C_in,
                                    int C_out, char* ws, const BwShape& s, hipStream_t stream) {
    switch (N) {
#define EQL_BW(n)                                                                           \
    case n:                                                                                 \
        return run_backward_weight<n, IO>(x, dy, dw, T, C_in, C_out, ws, s, stream);
        EQL_BW(1) EQL_BW(2) EQL_BW(3) EQL_BW(4) EQL_BW(5) EQL_BW(6) EQL_BW(7) EQL_BW(8)
        EQL_BW(9) EQL_BW(10) EQL_BW(11) EQL_BW(12) EQL_BW(13) EQL_BW(14) EQL_BW(15) EQL_BW(16)
#undef EQL_BW
        default: return hipErrorInvalidValue;
    }
}

__global__ __launch_bounds__(256) void bw_zero_kernel(float* __restrict__ p, int64_t n) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e < n) p[e] = 0.0f;
}

}  // namespace

hipError_t launch_w_hat_adjoint(int N, int io, const void* w_hat, void* w_hat_adj, int C_in, int C_out,
                                hipStream_t stream) {
    const dim3 grid((uint32_t)((C_in + 31) / 32), (uint32_t)((C_out + 31) / 32), (uint32_t)N);
    if (grid.y > 65535u) return hipErrorInvalidConfiguration;
    if (io == kIoF16)
        hipLaunchKernelGGL(w_hat_adjoint_kernel<_Float16>, grid, dim3(256), 0, stream, (const _Float16*)w_hat,
                           (_Float16*)w_hat_adj, N, C_in, C_out);
    else if (io == kIoBF16)
        hipLaunchKernelGGL(w_hat_adjoint_kernel<__bf16>, grid, dim3(256), 0, stream, (const __bf16*)w_hat,
                           (__bf16*)w_hat_adj, N, C_in, C_out);
    else
        hipLaunchKernelGGL(w_hat_adjoint_kernel<float>, grid, dim3(256), 0, stream, (const float*)w_hat,
                           (float*)w_hat_adj, N, C_in, C_out);
    return hipGetLastError();
}

size_t backward_weight_workspace(int N, int io, int64_t T, int C_in, int C_out) {
    if (T <= 0) return 0;
    return bw_shape(N, io, T, C_in, C_out).total;
}

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch` on each device, once known
}  // namespace

hipError_t noalloc_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_cn_backward_weight(int N, int io, const void* x, const void* dy, float* dw, int64_t T,
                                     int C_in, int C_out, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
    if (T == 0) {  // no tokens: the gradient is zero (a fill kernel, also fine inside a captured graph)
        const int64_t n = (int64_t)N * C_in * C_out;
        hipLaunchKernelGGL(bw_zero_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, stream, dw, n);
        return hipGetLastError();
    }
    const BwShape s = bw_shape(N, io, T, C_in, C_out);
    if (workspace_bytes < s.total) return hipErrorInvalidValue;
    // 32-bit buffer offsets over each operand's planes (under 2 GiB per plane
    // set); grid dimensions.  Past
    // these limits the call is not supported (the caller can split the tokens
    // and add the gradients).
    const int S = io == kIoF32 ? 4 : 2;
    if ((int64_t)N * C_in * s.Tp * S >= ((int64_t)1 << 31) || (int64_t)N * C_out * s.Tp * S >= ((int64_t)1 << 31))
        return hipErrorNotSupported;
    if (s.Tp / 64 > 0x7fffffff || (C_in + 7) / 8 > 65535 || (C_out + 7) / 8 > 65535 ||
        (int64_t)s.tiles * s.splits > 0x7fffffff)
        return hipErrorNotSupported;
    char* ws = static_cast<char*>(workspace);
    if (io == kIoF16) return dispatch_backward_weight<_Float16>(N, x, dy, dw, T, C_in, C_out, ws, s, stream);
    if (io == kIoBF16) return dispatch_backward_weight<__bf16>(N, x, dy, dw, T, C_in, C_out, ws, s, stream);
    return dispatch_backward_weight<float>(N, x, dy, dw, T, C_in, C_out, ws, s, stream);
}

hipError_t launch_cn_backward_weight_noalloc(int N, int io, const void* x, const void* dy, float* dw, int64_t T,
                                             int C_in, int C_out, hipStream_t stream) {
    const size_t need = T > 0 ? bw_shape(N, io, T, C_in, C_out).total : 0;
    if (need > kNoAllocScratchBytes) return hipErrorOutOfMemory;  // before any HIP call
    void* ws = nullptr;
    if (T > 0) {
        const hipError_t e = noalloc_scratch(&ws);
        if (e != hipSuccess) return e;
    }
    return launch_cn_backward_weight(N, io, x, dy, dw, T, C_in, C_out, ws, kNoAllocScratchBytes, stream);
}

}  // namespace eql
