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
    else return (e & 1) ? __uint_as_float(w[e >> 1] & 0xffff0000u) : __uint_as_float(w[e >> 1] << 16);
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
            for (int p = 0; p < N; ++p) pk[p][r / 2] = pack_bf16x2(Pa[p], Pb[p]);
        }
#pragma unroll
        for (int p = 0; p < N; ++p) {
            const u32x4 v = {pk[p][0], pk[p][1], pk[p][2], pk[p][3]};
            A[p] = __builtin_bit_cast(bf16x8, v);
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
                                        int64_t T, int C_out, int64_t tw0, int o0) {
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
            for (int p = 0; p < N; ++p) P[p] = acc[p][b][r];
            rdft_inverse<N>(P, yv);
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
                        const u32x4 v = {pack_bf16x2(yv[8 * j], yv[8 * j + 1]), pack_bf16x2(yv[8 * j + 2], yv[8 * j + 3]),
                                         pack_bf16x2(yv[8 * j + 4], yv[8 * j + 5]), pack_bf16x2(yv[8 * j + 6], yv[8 * j + 7])};
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
__global__ __launch_bounds__(C::kThreads) void cn_fused_kernel(
    const typename C::IO* __restrict__ x, const typename C::IO* __restrict__ w_hat,
    typename C::IO* __restrict__ y, int64_t T, int C_in, int C_out, int n_c_tiles,
    uint32_t total_tiles, int vec_ok, int w_dma_ok) {
    using IO = typename C::IO;
    using F = typename AFrag<IO>::T;
    __shared__ __attribute__((aligned(16))) char smem[2 * C::BUF_BYTES];

    const uint32_t tile = xcd_remap(blockIdx.x, total_tiles);
    const int64_t t0 = (int64_t)(tile / n_c_tiles) * C::TT;
    const int o0 = (int)(tile % n_c_tiles) * C::CT;
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
    store_y<C>(acc, y, T, C_out, tw0, o0);
}

// --- host side ----------------------------------------------------------------------

template <class C>
hipError_t launch_fused_cfg(const void* x, const void* w_hat, void* y, int64_t T, int C_in,
                            int C_out, hipStream_t stream) {
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
                       vec_ok, w_dma_ok);
    return hipGetLastError();
}

// Tile configurations (waves per workgroup, 16-channel output blocks per wave),
// largest output tile first.  Accumulators per lane = 4 * N * CB.
template <int N, typename IO>
struct FusedMenu {
    static constexpr int kCount = 7;
    static constexpr int waves[kCount] = {4, 4, 4, 4, 4, 1, 1};
    static constexpr int cb[kCount] = {6, 5, 4, 3, 2, 2, 1};
};

template <int N, typename IO, int I>
hipError_t launch_menu_entry(const void* x, const void* w_hat, void* y, int64_t T, int C_in,
                             int C_out, hipStream_t stream) {
    constexpr int W = FusedMenu<N, IO>::waves[I];
    constexpr int CBr = FusedMenu<N, IO>::cb[I];
    // keep the accumulators within 192 registers per lane
    constexpr int CB = (N * CBr <= 48) ? CBr : (48 / N > 0 ? 48 / N : 1);
    return launch_fused_cfg<FusedCfg<N, IO, W, CB>>(x, w_hat, y, T, C_in, C_out, stream);
}

template <int N, typename IO>
int choose_fused(int64_t T, int C_out) {
    using M = FusedMenu<N, IO>;
    const int nblk = (C_out + 15) / 16;
    int best = M::kCount - 1;
    for (int i = 0; i < M::kCount; ++i) {
        int cb = M::cb[i];
        if (N * cb > 48) continue;
        if (cb > nblk) continue;
        if (nblk % cb != 0 && i < 5) continue;  // whole tiles for the 4-wave shapes
        const int64_t tiles = ((T + 16 * M::waves[i] - 1) / (16 * M::waves[i])) * ((nblk + cb - 1) / cb);
        if (tiles >= 256) return i;
        best = i;
    }
    return best;
}

template <int N, typename IO>
hipError_t launch_fused(const void* x, const void* w_hat, void* y, int64_t T, int C_in, int C_out,
                        hipStream_t stream, int tile) {
    const int i = tile >= 0 ? tile : choose_fused<N, IO>(T, C_out);
    switch (i) {
        case 0: return launch_menu_entry<N, IO, 0>(x, w_hat, y, T, C_in, C_out, stream);
        case 1: return launch_menu_entry<N, IO, 1>(x, w_hat, y, T, C_in, C_out, stream);
        case 2: return launch_menu_entry<N, IO, 2>(x, w_hat, y, T, C_in, C_out, stream);
        case 3: return launch_menu_entry<N, IO, 3>(x, w_hat, y, T, C_in, C_out, stream);
        case 4: return launch_menu_entry<N, IO, 4>(x, w_hat, y, T, C_in, C_out, stream);
        case 5: return launch_menu_entry<N, IO, 5>(x, w_hat, y, T, C_in, C_out, stream);
        default: return launch_menu_entry<N, IO, 6>(x, w_hat, y, T, C_in, C_out, stream);
    }
}

}  // namespace eql
