// cn_stream.h -- persistent 16-bit C_N forward for the wide layers (bf16 or
// fp16, 2 <= N <= 8): the same arithmetic as cn_mf.h ("Flash EQ-Linear",
// Algorithmic Approach and Implementation: group DFT of x, per-bin channel
// products over the kept half of the spectrum, inverse DFT, one pass with no
// intermediate tensor in memory), scheduled for the memory system.
//
// One workgroup of eight waves per CU (two waves per SIMD).  A workgroup owns
// one slice of CT = 16 CB output channels for the whole launch and walks the
// token axis in 16-token blocks, one block per wave at a time (the workgroups
// of all output slices walk the same blocks in the same order, so a block's x
// is fetched from HBM once and read from L2 by the other slices; the slices of
// one block share an XCD).  Per wave, the input channels of a block are
// consumed in chunks of 32, and the chunks of successive blocks form one
// stream:
//   - x goes from memory straight into the wave's own exchange rows in LDS
//     (direct loads of whole 16-byte pieces, cn_mf's row layout); as soon as
//     the wave has read a chunk's channel records into registers it starts the
//     next chunk into the same rows, so one chunk per wave is always in flight
//     and the transform, the products and any epilogue run under its latency;
//   - the w_hat slice of the workgroup sits in LDS for the whole launch when
//     all of C_in fits (WSTAT: loaded once, then the waves run independently,
//     with no barrier); otherwise it streams through a two-stage LDS ring, one
//     barrier per chunk;
//   - group DFT on the matrix cores (block-diagonal 16 x 32 coefficient
//     fragments, as in cn_mf.h), the spectrum rounded once to the I/O type;
//     the per-bin products as the real 2 x 2 block form, fp32 accumulation;
//   - after a block's last chunk: inverse DFT on the matrix cores, the fused
//     bias/GELU, and y stored straight from registers (each lane writes 8N
//     contiguous bytes: four output channels of one token).
// The transform coefficients carry 1/N (forward) and N (inverse) so that no
// 16-bit intermediate exceeds the range of the inputs and outputs: |Xhat/N| <=
// max|x| and |Yhat/N| <= max|y| (fp16 keeps its range; for N = 2, 4, 8 the
// scaling is exact).
#pragma once

#include "cn_mf.h"

namespace eql {

// s_waitcnt immediate: vmcnt <= n (0..63), lgkmcnt and expcnt unconstrained.
constexpr int vmcnt_imm_st(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// WSTAT: the w_hat slice stays in LDS for the whole launch; otherwise it
// streams through a two-stage ring.
template <int N_, typename IO_, int CB_, bool WSTAT_, bool EPI_>
struct StCfg {
    using IO = IO_;
    using F8 = typename Half<IO_>::x8;
    static constexpr int N = N_, CB = CB_;
    static constexpr bool WSTAT = WSTAT_;
    static constexpr bool EPI = EPI_;    // the fused bias/GELU epilogue is compiled in
    static constexpr int CT = 16 * CB_;  // output channels of a workgroup
    static constexpr int KC = 32;        // input channels per chunk
    static constexpr int WAVES = 8, kThreads = 512;
    static constexpr int MQ = (N_ + 3) / 4;  // transform products per four channels
    static constexpr int H = (N_ - 1) / 2;   // complex bins
    static constexpr int NB = 1 + H + (N_ % 2 == 0 ? 1 : 0);
    // x: a chunk of a 16-token block is 16 rows of XP 16-byte pieces, held in
    // the wave's exchange rows as in cn_mf.h (rotated rows for N = 2, 4, 8,
    // else rows padded to an odd pitch)
    static constexpr int XP = 4 * N_;
    static constexpr bool XALIGN = (16 % (2 * N_)) == 0;  // records inside one piece
    static constexpr bool XROT = XALIGN && (XP % 8) == 0;
    static constexpr int XPITCH = XROT ? XP : (XP | 1);
    // slot s of the rows is written by lane s % 64 of load s / 64: whole loads
    static constexpr int XDMA = (16 * XPITCH + 63) / 64;
    static constexpr int XEX = XDMA * 1024;  // exchange bytes of one wave
    static constexpr int WSLOTS = N_ * CT * 4;  // 16-byte parts of one w_hat chunk
    static constexpr int WDMA = (WSLOTS + kThreads - 1) / kThreads;  // direct loads per thread and chunk
    static constexpr int WCH = WDMA * kThreads * 16;  // LDS bytes of a chunk, padded to whole loads
    // y: 8N bytes per lane and output block, in 16-byte stores (even N) or 8-byte ones
    static constexpr int YS = (N_ % 2 == 0) ? 16 : 8;
    static constexpr int YST = 8 * N_ / YS;  // stores per lane and output block
    static constexpr int E = CB_ * YST;      // stores per lane and token block
};

template <int N, typename IO>
constexpr bool stream_supported = (std::is_same_v<IO, __bf16> || std::is_same_v<IO, _Float16>) && N >= 2 && N <= 8;

// Scaled real-DFT fragments (A operand) of this lane: row (gr, ir) of fragment
// m, k-values (kg, e) -> s * coef(4m + ir, e) if kg == gr.  INV: inverse
// (rows = group elements, k = planes).
template <class C, bool INV>
__device__ __forceinline__ void st_frags(typename C::F8 (&Fa)[C::MQ]) {
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

template <class C>
__global__ __launch_bounds__(C::kThreads, 1) void cn_stream_kernel(
    const typename C::IO* __restrict__ x, const typename C::IO* __restrict__ w_hat, typename C::IO* __restrict__ y,
    int64_t T, int C_in, int C_out, int n_ct, int P, uint32_t n_wg, Epi epi) {
    constexpr int N = C::N, CB = C::CB, MQ = C::MQ, H = C::H, NB = C::NB, WAVES = C::WAVES;
    constexpr int S = 2;  // bytes per element
    using IO = typename C::IO;
    using F8 = typename C::F8;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    // workgroup -> (output slice, stream index); consecutive logical ids (the
    // slices of one stream) run on one XCD
    const uint32_t L = xcd_remap(blockIdx.x, n_wg);
    const int ct = (int)(L % (uint32_t)n_ct), wi = (int)(L / (uint32_t)n_ct);
    const int o0 = ct * C::CT;
    const int lane = (int)threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int kg = lane >> 4, tl = lane & 15;
    const int nch = (C_in + C::KC - 1) / C::KC;
    const int64_t nblk = (T + 15) / 16;
    // this wave's token blocks: (m P + wi) WAVES + wave, m = 0, 1, ...; in the
    // ring mode every wave runs the count of wave 0 (the largest), so that all
    // take part in every barrier
    const int64_t b0 = (int64_t)wi * WAVES + wave, stride = (int64_t)P * WAVES;
    const int64_t nmine = b0 < nblk ? (nblk - b0 + stride - 1) / stride : 0;
    const int64_t nlead = (int64_t)wi * WAVES < nblk ? (nblk - (int64_t)wi * WAVES + stride - 1) / stride : 0;
    const int64_t nsteps = (C::WSTAT ? nmine : nlead) * nch;

    const uint32_t row_x = (uint32_t)C_in * (N * S), row_y = (uint32_t)C_out * (N * S);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)(T * (int64_t)row_x));
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(y, (uint32_t)(T * (int64_t)row_y));
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_hat, (uint32_t)((int64_t)N * C_out * C_in * S));

    // --- w_hat: chunk c of the slice at smem + c WCH (WSTAT) or in stage c % 2.
    // Slot s of a chunk: plane s / (4 CT), row o = (s / 4) % CT, stored part
    // s % 4 holding part (s % 4) ^ ((o >> 1) & 3) of the row's 32 channels.
    uint32_t woff[C::WDMA];
    int wcol[C::WDMA];
#pragma unroll
    for (int it = 0; it < C::WDMA; ++it) {
        const int s = it * C::kThreads + (int)threadIdx.x;
        const int p = s / (4 * C::CT), o = (s / 4) % C::CT;
        const int q = (s & 3) ^ ((o >> 1) & 3);
        woff[it] = (s < C::WSLOTS && o0 + o < C_out)
                       ? (((uint32_t)p * (uint32_t)C_out + (uint32_t)(o0 + o)) * (uint32_t)C_in + (uint32_t)(8 * q)) * S
                       : kOOB;
        wcol[it] = 8 * q;
    }
    auto dma_w = [&](int c, char* dst) {
        const bool tail = c * C::KC + C::KC > C_in;
#pragma unroll
        for (int it = 0; it < C::WDMA; ++it) {
            const uint32_t off = (woff[it] == kOOB || (tail && c * C::KC + wcol[it] >= C_in))
                                     ? kOOB
                                     : woff[it] + (uint32_t)(c * C::KC * S);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rw, (__attribute__((address_space(3))) void*)(dst + (it * C::kThreads + wave * 64) * 16), 16, off, 0,
                0, 0);
        }
    };
    // parts never loaded (rows past C_out, channels past C_in) must be finite
    // (their x side is zero, or their rows are dropped): clear the LDS first
    const int wbytes = (C::WSTAT ? nch : 2) * C::WCH;
    if ((C_in % C::KC) != 0 || (C_out - o0) < C::CT) {
        for (int i = (int)threadIdx.x; i < wbytes / 16; i += C::kThreads)
            reinterpret_cast<u32x4*>(smem)[i] = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
    }
    if constexpr (C::WSTAT) {
        for (int c = 0; c < nch; ++c) dma_w(c, smem + c * C::WCH);
    } else {
        dma_w(0, smem);
    }

    // --- x: step s = (block index m, chunk c).  Chunk c of block (m P + wi)
    // WAVES + wave: token rows t0 .. t0+15, bytes 64 N c .. 64 N (c+1) of each
    // row.  Load j of this lane fills slot 64 j + lane of the exchange rows:
    // row r = slot / XPITCH, rotated position -> piece k (cn_mf's layout).  The
    // load cursor (mp, cp) runs one step ahead of the step's (m, c).
    char* xex = smem + wbytes + wave * C::XEX;
    uint32_t xoff[C::XDMA];  // offset of the slot's piece within a chunk's rows
#pragma unroll
    for (int j = 0; j < C::XDMA; ++j) {
        const int sl = 64 * j + lane, r = sl / C::XPITCH, pos = sl % C::XPITCH;
        const int k = C::XROT ? (pos + C::XP - r % C::XP) % C::XP : pos;
        xoff[j] = (r < 16 && k < C::XP) ? (uint32_t)r * row_x + (uint32_t)k * 16u : kOOB;
    }
    int64_t mp = 0;
    int cp = 0, sp = 0;  // cursor chunk; steps issued (saturates at nsteps)
    auto load_x = [&]() {
        bool on = false;
        uint32_t base = 0;
        int64_t t0 = 0;
        uint32_t valid = 0;  // bytes of the chunk's rows that hold channels < C_in
        if (sp < nsteps) {
            t0 = (b0 + mp * stride) * 16;
            on = t0 < T;
            base = (uint32_t)t0 * row_x + (uint32_t)(cp * C::KC) * (uint32_t)(N * S);
            valid = (uint32_t)(C_in - cp * C::KC) * (uint32_t)(N * S);
            ++sp;
            if (++cp == nch) {
                cp = 0;
                ++mp;
            }
        }
        if (on && t0 + 16 <= T && valid >= (uint32_t)(C::XP * 16)) {
            // (the offsets pass through locals: an array element given straight
            // to the builtin makes the host compilation drop the kernel's stub)
#pragma unroll
            for (int j = 0; j < C::XDMA; ++j) {
                const uint32_t off = xoff[j] == kOOB ? kOOB : xoff[j] + base;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (__attribute__((address_space(3))) void*)(xex + j * 1024), 16, off, 0, 0, 0);
            }
        } else {
            // a partial block, a partial chunk or past the end: rows past T and
            // pieces past C_in are not read (every slot still gets one load, so
            // that the count of loads in flight stays the same)
            const uint32_t rows = on ? (uint32_t)(T - t0 < 16 ? T - t0 : 16) : 0u;
#pragma unroll
            for (int j = 0; j < C::XDMA; ++j) {
                const int sl = 64 * j + lane, r = sl / C::XPITCH, pos = sl % C::XPITCH;
                const int k = C::XROT ? (pos + C::XP - r % C::XP) % C::XP : pos;
                const bool ok = xoff[j] != kOOB && (uint32_t)r < rows && (uint32_t)k * 16u < valid;
                const uint32_t off = ok ? xoff[j] + base : kOOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (__attribute__((address_space(3))) void*)(xex + j * 1024), 16, off, 0, 0, 0);
            }
        }
    };

    // bias of this lane's output channels (the slice is fixed for the launch)
    float bv[CB][4];
#pragma unroll
    for (int b = 0; b < CB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int o = o0 + 16 * b + 4 * kg + i;
            bv[b][i] = (C::EPI && epi.bias != nullptr && o < C_out) ? bias_value<IO>(bias_fetch<IO>(epi, C_out, o))
                                                                     : 0.0f;
        }

    F8 Fa[MQ];
    st_frags<C, false>(Fa);
    f32x4 acc[N][CB];
#pragma unroll
    for (int p = 0; p < N; ++p)
#pragma unroll
        for (int b = 0; b < CB; ++b) acc[p][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int o_l = lane & 15;
    const int lane_off = (o_l * 4 + (kg ^ ((o_l >> 1) & 3))) * 16;

    // the first chunk of x
    load_x();
    // the slice (or the first ring stage) has landed for every wave
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // One step: wait for x(s) (and, in ring mode, w_hat(s)); read its records,
    // start x(s + 1) into the rows they leave; transform, products; after a
    // block's last chunk the epilogue and its stores.  Loads and stores retire
    // in issue order, so a wait names the number of younger operations that may
    // stay in flight: x(s) went out in step s - 1 after its records were read,
    // and only the stores of step s - 1 (a block that ended there) are younger.
    int64_t m = 0;  // this step's block index (in the wave's sequence) and chunk
    int c = 0;
    for (int64_t s = 0; s < nsteps; ++s) {
        const bool ended = m > 0 && c == 0;  // step s - 1 ended a block and stored it
        if (ended) __builtin_amdgcn_s_waitcnt(vmcnt_imm_st(C::E));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm_st(0));
        const char* wbuf;
        if constexpr (C::WSTAT) {
            wbuf = smem + c * C::WCH;
        } else {
            // w_hat(s) went out in step s - 1 before x(s): it has landed too
            __builtin_amdgcn_s_barrier();  // every wave's share of w_hat(s) is in; stage (s+1)%2 is free
            const int cn = c + 1 == nch ? 0 : c + 1;
            dma_w(s + 1 < nsteps ? cn : nch, smem + ((s + 1) & 1) * C::WCH);  // nch: no access, same count
            wbuf = smem + (s & 1) * C::WCH;
        }

        // records of channels 8kg + j (j = 0..7) of token tl
        F8 rec[8];
        static_for<0, 8>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            rec[j] = read_record<C, j>(xex, tl, kg);
        });
        // the records are in registers: the exchange rows may be refilled
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        load_x();
        if (c * C::KC + C::KC > C_in) {  // channel tail: records past C_in are zero
            const int left = C_in - c * C::KC;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (8 * kg + j >= left) rec[j] = F8{};
        }

        // transform: Xh[p] = planes p / N of channels 8kg .. 8kg+7 of token tl
        F8 Xh[N];
        {
            uint32_t pk[N][4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                f32x4 d0[MQ], d1[MQ];
#pragma unroll
                for (int mq = 0; mq < MQ; ++mq) {
                    d0[mq] = f32x4{0.f, 0.f, 0.f, 0.f};
                    d1[mq] = f32x4{0.f, 0.f, 0.f, 0.f};
                    mma_ab(d0[mq], Fa[mq], rec[2 * jj]);
                    mma_ab(d1[mq], Fa[mq], rec[2 * jj + 1]);
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
        auto ldW = [&](int p, int b) {
            return *reinterpret_cast<const F8*>(wbuf + p * C::CT * 64 + b * 1024 + lane_off);
        };
        // products, one (bin, output block) at a time: the w_hat fragments of
        // the next pair are read from LDS while this pair multiplies
        constexpr int NP = NB * CB;  // (bin, block) pairs, bin-major
        auto load_pair = [&](auto ic, F8& wr, F8& wi) {
            constexpr int i = decltype(ic)::value;
            constexpr int sb = i / CB, b = i % CB;
            if constexpr (sb == 0) {
                wr = ldW(0, b);
            } else if constexpr (sb <= H) {
                wr = ldW(2 * sb - 1, b);
                wi = ldW(2 * sb, b);
            } else {
                wr = ldW(N - 1, b);
            }
        };
        F8 Wr[2], Wi[2];
        F8 nXi[H > 0 ? H : 1];
        static_for<1, H + 1>([&](auto sc) {
            constexpr int sb = decltype(sc)::value;
            nXi[sb - 1] = neg(Xh[2 * sb]);
        });
        load_pair(std::integral_constant<int, 0>{}, Wr[0], Wi[0]);
        static_for<0, NP>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            constexpr int sb = i / CB, b = i % CB, cur = i & 1;
            if constexpr (i + 1 < NP) load_pair(std::integral_constant<int, i + 1>{}, Wr[cur ^ 1], Wi[cur ^ 1]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (sb == 0) {
                mma_ab(acc[0][b], Wr[cur], Xh[0]);
            } else if constexpr (sb <= H) {
                constexpr int pr = 2 * sb - 1, pi = 2 * sb;
                mma_ab(acc[pr][b], Wr[cur], Xh[pr]);
                mma_ab(acc[pi][b], Wi[cur], Xh[pr]);
                mma_ab(acc[pr][b], Wi[cur], nXi[sb - 1]);
                mma_ab(acc[pi][b], Wr[cur], Xh[pi]);
            } else {
                mma_ab(acc[N - 1][b], Wr[cur], Xh[N - 1]);
            }
            __builtin_amdgcn_sched_barrier(0);
        });

        if (c == nch - 1) {
            // epilogue of block m: lane (tl, kg) holds token tl, channels
            // 16b + 4kg + i, all N planes (scaled by 1/N)
            const int64_t t = (b0 + m * stride) * 16 + tl;
            const bool live = (b0 + m * stride) < nblk && t < T;
            F8 Ga[MQ];
            st_frags<C, true>(Ga);
#pragma unroll
            for (int b = 0; b < CB; ++b) {
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
                    for (int mq = 0; mq < MQ; ++mq) {
                        f32x4 d = {0.f, 0.f, 0.f, 0.f};
                        mma_ab(d, Ga[mq], Bv);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (4 * mq + r < N) flat[i * N + 4 * mq + r] = d[r];
                    }
                }
                if constexpr (C::EPI) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) epi_apply<N>(flat + i * N, bv[b][i], epi.act);
                }
                uint32_t pk[2 * N];
#pragma unroll
                for (int q = 0; q < 2 * N; ++q) pk[q] = Half<IO>::pack2(flat[2 * q], flat[2 * q + 1]);
                const int o = o0 + 16 * b + 4 * kg;
                const uint32_t base = (live && o < C_out) ? (uint32_t)t * row_y + (uint32_t)o * (uint32_t)(N * S) : kOOB;
#pragma unroll
                for (int q = 0; q < C::YST; ++q) {
                    const uint32_t off = base == kOOB ? kOOB : base + (uint32_t)(q * C::YS);
                    if constexpr (C::YS == 16)
                        __builtin_amdgcn_raw_buffer_store_b128(
                            u32x4{pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]}, ry, off, 0, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pk[2 * q], pk[2 * q + 1]}, ry, off, 0, 0);
                }
            }
#pragma unroll
            for (int p = 0; p < N; ++p)
#pragma unroll
                for (int b = 0; b < CB; ++b) acc[p][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (++c == nch) {
            c = 0;
            ++m;
        }
    }
}

// --- host side ----------------------------------------------------------------------

// LDS bytes of one workgroup: the w_hat slice or ring, then the exchange rows.
template <class C>
constexpr int64_t stream_lds(int nch) {
    return (C::WSTAT ? (int64_t)nch * C::WCH : 2 * (int64_t)C::WCH) + (int64_t)C::WAVES * C::XEX;
}

// The launch: one workgroup per CU, the output slices spread evenly over them.
// hipErrorNotSupported when the shape does not suit the kernel (channel counts
// not multiples of 8, tensors of 2 GiB or more, LDS past the CU's 160 KiB).
template <class C>
hipError_t launch_stream_cfg(const void* x, const void* w_hat, void* y, int64_t T, int C_in, int C_out,
                             hipStream_t stream, Epi epi) {
    constexpr int S = 2;
    if (C_in % 8 || C_out % 8) return hipErrorNotSupported;
    if (T * C_in * C::N * S >= ((int64_t)1 << 31) || T * C_out * C::N * S >= ((int64_t)1 << 31) ||
        (int64_t)C::N * C_in * C_out * S >= ((int64_t)1 << 31))
        return hipErrorNotSupported;
    const int nch = (C_in + C::KC - 1) / C::KC;
    const int64_t lds = stream_lds<C>(nch);
    if (lds > 160 * 1024) return hipErrorNotSupported;
    static int cus = 0;
    static bool attr = false;
    if (!attr) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void*)cn_stream_kernel<C>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    160 * 1024);
        if (e != hipSuccess) return e;
        attr = true;
    }
    const int n_ct = (C_out + C::CT - 1) / C::CT;
    const int P = n_ct >= cus ? 1 : cus / n_ct;
    const uint32_t n_wg = (uint32_t)P * (uint32_t)n_ct;
    hipLaunchKernelGGL((cn_stream_kernel<C>), dim3(n_wg), dim3(C::kThreads), (uint32_t)lds, stream,
                       (const typename C::IO*)x, (const typename C::IO*)w_hat, (typename C::IO*)y, T, C_in, C_out,
                       n_ct, P, n_wg, epi);
    return hipGetLastError();
}

// w_hat resident in LDS when the whole slice fits, else the two-stage ring.
template <int N, typename IO, int CB>
hipError_t launch_stream(const void* x, const void* w_hat, void* y, int64_t T, int C_in, int C_out,
                         hipStream_t stream, Epi epi) {
    const int nch = (C_in + 31) / 32;
    const bool stat = stream_lds<StCfg<N, IO, CB, true, false>>(nch) <= 160 * 1024;
    if (epi.bias != nullptr || epi.act != 0) {
        if (stat) return launch_stream_cfg<StCfg<N, IO, CB, true, true>>(x, w_hat, y, T, C_in, C_out, stream, epi);
        return launch_stream_cfg<StCfg<N, IO, CB, false, true>>(x, w_hat, y, T, C_in, C_out, stream, epi);
    }
    if (stat) return launch_stream_cfg<StCfg<N, IO, CB, true, false>>(x, w_hat, y, T, C_in, C_out, stream, epi);
    return launch_stream_cfg<StCfg<N, IO, CB, false, false>>(x, w_hat, y, T, C_in, C_out, stream, epi);
}

}  // namespace eql
