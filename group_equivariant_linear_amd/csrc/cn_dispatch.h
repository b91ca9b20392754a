// cn_dispatch.h -- tile choice and dispatch of the C_N forward kernels.
#pragma once

#include <type_traits>

#include "cn_fused.h"
#include "cn_mf.h"
#include "cn_split.h"

namespace eql {

constexpr int kMfFirstTile = 7;     // tiles 7..13: entries 0..6 on the matrix-core transform kernel
constexpr int kSplitFirstTile = 14;  // tiles 14, 15: fp32, input channels split over 2 or 4 waves
constexpr int kStreamTile = 16;      // 16-bit, N <= 8: the persistent kernel (cn_stream.h)
constexpr int kWideTile = 17;        // 16-bit, N <= 8: the transform kernel with 8 waves over 128 tokens

// Output blocks per wave of the 8-wave tile: the most that keep two waves per
// SIMD without spilling (4 x N x CB accumulators beside the operands: N = 7
// takes four blocks in 251 VGPRs; five spill, as do four at N = 8).
template <int N>
constexpr int wide_cb() { return N == 7 ? 4 : 3; }

// cn_stream_{bf16,f16}.hip; hipErrorNotSupported for shapes the kernel does not take
hipError_t launch_cn_stream_bf16(int N, const void* x, const void* w_hat, void* y, int64_t T, int C_in, int C_out,
                                 hipStream_t stream, Epi epi);
hipError_t launch_cn_stream_f16(int N, const void* x, const void* w_hat, void* y, int64_t T, int C_in, int C_out,
                                hipStream_t stream, Epi epi);

// The automatic choice does not take the persistent kernel: on MI355X it ran
// the c3 trio (C8, 12608 tokens, 768->768, 768->3072, 3072->768 channels x
// group elements, bf16) in 116 us cache-cold and 95 us warm, against 99 us and
// 73 us for tile 10, and the C7 layer of 32768 tokens x 1120 in 96 us against
// 71 us.  EQL_STREAM_MIN_T sets a token count from which it would.
#ifndef EQL_STREAM_MIN_T
#define EQL_STREAM_MIN_T (int64_t)0x7fffffffffffffff
#endif
constexpr int kSplitMaxN = 10;       // larger orders: the split kernel's registers do not fit

#ifndef EQL_SPLIT_AUTO_KS
#define EQL_SPLIT_AUTO_KS 2
#endif

// Automatic choice (from tile sweeps on MI355X): 4-wave workgroups with the
// widest output tile that keeps two workgroups per CU (about 24/N output blocks:
// 4*N*CB accumulators plus ~130 other registers within 256, and the LDS tiles
// within half the CU's 160 KiB) while the grid still gives every CU a
// workgroup; one-wave workgroups for small problems.
template <int N>
int choose_shape(int64_t T, int C_in, int C_out) {
    (void)C_in;
    const int nblk = (C_out + 15) / 16;
    int cb = 24 / N;
    cb = cb < 2 ? 2 : (cb > 6 ? 6 : cb);
    if (cb > nblk) cb = nblk < 2 ? 2 : nblk;
    for (; cb >= 2; --cb) {
        const int64_t tiles = ((T + 63) / 64) * ((nblk + cb - 1) / cb);
        if (tiles >= 256) return 6 - cb;  // menu entries 0..4 hold CB = 6..2
    }
    return 6;  // one wave, one output block
}

template <int N, typename IO>
int choose_fused(int64_t T, int C_in, int C_out) {
    // 16-bit orders up to 8: the persistent kernel for long token batches of
    // whole 8-channel groups, else the matrix-core transform kernel
    if constexpr (mf_supported<N, IO>) {
        if (T >= EQL_STREAM_MIN_T && C_in % 8 == 0 && C_out % 8 == 0) return kStreamTile;
        // All output channels in one tile of at most six blocks, when the token
        // axis alone gives nearly every CU a workgroup: each x row is then read
        // once (cache-cold on MI355X, 12608 tokens, 96 output channels at N = 8:
        // 13.7 against 14.1 us from 96 inputs, 34.8 against 35.7 us from 384)
        const int nblk = (C_out + 15) / 16;
        // Six output blocks over that many token tiles: the 8-wave tile of 128
        // tokens x 48 channels instead.  Each weight chunk then serves 128
        // tokens, which halves the weight reloads; x is read once more, from L2
        // (cache-cold on MI355X, 12608 tokens at N = 8: 96 -> 96 13.6 -> 12.5 us,
        // 384 -> 96 32.2 -> 30.6 us; it is slower on 96 -> 384, 36.4 -> 39.7 us,
        // and on the C7 layer of 160 channels, 63.9 -> 70.2 us)
        if (nblk == 6 && (T + 63) / 64 >= 192) return kWideTile;
        // C7 layers wider than six blocks: 128 tokens x 64 channels, which
        // halves the weight reloads and cuts x's re-reads, when the tiles fill
        // every CU (cache-cold on MI355X, 32768 tokens x 160 channels:
        // 65.5-66.2 -> 56.9-59.9 us)
        if (N == 7 && nblk > 6 && ((T + 127) / 128) * ((nblk + 3) / 4) >= 256) return kWideTile;
        if (nblk <= 6 && (T + 63) / 64 >= 192) return kMfFirstTile + 6 - (nblk < 2 ? 2 : nblk);
        return kMfFirstTile + choose_shape<N>(T, C_in, C_out);
    } else {
        const int s = choose_shape<N>(T, C_in, C_out);
        // fp32 layers too small for one wave per SIMD at 16 x 16 per wave: split
        // the input channels of each such tile over 2 or 4 waves
        if constexpr (std::is_same_v<IO, float> && N <= kSplitMaxN)
            if (s == 6 && split_ok<N>(C_in, C_out)) return kSplitFirstTile + (EQL_SPLIT_AUTO_KS == 4 ? 1 : 0);
        return s;
    }
}

template <int N, typename IO>
hipError_t launch_fused(const void* x, const void* w_hat, void* y, int64_t T, int C_in, int C_out,
                        hipStream_t stream, int tile, Epi epi) {
    int i = tile >= 0 ? tile : choose_fused<N, IO>(T, C_in, C_out);
    if (i == kWideTile) {
        if constexpr (mf_supported<N, IO>) {
            using Cfg = MfCfg<N, 8, wide_cb<N>(), IO>;
            if (fast_ok<N, IO>(C_in, C_out, Cfg::TT))
                return launch_mf_cfg<Cfg>(x, w_hat, y, T, C_in, C_out, stream, epi);
            i = kMfFirstTile + choose_shape<N>(T, C_in, C_out);  // shapes it does not take
        } else {
            i = choose_fused<N, IO>(T, C_in, C_out);
        }
    }
    if (i == kStreamTile) {
        if constexpr (mf_supported<N, IO>) {
            const hipError_t e = std::is_same_v<IO, __bf16>
                                     ? launch_cn_stream_bf16(N, x, w_hat, y, T, C_in, C_out, stream, epi)
                                     : launch_cn_stream_f16(N, x, w_hat, y, T, C_in, C_out, stream, epi);
            if (e != hipErrorNotSupported) return e;
        }
        // shapes it does not take: the other kernels' automatic choice
        i = choose_shape<N>(T, C_in, C_out);
        if constexpr (mf_supported<N, IO>) i += kMfFirstTile;
        else if (std::is_same_v<IO, float> && N <= kSplitMaxN && i == 6 && split_ok<N>(C_in, C_out))
            i = kSplitFirstTile + (EQL_SPLIT_AUTO_KS == 4 ? 1 : 0);
    }
    if (i >= kSplitFirstTile) {
        if constexpr (std::is_same_v<IO, float> && N <= kSplitMaxN) {
            if (split_ok<N>(C_in, C_out)) {
                if (i == kSplitFirstTile) return launch_split<N, 2>(x, w_hat, y, T, C_in, C_out, stream, epi);
                return launch_split<N, 4>(x, w_hat, y, T, C_in, C_out, stream, epi);
            }
        }
        i = kMfFirstTile + 6;  // one-wave shape of the other kernels
    }
    if (i >= kMfFirstTile) {
        switch (i - kMfFirstTile) {
#define EQL_MF(k)                                                                       \
    case k:                                                                             \
        if constexpr (mf_supported<N, IO>)                                              \
            return launch_mf_entry<N, IO, k>(x, w_hat, y, T, C_in, C_out, stream, epi);          \
        else                                                                            \
            return launch_menu_entry<N, IO, k>(x, w_hat, y, T, C_in, C_out, stream, epi);
            EQL_MF(0) EQL_MF(1) EQL_MF(2) EQL_MF(3) EQL_MF(4) EQL_MF(5)
#undef EQL_MF
            default:
                if constexpr (mf_supported<N, IO>)
                    return launch_mf_entry<N, IO, 6>(x, w_hat, y, T, C_in, C_out, stream, epi);
                else
                    return launch_menu_entry<N, IO, 6>(x, w_hat, y, T, C_in, C_out, stream, epi);
        }
    }
    switch (i) {
#define EQL_ENTRY(k) \
    case k: return launch_menu_entry<N, IO, k>(x, w_hat, y, T, C_in, C_out, stream, epi);
        EQL_ENTRY(0) EQL_ENTRY(1) EQL_ENTRY(2) EQL_ENTRY(3) EQL_ENTRY(4) EQL_ENTRY(5)
#undef EQL_ENTRY
        default: return launch_menu_entry<N, IO, 6>(x, w_hat, y, T, C_in, C_out, stream, epi);
    }
}

}  // namespace eql
