// cn_dispatch.h -- tile choice and dispatch of the C_N forward kernels.
#pragma once

#include <type_traits>

#include "cn_fused.h"
#include "cn_mf.h"
#include "cn_split.h"

namespace eql {

constexpr int kMfFirstTile = 7;     // tiles 7..13: entries 0..6 on the matrix-core transform kernel
constexpr int kSplitFirstTile = 14;  // tiles 14, 15: fp32, input channels split over 2 or 4 waves
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
    // 16-bit orders up to 8 take the matrix-core transform kernel, same shapes
    if constexpr (mf_supported<N, IO>) {
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
