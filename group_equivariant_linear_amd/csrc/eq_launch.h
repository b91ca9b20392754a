// eq_launch.h -- internal host-side launchers of libeqlinear (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eql {

constexpr int kMaxGemmJobs = 16;  // D8: 6 jobs; D_n: n + 1 (odd n) or n + 2 (even n), n <= 12

// Element type of a launch's tensors ("io" arguments), the codes of the C ABI's
// eqlinear_dtype.
enum : int { kIoF32 = 0, kIoBF16 = 1, kIoF16 = 2 };

// Fused neighbours of the C_N forward: y = act(y + bias[o]) in the epilogue.
// bias: device, plan dtype, C_out elements, or null; act: 0 identity, 1 GELU.
struct Epi {
    const void* bias;
    int act;
};

// One independent product y[t][y_col+n] = sum_k W[n][k] x[t][x_col+k],
// n < Nn, k < K, W = w + w_off with row stride ldw (elements).
struct GemmJob {
    int x_col, y_col, K, Nn;
    int64_t w_off;
    int ldw;
    int tile_begin;  // first column tile of this job (filled by the launcher)
    int x_vec_ok, w_vec_ok, y_vec_ok;  // 16-byte (8-byte for bf16 y) access allowed
    int narrow;      // D8 kernel: narrower output tile for this job (filled by the launcher)
};

struct GemmJobs {
    GemmJob j[kMaxGemmJobs];
    int njobs;
    int tiles_per_row;  // column tiles per token tile (filled by the launcher)
};

// tile: -1 = automatic choice, else a fixed tile configuration (tests, tuning).
hipError_t launch_cn_forward(int N, int io, const void* x, const void* w_hat, void* y,
                             int64_t T, int C_in, int C_out, hipStream_t stream, int tile, Epi epi = Epi{nullptr, 0});

hipError_t launch_gemm_rows(int io, GemmJobs jobs, const void* x, const void* w, void* y,
                            int64_t T, int ldx, int ldy, hipStream_t stream);

// bf16 D8 jobs on the dedicated kernel (16*cb output channels per workgroup);
// hipErrorNotSupported when a job column, width or W row is not a whole number
// of 16-byte pieces (then use launch_gemm_rows).
hipError_t launch_d8_fast(int io, GemmJobs jobs, const void* x, const void* w, void* y, int64_t T, int ldx, int ldy,
                          int64_t w_elems, int cb, hipStream_t stream);

// Adjoint spectrum: w_hat_adj[p][i][o] = +-w_hat[p][o][i] (imaginary planes negated).
hipError_t launch_w_hat_adjoint(int N, int io, const void* w_hat, void* w_hat_adj, int C_in, int C_out,
                                hipStream_t stream);

// Weight gradient of the C_N layer into fp32 dw[C_out][C_in][N]; the workspace
// holds the operand planes and the per-range partial spectra.
size_t backward_weight_workspace(int N, int io, int64_t T, int C_in, int C_out);
hipError_t launch_cn_backward_weight(int N, int io, const void* x, const void* dy, float* dw, int64_t T,
                                     int C_in, int C_out, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

// The same weight gradient with the workspace in a library-held per-GPU array of
// kNoAllocScratchBytes (no allocation); hipErrorOutOfMemory, before any HIP
// call, when the shape needs more.  Calls that overlap on one GPU race.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
hipError_t launch_cn_backward_weight_noalloc(int N, int io, const void* x, const void* dy, float* dw, int64_t T,
                                             int C_in, int C_out, hipStream_t stream);

hipError_t launch_weight_dft(int N, int io, const void* w, void* w_hat, int C_in,
                             int C_out, hipStream_t stream);

hipError_t launch_cn_expand(int N, int io, const void* w, void* w_dense, int C_in,
                            int C_out, hipStream_t stream);

// dihedral D_n block matrix (n = 4: D8)
hipError_t launch_dn_expand(int n, int io, const void* wb, void* w_dense, int C_in, int C_out,
                            hipStream_t stream);

// d8_round_trip.hip: m = C/8 regular channels per token
hipError_t launch_d8_round_trip(int io, const void* y_in, void* y_out, const void* bias, int act, int m,
                                int64_t T, hipStream_t stream);
hipError_t launch_d8_to_fourier(int io, const void* x_reg, void* x_four, int m, int64_t T,
                                hipStream_t stream);
hipError_t launch_d8_to_regular(int io, const void* y_four, void* y_reg, int m, int64_t T,
                                hipStream_t stream);
// dn_regular.hip: the dihedral layer between regular-representation features in
// one launch, y_reg = act(F^T W F x_reg + b); 16-bit I/O, m_in and m_out multiples
// of 8 (hipErrorNotSupported otherwise)
hipError_t launch_dn_regular(int n, int io, const void* x_reg, const void* wb, const void* bias, int act,
                             void* y_reg, int64_t T, int m_in, int m_out, int64_t w_elems, hipStream_t stream);
// the same passes for D_n, m = C/2n regular channels (n = 4 takes the D8 kernels)
hipError_t launch_dn_round_trip(int n, int io, const void* y_in, void* y_out, const void* bias, int act,
                                int m, int64_t T, hipStream_t stream);
hipError_t launch_dn_to_fourier(int n, int io, const void* x_reg, void* x_four, int m, int64_t T,
                                hipStream_t stream);
hipError_t launch_dn_to_regular(int n, int io, const void* y_four, void* y_reg, int m, int64_t T,
                                hipStream_t stream);

}  // namespace eql
