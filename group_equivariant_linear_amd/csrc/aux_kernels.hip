// aux_kernels.hip -- off-hot-path kernels of libeqlinear:
//  - the weight spectrum ("Flash EQ-Linear", Algorithmic Approach; computed
//    once per weight, Implementation: plug-and-play on trained weights);
//  - the dense matrices a replicate-and-multiply implementation would use
//    ("Flash EQ-Linear", Problem Statement; "Quick ViTs", key design 2).
#include "eq_device.h"
#include "eq_launch.h"

namespace eql {

constexpr int kMaxN = 16;

struct TwArg {
    double cs[kMaxN];
    double sn[kMaxN];
};

template <typename IO>
__device__ __forceinline__ double load_f64(const IO* p) {
    return (double)(float)*p;
}

// fp64 -> fp32 rounded to odd: truncate toward zero, set the last bit if inexact.
// Rounding that value to bf16 with round-to-nearest-even gives the correctly
// rounded bf16 of the fp64 input (fp32 carries more than two extra bits).
__device__ __forceinline__ float f64_to_f32_odd(double d) {
    float f = (float)d;
    if ((double)f != d) {
        uint32_t u = __float_as_uint(f);
        if (__builtin_fabs((double)f) > __builtin_fabs(d)) u -= 1u;
        u |= 1u;
        f = __uint_as_float(u);
    }
    return f;
}

template <typename IO>
__device__ __forceinline__ IO round_out(double d);
template <>
__device__ __forceinline__ float round_out<float>(double d) {
    return (float)d;
}
template <>
__device__ __forceinline__ __bf16 round_out<__bf16>(double d) {
    return (__bf16)f64_to_f32_odd(d);
}
template <>
__device__ __forceinline__ _Float16 round_out<_Float16>(double d) {
    return (_Float16)f64_to_f32_odd(d);  // fp32 carries 13 more bits than fp16
}

// One thread per (o, i): the N-point real DFT of w[o][i][:], in fp64, packed
// into planes [N][C_out][C_in] (plane 0 = Re X0, 2k-1/2k = Re/Im Xk, N-1 = Re X_{N/2}).
template <typename IO>
__global__ void weight_dft_kernel(const IO* __restrict__ w, IO* __restrict__ w_hat, int N,
                                  int64_t plane, TwArg tw) {
    const int64_t oi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (oi >= plane) return;
    double wm[kMaxN];
#pragma unroll
    for (int m = 0; m < kMaxN; ++m) wm[m] = m < N ? load_f64(w + oi * N + m) : 0.0;
    for (int k = 0; k <= N / 2; ++k) {
        double re = 0.0, im = 0.0;
#pragma unroll
        for (int m = 0; m < kMaxN; ++m) {
            if (m < N) {
                const int j = (m * k) % N;
                re = __builtin_fma(wm[m], tw.cs[j], re);
                im = __builtin_fma(-wm[m], tw.sn[j], im);
            }
        }
        if (k == 0) {
            w_hat[oi] = round_out<IO>(re);
        } else if (2 * k == N) {
            w_hat[(int64_t)(N - 1) * plane + oi] = round_out<IO>(re);
        } else {
            w_hat[(int64_t)(2 * k - 1) * plane + oi] = round_out<IO>(re);
            w_hat[(int64_t)(2 * k) * plane + oi] = round_out<IO>(im);
        }
    }
}

hipError_t launch_weight_dft(int N, int io, const void* w, void* w_hat, int C_in,
                             int C_out, hipStream_t stream) {
    TwArg tw{};
    for (int j = 0; j < N; ++j) {
        tw.cs[j] = turn_trig(j, N, false);
        tw.sn[j] = turn_trig(j, N, true);
    }
    const int64_t plane = (int64_t)C_in * C_out;
    const int threads = 256;
    const int64_t blocks = (plane + threads - 1) / threads;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (io == kIoBF16)
        hipLaunchKernelGGL(weight_dft_kernel<__bf16>, dim3((uint32_t)blocks), dim3(threads), 0,
                           stream, (const __bf16*)w, (__bf16*)w_hat, N, plane, tw);
    else if (io == kIoF16)
        hipLaunchKernelGGL(weight_dft_kernel<_Float16>, dim3((uint32_t)blocks), dim3(threads), 0,
                           stream, (const _Float16*)w, (_Float16*)w_hat, N, plane, tw);
    else
        hipLaunchKernelGGL(weight_dft_kernel<float>, dim3((uint32_t)blocks), dim3(threads), 0,
                           stream, (const float*)w, (float*)w_hat, N, plane, tw);
    return hipGetLastError();
}

// W_dense[o*N+g][i*N+h] = w[o][i][(g-h) mod N].
template <typename IO>
__global__ void cn_expand_kernel(const IO* __restrict__ w, IO* __restrict__ W, int N, int C_in,
                                 int64_t total) {
    const int64_t cols = (int64_t)N * C_in;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = e / cols, c = e % cols;
        const int64_t o = r / N, g = r % N, i = c / N, h = c % N;
        const int64_t m = (g - h + N) % N;
        W[e] = w[(o * C_in + i) * N + m];
    }
}

// Block-diagonal D8 matrix [C_out][C_in] from [W_A1|W_A2|W_B1|W_B2|W_E].
// Dihedral block matrix W[C_out][C_in] from the packed blocks: a square block per
// 1-D irrep (n1 of them, m x m), then per 2-D irrep E_k one (2m x 2m) block on
// both of its coordinates (D8: n = 4, n1 = 4, one E).
template <typename IO>
__global__ void dn_expand_kernel(const IO* __restrict__ wb, IO* __restrict__ W, int n, int C_in, int C_out,
                                 int64_t total) {
    const int mi = C_in / (2 * n), mo = C_out / (2 * n), n1 = n % 2 == 0 ? 4 : 2;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int r = (int)(e / C_in), c = (int)(e % C_in);
        IO v = (IO)0.0f;
        if (r < n1 * mo) {
            const int b = r / mo;
            if (c >= b * mi && c < (b + 1) * mi)
                v = wb[(int64_t)b * mo * mi + (int64_t)(r - b * mo) * mi + (c - b * mi)];
        } else {
            const int er = r - n1 * mo, k = er / (4 * mo);
            const int ce = (er % (4 * mo)) / (2 * mo), rr = er % (2 * mo);
            const int c_lo = n1 * mi + 4 * k * mi + 2 * ce * mi;
            if (c >= c_lo && c < c_lo + 2 * mi)
                v = wb[(int64_t)n1 * mo * mi + (int64_t)k * 4 * mo * mi + (int64_t)rr * (2 * mi) + (c - c_lo)];
        }
        W[e] = v;
    }
}

static uint32_t grid_for(int64_t total, int threads) {
    int64_t b = (total + threads - 1) / threads;
    return (uint32_t)(b > 65536 ? 65536 : (b < 1 ? 1 : b));
}

hipError_t launch_cn_expand(int N, int io, const void* w, void* w_dense, int C_in,
                            int C_out, hipStream_t stream) {
    const int64_t total = (int64_t)N * C_out * N * C_in;
    if (io == kIoBF16)
        hipLaunchKernelGGL(cn_expand_kernel<__bf16>, dim3(grid_for(total, 256)), dim3(256), 0,
                           stream, (const __bf16*)w, (__bf16*)w_dense, N, C_in, total);
    else if (io == kIoF16)
        hipLaunchKernelGGL(cn_expand_kernel<_Float16>, dim3(grid_for(total, 256)), dim3(256), 0,
                           stream, (const _Float16*)w, (_Float16*)w_dense, N, C_in, total);
    else
        hipLaunchKernelGGL(cn_expand_kernel<float>, dim3(grid_for(total, 256)), dim3(256), 0,
                           stream, (const float*)w, (float*)w_dense, N, C_in, total);
    return hipGetLastError();
}

hipError_t launch_dn_expand(int n, int io, const void* wb, void* w_dense, int C_in, int C_out,
                            hipStream_t stream) {
    const int64_t total = (int64_t)C_out * C_in;
    if (io == kIoF16)
        hipLaunchKernelGGL(dn_expand_kernel<_Float16>, dim3(grid_for(total, 256)), dim3(256), 0,
                           stream, (const _Float16*)wb, (_Float16*)w_dense, n, C_in, C_out, total);
    else if (io == kIoBF16)
        hipLaunchKernelGGL(dn_expand_kernel<__bf16>, dim3(grid_for(total, 256)), dim3(256), 0,
                           stream, (const __bf16*)wb, (__bf16*)w_dense, n, C_in, C_out, total);
    else
        hipLaunchKernelGGL(dn_expand_kernel<float>, dim3(grid_for(total, 256)), dim3(256), 0,
                           stream, (const float*)wb, (float*)w_dense, n, C_in, C_out, total);
    return hipGetLastError();
}

}  // namespace eql
