// cn_forward.hip -- dispatch of the fused C_N forward over group order and dtype.
// The kernel (cn_fused.h) is instantiated in cn_fused_{f32,bf16,f16}_nXX.hip so the
// instantiations build in parallel.
#include "eq_launch.h"

namespace eql {

template <int N, typename IO>
hipError_t launch_fused(const void* x, const void* w_hat, void* y, int64_t T, int C_in, int C_out,
                        hipStream_t stream, int tile, Epi epi);

template <typename IO>
static hipError_t launch_dt(int N, const void* x, const void* w_hat, void* y, int64_t T,
                            int C_in, int C_out, hipStream_t stream, int tile, Epi epi) {
    switch (N) {
#define EQL_CASE(n) \
    case n: return launch_fused<n, IO>(x, w_hat, y, T, C_in, C_out, stream, tile, epi);
        EQL_CASE(1) EQL_CASE(2) EQL_CASE(3) EQL_CASE(4) EQL_CASE(5) EQL_CASE(6) EQL_CASE(7)
        EQL_CASE(8) EQL_CASE(9) EQL_CASE(10) EQL_CASE(11) EQL_CASE(12) EQL_CASE(13)
        EQL_CASE(14) EQL_CASE(15) EQL_CASE(16)
#undef EQL_CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_cn_forward(int N, int io, const void* x, const void* w_hat, void* y,
                             int64_t T, int C_in, int C_out, hipStream_t stream, int tile, Epi epi) {
    switch (io) {
        case kIoBF16: return launch_dt<__bf16>(N, x, w_hat, y, T, C_in, C_out, stream, tile, epi);
        case kIoF16: return launch_dt<_Float16>(N, x, w_hat, y, T, C_in, C_out, stream, tile, epi);
        case kIoF32: return launch_dt<float>(N, x, w_hat, y, T, C_in, C_out, stream, tile, epi);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace eql
