// cn_stream_bf16.hip -- the persistent C_N forward (cn_stream.h), bf16, N = 2..8.
// Built without the MFMA-results-in-VGPRs option: one wave per SIMD, so the
// accumulators may live in the accumulation registers and the wave may hold
// the whole register file.
#include "cn_stream.h"

namespace eql {

#define EQL_ST(n)                                                                                           \
    template hipError_t launch_stream<n, __bf16, 3>(const void*, const void*, void*, int64_t, int, int, \
                                                    hipStream_t, Epi);
EQL_ST(2) EQL_ST(3) EQL_ST(4) EQL_ST(5) EQL_ST(6) EQL_ST(7) EQL_ST(8)
#undef EQL_ST

hipError_t launch_cn_stream_bf16(int N, const void* x, const void* w_hat, void* y, int64_t T, int C_in, int C_out,
                               hipStream_t stream, Epi epi) {
    switch (N) {
#define EQL_STC(n) \
    case n: return launch_stream<n, __bf16, 3>(x, w_hat, y, T, C_in, C_out, stream, epi);
        EQL_STC(2) EQL_STC(3) EQL_STC(4) EQL_STC(5) EQL_STC(6) EQL_STC(7) EQL_STC(8)
#undef EQL_STC
        default: return hipErrorNotSupported;
    }
}

}  // namespace eql
