// cn_fwd_bf16_lo.hip -- fused C_N forward instantiations, bf16, N = 1..8.
#include "cn_forward_impl.h"

namespace eql {

template hipError_t launch_n<1, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<2, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<3, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<4, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<5, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<6, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<7, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<8, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);

}  // namespace eql
