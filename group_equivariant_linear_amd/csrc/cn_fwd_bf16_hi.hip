// cn_fwd_bf16_hi.hip -- fused C_N forward instantiations, bf16, N = 9..16.
#include "cn_forward_impl.h"

namespace eql {

template hipError_t launch_n<9, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<10, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<11, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<12, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<13, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<14, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<15, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<16, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);

}  // namespace eql
