// cn_fwd_f32_hi.hip -- fused C_N forward instantiations, f32, N = 9..16.
#include "cn_forward_impl.h"

namespace eql {

template hipError_t launch_n<9, float>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<10, float>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<11, float>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<12, float>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<13, float>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<14, float>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<15, float>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<16, float>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);

}  // namespace eql
