// cn_fwd_f32_lo.hip -- fused C_N forward instantiations, f32, N = 1..8.
#include "cn_forward_impl.h"

namespace eql {

template hipError_t launch_n<1, float>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<2, float>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<3, float>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<4, float>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<5, float>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<6, float>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<7, float>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);
template hipError_t launch_n<8, float>(const void*, const void*, void*, int64_t, int, int,
                                        hipStream_t, int);

}  // namespace eql
