// cn_fused_f16_n1.hip -- fused C_N forward instantiations, f16, N = 1..4.
#include "cn_dispatch.h"

namespace eql {

template hipError_t launch_fused<1, _Float16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<2, _Float16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<3, _Float16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<4, _Float16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);

}  // namespace eql
