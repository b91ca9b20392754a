// cn_fused_bf16_n1.hip -- fused C_N forward instantiations, bf16, N = 1..4.
#include "cn_dispatch.h"

namespace eql {

template hipError_t launch_fused<1, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<2, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<3, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<4, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);

}  // namespace eql
