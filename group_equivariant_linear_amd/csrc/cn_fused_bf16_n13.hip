// cn_fused_bf16_n13.hip -- fused C_N forward instantiations, bf16, N = 13..16.
#include "cn_dispatch.h"

namespace eql {

template hipError_t launch_fused<13, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<14, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<15, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<16, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);

}  // namespace eql
