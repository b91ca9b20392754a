// cn_fused_bf16_n9.hip -- fused C_N forward instantiations, bf16, N = 9..12.
#include "cn_dispatch.h"

namespace eql {

template hipError_t launch_fused<9, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<10, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<11, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<12, __bf16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);

}  // namespace eql
