// cn_fused_f16_n13.hip -- fused C_N forward instantiations, f16, N = 13..16.
#include "cn_dispatch.h"

namespace eql {

template hipError_t launch_fused<13, _Float16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<14, _Float16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<15, _Float16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<16, _Float16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);

}  // namespace eql
