// cn_fused_f32_n9.hip -- fused C_N forward instantiations, f32, N = 9..12.
#include "cn_dispatch.h"

namespace eql {

template hipError_t launch_fused<9, float>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<10, float>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<11, float>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<12, float>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);

}  // namespace eql
