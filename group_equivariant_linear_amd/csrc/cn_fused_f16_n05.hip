// cn_fused_f16_n5.hip -- fused C_N forward instantiations, f16, N = 5..8.
#include "cn_dispatch.h"

namespace eql {

template hipError_t launch_fused<5, _Float16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<6, _Float16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<7, _Float16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<8, _Float16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);

}  // namespace eql
