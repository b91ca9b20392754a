// cn_fused_f16_n9.hip -- fused C_N forward instantiations, f16, N = 9..12.
#include "cn_dispatch.h"

namespace eql {

template hipError_t launch_fused<9, _Float16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<10, _Float16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<11, _Float16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);
template hipError_t launch_fused<12, _Float16>(const void*, const void*, void*, int64_t, int, int,
                                            hipStream_t, int, Epi);

}  // namespace eql
