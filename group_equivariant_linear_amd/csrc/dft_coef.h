// dft_coef.h -- coefficients of the packed real DFT along the group axis, as
// compile-time doubles for the kernels that run the transform as a matrix
// product on the matrix cores.
#pragma once

#include "eq_device.h"

namespace eql {

// Coefficient of plane p at group element h, planes packed as in rdft_forward:
// plane 0 = DC, planes 2k-1 and 2k = Re and Im of bin k, plane N-1 = Nyquist
// for even N ("Flash EQ-Linear", Algorithmic Approach).
template <int N>
constexpr double fwd_coef(int p, int h) {
    if (p == 0) return 1.0;
    if (N % 2 == 0 && p == N - 1) return (h % 2) ? -1.0 : 1.0;
    const int k = (p + 1) / 2;
    return (p % 2) ? turn_trig((long)h * k, N, false) : -turn_trig((long)h * k, N, true);
}

}  // namespace eql
