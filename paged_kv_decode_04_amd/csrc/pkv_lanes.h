// pkv_lanes.h -- sums over aligned groups of lanes of a wavefront, on the VALU (DPP lane patterns and
// v_permlane16_swap), shared by the gfx950 kernels.  Every lane of a group gets the group's total.
#pragma once

#include <hip/hip_runtime.h>

namespace pkv {

// DPP lane patterns (GFX9 encodings of the dpp_ctrl field)
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppRowRor = 0x120;     // row_ror:n = 0x120 + n (rotate within a row of 16 lanes)
constexpr int kDppHalfMirror = 0x141; // row_half_mirror (lane i <-> 7 - i within each 8)

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N = 4, 8, 16 or 32): quad permutations, a half-row mirror, row rotations,
// and a v_permlane16_swap across the two rows of a 32-lane group.
template <int N>
__device__ __forceinline__ float lanes_sum(float x) {
    static_assert(N == 4 || N == 8 || N == 16 || N == 32, "groups of 4, 8, 16 or 32 lanes");
    if (N == 4) {
        x += dpp<kDppXor1>(x);
        x += dpp<kDppXor2>(x);
    } else if (N == 8) {
        x += dpp<kDppHalfMirror>(x);  // x_i + x_{7-i}: symmetric within the 8
        x += dpp<kDppXor1>(x);
        x += dpp<kDppXor2>(x);         // the quad and its mirror: all 8
    } else {
        x += dpp<kDppRowRor + 8>(x);
        x += dpp<kDppRowRor + 4>(x);
        x += dpp<kDppRowRor + 2>(x);
        x += dpp<kDppRowRor + 1>(x);   // all 16 of the row
        if (N == 32) {
            auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
            x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
        }
    }
    return x;
}

}  // namespace pkv
