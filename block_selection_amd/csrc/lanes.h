// lanes.h -- cross-lane moves, reductions and segmented sorts for 64-wide wavefronts (gfx950).
//
// DPP row operations move data inside 16-lane rows without the LDS crossbar;
// v_permlane16_swap / v_permlane32_swap (gfx950) exchange rows and wavefront
// halves. Every xor distance of a 64-lane bitonic network is a VALU move.
#pragma once

#include "pisa_device.h"

namespace pisa {

// value of lane (lane ^ J), by VALU moves only (no LDS crossbar round trip)
template <int J>
__device__ inline int lane_xor(int v) {
    if constexpr (J == 1) {
        return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);    // quad_perm 1,0,3,2
    } else if constexpr (J == 2) {
        return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);    // quad_perm 2,3,0,1
    } else if constexpr (J == 4) {
        // row_half_mirror takes lane ^ 7 inside each 8-lane half row, quad_perm 3,2,1,0 then
        // lane ^ 3: together lane ^ 4
        const int m = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
        return __builtin_amdgcn_update_dpp(0, m, 0x1B, 0xF, 0xF, false);
    } else if constexpr (J == 8) {
        return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);   // row_ror 8
    } else if constexpr (J == 16) {
        // v_permlane16_swap exchanges odd rows of its first operand with even rows of the
        // second; with both = v, result[0] holds row r ^ 1 on odd rows, result[1] on even rows
        const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
        return (int)(((threadIdx.x >> 4) & 1) ? r[0] : r[1]);
    } else {
        static_assert(J == 32, "lane_xor: J must be 1, 2, 4, 8, 16 or 32");
        const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
        return (int)(((threadIdx.x >> 5) & 1) ? r[0] : r[1]);
    }
}
template <int J>
__device__ inline float lane_xor_f(float v) { return __int_as_float(lane_xor<J>(__float_as_int(v))); }

// Sum over the 16 lanes of each DPP row; every lane of the row receives it.
__device__ inline float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror 4
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror 8
    return v;
}

// Combine lane l with lane l ^ 16 and with lane l ^ 32 (all four rows of one column).
__device__ inline float cols4_max(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float cols4_sum(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Does (sa, na) come before (sb, nb)? Higher score first, then lower index.
__device__ inline bool precedes(float sa, int na, float sb, int nb) {
    return sa > sb || (sa == sb && na < nb);
}

template <int J>
__device__ inline void bitonic_step(float& s, int& nd, int i, int k) {
    const float so = lane_xor_f<J>(s);
    const int no = lane_xor<J>(nd);
    const bool lower = (i & J) == 0;
    const bool up = (i & k) == 0;
    const bool self_first = precedes(s, nd, so, no);
    const bool keep_self = (lower == up) ? self_first : !self_first;
    if (!keep_self) { s = so; nd = no; }
}

// Bitonic sort of (s, nd) inside each segment of SLOTS lanes (i = lane % SLOTS):
// afterwards segment lane 0 holds the element that precedes all others.
template <int SLOTS>
__device__ inline void segment_sort(float& s, int& nd, int i) {
#pragma unroll
    for (int k = 2; k <= SLOTS; k <<= 1) {
        if (k >= 64) { bitonic_step<32>(s, nd, i, k); }
        if (k >= 32) { bitonic_step<16>(s, nd, i, k); }
        if (k >= 16) { bitonic_step<8>(s, nd, i, k); }
        if (k >= 8) { bitonic_step<4>(s, nd, i, k); }
        if (k >= 4) { bitonic_step<2>(s, nd, i, k); }
        bitonic_step<1>(s, nd, i, k);
    }
}

}  // namespace pisa
