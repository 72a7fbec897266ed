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
    // every source lane of these patterns exists, so no "old" value is needed
    if constexpr (J == 1) {
        return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);    // quad_perm 1,0,3,2
    } else if constexpr (J == 2) {
        return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);    // quad_perm 2,3,0,1
    } else if constexpr (J == 4) {
        // row_half_mirror takes lane ^ 7 inside each 8-lane half row, quad_perm 3,2,1,0 then
        // lane ^ 3: together lane ^ 4
        const int m = __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true);
        return __builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, true);
    } else if constexpr (J == 8) {
        return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true);   // row_ror 8
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

// ---------------------------------------------------------------- sorting --
// Selection order: higher score first, equal scores lower index first. A (score,
// index) pair is packed into one 64-bit key whose descending unsigned order is the
// selection order: the score's bits mapped to an order-preserving unsigned integer
// (-0 folded into +0 so the two tie), then the complemented index. A bitonic step
// is then two lane moves, one 64-bit compare and two selects.
__device__ inline uint64_t select_key(float s, int nd) {
    const uint32_t u = __float_as_uint(s + 0.0f);
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)o << 32) | (uint64_t)(~(uint32_t)nd);
}
__device__ inline int key_index(uint64_t key) { return (int)~(uint32_t)key; }

template <int X>
__device__ inline uint32_t lane_xor_u32(uint32_t v) { return (uint32_t)lane_xor<X>((int)v); }
template <int X>
__device__ inline uint64_t lane_xor_u64(uint64_t v) {
    const uint64_t lo = lane_xor_u32<X>((uint32_t)v), hi = lane_xor_u32<X>((uint32_t)(v >> 32));
    return (hi << 32) | lo;
}

// Compare-exchange of a descending bitonic network: this lane holds slot m, its
// partner slot m ^ J sits X lanes away; k is the size of the sequences being merged.
template <int J, int X, typename T>
__device__ inline void key_step(T& key, int m, int k) {
    T o;
    if constexpr (sizeof(T) == 8) o = lane_xor_u64<X>(key);
    else o = lane_xor_u32<X>(key);
    const bool flip = ((m & J) == 0) != ((m & k) == 0);
    key = ((key > o) != flip) ? key : o;
}

// Plain lane layout: slot i of a segment is lane offset i.
struct SegmentLanes {
    static constexpr int of(int J) { return J; }
};

// Descending sort of the keys of each segment of SLOTS slots (slot m of this lane).
template <int SLOTS, typename Lanes, typename T>
__device__ inline T bitonic_desc(T key, int m) {
#pragma unroll
    for (int k = 2; k <= SLOTS; k <<= 1) {
        if (k >= 64) key_step<32, Lanes::of(32)>(key, m, k);
        if (k >= 32) key_step<16, Lanes::of(16)>(key, m, k);
        if (k >= 16) key_step<8, Lanes::of(8)>(key, m, k);
        if (k >= 8) key_step<4, Lanes::of(4)>(key, m, k);
        if (k >= 4) key_step<2, Lanes::of(2)>(key, m, k);
        key_step<1, Lanes::of(1)>(key, m, k);
    }
    return key;
}

// The SLOTS/2 largest keys of each segment, in slots 0 .. SLOTS/2 - 1 in no particular
// order: the halves are sorted in opposite directions (the network above up to sequences
// of SLOTS/2), then one compare-exchange of slot m with m + SLOTS/2 splits the bitonic
// whole into its larger and smaller halves. log2(SLOTS) - 1 fewer steps than the sort.
template <int SLOTS, typename Lanes, typename T>
__device__ inline T bitonic_top_half(T key, int m) {
    static_assert(SLOTS >= 2, "a segment holds at least two slots");
#pragma unroll
    for (int k = 2; k < SLOTS; k <<= 1) {
        if (k >= 64) key_step<32, Lanes::of(32)>(key, m, k);
        if (k >= 32) key_step<16, Lanes::of(16)>(key, m, k);
        if (k >= 16) key_step<8, Lanes::of(8)>(key, m, k);
        if (k >= 8) key_step<4, Lanes::of(4)>(key, m, k);
        if (k >= 4) key_step<2, Lanes::of(2)>(key, m, k);
        key_step<1, Lanes::of(1)>(key, m, k);
    }
    key_step<SLOTS / 2, Lanes::of(SLOTS / 2)>(key, m, SLOTS);
    return key;
}

// Value of lane l ^ (B - 1) within blocks of B lanes (the mirror image inside the block), one
// DPP move for B <= 16.
template <int B>
__device__ inline uint32_t lane_mirror_u32(uint32_t v) {
    if constexpr (B == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);    // quad_perm 1,0,3,2
    else if constexpr (B == 4) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x1B, 0xF, 0xF, true);  // quad_perm 3,2,1,0
    else if constexpr (B == 8) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true); // row_half_mirror
    else {
        static_assert(B == 16, "lane_mirror: B must be 2, 4, 8 or 16");
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true);                       // row_mirror
    }
}

// Compare-exchange of slot m with slot m ^ (B - 1) (mirror, MIRROR) or m ^ B (xor) on plain
// lanes: the slot whose bit H = B / 2 (mirror) or B (xor) is clear keeps the larger key.
template <int B, bool MIRROR>
__device__ inline void key_step_fixed(uint64_t& key, int m) {
    uint64_t o;
    if constexpr (MIRROR) {
        o = ((uint64_t)lane_mirror_u32<B>((uint32_t)(key >> 32)) << 32) | lane_mirror_u32<B>((uint32_t)key);
    } else {
        o = lane_xor_u64<B>(key);
    }
    const bool low = (m & (MIRROR ? B / 2 : B)) == 0;
    key = ((key > o) == low) ? key : o;
}

// bitonic_top_half for segments of at most 16 plain lanes, in the form whose comparators all
// point one way: each merge of blocks of size k starts with a mirror step (slot m against m ^ (k
// - 1)) followed by xor steps at k/4 .. 1, so every block ends sorted descending; the final
// mirror step over the whole segment keeps max(A[i], B[SLOTS/2 - 1 - i]) of the two sorted
// halves A, B: the larger half as a set. Every move is one DPP instruction per 32-bit word
// (the xor network needs two for distance 4).
template <int SLOTS>
__device__ inline uint64_t top_half_mirror(uint64_t key, int m) {
    static_assert(SLOTS >= 2 && SLOTS <= 16, "segments of 2 .. 16 lanes");
    if constexpr (SLOTS >= 4) key_step_fixed<2, true>(key, m);
    if constexpr (SLOTS >= 8) {
        key_step_fixed<4, true>(key, m);
        key_step_fixed<1, false>(key, m);
    }
    if constexpr (SLOTS >= 16) {
        key_step_fixed<8, true>(key, m);
        key_step_fixed<2, false>(key, m);
        key_step_fixed<1, false>(key, m);
    }
    key_step_fixed<SLOTS, true>(key, m);
    return key;
}

// The index at slot m after ordering each segment's (score, index) pairs by selection
// order (slot 0 = the pair that precedes all others).
template <int SLOTS, typename Lanes = SegmentLanes>
__device__ inline int select_sort(float s, int nd, int m) {
    return key_index(bitonic_desc<SLOTS, Lanes>(select_key(s, nd), m));
}

// The index at slot m < SLOTS/2 after keeping each segment's SLOTS/2 (score, index) pairs
// that come first in selection order (unordered among themselves).
template <int SLOTS, typename Lanes = SegmentLanes>
__device__ inline int select_top_half(float s, int nd, int m) {
    return key_index(bitonic_top_half<SLOTS, Lanes>(select_key(s, nd), m));
}

// The index at slot m after sorting each segment's indices ascending (nonnegative
// indices; INT_MAX sorts last).
template <int SLOTS, typename Lanes = SegmentLanes>
__device__ inline int index_sort(int nd, int m) {
    return (int)~bitonic_desc<SLOTS, Lanes>(~(uint32_t)nd, m);
}

}  // namespace pisa
