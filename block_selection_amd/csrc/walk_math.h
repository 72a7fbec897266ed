// walk_math.h -- scoring arithmetic of the coarse-to-fine walk, shared by the
// prefill and decode kernels (gfx950).
//
// Reading note "Block Sparse Attention with Log-Linear Complexity", "Scoring:
// LogSumExp" and section 4.1: a candidate's score is, per query head, the LSE
// of the query's logits against the candidate's children (summaries above the
// leaf level, raw keys at the leaf level), summed over the heads of the GQA
// group. Logits are q.k/sqrt(64), handled in base 2 (the log2(e) factor is
// folded into the summaries or applied to the MFMA result).
//
// Prefill and decode use exactly these instruction sequences, so a decode step
// selects, bit for bit, what prefill selects at the same query position.
#pragma once

#include "lanes.h"

namespace pisa {

constexpr float kScale2 = 0.125f * 1.4426950408889634f;   // log2(e) / sqrt(64)

__device__ inline uint32_t rne_bf16_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// hi = rne_bf16(x * kScale2), lo = rne_bf16(x * kScale2 - hi): two bf16 planes whose
// sum carries a 17-bit mantissa of the scaled summary value.
__device__ inline void split_scaled(float x, uint32_t& hi, uint32_t& lo) {
    const float v = x * kScale2;
    hi = rne_bf16_bits(v);
    lo = rne_bf16_bits(v - __uint_as_float(hi << 16));
}

// Eight consecutive fp32 summary values -> hi and lo bf16x8 fragments (element e in
// half e & 1 of word e / 2, as the MFMA operand expects).
__device__ inline void split8(const float v[8], u32x4& h, u32x4& l) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t h0, l0, h1, l1;
        split_scaled(v[2 * i], h0, l0);
        split_scaled(v[2 * i + 1], h1, l1);
        h[i] = h0 | (h1 << 16);
        l[i] = l0 | (l1 << 16);
    }
}

// Base-2 logits of a 16-row tile of summaries (row = lane % 16) against the query
// fragments q0 (dims 8gq..8gq+7) and q1 (dims 32+8gq..32+8gq+7): hi plane then lo
// plane, two k-steps each, one accumulation chain.
__device__ inline f32x4 child_tile_mfma(const bf16x8 q0, const bf16x8 q1, u32x4 h0, u32x4 h1, u32x4 l0,
                                        u32x4 l1) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, h0), q0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, h1), q1, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, l0), q0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, l1), q1, acc, 0, 0, 0);
    return acc;
}

// log2(2^a + 2^b)
__device__ inline float log2_add_exp2(float a, float b) {
    const float m = fmaxf(a, b), d = fminf(a, b) - m;
    return m + __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(d));
}

// Scores of the two candidates whose children fill rows 4gq..4gq+3 of a child tile
// (candidate p: left child row 4gq+2p, right child row 4gq+2p+1). rows_ok bit r says
// row r is an eligible child; a candidate without an eligible left child scores -inf,
// one without an eligible right child takes its left child's logit alone. Every lane of
// row group gq receives both sums over the group's heads (columns n < GQ).
__device__ inline void pair_scores(const f32x4& acc, uint32_t rows_ok, int gq, int n, int GQ, float sc[2]) {
    if ((rows_ok & 0xffffu) == 0xffffu && GQ == kMaxGroup) {
        // every child eligible and every column a head of the group: no masks (same result)
#pragma unroll
        for (int p = 0; p < 2; ++p) sc[p] = row16_sum(log2_add_exp2(acc[2 * p], acc[2 * p + 1]));
        return;
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const bool lv = (rows_ok >> (4 * gq + 2 * p)) & 1u;
        const bool rv = (rows_ok >> (4 * gq + 2 * p + 1)) & 1u;
        const float lse2 = rv ? log2_add_exp2(acc[2 * p], acc[2 * p + 1]) : acc[2 * p];
        const float sm = row16_sum(n < GQ ? lse2 : 0.0f);
        sc[p] = lv ? sm : -INFINITY;
    }
}

// ---------------------------------------------------------------- delta form --
// For a candidate c with children a = 2c and b = 2c+1 and a query head, write the
// base-2 logits as L_a = p + d and L_b = p - d, with p the logit of c's own summary and
// d the logit of delta(c) = s(a) - s(c). L_a = p + d holds for every node; L_b = p - d
// holds when c is the plain mean of two children (every node except the one ragged
// node at the right edge of a level). Then LSE(L_a, L_b) = p + g(d) with
// g(d) = log2(2^d + 2^-d), and the group-summed score is P(c) + sum_h g(d_h), where
// P(c) = sum_h p_h is carried down the walk: P(a) = P + D, P(b) = P - D, D = sum_h d_h.
// One summary row (delta) per candidate replaces the two children rows.

// log2(2^d + 2^-d) = |d| + log2(1 + 2^(-2|d|))
__device__ inline float pair_lse_term(float d) {
    const float a = fabsf(d);
    return a + __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(-2.0f * a));
}

// Sums over the 16 head columns of four values per lane: v[i] in lane (g, n) belongs to
// tile row 4g + i and head column n. Afterwards every lane (g, n) holds the sum of row
// 4g + (n & 3); the four lanes of a row group that hold the same row get bitwise equal
// sums (a reduce-scatter over lane ^ 2 and lane ^ 1, then a symmetric butterfly over
// lane ^ 8 and lane ^ 4), so the result does not depend on which of them is read.
__device__ inline float head_sum4(const float v[4], int n) {
    const bool b1 = (n >> 1) & 1, b0 = n & 1;
    // lane ^ 2: lanes with b1 = 0 keep rows 0, 1 and hand over rows 2, 3 (and vice versa)
    const float k0 = b1 ? v[2] : v[0], k1 = b1 ? v[3] : v[1];
    const float s0 = b1 ? v[0] : v[2], s1 = b1 ? v[1] : v[3];
    const float r0 = k0 + lane_xor_f<2>(s0);
    const float r1 = k1 + lane_xor_f<2>(s1);
    // lane ^ 1: keep row 2 b1 + b0
    const float k = b0 ? r1 : r0, sd = b0 ? r0 : r1;
    float x = k + lane_xor_f<1>(sd);
    // the four quads of the row group
    x = x + lane_xor_f<8>(x);
    x = x + lane_xor_f<4>(x);
    return x;
}

// Selection key that also records the slot a candidate came from: selection order
// (score desc, node asc); low word (2^26 - 1 - node) << 6 | slot, 0 for an empty slot.
// Nodes of levels >= 2 are below 2^24.
__device__ inline uint64_t slot_key(float s, int node, int slot) {
    const uint32_t u = __float_as_uint(s + 0.0f);
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    const uint32_t low = (node >= 0) ? (((uint32_t)((1 << 26) - 1 - node) << 6) | (uint32_t)slot) : 0u;
    return ((uint64_t)o << 32) | low;
}
__device__ inline int key_node(uint32_t low) { return (low >> 6) ? (1 << 26) - 1 - (int)(low >> 6) : -1; }
__device__ inline int key_slot(uint32_t low) { return (int)(low & 63u); }

// This lane's sum over its 16 keys of one leaf (acc[tau][r]: key 16 tau + 4 gq + r) of
// 2^(logit * kScale2 - shift), keys past lim masked (kFull: none are). The 16 terms are
// added as a balanced tree in one fixed order, so every leaf scorer that uses this gets
// the same bits for the same logits.
template <bool kFull>
__device__ inline float leaf_exp_sum(const f32x4 (&acc)[4], int lim, int gq, float shift = 0.0f) {
    float e[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int tau = i >> 2, r = i & 3;
        const float x = (shift == 0.0f) ? acc[tau][r] * kScale2 : __builtin_fmaf(acc[tau][r], kScale2, -shift);
        const float e2 = __builtin_amdgcn_exp2f(x);
        e[i] = (kFull || 16 * tau + 4 * gq + r <= lim) ? e2 : 0.0f;
    }
#pragma unroll
    for (int w = 1; w < 16; w <<= 1)
#pragma unroll
        for (int i = 0; i < 16; i += 2 * w) e[i] = e[i] + e[i + w];
    return e[0];
}

// Largest unmasked logit (natural scale) of this lane's 16 keys of one leaf.
__device__ inline float leaf_lane_max(const f32x4 (&acc)[4], int lim, int gq) {
    float m = -INFINITY;
#pragma unroll
    for (int tau = 0; tau < 4; ++tau)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (16 * tau + 4 * gq + r <= lim) m = fmaxf(m, acc[tau][r]);
    return m;
}

// Leaf scores from the MFMA results of NL leaves: acc[j][tau] holds, in lane (gq, n),
// the natural-scale logits of keys 16*tau + 4*gq + r (r = 0..3) of leaf j for head n.
// Keys with offset > lim[j] are masked. Per head the base-2 LSE is taken without a max
// shift (sum of 2^x, then log2); a leaf whose sum overflowed or underflowed in any head
// is redone with each head's maximum logit subtracted. out[j] (every lane): the sum
// over the group's heads of the base-2 LSE.
template <int NL>
__device__ inline void leaf_lse_from_acc(const f32x4 (&acc)[NL][4], const int (&lim)[NL], int n, int gq, int GQ,
                                         float out[NL]) {
    bool full = true;
#pragma unroll
    for (int j = 0; j < NL; ++j) full = full && (lim[j] == kC - 1);
    float s[NL], shift[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        s[j] = cols4_sum(full ? leaf_exp_sum<true>(acc[j], lim[j], gq) : leaf_exp_sum<false>(acc[j], lim[j], gq));
        shift[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        if (ballot(!(s[j] < INFINITY && s[j] > 0x1p-100f))) {
            // rare: shift by the maximum logit of each column
            const float moff = cols4_max(leaf_lane_max(acc[j], lim[j], gq)) * kScale2;
            s[j] = cols4_sum(leaf_exp_sum<false>(acc[j], lim[j], gq, moff));
            shift[j] = moff;
        }
    }
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const float lse2 = shift[j] + __builtin_amdgcn_logf(s[j]);
        out[j] = row16_sum((n < GQ) ? lse2 : 0.0f);
    }
}

}  // namespace pisa
