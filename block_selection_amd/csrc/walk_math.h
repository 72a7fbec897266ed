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

// Truncated scores (the pages' ablations of the LSE): per head, mean(z) or
// mean(z) + var(z)/2 over the candidate's m eligible child logits z (population
// variance). Scores are kept in base-2 units x = z log2(e), i.e. log2(e) times the
// natural score (the order is the same): mean(x) + var(x) ln(2) / 2.
constexpr float kHalfVar2 = 0.5f * 0.6931471805599453f;    // ln(2) / 2

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

// Base-2 logits of 16 summary rows against the group's query heads, one MFMA tile: the
// queries are the A operand (tile row m = head m) and the rows the B operand (tile column
// n = the row that lane n % 16 supplies). Fragments: q0 / q1 hold dims 8gq..8gq+7 /
// 32+8gq..32+8gq+7 of head n, h* / l* the same dims of row n's hi / lo planes. Hi plane
// then lo plane, two k-steps each, one accumulation chain. Lane (gq, n) receives the logits
// of heads 4gq..4gq+3 against row n.
__device__ inline f32x4 summary_tile_mfma(const bf16x8 q0, const bf16x8 q1, u32x4 h0, u32x4 h1, u32x4 l0,
                                          u32x4 l1) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q0, __builtin_bit_cast(bf16x8, h0), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q1, __builtin_bit_cast(bf16x8, h1), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q0, __builtin_bit_cast(bf16x8, l0), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q1, __builtin_bit_cast(bf16x8, l1), acc, 0, 0, 0);
    return acc;
}

// Sum over the heads of a summary tile: lane (gq, n) adds its four heads as
// (v0 + v1) + (v2 + v3), then the four row groups are added pairwise (lane ^ 16, then
// lane ^ 32). Every lane of column n receives the same bits.
__device__ inline float heads_total(const float v[4]) { return cols4_sum((v[0] + v[1]) + (v[2] + v[3])); }

// Two column totals at once: sf and sd are a lane's in-lane parts of two quantities; one
// permlane16 exchange packs them into alternate row groups, one permlane32 exchange
// completes both as (r0 + r1) + (r2 + r3), and a last permlane16 exchange hands each lane
// both totals of its column.
__device__ inline void cols4_sum2(float sf, float sd, float& F, float& D) {
    // row groups 0..3 of the sum: f 0+1, d 0+1, f 2+3, d 2+3
    const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(sf), __float_as_uint(sd), false, false);
    const float S = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    // row groups: F, D, F, D
    const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(S), __float_as_uint(S), false, false);
    const float T = __uint_as_float(y[0]) + __uint_as_float(y[1]);
    const auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(T), __float_as_uint(T), false, false);
    F = __uint_as_float(z[0]);
    D = __uint_as_float(z[1]);
}

// Two head sums at once, in the order of heads_total.
__device__ inline void heads_total2(const float f[4], const float d[4], float& F, float& D) {
    cols4_sum2((f[0] + f[1]) + (f[2] + f[3]), (d[0] + d[1]) + (d[2] + d[3]), F, D);
}

// Head sum of the logits of each column of a summary tile. Heads past the group have zero
// query rows, so their logits are exactly 0 and add nothing.
__device__ inline float tile_head_sums(const f32x4& acc) {
    const float v[4] = {acc[0], acc[1], acc[2], acc[3]};
    return heads_total(v);
}

// log2(2^a + 2^b)
__device__ inline float log2_add_exp2(float a, float b) {
    const float m = fmaxf(a, b), d = fminf(a, b) - m;
    return m + __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(d));
}

// Base-2 score of one head over two child logits a and b: LSE, mean, or mean plus half
// the variance. The score S (kScore*) is a compile-time parameter throughout, so each
// kernel is built once per score and the LSE kernels carry no code of the others.
template <int S>
__device__ inline float combine2(float a, float b) {
    if constexpr (S == kScoreLse) return log2_add_exp2(a, b);
    const float mean = 0.5f * (a + b);
    if constexpr (S == kScoreMean) return mean;
    const float h = 0.5f * (a - b);                    // var of two values = ((a - b) / 2)^2
    return __builtin_fmaf(h * h, kHalfVar2, mean);
}

// Scores of the two candidates whose children fill rows 4gq..4gq+3 of a child tile
// (candidate p: left child row 4gq+2p, right child row 4gq+2p+1). rows_ok bit r says
// row r is an eligible child; a candidate without an eligible left child scores -inf,
// one without an eligible right child takes its left child's logit alone. Every lane of
// row group gq receives both sums over the group's heads (columns n < GQ).
template <int S>
__device__ inline void pair_scores(const f32x4& acc, uint32_t rows_ok, int gq, int n, int GQ, float sc[2]) {
    if ((rows_ok & 0xffffu) == 0xffffu && GQ == kMaxGroup) {
        // every child eligible and every column a head of the group: no masks (same result)
#pragma unroll
        for (int p = 0; p < 2; ++p) sc[p] = row16_sum(combine2<S>(acc[2 * p], acc[2 * p + 1]));
        return;
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const bool lv = (rows_ok >> (4 * gq + 2 * p)) & 1u;
        const bool rv = (rows_ok >> (4 * gq + 2 * p + 1)) & 1u;
        const float lse2 = rv ? combine2<S>(acc[2 * p], acc[2 * p + 1]) : acc[2 * p];
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
// One summary row (delta) per candidate replaces the two children rows. The delta rows
// are stored doubled (2 delta: exact, as is every step below), so a tile yields x = 2d.

// 2^-m, m = the number of heads of lane quarter gq (heads 4gq .. 4gq+3) past a group of GQ.
__device__ inline float past_group_scale(int gq, int GQ) {
    int m = 4 * gq + 4 - GQ;
    m = m < 0 ? 0 : (m > 4 ? 4 : m);
    return __uint_as_float((uint32_t)(127 - m) << 23);
}

// g(d) = log2(2^d + 2^-d) = |d| + log2(1 + 2^(-2|d|)); from x = 2d the exponent is -|x| (no
// multiply) and |d| = |x| / 2. Over the four heads a lane holds, the sum of the g is taken as
// (|x_1| + .. + |x_4|) / 2 + log2 of the product of the four factors 1 + 2^-|x_k|, each in
// (1, 2]: one logarithm per lane and tile rather than one per head.
//
// In-lane parts of one delta tile (column n = candidate n, its doubled delta row: acc = 2d;
// lane (gq, n) holds heads 4gq .. 4gq+3): x2 = the sum of the four 2d, as (x1 + x2) + (x3 +
// x4); f = the sum of the four pair terms: the above for the LSE, 0 for the mean (the
// children's logits p +- d have mean p: the score is the carried P), and for mean + var/2 the
// variance terms d^2 ln2/2 = x^2 ln2/8. A candidate without an eligible right child (rv
// false) has one child, whose logit is p + d for every score: f = x2 / 2 (halving is exact,
// so these are the bits of the sum of the d).
// Heads past the group have zero query rows, so their x are exactly 0: they add nothing to
// x2, the absolute sum or the variance terms, and a factor of exactly 2 each to the product,
// which scaling the last factor by 2^-m (past_group_scale) removes exactly (power-of-two
// scalings round exactly). For a full group the scale is 1 and the fma is the plain add.
template <int S>
__device__ inline void delta_tile_parts(const f32x4& acc, bool rv, int gq, int GQ, float& f, float& x2) {
    x2 = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    if constexpr (S == kScoreLse) {
        const float sc = past_group_scale(gq, GQ);
        const float e0 = 1.0f + __builtin_amdgcn_exp2f(-fabsf(acc[0]));
        const float e1 = 1.0f + __builtin_amdgcn_exp2f(-fabsf(acc[1]));
        const float e2 = 1.0f + __builtin_amdgcn_exp2f(-fabsf(acc[2]));
        const float e3 = __builtin_fmaf(sc, __builtin_amdgcn_exp2f(-fabsf(acc[3])), sc);
        const float a = (fabsf(acc[0]) + fabsf(acc[1])) + (fabsf(acc[2]) + fabsf(acc[3]));
        f = __builtin_fmaf(a, 0.5f, __builtin_amdgcn_logf((e0 * e1) * (e2 * e3)));
    } else if constexpr (S == kScoreMean) {
        f = 0.0f;
    } else {
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = (acc[k] * acc[k]) * (0.25f * kHalfVar2);
        f = (v[0] + v[1]) + (v[2] + v[3]);
    }
    f = rv ? f : 0.5f * x2;
}

// Pair sums of one delta tile: F = sum over the group's heads of the pair terms, D = sum of
// d (D = (sum of 2d) / 2 exactly). Every lane of column n receives both.
template <int S>
__device__ inline void delta_tile_sums(const f32x4& acc, bool rv, int gq, int GQ, float& F, float& D) {
    float f, x2, D2;
    delta_tile_parts<S>(acc, rv, gq, GQ, f, x2);
    cols4_sum2(f, x2, F, D2);
    D = 0.5f * D2;
}

// The pair sums of four delta tiles at once, scattered: lane (gq, n) receives F and D of
// tile gq, column n. f[i], x2[i] are tile i's in-lane parts (delta_tile_parts). The row
// groups are added as (r0 + r1) + (r2 + r3), the order of cols4_sum2, so every total has the
// bits delta_tile_sums gives the tile alone: four permlane16 exchanges add row pairs (0, 1)
// and (2, 3) while halving the values each lane holds, two permlane32 exchanges add the pairs.
__device__ inline void delta_sums4(const float (&f)[4], const float (&x2)[4], float& F, float& D) {
    auto pair16 = [](float a, float b) -> float {   // rows 0, 2: a of rows 0+1 / 2+3; rows 1, 3: b
        const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        return __uint_as_float(x[0]) + __uint_as_float(x[1]);
    };
    auto pair32 = [](float a, float b) -> float {   // rows 0, 1: a of (rows 0/1) + (rows 2/3); rows 2, 3: b
        const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        return __uint_as_float(y[0]) + __uint_as_float(y[1]);
    };
    // rows 0/2 hold tile 0 (resp. 2), rows 1/3 tile 1 (resp. 3), each summed over a row pair
    const float f01 = pair16(f[0], f[1]), f23 = pair16(f[2], f[3]);
    const float d01 = pair16(x2[0], x2[1]), d23 = pair16(x2[2], x2[3]);
    F = pair32(f01, f23);
    D = 0.5f * pair32(d01, d23);
}

// The ragged node's children read directly: column 0 of the tile holds the left child's
// logits, column 1 the right child's. F (read in column 0) = sum over the group's heads
// of the score of the two (log2(2^L + 2^R) for the LSE); Pc (column c) = the head sum of
// child c's logits. Call with every lane active (a lane exchange).
template <int S>
__device__ inline void ragged_sums(const f32x4& acc, int gq, int GQ, float& F, float& Pc) {
    float fv[4], pv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float r = lane_xor_f<1>(acc[k]);   // column 1 into column 0
        const bool h = 4 * gq + k < GQ;
        fv[k] = h ? combine2<S>(acc[k], r) : 0.0f;
        pv[k] = h ? acc[k] : 0.0f;
    }
    heads_total2(fv, pv, F, Pc);
}

// Selection key that also records the slot a candidate came from: selection order
// (score desc, node asc); low word (2^26 - 1 - node) << 6 | slot, and for an empty slot
// (node -1) the slot alone: low >> 6 = 0 marks it. Nodes of levels >= 2 are below 2^24.
__device__ inline uint64_t slot_key(float s, int node, int slot) {
    const uint32_t u = __float_as_uint(s + 0.0f);
    const uint32_t o = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
    // (~node) << 6 is (2^26 - 1 - node) << 6 for 0 <= node < 2^26, and 0 for node = -1
    const uint32_t low = ((uint32_t)~node << 6) | (uint32_t)slot;
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

// This lane's first and second moments over its 16 keys of one leaf: s1 = sum of x,
// s2 = sum of x^2 for the base-2 logits x = logit * kScale2 of the keys up to lim
// (kFull: all), in the balanced-tree order of leaf_exp_sum.
template <bool kFull>
__device__ inline void leaf_moments(const f32x4 (&acc)[4], int lim, int gq, float& s1, float& s2) {
#pragma clang fp contract(off)   // the same roundings wherever this is inlined
    float a[16], b[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int tau = i >> 2, r = i & 3;
        const float x = acc[tau][r] * kScale2;
        const bool in = kFull || 16 * tau + 4 * gq + r <= lim;
        a[i] = in ? x : 0.0f;
        b[i] = in ? x * x : 0.0f;
    }
#pragma unroll
    for (int w = 1; w < 16; w <<= 1)
#pragma unroll
        for (int i = 0; i < 16; i += 2 * w) {
            a[i] = a[i] + a[i + w];
            b[i] = b[i] + b[i + w];
        }
    s1 = a[0];
    s2 = b[0];
}

// Truncated score of one head over m keys from the moment totals (base-2 units).
template <int S>
__device__ inline float trunc_score2(float S1, float S2, int m) {
    const float inv = 1.0f / (float)m;
    const float mean = S1 * inv;
    if constexpr (S == kScoreMean) return mean;
    return __builtin_fmaf(__builtin_fmaf(S2, inv, -mean * mean), kHalfVar2, mean);
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

// The truncated scores of NL leaves from the same MFMA results (keys up to lim[j]):
// per head the moment totals over the leaf's lim[j] + 1 keys, then mean (+ var/2),
// summed over the group's heads.
template <int NL, int S>
__device__ inline void leaf_trunc_from_acc(const f32x4 (&acc)[NL][4], const int (&lim)[NL], int n, int gq, int GQ,
                                           float out[NL]) {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        float s1, s2;
        if (lim[j] == kC - 1) leaf_moments<true>(acc[j], lim[j], gq, s1, s2);
        else leaf_moments<false>(acc[j], lim[j], gq, s1, s2);
        const float v = trunc_score2<S>(cols4_sum(s1), cols4_sum(s2), lim[j] + 1);
        out[j] = row16_sum((n < GQ) ? v : 0.0f);
    }
}

// Leaf scores for any score: the LSE or a truncation.
template <int NL, int S>
__device__ inline void leaf_scores_from_acc(const f32x4 (&acc)[NL][4], const int (&lim)[NL], int n, int gq,
                                            int GQ, float out[NL]) {
    if constexpr (S == kScoreLse) leaf_lse_from_acc<NL>(acc, lim, n, gq, GQ, out);
    else leaf_trunc_from_acc<NL, S>(acc, lim, n, gq, GQ, out);
}

}  // namespace pisa
