// leaf.hip -- leaf level of the coarse-to-fine walk (gfx950).
//
// Reading note "Block Sparse Attention with Log-Linear Complexity":
//   section 3.2  -- the candidates of the leaf level are the children of the
//                   level-2 survivors; with at most K candidates all are kept,
//                   otherwise the K best are the selected blocks;
//   "Scoring: LogSumExp" -- at the leaf level the children of a candidate are
//                   its raw keys, so its score is the exact raw-key LSE;
//   section 4.1  -- the query heads of a GQA group add their scores.
//
// Lane layout of the 16x16 MFMA tiles: column n = lane % 16 is the query head
// of the group and lane group gq = lane / 16 supplies one quarter of the d = 64
// contraction; rows are 16 raw keys of the candidate leaf (4 tiles cover its
// 64 keys). A result tile holds, in lane (gq, n), keys 4*gq .. 4*gq+3 for head
// n. bf16 keys times bf16 queries on v_mfma_f32_16x16x32_bf16 (fp32 inputs on
// v_mfma_f32_16x16x4_f32): exact products accumulated in fp32. Keys after the
// query position are masked. The LSE reduces over the rows (in-lane, then xor
// 16/32), the group sum over the columns (xor 1..8).
#include "pisa_device.h"

namespace pisa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Query fragments of one walk: dims {8gq..8gq+7, 32+8gq..32+8gq+7} of head n.
template <typename KT>
struct QFrag;

template <>
struct QFrag<uint16_t> {
    bf16x8 lo, hi;     // bf16 MFMA B operand (two k-steps of 32)
    float f[16];       // the same 16 values widened to fp32
    __device__ void load(const uint16_t* qrow, bool valid, int gq) {
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (valid) {
            a = *reinterpret_cast<const u32x4*>(qrow + 8 * gq);
            b = *reinterpret_cast<const u32x4*>(qrow + 32 + 8 * gq);
        }
        lo = __builtin_bit_cast(bf16x8, a);
        hi = __builtin_bit_cast(bf16x8, b);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(a[i] << 16);
            f[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
            f[8 + 2 * i] = __uint_as_float(b[i] << 16);
            f[8 + 2 * i + 1] = __uint_as_float(b[i] & 0xffff0000u);
        }
    }
};

template <>
struct QFrag<float> {
    float f[16];
    __device__ void load(const float* qrow, bool valid, int gq) {
        float a[8] = {0, 0, 0, 0, 0, 0, 0, 0}, b[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (valid) {
            load8_f32(qrow + 8 * gq, a);
            load8_f32(qrow + 32 + 8 * gq, b);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) { f[i] = a[i]; f[8 + i] = b[i]; }
    }
};

// fp32 tile: rows' 16 fp32 values (same dim order as QFrag::f) against the query.
__device__ inline f32x4 mfma_rows_f32(const float a[16], const float qf[16]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 16; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], qf[s], acc, 0, 0, 0);
    return acc;
}

// Leaf-level tile of 16 raw keys starting at key `row0` (lane row = lane % 16).
template <typename KT>
__device__ inline f32x4 leaf_tile(const KT* kbase, int64_t row_stride, int64_t key,
                                  bool in_range, const QFrag<KT>& q, int gq);

template <>
__device__ inline f32x4 leaf_tile<uint16_t>(const uint16_t* kbase, int64_t row_stride, int64_t key,
                                            bool in_range, const QFrag<uint16_t>& q, int gq) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (in_range) {
        const uint16_t* row = kbase + key * row_stride;
        a = *reinterpret_cast<const u32x4*>(row + 8 * gq);
        b = *reinterpret_cast<const u32x4*>(row + 32 + 8 * gq);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), q.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b), q.hi, acc, 0, 0, 0);
    return acc;
}

template <>
__device__ inline f32x4 leaf_tile<float>(const float* kbase, int64_t row_stride, int64_t key,
                                         bool in_range, const QFrag<float>& q, int gq) {
    float a[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = 0.f;
    if (in_range) {
        const float* row = kbase + key * row_stride;
        load8_f32(row + 8 * gq, a);
        load8_f32(row + 32 + 8 * gq, a + 8);
    }
    return mfma_rows_f32(a, q.f);
}

// Sum over the group's heads (columns n < GQ) of a per-(lane group, head) value.
__device__ inline float group_sum(float v, int n, int GQ) {
    v = (n < GQ) ? v : 0.0f;
    v += xor_f(v, 1);
    v += xor_f(v, 2);
    v += xor_f(v, 4);
    v += xor_f(v, 8);
    return v;
}

// Score of one candidate leaf: exact LSE over its raw keys <= t, summed over the group.
template <typename KT>
__device__ inline float score_leaf(const KT* kbase, int64_t row_stride, const Geom& G, int64_t t,
                                   int64_t leaf, const QFrag<KT>& q, int lane) {
    const int n = lane & 15, gq = lane >> 4;
    const int64_t key0 = leaf * kC;
    f32x4 acc[4];
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
        const int64_t key = key0 + 16 * tau + n;
        acc[tau] = leaf_tile<KT>(kbase, row_stride, key, key <= t, q, gq);
    }
    // lane holds keys key0 + 16*tau + 4*gq + r for head n
    const float c2 = 0.125f * kLog2e;
    if (G.score != kScoreLse) {
        // truncated scores: moments of the base-2 logits of the keys <= t, then mean
        // (+ var/2), in natural units like the LSE below
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int tau = 0; tau < 4; ++tau)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t key = key0 + 16 * tau + 4 * gq + r;
                const float v = (key <= t) ? acc[tau][r] * c2 : 0.0f;
                s1 += v;
                s2 += v * v;
            }
        s1 += xor_f(s1, 16);
        s1 += xor_f(s1, 32);
        s2 += xor_f(s2, 16);
        s2 += xor_f(s2, 32);
        const int64_t m64 = t - key0 + 1;
        const float m = (float)((m64 < kC) ? m64 : kC);
        const float mean = s1 / m;
        const float var = s2 / m - mean * mean;
        const float sc = (G.score == kScoreMean) ? mean : mean + 0.5f * kLn2 * var;
        return group_sum(sc * kLn2, n, G.GQ);
    }
    float z[16];
    float mx = -INFINITY;
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t key = key0 + 16 * tau + 4 * gq + r;
            const float v = (key <= t) ? acc[tau][r] * c2 : -INFINITY;
            z[4 * tau + r] = v;
            mx = fmaxf(mx, v);
        }
    }
    mx = fmaxf(mx, xor_f(mx, 16));
    mx = fmaxf(mx, xor_f(mx, 32));
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += __builtin_amdgcn_exp2f(z[i] - mx);
    s += xor_f(s, 16);
    s += xor_f(s, 32);
    const float lse = (mx + __builtin_amdgcn_logf(s)) * kLn2;
    return group_sum(lse, n, G.GQ);
}

// Keep the K best of the candidate slots (score desc, node asc); returns the survivors
// compacted into lanes 0..K-1 (-1 elsewhere).
__device__ inline int topk_survivors(float my, int cand, int nslots, int K, int lane) {
    int rank = 0;
    for (int j = 0; j < nslots; ++j) {
        const int nj = readlane_i(cand, j);
        const float sj = readlane_f(my, j);
        if (nj >= 0) rank += (sj > my || (sj == my && nj < cand)) ? 1 : 0;
    }
    const bool keep = cand >= 0 && rank < K;
    const int got = push_to_lane(keep ? rank : 63, cand);
    return (lane < K) ? got : -1;
}

// Leaf level of the walk, one wavefront per walk: the candidate leaves come from
// the upper-level pass (ascending, -1 padded, ncand of them). With at most K
// candidates all are kept; otherwise each scores its exact raw-key LSE summed
// over the group and the K best are written in ascending order, -1 padded.
template <typename KT>
__global__ __launch_bounds__(256) void leaf_walk_kernel(const KT* __restrict__ q, const KT* __restrict__ k,
                                                        Geom G, int64_t t0, int64_t NT,
                                                        const int32_t* __restrict__ cand,
                                                        const int32_t* __restrict__ ncand,
                                                        int32_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int K = G.topk, CS = 2 * G.topk;
    const int64_t total = (int64_t)G.B * NT * G.Hkv;
    const int64_t stride = (int64_t)gridDim.x * 4;
    const int64_t row_stride = (int64_t)G.Hkv * kD;
    for (int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); w < total; w += stride) {
        const int kvh = (int)(w % G.Hkv);
        const int64_t bt = w / G.Hkv;
        const int64_t t = t0 + bt % NT;
        const int b = (int)(bt / NT);
        const int nc = ncand[w];
        const int c = (lane < CS) ? cand[w * CS + lane] : -1;
        int32_t* out_row = out + w * K;
        if (nc <= K) {
            if (lane < K) out_row[lane] = c;          // already ascending, -1 padded
            continue;
        }
        const int n = lane & 15, gq = lane >> 4;
        QFrag<KT> qf;
        qf.load(q + (bt * G.Hq + (int64_t)kvh * G.GQ + n) * kD, n < G.GQ, gq);
        const KT* kbase = k + ((int64_t)b * G.cap * G.Hkv + kvh) * kD;
        float my = -INFINITY;
        for (int m = 0; m < CS; ++m) {
            const int leaf = readlane_i(c, m);
            if (leaf < 0) break;
            const float s = score_leaf<KT>(kbase, row_stride, G, t, leaf, qf, lane);
            if (lane == m) my = s;
        }
        const int surv = topk_survivors(my, c, CS, K, lane);
        int pos = 0;
        for (int j = 0; j < K; ++j) {
            const int sj = readlane_i(surv, j);
            pos += (sj >= 0 && sj < surv) ? 1 : 0;
        }
        if (lane < K) out_row[pos] = surv;
    }
}

template __global__ void leaf_walk_kernel<float>(const float*, const float*, Geom, int64_t, int64_t,
                                                 const int32_t*, const int32_t*, int32_t*);

}  // namespace pisa
